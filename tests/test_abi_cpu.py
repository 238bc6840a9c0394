"""The C-ABI library: loads, exports every declared symbol, validates on the host.

No call here reaches the GPU: each either only sizes, or fails validation
before anything would be enqueued.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "replayssm.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|int)\s+(replayssm_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def rs():
    import ssm_decode_amd

    ssm_decode_amd.lib()
    return ssm_decode_amd


def test_header_declares_the_five_path_calls():
    names = declared_functions()
    for n in ("replayssm_append", "replayssm_decode", "replayssm_verify", "replayssm_flush", "replayssm_accept"):
        assert n in names


def test_library_exports_every_declared_symbol(rs):
    out = subprocess.run(["nm", "-D", "--defined-only", rs.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (replayssm_\w+)", out))
    missing = set(declared_functions()) - exported
    assert not missing, missing
    # and the binding wraps every one of them
    assert set(declared_functions()) == set(rs.SIGNATURES) | set(rs.STRING_FUNCTIONS)


def test_library_has_no_oracle_dependency(rs):
    out = subprocess.run(["nm", "-D", rs.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "oracle_" not in out
    ldd = subprocess.run(["readelf", "-d", rs.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "liboracle" not in ldd


def test_sizes_of_the_b256_mamba2_layer(rs):
    s = rs.get_sizes(rs.make_config("mamba2", "fp32", 256, 128, 64, 128, 16, 1))
    assert s.C == 17
    assert s.hp_bytes == 256 * 128 * 64 * 128 * 4 == 1 << 30
    assert s.lp_bytes == 0
    assert s.ring_k_bytes == 256 * 128 * 17 * 128 * 4
    assert s.ring_v_bytes == 256 * 128 * 17 * 64 * 4
    s2 = rs.get_sizes(rs.make_config("mamba2", "fp32_hp_bf16_lp", 256, 128, 64, 128, 16, 4))
    assert s2.C == 20 and s2.lp_bytes == s2.hp_bytes // 2
    s3 = rs.get_sizes(rs.make_config("mamba2", "bf16_shared", 2, 2, 64, 128, 16, 4))
    assert s3.hp_bytes == 0 and s3.lp_bytes > 0
    s4 = rs.get_sizes(rs.make_config("gdn", "fp32", 256, 32, 128, 128, 16, 4))
    assert s4.ring_beta_bytes == 256 * 32 * 20 * 4 and s4.ring_vraw_bytes == 0
    s5 = rs.get_sizes(rs.make_config("gdn", "fp32_hp_bf16_lp", 256, 32, 128, 128, 16, 4))
    assert s5.ring_vraw_bytes == s5.ring_v_bytes == 256 * 32 * 20 * 128 * 4 and s5.lp_bytes == s5.hp_bytes // 2
    assert s2.ring_vraw_bytes == 0
    s6 = rs.get_sizes(rs.make_config("kda", "fp32", 256, 32, 128, 128, 16, 4))
    assert s6.ring_alpha_bytes == 256 * 32 * 20 * 128 * 4 and s6.ring_beta_bytes == 256 * 32 * 20 * 4
    assert s6.ring_vraw_bytes == 0 and s6.hp_bytes == 256 * 32 * 128 * 128 * 4


@pytest.mark.parametrize("L,T", [(4, 1), (4, 4), (8, 8), (16, 8), (32, 8), (64, 1), (64, 4), (64, 8)])
def test_window_sweep_configs_fit(rs, L, T):
    """Every window of the sweep fits a gfx950 workgroup's LDS at the real head shape (dv=64,
    dk=128); from L=64 with T=4 on with unpadded record rows, L=64 with T=8 past 64 KiB."""
    cfg = rs.make_config("mamba2", "fp32", 256, 128, 64, 128, L, T)
    assert rs.get_sizes(cfg).C == L + T


@pytest.mark.parametrize("kw,code", [
    (dict(kind=5), -1), (dict(precision=7), -1), (dict(B=0), -1), (dict(B=70000), -1), (dict(H=0), -1), (dict(B=65535, H=16385), -1), (dict(B=1, H=1 << 21), -1),
    (dict(dv=24), -1), (dict(dv=272), -1), (dict(dk=48), -1), (dict(dk=256), -1), (dict(L=0), -1),
    (dict(L=65), -1), (dict(T_max=0), -1), (dict(T_max=9, L=16), -1), (dict(T_max=5, L=4), -1),
    (dict(precision="fp32_hp_bf16_lp", dk=16, dv=16), -2), (dict(kind="gdn", precision="bf16_shared"), -2),
    (dict(kind="gdn", precision="fp32_hp_bf16_lp", L=64, T_max=4, dv=128), 0),
    (dict(L=64, T_max=8, dv=256, dk=128), 0), (dict(L=64, T_max=8), 0),
    (dict(kind="kda", precision="fp32_hp_bf16_lp"), -2), (dict(kind="kda", precision="bf16_shared"), -2),
    (dict(kind="kda", L=64, T_max=8, dv=128), 0), (dict(kind="kda", L=64, T_max=8, dv=256), -2),
    (dict(kind="kda"), 0), (dict(kind="kda", dk=16, dv=16, L=64), 0),
])
def test_config_validation(rs, kw, code):
    base = dict(kind="mamba2", precision="fp32", B=2, H=3, dv=64, dk=128, L=16, T_max=4)
    base.update(kw)
    cfg = rs.make_config(**base)
    sz = rs.Sizes()
    assert rs.lib().replayssm_get_sizes(ctypes.byref(cfg), ctypes.byref(sz)) == code
    assert rs.last_error()


def test_calls_reject_bad_arguments_before_enqueueing(rs):
    L = rs.lib()
    cfg = rs.make_config("mamba2", "fp32", 2, 3, 64, 128, 16, 4)
    st = rs.State()  # all NULL
    assert L.replayssm_init(ctypes.byref(cfg), ctypes.byref(st), None) == rs.EINVAL
    assert L.replayssm_init(ctypes.byref(cfg), None, None) == rs.EINVAL
    assert L.replayssm_decode(None, ctypes.byref(st), None, None, None) == rs.EINVAL
    fake = 1 << 20  # aligned, never dereferenced: validation fails first
    st_ok = rs.State(*([fake] * 13))
    st_ok.lp = None
    st_ok.ring_beta = None
    assert L.replayssm_append(ctypes.byref(cfg), ctypes.byref(st_ok), 0, fake, fake, fake, None, None) == rs.EINVAL
    assert L.replayssm_append(ctypes.byref(cfg), ctypes.byref(st_ok), 5, fake, fake, fake, None, None) == rs.EINVAL
    assert "T=5" in rs.last_error()
    assert L.replayssm_append_dt(ctypes.byref(cfg), ctypes.byref(st_ok), 0, fake, fake, None, fake, fake, None,
                                 None) == rs.EINVAL
    assert L.replayssm_append_dt(ctypes.byref(cfg), ctypes.byref(st_ok), 1, fake, None, None, fake, fake, None,
                                 None) == rs.EINVAL
    assert "A is NULL" in rs.last_error()
    assert L.replayssm_append_dt(ctypes.byref(cfg), ctypes.byref(st_ok), 1, None, fake, None, fake, fake, None,
                                 None) == rs.EINVAL
    cfg_k = rs.make_config("kda", "fp32", 2, 3, 64, 128, 16, 4)
    st_k = rs.State(*([fake] * 13))
    st_k.lp = None
    st_k.ring_vraw = None
    assert L.replayssm_append_dt(ctypes.byref(cfg_k), ctypes.byref(st_k), 1, fake, fake, None, fake, fake, fake,
                                 None) == rs.ENOTSUP
    assert L.replayssm_verify(ctypes.byref(cfg), ctypes.byref(st_ok), 9, fake, fake, None) == rs.EINVAL
    assert L.replayssm_decode(ctypes.byref(cfg), ctypes.byref(st_ok), fake + 4, fake, None) == rs.EINVAL
    assert "aligned" in rs.last_error()
    assert L.replayssm_accept(ctypes.byref(cfg), ctypes.byref(st_ok), None, None) == rs.EINVAL
    cfg_lp = rs.make_config("mamba2", "fp32_hp_bf16_lp", 2, 3, 64, 128, 16, 4)
    assert L.replayssm_flush(ctypes.byref(cfg_lp), ctypes.byref(st_ok), None) == rs.EINVAL  # lp missing
    assert L.replayssm_eager_step(ctypes.byref(cfg_lp), fake, fake, fake, fake, None, fake, fake, None) == rs.EINVAL
    cfg_g = rs.make_config("gdn", "fp32", 2, 3, 64, 128, 16, 4)
    assert L.replayssm_eager_step(ctypes.byref(cfg_g), fake, fake, fake, fake, None, fake, fake, None) == rs.EINVAL
    assert L.replayssm_eager_accept(ctypes.byref(cfg), fake, fake, 0, None) == rs.EINVAL
    assert L.replayssm_pack_state(ctypes.byref(cfg), fake, None, None, None) == rs.EINVAL
    assert L.replayssm_unpack_state(ctypes.byref(cfg), None, None, fake, None) == rs.EINVAL
    assert L.replayssm_read_error(None, None, None) == rs.EINVAL
    assert L.replayssm_flush_selected(ctypes.byref(cfg), ctypes.byref(st_ok), None, None) == rs.EINVAL
    assert L.replayssm_snapshot(ctypes.byref(cfg), ctypes.byref(st_ok), -1, fake, fake, None) == rs.EINVAL
    assert L.replayssm_snapshot(ctypes.byref(cfg), ctypes.byref(st_ok), 0, None, None, None) == rs.OK  # nothing to do
    assert L.replayssm_snapshot(ctypes.byref(cfg), ctypes.byref(st_ok), 2, None, fake, None) == rs.EINVAL
    assert L.replayssm_restore(ctypes.byref(cfg), ctypes.byref(st_ok), 2, fake, None, None) == rs.EINVAL
    assert L.replayssm_probe_read(None, 1024, fake, None) == rs.EINVAL
    assert L.replayssm_probe_read(fake, 1000, fake, None) == rs.EINVAL
    assert "multiple of 16" in rs.last_error()
    assert L.replayssm_probe_read(fake, 0, fake, None) == rs.EINVAL
    assert L.replayssm_probe_read(fake, 1024, None, None) == rs.EINVAL


@pytest.mark.parametrize("kw,ok", [
    (dict(), True), (dict(W=1), True), (dict(W=0), False), (dict(W=5), False), (dict(D=6), False),
    (dict(D=0), False), (dict(T_max=0), False), (dict(T_max=9), False), (dict(B=0), False), (dict(B=70000), False),
])
def test_conv_config_validation(rs, kw, ok):
    base = dict(B=2, D=64, W=4, T_max=4)
    base.update(kw)
    cfg = rs.make_conv_config(**base)
    ring, ptr = ctypes.c_int64(0), ctypes.c_int64(0)
    code = rs.lib().replayssm_conv_sizes(ctypes.byref(cfg), ctypes.byref(ring), ctypes.byref(ptr))
    assert (code == rs.OK) == ok
    if ok:
        assert ring.value == base["B"] * (base["W"] - 1 + base["T_max"]) * base["D"] * 4 and ptr.value == base["B"] * 4


def test_conv_calls_reject_bad_arguments_before_enqueueing(rs):
    L = rs.lib()
    cfg = rs.make_conv_config(2, 64, 4, 4)
    fake = 1 << 20
    st = rs.ConvState(fake, fake, fake, fake, fake)
    assert L.replayssm_conv_init(ctypes.byref(cfg), None, None) == rs.EINVAL
    assert L.replayssm_conv_step(ctypes.byref(cfg), ctypes.byref(st), 0, fake, fake, None, 1, 0, fake, None) == rs.EINVAL
    assert L.replayssm_conv_step(ctypes.byref(cfg), ctypes.byref(st), 5, fake, fake, None, 1, 0, fake, None) == rs.EINVAL
    assert L.replayssm_conv_step(ctypes.byref(cfg), ctypes.byref(st), 1, fake, None, None, 1, 0, fake, None) == rs.EINVAL
    assert L.replayssm_conv_step(ctypes.byref(cfg), ctypes.byref(st), 1, fake, fake, fake + 4, 1, 0, fake,
                                 None) == rs.EINVAL
    assert "bias" in rs.last_error()
    assert L.replayssm_conv_accept(ctypes.byref(cfg), ctypes.byref(st), None, None) == rs.EINVAL
    bad = rs.ConvState(fake, None, fake, fake, fake)
    assert L.replayssm_conv_init(ctypes.byref(cfg), ctypes.byref(bad), None) == rs.EINVAL


def test_status_strings(rs):
    assert rs.status_string(0) == "ok"
    assert rs.status_string(-1) == "invalid argument"
    assert rs.status_string(-2) == "not supported"
    assert rs.status_string(-3) == "HIP runtime error"


def test_tiling_policy(rs):
    """The tiling switch is host state only: validated, stored, read back; no GPU needed."""
    assert rs.get_tiling() == rs.TILES_AUTO
    try:
        for p in (rs.TILES_ONE, rs.TILES_TWO, rs.TILES_AUTO):
            rs.set_tiling(p)
            assert rs.get_tiling() == p
        rs.set_tiling(rs.TILES_TWO)
        for bad in (3, -1, 1 << 20):
            assert rs.lib().replayssm_set_tiling(bad) == rs.EINVAL
            assert "tiling policy" in rs.last_error()
            assert rs.get_tiling() == rs.TILES_TWO
    finally:
        rs.set_tiling(rs.TILES_AUTO)


def test_binding_constants_match_the_header(rs):
    """Every status, device-error and tiling constant the binding mirrors has the header's value."""
    text = open(HEADER).read()
    defined = {m.group(1): int(m.group(2)) for m in
               re.finditer(r"^#define REPLAYSSM_(\w+)\s+\(?(-?\d+)\)?", text, re.M)}
    mirrored = [n for n in ("OK", "EINVAL", "ENOTSUP", "EHIP", "TILES_AUTO", "TILES_ONE", "TILES_TWO")]
    mirrored += [n for n in defined if n.startswith("DEVERR_")]
    for name in mirrored:
        assert getattr(rs, name) == defined[name], name
    assert {"TILES_AUTO", "TILES_ONE", "TILES_TWO", "DEVERR_INDEX"} <= set(defined)


def test_static_append_rejects_more_sequences_than_its_scratch(rs):
    """replayssm_append_static holds REPLAYSSM_STATIC_SCRATCH_SEQS counters: one sequence more is
    refused on the host, before anything would reach a device (no GPU needed), while st->arrive
    may be NULL."""
    limit = int(re.search(r"#define REPLAYSSM_STATIC_SCRATCH_SEQS (\d+)", open(HEADER).read()).group(1))
    assert limit == 16384
    fake = 1 << 20  # an aligned address that is never dereferenced
    for B, want in ((limit + 1, rs.EINVAL),):
        cfg = rs.make_config("mamba2", "fp32", B, 1, 16, 16, 4, 1)
        st = rs.State(*([fake] * len(rs.State._fields_)))
        st.lp = st.ring_beta = st.ring_vraw = st.arrive = None
        status = rs.lib().replayssm_append_static(ctypes.byref(cfg), ctypes.byref(st), 1, fake, fake, fake, None, None)
        assert status == want
        assert str(limit).encode() in rs.lib().replayssm_last_error()
