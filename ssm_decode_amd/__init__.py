"""ReplaySSM decode path for AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
include/replayssm.h (libreplayssm.so, built by `python -m ssm_decode_amd.build`).
This package only marshals torch tensors into those calls; see _lib.py.
"""
from ._lib import (  # noqa: F401
    BF16_SHARED, DEVERR_ACCEPT, DEVERR_APPEND_OVERFLOW, DEVERR_CORRUPT, DEVERR_INDEX, DEVERR_PENDING,
    DEVERR_STALE, EHIP, EINVAL, ENOTSUP, FP32, FP32_HP_BF16_LP, GDN, KDA, MAMBA2, OK, Config, LayerState,
    ReplaySSMError, SIGNATURES, STRING_FUNCTIONS, LIB_PATH, State, Sizes, accept, append, append_dt, append_static,
    decode, decode_step,
    eager_accept, eager_step, eager_verify, flush, flush_selected, get_sizes, init, last_error, lib, make_config,
    pack_state, probe_read, read_error, restore, snapshot, status_string, unpack_state, verify, verify_step,
    TILES_AUTO, TILES_ONE, TILES_TWO, get_tiling, set_tiling,
    ConvConfig, ConvLayer, ConvState, conv_accept, conv_init, conv_sizes, conv_step, make_conv_config,
)
