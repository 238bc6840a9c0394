"""Seeded synthetic inputs for the ReplaySSM decode path.

This package only draws random numbers in the shapes and distributions of the
workloads; it holds none of the method's arithmetic, so that both the CPU oracle
(tests) and the GPU path (tests, bench) can take the very same inputs from it.
"""
from .inputs import (  # noqa: F401
    LayerShape,
    WORKLOADS,
    Workload,
    host_accept,
    host_conv_inputs,
    host_conv_params,
    host_decay_params,
    host_time_steps,
    host_initial_state,
    host_step,
    device_accept,
    device_conv_inputs,
    device_decay_params,
    device_time_steps,
    device_initial_state,
    device_step,
)
