"""Seeded synthetic inputs for the Stable LatentMoE layer.

This package is the only thing the CPU oracle and the GPU path share: it turns a
workload description into bit-identical inputs on the host (for the oracle) and
in device memory (for the GPU library).  It holds none of the layer's
arithmetic: the generator is SplitMix64 + a 12-term Irwin-Hall sum, defined in
``synth_core.h``.
"""
from .gen import (  # noqa: F401
    TID, scale_for, host_fill, host_fill_values, numpy_fill_f32, bf16_bits_to_f64,
    f64_to_bf16_bits, device_fill, splitmix_output, load_host_lib,
)
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .params import HostParams, device_params, outlier_rows, zipf_logit_offset  # noqa: F401
