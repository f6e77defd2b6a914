"""Seeded synthetic inputs for the HiLS attention hot path.

This module is shared by the tests, the benchmark and the smoke check. It
holds no part of the attention method's arithmetic: it only draws numbers
(a counter-based generator, see ``gen``) and shapes them into the workloads
(``configs``). Both the CPU oracle and the GPU library receive the arrays it
produces; neither imports the other.
"""
from .gen import (  # noqa: F401
    normal_f32, normal_bf16_bits, bf16_bits_to_f32, f32_to_bf16_bits,
    uniform_u64, splitmix64_key, TENSOR_IDS,
)
from .configs import CONFIGS, make_inputs, LazyNormalBF16  # noqa: F401
