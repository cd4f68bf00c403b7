"""Seeded synthetic inputs for the DeepSeekMoE layer forward pass.

This package only *makes inputs*: the named workload shapes and the seeded
random tensors in their stored form (bf16, fp32, or fp8-e4m3 codes with fp32
per-output-row scales). It holds none of the layer's arithmetic, so both the
fp64 oracle and the HIP path can consume the very same stored values without
sharing any code of the method.
"""

from .configs import CONFIGS, MoEConfig, get_config, scaled_config  # noqa: F401
from .generate import make_inputs, make_x, to_numpy_stored  # noqa: F401
