"""Seeded synthetic workloads for the hybrid-block attention hot path.

This package only draws random numbers and stores them in the byte formats the
library consumes (fp32, bf16 bit patterns, FP8 E4M3FN codes with a per-row fp32
scale).  It holds none of the method's arithmetic: no attention, no scores, no
selection, no projection.  Both the float64 oracle (``oracle/``) and the HIP
path consume the bytes produced here.
"""
from .configs import CONFIGS, Config, get_config, small_config  # noqa: F401
from .gen import Workload, make_workload  # noqa: F401
from .agentic import AGENTIC, AgenticConfig, AgenticInputs, make_agentic  # noqa: F401
from .bridge_fp8 import BRIDGE_FP8, BridgeFp8Config, BridgeFp8Inputs, make_bridge_fp8_inputs  # noqa: F401
