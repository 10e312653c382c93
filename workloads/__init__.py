"""Seeded synthetic inputs for the routed-expert MoE forward.

This package only draws random numbers and converts them to bf16 / fp32
storage (via torch's RN casts). It holds none of the method's arithmetic: no
routing, sorting, quantisation, GEMM or combine. Both the oracle (oracle/)
and the HIP path consume what it produces.

The shapes are the workloads the pages name (see configs.py); the value
distributions are x ~ N(0, 1), weights ~ N(0, sigma) drawn in fp32 and
rounded RN to bf16; router logits are the fp32 rounding of x . Wr computed in
float64 on the host (the router projection is not part of the routed path).
"""
from .configs import CONFIGS, P5_GRID, Config, get_config  # noqa: F401
from .generate import Inputs, make_dout, make_inputs, make_inputs_device, make_expert_weights, to_f64  # noqa: F401
