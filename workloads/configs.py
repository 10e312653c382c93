"""The workloads, by name and size.

Shapes follow the pages' workloads: the BF16 routed-expert MoE MLP with
Qwen3-30B-A3B and Llama 4 Scout shapes at T=8192 (Liger-Kernel PR #1463,
MoEBenchmark results), the FP8 E4M3 per-128-scaled one-GPU expert share
(TileScale PR #70, Design), and the MXFP4-weight x FP8-activation shape
H=2560, 512 experts, top-10, I=640 swept over tokens (FlashInfer PR #6465,
Benchmark configuration and Performance).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

DTYPE_BF16 = 0
DTYPE_FP8_BLOCK128 = 1
DTYPE_MXFP4W_MXFP8A = 2
SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1
ACT_SWIGLU = 0       # W1 [E, 2I, H]: gate and up
ACT_RELU2 = 1        # W1 [E, I, H]: one projection, squared ReLU


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int          # seeds: SeedSequence([cfg_id, tensor_id, index])
    T: int
    H: int
    E: int
    k: int
    I: int
    dtype: int
    score: int
    w_std: float         # std of W1 / W2 entries
    wr_std: float = 0.02  # std of the router projection
    routing: str = "uniform"   # "uniform" (x . Wr) or "zipf" (Gumbel-top-k, s = 1.2)
    act: int = ACT_SWIGLU
    n_shared: int = 0    # shared experts (used by every token, weight 1), after the E routed ones

    @property
    def E_total(self) -> int:
        return self.E + self.n_shared

    @property
    def w1_rows(self) -> int:
        """Rows of one expert's W1."""
        return 2 * self.I if self.act == ACT_SWIGLU else self.I

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)

    @property
    def A(self) -> int:
        return self.T * self.k

    @property
    def flops(self) -> int:
        """Routed GEMM FLOPs (shared experts are not counted, as on the pages)."""
        return (6 if self.act == ACT_SWIGLU else 4) * self.T * self.k * self.H * self.I


CONFIGS = {
    # tiny BF16 case: T=64, H=256, 8 experts, top-2, I=128
    "tiny_bf16": Config("tiny_bf16", 1, 64, 256, 8, 2, 128, DTYPE_BF16, SCORE_SOFTMAX, 0.02),
    # Qwen3-30B-A3B-shaped BF16 fine-grained MoE
    "qwen3_30b_a3b_bf16": Config("qwen3_30b_a3b_bf16", 2, 8192, 2048, 128, 8, 768,
                                 DTYPE_BF16, SCORE_SOFTMAX, 0.02),
    # same, Zipf(s=1.2)-skewed expert load
    "qwen3_30b_a3b_bf16_zipf": Config("qwen3_30b_a3b_bf16_zipf", 2, 8192, 2048, 128, 8, 768,
                                      DTYPE_BF16, SCORE_SOFTMAX, 0.02, routing="zipf"),
    # Llama-4-Scout-shaped BF16 coarse MoE, routed experts only, top-1 sigmoid gate
    "llama4_scout_bf16": Config("llama4_scout_bf16", 3, 8192, 5120, 16, 1, 8192,
                                DTYPE_BF16, SCORE_SIGMOID, 0.01),
    # FP8 E4M3 128-block scaled, one GPU's 64-expert share
    "fp8_block128_share": Config("fp8_block128_share", 4, 8192, 7168, 64, 8, 2048,
                                 DTYPE_FP8_BLOCK128, SCORE_SOFTMAX, 0.02),
    # MXFP4 weights x MXFP8 activations, T swept 128 / 1024 / 8192 / 16384
    "mxfp4_moe_t128": Config("mxfp4_moe_t128", 5, 128, 2560, 512, 10, 640,
                             DTYPE_MXFP4W_MXFP8A, SCORE_SOFTMAX, 0.02),
    "mxfp4_moe_t1024": Config("mxfp4_moe_t1024", 5, 1024, 2560, 512, 10, 640,
                              DTYPE_MXFP4W_MXFP8A, SCORE_SOFTMAX, 0.02),
    "mxfp4_moe_t8192": Config("mxfp4_moe_t8192", 5, 8192, 2560, 512, 10, 640,
                              DTYPE_MXFP4W_MXFP8A, SCORE_SOFTMAX, 0.02),
    "mxfp4_moe_t16384": Config("mxfp4_moe_t16384", 5, 16384, 2560, 512, 10, 640,
                               DTYPE_MXFP4W_MXFP8A, SCORE_SOFTMAX, 0.02),
    # the Qwen3-30B-A3B shape plus one shared expert of the routed experts' size
    "qwen3_30b_a3b_bf16_shared": Config("qwen3_30b_a3b_bf16_shared", 7, 8192, 2048, 128, 8, 768,
                                        DTYPE_BF16, SCORE_SOFTMAX, 0.02, n_shared=1),
    # the Nemotron shape with ungated squared-ReLU experts (FlashInfer PR #5129,
    # Measured: H=2688, I=1856, 128 experts, top-6, ReLU2; 2048..8192 tokens)
    "nemotron_relu2_bf16": Config("nemotron_relu2_bf16", 6, 8192, 2688, 128, 6, 1856,
                                  DTYPE_BF16, SCORE_SOFTMAX, 0.02, act=ACT_RELU2),
}


# The parameter grid of Liger-Kernel PR #1463 ("Additional eight-GPU sweeps",
# H200 parameter grid): T=8192, hidden = intermediate = D in {2048, 4096},
# E in {8, 16, 32, 64, 128}, top-K in {1, 2, 4, 8} with K < E (38 shapes).
# BF16, softmax top-K. Run whole on one GPU, each shape has the per-expert
# GEMM shapes (8192 K / E rows per expert) of one rank's share under expert
# parallelism.
P5_GRID = []
for _d in (2048, 4096):
    for _e in (8, 16, 32, 64, 128):
        for _k in (1, 2, 4, 8):
            if _k < _e:
                _name = f"grid_d{_d}_e{_e}_k{_k}"
                CONFIGS[_name] = Config(_name, 10 + len(P5_GRID), 8192, _d, _e, _k, _d, DTYPE_BF16, SCORE_SOFTMAX, 0.02)
                P5_GRID.append(_name)


def get_config(name: str) -> Config:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}") from None
