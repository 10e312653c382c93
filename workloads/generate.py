"""Seeded tensors for a workload (random draws and storage casts only).

Recipe (each stream is numpy's default_rng(SeedSequence([cfg_id, tensor_id,
index, seed]))):
  tensor 0  x   [T, H]  ~ N(0, 1)            index = T
  tensor 1  Wr  [H, E]  ~ N(0, wr_std)       index = 0
  tensor 2  W1  [E, 2I, H] ~ N(0, w_std)     index = expert (one stream per expert;
                                              [E, I, H] for the ungated ReLU2 expert)
  tensor 3  W2  [E, H, I]  ~ N(0, w_std)     index = expert
  (W1 and W2 carry E + n_shared experts: the shared ones last)
  tensor 4  Gumbel noise [T, E] (Zipf routing only)   index = T
  tensor 5  permutation of expert popularity ranks (Zipf routing only)
  tensor 6  dout [T, H] ~ N(0, 1)            index = T (the output gradient of
                                              a training step)
Draws are fp32 and rounded RN to bf16 with torch. Router logits:
  uniform: fp32( x . Wr ) evaluated in float64 from the bf16 values;
  zipf:    fp32( log p_e + G[t, e] ), p_e proportional to (rank_e + 1)^-1.2,
           which makes the top-k a Zipf-weighted draw without replacement
           (Gumbel-top-k).

make_inputs_device draws the same distributions with torch's generator on
the GPU (seeded from the same SeedSequence) and computes the uniform-routing
logits in fp32 there: for throughput sweeps over large shapes, where drawing
gigabytes of weights on the host would dominate. Parity tests use
make_inputs.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import Config

ZIPF_S = 1.2


def _rng(cfg: Config, tensor_id: int, index: int, seed: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg.cfg_id, tensor_id, index, seed]))


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """bf16 / fp32 torch tensor -> float64 numpy array (exact)."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def make_expert_weights(cfg: Config, tensor_id: int, e: int, seed: int = 0) -> torch.Tensor:
    """One expert's W1 ([2I or I, H], tensor_id 2) or W2 ([H, I], tensor_id 3) in bf16."""
    shape = (cfg.w1_rows, cfg.H) if tensor_id == 2 else (cfg.H, cfg.I)
    g = _rng(cfg, tensor_id, e, seed)
    return _bf16(g.standard_normal(shape, dtype=np.float32) * np.float32(cfg.w_std))


def _stack_experts(cfg: Config, tensor_id: int, seed: int) -> torch.Tensor:
    shape = (cfg.w1_rows, cfg.H) if tensor_id == 2 else (cfg.H, cfg.I)
    out = torch.empty((cfg.E_total,) + shape, dtype=torch.bfloat16)

    def fill(e):
        out[e].copy_(make_expert_weights(cfg, tensor_id, e, seed))

    workers = max(1, min(16, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill, range(cfg.E_total)))
    return out


@dataclass
class Inputs:
    cfg: Config
    x: torch.Tensor                 # bf16 [T, H]
    logits: torch.Tensor            # fp32 [T, E]
    w1: Optional[torch.Tensor]      # bf16 [E, 2I, H]
    w2: Optional[torch.Tensor]      # bf16 [E, H, I]
    seed: int = 0

    def expert_w1(self, e: int) -> torch.Tensor:
        return self.w1[e] if self.w1 is not None else make_expert_weights(self.cfg, 2, e, self.seed)

    def expert_w2(self, e: int) -> torch.Tensor:
        return self.w2[e] if self.w2 is not None else make_expert_weights(self.cfg, 3, e, self.seed)


def make_dout(cfg: Config, seed: int = 0, device=None) -> torch.Tensor:
    """Output gradient dout [T, H] bf16 ~ N(0, 1) (tensor 6). device: draw it
    there with torch's generator (seeded from the same SeedSequence)."""
    if device is None:
        return _bf16(_rng(cfg, 6, cfg.T, seed).standard_normal((cfg.T, cfg.H), dtype=np.float32))
    s = np.random.SeedSequence([cfg.cfg_id, 6, cfg.T, seed]).generate_state(1, np.uint64)[0]
    g = torch.Generator(device=device)
    g.manual_seed(int(s) & ((1 << 63) - 1))
    return torch.randn((cfg.T, cfg.H), generator=g, device=device).to(torch.bfloat16)


def make_logits(cfg: Config, x: torch.Tensor, seed: int = 0) -> torch.Tensor:
    T, E = x.shape[0], cfg.E
    if cfg.routing == "uniform":
        wr = _bf16(_rng(cfg, 1, 0, seed).standard_normal((cfg.H, E), dtype=np.float32)
                   * np.float32(cfg.wr_std))
        l64 = to_f64(x) @ to_f64(wr)
        return torch.from_numpy(l64.astype(np.float32))
    if cfg.routing == "zipf":
        ranks = _rng(cfg, 5, 0, seed).permutation(E)
        logp = -ZIPF_S * np.log(ranks + 1.0)
        logp -= np.log(np.exp(logp).sum())
        gumbel = _rng(cfg, 4, T, seed).gumbel(size=(T, E))
        return torch.from_numpy((logp[None, :] + gumbel).astype(np.float32))
    raise ValueError(f"unknown routing {cfg.routing!r}")


def make_inputs(cfg: Config, seed: int = 0, with_weights: bool = True) -> Inputs:
    """All inputs of one batch. with_weights=False leaves W1/W2 to be drawn
    one expert at a time (Inputs.expert_w1 / expert_w2)."""
    x = _bf16(_rng(cfg, 0, cfg.T, seed).standard_normal((cfg.T, cfg.H), dtype=np.float32))
    logits = make_logits(cfg, x, seed)
    w1 = _stack_experts(cfg, 2, seed) if with_weights else None
    w2 = _stack_experts(cfg, 3, seed) if with_weights else None
    return Inputs(cfg, x, logits, w1, w2, seed)


def make_inputs_device(cfg: Config, device, seed: int = 0) -> Inputs:
    """Inputs of the same distributions drawn on `device` (uniform routing;
    logits = fp32(x . Wr) in fp32 on the device)."""
    if cfg.routing != "uniform":
        raise ValueError("make_inputs_device: uniform routing only")

    def gen(tensor_id, index):
        s = np.random.SeedSequence([cfg.cfg_id, tensor_id, index, seed]).generate_state(1, np.uint64)[0]
        g = torch.Generator(device=device)
        g.manual_seed(int(s) & ((1 << 63) - 1))
        return g

    x = torch.randn((cfg.T, cfg.H), generator=gen(0, cfg.T), device=device).to(torch.bfloat16)
    wr = (torch.randn((cfg.H, cfg.E), generator=gen(1, 0), device=device) * cfg.wr_std).to(torch.bfloat16)
    logits = x.float() @ wr.float()
    w1 = torch.empty((cfg.E_total, cfg.w1_rows, cfg.H), dtype=torch.bfloat16, device=device)
    w2 = torch.empty((cfg.E_total, cfg.H, cfg.I), dtype=torch.bfloat16, device=device)
    for e in range(cfg.E_total):
        w1[e] = (torch.randn((cfg.w1_rows, cfg.H), generator=gen(2, e), device=device) * cfg.w_std).to(torch.bfloat16)
        w2[e] = (torch.randn((cfg.H, cfg.I), generator=gen(3, e), device=device) * cfg.w_std).to(torch.bfloat16)
    return Inputs(cfg, x, logits, w1, w2, seed)
