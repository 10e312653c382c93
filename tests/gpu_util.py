"""Helpers for the GPU parity tests (comparison metrics, device transfer)."""
import sys

import numpy as np
import torch

DEV = "cuda:0"


def say(*a):
    """Name the case before each GPU step (flushed, so it survives a crash)."""
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def cuda(t):
    return t.to(DEV).contiguous()


def f64(t):
    """float64 copy of a tensor (slice before converting: unwritten memory may hold NaN patterns)."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def assert_route_weights(got, ref):
    """Gate weights: the kernel evaluates them in double precision and rounds
    once to fp32, the oracle in float64 and rounds once to fp32; the two
    agree bit for bit except where the exact weight lies within a few units in
    2^-53 of an fp32 rounding midpoint, and then differ by one fp32 step."""
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    step = np.spacing(np.abs(ref))
    assert np.all(np.abs(got.astype(np.float64) - ref) <= step), "route weight off by more than one fp32 step"
    assert np.mean(got == ref) >= 0.999, f"only {np.mean(got == ref):.5f} of the route weights bit-exact"


def rel_fro(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def min_row_cos(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    na, nb = np.linalg.norm(a, axis=1), np.linalg.norm(b, axis=1)
    ok = (na > 0) & (nb > 0)
    if not ok.any():
        return 1.0
    cos = (a[ok] * b[ok]).sum(1) / (na[ok] * nb[ok])
    return float(cos.min())


def bf16_ulp(v):
    """Spacing of bf16 values at |v| (normal range)."""
    a = np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.frexp(a)[1] - 8)


U32 = 2.0 ** -24   # unit roundoff of fp32

# The scaled f8f6f4 MFMA (FP8 and MX GEMMs) adds the products of each aligned
# group of 8 K elements after aligning them to the group's largest product and
# drops the bits more than 13 places below that product's leading bit (the
# "accum" lines of mixture_experts_routed_top_amd/probes/mfma_probe: with
# products 448 and -448 in a group, six products of 2^-5 survive and six of
# 2^-6 vanish). A group loses less than 2^-13 of its largest product per
# other product, so a dot product loses at most F8F6F4_GROUP_LOSS times the
# sum of its product magnitudes on top of the fp32 rounding of the group sums.
# (The BF16 MFMA keeps at least 24 bits in the same test, within fp32.)
F8F6F4_GROUP_LOSS = 7 * 2.0 ** -13


def assert_within_rounding(got, ref, delta, min_exact=None):
    """got was rounded to bf16 from a value within `delta` of the exact value
    whose bf16 rounding is ref: |got - ref| <= delta + one bf16 step.

    delta is the caller's bound on the fp32 arithmetic error of the kernel
    (e.g. n * 2^-24 * sum|terms| for an n-term fp32 sum)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    lim = bf16_ulp(np.abs(ref) + delta) + delta + 1e-38
    bad = np.abs(got - ref) > lim
    assert not bad.any(), (f"{bad.sum()} of {bad.size} beyond the rounding bound; worst "
                           f"{np.max(np.abs(got - ref) - lim):.3e}")
    if min_exact is not None:
        frac = float(np.mean(got == ref))
        assert frac >= min_exact, f"only {frac:.4f} identical"


# pass criteria for the routed forward output: relative Frobenius error of
# the whole [T, H] output per numeric path, and the worst per-token cosine
TOL_FRO = {0: 1e-2, 1: 2e-2, 2: 2e-2}
TOL_COS = 0.9995
