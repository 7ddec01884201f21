"""Seeded synthetic inputs for the fused-linear generalized-JSD distillation pass.

This module holds input generation only: random draws, dtype rounding of the
draws, and the structural edits that build the tie workloads. It holds none of
the method's arithmetic (no GEMM, no softmax, no divergence), so both the CPU
oracle's tests and the GPU path's tests, the smoke check and the benchmark can
draw identical inputs from it.

Recipe (shared by every consumer):
  * numpy ``Generator(PCG64(seed))``; for workload k and draw j the seed is
    ``1000 * k + j`` with j = 0 (X_s), 1 (W_s), 2 (X_t), 3 (W_t). Arrays
    larger than 2^22 elements are drawn in 2^22-element blocks, block i from
    ``PCG64(seed).jumped(i)``.
  * ``standard_normal(dtype=float32) * sigma`` with sigma_X = 1 and
    sigma_W = 0.02 (0.02 read as a standard deviation), then rounded to
    bfloat16 with round-to-nearest-even for bfloat16 workloads.
  * bfloat16 values travel as their raw uint16 bit patterns; ``bf16_to_f64``
    widens them losslessly for the oracle.

The workloads follow the pages' test and benchmark shapes (Liger-Kernel PR
#1352 "Fuse log-softmax into fused_linear_jsd kernel": the multi-block test
shape in "Testing Done" and the H=4096, V=128256 benchmark tables; PR #1374
"Fix TVD gradient at p == q": the (8, 512) fp32 tie shape and the two tie
scenarios in its Summary).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Dict, Tuple

import numpy as np

SIGMA_X = 1.0
SIGMA_W = 0.02
# Logit value given to padded vocabulary slots in the padded-vocabulary tie
# workload. -9984 is exactly representable in bfloat16 and drives
# exp(z - max) to 0.0 in fp32 and fp64 alike, so both distributions put
# exactly zero mass on those slots.
PAD_LOGIT = -9984.0
PAD_ROWS = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    index: int          # seed base: seed = 1000 * index + draw
    BT: int
    H_s: int
    H_t: int
    V: int
    dtype: str          # "f32" or "bf16"
    beta: float
    temperature: float
    reduction: str
    structure: str      # "independent", "tied", "padded"

    def seed(self, draw: int) -> int:
        return 1000 * self.index + draw


# The five workload families; beta / num_chunks sweeps are applied by callers.
WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", 1, 8, 64, 64, 512, "f32", 0.5, 1.0, "batchmean", "independent"),
    "multiblock_tail": Workload("multiblock_tail", 2, 64, 256, 256, 40960, "bf16", 0.5, 1.0, "batchmean", "independent"),
    "ties_self": Workload("ties_self", 3, 512, 1024, 1024, 32064, "bf16", 0.5, 1.0, "batchmean", "tied"),
    "ties_padded": Workload("ties_padded", 3, 512, 1024, 1024, 32064, "bf16", 0.5, 1.0, "batchmean", "padded"),
    "llama3_head": Workload("llama3_head", 4, 1024, 4096, 4096, 128256, "bf16", 0.5, 1.0, "batchmean", "independent"),
    "large_batch": Workload("large_batch", 5, 8192, 4096, 4096, 128256, "bf16", 0.5, 2.0, "batchmean", "independent"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # Inputs here are finite draws; NaN payloads are not handled.
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    t += u
    t >>= np.uint32(16)
    return t.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


# Draws are made in blocks of BLOCK elements; block i comes from the stream
# PCG64(seed).jumped(i), so large arrays fill in parallel and an array of at
# most BLOCK elements is exactly PCG64(seed)'s first draws.
BLOCK = 1 << 22


def draw(seed: int, shape: Tuple[int, ...], sigma: float, dtype: str) -> np.ndarray:
    """One seeded normal draw. Returns float32 values or bfloat16 bits (uint16)."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"unknown dtype {dtype!r}")
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    base = np.random.PCG64(seed)

    def fill(i: int) -> None:
        lo = i * BLOCK
        hi = min(n, lo + BLOCK)
        rng = np.random.Generator(base.jumped(i))
        x = rng.standard_normal(size=hi - lo, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out[lo:hi] = x if dtype == "f32" else f32_to_bf16_bits(x)

    nblocks = max(1, -(-n // BLOCK))
    if nblocks == 1:
        fill(0)
    else:
        with concurrent.futures.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as pool:
            list(pool.map(fill, range(nblocks)))
    return out.reshape(shape)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Lossless widening of a generated array (float32 values or bf16 bits)."""
    if dtype == "f32":
        return a.astype(np.float64)
    return bf16_to_f64(a)


def make_inputs(w: Workload, BT: int | None = None, V: int | None = None,
                H_s: int | None = None, H_t: int | None = None) -> Dict[str, np.ndarray]:
    """Inputs for workload ``w`` (optionally resized), as storage arrays.

    Returns X_s [BT,H_s], W_s [V,H_s], X_t [BT,H_t], W_t [V,H_t]; float32 for
    "f32" workloads and uint16 bfloat16 bit patterns for "bf16" ones.
    Structures:
      * "independent": four independent draws.
      * "tied": the teacher's X and W are bit-identical copies of the
        student's (separate arrays), so every element is a tie.
      * "padded": independent draws; feature column H-1 of X_s and X_t is set
        to 1.0 and the last PAD_ROWS vocabulary rows of W_s and W_t are zero
        except column H-1, which holds PAD_LOGIT. Those rows' logits are then
        exactly PAD_LOGIT in both models (a bias-equivalent constant), so
        the padded slots carry probability exactly 0.0 in both distributions.
    """
    BT = w.BT if BT is None else BT
    V = w.V if V is None else V
    H_s = w.H_s if H_s is None else H_s
    H_t = w.H_t if H_t is None else H_t
    dt = w.dtype
    X_s = draw(w.seed(0), (BT, H_s), SIGMA_X, dt)
    W_s = draw(w.seed(1), (V, H_s), SIGMA_W, dt)
    if w.structure == "tied":
        if H_t != H_s:
            raise ValueError("tied workload needs H_t == H_s")
        X_t = X_s.copy()
        W_t = W_s.copy()
    else:
        X_t = draw(w.seed(2), (BT, H_t), SIGMA_X, dt)
        W_t = draw(w.seed(3), (V, H_t), SIGMA_W, dt)
    if w.structure == "padded":
        if V <= PAD_ROWS:
            raise ValueError("padded workload needs V > PAD_ROWS")
        one = np.float32(1.0) if dt == "f32" else f32_to_bf16_bits(np.array([1.0], np.float32))[0]
        pad = np.float32(PAD_LOGIT) if dt == "f32" else f32_to_bf16_bits(np.array([PAD_LOGIT], np.float32))[0]
        for X, H in ((X_s, H_s), (X_t, H_t)):
            X[:, H - 1] = one
        for W, H in ((W_s, H_s), (W_t, H_t)):
            W[V - PAD_ROWS:, :] = 0
            W[V - PAD_ROWS:, H - 1] = pad
    return {"X_s": X_s, "W_s": W_s, "X_t": X_t, "W_t": W_t}


def make_logits(seed: int, BT: int, V: int, scale: float, dtype: str) -> np.ndarray:
    """A standalone logits draw for the logits-level entry point's tests."""
    return draw(seed, (BT, V), scale, dtype)
