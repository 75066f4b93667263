"""Seeded synthetic inputs for the FP8 delayed-scaling Linear.

This module is shared by the tests, the benchmark and the oracle checks.  It
holds none of the method's arithmetic: it only draws random numbers, shapes
them into the distributions below and rounds fp32 draws to bf16 where a tensor
is bf16 (with torch's fp32->bf16 conversion, round to nearest even).

Recipe (every draw is numpy PCG64):

* ``seed = 1_000_000 * cfg + 1_000 * step + tensor_id`` with tensor ids X=1,
  W=2, dY=3, and ``10 * p + role`` for projection ``p`` of the decoder-layer set.
* Large tensors are drawn in fixed 2**20-element chunks, chunk ``c`` from
  ``default_rng(SeedSequence(seed).spawn(...)[c])``, so the bytes do not depend
  on the number of threads.
* Outlier and mixture positions are exact counts ``round(p * n)`` drawn
  without replacement from ``default_rng(seed + 500)``.

Distributions are those of the pages' workloads: activations near-normal and
mostly inside [-4, 4] ([P2] §一, "格式选择的数学直觉"); gradients heavy-tailed,
about 99% inside [-0.01, 0.01] with about 0.1% outliers of magnitude 10 to 100
([P2] §三, "为什么权重梯度用 E5M2？"); weights N(0, 0.02^2).

Page references: [P2] "FP8 混合精度训练工程实践：从 H100 到大模型训练的范式跃迁".
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 20

TID_X, TID_W, TID_DY = 1, 2, 3

# Llama-style decoder-layer Linears: name -> (in_features, out_features).
LLAMA_PROJ = {
    "q_proj": (4096, 4096),
    "k_proj": (4096, 1024),
    "v_proj": (4096, 1024),
    "o_proj": (4096, 4096),
    "gate_proj": (4096, 14336),
    "up_proj": (4096, 14336),
    "down_proj": (14336, 4096),
}


def seed_of(cfg: int, step: int, tensor_id: int) -> int:
    return 1_000_000 * cfg + 1_000 * step + tensor_id


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _chunked(n: int, seed: int, fill) -> np.ndarray:
    """Fill an fp32 vector of ``n`` elements chunk by chunk; ``fill(rng, out)``."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK
    kids = np.random.SeedSequence(seed).spawn(nchunks)

    def work(c):
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        fill(np.random.default_rng(kids[c]), out[lo:hi])

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def normal(n: int, seed: int, std: float = 1.0) -> np.ndarray:
    def fill(rng, o):
        rng.standard_normal(o.size, dtype=np.float32, out=o)
        if std != 1.0:
            o *= np.float32(std)

    return _chunked(n, seed, fill)


def uniform(n: int, seed: int, lo: float, hi: float) -> np.ndarray:
    def fill(rng, o):
        o[:] = rng.uniform(lo, hi, o.size).astype(np.float32)

    return _chunked(n, seed, fill)


def _positions(n: int, k: int, seed: int) -> np.ndarray:
    if k == 0:
        return np.zeros(0, dtype=np.int64)
    return np.random.default_rng(seed + 500).choice(n, size=k, replace=False)


def with_outliers(x: np.ndarray, frac: float, lo: float, hi: float, seed: int) -> np.ndarray:
    """Replace ``round(frac * n)`` entries by ``+-U(lo, hi)`` with a random sign."""
    n = x.size
    k = int(round(frac * n))
    pos = _positions(n, k, seed)
    rng = np.random.default_rng(seed + 501)
    mag = rng.uniform(lo, hi, k).astype(np.float32)
    sgn = np.where(rng.random(k) < 0.5, -1.0, 1.0).astype(np.float32)
    x[pos] = mag * sgn
    return x


def heavy_tail_grad(n: int, seed: int) -> np.ndarray:
    """99% U(-0.01, 0.01), 0.9% N(0, 0.1^2), 0.1% +-U(10, 100)."""
    x = uniform(n, seed, -0.01, 0.01)
    k_mid = int(round(0.009 * n))
    k_out = int(round(0.001 * n))
    pos = _positions(n, k_mid + k_out, seed)
    rng = np.random.default_rng(seed + 502)
    x[pos[:k_mid]] = (rng.standard_normal(k_mid) * 0.1).astype(np.float32)
    mag = rng.uniform(10.0, 100.0, k_out).astype(np.float32)
    sgn = np.where(rng.random(k_out) < 0.5, -1.0, 1.0).astype(np.float32)
    x[pos[k_mid:]] = mag * sgn
    return x


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (torch's conversion)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------------------
# Per-configuration tensors.  Each returns fp32 arrays for fp32 tensors and
# uint16 bf16 bit patterns for bf16 tensors, shaped row-major.
# ---------------------------------------------------------------------------


def tiny_linear_step(step: int, m: int = 64, k: int = 128, n: int = 128):
    """Tiny single Linear (fp32): X ~ N(0,1) [m,k], W ~ N(0,0.02^2) [k,n],
    dY ~ N(0, 1e-3^2) [m,n] with 0.1% entries -> +-U(1,10).  Fresh each step."""
    cfg = 1
    x = normal(m * k, seed_of(cfg, step, TID_X)).reshape(m, k)
    w = normal(k * n, seed_of(cfg, step, TID_W), 0.02).reshape(k, n)
    dy = normal(m * n, seed_of(cfg, step, TID_DY), 1e-3)
    dy = with_outliers(dy, 0.001, 1.0, 10.0, seed_of(cfg, step, TID_DY)).reshape(m, n)
    return x, w, dy


def forward_4096(m: int = 8192, k: int = 4096, n: int = 4096, step: int = 0):
    """Forward-only Linear: X bf16 ~ N(0,1) clipped to [-4,4], W bf16 ~ N(0,0.02^2)."""
    cfg = 2
    x = np.clip(normal(m * k, seed_of(cfg, step, TID_X)), -4.0, 4.0)
    w = normal(k * n, seed_of(cfg, 0, TID_W), 0.02)
    return to_bf16_bits(x).reshape(m, k), to_bf16_bits(w).reshape(k, n)


def fwd_bwd_4096(m: int = 16384, k: int = 4096, n: int = 4096, step: int = 0):
    """Full fwd+bwd Linear: X ~ N(0,1), W ~ N(0,0.02^2), heavy-tailed dY; all bf16."""
    cfg = 3
    x = normal(m * k, seed_of(cfg, step, TID_X))
    w = normal(k * n, seed_of(cfg, 0, TID_W), 0.02)
    dy = heavy_tail_grad(m * n, seed_of(cfg, step, TID_DY))
    return (to_bf16_bits(x).reshape(m, k), to_bf16_bits(w).reshape(k, n),
            to_bf16_bits(dy).reshape(m, n))


def llama_sigma(step: int, steps: int = 10) -> float:
    """Activation std drifting linearly from 1.0 to 3.0 over ``steps`` steps."""
    return 1.0 + 2.0 * step / (steps - 1)


LLAMA_OUTLIER_STEP = 6
LLAMA_OUTLIER_FACTOR = 50.0


def llama_tensors(proj: str, step: int, m: int = 8192):
    """Decoder-layer Linear ``proj`` at ``step``: X bf16 [m,in] ~ N(0, sigma_t^2)
    (x50 at the outlier step), W bf16 [in,out] ~ N(0,0.02^2) fixed, dY heavy-tailed."""
    cfg = 4
    p = list(LLAMA_PROJ).index(proj) + 1
    fin, fout = LLAMA_PROJ[proj]
    sig = llama_sigma(step)
    x = normal(m * fin, seed_of(cfg, step, 10 * p + TID_X), sig)
    if step == LLAMA_OUTLIER_STEP:
        x *= np.float32(LLAMA_OUTLIER_FACTOR)
    w = normal(fin * fout, seed_of(cfg, 0, 10 * p + TID_W), 0.02)
    dy = heavy_tail_grad(m * fout, seed_of(cfg, step, 10 * p + TID_DY))
    return (to_bf16_bits(x).reshape(m, fin), to_bf16_bits(w).reshape(fin, fout),
            to_bf16_bits(dy).reshape(m, fout))


def big_cast_input(n: int = 1 << 30, step: int = 0):
    """Bandwidth stress: bf16 ~ N(0,1) with round(1e-5 n) entries at +-1000."""
    cfg = 5
    x = normal(n, seed_of(cfg, step, TID_X))
    k = int(round(1e-5 * n))
    pos = _positions(n, k, seed_of(cfg, step, TID_X))
    sgn = np.where(np.random.default_rng(seed_of(cfg, step, TID_X) + 501).random(k) < 0.5,
                   -1000.0, 1000.0).astype(np.float32)
    x[pos] = sgn
    return to_bf16_bits(x)


def small_batch(batch: int = 512, m: int = 256, k: int = 256, n: int = 256, step: int = 0):
    """Batch of small Linears: X_i ~ N(0,1) [m,k], W_i ~ N(0,0.02^2) [k,n], bf16."""
    cfg = 5
    x = normal(batch * m * k, seed_of(cfg, step, 100 + TID_X))
    w = normal(batch * k * n, seed_of(cfg, 0, 100 + TID_W), 0.02)
    return (to_bf16_bits(x).reshape(batch, m, k), to_bf16_bits(w).reshape(batch, k, n))


TID_M, TID_V, TID_G = 4, 5, 6


def adamw_state(rows: int, cols: int, step: int = 0):
    """Optimizer state of a [rows, cols] weight: fp32 master W ~ N(0, 0.02^2),
    first moment ~ N(0, 1e-3^2), second moment ~ U(0, 1e-4) (the size of squared
    gradients of about 1e-2), and a heavy-tailed bf16 gradient (dW)."""
    cfg = 6
    n = rows * cols
    w = normal(n, seed_of(cfg, 0, TID_W), 0.02).reshape(rows, cols)
    m = normal(n, seed_of(cfg, 0, TID_M), 1e-3).reshape(rows, cols)
    v = uniform(n, seed_of(cfg, 0, TID_V), 0.0, 1e-4).reshape(rows, cols)
    g = heavy_tail_grad(n, seed_of(cfg, step, TID_G))
    return w, m, v, to_bf16_bits(g).reshape(rows, cols)
