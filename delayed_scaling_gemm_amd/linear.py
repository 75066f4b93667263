"""One FP8 delayed-scaling Linear step composed from the C-ABI calls.

Host-side orchestration only (every arithmetic step runs in the HIP library):

  fwd:  cast X (E4M3), cast W (E4M3)          -> Xq, Wq (+ Wq^T), amax_X, amax_W, snapshots
        Y  = Xq . Wq         (NT on Wq^T)     -> BF16 Y + amax_Y  (FP8 matrix instructions
                                                                   when K >= 4096)
  bwd:  cast dY (E5M2)                        -> dYq, amax_dY
        dX = dYq . Wq^T      (NT)             -> BF16 dX           (exact F16-widened path)
        dW = Xq^T . dYq      (TN)             -> BF16 dW           (exact F16-widened path)
  end:  one scale update over the X, W, dY histories -> scales of the next step
        (the same launch zeroes the accumulators the next step's casts and
        GEMMs combine into, so the step runs no reset kernels)
  opt:  (optional) adamw_step: fused AdamW on the fp32 master weights with this
        step's dW, writing Wq, Wq^T, amax_W and the W scale snapshot of the next
        step, whose forward then skips the W cast

This is the HYBRID recipe ("LLM FP8 微调上线生产实战" §核心原理: E4M3 for forward
tensors, E5M2 for gradients) with delayed scaling: each cast uses the scale that
the previous steps' amax history produced, and the GEMMs use the snapshot of the
scale their operands were cast with ("FP8 混合精度训练工程实践" §四 动态缩放).
W is stored [in, out].  The cast of W also writes the transposed bytes Wq^T
[out, in], so the forward product runs with both operands K-contiguous (the
GEMM's fastest layout); the backward products reuse the forward FP8 bytes of X
and W.

Everything stays on the device and on one stream: there is no host
synchronisation inside a step.
"""

from __future__ import annotations

import torch

from . import (ALGO_MAX, E4M3, E5M2, HEALTH_COUNTS, HEALTH_NAMES, MMA_EXACT, MMA_FP8, OP_N, OP_T,
               fp8ds_adamw, fp8ds_cast_acc, fp8ds_cast_health, fp8ds_cast_mx, fp8ds_gemm,
               fp8ds_gemm_acc, fp8ds_gemm_mx, fp8ds_scale_update, fp8ds_scale_update_clear)

X, W, DY = 0, 1, 2
# shortest forward reduction that runs on the FP8 matrix instructions by default
FP8_FWD_MIN_K = 4096


class DelayedScalingLinear:
    """Delayed-scaling state of one Linear (history ring, cursor and scale per
    tensor X, W, dY) and its fwd(+bwd) step."""

    def __init__(self, hist_len: int = 16, algo: int = ALGO_MAX, margin: int = 0,
                 fmts=(E4M3, E4M3, E5M2), device="cuda", health: bool = False,
                 health_every: int = 1, mma_fwd=None, mma_bwd: int = MMA_EXACT):
        # GEMM datapaths (fp8ds_mma) of the forward and of the two backward
        # products.  mma_fwd=None picks per call: gfx950's FP8 matrix
        # instructions when the reduction is at least FP8_FWD_MIN_K long, else the
        # exact F16-widened path.  The FP8 instructions add each group of 8
        # products at a fixed point 13 bits below the group's largest, so the
        # error relative to sum|ab| falls with the number of groups: on the
        # forward operands (near-normal activations, N(0, 0.02^2) weights, both
        # E4M3) it stays within 1e-5 * sum|ab| at K >= 4096 (measured max 2.3e-6
        # over the configurations' forwards, checked element by element), but at
        # K = 256 it reached 1.1e-5 on one of 33.5M outputs.  The bound is a
        # property of the data, not of the datapath: heavy-tailed E5M2 gradients
        # exceed it at any K (up to ~2e-3), so both backward products stay exact.
        self.mma_fwd = mma_fwd
        self.mma_bwd = mma_bwd
        self.health = health
        # the counting cast costs ~30% more than the plain one on large tensors:
        # run it on every `health_every`-th step only (the pages check every 100)
        self.health_every = max(1, int(health_every))
        self.steps = 0
        self.health_step = -1  # step whose counts `counts` holds
        self.hist_len = hist_len
        self.algo = algo
        self.margin = margin
        self.fmts = tuple(fmts)
        self.device = torch.device(device)
        f32 = dict(dtype=torch.float32, device=self.device)
        self.history = torch.zeros(3, hist_len, **f32)
        self.cursor = torch.zeros(3, dtype=torch.int32, device=self.device)
        self.scale = torch.ones(3, **f32)
        self.scale_used = torch.zeros(3, **f32)
        # Per-step accumulators, two sets used on alternate steps: the casts and
        # GEMMs of step t combine into set t % 2 (fp8ds_cast_acc, fp8ds_gemm_acc),
        # and the scale update that ends step t zeroes set (t + 1) % 2 for the
        # next step, so no reset kernel runs inside a step and step t's values
        # stay readable until the end of step t + 1.  Words of a set: amax of X,
        # W, dY (fp32) at 0..2, amax of Y at 3, of dW at 4, saturation counts
        # of X, W, dY (int64) at 8..13.
        self._acc = torch.zeros(2, 16, dtype=torch.int32, device=self.device)
        self._w_prepared = None  # master weights whose FP8 copy adamw_step wrote
        self.w_counts_valid = True
        # health=True: each cast also counts saturated, NaN, Inf, zero and
        # top-binade values (fp8ds_cast_health) into counts[X | W | DY]
        self.counts = (torch.zeros(3, HEALTH_COUNTS, dtype=torch.int64, device=self.device)
                       if health else None)
        self._bufs = {}

    # views of an accumulator set
    def _amax_of(self, slot):
        return self._acc[slot, 0:3].view(torch.float32)

    def _sat_of(self, slot):
        return self._acc[slot, 8:14].view(torch.int64)

    @property
    def _slot(self):
        """The accumulator set of the step that runs next."""
        return self.steps & 1

    @property
    def amax(self):
        """amax of X, W and dY of the last step (fp32 [3], device)."""
        return self._amax_of((self.steps - 1) & 1)

    @property
    def sat(self):
        """Saturation counts of the last step's casts (int64 [3], device)."""
        return self._sat_of((self.steps - 1) & 1)

    @property
    def amax_y(self):
        """Fused output amax of the last step's forward GEMM (fp32 [1], device)."""
        return self._acc[(self.steps - 1) & 1, 3:4].view(torch.float32)

    @property
    def amax_dw(self):
        """Fused output amax of the last step's dW GEMM (fp32 [1], device; the
        optimizer's skip rule)."""
        return self._acc[(self.steps - 1) & 1, 4:5].view(torch.float32)

    def _cast(self, t, x, q, q_t, stream):
        s, su = self.scale, self.scale_used
        am, sat = self._amax_of(self._slot), self._sat_of(self._slot)
        if self.health and self.steps % self.health_every == 0:
            self.health_step = self.steps
            fp8ds_cast_health(x, self.fmts[t], s[t:t + 1], q, self.counts[t], q_t, su[t:t + 1],
                              am[t:t + 1], stream)
        else:
            fp8ds_cast_acc(x, self.fmts[t], s[t:t + 1], q, q_t, su[t:t + 1], am[t:t + 1],
                           sat[t:t + 1], stream)

    def fwd_datapath(self, K: int) -> int:
        """The forward GEMM's datapath for a reduction of length K."""
        if self.mma_fwd is not None:
            return self.mma_fwd
        return MMA_FP8 if K >= FP8_FWD_MIN_K else MMA_EXACT

    def health_report(self):
        """Host copy of the counts of the last counted step:
        {"step": i, "x"|"w"|"dy": {name: count}} (synchronises), or None."""
        if self.counts is None or self.health_step < 0:
            return None
        c = self.counts.cpu().tolist()
        rep = {k: dict(zip(HEALTH_NAMES, c[i])) for i, k in enumerate(("x", "w", "dy"))}
        if not self.w_counts_valid:
            rep["w"] = None  # the weights' cast was fused into adamw_step: not counted
        rep["step"] = self.health_step
        return rep

    def _buf(self, name, shape, dtype):
        t = self._bufs.get(name)
        if t is None or tuple(t.shape) != tuple(shape) or t.dtype != dtype:
            t = torch.empty(shape, dtype=dtype, device=self.device)
            self._bufs[name] = t
        return t

    def state(self):
        """Copies of the scaling state (history, cursor, scale)."""
        return self.history.clone(), self.cursor.clone(), self.scale.clone()

    # Checkpoint / resume ("LLM FP8 微调上线生产实战" §核心原理 "Delayed Scaling 用
    # 历史换取稳定性": the scale of a step comes from the amax history; a restore
    # that keeps the scale but drops the history changes the scales that follow).
    # The state is exactly the recipe plus, per tensor, the history ring, its
    # cursor and the current scale.

    def state_dict(self) -> dict:
        """Host copies of the scaling state and the recipe."""
        return {"history": self.history.detach().cpu().clone(),
                "cursor": self.cursor.detach().cpu().clone(),
                "scale": self.scale.detach().cpu().clone(),
                "recipe": torch.tensor([self.hist_len, self.algo, self.margin, *self.fmts],
                                       dtype=torch.int64)}

    def load_state_dict(self, d: dict):
        """Restore a state saved by :meth:`state_dict` (the recipe must match)."""
        recipe = [int(v) for v in d["recipe"].tolist()]
        if recipe != [self.hist_len, self.algo, self.margin, *self.fmts]:
            raise ValueError(f"recipe {recipe} does not match this Linear's "
                             f"{[self.hist_len, self.algo, self.margin, *self.fmts]}")
        for name in ("history", "cursor", "scale"):
            src, dst = d[name], getattr(self, name)
            if tuple(src.shape) != tuple(dst.shape) or src.dtype != dst.dtype:
                raise ValueError(f"{name}: {tuple(src.shape)} {src.dtype} vs "
                                 f"{tuple(dst.shape)} {dst.dtype}")
            dst.copy_(src.to(dst.device))

    def save(self, path: str):
        torch.save(self.state_dict(), path)

    def load(self, path: str):
        self.load_state_dict(torch.load(path, map_location="cpu", weights_only=True))

    def step(self, x, w, dy=None, stream=None):
        """One step; returns a dict with the FP8 operands and the BF16 outputs."""
        M, K = x.shape
        K2, N = w.shape
        assert K == K2, "x is [M, in] and w is [in, out]"
        u8 = torch.uint8
        xq = self._buf("xq", (M, K), u8)
        wq = self._buf("wq", (K, N), u8)
        wqt = self._buf("wqt", (N, K), u8)
        y = self._buf("y", (M, N), torch.bfloat16)
        slot = self._slot
        s, su, am = self.scale, self.scale_used, self._amax_of(slot)
        amax_y = self._acc[slot, 3:4].view(torch.float32)
        amax_dw = self._acc[slot, 4:5].view(torch.float32)
        self._cast(X, x, xq, None, stream)
        if self._w_prepared is not None and self._w_prepared is w:
            # adamw_step already wrote Wq, Wq^T, amax_W and the W snapshot
            if self.health and self.steps % self.health_every == 0:
                self.w_counts_valid = False
        else:
            if self.health and self.steps % self.health_every == 0:
                self.w_counts_valid = True
            self._cast(W, w, wq, wqt, stream)
        self._w_prepared = None
        # Y[M, N] = Xq[M, K] . Wq[K, N], with Wq^T stored [N, K] -> op T
        fp8ds_gemm_acc(OP_N, OP_T, M, N, K, xq, self.fmts[X], K, su[X:X + 1], wqt, self.fmts[W],
                       K, su[W:W + 1], y, N, amax_y, stream, mma=self.fwd_datapath(K))
        out = {"xq": xq, "wq": wq, "wqt": wqt, "y": y}
        n_upd = 2
        if dy is not None:
            assert tuple(dy.shape) == (M, N)
            dyq = self._buf("dyq", (M, N), u8)
            dx = self._buf("dx", (M, K), torch.bfloat16)
            dw = self._buf("dw", (K, N), torch.bfloat16)
            self._cast(DY, dy, dyq, None, stream)
            # dX[M, K] = dYq[M, N] . Wq^T   (Wq stored [K, N] = [N' x K'] -> op T)
            fp8ds_gemm(OP_N, OP_T, M, K, N, dyq, self.fmts[DY], N, su[DY:DY + 1], wq, self.fmts[W],
                       N, su[W:W + 1], dx, K, None, stream, mma=self.mma_bwd)
            # dW[K, N] = Xq^T . dYq         (Xq stored [M, K] = [K' x M'] -> op T)
            fp8ds_gemm_acc(OP_T, OP_N, K, N, M, xq, self.fmts[X], K, su[X:X + 1], dyq,
                           self.fmts[DY], N, su[DY:DY + 1], dw, N, amax_dw, stream,
                           mma=self.mma_bwd)
            out.update(dyq=dyq, dx=dx, dw=dw)
            n_upd = 3
        # the scale update also zeroes the next step's accumulator set
        fp8ds_scale_update_clear(self.history[:n_upd], self.cursor[:n_upd], am[:n_upd],
                                 self.fmts[:n_upd], self.algo, self.margin, s[:n_upd],
                                 self._acc[slot ^ 1], None, stream)
        self.steps += 1
        return out

    def adamw_step(self, w, m, v, lr, step, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                   grad_scale=1.0, stream=None):
        """Fused AdamW on the fp32 master weights ``w`` [in, out] and moments ``m``,
        ``v`` with the dW of the last :meth:`step` (step count ``step`` >= 1).

        The same kernel casts the new weights with the W scale the last step's
        scale update produced, into the Wq / Wq^T buffers, and records their amax:
        the next :meth:`step` given this ``w`` skips its W cast ("算子与编译器：
        FP8 训练与优化器 Kernel" §FP8 训练主路径图: fused optimizer -> master weight ->
        cast to FP8).  The result is bit-identical to updating ``w`` and casting it
        at the start of the next step.  A non-finite dW amax skips the update
        (weights and moments stay; their FP8 copy is still made)."""
        dw = self._bufs.get("dw")
        if dw is None or tuple(dw.shape) != tuple(w.shape):
            raise RuntimeError("adamw_step needs the dW of a preceding fwd+bwd step of this shape")
        if w.dtype != torch.float32:
            raise TypeError("the master weights must be fp32")
        K, N = w.shape
        wq = self._buf("wq", (K, N), torch.uint8)
        wqt = self._buf("wqt", (N, K), torch.uint8)
        # the new weights' amax and saturation go into the next step's set
        s, su = self.scale, self.scale_used
        am, sat = self._amax_of(self._slot), self._sat_of(self._slot)
        fp8ds_adamw(w, dw, m, v, lr, beta1, beta2, eps, weight_decay, step, grad_scale=grad_scale,
                    grad_amax=self.amax_dw, fmt=self.fmts[W], scale=s[W:W + 1], q=wq, q_t=wqt,
                    scale_used=su[W:W + 1], amax=am[W:W + 1], sat_count=sat[W:W + 1],
                    stream=stream)
        self._w_prepared = w


class BatchedDelayedScalingLinear:
    """Forward pass of ``batch`` independent small Linears, each with its own
    delayed-scaling state for X and W.

    Shapes with M, N, K multiples of 16 up to 256 (BF16 inputs, exact datapath)
    take one launch per step (``fp8ds_linear_batched``: casts, products and the
    scale update of a problem in one workgroup).  Other shapes, FP32 inputs, the
    FP8 datapath or ``fused=False`` take four: the batched casts of all X and of
    all W, one batched GEMM, one scale update over all 2 * batch histories.
    Both give the same results.

    Histories are laid out [X_0 .. X_{B-1}, W_0 .. W_{B-1}].
    """

    def __init__(self, batch: int, hist_len: int = 16, algo: int = ALGO_MAX, margin: int = 0,
                 fmt: int = E4M3, device="cuda", mma: int = MMA_EXACT, fused: bool = True):
        # exact datapath by default: with K = 256 the FP8 matrix instructions
        # missed 1e-5 * sum|ab| on one of 33.5M outputs of the 512-problem batch
        self.mma = mma
        self.fused = fused
        self.batch = batch
        self.hist_len = hist_len
        self.algo = algo
        self.margin = margin
        self.fmt = fmt
        self.device = torch.device(device)
        f32 = dict(dtype=torch.float32, device=self.device)
        n = 2 * batch
        self.history = torch.zeros(n, hist_len, **f32)
        self.cursor = torch.zeros(n, dtype=torch.int32, device=self.device)
        self.scale = torch.ones(n, **f32)
        self.scale_used = torch.zeros(n, **f32)
        self.amax = torch.zeros(n, **f32)
        self.sat = torch.zeros(n, dtype=torch.int64, device=self.device)
        self.amax_y = torch.zeros(batch, **f32)
        self._bufs = {}

    def _buf(self, name, shape, dtype):
        t = self._bufs.get(name)
        if t is None or tuple(t.shape) != tuple(shape) or t.dtype != dtype:
            t = torch.empty(shape, dtype=dtype, device=self.device)
            self._bufs[name] = t
        return t

    def takes_fused(self, x, w) -> bool:
        """Whether ``step`` runs as the one-launch fused kernel for these inputs."""
        B, M, K = x.shape
        N = w.shape[2]
        dims = all(16 <= v <= 256 and v % 16 == 0 for v in (M, N, K))
        return (self.fused and self.mma == MMA_EXACT and dims and B <= 65535
                and x.dtype == torch.bfloat16 and w.dtype == torch.bfloat16
                and x.is_contiguous() and w.is_contiguous())

    def step(self, x, w, stream=None):
        """x: [B, M, K], w: [B, K, N] (bf16 or fp32, contiguous) -> dict of xq, wq, y."""
        from . import fp8ds_cast_batched, fp8ds_gemm_batched, fp8ds_linear_batched

        B, M, K = x.shape
        B2, K2, N = w.shape
        assert B == B2 == self.batch and K == K2
        xq = self._buf("xq", (B, M, K), torch.uint8)
        wq = self._buf("wq", (B, K, N), torch.uint8)
        y = self._buf("y", (B, M, N), torch.bfloat16)
        s, su, am, sat = self.scale, self.scale_used, self.amax, self.sat
        if self.takes_fused(x, w):
            fp8ds_linear_batched(x, w, self.fmt, self.fmt, self.history, self.cursor, self.algo,
                                 self.margin, s, am, y, scale_used=su, sat_count=sat, xq=xq,
                                 wq=wq, amax_y=self.amax_y, stream=stream)
            return {"xq": xq, "wq": wq, "y": y}
        fp8ds_cast_batched(x, self.fmt, s[:B], xq, su[:B], am[:B], sat[:B], stream)
        fp8ds_cast_batched(w, self.fmt, s[B:], wq, su[B:], am[B:], sat[B:], stream)
        fp8ds_gemm_batched(OP_N, OP_N, M, N, K, B, xq, self.fmt, K, M * K, su[:B], wq, self.fmt,
                           N, K * N, su[B:], y, N, M * N, self.amax_y, stream, mma=self.mma)
        fp8ds_scale_update(self.history, self.cursor, am, [self.fmt] * (2 * B), self.algo,
                           self.margin, s, None, stream)
        return {"xq": xq, "wq": wq, "y": y}


class MXLinear:
    """The same Linear step in MXFP8 ("FP8 混合精度训练工程实践" §九: blocks of 32
    values along the contraction sharing an E8M0 scale).  There is no scaling
    state: every block's scale comes from the block itself.  Each tensor is cast
    once with its transposed copy (fp8ds_cast_mx), which gives every product
    both operands blocked along its own K:

      Y  = X W        fp8ds_gemm_mx(q of X,     q_t of W)    K = in
      dX = dY W^T     fp8ds_gemm_mx(q of dY,    q of W)      K = out
      dW = X^T dY     fp8ds_gemm_mx(q_t of X,   q_t of dY)   K = tokens

    Shapes: tokens, in and out multiples of 128.  ``mma`` picks the GEMM
    datapath (exact BF16 widening, or the block-scaled FP8 instruction)."""

    def __init__(self, fmts=(E4M3, E4M3, E5M2), device="cuda", mma: int = MMA_EXACT):
        self.fmts = tuple(fmts)
        self.device = torch.device(device)
        self.mma = mma
        self._bufs = {}
        self.amax_y = torch.zeros(1, dtype=torch.float32, device=self.device)

    def _buf(self, name, shape, dtype):
        b = self._bufs.get(name)
        if b is None or tuple(b.shape) != tuple(shape) or b.dtype != dtype:
            b = torch.empty(shape, dtype=dtype, device=self.device)
            self._bufs[name] = b
        return b

    def _cast(self, t, name, x, stream):
        r, c = x.shape
        u8 = torch.uint8
        q, s = self._buf(name + "q", (r, c), u8), self._buf(name + "s", (r, c // 32), u8)
        qt, st = self._buf(name + "qt", (c, r), u8), self._buf(name + "st", (c, r // 32), u8)
        fp8ds_cast_mx(x, self.fmts[t], q, s, qt, st, stream)
        return q, s, qt, st

    def _gemm(self, m, n, k, a, sa, fa, b, sb, fb, out, stream, amax=None):
        fp8ds_gemm_mx(m, n, k, a, fa, k, sa, k // 32, b, fb, k, sb, k // 32, out, n, amax, stream,
                      self.mma)

    def step(self, x, w, dy=None, stream=None):
        """x [M, K], w [K, N] (and dy [M, N]), BF16 or FP32 on the device.
        Returns the BF16 outputs y (and dx, dw) and the MX copies of the inputs."""
        M, K = x.shape
        N = w.shape[1]
        bf = torch.bfloat16
        xq, xs, xqt, xst = self._cast(X, "x", x, stream)
        wq, ws, wqt, wst = self._cast(W, "w", w, stream)
        y = self._buf("y", (M, N), bf)
        self._gemm(M, N, K, xq, xs, self.fmts[X], wqt, wst, self.fmts[W], y, stream, self.amax_y)
        out = {"y": y, "xq": xq, "xs": xs, "xqt": xqt, "xst": xst, "wq": wq, "ws": ws,
               "wqt": wqt, "wst": wst}
        if dy is not None:
            dyq, dys, dyqt, dyst = self._cast(DY, "dy", dy, stream)
            dx, dw = self._buf("dx", (M, K), bf), self._buf("dw", (K, N), bf)
            self._gemm(M, K, N, dyq, dys, self.fmts[DY], wq, ws, self.fmts[W], dx, stream)
            self._gemm(K, N, M, xqt, xst, self.fmts[X], dyqt, dyst, self.fmts[DY], dw, stream)
            out.update(dx=dx, dw=dw, dyq=dyq, dys=dys, dyqt=dyqt, dyst=dyst)
        return out
