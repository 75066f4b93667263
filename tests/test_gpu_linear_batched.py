"""GPU parity of the one-launch forward step of a batch of small Linears
(``fp8ds_linear_batched``): casts of X_i and W_i with their delayed scales, the
exact-datapath products with the dequant epilogue, and the scaling-state update
of all 2B tensors, against the oracle on every element.

Shapes span one and two K stages, K ending inside a stage, M and N below one
output tile, and the smallest shape (16^3); formats cover the four (X, W)
pairs.  Inputs hold saturating outliers, and one problem holds a NaN and an
infinity, so that its amax is NaN and its next scale falls back to 1.0.

Outputs compared: codes of X_i and W_i (every byte), saturation counts, amax and
scale snapshots (bits), every output element (1e-5 * sum|ab| + 1 BF16 ulp),
output amax (bits, against the device's own output), histories, cursors and
next scales (bits) over three steps.  The fused step is also compared with the
four-launch sequence of the same library (batched casts, batched GEMM, scale
update), which must give identical bits everywhere.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import delayed_scaling_gemm_amd as dsg  # noqa: E402
import workloads  # noqa: E402
from delayed_scaling_gemm_amd.linear import BatchedDelayedScalingLinear  # noqa: E402
from oracle import amax as oamax  # noqa: E402
from oracle import bf16 as obf16  # noqa: E402
from oracle import fp8 as ofp8  # noqa: E402
from oracle import gemm as ogemm  # noqa: E402
from oracle.scaling import ScalingState  # noqa: E402
from tests.parity import bf16_bits, check_bf16_out, f32_bits  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def batch_inputs(B, M, N, K, step, seed, specials=True):
    """X_i ~ N(0, 1) with 0.1% outliers of 1e3..1e4 (they saturate E4M3 once the
    history scale applies), W_i ~ N(0, 0.02^2); problem 1 (if any) holds a NaN
    and an infinity in X at step 1."""
    x = workloads.normal(B * M * K, seed + 1000 * step)
    x = workloads.with_outliers(x, 1e-3, 1e3, 1e4, seed + 1000 * step + 7)
    w = workloads.normal(B * K * N, seed + 1000 * step + 3, 0.02)
    xb = workloads.to_bf16_bits(x).reshape(B, M, K)
    wb = workloads.to_bf16_bits(w).reshape(B, K, N)
    if specials and step == 1 and B > 1:
        xb[1, 0, 0] = 0x7FC0  # NaN
        xb[1, M - 1, K - 1] = 0xFF80  # -inf
    return xb, wb


def oracle_check(lin, out, xb, wb, states, fx, fw, what):
    """Every output of one step against the oracle; advances `states`."""
    B = xb.shape[0]
    xq, wq = out["xq"].cpu().numpy(), out["wq"].cpu().numpy()
    y = bf16_bits(out["y"])
    amy = lin.amax_y.cpu().numpy().view(np.uint32)
    am = lin.amax.cpu().numpy().view(np.uint32)
    su = lin.scale_used.cpu().numpy().view(np.uint32)
    sat = lin.sat.cpu().numpy()
    for b in range(B):
        sx, sw = states[b], states[B + b]
        vx, vw = obf16.widen(xb[b]), obf16.widen(wb[b])
        cx, nx = ofp8.cast(vx, sx.scale, fx)
        cw, nw = ofp8.cast(vw, sw.scale, fw)
        assert np.array_equal(xq[b], cx), f"{what}: xq[{b}]"
        assert np.array_equal(wq[b], cw), f"{what}: wq[{b}]"
        assert sat[b] == nx and sat[B + b] == nw, (what, b, sat[b], nx, sat[B + b], nw)
        assert su[b] == f32_bits(sx.scale) and su[B + b] == f32_bits(sw.scale), (what, b)
        ax, aw = oamax.amax(vx), oamax.amax(vw)
        assert am[b] == f32_bits(ax) and am[B + b] == f32_bits(aw), (what, b)
        if not np.isnan(ax):
            acc, sum_abs = ogemm.gemm_exact(cx, fx, 0, cw, fw, 0)
            y_ref = ogemm.dequant_to_bf16(acc, sx.scale, sw.scale)
            check_bf16_out(y[b], acc, sum_abs, y_ref,
                           1.0 / float(ogemm.dequant_scale(sx.scale, sw.scale)), f"{what}: y[{b}]")
        else:  # a NaN code in X_b: its row of Y is NaN, the other rows as usual
            rows = np.unique(np.nonzero(np.isnan(ofp8.decode(cx, fx)))[0])
            keep = np.setdiff1d(np.arange(cx.shape[0]), rows)
            acc, sum_abs = ogemm.gemm_exact(cx[keep], fx, 0, cw, fw, 0)
            y_ref = ogemm.dequant_to_bf16(acc, sx.scale, sw.scale)
            check_bf16_out(y[b][keep], acc, sum_abs, y_ref,
                           1.0 / float(ogemm.dequant_scale(sx.scale, sw.scale)), f"{what}: y[{b}]")
            assert np.isnan(obf16.widen(y[b][rows])).all(), f"{what}: NaN rows of y[{b}]"
        assert amy[b] == f32_bits(ogemm.output_amax(y[b])) or (
            np.isnan(ogemm.output_amax(y[b])) and amy[b] == 0x7FC00000), (what, b)
        sx.update(ax, lin.algo, lin.margin)
        sw.update(aw, lin.algo, lin.margin)
    s = lin.scale.cpu().numpy()
    assert np.array_equal(s.view(np.uint32),
                          np.array([st.scale for st in states], np.float32).view(np.uint32)), what
    h = lin.history.cpu().numpy()
    assert np.array_equal(h.view(np.uint32),
                          np.stack([st.history for st in states]).view(np.uint32)), what
    assert np.array_equal(lin.cursor.cpu().numpy(), [st.cursor for st in states]), what


CASES = [
    # B, M, N, K, fx, fw, hist_len, algo, margin
    (6, 256, 256, 256, dsg.E4M3, dsg.E4M3, 16, dsg.ALGO_MAX, 0),
    (5, 48, 80, 144, dsg.E5M2, dsg.E4M3, 4, dsg.ALGO_MAX, 1),
    (4, 256, 128, 96, dsg.E4M3, dsg.E5M2, 1024, dsg.ALGO_MOST_RECENT, 0),
    (3, 112, 256, 240, dsg.E5M2, dsg.E5M2, 1, dsg.ALGO_MAX, 2),
    (9, 16, 16, 16, dsg.E4M3, dsg.E4M3, 16, dsg.ALGO_MAX, 0),
    (2, 160, 208, 128, dsg.E4M3, dsg.E4M3, 7, dsg.ALGO_MAX, 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:4])) + f"_f{c[4]}{c[5]}")
def test_fused_step_vs_oracle(case):
    B, M, N, K, fx, fw, L, algo, margin = case
    print(f"[linear_batched] {case}", flush=True)
    lin = BatchedDelayedScalingLinear(B, hist_len=L, algo=algo, margin=margin, fmt=fx)
    states = [ScalingState(fx if t < B else fw, L) for t in range(2 * B)]
    for step in range(3):
        xb, wb = batch_inputs(B, M, N, K, step, seed=17 + B)
        x, w = dev_bf16(xb), dev_bf16(wb)
        assert lin.takes_fused(x, w)
        out = step_formats(lin, x, w, fx, fw)
        torch.cuda.synchronize()
        oracle_check(lin, out, xb, wb, states, fx, fw, f"{case} step {step}")


def step_formats(lin, x, w, fx, fw):
    """lin.step with distinct X and W formats (the Linear itself uses one format)."""
    B, M, K = x.shape
    N = w.shape[2]
    xq = lin._buf("xq", (B, M, K), torch.uint8)
    wq = lin._buf("wq", (B, K, N), torch.uint8)
    y = lin._buf("y", (B, M, N), torch.bfloat16)
    dsg.fp8ds_linear_batched(x, w, fx, fw, lin.history, lin.cursor, lin.algo, lin.margin,
                             lin.scale, lin.amax, y, scale_used=lin.scale_used,
                             sat_count=lin.sat, xq=xq, wq=wq, amax_y=lin.amax_y)
    return {"xq": xq, "wq": wq, "y": y}


@pytest.mark.parametrize("shape", [(512, 256, 256, 256), (259, 256, 256, 256), (7, 80, 144, 208)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fused_equals_four_launches(shape):
    """The fused step and the four-launch sequence give identical bits (batches
    beyond the CU count take two problems per workgroup, an odd one leaves the
    last workgroup a single problem)."""
    B, M, N, K = shape
    print(f"[linear_batched] fused vs four launches {shape}", flush=True)
    fused = BatchedDelayedScalingLinear(B, hist_len=16)
    split = BatchedDelayedScalingLinear(B, hist_len=16, fused=False)
    for step in range(3):
        xb, wb = batch_inputs(B, M, N, K, step, seed=91)
        x, w = dev_bf16(xb), dev_bf16(wb)
        assert fused.takes_fused(x, w) and not split.takes_fused(x, w)
        a = fused.step(x, w)
        b = split.step(x, w)
        torch.cuda.synchronize()
        for k in ("xq", "wq"):
            assert torch.equal(a[k], b[k]), (step, k)
        assert torch.equal(a["y"].view(torch.int16), b["y"].view(torch.int16)), step
        for name in ("amax", "scale_used", "scale", "history", "amax_y"):
            ta, tb = getattr(fused, name), getattr(split, name)
            assert torch.equal(ta.view(torch.int32), tb.view(torch.int32)), (step, name)
        assert torch.equal(fused.cursor, split.cursor) and torch.equal(fused.sat, split.sat), step


def test_nullable_outputs():
    """Without xq, wq, scale_used, sat_count and amax_y the remaining outputs are
    unchanged."""
    B, M, N, K = 4, 64, 96, 192
    xb, wb = batch_inputs(B, M, N, K, 0, seed=5)
    x, w = dev_bf16(xb), dev_bf16(wb)
    full = BatchedDelayedScalingLinear(B, hist_len=8)
    bare = BatchedDelayedScalingLinear(B, hist_len=8)
    for step in range(2):
        a = full.step(x, w)
        y = torch.empty(B, M, N, dtype=torch.bfloat16, device=DEV)
        dsg.fp8ds_linear_batched(x, w, dsg.E4M3, dsg.E4M3, bare.history, bare.cursor, bare.algo,
                                 bare.margin, bare.scale, bare.amax, y)
        torch.cuda.synchronize()
        assert torch.equal(a["y"].view(torch.int16), y.view(torch.int16)), step
        for name in ("amax", "scale", "history", "cursor"):
            assert torch.equal(getattr(full, name), getattr(bare, name)), (step, name)


def test_rejects_unsupported_shapes():
    B = 2
    lin = BatchedDelayedScalingLinear(B, hist_len=4)
    for (M, N, K) in ((272, 16, 16), (16, 24, 16), (16, 16, 0)):
        x = torch.zeros(B, M, K, dtype=torch.bfloat16, device=DEV)
        w = torch.zeros(B, K, N, dtype=torch.bfloat16, device=DEV)
        y = torch.empty(B, M, N, dtype=torch.bfloat16, device=DEV)
        with pytest.raises(dsg.Fp8dsError) as e:
            dsg.fp8ds_linear_batched(x, w, dsg.E4M3, dsg.E4M3, lin.history, lin.cursor, lin.algo,
                                     lin.margin, lin.scale, lin.amax, y)
        assert e.value.status == -2
        assert not lin.takes_fused(x, w)


def test_prepared_launches_equal_step():
    """dsg.prepare records the step's one call once; replaying it gives what
    calling step() each time gives (states, codes and outputs, bit for bit)."""
    B, M, N, K = 24, 256, 256, 256
    prepared = BatchedDelayedScalingLinear(B, hist_len=4)
    called = BatchedDelayedScalingLinear(B, hist_len=4)
    xb, wb = batch_inputs(B, M, N, K, 0, seed=3)
    x, w = dev_bf16(xb), dev_bf16(wb)
    launch = dsg.prepare(lambda: prepared.step(x, w))
    torch.cuda.synchronize()
    assert torch.equal(prepared.cursor, torch.zeros_like(prepared.cursor))  # nothing launched
    for step in range(5):
        launch()
        out = called.step(x, w)
        torch.cuda.synchronize()
        for name in ("scale", "scale_used", "history", "amax", "amax_y"):
            assert torch.equal(getattr(prepared, name).view(torch.int32),
                               getattr(called, name).view(torch.int32)), (step, name)
        assert torch.equal(prepared.cursor, called.cursor), step
        for k in ("xq", "wq"):
            assert torch.equal(prepared._bufs[k], out[k]), (step, k)
        assert torch.equal(prepared._bufs["y"].view(torch.int16), out["y"].view(torch.int16)), step
