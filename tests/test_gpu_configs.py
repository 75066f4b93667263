"""GPU parity of the benchmark-scale configurations, at their full sizes:

* the forward-only 8192 x 4096 x 4096 Linear with a 1024-entry history;
* the decoder-layer projections (q, k, v, o, gate, up, down) at M = 8192 tokens over
  10 steps of drifting activations with the 50x outlier batch at step 6, under the
  `max` and `most_recent` window reductions;
* the 2^30-element stress cast at its second step (scale from the history);
* 512 independent 256^3 Linears with per-problem scales, checked everywhere.

amax, scales, histories, cursors and saturation counts are exact against the
oracle on the whole tensors; cast bytes on samples; GEMM outputs on sampled rows
(the oracle computes those rows exactly), output amax exactly against the GPU's
own full output.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import delayed_scaling_gemm_amd as dsg  # noqa: E402
import workloads  # noqa: E402
from delayed_scaling_gemm_amd.linear import (BatchedDelayedScalingLinear,  # noqa: E402
                                             DelayedScalingLinear)
from oracle import amax as oamax  # noqa: E402
from oracle import bf16 as obf16  # noqa: E402
from oracle import fp8 as ofp8  # noqa: E402
from oracle import gemm as ogemm  # noqa: E402
from oracle.scaling import ScalingState  # noqa: E402
from tests.parity import band_rows, bf16_bits, check_bf16_out, f32_bits  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def check_sampled_cast(q_dev, bits, scale, fmt, rng, n=1 << 16, what=""):
    flat = bits.ravel()
    pos = rng.choice(flat.size, min(n, flat.size), replace=False)
    codes, _ = ofp8.cast(obf16.widen(flat[pos]), np.float32(scale), fmt)
    got = q_dev.reshape(-1)[torch.from_numpy(pos).to(DEV)].cpu().numpy()
    assert np.array_equal(got, codes), what


def check_gemm_rows(gpu_out, a_codes, fa, opa, b_codes, fb, opb, sa, sb, rows, what):
    """Oracle GEMM on output rows `rows` only (A as stored, op N or T)."""
    a_rows = a_codes[rows] if opa == dsg.OP_N else a_codes[:, rows].T
    acc, sum_abs = ogemm.gemm_exact(np.ascontiguousarray(a_rows), fa, 0, b_codes, fb, opb)
    y_ref = ogemm.dequant_to_bf16(acc, sa, sb)
    yb = bf16_bits(gpu_out[torch.from_numpy(rows).to(DEV)])
    check_bf16_out(yb, acc, sum_abs, y_ref, 1.0 / float(ogemm.dequant_scale(sa, sb)), what)


def compare_state(lin, states, names):
    h = lin.history.cpu().numpy()
    c = lin.cursor.cpu().numpy()
    s = lin.scale.cpu().numpy()
    for i, nm in enumerate(names):
        st = states[nm]
        assert np.array_equal(h[i].view(np.uint32), st.history.view(np.uint32)), nm
        assert c[i] == st.cursor, nm
        assert f32_bits(s[i]) == f32_bits(st.scale), (nm, s[i], st.scale)


def test_forward_linear_4096_history_1024():
    """Forward-only Linear in = out = 4096, M = 8192, E4M3 both operands, history
    1024: two steps (scale 1.0, then the history scale)."""
    L = 1024
    lin = DelayedScalingLinear(hist_len=L, algo=dsg.ALGO_MAX, margin=0)
    states = {"x": ScalingState(ofp8.E4M3, L), "w": ScalingState(ofp8.E4M3, L)}
    rng = np.random.default_rng(2)
    for step in range(2):
        xb, wb = workloads.forward_4096(step=step)
        print(f"[forward_4096] step {step}", flush=True)
        out = lin.step(dev_bf16(xb), dev_bf16(wb))
        torch.cuda.synchronize()
        for i, (nm, bits, key) in enumerate((("x", xb, "xq"), ("w", wb, "wq"))):
            st = states[nm]
            assert f32_bits(lin.scale_used[i].item()) == f32_bits(st.scale)
            check_sampled_cast(out[key], bits, st.scale, st.fmt, rng, what=(step, nm))
            a = oamax.amax(obf16.widen(bits))
            assert f32_bits(lin.amax[i].item()) == f32_bits(a)
            assert lin.sat[i].item() == ofp8.saturation_count(obf16.widen(bits), st.scale, st.fmt)
        xq, wq = out["xq"].cpu().numpy(), out["wq"].cpu().numpy()
        assert np.array_equal(out["wqt"].cpu().numpy(), wq.T)
        for r0 in range(0, xb.shape[0], 2048):  # every output row (FP8 forward datapath)
            check_gemm_rows(out["y"], xq, dsg.E4M3, dsg.OP_N, wq, dsg.E4M3, dsg.OP_N,
                            states["x"].scale, states["w"].scale,
                            np.arange(r0, min(r0 + 2048, xb.shape[0])), f"y step {step}")
        yb = bf16_bits(out["y"])
        assert f32_bits(lin.amax_y.item()) == f32_bits(ogemm.output_amax(yb))
        for nm, bits in (("x", xb), ("w", wb)):
            states[nm].update(oamax.amax(obf16.widen(bits)), dsg.ALGO_MAX, 0)
        compare_state(lin, states, ("x", "w"))


def test_decoder_layer_projections_10_steps():
    """All seven decoder-layer projections at M = 8192 over 10 steps (activation
    std 1 -> 3, 50x batch at step 6), run with `max` and with `most_recent`: the
    scale trajectories, histories and amaxes bit-exact every step; saturation
    counts exact at the outlier steps; cast bytes on samples every step; the three
    GEMMs on sampled rows at steps 0, 6 and 9 (`max` run)."""
    M = 8192
    projs = list(workloads.LLAMA_PROJ)
    algos = (dsg.ALGO_MAX, dsg.ALGO_MOST_RECENT)
    lins = {(p, a): DelayedScalingLinear(hist_len=16, algo=a) for p in projs for a in algos}
    states = {(p, a): {"x": ScalingState(ofp8.E4M3, 16), "w": ScalingState(ofp8.E4M3, 16),
                       "dy": ScalingState(ofp8.E5M2, 16)} for p in projs for a in algos}
    rng = np.random.default_rng(4)
    for step in range(10):
        for p in projs:
            xb, wb, dyb = workloads.llama_tensors(p, step, m=M)
            print(f"[decoder] step {step} {p} {xb.shape} {wb.shape}", flush=True)
            xd, wd, dyd = dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb)
            amaxes = {"x": oamax.amax(obf16.widen(xb)), "w": oamax.amax(obf16.widen(wb)),
                      "dy": oamax.amax(obf16.widen(dyb))}
            for a in algos:
                lin, st = lins[(p, a)], states[(p, a)]
                out = lin.step(xd, wd, dyd)
                torch.cuda.synchronize()
                for i, (nm, bits, key) in enumerate((("x", xb, "xq"), ("w", wb, "wq"),
                                                     ("dy", dyb, "dyq"))):
                    s = st[nm]
                    assert f32_bits(lin.scale_used[i].item()) == f32_bits(s.scale)
                    assert f32_bits(lin.amax[i].item()) == f32_bits(amaxes[nm])
                    check_sampled_cast(out[key], bits, s.scale, s.fmt, rng, n=1 << 14,
                                       what=(step, p, a, nm))
                    if step in (6, 7) and nm == "x":
                        assert lin.sat[i].item() == ofp8.saturation_count(obf16.widen(bits),
                                                                          s.scale, s.fmt)
                if a == dsg.ALGO_MAX and step in (0, 6, 9):
                    xq, wq, dyq = (out[k].cpu().numpy() for k in ("xq", "wq", "dyq"))
                    sx, sw, sdy = st["x"].scale, st["w"].scale, st["dy"].scale
                    rm = band_rows(M)
                    rk = band_rows(wb.shape[0])
                    check_gemm_rows(out["y"], xq, 0, 0, wq, 0, 0, sx, sw, rm, f"y {p} {step}")
                    check_gemm_rows(out["dx"], dyq, 1, 0, wq, 0, 1, sdy, sw, rm,
                                    f"dx {p} {step}")
                    check_gemm_rows(out["dw"], xq, 0, 1, dyq, 1, 0, sx, sdy, rk,
                                    f"dw {p} {step}")
                for nm in ("x", "w", "dy"):
                    st[nm].update(amaxes[nm], a, 0)
                compare_state(lin, st, ("x", "w", "dy"))
    # the outlier step dominates the `max` window for the remaining steps, while
    # `most_recent` forgets it one step later
    for p in projs:
        s_max = states[(p, dsg.ALGO_MAX)]["x"].scale
        s_rec = states[(p, dsg.ALGO_MOST_RECENT)]["x"].scale
        assert s_rec > s_max


def test_stress_cast_second_step():
    """The 2^30-element stress tensor cast a second time with the scale derived from
    the first step's amax (history 16, max): saturation count and amax exact over
    the whole tensor, bytes on a sample including every outlier."""
    n = 1 << 30
    bits = workloads.big_cast_input(n)
    x = dev_bf16(bits)
    for fmt in (dsg.E4M3, dsg.E5M2):
        print(f"[stress step 2] fmt {fmt}", flush=True)
        hist = torch.zeros((1, 16), dtype=torch.float32, device=DEV)
        cur = torch.zeros(1, dtype=torch.int32, device=DEV)
        s = torch.ones(1, dtype=torch.float32, device=DEV)
        q = torch.empty(n, dtype=torch.uint8, device=DEV)
        am = torch.zeros(1, dtype=torch.float32, device=DEV)
        sat = torch.zeros(1, dtype=torch.int64, device=DEV)
        dsg.fp8ds_cast(x, fmt, s, q, None, None, am, sat)
        dsg.fp8ds_scale_update(hist, cur, am, [fmt], dsg.ALGO_MAX, 0, s)
        dsg.fp8ds_cast(x, fmt, s, q, None, None, am, sat)
        torch.cuda.synchronize()
        state = ScalingState(fmt, 16)
        a_all = np.float32(0.0)
        for lo in range(0, n, 1 << 26):
            a_all = max(a_all, oamax.amax(obf16.widen(bits[lo:lo + (1 << 26)])))
        state.update(a_all, dsg.ALGO_MAX, 0)
        assert f32_bits(s.item()) == f32_bits(state.scale)
        assert f32_bits(am.item()) == f32_bits(a_all)
        osat = 0
        for lo in range(0, n, 1 << 26):
            osat += ofp8.saturation_count(obf16.widen(bits[lo:lo + (1 << 26)]), state.scale, fmt)
        assert sat.item() == osat
        rng = np.random.default_rng(5)
        big = np.flatnonzero((bits & 0x7FFF) == 0x447A)
        pos = np.unique(np.concatenate([rng.choice(n, 1 << 20, replace=False), big]))
        codes, _ = ofp8.cast(obf16.widen(bits[pos]), state.scale, fmt)
        assert np.array_equal(q[torch.from_numpy(pos).to(DEV)].cpu().numpy(), codes)
    del x
    torch.cuda.empty_cache()


def test_batched_small_linears_512():
    """512 independent 256 x 256 x 256 Linears, per-problem scales and histories
    (16), two steps: every byte, amax, scale and history exact; every output
    element within tolerance; per-problem output amax exact."""
    B, m = 512, 256
    lin = BatchedDelayedScalingLinear(B, hist_len=16)
    states = [ScalingState(ofp8.E4M3, 16) for _ in range(2 * B)]
    for step in range(2):
        xb, wb = workloads.small_batch(B, m, m, m, step=step)
        print(f"[batched] step {step}", flush=True)
        out = lin.step(dev_bf16(xb), dev_bf16(wb))
        torch.cuda.synchronize()
        xq, wq = out["xq"].cpu().numpy(), out["wq"].cpu().numpy()
        y = bf16_bits(out["y"])
        amy = lin.amax_y.cpu().numpy()
        am = lin.amax.cpu().numpy()
        for b in range(B):
            sx, sw = states[b], states[B + b]
            cx, _ = ofp8.cast(obf16.widen(xb[b]), sx.scale, ofp8.E4M3)
            cw, _ = ofp8.cast(obf16.widen(wb[b]), sw.scale, ofp8.E4M3)
            assert np.array_equal(xq[b], cx) and np.array_equal(wq[b], cw), b
            acc, sum_abs = ogemm.gemm_exact(cx, 0, 0, cw, 0, 0)
            y_ref = ogemm.dequant_to_bf16(acc, sx.scale, sw.scale)
            check_bf16_out(y[b], acc, sum_abs, y_ref,
                           1.0 / float(ogemm.dequant_scale(sx.scale, sw.scale)), f"y[{b}]")
            assert amy.view(np.uint32)[b] == f32_bits(ogemm.output_amax(y[b]))
            ax, aw = oamax.amax(obf16.widen(xb[b])), oamax.amax(obf16.widen(wb[b]))
            assert am.view(np.uint32)[b] == f32_bits(ax) and am.view(np.uint32)[B + b] == f32_bits(aw)
            sx.update(ax, dsg.ALGO_MAX, 0)
            sw.update(aw, dsg.ALGO_MAX, 0)
        s = lin.scale.cpu().numpy()
        assert np.array_equal(s.view(np.uint32),
                              np.array([st.scale for st in states], np.float32).view(np.uint32))
        h = lin.history.cpu().numpy()
        assert np.array_equal(h.view(np.uint32), np.stack([st.history for st in states]).view(np.uint32))
