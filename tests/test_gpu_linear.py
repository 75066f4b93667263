"""GPU parity of whole Linear steps (casts, three GEMMs, scale update) against the
oracle's training step: the tiny Linear over 4 steps, the decoder-layer
projections' scale trajectories with the step-6 outlier, and the 4096-hidden
Linear at full size in the benchmark's launch configuration (sampled rows)."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import delayed_scaling_gemm_amd as dsg  # noqa: E402
import workloads  # noqa: E402
from delayed_scaling_gemm_amd.linear import DelayedScalingLinear  # noqa: E402
from oracle import bf16 as obf16  # noqa: E402
from oracle import fp8 as ofp8  # noqa: E402
from oracle import gemm as ogemm  # noqa: E402
from oracle import linear as olinear  # noqa: E402
from oracle.scaling import ScalingState  # noqa: E402
from tests.parity import band_rows, bf16_bits, check_bf16_out, f32_bits  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def oracle_states(L):
    return {"x": ScalingState(ofp8.E4M3, L), "w": ScalingState(ofp8.E4M3, L),
            "dy": ScalingState(ofp8.E5M2, L)}


def compare_state(lin, states, names=("x", "w", "dy")):
    torch.cuda.synchronize()
    h = lin.history.cpu().numpy()
    c = lin.cursor.cpu().numpy()
    s = lin.scale.cpu().numpy()
    for i, nm in enumerate(names):
        st = states[nm]
        assert np.array_equal(h[i].view(np.uint32), st.history.view(np.uint32)), nm
        assert c[i] == st.cursor and f32_bits(s[i]) == f32_bits(st.scale), (nm, s[i], st.scale)


def compare_gemm(gpu_bf16, res: olinear.GemmResult, what):
    yb = bf16_bits(gpu_bf16)
    d = 1.0 / float(ogemm.dequant_scale(res.scale_a, res.scale_b))
    check_bf16_out(yb, res.acc, res.sum_abs, res.y_bits, d, what)
    return yb


def test_tiny_linear_four_steps():
    lin = DelayedScalingLinear(hist_len=16, algo=dsg.ALGO_MAX, margin=0)
    states = oracle_states(16)
    for step in range(4):
        x, w, dy = workloads.tiny_linear_step(step)
        tx, tw, tdy = (torch.from_numpy(a).to(DEV) for a in (x, w, dy))
        out = lin.step(tx, tw, tdy)
        torch.cuda.synchronize()
        ref = olinear.train_step(x, w, dy, states, 0, 0)
        for key, ck, i in (("xq", "cast_x", 0), ("wq", "cast_w", 1), ("dyq", "cast_dy", 2)):
            c = ref[ck]
            assert np.array_equal(out[key].cpu().numpy().ravel(), c.codes.ravel()), (step, key)
            assert f32_bits(lin.amax[i].item()) == f32_bits(c.amax)
            assert f32_bits(lin.scale_used[i].item()) == f32_bits(c.scale_used)
            assert lin.sat[i].item() == c.sat
        yb = compare_gemm(out["y"], ref["y"], f"y step {step}")
        assert f32_bits(lin.amax_y.item()) == f32_bits(ogemm.output_amax(yb))
        compare_gemm(out["dx"], ref["dx"], f"dx step {step}")
        compare_gemm(out["dw"], ref["dw"], f"dw step {step}")
        compare_state(lin, states)


@pytest.mark.parametrize("algo", [dsg.ALGO_MAX, dsg.ALGO_MOST_RECENT])
def test_decoder_projection_outlier_trajectory(algo):
    """10 steps of the k_proj Linear with drifting activations and the 50x batch at
    step 6 (first 512 token rows): every byte of the casts, every scale, history
    and cursor bit-exact; all three GEMMs within tolerance."""
    M = 512
    lin = DelayedScalingLinear(hist_len=16, algo=algo, margin=0)
    states = oracle_states(16)
    for step in range(10):
        xb, wb, dyb = workloads.llama_tensors("k_proj", step, m=M)
        out = lin.step(dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb))
        x, w, dy = obf16.widen(xb), obf16.widen(wb), obf16.widen(dyb)
        ref = olinear.train_step(x, w, dy, states, algo, 0)
        torch.cuda.synchronize()
        for key, ck in (("xq", "cast_x"), ("wq", "cast_w"), ("dyq", "cast_dy")):
            assert np.array_equal(out[key].cpu().numpy(), ref[ck].codes), (step, key)
        assert lin.sat[0].item() == ref["cast_x"].sat
        compare_gemm(out["y"], ref["y"], f"y {step}")
        compare_gemm(out["dx"], ref["dx"], f"dx {step}")
        compare_gemm(out["dw"], ref["dw"], f"dw {step}")
        compare_state(lin, states)


def _sampled_rows_check(gpu_out, a_codes, fa, opa, b_codes, fb, opb, sa, sb, rows, what):
    """Oracle GEMM on a sample of output rows only."""
    a_rows = a_codes[rows] if opa == dsg.OP_N else a_codes[:, rows].T
    acc, sum_abs = ogemm.gemm_exact(np.ascontiguousarray(a_rows), fa, 0, b_codes, fb, opb)
    y_ref = ogemm.dequant_to_bf16(acc, sa, sb)
    yb = bf16_bits(gpu_out[torch.from_numpy(rows).to(DEV)])
    d = 1.0 / float(ogemm.dequant_scale(sa, sb))
    check_bf16_out(yb, acc, sum_abs, y_ref, d, what)


def test_fwd_bwd_4096_full_size_sampled():
    """The M=16384, 4096-hidden Linear at full size, launched exactly as the
    benchmark launches it: all cast bytes on a sample, amax and saturation exact,
    every output of the forward GEMM (FP8 matrix instructions) and rows of the
    backward GEMMs (first, last and one moving row of every 256-row tile band)
    against the oracle, output amax exact."""
    xb, wb, dyb = workloads.fwd_bwd_4096()
    print("[fwd_bwd_4096] inputs ready", flush=True)
    lin = DelayedScalingLinear(hist_len=16)
    # step 0 runs at scale 1.0; step 1 at the scales derived from step 0
    states = oracle_states(16)
    for step in range(2):
        out = lin.step(dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb))
        torch.cuda.synchronize()
        xq, wq, dyq = (out[k].cpu().numpy() for k in ("xq", "wq", "dyq"))
        rng = np.random.default_rng(step)
        for name, st, bits, q in (("x", states["x"], xb, xq), ("w", states["w"], wb, wq),
                                  ("dy", states["dy"], dyb, dyq)):
            flat = bits.ravel()
            pos = rng.choice(flat.size, 1 << 18, replace=False)
            codes, _ = ofp8.cast(obf16.widen(flat[pos]), st.scale, st.fmt)
            assert np.array_equal(q.ravel()[pos], codes), (step, name)
        i_x, i_w, i_dy = 0, 1, 2
        su = lin.scale_used.cpu().numpy()
        assert f32_bits(su[i_x]) == f32_bits(states["x"].scale)
        # the forward runs on the FP8 matrix instructions: every output row checked
        for r0 in range(0, 16384, 2048):
            _sampled_rows_check(out["y"], xq, 0, 0, wq, 0, 0, su[i_x], su[i_w],
                                np.arange(r0, r0 + 2048), "y")
        rows = band_rows(16384)
        _sampled_rows_check(out["dx"], dyq, 1, 0, wq, 0, 1, su[i_dy], su[i_w], rows, "dx")
        rows_k = band_rows(4096)
        _sampled_rows_check(out["dw"], xq, 0, 1, dyq, 1, 0, su[i_x], su[i_dy], rows_k, "dw")
        yb = bf16_bits(out["y"])
        assert f32_bits(lin.amax_y.item()) == f32_bits(ogemm.output_amax(yb))
        # advance the oracle's scaling state with exact amaxes of the full tensors
        from oracle import amax as oamax
        for name, bits in (("x", xb), ("w", wb), ("dy", dyb)):
            states[name].update(oamax.amax(obf16.widen(bits)), 0, 0)
        compare_state(lin, states)
        print(f"[fwd_bwd_4096] step {step} ok", flush=True)


def test_decoder_projection_health_counts():
    """health=True on the k_proj trajectory (drift, 50x batch at step 6): each
    step's counts for X, W and dY equal the oracle's for the cast with the
    step's scale snapshot, and the codes are those of the plain step."""
    from oracle import health as ohealth

    M = 512
    lin = DelayedScalingLinear(hist_len=16, algo=dsg.ALGO_MAX, margin=0, health=True)
    sparse = DelayedScalingLinear(hist_len=16, algo=dsg.ALGO_MAX, margin=0, health=True,
                                  health_every=4)
    states = oracle_states(16)
    saw_saturation = False
    for step in range(10):
        xb, wb, dyb = workloads.llama_tensors("k_proj", step, m=M)
        out = lin.step(dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb))
        sparse.step(dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb))
        x, w, dy = obf16.widen(xb), obf16.widen(wb), obf16.widen(dyb)
        ref = olinear.train_step(x, w, dy, states, dsg.ALGO_MAX, 0)
        rep = lin.health_report()
        srep = sparse.health_report()
        assert srep["step"] == step - step % 4  # counted every 4th step only
        if step % 4 == 0:
            assert {k: srep[k] for k in ("x", "w", "dy")} == {k: rep[k] for k in ("x", "w", "dy")}
        for nm, ck, v in (("x", "cast_x", x), ("w", "cast_w", w), ("dy", "cast_dy", dy)):
            c = ref[ck]
            exp = ohealth.cast_health(v, c.scale_used, states[nm].fmt)
            assert rep[nm] == exp, (step, nm, rep[nm], exp)
            saw_saturation |= exp["saturated"] > 0
        assert rep["step"] == step
        assert np.array_equal(out["xq"].cpu().numpy(), ref["cast_x"].codes)
        compare_state(lin, states)
    assert saw_saturation  # the 50x batch saturates X's cast


def test_checkpoint_resume_is_bit_identical(tmp_path):
    """Save the scaling state after step 7 of the k_proj trajectory (the 50x batch
    of step 6 is in every window), restore it into a fresh Linear and continue:
    steps 8 and 9 reproduce the uninterrupted run bit for bit.  The same saved
    file also restores the oracle's ScalingState of X, W and dY, and the resumed
    GPU steps match the oracle's steps from it (every byte, scale, history and
    cursor exact; GEMMs within tolerance).  Restoring only the scale (dropping
    the history) does not reproduce the run: the outlier leaves the window early
    and the next scale changes, the pages' scale-mismatch incident."""
    M = 256

    def inputs(step):
        xb, wb, dyb = workloads.llama_tensors("k_proj", step, m=M)
        return dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb)

    ref = DelayedScalingLinear(hist_len=16)
    run = DelayedScalingLinear(hist_len=16)
    outs = {}
    for step in range(10):
        o = ref.step(*inputs(step))
        outs[step] = ({k: v.clone() for k, v in o.items()},
                      {k: t.clone() for k, t in (("scale", ref.scale), ("amax", ref.amax),
                                                 ("history", ref.history),
                                                 ("cursor", ref.cursor))})
        if step < 8:
            run.step(*inputs(step))
    path = str(tmp_path / "k_proj_scaling.pt")
    run.save(path)
    resumed = DelayedScalingLinear(hist_len=16)
    resumed.load(path)
    scale_only = DelayedScalingLinear(hist_len=16)
    scale_only.scale.copy_(run.scale)
    # the oracle's scaling state, restored from the same file
    saved = torch.load(path, map_location="cpu", weights_only=True)
    states = oracle_states(16)
    for i, nm in enumerate(("x", "w", "dy")):
        st = states[nm]
        st.history = saved["history"][i].numpy().astype(np.float32).copy()
        st.cursor = int(saved["cursor"][i])
        st.scale = np.float32(saved["scale"][i].item())
    for step in (8, 9):
        o = resumed.step(*inputs(step))
        scale_only.step(*inputs(step))
        torch.cuda.synchronize()
        xb, wb, dyb = workloads.llama_tensors("k_proj", step, m=M)
        oref = olinear.train_step(obf16.widen(xb), obf16.widen(wb), obf16.widen(dyb), states,
                                  dsg.ALGO_MAX, 0)
        for key, ck in (("xq", "cast_x"), ("wq", "cast_w"), ("dyq", "cast_dy")):
            assert np.array_equal(o[key].cpu().numpy(), oref[ck].codes), (step, key)
        compare_gemm(o["y"], oref["y"], f"resumed y {step}")
        compare_gemm(o["dx"], oref["dx"], f"resumed dx {step}")
        compare_gemm(o["dw"], oref["dw"], f"resumed dw {step}")
        compare_state(resumed, states)
        ro, rs = outs[step]
        for k in ("xq", "wq", "wqt", "dyq"):
            assert torch.equal(o[k], ro[k]), (step, k)
        for k in ("y", "dx", "dw"):
            assert torch.equal(o[k].view(torch.int16), ro[k].view(torch.int16)), (step, k)
        for k in ("scale", "amax", "history", "cursor"):
            assert torch.equal(getattr(resumed, k), rs[k]), (step, k)
    assert not torch.equal(scale_only.scale, outs[9][1]["scale"])


def test_fused_adamw_step_matches_the_unfused_loop():
    """Six training steps of the k_proj Linear with fp32 master weights, once with
    the AdamW update followed by the next step's W cast (unfused), once with
    adamw_step (update and W cast in one kernel, the next forward skipping its
    W cast).  Every FP8 operand, every output, the weights, the moments and the
    scaling state agree bit for bit; at step 3 a NaN in dY makes dW non-finite
    and both runs skip the update."""
    M, NAN_STEP = 256, 3
    hp = dict(lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    _, wb, _ = workloads.llama_tensors("k_proj", 0, m=M)
    w0 = torch.from_numpy((wb.astype(np.uint32) << 16).view(np.float32)).to(DEV)
    runs = {}
    for name in ("unfused", "fused"):
        runs[name] = dict(lin=DelayedScalingLinear(hist_len=16), w=w0.clone(),
                          m=torch.zeros_like(w0), v=torch.zeros_like(w0))
    w_casts = []
    orig_cast = runs["fused"]["lin"]._cast
    runs["fused"]["lin"]._cast = lambda t, *a: (w_casts.append(t), orig_cast(t, *a))
    for step in range(6):
        xb, _, dyb = workloads.llama_tensors("k_proj", step, m=M)
        x, dy = dev_bf16(xb), dev_bf16(dyb)
        if step == NAN_STEP:
            dy = dy.clone()
            dy[3, 5] = float("nan")
        outs = {}
        for name, r in runs.items():
            lin = r["lin"]
            w_before = r["w"].clone()
            o = lin.step(x, r["w"], dy)
            outs[name] = {k: t.clone() for k, t in o.items()}
            if name == "unfused":
                dsg.fp8ds_adamw(r["w"], o["dw"], r["m"], r["v"], hp["lr"], hp["beta1"],
                                hp["beta2"], hp["eps"], hp["weight_decay"], step + 1,
                                grad_amax=lin.amax_dw)
            else:
                lin.adamw_step(r["w"], r["m"], r["v"], hp["lr"], step + 1, hp["beta1"],
                               hp["beta2"], hp["eps"], hp["weight_decay"])
            torch.cuda.synchronize()
            assert torch.equal(r["w"], w_before) == (step == NAN_STEP), (name, step)
        a, b = runs["unfused"], runs["fused"]
        for k in ("xq", "wq", "wqt", "dyq"):
            assert torch.equal(outs["unfused"][k], outs["fused"][k]), (step, k)
        for k in ("y", "dx", "dw"):
            assert torch.equal(outs["unfused"][k].view(torch.int16),
                               outs["fused"][k].view(torch.int16)), (step, k)
        for k in ("w", "m", "v"):
            assert torch.equal(a[k].view(torch.int32), b[k].view(torch.int32)), (step, k)
        for k in ("scale", "history", "cursor"):  # as bits: the dY history holds a NaN
            assert torch.equal(getattr(a["lin"], k).view(torch.int32),
                               getattr(b["lin"], k).view(torch.int32)), (step, k)
        # the fused run wrote the new weights' amax into the next step's
        # accumulator set (its push into the history is compared above, one step
        # later); the last step's amaxes of X and dY agree
        assert torch.equal(a["lin"].amax[0::2].view(torch.int32),
                           b["lin"].amax[0::2].view(torch.int32)), step
        lb = b["lin"]
        assert lb._amax_of(lb._slot)[1].item() == b["w"].abs().max().item()
    # the fused run cast W only in its first forward
    assert w_casts.count(1) == 1
