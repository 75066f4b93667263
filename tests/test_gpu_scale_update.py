"""GPU parity: history push, window reduction and scale formula against the
oracle's ScalingState (bit-exact scales, histories and cursors)."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import delayed_scaling_gemm_amd as dsg  # noqa: E402
from oracle.scaling import ScalingState  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_sequence(fmts, L, algo, margin, amax_seq):
    T = len(fmts)
    hist = torch.zeros((T, L), dtype=torch.float32, device=DEV)
    cur = torch.zeros(T, dtype=torch.int32, device=DEV)
    scale = torch.ones(T, dtype=torch.float32, device=DEV)
    sinv = torch.zeros(T, dtype=torch.float32, device=DEV)
    states = [ScalingState(f, L) for f in fmts]
    for step, amaxes in enumerate(amax_seq):
        am = torch.from_numpy(amaxes.astype(np.float32)).to(DEV)
        dsg.fp8ds_scale_update(hist, cur, am, fmts, algo, margin, scale, sinv)
        torch.cuda.synchronize()
        for t, st in enumerate(states):
            st.update(np.float32(amaxes[t]), algo, margin)
        got_s = scale.cpu().numpy()
        exp_s = np.array([st.scale for st in states], dtype=np.float32)
        assert np.array_equal(got_s.view(np.uint32), exp_s.view(np.uint32)), (step, got_s, exp_s)
        assert np.array_equal(sinv.cpu().numpy(), (np.float32(1.0) / exp_s).astype(np.float32))
        assert np.array_equal(cur.cpu().numpy(), [st.cursor for st in states])
        got_h = hist.cpu().numpy()
        exp_h = np.stack([st.history for st in states])
        assert np.array_equal(got_h.view(np.uint32), exp_h.view(np.uint32))


@pytest.mark.parametrize("L", [1, 16, 100, 1024])
@pytest.mark.parametrize("algo", [dsg.ALGO_MAX, dsg.ALGO_MOST_RECENT])
@pytest.mark.parametrize("margin", [0, 1, -2])
def test_random_sequences(L, algo, margin):
    rng = np.random.default_rng(L * 7 + algo * 3 + margin)
    fmts = [dsg.E4M3, dsg.E4M3, dsg.E5M2, dsg.E5M2, dsg.E4M3]
    steps = 40 if L < 1024 else 12
    seq = (rng.random((steps, len(fmts))) * 2.0 ** rng.integers(-20, 20, (steps, len(fmts))))
    run_sequence(fmts, L, algo, margin, seq)


def test_special_amax_values():
    """Zero, NaN, inf, a subnormal (scale overflow) and huge values take the 1.0
    fallback exactly where the oracle does; NaN leaves the window after L steps."""
    fmts = [dsg.E4M3, dsg.E5M2, dsg.E4M3]
    seq = np.array([
        [0.0, 3.0, 1.0],
        [np.nan, 0.0, 2.0],
        [2.0, np.inf, 1e-40],
        [3.0e38, 5.0, 4.0],
        [2.0, 5.0, 4.0],
        [2.0, 5.0, 4.0],
        [2.0, 5.0, 4.0],
    ], dtype=np.float32)
    for algo in (dsg.ALGO_MAX, dsg.ALGO_MOST_RECENT):
        run_sequence(fmts, 4, algo, 0, seq)
        run_sequence(fmts, 4, algo, 120, seq)


def test_many_tensors():
    """A batch of 1024 histories (the small-Linear batch's X and W) in one launch."""
    rng = np.random.default_rng(3)
    fmts = [dsg.E4M3 if i % 3 else dsg.E5M2 for i in range(1024)]
    seq = rng.random((20, 1024)) * 50
    run_sequence(fmts, 16, dsg.ALGO_MAX, 0, seq)
