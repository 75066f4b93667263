"""Every call takes the caller's stream: Linear steps run on a side stream, whose
inputs are produced by work queued on that same stream just before each step
(no synchronization in between), must equal the same steps on the default
stream, bit for bit."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import delayed_scaling_gemm_amd as dsg  # noqa: E402
from delayed_scaling_gemm_amd.linear import DelayedScalingLinear  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_linear_steps_on_a_side_stream():
    M, K, N = 2048, 4096, 1024  # forward on the FP8 instructions, K-split backward
    rng = np.random.default_rng(3)
    x0 = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(DEV)
    w0 = torch.from_numpy((rng.standard_normal((K, N)) * 0.02).astype(np.float32)).to(DEV)
    dy0 = torch.from_numpy((rng.standard_t(3, (M, N)) * 1e-3).astype(np.float32)).to(DEV)
    torch.cuda.synchronize()

    ref = DelayedScalingLinear(hist_len=16, algo=dsg.ALGO_MAX, margin=0, device=DEV)
    side_lin = DelayedScalingLinear(hist_len=16, algo=dsg.ALGO_MAX, margin=0, device=DEV)
    keys = ("xq", "wq", "dyq", "y", "dx", "dw")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for i in range(3):
        f = float(i + 1)
        x, w, dy = ((t * f).to(torch.bfloat16) for t in (x0, w0, dy0))
        out = ref.step(x, w, dy)
        want = {k: out[k].clone() for k in keys}
        with torch.cuda.stream(side):
            # inputs produced on the side stream right before the step
            sx, sw, sdy = ((t * f).to(torch.bfloat16) for t in (x0, w0, dy0))
            got = side_lin.step(sx, sw, sdy, stream=side)
            got = {k: got[k].clone() for k in keys}
        side.synchronize()
        torch.cuda.synchronize()
        for k in keys:
            a, b = want[k], got[k]
            if a.dtype != torch.uint8:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), (i, k)
        for k in ("history", "cursor", "scale", "scale_used"):
            assert torch.equal(getattr(ref, k), getattr(side_lin, k)), (i, k)
