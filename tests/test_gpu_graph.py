"""A pair of Linear training steps captured in a HIP graph and replayed.

The library's calls allocate nothing and clear their accumulators with kernels
(no memsets), so a caller can capture a training step.  The Linear alternates
two accumulator sets by step parity on the host, so two steps are captured
together (parity back where it started).  Every replay, with new inputs copied
into the captured buffers and eager work of the program between replays, must
equal the same two steps run eagerly on a twin Linear, bit for bit: outputs, FP8
bytes, histories, cursors, scales and scale snapshots."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import delayed_scaling_gemm_amd as dsg  # noqa: E402
from delayed_scaling_gemm_amd.linear import DelayedScalingLinear  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def inputs(seed, M, K, N):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    dy = (rng.standard_t(3, (M, N)) * 1e-3).astype(np.float32)  # heavy-tailed gradients
    return [torch.from_numpy(a).to(DEV).to(torch.bfloat16) for a in (x, w, dy)]


def snapshot(lin):
    torch.cuda.synchronize()
    out = {k: lin._bufs[k].clone() for k in ("xq", "wq", "wqt", "y", "dyq", "dx", "dw")}
    for k in ("history", "cursor", "scale", "scale_used"):
        out[k] = getattr(lin, k).clone()
    return out


def assert_same(a, b, what):
    for k in a:
        ta, tb = a[k], b[k]
        same = torch.equal(ta.view(torch.uint8) if ta.dtype != torch.uint8 else ta,
                           tb.view(torch.uint8) if tb.dtype != torch.uint8 else tb)
        assert same, f"{what}: {k} differs between the graph replay and the eager steps"


# (M, K, N): 128 x 128 tiles with the K split on the exact datapath; 256 x 256
# tiles with direct loads, the forward (K = 4096) on the FP8 instructions
@pytest.mark.parametrize("shape", [(2048, 1024, 1024), (4096, 4096, 4096)])
def test_captured_step_pair_replays_like_eager_steps(shape):
    M, K, N = shape
    print(f"[graph] shape={shape}", flush=True)
    eager = DelayedScalingLinear(hist_len=16, algo=dsg.ALGO_MAX, margin=0, device=DEV)
    graphed = DelayedScalingLinear(hist_len=16, algo=dsg.ALGO_MAX, margin=0, device=DEV)
    sx, sw, sdy = inputs(1, M, K, N)  # the captured input buffers
    # warm-up pair on both (allocates the Linears' buffers before capture)
    for lin in (eager, graphed):
        lin.step(sx, sw, sdy)
        lin.step(sx, sw, sdy)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        graphed.step(sx, sw, sdy)
        graphed.step(sx, sw, sdy)
    torch.cuda.synchronize()

    scratch = torch.randn(512, 512, device=DEV)
    for it in range(4):
        x, w, dy = inputs(100 + it, M, K, N)
        sx.copy_(x)
        sw.copy_(w)
        sdy.copy_(dy)
        g.replay()
        torch.cuda.synchronize()
        scratch = scratch @ scratch.T * 1e-3  # eager work of the program between replays
        eager.step(x, w, dy)
        eager.step(x, w, dy)
        assert_same(snapshot(graphed), snapshot(eager), f"{shape} replay {it}")
    assert int(graphed.cursor[0].item()) == (2 + 2 * 4) % 16
