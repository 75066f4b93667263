"""Scaling-state checkpoint round trip (host only: no kernel runs)."""

import pytest
import torch

from delayed_scaling_gemm_amd.linear import DelayedScalingLinear


def test_state_round_trips_through_a_file(tmp_path):
    a = DelayedScalingLinear(hist_len=8, device="cpu")
    a.history.copy_(torch.arange(24, dtype=torch.float32).reshape(3, 8))
    a.cursor.copy_(torch.tensor([3, 0, 7], dtype=torch.int32))
    a.scale.copy_(torch.tensor([2.5, 0.125, 1024.0]))
    path = str(tmp_path / "scaling.pt")
    a.save(path)
    b = DelayedScalingLinear(hist_len=8, device="cpu")
    b.load(path)
    for name in ("history", "cursor", "scale"):
        assert torch.equal(getattr(a, name), getattr(b, name))


def test_recipe_mismatch_is_refused():
    a = DelayedScalingLinear(hist_len=8, device="cpu")
    with pytest.raises(ValueError, match="recipe"):
        DelayedScalingLinear(hist_len=16, device="cpu").load_state_dict(a.state_dict())
    with pytest.raises(ValueError, match="recipe"):
        DelayedScalingLinear(hist_len=8, margin=1, device="cpu").load_state_dict(a.state_dict())
