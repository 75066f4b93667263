"""CPU oracle for the FP8 delayed-scaling Linear.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``delayed_scaling_gemm_amd`` and its HIP library) never imports, calls or links
anything here, and nothing here imports the product path.  The two share no code.

The oracle is a plain, slow, obviously correct restatement of what the method
computes, in numpy (fp64 where floating point is involved; fp32 only where the
method itself fixes fp32, e.g. the scale quotient).

Sources, cited by page title and section:

* [P1] "算子与编译器：FP8 训练与优化器 Kernel" (charles2530.github.io)
* [P2] "FP8 混合精度训练工程实践：从 H100 到大模型训练的范式跃迁" (ybb.press)
* [P3] "LLM FP8 微调上线生产实战：用 Amax Scaling、层级白名单与 BF16 回退守住收敛"
  (oh-bug.com)
* [OCP] the OCP 8-bit floating point formats (Micikevicius et al., "FP8 Formats
  for Deep Learning", listed in [P3] §参考资料), for the special values that
  the pages leave open.

Parity status of each function (what pins it, see ``tests/test_oracle_*.py``):

* ``fp8.decode``/``fp8.encode``/``fp8.cast``: pinned (256-code tables, page
  constants, saturation and underflow cases, torch's in-range fp8 conversion,
  brute force).
* ``amax.amax``: pinned (numpy max/abs, invariants, NaN/inf/empty cases).
* ``scaling.*``: pinned (exact rational bound on the fp32 quotient, exact
  power-of-two cases, brute-force sliding windows, L=1 equivalence).
* ``gemm.gemm_exact``: pinned (int64 small-integer matmul, code-pair table,
  brute-force triple loop).
* ``bf16.round_to_bf16``: pinned (torch's fp32->bf16 conversion on fp32
  inputs, exhaustive bf16 round trip, hand-checked ties).
* ``adamw.*``: pinned (torch.optim.AdamW in float64 over 25 steps, the
  first-step lr*sign(g) closed form, pure decay under zero gradients, linear
  motion under a constant gradient, a 50-digit decimal evaluation of one step,
  the unscale and skip rules).
* ``health.cast_health``: pinned (hand-worked E4M3 / E5M2 cases).
* ``finer.*``: pinned (a hand-worked per-row E4M3 case in ``tests/golden/``,
  power-of-two row invariance, the row maximum on FP8_MAX, degenerate rows, a
  brute-force scaled GEMM in exact fractions, the per-tensor special case).
* ``mx.*``: pinned (hand-worked blocks of both formats in ``tests/golden/``,
  E8M0 code values, power-of-two shifts, the largest element in the top binade,
  a brute-force nearest-value search for every element, block independence,
  zero/NaN/Inf blocks, the unit-scale GEMM equal to ``gemm.gemm_exact`` and an
  exact-fraction triple loop).
* Parity unpinned: nothing in the oracle; on the GPU side the fp32 summation
  order of the accumulator is bounded, not pinned (see ``gemm.py``).
"""

from . import adamw, amax, bf16, finer, fp8, gemm, health, linear, mx, scaling  # noqa: F401
