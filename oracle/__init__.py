"""CPU oracle for the fused NVFP4 Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) may import or call this package; only the tests, the smoke check
and the CPU-baseline leg of the benchmark do.  It shares no code with the HIP
path: no kernels, headers, tables or helpers.

What it computes follows the page "Serving Solar Open 2 on DGX Spark"
(backend.ai, 2026-07), which describes:
  * the model: 320 routed experts, one shared expert, top-8 routing
    (section "Solar Open 2 개요");
  * the expert-parallel change to the b12x fused-MoE kernels: a contiguous shard
    of experts per node, a `local_expert_offset` that maps the globally routed
    expert id to a shard-relative index, and a guard that drops token-expert
    pairs outside the shard; the output of a shard is a partial sum that the
    caller adds up across shards (section "수정 사항 › b12x에서의 Expert
    Parallelism 구현 추가");
  * the NVFP4 tensors: packed FP4 weights, FP8 block scales clamped to 448 and a
    per-expert fp32 global scale, with fused gate/up rows (section "b12x 버전이
    실제 NVFP4 체크포인트를 읽어들이도록 만들기").
The NVFP4 element/scale formats themselves (E2M1 codes, one E4M3 scale per 16
contiguous elements, fp32 per-tensor scale) are NVIDIA's published NVFP4
definition; the pages name the format but do not define it.

Arithmetic is fp64 throughout, except inside the NVFP4 quantizers, whose scale
arithmetic is fp32 by the format: the per-tensor global scale is an fp32 number
(amax / (6 * 448) rounded to fp32), and the recipe derives the block scale and
the effective decode multiplier (block scale * global) from it in that same fp32
arithmetic, so the division that picks each E2M1 code is by that fp32 multiplier
and is itself an fp32 operation.  For the dynamic activation scale the choice is
immaterial: fp32(amax / 6) never lands on the other side of an E4M3 rounding
midpoint than the exact quotient (the midpoints have at most 5 significant
bits).  For weights, fp32(s * g) is a real choice, taken from the format's fp32
global scale.

Modules:
  nvfp4   - E2M1 / E4M3 codecs, NVFP4 weight and activation quantizers.
  moe     - router, shard filter, permutation, layer forward (vectorised).
  brute   - the same layer as plain per-token / per-expert Python loops, with
            its own decoding by formula, used to pin `moe` on tiny inputs.
  checkpoint - preparation of pre-quantized checkpoints (global-scale
            convention, gate/up row order, shard slicing), section "b12x 버전이
            실제 NVFP4 체크포인트를 읽어들이도록 만들기".

Parity status: every function here is pinned by a CPU test against the format
definitions, closed forms, invariants or brute force (tests/test_oracle_*.py);
`moe.forward` is pinned by `brute` (explicit loops), by the dense-FFN special
case and by the half-shard sum, with the builtin map and with a process pool.
End-to-end values at the workload sizes have no printed worked example on the
pages; they are pinned only through those invariants.
"""
from . import nvfp4, moe, brute, checkpoint  # noqa: F401
