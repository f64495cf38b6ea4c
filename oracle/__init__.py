"""CPU oracle for the DeepSeekMoE layer forward — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct NumPy implementation (float64 unless a step fixes
float32) of what the GPU path computes. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package. It shares no code with the HIP library and never imports it; its inputs
come from ``synth`` (seeded generators) and nowhere else.

Each function cites the passage it follows, by page title and section:
  * the lpnh.cn guide "从技术报告到可跑配置" (section 3: model JSON and the [fp8]
    block with e4m3, tile_wise_1x128 inputs and block_wise_128x128 weights);
  * the 2kiu.com DeepSeek-V3 report digest (section 3.2: sigmoid affinities, bias
    used only for ranking, normalised gates, bincount load and the +-gamma update;
    section 3.3: the sequence-level balance loss; section 3.4: node/group-limited
    routing, no token dropping; section 4.3: block scales and higher-precision
    accumulation; section 5.5: the per-sequence allocation entropy);
  * the zhihu infra commentary on the report (training part: E4M3 everywhere,
    1x128 / 128x128 groups, GEMM by partial-sum promotion; SwiGLU recomputed);
  * for the backward (``backward.py``): the guide's [fp8] block (gemm_dgrad and
    gemm_wgrad in FP8, moe_gating kept in BF16/FP32) and the zhihu commentary (E4M3 in
    both directions).

Every function here is pinned by a CPU test against something other than itself
(closed forms, brute force, library routines, invariants). None is "parity unpinned".
"""
from .backward import (  # noqa: F401
    combine_backward,
    dequant_128x1,
    expert_ffn_backward,
    layer_backward,
    quantize_128x1,
    round_bf16,
    route_backward,
    silu_grad,
)
from .e4m3 import E4M3_MAX, decode, encode, finite_values  # noqa: F401
from .moe import (  # noqa: F401
    bias_update,
    combine,
    dequant_1x128,
    dequant_128x128,
    expert_ffn,
    layer_forward,
    permute,
    quantize_1x128,
    quantize_1x128_pow2,
    quantize_128x128,
    quantize_128x128_pow2,
    route,
    seq_assignment_entropy,
    seq_balance_loss,
    silu,
)
