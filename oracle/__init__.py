"""CPU oracle for the real-time MoE expert load-balancing path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
anything here: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and does not import the ``moe_expert_load_amd`` package.

Every function is a plain, slow, obviously-correct statement of what the pages
define, in Python + numpy (fp64 wherever floating point appears, except where
the path itself fixes fp32).  Sources:

* "300 微秒调平 MoE 专家负载！小红书 UltraEP 逼近 94.3% 理想训推吞吐" (UltraEP
  article on m.163.com), sections
    - "在 Gate 之后获取当前层真实负载"  (real load after Gate)           -> load_matrix
    - "Quota 同时决定专家副本与 token 分流" (quota decides replicas/split) -> quota, reroute
    - "共享冗余 slot 管理动态专家副本"   (shared redundant slots)         -> stage
    - "复用前向方案，完成权重恢复与梯度归约" (backward replay)            -> stage
* "Improving DeepEP MoE Load Balance in SGLang with Waterfill and LPLB"
  (papercache notes of the lmsys blog), sections
    - "Waterfill算法执行步骤"  (Waterfill steps)                          -> waterfill
    - "共享专家融合作为启用机制" (shared-expert fusion)                     -> waterfill
    - "线性规划（LP）公式化构建", "决策变量与矩阵规模优化" (LP, variables)  -> lplb
    - "从LP解决方案到Token调度" (from LP to token dispatch)               -> lplb
    - "背景知识与设计原则", "共享专家融合作为启用机制" (dispatch and combine) -> combine

Parity status of each function (what pins it) is listed in the module headers.
"""

from .load_matrix import load_matrix, OracleInputError
from .quota import solve_quota
from .reroute import reroute, assign, identity_quota
from .permute import permute, permute_rows, row_sources, rows_of
from .combine import combine, combine_f32, combine_tokens, f32_to_bf16_bits, bf16_bits_to_f32
from .stage import stage_forward, grad_reduce
from .philox import philox4x64_10, philox4x64_10_np
from .waterfill import waterfill, extend_topk
from .lplb import lplb_structure, lplb_lp, simplex, hamilton_quotas, lplb, lplb_sample

__all__ = [
    "load_matrix", "OracleInputError", "solve_quota", "reroute", "assign", "identity_quota",
    "permute", "permute_rows", "row_sources", "rows_of", "combine", "combine_f32", "combine_tokens", "f32_to_bf16_bits",
    "bf16_bits_to_f32", "stage_forward", "grad_reduce", "philox4x64_10", "philox4x64_10_np",
    "waterfill", "extend_topk", "lplb_structure", "lplb_lp", "simplex", "hamilton_quotas", "lplb",
    "lplb_sample",
]
