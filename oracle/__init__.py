"""fp64 CPU oracle of the DeepSeekMoE layer forward pass -- TEST INFRASTRUCTURE.

This package is the checker, not the product. Only the test suite, the
package's smoke check and the benchmark's CPU-baseline leg may import it. It
shares no code with the HIP library and imports nothing from it; it reads the
same stored inputs (bf16 bits, fp32 values, fp8-e4m3 codes with fp32 row
scales) and decodes them with its own converters written from the format
definitions.

Sources (the web pages this library is built from):
  [DSMoE]  "DeepSeekMoE架构解析：共享+路由专家协同与无丢弃门控设计" (jsqmd.com),
           sections 1, 2.1 (eqs. 13-15), 2.2 (eq. 16 and the bias update rule),
           3.1 (PyTorch sketch).
  [V3ARCH] "DeepSeek-V3：MoE大模型架构" (aiqz.cc), sections "MoE核心思想" and
           "路由机制".
  [COURSE] "省钱第一招：把一个大厨换成专家团" (blog.zero43.top, DeepSeek paper
           course 07), sections 三 to 六.
  The fine-grained FP8 path (fp8block.py) follows [DSMoE] section 4.3.

Every function is the plain definition written out in float64 (the bias
update is the one step done in fp32, because the bias is an fp32 state
vector). Readings of points the pages leave open are listed where they are
used.

Parity status: every function here is pinned by tests/test_oracle_pins.py
against closed forms, brute force, library routines or invariants; none is
"parity unpinned".
"""

from .formats import bf16_to_f64, e4m3_to_f64, E4M3_TABLE, decode_stored, f64_to_bf16_bits  # noqa: F401
from .moe import (  # noqa: F401
    GAMMA_F32,
    NEAR_TIE_GAP,
    RMS_EPS,
    rmsnorm,
    router_logits,
    scores,
    select_topk,
    select_groups,
    gate_values,
    expert_loads,
    sequence_loads,
    permutation,
    silu,
    swiglu_expert,
    route,
    selection_valid,
    ExpertBank,
    layer_rows,
    bias_update,
)
from .fp8block import (  # noqa: F401
    E4M3_MAX,
    TILE,
    e4m3_encode,
    quantize_tiles,
    dequantize_tiles,
    dequantize_blocks,
    expert_h_fp8,
    swiglu_expert_fp8,
    BlockExpertBank,
    quantize_x,
    layer_rows_fp8,
)
