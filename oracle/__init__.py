"""CPU oracle for the DFlash draft step.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow float64 NumPy
restatement of what the draft step computes.  It exists to check the HIP path
and shares no code with it.  Only the test suite, the smoke check in
`__graft_entry__.py` and the CPU-baseline leg of `bench.py` may import it; the
product path never does.

Sources (web pages on the method; cited by page title and section):
  * "DFlash 投机解码：块扩散草稿与 KV 注入" (caijizhuo.github.io): notation table,
    section 二 "注意力模式", section 三 (KV injection, fusion equation),
    section 四 (inference pseudocode; engineering note on cached projected KV).
  * "DFlow 完全拆解" (pinghaoyang.com.cn): the fusion equation in the section on
    DFlash's recomputation window; the accept/reject split in the opening section;
    relay steps 1-3 and the inference-loop section (the relay, `oracle/dflow.py`).
  * DFlash system/training/deployment notes (blog.hotdry.top), section 2.
  * "DFlash 2：正确 token 已在候选里，选一条连贯的路就好": the path selector
    (first insight section) and the two-tap dynamic convolution (second
    insight section), both in `oracle/dflash2.py`.

Where the pages leave a step open, the reading taken is stated at the function.

Parity status: every function here is pinned by tests under tests/ (closed
forms, invariants, library-routine special cases, brute force on tiny inputs,
and the worked examples stored under tests/golden/).  Forward values at the
full model shapes are pinned only through those properties: the pages print no
output values for any input.
"""
from .dflash2 import (  # noqa: F401
    CONV_SITES,
    conv_param_count,
    draft_block_conv,
    gate as selector_gate,
    pair_scores,
    select_path,
    two_tap_conv,
    walk,
)
from .specsample import (  # noqa: F401
    draft_tokens,
    philox4x64_10,
    spec_sample,
    uniforms,
)
from .dflow import (  # noqa: F401
    RelayState,
    block_inputs,
    layer_norm,
    relay_inputs,
    relay_plan,
)
from .dflash import (  # noqa: F401
    ContextCache,
    OracleDrafter,
    accept,
    block_attention,
    draft_block,
    fuse_context,
    normed_stored,
    project_context_kv,
    rms_norm,
    round_bf16,
    rope,
    swiglu_ffn,
    topk,
)
