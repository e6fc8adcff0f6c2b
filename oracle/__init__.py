"""Plain fp64 CPU oracle for Flash-LoRA-Attention and the LR precompute.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, links or runs
this package: only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it. It shares no code, headers, tables or helpers with
the HIP library; the only thing both sides share is the seeded input module
``workloads`` (which holds none of the method's arithmetic).

The method reaches the plain result exactly (up to rounding order): attention
over the agent's full value cache ``V_a = V_base + V_lr[:, agent slice] B_a``.
So the oracle is that definition written out in float64: it materialises
``V_a``, forms the whole score matrix, and applies a two-pass softmax. See
``oracle.lora_attention`` for each step and the passage it follows.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` (library special case, associativity identity,
invariants, closed forms, hand-derived fixtures in ``tests/golden/`` and a
pure-Python brute force). Bit-for-bit agreement with the bf16 rounding points
of the GPU path (prefill rounds P to fp16 before the P.V product; decode splits
P into bf16 hi + lo parts) is not something the pages fix: that part is
"parity unpinned" beyond the stated tolerance.
"""
from .lora_attention import (  # noqa: F401
    lr_precompute,
    lr_precompute_into,
    kv_head_of,
    agent_columns,
    agent_values,
    expand_values,
    visible,
    softmax_rows,
    attention_probs,
    attention,
    attn_prefill,
    attn_prefill_varlen,
    attn_prefill_paged,
    attn_prefill_qkvo,
    agent_keys,
    rope_rotate,
    attn_decode,
    attn_decode_paged,
    attn_decode_qkvo,
    gather_pages,
    attn_factored,
    ADAPTER_FREE,
)
