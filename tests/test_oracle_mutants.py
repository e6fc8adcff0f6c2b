"""Planted mistakes in the oracle (CPU only) must each be caught by the pins.

Every mutant below replaces one step of ``oracle.lora_attention`` with a
plausible slip (dropped term, wrong sign, off-by-one, wrong index, transposed
operand). The test runs the pin checks of ``test_oracle_pins`` against the
mutated oracle and asserts that at least one of them fails. The mutation is
undone after each test by ``monkeypatch``.
"""
import numpy as np
import pytest

import oracle
from oracle import lora_attention as LA
from tests import test_oracle_pins as pins

_orig_softmax = LA.softmax_rows
_orig_agent_values = LA.agent_values
_orig_rope = LA.rope_rotate
_orig_expand_values = LA.expand_values


def _checks():
    golden = pins._load_golden()
    yield lambda: [pins.test_golden_prefill(c) for c in golden["prefill"]]
    yield lambda: [pins.test_golden_decode(c) for c in golden["decode"]]
    yield lambda: [pins.test_golden_precompute(c) for c in golden["precompute"]]
    yield lambda: pins.test_zero_lora_is_standard_causal_gqa_attention(4, 2, 5, 7)
    yield lambda: pins.test_bruteforce_prefill(4, 2, 8, 2, 3, 5, 2)
    yield lambda: pins.test_bruteforce_prefill(8, 2, 4, 4, 0, 7, 1)
    yield lambda: pins.test_bruteforce_decode_with_shared_and_empty_ranges()
    yield lambda: pins.test_bruteforce_decode_mixed_adapted_and_adapter_free()
    yield lambda: pins.test_bruteforce_prefill_varlen_batch()
    yield lambda: pins.test_bruteforce_decode_paged_cache()
    yield lambda: pins.test_bruteforce_prefill_paged_cache()
    yield lambda: pins.test_bruteforce_prefill_with_key_lora(2)
    yield lambda: pins.test_key_lora_special_cases()
    yield lambda: pins.test_bruteforce_decode_with_key_lora()
    yield lambda: pins.test_precompute_triple_loop_and_one_hot()
    yield lambda: pins.test_bruteforce_expand_values_and_expand_then_attend()
    yield lambda: pins.test_projection_level_lora_split()
    yield lambda: pins.test_probability_rows_and_causal_zeros()


def _some_pin_fails():
    for check in _checks():
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


def _mut_agent_values_no_lr(V_base, V_lr, B, agent):
    return np.asarray(V_base, np.float64).copy()


def _mut_agent_values_transposed(V_base, V_lr, B, agent):
    V_base = np.asarray(V_base, np.float64)
    L, n_kv, d = V_base.shape
    r = np.asarray(B).shape[1]
    lr = np.asarray(V_lr, np.float64)[:, agent * r:(agent + 1) * r] @ np.asarray(B, np.float64)[agent]
    return V_base + lr.reshape(L, d, n_kv).transpose(0, 2, 1)


def _mut_agent_values_minus(V_base, V_lr, B, agent):
    return 2 * np.asarray(V_base, np.float64) - _orig_agent_values(V_base, V_lr, B, agent)


def _mut_softmax_no_normalise(S, mask):
    S = np.where(mask, np.asarray(S, np.float64), -np.inf)
    return np.where(mask, np.exp(S - S.max(-1, keepdims=True)), 0.0)


def _mut_softmax_flipped(S, mask):
    return _orig_softmax(-np.asarray(S, np.float64), mask)


def _mut_adapter_free_reads_agent_zero(V_base, V_lr, B, agent):
    return _orig_agent_values(V_base, V_lr, B, max(agent, 0))


def _mut_rope_adjacent_pairs(Y, cos, sin):
    Y = np.asarray(Y, np.float64)
    L, d = Y.shape[0], Y.shape[-1]
    c = np.asarray(cos, np.float64)[:L].reshape((L,) + (1,) * (Y.ndim - 2) + (d // 2,))
    s_ = np.asarray(sin, np.float64)[:L].reshape(c.shape)
    ev, od = Y[..., 0::2], Y[..., 1::2]
    out = np.empty_like(Y)
    out[..., 0::2] = ev * c - od * s_
    out[..., 1::2] = od * c + ev * s_
    return out


def _mut_decode_qkvo_absolute_rows(Q, K_base, V_base, V_lr, K_lr, B, B_k, cos, sin, kv_start, kv_len, agents,
                                   scale, requests=None):
    # rotates request b's keys at their absolute cache rows instead of positions 0 .. kv_len-1
    out = []
    for b in range(len(Q)):
        n, r0 = int(kv_len[b]), int(kv_start[b])
        Ka = LA.agent_keys(np.asarray(K_base[r0:r0 + n], float), np.asarray(K_lr[r0:r0 + n], float), B_k, int(agents[b]),
                           np.asarray(cos)[r0:], np.asarray(sin)[r0:])
        Va = LA.agent_values(V_base[r0:r0 + n], V_lr[r0:r0 + n], B, int(agents[b]))
        out.append(LA.attention(np.asarray(Q, float)[b:b + 1], Ka, Va, [n - 1], scale)[0])
    return np.stack(out)


def _mut_expand_values_at_source_rows(V_out, V_base, V_lr, B, src_start, length, agents, dst_start):
    # writes each request's expanded rows at its source rows instead of its destination rows
    return _orig_expand_values(V_out, V_base, V_lr, B, src_start, length, agents, src_start)


def _mut_expand_values_first_agent(V_out, V_base, V_lr, B, src_start, length, agents, dst_start):
    # expands every request with the first request's agent
    return _orig_expand_values(V_out, V_base, V_lr, B, src_start, length, [agents[0]] * len(agents), dst_start)


MUTANTS = {
    "expand_at_source_rows": ("expand_values", _mut_expand_values_at_source_rows),
    "expand_first_agent_only": ("expand_values", _mut_expand_values_first_agent),
    "decode_key_rope_absolute_rows": ("attn_decode_qkvo", _mut_decode_qkvo_absolute_rows),
    "rope_adjacent_pairs": ("rope_rotate", _mut_rope_adjacent_pairs),
    "rope_sign": ("rope_rotate", lambda Y, c, s_: _orig_rope(Y, c, -np.asarray(s_, np.float64))),
    "page_offset_off_by_one": ("gather_pages", lambda pages, row, n: np.asarray(pages)[
        np.asarray(row, np.int64)[np.arange(n) // np.asarray(pages).shape[1]],
        (np.arange(n) + 1) % np.asarray(pages).shape[1]]),
    "adapter_free_reads_agent_zero": ("agent_values", _mut_adapter_free_reads_agent_zero),
    "head_map_interleaved": ("kv_head_of", lambda h, group: h % group),
    "head_map_coarse": ("kv_head_of", lambda h, group: h // (2 * group)),
    "agent_cols_off_by_one": ("agent_columns", lambda a, r: slice(a * r + 1, (a + 1) * r + 1)),
    "agent_cols_wrong_agent": ("agent_columns", lambda a, r: slice(((a + 1) % 3) * r, ((a + 1) % 3 + 1) * r)),
    "mask_strict": ("visible", lambda q_pos, L: np.arange(L)[None, :] < np.asarray(q_pos)[:, None]),
    "mask_top_left": ("visible", lambda q_pos, L: np.arange(L)[None, :] <= (np.asarray(q_pos) - np.min(q_pos))[:, None]),
    "mask_none": ("visible", lambda q_pos, L: np.ones((len(np.asarray(q_pos)), L), bool)),
    "lr_term_dropped": ("agent_values", _mut_agent_values_no_lr),
    "lr_term_transposed": ("agent_values", _mut_agent_values_transposed),
    "lr_term_sign": ("agent_values", _mut_agent_values_minus),
    "softmax_unnormalised": ("softmax_rows", _mut_softmax_no_normalise),
    "softmax_sign": ("softmax_rows", _mut_softmax_flipped),
    "precompute_transposed_operand": ("lr_precompute", lambda X, A: np.asarray(X, float) @ np.asarray(A, float)[::-1]),
    "precompute_dropped_row": ("lr_precompute", lambda X, A: (np.asarray(X, float) @ np.asarray(A, float)) * (np.arange(len(X)) > 0)[:, None]),
}


def test_unmutated_oracle_passes_every_pin():
    assert not _some_pin_fails()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(LA, attr, fn)
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    assert _some_pin_fails(), f"mutant {name} passed every pin"


def test_scale_dropped_is_caught(monkeypatch):
    orig = LA.attention_probs
    monkeypatch.setattr(LA, "attention_probs", lambda Q, K, q_pos, scale, heads=None: orig(Q, K, q_pos, 1.0, heads))
    assert _some_pin_fails()
