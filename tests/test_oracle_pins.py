"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test checks the oracle against what the pages and the mathematics fix:
a library routine for the B = 0 special case, the associativity identity the
kernel is built on, invariants of softmax attention, closed forms, the
hand-derived fixtures in tests/golden/, and a pure-Python brute force.
``test_oracle_mutants.py`` plants mistakes in the oracle and checks that these
pins catch them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import bruteforce

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def small_shape(n_q=4, n_kv=2, d=8, r=2, N=3, d_model=16):
    return W.Shape(n_q=n_q, n_kv=n_kv, d_head=d, rank=r, n_agents=N, d_model=d_model, dtype="f32")


def f64(t):
    return t.as_f64()


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ----------------------------------------------------------------------------- golden fixtures
def _load_golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _load_golden()["prefill"], ids=lambda c: c["name"])
def test_golden_prefill(case):
    for agent, exp in case["expected"].items():
        O = oracle.attn_prefill(case["Q"], case["K"], case["V_base"], case["V_lr"], case["B"],
                                int(agent), case["L_P"], case["scale"])
        np.testing.assert_allclose(O, np.array(exp), rtol=0, atol=1e-13)


@pytest.mark.parametrize("case", _load_golden()["decode"], ids=lambda c: c["name"])
def test_golden_decode(case):
    O = oracle.attn_decode(case["Q"], np.array(case["K"]), np.array(case["V_base"]), np.array(case["V_lr"]),
                           case["B"], case["kv_start"], case["kv_len"], case["agent"], case["scale"])
    np.testing.assert_allclose(O, np.array(case["expected"]), rtol=0, atol=1e-13)


@pytest.mark.parametrize("case", _load_golden()["precompute"], ids=lambda c: c["name"])
def test_golden_precompute(case):
    np.testing.assert_array_equal(oracle.lr_precompute(case["X"], case["A"]), np.array(case["expected_product"]))
    cache = np.zeros((case["cache_rows"], case["cache_cols"]))
    got = oracle.lr_precompute_into(cache, case["X"], case["A"], case["out_rows"])
    np.testing.assert_array_equal(got, np.array(case["expected_cache"]))


# ----------------------------------------------------------------------------- library special case
@pytest.mark.parametrize("n_q,n_kv,L_P,L_C", [(4, 2, 5, 7), (8, 2, 0, 9), (6, 6, 11, 3), (4, 1, 3, 1)])
def test_zero_lora_is_standard_causal_gqa_attention(n_q, n_kv, L_P, L_C):
    """B = 0 (and separately V_lr = 0) must reduce to torch's scaled_dot_product_attention in float64
    with an explicit bottom-right causal mask and KV heads shared by contiguous query-head groups."""
    s = small_shape(n_q=n_q, n_kv=n_kv, d=16, r=4)
    c = W.random_prefill((900, n_q, n_kv, L_P, L_C), s, L_P, L_C, agent=1, b_std=1.0)
    L = L_P + L_C
    q = torch.from_numpy(f64(c.Q)).permute(1, 0, 2)          # [n_q, L_C, d]
    k = torch.from_numpy(f64(c.K)).permute(1, 0, 2)          # [n_kv, L, d]
    v = torch.from_numpy(f64(c.V)).permute(1, 0, 2)
    mask = torch.arange(L)[None, :] <= (L_P + torch.arange(L_C))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        q[None], k[None], v[None], attn_mask=mask, scale=s.scale, enable_gqa=True)[0].permute(1, 0, 2).numpy()
    # second library route: explicit repeat of each KV head over its query-head group
    G = n_q // n_kv
    ref2 = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(G, dim=0), v.repeat_interleave(G, dim=0), attn_mask=mask,
        scale=s.scale).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(ref, ref2, rtol=1e-13, atol=1e-14)
    zero_B = np.zeros_like(f64(c.B))
    O = oracle.attn_prefill(f64(c.Q), f64(c.K), f64(c.V), f64(c.V_lr), zero_B, 1, L_P, s.scale)
    assert rel_err(O, ref) <= 1e-12
    O2 = oracle.attn_prefill(f64(c.Q), f64(c.K), f64(c.V), np.zeros_like(f64(c.V_lr)), f64(c.B), 1, L_P, s.scale)
    assert rel_err(O2, ref) <= 1e-12
    # the adapter-free view (agent -1) attends the base cache alone, whatever V_lr and B hold
    O3 = oracle.attn_prefill(f64(c.Q), f64(c.K), f64(c.V), f64(c.V_lr), f64(c.B), oracle.ADAPTER_FREE, L_P, s.scale)
    assert rel_err(O3, ref) <= 1e-12
    Of = oracle.attn_factored(f64(c.Q), f64(c.K), f64(c.V), f64(c.V_lr), f64(c.B), oracle.ADAPTER_FREE,
                              L_P + np.arange(L_C), s.scale)
    assert rel_err(Of, ref) <= 1e-12


# ----------------------------------------------------------------------------- associativity
@pytest.mark.parametrize("agent", [0, 1, 2])
def test_associativity_materialised_equals_factored(agent):
    """P (V_lr B) = (P V_lr) B: expand-then-attend equals attend-then-expand (LRAgent, core method)."""
    s = small_shape(n_q=8, n_kv=2, d=16, r=4)
    c = W.random_prefill((901, agent), s, 9, 12, agent=agent, b_std=1.0)
    O = oracle.attn_prefill(f64(c.Q), f64(c.K), f64(c.V), f64(c.V_lr), f64(c.B), agent, c.L_P, s.scale)
    Of = oracle.attn_factored(f64(c.Q), f64(c.K), f64(c.V), f64(c.V_lr), f64(c.B), agent,
                              c.L_P + np.arange(c.L_C), s.scale)
    assert rel_err(O, Of) <= 1e-12


def test_projection_level_lora_split():
    """X (W0 + A_a B_a) = X W0 + (X A_a) B_a: the merged LoRA weight (LRAgent, Multi-LoRA prerequisite)
    against the oracle's precompute + agent value cache, for every agent."""
    s = W.TINY_SHAPE
    tw = W.tiny_workload()
    X = tw.X.as_f64()
    A = tw.A.as_f64()
    B = tw.B.as_f64()
    W0 = tw.W0_v.astype(np.float64)
    V_base = (X @ W0).reshape(-1, s.n_kv, s.d_head)
    V_lr = oracle.lr_precompute(X, A)
    for a in range(s.n_agents):
        merged = X @ (W0 + A[:, a * s.rank:(a + 1) * s.rank] @ B[a])
        got = oracle.agent_values(V_base, V_lr, B, a).reshape(X.shape[0], -1)
        assert rel_err(got, merged) <= 1e-12


# ----------------------------------------------------------------------------- invariants
def test_probability_rows_and_causal_zeros():
    s = small_shape(n_q=4, n_kv=2, d=8)
    c = W.random_prefill((902,), s, 6, 10)
    L = c.L_P + c.L_C
    qpos = c.L_P + np.arange(c.L_C)
    P = oracle.attention_probs(f64(c.Q), f64(c.K), qpos, s.scale)
    assert P.shape == (s.n_q, c.L_C, L)
    assert np.all(P >= 0)
    assert np.max(np.abs(P.sum(-1) - 1.0)) <= 1e-14
    hidden = np.arange(L)[None, :] > qpos[:, None]
    assert np.all(P[:, hidden] == 0.0)
    assert np.all(P[:, ~hidden] > 0.0)


def test_softmax_shift_invariance():
    g = np.random.default_rng(5)
    S = g.standard_normal((7, 13))
    mask = g.random((7, 13)) < 0.7
    mask[:, 0] = True
    shift = g.standard_normal((7, 1)) * 50
    np.testing.assert_allclose(oracle.softmax_rows(S + shift, mask), oracle.softmax_rows(S, mask), rtol=0, atol=1e-14)


def test_output_is_affine_in_B():
    s = small_shape(n_q=4, n_kv=2, d=8, r=2)
    c = W.random_prefill((903,), s, 4, 6, agent=2, b_std=1.0)
    g = np.random.default_rng(6)
    B1 = g.standard_normal(f64(c.B).shape)
    B2 = g.standard_normal(f64(c.B).shape)
    run = lambda B: oracle.attn_prefill(f64(c.Q), f64(c.K), f64(c.V), f64(c.V_lr), B, 2, c.L_P, s.scale)
    lhs = run(B1 + B2)
    rhs = run(B1) + run(B2) - run(np.zeros_like(B1))
    assert rel_err(lhs, rhs) <= 1e-12


def test_equal_queries_in_one_group_give_equal_outputs():
    s = small_shape(n_q=8, n_kv=2, d=8)
    c = W.random_prefill((904,), s, 3, 5)
    Q = f64(c.Q).copy()
    Q[:, 1] = Q[:, 0]   # heads 0..3 share KV head 0
    Q[:, 5] = Q[:, 0]   # head 5 reads KV head 1
    O = oracle.attn_prefill(Q, f64(c.K), f64(c.V), f64(c.V_lr), f64(c.B), 0, c.L_P, s.scale)
    np.testing.assert_array_equal(O[:, 1], O[:, 0])
    assert np.max(np.abs(O[:, 5] - O[:, 0])) > 1e-3


def test_decode_equals_last_prefill_row():
    s = small_shape(n_q=4, n_kv=2, d=8)
    L = 13
    c = W.random_prefill((905,), s, L - 1, 1, agent=1)
    Op = oracle.attn_prefill(f64(c.Q), f64(c.K), f64(c.V), f64(c.V_lr), f64(c.B), 1, L - 1, s.scale)
    Od = oracle.attn_decode(f64(c.Q), f64(c.K), f64(c.V), f64(c.V_lr), f64(c.B), [0], [L], [1], s.scale)
    assert rel_err(Od, Op) <= 1e-13


def test_chunk_split_equivalence():
    """Prefilling L_C = c1 + c2 tokens equals prefilling c1 then c2 with L_P advanced by c1."""
    s = small_shape(n_q=4, n_kv=2, d=8)
    c = W.random_prefill((906,), s, 5, 11, agent=2)
    args = (f64(c.K), f64(c.V), f64(c.V_lr), f64(c.B), 2)
    full = oracle.attn_prefill(f64(c.Q), *args, c.L_P, s.scale)
    first = oracle.attn_prefill(f64(c.Q)[:4], *args, c.L_P, s.scale)
    second = oracle.attn_prefill(f64(c.Q)[4:], *args, c.L_P + 4, s.scale)
    assert rel_err(np.concatenate([first, second]), full) <= 1e-13


# ----------------------------------------------------------------------------- closed forms
def test_single_key_returns_its_value_row():
    s = small_shape(n_q=4, n_kv=2, d=8)
    c = W.random_prefill((907,), s, 0, 1, agent=1)
    O = oracle.attn_prefill(f64(c.Q), f64(c.K), f64(c.V), f64(c.V_lr), f64(c.B), 1, 0, s.scale)
    Va = f64(c.V)[0] + (f64(c.V_lr)[0, 2:4] @ f64(c.B)[1]).reshape(s.n_kv, s.d_head)
    for h in range(s.n_q):
        np.testing.assert_allclose(O[0, h], Va[h // 2], rtol=0, atol=1e-15)


def test_zero_query_averages_visible_rows():
    s = small_shape(n_q=2, n_kv=1, d=8, r=2)
    c = W.random_prefill((908,), s, 4, 6, agent=0)
    Q = np.zeros_like(f64(c.Q))
    O = oracle.attn_prefill(Q, f64(c.K), f64(c.V), f64(c.V_lr), f64(c.B), 0, c.L_P, s.scale)
    Va = f64(c.V)[:, 0] + f64(c.V_lr)[:, 0:2] @ f64(c.B)[0]
    for i in range(c.L_C):
        np.testing.assert_allclose(O[i, 0], Va[: c.L_P + i + 1].mean(0), rtol=0, atol=1e-14)


def test_dominant_score_selects_its_row():
    """One visible score above all others by >= 60 gives that key's value row to within e^-60."""
    s = small_shape(n_q=1, n_kv=1, d=8, r=2)
    c = W.random_prefill((909,), s, 7, 1, agent=0)
    Q = np.zeros((1, 1, 8))
    Q[0, 0, 0] = 1.0
    K = np.zeros_like(f64(c.K))
    K[3, 0, 0] = 60.0 / s.scale
    O = oracle.attn_prefill(Q, K, f64(c.V), f64(c.V_lr), f64(c.B), 0, c.L_P, s.scale)
    Va3 = f64(c.V)[3, 0] + f64(c.V_lr)[3, 0:2] @ f64(c.B)[0]
    assert np.max(np.abs(O[0, 0] - Va3)) <= 8 * math.exp(-60) * (1 + np.max(np.abs(f64(c.V))) * 10)


# ----------------------------------------------------------------------------- brute force
@pytest.mark.parametrize("n_q,n_kv,d,r,L_P,L_C,agent", [
    (4, 2, 8, 2, 3, 5, 0), (4, 2, 8, 2, 3, 5, 2), (8, 2, 4, 4, 0, 7, 1), (2, 2, 5, 1, 10, 6, 1), (4, 1, 8, 3, 15, 1, 2)])
def test_bruteforce_prefill(n_q, n_kv, d, r, L_P, L_C, agent):
    s = small_shape(n_q=n_q, n_kv=n_kv, d=d, r=r)
    c = W.random_prefill((910, n_q, d, r, L_P, L_C), s, L_P, L_C, agent=agent, b_std=0.7)
    O = oracle.attn_prefill(f64(c.Q), f64(c.K), f64(c.V), f64(c.V_lr), f64(c.B), agent, L_P, s.scale)
    ref = bruteforce.prefill(f64(c.Q), f64(c.K), f64(c.V), f64(c.V_lr), f64(c.B), agent, L_P, s.scale)
    assert rel_err(O, ref) <= 1e-13


def test_bruteforce_decode_with_shared_and_empty_ranges():
    s = small_shape(n_q=4, n_kv=2, d=6, r=2)
    c = W.random_decode((911,), s, kv_lens=[9, 16, 0, 1, 5], kv_starts=[0, 0, 3, 15, 4], rows=16,
                        agents=[0, 1, 2, 1, 2], b_std=0.7)
    O = oracle.attn_decode(f64(c.Q), f64(c.K), f64(c.V), f64(c.V_lr), f64(c.B), c.kv_start, c.kv_len, c.agent, s.scale)
    ref = bruteforce.decode(f64(c.Q), f64(c.K), f64(c.V), f64(c.V_lr), f64(c.B), c.kv_start, c.kv_len, c.agent, s.scale)
    assert rel_err(O, ref) <= 1e-13
    assert np.all(O[2] == 0.0)


def test_bruteforce_prefill_varlen_batch():
    """Several prefills in one batch (own query rows, cache offsets, L_P and agent; shared cache rows;
    an empty chunk; the adapter-free view) against the brute force, request by request."""
    s = small_shape(n_q=4, n_kv=2, d=6, r=2)
    rng = np.random.default_rng(913)
    rows, q_rows = 30, 20
    K = rng.standard_normal((rows, s.n_kv, s.d_head))
    V = rng.standard_normal((rows, s.n_kv, s.d_head))
    Vlr = rng.standard_normal((rows, s.n_agents * s.rank))
    B = 0.7 * rng.standard_normal((s.n_agents, s.rank, s.d_kv))
    Q = rng.standard_normal((q_rows, s.n_q, s.d_head))
    q_start, q_len = [0, 5, 9, 9, 14], [5, 4, 0, 3, 6]
    kv_start, kv_prefix = [0, 0, 7, 10, 2], [3, 12, 4, 0, 22]
    agents = [1, oracle.ADAPTER_FREE, 0, 2, 0]
    O = oracle.attn_prefill_varlen(Q, K, V, Vlr, B, q_start, q_len, kv_start, kv_prefix, agents, s.scale)
    for b in range(5):
        q0, n, k0, lp = q_start[b], q_len[b], kv_start[b], kv_prefix[b]
        if n == 0:
            continue
        ref = bruteforce.prefill(Q[q0:q0 + n], K[k0:k0 + lp + n], V[k0:k0 + lp + n], Vlr[k0:k0 + lp + n], B,
                                 agents[b], lp, s.scale)
        assert rel_err(O[q0:q0 + n], ref) <= 1e-13, b
    assert np.all(O[12:14] == 0.0)   # rows no request covers


def test_bruteforce_decode_paged_cache():
    """A paged cache (pages of 4 rows, shuffled, one page shared by two requests as a common prefix)
    against the brute force on the same rows laid out contiguously by hand."""
    s = small_shape(n_q=4, n_kv=2, d=6, r=2)
    rng = np.random.default_rng(914)
    P, n_pages = 4, 9
    Kp = rng.standard_normal((n_pages, P, s.n_kv, s.d_head))
    Vp = rng.standard_normal((n_pages, P, s.n_kv, s.d_head))
    Lp = rng.standard_normal((n_pages, P, s.n_agents * s.rank))
    B = 0.7 * rng.standard_normal((s.n_agents, s.rank, s.d_kv))
    Q = rng.standard_normal((3, s.n_q, s.d_head))
    table = np.array([[5, 2, 7, 0], [5, 8, 1, 0], [3, 0, 0, 0]])
    kv_len, agents = [14, 9, 0], [2, oracle.ADAPTER_FREE, 1]
    O = oracle.attn_decode_paged(Q, Kp, Vp, Lp, B, table, kv_len, agents, s.scale)
    for b in range(2):
        pages = table[b][:(kv_len[b] + P - 1) // P]
        K = np.concatenate([Kp[i] for i in pages])[:kv_len[b]]
        V = np.concatenate([Vp[i] for i in pages])[:kv_len[b]]
        L = np.concatenate([Lp[i] for i in pages])[:kv_len[b]]
        ref = bruteforce.decode(Q[b:b + 1], K, V, L, B, [0], [kv_len[b]], [agents[b]], s.scale)
        assert rel_err(O[b:b + 1], ref) <= 1e-13, b
    assert np.all(O[2] == 0.0)


def test_bruteforce_prefill_paged_cache():
    """Two prefills over a paged cache (pages of 4 rows, shuffled, a shared first page) against the
    brute force on the same rows laid out contiguously by hand."""
    s = small_shape(n_q=4, n_kv=2, d=6, r=2)
    rng = np.random.default_rng(915)
    P, n_pages = 4, 8
    Kp = rng.standard_normal((n_pages, P, s.n_kv, s.d_head))
    Vp = rng.standard_normal((n_pages, P, s.n_kv, s.d_head))
    Lp = rng.standard_normal((n_pages, P, s.n_agents * s.rank))
    B = 0.7 * rng.standard_normal((s.n_agents, s.rank, s.d_kv))
    Q = rng.standard_normal((12, s.n_q, s.d_head))
    table = np.array([[6, 1, 3, 0], [6, 4, 7, 2]])
    q_start, q_len, kv_prefix, agents = [0, 5], [5, 7], [6, 9], [1, oracle.ADAPTER_FREE]
    O = oracle.attn_prefill_paged(Q, Kp, Vp, Lp, B, table, q_start, q_len, kv_prefix, agents, s.scale)
    for b in range(2):
        L = kv_prefix[b] + q_len[b]
        pages = table[b][:(L + P - 1) // P]
        K = np.concatenate([Kp[i] for i in pages])[:L]
        V = np.concatenate([Vp[i] for i in pages])[:L]
        Vl = np.concatenate([Lp[i] for i in pages])[:L]
        q0 = q_start[b]
        ref = bruteforce.prefill(Q[q0:q0 + q_len[b]], K, V, Vl, B, agents[b], kv_prefix[b], s.scale)
        assert rel_err(O[q0:q0 + q_len[b]], ref) <= 1e-13, b


def _rope_tables(L, d, base=10000.0):
    ang = np.arange(L)[:, None] * base ** (-2.0 * np.arange(d // 2)[None, :] / d)
    return np.cos(ang), np.sin(ang)


@pytest.mark.parametrize("agent", [0, 2, -1])
def test_bruteforce_prefill_with_key_lora(agent):
    """LoRA on the keys too (the qkvo configuration): rotated rank-r key part, against the brute force."""
    s = small_shape(n_q=4, n_kv=2, d=6, r=2)
    rng = np.random.default_rng(916 + agent)
    L_P, L_C = 5, 4
    L = L_P + L_C
    K = rng.standard_normal((L, s.n_kv, s.d_head))
    V = rng.standard_normal((L, s.n_kv, s.d_head))
    Klr = rng.standard_normal((L, s.n_agents * s.rank))
    Vlr = rng.standard_normal((L, s.n_agents * s.rank))
    B = 0.7 * rng.standard_normal((s.n_agents, s.rank, s.d_kv))
    Bk = 0.7 * rng.standard_normal((s.n_agents, s.rank, s.d_kv))
    Q = rng.standard_normal((L_C, s.n_q, s.d_head))
    cos, sin = _rope_tables(L, s.d_head)
    O = oracle.attn_prefill_qkvo(Q, K, V, Vlr, Klr, B, Bk, cos, sin, agent, L_P, s.scale)
    ref = bruteforce.prefill_qkvo(Q, K, V, Klr, Vlr, B, Bk, cos, sin, agent, L_P, s.scale)
    assert rel_err(O, ref) <= 1e-13


def test_bruteforce_decode_with_key_lora():
    """Decode with LoRA on the keys: requests over shared and offset rows, mixed agents (incl. the
    adapter-free view); each request's keys are rotated from table position 0 at its first row."""
    s = small_shape(n_q=4, n_kv=2, d=6, r=2)
    rng = np.random.default_rng(918)
    rows = 12
    K = rng.standard_normal((rows, s.n_kv, s.d_head))
    V = rng.standard_normal((rows, s.n_kv, s.d_head))
    Klr = rng.standard_normal((rows, s.n_agents * s.rank))
    Vlr = rng.standard_normal((rows, s.n_agents * s.rank))
    B = 0.7 * rng.standard_normal((s.n_agents, s.rank, s.d_kv))
    Bk = 0.7 * rng.standard_normal((s.n_agents, s.rank, s.d_kv))
    Q = rng.standard_normal((5, s.n_q, s.d_head))
    cos, sin = _rope_tables(rows, s.d_head)
    kv_start, kv_len, agents = [0, 0, 5, 5, 11], [12, 12, 7, 7, 1], [1, -1, 2, 0, 2]
    O = oracle.attn_decode_qkvo(Q, K, V, Vlr, Klr, B, Bk, cos, sin, kv_start, kv_len, agents, s.scale)
    ref = bruteforce.decode_qkvo(Q, K, V, Klr, Vlr, B, Bk, cos, sin, kv_start, kv_len, agents, s.scale)
    assert rel_err(O, ref) <= 1e-13
    # a request at offset 5 uses table positions 0 .. 6, not 5 .. 11: same keys as a request at 0
    O5 = oracle.attn_decode_qkvo(Q[2:3], K[5:], V[5:], Vlr[5:], Klr[5:], B, Bk, cos, sin, [0], [7], [2], s.scale)
    assert rel_err(O[2:3], O5) <= 1e-14
    # B_k = 0 is the plain decode
    base = oracle.attn_decode(Q, K, V, Vlr, B, kv_start, kv_len, agents, s.scale)
    Oz = oracle.attn_decode_qkvo(Q, K, V, Vlr, Klr, B, np.zeros_like(Bk), cos, sin, kv_start, kv_len, agents, s.scale)
    assert rel_err(Oz, base) <= 1e-13


def test_key_lora_special_cases():
    """B_k = 0 is the value-only method; cos = 1, sin = 0 is an unrotated LoRA key; a rotation keeps
    every pair's norm; with K_lr = 0 the keys are the base keys whatever the tables."""
    s = small_shape(n_q=4, n_kv=2, d=8, r=2)
    c = W.random_prefill((917,), s, 6, 5, agent=1, b_std=0.7)
    rng = np.random.default_rng(917)
    L = 11
    Klr = rng.standard_normal((L, s.n_agents * s.rank))
    Bk = 0.7 * rng.standard_normal((s.n_agents, s.rank, s.d_kv))
    cos, sin = _rope_tables(L, s.d_head)
    args = (f64(c.Q), f64(c.K), f64(c.V), f64(c.V_lr))
    base = oracle.attn_prefill(*args, f64(c.B), 1, 6, s.scale)
    assert rel_err(oracle.attn_prefill_qkvo(*args, Klr, f64(c.B), np.zeros_like(Bk), cos, sin, 1, 6, s.scale), base) <= 1e-13
    assert rel_err(oracle.attn_prefill_qkvo(*args, np.zeros_like(Klr), f64(c.B), Bk, cos, sin, 1, 6, s.scale), base) <= 1e-13
    Ka = oracle.agent_keys(f64(c.K), Klr, Bk, 1, np.ones_like(cos), np.zeros_like(sin))
    plain = f64(c.K) + (Klr[:, 2:4] @ Bk[1]).reshape(L, s.n_kv, s.d_head)
    assert rel_err(Ka, plain) <= 1e-14
    Y = rng.standard_normal((L, s.n_kv, s.d_head))
    R = oracle.rope_rotate(Y, cos, sin)
    h = s.d_head // 2
    np.testing.assert_allclose(R[..., :h] ** 2 + R[..., h:] ** 2, Y[..., :h] ** 2 + Y[..., h:] ** 2, rtol=1e-12)


def test_bruteforce_decode_mixed_adapted_and_adapter_free():
    """Double batching (PReCache paper page, section 3): adapted and adapter-free requests over the
    same rows in one batch; the adapter-free ones (agent -1) see the base cache alone."""
    s = small_shape(n_q=4, n_kv=2, d=6, r=2)
    c = W.random_decode((912,), s, kv_lens=[12, 12, 7, 7, 1], kv_starts=[0, 0, 5, 5, 11], rows=12,
                        agents=[1, -1, -1, 2, -1], b_std=0.7)
    O = oracle.attn_decode(f64(c.Q), f64(c.K), f64(c.V), f64(c.V_lr), f64(c.B), c.kv_start, c.kv_len, c.agent, s.scale)
    ref = bruteforce.decode(f64(c.Q), f64(c.K), f64(c.V), f64(c.V_lr), f64(c.B), c.kv_start, c.kv_len, c.agent, s.scale)
    assert rel_err(O, ref) <= 1e-13
    # the adapted request differs from the adapter-free one over the same rows with the same query
    Q2 = f64(c.Q).copy()
    Q2[1] = Q2[0]
    O2 = oracle.attn_decode(Q2, f64(c.K), f64(c.V), f64(c.V_lr), f64(c.B), c.kv_start, c.kv_len, c.agent, s.scale)
    assert np.max(np.abs(O2[0] - O2[1])) > 1e-3


def test_precompute_triple_loop_and_one_hot():
    g = np.random.default_rng(7)
    X = g.standard_normal((6, 11))
    A = g.standard_normal((11, 9))
    assert rel_err(oracle.lr_precompute(X, A), bruteforce.precompute(X, A)) <= 1e-14
    onehot = np.zeros((11, 4))
    cols = [3, 0, 10, 3]
    for n, c in enumerate(cols):
        onehot[c, n] = 1.0
    np.testing.assert_array_equal(oracle.lr_precompute(X, onehot), X[:, cols])


def test_precompute_scatter_leaves_other_rows_and_columns():
    g = np.random.default_rng(8)
    X = g.standard_normal((3, 5))
    A = g.standard_normal((5, 4))
    cache = g.standard_normal((7, 6))
    got = oracle.lr_precompute_into(cache, X, A, [6, 0, 2])
    np.testing.assert_array_equal(got[[1, 3, 4, 5]], cache[[1, 3, 4, 5]])
    np.testing.assert_array_equal(got[:, 4:], cache[:, 4:])
    np.testing.assert_array_equal(got[[6, 0, 2], :4], X @ A)


def test_bruteforce_expand_values_and_expand_then_attend():
    """Expand-then-attend (the order the LRAgent page's Flash-LoRA-Attention avoids): the expansion
    against the brute force on a batch with shared sources, distinct destinations, an adapter-free
    request and an empty one; rows no request names keep their values. Attending the expanded rows
    with no LR term (agent -1) gives the adapted decode."""
    s = small_shape(n_q=4, n_kv=2, d=6, r=2)
    c = W.random_decode((913,), s, kv_lens=[5, 5, 3, 0, 4], kv_starts=[0, 0, 6, 2, 7], rows=12,
                        agents=[2, 0, -1, 1, 1], b_std=0.8)
    dst = [12, 0, 6, 3, 17]
    g = np.random.default_rng(913)
    V_out = g.standard_normal((22, s.n_kv, s.d_head))
    got = oracle.expand_values(V_out, f64(c.V), f64(c.V_lr), f64(c.B), c.kv_start, c.kv_len, c.agent, dst)
    ref = bruteforce.expand_values(V_out, f64(c.V), f64(c.V_lr), f64(c.B), c.kv_start, c.kv_len, c.agent, dst)
    assert rel_err(got, ref) <= 1e-14
    np.testing.assert_array_equal(got[[5, 9, 10, 11, 21]], V_out[[5, 9, 10, 11, 21]])
    np.testing.assert_array_equal(got[6:9], f64(c.V)[6:9])     # agent -1 copies the base rows
    # attention over the expanded rows without the LR term equals the adapted decode
    K2 = np.zeros((22, s.n_kv, s.d_head))
    for b in range(5):
        n = int(c.kv_len[b])
        K2[dst[b]:dst[b] + n] = f64(c.K)[int(c.kv_start[b]):int(c.kv_start[b]) + n]
    none = np.full(5, oracle.ADAPTER_FREE)
    O_exp = oracle.attn_decode(f64(c.Q), K2, got, np.zeros((22, f64(c.V_lr).shape[1])), f64(c.B), dst, c.kv_len,
                               none, s.scale)
    O_ref = bruteforce.decode(f64(c.Q), f64(c.K), f64(c.V), f64(c.V_lr), f64(c.B), c.kv_start, c.kv_len, c.agent, s.scale)
    assert rel_err(O_exp, O_ref) <= 1e-13
