"""Seeded random configurations of the decode, the prefill and the value expansion against the fp64
oracle (needs an MI355X and liblra.so).

Each case draws its shape (element type, KV heads, group size, d_head, rank), its lengths (ragged,
including empty requests and lengths on and around tile and split edges), its agents (including the
adapter-free view) and its split size from one seed, so a failure names a reproducible case.
"""
import numpy as np
import pytest
import torch

import oracle
import rank_kv_cache_amd as lra
import workloads as W
from tests.gpu_util import check, dev, dev_idx, host64, say

pytestmark = pytest.mark.gpu

EDGES = [0, 1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512, 513]


def draw_shape(g: np.random.Generator) -> W.Shape:
    dtype = "f32" if g.random() < 0.25 else "bf16"
    n_kv = int(g.choice([1, 2, 3, 4, 8]))
    G = int(g.integers(1, 9))
    d = int(g.choice([64, 128]))
    r = int(g.choice([8, 16]))
    return W.Shape(n_q=n_kv * G, n_kv=n_kv, d_head=d, rank=r, n_agents=int(g.integers(1, 5)), d_model=256,
                   dtype=dtype)


def draw_len(g: np.random.Generator, hi: int) -> int:
    if g.random() < 0.4:
        return int(g.choice(EDGES)) + int(g.choice([0, 0, 1024, 2048]))
    return int(g.integers(0, hi))


@pytest.mark.parametrize("seed", range(48))
def test_random_decode(seed):
    g = np.random.default_rng(1000 + seed)
    s = draw_shape(g)
    batch = int(g.integers(1, 7))
    lens = [draw_len(g, 3000) for _ in range(batch)]
    agents = [int(g.integers(-1, s.n_agents)) for _ in range(batch)]
    split = int(g.choice([0, 0, 64, 128, 192, 320, 1024]))
    say(f"random decode seed={seed} {s.dtype} n_q={s.n_q} n_kv={s.n_kv} d={s.d_head} r={s.rank} N={s.n_agents} "
        f"lens={lens} agents={agents} split={split}")
    c = W.random_decode((400, seed), s, lens, agents=agents, b_std=0.3)
    O = lra.lra_attn_decode(dev(c.Q), dev(c.K), dev(c.V), dev(c.V_lr), dev_idx(c.kv_start, torch.int64),
                            dev_idx(c.kv_len, torch.int32), max(c.max_kv_len, 1), dev(c.B),
                            dev_idx(c.agent, torch.int32), s.scale, split)
    torch.cuda.synchronize()
    got = host64(O)
    ref = oracle.attn_decode(c.Q.as_f64(), c.K.as_f64(), c.V.as_f64(), c.V_lr.as_f64(), c.B.as_f64(), c.kv_start,
                             c.kv_len, c.agent, s.scale)
    live = [b for b in range(batch) if lens[b] > 0]
    if live:
        check(got[live], ref[live], s.dtype, f"seed {seed}")
    for b in range(batch):
        if lens[b] == 0:
            assert np.all(got[b] == 0.0)


@pytest.mark.parametrize("seed", range(32))
def test_random_prefill(seed):
    g = np.random.default_rng(2000 + seed)
    s = draw_shape(g)
    L_P = draw_len(g, 700) % 1200
    L_C = max(1, draw_len(g, 400) % 600)
    agent = int(g.integers(-1, s.n_agents))
    say(f"random prefill seed={seed} {s.dtype} n_q={s.n_q} n_kv={s.n_kv} d={s.d_head} r={s.rank} N={s.n_agents} "
        f"L_P={L_P} L_C={L_C} agent={agent}")
    c = W.random_prefill((401, seed), s, L_P, L_C, agent=agent, b_std=0.3)
    O = lra.lra_attn_prefill(dev(c.Q), L_P, dev(c.K), dev(c.V), dev(c.V_lr), dev(c.B), agent, s.scale)
    torch.cuda.synchronize()
    ref = oracle.attn_prefill(c.Q.as_f64(), c.K.as_f64(), c.V.as_f64(), c.V_lr.as_f64(), c.B.as_f64(), agent, L_P,
                              s.scale)
    check(host64(O), ref, s.dtype, f"seed {seed}")


@pytest.mark.parametrize("seed", range(24))
def test_random_expand_then_decode_head_major(seed):
    """Random batches: the expansion element by element, the adapter-free decode over the expanded
    rows against the adapted oracle, and the head-major decode bit-identical to the token-major one."""
    g = np.random.default_rng(3000 + seed)
    s = draw_shape(g)
    batch = int(g.integers(1, 6))
    lens = [max(1, draw_len(g, 2500)) for _ in range(batch)]
    agents = [int(g.integers(-1, s.n_agents)) for _ in range(batch)]
    say(f"random expand/head-major seed={seed} {s.dtype} n_q={s.n_q} n_kv={s.n_kv} d={s.d_head} r={s.rank} "
        f"N={s.n_agents} lens={lens} agents={agents}")
    c = W.random_decode((402, seed), s, lens, agents=agents, b_std=0.3)
    ks, kl, ag = dev_idx(c.kv_start, torch.int64), dev_idx(c.kv_len, torch.int32), dev_idx(c.agent, torch.int32)
    K, V, L, B, Q = dev(c.K), dev(c.V), dev(c.V_lr), dev(c.B), dev(c.Q)
    V_exp = lra.lra_expand_values(V, L, B, ks, kl, ag, c.max_kv_len, ks)
    none = torch.full((batch,), lra.ADAPTER_FREE, dtype=torch.int32, device="cuda")
    O_x = lra.lra_attn_decode(Q, K, V_exp, L, ks, kl, c.max_kv_len, B, none, s.scale)
    O_t = lra.lra_attn_decode(Q, K, V, L, ks, kl, c.max_kv_len, B, ag, s.scale)
    Khm, Vhm = K.transpose(0, 1).contiguous(), V.transpose(0, 1).contiguous()
    O_h = lra.lra_attn_decode_strided(Q, Khm.transpose(0, 1), Vhm.transpose(0, 1), L, ks, kl, c.max_kv_len, B, ag,
                                      s.scale)
    torch.cuda.synchronize()
    ref_v = oracle.expand_values(np.zeros(tuple(V.shape)), c.V.as_f64(), c.V_lr.as_f64(), c.B.as_f64(), c.kv_start,
                                 c.kv_len, c.agent, c.kv_start)
    check(host64(V_exp), ref_v, s.dtype, f"seed {seed} expansion")
    ref = oracle.attn_decode(c.Q.as_f64(), c.K.as_f64(), c.V.as_f64(), c.V_lr.as_f64(), c.B.as_f64(), c.kv_start,
                             c.kv_len, c.agent, s.scale)
    check(host64(O_x), ref, s.dtype, f"seed {seed} expand-then-decode")
    check(host64(O_t), ref, s.dtype, f"seed {seed} decode")
    assert np.array_equal(host64(O_h), host64(O_t))


def draw_bf16_shape(g: np.random.Generator) -> W.Shape:
    s = draw_shape(g)
    return W.Shape(n_q=s.n_q, n_kv=s.n_kv, d_head=s.d_head, rank=s.rank, n_agents=s.n_agents, d_model=256,
                   dtype="bf16")


@pytest.mark.parametrize("seed", range(16))
def test_random_paged_decode(seed):
    """Random paged batches (page size, shared prefix pages, shuffled pages), token-major and
    head-major pages (bit-identical), against the oracle."""
    g = np.random.default_rng(4000 + seed)
    s = draw_bf16_shape(g)
    P = int(g.choice([32, 64, 128]))
    batch = int(g.integers(1, 6))
    lens = [draw_len(g, 2500) for _ in range(batch)]
    if max(lens) == 0:
        lens[0] = 1   # the block table needs one page
    shared = int(g.integers(0, 2)) if min(lens) > P else 0
    agents = [int(g.integers(-1, s.n_agents)) for _ in range(batch)]
    say(f"random paged decode seed={seed} n_q={s.n_q} n_kv={s.n_kv} d={s.d_head} r={s.rank} N={s.n_agents} P={P} "
        f"lens={lens} shared={shared} agents={agents}")
    c = W.random_paged_decode((403, seed), s, lens, P, agents=agents, shared_prefix_pages=shared)
    Q, Kp, Vp, Lp, B = dev(c.Q), dev(c.K_pages), dev(c.V_pages), dev(c.Vlr_pages), dev(c.B)
    table, kl, ag = dev_idx(c.block_table, torch.int32), dev_idx(c.kv_len, torch.int32), dev_idx(c.agents, torch.int32)
    mx = max(c.max_kv_len, 1)
    O = lra.lra_attn_decode_paged(Q, Kp, Vp, Lp, table, kl, mx, B, ag, s.scale)
    Khnd, Vhnd = Kp.transpose(1, 2).contiguous(), Vp.transpose(1, 2).contiguous()
    O_h = lra.lra_attn_decode_paged_strided(Q, Khnd.transpose(1, 2), Vhnd.transpose(1, 2), Lp, table, kl, mx, B, ag,
                                            s.scale)
    torch.cuda.synchronize()
    got = host64(O)
    assert np.array_equal(host64(O_h), got)
    ref = oracle.attn_decode_paged(c.Q.as_f64(), c.K_pages.as_f64(), c.V_pages.as_f64(), c.Vlr_pages.as_f64(),
                                   c.B.as_f64(), c.block_table, c.kv_len, c.agents, s.scale)
    live = [b for b in range(batch) if lens[b] > 0]
    if live:
        check(got[live], ref[live], "bf16", f"seed {seed}")


@pytest.mark.parametrize("seed", range(16))
def test_random_prefill_varlen(seed):
    g = np.random.default_rng(5000 + seed)
    s = draw_shape(g)
    nreq = int(g.integers(1, 5))
    reqs = [(draw_len(g, 500) % 900, max(1, draw_len(g, 300) % 400), int(g.integers(-1, s.n_agents)))
            for _ in range(nreq)]
    say(f"random varlen prefill seed={seed} {s.dtype} n_q={s.n_q} n_kv={s.n_kv} d={s.d_head} r={s.rank} "
        f"N={s.n_agents} requests={reqs}")
    c = W.random_prefill_batch((404, seed), s, reqs)
    O = lra.lra_attn_prefill_varlen(dev(c.Q), dev_idx(c.q_start, torch.int64), dev_idx(c.q_len, torch.int32),
                                    c.max_q_len, dev(c.K), dev(c.V), dev(c.V_lr), dev_idx(c.kv_start, torch.int64),
                                    dev_idx(c.kv_prefix, torch.int32), dev(c.B), dev_idx(c.agents, torch.int32),
                                    s.scale)
    torch.cuda.synchronize()
    got = host64(O)
    ref = oracle.attn_prefill_varlen(c.Q.as_f64(), c.K.as_f64(), c.V.as_f64(), c.V_lr.as_f64(), c.B.as_f64(),
                                     c.q_start, c.q_len, c.kv_start, c.kv_prefix, c.agents, s.scale)
    rows = np.concatenate([np.arange(int(c.q_start[b]), int(c.q_start[b]) + int(c.q_len[b])) for b in range(nreq)])
    check(got[rows], ref[rows], s.dtype, f"seed {seed}")


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


@pytest.mark.parametrize("seed", range(10))
def test_random_qkvo_decode_and_prefill(seed):
    """LoRA on the keys as well: a random decode batch and a random chunked prefill against the oracle."""
    g = np.random.default_rng(6000 + seed)
    s = draw_bf16_shape(g)
    batch = int(g.integers(1, 5))
    lens = [max(1, draw_len(g, 1500)) for _ in range(batch)]
    agents = [int(g.integers(-1, s.n_agents)) for _ in range(batch)]
    split = int(g.choice([0, 64, 256]))
    say(f"random qkvo decode seed={seed} n_q={s.n_q} n_kv={s.n_kv} d={s.d_head} r={s.rank} N={s.n_agents} "
        f"lens={lens} agents={agents} split={split}")
    c = W.random_decode_qkvo((405, seed), s, lens, agents=agents)
    b = c.base
    O = lra.lra_attn_decode_qkvo(dev(b.Q), dev(b.K), dev(b.V), dev(b.V_lr), dev(c.K_lr),
                                 dev_idx(b.kv_start, torch.int64), dev_idx(b.kv_len, torch.int32), b.max_kv_len,
                                 dev(b.B), dev(c.B_k), _f32(c.cos), _f32(c.sin), dev_idx(b.agent, torch.int32),
                                 s.scale, split)
    torch.cuda.synchronize()
    ref = oracle.attn_decode_qkvo(b.Q.as_f64(), b.K.as_f64(), b.V.as_f64(), b.V_lr.as_f64(), c.K_lr.as_f64(),
                                  b.B.as_f64(), c.B_k.as_f64(), c.cos, c.sin, b.kv_start, b.kv_len, b.agent, s.scale)
    check(host64(O), ref, "bf16", f"seed {seed} decode")
    L_P = draw_len(g, 600) % 900
    L_C = max(1, draw_len(g, 300) % 400)
    agent = int(g.integers(-1, s.n_agents))
    say(f"random qkvo prefill seed={seed} L_P={L_P} L_C={L_C} agent={agent}")
    cp = W.random_prefill_qkvo((406, seed), s, L_P, L_C, agent=agent)
    bp = cp.base
    O = lra.lra_attn_prefill_qkvo(dev(bp.Q), L_P, dev(bp.K), dev(bp.V), dev(bp.V_lr), dev(cp.K_lr), dev(bp.B),
                                  dev(cp.B_k), _f32(cp.cos), _f32(cp.sin), agent, s.scale)
    torch.cuda.synchronize()
    ref = oracle.attn_prefill_qkvo(bp.Q.as_f64(), bp.K.as_f64(), bp.V.as_f64(), bp.V_lr.as_f64(), cp.K_lr.as_f64(),
                                   bp.B.as_f64(), cp.B_k.as_f64(), cp.cos, cp.sin, agent, L_P, s.scale)
    check(host64(O), ref, "bf16", f"seed {seed} prefill")
