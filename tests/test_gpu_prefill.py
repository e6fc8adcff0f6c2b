"""GPU parity of lra_attn_prefill against the fp64 oracle (needs an MI355X and liblra.so)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import rank_kv_cache_amd as lra
import workloads as W
from tests.gpu_util import check, dev, dev_idx, host64, say

pytestmark = pytest.mark.gpu


def run_prefill(c: W.PrefillCase, agent=None):
    s = c.shape
    O = lra.lra_attn_prefill(dev(c.Q), c.L_P, dev(c.K), dev(c.V), dev(c.V_lr), dev(c.B),
                             c.agent if agent is None else agent, s.scale)
    torch.cuda.synchronize()
    return host64(O)


def ref_prefill(c: W.PrefillCase, agent=None, rows=None, heads=None):
    L = c.L_P + c.L_C
    return oracle.attn_prefill(c.Q.as_f64(), W.HostTensor(c.K.data[:L], c.K.dtype).as_f64(),
                               W.HostTensor(c.V.data[:L], c.V.dtype).as_f64(),
                               W.HostTensor(c.V_lr.data[:L], c.V_lr.dtype).as_f64(), c.B.as_f64(),
                               c.agent if agent is None else agent, c.L_P, c.shape.scale, rows=rows, heads=heads)


def run_prefill_varlen(c: W.PrefillBatch, max_q_len=None, O=None):
    s = c.shape
    O = lra.lra_attn_prefill_varlen(dev(c.Q), dev_idx(c.q_start, torch.int64), dev_idx(c.q_len, torch.int32),
                                    c.max_q_len if max_q_len is None else max_q_len, dev(c.K), dev(c.V), dev(c.V_lr),
                                    dev_idx(c.kv_start, torch.int64), dev_idx(c.kv_prefix, torch.int32), dev(c.B),
                                    dev_idx(c.agents, torch.int32), s.scale, O=O)
    torch.cuda.synchronize()
    return host64(O)


def ref_prefill_varlen(c: W.PrefillBatch):
    return oracle.attn_prefill_varlen(c.Q.as_f64(), c.K.as_f64(), c.V.as_f64(), c.V_lr.as_f64(), c.B.as_f64(),
                                      c.q_start, c.q_len, c.kv_start, c.kv_prefix, c.agents, c.shape.scale)


def covered_rows(c: W.PrefillBatch, only=None):
    rows = []
    for b in range(len(c.q_len)):
        if only is None or b in only:
            rows += list(range(int(c.q_start[b]), int(c.q_start[b]) + int(c.q_len[b])))
    return np.asarray(rows, np.int64)


def test_llama_prefill_full_size_sampled_rows():
    """L_P = 16,384 cached + L_C = 2,048 new queries over 18,432 keys (the timed launch); rows spanning
    first/last query tiles, tile edges and the diagonal are checked for every head against the oracle."""
    say("prefill llama 16384+2048: generating inputs")
    c = W.llama_prefill()
    say("prefill llama 16384+2048: running")
    got = run_prefill(c)
    rows = np.array([0, 1, 2, 15, 16, 31, 32, 33, 63, 64, 127, 128, 129, 511, 1000, 1023, 1024, 1500, 2015, 2046, 2047])
    say("prefill llama 16384+2048: oracle on sampled rows")
    ref = ref_prefill(c, rows=rows)
    check(got[rows], ref, "bf16")


def test_llama_prefill_full_size_every_row_of_one_group():
    """The timed launch (16,384 + 2,048 over 18,432 keys): all 2,048 query rows of KV head 0's query
    group (query heads 0-3), the oracle run one head at a time."""
    say("prefill llama 16384+2048 all rows: generating inputs")
    c = W.llama_prefill()
    say("prefill llama 16384+2048 all rows: running")
    got = run_prefill(c)
    for h in range(c.shape.n_q // c.shape.n_kv):
        say(f"prefill llama 16384+2048 all rows: oracle head {h}")
        check(got[:, h:h + 1], ref_prefill(c, heads=[h]), "bf16", f"head {h}")


@pytest.mark.parametrize("agent", [0, 1, 2])
def test_prefill_every_agent(agent):
    s = W.LLAMA_SHAPE
    c = W.random_prefill((300, agent), s, L_P=300, L_C=200, agent=agent)
    say(f"prefill llama-shaped agent={agent}")
    check(run_prefill(c), ref_prefill(c), "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_adapter_free_reads_neither_V_lr_nor_B(dtype):
    """The adapter-free view (agent -1, PReCache paper, section 3) attends the base cache alone: with
    V_lr and B all NaN the output still matches the oracle's base-only attention."""
    s = W.LLAMA_SHAPE if dtype == "bf16" else W.Shape(n_q=8, n_kv=2, d_head=64, rank=16, n_agents=3, d_model=256,
                                                      dtype="f32")
    c = W.random_prefill((307, 0 if dtype == "bf16" else 1), s, L_P=250, L_C=140, agent=-1)
    nan_lr = W.to_storage(np.full(c.V_lr.shape, np.nan, np.float32), dtype)
    nan_B = W.to_storage(np.full(c.B.shape, np.nan, np.float32), dtype)
    cc = W.PrefillCase(s, c.Q, c.K, c.V, nan_lr, nan_B, c.L_P, c.L_C, -1)
    say(f"prefill adapter-free {dtype}")
    got = run_prefill(cc)
    assert np.all(np.isfinite(got))
    check(got, ref_prefill(c), dtype)


SHAPES = [
    # dtype, n_q, n_kv, d, r, L_P, L_C
    ("bf16", 32, 8, 128, 8, 0, 1), ("bf16", 32, 8, 128, 8, 0, 97), ("bf16", 32, 8, 128, 16, 63, 65),
    ("bf16", 8, 2, 64, 8, 200, 130), ("bf16", 64, 8, 128, 8, 1, 33), ("bf16", 24, 8, 128, 16, 128, 40),
    ("bf16", 8, 8, 64, 16, 64, 129), ("bf16", 40, 8, 64, 8, 17, 50), ("bf16", 7, 1, 128, 8, 5, 70),
    ("f32", 4, 2, 64, 8, 192, 64), ("f32", 32, 8, 128, 16, 40, 37), ("f32", 16, 2, 128, 8, 0, 100),
]


@pytest.mark.parametrize("dtype,n_q,n_kv,d,r,L_P,L_C", SHAPES)
def test_prefill_shapes(dtype, n_q, n_kv, d, r, L_P, L_C):
    s = W.Shape(n_q=n_q, n_kv=n_kv, d_head=d, rank=r, n_agents=3, d_model=256, dtype=dtype)
    c = W.random_prefill((301, n_q, n_kv, d, r, L_P, L_C), s, L_P, L_C, agent=2)
    say(f"prefill {dtype} n_q={n_q} n_kv={n_kv} d={d} r={r} L_P={L_P} L_C={L_C}")
    check(run_prefill(c), ref_prefill(c), dtype, f"{dtype} {n_q}/{n_kv} d={d} r={r} L_P={L_P} L_C={L_C}")


def test_prefill_never_reads_past_the_chunk():
    """Cache rows after L_P + L_C hold NaN; the kernel must not read them."""
    s = W.LLAMA_SHAPE
    L_P, L_C = 150, 77
    c = W.random_prefill((302,), s, L_P, L_C + 100, agent=1)
    c = W.PrefillCase(s, W.HostTensor(c.Q.data[:L_C], c.Q.dtype), c.K, c.V, c.V_lr, c.B, L_P, L_C, 1)
    tail = np.arange(L_P + L_C, L_P + L_C + 100)
    for t in (c.K, c.V, c.V_lr):
        W.fill_rows(t, tail, float("nan"))
    say("prefill NaN past the chunk")
    check(run_prefill(c), ref_prefill(c), "bf16")


def test_prefill_mask_bombs():
    """Keys just past a query's diagonal get huge scores and values: a mask leak shows as O ~ 1e4."""
    s = W.LLAMA_SHAPE
    L_P, L_C = 100, 300
    c = W.random_prefill((303,), s, L_P, L_C, agent=0)
    g = np.random.default_rng(3)
    u = g.standard_normal(s.d_head).astype(np.float32)
    u /= np.linalg.norm(u)
    Q = c.Q.as_f32() * 0.1 + u[None, None, :] * 3.0
    K = c.K.as_f32()
    V = c.V.as_f32()
    bombs = [L_P + 16 * k + 1 for k in range(0, L_C // 16)]
    for j in bombs:
        K[j] = 1e3 * u / np.sqrt(s.d_head) * 0.5 + 0.0 * K[j]
        V[j] = 1e4
    cc = W.PrefillCase(s, W.to_storage(Q, "bf16"), W.to_storage(K, "bf16"), W.to_storage(V, "bf16"), c.V_lr, c.B,
                       L_P, L_C, 0)
    say("prefill mask bombs")
    ref = ref_prefill(cc)
    got = run_prefill(cc)
    # rows before the first bomb must stay O(1); rows after see one and saturate to it
    assert np.abs(ref[0]).max() < 100 and np.abs(ref[-1]).max() > 1e3
    check(got, ref, "bf16")


def test_prefill_agent_signature_and_lr_isolation():
    s = W.LLAMA_SHAPE
    c = W.random_prefill((304,), s, 64, 96, agent=0, b_std=1.0)
    lr = c.V_lr.as_f32()
    for k in range(3):
        lr[:, k * s.rank:(k + 1) * s.rank] += 10.0 * k
    B = np.concatenate([np.full((1, s.rank, s.d_kv), 0.5 * (k + 1), np.float32) for k in range(3)])
    sig = W.PrefillCase(s, c.Q, c.K, c.V, W.to_storage(lr, "bf16"), W.to_storage(B, "bf16"), 64, 96, 0)
    for a in range(3):
        say(f"prefill agent signature agent={a}")
        check(run_prefill(sig, agent=a), ref_prefill(sig, agent=a), "bf16", f"signature agent {a}")
    zero = W.to_storage(np.zeros(c.V.shape, np.float32), "bf16")
    iso = W.PrefillCase(s, c.Q, c.K, zero, c.V_lr, c.B, 64, 96, 2)
    say("prefill LR isolation")
    st = check(run_prefill(iso), ref_prefill(iso), "bf16")
    assert st["normwise"] < 2e-2


def test_prefill_is_deterministic():
    s = W.LLAMA_SHAPE
    c = W.random_prefill((305,), s, 500, 300, agent=1)
    assert np.array_equal(run_prefill(c), run_prefill(c))


@pytest.mark.parametrize("big", [1.0e5, 1.0e30, 3.0e38])
def test_prefill_large_values_match_the_oracle(big):
    """Large entries of V_base and of the agent's V_lr slice: beyond the fp16 range (1e5, 1e30) they
    stage as inf in the fast pass's fp16 operands, and near the bf16 maximum (3e38 on several keys)
    even exact fp32 sums would overflow; either leaves non-finite sums, which send the workgroup
    through the range-safe pass (bf16 values prescaled by a power of two, P as hi + lo parts). Every
    row still matches the oracle, including rows that never see the large keys but share their
    workgroup, and rows of other KV heads."""
    s = W.LLAMA_SHAPE
    c = W.random_prefill((306,), s, 40, 60, agent=1)
    V = c.V.as_f32()
    if big > 1e36:
        V[10:22, 3, 7] = big   # twelve keys seen by every query row of KV head 3: their sum overflows
    else:
        V[10, 3, 7] = big      # seen by every query row of KV head 3
    V[95, 3, 0] = -big         # seen only by the last query rows (position 95 = L_P + 55)
    V[50, 6, 127] = big
    lr_big = min(big, 1.0e30)  # O_lr B must stay inside the bf16 range of the output
    Vlr = c.V_lr.as_f32()
    Vlr[33, 1 * s.rank + 2] = lr_big   # agent 1's slice: every head's rows carry it through B
    Vlr[7, 0] = np.float32(lr_big)     # agent 0's columns: not read for agent 1
    cc = W.PrefillCase(s, c.Q, c.K, W.to_storage(V, "bf16"), W.to_storage(Vlr, "bf16"), c.B, 40, 60, 1)
    say(f"prefill large values ({big:g})")
    check(run_prefill(cc), ref_prefill(cc), "bf16", f"V = {big:g}")
    # the fp16 maximum itself stays on the fast pass
    V2 = c.V.as_f32()
    V2[10, 3, 7] = 65504.0
    c2 = W.PrefillCase(s, c.Q, c.K, W.to_storage(V2, "bf16"), c.V_lr, c.B, 40, 60, 1)
    check(run_prefill(c2), ref_prefill(c2), "bf16", "V = 65504")


def test_prefill_huge_scores_match_the_oracle():
    """Scores far beyond the usual range (|q.k| up to ~1e8): the fast pass's folded exponent (one
    fma with the row max) would lose precision there, so those workgroups take the range-safe pass
    (exact differences to the row max)."""
    s = W.LLAMA_SHAPE
    c = W.random_prefill((308,), s, 100, 80, agent=2)
    Q = c.Q.as_f32()
    Q[7, 9, 11] = 3.0e4       # query head 9 -> KV head 2
    Q[50, 20, 0] = -2.0e4     # query head 20 -> KV head 5
    K = c.K.as_f32()
    K[:, 2, 11] *= 1000.0
    K[:, 5, 0] *= 1000.0
    cc = W.PrefillCase(s, W.to_storage(Q, "bf16"), W.to_storage(K, "bf16"), c.V, c.V_lr, c.B, 100, 80, 2)
    say("prefill huge scores")
    check(run_prefill(cc), ref_prefill(cc), "bf16", "huge scores")


def test_prefill_large_values_varlen_and_paged():
    """The range-safe pass serves the batched and the paged calls too (same kernel): a huge value in
    one request's rows leaves every request's rows at the oracle's values."""
    s = W.LLAMA_SHAPE
    c = W.random_prefill_batch((307,), s, [(30, 70, 0), (0, 1, -1), (200, 300, 2)])
    V = c.V.as_f32()
    V[int(c.kv_start[2]) + 5, 1, 3] = 3.0e20
    Vlr = c.V_lr.as_f32()
    Vlr[int(c.kv_start[0]) + 2, 0 * s.rank + 1] = -2.0e6
    cb = dataclasses.replace(c, V=W.to_storage(V, "bf16"), V_lr=W.to_storage(Vlr, "bf16"))
    say("prefill varlen large values")
    got = run_prefill_varlen(cb)
    rows = covered_rows(cb)
    check(got[rows], ref_prefill_varlen(cb)[rows], "bf16")


# ------------------------------------------------------------------------------ batched variable length
def test_prefill_varlen_batch():
    """Six requests in one launch: own L_P / L_C / agent (one adapter-free, one empty chunk, one single
    query, one long chunk), ragged tails; uncovered rows of O stay as they were."""
    s = W.LLAMA_SHAPE
    c = W.random_prefill_batch((320,), s, [(300, 200, 1), (0, 64, -1), (1000, 1, 2), (77, 130, 0), (5, 0, 1),
                                          (900, 513, 2)])
    say("prefill varlen batch of 6")
    got = run_prefill_varlen(c)
    ref = ref_prefill_varlen(c)
    rows = covered_rows(c)
    check(got[rows], ref[rows], "bf16")
    uncovered = np.setdiff1d(np.arange(c.Q.shape[0]), rows)
    assert np.all(got[uncovered] == 0.0)


def test_prefill_varlen_shared_cache_rows_and_fp32():
    """Requests whose cache ranges overlap (agents sharing base rows), fp32, GQA 2:1, r = 16."""
    s = W.Shape(n_q=8, n_kv=4, d_head=64, rank=16, n_agents=3, d_model=256, dtype="f32")
    c = W.random_prefill_batch((321,), s, [(40, 30, 0), (40, 30, 2), (10, 60, 1), (0, 100, -1)],
                               kv_starts=[0, 0, 20, 5])
    say("prefill varlen shared cache rows fp32")
    got = run_prefill_varlen(c)
    rows = covered_rows(c)
    check(got[rows], ref_prefill_varlen(c)[rows], "f32")


def test_prefill_varlen_matches_single_request_calls():
    """Each request of the batch gives the same bits as lra_attn_prefill on that request alone."""
    s = W.LLAMA_SHAPE
    reqs = [(200, 97, 0), (33, 128, 1), (0, 1, 2)]
    c = W.random_prefill_batch((322,), s, reqs)
    say("prefill varlen vs single calls")
    got = run_prefill_varlen(c)
    Q, K, V, L, B = dev(c.Q), dev(c.K), dev(c.V), dev(c.V_lr), dev(c.B)
    for b, (lp, lc, a) in enumerate(reqs):
        q0, k0 = int(c.q_start[b]), int(c.kv_start[b])
        one = lra.lra_attn_prefill(Q[q0:q0 + lc].contiguous(), lp, K[k0:k0 + lp + lc].contiguous(),
                                   V[k0:k0 + lp + lc].contiguous(), L[k0:k0 + lp + lc].contiguous(), B, a, s.scale)
        torch.cuda.synchronize()
        assert np.array_equal(host64(one), got[q0:q0 + lc]), b


def test_prefill_varlen_invalid_requests_give_nan_rows():
    """A cache range past kv_rows, an agent outside [-1, N), a chunk longer than max_q_len: NaN in every
    row of that request; the valid request beside them is exact."""
    s = W.LLAMA_SHAPE
    c = W.random_prefill_batch((323,), s, [(100, 50, 0), (60, 40, 1), (30, 20, 3), (10, 300, 1)])
    kv_start = c.kv_start.copy()
    kv_start[1] = c.K.shape[0] - 50          # range runs past the cache
    cc = W.PrefillBatch(s, c.Q, c.K, c.V, c.V_lr, c.B, c.q_start, c.q_len, kv_start, c.kv_prefix, c.agents)
    say("prefill varlen invalid requests")
    got = run_prefill_varlen(cc, max_q_len=64)  # request 3 (300 queries) exceeds it
    for b in (1, 2, 3):
        assert np.all(np.isnan(got[covered_rows(cc, only=[b])])), b
    rows = covered_rows(cc, only=[0])
    first = W.PrefillBatch(s, c.Q, c.K, c.V, c.V_lr, c.B, c.q_start[:1], c.q_len[:1], c.kv_start[:1],
                           c.kv_prefix[:1], c.agents[:1])
    check(got[rows], ref_prefill_varlen(first)[rows], "bf16")


def test_prefill_varlen_never_reads_outside_ranges():
    """Cache rows outside every request's range and query rows outside every chunk hold NaN."""
    s = W.LLAMA_SHAPE
    c = W.random_prefill_batch((324,), s, [(129, 70, 2), (0, 33, 0), (64, 64, -1)], gap=5)
    used = np.zeros(c.K.shape[0], bool)
    for b in range(3):
        used[int(c.kv_start[b]):int(c.kv_start[b]) + int(c.kv_prefix[b]) + int(c.q_len[b])] = True
    for t in (c.K, c.V, c.V_lr):
        W.fill_rows(t, np.where(~used)[0], float("nan"))
    rows = covered_rows(c)
    W.fill_rows(c.Q, np.setdiff1d(np.arange(c.Q.shape[0]), rows), float("nan"))
    say("prefill varlen NaN outside ranges")
    got = run_prefill_varlen(c)
    assert np.all(np.isfinite(got[rows]))
    check(got[rows], ref_prefill_varlen(c)[rows], "bf16")



# ------------------------------------------------------------------------------ paged cache
def run_prefill_paged(c: W.PagedPrefillBatch, table=None):
    s = c.shape
    O = lra.lra_attn_prefill_paged(dev(c.Q), dev_idx(c.q_start, torch.int64), dev_idx(c.q_len, torch.int32),
                                   c.max_q_len, dev(c.K_pages), dev(c.V_pages), dev(c.Vlr_pages),
                                   dev_idx(c.block_table if table is None else table, torch.int32),
                                   dev_idx(c.kv_prefix, torch.int32), dev(c.B), dev_idx(c.agents, torch.int32), s.scale)
    torch.cuda.synchronize()
    return host64(O)


def ref_prefill_paged(c: W.PagedPrefillBatch):
    return oracle.attn_prefill_paged(c.Q.as_f64(), c.K_pages.as_f64(), c.V_pages.as_f64(), c.Vlr_pages.as_f64(),
                                     c.B.as_f64(), c.block_table, c.q_start, c.q_len, c.kv_prefix, c.agents,
                                     c.shape.scale)


def paged_rows(c):
    return np.concatenate([np.arange(int(c.q_start[b]), int(c.q_start[b]) + int(c.q_len[b]))
                           for b in range(len(c.q_len))]).astype(np.int64)


@pytest.mark.parametrize("page_size", [64, 256])
def test_prefill_paged_cache(page_size):
    """Shuffled pages with a shared first page, requests of mixed L_P / L_C and agents (adapter-free too)."""
    s = W.LLAMA_SHAPE
    c = W.random_paged_prefill_batch((330, page_size), s, [(300, 200, 1), (0, 64, -1), (1000, 1, 2), (77, 130, 0),
                                                           (640, 257, 2)], page_size, shared_prefix_pages=1)
    say(f"prefill paged P={page_size}")
    rows = paged_rows(c)
    check(run_prefill_paged(c)[rows], ref_prefill_paged(c)[rows], "bf16")


def test_prefill_paged_equals_varlen_bits():
    """The paged call gives the same bits as lra_attn_prefill_varlen over the rows laid out contiguously."""
    s = W.LLAMA_SHAPE
    P = 64
    reqs = [(200, 97, 0), (65, 128, -1), (0, 1, 2)]
    c = W.random_paged_prefill_batch((331,), s, reqs, P, shared_prefix_pages=1)
    got = run_prefill_paged(c)
    idx, starts, n = [], [], 0
    for b, (lp, lc, _) in enumerate(reqs):
        L = lp + lc
        pages = c.block_table[b][:(L + P - 1) // P]
        idx.append(np.concatenate([np.arange(pg * P, pg * P + P) for pg in pages])[:L])
        starts.append(n)
        n += L
    idx = np.concatenate(idx)
    flat = lambda t: W.HostTensor(t.data.reshape((-1,) + t.data.shape[2:])[idx], t.dtype)
    v = W.PrefillBatch(s, c.Q, flat(c.K_pages), flat(c.V_pages), flat(c.Vlr_pages), c.B, c.q_start, c.q_len,
                       np.asarray(starts, np.int64), c.kv_prefix, c.agents)
    say("prefill paged vs varlen bits")
    assert np.array_equal(got, run_prefill_varlen(v))


def test_prefill_paged_bad_page_and_unnamed_pages():
    """Pages no request names hold NaN and are never read; a page id out of range makes NaN rows in
    its own request only (rows whose workgroups never reached it stay exact)."""
    s = W.LLAMA_SHAPE
    P = 64
    c = W.random_paged_prefill_batch((332,), s, [(300, 60, 0), (200, 90, 1)], P, spare_pages=3)
    named = np.unique(np.concatenate([c.block_table[b][:(int(c.kv_prefix[b] + c.q_len[b]) + P - 1) // P]
                                      for b in range(2)]))
    unnamed = np.setdiff1d(np.arange(c.K_pages.shape[0]), named)
    for t in (c.K_pages, c.V_pages, c.Vlr_pages):
        W.fill_rows(t, unnamed, float("nan"))
    ref = ref_prefill_paged(c)
    rows0 = paged_rows(W.PagedPrefillBatch(s, c.Q, c.K_pages, c.V_pages, c.Vlr_pages, c.B, c.block_table[:1],
                                           c.q_start[:1], c.q_len[:1], c.kv_prefix[:1], c.agents[:1]))
    rows1 = np.arange(int(c.q_start[1]), int(c.q_start[1]) + int(c.q_len[1]))
    say("prefill paged unnamed pages")
    got = run_prefill_paged(c)
    check(got[paged_rows(c)], ref[paged_rows(c)], "bf16")
    table = c.block_table.copy()
    table[1, 1] = c.K_pages.shape[0] + 7
    say("prefill paged bad page")
    bad = run_prefill_paged(c, table=table)
    check(bad[rows0], ref[rows0], "bf16")
    assert np.isnan(bad[rows1]).any()
    fin = np.isfinite(bad[rows1]).all(axis=(1, 2))
    if fin.any():
        check(bad[rows1][fin], ref[rows1][fin], "bf16")


# ---------------------------------------------------------------- LoRA on the keys (qkvo)
def _dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def run_prefill_qkvo(c: W.QkvoPrefillCase, agent=None, K_lr=None, B_k=None, V_lr=None, B=None, K=None,
                     workspace=None, V=None):
    b = c.base
    O = lra.lra_attn_prefill_qkvo(dev(b.Q), b.L_P, dev(b.K if K is None else K), dev(b.V if V is None else V),
                                  dev(b.V_lr if V_lr is None else V_lr), dev(c.K_lr if K_lr is None else K_lr),
                                  dev(b.B if B is None else B), dev(c.B_k if B_k is None else B_k),
                                  _dev_f32(c.cos), _dev_f32(c.sin), b.agent if agent is None else agent,
                                  b.shape.scale, workspace=workspace)
    torch.cuda.synchronize()
    return host64(O)


def ref_prefill_qkvo(c: W.QkvoPrefillCase, agent=None, rows=None):
    b = c.base
    return oracle.attn_prefill_qkvo(b.Q.as_f64(), b.K.as_f64(), b.V.as_f64(), b.V_lr.as_f64(), c.K_lr.as_f64(),
                                    b.B.as_f64(), c.B_k.as_f64(), c.cos, c.sin,
                                    b.agent if agent is None else agent, b.L_P, b.shape.scale, rows=rows)


QKVO_SHAPES = [
    # n_q, n_kv, d, r, L_P, L_C, agent
    (32, 8, 128, 8, 0, 97, 0), (32, 8, 128, 16, 63, 65, 2), (8, 2, 64, 8, 200, 130, 1),
    (8, 8, 64, 16, 64, 129, 0), (7, 1, 128, 8, 5, 70, 2), (24, 8, 128, 16, 128, 40, 1), (32, 8, 128, 8, 300, 1, 1),
]


@pytest.mark.parametrize("n_q,n_kv,d,r,L_P,L_C,agent", QKVO_SHAPES)
def test_prefill_qkvo_shapes(n_q, n_kv, d, r, L_P, L_C, agent):
    """LoRA on the keys as well: K_a = K_base + RoPE(K_lr B_k), several tiles and a ragged tail."""
    s = W.Shape(n_q=n_q, n_kv=n_kv, d_head=d, rank=r, n_agents=3, d_model=256, dtype="bf16")
    c = W.random_prefill_qkvo((320, n_q, n_kv, d, r, L_P, L_C), s, L_P, L_C, agent=agent)
    say(f"prefill qkvo n_q={n_q} n_kv={n_kv} d={d} r={r} L_P={L_P} L_C={L_C} agent={agent}")
    check(run_prefill_qkvo(c), ref_prefill_qkvo(c), "bf16", f"qkvo {n_q}/{n_kv} d={d} r={r} L_P={L_P} L_C={L_C}")


def test_prefill_qkvo_llama_full_size_sampled_rows():
    """The Llama chunked prefill (16,384 cached + 2,048 new queries) with LoRA on the keys, in the
    launch the benchmark times; sampled rows for every head against the oracle."""
    say("prefill qkvo llama 16384+2048: generating inputs")
    c = W.llama_prefill_qkvo()
    say("prefill qkvo llama 16384+2048: running")
    got = run_prefill_qkvo(c)
    rows = np.array([0, 1, 15, 16, 63, 64, 127, 128, 1023, 1024, 2046, 2047])
    say("prefill qkvo llama 16384+2048: oracle on sampled rows")
    check(got[rows], ref_prefill_qkvo(c, rows=rows), "bf16")


def test_prefill_qkvo_without_key_part_reduces_to_plain_prefill():
    """With B_k = 0 the agent's keys are K_base, so the output is the plain prefill's (oracle
    attn_prefill); the adapter-free view (agent -1) reads none of K_lr, B_k, V_lr, B (all NaN here)
    and gives the base-only attention. The key path takes fp16 score operands and the plain path bf16,
    so the two kernels agree to rounding, not bit for bit."""
    s = W.LLAMA_SHAPE
    c = W.random_prefill_qkvo((321,), s, L_P=190, L_C=150, agent=1)
    zero_bk = W.to_storage(np.zeros(c.B_k.shape, np.float32), "bf16")
    b = c.base
    say("prefill qkvo B_k = 0 vs plain prefill")
    check(run_prefill_qkvo(c, B_k=zero_bk), ref_prefill(b), "bf16")
    nan = lambda t: W.to_storage(np.full(t.shape, np.nan, np.float32), "bf16")
    say("prefill qkvo adapter-free with NaN adapters")
    got = run_prefill_qkvo(c, agent=-1, K_lr=nan(c.K_lr), B_k=nan(c.B_k), V_lr=nan(b.V_lr), B=nan(b.B))
    check(got, ref_prefill(b, agent=-1), "bf16")


@pytest.mark.parametrize("big", [1.0e5, 1.0e30])
def test_prefill_qkvo_query_beyond_fp16_range_matches_the_oracle(big):
    """A query entry beyond the fp16 range (the fast pass takes fp16 scores) sends its workgroups
    through the range-safe pass: bf16 queries against the keys rebuilt in fp32 (three bf16 parts).
    Every row matches the oracle."""
    s = W.LLAMA_SHAPE
    c = W.random_prefill_qkvo((324,), s, L_P=0, L_C=64, agent=0)
    q = c.base.Q.as_f64().astype(np.float32)
    q[5, 3 * s.group, 7] = big    # query head of KV head 3
    q[40, 6 * s.group + 1, 100] = -big
    cq = W.QkvoPrefillCase(W.PrefillCase(s, W.to_storage(q, "bf16"), *[getattr(c.base, f) for f in ("K", "V", "V_lr", "B")],
                                         c.base.L_P, c.base.L_C, 0), c.K_lr, c.B_k, c.cos, c.sin)
    say(f"prefill qkvo query {big:g}")
    check(run_prefill_qkvo(cq), ref_prefill_qkvo(cq), "bf16", f"Q = {big:g}")


def test_prefill_qkvo_expanded_keys_in_the_workspace():
    """The expansion pass leaves the agent's keys in the workspace (fp16, [L, n_kv, d]): each one is
    the oracle's K_base + RoPE(K_lr B_k) rounded once to fp16 (2^-11 relative, plus the fp32 sum)."""
    s = W.Shape(n_q=8, n_kv=2, d_head=128, rank=16, n_agents=3, d_model=256, dtype="bf16")
    c = W.random_prefill_qkvo((325,), s, L_P=70, L_C=60, agent=2)
    b = c.base
    L = b.L_P + b.L_C
    ws = torch.empty(lra.lra_attn_prefill_qkvo_workspace_bytes(L, s.n_kv, s.d_head), dtype=torch.uint8, device="cuda")
    check(run_prefill_qkvo(c, workspace=ws), ref_prefill_qkvo(c), "bf16")
    ka = ws[: L * s.n_kv * s.d_head * 2].view(torch.float16).float().cpu().numpy().astype(np.float64)
    ref = oracle.agent_keys(b.K.as_f64(), c.K_lr.as_f64(), c.B_k.as_f64(), 2, c.cos, c.sin).reshape(-1)
    assert np.all(np.abs(ka - ref) <= 2.0 ** -11 * np.abs(ref) + 1e-5)
    # the same workspace serves a smaller call next (no initialisation needed)
    c2 = W.random_prefill_qkvo((326,), s, L_P=10, L_C=20, agent=0)
    check(run_prefill_qkvo(c2, workspace=ws), ref_prefill_qkvo(c2), "bf16")


@pytest.mark.parametrize("big", [7.0e4, 1.0e30])
def test_prefill_qkvo_key_beyond_fp16_range_matches_the_oracle(big):
    """A summed key beyond the fp16 range (here through K_base) records its tile's largest |key|;
    every workgroup that stages the tile takes the range-safe pass and matches the oracle, and so do
    huge V_base / V_lr entries on the same call."""
    s = W.LLAMA_SHAPE
    c = W.random_prefill_qkvo((327,), s, L_P=100, L_C=50, agent=1)
    k = c.base.K.as_f64().astype(np.float32)
    k[10, 2, 0] = big
    k[120, 5, 64] = -big
    klr = c.K_lr.as_f64().astype(np.float32)
    klr[60, 1 * s.rank + 3] = big / 10
    v = c.base.V.as_f64().astype(np.float32)
    v[130, 2, 9] = big
    say(f"prefill qkvo keys {big:g}")
    got = run_prefill_qkvo(c, K=W.to_storage(k, "bf16"), K_lr=W.to_storage(klr, "bf16"), V=W.to_storage(v, "bf16"))
    ck = W.QkvoPrefillCase(W.PrefillCase(s, c.base.Q, W.to_storage(k, "bf16"), W.to_storage(v, "bf16"), c.base.V_lr,
                                         c.base.B, c.base.L_P, c.base.L_C, 1), W.to_storage(klr, "bf16"), c.B_k,
                           c.cos, c.sin)
    check(got, ref_prefill_qkvo(ck), "bf16", f"K = {big:g}")


def test_prefill_qkvo_key_part_matters():
    """The rotated rank-r key part changes the output (a kernel that dropped it would fail here)
    and each agent reads its own K_lr columns: NaN in another agent's columns leaves the rows finite."""
    s = W.LLAMA_SHAPE
    c = W.random_prefill_qkvo((322,), s, L_P=64, L_C=64, agent=2)
    got = run_prefill_qkvo(c)
    plain = run_prefill(c.base)
    assert np.max(np.abs(got - plain)) > 0.05
    klr = c.K_lr.as_f64().astype(np.float32)
    klr[:, : 2 * s.rank] = np.nan
    got2 = run_prefill_qkvo(c, K_lr=W.to_storage(klr, "bf16"))
    assert np.array_equal(got, got2)


def test_prefill_qkvo_rejects_fp32():
    s = W.Shape(n_q=4, n_kv=2, d_head=64, rank=8, n_agents=2, d_model=256, dtype="f32")
    c = W.random_prefill_qkvo((323,), s, L_P=8, L_C=8, agent=0)
    with pytest.raises(lra.LraError, match="UNSUPPORTED"):
        run_prefill_qkvo(c)


def test_prefill_varlen_and_paged_in_the_bench_configuration():
    """The Llama prefill as the bench times its batched and paged lines: four chunk requests of 512
    queries (request b at L_P = 16,384 + 512 b over the same cache rows) and the single chunk over
    64-row pages in a seeded random order. Both give the single call's bits; sampled rows match the
    oracle."""
    say("prefill bench configuration: generating inputs")
    c = W.llama_prefill()
    s = c.shape
    Q, K, V, L, B = dev(c.Q), dev(c.K), dev(c.V), dev(c.V_lr), dev(c.B)
    one = lra.lra_attn_prefill(Q, c.L_P, K, V, L, B, 0, s.scale)
    torch.cuda.synchronize()
    ref_bits = host64(one)
    nreq, lc = 4, c.L_C // 4
    say("prefill bench configuration: varlen 4 x 512")
    O = lra.lra_attn_prefill_varlen(Q, torch.arange(nreq, dtype=torch.int64, device="cuda") * lc,
                                    torch.full((nreq,), lc, dtype=torch.int32, device="cuda"), lc, K, V, L,
                                    torch.zeros(nreq, dtype=torch.int64, device="cuda"),
                                    (c.L_P + torch.arange(nreq, device="cuda") * lc).to(torch.int32), B,
                                    torch.zeros(nreq, dtype=torch.int32, device="cuda"), s.scale)
    torch.cuda.synchronize()
    assert np.array_equal(host64(O), ref_bits)
    say("prefill bench configuration: paged, 64-row pages")
    P = 64
    n_pages = K.shape[0] // P
    g = torch.Generator(device="cpu")
    g.manual_seed(42)
    table = torch.randperm(n_pages, generator=g).to(torch.int32)
    # logical block j lives in page table[j]
    Kp = torch.empty((n_pages, P) + tuple(K.shape[1:]), dtype=K.dtype, device="cuda")
    Vp, Lp = torch.empty_like(Kp), torch.empty((n_pages, P, L.shape[1]), dtype=L.dtype, device="cuda")
    tl = table.long().cuda()
    Kp[tl] = K.view(n_pages, P, *K.shape[1:])
    Vp[tl] = V.view(n_pages, P, *V.shape[1:])
    Lp[tl] = L.view(n_pages, P, L.shape[1])
    O = lra.lra_attn_prefill_paged(Q, torch.zeros(1, dtype=torch.int64, device="cuda"),
                                   torch.full((1,), c.L_C, dtype=torch.int32, device="cuda"), c.L_C, Kp, Vp, Lp,
                                   table.reshape(1, n_pages).cuda(), torch.full((1,), c.L_P, dtype=torch.int32,
                                                                                device="cuda"), B,
                                   torch.zeros(1, dtype=torch.int32, device="cuda"), s.scale)
    torch.cuda.synchronize()
    assert np.array_equal(host64(O), ref_bits)
    rows = np.array([0, 511, 512, 1023, 1024, 1535, 1536, 2047])
    say("prefill bench configuration: oracle on sampled rows")
    check(ref_bits[rows], ref_prefill(c, rows=rows), "bf16")
