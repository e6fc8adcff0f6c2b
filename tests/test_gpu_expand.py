"""GPU parity of lra_expand_values (the expand-then-attend baseline) against the fp64 oracle.

The expansion is one fp32 sum per element rounded once to the element type, so besides the stated
tolerance each element is held to one rounding of the exact value:
  |got - ref| <= u * |ref| + 2^-19 * (|V_base| + sum_j |V_lr_j B_j|)      u = 2^-8 (bf16), 2^-23 (fp32)
and attention over the expanded rows with the adapter-free view must match the adapted oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import rank_kv_cache_amd as lra
import workloads as W
from tests.gpu_util import check, dev, dev_idx, host64, say

pytestmark = pytest.mark.gpu

SENTINEL = 7.0   # value of V_out rows no request names (exact in bf16 and fp32)


def run_expand(c: W.DecodeBatch, dst, out_rows, max_len=None, lens=None, agents=None, starts=None):
    s = c.shape
    torch_dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    V_out = torch.full((out_rows, s.n_kv, s.d_head), SENTINEL, dtype=torch_dt, device="cuda")
    lens = c.kv_len if lens is None else lens
    lra.lra_expand_values(dev(c.V), dev(c.V_lr), dev(c.B), dev_idx(c.kv_start if starts is None else starts, torch.int64),
                          dev_idx(lens, torch.int32), dev_idx(c.agent if agents is None else agents, torch.int32),
                          int(max(lens)) if max_len is None else max_len, dev_idx(dst, torch.int64), V_out)
    torch.cuda.synchronize()
    return host64(V_out)


def ref_expand(c: W.DecodeBatch, dst, out_rows):
    s = c.shape
    V_out = np.full((out_rows, s.n_kv, s.d_head), SENTINEL)
    return oracle.expand_values(V_out, c.V.as_f64(), c.V_lr.as_f64(), c.B.as_f64(), c.kv_start, c.kv_len, c.agent, dst)


def abs_terms(c: W.DecodeBatch, dst, out_rows):
    """|V_base| + sum_j |V_lr_j B_j| at each destination element (the fp32 accumulation's scale)."""
    s = c.shape
    out = np.zeros((out_rows, s.n_kv, s.d_head))
    V, L, B = c.V.as_f64(), c.V_lr.as_f64(), c.B.as_f64()
    for b in range(c.batch):
        n, s0, d0, a = int(c.kv_len[b]), int(c.kv_start[b]), int(dst[b]), int(c.agent[b])
        if n <= 0:
            continue
        t = np.abs(V[s0:s0 + n])
        if a >= 0:
            t = t + (np.abs(L[s0:s0 + n, a * s.rank:(a + 1) * s.rank]) @ np.abs(B[a])).reshape(n, s.n_kv, s.d_head)
        out[d0:d0 + n] = t
    return out


def check_one_rounding(got, ref, terms, dtype, what):
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
    err = np.abs(got - ref)
    bound = u * np.abs(ref) + 2.0 ** -19 * terms
    assert np.all(err <= bound), f"{what}: {int((err > bound).sum())} elements beyond one rounding"


SHAPES = [
    # dtype, n_kv, d, r
    ("bf16", 8, 128, 8), ("bf16", 8, 128, 16), ("bf16", 2, 64, 8), ("bf16", 3, 128, 16), ("bf16", 40, 64, 8),
    ("f32", 2, 64, 8), ("f32", 8, 128, 16), ("f32", 1, 64, 16), ("f32", 72, 64, 8),
]


@pytest.mark.parametrize("dtype,n_kv,d,r", SHAPES)
def test_expand_values_shapes_ragged_lengths(dtype, n_kv, d, r):
    """Ragged lengths around the 256-row workgroup, an empty request, shared sources, adapter-free
    requests; destinations packed into a larger buffer whose other rows must keep their bits."""
    s = W.Shape(n_q=n_kv, n_kv=n_kv, d_head=d, rank=r, n_agents=3, d_model=256, dtype=dtype)
    lens = [1, 255, 256, 257, 700, 0, 1000, 3, 513]
    starts = [0, 10, 10, 300, 600, 5, 1300, 2299, 1500]
    agents = [0, 1, 2, -1, 1, 0, 2, 1, 0]
    c = W.random_decode((300, n_kv, d, r, 0 if dtype == "f32" else 1), s, lens, kv_starts=starts, rows=2302,
                        agents=agents, b_std=0.3)
    dst = np.concatenate([[5], 5 + np.cumsum(np.asarray(lens[:-1]) + 3)]).astype(np.int64)
    out_rows = int(dst[-1] + lens[-1] + 4)
    say(f"expand {dtype} n_kv={n_kv} d={d} r={r}")
    got = run_expand(c, dst, out_rows)
    ref = ref_expand(c, dst, out_rows)
    covered = np.zeros(out_rows, bool)
    for b in range(len(lens)):
        covered[dst[b]:dst[b] + lens[b]] = True
    assert np.all(got[~covered] == SENTINEL), "rows no request names were written"
    check(got[covered], ref[covered], dtype, f"{dtype} n_kv={n_kv} d={d} r={r}")
    check_one_rounding(got, ref, abs_terms(c, dst, out_rows), dtype, f"{dtype} n_kv={n_kv} d={d} r={r}")
    # the adapter-free request copies its base rows bit for bit
    b = 3
    np.testing.assert_array_equal(got[dst[b]:dst[b] + lens[b]], c.V.as_f64()[starts[b]:starts[b] + lens[b]])


def test_expand_values_invalid_requests():
    """Bad agent or source range: NaN destination rows; bad destination or negative length: nothing
    written; a length beyond max_len: NaN in the first max_len destination rows only."""
    s = W.Shape(n_q=8, n_kv=8, d_head=128, rank=8, n_agents=3, d_model=256, dtype="bf16")
    lens = [300, 300, 300, 300, 300, -4, 600, 300]
    starts = [0, 0, 1900, -1, 0, 0, 0, 100]
    agents = [3, -2, 0, 0, 0, 0, 1, 2]
    dst = [0, 400, 800, 1200, 5000, 1600, 2000, 2700]
    c = W.random_decode((301,), s, [max(n, 0) for n in lens], kv_starts=[max(x, 0) for x in starts], rows=2048,
                        agents=[max(a, 0) for a in agents])
    c.kv_len = np.asarray(lens, np.int32)
    c.kv_start = np.asarray(starts, np.int64)
    c.agent = np.asarray(agents, np.int32)
    say("expand invalid requests")
    got = run_expand(c, np.asarray(dst, np.int64), 3100, max_len=512)
    rows = lambda b, n: got[dst[b]:dst[b] + n]
    for b in (0, 1, 2, 3):
        assert np.all(np.isnan(rows(b, 300))), f"request {b} not NaN"
    assert np.all(got[300:400] == SENTINEL)
    assert np.all(got[1600:2000] == SENTINEL)          # negative length: skipped
    assert np.all(np.isnan(got[2000:2512])) and np.all(got[2512:2700] == SENTINEL)   # 600 > max_len = 512
    # the one valid request is exact to one rounding
    ref = oracle.agent_values(c.V.as_f64()[100:400], c.V_lr.as_f64()[100:400], c.B.as_f64(), 2)
    check(rows(7, 300), ref, "bf16", "valid request beside invalid ones")


def expand_then_decode(c: W.DecodeBatch, keys_per_split=0):
    """Expand every request's rows in place of a copy of V_base, then decode with no LR term."""
    s = c.shape
    V_exp = lra.lra_expand_values(dev(c.V), dev(c.V_lr), dev(c.B), dev_idx(c.kv_start, torch.int64),
                                  dev_idx(c.kv_len, torch.int32), dev_idx(c.agent, torch.int32), c.max_kv_len,
                                  dev_idx(c.kv_start, torch.int64))
    none = torch.full((c.batch,), lra.ADAPTER_FREE, dtype=torch.int32, device="cuda")
    O = lra.lra_attn_decode(dev(c.Q), dev(c.K), V_exp, dev(c.V_lr), dev_idx(c.kv_start, torch.int64),
                            dev_idx(c.kv_len, torch.int32), c.max_kv_len, dev(c.B), none, s.scale, keys_per_split)
    torch.cuda.synchronize()
    return host64(O)


@pytest.mark.parametrize("dtype,n_q,n_kv,d,r", [("bf16", 32, 8, 128, 8), ("bf16", 32, 8, 128, 16), ("f32", 4, 2, 64, 8)])
def test_expand_then_attend_decode(dtype, n_q, n_kv, d, r):
    s = W.Shape(n_q=n_q, n_kv=n_kv, d_head=d, rank=r, n_agents=3, d_model=256, dtype=dtype)
    lens = [1, 64, 257, 1900, 700, 33]
    c = W.random_decode((302, n_q, r), s, lens, agents=[0, 1, 2, 1, 0, 2])
    say(f"expand-then-decode {dtype} {n_q}/{n_kv} d={d} r={r}")
    got = expand_then_decode(c)
    ref = oracle.attn_decode(c.Q.as_f64(), c.K.as_f64(), c.V.as_f64(), c.V_lr.as_f64(), c.B.as_f64(), c.kv_start,
                             c.kv_len, c.agent, s.scale)
    check(got, ref, dtype, "expand-then-decode")


def test_expand_then_attend_prefill():
    """Tiny fp32 workload shape (GQA 4/2, d 64, r 8): expand the agent's L_P + L_C rows, prefill with
    the adapter-free view, compare with the adapted oracle for every agent."""
    s = W.TINY_SHAPE
    tw = W.tiny_workload()
    L_P, L_C = tw.L_P, tw.L_C
    L = L_P + L_C
    # the LR cache as the precompute stores it: X A in fp32 (input synthesis, fp64 product)
    V_lr = W.HostTensor((tw.X.as_f64() @ tw.A.as_f64()).astype(np.float32), "f32")
    for agent in range(s.n_agents):
        say(f"expand-then-prefill tiny fp32 agent={agent}")
        V_exp = lra.lra_expand_values(dev(tw.V), dev(V_lr), dev(tw.B), dev_idx([0], torch.int64),
                                      dev_idx([L], torch.int32), dev_idx([agent], torch.int32), L,
                                      dev_idx([0], torch.int64))
        O = lra.lra_attn_prefill(dev(tw.Q), L_P, dev(tw.K), V_exp, dev(V_lr), dev(tw.B), lra.ADAPTER_FREE, s.scale)
        torch.cuda.synchronize()
        ref = oracle.attn_prefill(tw.Q.as_f64(), tw.K.as_f64(), tw.V.as_f64(), V_lr.as_f64(), tw.B.as_f64(), agent,
                                  L_P, s.scale)
        check(host64(O), ref, "f32", f"agent {agent}")


def test_expand_long_decode_full_size_sampled():
    """The 16 x 66,400 decode workload in the bench's launch configuration: every request expanded in
    place of its own rows, sampled rows of every request checked element by element, then two
    requests decoded end to end with the adapter-free view over the expanded rows."""
    say("expand 16 x 66400: generating inputs")
    c = W.llama_long_decode()
    s = c.shape
    say("expand 16 x 66400: running")
    V_exp = lra.lra_expand_values(dev(c.V), dev(c.V_lr), dev(c.B), dev_idx(c.kv_start, torch.int64),
                                  dev_idx(c.kv_len, torch.int32), dev_idx(c.agent, torch.int32), c.max_kv_len,
                                  dev_idx(c.kv_start, torch.int64))
    torch.cuda.synchronize()
    g = np.random.default_rng(303)
    for b in range(c.batch):
        L = int(c.kv_len[b])
        t = np.unique(np.concatenate([[0, 255, 256, L - 1], g.integers(0, L, 60)]))
        rows = int(c.kv_start[b]) + t
        got = host64(V_exp[torch.as_tensor(rows, device="cuda")])
        ref = oracle.agent_values(W.HostTensor(c.V.data[rows], "bf16").as_f64(),
                                  W.HostTensor(c.V_lr.data[rows], "bf16").as_f64(), c.B.as_f64(), int(c.agent[b]))
        check(got, ref, "bf16", f"request {b} sampled rows")
    none = torch.full((c.batch,), lra.ADAPTER_FREE, dtype=torch.int32, device="cuda")
    O = lra.lra_attn_decode(dev(c.Q), dev(c.K), V_exp, dev(c.V_lr), dev_idx(c.kv_start, torch.int64),
                            dev_idx(c.kv_len, torch.int32), c.max_kv_len, dev(c.B), none, s.scale)
    torch.cuda.synchronize()
    got = host64(O)
    for b in (0, 11):
        say(f"expand 16 x 66400: oracle request {b}")
        r0, n = int(c.kv_start[b]), int(c.kv_len[b])
        ref = oracle.attn_decode(c.Q.as_f64()[b:b + 1], W.HostTensor(c.K.data[r0:r0 + n], "bf16").as_f64(),
                                 W.HostTensor(c.V.data[r0:r0 + n], "bf16").as_f64(),
                                 W.HostTensor(c.V_lr.data[r0:r0 + n], "bf16").as_f64(), c.B.as_f64(), [0], [n],
                                 [int(c.agent[b])], s.scale)
        check(got[b:b + 1], ref, "bf16", f"request {b}")


def test_expand_then_attend_prefill_llama_full_size_sampled_rows():
    """The Llama chunked prefill (L_P 16,384 + L_C 2,048) in the bench's launch configuration:
    agent 1's 18,432 value rows expanded, sampled rows checked element by element, then the
    adapter-free prefill over them against the adapted oracle on sampled query rows."""
    say("expand-then-prefill llama 16384+2048: generating inputs")
    c = W.llama_prefill(agent=1)
    s = c.shape
    n = c.L_P + c.L_C
    zero = dev_idx([0], torch.int64)
    V_exp = lra.lra_expand_values(dev(c.V), dev(c.V_lr), dev(c.B), zero, dev_idx([n], torch.int32),
                                  dev_idx([1], torch.int32), n, zero)
    O = lra.lra_attn_prefill(dev(c.Q), c.L_P, dev(c.K), V_exp, dev(c.V_lr), dev(c.B), lra.ADAPTER_FREE, s.scale)
    torch.cuda.synchronize()
    vrows = np.array([0, 15, 16, 255, 256, 4095, 16383, 16384, 18000, n - 1])
    got_v = host64(V_exp[torch.as_tensor(vrows, device="cuda")])
    ref_v = oracle.agent_values(W.HostTensor(c.V.data[vrows], "bf16").as_f64(),
                                W.HostTensor(c.V_lr.data[vrows], "bf16").as_f64(), c.B.as_f64(), 1)
    check(got_v, ref_v, "bf16", "expanded rows")
    rows = np.array([0, 1, 31, 32, 127, 128, 1023, 1024, 2046, 2047])
    say("expand-then-prefill llama 16384+2048: oracle on sampled rows")
    ref = oracle.attn_prefill(c.Q.as_f64(), c.K.as_f64(), c.V.as_f64(), c.V_lr.as_f64(), c.B.as_f64(), 1, c.L_P,
                              s.scale, rows=rows)
    check(host64(O)[rows], ref, "bf16", "expand-then-prefill")
