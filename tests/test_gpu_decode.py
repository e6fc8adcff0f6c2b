"""GPU parity of lra_attn_decode against the fp64 oracle (needs an MI355X and liblra.so)."""
import numpy as np
import pytest
import torch

import oracle
import rank_kv_cache_amd as lra
import workloads as W
from tests.gpu_util import check, dev, dev_idx, host64, say

pytestmark = pytest.mark.gpu


class F64Rows:
    """Row-sliceable view of a host tensor that widens only the rows asked for (big caches)."""

    def __init__(self, t: W.HostTensor):
        self.t = t

    def __getitem__(self, idx):
        return W.HostTensor(self.t.data[idx], self.t.dtype).as_f64()


def run_decode(c: W.DecodeBatch, keys_per_split=0, max_kv_len=None, kv_rows=None):
    s = c.shape
    K, V, L = dev(c.K), dev(c.V), dev(c.V_lr)
    O = lra.lra_attn_decode(dev(c.Q), K, V, L, dev_idx(c.kv_start, torch.int64), dev_idx(c.kv_len, torch.int32),
                            c.max_kv_len if max_kv_len is None else max_kv_len, dev(c.B),
                            dev_idx(c.agent, torch.int32), s.scale, keys_per_split)
    torch.cuda.synchronize()
    return host64(O)


def ref_decode(c: W.DecodeBatch, requests=None):
    return oracle.attn_decode(c.Q.as_f64(), F64Rows(c.K), F64Rows(c.V), F64Rows(c.V_lr), c.B.as_f64(),
                              c.kv_start, c.kv_len, c.agent, c.shape.scale, requests=requests)


@pytest.mark.parametrize("agent", [0, 1, 2])
def test_llama_decode_L1900_every_agent(agent):
    c = W.llama_decode(agent=agent)
    say(f"decode llama L=1900 agent={agent}")
    check(run_decode(c), ref_decode(c), "bf16", f"agent {agent}")


@pytest.mark.parametrize("split", [64, 128, 192, 256, 512, 1024, 2048, 4096])
def test_llama_decode_every_split_size(split):
    c = W.llama_decode(agent=1)
    say(f"decode llama L=1900 keys_per_split={split}")
    check(run_decode(c, keys_per_split=split), ref_decode(c), "bf16", f"split {split}")


SHAPES = [
    # dtype, n_q, n_kv, d, r
    ("bf16", 32, 8, 128, 8), ("bf16", 32, 8, 128, 16), ("bf16", 8, 2, 64, 8), ("bf16", 64, 8, 128, 8),
    ("bf16", 24, 8, 128, 16), ("bf16", 8, 8, 64, 16), ("bf16", 40, 8, 64, 8),
    ("f32", 4, 2, 64, 8), ("f32", 32, 8, 128, 16), ("f32", 16, 2, 128, 8),
]


@pytest.mark.parametrize("dtype,n_q,n_kv,d,r", SHAPES)
def test_decode_shapes_ragged_lengths(dtype, n_q, n_kv, d, r):
    s = W.Shape(n_q=n_q, n_kv=n_kv, d_head=d, rank=r, n_agents=3, d_model=256, dtype=dtype)
    lens = [1, 2, 15, 16, 17, 63, 64, 65, 255, 256, 257, 700, 0, 1000]
    c = W.random_decode((100, n_q, n_kv, d, r, 0 if dtype == "f32" else 1), s, lens)
    say(f"decode shape {dtype} n_q={n_q} n_kv={n_kv} d={d} r={r}")
    ref = ref_decode(c)
    for split in (0, 64, 320):
        got = run_decode(c, keys_per_split=split)
        check(got, ref, dtype, f"{dtype} {n_q}/{n_kv} d={d} r={r} split={split}")
        assert np.all(got[12] == 0.0)


def test_tiny_fp32_decode_shared_ranges():
    s = W.TINY_SHAPE
    c = W.random_decode((101,), s, kv_lens=[257, 257, 257, 100, 1], kv_starts=[0, 0, 0, 157, 256], rows=257,
                        agents=[0, 1, 2, 1, 0])
    say("decode tiny fp32 shared ranges")
    check(run_decode(c), ref_decode(c), "f32")


def test_decode_never_reads_outside_ranges():
    """Rows outside every request's range hold NaN; a tile that over-read them would poison O."""
    s = W.LLAMA_SHAPE
    lens = [1, 70, 129, 300, 64]
    starts = [3, 80, 160, 400, 900]
    c = W.random_decode((102,), s, kv_lens=lens, kv_starts=starts, rows=1100, agents=[0, 1, 2, 0, 2])
    used = np.zeros(1100, bool)
    for a, n in zip(starts, lens):
        used[a:a + n] = True
    for t in (c.K, c.V, c.V_lr):
        W.fill_rows(t, np.where(~used)[0], float("nan"))
    say("decode NaN poison outside ranges")
    for split in (0, 64, 128):
        check(run_decode(c, keys_per_split=split), ref_decode(c), "bf16", f"split {split}")


def test_decode_invalid_requests_give_nan_rows():
    s = W.LLAMA_SHAPE
    c = W.random_decode((103,), s, kv_lens=[50, 60, 40, 30, 20, 10], kv_starts=[0, 100, 0, 200, 10, 0], rows=300,
                        agents=[0, 3, 1, -2, 2, 0])
    kv_len = c.kv_len.copy()
    kv_start = c.kv_start.copy()
    kv_len[2] = 400            # beyond max_kv_len (passed as 100) and beyond the cache
    kv_start[4] = 290          # range runs past kv_rows = 300
    kv_start[5] = -1           # negative start
    cc = W.DecodeBatch(s, c.Q, c.K, c.V, c.V_lr, c.B, kv_start, kv_len, c.agent)
    say("decode invalid requests")
    got = run_decode(cc, max_kv_len=100)
    assert np.all(np.isnan(got[[1, 2, 3, 4, 5]]))
    check(got[[0]], ref_decode(c, requests=[0]), "bf16")


def test_decode_mixed_adapted_and_adapter_free():
    """Double batching (PReCache paper, section 3): adapted requests and adapter-free ones (agent -1,
    base cache alone) over shared rows in one launch."""
    s = W.LLAMA_SHAPE
    c = W.random_decode((106,), s, kv_lens=[900, 900, 900, 130, 130, 1, 0], kv_starts=[0, 0, 0, 700, 700, 5, 0],
                        rows=900, agents=[1, -1, 2, -1, 0, -1, -1], b_std=1.0)
    say("decode mixed adapted / adapter-free")
    ref = ref_decode(c)
    for split in (0, 64, 256):
        got = run_decode(c, keys_per_split=split)
        check(got, ref, "bf16", f"split {split}")
        assert np.all(got[6] == 0.0)


def test_decode_adapter_free_reads_no_B():
    """Adapter-free requests only, with B all NaN and agent 0's LR columns huge: B is never read and the
    LR product of the streamed V_lr columns is dropped."""
    s = W.LLAMA_SHAPE
    c = W.random_decode((107,), s, kv_lens=[500, 64, 1], kv_starts=[0, 400, 499], rows=500, agents=[-1, -1, -1])
    lr = c.V_lr.as_f32()
    lr[:, :s.rank] = 1.0e30
    nanB = W.to_storage(np.full(c.B.shape, np.nan, np.float32), "bf16")
    cc = W.DecodeBatch(s, c.Q, c.K, c.V, W.to_storage(lr, "bf16"), nanB, c.kv_start, c.kv_len, c.agent)
    say("decode adapter-free, B = NaN")
    got = run_decode(cc)
    assert np.all(np.isfinite(got))
    check(got, ref_decode(cc), "bf16")


def test_decode_agent_signature():
    """B_k = 0.5 (k+1) everywhere and the LR slice of agent k offset by 10k: a wrong slice or B is off by O(1)."""
    s = W.LLAMA_SHAPE
    c = W.random_decode((104,), s, kv_lens=[500, 500, 500, 333], kv_starts=[0, 0, 0, 50], rows=500,
                        agents=[0, 1, 2, 2])
    lr = c.V_lr.as_f32()
    for k in range(3):
        lr[:, k * s.rank:(k + 1) * s.rank] += 10.0 * k
    B = np.concatenate([np.full((1, s.rank, s.d_kv), 0.5 * (k + 1), np.float32) for k in range(3)])
    cc = W.DecodeBatch(s, c.Q, c.K, c.V, W.to_storage(lr, "bf16"), W.to_storage(B, "bf16"), c.kv_start, c.kv_len,
                       c.agent)
    say("decode agent signature")
    ref = ref_decode(cc)
    assert np.abs(ref[2] - ref[1]).max() > 50
    check(run_decode(cc), ref, "bf16")


def test_decode_lr_isolation():
    """V_base = 0 and B ~ N(0,1): the output is the LR path alone, so errors in it cannot hide under atol."""
    s = W.LLAMA_SHAPE
    c = W.random_decode((105,), s, kv_lens=[4000, 1234, 77], agents=[2, 0, 1], b_std=1.0)
    zero = W.to_storage(np.zeros(c.V.shape, np.float32), "bf16")
    cc = W.DecodeBatch(s, c.Q, c.K, zero, c.V_lr, c.B, c.kv_start, c.kv_len, c.agent)
    say("decode LR isolation")
    ref = ref_decode(cc)
    got = run_decode(cc)
    st = check(got, ref, "bf16")
    assert st["normwise"] < 2e-2


def test_decode_is_deterministic():
    c = W.llama_decode(agent=2)
    say("decode determinism")
    a = run_decode(c)
    b = run_decode(c)
    assert np.array_equal(a, b)


def test_long_context_decode_16x66400():
    """The full 16-request x 66,400-token launch in the configuration the benchmark times (the
    library's default slices), every request checked end to end against the oracle."""
    say("decode 16 x 66400: generating inputs")
    c = W.llama_long_decode()
    say("decode 16 x 66400: running")
    got = run_decode(c)
    for b in range(c.batch):
        say(f"decode 16 x 66400: oracle request {b}")
        check(got[b:b + 1], ref_decode(c, requests=[b]), "bf16", f"request {b}")


def test_ministral_layer_decode_full_size():
    """One Ministral-shaped layer (32 requests of 1,954 .. 28,958 keys, rank 16), every request."""
    say("decode ministral layer 0: generating inputs")
    dec, _ = W.ministral_layer(0)
    got = run_decode(dec)
    for b in range(dec.batch):
        say(f"decode ministral layer 0: oracle request {b} (L={int(dec.kv_len[b])})")
        check(got[b:b + 1], ref_decode(dec, requests=[b]), "bf16", f"request {b}")



@pytest.mark.parametrize("n_kv", [4, 12, 16])
def test_decode_long_batches_every_head_group(n_kv):
    """The library's split of long batches (8-16 slices per request) for KV head counts that
    leave waves of a workgroup without a head (4, 12) and that need two head groups (12, 16), with
    empty, adapter-free and one-tile requests between long ones."""
    s = W.Shape(n_q=2 * n_kv, n_kv=n_kv, d_head=64, rank=8, n_agents=3, d_model=256, dtype="bf16")
    long = 16000 if n_kv == 4 else 8200   # 4,006 tiles over 240 slices; 2,062 over 120
    lens = [long] * 7 + [1, 0, 33] + [long + 96]
    agents = [0, 1, 2, -1, 0, 1, 2, 1, 0, 2, 1]
    c = W.random_decode((940, n_kv), s, lens, agents=agents)
    say(f"decode long batch n_kv={n_kv}")
    got = run_decode(c)
    for b in range(c.batch):
        check(got[b:b + 1], ref_decode(c, requests=[b]), "bf16", f"n_kv={n_kv} request {b}")
    assert np.all(got[8] == 0.0)

# ------------------------------------------------------------------------------ paged cache
def run_decode_paged(c: W.PagedDecodeBatch, keys_per_split=0, max_kv_len=None):
    s = c.shape
    O = lra.lra_attn_decode_paged(dev(c.Q), dev(c.K_pages), dev(c.V_pages), dev(c.Vlr_pages),
                                  dev_idx(c.block_table, torch.int32), dev_idx(c.kv_len, torch.int32),
                                  c.max_kv_len if max_kv_len is None else max_kv_len, dev(c.B),
                                  dev_idx(c.agents, torch.int32), s.scale, keys_per_split)
    torch.cuda.synchronize()
    return host64(O)


def ref_decode_paged(c: W.PagedDecodeBatch, requests=None):
    return oracle.attn_decode_paged(c.Q.as_f64(), c.K_pages.as_f64(), c.V_pages.as_f64(), c.Vlr_pages.as_f64(),
                                    c.B.as_f64(), c.block_table, c.kv_len, c.agents, c.shape.scale, requests=requests)


@pytest.mark.parametrize("page_size", [32, 64, 256])
def test_decode_paged_cache(page_size):
    """Shuffled pages, a prefix of pages shared by the longer requests, ragged and empty requests,
    adapted and adapter-free; splits of several sizes."""
    s = W.LLAMA_SHAPE
    lens = [1, 31, 32, 33, 700, 0, 1999, 513, 64]
    c = W.random_paged_decode((130, page_size), s, lens, page_size, agents=[0, 1, 2, -1, 1, 0, 2, -1, 0],
                              shared_prefix_pages=1)
    say(f"decode paged P={page_size}")
    ref = ref_decode_paged(c)
    for split in (0, 64, 384):
        got = run_decode_paged(c, keys_per_split=split)
        check(got, ref, "bf16", f"P={page_size} split={split}")
        assert np.all(got[5] == 0.0)


def test_decode_paged_equals_contiguous_bits():
    """With the same split, the paged call gives the same bits as lra_attn_decode over the rows laid
    out contiguously (the arithmetic order is the same; only addresses differ)."""
    s = W.LLAMA_SHAPE
    lens = [900, 130, 64, 1]
    P = 64
    c = W.random_paged_decode((131,), s, lens, P, agents=[2, 0, -1, 1], shared_prefix_pages=1)
    got = run_decode_paged(c, keys_per_split=256)
    rows, starts = [], []
    for b, L in enumerate(lens):
        starts.append(sum(len(r) for r in rows))
        pages = c.block_table[b][:(L + P - 1) // P]
        rows.append(np.concatenate([np.arange(pg * P, pg * P + P) for pg in pages])[:L] if L else np.zeros(0, np.int64))
    idx = np.concatenate(rows)
    flat = lambda t: W.HostTensor(t.data.reshape((-1,) + t.data.shape[2:])[idx], t.dtype)
    cc = W.DecodeBatch(s, c.Q, flat(c.K_pages), flat(c.V_pages), flat(c.Vlr_pages), c.B, np.asarray(starts, np.int64),
                       c.kv_len, c.agents)
    say("decode paged vs contiguous bits")
    assert np.array_equal(got, run_decode(cc, keys_per_split=256))


def test_decode_paged_bad_page_gives_nan_request_and_unnamed_pages_are_unread():
    """A page id outside [0, n_pages) poisons only its request; pages that no request names hold NaN."""
    s = W.LLAMA_SHAPE
    P = 32
    c = W.random_paged_decode((132,), s, [200, 100, 64], P, agents=[0, 1, 2], spare_pages=4)
    named = np.unique(np.concatenate([c.block_table[b][:(int(L) + P - 1) // P] for b, L in enumerate(c.kv_len)]))
    unnamed = np.setdiff1d(np.arange(c.K_pages.shape[0]), named)
    assert len(unnamed) >= 4
    for t in (c.K_pages, c.V_pages, c.Vlr_pages):
        W.fill_rows(t, unnamed, float("nan"))
    ref = ref_decode_paged(c)
    table = c.block_table.copy()
    table[1, 2] = c.K_pages.shape[0] + 5      # request 1's third page is out of range
    cc = W.PagedDecodeBatch(s, c.Q, c.K_pages, c.V_pages, c.Vlr_pages, c.B, table, c.kv_len, c.agents)
    say("decode paged bad page / unread pages")
    got = run_decode_paged(cc)
    assert np.all(np.isnan(got[1]))
    check(got[[0, 2]], ref[[0, 2]], "bf16")


# ---------------------------------------------------------------- LoRA on the keys (qkvo)
def _dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def run_decode_qkvo(c: W.QkvoDecodeBatch, keys_per_split=0, K_lr=None, B_k=None, agent=None, Q=None):
    b = c.base
    O = lra.lra_attn_decode_qkvo(dev(b.Q if Q is None else Q), dev(b.K), dev(b.V), dev(b.V_lr),
                                 dev(c.K_lr if K_lr is None else K_lr), dev_idx(b.kv_start, torch.int64),
                                 dev_idx(b.kv_len, torch.int32), b.max_kv_len, dev(b.B),
                                 dev(c.B_k if B_k is None else B_k), _dev_f32(c.cos), _dev_f32(c.sin),
                                 dev_idx(b.agent if agent is None else agent, torch.int32), b.shape.scale,
                                 keys_per_split)
    torch.cuda.synchronize()
    return host64(O)


def ref_decode_qkvo(c: W.QkvoDecodeBatch, requests=None, Q=None):
    b = c.base
    return oracle.attn_decode_qkvo((b.Q if Q is None else Q).as_f64(), F64Rows(b.K), F64Rows(b.V), F64Rows(b.V_lr),
                                   F64Rows(c.K_lr), b.B.as_f64(), c.B_k.as_f64(), c.cos, c.sin, b.kv_start,
                                   b.kv_len, b.agent, b.shape.scale, requests=requests)


QKVO_CASES = [
    # n_q, n_kv, d, r, kv_lens, kv_starts, agents, keys_per_split
    (32, 8, 128, 8, [300, 1, 65, 200], None, [0, 2, 1, -1], 0),
    (32, 8, 128, 16, [513, 257, 31, 64], [0, 100, 400, 0], [2, 0, -1, 1], 128),
    (8, 2, 64, 8, [700, 129, 2], None, [1, 1, 0], 64),
    (8, 8, 64, 16, [97, 97, 33], [0, 0, 50], [0, 2, 1], 0),
    (7, 1, 128, 8, [1000, 5], None, [2, 0], 256),
    (64, 8, 128, 8, [160, 320], None, [1, 2], 64),
]


@pytest.mark.parametrize("n_q,n_kv,d,r,lens,starts,agents,split", QKVO_CASES)
def test_decode_qkvo_cases(n_q, n_kv, d, r, lens, starts, agents, split):
    """Decode with LoRA on the keys: ragged lengths, shared and offset rows, mixed agents (incl. the
    adapter-free view), several split sizes; every request against the oracle."""
    s = W.Shape(n_q=n_q, n_kv=n_kv, d_head=d, rank=r, n_agents=3, d_model=256, dtype="bf16")
    rows = None if starts is None else max(a + b for a, b in zip(starts, lens))
    c = W.random_decode_qkvo((330, n_q, n_kv, d, r, len(lens)), s, lens, starts, rows, agents)
    say(f"decode qkvo n_q={n_q} n_kv={n_kv} d={d} r={r} lens={lens} split={split}")
    check(run_decode_qkvo(c, split), ref_decode_qkvo(c), "bf16", f"qkvo {n_q}/{n_kv} d={d} r={r}")


def test_decode_qkvo_llama_long_sampled_requests():
    """Three of the 16 x 66,400-token requests with LoRA on the keys, at the split the benchmark's
    full batch uses, against the oracle."""
    reqs = [0, 7, 15]
    say("decode qkvo llama 66400: generating inputs")
    c = W.llama_long_decode_qkvo(requests=reqs)
    split = lra.lra_attn_decode_default_split(16, 8, 66400)
    say(f"decode qkvo llama 66400: running (keys_per_split={split})")
    got = run_decode_qkvo(c, split)
    say("decode qkvo llama 66400: oracle")
    check(got, ref_decode_qkvo(c), "bf16")


def test_decode_qkvo_reduces_to_plain_decode_bits():
    """B_k = 0 makes every rank-r score part exactly zero: the output equals lra_attn_decode's bit for
    bit at the same split. All-adapter-free requests read none of K_lr / B_k (NaN here) and equal
    the plain decode too."""
    s = W.LLAMA_SHAPE
    c = W.random_decode_qkvo((331,), s, [400, 130, 64], [0, 100, 300], 400, [2, 0, 1])
    zero = W.to_storage(np.zeros(c.B_k.shape, np.float32), "bf16")
    say("decode qkvo B_k = 0")
    assert np.array_equal(run_decode_qkvo(c, 128, B_k=zero), run_decode(c.base, 128))
    nan = lambda t: W.to_storage(np.full(t.shape, np.nan, np.float32), "bf16")
    free = np.full(3, -1, np.int32)
    say("decode qkvo adapter-free with NaN key operands")
    got = run_decode_qkvo(c, 128, K_lr=nan(c.K_lr), B_k=nan(c.B_k), agent=free)
    plain = W.DecodeBatch(s, c.base.Q, c.base.K, c.base.V, c.base.V_lr, c.base.B, c.base.kv_start, c.base.kv_len, free)
    assert np.array_equal(got, run_decode(plain, 128))


def test_decode_qkvo_key_part_matters_and_agents_are_isolated():
    s = W.LLAMA_SHAPE
    c = W.random_decode_qkvo((332,), s, [256, 256], None, None, [2, 2])
    got = run_decode_qkvo(c)
    assert np.max(np.abs(got - run_decode(c.base))) > 0.05
    klr = c.K_lr.as_f64().astype(np.float32)
    klr[:, : 2 * s.rank] = np.nan   # agents 0 and 1
    assert np.array_equal(got, run_decode_qkvo(c, K_lr=W.to_storage(klr, "bf16")))


@pytest.mark.parametrize("big", [1.0e5, 1.0e30])
def test_decode_qkvo_beyond_fp16_range_matches_the_oracle(big):
    """Large query, K_lr and B_k entries: the key-score blocks they reach come out non-finite or
    too large for the fp16 pass and are recomputed in fp32; every head of every request matches the
    oracle. An invalid agent still gives NaN rows."""
    s = W.LLAMA_SHAPE
    c = W.random_decode_qkvo((333,), s, [200, 150, 90, 700], None, None, [0, 1, 2, 1])
    q = c.base.Q.as_f64().astype(np.float32)
    q[1, 5, 3] = big
    q[3, 30, 120] = -big
    klr = c.K_lr.as_f64().astype(np.float32)
    klr[int(c.base.kv_start[0]) + 17, 0 * s.rank + 4] = big    # request 0 (agent 0)
    bk = c.B_k.as_f64().astype(np.float32)
    bk[2, 1, 6 * s.d_head + 9] = big / 100                     # agent 2, KV head 6
    Qb, Kb, Bb = W.to_storage(q, "bf16"), W.to_storage(klr, "bf16"), W.to_storage(bk, "bf16")
    say(f"decode qkvo operands {big:g}")
    got = run_decode_qkvo(c, Q=Qb, K_lr=Kb, B_k=Bb)
    cc = W.QkvoDecodeBatch(c.base, Kb, Bb, c.cos, c.sin)
    check(got, ref_decode_qkvo(cc, Q=Qb), "bf16", f"qkvo {big:g}")
    agents = np.array([0, 1, 7, 1], np.int32)
    got = run_decode_qkvo(c, agent=agents, Q=Qb, K_lr=Kb, B_k=Bb)
    assert np.all(np.isnan(got[2]))
    check(got[[0, 1, 3]], ref_decode_qkvo(cc, requests=[0, 1, 3], Q=Qb), "bf16")


def test_decode_split_boundaries_mixed_batch():
    """The library's split (512 keys here) with lengths around 256, 512 and the split: a request
    shorter than one split, one that ends on a split boundary, a long one, an empty and an invalid
    request, adapter-free and adapted requests, checked against the oracle."""
    s = W.Shape(n_q=32, n_kv=8, d_head=128, rank=16, n_agents=3, d_model=256, dtype="bf16")
    C = lra.lra_attn_decode_default_split(12, 8, 40000)
    assert C >= 512
    lens = [1, 255, 256, 511, 512, 513, C - 1, C, C + 1, 3 * C + 300, 0, 40000]
    agents = [0, 1, 2, -1, 0, 1, 2, 0, -1, 1, 0, 2]
    c = W.random_decode((105,), s, lens, agents=agents)
    c.agent = c.agent.copy()
    c.agent[4] = 3   # invalid agent: NaN row, no split
    say(f"decode split boundaries (chunk {C})")
    got = run_decode(c)
    ok = [b for b in range(12) if b != 4]
    check(got[ok], ref_decode(c, requests=ok), "bf16", "split boundaries")
    assert np.all(np.isnan(got[4]))
    assert np.all(got[10] == 0.0)


# ------------------------------------------------------------------------------ strided K/V (head-major)
def run_decode_strided(c: W.DecodeBatch, K_view, V_view, keys_per_split=0):
    s = c.shape
    O = lra.lra_attn_decode_strided(dev(c.Q), K_view, V_view, dev(c.V_lr), dev_idx(c.kv_start, torch.int64),
                                    dev_idx(c.kv_len, torch.int32), c.max_kv_len, dev(c.B),
                                    dev_idx(c.agent, torch.int32), s.scale, keys_per_split)
    torch.cuda.synchronize()
    return host64(O)


@pytest.mark.parametrize("dtype,n_q,n_kv,d,r", [("bf16", 32, 8, 128, 8), ("bf16", 32, 8, 128, 16), ("bf16", 8, 2, 64, 8),
                                                ("f32", 4, 2, 64, 8), ("f32", 16, 2, 128, 16)])
def test_decode_head_major_and_padded_layouts_are_bit_identical(dtype, n_q, n_kv, d, r):
    """The same cache values laid out head-major ([n_kv, rows, d]) and with padded token rows give
    bit-for-bit the token-major call's outputs, which match the oracle."""
    s = W.Shape(n_q=n_q, n_kv=n_kv, d_head=d, rank=r, n_agents=3, d_model=256, dtype=dtype)
    lens = [1, 31, 64, 700, 0, 1900, 257]
    c = W.random_decode((110, n_q, n_kv, d, r), s, lens, agents=[0, 1, 2, -1, 0, 2, 1])
    say(f"decode strided {dtype} {n_q}/{n_kv} d={d} r={r}")
    ref_tm = run_decode(c)
    K, V = dev(c.K), dev(c.V)
    Khm, Vhm = K.transpose(0, 1).contiguous(), V.transpose(0, 1).contiguous()   # [n_kv, rows, d]
    got_hm = run_decode_strided(c, Khm.transpose(0, 1), Vhm.transpose(0, 1))
    assert np.array_equal(got_hm, ref_tm)
    rows = K.shape[0]
    Kp = torch.zeros((rows, n_kv * d + 64), dtype=K.dtype, device="cuda")   # padded token rows
    Vp = torch.zeros_like(Kp)
    Kp[:, :n_kv * d] = K.reshape(rows, -1)
    Vp[:, :n_kv * d] = V.reshape(rows, -1)
    got_pad = run_decode_strided(c, Kp[:, :n_kv * d].view(rows, n_kv, d), Vp[:, :n_kv * d].view(rows, n_kv, d), 64)
    assert np.array_equal(got_pad, run_decode(c, keys_per_split=64))
    check(ref_tm, ref_decode(c), dtype, "token-major")


def test_decode_head_major_16x66400_bit_identical():
    """The 16 x 66,400 batch in the bench's launch configuration, head-major, against the token-major
    call (bit for bit) and the oracle on two requests."""
    say("decode head-major 16 x 66400: generating inputs")
    c = W.llama_long_decode()
    say("decode head-major 16 x 66400: running")
    ref_tm = run_decode(c)
    Khm = dev(c.K).transpose(0, 1).contiguous()
    Vhm = dev(c.V).transpose(0, 1).contiguous()
    got = run_decode_strided(c, Khm.transpose(0, 1), Vhm.transpose(0, 1))
    assert np.array_equal(got, ref_tm)
    for b in (3, 12):
        say(f"decode head-major 16 x 66400: oracle request {b}")
        check(got[b:b + 1], ref_decode(c, requests=[b]), "bf16", f"request {b}")


@pytest.mark.parametrize("page_size", [32, 64])
def test_decode_paged_head_major_pages_are_bit_identical(page_size):
    """The same pages laid out head-major ([n_pages, n_kv, P, d], each KV head's slice of a page
    contiguous) give bit-for-bit the token-major paged call's outputs, for the default and a
    given split."""
    s = W.LLAMA_SHAPE
    lens = [1, 31, 32, 33, 700, 0, 1999, 513, 64]
    c = W.random_paged_decode((132, page_size), s, lens, page_size, agents=[0, 1, 2, -1, 1, 0, 2, -1, 0],
                              shared_prefix_pages=1)
    say(f"decode paged head-major P={page_size}")
    Khnd = dev(c.K_pages).transpose(1, 2).contiguous()   # [n_pages, n_kv, P, d]
    Vhnd = dev(c.V_pages).transpose(1, 2).contiguous()
    for split in (0, 128):
        ref = run_decode_paged(c, keys_per_split=split)
        O = lra.lra_attn_decode_paged_strided(dev(c.Q), Khnd.transpose(1, 2), Vhnd.transpose(1, 2), dev(c.Vlr_pages),
                                              dev_idx(c.block_table, torch.int32), dev_idx(c.kv_len, torch.int32),
                                              c.max_kv_len, dev(c.B), dev_idx(c.agents, torch.int32), s.scale, split)
        torch.cuda.synchronize()
        assert np.array_equal(host64(O), ref), f"split {split}"
    check(ref, ref_decode_paged(c), "bf16", f"P={page_size}")


def test_decode_paged_bench_configuration_bit_identical():
    """The 16 x 66,400 batch as the bench times its paged lines: 32-row pages in a seeded random
    order, token-major and head-major pages, against the contiguous call; all three take the
    library's default slices, which do not depend on the cache layout."""
    say("decode paged bench configuration: generating inputs")
    c = W.llama_long_decode()
    s = c.shape
    Q, K, V, L, B = dev(c.Q), dev(c.K), dev(c.V), dev(c.V_lr), dev(c.B)
    kl = dev_idx(c.kv_len, torch.int32)
    ag = dev_idx(c.agent, torch.int32)
    P = 32
    assert lra.lra_attn_decode_paged_default_split(c.batch, s.n_kv, c.max_kv_len, P) == \
        lra.lra_attn_decode_default_split(c.batch, s.n_kv, c.max_kv_len)
    ref = lra.lra_attn_decode(Q, K, V, L, dev_idx(c.kv_start, torch.int64), kl, c.max_kv_len, B, ag, s.scale, 0)
    torch.cuda.synchronize()
    ref = host64(ref)
    n_pages = K.shape[0] // P
    blocks = int(c.kv_len[0]) // P
    g = torch.Generator(device="cpu")
    g.manual_seed(42)
    table = torch.randperm(n_pages, generator=g).to(torch.int32).reshape(c.batch, blocks)
    tl = table.reshape(-1).long().cuda()   # request b's block j (rows b*L + 32 j ..) lives in page table[b, j]
    Kp = torch.empty((n_pages, P, s.n_kv, s.d_head), dtype=K.dtype, device="cuda")
    Vp, Lp = torch.empty_like(Kp), torch.empty((n_pages, P, L.shape[1]), dtype=L.dtype, device="cuda")
    Kp[tl] = K.view(n_pages, P, s.n_kv, s.d_head)
    Vp[tl] = V.view(n_pages, P, s.n_kv, s.d_head)
    Lp[tl] = L.view(n_pages, P, L.shape[1])
    table = table.cuda()
    say("decode paged bench configuration: token-major pages")
    O = lra.lra_attn_decode_paged(Q, Kp, Vp, Lp, table, kl, c.max_kv_len, B, ag, s.scale, 0)
    torch.cuda.synchronize()
    assert np.array_equal(host64(O), ref)
    say("decode paged bench configuration: head-major pages")
    Khnd, Vhnd = Kp.transpose(1, 2).contiguous(), Vp.transpose(1, 2).contiguous()
    O = lra.lra_attn_decode_paged_strided(Q, Khnd.transpose(1, 2), Vhnd.transpose(1, 2), Lp, table, kl, c.max_kv_len,
                                          B, ag, s.scale, 0)
    torch.cuda.synchronize()
    assert np.array_equal(host64(O), ref)


# ------------------------------------------------------------------------------ shared workspace
def test_decode_workspace_shared_across_shapes_needs_no_initialisation():
    """One workspace, filled with NaN bytes once, serves decodes of growing batch and length in a
    row: every call gives the bits of a call with its own fresh workspace (no part of the workspace
    is read before the same launch writes it)."""
    s = W.LLAMA_SHAPE
    cases = [
        W.random_decode((930,), s, kv_lens=[40], agents=[1]),
        W.random_decode((931,), s, kv_lens=[2000, 3, 0, 1700, 64], agents=[0, 2, 1, -1, 1]),
        W.random_decode((932,), s, kv_lens=[900] * 24 + [33, 4100], agents=[b % 3 for b in range(26)]),
        W.random_decode((935,), s, kv_lens=[5000] * 24 + [70, 4100], agents=[b % 3 for b in range(26)]),
        W.random_decode((933,), s, kv_lens=[1], agents=[2]),
    ]
    need = max(lra.lra_attn_decode_workspace_bytes(c.batch, s.n_q, s.n_kv, s.d_head, s.rank, c.max_kv_len, kps)
               for c in cases for kps in (0, 64))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    for i, c in enumerate(cases):
        for kps in (0, 64):
            args = (dev(c.Q), dev(c.K), dev(c.V), dev(c.V_lr), dev_idx(c.kv_start, torch.int64),
                    dev_idx(c.kv_len, torch.int32), c.max_kv_len, dev(c.B), dev_idx(c.agent, torch.int32), s.scale, kps)
            say(f"decode shared workspace case {i} batch={c.batch} keys_per_split={kps}")
            got = lra.lra_attn_decode(*args, ws)
            fresh = lra.lra_attn_decode(*args)
            torch.cuda.synchronize()
            assert torch.equal(got, fresh)
        check(host64(got), ref_decode(c), "bf16", f"shared workspace case {i}")


SMALL_SHAPES = [("bf16", 32, 8, 128, 8), ("bf16", 32, 8, 128, 16), ("bf16", 64, 8, 128, 8), ("bf16", 8, 2, 64, 8),
                ("bf16", 24, 8, 64, 16), ("f32", 32, 8, 128, 8), ("f32", 8, 4, 64, 16)]


@pytest.mark.parametrize("dtype,n_q,n_kv,d,r", SMALL_SHAPES)
def test_small_batch_single_launch(dtype, n_q, n_kv, d, r):
    """Requests of at most 128 keys (one chunk of 4 tiles): finished in one launch, empty ones zero,
    invalid ones NaN."""
    s = W.Shape(n_q=n_q, n_kv=n_kv, d_head=d, rank=r, n_agents=3, d_model=256, dtype=dtype)
    lens = [1, 31, 32, 33, 0, 100, 128, 97]
    c = W.random_decode((120, n_q, n_kv, d, r), s, lens, agents=[0, 1, 2, -1, 1, 2, 0, 1])
    say(f"decode small single launch {dtype} {n_q}/{n_kv} d={d} r={r}")
    assert lra.lra_attn_decode_workspace_bytes(len(lens), n_q, n_kv, d, r, 128) > 0
    got = run_decode(c)
    check(got, ref_decode(c), dtype, "one chunk")
    assert np.all(got[4] == 0.0)
    kv_start = c.kv_start.copy()
    kv_start[7] = -5
    cc = W.DecodeBatch(s, c.Q, c.K, c.V, c.V_lr, c.B, kv_start, c.kv_len, c.agent)
    got = run_decode(cc)
    assert np.all(np.isnan(got[7]))
    check(got[:7], ref_decode(c, requests=list(range(7))), dtype, "one chunk, an invalid request")


@pytest.mark.parametrize("dtype,n_q,n_kv,d,r", SMALL_SHAPES)
def test_small_batch_chunks_match_the_split_launch(dtype, n_q, n_kv, d, r):
    """Several 256-key chunks per request (the small-batch launch and its merge) against the oracle,
    and against the split launch (an explicit keys_per_split) within the same tolerance."""
    s = W.Shape(n_q=n_q, n_kv=n_kv, d_head=d, rank=r, n_agents=3, d_model=256, dtype=dtype)
    lens = [1900, 257, 512, 0, 1, 1300]
    c = W.random_decode((121, n_q, n_kv, d, r), s, lens, agents=[0, 1, 2, 0, -1, 1])
    say(f"decode small chunks {dtype} {n_q}/{n_kv} d={d} r={r}")
    ref = ref_decode(c)
    got = run_decode(c)
    check(got, ref, dtype, "small-batch launch")
    assert np.all(got[3] == 0.0)
    check(run_decode(c, keys_per_split=256), ref, dtype, "split launch")


def test_small_batch_single_launch_256_key_chunks():
    """40 requests of at most 256 keys over 8 KV heads: one launch of 8-wave workgroups (256-key chunks)."""
    s = W.LLAMA_SHAPE
    lens = [int(x) for x in np.random.default_rng(123).integers(0, 257, size=40)]
    lens[:4] = [256, 1, 0, 129]
    c = W.random_decode((123,), s, lens, agents=[i % 4 - 1 for i in range(40)])
    say("decode 40 requests of <= 256 keys")
    got = run_decode(c)
    check(got, ref_decode(c), "bf16", "one 256-key chunk")
    assert np.all(got[2] == 0.0)


def test_small_batch_threshold():
    """Every regime of the small-batch choice over 8 KV heads: 2 requests of 1,900 keys (128-key
    chunks), 3, 7 and 8 (256-key chunks, up to 512 workgroups) and 9 (the split launch)."""
    s = W.LLAMA_SHAPE
    for nreq in (2, 3, 7, 8, 9):
        c = W.random_decode((122, nreq), s, [1900] * nreq, agents=[i % 3 for i in range(nreq)])
        say(f"decode {nreq} x 1900 around the small-batch limit")
        check(run_decode(c), ref_decode(c), "bf16", f"{nreq} requests")


def test_small_batch_chunks_invalid_and_empty_requests():
    """The chunked launch's merge: requests with a bad range, a bad agent, no keys, and valid ones
    of several chunks side by side; valid rows match the oracle, invalid rows are NaN, empty zero."""
    s = W.LLAMA_SHAPE
    c = W.random_decode((124,), s, kv_lens=[900, 300, 0, 700, 513], kv_starts=[0, 100, 0, 50, 200], rows=1000,
                        agents=[0, 1, 2, 2, 1])
    kv_start = c.kv_start.copy()
    agent = c.agent.copy()
    kv_start[1] = 800          # 800 + 300 runs past the 1,000 cache rows
    agent[3] = 7               # no such agent
    cc = W.DecodeBatch(s, c.Q, c.K, c.V, c.V_lr, c.B, kv_start, c.kv_len, agent)
    say("decode chunked launch, invalid and empty requests")
    got = run_decode(cc)
    assert np.all(np.isnan(got[[1, 3]]))
    assert np.all(got[2] == 0.0)
    check(got[[0, 4]], ref_decode(c, requests=[0, 4]), "bf16", "valid requests beside invalid ones")
