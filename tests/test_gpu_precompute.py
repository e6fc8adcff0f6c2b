"""GPU parity of lra_lr_precompute against the fp64 oracle (needs an MI355X and liblra.so)."""
import numpy as np
import pytest
import torch

import oracle
import rank_kv_cache_amd as lra
import workloads as W
from tests.gpu_util import check, dev, dev_idx, host64, say, stacked_A

pytestmark = pytest.mark.gpu


def run_pre(case: W.PrecomputeCase, V_lr_init: np.ndarray, out_rows=None, workspace=None):
    s = case.shape
    V = dev(W.to_storage(V_lr_init.astype(np.float32), s.dtype))
    rows = None if out_rows is None else dev_idx(out_rows, torch.int64)
    lra.lra_lr_precompute(dev(case.X), dev(stacked_A(case.A)), s.n_agents, s.rank, V, rows, workspace)
    torch.cuda.synchronize()
    return host64(V)


def test_llama_precompute_2048x4096():
    case = W.llama_precompute()
    say("precompute 2048 x 4096 -> 24")
    got = run_pre(case, np.zeros((2048, 24)))
    check(got, oracle.lr_precompute(case.X.as_f64(), case.A.as_f64()), "bf16")


def test_tiny_fp32_precompute():
    tw = W.tiny_workload()
    case = W.PrecomputeCase(W.TINY_SHAPE, tw.X, tw.A)
    say("precompute tiny fp32")
    got = run_pre(case, np.zeros((256, 24)))
    check(got, oracle.lr_precompute(case.X.as_f64(), case.A.as_f64()), "f32")


def test_ministral_precompute_scatter_into_cache():
    dec, pre = W.ministral_layer(3)
    rows = dec.kv_start + dec.kv_len.astype(np.int64) - 1
    cache = dec.V_lr.as_f64()
    say("precompute ministral scatter")
    got = run_pre(pre, cache, rows)
    ref = oracle.lr_precompute_into(cache, pre.X.as_f64(), pre.A.as_f64(), rows)
    check(got[rows], ref[rows], "bf16")
    untouched = np.setdiff1d(np.arange(cache.shape[0]), rows)
    assert np.array_equal(got[untouched], cache[untouched])


@pytest.mark.parametrize("dtype,T,d_model,N,r", [
    ("bf16", 1, 4096, 3, 8), ("bf16", 37, 4096, 3, 16), ("bf16", 100, 256, 3, 8), ("bf16", 513, 1024, 2, 16),
    ("bf16", 64, 512, 9, 8), ("bf16", 20, 2048, 5, 16), ("f32", 1, 256, 3, 8), ("f32", 300, 256, 3, 8),
    ("f32", 17, 1024, 9, 16),
    # long X: 256 row ranges of 16-17 (35-36) rows, so tiles end inside a range
    ("bf16", 4100, 512, 3, 8), ("bf16", 9000, 256, 2, 16),
    # 16 output columns (one group); d_model past what a wave keeps in registers (At reloaded per
    # batch of chunks: beyond 4096 for bf16, 2048 for fp32)
    ("bf16", 33, 4096, 2, 8), ("bf16", 70, 8192, 3, 8), ("f32", 40, 4096, 3, 8), ("bf16", 300, 12288, 3, 16),
    # 4096 rows and more take 32-column groups: with At reloaded per batch, and in fp32
    ("bf16", 4200, 8192, 3, 8), ("f32", 4500, 256, 3, 8),
    # 8-wave workgroups with both column tiles' At in registers (bf16, 17..32 columns, d_model up to
    # 4096): ragged row ranges, 32 columns, one agent of rank 24
    ("bf16", 4100, 4096, 2, 16), ("bf16", 5000, 2048, 3, 8), ("bf16", 4111, 4096, 1, 24), ("bf16", 8200, 4096, 3, 8),
])
def test_precompute_shapes(dtype, T, d_model, N, r):
    s = W.Shape(n_q=4, n_kv=2, d_head=64, rank=r, n_agents=N, d_model=d_model, dtype=dtype)
    case = W.random_precompute((200, T, d_model, N, r), s, T)
    say(f"precompute {dtype} T={T} d_model={d_model} N={N} r={r}")
    got = run_pre(case, np.zeros((T, N * r)))
    check(got, oracle.lr_precompute(case.X.as_f64(), case.A.as_f64()), dtype)


def test_precompute_calls_in_a_row_and_bad_rows():
    """Calls of different sizes in a row (a workspace argument is accepted and unused); out_rows
    entries outside the cache are skipped."""
    s = W.MINISTRAL_SHAPE
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    for T in (64, 32, 7, 64):
        case = W.random_precompute((201, T), s, T)
        rows = np.arange(T, dtype=np.int64) * 2
        rows[0] = -3
        rows[-1] = 10_000
        cache = np.full((2 * T, 48), 7.0)
        say(f"precompute workspace reuse T={T}")
        got = run_pre(case, cache, rows, ws)
        ref = oracle.lr_precompute_into(cache, case.X.as_f64()[1:-1], case.A.as_f64(), rows[1:-1])
        check(got, ref, "bf16")


def test_precompute_is_deterministic():
    case = W.llama_precompute(T=300)
    a = run_pre(case, np.zeros((300, 24)))
    b = run_pre(case, np.zeros((300, 24)))
    assert np.array_equal(a, b)


def test_llama_precompute_whole_context_every_row():
    """The Llama prefill's whole context through the precompute in one call (18,432 x 4,096 -> 24
    columns, 151 MB of X), every output against the oracle."""
    case = W.llama_precompute(T=18432)
    say("precompute 18432 x 4096 -> 24")
    got = run_pre(case, np.zeros((18432, 24)))
    check(got, oracle.lr_precompute(case.X.as_f64(), case.A.as_f64()), "bf16")


def test_precompute_long_x_scatter():
    """6,000 rows of 4,096 -> 24 (32-column groups) written through a row map: a permutation of the
    cache's rows with some entries outside it (skipped)."""
    s = W.LLAMA_SHAPE
    T = 6000
    case = W.random_precompute((202, T), s, T)
    rows = np.random.default_rng(202).permutation(T + 100)[:T].astype(np.int64)
    rows[5] = -1
    rows[77] = T + 100
    cache = np.full((T + 100, 24), 3.0)
    say("precompute long X, scattered rows")
    got = run_pre(case, cache, rows)
    keep = (rows >= 0) & (rows < T + 100)
    ref = oracle.lr_precompute_into(cache, case.X.as_f64()[keep], case.A.as_f64(), rows[keep])
    check(got, ref, "bf16")
