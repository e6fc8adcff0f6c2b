"""GPU parity of lra_attn_decode_step (the decode step with the newest tokens' LR rows formed in the
same launch) against the fp64 oracle: lr_precompute into each request's newest row, then attn_decode."""
import numpy as np
import pytest
import torch

import oracle
import rank_kv_cache_amd as lra
import workloads as W
from tests.gpu_util import check, dev, dev_idx, host64, say, stacked_A

pytestmark = pytest.mark.gpu


def newest_rows(c: W.DecodeBatch):
    """Requests whose newest row is written: a key, a valid range and agent."""
    s = c.shape
    out = {}
    for b in range(c.batch):
        n, st, a = int(c.kv_len[b]), int(c.kv_start[b]), int(c.agent[b])
        if n > 0 and st >= 0 and st + n <= c.K.shape[0] and -1 <= a < s.n_agents:
            out[b] = st + n - 1
    return out


def run_step(c: W.DecodeBatch, X: W.HostTensor, A_stacked: W.HostTensor, keys_per_split=0):
    s = c.shape
    Vlr = dev(c.V_lr)
    O = lra.lra_attn_decode_step(dev(c.Q), dev(c.K), dev(c.V), Vlr, dev_idx(c.kv_start, torch.int64),
                                 dev_idx(c.kv_len, torch.int32), c.max_kv_len, dev(c.B), dev_idx(c.agent, torch.int32),
                                 s.scale, dev(X), dev(A_stacked), keys_per_split)
    torch.cuda.synchronize()
    return host64(O), Vlr


def ref_step(c: W.DecodeBatch, X: W.HostTensor, A_pages: W.HostTensor, requests=None):
    """The oracle: the newest rows from lr_precompute (fp64), then the decode over them."""
    rows = newest_rows(c)
    lr = oracle.lr_precompute(X.as_f64(), A_pages.as_f64())
    reqs = range(c.batch) if requests is None else requests
    outs = []
    for b in reqs:
        st, n = int(c.kv_start[b]), int(c.kv_len[b])
        if b not in rows:
            outs.append(oracle.attn_decode(c.Q.as_f64()[b:b + 1], c.K.as_f64(), c.V.as_f64(), c.V_lr.as_f64(),
                                           c.B.as_f64(), [st], [n], [int(c.agent[b])], c.shape.scale))
            continue
        Vlr_b = W.HostTensor(c.V_lr.data[st:st + n], c.V_lr.dtype).as_f64()
        Vlr_b[-1, :lr.shape[1]] = lr[b]
        outs.append(oracle.attn_decode(c.Q.as_f64()[b:b + 1], W.HostTensor(c.K.data[st:st + n], c.K.dtype).as_f64(),
                                       W.HostTensor(c.V.data[st:st + n], c.V.dtype).as_f64(), Vlr_b, c.B.as_f64(),
                                       [0], [n], [int(c.agent[b])], c.shape.scale))
    return np.concatenate(outs), lr, rows


def check_rows(Vlr: torch.Tensor, c: W.DecodeBatch, lr: np.ndarray, rows: dict, dtype: str):
    """The written newest rows against the oracle; every other row untouched."""
    got = host64(Vlr)
    before = c.V_lr.as_f64()
    NR = lr.shape[1]
    written = np.zeros(got.shape[0], bool)
    for b, r in rows.items():
        check(got[r:r + 1, :NR], lr[b:b + 1], dtype, f"newest row of request {b}")
        written[r] = True
    assert np.array_equal(got[~written], before[~written])
    assert np.array_equal(got[written][:, NR:], before[written][:, NR:])


CASES = [
    # (dtype, n_q, n_kv, d, r, d_model, lens, agents)
    ("bf16", 32, 8, 128, 8, 512, [1, 31, 32, 33, 64, 300, 1900], [0, 1, 2, -1, 2, 1, 0]),
    ("bf16", 32, 8, 128, 16, 256, [2000, 5, 0, 640, 96], [1, 2, 0, 1, -1]),
    ("bf16", 8, 2, 64, 8, 128, [100, 1, 57], [2, 0, 1]),
    ("bf16", 24, 8, 128, 16, 1024, [700, 33], [0, 2]),
    ("f32", 4, 2, 64, 8, 128, [70, 1, 33, 64], [0, 1, 2, -1]),
    ("f32", 32, 8, 128, 16, 256, [129, 400], [1, 0]),
]


@pytest.mark.parametrize("dtype,n_q,n_kv,d,r,d_model,lens,agents", CASES)
@pytest.mark.parametrize("split", [0, 64])
def test_decode_step_cases(dtype, n_q, n_kv, d, r, d_model, lens, agents, split):
    s = W.Shape(n_q=n_q, n_kv=n_kv, d_head=d, rank=r, n_agents=3, d_model=d_model, dtype=dtype)
    c = W.random_decode((940, n_kv, d, r, len(lens)), s, lens, agents=agents)
    X = W.normal((941, len(lens)), (len(lens), d_model), 1.0, dtype)
    A = W.normal((942, d_model), (d_model, s.n_agents * r), 1.0 / np.sqrt(d_model), dtype)   # the pages' [d_model, N*r]
    say(f"decode step {dtype} {n_q}/{n_kv} d={d} r={r} d_model={d_model} lens={lens} split={split}")
    got, Vlr = run_step(c, X, stacked_A(A), split)
    ref, lr, rows = ref_step(c, X, A)
    check(got, ref, dtype, "outputs")
    check_rows(Vlr, c, lr, rows, dtype)


def test_decode_step_invalid_requests():
    """An invalid agent gives NaN and writes no row; an empty request gives zeros and writes none."""
    s = W.LLAMA_SHAPE
    c = W.random_decode((943,), s, [50, 0, 80], agents=[0, 1, 2])
    c.agent = c.agent.copy()
    c.agent[2] = 7
    X = W.normal((944,), (3, 256), 1.0, "bf16")
    A = W.normal((945,), (256, s.n_agents * s.rank), 1.0 / 16, "bf16")
    sh = W.Shape(n_q=s.n_q, n_kv=s.n_kv, d_head=s.d_head, rank=s.rank, n_agents=s.n_agents, d_model=256, dtype="bf16")
    c.shape = sh
    say("decode step invalid requests")
    got, Vlr = run_step(c, X, stacked_A(A))
    assert np.all(np.isnan(got[2])) and np.all(got[1] == 0.0)
    ref, lr, rows = ref_step(c, X, A, requests=[0])
    check(got[0:1], ref, "bf16", "valid request")
    assert set(rows) == {0}
    check_rows(Vlr, c, lr, rows, "bf16")


@pytest.mark.parametrize("layer", [0, 35])
def test_decode_step_ministral_layer_all_requests(layer):
    """A Ministral-shaped layer (32 requests of 1,954 .. 28,958 keys, rank 16, d_model 4,096): the step
    writes the 32 newest LR rows and decodes every request in the default launch configuration."""
    say(f"decode step ministral layer {layer}: generating inputs")
    dec, pre = W.ministral_layer(layer)
    got, Vlr = run_step(dec, pre.X, stacked_A(pre.A))
    rows = newest_rows(dec)
    lr = oracle.lr_precompute(pre.X.as_f64(), pre.A.as_f64())
    got_rows = host64(Vlr[torch.as_tensor(np.array([rows[b] for b in sorted(rows)]), device="cuda")])
    check(got_rows, lr[sorted(rows)], "bf16", "newest rows")
    for b in range(dec.batch):
        say(f"decode step ministral layer {layer}: oracle request {b}")
        ref, _, _ = ref_step(dec, pre.X, pre.A, requests=[b])
        check(got[b:b + 1], ref, "bf16", f"request {b}")


def test_decode_step_matches_precompute_then_decode():
    """The step and the two separate calls (lra_lr_precompute with the newest rows, then
    lra_attn_decode) agree within the decode's tolerance and write the same rows within one rounding."""
    s = W.LLAMA_SHAPE
    sh = W.Shape(n_q=s.n_q, n_kv=s.n_kv, d_head=s.d_head, rank=s.rank, n_agents=s.n_agents, d_model=4096, dtype="bf16")
    lens = [1900, 64, 7, 5000, 333]
    c = W.random_decode((946,), sh, lens, agents=[0, 1, 2, 1, -1])
    X = W.normal((947,), (len(lens), 4096), 1.0, "bf16")
    A = W.normal((948,), (4096, sh.n_agents * sh.rank), 1.0 / 64, "bf16")
    say("decode step against precompute + decode")
    got, Vlr_step = run_step(c, X, stacked_A(A))
    Vlr = dev(c.V_lr)
    rows = c.kv_start + c.kv_len.astype(np.int64) - 1
    lra.lra_lr_precompute(dev(X), dev(stacked_A(A)), sh.n_agents, sh.rank, Vlr, dev_idx(rows, torch.int64))
    O = lra.lra_attn_decode(dev(c.Q), dev(c.K), dev(c.V), Vlr, dev_idx(c.kv_start, torch.int64),
                            dev_idx(c.kv_len, torch.int32), c.max_kv_len, dev(c.B), dev_idx(c.agent, torch.int32), sh.scale)
    two = host64(O)
    check(got, two, "bf16", "step vs two calls")
    a, b = host64(Vlr_step)[rows], host64(Vlr)[rows]
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 1e-30)
