"""The agent-major LR cache layout ([N, rows, r] per agent) against the interleaved one ([rows, N*r]):
the same values give the same output bits on every entry point that takes vlr_agent_stride, and the
precompute and the decode step write the same values into either layout (needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
import rank_kv_cache_amd as lra
import workloads as W
from tests.gpu_util import check, dev, dev_idx, host64, say, stacked_A

pytestmark = pytest.mark.gpu


def agent_major(V_lr: torch.Tensor, n_agents: int, rank: int, pad: int = 0) -> torch.Tensor:
    """[rows, N*r] interleaved -> [N, rows, r] agent-major view (ld_vlr = r + pad, padded rows)."""
    rows = V_lr.shape[0]
    buf = torch.full((n_agents, rows, rank + pad), float("nan"), dtype=V_lr.dtype, device=V_lr.device)
    buf[:, :, :rank] = V_lr.view(rows, n_agents, rank).permute(1, 0, 2)
    return buf[:, :, :rank]


class F64Rows:
    def __init__(self, t: W.HostTensor):
        self.t = t

    def __getitem__(self, idx):
        return W.HostTensor(self.t.data[idx], self.t.dtype).as_f64()


def interleaved(V_am: torch.Tensor) -> torch.Tensor:
    n, rows, r = V_am.shape
    return V_am.permute(1, 0, 2).reshape(rows, n * r)


SHAPES = [("bf16", 32, 8, 128, 8), ("bf16", 32, 8, 128, 16), ("bf16", 8, 2, 64, 8), ("f32", 16, 2, 128, 16)]


@pytest.mark.parametrize("dtype,n_q,n_kv,d,r", SHAPES)
@pytest.mark.parametrize("pad", [0, 8])
def test_decode_agent_major_bits(dtype, n_q, n_kv, d, r, pad):
    s = W.Shape(n_q=n_q, n_kv=n_kv, d_head=d, rank=r, n_agents=3, d_model=256, dtype=dtype)
    lens = [1, 31, 32, 33, 700, 0, 1500, 64]
    c = W.random_decode((960, n_q, n_kv, d, r), s, lens, agents=[0, 1, 2, -1, 1, 0, 2, 1])
    say(f"decode agent-major {dtype} {n_q}/{n_kv} d={d} r={r} pad={pad}")
    L = dev(c.V_lr)
    args = (dev(c.Q), dev(c.K), dev(c.V))
    idx = (dev_idx(c.kv_start, torch.int64), dev_idx(c.kv_len, torch.int32), c.max_kv_len, dev(c.B),
           dev_idx(c.agent, torch.int32), s.scale)
    for split in (0, 64):
        ref = lra.lra_attn_decode(*args, L, *idx, split)
        got = lra.lra_attn_decode(*args, agent_major(L, 3, r, pad), *idx, split)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"split {split}"


def test_decode_agent_major_16x66400():
    """The long-context launch with the agent-major cache: the same bits as with the interleaved
    cache, and two requests end to end against the oracle."""
    say("decode 16 x 66400 agent-major: generating inputs")
    c = W.llama_long_decode()
    s = c.shape
    L = dev(c.V_lr)
    args = (dev(c.Q), dev(c.K), dev(c.V))
    idx = (dev_idx(c.kv_start, torch.int64), dev_idx(c.kv_len, torch.int32), c.max_kv_len, dev(c.B),
           dev_idx(c.agent, torch.int32), s.scale)
    say("decode 16 x 66400 agent-major: running")
    ref = lra.lra_attn_decode(*args, L, *idx)
    Lam = agent_major(L, s.n_agents, s.rank)
    del L
    got = lra.lra_attn_decode(*args, Lam, *idx)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    got = host64(got)
    for b in (0, c.batch - 1):
        say(f"decode 16 x 66400 agent-major: oracle request {b}")
        want = oracle.attn_decode(c.Q.as_f64(), F64Rows(c.K), F64Rows(c.V), F64Rows(c.V_lr), c.B.as_f64(),
                                  c.kv_start, c.kv_len, c.agent, s.scale, requests=[b])
        check(got[b:b + 1], want, "bf16", f"request {b}")


def test_decode_step_agent_major_bits():
    s = W.MINISTRAL_SHAPE
    lens = [1954, 40, 1, 3000, 700]
    c = W.random_decode((961,), s, lens, agents=[0, 1, 2, 1, -1])
    X = dev(W.normal((961, 1), (len(lens), s.d_model), 1.0, s.dtype))
    A = dev(W.normal((961, 2), (s.n_agents * s.rank, s.d_model), 1.0 / 64, s.dtype))
    say("decode step agent-major")
    L1 = dev(c.V_lr)
    L2 = agent_major(dev(c.V_lr), s.n_agents, s.rank, pad=8)
    args = (dev(c.Q), dev(c.K), dev(c.V))
    idx = (dev_idx(c.kv_start, torch.int64), dev_idx(c.kv_len, torch.int32), c.max_kv_len, dev(c.B),
           dev_idx(c.agent, torch.int32), s.scale, X, A)
    ref = lra.lra_attn_decode_step(*args, L1, *idx)
    got = lra.lra_attn_decode_step(*args, L2, *idx)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.equal(interleaved(L2), L1)   # the newest rows written into the same places


@pytest.mark.parametrize("T", [2048, 9000])
def test_precompute_agent_major_values(T):
    case = W.llama_precompute(T=T)
    s = case.shape
    say(f"precompute agent-major T={T}")
    X, A = dev(case.X), dev(stacked_A(case.A))
    V1 = torch.zeros((T, s.n_agents * s.rank), dtype=torch.bfloat16, device="cuda")
    V2 = agent_major(torch.zeros_like(V1), s.n_agents, s.rank, pad=8)
    lra.lra_lr_precompute(X, A, s.n_agents, s.rank, V1)
    lra.lra_lr_precompute(X, A, s.n_agents, s.rank, V2)
    rows = dev_idx(np.arange(T, dtype=np.int64)[::-1].copy(), torch.int64)
    V3 = agent_major(torch.zeros_like(V1), s.n_agents, s.rank)
    lra.lra_lr_precompute(X, A, s.n_agents, s.rank, V3, rows)
    torch.cuda.synchronize()
    assert torch.equal(interleaved(V2), V1)
    assert torch.equal(interleaved(V3), V1.flip(0))


def test_prefill_agent_major_bits():
    s = W.LLAMA_SHAPE
    c = W.random_prefill((962,), s, 700, 300, agent=2)
    say("prefill agent-major")
    L = dev(c.V_lr)
    args = (dev(c.Q), c.L_P, dev(c.K), dev(c.V))
    ref = lra.lra_attn_prefill(*args, L, dev(c.B), c.agent, s.scale)
    got = lra.lra_attn_prefill(*args, agent_major(L, s.n_agents, s.rank, pad=8), dev(c.B), c.agent, s.scale)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_prefill_varlen_agent_major_bits():
    s = W.LLAMA_SHAPE
    c = W.random_prefill_batch((963,), s, [(300, 100, 0), (0, 64, 1), (1000, 200, 2), (50, 1, -1)])
    say("prefill varlen agent-major")
    L = dev(c.V_lr)
    idx = (dev_idx(c.q_start, torch.int64), dev_idx(c.q_len, torch.int32), c.max_q_len, dev(c.K), dev(c.V))
    tail = (dev_idx(c.kv_start, torch.int64), dev_idx(c.kv_prefix, torch.int32), dev(c.B),
            dev_idx(c.agents, torch.int32), s.scale)
    ref = lra.lra_attn_prefill_varlen(dev(c.Q), *idx, L, *tail, O=torch.zeros_like(dev(c.Q)))
    got = lra.lra_attn_prefill_varlen(dev(c.Q), *idx, agent_major(L, s.n_agents, s.rank), *tail,
                                      O=torch.zeros_like(dev(c.Q)))
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_decode_step_agent_major_ministral_layer():
    """One layer of the Ministral step as the benchmark times it (agent-major cache) against the
    interleaved cache: the same outputs and the same newest rows."""
    s = W.MINISTRAL_SHAPE
    say("decode step ministral layer 0 agent-major: generating inputs")
    t = W.ministral_layer_device(0, torch)
    L1 = t["V_lr"]
    L2 = agent_major(L1, s.n_agents, s.rank)
    args = (t["Q"], t["K"], t["V"])
    idx = (dev_idx(t["kv_start"], torch.int64), dev_idx(t["kv_len"], torch.int32), int(t["kv_len"].max()), t["B"],
           dev_idx(t["agent"], torch.int32), s.scale, t["X"], t["A"])
    say("decode step ministral layer 0 agent-major: running")
    ref = lra.lra_attn_decode_step(*args, L1, *idx)
    got = lra.lra_attn_decode_step(*args, L2, *idx)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.equal(interleaved(L2), L1)
