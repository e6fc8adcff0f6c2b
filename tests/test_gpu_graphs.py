"""The calls the benchmark replays from HIP graphs (torch.cuda.CUDAGraph): each replay, with eager work
and synchronisations between replays, gives the eager call's bits (needs an MI355X)."""
import numpy as np
import pytest
import torch

import rank_kv_cache_amd as lra
import workloads as W
from tests.gpu_util import dev, dev_idx, say, stacked_A

pytestmark = pytest.mark.gpu

REPLAYS = 4


def replay_matches(fn, out, scribble):
    """Capture fn (which writes out), replay it REPLAYS times with out overwritten eagerly before
    each replay, and check every replay against the eager result."""
    fn()
    torch.cuda.synchronize()
    ref = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        scribble(i)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"


def test_graph_small_batch_decode():
    """1 x 1,900 keys (the chunked launch and its merge), as the benchmark replays it."""
    c = W.llama_decode(agent=1)
    s = c.shape
    Q, K, V, L, B = dev(c.Q), dev(c.K), dev(c.V), dev(c.V_lr), dev(c.B)
    ks, kl, ag = dev_idx(c.kv_start, torch.int64), dev_idx(c.kv_len, torch.int32), dev_idx(c.agent, torch.int32)
    ws = torch.empty(lra.lra_attn_decode_workspace_bytes(1, s.n_q, s.n_kv, s.d_head, s.rank, c.max_kv_len),
                     dtype=torch.uint8, device="cuda")
    O = torch.empty_like(Q)
    say("graph: decode 1 x 1900")
    replay_matches(lambda: lra.lra_attn_decode(Q, K, V, L, ks, kl, c.max_kv_len, B, ag, s.scale, 0, ws, O), O,
                   lambda i: (O.fill_(float(i)), ws.fill_(0xFF)))


def test_graph_split_decode_and_step():
    """A batch that takes the split launch, and the decode step (newest LR rows formed in the launch),
    each with its workspace overwritten between replays."""
    s = W.MINISTRAL_SHAPE
    lens = [3000, 1954, 4100, 2500, 3333, 2000, 2222, 3900, 2048, 2600]
    c = W.random_decode((140,), s, lens)
    X = dev(W.normal((140, 1), (len(lens), s.d_model), 1.0, s.dtype))
    A = dev(W.normal((140, 2), (s.n_agents * s.rank, s.d_model), 1.0 / 64, s.dtype))
    Q, K, V, B = dev(c.Q), dev(c.K), dev(c.V), dev(c.B)
    L = dev(c.V_lr)
    ks, kl, ag = dev_idx(c.kv_start, torch.int64), dev_idx(c.kv_len, torch.int32), dev_idx(c.agent, torch.int32)
    ws = torch.empty(lra.lra_attn_decode_workspace_bytes(len(lens), s.n_q, s.n_kv, s.d_head, s.rank, c.max_kv_len),
                     dtype=torch.uint8, device="cuda")
    O = torch.empty_like(Q)
    say("graph: split decode")
    replay_matches(lambda: lra.lra_attn_decode(Q, K, V, L, ks, kl, c.max_kv_len, B, ag, s.scale, 0, ws, O), O,
                   lambda i: (O.fill_(float(i)), ws.fill_(i)))
    say("graph: decode step")
    replay_matches(lambda: lra.lra_attn_decode_step(Q, K, V, L, ks, kl, c.max_kv_len, B, ag, s.scale, X, A, 0, ws, O),
                   O, lambda i: (O.fill_(float(i)), ws.fill_(0xFF)))


def test_graph_precompute():
    """2,048 x 4,096 -> 24 (16-column groups) and 4,096 rows (32-column groups)."""
    for T in (2048, 4096):
        case = W.llama_precompute(T=T)
        s = case.shape
        X, A = dev(case.X), dev(stacked_A(case.A))
        V = torch.zeros((T, s.n_agents * s.rank), dtype=torch.bfloat16, device="cuda")
        say(f"graph: precompute T={T}")
        replay_matches(lambda: lra.lra_lr_precompute(X, A, s.n_agents, s.rank, V), V, lambda i: V.fill_(float(i)))
