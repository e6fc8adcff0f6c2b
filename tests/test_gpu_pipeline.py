"""End-to-end chains of the three calls on the GPU against the same chain run by the oracle.

Each side computes its own LR cache rows (GPU: lra_lr_precompute; oracle: lr_precompute), so the
comparison covers the hand-over between the calls as well."""
import numpy as np
import pytest
import torch

import oracle
import rank_kv_cache_amd as lra
import workloads as W
from tests.gpu_util import check, dev, dev_idx, host64, say, stacked_A

pytestmark = pytest.mark.gpu


def test_tiny_fp32_precompute_prefill_and_eight_decode_steps():
    """One layer, 4/2 heads, d=64, r=8, 3 agents: LR precompute of the 256 context tokens, prefill of the
    last 64 (L_P = 192) for every agent, then 8 decode steps, each appending one token (its K/V row and
    its LR row via a one-row precompute) and decoding one query per agent over all keys so far."""
    tw = W.tiny_workload()
    s = tw.shape
    steps = tw.x_dec.shape[0]
    L0 = tw.L_P + tw.L_C
    rows = L0 + steps
    NR = s.n_agents * s.rank

    # ---- GPU chain
    X = dev(tw.X)
    A = dev(stacked_A(tw.A))
    B = dev(tw.B)
    K = torch.zeros((rows, s.n_kv, s.d_head), dtype=torch.float32, device="cuda")
    V = torch.zeros_like(K)
    K[:L0] = dev(tw.K)
    V[:L0] = dev(tw.V)
    Vlr = torch.zeros((rows, NR), dtype=torch.float32, device="cuda")
    say("tiny chain: precompute 256 rows")
    lra.lra_lr_precompute(X, A, s.n_agents, s.rank, Vlr)
    pre_out = []
    for a in range(s.n_agents):
        say(f"tiny chain: prefill agent {a}")
        pre_out.append(host64(lra.lra_attn_prefill(dev(tw.Q), tw.L_P, K, V, Vlr, B, a, s.scale)))
    dec_out = []
    for st in range(steps):
        L = L0 + st + 1
        K[L - 1] = dev(W.HostTensor(tw.K_dec.data[st], "f32"))
        V[L - 1] = dev(W.HostTensor(tw.V_dec.data[st], "f32"))
        say(f"tiny chain: decode step {st}")
        lra.lra_lr_precompute(dev(W.HostTensor(tw.x_dec.data[st:st + 1], "f32")), A, s.n_agents, s.rank, Vlr,
                              dev_idx(np.array([L - 1]), torch.int64))
        O = lra.lra_attn_decode(dev(W.HostTensor(tw.Q_dec.data[st], "f32")), K, V, Vlr,
                                dev_idx(np.zeros(3), torch.int64), dev_idx(np.full(3, L), torch.int32), L, B,
                                dev_idx(np.arange(3), torch.int32), s.scale)
        dec_out.append(host64(O))
    torch.cuda.synchronize()

    # ---- oracle chain
    Kf = np.concatenate([tw.K.as_f64(), tw.K_dec.as_f64()])
    Vf = np.concatenate([tw.V.as_f64(), tw.V_dec.as_f64()])
    lr = oracle.lr_precompute(np.concatenate([tw.X.as_f64(), tw.x_dec.as_f64()]), tw.A.as_f64())
    for a in range(s.n_agents):
        ref = oracle.attn_prefill(tw.Q.as_f64(), Kf[:L0], Vf[:L0], lr[:L0], tw.B.as_f64(), a, tw.L_P, s.scale)
        check(pre_out[a], ref, "f32", f"prefill agent {a}")
    for st in range(steps):
        L = L0 + st + 1
        ref = oracle.attn_decode(tw.Q_dec.as_f64()[st], Kf[:L], Vf[:L], lr[:L], tw.B.as_f64(), [0, 0, 0], [L] * 3,
                                 [0, 1, 2], s.scale)
        check(dec_out[st], ref, "f32", f"decode step {st}")


@pytest.mark.parametrize("layer", [0, 3, 35])
def test_ministral_layer_precompute_then_decode(layer):
    """One layer of the 36-layer step: the precompute writes each request's newest LR row, then the
    decode; every request of the layer against the oracle."""
    say(f"ministral layer {layer}: generating inputs")
    dec, pre = W.ministral_layer(layer)
    s = dec.shape
    rows = dec.kv_start + dec.kv_len.astype(np.int64) - 1
    Vlr = dev(dec.V_lr)
    say(f"ministral layer {layer}: precompute + decode")
    lra.lra_lr_precompute(dev(pre.X), dev(stacked_A(pre.A)), s.n_agents, s.rank, Vlr, dev_idx(rows, torch.int64))
    O = lra.lra_attn_decode(dev(dec.Q), dev(dec.K), dev(dec.V), Vlr, dev_idx(dec.kv_start, torch.int64),
                            dev_idx(dec.kv_len, torch.int32), dec.max_kv_len, dev(dec.B),
                            dev_idx(dec.agent, torch.int32), s.scale)
    got = host64(O)
    lr_ref = oracle.lr_precompute(pre.X.as_f64(), pre.A.as_f64())
    for b in range(dec.batch):
        say(f"ministral layer {layer}: oracle request {b}")
        r0, n = int(dec.kv_start[b]), int(dec.kv_len[b])
        Vlr_b = W.HostTensor(dec.V_lr.data[r0:r0 + n], "bf16").as_f64()
        Vlr_b[-1, :] = lr_ref[b]
        ref = oracle.attn_decode(dec.Q.as_f64()[b:b + 1], W.HostTensor(dec.K.data[r0:r0 + n], "bf16").as_f64(),
                                 W.HostTensor(dec.V.data[r0:r0 + n], "bf16").as_f64(), Vlr_b, dec.B.as_f64(),
                                 [0], [n], [int(dec.agent[b])], s.scale)
        check(got[b:b + 1], ref, "bf16", f"layer {layer} request {b}")


def _host(t: torch.Tensor) -> W.HostTensor:
    """A device bf16 tensor as the host bit pattern (the oracle reads the stored values)."""
    return W.HostTensor(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16), "bf16")


def test_ministral_bench_layer_all_requests():
    """Layer 0 of the benchmark's 36-layer step, with the exact inputs the benchmark times (drawn on
    the GPU by workloads.ministral_layer_device): the precompute of the 32 newest LR rows, then the
    decode of all 32 requests in the benchmark's launch configuration, every output against the
    oracle (precompute in fp64, then the decode over the oracle's own new rows)."""
    s = W.MINISTRAL_SHAPE
    say("ministral bench layer 0: drawing inputs on the GPU")
    d = W.ministral_layer_device(0, torch)
    starts, lens, agents = d["kv_start"], d["kv_len"], d["agent"]
    new_rows = starts + lens.astype(np.int64) - 1
    host = {k: _host(d[k]) for k in ("K", "V", "V_lr", "A", "B", "X", "Q")}   # before the precompute writes
    Vlr = d["V_lr"].clone()
    say("ministral bench layer 0: precompute + decode")
    lra.lra_lr_precompute(d["X"], d["A"], s.n_agents, s.rank, Vlr, dev_idx(new_rows, torch.int64))
    O = lra.lra_attn_decode(d["Q"], d["K"], d["V"], Vlr, dev_idx(starts, torch.int64), dev_idx(lens, torch.int32),
                            int(lens.max()), d["B"], dev_idx(agents, torch.int32), s.scale, 0)
    got = host64(O)
    got_rows = host64(Vlr[torch.as_tensor(new_rows, device="cuda")])
    # the pages' A_k side by side is the transpose of the stacked LoRA weights
    lr_ref = oracle.lr_precompute(host["X"].as_f64(), host["A"].as_f64().T)
    check(got_rows, lr_ref, "bf16", "newest LR rows")
    B64, Q64 = host["B"].as_f64(), host["Q"].as_f64()
    for b in range(len(lens)):
        r0, n = int(starts[b]), int(lens[b])
        say(f"ministral bench layer 0: oracle request {b} (L={n})")
        Vlr_b = W.HostTensor(host["V_lr"].data[r0:r0 + n], "bf16").as_f64()
        Vlr_b[-1, :] = lr_ref[b]
        ref = oracle.attn_decode(Q64[b:b + 1], W.HostTensor(host["K"].data[r0:r0 + n], "bf16").as_f64(),
                                 W.HostTensor(host["V"].data[r0:r0 + n], "bf16").as_f64(), Vlr_b, B64,
                                 [0], [n], [int(agents[b])], s.scale)
        check(got[b:b + 1], ref, "bf16", f"request {b}")
