#!/usr/bin/env python3
"""Throughput of the Flash-LoRA-Attention hot path on one MI355X.

Headline (the JSON line's ``value``): decode over 16 requests x 66,400 cached tokens each,
Llama-3.1-8B layer shapes (32 query / 8 KV heads, d_head 128), rank r = 8, 3 agents, bf16;
one step = one lra_attn_decode call over the whole batch. Reported as algorithmic HBM GB/s.

The same run also measures, as extra fields: the causal chunked prefill at L_P = 16,384 +
L_C = 2,048 (TFLOP/s), the LR precompute of 2,048 x 4,096 hidden states (GB/s), decode of one
request at L = 1,900, and the Ministral-8B-shaped 36-layer step (precompute + decode per layer,
32 requests, r = 16). The CPU baseline is the fp64 oracle timed on a bounded sample of the
headline workload on this host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME ...] [--headline-only]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode HBM GB/s & prefill TFLOP/s (frac. of peak) at 1.9k–66.4k ctx, r=8"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 (and fp16) matrix-core peak, TFLOP/s
PROFILE_DIR = os.path.join(ROOT, "profiles")
DECODE_SOURCES = ("rank_kv_cache_amd/csrc/decode.hip", "rank_kv_cache_amd/csrc/lra_device.h")
PREFILL_SOURCES = ("rank_kv_cache_amd/csrc/prefill.hip", "rank_kv_cache_amd/csrc/lra_device.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------------------- algorithmic work
def decode_bytes(kv_len, agents, n_q, n_kv, d, r, elem=2) -> int:
    """K and V_base rows once per request, the agent's r-column V_lr slice, Q and O, and each
    distinct agent's B once."""
    rows = int(sum(int(x) for x in kv_len))
    return (rows * (2 * n_kv * d + r) + len(kv_len) * 2 * n_q * d + len(set(int(a) for a in agents)) * r * n_kv * d) * elem


def precompute_bytes(T, d_model, NR, elem=2) -> int:
    return (T * d_model + NR * d_model + T * NR) * elem


def expand_bytes(rows, n_distinct_agents, n_kv, d, r, elem=2) -> int:
    """HBM bytes of the value expansion: each row reads its V_base row and its agent's r V_lr
    entries and writes the full row; B_a is read once per distinct agent."""
    return rows * (2 * n_kv * d + r) * elem + n_distinct_agents * r * n_kv * d * elem


def prefill_flops(L_P, L_C, n_q, d, r) -> int:
    """Unmasked (query, key) pairs x (4d: QK^T and PV_base, + 2r: PV_lr) per head, plus the
    up-projection O_lr B (2 r d per query row)."""
    pairs = L_C * L_P + L_C * (L_C + 1) // 2
    return pairs * n_q * (4 * d + 2 * r) + L_C * n_q * 2 * r * d


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_fields(name: str, sources) -> dict:
    """The fields of a committed counter summary, or {} when its kernel source has changed since."""
    path = os.path.join(PROFILE_DIR, name)
    if not os.path.exists(path):
        return {}
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    return fields if fields.get("source_sha256") == source_hash(sources) else {}


def counter_traffic(name: str, sources) -> tuple:
    """HBM bytes per launch from a committed counter summary, if it was taken on the current source."""
    path = os.path.join(PROFILE_DIR, name)
    if not os.path.exists(path):
        return None, "no counter summary"
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != source_hash(sources):
        return None, "kernel source changed since the counters were taken"
    try:
        return int(float(fields["hbm_bytes_per_launch"])), os.path.relpath(path, ROOT)
    except (KeyError, ValueError):
        return None, "summary lacks hbm_bytes_per_launch"


# ------------------------------------------------------------------------------- timing helpers
def time_launches(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per call


def time_launches_median(fn, groups, reps, warmup, torch):
    """Median over `groups` timed groups of `reps` back-to-back launches (ms per launch). The clock
    of a compute-bound kernel drifts over a run (power management); the median of the groups is the
    steady-state figure, and the spread is returned beside it."""
    fn_ms = [time_launches(fn, reps, warmup if g == 0 else 2, torch) for g in range(groups)]
    fn_ms.sort()
    return fn_ms[len(fn_ms) // 2], fn_ms[0], fn_ms[-1]


def time_graph(fn, calls, replays, torch):
    """ms per fn() call with `calls` calls captured in one HIP graph and the graph replayed `replays`
    times: the device-side rate of short launches, without the host's per-call cost. Returns None
    if the capture fails (then only the eager figure is reported)."""
    try:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for _ in range(calls):
                    fn()
            g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for _ in range(replays):
                g.replay()
            e1.record(s)
            torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) / (calls * replays)
    except Exception as exc:  # pragma: no cover - reported in the JSON instead
        log(f"[bench] graph capture failed: {exc}")
        return None


# ------------------------------------------------------------------------------- workloads
def upload(t, torch):
    import numpy as np
    if t.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(t.data)).cuda()


def agent_major(L, n_agents: int, rank: int):
    """[rows, N*r] LR cache (agent k in columns k*r .. k*r + r - 1) -> [N, rows, r], each agent's rows
    contiguous: a request then reads whole cache lines of its own agent's values only."""
    return L.view(L.shape[0], n_agents, rank).permute(1, 0, 2).contiguous()


def bench_long_decode(args, torch, lra, W, out):
    log("[bench] decode 16 x 66400: generating inputs")
    c = W.llama_long_decode()
    s = c.shape
    Q, K, V, L, B = (upload(t, torch) for t in (c.Q, c.K, c.V, c.V_lr, c.B))
    ks = torch.as_tensor(c.kv_start, dtype=torch.int64).cuda()
    kl = torch.as_tensor(c.kv_len, dtype=torch.int32).cuda()
    ag = torch.as_tensor(c.agent, dtype=torch.int32).cuda()
    ws = torch.zeros(lra.lra_attn_decode_workspace_bytes(c.batch, s.n_q, s.n_kv, s.d_head, s.rank, c.max_kv_len),
                     dtype=torch.uint8, device="cuda")
    O = torch.empty_like(Q)
    L_am = agent_major(L, s.n_agents, s.rank)

    def step():
        lra.lra_attn_decode(Q, K, V, L_am, ks, kl, c.max_kv_len, B, ag, s.scale, 0, ws, O)

    def step_interleaved():
        lra.lra_attn_decode(Q, K, V, L, ks, kl, c.max_kv_len, B, ag, s.scale, 0, ws, O)

    log(f"[bench] decode 16 x 66400: {args.warmup} warmup + {args.steps} timed steps")
    ms = time_launches(step, args.steps, args.warmup, torch)
    # (not in a counter run of the headline launch alone, which must count one variant)
    ms_i = None if args.headline_only else time_launches(step_interleaved, args.steps, args.warmup, torch)
    nbytes = decode_bytes(c.kv_len, c.agent, s.n_q, s.n_kv, s.d_head, s.rank)
    gbs = nbytes / (ms * 1e-3) / 1e9
    traffic, src = counter_traffic("decode_16x66400_counters.txt", DECODE_SOURCES)
    out["headline"] = {
        "ms_per_step": ms, "gbs": gbs, "bytes": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "lra_attn_decode = decode_split_kernel<bf16,128,8,4,false,false> + decode_combine_kernel<bf16,128,8,4,false>",
                     "bytes_per_launch": nbytes,
                     "traffic_source": src},
        "config": {"workload": W.WORKLOAD_NAMES[W.LLAMA_LONG_DECODE], "batch": c.batch, "kv_len": int(c.kv_len[0]),
                   "n_q": s.n_q, "n_kv": s.n_kv, "d_head": s.d_head, "rank": s.rank, "n_agents": s.n_agents,
                   "keys_per_split": lra.lra_attn_decode_default_split(c.batch, s.n_kv, c.max_kv_len),
                   "lr_cache": "agent-major [n_agents, rows, rank]", "parallelism": "none"},
    }
    out["_long_decode_case"] = c
    if ms_i is not None:
        gbs_i = nbytes / (ms_i * 1e-3) / 1e9
        out["decode_interleaved_lr_cache_llama_b16_L66400"] = {
            "ms": round(ms_i, 4), "gbs": round(gbs_i, 1), "bytes": nbytes, "frac": round(gbs_i / HBM_PEAK_GBS, 4),
            "bound": "hbm", "lr_cache": "interleaved [rows, n_agents*rank] (the same values; bit-identical outputs)"}
    if args.headline_only:   # the headline launch alone (for counter runs that must not mix variants)
        del Q, K, V, L, L_am, B, O, ws
        torch.cuda.empty_cache()
        return

    # double batching: every other request adapter-free (agent -1: K and V_base only, no LR term)
    ag_dual = ag.clone()
    ag_dual[1::2] = -1

    def step_dual():
        lra.lra_attn_decode(Q, K, V, L_am, ks, kl, c.max_kv_len, B, ag_dual, s.scale, 0, ws, O)

    ms_d = time_launches(step_dual, args.steps, args.warmup, torch)
    adapted = [int(a) for a in c.agent[0::2]]
    nbytes_d = (decode_bytes(c.kv_len[0::2], adapted, s.n_q, s.n_kv, s.d_head, s.rank)
                + (int(sum(int(x) for x in c.kv_len[1::2])) * 2 * s.n_kv * s.d_head
                   + len(c.kv_len[1::2]) * 2 * s.n_q * s.d_head) * 2)
    gbs_d = nbytes_d / (ms_d * 1e-3) / 1e9
    out["decode_dual_view_llama_b16_L66400"] = {
        "ms": round(ms_d, 4), "gbs": round(gbs_d, 1), "bytes": nbytes_d, "frac": round(gbs_d / HBM_PEAK_GBS, 4),
        "bound": "hbm", "requests": "8 adapted + 8 adapter-free (agent -1) in one launch"}

    # the same bytes as a paged cache: 32-row pages, the block table a seeded permutation of all pages
    P = 32
    n_pages = K.shape[0] // P
    blocks = int(c.kv_len[0]) // P
    g = torch.Generator(device="cpu")
    g.manual_seed(42)
    table = torch.randperm(n_pages, generator=g).to(torch.int32).reshape(c.batch, blocks).cuda()
    Kp = K.view(n_pages, P, s.n_kv, s.d_head)
    Vp = V.view(n_pages, P, s.n_kv, s.d_head)
    Lp = L.view(n_pages, P, L.shape[1])
    split_p = lra.lra_attn_decode_paged_default_split(c.batch, s.n_kv, c.max_kv_len, P)
    ws_p = torch.zeros(lra.lra_attn_decode_workspace_bytes(c.batch, s.n_q, s.n_kv, s.d_head, s.rank, c.max_kv_len,
                                                           0), dtype=torch.uint8, device="cuda")

    def step_paged():
        lra.lra_attn_decode_paged(Q, Kp, Vp, Lp, table, kl, c.max_kv_len, B, ag, s.scale, 0, ws_p, O)

    log("[bench] paged decode 16 x 66400, 32-row pages")
    ms_p = time_launches(step_paged, args.steps, args.warmup, torch)
    gbs_p = nbytes / (ms_p * 1e-3) / 1e9
    out["decode_paged_llama_b16_L66400_P32"] = {
        "ms": round(ms_p, 4), "gbs": round(gbs_p, 1), "bytes": nbytes, "frac": round(gbs_p / HBM_PEAK_GBS, 4),
        "bound": "hbm", "page_size": P, "n_pages": n_pages, "keys_per_split": split_p,
        "block_table": "seeded permutation of all pages"}
    # the same pages head-major ([n_pages, n_kv, P, d]): each KV head's slice of a page is one run
    Khnd = Kp.transpose(1, 2).contiguous()
    Vhnd = Vp.transpose(1, 2).contiguous()
    Kpv, Vpv = Khnd.transpose(1, 2), Vhnd.transpose(1, 2)

    def step_paged_hnd():
        lra.lra_attn_decode_paged_strided(Q, Kpv, Vpv, Lp, table, kl, c.max_kv_len, B, ag, s.scale, 0, ws_p, O)

    log("[bench] paged decode 16 x 66400, 32-row head-major pages")
    ms_ph = time_launches(step_paged_hnd, args.steps, args.warmup, torch)
    gbs_ph = nbytes / (ms_ph * 1e-3) / 1e9
    out["decode_paged_head_major_llama_b16_L66400_P32"] = {
        "ms": round(ms_ph, 4), "gbs": round(gbs_ph, 1), "bytes": nbytes, "frac": round(gbs_ph / HBM_PEAK_GBS, 4),
        "bound": "hbm", "page_size": P, "layout": "pages [n_pages, n_kv, P, d] (lra_attn_decode_paged_strided)",
        "block_table": "the same seeded permutation"}
    del Khnd, Vhnd, Kpv, Vpv
    # LoRA on the keys as well (qkvo): the key score pass plus the decode; algorithmic bytes add each
    # request's K_lr slice (r values per key) and one read of the rotary table rows (d/2 cos + sin)
    Klr_h, Bk_h, cos_h, sin_h = W.llama_long_decode_key_lora()
    Klr, Bk = upload(Klr_h, torch), upload(Bk_h, torch)
    rc, rs = torch.from_numpy(cos_h).cuda(), torch.from_numpy(sin_h).cuda()
    ws_k = torch.zeros(lra.lra_attn_decode_qkvo_workspace_bytes(c.batch, s.n_q, s.n_kv, s.d_head, s.rank,
                                                                c.max_kv_len, 0), dtype=torch.uint8, device="cuda")

    def step_qkvo():
        lra.lra_attn_decode_qkvo(Q, K, V, L, Klr, ks, kl, c.max_kv_len, B, Bk, rc, rs, ag, s.scale, 0,
                                 ws_k, O)

    log("[bench] decode 16 x 66400 with LoRA on the keys")
    ms_k = time_launches(step_qkvo, args.steps, args.warmup, torch)
    nbytes_k = nbytes + int(sum(int(x) for x in c.kv_len)) * s.rank * 2 + int(c.max_kv_len) * s.d_head * 4
    gbs_k = nbytes_k / (ms_k * 1e-3) / 1e9
    out["decode_qkvo_llama_b16_L66400"] = {
        "ms": round(ms_k, 4), "gbs": round(gbs_k, 1), "bytes": nbytes_k, "frac": round(gbs_k / HBM_PEAK_GBS, 4),
        "bound": "hbm", "keys": "K_base + RoPE(K_lr B_k), rank 8; key score pass + decode"}
    del ws_p, Kp, Vp, Lp, table, Klr, Bk, rc, rs, ws_k

    # expand-then-attend (the order Flash-LoRA-Attention avoids): every request's V_base + V_lr B_a
    # written once at full width, then the same decode kernels with no LR term (agent -1)
    V_exp = torch.empty_like(V)
    none = torch.full((c.batch,), -1, dtype=torch.int32, device="cuda")

    def step_expand():
        lra.lra_expand_values(V, L, B, ks, kl, ag, c.max_kv_len, ks, V_exp)

    def step_expand_attend():
        step_expand()
        lra.lra_attn_decode(Q, K, V_exp, L, ks, kl, c.max_kv_len, B, none, s.scale, 0, ws, O)

    log("[bench] decode 16 x 66400, expand-then-attend")
    ms_x = time_launches(step_expand, args.steps, args.warmup, torch)
    ms_xa = time_launches(step_expand_attend, args.steps, args.warmup, torch)
    rows = int(sum(int(x) for x in c.kv_len))
    nbytes_x = expand_bytes(rows, len(set(int(a) for a in c.agent)), s.n_kv, s.d_head, s.rank)
    out["decode_expand_then_attend_llama_b16_L66400"] = {
        "ms": round(ms_xa, 4), "ms_expand": round(ms_x, 4), "ms_fused_decode": round(ms, 4),
        "fused_speedup": round(ms_xa / ms, 3),
        "expand_gbs": round(nbytes_x / (ms_x * 1e-3) / 1e9, 1), "expand_bytes": nbytes_x,
        "expand_frac": round(nbytes_x / (ms_x * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bound": "hbm",
        "order": "lra_expand_values (V_base + V_lr B_a per request) then lra_attn_decode with agent -1"}
    del V_exp

    # the same cache kept head-major ([n_kv, rows, d]): each split workgroup streams one contiguous
    # range; same bytes, bit-identical outputs (lra_attn_decode_strided)
    Khm = K.transpose(0, 1).contiguous()
    Vhm = V.transpose(0, 1).contiguous()
    Kv, Vv = Khm.transpose(0, 1), Vhm.transpose(0, 1)

    def step_hm():
        lra.lra_attn_decode_strided(Q, Kv, Vv, L, ks, kl, c.max_kv_len, B, ag, s.scale, 0, ws, O)

    log("[bench] decode 16 x 66400, head-major cache")
    ms_h = time_launches(step_hm, args.steps, args.warmup, torch)
    gbs_h = nbytes / (ms_h * 1e-3) / 1e9
    out["decode_head_major_llama_b16_L66400"] = {
        "ms": round(ms_h, 4), "gbs": round(gbs_h, 1), "bytes": nbytes, "frac": round(gbs_h / HBM_PEAK_GBS, 4),
        "bound": "hbm", "layout": "K, V head-major [n_kv, rows, d] (lra_attn_decode_strided)"}
    del Q, K, V, L, B, O, ws, Khm, Vhm, Kv, Vv
    torch.cuda.empty_cache()


def bench_prefill(args, torch, lra, W, out):
    log("[bench] prefill 16384 + 2048: generating inputs")
    cq = W.llama_prefill_qkvo()
    c = cq.base
    s = c.shape
    Q, K, V, L, B = (upload(t, torch) for t in (c.Q, c.K, c.V, c.V_lr, c.B))
    O = torch.empty_like(Q)

    def step():
        lra.lra_attn_prefill(Q, c.L_P, K, V, L, B, 0, s.scale, O)

    # ~20 ms of warm-up launches first: the first launches after the inputs are built run at
    # lower clocks (about 0.75 ms against 0.55-0.6 ms in steady state on MI355X)
    reps = max(10, args.steps // 5)
    ms, ms_lo, ms_hi = time_launches_median(step, 5, reps, 30, torch)
    fl = prefill_flops(c.L_P, c.L_C, s.n_q, s.d_head, s.rank)
    tf = fl / (ms * 1e-3) / 1e12
    out["prefill_llama_LP16384_LC2048_r8"] = {
        "ms": round(ms, 4), "tflops": round(tf, 2), "flops": fl, "peak_tflops": BF16_PEAK_TFLOPS,
        "frac": round(tf / BF16_PEAK_TFLOPS, 4), "bound": "mfma",
        "timing": f"median of 5 groups of {reps} launches (group means {ms_lo:.4f}-{ms_hi:.4f} ms)"}
    # matrix-core counters of the same kernel (committed summary, used only while its source matches)
    mf = counter_fields("prefill_llama_LP16384_LC2048_mfma_counters.txt", PREFILL_SOURCES)
    if mf:
        out["prefill_llama_LP16384_LC2048_r8"]["counters"] = {
            "mfma_util": round(float(mf["mfma_util_percent"]) / 100.0, 4),
            "mfma_flops_per_launch": int(float(mf["mfma_flops_per_launch"])),
            "source": "profiles/prefill_llama_LP16384_LC2048_mfma_counters.txt"}
    if args.oracle_budget > 0:
        # a bounded sample: 64 query rows spread over the chunk, the query group of KV head 0
        import numpy as np
        import oracle
        rows = np.linspace(0, c.L_C - 1, 64).astype(np.int64)
        heads = list(range(s.n_q // s.n_kv))
        f = [t.as_f64() for t in (c.Q, c.K, c.V, c.V_lr, c.B)]
        per, calls, tot = oracle_seconds(lambda: oracle.attn_prefill(*f, c.agent, c.L_P, s.scale, rows=rows, heads=heads),
                                         args.oracle_budget)
        fl_s = sum(int(c.L_P + r + 1) for r in rows) * len(heads) * (4 * s.d_head + 2 * s.rank) \
            + len(rows) * len(heads) * 2 * s.rank * s.d_head
        out["prefill_llama_LP16384_LC2048_r8"]["oracle"] = oracle_entry(
            fl_s / per / 1e12, "TFLOP/s", per, calls, tot,
            f"{len(rows)} of the {c.L_C} query rows x query heads {heads[0]}-{heads[-1]} over their causal keys, "
            "the same per-pair FLOP count as the line; input widening excluded")

    # the same work as four chunk requests of 512 queries in one batched launch (request b: queries
    # 512b .., L_P = 16384 + 512b, all over the same cache rows)
    nreq, lc = 4, c.L_C // 4
    q_start = torch.arange(nreq, dtype=torch.int64, device="cuda") * lc
    q_len = torch.full((nreq,), lc, dtype=torch.int32, device="cuda")
    kv_start = torch.zeros(nreq, dtype=torch.int64, device="cuda")
    kv_prefix = (c.L_P + torch.arange(nreq, device="cuda") * lc).to(torch.int32)
    agents = torch.zeros(nreq, dtype=torch.int32, device="cuda")

    def step_varlen():
        lra.lra_attn_prefill_varlen(Q, q_start, q_len, lc, K, V, L, kv_start, kv_prefix, B, agents, s.scale, O)

    ms_v = time_launches_median(step_varlen, 5, reps, 10, torch)[0]
    tf_v = fl / (ms_v * 1e-3) / 1e12
    out["prefill_varlen_4x512_LP16384"] = {
        "ms": round(ms_v, 4), "tflops": round(tf_v, 2), "flops": fl, "frac": round(tf_v / BF16_PEAK_TFLOPS, 4),
        "bound": "mfma", "requests": "4 chunks of 512 queries, L_P = 16384 + 512 b, one launch"}

    # the same single prefill over a paged cache: 64-row pages, block table a seeded permutation
    P = 64
    n_pages = K.shape[0] // P
    g = torch.Generator(device="cpu")
    g.manual_seed(42)
    table = torch.randperm(n_pages, generator=g).to(torch.int32).reshape(1, n_pages).cuda()
    Kp, Vp, Lp = K.view(n_pages, P, s.n_kv, s.d_head), V.view(n_pages, P, s.n_kv, s.d_head), L.view(n_pages, P, -1)
    one64 = torch.zeros(1, dtype=torch.int64, device="cuda")
    len1 = torch.full((1,), c.L_C, dtype=torch.int32, device="cuda")
    pre1 = torch.full((1,), c.L_P, dtype=torch.int32, device="cuda")
    ag1 = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step_paged():
        lra.lra_attn_prefill_paged(Q, one64, len1, c.L_C, Kp, Vp, Lp, table, pre1, B, ag1, s.scale, O)

    ms_p = time_launches_median(step_paged, 5, reps, 10, torch)[0]
    tf_p = fl / (ms_p * 1e-3) / 1e12
    out["prefill_paged_llama_LP16384_LC2048_P64"] = {
        "ms": round(ms_p, 4), "tflops": round(tf_p, 2), "flops": fl, "frac": round(tf_p / BF16_PEAK_TFLOPS, 4),
        "bound": "mfma", "page_size": P, "n_pages": n_pages, "block_table": "seeded permutation of the pages"}

    # LoRA on the keys as well (qkvo): one pass expands the agent's keys K_base + RoPE(K_lr B_k) into
    # the workspace, then the attention runs over them; the algorithmic work adds one rank-r
    # expansion per cached key and KV head
    Klr, Bk = upload(cq.K_lr, torch), upload(cq.B_k, torch)
    rc, rs = torch.from_numpy(cq.cos).cuda(), torch.from_numpy(cq.sin).cuda()
    ws_k = torch.empty(lra.lra_attn_prefill_qkvo_workspace_bytes(c.L_P + c.L_C, s.n_kv, s.d_head),
                       dtype=torch.uint8, device="cuda")

    def step_qkvo():
        lra.lra_attn_prefill_qkvo(Q, c.L_P, K, V, L, Klr, B, Bk, rc, rs, 0, s.scale, ws_k, O)

    ms_k = time_launches_median(step_qkvo, 5, reps, 10, torch)[0]
    fl_k = fl + 2 * (c.L_P + c.L_C) * s.n_kv * s.d_head * s.rank
    tf_k = fl_k / (ms_k * 1e-3) / 1e12
    out["prefill_qkvo_llama_LP16384_LC2048_r8"] = {
        "ms": round(ms_k, 4), "tflops": round(tf_k, 2), "flops": fl_k, "frac": round(tf_k / BF16_PEAK_TFLOPS, 4),
        "bound": "mfma", "keys": "K_base + RoPE(K_lr B_k), rank 8, expanded once per call (one extra pass)"}
    del Kp, Vp, Lp, table, Klr, Bk, rc, rs, ws_k

    # expand-then-attend: the agent's L_P + L_C value rows written at full width, then the prefill
    # with no LR term (agent -1) over them
    n_rows = c.L_P + c.L_C
    V_exp = torch.empty_like(V)
    one32 = torch.full((1,), n_rows, dtype=torch.int32, device="cuda")

    def step_expand():
        lra.lra_expand_values(V, L, B, one64, one32, ag1, n_rows, one64, V_exp)

    def step_expand_attend():
        step_expand()
        lra.lra_attn_prefill(Q, c.L_P, K, V_exp, L, B, -1, s.scale, O)

    ms_x = time_launches_median(step_expand, 5, reps, 10, torch)[0]
    ms_xa = time_launches_median(step_expand_attend, 5, reps, 10, torch)[0]
    nbytes_x = expand_bytes(n_rows, 1, s.n_kv, s.d_head, s.rank)
    out["prefill_expand_then_attend_llama_LP16384_LC2048"] = {
        "ms": round(ms_xa, 4), "ms_expand": round(ms_x, 4), "ms_fused_prefill": round(ms, 4),
        "fused_speedup": round(ms_xa / ms, 3), "tflops": round(fl / (ms_xa * 1e-3) / 1e12, 2),
        "expand_gbs": round(nbytes_x / (ms_x * 1e-3) / 1e9, 1), "expand_bytes": nbytes_x,
        "order": "lra_expand_values (V_base + V_lr B_0) then lra_attn_prefill with agent -1"}
    del Q, K, V, L, B, O, V_exp
    torch.cuda.empty_cache()


def bench_precompute(args, torch, lra, W, out):
    """X rotates over enough copies (> 256 MB Infinity Cache) that every launch streams X from HBM."""
    case = W.llama_precompute()
    s = case.shape
    n_copies = 40
    X0 = upload(case.X, torch)
    Xs = [X0.clone() for _ in range(n_copies)]
    A = upload(W.HostTensor(case.A.data.T.copy(), case.A.dtype), torch)
    Vlr = torch.zeros((case.X.shape[0], s.n_agents * s.rank), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(lra.lra_lr_precompute_workspace_bytes(case.X.shape[0], s.d_model, s.n_agents, s.rank),
                     dtype=torch.uint8, device="cuda")
    it = [0]

    def step():
        lra.lra_lr_precompute(Xs[it[0] % n_copies], A, s.n_agents, s.rank, Vlr, None, ws)
        it[0] += 1

    ms = time_launches(step, 400, 40, torch)
    ms_g = time_graph(step, n_copies, 10, torch)
    nb = precompute_bytes(case.X.shape[0], s.d_model, s.n_agents * s.rank)
    best = ms_g if ms_g is not None else ms
    gbs = nb / (best * 1e-3) / 1e9
    out["precompute_llama_2048x4096_r8"] = {"us": round(best * 1e3, 2), "gbs": round(gbs, 1), "bytes": nb,
                                           "frac": round(gbs / HBM_PEAK_GBS, 4), "bound": "hbm",
                                           "us_eager": round(ms * 1e3, 2),
                                           "timing": "HIP graph of 40 launches" if ms_g is not None else "eager",
                                           "x_copies_rotated": n_copies}
    # the ceiling at this size: a plain streaming read of the same X copies, timed the same way
    rd = torch.empty(1024, dtype=torch.int32, device="cuda")
    best_rd = None
    for n_wg in (256, 1024):
        kt = [0]

        def step_read():
            lra.lra_stream_read(Xs[kt[0] % n_copies], n_wg, rd)
            kt[0] += 1

        ms_r = time_graph(step_read, n_copies, 10, torch)
        if ms_r is not None and (best_rd is None or ms_r < best_rd[0]):
            best_rd = (ms_r, n_wg)
    if best_rd is not None:
        x_bytes = Xs[0].numel() * Xs[0].element_size()
        gbs_rd = x_bytes / (best_rd[0] * 1e-3) / 1e9
        out["precompute_llama_2048x4096_r8"]["read_ceiling"] = {
            "us": round(best_rd[0] * 1e3, 2), "gbs": round(gbs_rd, 1), "frac": round(gbs_rd / HBM_PEAK_GBS, 4),
            "n_workgroups": best_rd[1], "bytes": x_bytes, "kernel": "lra_stream_read over the same X copies"}
        out["precompute_llama_2048x4096_r8"]["frac_of_read_ceiling"] = round(gbs / gbs_rd, 4)
    if args.oracle_budget > 0:
        import oracle
        Xf, Af = case.X.as_f64(), case.A.as_f64()
        per, calls, tot = oracle_seconds(lambda: oracle.lr_precompute(Xf, Af), args.oracle_budget)
        out["precompute_llama_2048x4096_r8"]["oracle"] = oracle_entry(
            nb / per / 1e9, "GB/s", per, calls, tot, "all 2,048 rows x 24 columns; input widening excluded")
    del Xs, X0, Vlr, ws
    torch.cuda.empty_cache()

    # the prefill's whole context (L_P + L_C = 18,432 rows, 151 MB of X): long enough to stream at
    # the HBM rate; two copies of X alternate (302 MB, beyond the 256 MB Infinity Cache)
    T = 18432
    big = W.llama_precompute(T=T)
    Xb = [upload(big.X, torch) for _ in range(2)]
    Vb = torch.zeros((T, s.n_agents * s.rank), dtype=torch.bfloat16, device="cuda")
    jt = [0]

    def step_big():
        lra.lra_lr_precompute(Xb[jt[0] % 2], A, s.n_agents, s.rank, Vb)
        jt[0] += 1

    ms_b = time_launches(step_big, 40, 4, torch)
    nb_b = precompute_bytes(T, s.d_model, s.n_agents * s.rank)
    gbs_b = nb_b / (ms_b * 1e-3) / 1e9
    # the ceiling at this size: a plain streaming read of the same two copies of X, timed the same way
    rd = torch.empty(2048, dtype=torch.int32, device="cuda")
    best_rd = None
    for n_wg in (256, 512, 1024, 2048):
        kt = [0]

        def step_read():
            lra.lra_stream_read(Xb[kt[0] % 2], n_wg, rd)
            kt[0] += 1

        ms_r = time_launches(step_read, 40, 4, torch)
        if best_rd is None or ms_r < best_rd[0]:
            best_rd = (ms_r, n_wg)
    x_bytes = Xb[0].numel() * Xb[0].element_size()
    gbs_rd = x_bytes / (best_rd[0] * 1e-3) / 1e9
    out["precompute_llama_18432x4096_r8"] = {"us": round(ms_b * 1e3, 2), "gbs": round(gbs_b, 1), "bytes": nb_b,
                                            "frac": round(gbs_b / HBM_PEAK_GBS, 4), "bound": "hbm",
                                            "timing": "eager, two copies of X alternating",
                                            "read_ceiling": {"us": round(best_rd[0] * 1e3, 2), "gbs": round(gbs_rd, 1),
                                                             "frac": round(gbs_rd / HBM_PEAK_GBS, 4),
                                                             "n_workgroups": best_rd[1], "bytes": x_bytes,
                                                             "kernel": "lra_stream_read over the same X copies"},
                                            "frac_of_read_ceiling": round(gbs_b / gbs_rd, 4)}
    if args.oracle_budget > 0:
        import oracle
        Xf, Af = big.X.as_f64()[:4096], big.A.as_f64()
        nb_s = precompute_bytes(4096, s.d_model, s.n_agents * s.rank)
        per, calls, tot = oracle_seconds(lambda: oracle.lr_precompute(Xf, Af), args.oracle_budget)
        out["precompute_llama_18432x4096_r8"]["oracle"] = oracle_entry(
            nb_s / per / 1e9, "GB/s", per, calls, tot, "the first 4,096 of the 18,432 rows; input widening excluded")
    del Xb, Vb, A
    torch.cuda.empty_cache()


def bench_copy(args, torch, lra, W, out):
    """Device-to-device copy of 1 GiB: the achievable streaming bandwidth on this GPU (context for the
    roofline fractions) and the reference kernel that scales the FETCH_SIZE / WRITE_SIZE counters."""
    n = 1 << 29
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    ms = time_launches(lambda: dst.copy_(src), 20, 3, torch)
    nb = 2 * n * 2
    out["copy_1GiB"] = {"ms": round(ms, 4), "gbs": round(nb / (ms * 1e-3) / 1e9, 1), "bytes_read": n * 2,
                        "bytes_written": n * 2}
    del src, dst
    torch.cuda.empty_cache()


def bench_stream_read(args, torch, lra, W, out):
    """The read bandwidth a plain streaming kernel reaches (lra_stream_read over 4 GiB, the size of
    the 16 x 66,400 caches): the practical ceiling of the decode, a read-only stream of the caches.
    The headline's roofline reports its fraction of this figure beside the fraction of the
    published peak."""
    n = 1 << 30
    x = torch.ones(n, dtype=torch.int32, device="cuda")
    best = None
    for n_wg in (256, 2048):
        ms = time_launches(lambda: lra.lra_stream_read(x, n_wg), 20, 3, torch)
        if best is None or ms < best[0]:
            best = (ms, n_wg)
    ms, n_wg = best
    gbs = 4 * n / (ms * 1e-3) / 1e9
    out["stream_read_4GiB"] = {"ms": round(ms, 4), "gbs": round(gbs, 1), "bytes": 4 * n, "n_workgroups": n_wg,
                               "frac": round(gbs / HBM_PEAK_GBS, 4),
                               "kernel": "lra_stream_read (16-byte loads, 8 in flight per lane, 8 waves per workgroup)"}
    head = out.get("headline")
    if head:
        head["roofline"]["practical_peak"] = round(gbs, 1)
        head["roofline"]["frac_of_practical_peak"] = round(head["gbs"] / gbs, 4)
    del x
    torch.cuda.empty_cache()


def bench_short_decode(args, torch, lra, W, out):
    """One request over 1,900 keys (7.8 MB): latency-bound; caches rotate over 64 copies."""
    c = W.llama_decode()
    s = c.shape
    n_copies = 64
    Ks = [upload(c.K, torch) for _ in range(n_copies)]
    Vs = [upload(c.V, torch) for _ in range(n_copies)]
    L, B, Q = upload(c.V_lr, torch), upload(c.B, torch), upload(c.Q, torch)
    ks = torch.as_tensor(c.kv_start, dtype=torch.int64).cuda()
    kl = torch.as_tensor(c.kv_len, dtype=torch.int32).cuda()
    ag = torch.as_tensor(c.agent, dtype=torch.int32).cuda()
    ws = torch.zeros(lra.lra_attn_decode_workspace_bytes(1, s.n_q, s.n_kv, s.d_head, s.rank, c.max_kv_len),
                     dtype=torch.uint8, device="cuda")
    O = torch.empty_like(Q)
    it = [0]

    def step():
        i = it[0] % n_copies
        lra.lra_attn_decode(Q, Ks[i], Vs[i], L, ks, kl, c.max_kv_len, B, ag, s.scale, 0, ws, O)
        it[0] += 1

    ms = time_launches(step, 400, 40, torch)
    ms_g = time_graph(step, n_copies, 10, torch)
    best = ms_g if ms_g is not None else ms
    nb = decode_bytes(c.kv_len, c.agent, s.n_q, s.n_kv, s.d_head, s.rank)
    gbs = nb / (best * 1e-3) / 1e9
    out["decode_llama_b1_L1900_r8"] = {"us": round(best * 1e3, 2), "gbs": round(gbs, 1), "bytes": nb,
                                       "frac": round(gbs / HBM_PEAK_GBS, 4), "bound": "latency (7.8 MB)",
                                       "us_eager": round(ms * 1e3, 2),
                                       "timing": "HIP graph of 64 calls" if ms_g is not None else "eager"}
    # context: one plain streaming read of about the same bytes per call, rotated and timed the same way
    n_rd = 7 << 20   # 7 MiB, a multiple of 16 x 1024
    bufs = [torch.empty(n_rd // 4, dtype=torch.int32, device="cuda") for _ in range(n_copies)]
    rd = torch.empty(1024, dtype=torch.int32, device="cuda")
    best_rd = None
    for n_wg in (128, 256, 1024):
        kt = [0]

        def step_read():
            lra.lra_stream_read(bufs[kt[0] % n_copies], n_wg, rd)
            kt[0] += 1

        t_rd = time_graph(step_read, n_copies, 10, torch)
        if t_rd is not None and (best_rd is None or t_rd < best_rd[0]):
            best_rd = (t_rd, n_wg)
    if best_rd is not None:
        out["decode_llama_b1_L1900_r8"]["read_floor"] = {
            "us": round(best_rd[0] * 1e3, 2), "bytes": n_rd, "n_workgroups": best_rd[1],
            "kernel": "lra_stream_read of 7 MiB in one launch (HIP graph, 64 rotated buffers)"}
    del bufs
    if args.oracle_budget > 0:
        import oracle
        f = [t.as_f64() for t in (c.Q, c.K, c.V, c.V_lr, c.B)]
        per, calls, tot = oracle_seconds(lambda: oracle.attn_decode(*f, c.kv_start, c.kv_len, c.agent, s.scale),
                                         args.oracle_budget)
        out["decode_llama_b1_L1900_r8"]["oracle"] = oracle_entry(
            nb / per / 1e9, "GB/s", per, calls, tot, "the whole 1 x 1,900-key request; input widening excluded")
    del Ks, Vs
    torch.cuda.empty_cache()


def bench_ministral_step(args, torch, lra, W, out):
    """36 layers x (LR precompute of the 32 newest tokens -> decode of 32 requests), per-layer caches,
    timed as one lra_attn_decode_step per layer and, beside it, as lra_lr_precompute + lra_attn_decode.
    Layer caches are drawn on the GPU (workloads.ministral_layer_device, seeded torch generator) to
    keep set-up to seconds; a GPU parity test checks layer 0 of these exact inputs against the
    oracle, and the host streams with identical shapes feed the tests of layers 0, 3 and 35. Each
    layer's LR cache is kept agent-major ([N, rows, r]); the same step over the interleaved cache
    ([rows, N*r], bit-identical outputs) is timed beside it."""
    s = W.MINISTRAL_SHAPE
    lens = W.ministral_lengths()
    agents = W.ministral_agents()
    starts = [0]
    for x in lens[:-1]:
        starts.append(starts[-1] + int(x))
    rows = int(sum(int(x) for x in lens))
    n_layers = W.MINISTRAL_LAYERS
    layers, inter = [], []   # per layer: the inputs with the agent-major LR cache; the interleaved cache
    log(f"[bench] ministral step: drawing {n_layers} layer caches ({rows} rows each) on the GPU")
    for layer in range(n_layers):
        d = W.ministral_layer_device(layer, torch)
        layers.append((d["K"], d["V"], agent_major(d["V_lr"], s.n_agents, s.rank), d["A"], d["B"], d["X"], d["Q"]))
        inter.append(d["V_lr"])
    ks = torch.as_tensor(starts, dtype=torch.int64).cuda()
    kl = torch.as_tensor(lens, dtype=torch.int32).cuda()
    ag = torch.as_tensor(agents, dtype=torch.int32).cuda()
    new_rows = ks + kl.to(torch.int64) - 1
    max_len = int(max(lens))
    ws_dec = torch.zeros(lra.lra_attn_decode_workspace_bytes(len(lens), s.n_q, s.n_kv, s.d_head, s.rank, max_len),
                         dtype=torch.uint8, device="cuda")
    ws_pre = torch.zeros(max(256, lra.lra_lr_precompute_workspace_bytes(len(lens), s.d_model, s.n_agents, s.rank)),
                         dtype=torch.uint8, device="cuda")
    O = torch.empty((len(lens), s.n_q, s.d_head), dtype=torch.bfloat16, device="cuda")

    def step_unfused():
        for (K, V, L, A, B, X, Q) in layers:
            lra.lra_lr_precompute(X, A, s.n_agents, s.rank, L, new_rows, ws_pre)
            lra.lra_attn_decode(Q, K, V, L, ks, kl, max_len, B, ag, s.scale, 0, ws_dec, O)

    # the step as one call per layer: the newest LR rows formed in the decode's own launch
    def step():
        for (K, V, L, A, B, X, Q) in layers:
            lra.lra_attn_decode_step(Q, K, V, L, ks, kl, max_len, B, ag, s.scale, X, A, 0, ws_dec, O)

    def step_interleaved():
        for (K, V, _, A, B, X, Q), L in zip(layers, inter):
            lra.lra_attn_decode_step(Q, K, V, L, ks, kl, max_len, B, ag, s.scale, X, A, 0, ws_dec, O)

    reps = max(3, args.steps // 10)
    ms_u = time_launches(step_unfused, reps, 1, torch)
    ms = time_launches(step, reps, 1, torch)
    ms_g = time_graph(step, 1, reps, torch)
    ms_i = time_launches(step_interleaved, reps, 1, torch)
    # the step is 72 launches of 0.01-0.25 ms: the faster of the graph replay and the eager loop
    graph_best = ms_g is not None and ms_g <= ms
    best = ms_g if graph_best else ms
    nb = n_layers * (decode_bytes(lens, agents, s.n_q, s.n_kv, s.d_head, s.rank)
                     + precompute_bytes(len(lens), s.d_model, s.n_agents * s.rank))
    gbs = nb / (best * 1e-3) / 1e9
    out["ministral_step_36x_b32_r16"] = {"ms": round(best, 3), "gbs": round(gbs, 1), "bytes": nb,
                                         "frac": round(gbs / HBM_PEAK_GBS, 4), "bound": "hbm", "reps": reps,
                                         "ms_eager": round(ms, 3),
                                         "ms_graph": round(ms_g, 3) if ms_g is not None else None,
                                         "timing": "HIP graph of one step" if graph_best else "eager launches",
                                         "call": "lra_attn_decode_step per layer (newest LR rows formed in the decode launch)",
                                         "ms_precompute_then_decode": round(ms_u, 3),
                                         "lr_cache": "agent-major [n_agents, rows, rank] per layer",
                                         "ms_eager_interleaved_lr_cache": round(ms_i, 3),
                                         "kv_rows_per_layer": rows, "min_len": int(min(lens)), "max_len": max_len,
                                         "inputs": "drawn on the GPU (torch generator, seeded per layer)"}
    if args.oracle_budget > 0:
        # a bounded sample of layer 0 of these inputs: the precompute of the 32 newest rows, then whole
        # requests (cycling over the 32) until the budget is spent; bytes as the line counts them
        import numpy as np
        import oracle
        K0, V0, _, A0, B0, X0, Q0 = layers[0]
        L0 = inter[0]   # the same values, [rows, N*r]
        hostf = lambda t: t.float().cpu().numpy().astype(np.float64)
        Xf, Af, Bf, Qf = hostf(X0), hostf(A0).T, hostf(B0), hostf(Q0)
        t0 = time.perf_counter()
        oracle.lr_precompute(Xf, Af)
        t_pre = time.perf_counter() - t0
        t_dec, nbytes_s, done = 0.0, precompute_bytes(len(lens), s.d_model, s.n_agents * s.rank), 0
        while t_dec + t_pre < args.oracle_budget or done == 0:
            b = done % len(lens)
            r0, n = int(starts[b]), int(lens[b])
            Kb, Vb_, Lb = hostf(K0[r0:r0 + n]), hostf(V0[r0:r0 + n]), hostf(L0[r0:r0 + n])
            t0 = time.perf_counter()
            oracle.attn_decode(Qf[b:b + 1], Kb, Vb_, Lb, Bf, [0], [n], [int(agents[b])], s.scale)
            t_dec += time.perf_counter() - t0
            nbytes_s += decode_bytes([n], [int(agents[b])], s.n_q, s.n_kv, s.d_head, s.rank)
            done += 1
        tot = t_pre + t_dec
        out["ministral_step_36x_b32_r16"]["oracle"] = oracle_entry(
            nbytes_s / tot / 1e9, "GB/s", tot, 1, tot,
            f"layer 0: the 32-row precompute and {done} whole requests; copies to the host excluded")

    # the same step with every layer's K and V kept head-major ([n_kv, rows, d]); same values, the
    # decode through lra_attn_decode_strided (bit-identical outputs)
    del inter
    for i, (K, V, L, A, B, X, Q) in enumerate(layers):
        layers[i] = (K.transpose(0, 1).contiguous().transpose(0, 1), V.transpose(0, 1).contiguous().transpose(0, 1),
                     L, A, B, X, Q)
        del K, V
    torch.cuda.empty_cache()

    def step_hm():
        for (K, V, L, A, B, X, Q) in layers:
            lra.lra_lr_precompute(X, A, s.n_agents, s.rank, L, new_rows, ws_pre)
            lra.lra_attn_decode_strided(Q, K, V, L, ks, kl, max_len, B, ag, s.scale, 0, ws_dec, O)

    ms_h = time_launches(step_hm, reps, 1, torch)
    gbs_h = nb / (ms_h * 1e-3) / 1e9
    out["ministral_step_head_major_36x_b32_r16"] = {
        "ms": round(ms_h, 3), "gbs": round(gbs_h, 1), "bytes": nb, "frac": round(gbs_h / HBM_PEAK_GBS, 4),
        "bound": "hbm", "timing": "eager launches",
        "layout": "K, V head-major [n_kv, rows, d] per layer (lra_attn_decode_strided)"}
    del layers
    torch.cuda.empty_cache()


def host_info() -> dict:
    """The host the oracle runs on: cores available to this process, CPU model, NumPy's BLAS."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = {}
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = {"vendor": i.get("internal_api"), "version": i.get("version"),
                        "threads": int(i.get("num_threads", 1))}
                break
    except Exception:  # pragma: no cover
        pass
    return {"host_cores": len(os.sched_getaffinity(0)), "cpu_model": model, "blas": blas}


def oracle_seconds(fn, budget_s: float):
    """Seconds per call of ``fn`` (the oracle as it stands), repeated until about budget_s of work."""
    t_total, calls = 0.0, 0
    while t_total < budget_s or calls == 0:
        t0 = time.perf_counter()
        fn()
        t_total += time.perf_counter() - t0
        calls += 1
    return t_total / calls, calls, t_total


def oracle_entry(value, unit, per_call, calls, total, sample) -> dict:
    return {"value": round(value, 4), "unit": unit, "seconds_per_call": round(per_call, 4), "calls": calls,
            "seconds": round(total, 2), "kind": "oracle", "sample": sample}


def cpu_baseline(case, W, budget_s: float):
    """The fp64 oracle (as it stands) on whole requests of the headline workload, until the budget is used."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    s = case.shape
    t_total, done, nbytes = 0.0, 0, 0
    widened = {}
    # whole requests, cycling over the batch, until the budget of CPU time is spent
    while t_total < budget_s or done == 0:
        b = done % case.batch
        r0, n = int(case.kv_start[b]), int(case.kv_len[b])
        if b not in widened:
            if len(widened) >= 2:
                widened.pop(next(iter(widened)))
            widened[b] = (W.HostTensor(case.K.data[r0:r0 + n], "bf16").as_f64(),
                          W.HostTensor(case.V.data[r0:r0 + n], "bf16").as_f64(),
                          W.HostTensor(case.V_lr.data[r0:r0 + n], "bf16").as_f64())
        K, V, L = widened[b]
        Q = case.Q.as_f64()[b:b + 1]
        t0 = time.perf_counter()
        oracle.attn_decode(Q, K, V, L, case.B.as_f64(), [0], [n], [int(case.agent[b])], s.scale)
        t_total += time.perf_counter() - t0
        done += 1
        nbytes += decode_bytes([n], [int(case.agent[b])], s.n_q, s.n_kv, s.d_head, s.rank)
    info = host_info()
    return {"value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} whole requests (cycling over the {case.batch}) of the 16 x 66,400 decode, fp64 oracle; "
                      f"{t_total:.1f} s of CPU work, input widening excluded",
            "seconds": round(t_total, 2), **info,
            "cores_note": "cores = BLAS threads the oracle used; host_cores = len(os.sched_getaffinity(0))"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", nargs="*", default=None,
                    choices=["decode", "prefill", "precompute", "short", "ministral", "copy", "read", "cpu"])
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--oracle-budget", type=float, default=2.0,
                    help="seconds of oracle work timed beside each other line (0: none)")
    ap.add_argument("--headline-only", action="store_true",
                    help="decode leg: time the headline launch only (no layout or variant lines)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import rank_kv_cache_amd as lra
    import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    only = set(args.only) if args.only is not None else {"decode", "prefill", "precompute", "short", "ministral", "copy",
                                                          "read", "cpu"}
    out = {}
    if "decode" in only or "cpu" in only:
        bench_long_decode(args, torch, lra, W, out)
    for name, fn in (("prefill", bench_prefill), ("precompute", bench_precompute), ("short", bench_short_decode),
                     ("ministral", bench_ministral_step), ("copy", bench_copy), ("read", bench_stream_read)):
        if name in only:
            log(f"[bench] {name}")
            fn(args, torch, lra, W, out)
    cpu = None
    if "cpu" in only:
        log("[bench] CPU baseline (fp64 oracle)")
        cpu = cpu_baseline(out["_long_decode_case"], W, args.cpu_budget)
    head = out.get("headline")
    extra = {k: v for k, v in out.items() if k not in ("headline", "_long_decode_case")}
    line = {
        "metric": METRIC,
        "value": round(head["gbs"], 1) if head else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4) if head else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"] if head else {"workload": "partial run"},
        "roofline": head["roofline"] if head else None,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
