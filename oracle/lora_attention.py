"""fp64 definition of LR precompute, the per-agent value cache and causal GQA attention.

TEST INFRASTRUCTURE ONLY (see the package docstring). Every array is widened
to float64 on entry; results are float64.

Notation (LRAgent page, "prerequisites" and "core method"; PReCache summary
page, "how it works"):
  X        hidden states, one row per token             [T, d_model]
  W0       frozen projection of the backbone
  A_k, B_k LoRA down / up projection of agent k, A_k: d_model x r, B_k: r x d_out
  V_base = X W0          the base value cache, shared by all agents
  V_lr   = X A_k         the agent's rank-r value cache (L x r)
  V_k    = V_base + V_lr B_k   the agent's full value cache (never built by the GPU path)
Keys carry no low-rank part (LoRA on the query and value projections only:
PReCache summary page, "setup and results"), so K_base is the key cache of
every agent.

Readings where the pages are silent (each is also listed in the design notes):
  * scale is passed in; the workloads use 1/sqrt(d_head) (FlashAttention's
    convention; the pages state no scale).
  * query head h reads KV head floor(h / G), G = n_q / n_kv (contiguous GQA
    groups, the Llama convention; the pages name Llama/Ministral models).
  * V_lr holds all agents side by side: agent k owns columns k*r .. k*r+r-1
    (PReCache: every agent's down-projection is applied to the same hidden
    states in one pass, so their outputs sit in one row per token).
  * B_k is r x (n_kv * d_head); KV head g uses its columns g*d .. g*d+d-1.
  * no LoRA scaling factor (alpha / r) appears on the pages: B_k is used as given.
  * causal mask is bottom-right aligned: query i of a chunk of L_C new tokens
    sits at absolute position L_P + i and sees keys 0 .. L_P + i. A decode
    query sits at the last position of its range and sees all kv_len keys.
  * a query with no visible key (kv_len = 0) returns zeros.
  * agent = -1 (ADAPTER_FREE) is the adapter-free view of double batching
    (PReCache paper page, section 3, ReBaseShared: the adapter-free path runs
    beside the adapted one over the same tokens and attends only to the
    neutral base cache). Its values are V_base; V_lr and B are not read.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------- a1: LR precompute
def lr_precompute(X, A) -> np.ndarray:
    """All agents' rank-r caches in one product: ``X [A_1 .. A_N]``.

    PReCache page, PreLRShared subsection: when a segment is first processed,
    every agent's down-projection is applied to its hidden states. LRAgent
    page, "method steps" step (2): ``V_lr = X A`` is stored with shape L x r.
    X: [T, d_model]; A: [d_model, N*r] (agent k = column block k). Returns [T, N*r].
    """
    return _f64(X) @ _f64(A)


def lr_precompute_into(V_lr, X, A, out_rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Return a copy of the cache ``V_lr`` [rows, ld] whose rows ``out_rows[t]`` (default t)
    hold row t of ``lr_precompute(X, A)`` in columns 0 .. N*r-1; every other entry is unchanged."""
    res = _f64(V_lr).copy()
    new = lr_precompute(X, A)
    rows = np.arange(new.shape[0]) if out_rows is None else np.asarray(out_rows, dtype=np.int64)
    res[rows, : new.shape[1]] = new
    return res


# --------------------------------------------------------------------------- layout maps
def kv_head_of(h: int, group: int) -> int:
    """KV head read by query head h: contiguous groups of ``group`` query heads share one KV head."""
    return h // group


def agent_columns(agent: int, rank: int) -> slice:
    """Columns of the stacked LR cache owned by ``agent``."""
    return slice(agent * rank, (agent + 1) * rank)


ADAPTER_FREE = -1


# --------------------------------------------------------------------------- V_k materialised
def agent_values(V_base, V_lr, B, agent: int) -> np.ndarray:
    """The agent's full value cache ``V_base + V_lr[:, agent cols] B_agent``, built explicitly.

    LRAgent page, "core method": the adapted value projection splits into the
    shared ``X W0`` and the agent's ``(X A_i) B_i``; the LR cache keeps
    ``X A_i`` and B_i restores the full width on demand.
    V_base: [L, n_kv, d]; V_lr: [L, >= N*r]; B: [N, r, n_kv*d]. Returns [L, n_kv, d].
    agent = ADAPTER_FREE gives the neutral base cache itself (PReCache paper page, section 3,
    double batching: the adapter-free path attends to the base cache only).
    """
    V_base = _f64(V_base)
    if agent == ADAPTER_FREE:
        return V_base.copy()
    B = _f64(B)
    L, n_kv, d = V_base.shape
    rank = B.shape[1]
    lr = _f64(V_lr)[:, agent_columns(agent, rank)] @ B[agent]  # [L, n_kv*d]
    return V_base + lr.reshape(L, n_kv, d)


def expand_values(V_out, V_base, V_lr, B, src_start, length, agents, dst_start) -> np.ndarray:
    """Expand-then-attend's first pass over a batch of requests (the order the LRAgent page's
    Flash-LoRA-Attention avoids): request b's full value rows ``agent_values`` of source rows
    src_start[b] .. src_start[b]+length[b]-1 land in rows dst_start[b] .. of a copy of ``V_out``.
    Rows no request names keep their values. Attending these rows with no LR term gives the same
    result as attention with the LR term deferred (associativity, LRAgent page, core method).
    V_out, V_base: [rows, n_kv, d]; V_lr: [rows, >= N*r]; B: [N, r, n_kv*d]. Returns float64.
    """
    out = _f64(V_out).copy()
    for b in range(len(length)):
        n = int(length[b])
        if n <= 0:
            continue
        s0, d0 = int(src_start[b]), int(dst_start[b])
        out[d0:d0 + n] = agent_values(V_base[s0:s0 + n], V_lr[s0:s0 + n], B, int(agents[b]))
    return out


# --------------------------------------------------------------------------- mask + softmax
def visible(q_pos: Iterable[int], L: int) -> np.ndarray:
    """Causal visibility [len(q_pos), L]: key j is visible to a query at absolute position p iff j <= p."""
    q_pos = np.asarray(list(q_pos) if not isinstance(q_pos, np.ndarray) else q_pos, dtype=np.int64)
    return np.arange(L, dtype=np.int64)[None, :] <= q_pos[:, None]


def softmax_rows(S, mask) -> np.ndarray:
    """Two-pass softmax of each row of S over its visible entries (fp64).

    Pass 1 takes the row maximum over visible entries, pass 2 exponentiates the
    shifted scores and divides by their sum. Masked entries are exactly 0; a
    row with no visible entry is all zeros.
    """
    S = _f64(S)
    mask = np.asarray(mask, dtype=bool)
    Sm = np.where(mask, S, -np.inf)
    m = Sm.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    E = np.where(mask, np.exp(Sm - m), 0.0)
    l = E.sum(axis=-1, keepdims=True)
    return np.divide(E, l, out=np.zeros_like(E), where=l > 0)


def attention_probs(Q, K, q_pos, scale: float, heads: Optional[Sequence[int]] = None) -> np.ndarray:
    """Softmax probabilities P [len(heads), Lq, L] of scaled dot-product scores under the causal mask.

    Q: [Lq, n_q, d] queries at absolute positions q_pos; K: [L, n_kv, d].
    Score of query i, head h, key j: ``scale * <Q[i, h], K[j, kv_head_of(h)]>``.
    """
    Q = _f64(Q)
    K = _f64(K)
    Lq, n_q, d = Q.shape
    L, n_kv, _ = K.shape
    G = n_q // n_kv
    heads = range(n_q) if heads is None else heads
    mask = visible(q_pos, L)
    out = []
    for h in heads:
        g = kv_head_of(h, G)
        S = scale * (Q[:, h, :] @ K[:, g, :].T)
        out.append(softmax_rows(S, mask))
    return np.stack(out) if out else np.zeros((0, Lq, L))


def attention(Q, K, Vfull, q_pos, scale: float, heads: Optional[Sequence[int]] = None) -> np.ndarray:
    """O[i, h] = sum_j P[h, i, j] * Vfull[j, kv_head_of(h)]  with P from ``attention_probs``.

    Returns [Lq, len(heads), d]."""
    Q = _f64(Q)
    Vfull = _f64(Vfull)
    n_q = Q.shape[1]
    G = n_q // Vfull.shape[1]
    heads = list(range(n_q)) if heads is None else list(heads)
    P = attention_probs(Q, K, q_pos, scale, heads)
    O = np.empty((Q.shape[0], len(heads), Vfull.shape[2]))
    for t, h in enumerate(heads):
        O[:, t, :] = P[t] @ Vfull[:, kv_head_of(h, G), :]
    return O


# --------------------------------------------------------------------------- the three calls
def attn_prefill(Q, K_base, V_base, V_lr, B, agent: int, L_P: int, scale: float,
                 rows: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None) -> np.ndarray:
    """Causal chunked prefill for one agent: L_C new queries over the L_P + L_C keys.

    LRAgent page, "method steps" (3)-(4): attention over the shared key cache
    and the agent's value cache; here the value cache is materialised.
    PReCache summary page: the new chunk L_C follows the reused context L_P.
    Q: [L_C, n_q, d]; K_base, V_base: [>= L_P+L_C, n_kv, d]; V_lr: [>= L_P+L_C, >= N*r];
    B: [N, r, n_kv*d]. ``rows``/``heads`` restrict the output to some query rows / heads.
    Returns [len(rows), len(heads), d].
    """
    Q = _f64(Q)
    L_C = Q.shape[0]
    L = L_P + L_C
    rows = np.arange(L_C) if rows is None else np.asarray(rows, dtype=np.int64)
    Va = agent_values(_f64(V_base)[:L], _f64(V_lr)[:L], B, agent)
    return attention(Q[rows], _f64(K_base)[:L], Va, L_P + rows, scale, heads)


def rope_rotate(Y, cos, sin) -> np.ndarray:
    """Rotary position embedding of rows Y [L, ..., d] at positions 0 .. L-1, rotate-half pairing:
    element i pairs with i + d/2 and turns by the angle whose cosine / sine are cos[p, i] / sin[p, i]
    (tables [>= L, d/2], given by the caller). Llama's convention; the pages name RoPE as the reason
    the key-side LR expansion cannot be reordered, without fixing its form."""
    Y = _f64(Y)
    L, d = Y.shape[0], Y.shape[-1]
    h = d // 2
    c = _f64(cos)[:L]
    s_ = _f64(sin)[:L]
    shape = (L,) + (1,) * (Y.ndim - 2) + (h,)
    c, s_ = c.reshape(shape), s_.reshape(shape)
    lo, hi = Y[..., :h], Y[..., h:]
    return np.concatenate([lo * c - hi * s_, hi * c + lo * s_], axis=-1)


def agent_keys(K_base, K_lr, B_k, agent: int, cos, sin) -> np.ndarray:
    """The agent's full key cache when LoRA also adapts the key projection (the qkvo configuration):
    ``K_base + RoPE(K_lr[:, agent cols] B_k[agent])``. K_base is stored after RoPE; the rank-r part
    is expanded and then rotated at each row's position, which is why it cannot be moved out of
    the key loop (LRAgent page, limitations; PReCache summary page, the QV default).
    K_base: [L, n_kv, d]; K_lr: [L, >= N*r]; B_k: [N, r, n_kv*d]. Returns [L, n_kv, d]."""
    K_base = _f64(K_base)
    if agent == ADAPTER_FREE:
        return K_base.copy()
    B_k = _f64(B_k)
    L, n_kv, d = K_base.shape
    rank = B_k.shape[1]
    lr = (_f64(K_lr)[:, agent_columns(agent, rank)] @ B_k[agent]).reshape(L, n_kv, d)
    return K_base + rope_rotate(lr, cos, sin)


def attn_prefill_qkvo(Q, K_base, V_base, V_lr, K_lr, B, B_k, cos, sin, agent: int, L_P: int,
                      scale: float, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """``attn_prefill`` with LoRA on the keys as well: the agent's keys are ``agent_keys``.
    ``rows`` restricts the output to some query rows."""
    Q = _f64(Q)
    L_C = Q.shape[0]
    L = L_P + L_C
    rows = np.arange(L_C) if rows is None else np.asarray(rows, dtype=np.int64)
    Ka = agent_keys(_f64(K_base)[:L], _f64(K_lr)[:L], B_k, agent, cos, sin)
    Va = agent_values(_f64(V_base)[:L], _f64(V_lr)[:L], B, agent)
    return attention(Q[rows], Ka, Va, L_P + rows, scale)


def attn_prefill_varlen(Q, K_base, V_base, V_lr, B, q_start, q_len, kv_start, kv_prefix, agents,
                        scale: float) -> np.ndarray:
    """Several causal chunked prefills in one batch: request b's q_len[b] queries are rows
    q_start[b] .. of Q, its cache rows start at kv_start[b], it has kv_prefix[b] cached tokens
    (L_P) before its chunk, and it attends with agent agents[b] (ADAPTER_FREE for the base view).

    Each request is ``attn_prefill`` on its own rows (PReCache summary page: a new chunk L_C
    follows the reused context L_P; requests are batched for concurrent serving). Returns an
    array shaped like Q holding every request's output rows; rows of Q that no request covers
    are zero.
    """
    Q = _f64(Q)
    out = np.zeros_like(Q)
    for b in range(len(q_len)):
        n = int(q_len[b])
        if n == 0:
            continue
        q0, k0, lp = int(q_start[b]), int(kv_start[b]), int(kv_prefix[b])
        L = lp + n
        out[q0:q0 + n] = attn_prefill(Q[q0:q0 + n], _f64(K_base[k0:k0 + L]), _f64(V_base[k0:k0 + L]),
                                      _f64(V_lr[k0:k0 + L]), B, int(agents[b]), lp, scale)
    return out


def attn_prefill_paged(Q, K_pages, V_pages, Vlr_pages, B, block_table, q_start, q_len, kv_prefix, agents,
                       scale: float) -> np.ndarray:
    """``attn_prefill_varlen`` over a paged cache: request b's cache rows 0 .. kv_prefix[b]+q_len[b]-1
    are gathered from the pages its block-table row names (``gather_pages``)."""
    Q = _f64(Q)
    out = np.zeros_like(Q)
    for b in range(len(q_len)):
        n = int(q_len[b])
        if n == 0:
            continue
        q0, lp = int(q_start[b]), int(kv_prefix[b])
        L = lp + n
        K = gather_pages(K_pages, block_table[b], L)
        V = gather_pages(V_pages, block_table[b], L)
        Vl = gather_pages(Vlr_pages, block_table[b], L)
        out[q0:q0 + n] = attn_prefill(Q[q0:q0 + n], K, V, Vl, B, int(agents[b]), lp, scale)
    return out


def attn_decode(Q, K_base, V_base, V_lr, B, kv_start, kv_len, agents, scale: float,
                requests: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None) -> np.ndarray:
    """One new query per request over its key range [kv_start[b], kv_start[b] + kv_len[b]).

    The query is the newest token of its range, so every key of the range is
    visible. Requests may share rows (agents share the base cache: PReCache
    page, PreLRShared; LRAgent page, "core method"). kv_len[b] = 0 gives zeros.
    Q: [batch, n_q, d]. Returns [len(requests), len(heads), d].
    """
    Q = _f64(Q)
    n_q, d = Q.shape[1], Q.shape[2]
    requests = range(Q.shape[0]) if requests is None else requests
    heads = list(range(n_q)) if heads is None else list(heads)
    out = []
    for b in requests:
        n = int(kv_len[b])
        if n == 0:
            out.append(np.zeros((len(heads), d)))
            continue
        r0 = int(kv_start[b])
        K = _f64(K_base[r0:r0 + n])
        Va = agent_values(V_base[r0:r0 + n], V_lr[r0:r0 + n], B, int(agents[b]))
        out.append(attention(Q[b:b + 1], K, Va, [n - 1], scale, heads)[0])
    return np.stack(out) if out else np.zeros((0, len(heads), d))


def attn_decode_qkvo(Q, K_base, V_base, V_lr, K_lr, B, B_k, cos, sin, kv_start, kv_len, agents,
                     scale: float, requests: Optional[Sequence[int]] = None) -> np.ndarray:
    """``attn_decode`` with LoRA on the keys as well: request b's keys are ``agent_keys`` of its rows,
    the row kv_start[b] + j sitting at position j (rows 0 .. of the tables cos / sin)."""
    Q = _f64(Q)
    n_q, d = Q.shape[1], Q.shape[2]
    requests = range(Q.shape[0]) if requests is None else requests
    out = []
    for b in requests:
        n = int(kv_len[b])
        if n == 0:
            out.append(np.zeros((n_q, d)))
            continue
        r0 = int(kv_start[b])
        Ka = agent_keys(_f64(K_base[r0:r0 + n]), _f64(K_lr[r0:r0 + n]), B_k, int(agents[b]), cos, sin)
        Va = agent_values(V_base[r0:r0 + n], V_lr[r0:r0 + n], B, int(agents[b]))
        out.append(attention(Q[b:b + 1], Ka, Va, [n - 1], scale)[0])
    return np.stack(out) if out else np.zeros((0, n_q, d))


def gather_pages(pages, block_table_row, n_rows: int) -> np.ndarray:
    """Logical rows 0 .. n_rows-1 of a paged cache: row j lives in page block_table_row[j // P] at
    offset j % P (pages: [n_pages, P, ...]). The layout of concurrent serving (the pages' vLLM
    deployments), written out as a plain gather."""
    pages = np.asarray(pages)
    P = pages.shape[1]
    idx = np.arange(n_rows)
    return pages[np.asarray(block_table_row, np.int64)[idx // P], idx % P]


def attn_decode_paged(Q, K_pages, V_pages, Vlr_pages, B, block_table, kv_len, agents, scale: float,
                      requests: Optional[Sequence[int]] = None) -> np.ndarray:
    """``attn_decode`` over a paged cache: request b's rows 0 .. kv_len[b]-1 are gathered from the
    pages its block-table row names, then attended as one contiguous range."""
    Q = _f64(Q)
    requests = range(Q.shape[0]) if requests is None else requests
    out = []
    for b in requests:
        n = int(kv_len[b])
        K = _f64(gather_pages(K_pages, block_table[b], n))
        V = _f64(gather_pages(V_pages, block_table[b], n))
        L = _f64(gather_pages(Vlr_pages, block_table[b], n))
        out.append(attn_decode(Q[b:b + 1], K, V, L, B, [0], [n], [agents[b]], scale)[0])
    return np.stack(out) if out else np.zeros((0,) + Q.shape[1:])


def attn_factored(Q, K, V_base, V_lr, B, agent: int, q_pos, scale: float) -> np.ndarray:
    """Attend-then-expand: ``P V_base + (P V_lr[:, agent cols]) B_agent`` per head.

    LRAgent page, "core method" and "technical novelty": by associativity the
    LR cache is attended in rank space and expanded by B once per query row,
    instead of expanding every cached row first. Equal to ``attention`` over
    ``agent_values`` in exact arithmetic; kept here so that identity can be
    tested. The adapter-free view (agent = ADAPTER_FREE) has no LR term.
    Returns [Lq, n_q, d].
    """
    Q = _f64(Q)
    V_base = _f64(V_base)
    B = _f64(B)
    Lq, n_q, d = Q.shape
    L, n_kv, _ = V_base.shape
    rank = B.shape[1]
    G = n_q // n_kv
    P = attention_probs(Q, K, q_pos, scale)
    lr = _f64(V_lr)[:L, agent_columns(agent, rank)]
    O = np.empty((Lq, n_q, d))
    for h in range(n_q):
        g = kv_head_of(h, G)
        O[:, h, :] = P[h] @ V_base[:, g, :]
        if agent != ADAPTER_FREE:
            O[:, h, :] += (P[h] @ lr) @ B[agent][:, g * d:(g + 1) * d]
    return O
