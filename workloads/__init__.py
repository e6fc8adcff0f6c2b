"""Seeded synthetic inputs for the Flash-LoRA-Attention workloads.

This module only draws random tensors of the right shapes, distributions and
storage dtype. It holds none of the attention or LoRA arithmetic: both the
fp64 CPU oracle (``oracle/``) and the HIP path consume what it produces, and
neither imports the other.

Sources of the shapes (LRAgent and PReCache pages):
  * LoRA on the query and value projections with rank r = 8; keys carry no
    low-rank part (PReCache summary page, "setup and results" paragraph;
    LRAgent page, "reproducibility" section). The qkvo cases add a key-side
    rank-r cache and its up-projection, with standard rotary angle tables.
  * Three role agents (plan / action / reflect) share one trajectory
    (PReCache page, section 4.1 agent setup).
  * Trajectories from 1.9k to 66.4k tokens (PReCache summary page, results).
  * LLaMA-3.1-8B / Ministral-8B layer shapes: 32 query heads, 8 KV heads,
    d_head = 128, d_model = 4096 (public model cards; the pages name the models).
  * Root seed 42, the seed the LRAgent page reports for its experiments.

Random streams: one PCG64 stream per (workload, layer, request, tensor, block)
via ``SeedSequence(42, spawn_key=...)``. Large tensors are drawn in fixed row
blocks, each with its own stream, so the values do not depend on how many
threads draw them. Normals are drawn in float32, multiplied by the standard
deviation in float32, then rounded to the storage dtype (bf16 by
round-to-nearest-even on the bit pattern).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

ROOT_SEED = 42

# Workload ids used in spawn keys (stable; never renumber).
TINY, LLAMA_DECODE, LLAMA_PREFILL, LLAMA_LONG_DECODE, MINISTRAL_STEP = 0, 1, 2, 3, 4
WORKLOAD_NAMES = {
    TINY: "tiny_fp32",
    LLAMA_DECODE: "llama31_8b_decode_b1_L1900_r8",
    LLAMA_PREFILL: "llama31_8b_prefill_LP16384_LC2048_r8",
    LLAMA_LONG_DECODE: "llama31_8b_decode_b16_L66400_r8",
    MINISTRAL_STEP: "ministral_8b_step_36x_b32_L1.9k-32k_r16",
}

# Tensor ids used in spawn keys.
T_X, T_W0K, T_W0V, T_A, T_B, T_Q, T_K, T_V, T_VLR, T_AGENT, T_LEN, T_XDEC, T_QDEC, T_KLR, T_BK = range(15)

_BLOCK_ROWS = 4096  # rows per independently seeded block of a large tensor


# --------------------------------------------------------------------------- dtype helpers
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits.

    NaN inputs stay NaN (quiet bit forced)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class HostTensor:
    """A host tensor in its storage dtype. ``data`` is float32, or uint16 bf16 bits."""
    data: np.ndarray
    dtype: str  # "f32" or "bf16"

    @property
    def shape(self) -> Tuple[int, ...]:
        return tuple(self.data.shape)

    def as_f64(self) -> np.ndarray:
        """Exact widening of the stored values to float64 (what the oracle consumes)."""
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.data).astype(np.float64)
        return self.data.astype(np.float64)

    def as_f32(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.data)
        return np.asarray(self.data, dtype=np.float32)


def to_storage(x32: np.ndarray, dtype: str) -> HostTensor:
    if dtype == "bf16":
        return HostTensor(f32_to_bf16_bits(x32), "bf16")
    if dtype == "f32":
        return HostTensor(np.ascontiguousarray(x32, dtype=np.float32), "f32")
    raise ValueError(dtype)


# --------------------------------------------------------------------------- random streams
def rng(*key: int) -> np.random.Generator:
    """Independent PCG64 stream for a spawn key (workload, layer, request, tensor, ...)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(ROOT_SEED, spawn_key=tuple(int(k) for k in key))))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal(key: Sequence[int], shape: Tuple[int, ...], std: float, dtype: str) -> HostTensor:
    """N(0, std^2) tensor, drawn in row blocks of ``_BLOCK_ROWS`` (block b uses key + (b,))."""
    shape = tuple(int(s) for s in shape)
    rows = shape[0] if shape else 1
    inner = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    nblk = max(1, math.ceil(rows / _BLOCK_ROWS))
    out_dtype = np.uint16 if dtype == "bf16" else np.float32
    out = np.empty((rows, inner), dtype=out_dtype)

    def fill(b: int) -> None:
        r0 = b * _BLOCK_ROWS
        r1 = min(rows, r0 + _BLOCK_ROWS)
        g = rng(*key, b)
        x = g.standard_normal((r1 - r0) * inner, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        x = x.reshape(r1 - r0, inner)
        out[r0:r1] = f32_to_bf16_bits(x) if dtype == "bf16" else x

    if nblk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return HostTensor(out.reshape(shape), dtype)


def fill_rows(t: HostTensor, rows: np.ndarray, value: float) -> None:
    """Overwrite whole rows (first axis) of a host tensor with ``value`` in its storage dtype."""
    v = np.full(t.data.shape[1:], value, dtype=np.float32)
    t.data[rows] = f32_to_bf16_bits(v) if t.dtype == "bf16" else v


# --------------------------------------------------------------------------- workload shapes
@dataclass(frozen=True)
class Shape:
    n_q: int
    n_kv: int
    d_head: int
    rank: int
    n_agents: int
    d_model: int
    dtype: str

    @property
    def group(self) -> int:
        return self.n_q // self.n_kv

    @property
    def d_kv(self) -> int:
        return self.n_kv * self.d_head

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_head)


TINY_SHAPE = Shape(n_q=4, n_kv=2, d_head=64, rank=8, n_agents=3, d_model=256, dtype="f32")
LLAMA_SHAPE = Shape(n_q=32, n_kv=8, d_head=128, rank=8, n_agents=3, d_model=4096, dtype="bf16")
MINISTRAL_SHAPE = Shape(n_q=32, n_kv=8, d_head=128, rank=16, n_agents=3, d_model=4096, dtype="bf16")


@dataclass
class DecodeBatch:
    """Inputs of one decode call: a packed key/value cache and per-request ranges."""
    shape: Shape
    Q: HostTensor            # [batch, n_q, d]
    K: HostTensor            # [rows, n_kv, d]
    V: HostTensor            # [rows, n_kv, d]
    V_lr: HostTensor         # [rows, n_agents * rank]
    B: HostTensor            # [n_agents, rank, n_kv * d]
    kv_start: np.ndarray     # int64 [batch]
    kv_len: np.ndarray       # int32 [batch]
    agent: np.ndarray        # int32 [batch]

    @property
    def batch(self) -> int:
        return int(self.kv_len.shape[0])

    @property
    def max_kv_len(self) -> int:
        return int(self.kv_len.max()) if self.batch else 0

    def attended_rows(self) -> int:
        return int(self.kv_len.astype(np.int64).sum())


@dataclass
class PrefillCase:
    shape: Shape
    Q: HostTensor            # [L_C, n_q, d]
    K: HostTensor            # [L_P + L_C, n_kv, d]
    V: HostTensor            # [L_P + L_C, n_kv, d]
    V_lr: HostTensor         # [L_P + L_C, n_agents * rank]
    B: HostTensor            # [n_agents, rank, n_kv * d]
    L_P: int
    L_C: int
    agent: int = 0


@dataclass
class PrefillBatch:
    """Several chunked prefills in one launch: request b's queries are rows q_start[b] .. of Q, its
    cache rows start at kv_start[b] (kv_prefix[b] cached tokens, then its chunk of q_len[b])."""
    shape: Shape
    Q: HostTensor            # [q_rows, n_q, d]
    K: HostTensor            # [kv_rows, n_kv, d]
    V: HostTensor            # [kv_rows, n_kv, d]
    V_lr: HostTensor         # [kv_rows, n_agents * rank]
    B: HostTensor            # [n_agents, rank, n_kv * d]
    q_start: np.ndarray      # int64 [batch]
    q_len: np.ndarray        # int32 [batch]
    kv_start: np.ndarray     # int64 [batch]
    kv_prefix: np.ndarray    # int32 [batch]
    agents: np.ndarray       # int32 [batch]

    @property
    def max_q_len(self) -> int:
        return int(self.q_len.max()) if len(self.q_len) else 0


@dataclass
class PagedDecodeBatch:
    """Decode over a paged cache: request b's logical row j is row j % P of page block_table[b, j // P]."""
    shape: Shape
    Q: HostTensor            # [batch, n_q, d]
    K_pages: HostTensor      # [n_pages, P, n_kv, d]
    V_pages: HostTensor      # [n_pages, P, n_kv, d]
    Vlr_pages: HostTensor    # [n_pages, P, n_agents * rank]
    B: HostTensor            # [n_agents, rank, n_kv * d]
    block_table: np.ndarray  # int32 [batch, max_blocks]
    kv_len: np.ndarray       # int32 [batch]
    agents: np.ndarray       # int32 [batch]

    @property
    def max_kv_len(self) -> int:
        return int(self.kv_len.max()) if len(self.kv_len) else 0


@dataclass
class PagedPrefillBatch:
    """Several chunked prefills over a paged cache: request b's cache row j is row j % P of page
    block_table[b, j // P]; its queries are rows q_start[b] .. of Q."""
    shape: Shape
    Q: HostTensor            # [q_rows, n_q, d]
    K_pages: HostTensor      # [n_pages, P, n_kv, d]
    V_pages: HostTensor      # [n_pages, P, n_kv, d]
    Vlr_pages: HostTensor    # [n_pages, P, n_agents * rank]
    B: HostTensor            # [n_agents, rank, n_kv * d]
    block_table: np.ndarray  # int32 [batch, max_blocks]
    q_start: np.ndarray      # int64 [batch]
    q_len: np.ndarray        # int32 [batch]
    kv_prefix: np.ndarray    # int32 [batch]
    agents: np.ndarray       # int32 [batch]

    @property
    def max_q_len(self) -> int:
        return int(self.q_len.max()) if len(self.q_len) else 0


@dataclass
class PrecomputeCase:
    shape: Shape
    X: HostTensor            # [T, d_model]
    A: HostTensor            # [d_model, n_agents * rank]


def _adapters(key: Tuple[int, ...], s: Shape, a_std: float) -> Tuple[HostTensor, HostTensor]:
    """Stacked down-projections A = [A_1 .. A_N] (column block k = agent k) and up-projections B."""
    A = normal(key + (T_A,), (s.d_model, s.n_agents * s.rank), a_std, s.dtype)
    B = normal(key + (T_B,), (s.n_agents, s.rank, s.d_kv), 0.05, s.dtype)
    return A, B


# ---- tiny fp32 workload: projections are drawn and K/V_base are X W0 (host fp64, rounded to fp32)
@dataclass
class TinyWorkload:
    shape: Shape
    X: HostTensor          # [256, d_model]
    W0_k: np.ndarray       # fp32 [d_model, d_kv]
    W0_v: np.ndarray       # fp32 [d_model, d_kv]
    A: HostTensor          # [d_model, N*r]
    B: HostTensor          # [N, r, d_kv]
    Q: HostTensor          # [L_C, n_q, d]
    K: HostTensor          # [L_P + L_C, n_kv, d]  (= X W0_k)
    V: HostTensor          # [L_P + L_C, n_kv, d]  (= X W0_v)
    L_P: int
    L_C: int
    x_dec: HostTensor      # [steps, d_model] new tokens appended one per decode step
    K_dec: HostTensor      # [steps, n_kv, d]  (= x_dec W0_k)
    V_dec: HostTensor      # [steps, n_kv, d]  (= x_dec W0_v)
    Q_dec: HostTensor      # [steps, N, n_q, d] one query per agent per step


def _base_projection(x: HostTensor, W: np.ndarray, s: Shape) -> HostTensor:
    """Input synthesis for the tiny workload: base keys/values of drawn tokens (fp64 product, fp32 storage)."""
    y = x.as_f64() @ W.astype(np.float64)
    return HostTensor(y.astype(np.float32).reshape(x.shape[0], s.n_kv, s.d_head), "f32")


def tiny_workload(steps: int = 8) -> TinyWorkload:
    s = TINY_SHAPE
    L_P, L_C = 192, 64
    key = (TINY, 0, 0)
    X = normal(key + (T_X,), (L_P + L_C, s.d_model), 1.0, "f32")
    W0_k = normal(key + (T_W0K,), (s.d_model, s.d_kv), 1.0 / math.sqrt(s.d_model), "f32").data
    W0_v = normal(key + (T_W0V,), (s.d_model, s.d_kv), 1.0 / math.sqrt(s.d_model), "f32").data
    A, B = _adapters(key, s, 1.0 / math.sqrt(s.d_model))
    Q = normal(key + (T_Q,), (L_C, s.n_q, s.d_head), 1.0, "f32")
    x_dec = normal(key + (T_XDEC,), (steps, s.d_model), 1.0, "f32")
    Q_dec = normal(key + (T_QDEC,), (steps, s.n_agents, s.n_q, s.d_head), 1.0, "f32")
    return TinyWorkload(s, X, W0_k, W0_v, A, B, Q,
                        _base_projection(X, W0_k, s), _base_projection(X, W0_v, s), L_P, L_C,
                        x_dec, _base_projection(x_dec, W0_k, s), _base_projection(x_dec, W0_v, s), Q_dec)


# ---- single-request decode (Llama-3.1-8B layer, L = 1900)
def llama_decode(L: int = 1900, agent: int = 0) -> DecodeBatch:
    s = LLAMA_SHAPE
    key = (LLAMA_DECODE, 0, 0)
    K = normal(key + (T_K,), (L, s.n_kv, s.d_head), 1.0, s.dtype)
    V = normal(key + (T_V,), (L, s.n_kv, s.d_head), 1.0, s.dtype)
    V_lr = normal(key + (T_VLR,), (L, s.n_agents * s.rank), 1.0, s.dtype)
    _, B = _adapters(key, s, 1.0 / math.sqrt(s.d_model))
    Q = normal(key + (T_Q,), (1, s.n_q, s.d_head), 1.0, s.dtype)
    return DecodeBatch(s, Q, K, V, V_lr, B, np.zeros(1, np.int64), np.array([L], np.int32),
                       np.array([agent], np.int32))


# ---- chunked prefill (L_P = 16384 cached, L_C = 2048 new) and its LR precompute
def llama_prefill(L_P: int = 16384, L_C: int = 2048, agent: int = 0) -> PrefillCase:
    s = LLAMA_SHAPE
    key = (LLAMA_PREFILL, 0, 0)
    L = L_P + L_C
    K = normal(key + (T_K,), (L, s.n_kv, s.d_head), 1.0, s.dtype)
    V = normal(key + (T_V,), (L, s.n_kv, s.d_head), 1.0, s.dtype)
    V_lr = normal(key + (T_VLR,), (L, s.n_agents * s.rank), 1.0, s.dtype)
    _, B = _adapters(key, s, 1.0 / math.sqrt(s.d_model))
    Q = normal(key + (T_Q,), (L_C, s.n_q, s.d_head), 1.0, s.dtype)
    return PrefillCase(s, Q, K, V, V_lr, B, L_P, L_C, agent)


def llama_prefill_qkvo(L_P: int = 16384, L_C: int = 2048, agent: int = 0) -> QkvoPrefillCase:
    """The chunked prefill above with LoRA on the keys as well (the qkvo configuration): the same
    Q, K_base, V_base, V_lr and B, plus K_lr ~ N(0, 1) and B_k ~ N(0, 0.3^2)."""
    s = LLAMA_SHAPE
    key = (LLAMA_PREFILL, 0, 0)
    base = llama_prefill(L_P, L_C, agent)
    L = L_P + L_C
    K_lr = normal(key + (T_KLR,), (L, s.n_agents * s.rank), 1.0, s.dtype)
    B_k = normal(key + (T_BK,), (s.n_agents, s.rank, s.d_kv), 0.3, s.dtype)
    cos, sin = rope_tables(L, s.d_head)
    return QkvoPrefillCase(base, K_lr, B_k, cos, sin)


def llama_precompute(T: int = 2048) -> PrecomputeCase:
    s = LLAMA_SHAPE
    key = (LLAMA_PREFILL, 0, 0)
    X = normal(key + (T_X,), (T, s.d_model), 1.0, s.dtype)
    A, _ = _adapters(key, s, 1.0 / math.sqrt(s.d_model))
    return PrecomputeCase(s, X, A)


# ---- concurrent long-context decode: 16 requests, each over its own 66,400-token trajectory
def llama_long_decode(n_req: int = 16, L: int = 66400, requests: Optional[Sequence[int]] = None) -> DecodeBatch:
    """Packed caches: request b owns rows [b*L, (b+1)*L). Every tensor of request b is drawn from
    its own stream, so a subset of requests (``requests``) can be drawn alone with identical values."""
    s = LLAMA_SHAPE
    reqs = list(range(n_req)) if requests is None else list(requests)
    Ks, Vs, Ls = [], [], []
    for b in reqs:
        key = (LLAMA_LONG_DECODE, 0, b)
        Ks.append(normal(key + (T_K,), (L, s.n_kv, s.d_head), 1.0, s.dtype).data)
        Vs.append(normal(key + (T_V,), (L, s.n_kv, s.d_head), 1.0, s.dtype).data)
        Ls.append(normal(key + (T_VLR,), (L, s.n_agents * s.rank), 1.0, s.dtype).data)
    key0 = (LLAMA_LONG_DECODE, 0, 10_000)
    _, B = _adapters(key0, s, 1.0 / math.sqrt(s.d_model))
    agents_all = rng(LLAMA_LONG_DECODE, 0, 10_000, T_AGENT).integers(0, s.n_agents, size=n_req).astype(np.int32)
    Qall = normal(key0 + (T_Q,), (n_req, s.n_q, s.d_head), 1.0, s.dtype)
    Q = HostTensor(Qall.data[reqs], s.dtype)
    n = len(reqs)
    return DecodeBatch(s, Q,
                       HostTensor(np.concatenate(Ks), s.dtype), HostTensor(np.concatenate(Vs), s.dtype),
                       HostTensor(np.concatenate(Ls), s.dtype), B,
                       np.arange(n, dtype=np.int64) * L, np.full(n, L, np.int32), agents_all[reqs])


# ---- Ministral-8B-shaped decode step: 36 layers x (precompute + decode), 32 requests
MINISTRAL_LAYERS = 36
MINISTRAL_REQUESTS = 32


def ministral_lengths(n_req: int = MINISTRAL_REQUESTS, lo: float = 1900.0, hi: float = 32000.0) -> np.ndarray:
    """Context lengths log-uniform in [lo, hi], rounded to the nearest integer; the same for every layer."""
    u = rng(MINISTRAL_STEP, 0, 10_000, T_LEN).uniform(math.log(lo), math.log(hi), size=n_req)
    return np.rint(np.exp(u)).astype(np.int32)


def ministral_agents(n_req: int = MINISTRAL_REQUESTS) -> np.ndarray:
    return rng(MINISTRAL_STEP, 0, 10_000, T_AGENT).integers(0, MINISTRAL_SHAPE.n_agents, size=n_req).astype(np.int32)


def ministral_layer(layer: int, requests: Optional[Sequence[int]] = None) -> Tuple[DecodeBatch, PrecomputeCase]:
    """One layer of the step. Request b's cache occupies rows [start_b, start_b + L_b) of the packed
    layer cache (starts are the prefix sums of all 32 lengths, also when only a subset is drawn).
    The precompute computes the LR rows of the 32 newest tokens (one per request)."""
    s = MINISTRAL_SHAPE
    lens = ministral_lengths()
    agents = ministral_agents()
    starts = np.concatenate([[0], np.cumsum(lens.astype(np.int64))[:-1]])
    reqs = list(range(len(lens))) if requests is None else list(requests)
    Ks, Vs, Ls = [], [], []
    for b in reqs:
        key = (MINISTRAL_STEP, layer, b)
        Ks.append(normal(key + (T_K,), (int(lens[b]), s.n_kv, s.d_head), 1.0, s.dtype).data)
        Vs.append(normal(key + (T_V,), (int(lens[b]), s.n_kv, s.d_head), 1.0, s.dtype).data)
        Ls.append(normal(key + (T_VLR,), (int(lens[b]), s.n_agents * s.rank), 1.0, s.dtype).data)
    keyL = (MINISTRAL_STEP, layer, 10_000)
    A, B = _adapters(keyL, s, 1.0 / math.sqrt(s.d_model))
    Qall = normal(keyL + (T_Q,), (len(lens), s.n_q, s.d_head), 1.0, s.dtype)
    X = normal(keyL + (T_X,), (len(lens), s.d_model), 1.0, s.dtype)
    sub_starts = np.concatenate([[0], np.cumsum(lens[reqs].astype(np.int64))[:-1]]) if requests is not None else starts
    dec = DecodeBatch(s, HostTensor(Qall.data[reqs], s.dtype),
                      HostTensor(np.concatenate(Ks), s.dtype), HostTensor(np.concatenate(Vs), s.dtype),
                      HostTensor(np.concatenate(Ls), s.dtype), B,
                      sub_starts.astype(np.int64), lens[reqs].astype(np.int32), agents[reqs].astype(np.int32))
    pre = PrecomputeCase(s, HostTensor(X.data[reqs], s.dtype), A)
    return dec, pre


def ministral_layer_device(layer: int, torch, device: str = "cuda") -> Dict[str, object]:
    """One layer of the step drawn on the GPU with torch's generator (seconds instead of minutes
    for 36 layers of 305,707 cache rows): the same shapes and distributions as ``ministral_layer``
    but other values. The benchmark times these layers and a GPU parity test checks layer 0 of
    exactly these values against the oracle. K, V, V_lr ~ N(0, 1); A ~ N(0, 1/64^2) stacked
    [N*r, d_model]; B ~ N(0, 0.05^2); X, Q ~ N(0, 1); all rounded to bf16. Also returns the packed
    row starts, lengths and agents of the 32 requests (the same every layer)."""
    s = MINISTRAL_SHAPE
    lens = ministral_lengths()
    agents = ministral_agents()
    starts = np.concatenate([[0], np.cumsum(lens.astype(np.int64))[:-1]])
    rows = int(lens.sum())
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * (layer + 1) + 42)
    f32, bf = torch.float32, torch.bfloat16
    out = {}
    out["K"] = torch.randn((rows, s.n_kv, s.d_head), generator=g, device=device, dtype=f32).to(bf)
    out["V"] = torch.randn((rows, s.n_kv, s.d_head), generator=g, device=device, dtype=f32).to(bf)
    out["V_lr"] = torch.randn((rows, s.n_agents * s.rank), generator=g, device=device, dtype=f32).to(bf)
    out["A"] = (torch.randn((s.n_agents * s.rank, s.d_model), generator=g, device=device, dtype=f32) / 64.0).to(bf)
    out["B"] = (torch.randn((s.n_agents, s.rank, s.d_kv), generator=g, device=device, dtype=f32) * 0.05).to(bf)
    out["X"] = torch.randn((len(lens), s.d_model), generator=g, device=device, dtype=f32).to(bf)
    out["Q"] = torch.randn((len(lens), s.n_q, s.d_head), generator=g, device=device, dtype=f32).to(bf)
    out["kv_start"], out["kv_len"], out["agent"] = starts.astype(np.int64), lens.astype(np.int32), agents.astype(np.int32)
    return out


# ---- small random cases (any shape) for tests
def random_decode(key: Sequence[int], s: Shape, kv_lens: Sequence[int], kv_starts: Optional[Sequence[int]] = None,
                  rows: Optional[int] = None, agents: Optional[Sequence[int]] = None, b_std: float = 0.05) -> DecodeBatch:
    key = tuple(key)
    n = len(kv_lens)
    kv_lens = np.asarray(kv_lens, np.int32)
    if kv_starts is None:
        kv_starts = np.concatenate([[0], np.cumsum(kv_lens.astype(np.int64))[:-1]]) if n else np.zeros(0, np.int64)
    kv_starts = np.asarray(kv_starts, np.int64)
    if rows is None:
        rows = int(max([0] + [int(a + b) for a, b in zip(kv_starts, kv_lens)]))
    rows = max(rows, 1)
    K = normal(key + (T_K,), (rows, s.n_kv, s.d_head), 1.0, s.dtype)
    V = normal(key + (T_V,), (rows, s.n_kv, s.d_head), 1.0, s.dtype)
    V_lr = normal(key + (T_VLR,), (rows, s.n_agents * s.rank), 1.0, s.dtype)
    B = normal(key + (T_B,), (s.n_agents, s.rank, s.d_kv), b_std, s.dtype)
    Q = normal(key + (T_Q,), (n, s.n_q, s.d_head), 1.0, s.dtype)
    if agents is None:
        agents = rng(*key, T_AGENT).integers(0, s.n_agents, size=n)
    return DecodeBatch(s, Q, K, V, V_lr, B, kv_starts, kv_lens, np.asarray(agents, np.int32))


@dataclass
class QkvoDecodeBatch:
    """A decode batch with LoRA on the keys as well (the qkvo configuration)."""
    base: DecodeBatch
    K_lr: HostTensor         # [rows, n_agents * rank]
    B_k: HostTensor          # [n_agents, rank, n_kv * d]
    cos: np.ndarray          # float32 [>= max_kv_len, d/2], row = a request's key position
    sin: np.ndarray


def random_decode_qkvo(key: Sequence[int], s: Shape, kv_lens: Sequence[int], kv_starts: Optional[Sequence[int]] = None,
                       rows: Optional[int] = None, agents: Optional[Sequence[int]] = None, b_std: float = 0.05,
                       bk_std: float = 0.3) -> QkvoDecodeBatch:
    """random_decode plus K_lr ~ N(0, 1), B_k ~ N(0, bk_std^2) and rotary tables of max(kv_lens) rows."""
    key = tuple(key)
    base = random_decode(key, s, kv_lens, kv_starts, rows, agents, b_std)
    K_lr = normal(key + (T_KLR,), (base.K.shape[0], s.n_agents * s.rank), 1.0, s.dtype)
    B_k = normal(key + (T_BK,), (s.n_agents, s.rank, s.d_kv), bk_std, s.dtype)
    cos, sin = rope_tables(max(1, base.max_kv_len), s.d_head)
    return QkvoDecodeBatch(base, K_lr, B_k, cos, sin)


def llama_long_decode_key_lora(n_req: int = 16, L: int = 66400, requests: Optional[Sequence[int]] = None):
    """The key-side operands of the 16 x 66,400 decode with LoRA on the keys: (K_lr, B_k, cos, sin).
    Request b's K_lr rows come from its own stream, B_k ~ N(0, 0.3^2), rotary tables of L rows."""
    s = LLAMA_SHAPE
    reqs = list(range(n_req)) if requests is None else list(requests)
    Klr = [normal((LLAMA_LONG_DECODE, 0, b, T_KLR), (L, s.n_agents * s.rank), 1.0, s.dtype).data for b in reqs]
    B_k = normal((LLAMA_LONG_DECODE, 0, 10_000, T_BK), (s.n_agents, s.rank, s.d_kv), 0.3, s.dtype)
    cos, sin = rope_tables(L, s.d_head)
    return HostTensor(np.concatenate(Klr), s.dtype), B_k, cos, sin


def llama_long_decode_qkvo(n_req: int = 16, L: int = 66400, requests: Optional[Sequence[int]] = None) -> QkvoDecodeBatch:
    """The 16 x 66,400 decode above with LoRA on the keys as well."""
    base = llama_long_decode(n_req, L, requests)
    return QkvoDecodeBatch(base, *llama_long_decode_key_lora(n_req, L, requests))


def random_prefill(key: Sequence[int], s: Shape, L_P: int, L_C: int, agent: int = 0, b_std: float = 0.05) -> PrefillCase:
    key = tuple(key)
    L = L_P + L_C
    K = normal(key + (T_K,), (L, s.n_kv, s.d_head), 1.0, s.dtype)
    V = normal(key + (T_V,), (L, s.n_kv, s.d_head), 1.0, s.dtype)
    V_lr = normal(key + (T_VLR,), (L, s.n_agents * s.rank), 1.0, s.dtype)
    B = normal(key + (T_B,), (s.n_agents, s.rank, s.d_kv), b_std, s.dtype)
    Q = normal(key + (T_Q,), (L_C, s.n_q, s.d_head), 1.0, s.dtype)
    return PrefillCase(s, Q, K, V, V_lr, B, L_P, L_C, agent)


@dataclass
class QkvoPrefillCase:
    """A prefill with LoRA on the keys as well (the qkvo configuration)."""
    base: PrefillCase
    K_lr: HostTensor         # [L_P + L_C, n_agents * rank]
    B_k: HostTensor          # [n_agents, rank, n_kv * d]
    cos: np.ndarray          # float32 [L_P + L_C, d/2]
    sin: np.ndarray


def rope_tables(positions: int, d_head: int, theta: float = 500000.0) -> Tuple[np.ndarray, np.ndarray]:
    """Cosine / sine tables [positions, d_head/2] (float32) of the standard rotary angles
    p * theta^(-2i/d_head) (theta 500,000 as in Llama 3.1). They are an input of the key-side LoRA
    path, which takes whatever tables the caller gives."""
    inv = theta ** (-np.arange(0, d_head, 2, dtype=np.float64) / d_head)
    ang = np.arange(positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def random_prefill_qkvo(key: Sequence[int], s: Shape, L_P: int, L_C: int, agent: int = 0, b_std: float = 0.05,
                        bk_std: float = 0.3) -> QkvoPrefillCase:
    """random_prefill plus the key-side rank-r cache K_lr ~ N(0, 1), B_k ~ N(0, bk_std^2) (so the
    rank-r part of a key is of the order of K_base's entries) and the rotary tables."""
    key = tuple(key)
    L = L_P + L_C
    base = random_prefill(key, s, L_P, L_C, agent, b_std)
    K_lr = normal(key + (T_KLR,), (L, s.n_agents * s.rank), 1.0, s.dtype)
    B_k = normal(key + (T_BK,), (s.n_agents, s.rank, s.d_kv), bk_std, s.dtype)
    cos, sin = rope_tables(L, s.d_head)
    return QkvoPrefillCase(base, K_lr, B_k, cos, sin)


def random_prefill_batch(key: Sequence[int], s: Shape, requests: Sequence[Tuple[int, int, int]],
                         gap: int = 3, kv_starts: Optional[Sequence[int]] = None, b_std: float = 0.05) -> PrefillBatch:
    """requests = [(L_P, L_C, agent), ...]. Query rows and (unless kv_starts is given) cache ranges are
    laid out one after the other with `gap` uncovered rows before each."""
    key = tuple(key)
    q_start, kv_start_auto = [], []
    q, k = 0, 0
    for (lp, lc, _) in requests:
        q += gap
        k += gap
        q_start.append(q)
        kv_start_auto.append(k)
        q += lc
        k += lp + lc
    kv_start = list(kv_starts) if kv_starts is not None else kv_start_auto
    kv_rows = max([ks + lp + lc for ks, (lp, lc, _) in zip(kv_start, requests)] + [k]) + gap
    q_rows = q + gap
    K = normal(key + (T_K,), (kv_rows, s.n_kv, s.d_head), 1.0, s.dtype)
    V = normal(key + (T_V,), (kv_rows, s.n_kv, s.d_head), 1.0, s.dtype)
    V_lr = normal(key + (T_VLR,), (kv_rows, s.n_agents * s.rank), 1.0, s.dtype)
    B = normal(key + (T_B,), (s.n_agents, s.rank, s.d_kv), b_std, s.dtype)
    Q = normal(key + (T_Q,), (q_rows, s.n_q, s.d_head), 1.0, s.dtype)
    return PrefillBatch(s, Q, K, V, V_lr, B, np.asarray(q_start, np.int64),
                        np.asarray([lc for (_, lc, _) in requests], np.int32), np.asarray(kv_start, np.int64),
                        np.asarray([lp for (lp, _, _) in requests], np.int32),
                        np.asarray([a for (_, _, a) in requests], np.int32))


def random_paged_decode(key: Sequence[int], s: Shape, kv_lens: Sequence[int], page_size: int,
                        agents: Optional[Sequence[int]] = None, shared_prefix_pages: int = 0,
                        spare_pages: int = 3, b_std: float = 0.05) -> PagedDecodeBatch:
    """Pages dealt out in a seeded random order. The first ``shared_prefix_pages`` pages of every request
    that is long enough are the same physical pages (a common prefix). ``spare_pages`` pages are
    named by no request."""
    key = tuple(key)
    n = len(kv_lens)
    blocks = [(int(L) + page_size - 1) // page_size for L in kv_lens]
    max_blocks = max(blocks + [1])
    shared = list(range(shared_prefix_pages))
    own = sum(max(0, bl - shared_prefix_pages) for bl in blocks)
    n_pages = shared_prefix_pages + own + spare_pages
    perm = rng(*key, T_AGENT + 1).permutation(n_pages).astype(np.int32)
    table = np.zeros((n, max_blocks), np.int32)
    nxt = shared_prefix_pages
    for b, bl in enumerate(blocks):
        for j in range(bl):
            if j < shared_prefix_pages:
                table[b, j] = perm[j]
            else:
                table[b, j] = perm[nxt]
                nxt += 1
    K = normal(key + (T_K,), (n_pages, page_size, s.n_kv, s.d_head), 1.0, s.dtype)
    V = normal(key + (T_V,), (n_pages, page_size, s.n_kv, s.d_head), 1.0, s.dtype)
    L = normal(key + (T_VLR,), (n_pages, page_size, s.n_agents * s.rank), 1.0, s.dtype)
    B = normal(key + (T_B,), (s.n_agents, s.rank, s.d_kv), b_std, s.dtype)
    Q = normal(key + (T_Q,), (n, s.n_q, s.d_head), 1.0, s.dtype)
    if agents is None:
        agents = rng(*key, T_AGENT).integers(0, s.n_agents, size=n)
    return PagedDecodeBatch(s, Q, K, V, L, B, table, np.asarray(kv_lens, np.int32), np.asarray(agents, np.int32))


def random_paged_prefill_batch(key: Sequence[int], s: Shape, requests: Sequence[Tuple[int, int, int]],
                               page_size: int, shared_prefix_pages: int = 0, spare_pages: int = 3,
                               gap: int = 2, b_std: float = 0.05) -> PagedPrefillBatch:
    """requests = [(L_P, L_C, agent), ...]; cache pages dealt out in a seeded random order, the first
    ``shared_prefix_pages`` shared by every request long enough; query rows one after the other with
    `gap` uncovered rows before each."""
    key = tuple(key)
    lens = [lp + lc for (lp, lc, _) in requests]
    dec = random_paged_decode(key, s, lens, page_size, agents=[a for (_, _, a) in requests],
                              shared_prefix_pages=shared_prefix_pages, spare_pages=spare_pages, b_std=b_std)
    q_start, q = [], 0
    for (_, lc, _) in requests:
        q += gap
        q_start.append(q)
        q += lc
    Q = normal(key + (T_Q, 1), (q + gap, s.n_q, s.d_head), 1.0, s.dtype)
    return PagedPrefillBatch(s, Q, dec.K_pages, dec.V_pages, dec.Vlr_pages, dec.B, dec.block_table,
                             np.asarray(q_start, np.int64), np.asarray([lc for (_, lc, _) in requests], np.int32),
                             np.asarray([lp for (lp, _, _) in requests], np.int32), dec.agents)


def random_precompute(key: Sequence[int], s: Shape, T: int) -> PrecomputeCase:
    key = tuple(key)
    X = normal(key + (T_X,), (T, s.d_model), 1.0, s.dtype)
    A = normal(key + (T_A,), (s.d_model, s.n_agents * s.rank), 1.0 / math.sqrt(s.d_model), s.dtype)
    return PrecomputeCase(s, X, A)
