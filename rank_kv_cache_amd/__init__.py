"""Python binding of liblra (Flash-LoRA-Attention for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels of
``liblra.so``. PyTorch is used for device memory and streams. The binding checks that the
tensors handed over agree with each other (device, dtype, contiguity), derives the sizes and
strides the C ABI asks for, and turns a negative status into ``LraError``.

Importing this package loads ``liblra.so`` and fails loudly if it has not been built
(``python -m rank_kv_cache_amd.build``).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "LraError", "LIB_PATH", "abi_version", "status_str",
    "lra_lr_precompute", "lra_lr_precompute_workspace_bytes",
    "lra_attn_prefill", "lra_attn_prefill_qkvo", "lra_attn_prefill_qkvo_workspace_bytes", "lra_attn_prefill_varlen", "lra_attn_prefill_paged",
    "lra_attn_decode", "lra_attn_decode_workspace_bytes", "lra_attn_decode_default_split", "lra_attn_decode_strided",
    "lra_attn_decode_noalloc", "NOALLOC_SCRATCH_BYTES", "lra_attn_decode_step",
    "lra_attn_decode_qkvo", "lra_attn_decode_qkvo_workspace_bytes",
    "lra_attn_decode_paged", "lra_attn_decode_paged_default_split", "lra_attn_decode_paged_strided",
    "lra_expand_values", "lra_stream_read",
    "LRA_F32", "LRA_BF16", "ADAPTER_FREE", "EXPORTED_SYMBOLS",
]

# the in-tree build; LRA_LIB_PATH names another build of the same sources (e.g. the sanitized one)
LIB_PATH = os.environ.get("LRA_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblra.so")
LRA_F32, LRA_BF16 = 0, 1
ADAPTER_FREE = -1   # agent index of the adapter-free view (attention over the base cache alone)
NOALLOC_SCRATCH_BYTES = 32 << 20   # the static partials array of lra_attn_decode_noalloc

_c = ctypes
_p = _c.c_void_p
_i32, _i64, _sz, _f = _c.c_int32, _c.c_int64, _c.c_size_t, _c.c_float

# name -> (restype, argtypes); mirrors include/lra.h
_SIGNATURES = {
    "lra_abi_version": (_c.c_int, []),
    "lra_status_str": (_c.c_char_p, [_c.c_int]),
    "lra_last_error": (_c.c_char_p, []),
    "lra_lr_precompute_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32]),
    "lra_lr_precompute": (_c.c_int, [_c.c_int, _p, _i64, _i32, _i64, _p, _i32, _i32, _p, _i64, _i64, _i64, _p, _p,
                                     _sz, _p]),
    "lra_attn_prefill": (_c.c_int, [_c.c_int, _p, _i64, _i64, _p, _p, _p, _i64, _i64, _p, _i32, _i32, _i32, _i32,
                                    _i32, _i32, _f, _p, _p]),
    "lra_attn_prefill_qkvo_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "lra_attn_prefill_qkvo": (_c.c_int, [_c.c_int, _p, _i64, _i64, _p, _p, _p, _i64, _i64, _p, _i64, _p, _p, _p, _p,
                                         _i32, _i32, _i32, _i32, _i32, _i32, _f, _p, _sz, _p, _p]),
    "lra_attn_prefill_varlen": (_c.c_int, [_c.c_int, _p, _i64, _i32, _p, _p, _i64, _p, _p, _i64, _p, _i64, _i64, _p,
                                           _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _f, _p, _p]),
    "lra_attn_prefill_paged": (_c.c_int, [_c.c_int, _p, _i64, _i32, _p, _p, _i64, _p, _p, _p, _i64, _i32, _i64, _p,
                                          _i32, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _f, _p, _p]),
    "lra_attn_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i64, _i32]),
    "lra_attn_decode": (_c.c_int, [_c.c_int, _p, _i32, _p, _p, _i64, _p, _i64, _i64, _p, _p, _i64, _p, _i32, _p,
                                   _i32, _i32, _i32, _i32, _f, _i32, _p, _sz, _p, _p]),
    "lra_attn_decode_default_split": (_i32, [_i32, _i32, _i64]),
    "lra_attn_decode_step": (_c.c_int, [_c.c_int, _p, _i32, _p, _p, _i64, _p, _i64, _i64, _p, _p, _i64, _p, _i32, _p,
                                        _i32, _i32, _i32, _i32, _f, _p, _i64, _p, _i32, _i32, _p, _sz, _p, _p]),
    "lra_attn_decode_noalloc": (_c.c_int, [_c.c_int, _p, _i32, _p, _p, _i64, _p, _i64, _i64, _p, _p, _i64, _p, _i32,
                                           _p, _i32, _i32, _i32, _i32, _f, _i32, _p, _p]),
    "lra_attn_decode_strided": (_c.c_int, [_c.c_int, _p, _i32, _p, _p, _i64, _i64, _i64, _p, _i64, _i64, _p, _p,
                                           _i64, _p, _i32, _p, _i32, _i32, _i32, _i32, _f, _i32, _p, _sz, _p, _p]),
    "lra_attn_decode_qkvo_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i64, _i32]),
    "lra_attn_decode_qkvo": (_c.c_int, [_c.c_int, _p, _i32, _p, _p, _i64, _p, _i64, _i64, _p, _i64, _p, _p, _i64, _p,
                                        _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _f, _i32, _p, _sz, _p, _p]),
    "lra_attn_decode_paged": (_c.c_int, [_c.c_int, _p, _i32, _p, _p, _p, _i64, _i32, _i64, _p, _i32, _p, _i64, _p, _i32,
                                         _p, _i32, _i32, _i32, _i32, _f, _i32, _p, _sz, _p, _p]),
    "lra_attn_decode_paged_default_split": (_i32, [_i32, _i32, _i64, _i32]),
    "lra_attn_decode_paged_strided": (_c.c_int, [_c.c_int, _p, _i32, _p, _p, _p, _i64, _i32, _i64, _i64, _i64, _i64,
                                                 _p, _i32, _p, _i64, _p, _i32, _p, _i32, _i32, _i32, _i32, _f, _i32,
                                                 _p, _sz, _p, _p]),
    "lra_expand_values": (_c.c_int, [_c.c_int, _p, _i64, _p, _i64, _p, _i32, _i32, _i32, _i32, _i32, _p, _p, _p,
                                     _i64, _p, _i64, _p, _p]),
    "lra_stream_read": (_c.c_int, [_p, _i64, _i32, _p, _p]),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)


class LraError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {status_str(status)} ({status}): {message}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m rank_kv_cache_amd.build` "
                          "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def abi_version() -> int:
    return int(_lib.lra_abi_version())


def status_str(status: int) -> str:
    return _lib.lra_status_str(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise LraError(status, where, _lib.lra_last_error().decode())


# ---------------------------------------------------------------------------------- marshalling
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LRA_F32
    if t.dtype == torch.bfloat16:
        return LRA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _same(ref: torch.Tensor, *ts: torch.Tensor) -> None:
    if not ref.is_cuda:
        raise ValueError(f"tensors must be on a GPU (got {ref.device}): the kernels take device pointers")
    for t in ts:
        if t.dtype != ref.dtype:
            raise TypeError(f"dtype mismatch: {t.dtype} vs {ref.dtype}")
        if t.device != ref.device:
            raise ValueError(f"device mismatch: {t.device} vs {ref.device}")


def _on_device(ref: torch.Tensor, **ts: Optional[torch.Tensor]) -> None:
    """Index tensors, row maps and workspaces: on the same GPU as the data, contiguous."""
    for name, t in ts.items():
        if t is None:
            continue
        if not t.is_cuda or t.device != ref.device:
            raise ValueError(f"{name} must be on {ref.device} (got {t.device})")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _dense(name: str, t: torch.Tensor) -> None:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _rows_dense(name: str, t: torch.Tensor) -> None:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")


def _vlr_check(name: str, t: torch.Tensor) -> None:
    """An LR cache: [rows, ld] with interleaved agents, or an agent-major [N, rows, ld] view."""
    if not ((t.dim() == 2 and t.stride(1) == 1) or (t.dim() == 3 and t.stride(2) == 1)):
        raise ValueError(f"{name} must be [rows, ld] (interleaved agents) or [N, rows, ld] (agent-major), unit column stride")


def _vlr_rows(t: torch.Tensor) -> int:
    return t.shape[-2]


def _vlr_strides(t: torch.Tensor, rank: int) -> tuple:
    """(ld_vlr, vlr_agent_stride) of an LR cache tensor."""
    if t.dim() == 2:
        return t.stride(0), rank
    return t.stride(1), t.stride(0)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _on(stream):
    """Context for the buffers the binding allocates (workspaces, outputs): they are allocated on the
    stream the kernels run on, so the caching allocator orders any reuse of that memory after them."""
    if stream is None:
        return contextlib.nullcontext()
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
    if s.cuda_stream == torch.cuda.current_stream().cuda_stream:
        return contextlib.nullcontext()
    return torch.cuda.stream(s)


# ---------------------------------------------------------------------------------- LR precompute
def lra_lr_precompute_workspace_bytes(T: int, d_model: int, n_agents: int, rank: int) -> int:
    return int(_lib.lra_lr_precompute_workspace_bytes(T, d_model, n_agents, rank))


def lra_lr_precompute(X: torch.Tensor, A: torch.Tensor, n_agents: int, rank: int, V_lr: torch.Tensor,
                      out_rows: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """V_lr[out_rows[t], :n_agents*rank] = X[t] @ A.T, with A = [A_1^T; ...; A_N^T] ([N*r, d_model]).

    ``workspace`` is accepted for compatibility; the kernel needs none (0 bytes)."""
    _same(X, A, V_lr)
    _rows_dense("X", X)
    _dense("A", A)
    _vlr_check("V_lr", V_lr)
    T, d_model = X.shape
    if A.shape != (n_agents * rank, d_model):
        raise ValueError(f"A has shape {tuple(A.shape)}, expected {(n_agents * rank, d_model)}")
    if out_rows is not None:
        if out_rows.dtype != torch.int64 or out_rows.numel() != T or not out_rows.is_contiguous():
            raise ValueError("out_rows must be a contiguous int64 tensor with one entry per row of X")
    need = lra_lr_precompute_workspace_bytes(T, d_model, n_agents, rank)
    if workspace is None and need:
        with _on(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _on_device(X, out_rows=out_rows, workspace=workspace)
    _check(_lib.lra_lr_precompute(_dtype_code(X), _ptr(X), T, d_model, X.stride(0), _ptr(A), n_agents, rank,
                                  _ptr(V_lr), *_vlr_strides(V_lr, rank), _vlr_rows(V_lr), _ptr(out_rows),
                                  _ptr(workspace), ws_bytes, _stream(stream)), "lra_lr_precompute")
    return V_lr


# ---------------------------------------------------------------------------------- prefill
def lra_attn_prefill(Q: torch.Tensor, L_P: int, K_base: torch.Tensor, V_base: torch.Tensor, V_lr: torch.Tensor,
                     B: torch.Tensor, agent: int, scale: float, O: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """Causal prefill of the L_C = Q.shape[0] new tokens over L_P cached + L_C new keys for ``agent``.

    Q [L_C, n_q, d]; K_base, V_base [>= L_P+L_C, n_kv, d]; V_lr [>= L_P+L_C, ld]; B [N, r, n_kv*d].
    ``agent`` = ADAPTER_FREE (-1) selects the adapter-free view: attention over the base cache
    alone, V_lr and B unread."""
    _same(Q, K_base, V_base, V_lr, B)
    for name, t in (("Q", Q), ("K_base", K_base), ("V_base", V_base), ("B", B)):
        _dense(name, t)
    _vlr_check("V_lr", V_lr)
    L_C, n_q, d = Q.shape
    n_kv = K_base.shape[1]
    n_agents, rank = B.shape[0], B.shape[1]
    L = L_P + L_C
    if K_base.shape[0] < L or V_base.shape[0] < L or _vlr_rows(V_lr) < L:
        raise ValueError(f"caches hold fewer than L_P + L_C = {L} rows")
    if K_base.shape[1:] != (n_kv, d) or V_base.shape[1:] != (n_kv, d) or B.shape[2] != n_kv * d:
        raise ValueError("K_base/V_base/B shapes disagree with Q")
    if O is None:
        with _on(stream):
            O = torch.empty_like(Q)
    _same(Q, O)
    _dense("O", O)
    _check(_lib.lra_attn_prefill(_dtype_code(Q), _ptr(Q), L_C, L_P, _ptr(K_base), _ptr(V_base), _ptr(V_lr),
                                 *_vlr_strides(V_lr, rank), _ptr(B), n_agents, agent, n_q, n_kv, d, rank, scale, _ptr(O),
                                 _stream(stream)), "lra_attn_prefill")
    return O


def lra_attn_prefill_qkvo(Q: torch.Tensor, L_P: int, K_base: torch.Tensor, V_base: torch.Tensor, V_lr: torch.Tensor,
                          K_lr: torch.Tensor, B: torch.Tensor, B_k: torch.Tensor, rope_cos: torch.Tensor,
                          rope_sin: torch.Tensor, agent: int, scale: float, workspace: Optional[torch.Tensor] = None,
                          O: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """``lra_attn_prefill`` with LoRA on the keys too: the agent's keys are
    K_base + RoPE(K_lr[:, agent cols] B_k[agent]) (rotate-half pairing, angle tables per position),
    expanded once per call into ``workspace`` (allocated here when None; size from
    ``lra_attn_prefill_qkvo_workspace_bytes``), then attended.

    K_lr [>= L_P+L_C, ld]; B_k [N, r, n_kv*d]; rope_cos, rope_sin fp32 [>= L_P+L_C, d/2]. bf16 only."""
    _same(Q, K_base, V_base, V_lr, K_lr, B, B_k)
    for name, t in (("Q", Q), ("K_base", K_base), ("V_base", V_base), ("B", B), ("B_k", B_k),
                    ("rope_cos", rope_cos), ("rope_sin", rope_sin)):
        _dense(name, t)
    _vlr_check("V_lr", V_lr)
    _rows_dense("K_lr", K_lr)
    L_C, n_q, d = Q.shape
    n_kv = K_base.shape[1]
    n_agents, rank = B.shape[0], B.shape[1]
    L = L_P + L_C
    if min(K_base.shape[0], V_base.shape[0], _vlr_rows(V_lr), K_lr.shape[0], rope_cos.shape[0], rope_sin.shape[0]) < L:
        raise ValueError(f"caches and angle tables hold fewer than L_P + L_C = {L} rows")
    if K_base.shape[1:] != (n_kv, d) or V_base.shape[1:] != (n_kv, d) or B.shape[2] != n_kv * d:
        raise ValueError("K_base/V_base/B shapes disagree with Q")
    if B_k.shape != B.shape:
        raise ValueError(f"B_k {tuple(B_k.shape)} must be shaped like B {tuple(B.shape)}")
    if rope_cos.dtype != torch.float32 or rope_sin.dtype != torch.float32 or rope_cos.device != Q.device \
            or rope_sin.device != Q.device:
        raise ValueError("rope_cos / rope_sin must be float32 tensors on Q's device")
    if rope_cos.shape[1:] != (d // 2,) or rope_sin.shape[1:] != (d // 2,):
        raise ValueError("rope tables must be [positions, d/2]")
    if O is None:
        with _on(stream):
            O = torch.empty_like(Q)
    _same(Q, O)
    _dense("O", O)
    ws_bytes = lra_attn_prefill_qkvo_workspace_bytes(L, n_kv, d)
    if workspace is None:
        with _on(stream):
            workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=Q.device)
    _on_device(Q, rope_cos=rope_cos, rope_sin=rope_sin, workspace=workspace)
    _check(_lib.lra_attn_prefill_qkvo(_dtype_code(Q), _ptr(Q), L_C, L_P, _ptr(K_base), _ptr(V_base), _ptr(V_lr),
                                      *_vlr_strides(V_lr, rank), _ptr(K_lr), K_lr.stride(0), _ptr(B), _ptr(B_k), _ptr(rope_cos),
                                      _ptr(rope_sin), n_agents, agent, n_q, n_kv, d, rank, scale, _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _ptr(O), _stream(stream)),
           "lra_attn_prefill_qkvo")
    return O


def lra_attn_prefill_qkvo_workspace_bytes(n_rows: int, n_kv: int, d_head: int) -> int:
    """Bytes of the qkvo prefill's workspace for a call over n_rows = L_P + L_C cache rows."""
    return int(_lib.lra_attn_prefill_qkvo_workspace_bytes(n_rows, n_kv, d_head))


def lra_attn_prefill_varlen(Q: torch.Tensor, q_start: torch.Tensor, q_len: torch.Tensor, max_q_len: int,
                            K_base: torch.Tensor, V_base: torch.Tensor, V_lr: torch.Tensor,
                            kv_start: torch.Tensor, kv_prefix: torch.Tensor, B: torch.Tensor, agent: torch.Tensor,
                            scale: float, O: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Several causal chunked prefills in one launch. Request b: queries Q[q_start[b] : +q_len[b]] at
    positions kv_prefix[b] .., cache rows kv_start[b] : +kv_prefix[b]+q_len[b], agent[b] (or
    ADAPTER_FREE). Q, O [q_rows, n_q, d]; K_base, V_base [kv_rows, n_kv, d]; V_lr [kv_rows, ld];
    q_start, kv_start int64 [batch]; q_len, kv_prefix, agent int32 [batch]; B [N, r, n_kv*d].
    ``max_q_len`` bounds every q_len[b]. Rows of O that no request covers are left as they were
    (O is allocated zeroed when omitted)."""
    _same(Q, K_base, V_base, V_lr, B)
    for name, t in (("Q", Q), ("K_base", K_base), ("V_base", V_base), ("B", B)):
        _dense(name, t)
    _vlr_check("V_lr", V_lr)
    q_rows, n_q, d = Q.shape
    kv_rows, n_kv = K_base.shape[0], K_base.shape[1]
    n_agents, rank = B.shape[0], B.shape[1]
    if K_base.shape[1:] != (n_kv, d) or V_base.shape != K_base.shape or B.shape[2] != n_kv * d:
        raise ValueError("K_base/V_base/B shapes disagree with Q")
    if _vlr_rows(V_lr) != kv_rows:
        raise ValueError("V_lr must have as many rows as K_base")
    for name, t, dt in (("q_start", q_start, torch.int64), ("q_len", q_len, torch.int32),
                        ("kv_start", kv_start, torch.int64), ("kv_prefix", kv_prefix, torch.int32),
                        ("agent", agent, torch.int32)):
        if t.dtype != dt or t.dim() != 1 or t.device != Q.device or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous 1-d {dt} tensor on {Q.device}")
    batch = q_start.shape[0]
    if any(t.shape[0] != batch for t in (q_len, kv_start, kv_prefix, agent)):
        raise ValueError("per-request tables disagree in length")
    if O is None:
        with _on(stream):
            O = torch.zeros_like(Q)
    _same(Q, O)
    _dense("O", O)
    if O.shape != Q.shape:
        raise ValueError("O must have Q's shape")
    _on_device(Q, q_start=q_start, q_len=q_len, kv_start=kv_start, kv_prefix=kv_prefix, agent=agent)
    _check(_lib.lra_attn_prefill_varlen(_dtype_code(Q), _ptr(Q), q_rows, batch, _ptr(q_start), _ptr(q_len), max_q_len,
                                        _ptr(K_base), _ptr(V_base), kv_rows, _ptr(V_lr), *_vlr_strides(V_lr, rank),
                                        _ptr(kv_start), _ptr(kv_prefix), _ptr(B), n_agents, _ptr(agent),
                                        n_q, n_kv, d, rank, scale, _ptr(O), _stream(stream)),
           "lra_attn_prefill_varlen")
    return O


def lra_attn_prefill_paged(Q: torch.Tensor, q_start: torch.Tensor, q_len: torch.Tensor, max_q_len: int,
                           K_pages: torch.Tensor, V_pages: torch.Tensor, Vlr_pages: torch.Tensor,
                           block_table: torch.Tensor, kv_prefix: torch.Tensor, B: torch.Tensor, agent: torch.Tensor,
                           scale: float, O: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """lra_attn_prefill_varlen over a paged cache: request b's cache row j is row j % P of page
    block_table[b, j // P]. K_pages, V_pages [n_pages, P, n_kv, d]; Vlr_pages [n_pages, P, ld];
    block_table int32 [batch, max_blocks]; q_start int64, q_len / kv_prefix / agent int32 [batch]."""
    _same(Q, K_pages, V_pages, Vlr_pages, B)
    for name, t in (("Q", Q), ("K_pages", K_pages), ("V_pages", V_pages), ("B", B)):
        _dense(name, t)
    q_rows, n_q, d = Q.shape
    n_pages, P, n_kv = K_pages.shape[0], K_pages.shape[1], K_pages.shape[2]
    n_agents, rank = B.shape[0], B.shape[1]
    if V_pages.shape != K_pages.shape or K_pages.shape[3] != d or B.shape[2] != n_kv * d:
        raise ValueError("K_pages/V_pages/B shapes disagree with Q")
    if Vlr_pages.dim() != 3 or Vlr_pages.shape[:2] != (n_pages, P) or Vlr_pages.stride(2) != 1 or \
            Vlr_pages.stride(0) != P * Vlr_pages.stride(1):
        raise ValueError("Vlr_pages must be [n_pages, P, ld] with rows of one page adjacent")
    batch = q_start.shape[0]
    for name, t, dt in (("q_start", q_start, torch.int64), ("q_len", q_len, torch.int32),
                        ("kv_prefix", kv_prefix, torch.int32), ("agent", agent, torch.int32)):
        if t.dtype != dt or t.shape != (batch,) or t.device != Q.device or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous 1-d {dt} tensor of length {batch} on {Q.device}")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous() or \
            block_table.shape[0] != batch:
        raise TypeError("block_table must be a contiguous int32 [batch, max_blocks] tensor")
    if O is None:
        with _on(stream):
            O = torch.zeros_like(Q)
    _same(Q, O)
    _dense("O", O)
    if O.shape != Q.shape:
        raise ValueError("O must have Q's shape")
    _on_device(Q, q_start=q_start, q_len=q_len, block_table=block_table, kv_prefix=kv_prefix, agent=agent)
    _check(_lib.lra_attn_prefill_paged(_dtype_code(Q), _ptr(Q), q_rows, batch, _ptr(q_start), _ptr(q_len), max_q_len,
                                       _ptr(K_pages), _ptr(V_pages), _ptr(Vlr_pages), n_pages, P, Vlr_pages.stride(1),
                                       _ptr(block_table), block_table.shape[1], _ptr(kv_prefix), _ptr(B), n_agents,
                                       _ptr(agent), n_q, n_kv, d, rank, scale, _ptr(O), _stream(stream)),
           "lra_attn_prefill_paged")
    return O


# ---------------------------------------------------------------------------------- decode
def lra_attn_decode_default_split(batch: int, n_kv: int, max_kv_len: int) -> int:
    return int(_lib.lra_attn_decode_default_split(batch, n_kv, max_kv_len))


def lra_attn_decode_workspace_bytes(batch: int, n_q: int, n_kv: int, d_head: int, rank: int, max_kv_len: int,
                                    keys_per_split: int = 0) -> int:
    return int(_lib.lra_attn_decode_workspace_bytes(batch, n_q, n_kv, d_head, rank, max_kv_len, keys_per_split))


def lra_attn_decode(Q: torch.Tensor, K_base: torch.Tensor, V_base: torch.Tensor, V_lr: torch.Tensor,
                    kv_start: torch.Tensor, kv_len: torch.Tensor, max_kv_len: int, B: torch.Tensor,
                    agent: torch.Tensor, scale: float, keys_per_split: int = 0,
                    workspace: Optional[torch.Tensor] = None, O: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """One query per request over rows [kv_start[b], kv_start[b] + kv_len[b]) of the shared caches.

    Q [batch, n_q, d]; K_base, V_base [rows, n_kv, d]; V_lr [rows, ld]; kv_start int64 [batch];
    kv_len, agent int32 [batch]; B [N, r, n_kv*d]. ``agent[b]`` = ADAPTER_FREE (-1) gives request b
    the adapter-free view (base cache alone, no LR term), so adapted and adapter-free requests
    share one launch. ``workspace`` (uint8, lra_attn_decode_workspace_bytes() bytes, contents
    need no initialisation) is allocated when omitted."""
    _same(Q, K_base, V_base, V_lr, B)
    for name, t in (("Q", Q), ("K_base", K_base), ("V_base", V_base), ("B", B)):
        _dense(name, t)
    _vlr_check("V_lr", V_lr)
    batch, n_q, d = Q.shape
    n_kv = K_base.shape[1]
    n_agents, rank = B.shape[0], B.shape[1]
    if kv_start.dtype != torch.int64 or kv_len.dtype != torch.int32 or agent.dtype != torch.int32:
        raise TypeError("kv_start must be int64, kv_len and agent int32")
    for name, t in (("kv_start", kv_start), ("kv_len", kv_len), ("agent", agent)):
        if t.numel() != batch or not t.is_contiguous() or t.device != Q.device:
            raise ValueError(f"{name} must be a contiguous device tensor with one entry per request")
    if V_base.shape != K_base.shape or _vlr_rows(V_lr) != K_base.shape[0] or B.shape[2] != n_kv * d:
        raise ValueError("K_base/V_base/V_lr/B shapes disagree")
    need = lra_attn_decode_workspace_bytes(batch, n_q, n_kv, d, rank, max_kv_len, keys_per_split)
    if workspace is None and need:
        with _on(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if O is None:
        with _on(stream):
            O = torch.empty_like(Q)
    _same(Q, O)
    _dense("O", O)
    _on_device(Q, kv_start=kv_start, kv_len=kv_len, agent=agent, workspace=workspace)
    _check(_lib.lra_attn_decode(_dtype_code(Q), _ptr(Q), batch, _ptr(K_base), _ptr(V_base), K_base.shape[0],
                                _ptr(V_lr), *_vlr_strides(V_lr, rank), _ptr(kv_start), _ptr(kv_len), max_kv_len, _ptr(B),
                                n_agents, _ptr(agent), n_q, n_kv, d, rank, scale, keys_per_split,
                                _ptr(workspace), ws_bytes, _ptr(O), _stream(stream)), "lra_attn_decode")
    return O


def lra_attn_decode_step(Q: torch.Tensor, K_base: torch.Tensor, V_base: torch.Tensor, V_lr: torch.Tensor,
                         kv_start: torch.Tensor, kv_len: torch.Tensor, max_kv_len: int, B: torch.Tensor,
                         agent: torch.Tensor, scale: float, X_new: torch.Tensor, A: torch.Tensor,
                         keys_per_split: int = 0, workspace: Optional[torch.Tensor] = None,
                         O: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """``lra_attn_decode`` after writing each request's newest LR row in the same launch:
    V_lr[kv_start[b] + kv_len[b] - 1, :N*r] = X_new[b] @ A.T (X_new [batch, d_model], A the stacked
    [N*r, d_model] down-projections). V_lr is updated in place."""
    _same(Q, K_base, V_base, V_lr, B, X_new, A)
    for name, t in (("Q", Q), ("K_base", K_base), ("V_base", V_base), ("B", B), ("A", A)):
        _dense(name, t)
    _vlr_check("V_lr", V_lr)
    _rows_dense("X_new", X_new)
    batch, n_q, d = Q.shape
    n_kv = K_base.shape[1]
    n_agents, rank = B.shape[0], B.shape[1]
    d_model = X_new.shape[1]
    if kv_start.dtype != torch.int64 or kv_len.dtype != torch.int32 or agent.dtype != torch.int32:
        raise TypeError("kv_start must be int64, kv_len and agent int32")
    for name, t in (("kv_start", kv_start), ("kv_len", kv_len), ("agent", agent)):
        if t.numel() != batch or not t.is_contiguous() or t.device != Q.device:
            raise ValueError(f"{name} must be a contiguous device tensor with one entry per request")
    if V_base.shape != K_base.shape or _vlr_rows(V_lr) != K_base.shape[0] or B.shape[2] != n_kv * d:
        raise ValueError("K_base/V_base/V_lr/B shapes disagree")
    if X_new.shape[0] != batch or A.shape != (n_agents * rank, d_model):
        raise ValueError("X_new must be [batch, d_model] and A [n_agents*rank, d_model]")
    need = lra_attn_decode_workspace_bytes(batch, n_q, n_kv, d, rank, max_kv_len, keys_per_split)
    if workspace is None and need:
        with _on(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if O is None:
        with _on(stream):
            O = torch.empty_like(Q)
    _same(Q, O)
    _dense("O", O)
    _on_device(Q, kv_start=kv_start, kv_len=kv_len, agent=agent, workspace=workspace)
    _check(_lib.lra_attn_decode_step(_dtype_code(Q), _ptr(Q), batch, _ptr(K_base), _ptr(V_base), K_base.shape[0],
                                     _ptr(V_lr), *_vlr_strides(V_lr, rank), _ptr(kv_start), _ptr(kv_len), max_kv_len, _ptr(B),
                                     n_agents, _ptr(agent), n_q, n_kv, d, rank, scale, _ptr(X_new), X_new.stride(0),
                                     _ptr(A), d_model, keys_per_split, _ptr(workspace), ws_bytes, _ptr(O),
                                     _stream(stream)), "lra_attn_decode_step")
    return O


def lra_attn_decode_noalloc(Q: torch.Tensor, K_base: torch.Tensor, V_base: torch.Tensor, V_lr: torch.Tensor,
                            kv_start: torch.Tensor, kv_len: torch.Tensor, max_kv_len: int, B: torch.Tensor,
                            agent: torch.Tensor, scale: float, O: torch.Tensor, keys_per_split: int = 0,
                            stream=None) -> torch.Tensor:
    """lra_attn_decode without a workspace: the library keeps the split partials in its own static
    device array (NOALLOC_SCRATCH_BYTES per GPU), so the call allocates nothing. The caller passes
    the output O. Calls on one GPU share that array: order them (e.g. on one stream)."""
    _same(Q, K_base, V_base, V_lr, B, O)
    for name, t in (("Q", Q), ("K_base", K_base), ("V_base", V_base), ("B", B), ("O", O)):
        _dense(name, t)
    _vlr_check("V_lr", V_lr)
    batch, n_q, d = Q.shape
    n_kv = K_base.shape[1]
    n_agents, rank = B.shape[0], B.shape[1]
    if kv_start.dtype != torch.int64 or kv_len.dtype != torch.int32 or agent.dtype != torch.int32:
        raise TypeError("kv_start must be int64, kv_len and agent int32")
    for name, t in (("kv_start", kv_start), ("kv_len", kv_len), ("agent", agent)):
        if t.numel() != batch:
            raise ValueError(f"{name} must have one entry per request")
    if V_base.shape != K_base.shape or _vlr_rows(V_lr) != K_base.shape[0] or B.shape[2] != n_kv * d or O.shape != Q.shape:
        raise ValueError("K_base/V_base/V_lr/B/O shapes disagree")
    _on_device(Q, kv_start=kv_start, kv_len=kv_len, agent=agent)
    _check(_lib.lra_attn_decode_noalloc(_dtype_code(Q), _ptr(Q), batch, _ptr(K_base), _ptr(V_base), K_base.shape[0],
                                        _ptr(V_lr), *_vlr_strides(V_lr, rank), _ptr(kv_start), _ptr(kv_len), max_kv_len, _ptr(B),
                                        n_agents, _ptr(agent), n_q, n_kv, d, rank, scale, keys_per_split, _ptr(O),
                                        _stream(stream)), "lra_attn_decode_noalloc")
    return O


def lra_attn_decode_strided(Q: torch.Tensor, K_base: torch.Tensor, V_base: torch.Tensor, V_lr: torch.Tensor,
                            kv_start: torch.Tensor, kv_len: torch.Tensor, max_kv_len: int, B: torch.Tensor,
                            agent: torch.Tensor, scale: float, keys_per_split: int = 0,
                            workspace: Optional[torch.Tensor] = None, O: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """``lra_attn_decode`` over K/V views [rows, n_kv, d] of any layout with contiguous d-vectors,
    e.g. ``K_hm.transpose(0, 1)`` of a head-major cache K_hm [n_kv, rows, d]. K_base and V_base
    must have the same strides; the row and head strides are passed to the library as they are."""
    _same(Q, K_base, V_base, V_lr, B)
    for name, t in (("Q", Q), ("B", B)):
        _dense(name, t)
    _vlr_check("V_lr", V_lr)
    if K_base.dim() != 3 or K_base.stride(2) != 1 or V_base.shape != K_base.shape or V_base.stride() != K_base.stride():
        raise ValueError("K_base and V_base must be [rows, n_kv, d] views with equal strides and unit last stride")
    batch, n_q, d = Q.shape
    n_kv = K_base.shape[1]
    n_agents, rank = B.shape[0], B.shape[1]
    if kv_start.dtype != torch.int64 or kv_len.dtype != torch.int32 or agent.dtype != torch.int32:
        raise TypeError("kv_start must be int64, kv_len and agent int32")
    for name, t in (("kv_start", kv_start), ("kv_len", kv_len), ("agent", agent)):
        if t.numel() != batch or not t.is_contiguous() or t.device != Q.device:
            raise ValueError(f"{name} must be a contiguous device tensor with one entry per request")
    if K_base.shape[2] != d or _vlr_rows(V_lr) != K_base.shape[0] or B.shape[2] != n_kv * d:
        raise ValueError("K_base/V_base/V_lr/B shapes disagree")
    need = lra_attn_decode_workspace_bytes(batch, n_q, n_kv, d, rank, max_kv_len, keys_per_split)
    if workspace is None and need:
        with _on(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if O is None:
        with _on(stream):
            O = torch.empty_like(Q)
    _same(Q, O)
    _dense("O", O)
    _on_device(Q, kv_start=kv_start, kv_len=kv_len, agent=agent, workspace=workspace)
    _check(_lib.lra_attn_decode_strided(_dtype_code(Q), _ptr(Q), batch, _ptr(K_base), _ptr(V_base), K_base.shape[0],
                                        K_base.stride(0), K_base.stride(1), _ptr(V_lr), *_vlr_strides(V_lr, rank), _ptr(kv_start),
                                        _ptr(kv_len), max_kv_len, _ptr(B), n_agents, _ptr(agent), n_q, n_kv, d, rank,
                                        scale, keys_per_split, _ptr(workspace), ws_bytes, _ptr(O), _stream(stream)),
           "lra_attn_decode_strided")
    return O


def lra_attn_decode_qkvo_workspace_bytes(batch: int, n_q: int, n_kv: int, d_head: int, rank: int, max_kv_len: int,
                                         keys_per_split: int = 0) -> int:
    return int(_lib.lra_attn_decode_qkvo_workspace_bytes(batch, n_q, n_kv, d_head, rank, max_kv_len, keys_per_split))


def lra_attn_decode_qkvo(Q: torch.Tensor, K_base: torch.Tensor, V_base: torch.Tensor, V_lr: torch.Tensor,
                         K_lr: torch.Tensor, kv_start: torch.Tensor, kv_len: torch.Tensor, max_kv_len: int,
                         B: torch.Tensor, B_k: torch.Tensor, rope_cos: torch.Tensor, rope_sin: torch.Tensor,
                         agent: torch.Tensor, scale: float, keys_per_split: int = 0,
                         workspace: Optional[torch.Tensor] = None, O: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """``lra_attn_decode`` with LoRA on the keys too: request b's key t is
    K_base + RoPE_t(K_lr[row, agent cols] B_k[agent]) at table row t. K_lr [rows, ld]; B_k like B;
    rope_cos, rope_sin fp32 [>= max_kv_len, d/2]. bf16 only. ``workspace`` (uint8,
    lra_attn_decode_qkvo_workspace_bytes() bytes) is allocated when omitted."""
    _same(Q, K_base, V_base, V_lr, K_lr, B, B_k)
    for name, t in (("Q", Q), ("K_base", K_base), ("V_base", V_base), ("B", B), ("B_k", B_k),
                    ("rope_cos", rope_cos), ("rope_sin", rope_sin)):
        _dense(name, t)
    _vlr_check("V_lr", V_lr)
    _rows_dense("K_lr", K_lr)
    batch, n_q, d = Q.shape
    n_kv = K_base.shape[1]
    n_agents, rank = B.shape[0], B.shape[1]
    if kv_start.dtype != torch.int64 or kv_len.dtype != torch.int32 or agent.dtype != torch.int32:
        raise TypeError("kv_start must be int64, kv_len and agent int32")
    for name, t in (("kv_start", kv_start), ("kv_len", kv_len), ("agent", agent)):
        if t.numel() != batch or not t.is_contiguous() or t.device != Q.device:
            raise ValueError(f"{name} must be a contiguous device tensor with one entry per request")
    if V_base.shape != K_base.shape or _vlr_rows(V_lr) != K_base.shape[0] or K_lr.shape[0] != K_base.shape[0] \
            or B.shape[2] != n_kv * d or B_k.shape != B.shape:
        raise ValueError("K_base/V_base/V_lr/K_lr/B/B_k shapes disagree")
    if rope_cos.dtype != torch.float32 or rope_sin.dtype != torch.float32 or rope_cos.device != Q.device \
            or rope_sin.device != Q.device:
        raise ValueError("rope_cos / rope_sin must be float32 tensors on Q's device")
    if rope_cos.shape[0] < max_kv_len or rope_sin.shape[0] < max_kv_len or rope_cos.shape[1:] != (d // 2,) \
            or rope_sin.shape[1:] != (d // 2,):
        raise ValueError("rope tables must be [>= max_kv_len, d/2]")
    need = lra_attn_decode_qkvo_workspace_bytes(batch, n_q, n_kv, d, rank, max_kv_len, keys_per_split)
    if workspace is None and need:
        with _on(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if O is None:
        with _on(stream):
            O = torch.empty_like(Q)
    _same(Q, O)
    _dense("O", O)
    _on_device(Q, rope_cos=rope_cos, rope_sin=rope_sin, kv_start=kv_start, kv_len=kv_len, agent=agent, workspace=workspace)
    _check(_lib.lra_attn_decode_qkvo(_dtype_code(Q), _ptr(Q), batch, _ptr(K_base), _ptr(V_base), K_base.shape[0],
                                     _ptr(V_lr), *_vlr_strides(V_lr, rank), _ptr(K_lr), K_lr.stride(0), _ptr(kv_start), _ptr(kv_len),
                                     max_kv_len, _ptr(B), _ptr(B_k), _ptr(rope_cos), _ptr(rope_sin), n_agents,
                                     _ptr(agent), n_q, n_kv, d, rank, scale, keys_per_split, _ptr(workspace), ws_bytes,
                                     _ptr(O), _stream(stream)), "lra_attn_decode_qkvo")
    return O


# ---------------------------------------------------------------------------------- paged decode
def lra_attn_decode_paged_default_split(batch: int, n_kv: int, max_kv_len: int, page_size: int) -> int:
    return int(_lib.lra_attn_decode_paged_default_split(batch, n_kv, max_kv_len, page_size))


def lra_attn_decode_paged(Q: torch.Tensor, K_pages: torch.Tensor, V_pages: torch.Tensor, Vlr_pages: torch.Tensor,
                          block_table: torch.Tensor, kv_len: torch.Tensor, max_kv_len: int, B: torch.Tensor,
                          agent: torch.Tensor, scale: float, keys_per_split: int = 0,
                          workspace: Optional[torch.Tensor] = None, O: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """lra_attn_decode over a paged cache: request b's row j is row j % P of page block_table[b, j // P].

    Q [batch, n_q, d]; K_pages, V_pages [n_pages, P, n_kv, d]; Vlr_pages [n_pages, P, ld];
    block_table int32 [batch, max_blocks]; kv_len, agent int32 [batch]; B [N, r, n_kv*d]."""
    _same(Q, K_pages, V_pages, Vlr_pages, B)
    for name, t in (("Q", Q), ("K_pages", K_pages), ("V_pages", V_pages), ("B", B)):
        _dense(name, t)
    batch, n_q, d = Q.shape
    n_pages, P, n_kv = K_pages.shape[0], K_pages.shape[1], K_pages.shape[2]
    n_agents, rank = B.shape[0], B.shape[1]
    if V_pages.shape != K_pages.shape or K_pages.shape[3] != d or B.shape[2] != n_kv * d:
        raise ValueError("K_pages/V_pages/B shapes disagree with Q")
    if Vlr_pages.dim() != 3 or Vlr_pages.shape[:2] != (n_pages, P) or Vlr_pages.stride(2) != 1 or \
            Vlr_pages.stride(0) != P * Vlr_pages.stride(1):
        raise ValueError("Vlr_pages must be [n_pages, P, ld] with rows of one page adjacent")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous() or \
            block_table.shape[0] != batch:
        raise TypeError("block_table must be a contiguous int32 [batch, max_blocks] tensor")
    for name, t in (("kv_len", kv_len), ("agent", agent)):
        if t.dtype != torch.int32 or t.shape != (batch,) or not t.is_contiguous() or t.device != Q.device:
            raise TypeError(f"{name} must be a contiguous int32 [batch] tensor on {Q.device}")
    need = lra_attn_decode_workspace_bytes(batch, n_q, n_kv, d, rank, max_kv_len, keys_per_split)
    if workspace is None:
        with _on(stream):
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=Q.device)
    if O is None:
        with _on(stream):
            O = torch.empty_like(Q)
    _same(Q, O)
    _dense("O", O)
    _on_device(Q, block_table=block_table, kv_len=kv_len, agent=agent, workspace=workspace)
    _check(_lib.lra_attn_decode_paged(_dtype_code(Q), _ptr(Q), batch, _ptr(K_pages), _ptr(V_pages), _ptr(Vlr_pages),
                                      n_pages, P, Vlr_pages.stride(1), _ptr(block_table), block_table.shape[1],
                                      _ptr(kv_len), max_kv_len, _ptr(B), n_agents, _ptr(agent), n_q, n_kv, d, rank,
                                      scale, keys_per_split, _ptr(workspace), workspace.numel(), _ptr(O),
                                      _stream(stream)), "lra_attn_decode_paged")
    return O


# ---------------------------------------------------------------------------------- value expansion
def lra_expand_values(V_base: torch.Tensor, V_lr: torch.Tensor, B: torch.Tensor, src_start: torch.Tensor,
                      length: torch.Tensor, agent: torch.Tensor, max_len: int, dst_start: torch.Tensor,
                      V_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Expand-then-attend baseline: V_out[dst_start[b] + t] = V_base[src_start[b] + t]
    + V_lr[src_start[b] + t, agent cols] B[agent[b]] for t < length[b] (a copy for agent -1).

    V_base [rows, n_kv, d]; V_lr [rows, ld]; B [N, r, n_kv*d]; src_start, dst_start int64 [batch];
    length, agent int32 [batch]; V_out [out_rows, n_kv, d] (like V_base when omitted; rows no
    request covers keep their contents, uninitialised when allocated here)."""
    _same(V_base, V_lr, B)
    for name, t in (("V_base", V_base), ("B", B)):
        _dense(name, t)
    _rows_dense("V_lr", V_lr)
    if V_base.dim() != 3:
        raise ValueError("V_base must be [rows, n_kv, d]")
    n_kv, d = V_base.shape[1], V_base.shape[2]
    n_agents, rank = B.shape[0], B.shape[1]
    if V_lr.shape[0] != V_base.shape[0] or B.shape[2] != n_kv * d:
        raise ValueError("V_base/V_lr/B shapes disagree")
    batch = src_start.numel()
    for name, t, dt in (("src_start", src_start, torch.int64), ("dst_start", dst_start, torch.int64),
                        ("length", length, torch.int32), ("agent", agent, torch.int32)):
        if t.dtype != dt or t.numel() != batch or not t.is_contiguous() or t.device != V_base.device:
            raise TypeError(f"{name} must be a contiguous {dt} device tensor with one entry per request")
    if V_out is None:
        with _on(stream):
            V_out = torch.empty_like(V_base)
    _same(V_base, V_out)
    _dense("V_out", V_out)
    if V_out.dim() != 3 or V_out.shape[1:] != V_base.shape[1:]:
        raise ValueError("V_out must be [out_rows, n_kv, d] like V_base")
    _on_device(V_base, src_start=src_start, length=length, agent=agent, dst_start=dst_start)
    _check(_lib.lra_expand_values(_dtype_code(V_base), _ptr(V_base), V_base.shape[0], _ptr(V_lr), V_lr.stride(0),
                                  _ptr(B), n_agents, n_kv, d, rank, batch, _ptr(src_start), _ptr(length),
                                  _ptr(agent), max_len, _ptr(V_out), V_out.shape[0], _ptr(dst_start),
                                  _stream(stream)), "lra_expand_values")
    return V_out


def lra_attn_decode_paged_strided(Q: torch.Tensor, K_pages: torch.Tensor, V_pages: torch.Tensor,
                                  Vlr_pages: torch.Tensor, block_table: torch.Tensor, kv_len: torch.Tensor,
                                  max_kv_len: int, B: torch.Tensor, agent: torch.Tensor, scale: float,
                                  keys_per_split: int = 0, workspace: Optional[torch.Tensor] = None,
                                  O: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """``lra_attn_decode_paged`` over K/V page views [n_pages, P, n_kv, d] of any layout with
    contiguous d-vectors, e.g. ``K_hnd.transpose(1, 2)`` of head-major pages K_hnd [n_pages, n_kv, P, d].
    K_pages and V_pages must have the same strides; Vlr_pages is [n_pages, P, ld] as for the
    token-major call."""
    _same(Q, K_pages, V_pages, Vlr_pages, B)
    for name, t in (("Q", Q), ("B", B)):
        _dense(name, t)
    if K_pages.dim() != 4 or K_pages.stride(3) != 1 or V_pages.shape != K_pages.shape or \
            V_pages.stride() != K_pages.stride():
        raise ValueError("K_pages and V_pages must be [n_pages, P, n_kv, d] views with equal strides")
    batch, n_q, d = Q.shape
    n_pages, P, n_kv = K_pages.shape[0], K_pages.shape[1], K_pages.shape[2]
    n_agents, rank = B.shape[0], B.shape[1]
    if K_pages.shape[3] != d or B.shape[2] != n_kv * d:
        raise ValueError("K_pages/V_pages/B shapes disagree with Q")
    if Vlr_pages.dim() != 3 or Vlr_pages.shape[:2] != (n_pages, P) or Vlr_pages.stride(2) != 1 or \
            Vlr_pages.stride(0) != P * Vlr_pages.stride(1):
        raise ValueError("Vlr_pages must be [n_pages, P, ld] with rows of one page adjacent")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous() or \
            block_table.shape[0] != batch:
        raise TypeError("block_table must be a contiguous int32 [batch, max_blocks] tensor")
    for name, t in (("kv_len", kv_len), ("agent", agent)):
        if t.dtype != torch.int32 or t.shape != (batch,) or not t.is_contiguous() or t.device != Q.device:
            raise TypeError(f"{name} must be a contiguous int32 [batch] tensor on {Q.device}")
    need = lra_attn_decode_workspace_bytes(batch, n_q, n_kv, d, rank, max_kv_len, keys_per_split)
    if workspace is None:
        with _on(stream):
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=Q.device)
    if O is None:
        with _on(stream):
            O = torch.empty_like(Q)
    _same(Q, O)
    _dense("O", O)
    _on_device(Q, block_table=block_table, kv_len=kv_len, agent=agent, workspace=workspace)
    _check(_lib.lra_attn_decode_paged_strided(
        _dtype_code(Q), _ptr(Q), batch, _ptr(K_pages), _ptr(V_pages), _ptr(Vlr_pages), n_pages, P,
        Vlr_pages.stride(1), K_pages.stride(0), K_pages.stride(1), K_pages.stride(2), _ptr(block_table),
        block_table.shape[1], _ptr(kv_len), max_kv_len, _ptr(B), n_agents, _ptr(agent), n_q, n_kv, d, rank, scale,
        keys_per_split, _ptr(workspace), workspace.numel(), _ptr(O), _stream(stream)), "lra_attn_decode_paged_strided")
    return O


def lra_stream_read(x: torch.Tensor, n_workgroups: int, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Reads all of the contiguous device tensor ``x`` (16-byte aligned, a multiple of
    16 * n_workgroups bytes) in n_workgroups contiguous chunks and returns the XOR fold of each
    chunk's 32-bit words (uint32 viewed as int32, [n_workgroups]): a measurement of the streaming
    read bandwidth, the practical ceiling for the decode."""
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    nbytes = x.numel() * x.element_size()
    if out is None:
        with _on(stream):
            out = torch.empty(n_workgroups, dtype=torch.int32, device=x.device)
    _on_device(x, out=out)
    _check(_lib.lra_stream_read(_ptr(x), nbytes, n_workgroups, _ptr(out), _stream(stream)), "lra_stream_read")
    return out
