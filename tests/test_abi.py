"""Host-side tests of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function that include/lra.h declares, and reject every
invalid scalar argument with the documented status before anything is enqueued. Pointers
passed here are fake but 16/256-byte aligned: validation never dereferences them, and every
call below fails validation, so nothing reaches the GPU runtime.
"""
import ctypes
import os
import re
import subprocess

import pytest

import rank_kv_cache_amd as lra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lra.h")

OK, E_NULL, E_SHAPE, E_UNSUP, E_INDEX, E_WS, E_HIP = 0, -1, -2, -3, -4, -5, -6
P = 0x10000  # fake aligned device address (never dereferenced: every call here fails validation)
WS = 0x20000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lra_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_match_binding():
    assert declared_functions() == sorted(lra.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(lra.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", lra.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (lra_[a-z0-9_]+)$", out, flags=re.M))
    assert exported == set(declared_functions())


def test_version_and_status_strings():
    assert lra.abi_version() == 8
    names = {s: lra.status_str(s) for s in (OK, E_NULL, E_SHAPE, E_UNSUP, E_INDEX, E_WS, E_HIP, -99)}
    assert names[OK] == "LRA_OK" and names[E_HIP] == "LRA_ERR_HIP" and names[-99] == "LRA_ERR_UNKNOWN"


# ---------------------------------------------------------------------------------------- decode
def decode(**kw):
    a = dict(dtype=1, Q=P, batch=2, K=P, V=P, kv_rows=100, Vlr=P, ld_vlr=24, vas=8, kv_start=P, kv_len=P,
             max_kv_len=100, B=P, n_agents=3, agent=P, n_q=32, n_kv=8, d=128, r=8, scale=0.088,
             split=0, ws=WS, ws_bytes=1 << 30, O=P, stream=0)
    a.update(kw)
    return lra._lib.lra_attn_decode(a["dtype"], a["Q"], a["batch"], a["K"], a["V"], a["kv_rows"], a["Vlr"], a["ld_vlr"], a["vas"],
                                    a["kv_start"], a["kv_len"], a["max_kv_len"], a["B"], a["n_agents"], a["agent"],
                                    a["n_q"], a["n_kv"], a["d"], a["r"], a["scale"], a["split"], a["ws"],
                                    a["ws_bytes"], a["O"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), E_UNSUP), (dict(d=96), E_UNSUP), (dict(r=4), E_UNSUP), (dict(n_q=36, n_kv=4), E_UNSUP),
    (dict(n_q=30, n_kv=8), E_SHAPE), (dict(n_kv=0), E_SHAPE), (dict(batch=-1), E_SHAPE),
    (dict(ld_vlr=16), E_SHAPE), (dict(ld_vlr=28), E_SHAPE), (dict(split=100), E_SHAPE), (dict(split=-64), E_SHAPE),
    # V_lr layouts: interleaved needs an agent stride of rank, agent-major one of at least kv_rows x ld_vlr
    (dict(vas=16), E_SHAPE), (dict(vas=12), E_SHAPE), (dict(vas=0), E_SHAPE), (dict(ld_vlr=8, vas=792), E_SHAPE),
    (dict(ld_vlr=4, vas=800), E_SHAPE),
    (dict(max_kv_len=-1), E_SHAPE), (dict(kv_rows=-5), E_SHAPE), (dict(n_agents=0), E_SHAPE),
    (dict(scale=float("nan")), E_SHAPE), (dict(scale=0.0), E_SHAPE), (dict(scale=-0.1), E_SHAPE), (dict(Q=None), E_NULL), (dict(kv_len=None), E_NULL),
    (dict(agent=None), E_NULL), (dict(O=None), E_NULL), (dict(K=P + 8), E_SHAPE),
    (dict(ws=None), E_WS), (dict(ws=WS + 64), E_WS), (dict(ws_bytes=16), E_WS),
    (dict(max_kv_len=1 << 31), E_SHAPE),
])
def test_decode_rejects_bad_arguments(kw, status):
    assert decode(**kw) == status
    assert lra._lib.lra_last_error().decode() != ""


def decode_qkvo(**kw):
    a = dict(dtype=1, Q=P, batch=2, K=P, V=P, kv_rows=100, Vlr=P, ld_vlr=24, vas=8, Klr=P, ld_klr=24, kv_start=P, kv_len=P,
             max_kv_len=100, B=P, Bk=P, cos=P, sin=P, n_agents=3, agent=P, n_q=32, n_kv=8, d=128, r=8, scale=0.088,
             split=0, ws=WS, ws_bytes=16, O=P, stream=0)
    a.update(kw)
    return lra._lib.lra_attn_decode_qkvo(a["dtype"], a["Q"], a["batch"], a["K"], a["V"], a["kv_rows"], a["Vlr"],
                                         a["ld_vlr"], a["vas"], a["Klr"], a["ld_klr"], a["kv_start"], a["kv_len"], a["max_kv_len"],
                                         a["B"], a["Bk"], a["cos"], a["sin"], a["n_agents"], a["agent"], a["n_q"],
                                         a["n_kv"], a["d"], a["r"], a["scale"], a["split"], a["ws"], a["ws_bytes"],
                                         a["O"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=0), E_UNSUP), (dict(d=96), E_UNSUP), (dict(r=4), E_UNSUP), (dict(n_q=30, n_kv=8), E_SHAPE),
    (dict(ld_klr=16), E_SHAPE), (dict(ld_klr=30), E_SHAPE), (dict(ld_vlr=16), E_SHAPE), (dict(split=100), E_SHAPE),
    (dict(max_kv_len=(1 << 24) + 1), E_SHAPE), (dict(scale=0.0), E_SHAPE),
    (dict(Klr=None), E_NULL), (dict(Bk=None), E_NULL), (dict(cos=None), E_NULL), (dict(sin=None), E_NULL),
    (dict(agent=None), E_NULL), (dict(cos=P + 4), E_SHAPE), (dict(Klr=P + 8), E_SHAPE),
    (dict(ws=None), E_WS), (dict(ws=WS + 64, ws_bytes=1 << 30), E_WS), (dict(ws_bytes=16), E_WS),
])
def test_decode_qkvo_rejects_bad_arguments(kw, status):
    assert decode_qkvo(**kw) == status


def test_decode_qkvo_workspace_size():
    # the decode workspace, 256-aligned, then fp32 key scores [batch x n_q x round_up(max_kv_len, 64)],
    # fp16 score weights [batch x n_q x d_head*rank], the repacked rotary tables, and one int32 flag
    # per workgroup of the score pass [batch x ceil(max_kv_len / 512) x ceil(n_q / 32)]
    plain = lra.lra_attn_decode_workspace_bytes(16, 32, 8, 128, 8, 66400, 0)
    need = lra.lra_attn_decode_qkvo_workspace_bytes(16, 32, 8, 128, 8, 66400, 0)
    assert need == (plain + 255) // 256 * 256 + 16 * 32 * 66432 * 4 + 16 * 32 * 1024 * 2 + 4150 * 32 * 128 + 16 * 130 * 4
    # (2 slices (one per tile) + 2 requests) x 2 KV heads = 8 record blocks of 4 x (64/4 + 8/4 + 1)
    # = 76 slots of 16 bytes, padded to 80, 2 x 4 x 64 fp32 scores, 2 x 4 x 512 fp16 weights,
    # 2 tiles of 16 steps x 128 bytes of repacked tables, 2 flags
    assert lra.lra_attn_decode_qkvo_workspace_bytes(2, 4, 2, 64, 8, 1, 64) == \
        8 * 80 * 16 + 2 * 4 * 64 * 4 + 2 * 4 * 512 * 2 + 2 * 16 * 128 + 2 * 4
    assert decode_qkvo(ws=WS, ws_bytes=lra.lra_attn_decode_qkvo_workspace_bytes(2, 32, 8, 128, 8, 100, 0) - 1) == E_WS
    assert decode_qkvo(batch=0, Q=None, O=None) == OK


def decode_step(**kw):
    a = dict(dtype=1, Q=P, batch=2, K=P, V=P, kv_rows=100, Vlr=P, ld_vlr=24, vas=8, kv_start=P, kv_len=P,
             max_kv_len=100, B=P, n_agents=3, agent=P, n_q=32, n_kv=8, d=128, r=8, scale=0.088,
             X=P, ldx=4096, A=P, d_model=4096, split=0, ws=WS, ws_bytes=1 << 30, O=P, stream=0)
    a.update(kw)
    return lra._lib.lra_attn_decode_step(a["dtype"], a["Q"], a["batch"], a["K"], a["V"], a["kv_rows"], a["Vlr"],
                                         a["ld_vlr"], a["vas"], a["kv_start"], a["kv_len"], a["max_kv_len"], a["B"],
                                         a["n_agents"], a["agent"], a["n_q"], a["n_kv"], a["d"], a["r"], a["scale"],
                                         a["X"], a["ldx"], a["A"], a["d_model"], a["split"], a["ws"], a["ws_bytes"],
                                         a["O"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(d_model=4000), E_SHAPE), (dict(d_model=0), E_SHAPE), (dict(ldx=4088), E_SHAPE), (dict(ldx=4100), E_SHAPE),
    (dict(X=None), E_NULL), (dict(A=None), E_NULL), (dict(X=P + 8), E_SHAPE), (dict(A=P + 4), E_SHAPE),
    (dict(dtype=2), E_UNSUP), (dict(n_q=30), E_SHAPE), (dict(ws=None), E_WS), (dict(ws_bytes=16), E_WS),
])
def test_decode_step_rejects_bad_arguments(kw, status):
    assert decode_step(**kw) == status


def test_decode_empty_batch_is_a_no_op():
    assert decode(batch=0, Q=None, ws=None, ws_bytes=0) == OK


def test_decode_workspace_size_follows_slices():
    """The batch's 32-key tiles are cut into n slices (a multiple of 8): about keys_per_split keys
    each at full lengths, or by default one round of 15/16 of the chip's 8-wave workgroup slots
    (240 slices at n_kv <= 8, 120 per group of 8 KV heads at n_kv = 16), and at most one slice
    per tile; the workspace holds the most that max_kv_len allows. A slice holds one piece of each
    request it touches, with its own record per query head: (n + batch) * n_q records of (m, l)
    and (O, O_lr), in blocks per KV head."""
    b, n_q, d, r = 16, 32, 128, 8

    def layout(n_slices, batch=b, n_kv=8):
        # one block per (slice + request, KV head) of 16-byte slots: O (d/16 x 4 x 4
        # heads), O_lr (4 heads x r/4), (m, l) (4 heads); group size n_q/n_kv rounded up to 4 or 8
        gp = 4 if n_q // n_kv <= 4 else 8
        slots = -(-gp * (d // 4 + r // 4 + 1) // 16) * 16   # padded to whole 256-byte runs
        return (n_slices + batch) * n_kv * slots * 16

    assert lra.lra_attn_decode_workspace_bytes(b, n_q, 8, d, r, 66400, 0) == layout(240)
    assert lra.lra_attn_decode_workspace_bytes(b, n_q, 4, d, r, 66400, 0) == layout(240, n_kv=4)
    assert lra.lra_attn_decode_workspace_bytes(b, n_q, 16, d, r, 66400, 0) == layout(120, n_kv=16)
    assert lra.lra_attn_decode_workspace_bytes(1, n_q, 8, d, r, 1900, 0) == layout(60, 1)   # 60 tiles: one each
    assert lra.lra_attn_decode_workspace_bytes(b, n_q, 8, d, r, 66400, 1024) == layout(1040)   # ceil(16 * 66400 / 1024) = 1038 -> 1040
    assert lra.lra_attn_decode_workspace_bytes(b, n_q, 8, d, r, 0, 0) == 0
    assert lra.lra_attn_decode_workspace_bytes(b, n_q, 8, d, r, 100, 65) == 0
    # the default keys per slice at full lengths: 16 x 66,400 keys over 240 slices; 4 x 66,400
    # over 240; one 1,900-key request (60 tiles) over 60 slices of one tile each
    assert lra.lra_attn_decode_default_split(16, 8, 66400) == 4480   # 4,426.7 rounded up to a multiple of 64
    assert lra.lra_attn_decode_default_split(4, 8, 66400) == 1152    # 1,106.7 -> 1,152
    assert lra.lra_attn_decode_default_split(1, 8, 1900) == 64
    assert lra.lra_attn_decode_default_split(1, 1, 1900) == 64
    assert lra.lra_attn_decode_default_split(0, 8, 1900) == 0


# ---------------------------------------------------------------------------------------- prefill
def prefill(**kw):
    a = dict(dtype=1, Q=P, L_C=64, L_P=192, K=P, V=P, Vlr=P, ld_vlr=24, vas=8, B=P, n_agents=3, agent=0,
             n_q=4, n_kv=2, d=64, r=8, scale=0.125, O=P, stream=0)
    a.update(kw)
    return lra._lib.lra_attn_prefill(a["dtype"], a["Q"], a["L_C"], a["L_P"], a["K"], a["V"], a["Vlr"], a["ld_vlr"], a["vas"],
                                     a["B"], a["n_agents"], a["agent"], a["n_q"], a["n_kv"], a["d"], a["r"],
                                     a["scale"], a["O"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=-1), E_UNSUP), (dict(d=32), E_UNSUP), (dict(r=32), E_UNSUP), (dict(n_q=3), E_SHAPE),
    (dict(L_C=-1), E_SHAPE), (dict(L_P=-1), E_SHAPE), (dict(L_P=1 << 31), E_SHAPE), (dict(agent=3), E_INDEX),
    (dict(agent=-2), E_INDEX), (dict(n_agents=0), E_SHAPE), (dict(ld_vlr=8), E_SHAPE), (dict(scale=float("inf")), E_SHAPE),
    (dict(scale=0.0), E_SHAPE), (dict(scale=-1.0), E_SHAPE),
    (dict(B=None), E_NULL), (dict(Vlr=None), E_NULL), (dict(O=P + 2), E_SHAPE),
])
def test_prefill_rejects_bad_arguments(kw, status):
    assert prefill(**kw) == status


def test_prefill_accepts_the_adapter_free_view():
    # agent -1 passes the index check; the ld_vlr check that follows it then fails, so nothing launches
    assert prefill(agent=lra.ADAPTER_FREE, ld_vlr=8) == E_SHAPE
    assert prefill(agent=-2, ld_vlr=8) == E_INDEX


def prefill_varlen(**kw):
    a = dict(dtype=1, Q=P, q_rows=100, batch=3, q_start=P, q_len=P, max_q_len=64, K=P, V=P, kv_rows=500, Vlr=P,
             ld_vlr=24, vas=8, kv_start=P, kv_prefix=P, B=P, n_agents=3, agent=P, n_q=32, n_kv=8, d=128, r=8, scale=0.088,
             O=P, stream=0)
    a.update(kw)
    return lra._lib.lra_attn_prefill_varlen(a["dtype"], a["Q"], a["q_rows"], a["batch"], a["q_start"], a["q_len"],
                                            a["max_q_len"], a["K"], a["V"], a["kv_rows"], a["Vlr"], a["ld_vlr"], a["vas"],
                                            a["kv_start"], a["kv_prefix"], a["B"], a["n_agents"], a["agent"], a["n_q"],
                                            a["n_kv"], a["d"], a["r"], a["scale"], a["O"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=-1), E_UNSUP), (dict(d=32), E_UNSUP), (dict(r=32), E_UNSUP), (dict(n_q=3), E_SHAPE),
    (dict(batch=-1), E_SHAPE), (dict(q_rows=-1), E_SHAPE), (dict(kv_rows=-1), E_SHAPE), (dict(max_q_len=-1), E_SHAPE),
    (dict(max_q_len=1 << 31), E_SHAPE), (dict(n_agents=0), E_SHAPE), (dict(ld_vlr=8), E_SHAPE),
    (dict(scale=0.0), E_SHAPE), (dict(scale=float("nan")), E_SHAPE),
    (dict(q_start=None), E_NULL), (dict(q_len=None), E_NULL), (dict(kv_start=None), E_NULL),
    (dict(kv_prefix=None), E_NULL), (dict(agent=None), E_NULL), (dict(B=None), E_NULL), (dict(O=P + 2), E_SHAPE),
])
def test_prefill_varlen_rejects_bad_arguments(kw, status):
    assert prefill_varlen(**kw) == status


def test_prefill_varlen_empty_batch_is_a_no_op():
    assert prefill_varlen(batch=0, Q=None, O=None, q_start=None) == OK
    assert prefill_varlen(max_q_len=0, Q=None, O=None) == OK


def test_prefill_empty_chunk_is_a_no_op():
    assert prefill(L_C=0, Q=None, O=None) == OK


def prefill_qkvo(**kw):
    a = dict(dtype=1, Q=P, L_C=64, L_P=192, K=P, V=P, Vlr=P, ld_vlr=24, vas=8, Klr=P, ld_klr=24, B=P, Bk=P, cos=P, sin=P,
             n_agents=3, agent=0, n_q=4, n_kv=2, d=64, r=8, scale=0.125, ws=None, ws_bytes=0, O=P, stream=0)
    a.update(kw)
    return lra._lib.lra_attn_prefill_qkvo(a["dtype"], a["Q"], a["L_C"], a["L_P"], a["K"], a["V"], a["Vlr"],
                                          a["ld_vlr"], a["vas"], a["Klr"], a["ld_klr"], a["B"], a["Bk"], a["cos"], a["sin"],
                                          a["n_agents"], a["agent"], a["n_q"], a["n_kv"], a["d"], a["r"], a["scale"],
                                          a["ws"], a["ws_bytes"], a["O"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=0), E_UNSUP), (dict(dtype=-1), E_UNSUP), (dict(d=32), E_UNSUP), (dict(r=32), E_UNSUP),
    (dict(n_q=3), E_SHAPE), (dict(L_C=-1), E_SHAPE), (dict(agent=3), E_INDEX), (dict(agent=-2), E_INDEX),
    (dict(ld_vlr=8), E_SHAPE), (dict(ld_klr=8), E_SHAPE), (dict(ld_klr=28), E_SHAPE), (dict(scale=0.0), E_SHAPE),
    (dict(Klr=None), E_NULL), (dict(Bk=None), E_NULL), (dict(cos=None), E_NULL), (dict(sin=None), E_NULL),
    (dict(B=None), E_NULL), (dict(cos=P + 4), E_SHAPE), (dict(Klr=P + 8), E_SHAPE), (dict(O=P + 2), E_SHAPE),
    (dict(ws=None), E_WS), (dict(ws=WS + 64, ws_bytes=1 << 30), E_WS), (dict(ws=WS, ws_bytes=1000), E_WS),
])
def test_prefill_qkvo_rejects_bad_arguments(kw, status):
    assert prefill_qkvo(**kw) == status


def test_prefill_qkvo_empty_chunk_is_a_no_op():
    assert prefill_qkvo(L_C=0, Q=None, O=None, Klr=None) == OK


def test_prefill_qkvo_workspace_size():
    # fp16 expanded keys (256-byte aligned part), then the largest |key| (fp32) per (64-key tile, KV head)
    assert lra.lra_attn_prefill_qkvo_workspace_bytes(18432, 8, 128) == 18432 * 8 * 128 * 2 + 288 * 8 * 4
    assert lra.lra_attn_prefill_qkvo_workspace_bytes(65, 2, 64) == 65 * 2 * 64 * 2 + 2 * 2 * 4
    assert lra.lra_attn_prefill_qkvo_workspace_bytes(3, 1, 64) == 512 + 4
    assert lra.lra_attn_prefill_qkvo_workspace_bytes(0, 8, 128) == 0
    # one byte short of the size is refused
    need = lra.lra_attn_prefill_qkvo_workspace_bytes(256, 2, 64)
    assert prefill_qkvo(ws=WS, ws_bytes=need - 1) == E_WS


# ---------------------------------------------------------------------------------------- precompute
def precompute(**kw):
    a = dict(dtype=1, X=P, T=2048, d_model=4096, ldx=4096, A=P, n_agents=3, r=8, Vlr=P, ld_vlr=24, vas=8,
             vlr_rows=18432, out_rows=None, ws=WS, ws_bytes=1 << 30, stream=0)
    a.update(kw)
    return lra._lib.lra_lr_precompute(a["dtype"], a["X"], a["T"], a["d_model"], a["ldx"], a["A"], a["n_agents"],
                                      a["r"], a["Vlr"], a["ld_vlr"], a["vas"], a["vlr_rows"], a["out_rows"], a["ws"],
                                      a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), E_UNSUP), (dict(d_model=4004), E_UNSUP), (dict(n_agents=3, r=3), E_UNSUP),
    (dict(T=-1), E_SHAPE), (dict(ldx=4095), E_SHAPE), (dict(ldx=4092), E_SHAPE), (dict(ld_vlr=20), E_SHAPE),
    (dict(vas=16), E_SHAPE), (dict(ld_vlr=8, vas=8 * 2047), E_SHAPE),
    (dict(vlr_rows=100), E_SHAPE), (dict(vlr_rows=-1, out_rows=P), E_SHAPE), (dict(n_agents=0), E_SHAPE),
    (dict(X=None), E_NULL), (dict(A=None), E_NULL), (dict(Vlr=P + 4), E_SHAPE),
])
def test_precompute_rejects_bad_arguments(kw, status):
    assert precompute(**kw) == status


def test_precompute_empty_is_a_no_op():
    assert precompute(T=0, X=None, ws=None, ws_bytes=0) == OK


def test_precompute_needs_no_workspace():
    # one launch: each workgroup sums its 16 waves' partials itself, so no partials leave it
    for T, d_model, n_agents, r in ((2048, 4096, 3, 8), (8192, 4096, 3, 8), (32, 4096, 3, 16), (1, 256, 3, 8),
                                    (0, 4096, 3, 8), (18432, 8192, 3, 8)):
        assert lra.lra_lr_precompute_workspace_bytes(T, d_model, n_agents, r) == 0
    assert precompute(T=32, ws=None, ws_bytes=0, X=P, A=P, Vlr=None) == E_NULL   # validation still runs


# ---------------------------------------------------------------------------------------- paged decode
def decode_paged(**kw):
    a = dict(dtype=1, Q=P, batch=4, K=P, V=P, Vlr=P, n_pages=100, P=64, ld_vlr=24, table=P, max_blocks=10, kv_len=P,
             max_kv_len=600, B=P, n_agents=3, agent=P, n_q=32, n_kv=8, d=128, r=8, scale=0.088, split=0, ws=P,
             ws_bytes=1 << 30, O=P, stream=0)
    a.update(kw)
    return lra._lib.lra_attn_decode_paged(a["dtype"], a["Q"], a["batch"], a["K"], a["V"], a["Vlr"], a["n_pages"],
                                          a["P"], a["ld_vlr"], a["table"], a["max_blocks"], a["kv_len"], a["max_kv_len"],
                                          a["B"], a["n_agents"], a["agent"], a["n_q"], a["n_kv"], a["d"], a["r"],
                                          a["scale"], a["split"], a["ws"], a["ws_bytes"], a["O"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(P=48), E_UNSUP), (dict(P=16), E_UNSUP), (dict(P=1 << 17), E_UNSUP), (dict(n_pages=0), E_SHAPE),
    (dict(max_blocks=0), E_SHAPE), (dict(max_kv_len=641), E_SHAPE), (dict(max_kv_len=-1), E_SHAPE),
    (dict(split=100), E_SHAPE), (dict(batch=-1), E_SHAPE),
    (dict(n_agents=0), E_SHAPE), (dict(ld_vlr=8), E_SHAPE), (dict(scale=0.0), E_SHAPE), (dict(d=32), E_UNSUP),
    (dict(table=None), E_NULL), (dict(kv_len=None), E_NULL), (dict(agent=None), E_NULL), (dict(Vlr=None), E_NULL),
    (dict(ws=None), E_WS), (dict(ws_bytes=16), E_WS), (dict(O=P + 4), E_SHAPE),
])
def test_decode_paged_rejects_bad_arguments(kw, status):
    assert decode_paged(**kw) == status


def test_decode_paged_empty_batch_is_a_no_op():
    assert decode_paged(batch=0, Q=None, O=None, ws=None) == OK


def test_decode_paged_default_split_is_the_contiguous_one():
    for P in (32, 64, 128, 1024):
        for batch, L in ((1, 1900), (16, 66400), (64, 131072), (1, 10 ** 6)):
            assert lra.lra_attn_decode_paged_default_split(batch, 8, L, P) == lra.lra_attn_decode_default_split(batch, 8, L)
    assert lra.lra_attn_decode_paged_default_split(16, 8, 66400, 48) == 0


# ---------------------------------------------------------------------------------------- paged prefill
def prefill_paged(**kw):
    a = dict(dtype=1, Q=P, q_rows=100, batch=3, q_start=P, q_len=P, max_q_len=64, K=P, V=P, Vlr=P, n_pages=50, P=64,
             ld_vlr=24, table=P, max_blocks=8, kv_prefix=P, B=P, n_agents=3, agent=P, n_q=32, n_kv=8, d=128, r=8,
             scale=0.088, O=P, stream=0)
    a.update(kw)
    return lra._lib.lra_attn_prefill_paged(a["dtype"], a["Q"], a["q_rows"], a["batch"], a["q_start"], a["q_len"],
                                           a["max_q_len"], a["K"], a["V"], a["Vlr"], a["n_pages"], a["P"], a["ld_vlr"],
                                           a["table"], a["max_blocks"], a["kv_prefix"], a["B"], a["n_agents"],
                                           a["agent"], a["n_q"], a["n_kv"], a["d"], a["r"], a["scale"], a["O"],
                                           a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(P=32), E_UNSUP), (dict(P=96), E_UNSUP), (dict(P=1 << 17), E_UNSUP), (dict(n_pages=0), E_SHAPE),
    (dict(max_blocks=0), E_SHAPE), (dict(batch=-1), E_SHAPE), (dict(q_rows=-1), E_SHAPE), (dict(max_q_len=-1), E_SHAPE),
    (dict(n_agents=0), E_SHAPE), (dict(ld_vlr=8), E_SHAPE), (dict(scale=-1.0), E_SHAPE), (dict(r=4), E_UNSUP),
    (dict(table=None), E_NULL), (dict(kv_prefix=None), E_NULL), (dict(q_start=None), E_NULL), (dict(Vlr=None), E_NULL),
    (dict(O=P + 2), E_SHAPE),
])
def test_prefill_paged_rejects_bad_arguments(kw, status):
    assert prefill_paged(**kw) == status


def test_prefill_paged_empty_batch_is_a_no_op():
    assert prefill_paged(batch=0, Q=None, O=None, table=None) == OK


# ---------------------------------------------------------------------------------------- value expansion
def expand(**kw):
    a = dict(dtype=1, V=P, kv_rows=100, Vlr=P, ld_vlr=24, B=P, n_agents=3, n_kv=8, d=128, r=8, batch=2,
             src=P, len=P, agent=P, max_len=100, out=P, out_rows=100, dst=P, stream=0)
    a.update(kw)
    return lra._lib.lra_expand_values(a["dtype"], a["V"], a["kv_rows"], a["Vlr"], a["ld_vlr"], a["B"], a["n_agents"],
                                      a["n_kv"], a["d"], a["r"], a["batch"], a["src"], a["len"], a["agent"],
                                      a["max_len"], a["out"], a["out_rows"], a["dst"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), E_UNSUP), (dict(d=96), E_UNSUP), (dict(r=4), E_UNSUP), (dict(n_kv=0), E_SHAPE),
    (dict(n_agents=0), E_SHAPE), (dict(batch=-1), E_SHAPE), (dict(kv_rows=-1), E_SHAPE), (dict(out_rows=-1), E_SHAPE),
    (dict(max_len=-1), E_SHAPE), (dict(max_len=1 << 31), E_SHAPE), (dict(ld_vlr=16), E_SHAPE), (dict(ld_vlr=28), E_SHAPE),
    (dict(batch=1 << 20, max_len=1 << 20), E_SHAPE),
    (dict(V=None), E_NULL), (dict(Vlr=None), E_NULL), (dict(B=None), E_NULL), (dict(out=None), E_NULL),
    (dict(src=None), E_NULL), (dict(len=None), E_NULL), (dict(agent=None), E_NULL), (dict(dst=None), E_NULL),
    (dict(V=P + 8), E_SHAPE), (dict(out=P + 2), E_SHAPE),
])
def test_expand_values_rejects_bad_arguments(kw, status):
    assert expand(**kw) == status
    assert lra._lib.lra_last_error().decode() != ""


def test_expand_values_empty_is_a_no_op():
    assert expand(batch=0, V=None, out=None, src=None) == OK
    assert expand(max_len=0, V=None, out=None, src=None) == OK


# ---------------------------------------------------------------------------------------- strided decode
def decode_strided(**kw):
    a = dict(dtype=1, Q=P, batch=2, K=P, V=P, kv_rows=100, rs=128, hs=12800, Vlr=P, ld_vlr=24, vas=8, kv_start=P, kv_len=P,
             max_kv_len=100, B=P, n_agents=3, agent=P, n_q=32, n_kv=8, d=128, r=8, scale=0.088, split=0, ws=WS,
             ws_bytes=1 << 30, O=P, stream=0)
    a.update(kw)
    return lra._lib.lra_attn_decode_strided(a["dtype"], a["Q"], a["batch"], a["K"], a["V"], a["kv_rows"], a["rs"],
                                            a["hs"], a["Vlr"], a["ld_vlr"], a["vas"], a["kv_start"], a["kv_len"],
                                            a["max_kv_len"], a["B"], a["n_agents"], a["agent"], a["n_q"], a["n_kv"],
                                            a["d"], a["r"], a["scale"], a["split"], a["ws"], a["ws_bytes"], a["O"],
                                            a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(rs=0), E_SHAPE), (dict(hs=-128), E_SHAPE), (dict(rs=100), E_SHAPE), (dict(hs=12), E_SHAPE),
    (dict(rs=(1 << 24) + 8), E_SHAPE), (dict(d=96), E_UNSUP), (dict(r=4), E_UNSUP), (dict(n_q=30), E_SHAPE),
    (dict(ld_vlr=16), E_SHAPE), (dict(split=100), E_SHAPE), (dict(scale=0.0), E_SHAPE), (dict(K=None), E_NULL),
    (dict(agent=None), E_NULL), (dict(V=P + 8), E_SHAPE), (dict(ws=None), E_WS), (dict(ws_bytes=16), E_WS),
])
def test_decode_strided_rejects_bad_arguments(kw, status):
    assert decode_strided(**kw) == status
    assert lra._lib.lra_last_error().decode() != ""


def test_decode_strided_empty_batch_is_a_no_op():
    assert decode_strided(batch=0, Q=None, O=None, K=None) == OK


# ---------------------------------------------------------------------------------------- strided paged decode
def decode_paged_strided(**kw):
    a = dict(dtype=1, Q=P, batch=4, K=P, V=P, Vlr=P, n_pages=100, P=64, ld_vlr=24, ps=65536, rs=128, hs=8192,
             table=P, max_blocks=10, kv_len=P, max_kv_len=600, B=P, n_agents=3, agent=P, n_q=32, n_kv=8, d=128, r=8,
             scale=0.088, split=0, ws=P, ws_bytes=1 << 30, O=P, stream=0)
    a.update(kw)
    return lra._lib.lra_attn_decode_paged_strided(
        a["dtype"], a["Q"], a["batch"], a["K"], a["V"], a["Vlr"], a["n_pages"], a["P"], a["ld_vlr"], a["ps"], a["rs"],
        a["hs"], a["table"], a["max_blocks"], a["kv_len"], a["max_kv_len"], a["B"], a["n_agents"], a["agent"],
        a["n_q"], a["n_kv"], a["d"], a["r"], a["scale"], a["split"], a["ws"], a["ws_bytes"], a["O"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(ps=0), E_SHAPE), (dict(rs=-8), E_SHAPE), (dict(hs=12), E_SHAPE), (dict(ps=65540), E_SHAPE),
    (dict(rs=(1 << 24) + 8), E_SHAPE), (dict(P=48), E_UNSUP), (dict(d=96), E_UNSUP), (dict(n_pages=0), E_SHAPE),
    (dict(max_kv_len=641), E_SHAPE), (dict(table=None), E_NULL),
    (dict(K=P + 8), E_SHAPE), (dict(ws=None), E_WS), (dict(ws_bytes=16), E_WS),
])
def test_decode_paged_strided_rejects_bad_arguments(kw, status):
    assert decode_paged_strided(**kw) == status
    assert lra._lib.lra_last_error().decode() != ""


def test_decode_paged_strided_empty_batch_is_a_no_op():
    assert decode_paged_strided(batch=0, Q=None, O=None, table=None) == OK


# ------------------------------------------------------------------------------ binding argument checks
def test_binding_rejects_host_tensors_before_any_launch():
    """The kernels take device pointers: host tensors (data, index tables) are refused by the binding
    with a ValueError, before the library is called."""
    import torch
    Q = torch.zeros(2, 4, 64)
    K = torch.zeros(10, 2, 64)
    Vlr = torch.zeros(10, 24)
    B = torch.zeros(3, 8, 128)
    idx64, idx32 = torch.zeros(2, dtype=torch.int64), torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        lra.lra_attn_decode(Q, K, K, Vlr, idx64, idx32, 10, B, idx32, 0.125)
    with pytest.raises(ValueError, match="GPU"):
        lra.lra_attn_prefill(Q, 8, K, K, Vlr, B, 0, 0.125)
    with pytest.raises(ValueError, match="GPU"):
        lra.lra_lr_precompute(torch.zeros(4, 64), torch.zeros(24, 64), 3, 8, Vlr)


@pytest.mark.parametrize("x,nbytes,n_wg,out,status", [
    (None, 1 << 20, 16, P, E_NULL), (P, 1 << 20, 16, None, E_NULL), (P + 8, 1 << 20, 16, P, E_SHAPE),
    (P, 1 << 20, 0, P, E_SHAPE), (P, 1 << 20, (1 << 20) + 1, P, E_SHAPE), (P, 0, 16, P, E_SHAPE),
    (P, (1 << 20) + 16, 16, P, E_SHAPE), (P, 16 * 15, 16, P, E_SHAPE),
])
def test_stream_read_rejects_bad_arguments(x, nbytes, n_wg, out, status):
    assert lra._lib.lra_stream_read(x, nbytes, n_wg, out, 0) == status



def test_prefill_rejects_rows_beyond_32_bit_tile_offsets():
    """n_kv*d_head or ld_vlr above 2^22: the contiguous prefill reads 64-row tiles through 32-bit
    buffer offsets, so the host refuses them (before any pointer is used)."""
    assert prefill(n_q=32769, n_kv=32769, d=128) == E_SHAPE           # n_kv*d_head = 2^22 + 128
    assert prefill(ld_vlr=(1 << 22) + 8, vas=8) == E_SHAPE
