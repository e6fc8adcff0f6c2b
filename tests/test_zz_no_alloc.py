"""lra_attn_decode_noalloc (partials in the library's static device array) against lra_attn_decode
(caller's workspace): two calls in a row, the second smaller, each bit-identical to the workspace
call with the same split and within the bf16 tolerance of the oracle."""
import numpy as np
import pytest
import torch

import oracle
import rank_kv_cache_amd as lra
import workloads as W
from tests.gpu_util import check, dev, dev_idx, host64, say

pytestmark = pytest.mark.gpu


def _args(c: W.DecodeBatch):
    return (dev(c.Q), dev(c.K), dev(c.V), dev(c.V_lr), dev_idx(c.kv_start, torch.int64), dev_idx(c.kv_len, torch.int32),
            c.max_kv_len, dev(c.B), dev_idx(c.agent, torch.int32), c.shape.scale)


def _ref(c: W.DecodeBatch):
    return oracle.attn_decode(c.Q.as_f64(), c.K.as_f64(), c.V.as_f64(), c.V_lr.as_f64(), c.B.as_f64(), c.kv_start,
                              c.kv_len, c.agent, c.shape.scale)


def test_noalloc_matches_workspace_call_twice_second_smaller():
    s = W.LLAMA_SHAPE
    big = W.random_decode((901,), s, kv_lens=[3000, 1900, 77, 0, 2500, 1], agents=[0, 2, 1, 0, -1, 2])
    small = W.random_decode((902,), s, kv_lens=[300, 5], agents=[1, 0])
    for name, c, split in (("large", big, 0), ("small", small, 128)):
        a = _args(c)
        say(f"noalloc decode {name}: workspace call")
        O_ws = lra.lra_attn_decode(*a, keys_per_split=split)
        say(f"noalloc decode {name}: static scratch")
        O_na = torch.full_like(O_ws, float("nan"))
        lra.lra_attn_decode_noalloc(*a, O_na, keys_per_split=split)
        torch.cuda.synchronize()
        assert torch.equal(O_na, O_ws), f"{name}: outputs differ from the workspace call"
        check(host64(O_na), _ref(c), "bf16", f"noalloc {name}")


def test_noalloc_rejects_sizes_beyond_its_array():
    s = W.LLAMA_SHAPE
    c = W.random_decode((903,), s, kv_lens=[64], agents=[0])
    a = list(_args(c))
    a[6] = 1 << 30   # max_kv_len: the partials of the largest split count would not fit
    O = torch.empty_like(a[0])
    need = lra.lra_attn_decode_workspace_bytes(1, s.n_q, s.n_kv, s.d_head, s.rank, 1 << 30, 128)
    assert need > lra.NOALLOC_SCRATCH_BYTES
    with pytest.raises(lra.LraError, match="static"):
        lra.lra_attn_decode_noalloc(*a, O, keys_per_split=128)
