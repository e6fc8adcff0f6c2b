"""GPU check of the streaming-read probe: each chunk's XOR fold against NumPy's (needs an MI355X)."""
import numpy as np
import pytest
import torch

import rank_kv_cache_amd as lra
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_words,n_wg", [(4 * 16, 1), (4 * 512 * 8 * 3, 2), (1 << 22, 64), (5 * 4 * 512 * 8 * 7 + 4 * 40, 5)])
def test_stream_read_folds_every_word(n_words, n_wg):
    rng = np.random.default_rng(n_words)
    words = rng.integers(0, 2**32, size=n_words, dtype=np.uint64).astype(np.uint32)
    say(f"stream read {n_words} words over {n_wg} workgroups")
    x = torch.from_numpy(words.view(np.int32)).cuda()
    got = lra.lra_stream_read(x, n_wg).cpu().numpy().view(np.uint32)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(words.reshape(n_wg, -1), axis=1)
    assert np.array_equal(got, want)
