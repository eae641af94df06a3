"""GPU check of the streaming-read probe: the XOR fold of every 32-bit word is exact."""
import numpy as np
import pytest
import torch

from decode_attention_compressed_quantize_amd import kvc_stream_read_probe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_words", [4, 1 << 10, (1 << 20) + 12, 3 * (1 << 22) + 4])
def test_probe_xor_fold_is_exact(n_words):
    rng = np.random.default_rng(n_words)
    host = rng.integers(0, 2**32, n_words, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc_stream_read_probe(buf, out)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host)
    assert int(out.cpu().numpy().view(np.uint32)[0]) == int(want)
