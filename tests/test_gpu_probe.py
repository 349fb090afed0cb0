"""The plain-read probe (a measurement helper): every 16-byte word of the buffer is read
exactly once, whatever the grid.  The xor of all the words the threads write equals the
xor of the buffer's 32-bit words."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,grid", [(16, 1), (4096, 7), (1 << 20, 512), (3 << 20, 2048),
                                         (1000016, 1024)])
def test_read_probe_reads_every_word_once(nbytes, grid):
    from mla_latent_kv_attention_amd import read_probe as mla
    rng = np.random.default_rng(nbytes + grid)
    words = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).to("cuda:0")
    sink = torch.full((grid * 256,), -1, dtype=torch.int32, device="cuda:0")
    print("probe", nbytes, grid, flush=True)
    mla.hbm_read_probe(src, sink, grid=grid)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
