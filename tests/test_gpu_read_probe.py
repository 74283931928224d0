"""The plain read probe (a measurement aid): every tile it is given is read exactly once,
also when one or two waves read hundreds of tiles each (1 KB tiles: 341 or 171 per wave).

Each lane XOR-folds the 32-bit words it reads into its sink word, so the XOR of all sink
words equals the XOR of every word of every tile read, a value the host computes from the
buffer's contents."""
import numpy as np
import pytest

from gpu_util import torch_mod

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("tile_bytes,workgroups", [(4096, 8), (2048, 3), (1024, 5), (65536, 2),
                                                  (4096, 1000), (1024, 2), (1024, 1)])
def test_read_probe_reads_every_tile_once(tile_bytes, workgroups):
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    rng = np.random.default_rng(tile_bytes + workgroups)
    nbytes = 1 << 20
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    n = nbytes // tile_bytes
    sink = torch.empty(workgroups * 64, dtype=torch.int32, device="cuda")
    words = host.reshape(n, tile_bytes // 4)
    # sequential: all tiles
    pkv.read_probe(buf, tile_bytes, None, n, sink, workgroups)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
    # a random subset of tiles, in random order
    ids = rng.permutation(n)[: max(1, n // 3)]
    pkv.read_probe(buf, tile_bytes, torch.from_numpy(ids.astype(np.int64)).cuda(), len(ids), sink,
                   workgroups)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words[ids].ravel())


def test_read_probe_rejects_bad_arguments():
    import paged_kv_cache_104_amd as pkv

    torch = torch_mod()
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    sink = torch.empty(64, dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PagedKVError):
        pkv.read_probe(buf, 3000, None, 4, sink, 1)            # not a power of two
    with pytest.raises(pkv.PagedKVError):
        pkv.read_probe(buf, 4096, None, 17, sink, 1)           # past the buffer
    ids = torch.zeros(4, dtype=torch.int64, device="cuda")
    with pytest.raises(pkv.PagedKVError):
        pkv.read_probe(buf, 512, ids, 4, sink, 1)              # tiles by id below 1 KB
    with pytest.raises(pkv.PagedKVError):
        pkv.read_probe(buf, 16, None, 3, sink, 1)              # not whole 1 KB rows
