"""bench.py's measurement helpers.  The measurement-only tile-read kernel
(the read ceiling bench.py reports) reads exactly the tiles it is given:
every thread's XOR-fold of the 16-byte words it loaded matches numpy's.  The
graph timer that gives the dominant kernel's mean launch duration runs every
call it claims to time."""
import ctypes
import os

import numpy as np
import pytest

from conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.mark.parametrize("unroll", [1, 2, 4])
def test_tile_read_reads_the_listed_tiles(unroll):
    import torch

    from lookahead_chunk_sparse_amd import build as B
    L = ctypes.CDLL(B.MEASURE_LIB_PATH)
    L.lsa_measure_tile_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    rng = np.random.default_rng(unroll)
    tile_u4, n_all, n_tiles = 1024, 64, 24                     # 16 KB tiles of a 1 MiB buffer
    host = rng.integers(0, 2 ** 32, size=(n_all, tile_u4, 4), dtype=np.uint64).astype(np.uint32)
    tiles = rng.choice(n_all, n_tiles, replace=False)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    off = torch.from_numpy((tiles * tile_u4).astype(np.int64)).cuda()
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")  # one workgroup reads every tile
    rc = L.lsa_measure_tile_read(buf.data_ptr(), off.data_ptr(), n_tiles, tile_u4, sink.data_ptr(), 1, unroll,
                                 torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    words = np.bitwise_xor.reduce(host, axis=2)                # each 16-byte word folded to 32 bits
    # thread t reads words t, t + 256, t + 512, t + 768 of every tile
    want = np.bitwise_xor.reduce(words[tiles].reshape(n_tiles, 4, 256), axis=(0, 1))
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)


def test_graph_timed_runs_every_call():
    """graph_timed(fn, n, reps) makes one eager call, captures n calls in a
    graph and replays it once untimed and reps times timed: a counter that
    every call increments ends at 1 + n * (1 + reps), and the reported mean is
    the median of the reps per-call means."""
    import torch

    import bench
    x = torch.zeros(1, dtype=torch.int64, device="cuda")
    mean_ms, per_call = bench.graph_timed(lambda j: x.add_(1 + 0 * j), 10, reps=3)
    torch.cuda.synchronize()
    assert int(x.item()) == 1 + 10 * 4
    assert len(per_call) == 3 and all(p > 0 for p in per_call)
    assert mean_ms == sorted(per_call)[1]
