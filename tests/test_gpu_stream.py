"""The benchmark's read-ceiling kernel (libcda_stream.so) reads exactly the
tiles it is given: its per-wave fold of the words of a K tile and a V tile
equals the XOR of those words computed on the host."""
import ctypes as C
import os

import numpy as np
import pytest
import torch

from _cda_testlib import dev, log

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "compressed_decode_attention_amd", "libcda_stream.so")


@pytest.mark.parametrize("tile_bytes,listed", [(8192, False), (8192, True), (16384, True),
                                               (4096, True)])
def test_stream_tiles_fold(tile_bytes, listed):
    log(f"stream tiles {tile_bytes} B, listed={listed}")
    L = C.CDLL(LIB)
    L.cda_stream_tiles.argtypes = [C.c_void_p] * 3 + [C.c_int32, C.c_int32] + [C.c_void_p] * 2
    L.cda_stream_tiles.restype = C.c_int32
    n_pool = 37
    rng = np.random.default_rng(5)
    k = rng.integers(0, 2**32, size=(n_pool, tile_bytes // 4), dtype=np.uint32)
    v = rng.integers(0, 2**32, size=(n_pool, tile_bytes // 4), dtype=np.uint32)
    tiles = rng.integers(0, n_pool, size=29).astype(np.int32) if listed else np.arange(
        n_pool, dtype=np.int32)
    kd, vd = torch.from_numpy(k.view(np.int32)).to(dev()), torch.from_numpy(v.view(np.int32)).to(dev())
    td = torch.from_numpy(tiles).to(dev())
    sink = torch.zeros(len(tiles), dtype=torch.int32, device=dev())
    st = L.cda_stream_tiles(kd.data_ptr(), vd.data_ptr(), td.data_ptr() if listed else None,
                            len(tiles), tile_bytes, sink.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(k[tiles], axis=1) ^ np.bitwise_xor.reduce(v[tiles], axis=1)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)
    # invalid arguments are refused before any launch
    assert L.cda_stream_tiles(kd.data_ptr(), vd.data_ptr(), None, 1, 1000, sink.data_ptr(),
                              None) == 1
