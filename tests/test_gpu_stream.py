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


@pytest.mark.parametrize("tile_bytes,listed,waves,split", [
    (8192, False, 8, 0), (8192, True, 8, 0), (16384, True, 3, 0), (4096, True, 1, 0),
    (8192, True, 4, 1), (8192, False, 1, 1), (4096, True, 7, 1)])
def test_stream_tiles_fold(tile_bytes, listed, waves, split):
    log(f"stream tiles {tile_bytes} B, listed={listed}, waves={waves}, split={split}")
    L = C.CDLL(LIB)
    L.cda_stream_tiles.argtypes = ([C.c_void_p] * 3 + [C.c_int32] * 4 + [C.c_void_p] * 2)
    L.cda_stream_tiles.restype = C.c_int32
    n_pool = 37
    rng = np.random.default_rng(5)
    k = rng.integers(0, 2**32, size=(n_pool, tile_bytes // 4), dtype=np.uint32)
    v = rng.integers(0, 2**32, size=(n_pool, tile_bytes // 4), dtype=np.uint32)
    tiles = rng.integers(0, n_pool, size=29).astype(np.int32) if listed else np.arange(
        n_pool, dtype=np.int32)
    kd, vd = torch.from_numpy(k.view(np.int32)).to(dev()), torch.from_numpy(v.view(np.int32)).to(dev())
    td = torch.from_numpy(tiles).to(dev())
    sink = torch.zeros(2 * len(tiles), dtype=torch.int32, device=dev())
    st = L.cda_stream_tiles(kd.data_ptr(), vd.data_ptr(), td.data_ptr() if listed else None,
                            len(tiles), tile_bytes, waves, split, sink.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    fk, fv = np.bitwise_xor.reduce(k[tiles], axis=1), np.bitwise_xor.reduce(v[tiles], axis=1)
    got = sink.cpu().numpy().view(np.uint32)
    if split:
        assert np.array_equal(got[0::2], fk) and np.array_equal(got[1::2], fv)
    else:
        assert np.array_equal(got[:len(tiles)], fk ^ fv)
    # invalid arguments are refused before any launch
    for bad in ((1, 1000, 1, 0), (1, 1024, 0, 0), (1, 1024, 9, 0), (1, 1024, 1, 2)):
        assert L.cda_stream_tiles(kd.data_ptr(), vd.data_ptr(), None, *bad, sink.data_ptr(),
                                  None) == 1
