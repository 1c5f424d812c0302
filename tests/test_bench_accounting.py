"""The benchmark's byte accounting against the oracle: the stored-row counts
bench.py derives from the keep bits (stored_rows_host after every append,
rows_before_host ahead of a chunk) equal the rows the oracle's store holds,
and its compression figures equal the oracle's pinned helpers
(compact_kv_bytes, pinned to the bytes the oracle's pools hold;
dense_kv_bytes, pinned to the FastDMS memory table)."""
import numpy as np
import pytest

import bench
import oracle
import workload

DT = {"bf16": oracle.BF16, "fp8": oracle.FP8, "fp4": oracle.FP4}


@pytest.mark.parametrize("W", [0, 5, 64])
@pytest.mark.parametrize("kv", ["bf16", "fp8", "fp4"])
def test_stored_rows_and_bytes_match_the_oracle_store(W, kv):
    B, Hkv, D, T, S = 2, 2, 128, 150, 12
    keep = workload.random_keep((B, Hkv, T + S), 0.3, seed=41 + W)
    k = workload.random_bf16((B, T + S, Hkv, D), seed=42)
    v = workload.random_bf16((B, T + S, Hkv, D), seed=43)
    c = oracle.prefill_pack(k, v, keep, T, W, S, DT[kv], align=64)
    rows = bench.stored_rows_host(keep.numpy(), T, W, S)
    assert np.array_equal(bench.rows_before_host(keep.numpy(), T, W, 0).reshape(-1),
                          c.stored_rows())
    for s in range(S):
        c.append(k[:, T + s], v[:, T + s], keep[:, :, T + s].contiguous())
        assert np.array_equal(rows[s].reshape(-1), c.stored_rows()), f"step {s}"
        if s + 1 < S:
            assert np.array_equal(bench.rows_before_host(keep.numpy(), T, W, s + 1).reshape(-1),
                                  c.stored_rows()), f"before step {s + 1}"
    got = bench.compression_ratio(int(c.stored_rows().sum()), 1, B, Hkv, D, T + S, kv)
    assert got["compact_kv_bytes"] == oracle.compact_kv_bytes(int(c.stored_rows().sum()), D,
                                                              DT[kv], B * Hkv)
    assert got["dense_bf16_bytes"] == oracle.dense_kv_bytes(1, B * Hkv, D, T + S, 2)
    same = oracle.dense_kv_bytes(1, B * Hkv, D, T + S, oracle.bytes_per_elem(DT[kv]))
    assert abs(got["vs_dense_same_dtype"] - same / got["compact_kv_bytes"]) < 1e-3


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    """The benchmark measures one device: asked for several (by flag or by a
    launcher's WORLD_SIZE) it exits with status 2 and says so, before any
    device work."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *argv],
                       env={**os.environ, **env}, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
