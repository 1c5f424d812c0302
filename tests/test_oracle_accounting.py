"""Pins for the accounting helpers against the FastDMS page's memory table.

The page's vLLM baselines use token pools sized exactly for the workload
(ctx 8192 + gen 128).  With the public attention shapes of the two models
(Llama-3.2-1B: 16 layers, 8 KV heads, head_dim 64; Qwen3-8B: 36 layers,
8 KV heads, head_dim 128) the printed GiB come out exactly for pools of
10,240 tokens (c = 1) and 8 x 8,448 tokens (c = 8; 8,320 rounded up to a
multiple of 256), halved for FP8.  The "saved" columns are the ratio of the
printed GiB.  The c = 1 pool size is not explained on the page; it is taken
as the value that reproduces the table.
"""
import os

import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fastdms_memory_table.txt")
SHAPES = {"llama-3.2-1b": (16, 8, 64), "qwen3-8b": (36, 8, 128)}
POOL = {1: 10240, 8: 8 * 8448}


def _rows():
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            yield line.split()


def test_dense_pool_sizes_match_table(orc):
    n = 0
    for f in _rows():
        model, c = f[0], int(f[1])
        L, Hkv, D = SHAPES[model]
        gib = 2.0 ** 30
        bf16 = orc.dense_kv_bytes(L, Hkv, D, POOL[c], 2) / gib
        fp8 = orc.dense_kv_bytes(L, Hkv, D, POOL[c], 1) / gib
        assert f"{bf16:.3f}" == f[2], (model, c, bf16)
        assert f"{fp8:.3f}" == f[5], (model, c, fp8)
        n += 1
    assert n == 4


def test_saved_ratios_match_table():
    for f in _rows():
        fast = float(f[3])
        for col_v, col_r in ((2, 4), (5, 6), (7, 8)):
            if f[col_v] == "-":
                continue
            assert f"{float(f[col_v]) / fast:.1f}" == f[col_r], (f[0], f[1], col_v)


def test_fastdms_rows_imply_kept_fraction():
    # FastDMS GiB / (bytes per BF16 token) / 8,320 tokens: a sanity range for
    # the synthetic keep rates, not a parity pin.
    for f in _rows():
        L, Hkv, D = SHAPES[f[0]]
        per_tok = L * Hkv * D * 2 * 2
        tokens = float(f[3]) * 2 ** 30 / per_tok / int(f[1])
        frac = tokens / 8320
        assert 0.12 < frac < 0.26, (f[0], f[1], frac)
