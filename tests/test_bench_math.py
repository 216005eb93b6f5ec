"""The benchmark's algorithmic byte counts (CPU only): the figures the
roofline divides by, against hand arithmetic and against the oracle's own
definition of the draft view."""
import numpy as np

import bench
import oracle


def test_1m_verify_bytes_by_hand():
    # K and V of 8 KV heads over 1,048,576 cache keys + 3 tree keys, 512 B a key
    kv = 8 * (1048576 + 3) * 2 * 128 * 2
    q_out = 2 * 3 * 32 * 128 * 2          # queries in, outputs out (bf16)
    lse_pos = 3 * 32 * 4 + 3 * 4           # fp32 lse, int32 position ids
    assert kv + q_out + lse_pos == 4_295_029_132
    assert bench.verify_bytes(1, 1 << 20, 3) == 4_295_029_132


def test_acceptance_bytes_by_hand():
    # 8 sequences x 65 rows x 128,256 fp32 logits, plus tokens and paths
    assert bench.accept_bytes(8, 64, 128256) == 8 * 65 * 128256 * 4 + 8 * 64 * 8 == 266_776_576


def test_window_view_length_equals_the_oracle_views():
    """Keys one KV head reads for T chained window queries: the size of the
    union of the oracle's per-query views, every key once."""
    for L, T, sink, win in [(1 << 12, 3, 4, 64), (1 << 12, 1, 4, 64), (100, 3, 4, 4096),
                            (70, 2, 4, 64), (70, 3, 0, 16), (5, 3, 4, 2), (300, 3, 10, 5)]:
        union = set()
        for t in range(T):
            union |= set(oracle.draft_view(L, T, t, n_sink=sink, window=win).tolist())
        assert bench.window_view_len(L, T, sink, win) == len(union), (L, T, sink, win)
    assert bench.window_view_len(1 << 20, 3, 4, 4096) == 4102
    assert bench.window_view_len(1 << 20, 1, 4, 4096) == 4100


def test_draft_bytes_of_the_1m_calls():
    view = bench.window_view_len(1 << 20, 3, 4, 4096)
    assert bench.draft_bytes(1, 1 << 20, 3, view) == 8 * 4102 * 512 + 2 * 3 * 32 * 128 * 2 + 3 * 32 * 4
    assert bench.draft_bytes(1, 1 << 20, 1, 4100) == 8 * 4100 * 512 + 2 * 32 * 128 * 2 + 32 * 4


def test_ragged_verify_bytes_count_pad_bytes_once():
    lens = np.array([2048, 32768, 5000])
    base = bench.verify_bytes(3, int(lens.sum()), 64)
    assert bench.verify_bytes(3, int(lens.sum()), 64, pad=True) == base + int(lens.sum())
