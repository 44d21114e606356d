"""The process-pool driver of the oracle computes exactly what
oracle.attention computes (the same float64 operations head by head), for
grouped heads, masks and a softcap, whether a unit's heads go to one worker
or are split across several."""
import numpy as np

import oracle
from masked_gqa_attention_amd import synth
from oracle.pool import _tasks


def test_pool_equals_oracle_bit_for_bit(oracle_pool):
    for (B, Hq, Hkv, Lq, Lkv, d, causal, window, cap) in [(2, 6, 2, 33, 50, 16, True, 7, 5.0),
                                                          (1, 4, 4, 20, 20, 8, False, 0, 0.0),
                                                          (1, 8, 1, 1, 90, 24, True, 40, 0.0),
                                                          (1, 16, 1, 9, 40, 8, True, 0, 3.0),
                                                          (3, 12, 4, 5, 30, 8, False, 9, 0.0)]:
        q = synth.storage_to_f64(synth.draw_array(1, (B, Hq, Lq, d)), "bf16")
        k = synth.storage_to_f64(synth.draw_array(2, (B, Hkv, Lkv, d)), "bf16")
        v = synth.storage_to_f64(synth.draw_array(3, (B, Hkv, Lkv, d)), "bf16")
        want = oracle.attention(q, k, v, causal, window, cap)
        got = oracle_pool.attention(q, k, v, causal, window, cap)
        assert got.shape == want.shape
        assert np.array_equal(got, want)
    assert oracle_pool.workers >= 1


def test_tasks_cover_every_head_once():
    for (B, Hq, Hkv, workers) in [(2, 32, 4, 16), (8, 32, 8, 16), (1, 16, 16, 16), (4, 64, 4, 3), (1, 7, 1, 64)]:
        q = np.zeros((B, Hq, 1, 1))
        k = np.zeros((B, Hkv, 1, 1))
        seen = []
        for (h0, h1), (qs, ks, vs, *_ ) in _tasks(q, k, k, False, 0, 0.0, workers):
            assert qs.shape[1] == h1 - h0 and ks.shape[1] == 1
            assert h0 // (Hq // Hkv) == (h1 - 1) // (Hq // Hkv)  # one K/V head per task
            seen.extend(range(h0, h1))
        assert sorted(seen) == sorted(list(range(Hq)) * B)
