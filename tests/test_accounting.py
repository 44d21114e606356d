"""The benchmark's work counts (closed form per row) against the oracle's
mask, counted pair by pair."""
import itertools

import numpy as np

import oracle
from masked_gqa_attention_amd import accounting, synth


def test_pairs_match_mask_count():
    for Lq, Lkv in [(1, 1), (1, 50), (7, 7), (20, 33), (64, 64), (100, 300)]:
        for causal, W in itertools.product([False, True], [0, 1, 2, 5, 17, 1000]):
            if (causal or W) and Lq > Lkv:
                continue
            assert accounting.pairs_per_head(Lq, Lkv, causal, W) == oracle.visible_pairs(Lq, Lkv, causal, W)


def test_keys_touched_match_mask_union():
    for Lq, Lkv in [(1, 50), (7, 7), (20, 33), (64, 200)]:
        for causal, W in itertools.product([False, True], [0, 1, 5, 17]):
            band = oracle.band(Lq, Lkv, causal, W)
            assert accounting.keys_touched_per_unit(Lq, Lkv, causal, W) == int(band.any(axis=0).sum())


def test_workload_figures():
    w = synth.WORKLOADS["prefill_gqa8_L4096_w1024_cap50"]
    W = w.window
    per_head = W * (W + 1) // 2 + (w.Lq - W) * W      # sum_i min(i+1, W)
    assert accounting.workload_work(w)["pairs"] == per_head * w.B * w.Hq
    w5 = synth.WORKLOADS["decode_gqa16_kv32768_w4096_cap30"]
    assert accounting.workload_work(w5)["kv_bytes"] == 2 * w5.B * w5.Hkv * 4096 * w5.d * 2
    w2 = synth.WORKLOADS["decode_gqa4_kv8192"]
    assert accounting.workload_work(w2)["bytes"] == 268_566_528
    assert accounting.workload_work(synth.WORKLOADS["encoder_siglip_L729_d72"])["flops"] == 4 * 72 * 729 * 729 * 16
