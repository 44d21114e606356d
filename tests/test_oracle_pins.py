"""Pins for the float64 oracle, each tied to something other than the oracle
itself: an independent pure-Python brute force, closed forms, and invariants
that the definition on the task page "TPU v6e Masked GQA Kernel Optimization"
("What You Have": GQA ratios, causal mask, sliding window, logit softcap)
fixes under the readings stated in oracle/attention_fp64.py.

The checks are plain functions so that test_planted_mutants can run the same
battery against deliberately broken copies of the oracle (planted on the CPU)
and show that each mistake turns at least one check red.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from oracle import attention_fp64 as oa


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def _tolist(a):
    return np.asarray(a, dtype=np.float64).tolist()


# ---------------------------------------------------------------------------
# Check battery
# ---------------------------------------------------------------------------

def check_vs_brute(seed=0, quick=False):
    """Oracle == pure-Python brute force over a sweep of tiny shapes and all
    option combinations (relative 1e-12)."""
    rng = np.random.default_rng(seed)
    shapes = [  # B, Hq, Hkv, Lq, Lkv, d
        (1, 1, 1, 1, 1, 1),
        (1, 2, 1, 3, 5, 3),
        (2, 4, 2, 4, 4, 8),
        (1, 4, 1, 7, 9, 4),
        (1, 3, 3, 5, 6, 2),
        (2, 4, 4, 6, 6, 5),
    ]
    opts = list(itertools.product([False, True], [0, 1, 2, 3, 5, 100], [0.0, 0.7, 5.0]))
    if quick:
        opts = opts[::5]
    for (B, Hq, Hkv, Lq, Lkv, d) in shapes:
        q = _rand(rng, B, Hq, Lq, d, scale=1.5)
        k = _rand(rng, B, Hkv, Lkv, d, scale=1.5)
        v = _rand(rng, B, Hkv, Lkv, d + 1)
        for causal, window, cap in opts:
            if (causal or window) and Lq > Lkv:
                continue
            ref = oracle.attention_brute(_tolist(q), _tolist(k), _tolist(v), causal, window, cap)
            got = oracle.attention(q, k, v, causal, window, cap)
            np.testing.assert_allclose(got, np.array(ref), rtol=1e-12, atol=1e-13,
                                       err_msg=f"{(B,Hq,Hkv,Lq,Lkv,d)} causal={causal} W={window} cap={cap}")


def check_two_key_closed_form():
    """Two keys, one query: with a = q.k0 and b = q.k1 the output is
    p0*v0 + (1-p0)*v1 with p0 = 1/(1+exp(f(b)-f(a))), f(x) = x/sqrt(d), or
    c*tanh(x/(c*sqrt(d))) under a softcap c.  A window of one key keeps only
    the diagonal key; the bottom-right causal mask keeps both keys for a
    single query row."""
    d = 3
    q = np.array([0.9, -1.3, 2.2])
    k0 = np.array([1.1, 0.4, 1.7])
    k1 = np.array([-0.8, 2.5, 0.3])
    v0 = np.array([1.0, -2.0, 0.5, 3.0])
    v1 = np.array([-1.5, 0.25, 4.0, -0.75])
    a = float(q @ k0)
    b = float(q @ k1)
    Q = q.reshape(1, 1, 1, d)
    K = np.stack([k0, k1]).reshape(1, 1, 2, d)
    V = np.stack([v0, v1]).reshape(1, 1, 2, 4)
    for cap in (0.0, 0.5, 2.0, 30.0):
        if cap > 0:
            f = lambda x: cap * math.tanh(x / (cap * math.sqrt(d)))  # noqa: E731
        else:
            f = lambda x: x / math.sqrt(d)  # noqa: E731
        p0 = 1.0 / (1.0 + math.exp(f(b) - f(a)))
        want = p0 * v0 + (1 - p0) * v1
        for causal in (False, True):
            got = oracle.attention(Q, K, V, causal=causal, softcap=cap)[0, 0, 0]
            np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-14)
        # window of one key: only the diagonal key (position Lkv-1) is visible
        got = oracle.attention(Q, K, V, causal=True, window=1, softcap=cap)[0, 0, 0]
        np.testing.assert_allclose(got, v1, rtol=0, atol=1e-15)
        got = oracle.attention(Q, K, V, causal=False, window=1, softcap=cap)[0, 0, 0]
        np.testing.assert_allclose(got, v1, rtol=0, atol=1e-15)


def check_rows_and_constants(seed=1):
    """Probabilities are non-negative and sum to 1 per row; V = 1 gives O = 1;
    a constant V = c gives O = c on every element (the constant-input check of
    the Graphcore page, "SigLIP batch-1 hardware results")."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, Lq, Lkv, d = 2, 4, 2, 9, 13, 8
    q = _rand(rng, B, Hq, Lq, d, scale=3)
    k = _rand(rng, B, Hkv, Lkv, d, scale=3)
    for causal, window, cap in [(False, 0, 0.0), (True, 0, 0.0), (True, 4, 5.0), (False, 3, 0.0)]:
        P = oracle.probabilities(q, k, np.zeros((B, Hkv, Lkv, 1)), causal, window, cap)
        assert (P >= 0).all()
        np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-14)
        for c in (1.0, -0.375, 7.25):
            v = np.full((B, Hkv, Lkv, 5), c)
            o = oracle.attention(q, k, v, causal, window, cap)
            np.testing.assert_allclose(o, c, rtol=1e-14, atol=0)


def _band_edges(i, Lq, Lkv, causal, W):
    """Independent statement of the band for row i: [lo, hi] inclusive."""
    pos = Lkv - Lq + i
    lo, hi = 0, Lkv - 1
    if causal:
        hi = min(hi, pos)
    if W > 0:
        lo = max(lo, pos - W + 1)
        if not causal:
            hi = min(hi, pos + W - 1)
    return lo, hi


def check_mask_readout():
    """Q = 0 makes every score 0 (softcap(0) = 0), so each visible key gets
    1/n.  With V one-hot per key, O[i, j] = 1/n_i inside the band and exactly
    0 outside; with the ramp V[j] = j, O[i] = (lo_i + hi_i)/2 gives both band
    edges.  Covers the bottom-right offset and the window's off-by-one."""
    for (Lq, Lkv) in [(1, 1), (5, 5), (3, 9), (9, 9), (1, 12)]:
        for causal, W, cap in itertools.product([False, True], [0, 1, 2, 3, 4, 50], [0.0, 3.0]):
            q = np.zeros((1, 1, Lq, 4))
            k = np.random.default_rng(Lq * 100 + Lkv).standard_normal((1, 1, Lkv, 4))
            v1 = np.eye(Lkv).reshape(1, 1, Lkv, Lkv)
            o = oracle.attention(q, k, v1, causal, W, cap)[0, 0]
            ramp = np.arange(Lkv, dtype=np.float64).reshape(1, 1, Lkv, 1)
            r = oracle.attention(q, k, ramp, causal, W, cap)[0, 0, :, 0]
            for i in range(Lq):
                lo, hi = _band_edges(i, Lq, Lkv, causal, W)
                want = np.zeros(Lkv)
                want[lo:hi + 1] = 1.0 / (hi - lo + 1)
                np.testing.assert_allclose(o[i], want, rtol=1e-14, atol=0,
                                           err_msg=f"Lq={Lq} Lkv={Lkv} causal={causal} W={W} row {i}")
                assert np.all(o[i][want == 0] == 0.0)
                assert abs(r[i] - (lo + hi) / 2) < 1e-12


def check_suffix_consistency(seed=2):
    """Bottom-right alignment: attending with the last Lq query rows of a
    longer query equals the last Lq rows of the full result; decode (Lq=1)
    equals the last row of prefill."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, L, d = 1, 4, 2, 11, 6
    q = _rand(rng, B, Hq, L, d, scale=2)
    k = _rand(rng, B, Hkv, L, d, scale=2)
    v = _rand(rng, B, Hkv, L, d)
    for causal, W, cap in [(True, 0, 0.0), (True, 3, 0.0), (True, 5, 2.0), (False, 0, 0.0), (False, 4, 0.0)]:
        full = oracle.attention(q, k, v, causal, W, cap)
        for Lq in (1, 2, 5, L):
            part = oracle.attention(q[:, :, L - Lq:], k, v, causal, W, cap)
            np.testing.assert_allclose(part, full[:, :, L - Lq:], rtol=1e-13, atol=1e-14)


def check_gqa_equals_repeated_kv(seed=3):
    """Grouped-query sharing equals multi-head attention with each K/V head
    repeated G times consecutively."""
    rng = np.random.default_rng(seed)
    for (Hq, Hkv) in [(4, 2), (8, 2), (6, 3), (4, 4), (4, 1)]:
        B, Lq, Lkv, d = 2, 5, 7, 4
        q = _rand(rng, B, Hq, Lq, d, scale=2)
        k = _rand(rng, B, Hkv, Lkv, d, scale=2)
        v = _rand(rng, B, Hkv, Lkv, d)
        G = Hq // Hkv
        kr = np.repeat(k, G, axis=1)
        vr = np.repeat(v, G, axis=1)
        for causal, W in [(False, 0), (True, 3)]:
            a = oracle.attention(q, k, v, causal, W, 1.5)
            # MHA path computed head by head from the brute force
            b = np.array(oracle.attention_brute(_tolist(q), _tolist(kr), _tolist(vr), causal, W, 1.5))
            np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def check_limits(seed=4):
    """An unbounded window equals no window (exactly); a large softcap tends
    to no softcap with error shrinking like 1/c^2; a single key returns V."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, Lq, Lkv, d = 1, 2, 1, 6, 8, 5
    q = _rand(rng, B, Hq, Lq, d, scale=2)
    k = _rand(rng, B, Hkv, Lkv, d, scale=2)
    v = _rand(rng, B, Hkv, Lkv, d)
    for causal in (False, True):
        a = oracle.attention(q, k, v, causal, 0, 0.0)
        b = oracle.attention(q, k, v, causal, Lq + Lkv, 0.0)
        assert np.array_equal(a, b)
        errs = []
        for c in (10.0, 100.0, 1000.0):
            errs.append(np.abs(oracle.attention(q, k, v, causal, 0, c) - a).max())
        assert errs[0] > 0
        # |c tanh(s/c) - s| <= |s|^3 / (3 c^2): error ratio ~100 per decade
        assert errs[1] < errs[0] / 50 and errs[2] < errs[1] / 50
    k1 = k[:, :, :1]
    v1 = v[:, :, :1]
    for causal, W, cap in [(False, 0, 0.0), (True, 1, 2.0)]:
        o = oracle.attention(q[:, :, :1], k1, v1, causal, W, cap)
        np.testing.assert_allclose(o[:, :, 0], np.repeat(v1[:, :, 0], Hq // Hkv, axis=1), rtol=1e-15)


def check_linearity_shift_permutation(seed=5):
    """O(aV + b) = a O(V) + b; adding the same vector u to every key leaves O
    unchanged without softcap (each row's scores shift by q.u); permuting
    keys and values together leaves O unchanged without a mask."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, Lq, Lkv, d = 1, 4, 2, 5, 9, 6
    q = _rand(rng, B, Hq, Lq, d, scale=2)
    k = _rand(rng, B, Hkv, Lkv, d, scale=2)
    v = _rand(rng, B, Hkv, Lkv, d)
    for causal, W in [(False, 0), (True, 4)]:
        o = oracle.attention(q, k, v, causal, W)
        np.testing.assert_allclose(oracle.attention(q, k, -2.5 * v + 0.75, causal, W), -2.5 * o + 0.75,
                                   rtol=1e-12, atol=1e-12)
        u = rng.standard_normal(d)
        np.testing.assert_allclose(oracle.attention(q, k + u, v, causal, W), o, rtol=1e-11, atol=1e-12)
    perm = rng.permutation(Lkv)
    o = oracle.attention(q, k, v, False, 0, 3.0)
    np.testing.assert_allclose(oracle.attention(q, k[:, :, perm], v[:, :, perm], False, 0, 3.0), o,
                               rtol=1e-12, atol=1e-13)


def check_hot_inputs(seed=6):
    """Scores of order 1e3 stay finite, and the result matches the
    brute force (max subtraction)."""
    rng = np.random.default_rng(seed)
    q = _rand(rng, 1, 2, 3, 4, scale=30)
    k = _rand(rng, 1, 1, 5, 4, scale=30)
    v = _rand(rng, 1, 1, 5, 4)
    for causal, W, cap in [(False, 0, 0.0), (True, 2, 0.0), (True, 0, 50.0)]:
        o = oracle.attention(q, k, v, causal, W, cap)
        assert np.isfinite(o).all()
        ref = np.array(oracle.attention_brute(_tolist(q), _tolist(k), _tolist(v), causal, W, cap))
        np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-12)


def check_rows_api(seed=7):
    """attention_rows (one row at a time) agrees with the full brute force."""
    rng = np.random.default_rng(seed)
    q = _rand(rng, 2, 4, 6, 5, scale=2)
    k = _rand(rng, 2, 2, 8, 5, scale=2)
    v = _rand(rng, 2, 2, 8, 3)
    rows = [(0, 0, 0), (1, 3, 5), (0, 2, 3), (1, 1, 1)]
    for causal, W, cap in [(False, 0, 0.0), (True, 3, 2.0), (False, 2, 0.0)]:
        ref = oracle.attention_brute(_tolist(q), _tolist(k), _tolist(v), causal, W, cap)
        got = oracle.attention_rows(q, k, v, rows, causal, W, cap)
        for n, (b, h, i) in enumerate(rows):
            np.testing.assert_allclose(got[n], ref[b][h][i], rtol=1e-12, atol=1e-13)


def check_pair_count():
    """visible_pairs() against a closed form: causal window W over a square
    L x L problem has sum_i min(i+1, W) pairs."""
    for L, W in [(16, 4), (64, 64), (100, 7), (33, 1)]:
        want = sum(min(i + 1, W) for i in range(L))
        assert oracle.visible_pairs(L, L, True, W) == want
        assert oracle.visible_pairs(L, L, True, 0) == L * (L + 1) // 2
        assert oracle.visible_pairs(L, L, False, 0) == L * L


BATTERY = [
    check_vs_brute,
    check_two_key_closed_form,
    check_rows_and_constants,
    check_mask_readout,
    check_suffix_consistency,
    check_gqa_equals_repeated_kv,
    check_limits,
    check_linearity_shift_permutation,
    check_hot_inputs,
    check_rows_api,
]


@pytest.mark.parametrize("check", BATTERY + [check_pair_count], ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()


def test_empty_row_is_an_error():
    q = np.zeros((1, 1, 3, 2))
    k = np.zeros((1, 1, 2, 2))
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, causal=True)


# ---------------------------------------------------------------------------
# Planted mutants: each plants one plausible mistake in the oracle (on the
# CPU) and the battery must catch it.
# ---------------------------------------------------------------------------

def _mut_no_softcap(s, softcap):
    return s


def _mut_window_plus_one(pos, j, causal, window):
    return _orig_visible(pos, j, causal, window + 1 if window > 0 else 0)


def _mut_top_left_band(Lq, Lkv, causal, window):
    i = np.arange(Lq)[:, None]
    j = np.arange(Lkv)[None, :]
    return _orig_visible(i, j, causal, window)


def _mut_top_left_row(i, Lq, Lkv, causal, window):
    return _orig_visible(i, np.arange(Lkv), causal, window)


def _mut_interleaved_heads(h, Hq, Hkv):
    return h % Hkv


def _mut_scale_one_over_d(d):
    return 1.0 / d


def _mut_unnormalised(s, ok):
    s = np.where(ok, s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    return np.exp(s - m)


def _mut_no_max_subtraction(s, ok):
    s = np.where(ok, s, -np.inf)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def _mut_causal_strict(pos, j, causal, window):
    ok = _orig_visible(pos, j, False, window)
    if causal:
        ok &= j < pos
    return ok


def _mut_window_minus_one(pos, j, causal, window):
    return _orig_visible(pos, j, causal, window - 1 if window > 1 else window)


def _mut_softcap_unscaled_tanh(s, softcap):
    return np.tanh(s) if softcap > 0 else s


def _mut_one_sided_window_noncausal(pos, j, causal, window):
    ok = np.ones(np.broadcast(pos, j).shape, dtype=bool)
    if causal:
        ok &= j <= pos
    if window > 0:
        ok &= (pos - j) < window
    return ok


_orig_visible = oa.visible

MUTANTS = {
    "softcap_ignored": [("apply_softcap", _mut_no_softcap)],
    "window_plus_one": [("visible", _mut_window_plus_one)],
    "causal_top_left": [("band", _mut_top_left_band), ("band_row", _mut_top_left_row)],
    "heads_interleaved": [("kv_head", _mut_interleaved_heads)],
    "scale_one_over_d": [("scale", _mut_scale_one_over_d)],
    "unnormalised": [("softmax_masked", _mut_unnormalised)],
    "causal_excludes_diagonal": [("visible", _mut_causal_strict)],
    "window_minus_one": [("visible", _mut_window_minus_one)],
    "softcap_tanh_unscaled": [("apply_softcap", _mut_softcap_unscaled_tanh)],
    "window_one_sided_without_causal": [("visible", _mut_one_sided_window_noncausal)],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mutant_is_caught(name, monkeypatch):
    for attr, fn in MUTANTS[name]:
        monkeypatch.setattr(oa, attr, fn)
    caught = []
    for check in BATTERY:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"mutant {name} passed every oracle pin"


def test_max_subtraction_mutant_overflows(monkeypatch):
    """Dropping the max subtraction is invisible at small scores but the hot
    input check must catch it."""
    monkeypatch.setattr(oa, "softmax_masked", _mut_no_max_subtraction)
    with pytest.raises((AssertionError, FloatingPointError)):
        with np.errstate(over="ignore", invalid="ignore"):
            check_hot_inputs()
