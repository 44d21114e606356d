"""Controls for the GPU parity case set (CPU only): each planted oracle
mutant stands in for a kernel that made that mistake; its output on the
parity cases goes through the same comparator the GPU tests use, and at
least one case must turn red.  This shows the tolerance-based parity gate
has teeth for each class of mistake, which the configurations alone do not
give (their outputs are small next to atol = 2e-2)."""
import numpy as np
import pytest

import oracle
from oracle import attention_fp64 as oa

from .cases import CASES, as_f64, compare, make_inputs
from .test_oracle_pins import MUTANTS

_SMALL = [c for c in CASES if c.B * c.Hq * c.Lq * c.Lkv <= 600_000]


@pytest.fixture(scope="module")
def references():
    refs = {}
    for c in _SMALL:
        qf, kf, vf = as_f64(c, make_inputs(c))
        refs[c.name] = (qf, kf, vf, oracle.attention(qf, kf, vf, c.causal, c.window, c.softcap))
    return refs


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_case_set_flags_mutant(name, references, monkeypatch):
    for attr, fn in MUTANTS[name]:
        monkeypatch.setattr(oa, attr, fn)
    red = []
    for c in _SMALL:
        qf, kf, vf, ref = references[c.name]
        try:
            mut = oracle.attention(qf, kf, vf, c.causal, c.window, c.softcap)
        except (ValueError, IndexError):
            red.append(c.name)
            continue
        if not compare(mut, ref)[0]:
            red.append(c.name)
    assert red, f"no parity case flags mutant {name}"
