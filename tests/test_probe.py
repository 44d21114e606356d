"""CPU checks of the throughput-probe library (include/mgqa_probe.h): it
exports what the header declares and rejects bad arguments before any HIP
call.  No launch is made here (no GPU)."""
import os

import pytest

from masked_gqa_attention_amd import _lib, probe
from tests.test_abi import ROOT, _exported, header_functions

pytestmark = pytest.mark.skipif(not os.path.exists(probe.LIB_PATH),
                                reason="libmgqa_probe.so not built (python -m masked_gqa_attention_amd.build)")

HEADER = os.path.join(ROOT, "include", "mgqa_probe.h")


def test_probe_library_exports_header():
    assert header_functions(HEADER) == sorted(probe.EXPORTS)
    exported = _exported(probe.LIB_PATH)
    for name in probe.EXPORTS:
        assert name in exported, name
    # The attention library carries none of the probes.
    assert not _exported(_lib.LIB_PATH) & set(probe.EXPORTS)


def test_probe_kinds_match_header():
    text = open(HEADER).read()
    for name in ("PROBE_MFMA", "PROBE_EXP", "PROBE_RCP", "PROBE_MUL", "PROBE_MFMA_EXP", "PROBE_MFMA_MUL",
                 "PROBE_STEP_MFMA", "PROBE_STEP_VEC", "PROBE_STEP_BOTH"):
        value = int(text.split(f"#define {name} ")[1].split()[0])
        assert getattr(probe, name) == value, name
    assert set(probe.WORK) == set(range(9))


def test_probe_arguments_validated_before_hip():
    lib = probe.load()
    sink = 16  # never dereferenced: every call below fails its checks first
    assert lib.probe_alu(probe.PROBE_MFMA, 1, 1, 1, None, None) == _lib.MGQA_ERR_NULL
    assert lib.probe_alu(probe.PROBE_MFMA, 0, 1, 1, sink, None) == _lib.MGQA_ERR_SHAPE
    assert lib.probe_alu(probe.PROBE_MFMA, 1, 0, 1, sink, None) == _lib.MGQA_ERR_SHAPE
    assert lib.probe_alu(probe.PROBE_MFMA, 1, 17, 1, sink, None) == _lib.MGQA_ERR_SHAPE
    assert lib.probe_alu(probe.PROBE_MFMA, 1, 1, 0, sink, None) == _lib.MGQA_ERR_SHAPE
    assert lib.probe_alu(9, 1, 1, 1, sink, None) == _lib.MGQA_ERR_SHAPE
    assert lib.probe_alu(-1, 1, 1, 1, sink, None) == _lib.MGQA_ERR_SHAPE
    assert lib.probe_read(None, 16, 1, 0, sink, None) == _lib.MGQA_ERR_NULL
    assert lib.probe_read(sink, 16, 1, 0, None, None) == _lib.MGQA_ERR_NULL
    assert lib.probe_read(sink, 24, 1, 0, sink, None) == _lib.MGQA_ERR_SHAPE
    assert lib.probe_read(sink, 16, 0, 0, sink, None) == _lib.MGQA_ERR_SHAPE
    assert lib.probe_read(sink, 16, 1, 2, sink, None) == _lib.MGQA_ERR_SHAPE
