"""The throughput probes run and compute what include/mgqa_probe.h says: the
streaming read's sink words XOR to the XOR of the buffer, every ALU probe
leaves finite values.  Tiny sizes: a correctness check, not a measurement."""
import numpy as np
import pytest
import torch

from masked_gqa_attention_amd import probe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nontemporal", [0, 1])
@pytest.mark.parametrize("nbytes,workgroups", [(16, 1), (4096, 1), (1 << 20, 7), ((1 << 20) + 48, 256),
                                               (3 * (1 << 16) + 16, 1000)])
def test_probe_read_xor(nbytes, workgroups, nontemporal):
    print(f"probe_read bytes={nbytes} workgroups={workgroups} nontemporal={nontemporal}", flush=True)
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    buf = host.cuda()
    sink = torch.zeros(workgroups * 256, dtype=torch.int32, device="cuda")
    rc = probe.load().probe_read(buf.data_ptr(), nbytes, workgroups, nontemporal, sink.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


@pytest.mark.parametrize("kind", sorted(probe.WORK))
def test_probe_alu_runs(kind):
    print(f"probe_alu kind={kind}", flush=True)
    r = probe.run_alu(kind, workgroups=8, waves=4, iters=3, reps=1)
    assert r["finite"] and r["ms"] > 0
