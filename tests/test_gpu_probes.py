"""The measurement probes through the C ABI: the streaming read, the
matrix-instruction issue-rate probe and the LDS read probe launch, finish
and leave their sinks alone (a sink word is written only when a fold hits
one fixed value)."""
import pytest
import torch

import structured_sparse_gemm_amd as ssg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    torch.cuda.init()
    return torch.device("cuda:0")


@pytest.mark.parametrize("nbytes", [16, 4096, 1 << 20, (1 << 24) + 48])
def test_stream_read_runs(nbytes):
    src = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(ssg.ssg_stream_read_sink_words(nbytes), dtype=torch.int32, device="cuda")
    ssg.ssg_stream_read(src, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0                       # the fold of zeros is zero


@pytest.mark.parametrize("form", range(10))
def test_mfma_probe_runs_every_form(form):
    assert ssg.ssg_mfma_probe_name(form) is not None
    wg = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(wg, dtype=torch.int32, device="cuda")
    ssg.ssg_mfma_probe(form, wg, 4, sink)
    ssg.ssg_mfma_probe(form, 3, 1, sink)                    # fewer workgroups than CUs
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


def test_lds_read_probe_runs_and_sees_bank_conflicts():
    import bench
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(cus, dtype=torch.int32, device="cuda")
    pats = dict(bench.lds_patterns())
    for offs in pats.values():
        ssg.ssg_lds_read_probe(offs, 3, 2, sink)
    torch.cuda.synchronize()
    assert int(sink.ne(0).sum()) == 0 or int(sink.ne(0).sum()) == int(sink.eq(-1640531527).sum())
    # sixteen lanes on one bank take many times longer than a contiguous read
    stream = torch.cuda.current_stream()
    t = {}
    for name in ("contiguous (lane l at 16 l)", "the 16 lanes of each group on one bank, 256 B apart"):
        ssg.ssg_lds_read_probe(pats[name], cus, 10, sink)
        t[name] = min(bench.time_kernel(lambda i: ssg.ssg_lds_read_probe(pats[name], cus, 500, sink), 1, stream)
                      for _ in range(3))
    assert t["the 16 lanes of each group on one bank, 256 B apart"] > 3 * t["contiguous (lane l at 16 l)"]
