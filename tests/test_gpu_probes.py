"""The measurement probes through the C ABI: the streaming read and the
matrix-instruction issue-rate probe launch, finish and leave their sinks
alone (a sink word is written only when a fold hits one fixed value)."""
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
