"""The matrix-core probes (measurement aids) on the GPU: both kinds run,
report the operations of one launch, and give the same sink twice; the data
form reads only the given arrays (a one-fragment array is reused by every
lane)."""
import pytest
import torch

from long_context_sparse_lsa_amd import _lib as L
from tests._util import need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    L.load()


@pytest.mark.parametrize("kind", [0, 1])
def test_probes_run_and_repeat(kind):
    n_wg, iters = 64, 16
    sink = torch.zeros(n_wg, dtype=torch.int32, device="cuda")
    ops = L.lsa_probe_mfma(kind, n_wg, iters, sink)
    assert ops == (65536.0 if kind == 0 else 32768.0) * 8 * iters * 4 * n_wg
    s1 = sink.clone()
    L.lsa_probe_mfma(kind, n_wg, iters, sink)
    assert torch.equal(s1, sink)
    g = torch.Generator(device="cuda").manual_seed(5)
    if kind == 0:
        a = torch.randint(-128, 128, (4096,), dtype=torch.int8, device="cuda", generator=g)
        b = torch.randint(-16, 16, (16,), dtype=torch.int8, device="cuda", generator=g)
    else:
        a = torch.randn(2048, dtype=torch.bfloat16, device="cuda", generator=g)
        b = torch.randn(8, dtype=torch.bfloat16, device="cuda", generator=g)
    ops = L.lsa_probe_mfma_data(kind, n_wg, iters, a, b, sink)
    assert ops == (65536.0 if kind == 0 else 32768.0) * 8 * iters * 4 * n_wg
    s1 = sink.clone()
    L.lsa_probe_mfma_data(kind, n_wg, iters, a, b, sink)
    torch.cuda.synchronize()
    assert torch.equal(s1, sink)
