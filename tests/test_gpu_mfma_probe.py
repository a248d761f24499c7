"""The matrix-core probe (pkv_mfma_probe) runs every product it is asked for: with all operands 1 each product adds
16 to every accumulator element, so each lane's sink value is exactly 2048 * iters + 8 * valu * iters; its clock
record gives a shader clock between the reference clock's plausible bounds."""
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_383_amd import build as b
    b.ensure_built()
    import paged_kv_cache_383_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("valu", [0, 4, 8])
def test_probe_sums_are_exact(pkv, dtype, valu):
    groups, iters = 300, 123
    sink = torch.full((groups * 256,), -1.0, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(groups * 8, dtype=torch.int64, device="cuda")
    pkv.mfma_probe(dtype, groups, iters, sink, clocks, valu=valu)
    torch.cuda.synchronize()
    want = 2048 * iters + 8 * valu * iters
    assert torch.equal(sink, torch.full_like(sink, float(want)))
    c = clocks.view(-1, 2).cpu().double()
    assert bool((c[:, 0] > 0).all()) and bool((c[:, 1] > 0).all())
    ghz = (c[:, 0] / c[:, 1] * 0.1)                       # cycles per 100 MHz tick x 0.1 GHz
    assert 0.3 < float(ghz.median()) < 3.5


def test_probe_without_clocks_and_at_the_iteration_limit(pkv):
    sink = torch.zeros(256, dtype=torch.float32, device="cuda")
    pkv.mfma_probe(torch.bfloat16, 1, pkv.MFMA_PROBE_MAX_ITERS, sink)
    torch.cuda.synchronize()
    assert torch.equal(sink, torch.full_like(sink, 2048.0 * pkv.MFMA_PROBE_MAX_ITERS))
    with pytest.raises(pkv.PagedKVError):
        pkv.mfma_probe(torch.bfloat16, 1, pkv.MFMA_PROBE_MAX_ITERS + 1, sink)
