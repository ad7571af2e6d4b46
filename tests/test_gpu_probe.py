"""The matrix-core rate probe used by the benchmark: every thread's sink
value is fixed by the arithmetic (each v_mfma_f32_32x32x16_bf16 adds
16·a·b to each of a wave's 4 × 16 accumulator elements per lane), so a
wrong operand layout, a dropped MFMA or a lost round changes it; bad
arguments are rejected on the host."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    m.context(0)
    return m


@pytest.mark.parametrize("blocks,iters,a,b", [(1, 1, 1.0, 1.0), (8, 100, 1.5, -2.0), (300, 7, 0.25, 3.0)])
def test_mfma_probe_sink(moe, blocks, iters, a, b):
    sink = moe.moe_mfma_peak_probe(blocks, iters, a, b)
    torch.cuda.synchronize()
    want = 1024.0 * a * b * iters
    assert torch.equal(sink, torch.full_like(sink, want))


def test_mfma_probe_rejects(moe):
    with pytest.raises(moe.MoeError):
        moe.moe_mfma_peak_probe(0, 10)
    with pytest.raises(moe.MoeError):
        moe.moe_mfma_peak_probe(4, 0)
