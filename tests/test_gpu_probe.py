"""The MFMA-rate probe the benchmark reports beside the published peak: it
runs, its FLOP count matches the launch (the rate never exceeds the part's
published 2.5 PFLOP/s bf16 peak), and zero operands are not slower than
random ones."""
import math

import pytest
import torch

import long_context_sparse_patsearch_amd as crisp

pytestmark = pytest.mark.gpu


def _rate(ops, iters):
    crisp.mfma_probe(ops, iters=100)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sink = torch.full((crisp.PROBE_SINK_FLOATS,), float("nan"), dtype=torch.float32, device="cuda")
    e0.record()
    flop = crisp.mfma_probe(ops, iters=iters, sink=sink)
    e1.record()
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert flop == cus * 8 * iters * 32 * 32768
    assert torch.isfinite(sink[:cus]).all()
    return flop / (e0.elapsed_time(e1) * 1e-3) / 1e12


def test_mfma_probe_rate_is_physical():
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    rnd = torch.empty(crisp.PROBE_OPERAND_BYTES // 2, dtype=torch.bfloat16, device="cuda").uniform_(-2, 2, generator=g)
    zero = torch.zeros_like(rnd)
    r, z = _rate(rnd, 5000), _rate(zero, 5000)
    print(f"[probe] random {r:.0f} TFLOP/s, zero {z:.0f} TFLOP/s", flush=True)
    assert 100 < r <= 2600 and 100 < z <= 2600
    assert z >= 0.95 * r
    assert not math.isnan(r)


def test_mfma_probe_rejects_wrong_operand_size():
    with pytest.raises(crisp.CrispError):
        crisp.mfma_probe(torch.zeros(16, dtype=torch.bfloat16, device="cuda"))
