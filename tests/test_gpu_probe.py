"""The bf16 MFMA ceiling probe (include/tsa_probe.h) runs and reports a plausible rate."""
import pytest
import torch

from token_sparse_attention_proxy_amd import tsa as T

pytestmark = pytest.mark.gpu


def test_probe_runs_and_rates_are_plausible():
    sink = torch.full((T.probe_sink_bytes() // 4,), float("nan"), dtype=torch.float32,
                      device="cuda")
    st = torch.cuda.current_stream()
    rates = {}
    for rnd in (True, False):
        T.probe_mfma_bf16(rnd, 10, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        fl = T.probe_mfma_bf16(rnd, 2000, sink)
        e1.record(st)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(sink).all())
        rates[rnd] = fl / (e0.elapsed_time(e1) * 1e-3) / 1e12
    # every thread wrote its accumulators; both rates positive and below the published peak
    for r in rates.values():
        assert 100.0 < r < 2600.0, rates
    # a too-small sink is refused without a launch
    with pytest.raises(RuntimeError):
        T.probe_mfma_bf16(True, 10, sink[:16])
