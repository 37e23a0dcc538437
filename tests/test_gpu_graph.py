"""The whole op captured in a HIP graph and replayed (GPU).

The library keeps the budget on the device, allocates nothing and issues no
memset, so one forward call can be captured once and replayed with new
inputs copied into the captured buffers.  Every replay must reproduce the
eager result for its inputs bit for bit.  Between replays the test does its
own eager work (input copies, poisoning of the outputs) and synchronises.
"""
import pytest
import torch

from tests.parity import say, to_dev
from token_sparse_attention_proxy_amd import inputs
from token_sparse_attention_proxy_amd import tsa as T

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("flags", [0, T.TSA_FLAG_PER_HEAD_BUDGET], ids=["global", "per_head"])
@pytest.mark.parametrize("fused", [False, True], ids=["steps", "fused"])
def test_forward_graph_replay(fused, flags):
    say(f"case graph replay fused={fused} flags={flags}")
    B, Hq, Hkv, L, d, w, tau = 1, 8, 2, 1000, 128, 64, 0.05
    sets = []
    for seed_base, zipf in ((9900, 0.0), (9910, 1.1)):     # two input sets with different budgets
        wl = inputs.small_workload("bf16", B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, w=w, tau=tau,
                                   zipf_s=zipf, seed_base=seed_base)
        sets.append(tuple(to_dev(x, "bf16") for x in inputs.make_qkv(wl)))
    prob = T.Problem(B, Hq, Hkv, L, d, w, tau, "bf16", flags=flags)
    run = T.tsa_forward_fused if fused else T.tsa_forward
    wsb = T.fused_workspace_bytes(prob) if fused else T.forward_workspace_bytes(prob)

    # Eager results, one per input set, in buffers of their own.
    want = []
    for qs, ks, vs in sets:
        o, budget, idx = run(prob, qs, ks, vs)
        torch.cuda.synchronize()
        want.append((o.clone(), budget.clone(), idx.clone()))
    assert not torch.equal(want[0][1], want[1][1]), "the two input sets should give different budgets"

    # Captured buffers: inputs, outputs and workspace all allocated before capture.
    qd, kd, vd = (torch.empty_like(x) for x in sets[0])
    o = torch.empty_like(qd)
    budget = torch.empty(prob.budget_shape, dtype=torch.int32, device=qd.device)
    idx = torch.empty((B, Hq, L), dtype=torch.int32, device=qd.device)
    ws = torch.empty(wsb, dtype=torch.uint8, device=qd.device)
    for dst, src in zip((qd, kd, vd), sets[0]):
        dst.copy_(src)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                  # warm-up off the capture
        run(prob, qd, kd, vd, o, budget, idx, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(prob, qd, kd, vd, o, budget, idx, ws)
    torch.cuda.synchronize()

    for r in range(4):
        s = r % 2
        for dst, src in zip((qd, kd, vd), sets[s]):
            dst.copy_(src)
        _bits(o).fill_(0x7F7F)                     # every row must be rewritten by the replay
        budget.fill_(-1)
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        wo, wb, wi = want[s]
        say(f"  replay {r}: input set {s}, budget {budget.cpu().tolist()}")
        assert torch.equal(budget, wb)
        assert torch.equal(idx, wi)
        assert torch.equal(_bits(o), _bits(wo))
