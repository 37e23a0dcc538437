"""The Python binding rejects tensors whose shape or dtype does not match the problem
before anything reaches the library (no GPU needed: the check runs before the device
check, so host tensors of the wrong shape are refused with a ValueError naming them)."""
import pytest
import torch

from token_sparse_attention_proxy_amd import tsa as T

P = T.Problem(B=1, Hq=8, Hkv=2, L=64, d=128, w=16, tau=0.05, dtype="bf16")


def _t(shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


Q = _t((1, 8, 64, 128))
KV = _t((1, 2, 64, 128))
ROWS = _t((1, 8, 64), torch.int32)
S = _t((1, 8, 64), torch.float32)
BUD = _t((1,), torch.int32)


@pytest.mark.parametrize("call,name", [
    (lambda: T.tsa_score(P, Q, Q), "k"),                                  # k with Hq heads
    (lambda: T.tsa_score(P, Q.float(), KV), "q"),                         # f32 data, bf16 problem
    (lambda: T.tsa_score(P, Q, KV, s=_t((1, 8, 63), torch.float32)), "s"),
    (lambda: T.tsa_budget(P, S, budget=_t((2,), torch.int32)), "budget"),
    (lambda: T.tsa_select(P, S, BUD, idx=_t((1, 8, 64), torch.int64)), "idx"),
    (lambda: T.tsa_select(P, S, BUD, rank=_t((1, 8, 32), torch.int32)), "rank"),
    (lambda: T.tsa_gather(P, Q, KV, KV, ROWS, BUD, kc=_t((1, 8, 32, 128))), "kc"),
    (lambda: T.tsa_attention(P, Q, KV, KV, BUD, 1), "k"),                 # compact needs Hq heads
    (lambda: T.tsa_attention(P, Q, KV, KV, BUD, 4, o=_t((1, 8, 64, 64))), "o"),
    (lambda: T.tsa_scatter(P, Q, _t((1, 8, 64), torch.float32)), "rank"),
    (lambda: T.tsa_forward(P, Q, KV, KV, budget=_t((1, 8), torch.int32)), "budget"),
    (lambda: T.tsa_forward_fused(P, Q, KV, _t((1, 2, 64, 64))), "v"),
    (lambda: T.tsa_attention_indexed(P, Q, KV, KV, _t((1, 8, 65), torch.int32), BUD), "idx"),
    (lambda: T.tsa_attention_qo_indexed(P, Q, KV, KV, ROWS, BUD), "k"),
    (lambda: T.tsa_zero_unselected(P, ROWS, _t((1, 8, 64, 128), torch.float32)), "o"),
])
def test_mismatch_is_refused(call, name):
    with pytest.raises(ValueError, match=rf"^{name}\b"):
        call()


def test_per_head_budget_shape():
    p = T.Problem(1, 8, 2, 64, 128, 16, 0.05, "bf16", T.TSA_FLAG_PER_HEAD_BUDGET)
    with pytest.raises(ValueError, match="^budget"):
        T.tsa_select(p, S, BUD)
    # the right shapes pass the binding's checks and stop at the device check
    with pytest.raises(ValueError, match="device memory"):
        T.tsa_select(p, S, _t((1, 8), torch.int32))


def test_bad_kv_group():
    with pytest.raises(ValueError, match="kv_group"):
        T.tsa_attention(P, Q, KV, KV, BUD, 3)
