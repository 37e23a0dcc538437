"""The C ABI on the host: symbols, workspace sizing, validation (no GPU needed).

Only invalid arguments are passed with placeholder pointers: validation
rejects them before anything is enqueued, so no kernel ever runs here.
"""
import ctypes
import os
import re

import pytest

from token_sparse_attention_proxy_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tsa.h")
FAKE = 1 << 20          # aligned placeholder pointer value; never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from token_sparse_attention_proxy_amd import build
        build.build()
    return _lib.load()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tsa_[a-z_]+)\s*\(", text)))


def prob(**kw):
    base = dict(B=1, Hq=8, Hkv=2, L=1000, d=128, w=64, tau=0.05, dtype=_lib.TSA_BF16)
    base.update(kw)
    return _lib.TsaProblem(**base)


def test_exports_every_declared_symbol(lib):
    syms = declared_symbols()
    assert set(syms) == set(_lib.EXPORTS), syms
    for name in syms:
        assert hasattr(lib, name), name


def test_nm_lists_exports():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    for name in declared_symbols():
        assert re.search(rf"\bT {name}$", out, re.M), name


def test_version_and_status_strings(lib):
    assert lib.tsa_version().decode().startswith("tsa ")
    names = [lib.tsa_status_string(i).decode() for i in range(5)]
    assert names == ["TSA_OK", "TSA_ERR_INVALID_ARG", "TSA_ERR_UNSUPPORTED", "TSA_ERR_WORKSPACE",
                     "TSA_ERR_HIP"]


def test_workspace_sizes(lib):
    p = prob()
    step = lib.tsa_workspace_bytes(ctypes.byref(p))
    fwd = lib.tsa_forward_workspace_bytes(ctypes.byref(p))
    assert step > 0 and step % 256 == 0
    # forward scratch holds scores, rank and the compact K and V (not Q or O)
    assert step + 2 * 4 * 8 * 1000 + 2 * 8 * 1000 * 128 * 2 <= fwd
    assert fwd < step + 2 * 4 * 8 * 1000 + 3 * 8 * 1000 * 128 * 2
    assert lib.tsa_workspace_bytes(ctypes.byref(prob(Hkv=3))) == 0
    assert lib.tsa_workspace_bytes(None) == 0
    # the fused forward needs the step scratch, scores and rank, not the compact tensors
    fused = lib.tsa_fused_workspace_bytes(ctypes.byref(p))
    assert step + 2 * 4 * 8 * 1000 <= fused < step + 2 * 4 * 8 * 1000 + 1024
    assert fused % 256 == 0 and fused < fwd
    assert lib.tsa_fused_workspace_bytes(None) == 0


def test_block_mask_words(lib):
    # L=1000: 16 blocks of 64, one word per mask row
    assert lib.tsa_block_mask_words(ctypes.byref(prob())) == 1 * 8 * 16 * 1
    # L=131072: 2048 blocks, 64 words per row
    assert lib.tsa_block_mask_words(ctypes.byref(prob(Hq=32, Hkv=8, L=131072))) == 32 * 2048 * 64
    assert lib.tsa_block_mask_words(ctypes.byref(prob(Hkv=3))) == 0


def test_workspace_per_head_budget(lib):
    """Per-head budgets need one mass row per head instead of one per sequence."""
    g = lib.tsa_workspace_bytes(ctypes.byref(prob()))
    ph = lib.tsa_workspace_bytes(ctypes.byref(prob(flags=_lib.TSA_FLAG_PER_HEAD_BUDGET)))
    assert ph - g >= 8 * (8 - 1) * 1000 - 512     # up to alignment
    for f in (_lib.TSA_FLAG_NONCAUSAL_PROXY, _lib.TSA_FLAG_KEEP_WINDOW):
        assert lib.tsa_workspace_bytes(ctypes.byref(prob(flags=f))) == g


def test_workspace_scales_with_headline_shape(lib):
    p = prob(Hq=32, Hkv=8, L=131072, w=64)
    fwd = lib.tsa_forward_workspace_bytes(ctypes.byref(p))
    tens = 32 * 131072 * 128 * 2
    assert 2 * tens < fwd < 2 * tens + 64 * 2 ** 20


BAD_PROBLEMS = [
    (dict(B=0), _lib.TSA_ERR_INVALID_ARG),
    (dict(Hq=0), _lib.TSA_ERR_INVALID_ARG),
    (dict(Hkv=3), _lib.TSA_ERR_INVALID_ARG),
    (dict(L=0), _lib.TSA_ERR_INVALID_ARG),
    (dict(w=0), _lib.TSA_ERR_INVALID_ARG),
    (dict(w=1001), _lib.TSA_ERR_INVALID_ARG),
    (dict(tau=-0.01), _lib.TSA_ERR_INVALID_ARG),
    (dict(tau=1.0), _lib.TSA_ERR_INVALID_ARG),
    (dict(tau=float("nan")), _lib.TSA_ERR_INVALID_ARG),
    (dict(Hq=8192, Hkv=8192), _lib.TSA_ERR_INVALID_ARG),
    (dict(d=96), _lib.TSA_ERR_UNSUPPORTED),
    (dict(d=256), _lib.TSA_ERR_UNSUPPORTED),
    (dict(dtype=7), _lib.TSA_ERR_UNSUPPORTED),
    (dict(L=4096, w=2945), _lib.TSA_ERR_UNSUPPORTED),
    (dict(B=16, Hq=4096, Hkv=4096), _lib.TSA_ERR_UNSUPPORTED),     # B*Hq = 65536 > grid y
    (dict(flags=8), _lib.TSA_ERR_UNSUPPORTED),
    (dict(flags=-1), _lib.TSA_ERR_UNSUPPORTED),
]


def _call_all(lib, p, ptr=FAKE, ws_bytes=1 << 40, kv_group=1):
    P = ctypes.byref(p)
    return {
        "score": lib.tsa_score(P, ptr, ptr, ptr, ptr, ws_bytes, None),
        "budget": lib.tsa_budget(P, ptr, ptr, ptr, ws_bytes, None),
        "select": lib.tsa_select(P, ptr, ptr, ptr, ptr, ptr, ws_bytes, None),
        "gather": lib.tsa_gather(P, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, None),
        "gather_kv": lib.tsa_gather_kv(P, ptr, ptr, ptr, ptr, ptr, None),
        "attention": lib.tsa_attention(P, ptr, ptr, ptr, ptr, kv_group, ptr, None),
        "scatter": lib.tsa_scatter(P, ptr, ptr, ptr, None),
        "forward": lib.tsa_forward(P, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ws_bytes, None),
        "attention_indexed": lib.tsa_attention_indexed(P, ptr, ptr, ptr, ptr, ptr, ptr, None),
        "attention_qo_indexed": lib.tsa_attention_qo_indexed(P, ptr, ptr, ptr, ptr, ptr, ptr, None),
        "forward_fused": lib.tsa_forward_fused(P, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ws_bytes,
                                               None),
        "zero_unselected": lib.tsa_zero_unselected(P, ptr, ptr, None),
        "attention_block_sparse": lib.tsa_attention_block_sparse(P, ptr, ptr, ptr, ptr, kv_group,
                                                                 ptr, ptr, None),
    }


@pytest.mark.parametrize("kw,status", BAD_PROBLEMS, ids=[str(k) for k, _ in BAD_PROBLEMS])
def test_bad_problem_rejected_everywhere(lib, kw, status):
    res = _call_all(lib, prob(**kw))
    assert set(res.values()) == {status}, res
    assert lib.tsa_last_error().decode() != ""


def test_null_problem(lib):
    assert lib.tsa_score(None, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == _lib.TSA_ERR_INVALID_ARG
    assert "NULL" in lib.tsa_last_error().decode()


def test_null_and_misaligned_pointers(lib):
    p = prob()
    res = _call_all(lib, p, ptr=None)
    assert set(res.values()) == {_lib.TSA_ERR_INVALID_ARG}, res
    res = _call_all(lib, p, ptr=FAKE + 8)
    assert set(res.values()) == {_lib.TSA_ERR_INVALID_ARG}, res
    assert "aligned" in lib.tsa_last_error().decode()


def test_workspace_too_small(lib):
    p = prob()
    P = ctypes.byref(p)
    need = lib.tsa_workspace_bytes(P)
    for st in [lib.tsa_score(P, FAKE, FAKE, FAKE, FAKE, need - 1, None),
               lib.tsa_budget(P, FAKE, FAKE, FAKE, need - 1, None),
               lib.tsa_select(P, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None)]:
        assert st == _lib.TSA_ERR_WORKSPACE
    fneed = lib.tsa_forward_workspace_bytes(P)
    assert lib.tsa_forward(P, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, fneed - 1, None) == \
        _lib.TSA_ERR_WORKSPACE
    uneed = lib.tsa_fused_workspace_bytes(P)
    assert lib.tsa_forward_fused(P, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, uneed - 1, None) == \
        _lib.TSA_ERR_WORKSPACE
    # misaligned workspace
    assert lib.tsa_score(P, FAKE, FAKE, FAKE, FAKE + 16, need, None) == _lib.TSA_ERR_WORKSPACE


def test_bad_kv_group(lib):
    p = prob()
    P = ctypes.byref(p)
    for g in (0, -1, 3, 16):
        assert lib.tsa_attention(P, FAKE, FAKE, FAKE, None, g, FAKE, None) == _lib.TSA_ERR_INVALID_ARG


def test_injected_launch_failure_propagates(lib, monkeypatch):
    """A host-forced launch failure surfaces as TSA_ERR_HIP and as TsaError in Python."""
    monkeypatch.setenv("TSA_FAULT_INJECT", "launch")
    p = prob()
    res = _call_all(lib, p)
    assert set(res.values()) == {_lib.TSA_ERR_HIP}, res
    assert "injected" in lib.tsa_last_error().decode()
    with pytest.raises(_lib.TsaError) as ei:
        _lib.check(res["forward"], "tsa_forward")
    assert ei.value.name == "TSA_ERR_HIP"


def test_last_error_is_per_thread(lib):
    """Each thread reads back the detail of its own failed call, whatever the others did."""
    import threading
    gate = threading.Barrier(2)
    seen = {}

    def null_problem():
        lib.tsa_score(None, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
        gate.wait()
        seen["null"] = lib.tsa_last_error().decode()

    def misaligned():
        lib.tsa_scatter(ctypes.byref(prob()), FAKE + 8, FAKE, FAKE, None)
        gate.wait()
        seen["misaligned"] = lib.tsa_last_error().decode()

    threads = [threading.Thread(target=f) for f in (null_problem, misaligned)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert "NULL" in seen["null"] and "aligned" not in seen["null"], seen
    assert "aligned" in seen["misaligned"] and "NULL" not in seen["misaligned"], seen


def test_gather_without_q_passes_validation(lib, monkeypatch):
    """qc = NULL asks for K and V only: validation accepts it (the injected launch failure is
    what comes back), while a NULL kc is still rejected."""
    monkeypatch.setenv("TSA_FAULT_INJECT", "launch")
    P = ctypes.byref(prob())
    assert lib.tsa_gather(P, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == _lib.TSA_ERR_HIP
    assert lib.tsa_gather(P, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == \
        _lib.TSA_ERR_INVALID_ARG
    assert "kc" in lib.tsa_last_error().decode()


def test_score_tile_bound(lib, monkeypatch):
    """bf16 scoring holds at most 92 proxy-row tiles of 32 rows per query head in LDS: 92 pass
    validation (the injected launch failure comes back), 93 are unsupported, whatever the
    number of query heads per KV head; fp32 has no bound."""
    monkeypatch.setenv("TSA_FAULT_INJECT", "launch")

    def score(**kw):
        p = prob(**kw)
        return lib.tsa_score(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert score(Hq=2, Hkv=2, L=4096, w=92 * 32) == _lib.TSA_ERR_HIP
    assert score(Hq=2, Hkv=2, L=4096, w=92 * 32 + 1) == _lib.TSA_ERR_UNSUPPORTED
    assert score(Hq=4, Hkv=1, L=4096, w=92 * 32) == _lib.TSA_ERR_HIP
    assert score(Hq=64, Hkv=1, L=4096, w=64) == _lib.TSA_ERR_HIP         # 128 tiles per KV head
    assert score(Hq=64, Hkv=1, L=4096, w=92 * 32 + 1) == _lib.TSA_ERR_UNSUPPORTED
    assert score(Hq=4, Hkv=1, L=4096, w=92 * 32 + 1, dtype=_lib.TSA_F32) == _lib.TSA_ERR_HIP
    assert score(Hq=2, Hkv=2, L=4096, w=4096, dtype=_lib.TSA_F32) == _lib.TSA_ERR_HIP


PROBE_HEADER = os.path.join(ROOT, "include", "tsa_probe.h")


def test_probe_library_exports_its_header():
    if not os.path.exists(_lib.PROBE_PATH):
        from token_sparse_attention_proxy_amd import build
        build.build()
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    syms = sorted(set(re.findall(r"\b(tsa_[a-z_0-9]+)\s*\(", text)))
    assert set(syms) == set(_lib.PROBE_EXPORTS), syms
    probe = _lib.load_probe()
    for name in syms:
        assert hasattr(probe, name), name


def test_probe_rejects_bad_arguments_without_launching():
    probe = _lib.load_probe()
    flops = ctypes.c_double(0.0)
    # null sink, null flops, iters < 1: rejected before any device query or launch
    assert probe.tsa_probe_mfma_bf16(1, 10, None, 1 << 20, ctypes.byref(flops), None) == 1
    assert probe.tsa_probe_mfma_bf16(1, 10, FAKE, 1 << 20, None, None) == 1
    assert probe.tsa_probe_mfma_bf16(1, 0, FAKE, 1 << 20, ctypes.byref(flops), None) == 1
