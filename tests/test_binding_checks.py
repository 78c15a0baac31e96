"""CPU checks of the Python binding's argument validation: the C ABI sees
only pointers, so every tensor whose extent, dtype, layout or device does
not match the cache must be refused before any call into the library."""

import os

import pytest
import torch

import sparse_attention_decode_loki_amd as loki

B, HKV, HQ, SMAX, D, d = 2, 2, 4, 64, 128, 32


@pytest.fixture(scope="module")
def built():
    if not os.path.exists(loki.LIB_PATH):
        pytest.fail("libloki.so not built: run python -m sparse_attention_decode_loki_amd.build_lib")
    loki.load()


@pytest.fixture()
def cache(built):
    c = loki.KVCache(B, HKV, SMAX, D, d, torch.bfloat16, device="cpu")
    c.length = 40
    return c


def _q(hq=HQ, dt=torch.bfloat16, dd=D, b=B):
    return torch.zeros((b, hq, dd), dtype=dt)


def _P(hkv=HKV, dd=D, dt=torch.float32):
    return torch.zeros((hkv, dd, dd), dtype=dt)


def _raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_decode_rejects_bad_queries(cache):
    _raises("shape", loki.decode, _q(b=B + 1), cache, _P(), 10)
    _raises("shape", loki.decode, _q(dd=64), cache, _P(), 10)
    _raises("not a multiple", loki.decode, _q(hq=3), cache, _P(), 10)
    _raises(r"\[B, Hq, D\]", loki.decode, torch.zeros((B, HQ * D), dtype=torch.bfloat16), cache,
            _P(), 10)
    _raises("bfloat16", loki.decode, _q(dt=torch.float32), cache, _P(), 10)
    strided = torch.zeros((B, HQ, 2 * D), dtype=torch.bfloat16)[:, :, ::2]
    _raises("contiguous", loki.decode, strided, cache, _P(), 10)


def test_decode_rejects_bad_basis(cache):
    _raises("P must have shape", loki.decode, _q(), cache, _P(hkv=HQ), 10)   # one basis per q head
    _raises("P must have shape", loki.decode, _q(), cache, _P(dd=64), 10)
    _raises("P must be torch.float32", loki.decode, _q(), cache, _P(dt=torch.bfloat16), 10)


def test_decode_rejects_bad_outputs(cache):
    out_bad = torch.zeros((B, HQ, D - 1), dtype=torch.float32)
    _raises("out must have shape", loki.decode, _q(), cache, _P(), 10, out=out_bad)
    out_bf = torch.zeros((B, HQ, D), dtype=torch.bfloat16)
    _raises("out must be torch.float32", loki.decode, _q(), cache, _P(), 10, out=out_bf)
    idx_short = torch.zeros((B, HQ, 9), dtype=torch.int32)
    _raises("idx must have shape", loki.decode, _q(), cache, _P(), 10, idx=idx_short)
    idx_i64 = torch.zeros((B, HQ, 10), dtype=torch.int64)
    _raises("idx must be torch.int32", loki.decode, _q(), cache, _P(), 10, idx=idx_i64)
    # k > S keeps S tokens: idx must then have S columns
    idx_k = torch.zeros((B, HQ, 50), dtype=torch.int32)
    _raises("idx must have shape", loki.decode, _q(), cache, _P(), 50, idx=idx_k)


def test_host_tensors_refused(cache):
    # every shape right, but host memory: refused before the library sees it
    _raises("device tensor", loki.decode, _q(), cache, _P(), 10)
    _raises("device tensor", loki.dense_decode, _q(), cache, _P())
    _raises("device tensor", loki.DecodePlan, _q(), cache, _P(), 10)


def test_step_and_append_reject_bad_new_tokens(cache):
    kn = torch.zeros((B, HKV, D), dtype=torch.bfloat16)
    _raises("k_new must have shape", loki.decode_step, _q(), kn[:1], kn, cache, _P(), 10)
    _raises(r"k_new must be \[B, Hkv, D\]", loki.decode_step, _q(), kn[:, :, None], kn, cache,
            _P(), 10)
    _raises("v_new must have shape", loki.decode_step, _q(), kn, kn[:, :1], cache, _P(), 10)
    _raises("v_new must be torch.bfloat16", loki.StepPlan, _q(), kn, kn.float(), cache, _P(), 10,
            pos=40)
    kt = torch.zeros((B, HKV, 3, D), dtype=torch.bfloat16)
    _raises(r"k_new must be \[B, Hkv, T, D\]", loki.append, cache, kn, kn, _P())
    _raises("v_new must have shape", loki.append, cache, kt, kt[:, :, :2], _P())
    _raises("P must have shape", loki.AppendPlan, cache, kt, kt, _P(hkv=1), 0)


def test_other_entry_points_check_shapes(cache):
    _raises("scores must have shape", loki.scores, _q(), cache, _P(),
            out=torch.zeros((B, HQ, 39), dtype=torch.float32))
    _raises("idx must have shape", loki.attend_indices, _q(), cache, _P(),
            torch.zeros((B, HQ + 1, 5), dtype=torch.int32))
    _raises(r"idx must be \[B, Hq, k\]", loki.attend_indices, _q(), cache, _P(),
            torch.zeros((B * HQ, 5), dtype=torch.int32))
    _raises("out must have shape", loki.DensePlan, _q(), cache, _P(),
            out=torch.zeros((B, HQ, D, 1), dtype=torch.float32))
    _raises(r"S must be in \[1, 8\]", loki.topk, torch.zeros((3, 8)), 2, S=9)
    _raises(r"scores must be \[rows, ld\]", loki.topk, torch.zeros(8), 2)
