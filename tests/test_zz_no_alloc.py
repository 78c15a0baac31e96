"""The allocation-free decode (loki_decode_noalloc) against loki_decode_ex
with a caller workspace: the same selections and bit-identical outputs,
over two calls in a row whose second is smaller (it finds the first call's
contents in the library's scratch), on every path that uses the scratch
(the fused path for its grouped ranking), and against the oracle.  A shape whose workspace exceeds the scratch is
refused before anything is launched."""

import numpy as np
import pytest

import synth
from gpu_cases import all_pairs, check_decode, device_cache, make_case, src_of, to_dev

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402

CALLS = [  # (workload, paths): the first call is the larger one
    (synth.custom("noalloc_big", 801, B=4, Hq=32, Hkv=8, S=8192, k_f=0.25), [0, 1, 2, 3, 4]),
    (synth.custom("noalloc_small", 802, B=2, Hq=8, Hkv=2, S=1500, k_f=0.25), [0, 2, 3, 4]),
    (synth.custom("noalloc_f32", 803, B=1, Hq=4, Hkv=2, D=64, d=16, S=700, k_f=0.2,
                  dtype="f32"), [2, 3, 4]),
]


def _pair(lib, c, path):
    import torch
    w = c.w
    q, P = to_dev(c.q, w.dtype), to_dev(c.P, "f32")
    cache = device_cache(lib, c)
    kk = min(c.k, c.S)
    ws = lib.alloc_workspace(w.B, w.Hq, c.S_max, w.D, kk, torch.device("cuda"))
    ref_out, ref_idx = lib.decode(q, cache, P, c.k, workspace=ws, path=path)
    out = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((w.B, w.Hq, kk), -1, dtype=torch.int32, device="cuda")
    lib.decode_noalloc(q, cache, P, c.k, out, idx, path=path)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), idx.cpu().numpy(), ref_out.cpu().numpy(), ref_idx.cpu().numpy())


def test_noalloc_matches_decode_with_workspace_over_successive_calls(lib):
    for w, paths in CALLS:
        c = make_case(w)
        o_ref, i_ref, s_ref = oracle.decode(c.q, c.slab, c.rest, c.v, c.P, c.k, w.dtype, S=c.S)
        for path in paths:
            print(f"noalloc: {w.name} path {path}", flush=True)
            out, idx, ex_out, ex_idx = _pair(lib, c, path)
            assert np.array_equal(idx, ex_idx), (w.name, path)
            assert np.array_equal(out.view(np.uint32), ex_out.view(np.uint32)), (w.name, path)
            check_decode(w.dtype, c.k, out, idx, o_ref, i_ref, s_ref, all_pairs(w), src_of(c))


def test_noalloc_refuses_shapes_beyond_its_scratch(lib):
    import torch
    w = synth.custom("noalloc_over", 804, B=2, Hq=8, Hkv=8, S=600, k_f=0.25)
    c = make_case(w)
    cache = device_cache(lib, c)
    q, P = to_dev(c.q, w.dtype), to_dev(c.P, "f32")
    out = torch.zeros((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    idx = torch.zeros((w.B, w.Hq, c.k), dtype=torch.int32, device="cuda")
    # S beyond the scratch: the score rows alone need B*Hq*S*4 bytes
    S_big = (lib.NOALLOC_SCRATCH_BYTES // (w.B * w.Hq * 4)) + 1024
    assert lib.workspace_size(w.B, w.Hq, S_big, w.D, 1) > lib.NOALLOC_SCRATCH_BYTES
    big = lib.KVCache(w.B, w.Hkv, S_big, w.D, w.d, torch.bfloat16)
    big.length = S_big
    with pytest.raises(lib.LokiError) as e:
        lib.decode_noalloc(q, big, P, 10, out, idx[:, :, :10].contiguous(), path=2)
    assert e.value.status == lib.LOKI_EWORKSPACE
    # the fused path needs no scratch at all
    lib.decode_noalloc(q, cache, P, c.k, out, idx, path=1)
    ref_out, ref_idx = lib.decode(q, cache, P, c.k, path=1)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ref_idx.cpu().numpy())
    assert np.array_equal(out.cpu().numpy(), ref_out.cpu().numpy())
