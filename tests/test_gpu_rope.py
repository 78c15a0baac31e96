"""GPU parity of the rotary-position-embedding variant (the _rope entry
points) against the oracle: keys embedded at their cache positions before the
PCA rotation, the query at its own position.  Caches are built by the
oracle's float64 append with the same embedding; nothing from the GPU feeds
the oracle."""

import numpy as np
import pytest

import oracle
import synth
from gpu_cases import (TOL, OracleSrc, all_pairs, basis, check_decode, device_cache, make_case,
                       out_error, random_workload, src_of, to_dev, to_host, ulp_diff_bf16,
                       ulp_diff_f32)

pytestmark = pytest.mark.gpu

# (workload, S, S_max, rope base)
CASES = {
    "rope_mha": (synth.custom("rope_mha", 601, B=2, Hq=4, Hkv=4, S=700), 700, 720, 10000.0),
    "rope_gqa4": (synth.custom("rope_gqa4", 602, B=2, Hq=8, Hkv=2, S=1000), 1000, 1000, 500000.0),
    "rope_f32": (synth.custom("rope_f32", 603, B=1, Hq=2, Hkv=2, D=64, d=16, S=300, dtype="f32",
                              tau=8.0), 300, 310, 10000.0),
    "rope_long": (synth.custom("rope_long", 604, B=1, Hq=4, Hkv=2, S=5000), 5000, 5000, 10000.0),
    # the benchmark's --rope-base 10000 shape at full size (13B, S=3584)
    "rope_l2_13b_full": (synth.WORKLOADS["l2_13b_run"], 3584, 3584, 10000.0),
}
_cache = {}


def case(name):
    if name not in _cache:
        w, S, S_max, base = CASES[name]
        _cache[name] = (make_case(w, S, S_max, rope_base=base), base)
    return _cache[name]


def _paths(w):
    paths = [2]
    if w.Hq == w.Hkv:
        paths.append(1)
    if w.Hq // w.Hkv in (2, 4):
        paths.append(3)
    return paths


@pytest.mark.parametrize("name", sorted(CASES))
def test_rope_decode_matches_oracle(lib, name):
    c, base = case(name)
    cache = device_cache(lib, c)
    q = to_dev(c.q, c.w.dtype)
    P = to_dev(c.P, "f32")
    for q_pos in (c.S - 1, 3 * c.S + 17):  # the usual position, and one past the cache
        ref_out, ref_idx, ref_s = oracle.decode(c.q, c.slab, c.rest, c.v, c.P, c.k, c.w.dtype,
                                                S=c.S, rope=(base, q_pos))
        for path in _paths(c.w):
            out, idx = lib.decode(q, cache, P, c.k, path=path, rope_base=base, q_pos=q_pos)
            check_decode(c.w.dtype, c.k, out.cpu().numpy(), idx.cpu().numpy(), ref_out, ref_idx,
                         ref_s, all_pairs(c.w), src_of(c, (base, q_pos)))


@pytest.mark.parametrize("i", range(8))
def test_rope_decode_random_family(lib, i):
    # random shapes with embedded keys, the query at the last position, on AUTO
    # and every path that applies
    w, S, S_max = random_workload(200 + i)
    base = (10000.0, 500000.0)[i % 2]
    c = make_case(w, S, S_max, rope_base=base)
    k = max(1, min(int(w.k_f * S), S + 3))
    print(f"random rope case {i}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} d={w.d} S={S} k={k} "
          f"{w.dtype} base={base}", flush=True)
    cache = device_cache(lib, c)
    q, P = to_dev(c.q, w.dtype), to_dev(c.P, "f32")
    ref_out, ref_idx, ref_s = oracle.decode(c.q, c.slab, c.rest, c.v, c.P, k, w.dtype, S=S,
                                            rope=(base, S - 1))
    ran = 0
    for path in (0, 1, 2, 3, 4):
        try:
            lib.decode_path(w.B, w.Hq, w.Hkv, w.D, w.d, S, k, w.dtype, path)
        except lib.LokiError:
            continue
        out, idx = lib.decode(q, cache, P, k, path=path, rope_base=base)
        check_decode(w.dtype, k, out.cpu().numpy(), idx.cpu().numpy(), ref_out, ref_idx, ref_s,
                     all_pairs(w), src_of(c, (base, S - 1)))
        ran += 1
    assert ran >= 2


@pytest.mark.parametrize("name", sorted(CASES))
def test_rope_paths_select_identically(lib, name):
    """The embedded query is formed once per path with the same float64
    arithmetic and rounded once, so every path ranks with the same q'."""
    c, base = case(name)
    cache = device_cache(lib, c)
    q = to_dev(c.q, c.w.dtype)
    P = to_dev(c.P, "f32")
    res = [lib.decode(q, cache, P, c.k, path=p, rope_base=base) for p in _paths(c.w)]
    for out, idx in res[1:]:
        assert np.array_equal(idx.cpu().numpy(), res[0][1].cpu().numpy())
        assert np.max(np.abs(out.cpu().numpy() - res[0][0].cpu().numpy())) < 1e-5


@pytest.mark.parametrize("name", sorted(CASES))
def test_rope_dense_matches_oracle(lib, name):
    c, base = case(name)
    cache = device_cache(lib, c)
    out = lib.dense_decode(to_dev(c.q, c.w.dtype), cache, to_dev(c.P, "f32"), rope_base=base,
                           q_pos=c.S + 5).cpu().numpy()
    ref = oracle.dense_decode(c.q, c.slab, c.rest, c.v, c.P, c.w.dtype, S=c.S, rope=(base, c.S + 5))
    for b, h in all_pairs(c.w):
        assert out_error(c.w.dtype, out[b, h], ref[b, h]) <= TOL[c.w.dtype]


@pytest.mark.parametrize("wname", ["rope_mha", "rope_f32"])
@pytest.mark.parametrize("pos,T", [(0, 1), (5, 37), (250, 50), (4000, 3)])
def test_rope_append_matches_oracle(lib, wname, pos, T):
    import torch
    w, _, _, base = CASES[wname]
    P = basis(w)
    K, V = synth.raw_cache(w, T)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    cache = lib.KVCache(w.B, w.Hkv, pos + T + 2, w.D, w.d, tdt)
    lib.append(cache, to_dev(K, w.dtype), to_dev(V, w.dtype), to_dev(P, "f32"), pos=pos,
               rope_base=base)
    torch.cuda.synchronize()
    slab = to_host(cache.k_slab, w.dtype)[:, :, pos:pos + T]
    rest = to_host(cache.k_rest, w.dtype)[:, :, pos:pos + T]
    vv = to_host(cache.v, w.dtype)[:, :, pos:pos + T]
    for g in range(w.Hkv):
        rs, rr, rv = oracle.append(oracle.to_f64(K[:, g], w.dtype), oracle.to_f64(V[:, g], w.dtype),
                                   P[g].astype(np.float64), w.d, w.dtype, rope_base=base, pos=pos)
        for a, e in ((slab[:, g], rs), (rest[:, g], rr)):
            ud = ulp_diff_bf16(a, e) if w.dtype == "bf16" else ulp_diff_f32(a, e)
            assert ud.max() <= 1
            assert (ud == 0).mean() >= 0.999
        assert np.array_equal(vv[:, g], rv)
    # the embedding really was applied: it changes the stored keys
    plain = oracle.append(oracle.to_f64(K[:, 0], w.dtype), oracle.to_f64(V[:, 0], w.dtype),
                          P[0].astype(np.float64), w.d, w.dtype)[0]
    if pos > 0:
        assert not np.array_equal(slab[:, 0], plain)


@pytest.mark.parametrize("path", [1, 2], ids=["fused", "split"])
def test_rope_decode_step_matches_oracle(lib, path):
    """Append at pos = S - 1 with the key embedded there, query embedded at
    the same position, decode over S tokens; three steps in a row."""
    import torch
    w, S, S_max, base = CASES["rope_mha"]
    c = make_case(w, S - 3, S_max, rope_base=base)
    cache = device_cache(lib, c)
    P = to_dev(c.P, "f32")
    full = {nm: getattr(c, nm).copy() for nm in ("slab", "rest", "v")}
    for step in range(3):
        pos = S - 3 + step
        kn, vn = synth.new_tokens(w, 40 + step)
        for g in range(w.Hkv):
            s_, r_, v_ = oracle.append(oracle.to_f64(kn[:, g], w.dtype), oracle.to_f64(vn[:, g], w.dtype),
                                       c.P[g].astype(np.float64), w.d, w.dtype, rope_base=base, pos=pos)
            full["slab"][:, g, pos], full["rest"][:, g, pos], full["v"][:, g, pos] = s_[:, 0], r_[:, 0], v_[:, 0]
        q = synth.queries(w, step=40 + step)
        k = w.k_at(pos + 1)
        out, idx = lib.decode_step(to_dev(q, w.dtype), to_dev(kn[:, :, 0], w.dtype),
                                   to_dev(vn[:, :, 0], w.dtype), cache, P, k, path=path,
                                   rope_base=base)
        torch.cuda.synchronize()
        got = to_host(cache.k_slab, w.dtype)[:, :, pos]
        assert ulp_diff_bf16(got, full["slab"][:, :, pos]).max() <= 1
        ref_out, ref_idx, ref_s = oracle.decode(q, full["slab"], full["rest"], full["v"], c.P, k,
                                                w.dtype, S=pos + 1, rope=(base, pos))
        check_decode(w.dtype, k, out.cpu().numpy(), idx.cpu().numpy(), ref_out, ref_idx, ref_s,
                     all_pairs(w),
                     OracleSrc(q, full["slab"], full["rest"], full["v"], c.P, (base, pos)))


def test_rope_pre_and_post_rotary_bases_both_decode(lib):
    """Pre-rotary: the basis from keys before the embedding; post-rotary: from
    the same keys embedded at positions 0..n-1.  Either way the cache holds
    embedded keys and the decode matches the oracle with that basis."""
    import torch
    w, S, S_max, base = CASES["rope_gqa4"]
    Ks = [synth.calib_keys(w, g) for g in range(w.Hkv)]
    # both bases from the oracle's calibration: no library output enters the
    # oracle side
    pre = np.stack([oracle.calibrate(K)[0] for K in Ks]).astype(np.float32)
    post = np.stack([oracle.calibrate(oracle.rope_embed(K, np.arange(K.shape[0]), base))[0]
                     for K in Ks]).astype(np.float32)
    assert not np.allclose(pre, post, atol=1e-3)
    Kr, Vr = synth.raw_cache(w, S)
    q = synth.queries(w)
    for P in (pre, post):
        st = np.uint16
        slab = np.empty((w.B, w.Hkv, S, w.d), st)
        rest = np.empty((w.B, w.Hkv, S, w.D - w.d), st)
        vv = np.empty((w.B, w.Hkv, S, w.D), st)
        tdt = torch.bfloat16
        cache = lib.KVCache(w.B, w.Hkv, S, w.D, w.d, tdt)
        lib.append(cache, to_dev(Kr, w.dtype), to_dev(Vr, w.dtype), to_dev(P, "f32"), pos=0,
                   rope_base=base)
        for g in range(w.Hkv):
            slab[:, g], rest[:, g], vv[:, g] = oracle.append(
                oracle.to_f64(Kr[:, g], w.dtype), oracle.to_f64(Vr[:, g], w.dtype),
                P[g].astype(np.float64), w.d, w.dtype, rope_base=base, pos=0)
        # decode from the GPU-appended cache against the oracle's own cache
        out, idx = lib.decode(to_dev(q, w.dtype), cache, to_dev(P, "f32"), w.k, rope_base=base)
        ref_out, ref_idx, ref_s = oracle.decode(q, slab, rest, vv, P, w.k, w.dtype, S=S,
                                                rope=(base, S - 1))
        check_decode(w.dtype, w.k, out.cpu().numpy(), idx.cpu().numpy(), ref_out, ref_idx, ref_s,
                     all_pairs(w), OracleSrc(q, slab, rest, vv, P, (base, S - 1)))


@pytest.mark.parametrize("path", [1, 2, 3], ids=["fused", "split", "union"])
def test_rope_decode_step_replays_from_a_captured_graph(lib, path):
    """The RoPE step launches only kernels, so it captures into a HIP graph:
    three replays, with eager work between them, each writing the same slot
    and producing the same output as an eager step on a fresh copy."""
    import torch
    w, S, S_max, base = CASES["rope_gqa4"]
    if path == 1:
        w, S, S_max, base = CASES["rope_mha"]
    c, _ = case("rope_gqa4" if path != 1 else "rope_mha")
    P = to_dev(c.P, "f32")
    kn, vn = synth.new_tokens(w, 77)
    q = to_dev(synth.queries(w, step=77), w.dtype)
    kd, vd = to_dev(kn[:, :, 0], w.dtype), to_dev(vn[:, :, 0], w.dtype)
    pos = S - 1
    k = w.k_at(pos + 1)
    ws = lib.alloc_workspace(w.B, w.Hq, c.S_max, w.D, k, torch.device("cuda"))
    ref_cache = device_cache(lib, c)
    ref_out, ref_idx = lib.decode_step(q, kd, vd, ref_cache, P, k, pos=pos, workspace=ws, path=path,
                                       rope_base=base)
    ref_out, ref_idx = ref_out.cpu().numpy(), ref_idx.cpu().numpy()
    ref_slab = to_host(ref_cache.k_slab, w.dtype)
    cache = device_cache(lib, c)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.B, w.Hq, k), dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up on the capture stream
        lib.decode_step(q, kd, vd, cache, P, k, pos=pos, out=out, idx=idx, workspace=ws, path=path,
                        rope_base=base)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.decode_step(q, kd, vd, cache, P, k, pos=pos, out=out, idx=idx, workspace=ws, path=path,
                        rope_base=base)
    for rep in range(3):
        out.fill_(float("nan"))
        idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ref_idx), f"replay {rep}"
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref_out.view(np.uint32)), rep
        assert np.array_equal(to_host(cache.k_slab, w.dtype), ref_slab), rep
        lib.decode(q, cache, P, 7, workspace=ws, path=2, rope_base=base)  # eager work between
        torch.cuda.synchronize()
