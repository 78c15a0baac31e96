"""GPU parity: the HIP library, called through its C ABI, against the CPU
oracle on the same seeded inputs.

Stages are checked one at a time (ranking scores, selection, attention over
a given index set, append, dense baseline) and end to end (both decode
paths), at sizes that span several tiles and ragged tails, on edge cases,
and at the full benchmark shapes on every (sequence, head) pair.
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_cases import (TOL, OracleSrc, all_pairs, check_decode, check_rounded_rotation,
                       device_cache, make_case, out_error, random_workload, src_of, to_dev,
                       to_host, ulp_diff_bf16, ulp_diff_f32)

pytestmark = pytest.mark.gpu

# small shapes: (name, workload kwargs, S, S_max)
SMALL = {
    "tiny": (synth.WORKLOADS["tiny"], None, None),
    "ragged_gqa2": (synth.custom("ragged_gqa2", 101, B=2, Hq=6, Hkv=3, S=1000), 1000, 1100),
    "full_rank_f32": (synth.custom("full_rank_f32", 102, B=1, Hq=2, Hkv=2, D=64, d=64, S=300,
                                   dtype="f32", tau=8.0), 300, 301),
    "d8_bf16": (synth.custom("d8_bf16", 103, B=3, Hq=4, Hkv=4, d=8, S=777), 777, 800),
    "d64_D64_bf16": (synth.custom("d64_D64_bf16", 104, B=2, Hq=4, Hkv=1, D=64, d=16, S=513), 513, 600),
    "gqa8": (synth.custom("gqa8", 105, B=2, Hq=8, Hkv=1, S=640), 640, 640),
    "gqa5": (synth.custom("gqa5", 106, B=1, Hq=10, Hkv=2, S=333, k_f=0.3), 333, 340),
    "sinks": (synth.custom("sinks", 107, B=2, Hq=8, Hkv=2, S=2000, sinks=4), 2000, 2048),
    "S1": (synth.custom("S1", 108, B=2, Hq=2, Hkv=2, S=1), 1, 8),
    "long_5000": (synth.custom("long_5000", 109, B=1, Hq=2, Hkv=2, S=5000, k_f=0.5), 5000, 5000),
    "long_20000": (synth.custom("long_20000", 110, B=1, Hq=2, Hkv=1, S=20000, d=64, k_f=0.125,
                                tau=48.0), 20000, 20000),
    "f32_D128": (synth.custom("f32_D128", 111, B=2, Hq=2, Hkv=2, S=600, dtype="f32", d=16), 600, 640),
    "gqa4_f32": (synth.custom("gqa4_f32", 112, B=2, Hq=8, Hkv=2, D=64, d=16, S=900, dtype="f32",
                              tau=8.0), 900, 960),
    # bf16 with d < 32 at D = 128: the union gather takes its VALU kernel
    "gqa4_d16": (synth.custom("gqa4_d16", 113, B=2, Hq=8, Hkv=2, d=16, S=700), 700, 720),
    # more rows than compute units: on the sliced path 256 whole rows and a
    # remainder of 32 (40) rows in slices that share the ranking
    "tail_rows_288": (synth.custom("tail_rows_288", 114, B=2, Hq=144, Hkv=144, S=700), 700, 720),
    "tail_gqa_296": (synth.custom("tail_gqa_296", 115, B=1, Hq=296, Hkv=74, S=2100), 2100, 2100),
}


def union_applies(w):
    """The union gather takes 2 or 4 query heads per KV head."""
    return w.Hq // w.Hkv in (2, 4)

_cases = {}


def case(name):
    if name not in _cases:
        w, S, S_max = SMALL[name]
        _cases[name] = make_case(w, S, S_max)
    return _cases[name]


def _P(c):
    return to_dev(c.P, "f32")


def _q(c):
    return to_dev(c.q, c.w.dtype)


# ------------------------------------------------------------------ scores --

@pytest.mark.parametrize("name", sorted(SMALL))
def test_scores_match_oracle(lib, name):
    c = case(name)
    cache = device_cache(lib, c)
    s = lib.scores(_q(c), cache, _P(c)).cpu().numpy()
    _, _, ref_s = oracle.decode(c.q, c.slab, c.rest, c.v, c.P, 1, c.w.dtype, S=c.S)
    assert s.shape == ref_s.shape
    # float32 sums of d products against the float64 value
    err = np.abs(s - ref_s).max(axis=-1)
    mag = np.abs(ref_s).max(axis=-1)
    assert np.all(err <= 1e-5 * np.maximum(mag, 1.0)), (err / np.maximum(mag, 1.0)).max()


# --------------------------------------------------------------- selection --

TOPK_CASES = [
    # (kind, S, ld, k)
    ("normal", 256, 256, 64), ("normal", 1000, 1000, 250), ("normal", 1001, 1004, 1),
    ("normal", 4096, 4096, 1024), ("normal", 4097, 4100, 1023), ("normal", 3584, 3584, 896),
    ("normal", 8192, 8192, 2048), ("normal", 12289, 12292, 3000), ("normal", 32768, 32768, 4096),
    ("dup", 777, 780, 300), ("dup", 5000, 5000, 2500), ("dup", 20000, 20000, 1),
    ("zeros", 300, 300, 150), ("zeros", 9000, 9000, 4000), ("sorted", 2048, 2048, 512),
    ("normal", 50, 52, 50), ("normal", 50, 52, 70), ("normal", 1, 4, 1), ("normal", 33, 36, 32),
    ("dup", 32768, 32768, 16384), ("normal", 32769, 32772, 4096), ("normal", 40000, 40000, 5000),
]


@pytest.mark.parametrize("kind,S,ld,k", TOPK_CASES)
def test_topk_bit_exact(lib, kind, S, ld, k):
    import torch
    rows = 5
    host = np.zeros((rows, ld), np.float32)
    for r in range(rows):
        host[r, :S] = synth.score_vector(1000 * r + S + k, S, kind)
        host[r, S:] = 1e30  # beyond S: must be ignored
    idx = lib.topk(torch.from_numpy(host).cuda(), k, S=S).cpu().numpy()
    for r in range(rows):
        want = oracle.select_topk(host[r, :S].astype(np.float64), k)
        assert np.array_equal(idx[r].astype(np.int64), want), f"row {r}"


def test_topk_all_equal_and_negative_zero(lib):
    import torch
    S = 3000
    host = np.zeros((3, S), np.float32)
    host[1, ::2] = -0.0
    host[2] = -1.5
    idx = lib.topk(torch.from_numpy(host).cuda(), 1000).cpu().numpy()
    for r in range(3):
        assert idx[r].tolist() == list(range(1000))


def _crossing_bin_row(rng, S, k, n, kept, values):
    """A float32 row whose k-th largest value lies in one first-digit bin
    (sign, exponent and the top two mantissa bits of the order key) holding
    exactly n scores, `kept` of which are selected: k - kept scores far
    above, n in [1, 1.25) drawn from `values`, the rest below."""
    row = np.empty(S, np.float32)
    row[:] = rng.uniform(-4.0, 0.5, S)
    pos = rng.permutation(S)
    row[pos[:k - kept]] = rng.uniform(100.0, 1000.0, k - kept)
    row[pos[k - kept:k - kept + n]] = rng.choice(values, n)
    return row


@pytest.mark.parametrize("n", [1, 2, 3, 64, 255, 256, 257, 600])
@pytest.mark.parametrize("ties", [False, True])
def test_topk_crossing_bin_sizes(lib, n, ties):
    """Rows whose k-th largest score sits in a first-digit bin of n scores
    (the bin the selection resolves further, or ranks directly when small),
    with and without repeated values inside it, give the oracle's set."""
    import torch
    rng = np.random.default_rng(7 * n + ties)
    S, k = 4096, 1024
    values = (np.float32(1.0) + np.arange(4, dtype=np.float32) / 32) if ties else \
        rng.uniform(1.0, 1.2, 4096).astype(np.float32)
    rows = [_crossing_bin_row(rng, S, k, n, kept, values)
            for kept in sorted({1, (n + 1) // 2, n})]
    host = np.stack(rows)
    idx = lib.topk(torch.from_numpy(host).cuda(), k).cpu().numpy()
    for r in range(host.shape[0]):
        want = oracle.select_topk(host[r].astype(np.float64), k)
        assert np.array_equal(idx[r].astype(np.int64), want), f"row {r}"


@pytest.mark.parametrize("kind", ["denormal", "huge_range", "outliers", "two_values", "tiny_range"])
def test_topk_extreme_value_ranges(lib, kind):
    """Rows whose value range is zero, denormal, beyond float32 (max - min
    overflows) or dominated by a few outliers: selections whose first pass
    cannot bin linearly, or whose crossing bin is crowded, still match the
    oracle."""
    import torch
    rng = np.random.default_rng(["denormal", "huge_range", "outliers", "two_values",
                                 "tiny_range"].index(kind) + 500)
    S, k = 5000, 1234
    if kind == "denormal":
        row = (rng.integers(1, 1 << 20, S) * np.float32(1e-45)).astype(np.float32)
    elif kind == "huge_range":
        row = rng.standard_normal(S).astype(np.float32)
        row[rng.integers(0, S, 3)] = np.float32(3e38)
        row[rng.integers(0, S, 3)] = np.float32(-3e38)
    elif kind == "outliers":
        row = rng.standard_normal(S).astype(np.float32)
        row[:4] = np.float32(1e6)
    elif kind == "two_values":
        row = np.where(rng.random(S) < 0.5, np.float32(2.0), np.float32(-7.0)).astype(np.float32)
    else:
        row = (np.float32(1.0) + rng.integers(0, 64, S).astype(np.float32) * np.float32(2 ** -23))
    host = np.stack([row, row[::-1].copy()])
    assert np.all(np.isfinite(host))
    idx = lib.topk(torch.from_numpy(host).cuda(), k).cpu().numpy()
    for r in range(2):
        want = oracle.select_topk(host[r].astype(np.float64), k)
        assert np.array_equal(idx[r].astype(np.int64), want), f"row {r}"


def _random_topk_case(i):
    """Case i of a fixed pseudo-random family: log-uniform S in [1, 40000],
    any k in [1, S + 5], a padded row stride, and one of several value
    distributions (continuous, few distinct values, signed zeros, outliers,
    a narrow range)."""
    rng = np.random.default_rng(9000 + i)
    S = int(np.exp(rng.uniform(0.0, np.log(40000.0))))
    k = int(rng.integers(1, S + 6))
    ld = (S + 3) // 4 * 4 + 4 * int(rng.integers(0, 3))
    kind = i % 5
    if kind == 0:
        row = rng.standard_normal(S) * 10.0 ** rng.uniform(-3, 3)
    elif kind == 1:
        row = rng.integers(-3, 4, S).astype(np.float64)
    elif kind == 2:
        row = np.where(rng.random(S) < 0.3, 0.0, rng.standard_normal(S))
        row = np.where(rng.random(S) < 0.5, -row, row)  # -0.0 and +0.0 mixed
    elif kind == 3:
        row = rng.standard_normal(S)
        row[rng.integers(0, S, max(1, S // 1000))] = 1e6
    else:
        row = 1.0 + rng.integers(0, 1000, S) * 2.0 ** -20
    return S, k, ld, row.astype(np.float32)


@pytest.mark.parametrize("i", range(40))
def test_topk_random_family(lib, i):
    import torch
    S, k, ld, row = _random_topk_case(i)
    host = np.full((2, ld), 1e30, np.float32)  # beyond S: must be ignored
    host[0, :S] = row
    host[1, :S] = row[::-1]
    idx = lib.topk(torch.from_numpy(host).cuda(), k, S=S).cpu().numpy()
    for r in range(2):
        want = oracle.select_topk(host[r, :S].astype(np.float64), k)
        assert np.array_equal(idx[r].astype(np.int64), want), f"S={S} k={k} row {r}"


def test_topk_crossing_bin_of_signed_zeros(lib):
    """A crossing bin made of +0.0 and -0.0 only: they rank equal, so the
    lowest indices among them are kept."""
    import torch
    rng = np.random.default_rng(11)
    S, k = 3000, 1000
    host = rng.uniform(-3.0, -1.0, (2, S)).astype(np.float32)
    for r, nz in enumerate((100, 300)):
        pos = rng.permutation(S)
        host[r, pos[:976]] = 5.0
        zeros = pos[976:976 + nz]
        host[r, zeros] = np.where(rng.random(nz) < 0.5, np.float32(-0.0), np.float32(0.0))
    idx = lib.topk(torch.from_numpy(host).cuda(), k).cpu().numpy()
    for r in range(2):
        want = oracle.select_topk(host[r].astype(np.float64), k)
        assert np.array_equal(idx[r].astype(np.int64), want), f"row {r}"


# --------------------------------------------------- attention over given ids --

@pytest.mark.parametrize("name", sorted(SMALL))
def test_attend_given_indices_matches_oracle(lib, name):
    import torch
    c = case(name)
    cache = device_cache(lib, c)
    _, ref_idx, _ = oracle.decode(c.q, c.slab, c.rest, c.v, c.P, c.k, c.w.dtype, S=c.S)
    idx_dev = torch.from_numpy(ref_idx.astype(np.int32)).cuda()
    out = lib.attend_indices(_q(c), cache, _P(c), idx_dev).cpu().numpy()
    ref = oracle.attend_indices(c.q, c.slab, c.rest, c.v, c.P, ref_idx, c.w.dtype)
    for b, h in all_pairs(c.w):
        assert out_error(c.w.dtype, out[b, h], ref[b, h]) <= TOL[c.w.dtype]


# ------------------------------------------------------------- end to end --

@pytest.mark.parametrize("path", [1, 2, 3, 4], ids=["fused", "split", "union", "sliced"])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_decode_matches_oracle(lib, name, path):
    c = case(name)
    kk = min(c.k, c.S)
    if path in (1, 4) and (c.w.D + c.S + kk) * 4 > 56 * 1024:
        pytest.skip("fused path needs q', scores and kept ids within 56 KiB of LDS")
    if path == 3 and not union_applies(c.w):
        pytest.skip("union gather needs 2 or 4 query heads per KV head")
    cache = device_cache(lib, c)
    out, idx = lib.decode(_q(c), cache, _P(c), c.k, path=path)
    out, idx = out.cpu().numpy(), idx.cpu().numpy()
    ref_out, ref_idx, ref_s = oracle.decode(c.q, c.slab, c.rest, c.v, c.P, c.k, c.w.dtype, S=c.S)
    assert idx.dtype == np.int32 and idx.shape == (c.w.B, c.w.Hq, kk)
    check_decode(c.w.dtype, c.k, out, idx, ref_out, ref_idx, ref_s, all_pairs(c.w), src_of(c))


@pytest.mark.parametrize("i", range(24))
def test_decode_random_family(lib, i):
    # every path the library takes for the shape (AUTO included) against the oracle
    w, S, S_max = random_workload(i)
    c = make_case(w, S, S_max)
    k = max(1, min(int(w.k_f * S), S + 3))
    print(f"random decode case {i}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} d={w.d} S={S} "
          f"S_max={S_max} k={k} {w.dtype} sinks={w.sinks}", flush=True)
    cache = device_cache(lib, c)
    ref_out, ref_idx, ref_s = oracle.decode(c.q, c.slab, c.rest, c.v, c.P, k, w.dtype, S=S)
    ran = 0
    for path in (0, 1, 2, 3, 4):
        try:
            lib.decode_path(w.B, w.Hq, w.Hkv, w.D, w.d, S, k, w.dtype, path)
        except lib.LokiError:
            continue
        out, idx = lib.decode(_q(c), cache, _P(c), k, path=path)
        check_decode(w.dtype, k, out.cpu().numpy(), idx.cpu().numpy(), ref_out, ref_idx, ref_s,
                     all_pairs(w), src_of(c))
        ran += 1
    assert ran >= 2  # AUTO and at least the split path


@pytest.mark.parametrize("k", [1, 2, 499, 999, 1000, 5000])
def test_decode_budget_edges(lib, k):
    c = case("ragged_gqa2")
    cache = device_cache(lib, c)
    ref_out, ref_idx, ref_s = oracle.decode(c.q, c.slab, c.rest, c.v, c.P, k, c.w.dtype, S=c.S)
    for path in (1, 2, 3, 4):
        out, idx = lib.decode(_q(c), cache, _P(c), k, path=path)
        check_decode(c.w.dtype, k, out.cpu().numpy(), idx.cpu().numpy(), ref_out, ref_idx, ref_s,
                     all_pairs(c.w), src_of(c))


def test_decode_shorter_S_than_filled(lib):
    # S below the filled length: only the first S tokens may be read
    c = case("sinks")
    cache = device_cache(lib, c)
    S = 1234
    ref_out, ref_idx, ref_s = oracle.decode(c.q, c.slab, c.rest, c.v, c.P, 300, c.w.dtype, S=S)
    for path in (1, 2, 3, 4):
        out, idx = lib.decode(_q(c), cache, _P(c), 300, S=S, path=path)
        check_decode(c.w.dtype, 300, out.cpu().numpy(), idx.cpu().numpy(), ref_out, ref_idx,
                     ref_s, all_pairs(c.w), src_of(c))


def test_decode_deterministic_and_paths_agree(lib):
    c = case("ragged_gqa2")
    cache = device_cache(lib, c)
    o1, i1 = lib.decode(_q(c), cache, _P(c), c.k, path=2)
    o2, i2 = lib.decode(_q(c), cache, _P(c), c.k, path=2)
    o3, i3 = lib.decode(_q(c), cache, _P(c), c.k, path=1)
    o4, i4 = lib.decode(_q(c), cache, _P(c), c.k, path=3)
    o5, _ = lib.decode(_q(c), cache, _P(c), c.k, path=3)
    o6, i6 = lib.decode(_q(c), cache, _P(c), c.k, path=4)
    assert np.array_equal(i1.cpu().numpy(), i6.cpu().numpy())
    assert np.max(np.abs(o1.cpu().numpy() - o6.cpu().numpy())) < 1e-5
    assert np.array_equal(o1.cpu().numpy(), o2.cpu().numpy())
    assert np.array_equal(i1.cpu().numpy(), i2.cpu().numpy())
    assert np.array_equal(o4.cpu().numpy(), o5.cpu().numpy())
    # same float32 scores on every path -> same selection
    assert np.array_equal(i1.cpu().numpy(), i3.cpu().numpy())
    assert np.array_equal(i1.cpu().numpy(), i4.cpu().numpy())
    assert np.max(np.abs(o1.cpu().numpy() - o3.cpu().numpy())) < 1e-5
    assert np.max(np.abs(o1.cpu().numpy() - o4.cpu().numpy())) < 1e-5


# ------------------------------------------------------------------ append --

APPEND_CASES = [
    synth.custom("ap_bf16", 201, B=2, Hq=3, Hkv=3, S=100),
    synth.custom("ap_f32", 202, B=2, Hq=2, Hkv=2, D=64, d=16, S=100, dtype="f32", tau=8.0),
    synth.custom("ap_D64", 203, B=3, Hq=2, Hkv=1, D=64, d=32, S=100),
    synth.custom("ap_full", 204, B=1, Hq=2, Hkv=2, D=128, d=128, S=100),
]


@pytest.mark.parametrize("w", APPEND_CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("pos,T", [(0, 1), (5, 37), (0, 100), (99, 1)])
def test_append_matches_oracle(lib, w, pos, T):
    import torch
    from gpu_cases import basis
    P = basis(w)
    K, V = synth.raw_cache(w, T)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    cache = lib.KVCache(w.B, w.Hkv, w.S, w.D, w.d, tdt)
    lib.append(cache, to_dev(K, w.dtype), to_dev(V, w.dtype), to_dev(P, "f32"), pos=pos)
    torch.cuda.synchronize()
    slab = to_host(cache.k_slab, w.dtype)[:, :, pos:pos + T]
    vv = to_host(cache.v, w.dtype)[:, :, pos:pos + T]
    off = n = 0
    for g in range(w.Hkv):
        kg = oracle.to_f64(K[:, g], w.dtype)
        rs, rr, rv = oracle.append(kg, oracle.to_f64(V[:, g], w.dtype),
                                   P[g].astype(np.float64), w.d, w.dtype)
        x = kg @ P[g].astype(np.float64)
        mag = np.abs(kg) @ np.abs(P[g].astype(np.float64))
        off += check_rounded_rotation(slab[:, g], rs, x[..., :w.d], mag[..., :w.d], w.dtype)
        n += rs.size
        if w.d < w.D:
            off += check_rounded_rotation(to_host(cache.k_rest, w.dtype)[:, g, pos:pos + T], rr,
                                          x[..., w.d:], mag[..., w.d:], w.dtype)
            n += rr.size
        assert np.array_equal(vv[:, g], rv)
    assert off <= max(1, n // 1000)  # neighbours at rounding boundaries are rare
    # untouched slots stay zero
    full = to_host(cache.v, w.dtype)
    assert not np.any(full[:, :, :pos]) and not np.any(full[:, :, pos + T:])


# ------------------------------------------------------------------- dense --

@pytest.mark.parametrize("name", ["tiny", "ragged_gqa2", "gqa8", "gqa5", "full_rank_f32", "long_5000",
                                  "sinks", "long_20000", "d64_D64_bf16", "gqa4_d16", "gqa4_f32"])
def test_dense_matches_oracle(lib, name):
    c = case(name)
    cache = device_cache(lib, c)
    out = lib.dense_decode(_q(c), cache, _P(c)).cpu().numpy()
    ref = oracle.dense_decode(c.q, c.slab, c.rest, c.v, c.P, c.w.dtype, S=c.S)
    for b, h in all_pairs(c.w):
        assert out_error(c.w.dtype, out[b, h], ref[b, h]) <= TOL[c.w.dtype]


# ------------------------------------------------------------ size limits --

LIMITS = {
    # the longest context the union gather takes (its bitmap row in LDS), and
    # rows far beyond the top-k's LDS staging (selected from global memory)
    "union_max_S": (synth.custom("union_max_S", 701, B=1, Hq=4, Hkv=1, S=1 << 17, k_f=0.125),
                    [2, 3]),
    # q' + scores + kept ids just under the fused kernel's 56 KiB of LDS
    "fused_lds_max": (synth.custom("fused_lds_max", 702, B=1, Hq=2, Hkv=2, S=11000,
                                   k_f=2999.5 / 11000), [1, 2, 4]),
}


@pytest.mark.parametrize("name", sorted(LIMITS))
def test_decode_at_size_limits(lib, name):
    """Decode at the largest sizes each path accepts, every (sequence, head)
    pair against the oracle; one past the limit is refused."""
    w, paths = LIMITS[name]
    c = make_case(w)
    cache = device_cache(lib, c)
    ref_out, ref_idx, ref_s = oracle.decode(c.q, c.slab, c.rest, c.v, c.P, c.k, w.dtype)
    for path in paths:
        out, idx = lib.decode(_q(c), cache, _P(c), c.k, path=path)
        check_decode(w.dtype, c.k, out.cpu().numpy(), idx.cpu().numpy(), ref_out, ref_idx, ref_s,
                     all_pairs(w), src_of(c))
    if name == "union_max_S":
        assert lib.decode_path(1, 4, 1, 128, 32, (1 << 17) + 1, c.k, "bf16", 0) == 2
    else:
        # (128 + 11000 + 3209) floats is one past 56 KiB
        assert lib.decode_path(1, 2, 2, 128, 32, 11000, 3208, "bf16", 1) == 1
        with pytest.raises(lib.LokiError):
            lib.decode_path(1, 2, 2, 128, 32, 11000, 3209, "bf16", 1)


# ------------------------------------------------------- full bench shapes --

FULL = ["l2_7b", "l2_13b_run", "l3_8b_gqa", "mistral_32k"]


@pytest.mark.parametrize("name,path", [(n, 0) for n in FULL] +
                         [("l2_7b", 2), ("l3_8b_gqa", 2), ("l3_8b_gqa", 3), ("mistral_32k", 3)])
def test_full_size_decode_sampled(lib, name, path):
    """Full benchmark shapes, launched exactly as the benchmark launches them
    (AUTO path: sliced, fused, fused and split), and on the split and union
    paths where AUTO takes another; every (sequence, head) pair checked
    against the oracle, with at most 1 in 100 near-tie swaps (at least one
    allowed)."""
    w = synth.WORKLOADS[name]
    c = make_case(w)
    cache = device_cache(lib, c)
    out, idx = lib.decode(_q(c), cache, _P(c), w.k, path=path)
    out, idx = out.cpu().numpy(), idx.cpu().numpy()
    pairs = all_pairs(w)
    ref_out, ref_idx, ref_s = oracle.decode(c.q, c.slab, c.rest, c.v, c.P, w.k, w.dtype, heads=pairs)
    check_decode(w.dtype, w.k, out, idx, ref_out, ref_idx, ref_s, pairs, src_of(c))
    # every row: k distinct ascending ids in range, finite outputs
    assert np.all(np.diff(idx.astype(np.int64), axis=-1) > 0)
    assert idx.min() >= 0 and idx.max() < w.S
    assert np.all(np.isfinite(out))


# ------------------------------------------------------- decode step (fused append) --

STEP_CASES = {
    "step_mha": synth.custom("step_mha", 301, B=2, Hq=4, Hkv=4, S=700),
    "step_gqa": synth.custom("step_gqa", 302, B=2, Hq=8, Hkv=2, S=1000),
    "step_f32": synth.custom("step_f32", 303, B=1, Hq=2, Hkv=2, D=64, d=16, S=300, dtype="f32",
                             tau=8.0),
    "step_first": synth.custom("step_first", 304, B=2, Hq=2, Hkv=2, S=1),
    # 288 rows: the sliced path's whole rows and sliced remainder in one step
    "step_tail": synth.custom("step_tail", 306, B=2, Hq=144, Hkv=144, S=700),
    # the benchmark's step at full size (B=16, 40 heads, S=3584, k=896): every
    # (sequence, head) pair and every written slot against the oracle
    "step_l2_13b_full": synth.WORKLOADS["l2_13b_run"],
}


def _oracle_token(w, P, kn, vn):
    """The oracle's cache rows for the step's token: [B, Hkv, 1, ...]."""
    st = np.uint16 if w.dtype == "bf16" else np.float32
    slab = np.empty((w.B, w.Hkv, 1, w.d), st)
    rest = np.empty((w.B, w.Hkv, 1, w.D - w.d), st)
    vv = np.empty((w.B, w.Hkv, 1, w.D), st)
    for g in range(w.Hkv):
        slab[:, g], rest[:, g], vv[:, g] = oracle.append(
            oracle.to_f64(kn[:, g], w.dtype), oracle.to_f64(vn[:, g], w.dtype),
            P[g].astype(np.float64), w.d, w.dtype)
    return slab, rest, vv


@pytest.mark.parametrize("path", [1, 2, 3, 4], ids=["fused", "split", "union", "sliced"])
@pytest.mark.parametrize("name", sorted(STEP_CASES))
def test_decode_step_matches_oracle(lib, name, path):
    """Append at pos = S-1 and decode over S tokens in one call; the written
    slot equals the oracle's append and the decode equals the oracle's decode
    over the oracle's full cache."""
    w = STEP_CASES[name]
    if path == 3 and not union_applies(w):
        pytest.skip("union gather needs 2 or 4 query heads per KV head")
    _check_step(lib, w, path)


@pytest.mark.parametrize("i", range(12))
def test_decode_step_random_family(lib, i):
    # the random decode shapes as one generation step, on every applicable path
    w, _, _ = random_workload(100 + i)
    print(f"random step case {i}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} d={w.d} S={w.S} "
          f"k={w.k_at(w.S)} {w.dtype} sinks={w.sinks}", flush=True)
    ran = 0
    for path in (0, 1, 2, 3, 4):
        try:
            lib.decode_path(w.B, w.Hq, w.Hkv, w.D, w.d, w.S, w.k_at(w.S), w.dtype, path)
        except lib.LokiError:
            continue
        _check_step(lib, w, path)
        ran += 1
    assert ran >= 2


def _check_step(lib, w, path):
    S = w.S
    c = make_case(w, S - 1, S + 3) if S > 1 else None
    from gpu_cases import basis
    P = basis(w) if c is None else c.P
    kn, vn = synth.new_tokens(w, 7)            # [B, Hkv, 1, D]
    o_slab, o_rest, o_v = _oracle_token(w, P, kn, vn)
    st = np.uint16 if w.dtype == "bf16" else np.float32
    full = {}
    for nm, tok, width in (("slab", o_slab, w.d), ("rest", o_rest, w.D - w.d), ("v", o_v, w.D)):
        arr = np.zeros((w.B, w.Hkv, S + 3, width), st)
        if c is not None:
            arr[:, :, :S - 1] = getattr(c, nm)[:, :, :S - 1]
        arr[:, :, S - 1] = tok[:, :, 0]
        full[nm] = arr
    import torch
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    cache = lib.KVCache(w.B, w.Hkv, S + 3, w.D, w.d, tdt)
    if c is not None:
        cache.k_slab[:, :, :S - 1].copy_(to_dev(c.slab[:, :, :S - 1], w.dtype))
        if w.d < w.D:
            cache.k_rest[:, :, :S - 1].copy_(to_dev(c.rest[:, :, :S - 1], w.dtype))
        cache.v[:, :, :S - 1].copy_(to_dev(c.v[:, :, :S - 1], w.dtype))
    cache.length = S - 1
    q = synth.queries(w, step=7)
    k = w.k_at(S)
    out, idx = lib.decode_step(to_dev(q, w.dtype), to_dev(kn[:, :, 0], w.dtype),
                               to_dev(vn[:, :, 0], w.dtype), cache, to_dev(P, "f32"), k,
                               pos=S - 1, path=path)
    torch.cuda.synchronize()
    # the written slot: the value row stored as given, the key row the rounding
    # of its float64 rotation (neighbouring values only at a rounding boundary)
    kx = np.stack([oracle.to_f64(kn[:, g, 0], w.dtype) @ P[g].astype(np.float64)
                   for g in range(w.Hkv)], axis=1)
    kmag = np.stack([np.abs(oracle.to_f64(kn[:, g, 0], w.dtype)) @ np.abs(P[g].astype(np.float64))
                     for g in range(w.Hkv)], axis=1)
    for nm, t, cols in (("slab", cache.k_slab, slice(0, w.d)), ("rest", cache.k_rest, slice(w.d, w.D)),
                        ("v", cache.v, None)):
        if t is None:
            continue
        got = to_host(t, w.dtype)[:, :, S - 1]
        want = full[nm][:, :, S - 1]
        if cols is None:
            assert np.array_equal(got, want), nm
        else:
            check_rounded_rotation(got, want, kx[..., cols], kmag[..., cols], w.dtype)
    ref_out, ref_idx, ref_s = oracle.decode(q, full["slab"], full["rest"], full["v"], P, k,
                                            w.dtype, S=S)
    check_decode(w.dtype, k, out.cpu().numpy(), idx.cpu().numpy(), ref_out, ref_idx, ref_s,
                 all_pairs(w), OracleSrc(q, full["slab"], full["rest"], full["v"], P))


def test_decode_steps_in_sequence_paths_agree(lib):
    """Eight consecutive steps on the fused and on the split path from the same
    starting cache: identical selections, outputs within float32 rounding, and
    identical cache contents afterwards."""
    import torch
    w = synth.custom("step_seq", 305, B=2, Hq=4, Hkv=4, S=500)
    c = make_case(w, 500, 520)
    caches = [device_cache(lib, c), device_cache(lib, c)]
    P = to_dev(c.P, "f32")
    for step in range(8):
        kn, vn = synth.new_tokens(w, 100 + step)
        q = to_dev(synth.queries(w, step=100 + step), w.dtype)
        res = [lib.decode_step(q, to_dev(kn[:, :, 0], w.dtype), to_dev(vn[:, :, 0], w.dtype),
                               caches[i], P, w.k_at(501 + step), path=p)
               for i, p in ((0, 1), (1, 2))]
        assert np.array_equal(res[0][1].cpu().numpy(), res[1][1].cpu().numpy())
        assert np.max(np.abs(res[0][0].cpu().numpy() - res[1][0].cpu().numpy())) < 1e-5
    torch.cuda.synchronize()
    for a, b in ((caches[0].k_slab, caches[1].k_slab), (caches[0].k_rest, caches[1].k_rest),
                 (caches[0].v, caches[1].v)):
        ud = ulp_diff_bf16(to_host(a, "bf16"), to_host(b, "bf16"))
        assert ud.max() <= 1 and (ud == 0).mean() >= 0.9999
    assert caches[0].length == caches[1].length == 508


@pytest.mark.parametrize("S,k,nrows", [(3000, 750, 7), (4096, 1000, 3), (2048, 17, 2), (1500, 1499, 5)])
def test_decode_exact_ties_from_repeated_rows(lib, S, k, nrows):
    """Slab rows drawn from a handful of distinct rows: scores tie exactly
    (bit-identical on every side), so thousands of tokens share the crossing
    bin; equal scores must go to the lower index on both paths."""
    import torch
    w = synth.custom("ties", 400 + nrows, B=2, Hq=3, Hkv=3, S=S)
    c = make_case(w, S, S)
    rng = np.random.default_rng(S + nrows)
    pick = rng.integers(0, nrows, size=(w.B, w.Hkv, S))
    for b in range(w.B):
        for g in range(w.Hkv):
            c.slab[b, g] = c.slab[b, g, pick[b, g]]
    cache = device_cache(lib, c)
    ref_out, ref_idx, ref_s = oracle.decode(c.q, c.slab, c.rest, c.v, c.P, k, w.dtype, S=S)
    for path in (1, 2):
        out, idx = lib.decode(to_dev(c.q, w.dtype), cache, to_dev(c.P, "f32"), k, path=path)
        idx = idx.cpu().numpy()
        assert np.array_equal(idx.astype(np.int64), ref_idx), f"path {path}"
        out = out.cpu().numpy()
        for b, h in all_pairs(w):
            assert out_error(w.dtype, out[b, h], ref_out[b, h]) <= TOL[w.dtype]


# ------------------------------------------------------- measurement helper --

def test_stream_read_probe_reads_every_element(lib):
    """The streaming-read probe's per-thread sums add up to the sum of the
    buffer, so every 16-byte chunk was read exactly once."""
    import torch
    n = (1 << 20) + 12  # float32 elements: a ragged tail for the grid-stride loop
    buf = torch.arange(n, dtype=torch.float32, device="cuda") % 7
    for wg in (1, 3, 64):
        sink = torch.full((wg * 256,), float("nan"), dtype=torch.float32, device="cuda")
        lib.stream_read(buf, sink, wg)
        got = sink.double().sum().item()
        assert got == float((torch.arange(n, dtype=torch.float64) % 7).sum())


@pytest.mark.parametrize("threads,loads", [(256, 1), (512, 4), (1024, 16), (256, 8)])
def test_share_read_probe_reads_every_element(lib, threads, loads):
    """Each workgroup of the per-share probe reads exactly its share: the
    per-thread sums add up to the sum of the buffer, also when a share is not
    a multiple of the workgroup's loads."""
    import torch
    for wg in (1, 5, 256):
        n = wg * 4 * (3 * threads * loads + 7)  # float32 elements: ragged shares
        buf = (torch.arange(n, dtype=torch.int64, device="cuda") % 7).to(torch.float32)
        sink = torch.full((wg * threads,), float("nan"), dtype=torch.float32, device="cuda")
        lib.stream_read_shares(buf, sink, wg, threads, loads)
        got = sink.double().sum().item()
        assert got == float((n // 7) * 21 + sum(range(n % 7))), (wg, threads, loads)


@pytest.mark.parametrize("path", [1, 2, 3, 4], ids=["fused", "split", "union", "sliced"])
def test_split_paths_ignore_stale_workspace(lib, path):
    """The split and union paths read nothing from the workspace that the same
    call did not write: a workspace full of NaN bit patterns and a zeroed one
    give bit-identical selections and outputs."""
    import torch
    c = case("sinks")
    cache = device_cache(lib, c)
    ws = lib.alloc_workspace(c.w.B, c.w.Hq, c.S_max, c.w.D, c.k, torch.device("cuda"))
    res = []
    for fill in (0xFF, 0x00):
        ws.fill_(fill)
        out, idx = lib.decode(_q(c), cache, _P(c), c.k, workspace=ws, path=path)
        res.append((out.cpu().numpy(), idx.cpu().numpy()))
    assert np.array_equal(res[0][1], res[1][1])
    assert np.array_equal(res[0][0].view(np.uint32), res[1][0].view(np.uint32))


GROUPED = {
    # four query heads per KV head, bf16, D = 128, S a multiple of 16: given a
    # workspace, the single-kernel decode shares each KV head's ranking among
    # its four query heads' workgroups
    "grp_d32": (synth.custom("grp_d32", 120, B=2, Hq=8, Hkv=2, S=1024), [1, 16, 256, 1024]),
    "grp_d64": (synth.custom("grp_d64", 121, B=1, Hq=16, Hkv=4, d=64, S=4096, k_f=0.125), [512]),
    "grp_d16": (synth.custom("grp_d16", 122, B=3, Hq=4, Hkv=1, d=16, S=512, sinks=4), [128]),
    "grp_d8": (synth.custom("grp_d8", 123, B=2, Hq=8, Hkv=2, d=8, S=4992), [1248]),
}


@pytest.mark.parametrize("name", sorted(GROUPED))
def test_grouped_ranking_matches_oracle_and_the_single_head_pass(lib, name):
    """The fused decode with a workspace (grouped ranking) against the oracle,
    and bit-identical to the fused decode without one (each workgroup ranks
    its own row), at several budgets."""
    import torch
    w, ks = GROUPED[name]
    c = make_case(w)
    cache = device_cache(lib, c)
    ws = lib.alloc_workspace(w.B, w.Hq, c.S_max, w.D, max(ks), torch.device("cuda"))
    for k in ks:
        print(f"grouped: {name} k={k}", flush=True)
        out, idx = lib.decode(_q(c), cache, _P(c), k, workspace=ws, path=1)
        one_out, one_idx = lib.decode(_q(c), cache, _P(c), k, path=1)
        out, idx = out.cpu().numpy(), idx.cpu().numpy()
        assert np.array_equal(idx, one_idx.cpu().numpy())
        assert np.array_equal(out.view(np.uint32), one_out.cpu().numpy().view(np.uint32))
        ref_out, ref_idx, ref_s = oracle.decode(c.q, c.slab, c.rest, c.v, c.P, k, w.dtype, S=c.S)
        check_decode(w.dtype, k, out, idx, ref_out, ref_idx, ref_s, all_pairs(w), src_of(c))


def test_grouped_ranking_steps_match_the_single_head_step(lib):
    """Decode steps (append + decode in one launch) with a workspace, so the
    four query heads of a KV head share the ranking, from the same starting
    cache as steps without one: identical selections, bit-identical outputs
    and cache contents after each step, at lengths that take the grouped
    ranking (a multiple of 16) and one that does not, and the first step's
    decode against the oracle."""
    import torch
    w = synth.custom("grp_step", 124, B=2, Hq=8, Hkv=2, S=1023)
    c = make_case(w, 1023, 1040)
    caches = [device_cache(lib, c), device_cache(lib, c)]
    P = to_dev(c.P, "f32")
    ws = lib.alloc_workspace(w.B, w.Hq, c.S_max, w.D, 300, torch.device("cuda"))
    for step in range(3):  # S = 1024, 1025, 1026
        kn, vn = synth.new_tokens(w, 200 + step)
        q = synth.queries(w, step=200 + step)
        S = 1024 + step
        k = w.k_at(S)
        print(f"grouped step: S={S} k={k}", flush=True)
        res = [lib.decode_step(to_dev(q, w.dtype), to_dev(kn[:, :, 0], w.dtype),
                               to_dev(vn[:, :, 0], w.dtype), caches[i], P, k, path=1,
                               workspace=wsi)
               for i, wsi in ((0, ws), (1, None))]
        torch.cuda.synchronize()
        assert np.array_equal(res[0][1].cpu().numpy(), res[1][1].cpu().numpy()), S
        assert np.array_equal(res[0][0].cpu().numpy().view(np.uint32),
                              res[1][0].cpu().numpy().view(np.uint32)), S
        for a, b in ((caches[0].k_slab, caches[1].k_slab), (caches[0].k_rest, caches[1].k_rest),
                     (caches[0].v, caches[1].v)):
            assert torch.equal(a, b), S
        if step == 0:
            full = {nm: to_host(t, w.dtype)[:, :, :S] for nm, t in
                    (("slab", caches[0].k_slab), ("rest", caches[0].k_rest), ("v", caches[0].v))}
            ref_out, ref_idx, ref_s = oracle.decode(q, full["slab"], full["rest"], full["v"], c.P,
                                                    k, w.dtype, S=S)
            check_decode(w.dtype, k, res[0][0].cpu().numpy(), res[0][1].cpu().numpy(), ref_out,
                         ref_idx, ref_s, all_pairs(w),
                         OracleSrc(q, full["slab"], full["rest"], full["v"], c.P))


def test_per_layer_slab_width(lib):
    """Per-layer d (the pages' ablation over d): one cache per layer, each
    with its own slab width, decoded one after another with the same query
    heads and each checked against the oracle at its own d."""
    import torch
    for layer, d in enumerate((8, 16, 40, 64, 128)):
        w = synth.custom(f"layer{layer}", 500 + layer, B=2, Hq=8, Hkv=2, d=d, S=900)
        c = make_case(w)
        cache = device_cache(lib, c)
        out, idx = lib.decode(_q(c), cache, _P(c), c.k)
        ref_out, ref_idx, ref_s = oracle.decode(c.q, c.slab, c.rest, c.v, c.P, c.k, w.dtype, S=c.S)
        check_decode(w.dtype, c.k, out.cpu().numpy(), idx.cpu().numpy(), ref_out, ref_idx, ref_s,
                     all_pairs(w), src_of(c))


# ------------------------------------------------------------ graph capture --

@pytest.mark.parametrize("path", [1, 2, 3, 4], ids=["fused", "split", "union", "sliced"])
def test_decode_replays_from_a_captured_graph(lib, path):
    """Each path launches only kernels (no allocation, no memset), so a decode
    captured into a HIP graph replays correctly: three replays, with eager
    work and synchronisation between them, each equal to the eager call."""
    import torch
    c = case("sinks")  # G = 4: every path applies
    cache = device_cache(lib, c)
    q = _q(c)
    P = _P(c)
    ws = lib.alloc_workspace(c.w.B, c.w.Hq, c.S_max, c.w.D, c.k, torch.device("cuda"))
    out = torch.empty((c.w.B, c.w.Hq, c.w.D), dtype=torch.float32, device="cuda")
    idx = torch.empty((c.w.B, c.w.Hq, c.k), dtype=torch.int32, device="cuda")
    ref_out, ref_idx = lib.decode(q, cache, P, c.k, workspace=ws, path=path)
    ref_out, ref_idx = ref_out.cpu().numpy(), ref_idx.cpu().numpy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up on the capture stream
        lib.decode(q, cache, P, c.k, out=out, idx=idx, workspace=ws, path=path)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.decode(q, cache, P, c.k, out=out, idx=idx, workspace=ws, path=path)
    for rep in range(3):
        out.fill_(float("nan"))
        idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ref_idx), f"replay {rep}"
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref_out.view(np.uint32)), rep
        # eager work between replays
        lib.decode(q, cache, P, 7, workspace=ws, path=path)
        torch.cuda.synchronize()
