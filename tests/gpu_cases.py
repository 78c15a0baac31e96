"""Builders shared by the GPU parity tests.

Every input comes from the seeded generators (synth) and the oracle: the
PCA basis is the oracle's calibration of the generator's calibration keys,
and the rotated cache is the oracle's float64 append of the generator's raw
keys, rounded to the cache dtype.  The GPU library only ever receives these
bytes; nothing produced by the GPU feeds the oracle.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

import oracle
import synth

# a finite value far outside the data: any read past the S valid tokens
# would dominate a score or a softmax and fail the comparison
_POISON = 3.0e4


@dataclass
class Case:
    w: synth.Workload
    S: int
    S_max: int
    P: np.ndarray          # [Hkv, D, D] float32
    q: np.ndarray          # [B, Hq, D] storage
    K: np.ndarray          # raw keys [B, Hkv, S, D] storage
    V: np.ndarray          # raw values [B, Hkv, S, D] storage
    slab: np.ndarray       # [B, Hkv, S_max, d] storage
    rest: np.ndarray       # [B, Hkv, S_max, D-d] storage (width 0 when d == D)
    v: np.ndarray          # [B, Hkv, S_max, D] storage

    @property
    def k(self):
        return self.w.k_at(self.S)


def storage_dtype(dtype: str):
    return np.uint16 if dtype == "bf16" else np.float32


def basis(w: synth.Workload) -> np.ndarray:
    P = np.empty((w.Hkv, w.D, w.D), np.float32)
    for g in range(w.Hkv):
        Pg, _ = oracle.calibrate(synth.calib_keys(w, g))
        P[g] = Pg.astype(np.float32)
    return P


def make_case(w: synth.Workload, S: int | None = None, S_max: int | None = None,
              rope_base: float | None = None) -> Case:
    """The oracle's cache of the generator's keys and values; with rope_base
    each key is embedded at its position before the rotation."""
    S = w.S if S is None else S
    S_max = S if S_max is None else S_max
    P = basis(w)
    K, V = synth.raw_cache(w, S)
    st = storage_dtype(w.dtype)
    poison = oracle.from_f64(np.array(_POISON), w.dtype)
    slab = np.full((w.B, w.Hkv, S_max, w.d), poison, st)
    rest = np.full((w.B, w.Hkv, S_max, w.D - w.d), poison, st)
    vv = np.full((w.B, w.Hkv, S_max, w.D), poison, st)
    for g in range(w.Hkv):
        s_, r_, v_ = oracle.append(oracle.to_f64(K[:, g], w.dtype), oracle.to_f64(V[:, g], w.dtype),
                                   P[g].astype(np.float64), w.d, w.dtype, rope_base=rope_base)
        slab[:, g, :S], rest[:, g, :S], vv[:, g, :S] = s_, r_, v_
    return Case(w, S, S_max, P, synth.queries(w), K, V, slab, rest, vv)


# ------------------------------------------------------------- torch glue --

def to_dev(a: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t, dtype: str) -> np.ndarray:
    import torch
    if dtype == "bf16":
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def device_cache(loki, c: Case):
    import torch
    w = c.w
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    cache = loki.KVCache(w.B, w.Hkv, c.S_max, w.D, w.d, tdt)
    cache.k_slab.copy_(to_dev(c.slab, w.dtype))
    if w.d < w.D:
        cache.k_rest.copy_(to_dev(c.rest, w.dtype))
    cache.v.copy_(to_dev(c.v, w.dtype))
    cache.length = c.S
    return cache


# ------------------------------------------------------------- comparison --

def out_error(dtype: str, got: np.ndarray, ref: np.ndarray) -> float:
    """fp32 caches: max-abs error; bf16 caches: relative L2 error."""
    got = np.asarray(got, np.float64)
    if dtype == "f32":
        return float(np.max(np.abs(got - ref)))
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))


TOL = {"f32": 1e-5, "bf16": 2e-3}


@dataclass
class OracleSrc:
    """The oracle-side inputs of a decode (storage form), from which the
    oracle's attention over any index set is formed."""
    q: np.ndarray
    slab: np.ndarray
    rest: np.ndarray
    v: np.ndarray
    P: np.ndarray
    rope: tuple | None = None   # (base, q_pos) for the RoPE variant


def src_of(c: Case, rope=None) -> OracleSrc:
    return OracleSrc(c.q, c.slab, c.rest, c.v, c.P, rope)


def check_decode(dtype, k, out, idx, ref_out, ref_idx, ref_s, pairs, src: OracleSrc,
                 max_swaps=None):
    """Index sets: equal to the oracle's whenever the relative gap at the k-th
    place exceeds 1e-4; otherwise a valid choice inside the tie band, and at
    most 1 in 100 pairs (at least one) may differ from the oracle's set.
    Outputs: every pair is compared with the oracle's exact attention over the
    GPU's own index set (the oracle's decode output where the sets agree,
    oracle.attend_indices over the GPU's set where they do not).
    Returns (n_band, n_swapped, worst_output_error)."""
    n_band = n_swap = 0
    worst = 0.0
    for b, h in pairs:
        s = ref_s[b, h]
        kk = min(k, s.shape[0])
        gi = idx[b, h].astype(np.int64)
        assert gi.shape == (kk,)
        gap = oracle.topk_gap(s, kk)
        if gap > 1e-4:
            assert np.array_equal(gi, ref_idx[b, h]), f"idx mismatch at (b={b}, h={h}), gap {gap:.3g}"
        else:
            n_band += 1
            assert oracle.valid_in_band(s, kk, gi), f"invalid near-tie set at (b={b}, h={h})"
        if np.array_equal(gi, ref_idx[b, h]):
            ref = ref_out[b, h]
        else:
            n_swap += 1
            ref = oracle.attend_indices(src.q, src.slab, src.rest, src.v, src.P, idx, dtype,
                                        heads=[(b, h)], rope=src.rope)[b, h]
        e = out_error(dtype, out[b, h], ref)
        worst = max(worst, e)
        assert e <= TOL[dtype], f"output error {e:.3g} at (b={b}, h={h})"
    limit = max(1, len(pairs) // 100) if max_swaps is None else max_swaps
    assert n_swap <= limit, f"{n_swap} near-tie swaps in {len(pairs)} head-queries"
    return n_band, n_swap, worst


def all_pairs(w):
    return [(b, h) for b in range(w.B) for h in range(w.Hq)]


def ulp_diff_bf16(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|a - b| in units of bf16 steps for same-sign finite bf16 patterns
    (ordered integer distance of the bit patterns)."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + x)
    return np.abs(ordered(a) - ordered(b))


def ulp_diff_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    def ordered(x):
        x = x.view(np.int32).astype(np.int64)
        return np.where(x < 0, -(x & 0x7FFFFFFF), x)
    return np.abs(ordered(np.ascontiguousarray(a)) - ordered(np.ascontiguousarray(b)))


def random_workload(i):
    """A seeded random shape: dtype, head dim, slab width, query heads per KV
    head (1, 2, 4 or 8), batch, length (log-uniform up to 20000, ragged
    capacity), budget (sometimes past S) and key spectrum, with or without
    sink tokens."""
    r = np.random.default_rng(91000 + i)
    dtype = "bf16" if r.random() < 0.7 else "f32"
    D = 128 if r.random() < 0.7 else 64
    unit = 8 if dtype == "bf16" else 4
    d = int(r.choice([x for x in (4, 8, 16, 24, 32, 48, 64, 128) if x % unit == 0 and x <= D]))
    G = int(r.choice([1, 2, 4, 8]))
    Hkv = int(r.integers(1, 4))
    B = int(r.integers(1, 4))
    S = max(1, int(np.exp(r.uniform(0.0, np.log(20000.0)))))
    k_f = float(r.choice([0.01, 0.1, 0.25, 0.5, 0.9, 1.5]))
    w = synth.custom(f"random_{i}", 950 + i, B=B, Hq=G * Hkv, Hkv=Hkv, D=D, d=d, S=S, k_f=k_f,
                     dtype=dtype, tau=float(r.choice([8.0, 24.0, 48.0])),
                     sinks=min(S, 4) if r.random() < 0.3 else 0)
    return w, S, S + int(r.integers(0, 40))


def check_rounded_rotation(got, want, x, mag, dtype):
    """got (the library's) and want (the oracle's) are storage-dtype roundings
    of the same rotated values, whose exact float64 sums are x, each a sum of
    terms whose magnitudes add up to mag.  Both sides sum in float64 in
    different orders, so they may round to neighbouring values where x lies
    within float64 summation error (here 64 units of 2^-53 times mag) of the
    boundary between them; everywhere else they must be equal."""
    ud = ulp_diff_bf16(got, want) if dtype == "bf16" else ulp_diff_f32(got, want)
    assert ud.max() <= 1, f"{int(ud.max())} units apart"
    off = ud == 1
    if off.any():
        mid = (oracle.to_f64(got[off], dtype) + oracle.to_f64(want[off], dtype)) / 2.0
        slack = np.abs(x[off] - mid) / mag[off]
        assert np.all(slack <= 64 * 2.0 ** -53), f"a neighbour {slack.max():.3g} (of the terms) away"
    return int(off.sum())


def scale(D):
    return 1.0 / math.sqrt(D)
