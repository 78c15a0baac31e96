"""Seeded synthetic inputs for decode-step sparse attention.

This module only draws numbers.  It holds no step of the attention method
itself (no PCA, no rotation into a calibrated basis, no scoring, selection or
softmax), so the CPU oracle and the GPU library can both be fed from it
without sharing any of the method's arithmetic.

Recipe (the same for every workload):

* a per-KV-head orthogonal matrix Q, drawn as the QR factor of a D x D
  standard Gaussian with each column's sign fixed by the sign of diag(R)
  (this makes Q Haar-distributed);
* key spectrum sigma_i = exp(-i / tau), i = 0..D-1;
* keys  = z . diag(sigma) . Q^T with z ~ N(0, 1) per element, so the keys'
  covariance has eigenvectors Q and eigenvalues sigma_i^2 (keys lying in a
  low-dimensional subspace, as the Loki pages report for real models);
* optional "sink" tokens at positions 0..n_sinks-1 whose keys are scaled by
  SINK_SCALE (high-norm tokens, as in the GQA workload);
* values and queries ~ N(0, 1);
* calibration keys: a separate draw of keys from the same distribution,
  never containing sinks.

All draws are float64 from numpy's PCG64 seeded with
SeedSequence([workload_id, role, b, h, step]).  Storage rounding: float32
storage rounds float64 -> float32 to nearest even; bf16 storage rounds
float64 -> float32 -> bf16, each step to nearest even, and is returned as raw
uint16 bit patterns.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

ROLE_BASIS = 0
ROLE_CALIB = 1
ROLE_KEYS = 2
ROLE_VALUES = 3
ROLE_QUERIES = 4
ROLE_NEW_KEYS = 5
ROLE_NEW_VALUES = 6
ROLE_SCORES = 7  # free-standing score vectors for selection tests

SINK_SCALE = 8.0


@dataclass(frozen=True)
class Workload:
    """One synthetic decode workload (shapes, Loki budget and key spectrum)."""

    name: str
    wid: int          # seed namespace
    B: int            # batch
    Hq: int           # query heads
    Hkv: int          # key/value heads
    D: int            # head dimension
    S: int            # cached tokens at the measured decode step
    d: int            # leading principal dimensions used for ranking
    k_f: float        # fraction of tokens kept
    tau: float        # spectrum decay constant
    dtype: str        # "f32" or "bf16"
    calib_n: int      # calibration keys per KV head
    sinks: int = 0    # high-norm tokens at positions 0..sinks-1
    prefill: int = 0  # prompt length of the generation run (0: no run)
    steps: int = 0    # decode steps of the generation run

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def k_at(self, S: int) -> int:
        """Tokens kept at cache length S: floor(k_f * S) clamped to [1, S]."""
        return int(min(max(int(np.floor(self.k_f * S)), 1), S))

    @property
    def k(self) -> int:
        return self.k_at(self.S)

    @property
    def esize(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS = {
    "tiny": Workload("tiny", 0, B=1, Hq=1, Hkv=1, D=64, S=256, d=16, k_f=0.25,
                     tau=8.0, dtype="f32", calib_n=1024),
    "l2_7b": Workload("l2_7b", 1, B=1, Hq=32, Hkv=32, D=128, S=4096, d=32,
                      k_f=0.25, tau=24.0, dtype="bf16", calib_n=4096),
    "l2_13b_run": Workload("l2_13b_run", 2, B=16, Hq=40, Hkv=40, D=128, S=3584,
                           d=32, k_f=0.25, tau=24.0, dtype="bf16",
                           calib_n=4096, prefill=3072, steps=512),
    "l3_8b_gqa": Workload("l3_8b_gqa", 3, B=8, Hq=32, Hkv=8, D=128, S=8192,
                          d=32, k_f=0.25, tau=24.0, dtype="bf16",
                          calib_n=4096, sinks=4),
    "mistral_32k": Workload("mistral_32k", 4, B=4, Hq=32, Hkv=8, D=128,
                            S=32768, d=64, k_f=0.125, tau=48.0, dtype="bf16",
                            calib_n=4096),
}


def custom(name: str, wid: int, **kw) -> Workload:
    """A workload of arbitrary shape (used for edge-case and tile-span tests)."""
    base = dict(B=1, Hq=1, Hkv=1, D=128, S=256, d=32, k_f=0.25, tau=24.0,
                dtype="bf16", calib_n=1024)
    base.update(kw)
    return Workload(name, wid, **base)


def rng(wid: int, role: int, b: int = 0, h: int = 0, step: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([wid, role, b, h, step])))


def head_basis(w: Workload, g: int) -> np.ndarray:
    """Haar-random orthogonal D x D matrix Q for KV head g (float64)."""
    a = rng(w.wid, ROLE_BASIS, 0, g).standard_normal((w.D, w.D))
    q, r = np.linalg.qr(a)
    return q * np.where(np.diag(r) < 0, -1.0, 1.0)[None, :]


def spectrum(w: Workload) -> np.ndarray:
    return np.exp(-np.arange(w.D, dtype=np.float64) / w.tau)


def _keys_from(z: np.ndarray, w: Workload, Q: np.ndarray) -> np.ndarray:
    return (z * spectrum(w)[None, :]) @ Q.T


def calib_keys(w: Workload, g: int, Q: np.ndarray | None = None) -> np.ndarray:
    """calib_n float64 calibration keys for KV head g (no sinks)."""
    Q = head_basis(w, g) if Q is None else Q
    z = rng(w.wid, ROLE_CALIB, 0, g).standard_normal((w.calib_n, w.D))
    return _keys_from(z, w, Q)


def cache_keys(w: Workload, b: int, g: int, n: int, Q: np.ndarray | None = None) -> np.ndarray:
    """Keys of token positions 0..n-1 of sequence b, KV head g (float64)."""
    Q = head_basis(w, g) if Q is None else Q
    z = rng(w.wid, ROLE_KEYS, b, g).standard_normal((n, w.D))
    k = _keys_from(z, w, Q)
    ns = min(w.sinks, n)
    if ns:
        k[:ns] *= SINK_SCALE
    return k


def cache_values(w: Workload, b: int, g: int, n: int) -> np.ndarray:
    return rng(w.wid, ROLE_VALUES, b, g).standard_normal((n, w.D))


def query(w: Workload, b: int, h: int, step: int = 0) -> np.ndarray:
    return rng(w.wid, ROLE_QUERIES, b, h, step).standard_normal(w.D)


def new_token(w: Workload, b: int, g: int, step: int, Q: np.ndarray | None = None):
    """Key and value appended at decode step `step` (float64, shape [D])."""
    Q = head_basis(w, g) if Q is None else Q
    z = rng(w.wid, ROLE_NEW_KEYS, b, g, step).standard_normal((1, w.D))
    v = rng(w.wid, ROLE_NEW_VALUES, b, g, step).standard_normal(w.D)
    return _keys_from(z, w, Q)[0], v


def score_vector(seed: int, n: int, kind: str = "normal") -> np.ndarray:
    """Free-standing float32 score vectors for selection tests.

    kind: "normal" (continuous), "dup" (few distinct values, many exact ties),
    "zeros" (mixed +0.0 / -0.0 / small values), "sorted" (descending run).
    """
    g = rng(9999, ROLE_SCORES, seed, n)
    if kind == "normal":
        return g.standard_normal(n).astype(np.float32) * np.float32(3.0)
    if kind == "dup":
        return g.integers(-4, 5, n).astype(np.float32) * np.float32(0.5)
    if kind == "zeros":
        x = g.integers(-1, 2, n).astype(np.float32) * np.float32(1e-3)
        z = g.random(n) < 0.5
        x[z] = np.where(g.random(int(z.sum())) < 0.5, np.float32(0.0), np.float32(-0.0))
        return x
    if kind == "sorted":
        return np.sort(g.standard_normal(n).astype(np.float32))[::-1].copy()
    raise ValueError(kind)


# ---------------------------------------------------------------- rounding --

def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 draws to the storage dtype.

    "f32" -> float32 array; "bf16" -> uint16 bit patterns (float64 -> float32
    -> bf16, each to nearest even); "f64" -> unchanged float64.
    """
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    f = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return f
    if dtype != "bf16":
        raise ValueError(dtype)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements (used only to inspect draws)."""
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


# ------------------------------------------------------------ bulk builders --

def _pool_map(fn, items, threads=None):
    threads = threads or min(16, os.cpu_count() or 1)
    if threads <= 1 or len(items) <= 1:
        return [fn(i) for i in items]
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(fn, items))


def bases(w: Workload) -> list[np.ndarray]:
    return [head_basis(w, g) for g in range(w.Hkv)]


def raw_cache(w: Workload, n: int, Qs: list[np.ndarray] | None = None,
              threads=None) -> tuple[np.ndarray, np.ndarray]:
    """Unrotated keys and values of positions 0..n-1, in storage form.

    Returns (K, V) with shape [B, Hkv, n, D]; uint16 bf16 bits or float32.
    """
    Qs = bases(w) if Qs is None else Qs
    st = np.uint16 if w.dtype == "bf16" else np.float32
    K = np.empty((w.B, w.Hkv, n, w.D), st)
    V = np.empty((w.B, w.Hkv, n, w.D), st)

    def one(bg):
        b, g = bg
        K[b, g] = to_storage(cache_keys(w, b, g, n, Qs[g]), w.dtype)
        V[b, g] = to_storage(cache_values(w, b, g, n), w.dtype)

    _pool_map(one, [(b, g) for b in range(w.B) for g in range(w.Hkv)], threads)
    return K, V


def queries(w: Workload, step: int = 0) -> np.ndarray:
    """Queries [B, Hq, D] in storage form."""
    q = np.stack([np.stack([query(w, b, h, step) for h in range(w.Hq)]) for b in range(w.B)])
    return to_storage(q, w.dtype)


def new_tokens(w: Workload, step: int, Qs: list[np.ndarray] | None = None):
    """Key/value appended at `step`: ([B, Hkv, 1, D], [B, Hkv, 1, D]) storage."""
    Qs = bases(w) if Qs is None else Qs
    ks = np.empty((w.B, w.Hkv, 1, w.D))
    vs = np.empty((w.B, w.Hkv, 1, w.D))
    for b in range(w.B):
        for g in range(w.Hkv):
            ks[b, g, 0], vs[b, g, 0] = new_token(w, b, g, step, Qs[g])
    return to_storage(ks, w.dtype), to_storage(vs, w.dtype)
