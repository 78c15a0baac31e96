"""CPU oracle for Loki decode-step sparse attention (float64, numpy).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or call this module.  The GPU library
never routes through it and shares no code with it.

Sources.  Citations name sections of the two web pages titled "Loki: Low-rank
Keys for Efficient Sparse Attention": the AI-extracted summary page
(sections: summary line, "Problem", "Approach", "Key results", "Measured
effects" table, "Limitations") and the arXiv abstract page ("Abstract").
What the method computes, per those pages:

* keys and queries are projected onto a PCA basis calibrated offline
  [summary: summary line; Approach];
* tokens are ranked by attention scores computed from only the top-d
  principal dimensions [summary: Approach; abstract];
* exact attention is computed on the top-k tokens, with no cache entry
  deleted [summary: summary line; Approach].

The pages give no formulas.  Readings taken where they are silent (each one
is listed in the design notes):

  A  exact scores are scaled by 1/sqrt(D), D the full head dimension; the
     ranking scores are left unscaled (a positive scale cannot change a rank);
  B  exact attention uses the rotated query against the rotated full key
     [slab | rest]; for an orthogonal P this equals q.k exactly in real
     arithmetic;
  C  the softmax is normalised over the selected tokens only;
  D  tokens are ranked by the signed score, largest first;
  E  equal scores go to the lower token index; -0.0 equals +0.0;
  F  the selected indices are reported in ascending token order;
  G  k = floor(k_f * S) clamped to [1, S]; k larger than S selects all S;
  H  P holds the eigenvectors of the centred sample covariance (divisor n-1)
     of the calibration keys as columns, eigenvalues descending, each column's
     sign fixed so that its largest-magnitude entry (lowest index among equal
     magnitudes) is positive; cached keys are rotated without subtracting the
     mean;
  J  query head h reads KV head floor(h / (Hq / Hkv));
  R  (RoPE variant) keys carry the rotary position embedding of their cache
     position and the query that of its own position, applied before the PCA
     rotation; dims i and i + D/2 are rotated together by the angle
     pos * base^(-2i/D).  Attention always uses embedded keys; "pre-rotary"
     and "post-rotary" differ only in whether P is calibrated from keys before
     or after the embedding [summary: Measured effects (pre-rotary ablation);
     Surprising findings].

Every function here computes in float64 from the exact values of its inputs
(bf16 and float32 values are exactly representable in float64).
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------- storage --


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16): the pattern is the upper
    half of a float32 whose lower 16 bits are zero."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (8 significant bits, float32's exponent
    range) to nearest, ties to even, and return the uint16 bit patterns.

    The value is written as m * 2**e with 0.5 <= |m| < 1.  Its bf16 quantum is
    2**(e - 8) for normal results and 2**-133 below the smallest normal
    (2**-126), so the rounded value is rint(x / quantum) * quantum (numpy's
    rint rounds half to even; dividing by a power of two is exact).
    """
    x = np.asarray(x, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)
    quantum_exp = np.maximum(e, -125) - 8
    r = np.ldexp(np.rint(np.ldexp(xf, -quantum_exp)), quantum_exp)
    big = np.abs(r) >= 2.0 ** 128  # rounded past the largest bf16: infinity
    r = np.where(big, np.copysign(np.inf, r), r)
    out = np.where(finite, r, x)
    with np.errstate(over="ignore", invalid="ignore"):
        f32 = out.astype(np.float32)  # exact: r has at most 8 significant bits
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored array ("bf16" bits, "f32", "f64")."""
    if dtype == "bf16":
        return bf16_to_f64(a)
    return np.asarray(a, dtype=np.float64)


def from_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 to a storage dtype, to nearest even."""
    if dtype == "bf16":
        return f64_to_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64).copy()
    raise ValueError(dtype)


# ------------------------------------------------------------ calibration --


def calibrate(keys: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Offline PCA of sample keys [summary: summary line ("calibrated
    offline"); Approach ("PCA-project queries and keys")].

    keys: [n, D].  Returns (P, eigvals): P [D, D] float64 whose column c is
    the c-th principal axis, eigvals [D] descending (reading H).
    """
    X = np.asarray(keys, dtype=np.float64)
    n, D = X.shape
    mu = X.mean(axis=0)
    Xc = X - mu
    C = (Xc.T @ Xc) / (n - 1)
    w, V = np.linalg.eigh(C)
    order = np.argsort(-w, kind="stable")
    w = w[order]
    V = V[:, order].copy()
    for c in range(D):
        i = int(np.argmax(np.abs(V[:, c])))
        if V[i, c] < 0:
            V[:, c] = -V[:, c]
    return V, w


# -------------------------------------------------------------------- RoPE --


def rope_embed(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotary position embedding of row vectors (the rotation the pages list
    Loki as building on [summary: "Builds on"]; reading R).

    x [..., D] with D even; pos a scalar or an array broadcasting against
    x[..., 0] (one position per row).  For i < D/2 the pair (x_i, x_{i+D/2})
    is rotated by the angle pos * base^(-2i/D):
        x_i       -> x_i cos - x_{i+D/2} sin
        x_{i+D/2} -> x_{i+D/2} cos + x_i sin
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    h = D // 2
    theta = float(base) ** (-2.0 * np.arange(h, dtype=np.float64) / D)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# ------------------------------------------------------------------ append --


def rotate(x: np.ndarray, P: np.ndarray) -> np.ndarray:
    """Row vectors in the PCA basis: x' = x . P [summary: Approach]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(P, dtype=np.float64)


def append(k_new: np.ndarray, v_new: np.ndarray, P: np.ndarray, d: int, dtype: str,
           rope_base: float | None = None, pos: int = 0):
    """Cache entries for new tokens: keys rotated into the PCA basis and split
    into the leading-d slab and the remaining D-d columns; values unchanged.

    k_new, v_new: [..., T, D] exact float64 values; P [D, D].  With
    rope_base, token t is first embedded at position pos + t (reading R).
    Returns (slab [..., T, d], rest [..., T, D-d], v [..., T, D]) rounded to
    `dtype` to nearest even.
    """
    if rope_base is not None:
        T = np.asarray(k_new).shape[-2]
        k_new = rope_embed(k_new, pos + np.arange(T), rope_base)
    kp = rotate(k_new, P)
    return (from_f64(kp[..., :d], dtype), from_f64(kp[..., d:], dtype),
            from_f64(v_new, dtype))


# -------------------------------------------------------------- selection --


def low_rank_scores(q: np.ndarray, P: np.ndarray, kslab: np.ndarray) -> np.ndarray:
    """Ranking scores from the top-d principal dimensions [summary: Approach;
    abstract]: s_j = sum_{i<d} (q.P)_i * slab[j, i].  Unscaled (reading A).

    q [D], P [D, D], kslab [S, d] -> s [S].
    """
    d = kslab.shape[-1]
    qp = rotate(q, P)
    return np.asarray(kslab, dtype=np.float64) @ qp[:d]


def select_topk(s: np.ndarray, k: int) -> np.ndarray:
    """The min(k, S) tokens with the largest scores, equal scores going to the
    lower index, returned in ascending index order (readings D, E, F).

    A full stable sort by (-s_j, j): np.argsort with kind="stable" on -s keeps
    the original (ascending) index order among equal keys; -0.0 and +0.0
    compare equal.
    """
    s = np.asarray(s, dtype=np.float64)
    kk = min(int(k), s.shape[0])
    order = np.argsort(-s, kind="stable")
    return np.sort(order[:kk]).astype(np.int64)


# -------------------------------------------------------------- attention --


def softmax(e: np.ndarray) -> np.ndarray:
    e = np.asarray(e, dtype=np.float64)
    z = np.exp(e - e.max())
    return z / z.sum()


def attend(q, P, kslab, krest, v, idx):
    """Exact attention over the selected tokens [summary: summary line
    ("exact attention over the selected keys"); Approach].

    e_j = (q.P) . [slab_j | rest_j] / sqrt(D) for j in idx (readings A, B);
    w = softmax(e) over idx only (reading C); out = sum_j w_j v_j.
    Returns (out [D], w [len(idx)]).
    """
    kslab = np.asarray(kslab, dtype=np.float64)
    krest = np.asarray(krest, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    D = kslab.shape[-1] + krest.shape[-1]
    qp = rotate(q, P)
    K = np.concatenate([kslab[idx], krest[idx]], axis=-1)
    e = (K @ qp) / np.sqrt(D)
    w = softmax(e)
    return w @ v[idx], w


def decode_head(q, P, kslab, krest, v, k):
    """One decode step for one (sequence, query head): rank every cached
    token by its low-rank score, keep the top k, attend exactly over them.

    Returns (out [D], idx [min(k,S)] ascending, s [S]).
    """
    s = low_rank_scores(q, P, kslab)
    idx = select_topk(s, k)
    out, _ = attend(q, P, kslab, krest, v, idx)
    return out, idx, s


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head h (reading J)."""
    return h // (Hq // Hkv)


def decode(q, kslab, krest, v, P, k, dtype, S=None, heads=None, rope=None):
    """Decode step for a batch (the oracle of loki_decode).

    q [B, Hq, D], kslab [B, Hkv, S_max, d], krest [B, Hkv, S_max, D-d],
    v [B, Hkv, S_max, D] in storage form (`dtype` "bf16" bits, "f32", "f64");
    P [Hkv, D, D].  Only the first S cached positions are read.
    heads: optional iterable of (b, h) pairs to compute (others are left NaN /
    -1).  rope: optional (base, q_pos), the query's embedding (reading R; the
    cache then holds embedded keys).  Returns (out [B, Hq, D] float64,
    idx [B, Hq, min(k,S)] int64, s [B, Hq, S] float64).
    """
    B, Hq, D = q.shape
    Hkv = kslab.shape[1]
    S = kslab.shape[2] if S is None else S
    kk = min(int(k), S)
    out = np.full((B, Hq, D), np.nan)
    idx = np.full((B, Hq, kk), -1, dtype=np.int64)
    s = np.full((B, Hq, S), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    cache = {}
    for b, h in pairs:
        g = kv_head(h, Hq, Hkv)
        if (b, g) not in cache:
            cache.clear()
            cache[(b, g)] = (to_f64(kslab[b, g, :S], dtype), to_f64(krest[b, g, :S], dtype),
                             to_f64(v[b, g, :S], dtype))
        ks, kr, vv = cache[(b, g)]
        qv = to_f64(q[b, h], dtype)
        if rope is not None:
            qv = rope_embed(qv, rope[1], rope[0])
        o, i, sc = decode_head(qv, np.asarray(P[g], np.float64), ks, kr, vv, kk)
        out[b, h], idx[b, h], s[b, h] = o, i, sc
    return out, idx, s


def attend_indices(q, kslab, krest, v, P, idx, dtype, heads=None, rope=None):
    """Exact attention over a given ascending index set per (b, h): the
    oracle of loki_attend_indices, and of a decode's output over whatever set
    that decode selected.  idx [B, Hq, k]; rope: optional (base, q_pos), the
    query's embedding as in decode() (reading R)."""
    B, Hq, D = q.shape
    Hkv = kslab.shape[1]
    out = np.full((B, Hq, D), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    for b, h in pairs:
        g = kv_head(h, Hq, Hkv)
        sel = np.asarray(idx[b, h], dtype=np.int64)
        qv = to_f64(q[b, h], dtype)
        if rope is not None:
            qv = rope_embed(qv, rope[1], rope[0])
        o, _ = attend(qv, np.asarray(P[g], np.float64),
                      to_f64(kslab[b, g], dtype), to_f64(krest[b, g], dtype),
                      to_f64(v[b, g], dtype), sel)
        out[b, h] = o
    return out


# ------------------------------------------------------------------ dense --


def dense_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Full ("vanilla") attention for one query: softmax(q.K^T / sqrt(D)).V
    [summary: Key results and Measured effects, the baseline Loki is
    compared with]."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    w = softmax((K @ q) / np.sqrt(q.shape[0]))
    return w @ V


def dense_decode(q, kslab, krest, v, P, dtype, S=None, heads=None, rope=None):
    """Full attention over all S cached tokens of the rotated cache: the
    oracle of loki_dense_decode.  Same layouts (and rope) as decode()."""
    B, Hq, D = q.shape
    Hkv = kslab.shape[1]
    S = kslab.shape[2] if S is None else S
    out = np.full((B, Hq, D), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    for b, h in pairs:
        g = kv_head(h, Hq, Hkv)
        K = np.concatenate([to_f64(kslab[b, g, :S], dtype), to_f64(krest[b, g, :S], dtype)], axis=-1)
        qv = to_f64(q[b, h], dtype)
        if rope is not None:
            qv = rope_embed(qv, rope[1], rope[0])
        qp = rotate(qv, np.asarray(P[g], np.float64))
        out[b, h] = dense_attention(qp, K, to_f64(v[b, g, :S], dtype))
    return out


# ------------------------------------------------------- index-set checks --


def topk_gap(s: np.ndarray, k: int) -> float:
    """Relative gap between the k-th and (k+1)-th largest score:
    (tau_k - tau_{k+1}) / max(|tau_k|, |tau_{k+1}|, 1e-30); +inf when k >= S."""
    s = np.asarray(s, dtype=np.float64)
    if k >= s.shape[0]:
        return float("inf")
    srt = np.sort(s)[::-1]
    a, b = srt[k - 1], srt[k]
    return float((a - b) / max(abs(a), abs(b), 1e-30))


def valid_in_band(s: np.ndarray, k: int, cand: np.ndarray, rel: float = 1e-4) -> bool:
    """Whether `cand` is an acceptable top-k set when the k-th place is within
    a relative band `rel` of a tie: it holds min(k,S) distinct ascending
    indices, every score clearly above the k-th is present and no score
    clearly below the (k+1)-th is."""
    s = np.asarray(s, dtype=np.float64)
    S = s.shape[0]
    kk = min(int(k), S)
    cand = np.asarray(cand, dtype=np.int64)
    if cand.shape[0] != kk or np.any(cand < 0) or np.any(cand >= S):
        return False
    if kk > 1 and np.any(np.diff(cand) <= 0):
        return False
    if kk == S:
        return True
    srt = np.sort(s)[::-1]
    tk, tk1 = srt[kk - 1], srt[kk]
    must = np.nonzero(s > tk + rel * abs(tk))[0]
    never = np.nonzero(s < tk1 - rel * abs(tk1))[0]
    cs = set(cand.tolist())
    return all(int(j) in cs for j in must) and not any(int(j) in cs for j in never)
