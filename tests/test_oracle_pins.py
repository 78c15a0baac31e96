"""Pins for the CPU oracle: closed forms, invariants, brute force and a
hand-worked example, chosen so that a plausible slip in the oracle (a dropped
term, a wrong sign, a wrong index, a transposed operand, the wrong scale)
fails at least one of them.  Nothing here compares the oracle with itself.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _haar(rng, D):
    q, r = np.linalg.qr(rng.standard_normal((D, D)))
    return q * np.where(np.diag(r) < 0, -1.0, 1.0)[None, :]


def _rand_case(seed, S=40, D=8, d=3):
    rng = np.random.default_rng(seed)
    P = _haar(rng, D)
    K = rng.standard_normal((S, D))
    V = rng.standard_normal((S, D))
    q = rng.standard_normal(D)
    slab, rest, vv = oracle.append(K, V, P, d, "f64")
    return q, P, K, V, slab, rest, vv


# ------------------------------------------------------ hand-worked example --

def _golden():
    with open(os.path.join(GOLDEN, "worked_example_d4.json")) as fh:
        return json.load(fh)


def test_worked_example_rotation_and_scores():
    f = _golden()
    P = np.array(f["P_rows"], float)
    q = np.array(f["q"], float)
    slab = np.array(f["slab"], float)
    assert np.array_equal(oracle.rotate(q, P), np.array(f["expected"]["q_rot"], float))
    assert np.array_equal(oracle.low_rank_scores(q, P, slab), np.array(f["expected"]["scores"], float))


@pytest.mark.parametrize("kname,k", [("k1", 1), ("k2", 2), ("k3", 3)])
def test_worked_example_decode(kname, k):
    f = _golden()
    P = np.array(f["P_rows"], float)
    q = np.array(f["q"], float)
    slab, rest, V = (np.array(f[n], float) for n in ("slab", "rest", "V"))
    out, idx, _ = oracle.decode_head(q, P, slab, rest, V, k)
    exp = f["expected"][kname]
    assert idx.tolist() == exp["idx"]
    if kname == "k1":
        assert np.array_equal(out, np.array(exp["out"], float))
        return
    z = np.array([math.exp(x) for x in exp["scaled_exact"]])
    w = z / z.sum()
    want = np.zeros(4)
    for wi, j in zip(w, exp["idx"]):
        want += wi * np.array(f["V"][j], float)
    assert np.allclose(out, want, rtol=0, atol=1e-15)


def test_worked_example_dense():
    f = _golden()
    P = np.array(f["P_rows"], float)
    q = np.array(f["q"], float)
    K = np.concatenate([np.array(f["slab"], float), np.array(f["rest"], float)], axis=1)
    V = np.array(f["V"], float)
    out = oracle.dense_attention(oracle.rotate(q, P), K, V)
    z = np.array([math.exp(x) for x in f["expected"]["dense_scaled"]])
    assert np.allclose(out, (z / z.sum()) @ V, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ scores --

def test_full_rank_scores_invariant_under_orthogonal_P():
    # with d = D the ranking score is q'.k' = q P P^T k^T = q.k
    q, P, K, V, slab, rest, vv = _rand_case(1, d=8)
    assert np.allclose(oracle.low_rank_scores(q, P, slab), K @ q, rtol=0, atol=1e-12)


def test_identity_basis_scores_are_leading_dims():
    rng = np.random.default_rng(2)
    K = rng.standard_normal((30, 6))
    q = rng.standard_normal(6)
    slab, rest, _ = oracle.append(K, K, np.eye(6), 2, "f64")
    assert np.array_equal(slab, K[:, :2]) and np.array_equal(rest, K[:, 2:])
    want = [q[0] * K[j, 0] + q[1] * K[j, 1] for j in range(30)]
    assert np.allclose(oracle.low_rank_scores(q, np.eye(6), slab), want, rtol=0, atol=1e-14)


def test_scores_pure_python_brute_force():
    # explicit double loops, transposition-sensitive (P not symmetric)
    q, P, K, V, slab, rest, vv = _rand_case(3, S=12, D=5, d=2)
    s = oracle.low_rank_scores(q, P, slab)
    for j in range(12):
        kj = [sum(K[j][m] * P[m][i] for m in range(5)) for i in range(5)]
        qp = [sum(q[m] * P[m][i] for m in range(5)) for i in range(5)]
        assert abs(s[j] - (qp[0] * kj[0] + qp[1] * kj[1])) < 1e-12


# --------------------------------------------------------------- selection --

def _rank_count_topk(s, k):
    """Independent formulation: j is kept iff fewer than k tokens beat it,
    where l beats j when s_l > s_j, or s_l == s_j and l < j."""
    S = len(s)
    keep = []
    for j in range(S):
        beats = sum(1 for l in range(S) if s[l] > s[j] or (s[l] == s[j] and l < j))
        if beats < k:
            keep.append(j)
    return keep


@pytest.mark.parametrize("kind", ["normal", "dup", "zeros", "sorted"])
@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (64, 16), (100, 99), (130, 1), (130, 130), (50, 70)])
def test_topk_matches_rank_counting(kind, n, k):
    s = synth.score_vector(n * 31 + k, n, kind).astype(np.float64)
    assert oracle.select_topk(s, k).tolist() == _rank_count_topk(s, min(k, n))


def test_topk_brute_force_full_sort_tiny():
    s = synth.score_vector(5, 256, "normal").astype(np.float64)
    srt = sorted(range(256), key=lambda j: (-s[j], j))
    assert oracle.select_topk(s, 64).tolist() == sorted(srt[:64])


def test_topk_special_cases():
    s = synth.score_vector(6, 50, "normal").astype(np.float64)
    assert oracle.select_topk(s, 50).tolist() == list(range(50))
    assert oracle.select_topk(s, 1).tolist() == [int(np.argmax(s))]
    assert oracle.select_topk(np.zeros(20), 7).tolist() == list(range(7))
    # -0.0 and +0.0 are equal: lower index wins
    assert oracle.select_topk(np.array([-0.0, 0.0, -1.0, 0.0]), 2).tolist() == [0, 1]
    # signed ranking, not by magnitude
    assert oracle.select_topk(np.array([-5.0, 1.0, 0.5]), 1).tolist() == [1]


def test_gap_and_band_rule():
    s = np.array([5.0, 4.0, 3.0, 2.0])
    assert oracle.topk_gap(s, 2) == pytest.approx(0.25)
    s2 = np.array([5.0, 3.0, 3.0 * (1 - 1e-6), 1.0])
    assert oracle.topk_gap(s2, 2) < 1e-4
    assert oracle.valid_in_band(s2, 2, np.array([0, 1]))
    assert oracle.valid_in_band(s2, 2, np.array([0, 2]))
    assert not oracle.valid_in_band(s2, 2, np.array([1, 2]))
    assert not oracle.valid_in_band(s2, 2, np.array([2, 0]))


# --------------------------------------------------------------- attention --

def test_full_budget_equals_dense_attention_on_original_keys():
    # d = D, k = S: Loki is dense attention (orthogonal invariance)
    q, P, K, V, slab, rest, vv = _rand_case(7, S=33, D=8, d=8)
    out, idx, _ = oracle.decode_head(q, P, slab, rest, vv, 33)
    assert idx.tolist() == list(range(33))
    assert np.allclose(out, oracle.dense_attention(q, K, V), rtol=0, atol=1e-12)


def test_all_tokens_kept_with_small_d_is_still_dense():
    # k = S with d < D: the exact scores must use all D dims and 1/sqrt(D)
    q, P, K, V, slab, rest, vv = _rand_case(8, S=25, D=8, d=2)
    out, _, _ = oracle.decode_head(q, P, slab, rest, vv, 25)
    e = K @ q / math.sqrt(8)
    w = np.exp(e - e.max())
    assert np.allclose(out, (w / w.sum()) @ V, rtol=0, atol=1e-12)


def test_weights_sum_to_one_and_k1_returns_argmax_row():
    q, P, K, V, slab, rest, vv = _rand_case(9, S=40, D=8, d=3)
    idx = oracle.select_topk(oracle.low_rank_scores(q, P, slab), 10)
    _, w = oracle.attend(q, P, slab, rest, vv, idx)
    assert abs(w.sum() - 1.0) < 1e-15 and np.all(w > 0)
    out, idx1, s = oracle.decode_head(q, P, slab, rest, vv, 1)
    assert idx1.tolist() == [int(np.argmax(s))]
    assert np.array_equal(out, V[idx1[0]])


def test_constant_values_and_linearity_in_v():
    q, P, K, V, slab, rest, vv = _rand_case(10, S=30, D=8, d=3)
    c = np.arange(8, dtype=float) - 3.0
    out, _, _ = oracle.decode_head(q, P, slab, rest, np.tile(c, (30, 1)), 9)
    assert np.allclose(out, c, rtol=0, atol=1e-13)
    o1, _, _ = oracle.decode_head(q, P, slab, rest, vv, 9)
    o2, _, _ = oracle.decode_head(q, P, slab, rest, -2.5 * vv, 9)
    assert np.allclose(o2, -2.5 * o1, rtol=0, atol=1e-13)


def test_softmax_over_selected_tokens_only():
    # two selected tokens whose exact scores differ by ln 3 after scaling;
    # an unselected token with a huge exact score must get no weight
    D = 4
    P = np.eye(D)
    q = np.array([1.0, 0.0, 1.0, 0.0])
    a = 2.0 * math.log(3.0)  # scaled by 1/sqrt(4) -> ln 3
    slab = np.array([[5.0, 0.0], [4.0, 0.0], [-9.0, 0.0]])
    rest = np.array([[a, 0.0], [0.0, 0.0], [1000.0, 0.0]])
    V = np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0], [0, 0, 1.0, 0]])
    out, idx, _ = oracle.decode_head(q, P, slab, rest, V, 2)
    assert idx.tolist() == [0, 1]
    # e0 - e1 = (5 + a - 4) / 2 = 0.5 + ln 3 -> w0/w1 = 3 e^0.5
    r = 3.0 * math.exp(0.5)
    assert np.allclose(out, [r / (1 + r), 1 / (1 + r), 0, 0], rtol=0, atol=1e-15)


def test_permutation_equivariance():
    q, P, K, V, slab, rest, vv = _rand_case(11, S=50, D=8, d=3)
    out, idx, s = oracle.decode_head(q, P, slab, rest, vv, 12)
    perm = np.random.default_rng(0).permutation(50)
    out2, idx2, _ = oracle.decode_head(q, P, slab[perm], rest[perm], vv[perm], 12)
    inv = np.argsort(perm)
    assert sorted(perm[idx2].tolist()) == idx.tolist()
    assert np.allclose(out2, out, rtol=0, atol=1e-13)
    assert inv.shape == (50,)


def test_gqa_head_mapping_consecutive_groups():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, S, D, d = 2, 6, 2, 20, 8, 3
    P = np.stack([_haar(rng, D) for _ in range(Hkv)])
    q = rng.standard_normal((B, Hq, D))
    Kraw = rng.standard_normal((B, Hkv, S, D))
    V = rng.standard_normal((B, Hkv, S, D))
    slab = np.empty((B, Hkv, S, d)); rest = np.empty((B, Hkv, S, D - d))
    for g in range(Hkv):
        slab[:, g], rest[:, g], _ = oracle.append(Kraw[:, g], V[:, g], P[g], d, "f64")
    out, idx, _ = oracle.decode(q, slab, rest, V, P, 5, "f64")
    for b in range(B):
        for h in range(Hq):
            g = h // 3  # heads 0,1,2 -> KV 0; 3,4,5 -> KV 1
            o, i, _ = oracle.decode_head(q[b, h], P[g], slab[b, g], rest[b, g], V[b, g], 5)
            assert np.array_equal(i, idx[b, h]) and np.array_equal(o, out[b, h])
    assert oracle.kv_head(2, 6, 2) == 0 and oracle.kv_head(3, 6, 2) == 1


def test_decode_reads_only_first_S_positions():
    q, P, K, V, slab, rest, vv = _rand_case(13, S=30, D=8, d=3)
    big = lambda a: np.concatenate([a, 1e6 * np.ones((5, a.shape[1]))])[None, None]
    out, idx, _ = oracle.decode(q[None, None], big(slab), big(rest), big(vv), P[None], 7, "f64", S=30)
    o, i, _ = oracle.decode_head(q, P, slab, rest, vv, 7)
    assert np.array_equal(out[0, 0], o) and np.array_equal(idx[0, 0], i)


# ------------------------------------------------------------- calibration --

def test_calibration_orthogonal_descending_and_spectrum():
    w = synth.WORKLOADS["l2_7b"]
    Q = synth.head_basis(w, 0)
    keys = synth.calib_keys(w, 0, Q)
    P, ev = oracle.calibrate(keys)
    assert np.allclose(P.T @ P, np.eye(w.D), rtol=0, atol=1e-12)
    assert np.all(np.diff(ev) <= 0)
    sig2 = synth.spectrum(w) ** 2
    # sample eigenvalues within 6 standard errors sigma^2 sqrt(2/n) of truth
    # for the well-separated leading ones
    lead = 8
    assert np.all(np.abs(ev[:lead] - sig2[:lead]) < 6 * sig2[:lead] * math.sqrt(2 / w.calib_n))
    # the leading-d columns capture (nearly) the true top-d key variance:
    # sum_c P_c^T C P_c for C = Q diag(sigma^2) Q^T against sum_{i<d} sigma_i^2
    d = w.d
    C = (Q * sig2[None, :]) @ Q.T
    captured = np.trace(P[:, :d].T @ C @ P[:, :d])
    assert 0.999 < captured / sig2[:d].sum() <= 1.0 + 1e-12


def test_calibration_exact_low_rank_subspace_and_signs():
    rng = np.random.default_rng(14)
    D, r, n = 10, 3, 500
    Q = _haar(rng, D)
    z = rng.standard_normal((n, r)) * np.array([3.0, 2.0, 1.0])
    X = z @ Q[:, :r].T + np.arange(D) * 0.1  # mean offset must not matter
    P, ev = oracle.calibrate(X)
    assert np.allclose(P[:, :r] @ P[:, :r].T, Q[:, :r] @ Q[:, :r].T, atol=1e-10)
    assert np.all(np.abs(ev[r:]) < 1e-10)
    for c in range(D):
        i = int(np.argmax(np.abs(P[:, c])))
        assert P[i, c] > 0


def test_calibration_known_covariance_closed_form():
    # keys +-a e1, +-b e2 exactly (zero mean): covariance diag(a^2, b^2, 0) * n/(n-1)
    a, b = 3.0, 2.0
    X = np.array([[a, 0, 0], [-a, 0, 0], [0, b, 0], [0, -b, 0]])
    P, ev = oracle.calibrate(X)
    assert np.allclose(ev, [2 * a * a / 3, 2 * b * b / 3, 0.0], atol=1e-12)
    assert np.allclose(np.abs(P), np.eye(3), atol=1e-12)
    assert np.allclose(P, np.eye(3), atol=1e-12)  # sign convention


# ------------------------------------------------------------------ append --

def test_append_rotation_is_invertible_and_split():
    rng = np.random.default_rng(15)
    P = _haar(rng, 8)
    K = rng.standard_normal((5, 8))
    slab, rest, v = oracle.append(K, -K, P, 3, "f64")
    assert np.allclose(np.concatenate([slab, rest], axis=1) @ P.T, K, atol=1e-13)
    assert np.array_equal(v, -K)


def test_bf16_rounding_exhaustive_roundtrip():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_to_f64(bits)
    fin = np.isfinite(vals)
    back = oracle.f64_to_bf16(vals[fin])
    same = back == bits[fin]
    # -0.0 maps to itself, every finite pattern round-trips
    assert same.all()


def test_bf16_rounding_ties_and_halfway():
    one = 1.0
    ulp = 2.0 ** -7
    x = np.array([one + ulp / 2, one + 3 * ulp / 2, one + ulp / 2 + 2.0 ** -40,
                  -(one + ulp / 2), 2.0 ** -130, 3.0 * 2.0 ** -134, 2.0 ** 200])
    got = oracle.bf16_to_f64(oracle.f64_to_bf16(x))
    want = [1.0, 1.0 + 2 * ulp, 1.0 + ulp, -1.0, 2.0 ** -130, 4.0 * 2.0 ** -134, np.inf]
    assert got.tolist() == want


def test_bf16_rounding_matches_torch_for_float32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(16)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f64_to_bf16(x.astype(np.float64)), ref)


def test_append_bf16_within_half_ulp():
    rng = np.random.default_rng(17)
    P = _haar(rng, 16)
    K = rng.standard_normal((64, 16))
    slab, rest, _ = oracle.append(K, K, P, 4, "bf16")
    exact = K @ P
    got = np.concatenate([oracle.bf16_to_f64(slab), oracle.bf16_to_f64(rest)], axis=1)
    _, e = np.frexp(exact)
    assert np.all(np.abs(got - exact) <= np.ldexp(1.0, e - 9) * (1 + 1e-12))


# ------------------------------------------------------------------- RoPE --

def test_rope_closed_form_on_basis_vectors():
    # D = 4, base 10000: pair (0, 2) turns by pos, pair (1, 3) by pos / 100
    p = 3.0
    e0, e1, e2 = np.eye(4)[0], np.eye(4)[1], np.eye(4)[2]
    assert np.allclose(oracle.rope_embed(e0, p, 10000.0), [math.cos(p), 0, math.sin(p), 0],
                       rtol=0, atol=1e-15)
    assert np.allclose(oracle.rope_embed(e1, p, 10000.0),
                       [0, math.cos(p / 100), 0, math.sin(p / 100)], rtol=0, atol=1e-15)
    # the second member of a pair turns the same way: (0, 1) -> (-sin, cos)
    assert np.allclose(oracle.rope_embed(e2, p, 10000.0), [-math.sin(p), 0, math.cos(p), 0],
                       rtol=0, atol=1e-15)
    # D = 8, base 4: theta_i = 4^(-i/4) = 2^(-i/2)
    x = np.zeros(8)
    x[3] = 1.0
    got = oracle.rope_embed(x, 2.0, 4.0)
    ang = 2.0 * 2.0 ** -1.5
    want = np.zeros(8)
    want[3], want[7] = math.cos(ang), math.sin(ang)
    assert np.allclose(got, want, rtol=0, atol=1e-15)


def test_rope_position_zero_identity_norms_and_composition():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 16))
    assert np.array_equal(oracle.rope_embed(x, 0, 10000.0), x)
    y = oracle.rope_embed(x, 37, 10000.0)
    # every (i, i + D/2) pair keeps its length
    assert np.allclose(x[:, :8] ** 2 + x[:, 8:] ** 2, y[:, :8] ** 2 + y[:, 8:] ** 2, rtol=1e-13)
    # turning by a then by b is turning by a + b; by -a undoes a
    assert np.allclose(oracle.rope_embed(y, 5, 10000.0), oracle.rope_embed(x, 42, 10000.0),
                       rtol=0, atol=1e-12)
    assert np.allclose(oracle.rope_embed(y, -37, 10000.0), x, rtol=0, atol=1e-12)


def test_rope_scores_depend_on_relative_position_only():
    # <R_m q, R_n k> = <R_(m-n) q, k>: the property rotary embedding is built for
    rng = np.random.default_rng(12)
    q, K = rng.standard_normal(32), rng.standard_normal((6, 32))
    n = np.array([0, 3, 10, 100, 4000, 32767])
    m = 32767
    lhs = oracle.rope_embed(K, n, 500000.0) @ oracle.rope_embed(q, m, 500000.0)
    rhs = np.array([oracle.rope_embed(q, m - nj, 500000.0) @ K[j] for j, nj in enumerate(n)])
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-9)


def test_rope_per_row_positions_match_scalar_calls():
    rng = np.random.default_rng(13)
    K = rng.standard_normal((4, 8))
    pos = np.array([0, 1, 7, 1000])
    rows = np.stack([oracle.rope_embed(K[i], pos[i], 10000.0) for i in range(4)])
    assert np.array_equal(oracle.rope_embed(K, pos, 10000.0), rows)


def test_rope_append_embeds_each_token_at_its_slot():
    rng = np.random.default_rng(14)
    D, d, T, pos = 8, 3, 5, 20
    P = _haar(rng, D)
    K, V = rng.standard_normal((T, D)), rng.standard_normal((T, D))
    slab, rest, vv = oracle.append(K, V, P, d, "f64", rope_base=10000.0, pos=pos)
    want = np.stack([oracle.rope_embed(K[t], pos + t, 10000.0) for t in range(T)]) @ P
    assert np.allclose(np.concatenate([slab, rest], axis=-1), want, rtol=0, atol=1e-13)
    assert np.array_equal(vv, V)


def test_rope_decode_full_budget_is_dense_attention_on_embedded_keys():
    # d = D, k = S with embedded keys and query: softmax((R_m q).(R_j k_j)/sqrt(D)).V
    rng = np.random.default_rng(15)
    S, D, m, base = 30, 8, 29, 10000.0
    P = _haar(rng, D)
    K, V, q = rng.standard_normal((S, D)), rng.standard_normal((S, D)), rng.standard_normal(D)
    slab, rest, vv = oracle.append(K, V, P, D, "f64", rope_base=base, pos=0)
    out, idx, _ = oracle.decode(q[None, None], slab[None, None], rest[None, None], vv[None, None],
                                P[None], S, "f64", rope=(base, m))
    Ke = oracle.rope_embed(K, np.arange(S), base)
    want = oracle.dense_attention(oracle.rope_embed(q, m, base), Ke, V)
    assert idx[0, 0].tolist() == list(range(S))
    assert np.allclose(out[0, 0], want, rtol=0, atol=1e-12)
    dense = oracle.dense_decode(q[None, None], slab[None, None], rest[None, None], vv[None, None],
                                P[None], "f64", rope=(base, m))
    assert np.allclose(dense[0, 0], want, rtol=0, atol=1e-12)
    # without the query's embedding the result differs: the option is applied
    plain, _, _ = oracle.decode(q[None, None], slab[None, None], rest[None, None],
                                vv[None, None], P[None], S, "f64")
    assert not np.allclose(plain[0, 0], want, atol=1e-6)


# ------------------------------------- given-index and dense attention, GQA --
# Brute force written out with Python floats from the unrotated keys: for an
# orthogonal P, (q.P).(k.P) = q.k, so exact attention over any token set can be
# formed without the basis.  B > 1 and G = Hq/Hkv = 3 make a wrong KV-head
# mapping (h mod Hkv), a per-query-head basis (P[h]) or a dropped rest block
# disagree with it.

def _gqa_cache(seed, B=2, Hq=6, Hkv=2, S=24, D=8, d=3, S_max=None):
    rng = np.random.default_rng(seed)
    S_max = S if S_max is None else S_max
    P = np.stack([_haar(rng, D) for _ in range(Hkv)])
    q = rng.standard_normal((B, Hq, D))
    K = rng.standard_normal((B, Hkv, S_max, D))
    V = rng.standard_normal((B, Hkv, S_max, D))
    slab = np.empty((B, Hkv, S_max, d))
    rest = np.empty((B, Hkv, S_max, D - d))
    for g in range(Hkv):
        slab[:, g], rest[:, g], _ = oracle.append(K[:, g], V[:, g], P[g], d, "f64")
    return q, P, K, V, slab, rest


def _brute_attention(qv, K, V, sel):
    """softmax over sel of q.K_j / sqrt(D), then the weighted sum of V rows."""
    D = len(qv)
    e = [sum(float(qv[m]) * float(K[j][m]) for m in range(D)) / math.sqrt(D) for j in sel]
    top = max(e)
    z = [math.exp(x - top) for x in e]
    tot = sum(z)
    return [sum(z[i] * float(V[j][c]) for i, j in enumerate(sel)) / tot for c in range(D)]


def test_attend_indices_gqa_batch_brute_force():
    B, Hq, Hkv, S, D = 2, 6, 2, 24, 8
    q, P, K, V, slab, rest = _gqa_cache(21, B, Hq, Hkv, S, D)
    rng = np.random.default_rng(22)
    k = 7
    idx = np.stack([np.stack([np.sort(rng.choice(S, k, replace=False)) for _ in range(Hq)])
                    for _ in range(B)])
    out = oracle.attend_indices(q, slab, rest, V, P, idx, "f64")
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)  # heads 0-2 read KV head 0, heads 3-5 KV head 1
            want = _brute_attention(q[b, h], K[b, g], V[b, g], idx[b, h].tolist())
            assert np.allclose(out[b, h], want, rtol=0, atol=1e-12), (b, h)


def test_attend_indices_single_token_returns_its_value_row():
    B, Hq, Hkv, S, D = 2, 6, 2, 24, 8
    q, P, K, V, slab, rest = _gqa_cache(23, B, Hq, Hkv, S, D)
    idx = np.array([[[(5 * h + 3 * b) % S] for h in range(Hq)] for b in range(B)])
    out = oracle.attend_indices(q, slab, rest, V, P, idx, "f64")
    for b in range(B):
        for h in range(Hq):
            assert np.array_equal(out[b, h], V[b, h // 3, idx[b, h, 0]])


def test_dense_decode_gqa_batch_brute_force_on_original_keys():
    # S < S_max: the positions past S hold huge values that must not be read
    B, Hq, Hkv, S, S_max, D, d = 2, 6, 2, 20, 26, 8, 3
    q, P, K, V, slab, rest = _gqa_cache(24, B, Hq, Hkv, S, D, d, S_max)
    slab[:, :, S:] = 1e6
    rest[:, :, S:] = 1e6
    V[:, :, S:] = 1e6
    out = oracle.dense_decode(q, slab, rest, V, P, "f64", S=S)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            want = _brute_attention(q[b, h], K[b, g], V[b, g], list(range(S)))
            assert np.allclose(out[b, h], want, rtol=0, atol=1e-12), (b, h)


def test_dense_decode_equals_full_budget_decode_for_any_slab_width():
    # dense attention is Loki with every token kept, whatever d is
    B, Hq, Hkv, S, D = 2, 6, 2, 16, 8
    for d in (1, 3, 8):
        q, P, K, V, slab, rest = _gqa_cache(25 + d, B, Hq, Hkv, S, D, d)
        dense = oracle.dense_decode(q, slab, rest, V, P, "f64")
        full, idx, _ = oracle.decode(q, slab, rest, V, P, S, "f64")
        assert np.array_equal(idx, np.broadcast_to(np.arange(S), idx.shape))
        assert np.allclose(dense, full, rtol=0, atol=1e-13)


def test_rope_attend_indices_brute_force_on_embedded_keys():
    # a subset of tokens with the query embedded at q_pos: brute force over the
    # embedded (unrotated) keys; without the embedding the result differs
    rng = np.random.default_rng(31)
    B, Hq, Hkv, S, D, d, base, m = 2, 4, 2, 18, 8, 3, 10000.0, 40
    P = np.stack([_haar(rng, D) for _ in range(Hkv)])
    q = rng.standard_normal((B, Hq, D))
    K = rng.standard_normal((B, Hkv, S, D))
    V = rng.standard_normal((B, Hkv, S, D))
    slab = np.empty((B, Hkv, S, d))
    rest = np.empty((B, Hkv, S, D - d))
    for g in range(Hkv):
        slab[:, g], rest[:, g], _ = oracle.append(K[:, g], V[:, g], P[g], d, "f64",
                                                  rope_base=base, pos=0)
    idx = np.stack([np.stack([np.sort(rng.choice(S, 6, replace=False)) for _ in range(Hq)])
                    for _ in range(B)])
    out = oracle.attend_indices(q, slab, rest, V, P, idx, "f64", rope=(base, m))
    plain = oracle.attend_indices(q, slab, rest, V, P, idx, "f64")
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            Ke = [oracle.rope_embed(K[b, g, j], j, base) for j in range(S)]
            want = _brute_attention(oracle.rope_embed(q[b, h], m, base), Ke, V[b, g],
                                    idx[b, h].tolist())
            assert np.allclose(out[b, h], want, rtol=0, atol=1e-12), (b, h)
            assert not np.allclose(plain[b, h], want, atol=1e-6)
