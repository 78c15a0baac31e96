"""C-ABI checks that need no GPU: the library loads, exports every function
include/loki.h declares, rejects bad arguments on the host before launching
anything, and its host-only PCA calibration matches the oracle."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "loki.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(loki_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    import sparse_attention_decode_loki_amd as loki
    if not os.path.exists(loki.LIB_PATH):
        pytest.fail("libloki.so not built: run python -m sparse_attention_decode_loki_amd.build_lib")
    loki.load()
    return loki


def test_header_declarations_exported(L):
    names = _declared()
    assert len(names) >= 11
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (loki_[a-z_]+)", out))
    assert set(names) <= exported, set(names) - exported
    assert set(names) == set(L.exported_symbols())


def test_version_and_status_strings(L):
    lib = L.load()
    with open(os.path.join(ROOT, "include", "loki.h")) as fh:
        header = int(re.search(r"#define LOKI_ABI_VERSION (\d+)", fh.read()).group(1))
    assert lib.loki_abi_version() == header == 4
    for st in (0, -1, -2, -3, -4, 7):
        assert lib.loki_status_string(st)
    assert L.status_string(-2).startswith("LOKI_EWORKSPACE")


FAKE = ctypes.c_void_p(0x100000)       # never dereferenced on rejected calls
FAKE_MIS = ctypes.c_void_p(0x100004)   # misaligned


def _decode(lib, **kw):
    a = dict(q=FAKE, ks=FAKE, kr=FAKE, v=FAKE, P=FAKE, B=2, Hq=4, Hkv=2, D=128, d=32, S=100,
             S_max=128, k=25, dt=1, out=FAKE, idx=FAKE, ws=FAKE, wsb=1 << 40, path=2)
    a.update(kw)
    return lib.loki_decode_ex(a["q"], a["ks"], a["kr"], a["v"], a["P"], a["B"], a["Hq"], a["Hkv"],
                              a["D"], a["d"], a["S"], a["S_max"], a["k"], a["dt"], a["out"],
                              a["idx"], a["ws"], a["wsb"], a["path"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(d=0), -1), (dict(d=129), -1), (dict(k=0), -1), (dict(S=0), -1), (dict(S=200), -1),
    (dict(Hq=3), -1), (dict(Hkv=0), -1), (dict(dt=7), -1), (dict(B=-1), -1), (dict(path=9), -1),
    (dict(q=None), -1), (dict(ks=None), -1), (dict(kr=None), -1), (dict(v=None), -1),
    (dict(P=None), -1), (dict(out=None), -1), (dict(idx=None), -1),
    (dict(ks=FAKE_MIS), -1), (dict(v=FAKE_MIS), -1), (dict(out=FAKE_MIS), -1),
    (dict(D=96, d=32), -4), (dict(d=20), -4), (dict(dt=0, d=18), -4),
    (dict(ws=None), -2), (dict(wsb=1024), -2), (dict(ws=FAKE_MIS), -2),
])
def test_decode_rejects_bad_arguments(L, kw, want):
    assert _decode(L.load(), **kw) == want


def test_decode_fused_rejects_when_lds_too_small(L):
    # q' + scores + kept ids over 56 KiB cannot take the fused path
    assert _decode(L.load(), path=1, S=20000, S_max=20000, k=5000) == -4
    lib = L.load()
    assert lib.loki_decode_path(1, 4, 4, 128, 32, 20000, 5000, 1, 1) == -4
    assert lib.loki_decode_path(16, 40, 40, 128, 32, 3584, 896, 1, 0) == 1   # auto -> fused
    assert lib.loki_decode_path(8, 32, 8, 128, 32, 8192, 2048, 1, 0) == 1    # GQA that fits -> fused
    assert lib.loki_decode_path(8, 32, 8, 128, 32, 8192, 2048, 0, 0) == 1    # ... float32 cache too
    assert lib.loki_decode_path(4, 32, 8, 128, 64, 32768, 4096, 1, 0) == 2   # GQA, k = S/8 -> split
    assert lib.loki_decode_path(4, 32, 8, 128, 32, 32768, 8192, 1, 0) == 3   # GQA, k = S/4 -> union
    assert lib.loki_decode_path(4, 32, 8, 128, 32, 32768, 8192, 0, 0) == 2   # ... float32 cache -> split
    assert lib.loki_decode_path(4, 32, 8, 128, 16, 32768, 8192, 1, 0) == 2   # d < D - 96 -> split
    assert lib.loki_decode_path(1, 32, 32, 128, 32, 4096, 1024, 1, 0) == 4   # few heads -> sliced
    assert lib.loki_decode_path(1, 4, 4, 128, 32, 100, 25, 1, 2) == 2
    assert lib.loki_decode_path(1, 4, 4, 128, 32, 100, 25, 1, 1) == 1
    assert lib.loki_decode_path(1, 4, 4, 128, 33, 100, 25, 1, 0) == -4


def test_auto_takes_fused_by_rows_and_context(L):
    # where the sliced path does not apply (k <= 64 leaves one slice per
    # row): fused when rows * S + 420000 >= 190 * S
    lib = L.load()
    assert lib.loki_decode_path(1, 1, 1, 128, 32, 2222, 64, 1, 0) == 1     # short rows: any count
    assert lib.loki_decode_path(1, 1, 1, 128, 32, 2223, 64, 1, 0) == 2
    assert lib.loki_decode_path(1, 87, 87, 128, 32, 4097, 64, 1, 0) == 2
    assert lib.loki_decode_path(1, 88, 88, 128, 32, 4097, 64, 1, 0) == 1
    assert lib.loki_decode_path(1, 138, 138, 128, 32, 8192, 64, 1, 0) == 2
    assert lib.loki_decode_path(1, 139, 139, 128, 32, 8192, 64, 1, 0) == 1
    assert lib.loki_decode_path(2, 4, 2, 128, 32, 500, 125, 1, 0) == 1     # grouped heads too
    assert lib.loki_decode_path(1, 4, 4, 128, 32, 12000, 3000, 1, 0) == 2  # LDS too small
    assert lib.loki_decode_path(1, 224, 224, 128, 32, 4096, 1024, 1, 0) == 1  # slices gain nothing


def test_auto_takes_sliced_where_its_plan_slices(L):
    lib = L.load()
    # fewer rows than compute units, rows of at least 2048 tokens
    assert lib.loki_decode_path(1, 32, 32, 128, 32, 4096, 1024, 1, 0) == 4
    assert lib.loki_decode_path(1, 1, 1, 128, 32, 2223, 555, 1, 0) == 4
    assert lib.loki_decode_path(2, 32, 8, 128, 32, 4096, 1024, 1, 0) == 4    # grouped heads
    assert lib.loki_decode_path(1, 190, 190, 128, 32, 11000, 2750, 1, 0) == 4
    assert lib.loki_decode_path(1, 32, 32, 128, 32, 2048, 512, 1, 0) == 4
    assert lib.loki_decode_path(1, 32, 32, 128, 32, 2047, 512, 1, 0) == 1    # shorter rows: fused
    # whole rounds of the compute units plus a remainder of at most 64 rows
    assert lib.loki_decode_path(9, 32, 32, 128, 32, 3584, 896, 1, 0) == 4    # 288 rows
    assert lib.loki_decode_path(18, 32, 32, 128, 32, 3584, 896, 1, 0) == 4   # 576 rows
    assert lib.loki_decode_path(16, 32, 32, 128, 32, 3584, 896, 1, 0) == 1   # 512: no remainder
    assert lib.loki_decode_path(16, 40, 40, 128, 32, 3584, 896, 1, 0) == 1   # remainder 128
    assert lib.loki_decode_path(1, 289, 289, 128, 32, 3584, 896, 1, 0) == 1  # rows not a multiple of 8


def test_union_path_only_for_two_or_four_heads_per_kv_head(L):
    lib = L.load()
    assert lib.loki_decode_path(8, 32, 8, 128, 32, 8192, 2048, 1, 3) == 3    # G = 4
    assert lib.loki_decode_path(2, 8, 4, 128, 32, 700, 100, 1, 3) == 3       # G = 2
    assert lib.loki_decode_path(2, 8, 8, 128, 32, 700, 100, 1, 3) == -4      # G = 1
    assert lib.loki_decode_path(2, 16, 2, 128, 32, 700, 100, 1, 3) == -4     # G = 8
    assert lib.loki_decode_path(1, 4, 1, 128, 32, 1 << 17, 100, 1, 3) == 3
    assert lib.loki_decode_path(1, 4, 1, 128, 32, (1 << 17) + 1, 100, 1, 3) == -4
    assert lib.loki_decode_path(1, 4, 1, 128, 32, 100, 10, 1, 5) == -1       # no such path
    # rejected before any pointer is looked at
    assert _decode(lib, Hq=4, Hkv=4, path=3) == -4
    assert _decode(lib, path=5) == -1


def test_sliced_path_needs_the_fused_kernels_lds(L):
    # the sliced path runs the single-kernel decode with each row's gather
    # split: same LDS limit as FUSED, (D + S + min(k, S)) floats <= 56 KiB
    lib = L.load()
    assert lib.loki_decode_path(1, 32, 32, 128, 32, 4096, 1024, 1, 4) == 4
    assert lib.loki_decode_path(1, 2, 2, 128, 32, 11000, 3208, 1, 4) == 4
    assert lib.loki_decode_path(1, 2, 2, 128, 32, 11000, 3209, 1, 4) == -4
    # it needs a workspace (for its slice partials) when a row has several slices
    assert _decode(lib, Hq=4, Hkv=4, S=100, S_max=128, k=100, path=4, ws=None, wsb=0) == -2


def test_empty_batch_is_a_noop(L):
    lib = L.load()
    assert _decode(lib, B=0) == 0
    assert lib.loki_kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 2, 128, 32, 64, 0, 4, 1, None) == 0
    assert lib.loki_kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 128, 32, 64, 0, 0, 1, None) == 0
    assert lib.loki_topk(FAKE, 0, 10, 12, 3, FAKE, None) == 0


def test_append_rejects_bad_arguments(L):
    lib = L.load()
    ap = lambda **kw: lib.loki_kv_append(
        kw.get("k", FAKE), kw.get("v", FAKE), FAKE, kw.get("ks", FAKE), kw.get("kr", FAKE), FAKE,
        2, 2, kw.get("D", 128), kw.get("d", 32), kw.get("S_max", 64), kw.get("pos", 0),
        kw.get("T", 4), kw.get("dt", 1), None)
    assert ap(pos=62) == -1          # pos + T > S_max
    assert ap(pos=-1) == -1
    assert ap(T=-1) == -1
    assert ap(d=0) == -1
    assert ap(k=None) == -1
    assert ap(kr=None) == -1
    assert ap(ks=FAKE_MIS) == -1
    assert ap(D=96) == -4
    assert ap(d=4) == -4
    assert ap(dt=3) == -1


@pytest.mark.parametrize("base", [0.0, -10000.0, float("nan"), float("inf")])
def test_rope_entry_points_reject_bad_base(L, base):
    lib = L.load()
    assert lib.loki_kv_append_rope(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 128, 32, 64, 0, 4, 1,
                                   base, None) == -1
    assert lib.loki_decode_rope(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 2, 128, 32, 100, 128, 25, 1, 99,
                                base, FAKE, FAKE, FAKE, 1 << 40, 2, None) == -1
    assert lib.loki_decode_step_rope(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 2, 128, 32, 99,
                                     128, 25, 1, base, FAKE, FAKE, FAKE, 1 << 40, 2, None) == -1
    assert lib.loki_dense_decode_rope(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 2, 128, 32, 10, 10, 1, 9,
                                      base, FAKE, FAKE, 1 << 40, None) == -1


def test_rope_entry_points_check_like_the_plain_ones(L):
    lib = L.load()
    base = 10000.0
    dec = lambda **kw: lib.loki_decode_rope(
        FAKE, FAKE, FAKE, FAKE, FAKE, kw.get("B", 2), 4, 2, 128, kw.get("d", 32), 100, 128, 25, 1,
        kw.get("q_pos", 99), base, FAKE, FAKE, kw.get("ws", FAKE), kw.get("wsb", 1 << 40),
        kw.get("path", 2), None)
    assert dec(q_pos=-1) == -1
    assert dec(d=20) == -4
    assert dec(ws=None) == -2
    assert dec(B=0) == 0                 # empty batch: nothing launched
    assert dec(path=9) == -1
    assert lib.loki_kv_append_rope(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 128, 32, 64, 62, 4, 1,
                                   base, None) == -1     # pos + T > S_max
    assert lib.loki_kv_append_rope(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 128, 32, 64, 0, 0, 1,
                                   base, None) == 0      # T = 0
    assert lib.loki_decode_step_rope(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 2, 128, 32,
                                     128, 128, 25, 1, base, FAKE, FAKE, FAKE, 1 << 40, 2,
                                     None) == -1         # pos >= S_max
    assert lib.loki_dense_decode_rope(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 2, 128, 32, 10, 10, 1, -3,
                                      base, FAKE, FAKE, 1 << 40, None) == -1


def test_topk_and_scores_reject_bad_arguments(L):
    lib = L.load()
    assert lib.loki_topk(FAKE, 3, 10, 9, 3, FAKE, None) == -1      # ld < S
    assert lib.loki_topk(FAKE, 3, 10, 12, 0, FAKE, None) == -1
    assert lib.loki_topk(FAKE_MIS, 3, 10, 12, 3, FAKE, None) == -1
    assert lib.loki_topk(FAKE, 3, 10, 10, 3, FAKE, None) == -1     # ld not a multiple of 4
    assert lib.loki_scores(FAKE, FAKE, FAKE, 1, 2, 2, 128, 32, 10, 10, 1, FAKE, None, 0, None) == -2
    assert lib.loki_attend_indices(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 2, 128, 32, 10, 10, FAKE,
                                   11, 1, FAKE, FAKE, 1 << 30, None) == -1   # k > S
    assert lib.loki_dense_decode(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 2, 128, 32, 10, 10, 1, FAKE,
                                 FAKE, 16, None) == -2


def test_workspace_size_properties(L):
    lib = L.load()
    ws = lambda *a: lib.loki_decode_workspace_size(*a)
    assert ws(0, 4, 100, 128, 10) == 0 and ws(1, 4, 0, 128, 10) == 0 and ws(1, 4, 100, 0, 1) == 0
    for args in [(16, 40, 3584, 128, 896), (1, 32, 4096, 128, 1024), (4, 32, 32768, 128, 4096),
                 (1, 1, 256, 64, 64)]:
        n = ws(*args)
        assert n % 256 == 0 and n > 0
        B, Hq, S_max, D, k = args
        # q', the score rows and the kept-position bitmaps at least
        assert n >= B * Hq * (D * 4 + S_max * 4 + S_max // 8)
        assert ws(B, Hq, S_max, D, k + 100) >= n


def test_workspace_size_argument_order(L):
    # (B, Hq, S_max, D, k_max): a long cache with a small head dim needs about
    # 4 bytes per cached position per row; a short cache with a huge head dim
    # needs at least two D-wide rows (q' and a slice partial)
    ws = L.load().loki_decode_workspace_size
    long_cache = ws(1, 1, 1 << 20, 64, 1)
    assert 4 << 20 <= long_cache < 6 << 20
    assert ws(1, 1, 64, 1 << 20, 1) >= 8 << 20
    assert L.workspace_size(1, 1, 1 << 20, 64, 1) == long_cache


def test_calibrate_matches_oracle(L):
    w = synth.WORKLOADS["l2_7b"]
    keys = synth.calib_keys(w, 3).astype(np.float32)
    P, ev = L.calibrate(keys)
    Po, evo = oracle.calibrate(keys.astype(np.float64))
    assert np.allclose(ev, evo, rtol=1e-9, atol=1e-12)
    assert np.max(np.abs(P.astype(np.float64) - Po)) < 1e-6
    assert np.allclose(P.T.astype(np.float64) @ P, np.eye(w.D), atol=1e-5)


def test_calibrate_small_and_degenerate(L):
    X = np.array([[3, 0, 0], [-3, 0, 0], [0, 2, 0], [0, -2, 0]], dtype=np.float32)
    P, ev = L.calibrate(X)
    assert np.allclose(ev, [6.0, 8.0 / 3.0, 0.0], atol=1e-12)
    assert np.allclose(P, np.eye(3), atol=1e-7)
    lib = L.load()
    P1 = np.zeros(1, np.float32)
    assert lib.loki_calibrate(np.ones(1, np.float32).ctypes.data, 1, 1, P1.ctypes.data, None) == -1
    assert lib.loki_calibrate(None, 5, 1, P1.ctypes.data, None) == -1


def test_stream_read_rejects_bad_arguments(L):
    lib = L.load()
    assert lib.loki_stream_read(FAKE, 1024, FAKE, 0, None) == -1
    assert lib.loki_stream_read(FAKE, 1024, FAKE, 65537, None) == -1
    assert lib.loki_stream_read(FAKE, 1000, FAKE, 4, None) == -1
    assert lib.loki_stream_read(None, 1024, FAKE, 4, None) == -1
    assert lib.loki_stream_read(FAKE_MIS, 1024, FAKE, 4, None) == -1
    assert lib.loki_stream_read(FAKE, 0, FAKE, 4, None) == 0


def test_stream_read_shares_rejects_bad_arguments(L):
    lib = L.load()
    f = lib.loki_stream_read_shares
    assert f(FAKE, 4096, FAKE, 0, 256, 4, None) == -1       # no workgroups
    assert f(FAKE, 4096, FAKE, 65537, 256, 4, None) == -1
    assert f(FAKE, 4096, FAKE, 4, 128, 4, None) == -1       # block size
    assert f(FAKE, 4096, FAKE, 4, 256, 3, None) == -1       # loads in flight
    assert f(FAKE, 4096, FAKE, 3, 256, 4, None) == -1       # shares not whole chunks
    assert f(None, 4096, FAKE, 4, 256, 4, None) == -1
    assert f(FAKE_MIS, 4096, FAKE, 4, 256, 4, None) == -1
    assert f(FAKE, 0, FAKE, 4, 1024, 16, None) == 0


def test_decode_noalloc_rejects_before_touching_a_device(L):
    lib = L.load()
    a = [FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 2, 128, 32, 100, 128, 25, 1, FAKE, FAKE, 2, None]
    bad = list(a); bad[12] = 0          # k < 1
    assert lib.loki_decode_noalloc(*bad) == -1
    bad = list(a); bad[13] = 7          # dtype
    assert lib.loki_decode_noalloc(*bad) == -1
    bad = list(a); bad[16] = 9          # path
    assert lib.loki_decode_noalloc(*bad) == -1
    bad = list(a); bad[8] = 96          # D
    assert lib.loki_decode_noalloc(*bad) == -4
    bad = list(a); bad[16] = 3; bad[6] = 3; bad[7] = 1  # union with 3 query heads per KV head
    assert lib.loki_decode_noalloc(*bad) == -4
    # split path over 64 x 64 rows of 32768 tokens: 512 MiB of scores > the scratch
    big = list(a); big[5:12] = [64, 64, 64, 128, 32, 32768, 32768]
    assert lib.loki_decode_noalloc(*big) == -2
    assert L.NOALLOC_SCRATCH_BYTES == 32 << 20
    zero = list(a); zero[5] = 0         # B == 0: nothing to do
    assert lib.loki_decode_noalloc(*zero) == 0
