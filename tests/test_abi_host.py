"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every symbol include/mx.h declares, and rejects bad arguments before any HIP
call (fake device addresses are never dereferenced)."""

import ctypes
import os
import re

import pytest

from helpers import ROOT, mx

HEADER = os.path.join(ROOT, "include", "mx.h")
P = ctypes.c_void_p


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return mx().lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(mx().SIGNATURES), "binding and header disagree"


def test_version_and_status_strings(L):
    assert L.mx_abi_version() == 12
    assert L.mx_status_string(0) == b"MX_OK"
    assert L.mx_status_string(1) == b"MX_ERR_INVALID_ARGUMENT"
    assert L.mx_status_string(2) == b"MX_ERR_UNSUPPORTED"
    assert L.mx_status_string(3) == b"MX_ERR_HIP"
    assert L.mx_status_string(42) == b"MX_UNKNOWN_STATUS"


A = 0x10000  # aligned fake addresses
B = 0x20000000
C = 0x30000000
D = 0x40000000


def qa(x=A, M=4, K=64, ld=64, q=B, s=C):
    return mx().lib().mx_quantize_act(P(x), M, K, ld, P(q), P(s), P(0))


def test_quantize_act_rejects_bad_arguments(L):
    INV = 1
    assert qa(K=33) == INV
    assert qa(K=0) == INV
    assert qa(K=-32) == INV
    assert qa(M=-1) == INV
    assert qa(ld=32) == INV  # ld < K
    assert qa(ld=68) == INV  # rows not 16-byte aligned
    assert qa(x=0) == INV
    assert qa(q=0) == INV
    assert qa(s=0) == INV
    assert qa(x=A + 2) == INV  # misaligned
    assert qa(q=B + 8) == INV
    assert qa(q=A + 64) == INV  # q overlaps x
    assert qa(s=B + 100) == INV  # s overlaps q
    assert b"K" in L.mx_last_error_message() or len(L.mx_last_error_message()) > 0
    assert qa(M=0) == 0  # empty call: nothing to do
    assert qa(M=0, x=0, q=0, s=0) == 0


def test_quantize_weight_rejects_bad_arguments(L):
    f = L.mx_quantize_weight
    assert f(P(A), 7, 4, 64, 64, P(B), P(C), P(0)) == 1  # dtype
    assert f(P(A), 1, 4, 48, 48, P(B), P(C), P(0)) == 1  # K % 32
    assert f(P(A), 1, 4, 64, 66, P(B), P(C), P(0)) == 1  # f32 rows not 16-byte aligned
    assert f(P(A), 0, 4, 64, 68, P(B), P(C), P(0)) == 1  # bf16 rows not 16-byte aligned
    assert f(P(0), 1, 4, 64, 64, P(B), P(C), P(0)) == 1
    assert f(P(A), 1, 0, 64, 64, P(0), P(0), P(0)) == 0


def lin(x=A, M=8, K=64, wq=B, ws=C, N=256, bias=0, epi=0, y=D):
    return mx().lib().mx_linear_fused(P(x), M, K, P(wq), P(ws), N, P(bias), epi, P(y), P(0))


def test_linear_rejects_bad_arguments(L):
    assert lin(K=40) == 1
    assert lin(epi=5) == 1
    assert lin(M=-3) == 1
    assert lin(N=-16) == 1
    assert lin(x=0) == 1
    assert lin(wq=0) == 1
    assert lin(y=0) == 1
    assert lin(y=D + 4) == 1  # misaligned
    assert lin(bias=A + 1) == 1  # odd bias address
    assert lin(y=B) == 1  # y overlaps wq
    assert lin(y=A) == 1  # y overlaps x
    assert lin(N=264) == 2  # N % 16: outside the kernel's tiling
    assert lin(K=1 << 21) == 2
    assert lin(M=0) == 0
    assert lin(N=0) == 0
    q = L.mx_linear_q
    assert q(P(A), P(0), 8, 64, P(B), P(C), 256, P(0), 0, P(D), P(0)) == 1  # NULL xs
    assert q(P(A), P(C + 64), 8, 64, P(B), P(C), 256, P(0), 0, P(A), P(0)) == 1  # y overlaps xq


def test_slab_rows(L):
    assert [L.mx_slab_rows(r) for r in (0, 1, 255, 256, 257, 75348)] == [0, 256, 256, 256, 512, 75520]
    assert L.mx_slab_rows(-1) == -1


def test_slab_calls_reject_bad_arguments(L):
    qs = L.mx_quantize_act_slab
    assert qs(P(A), 4, 96, 96, P(B), P(C), P(0)) == 1  # K % 64
    assert qs(P(A), 4, 64, 64, P(B), P(0), P(0)) == 1  # NULL s
    # codes of a slab cover R = 256 rows: 256 * 64 bytes from B; scales at B + 8192 overlap them
    assert qs(P(A), 4, 64, 64, P(B), P(B + 8192), P(0)) == 1
    assert qs(P(A), 0, 64, 64, P(0), P(0), P(0)) == 0
    qw = L.mx_quantize_weight_slab
    assert qw(P(A), 1, 4, 32, 32, P(B), P(C), P(0)) == 1  # K % 64
    assert qw(P(A), 9, 4, 64, 64, P(B), P(C), P(0)) == 1  # dtype
    pk = L.mx_slab_pack
    assert pk(P(A), P(C), 4, 96, P(B), P(D), P(0)) == 1  # K % 64
    assert pk(P(A), P(C + 1), 4, 64, P(B), P(D), P(0)) == 1  # odd scale address
    assert pk(P(A), P(C), 4, 64, P(A + 128), P(D), P(0)) == 1  # output overlaps input
    assert pk(P(A), P(C), 0, 64, P(0), P(0), P(0)) == 0
    ls = L.mx_linear_slab

    def lsl(xq=A, xs=C, M=8, K=64, wq=B, ws=C + 0x100000, N=256, bias=0, epi=0, y=D):
        return ls(P(xq), P(xs), M, K, P(wq), P(ws), N, P(bias), epi, P(y), P(0))

    assert lsl(K=96) == 1
    assert lsl(epi=3) == 1
    assert lsl(xs=C + 2) == 1  # scales 4-byte aligned
    assert lsl(xq=0) == 1
    assert lsl(y=A + 8192) == 1  # y overlaps the token slab (256 rows x 64 B)
    assert lsl(N=264) == 2
    assert lsl(M=0) == 0 and lsl(N=0) == 0
    # The 128-token-tile form takes the same arguments and checks.
    ls = L.mx_linear_slab_m128
    assert lsl(K=96) == 1 and lsl(epi=3) == 1 and lsl(xs=C + 2) == 1 and lsl(xq=0) == 1
    assert lsl(y=A + 8192) == 1 and lsl(y=D + 8) == 1 and lsl(y=0) == 1
    assert lsl(N=264) == 2
    assert lsl(M=0) == 0 and lsl(N=0) == 0
    rq = L.mx_linear_slab_requant

    def lrq(xq=A, xs=C, M=8, K=64, wq=B, ws=C + 0x100000, N=256, epi=1, hq=D, hs=D + 0x1000000):
        return rq(P(xq), P(xs), M, K, P(wq), P(ws), N, P(0), epi, P(hq), P(hs), P(0))

    assert lrq(N=272) == 1  # N (the next linear's K) must be a multiple of 64
    assert lrq(hq=0) == 1 and lrq(hs=0) == 1
    assert lrq(hq=D + 8) == 1  # misaligned codes
    assert lrq(hs=D + 1024) == 1  # hs inside hq (256 rows x 256 B)
    assert lrq(hq=A) == 1  # hq overlaps the token slab
    assert lrq(K=96) == 1
    assert lrq(M=1 << 20, N=4096) == 2  # output slab of 2^32 bytes
    assert lrq(M=0) == 0 and lrq(N=0) == 0


def test_linear_one_call_sizes_and_bad_arguments(L):
    # activation slab, then the largest partial-sum workspace of the tuner's
    # candidates; each rounded to 256
    r256 = lambda v: (v + 255) // 256 * 256  # noqa: E731
    act = r256(512 * 5120 + 512 * 160)
    assert L.mx_linear_ws_bytes(300, 5120, 5120) == act + r256(L.mx_linear_tune_ws_bytes(300, 5120, 5120))
    assert L.mx_linear_tune_ws_bytes(300, 5120, 5120) == 8 * 2 * 20 * 65536 * 4  # split-K 8: the largest
    assert L.mx_linear_ws_bytes(0, 64, 16) == 0 and L.mx_linear_ws_bytes(4, 64, 0) == 0
    assert L.mx_linear_ws_bytes(1, 96, 16) == -1 and L.mx_linear_ws_bytes(-1, 64, 16) == -1
    f = L.mx_linear
    need = L.mx_linear_ws_bytes(8, 64, 256)
    assert need == r256(256 * 64 + 256 * 2)  # one K slab: only unsplit plans, no partial sums
    E = 0x50000000

    def call(x=A, M=8, K=64, ldx=64, wq=B, ws=C, N=256, epi=0, y=D, wsp=E, nb=need):
        return f(P(x), M, K, ldx, P(wq), P(ws), N, P(0), epi, P(y), P(wsp), nb, P(0))

    assert call(K=96, ldx=96) == 1  # K % 64
    assert call(nb=need - 1) == 1  # workspace too small
    assert call(wsp=0) == 1 and call(x=0) == 1 and call(y=0) == 1
    assert call(wsp=E + 16) == 1  # workspace not 256-byte aligned
    assert call(ldx=60) == 1
    assert call(wsp=A) == 1  # workspace overlaps x
    assert call(y=B) == 1  # y overlaps the weights
    assert call(N=264) == 2
    assert call(M=0) == 0


def test_splitk_sizes_and_choice(L):
    # fp32 partial tiles: splits * ceil(M/256) * ceil(N/256) * 256 KiB
    assert L.mx_linear_splitk_ws_bytes(128, 5120, 12) == 12 * 20 * 65536 * 4
    assert L.mx_linear_splitk_ws_bytes(0, 64, 1) == 0
    assert L.mx_linear_splitk_ws_bytes(1, 16, 0) == -1 and L.mx_linear_splitk_ws_bytes(-1, 16, 1) == -1
    # about one workgroup per CU, at least two K slabs per range
    assert L.mx_linear_splitk_choose(128, 5120, 5120) == 8  # 20 tiles; capped at 8
    assert L.mx_linear_splitk_choose(512, 5120, 10240) == 3  # 80 tiles
    assert L.mx_linear_splitk_choose(75348, 5120, 15360) == 1
    assert L.mx_linear_splitk_choose(1, 256, 256) == 2  # K/64 = 4 slabs: two per range
    assert L.mx_linear_splitk_choose(1, 64, 256) == 1
    assert L.mx_linear_splitk_choose(0, 64, 256) == 1


def test_splitk_rejects_bad_arguments(L):
    f = L.mx_linear_slab_splitk
    need = L.mx_linear_splitk_ws_bytes(8, 256, 2)
    E = 0x50000000

    def call(xq=A, xs=B, M=8, K=256, wq=C, ws=C + (1 << 20), N=256, epi=0, y=D, splits=2, wsp=E, nb=need):
        return f(P(xq), P(xs), M, K, P(wq), P(ws), N, P(0), epi, P(y), splits, P(wsp), nb, P(0))

    assert call(splits=0) == 1 and call(splits=5) == 1  # outside [1, K/64]
    assert call(K=96) == 1  # K % 64
    assert call(nb=need - 1) == 1
    assert call(wsp=0) == 1 and call(y=0) == 1 and call(xq=0) == 1
    assert call(wsp=E + 16) == 1
    assert call(wsp=A) == 1  # workspace overlaps the token codes
    assert call(y=E) == 1  # y overlaps the workspace
    assert call(epi=7) == 1
    assert call(N=264) == 2
    assert call(M=0) == 0 and call(N=0) == 0


def test_small_sizes_and_choice(L):
    # No GPU here: the choice assumes 256 compute units (MI355X).
    assert L.mx_linear_small_ws_bytes(128, 5120, 3) == 3 * 128 * 5120 * 4  # fp32 partials [splits][M][N]
    assert L.mx_linear_small_ws_bytes(128, 5120, 1) == 0  # one range writes y directly
    assert L.mx_linear_small_ws_bytes(1, 16, 0) == -1 and L.mx_linear_small_ws_bytes(-1, 16, 2) == -1
    assert L.mx_linear_small_choose(128, 5120, 5120) == 3  # 80 tiles of 128 x 64
    assert L.mx_linear_small_choose(512, 5120, 10240) == 1  # 640 tiles fill the CUs
    assert L.mx_linear_small_choose(1, 256, 256) == 2  # 4 tiles; K/64 = 4 slabs: two per range
    assert L.mx_linear_small_choose(1, 64, 256) == 1
    assert L.mx_linear_small_choose(1, 5120, 64) == 8  # capped at 8
    assert L.mx_linear_small_choose(0, 64, 256) == 1


def test_small_rejects_bad_arguments(L):
    f = L.mx_linear_slab_small
    need = L.mx_linear_small_ws_bytes(8, 256, 2)
    E = 0x50000000

    def call(xq=A, xs=B, M=8, K=256, wq=C, ws=C + (1 << 20), N=256, epi=0, y=D, splits=2, wsp=E, nb=need):
        return f(P(xq), P(xs), M, K, P(wq), P(ws), N, P(0), epi, P(y), splits, P(wsp), nb, P(0))

    assert call(splits=0) == 1 and call(splits=5) == 1  # outside [1, K/64]
    assert call(K=96) == 1  # K % 64
    assert call(nb=need - 1) == 1
    assert call(wsp=0) == 1 and call(y=0) == 1 and call(xq=0) == 1
    assert call(wsp=E + 16) == 1
    assert call(wsp=A) == 1  # workspace overlaps the token codes
    assert call(y=E) == 1  # y overlaps the workspace
    assert call(epi=7) == 1
    assert call(N=264) == 2
    assert call(M=0) == 0 and call(N=0) == 0
    # 32-bit K-range offsets: (K/64 + 16) * 64 * rows must stay below 2^31
    # (checked before the buffers' extents, so fake addresses do).
    assert call(M=1 << 20, K=5120, nb=1 << 40) == 2  # (80 + 16) * 64 * 2^20 > 2^31
    assert call(M=8, K=5120, N=1 << 20, nb=1 << 40) == 2


def test_balanced_plan_sizes(L):
    # No GPU here: the plan assumes 256 compute units (MI355X).
    KB256 = 65536 * 4
    assert L.mx_linear_balanced_ws_bytes(75348, 5120, 5120) == 8 * 12 * KB256  # 5900 tiles: 12 in the last round
    assert L.mx_linear_balanced_ws_bytes(75348, 5120, 15360) == 7 * 36 * KB256  # 17700 tiles: 36, 256 // 36 = 7
    assert L.mx_linear_balanced_ws_bytes(128, 5120, 5120) == 8 * 20 * KB256  # 20 tiles, all split
    assert L.mx_linear_balanced_ws_bytes(256 * 16, 512, 256 * 16) == 0  # 256 tiles: whole rounds
    assert L.mx_linear_balanced_ws_bytes(300, 128, 256) == 0  # K/128 = 1: nothing to split
    assert L.mx_linear_balanced_ws_bytes(0, 64, 16) == 0
    assert L.mx_linear_balanced_ws_bytes(8, 96, 16) == -1 and L.mx_linear_balanced_ws_bytes(-1, 64, 16) == -1


def test_balanced_rejects_bad_arguments(L):
    f = L.mx_linear_slab_balanced
    need = L.mx_linear_balanced_ws_bytes(8, 256, 256)
    assert need > 0
    E = 0x50000000

    def call(xq=A, xs=B, M=8, K=256, wq=C, ws=C + (1 << 20), N=256, epi=0, y=D, wsp=E, nb=need):
        return f(P(xq), P(xs), M, K, P(wq), P(ws), N, P(0), epi, P(y), P(wsp), nb, P(0))

    assert call(K=96) == 1 and call(epi=3) == 1 and call(y=0) == 1
    assert call(nb=need - 1) == 1 and call(wsp=0) == 1 and call(wsp=E + 16) == 1
    assert call(wsp=A) == 1 and call(y=E) == 1
    assert call(N=264) == 2
    assert call(M=0) == 0


def test_pc_calls_reject_bad_arguments(L):
    qa = L.mx_pc_quantize_act_slab
    qw = L.mx_pc_quantize_weight_slab
    E = 0x50000000
    assert qa(P(A), 8, 96, 96, P(B), P(E), P(0)) == 1  # K % 64
    assert qa(P(A), 8, 64, 60, P(B), P(E), P(0)) == 1  # pitch < K
    assert qa(P(A), 8, 64, 64, P(0), P(E), P(0)) == 1
    assert qa(P(A), 8, 64, 64, P(B), P(E + 2), P(0)) == 1  # scales not 4-byte aligned
    assert qa(P(A), 8, 64, 64, P(A), P(E), P(0)) == 1  # codes overlap x
    assert qa(P(A), 0, 64, 64, P(B), P(E), P(0)) == 0
    assert qw(P(A), 7, 8, 64, 64, P(B), P(E), P(0)) == 1  # dtype
    assert qw(P(A), 1, 8, 64, 66, P(B), P(E), P(0)) == 1  # f32 pitch not 16-byte aligned
    f = L.mx_pc_linear_slab

    def call(xq=A, xs=E, M=8, K=128, wq=C, ws=E + 4096, N=256, epi=0, y=D):
        return f(P(xq), P(xs), M, K, P(wq), P(ws), N, P(0), epi, P(y), P(0))

    assert call(K=96) == 1 and call(epi=5) == 1 and call(xs=0) == 1 and call(y=0) == 1
    assert call(ws=E + 2) == 1 and call(y=C) == 1
    assert call(N=264) == 2
    assert call(M=0) == 0 and call(N=0) == 0


def test_forced_unsupported_path(L, monkeypatch):
    monkeypatch.setenv("MX_FORCE_UNSUPPORTED", "1")
    assert qa() == 2
    assert lin() == 2
    assert b"MX_FORCE_UNSUPPORTED" in L.mx_last_error_message()


def test_oracle_and_product_share_no_code():
    pkg = os.path.join(ROOT, "mxfp8_w8a8_quantized_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, re.M), fn
                assert "oracle/" not in text, fn
    for fn in os.listdir(os.path.join(ROOT, "oracle")):
        if fn.endswith(".py"):
            text = open(os.path.join(ROOT, "oracle", fn)).read()
            assert "mxfp8_w8a8_quantized_amd" not in text, fn
            assert "synth" not in text, fn


def test_per_shape_plan():
    # No GPU here: the split choices assume 256 compute units (MI355X).
    import mxfp8_w8a8_quantized_amd as pkg

    assert pkg.plan_linear(128, 5120, 5120) == ("small", 3)
    assert pkg.plan_linear(256, 5120, 5120) == ("small", 1)
    assert pkg.plan_linear(512, 5120, 10240) == ("slab_m128", 1)
    assert pkg.plan_linear(512, 1024, 1024) == ("splitk", 8)  # 8 tiles: too few for one round of 128-token tiles
    assert pkg.plan_linear(1024, 5120, 15360) == ("slab", 1)  # 240 tiles
    assert pkg.plan_linear(75348, 5120, 15360) == ("slab", 1)
    assert pkg.plan_ws_bytes(("small", 3), 128, 5120) == 3 * 128 * 5120 * 4
    assert pkg.plan_ws_bytes(("small", 1), 128, 5120) == 0
    assert pkg.plan_ws_bytes(("splitk", 3), 512, 10240) == 3 * 2 * 40 * 65536 * 4
    assert pkg.plan_ws_bytes(("slab", 1), 75348, 15360) == 0
    assert pkg.plan_ws_bytes(("balanced", 1), 75348, 5120, 5120) == 8 * 12 * 65536 * 4


def test_plan_entry_points_host_side(L):
    import ctypes

    kind, splits = ctypes.c_int(-1), ctypes.c_int(-1)

    def default(M, K, N):
        st = L.mx_linear_plan_default(M, K, N, ctypes.byref(kind), ctypes.byref(splits))
        return st, kind.value, splits.value

    # The rule: few-token kernel up to 256 tokens; 128-token tiles when the
    # 256 x 256 tiles number 32 to 128; split-K while they are fewer than the
    # CUs (256 assumed without a GPU); else slab.
    assert default(128, 5120, 5120) == (0, 2, 3)
    assert default(256, 5120, 5120) == (0, 2, 1)
    assert default(512, 5120, 10240) == (0, 4, 1)
    assert default(300, 5120, 5120) == (0, 4, 1)  # 40 tiles
    assert default(300, 5120, 3840) == (0, 1, 8)  # 30 tiles: split-K
    assert default(2048, 5120, 4096) == (0, 4, 1)  # 128 tiles
    assert default(2048, 5120, 4352) == (0, 0, 1)  # 136 tiles: split-K would be 1
    assert default(75348, 5120, 15360) == (0, 0, 1)
    assert default(0, 64, 64) == (0, 0, 1)  # empty: nothing to split
    assert default(8, 96, 64)[0] == 1 and default(-1, 64, 64)[0] == 1
    assert L.mx_linear_plan_default(8, 64, 64, None, ctypes.byref(splits)) == 1
    # Workspace of each kind
    assert L.mx_linear_plan_ws_bytes(0, 1, 75348, 5120, 15360) == 0
    assert L.mx_linear_plan_ws_bytes(0, 2, 75348, 5120, 15360) == -1  # slab takes splits 1
    assert L.mx_linear_plan_ws_bytes(1, 3, 512, 5120, 10240) == L.mx_linear_splitk_ws_bytes(512, 10240, 3)
    assert L.mx_linear_plan_ws_bytes(2, 3, 128, 5120, 5120) == 3 * 128 * 5120 * 4
    assert L.mx_linear_plan_ws_bytes(3, 1, 75348, 5120, 5120) == L.mx_linear_balanced_ws_bytes(75348, 5120, 5120)
    assert L.mx_linear_plan_ws_bytes(4, 1, 512, 5120, 10240) == 0
    assert L.mx_linear_plan_ws_bytes(4, 2, 512, 5120, 10240) == -1  # 128-token tiles take splits 1
    assert L.mx_linear_plan_ws_bytes(7, 1, 8, 64, 64) == -1
    # The tuner's workspace covers its largest candidate: at 128 x 5120 x 5120
    # split-K with 8 ranges (8 x 20 partial tiles of 256 KiB).
    assert L.mx_linear_tune_ws_bytes(128, 5120, 5120) == 8 * 20 * 65536 * 4
    assert L.mx_linear_tune_ws_bytes(8, 96, 64) == -1
    # Argument errors before any device call
    E = 0x50000000
    assert L.mx_linear_slab_plan(9, 1, P(A), P(B), 8, 256, P(C), P(C + (1 << 20)), 256, P(0), 0, P(D), P(E), 1 << 20,
                                 P(0)) == 1
    assert L.mx_linear_slab_plan(0, 2, P(A), P(B), 8, 256, P(C), P(C + (1 << 20)), 256, P(0), 0, P(D), P(E), 1 << 20,
                                 P(0)) == 1
    assert L.mx_linear_slab_plan(4, 2, P(A), P(B), 8, 256, P(C), P(C + (1 << 20)), 256, P(0), 0, P(D), P(E), 1 << 20,
                                 P(0)) == 1
    assert L.mx_linear_tune(P(A), P(B), 8, 256, P(C), P(C + (1 << 20)), 256, P(0), 0, P(D), P(E), 1 << 20, 0, P(0),
                            ctypes.byref(kind), ctypes.byref(splits)) == 1  # reps 0
    assert L.mx_linear_tune(P(A), P(B), 8, 256, P(C), P(C + (1 << 20)), 256, P(0), 0, P(D), P(E), 1 << 20, 5, P(0),
                            None, ctypes.byref(splits)) == 1
    L.mx_linear_plan_clear()


def test_probe_rejects_bad_arguments(L):
    f = L.mx_probe_mfma
    assert f(P(0), P(B), 1024, 10, 256, P(D), P(0)) == 1
    assert f(P(A), P(B), 1022, 10, 256, P(D), P(0)) == 1  # bytes % 4
    assert f(P(A), P(B), 0, 10, 256, P(D), P(0)) == 1
    assert f(P(A), P(B), (1 << 31) + 4, 10, 256, P(D), P(0)) == 1
    assert f(P(A), P(B), 1024, 0, 256, P(D), P(0)) == 1
    assert f(P(A), P(B), 1024, 10, 0, P(D), P(0)) == 1
    assert f(P(A + 2), P(B), 1024, 10, 256, P(D), P(0)) == 1


def test_linear_noalloc_rejects_bad_arguments_before_any_launch(L):
    f = L.mx_linear_noalloc

    def call(x=A, M=8, K=64, ldx=64, wq=B, ws=C, N=256, epi=0, y=D):
        return f(P(x), M, K, ldx, P(wq), P(ws), N, P(0), epi, P(y), P(0))

    assert call(K=96, ldx=96) == 1  # K % 64
    assert call(x=0) == 1 and call(y=0) == 1 and call(wq=0) == 1
    assert call(ldx=60) == 1
    assert call(y=B) == 1  # y overlaps the weights
    assert call(N=264) == 2
    assert call(M=20000, K=5120, ldx=5120) == 2  # activation slab past the 64 MiB scratch array
    assert b"scratch" in L.mx_last_error_message() or b"needed" in L.mx_last_error_message()
    assert call(M=0) == 0 and call(N=0) == 0
