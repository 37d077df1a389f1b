"""The C ABI on the CPU: the library loads without a GPU, exports every symbol
declared in include/w4a16.h, and rejects bad arguments before any HIP call."""

import ctypes
import os
import re
import subprocess

import pytest

import w4a16_decode_gemv_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")

pytestmark = pytest.mark.skipif(not os.path.exists(w4.LIB_PATH), reason="library not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    return sorted({n for n in names if n.startswith(("w4a16_", "w3a16_", "awq_", "nf4_"))})


def test_header_declares_the_binding_set():
    assert _declared() == sorted(w4.exported_symbols())


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", w4.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", out, flags=re.M))
    for name in _declared():
        assert name in exported, name


def test_version_and_status_text():
    lib = w4.load()
    assert lib.w4a16_layout_version() == 1
    assert lib.w4a16_status_str(0) == b"ok"
    assert lib.w4a16_status_str(5) == b"HIP runtime error"
    assert lib.w4a16_status_str(99) == b"unknown status"
    assert lib.w4a16_gemv_max_m() == 8


# fake, suitably aligned addresses: the calls must fail before touching them
A16 = 0x10000
A2 = 0x10002


def _linear(**kw):
    a = dict(x=A16, q=A16, s=A16, z=A16, M=1, N=64, K=256, group=128, y=A16)
    a.update(kw)
    lib = w4.load()
    return lib.w4a16_linear(a["x"], a["q"], a["s"], a["z"], a["M"], a["N"], a["K"], a["group"], a["y"], None)


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(x=None), w4.ERR_NULL),
        (dict(q=None), w4.ERR_NULL),
        (dict(y=None), w4.ERR_NULL),
        (dict(group=16), w4.ERR_UNSUPPORTED),
        (dict(M=0), w4.ERR_SHAPE),
        (dict(N=-1), w4.ERR_SHAPE),
        (dict(K=200), w4.ERR_SHAPE),
        (dict(K=131072 + 128), w4.ERR_SHAPE),
        (dict(M=65537), w4.ERR_SHAPE),
        (dict(x=A2), w4.ERR_ALIGN),
        (dict(q=A16 + 4), w4.ERR_ALIGN),
        (dict(y=A16 + 1), w4.ERR_ALIGN),
        (dict(s=A16 + 1), w4.ERR_ALIGN),
    ],
)
def test_linear_rejects_before_any_hip_call(kw, status):
    assert _linear(**kw) == status
    assert w4.load().w4a16_last_error() != b""


def test_linear_path_rejects_unknown_path_and_big_m_on_gemv():
    lib = w4.load()
    assert lib.w4a16_linear_path(6, A16, A16, A16, A16, 1, 64, 256, 128, A16, None) == w4.ERR_UNSUPPORTED
    assert lib.w4a16_linear_path(-1, A16, A16, A16, A16, 1, 64, 256, 128, A16, None) == w4.ERR_UNSUPPORTED
    # the K-lane MFMA kernel (path 4) and the one-range split-K kernel (path 5) take groups of 128 only
    assert lib.w4a16_linear_path(4, A16, A16, A16, A16, 64, 64, 256, 64, A16, None) == w4.ERR_UNSUPPORTED
    assert lib.w4a16_linear_path(5, A16, A16, A16, A16, 64, 64, 256, 32, A16, None) == w4.ERR_UNSUPPORTED
    assert lib.w4a16_linear_path(1, A16, A16, A16, A16, 9, 64, 256, 128, A16, None) == w4.ERR_UNSUPPORTED
    # the small-batch MFMA kernel takes M <= 32
    assert lib.w4a16_linear_path(3, A16, A16, A16, A16, 33, 64, 256, 128, A16, None) == w4.ERR_UNSUPPORTED
    # M * ceil(K / 16384) must stay <= 8 on the GEMV path
    assert lib.w4a16_linear_path(1, A16, A16, A16, A16, 8, 64, 32768, 128, A16, None) == w4.ERR_UNSUPPORTED


@pytest.mark.parametrize(
    "args,status",
    [
        ((None, None, 64, 256, 4, 128, A16, A16, A16), w4.ERR_NULL),
        ((A16, None, 64, 256, 2, 128, A16, A16, A16), w4.ERR_UNSUPPORTED),
        ((A16, None, 64, 256, 5, 128, A16, A16, A16), w4.ERR_UNSUPPORTED),
        ((A16, None, 64, 256, 4, 16, A16, A16, A16), w4.ERR_UNSUPPORTED),
        ((A16, None, 64, 256, 3, 256, A16, A16, A16), w4.ERR_UNSUPPORTED),
        ((A16, None, 64, 96, 4, 64, A16, A16, A16), w4.ERR_SHAPE),
        ((A16, None, 64, 48, 3, 32, A16, A16, A16), w4.ERR_SHAPE),
        ((A16, None, 64, 250, 4, 128, A16, A16, A16), w4.ERR_SHAPE),
        ((A16, None, 0, 256, 4, 128, A16, A16, A16), w4.ERR_SHAPE),
        ((A2, None, 64, 256, 4, 128, A16, A16, A16), w4.ERR_ALIGN),
        ((A16, A16 + 4, 64, 256, 4, 128, A16, A16, A16), w4.ERR_ALIGN),
        ((A16, None, 64, 256, 4, 128, A16, A16 + 1, A16), w4.ERR_ALIGN),
    ],
)
def test_quantize_pack_rejects(args, status):
    lib = w4.load()
    assert lib.awq_quantize_pack(*args, None) == status


def test_channel_scale_and_scale_input_reject():
    lib = w4.load()
    assert lib.awq_channel_scale(None, 4, 64, 0.5, A16, None) == w4.ERR_NULL
    assert lib.awq_channel_scale(A16, 0, 64, 0.5, A16, None) == w4.ERR_SHAPE
    assert lib.awq_channel_scale(A16, 4, 64, 1.5, A16, None) == w4.ERR_ARG
    assert lib.awq_channel_scale(A16, 4, 64, float("nan"), A16, None) == w4.ERR_ARG
    assert lib.awq_channel_scale(A16 + 1, 4, 64, 0.5, A16, None) == w4.ERR_ALIGN
    assert lib.awq_scale_input(A16, None, 1, 64, A16, None) == w4.ERR_NULL
    assert lib.awq_scale_input(A16, A16, 1, 0, A16, None) == w4.ERR_SHAPE
    assert lib.awq_scale_input(A16, A16 + 2, 1, 64, A16, None) == w4.ERR_ALIGN


def test_rmsnorm_fold_rejects():
    lib = w4.load()
    assert lib.awq_rmsnorm_fold(None, A16, A16, 2, 64, 1e-5, A16, None) == w4.ERR_NULL
    assert lib.awq_rmsnorm_fold(A16, A16, A16, 2, 64, 1e-5, None, None) == w4.ERR_NULL
    assert lib.awq_rmsnorm_fold(A16, A16, A16, 0, 64, 1e-5, A16, None) == w4.ERR_SHAPE
    assert lib.awq_rmsnorm_fold(A16, A16, A16, 2, 60, 1e-5, A16, None) == w4.ERR_SHAPE
    assert lib.awq_rmsnorm_fold(A16, A16, A16, 2, 64, 0.0, A16, None) == w4.ERR_ARG
    assert lib.awq_rmsnorm_fold(A16, A16, A16, 2, 64, float("inf"), A16, None) == w4.ERR_ARG
    assert lib.awq_rmsnorm_fold(A16 + 2, A16, A16, 2, 64, 1e-5, A16, None) == w4.ERR_ALIGN
    assert lib.awq_rmsnorm_fold(A16, A16 + 1, A16, 2, 64, 1e-5, A16, None) == w4.ERR_ALIGN
    assert lib.awq_rmsnorm_fold(A16, A16, A16 + 2, 2, 64, 1e-5, A16, None) == w4.ERR_ALIGN


def test_alpha_loss_workspace_and_rejects():
    lib = w4.load()
    assert lib.awq_alpha_loss_workspace(512, 4096) == 8 * 32  # 64 x 128 tiles
    assert lib.awq_alpha_loss_workspace(65, 63) == 2
    assert lib.awq_alpha_loss_workspace(0, 64) == -1
    assert lib.awq_alpha_loss_workspace(64, (1 << 24) + 1) == -1
    assert lib.awq_alpha_loss_workspace(1 << 20, 1 << 24) == -1  # more than 2^31 - 1 tiles

    def call(xs=A16, q=A16, sc=A16, z=A16, y=A16, T=100, N=200, K=256, group=128, ws=A16, wl=8, loss=A16):
        return lib.awq_alpha_loss(xs, q, sc, z, y, T, N, K, group, ws, wl, loss, None)

    assert lib.awq_alpha_loss_workspace(100, 200) == 2 * 2
    assert call(xs=None) == w4.ERR_NULL
    assert call(y=None) == w4.ERR_NULL
    assert call(ws=None) == w4.ERR_NULL
    assert call(loss=None) == w4.ERR_NULL
    assert call(group=64) == w4.ERR_UNSUPPORTED
    assert call(T=0) == w4.ERR_SHAPE
    assert call(K=200) == w4.ERR_SHAPE
    assert call(K=131072 + 128) == w4.ERR_SHAPE
    assert call(T=(1 << 20) + 1) == w4.ERR_SHAPE
    assert call(wl=3) == w4.ERR_ARG
    assert call(xs=A16 + 2) == w4.ERR_ALIGN
    assert call(q=A16 + 8) == w4.ERR_ALIGN
    assert call(sc=A16 + 1) == w4.ERR_ALIGN
    assert call(y=A16 + 2) == w4.ERR_ALIGN
    assert call(ws=A16 + 4) == w4.ERR_ALIGN
    assert call(loss=A16 + 4) == w4.ERR_ALIGN


def test_format_variants_reject():
    lib = w4.load()
    # groups other than 32/64/128; K not a multiple of 128
    assert lib.w4a16_linear(A16, A16, A16, A16, 1, 64, 256, 16, A16, None) == w4.ERR_UNSUPPORTED
    assert lib.w4a16_linear(A16, A16, A16, A16, 1, 64, 96, 32, A16, None) == w4.ERR_SHAPE
    # the small-batch path with groups of 32/64: M <= 32, scales and zeros 4-byte aligned
    assert lib.w4a16_linear_path(3, A16, A16, A16, A16, 33, 64, 256, 64, A16, None) == w4.ERR_UNSUPPORTED
    assert lib.w4a16_linear_path(3, A16, A16, A16 + 2, A16, 4, 64, 256, 64, A16, None) == w4.ERR_ALIGN
    assert lib.w4a16_linear_path(3, A16, A16, A16, A16 + 2, 4, 64, 256, 32, A16, None) == w4.ERR_ALIGN
    assert lib.w3a16_linear(A16, A16, A16, A16, 1, 64, 256, 256, A16, None) == w4.ERR_UNSUPPORTED
    assert lib.w3a16_linear(None, A16, A16, A16, 1, 64, 256, 128, A16, None) == w4.ERR_NULL
    assert lib.w3a16_linear(A16, A16, A16, A16, 1, 64, 200, 128, A16, None) == w4.ERR_SHAPE
    assert lib.w3a16_linear(A16 + 8, A16, A16, A16, 1, 64, 256, 128, A16, None) == w4.ERR_ALIGN
    assert lib.w3a16_linear_path(4, A16, A16, A16, A16, 1, 64, 256, 128, A16, None) == w4.ERR_UNSUPPORTED
    assert lib.w3a16_linear_path(3, A16, A16, A16, A16, 33, 64, 256, 128, A16, None) == w4.ERR_UNSUPPORTED
    assert lib.w3a16_linear_path(3, A16, A16, A16 + 2, A16, 4, 64, 256, 64, A16, None) == w4.ERR_ALIGN
    assert lib.w3a16_linear_path(1, A16, A16, A16, A16, 9, 64, 256, 128, A16, None) == w4.ERR_UNSUPPORTED
    assert lib.w3a16_linear_path(1, A16, A16, A16, A16, 8, 64, 32768 + 128, 128, A16, None) == w4.ERR_UNSUPPORTED


def test_nf4_codebook_is_the_oracles_fp16_codebook():
    # the library derives its codebook itself (its own normal quantiles); both must round to
    # the same fp16 levels
    import numpy as np

    import oracle

    assert w4.nf4_codebook() == [int(b) for b in oracle.NF4_LEVELS_F16.view(np.uint16)]


def test_nf4_and_sym_reject():
    lib = w4.load()
    assert lib.nf4_quantize_pack(None, None, 4, 128, 64, A16, A16, None) == w4.ERR_NULL
    assert lib.nf4_quantize_pack(A16, None, 4, 128, 16, A16, A16, None) == w4.ERR_UNSUPPORTED
    assert lib.nf4_quantize_pack(A16, None, 4, 96, 64, A16, A16, None) == w4.ERR_SHAPE
    assert lib.nf4_quantize_pack(A16, None, 4, 128, 64, A16, A16 + 2, None) == w4.ERR_ALIGN
    assert lib.nf4_linear(A16, A16, A16, 1, 64, 256, 48, A16, None) == w4.ERR_UNSUPPORTED
    assert lib.nf4_linear(A16, A16, A16, 1, 64, 192, 64, A16, None) == w4.ERR_SHAPE
    assert lib.nf4_linear(A16, A16, A16 + 2, 1, 64, 256, 64, A16, None) == w4.ERR_ALIGN
    assert lib.nf4_linear_path(4, A16, A16, A16, 1, 64, 256, 64, A16, None) == w4.ERR_UNSUPPORTED
    assert lib.nf4_linear_path(3, A16, A16, A16, 33, 64, 256, 64, A16, None) == w4.ERR_UNSUPPORTED
    assert lib.nf4_linear_path(1, A16, A16, A16, 9, 64, 256, 64, A16, None) == w4.ERR_UNSUPPORTED
    assert lib.awq_quantize_pack_sym(A16, None, 4, 256, 2, 128, A16, A16, A16, None) == w4.ERR_UNSUPPORTED
    assert lib.awq_quantize_pack_sym(A16, None, 4, 200, 4, 128, A16, A16, A16, None) == w4.ERR_SHAPE
    assert lib.awq_quantize_pack_sym(None, None, 4, 256, 4, 128, A16, A16, A16, None) == w4.ERR_NULL


def test_splitk_workspace_and_rejects():
    lib = w4.load()
    assert lib.w4a16_linear_splitk_workspace(128, 4096, 4096, 4) == 4 * 128 * 4096 * 4
    assert lib.w4a16_linear_splitk_workspace(128, 4096, 4096, 0) > 0
    # the default split count (splits = 0): about 512 workgroups of 64 x 128 tiles, rounded up to
    # a power of two, at most 4, and at least four groups per split
    for (m, n, k), s in {(128, 4096, 4096): 4, (128, 11008, 4096): 4, (256, 11008, 4096): 2,
                         (128, 4096, 11008): 4, (4096, 4096, 4096): 1, (128, 4096, 256): 1,
                         (128, 4096, 1024): 2}.items():
        assert lib.w4a16_linear_splitk_workspace(m, n, k, 0) == s * m * n * 4, (m, n, k)
    assert lib.w4a16_linear_splitk_workspace(128, 4096, 256, 3) == -1   # more splits than groups
    assert lib.w4a16_linear_splitk_workspace(128, 4096, 4096, 17) == -1
    assert lib.w4a16_linear_splitk_workspace(0, 4096, 4096, 2) == -1

    def call(group=128, splits=2, ws=A16, wb=1 << 30, M=128, K=4096):
        return lib.w4a16_linear_splitk(A16, A16, A16, A16, M, 4096, K, group, splits, ws, wb, A16, None)

    assert call(group=64) == w4.ERR_UNSUPPORTED
    assert call(ws=None) == w4.ERR_NULL
    assert call(splits=-1) == w4.ERR_ARG
    assert call(splits=17) == w4.ERR_ARG
    assert call(splits=3, K=256) == w4.ERR_ARG
    assert call(wb=100) == w4.ERR_ARG
    assert call(ws=A16 + 8) == w4.ERR_ALIGN
    assert call(K=200) == w4.ERR_SHAPE


def _xres_ranges(m, n, k):
    # K ranges of the x-resident kernel: 256 inputs per wave; with M <= 16 workgroups of 64
    # columns, eight waves where they come to 512 or more (else four); with M > 16 128
    # columns, four waves where eight-wave workgroups would come to 512 or more (else eight)
    g = k // 128
    r8 = -(-g // 16)
    if m <= 16:
        waves = 8 if -(-n // 64) * r8 >= 512 else 4
    else:
        waves = 4 if -(-n // 128) * r8 >= 512 else 8
    return -(-g // (2 * waves))


def test_xres_workspace_and_rejects():
    lib = w4.load()
    # S float32 partials of M x N, none for one range
    assert lib.w4a16_linear_xres_workspace(32, 8192, 8192) == 4 * 32 * 8192 * 4
    assert lib.w4a16_linear_xres_workspace(16, 8192, 8192) == 4 * 16 * 8192 * 4     # 512 workgroups of 8 waves
    assert lib.w4a16_linear_xres_workspace(16, 4096, 11008) == 11 * 16 * 4096 * 4   # 4-wave ranges of 1024
    assert lib.w4a16_linear_xres_workspace(32, 4096, 2048) == 0
    assert lib.w4a16_linear_xres_workspace(16, 4096, 2048) == 2 * 16 * 4096 * 4
    assert lib.w4a16_linear_xres_workspace(32, 8192, 22016) == 22 * 32 * 8192 * 4   # four-wave ranges of 1024
    assert lib.w4a16_linear_xres_workspace(16, 8192, 22016) == 11 * 16 * 8192 * 4
    for m, n, k in [(4, 1024, 8192), (9, 11008, 4096), (24, 28672, 8192), (17, 4096, 4096), (1, 1, 256)]:
        s = _xres_ranges(m, n, k)
        assert lib.w4a16_linear_xres_workspace(m, n, k) == (s * m * n * 4 if s > 1 else 0), (m, n, k)
    assert lib.w4a16_linear_xres_workspace(33, 4096, 4096) == -1   # M > 32
    assert lib.w4a16_linear_xres_workspace(8, 4096, 384) == -1     # odd number of groups
    assert lib.w4a16_linear_xres_workspace(0, 4096, 4096) == -1

    def call(group=128, ws=A16, wb=1 << 30, M=32, K=8192, sc=A16):
        return lib.w4a16_linear_xres(A16, A16, sc, A16, M, 4096, K, group, ws, wb, A16, None)

    assert call(group=32) == w4.ERR_UNSUPPORTED   # groups of 128 and 64 only
    assert call(M=33) == w4.ERR_UNSUPPORTED
    assert call(K=384) == w4.ERR_UNSUPPORTED
    assert call(ws=None) == w4.ERR_NULL
    assert call(wb=100) == w4.ERR_ARG
    assert call(ws=A16 + 8) == w4.ERR_ALIGN
    assert call(sc=A16 + 2) == w4.ERR_ALIGN
    assert call(K=200) == w4.ERR_SHAPE


def test_linear_ws_split_choice_and_rejects():
    lib = w4.load()
    # the automatic path's split choice with a workspace (4-bit, groups of 128): no split at
    # M <= 16 and below K = 4096; for K >= 8192 none up to M = 32 on rows of at most 16384
    # where ceil(N / 32) is a multiple of 256, else the largest S of 8, 4, 2 with
    # S * tiles < 1024 (<= 256 on up to 64 tiles; tiles are 32 x 128 up to M = 32, else
    # 64 x 128) and >= 8 groups per range, none where only one range would be left (the
    # automatic path without a workspace takes those); for 4096 <= K < 8192 from M = 21, two
    # ranges on 65..128 tiles / four on <= 48 at M > 32
    cases = {(1, 8192, 8192): 0, (16, 4096, 11008): 0, (20, 4096, 11008): 8, (32, 8192, 8192): 0, (24, 8192, 8192): 0,
             (20, 11008, 4096): 0, (17, 8192, 22016): 4, (32, 16384, 8192): 0,
             (32, 4096, 11008): 8, (32, 8192, 22016): 4, (24, 22016, 8192): 4, (32, 11008, 4096): 2,
             (32, 4096, 4096): 0,
             (64, 4096, 11008): 8, (128, 4096, 11008): 4, (256, 4096, 11008): 4, (512, 4096, 11008): 2,
             (128, 8192, 8192): 4, (64, 8192, 8192): 4, (48, 8192, 8192): 4, (256, 8192, 8192): 2, (512, 8192, 8192): 0, (512, 8192, 22016): 0,
             (192, 22016, 8192): 0, (128, 22016, 8192): 2, (64, 1024, 8192): 8,
             (256, 4096, 4096): 2, (192, 4096, 4096): 2, (128, 4096, 4096): 0, (64, 4096, 4096): 4,
             (48, 11008, 4096): 2, (128, 11008, 4096): 0, (64, 8192, 1024): 0, (64, 64, 2048): 0}
    # the x-resident kernel (K > 2048, an even number of groups; M = 4..16: N K >= 2^27, or
    # M >= 8 with N K >= 2^25 and N > K, or M >= 8 with ceil(N / 32) <= 64 and K >= 8192, or
    # M >= 12 with N K >= 2^25; M = 17..32, with W = ceil(N / 128) ceil(K / 2048): W >= 160); the
    # workspace covers both kernels' needs
    xres = {(4, 8192, 22016), (8, 8192, 22016), (8, 11008, 4096), (8, 28672, 8192), (12, 8192, 8192),
            (12, 11008, 4096), (16, 4096, 11008), (16, 8192, 8192), (17, 8192, 22016), (20, 11008, 4096),
            (24, 8192, 8192), (24, 22016, 8192), (32, 8192, 8192), (32, 8192, 22016), (32, 11008, 4096),
            (32, 16384, 8192), (20, 4096, 11008), (32, 4096, 11008)}
    for extra in ((12, 11008, 4096), (12, 8192, 8192), (16, 8192, 8192), (8, 8192, 22016), (8, 28672, 8192),
                  (4, 8192, 22016), (8, 11008, 4096)):
        cases[extra] = 0
    for (m, n, k), s in cases.items():
        assert lib.w4a16_linear_ws_splits(m, n, k, 128) == s, (m, n, k)
        want_x = (m, n, k) in xres
        assert lib.w4a16_linear_ws_kernel(m, n, k, 128) == (2 if want_x else 1 if s else 0), (m, n, k)
        xf = _xres_ranges(m, n, k) * m * n if want_x else 0
        assert lib.w4a16_linear_workspace(m, n, k, 128) == max(s * m * n, xf) * 4, (m, n, k)
        # groups of 64: the x-resident kernel on the same shapes, else w4a16_linear's kernels
        assert lib.w4a16_linear_ws_kernel(m, n, k, 64) == (2 if want_x else 0), (m, n, k)
        assert lib.w4a16_linear_workspace(m, n, k, 64) == xf * 4, (m, n, k)
        assert lib.w4a16_linear_ws_splits(m, n, k, 64) == 0, (m, n, k)
    assert lib.w4a16_linear_ws_kernel(32, 8192, 8192, 32) == 0
    assert lib.w4a16_linear_ws_kernel(32, 8192, 8320, 64) == 0    # odd number of 128-input blocks
    assert lib.w4a16_linear_ws_kernel(32, 8192, 8320, 128) == 0   # odd number of groups
    assert lib.w4a16_linear_ws_kernel(16, 20480, 2048, 128) == 0  # one K range: not on this path
    assert lib.w4a16_linear_ws_splits(256, 4096, 11008, 64) == 0   # split-K takes groups of 128 only
    assert lib.w4a16_linear_workspace(256, 4096, 11008, 32) == 0
    assert lib.w4a16_linear_workspace(0, 4096, 4096, 128) == -1
    assert lib.w4a16_linear_workspace(64, 4096, 200, 128) == -1
    assert lib.w4a16_linear_ws_splits(64, 4096, 4096, 16) == -1

    def call(ws=A16, wb=1 << 30, M=128, N=4096, K=11008, group=128, x=A16):
        return lib.w4a16_linear_ws(x, A16, A16, A16, M, N, K, group, ws, wb, A16, None)

    assert call(x=None) == w4.ERR_NULL
    assert call(K=200) == w4.ERR_SHAPE
    assert call(group=16) == w4.ERR_UNSUPPORTED
    assert call(wb=100) == w4.ERR_ARG                          # too small for the 4 ranges chosen
    assert call(ws=A16 + 8) == w4.ERR_ALIGN
    assert lib.w4a16_last_error() != b""


def test_output_reference_rejects():
    lib = w4.load()
    assert lib.awq_output_reference(None, A16, 4, 4, 128, A16, None) == w4.ERR_NULL
    assert lib.awq_output_reference(A16, A16, 4, 4, 128, None, None) == w4.ERR_NULL
    assert lib.awq_output_reference(A16, A16, 0, 4, 128, A16, None) == w4.ERR_SHAPE
    assert lib.awq_output_reference(A16, A16, 4, 4, 100, A16, None) == w4.ERR_SHAPE
    assert lib.awq_output_reference(A16, A16, 4, (1 << 24) + 1, 128, A16, None) == w4.ERR_SHAPE
    assert lib.awq_output_reference(A16 + 8, A16, 4, 4, 128, A16, None) == w4.ERR_ALIGN
    assert lib.awq_output_reference(A16, A16, 4, 4, 128, A16 + 2, None) == w4.ERR_ALIGN


def test_binding_refuses_cpu_tensors():
    import torch

    with pytest.raises(ValueError):
        w4.linear(torch.zeros(1, 256, dtype=torch.float16), torch.zeros(64, 32, dtype=torch.int32),
                  torch.zeros(64, 2, dtype=torch.float16), torch.zeros(64, 2, dtype=torch.float16))


def test_library_links_no_oracle_and_no_torch():
    out = subprocess.run(["ldd", w4.LIB_PATH], capture_output=True, text=True).stdout
    assert "torch" not in out and "python" not in out
    assert ctypes.CDLL(w4.LIB_PATH) is not None


def test_stream_read_sizes_and_rejects():
    lib = w4.load()
    vp = ctypes.c_void_p
    # one word per workgroup: W = max(min(1024, ceil(P/256)), ceil(P/4096)) workgroups of
    # ceil(P/W) pieces, P = bytes/16
    assert lib.w4a16_stream_read_sink_bytes(32768) == 4 * 8
    assert lib.w4a16_stream_read_sink_bytes(32768 + 16) == 4 * 9
    assert lib.w4a16_stream_read_sink_bytes(16) == 4
    assert lib.w4a16_stream_read_sink_bytes(35684352) == 4 * 1024  # the headline layer's bytes, 2178 pieces each
    assert lib.w4a16_stream_read_sink_bytes(1 << 30) == 4 * 16384  # 4096 pieces per workgroup at most
    assert lib.w4a16_stream_read_sink_bytes(0) == -1
    assert lib.w4a16_stream_read_sink_bytes(24) == -1
    buf, sink = vp(1 << 20), vp(1 << 21)
    assert lib.w4a16_stream_read(None, 4096, sink, None) == w4.ERR_NULL
    assert lib.w4a16_stream_read(buf, 4096, None, None) == w4.ERR_NULL
    assert lib.w4a16_stream_read(buf, 0, sink, None) == w4.ERR_SHAPE
    assert lib.w4a16_stream_read(buf, 4100, sink, None) == w4.ERR_SHAPE
    assert lib.w4a16_stream_read(vp((1 << 20) + 8), 4096, sink, None) == w4.ERR_ALIGN
    assert lib.w4a16_stream_read(buf, 4096, vp((1 << 21) + 2), None) == w4.ERR_ALIGN


def test_stream_read_grid_rejects():
    lib = w4.load()
    vp = ctypes.c_void_p
    buf, sink = vp(1 << 20), vp(1 << 21)
    assert lib.w4a16_stream_read_grid(None, 4096, 256, 8, 4, sink, None) == w4.ERR_NULL
    assert lib.w4a16_stream_read_grid(buf, 4096, 256, 8, 4, None, None) == w4.ERR_NULL
    assert lib.w4a16_stream_read_grid(buf, 0, 256, 8, 4, sink, None) == w4.ERR_SHAPE
    assert lib.w4a16_stream_read_grid(buf, 4100, 256, 8, 4, sink, None) == w4.ERR_SHAPE
    for threads, blocks, unroll in ((32, 8, 4), (384, 8, 4), (2048, 8, 4), (256, 0, 4), (256, (1 << 20) + 1, 4),
                                    (256, 8, 3), (256, 8, 32), (256, 8, 0)):
        assert lib.w4a16_stream_read_grid(buf, 4096, threads, blocks, unroll, sink, None) == w4.ERR_ARG
    assert lib.w4a16_stream_read_grid(vp((1 << 20) + 8), 4096, 256, 8, 4, sink, None) == w4.ERR_ALIGN
    assert lib.w4a16_stream_read_grid(buf, 4096, 256, 8, 4, vp((1 << 21) + 2), None) == w4.ERR_ALIGN


def test_splitk_noalloc_rejects_before_any_hip_call():
    lib = w4.load()

    def call(group=128, splits=2, M=128, N=4096, K=4096, x=A16):
        return lib.w4a16_linear_splitk_noalloc(x, A16, A16, A16, M, N, K, group, splits, A16, None)

    assert call(x=None) == w4.ERR_NULL
    assert call(group=64) == w4.ERR_UNSUPPORTED
    assert call(splits=-1) == w4.ERR_ARG
    assert call(splits=17) == w4.ERR_ARG
    assert call(splits=3, K=256) == w4.ERR_ARG
    assert call(K=200) == w4.ERR_SHAPE
    # the library's scratch holds 2^23 float partials: splits * M * N beyond that is refused
    assert call(M=256, N=11008, splits=4) == w4.ERR_SHAPE
    assert call(M=2049, N=4096, splits=1) == w4.ERR_SHAPE  # 2048 x 4096 x 1 = 2^23 fits exactly


def test_search_alpha_workspace_and_rejects():
    lib = w4.load()
    vp = ctypes.c_void_p
    need = lib.awq_search_alpha_workspace(512, 4096, 4096)
    # y_ref, 21 scales, x_s, codes, scales, zeros, loss partials; each region 256-byte aligned
    parts = lib.awq_alpha_loss_workspace(512, 4096)
    r = lambda b: (b + 255) // 256 * 256  # noqa: E731
    assert need == (r(512 * 4096 * 4) + r(21 * 4096 * 4) + r(512 * 4096 * 2) + r(4096 * 4096 // 2)
                    + 2 * r(4096 * 32 * 2) + r(parts * 8))
    assert lib.awq_search_alpha_workspace(0, 4096, 4096) == -1
    assert lib.awq_search_alpha_workspace(512, 4096, 4100) == -1
    assert lib.awq_search_alpha_workspace(65537, 64, 128) == -1
    ws, out = vp(1 << 20), vp(1 << 22)

    def call(x=A16, w=A16, T=512, N=4096, K=4096, ws=ws, wb=need, losses=out, best=out, alpha=out):
        return lib.awq_search_alpha(x, w, T, N, K, ws, wb, losses, best, alpha, None, None)

    assert call(x=None) == w4.ERR_NULL
    assert call(ws=None) == w4.ERR_NULL
    assert call(best=None) == w4.ERR_NULL
    assert call(K=200) == w4.ERR_SHAPE
    assert call(T=0) == w4.ERR_SHAPE
    assert call(wb=need - 1) == w4.ERR_ARG
    assert call(ws=vp((1 << 20) + 128)) == w4.ERR_ALIGN
    assert call(losses=vp((1 << 22) + 4)) == w4.ERR_ALIGN
