"""MI355X (gfx950) W4A16 group-quantized linear layers - Python binding.

A thin ctypes layer over ``libw4a16.so`` (C ABI in ``include/w4a16.h``): it
checks dtypes/devices, allocates outputs with torch on the input's device and
passes raw device pointers plus torch's current HIP stream. Every step of the
computation runs in the library's HIP kernels; there is no fallback. If the
library is missing, every call raises.

    s   = channel_scale(x_cal, alpha=0.5)          # AWQ statistic, float32 [K]
    x_s = scale_input(x, s)                         # the 1/s fold, fp16 [M][K]
    qweight, scales, zeros = quantize_pack(W, s)    # RTN 4-bit, group 128
    y   = linear(x_s, qweight, scales, zeros)       # fused dequant GEMV/GEMM
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw4a16.so")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_HIP, ERR_ARG = range(7)
PATH_AUTO, PATH_GEMV, PATH_MFMA, PATH_SKINNY, PATH_KLANE, PATH_ONE_RANGE = 0, 1, 2, 3, 4, 5
GROUP = 128
LAYOUT_VERSION = 1

_lib = None


class W4A16Error(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


def load():
    """Load the built library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m w4a16_decode_gemv_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    sig = {
        "w4a16_layout_version": ([], i32),
        "w4a16_status_str": ([i32], ctypes.c_char_p),
        "w4a16_last_error": ([], ctypes.c_char_p),
        "w4a16_gemv_max_m": ([], i32),
        "awq_channel_scale": ([vp, i64, i64, ctypes.c_double, vp, vp], i32),
        "awq_scale_input": ([vp, vp, i64, i64, vp, vp], i32),
        "awq_rmsnorm_fold": ([vp, vp, vp, i64, i64, ctypes.c_double, vp, vp], i32),
        "awq_quantize_pack": ([vp, vp, i64, i64, i32, i32, vp, vp, vp, vp], i32),
        "w4a16_linear": ([vp, vp, vp, vp, i64, i64, i64, i32, vp, vp], i32),
        "w4a16_linear_path": ([i32, vp, vp, vp, vp, i64, i64, i64, i32, vp, vp], i32),
        "w4a16_linear_workspace": ([i64, i64, i64, i32], i64),
        "w4a16_linear_ws_splits": ([i64, i64, i64, i32], i32),
        "w4a16_linear_ws_kernel": ([i64, i64, i64, i32], i32),
        "w4a16_linear_ws": ([vp, vp, vp, vp, i64, i64, i64, i32, vp, i64, vp, vp], i32),
        "awq_alpha_loss_workspace": ([i64, i64], i64),
        "w4a16_linear_splitk_workspace": ([i64, i64, i64, i32], i64),
        "w4a16_linear_splitk": ([vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, i64, vp, vp], i32),
        "w4a16_linear_splitk_noalloc": ([vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, vp], i32),
        "w4a16_linear_xres_workspace": ([i64, i64, i64], i64),
        "w4a16_linear_xres": ([vp, vp, vp, vp, i64, i64, i64, i32, vp, i64, vp, vp], i32),
        "w3a16_linear": ([vp, vp, vp, vp, i64, i64, i64, i32, vp, vp], i32),
        "w3a16_linear_path": ([i32, vp, vp, vp, vp, i64, i64, i64, i32, vp, vp], i32),
        "awq_quantize_pack_sym": ([vp, vp, i64, i64, i32, i32, vp, vp, vp, vp], i32),
        "nf4_codebook": ([vp], None),
        "nf4_quantize_pack": ([vp, vp, i64, i64, i32, vp, vp, vp], i32),
        "nf4_linear": ([vp, vp, vp, i64, i64, i64, i32, vp, vp], i32),
        "nf4_linear_path": ([i32, vp, vp, vp, i64, i64, i64, i32, vp, vp], i32),
        "awq_output_reference": ([vp, vp, i64, i64, i64, vp, vp], i32),
        "awq_alpha_loss": ([vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, i64, vp, vp], i32),
        "w4a16_stream_read_sink_bytes": ([i64], i64),
        "w4a16_stream_read": ([vp, i64, vp, vp], i32),
        "w4a16_stream_read_grid": ([vp, i64, i32, i32, i32, vp, vp], i32),
        "awq_search_alpha_workspace": ([i64, i64, i64], i64),
        "awq_search_alpha": ([vp, vp, i64, i64, i64, vp, i64, vp, vp, vp, vp, vp], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def exported_symbols():
    return ["w4a16_layout_version", "w4a16_status_str", "w4a16_last_error", "w4a16_gemv_max_m",
            "awq_channel_scale", "awq_scale_input", "awq_rmsnorm_fold", "awq_quantize_pack", "w4a16_linear",
            "w4a16_linear_path", "w4a16_linear_workspace", "w4a16_linear_ws_splits", "w4a16_linear_ws_kernel",
            "w4a16_linear_ws",
            "w4a16_linear_splitk_workspace", "w4a16_linear_splitk", "w4a16_linear_splitk_noalloc", "w4a16_linear_xres_workspace", "w4a16_linear_xres",
            "w3a16_linear", "w3a16_linear_path", "awq_quantize_pack_sym", "nf4_codebook", "nf4_quantize_pack", "nf4_linear", "nf4_linear_path", "awq_alpha_loss_workspace", "awq_output_reference",
            "awq_alpha_loss", "w4a16_stream_read_sink_bytes", "w4a16_stream_read", "w4a16_stream_read_grid",
            "awq_search_alpha_workspace", "awq_search_alpha"]


def _check(status):
    if status != OK:
        lib = load()
        raise W4A16Error(status, f"{lib.w4a16_status_str(status).decode()}: {lib.w4a16_last_error().decode()}")


def _torch():
    import torch

    return torch


def _dev_tensor(t, dtype, name, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got {t.dim()})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _out(out, shape, dtype, like, name="out"):
    """A new output tensor, or the caller's, checked: a contiguous GPU tensor of this dtype
    and shape on the device of `like` (the kernels write through its pointer)."""
    torch = _torch()
    shape = tuple(int(d) for d in shape)
    if out is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    out = _dev_tensor(out, dtype, name, len(shape))
    if tuple(out.shape) != shape:
        raise ValueError(f"{name} must have shape {shape} (got {tuple(out.shape)})")
    if out.device != like.device:
        raise ValueError(f"{name} must be on {like.device} (got {out.device})")
    return out


def _workspace(ws, dtype, like):
    """A caller's workspace: a contiguous GPU tensor of this dtype on the device of `like`
    (its size is checked by the library)."""
    torch = _torch()
    if not isinstance(ws, torch.Tensor) or ws.device != like.device or ws.dtype != dtype or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous {dtype} tensor on {like.device}")
    return ws


def _outs(out, count, name):
    if out is None:
        return (None,) * count
    out = tuple(out)
    if len(out) != count:
        raise ValueError(f"{name} out must hold {count} tensors")
    return out


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def channel_scale(x_cal, alpha=0.5, out=None):
    """AWQ statistic s[k] = (mean_t |x_cal[t, k]|) ** alpha (float32 [K])."""
    torch = _torch()
    lib = load()
    x_cal = _dev_tensor(x_cal, torch.float16, "x_cal", 2)
    t_, k = x_cal.shape
    s = _out(out, (k,), torch.float32, x_cal)
    _check(lib.awq_channel_scale(x_cal.data_ptr(), t_, k, float(alpha), s.data_ptr(), _stream(x_cal)))
    return s


def scale_input(x, s, out=None):
    """The 1/s fold: x_s = f16(x / s) (fp16 [M][K])."""
    torch = _torch()
    lib = load()
    x = _dev_tensor(x, torch.float16, "x", 2)
    s = _dev_tensor(s, torch.float32, "s", 1)
    m, k = x.shape
    if s.shape[0] != k:
        raise ValueError("s must have K entries")
    xs = _out(out, (m, k), torch.float16, x)
    _check(lib.awq_scale_input(x.data_ptr(), s.data_ptr(), m, k, xs.data_ptr(), _stream(x)))
    return xs


def rmsnorm_fold(h, gamma, s=None, eps=1e-5, out=None):
    """RMSNorm of h with the 1/s folded in: x_s = f16(((h * r) * gamma) / s), fp16 [M][K]."""
    torch = _torch()
    lib = load()
    h = _dev_tensor(h, torch.float16, "h", 2)
    gamma = _dev_tensor(gamma, torch.float16, "gamma", 1)
    m, k = h.shape
    if gamma.shape[0] != k:
        raise ValueError("gamma must have K entries")
    sp = 0
    if s is not None:
        s = _dev_tensor(s, torch.float32, "s", 1)
        if s.shape[0] != k:
            raise ValueError("s must have K entries")
        sp = s.data_ptr()
    xs = _out(out, (m, k), torch.float16, h)
    _check(lib.awq_rmsnorm_fold(h.data_ptr(), gamma.data_ptr(), sp, m, k, float(eps), xs.data_ptr(), _stream(h)))
    return xs


def quantize_pack(W, s=None, bits=4, group=GROUP, out=None):
    """RTN zero-point quantize + pack of an nn.Linear weight fp16 [N][K].

    Returns (qweight int32 [N][K/8] holding layout-v1 uint32 words,
    scales fp16 [N][K/128], zeros fp16 [N][K/128]).
    """
    torch = _torch()
    lib = load()
    W = _dev_tensor(W, torch.float16, "W", 2)
    n, k = W.shape
    sp = None
    if s is not None:
        s = _dev_tensor(s, torch.float32, "s", 1)
        if s.shape[0] != k:
            raise ValueError("s must have K entries")
        sp = s.data_ptr()
    g = max(k // group, 1)
    words = k // 8 if bits == 4 else 3 * (k // 32)
    o = _outs(out, 3, "quantize_pack")
    qweight = _out(o[0], (n, max(words, 1)), torch.int32, W, "qweight")
    scales = _out(o[1], (n, g), torch.float16, W, "scales")
    zeros = _out(o[2], (n, g), torch.float16, W, "zeros")
    _check(lib.awq_quantize_pack(W.data_ptr(), sp, n, k, bits, group, qweight.data_ptr(), scales.data_ptr(),
                                 zeros.data_ptr(), _stream(W)))
    return qweight, scales, zeros


def splitk_workspace_bytes(M, N, K, splits=0):
    n = int(load().w4a16_linear_splitk_workspace(int(M), int(N), int(K), int(splits)))
    if n < 0:
        raise ValueError(f"shape M={M} N={N} K={K} with splits={splits} is not accepted by the split-K kernel")
    return n


def linear_workspace_bytes(M, N, K, group=GROUP):
    """Bytes of float32 workspace the automatic 4-bit path may use (0: none)."""
    n = int(load().w4a16_linear_workspace(int(M), int(N), int(K), int(group)))
    if n < 0:
        raise ValueError(f"M={M}, N={N}, K={K}, group={group} outside the limits of the linear call")
    return n


def linear_ws_splits(M, N, K, group=GROUP):
    """The K ranges the automatic 4-bit path splits this shape into when given its workspace (0: none)."""
    n = int(load().w4a16_linear_ws_splits(int(M), int(N), int(K), int(group)))
    if n < 0:
        raise ValueError(f"M={M}, N={N}, K={K}, group={group} outside the limits of the linear call")
    return n


def linear_ws_kernel(M, N, K, group=GROUP):
    """The kernel the automatic 4-bit path runs when given its workspace: 0 the no-workspace
    choice, 1 split-K, 2 the x-resident kernel."""
    n = int(load().w4a16_linear_ws_kernel(int(M), int(N), int(K), int(group)))
    if n < 0:
        raise ValueError(f"M={M}, N={N}, K={K}, group={group} outside the limits of the linear call")
    return n


def linear_splitk(x, qweight, scales, zeros, splits=0, workspace=None, out=None, group=GROUP):
    """``linear`` (4-bit, groups of 128) on the split-K MFMA kernel; workspace: a float32 device
    tensor of at least splitk_workspace_bytes(M, N, K, splits) bytes (allocated when omitted)."""
    torch = _torch()
    lib = load()
    x = _dev_tensor(x, torch.float16, "x", 2)
    qweight = _dev_tensor(qweight, torch.int32, "qweight", 2)
    scales = _dev_tensor(scales, torch.float16, "scales", 2)
    zeros = _dev_tensor(zeros, torch.float16, "zeros", 2)
    m, k = x.shape
    n = qweight.shape[0]
    if qweight.shape[1] * 8 != k or scales.shape != zeros.shape or tuple(scales.shape) != (n, k // group):
        raise ValueError("qweight must be [N][K/8] and scales/zeros [N][K/group]")
    if workspace is None:
        workspace = torch.empty(splitk_workspace_bytes(m, n, k, splits) // 4, dtype=torch.float32, device=x.device)
    workspace = _workspace(workspace, torch.float32, x)
    y = _out(out, (m, n), torch.float16, x)
    _check(lib.w4a16_linear_splitk(x.data_ptr(), qweight.data_ptr(), scales.data_ptr(), zeros.data_ptr(), m, n, k,
                                   group, splits, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   y.data_ptr(), _stream(x)))
    return y


def linear_splitk_noalloc(x, qweight, scales, zeros, out, splits=0, group=GROUP):
    """``linear_splitk`` with the partials in the library's own static scratch: the call
    allocates nothing (`out`, the fp16 [M][N] result, is the caller's). Calls that overlap
    on one GPU share that scratch and race."""
    torch = _torch()
    lib = load()
    x = _dev_tensor(x, torch.float16, "x", 2)
    qweight = _dev_tensor(qweight, torch.int32, "qweight", 2)
    scales = _dev_tensor(scales, torch.float16, "scales", 2)
    zeros = _dev_tensor(zeros, torch.float16, "zeros", 2)
    m, k = x.shape
    n = qweight.shape[0]
    if qweight.shape[1] * 8 != k or scales.shape != zeros.shape or tuple(scales.shape) != (n, k // group):
        raise ValueError("qweight must be [N][K/8] and scales/zeros [N][K/group]")
    if out is None:
        raise ValueError("out is required: this call allocates nothing")
    y = _out(out, (m, n), torch.float16, x)
    _check(lib.w4a16_linear_splitk_noalloc(x.data_ptr(), qweight.data_ptr(), scales.data_ptr(), zeros.data_ptr(), m,
                                           n, k, group, splits, y.data_ptr(), _stream(x)))
    return y


def xres_workspace_bytes(M, N, K):
    n = int(load().w4a16_linear_xres_workspace(int(M), int(N), int(K)))
    if n < 0:
        raise ValueError(f"shape M={M} N={N} K={K} is not accepted by the x-resident kernel")
    return n


def linear_xres(x, qweight, scales, zeros, workspace=None, out=None, group=GROUP):
    """``linear`` (4-bit, groups of 128 or 64, M <= 32) on the x-resident MFMA kernel; workspace: a
    float32 device tensor of at least xres_workspace_bytes(M, N, K) bytes (allocated when
    omitted and needed)."""
    torch = _torch()
    lib = load()
    x = _dev_tensor(x, torch.float16, "x", 2)
    qweight = _dev_tensor(qweight, torch.int32, "qweight", 2)
    scales = _dev_tensor(scales, torch.float16, "scales", 2)
    zeros = _dev_tensor(zeros, torch.float16, "zeros", 2)
    m, k = x.shape
    n = qweight.shape[0]
    if qweight.shape[1] * 8 != k or scales.shape != zeros.shape or tuple(scales.shape) != (n, k // group):
        raise ValueError("qweight must be [N][K/8] and scales/zeros [N][K/group]")
    need = xres_workspace_bytes(m, n, k)
    wp, wbytes = None, 0
    if workspace is None and need > 0:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=x.device)
    if workspace is not None:
        workspace = _workspace(workspace, torch.float32, x)
        wp, wbytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    y = _out(out, (m, n), torch.float16, x)
    _check(lib.w4a16_linear_xres(x.data_ptr(), qweight.data_ptr(), scales.data_ptr(), zeros.data_ptr(), m, n, k,
                                 group, wp, wbytes, y.data_ptr(), _stream(x)))
    return y


def quantize_pack_sym(W, s=None, bits=4, group=GROUP, out=None):
    """Symmetric absmax quantize-pack: codes q + 2^(b-1) in the packed layouts, fp16 scales,
    zeros 2^(b-1) (so ``linear`` computes with them unchanged)."""
    torch = _torch()
    lib = load()
    W = _dev_tensor(W, torch.float16, "W", 2)
    n, k = W.shape
    sp = None
    if s is not None:
        s = _dev_tensor(s, torch.float32, "s", 1)
        if s.shape[0] != k:
            raise ValueError("s must have K entries")
        sp = s.data_ptr()
    words = k // 8 if bits == 4 else 3 * (k // 32)
    o = _outs(out, 3, "quantize_pack_sym")
    qweight = _out(o[0], (n, max(words, 1)), torch.int32, W, "qweight")
    scales = _out(o[1], (n, max(k // group, 1)), torch.float16, W, "scales")
    zeros = _out(o[2], (n, max(k // group, 1)), torch.float16, W, "zeros")
    _check(lib.awq_quantize_pack_sym(W.data_ptr(), sp, n, k, bits, group, qweight.data_ptr(), scales.data_ptr(),
                                     zeros.data_ptr(), _stream(W)))
    return qweight, scales, zeros


NF4_BLOCK = 64


def nf4_codebook():
    """The library's 16 fp16 NF4 levels (bit patterns, ascending), as a list of ints."""
    buf = (ctypes.c_uint16 * 16)()
    load().nf4_codebook(buf)
    return list(buf)


def nf4_quantize_pack(W, s=None, block=NF4_BLOCK, out=None):
    """NF4 quantize-pack: (qweight int32 [N][K/8] in layout v1, absmax float32 [N][K/block])."""
    torch = _torch()
    lib = load()
    W = _dev_tensor(W, torch.float16, "W", 2)
    n, k = W.shape
    sp = None
    if s is not None:
        s = _dev_tensor(s, torch.float32, "s", 1)
        if s.shape[0] != k:
            raise ValueError("s must have K entries")
        sp = s.data_ptr()
    o = _outs(out, 2, "nf4_quantize_pack")
    qweight = _out(o[0], (n, max(k // 8, 1)), torch.int32, W, "qweight")
    absmax = _out(o[1], (n, max(k // block, 1)), torch.float32, W, "absmax")
    _check(lib.nf4_quantize_pack(W.data_ptr(), sp, n, k, block, qweight.data_ptr(), absmax.data_ptr(), _stream(W)))
    return qweight, absmax


def nf4_linear(x, qweight, absmax, block=NF4_BLOCK, out=None, path=PATH_AUTO):
    """y = x @ (codebook[q] * absmax)^T, fp16 [M][N] (float32 accumulation)."""
    torch = _torch()
    lib = load()
    x = _dev_tensor(x, torch.float16, "x", 2)
    qweight = _dev_tensor(qweight, torch.int32, "qweight", 2)
    absmax = _dev_tensor(absmax, torch.float32, "absmax", 2)
    m, k = x.shape
    n = qweight.shape[0]
    if qweight.shape[1] * 8 != k:
        raise ValueError("qweight must be [N][K/8]")
    if tuple(absmax.shape) != (n, k // block):
        raise ValueError("absmax must be [N][K/block]")
    y = _out(out, (m, n), torch.float16, x)
    _check(lib.nf4_linear_path(path, x.data_ptr(), qweight.data_ptr(), absmax.data_ptr(), m, n, k, block,
                               y.data_ptr(), _stream(x)))
    return y


def linear(x, qweight, scales, zeros, group=GROUP, out=None, path=PATH_AUTO, bits=4, workspace="auto"):
    """y = x @ dequant(qweight, scales, zeros)^T, fp16 [M][N] (float32 accumulation).

    bits 4: qweight in layout v1 [N][K/8]; bits 3: the 3-bit layout [N][3K/32].
    The automatic path (4-bit) runs w4a16_linear_ws: with workspace "auto" a float32 workspace
    is allocated from torch when the library asks for one (it may then take the split-K
    kernels); None runs w4a16_linear (no workspace); a float32 device tensor is used as given."""
    torch = _torch()
    lib = load()
    x = _dev_tensor(x, torch.float16, "x", 2)
    qweight = _dev_tensor(qweight, torch.int32, "qweight", 2)
    scales = _dev_tensor(scales, torch.float16, "scales", 2)
    zeros = _dev_tensor(zeros, torch.float16, "zeros", 2)
    m, k = x.shape
    n = qweight.shape[0]
    if bits not in (3, 4):
        raise ValueError("bits must be 3 or 4")
    if (bits == 4 and qweight.shape[1] * 8 != k) or (bits == 3 and qweight.shape[1] * 32 != 3 * k):
        raise ValueError("qweight must be [N][K/8] (4-bit) or [N][3K/32] (3-bit)")
    if scales.shape != zeros.shape or scales.shape[0] != n or scales.shape[1] * group != k:
        raise ValueError("scales/zeros must be [N][K/group]")
    y = _out(out, (m, n), torch.float16, x)
    args = (x.data_ptr(), qweight.data_ptr(), scales.data_ptr(), zeros.data_ptr(), m, n, k, group, y.data_ptr(),
            _stream(x))
    if bits == 4 and path == PATH_AUTO and workspace is not None:
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError('workspace must be "auto", None or a float32 device tensor')
            need = int(lib.w4a16_linear_workspace(m, n, k, group))
            workspace = torch.empty(need // 4, dtype=torch.float32, device=x.device) if need > 0 else None
        else:
            workspace = _workspace(workspace, torch.float32, x)
        wp, wb = (0, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * 4)
        status = lib.w4a16_linear_ws(*args[:8], wp or None, wb, *args[8:])
    elif bits == 4:
        status = lib.w4a16_linear(*args) if path == PATH_AUTO else lib.w4a16_linear_path(path, *args)
    else:
        status = lib.w3a16_linear(*args) if path == PATH_AUTO else lib.w3a16_linear_path(path, *args)
    _check(status)
    return y


def alpha_loss_workspace(T, N):
    """Number of float64 values the loss call needs as workspace for T rows and N outputs."""
    n = int(load().awq_alpha_loss_workspace(int(T), int(N)))
    if n < 0:
        raise ValueError(f"T={T}, N={N} outside the limits of the loss call")
    return n


def output_reference(x, W, out=None):
    """The original layer's output on the calibration activations, float32 [T][N]: x @ W^T."""
    torch = _torch()
    lib = load()
    x = _dev_tensor(x, torch.float16, "x", 2)
    W = _dev_tensor(W, torch.float16, "W", 2)
    t_, k = x.shape
    n = W.shape[0]
    if W.shape[1] != k:
        raise ValueError("x must be [T][K] and W [N][K]")
    y = _out(out, (t_, n), torch.float32, x)
    _check(lib.awq_output_reference(x.data_ptr(), W.data_ptr(), t_, n, k, y.data_ptr(), _stream(x)))
    return y


def alpha_loss(x_s, qweight, scales, zeros, y_ref, group=GROUP, workspace=None, out=None):
    """Output-error loss of one candidate scale, float64 [1] on the device:
    sum_{t,n} (x_s @ w_hat^T - y_ref)^2 with w_hat the dequantized (qweight, scales, zeros)."""
    torch = _torch()
    lib = load()
    x_s = _dev_tensor(x_s, torch.float16, "x_s", 2)
    qweight = _dev_tensor(qweight, torch.int32, "qweight", 2)
    scales = _dev_tensor(scales, torch.float16, "scales", 2)
    zeros = _dev_tensor(zeros, torch.float16, "zeros", 2)
    y_ref = _dev_tensor(y_ref, torch.float32, "y_ref", 2)
    t_, k = x_s.shape
    n = qweight.shape[0]
    if tuple(qweight.shape) != (n, k // 8) or scales.shape != zeros.shape or tuple(scales.shape) != (n, k // group):
        raise ValueError("qweight must be [N][K/8] and scales/zeros [N][K/group]")
    if tuple(y_ref.shape) != (t_, n):
        raise ValueError("y_ref must be [T][N]")
    if workspace is None:
        workspace = torch.empty(alpha_loss_workspace(t_, n), dtype=torch.float64, device=x_s.device)
    workspace = _workspace(workspace, torch.float64, x_s)
    loss = _out(out, (1,), torch.float64, x_s)
    _check(lib.awq_alpha_loss(x_s.data_ptr(), qweight.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                              y_ref.data_ptr(), t_, n, k, group, workspace.data_ptr(), workspace.numel(),
                              loss.data_ptr(), _stream(x_s)))
    return loss


ALPHA_GRID_POINTS = 21


def search_alpha_workspace(t_, n, k):
    """Bytes of device workspace that search_alpha needs for T calibration rows, N outputs,
    K inputs."""
    nbytes = int(load().awq_search_alpha_workspace(int(t_), int(n), int(k)))
    if nbytes < 0:
        raise ValueError(f"T={t_}, N={n}, K={k} outside the limits of the search")
    return nbytes


def search_alpha(x_cal, W, workspace=None, out=None):
    """The AWQ grid search on the device (awq_search_alpha): the original output once, then
    for every alpha = i/20 the channel scale, the 1/s fold, the quantize-pack and the
    output-error loss, then the choice (first minimum). Returns device tensors
    (losses float64 [21], best int32 [1], alpha float64 [1], s float32 [K]); nothing is read
    back to the host. out: optional (losses, best, alpha, s) tensors to fill."""
    torch = _torch()
    lib = load()
    x_cal = _dev_tensor(x_cal, torch.float16, "x_cal", 2)
    W = _dev_tensor(W, torch.float16, "W", 2)
    t_, k = x_cal.shape
    n = W.shape[0]
    if W.shape[1] != k:
        raise ValueError("x_cal must be [T][K] and W [N][K]")
    need = search_alpha_workspace(t_, n, k)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x_cal.device)
    workspace = _workspace(workspace, torch.uint8, x_cal)
    o = _outs(out, 4, "search")
    losses = _out(o[0], (ALPHA_GRID_POINTS,), torch.float64, x_cal, "losses")
    best = _out(o[1], (1,), torch.int32, x_cal, "best")
    alpha = _out(o[2], (1,), torch.float64, x_cal, "alpha")
    s = _out(o[3], (k,), torch.float32, x_cal, "s")
    _check(lib.awq_search_alpha(x_cal.data_ptr(), W.data_ptr(), t_, n, k, workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), losses.data_ptr(), best.data_ptr(),
                                alpha.data_ptr(), s.data_ptr(), _stream(x_cal)))
    return losses, best, alpha, s


STREAM_READ_MAGIC = 0x5EAD5EAD


def stream_read(buf, sink=None):
    """Measurement aid: one launch that reads `buf` once with the GEMV's access pattern.
    buf: any contiguous GPU tensor whose size is a multiple of 16 bytes. Returns the sink
    (int32, one word per workgroup; a word is set to STREAM_READ_MAGIC only where a
    thread's XOR of its words equals it)."""
    torch = _torch()
    lib = load()
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    nbytes = buf.numel() * buf.element_size()
    words = int(lib.w4a16_stream_read_sink_bytes(nbytes))
    if words < 0:
        raise ValueError("buf must hold a positive multiple of 16 bytes")
    sink = _out(sink, (words // 4,), torch.int32, buf, "sink")
    _check(lib.w4a16_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), _stream(buf)))
    return sink


def stream_read_grid(buf, threads=256, blocks=1024, unroll=4, sink=None):
    """Measurement aid: a grid-stride read of `buf` in tiles of threads x unroll 16-byte
    pieces over `blocks` workgroups (a read pattern independent of the GEMV's grid).
    Returns the sink (int32, one word per workgroup, set to STREAM_READ_MAGIC only where
    one thread's XOR of its words over all its tiles equals it)."""
    torch = _torch()
    lib = load()
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    nbytes = buf.numel() * buf.element_size()
    sink = _out(sink, (int(blocks),), torch.int32, buf, "sink")
    _check(lib.w4a16_stream_read_grid(buf.data_ptr(), nbytes, int(threads), int(blocks), int(unroll), sink.data_ptr(),
                                      _stream(buf)))
    return sink


def gemv_max_m():
    return int(load().w4a16_gemv_max_m())
