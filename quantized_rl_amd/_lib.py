"""ctypes binding of libjetfp8.so (argument marshalling only).

Each wrapper takes torch tensors that live on a HIP device, allocates any
missing outputs with torch (the library itself never allocates), and calls
the C entry point of the same name on the current torch stream.  There is no
fallback: if the library is missing or a call fails, an exception is raised.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libjetfp8.so")

_c_p = ctypes.c_void_p
_c_i64 = ctypes.c_int64

SIGNATURES = {
    "quantize_act_1x128": [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p],
    "quantize_weight_128x128": [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p],
    "rmsnorm_quant": [_c_p, _c_p, _c_i64, _c_i64, ctypes.c_float, _c_p, _c_p, _c_p],
    "rmsnorm_quant_rstd": [_c_p, _c_p, _c_i64, _c_i64, ctypes.c_float, _c_p, _c_p, _c_p, _c_p],
    "rmsnorm_backward": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p],
    "requant_transpose_128x1": [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p],
    "swiglu_quant": [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p],
    "gemm_fprop": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p],
    "gemm_fprop_splitk": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_i64, _c_p],
    "gemm_fprop_splitk_noalloc": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p],
    "pack_weight_rollout": [_c_p, _c_i64, _c_i64, _c_p, _c_p],
    "gemm_fprop_packed": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p],
    "gemm_fprop_swiglu_quant": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p],
    "gemm_fprop_quant": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p],
    "gemm_dgrad": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p],
    "gemm_wgrad": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p],
    "gemm_wgrad_f32": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, ctypes.c_int, _c_p],
}

STATUS = {0: "JETFP8_OK", 1: "JETFP8_EINVAL", 2: "JETFP8_EALIGN", 3: "JETFP8_ENULL",
          4: "JETFP8_EALIAS", 5: "JETFP8_EUNSUPPORTED", 6: "JETFP8_ELAUNCH"}

_lib = None


class JetFP8Error(RuntimeError):
    def __init__(self, name, status, msg):
        super().__init__(f"{name}: {STATUS.get(status, status)} ({msg})")
        self.status = status


def lib():
    """Load libjetfp8.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m quantized_rl_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, argt in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = argt
            fn.restype = ctypes.c_int
        L.rmsnorm_backward_workspace_bytes.argtypes = [_c_i64, _c_i64]
        L.rmsnorm_backward_workspace_bytes.restype = _c_i64
        L.gemm_fprop_splitk_workspace_bytes.argtypes = [_c_i64, _c_i64, _c_i64]
        L.gemm_fprop_splitk_workspace_bytes.restype = _c_i64
        L.jetfp8_status_string.argtypes = [ctypes.c_int]
        L.jetfp8_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def call_raw(name, *args):
    """Call an entry point with raw integer pointers; returns the status code."""
    return getattr(lib(), name)(*args)


def _check(name, status):
    if status != 0:
        raise JetFP8Error(name, status, lib().jetfp8_status_string(status).decode())


def _torch():
    import torch
    return torch


def _stream(dev):
    torch = _torch()
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t, dtype, shape, what):
    torch = _torch()
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{what}: expected contiguous {dtype} {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")
    if t.device.type != "cuda":
        raise ValueError(f"{what}: expected a device tensor")
    return t


def _empty(shape, dtype, dev):
    return _torch().empty(shape, dtype=dtype, device=dev)


def quantize_act_1x128(x, q=None, s=None):
    """x bf16 [M, K] -> (q uint8 [M, K], s float32 [K/128, M])."""
    torch = _torch()
    M, K = x.shape
    _need(x, torch.bfloat16, (M, K), "x")
    q = _empty((M, K), torch.uint8, x.device) if q is None else _need(q, torch.uint8, (M, K), "q")
    s = _empty((K // 128, M), torch.float32, x.device) if s is None else \
        _need(s, torch.float32, (K // 128, M), "s")
    _check("quantize_act_1x128", lib().quantize_act_1x128(
        x.data_ptr(), M, K, q.data_ptr(), s.data_ptr(), _stream(x.device)))
    return q, s


def quantize_weight_128x128(w, q=None, s=None):
    """w bf16 [N, K] -> (q uint8 [N, K], s float32 [N/128, K/128])."""
    torch = _torch()
    N, K = w.shape
    _need(w, torch.bfloat16, (N, K), "w")
    q = _empty((N, K), torch.uint8, w.device) if q is None else _need(q, torch.uint8, (N, K), "q")
    s = _empty((N // 128, K // 128), torch.float32, w.device) if s is None else \
        _need(s, torch.float32, (N // 128, K // 128), "s")
    _check("quantize_weight_128x128", lib().quantize_weight_128x128(
        w.data_ptr(), N, K, q.data_ptr(), s.data_ptr(), _stream(w.device)))
    return q, s


def rmsnorm_quant(x, gamma, eps, q=None, s=None):
    """x bf16 [M, K], gamma bf16 [K] -> (q uint8 [M, K], s float32 [K/128, M])."""
    torch = _torch()
    M, K = x.shape
    _need(x, torch.bfloat16, (M, K), "x")
    _need(gamma, torch.bfloat16, (K,), "gamma")
    q = _empty((M, K), torch.uint8, x.device) if q is None else _need(q, torch.uint8, (M, K), "q")
    s = _empty((K // 128, M), torch.float32, x.device) if s is None else \
        _need(s, torch.float32, (K // 128, M), "s")
    _check("rmsnorm_quant", lib().rmsnorm_quant(
        x.data_ptr(), gamma.data_ptr(), M, K, float(eps), q.data_ptr(), s.data_ptr(),
        _stream(x.device)))
    return q, s


def rmsnorm_quant_rstd(x, gamma, eps, q=None, s=None, rstd=None):
    """rmsnorm_quant that also returns the per-row factor: (q, s, rstd float32 [M])."""
    torch = _torch()
    M, K = x.shape
    _need(x, torch.bfloat16, (M, K), "x")
    _need(gamma, torch.bfloat16, (K,), "gamma")
    q = _empty((M, K), torch.uint8, x.device) if q is None else _need(q, torch.uint8, (M, K), "q")
    s = _empty((K // 128, M), torch.float32, x.device) if s is None else \
        _need(s, torch.float32, (K // 128, M), "s")
    rstd = _empty((M,), torch.float32, x.device) if rstd is None else _need(rstd, torch.float32, (M,), "rstd")
    _check("rmsnorm_quant_rstd", lib().rmsnorm_quant_rstd(
        x.data_ptr(), gamma.data_ptr(), M, K, float(eps), q.data_ptr(), s.data_ptr(), rstd.data_ptr(),
        _stream(x.device)))
    return q, s, rstd


def rmsnorm_backward_workspace_bytes(M, K):
    return int(lib().rmsnorm_backward_workspace_bytes(M, K))


def rmsnorm_backward(x, gamma, rstd, dy, dx=None, dgamma=None, workspace=None):
    """(dx bf16 [M, K], dgamma float32 [K]) of the RMSNorm for upstream dy bf16 [M, K];
    rstd float32 [M] from rmsnorm_quant_rstd.  The workspace (float32, at least
    rmsnorm_backward_workspace_bytes(M, K) bytes) is allocated with torch if not given."""
    torch = _torch()
    M, K = x.shape
    _need(x, torch.bfloat16, (M, K), "x")
    _need(gamma, torch.bfloat16, (K,), "gamma")
    _need(rstd, torch.float32, (M,), "rstd")
    _need(dy, torch.bfloat16, (M, K), "dy")
    dx = _empty((M, K), torch.bfloat16, x.device) if dx is None else _need(dx, torch.bfloat16, (M, K), "dx")
    dgamma = _empty((K,), torch.float32, x.device) if dgamma is None else \
        _need(dgamma, torch.float32, (K,), "dgamma")
    nbytes = rmsnorm_backward_workspace_bytes(M, K)
    if nbytes < 0:
        raise JetFP8Error("rmsnorm_backward", 1, "invalid shape")
    if workspace is None:
        workspace = _empty((max(nbytes // 4, 1),), torch.float32, x.device)
    elif workspace.dtype != torch.float32 or not workspace.is_contiguous() or workspace.numel() * 4 < nbytes:
        raise ValueError(f"workspace: expected contiguous float32 of at least {nbytes} bytes")
    _check("rmsnorm_backward", lib().rmsnorm_backward(
        x.data_ptr(), gamma.data_ptr(), rstd.data_ptr(), dy.data_ptr(), M, K, dx.data_ptr(),
        dgamma.data_ptr(), workspace.data_ptr(), _stream(x.device)))
    return dx, dgamma


def swiglu_quant(y, q=None, s=None):
    """y bf16 [M, 2I] (gate | up) -> (q uint8 [M, I], s float32 [I/128, M]): the 1x128
    quantisation of silu(gate) * up."""
    torch = _torch()
    M, I2 = y.shape
    I = I2 // 2
    _need(y, torch.bfloat16, (M, I2), "y")
    if I2 % 2:
        raise ValueError(f"y: expected an even column count (gate | up), got {I2}")
    q = _empty((M, I), torch.uint8, y.device) if q is None else _need(q, torch.uint8, (M, I), "q")
    s = _empty((I // 128, M), torch.float32, y.device) if s is None else \
        _need(s, torch.float32, (I // 128, M), "s")
    _check("swiglu_quant", lib().swiglu_quant(y.data_ptr(), M, I, q.data_ptr(), s.data_ptr(), _stream(y.device)))
    return q, s


def requant_transpose_128x1(q, s, qt=None, st=None):
    """(q uint8 [M, K], s f32 [K/128, M]) -> (qt uint8 [K, M], st f32 [M/128, K])."""
    torch = _torch()
    M, K = q.shape
    _need(q, torch.uint8, (M, K), "q")
    _need(s, torch.float32, (K // 128, M), "s")
    qt = _empty((K, M), torch.uint8, q.device) if qt is None else _need(qt, torch.uint8, (K, M), "qt")
    st = _empty((M // 128, K), torch.float32, q.device) if st is None else \
        _need(st, torch.float32, (M // 128, K), "st")
    _check("requant_transpose_128x1", lib().requant_transpose_128x1(
        q.data_ptr(), s.data_ptr(), M, K, qt.data_ptr(), st.data_ptr(), _stream(q.device)))
    return qt, st


def gemm_fprop(qx, sx, qw, sw, y=None):
    """Y bf16 [M, N] = X W^T from (qx [M,K], sx [K/128,M]) and (qw [N,K], sw [N/128,K/128])."""
    torch = _torch()
    M, K = qx.shape
    N = qw.shape[0]
    _need(qx, torch.uint8, (M, K), "qx")
    _need(sx, torch.float32, (K // 128, M), "sx")
    _need(qw, torch.uint8, (N, K), "qw")
    _need(sw, torch.float32, (N // 128, K // 128), "sw")
    y = _empty((M, N), torch.bfloat16, qx.device) if y is None else _need(y, torch.bfloat16, (M, N), "y")
    _check("gemm_fprop", lib().gemm_fprop(
        qx.data_ptr(), sx.data_ptr(), qw.data_ptr(), sw.data_ptr(), M, N, K, y.data_ptr(),
        _stream(qx.device)))
    return y


def gemm_fprop_splitk_workspace_bytes(M, N, K):
    """Bytes of fp32 workspace gemm_fprop_splitk needs (0: it runs gemm_fprop)."""
    n = lib().gemm_fprop_splitk_workspace_bytes(M, N, K)
    if n < 0:
        raise JetFP8Error("gemm_fprop_splitk_workspace_bytes", 1, f"invalid shape {M}x{N}x{K}")
    return n


def gemm_fprop_splitk(qx, sx, qw, sw, y=None, workspace=None):
    """gemm_fprop with K split across workgroups for 65..256-row batches with few
    output tiles, through an fp32 workspace (allocated here when not given)."""
    torch = _torch()
    M, K = qx.shape
    N = qw.shape[0]
    _need(qx, torch.uint8, (M, K), "qx")
    _need(sx, torch.float32, (K // 128, M), "sx")
    _need(qw, torch.uint8, (N, K), "qw")
    _need(sw, torch.float32, (N // 128, K // 128), "sw")
    y = _empty((M, N), torch.bfloat16, qx.device) if y is None else _need(y, torch.bfloat16, (M, N), "y")
    need = gemm_fprop_splitk_workspace_bytes(M, N, K)
    if workspace is None:
        workspace = _empty((max(need, 4) // 4,), torch.float32, qx.device)
    if workspace.dtype != torch.float32 or not workspace.is_contiguous() or workspace.device != qx.device:
        raise ValueError("workspace: a contiguous float32 tensor on the operands' device")
    _check("gemm_fprop_splitk", lib().gemm_fprop_splitk(
        qx.data_ptr(), sx.data_ptr(), qw.data_ptr(), sw.data_ptr(), M, N, K, y.data_ptr(),
        workspace.data_ptr(), workspace.numel() * 4, _stream(qx.device)))
    return y


def pack_weight_rollout(qw, qwp=None):
    """Rollout-packed copy of the weight codes qw uint8 [N, K]: a uint8 tensor of the
    same shape whose bytes are in the order gemm_fprop_packed streams (each 16-row
    strip's 128-deep K-block one contiguous 2 KB chunk; the scales are unchanged)."""
    torch = _torch()
    N, K = qw.shape
    _need(qw, torch.uint8, (N, K), "qw")
    qwp = _empty((N, K), torch.uint8, qw.device) if qwp is None else _need(qwp, torch.uint8, (N, K), "qwp")
    _check("pack_weight_rollout", lib().pack_weight_rollout(qw.data_ptr(), N, K, qwp.data_ptr(), _stream(qw.device)))
    return qwp


def gemm_fprop_packed(qx, sx, qwp, sw, y=None):
    """gemm_fprop for up to 256 rows over the packed weight qwp = pack_weight_rollout(qw):
    Y bf16 [M, N], bit for bit gemm_fprop(qx, sx, qw, sw)."""
    torch = _torch()
    M, K = qx.shape
    N = qwp.shape[0]
    _need(qx, torch.uint8, (M, K), "qx")
    _need(sx, torch.float32, (K // 128, M), "sx")
    _need(qwp, torch.uint8, (N, K), "qwp")
    _need(sw, torch.float32, (N // 128, K // 128), "sw")
    y = _empty((M, N), torch.bfloat16, qx.device) if y is None else _need(y, torch.bfloat16, (M, N), "y")
    _check("gemm_fprop_packed", lib().gemm_fprop_packed(
        qx.data_ptr(), sx.data_ptr(), qwp.data_ptr(), sw.data_ptr(), M, N, K, y.data_ptr(),
        _stream(qx.device)))
    return y


def gemm_fprop_swiglu_quant(qx, sx, qw, sw, qh=None, sh=None):
    """FProp of a gate+up weight qw [2I, K] (gate rows, then up rows) fused with
    SwiGLU and the 1x128 quantisation: (qh uint8 [M, I], sh float32 [I/128, M]),
    bit for bit swiglu_quant(gemm_fprop(qx, sx, qw, sw))."""
    torch = _torch()
    M, K = qx.shape
    N = qw.shape[0]
    I = N // 2
    _need(qx, torch.uint8, (M, K), "qx")
    _need(sx, torch.float32, (K // 128, M), "sx")
    _need(qw, torch.uint8, (N, K), "qw")
    _need(sw, torch.float32, (N // 128, K // 128), "sw")
    qh = _empty((M, I), torch.uint8, qx.device) if qh is None else _need(qh, torch.uint8, (M, I), "qh")
    sh = _empty((I // 128, M), torch.float32, qx.device) if sh is None else \
        _need(sh, torch.float32, (I // 128, M), "sh")
    _check("gemm_fprop_swiglu_quant", lib().gemm_fprop_swiglu_quant(
        qx.data_ptr(), sx.data_ptr(), qw.data_ptr(), sw.data_ptr(), M, N, K, qh.data_ptr(), sh.data_ptr(),
        _stream(qx.device)))
    return qh, sh


NOALLOC_SCRATCH_BYTES = 32 << 20


def gemm_fprop_splitk_noalloc(qx, sx, qw, sw, y):
    """gemm_fprop_splitk through the library's own static workspace (at most
    NOALLOC_SCRATCH_BYTES): no device allocation by the library, nor here, so
    the output y (bf16 [M, N]) is required."""
    torch = _torch()
    M, K = qx.shape
    N = qw.shape[0]
    _need(qx, torch.uint8, (M, K), "qx")
    _need(sx, torch.float32, (K // 128, M), "sx")
    _need(qw, torch.uint8, (N, K), "qw")
    _need(sw, torch.float32, (N // 128, K // 128), "sw")
    _need(y, torch.bfloat16, (M, N), "y")
    _check("gemm_fprop_splitk_noalloc", lib().gemm_fprop_splitk_noalloc(
        qx.data_ptr(), sx.data_ptr(), qw.data_ptr(), sw.data_ptr(), M, N, K, y.data_ptr(), _stream(qx.device)))
    return y


def gemm_fprop_quant(qx, sx, qw, sw, y=None, qy=None, sy=None):
    """gemm_fprop plus the 1x128 quantisation of Y for the next layer:
    returns (y bf16 [M, N], qy uint8 [M, N], sy float32 [N/128, M])."""
    torch = _torch()
    M, K = qx.shape
    N = qw.shape[0]
    _need(qx, torch.uint8, (M, K), "qx")
    _need(sx, torch.float32, (K // 128, M), "sx")
    _need(qw, torch.uint8, (N, K), "qw")
    _need(sw, torch.float32, (N // 128, K // 128), "sw")
    y = _empty((M, N), torch.bfloat16, qx.device) if y is None else _need(y, torch.bfloat16, (M, N), "y")
    qy = _empty((M, N), torch.uint8, qx.device) if qy is None else _need(qy, torch.uint8, (M, N), "qy")
    sy = _empty((N // 128, M), torch.float32, qx.device) if sy is None else \
        _need(sy, torch.float32, (N // 128, M), "sy")
    _check("gemm_fprop_quant", lib().gemm_fprop_quant(
        qx.data_ptr(), sx.data_ptr(), qw.data_ptr(), sw.data_ptr(), M, N, K, y.data_ptr(),
        qy.data_ptr(), sy.data_ptr(), _stream(qx.device)))
    return y, qy, sy


def gemm_dgrad(qdy, sdy, qw, sw, dx=None):
    """dX bf16 [M, K] = dY W from (qdy [M,N], sdy [N/128,M]) and (qw [N,K], sw [N/128,K/128])."""
    torch = _torch()
    M, N = qdy.shape
    K = qw.shape[1]
    _need(qdy, torch.uint8, (M, N), "qdy")
    _need(sdy, torch.float32, (N // 128, M), "sdy")
    _need(qw, torch.uint8, (N, K), "qw")
    _need(sw, torch.float32, (N // 128, K // 128), "sw")
    dx = _empty((M, K), torch.bfloat16, qdy.device) if dx is None else \
        _need(dx, torch.bfloat16, (M, K), "dx")
    _check("gemm_dgrad", lib().gemm_dgrad(
        qdy.data_ptr(), sdy.data_ptr(), qw.data_ptr(), sw.data_ptr(), M, N, K, dx.data_ptr(),
        _stream(qdy.device)))
    return dx


def gemm_wgrad(qdyt, sdyt, qxt, sxt, dw=None):
    """dW bf16 [N, K] = dY^T X from (qdyt [N,M], sdyt [M/128,N]) and (qxt [K,M], sxt [M/128,K])."""
    torch = _torch()
    N, M = qdyt.shape
    K = qxt.shape[0]
    _need(qdyt, torch.uint8, (N, M), "qdyt")
    _need(sdyt, torch.float32, (M // 128, N), "sdyt")
    _need(qxt, torch.uint8, (K, M), "qxt")
    _need(sxt, torch.float32, (M // 128, K), "sxt")
    dw = _empty((N, K), torch.bfloat16, qdyt.device) if dw is None else \
        _need(dw, torch.bfloat16, (N, K), "dw")
    _check("gemm_wgrad", lib().gemm_wgrad(
        qdyt.data_ptr(), sdyt.data_ptr(), qxt.data_ptr(), sxt.data_ptr(), M, N, K, dw.data_ptr(),
        _stream(qdyt.device)))
    return dw


def gemm_wgrad_f32(qdyt, sdyt, qxt, sxt, dw=None, accumulate=False):
    """dW fp32 [N, K] = dY^T X (operands as gemm_wgrad), written into a new or given
    tensor, or added to the given ``dw`` when ``accumulate`` is true."""
    torch = _torch()
    N, M = qdyt.shape
    K = qxt.shape[0]
    _need(qdyt, torch.uint8, (N, M), "qdyt")
    _need(sdyt, torch.float32, (M // 128, N), "sdyt")
    _need(qxt, torch.uint8, (K, M), "qxt")
    _need(sxt, torch.float32, (M // 128, K), "sxt")
    if dw is None:
        if accumulate:
            raise ValueError("gemm_wgrad_f32: accumulate=True needs the dw tensor to add to")
        dw = _empty((N, K), torch.float32, qdyt.device)
    else:
        _need(dw, torch.float32, (N, K), "dw")
    _check("gemm_wgrad_f32", lib().gemm_wgrad_f32(
        qdyt.data_ptr(), sdyt.data_ptr(), qxt.data_ptr(), sxt.data_ptr(), M, N, K, dw.data_ptr(),
        1 if accumulate else 0, _stream(qdyt.device)))
    return dw
