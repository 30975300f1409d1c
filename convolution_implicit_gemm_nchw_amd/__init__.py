"""Python binding of ``libmiconv.so``, the gfx950 implicit-GEMM convolution library.

Argument marshalling only: every computation runs in the library's HIP
kernels.  Tensors are torch CUDA (ROCm) tensors; torch supplies device memory
and the current stream.  The functions carry the C ABI's names
(``include/miconv.h``):

  conv2d_fwd(x, w, pad, stride)                 -> y   [N,K,P,Q] fp32
  conv2d_fwd_ex(x, w, pad, stride, bias, alpha, beta, relu, y, out_dtype)
                                                -> y = act(alpha*conv + beta*y + bias[k]), fp32 or bf16
  conv2d_bwd_data(dy, w, (H, W), pad, stride)   -> dx  [N,C,H,W] fp32
  conv2d_bwd_filter(x, dy, (R, S), pad, stride) -> dw  [K,C,R,S] fp32
  deconv2d_fwd(x, w, (H_out, W_out), pad, stride) -> y [N,C_out,H_out,W_out] fp32
  deconv2d_bwd_data(dy, w, (H_in, W_in), pad, stride)     -> dx [N,C_in,H_in,W_in] fp32
  deconv2d_bwd_filter(x, dy, (R, S), pad, stride)         -> dw [C_in,C_out,R,S] fp32
  conv2d_bwd_data_ex / conv2d_bwd_filter_ex / deconv2d_bwd_data_ex / deconv2d_bwd_filter_ex
                                                -> out = alpha*result + beta*out, fp32 or bf16
  deconv2d_fwd_ex(x, w, (H_out, W_out), pad, stride, bias, alpha, beta, relu, y, out_dtype)
                                                -> y = act(alpha*deconv + beta*y + bias[c_out])
  conv2d_bwd_bias(dy, alpha, beta, db)          -> db[k] = alpha*sum_{n,p,q} dy[n,k,p,q] + beta*db
  conv2d_bwd_filter_noalloc(x, dy, (R, S), pad, stride) -> dw, no workspace (static device scratch)
  find_plan(pass, in0, in1, out, sizes13)       -> timed candidate plans, fastest installed
  convnd_fwd / convnd_bwd_data / convnd_bwd_filter  (1-3 spatial dims, groups, dilation,
                                                asymmetric or "same"/"valid" padding)
  plan_candidates / plan_select / plan_cache_clear / plan_cache_entries   (the plan cache)

Inputs must all be float32 or all bfloat16, contiguous, on the current device.
If the shared library is missing this module raises on import: there is no
fallback path.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmiconv.so")

F32, BF16 = 0, 1
FWD, BWD_DATA, BWD_FILTER, DECONV_FWD, DECONV_BWD_DATA, DECONV_BWD_FILTER = 0, 1, 2, 3, 4, 5
MAX_WORKSPACE_BYTES = 1_000_000_000
ERR_HIP = 8

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python convolution_implicit_gemm_nchw_amd/build.py` "
        "(hipcc, gfx950).  There is no non-HIP fallback.")

_lib = ctypes.CDLL(LIB_PATH)
_I, _SZ, _VP = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
_ARGS13 = [_I] * 13
for _name in ("conv2d_fwd", "conv2d_bwd_data", "conv2d_bwd_filter", "deconv2d_fwd", "deconv2d_bwd_data",
              "deconv2d_bwd_filter"):
    _fn = getattr(_lib, _name)
    _fn.argtypes = _ARGS13 + [_I, _VP, _VP, _VP, _VP, _SZ, _VP]
    _fn.restype = _I
_lib.conv2d_fwd_ex.argtypes = _ARGS13 + [_I, _VP, _VP, _VP, ctypes.c_float, ctypes.c_float, _I, _I, _VP, _VP,
                                          _SZ, _VP]
_lib.conv2d_fwd_ex.restype = _I
_F = ctypes.c_float
for _name in ("conv2d_bwd_data_ex", "conv2d_bwd_filter_ex", "deconv2d_bwd_data_ex", "deconv2d_bwd_filter_ex"):
    _fn = getattr(_lib, _name)
    _fn.argtypes = _ARGS13 + [_I, _VP, _VP, _F, _F, _I, _VP, _VP, _SZ, _VP]
    _fn.restype = _I
_lib.deconv2d_fwd_ex.argtypes = _ARGS13 + [_I, _VP, _VP, _VP, _F, _F, _I, _I, _VP, _VP, _SZ, _VP]
_lib.deconv2d_fwd_ex.restype = _I
_lib.conv2d_bwd_bias.argtypes = [_I, _I, _I, _I, _I, _VP, _F, _F, _VP, _VP]
_lib.conv2d_bwd_bias.restype = _I
_lib.conv2d_bwd_filter_noalloc.argtypes = _ARGS13 + [_I, _VP, _VP, _VP, _VP]
_lib.conv2d_bwd_filter_noalloc.restype = _I


class NdDesc(ctypes.Structure):
    """miconv_nd_desc_t: spatial arrays outermost first, first ndim entries used."""
    _fields_ = [("ndim", _I), ("N", _I), ("C", _I), ("K", _I), ("groups", _I), ("in_", _I * 3),
                ("filter", _I * 3), ("out", _I * 3), ("pad_lo", _I * 3), ("pad_hi", _I * 3),
                ("stride", _I * 3), ("dilation", _I * 3)]


_NDP = ctypes.POINTER(NdDesc)
_lib.miconv_nd_padding.argtypes = [_NDP, _I]
_lib.miconv_nd_padding.restype = _I
for _name in ("convnd_fwd", "convnd_bwd_data", "convnd_bwd_filter"):
    _fn = getattr(_lib, _name)
    _fn.argtypes = [_NDP, _I, _VP, _VP, _VP, _VP, _SZ, _VP]
    _fn.restype = _I
_lib.convnd_workspace_size.argtypes = [_I, _NDP, _I, _SZ, ctypes.POINTER(_SZ)]
_lib.convnd_workspace_size.restype = _I
_lib.convnd_describe.argtypes = [_I, _NDP, _I, _SZ, ctypes.c_char_p, _SZ]
_lib.convnd_describe.restype = _I


class PerfResult(ctypes.Structure):
    _fields_ = [("index", _I), ("status", _I), ("time_ms", ctypes.c_float), ("workspace_bytes", _SZ),
                ("plan", ctypes.c_char * 256)]


_lib.miconv_plan_candidates.argtypes = [_I, _I] + _ARGS13 + [_SZ, ctypes.POINTER(_I), ctypes.POINTER(_SZ)]
_lib.miconv_plan_candidates.restype = _I
_lib.miconv_plan_select.argtypes = [_I, _I] + _ARGS13 + [_SZ, _I]
_lib.miconv_plan_select.restype = _I
_lib.miconv_find_plan.argtypes = [_I, _I] + _ARGS13 + [_VP, _VP, _VP, _VP, _SZ, _VP, _I, ctypes.POINTER(_I),
                                                      ctypes.POINTER(PerfResult)]
_lib.miconv_find_plan.restype = _I
_lib.miconv_plan_cache_clear.argtypes = []
_lib.miconv_plan_cache_clear.restype = _I
_lib.miconv_plan_cache_entries.argtypes = [ctypes.POINTER(_I), ctypes.POINTER(_I)]
_lib.miconv_plan_cache_entries.restype = _I
_lib.miconv_workspace_size.argtypes = [_I, _I] + _ARGS13 + [_SZ, ctypes.POINTER(_SZ)]
_lib.miconv_workspace_size.restype = _I
_lib.miconv_plan_describe.argtypes = [_I, _I] + _ARGS13 + [_SZ, ctypes.c_char_p, _SZ]
_lib.miconv_plan_describe.restype = _I
_lib.miconv_status_string.argtypes = [_I]
_lib.miconv_status_string.restype = ctypes.c_char_p
_lib.miconv_abi_version.argtypes = []
_lib.miconv_abi_version.restype = _I


class MiconvError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


def lib():
    """The loaded ctypes library (for calling the C ABI directly)."""
    return _lib


def status_string(status: int) -> str:
    return _lib.miconv_status_string(int(status)).decode()


def _check(status, where):
    if status != 0:
        raise (MiconvError(status, where) if status == ERR_HIP else ValueError(
            f"{where}: status {status} ({status_string(status)})"))


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def out_size(H, W, R, S, pad, stride):
    """P, Q for the given sizes (floor((in + 2 pad - f) / stride) + 1)."""
    return (H + 2 * pad[0] - R) // stride[0] + 1, (W + 2 * pad[1] - S) // stride[1] + 1


def _pair(v):
    return (v, v) if isinstance(v, int) else tuple(v)


def workspace_size(pass_id, dtype, args13, limit=MAX_WORKSPACE_BYTES) -> int:
    out = _SZ(0)
    _check(_lib.miconv_workspace_size(pass_id, dtype, *args13, limit, ctypes.byref(out)),
           "miconv_workspace_size")
    return int(out.value)


def plan_describe(pass_id, dtype, args13, workspace_bytes=MAX_WORKSPACE_BYTES) -> str:
    buf = ctypes.create_string_buffer(512)
    _check(_lib.miconv_plan_describe(pass_id, dtype, *args13, workspace_bytes, buf, 512),
           "miconv_plan_describe")
    return buf.value.decode()


def _stream(stream):
    return stream if stream is not None else torch.cuda.current_stream()


def _workspace(pass_id, dtype, args13, workspace, stream):
    """(pointer, bytes, owner) of the workspace: the caller's tensor, or a fresh one sized for
    the plan.  A fresh one is allocated from the pool of the stream the kernels run on, so when
    ``owner`` is released after the call the caching allocator hands that block only to work
    ordered after those kernels on the same stream (no cross-stream reuse, no global state)."""
    if workspace is not None:
        return workspace.data_ptr(), workspace.numel() * workspace.element_size(), workspace
    need = workspace_size(pass_id, dtype, args13)
    if need == 0:
        return None, 0, None
    with torch.cuda.stream(stream):
        ws = torch.empty(need, dtype=torch.uint8, device=stream.device)
    return ws.data_ptr(), need, ws


def _inputs(*ts):
    d = dtype_code(ts[0])
    for t in ts:
        if dtype_code(t) != d:
            raise ValueError("all inputs must share one dtype")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("inputs must be contiguous device tensors")
    return d


def conv2d_fwd(x, w, pad=0, stride=1, y=None, workspace=None, stream=None):
    """y[n,k,p,q] = sum_{c,r,s} w[k,c,r,s] * x~(n, c, p*sh - ph + r, q*sw - pw + s)."""
    pad, stride = _pair(pad), _pair(stride)
    d = _inputs(x, w)
    N, C, H, W = x.shape
    K, _, R, S = w.shape
    P, Q = out_size(H, W, R, S, pad, stride)
    if y is None:
        y = torch.empty((N, K, max(P, 0), max(Q, 0)), dtype=torch.float32, device=x.device)
    a = (N, C, H, W, K, R, S, pad[0], pad[1], stride[0], stride[1], P, Q)
    st = _stream(stream)
    wp, wb, _keep = _workspace(FWD, d, a, workspace, st)
    _check(_lib.conv2d_fwd(*a, d, x.data_ptr(), w.data_ptr(), y.data_ptr(), wp, wb,
                           st.cuda_stream), "conv2d_fwd")
    return y


def conv2d_fwd_ex(x, w, pad=0, stride=1, bias=None, alpha=1.0, beta=0.0, relu=False, y=None, workspace=None,
                  stream=None, out_dtype=torch.float32):
    """y = act(alpha * conv2d(x, w) + beta * y + bias[k]) in one pass (act = ReLU when relu).
    bias: fp32 [K] device tensor or None; y is read only when beta != 0.  y (or out_dtype
    when y is None) is float32 or bfloat16; a bf16 y gets the fp32 result rounded once."""
    pad, stride = _pair(pad), _pair(stride)
    d = _inputs(x, w)
    N, C, H, W = x.shape
    K, _, R, S = w.shape
    P, Q = out_size(H, W, R, S, pad, stride)
    if y is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs the previous output y")
        y = torch.empty((N, K, max(P, 0), max(Q, 0)), dtype=out_dtype, device=x.device)
    if not y.is_cuda or not y.is_contiguous():
        raise ValueError("y must be a contiguous device tensor")
    od = dtype_code(y)
    bp = None
    if bias is not None:
        if bias.dtype != torch.float32 or not bias.is_cuda or not bias.is_contiguous() or bias.numel() != K:
            raise ValueError("bias must be a contiguous float32 device tensor of K elements")
        bp = bias.data_ptr()
    a = (N, C, H, W, K, R, S, pad[0], pad[1], stride[0], stride[1], P, Q)
    st = _stream(stream)
    wp, wb, _keep = _workspace(FWD, d, a, workspace, st)
    _check(_lib.conv2d_fwd_ex(*a, d, x.data_ptr(), w.data_ptr(), bp, float(alpha), float(beta), int(bool(relu)),
                              od, y.data_ptr(), wp, wb, st.cuda_stream), "conv2d_fwd_ex")
    return y


def conv2d_bwd_data(dy, w, in_hw, pad=0, stride=1, dx=None, workspace=None, stream=None):
    """dx = adjoint of conv2d_fwd in x, applied to dy."""
    pad, stride = _pair(pad), _pair(stride)
    d = _inputs(dy, w)
    N, K, P, Q = dy.shape
    _, C, R, S = w.shape
    H, W = in_hw
    if dx is None:
        dx = torch.empty((N, C, H, W), dtype=torch.float32, device=dy.device)
    a = (N, C, H, W, K, R, S, pad[0], pad[1], stride[0], stride[1], P, Q)
    st = _stream(stream)
    wp, wb, _keep = _workspace(BWD_DATA, d, a, workspace, st)
    _check(_lib.conv2d_bwd_data(*a, d, dy.data_ptr(), w.data_ptr(), dx.data_ptr(), wp, wb,
                                st.cuda_stream), "conv2d_bwd_data")
    return dx


def conv2d_bwd_filter(x, dy, filter_rs, pad=0, stride=1, dw=None, workspace=None, stream=None):
    """dw = adjoint of conv2d_fwd in w, applied to dy."""
    pad, stride = _pair(pad), _pair(stride)
    d = _inputs(x, dy)
    N, C, H, W = x.shape
    _, K, P, Q = dy.shape
    R, S = filter_rs
    if dw is None:
        dw = torch.empty((K, C, R, S), dtype=torch.float32, device=x.device)
    a = (N, C, H, W, K, R, S, pad[0], pad[1], stride[0], stride[1], P, Q)
    st = _stream(stream)
    wp, wb, _keep = _workspace(BWD_FILTER, d, a, workspace, st)
    _check(_lib.conv2d_bwd_filter(*a, d, x.data_ptr(), dy.data_ptr(), dw.data_ptr(), wp, wb,
                                  st.cuda_stream), "conv2d_bwd_filter")
    return dw


def deconv2d_fwd(x, w, out_hw, pad=0, stride=1, y=None, workspace=None, stream=None):
    """Transposed convolution; w is [C_in][C_out][R][S] (backward-data with the role swap)."""
    pad, stride = _pair(pad), _pair(stride)
    d = _inputs(x, w)
    N, Cin, Hin, Win = x.shape
    _, Cout, R, S = w.shape
    Hout, Wout = out_hw
    if y is None:
        y = torch.empty((N, Cout, Hout, Wout), dtype=torch.float32, device=x.device)
    a = (N, Cin, Hin, Win, Cout, R, S, pad[0], pad[1], stride[0], stride[1], Hout, Wout)
    st = _stream(stream)
    wp, wb, _keep = _workspace(DECONV_FWD, d, a, workspace, st)
    _check(_lib.deconv2d_fwd(*a, d, x.data_ptr(), w.data_ptr(), y.data_ptr(), wp, wb,
                             st.cuda_stream), "deconv2d_fwd")
    return y


def deconv2d_bwd_data(dy, w, in_hw, pad=0, stride=1, dx=None, workspace=None, stream=None):
    """Adjoint of deconv2d_fwd in its input: dy [N,C_out,H_out,W_out], w [C_in,C_out,R,S]
    -> dx [N,C_in,H_in,W_in] (the forward convolution with the role swap)."""
    pad, stride = _pair(pad), _pair(stride)
    d = _inputs(dy, w)
    N, Cout, Hout, Wout = dy.shape
    Cin, _, R, S = w.shape
    Hin, Win = in_hw
    if dx is None:
        dx = torch.empty((N, Cin, Hin, Win), dtype=torch.float32, device=dy.device)
    a = (N, Cin, Hin, Win, Cout, R, S, pad[0], pad[1], stride[0], stride[1], Hout, Wout)
    st = _stream(stream)
    wp, wb, _keep = _workspace(DECONV_BWD_DATA, d, a, workspace, st)
    _check(_lib.deconv2d_bwd_data(*a, d, dy.data_ptr(), w.data_ptr(), dx.data_ptr(), wp, wb,
                                  st.cuda_stream), "deconv2d_bwd_data")
    return dx


def deconv2d_bwd_filter(x, dy, filter_rs, pad=0, stride=1, dw=None, workspace=None, stream=None):
    """Adjoint of deconv2d_fwd in w: x [N,C_in,H_in,W_in], dy [N,C_out,H_out,W_out]
    -> dw [C_in,C_out,R,S] (backward-filter with the role swap)."""
    pad, stride = _pair(pad), _pair(stride)
    d = _inputs(x, dy)
    N, Cin, Hin, Win = x.shape
    _, Cout, Hout, Wout = dy.shape
    R, S = filter_rs
    if dw is None:
        dw = torch.empty((Cin, Cout, R, S), dtype=torch.float32, device=x.device)
    a = (N, Cin, Hin, Win, Cout, R, S, pad[0], pad[1], stride[0], stride[1], Hout, Wout)
    st = _stream(stream)
    wp, wb, _keep = _workspace(DECONV_BWD_FILTER, d, a, workspace, st)
    _check(_lib.deconv2d_bwd_filter(*a, d, x.data_ptr(), dy.data_ptr(), dw.data_ptr(), wp, wb,
                                    st.cuda_stream), "deconv2d_bwd_filter")
    return dw


def _epi_out(out, shape, out_dtype, beta, device, name):
    """The output tensor of an epilogue call: the caller's (contiguous, fp32 or bf16, on the
    device), or a fresh one of out_dtype when beta == 0."""
    if out is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs the previous output " + name)
        out = torch.empty(shape, dtype=out_dtype, device=device)
    if not out.is_cuda or not out.is_contiguous() or tuple(out.shape) != tuple(shape):
        raise ValueError(name + " must be a contiguous device tensor of shape " + str(tuple(shape)))
    return out, dtype_code(out)


def _bias_ptr(bias, n):
    if bias is None:
        return None
    if bias.dtype != torch.float32 or not bias.is_cuda or not bias.is_contiguous() or bias.numel() != n:
        raise ValueError("bias must be a contiguous float32 device tensor of %d elements" % n)
    return bias.data_ptr()


def conv2d_bwd_data_ex(dy, w, in_hw, pad=0, stride=1, alpha=1.0, beta=0.0, dx=None, workspace=None,
                       stream=None, out_dtype=torch.float32):
    """dx = alpha * conv2d_bwd_data(dy, w) + beta * dx (dx read only when beta != 0), written as
    float32 or bfloat16 (dx's dtype, or out_dtype when dx is None)."""
    pad, stride = _pair(pad), _pair(stride)
    d = _inputs(dy, w)
    N, K, P, Q = dy.shape
    _, C, R, S = w.shape
    H, W = in_hw
    dx, od = _epi_out(dx, (N, C, H, W), out_dtype, beta, dy.device, "dx")
    a = (N, C, H, W, K, R, S, pad[0], pad[1], stride[0], stride[1], P, Q)
    st = _stream(stream)
    wp, wb, _keep = _workspace(BWD_DATA, d, a, workspace, st)
    _check(_lib.conv2d_bwd_data_ex(*a, d, dy.data_ptr(), w.data_ptr(), float(alpha), float(beta), od,
                                   dx.data_ptr(), wp, wb, st.cuda_stream), "conv2d_bwd_data_ex")
    return dx


def conv2d_bwd_filter_ex(x, dy, filter_rs, pad=0, stride=1, alpha=1.0, beta=0.0, dw=None, workspace=None,
                         stream=None, out_dtype=torch.float32):
    """dw = alpha * conv2d_bwd_filter(x, dy) + beta * dw, float32 or bfloat16 dw."""
    pad, stride = _pair(pad), _pair(stride)
    d = _inputs(x, dy)
    N, C, H, W = x.shape
    _, K, P, Q = dy.shape
    R, S = filter_rs
    dw, od = _epi_out(dw, (K, C, R, S), out_dtype, beta, x.device, "dw")
    a = (N, C, H, W, K, R, S, pad[0], pad[1], stride[0], stride[1], P, Q)
    st = _stream(stream)
    wp, wb, _keep = _workspace(BWD_FILTER, d, a, workspace, st)
    _check(_lib.conv2d_bwd_filter_ex(*a, d, x.data_ptr(), dy.data_ptr(), float(alpha), float(beta), od,
                                     dw.data_ptr(), wp, wb, st.cuda_stream), "conv2d_bwd_filter_ex")
    return dw


def deconv2d_fwd_ex(x, w, out_hw, pad=0, stride=1, bias=None, alpha=1.0, beta=0.0, relu=False, y=None,
                    workspace=None, stream=None, out_dtype=torch.float32):
    """y = act(alpha * deconv2d_fwd(x, w) + beta * y + bias[c_out]) (act = ReLU when relu);
    bias: fp32 [C_out] device tensor or None."""
    pad, stride = _pair(pad), _pair(stride)
    d = _inputs(x, w)
    N, Cin, Hin, Win = x.shape
    _, Cout, R, S = w.shape
    Hout, Wout = out_hw
    y, od = _epi_out(y, (N, Cout, Hout, Wout), out_dtype, beta, x.device, "y")
    bp = _bias_ptr(bias, Cout)
    a = (N, Cin, Hin, Win, Cout, R, S, pad[0], pad[1], stride[0], stride[1], Hout, Wout)
    st = _stream(stream)
    wp, wb, _keep = _workspace(DECONV_FWD, d, a, workspace, st)
    _check(_lib.deconv2d_fwd_ex(*a, d, x.data_ptr(), w.data_ptr(), bp, float(alpha), float(beta),
                                int(bool(relu)), od, y.data_ptr(), wp, wb, st.cuda_stream), "deconv2d_fwd_ex")
    return y


def deconv2d_bwd_data_ex(dy, w, in_hw, pad=0, stride=1, alpha=1.0, beta=0.0, dx=None, workspace=None,
                         stream=None, out_dtype=torch.float32):
    """dx = alpha * deconv2d_bwd_data(dy, w) + beta * dx, float32 or bfloat16 dx."""
    pad, stride = _pair(pad), _pair(stride)
    d = _inputs(dy, w)
    N, Cout, Hout, Wout = dy.shape
    Cin, _, R, S = w.shape
    Hin, Win = in_hw
    dx, od = _epi_out(dx, (N, Cin, Hin, Win), out_dtype, beta, dy.device, "dx")
    a = (N, Cin, Hin, Win, Cout, R, S, pad[0], pad[1], stride[0], stride[1], Hout, Wout)
    st = _stream(stream)
    wp, wb, _keep = _workspace(DECONV_BWD_DATA, d, a, workspace, st)
    _check(_lib.deconv2d_bwd_data_ex(*a, d, dy.data_ptr(), w.data_ptr(), float(alpha), float(beta), od,
                                     dx.data_ptr(), wp, wb, st.cuda_stream), "deconv2d_bwd_data_ex")
    return dx


def deconv2d_bwd_filter_ex(x, dy, filter_rs, pad=0, stride=1, alpha=1.0, beta=0.0, dw=None, workspace=None,
                           stream=None, out_dtype=torch.float32):
    """dw = alpha * deconv2d_bwd_filter(x, dy) + beta * dw, float32 or bfloat16 dw."""
    pad, stride = _pair(pad), _pair(stride)
    d = _inputs(x, dy)
    N, Cin, Hin, Win = x.shape
    _, Cout, Hout, Wout = dy.shape
    R, S = filter_rs
    dw, od = _epi_out(dw, (Cin, Cout, R, S), out_dtype, beta, x.device, "dw")
    a = (N, Cin, Hin, Win, Cout, R, S, pad[0], pad[1], stride[0], stride[1], Hout, Wout)
    st = _stream(stream)
    wp, wb, _keep = _workspace(DECONV_BWD_FILTER, d, a, workspace, st)
    _check(_lib.deconv2d_bwd_filter_ex(*a, d, x.data_ptr(), dy.data_ptr(), float(alpha), float(beta), od,
                                       dw.data_ptr(), wp, wb, st.cuda_stream), "deconv2d_bwd_filter_ex")
    return dw


def conv2d_bwd_bias(dy, alpha=1.0, beta=0.0, db=None, stream=None):
    """db[k] = alpha * sum_{n,p,q} dy[n,k,p,q] + beta * db[k] (fp32 [K]).  For a deconvolution
    bias, pass the deconvolution's output gradient [N, C_out, H_out, W_out]."""
    d = _inputs(dy)
    N, K, P, Q = dy.shape
    if db is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs the previous db")
        db = torch.empty(K, dtype=torch.float32, device=dy.device)
    if db.dtype != torch.float32 or not db.is_cuda or not db.is_contiguous() or db.numel() != K:
        raise ValueError("db must be a contiguous float32 device tensor of K elements")
    st = _stream(stream)
    _check(_lib.conv2d_bwd_bias(N, K, P, Q, d, dy.data_ptr(), float(alpha), float(beta), db.data_ptr(),
                                st.cuda_stream), "conv2d_bwd_bias")
    return db


def conv2d_bwd_filter_noalloc(x, dy, filter_rs, pad=0, stride=1, dw=None, stream=None):
    """conv2d_bwd_filter with no workspace argument: split-K partial sums go to the library's
    static per-device scratch array (calls that overlap in time on one device race)."""
    pad, stride = _pair(pad), _pair(stride)
    d = _inputs(x, dy)
    N, C, H, W = x.shape
    _, K, P, Q = dy.shape
    R, S = filter_rs
    if dw is None:
        dw = torch.empty((K, C, R, S), dtype=torch.float32, device=x.device)
    a = (N, C, H, W, K, R, S, pad[0], pad[1], stride[0], stride[1], P, Q)
    st = _stream(stream)
    _check(_lib.conv2d_bwd_filter_noalloc(*a, d, x.data_ptr(), dy.data_ptr(), dw.data_ptr(), st.cuda_stream),
           "conv2d_bwd_filter_noalloc")
    return dw


def plan_candidates(pass_id, dtype, args13, limit=MAX_WORKSPACE_BYTES):
    """(number of candidate plans, largest workspace any of them uses) under the budget."""
    n, ws = _I(0), _SZ(0)
    _check(_lib.miconv_plan_candidates(pass_id, dtype, *args13, limit, ctypes.byref(n), ctypes.byref(ws)),
           "miconv_plan_candidates")
    return n.value, ws.value


def plan_select(pass_id, dtype, args13, index, limit=MAX_WORKSPACE_BYTES):
    """Installs candidate `index` as the plan for these sizes (index < 0: back to the default)."""
    _check(_lib.miconv_plan_select(pass_id, dtype, *args13, limit, int(index)), "miconv_plan_select")


def plan_cache_clear():
    _check(_lib.miconv_plan_cache_clear(), "miconv_plan_cache_clear")


def plan_cache_entries():
    """(installed plans, all cached plans)."""
    t, n = _I(0), _I(0)
    _check(_lib.miconv_plan_cache_entries(ctypes.byref(t), ctypes.byref(n)), "miconv_plan_cache_entries")
    return t.value, n.value


def find_plan(pass_id, in0, in1, out, args13, workspace=None, stream=None, requested=16,
              limit=MAX_WORKSPACE_BYTES):
    """Times every candidate plan on these buffers (the pass's compute reading of in0, in1, out),
    installs the fastest for these sizes and returns the results fastest first, as dicts with
    index, status, time_ms, workspace_bytes and plan.  Without a workspace, one large enough for
    every candidate under `limit` is allocated on the stream."""
    d = _inputs(in0, in1)
    if not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous device tensor")
    st = _stream(stream)
    if workspace is None:
        _, need = plan_candidates(pass_id, d, args13, limit)
        with torch.cuda.stream(st):
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=st.device)
        wp, wb = workspace.data_ptr(), need
    else:
        wp, wb = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    res = (PerfResult * max(int(requested), 1))()
    got = _I(0)
    _check(_lib.miconv_find_plan(pass_id, d, *args13, in0.data_ptr(), in1.data_ptr(), out.data_ptr(),
                                 wp if wb else None, wb, st.cuda_stream, int(requested), ctypes.byref(got), res),
           "miconv_find_plan")
    return [dict(index=r.index, status=r.status, time_ms=r.time_ms, workspace_bytes=r.workspace_bytes,
                 plan=r.plan.decode()) for r in res[:got.value]]


PAD_VALID, PAD_SAME = 0, 1


def nd_desc(N, C, K, in_sizes, filt, groups=1, pad_lo=None, pad_hi=None, stride=None, dilation=None,
            padding=None):
    """The descriptor of a generalised convolution.  ``padding`` "same" / "valid" lets the library
    derive pad_lo, pad_hi and the output sizes (miconv_nd_padding); otherwise pad_lo / pad_hi
    (default 0, pad_hi defaulting to pad_lo) give them and the output sizes follow the floor rule."""
    nd = len(in_sizes)
    if not 1 <= nd <= 3 or len(filt) != nd:
        raise ValueError("1 to 3 spatial dimensions, filter of the same rank")
    stride = tuple(stride) if stride is not None else (1,) * nd
    dilation = tuple(dilation) if dilation is not None else (1,) * nd
    d = NdDesc()
    d.ndim, d.N, d.C, d.K, d.groups = nd, N, C, K, groups
    for i in range(nd):
        d.in_[i], d.filter[i], d.stride[i], d.dilation[i] = in_sizes[i], filt[i], stride[i], dilation[i]
    if padding is not None:
        mode = {"valid": PAD_VALID, "same": PAD_SAME}[padding]
        _check(_lib.miconv_nd_padding(ctypes.byref(d), mode), "miconv_nd_padding")
        return d
    lo = tuple(pad_lo) if pad_lo is not None else (0,) * nd
    hi = tuple(pad_hi) if pad_hi is not None else lo
    for i in range(nd):
        d.pad_lo[i], d.pad_hi[i] = lo[i], hi[i]
        d.out[i] = (in_sizes[i] + lo[i] + hi[i] - dilation[i] * (filt[i] - 1) - 1) // stride[i] + 1
    return d


def nd_out(d):
    return tuple(d.out[i] for i in range(d.ndim))


def convnd_workspace_size(pass_id, d, dtype, limit=MAX_WORKSPACE_BYTES):
    out = _SZ(0)
    _check(_lib.convnd_workspace_size(pass_id, ctypes.byref(d), dtype, limit, ctypes.byref(out)),
           "convnd_workspace_size")
    return out.value


def convnd_describe(pass_id, d, dtype, workspace_bytes=MAX_WORKSPACE_BYTES):
    buf = ctypes.create_string_buffer(512)
    _check(_lib.convnd_describe(pass_id, ctypes.byref(d), dtype, workspace_bytes, buf, 512), "convnd_describe")
    return buf.value.decode()


def _nd_workspace(pass_id, d, dtype, workspace, stream):
    if workspace is not None:
        return workspace.data_ptr(), workspace.numel() * workspace.element_size(), workspace
    need = convnd_workspace_size(pass_id, d, dtype)
    if need == 0:
        return None, 0, None
    with torch.cuda.stream(stream):
        ws = torch.empty(need, dtype=torch.uint8, device=stream.device)
    return ws.data_ptr(), need, ws


def convnd_fwd(x, w, groups=1, pad_lo=None, pad_hi=None, stride=None, dilation=None, padding=None, y=None,
               workspace=None, stream=None):
    """Generalised forward: x [N, C, *in], w [K, C/groups, *filt] -> y [N, K, *out] fp32."""
    dt = _inputs(x, w)
    d = nd_desc(x.shape[0], x.shape[1], w.shape[0], tuple(x.shape[2:]), tuple(w.shape[2:]), groups, pad_lo,
                pad_hi, stride, dilation, padding)
    if y is None:
        y = torch.empty((x.shape[0], w.shape[0]) + tuple(max(o, 0) for o in nd_out(d)), dtype=torch.float32,
                        device=x.device)
    st = _stream(stream)
    wp, wb, _keep = _nd_workspace(FWD, d, dt, workspace, st)
    _check(_lib.convnd_fwd(ctypes.byref(d), dt, x.data_ptr(), w.data_ptr(), y.data_ptr(), wp, wb, st.cuda_stream),
           "convnd_fwd")
    return y


def convnd_bwd_data(dy, w, in_sizes, groups=1, pad_lo=None, pad_hi=None, stride=None, dilation=None, padding=None,
                    dx=None, workspace=None, stream=None):
    """Adjoint of convnd_fwd in x: dy [N, K, *out], w [K, C/groups, *filt] -> dx [N, C, *in] fp32."""
    dt = _inputs(dy, w)
    C = w.shape[1] * groups
    d = nd_desc(dy.shape[0], C, dy.shape[1], tuple(in_sizes), tuple(w.shape[2:]), groups, pad_lo, pad_hi, stride,
                dilation, padding)
    if dx is None:
        dx = torch.empty((dy.shape[0], C) + tuple(in_sizes), dtype=torch.float32, device=dy.device)
    st = _stream(stream)
    wp, wb, _keep = _nd_workspace(BWD_DATA, d, dt, workspace, st)
    _check(_lib.convnd_bwd_data(ctypes.byref(d), dt, dy.data_ptr(), w.data_ptr(), dx.data_ptr(), wp, wb,
                                st.cuda_stream), "convnd_bwd_data")
    return dx


def convnd_bwd_filter(x, dy, filt, groups=1, pad_lo=None, pad_hi=None, stride=None, dilation=None, padding=None,
                      dw=None, workspace=None, stream=None):
    """Adjoint of convnd_fwd in w: x [N, C, *in], dy [N, K, *out] -> dw [K, C/groups, *filt] fp32."""
    dt = _inputs(x, dy)
    d = nd_desc(x.shape[0], x.shape[1], dy.shape[1], tuple(x.shape[2:]), tuple(filt), groups, pad_lo, pad_hi,
                stride, dilation, padding)
    if dw is None:
        dw = torch.empty((dy.shape[1], x.shape[1] // groups) + tuple(filt), dtype=torch.float32, device=x.device)
    st = _stream(stream)
    wp, wb, _keep = _nd_workspace(BWD_FILTER, d, dt, workspace, st)
    _check(_lib.convnd_bwd_filter(ctypes.byref(d), dt, x.data_ptr(), dy.data_ptr(), dw.data_ptr(), wp, wb,
                                  st.cuda_stream), "convnd_bwd_filter")
    return dw

