"""ctypes binding over libfftconv.so (the C ABI in include/fftconv.h).

Argument marshalling only: every step of the convolution runs in the HIP
library.  PyTorch supplies device memory (tensors) and the current stream.
If the library is not built, calls raise -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfftconv.so")

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "alignment",
          4: "workspace", 5: "hip error"}
DTYPES = {"f32": 0, "f16": 1, "bf16": 2}

_lib = None


class FFTConvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what, STATUS.get(status, "?"),
                                                 status))


class PlanInfo(ctypes.Structure):
    _fields_ = [("N", ctypes.c_size_t), ("M", ctypes.c_size_t),
                ("order", ctypes.c_int), ("factors", ctypes.c_int * 8),
                ("path", ctypes.c_int), ("outer_factors", ctypes.c_int),
                ("dtype", ctypes.c_int),
                ("spectrum_bytes_per_channel", ctypes.c_size_t),
                ("workspace_bytes_per_row", ctypes.c_size_t),
                ("mfma_flops_per_row", ctypes.c_double),
                ("kernel_variant", ctypes.c_int),
                ("sparse_outer", ctypes.c_int),
                ("circular", ctypes.c_int)]

    def as_dict(self) -> dict:
        return {"N": self.N, "M": self.M, "order": self.order,
                "factors": list(self.factors[:self.order]),
                "path": "fused" if self.path == 0 else "multipass",
                "outer_factors": self.outer_factors,
                "dtype": {v: k for k, v in DTYPES.items()}[self.dtype],
                "spectrum_bytes_per_channel": self.spectrum_bytes_per_channel,
                "workspace_bytes_per_row": self.workspace_bytes_per_row,
                "mfma_flops_per_row": self.mfma_flops_per_row,
                "sparse_outer": self.sparse_outer,
                "circular": bool(self.circular),
                "kernel": {0: "fused_kernel", 1: "row_kernel", 3: "wide_kernel",
                           # one outer level: per-column passes; two: both
                           # levels in one column pass each way (on the
                           # matrix cores when both are 32)
                           4: ("mp_col_kernel+mp_inner_kernel"
                               if self.outer_factors <= 1 else
                               "mp_col2m_fwd_kernel+mp_inner_kernel+mp_col2m_inv_kernel"
                               if list(self.factors[:2]) == [32, 32] else
                               "mp_col2_kernel+mp_inner_kernel"),
                           2: "outer_fwd_kernel+inner_kernel+outer_inv_kernel"
                           }[self.kernel_variant]}


# fftconv_kernel_kind values of the C header
KERNEL_KINDS = {"causal": 0, "causal_adjoint": 1, "circular": 2,
                "circular_adjoint": 3}


def lib() -> ctypes.CDLL:
    """Open libfftconv.so (built in-tree by fft_long_convolution_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libfftconv.so is not built; run "
                "'python -m fft_long_convolution_amd.build'")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.fftconv_plan.argtypes = [sz, i, i, ctypes.POINTER(vp)]
        L.fftconv_plan.restype = i
        L.fftconv_plan_query.argtypes = [sz, i, i, ctypes.POINTER(PlanInfo)]
        L.fftconv_plan_query.restype = i
        L.fftconv_plan_circular.argtypes = [sz, i, i, ctypes.POINTER(vp)]
        L.fftconv_plan_circular.restype = i
        L.fftconv_plan_circular_query.argtypes = [sz, i, i, ctypes.POINTER(PlanInfo)]
        L.fftconv_plan_circular_query.restype = i
        L.fftconv_plan_estimate.argtypes = [sz, i, i, i, sz, sz, ctypes.POINTER(Estimate)]
        L.fftconv_plan_estimate.restype = i
        L.fftconv_plan_get_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
        L.fftconv_plan_get_info.restype = i
        L.fftconv_plan_destroy.argtypes = [vp]
        L.fftconv_plan_destroy.restype = None
        L.fftconv_spectrum_bytes.argtypes = [vp, sz]
        L.fftconv_spectrum_bytes.restype = sz
        L.fftconv_workspace_bytes.argtypes = [vp, sz, sz]
        L.fftconv_workspace_bytes.restype = sz
        L.fftconv_kernel_spectrum.argtypes = [vp, vp, sz, vp, vp]
        L.fftconv_kernel_spectrum.restype = i
        L.fftconv_kernel_spectrum_lowpass.argtypes = [vp, vp, sz, sz, vp, vp]
        L.fftconv_kernel_spectrum_lowpass.restype = i
        L.fftconv_forward_lowpass.argtypes = [vp, vp, vp, sz, vp, sz, sz, sz,
                                              vp, sz, vp]
        L.fftconv_forward_lowpass.restype = i
        L.fftconv_kernel_spectrum_blocksparse.argtypes = [vp, vp, sz, i, i, vp, vp]
        L.fftconv_kernel_spectrum_blocksparse.restype = i
        L.fftconv_forward_blocksparse.argtypes = [vp, vp, vp, i, i, vp, sz, sz, sz, vp, sz, vp]
        L.fftconv_forward_blocksparse.restype = i
        L.fftconv_kernel_spectrum_kind.argtypes = [vp, vp, sz, i, vp, vp]
        L.fftconv_kernel_spectrum_kind.restype = i
        L.fftconv_forward.argtypes = [vp, vp, vp, vp, sz, sz, sz, vp, sz, vp]
        L.fftconv_forward.restype = i
        L.fftconv_forward_noalloc.argtypes = [vp, vp, vp, vp, sz, sz, sz, vp]
        L.fftconv_forward_noalloc.restype = i
        L.fftconv_forward_gated.argtypes = [vp, vp, vp, vp, vp, vp, sz, sz,
                                            sz, vp, sz, vp]
        L.fftconv_forward_gated.restype = i
        L.fftconv_backward_workspace_bytes.argtypes = [vp, sz, sz]
        L.fftconv_backward_workspace_bytes.restype = sz
        L.fftconv_backward.argtypes = [vp, vp, vp, vp, vp, vp, sz, sz, sz,
                                       vp, sz, vp]
        L.fftconv_backward.restype = i
        L.fftconv_stream_copy.argtypes = [vp, vp, sz, vp]
        L.fftconv_stream_copy.restype = i
        L.fftconv_status_string.argtypes = [i]
        L.fftconv_status_string.restype = ctypes.c_char_p
        L.fftconv_version.argtypes = []
        L.fftconv_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def plan_query(N: int, p: int = 0, dtype: str = "bf16", circular: bool = False) -> dict:
    """What fftconv_plan(N, p, dtype) -- or, circular=True,
    fftconv_plan_circular -- would build (no device needed)."""
    info = PlanInfo()
    fn = lib().fftconv_plan_circular_query if circular else lib().fftconv_plan_query
    st = fn(N, p, DTYPES[dtype], ctypes.byref(info))
    if st != 0:
        raise FFTConvError(st, "plan query (N=%d, p=%d, circular=%s)" % (N, p, circular))
    return info.as_dict()


class Estimate(ctypes.Structure):
    _fields_ = [("order", ctypes.c_int), ("factors", ctypes.c_int * 8),
                ("path", ctypes.c_int), ("kernel_variant", ctypes.c_int),
                ("hbm_bytes", ctypes.c_double), ("mfma_flops", ctypes.c_double),
                ("valu_flops", ctypes.c_double), ("lds_bytes", ctypes.c_double),
                ("t_hbm", ctypes.c_double), ("t_mfma", ctypes.c_double),
                ("t_valu", ctypes.c_double), ("t_lds", ctypes.c_double),
                ("t_pred", ctypes.c_double)]

    def as_dict(self) -> dict:
        d = {k: getattr(self, k) for k, _ in self._fields_ if k != "factors"}
        d["factors"] = list(self.factors[:self.order])
        return d


def plan_estimate(N: int, p: int = 0, dtype: str = "bf16", lds_staged: bool = False,
                  B: int = 1, H: int = 1) -> dict:
    """fftconv_plan_estimate: the cost model's prediction for one forward
    call over B x H rows (no device needed)."""
    e = Estimate()
    st = lib().fftconv_plan_estimate(N, p, DTYPES[dtype], 1 if lds_staged else 0,
                                     B, H, ctypes.byref(e))
    if st != 0:
        raise FFTConvError(st, "fftconv_plan_estimate(N=%d, p=%d)" % (N, p))
    return e.as_dict()


def stream_copy(src, dst, stream=None):
    """fftconv_stream_copy of a contiguous CUDA tensor into another of the
    same byte size (non-temporal 16-byte loads and stores)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same size in bytes")
    st = lib().fftconv_stream_copy(src.data_ptr(), dst.data_ptr(), nbytes,
                                   _stream_handle(stream))
    if st != 0:
        raise FFTConvError(st, "fftconv_stream_copy")
    return dst


def _torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16,
            "bf16": torch.bfloat16}[dtype]


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class FFTConv:
    """FFT long convolution for one (N, order, dtype) plan.

    >>> conv = FFTConv(1024, dtype="bf16")
    >>> k_f = conv.kernel_spectrum(k)          # k: [H, N] fp32, once
    >>> y = conv.forward(u, k_f)               # u: [B, H, N] bf16

    circular=True builds the plan of the circular operators at FFT size N
    (fftconv_plan_circular): kernel_spectrum then takes kind="circular" or
    "circular_adjoint".
    """

    def __init__(self, N: int, p: int = 0, dtype: str = "bf16", circular: bool = False):
        if dtype not in DTYPES:
            raise ValueError("dtype must be one of %s" % list(DTYPES))
        import torch
        if not torch.cuda.is_available():
            raise RuntimeError("FFTConv needs a ROCm GPU")
        self.N, self.dtype, self.circular = N, dtype, circular
        h = ctypes.c_void_p()
        fn = lib().fftconv_plan_circular if circular else lib().fftconv_plan
        st = fn(N, p, DTYPES[dtype], ctypes.byref(h))
        if st != 0:
            raise FFTConvError(st, "plan (N=%d, p=%d, %s, circular=%s)" % (N, p, dtype, circular))
        self._plan = h
        info = PlanInfo()
        lib().fftconv_plan_get_info(h, ctypes.byref(info))
        self.info = info.as_dict()
        self.device = torch.cuda.current_device()

    def close(self):
        if getattr(self, "_plan", None):
            lib().fftconv_plan_destroy(self._plan)
            self._plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def spectrum_bytes(self, H: int) -> int:
        return int(lib().fftconv_spectrum_bytes(self._plan, H))

    def workspace_bytes(self, B: int, H: int) -> int:
        return int(lib().fftconv_workspace_bytes(self._plan, B, H))

    def kernel_spectrum_lowpass(self, k, cutoff: int, out=None, stream=None):
        """Band-limited spectrum of the causal kernel k ([H, N] fp32): kept
        at frequencies within `cutoff` of zero (of the 2N-point transform)."""
        import torch
        if k.dtype != torch.float32 or k.dim() != 2 or k.shape[1] != self.N:
            raise ValueError("k must be fp32 [H, %d]" % self.N)
        k = k.contiguous()
        H = k.shape[0]
        nb = self.spectrum_bytes(H)
        if out is None:
            out = torch.empty(nb, dtype=torch.uint8, device=k.device)
        st = lib().fftconv_kernel_spectrum_lowpass(self._plan, k.data_ptr(), H,
                                                   int(cutoff), out.data_ptr(),
                                                   _stream_handle(stream))
        if st != 0:
            raise FFTConvError(st, "fftconv_kernel_spectrum_lowpass")
        return out

    def forward_lowpass(self, u, k_f, cutoff: int, out=None, workspace=None,
                        stream=None):
        """The frequency-sparse convolution (k_f from kernel_spectrum_lowpass
        with the same cutoff)."""
        u = u.contiguous()
        out, ws_ptr, ws_bytes = self._prepare(u, out, workspace)
        B, H, N = u.shape
        st = lib().fftconv_forward_lowpass(self._plan, u.data_ptr(),
                                           k_f.data_ptr(), int(cutoff),
                                           out.data_ptr(), B, H, N, ws_ptr,
                                           ws_bytes, _stream_handle(stream))
        if st != 0:
            raise FFTConvError(st, "fftconv_forward_lowpass")
        return out

    def kernel_spectrum_blocksparse(self, k, a: int, d: int, out=None, stream=None):
        """Spectrum of the causal kernel k ([H, N] fp32) with the digit-block
        zero pattern (a middle values of the top digit, d outer classes)."""
        import torch
        if k.dtype != torch.float32 or k.dim() != 2 or k.shape[1] != self.N:
            raise ValueError("k must be fp32 [H, %d]" % self.N)
        k = k.contiguous()
        H = k.shape[0]
        if out is None:
            out = torch.empty(self.spectrum_bytes(H), dtype=torch.uint8, device=k.device)
        st = lib().fftconv_kernel_spectrum_blocksparse(self._plan, k.data_ptr(), H, int(a),
                                                       int(d), out.data_ptr(),
                                                       _stream_handle(stream))
        if st != 0:
            raise FFTConvError(st, "fftconv_kernel_spectrum_blocksparse")
        return out

    def forward_blocksparse(self, u, k_f, a: int, d: int, out=None, workspace=None,
                            stream=None):
        """The frequency-sparse convolution with zero blocks along the digits
        (k_f from kernel_spectrum_blocksparse with the same a, d)."""
        u = u.contiguous()
        out, ws_ptr, ws_bytes = self._prepare(u, out, workspace)
        B, H, N = u.shape
        st = lib().fftconv_forward_blocksparse(self._plan, u.data_ptr(), k_f.data_ptr(),
                                               int(a), int(d), out.data_ptr(), B, H, N,
                                               ws_ptr, ws_bytes, _stream_handle(stream))
        if st != 0:
            raise FFTConvError(st, "fftconv_forward_blocksparse")
        return out

    def kernel_spectrum(self, k, out=None, stream=None, kind=None):
        """k: [H, N] fp32 CUDA tensor -> opaque k_f (uint8 CUDA tensor).
        kind: "causal", "causal_adjoint", "circular" or "circular_adjoint"
        (the operator fftconv_forward then computes); by default "causal",
        or "circular" on a circular plan."""
        import torch
        if kind is None:
            kind = "circular" if self.circular else "causal"
        if k.dtype != torch.float32 or k.dim() != 2 or k.shape[1] != self.N:
            raise ValueError("k must be fp32 [H, %d]" % self.N)
        k = k.contiguous()
        H = k.shape[0]
        nb = self.spectrum_bytes(H)
        if out is None:
            out = torch.empty(nb, dtype=torch.uint8, device=k.device)
        elif out.numel() * out.element_size() < nb:
            raise ValueError("k_f buffer too small")
        if kind not in KERNEL_KINDS:
            raise ValueError("unknown kernel kind %r" % (kind,))
        st = lib().fftconv_kernel_spectrum_kind(self._plan, k.data_ptr(), H,
                                                KERNEL_KINDS[kind],
                                                out.data_ptr(),
                                                _stream_handle(stream))
        if st != 0:
            raise FFTConvError(st, "fftconv_kernel_spectrum_kind")
        return out

    def _prepare(self, u, out, workspace):
        import torch
        if u.dim() != 3 or u.shape[2] != self.N:
            raise ValueError("u must be [B, H, %d]" % self.N)
        if u.dtype != _torch_dtype(self.dtype):
            raise ValueError("u dtype must be %s" % self.dtype)
        B, H, N = u.shape
        if out is None:
            out = torch.empty_like(u)
        elif out.shape != u.shape or out.dtype != u.dtype:
            raise ValueError("out must match u")
        need = self.workspace_bytes(B, H)
        ws_ptr, ws_bytes = None, 0
        if need:
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8,
                                        device=u.device)
            ws_ptr = workspace.data_ptr()
            ws_bytes = workspace.numel() * workspace.element_size()
        return out, ws_ptr, ws_bytes

    def forward(self, u, k_f, out=None, workspace=None, stream=None):
        """u: [B, H, N] CUDA tensor of the plan dtype -> y (same shape)."""
        u = u.contiguous()
        out, ws_ptr, ws_bytes = self._prepare(u, out, workspace)
        B, H, N = u.shape
        st = lib().fftconv_forward(self._plan, u.data_ptr(), k_f.data_ptr(),
                                   out.data_ptr(), B, H, N, ws_ptr, ws_bytes,
                                   _stream_handle(stream))
        if st != 0:
            raise FFTConvError(st, "fftconv_forward")
        return out

    def forward_noalloc(self, u, k_f, out, stream=None):
        """fftconv_forward_noalloc: y into the caller's `out` ([B, H, N],
        plan dtype) with the library's static scratch as the workspace."""
        u = u.contiguous()
        if out.shape != u.shape or out.dtype != u.dtype or not out.is_contiguous():
            raise ValueError("out must be a contiguous tensor of u's shape and dtype")
        B, H, N = u.shape
        st = lib().fftconv_forward_noalloc(self._plan, u.data_ptr(), k_f.data_ptr(),
                                           out.data_ptr(), B, H, N,
                                           _stream_handle(stream))
        if st != 0:
            raise FFTConvError(st, "fftconv_forward_noalloc")
        return out

    def forward_gated(self, u, w, v, k_f, out=None, workspace=None,
                      stream=None):
        """y = v * conv(u * w, k): u, w, v are [B, H, N] CUDA tensors of the
        plan dtype; returns y (same shape)."""
        u = u.contiguous()
        w = w.contiguous()
        v = v.contiguous()
        if w.shape != u.shape or v.shape != u.shape:
            raise ValueError("gates must have the shape of u")
        if w.dtype != u.dtype or v.dtype != u.dtype:
            raise ValueError("gates must have the dtype of u")
        out, ws_ptr, ws_bytes = self._prepare(u, out, workspace)
        B, H, N = u.shape
        st = lib().fftconv_forward_gated(
            self._plan, u.data_ptr(), w.data_ptr(), v.data_ptr(),
            k_f.data_ptr(), out.data_ptr(), B, H, N, ws_ptr, ws_bytes,
            _stream_handle(stream))
        if st != 0:
            raise FFTConvError(st, "fftconv_forward_gated")
        return out

    def backward_workspace_bytes(self, B: int, H: int) -> int:
        return int(lib().fftconv_backward_workspace_bytes(self._plan, B, H))

    def backward(self, u, dy, k_f_adj, need_du=True, need_dk=True,
                 workspace=None, stream=None, out_du=None, out_dk=None):
        """Gradients of the causal convolution: returns (du, dk) for
        dy = dL/dy ([B, H, N], plan dtype); k_f_adj from
        kernel_spectrum(k, kind="causal_adjoint").  du has u's shape and
        dtype, dk is fp32 [H, N]; either may be skipped (None)."""
        import torch
        if dy.dim() != 3 or dy.shape[2] != self.N:
            raise ValueError("dy must be [B, H, %d]" % self.N)
        if dy.dtype != _torch_dtype(self.dtype):
            raise ValueError("dy dtype must be %s" % self.dtype)
        if not (need_du or need_dk):
            raise ValueError("nothing to compute")
        dy = dy.contiguous()
        B, H, N = dy.shape
        if need_dk:
            if u is None or u.shape != dy.shape or u.dtype != dy.dtype:
                raise ValueError("u must match dy")
            u = u.contiguous()
        du = dk = None
        if need_du:
            du = torch.empty_like(dy) if out_du is None else out_du
            if du.shape != dy.shape or du.dtype != dy.dtype:
                raise ValueError("out_du must match dy")
        if need_dk:
            dk = (torch.empty(H, N, dtype=torch.float32, device=dy.device)
                  if out_dk is None else out_dk)
            if dk.shape != (H, N) or dk.dtype != torch.float32:
                raise ValueError("out_dk must be fp32 [H, N]")
        need = self.backward_workspace_bytes(B, H)
        ws_ptr, ws_bytes = None, 0
        if need:
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8,
                                        device=dy.device)
            ws_ptr = workspace.data_ptr()
            ws_bytes = workspace.numel() * workspace.element_size()
        st = lib().fftconv_backward(
            self._plan, u.data_ptr() if need_dk else None, dy.data_ptr(),
            k_f_adj.data_ptr() if need_du else None,
            du.data_ptr() if need_du else None,
            dk.data_ptr() if need_dk else None, B, H, N, ws_ptr, ws_bytes,
            _stream_handle(stream))
        if st != 0:
            raise FFTConvError(st, "fftconv_backward")
        return du, dk
