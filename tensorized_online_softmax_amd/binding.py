"""ctypes binding of libtos.so (include/tos.h): argument marshalling only.

Every step of the attention pass runs in the library's HIP kernels.  torch is
used only to hand over device memory and the current HIP stream.  The binding
raises if the built library is missing; there is no other code path.
"""
import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtos.so")

TOS_OK, TOS_ERR_INVALID_ARG, TOS_ERR_UNSUPPORTED, TOS_ERR_HIP, TOS_ERR_SCRATCH = 0, 1, 2, 3, 4
TOS_F32, TOS_BF16, TOS_FP8_E4M3, TOS_F16 = 0, 1, 2, 3
(TOS_SPLIT_VALU, TOS_SPLIT_ROWSUM_MFMA, TOS_SPLIT_SCALE_MFMA, TOS_SPLIT_HSPLIT, TOS_SPLIT_VSPLIT,
 TOS_SPLIT_ALL_MFMA) = range(6)
TOS_FALLBACK_OFF, TOS_FALLBACK_AUTO, TOS_FALLBACK_FORCE = 0, 1, 2
TOS_SCHEDULE_COSCHED, TOS_SCHEDULE_SEQUENTIAL = 0, 1

EXPORTED = ("tos_attn_fwd", "tos_attn_fwd_noalloc", "tos_fwd_opts_default", "tos_attn_fwd_flops",
            "tos_attn_fwd_workspace_size", "tos_status_string", "tos_version")


class tos_fwd_opts(ctypes.Structure):
    _fields_ = [("size", ctypes.c_int), ("x_tile", ctypes.c_int),
                ("softmax_split", ctypes.c_int), ("fallback", ctypes.c_int),
                ("fallback_tau", ctypes.c_float), ("q_descale", ctypes.c_float),
                ("k_descale", ctypes.c_float), ("v_descale", ctypes.c_float),
                ("fallback_tiles", ctypes.c_void_p), ("schedule", ctypes.c_int),
                ("split_num", ctypes.c_int), ("split_den", ctypes.c_int),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("trace", ctypes.c_void_p), ("trace_bytes", ctypes.c_size_t)]


class TosError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(tos_status_string(status))


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        # torch first: libtos.so must bind to the HIP runtime torch already
        # loaded (same soname), so that torch's streams and allocations are
        # valid handles for the library's launches
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        L.tos_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                   ctypes.c_float, ctypes.c_int, ctypes.POINTER(tos_fwd_opts), vp]
        L.tos_attn_fwd.restype = ctypes.c_int
        L.tos_attn_fwd_noalloc.argtypes = L.tos_attn_fwd.argtypes
        L.tos_attn_fwd_noalloc.restype = ctypes.c_int
        L.tos_fwd_opts_default.argtypes = [ctypes.POINTER(tos_fwd_opts)]
        L.tos_fwd_opts_default.restype = ctypes.c_int
        L.tos_attn_fwd_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                                  ctypes.POINTER(tos_fwd_opts),
                                                  ctypes.POINTER(ctypes.c_size_t)]
        L.tos_attn_fwd_workspace_size.restype = ctypes.c_int
        L.tos_attn_fwd_flops.argtypes = [i64, i64, i64, i64, ctypes.c_int]
        L.tos_attn_fwd_flops.restype = ctypes.c_double
        L.tos_status_string.argtypes = [ctypes.c_int]
        L.tos_status_string.restype = ctypes.c_char_p
        L.tos_version.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(x):
    """A device pointer from a torch tensor, an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def tos_fwd_opts_default():
    o = tos_fwd_opts()
    rc = lib().tos_fwd_opts_default(ctypes.byref(o))
    if rc != TOS_OK:
        raise TosError(rc)
    return o


def tos_attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, opts=None, stream=None):
    """Direct call of the C entry point; returns the tos_status code."""
    return lib().tos_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                              int(N), int(d), int(causal), float(scale), int(dtype),
                              ctypes.byref(opts) if opts is not None else None, _stream(stream))


def tos_attn_fwd_noalloc(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, opts=None,
                         stream=None):
    """Direct call of the allocation-free entry point; returns the tos_status code."""
    return lib().tos_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B),
                                      int(H), int(N), int(d), int(causal), float(scale),
                                      int(dtype), ctypes.byref(opts) if opts is not None else None,
                                      _stream(stream))


def tos_attn_fwd_workspace_size(B, H, N, d, causal, dtype, opts=None):
    """Bytes of device workspace tos_attn_fwd would use (0: none); raises TosError."""
    n = ctypes.c_size_t(0)
    rc = lib().tos_attn_fwd_workspace_size(int(B), int(H), int(N), int(d), int(causal), int(dtype),
                                           ctypes.byref(opts) if opts is not None else None,
                                           ctypes.byref(n))
    if rc != TOS_OK:
        raise TosError(rc)
    return int(n.value)


_workspaces = {}


def workspace(nbytes, device):
    """A cached device buffer of at least nbytes on `device` (torch allocates it;
    the library allocates nothing).  Calls on one device share it, in stream
    order on the stream they are launched on."""
    import torch
    key = str(device)
    buf = _workspaces.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        _workspaces[key] = buf
    return buf


def tos_attn_fwd_flops(B, H, N, d, causal):
    return float(lib().tos_attn_fwd_flops(int(B), int(H), int(N), int(d), int(causal)))


def tos_status_string(status):
    return lib().tos_status_string(int(status)).decode()


def tos_version():
    return int(lib().tos_version())


_DTYPE_CODES = {"f32": TOS_F32, "bf16": TOS_BF16, "fp8": TOS_FP8_E4M3, "f16": TOS_F16}
_SPLITS = {"valu": TOS_SPLIT_VALU, "rowsum_mfma": TOS_SPLIT_ROWSUM_MFMA,
           "scale_mfma": TOS_SPLIT_SCALE_MFMA, "hsplit": TOS_SPLIT_HSPLIT,
           "vsplit": TOS_SPLIT_VSPLIT, "all_mfma": TOS_SPLIT_ALL_MFMA}
_FALLBACKS = {"off": TOS_FALLBACK_OFF, "auto": TOS_FALLBACK_AUTO, "force": TOS_FALLBACK_FORCE}
_SCHEDULES = {"cosched": TOS_SCHEDULE_COSCHED, "sequential": TOS_SCHEDULE_SEQUENTIAL}


def make_opts(x_tile=32, split="valu", fallback="off", tau=0.0, descale=None,
              fallback_tiles=None, schedule="cosched", share=None, trace=None):
    """Options for tos_attn_fwd.  split names a tos_softmax_split value;
    share = (num, den) is the matrix unit's share of it (None: the default)."""
    op = tos_fwd_opts_default()
    if share is not None:
        op.split_num, op.split_den = int(share[0]), int(share[1])
    op.x_tile = int(x_tile)
    op.softmax_split = _SPLITS[split]
    op.fallback = _FALLBACKS[fallback]
    op.fallback_tau = float(tau)
    if descale is not None:
        op.q_descale, op.k_descale, op.v_descale = (float(descale[n]) for n in ("q", "k", "v"))
    op.fallback_tiles = _ptr(fallback_tiles)
    op.schedule = _SCHEDULES[schedule]
    if trace is not None:   # a zeroed uint64 device buffer for the phase stamps
        op.trace, op.trace_bytes = _ptr(trace), trace.numel() * trace.element_size()
    return op


def _torch_dtypes():
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
            "fp8": torch.float8_e4m3fn}


def out_dtype(dtype):
    """torch dtype of O for an input dtype name (fp8 inputs give bf16 O)."""
    import torch
    return {"f32": torch.float32, "f16": torch.float16}.get(dtype, torch.bfloat16)


def check_tensors(q, k, v, dtype=None, out=None, lse=None, fallback_tiles=None):
    """Checks what the C ABI cannot see from raw pointers, before any launch:
    q, k, v are contiguous [B, H, N, d] tensors of the named dtype on one CUDA
    device; out (if given) is a contiguous [B, H, N, d] tensor of O's dtype there;
    lse (if given) a contiguous float32 [B, H, N] tensor there; fallback_tiles
    (if given) an int32 tensor of at least one element there.  Raises
    ValueError on any mismatch; returns (B, H, N, d, dtype name)."""
    tdt = _torch_dtypes()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not hasattr(t, "dim") or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D tensor [B, H, N, d]")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)}, {tuple(k.shape)}, "
                         f"{tuple(v.shape)}")
    if dtype is None:
        inv = {t: n for n, t in tdt.items()}
        if q.dtype not in inv:
            raise ValueError(f"unsupported input dtype {q.dtype}")
        dtype = inv[q.dtype]
    if dtype not in tdt:
        raise ValueError(f"unknown dtype name {dtype!r}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != tdt[dtype]:
            raise ValueError(f"{name} is {t.dtype}, dtype {dtype!r} needs {tdt[dtype]}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous (got strides {t.stride()})")
    B, H, N, d = (int(x) for x in q.shape)
    if out is not None:
        if tuple(out.shape) != (B, H, N, d) or out.dtype != out_dtype(dtype):
            raise ValueError(f"out must be {out_dtype(dtype)} [B, H, N, d] = {(B, H, N, d)}, "
                             f"got {out.dtype} {tuple(out.shape)}")
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
    if lse is not None:
        import torch
        if tuple(lse.shape) != (B, H, N) or lse.dtype != torch.float32:
            raise ValueError(f"lse must be float32 [B, H, N] = {(B, H, N)}, "
                             f"got {lse.dtype} {tuple(lse.shape)}")
        if not lse.is_contiguous():
            raise ValueError("lse must be contiguous")
    if fallback_tiles is not None and not isinstance(fallback_tiles, int):
        import torch
        if fallback_tiles.dtype != torch.int32 or fallback_tiles.numel() < 1:
            raise ValueError("fallback_tiles must be an int32 tensor of at least one element")
    tensors = [("q", q), ("k", k), ("v", v)] + [(n, t) for n, t in (
        ("out", out), ("lse", lse), ("fallback_tiles", fallback_tiles))
        if t is not None and not isinstance(t, int)]
    for name, t in tensors:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA (HIP) tensor, got device {t.device}")
    devs = {t.device for _, t in tensors}
    if len(devs) != 1:
        raise ValueError(f"every tensor must be on one device, got {sorted(map(str, devs))}")
    return B, H, N, d, dtype


def attn_fwd(q, k, v, causal=False, scale=None, dtype=None, x_tile=32, split="valu",
             fallback="off", tau=0.0, descale=None, with_lse=True, fallback_tiles=None,
             out=None, lse=None, stream=None, schedule="cosched", share=None,
             use_workspace=True, trace=None):
    """Allocate O (and lse) with torch and run tos_attn_fwd on the current stream.

    With use_workspace (the default) a problem with fewer query blocks than
    compute units gets the device workspace tos_attn_fwd_workspace_size asks
    for (a cached torch buffer), so that its query blocks' keys are cut into
    pieces across the compute units; use_workspace=False runs whole blocks.

    q, k, v: contiguous CUDA tensors [B, H, N, d] of float32, bfloat16, float16
    or float8_e4m3fn (then `descale` = {"q":..., "k":..., "v":...} is required).
    Returns (o, lse); lse is None when with_lse is False.
    """
    import torch
    B, H, N, d, dtype = check_tensors(q, k, v, dtype, out, lse if with_lse else None,
                                      fallback_tiles)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = out if out is not None else torch.empty((B, H, N, d), dtype=out_dtype(dtype),
                                                device=q.device)
    if with_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if not with_lse:
        lse = None
    op = make_opts(x_tile, split, fallback, tau, descale, fallback_tiles, schedule, share, trace)
    if use_workspace:
        nbytes = tos_attn_fwd_workspace_size(B, H, N, d, causal, _DTYPE_CODES[dtype], op)
        if nbytes > 0:
            op.workspace = workspace(nbytes, q.device).data_ptr()
            op.workspace_bytes = nbytes
    rc = tos_attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, _DTYPE_CODES[dtype], op,
                      stream)
    if rc != TOS_OK:
        raise TosError(rc)
    return o, lse
