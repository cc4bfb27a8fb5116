"""ctypes binding of libqknorm.so (argument marshalling only).

The three calls keep the C names. Tensors are torch CUDA tensors used as
device memory: each Q or K operand is a 2-D view whose columns are contiguous
(for instance ``qkv[:, :hq]`` and ``qkv[:, hq:hq + hk]`` of a packed
[T, Hq + Hk + Hv] buffer); its row stride becomes the C ``ld``. The work is
enqueued on torch's current stream of the tensors' device (or on ``stream``).
No step of the computation runs here; if the library is missing, the first
call raises.
"""

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqknorm.so")

QKNORM_F32 = 0
QKNORM_BF16 = 1
QKNORM_FP8_E4M3 = 2
QKNORM_OK = 0
QKNORM_ERR_INVALID_ARG = 1
QKNORM_ERR_UNSUPPORTED = 2
QKNORM_ERR_HIP = 3
OP_FUSED, OP_PARTIAL_STATS, OP_APPLY_WITH_STATS = 0, 1, 2
ABI_VERSION = 3
EXPORTS = ("qknorm_fused", "qknorm_partial_stats", "qknorm_apply_with_stats", "qknorm_headwise",
           "qknorm_last_error", "qknorm_abi_version", "qknorm_describe_plan", "qknorm_describe_headwise_plan")


_DTYPES = {"f32": (QKNORM_F32, 4), "bf16": (QKNORM_BF16, 2), "fp8": (QKNORM_FP8_E4M3, 1)}


class QKNormError(RuntimeError):
    """A non-OK status from libqknorm.so; ``status`` holds the code."""

    def __init__(self, status, message):
        super().__init__(f"[status {status}] {message}")
        self.status = status


class Operand(ctypes.Structure):
    """qknorm_operand_t."""

    _fields_ = [
        ("x", ctypes.c_void_p),
        ("ld_x", ctypes.c_int64),
        ("y", ctypes.c_void_p),
        ("ld_y", ctypes.c_int64),
        ("gamma", ctypes.c_void_p),
        ("h", ctypes.c_int64),
    ]


_lock = threading.Lock()
_lib = None


def library_path():
    return _LIB_PATH


def load_library():
    """Loads libqknorm.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:   # loaded: no lock needed to read the reference
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise QKNormError(-1, f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                                  "(hipcc --offload-arch=gfx950)")
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER(Operand)
        i64, vp, fl, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
        lib.qknorm_fused.argtypes = [P, P, i64, ci, fl, ci, vp]
        lib.qknorm_partial_stats.argtypes = [P, P, i64, ci, ci, vp, vp]
        lib.qknorm_apply_with_stats.argtypes = [P, P, i64, ci, fl, vp, ci, i64, i64, vp]
        lib.qknorm_describe_plan.argtypes = [ci, P, P, i64, ci, ci, ctypes.c_char_p, ctypes.c_size_t]
        lib.qknorm_headwise.argtypes = [P, P, i64, ci, fl, i64, i64, vp]
        lib.qknorm_describe_headwise_plan.argtypes = [P, P, i64, ci, i64, i64, ctypes.c_char_p, ctypes.c_size_t]
        for fn in ("qknorm_fused", "qknorm_partial_stats", "qknorm_apply_with_stats", "qknorm_headwise",
                   "qknorm_describe_plan", "qknorm_describe_headwise_plan", "qknorm_abi_version"):
            getattr(lib, fn).restype = ci
        lib.qknorm_last_error.restype = ctypes.c_char_p
        lib.qknorm_last_error.argtypes = []
        lib.qknorm_abi_version.argtypes = []
        if lib.qknorm_abi_version() != ABI_VERSION:
            raise QKNormError(-1, f"libqknorm.so ABI {lib.qknorm_abi_version()} != {ABI_VERSION}")
        _lib = lib
        return lib


def abi_version():
    return load_library().qknorm_abi_version()


def _check(rc):
    if rc != QKNORM_OK:
        raise QKNormError(rc, load_library().qknorm_last_error().decode())


# --------------------------------------------------------------------- marshalling
_torch = None
_CODES = {}


def _torch_mod():
    global _torch
    if _torch is None:
        import torch
        _CODES.update({torch.bfloat16: QKNORM_BF16, torch.float32: QKNORM_F32,
                       torch.float8_e4m3fn: QKNORM_FP8_E4M3})
        _torch = torch
    return _torch


def _dtype_code(t):
    _torch_mod()
    code = _CODES.get(t.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {t.dtype} (bfloat16, float32 or float8_e4m3fn)")
    return code


def _gamma_dtype(x):
    """gamma is bf16 for FP8 rows, the row dtype otherwise."""
    torch = _torch_mod()
    return torch.bfloat16 if x.dtype == torch.float8_e4m3fn else x.dtype


def _rows(t, name):
    shape, st = t.shape, t.stride()
    if len(shape) != 2:
        raise ValueError(f"{name} must be 2-D [T, h], got {tuple(shape)}")
    if shape[1] > 1 and st[1] != 1:
        raise ValueError(f"{name} columns must be contiguous (stride(1) == 1)")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    # one-row (or empty) views can carry any stride(0); the row length is a valid ld
    return st[0] if shape[0] > 1 else max(st[0], shape[1])


def _same_device(t, ref, name):
    """Every tensor a call hands to the library must be device memory of the
    q tensor's GPU: a host pointer reaching a kernel faults the GPU."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.get_device() != ref.get_device():
        raise ValueError(f"{name} is on device {t.get_device()}, q on device {ref.get_device()}")


def _operand(x, y, gamma, name):
    op = Operand()
    op.ld_x = _rows(x, name)
    shape = x.shape
    op.x = x.data_ptr()
    op.h = shape[1]
    if y is not None:
        if y.shape != shape:
            raise ValueError(f"output for {name} has shape {tuple(y.shape)}, expected {tuple(shape)}")
        op.ld_y = _rows(y, "output for " + name)
        _same_device(y, x, "output for " + name)
        if y.dtype != x.dtype:
            raise TypeError(f"output for {name} must have dtype {x.dtype}")
        op.y = y.data_ptr()
    if gamma is not None:
        gs = gamma.shape
        if len(gs) != 1 or gs[0] != shape[1] or (gs[0] > 1 and gamma.stride(0) != 1):
            raise ValueError(f"gamma for {name} must be contiguous [{shape[1]}]")
        if gamma.dtype != _gamma_dtype(x):
            raise TypeError(f"gamma for {name} must have dtype {_gamma_dtype(x)}")
        _same_device(gamma, x, "gamma for " + name)
        op.gamma = gamma.data_ptr()
    return op


def _stream(t, stream):
    torch = _torch_mod()
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:   # the current stream's handle without building a Stream object
        return raw(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _tokens(q, k):
    if q.shape[0] != k.shape[0]:
        raise ValueError(f"q has {q.shape[0]} rows, k has {k.shape[0]}")
    if q.dtype != k.dtype:
        raise TypeError("q and k must have the same dtype")
    if q.get_device() != k.get_device():
        raise ValueError("q and k must be on the same device")
    return q.shape[0]


def qknorm_fused(q, k, gamma_q, gamma_k, eps, shards=1, out_q=None, out_k=None, stream=None):
    """Layerwise QK-Norm of q [T, hq] and k [T, hk] in one kernel.

    Writes ``out_q``/``out_k`` (default: in place into q and k) and returns them.
    """
    lib = load_library()
    T = _tokens(q, k)
    out_q = q if out_q is None else out_q
    out_k = k if out_k is None else out_k
    oq = _operand(q, out_q, gamma_q, "q")
    ok = _operand(k, out_k, gamma_k, "k")
    _check(lib.qknorm_fused(ctypes.byref(oq), ctypes.byref(ok), T, _dtype_code(q), float(eps),
                            int(shards), _stream(q, stream)))
    return out_q, out_k


def qknorm_partial_stats(q, k, shards, partials=None, stream=None):
    """Per-shard float32 sums of squares -> ``partials`` [S, 2, T] (allocated if None)."""
    import torch
    lib = load_library()
    T = _tokens(q, k)
    if partials is None:
        partials = torch.empty((shards, 2, T), dtype=torch.float32, device=q.device)
    if (partials.dtype != torch.float32 or tuple(partials.shape) != (shards, 2, T)
            or not partials.is_contiguous()):
        raise ValueError(f"partials must be contiguous float32 [{shards}, 2, {T}]")
    oq = _operand(q, None, None, "q")
    _same_device(partials, q, "partials")
    ok = _operand(k, None, None, "k")
    _check(lib.qknorm_partial_stats(ctypes.byref(oq), ctypes.byref(ok), T, _dtype_code(q), int(shards),
                                    partials.data_ptr(), _stream(q, stream)))
    return partials


def qknorm_apply_with_stats(q, k, gamma_q, gamma_k, eps, stats, hq_full, hk_full,
                            out_q=None, out_k=None, stream=None):
    """Scale q/k with statistic planes ``stats`` [P, 2, T] (float32, added in order)
    over full widths ``hq_full``/``hk_full``. Returns the outputs (default in place)."""
    import torch
    lib = load_library()
    T = _tokens(q, k)
    if stats.dim() != 3 or stats.shape[1] != 2 or stats.shape[2] != T or stats.dtype != torch.float32 \
            or not stats.is_contiguous():
        raise ValueError(f"stats must be contiguous float32 [P, 2, {T}]")
    _rows(q, "q")
    _same_device(stats, q, "stats")
    out_q = q if out_q is None else out_q
    out_k = k if out_k is None else out_k
    oq = _operand(q, out_q, gamma_q, "q")
    ok = _operand(k, out_k, gamma_k, "k")
    _check(lib.qknorm_apply_with_stats(ctypes.byref(oq), ctypes.byref(ok), T, _dtype_code(q), float(eps),
                                       stats.data_ptr(), int(stats.shape[0]), int(hq_full), int(hk_full),
                                       _stream(q, stream)))
    return out_q, out_k


def qknorm_headwise(q, k, gamma_q, gamma_k, eps, head_dim, gamma_head_stride=0, out_q=None, out_k=None,
                    stream=None):
    """Headwise QK-Norm of q [T, hq] and k [T, hk]: every head of ``head_dim``
    columns normalized on its own. gamma element (head, j) is
    gamma[head * gamma_head_stride + j] (0: one [head_dim] vector shared by all
    heads). Writes ``out_q``/``out_k`` (default: in place) and returns them."""
    lib = load_library()
    T = _tokens(q, k)
    out_q = q if out_q is None else out_q
    out_k = k if out_k is None else out_k
    oq = _operand(q, out_q, None, "q")
    ok = _operand(k, out_k, None, "k")
    for g, o, name in ((gamma_q, oq, "q"), (gamma_k, ok, "k")):
        need = (o.h // head_dim - 1) * gamma_head_stride + head_dim if head_dim > 0 else 0
        if g.dim() != 1 or g.shape[0] < need or (g.shape[0] > 1 and g.stride(0) != 1) or g.dtype != _gamma_dtype(q):
            raise ValueError(f"gamma for {name} must be contiguous, dtype {_gamma_dtype(q)}, >= {need} elements")
        _same_device(g, q, "gamma for " + name)
        o.gamma = g.data_ptr()
    _check(lib.qknorm_headwise(ctypes.byref(oq), ctypes.byref(ok), T, _dtype_code(q), float(eps), int(head_dim),
                               int(gamma_head_stride), _stream(q, stream)))
    return out_q, out_k


class PreparedCall:
    """A library call with its tensors checked and marshalled once.

    Calling it enqueues the same call again, on torch's current stream of the
    tensors' device (or on ``stream``), with no Python-side checks: for
    launch loops over fixed buffers (a decode step's Q/K views, say), where
    the per-call marshalling would cost more host time than the kernel takes
    on the GPU. The library still validates every launch. The caller keeps
    the tensors alive and unchanged in shape, stride and place while the
    object is used (it holds references to them).
    """

    def __init__(self, fn, args, tensors, device, result):
        self._fn = fn
        self._args = args            # ctypes arguments, the stream last
        self._tensors = tensors      # kept alive with the pointers in _args
        self._device = device
        self._result = result
        torch = _torch_mod()
        self._raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)

    def __call__(self, stream=None):
        if stream is not None:
            s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        elif self._raw is not None:
            s = self._raw(self._device)
        else:
            s = _torch_mod().cuda.current_stream(self._device).cuda_stream
        rc = self._fn(*self._args, s)
        if rc != QKNORM_OK:
            _check(rc)
        return self._result


def prepare_fused(q, k, gamma_q, gamma_k, eps, shards=1, out_q=None, out_k=None):
    """qknorm_fused with its arguments checked and marshalled once (PreparedCall)."""
    lib = load_library()
    T = _tokens(q, k)
    out_q = q if out_q is None else out_q
    out_k = k if out_k is None else out_k
    oq = _operand(q, out_q, gamma_q, "q")
    ok = _operand(k, out_k, gamma_k, "k")
    args = (ctypes.byref(oq), ctypes.byref(ok), T, _dtype_code(q), float(eps), int(shards))
    return PreparedCall(lib.qknorm_fused, args, (q, k, gamma_q, gamma_k, out_q, out_k, oq, ok), q.get_device(),
                        (out_q, out_k))


def prepare_apply_with_stats(q, k, gamma_q, gamma_k, eps, stats, hq_full, hk_full, out_q=None, out_k=None):
    """qknorm_apply_with_stats with its arguments checked and marshalled once (PreparedCall)."""
    torch = _torch_mod()
    lib = load_library()
    T = _tokens(q, k)
    if stats.dim() != 3 or stats.shape[1] != 2 or stats.shape[2] != T or stats.dtype != torch.float32 \
            or not stats.is_contiguous():
        raise ValueError(f"stats must be contiguous float32 [P, 2, {T}]")
    _rows(q, "q")
    _same_device(stats, q, "stats")
    out_q = q if out_q is None else out_q
    out_k = k if out_k is None else out_k
    oq = _operand(q, out_q, gamma_q, "q")
    ok = _operand(k, out_k, gamma_k, "k")
    args = (ctypes.byref(oq), ctypes.byref(ok), T, _dtype_code(q), float(eps), stats.data_ptr(),
            int(stats.shape[0]), int(hq_full), int(hk_full))
    return PreparedCall(lib.qknorm_apply_with_stats, args, (q, k, gamma_q, gamma_k, stats, out_q, out_k, oq, ok),
                        q.get_device(), (out_q, out_k))


def prepare_headwise(q, k, gamma_q, gamma_k, eps, head_dim, gamma_head_stride=0, out_q=None, out_k=None):
    """qknorm_headwise with its arguments checked and marshalled once (PreparedCall)."""
    lib = load_library()
    T = _tokens(q, k)
    out_q = q if out_q is None else out_q
    out_k = k if out_k is None else out_k
    oq = _operand(q, out_q, None, "q")
    ok = _operand(k, out_k, None, "k")
    for g, o, name in ((gamma_q, oq, "q"), (gamma_k, ok, "k")):
        need = (o.h // head_dim - 1) * gamma_head_stride + head_dim if head_dim > 0 else 0
        if g.dim() != 1 or g.shape[0] < need or (g.shape[0] > 1 and g.stride(0) != 1) or g.dtype != _gamma_dtype(q):
            raise ValueError(f"gamma for {name} must be contiguous, dtype {_gamma_dtype(q)}, >= {need} elements")
        _same_device(g, q, "gamma for " + name)
        o.gamma = g.data_ptr()
    args = (ctypes.byref(oq), ctypes.byref(ok), T, _dtype_code(q), float(eps), int(head_dim), int(gamma_head_stride))
    return PreparedCall(lib.qknorm_headwise, args, (q, k, gamma_q, gamma_k, out_q, out_k, oq, ok), q.get_device(),
                        (out_q, out_k))


def prepare_partial_stats(q, k, shards, partials):
    """qknorm_partial_stats into ``partials`` [S, 2, T], checked and marshalled once (PreparedCall)."""
    torch = _torch_mod()
    lib = load_library()
    T = _tokens(q, k)
    if (partials.dtype != torch.float32 or tuple(partials.shape) != (shards, 2, T)
            or not partials.is_contiguous()):
        raise ValueError(f"partials must be contiguous float32 [{shards}, 2, {T}]")
    oq = _operand(q, None, None, "q")
    _same_device(partials, q, "partials")
    ok = _operand(k, None, None, "k")
    args = (ctypes.byref(oq), ctypes.byref(ok), T, _dtype_code(q), int(shards), partials.data_ptr())
    return PreparedCall(lib.qknorm_partial_stats, args, (q, k, partials, oq, ok), q.get_device(), partials)


def describe_headwise_plan(hq, hk, T, head_dim, dtype="bf16", gamma_head_stride=0, ld=None):
    """The launch qknorm_headwise would make, for shapes alone (no GPU needed)."""
    lib = load_library()
    code, esz = _DTYPES[dtype]
    ld = ld if ld is not None else hq + hk
    xq, xk = (1 << 32), (1 << 32) + hq * esz if ld >= hq + hk else (1 << 40)
    oq = Operand(xq, ld, xq + (1 << 44), ld, 1 << 46, hq)
    ok = Operand(xk, ld, xk + (1 << 44), ld, (1 << 46) + (1 << 30), hk)
    buf = ctypes.create_string_buffer(512)
    _check(lib.qknorm_describe_headwise_plan(ctypes.byref(oq), ctypes.byref(ok), T, code, head_dim,
                                             gamma_head_stride, buf, 512))
    return buf.value.decode()


def describe_plan(op, hq, hk, T, dtype="bf16", shards=1, ld=None, aligned=True):
    """The launch a call would make, for shapes alone (no GPU needed).

    Uses stand-in addresses for a packed layout (never dereferenced).
    """
    lib = load_library()
    code, esz = _DTYPES[dtype]
    ld = ld if ld is not None else hq + hk
    off = 0 if aligned else esz
    if ld >= hq + hk:      # packed rows: K follows Q in the same rows
        xq, xk = (1 << 32) + off, (1 << 32) + off + hq * esz
    else:                  # separate arrays
        xq, xk = (1 << 32) + off, (1 << 40) + off
    yd = 1 << 44           # outputs and gamma far away from the inputs
    goff = 0 if aligned else (4 if dtype == "f32" else 2)   # gamma: element-aligned, not 16-byte aligned
    oq = Operand(xq, ld, xq + yd, ld, (1 << 46) + goff, hq)
    ok = Operand(xk, ld, xk + yd, ld, (1 << 46) + (1 << 30) + goff, hk)
    buf = ctypes.create_string_buffer(512)
    _check(lib.qknorm_describe_plan(op, ctypes.byref(oq), ctypes.byref(ok), T, code, shards, buf, 512))
    return buf.value.decode()
