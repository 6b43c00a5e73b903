"""ctypes binding of libfp8fg.so -- argument marshalling only.

Each function has the name and the parameter list of the C entry point in
``include/fp8fg.h``.  Pointer parameters accept a torch tensor (its
``data_ptr()`` is passed), a raw integer address, or None (NULL).  ``stream``
accepts a ``torch.cuda.Stream``, a raw ``hipStream_t`` integer, or None: the
current torch stream of the tensors' device, or NULL when no CUDA tensor is
involved.  The call runs with the tensors' device made current.

A nonzero status raises ``Fp8fgError`` unless ``check=False`` (then the
status is returned).  All computation happens in the library's HIP kernels;
there is no fallback: if the library is missing, the import of its handle
raises.
"""

import contextlib
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8fg.so")

# mirrors of the header's enums
FP8FG_OK, FP8FG_EINVAL, FP8FG_ESHAPE, FP8FG_EALIGN, FP8FG_EUNSUPPORTED, FP8FG_ELAUNCH = range(6)
FP8FG_BF16, FP8FG_F32, FP8FG_E4M3 = 0, 1, 2
FP8FG_TILE_1x128, FP8FG_TILE_128x1 = 0, 1
FP8FG_SCALE_AMAX, FP8FG_SCALE_POW2 = 0, 1
FP8FG_BSCALE_BLOCK128, FP8FG_BSCALE_COL = 0, 1
FP8FG_GEMM_DEFAULT, FP8FG_GEMM_NO_PROMOTION, FP8FG_GEMM_FP8_MFMA, FP8FG_GEMM_E8M0_SCALES = 0, 1, 2, 4
FP8FG_GEMM_TILES_WIDE, FP8FG_GEMM_TILES_NARROW = 8, 16

EXPORTED = ("fp8_quantize_rowtile", "fp8_quantize_block", "fp8_gemm_blockscaled",
            "fp8_grouped_gemm_blockscaled", "fp8fg_status_string")


class Fp8fgError(RuntimeError):
    def __init__(self, status, func):
        self.status = status
        super().__init__("%s failed: status %d (%s)" % (func, status, status_string(status)))


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64

_SIGS = {
    "fp8_quantize_rowtile": [_P, _I, _L, _L, _L, _P, _L, _L, _I, _I, _P, _L, _P, _L, _L, _P],
    "fp8_quantize_block": [_P, _I, _L, _L, _L, _I, _I, _P, _L, _P, _L, _L, _P],
    "fp8_gemm_blockscaled": [_L, _L, _L, _P, _L, _P, _L, _L, _P, _L, _P, _L, _L, _I, _P, _I, _L,
                             _I, _P],
    "fp8_grouped_gemm_blockscaled": [_L, _P, _L, _L, _L, _P, _L, _P, _L, _L, _P, _L, _L, _P, _L,
                                     _L, _L, _P, _I, _L, _I, _P],
}


def lib():
    """The loaded library (loaded once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libfp8fg.so is not built; run `python -m fp8_fine_grained_x1_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(l, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        l.fp8fg_status_string.argtypes = [ctypes.c_int]
        l.fp8fg_status_string.restype = ctypes.c_char_p
        _lib = l
    return _lib


def status_string(status):
    return lib().fp8fg_status_string(int(status)).decode()


def _is_tensor(x):
    return hasattr(x, "data_ptr") and hasattr(x, "device")


def _ptr(x):
    if x is None:
        return None
    if _is_tensor(x):
        return x.data_ptr()
    return int(x)


def _cuda_device(args):
    for a in args:
        if _is_tensor(a) and a.device.type == "cuda":
            return a.device
    return None


def _stream(stream, device):
    if stream is None:
        if device is None:
            return None
        import torch
        return torch.cuda.current_stream(device).cuda_stream
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


@contextlib.contextmanager
def _on(device):
    if device is None:
        yield
        return
    import torch
    with torch.cuda.device(device):
        yield


def _call(name, check, ptr_args, build):
    dev = _cuda_device(ptr_args)
    with _on(dev):
        st = build(dev)
        rc = getattr(lib(), name)(*st)
    if check and rc != FP8FG_OK:
        raise Fp8fgError(rc, name)
    return rc


def fp8_quantize_rowtile(x, x_type, rows, cols, ldx, x_scale, xs_rs, xs_ts, tile, scale_rule,
                         q, ldq, s, s_rs, s_ts, stream=None, check=True):
    return _call("fp8_quantize_rowtile", check, (x, x_scale, q, s), lambda dev: (
        _ptr(x), x_type, rows, cols, ldx, _ptr(x_scale), xs_rs, xs_ts, tile, scale_rule,
        _ptr(q), ldq, _ptr(s), s_rs, s_ts, _stream(stream, dev)))


def fp8_quantize_block(w, w_type, rows, cols, ldw, scale_rule, transpose_out, q, ldq, s, s_rs,
                       s_cs, stream=None, check=True):
    return _call("fp8_quantize_block", check, (w, q, s), lambda dev: (
        _ptr(w), w_type, rows, cols, ldw, scale_rule, transpose_out, _ptr(q), ldq, _ptr(s),
        s_rs, s_cs, _stream(stream, dev)))


def fp8_gemm_blockscaled(M, N, K, a, lda, sa, sa_ms, sa_ks, b, ldb, sb, sb_ns, sb_ks,
                         b_scale_mode, c, c_type, ldc, flags, stream=None, check=True):
    return _call("fp8_gemm_blockscaled", check, (a, sa, b, sb, c), lambda dev: (
        M, N, K, _ptr(a), lda, _ptr(sa), sa_ms, sa_ks, _ptr(b), ldb, _ptr(sb), sb_ns, sb_ks,
        b_scale_mode, _ptr(c), c_type, ldc, flags, _stream(stream, dev)))


def fp8_grouped_gemm_blockscaled(G, offsets, M_total, N, K, a, lda, sa, sa_ms, sa_ks, b, ldb,
                                 b_gs, sb, sb_ns, sb_ks, sb_gs, c, c_type, ldc, flags,
                                 stream=None, check=True):
    return _call("fp8_grouped_gemm_blockscaled", check, (offsets, a, sa, b, sb, c), lambda dev: (
        G, _ptr(offsets), M_total, N, K, _ptr(a), lda, _ptr(sa), sa_ms, sa_ks, _ptr(b), ldb,
        b_gs, _ptr(sb), sb_ns, sb_ks, sb_gs, _ptr(c), c_type, ldc, flags,
        _stream(stream, dev)))
