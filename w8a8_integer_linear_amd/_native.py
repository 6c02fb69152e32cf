"""ctypes binding of libqlin.so (include/qlin.h).

Argument marshalling only: torch tensors are checked for device, dtype, shape
and contiguity, their device pointers and the current HIP stream are passed to
the C ABI, and a nonzero status raises QlinError.  Every step of the layer runs
in the library's HIP kernels; there is no fallback.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqlin.so")

QLIN_OK, QLIN_EINVAL, QLIN_EUNSUPPORTED, QLIN_EDEVICE = 0, 1, 2, 3
QLIN_F32, QLIN_BF16 = 0, 1
QLIN_OP_FWD, QLIN_OP_DX, QLIN_OP_DW = 0, 1, 2
MAX_CONTRACTION = 131071

# Exported symbols and their C signatures (kept in step with include/qlin.h).
_vp, _i64, _i32, _f32, _u64 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                               ctypes.c_uint64)
SIGNATURES = {
    "qlin_status_string": ([_i32], ctypes.c_char_p),
    "qlin_abi_version": ([], _i32),
    "qlin_quantize_rows": ([_vp, _i32, _i64, _i64, _vp, _i32, _vp, _vp, _vp], _i32),
    "qlin_quantize_cols": ([_vp, _i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp], _i32),
    "qlin_quantize_grad": ([_vp, _i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
                           _i32),
    "qlin_hadamard": ([_vp, _i32, _i64, _i64, _i32, _vp, _vp], _i32),
    "qlin_dequantize_weight": ([_vp, _vp, _i64, _i64, _i32, _vp, _vp], _i32),
    "qlin_fwd": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp], _i32),
    "qlin_bwd_dx": ([_vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _vp], _i32),
    "qlin_bwd_dw": ([_vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp], _i32),
    "qlin_sgd_requant": ([_vp, _vp, _vp, _i64, _i64, _f32, _u64, _u64, _vp, _vp, _vp], _i32),
    "qlin_wn_init": ([_vp, _vp, _i64, _i64, _vp, _vp, _vp], _i32),
    "qlin_wn_sgd_requant": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _u64, _u64, _vp, _vp,
                             _vp], _i32),
    "qlin_adamw_requant": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _f32, _f32, _f32, _f32,
                            _u64, _u64, _vp, _vp, _vp, _vp, _vp], _i32),
    "qlin_gemm_s32": ([_i32, _vp, _vp, _i64, _i64, _i64, _vp, _vp], _i32),
    "qlin_product_ws": ([_i32, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _vp,
                         ctypes.c_size_t, _vp], _i32),
    "qlin_product_ws_bytes": ([_i32, _i64, _i64, _i64], ctypes.c_size_t),
    "qlin_stream_copy": ([_vp, _vp, _i64, _vp], _i32),
    "qlin_product_noalloc": ([_i32, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _vp],
                             _i32),
    "qlin_mfma_ceiling": ([_vp, _vp, _i32, _i32, _vp], _i32),
}
MFMA_CEILING_FRAG_BYTES = 24 * 1024
NOALLOC_SCRATCH_BYTES = 4096 + 160 * 262144


class QlinError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {lib().qlin_status_string(status).decode()} ({status})")


_lib = None


def lib():
    """Load libqlin.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                "g.build()'` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _opt(t, name, dtype, shape):
    return None if t is None else _need(t, name, dtype, shape)


def _dtype_code(x):
    if x.dtype == torch.float32:
        return QLIN_F32
    if x.dtype == torch.bfloat16:
        return QLIN_BF16
    raise TypeError(f"floating input must be float32 or bfloat16, got {x.dtype}")


def _check(fn, status):
    if status != QLIN_OK:
        raise QlinError(fn, status)


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def qlin_quantize_rows(x, prescale=None, had_block=0, q=None, s=None, stream=None):
    rows, cols = x.shape
    _need(x, "x", x.dtype)
    code = _dtype_code(x)
    _opt(prescale, "prescale", torch.float32, (cols,))
    q = _empty((rows, cols), torch.int8, x) if q is None else _need(q, "q", torch.int8, (rows, cols))
    s = _empty((rows,), torch.float32, x) if s is None else _need(s, "s", torch.float32, (rows,))
    _check("qlin_quantize_rows", lib().qlin_quantize_rows(
        _ptr(x), code, rows, cols, _ptr(prescale), int(had_block), _ptr(q), _ptr(s),
        _stream(stream)))
    return q, s


def qlin_quantize_cols(x, prescale=None, q=None, s=None, col_sum=None, want_sum=False,
                       stream=None):
    rows, cols = x.shape
    _need(x, "x", x.dtype)
    code = _dtype_code(x)
    _opt(prescale, "prescale", torch.float32, (rows,))
    q = _empty((rows, cols), torch.int8, x) if q is None else _need(q, "q", torch.int8, (rows, cols))
    s = _empty((cols,), torch.float32, x) if s is None else _need(s, "s", torch.float32, (cols,))
    if col_sum is None and want_sum:
        col_sum = _empty((cols,), torch.float32, x)
    _opt(col_sum, "col_sum", torch.float32, (cols,))
    _check("qlin_quantize_cols", lib().qlin_quantize_cols(
        _ptr(x), code, rows, cols, _ptr(prescale), _ptr(q), _ptr(s), _ptr(col_sum),
        _stream(stream)))
    return (q, s, col_sum) if col_sum is not None else (q, s)


def qlin_quantize_grad(dy, sw, sx, q1=None, s1=None, q2=None, s2=None, col_sum=None,
                       want_sum=False, stream=None):
    """Both quantizations of dY: (q1, s1) per row of dY * sw, (q2, s2) per column
    of dY * sx[:, None], and optionally the column sums.  Returns
    (q1, s1, q2, s2, col_sum)."""
    rows, cols = dy.shape
    _need(dy, "dy", dy.dtype)
    code = _dtype_code(dy)
    _need(sw, "sw", torch.float32, (cols,))
    _need(sx, "sx", torch.float32, (rows,))
    q1 = _empty((rows, cols), torch.int8, dy) if q1 is None else _need(q1, "q1", torch.int8,
                                                                       (rows, cols))
    s1 = _empty((rows,), torch.float32, dy) if s1 is None else _need(s1, "s1", torch.float32,
                                                                     (rows,))
    q2 = _empty((rows, cols), torch.int8, dy) if q2 is None else _need(q2, "q2", torch.int8,
                                                                       (rows, cols))
    s2 = _empty((cols,), torch.float32, dy) if s2 is None else _need(s2, "s2", torch.float32,
                                                                     (cols,))
    if col_sum is None and want_sum:
        col_sum = _empty((cols,), torch.float32, dy)
    _opt(col_sum, "col_sum", torch.float32, (cols,))
    _check("qlin_quantize_grad", lib().qlin_quantize_grad(
        _ptr(dy), code, rows, cols, _ptr(sw), _ptr(sx), _ptr(q1), _ptr(s1), _ptr(q2), _ptr(s2),
        _ptr(col_sum), _stream(stream)))
    return q1, s1, q2, s2, col_sum


def qlin_hadamard(x, block, y=None, stream=None):
    rows, cols = x.shape
    _need(x, "x", x.dtype)
    code = _dtype_code(x)
    y = _empty((rows, cols), torch.float32, x) if y is None else _need(y, "y", torch.float32,
                                                                       (rows, cols))
    _check("qlin_hadamard", lib().qlin_hadamard(_ptr(x), code, rows, cols, int(block), _ptr(y),
                                                _stream(stream)))
    return y


def qlin_dequantize_weight(qw, sw, had_block=0, w=None, stream=None):
    """fl(sw * qw) per row, rotated back to the original basis when had_block."""
    N, K = qw.shape
    _need(qw, "qw", torch.int8)
    _need(sw, "sw", torch.float32, (N,))
    w = _empty((N, K), torch.float32, qw) if w is None else _need(w, "w", torch.float32, (N, K))
    _check("qlin_dequantize_weight", lib().qlin_dequantize_weight(
        _ptr(qw), _ptr(sw), N, K, int(had_block), _ptr(w), _stream(stream)))
    return w


def qlin_fwd(qx, sx, qw, sw, bias=None, y=None, stream=None):
    M, K = qx.shape
    N = qw.shape[0]
    _need(qx, "qx", torch.int8)
    _need(qw, "qw", torch.int8, (N, K))
    _need(sx, "sx", torch.float32, (M,))
    _need(sw, "sw", torch.float32, (N,))
    _opt(bias, "bias", torch.float32, (N,))
    y = _empty((M, N), torch.float32, qx) if y is None else _need(y, "y", torch.float32, (M, N))
    _check("qlin_fwd", lib().qlin_fwd(_ptr(qx), _ptr(sx), _ptr(qw), _ptr(sw), _ptr(bias), M, N, K,
                                      _ptr(y), _stream(stream)))
    return y


def qlin_bwd_dx(qg1, sg1, qw, had_block=0, dx=None, stream=None):
    M, N = qg1.shape
    K = qw.shape[1]
    _need(qg1, "qg1", torch.int8)
    _need(qw, "qw", torch.int8, (N, K))
    _need(sg1, "sg1", torch.float32, (M,))
    dx = _empty((M, K), torch.float32, qg1) if dx is None else _need(dx, "dx", torch.float32,
                                                                     (M, K))
    _check("qlin_bwd_dx", lib().qlin_bwd_dx(_ptr(qg1), _ptr(sg1), _ptr(qw), M, N, K,
                                            int(had_block), _ptr(dx), _stream(stream)))
    return dx


def qlin_bwd_dw(qg2, sg2, qx, dw=None, stream=None):
    M, N = qg2.shape
    K = qx.shape[1]
    _need(qg2, "qg2", torch.int8)
    _need(qx, "qx", torch.int8, (M, K))
    _need(sg2, "sg2", torch.float32, (N,))
    dw = _empty((N, K), torch.float32, qg2) if dw is None else _need(dw, "dw", torch.float32,
                                                                     (N, K))
    _check("qlin_bwd_dw", lib().qlin_bwd_dw(_ptr(qg2), _ptr(sg2), _ptr(qx), M, N, K, _ptr(dw),
                                            _stream(stream)))
    return dw


def qlin_sgd_requant(qw, sw, dw, lr, seed, step, bias=None, db=None, stream=None):
    """In place on qw, sw (and bias)."""
    N, K = qw.shape
    _need(qw, "qw", torch.int8)
    _need(sw, "sw", torch.float32, (N,))
    _need(dw, "dw", torch.float32, (N, K))
    _opt(bias, "bias", torch.float32, (N,))
    _opt(db, "db", torch.float32, (N,))
    _check("qlin_sgd_requant", lib().qlin_sgd_requant(
        _ptr(qw), _ptr(sw), _ptr(dw), N, K, float(lr), int(seed), int(step), _ptr(bias),
        _ptr(db), _stream(stream)))
    return qw, sw


def qlin_wn_init(q, s, g=None, sw=None, stream=None):
    """Magnitudes g and column scales sw of a weight-normalized layer from its
    direction codes q and row scales s.  Returns (g, sw)."""
    N, K = q.shape
    _need(q, "q", torch.int8)
    _need(s, "s", torch.float32, (N,))
    g = _empty((N,), torch.float32, q) if g is None else _need(g, "g", torch.float32, (N,))
    sw = _empty((N,), torch.float32, q) if sw is None else _need(sw, "sw", torch.float32, (N,))
    _check("qlin_wn_init", lib().qlin_wn_init(_ptr(q), _ptr(s), N, K, _ptr(g), _ptr(sw),
                                              _stream(stream)))
    return g, sw


def qlin_wn_sgd_requant(q, s, g, sw, dw, lr, seed, step, bias=None, db=None, stream=None):
    """In place on q, s, g, sw (and bias)."""
    N, K = q.shape
    _need(q, "q", torch.int8)
    for t, name in ((s, "s"), (g, "g"), (sw, "sw")):
        _need(t, name, torch.float32, (N,))
    _need(dw, "dw", torch.float32, (N, K))
    _opt(bias, "bias", torch.float32, (N,))
    _opt(db, "db", torch.float32, (N,))
    _check("qlin_wn_sgd_requant", lib().qlin_wn_sgd_requant(
        _ptr(q), _ptr(s), _ptr(g), _ptr(sw), _ptr(dw), N, K, float(lr), int(seed), int(step),
        _ptr(bias), _ptr(db), _stream(stream)))
    return q, s, g, sw


def qlin_adamw_requant(qw, sw, dw, m, v, lr, beta1, beta2, eps, weight_decay, seed, step,
                       bias=None, db=None, bias_m=None, bias_v=None, stream=None):
    """In place on qw, sw, m, v (and bias, bias_m, bias_v).  step >= 1."""
    N, K = qw.shape
    _need(qw, "qw", torch.int8)
    _need(sw, "sw", torch.float32, (N,))
    _need(dw, "dw", torch.float32, (N, K))
    _need(m, "m", torch.float32, (N, K))
    _need(v, "v", torch.float32, (N, K))
    for t, name in ((bias, "bias"), (db, "db"), (bias_m, "bias_m"), (bias_v, "bias_v")):
        _opt(t, name, torch.float32, (N,))
    _check("qlin_adamw_requant", lib().qlin_adamw_requant(
        _ptr(qw), _ptr(sw), _ptr(dw), _ptr(m), _ptr(v), N, K, float(lr), float(beta1),
        float(beta2), float(eps), float(weight_decay), int(seed), int(step), _ptr(bias),
        _ptr(db), _ptr(bias_m), _ptr(bias_v), _stream(stream)))
    return qw, sw


def qlin_product_ws_bytes(op, M, N, K):
    return int(lib().qlin_product_ws_bytes(int(op), int(M), int(N), int(K)))


def qlin_product_ws(op, a, srow, b, M, N, K, scol=None, bias=None, had_block=0, out=None,
                    workspace=None, stream=None):
    """Any product with a contraction of any length, using a caller workspace
    (allocated zero-filled here when not given; a reused workspace comes back
    from every call with its arrival counters zero again).  Within the int32
    bound the workspace lets the last round of tiles be split along the
    contraction; beyond it, int32 chunks are combined in int64 there."""
    shape = {QLIN_OP_FWD: (M, N), QLIN_OP_DX: (M, K), QLIN_OP_DW: (N, K)}[op]
    _need(a, "a", torch.int8)
    _need(b, "b", torch.int8)
    _need(srow, "srow", torch.float32)
    _opt(scol, "scol", torch.float32, (N,))
    _opt(bias, "bias", torch.float32, (N,))
    out = _empty(shape, torch.float32, a) if out is None else _need(out, "out", torch.float32,
                                                                     shape)
    need = qlin_product_ws_bytes(op, M, N, K)
    if workspace is None and need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=a.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("qlin_product_ws", lib().qlin_product_ws(
        int(op), _ptr(a), _ptr(srow), _ptr(b), _ptr(scol), _ptr(bias), M, N, K, int(had_block),
        _ptr(out), _ptr(workspace), nbytes, _stream(stream)))
    return out


def qlin_product_noalloc(op, a, srow, b, M, N, K, out, scol=None, bias=None, had_block=0,
                         stream=None):
    """qlin_product_ws with the library's own device scratch in place of a
    workspace: nothing is allocated, `out` included (the caller passes it)."""
    shape = {QLIN_OP_FWD: (M, N), QLIN_OP_DX: (M, K), QLIN_OP_DW: (N, K)}[op]
    _need(a, "a", torch.int8)
    _need(b, "b", torch.int8)
    _need(srow, "srow", torch.float32)
    _opt(scol, "scol", torch.float32, (N,))
    _opt(bias, "bias", torch.float32, (N,))
    _need(out, "out", torch.float32, shape)
    _check("qlin_product_noalloc", lib().qlin_product_noalloc(
        int(op), _ptr(a), _ptr(srow), _ptr(b), _ptr(scol), _ptr(bias), M, N, K, int(had_block),
        _ptr(out), _stream(stream)))
    return out


def qlin_gemm_s32(op, a, b, M, N, K, c=None, stream=None):
    shape = {QLIN_OP_FWD: (M, N), QLIN_OP_DX: (M, K), QLIN_OP_DW: (N, K)}[op]
    _need(a, "a", torch.int8)
    _need(b, "b", torch.int8)
    c = _empty(shape, torch.int32, a) if c is None else _need(c, "c", torch.int32, shape)
    _check("qlin_gemm_s32", lib().qlin_gemm_s32(op, _ptr(a), _ptr(b), M, N, K, _ptr(c),
                                                _stream(stream)))
    return c


def qlin_stream_copy(src, dst, stream=None):
    """Copy the bytes of src into dst (same size, contiguous) with the
    library's streaming kernel."""
    _need(src, "src", src.dtype)
    _need(dst, "dst", dst.dtype)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst differ in size")
    _check("qlin_stream_copy", lib().qlin_stream_copy(_ptr(src), _ptr(dst), nbytes,
                                                      _stream(stream)))
    return dst


def qlin_mfma_ceiling(frags, out, workgroups, iters, stream=None):
    """The library's matrix-core ceiling kernel: `workgroups` workgroups repeat
    the products' MFMA sequence `iters` times on the int8 fragments in frags
    (MFMA_CEILING_FRAG_BYTES); out (int32, workgroups * 512 * 4) gets each
    lane's sums."""
    _need(frags, "frags", torch.int8, (MFMA_CEILING_FRAG_BYTES,))
    _need(out, "out", torch.int32, (int(workgroups) * 512 * 4,))
    _check("qlin_mfma_ceiling", lib().qlin_mfma_ceiling(_ptr(frags), _ptr(out), int(workgroups),
                                                        int(iters), _stream(stream)))
    return out
