"""CPU oracle for the INT8 W8A8 linear layer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``qlin_oracle.c`` (plain C,
built with gcc) through ctypes on numpy arrays and shares nothing with the HIP
library.  bf16 arrays are passed as ``uint16`` bit patterns.

Each function follows the passage cited in ``qlin_oracle.c``:
mini_trainer "quantized-training" guide (INT8 weights with per-row float
magnitude, integer forward/backward products, stochastic requantization) and
OneTrainer PR #1681 "Int8 conv rot" (block-Hadamard rotation of activations,
per-row activation quantization).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qlin_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1
OK = 0
EINVAL = 1
EUNSUPPORTED = 2

OP_FWD, OP_DX, OP_DW = 0, 1, 2

# gcc flags: IEEE binary32 arithmetic with no contraction into FMA and no
# fast-math, so every fl() in the definitions is one correctly rounded op.
CFLAGS = ["-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp",
          "-ffp-contract=off", "-fno-fast-math", "-fno-finite-math-only"]


def build(verbose=False):
    """Compile qlin_oracle.c into liboracle.so (always recompiles)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    global _lib
    _lib = None


_lib = None

# Flags of the build the CPU baseline times: the same arithmetic (no FMA
# contraction, no fast-math), optimised for the host it runs on.
HOST_CFLAGS = ["-O3", "-march=native", "-std=gnu11", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-fno-finite-math-only"]


def use_host_build():
    """Compile qlin_oracle.c with HOST_CFLAGS into a private temporary file
    and load it in place of liboracle.so for the rest of the process (the
    CPU-baseline leg of the benchmark).  Returns the flags used."""
    import tempfile
    global _lib
    out = os.path.join(tempfile.mkdtemp(prefix="oracle_host_"), "liboracle_host.so")
    subprocess.run(["gcc", *HOST_CFLAGS, _SRC, "-o", out, "-lm"], check=True)
    _lib = None
    lib(out)
    return HOST_CFLAGS


def lib(path=None):
    """Load liboracle.so, building it first only if it does not exist."""
    global _lib
    if _lib is None:
        if path is None:
            path = _LIB
            if not os.path.exists(path):
                build()
        L = ctypes.CDLL(path)
        vp, i64, i32, f32, u64 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                  ctypes.c_float, ctypes.c_uint64)
        L.orc_threads.argtypes = []
        L.orc_threads.restype = i32
        L.orc_hadamard_scale.argtypes = [i32]
        L.orc_hadamard_scale.restype = f32
        L.orc_hadamard.argtypes = [vp, i32, i64, i64, i32, vp]
        L.orc_quantize_rows.argtypes = [vp, i32, i64, i64, vp, i32, vp, vp]
        L.orc_quantize_cols.argtypes = [vp, i32, i64, i64, vp, vp, vp, vp]
        L.orc_gemm_s32.argtypes = [i32, vp, vp, i64, i64, i64, vp]
        L.orc_gemm_s32_at.argtypes = [i32, vp, vp, i64, i64, i64, vp, vp, i64, vp]
        L.orc_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
        L.orc_bwd_dx.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        L.orc_bwd_dw.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        L.orc_op_at.argtypes = [i32, vp, vp, vp, vp, vp, i64, i64, i64, vp, vp, i64, vp]
        L.orc_philox4x32_10.argtypes = [vp, vp, vp]
        L.orc_philox4x32_10.restype = None
        L.orc_philox4x64_10.argtypes = [vp, vp, vp]
        L.orc_philox4x64_10.restype = None
        L.orc_sr_bits16.argtypes = [u64, u64, u64]
        L.orc_sr_bits16.restype = ctypes.c_uint32
        L.orc_sgd_requant.argtypes = [vp, vp, vp, i64, i64, f32, u64, u64, vp, vp, vp]
        L.orc_bwd_dw_rows.argtypes = [vp, vp, vp, i64, i64, i64, vp, i64, vp]
        L.orc_dequantize_weight.argtypes = [vp, vp, i64, i64, i32, vp]
        L.orc_gemm_s64_at.argtypes = [i32, vp, vp, i64, i64, i64, vp, vp, i64, vp]
        L.orc_op_at_long.argtypes = [i32, vp, vp, vp, vp, vp, i64, i64, i64, vp, vp, i64, vp]
        L.orc_wn_init.argtypes = [vp, vp, i64, i64, vp, vp]
        L.orc_wn_grads.argtypes = [vp, vp, vp, vp, i64, i64, vp, vp]
        L.orc_wn_sgd_requant.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, u64, u64, vp, vp,
                                         vp]
        L.orc_adamw_constants.argtypes = [f32, f32, f32, f32, u64, vp]
        L.orc_adamw_constants.restype = None
        L.orc_adamw_update.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, f32, f32, f32, f32,
                                       u64, vp]
        L.orc_adamw_requant.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, f32, f32, f32, f32,
                                        u64, u64, vp, vp, vp, vp, vp]
        for name in ("orc_hadamard", "orc_quantize_rows", "orc_quantize_cols",
                     "orc_gemm_s32", "orc_gemm_s32_at", "orc_fwd", "orc_bwd_dx",
                     "orc_bwd_dw", "orc_bwd_dw_rows", "orc_op_at", "orc_sgd_requant",
                     "orc_adamw_update", "orc_adamw_requant", "orc_dequantize_weight",
                     "orc_gemm_s64_at", "orc_op_at_long", "orc_wn_init", "orc_wn_grads",
                     "orc_wn_sgd_requant"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return None if a is None else a.ctypes.data


def _chk(st):
    if st != OK:
        raise OracleError(f"oracle status {st}")


def _as_input(x):
    """(contiguous array, dtype code) for an fp32 array or uint16 bf16 bits."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, BF16
    if x.dtype != np.float32:
        raise TypeError(f"oracle input must be float32 or uint16 (bf16 bits), got {x.dtype}")
    return x, F32


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def threads():
    """Host threads the oracle's parallel loops use."""
    return int(lib().orc_threads())


def hadamard_scale(b):
    return float(np.float32(lib().orc_hadamard_scale(int(b))))


def hadamard(x, block):
    """Block-Hadamard rotation of each row of x (fp32 or bf16 bits) -> fp32."""
    x, dt = _as_input(x)
    rows, cols = x.shape
    y = np.empty((rows, cols), np.float32)
    _chk(lib().orc_hadamard(_ptr(x), dt, rows, cols, int(block), _ptr(y)))
    return y


def dequantize_weight(qw, sw, had_block=0):
    """The represented weight fl(s * q) per row, un-rotated when had_block != 0."""
    qw = np.ascontiguousarray(qw, np.int8)
    N, K = qw.shape
    w = np.empty((N, K), np.float32)
    _chk(lib().orc_dequantize_weight(_ptr(qw), _ptr(_f32(sw)), N, K, int(had_block), _ptr(w)))
    return w


def quantize_rows(x, prescale=None, had_block=0):
    """Per-row absmax INT8 quantization (optional rotation, then prescale)."""
    x, dt = _as_input(x)
    rows, cols = x.shape
    p = _f32(prescale)
    q = np.empty((rows, cols), np.int8)
    s = np.empty(rows, np.float32)
    _chk(lib().orc_quantize_rows(_ptr(x), dt, rows, cols, _ptr(p), int(had_block),
                                 _ptr(q), _ptr(s)))
    return q, s


def quantize_cols(x, prescale=None, want_sum=False):
    """Per-column absmax INT8 quantization of x * prescale[:, None]."""
    x, dt = _as_input(x)
    rows, cols = x.shape
    p = _f32(prescale)
    q = np.empty((rows, cols), np.int8)
    s = np.empty(cols, np.float32)
    cs = np.empty(cols, np.float32) if want_sum else None
    _chk(lib().orc_quantize_cols(_ptr(x), dt, rows, cols, _ptr(p), _ptr(q), _ptr(s),
                                 _ptr(cs)))
    return (q, s, cs) if want_sum else (q, s)


def _op_dims(op, M, N, K):
    return {OP_FWD: (M, N), OP_DX: (M, K), OP_DW: (N, K)}[op]


def gemm_s32(op, a, b, M, N, K):
    """Raw int32 accumulators of product ``op`` (OP_FWD, OP_DX or OP_DW)."""
    a = np.ascontiguousarray(a, np.int8)
    b = np.ascontiguousarray(b, np.int8)
    R, C = _op_dims(op, M, N, K)
    c = np.empty((R, C), np.int32)
    _chk(lib().orc_gemm_s32(op, _ptr(a), _ptr(b), M, N, K, _ptr(c)))
    return c


def gemm_s32_at(op, a, b, M, N, K, ii, jj):
    a = np.ascontiguousarray(a, np.int8)
    b = np.ascontiguousarray(b, np.int8)
    ii = np.ascontiguousarray(ii, np.int64)
    jj = np.ascontiguousarray(jj, np.int64)
    out = np.empty(len(ii), np.int32)
    _chk(lib().orc_gemm_s32_at(op, _ptr(a), _ptr(b), M, N, K, _ptr(ii), _ptr(jj),
                               len(ii), _ptr(out)))
    return out


def fwd(qx, sx, qw, sw, bias=None):
    qx = np.ascontiguousarray(qx, np.int8)
    qw = np.ascontiguousarray(qw, np.int8)
    M, K = qx.shape
    N = qw.shape[0]
    y = np.empty((M, N), np.float32)
    _chk(lib().orc_fwd(_ptr(qx), _ptr(_f32(sx)), _ptr(qw), _ptr(_f32(sw)),
                       _ptr(_f32(bias)), M, N, K, _ptr(y)))
    return y


def bwd_dx(qg1, sg1, qw):
    qg1 = np.ascontiguousarray(qg1, np.int8)
    qw = np.ascontiguousarray(qw, np.int8)
    M, N = qg1.shape
    K = qw.shape[1]
    dx = np.empty((M, K), np.float32)
    _chk(lib().orc_bwd_dx(_ptr(qg1), _ptr(_f32(sg1)), _ptr(qw), M, N, K, _ptr(dx)))
    return dx


def bwd_dw(qg2, sg2, qx):
    qg2 = np.ascontiguousarray(qg2, np.int8)
    qx = np.ascontiguousarray(qx, np.int8)
    M, N = qg2.shape
    K = qx.shape[1]
    dw = np.empty((N, K), np.float32)
    _chk(lib().orc_bwd_dw(_ptr(qg2), _ptr(_f32(sg2)), _ptr(qx), M, N, K, _ptr(dw)))
    return dw


def bwd_dw_rows(qg2, sg2, qx, rows):
    """Rows ``rows`` of dW (each a full row of K outputs)."""
    qg2 = np.ascontiguousarray(qg2, np.int8)
    qx = np.ascontiguousarray(qx, np.int8)
    rows = np.ascontiguousarray(rows, np.int64)
    M, N = qg2.shape
    K = qx.shape[1]
    out = np.empty((len(rows), K), np.float32)
    _chk(lib().orc_bwd_dw_rows(_ptr(qg2), _ptr(_f32(sg2)), _ptr(qx), M, N, K, _ptr(rows),
                               len(rows), _ptr(out)))
    return out


def op_at(op, a, srow, b, scol, bias, M, N, K, ii, jj):
    """Dequantized outputs of product ``op`` at positions (ii[t], jj[t])."""
    a = np.ascontiguousarray(a, np.int8)
    b = np.ascontiguousarray(b, np.int8)
    ii = np.ascontiguousarray(ii, np.int64)
    jj = np.ascontiguousarray(jj, np.int64)
    out = np.empty(len(ii), np.float32)
    _chk(lib().orc_op_at(op, _ptr(a), _ptr(_f32(srow)), _ptr(b), _ptr(_f32(scol)),
                         _ptr(_f32(bias)), M, N, K, _ptr(ii), _ptr(jj), len(ii),
                         _ptr(out)))
    return out


def gemm_s64_at(op, a, b, M, N, K, ii, jj):
    """Exact (int64) accumulators at positions, for any contraction length."""
    a = np.ascontiguousarray(a, np.int8)
    b = np.ascontiguousarray(b, np.int8)
    ii = np.ascontiguousarray(ii, np.int64)
    jj = np.ascontiguousarray(jj, np.int64)
    out = np.empty(len(ii), np.int64)
    _chk(lib().orc_gemm_s64_at(op, _ptr(a), _ptr(b), M, N, K, _ptr(ii), _ptr(jj), len(ii),
                               _ptr(out)))
    return out


def op_at_long(op, a, srow, b, scol, bias, M, N, K, ii, jj):
    """op_at for any contraction length: int32 chunk sums combined in int64
    (equal to the exact dot product), converted once to fp32, dequantized."""
    a = np.ascontiguousarray(a, np.int8)
    b = np.ascontiguousarray(b, np.int8)
    ii = np.ascontiguousarray(ii, np.int64)
    jj = np.ascontiguousarray(jj, np.int64)
    out = np.empty(len(ii), np.float32)
    _chk(lib().orc_op_at_long(op, _ptr(a), _ptr(_f32(srow)), _ptr(b), _ptr(_f32(scol)),
                              _ptr(_f32(bias)), M, N, K, _ptr(ii), _ptr(jj), len(ii),
                              _ptr(out)))
    return out


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, np.uint32)
    k = np.ascontiguousarray(key, np.uint32)
    out = np.empty(4, np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def philox4x64_10(ctr, key):
    c = np.ascontiguousarray(ctr, np.uint64)
    k = np.ascontiguousarray(key, np.uint64)
    out = np.empty(4, np.uint64)
    lib().orc_philox4x64_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_bits16(seed, step, i):
    return int(lib().orc_sr_bits16(int(seed), int(step), int(i)))


def sgd_requant(qw, sw, dw, lr, seed, step, bias=None, db=None, row_ids=None):
    """Returns updated (qw, sw, bias) copies; the inputs are left unchanged.

    row_ids: global row index of each given row (keys the random stream)."""
    qw = np.array(qw, np.int8, copy=True, order="C")
    sw = np.array(sw, np.float32, copy=True)
    dw = np.ascontiguousarray(dw, np.float32)
    b = None if bias is None else np.array(bias, np.float32, copy=True)
    N, K = qw.shape
    ids = None if row_ids is None else np.ascontiguousarray(row_ids, np.int64)
    _chk(lib().orc_sgd_requant(_ptr(qw), _ptr(sw), _ptr(dw), N, K, float(lr), int(seed),
                               int(step), _ptr(b), _ptr(_f32(db)), _ptr(ids)))
    return qw, sw, b


def adamw_constants(lr, beta1, beta2, weight_decay, step):
    """(a1, a2, c1, c2, decay) as the oracle uses them (fp32 values)."""
    k = (ctypes.c_float * 5)()
    lib().orc_adamw_constants(ctypes.c_float(lr), ctypes.c_float(beta1), ctypes.c_float(beta2),
                              ctypes.c_float(weight_decay), ctypes.c_uint64(step), k)
    return tuple(np.float32(x) for x in k)


def adamw_update(qw, sw, dw, m, v, lr, beta1, beta2, eps, weight_decay, step):
    """The float AdamW update of the represented weight: returns (w, m, v)."""
    qw = np.ascontiguousarray(qw, np.int8)
    N, K = qw.shape
    m = np.array(m, np.float32, copy=True)
    v = np.array(v, np.float32, copy=True)
    w = np.empty((N, K), np.float32)
    _chk(lib().orc_adamw_update(_ptr(qw), _ptr(_f32(sw)), _ptr(_f32(dw)), _ptr(m), _ptr(v), N, K,
                                ctypes.c_float(lr), ctypes.c_float(beta1), ctypes.c_float(beta2),
                                ctypes.c_float(eps), ctypes.c_float(weight_decay),
                                ctypes.c_uint64(step), _ptr(w)))
    return w, m, v


def adamw_requant(qw, sw, dw, m, v, lr, beta1, beta2, eps, weight_decay, seed, step,
                  bias=None, db=None, bm=None, bv=None, row_ids=None):
    """AdamW + stochastic requant; returns updated copies
    (qw, sw, m, v, bias, bm, bv).  step >= 1 is AdamW's t and the Philox step."""
    qw = np.array(qw, np.int8, copy=True, order="C")
    sw = np.array(sw, np.float32, copy=True)
    m = np.array(m, np.float32, copy=True)
    v = np.array(v, np.float32, copy=True)
    N, K = qw.shape
    cp = lambda a: None if a is None else np.array(a, np.float32, copy=True)
    b, bm, bv = cp(bias), cp(bm), cp(bv)
    ids = None if row_ids is None else np.ascontiguousarray(row_ids, np.int64)
    _chk(lib().orc_adamw_requant(_ptr(qw), _ptr(sw), _ptr(_f32(dw)), _ptr(m), _ptr(v), N, K,
                                 ctypes.c_float(lr), ctypes.c_float(beta1), ctypes.c_float(beta2),
                                 ctypes.c_float(eps), ctypes.c_float(weight_decay),
                                 ctypes.c_uint64(seed), ctypes.c_uint64(step), _ptr(b),
                                 _ptr(_f32(db)), _ptr(bm), _ptr(bv), _ptr(ids)))
    return qw, sw, m, v, b, bm, bv


def wn_init(q, s):
    """Row weight normalization at preparation: (g, sw) from the direction
    codes q [N, K] and row scales s [N]; rejects all-zero directions."""
    q = np.ascontiguousarray(q, np.int8)
    N, K = q.shape
    g = np.empty(N, np.float32)
    sw = np.empty(N, np.float32)
    _chk(lib().orc_wn_init(_ptr(q), _ptr(_f32(s)), N, K, _ptr(g), _ptr(sw)))
    return g, sw


def wn_grads(q, s, g, dw):
    """(dg [N], dv [N, K]): gradients of the magnitude and the direction."""
    q = np.ascontiguousarray(q, np.int8)
    N, K = q.shape
    dg = np.empty(N, np.float32)
    dv = np.empty((N, K), np.float32)
    _chk(lib().orc_wn_grads(_ptr(q), _ptr(_f32(s)), _ptr(_f32(g)), _ptr(_f32(dw)), N, K,
                            _ptr(dg), _ptr(dv)))
    return dg, dv


def wn_sgd_requant(q, s, g, dw, lr, seed, step, bias=None, db=None, row_ids=None):
    """One SGD step of the weight-normalized row state; returns updated copies
    (q, s, g, sw, bias)."""
    q = np.array(q, np.int8, copy=True, order="C")
    s = np.array(s, np.float32, copy=True)
    g = np.array(g, np.float32, copy=True)
    N, K = q.shape
    sw = np.empty(N, np.float32)
    b = None if bias is None else np.array(bias, np.float32, copy=True)
    ids = None if row_ids is None else np.ascontiguousarray(row_ids, np.int64)
    _chk(lib().orc_wn_sgd_requant(_ptr(q), _ptr(s), _ptr(g), _ptr(sw), _ptr(_f32(dw)), N, K,
                                  ctypes.c_float(lr), ctypes.c_uint64(seed),
                                  ctypes.c_uint64(step), _ptr(b), _ptr(_f32(db)), _ptr(ids)))
    return q, s, g, sw, b


def prepare_weight(w, had_block=0):
    """Weight preparation: rotate each row (optional), then per-row quantize.

    Rejects all-zero rows (mini_trainer guide: initial zero directions are
    rejected)."""
    w = np.ascontiguousarray(w, np.float32)
    if np.any(np.all(w == 0, axis=1)):
        raise ValueError("weight has an all-zero row (zero direction)")
    return quantize_rows(w, had_block=had_block)
