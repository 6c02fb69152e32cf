"""The C-ABI library: it loads, exports every entry point include/qlin.h
declares, and rejects bad arguments before launching anything.

The rejection tests pass fake (never dereferenced) device addresses and only
run where no GPU is present, so that an accepted call could not touch memory."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlin.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlin_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    from w8a8_integer_linear_amd import _native
    if not os.path.exists(_native.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return _native.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n


def test_binding_covers_header():
    from w8a8_integer_linear_amd import _native
    assert sorted(_native.SIGNATURES) == _declared()


def test_status_strings(L):
    assert L.qlin_status_string(0) == b"ok"
    assert L.qlin_status_string(1) == b"invalid argument"
    assert L.qlin_status_string(2) == b"unsupported shape"
    assert L.qlin_abi_version() == 1


def _cpu_only():
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation tests run only without a GPU")


P = 0x10000   # a 16-byte aligned fake device address, never dereferenced
Q = 0x20000
R = 0x30000
S = 0x40000
ODD = 0x10008  # 8-byte aligned only


@pytest.mark.parametrize("args,expect", [
    ((None, 0, 4, 16, None, 0, Q, R), 1),          # null x
    ((P, 2, 4, 16, None, 0, Q, R), 1),             # bad dtype
    ((P, 0, 4, 24, None, 0, Q, R), 1),             # cols not a multiple of 16
    ((P, 0, 4, 0, None, 0, Q, R), 1),              # empty rows of zero length
    ((P, 0, -1, 16, None, 0, Q, R), 1),            # negative rows
    ((P, 0, 4, 48, None, 32, Q, R), 1),            # block does not divide cols
    ((P, 0, 4, 96, None, 3, Q, R), 1),             # block not a power of two
    ((P, 0, 4, 1024, None, 1024, Q, R), 1),        # block too large
    ((ODD, 0, 4, 16, None, 0, Q, R), 1),           # misaligned x
    ((P, 0, 4, 16, ODD, 0, Q, R), 1),              # misaligned prescale
    ((P, 0, 4, 131072 + 16, None, 0, Q, R), 2),    # row too long
    ((P, 0, 0, 16, None, 0, Q, R), 0),             # no rows: nothing to do
])
def test_quantize_rows_validation(L, args, expect):
    _cpu_only()
    assert L.qlin_quantize_rows(*args, None) == expect


def test_product_validation(L):
    _cpu_only()
    # forward: K beyond the int32-exact contraction bound
    assert L.qlin_fwd(P, Q, R, S, None, 4, 16, 131072, P, None) == 2
    # dX: N (its contraction) beyond the bound
    assert L.qlin_bwd_dx(P, Q, R, 4, 131072, 16, 0, S, None) == 2
    # dW: M (its contraction) beyond the bound
    assert L.qlin_bwd_dw(P, Q, R, 131072, 16, 16, S, None) == 2
    assert L.qlin_fwd(P, Q, R, S, None, 4, 24, 16, P, None) == 1     # N % 16
    assert L.qlin_fwd(P, Q, R, S, None, 4, 16, 8, P, None) == 1      # K % 16
    assert L.qlin_fwd(P, None, R, S, None, 4, 16, 16, P, None) == 1  # null sx
    assert L.qlin_fwd(P, Q, R, S, None, -1, 16, 16, P, None) == 1    # negative M
    assert L.qlin_fwd(P, Q, R, S, None, 0, 16, 16, P, None) == 0     # M = 0: no-op
    assert L.qlin_bwd_dx(P, Q, R, 0, 16, 16, 0, S, None) == 0
    assert L.qlin_bwd_dx(P, Q, R, 4, 16, 96, 64, S, None) == 1     # block does not divide K
    assert L.qlin_bwd_dx(P, Q, R, 4, 16, 96, 3, S, None) == 1      # not a power of two
    assert L.qlin_gemm_s32(7, P, Q, 4, 16, 16, R, None) == 1          # unknown product
    assert L.qlin_gemm_s32(0, ODD, Q, 4, 16, 16, R, None) == 1        # misaligned


# Operand reach of the product kernels (32-bit buffer offsets, at most
# 2,147,483,632 bytes from a base at the tile's first row or the stage's first
# contraction row).
KM_ROW_MAX = 16909312        # (128 - 1) * row + 256 <= 2,147,483,632
LONG_T_MAX = 8420976         # (256 - 1) * T + 130,944 <= 2,147,483,632


def test_operand_reach_bounds():
    lim = 2147483632
    assert 127 * KM_ROW_MAX + 256 <= lim < 127 * (KM_ROW_MAX + 16) + 256
    assert 255 * LONG_T_MAX + 130944 <= lim < 255 * (LONG_T_MAX + 16) + 130944


def test_product_operand_reach(L):
    _cpu_only()
    F = lambda i: (i + 1) << 40     # widely spaced fake addresses
    past = KM_ROW_MAX + 16
    # dX: qw is read down its columns, rows of K bytes
    assert L.qlin_bwd_dx(F(0), F(1), F(2), 4, 128, past, 0, F(3), None) == 2
    assert L.qlin_gemm_s32(1, F(0), F(2), 4, 128, past, F(3), None) == 2
    assert L.qlin_bwd_dx(F(0), F(1), F(2), 0, 128, KM_ROW_MAX, 0, F(3), None) == 0
    # dW: qg2 (rows of N bytes) and qx (rows of K bytes), both down their columns
    assert L.qlin_bwd_dw(F(0), F(1), F(2), 128, past, 16, F(3), None) == 2
    assert L.qlin_bwd_dw(F(0), F(1), F(2), 128, 16, past, F(3), None) == 2
    assert L.qlin_gemm_s32(2, F(0), F(2), 128, 16, past, F(3), None) == 2
    # a contraction of 127 rows reaches less far: accepted up to the row count
    # bound (the call then fails to launch here, where no GPU exists)
    assert L.qlin_bwd_dw(F(0), F(1), F(2), 127, 16, past, F(3), None) != 2
    # qlin_product_ws past the int32 bound: the forward and dX contraction is
    # also the row stride of their contiguous operand
    C = 4096
    def ws_call(op, M, N, K, ws):
        return L.qlin_product_ws(op, F(0), F(1), F(2), F(4) if op == 0 else None, None, M, N, K,
                                 0, F(3), ws, C + 8 * 256 * 256 * 16, None)
    assert ws_call(0, 256, 16, LONG_T_MAX + 16, F(5)) == 2
    assert ws_call(1, 256, LONG_T_MAX + 16, 16, F(5)) == 2
    assert ws_call(0, 256, 16, LONG_T_MAX, None) == 1      # within reach: the workspace is next
    assert ws_call(1, 256, LONG_T_MAX, 16, None) == 1
    assert ws_call(0, 255, 16, LONG_T_MAX + 16, None) == 1  # 255 rows reach less far
    # a long dW contraction only moves the base: its reach is that of N and K
    assert ws_call(2, 1 << 24, 16, past, F(5)) == 2
    assert ws_call(2, 1 << 24, 16, 16, None) == 1


def test_stream_copy_validation(L):
    _cpu_only()
    assert L.qlin_stream_copy(P, Q, 24, None) == 1          # not a multiple of 16
    assert L.qlin_stream_copy(ODD, Q, 32, None) == 1        # misaligned
    assert L.qlin_stream_copy(P, P + 16, 64, None) == 1     # overlapping
    assert L.qlin_stream_copy(None, Q, 16, None) == 1
    assert L.qlin_stream_copy(None, None, 0, None) == 0     # nothing to copy


def test_mfma_ceiling_validation(L):
    _cpu_only()
    assert L.qlin_mfma_ceiling(P, Q, 0, 10, None) == 1             # no workgroups
    assert L.qlin_mfma_ceiling(P, Q, 65536, 10, None) == 1
    assert L.qlin_mfma_ceiling(P, Q, 4, 0, None) == 1              # no repetitions
    assert L.qlin_mfma_ceiling(P, Q, 4, (1 << 20) + 1, None) == 1
    assert L.qlin_mfma_ceiling(None, Q, 4, 10, None) == 1
    assert L.qlin_mfma_ceiling(P, None, 4, 10, None) == 1
    assert L.qlin_mfma_ceiling(ODD, Q, 4, 10, None) == 1           # misaligned
    assert L.qlin_mfma_ceiling(P, P + 1024, 4, 10, None) == 1      # out overlaps the fragments


def test_weight_norm_validation(L):
    _cpu_only()
    T = 0x50000
    assert L.qlin_wn_init(P, Q, 4, 24, R, S, None) == 1              # K % 16
    assert L.qlin_wn_init(P, Q, 4, 16, R, R, None) == 1              # g aliases sw
    assert L.qlin_wn_init(P, None, 4, 16, R, S, None) == 1           # no row scales
    assert L.qlin_wn_init(P, Q, 4, 32784, R, S, None) == 2           # row too long
    assert L.qlin_wn_init(P, Q, 0, 16, R, S, None) == 0
    assert L.qlin_wn_sgd_requant(P, Q, R, S, T, 4, 16, 1e-3, 0, 0, Q, None, None) == 1  # bias w/o db
    assert L.qlin_wn_sgd_requant(P, Q, R, S, T, 4, 16, float("inf"), 0, 0, None, None, None) == 1
    assert L.qlin_wn_sgd_requant(P, Q, Q, S, T, 4, 16, 1e-3, 0, 0, None, None, None) == 1  # s = g
    assert L.qlin_wn_sgd_requant(ODD, Q, R, S, T, 4, 16, 1e-3, 0, 0, None, None, None) == 1
    assert L.qlin_wn_sgd_requant(P, Q, R, S, T, 4, 32784, 1e-3, 0, 0, None, None, None) == 2
    assert L.qlin_wn_sgd_requant(P, Q, R, S, T, 0, 16, 1e-3, 0, 0, None, None, None) == 0


def test_sgd_and_hadamard_validation(L):
    _cpu_only()
    assert L.qlin_sgd_requant(P, Q, R, 4, 16, 1e-3, 0, 0, S, None, None) == 1    # bias w/o db
    assert L.qlin_sgd_requant(P, Q, R, 4, 24, 1e-3, 0, 0, None, None, None) == 1  # K % 16
    assert L.qlin_sgd_requant(P, Q, R, 4, 16, float("nan"), 0, 0, None, None, None) == 1
    assert L.qlin_sgd_requant(P, Q, R, 0, 16, 1e-3, 0, 0, None, None, None) == 0
    assert L.qlin_hadamard(P, 0, 4, 128, 0, Q, None) == 1        # block 0 is not a rotation
    assert L.qlin_hadamard(P, 0, 4, 96, 64, Q, None) == 1
    assert L.qlin_hadamard(P, 1, 4, 128, 128, P, None) == 1      # bf16 -> fp32 cannot be in place
    assert L.qlin_hadamard(P, 0, 0, 128, 128, P, None) == 0
    assert L.qlin_quantize_cols(P, 0, 4, 16, None, Q, R, R, None) == 1   # s aliases col_sum
    assert L.qlin_quantize_cols(P, 0, 4, 20, None, Q, R, None, None) == 1


def test_quantize_grad_validation(L):
    _cpu_only()
    # dy, dtype, rows, cols, sw, sx, q1, s1, q2, s2, col_sum
    ok = (P, 0, 4, 16, Q, R, S, R + 64, 0x50000, 0x60000, 0x70000)
    def call(**kw):
        a = list(ok)
        names = ["dy", "dtype", "rows", "cols", "sw", "sx", "q1", "s1", "q2", "s2", "col_sum"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return L.qlin_quantize_grad(*a, None)
    assert call(dy=None) == 1
    assert call(dtype=2) == 1
    assert call(rows=-1) == 1
    assert call(cols=24) == 1                     # not a multiple of 16
    assert call(sw=None) == 1                     # weight scales are required
    assert call(sx=None) == 1
    assert call(s2=None) == 1
    assert call(q2=P + 16) == 1                   # q2 (scratch) overlaps dy
    assert call(q2=S) == 1                        # q2 overlaps q1
    assert call(col_sum=0x60000) == 1             # col_sum aliases s2
    assert call(dy=ODD) == 1
    far = {k: (i + 1) << 32 for i, k in enumerate(["dy", "sw", "sx", "q1", "s1", "q2", "s2",
                                                     "col_sum"])}
    assert call(cols=131072 + 16, **far) == 2     # row longer than the row quantizer takes
    assert call(rows=1 << 21, **far) == 2         # beyond the column pass's grid


def test_adamw_validation(L):
    _cpu_only()
    # qw, sw, dw, m, v, N, K, lr, b1, b2, eps, wd, seed, step, bias, db, bm, bv
    base = [P, Q, R, S, 0x50000, 4, 16, 1e-3, 0.9, 0.999, 1e-8, 0.01, 0, 1, None, None, None,
            None]
    names = ["qw", "sw", "dw", "m", "v", "N", "K", "lr", "b1", "b2", "eps", "wd", "seed", "step",
             "bias", "db", "bm", "bv"]
    def call(**kw):
        a = list(base)
        for k, val in kw.items():
            a[names.index(k)] = val
        return L.qlin_adamw_requant(*a, None)
    assert call(step=0) == 1                      # steps count from 1
    assert call(b1=1.0) == 1
    assert call(b2=-0.1) == 1
    assert call(eps=0.0) == 1
    assert call(wd=-1.0) == 1
    assert call(lr=float("nan")) == 1
    assert call(K=24) == 1
    assert call(m=None) == 1
    assert call(v=S + 16) == 1                    # moments overlap
    assert call(bias=0x60000) == 1                # bias without db and its moments
    assert call(bias=0x60000, db=0x70000, bm=0x80000) == 1
    assert call(N=0, qw=None, dw=None, m=None, v=None) == 0


def test_dequantize_weight_validation(L):
    _cpu_only()
    assert L.qlin_dequantize_weight(P, Q, 4, 24, 0, R, None) == 1        # K % 16
    assert L.qlin_dequantize_weight(P, Q, 4, 96, 64, R, None) == 1       # block does not divide K
    assert L.qlin_dequantize_weight(P, Q, 4, 128, 3, R, None) == 1       # not a power of two
    assert L.qlin_dequantize_weight(None, Q, 4, 128, 0, R, None) == 1
    assert L.qlin_dequantize_weight(P, Q, 4, 128, 0, P + 16, None) == 1  # w overlaps the codes
    assert L.qlin_dequantize_weight(P, Q, 0, 128, 128, R, None) == 0


def test_product_ws_validation(L):
    _cpu_only()
    F = lambda i: (i + 1) << 33     # widely spaced fake addresses
    C, BLK = 4096, 256 * 256 * 4       # counter area; one tile of int32 partial sums
    # beyond the int32 bound: the counter area, then 8 bytes per output
    assert L.qlin_product_ws_bytes(2, 200000, 16, 32) == C + 8 * 16 * 32
    assert L.qlin_product_ws_bytes(0, 4, 16, 262144) == C + 8 * 4 * 16
    # within it: the partial sums of the split tiles of the last round
    assert L.qlin_product_ws_bytes(0, 12000, 7168, 5376) == C + 36 * 3 * BLK  # 1316 tiles
    assert L.qlin_product_ws_bytes(1, 12000, 7168, 5376) == 0     # 987 tiles: 219 left, no split
    assert L.qlin_product_ws_bytes(2, 12000, 7168, 5376) == C + 76 * 2 * BLK  # 588 tiles
    assert L.qlin_product_ws_bytes(2, 8192, 14336, 4096) == C + 128 * 2 * BLK  # 896 tiles
    assert L.qlin_product_ws_bytes(1, 8192, 14336, 4096) == 0     # 512 tiles: whole rounds
    assert L.qlin_product_ws_bytes(2, 1000, 16, 32) == C + 2 * BLK   # 8 stages in 2 pieces
    assert L.qlin_product_ws_bytes(2, 100, 16, 32) == 0           # one stage: nothing to split
    assert L.qlin_product_ws_bytes(0, 16, 7168, 5376) == 0        # weight-streaming kernel
    assert L.qlin_product_ws_bytes(0, 1792, 7168, 5376) == 0      # 196 tiles: 256 / 196 < 2 pieces
    # op, a, srow, b, scol, bias, M, N, K, had, out, ws, ws_bytes
    long_dw = [2, F(0), F(1), F(2), None, None, 200000, 16, 32, 0, F(3), F(4), C + 8 * 16 * 32]
    def call(**kw):
        a = list(long_dw)
        names = ["op", "a", "srow", "b", "scol", "bias", "M", "N", "K", "had", "out", "ws",
                 "ws_bytes"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return L.qlin_product_ws(*a, None)
    assert call(op=3) == 1
    assert call(scol=F(5)) == 1                     # column scales: forward only
    assert call(had=128) == 1                       # rotation: dX only
    assert call(ws=None) == 1                       # a long contraction needs the workspace
    assert call(ws_bytes=C + 8 * 16 * 32 - 8) == 1  # too small
    assert call(ws=F(3) + 16) == 1                  # overlaps the output
    assert call(K=24) == 1
    assert call(M=1 << 31) == 2                     # beyond the longest contraction
    # a within-bound product that splits its last round needs the workspace
    need = C + 36 * 3 * BLK
    split_fwd = dict(op=0, M=12000, N=7168, K=5376, scol=F(5), ws_bytes=need)
    assert call(**split_fwd, ws=None) == 1
    assert call(**{**split_fwd, "ws_bytes": need - 1}) == 1
    assert call(**split_fwd, ws=F(3) + 64) == 1      # overlaps the output


def test_huge_sizes_are_rejected_without_overflow(L):
    """Sizes whose byte counts overflow 64 bits are rejected: the argument
    checks saturate instead of wrapping (with wrapping, (2^62 + 16)^2 * 4
    would read as 1024 bytes and such calls would pass).  Buffers that large
    necessarily overlap the other arguments (fake addresses 2^40 apart), which
    is what rejects most of them; otherwise the size limits do."""
    _cpu_only()
    F = lambda i: (i + 1) << 40
    big = (1 << 62) + 16          # a multiple of 16 whose products overflow
    assert L.qlin_quantize_grad(F(0), 1, big, 1 << 40, F(1), F(2), F(3), F(4), F(5), F(6),
                                None, None) == 1
    # fp32 hadamard has no alias check: rows * cols saturates past the grid limit
    assert L.qlin_hadamard(F(0), 0, 1 << 40, big, 16, F(1), None) == 2
    assert L.qlin_dequantize_weight(F(0), F(1), big, big, 0, F(2), None) == 1
    assert L.qlin_wn_init(F(0), F(1), big, 16, F(2), F(3), None) == 1
    assert L.qlin_adamw_requant(F(0), F(1), F(2), F(3), F(4), big, big, 1e-3, 0.9, 0.999,
                                1e-8, 0.0, 0, 1, None, None, None, None, None) == 1
    # products: dimensions past 2^30 have no workspace size and are unsupported
    assert L.qlin_product_ws_bytes(0, 1 << 31, 1 << 40, 1 << 40) == 0
    assert L.qlin_product_ws_bytes(0, 1 << 30, 1 << 30, 1 << 30) == 4096 + 8 * (1 << 60)
    assert L.qlin_product_ws(0, F(0), F(1), F(2), F(3), None, 1 << 31, big, big, 0, F(4),
                             F(5), 1 << 20, None) == 2
    # raw products with 2^22 x 2^22 output tiles (each dimension allowed)
    assert L.qlin_gemm_s32(0, F(0), F(1), 1 << 30, 1 << 30, 16, F(2), None) == 2
    assert L.qlin_gemm_s32(0, F(0), F(1), 1 << 24, 1 << 23, 16, F(2), None) == 2   # 2^31 tiles
    # overlapping ranges near the top of the address space, whose ends would
    # wrap past 2^64, are still seen to overlap
    top = (1 << 64) - (1 << 20)
    assert L.qlin_stream_copy(top, top - (1 << 21), 1 << 30, None) == 1
