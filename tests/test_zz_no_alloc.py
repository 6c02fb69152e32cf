"""The allocation-free product call (qlin_product_noalloc, for callers that
cannot allocate device memory) against qlin_product_ws, bit for bit, through
the C ABI: each case makes two calls in a row on the shared scratch, the
second with a smaller input, and compares both with the workspace call on
the same inputs."""
import ctypes

import numpy as np
import pytest

from tests.gpu_util import announce, torch_cuda

pytestmark = pytest.mark.gpu

FWD, DX, DW = 0, 1, 2


def _inputs(T, op, M, N, K, seed, bias):
    g = T.Generator(device="cuda")
    g.manual_seed(seed)
    codes = lambda r, c: T.randint(-127, 128, (r, c), dtype=T.int8, device="cuda", generator=g)
    scales = lambda n: T.rand(n, device="cuda", generator=g) * 1e-2 + 1e-4
    if op == FWD:
        a, b, srow = codes(M, K), codes(N, K), scales(M)
    elif op == DX:
        a, b, srow = codes(M, N), codes(N, K), scales(M)
    else:
        a, b, srow = codes(M, N), codes(M, K), scales(N)
    scol = scales(N) if op == FWD else None
    bvec = T.randn(N, device="cuda", generator=g) if (op == FWD and bias) else None
    shape = {FWD: (M, N), DX: (M, K), DW: (N, K)}[op]
    return a, b, srow, scol, bvec, shape


def _noalloc(T, op, a, srow, b, scol, bias, M, N, K, had, out):
    """The raw C call: device pointers, sizes, the current stream."""
    from w8a8_integer_linear_amd import _native
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    return _native.lib().qlin_product_noalloc(
        op, p(a), p(srow), p(b), p(scol), p(bias), M, N, K, had, p(out),
        ctypes.c_void_p(T.cuda.current_stream().cuda_stream))


def _ws_call(T, op, a, srow, b, scol, bias, M, N, K, had):
    from w8a8_integer_linear_amd import _native
    return _native.qlin_product_ws(op, a, srow, b, M, N, K, scol=scol, bias=bias, had_block=had)


# (op, M, N, K, had, bias): first call, then a smaller second call.
CASES = [
    # dW splits its last round: 76 tiles in 2 pieces, then 32 tiles in 2.
    ("dw split", (DW, 2048, 7168, 5376, 0, False), (DW, 1000, 2048, 1024, 0, False)),
    # forward with 36 tiles in 3 pieces, then 24 tiles in 2 with a bias.
    ("fwd split", (FWD, 12000, 7168, 5376, 0, True), (FWD, 600, 2048, 1024, 0, True)),
    # dX rotated back: 160 pieces fill the scratch exactly; then block 64.
    ("dx split", (DX, 4096, 7168, 5376, 128, False), (DX, 512, 1024, 2048, 64, False)),
    # contractions past the int32 bound: int64 sums in the scratch.
    ("dw long", (DW, 140000, 64, 256, 0, False), (DW, 131200, 32, 128, 0, False)),
    ("fwd long", (FWD, 64, 48, 262144, 0, True), (FWD, 16, 32, 140000, 0, False)),
    # 256 pieces do not fit: the unbalanced product, then a split one.
    ("dw too many pieces", (DW, 8192, 14336, 4096, 0, False), (DW, 2048, 7168, 5376, 0, False)),
]


@pytest.mark.parametrize("name,first,second", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_call(name, first, second):
    T = torch_cuda()
    for call, (op, M, N, K, had, bias) in enumerate((first, second)):
        announce("noalloc", name, call, op, M, N, K, had)
        a, b, srow, scol, bvec, shape = _inputs(T, op, M, N, K, 100 * call + op, bias)
        out = T.full(shape, float("nan"), device="cuda")
        st = _noalloc(T, op, a, srow, b, scol, bvec, M, N, K, had, out)
        assert st == 0, st
        ref = _ws_call(T, op, a, srow, b, scol, bvec, M, N, K, had)
        T.cuda.synchronize()
        assert T.equal(out.view(T.int32), ref.view(T.int32)), (name, call)


def test_noalloc_rejects_long_sums_past_the_scratch():
    """A long contraction whose int64 sums exceed the scratch is refused
    before anything runs; the output is untouched."""
    from w8a8_integer_linear_amd import _native
    T = torch_cuda()
    M, N, K = 140000, 2048, 4096             # 8 * N * K = 64 MiB of sums
    assert 4096 + 8 * N * K > _native.NOALLOC_SCRATCH_BYTES
    announce("noalloc reject", M, N, K)
    a, b, srow, _, _, shape = _inputs(T, DW, M, N, K, 7, False)
    out = T.full(shape, 3.0, device="cuda")
    assert _noalloc(T, DW, a, srow, b, None, None, M, N, K, 0, out) == _native.QLIN_EUNSUPPORTED
    T.cuda.synchronize()
    assert bool((out == 3.0).all())
