"""Philox4x32-10 blocks computed by an independent implementation: Triton's
``tl.philox_impl``, run on the CPU by Triton's interpreter.

Used only by the CPU tests, as a second implementation of the generator of
Salmon et al. (SC'11) against which the oracle's is compared.  Run as a
script: reads counters and keys (decimal, one block per line: c0 c1 c2 c3 k0
k1) on stdin and prints the four output words of each block.  It runs in its
own process because the interpreter must be selected before Triton is
imported.
"""
import os
import sys

os.environ["TRITON_INTERPRET"] = "1"

import numpy as np  # noqa: E402
import torch  # noqa: E402
import triton  # noqa: E402
import triton.language as tl  # noqa: E402

BLOCK = 64


@triton.jit
def _philox_blocks(c_ptr, k_ptr, o_ptr, n, BLOCK: tl.constexpr):
    i = tl.program_id(0) * BLOCK + tl.arange(0, BLOCK)
    m = i < n
    u32 = tl.uint32
    c0 = tl.load(c_ptr + 4 * i, mask=m).to(u32, bitcast=True)
    c1 = tl.load(c_ptr + 4 * i + 1, mask=m).to(u32, bitcast=True)
    c2 = tl.load(c_ptr + 4 * i + 2, mask=m).to(u32, bitcast=True)
    c3 = tl.load(c_ptr + 4 * i + 3, mask=m).to(u32, bitcast=True)
    k0 = tl.load(k_ptr + 2 * i, mask=m).to(u32, bitcast=True)
    k1 = tl.load(k_ptr + 2 * i + 1, mask=m).to(u32, bitcast=True)
    x0, x1, x2, x3 = tl.philox_impl(c0, c1, c2, c3, k0, k1, 10)
    tl.store(o_ptr + 4 * i, x0.to(tl.int32, bitcast=True), mask=m)
    tl.store(o_ptr + 4 * i + 1, x1.to(tl.int32, bitcast=True), mask=m)
    tl.store(o_ptr + 4 * i + 2, x2.to(tl.int32, bitcast=True), mask=m)
    tl.store(o_ptr + 4 * i + 3, x3.to(tl.int32, bitcast=True), mask=m)


def blocks(ctr, key):
    """ctr [n, 4], key [n, 2] (uint32) -> [n, 4] uint32 output words."""
    ctr = np.ascontiguousarray(ctr, np.uint32)
    key = np.ascontiguousarray(key, np.uint32)
    n = ctr.shape[0]
    out = torch.zeros(4 * n, dtype=torch.int32)
    _philox_blocks[((n + BLOCK - 1) // BLOCK,)](
        torch.from_numpy(ctr.view(np.int32).ravel().copy()),
        torch.from_numpy(key.view(np.int32).ravel().copy()), out, n, BLOCK=BLOCK)
    return out.numpy().view(np.uint32).reshape(n, 4)


if __name__ == "__main__":
    rows = [list(map(int, line.split())) for line in sys.stdin if line.strip()]
    a = np.array(rows, np.uint64).astype(np.uint32)
    for r in blocks(a[:, :4], a[:, 4:6]):
        print(" ".join(str(int(v)) for v in r))
