"""Host <-> device helpers for the GPU parity tests (no arithmetic of the layer)."""
import sys

import numpy as np
import pytest


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_integer_linear_amd  # noqa: F401  (fails loudly if libqlin.so is missing)
    return torch


def dev(a):
    """numpy -> cuda tensor; uint16 arrays are bf16 bit patterns."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t):
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def announce(*parts):
    """Name the case on stdout before a GPU step (so a fault is attributable)."""
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def assert_bitwise(got, ref, what):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if got.dtype.kind == "f":
        same = got.view(np.uint32 if got.itemsize == 4 else np.uint64) == \
            ref.view(np.uint32 if ref.itemsize == 4 else np.uint64)
    else:
        same = got == ref
    if not same.all():
        idx = np.argwhere(~same)
        first = tuple(idx[0])
        raise AssertionError(f"{what}: {(~same).sum()} of {same.size} differ; first at {first}: "
                             f"got {got[first]!r} ref {ref[first]!r}")
