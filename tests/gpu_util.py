"""Helpers for the GPU parity tests (device transfer, poison fill, bit compare)."""
import numpy as np
import torch

POISON = 0xAA


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> contiguous device tensor (uint32 travels as int32 bits)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).cuda()
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def poisoned(shape, dtype, canary: int = 256):
    """A device buffer pre-filled with 0xAA bytes plus a canary tail; returns
    (view of the requested shape, the whole flat byte buffer)."""
    nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    raw = torch.full((nbytes + canary,), POISON, dtype=torch.uint8, device="cuda")
    view = raw[:nbytes].view(dtype).view(shape)
    return view, raw


def assert_canary(raw: torch.Tensor, nbytes: int):
    tail = raw[nbytes:].cpu().numpy()
    assert np.all(tail == POISON), "kernel wrote past the end of its output"


def assert_bits_equal(got: np.ndarray, ref: np.ndarray, what: str, zero_by_value: bool = False):
    got = np.ascontiguousarray(got)
    ref = np.ascontiguousarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if got.dtype == np.float32:
        gb, rb = got.view(np.uint32), ref.view(np.uint32)
        diff = gb != rb
        if zero_by_value:
            diff &= ~((got == 0) & (ref == 0))
    else:
        diff = got != ref
    if diff.any():
        idx = np.argwhere(diff)[:5]
        raise AssertionError(f"{what}: {int(diff.sum())} mismatches, first at {idx.tolist()}: "
                             f"got {got[tuple(idx[0])]!r} want {ref[tuple(idx[0])]!r}")
