"""Physically contiguous device buffers for the large arrays of the emulated
ranks (send, expert-batch, expert-output and return buffers).

The HIP runtime grants a physically contiguous allocation through
hipExtMallocWithFlags with hipDeviceMallocContiguous. On the MI355X the
kernels that scatter rows into those buffers run faster on them than on the
caching allocator's blocks (at the DS-V3 shape the pack about 77 against
81 us and the expert batch copy about 137-145 against 140-148 us per rank
share, over fresh processes), so the emulation asks for them once, at
set-up, as a deployment would for its long-lived communication buffers.

The functions are looked up through libmoe_ep.so, so they belong to the HIP
runtime that the library's kernels are launched with. A block is freed
(hipFree, which waits for the device) when the last tensor over it is gone;
nothing is freed at interpreter exit, where the process ends anyway.
"""
from __future__ import annotations

import ctypes
import weakref
from typing import Optional, Sequence

import torch

from . import binding as B

HIP_DEVICE_MALLOC_CONTIGUOUS = 0x4
_fns = None


def _hip():
    global _fns
    if _fns is None:
        lib = B.load()
        alloc = lib.hipExtMallocWithFlags
        alloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_uint]
        alloc.restype = ctypes.c_int
        free = lib.hipFree
        free.argtypes = [ctypes.c_void_p]
        free.restype = ctypes.c_int
        last = lib.hipGetLastError
        last.argtypes = []
        last.restype = ctypes.c_int
        _fns = (alloc, free, last)
    return _fns


def _free(ptr: int):
    _hip()[1](ctypes.c_void_p(ptr))


class _Block:
    """One contiguous allocation, exposed to torch through the CUDA array
    interface (torch holds a reference to it for as long as a tensor views
    the memory)."""

    def __init__(self, ptr: int, nbytes: int):
        self.ptr = ptr
        self.nbytes = nbytes
        self.__cuda_array_interface__ = {"shape": (nbytes,), "typestr": "|u1",
                                         "data": (ptr, False), "version": 3}
        fin = weakref.finalize(self, _free, ptr)
        fin.atexit = False


def empty_contiguous(shape: Sequence[int], dtype: torch.dtype,
                     device) -> Optional[torch.Tensor]:
    """An uninitialised tensor over a physically contiguous allocation on
    `device`, or None when the device does not grant one (the caller then
    allocates as usual)."""
    device = torch.device(device)
    if device.type != "cuda":
        return None
    nbytes = torch.Size(shape).numel() * torch.empty((), dtype=dtype).element_size()
    if nbytes == 0:
        return None
    alloc, _, last = _hip()
    p = ctypes.c_void_p()
    with torch.cuda.device(device):
        rc = alloc(ctypes.byref(p), ctypes.c_size_t(nbytes), HIP_DEVICE_MALLOC_CONTIGUOUS)
        if rc != 0 or not p.value:
            last()          # clear the runtime's last error: the next launch must not see it
            return None
        t = torch.as_tensor(_Block(p.value, nbytes), device=device)
    if t.data_ptr() != p.value:
        raise RuntimeError("device tensor does not view the contiguous allocation")
    return t.view(dtype).view(tuple(shape))
