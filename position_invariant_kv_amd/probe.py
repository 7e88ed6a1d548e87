"""Binding of the copy-ceiling probe (libkamera_probe.so, include/kamera_probe.h).

A measurement helper, not part of the operator: it copies the bytes a
relocation call moves, in the same block pattern, with no arithmetic, so that
the operator's rate can be read against what a plain 16-byte copy reaches in
that pattern on this GPU.  Argument marshalling only.
"""

from __future__ import annotations

import ctypes

from ._abi import load_probe_library

PROBE_STATUS = {0: "KAMERA_PROBE_OK", 1: "KAMERA_PROBE_ERR_NULL", 2: "KAMERA_PROBE_ERR_ALIGN",
                4: "KAMERA_PROBE_ERR_RANGE", 7: "KAMERA_PROBE_ERR_HIP"}


class CopyProbe:
    """A prepared kamera_probe_copy_blocks call.

    src/dst: (device address, size in bytes) of the two buffers; src_off /
    dst_off: int64 device tensors of per-block byte offsets, or None for a
    sequential side (block b at b * block_bytes).  Calling it enqueues the
    copy on ``stream`` (a torch stream; None = the current stream).
    """

    def __init__(self, src, dst, nblocks: int, block_bytes: int, src_off=None, dst_off=None,
                 vectors_per_thread: int = 1):
        for name, t in (("src_off", src_off), ("dst_off", dst_off)):
            if t is not None:
                import torch
                if t.dtype != torch.int64 or not t.is_cuda or not t.is_contiguous() or t.numel() != nblocks:
                    raise ValueError(f"{name} must be a contiguous int64 GPU tensor of {nblocks} entries")
        self._lib = load_probe_library()
        self._keep = (src_off, dst_off)
        self._args = (ctypes.c_void_p(int(src[0])), int(src[1]), ctypes.c_void_p(int(dst[0])), int(dst[1]),
                      ctypes.c_void_p(0 if src_off is None else int(src_off.data_ptr())),
                      ctypes.c_void_p(0 if dst_off is None else int(dst_off.data_ptr())),
                      int(nblocks), int(block_bytes), int(vectors_per_thread))

    def __call__(self, stream=None):
        import torch
        if stream is None:
            stream = torch.cuda.current_stream()
        st = self._lib.kamera_probe_copy_blocks(*self._args, ctypes.c_void_p(int(stream.cuda_stream)))
        if st != 0:
            raise RuntimeError(f"kamera_probe_copy_blocks: {PROBE_STATUS.get(st, st)}")
