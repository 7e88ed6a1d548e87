"""Python binding of the Kamera C-ABI library (libkamera.so, include/kamera.h).

Argument marshalling only: every step of the operator runs in the HIP kernels
of the library.  Tensors are PyTorch tensors on the GPU (PyTorch provides
device memory and the current stream); bfloat16 data is passed as raw bits.
If the library is missing this module raises: there is no fallback.

Entry points mirror the C names:

* ``relocate``        R(delta) only (sliding-window survival)
* ``relocate_patch``  R(delta) x + U V^T
* ``reorder``         output slot k holds store chunk perm[k] at base + k*T
* ``recall``          store chunk ids[i] rehydrated at target_pos[i]
* ``relocate_patch_varlen`` / ``recall_varlen``  the same over a store of
  variable-length chunks (packed rows [total_rows, F] per stream)
* ``form_patch``      rank-m factors of KV(B|A) - R(delta) KV(B|empty) (patch formation)

Paged calls take ``page_order``: "auto" (the default) allocates the page-order
scratch of kamera_dst (n * ceil(T/P) int32) with the prepared call, so the
library may write the pool in ascending page order; None keeps the page-table
order; an int32 tensor is used as given.  The output is the same either way.

Kamera summary on gist.science (paper 2606.23581), section 2 (operator) and
section 3 (window operations).
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

from ._abi import (KameraAttnPool, KameraDst, KameraFactors, KameraLayout, KameraPatch, KameraSketch, KameraSrc,
                   KameraVarlen, STATUS, load_library, lib_path)

ROPE_HALF = 0
ROPE_INTERLEAVED = 1

EW_PAGE, EW_OFFSET, EW_CHUNK = 1, 2, 4


class KameraError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status})")


@dataclass(frozen=True)
class Layout:
    num_layers: int
    num_heads: int
    head_dim: int
    rope_offset: int
    rope_dim: int
    rope_base: float
    num_streams: int
    rope_style: int = ROPE_HALF

    @property
    def row_width(self) -> int:
        return self.num_heads * self.head_dim

    def c(self) -> KameraLayout:
        return KameraLayout(self.num_layers, self.num_heads, self.head_dim, self.rope_offset,
                            self.rope_dim, self.rope_style, float(self.rope_base), self.num_streams)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _check_dev(name, t, dtype_names, ndim=None):
    import torch
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if str(t.dtype).replace("torch.", "") not in dtype_names:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtype_names}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _bf16_like(name, t, ndim):
    _check_dev(name, t, ("bfloat16", "int16", "uint16"), ndim)


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


def _src_struct(layout: Layout, src, canon_pos):
    S = layout.num_streams
    if len(src) != S:
        raise ValueError(f"need {S} source tensors")
    ref = src[0]
    for k, t in enumerate(src):
        _bf16_like(f"src[{k}]", t, 4)
        if t.shape != ref.shape or t.stride() != ref.stride():
            raise ValueError("source streams must share shape and strides")
    ns, L, T, F = ref.shape
    if L != layout.num_layers or F != layout.row_width:
        raise ValueError(f"source shape {tuple(ref.shape)} does not match the layout")
    if ref.stride(3) != 1 or (T > 1 and ref.stride(2) != F):
        raise ValueError("source rows must be contiguous [T][F]")
    _check_dev("canon_pos", canon_pos, ("int64",), 1)
    if canon_pos is not None and canon_pos.numel() != ns:
        raise ValueError("canon_pos must have n_store entries")
    rows = (ctypes.c_void_p * 2)(_ptr(src[0]), _ptr(src[1]) if S > 1 else 0)
    return KameraSrc(rows, ref.stride(0), ref.stride(1), T, ns, _ptr(canon_pos)), ns, T


def _patch_struct(layout: Layout, u, v, ns, T):
    if u is None and v is None:
        return KameraPatch(0, (ctypes.c_void_p * 2)(0, 0), (ctypes.c_void_p * 2)(0, 0)), 0
    S = layout.num_streams
    if len(u) != S or len(v) != S:
        raise ValueError(f"need {S} U and {S} V factor tensors")
    m = u[0].shape[-1]
    for k in range(S):
        _bf16_like(f"u[{k}]", u[k], 4)
        _bf16_like(f"v[{k}]", v[k], 4)
        if tuple(u[k].shape) != (ns, layout.num_layers, T, m) or not u[k].is_contiguous():
            raise ValueError(f"u[{k}] must be contiguous [n_store, L, T, m]")
        if tuple(v[k].shape) != (ns, layout.num_layers, layout.row_width, m) or not v[k].is_contiguous():
            raise ValueError(f"v[{k}] must be contiguous [n_store, L, F, m]")
    us = (ctypes.c_void_p * 2)(_ptr(u[0]), _ptr(u[1]) if S > 1 else 0)
    vs = (ctypes.c_void_p * 2)(_ptr(v[0]), _ptr(v[1]) if S > 1 else 0)
    return KameraPatch(m, us, vs), m


def _page_order(page_order, page_size, n, T, device):
    """Scratch of the destination order (kamera_dst.page_order): "auto" allocates
    it for a paged pool, None leaves it out, a tensor is used as given."""
    if not page_size:
        return None
    need = n * (-(-T // page_size)) if T else 0
    if isinstance(page_order, str):
        if page_order != "auto":
            raise ValueError(f"page_order must be 'auto', None or an int32 tensor, not {page_order!r}")
        import torch
        return torch.empty(max(need, 1), dtype=torch.int32, device=device)
    if page_order is None:
        return None
    _check_dev("page_order", page_order, ("int32",), 1)
    if page_order.numel() < need or not page_order.is_contiguous():
        raise ValueError(f"page_order must be a contiguous int32 tensor of at least {need} entries")
    return page_order


def _check_scratch(check_scratch, error_word, page_size, n, T, device):
    """Scratch of the content checks (kamera_dst.check_scratch): used only with an
    error word.  "auto" allocates it then, None leaves it out, a tensor is used
    as given."""
    if error_word is None:
        return None
    need = n * (-(-T // page_size) if (page_size and T) else 0) + n
    if isinstance(check_scratch, str):
        if check_scratch != "auto":
            raise ValueError(f"check_scratch must be 'auto', None or an int32 tensor, not {check_scratch!r}")
        import torch
        return torch.empty(max(need, 1), dtype=torch.int32, device=device)
    if check_scratch is None:
        return None
    _check_dev("check_scratch", check_scratch, ("int32",), 1)
    if check_scratch.numel() < need or not check_scratch.is_contiguous():
        raise ValueError(f"check_scratch must be a contiguous int32 tensor of at least {need} entries")
    return check_scratch


def _dst_struct(layout: Layout, pool, page_size, page_table, dst_offset, error_word, n, T, page_order=None,
                check_scratch="auto"):
    S = layout.num_streams
    if len(pool) != S:
        raise ValueError(f"need {S} pool tensors")
    ref = pool[0]
    for k, t in enumerate(pool):
        _bf16_like(f"pool[{k}]", t, 3)
        if t.shape != ref.shape or t.stride() != ref.stride():
            raise ValueError("pool streams must share shape and strides")
    L, slots, F = ref.shape
    if L != layout.num_layers or F != layout.row_width:
        raise ValueError(f"pool shape {tuple(ref.shape)} does not match the layout")
    if ref.stride(2) != 1 or (slots > 1 and ref.stride(1) != F):
        raise ValueError("pool rows must be contiguous [slots][F]")
    if page_size:
        _check_dev("page_table", page_table, ("int32",), 2)
        ppc = -(-T // page_size) if T else 0
        if page_table is None or tuple(page_table.shape) != (n, ppc) or not page_table.is_contiguous():
            raise ValueError(f"page_table must be contiguous int32 [{n}, {ppc}]")
    else:
        _check_dev("dst_offset", dst_offset, ("int64",), 1)
        if dst_offset is None or dst_offset.numel() != n:
            raise ValueError(f"dst_offset must be int64 [{n}]")
    _check_dev("error_word", error_word, ("int32",), 1)
    rows = (ctypes.c_void_p * 2)(_ptr(pool[0]), _ptr(pool[1]) if S > 1 else 0)
    chk = _check_scratch(check_scratch, error_word, page_size, n, T, ref.device)
    d = KameraDst(rows, ref.stride(0), slots, int(page_size), _ptr(page_table),
                  _ptr(dst_offset), _ptr(error_word), _ptr(page_order), _ptr(chk))
    d._check_scratch = chk  # kept alive with the struct
    return d


def _idx(name, t, dtype, n):
    _check_dev(name, t, (dtype,), 1)
    if t is None or t.numel() != n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of {n} entries")


class Call:
    """One validated, marshalled call of an entry point.

    Building it checks every tensor and fills the C structs once; calling it
    only passes the prepared arguments to the library (a few microseconds of
    host time), on ``stream`` or, if None, on the stream bound at preparation
    or torch's current stream.  The tensors must stay alive and unchanged in
    shape while the Call is used.
    """

    __slots__ = ("_fn", "_args", "_keep", "_name", "_stream")

    def __init__(self, name, fn, args, keep, stream):
        self._name = name
        self._fn = fn
        self._args = args
        self._keep = keep
        self._stream = None if stream is None else _stream_handle(stream)

    def __call__(self, stream=None):
        if stream is not None:
            h = _stream_handle(stream)
        elif self._stream is not None:
            h = self._stream
        else:
            h = _stream_handle(None)
        status = self._fn(*self._args, h)
        if status != 0:
            raise KameraError(status, self._name)


def prepare_relocate(layout: Layout, src, delta, pool, *, page_size=0, page_table=None, dst_offset=None,
                     canon_pos=None, error_word=None, page_order="auto", check_scratch="auto", stream=None) -> Call:
    """Prepared kamera_relocate: pool <- R(delta_i) src[i] for every output chunk i."""
    lib = load_library()
    n = delta.numel() if delta is not None else 0
    _idx("delta", delta, "int64", n)
    s, ns, T = _src_struct(layout, src, canon_pos)
    order = _page_order(page_order, page_size, n, T, pool[0].device)
    d = _dst_struct(layout, pool, page_size, page_table, dst_offset, error_word, n, T, order,
                    check_scratch=check_scratch)
    lay = layout.c()
    args = (ctypes.byref(lay), ctypes.byref(s), n, ctypes.c_void_p(_ptr(delta)), ctypes.byref(d))
    return Call("kamera_relocate", lib.kamera_relocate, args,
                (lay, s, d, src, delta, pool, page_table, dst_offset, canon_pos, error_word, order), stream)


def prepare_relocate_patch(layout: Layout, src, delta, u, v, pool, *, page_size=0, page_table=None,
                           dst_offset=None, canon_pos=None, error_word=None,
                           page_order="auto", check_scratch="auto", stream=None) -> Call:
    """Prepared kamera_relocate_patch: pool <- R(delta_i) src[i] + U_i V_i^T."""
    lib = load_library()
    n = delta.numel()
    _idx("delta", delta, "int64", n)
    s, ns, T = _src_struct(layout, src, canon_pos)
    pt, _ = _patch_struct(layout, u, v, ns, T)
    order = _page_order(page_order, page_size, n, T, pool[0].device)
    d = _dst_struct(layout, pool, page_size, page_table, dst_offset, error_word, n, T, order,
                    check_scratch=check_scratch)
    lay = layout.c()
    args = (ctypes.byref(lay), ctypes.byref(s), n, ctypes.c_void_p(_ptr(delta)), ctypes.byref(pt),
            ctypes.byref(d))
    return Call("kamera_relocate_patch", lib.kamera_relocate_patch, args,
                (lay, s, pt, d, src, delta, u, v, pool,
                 page_table, dst_offset, canon_pos, error_word, order), stream)


def prepare_relocate_patch_noalloc(layout: Layout, src, delta, u, v, pool, *, page_size=0, page_table=None,
                                   dst_offset=None, canon_pos=None, error_word=None, stream=None) -> Call:
    """Prepared kamera_relocate_patch_noalloc: kamera_relocate_patch with the
    call's scratch (page order, content checks) in the library's static device
    array instead of caller memory; nothing is allocated for it."""
    lib = load_library()
    n = delta.numel()
    _idx("delta", delta, "int64", n)
    s, ns, T = _src_struct(layout, src, canon_pos)
    pt, _ = _patch_struct(layout, u, v, ns, T)
    d = _dst_struct(layout, pool, page_size, page_table, dst_offset, error_word, n, T, None, check_scratch=None)
    lay = layout.c()
    args = (ctypes.byref(lay), ctypes.byref(s), n, ctypes.c_void_p(_ptr(delta)), ctypes.byref(pt),
            ctypes.byref(d))
    return Call("kamera_relocate_patch_noalloc", lib.kamera_relocate_patch_noalloc, args,
                (lay, s, pt, d, src, delta, u, v, pool, page_table, dst_offset, canon_pos, error_word), stream)


def prepare_reorder(layout: Layout, src, perm, base_pos, pool, *, u=None, v=None, page_size=0,
                    page_table=None, dst_offset=None, canon_pos=None, error_word=None,
                    page_order="auto", check_scratch="auto", stream=None) -> Call:
    """Prepared kamera_reorder: output k <- chunk perm[k] at base_pos + k*T, with its orbit patch."""
    lib = load_library()
    n = perm.numel()
    _idx("perm", perm, "int32", n)
    s, ns, T = _src_struct(layout, src, canon_pos)
    pt, m = _patch_struct(layout, u, v, ns, T)
    order = _page_order(page_order, page_size, n, T, pool[0].device)
    d = _dst_struct(layout, pool, page_size, page_table, dst_offset, error_word, n, T, order,
                    check_scratch=check_scratch)
    lay = layout.c()
    args = (ctypes.byref(lay), ctypes.byref(s), n, ctypes.c_void_p(_ptr(perm)),
            ctypes.c_int64(int(base_pos)), ctypes.byref(pt) if m else None, ctypes.byref(d))
    return Call("kamera_reorder", lib.kamera_reorder, args,
                (lay, s, pt, d, src, perm, u, v, pool,
                 page_table, dst_offset, canon_pos, error_word, order), stream)


def prepare_recall(layout: Layout, src, chunk_ids, target_pos, pool, *, u=None, v=None, page_size=0,
                   page_table=None, dst_offset=None, canon_pos=None, error_word=None,
                   page_order="auto", check_scratch="auto", stream=None) -> Call:
    """Prepared kamera_recall: output i <- store chunk ids[i] rehydrated at target_pos[i]."""
    lib = load_library()
    n = chunk_ids.numel()
    _idx("chunk_ids", chunk_ids, "int32", n)
    _idx("target_pos", target_pos, "int64", n)
    s, ns, T = _src_struct(layout, src, canon_pos)
    pt, m = _patch_struct(layout, u, v, ns, T)
    order = _page_order(page_order, page_size, n, T, pool[0].device)
    d = _dst_struct(layout, pool, page_size, page_table, dst_offset, error_word, n, T, order,
                    check_scratch=check_scratch)
    lay = layout.c()
    args = (ctypes.byref(lay), ctypes.byref(s), n, ctypes.c_void_p(_ptr(chunk_ids)),
            ctypes.c_void_p(_ptr(target_pos)), ctypes.byref(pt) if m else None, ctypes.byref(d))
    return Call("kamera_recall", lib.kamera_recall, args,
                (lay, s, pt, d, src, chunk_ids, target_pos, u, v, pool, page_table, dst_offset, canon_pos,
                 error_word, order), stream)


def _varlen_structs(layout: Layout, src, row_offset, n_tokens, max_tokens, canon_pos, u, v):
    """kamera_src + kamera_varlen + kamera_patch of a packed variable-length store.

    src[s]: [total_rows, F] rows; store chunk c holds n_tokens[c] tokens per
    layer from row row_offset[c] on, layer by layer.  u[s]: [total_rows, m] in
    the same row order; v[s]: [n_store, L, F, m].  max_tokens (host int) bounds
    every n_tokens[c] the call uses.
    """
    S = layout.num_streams
    if len(src) != S:
        raise ValueError(f"need {S} source tensors")
    ref = src[0]
    for k, t in enumerate(src):
        _bf16_like(f"src[{k}]", t, 2)
        if t.shape != ref.shape or not t.is_contiguous():
            raise ValueError("source streams must be contiguous [total_rows, F] of one shape")
    total_rows, F = ref.shape
    if F != layout.row_width:
        raise ValueError(f"source rows of width {F} do not match the layout")
    _check_dev("row_offset", row_offset, ("int64",), 1)
    _check_dev("n_tokens", n_tokens, ("int32",), 1)
    if row_offset is None or n_tokens is None or row_offset.numel() != n_tokens.numel() or \
            not row_offset.is_contiguous() or not n_tokens.is_contiguous():
        raise ValueError("row_offset (int64) and n_tokens (int32) must be contiguous [n_store]")
    ns = n_tokens.numel()
    _check_dev("canon_pos", canon_pos, ("int64",), 1)
    if canon_pos is not None and canon_pos.numel() != ns:
        raise ValueError("canon_pos must have n_store entries")
    T = int(max_tokens)
    rows = (ctypes.c_void_p * 2)(_ptr(src[0]), _ptr(src[1]) if S > 1 else 0)
    sc = KameraSrc(rows, 0, 0, T, ns, _ptr(canon_pos))
    vl = KameraVarlen(_ptr(row_offset), _ptr(n_tokens), int(total_rows))
    if u is None and v is None:
        return sc, vl, KameraPatch(0, (ctypes.c_void_p * 2)(0, 0), (ctypes.c_void_p * 2)(0, 0)), 0, ns, T
    if len(u) != S or len(v) != S:
        raise ValueError(f"need {S} U and {S} V factor tensors")
    m = u[0].shape[-1]
    for k in range(S):
        _bf16_like(f"u[{k}]", u[k], 2)
        _bf16_like(f"v[{k}]", v[k], 4)
        if tuple(u[k].shape) != (total_rows, m) or not u[k].is_contiguous():
            raise ValueError(f"u[{k}] must be contiguous [total_rows, m]")
        if tuple(v[k].shape) != (ns, layout.num_layers, F, m) or not v[k].is_contiguous():
            raise ValueError(f"v[{k}] must be contiguous [n_store, L, F, m]")
    us = (ctypes.c_void_p * 2)(_ptr(u[0]), _ptr(u[1]) if S > 1 else 0)
    vs = (ctypes.c_void_p * 2)(_ptr(v[0]), _ptr(v[1]) if S > 1 else 0)
    return sc, vl, KameraPatch(m, us, vs), m, ns, T


def prepare_relocate_patch_varlen(layout: Layout, src, row_offset, n_tokens, max_tokens, delta, pool, *, u=None,
                                  v=None, page_size=0, page_table=None, dst_offset=None, canon_pos=None,
                                  error_word=None, check_scratch="auto", stream=None) -> Call:
    """Prepared kamera_relocate_patch_varlen: output i <- R(delta_i) chunk i (+ U_i V_i^T), chunk i of
    n_tokens[i] tokens in a packed store."""
    lib = load_library()
    n = delta.numel()
    _idx("delta", delta, "int64", n)
    sc, vl, pt, m, ns, T = _varlen_structs(layout, src, row_offset, n_tokens, max_tokens, canon_pos, u, v)
    d = _dst_struct(layout, pool, page_size, page_table, dst_offset, error_word, n, T,
                    check_scratch=check_scratch)
    lay = layout.c()
    args = (ctypes.byref(lay), ctypes.byref(sc), ctypes.byref(vl), n, ctypes.c_void_p(_ptr(delta)),
            ctypes.byref(pt) if m else None, ctypes.byref(d))
    return Call("kamera_relocate_patch_varlen", lib.kamera_relocate_patch_varlen, args,
                (lay, sc, vl, pt, d, src, row_offset, n_tokens, delta, u, v, pool, page_table, dst_offset,
                 canon_pos, error_word), stream)


def prepare_recall_varlen(layout: Layout, src, row_offset, n_tokens, max_tokens, chunk_ids, target_pos, pool, *,
                          u=None, v=None, page_size=0, page_table=None, dst_offset=None, canon_pos=None,
                          error_word=None, check_scratch="auto", stream=None) -> Call:
    """Prepared kamera_recall_varlen: output i <- store chunk ids[i] (of n_tokens[ids[i]] tokens)
    rehydrated at target_pos[i]."""
    lib = load_library()
    n = chunk_ids.numel()
    _idx("chunk_ids", chunk_ids, "int32", n)
    _idx("target_pos", target_pos, "int64", n)
    sc, vl, pt, m, ns, T = _varlen_structs(layout, src, row_offset, n_tokens, max_tokens, canon_pos, u, v)
    d = _dst_struct(layout, pool, page_size, page_table, dst_offset, error_word, n, T,
                    check_scratch=check_scratch)
    lay = layout.c()
    args = (ctypes.byref(lay), ctypes.byref(sc), ctypes.byref(vl), n, ctypes.c_void_p(_ptr(chunk_ids)),
            ctypes.c_void_p(_ptr(target_pos)), ctypes.byref(pt) if m else None, ctypes.byref(d))
    return Call("kamera_recall_varlen", lib.kamera_recall_varlen, args,
                (lay, sc, vl, pt, d, src, row_offset, n_tokens, chunk_ids, target_pos, u, v, pool, page_table,
                 dst_offset, canon_pos, error_word), stream)


def form_patch_workspace_bytes(layout: Layout, n: int, n_tokens: int, rank: int, oversample: int) -> int:
    """Bytes of device workspace kamera_form_patch needs (raises if unsupported)."""
    b = int(load_library().kamera_form_patch_workspace(ctypes.byref(layout.c()), int(n), int(n_tokens),
                                                       int(rank), int(oversample)))
    if b < 0:
        raise KameraError(6, "kamera_form_patch_workspace")
    return b


def _prepare_form(layout: Layout, canon, target, delta, views: int, u_out, v_out, omega, oversample: int,
                  power_iters: int, workspace, stream, orbit: bool) -> Call:
    import torch
    lib = load_library()
    if views < 1 or delta.numel() % views:
        raise ValueError("views must be >= 1 and divide the number of shifts")
    n = delta.numel() // views
    _idx("delta", delta, "int64", n * views)
    cs, ns_c, T = _src_struct(layout, canon, None)
    ts, ns_t, T2 = _src_struct(layout, target, None)
    if T2 != T:
        raise ValueError("canon and target must have the same number of tokens")
    S = layout.num_streams
    if len(u_out) != S or len(v_out) != S:
        raise ValueError(f"need {S} U and {S} V output tensors")
    m = u_out[0].shape[-1]
    for k in range(S):
        _bf16_like(f"u_out[{k}]", u_out[k], 4)
        _bf16_like(f"v_out[{k}]", v_out[k], 4)
        if tuple(u_out[k].shape) != (n, layout.num_layers, T, m) or not u_out[k].is_contiguous():
            raise ValueError(f"u_out[{k}] must be contiguous [n, L, T, m]")
        if tuple(v_out[k].shape) != (n, layout.num_layers, layout.row_width, m) or not v_out[k].is_contiguous():
            raise ValueError(f"v_out[{k}] must be contiguous [n, L, F, m]")
    _bf16_like("omega", omega, 2)
    if tuple(omega.shape) != (m + oversample, layout.row_width) or not omega.is_contiguous():
        raise ValueError(f"omega must be contiguous [{m + oversample}, {layout.row_width}]")
    need = form_patch_workspace_bytes(layout, n, T, m, oversample)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=u_out[0].device)
    _check_dev("workspace", workspace, ("uint8",), 1)
    sk = KameraSketch(int(oversample), int(power_iters), _ptr(omega))
    fa = KameraFactors(m, (ctypes.c_void_p * 2)(_ptr(u_out[0]), _ptr(u_out[1]) if S > 1 else 0),
                       (ctypes.c_void_p * 2)(_ptr(v_out[0]), _ptr(v_out[1]) if S > 1 else 0))
    lay = layout.c()
    tail = (ctypes.c_void_p(_ptr(delta)), ctypes.byref(sk), ctypes.byref(fa), ctypes.c_void_p(_ptr(workspace)),
            ctypes.c_int64(workspace.numel()))
    keep = (lay, cs, ts, sk, fa, canon, target, delta, u_out, v_out, omega, workspace)
    if not orbit:
        return Call("kamera_form_patch", lib.kamera_form_patch,
                    (ctypes.byref(lay), ctypes.byref(cs), ctypes.byref(ts), n) + tail, keep, stream)
    return Call("kamera_form_orbit_patch", lib.kamera_form_orbit_patch,
                (ctypes.byref(lay), ctypes.byref(cs), ctypes.byref(ts), n, int(views)) + tail, keep, stream)


def prepare_form_patch(layout: Layout, canon, target, delta, u_out, v_out, omega, *, oversample: int,
                       power_iters: int, workspace=None, stream=None) -> Call:
    """Prepared kamera_form_patch: the rank-m factors of
    Delta = target - R(delta_i) canon[i] for every chunk, layer and stream,
    written into u_out[s] [n, L, T, m] and v_out[s] [n, L, F, m] (bfloat16).

    omega: [m + oversample, F] bfloat16 test matrix drawn by the caller.  The
    device workspace is allocated here (torch) unless given.
    """
    return _prepare_form(layout, canon, target, delta, 1, u_out, v_out, omega, oversample, power_iters,
                         workspace, stream, False)


def prepare_form_orbit_patch(layout: Layout, canon, targets, deltas, u_out, v_out, omega, *, oversample: int,
                             power_iters: int, workspace=None, stream=None) -> Call:
    """Prepared kamera_form_orbit_patch: the rank-m factors of the mean over
    the views v of targets[i * views + v] - R(deltas[i, v]) canon[i].

    deltas: contiguous int64 [n, views]; targets holds n * views chunks, view v
    of chunk i at chunk index i * views + v.  Outputs as for prepare_form_patch.
    """
    if getattr(deltas, "dim", lambda: 0)() != 2 or not deltas.is_contiguous():
        raise ValueError("deltas must be a contiguous [n, views] tensor")
    return _prepare_form(layout, canon, targets, deltas.view(-1), int(deltas.shape[1]), u_out, v_out, omega,
                         oversample, power_iters, workspace, stream, True)


def form_patch(layout: Layout, canon, target, delta, u_out, v_out, omega, *, oversample: int,
               power_iters: int, stream=None, **kw):
    """kamera_form_patch: the rank-m factors of target - R(delta) canon."""
    prepare_form_patch(layout, canon, target, delta, u_out, v_out, omega, oversample=oversample,
                       power_iters=power_iters, **kw)(stream)


def form_orbit_patch(layout: Layout, canon, targets, deltas, u_out, v_out, omega, *, oversample: int,
                     power_iters: int, stream=None, **kw):
    """kamera_form_orbit_patch: the rank-m factors of the mean per-view deficit."""
    prepare_form_orbit_patch(layout, canon, targets, deltas, u_out, v_out, omega, oversample=oversample,
                             power_iters=power_iters, **kw)(stream)


def decode_attention_workspace_bytes(layout: Layout, num_q_heads: int, num_entries: int, n_tokens: int) -> int:
    """Bytes of device workspace kamera_decode_attention needs (raises if unsupported)."""
    b = int(load_library().kamera_decode_attention_workspace(ctypes.byref(layout.c()), int(num_q_heads),
                                                             int(num_entries), int(n_tokens)))
    if b < 0:
        raise KameraError(6, "kamera_decode_attention_workspace")
    return b


def decode_attention_paged_workspace_bytes(layout: Layout, num_q_heads: int, num_entries: int, n_tokens: int,
                                           num_seqs: int, pool_max_tokens: int) -> int:
    """Bytes of device workspace kamera_decode_attention_paged needs (raises if unsupported)."""
    b = int(load_library().kamera_decode_attention_paged_workspace(ctypes.byref(layout.c()), int(num_q_heads),
                                                                   int(num_entries), int(n_tokens), int(num_seqs),
                                                                   int(pool_max_tokens)))
    if b < 0:
        raise KameraError(6, "kamera_decode_attention_paged_workspace")
    return b


def prepare_decode_attention(layout: Layout, layer: int, canon, q, seq_entries, chunk_ids, delta, out, *,
                             scale: float, lse=None, u=None, v=None, error_word=None, workspace=None,
                             pool=None, block_table=None, pool_tokens=None, pool_page_size=0,
                             stream=None) -> Call:
    """Prepared kamera_decode_attention: every sequence's queries attend its
    reused context at one layer, keys and values relocated and patched on read.

    canon: per-stream [n_store, L, T, F] canonical rows; q: [B, Hq, D] bfloat16;
    seq_entries: int32 [B + 1]; chunk_ids: int32 [E]; delta: int64 [E];
    out: float32 [B, Hq, Dv] (Dv = D, or the c_KV width for MLA); lse: float32
    [B, Hq] or None; u, v: the patch
    factors indexed by store chunk (or None).  The device workspace is
    allocated here (torch) unless given.

    pool (per-stream [L, slots, F] rows), block_table (int32 [B, max_pages]),
    pool_tokens (int32 [B]) and pool_page_size: the sequences' tokens in a
    paged pool, attended as well (kamera_decode_attention_paged).
    """
    import torch
    lib = load_library()
    cs, ns, T = _src_struct(layout, canon, None)
    pt, m = _patch_struct(layout, u, v, ns, T)
    _check_dev("q", q, ("bfloat16", "int16", "uint16"), 3)
    B, Hq, D = q.shape
    if D != layout.head_dim or not q.is_contiguous():
        raise ValueError(f"q must be contiguous [B, Hq, {layout.head_dim}]")
    _idx("seq_entries", seq_entries, "int32", B + 1)
    E = chunk_ids.numel() if chunk_ids is not None else 0
    _idx("chunk_ids", chunk_ids, "int32", E)
    _idx("delta", delta, "int64", E)
    Dv = D if layout.num_streams == 2 else layout.rope_offset  # MLA: the c_KV part of the row
    _check_dev("out", out, ("float32",), 3)
    if tuple(out.shape) != (B, Hq, Dv) or not out.is_contiguous():
        raise ValueError(f"out must be contiguous float32 [{B}, {Hq}, {Dv}]")
    if lse is not None:
        _check_dev("lse", lse, ("float32",), 2)
        if tuple(lse.shape) != (B, Hq) or not lse.is_contiguous():
            raise ValueError(f"lse must be contiguous float32 [{B}, {Hq}]")
    _check_dev("error_word", error_word, ("int32", "uint32"), 1)
    pstruct = None
    if pool is not None:
        S = layout.num_streams
        if len(pool) != S:
            raise ValueError(f"need {S} pool tensors")
        for k, t in enumerate(pool):
            _bf16_like(f"pool[{k}]", t, 3)
            if t.shape != pool[0].shape or t.stride() != pool[0].stride():
                raise ValueError("pool streams must share shape and strides")
        Lp, slots, Fp = pool[0].shape
        if Lp != layout.num_layers or Fp != layout.row_width or pool[0].stride(2) != 1 or \
                (slots > 1 and pool[0].stride(1) != Fp):
            raise ValueError("pool rows must be contiguous [L, slots, F] of the layout")
        _check_dev("block_table", block_table, ("int32",), 2)
        _idx("pool_tokens", pool_tokens, "int32", B)
        if block_table is None or block_table.shape[0] != B or not block_table.is_contiguous():
            raise ValueError(f"block_table must be contiguous int32 [{B}, max_pages]")
        max_pages = block_table.shape[1]
        pstruct = KameraAttnPool((ctypes.c_void_p * 2)(_ptr(pool[0]), _ptr(pool[1]) if S > 1 else 0),
                                 pool[0].stride(0), slots, int(pool_page_size), int(max_pages), _ptr(block_table),
                                 _ptr(pool_tokens))
        need = decode_attention_paged_workspace_bytes(layout, Hq, E, T, B, max_pages * pool_page_size)
    else:
        need = decode_attention_workspace_bytes(layout, Hq, E, T)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check_dev("workspace", workspace, ("uint8",), 1)
    lay = layout.c()
    head = (ctypes.byref(lay), int(layer), ctypes.byref(cs), ctypes.byref(pt))
    tail = (int(B), ctypes.c_void_p(_ptr(seq_entries)), int(E), ctypes.c_void_p(_ptr(chunk_ids)),
            ctypes.c_void_p(_ptr(delta)), int(Hq), ctypes.c_void_p(_ptr(q)), ctypes.c_float(scale),
            ctypes.c_void_p(_ptr(out)), ctypes.c_void_p(_ptr(lse)), ctypes.c_void_p(_ptr(error_word)),
            ctypes.c_void_p(_ptr(workspace)), ctypes.c_int64(workspace.numel()))
    keep = (lay, cs, pt, canon, q, seq_entries, chunk_ids, delta, out, lse, u, v, error_word, workspace)
    if pstruct is not None:
        return Call("kamera_decode_attention_paged", lib.kamera_decode_attention_paged,
                    head + (ctypes.byref(pstruct),) + tail, keep + (pstruct, pool, block_table, pool_tokens), stream)
    return Call("kamera_decode_attention", lib.kamera_decode_attention, head + tail, keep, stream)


def decode_attention(layout: Layout, layer: int, canon, q, seq_entries, chunk_ids, delta, out, *,
                     scale: float, stream=None, **kw):
    """kamera_decode_attention: attention over the reused context, relocated on read."""
    prepare_decode_attention(layout, layer, canon, q, seq_entries, chunk_ids, delta, out, scale=scale,
                             **kw)(stream)


def host_staging_bytes(layout: Layout, n_tokens: int, slots: int = 2) -> int:
    """Bytes of device staging kamera_relocate_patch_host needs for `slots` chunk slots."""
    b = int(load_library().kamera_host_staging_bytes(ctypes.byref(layout.c()), int(n_tokens), int(slots)))
    if b < 0:
        raise KameraError(4, "kamera_host_staging_bytes")
    return b


def prepare_relocate_patch_host(layout: Layout, host_src, chunk_ids, delta, pool, *, u=None, v=None,
                                page_size=0, page_table=None, dst_offset=None, error_word=None,
                                page_order="auto", staging=None, slots: int = 2, copy_stream=None,
                                stream=None) -> Call:
    """Prepared kamera_relocate_patch_host: output i <- store chunk chunk_ids[i]
    (host_src: per-stream PINNED host tensors [n_store, L, T, F]) relocated by
    delta[i] (device int64) plus patch i (u, v: device [n, L, T, m] / [n, L, F, m]
    indexed by output), copied over the host link through `slots` device
    staging slots on copy_stream (a new default-priority stream if None) and
    relocated on the call's stream."""
    import torch
    lib = load_library()
    S = layout.num_streams
    if len(host_src) != S:
        raise ValueError(f"need {S} host source tensors")
    ref = host_src[0]
    for k, t in enumerate(host_src):
        if not isinstance(t, torch.Tensor) or t.is_cuda or t.dim() != 4:
            raise ValueError(f"host_src[{k}] must be a 4-D host tensor")
        if str(t.dtype).replace("torch.", "") not in ("bfloat16", "int16", "uint16"):
            raise TypeError(f"host_src[{k}]: dtype {t.dtype} is not 16-bit")
        if not t.is_pinned():
            raise ValueError(f"host_src[{k}] must be in pinned host memory (pin_memory=True)")
        if t.shape != ref.shape or t.stride() != ref.stride():
            raise ValueError("host source streams must share shape and strides")
    ns, L, T, F = ref.shape
    if L != layout.num_layers or F != layout.row_width:
        raise ValueError(f"host source shape {tuple(ref.shape)} does not match the layout")
    if ref.stride(3) != 1 or (T > 1 and ref.stride(2) != F):
        raise ValueError("host source rows must be contiguous [T][F]")
    ids = [int(x) for x in (chunk_ids.tolist() if hasattr(chunk_ids, "tolist") else chunk_ids)]
    n = len(ids)
    _idx("delta", delta, "int64", n)
    ids_c = (ctypes.c_int32 * max(n, 1))(*ids)
    src = KameraSrc((ctypes.c_void_p * 2)(_ptr(host_src[0]), _ptr(host_src[1]) if S > 1 else 0),
                    ref.stride(0), ref.stride(1), T, ns, 0)
    pt, _ = _patch_struct(layout, u, v, n, T)
    order = _page_order(page_order, page_size, n, T, pool[0].device)
    d = _dst_struct(layout, pool, page_size, page_table, dst_offset, error_word, n, T, order, check_scratch=None)
    if staging is None:
        staging = torch.empty(max(host_staging_bytes(layout, T, slots), 256), dtype=torch.uint8,
                              device=pool[0].device)
    _check_dev("staging", staging, ("uint8",), 1)
    if copy_stream is None:
        copy_stream = torch.cuda.Stream(device=pool[0].device)
    lay = layout.c()
    args = (ctypes.byref(lay), ctypes.byref(src), n, ids_c, ctypes.c_void_p(_ptr(delta)), ctypes.byref(pt),
            ctypes.byref(d), ctypes.c_void_p(_ptr(staging)), ctypes.c_int64(staging.numel()),
            ctypes.c_void_p(int(copy_stream.cuda_stream)))
    return Call("kamera_relocate_patch_host", lib.kamera_relocate_patch_host, args,
                (lay, src, ids_c, pt, d, host_src, delta, u, v, pool, page_table, dst_offset, error_word,
                 order, staging, copy_stream), stream)


def prepare_relocate_patch_host_varlen(layout: Layout, host_src, row_offset, n_tokens, max_tokens, chunk_ids,
                                       delta, pool, *, u=None, v=None, page_size=0, page_table=None,
                                       dst_offset=None, error_word=None, staging=None, slots: int = 2,
                                       copy_stream=None, stream=None) -> Call:
    """Prepared kamera_relocate_patch_host_varlen: output i <- store chunk chunk_ids[i] of a packed
    variable-length store in PINNED host memory (host_src: per stream [total_rows, F]; row_offset,
    n_tokens: host sequences [n_store]) relocated by delta[i] (device int64) plus patch i (u: device
    [sum of output rows, m] packed in output order, v: [n, L, F, m])."""
    import torch
    lib = load_library()
    S = layout.num_streams
    if len(host_src) != S:
        raise ValueError(f"need {S} host source tensors")
    ref = host_src[0]
    for k, t in enumerate(host_src):
        if not isinstance(t, torch.Tensor) or t.is_cuda or t.dim() != 2:
            raise ValueError(f"host_src[{k}] must be a 2-D host tensor [total_rows, F]")
        if str(t.dtype).replace("torch.", "") not in ("bfloat16", "int16", "uint16"):
            raise TypeError(f"host_src[{k}]: dtype {t.dtype} is not 16-bit")
        if not t.is_pinned():
            raise ValueError(f"host_src[{k}] must be in pinned host memory (pin_memory=True)")
        if t.shape != ref.shape or not t.is_contiguous():
            raise ValueError("host source streams must be contiguous and of one shape")
    total_rows, F = ref.shape
    if F != layout.row_width:
        raise ValueError(f"host rows of width {F} do not match the layout")
    ro = [int(x) for x in (row_offset.tolist() if hasattr(row_offset, "tolist") else row_offset)]
    nt = [int(x) for x in (n_tokens.tolist() if hasattr(n_tokens, "tolist") else n_tokens)]
    if len(ro) != len(nt):
        raise ValueError("row_offset and n_tokens must have n_store entries each")
    ns = len(nt)
    ids = [int(x) for x in (chunk_ids.tolist() if hasattr(chunk_ids, "tolist") else chunk_ids)]
    n = len(ids)
    _idx("delta", delta, "int64", n)
    T = int(max_tokens)
    ro_c = (ctypes.c_int64 * max(ns, 1))(*ro)
    nt_c = (ctypes.c_int32 * max(ns, 1))(*nt)
    ids_c = (ctypes.c_int32 * max(n, 1))(*ids)
    vl = KameraVarlen(ctypes.addressof(ro_c), ctypes.addressof(nt_c), int(total_rows))
    src = KameraSrc((ctypes.c_void_p * 2)(_ptr(host_src[0]), _ptr(host_src[1]) if S > 1 else 0), 0, 0, T, ns, 0)
    m = 0
    if u is None and v is None:
        pt = KameraPatch(0, (ctypes.c_void_p * 2)(0, 0), (ctypes.c_void_p * 2)(0, 0))
    else:
        m = u[0].shape[-1]
        out_rows = sum(layout.num_layers * nt[c] for c in ids if 0 <= c < ns)
        for k in range(S):
            _bf16_like(f"u[{k}]", u[k], 2)
            _bf16_like(f"v[{k}]", v[k], 4)
            if tuple(u[k].shape) != (out_rows, m) or not u[k].is_contiguous():
                raise ValueError(f"u[{k}] must be contiguous [{out_rows}, m] (output chunks' rows, in output order)")
            if tuple(v[k].shape) != (n, layout.num_layers, F, m) or not v[k].is_contiguous():
                raise ValueError(f"v[{k}] must be contiguous [n, L, F, m]")
        pt = KameraPatch(m, (ctypes.c_void_p * 2)(_ptr(u[0]), _ptr(u[1]) if S > 1 else 0),
                         (ctypes.c_void_p * 2)(_ptr(v[0]), _ptr(v[1]) if S > 1 else 0))
    d = _dst_struct(layout, pool, page_size, page_table, dst_offset, error_word, n, T, check_scratch=None)
    if staging is None:
        staging = torch.empty(max(host_staging_bytes(layout, T, slots), 256), dtype=torch.uint8,
                              device=pool[0].device)
    _check_dev("staging", staging, ("uint8",), 1)
    if copy_stream is None:
        copy_stream = torch.cuda.Stream(device=pool[0].device)
    lay = layout.c()
    args = (ctypes.byref(lay), ctypes.byref(src), ctypes.byref(vl), n, ids_c, ctypes.c_void_p(_ptr(delta)),
            ctypes.byref(pt) if m else None, ctypes.byref(d), ctypes.c_void_p(_ptr(staging)),
            ctypes.c_int64(staging.numel()), ctypes.c_void_p(int(copy_stream.cuda_stream)))
    return Call("kamera_relocate_patch_host_varlen", lib.kamera_relocate_patch_host_varlen, args,
                (lay, src, vl, ro_c, nt_c, ids_c, pt, d, host_src, delta, u, v, pool, page_table, dst_offset,
                 error_word, staging, copy_stream), stream)


def relocate_patch_host_varlen(layout: Layout, host_src, row_offset, n_tokens, max_tokens, chunk_ids, delta, pool,
                               *, stream=None, **kw):
    prepare_relocate_patch_host_varlen(layout, host_src, row_offset, n_tokens, max_tokens, chunk_ids, delta, pool,
                                       stream=stream, **kw)()


def relocate_patch_host(layout: Layout, host_src, chunk_ids, delta, pool, *, stream=None, **kw):
    """kamera_relocate_patch_host: relocation (+ patch) from a pinned host store."""
    prepare_relocate_patch_host(layout, host_src, chunk_ids, delta, pool, **kw)(stream)


def relocate(layout: Layout, src, delta, pool, *, stream=None, **kw):
    """kamera_relocate: pool <- R(delta_i) src[i] for every output chunk i."""
    prepare_relocate(layout, src, delta, pool, **kw)(stream)


def relocate_patch(layout: Layout, src, delta, u, v, pool, *, stream=None, **kw):
    """kamera_relocate_patch: pool <- R(delta_i) src[i] + U_i V_i^T."""
    prepare_relocate_patch(layout, src, delta, u, v, pool, **kw)(stream)


def reorder(layout: Layout, src, perm, base_pos, pool, *, stream=None, **kw):
    """kamera_reorder: output k <- chunk perm[k] at base_pos + k*T, with its orbit patch."""
    prepare_reorder(layout, src, perm, base_pos, pool, **kw)(stream)


def recall(layout: Layout, src, chunk_ids, target_pos, pool, *, stream=None, **kw):
    """kamera_recall: output i <- store chunk ids[i] rehydrated at target_pos[i]."""
    prepare_recall(layout, src, chunk_ids, target_pos, pool, **kw)(stream)


def relocate_patch_varlen(layout: Layout, src, row_offset, n_tokens, max_tokens, delta, pool, *, stream=None,
                          **kw):
    prepare_relocate_patch_varlen(layout, src, row_offset, n_tokens, max_tokens, delta, pool, stream=stream,
                                  **kw)()


def recall_varlen(layout: Layout, src, row_offset, n_tokens, max_tokens, chunk_ids, target_pos, pool, *,
                  stream=None, **kw):
    prepare_recall_varlen(layout, src, row_offset, n_tokens, max_tokens, chunk_ids, target_pos, pool,
                          stream=stream, **kw)()


def status_string(status: int) -> str:
    return load_library().kamera_status_string(int(status)).decode()


def version() -> int:
    return int(load_library().kamera_version())


__all__ = ["Layout", "KameraError", "Call", "relocate", "relocate_patch", "reorder", "recall",
           "prepare_relocate", "prepare_relocate_patch", "prepare_reorder", "prepare_recall",
           "status_string", "version", "lib_path", "load_library", "ROPE_HALF", "ROPE_INTERLEAVED",
           "EW_PAGE", "EW_OFFSET", "EW_CHUNK", "KameraLayout", "KameraSrc", "KameraPatch", "KameraDst",
           "KameraSketch", "KameraFactors", "form_patch", "prepare_form_patch", "form_patch_workspace_bytes",
           "form_orbit_patch", "prepare_form_orbit_patch", "decode_attention", "prepare_decode_attention",
           "decode_attention_workspace_bytes", "relocate_patch_host", "prepare_relocate_patch_host",
           "host_staging_bytes", "KameraVarlen", "relocate_patch_varlen", "recall_varlen",
           "prepare_relocate_patch_varlen", "prepare_recall_varlen", "relocate_patch_host_varlen",
           "prepare_relocate_patch_host_varlen", "KameraAttnPool", "decode_attention_paged_workspace_bytes"]
