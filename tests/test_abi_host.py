"""The C-ABI library on a host without a GPU: it loads, exports every symbol
include/kamera.h declares, and rejects bad arguments with the documented
status before any HIP call.  No call here reaches a kernel launch: each one
either fails validation or is an empty call (n = 0), so no pointer passed here
is ever dereferenced.
"""

import ctypes
import os
import re
import subprocess

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "kamera.h")


@pytest.fixture(scope="module")
def lib():
    from position_invariant_kv_amd import _abi
    if not os.path.exists(_abi.lib_path()):
        from position_invariant_kv_amd import build
        build.build()
    return _abi.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kamera_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    from position_invariant_kv_amd import _abi
    assert declared_functions() == sorted(_abi.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    from position_invariant_kv_amd import _abi
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kamera_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_struct_layouts_match_header():
    # compile a tiny C program against the header and compare sizeof/offsetof
    from position_invariant_kv_amd import _abi
    src = r'''
#include <stddef.h>
#include <stdio.h>
#include "kamera.h"
int main(void) {
  printf("%zu %zu %zu %zu\n", sizeof(kamera_layout), sizeof(kamera_src), sizeof(kamera_patch), sizeof(kamera_dst));
  printf("%zu %zu %zu\n", offsetof(kamera_layout, rope_base), offsetof(kamera_src, canon_pos), offsetof(kamera_dst, error_word));
  printf("%zu %zu\n", offsetof(kamera_patch, v), offsetof(kamera_dst, page_size));
  printf("%zu %zu %zu %zu %zu %zu\n", sizeof(kamera_sketch), sizeof(kamera_factors), offsetof(kamera_sketch, omega),
         offsetof(kamera_factors, v), offsetof(kamera_dst, page_order), offsetof(kamera_dst, check_scratch));
  return 0;
}
'''
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        exe = os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        lines = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    sizes = [int(x) for x in lines[0].split()]
    assert sizes == [ctypes.sizeof(_abi.KameraLayout), ctypes.sizeof(_abi.KameraSrc),
                     ctypes.sizeof(_abi.KameraPatch), ctypes.sizeof(_abi.KameraDst)]
    offs = [int(x) for x in lines[1].split()] + [int(x) for x in lines[2].split()]
    assert offs == [_abi.KameraLayout.rope_base.offset, _abi.KameraSrc.canon_pos.offset,
                    _abi.KameraDst.error_word.offset, _abi.KameraPatch.v.offset,
                    _abi.KameraDst.page_size.offset]
    assert [int(x) for x in lines[3].split()] == [
        ctypes.sizeof(_abi.KameraSketch), ctypes.sizeof(_abi.KameraFactors), _abi.KameraSketch.omega.offset,
        _abi.KameraFactors.v.offset, _abi.KameraDst.page_order.offset, _abi.KameraDst.check_scratch.offset]


def test_status_strings(lib):
    for code in range(8):
        s = lib.kamera_status_string(code)
        assert s and isinstance(s, bytes)
    assert lib.kamera_status_string(99) == b"unknown status"
    assert lib.kamera_version() >= 100


# --------------------------------------------------------------------------
# Validation paths.  Fake device addresses are plain integers: validation
# only looks at their values (NULL, alignment, overlap) and never reads them.
# --------------------------------------------------------------------------

A = 0x10000000   # fake, 16-byte aligned "device" addresses, far apart
B = 0x20000000
C = 0x30000000
D = 0x40000000
E = 0x50000000


def make(L=2, H=2, Dh=64, o=0, R=64, style=0, base=1e4, S=2, T=40, n_store=3, m=8, P=16,
         slots=4096):
    from position_invariant_kv_amd import _abi
    F = H * Dh
    lay = _abi.KameraLayout(L, H, Dh, o, R, style, base, S)
    P2 = ctypes.c_void_p * 2
    src = _abi.KameraSrc(P2(A, A + 0x1000000), L * T * F, T * F, T, n_store, 0)
    patch = _abi.KameraPatch(m, P2(B, B + 0x1000000), P2(C, C + 0x1000000))
    dst = _abi.KameraDst(P2(D, D + 0x4000000), slots * F, slots, P, E, E + 0x100, 0)
    return lay, src, patch, dst


def call(lib, fn, lay, src, patch, dst, n=2):
    b = ctypes.byref
    if fn == "relocate":
        return lib.kamera_relocate(b(lay), b(src), n, ctypes.c_void_p(E + 0x200), b(dst), None)
    if fn == "relocate_patch":
        return lib.kamera_relocate_patch(b(lay), b(src), n, ctypes.c_void_p(E + 0x200), b(patch), b(dst), None)
    if fn == "reorder":
        return lib.kamera_reorder(b(lay), b(src), n, ctypes.c_void_p(E + 0x300), 0, b(patch), b(dst), None)
    return lib.kamera_recall(b(lay), b(src), n, ctypes.c_void_p(E + 0x300), ctypes.c_void_p(E + 0x400),
                             b(patch), b(dst), None)


OK, NULL, ALIGN, SHAPE, RANGE, ALIAS, UNSUP, HIPERR = range(8)
FNS = ["relocate", "relocate_patch", "reorder", "recall"]


@pytest.mark.parametrize("fn", FNS)
def test_empty_call_is_ok(lib, fn):
    lay, src, patch, dst = make()
    assert call(lib, fn, lay, src, patch, dst, n=0) == OK
    src.n_tokens = 0
    assert call(lib, fn, lay, src, patch, dst, n=2) == OK


@pytest.mark.parametrize("fn", FNS)
def test_null_pointers(lib, fn):
    lay, src, patch, dst = make()
    b = ctypes.byref
    assert lib.kamera_relocate(None, b(src), 1, ctypes.c_void_p(E), b(dst), None) == NULL
    assert lib.kamera_relocate(b(lay), None, 1, ctypes.c_void_p(E), b(dst), None) == NULL
    src.rows[0] = 0
    assert call(lib, fn, lay, src, patch, dst) == NULL
    lay, src, patch, dst = make()
    dst.rows[1] = 0
    assert call(lib, fn, lay, src, patch, dst) == NULL
    lay, src, patch, dst = make()
    dst.page_table = 0
    assert call(lib, fn, lay, src, patch, dst) == NULL


def test_null_shift_arrays(lib):
    lay, src, patch, dst = make()
    b = ctypes.byref
    assert lib.kamera_relocate(b(lay), b(src), 2, None, b(dst), None) == NULL
    assert lib.kamera_relocate_patch(b(lay), b(src), 2, ctypes.c_void_p(E), None, b(dst), None) == NULL
    assert lib.kamera_reorder(b(lay), b(src), 2, None, 0, b(patch), b(dst), None) == NULL
    assert lib.kamera_recall(b(lay), b(src), 2, ctypes.c_void_p(E), None, b(patch), b(dst), None) == NULL


def test_null_factors(lib):
    lay, src, patch, dst = make()
    patch.v[1] = 0
    assert call(lib, "relocate_patch", lay, src, patch, dst) == NULL
    patch.rank = 0          # m = 0 needs no factors
    assert call(lib, "relocate_patch", lay, src, patch, dst, n=0) == OK


def test_contiguous_needs_offsets(lib):
    lay, src, patch, dst = make(P=0)
    dst.dst_offset = 0
    assert call(lib, "relocate", lay, src, patch, dst) == NULL


@pytest.mark.parametrize("field,value", [("src_row", 8), ("dst_row", 2), ("u", 4), ("v", 8),
                                         ("chunk_stride", 4), ("layer_stride", 2), ("dst_stride", 4)])
def test_alignment(lib, field, value):
    lay, src, patch, dst = make()
    if field == "src_row":
        src.rows[1] = A + 0x1000000 + value
    elif field == "dst_row":
        dst.rows[0] = D + value
    elif field == "u":
        patch.u[0] = B + value
    elif field == "v":
        patch.v[1] = C + 0x1000000 + value
    elif field == "chunk_stride":
        src.chunk_stride += value
    elif field == "layer_stride":
        src.layer_stride += value
    else:
        dst.layer_stride += value
    assert call(lib, "relocate_patch", lay, src, patch, dst) == ALIGN


@pytest.mark.parametrize("kw", [dict(Dh=96), dict(o=32, R=64, Dh=128), dict(R=32), dict(Dh=1088, R=64),
                                dict(H=8, Dh=1024, R=64), dict(m=12)])
def test_unsupported_shapes(lib, kw):
    lay, src, patch, dst = make(**kw)
    assert call(lib, "relocate_patch", lay, src, patch, dst) == UNSUP


@pytest.mark.parametrize("kw", [dict(L=0), dict(H=0), dict(S=3), dict(S=0), dict(style=2),
                                dict(o=64, R=64, Dh=64), dict(base=0.0), dict(base=-1.0),
                                dict(base=float("inf")), dict(m=72), dict(m=-8), dict(P=-1),
                                dict(slots=16), dict(L=65536)])
def test_out_of_range(lib, kw):
    lay, src, patch, dst = make(**kw)
    assert call(lib, "relocate_patch", lay, src, patch, dst) == RANGE


def test_slice_offsets_fit_32_bits(lib):
    # one (chunk, layer) slice of T x F elements must stay under 2^31 elements
    lay, src, patch, dst = make(T=1 << 24)        # F = 128: T * F = 2^31
    for fn in FNS:
        assert call(lib, fn, lay, src, patch, dst) == RANGE


def test_more_outputs_than_store(lib):
    lay, src, patch, dst = make(n_store=2)
    assert call(lib, "relocate", lay, src, patch, dst, n=3) == RANGE
    # reorder and recall may name any store chunk: their n is not bounded by n_store
    assert call(lib, "reorder", lay, src, patch, dst, n=0) == OK


def test_shape_inconsistency(lib):
    lay, src, patch, dst = make()
    src.layer_stride = 8            # layers overlap
    assert call(lib, "relocate", lay, src, patch, dst) == SHAPE
    lay, src, patch, dst = make()
    src.chunk_stride = 8
    assert call(lib, "relocate", lay, src, patch, dst) == SHAPE
    lay, src, patch, dst = make()
    dst.layer_stride = 8
    assert call(lib, "relocate", lay, src, patch, dst) == SHAPE


def test_alias(lib):
    lay, src, patch, dst = make()
    dst.rows[0] = A + 0x100           # inside stream 0's source rows
    assert call(lib, "relocate", lay, src, patch, dst) == ALIAS
    lay, src, patch, dst = make()
    dst.rows[1] = B                   # on top of the U factors
    assert call(lib, "relocate_patch", lay, src, patch, dst) == ALIAS
    lay, src, patch, dst = make()
    dst.rows[1] = dst.rows[0] + 0x10  # the two pools overlap
    assert call(lib, "relocate", lay, src, patch, dst) == ALIAS


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    import importlib
    from position_invariant_kv_amd import _abi
    monkeypatch.setattr(_abi, "_LIB", None)
    monkeypatch.setenv("KAMERA_LIB", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        _abi.load_library()


def test_page_order_scratch_checks(lib):
    # the destination-order scratch: 4-byte aligned, disjoint from every other argument
    lay, src, patch, dst = make()
    dst.page_order = E + 0x802
    assert call(lib, "relocate_patch", lay, src, patch, dst) == ALIGN
    lay, src, patch, dst = make()
    dst.page_order = E + 4            # overlaps the page table [2 x 3] at E
    assert call(lib, "relocate", lay, src, patch, dst) == ALIAS
    lay, src, patch, dst = make()
    dst.page_order = D + 0x40         # inside the stream-0 pool
    assert call(lib, "reorder", lay, src, patch, dst) == ALIAS
    lay, src, patch, dst = make()
    dst.page_order = A + 0x40         # inside the source rows
    assert call(lib, "recall", lay, src, patch, dst) == ALIAS
    lay, src, patch, dst = make()
    dst.page_order = C + 0x1000040    # inside stream 1's V factors
    assert call(lib, "relocate_patch", lay, src, patch, dst) == ALIAS
    # a contiguous pool ignores the scratch
    lay, src, patch, dst = make(P=0)
    dst.page_order = E + 0x802
    assert call(lib, "relocate", lay, src, patch, dst, n=0) == OK


def test_check_scratch_checks(lib):
    # the content-check scratch (used with an error word): 4-byte aligned,
    # disjoint from every other argument, including the perm / chunk ids
    lay, src, patch, dst = make()
    dst.error_word = E + 0x900
    dst.check_scratch = E + 0x802
    assert call(lib, "relocate_patch", lay, src, patch, dst) == ALIGN
    lay, src, patch, dst = make()
    dst.error_word = E + 0x900
    dst.check_scratch = E + 4            # overlaps the page table [2 x 3] at E
    assert call(lib, "relocate", lay, src, patch, dst) == ALIAS
    lay, src, patch, dst = make()
    dst.error_word = E + 0x900
    dst.check_scratch = D + 0x40         # inside the stream-0 pool
    assert call(lib, "reorder", lay, src, patch, dst) == ALIAS
    lay, src, patch, dst = make()
    dst.error_word = E + 0x900
    dst.check_scratch = E + 0x2F8        # [2*3 + 2] int32 reaches the perm at E + 0x300
    assert call(lib, "reorder", lay, src, patch, dst) == ALIAS
    lay, src, patch, dst = make()
    dst.error_word = E + 0x900
    dst.check_scratch = C + 0x1000040    # inside stream 1's V factors
    assert call(lib, "recall", lay, src, patch, dst) == ALIAS
    # without an error word the scratch is not used, so not checked
    lay, src, patch, dst = make()
    dst.check_scratch = E + 0x802
    dst.page_order = E + 0x806            # misaligned: the page-order check still applies
    assert call(lib, "relocate", lay, src, patch, dst) == ALIGN


# --------------------------------------------------------------------------
# kamera_form_patch validation (fake addresses, never dereferenced)
# --------------------------------------------------------------------------

W = 0x60000000   # workspace (256-byte aligned)
O = 0x70000000   # omega
UO = 0x80000000  # output factors
VO = 0x90000000


def make_form(L=2, H=2, Dh=64, T=40, n=2, m=8, p=8, q=1, S=2):
    from position_invariant_kv_amd import _abi
    F = H * Dh
    lay = _abi.KameraLayout(L, H, Dh, 0, Dh, 0, 1e4, S)
    P2 = ctypes.c_void_p * 2
    canon = _abi.KameraSrc(P2(A, A + 0x1000000), L * T * F, T * F, T, n, 0)
    target = _abi.KameraSrc(P2(B, B + 0x1000000), L * T * F, T * F, T, n, 0)
    sk = _abi.KameraSketch(p, q, O)
    out = _abi.KameraFactors(m, P2(UO, UO + 0x1000000), P2(VO, VO + 0x1000000))
    return lay, canon, target, sk, out


def form_call(lib, lay, canon, target, sk, out, n=2, ws=W, wsb=1 << 40):
    b = ctypes.byref
    return lib.kamera_form_patch(b(lay), b(canon), b(target), n, ctypes.c_void_p(C), b(sk), b(out),
                                 ctypes.c_void_p(ws), ctypes.c_int64(wsb), None)


def test_form_workspace_query(lib):
    from position_invariant_kv_amd import _abi
    lay = make_form()[0]
    b = ctypes.byref
    need = lib.kamera_form_patch_workspace(b(lay), 2, 40, 8, 8)
    # 2 chunks x 2 layers x 2 streams; T padded to 64, F = 128, k = 16 -> 32 columns
    blocks, Tp, F, kp = 8, 64, 128, 32
    per = [blocks * Tp * F * 2] * 2 + [blocks * Tp * kp * 4] + [blocks * kp * Tp * 2] * 2 + \
          [blocks * F * kp * 4, blocks * kp * F * 2] + \
          [2 * blocks * kp * kp * 8, blocks * kp * kp * 4] + [blocks * kp * 64 * 4] * 2
    assert need == sum((x + 255) // 256 * 256 for x in per)
    assert lib.kamera_form_patch_workspace(b(lay), 2, 40, 60, 8) == -1     # k > 64
    assert lib.kamera_form_patch_workspace(None, 2, 40, 8, 8) == -1


def test_form_validation(lib):
    lay, canon, target, sk, out = make_form()
    assert form_call(lib, lay, canon, target, sk, out, n=0) == OK
    assert form_call(lib, lay, canon, target, sk, out, ws=W + 64) == ALIGN
    assert form_call(lib, lay, canon, target, sk, out, wsb=1000) == RANGE
    assert form_call(lib, lay, canon, target, sk, out, ws=0) == NULL
    lay, canon, target, sk, out = make_form(m=7)
    assert form_call(lib, lay, canon, target, sk, out) == UNSUP            # odd rank
    lay, canon, target, sk, out = make_form(m=48, p=24)
    assert form_call(lib, lay, canon, target, sk, out) == RANGE            # k = 72 > 64
    lay, canon, target, sk, out = make_form(q=17)
    assert form_call(lib, lay, canon, target, sk, out) == RANGE
    lay, canon, target, sk, out = make_form()
    sk.omega = O + 4
    assert form_call(lib, lay, canon, target, sk, out) == ALIGN
    lay, canon, target, sk, out = make_form()
    target.n_tokens = 41
    assert form_call(lib, lay, canon, target, sk, out) == SHAPE
    lay, canon, target, sk, out = make_form()
    out.u[1] = 0
    assert form_call(lib, lay, canon, target, sk, out) == NULL
    lay, canon, target, sk, out = make_form()
    out.v[0] = A + 0x40                                                       # inside the canonical rows
    assert form_call(lib, lay, canon, target, sk, out) == ALIAS
    lay, canon, target, sk, out = make_form()
    out.u[0] = W + 0x100                                                      # inside the workspace
    assert form_call(lib, lay, canon, target, sk, out) == ALIAS


def orbit_call(lib, lay, canon, target, sk, out, n=2, views=3, ws=W, wsb=1 << 40):
    b = ctypes.byref
    return lib.kamera_form_orbit_patch(b(lay), b(canon), b(target), n, views, ctypes.c_void_p(C), b(sk), b(out),
                                       ctypes.c_void_p(ws), ctypes.c_int64(wsb), None)


def test_form_orbit_validation(lib):
    lay, canon, target, sk, out = make_form()
    target.n_store = 6
    assert orbit_call(lib, lay, canon, target, sk, out, n=0) == OK
    assert orbit_call(lib, lay, canon, target, sk, out, views=0) == RANGE
    assert orbit_call(lib, lay, canon, target, sk, out, views=-2) == RANGE
    assert orbit_call(lib, lay, canon, target, sk, out, n=1 << 20, views=1 << 12) == RANGE  # n * views overflows
    target.n_store = 5                                                         # needs n * views = 6 chunks
    assert orbit_call(lib, lay, canon, target, sk, out) == RANGE
    lay, canon, target, sk, out = make_form()
    target.n_store = 6
    target.chunk_stride = 40 * 128 - 8                                         # shorter than one chunk
    assert orbit_call(lib, lay, canon, target, sk, out) == SHAPE
    lay, canon, target, sk, out = make_form()
    target.n_store = 6
    chunk_bytes = 2 * 40 * 128 * 2
    out.u[0] = B + 5 * chunk_bytes + 0x40                                     # inside the last view's rows
    assert orbit_call(lib, lay, canon, target, sk, out) == ALIAS
    lay, canon, target, sk, out = make_form()
    target.n_store = 6
    assert orbit_call(lib, lay, canon, target, sk, out, wsb=1000) == RANGE


def make_attn(L=2, H=2, Dh=128, T=40, ns=3, m=16, S=2):
    from position_invariant_kv_amd import _abi
    F = H * Dh
    lay = _abi.KameraLayout(L, H, Dh, 0, Dh, 0, 1e4, S)
    P2 = ctypes.c_void_p * 2
    canon = _abi.KameraSrc(P2(A, A + 0x1000000), L * T * F, T * F, T, ns, 0)
    patch = _abi.KameraPatch(m, P2(B, B + 0x1000000), P2(C, C + 0x1000000))
    return lay, canon, patch


QA, OA, LA, SE, CI, DL = 0xA0000000, 0xB0000000, 0xB8000000, 0xC0000000, 0xC8000000, 0xD0000000


def attn_call(lib, lay, canon, patch, layer=1, B=2, E=3, Hq=8, q=QA, scale=0.08, out=OA, lse=LA, ws=W,
              wsb=1 << 40, ew=0):
    b = ctypes.byref
    return lib.kamera_decode_attention(b(lay), layer, b(canon), b(patch) if patch is not None else None, B,
                                       ctypes.c_void_p(SE), E, ctypes.c_void_p(CI), ctypes.c_void_p(DL), Hq,
                                       ctypes.c_void_p(q), ctypes.c_float(scale), ctypes.c_void_p(out),
                                       ctypes.c_void_p(lse), ctypes.c_void_p(ew), ctypes.c_void_p(ws),
                                       ctypes.c_int64(wsb), None)


def test_attention_workspace_query(lib):
    from position_invariant_kv_amd import _abi
    b = ctypes.byref
    lay = make_attn()[0]
    # 128-token tiles at least (4 waves x 32 tokens); 3 entries x 1 tile x 2 KV
    # heads is far below 512 workgroups
    need = lib.kamera_decode_attention_workspace(b(lay), 8, 3, 40)
    parts = 3 * 1 * 2 * 4          # units x KV heads x query heads per KV head
    al = lambda x: (x + 255) // 256 * 256
    assert need == al(parts * 128 * 4) + al(parts * 8)
    assert lib.kamera_decode_attention_workspace(b(lay), 7, 3, 40) == -1     # Hq not a multiple of Hkv
    assert lib.kamera_decode_attention_workspace(b(lay), 34, 3, 40) == -1     # G = 17 > 16
    assert lib.kamera_decode_attention_workspace(b(lay), 8, 0, 40) == 0
    lay1 = _abi.KameraLayout(2, 1, 576, 512, 64, 0, 1e4, 1)
    # MLA: one partial per (tile, query head), output width 512 (the key
    # patch's query weights are formed inside the attention kernel)
    parts1 = 3 * 1 * 16
    assert lib.kamera_decode_attention_workspace(b(lay1), 16, 3, 40) == al(parts1 * 512 * 4) + al(parts1 * 8)
    lay2 = _abi.KameraLayout(2, 1, 576, 448, 128, 0, 1e4, 1)
    assert lib.kamera_decode_attention_workspace(b(lay2), 16, 3, 40) == -1    # one stream, not 512 + 64


def test_attention_tile_plan_floors(lib):
    # the decode tile plan at the benchmark shapes (8 KV heads x 128, 32 query
    # heads), read back through the workspace size: partials = units x query
    # heads.  Entries alone: tiles double while the launch keeps 256
    # workgroups -> one 2048-token tile per (entry, KV head), 32 units.
    # Entries and pooled tokens in one launch: a floor of 1024, split by
    # tokens -> 512-token tiles, 16 x 4 entry units + 64 pooled units.
    from position_invariant_kv_amd import _abi
    b = ctypes.byref
    al = lambda x: (x + 255) // 256 * 256
    lay = _abi.KameraLayout(36, 8, 128, 0, 128, 0, 1e6, 2)
    need = lib.kamera_decode_attention_workspace(b(lay), 32, 32, 2048)
    assert need == al(32 * 32 * 128 * 4) + al(32 * 32 * 8)
    need = lib.kamera_decode_attention_paged_workspace(b(lay), 32, 16, 2048, 1, 32768)
    assert need == al(128 * 32 * 128 * 4) + al(128 * 32 * 8)


def test_attention_validation(lib):
    from position_invariant_kv_amd import _abi
    lay, canon, patch = make_attn()
    assert attn_call(lib, lay, canon, patch, B=0) == OK
    assert attn_call(lib, lay, canon, patch, layer=2) == RANGE
    assert attn_call(lib, lay, canon, patch, layer=-1) == RANGE
    assert attn_call(lib, lay, canon, patch, Hq=7) == SHAPE
    assert attn_call(lib, lay, canon, patch, Hq=34) == UNSUP
    assert attn_call(lib, lay, canon, patch, scale=float("nan")) == RANGE
    assert attn_call(lib, lay, canon, patch, scale=float("inf")) == RANGE
    assert attn_call(lib, lay, canon, patch, q=QA + 2) == ALIGN
    assert attn_call(lib, lay, canon, patch, out=OA + 4) == ALIGN
    assert attn_call(lib, lay, canon, patch, ws=W + 64) == ALIGN
    assert attn_call(lib, lay, canon, patch, wsb=100) == RANGE
    assert attn_call(lib, lay, canon, patch, ws=0) == NULL
    assert attn_call(lib, lay, canon, patch, q=0) == NULL
    assert attn_call(lib, lay, canon, patch, out=QA) == ALIAS                  # out over the queries
    assert attn_call(lib, lay, canon, patch, lse=OA + 16) == ALIAS             # lse inside out
    assert attn_call(lib, lay, canon, patch, out=A + 0x100) == ALIAS           # out inside the store
    assert attn_call(lib, lay, canon, patch, ws=B) == ALIAS                    # workspace over U_K
    lay, canon, patch = make_attn(m=12)
    assert attn_call(lib, lay, canon, patch) == RANGE                          # rank not a multiple of 8
    lay, canon, patch = make_attn(m=16)
    patch.u[1] = 0
    assert attn_call(lib, lay, canon, patch) == NULL
    lay, canon, patch = make_attn(Dh=96)
    assert attn_call(lib, lay, canon, patch) == UNSUP
    lay, canon, patch = make_attn(Dh=576, H=1, S=1)
    lay.rope_offset, lay.rope_dim = 448, 128
    assert attn_call(lib, lay, canon, patch, Hq=16) == UNSUP                   # one stream, not 512 + 64
    lay.rope_offset, lay.rope_dim = 512, 64
    assert attn_call(lib, lay, canon, patch, Hq=17) == UNSUP                   # MLA: at most 16 heads
    assert attn_call(lib, lay, canon, patch, Hq=16, out=A + 0x40) == ALIAS     # out inside the store
    lay, canon, patch = make_attn()
    canon.chunk_stride = 40 * 256 - 8
    assert attn_call(lib, lay, canon, patch) == SHAPE
    lay, canon, patch = make_attn()
    canon.rows[0] = A + 2
    assert attn_call(lib, lay, canon, patch) == ALIGN


def host_call(lib, lay, canon, n=2, ids=(0, 1), delta=C, patch=None, dst=None, staging=W, sb=1 << 40):
    from position_invariant_kv_amd import _abi
    b = ctypes.byref
    ids_c = (ctypes.c_int32 * max(len(ids), 1))(*ids)
    if dst is None:
        dst = _abi.KameraDst((ctypes.c_void_p * 2)(D, D + 0x1000000), 2 * 40 * 128, 2 * 40, 16, E, 0, 0, 0)
    return lib.kamera_relocate_patch_host(b(lay), b(canon), n, ids_c, ctypes.c_void_p(delta),
                                          b(patch) if patch is not None else None, b(dst), ctypes.c_void_p(staging),
                                          ctypes.c_int64(sb), None, None)


def test_host_staging_query(lib):
    b = ctypes.byref
    lay = make_form()[0]                       # 2 layers, 2 heads x 64, 2 streams
    assert lib.kamera_host_staging_bytes(b(lay), 40, 1) == 2 * 2 * 40 * 128 * 2
    assert lib.kamera_host_staging_bytes(b(lay), 41, 3) == 3 * ((2 * 2 * 41 * 128 * 2 + 255) // 256 * 256)
    assert lib.kamera_host_staging_bytes(b(lay), 40, 0) == -1
    assert lib.kamera_host_staging_bytes(None, 40, 1) == -1


def test_host_relocation_validation(lib):
    # checks that come before the pinned-memory query (which needs a device)
    lay, canon, _, _, _ = make_form()
    assert host_call(lib, lay, canon, n=0) == OK
    assert host_call(lib, lay, canon, n=-1) == RANGE
    canon.canon_pos = 0x1234000
    assert host_call(lib, lay, canon) == UNSUP                # shifts come in delta
    lay, canon, _, _, _ = make_form()
    assert host_call(lib, lay, canon, delta=0) == NULL
    canon.layer_stride = 40 * 128 - 8
    assert host_call(lib, lay, canon) == SHAPE
    lay, canon, _, _, _ = make_form()
    canon.rows[1] = 0
    assert host_call(lib, lay, canon) == NULL
    lay, canon, _, _, _ = make_form()
    canon.rows[0] = A + 2
    assert host_call(lib, lay, canon) == ALIGN
    from position_invariant_kv_amd import _abi
    P2 = ctypes.c_void_p * 2
    lay, canon, _, _, _ = make_form()
    assert host_call(lib, lay, canon, patch=_abi.KameraPatch(72, P2(B, B), P2(C, C))) == RANGE


# --------------------------------------------------------------------------
# Variable-length chunks (kamera_relocate_patch_varlen, kamera_recall_varlen)
# --------------------------------------------------------------------------

def test_varlen_struct_layout_matches_header():
    from position_invariant_kv_amd import _abi
    src = r'''
#include <stddef.h>
#include <stdio.h>
#include "kamera.h"
int main(void) {
  printf("%zu %zu %zu\n", sizeof(kamera_varlen), offsetof(kamera_varlen, n_tokens), offsetof(kamera_varlen, total_rows));
  return 0;
}
'''
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        exe = os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        got = [int(x) for x in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    assert got == [ctypes.sizeof(_abi.KameraVarlen), _abi.KameraVarlen.n_tokens.offset,
                   _abi.KameraVarlen.total_rows.offset]


def make_vl(total_rows=1000):
    from position_invariant_kv_amd import _abi
    return _abi.KameraVarlen(E + 0x800, E + 0x900, total_rows)


def call_vl(lib, fn, lay, src, vl, patch, dst, n=2):
    b = ctypes.byref
    vlp = b(vl) if vl is not None else None
    pp = b(patch) if patch is not None else None
    if fn == "relocate_patch_varlen":
        return lib.kamera_relocate_patch_varlen(b(lay), b(src), vlp, n, ctypes.c_void_p(E + 0x200), pp, b(dst),
                                                None)
    return lib.kamera_recall_varlen(b(lay), b(src), vlp, n, ctypes.c_void_p(E + 0x300), ctypes.c_void_p(E + 0x400),
                                    pp, b(dst), None)


VL_FNS = ["relocate_patch_varlen", "recall_varlen"]


@pytest.mark.parametrize("fn", VL_FNS)
def test_varlen_empty_call_is_ok(lib, fn):
    lay, src, patch, dst = make()
    assert call_vl(lib, fn, lay, src, make_vl(), patch, dst, n=0) == OK
    src.n_tokens = 0           # T_max = 0: every chunk is empty
    assert call_vl(lib, fn, lay, src, make_vl(), patch, dst, n=2) == OK


@pytest.mark.parametrize("fn", VL_FNS)
def test_varlen_null_pointers(lib, fn):
    lay, src, patch, dst = make()
    assert call_vl(lib, fn, lay, src, None, patch, dst) == NULL
    vl = make_vl()
    vl.row_offset = 0
    assert call_vl(lib, fn, lay, src, vl, patch, dst) == NULL
    vl = make_vl()
    vl.n_tokens = 0
    assert call_vl(lib, fn, lay, src, vl, patch, dst) == NULL
    lay, src, patch, dst = make()
    patch.u[1] = 0
    assert call_vl(lib, fn, lay, src, make_vl(), patch, dst) == NULL


@pytest.mark.parametrize("fn", VL_FNS)
def test_varlen_alignment_and_range(lib, fn):
    lay, src, patch, dst = make()
    vl = make_vl()
    vl.row_offset += 4         # int64 array: 8-byte aligned
    assert call_vl(lib, fn, lay, src, vl, patch, dst) == ALIGN
    vl = make_vl()
    vl.n_tokens += 2           # int32 array: 4-byte aligned
    assert call_vl(lib, fn, lay, src, vl, patch, dst) == ALIGN
    assert call_vl(lib, fn, lay, src, make_vl(total_rows=-1), patch, dst) == RANGE
    lay, src, patch, dst = make(m=12)
    assert call_vl(lib, fn, lay, src, make_vl(), patch, dst) == UNSUP


@pytest.mark.parametrize("fn", VL_FNS)
def test_varlen_destination_overlapping_store_or_factors(lib, fn):
    # the store spans total_rows * F elements from rows[s]; U spans total_rows * m
    lay, src, patch, dst = make()
    F = 2 * 64
    rows_to_pool = (D - A) // (2 * F)
    assert call_vl(lib, fn, lay, src, make_vl(total_rows=rows_to_pool + 1), patch, dst) == ALIAS
    lay, src, patch, dst = make()
    patch.u[0] = D - 64        # U rows run into the pool
    assert call_vl(lib, fn, lay, src, make_vl(total_rows=10), patch, dst) == ALIAS


def host_vl_call(lib, lay, canon, vl, n=2, ids=(0, 1), delta=C, patch=None):
    from position_invariant_kv_amd import _abi
    b = ctypes.byref
    ids_c = (ctypes.c_int32 * max(len(ids), 1))(*ids)
    dst = _abi.KameraDst((ctypes.c_void_p * 2)(D, D + 0x1000000), 2 * 40 * 128, 2 * 40, 16, E, 0, 0, 0)
    return lib.kamera_relocate_patch_host_varlen(b(lay), b(canon), b(vl) if vl is not None else None, n, ids_c,
                                                 ctypes.c_void_p(delta), b(patch) if patch is not None else None,
                                                 b(dst), ctypes.c_void_p(W), ctypes.c_int64(1 << 40), None, None)


def test_host_varlen_validation(lib):
    # checks that come before the pinned-memory query (which needs a device)
    from position_invariant_kv_amd import _abi
    lay, canon, _, _, _ = make_form()
    ro = (ctypes.c_int64 * 3)(0, 80, 160)      # host arrays in this call
    nt = (ctypes.c_int32 * 3)(40, 40, 40)
    vl = _abi.KameraVarlen(ctypes.addressof(ro), ctypes.addressof(nt), 240)
    assert host_vl_call(lib, lay, canon, vl, n=0) == OK
    assert host_vl_call(lib, lay, canon, None) == NULL
    assert host_vl_call(lib, lay, canon, vl, delta=0) == NULL
    bad = _abi.KameraVarlen(0, ctypes.addressof(nt), 240)
    assert host_vl_call(lib, lay, canon, bad) == NULL
    bad = _abi.KameraVarlen(ctypes.addressof(ro), ctypes.addressof(nt), -1)
    assert host_vl_call(lib, lay, canon, bad) == RANGE
    canon.canon_pos = 0x1234000
    assert host_vl_call(lib, lay, canon, vl) == UNSUP          # shifts come in delta
    lay, canon, _, _, _ = make_form()
    canon.rows[0] = A + 2
    assert host_vl_call(lib, lay, canon, vl) == ALIGN


# --------------------------------------------------------------------------
# The copy-ceiling probe library (include/kamera_probe.h)
# --------------------------------------------------------------------------

PROBE_HEADER = os.path.join(ROOT, "include", "kamera_probe.h")


@pytest.fixture(scope="module")
def probe_lib():
    from position_invariant_kv_amd import _abi
    if not os.path.exists(_abi.probe_lib_path()):
        from position_invariant_kv_amd import build
        build.build()
    return _abi.load_probe_library()


def test_probe_exports_every_declared_symbol(probe_lib):
    from position_invariant_kv_amd import _abi
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(kamera_probe_[a-z_]+)\s*\(", text)))
    assert declared == sorted(_abi.PROBE_SIGNATURES)
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.probe_lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kamera_probe_\w+)", out))
    for name in declared:
        assert name in exported, name


def test_probe_validation(probe_lib):
    # fake addresses, never dereferenced: every call fails validation or is empty
    f = probe_lib.kamera_probe_copy_blocks
    V = ctypes.c_void_p
    assert f(None, 1 << 20, V(B), 1 << 20, None, None, 4, 4096, 1, None) == 1          # NULL src
    assert f(V(A + 8), 1 << 20, V(B), 1 << 20, None, None, 4, 4096, 1, None) == 2      # misaligned src
    assert f(V(A), 1 << 20, V(B), 1 << 20, V(C + 4), None, 4, 4096, 1, None) == 2      # misaligned offsets
    assert f(V(A), 1 << 20, V(B), 1 << 20, None, None, 4, 4100, 1, None) == 2          # block not 16-B
    assert f(V(A), 1 << 20, V(B), 1 << 20, None, None, 4, 4096, 3, None) == 4          # vectors per thread
    assert f(V(A), 1 << 20, V(B), 1 << 20, None, None, -1, 4096, 1, None) == 4         # negative count
    assert f(V(A), 1 << 40, V(B), 1 << 40, None, None, 1 << 20, 1 << 20, 1, None) == 4  # >= 2^31 vectors
    assert f(V(A), 1 << 20, V(B), 1 << 20, None, None, 0, 4096, 1, None) == 0          # empty


def test_noalloc_validation(lib):
    # the allocation-free call refuses, before any HIP call, a call whose page
    # order would not fit its static scratch (262,144 int32), and NULL structs
    b = ctypes.byref
    lay, src, patch, dst = make(T=1024, P=16)
    src.n_store = 5000
    st = lib.kamera_relocate_patch_noalloc(b(lay), b(src), 5000, ctypes.c_void_p(E + 0x200), b(patch), b(dst),
                                           None)
    assert st == RANGE   # 5000 x 64 pages
    dst.error_word = E + 0x900
    st = lib.kamera_relocate_patch_noalloc(b(lay), b(src), 2100, ctypes.c_void_p(E + 0x200), b(patch), b(dst),
                                           None)
    assert st == RANGE   # 2100 x 64 x 2 + 2100 with the content checks
    assert lib.kamera_relocate_patch_noalloc(b(lay), b(src), 2, ctypes.c_void_p(E + 0x200), None, b(dst),
                                             None) == NULL
    assert lib.kamera_relocate_patch_noalloc(b(lay), None, 2, ctypes.c_void_p(E + 0x200), b(patch), b(dst),
                                             None) == NULL
