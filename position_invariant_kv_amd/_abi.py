"""ctypes mirror of include/kamera.h and the loader of libkamera.so."""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

STATUS = {
    0: "KAMERA_OK",
    1: "KAMERA_ERR_NULL",
    2: "KAMERA_ERR_ALIGN",
    3: "KAMERA_ERR_SHAPE",
    4: "KAMERA_ERR_RANGE",
    5: "KAMERA_ERR_ALIAS",
    6: "KAMERA_ERR_UNSUPPORTED",
    7: "KAMERA_ERR_HIP",
}

_P2 = ctypes.c_void_p * 2


class KameraLayout(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("rope_offset", ctypes.c_int32),
                ("rope_dim", ctypes.c_int32), ("rope_style", ctypes.c_int32),
                ("rope_base", ctypes.c_double), ("num_streams", ctypes.c_int32)]


class KameraSrc(ctypes.Structure):
    _fields_ = [("rows", _P2), ("chunk_stride", ctypes.c_int64), ("layer_stride", ctypes.c_int64),
                ("n_tokens", ctypes.c_int32), ("n_store", ctypes.c_int32),
                ("canon_pos", ctypes.c_void_p)]


class KameraPatch(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("u", _P2), ("v", _P2)]


class KameraDst(ctypes.Structure):
    _fields_ = [("rows", _P2), ("layer_stride", ctypes.c_int64), ("num_slots", ctypes.c_int64),
                ("page_size", ctypes.c_int32), ("page_table", ctypes.c_void_p),
                ("dst_offset", ctypes.c_void_p), ("error_word", ctypes.c_void_p),
                ("page_order", ctypes.c_void_p), ("check_scratch", ctypes.c_void_p)]


class KameraVarlen(ctypes.Structure):
    _fields_ = [("row_offset", ctypes.c_void_p), ("n_tokens", ctypes.c_void_p), ("total_rows", ctypes.c_int64)]


class KameraAttnPool(ctypes.Structure):
    _fields_ = [("rows", _P2), ("layer_stride", ctypes.c_int64), ("num_slots", ctypes.c_int64),
                ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32), ("block_table", ctypes.c_void_p),
                ("seq_tokens", ctypes.c_void_p)]


class KameraSketch(ctypes.Structure):
    _fields_ = [("oversample", ctypes.c_int32), ("power_iters", ctypes.c_int32), ("omega", ctypes.c_void_p)]


class KameraFactors(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("u", _P2), ("v", _P2)]


# Every symbol include/kamera.h declares, with its ctypes signature.
_PL, _PS, _PP, _PD = (ctypes.POINTER(KameraLayout), ctypes.POINTER(KameraSrc),
                      ctypes.POINTER(KameraPatch), ctypes.POINTER(KameraDst))
_VP, _I32, _I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
SIGNATURES = {
    "kamera_relocate": (ctypes.c_int, [_PL, _PS, _I32, _VP, _PD, _VP]),
    "kamera_relocate_patch": (ctypes.c_int, [_PL, _PS, _I32, _VP, _PP, _PD, _VP]),
    "kamera_relocate_patch_noalloc": (ctypes.c_int, [_PL, _PS, _I32, _VP, _PP, _PD, _VP]),
    "kamera_reorder": (ctypes.c_int, [_PL, _PS, _I32, _VP, _I64, _PP, _PD, _VP]),
    "kamera_recall": (ctypes.c_int, [_PL, _PS, _I32, _VP, _VP, _PP, _PD, _VP]),
    "kamera_relocate_patch_varlen": (ctypes.c_int, [_PL, _PS, ctypes.POINTER(KameraVarlen), _I32, _VP, _PP, _PD,
                                                    _VP]),
    "kamera_recall_varlen": (ctypes.c_int, [_PL, _PS, ctypes.POINTER(KameraVarlen), _I32, _VP, _VP, _PP, _PD, _VP]),
    "kamera_form_patch_workspace": (ctypes.c_int64, [_PL, _I32, _I32, _I32, _I32]),
    "kamera_form_patch": (ctypes.c_int, [_PL, _PS, _PS, _I32, _VP, ctypes.POINTER(KameraSketch),
                                         ctypes.POINTER(KameraFactors), _VP, _I64, _VP]),
    "kamera_form_orbit_patch": (ctypes.c_int, [_PL, _PS, _PS, _I32, _I32, _VP, ctypes.POINTER(KameraSketch),
                                               ctypes.POINTER(KameraFactors), _VP, _I64, _VP]),
    "kamera_decode_attention_workspace": (ctypes.c_int64, [_PL, _I32, _I32, _I32]),
    "kamera_decode_attention": (ctypes.c_int, [_PL, _I32, _PS, _PP, _I32, _VP, _I32, _VP, _VP, _I32, _VP,
                                               ctypes.c_float, _VP, _VP, _VP, _VP, _I64, _VP]),
    "kamera_decode_attention_paged_workspace": (ctypes.c_int64, [_PL, _I32, _I32, _I32, _I32, _I32]),
    "kamera_decode_attention_paged": (ctypes.c_int, [_PL, _I32, _PS, _PP, ctypes.POINTER(KameraAttnPool), _I32, _VP,
                                                     _I32, _VP, _VP, _I32, _VP, ctypes.c_float, _VP, _VP, _VP, _VP,
                                                     _I64, _VP]),
    "kamera_host_staging_bytes": (ctypes.c_int64, [_PL, _I32, _I32]),
    "kamera_relocate_patch_host": (ctypes.c_int, [_PL, _PS, _I32, _VP, _VP, _PP, _PD, _VP, _I64, _VP, _VP]),
    "kamera_relocate_patch_host_varlen": (ctypes.c_int, [_PL, _PS, ctypes.POINTER(KameraVarlen), _I32, _VP, _VP,
                                                         _PP, _PD, _VP, _I64, _VP, _VP]),
    "kamera_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kamera_version": (ctypes.c_int32, []),
}


def lib_path() -> str:
    return os.environ.get("KAMERA_LIB", os.path.join(_HERE, "libkamera.so"))


def load_library():
    """Load libkamera.so once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"Kamera HIP library not found at {path}: build it with "
                "`python -m position_invariant_kv_amd.build` (there is no CPU fallback)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


# include/kamera_probe.h: the copy-ceiling probe (a measurement helper, its own library)
PROBE_SIGNATURES = {
    "kamera_probe_copy_blocks": (ctypes.c_int32, [_VP, _I64, _VP, _I64, _VP, _VP, _I64, _I64, _I32, _VP]),
}
_PROBE_LIB = None


def probe_lib_path() -> str:
    return os.path.join(_HERE, "libkamera_probe.so")


def load_probe_library():
    """Load libkamera_probe.so once; raise if it has not been built."""
    global _PROBE_LIB
    if _PROBE_LIB is None:
        path = probe_lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"copy probe library not found at {path}: build it with "
                               "`python -m position_invariant_kv_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in PROBE_SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _PROBE_LIB = lib
    return _PROBE_LIB
