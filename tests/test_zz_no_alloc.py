"""kamera_relocate_patch_noalloc against kamera_relocate_patch, through the C ABI.

The allocation-free entry point keeps the call's scratch (the page order of a
paged pool, the content checks' copies with an error word) in the library's
static device array.  Its output must be the existing entry point's, bit for
bit (the same kernels), on two calls in a row, the second with a smaller
input (so the array holds the first call's leftovers), with and without an
error word; a call that needs more scratch than the array holds is refused
before any work.
"""

import ctypes

import pytest
import torch

import position_invariant_kv_amd as kam
from position_invariant_kv_amd import _abi
from tests import harness as H
from workloads import make_inputs, small_workload

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-noalloc] {msg}", flush=True)


def run_both(w, seed, with_error_word):
    a = make_inputs(w, "cuda", seed=seed)
    b = make_inputs(w, "cuda", seed=seed)
    _, lay = H.layouts(w)
    ea = torch.zeros(1, dtype=torch.int32, device="cuda") if with_error_word else None
    eb = torch.zeros(1, dtype=torch.int32, device="cuda") if with_error_word else None
    kw = dict(page_size=w.page_size, canon_pos=a["canon_pos"])
    kam.prepare_relocate_patch(lay, a["src"], a["delta"], a["u"], a["v"], a["pool"], page_table=a["page_table"],
                               dst_offset=a["dst_offset"], error_word=ea, **kw)()
    kam.prepare_relocate_patch_noalloc(lay, b["src"], b["delta"], b["u"], b["v"], b["pool"],
                                       page_table=b["page_table"], dst_offset=b["dst_offset"], error_word=eb,
                                       **kw)()
    torch.cuda.synchronize()
    for s in range(w.num_streams):
        assert torch.equal(a["pool"][s].view(torch.int16), b["pool"][s].view(torch.int16)), f"stream {s}"
    if with_error_word:
        assert int(ea.item()) == int(eb.item()) == 0
    H.check_blocks(w, b, [(i, l, s) for i in range(w.n_chunks) for l in range(w.num_layers)
                          for s in range(w.num_streams)], "noalloc")


CASES = {
    # two calls in a row per case: a larger then a smaller input
    "mla_pages64": [dict(family="MLA", num_heads=1, head_dim=576, rope_offset=512, rope_dim=64, num_streams=1,
                         rank=32, sigma=0.02, page_size=64, delta_range=(-32768, 32768), n_tokens=300, n_chunks=6),
                    dict(family="MLA", num_heads=1, head_dim=576, rope_offset=512, rope_dim=64, num_streams=1,
                         rank=32, sigma=0.02, page_size=64, delta_range=(-32768, 32768), n_tokens=130, n_chunks=2)],
    "gqa_pages16": [dict(num_heads=4, head_dim=128, rope_dim=128, rope_base=1e6, rank=16, sigma=0.02,
                         page_size=16, n_tokens=200, n_chunks=5),
                    dict(num_heads=4, head_dim=128, rope_dim=128, rope_base=1e6, rank=16, sigma=0.02,
                         page_size=16, n_tokens=70, n_chunks=2)],
    "contiguous": [dict(rank=8, n_tokens=150, n_chunks=3), dict(rank=8, n_tokens=40, n_chunks=1)],
}


@pytest.mark.parametrize("with_error_word", [False, True])
@pytest.mark.parametrize("name", sorted(CASES))
def test_noalloc_matches_relocate_patch(name, with_error_word):
    for k, kw in enumerate(CASES[name]):
        w = small_workload(name=f"{name}_{k}", **kw)
        _say(f"{name} call {k} error_word={with_error_word}: {w}")
        run_both(w, 900 + k, with_error_word)


def test_noalloc_refuses_more_than_its_scratch():
    # 5000 chunks x 64 pages = 320,000 page-order entries > 262,144: refused
    # on the host (no kernel runs; the pointers are never read)
    w = small_workload(rank=8, n_tokens=16, n_chunks=1, page_size=16)
    inp = make_inputs(w, "cuda", seed=1)
    _, lay = H.layouts(w)
    lib = kam.load_library()
    src = _abi.KameraSrc((ctypes.c_void_p * 2)(inp["src"][0].data_ptr(), inp["src"][1].data_ptr()),
                         inp["src"][0].stride(0), inp["src"][0].stride(1), 1024, 1, 0)
    pool = inp["pool"]
    dst = _abi.KameraDst((ctypes.c_void_p * 2)(pool[0].data_ptr(), pool[1].data_ptr()), pool[0].stride(0),
                         pool[0].shape[1], 16, inp["page_table"].data_ptr(), 0, 0, 0, 0)
    patch = _abi.KameraPatch(8, (ctypes.c_void_p * 2)(inp["u"][0].data_ptr(), inp["u"][1].data_ptr()),
                             (ctypes.c_void_p * 2)(inp["v"][0].data_ptr(), inp["v"][1].data_ptr()))
    st = lib.kamera_relocate_patch_noalloc(ctypes.byref(lay.c()), ctypes.byref(src), 5000,
                                           ctypes.c_void_p(inp["delta"].data_ptr()), ctypes.byref(patch),
                                           ctypes.byref(dst), None)
    assert st == 4
