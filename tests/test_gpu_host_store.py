"""GPU parity of relocation from a pinned host store (kamera_relocate_patch_host).

Each case is a recall workload from the seeded generators whose canonical
store is copied to pinned host memory.  The pool the call writes is compared
with the oracle (the same bar as the device-store parity tests: bit-exact
scatter map, sentinel and copied elements; otherwise within 1 bf16 ulp of the
oracle's single rounding or 4e-3 of the block's max|y|) and, bit for bit,
with kamera_recall on the device copy of the same store.
"""

import ctypes
from dataclasses import replace

import numpy as np
import pytest
import torch

import position_invariant_kv_amd as kam
from tests import harness as H
from workloads import RECALL_CONFIG, bits, make_inputs, small_workload

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-host] {msg}", flush=True)


def run_host(w, inp, slots, same_stream=False, strided=False):
    """The recall of `inp` through the host-store entry point (a fresh pool)."""
    ids = inp["chunk_ids"].cpu().tolist()
    canon = inp["canon_pos"]
    tp = inp["target_pos"]
    delta = (tp - (canon[inp["chunk_ids"].long()] if canon is not None else 0)).contiguous()
    if strided:
        # a host store whose layers are further apart than T rows
        host = []
        for x in inp["src"]:
            big = torch.empty((x.shape[0], x.shape[1], x.shape[2] + 8, x.shape[3]), dtype=x.dtype, pin_memory=True)
            big[:, :, : x.shape[2]] = x.cpu()
            host.append(big[:, :, : x.shape[2]])
    else:
        host = [x.cpu().pin_memory() for x in inp["src"]]
    u = v = None
    if w.rank > 0:
        sel = inp["chunk_ids"].long()
        u = [x[sel].contiguous() for x in inp["u"]]
        v = [x[sel].contiguous() for x in inp["v"]]
    pool = [p.clone() for p in inp["pool0"]]
    copy_stream = torch.cuda.current_stream() if same_stream else None
    kam.relocate_patch_host(H.layouts(w)[1], host, ids, delta, pool, u=u, v=v, page_size=w.page_size,
                            page_table=inp["page_table"], dst_offset=inp["dst_offset"], slots=slots,
                            copy_stream=copy_stream)
    torch.cuda.synchronize()
    return pool


def check_case(w, seed, slots, **kw):
    inp = make_inputs(w, "cuda", seed=seed)
    inp["pool0"] = [p.clone() for p in inp["pool"]]
    pool = run_host(w, inp, slots, **kw)
    # the device path on the same inputs
    H.run_gpu(w, inp)
    torch.cuda.synchronize()
    for s in range(w.num_streams):
        assert torch.equal(pool[s].view(torch.int16), inp["pool"][s].view(torch.int16)), \
            f"stream {s}: host-store result differs from the device recall"
    inp["pool"] = pool
    blocks = [(i, l, s) for i in range(w.n_chunks) for l in range(w.num_layers) for s in range(w.num_streams)]
    H.check_blocks(w, inp, blocks, "host store")
    H.check_untouched_slots(w, inp)


CASES = {
    # name: (workload keywords, slots, extra)
    "gqa_paged_m16_two_slots": (dict(op="recall", n_tokens=100, n_chunks=5, n_store=6, rank=16, page_size=16,
                                     canon_pos_range=(0, 3000)), 2, {}),
    "gqa_paged_m16_one_slot_same_stream": (dict(op="recall", n_tokens=100, n_chunks=4, n_store=6, rank=16,
                                                page_size=16), 1, dict(same_stream=True)),
    "gqa_contiguous_no_patch_three_slots": (dict(op="recall", n_tokens=64, n_chunks=5, n_store=5, rank=0), 3, {}),
    "mla_paged_m8_strided_host": (dict(op="recall", family="MLA", num_heads=1, head_dim=576, rope_offset=512,
                                       rope_dim=64, num_streams=1, n_tokens=70, n_chunks=3, n_store=4, rank=8,
                                       page_size=64), 2, dict(strided=True)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_host_store_matches_oracle_and_device(name):
    kw, slots, extra = CASES[name]
    w = small_workload(name=name, **kw)
    _say(f"{name}: {w} slots={slots} {extra}")
    check_case(w, 300 + len(name), slots, **extra)


def test_host_store_pageable_memory_is_refused():
    # the C ABI refuses pageable host rows (the binding refuses them earlier)
    from position_invariant_kv_amd import _abi
    w = small_workload(op="recall", n_tokens=32, n_chunks=2, n_store=2, rank=0)
    inp = make_inputs(w, "cuda", seed=1)
    host = [x.cpu() for x in inp["src"]]           # not pinned
    lib = kam.load_library()
    lay = H.layouts(w)[1].c()
    src = _abi.KameraSrc((ctypes.c_void_p * 2)(host[0].data_ptr(), host[1].data_ptr()),
                         host[0].stride(0), host[0].stride(1), 32, 2, 0)
    pool = inp["pool"]
    dst = _abi.KameraDst((ctypes.c_void_p * 2)(pool[0].data_ptr(), pool[1].data_ptr()), pool[0].stride(0),
                         pool[0].shape[1], 0, 0, inp["dst_offset"].data_ptr(), 0, 0)
    ids = (ctypes.c_int32 * 2)(0, 1)
    delta = torch.zeros(2, dtype=torch.int64, device="cuda")
    staging = torch.empty(kam.host_staging_bytes(H.layouts(w)[1], 32, 1), dtype=torch.uint8, device="cuda")
    st = lib.kamera_relocate_patch_host(ctypes.byref(lay), ctypes.byref(src), 2, ids,
                                        ctypes.c_void_p(delta.data_ptr()), None, ctypes.byref(dst),
                                        ctypes.c_void_p(staging.data_ptr()), ctypes.c_int64(staging.numel()),
                                        None, None)
    assert st == 6


def test_host_store_back_to_back_calls_share_staging():
    # Two calls issued back to back on one compute stream, sharing one
    # staging buffer and one copy stream, with no host synchronisation in
    # between: the second call's first copies must wait for the first call's
    # relocations still reading the same slots.  Call A recalls outputs 0..3,
    # call B outputs 4..7, into disjoint pages of one pool; both are then
    # compared with the oracle, and the pool with the device recall.
    w = small_workload(name="back_to_back", op="recall", n_tokens=700, n_chunks=8, n_store=8, rank=32,
                       sigma=0.05, page_size=16, num_layers=6, num_heads=4, head_dim=128, rope_dim=128,
                       rope_base=1e6, canon_pos_range=(0, 3000))
    _say(f"back-to-back: {w}")
    inp = make_inputs(w, "cuda", seed=808)
    inp["pool0"] = [p.clone() for p in inp["pool"]]
    lay = H.layouts(w)[1]
    ids = inp["chunk_ids"].cpu().tolist()
    canon = inp["canon_pos"]
    delta = (inp["target_pos"] - canon[inp["chunk_ids"].long()]).contiguous()
    host = [x.cpu().pin_memory() for x in inp["src"]]
    sel = inp["chunk_ids"].long()
    u = [x[sel].contiguous() for x in inp["u"]]
    v = [x[sel].contiguous() for x in inp["v"]]
    pool = [p.clone() for p in inp["pool0"]]
    staging = torch.empty(kam.host_staging_bytes(lay, w.n_tokens, 2), dtype=torch.uint8, device="cuda")
    copy_stream = torch.cuda.Stream()
    calls = []
    for lo, hi in ((0, 4), (4, 8)):
        calls.append(kam.prepare_relocate_patch_host(
            lay, host, ids[lo:hi], delta[lo:hi].contiguous(), pool, u=[x[lo:hi].contiguous() for x in u],
            v=[x[lo:hi].contiguous() for x in v], page_size=w.page_size,
            page_table=inp["page_table"][lo:hi].contiguous(), staging=staging, copy_stream=copy_stream))
    torch.cuda.synchronize()
    for c in calls:
        c()
    torch.cuda.synchronize()
    H.run_gpu(w, inp)
    torch.cuda.synchronize()
    for s in range(w.num_streams):
        assert torch.equal(pool[s].view(torch.int16), inp["pool"][s].view(torch.int16)), f"stream {s}"
    inp["pool"] = pool
    blocks = [(i, l, s) for i in range(w.n_chunks) for l in range(w.num_layers) for s in range(w.num_streams)]
    H.check_blocks(w, inp, blocks, "host store back to back")
    H.check_untouched_slots(w, inp)


def test_host_store_full_size_sampled():
    # the benchmark's host-recall workload (reorder shapes, 8 of 16 stored
    # chunks recalled, rank 32, 16-token pages) in bench's launch configuration
    # (two slots, separate copy stream); every chunk checked bit for bit against
    # the device recall, six seeded blocks against the oracle
    import random
    w = replace(RECALL_CONFIG, name="recall_host_rank32", n_chunks=8, n_store=16)
    _say(f"full size: {w}")
    inp = make_inputs(w, "cuda")
    inp["pool0"] = [p.clone() for p in inp["pool"]]
    pool = run_host(w, inp, 2)
    H.run_gpu(w, inp)
    torch.cuda.synchronize()
    for s in range(w.num_streams):
        assert torch.equal(pool[s].view(torch.int16), inp["pool"][s].view(torch.int16)), f"stream {s}"
    inp["pool"] = pool
    rng = random.Random(5)
    blocks = {(0, 0, 0), (w.n_chunks - 1, w.num_layers - 1, 1)}
    while len(blocks) < 6:
        blocks.add((rng.randrange(w.n_chunks), rng.randrange(w.num_layers), rng.randrange(2)))
    H.check_blocks(w, inp, sorted(blocks), "host store full size")
    del inp, pool
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# Variable-length chunks from a pinned host store
# (kamera_relocate_patch_host_varlen): bit for bit against kamera_recall_varlen
# on a device copy of the same packed store, and against the oracle.
# --------------------------------------------------------------------------

def run_host_varlen(vw, inp, slots, same_stream=False):
    from tests.test_gpu_varlen import plan
    w = vw.base
    ids, deltas = plan(vw, inp)
    host = [x.cpu().pin_memory() for x in inp["src"]]
    delta = torch.tensor(deltas, dtype=torch.int64, device="cuda")
    u = v = None
    if w.rank > 0:
        ro = inp["row_offset"].cpu().tolist()
        lengths = inp["lengths"]
        u = [torch.cat([x[ro[c]:ro[c] + w.num_layers * lengths[c]] for c in ids]).contiguous() for x in inp["u"]]
        sel = torch.tensor(ids, dtype=torch.long, device="cuda")
        v = [x[sel].contiguous() for x in inp["v"]]
    pool = [p.clone() for p in inp["pool0"]]
    copy_stream = torch.cuda.current_stream() if same_stream else None
    kam.relocate_patch_host_varlen(H.layouts(w)[1], host, inp["row_offset"].cpu(), inp["n_tokens"].cpu(),
                                   inp["max_tokens"], ids, delta, pool, u=u, v=v, page_size=w.page_size,
                                   page_table=inp["page_table"], dst_offset=inp["dst_offset"], slots=slots,
                                   copy_stream=copy_stream)
    torch.cuda.synchronize()
    return pool


VL_CASES = {
    # name: (base workload keywords, length range, multiple, slots, same stream)
    "gqa_recall_paged_m16_two_slots": (dict(op="recall", n_store=6, n_chunks=5, rank=16, page_size=16), (1, 100), 1,
                                       2, False),
    "gqa_relocate_contiguous_m0_one_slot": (dict(op="relocate", n_store=4, n_chunks=4, rank=0), (0, 90), 1, 1, True),
    "mla_recall_paged64_m8_three_slots": (dict(op="recall", family="MLA", num_heads=1, head_dim=576, rope_offset=512,
                                               rope_dim=64, num_streams=1, n_store=4, n_chunks=3, rank=8,
                                               page_size=64), (1, 150), 1, 3, False),
}


@pytest.mark.parametrize("name", sorted(VL_CASES))
def test_host_store_varlen_matches_device_and_oracle(name):
    from tests.test_gpu_varlen import all_blocks, check_blocks, check_untouched, run_varlen
    from workloads import VarlenWorkload, make_varlen_inputs
    kw, lr, q, slots, same = VL_CASES[name]
    vw = VarlenWorkload(name, small_workload(name=name, **kw), len_range=lr, len_multiple=q)
    inp = make_varlen_inputs(vw, "cuda", seed=500 + len(name))
    _say(f"{name}: lengths {inp['lengths']} out {inp['out_ids']} slots={slots}")
    inp["pool0"] = [p.clone() for p in inp["pool"]]
    pool = run_host_varlen(vw, inp, slots, same_stream=same)
    run_varlen(vw, inp)
    torch.cuda.synchronize()
    for s in range(vw.base.num_streams):
        assert torch.equal(pool[s].view(torch.int16), inp["pool"][s].view(torch.int16)), \
            f"stream {s}: host-store result differs from the device call"
    inp["pool"] = pool
    check_blocks(vw, inp, all_blocks(vw), f"host varlen {name}")
    check_untouched(vw, inp)


def test_host_store_varlen_bad_length_is_refused():
    # host lengths are checked before any copy: the pool stays untouched
    from workloads import VarlenWorkload, make_varlen_inputs
    vw = VarlenWorkload("bad", small_workload(op="recall", n_store=3, n_chunks=2, rank=0, page_size=16),
                        len_range=(16, 64))
    inp = make_varlen_inputs(vw, "cuda", seed=77)
    host = [x.cpu().pin_memory() for x in inp["src"]]
    nt = inp["n_tokens"].cpu().clone()
    c = inp["out_ids"][0]
    nt[c] = vw.max_tokens + 16
    pool0 = [p.clone() for p in inp["pool"]]
    with pytest.raises(kam.KameraError) as e:
        kam.relocate_patch_host_varlen(H.layouts(vw.base)[1], host, inp["row_offset"].cpu(), nt, vw.max_tokens,
                                       inp["out_ids"], torch.zeros(2, dtype=torch.int64, device="cuda"),
                                       inp["pool"], page_size=16, page_table=inp["page_table"])
    assert e.value.status == 4
    torch.cuda.synchronize()
    for s in range(2):
        assert torch.equal(pool0[s].view(torch.int16), inp["pool"][s].view(torch.int16))
