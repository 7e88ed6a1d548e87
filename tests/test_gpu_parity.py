"""GPU parity of the HIP library against the CPU oracle, through the C ABI.

Small cases compare every output block element by element (several 32-token
tiles, ragged tails, every entry point, both RoPE pairings, partial rotary
spans, MLA rows, m from 0 to 64).  The full-size workloads run in the same
launch configuration as bench.py and compare a seeded sample of whole
(chunk, layer, stream) blocks, plus properties checked over the whole pool:
the scatter writes every target slot and nothing else, and at m = 0 the copied
elements are bit-exact.
"""

import random
import zlib

import numpy as np
import pytest
import torch

import position_invariant_kv_amd as kam
from oracle import kamera_oracle as ko
from tests import harness as H
from workloads import (MLA, RECALL_CONFIG, REORDER, SENTINEL_BITS, SINGLE_FRAME, SURVIVAL, TINY, bits, by_name,
                       make_inputs, small_workload)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


SMALL = {
    "gqa_paged_ragged_m8": dict(kw=dict(n_tokens=80, page_size=16)),
    "gqa_contig_relocate_m0": dict(kw=dict(op="relocate", rank=0, n_tokens=47)),
    "gqa_d128_m16_paged": dict(kw=dict(num_heads=4, head_dim=128, rope_dim=128, rope_base=1e6,
                                       n_tokens=100, rank=16, sigma=0.02, page_size=16,
                                       delta_range=(-4096, 8192))),
    "gqa_m64_single_head": dict(kw=dict(num_heads=1, head_dim=128, rope_dim=128, n_tokens=33,
                                        rank=64, sigma=0.05)),
    "gqa_m24": dict(kw=dict(rank=24, n_tokens=65, sigma=0.1)),
    "interleaved_m8": dict(kw=dict(rope_style=1, n_tokens=70, page_size=16)),
    "interleaved_m0": dict(kw=dict(rope_style=1, op="relocate", rank=0, n_tokens=70)),
    "partial_rope_m8": dict(kw=dict(head_dim=128, rope_offset=64, rope_dim=64, n_tokens=40)),
    "partial_rope_m0": dict(kw=dict(head_dim=192, rope_offset=64, rope_dim=64, op="relocate",
                                    rank=0, n_tokens=40)),
    "mla_small_m32": dict(kw=dict(family="MLA", num_heads=1, head_dim=576, rope_offset=512,
                                  rope_dim=64, num_streams=1, n_tokens=70, rank=32, sigma=0.02,
                                  page_size=64, delta_range=(-32768, 32768))),
    "mla_small_m0": dict(kw=dict(family="MLA", num_heads=1, head_dim=576, rope_offset=512,
                                 rope_dim=64, num_streams=1, n_tokens=70, rank=0, op="relocate",
                                 page_size=64, delta_range=(-32768, 32768))),
    "reorder_m16": dict(kw=dict(op="reorder", n_chunks=5, n_tokens=40, rank=16, page_size=16,
                                canon_pos_range=(0, 5000), base_pos=123)),
    "reorder_m0": dict(kw=dict(op="reorder", n_chunks=4, n_tokens=40, rank=0, page_size=16,
                               canon_pos_range=(0, 5000), base_pos=7)),
    "recall_m8_contig": dict(kw=dict(op="recall", n_chunks=3, n_store=6, n_tokens=40, rank=8,
                                     canon_pos_range=(0, 3000))),
    "recall_m0_paged": dict(kw=dict(op="recall", n_chunks=3, n_store=6, n_tokens=40, rank=0,
                                    page_size=16, canon_pos_range=(0, 3000))),
    "single_token": dict(kw=dict(n_tokens=1, page_size=16)),
    "huge_delta": dict(kw=dict(delta_range=(-10_000_000, 10_000_000), rope_base=1e6, n_tokens=50)),
    "page_size_1": dict(kw=dict(n_tokens=37, page_size=1)),
    "page_size_48": dict(kw=dict(n_tokens=100, page_size=48, rank=16)),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_case_full_parity(name):
    w = small_workload(name=name, **SMALL[name]["kw"])
    _say(f"{name}: {w}")
    inp = make_inputs(w, "cuda", seed=zlib.crc32(name.encode()) % 100000)
    H.run_gpu(w, inp)
    torch.cuda.synchronize()
    blocks = [(i, l, s) for i in range(w.n_chunks) for l in range(w.num_layers)
              for s in range(w.num_streams)]
    H.check_blocks(w, inp, blocks, name)
    H.check_untouched_slots(w, inp)
    if w.rank == 0:
        for s in range(w.num_streams):
            o_lay, _ = H.layouts(w)
            cols = None if s == 1 else torch.from_numpy(~ko.rope_touched_mask(o_lay)).cuda()
            if cols is None or bool(cols.any()):
                H.check_copy_stream(w, inp, s, cols)


# Paged calls write the pool either in page-table order or, with the
# destination-order scratch, in ascending page-id order.  Both must give the
# same bits.  Cases: partial last pages, blocks and token groups that lie
# wholly past a partial page (early exit), page sizes holding one or two token
# groups of the patch kernel, and a call whose sort spans several runs.
ORDER_CASES = {
    "rows_partial_page": dict(op="relocate", rank=0, n_tokens=70, page_size=32),
    "rows_pages16_ragged": dict(op="relocate", rank=0, n_tokens=70, page_size=16, n_chunks=3),
    "rows_interleaved": dict(op="relocate", rank=0, rope_style=1, n_tokens=45, page_size=16),
    "rows_recall": dict(op="recall", rank=0, n_chunks=3, n_store=6, n_tokens=40, page_size=16,
                        canon_pos_range=(0, 3000)),
    "rows_mla": dict(family="MLA", num_heads=1, head_dim=576, rope_offset=512, rope_dim=64,
                     num_streams=1, n_tokens=150, rank=0, op="relocate", page_size=64,
                     delta_range=(-32768, 32768)),
    # pages of P*F = 2048 elements force one vector per thread in destination
    # order, where rotate-half partners 8, 16 and 32 lanes away come from
    # cross-lane moves (the page-table order runs pair units instead)
    "rows_partner_lanes8": dict(op="relocate", rank=0, num_heads=2, head_dim=128, rope_dim=128,
                                rope_base=1e6, n_tokens=70, page_size=8),
    "rows_partner_lanes16": dict(op="relocate", rank=0, num_heads=1, head_dim=256, rope_dim=256,
                                 n_tokens=37, page_size=8),
    "rows_partner_lanes32": dict(op="relocate", rank=0, num_heads=1, head_dim=512, rope_dim=512,
                                 n_tokens=21, page_size=4),
    "patch_w4_p32": dict(num_heads=2, head_dim=128, rope_dim=128, n_tokens=70, rank=16, sigma=0.05,
                         page_size=32),
    "patch_w2_p64": dict(n_tokens=150, rank=8, page_size=64),
    "patch_w2_p128_two_groups": dict(n_tokens=150, rank=24, sigma=0.1, page_size=128, n_chunks=3),
    "patch_mla_p64": dict(family="MLA", num_heads=1, head_dim=576, rope_offset=512, rope_dim=64,
                          num_streams=1, n_tokens=130, rank=32, sigma=0.02, page_size=64,
                          delta_range=(-32768, 32768)),
    # pages smaller than a token group (the patch kernel keeps the table order)
    "patch_reorder_p16_units2": dict(op="reorder", n_chunks=4, num_heads=2, head_dim=128, rope_dim=128,
                                     n_tokens=70, rank=32, sigma=0.05, page_size=16,
                                     canon_pos_range=(0, 5000), base_pos=40),
    "patch_w2_p16_units4": dict(n_tokens=150, rank=16, sigma=0.05, page_size=16, n_chunks=3),
    "patch_recall_p1": dict(op="recall", n_chunks=3, n_store=5, n_tokens=37, rank=8, page_size=1,
                            canon_pos_range=(0, 3000)),
    "patch_reorder_p64": dict(op="reorder", n_chunks=5, n_tokens=100, rank=16, page_size=64,
                              canon_pos_range=(0, 5000), base_pos=123),
    # more pages of 16 tokens (the patch kernel keeps the table order): an odd
    # page count, MLA rows, interleaved pairs, rank 64, a partial rotary span
    "patch_p16_odd_entries": dict(op="reorder", n_chunks=3, num_heads=2, head_dim=128, rope_dim=128,
                                     n_tokens=70, rank=32, sigma=0.05, page_size=16, canon_pos_range=(0, 5000),
                                     base_pos=40),
    "patch_p16_mla_recall": dict(op="recall", family="MLA", num_heads=1, head_dim=576, rope_offset=512,
                                    rope_dim=64, num_streams=1, n_chunks=3, n_store=5, n_tokens=37, rank=32,
                                    sigma=0.02, page_size=16, canon_pos_range=(0, 3000)),
    "patch_p16_interleaved": dict(rope_style=1, n_tokens=50, rank=8, page_size=16, n_chunks=3),
    "patch_p16_rank64": dict(num_heads=2, head_dim=128, rope_dim=128, n_tokens=33, rank=64, sigma=0.05,
                                page_size=16, n_chunks=4),
    "patch_p16_partial_rope": dict(head_dim=128, rope_offset=64, rope_dim=64, n_tokens=45, rank=16,
                                      page_size=16, n_chunks=2),
}


@pytest.mark.parametrize("name", sorted(ORDER_CASES))
def test_page_order_same_bits(name):
    w = small_workload(name=name, **ORDER_CASES[name])
    _say(f"page order {name}: {w}")
    seed = zlib.crc32(name.encode()) % 100000
    a = make_inputs(w, "cuda", seed=seed)
    b = make_inputs(w, "cuda", seed=seed)
    H.run_gpu(w, a, page_order=None)
    H.run_gpu(w, b)          # destination order
    torch.cuda.synchronize()
    for s in range(w.num_streams):
        assert torch.equal(a["pool"][s].view(torch.int16), b["pool"][s].view(torch.int16)), f"stream {s}"
    blocks = [(i, l, s) for i in range(w.n_chunks) for l in range(w.num_layers)
              for s in range(w.num_streams)]
    H.check_blocks(w, b, blocks, name)
    H.check_untouched_slots(w, b)


def test_page_order_multi_run_sort():
    # 200 chunks x 44 pages = 8800 page-table entries: the sort runs in two
    # workgroups (8192 + 608 entries); sampled blocks against the oracle
    w = small_workload(name="order_runs", op="relocate", rank=0, n_chunks=200, n_tokens=700,
                       page_size=16, num_layers=2)
    _say(f"page order multi-run: {w}")
    a = make_inputs(w, "cuda", seed=41)
    b = make_inputs(w, "cuda", seed=41)
    H.run_gpu(w, a, page_order=None)
    H.run_gpu(w, b)
    torch.cuda.synchronize()
    for s in range(2):
        assert torch.equal(a["pool"][s].view(torch.int16), b["pool"][s].view(torch.int16)), f"stream {s}"
    rng = random.Random(3)
    blocks = {(0, 0, 0), (199, 1, 1)} | {(rng.randrange(200), rng.randrange(2), rng.randrange(2))
                                         for _ in range(6)}
    H.check_blocks(w, b, sorted(blocks), "order_runs")
    H.check_untouched_slots(w, b)
    del a, b
    _free()


@pytest.mark.parametrize("n_chunks,n_tokens,page_size", [(3, 70, 16), (200, 700, 16), (1, 1, 16)])
def test_page_order_scratch_is_sorted(n_chunks, n_tokens, page_size):
    # the scratch holds, run by run (8192 entries), the page-table entries in
    # ascending (page id, entry) order; page ids here include out-of-range ones
    w = small_workload(op="relocate", rank=0, n_chunks=n_chunks, n_tokens=n_tokens, page_size=page_size)
    inp = make_inputs(w, "cuda", seed=n_chunks)
    pt = inp["page_table"].clone()
    flat = pt.view(-1)
    if flat.numel() > 2:
        flat[1] = -7                      # rejected by the kernels, still sorted
        flat[-1] = inp["num_pages"] + 5
    inp["page_table"] = pt
    entries = flat.numel()
    order = torch.full((entries + 3,), -99, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    H.prepare_gpu(w, inp, error_word=err, page_order=order)()
    torch.cuda.synchronize()
    got = order.cpu().numpy()
    ids = flat.cpu().numpy().astype(np.int64)
    want = np.concatenate([r0 + np.lexsort((np.arange(r0, min(entries, r0 + 8192)), ids[r0:r0 + 8192]))
                           for r0 in range(0, entries, 8192)])
    assert np.array_equal(got[:entries], want)
    assert (got[entries:] == -99).all()   # nothing written past the entries


def test_tiny_config_full():
    w = TINY
    _say(w.name)
    inp = make_inputs(w, "cuda")
    H.run_gpu(w, inp)
    torch.cuda.synchronize()
    H.check_blocks(w, inp, [(0, 0, 0), (0, 0, 1)], w.name)
    H.check_untouched_slots(w, inp)


FULL = [c.name for c in (SINGLE_FRAME, SURVIVAL, REORDER, MLA, RECALL_CONFIG)]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    w = by_name(name)
    _say(f"full size {name}")
    inp = make_inputs(w, "cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    H.run_gpu(w, inp, error_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    rng = random.Random(7)
    blocks = {(0, 0, 0), (w.n_chunks - 1, w.num_layers - 1, w.num_streams - 1)}
    while len(blocks) < 6:
        blocks.add((rng.randrange(w.n_chunks), rng.randrange(w.num_layers), rng.randrange(w.num_streams)))
    stats = H.check_blocks(w, inp, sorted(blocks), name)
    _say(f"{name}: max ulp / identical fraction per block {stats}")
    H.check_untouched_slots(w, inp)
    if w.rank == 0:
        H.check_copy_stream(w, inp, 1)
    del inp
    _free()


def test_identity_shift_is_bit_exact_copy():
    # R(0) = I: with delta 0 and m = 0 every stream is copied bit for bit
    w = small_workload(op="relocate", rank=0, n_tokens=96, page_size=16, delta_fixed=0,
                       num_heads=4, head_dim=128, rope_dim=128)
    inp = make_inputs(w, "cuda", seed=11)
    H.run_gpu(w, inp)
    for s in range(2):
        H.check_copy_stream(w, inp, s)


@pytest.mark.parametrize("style", [0, 1])
def test_two_pass_group_law(style):
    # P2 on the GPU (informational bound): R(d2) R(d1) = R(d1 + d2) and
    # R(-d) R(d) = I through two calls, each rounding to bf16.  The pool of the
    # first call (contiguous, one chunk) is the canonical source of the second.
    # Every rotated element must lie within 3 bf16 ulps of its pair's norm of
    # the one-call result (three roundings of values no larger than the norm,
    # each at most half an ulp of it, and a rotation of the first: below 2 ulps;
    # a wrong sign, pairing or angle is off by the order of the norm, 2^7 ulps);
    # the unrotated stream comes back bit for bit.
    L, Hh, D, T = 2, 2, 64, 48
    F = Hh * D
    lay = kam.Layout(L, Hh, D, 0, D, 1e4, 2, style)
    rng = np.random.default_rng(70 + style)

    def dev(x):
        return torch.from_numpy(ko.f64_to_bf16_bits(x).view(np.int16)).cuda().view(torch.bfloat16)

    x = [dev(rng.standard_normal((1, L, T, F))) for _ in range(2)]

    def reloc(src, d):
        pool = [torch.zeros((L, T, F), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
        kam.relocate(lay, src, torch.tensor([d], dtype=torch.int64, device="cuda"), pool,
                     dst_offset=torch.zeros(1, dtype=torch.int64, device="cuda"))
        return pool

    def as_src(pool):
        return [p.view(1, L, T, F) for p in pool]

    # the pair partner of every rotated element
    f = np.arange(F)
    j = f % D
    partner = f - j + ((j + D // 2) % D if style == 0 else j ^ 1)
    for d1, d2 in ((12345, -4000), (3_000_001, -2_999_000), (-777, 777)):
        two = reloc(as_src(reloc(x, d1)), d2)
        one = reloc(x, d1 + d2) if d1 + d2 != 0 else [t.view(L, T, F).clone() for t in x]
        torch.cuda.synchronize()
        a = ko.bf16_bits_to_f64(bits(two[0]))
        b = ko.bf16_bits_to_f64(bits(one[0]))
        norm = np.sqrt(b ** 2 + b[..., partner] ** 2)
        assert (norm > 0).all()
        ulp = np.exp2(np.floor(np.log2(norm)) - 7)   # bf16 ulp at the norm's binade
        err = np.abs(a - b) / ulp
        assert (err <= 3).all(), (style, d1, d2, float(err.max()))
        assert np.array_equal(bits(two[1]), bits(x[1].view(L, T, F))), (style, d1, d2)
        _say(f"group law style {style} d1 {d1} d2 {d2}: max error {float(err.max()):.2f} ulps of the pair norm")


def test_rank0_patch_equals_relocate():
    w = small_workload(op="relocate", rank=0, n_tokens=64, page_size=16)
    a = make_inputs(w, "cuda", seed=5)
    b = make_inputs(w, "cuda", seed=5)
    _, lay = H.layouts(w)
    kam.relocate(lay, a["src"], a["delta"], a["pool"], page_size=16, page_table=a["page_table"])
    # an explicit rank-0 factor set goes through the same entry point
    z = [torch.zeros((w.n_chunks, w.num_layers, w.n_tokens, 0), dtype=torch.bfloat16, device="cuda")] * 2
    zv = [torch.zeros((w.n_chunks, w.num_layers, w.row_width, 0), dtype=torch.bfloat16, device="cuda")] * 2
    kam.relocate_patch(lay, b["src"], b["delta"], z, zv, b["pool"], page_size=16, page_table=b["page_table"])
    torch.cuda.synchronize()
    for s in range(2):
        assert torch.equal(a["pool"][s].view(torch.int16), b["pool"][s].view(torch.int16))


def test_patch_alone_large_factors():
    # canonical rows = 0 and sigma = 1 factors: the output is bf16(U V^T), so a
    # dropped, misindexed or transposed patch cannot hide under rounding.
    w = small_workload(rank=32, sigma=1.0, n_tokens=96, num_heads=2, head_dim=128, rope_dim=128,
                       page_size=16)
    inp = make_inputs(w, "cuda", seed=3)
    for s in range(2):
        inp["src"][s].zero_()
    H.run_gpu(w, inp)
    torch.cuda.synchronize()
    for i in range(w.n_chunks):
        for l in range(w.num_layers):
            for s in range(2):
                slots = torch.from_numpy(H.slots_of(w, inp, i)).cuda()
                got = bits(inp["pool"][s][l].index_select(0, slots))
                u = ko.bf16_bits_to_f64(bits(inp["u"][s][i, l]))
                v = ko.bf16_bits_to_f64(bits(inp["v"][s][i, l]))
                y = u @ v.T
                want = ko.f64_to_bf16_bits(y)
                H.compare_block(got, want, y, np.ones(w.row_width, bool), f"patch-only {i},{l},{s}")


def test_id_payload_scatter():
    # every (chunk, layer, stream, token) row carries its own id as small exact
    # integers; after delta 0, m 0 every pool slot holds exactly its id
    w = small_workload(op="relocate", rank=0, n_tokens=50, n_chunks=3, page_size=16, delta_fixed=0,
                       num_layers=3)
    inp = make_inputs(w, "cuda", seed=9)
    for s in range(2):
        x = inp["src"][s]
        ns, L, T, F = x.shape
        c = torch.arange(ns, device="cuda").view(ns, 1, 1, 1).expand(ns, L, T, F)
        l = torch.arange(L, device="cuda").view(1, L, 1, 1).expand(ns, L, T, F)
        t = torch.arange(T, device="cuda").view(1, 1, T, 1).expand(ns, L, T, F)
        f = torch.arange(F, device="cuda").view(1, 1, 1, F).expand(ns, L, T, F) % 4
        ids = torch.where(f == 0, c, torch.where(f == 1, l, torch.where(f == 2, t, torch.full_like(t, s))))
        x.copy_(ids.to(torch.bfloat16))
    H.run_gpu(w, inp)
    torch.cuda.synchronize()
    pt = inp["page_table"].cpu().numpy()
    for s in range(2):
        pool = inp["pool"][s].float().cpu().numpy()
        for i in range(w.n_chunks):
            for tok in range(w.n_tokens):
                slot = pt[i][tok // 16] * 16 + tok % 16
                for l in range(w.num_layers):
                    assert list(pool[l, slot, :4]) == [i, l, tok, s]
    H.check_untouched_slots(w, inp)


def test_error_word_bad_page_id_skips_rows():
    w = small_workload(op="relocate_patch", n_tokens=64, page_size=16)
    inp = make_inputs(w, "cuda", seed=21)
    num_pages = inp["num_slots"] // 16
    pt = inp["page_table"].clone()
    pt[1, 2] = num_pages          # one past the last page: the kernel must skip it
    inp["page_table"] = pt
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    H.run_gpu(w, inp, error_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) & kam.EW_PAGE
    # chunk 0 is intact; chunk 1's other pages are intact
    H.check_blocks(w, inp, [(0, l, s) for l in range(w.num_layers) for s in range(2)], "bad-page")
    plan = H.chunk_plan(w, inp)
    for l in range(w.num_layers):
        for s in range(2):
            slots = H.slots_of(w, inp, 1)
            keep = np.array([t // 16 != 2 for t in range(w.n_tokens)])
            got = bits(inp["pool"][s][l].index_select(0, torch.from_numpy(slots[keep]).cuda()))
            want, y, touched, _ = H.expected_block(w, inp, 1, l, s, plan)
            H.compare_block(got, want[keep], y[keep], touched, "bad-page rest")


def test_error_word_bad_chunk_id_skips_chunk():
    w = small_workload(op="reorder", n_chunks=4, n_tokens=40, rank=8, page_size=16)
    inp = make_inputs(w, "cuda", seed=22)
    perm = inp["perm"].clone()
    perm[2] = 99                  # not a store chunk: output 2 must be skipped
    inp["perm"] = perm
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    H.run_gpu(w, inp, error_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) & kam.EW_CHUNK
    pool = inp["pool"][0]
    slots = torch.from_numpy(H.slots_of(w, inp, 2)).cuda()
    assert bool((pool.view(torch.int16)[:, slots] == SENTINEL_BITS).all())
    H.check_blocks(w, inp, [(i, 0, s) for i in (0, 1, 3) for s in range(2)], "bad-chunk")


def test_error_word_bad_offset():
    w = small_workload(op="relocate", rank=0, n_tokens=40, n_chunks=2)
    inp = make_inputs(w, "cuda", seed=23)
    off = inp["dst_offset"].clone()
    off[1] = inp["num_slots"] - 10   # the chunk would run past the pool end
    inp["dst_offset"] = off
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    H.run_gpu(w, inp, error_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) & kam.EW_OFFSET
    H.check_blocks(w, inp, [(0, l, s) for l in range(w.num_layers) for s in range(2)], "bad-offset")


def test_empty_calls():
    w = small_workload(n_tokens=16, page_size=16)
    inp = make_inputs(w, "cuda", seed=1)
    _, lay = H.layouts(w)
    before = [p.clone() for p in inp["pool"]]
    e = torch.zeros(0, dtype=torch.int64, device="cuda")
    kam.relocate(lay, inp["src"], e, inp["pool"], page_size=16,
                 page_table=torch.zeros((0, 1), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    for a, b in zip(before, inp["pool"]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_stream_ordering_on_side_stream():
    # the call is enqueued on the given stream: work queued after it on that
    # stream sees the result
    w = small_workload(n_tokens=64, page_size=16)
    inp = make_inputs(w, "cuda", seed=31)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        H.run_gpu(w, inp, stream=st)
        snap = [p.clone() for p in inp["pool"]]
    st.synchronize()
    inp["pool"] = snap
    H.check_blocks(w, inp, [(i, l, s) for i in range(2) for l in range(2) for s in range(2)], "stream")


# P5: unit vectors in, (cos, sin) of the phase out.  Canonical rows e_j (exact
# in bfloat16) relocated by delta give, at the pair of j, exactly cos(delta
# theta_j) and sin(delta theta_j) (first half) or -sin and cos (second half),
# and zero elsewhere.  The reference is the float64 library cos/sin of
# delta * base^(-2j/R), rounded once to bfloat16; every element must be within
# 1 ulp of it, with no absolute clause.  Shifts reach the configs' +-32768
# and the +-1e7 the kernels accept; each is chosen so that no cos or sin is
# below 1e-4 in magnitude, where the float64 angle's own error (<= 1.5e-8 rad
# at 1e7) stays far below a bfloat16 ulp.
P5_SHIFTS = [32768, -32768, 30001, -29999, 12345, 300, 10_000_000, -10_000_000, 9_999_991, -7_777_777]
P5_CASES = {
    "gqa_base1e6_m0": dict(op="relocate", rank=0, rope_base=1e6),
    "gqa_base1e4_m0": dict(op="relocate", rank=0, rope_base=1e4),
    "gqa_base1e6_patch_zero": dict(op="relocate_patch", rank=16, rope_base=1e6),
    "mla_base1e4_m0": dict(op="relocate", rank=0, family="MLA", num_heads=1, head_dim=576, rope_offset=512,
                           rope_dim=64, num_streams=1, rope_base=1e4, page_size=64),
    "mla_base1e4_patch_zero": dict(op="relocate_patch", rank=32, family="MLA", num_heads=1, head_dim=576,
                                   rope_offset=512, rope_dim=64, num_streams=1, rope_base=1e4, page_size=64),
}


@pytest.mark.parametrize("name", sorted(P5_CASES))
def test_unit_vectors_give_cos_sin_within_one_ulp(name):
    kw = dict(num_layers=1, num_heads=1, head_dim=128, rope_dim=128, page_size=16, sigma=0.05)
    kw.update(P5_CASES[name])
    R, o = kw["rope_dim"], kw.get("rope_offset", 0)
    w = small_workload(name=name, n_tokens=R, n_chunks=len(P5_SHIFTS), **kw)
    _say(f"P5 {name}: {w}")
    inp = make_inputs(w, "cuda", seed=55)
    inp["delta"] = torch.tensor(P5_SHIFTS, dtype=torch.int64, device="cuda")
    x = torch.zeros_like(inp["src"][0])
    for t in range(R):
        x[:, :, t, o + t] = 1.0
    inp["src"][0].copy_(x)
    if w.rank > 0:
        for s in range(w.num_streams):
            inp["u"][s].zero_()
            inp["v"][s].zero_()
    H.run_gpu(w, inp)
    torch.cuda.synchronize()
    j = np.arange(R // 2)
    theta = np.power(np.float64(w.rope_base), -2.0 * j / R)
    for i, d in enumerate(P5_SHIFTS):
        phi = np.float64(d) * theta
        c, s = np.cos(phi), np.sin(phi)
        assert min(np.abs(c).min(), np.abs(s).min()) >= 1e-4
        y = np.zeros((R, w.row_width))
        y[j, o + j] = c               # token j holds e at the first element of pair j
        y[j, o + R // 2 + j] = s
        y[R // 2 + j, o + j] = -s     # token R/2 + j holds it at the second
        y[R // 2 + j, o + R // 2 + j] = c
        want = ko.f64_to_bf16_bits(y)
        slots = torch.from_numpy(H.slots_of(w, inp, i)).cuda()
        got = bits(inp["pool"][0][0].index_select(0, slots))
        ulp = np.abs(H.ordinal(got) - H.ordinal(want))
        assert ulp.max() <= 1, (name, d, np.argwhere(ulp > 1)[:5].tolist())
