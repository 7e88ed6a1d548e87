"""GPU tests of the content checks (kamera_dst.check_scratch with an error word).

A page id that repeats an earlier page-table entry, and a perm / chunk_ids
entry that repeats an earlier one, are removed before the operator runs: the
first occurrence (in entry order) is written, the repeat writes nothing, and
KAMERA_EW_DUP_PAGE / KAMERA_EW_DUP_CHUNK is raised.  Everything else must
still match the oracle under the usual bar.  Reorder is defined on a
permutation of the cached set (Kamera summary, section 3, "Reorder"), so a
repeated perm entry is a content error; so is a page two chunks would share.
"""

import numpy as np
import pytest
import torch

import position_invariant_kv_amd as kam
from tests import harness as H
from workloads import SENTINEL_BITS, bits, make_inputs, small_workload

pytestmark = pytest.mark.gpu

EW_DUP_PAGE, EW_DUP_CHUNK = 8, 16


def _say(msg):
    print(f"[gpu-check] {msg}", flush=True)


def token_rows(w, inp, i, keep):
    """Pool rows of output chunk i's tokens where keep[t] is True."""
    return torch.from_numpy(H.slots_of(w, inp, i)[keep]).cuda()


def check_partial(w, inp, i, keep, where):
    plan = H.chunk_plan(w, inp)
    for l in range(w.num_layers):
        for s in range(w.num_streams):
            got = bits(inp["pool"][s][l].index_select(0, token_rows(w, inp, i, keep)))
            want, y, touched, _ = H.expected_block(w, inp, i, l, s, plan)
            H.compare_block(got, want[keep], y[keep], touched, f"{where} chunk {i} layer {l} stream {s}")


def assert_sentinel(w, inp, slots, where):
    for s in range(w.num_streams):
        rows = inp["pool"][s].view(torch.int16)[:, slots]
        assert bool((rows == SENTINEL_BITS).all()), f"{where}: stream {s} rows were written"


CASES = {
    # name: workload keywords (page tables of 16-token pages unless stated);
    # the "_table" case runs without the page-order scratch
    "reorder_patch_p16": dict(op="reorder", n_chunks=5, n_store=6, n_tokens=70, rank=16, page_size=16,
                              canon_pos_range=(0, 5000), base_pos=123),
    "reorder_rows_p16_table": dict(op="reorder", n_chunks=5, n_store=6, n_tokens=70, rank=0, page_size=16,
                                   canon_pos_range=(0, 5000), base_pos=123),
    "reorder_rows_m0": dict(op="reorder", n_chunks=5, n_store=6, n_tokens=70, rank=0, page_size=16,
                            canon_pos_range=(0, 5000), base_pos=7),
    # pages of 64 with the MLA row: the patch kernel walks the pages in id order
    "recall_mla_page_order": dict(op="recall", family="MLA", num_heads=1, head_dim=576, rope_offset=512,
                                  rope_dim=64, num_streams=1, n_chunks=5, n_store=7, n_tokens=150, rank=32,
                                  sigma=0.02, page_size=64, canon_pos_range=(0, 3000)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_repeated_page_and_chunk_are_skipped(name):
    w = small_workload(name=name, **CASES[name])
    _say(f"{name}: {w}")
    inp = make_inputs(w, "cuda", seed=4242)
    key = "perm" if w.op == "reorder" else "chunk_ids"
    ids = inp[key].clone()
    ids[3] = ids[1]                      # output 3 repeats output 1's store chunk
    inp[key] = ids
    pt = inp["page_table"].clone()
    P = w.page_size
    ppc = pt.shape[1]
    pt[4, ppc - 1] = pt[0, 1]            # output 4's last page repeats output 0's second
    inp["page_table"] = pt
    orig_pages = inp["page_table"].cpu().numpy()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    H.run_gpu(w, inp, error_word=err, page_order=None if name.endswith("_table") else "auto")
    torch.cuda.synchronize()
    ew = int(err.item())
    assert ew == EW_DUP_PAGE | EW_DUP_CHUNK, ew
    # outputs 0, 1, 2 are whole (output 0 owns the shared page)
    H.check_blocks(w, inp, [(i, l, s) for i in (0, 1, 2) for l in range(w.num_layers)
                            for s in range(w.num_streams)], name)
    # output 4: every page but the repeated one
    keep = np.array([t // P != ppc - 1 for t in range(w.n_tokens)])
    check_partial(w, inp, 4, keep, name)
    # output 3 (the repeated chunk) wrote nothing
    assert_sentinel(w, inp, token_rows(w, inp, 3, np.ones(w.n_tokens, bool)), f"{name} output 3")
    # nothing else was written: the pages of outputs 0, 1, 2 and 4 (less the repeat)
    written = set(orig_pages[[0, 1, 2]].ravel().tolist()) | set(orig_pages[4, :ppc - 1].tolist())
    num_pages = inp["pool"][0].shape[1] // P
    rest = [pg for pg in range(num_pages) if pg not in written]
    slots = torch.tensor([pg * P + k for pg in rest for k in range(P)], dtype=torch.int64, device="cuda")
    assert_sentinel(w, inp, slots, f"{name} other pages")


def test_clean_call_is_unchanged_by_the_checks():
    # no repeats: the same bits with and without the checks, and no flag
    w = small_workload(name="clean", op="recall", n_chunks=4, n_store=6, n_tokens=90, rank=8, page_size=16,
                       canon_pos_range=(0, 3000))
    a = make_inputs(w, "cuda", seed=77)
    b = make_inputs(w, "cuda", seed=77)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    H.run_gpu(w, a)
    H.run_gpu(w, b, error_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for s in range(2):
        assert torch.equal(a["pool"][s].view(torch.int16), b["pool"][s].view(torch.int16))


def test_repeat_across_sort_runs():
    # 200 chunks x 44 pages = 8800 entries: the checks sort two runs (8192 +
    # 608); entry 8500 repeats entry 10's page, so its page is skipped
    w = small_workload(name="runs", op="relocate", rank=0, n_chunks=200, n_tokens=700, page_size=16,
                       num_layers=2)
    inp = make_inputs(w, "cuda", seed=41)
    pt = inp["page_table"].clone()
    flat = pt.view(-1)
    flat[8500] = flat[10]
    inp["page_table"] = pt
    i_rep, j_rep = divmod(8500, 44)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    H.run_gpu(w, inp, error_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == EW_DUP_PAGE
    H.check_blocks(w, inp, [(0, l, s) for l in range(2) for s in range(2)], "runs: owner of the page")
    keep = np.array([t // 16 != j_rep for t in range(w.n_tokens)])
    check_partial(w, inp, i_rep, keep, "runs: repeat's chunk")


def test_without_scratch_repeats_are_not_flagged():
    # an error word alone keeps the range checks only (the binding is told
    # not to bring the scratch): the repeat is written, nothing is flagged
    w = small_workload(name="noscratch", op="reorder", n_chunks=3, n_store=4, n_tokens=40, rank=0, page_size=16)
    inp = make_inputs(w, "cuda", seed=5)
    perm = inp["perm"].clone()
    perm[2] = perm[0]
    inp["perm"] = perm
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    _, lay = H.layouts(w)
    kam.prepare_reorder(lay, inp["src"], inp["perm"], inp["base_pos"], inp["pool"], page_size=16,
                        page_table=inp["page_table"], error_word=err, check_scratch=None)()
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    H.check_blocks(w, inp, [(i, l, s) for i in range(3) for l in range(w.num_layers) for s in range(2)],
                   "no scratch")
