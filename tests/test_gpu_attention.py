"""GPU parity of decode attention over a reused context (kamera_decode_attention)
against the CPU oracle (oracle/attention_oracle.py).

Inputs: seeded canonical stores, patch factors, queries and contexts drawn
here with NumPy (bfloat16 bits), the same bits given to both sides.

Bar: the GPU computes in fp32 with no bfloat16
rounding between the store and the output, so out may differ from the
oracle's float64 result by fp32 rounding only: logits to a few 1e-6, the
weights relative to that, the output to ~1e-5 of the largest value entry.
Every output element must be within 1e-4 * max|V| of the oracle (max over the
sequence's reconstructed values) and every lse within 1e-4 (absolute; lse is
a natural logarithm of order 1-10).  Empty contexts must give exactly 0 and
-inf.
"""

import numpy as np
import pytest
import torch

import position_invariant_kv_amd as kam
from oracle import attention_oracle as ao
from oracle import kamera_oracle as ko

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-4
LSE_TOL = 1e-4


def _say(msg):
    print(f"[gpu-attn] {msg}", flush=True)


def _bits(x):
    return ko.f64_to_bf16_bits(np.asarray(x, np.float64))


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def make_case(H, D, T, ns, L, m, Hq, seqs, seed, rope_offset=0, rope_dim=None, style=ko.ROPE_HALF, base=1e6,
              delta_range=(-8192, 8192), sigma=0.05, streams=2):
    """A store, factors, queries and contexts.  seqs: list of lists of store chunk ids.
    streams=1 is the MLA joint row (H = 1, D = 576, rope span 512..575)."""
    rng = np.random.default_rng(seed)
    R = D if rope_dim is None else rope_dim
    o_lay = ko.Layout(L, H, D, rope_offset, R, base, streams, style)
    g_lay = kam.Layout(L, H, D, rope_offset, R, base, streams, style)
    F = H * D
    canon = [_bits(rng.standard_normal((ns, L, T, F))) for _ in range(streams)]
    patch = None
    if m:
        patch = ([_bits(sigma * rng.standard_normal((ns, L, T, m))) for _ in range(streams)],
                 [_bits(sigma * rng.standard_normal((ns, L, F, m))) for _ in range(streams)])
    ids = [c for s in seqs for c in s]
    se = np.concatenate([[0], np.cumsum([len(s) for s in seqs])]).astype(np.int32)
    deltas = rng.integers(delta_range[0], delta_range[1] + 1, size=len(ids)).astype(np.int64)
    q = _bits(rng.standard_normal((len(seqs), Hq, D)))
    return o_lay, g_lay, canon, patch, se, np.array(ids, np.int32), deltas, q


def run_gpu(g_lay, layer, canon, patch, se, ids, deltas, q, scale, error_word=None):
    B, Hq, D = q.shape
    Dv = D if len(canon) == 2 else g_lay.rope_offset
    out = torch.full((B, Hq, Dv), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    u = v = None
    if patch is not None:
        u = [_dev(x) for x in patch[0]]
        v = [_dev(x) for x in patch[1]]
    kam.decode_attention(g_lay, layer, [_dev(c) for c in canon], _dev(q), torch.from_numpy(se).cuda(),
                         torch.from_numpy(ids).cuda(), torch.from_numpy(deltas).cuda(), out, scale=scale,
                         lse=lse, u=u, v=v, error_word=error_word)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check(o_lay, layer, canon, patch, se, ids, deltas, q, scale, out, lse, where):
    Hq = q.shape[1]
    ro, rl = ao.decode_attention_f64(o_lay, layer, canon, patch, se, ids.tolist(), deltas.tolist(),
                                     ko.bf16_bits_to_f64(q), Hq, scale)
    worst = 0.0
    for b in range(len(se) - 1):
        e0, e1 = int(se[b]), int(se[b + 1])
        if e0 == e1:
            assert np.all(out[b] == 0.0), f"{where}: empty context of sequence {b} must give 0"
            assert np.all(np.isneginf(lse[b])), f"{where}: empty context of sequence {b} must give -inf"
            continue
        K, V = ao.context_rows_f64(o_lay, layer, canon, patch, ids[e0:e1].tolist(), deltas[e0:e1].tolist())
        vmax = float(np.abs(V if V is not None else K[:, :ao.value_dim(o_lay)]).max())
        err = float(np.abs(out[b] - ro[b]).max())
        assert err <= OUT_TOL * vmax, f"{where}: sequence {b} output off by {err:.3e} (max|V| {vmax:.2f})"
        lerr = float(np.abs(lse[b] - rl[b]).max())
        assert lerr <= LSE_TOL, f"{where}: sequence {b} lse off by {lerr:.3e}"
        worst = max(worst, err / vmax)
    return worst


CASES = {
    # name: (H, D, T, n_store, L, m, Hq, contexts, extra)
    "gqa_g4_m16_ragged": (2, 128, 100, 4, 2, 16, 8, [[2, 0, 3], [1]], {}),
    "mha_d64_interleaved_partial_nopatch": (2, 64, 77, 3, 1, 0, 2, [[0, 1, 2], [2]],
                                            dict(rope_offset=32, rope_dim=32, style=ko.ROPE_INTERLEAVED, base=1e4)),
    "gqa_g7_m32": (2, 128, 64, 3, 1, 32, 14, [[1, 2], [0, 0, 1]], {}),
    "gqa_g2_d256_m8": (1, 256, 33, 2, 2, 8, 2, [[1], [0, 1]], {}),
    "g3_m64_one_token_chunks": (2, 64, 1, 5, 1, 64, 6, [[4, 3, 2, 1, 0]], {}),
    "empty_contexts": (2, 128, 40, 2, 1, 16, 4, [[], [0, 1], [], [1]], {}),
    "long_chunks_many_tiles": (2, 128, 2048, 2, 1, 16, 8, [[1, 0]], dict(delta_range=(-32768, 32768))),
    "g8_m64_d128": (1, 128, 300, 2, 1, 64, 8, [[0, 1]], {}),
    "g5_no_patch_d256": (2, 256, 130, 2, 1, 0, 10, [[1, 0], [0]], {}),
    "g16_m32_d128": (2, 128, 200, 3, 1, 32, 32, [[2, 1], [0]], {}),
    "g16_no_patch_d64_one_kv_head": (1, 64, 96, 2, 1, 0, 16, [[0, 1, 0]], {}),
    "g12_m64_d256": (1, 256, 70, 2, 1, 64, 12, [[1, 0]], {}),
    "mla_h16_m32": (1, 576, 150, 3, 2, 32, 16, [[2, 0], [1]],
                    dict(rope_offset=512, rope_dim=64, base=1e4, streams=1, delta_range=(-32768, 32768))),
    "mla_h8_no_patch_interleaved": (1, 576, 64, 2, 1, 0, 8, [[0, 1, 1]],
                                    dict(rope_offset=512, rope_dim=64, base=1e4, streams=1,
                                         style=ko.ROPE_INTERLEAVED)),
    "mla_h3_m64_ragged": (1, 576, 333, 2, 1, 64, 3, [[1], [], [0, 1]],
                          dict(rope_offset=512, rope_dim=64, base=1e4, streams=1)),
    # more partials per head than the combine loads in one batch (512 for
    # 512-wide rows, 128 for 128-wide), ending in a partial batch
    "mla_h16_m32_600_one_token_entries": (1, 576, 1, 5, 1, 32, 16, [[i % 5 for i in range(600)], [3]],
                                          dict(rope_offset=512, rope_dim=64, base=1e4, streams=1)),
    "gqa_g4_m16_300_one_token_entries": (2, 128, 1, 7, 1, 16, 8, [[i % 7 for i in range(300)]], {}),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_decode_attention_small(name):
    H, D, T, ns, L, m, Hq, seqs, extra = CASES[name]
    _say(f"{name}: H={H} D={D} T={T} n_store={ns} L={L} m={m} Hq={Hq} contexts={seqs}")
    o_lay, g_lay, canon, patch, se, ids, deltas, q = make_case(H, D, T, ns, L, m, Hq, seqs, 100 + len(name),
                                                               **extra)
    layer = L - 1
    scale = 1.0 / np.sqrt(D)
    out, lse = run_gpu(g_lay, layer, canon, patch, se, ids, deltas, q, scale)
    worst = check(o_lay, layer, canon, patch, se, ids, deltas, q, scale, out, lse, name)
    _say(f"{name}: worst output error {worst:.2e} of max|V|")


def _prepared(name, seed, workspace=None):
    """A prepared call of CASES[name] with its own outputs, and the oracle's arguments."""
    H, D, T, ns, L, m, Hq, seqs, extra = CASES[name]
    o_lay, g_lay, canon, patch, se, ids, deltas, q = make_case(H, D, T, ns, L, m, Hq, seqs, seed, **extra)
    B = q.shape[0]
    Dv = D if len(canon) == 2 else g_lay.rope_offset
    out = torch.full((B, Hq, Dv), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    u = v = None
    if patch is not None:
        u = [_dev(x) for x in patch[0]]
        v = [_dev(x) for x in patch[1]]
    scale = 1.0 / np.sqrt(D)
    call = kam.prepare_decode_attention(g_lay, L - 1, [_dev(c) for c in canon], _dev(q), torch.from_numpy(se).cuda(),
                                        torch.from_numpy(ids).cuda(), torch.from_numpy(deltas).cuda(), out,
                                        scale=scale, lse=lse, u=u, v=v, workspace=workspace)
    return call, (o_lay, L - 1, canon, patch, se, ids, deltas, q, scale), out, lse


def _check_prepared(name, args, out, lse):
    return check(*args, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), name)


def test_decode_attention_back_to_back_calls_share_one_workspace():
    # Calls of five shapes (GQA, MLA, empty contexts) run back to back three
    # times on one stream with no host synchronisation, sharing one workspace:
    # a merge that read partials before its own call's tiles had written them
    # would read the previous call's.
    names = ["gqa_g4_m16_ragged", "mla_h16_m32", "g16_m32_d128", "mla_h3_m64_ragged", "empty_contexts"]
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
    preps = [_prepared(n, 300 + i, workspace=ws) for i, n in enumerate(names)]
    torch.cuda.synchronize()
    for rep in range(3):
        for call, _, out, lse in preps:
            out.fill_(float("nan"))
            lse.fill_(float("nan"))
            call()
    torch.cuda.synchronize()
    for name, (_, args, out, lse) in zip(names, preps):
        _check_prepared(name, args, out, lse)
    _say("15 calls back to back on one stream: all match the oracle")


def test_decode_attention_on_two_streams():
    # calls on two streams at once, each with its own workspace and outputs
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    a = _prepared("gqa_g7_m32", 401)
    b = _prepared("mla_h16_m32", 402)
    torch.cuda.synchronize()
    for _ in range(4):
        a[0](s1)
        b[0](s2)
    torch.cuda.synchronize()
    _check_prepared("gqa_g7_m32 on stream 1", *a[1:])
    _check_prepared("mla_h16_m32 on stream 2", *b[1:])


def test_decode_attention_zero_shift_no_patch_is_plain_attention():
    # delta = 0 and no patch: the keys are the stored rows as they are, so the
    # result is plain attention over the store (checked against the oracle,
    # whose R(0) is the identity)
    o_lay, g_lay, canon, _, se, ids, _, q = make_case(2, 128, 90, 2, 1, 0, 8, [[0, 1]], 7)
    deltas = np.zeros(ids.size, np.int64)
    out, lse = run_gpu(g_lay, 0, canon, None, se, ids, deltas, q, 0.1)
    check(o_lay, 0, canon, None, se, ids, deltas, q, 0.1, out, lse, "zero shift")


def test_decode_attention_bad_chunk_id_is_flagged_and_skipped():
    # an entry whose chunk id is outside the store contributes nothing and
    # sets KAMERA_EW_CHUNK; the rest of the context is attended as usual
    o_lay, g_lay, canon, patch, se, ids, deltas, q = make_case(2, 128, 50, 3, 1, 16, 4, [[0, 1, 2]], 9)
    bad = ids.copy()
    bad[1] = 7
    ew = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, lse = run_gpu(g_lay, 0, canon, patch, se, bad, deltas, q, 0.09, error_word=ew)
    assert int(ew.item()) == 4
    keep = np.array([0, 2])
    check(o_lay, 0, canon, patch, np.array([0, 2], np.int32), ids[keep], deltas[keep], q, 0.09, out, lse,
          "bad chunk id skipped")


def test_decode_attention_matches_reuse_then_attend():
    # the fused path against the two-step path on the GPU: kamera_relocate_patch
    # writes the reconstructed cache (bfloat16) into a pool, then the same
    # attention reads the pool with delta = 0 and no patch.  The two differ by
    # the pool's bfloat16 rounding of every key and value (relative 2^-9), so
    # the bar here is looser: 4e-3 of max|V|.
    o_lay, g_lay, canon, patch, se, ids, deltas, q = make_case(2, 128, 128, 2, 1, 16, 8, [[1, 0]], 13,
                                                               delta_range=(-2000, 2000))
    n, T, F = ids.size, 128, 256
    src = [_dev(c) for c in canon]
    u = [_dev(x) for x in patch[0]]
    v = [_dev(x) for x in patch[1]]
    # the pool holds entry i at slots i*T .. i*T+T-1; as a store: chunk i, layer stride n*T*F
    pool = [torch.zeros((1, n * T, F), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    sel_src = [s[torch.from_numpy(ids.astype(np.int64)).cuda()].contiguous() for s in src]
    sel_u = [x[torch.from_numpy(ids.astype(np.int64)).cuda()].contiguous() for x in u]
    sel_v = [x[torch.from_numpy(ids.astype(np.int64)).cuda()].contiguous() for x in v]
    kam.relocate_patch(g_lay, sel_src, torch.from_numpy(deltas).cuda(), sel_u, sel_v, pool,
                       dst_offset=torch.arange(n, dtype=torch.int64, device="cuda") * T)
    pool_store = [p.view(1, n, T, F).permute(1, 0, 2, 3) for p in pool]
    B, Hq, D = q.shape
    out2 = torch.zeros((B, Hq, D), dtype=torch.float32, device="cuda")
    kam.decode_attention(g_lay, 0, pool_store, _dev(q), torch.from_numpy(se).cuda(),
                         torch.arange(n, dtype=torch.int32, device="cuda"),
                         torch.zeros(n, dtype=torch.int64, device="cuda"), out2, scale=0.088)
    out1, _ = run_gpu(g_lay, 0, canon, patch, se, ids, deltas, q, 0.088)
    torch.cuda.synchronize()
    _, V = ao.context_rows_f64(o_lay, 0, canon, patch, ids.tolist(), deltas.tolist())
    err = float(np.abs(out1 - out2.cpu().numpy()).max())
    assert err <= 4e-3 * float(np.abs(V).max()), err
    _say(f"fused vs reuse-then-attend: {err:.2e}")


def test_decode_attention_full_size_sampled():
    # the benchmark's decode workload (reorder shapes: 36 layers, 8 KV heads x
    # 128, 32 stored chunks of 2048 tokens, rank-32 patches, 32 query heads),
    # one layer, the whole 65,536-token context against the oracle
    from workloads import decode_by_name, make_decode_inputs

    dw = decode_by_name("decode_reorder_rank32")
    b = dw.base
    _say(f"full size: {dw}")
    inp = make_decode_inputs(dw, "cuda")
    g_lay = kam.Layout(b.num_layers, b.num_heads, b.head_dim, b.rope_offset, b.rope_dim, b.rope_base, 2,
                       b.rope_style)
    layer = 17
    B, Hq, D = inp["q"].shape[1:]
    out = torch.zeros((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.zeros((B, Hq), dtype=torch.float32, device="cuda")
    kam.decode_attention(g_lay, layer, inp["src"], inp["q"][layer], inp["seq_entries"], inp["chunk_ids"],
                         inp["delta"], out, scale=dw.scale, lse=lse, u=inp["u"], v=inp["v"])
    torch.cuda.synchronize()
    # oracle on one layer of the store (the only layer it reads)
    from workloads import bits
    canon = [bits(s[:, layer:layer + 1]) for s in inp["src"]]
    patch = ([bits(x[:, layer:layer + 1]) for x in inp["u"]], [bits(x[:, layer:layer + 1]) for x in inp["v"]])
    o1 = ko.Layout(1, b.num_heads, b.head_dim, b.rope_offset, b.rope_dim, b.rope_base, 2, b.rope_style)
    q = bits(inp["q"][layer])
    se = inp["seq_entries"].cpu().numpy()
    ids = inp["chunk_ids"].cpu().numpy()
    deltas = inp["delta"].cpu().numpy()
    worst = check(o1, 0, canon, patch, se, ids, deltas, q, dw.scale, out.cpu().numpy().astype(np.float64),
                  lse.cpu().numpy().astype(np.float64), "full size")
    _say(f"full size: worst output error {worst:.2e} of max|V|")
    del inp
    torch.cuda.empty_cache()


def test_decode_attention_mla_full_size_sampled():
    # the MLA decode workload (mla_reuse shapes: 27 layers, one 576-wide row,
    # 16 stored chunks of 4096 tokens, rank-32 patches, 16 query heads), one
    # layer, the whole 65,536-token context against the oracle
    from workloads import bits, decode_by_name, make_decode_inputs

    dw = decode_by_name("decode_mla_rank32")
    b = dw.base
    _say(f"full size MLA: {dw}")
    inp = make_decode_inputs(dw, "cuda")
    g_lay = kam.Layout(b.num_layers, b.num_heads, b.head_dim, b.rope_offset, b.rope_dim, b.rope_base, 1,
                       b.rope_style)
    layer = 9
    B, Hq, _ = inp["q"].shape[1:]
    out = torch.zeros((B, Hq, b.rope_offset), dtype=torch.float32, device="cuda")
    lse = torch.zeros((B, Hq), dtype=torch.float32, device="cuda")
    kam.decode_attention(g_lay, layer, inp["src"], inp["q"][layer], inp["seq_entries"], inp["chunk_ids"],
                         inp["delta"], out, scale=dw.scale, lse=lse, u=inp["u"], v=inp["v"])
    torch.cuda.synchronize()
    canon = [bits(s[:, layer:layer + 1]) for s in inp["src"]]
    patch = ([bits(x[:, layer:layer + 1]) for x in inp["u"]], [bits(x[:, layer:layer + 1]) for x in inp["v"]])
    o1 = ko.Layout(1, b.num_heads, b.head_dim, b.rope_offset, b.rope_dim, b.rope_base, 1, b.rope_style)
    worst = check(o1, 0, canon, patch, inp["seq_entries"].cpu().numpy(), inp["chunk_ids"].cpu().numpy(),
                  inp["delta"].cpu().numpy(), bits(inp["q"][layer]), dw.scale,
                  out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), "MLA full size")
    _say(f"MLA full size: worst output error {worst:.2e} of max|V|")
    del inp
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# Pooled tokens (kamera_decode_attention_paged): each sequence attends its
# reused entries and its own tokens in a paged pool
# --------------------------------------------------------------------------

def make_pool(rng, L, F, streams, n_seqs, max_pages, P, counts, slack_pages=3):
    """A pool [L][slots][F] per stream with distinct seeded pages per sequence."""
    num_pages = n_seqs * max_pages + slack_pages
    pool = [_bits(rng.standard_normal((L, num_pages * P, F))) for _ in range(streams)]
    table = rng.permutation(num_pages)[:n_seqs * max_pages].reshape(n_seqs, max_pages).astype(np.int32)
    return pool, table, np.asarray(counts, np.int32)


def run_gpu_paged(g_lay, layer, canon, patch, se, ids, deltas, q, scale, pool, table, counts, P, error_word=None):
    B, Hq, D = q.shape
    Dv = D if len(canon) == 2 else g_lay.rope_offset
    out = torch.full((B, Hq, Dv), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    u = v = None
    if patch is not None:
        u = [_dev(x) for x in patch[0]]
        v = [_dev(x) for x in patch[1]]
    kam.decode_attention(g_lay, layer, [_dev(c) for c in canon], _dev(q), torch.from_numpy(se).cuda(),
                         torch.from_numpy(ids).cuda(), torch.from_numpy(deltas).cuda(), out, scale=scale,
                         lse=lse, u=u, v=v, error_word=error_word, pool=[_dev(x) for x in pool],
                         block_table=torch.from_numpy(table).cuda(), pool_tokens=torch.from_numpy(counts).cuda(),
                         pool_page_size=P)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check_paged(o_lay, layer, canon, patch, se, ids, deltas, q, scale, pool, table, counts, P, out, lse, where):
    Hq = q.shape[1]
    ro, rl = ao.decode_attention_f64(o_lay, layer, canon, patch, se, ids.tolist(), deltas.tolist(),
                                     ko.bf16_bits_to_f64(q), Hq, scale, pool=(pool, P, table, counts))
    worst = 0.0
    for b in range(len(se) - 1):
        e0, e1 = int(se[b]), int(se[b + 1])
        K, V = ao.context_rows_f64(o_lay, layer, canon, patch, ids[e0:e1].tolist(), deltas[e0:e1].tolist())
        Kp, Vp = ao.pool_rows_f64(o_lay, layer, pool, P, table[b], counts[b])
        Vall = np.concatenate([V, Vp]) if V is not None else np.concatenate([K, Kp])[:, :ao.value_dim(o_lay)]
        if Vall.shape[0] == 0:
            assert np.all(out[b] == 0.0) and np.all(np.isneginf(lse[b])), f"{where}: sequence {b} must be empty"
            continue
        vmax = float(np.abs(Vall).max())
        err = float(np.abs(out[b] - ro[b]).max())
        assert err <= OUT_TOL * vmax, f"{where}: sequence {b} output off by {err:.3e} (max|V| {vmax:.2f})"
        lerr = float(np.abs(lse[b] - rl[b]).max())
        assert lerr <= LSE_TOL, f"{where}: sequence {b} lse off by {lerr:.3e}"
        worst = max(worst, err / vmax)
    return worst


PAGED_CASES = {
    # name: (H, D, T, n_store, L, m, Hq, contexts, page size, max pages, pooled tokens per sequence, extra)
    "gqa_g4_m16_entries_and_pool": (2, 128, 100, 3, 2, 16, 8, [[2, 0], [1]], 16, 6, [37, 96], {}),
    "gqa_d64_pool_only": (2, 64, 40, 1, 1, 0, 4, [[], [], []], 32, 5, [1, 160, 77], {}),
    "gqa_g8_d256_no_patch": (1, 256, 50, 2, 1, 0, 8, [[1, 0]], 16, 40, [600], {}),
    "gqa_mixed_empty": (2, 128, 33, 2, 1, 8, 4, [[0], [], [1, 0], []], 64, 3, [0, 0, 130, 192], {}),
    "mla_h16_m32_entries_and_pool": (1, 576, 150, 3, 2, 32, 16, [[2, 0], [1]], 64, 4, [200, 17],
                                     dict(rope_offset=512, rope_dim=64, base=1e4, streams=1,
                                          delta_range=(-32768, 32768))),
    "mla_h8_pool_only": (1, 576, 16, 1, 1, 0, 8, [[], []], 16, 9, [144, 45],
                         dict(rope_offset=512, rope_dim=64, base=1e4, streams=1)),
}


@pytest.mark.parametrize("name", sorted(PAGED_CASES))
def test_decode_attention_paged(name):
    H, D, T, ns, L, m, Hq, seqs, P, mp, counts, extra = PAGED_CASES[name]
    _say(f"{name}: H={H} D={D} T={T} m={m} Hq={Hq} contexts={seqs} P={P} pooled={counts}")
    o_lay, g_lay, canon, patch, se, ids, deltas, q = make_case(H, D, T, ns, L, m, Hq, seqs, 200 + len(name),
                                                               **extra)
    rng = np.random.default_rng(300 + len(name))
    pool, table, cnt = make_pool(rng, L, H * D, len(canon), len(seqs), mp, P, counts)
    layer = L - 1
    scale = 1.0 / np.sqrt(D)
    ew = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, lse = run_gpu_paged(g_lay, layer, canon, patch, se, ids, deltas, q, scale, pool, table, cnt, P,
                             error_word=ew)
    assert int(ew.item()) == 0
    worst = check_paged(o_lay, layer, canon, patch, se, ids, deltas, q, scale, pool, table, cnt, P, out, lse, name)
    _say(f"{name}: worst output error {worst:.2e} of max|V|")


def test_decode_attention_paged_without_pooled_tokens_equals_plain_call():
    o_lay, g_lay, canon, patch, se, ids, deltas, q = make_case(2, 128, 90, 3, 1, 16, 8, [[0, 2], [1]], 31)
    rng = np.random.default_rng(5)
    pool, table, cnt = make_pool(rng, 1, 256, 2, 2, 2, 16, [0, 0])
    out1, lse1 = run_gpu(g_lay, 0, canon, patch, se, ids, deltas, q, 0.1)
    out2, lse2 = run_gpu_paged(g_lay, 0, canon, patch, se, ids, deltas, q, 0.1, pool, table, cnt, 16)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def test_decode_attention_paged_bad_page_is_masked_and_flagged():
    # a page id outside the pool: its tokens drop out of the softmax and
    # KAMERA_EW_PAGE is set; the rest equals the oracle without those tokens
    o_lay, g_lay, canon, patch, se, ids, deltas, q = make_case(2, 128, 60, 2, 1, 16, 4, [[0], [1]], 41)
    rng = np.random.default_rng(6)
    P = 16
    pool, table, cnt = make_pool(rng, 1, 256, 2, 2, 4, P, [64, 50])
    bad = table.copy()
    bad[1, 3] = 1 << 20                      # sequence 1's last page (tokens 48..49)
    ew = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, lse = run_gpu_paged(g_lay, 0, canon, patch, se, ids, deltas, q, 0.09, pool, bad, cnt, P, error_word=ew)
    assert int(ew.item()) == kam.EW_PAGE
    keep = np.array([64, 48], np.int32)
    check_paged(o_lay, 0, canon, patch, se, ids, deltas, q, 0.09, pool, table, keep, P, out, lse, "bad page")


def test_decode_attention_paged_pool_written_by_relocate_patch():
    # the engine's flow end to end: kamera_relocate_patch writes two reused
    # chunks into a paged pool; attending them there (pooled tokens) must
    # equal the oracle over the pool's rows, and come within the pool's
    # bfloat16 rounding (4e-3 of max|V|) of attending them relocated on read
    o_lay, g_lay, canon, patch, se, ids, deltas, q = make_case(2, 128, 96, 2, 1, 16, 8, [[1, 0]], 17,
                                                               delta_range=(-3000, 3000))
    n, T, F, P = ids.size, 96, 256, 32
    ppc = T // P
    num_pages = n * ppc + 4
    rng = np.random.default_rng(8)
    pages = rng.permutation(num_pages)[:n * ppc].reshape(n, ppc).astype(np.int32)
    pool_t = [torch.zeros((1, num_pages * P, F), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    sel = torch.from_numpy(ids.astype(np.int64)).cuda()
    kam.relocate_patch(g_lay, [_dev(c)[sel].contiguous() for c in canon], torch.from_numpy(deltas).cuda(),
                       [_dev(x)[sel].contiguous() for x in patch[0]], [_dev(x)[sel].contiguous() for x in patch[1]],
                       pool_t, page_size=P, page_table=torch.from_numpy(pages).cuda())
    torch.cuda.synchronize()
    table = pages.reshape(1, n * ppc)        # one sequence: chunk 1's pages, then chunk 0's
    cnt = np.array([n * T], np.int32)
    pool_bits = [p.view(torch.int16).cpu().numpy().view(np.uint16) for p in pool_t]
    empty = np.array([0, 0], np.int32)
    out, lse = run_gpu_paged(g_lay, 0, canon, patch, empty, np.zeros(0, np.int32), np.zeros(0, np.int64), q, 0.088,
                             pool_bits, table, cnt, P)
    check_paged(o_lay, 0, canon, patch, empty, np.zeros(0, np.int32), np.zeros(0, np.int64), q, 0.088, pool_bits,
                table, cnt, P, out, lse, "pool from relocate_patch")
    out_fused, _ = run_gpu(g_lay, 0, canon, patch, se, ids, deltas, q, 0.088)
    _, V = ao.context_rows_f64(o_lay, 0, canon, patch, ids.tolist(), deltas.tolist())
    err = float(np.abs(out - out_fused).max())
    assert err <= 4e-3 * float(np.abs(V).max()), err
    _say(f"pooled vs relocated on read: {err:.2e}")
