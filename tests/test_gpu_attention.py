"""GPU parity of decode attention over a reused context (kamera_decode_attention)
against the CPU oracle (oracle/attention_oracle.py).

Inputs: seeded canonical stores, patch factors, queries and contexts drawn
here with NumPy (bfloat16 bits), the same bits given to both sides.

Bar (derived in the design doc): the GPU computes in fp32 with no bfloat16
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
