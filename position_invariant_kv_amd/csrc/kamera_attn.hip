// kamera_attn.hip — decode attention over a reused context, relocating on read
// (include/kamera.h, kamera_decode_attention).
//
// The reused keys and values are never written to a pool: each workgroup reads
// the canonical rows of its tile once and folds the reuse equation
// (Kamera summary, section 2) into the attention itself.
//
//   keys:   q . (R(delta) k + U_K[t] V_K^T) = (R(-delta) q) . k + U_K[t] . (V_K^T q)
//           R(delta) is orthogonal, so the chunk's one shift turns the query
//           once instead of every key, and the rank-m patch reduces to an
//           m-vector w = V_K^T q per query head and chunk.
//   values: sum_t p_t (v_t + U_V[t] V_V^T) = sum_t p_t v_t + V_V (sum_t p_t U_V[t])
//           so the value patch is an m-vector accumulated next to the output
//           and multiplied by V_V once per workgroup.
//
// Two launches per call:
//   attn_mfma_kernel: per (entry, token tile, KV head), the tile's partial
//     softmax (max, sum, unnormalised output per query head) on the matrix
//     cores (layout described at the kernel);
//   attn_combine_kernel: per (sequence, query head), the log-sum-exp merge of
//     the partials of every entry and tile of the sequence.

#include "kamera.h"
#include "kamera_common.h"

#include <stdlib.h>
#include <string.h>

namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kMaxRank = 64;
constexpr int kMfmaPass = 32;     // tile sizes are multiples of 4 waves x 32 tokens
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kEmpty = -1e30f;  // max of a partial with no token (finite: merges stay NaN-free)
constexpr int kMaxTilePages = kAttnWaves * kMfmaPass * 16 / 16 + 1;  // pages a token tile can touch

struct AttnParams {
    const uint16_t* k_rows;    // key stream of the store (chunk 0, layer 0)
    const uint16_t* v_rows;    // value stream
    int64_t chunk_stride, layer_stride;
    const uint16_t* uk;        // patch factors (NULL when m == 0)
    const uint16_t* vk;
    const uint16_t* uv;
    const uint16_t* vv;
    const int32_t* seq_entries;  // [B + 1]
    const int32_t* chunk_ids;    // [E]
    const int64_t* delta;        // [E]
    const uint16_t* q;           // [B][Hq][D]
    float* part_o;               // [Hq][units][D]: a head's partials are contiguous for the combine
    float2* part_ml;             // [Hq][units]: (max, sum), log2 domain
    uint32_t* error_word;
    double log2_base;
    float qscale;                // scale * log2(e)
    int32_t B, E, layer, L, T, n_store, Hkv, Hq, G, F, rope_offset, rope_dim, rope_style, m;
    int32_t tiles, tile_tokens;
    // The sequences' tokens in a paged pool (the kernels' POOL variants):
    // rows [L][slots][F] per stream, pool_layer_stride apart; sequence b's
    // t-th pooled token sits in slot pool_table[b][t / P] * P + t % P.
    const uint16_t* pool_k;
    const uint16_t* pool_v;
    int64_t pool_layer_stride;
    const int32_t* pool_table;   // [B][pool_max_pages]
    const int32_t* pool_tokens;  // [B]
    int32_t pool_page, pool_max_pages, pool_num_pages;
    int32_t pool_tiles;          // token tiles per sequence
    int32_t pool_tile_tokens;    // tokens per pool tile (the entries' tiles have tile_tokens)
    int64_t pool_unit0;          // partial index of sequence 0's first pool tile (E * tiles)
    int64_t units;               // partials per head: E * tiles + B * pool_tiles
};

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf_at(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ __bf16 bf_hi_part(float x) { return (__bf16)x; }
__device__ __forceinline__ __bf16 bf_lo_part(float x) { return (__bf16)(x - (float)(__bf16)x); }

// Sequence owning entry e: the largest b < B with seq_entries[b] <= e (the
// entries of a sequence are contiguous and the offsets non-decreasing).
__device__ __forceinline__ int seq_of_entry(const int32_t* se, int B, int e) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ld_uniform(se + mid) <= e) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Slot of pooled token t of sequence b (t < the sequence's pooled tokens), or
// -1 when its page id is outside the pool.  t is uniform over the wave.
__device__ __forceinline__ int64_t pool_slot(const AttnParams& p, int b, int t) {
    const int j = t / p.pool_page;
    const int page = ld_uniform(p.pool_table + (int64_t)b * p.pool_max_pages + j);
    if (page < 0 || page >= p.pool_num_pages) return -1;
    return (int64_t)page * p.pool_page + (t - j * p.pool_page);
}

// Pooled tokens of sequence b, clamped to its block-table row.
__device__ __forceinline__ int pool_count(const AttnParams& p, int b) {
    const int n = ld_uniform(p.pool_tokens + b);
    return min(max(n, 0), p.pool_max_pages * p.pool_page);
}

__device__ __forceinline__ void wave_lds_sync() {
    // LDS written by some lanes of a wave and read by others: compiler
    // barriers around a wave barrier (one wave's LDS operations complete in
    // order)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The transposing LDS read of 8 bytes per lane: within each 16-lane group,
// lane i receives element i % 4 of the 4 elements that lanes i / 4, 4 + i / 4,
// 8 + i / 4 and 12 + i / 4 of the group point at.  With lane (n, g) pointing
// at row 4 g + n / 4, columns 4 (n % 4) .. 4 (n % 4) + 3 of a row-major
// block, lane (n, g) receives column n of rows 4 g .. 4 g + 3: the B operand
// of a 16x16x16 product whose k runs down the rows.  The address must be
// 8-byte aligned.
__device__ __forceinline__ bf16x4 lds_read_tr16(const uint16_t* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const_cast<uint16_t*>(p)));
    return __builtin_bit_cast(bf16x4, r);
}

// ---------------------------------------------------------------------------
// attn_mfma_kernel: one workgroup (4 waves) per (entry, token tile, KV head)
// ---------------------------------------------------------------------------
//
// Per wave, tokens go in groups of 16:
//   S[t][h] = K[t][:] . q_rot[h][:]  on v_mfma_f32_16x16x32_bf16: A = the K rows
//             as stored (lane l: token l%16, 8 elements at 8(l/16) + 32s),
//             B = the turned, scaled query in bf16 high + low parts (16
//             query-head columns, zero past G; formed once and kept in LDS);
//             the key patch adds U_K[t][:] . w[h][:] the same way (A = U_K
//             rows, B = w hi + lo).
//   The output layout (lane l: tokens 4(l/16)+i of head l%16) is the A layout
//   of v_mfma_f32_16x16x16_bf16 with the heads as rows, so after the online
//   softmax the weights p feed the value product directly (hi + lo):
//   O[h][c] += P[h][t] Vx[t][c] over the value columns c (and the value
//   patch's U_V columns appended after them).  A group's value rows are
//   parked row-major in a per-wave LDS tile with 16-byte writes and read back
//   as B operands (4 consecutive tokens of one column) by the transposing LDS
//   read.
// A wave keeps two groups' loads in flight (one register set each; one set
// for rows of 256 or a patch of rank above 32): a group's rows are requested
// two groups ahead of their use.  Loads are unconditional -- rows past the wave's tokens re-read its
// last row (pooled: slot 0's), whose logits are masked -- since a load behind
// a branch makes the compiler wait for every load in flight at the join.  The
// first groups' loads go out before the operand set-up, whose work then hides
// their latency.
// The four waves' partials are merged in LDS, the value patch V_V u is added
// (u merged the same way), and the workgroup writes (max, sum, output) per
// query head.
// POOL: the workgroup reads sequence b's pooled tokens (tile `tile` of them)
// instead of an entry: keys and values as stored, no shift, no patch; its
// partial goes to unit pool_unit0 + blockIdx.x.
// NB: rank blocks of 16 the patch variant is built for (2: m <= 32, 4: m <= 64).
// Occupancy: two waves per SIMD up to D = 128; rows of 256 keep one.
// groups in flight per wave: two, one for rows of 256 or a patch of rank
// above 32 (the register budget of two waves per SIMD)
template <int D, bool PATCH, int NB>
constexpr int attn_sets() { return D > 128 || (PATCH && NB > 2) ? 1 : 2; }
template <int D, bool PATCH, int NB>
constexpr int attn_cols() { return D + (PATCH ? 16 * NB : 0); }
// LDS of a workgroup: the query's (and w's) operands, then a general area --
// the operand staging during the set-up, the value tiles during the token
// loop -- and the merge after the loop (over everything: the operands are
// dead by then).
template <int D, bool PATCH, int NB>
constexpr int attn_op_bytes() { return (D / 32) * 2 * 64 * 16 + (PATCH ? ((16 * NB + 31) / 32) * 2 * 64 * 16 : 0); }
template <int D, bool PATCH, int NB>
constexpr int attn_lds_bytes() {
    constexpr int COLS = attn_cols<D, PATCH, NB>();
    constexpr int TILES = kAttnWaves * attn_sets<D, PATCH, NB>() * 16 * (COLS + 8) * 2;
    constexpr int STAGE = 16 * D * 4 + (PATCH ? 16 * kMaxRank * 4 + 16 * D * 2 + D * kMaxRank * 2 : 0);
    constexpr int RED = kAttnWaves * 16 * COLS * 4;
    constexpr int A = attn_op_bytes<D, PATCH, NB>() + (TILES > STAGE ? TILES : STAGE);
    return A > RED ? A : RED;
}

constexpr int cmax(int a, int b) { return a > b ? a : b; }
// The LDS of one workgroup, sized for every variant a kernel may run (the
// entries' path with 32 or 64 patch columns -- the variants keep different
// numbers of groups in flight -- and the plain or pooled tokens' path).
template <int D>
struct AttnShared {
    static constexpr int kBytes = cmax(cmax(attn_lds_bytes<D, true, 2>(), attn_lds_bytes<D, true, 4>()),
                                       attn_lds_bytes<D, false, 2>());
    __attribute__((aligned(16))) uint8_t lds[kBytes];
    float red_m[kAttnWaves][16];
    float red_l[kAttnWaves][16];
    float um[16][kMaxRank];
};

template <int D, bool PATCH, bool POOL, int NB>
__device__ __forceinline__ void attn_tile(const AttnParams& p, const int unit, const int g, AttnShared<D>& sh) {
    static_assert(!(POOL && PATCH), "pooled tokens carry no patch");
    constexpr int KS = D / 32;                    // k-steps of the key product
    constexpr int MP = PATCH ? 16 * NB : 0;       // value-patch columns (at most)
    constexpr int COLS = D + MP;                  // columns of the value tile
    constexpr int VP = COLS + 8;                  // its LDS row pitch (elements)
    constexpr int VC = D / 16;                    // value chunks of 16 columns
    constexpr int UCM = MP / 16;                  // value-patch chunks
    constexpr int KR = PATCH ? (MP + 31) / 32 : 1;  // key-patch k-steps of 32 ranks
    constexpr int CSEG = COLS / 8;                // 16-byte segments of a value row
    constexpr int NVL = (16 * CSEG + 63) / 64;    // of a group's value rows, per lane
    constexpr int NSET = attn_sets<D, PATCH, NB>();  // groups in flight per wave
    constexpr int TILE = 16 * VP;                 // elements of a group's value tile
    uint8_t* lds = sh.lds;
    u32x4* qop = reinterpret_cast<u32x4*>(lds);   // [KS][2][64]: turned query, hi and lo
    u32x4* wop = qop + KS * 2 * 64;               // [KR][2][64]: w, hi and lo (patch)
    uint8_t* area = lds + attn_op_bytes<D, PATCH, NB>();
    auto& red_m = sh.red_m;
    auto& red_l = sh.red_l;
    auto& um = sh.um;

    const int tiles_of = POOL ? p.pool_tiles : p.tiles;
    const int e = unit / tiles_of;              // POOL: the sequence
    const int tile = unit - e * tiles_of;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: its branches are scalar
    const int n16 = lane & 15, q4 = lane >> 4;
    const int G = p.G;
    const int cid = POOL ? 0 : ld_uniform(p.chunk_ids + e);
    // partial of local head h: row (g * G + h) * units + this unit
    const int64_t pidx = (int64_t)g * G * p.units + (POOL ? p.pool_unit0 + unit : unit);
    if (!POOL && !(cid >= 0 && cid < p.n_store)) {  // uniform: this entry contributes nothing
        for (int i = tid; i < G * D; i += kAttnThreads) p.part_o[(pidx + (i / D) * p.units) * D + i % D] = 0.0f;
        if (tid < G) p.part_ml[pidx + tid * p.units] = make_float2(kEmpty, 0.0f);
        if (tid == 0 && p.error_word && tile == 0) atomicOr(p.error_word, (uint32_t)KAMERA_EW_CHUNK);
        return;
    }
    const int m = PATCH ? p.m : 0;
    const int64_t blk = (int64_t)cid * p.L + p.layer;

    // ---- this wave's tokens
    const int tile_tokens = POOL ? p.pool_tile_tokens : p.tile_tokens;
    const int per_wave = tile_tokens / kAttnWaves;
    const int wt0 = tile * tile_tokens + wave * per_wave;
    const int wt1 = min(POOL ? pool_count(p, e) : p.T, wt0 + per_wave);
    const uint16_t* kb = POOL ? p.pool_k + p.layer * p.pool_layer_stride + (int64_t)g * D
                              : p.k_rows + cid * p.chunk_stride + p.layer * p.layer_stride + (int64_t)g * D;
    const uint16_t* vb = POOL ? p.pool_v + p.layer * p.pool_layer_stride + (int64_t)g * D
                              : p.v_rows + cid * p.chunk_stride + p.layer * p.layer_stride + (int64_t)g * D;
    const uint16_t* ukb = PATCH ? p.uk + blk * p.T * m : nullptr;
    const uint16_t* uvb = PATCH ? p.uv + blk * p.T * m : nullptr;
    uint16_t* tiles = reinterpret_cast<uint16_t*>(area) + wave * NSET * TILE;
    const int mcols = PATCH ? (m + 15) & ~15 : 0;     // patch columns padded to chunks of 16
    const u32x4 zero = {0u, 0u, 0u, 0u};

    // POOL: the wave's page ids, one per lane (a wave's tokens span at most 32
    // pages: pages hold a multiple of 16 tokens and a wave at most 512); a
    // group's page is then a lane read, not a load in its address path.  -1:
    // a page id outside the pool.
    int pg_lane = -1, pg0 = 0;
    if (POOL) {
        pg0 = wt0 / p.pool_page;
        const int page = p.pool_table[(int64_t)e * p.pool_max_pages + min(pg0 + lane, p.pool_max_pages - 1)];
        pg_lane = page >= 0 && page < p.pool_num_pages ? page : -1;
    }
    // slot of pooled token t (t < wt1) of this wave, -1 outside the pool
    auto tile_slot = [&](int t) -> int64_t {
        const int jp = t / p.pool_page;
        const int page = __builtin_amdgcn_readlane(pg_lane, jp - pg0);
        return page < 0 ? -1 : (int64_t)page * p.pool_page + (t - jp * p.pool_page);
    };
    // A lane's value segments of a group: row vrow, column vcol (past D: the
    // U_V column vcol - D), fixed per lane.
    int vrow[NVL], vcol[NVL];
#pragma unroll
    for (int j = 0; j < NVL; ++j) {
        const int sg = min(lane + 64 * j, 16 * CSEG - 1);
        vrow[j] = sg / CSEG;
        vcol[j] = 8 * (sg % CSEG);
    }
    // one group's loads (tokens tg .. tg + 15): K rows as key-product
    // operands, U_K rows likewise, and the value (and U_V) rows as segments
    auto load_group = [&](int tg, u32x4 (&ka)[KS], u32x4 (&ua)[KR], u32x4 (&vr)[NVL]) {
        // pooled tokens: the group of 16 lies in one page (P % 16 == 0); a
        // page outside the pool, or a group past the end, reads slot 0
        const int tb = min(tg, wt1 - 1);  // tokens tb .. tb + lim exist
        int lim = wt1 - 1 - tb;
        int64_t row0 = tb;                // the row of token tb in kb and vb
        if (POOL) {
            const int64_t slot = tg < wt1 ? tile_slot(tg) : -1;
            row0 = slot >= 0 ? slot : 0;
            if (slot < 0) lim = 0;
        }
        const int rk = min(n16, lim);
        const uint16_t* krow = kb + (row0 + rk) * (int64_t)p.F + 8 * q4;
#pragma unroll
        for (int s = 0; s < KS; ++s) ka[s] = ld_cached(krow + 32 * s);
        if (PATCH) {
            const uint16_t* urow = ukb + (int64_t)(tb + rk) * m;
#pragma unroll
            for (int s = 0; s < KR; ++s) ua[s] = ld_cached(urow + min(32 * s + 8 * q4, m - 8));
        }
#pragma unroll
        for (int j = 0; j < NVL; ++j) {
            const int r = min(vrow[j], lim);
            const uint16_t* av = vb + (row0 + r) * (int64_t)p.F + vcol[j];
            if (PATCH) {
                const uint16_t* au = uvb + (int64_t)(tb + r) * m + min(vcol[j] - D, m - 8);
                vr[j] = ld_cached(vcol[j] < D ? av : au);
            } else {
                vr[j] = ld_cached(av);
            }
        }
    };

    // ---- operands of (entry, KV head).  Query head n (n < 16, zero past G):
    // q_rot = R(-delta) q (for a key pair (a, b) the rotation by delta is
    // a' = a c - b s, b' = b c + a s, so q . R(delta) k =
    // (q_a c + q_b s) a + (q_b c - q_a s) b) and w[k] = sum_d V_K[d][k] q[d]
    // with the unturned q (the patch sits in the destination frame), both
    // scaled by scale * log2(e), staged in LDS (the general area, not yet in
    // use) and split into bf16 high and low parts, kept in LDS as the lanes'
    // B operands: 8 values of head l % 16 at 32 s + 8 (l / 16).
    float* qs = reinterpret_cast<float*>(area);        // [16][D] turned, scaled
    float* wsh = qs + 16 * D;                          // [16][64] (patch only)
    uint16_t* qraw = reinterpret_cast<uint16_t*>(wsh + (PATCH ? 16 * kMaxRank : 0));  // [16][D] as given
    uint16_t* vks = qraw + (PATCH ? 16 * D : 0);       // [D][m]
    const int b = POOL ? e : seq_of_entry(p.seq_entries, p.B, e);
    const int64_t delta = POOL ? 0 : ld_uniform(p.delta + e);  // R(0) = I exactly
    const uint16_t* qb = p.q + ((int64_t)b * p.Hq + (int64_t)g * G) * D;
    // this thread's items i = tid + 256 r share column d = tid % D (256 is a
    // multiple of D), so the turn's cos/sin is evaluated once
    static_assert(kAttnThreads % D == 0, "one column per thread");
    const int d = tid % D, dd = d - p.rope_offset;
    const bool turned = dd >= 0 && dd < p.rope_dim;
    int jj = 0, partner = d;
    float sg = 0.0f;
    if (turned) {
        if (p.rope_style == KAMERA_ROPE_HALF) {
            const int half = p.rope_dim >> 1;
            const bool first = dd < half;
            jj = first ? dd : dd - half;
            partner = first ? d + half : d - half;
            sg = first ? 1.0f : -1.0f;
        } else {
            jj = dd >> 1;
            partner = d ^ 1;
            sg = (dd & 1) ? -1.0f : 1.0f;
        }
    }
    // the set-up's loads first (heads clamped to G - 1 and zeroed at use;
    // V_K's segments clamped to its last), then the first groups' loads: loads
    // complete in issue order, so the waits for the set-up's loads do not wait
    // for the groups'
    constexpr int NQ = 16 * D / kAttnThreads;          // items per thread
    constexpr int NV = D * kMaxRank / 8 / kAttnThreads;  // V_K segments per thread (at most)
    uint16_t qx[NQ], qp[NQ];
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
        const uint16_t* qh = qb + min((tid + kAttnThreads * r) / D, G - 1) * D;
        qx[r] = qh[d];
        qp[r] = qh[partner];
    }
    u32x4 vkl[PATCH ? NV : 1];
    if (PATCH) {
        const uint16_t* vkh = p.vk + (blk * p.F + (int64_t)g * D) * m;
#pragma unroll
        for (int j = 0; j < NV; ++j) vkl[j] = ld_cached(vkh + 8 * min(tid + kAttnThreads * j, D * m / 8 - 1));
    }
    u32x4 ka0[KS], ua0[KR], vr0[NVL], ka1[NSET > 1 ? KS : 1], ua1[KR], vr1[NSET > 1 ? NVL : 1];
    load_group(wt0, ka0, ua0, vr0);
    if constexpr (NSET > 1) load_group(wt0 + 16, ka1, ua1, vr1);
    // keep the scheduler from moving the uses below (and their waits) above
    // the loads
    __builtin_amdgcn_sched_barrier(0);
    {
        const float2 cs = turned ? rope_cos_sin(p.log2_base, p.rope_dim, jj, delta) : make_float2(1.0f, 0.0f);
#pragma unroll
        for (int r = 0; r < NQ; ++r) {
            const int i = tid + kAttnThreads * r, h = i / D;
            float x = __uint_as_float((uint32_t)qx[r] << 16);
            if (turned) x = fmaf(x, cs.x, sg * __uint_as_float((uint32_t)qp[r] << 16) * cs.y);
            qs[i] = h < G ? x * p.qscale : 0.0f;
            if (PATCH) qraw[i] = h < G ? qx[r] : (uint16_t)0;
        }
        if (PATCH) {
#pragma unroll
            for (int j = 0; j < NV; ++j)
                if (tid + kAttnThreads * j < D * m / 8) *reinterpret_cast<u32x4*>(vks + 8 * (tid + kAttnThreads * j)) = vkl[j];
        }
        __syncthreads();
        if (PATCH) {
            // w[h][k] = qscale sum_d q[h][d] V_K[d][k] on the matrix cores
            // (16x16x16: A = the query as given, 4 columns per lane; B = 4
            // rows of V_K's column k by the transposing LDS read).  Wave w
            // takes rank block w (m <= 64: at most 4 blocks of 16).
            if (16 * wave < m) {
                f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
                // lane (n16, q4): rows 16 s + 4 q4 + n16 / 4, columns 16 wave + 4 (n16 % 4) ..
                const int vrw = 4 * q4 + (n16 >> 2);
                const int vcl = min(16 * wave + 4 * (n16 & 3), m - 4);
#pragma unroll
                for (int s = 0; s < D / 16; ++s) {
                    const bf16x4 a = __builtin_bit_cast(bf16x4,
                        *reinterpret_cast<const uint2*>(qraw + n16 * D + 16 * s + 4 * q4));
                    const bf16x4 bv = lds_read_tr16(vks + (16 * s + vrw) * m + vcl);
                    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bv, c, 0, 0, 0);
                }
                // lane (n16, q4) holds C[4 q4 + i][16 wave + n16]
                const int k = 16 * wave + n16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int h = 4 * q4 + i;
                    wsh[h * kMaxRank + k] = h < G && k < m ? c[i] * p.qscale : 0.0f;
                }
            } else {
                // rank blocks past m: zeros (heads past G are zero above)
#pragma unroll
                for (int i = 0; i < 4; ++i) wsh[(4 * q4 + i) * kMaxRank + 16 * wave + n16] = 0.0f;
            }
            __syncthreads();
        }
        // the lanes' B operands, hi and lo, into LDS for the token loop
        for (int idx = tid; idx < KS * 64; idx += kAttnThreads) {
            const int s = idx / 64, l = idx % 64;
            bf16x8 hi, lo;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = qs[(l & 15) * D + 32 * s + 8 * (l >> 4) + j];
                hi[j] = bf_hi_part(x);
                lo[j] = bf_lo_part(x);
            }
            qop[(2 * s) * 64 + l] = __builtin_bit_cast(u32x4, hi);
            qop[(2 * s + 1) * 64 + l] = __builtin_bit_cast(u32x4, lo);
        }
        if (PATCH) {
            for (int idx = tid; idx < KR * 64; idx += kAttnThreads) {
                const int s = idx / 64, l = idx % 64;
                bf16x8 hi, lo;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float x = wsh[(l & 15) * kMaxRank + 32 * s + 8 * (l >> 4) + j];
                    hi[j] = bf_hi_part(x);
                    lo[j] = bf_lo_part(x);
                }
                wop[(2 * s) * 64 + l] = __builtin_bit_cast(u32x4, hi);
                wop[(2 * s + 1) * 64 + l] = __builtin_bit_cast(u32x4, lo);
            }
        }
        __syncthreads();  // operands ready; the staging area is free for the tiles
    }

    f32x4 acc[VC + UCM];
#pragma unroll
    for (int c = 0; c < VC + UCM; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float mrun = kEmpty, lrun = 0.0f;  // of head n16
    // value operands: lane (n16, q4) names row 4 q4 + n16 / 4, columns
    // 4 (n16 % 4) .. of a 16-column chunk
    const int vta = (4 * q4 + (n16 >> 2)) * VP + 4 * (n16 & 3);
    auto process = [&](int tg, u32x4 (&ka)[KS], u32x4 (&ua)[KR], u32x4 (&vr)[NVL], uint16_t* tb_, const bool prefetch) {
        // the value rows to this wave's tile, as loaded (a row past the end
        // holds an in-range row's finite values; its weight is exactly 0)
#pragma unroll
        for (int j = 0; j < NVL; ++j)
            if (lane + 64 * j < 16 * CSEG) *reinterpret_cast<u32x4*>(tb_ + vrow[j] * VP + vcol[j]) = vr[j];
        // logits (log2 units): tokens 4 q4 + i of head n16
        f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, ka[s]);
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, qop[(2 * s) * 64 + lane]), c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, qop[(2 * s + 1) * 64 + lane]), c, 0, 0, 0);
        }
        if (PATCH) {
#pragma unroll
            for (int s = 0; s < KR; ++s) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, ua[s]);
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, wop[(2 * s) * 64 + lane]), c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, wop[(2 * s + 1) * 64 + lane]), c, 0, 0, 0);
            }
        }
        if (prefetch) load_group(tg + 16 * NSET, ka, ua, vr);  // these registers are free again (a constant at each call)
        if (POOL || tg + 16 > wt1) {  // uniform: a group with masked tokens
            bool gbad = false;  // pooled tokens of a page outside the pool: masked
            if (POOL) {
                gbad = tg < wt1 && tile_slot(tg) < 0;
                if (gbad && lane == 0 && p.error_word) atomicOr(p.error_word, (uint32_t)KAMERA_EW_PAGE);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (tg + 4 * q4 + i >= wt1 || gbad) c[i] = -INFINITY;
        }
        // online softmax of head n16 (the group has at least one valid
        // token); exp2 of a logit below the maximum by more than 126 flushes
        // to zero
        float mx = fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(mrun, mx);
        const float alpha = __builtin_amdgcn_exp2f(mrun - mn);
        mrun = mn;
        bf16x4 phi, plo;
        float psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float pp = __builtin_amdgcn_exp2f(c[i] - mn);
            psum += pp;
            phi[i] = bf_hi_part(pp);
            plo[i] = bf_lo_part(pp);
        }
        lrun = fmaf(lrun, alpha, psum);
        // rescale the output rows (heads 4 q4 + i) by their heads' alpha; once
        // the running maxima settle, alpha is exactly 1 for every head and the
        // rescale (an exact no-op then) is skipped on a wave-uniform branch
        if (__any(alpha != 1.0f)) {
            float ar[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * q4 + i);
#pragma unroll
            for (int cc = 0; cc < VC + UCM; ++cc)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[cc][i] *= ar[i];
        }
        wave_lds_sync();  // the parked tile is visible to the whole wave
        // values: O[h][col] += P[h][t] Vx[t][col]
#pragma unroll
        for (int cc = 0; cc < VC + UCM; ++cc) {
            if (cc >= VC && 16 * (cc - VC) >= mcols) break;
            const bf16x4 bv = lds_read_tr16(tb_ + vta + 16 * cc);
            acc[cc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, bv, acc[cc], 0, 0, 0);
            acc[cc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, bv, acc[cc], 0, 0, 0);
        }
        wave_lds_sync();  // the tile's reads are done before it is rewritten
    };
    // every pass but the last requests the groups after it; the last requests
    // nothing (loads past the wave's tokens would only be waited for)
    int tg = wt0;
    if constexpr (NSET > 1) {
        for (; tg + 32 < wt1; tg += 32) {  // uniform over the wave
            process(tg, ka0, ua0, vr0, tiles, true);
            process(tg + 16, ka1, ua1, vr1, tiles + TILE, true);
        }
        if (tg < wt1) {
            process(tg, ka0, ua0, vr0, tiles, false);
            if (tg + 16 < wt1) process(tg + 16, ka1, ua1, vr1, tiles + TILE, false);
        }
    } else {
        for (; tg + 16 < wt1; tg += 16) process(tg, ka0, ua0, vr0, tiles, true);
        if (tg < wt1) process(tg, ka0, ua0, vr0, tiles, false);
    }
    // ---- sums of head n16 over the wave; then the workgroup's merge
    lrun += __shfl_xor(lrun, 16);
    lrun += __shfl_xor(lrun, 32);
    // the value patch's row d of V_V (this thread's outputs are column d of
    // several heads), requested before the merge so that its latency hides
    // behind it; clamped to the rank, skipped at use
    u32x4 xr[PATCH ? MP / 8 : 1];
    if (PATCH) {
        const uint16_t* vrow = p.vv + (blk * p.F + (int64_t)g * D + d) * m;
#pragma unroll
        for (int kk = 0; kk < MP / 8; ++kk) xr[kk] = ld_cached(vrow + min(8 * kk, m - 8));
    }
    __syncthreads();  // every wave is done with its tiles
    float* red = reinterpret_cast<float*>(lds);  // [wave][16][COLS]
#pragma unroll
    for (int c = 0; c < VC + UCM; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[(wave * 16 + 4 * q4 + i) * COLS + 16 * c + n16] = acc[c][i];
    if (q4 == 0) {
        red_m[wave][n16] = mrun;
        red_l[wave][n16] = lrun;
    }
    __syncthreads();
    if (PATCH) {
        for (int i = tid; i < G * m; i += kAttnThreads) {
            const int h = i / m, k = i % m;
            float M = red_m[0][h];
#pragma unroll
            for (int w = 1; w < kAttnWaves; ++w) M = fmaxf(M, red_m[w][h]);
            float a = 0.0f;
#pragma unroll
            for (int w = 0; w < kAttnWaves; ++w) a = fmaf(red[(w * 16 + h) * COLS + D + k], __builtin_amdgcn_exp2f(red_m[w][h] - M), a);
            um[h][k] = a;
        }
        __syncthreads();
    }
    for (int h = tid / D; h < G; h += kAttnThreads / D) {
        float M = red_m[0][h];
#pragma unroll
        for (int w = 1; w < kAttnWaves; ++w) M = fmaxf(M, red_m[w][h]);
        float a = 0.0f, lsum = 0.0f;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) {
            const float f = __builtin_amdgcn_exp2f(red_m[w][h] - M);  // 1 for every wave when the tile is empty (all 0)
            a = fmaf(red[(w * 16 + h) * COLS + d], f, a);
            lsum = fmaf(red_l[w][h], f, lsum);
        }
        if (PATCH) {
#pragma unroll
            for (int kk = 0; kk < MP / 8; ++kk) {
                if (8 * kk >= m) break;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    a = fmaf(bf_lo(xr[kk][w]), um[h][8 * kk + 2 * w], a);
                    a = fmaf(bf_hi(xr[kk][w]), um[h][8 * kk + 2 * w + 1], a);
                }
            }
        }
        p.part_o[(pidx + h * p.units) * D + d] = a;
        if (d == 0) p.part_ml[pidx + h * p.units] = make_float2(M, lsum);
    }
}

template <int D, bool PATCH, bool POOL = false, int NB = 2>
__global__ __launch_bounds__(kAttnThreads, D <= 128 ? 2 : 1) void attn_mfma_kernel(const AttnParams p) {
    __shared__ AttnShared<D> sh;
    attn_tile<D, PATCH, POOL, NB>(p, (int)blockIdx.x, (int)blockIdx.y, sh);
}

// A reused context and pooled tokens in one launch: x in [0, pool_unit0)
// takes the entries' tiles, the rest the pooled tokens' tiles (y = KV head).
template <int D, bool PATCH, int NB = 2>
__global__ __launch_bounds__(kAttnThreads, D <= 128 ? 2 : 1) void attn_mfma_mixed_kernel(const AttnParams p) {
    __shared__ AttnShared<D> sh;
    const int64_t u = blockIdx.x;
    if (u < p.pool_unit0)
        attn_tile<D, PATCH, false, NB>(p, (int)u, (int)blockIdx.y, sh);
    else
        attn_tile<D, false, true, 2>(p, (int)(u - p.pool_unit0), (int)blockIdx.y, sh);
}

// ---------------------------------------------------------------------------
// MLA: one joint row per token [c_KV (512) | k_rope (64)], read by every query
// head: the key is the whole row, the value its c_KV part (the caller's
// queries are the absorbed ones, 576 wide).  Only the 64 k_rope dimensions
// carry RoPE, so only the query's last 64 dimensions turn: its first 512 go
// into the key product exactly as given (bf16, unscaled; the scale is applied
// to the logits) and only the turned part is split into high + low halves.
// ---------------------------------------------------------------------------
constexpr int kMlaDK = 576;
constexpr int kMlaDV = 512;

// One workgroup (4 waves) per (entry, token tile); the waves share every
// 16-token group.  The set-up forms the query operands and, with a patch, the
// key patch's weights w = V^T q on the matrix cores (one launch per call:
// no separate kernel for w).  A group's rows (and U's) are loaded once,
// coalesced, two groups ahead into one of two register sets, and parked in
// one of two LDS buffers.  The key product's 18 k-steps are dealt to the
// waves -- the query's 16 c_KV steps round-robin (as given, staged in LDS),
// then one step of each wave's own: its turned k_rope part hi + lo on waves
// 0 and 1, the key patch U w on waves 2 and 3 -- and the four partial logit
// tiles are added in LDS, in a fixed order, so every wave holds the same
// logits and the same softmax.  Each wave then accumulates its own 128 value
// columns (and one 16-column chunk of u = sum_t p_t U[t]) with the value
// operands read transposed from the same LDS rows: no cross-wave merge is
// needed.  At the end the value patch V_c u is one more matrix product per
// wave.
// POOL: as in attn_mfma_kernel, the workgroup reads a sequence's pooled tokens.
constexpr int kMlaKN = kMlaDV / 32;                 // 16 k-steps on c_KV
constexpr int kMlaKP = kMlaDK + 8;                  // LDS row pitch of a group's rows (elements)
constexpr int kMlaUP = kMaxRank + 8;                // ... of U's rows

// The LDS of one MLA workgroup, shared by the entries' and the pooled
// tokens' paths of the one-launch kernel below.
constexpr int kMlaThreads = 512;                    // two teams of four waves
constexpr int kMlaWaves = kMlaThreads / 64;
constexpr int kMlaTW = 4;                           // waves per team
constexpr int kMlaTT = 64 * kMlaTW;                 // threads per team
struct MlaShared {
    u32x4 qn[kMlaKN][64];                           // c_KV operands of the query, lane layout
    float qr[16][64];                               // turned k_rope part of the query
    __attribute__((aligned(16))) uint16_t kbuf[2][2][16 * kMlaKP];  // [team][buffer]: groups' rows
    __attribute__((aligned(16))) uint16_t ubuf[2][2][16 * kMlaUP];
    f32x4 spart[2][kMlaTW][64];                     // [team][team wave]: partial logits
    float um[16][kMaxRank];
    float uv[16][kMaxRank];                         // u = sum_t p_t U[t] per head (value patch)
    float tm[16], tl[16];                           // team 1's running max and sum per head
};
// the partial, row-major in a tile's group buffers at the end: rows padded
// so that the accumulator layout's writes hit distinct banks
constexpr int kMlaStgPitch = kMlaDV + 4;
static_assert(16 * kMlaStgPitch * 4 <= 2 * 16 * kMlaKP * 2, "the staged partial fits a team's group buffers");

// 8 x 8 transpose of 16-bit elements within each aligned octet of lanes:
// lane r of the octet holds row r on entry (element 2 i in the low half of
// dword i) and column r on exit.  Three exchanges, between lanes 4, 2 and 1
// apart: the first swaps the off-diagonal 4 x 4 blocks, the second the
// off-diagonal 2 x 2 blocks of each, the third transposes each 2 x 2 block.
__device__ __forceinline__ u32x4 transpose8x8_b16(u32x4 x, int lane) {
    const bool b2 = lane & 4, b1 = lane & 2, b0 = lane & 1;
    {
        const uint32_t r0 = __shfl_xor((int)(b2 ? x[0] : x[2]), 4);
        const uint32_t r1 = __shfl_xor((int)(b2 ? x[1] : x[3]), 4);
        if (b2) { x[0] = r0; x[1] = r1; } else { x[2] = r0; x[3] = r1; }
    }
#pragma unroll
    for (int lo = 0; lo < 4; lo += 2) {
        const uint32_t r = __shfl_xor((int)(b1 ? x[lo] : x[lo + 1]), 2);
        if (b1) x[lo] = r; else x[lo + 1] = r;
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t r = __shfl_xor((int)x[d], 1);
        x[d] = b0 ? __builtin_amdgcn_perm(x[d], r, 0x07060302u) : __builtin_amdgcn_perm(r, x[d], 0x05040100u);
    }
    return x;
}

// NB: rank blocks of 16 the kernel is built for (2: m <= 32, 4: m <= 64).
template <bool PATCH, bool POOL, int NB>
__device__ __forceinline__ void mla_tile(const AttnParams& p, const int unit, MlaShared& sh) {
    static_assert(!(POOL && PATCH), "pooled tokens carry no patch");
    constexpr int KS = kMlaDK / 32;               // 18
    constexpr int KN = kMlaKN;
    constexpr int KP = kMlaKP;
    constexpr int UP = kMlaUP;
    constexpr int VCW = kMlaDV / kMlaTW / 16;     // value chunks per wave (8)
    constexpr int SEGS = 16 * kMlaDK / 8;         // 16-byte segments of a group's rows (1152)
    constexpr int NLD = (SEGS + kMlaTT - 1) / kMlaTT;  // per thread of a team (5)
    auto& qn = sh.qn;
    auto& qr = sh.qr;
    auto& kbuf = sh.kbuf;
    auto& ubuf = sh.ubuf;
    auto& spart = sh.spart;
    auto& um = sh.um;

    const int tiles_of = POOL ? p.pool_tiles : p.tiles;
    const int e = unit / tiles_of;              // POOL: the sequence
    const int tile = unit - e * tiles_of;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: its branches are scalar
    const int team = wave / kMlaTW, tw = wave % kMlaTW, ttid = tid % kMlaTT;
    const int n16 = lane & 15, q4 = lane >> 4;
    const int G = p.G;
    const int cid = POOL ? 0 : ld_uniform(p.chunk_ids + e);
    // partial of head h: row h * units + this unit
    const int64_t pidx = POOL ? p.pool_unit0 + unit : unit;
    if (!POOL && !(cid >= 0 && cid < p.n_store)) {  // uniform: this entry contributes nothing
        for (int i = tid; i < G * kMlaDV; i += kMlaThreads)
            p.part_o[(pidx + (i / kMlaDV) * p.units) * kMlaDV + i % kMlaDV] = 0.0f;
        if (tid < G) p.part_ml[pidx + tid * p.units] = make_float2(kEmpty, 0.0f);
        if (tid == 0 && p.error_word && tile == 0) atomicOr(p.error_word, (uint32_t)KAMERA_EW_CHUNK);
        return;
    }
    const int m = PATCH ? p.m : 0;
    const int64_t blk = (int64_t)cid * p.L + p.layer;

    // ---- the tile's tokens, 16 at a time.  The first two groups' loads are
    // issued before the query set-up below (with a patch: once w's products
    // have V's rows), whose work then hides their latency.
    const int tile_tokens = POOL ? p.pool_tile_tokens : p.tile_tokens;
    const int t_begin = tile * tile_tokens;
    const int t_end = min(POOL ? pool_count(p, e) : p.T, t_begin + tile_tokens);
    const uint16_t* kb = POOL ? p.pool_k + p.layer * p.pool_layer_stride
                              : p.k_rows + cid * p.chunk_stride + p.layer * p.layer_stride;
    const uint16_t* ub = PATCH ? p.uk + blk * p.T * m : nullptr;
    const int mcols = PATCH ? (m + 15) & ~15 : 0;
    const bool uwave = PATCH && 16 * tw < mcols;     // this wave accumulates u columns 16 tw ..
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // POOL: the tile's page ids, one per lane (a tile spans at most 64 pages:
    // pages hold a multiple of 16 tokens and tiles at most 1024), loaded
    // first; a group's page is then a lane read, not a load in the group's
    // address path.  -1: a page id outside the pool.
    int pg_lane = -1, pg0 = 0;
    if (POOL) {
        pg0 = t_begin / p.pool_page;
        const int page = p.pool_table[(int64_t)e * p.pool_max_pages + min(pg0 + lane, p.pool_max_pages - 1)];
        pg_lane = page >= 0 && page < p.pool_num_pages ? page : -1;
    }
    // slot of pooled token t (t < t_end) of this tile, -1 outside the pool
    auto tile_slot = [&](int t) -> int64_t {
        const int jp = t / p.pool_page;
        const int page = __builtin_amdgcn_readlane(pg_lane, jp - pg0);
        return page < 0 ? -1 : (int64_t)page * p.pool_page + (t - jp * p.pool_page);
    };
    // Group loads are unconditional -- past the tile's end (or a padding
    // segment) they re-read an in-range row, whose logits are masked -- since
    // a load behind a branch makes the compiler wait for every load in flight
    // at the join, which would undo the prefetch.  Groups past the tile's end
    // are loaded too (the tile's last row), so that every pass of the loop
    // below issues the same loads: the compiler can then count exactly which
    // loads a wait needs.
    // A lane's segments of a group: rows and columns fixed per lane, so a
    // group's loads are a uniform base (the group's first row, clamped to the
    // tile's last) plus small non-negative offsets.
    int lrow[NLD], lcol[NLD];
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
        const int seg = min(ttid + kMlaTT * j, SEGS - 1);
        lrow[j] = seg / (kMlaDK / 8);
        lcol[j] = 8 * (seg % (kMlaDK / 8));
    }
    const int urow = (ttid >> 3) & 15, ucol = PATCH ? 8 * min(ttid & 7, m / 8 - 1) : 0;  // 16 rows x 8 segments
    auto load_group = [&](int tg, u32x4 (&pk)[NLD], u32x4& pu) {
        // pooled tokens: the group of 16 lies in one page (P % 16 == 0); a
        // page outside the pool, or a group past the end, reads slot 0
        const int tb = min(tg, t_end - 1);   // rows tb .. tb + lim exist
        int lim = t_end - 1 - tb;
        int64_t row0 = tb;
        if (POOL) {
            const int64_t slot = tg < t_end ? tile_slot(tg) : -1;
            row0 = slot >= 0 ? slot : 0;
            if (slot < 0) lim = 0;
        }
        // byte offsets in 32 bits: the loads take the uniform base as is
        const char* base = reinterpret_cast<const char*>(kb + row0 * kMlaDK);
#pragma unroll
        for (int j = 0; j < NLD; ++j)
            pk[j] = ld_cached(reinterpret_cast<const uint16_t*>(
                base + (__umul24((uint32_t)min(lrow[j], lim), 2u * kMlaDK) + 2u * (uint32_t)lcol[j])));
        if (PATCH)
            pu = ld_cached(reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(ub + (int64_t)tb * m) +
                                                             (__umul24((uint32_t)min(urow, lim), 2u * (uint32_t)m) +
                                                              2u * (uint32_t)ucol)));
    };
    // ---- the query's operands, and V's rows for w below, are loaded into
    // registers first, then the first two groups' rows.  Loads complete in
    // issue order, so the waits for the set-up's loads do not wait for the
    // groups, whose latency the set-up's work then hides.  Every load is
    // unconditional (a head past G, a k-step past the row or a rank column
    // past m reads an in-range address and is zeroed at use).
    const int b = POOL ? e : seq_of_entry(p.seq_entries, p.B, e);
    const int64_t delta = POOL ? 0 : ld_uniform(p.delta + e);  // R(0) = I exactly
    const uint16_t* qb = p.q + (int64_t)b * p.Hq * kMlaDK;
    const bool hok = n16 < G;
    // c_KV operands of k-steps wave + 8 r (staged in LDS by this wave, and
    // its A operands of w below)
    u32x4 qv[KN / kMlaWaves];
    {
        const uint16_t* qh = qb + (int64_t)min(n16, G - 1) * kMlaDK + 8 * q4;
#pragma unroll
        for (int r = 0; r < KN / kMlaWaves; ++r) qv[r] = ld_cached(qh + 32 * (wave + kMlaWaves * r));
    }
    // k_rope entries of heads wave + 8 r, column `lane`, and their partners
    const int R = p.rope_dim, half_r = R >> 1;  // 64 (checked on the host)
    int jj, partner;
    float sg;
    if (p.rope_style == KAMERA_ROPE_HALF) {
        const bool first = lane < half_r;
        jj = first ? lane : lane - half_r;
        partner = first ? lane + half_r : lane - half_r;
        sg = first ? 1.0f : -1.0f;
    } else {
        jj = lane >> 1;
        partner = lane ^ 1;
        sg = (lane & 1) ? -1.0f : 1.0f;
    }
    uint32_t qx[16 / kMlaWaves], qp[16 / kMlaWaves];
#pragma unroll
    for (int r = 0; r < 16 / kMlaWaves; ++r) {
        const uint16_t* qh = qb + (int64_t)min(wave + kMlaWaves * r, G - 1) * kMlaDK + p.rope_offset;
        qx[r] = qh[lane];
        qp[r] = qh[partner];
    }
    // w's operands: the k_rope step (16 or 17) of waves 0 and 1 as given, and
    // for k-step s = wave + 8 j and rank block cb the 16 bytes of V row
    // 32 s + 8 q4 + (n16 & 7), rank columns 16 cb + 8 (n16 >> 3) ..: a lane
    // octet holds an 8 x 8 block, turned into B operands below
    constexpr int WJ = (KS + kMlaWaves - 1) / kMlaWaves;  // 3
    u32x4 qa4 = zero, vt[PATCH ? WJ : 1][PATCH ? NB : 1];
    if (PATCH) {
        qa4 = ld_cached(qb + (int64_t)min(n16, G - 1) * kMlaDK + 32 * min(KN + wave, KS - 1) + 8 * q4);
        const uint16_t* vb = p.vk + blk * p.F * m;
#pragma unroll
        for (int j = 0; j < WJ; ++j) {
            const int srow = 32 * min(wave + kMlaWaves * j, KS - 1) + 8 * q4 + (n16 & 7);
#pragma unroll
            for (int cb = 0; cb < NB; ++cb)
                vt[j][cb] = ld_cached(vb + (int64_t)srow * m + min(16 * cb + 8 * (n16 >> 3), m - 8));
        }
    }
    // The teams take alternate groups: team t the groups at t_begin + 16 t,
    // + 32 + 16 t, + 64 + 16 t, ...  Two register sets of group loads per
    // thread: a team's group is requested two of its groups ahead of its use.
    u32x4 pk0[NLD], pk1[NLD], pu0 = zero, pu1 = zero;
    // Two groups of each team per pass, all processed (a group past the end
    // has every token masked and adds nothing).  Issued unconditionally: an
    // entry's tile is never empty, and a pooled tile past the sequence's
    // tokens reads slot 0 (load_group); a branch here would leave the
    // compiler unsure how many loads follow the set-up's, so every wait below
    // would wait for all of them.  With a patch, the first groups are
    // requested only once w's products have their V rows (below): every
    // workgroup's first groups, requested at once, would queue ahead of V's
    // rows, and w would wait for the flood.
    if (!PATCH) {
        load_group(t_begin + 16 * team, pk0, pu0);
        load_group(t_begin + 32 + 16 * team, pk1, pu1);
    }
    // keep the scheduler from moving the uses below (and their waits) above
    // the loads
    __builtin_amdgcn_sched_barrier(0);

    // ---- query operands to LDS: c_KV steps as given, the k_rope part turned
#pragma unroll
    for (int r = 0; r < KN / kMlaWaves; ++r) qn[wave + kMlaWaves * r][lane] = hok ? qv[r] : zero;
    const float2 cs = rope_cos_sin(p.log2_base, R, jj, delta);  // the same for every head
#pragma unroll
    for (int r = 0; r < 16 / kMlaWaves; ++r) {
        const int h = wave + kMlaWaves * r;
        const float x = fmaf(__uint_as_float(qx[r] << 16), cs.x, sg * __uint_as_float(qp[r] << 16) * cs.y);
        qr[h][lane] = h < G ? x : 0.0f;
    }
    // ---- the key patch's query weights w[h][k] = qscale sum_d q_h[d] V[d][k]
    // over the joint row's 576 columns (q as given: the patch sits in the
    // destination frame), on the matrix cores: A = the query, B = 8 rows of
    // V's column k (V's rows run along k, so each lane octet transposes the
    // 8 x 8 block it loaded).  Wave w takes the k-steps w, w + 8, ... of
    // every rank block; the eight partial products meet in LDS (the group
    // buffers, not yet in use) and are added in a fixed order into um[h][k]
    // (zero past the rank or the heads).
    if (PATCH) {
        f32x4 wc[NB];
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) wc[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        // Branch-free: a step past the row multiplies a zero query, and rank
        // columns past m are dropped below (a load left unused on one path of
        // a branch makes the compiler wait for every load in flight).
#pragma unroll
        for (int j = 0; j < WJ; ++j) {
            const bool aok = hok && wave + kMlaWaves * j < KS;
            const bf16x8 a = __builtin_bit_cast(bf16x8, aok ? (j < KN / kMlaWaves ? qv[j] : qa4) : zero);
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                const bf16x8 bv = __builtin_bit_cast(bf16x8, transpose8x8_b16(vt[j][cb], lane));
                wc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, wc[cb], 0, 0, 0);
            }
        }
        load_group(t_begin + 16 * team, pk0, pu0);
        load_group(t_begin + 32 + 16 * team, pk1, pu1);
        __builtin_amdgcn_sched_barrier(0);
        f32x4* wred = reinterpret_cast<f32x4*>(&kbuf[0][0][0]);  // [wave][rank block][lane]: <= 32 KB
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) wred[(wave * NB + cb) * 64 + lane] = wc[cb];
        __syncthreads();
        for (int i = tid; i < 16 * kMaxRank; i += kMlaThreads) {
            const int h = i / kMaxRank, k = i % kMaxRank;
            float x = 0.0f;
            if (h < G && k < m) {
                // C[h][k] of block k / 16 sits in lane (k % 16) + 16 (h / 4), element h % 4
                const int cb = k / 16, ln = (k % 16) + 16 * (h / 4);
#pragma unroll
                for (int w = 0; w < kMlaWaves; ++w) x += wred[(w * NB + cb) * 64 + ln][h % 4];
            }
            um[h][k] = x * p.qscale;
        }
        for (int i = tid; i < 16 * kMaxRank; i += kMlaThreads) sh.uv[i / kMaxRank][i % kMaxRank] = 0.0f;
    }
    __syncthreads();
    // The key product per wave of a team: the c_KV steps tw + 4 r (r < 4)
    // against the query as given, then one step of its own -- team waves 0
    // and 1 the turned k_rope step KN + tw, team waves 2 and 3 (with a patch)
    // the key patch's rank step tw - 2 -- against fp32 operands split into
    // bf16 high and low parts.  The qscale of the logits is folded into the
    // turned query (w carries it already), so the c_KV sum alone is scaled.
    const bool rope_wave = tw < KS - KN;
    bf16x8 xhi, xlo;
    {
        const int sr = rope_wave ? tw : tw - (KS - KN);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = rope_wave ? qr[n16][32 * sr + 8 * q4 + j] * p.qscale
                                      : (PATCH ? um[n16][32 * sr + 8 * q4 + j] : 0.0f);
            xhi[j] = bf_hi_part(x);
            xlo[j] = bf_lo_part(x);
        }
    }
    // LDS offsets of this lane's operands in a group's buffers
    const int ka = n16 * KP + 32 * tw + 8 * q4;  // c_KV step tw (+ 128 per r)
    const int xa = rope_wave ? n16 * KP + 32 * (KN + tw) + 8 * q4 : n16 * UP + 32 * (tw - (KS - KN)) + 8 * q4;
    const int vta = (4 * q4 + (n16 >> 2)) * KP + 4 * (n16 & 3);  // value operands (+ the chunk's column)
    const int uta = (4 * q4 + (n16 >> 2)) * UP + 4 * (n16 & 3);

    f32x4 acc[VCW], uacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < VCW; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float mrun = kEmpty, lrun = 0.0f;
    // A team's groups alternate between its two LDS buffers, so a group's
    // rows can be parked while slower waves still read the previous group's:
    // every wave has finished the group before last when it passes the
    // previous group's barriers.  Both teams pass every barrier together.
    auto process_group = [&](int tg, u32x4 (&pk)[NLD], u32x4& pu, const int bi, const bool prefetch) {
        uint16_t* kb_ = kbuf[team][bi];
        uint16_t* ub_ = ubuf[team][bi];
        // rows as loaded: a row past the tile's end (or of a page outside the
        // pool) holds an in-range row's finite values, and its logits are
        // masked to -inf below, so it adds exactly nothing
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int seg = ttid + kMlaTT * j;
            if (seg < SEGS) {
                const int row = seg / (kMlaDK / 8), c16 = seg % (kMlaDK / 8);
                *reinterpret_cast<u32x4*>(kb_ + row * KP + 8 * c16) = pk[j];
            }
        }
        if (PATCH && ttid < 128) *reinterpret_cast<u32x4*>(ub_ + (ttid >> 3) * UP + 8 * (ttid & 7)) = pu;
        __syncthreads();
        if (prefetch) load_group(tg + 64, pk, pu);  // this set is free again (a constant at each call)
        // this wave's share of the key product: operands read first, then the
        // two independent chains of products
        u32x4 av[KN / kMlaTW], qb4[KN / kMlaTW];
#pragma unroll
        for (int r = 0; r < KN / kMlaTW; ++r) {
            av[r] = *reinterpret_cast<const u32x4*>(kb_ + ka + 32 * kMlaTW * r);
            qb4[r] = qn[tw + kMlaTW * r][lane];
        }
        const u32x4 ax = *reinterpret_cast<const u32x4*>((rope_wave ? kb_ : ub_) + xa);
        f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f}, cx = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int r = 0; r < KN / kMlaTW; ++r)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[r]),
                                                         __builtin_bit_cast(bf16x8, qb4[r]), c, 0, 0, 0);
        if (PATCH || rope_wave) {
            cx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ax), xhi, cx, 0, 0, 0);
            cx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ax), xlo, cx, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = fmaf(c[i], p.qscale, cx[i]);
        spart[team][tw][lane] = c;
        __syncthreads();
        f32x4 sc = spart[team][0][lane];
#pragma unroll
        for (int w = 1; w < kMlaTW; ++w) {
            const f32x4 o = spart[team][w][lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[i] += o[i];
        }
        if (POOL || tg + 16 > t_end) {  // uniform: a group with masked tokens
            bool gbad = false;  // pooled tokens of a page outside the pool: masked
            if (POOL) {
                gbad = tg < t_end && tile_slot(tg) < 0;
                if (gbad && ttid == 0 && p.error_word) atomicOr(p.error_word, (uint32_t)KAMERA_EW_PAGE);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (tg + 4 * q4 + i >= t_end || gbad) sc[i] = -INFINITY;
        }
        // online softmax of head n16 (identical in every wave); exp2 of a
        // logit below the maximum by more than 126 flushes to zero
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(mrun, mx);
        const float alpha = __builtin_amdgcn_exp2f(mrun - mn);
        mrun = mn;
        bf16x4 phi, plo;
        float psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float pp = __builtin_amdgcn_exp2f(sc[i] - mn);
            psum += pp;
            phi[i] = bf_hi_part(pp);
            plo[i] = bf_lo_part(pp);
        }
        lrun = fmaf(lrun, alpha, psum);
        if (__any(alpha != 1.0f)) {  // exact no-op when no head's maximum moved
            float ar[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * q4 + i);
#pragma unroll
            for (int cc = 0; cc < VCW; ++cc)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[cc][i] *= ar[i];
#pragma unroll
            for (int i = 0; i < 4; ++i) uacc[i] *= ar[i];
        }
        // this wave's value columns: B = 4 consecutive tokens of one column,
        // read by the transposing LDS read (lane (n16, q4) names row
        // 4 q4 + n16 / 4, columns 4 (n16 % 4) .. of the 16-column chunk)
#pragma unroll
        for (int cc = 0; cc < VCW; ++cc) {
            const bf16x4 bv = lds_read_tr16(kb_ + vta + 16 * (VCW * tw + cc));
            acc[cc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, bv, acc[cc], 0, 0, 0);
            acc[cc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, bv, acc[cc], 0, 0, 0);
        }
        if (uwave) {
            const bf16x4 bv = lds_read_tr16(ub_ + uta + 16 * tw);
            uacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, bv, uacc, 0, 0, 0);
            uacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, bv, uacc, 0, 0, 0);
        }
    };
    // every pass but the last requests the groups of the pass after it; the
    // last requests nothing (loads past the tile would only be waited for)
    int tg = t_begin;
    for (; tg + 64 < t_end; tg += 64) {  // uniform over the workgroup
        process_group(tg + 16 * team, pk0, pu0, 0, true);
        process_group(tg + 32 + 16 * team, pk1, pu1, 1, true);
    }
    if (tg < t_end) {
        process_group(tg + 16 * team, pk0, pu0, 0, false);
        process_group(tg + 32 + 16 * team, pk1, pu1, 1, false);
    }
    lrun += __shfl_xor(lrun, 16);
    lrun += __shfl_xor(lrun, 32);
    // the value patch's B operands (8 consecutive k of V_c row col), requested
    // before the merge so that their latency hides behind it; clamped to the
    // rank, zeroed at use
    constexpr int NS = (NB + 1) / 2;  // 32-wide rank steps
    u32x4 vbr[PATCH ? NS : 1][VCW];
    if (PATCH) {
        const uint16_t* vvh = p.vk + blk * p.F * m;  // V's c_KV rows
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int cc = 0; cc < VCW; ++cc) {
                const int col = 16 * (VCW * tw + cc) + n16;
                vbr[s][cc] = ld_cached(vvh + (int64_t)col * m + min(32 * s + 8 * q4, m - 8));
            }
    }
    // ---- the teams' softmax states merge: team 1 parks its accumulators
    // (and its per-head max and sum) in its group buffers, team 0 rescales
    // both to the common maximum and adds them
    __syncthreads();  // every group's reads of the buffers are done
    f32x4* tacc = reinterpret_cast<f32x4*>(&kbuf[1][0][0]);  // [team wave][VCW + 1][lane]: 36 KB
    if (team == 1) {
#pragma unroll
        for (int cc = 0; cc < VCW; ++cc) tacc[(tw * (VCW + 1) + cc) * 64 + lane] = acc[cc];
        tacc[(tw * (VCW + 1) + VCW) * 64 + lane] = uacc;
        if (tw == 0 && q4 == 0) {
            sh.tm[n16] = mrun;
            sh.tl[n16] = lrun;
        }
    }
    __syncthreads();
    if (team == 0) {
        const float m1 = sh.tm[n16];
        const float M = fmaxf(mrun, m1);
        const float f0 = __builtin_amdgcn_exp2f(mrun - M), f1 = __builtin_amdgcn_exp2f(m1 - M);
        lrun = fmaf(lrun, f0, sh.tl[n16] * f1);
        mrun = M;
        float r0[4], r1[4];  // factors of this lane's accumulator rows (heads 4 q4 + i)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            r0[i] = __shfl(f0, 4 * q4 + i);
            r1[i] = __shfl(f1, 4 * q4 + i);
        }
#pragma unroll
        for (int cc = 0; cc <= VCW; ++cc) {
            const f32x4 o = tacc[(tw * (VCW + 1) + cc) * 64 + lane];
            f32x4& a = cc < VCW ? acc[cc] : uacc;
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = fmaf(a[i], r0[i], o[i] * r1[i]);
        }
    }
    if (PATCH) {
        // u, shared: uv[h][k] (zero past the rank since the set-up); then
        // O += u V_c^T on the matrix cores (A = u hi + lo [16 heads x 32 k],
        // B = vbr above).
        if (team == 0 && uwave)
#pragma unroll
            for (int i = 0; i < 4; ++i) sh.uv[4 * q4 + i][16 * tw + n16] = uacc[i];
        __syncthreads();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (team != 0 || 32 * s >= m) break;
            bf16x8 ahi, alo;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = sh.uv[n16][32 * s + 8 * q4 + j];
                ahi[j] = bf_hi_part(x);
                alo[j] = bf_lo_part(x);
            }
#pragma unroll
            for (int cc = 0; cc < VCW; ++cc) {
                const u32x4 bw = 32 * s + 8 * q4 < m ? vbr[s][cc] : zero;
                const bf16x8 bv = __builtin_bit_cast(bf16x8, bw);
                acc[cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bv, acc[cc], 0, 0, 0);
                acc[cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bv, acc[cc], 0, 0, 0);
            }
        }
    }
    // the partial: team 0 parks it row-major in its group buffers (free
    // since the merge's first barrier), then every wave stores it with
    // 16-byte stores (4 per thread)
    float* stg = reinterpret_cast<float*>(&kbuf[0][0][0]);  // [16][kMlaStgPitch]
    if (team == 0) {
#pragma unroll
        for (int cc = 0; cc < VCW; ++cc)
#pragma unroll
            for (int i = 0; i < 4; ++i) stg[(4 * q4 + i) * kMlaStgPitch + 16 * (VCW * tw + cc) + n16] = acc[cc][i];
        if (tw == 0 && q4 == 0 && n16 < G) p.part_ml[pidx + n16 * p.units] = make_float2(mrun, lrun);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16 * kMlaDV / 4 / kMlaThreads; ++k) {
        const int v = tid + kMlaThreads * k, row = v / (kMlaDV / 4), c4 = v % (kMlaDV / 4);
        if (row < G)
            *reinterpret_cast<float4*>(p.part_o + (pidx + row * p.units) * kMlaDV + 4 * c4) =
                *reinterpret_cast<const float4*>(stg + row * kMlaStgPitch + 4 * c4);
    }
}

// Workgroup b runs on XCD b % 8, and the tiles of one entry share its V
// (read for w): spread over the XCDs, every XCD's L2 would fetch V from HBM.
// With the units a multiple of 8, XCD k takes units k n / 8 .. (k + 1) n / 8 - 1
// -- an entry's consecutive tiles on one XCD -- else the identity.
__device__ __forceinline__ int xcd_unit(int b, int n) {
    return n % 8 ? b : (b % 8) * (n / 8) + b / 8;
}

template <bool PATCH, bool POOL = false, int NB = 2>
__global__ __launch_bounds__(kMlaThreads, 1) void attn_mla_kernel(const AttnParams p) {
    __shared__ MlaShared sh;
    mla_tile<PATCH, POOL, NB>(p, xcd_unit((int)blockIdx.x, (int)gridDim.x), sh);
}

// A reused context and pooled tokens in one launch: blocks [0, pool_unit0)
// take the entries' tiles, the rest the pooled tokens' tiles.  One launch
// fills the chip with half as many (twice as long) tiles as two launches
// would need, so the combine merges half as many partials.
template <bool PATCH, int NB = 2>
__global__ __launch_bounds__(kMlaThreads, 1) void attn_mla_mixed_kernel(const AttnParams p) {
    __shared__ MlaShared sh;
    // each XCD takes its eighth of the entries' tiles and of the pooled
    // tokens' tiles (both sets a multiple of 8; else blocks map to units as
    // they are)
    const int bx = blockIdx.x, n = gridDim.x, ne = (int)p.pool_unit0, np = n - ne;
    int64_t u = bx;
    if (ne % 8 == 0 && np % 8 == 0) {
        const int k = bx % 8, slot = bx / 8;
        u = slot < ne / 8 ? (int64_t)k * (ne / 8) + slot : ne + (int64_t)k * (np / 8) + (slot - ne / 8);
    }
    if (u < p.pool_unit0)
        mla_tile<PATCH, false, NB>(p, (int)u, sh);
    else
        mla_tile<false, true, 2>(p, (int)(u - p.pool_unit0), sh);
}

// ---------------------------------------------------------------------------
// attn_combine_kernel: one workgroup per (query head, sequence)
// ---------------------------------------------------------------------------
// Threads (slice, 4 columns) over a block of CW columns: each slice merges
// every NS-th partial of the sequence (online log-sum-exp), then slice 0
// merges the slices and normalises.  Each thread issues the loads of a batch
// of partials before merging any.  Rows of 512 columns are split into 32-wide
// blocks, which gives Hq x B x 16 workgroups (256 for 16 heads); rows of up
// to 128 columns are read whole by 32 slices, consecutive partials of a head
// being adjacent rows.
struct CombineArgs {
    const float* part_o;
    const float2* part_ml;
    const int32_t* seq_entries;
    float* out;
    float* lse;
    int32_t B, E, tiles, Hkv, Hq, G;
    int32_t pool_tiles;   // partials of each sequence's pooled tokens (0: none),
    int64_t pool_unit0;   // from unit pool_unit0 + b * pool_tiles on
    int64_t units;        // partials per head
};

template <int D>
constexpr int combine_cols() { return D > 256 ? 32 : (D < 128 ? D : 128); }  // columns per workgroup
constexpr int kCombineSlices = 32;

// grid (query head, sequence, column block of combine_cols<D>()).  NBAT:
// partials in flight per thread, chosen at launch so that one batch covers a
// sequence's partials where it can (loads past the end are wasted work).
template <int D, int NBAT>
__global__ __launch_bounds__(kCombineSlices * combine_cols<D>() / 4) void attn_combine_kernel(const CombineArgs a) {
    constexpr int CW = combine_cols<D>();
    static_assert(D % CW == 0, "whole column blocks");
    constexpr int NS = kCombineSlices;
    constexpr int kCombineBatch = NBAT;
    constexpr int TPS = CW / 4;  // threads per slice, 4 columns each
    __shared__ float sm[NS], sl[NS];
    __shared__ float4 so[NS][TPS];
    const int h = blockIdx.x, b = blockIdx.y;
    const int c4 = threadIdx.x % TPS, slice = threadIdx.x / TPS;
    const int col = blockIdx.z * CW + 4 * c4;
    int e0 = ld_uniform(a.seq_entries + b), e1 = ld_uniform(a.seq_entries + b + 1);
    e0 = min(max(e0, 0), a.E);
    e1 = min(max(e1, e0), a.E);
    float M = kEmpty, L = 0.0f;
    float4 O = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    auto merge = [&](const float2 ml, const float4 o) {
        const float mn = fmaxf(M, ml.x);
        const float fa = __builtin_amdgcn_exp2f(M - mn), fb = __builtin_amdgcn_exp2f(ml.x - mn);
        O.x = fmaf(O.x, fa, o.x * fb);
        O.y = fmaf(O.y, fa, o.y * fb);
        O.z = fmaf(O.z, fa, o.z * fb);
        O.w = fmaf(O.w, fa, o.w * fb);
        L = fmaf(L, fa, ml.y * fb);
        M = mn;
    };
    // The sequence's partials: its entries' tiles, then its pooled tokens'
    // tiles, as one list (one batch of loads covers both).  Slice s merges
    // items s, s + NS, ... in that order; a batch's loads past the end
    // re-read the last item and are not merged.
    const int64_t lo1 = (int64_t)e0 * a.tiles, n1 = (int64_t)(e1 - e0) * a.tiles;
    const int64_t lo2 = a.pool_unit0 + (int64_t)b * a.pool_tiles;
    const int64_t n = n1 + (a.pool_tiles > 0 ? a.pool_tiles : 0);
    for (int64_t base = slice; base < n; base += (int64_t)NS * kCombineBatch) {
        float2 ml[kCombineBatch];
        float4 o[kCombineBatch];
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) {
            const int64_t i = min(base + (int64_t)NS * j, n - 1);
            const int64_t u = i < n1 ? lo1 + i : lo2 + (i - n1);
            const int64_t idx = (int64_t)h * a.units + u;
            ml[j] = a.part_ml[idx];
            o[j] = *reinterpret_cast<const float4*>(a.part_o + idx * D + col);
        }
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j)
            if (base + (int64_t)NS * j < n) merge(ml[j], o[j]);
    }
    so[slice][c4] = O;
    if (c4 == 0) {
        sm[slice] = M;
        sl[slice] = L;
    }
    __syncthreads();
    if (slice != 0) return;
    float Mt = sm[0];
#pragma unroll
    for (int s = 1; s < NS; ++s) Mt = fmaxf(Mt, sm[s]);
    float4 Ot = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float Lt = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const float f = __builtin_amdgcn_exp2f(sm[s] - Mt);
        Ot.x = fmaf(so[s][c4].x, f, Ot.x);
        Ot.y = fmaf(so[s][c4].y, f, Ot.y);
        Ot.z = fmaf(so[s][c4].z, f, Ot.z);
        Ot.w = fmaf(so[s][c4].w, f, Ot.w);
        Lt = fmaf(sl[s], f, Lt);
    }
    const int64_t oi = (int64_t)b * a.Hq + h;
    const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
    *reinterpret_cast<float4*>(a.out + oi * D + col) = make_float4(Ot.x * inv, Ot.y * inv, Ot.z * inv, Ot.w * inv);
    if (c4 == 0 && blockIdx.z == 0 && a.lse) a.lse[oi] = Lt > 0.0f ? (Mt + log2f(Lt)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_combine(int Hq, int B, hipStream_t hs, const CombineArgs& ca) {
    const dim3 grid((unsigned)Hq, (unsigned)B, (unsigned)(D / combine_cols<D>()));
    const dim3 block(kCombineSlices * combine_cols<D>() / 4);
    // partials per slice of an average sequence
    const int64_t per_slice = (ca.units / std::max(B, 1) + kCombineSlices - 1) / kCombineSlices;
    if (per_slice <= 2) return launch_kernel(attn_combine_kernel<D, 2>, grid, block, hs, ca);
    if (per_slice <= 4) return launch_kernel(attn_combine_kernel<D, 4>, grid, block, hs, ca);
    if constexpr (D > 256) {  // (rows of 256 or fewer columns would spill at 16)
        if (per_slice > 8) return launch_kernel(attn_combine_kernel<D, 16>, grid, block, hs, ca);
    }
    return launch_kernel(attn_combine_kernel<D, 8>, grid, block, hs, ca);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

struct AttnPlan {
    bool mla;
    int tiles, tile_tokens, dv;
    int pool_tiles;      // token tiles of each sequence's pooled tokens
    int pool_tile_tokens;
    int64_t entry_units; // E * tiles (the pool's partials follow)
    int64_t units, part_o_bytes, part_ml_bytes, total;
};

bool is_mla(const kamera_layout& L) { return L.num_streams == 1; }

inline int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

// Token tiles: whole passes of every wave, doubled while the grid keeps at
// least a floor of workgroups, since fewer, longer tiles spend less on each
// workgroup's set-up and merge and leave fewer partials to combine; up to 16
// passes per wave.  A reused context with pooled tokens runs one launch over
// both sets of tiles, each set sized by its share of the floor.  Floors
// (measured on MI355X, ms per 36-layer step):
//  * 8-wave MLA kernel: 256, one per CU (paged MLA 0.734 against 0.934 at
//    128 and 1.007 at 512);
//  * 4-wave GQA kernel, entries or pooled tokens alone: 256, one per CU
//    (reorder 2.161 against 2.188 at 512 and 2.230 at 1024);
//  * 4-wave GQA kernel, both in one launch: 1024, two rounds of two per CU,
//    so that the dispatcher evens out the entries' tiles, whose set-up is
//    longer, against the pooled ones (paged reorder 2.218 against 2.275 at
//    512 and 2.247 at 256).
// KAMERA_ATTN_MIN_WG overrides the GQA floor (tuning; MLA takes half of it).
void attn_plan(const kamera_layout& L, int Hq, int E, int T, int B, int pool_T, AttnPlan& pl) {
    pl.mla = is_mla(L);
    pl.dv = pl.mla ? kMlaDV : L.head_dim;           // output width per query head
    const int G = Hq / L.num_heads;
    const int per_tile_wgs = pl.mla ? 1 : L.num_heads;  // MLA: one workgroup per tile
    // GQA: one pass of every wave; MLA: one pass of its loop (two 16-token
    // groups of each of its two teams)
    const int64_t per_tile_min = pl.mla ? 64 : (int64_t)kAttnWaves * kMfmaPass;
    static const int64_t min_wg_env = [] {
        const char* v = getenv("KAMERA_ATTN_MIN_WG");
        return v ? (int64_t)atol(v) : (int64_t)0;
    }();
    const bool mixed = E > 0 && T > 0 && B > 0 && pool_T > 0;
    const int64_t min_wg = min_wg_env > 0 ? min_wg_env : (pl.mla ? 512 : (mixed ? 1024 : 256));
    // tokens per tile for `count` sequences (or entries) of n tokens each:
    // doubled while the launch keeps at least `need` workgroups.  A reused
    // context with pooled tokens runs one launch over both sets of tiles:
    // each set then needs only its share of the floor (by tokens), so the
    // tiles come out twice as long and leave half the partials to combine
    const int64_t floor_wg = pl.mla ? std::max<int64_t>(1, min_wg / 2) : min_wg;
    int64_t min_e = floor_wg, min_p = floor_wg;
    if (mixed) {
        const double te = (double)E * T, tp = (double)B * pool_T;
        min_e = std::max<int64_t>(1, (int64_t)(floor_wg * te / (te + tp)));
        min_p = std::max<int64_t>(1, floor_wg - min_e);
    }
    auto tile_for_min = [&](int64_t count, int64_t n, int64_t need) {
        int passes = 1;
        while (passes < 16) {
            const int64_t tt = per_tile_min * passes * 2;
            if (count * ((n + tt - 1) / tt) * per_tile_wgs < need) break;
            passes *= 2;
        }
        return (int)(per_tile_min * passes);
    };
    pl.tile_tokens = tile_for_min(E, T, min_e);
    pl.pool_tile_tokens = tile_for_min(B, pool_T, min_p);
    pl.tiles = T > 0 ? (T + pl.tile_tokens - 1) / pl.tile_tokens : 0;
    pl.pool_tiles = pool_T > 0 ? (pool_T + pl.pool_tile_tokens - 1) / pl.pool_tile_tokens : 0;
    pl.entry_units = (int64_t)E * pl.tiles;
    pl.units = pl.entry_units + (int64_t)B * pl.pool_tiles;
    const int64_t parts = pl.units * L.num_heads * G;
    pl.part_o_bytes = align256(parts * pl.dv * 4);
    pl.part_ml_bytes = align256(parts * 8);
    pl.total = pl.part_o_bytes + pl.part_ml_bytes;
}

kamera_status check_attn_layout(const kamera_layout* L, int Hq) {
    if (!L) return KAMERA_ERR_NULL;
    if (L->num_layers < 1 || L->num_layers > 65535 || L->num_heads < 1 || L->head_dim < 1) return KAMERA_ERR_RANGE;
    if (L->num_streams < 1 || L->num_streams > 2) return KAMERA_ERR_RANGE;
    if (L->rope_style != KAMERA_ROPE_HALF && L->rope_style != KAMERA_ROPE_INTERLEAVED) return KAMERA_ERR_RANGE;
    if (L->rope_offset < 0 || L->rope_dim < 0 || L->rope_offset + L->rope_dim > L->head_dim) return KAMERA_ERR_RANGE;
    if (L->rope_dim % 2 || L->rope_offset % 2) return KAMERA_ERR_RANGE;
    if (!(L->rope_base > 0.0) || !isfinite(L->rope_base)) return KAMERA_ERR_RANGE;
    if (Hq < 1 || Hq % L->num_heads) return KAMERA_ERR_SHAPE;
    if (L->num_streams == 1) {  // MLA: one 576-wide joint row [c_KV 512 | k_rope 64], one KV head
        if (L->num_heads != 1 || L->head_dim != kMlaDK || L->rope_offset != kMlaDV || L->rope_dim != 64)
            return KAMERA_ERR_UNSUPPORTED;
        return Hq > 16 ? KAMERA_ERR_UNSUPPORTED : KAMERA_OK;
    }
    if (L->head_dim != 64 && L->head_dim != 128 && L->head_dim != 256) return KAMERA_ERR_UNSUPPORTED;
    if (Hq / L->num_heads > 16 || L->num_heads > 65535) return KAMERA_ERR_UNSUPPORTED;
    if ((int64_t)L->num_heads * L->head_dim > 4096) return KAMERA_ERR_UNSUPPORTED;
    return KAMERA_OK;
}

hipError_t launch_mla(bool patch, int m, const AttnPlan& pl, int Hq, int B, hipStream_t hs, const AttnParams& p,
                      const CombineArgs& ca) {
    hipError_t e = hipSuccess;
    const bool wide = m > 32;  // rank blocks: 2 up to rank 32, else 4
    if (pl.entry_units > 0 && pl.pool_tiles > 0 && B > 0) {
        // reused entries and pooled tokens: one launch over both sets of tiles
        const dim3 gs((unsigned)(pl.entry_units + (int64_t)B * pl.pool_tiles));
        if (!patch)
            e = launch_kernel(attn_mla_mixed_kernel<false>, gs, dim3(kMlaThreads), hs, p);
        else if (wide)
            e = launch_kernel(attn_mla_mixed_kernel<true, 4>, gs, dim3(kMlaThreads), hs, p);
        else
            e = launch_kernel(attn_mla_mixed_kernel<true, 2>, gs, dim3(kMlaThreads), hs, p);
        if (e == hipSuccess) e = launch_combine<kMlaDV>(Hq, B, hs, ca);
        return e;
    }
    if (pl.entry_units > 0) {
        const dim3 gs((unsigned)pl.entry_units);
        if (!patch)
            e = launch_kernel(attn_mla_kernel<false>, gs, dim3(kMlaThreads), hs, p);
        else if (wide)
            e = launch_kernel(attn_mla_kernel<true, false, 4>, gs, dim3(kMlaThreads), hs, p);
        else
            e = launch_kernel(attn_mla_kernel<true, false, 2>, gs, dim3(kMlaThreads), hs, p);
    }
    if (e == hipSuccess && pl.pool_tiles > 0 && B > 0)
        e = launch_kernel(attn_mla_kernel<false, true>, dim3((unsigned)((int64_t)B * pl.pool_tiles)),
                          dim3(kMlaThreads), hs, p);
    if (e == hipSuccess) e = launch_combine<kMlaDV>(Hq, B, hs, ca);
    return e;
}

template <int D>
hipError_t launch_attn(bool patch, int m, const AttnPlan& pl, int Hkv, int Hq, int B, hipStream_t hs,
                       const AttnParams& p, const CombineArgs& ca) {
    hipError_t e = hipSuccess;
    const bool wide = m > 32;  // rank blocks: 2 up to rank 32, else 4
    if (pl.entry_units > 0 && pl.pool_tiles > 0 && B > 0) {
        // reused entries and pooled tokens: one launch over both sets of tiles
        const dim3 gs((unsigned)(pl.entry_units + (int64_t)B * pl.pool_tiles), (unsigned)Hkv);
        if (!patch)
            e = launch_kernel(attn_mfma_mixed_kernel<D, false>, gs, dim3(kAttnThreads), hs, p);
        else if (wide)
            e = launch_kernel(attn_mfma_mixed_kernel<D, true, 4>, gs, dim3(kAttnThreads), hs, p);
        else
            e = launch_kernel(attn_mfma_mixed_kernel<D, true, 2>, gs, dim3(kAttnThreads), hs, p);
        if (e == hipSuccess) e = launch_combine<D>(Hq, B, hs, ca);
        return e;
    }
    if (pl.entry_units > 0) {
        const dim3 gs((unsigned)pl.entry_units, (unsigned)Hkv);
        if (!patch)
            e = launch_kernel(attn_mfma_kernel<D, false>, gs, dim3(kAttnThreads), hs, p);
        else if (wide)
            e = launch_kernel(attn_mfma_kernel<D, true, false, 4>, gs, dim3(kAttnThreads), hs, p);
        else
            e = launch_kernel(attn_mfma_kernel<D, true, false, 2>, gs, dim3(kAttnThreads), hs, p);
    }
    if (e == hipSuccess && pl.pool_tiles > 0 && B > 0)
        e = launch_kernel(attn_mfma_kernel<D, false, true>, dim3((unsigned)((int64_t)B * pl.pool_tiles), (unsigned)Hkv),
                          dim3(kAttnThreads), hs, p);
    if (e == hipSuccess) e = launch_combine<D>(Hq, B, hs, ca);
    return e;
}

}  // namespace

extern "C" {

int64_t kamera_decode_attention_workspace(const kamera_layout* layout, int32_t num_q_heads, int32_t num_entries,
                                          int32_t n_tokens) {
    if (check_attn_layout(layout, num_q_heads) != KAMERA_OK || num_entries < 0 || n_tokens < 0) return -1;
    AttnPlan pl;
    attn_plan(*layout, num_q_heads, num_entries, n_tokens, 0, 0, pl);
    return pl.total;
}

int64_t kamera_decode_attention_paged_workspace(const kamera_layout* layout, int32_t num_q_heads,
                                                int32_t num_entries, int32_t n_tokens, int32_t num_seqs,
                                                int32_t pool_max_tokens) {
    if (check_attn_layout(layout, num_q_heads) != KAMERA_OK || num_entries < 0 || n_tokens < 0 || num_seqs < 0 ||
        pool_max_tokens < 0)
        return -1;
    AttnPlan pl;
    attn_plan(*layout, num_q_heads, num_entries, n_tokens, num_seqs, pool_max_tokens, pl);
    return pl.total;
}

}  // extern "C"

namespace {

// Both decode-attention calls; pool == NULL: the context is the entries alone.
kamera_status decode_attention(const kamera_layout* layout, int32_t layer, const kamera_src* canon,
                               const kamera_patch* patch, const kamera_attn_pool* pool, int32_t num_seqs,
                               const int32_t* seq_entries, int32_t num_entries, const int32_t* chunk_ids,
                               const int64_t* delta, int32_t num_q_heads, const uint16_t* q, float scale, float* out,
                               float* lse, uint32_t* error_word, void* workspace, int64_t workspace_bytes,
                               void* hip_stream) {
    kamera_status st = check_attn_layout(layout, num_q_heads);
    if (st != KAMERA_OK) return st;
    const kamera_layout& L = *layout;
    if (!canon) return KAMERA_ERR_NULL;
    if (layer < 0 || layer >= L.num_layers) return KAMERA_ERR_RANGE;
    if (num_seqs < 0 || num_entries < 0) return KAMERA_ERR_RANGE;
    if (!(scale == scale) || isinf(scale)) return KAMERA_ERR_RANGE;
    const int D = L.head_dim, Hkv = L.num_heads, Hq = num_q_heads;
    const int S = L.num_streams;
    const int Dv = S == 1 ? kMlaDV : D;  // output width per query head
    const int64_t F = (int64_t)Hkv * D;
    const int T = canon->n_tokens;
    if (T < 0 || canon->n_store < 1) return KAMERA_ERR_RANGE;
    for (int s = 0; s < S; ++s) {
        if (!canon->rows[s]) return KAMERA_ERR_NULL;
        if (!aligned16(canon->rows[s])) return KAMERA_ERR_ALIGN;
    }
    if (canon->chunk_stride < 0 || canon->layer_stride < 0) return KAMERA_ERR_RANGE;
    if (canon->chunk_stride % 8 || canon->layer_stride % 8) return KAMERA_ERR_ALIGN;
    if (L.num_layers > 1 && canon->layer_stride < (int64_t)T * F) return KAMERA_ERR_SHAPE;
    if (canon->n_store > 1 && canon->chunk_stride < (int64_t)T * F) return KAMERA_ERR_SHAPE;
    const int m = patch ? patch->rank : 0;
    if (m < 0 || m > kMaxRank || m % 8) return KAMERA_ERR_RANGE;
    if (m > 0) {
        for (int s = 0; s < S; ++s) {
            if (!patch->u[s] || !patch->v[s]) return KAMERA_ERR_NULL;
            if (!aligned16(patch->u[s]) || !aligned16(patch->v[s])) return KAMERA_ERR_ALIGN;
        }
    }
    // pooled tokens: pages of a multiple of 16 tokens (a 16-token group never
    // straddles two pages), rows as in kamera_dst's pool
    int pool_T = 0;
    int64_t pool_el = 0;
    if (pool) {
        if (pool->page_size < 16 || pool->page_size % 16) return KAMERA_ERR_UNSUPPORTED;
        if (pool->max_pages < 0 || pool->num_slots < 0 || pool->layer_stride < 0) return KAMERA_ERR_RANGE;
        if ((int64_t)pool->max_pages * pool->page_size > INT32_MAX / 2) return KAMERA_ERR_RANGE;
        if (pool->num_slots / pool->page_size > INT32_MAX) return KAMERA_ERR_RANGE;
        if (pool->layer_stride % 8) return KAMERA_ERR_ALIGN;
        if (L.num_layers > 1 && pool->layer_stride < pool->num_slots * F) return KAMERA_ERR_SHAPE;
        for (int s = 0; s < S; ++s) {
            if (!pool->rows[s]) return KAMERA_ERR_NULL;
            if (!aligned16(pool->rows[s])) return KAMERA_ERR_ALIGN;
        }
        pool_T = pool->max_pages * pool->page_size;
        pool_el = (int64_t)(L.num_layers - 1) * pool->layer_stride + pool->num_slots * F;
        if (pool_T > 0 && num_seqs > 0) {
            if (!pool->block_table || !pool->seq_tokens) return KAMERA_ERR_NULL;
            if (((uintptr_t)pool->block_table & 3u) || ((uintptr_t)pool->seq_tokens & 3u)) return KAMERA_ERR_ALIGN;
        }
    }
    if (num_seqs == 0) return KAMERA_OK;
    if (!seq_entries || !q || !out) return KAMERA_ERR_NULL;
    if (num_entries > 0 && (!chunk_ids || !delta)) return KAMERA_ERR_NULL;
    if (!aligned16(q) || !aligned16(out) || ((uintptr_t)lse & 3u) || ((uintptr_t)error_word & 3u))
        return KAMERA_ERR_ALIGN;
    if ((int64_t)num_seqs * Hq > 65535LL * 65535LL || num_seqs > 65535) return KAMERA_ERR_RANGE;
    AttnPlan pl;
    attn_plan(L, Hq, num_entries, T, pool_T > 0 ? num_seqs : 0, pool_T, pl);
    if (pl.units > INT32_MAX) return KAMERA_ERR_RANGE;
    if (pl.total > 0) {
        if (!workspace) return KAMERA_ERR_NULL;
        if (((uintptr_t)workspace & 255u) != 0) return KAMERA_ERR_ALIGN;
        if (workspace_bytes < pl.total) return KAMERA_ERR_RANGE;
    }
    // outputs may not overlap each other, the workspace or any input
    {
        const Span os{(uintptr_t)out, (uintptr_t)out + (uintptr_t)((int64_t)num_seqs * Hq * Dv * 4)};
        const Span ls{(uintptr_t)lse, (uintptr_t)lse + (lse ? (uintptr_t)((int64_t)num_seqs * Hq * 4) : 0)};
        const Span ws{(uintptr_t)workspace, (uintptr_t)workspace + (uintptr_t)pl.total};
        const Span ew{(uintptr_t)error_word, (uintptr_t)error_word + (error_word ? 4u : 0u)};
        const int64_t c_el = (int64_t)(canon->n_store - 1) * canon->chunk_stride +
                             (int64_t)(L.num_layers - 1) * canon->layer_stride + (int64_t)T * F;
        Span ins[20];
        int ni = 0;
        if (pool_T > 0) {
            for (int s = 0; s < S; ++s) ins[ni++] = span_of(pool->rows[s], pool_el);
            ins[ni++] = Span{(uintptr_t)pool->block_table,
                             (uintptr_t)pool->block_table + (uintptr_t)((int64_t)num_seqs * pool->max_pages * 4)};
            ins[ni++] = Span{(uintptr_t)pool->seq_tokens, (uintptr_t)pool->seq_tokens + (uintptr_t)num_seqs * 4u};
        }
        for (int s = 0; s < S; ++s) ins[ni++] = span_of(canon->rows[s], c_el);
        ins[ni++] = Span{(uintptr_t)q, (uintptr_t)q + (uintptr_t)((int64_t)num_seqs * Hq * D * 2)};
        ins[ni++] = Span{(uintptr_t)seq_entries, (uintptr_t)seq_entries + (uintptr_t)(num_seqs + 1) * 4u};
        ins[ni++] = Span{(uintptr_t)chunk_ids, (uintptr_t)chunk_ids + (uintptr_t)num_entries * 4u};
        ins[ni++] = Span{(uintptr_t)delta, (uintptr_t)delta + (uintptr_t)num_entries * 8u};
        if (m > 0) {
            const int64_t u_el = (int64_t)canon->n_store * L.num_layers * T * m;
            const int64_t v_el = (int64_t)canon->n_store * L.num_layers * F * m;
            for (int s = 0; s < S; ++s) {
                ins[ni++] = span_of(patch->u[s], u_el);
                ins[ni++] = span_of(patch->v[s], v_el);
            }
        }
        const Span outs[4] = {os, ls, ws, ew};
        for (int a = 0; a < 4; ++a) {
            if (outs[a].lo == outs[a].hi) continue;
            for (int k = a + 1; k < 4; ++k)
                if (outs[k].lo != outs[k].hi && overlap(outs[a], outs[k])) return KAMERA_ERR_ALIAS;
            for (int k = 0; k < ni; ++k)
                if (ins[k].lo != ins[k].hi && overlap(outs[a], ins[k])) return KAMERA_ERR_ALIAS;
        }
    }

    AttnParams p;
    memset(&p, 0, sizeof(p));
    p.k_rows = canon->rows[0];
    p.v_rows = S > 1 ? canon->rows[1] : nullptr;
    p.chunk_stride = canon->chunk_stride;
    p.layer_stride = canon->layer_stride;
    if (m > 0) {
        p.uk = patch->u[0];
        p.vk = patch->v[0];
        p.uv = S > 1 ? patch->u[1] : nullptr;
        p.vv = S > 1 ? patch->v[1] : nullptr;
    }
    p.seq_entries = seq_entries;
    p.chunk_ids = chunk_ids;
    p.delta = delta;
    p.q = q;
    uint8_t* w = (uint8_t*)workspace;
    p.part_o = (float*)w;
    p.part_ml = (float2*)(w + pl.part_o_bytes);
    p.error_word = error_word;
    p.log2_base = log2(L.rope_base);
    p.qscale = scale * kLog2e;
    p.B = num_seqs;
    p.E = num_entries;
    p.layer = layer;
    p.L = L.num_layers;
    p.T = T;
    p.n_store = canon->n_store;
    p.Hkv = Hkv;
    p.Hq = Hq;
    p.G = Hq / Hkv;
    p.F = (int32_t)F;
    p.rope_offset = L.rope_offset;
    p.rope_dim = L.rope_dim;
    p.rope_style = L.rope_style;
    p.m = m;
    p.tiles = pl.tiles;
    p.tile_tokens = pl.tile_tokens;
    if (pool_T > 0) {
        p.pool_k = pool->rows[0];
        p.pool_v = S > 1 ? pool->rows[1] : nullptr;
        p.pool_layer_stride = pool->layer_stride;
        p.pool_table = pool->block_table;
        p.pool_tokens = pool->seq_tokens;
        p.pool_page = pool->page_size;
        p.pool_max_pages = pool->max_pages;
        p.pool_num_pages = (int32_t)(pool->num_slots / pool->page_size);
        p.pool_tiles = pl.pool_tiles;
        p.pool_tile_tokens = pl.pool_tile_tokens;
        p.pool_unit0 = pl.entry_units;
    }
    p.units = pl.units;

    hipStream_t hs = (hipStream_t)hip_stream;
    const CombineArgs ca{p.part_o, p.part_ml, seq_entries, out, lse, num_seqs, num_entries, pl.tiles, Hkv, Hq, p.G,
                         p.pool_tiles, p.pool_unit0, pl.units};
    hipError_t e;
    if (pl.mla) {
        e = launch_mla(m > 0, m, pl, Hq, num_seqs, hs, p, ca);
        return e == hipSuccess ? KAMERA_OK : KAMERA_ERR_HIP;
    }
    switch (D) {
        case 64: e = launch_attn<64>(m > 0, m, pl, Hkv, Hq, num_seqs, hs, p, ca); break;
        case 128: e = launch_attn<128>(m > 0, m, pl, Hkv, Hq, num_seqs, hs, p, ca); break;
        default: e = launch_attn<256>(m > 0, m, pl, Hkv, Hq, num_seqs, hs, p, ca); break;
    }
    return e == hipSuccess ? KAMERA_OK : KAMERA_ERR_HIP;
}

}  // namespace

extern "C" {

kamera_status kamera_decode_attention(const kamera_layout* layout, int32_t layer, const kamera_src* canon,
                                      const kamera_patch* patch, int32_t num_seqs, const int32_t* seq_entries,
                                      int32_t num_entries, const int32_t* chunk_ids, const int64_t* delta,
                                      int32_t num_q_heads, const uint16_t* q, float scale, float* out, float* lse,
                                      uint32_t* error_word, void* workspace, int64_t workspace_bytes,
                                      void* hip_stream) {
    return decode_attention(layout, layer, canon, patch, nullptr, num_seqs, seq_entries, num_entries, chunk_ids, delta,
                            num_q_heads, q, scale, out, lse, error_word, workspace, workspace_bytes, hip_stream);
}

kamera_status kamera_decode_attention_paged(const kamera_layout* layout, int32_t layer, const kamera_src* canon,
                                            const kamera_patch* patch, const kamera_attn_pool* pool,
                                            int32_t num_seqs, const int32_t* seq_entries, int32_t num_entries,
                                            const int32_t* chunk_ids, const int64_t* delta, int32_t num_q_heads,
                                            const uint16_t* q, float scale, float* out, float* lse,
                                            uint32_t* error_word, void* workspace, int64_t workspace_bytes,
                                            void* hip_stream) {
    if (!pool) return KAMERA_ERR_NULL;
    return decode_attention(layout, layer, canon, patch, pool, num_seqs, seq_entries, num_entries, chunk_ids, delta,
                            num_q_heads, q, scale, out, lse, error_word, workspace, workspace_bytes, hip_stream);
}

}  // extern "C"
