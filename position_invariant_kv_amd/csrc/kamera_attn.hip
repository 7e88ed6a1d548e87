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
// attn_split_kernel: one workgroup (4 waves) per (context entry, token tile,
// KV head).  A wave reads its tokens' K and V rows with D/8 lanes per row, 16
// bytes per lane (whole rows per instruction), takes each row's dot products
// with the G query heads of the KV head (sum over the row's lanes by
// butterfly shuffles) and keeps an online softmax in the log2 domain: running
// max, sum and output per head.  The four waves' partials are merged in LDS;
// the workgroup writes (max, sum, unnormalised output) per query head.
// attn_combine_kernel: per (sequence, query head), the log-sum-exp merge of
// every partial of the sequence's entries and tiles.

#include "kamera.h"
#include "kamera_common.h"

#include <string.h>

namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kAttnNit = 8;       // row groups per pass of a wave
constexpr int kMaxRank = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnParams {
    const uint16_t* k_rows;    // key stream of the store (chunk 0, layer 0)
    const uint16_t* v_rows;    // value stream
    int64_t k_chunk_stride, k_layer_stride;
    int64_t v_chunk_stride, v_layer_stride;
    const uint16_t* uk;        // patch factors (NULL when m == 0)
    const uint16_t* vk;
    const uint16_t* uv;
    const uint16_t* vv;
    const int32_t* seq_entries;  // [B + 1]
    const int32_t* chunk_ids;    // [E]
    const int64_t* delta;        // [E]
    const uint16_t* q;           // [B][Hq][D]
    float* part_o;               // [units][Hkv][G][D]
    float2* part_ml;             // [units][Hkv][G]: (max, sum), log2 domain
    uint32_t* error_word;
    double log2_base;
    float qscale;                // scale * log2(e)
    int32_t B, E, layer, L, T, n_store, Hkv, Hq, G, F, rope_offset, rope_dim, rope_style, m;
    int32_t tiles, tile_tokens;
};

__device__ __forceinline__ float bf_at(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }

template <int W>
__device__ __forceinline__ float row_sum(float x) {
    // sum over the W consecutive lanes of a row (W a power of two)
#pragma unroll
    for (int d = 1; d < W; d <<= 1) x += __shfl_xor(x, d);
    return x;
}

template <int W>
__device__ __forceinline__ float rows_max(float x) {
    // max over the rows of a wave (rows of W lanes): lanes c, c + W, c + 2W ...
#pragma unroll
    for (int d = W; d < 64; d <<= 1) x = fmaxf(x, __shfl_xor(x, d));
    return x;
}

template <int W>
__device__ __forceinline__ float rows_sum(float x) {
#pragma unroll
    for (int d = W; d < 64; d <<= 1) x += __shfl_xor(x, d);
    return x;
}

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

template <int D, int GT, bool PATCH>
__global__ __launch_bounds__(kAttnThreads) void attn_split_kernel(const AttnParams p) {
    constexpr int LPR = D / 8;         // lanes per row (16 bytes each)
    constexpr int RPI = 64 / LPR;      // rows per wave instruction
    constexpr int PASS = RPI * kAttnNit;
    __shared__ float qs[GT][D];                  // R(-delta) q, scaled to log2 units
    __shared__ float ws[GT][kMaxRank];           // V_K^T q, scaled
    __shared__ float red_o[kAttnWaves][GT][D];
    __shared__ float red_u[PATCH ? kAttnWaves : 1][GT][kMaxRank];
    __shared__ float red_m[kAttnWaves][GT];
    __shared__ float red_l[kAttnWaves][GT];
    __shared__ float um[GT][kMaxRank];           // merged value-patch weights

    const int unit = blockIdx.x;
    const int g = blockIdx.y;
    const int e = unit / p.tiles;
    const int tile = unit - e * p.tiles;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane / LPR, c = lane % LPR;
    const int b = seq_of_entry(p.seq_entries, p.B, e);
    const int cid = ld_uniform(p.chunk_ids + e);
    const int64_t delta = ld_uniform(p.delta + e);
    const int64_t pidx = ((int64_t)unit * p.Hkv + g) * GT;  // first partial of this workgroup
    const bool chunk_ok = cid >= 0 && cid < p.n_store;
    if (!chunk_ok) {  // uniform: this entry contributes nothing
        if (tid < GT) p.part_ml[pidx + tid] = make_float2(-INFINITY, 0.0f);
        if (tid == 0 && p.error_word && tile == 0) atomicOr(p.error_word, (uint32_t)KAMERA_EW_CHUNK);
        return;
    }

    // ---- the query turned by R(-delta), and w = V_K^T q (unturned), per head
    const uint16_t* qb = p.q + ((int64_t)b * p.Hq + (int64_t)g * p.G) * D;
    for (int i = tid; i < GT * D; i += kAttnThreads) {
        const int h = i / D, d = i % D;
        float x = 0.0f;
        if (h < p.G) {
            const uint16_t* qh = qb + h * D;
            x = bf_at(qh + d);
            const int dd = d - p.rope_offset;
            if (dd >= 0 && dd < p.rope_dim) {
                int jj, partner;
                float sg;
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
                const float2 cs = rope_cos_sin(p.log2_base, p.rope_dim, jj, delta);
                x = fmaf(x, cs.x, sg * bf_at(qh + partner) * cs.y);
            }
        }
        qs[h][d] = x * p.qscale;
    }
    const int64_t blk = (int64_t)cid * p.L + p.layer;  // (chunk, layer) block of the factors
    if (PATCH) {
        const uint16_t* vkh = p.vk + (blk * p.F + (int64_t)g * D) * p.m;
        for (int i = tid; i < GT * p.m; i += kAttnThreads) {
            const int h = i / p.m, k = i % p.m;
            float acc = 0.0f;
            if (h < p.G) {
                const uint16_t* qh = qb + h * D;
                for (int d = 0; d < D; ++d) acc = fmaf(bf_at(vkh + (int64_t)d * p.m + k), bf_at(qh + d), acc);
            }
            ws[h][k] = acc * p.qscale;
        }
    }
    __syncthreads();
    float qr[GT][8];
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
        for (int x = 0; x < 8; ++x) qr[h][x] = qs[h][8 * c + x];
    const bool plane = PATCH && 8 * c < p.m;  // this lane carries 8 of the m patch columns
    float wr[PATCH ? GT : 1][8];
    if (PATCH) {
#pragma unroll
        for (int h = 0; h < GT; ++h)
#pragma unroll
            for (int x = 0; x < 8; ++x) wr[h][x] = plane ? ws[h][8 * c + x] : 0.0f;
    }

    // ---- this wave's tokens
    const int per_wave = p.tile_tokens / kAttnWaves;
    const int wt0 = tile * p.tile_tokens + wave * per_wave;
    const int wt1 = min(p.T, wt0 + per_wave);
    const uint16_t* kb = p.k_rows + cid * p.k_chunk_stride + p.layer * p.k_layer_stride + (int64_t)g * D + 8 * c;
    const uint16_t* vb = p.v_rows + cid * p.v_chunk_stride + p.layer * p.v_layer_stride + (int64_t)g * D + 8 * c;
    const uint16_t* ukb = PATCH ? p.uk + blk * p.T * p.m + 8 * c : nullptr;
    const uint16_t* uvb = PATCH ? p.uv + blk * p.T * p.m + 8 * c : nullptr;

    float mrun[GT], lrun[GT], o[GT][8], ua[PATCH ? GT : 1][8];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
        mrun[h] = -INFINITY;
        lrun[h] = 0.0f;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
            o[h][x] = 0.0f;
            if (PATCH) ua[h][x] = 0.0f;
        }
    }
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int t0 = wt0; t0 < wt1; t0 += PASS) {
        u32x4 kv[kAttnNit], vv[kAttnNit], ukv[PATCH ? kAttnNit : 1], uvv[PATCH ? kAttnNit : 1];
#pragma unroll
        for (int it = 0; it < kAttnNit; ++it) {
            const int t = t0 + it * RPI + r;
            const bool valid = t < wt1;
            kv[it] = valid ? ld_stream(kb + (int64_t)t * p.F) : zero;
            vv[it] = valid ? ld_stream(vb + (int64_t)t * p.F) : zero;
            if (PATCH) {
                ukv[it] = valid && plane ? ld_cached(ukb + (int64_t)t * p.m) : zero;
                uvv[it] = valid && plane ? ld_cached(uvb + (int64_t)t * p.m) : zero;
            }
        }
        // logits of this lane's row, every head (log2 units)
        float s[kAttnNit][GT];
#pragma unroll
        for (int it = 0; it < kAttnNit; ++it) {
            float kf[8];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                kf[2 * w] = bf_lo(kv[it][w]);
                kf[2 * w + 1] = bf_hi(kv[it][w]);
            }
            float uf[8];
            if (PATCH) {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    uf[2 * w] = bf_lo(ukv[it][w]);
                    uf[2 * w + 1] = bf_hi(ukv[it][w]);
                }
            }
            const bool valid = t0 + it * RPI + r < wt1;
#pragma unroll
            for (int h = 0; h < GT; ++h) {
                float acc = 0.0f;
#pragma unroll
                for (int x = 0; x < 8; ++x) acc = fmaf(kf[x], qr[h][x], acc);
                if (PATCH) {
#pragma unroll
                    for (int x = 0; x < 8; ++x) acc = fmaf(uf[x], wr[h][x], acc);
                }
                acc = row_sum<LPR>(acc);
                s[it][h] = valid ? acc : -INFINITY;
            }
        }
#pragma unroll
        for (int h = 0; h < GT; ++h) {
            float mx = s[0][h];
#pragma unroll
            for (int it = 1; it < kAttnNit; ++it) mx = fmaxf(mx, s[it][h]);
            mx = rows_max<LPR>(mx);
            const float mn = fmaxf(mrun[h], mx);
            if (mn == -INFINITY) continue;  // no valid token yet (uniform over the wave)
            const float alpha = exp2f(mrun[h] - mn);  // 0 when mrun is -inf
            mrun[h] = mn;
            lrun[h] *= alpha;
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                o[h][x] *= alpha;
                if (PATCH) ua[h][x] *= alpha;
            }
#pragma unroll
            for (int it = 0; it < kAttnNit; ++it) {
                const float pp = exp2f(s[it][h] - mn);  // 0 for invalid rows
                lrun[h] += pp;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    o[h][2 * w] = fmaf(pp, bf_lo(vv[it][w]), o[h][2 * w]);
                    o[h][2 * w + 1] = fmaf(pp, bf_hi(vv[it][w]), o[h][2 * w + 1]);
                    if (PATCH) {
                        ua[h][2 * w] = fmaf(pp, bf_lo(uvv[it][w]), ua[h][2 * w]);
                        ua[h][2 * w + 1] = fmaf(pp, bf_hi(uvv[it][w]), ua[h][2 * w + 1]);
                    }
                }
            }
        }
    }
    // ---- wave totals (sum over the rows), then the workgroup's merge
#pragma unroll
    for (int h = 0; h < GT; ++h) {
        lrun[h] = rows_sum<LPR>(lrun[h]);
#pragma unroll
        for (int x = 0; x < 8; ++x) {
            o[h][x] = rows_sum<LPR>(o[h][x]);
            if (PATCH) ua[h][x] = rows_sum<LPR>(ua[h][x]);
        }
    }
    if (r == 0) {
#pragma unroll
        for (int h = 0; h < GT; ++h) {
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                red_o[wave][h][8 * c + x] = o[h][x];
                if (PATCH && plane) red_u[wave][h][8 * c + x] = ua[h][x];
            }
            if (c == 0) {
                red_m[wave][h] = mrun[h];
                red_l[wave][h] = lrun[h];
            }
        }
    }
    __syncthreads();
    if (PATCH) {
        for (int i = tid; i < GT * p.m; i += kAttnThreads) {
            const int h = i / p.m, k = i % p.m;
            float M = red_m[0][h];
#pragma unroll
            for (int w = 1; w < kAttnWaves; ++w) M = fmaxf(M, red_m[w][h]);
            float acc = 0.0f;
            if (M != -INFINITY) {
#pragma unroll
                for (int w = 0; w < kAttnWaves; ++w)
                    if (red_m[w][h] != -INFINITY) acc = fmaf(red_u[w][h][k], exp2f(red_m[w][h] - M), acc);
            }
            um[h][k] = acc;
        }
        __syncthreads();
    }
    const uint16_t* vvh = PATCH ? p.vv + (blk * p.F + (int64_t)g * D) * p.m : nullptr;
    for (int i = tid; i < GT * D; i += kAttnThreads) {
        const int h = i / D, d = i % D;
        float M = red_m[0][h];
#pragma unroll
        for (int w = 1; w < kAttnWaves; ++w) M = fmaxf(M, red_m[w][h]);
        float acc = 0.0f, lsum = 0.0f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kAttnWaves; ++w) {
                if (red_m[w][h] == -INFINITY) continue;
                const float f = exp2f(red_m[w][h] - M);
                acc = fmaf(red_o[w][h][d], f, acc);
                lsum = fmaf(red_l[w][h], f, lsum);
            }
            if (PATCH) {
                const uint16_t* vrow = vvh + (int64_t)d * p.m;
                for (int k = 0; k < p.m; ++k) acc = fmaf(bf_at(vrow + k), um[h][k], acc);
            }
        }
        p.part_o[(pidx + h) * D + d] = acc;
        if (d == 0) p.part_ml[pidx + h] = make_float2(M, lsum);
    }
}

struct CombineArgs {
    const float* part_o;
    const float2* part_ml;
    const int32_t* seq_entries;
    float* out;
    float* lse;
    int32_t B, E, tiles, Hkv, Hq, G, GT;
};

template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(const CombineArgs a) {
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const int g = h / a.G, hl = h - g * a.G;
    int e0 = ld_uniform(a.seq_entries + b), e1 = ld_uniform(a.seq_entries + b + 1);
    e0 = min(max(e0, 0), a.E);
    e1 = min(max(e1, e0), a.E);
    float M = -INFINITY, L = 0.0f, O = 0.0f;
    for (int64_t u = (int64_t)e0 * a.tiles; u < (int64_t)e1 * a.tiles; ++u) {
        const int64_t idx = (u * a.Hkv + g) * a.GT + hl;
        const float2 ml = a.part_ml[idx];
        if (ml.x == -INFINITY) continue;
        const float mn = fmaxf(M, ml.x);
        const float fa = exp2f(M - mn), fb = exp2f(ml.x - mn);
        O = fmaf(O, fa, a.part_o[idx * D + d] * fb);
        L = fmaf(L, fa, ml.y * fb);
        M = mn;
    }
    const int64_t oi = (int64_t)b * a.Hq + h;
    a.out[oi * D + d] = L > 0.0f ? O / L : 0.0f;
    if (d == 0 && a.lse) a.lse[oi] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

int group_template(int G) { return G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8; }

struct AttnPlan {
    int tiles, tile_tokens, GT;
    int64_t units, part_o_bytes, part_ml_bytes, total;
};

inline int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

// Token tiles: whole passes of every wave, as long as the grid has at least
// ~2048 workgroups; at least one pass per wave.
bool attn_plan(const kamera_layout& L, int Hq, int E, int T, AttnPlan& pl) {
    const int D = L.head_dim;
    const int pass = (64 / (D / 8)) * kAttnNit;
    const int G = Hq / L.num_heads;
    pl.GT = group_template(G);
    int passes = 1;
    const int64_t per_tile_min = (int64_t)kAttnWaves * pass;
    while (passes < 8) {
        const int64_t tt = per_tile_min * passes * 2;
        const int64_t tiles = (T + tt - 1) / tt;
        if ((int64_t)E * tiles * L.num_heads < 2048) break;
        passes *= 2;
    }
    pl.tile_tokens = (int)(per_tile_min * passes);
    pl.tiles = T > 0 ? (T + pl.tile_tokens - 1) / pl.tile_tokens : 0;
    pl.units = (int64_t)E * pl.tiles;
    const int64_t parts = pl.units * L.num_heads * pl.GT;
    pl.part_o_bytes = align256(parts * D * 4);
    pl.part_ml_bytes = align256(parts * 8);
    pl.total = pl.part_o_bytes + pl.part_ml_bytes;
    return true;
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
    if (L->num_streams != 2) return KAMERA_ERR_UNSUPPORTED;
    if (L->head_dim != 64 && L->head_dim != 128 && L->head_dim != 256) return KAMERA_ERR_UNSUPPORTED;
    if (Hq / L->num_heads > 8 || L->num_heads > 65535) return KAMERA_ERR_UNSUPPORTED;
    if ((int64_t)L->num_heads * L->head_dim > 4096) return KAMERA_ERR_UNSUPPORTED;
    return KAMERA_OK;
}

template <int D, int GT, bool PATCH>
hipError_t launch_split(dim3 grid, hipStream_t s, const AttnParams& p) {
    return launch_kernel(attn_split_kernel<D, GT, PATCH>, grid, dim3(kAttnThreads), s, p);
}

template <int D, bool PATCH>
hipError_t launch_split_g(int GT, dim3 grid, hipStream_t s, const AttnParams& p) {
    switch (GT) {
        case 1: return launch_split<D, 1, PATCH>(grid, s, p);
        case 2: return launch_split<D, 2, PATCH>(grid, s, p);
        case 4: return launch_split<D, 4, PATCH>(grid, s, p);
        default: return launch_split<D, 8, PATCH>(grid, s, p);
    }
}

template <int D>
hipError_t launch_split_d(bool patch, int GT, dim3 grid, hipStream_t s, const AttnParams& p) {
    return patch ? launch_split_g<D, true>(GT, grid, s, p) : launch_split_g<D, false>(GT, grid, s, p);
}

}  // namespace

extern "C" {

int64_t kamera_decode_attention_workspace(const kamera_layout* layout, int32_t num_q_heads, int32_t num_entries,
                                          int32_t n_tokens) {
    if (check_attn_layout(layout, num_q_heads) != KAMERA_OK || num_entries < 0 || n_tokens < 0) return -1;
    AttnPlan pl;
    attn_plan(*layout, num_q_heads, num_entries, n_tokens, pl);
    return pl.total;
}

kamera_status kamera_decode_attention(const kamera_layout* layout, int32_t layer, const kamera_src* canon,
                                      const kamera_patch* patch, int32_t num_seqs, const int32_t* seq_entries,
                                      int32_t num_entries, const int32_t* chunk_ids, const int64_t* delta,
                                      int32_t num_q_heads, const uint16_t* q, float scale, float* out, float* lse,
                                      uint32_t* error_word, void* workspace, int64_t workspace_bytes,
                                      void* hip_stream) {
    kamera_status st = check_attn_layout(layout, num_q_heads);
    if (st != KAMERA_OK) return st;
    const kamera_layout& L = *layout;
    if (!canon) return KAMERA_ERR_NULL;
    if (layer < 0 || layer >= L.num_layers) return KAMERA_ERR_RANGE;
    if (num_seqs < 0 || num_entries < 0) return KAMERA_ERR_RANGE;
    if (!(scale == scale) || isinf(scale)) return KAMERA_ERR_RANGE;
    const int D = L.head_dim, Hkv = L.num_heads, Hq = num_q_heads;
    const int64_t F = (int64_t)Hkv * D;
    const int T = canon->n_tokens;
    if (T < 0 || canon->n_store < 1) return KAMERA_ERR_RANGE;
    for (int s = 0; s < 2; ++s) {
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
        for (int s = 0; s < 2; ++s) {
            if (!patch->u[s] || !patch->v[s]) return KAMERA_ERR_NULL;
            if (!aligned16(patch->u[s]) || !aligned16(patch->v[s])) return KAMERA_ERR_ALIGN;
        }
    }
    if (num_seqs == 0) return KAMERA_OK;
    if (!seq_entries || !q || !out) return KAMERA_ERR_NULL;
    if (num_entries > 0 && (!chunk_ids || !delta)) return KAMERA_ERR_NULL;
    if (!aligned16(q) || !aligned16(out) || ((uintptr_t)lse & 3u) || ((uintptr_t)error_word & 3u))
        return KAMERA_ERR_ALIGN;
    if ((int64_t)num_seqs * Hq > 65535LL * 65535LL || num_seqs > 65535) return KAMERA_ERR_RANGE;
    AttnPlan pl;
    attn_plan(L, Hq, num_entries, T, pl);
    if (pl.units > INT32_MAX) return KAMERA_ERR_RANGE;
    if (pl.total > 0) {
        if (!workspace) return KAMERA_ERR_NULL;
        if (((uintptr_t)workspace & 255u) != 0) return KAMERA_ERR_ALIGN;
        if (workspace_bytes < pl.total) return KAMERA_ERR_RANGE;
    }
    // outputs may not overlap each other, the workspace or any input
    {
        const Span os{(uintptr_t)out, (uintptr_t)out + (uintptr_t)((int64_t)num_seqs * Hq * D * 4)};
        const Span ls{(uintptr_t)lse, (uintptr_t)lse + (lse ? (uintptr_t)((int64_t)num_seqs * Hq * 4) : 0)};
        const Span ws{(uintptr_t)workspace, (uintptr_t)workspace + (uintptr_t)pl.total};
        const Span ew{(uintptr_t)error_word, (uintptr_t)error_word + (error_word ? 4u : 0u)};
        const int64_t c_el = (int64_t)(canon->n_store - 1) * canon->chunk_stride +
                             (int64_t)(L.num_layers - 1) * canon->layer_stride + (int64_t)T * F;
        Span ins[12];
        int ni = 0;
        ins[ni++] = span_of(canon->rows[0], c_el);
        ins[ni++] = span_of(canon->rows[1], c_el);
        ins[ni++] = Span{(uintptr_t)q, (uintptr_t)q + (uintptr_t)((int64_t)num_seqs * Hq * D * 2)};
        ins[ni++] = Span{(uintptr_t)seq_entries, (uintptr_t)seq_entries + (uintptr_t)(num_seqs + 1) * 4u};
        ins[ni++] = Span{(uintptr_t)chunk_ids, (uintptr_t)chunk_ids + (uintptr_t)num_entries * 4u};
        ins[ni++] = Span{(uintptr_t)delta, (uintptr_t)delta + (uintptr_t)num_entries * 8u};
        if (m > 0) {
            const int64_t u_el = (int64_t)canon->n_store * L.num_layers * T * m;
            const int64_t v_el = (int64_t)canon->n_store * L.num_layers * F * m;
            for (int s = 0; s < 2; ++s) {
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
    p.v_rows = canon->rows[1];
    p.k_chunk_stride = p.v_chunk_stride = canon->chunk_stride;
    p.k_layer_stride = p.v_layer_stride = canon->layer_stride;
    if (m > 0) {
        p.uk = patch->u[0];
        p.vk = patch->v[0];
        p.uv = patch->u[1];
        p.vv = patch->v[1];
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

    hipStream_t hs = (hipStream_t)hip_stream;
    hipError_t e = hipSuccess;
    if (pl.units > 0) {
        const dim3 grid((unsigned)pl.units, (unsigned)Hkv);
        switch (D) {
            case 64: e = launch_split_d<64>(m > 0, pl.GT, grid, hs, p); break;
            case 128: e = launch_split_d<128>(m > 0, pl.GT, grid, hs, p); break;
            default: e = launch_split_d<256>(m > 0, pl.GT, grid, hs, p); break;
        }
    }
    if (e == hipSuccess) {
        CombineArgs ca{p.part_o, p.part_ml, seq_entries, out, lse, num_seqs, num_entries, pl.tiles, Hkv, Hq,
                       p.G, pl.GT};
        const dim3 grid((unsigned)Hq, (unsigned)num_seqs);
        switch (D) {
            case 64: e = launch_kernel(attn_combine_kernel<64>, grid, dim3(64), hs, ca); break;
            case 128: e = launch_kernel(attn_combine_kernel<128>, grid, dim3(128), hs, ca); break;
            default: e = launch_kernel(attn_combine_kernel<256>, grid, dim3(256), hs, ca); break;
        }
    }
    return e == hipSuccess ? KAMERA_OK : KAMERA_ERR_HIP;
}

}  // extern "C"
