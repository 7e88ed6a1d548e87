// kamera_form.hip — Kamera patch formation on MI355X (gfx950): the rank-m
// factors of the deficit Delta = KV(B|A) - R(delta) KV(B|empty), for every
// (chunk, layer, stream) block of a call (include/kamera.h, kamera_form_patch).
//
// Kamera summary on gist.science (paper 2606.23581), section 2, "Patch
// application": the patch is computed once by a forward pass on [A, B]
// followed by an SVD that keeps the top-m factors.  The forward pass is the
// caller's; this file computes the SVD part with randomized subspace
// iteration (Halko, Martinsson & Tropp, "Finding structure with randomness",
// SIAM Review 2011: Algorithm 4.4 for the range, Algorithm 5.1 for the
// factors), k = m + p sketch columns, q power iterations:
//
//   Y = Delta Omega; Q = orth(Y)
//   q times: Z = orth(Delta^T Q); Q = orth(Delta Z)
//   Z = Delta^T Q (= B^T with B = Q^T Delta); B B^T = W L W^T
//   U = Q W_m L_m^(1/2),  V = Z W_m L_m^(-1/2)
//
// Kernels, one launch each, every block of the call at once:
//  * delta_kernel: Delta in fp32 from the bf16 rows (relocation exactly as the
//    reuse kernels do it), split into a bf16 high part and a bf16 low part
//    (Delta - hi), stored row-major [Tp][F] in panels 64 features wide, each
//    panel row its 64 high parts then its 64 low parts ([F/64][Tp][2][64]): a
//    chunk of 64 features of 128 tokens (Delta Z) or of 64 tokens of 128
//    features (Delta^T Q) is one 32 KB or two 16 KB pieces, high and low
//    parts together.
//  * sketch_kernel: out[R][kp] = A[R][X] B[X][kp] on v_mfma_f32_32x32x16_bf16
//    with A = hi + lo (two products, or three with a split B): Delta Omega,
//    Delta Z and Delta^T Q (A = Delta^T through transposing LDS reads).
//  * delta_sketch_kernel (one view): Delta Omega with Delta formed as
//    delta_kernel forms it, stored, and multiplied on the way, so the range
//    finder's first product costs no pass over Delta; calls with several
//    views (orbit patches) run delta_kernel, then sketch_kernel.
//  * orthonormalization of X [R][kp] (Y or Z), shifted Cholesky QR twice:
//    the fp64 Gram matrix X^T X comes from the kernel that wrote X (summed
//    atomically over its workgroups); chol_lds_kernel (four waves per block:
//    Cholesky and R^-1); apply_kernel (X <- X R^-1, then the next Gram
//    matrix or the bf16 transpose the next product reads);
//  * eig_kernel: B B^T = Z^T Z by cyclic Jacobi (fp64, one workgroup per
//    block), then the oracle's conventions (V column's largest entry
//    positive, singular values <= 1e-6 sigma_1 give zero columns);
//  * out_kernel: U = Q (W sigma) and V = Z (W / sigma) in bf16.
// The Jacobi method uses the round-robin parallel ordering (Golub & Van
// Loan, Matrix Computations, sections 8.5.2 and 8.5.5).

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <type_traits>

#include "kamera.h"
#include "kamera_common.h"

namespace {

constexpr int kFormThreads = 256;
constexpr int kMaxKp = 64;            // sketch columns after padding (32 or 64)
constexpr int kMaxHalfRopeF = 512;
constexpr int kTileT = 64;            // delta_kernel tile: 64 tokens x 64 features
constexpr double kDropL = 1e-13;      // SVQB: eigenvalues <= kDropL * L_max are dropped
constexpr double kNegligible = 1e-6;  // factors: sigma <= kNegligible * sigma_1 -> zero column
constexpr int kMaxSweeps = 20;

struct FormParams {
    const uint16_t* canon[2];
    int64_t canon_chunk_stride, canon_layer_stride;
    const uint16_t* target[2];
    int64_t target_chunk_stride, target_layer_stride;
    const int64_t* delta;
    const uint16_t* omega;  // [k][F] bf16 test matrix, shared by every block
    uint16_t* u[2];         // [n][L][T][m]
    uint16_t* v[2];         // [n][L][F][m]
    // workspace, per block
    uint16_t *dr_hi, *dr_lo;  // [F/64][Tp][2][64]: dr_lo = dr_hi + 64
    float* y;                 // [Tp][kp]
    uint16_t *qt_hi, *qt_lo;  // [kp][Tp]
    float* z;                 // [F][kp]
    uint16_t* zt_hi;          // [kp][F]
    double* g;                // [kp][kp] fp64 Gram matrix
    float* mm;                // [kp][kp] R^-1
    float *wu, *wv;           // [kp][m]
    double log2_base;
    int32_t n, L, S, T, Tp, F, D, rope_offset, rope_dim, rope_style;
    int32_t m, k, kp;
    int32_t views;            // targets (and shifts) per chunk: view v of chunk i is i * views + v
};

__device__ __forceinline__ int64_t block_of(const FormParams& p, int i, int s, int l) {
    return ((int64_t)i * p.S + s) * p.L + l;
}

// bf16 high part and low part (x - hi) of eight fp32 values, as two 16-byte vectors.
__device__ __forceinline__ void split8(const float (&x)[8], u32x4& hi, u32x4& lo) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t h = pack_bf16x2(x[2 * q], x[2 * q + 1]);
        hi[q] = h;
        lo[q] = pack_bf16x2(x[2 * q] - bf_lo(h), x[2 * q + 1] - bf_hi(h));
    }
}

// One view's contribution to eight consecutive deficit features: d += target
// - R(delta) canon, where cv holds the canonical features, pv their
// rotate-half partners (unused otherwise), tv the target features and cs the
// view's cos/sin table; e is the first feature's place in the rotary span,
// rv whether the vector is rotated and first whether it lies in the span's
// first half.  Rows past T (ok false) add nothing.
__device__ __forceinline__ void delta_add8(float (&d)[8], const u32x4 cv, const u32x4 pv, const u32x4 tv,
                                           const float2* cs, const int e, const bool rv, const bool first,
                                           const int half, const int style, const bool ok) {
    float c8[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        c8[2 * w] = bf_lo(cv[w]);
        c8[2 * w + 1] = bf_hi(cv[w]);
    }
    if (rv) {
        if (style == KAMERA_ROPE_HALF) {
            const int j0 = first ? e : e - half;
            const float sg = first ? -1.0f : 1.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float2 a = cs[j0 + 2 * w], bb = cs[j0 + 2 * w + 1];
                const float x0 = c8[2 * w], x1 = c8[2 * w + 1];
                c8[2 * w] = fmaf(x0, a.x, sg * bf_lo(pv[w]) * a.y);
                c8[2 * w + 1] = fmaf(x1, bb.x, sg * bf_hi(pv[w]) * bb.y);
            }
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float2 a = cs[(e >> 1) + w];
                const float A = c8[2 * w], B = c8[2 * w + 1];
                c8[2 * w] = fmaf(A, a.x, -B * a.y);
                c8[2 * w + 1] = fmaf(B, a.x, A * a.y);
            }
        }
    }
    if (ok) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            d[2 * w] += bf_lo(tv[w]) - c8[2 * w];
            d[2 * w + 1] += bf_hi(tv[w]) - c8[2 * w + 1];
        }
    }
}

// ---------------------------------------------------------------------------
// Delta = target - R(delta) canon, split hi/lo, in 64-feature panels
// ---------------------------------------------------------------------------
//
// Grid: x = token tile * (F/64) + feature tile, y = layer, z = chunk * S +
// stream.  A 256-thread workgroup owns 64 tokens x 64 features: each thread
// forms two 8-feature vectors (loading the rotate-half partner vector of the
// canonical row when the feature is rotated) and stores them in the panel of
// its 64 features: the tile's high and low parts are 16 KB in one piece.
// Rows past T are zero.
__global__ __launch_bounds__(kFormThreads) void delta_kernel(const FormParams p) {
    __shared__ float2 cs[kMaxHalfRopeF];
    const int ftiles = p.F / 64;
    const int tt = (int)blockIdx.x / ftiles;
    const int ft = (int)blockIdx.x - tt * ftiles;
    const int l = blockIdx.y;
    const int z = blockIdx.z;
    const int s = p.S == 2 ? (z & 1) : 0;
    const int i = p.S == 2 ? (z >> 1) : z;
    const int64_t b = block_of(p, i, s, l);
    const int t0 = tt * kTileT, f0 = ft * 64;
    const bool rot = s == 0 && p.rope_dim > 0;
    const int half = p.rope_dim >> 1;
    const uint16_t* cb = p.canon[s] + (int64_t)i * p.canon_chunk_stride + (int64_t)l * p.canon_layer_stride;
    uint16_t* drh = p.dr_hi + b * p.Tp * p.F * 2;  // rows of 64 high then 64 low parts
    // This thread's two 8-feature vectors: their canonical rows (and rotate-half
    // partners) are the same for every view, so they are loaded once, before
    // anything else; each view's target rows are issued before its cos/sin
    // table is built, so the table's arithmetic overlaps the loads.  Loads are
    // unconditional (rows past T re-read row T - 1 and are not used).
    int tt_[2], f_[2], e_[2];
    bool ok_[2], rv_[2], first_[2];
    u32x4 cvv[2], pvv[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int q = threadIdx.x + kk * kFormThreads;
        const int r = q >> 3, cv = q & 7;
        ok_[kk] = t0 + r < p.T;
        tt_[kk] = min(t0 + r, p.T - 1);
        f_[kk] = f0 + 8 * cv;
        e_[kk] = (f_[kk] % p.D) - p.rope_offset;  // vector start inside the rotary span
        rv_[kk] = rot && e_[kk] >= 0 && e_[kk] < p.rope_dim;
        first_[kk] = e_[kk] < half;
        const int poff = (rv_[kk] && p.rope_style == KAMERA_ROPE_HALF) ? (first_[kk] ? half : -half) : 0;
        cvv[kk] = ld_cached(cb + (int64_t)tt_[kk] * p.F + f_[kk]);
        pvv[kk] = ld_cached(cb + (int64_t)tt_[kk] * p.F + f_[kk] + poff);
    }
    float d[2][8];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int w = 0; w < 8; ++w) d[kk][w] = 0.0f;
    for (int vw = 0; vw < p.views; ++vw) {
        const int iv = i * p.views + vw;
        const uint16_t* tb = p.target[s] + (int64_t)iv * p.target_chunk_stride + (int64_t)l * p.target_layer_stride;
        u32x4 tv[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) tv[kk] = ld_cached(tb + (int64_t)tt_[kk] * p.F + f_[kk]);
        // each view has its own shift, so its own cos/sin table (built between
        // two barriers)
        if (rot) {
            const int64_t delta = p.delta[iv];
            for (int j = threadIdx.x; j < half; j += kFormThreads)
                cs[j] = rope_cos_sin(p.log2_base, p.rope_dim, j, delta);
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            delta_add8(d[kk], cvv[kk], pvv[kk], tv[kk], cs, e_[kk], rv_[kk], first_[kk], half, p.rope_style, ok_[kk]);
        __syncthreads();  // the next view's table overwrites cs
    }
    const float inv_views = 1.0f / (float)p.views;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int q = threadIdx.x + kk * kFormThreads;
        const int r = q >> 3, cv = q & 7;
        const int t = t0 + r;
        const int f = f0 + 8 * cv;
        float dd[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) dd[w] = p.views == 1 ? d[kk][w] : d[kk][w] * inv_views;
        u32x4 h, lo;
        split8(dd, h, lo);
        // panel ft: [Tp][2][64], this tile's 64 rows (high and low parts)
        // are 16 KB in one piece
        const int64_t ro = (int64_t)ft * p.Tp * 128 + (int64_t)t * 128 + (f - f0);
        *reinterpret_cast<u32x4*>(drh + ro) = h;
        *reinterpret_cast<u32x4*>(drh + ro + 64) = lo;
    }
}

// ---------------------------------------------------------------------------
// out[R][kp] = (A_hi + A_lo)[R][X] B[X][kp], A in 64-wide panels whose rows
// hold 64 high then 64 low parts ([X/64][R][2][64]; a_lo = a_hi + 64), B
// given transposed: bt[kp][X]
// ---------------------------------------------------------------------------
//
// v_mfma_f32_32x32x16_bf16: lane l holds A[l%32][8(l/32) .. +8] and
// B[8(l/32) .. +8][l%32]; its 16 results are D[8(v/4) + 4(l/32) + v%4][l%32].
// A workgroup of four waves owns 128 rows and all kp = 32 KC columns: chunks
// of 64 inner values of A (high and low parts) and of B go through LDS with
// whole-line coalesced loads (the next chunk's loads in flight during the
// current chunk's products), and each wave multiplies its own 32 rows.  Columns of B at or past nb_valid read as zero.  With
// a low part of B the product adds hi*lo_B as well (three products).  With g
// non-NULL, the workgroup also adds its rows' Gram matrix out^T out (fp64)
// into g (atomically; g cleared beforehand), for the orthonormalization.
struct SketchArgs {
    const uint16_t* a_hi;
    const uint16_t* a_lo;
    int64_t a_block;        // elements between blocks of A
    const uint16_t* bt_hi;
    const uint16_t* bt_lo;  // may be NULL
    int64_t bt_block;       // elements between blocks of B (0: shared)
    float* out;
    int64_t out_block;
    double* g;              // may be NULL: [blocks][kp][kp]
    int32_t R, X;           // rows, inner length (multiple of 16)
    int32_t nb_valid;       // columns of B that exist (others are zero)
    int32_t row_tiles;      // 128-row tiles per workgroup
};

// The Gram matrix X^T X of 128-row tiles xs (fp32, LDS), accumulated in fp64
// on the matrix cores (v_mfma_f64_16x16x4f64, exact products, fp64 sums).
// Only its lower 16 x 16 tiles are formed, (ti, tj) with ti >= tj, numbered
// n = ti (ti + 1) / 2 + tj: the matrix is symmetric, its readers take the
// lower triangle (with the diagonal), and the tiles above it stay as
// cleared.  Wave w owns tiles w, w + 4, ... over every row of the tile; per
// step of 4 rows, lane (n16, q4) feeds row 4s + q4, column 16 ti + n16 as A
// (X^T) and column 16 tj + n16 as B (X), and holds rows q4, q4 + 4, q4 + 8,
// q4 + 12, column n16 of its tiles (the fp64 product's result order, checked
// on MI355X: it differs from the fp32 16x16x4 product's 4 q4 + i).
typedef double f64x4 __attribute__((ext_vector_type(4)));
template <int KP>
struct GramTiles {
    static constexpr int NT = (KP / 16) * (KP / 16 + 1) / 2;  // lower tiles
    static constexpr int PER = (NT + 3) / 4;                  // per wave
};
__device__ __forceinline__ void lower_tile(int n, int& ti, int& tj) {
    ti = 0;
    while ((ti + 1) * (ti + 2) / 2 <= n) ++ti;
    tj = n - ti * (ti + 1) / 2;
}
template <int KP, int PITCH = KP + 1>
__device__ __forceinline__ void gram_tile_acc(const float (*xs)[PITCH], int rows,
                                              f64x4 (&acc)[GramTiles<KP>::PER]) {
    constexpr int NT = GramTiles<KP>::NT, PER = GramTiles<KP>::PER;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int n16 = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        // 64 columns (10 lower tiles): tiles wave and wave + 4 whole, and half
        // the steps of tile 8 + wave / 2, so every wave runs 80 steps instead
        // of 96, 96, 64, 64 (on MI355X, MLA formation -0.1 ms; the two halves
        // of tiles 8 and 9 meet in the atomics)
        const bool split = KP == 64 && u == 2;
        const int n = split ? 8 + (wave >> 1) : wave + 4 * u;
        if (n >= NT) break;  // uniform
        int ti, tj;
        lower_tile(n, ti, tj);
        const int s0 = split ? 16 * (wave & 1) : 0, s1 = split ? s0 + 16 : 32;
#pragma unroll 4
        for (int st = s0; st < s1; ++st) {  // uniform: every lane runs every step
            const int r = 4 * st + q4;
            const double av = r < rows ? (double)xs[r][16 * ti + n16] : 0.0;
            const double bv = r < rows ? (double)xs[r][16 * tj + n16] : 0.0;
            acc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[u], 0, 0, 0);
        }
    }
}
template <int KP>
__device__ __forceinline__ void gram_zero(f64x4 (&acc)[GramTiles<KP>::PER]) {
#pragma unroll
    for (int u = 0; u < GramTiles<KP>::PER; ++u) acc[u] = f64x4{0.0, 0.0, 0.0, 0.0};
}
template <int KP>
__device__ __forceinline__ void gram_flush(const f64x4 (&acc)[GramTiles<KP>::PER], double* __restrict__ gb) {
    constexpr int NT = GramTiles<KP>::NT, PER = GramTiles<KP>::PER;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int n16 = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int n = KP == 64 && u == 2 ? 8 + (wave >> 1) : wave + 4 * u;  // as gram_tile_acc
        if (n >= NT) break;  // uniform
        int ti, tj;
        lower_tile(n, ti, tj);
#pragma unroll
        for (int i = 0; i < 4; ++i) atomicAdd(gb + (16 * ti + q4 + 4 * i) * KP + 16 * tj + n16, acc[u][i]);
    }
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// i % 4 of the 8-byte pieces lanes i / 4, 4 + i / 4, 8 + i / 4 and
// 12 + i / 4 name (lane layout checked on MI355X).
__device__ __forceinline__ bf16x4 lds_read_tr16(const uint8_t* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const_cast<uint8_t*>(p)));
    return __builtin_bit_cast(bf16x4, r);
}

// PAIR: two chunks in flight (an odd count peels its last chunk); otherwise
// one.  Rank-64 sketches always take PAIR (they hold two waves per SIMD
// either way); rank-32 ones with an odd count keep the single-set loop,
// whose smaller register count holds a third wave per SIMD.
// TA: A is the transpose of the operand stored, out = Delta^T B with Delta in
// its row-major panels [R/64][X][64] (R = F features, X = Tp tokens): a
// chunk (64 tokens of two panels) is parked as stored, [64 tokens][128
// features], and each lane's A operand (8 consecutive tokens of one feature)
// comes from two transposing LDS reads (ds_read_b64_tr_b16).
// DV > 0 (deficit mode, A = Delta, up to DV views): instead of loading A, a
// chunk's loads are the canonical rows (and rotate-half partners) and every
// view's target rows, and its park forms Delta exactly as delta_kernel does,
// stores its high and low parts in Delta's panels for the later products and
// parks them in LDS for this one: the first product of the range finder
// then costs no pass over Delta (p: the call's parameters; its rows and
// blocks are A's).
template <int KC, bool SPLIT_B, bool PAIR, bool TA, int DV>
__device__ __forceinline__ void sketch_body(const SketchArgs& a, const FormParams& p) {
    constexpr int KP = 32 * KC;
    constexpr int XC = 64;               // inner values per chunk: four 16-wide MFMA steps
    constexpr int PITCH = XC * 2 + 16;   // bytes per LDS row: 128 + 16 (16 lanes hit 16 bank groups)
    // TA: bytes per LDS row of 128 features: 256 + 32 (a 320-byte pitch,
    // which keeps the four rows of a transposing read on disjoint banks,
    // measured the same on MI355X)
    constexpr int PITCH_T = 128 * 2 + 32;
    constexpr int NBP = SPLIT_B ? 2 : 1;
    constexpr int A_HALF = TA ? 64 * PITCH_T : 128 * PITCH;  // the low part's offset
    constexpr int A_BYTES = 2 * A_HALF;
    static_assert(A_BYTES >= 128 * (KP + 1) * 4, "the Gram tile reuses the A buffers");
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[A_BYTES];          // [hi|lo][128 rows][PITCH] (TA: [64][PITCH_T])
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[NBP * KP * PITCH]; // [hi|lo][KP cols][PITCH]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hh = lane >> 5, col = lane & 31;
    // XCD-aware order: the hardware hands workgroup h (x fastest) to XCD h % 8;
    // logical workgroups are numbered so that each XCD runs one contiguous
    // range of them, so a block's row tiles share one L2 and B reaches HBM
    // once per block instead of once per XCD (MI355X, orbit shapes: the
    // Delta^T Q products 548-559 -> 483-489 us with nontemporal A loads)
    int64_t b, tx;
    {
        const int64_t n = (int64_t)gridDim.x * gridDim.y;
        const int64_t h = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
        const int64_t q = n / 8, rm = n % 8, x = h % 8, j = h / 8;
        const int64_t lg = x < rm ? x * (q + 1) + j : rm * (q + 1) + (x - rm) * q + j;
        b = lg / gridDim.x;
        tx = lg - b * gridDim.x;
    }
    // deficit mode: the block's chunk, stream and layer, rotary set-up, rows
    int half = 0;
    bool rot = false;
    const uint16_t* cb = nullptr;
    const uint16_t* tb0 = nullptr;
    uint16_t* drh = nullptr;
    int ci = 0;
    __shared__ float2 cs_tab[DV > 0 ? DV * kMaxHalfRopeF : 1];  // view v's cos/sin at [v * half]
    if constexpr (DV > 0) {
        const int l = (int)(b % p.L);
        const int zs = (int)(b / p.L);
        const int s = p.S == 2 ? (zs & 1) : 0;
        const int i = p.S == 2 ? (zs >> 1) : zs;
        ci = i;
        rot = s == 0 && p.rope_dim > 0;
        half = p.rope_dim >> 1;
        cb = p.canon[s] + (int64_t)i * p.canon_chunk_stride + (int64_t)l * p.canon_layer_stride;
        tb0 = p.target[s] + (int64_t)i * p.views * p.target_chunk_stride + (int64_t)l * p.target_layer_stride;
        drh = p.dr_hi + b * p.Tp * p.F * 2;
    }
    // a workgroup walks row_tiles tiles of 128 rows; the Gram partial sums stay
    // in registers across them and go out with one set of atomics
    f64x4 gacc[GramTiles<KP>::PER];
    gram_zero<KP>(gacc);
    for (int rt = 0; rt < a.row_tiles; ++rt) {
    const int r0 = ((int)tx * a.row_tiles + rt) * 128;
    if (r0 >= a.R) break;  // uniform
    const int rw = r0 + wave * 32;       // first row of this wave
    const bool active = rw < a.R;        // uniform over the wave
    const uint16_t* abase_hi = a.a_hi + b * a.a_block;
    const uint16_t* abase_lo = a.a_lo + b * a.a_block;
    const uint16_t* bbase_hi = a.bt_hi + b * a.bt_block;
    const uint16_t* bbase_lo = SPLIT_B ? a.bt_lo + b * a.bt_block : nullptr;
    // coalesced chunk loads: 8 threads per 128-byte row segment
    constexpr int AQ = 128 * 8 / 256;                 // A vectors per thread (4)
    constexpr int BQ = (KP * 8 + 255) / 256;          // B vectors per thread (1 or 2)
    struct RegsA {
        u32x4 ah[AQ], al[AQ], bh[BQ], bl[BQ];
    };
    struct RegsD {  // deficit mode: canonical, partner and per-view target vectors
        u32x4 c[AQ], pv[AQ], t[DV > 0 ? DV : 1][AQ], bh[BQ], bl[BQ];
    };
    using Regs = typename std::conditional<DV == 0, RegsA, RegsD>::type;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    auto load = [&](Regs& g, int x0) {
        if constexpr (DV > 0) {
            // rows past T re-read row T - 1 (their deficit is zero)
#pragma unroll
            for (int k = 0; k < AQ; ++k) {
                const int q = tid + 256 * k;
                const int t = min(r0 + (q >> 3), p.T - 1);
                const int f = x0 + 8 * (q & 7);
                const int e = (f % p.D) - p.rope_offset;
                const bool rv = rot && e >= 0 && e < p.rope_dim;
                const int poff = (rv && p.rope_style == KAMERA_ROPE_HALF) ? (e < half ? half : -half) : 0;
                const int64_t ro = (int64_t)t * p.F + f;
                g.c[k] = ld_cached(cb + ro);
                g.pv[k] = ld_cached(cb + ro + poff);
#pragma unroll
                for (int v = 0; v < DV; ++v)
                    if (v < p.views) g.t[v][k] = ld_cached(tb0 + v * p.target_chunk_stride + ro);
            }
        } else {
#pragma unroll
        for (int k = 0; k < AQ; ++k) {
            const int q = tid + 256 * k;
            int64_t off;
            if constexpr (TA) {
                // tokens x0 .. x0 + 63 of panels r0/64 and r0/64 + 1 (a missing
                // second panel re-reads the first: its rows are never stored)
                const int pn = min(r0 / 64 + (q >> 9), a.R / 64 - 1);
                off = (int64_t)pn * a.X * 128 + (int64_t)(x0 + ((q >> 3) & 63)) * 128 + 8 * (q & 7);
            } else {
                const int r = min(r0 + (q >> 3), a.R - 1);   // rows past R re-read the last (never stored)
                // A in 64-wide panels [X/64][R][2][64]: a chunk's rows, high and
            // low parts, are one piece
                off = (int64_t)(x0 / XC) * a.R * 128 + (int64_t)r * 128 + 8 * (q & 7);
            }
            // read once per product, so streamed past the caches (nontemporal)
            g.ah[k] = ld_stream(abase_hi + off);
            g.al[k] = ld_stream(abase_lo + off);
        }
        }
#pragma unroll
        for (int k = 0; k < BQ; ++k) {
            const int q = tid + 256 * k;
            const int c = min(q >> 3, a.nb_valid - 1);
            const int64_t off = (int64_t)c * a.X + x0 + 8 * (q & 7);
            g.bh[k] = ld_cached(bbase_hi + off);
            if (SPLIT_B) g.bl[k] = ld_cached(bbase_lo + off);
        }
    };
    auto park = [&](const Regs& g, int x0) {
        if constexpr (DV > 0) {
            const float inv_views = 1.0f / (float)p.views;
#pragma unroll
            for (int k = 0; k < AQ; ++k) {
                const int q = tid + 256 * k;
                const int t = r0 + (q >> 3);
                const int f = x0 + 8 * (q & 7);
                const int e = (f % p.D) - p.rope_offset;
                const bool rv = rot && e >= 0 && e < p.rope_dim;
                float d[8];
#pragma unroll
                for (int w = 0; w < 8; ++w) d[w] = 0.0f;
#pragma unroll
                for (int v = 0; v < DV; ++v)
                    if (v < p.views)
                        delta_add8(d, g.c[k], g.pv[k], g.t[v][k], cs_tab + v * half, e, rv, e < half, half,
                                   p.rope_style, t < p.T);
                if (p.views != 1) {
#pragma unroll
                    for (int w = 0; w < 8; ++w) d[w] *= inv_views;
                }
                u32x4 h, lo;
                split8(d, h, lo);
                if (t < p.Tp) {
                    // Delta's panel x0 / 64, row t: 64 high then 64 low parts,
                    // read by later launches only, so streamed (nontemporal;
                    // on MI355X the single-frame launch 54.6 -> 52.1 us)
                    const int64_t ro = (int64_t)(x0 / XC) * p.Tp * 128 + (int64_t)t * 128 + 8 * (q & 7);
                    st_stream(drh + ro, h);
                    st_stream(drh + ro + 64, lo);
                }
                const int o = (q >> 3) * PITCH + 16 * (q & 7);
                *reinterpret_cast<u32x4*>(lds_a + o) = h;
                *reinterpret_cast<u32x4*>(lds_a + A_HALF + o) = lo;
            }
        } else {
#pragma unroll
        for (int k = 0; k < AQ; ++k) {
            const int q = tid + 256 * k;
            const int o = TA ? ((q >> 3) & 63) * PITCH_T + 128 * (q >> 9) + 16 * (q & 7)
                             : (q >> 3) * PITCH + 16 * (q & 7);
            *reinterpret_cast<u32x4*>(lds_a + o) = g.ah[k];
            *reinterpret_cast<u32x4*>(lds_a + A_HALF + o) = g.al[k];
        }
        }
#pragma unroll
        for (int k = 0; k < BQ; ++k) {
            const int q = tid + 256 * k;
            if (q < KP * 8) {
                const bool valid = (q >> 3) < a.nb_valid;    // columns past nb_valid are zero
                const int o = (q >> 3) * PITCH + 16 * (q & 7);
                *reinterpret_cast<u32x4*>(lds_b + o) = valid ? g.bh[k] : zero;
                if (SPLIT_B) *reinterpret_cast<u32x4*>(lds_b + KP * PITCH + o) = valid ? g.bl[k] : zero;
            }
        }
    };
    f32x16 acc[KC];
#pragma unroll
    for (int cb = 0; cb < KC; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[cb][v] = 0.0f;
    const int chunks = a.X / XC;
    // TA: lane (i = lane % 16) names token row (i / 4) of a 4-row group and
    // features 4 (i % 4) .. of its 16-feature half; the transposing read then
    // gives it feature 16 half + i of the wave's 32, four consecutive tokens
    const uint8_t* atr = lds_a + (lane & 15) / 4 * PITCH_T +
                         2 * (32 * wave + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    auto products = [&]() {
        const uint8_t* arow = lds_a + (wave * 32 + col) * PITCH;
#pragma unroll
        for (int st = 0; st < XC / 16; ++st) {
            const int ko = (16 * st + 8 * hh) * 2;
            bf16x8 A0, A1;
            if constexpr (TA) {
                const uint8_t* t0 = atr + (16 * st + 8 * hh) * PITCH_T;
                const bf16x4 h0 = lds_read_tr16(t0), h1 = lds_read_tr16(t0 + 4 * PITCH_T);
                const bf16x4 l0 = lds_read_tr16(t0 + A_HALF), l1 = lds_read_tr16(t0 + A_HALF + 4 * PITCH_T);
                A0 = bf16x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
                A1 = bf16x8{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
            } else {
                A0 = *reinterpret_cast<const bf16x8*>(arow + ko);
                A1 = *reinterpret_cast<const bf16x8*>(arow + A_HALF + ko);
            }
#pragma unroll
            for (int cb = 0; cb < KC; ++cb) {
                const uint8_t* brow = lds_b + (cb * 32 + col) * PITCH + ko;
                const bf16x8 B0 = *reinterpret_cast<const bf16x8*>(brow);
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, B0, acc[cb], 0, 0, 0);
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B0, acc[cb], 0, 0, 0);
                if (SPLIT_B) {
                    const bf16x8 B1 = *reinterpret_cast<const bf16x8*>(brow + KP * PITCH);
                    acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, B1, acc[cb], 0, 0, 0);
                }
            }
        }
    };
    // deficit mode: every view's cos/sin table, built once per workgroup while
    // its first chunks' loads are in flight
    auto tables = [&]() {
        if constexpr (DV > 0) {
            if (rt == 0) {
                if (rot)
                    for (int v = 0; v < p.views; ++v) {
                        const int64_t dl = p.delta[(int64_t)ci * p.views + v];
                        for (int j = tid; j < half; j += 256)
                            cs_tab[v * half + j] = rope_cos_sin(p.log2_base, p.rope_dim, j, dl);
                    }
                __syncthreads();
            }
        }
    };
    if constexpr (PAIR) {
        // Two register sets: chunk ch + 2 is requested while chunk ch is
        // multiplied.  Every pass loads and parks both sets (past the end the
        // loads repeat the last chunk, unused), so the loop body issues the
        // same loads every time and each wait retires exactly its set.
        Regs g0, g1;
        load(g0, 0);
        load(g1, min(1, chunks - 1) * XC);
        tables();
        int ch = 0;
        for (; ch + 1 < chunks; ch += 2) {
            park(g0, ch * XC);
            __syncthreads();
            load(g0, min(ch + 2, chunks - 1) * XC);
            products();
            __syncthreads();   // the next park overwrites the buffers
            park(g1, (ch + 1) * XC);
            __syncthreads();
            load(g1, min(ch + 3, chunks - 1) * XC);
            products();
            __syncthreads();
        }
        if (ch < chunks) {  // an odd count: the last chunk is in g0 (g1 repeats it, unused)
            park(g0, ch * XC);
            __syncthreads();
            products();
            __syncthreads();
        }
    } else {
        // one set: the next chunk is in flight during each chunk's products
        Regs g;
        load(g, 0);
        tables();
        for (int ch = 0; ch < chunks; ++ch) {
            park(g, ch * XC);
            __syncthreads();
            if (ch + 1 < chunks) load(g, (ch + 1) * XC);
            products();
            __syncthreads();   // the next chunk's park overwrites the buffers
        }
    }
    float* o = a.out + b * a.out_block;
    float (*tile)[KP + 1] = reinterpret_cast<float (*)[KP + 1]>(lds_a);  // buffers are free now
#pragma unroll
    for (int cb = 0; cb < KC; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = 8 * (v >> 2) + 4 * hh + (v & 3);
            if (active) o[(int64_t)(rw + r) * KP + cb * 32 + col] = acc[cb][v];
            tile[wave * 32 + r][cb * 32 + col] = active ? acc[cb][v] : 0.0f;
        }
    if (a.g) {  // uniform
        __syncthreads();
        gram_tile_acc<KP>(tile, min(128, a.R - r0), gacc);
    }
    __syncthreads();  // the next tile's park overwrites the tile
    }
    if (a.g) gram_flush<KP>(gacc, a.g + b * KP * KP);
}

template <int KC, bool SPLIT_B, bool PAIR, bool TA>
__global__ __launch_bounds__(256, KC == 1 && !(SPLIT_B && PAIR) ? 3 : 2) void sketch_kernel(const SketchArgs a) {
    sketch_body<KC, SPLIT_B, PAIR, TA, 0>(a, FormParams{});  // (p unused)
}

// Delta Omega with Delta formed on the way (the first product of the range
// finder; at most DV views)
template <int KC, bool PAIR, int DV>
__global__ __launch_bounds__(256, 2) void delta_sketch_kernel(const SketchArgs a, const FormParams p) {
    sketch_body<KC, false, PAIR, false, DV>(a, p);
}

// ---------------------------------------------------------------------------
// Orthonormalization: shifted Cholesky QR, twice
// ---------------------------------------------------------------------------
//
// X [R][kp] -> X R^-1 with G = X^T X = R^T R (fp64).  A shift of 1e-14 of the
// largest diagonal entry keeps the factorization defined when X is (nearly)
// rank deficient: such directions come out as short or noisy columns, which
// the second pass turns into orthonormal ones (shifted CholeskyQR: Fukaya,
// Kannan, Nakatsukasa, Yamamoto & Yamamoto, SIAM J. Sci. Comput. 2020).
// Only the span matters to the range finder, so an inexact first pass is
// harmless.  Zero columns (sketch padding) stay zero.  The Gram matrix of the
// first pass comes from the sketch kernel that produced X, that of the
// second from the first apply; per pass:
//  * chol_lds_kernel<KP>: four waves per block factor G and invert R (fp32 M);
//  * apply_kernel<KP, GRAM>: X <- X M in 128-row tiles (two or four per
//    workgroup for tall X), plus either the Gram matrix of the new rows (GRAM,
//    from the product's registers) or (last pass) the bf16 transpose (high and
//    optionally low part) the next product reads, the next tile's rows in
//    flight.
// Gram matrices hold their lower triangle only (with the diagonal); the
// Cholesky kernels read no more, and the eigen step mirrors it.  A call
// clears its two Gram matrices once; every kernel that reads one clears it
// after reading, for the next accumulation.

__global__ __launch_bounds__(256) void zero_kernel(double* __restrict__ g, const int64_t count) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < count) g[i] = 0.0;
}

// One workgroup of four waves per block: G = L L^T (shifted), M = L^-T = R^-1
// (upper triangular).  Right-looking Cholesky in LDS: each step's scaled
// pivot column also goes to a separate array, and the step's trailing update
// is spread over the 256 threads by a table of lower-triangle items (on
// MI355X: 92 -> 50 us per launch on MLA's 64 columns against one wave walking
// its rows, and 26.7 -> 24.2 us at 32 columns against a one-wave version
// holding the matrix in registers).  Then column `lane` of L^-1 (row `lane` of M)
// by forward substitution on the first wave, held in registers (fully
// unrolled), with L read by broadcast from LDS.
template <int KP>
__global__ __launch_bounds__(256) void chol_lds_kernel(double* __restrict__ g, float* __restrict__ m_out,
                                                       const int n) {
    __shared__ double a[KP][KP + 1];
    __shared__ double col[KP];
    __shared__ double inv_diag[KP];
    __shared__ uint16_t tri[KP * (KP + 1) / 2];  // lower-triangle item e -> (row << 8) | column
    const int64_t b = blockIdx.x;
    const int tid = threadIdx.x;
    double* gb = g + b * KP * KP;
    for (int q = tid; q < KP * KP; q += 256) a[q / KP][q % KP] = gb[q];
    if (tid < KP)
        for (int c = 0; c <= tid; ++c) tri[tid * (tid + 1) / 2 + c] = (uint16_t)((tid << 8) | c);
    __syncthreads();
    // G is read: cleared for the next Gram matrix accumulated into it
    for (int q = tid; q < KP * KP; q += 256) gb[q] = 0.0;
    double dmax = 0.0;
    for (int c = 0; c < KP; ++c) dmax = fmax(dmax, a[c][c]);
    float* mb = m_out + b * KP * KP;
    if (!(dmax > 0.0)) {  // X = 0: nothing to orthonormalize (uniform)
        for (int q = tid; q < KP * KP; q += 256) mb[q] = 0.0f;
        return;
    }
    const double shift = 1e-14 * dmax;
    __syncthreads();  // every thread has read the diagonal before it is shifted
    if (tid < KP) a[tid][tid] += shift;
    __syncthreads();
    // the n sketch columns only: past them G is zero, and so is M.  Step j:
    // column j below the pivot, then the trailing rank-1 update of the rows
    // and columns past j, its lower-triangle items spread over the 256 threads
    for (int j = 0; j < n; ++j) {
        const double d = a[j][j];
        // one reciprocal square root per pivot: 1 / L_jj scales the column
        // and L_jj = d / sqrt(d) (a square root and divisions measured 24.2
        // against 21.6 us per launch at 32 columns on MI355X)
        const double dd = d > shift ? d : shift;
        const double inv = rsqrt(dd);
        if (tid > j && tid < n) {
            const double lij = a[tid][j] * inv;
            a[tid][j] = lij;
            col[tid] = lij;
        }
        __syncthreads();
        if (tid == j) {
            a[j][j] = dd * inv;
            inv_diag[j] = inv;
        }
        const int w = n - 1 - j;  // trailing rows (and columns)
        for (int e = tid; e < w * (w + 1) / 2; e += 256) {
            const int t = tri[e];
            const int r = j + 1 + (t >> 8), c = j + 1 + (t & 255);
            a[r][c] = fma(-col[r], col[c], a[r][c]);
        }
        __syncthreads();
    }
    if (tid >= KP) return;  // no barrier follows
    const int lane = tid;
    // X = L^-1: column `lane`, X[i] = (e_lane[i] - sum_{k<i} L[i][k] X[k]) / L[i][i]
    double x[KP];
#pragma unroll
    for (int i = 0; i < KP; ++i) {
        if (i >= n || lane >= n) {  // uniform in i; lanes past n give zero rows of M
            x[i] = 0.0;
            continue;
        }
        double s = i == lane ? 1.0 : 0.0;
#pragma unroll
        for (int k = 0; k < i; ++k) s = fma(-a[i][k], x[k], s);
        x[i] = s * inv_diag[i];
    }
    // M = L^-T: row `lane` of M is column `lane` of L^-1
    if (lane < KP) {
#pragma unroll
        for (int i = 0; i < KP; i += 4)
            *reinterpret_cast<float4*>(mb + lane * KP + i) =
                make_float4((float)x[i], (float)x[i + 1], (float)x[i + 2], (float)x[i + 3]);
    }
}

// X_b <- X_b M_b over row_tiles tiles of 128 rows per workgroup; then either
// (GRAM, g non-NULL) the Gram matrix of the new rows into g, its partial sums
// in registers across the tiles and out with one set of atomics, or (not GRAM)
// the bf16 transpose if xt_hi is non-NULL, the next tile's rows loaded into
// registers during the current one's work (on MI355X at 64 columns: 164 VGPRs
// and three waves per SIMD without the Gram code; the Gram variant, 256 VGPRs
// at two, loads each tile after the previous one's work).
template <int KP, bool GRAM>
__global__ __launch_bounds__(256, 2) void apply_kernel(float* __restrict__ x, const int64_t x_block, const int R,
                                                     const float* __restrict__ m_in, double* __restrict__ g,
                                                     uint16_t* __restrict__ xt_hi, uint16_t* __restrict__ xt_lo,
                                                     const int64_t xt_block, const int store_x, const int row_tiles) {
    // X M on v_mfma_f32_16x16x4f32: wave w takes rows 32w .. 32w + 31 (two
    // 16-row tiles) and every column tile; M's operands are read once from
    // global memory (L2: every workgroup of the block reads the same M) into
    // registers.  The LDS pitch KP + 4 keeps the operand reads of 16 rows x
    // 4 k on distinct banks.
    constexpr int CT = KP / 16, KS = KP / 4;
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    __shared__ float xs[128][KP + 4];
    const int64_t b = blockIdx.y;
    float* xb = x + b * x_block;
    const float* mb = m_in + b * KP * KP;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n16 = lane & 15, q4 = lane >> 4;
    float bm[CT][KS];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int s = 0; s < KS; ++s) bm[ct][s] = mb[(4 * s + q4) * KP + 16 * ct + n16];
    // GRAM: every lower 16 x 16 tile of the Gram matrix over this wave's
    // rows, from the product's registers (below); the waves' sums meet in LDS
    constexpr int NT = GramTiles<KP>::NT;
    f64x4 gt[GRAM ? NT : 1];
#pragma unroll
    for (int t = 0; t < (GRAM ? NT : 1); ++t) gt[t] = f64x4{0.0, 0.0, 0.0, 0.0};
    __shared__ double gred[GRAM ? NT * 256 : 1];
    // the next tile's rows are requested into registers while the current
    // tile is multiplied and stored (not with GRAM, whose accumulators take
    // those registers)
    constexpr int XV = 128 * KP / 4 / 256;  // float4 per thread per tile
    float4 nx[XV];
    auto load_x = [&](int r0) {
#pragma unroll
        for (int k = 0; k < XV; ++k) {
            const int q = threadIdx.x + 256 * k;
            const int r = q / (KP / 4), c = 4 * (q % (KP / 4));
            nx[k] = r0 + r < R ? *reinterpret_cast<const float4*>(xb + (int64_t)(r0 + r) * KP + c)
                               : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    };
    load_x(blockIdx.x * row_tiles * 128);
    for (int t = 0; t < row_tiles; ++t) {
        const int r0 = (blockIdx.x * row_tiles + t) * 128;
        if (r0 >= R) break;  // uniform
        const int rows = min(128, R - r0);
#pragma unroll
        for (int k = 0; k < XV; ++k) {
            const int q = threadIdx.x + 256 * k;
            const int r = q / (KP / 4), c = 4 * (q % (KP / 4));
            *reinterpret_cast<float4*>(&xs[r][c]) = nx[k];
        }
        __syncthreads();
        if (!GRAM && t + 1 < row_tiles && r0 + 128 < R) load_x(r0 + 128);  // uniform
        f32x4v out[2][CT];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int ra = 32 * wave + 16 * rt + n16;  // A row of this lane
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) out[rt][ct] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const float a = xs[ra][4 * s + q4];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    out[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bm[ct][s], out[rt][ct], 0, 0, 0);
            }
        }
        if constexpr (GRAM) {
            // the fp64 product's operands straight from the D layout: for each
            // (rt, i), lane (n16, q4) holds row 32w + 16rt + 4q4 + i of every
            // column tile, which is a 4-row step of A = X^T (k = q4) and of B
            // = X; so each wave sums all lower tiles over its 32 rows (80
            // steps at 64 columns, no LDS reads)
            constexpr int TI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
            constexpr int TJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool in = 32 * wave + 16 * rt + 4 * q4 + i < rows;
                    double v[CT];
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) v[ct] = in ? (double)out[rt][ct][i] : 0.0;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        gt[nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(v[TI[nt]], v[TJ[nt]], gt[nt], 0, 0, 0);
                }
        }
        __syncthreads();
        // D layout: row 32w + 16rt + 4q4 + i, column 16ct + n16
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 32 * wave + 16 * rt + 4 * q4 + i;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) xs[r][16 * ct + n16] = r < rows ? out[rt][ct][i] : 0.0f;
            }
        __syncthreads();
        // the new rows, back in place (only where a later step reads them)
        if (store_x) {
            for (int q = threadIdx.x; q < 128 * KP / 4; q += 256) {
                const int r = q / (KP / 4), c = 4 * (q % (KP / 4));
                if (r < rows)
                    *reinterpret_cast<float4*>(xb + (int64_t)(r0 + r) * KP + c) =
                        *reinterpret_cast<const float4*>(&xs[r][c]);
            }
        }
        if (xt_hi) {  // uniform
            // transpose: column c, 16 rows per item (R is a multiple of 64)
            for (int q = threadIdx.x; q < KP * 8; q += 256) {
                const int c = q >> 3, rr = (q & 7) * 16;
                if (rr >= rows) continue;
                float va[8], vb[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    va[e] = xs[rr + e][c];
                    vb[e] = xs[rr + 8 + e][c];
                }
                u32x4 h0, h1, l0, l1;
                split8(va, h0, l0);
                split8(vb, h1, l1);
                uint16_t* dh = xt_hi + b * xt_block + (int64_t)c * R + r0 + rr;
                *reinterpret_cast<u32x4*>(dh) = h0;
                *reinterpret_cast<u32x4*>(dh + 8) = h1;
                if (xt_lo) {
                    uint16_t* dl = xt_lo + b * xt_block + (int64_t)c * R + r0 + rr;
                    *reinterpret_cast<u32x4*>(dl) = l0;
                    *reinterpret_cast<u32x4*>(dl + 8) = l1;
                }
            }
        }
        __syncthreads();  // the next tile's loads overwrite xs
        if (GRAM && t + 1 < row_tiles && r0 + 128 < R) load_x(r0 + 128);  // uniform
    }
    if constexpr (GRAM) {
        // the four waves' tiles added in LDS (result row q4 + 4j, column
        // n16), then one global atomic per element
        for (int q = threadIdx.x; q < NT * 256; q += 256) gred[q] = 0.0;
        __syncthreads();
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int j = 0; j < 4; ++j) atomicAdd(&gred[nt * 256 + (q4 + 4 * j) * 16 + n16], gt[nt][j]);
        __syncthreads();
        double* gb = g + b * KP * KP;
        for (int q = threadIdx.x; q < NT * 256; q += 256) {
            int ti, tj;
            lower_tile(q >> 8, ti, tj);
            atomicAdd(gb + (16 * ti + ((q & 255) >> 4)) * KP + 16 * tj + (q & 15), gred[q]);
        }
    }
}

// ---------------------------------------------------------------------------
// Factors from Z = Delta^T Q and Q: U = Q W_m L_m^(1/2), V = Z W_m L_m^(-1/2)
// ---------------------------------------------------------------------------
//
// eig_kernel (one workgroup per block): eigen-decomposition of G = Z^T Z =
// B B^T by cyclic Jacobi in fp64 with the round-robin parallel ordering over
// the n sketch columns (k rounded up to even; the columns past them are zero
// and stay so): each step rotates n/2 disjoint pairs at once, in place: rows
// (J^T G), then columns (G J and W J).  Sweeps stop when the off-diagonal
// mass is below 1e-14 of the diagonal's or after kMaxSweeps.  Entries are
// then ~1e-7 of the largest eigenvalue L_1, which turns an eigenvector pair
// (i, j) by ~1e-7 L_1 / (L_i - L_j): a relative gap of 1e-3 at the
// truncation moves the product U V^T by ~1e-4, against a bfloat16 ulp of
// 4e-3 (on MI355X the single frame's step 156 -> 132 us against 1e-20, MLA's
// 635 -> 620 us; 1e-26 had taken 12% more than 1e-20).  A pair whose
// off-diagonal entry is below 1e-18 of its diagonal pair is not rotated.  Then, in descending eigenvalue order,
// sigma_j = sqrt(L_j) (0 when <= kNegligible sigma_1), the sign that makes
// V's largest entry positive (first on ties), and the kp x m matrices
// Wu = W_j sigma_j s_j and Wv = W_j / sigma_j s_j for out_kernel.
template <int KP>
__global__ __launch_bounds__(256) void eig_kernel(double* __restrict__ g, const float* __restrict__ z,
                                                   const int64_t z_block, const int F, const int m, const int n,
                                                   float* __restrict__ wu, float* __restrict__ wv) {
    __shared__ double A[KP][KP + 1];
    __shared__ double W[KP][KP + 1];
    __shared__ int pp[KP / 2], qq[KP / 2];
    __shared__ double rc[KP / 2], rs[KP / 2];
    __shared__ double red[2][256];
    __shared__ double lam[KP];
    __shared__ int order[KP];
    __shared__ double sig[KP];
    __shared__ float vbest[256];
    __shared__ int vidx[256];
    __shared__ float sgn[KP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t b = blockIdx.x;
    double* gb = g + b * KP * KP;
    for (int q = tid; q < KP * KP; q += 256) {
        const int i = q / KP, j = q % KP;
        A[i][j] = gb[max(i, j) * KP + min(i, j)];  // the lower triangle holds G
        W[i][j] = i == j ? 1.0 : 0.0;
    }
    __syncthreads();
    for (int q = tid; q < KP * KP; q += 256) gb[q] = 0.0;  // read: cleared, as the Cholesky kernel does
    for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
        double off = 0.0, dia = 0.0;
        for (int q = tid; q < KP * KP; q += 256) {
            const int i = q / KP, j = q % KP;
            const double e = A[i][j];
            if (i == j) dia += e * e; else off += e * e;
        }
        red[0][tid] = off;
        red[1][tid] = dia;
        __syncthreads();
        for (int h = 128; h > 0; h >>= 1) {
            if (tid < h) {
                red[0][tid] += red[0][tid + h];
                red[1][tid] += red[1][tid + h];
            }
            __syncthreads();
        }
        const bool done = red[0][0] <= 1e-14 * red[1][0];
        __syncthreads();
        if (done) break;
        for (int step = 0; step < n - 1; ++step) {
            if (tid < n / 2) {
                auto slot = [&](int s) {  // (s - 1 + step) mod (n - 1), both terms below n - 1
                    const int v = s - 1 + step;
                    return s == 0 ? 0 : (v >= n - 1 ? v - (n - 1) : v) + 1;
                };
                int p = slot(tid), q = slot(n - 1 - tid);
                if (p > q) { const int t = p; p = q; q = t; }
                const double app = A[p][p], aqq = A[q][q], apq = A[p][q];
                double c = 1.0, s = 0.0;
                if (apq * apq > 1e-36 * fabs(app * aqq)) {
                    // t = tan of the angle that zeroes apq:
                    // sgn(tau) 2 apq / (|tau| + sqrt(tau^2 + 4 apq^2)), tau = aqq - app
                    const double tau = aqq - app;
                    const double r = sqrt(fma(tau, tau, 4.0 * apq * apq));
                    double t = 2.0 * apq / (fabs(tau) + r);
                    if (tau < 0.0) t = -t;
                    c = rsqrt(fma(t, t, 1.0));
                    s = t * c;
                }
                pp[tid] = p;
                qq[tid] = q;
                rc[tid] = c;
                rs[tid] = s;
            }
            __syncthreads();
            // The items of a phase touch disjoint elements, so each thread loads all
            // of its items before it stores any: the loads pipeline instead of
            // waiting on stores the compiler cannot prove disjoint.
            // items: (pair, column) over the n / 2 pairs and the n columns that
            // are not zero (G and W are zero past n, and rotations keep them so)
            constexpr int IT = (KP / 2) * KP / 256;  // items per thread, at most
            const int items = (n / 2) * n;
            // rows: G <- J^T G (J: column p = c e_p - s e_q, column q = s e_p + c e_q)
            {
                int ip[IT], iq[IT], ik[IT];
                double gp[IT], gq[IT], cc[IT], ss[IT];
#pragma unroll
                for (int it = 0; it < IT; ++it) {
                    const int u = min(tid + 256 * it, items - 1), pr = u / n;
                    ik[it] = u - pr * n;
                    ip[it] = pp[pr];
                    iq[it] = qq[pr];
                    cc[it] = rc[pr];
                    ss[it] = rs[pr];
                    gp[it] = A[ip[it]][ik[it]];
                    gq[it] = A[iq[it]][ik[it]];
                }
#pragma unroll
                for (int it = 0; it < IT; ++it) {
                    if (tid + 256 * it >= items) continue;
                    A[ip[it]][ik[it]] = cc[it] * gp[it] - ss[it] * gq[it];
                    A[iq[it]][ik[it]] = ss[it] * gp[it] + cc[it] * gq[it];
                }
            }
            __syncthreads();
            // columns: G <- G J, W <- W J
            {
                int ip[IT], iq[IT], ik[IT];
                double gp[IT], gq[IT], wp[IT], wq[IT], cc[IT], ss[IT];
#pragma unroll
                for (int it = 0; it < IT; ++it) {
                    const int u = min(tid + 256 * it, items - 1), pr = u / n;
                    ik[it] = u - pr * n;
                    ip[it] = pp[pr];
                    iq[it] = qq[pr];
                    cc[it] = rc[pr];
                    ss[it] = rs[pr];
                    gp[it] = A[ik[it]][ip[it]];
                    gq[it] = A[ik[it]][iq[it]];
                    wp[it] = W[ik[it]][ip[it]];
                    wq[it] = W[ik[it]][iq[it]];
                }
#pragma unroll
                for (int it = 0; it < IT; ++it) {
                    if (tid + 256 * it >= items) continue;
                    A[ik[it]][ip[it]] = cc[it] * gp[it] - ss[it] * gq[it];
                    A[ik[it]][iq[it]] = ss[it] * gp[it] + cc[it] * gq[it];
                    W[ik[it]][ip[it]] = cc[it] * wp[it] - ss[it] * wq[it];
                    W[ik[it]][iq[it]] = ss[it] * wp[it] + cc[it] * wq[it];
                }
            }
            __syncthreads();
        }
    }
    // eigenvalues in descending order (ties: lower index first)
    if (tid < KP) lam[tid] = A[tid][tid];
    __syncthreads();
    if (tid < KP) {
        const double me = lam[tid];
        int rank = 0;
        for (int c = 0; c < KP; ++c) rank += (lam[c] > me) || (lam[c] == me && c < tid);
        order[rank] = tid;
    }
    __syncthreads();
    if (tid < KP) {
        const double l1 = fmax(lam[order[0]], 0.0);
        const double sj = sqrt(fmax(lam[order[tid]], 0.0));
        sig[tid] = (sj > kNegligible * sqrt(l1) && sj > 0.0) ? sj : 0.0;
    }
    __syncthreads();
    // sign of every output column: the largest |V| entry (first on ties)
    // positive, V_j = Z W_{order j}.  Columns 16 at a time: each thread reads
    // its features' Z rows (16-byte loads) and forms their entries of the 16
    // columns in fp64 (W's columns from LDS), keeping per column the largest
    // magnitude (as float), its feature and its sign; the columns' maxima then
    // meet by exchanges within each wave and through LDS across the waves.
    const float* zb = z + b * z_block;
    constexpr int CJ = 16;
    for (int j0 = 0; j0 < m; j0 += CJ) {
        float best[CJ];
        int bi[CJ], neg[CJ];
#pragma unroll
        for (int jj = 0; jj < CJ; ++jj) {
            best[jj] = -1.0f;
            bi[jj] = 0x7fffffff;
            neg[jj] = 0;
        }
        for (int f = tid; f < F; f += 256) {  // f increases: the first maximum stays
            float zr[KP];
            const float4* zf = reinterpret_cast<const float4*>(zb + (int64_t)f * KP);
#pragma unroll
            for (int c4 = 0; c4 < KP / 4; ++c4) {
                const float4 x = zf[c4];
                zr[4 * c4] = x.x;
                zr[4 * c4 + 1] = x.y;
                zr[4 * c4 + 2] = x.z;
                zr[4 * c4 + 3] = x.w;
            }
#pragma unroll
            for (int jj = 0; jj < CJ; ++jj) {
                const int j = j0 + jj;
                if (j >= m || !(sig[j] > 0.0)) continue;
                const int oj = order[j];
                double vv = 0.0;
#pragma unroll
                for (int c = 0; c < KP; ++c) vv = fma((double)zr[c], W[c][oj], vv);
                const float av = (float)fabs(vv);
                if (av > best[jj]) {
                    best[jj] = av;
                    bi[jj] = f;
                    neg[jj] = vv < 0.0;
                }
            }
        }
        // within the wave: the larger magnitude, the lower feature on ties
#pragma unroll
        for (int jj = 0; jj < CJ; ++jj) {
#pragma unroll
            for (int x = 1; x < 64; x *= 2) {
                const float ob = __shfl_xor(best[jj], x);
                const int oi = __shfl_xor(bi[jj], x), on = __shfl_xor(neg[jj], x);
                if (ob > best[jj] || (ob == best[jj] && oi < bi[jj])) {
                    best[jj] = ob;
                    bi[jj] = oi;
                    neg[jj] = on;
                }
            }
        }
        if (lane == 0) {
#pragma unroll
            for (int jj = 0; jj < CJ; ++jj) {
                vbest[wave * CJ + jj] = best[jj];
                vidx[wave * CJ + jj] = bi[jj];
                vidx[128 + wave * CJ + jj] = neg[jj];
            }
        }
        __syncthreads();
        if (tid < CJ && j0 + tid < m) {
            float bb = vbest[tid];
            int ii = vidx[tid], nn = vidx[128 + tid];
            for (int w = 1; w < 4; ++w) {
                const float ob = vbest[w * CJ + tid];
                const int oi = vidx[w * CJ + tid];
                if (ob > bb || (ob == bb && oi < ii)) {
                    bb = ob;
                    ii = oi;
                    nn = vidx[128 + w * CJ + tid];
                }
            }
            const int j = j0 + tid;
            sgn[j] = sig[j] > 0.0 && ii >= 0 && ii < F && nn ? -1.0f : 1.0f;
        }
        __syncthreads();
    }
    float* wub = wu + b * KP * m;
    float* wvb = wv + b * KP * m;
    for (int q = tid; q < KP * m; q += 256) {
        const int c = q / m, j = q % m;
        const double sj = sig[j];
        const double wcj = W[c][order[j]];
        wub[q] = sj > 0.0 ? (float)(wcj * sj) * sgn[j] : 0.0f;
        wvb[q] = sj > 0.0 ? (float)(wcj / sj) * sgn[j] : 0.0f;
    }
}

// U_b = Q_b Wu_b (T x m) and V_b = Z_b Wv_b (F x m), bf16, 128 rows per
// workgroup (grid x covers ceil(T/128) row tiles of U, then ceil(F/128) of V),
// on v_mfma_f32_16x16x4f32 as in apply_kernel: the rows staged in LDS with
// 16-byte loads, W's operands in registers (columns past m zero), the result
// parked in LDS and stored as whole bf16 rows, consecutive threads on
// consecutive column pairs.
struct OutArgs {
    const float* q;
    const float* z;
    int64_t q_block, z_block;
    const float* wu;
    const float* wv;
    int32_t m, T, F, L, S;
    uint16_t* u[2];
    uint16_t* v[2];
};

template <int KP>
__global__ __launch_bounds__(256) void out_kernel(const OutArgs a) {
    constexpr int KS = KP / 4, CT = kMaxKp / 16;
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    __shared__ float xs[128][KP + 4];
    const int64_t blk = blockIdx.y;  // ((i * S) + s) * L + l
    const int l = (int)(blk % a.L);
    const int s = (int)((blk / a.L) % a.S);
    const int i = (int)(blk / ((int64_t)a.L * a.S));
    const int m = a.m;
    const int ugroups = (a.T + 127) / 128;
    const bool is_u = (int)blockIdx.x < ugroups;
    const int r0 = (is_u ? (int)blockIdx.x : (int)blockIdx.x - ugroups) * 128;
    const int R = is_u ? a.T : a.F;
    const int rows = min(128, R - r0);
    const float* x = is_u ? a.q + blk * a.q_block : a.z + blk * a.z_block;
    const float* wb = (is_u ? a.wu : a.wv) + blk * KP * m;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n16 = lane & 15, q4 = lane >> 4;
    const int ctn = (m + 15) / 16;  // column tiles of the result (uniform)
    for (int q = threadIdx.x; q < 128 * KP / 4; q += 256) {
        const int r = q / (KP / 4), c = 4 * (q % (KP / 4));
        *reinterpret_cast<float4*>(&xs[r][c]) =
            r < rows ? *reinterpret_cast<const float4*>(x + (int64_t)(r0 + r) * KP + c)
                     : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    float bm[CT][KS];  // B[k][j] = W[k][j], k = 4 s + q4, j = 16 ct + n16
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int st = 0; st < KS; ++st) {
            const int j = 16 * ct + n16;
            bm[ct][st] = j < m ? wb[(4 * st + q4) * m + j] : 0.0f;
        }
    __syncthreads();
    f32x4v acc[2][CT];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int ra = 32 * wave + 16 * rt + n16;  // A row of this lane
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < KS; ++st) {
            const float av = xs[ra][4 * st + q4];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                if (ct < ctn) acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bm[ct][st], acc[rt][ct], 0, 0, 0);
        }
    }
    __syncthreads();
    // D layout: row 32w + 16rt + 4q4 + i, column 16ct + n16 (m <= KP: it fits xs)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                if (ct < ctn && 16 * ct + n16 < m) xs[32 * wave + 16 * rt + 4 * q4 + e][16 * ct + n16] = acc[rt][ct][e];
    __syncthreads();
    uint16_t* o = is_u ? a.u[s] + (((int64_t)i * a.L + l) * a.T) * m : a.v[s] + (((int64_t)i * a.L + l) * a.F) * m;
    const int hp = m / 2;  // column pairs per row (m is even)
    for (int q = threadIdx.x; q < rows * hp; q += 256) {
        const int r = q / hp, j = 2 * (q - r * hp);
        *reinterpret_cast<uint32_t*>(o + (int64_t)(r0 + r) * m + j) = pack_bf16x2(xs[r][j], xs[r][j + 1]);
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

inline int64_t align256(int64_t bytes) { return (bytes + 255) & ~int64_t(255); }

struct FormSizes {
    int64_t blocks;
    int T, Tp, F, kp;
    int64_t dr, y, qt, z, zt, g, mm, wf, total;  // bytes per array over all blocks
};

bool form_sizes(const kamera_layout& L, int32_t n, int32_t T, int32_t k, FormSizes& fs) {
    fs.blocks = (int64_t)n * L.num_layers * L.num_streams;
    fs.T = T;
    fs.Tp = (T + kTileT - 1) / kTileT * kTileT;
    fs.F = L.num_heads * L.head_dim;
    fs.kp = k <= 32 ? 32 : 64;
    const int64_t bl = fs.blocks;
    fs.dr = align256(bl * fs.Tp * fs.F * 2);
    fs.y = align256(bl * fs.Tp * fs.kp * 4);
    fs.qt = align256(bl * fs.kp * fs.Tp * 2);
    fs.z = align256(bl * fs.F * fs.kp * 4);
    fs.zt = align256(bl * fs.kp * fs.F * 2);
    fs.g = align256(2 * bl * fs.kp * fs.kp * 8);  // two fp64 Gram matrices per block
    fs.mm = align256(bl * fs.kp * fs.kp * 4);  // R^-1 of each block
    fs.wf = align256(bl * fs.kp * kMaxKp * 4); // Wu or Wv of each block (m <= 64)
    fs.total = 2 * fs.dr + fs.y + 2 * fs.qt + fs.z + fs.zt + fs.g + fs.mm + 2 * fs.wf;
    return true;
}

kamera_status check_form_layout(const kamera_layout* L) {
    if (!L) return KAMERA_ERR_NULL;
    if (L->num_layers < 1 || L->num_layers > 65535 || L->num_heads < 1 || L->head_dim < 1) return KAMERA_ERR_RANGE;
    if (L->num_streams < 1 || L->num_streams > 2) return KAMERA_ERR_RANGE;
    if (L->rope_style != KAMERA_ROPE_HALF && L->rope_style != KAMERA_ROPE_INTERLEAVED) return KAMERA_ERR_RANGE;
    if (L->rope_offset < 0 || L->rope_dim < 0 || L->rope_offset + L->rope_dim > L->head_dim) return KAMERA_ERR_RANGE;
    if (!(L->rope_base > 0.0) || !isfinite(L->rope_base)) return KAMERA_ERR_RANGE;
    if (L->head_dim % 64 || L->rope_offset % 64 || L->rope_dim % 64) return KAMERA_ERR_UNSUPPORTED;
    if (L->head_dim > 1024 || (int64_t)L->num_heads * L->head_dim > 4096) return KAMERA_ERR_UNSUPPORTED;
    return KAMERA_OK;
}

kamera_status check_rows(const kamera_src* r, int S, int L, int T, int64_t F, int n) {
    if (!r) return KAMERA_ERR_NULL;
    for (int s = 0; s < S; ++s) {
        if (!r->rows[s]) return KAMERA_ERR_NULL;
        if (!aligned16(r->rows[s])) return KAMERA_ERR_ALIGN;
    }
    if (r->chunk_stride < 0 || r->layer_stride < 0) return KAMERA_ERR_RANGE;
    if (r->chunk_stride % 8 || r->layer_stride % 8) return KAMERA_ERR_ALIGN;
    if (r->n_tokens != T) return KAMERA_ERR_SHAPE;
    if (r->n_store < n) return KAMERA_ERR_RANGE;
    if (L > 1 && r->layer_stride < (int64_t)T * F) return KAMERA_ERR_SHAPE;
    if (n > 1 && r->chunk_stride < (int64_t)T * F) return KAMERA_ERR_SHAPE;
    return KAMERA_OK;
}

// Both formation entry points: views targets (and shifts) per chunk, whose
// deficits are averaged before the decomposition (views == 1: the plain patch).
kamera_status form_patch_impl(const kamera_layout* layout, const kamera_src* canon, const kamera_src* target,
                              int32_t n, int32_t views, const int64_t* delta, const kamera_sketch* sketch,
                              const kamera_factors* out, void* workspace, int64_t workspace_bytes,
                              void* hip_stream);

}  // namespace

extern "C" {

int64_t kamera_form_patch_workspace(const kamera_layout* layout, int32_t n, int32_t n_tokens, int32_t rank,
                                    int32_t oversample) {
    if (check_form_layout(layout) != KAMERA_OK || n < 0 || n_tokens < 0 || rank < 1 || oversample < 0 ||
        rank + oversample > kMaxKp)
        return -1;
    FormSizes fs;
    form_sizes(*layout, n, n_tokens, rank + oversample, fs);
    return fs.total;
}

kamera_status kamera_form_patch(const kamera_layout* layout, const kamera_src* canon, const kamera_src* target,
                                int32_t n, const int64_t* delta, const kamera_sketch* sketch,
                                const kamera_factors* out, void* workspace, int64_t workspace_bytes,
                                void* hip_stream) {
    return form_patch_impl(layout, canon, target, n, 1, delta, sketch, out, workspace, workspace_bytes, hip_stream);
}

kamera_status kamera_form_orbit_patch(const kamera_layout* layout, const kamera_src* canon,
                                      const kamera_src* targets, int32_t n, int32_t views, const int64_t* deltas,
                                      const kamera_sketch* sketch, const kamera_factors* out, void* workspace,
                                      int64_t workspace_bytes, void* hip_stream) {
    return form_patch_impl(layout, canon, targets, n, views, deltas, sketch, out, workspace, workspace_bytes,
                           hip_stream);
}

}  // extern "C"

namespace {

kamera_status form_patch_impl(const kamera_layout* layout, const kamera_src* canon, const kamera_src* target,
                              int32_t n, int32_t views, const int64_t* delta, const kamera_sketch* sketch,
                              const kamera_factors* out, void* workspace, int64_t workspace_bytes,
                              void* hip_stream) {
    kamera_status st = check_form_layout(layout);
    if (st != KAMERA_OK) return st;
    if (!canon || !target || !sketch || !out) return KAMERA_ERR_NULL;
    const kamera_layout& L = *layout;
    const int S = L.num_streams;
    const int64_t F = (int64_t)L.num_heads * L.head_dim;
    const int T = canon->n_tokens;
    if (n < 0 || T < 0 || views < 1 || (int64_t)n * views > INT32_MAX) return KAMERA_ERR_RANGE;
    const int nv = n * views;  // target chunks (and shifts)
    if ((st = check_rows(canon, S, L.num_layers, T, F, n)) != KAMERA_OK) return st;
    if ((st = check_rows(target, S, L.num_layers, T, F, nv)) != KAMERA_OK) return st;
    const int m = out->rank;
    if (m < 2 || m > kMaxKp || (m & 1)) return m < 0 || m > kMaxKp ? KAMERA_ERR_RANGE : KAMERA_ERR_UNSUPPORTED;
    if (sketch->oversample < 0 || sketch->power_iters < 0 || sketch->power_iters > 16) return KAMERA_ERR_RANGE;
    const int k = m + sketch->oversample;
    if (k > kMaxKp) return KAMERA_ERR_RANGE;
    if (!sketch->omega) return KAMERA_ERR_NULL;
    if (!aligned16(sketch->omega)) return KAMERA_ERR_ALIGN;
    for (int s = 0; s < S; ++s) {
        if (!out->u[s] || !out->v[s]) return KAMERA_ERR_NULL;
        if (((uintptr_t)out->u[s] & 3u) || ((uintptr_t)out->v[s] & 3u)) return KAMERA_ERR_ALIGN;
    }
    if (n == 0 || T == 0) return KAMERA_OK;
    if (!delta) return KAMERA_ERR_NULL;
    FormSizes fs;
    form_sizes(L, n, T, k, fs);
    if (fs.Tp > 65536 || (int64_t)fs.Tp * F > INT32_MAX) return KAMERA_ERR_RANGE;
    if (fs.blocks > 65535) return KAMERA_ERR_RANGE;
    if (!workspace) return KAMERA_ERR_NULL;
    if (((uintptr_t)workspace & 255u) != 0) return KAMERA_ERR_ALIGN;
    if (workspace_bytes < fs.total) return KAMERA_ERR_RANGE;
    // outputs must not overlap the inputs, each other or the workspace
    {
        const Span ws{(uintptr_t)workspace, (uintptr_t)workspace + (uintptr_t)fs.total};
        const int64_t u_el = (int64_t)n * L.num_layers * T * m, v_el = (int64_t)n * L.num_layers * F * m;
        const int64_t c_el = (int64_t)(n - 1) * canon->chunk_stride + (int64_t)(L.num_layers - 1) * canon->layer_stride + (int64_t)T * F;
        const int64_t t_el = (int64_t)(nv - 1) * target->chunk_stride + (int64_t)(L.num_layers - 1) * target->layer_stride + (int64_t)T * F;
        for (int s = 0; s < S; ++s) {
            const Span us = span_of(out->u[s], u_el), vs = span_of(out->v[s], v_el);
            if (overlap(us, vs) || overlap(us, ws) || overlap(vs, ws)) return KAMERA_ERR_ALIAS;
            for (int s2 = 0; s2 < S; ++s2) {
                const Span cs_ = span_of(canon->rows[s2], c_el), ts = span_of(target->rows[s2], t_el);
                if (overlap(us, cs_) || overlap(vs, cs_) || overlap(us, ts) || overlap(vs, ts)) return KAMERA_ERR_ALIAS;
                if (s2 != s && (overlap(us, span_of(out->u[s2], u_el)) || overlap(vs, span_of(out->v[s2], v_el)) ||
                                overlap(us, span_of(out->v[s2], v_el))))
                    return KAMERA_ERR_ALIAS;
            }
            if (overlap(ws, span_of(canon->rows[s], c_el)) || overlap(ws, span_of(target->rows[s], t_el)))
                return KAMERA_ERR_ALIAS;
        }
    }

    FormParams p;
    memset(&p, 0, sizeof(p));
    for (int s = 0; s < S; ++s) {
        p.canon[s] = canon->rows[s];
        p.target[s] = target->rows[s];
        p.u[s] = out->u[s];
        p.v[s] = out->v[s];
    }
    p.canon_chunk_stride = canon->chunk_stride;
    p.canon_layer_stride = canon->layer_stride;
    p.target_chunk_stride = target->chunk_stride;
    p.target_layer_stride = target->layer_stride;
    p.delta = delta;
    p.omega = sketch->omega;
    uint8_t* w = (uint8_t*)workspace;
    p.dr_hi = (uint16_t*)w; w += 2 * fs.dr;
    p.dr_lo = p.dr_hi + 64;
    p.y = (float*)w; w += fs.y;
    p.qt_hi = (uint16_t*)w; w += fs.qt;
    p.qt_lo = (uint16_t*)w; w += fs.qt;
    p.z = (float*)w; w += fs.z;
    p.zt_hi = (uint16_t*)w; w += fs.zt;
    p.g = (double*)w; w += fs.g;
    p.mm = (float*)w; w += fs.mm;
    p.wu = (float*)w; w += fs.wf;
    p.wv = (float*)w;
    p.log2_base = log2(L.rope_base);
    p.n = n;
    p.L = L.num_layers;
    p.S = S;
    p.T = T;
    p.Tp = fs.Tp;
    p.F = (int32_t)F;
    p.D = L.head_dim;
    p.rope_offset = L.rope_offset;
    p.rope_dim = L.rope_dim;
    p.rope_style = L.rope_style;
    p.m = m;
    p.k = k;
    p.kp = fs.kp;
    p.views = views;

    hipStream_t hs = (hipStream_t)hip_stream;
    const int nb = (int)fs.blocks;
    const int Tp = fs.Tp, kp = fs.kp, Fi = (int)F;
    // one view: the first product forms Delta itself (delta_sketch_kernel);
    // orbit calls take delta_kernel's pass first (holding every view's target
    // rows in registers spills at 64 columns: four views measured 2.27 ms for
    // the fused kernel against 2.23 ms for the two on MI355X)
    const bool fused = views == 1;
    hipError_t e = hipSuccess;
    if (!fused)
        e = launch_kernel(delta_kernel, dim3((unsigned)((Tp / kTileT) * (Fi / 64)), (unsigned)L.num_layers,
                                             (unsigned)(n * S)),
                          dim3(kFormThreads), hs, p);
    const int64_t gcount = (int64_t)nb * kp * kp;  // one Gram set
    const int nk = (k + 1) & ~1;  // sketch columns the small dense steps work on (even)
    double* g1 = p.g;
    double* g2 = p.g + gcount;
    auto zero_grams = [&]() {
        return launch_kernel(zero_kernel, dim3((unsigned)((2 * gcount + 255) / 256)), dim3(256), hs, p.g,
                             2 * gcount);
    };
    // out = A B (every block), with the Gram matrix of out into g1; ta: A =
    // Delta^T, read from Delta's row-major panels.  g1 and g2 are cleared once
    // per call (below); every kernel that reads a Gram matrix clears it after
    // reading, so the next one accumulates into zeros.
    auto sketch_launch = [&](bool ta, const uint16_t* ah, const uint16_t* al, int64_t ablk, const uint16_t* bh,
                             const uint16_t* bl, int64_t bblk, float* o, int64_t oblk, int R, int X, int nbv) {
        hipError_t r = hipSuccess;
        // one 128-row tile per workgroup (the kernel can walk several, with
        // one set of Gram atomics for all of them; with the Gram on the
        // matrix cores and only its lower tiles flushed, one tile is faster on
        // MI355X: MLA's 4096-row products 1039 -> 950 us against four tiles,
        // the orbit's 2048-row ones 542 -> 501 us against two)
        const int rtiles = 1;
        SketchArgs sa{ah, al, ablk, bh, bl, bblk, o, oblk, g1, R, X, nbv, rtiles};
        const dim3 grid((unsigned)((R + 128 * rtiles - 1) / (128 * rtiles)), (unsigned)nb);
        if (r != hipSuccess) return r;
        auto go = [&](auto kern) { return launch_kernel(kern, grid, dim3(256), hs, sa); };
        auto pick = [&](auto ta_tag) {
            constexpr bool TA = decltype(ta_tag)::value;
            if ((X / 64) % 2 == 0 || kp == 64) {  // two chunks in flight
                if (kp == 32) return bl ? go(sketch_kernel<1, true, true, TA>) : go(sketch_kernel<1, false, true, TA>);
                return bl ? go(sketch_kernel<2, true, true, TA>) : go(sketch_kernel<2, false, true, TA>);
            }
            if (kp == 32) return bl ? go(sketch_kernel<1, true, false, TA>) : go(sketch_kernel<1, false, false, TA>);
            return bl ? go(sketch_kernel<2, true, false, TA>) : go(sketch_kernel<2, false, false, TA>);
        };
        return ta ? pick(std::true_type{}) : pick(std::false_type{});
    };
    // orthonormalize X whose Gram matrix is in g1 and write its bf16
    // transpose: two Cholesky QR passes for the basis the factors come from,
    // one for the bases inside the power iteration, which only have to span
    // the right subspace (a shifted Cholesky QR pass keeps the span exactly)
    auto orth_launch = [&](float* x, int64_t xblk, uint16_t* xth, uint16_t* xtl, int64_t xtblk, int R,
                           bool final_basis) {
        auto chol = [&](double* gg) {
            return kp == 32 ? launch_kernel(chol_lds_kernel<32>, dim3((unsigned)nb), dim3(256), hs, gg, p.mm, nk)
                            : launch_kernel(chol_lds_kernel<64>, dim3((unsigned)nb), dim3(256), hs, gg, p.mm, nk);
        };
        // the fp32 rows are stored back only where a later step reads them: the
        // first pass of a final basis (the second pass's input) and the final
        // basis itself (the factors' U); the power iteration's bases are read
        // only through their bf16 transpose
        // a tall X takes several 128-row tiles per workgroup, the next tile's
        // rows in flight during each tile's work: four at 4096 rows, a quarter
        // of the Gram atomics (MLA's final basis: 1326 -> 562 us per pass on
        // MI355X; eight tiles measured the same, transposes 243 -> 194 us; one
        // or two tiles slower), two at 2048 rows (orbit applies 92.7 -> 89 us
        // against four)
        auto apply = [&](double* gnext, uint16_t* th, uint16_t* tl, int64_t tblk, int store) {
            const int rt = R >= 4096 ? 4 : (R >= 2048 ? 2 : 1);
            const dim3 ga((unsigned)((R + 128 * rt - 1) / (128 * rt)), (unsigned)nb);
            auto go = [&](auto kern) {
                return launch_kernel(kern, ga, dim3(256), hs, x, xblk, R, (const float*)p.mm, gnext, th, tl, tblk,
                                     store, rt);
            };
            if (gnext) return kp == 32 ? go(apply_kernel<32, true>) : go(apply_kernel<64, true>);
            return kp == 32 ? go(apply_kernel<32, false>) : go(apply_kernel<64, false>);
        };
        hipError_t r = chol(g1);
        if (final_basis) {
            if (r == hipSuccess) r = apply(g2, nullptr, nullptr, 0, 1);
            if (r == hipSuccess) r = chol(g2);
        }
        if (r == hipSuccess) r = apply(nullptr, xth, xtl, xtblk, final_basis ? 1 : 0);
        return r;
    };
    const int64_t drb = (int64_t)Tp * Fi * 2, yb = (int64_t)Tp * kp, zb = (int64_t)Fi * kp;
    // Y = Delta Omega with Delta formed and stored on the way, one 128-row
    // tile per workgroup (on MI355X, MLA: 1775 us with four tiles per
    // workgroup as the other row-major products take, 1740 with two, 1680
    // with one)
    auto delta_sketch_launch = [&]() {
        const int rtiles = 1;
        SketchArgs sa{p.dr_hi, p.dr_lo, drb, p.omega, nullptr, 0, p.y, yb, g1, Tp, Fi, k, rtiles};
        const dim3 grid((unsigned)((Tp + 128 * rtiles - 1) / (128 * rtiles)), (unsigned)nb);
        auto go = [&](auto kern) { return launch_kernel(kern, grid, dim3(256), hs, sa, p); };
        // two chunks in flight at 32 columns with an even chunk count; at 64
        // columns the second register set spills (MLA: 1.83 against 1.78 ms)
        if (kp == 32 && (Fi / 64) % 2 == 0) return go(delta_sketch_kernel<1, true, 1>);
        return kp == 32 ? go(delta_sketch_kernel<1, false, 1>) : go(delta_sketch_kernel<2, false, 1>);
    };
    const int q = sketch->power_iters;
    // Y = Delta Omega, Q = orth(Y)
    if (e == hipSuccess) e = zero_grams();
    if (e == hipSuccess)
        e = fused ? delta_sketch_launch()
                  : sketch_launch(false, p.dr_hi, p.dr_lo, drb, p.omega, nullptr, 0, p.y, yb, Tp, Fi, k);
    if (e == hipSuccess) e = orth_launch(p.y, yb, p.qt_hi, q == 0 ? p.qt_lo : nullptr, yb, Tp, q == 0);
    for (int it = 0; it < q && e == hipSuccess; ++it) {
        // Z = orth(Delta^T Q); Y = Delta Z; Q = orth(Y)
        e = sketch_launch(true, p.dr_hi, p.dr_lo, drb, p.qt_hi, nullptr, yb, p.z, zb, Fi, Tp, kp);
        if (e == hipSuccess) e = orth_launch(p.z, zb, p.zt_hi, nullptr, zb, Fi, false);
        if (e == hipSuccess) e = sketch_launch(false, p.dr_hi, p.dr_lo, drb, p.zt_hi, nullptr, zb, p.y, yb, Tp, Fi, kp);
        if (e == hipSuccess) e = orth_launch(p.y, yb, p.qt_hi, it == q - 1 ? p.qt_lo : nullptr, yb, Tp, it == q - 1);
    }
    // Z = Delta^T Q with Q split in hi + lo (and Z^T Z into g1); eigenvectors; the factors
    if (e == hipSuccess) e = sketch_launch(true, p.dr_hi, p.dr_lo, drb, p.qt_hi, p.qt_lo, yb, p.z, zb, Fi, Tp, kp);
    if (e == hipSuccess) {
        auto eig = [&](auto kern) {
            return launch_kernel(kern, dim3((unsigned)nb), dim3(256), hs, g1, (const float*)p.z, zb,
                                 Fi, m, nk, p.wu, p.wv);
        };
        e = kp == 32 ? eig(eig_kernel<32>) : eig(eig_kernel<64>);
    }
    if (e == hipSuccess) {
        OutArgs oa;
        oa.q = p.y;
        oa.z = p.z;
        oa.q_block = yb;
        oa.z_block = zb;
        oa.wu = p.wu;
        oa.wv = p.wv;
        oa.m = m;
        oa.T = T;
        oa.F = Fi;
        oa.L = L.num_layers;
        oa.S = S;
        for (int s = 0; s < 2; ++s) {
            oa.u[s] = s < S ? out->u[s] : nullptr;
            oa.v[s] = s < S ? out->v[s] : nullptr;
        }
        const dim3 go((unsigned)((T + 127) / 128 + (Fi + 127) / 128), (unsigned)nb);
        e = kp == 32 ? launch_kernel(out_kernel<32>, go, dim3(256), hs, oa)
                     : launch_kernel(out_kernel<64>, go, dim3(256), hs, oa);
    }
    return e == hipSuccess ? KAMERA_OK : KAMERA_ERR_HIP;
}

}  // namespace
