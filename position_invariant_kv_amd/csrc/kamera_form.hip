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
//    (Delta - hi), stored row-major [Tp][F] and column-major [F][Tp], so that
//    both products below read 16-byte MFMA operand rows.
//  * sketch_kernel: out[R][kp] = A[R][X] B[X][kp] on v_mfma_f32_32x32x16_bf16
//    with A = hi + lo (two products, or three with a split B): Delta Omega,
//    Delta Z (A row-major) and Delta^T Q (A column-major).
//  * orth_kernel: one workgroup per block orthonormalizes the columns of
//    X [R][kp] by the eigenvectors of its fp64 Gram matrix (SVQB: X <- X W
//    L^(-1/2), directions with L <= 1e-13 L_max dropped), twice, and writes
//    the bf16 transpose the next product reads.
//  * final_kernel: B B^T = Z^T Z, its eigenvectors, and the bf16 factors
//    with the oracle's conventions (V column's largest entry positive,
//    singular values <= 1e-6 sigma_1 give zero columns).
// The small symmetric eigenproblems use the cyclic Jacobi method with the
// round-robin parallel ordering (Golub & Van Loan, Matrix Computations,
// sections 8.5.2 and 8.5.5) in fp64, one workgroup per block.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "kamera.h"
#include "kamera_common.h"

namespace {

constexpr int kFormThreads = 256;
constexpr int kMaxKp = 64;            // sketch columns after padding (32 or 64)
constexpr int kMaxHalfRopeF = 512;
constexpr int kTileT = 64;            // delta_kernel tile: 64 tokens x 64 features
constexpr double kDropL = 1e-13;      // SVQB: eigenvalues <= kDropL * L_max are dropped
constexpr double kNegligible = 1e-6;  // factors: sigma <= kNegligible * sigma_1 -> zero column
constexpr int kMaxSweeps = 30;

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
    uint16_t *dr_hi, *dr_lo;  // [Tp][F]
    uint16_t *dc_hi, *dc_lo;  // [F][Tp]
    float* y;                 // [Tp][kp]
    uint16_t *qt_hi, *qt_lo;  // [kp][Tp]
    float* z;                 // [F][kp]
    uint16_t* zt_hi;          // [kp][F]
    double log2_base;
    int32_t n, L, S, T, Tp, F, D, rope_offset, rope_dim, rope_style;
    int32_t m, k, kp;
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

// ---------------------------------------------------------------------------
// Delta = target - R(delta) canon, split hi/lo, row- and column-major
// ---------------------------------------------------------------------------
//
// Grid: x = token tile * (F/64) + feature tile, y = layer, z = chunk * S +
// stream.  A 256-thread workgroup owns 64 tokens x 64 features: each thread
// forms two 8-feature vectors (loading the rotate-half partner vector of the
// canonical row when the feature is rotated), stores them row-major and parks
// them in LDS, then stores 8-token vectors of the transpose.  Rows past T are
// zero.
__global__ __launch_bounds__(kFormThreads) void delta_kernel(const FormParams p) {
    __shared__ float2 cs[kMaxHalfRopeF];
    __shared__ uint16_t hi_t[kTileT][kTileT + 8];
    __shared__ uint16_t lo_t[kTileT][kTileT + 8];
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
    if (rot) {
        const int64_t delta = p.delta[i];
        for (int j = threadIdx.x; j < half; j += kFormThreads) cs[j] = rope_cos_sin(p.log2_base, p.rope_dim, j, delta);
    }
    __syncthreads();
    const uint16_t* cb = p.canon[s] + (int64_t)i * p.canon_chunk_stride + (int64_t)l * p.canon_layer_stride;
    const uint16_t* tb = p.target[s] + (int64_t)i * p.target_chunk_stride + (int64_t)l * p.target_layer_stride;
    uint16_t* drh = p.dr_hi + b * p.Tp * p.F;
    uint16_t* drl = p.dr_lo + b * p.Tp * p.F;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int q = threadIdx.x + kk * kFormThreads;
        const int r = q >> 3, cv = q & 7;
        const int t = t0 + r;
        const int f = f0 + 8 * cv;
        float d[8];
        if (t < p.T) {
            const u32x4 tv = ld_cached(tb + (int64_t)t * p.F + f);
            const u32x4 cvv = ld_cached(cb + (int64_t)t * p.F + f);
            float c8[8];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                c8[2 * w] = bf_lo(cvv[w]);
                c8[2 * w + 1] = bf_hi(cvv[w]);
            }
            const int e = (f % p.D) - p.rope_offset;  // vector start inside the rotary span
            if (rot && e >= 0 && e < p.rope_dim) {
                if (p.rope_style == KAMERA_ROPE_HALF) {
                    const bool first = e < half;
                    const u32x4 pv = ld_cached(cb + (int64_t)t * p.F + f + (first ? half : -half));
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
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                d[2 * w] = bf_lo(tv[w]) - c8[2 * w];
                d[2 * w + 1] = bf_hi(tv[w]) - c8[2 * w + 1];
            }
        } else {
#pragma unroll
            for (int w = 0; w < 8; ++w) d[w] = 0.0f;
        }
        u32x4 h, lo;
        split8(d, h, lo);
        *reinterpret_cast<u32x4*>(drh + (int64_t)t * p.F + f) = h;
        *reinterpret_cast<u32x4*>(drl + (int64_t)t * p.F + f) = lo;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            hi_t[r][8 * cv + 2 * w] = (uint16_t)(h[w] & 0xffffu);
            hi_t[r][8 * cv + 2 * w + 1] = (uint16_t)(h[w] >> 16);
            lo_t[r][8 * cv + 2 * w] = (uint16_t)(lo[w] & 0xffffu);
            lo_t[r][8 * cv + 2 * w + 1] = (uint16_t)(lo[w] >> 16);
        }
    }
    __syncthreads();
    uint16_t* dch = p.dc_hi + b * p.F * p.Tp;
    uint16_t* dcl = p.dc_lo + b * p.F * p.Tp;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int q = threadIdx.x + kk * kFormThreads;
        const int fi = q >> 3, tv = q & 7;  // feature of the tile, 8-token vector
        u32x4 h, lo;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            h[w] = (uint32_t)hi_t[8 * tv + 2 * w][fi] | ((uint32_t)hi_t[8 * tv + 2 * w + 1][fi] << 16);
            lo[w] = (uint32_t)lo_t[8 * tv + 2 * w][fi] | ((uint32_t)lo_t[8 * tv + 2 * w + 1][fi] << 16);
        }
        *reinterpret_cast<u32x4*>(dch + (int64_t)(f0 + fi) * p.Tp + t0 + 8 * tv) = h;
        *reinterpret_cast<u32x4*>(dcl + (int64_t)(f0 + fi) * p.Tp + t0 + 8 * tv) = lo;
    }
}

// ---------------------------------------------------------------------------
// out[R][kp] = (A_hi + A_lo)[R][X] B[X][kp], B given transposed: bt[kp][X]
// ---------------------------------------------------------------------------
//
// v_mfma_f32_32x32x16_bf16: lane l holds A[l%32][8(l/32) .. +8] and
// B[8(l/32) .. +8][l%32]; its 16 results are D[8(v/4) + 4(l/32) + v%4][l%32].
// A workgroup of four waves owns 32 rows and all kp = 32 KC columns; the
// waves take interleaved 16-wide slices of X and their partial sums are added
// through LDS.  Columns of B at or past nb_valid read as zero.  With a low
// part of B (bt_lo) the product adds hi*lo_B as well (three products).
struct SketchArgs {
    const uint16_t* a_hi;
    const uint16_t* a_lo;
    int64_t a_block;        // elements between blocks of A
    const uint16_t* bt_hi;
    const uint16_t* bt_lo;  // may be NULL
    int64_t bt_block;       // elements between blocks of B (0: shared)
    float* out;
    int64_t out_block;
    int32_t R, X;           // rows, inner length (multiple of 16)
    int32_t nb_valid;       // columns of B that exist (others are zero)
};

template <int KC, bool SPLIT_B>
__global__ __launch_bounds__(256) void sketch_kernel(const SketchArgs a) {
    __shared__ float part[3][KC][16][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int hh = lane >> 5, col = lane & 31;
    const int64_t b = blockIdx.y;
    const int r0 = blockIdx.x * 32;
    const uint16_t* ah = a.a_hi + b * a.a_block + (int64_t)(r0 + col) * a.X + 8 * hh;
    const uint16_t* al = a.a_lo + b * a.a_block + (int64_t)(r0 + col) * a.X + 8 * hh;
    const uint16_t* bh[KC];
    const uint16_t* bl[KC];
    bool bvalid[KC];
#pragma unroll
    for (int cb = 0; cb < KC; ++cb) {
        const int c = cb * 32 + col;
        bvalid[cb] = c < a.nb_valid;
        const int cc = bvalid[cb] ? c : 0;
        bh[cb] = a.bt_hi + b * a.bt_block + (int64_t)cc * a.X + 8 * hh;
        bl[cb] = SPLIT_B ? a.bt_lo + b * a.bt_block + (int64_t)cc * a.X + 8 * hh : nullptr;
    }
    f32x16 acc[KC];
#pragma unroll
    for (int cb = 0; cb < KC; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[cb][v] = 0.0f;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const int steps = a.X / 16;
    for (int st = wave; st < steps; st += 4) {
        const int x0 = st * 16;
        const bf16x8 A0 = __builtin_bit_cast(bf16x8, ld_cached(ah + x0));
        const bf16x8 A1 = __builtin_bit_cast(bf16x8, ld_cached(al + x0));
#pragma unroll
        for (int cb = 0; cb < KC; ++cb) {
            const u32x4 bw = ld_cached(bh[cb] + x0);
            const bf16x8 B0 = __builtin_bit_cast(bf16x8, bvalid[cb] ? bw : zero);
            acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, B0, acc[cb], 0, 0, 0);
            acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B0, acc[cb], 0, 0, 0);
            if (SPLIT_B) {
                const u32x4 bw2 = ld_cached(bl[cb] + x0);
                const bf16x8 B1 = __builtin_bit_cast(bf16x8, bvalid[cb] ? bw2 : zero);
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, B1, acc[cb], 0, 0, 0);
            }
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int cb = 0; cb < KC; ++cb)
#pragma unroll
            for (int v = 0; v < 16; ++v) part[wave - 1][cb][v][lane] = acc[cb][v];
    }
    __syncthreads();
    if (wave == 0) {
        float* o = a.out + b * a.out_block;
#pragma unroll
        for (int cb = 0; cb < KC; ++cb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float sum = acc[cb][v] + part[0][cb][v][lane] + part[1][cb][v][lane] + part[2][cb][v][lane];
                const int row = 8 * (v >> 2) + 4 * hh + (v & 3);
                o[(int64_t)(r0 + row) * (KC * 32) + cb * 32 + col] = sum;
            }
    }
}

// ---------------------------------------------------------------------------
// Workgroup routines for one block: fp64 Gram matrix and Jacobi eigenvectors
// ---------------------------------------------------------------------------

// G = X^T X (kp x kp, fp64, into LDS g) for X [R][kp] fp32 in global memory;
// rows are staged 64 at a time in LDS (xs).  Thread (ti, tj) owns a
// (kp/16) x (kp/16) square of G.
__device__ void gram64(const float* __restrict__ x, int R, int kp, float (*xs)[kMaxKp], double* g) {
    const int bs = kp / 16;
    const int ti = threadIdx.x >> 4, tj = threadIdx.x & 15;
    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
    for (int r0 = 0; r0 < R; r0 += 64) {
        const int rows = min(64, R - r0);
        __syncthreads();
        for (int q = threadIdx.x; q < 64 * kp; q += blockDim.x) {
            const int r = q / kp, c = q - r * kp;
            xs[r][c] = r < rows ? x[(int64_t)(r0 + r) * kp + c] : 0.0f;
        }
        __syncthreads();
        for (int r = 0; r < rows; ++r) {
            double av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[i] = i < bs ? (double)xs[r][ti * bs + i] : 0.0;
                bv[i] = i < bs ? (double)xs[r][tj * bs + i] : 0.0;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fma(av[i], bv[j], acc[i][j]);
        }
    }
    for (int i = 0; i < bs; ++i)
        for (int j = 0; j < bs; ++j) g[(ti * bs + i) * kp + tj * bs + j] = acc[i][j];
    __syncthreads();
}

// Eigen-decomposition G = W diag(G') W^T of the symmetric kp x kp matrix g
// (fp64, LDS, overwritten by G' whose diagonal holds the eigenvalues) by
// cyclic Jacobi with the round-robin ordering: each step rotates kp/2
// disjoint pairs at once (rows first, then columns, which together give
// J^T G J), kp - 1 steps per sweep, until the off-diagonal mass is below
// 1e-30 of the diagonal's (or kMaxSweeps sweeps).  w: kp x kp, LDS.
__device__ void jacobi_eig(double* g, double* w, int kp, double* rot_c, double* rot_s, int* pp, int* qq,
                           double* red) {
    const int tid = threadIdx.x;
    for (int q = tid; q < kp * kp; q += blockDim.x) w[q] = (q / kp == q % kp) ? 1.0 : 0.0;
    const int np = kp / 2;
    for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
        __syncthreads();
        // convergence: off-diagonal vs diagonal mass
        double off = 0.0, dia = 0.0;
        for (int q = tid; q < kp * kp; q += blockDim.x) {
            const double e = g[q];
            if (q / kp == q % kp) dia += e * e; else off += e * e;
        }
        red[tid] = off;
        red[blockDim.x + tid] = dia;
        __syncthreads();
        for (int h = blockDim.x / 2; h > 0; h >>= 1) {
            if (tid < h) {
                red[tid] += red[tid + h];
                red[blockDim.x + tid] += red[blockDim.x + tid + h];
            }
            __syncthreads();
        }
        const bool done = red[0] <= 1e-30 * red[blockDim.x];
        __syncthreads();
        if (done) break;
        for (int step = 0; step < kp - 1; ++step) {
            // pairs of this step and their rotations
            if (tid < np) {
                auto slot = [&](int a) { return a == 0 ? 0 : ((a - 1 + step) % (kp - 1)) + 1; };
                int p = slot(tid), q = slot(kp - 1 - tid);
                if (p > q) { const int t = p; p = q; q = t; }
                const double apq = g[p * kp + q];
                double c = 1.0, s = 0.0;
                if (apq != 0.0) {
                    const double theta = (g[q * kp + q] - g[p * kp + p]) / (2.0 * apq);
                    const double t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
                    c = 1.0 / sqrt(t * t + 1.0);
                    s = t * c;
                }
                pp[tid] = p;
                qq[tid] = q;
                rot_c[tid] = c;
                rot_s[tid] = s;
            }
            __syncthreads();
            // rows: G <- J^T G
            for (int u = tid; u < np * kp; u += blockDim.x) {
                const int pr = u / kp, k = u - pr * kp;
                const int p = pp[pr], q = qq[pr];
                const double c = rot_c[pr], s = rot_s[pr];
                const double gp = g[p * kp + k], gq = g[q * kp + k];
                g[p * kp + k] = c * gp - s * gq;
                g[q * kp + k] = s * gp + c * gq;
            }
            __syncthreads();
            // columns: G <- G J, W <- W J
            for (int u = tid; u < np * kp; u += blockDim.x) {
                const int pr = u / kp, k = u - pr * kp;
                const int p = pp[pr], q = qq[pr];
                const double c = rot_c[pr], s = rot_s[pr];
                const double gp = g[k * kp + p], gq = g[k * kp + q];
                g[k * kp + p] = c * gp - s * gq;
                g[k * kp + q] = s * gp + c * gq;
                const double wp = w[k * kp + p], wq = w[k * kp + q];
                w[k * kp + p] = c * wp - s * wq;
                w[k * kp + q] = s * wp + c * wq;
            }
            __syncthreads();
        }
    }
    __syncthreads();
}

// Shared memory of the per-block workgroups.
struct SmallLds {
    double g[kMaxKp * kMaxKp];
    double w[kMaxKp * kMaxKp];
    float xs[64][kMaxKp];
    float mt[kMaxKp][kMaxKp];   // the kp x kp factor applied to the rows
    double rot_c[kMaxKp / 2], rot_s[kMaxKp / 2];
    int pp[kMaxKp / 2], qq[kMaxKp / 2];
    double red[2 * kFormThreads];
    double lam[kMaxKp];
    int order[kMaxKp];
};

// ---------------------------------------------------------------------------
// Orthonormalize the columns of X [R][kp] (SVQB, twice) and write X^T in bf16
// ---------------------------------------------------------------------------
//
// One workgroup per block (grid y).  X <- X W L^(-1/2) with the eigenvectors
// W and eigenvalues L of X^T X; directions with L <= kDropL L_max become zero
// columns.  The second pass starts from a nearly orthonormal X, so its Jacobi
// converges in a sweep or two.  Then xt_hi[kp][R] = bf16(X^T), and with
// xt_lo the low part as well.
struct OrthArgs {
    float* x;
    int64_t x_block;
    uint16_t* xt_hi;
    uint16_t* xt_lo;  // may be NULL
    int64_t xt_block;
    int32_t R, kp;
};

__global__ __launch_bounds__(kFormThreads) void orth_kernel(const OrthArgs a) {
    __shared__ SmallLds sm;
    const int tid = threadIdx.x;
    const int kp = a.kp;
    float* x = a.x + (int64_t)blockIdx.y * a.x_block;
    for (int pass = 0; pass < 2; ++pass) {
        gram64(x, a.R, kp, sm.xs, sm.g);
        jacobi_eig(sm.g, sm.w, kp, sm.rot_c, sm.rot_s, sm.pp, sm.qq, sm.red);
        double lmax = 0.0;
        for (int c = 0; c < kp; ++c) lmax = fmax(lmax, sm.g[c * kp + c]);
        // mt[c][j] = W[c][j] / sqrt(L_j), or 0 for a dropped direction
        for (int q = tid; q < kp * kp; q += blockDim.x) {
            const int c = q / kp, j = q - c * kp;
            const double lj = sm.g[j * kp + j];
            sm.mt[c][j] = (lj > kDropL * lmax && lj > 0.0) ? (float)(sm.w[c * kp + j] / sqrt(lj)) : 0.0f;
        }
        __syncthreads();
        // X <- X mt, 64 rows at a time through LDS
        const int cpt = kp / 4;  // output columns per thread (4 threads per row)
        for (int r0 = 0; r0 < a.R; r0 += 64) {
            const int rows = min(64, a.R - r0);
            __syncthreads();
            for (int q = tid; q < 64 * kp; q += blockDim.x) {
                const int r = q / kp, c = q - r * kp;
                sm.xs[r][c] = r < rows ? x[(int64_t)(r0 + r) * kp + c] : 0.0f;
            }
            __syncthreads();
            const int r = tid >> 2, j0 = (tid & 3) * cpt;
            float out[16];
            for (int j = 0; j < cpt; ++j) out[j] = 0.0f;
            for (int c = 0; c < kp; ++c) {
                const float xv = sm.xs[r][c];
                for (int j = 0; j < cpt; ++j) out[j] = fmaf(xv, sm.mt[c][j0 + j], out[j]);
            }
            __syncthreads();
            for (int j = 0; j < cpt; ++j) sm.xs[r][j0 + j] = out[j];
            __syncthreads();
            if (r < rows)
                for (int j = 0; j < cpt; ++j) x[(int64_t)(r0 + r) * kp + j0 + j] = out[j];
            if (pass == 1) {
                // transpose: column c, 16 rows per thread (kp columns x 64 rows)
                for (int q = tid; q < kp * 4; q += blockDim.x) {
                    const int c = q >> 2, rr = (q & 3) * 16;
                    u32x4 h0, h1, l0, l1;
                    float v[16];
                    for (int e = 0; e < 16; ++e) v[e] = sm.xs[rr + e][c];
                    float va[8], vb[8];
                    for (int e = 0; e < 8; ++e) { va[e] = v[e]; vb[e] = v[8 + e]; }
                    split8(va, h0, l0);
                    split8(vb, h1, l1);
                    uint16_t* dh = a.xt_hi + (int64_t)blockIdx.y * a.xt_block + (int64_t)c * a.R + r0 + rr;
                    if (r0 + rr + 16 <= a.R) {
                        *reinterpret_cast<u32x4*>(dh) = h0;
                        *reinterpret_cast<u32x4*>(dh + 8) = h1;
                        if (a.xt_lo) {
                            uint16_t* dl = a.xt_lo + (int64_t)blockIdx.y * a.xt_block + (int64_t)c * a.R + r0 + rr;
                            *reinterpret_cast<u32x4*>(dl) = l0;
                            *reinterpret_cast<u32x4*>(dl + 8) = l1;
                        }
                    }
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Factors from Z = Delta^T Q and Q: U = Q W_m L_m^(1/2), V = Z W_m L_m^(-1/2)
// ---------------------------------------------------------------------------
struct FinalArgs {
    const float* q;  // [Tp][kp] per block
    const float* z;  // [F][kp] per block
    int64_t q_block, z_block;
    int32_t kp, m, T, Tp, F, L, S;
    uint16_t* u[2];
    uint16_t* v[2];
};

__global__ __launch_bounds__(kFormThreads) void final_kernel(const FinalArgs a) {
    __shared__ SmallLds sm;
    __shared__ float sgn[kMaxKp];
    __shared__ float vmax[kFormThreads];
    __shared__ int vidx[kFormThreads];
    const int tid = threadIdx.x;
    const int kp = a.kp, m = a.m;
    const int64_t blk = blockIdx.y;  // ((i * S) + s) * L + l
    const int l = (int)(blk % a.L);
    const int s = (int)((blk / a.L) % a.S);
    const int i = (int)(blk / ((int64_t)a.L * a.S));
    const float* z = a.z + blk * a.z_block;
    const float* q = a.q + blk * a.q_block;
    gram64(z, a.F, kp, sm.xs, sm.g);
    jacobi_eig(sm.g, sm.w, kp, sm.rot_c, sm.rot_s, sm.pp, sm.qq, sm.red);
    // eigenvalues in descending order (ties: lower index first)
    if (tid < kp) sm.lam[tid] = sm.g[tid * kp + tid];
    __syncthreads();
    if (tid < kp) {
        const double me = sm.lam[tid];
        int rank = 0;
        for (int c = 0; c < kp; ++c) {
            const double o = sm.lam[c];
            rank += (o > me) || (o == me && c < tid);
        }
        sm.order[rank] = tid;
    }
    __syncthreads();
    const double l1 = fmax(sm.lam[sm.order[0]], 0.0);
    // mt[c][j]: columns j < m of W in eigenvalue order, scaled for V (1/sigma);
    // sm.red[j] holds sigma_j (0 for a negligible direction)
    if (tid < m) {
        const double lj = tid < kp ? fmax(sm.lam[sm.order[tid]], 0.0) : 0.0;
        const double sj = sqrt(lj);
        sm.red[tid] = (tid < kp && sj > kNegligible * sqrt(l1) && sj > 0.0) ? sj : 0.0;
    }
    __syncthreads();
    for (int e = tid; e < kp * m; e += blockDim.x) {
        const int c = e / m, j = e - c * m;
        const double sj = sm.red[j];
        sm.mt[c][j] = sj > 0.0 ? (float)(sm.w[c * kp + sm.order[j]] / sj) : 0.0f;
    }
    __syncthreads();
    // sign: largest |V| entry of every column, first on ties
    for (int j = 0; j < m; ++j) {
        float best = -1.0f;
        int bi = 0x7fffffff;
        for (int f = tid; f < a.F; f += blockDim.x) {
            float vv = 0.0f;
            for (int c = 0; c < kp; ++c) vv = fmaf(z[(int64_t)f * kp + c], sm.mt[c][j], vv);
            const float av = fabsf(vv);
            if (av > best) { best = av; bi = f; }  // f increases: the first max stays
            if (av == best && f < bi) bi = f;
        }
        vmax[tid] = best;
        vidx[tid] = bi;
        __syncthreads();
        for (int h = blockDim.x / 2; h > 0; h >>= 1) {
            if (tid < h) {
                const float o = vmax[tid + h];
                const int oi = vidx[tid + h];
                if (o > vmax[tid] || (o == vmax[tid] && oi < vidx[tid])) {
                    vmax[tid] = o;
                    vidx[tid] = oi;
                }
            }
            __syncthreads();
        }
        if (tid == 0) {
            const int f = vidx[0];
            float vv = 0.0f;
            if (f >= 0 && f < a.F)
                for (int c = 0; c < kp; ++c) vv = fmaf(z[(int64_t)f * kp + c], sm.mt[c][j], vv);
            sgn[j] = vv < 0.0f ? -1.0f : 1.0f;
        }
        __syncthreads();
    }
    // V [F][m] and U [T][m] in bf16 (m even: pairs of columns per 32-bit store)
    uint16_t* vo = a.v[s] + (((int64_t)i * a.L + l) * a.F) * m;
    uint16_t* uo = a.u[s] + (((int64_t)i * a.L + l) * a.T) * m;
    for (int e = tid; e < a.F * (m / 2); e += blockDim.x) {
        const int f = e / (m / 2), j = 2 * (e - f * (m / 2));
        float v0 = 0.0f, v1 = 0.0f;
        for (int c = 0; c < kp; ++c) {
            const float zv = z[(int64_t)f * kp + c];
            v0 = fmaf(zv, sm.mt[c][j], v0);
            v1 = fmaf(zv, sm.mt[c][j + 1], v1);
        }
        *reinterpret_cast<uint32_t*>(vo + (int64_t)f * m + j) = pack_bf16x2(v0 * sgn[j], v1 * sgn[j + 1]);
    }
    for (int e = tid; e < a.T * (m / 2); e += blockDim.x) {
        const int t = e / (m / 2), j = 2 * (e - t * (m / 2));
        float u0 = 0.0f, u1 = 0.0f;
        const double s0 = sm.red[j], s1 = sm.red[j + 1];
        for (int c = 0; c < kp; ++c) {
            const float qv = q[(int64_t)t * kp + c];
            // W[c][order[j]] * sigma_j = mt[c][j] * sigma_j^2
            u0 = fmaf(qv, (float)(sm.w[c * kp + sm.order[j]] * s0), u0);
            u1 = fmaf(qv, (float)(sm.w[c * kp + sm.order[j + 1]] * s1), u1);
        }
        *reinterpret_cast<uint32_t*>(uo + (int64_t)t * m + j) = pack_bf16x2(u0 * sgn[j], u1 * sgn[j + 1]);
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

inline int64_t align256(int64_t bytes) { return (bytes + 255) & ~int64_t(255); }

struct FormSizes {
    int64_t blocks;
    int T, Tp, F, kp;
    int64_t dr, dc, y, qt, z, zt, total;  // bytes per array over all blocks
};

bool form_sizes(const kamera_layout& L, int32_t n, int32_t T, int32_t k, FormSizes& fs) {
    fs.blocks = (int64_t)n * L.num_layers * L.num_streams;
    fs.T = T;
    fs.Tp = (T + kTileT - 1) / kTileT * kTileT;
    fs.F = L.num_heads * L.head_dim;
    fs.kp = k <= 32 ? 32 : 64;
    const int64_t bl = fs.blocks;
    fs.dr = align256(bl * fs.Tp * fs.F * 2);
    fs.dc = fs.dr;
    fs.y = align256(bl * fs.Tp * fs.kp * 4);
    fs.qt = align256(bl * fs.kp * fs.Tp * 2);
    fs.z = align256(bl * fs.F * fs.kp * 4);
    fs.zt = align256(bl * fs.kp * fs.F * 2);
    fs.total = 2 * fs.dr + 2 * fs.dc + fs.y + 2 * fs.qt + fs.z + fs.zt;
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
    kamera_status st = check_form_layout(layout);
    if (st != KAMERA_OK) return st;
    if (!canon || !target || !sketch || !out) return KAMERA_ERR_NULL;
    const kamera_layout& L = *layout;
    const int S = L.num_streams;
    const int64_t F = (int64_t)L.num_heads * L.head_dim;
    const int T = canon->n_tokens;
    if (n < 0 || T < 0) return KAMERA_ERR_RANGE;
    if ((st = check_rows(canon, S, L.num_layers, T, F, n)) != KAMERA_OK) return st;
    if ((st = check_rows(target, S, L.num_layers, T, F, n)) != KAMERA_OK) return st;
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
        const int64_t t_el = (int64_t)(n - 1) * target->chunk_stride + (int64_t)(L.num_layers - 1) * target->layer_stride + (int64_t)T * F;
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
    p.dr_hi = (uint16_t*)w; w += fs.dr;
    p.dr_lo = (uint16_t*)w; w += fs.dr;
    p.dc_hi = (uint16_t*)w; w += fs.dc;
    p.dc_lo = (uint16_t*)w; w += fs.dc;
    p.y = (float*)w; w += fs.y;
    p.qt_hi = (uint16_t*)w; w += fs.qt;
    p.qt_lo = (uint16_t*)w; w += fs.qt;
    p.z = (float*)w; w += fs.z;
    p.zt_hi = (uint16_t*)w;
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

    hipStream_t hs = (hipStream_t)hip_stream;
    const int nb = (int)fs.blocks;
    const int Tp = fs.Tp, kp = fs.kp, Fi = (int)F;
    hipError_t e = launch_kernel(delta_kernel, dim3((unsigned)((Tp / kTileT) * (Fi / 64)), (unsigned)L.num_layers,
                                                    (unsigned)(n * S)),
                                 dim3(kFormThreads), hs, p);
    auto sketch_launch = [&](const uint16_t* ah, const uint16_t* al, int64_t ablk, const uint16_t* bh,
                             const uint16_t* bl, int64_t bblk, float* o, int64_t oblk, int R, int X, int nbv) {
        SketchArgs sa{ah, al, ablk, bh, bl, bblk, o, oblk, R, X, nbv};
        const dim3 grid((unsigned)(R / 32), (unsigned)nb);
        if (kp == 32)
            return bl ? launch_kernel(sketch_kernel<1, true>, grid, dim3(256), hs, sa)
                      : launch_kernel(sketch_kernel<1, false>, grid, dim3(256), hs, sa);
        return bl ? launch_kernel(sketch_kernel<2, true>, grid, dim3(256), hs, sa)
                  : launch_kernel(sketch_kernel<2, false>, grid, dim3(256), hs, sa);
    };
    auto orth_launch = [&](float* x, int64_t xblk, uint16_t* xth, uint16_t* xtl, int64_t xtblk, int R) {
        OrthArgs oa{x, xblk, xth, xtl, xtblk, R, kp};
        return launch_kernel(orth_kernel, dim3(1, (unsigned)nb), dim3(kFormThreads), hs, oa);
    };
    const int64_t drb = (int64_t)Tp * Fi, yb = (int64_t)Tp * kp, zb = (int64_t)Fi * kp;
    const int q = sketch->power_iters;
    // Y = Delta Omega, Q = orth(Y)
    if (e == hipSuccess) e = sketch_launch(p.dr_hi, p.dr_lo, drb, p.omega, nullptr, 0, p.y, yb, Tp, Fi, k);
    if (e == hipSuccess) e = orth_launch(p.y, yb, p.qt_hi, q == 0 ? p.qt_lo : nullptr, yb, Tp);
    for (int it = 0; it < q && e == hipSuccess; ++it) {
        // Z = orth(Delta^T Q); Y = Delta Z; Q = orth(Y)
        e = sketch_launch(p.dc_hi, p.dc_lo, drb, p.qt_hi, nullptr, yb, p.z, zb, Fi, Tp, kp);
        if (e == hipSuccess) e = orth_launch(p.z, zb, p.zt_hi, nullptr, zb, Fi);
        if (e == hipSuccess) e = sketch_launch(p.dr_hi, p.dr_lo, drb, p.zt_hi, nullptr, zb, p.y, yb, Tp, Fi, kp);
        if (e == hipSuccess) e = orth_launch(p.y, yb, p.qt_hi, it == q - 1 ? p.qt_lo : nullptr, yb, Tp);
    }
    // Z = Delta^T Q with Q split in hi + lo, then the factors
    if (e == hipSuccess) e = sketch_launch(p.dc_hi, p.dc_lo, drb, p.qt_hi, p.qt_lo, yb, p.z, zb, Fi, Tp, kp);
    if (e == hipSuccess) {
        FinalArgs fa;
        fa.q = p.y;
        fa.z = p.z;
        fa.q_block = yb;
        fa.z_block = zb;
        fa.kp = kp;
        fa.m = m;
        fa.T = T;
        fa.Tp = Tp;
        fa.F = Fi;
        fa.L = L.num_layers;
        fa.S = S;
        for (int s = 0; s < 2; ++s) {
            fa.u[s] = s < S ? out->u[s] : nullptr;
            fa.v[s] = s < S ? out->v[s] : nullptr;
        }
        e = launch_kernel(final_kernel, dim3(1, (unsigned)nb), dim3(kFormThreads), hs, fa);
    }
    return e == hipSuccess ? KAMERA_OK : KAMERA_ERR_HIP;
}

}  // extern "C"
