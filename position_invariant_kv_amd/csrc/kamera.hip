// kamera.hip — Kamera reuse operator on MI355X (gfx950): host dispatch, the
// two kernels and the C ABI declared in include/kamera.h.
//
// Operator (Kamera: Unified Position-Invariant Multimodal KV Cache for
// Training-Free Reuse, gist.science paper 2606.23581, section 2, reuse
// equation): out = R(delta) x + U V^T per (chunk, layer, stream) block, then a
// scatter into the KV pool.
//
// Two kernels, both one launch per call covering every layer and stream:
//
//  * relocate_rows_kernel (m = 0: relocation / sliding-window survival).
//    Pure streaming.  One 16-byte vector (8 bf16) per thread step, 256-thread
//    workgroups over a tile of rows of one (chunk, stream, layer).  Rotated
//    vectors also read their rotate-half partner (same 128-byte lines, so it
//    costs L1 traffic, not HBM traffic); unrotated vectors are copied as raw
//    bits.  The cos/sin table of the chunk sits in LDS.
//
//  * relocate_patch_kernel (m > 0).  The rank-m patch is a dense contraction
//    over m, so it runs on the matrix cores: one wave owns 32 tokens x one
//    "segment" of 64 features, and keeps the rotated canonical tile in
//    the fp32 accumulator of v_mfma_f32_32x32x16_bf16, so that
//    D = R(delta) x + V_f U_t^T comes out of the MFMA already in place.  The
//    MFMA rows (features) are relabelled so that each lane's 16 accumulator
//    values per block are contiguous features of its token: every lane then
//    reads and writes its token's row with plain 16-byte loads and stores, and
//    the rotate-half partner of every value lives in the same lane.
//
// Rounding: fp32 -> bf16 with v_cvt_pk_bf16_f32 (round to nearest even).

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "kamera.h"

namespace {

constexpr int kMaxSegments = 64;       // 64 x 64 elements: rows up to 4096 wide
constexpr int kMaxHalfRope = 512;
constexpr int kThreads = 256;          // both kernels: 4 waves of 64
constexpr int kWaves = kThreads / 64;
constexpr int kXcds = 8;               // MI355X: workgroups go round-robin over 8 XCDs

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Division by a runtime constant with a multiply-high (Granlund & Montgomery,
// "Division by invariant integers using multiplication", 1994): for
// 0 <= x < 2^31, x / d = (mulhi(x, mul) + x) >> shr.
struct FastDiv {
    uint32_t d, mul, shr;
};

FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    uint64_t mul = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    return FastDiv{d, (uint32_t)mul, l};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t x, const FastDiv& f) {
    return (__umulhi(x, f.mul) + x) >> f.shr;
}

// One wave's share of a row: 64 elements in two runs of 32 starting at r0 and
// r1.  Lane half h (lanes 32h..32h+31) owns [r + 16h, r + 16h + 16) of both
// runs.  rot: the runs carry RoPE; j0 is the first pair (frequency) index.
struct Segment {
    int16_t r0, r1, j0, rot;
};

struct SegmentTable {
    Segment seg[kMaxSegments];
    int32_t count;
};

struct Params {
    const uint16_t* src[2];
    int64_t src_chunk_stride, src_layer_stride;
    const int64_t* canon_pos;
    const uint16_t* u[2];
    const uint16_t* v[2];
    uint16_t* dst[2];
    int64_t dst_layer_stride;
    int64_t num_slots;
    const int32_t* page_table;
    const int64_t* dst_offset;
    uint32_t* error_word;
    const int64_t* delta;
    const int32_t* ids;
    const int64_t* target;
    int64_t base_pos;
    double log2_base;
    int32_t mode;  // 0: delta given, 1: reorder, 2: recall
    int32_t rank;
    int32_t page_size, pages_per_chunk;
    int32_t page_shift;  // log2(page_size) when it is a power of two, else -1
    int32_t n, n_store, L, S, T, F;
    int32_t D, rope_offset, rope_dim, rope_style;
};

enum { MODE_DELTA = 0, MODE_REORDER = 1, MODE_RECALL = 2 };

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ u32x4 ld_stream(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld_cached(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
// A workgroup-uniform read of an input the kernels never write, through the
// constant address space: it becomes a scalar load, which is counted apart
// from the vector loads and so never holds up a wait on them.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* ptr) {
    return *(const __attribute__((address_space(4))) T*)ptr;
}
__device__ __forceinline__ void st_stream(uint16_t* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// RoPE frequencies theta_j = base^(-2j/R), computed once per call on the host
// in fp64 and passed by value; spans with more than kMaxThetas pairs compute
// theta_j on the device instead (count = 0).
constexpr int kMaxThetas = 128;
static_assert(kThreads > kMaxThetas, "the rows kernel reads theta for j < kThreads only");
struct ThetaTable {
    double theta[kMaxThetas];
    int32_t count;
};

// cos/sin of phi = delta * theta_j.  phi reaches ~1e7 rad for the largest
// shifts, where an fp32 product is useless, so phi and its reduction
// r = phi - k*pi/2 (|r| <= pi/4, Cody-Waite with a two-term pi/2) are fp64.
// sin r and cos r then come from their Taylor series in fp32; truncated after
// r^11 and r^12 they are off by < 1e-11 on |r| <= pi/4, so the fp32 rounding
// (a few 1e-8) dominates and the table is far finer than the bf16 spacing of
// the results.  The quadrant k mod 4 picks signs and swaps.
// theta_j: the host's fp64 table for j < tt.count (value passed in as
// `tabled`, read by the caller), computed on the device beyond it.
__device__ __forceinline__ double rope_theta(const ThetaTable& tt, double tabled, double log2_base, int rope_dim,
                                             int j) {
    return (j < tt.count) ? tabled : exp2(log2_base * (-2.0 * (double)j / (double)rope_dim));
}

__device__ __forceinline__ float2 rope_phase_of(double theta, int64_t delta) {
    const double kHalfPiHi = 1.5707963267948966;       // fp64(pi/2)
    const double kHalfPiLo = 6.123233995736766e-17;    // pi/2 - kHalfPiHi
    const double kTwoOverPi = 0.6366197723675814;
    const double phi = (double)delta * theta;
    const double k = rint(phi * kTwoOverPi);
    double r = fma(-k, kHalfPiHi, phi);
    r = fma(-k, kHalfPiLo, r);
    const float x = (float)r;
    const float x2 = x * x;
    // sin x = x (1 - x^2/3! + x^4/5! - x^6/7! + x^8/9! - x^10/11!)
    float sp = -2.5052108385441720e-08f;
    sp = fmaf(sp, x2, 2.7557319223985893e-06f);
    sp = fmaf(sp, x2, -1.9841269841269841e-04f);
    sp = fmaf(sp, x2, 8.3333333333333332e-03f);
    sp = fmaf(sp, x2, -1.6666666666666666e-01f);
    const float sn = fmaf(sp * x2, x, x);
    // cos x = 1 - x^2/2! + x^4/4! - x^6/6! + x^8/8! - x^10/10! + x^12/12!
    float cp = 2.0876756987868099e-09f;
    cp = fmaf(cp, x2, -2.7557319223985888e-07f);
    cp = fmaf(cp, x2, 2.4801587301587302e-05f);
    cp = fmaf(cp, x2, -1.3888888888888889e-03f);
    cp = fmaf(cp, x2, 4.1666666666666664e-02f);
    cp = fmaf(cp, x2, -0.5f);
    const float cn = fmaf(cp, x2, 1.0f);
    const int q = (int)((long long)k & 3);
    float c, s;
    switch (q) {
        case 0: c = cn; s = sn; break;
        case 1: c = -sn; s = cn; break;
        case 2: c = -cn; s = -sn; break;
        default: c = sn; s = -cn; break;
    }
    return make_float2(c, s);
}

__device__ __forceinline__ float2 rope_phase(const ThetaTable& tt, double log2_base, int rope_dim, int j,
                                             int64_t delta) {
    const double tabled = tt.theta[max(0, min(j, kMaxThetas - 1))];
    return rope_phase_of(rope_theta(tt, tabled, log2_base, rope_dim, j), delta);
}

// Page-table column of token t of a chunk.
__device__ __forceinline__ int page_of(const Params& p, int t) {
    return p.page_shift >= 0 ? (t >> p.page_shift) : t / p.page_size;
}

// Pool slot of token t of output chunk i from its page id (paged pool; the id
// read from the page table) or from the chunk's offset (contiguous pool), or
// -1 when the id or the offset is out of range (then the row is skipped and
// the error bit recorded).  The reads happen in the caller, ahead of the bulk
// loads, so that no wait on them holds up the rows.
__device__ __forceinline__ int64_t slot_from(const Params& p, int t, int32_t page_id, int64_t offset,
                                             uint32_t& err) {
    if (p.page_size > 0) {
        if (page_id < 0 || (int64_t)page_id >= p.num_slots / p.page_size) {
            err |= KAMERA_EW_PAGE;
            return -1;
        }
        return (int64_t)page_id * p.page_size + (t - page_of(p, t) * p.page_size);
    }
    if (offset < 0 || offset + p.T > p.num_slots) {
        err |= KAMERA_EW_OFFSET;
        return -1;
    }
    return offset + t;
}

// Pool slot of token t of output chunk i, its page id / offset read here.
__device__ __forceinline__ int64_t dest_slot(const Params& p, int i, int t, uint32_t& err) {
    if (p.page_size > 0) return slot_from(p, t, p.page_table[(int64_t)i * p.pages_per_chunk + page_of(p, t)], 0, err);
    return slot_from(p, t, 0, ld_uniform(p.dst_offset + i), err);
}

// ---------------------------------------------------------------------------
// m = 0: relocation only
// ---------------------------------------------------------------------------

// Rotates the 8 bf16 of vector a (pair partner vector b, R/2 elements away)
// and returns the rounded result.  first: a holds x_j (A' = A c - B s), else a
// holds x_{j+R/2} (B' = B c + A s).
__device__ __forceinline__ u32x4 rotate_half_vec(u32x4 a, u32x4 b, const float2* cs, int j0, bool first) {
    const float sg = first ? -1.0f : 1.0f;
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float2 t0 = cs[j0 + 2 * q], t1 = cs[j0 + 2 * q + 1];
        const float o0 = fmaf(bf_lo(a[q]), t0.x, sg * bf_lo(b[q]) * t0.y);
        const float o1 = fmaf(bf_hi(a[q]), t1.x, sg * bf_hi(b[q]) * t1.y);
        out[q] = pack_bf16x2(o0, o1);
    }
    return out;
}

// Interleaved pairs (2j, 2j+1) inside one vector.
__device__ __forceinline__ u32x4 rotate_pairs_vec(u32x4 a, const float2* cs, int j0) {
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float2 t = cs[j0 + q];
        const float A = bf_lo(a[q]), B = bf_hi(a[q]);
        out[q] = pack_bf16x2(fmaf(A, t.x, -B * t.y), fmaf(B, t.x, A * t.y));
    }
    return out;
}

// Workgroup = 256*U consecutive 16-byte vectors of the flattened [T][F] rows of
// one (output chunk, stream, layer); each thread moves U vectors, once, with no
// loop (measured on MI355X: one or two vectors per thread over a small
// contiguous block stream at the plain-copy rate; more work per thread streams
// slower).  For U = 2 on a stream whose heads are rotated whole with the
// rotate-half pairing (GQA/MHA keys), a thread owns one "pair unit" instead:
// vector q of a head's first half and vector q of its second half, so every
// element is loaded exactly once.  Otherwise a rotated vector also loads its
// partner (an L1 hit).  The row loads are issued first; while they are in
// flight the chunk's cos/sin table and the pool slot of every row the block
// touches go to LDS.
template <int U>
__global__ __launch_bounds__(kThreads) void relocate_rows_kernel(const Params p, const ThetaTable tt,
                                                                 const int blocks_per_slice,
                                                                 const FastDiv div_vr, const FastDiv div_hd,
                                                                 const FastDiv div_upr, const FastDiv div_uph) {
    __shared__ float2 cs[kMaxHalfRope];
    __shared__ int64_t slot_of_row[kThreads * U / 8 + 2];
    int b = blockIdx.x;
    const int blk = b % blocks_per_slice;
    b /= blocks_per_slice;
    const int l = b % p.L;
    b /= p.L;
    const int s = b % p.S;
    const int i = b / p.S;

    bool ok = true;
    int c = i;
    uint32_t err = 0;
    if (p.mode != MODE_DELTA) {
        c = ld_uniform(p.ids + i);
        if (c < 0 || c >= p.n_store) {
            err |= KAMERA_EW_CHUNK;
            ok = false;
        }
    }
    const bool rot = (s == 0) && (p.rope_dim > 0);
    const bool pairs = (U == 2) && rot && p.rope_style == KAMERA_ROPE_HALF && p.rope_offset == 0 &&
                       p.rope_dim == p.D;
    const int VR = p.F >> 3;
    const int VD = p.D >> 3;
    const int half = p.rope_dim >> 1;
    const int nvec = p.T * VR;
    const int v0 = blk * kThreads * U;
    const int r_first = (int)fdiv((uint32_t)v0, div_vr);
    // a rejected chunk id reads chunk 0 (in range) and stores nothing
    const uint16_t* __restrict__ sb =
        p.src[s] + (int64_t)(ok ? c : 0) * p.src_chunk_stride + (int64_t)l * p.src_layer_stride;
    uint16_t* __restrict__ db = p.dst[s] + (int64_t)l * p.dst_layer_stride;

    // The small loads go first -- the page id (or offset) of the row this
    // thread resolves and theta of its frequency -- and stay raw until the row
    // loads are issued: loads retire in issue order, so a wait on them then
    // costs nothing.  Every path issues the same row loads (addresses past the
    // end are clamped and their results not stored), so the waits the
    // compiler places stay exact.
    const int r_end = min(p.T, (int)fdiv((uint32_t)min(v0 + kThreads * U, nvec) - 1u, div_vr) + 1);
    const int nrows = r_end - r_first;
    const int t_own = r_first + min((int)threadIdx.x, nrows - 1);
    int32_t page_raw = 0;
    int64_t off_raw = 0;
    if (p.page_size > 0) page_raw = p.page_table[(int64_t)i * p.pages_per_chunk + page_of(p, t_own)];
    else off_raw = ld_uniform(p.dst_offset + i);
    const double theta_raw = tt.theta[min((int)threadIdx.x, kMaxThetas - 1)];

    int row[U], col[U], ecol[U];
    uint32_t so[U], yo[U];  // element offsets of the vector and of its rotate-half partner
#pragma unroll
    for (int k = 0; k < U; ++k) {
        row[k] = -1;
        ecol[k] = -1;
    }
    if (pairs) {
        // unit g of the slice: row g / (F/16), head (g % (F/16)) / (D/16), q
        const int g = (v0 >> 1) + (int)threadIdx.x;
        const int gc = min(g, (nvec >> 1) - 1);
        const int r = (int)fdiv((uint32_t)gc, div_upr);
        const int w = gc - r * (VR >> 1);
        const int h = (int)fdiv((uint32_t)w, div_uph);
        const int q = w - h * (VD >> 1);
        const int va = h * VD + q;
        so[0] = (uint32_t)(r * p.F + (va << 3));
        so[U - 1] = so[0] + (uint32_t)half;
        if (U == 2 && g == gc) {
            row[0] = row[U - 1] = r - r_first;
            col[0] = va << 3;
            col[U - 1] = (va << 3) + half;
            ecol[0] = q << 3;
            ecol[U - 1] = (q << 3) + half;
        }
    } else {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int v = v0 + (int)threadIdx.x + k * kThreads;
            const int vc = min(v, nvec - 1);
            const int r = (int)fdiv((uint32_t)vc, div_vr);
            const int vec = vc - r * VR;
            const int h = (int)fdiv((uint32_t)vec, div_hd);
            const int e = ((vec - h * VD) << 3) - p.rope_offset;
            const bool in_rope = rot && e >= 0 && e < p.rope_dim;
            so[k] = (uint32_t)vc << 3;
            // vectors outside the rotary span re-read themselves
            yo[k] = so[k] + (uint32_t)(in_rope ? ((e < half) ? half : -half) : 0);
            if (v == vc) {
                if (in_rope) ecol[k] = e;
                row[k] = r - r_first;
                col[k] = vec << 3;
            }
        }
    }
    u32x4 x[U], y[U];
#pragma unroll
    for (int k = 0; k < U; ++k) x[k] = ld_stream(sb + so[k]);
    // the rotate-half partner, R/2 elements away (an L1 hit)
    if (!pairs && rot && p.rope_style == KAMERA_ROPE_HALF) {
#pragma unroll
        for (int k = 0; k < U; ++k) y[k] = ld_stream(sb + yo[k]);
    }
    if (!ok) {
#pragma unroll
        for (int k = 0; k < U; ++k) row[k] = -1;
    }
    if (ok && (int)threadIdx.x < nrows) slot_of_row[threadIdx.x] = slot_from(p, t_own, page_raw, off_raw, err);
    if (ok && rot) {
        int64_t delta;
        if (p.mode == MODE_DELTA) {
            delta = ld_uniform(p.delta + i);
        } else {
            const int64_t pc = p.canon_pos ? ld_uniform(p.canon_pos + c) : 0;
            delta = (p.mode == MODE_REORDER) ? p.base_pos + (int64_t)i * p.T - pc : ld_uniform(p.target + i) - pc;
        }
        if ((int)threadIdx.x < half)
            cs[threadIdx.x] = rope_phase_of(rope_theta(tt, theta_raw, p.log2_base, p.rope_dim, threadIdx.x), delta);
        // j >= kThreads > kMaxThetas: never in the host's table
        for (int j = threadIdx.x + kThreads; j < half; j += kThreads)
            cs[j] = rope_phase_of(rope_theta(tt, 0.0, p.log2_base, p.rope_dim, j), delta);
    }
    __syncthreads();

    if (pairs) {
        if (row[0] < 0) goto done;
        const int64_t slot = slot_of_row[row[0]];
        if (slot < 0) goto done;
        const int j0 = ecol[0];
        const u32x4 oa = rotate_half_vec(x[0], x[U - 1], cs, j0, true);
        const u32x4 ob = rotate_half_vec(x[U - 1], x[0], cs, j0, false);
        st_stream(db + slot * p.F + col[0], oa);
        st_stream(db + slot * p.F + col[U - 1], ob);
        goto done;
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
        if (row[k] < 0) continue;
        const int64_t slot = slot_of_row[row[k]];
        if (slot < 0) continue;
        u32x4 out = x[k];
        const int e = ecol[k];
        if (e >= 0) {
            if (p.rope_style == KAMERA_ROPE_HALF) {
                const bool first = e < half;
                out = rotate_half_vec(x[k], y[k], cs, first ? e : e - half, first);
            } else {
                out = rotate_pairs_vec(x[k], cs, e >> 1);
            }
        }
        st_stream(db + slot * p.F + col[k], out);
    }
done:
    if (err && p.error_word) atomicOr(p.error_word, err);
}

// ---------------------------------------------------------------------------
// m > 0: relocation + rank-m patch on the matrix cores
// ---------------------------------------------------------------------------
//
// v_mfma_f32_32x32x16_bf16 computes D[32x32] = A[32x16] B[16x32] + C with
//   A: lane l holds A[l%32][8*(l/32) .. +8]    (row i, 8 consecutive k)
//   B: lane l holds B[8*(l/32) .. +8][l%32]    (8 consecutive k, column n)
//   C/D: lane l value v holds row 8*(v/4) + 4*(l/32) + v%4 of column l%32.
// Here A = patch factor V (rows = features), B = U^T (columns = tokens), so all
// C/D values of a lane belong to token l%32.  A wave owns a 64-feature segment
// made of two 32-feature runs; MFMA block b covers run b.  The rows of a block
// are relabelled so that value v of lane half h holds run offset
//   off(v, h) = 8h + v        (v < 8)
//             = 8 + 8h + v    (v >= 8),
// i.e. row i (v = 4*(i>>3) + (i&3), h = (i>>2)&1) carries feature run_b +
// off(v, h).  Each lane then holds two 8-feature vectors of its token per run,
// one 16-byte load or store each, and in every such instruction the two lane
// halves of a token cover 32 contiguous bytes.  The rotate-half partner of
// value v of run 0 is value v of run 1, in the same lane.

__device__ __forceinline__ int run_offset(int v, int h) { return (v < 8) ? 8 * h + v : 8 + 8 * h + v; }

__device__ __forceinline__ int row_feature(const Segment& sg, int b, int i) {
    return (b ? sg.r1 : sg.r0) + run_offset(4 * (i >> 3) + (i & 3), (i >> 2) & 1);
}

// Loads of one 32-token tile: this lane's 32 canonical elements (two 16-byte
// vectors per run), its U row slice, and the destination slot of its token.
// Cache policy of the canonical-row loads and pool-row stores.
template <int NT>
struct LoadRow;
template <>
struct LoadRow<1> {
    static __device__ __forceinline__ u32x4 ld(const uint16_t* p) { return ld_stream(p); }
    static __device__ __forceinline__ void st(uint16_t* p, u32x4 v) { st_stream(p, v); }
};
template <>
struct LoadRow<0> {
    static __device__ __forceinline__ u32x4 ld(const uint16_t* p) { return ld_cached(p); }
    static __device__ __forceinline__ void st(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
};

template <int KS>
struct PatchTile {
    u32x4 raw[4];
    bf16x8 bop[KS];
    int64_t slot;
};

template <int KS, int NT>
__device__ __forceinline__ void load_patch_tile(const Params& p, PatchTile<KS>& tl, const uint16_t* srow0,
                                                const uint16_t* U, int i, int t, int o0, int o1, int hh,
                                                uint32_t& err) {
    const bool tv = t < p.T;
#pragma unroll
    for (int q = 0; q < 4; ++q) tl.raw[q] = u32x4{0u, 0u, 0u, 0u};
    if (tv) {
        const uint16_t* srow = srow0 + (int64_t)t * p.F;
        tl.raw[0] = LoadRow<NT>::ld(srow + o0);
        tl.raw[1] = LoadRow<NT>::ld(srow + o0 + 16);
        tl.raw[2] = LoadRow<NT>::ld(srow + o1);
        tl.raw[3] = LoadRow<NT>::ld(srow + o1 + 16);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int k0 = 16 * ks + 8 * hh;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (tv && k0 < p.rank) w = ld_cached(U + (int64_t)t * p.rank + k0);
        tl.bop[ks] = __builtin_bit_cast(bf16x8, w);
    }
    tl.slot = tv ? dest_slot(p, i, t, err) : -1;
}

template <int KS, int NT, int DEPTH>
__global__ __launch_bounds__(kThreads) void relocate_patch_kernel(const Params p, const ThetaTable tt,
                                                                   const SegmentTable st,
                                                                   const int tiles_per_wave,
                                                                   const int groups,
                                                                   const int total_items,
                                                                   const int grid_per_xcd) {
    __shared__ float2 cs_lds[kWaves][32];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int hh = lane >> 5;   // lane half
    const int col = lane & 31;  // token inside the tile

    // XCD-aware order: consecutive logical workgroups (which share a chunk's
    // factors) land on the same XCD and its L2.
    const int wg = blockIdx.x;
    const int logical = (wg % kXcds) * grid_per_xcd + wg / kXcds;
    const int item = logical * kWaves + wave;
    const bool live = item < total_items;

    int it = live ? item : 0;
    const int sgi = it % st.count;
    it /= st.count;
    const int g = it % groups;
    it /= groups;
    const int l = it % p.L;
    it /= p.L;
    const int s = it % p.S;
    const int i = it / p.S;
    const Segment sg = st.seg[sgi];
    const bool rot = sg.rot && s == 0;

    // store chunk of this output chunk
    bool ok = live;
    int c = i;
    uint32_t err = 0;
    if (ok && p.mode != MODE_DELTA) {
        c = ld_uniform(p.ids + i);
        if (c < 0 || c >= p.n_store) {
            err |= KAMERA_EW_CHUNK;
            ok = false;
        }
    }

    const int F = p.F;
    const int64_t blk = (int64_t)c * p.L + l;  // factor block of (chunk, layer)
    const uint16_t* __restrict__ U = p.u[s] + blk * p.T * p.rank;
    const uint16_t* __restrict__ V = p.v[s] + blk * F * p.rank;
    const uint16_t* __restrict__ srow0 =
        p.src[s] + (int64_t)c * p.src_chunk_stride + (int64_t)l * p.src_layer_stride;
    uint16_t* __restrict__ drow0 = p.dst[s] + (int64_t)l * p.dst_layer_stride;
    const int o0 = sg.r0 + 8 * hh;
    const int o1 = sg.r1 + 8 * hh;
    const int tile0 = g * tiles_per_wave;
    const int ntiles = min(tiles_per_wave, (p.T + 31) / 32 - tile0);

    // Issue every independent load first: the factor rows of this segment and
    // the first tile; the shift and its cos/sin table are worked out while
    // they are in flight.
    bf16x8 aop[2][KS];
    PatchTile<KS> nxt[DEPTH];  // the next DEPTH tiles, in flight
    if (ok) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int f = row_feature(sg, b, col);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int k0 = 16 * ks + 8 * hh;
                u32x4 w = {0u, 0u, 0u, 0u};
                if (k0 < p.rank) w = ld_cached(V + (int64_t)f * p.rank + k0);
                aop[b][ks] = __builtin_bit_cast(bf16x8, w);
            }
        }
#pragma unroll
        for (int d = 0; d < DEPTH; ++d)
            if (d < ntiles) load_patch_tile<KS, NT>(p, nxt[d], srow0, U, i, (tile0 + d) * 32 + col, o0, o1, hh, err);
    }

    if (ok && rot && lane < 32) {
        int64_t delta;
        if (p.mode == MODE_DELTA) {
            delta = ld_uniform(p.delta + i);
        } else {
            const int64_t pc = p.canon_pos ? ld_uniform(p.canon_pos + c) : 0;
            delta = (p.mode == MODE_REORDER) ? p.base_pos + (int64_t)i * p.T - pc : ld_uniform(p.target + i) - pc;
        }
        cs_lds[wave][lane] = rope_phase(tt, p.log2_base, p.rope_dim, sg.j0 + lane, delta);
    }
    __syncthreads();
    if (!ok) {
        if (err && p.error_word) atomicOr(p.error_word, err);
        return;
    }

    // cos/sin of this lane's 16 pairs, read from the wave's LDS table (indexed
    // by pair number inside the segment) on every tile: registers are the
    // scarcer resource.  Rotate-half: pair q joins value q of run 0 and value q
    // of run 1, pair number off(q, h).  Interleaved: pair q joins values
    // 2(q&7), 2(q&7)+1 of run q>>3, pair number (32*(q>>3) + off(2(q&7), h))/2.
    const float2* cs_w = cs_lds[wave];
    const bool half_style = p.rope_style == KAMERA_ROPE_HALF;

    for (int tt = 0; tt < ntiles; ++tt) {
        const PatchTile<KS> cur = nxt[0];
#pragma unroll
        for (int d = 0; d + 1 < DEPTH; ++d) nxt[d] = nxt[d + 1];
        if (tt + DEPTH < ntiles)
            load_patch_tile<KS, NT>(p, nxt[DEPTH - 1], srow0, U, i, (tile0 + tt + DEPTH) * 32 + col, o0, o1, hh, err);

        // widen: block b value v = element v of this lane's 16 features of run b
        f32x16 acc[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const uint32_t word = cur.raw[2 * b + (w >> 2)][w & 3];
                acc[b][2 * w] = bf_lo(word);
                acc[b][2 * w + 1] = bf_hi(word);
            }
        }

        if (rot) {
            if (half_style) {
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const float2 t = cs_w[run_offset(q, hh)];
                    const float A = acc[0][q], B = acc[1][q];
                    acc[0][q] = fmaf(A, t.x, -B * t.y);
                    acc[1][q] = fmaf(B, t.x, A * t.y);
                }
            } else {
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int b = q >> 3, v = 2 * (q & 7);
                    const float2 t = cs_w[(32 * b + run_offset(v, hh)) >> 1];
                    const float A = acc[b][v], B = acc[b][v + 1];
                    acc[b][v] = fmaf(A, t.x, -B * t.y);
                    acc[b][v + 1] = fmaf(B, t.x, A * t.y);
                }
            }
        }

        // D = V_f U_t^T + C on the matrix cores
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[b][ks], cur.bop[ks], acc[b], 0, 0, 0);
        }

        if (cur.slot >= 0) {
            uint16_t* drow = drow0 + cur.slot * F;
            u32x4 w[4];
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int k = 0; k < 8; ++k) w[2 * b + (k >> 2)][k & 3] = pack_bf16x2(acc[b][2 * k], acc[b][2 * k + 1]);
            LoadRow<NT>::st(drow + o0, w[0]);
            LoadRow<NT>::st(drow + o0 + 16, w[1]);
            LoadRow<NT>::st(drow + o1, w[2]);
            LoadRow<NT>::st(drow + o1 + 16, w[3]);
        }
    }
    if (err && p.error_word) atomicOr(p.error_word, err);
}

// LDS-staged variant.  A workgroup of W waves owns 32 tokens x one window of
// 64*W contiguous features (W whole segments) of one (output chunk, stream,
// layer).  1) every thread loads 4 of the tile's 16-byte vectors with plain
// coalesced loads (each wave instruction covers whole 128-byte lines) and puts
// them in an LDS tile whose rows are padded by 16 bytes, so the MFMA-layout
// reads below hit 16 distinct bank groups per 16 lanes; 2) each wave reads its
// segment in the MFMA layout from LDS, rotates, runs the patch on the matrix
// cores and writes the rounded result back in place; 3) every thread stores
// its 4 vectors to the pool rows, again whole lines per instruction.
constexpr int kTileTokens = 32;
constexpr int kMaxTilesPerGroup = 8;  // tiles one LDS-staged workgroup processes

constexpr int kMaxWindowWaves = 4;

// Ranks up to 16 (KS = 1) fit 128 VGPRs without spilling, which allows 4 waves
// per SIMD; larger ranks would spill under that bound and keep 3.
template <int KS, int DEPTH>
__global__ __launch_bounds__(64 * kMaxWindowWaves, (KS == 1 && DEPTH == 1) ? 4 : 1) void relocate_patch_lds_kernel(
    const Params p, const ThetaTable tt, const SegmentTable st, const int W, const int windows,
    const int tiles, const int tiles_per_wg, const int groups) {
    __shared__ __attribute__((aligned(16))) uint8_t tile_lds[kTileTokens * (128 * kMaxWindowWaves + 16)];
    __shared__ float2 cs_lds[kMaxWindowWaves][32];
    __shared__ int64_t slot_lds[kTileTokens * kMaxTilesPerGroup];  // pool slot of every token of the group
    const int nthreads = 64 * W;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: segment reads are scalar
    const int hh = lane >> 5;
    const int col = lane & 31;
    const int pitch = 128 * W + 16;  // bytes per LDS row

    int b = blockIdx.x;
    const int g = b % groups;
    b /= groups;
    const int win = b % windows;
    b /= windows;
    const int l = b % p.L;
    b /= p.L;
    const int s = b % p.S;
    const int i = b / p.S;

    bool ok = true;
    int c = i;
    uint32_t err = 0;
    if (p.mode != MODE_DELTA) {
        c = ld_uniform(p.ids + i);
        if (c < 0 || c >= p.n_store) {
            if (p.error_word && tid == 0) atomicOr(p.error_word, (uint32_t)KAMERA_EW_CHUNK);
            return;  // uniform over the workgroup: nobody reaches a barrier
        }
    }
    const Segment sg = st.seg[win * W + wave];
    const bool rot = sg.rot && s == 0;
    const int fw0 = st.seg[win * W].r0;  // first feature of the window
    const int F = p.F;
    const int64_t blk = (int64_t)c * p.L + l;
    const uint16_t* __restrict__ U = p.u[s] + blk * p.T * p.rank;
    const uint16_t* __restrict__ V = p.v[s] + blk * F * p.rank;
    const uint16_t* __restrict__ src = p.src[s] + (int64_t)c * p.src_chunk_stride + (int64_t)l * p.src_layer_stride;
    uint16_t* __restrict__ dst = p.dst[s] + (int64_t)l * p.dst_layer_stride;

    const int tile_begin = g * tiles_per_wg;
    const int tile_end = min(tiles, tile_begin + tiles_per_wg);
    const int tok0 = tile_begin * kTileTokens;
    const int ntok = min(p.T, tile_end * kTileTokens) - tok0;

    // Pool slots of the group's tokens: the page ids (or the chunk's offset)
    // are loaded before anything else, with clamped indices, and turned into
    // slots only after the first tile's loads are issued.
    constexpr int kSlotLoads = (kTileTokens * kMaxTilesPerGroup + 63) / 64;
    int32_t page_raw[kSlotLoads];
    int64_t off_raw = 0;
    if (p.page_size > 0) {
#pragma unroll
        for (int k = 0; k < kSlotLoads; ++k) {
            const int t = tok0 + min(tid + k * nthreads, ntok - 1);
            page_raw[k] = p.page_table[(int64_t)i * p.pages_per_chunk + page_of(p, t)];
        }
    } else {
        off_raw = ld_uniform(p.dst_offset + i);
    }

    // the shift's inputs next (small loads ahead of the big ones); theta of this
    // lane's frequency is read unconditionally from a clamped table index
    const int jph = sg.j0 + (lane & 31);
    const double theta_in = tt.theta[max(0, min(jph, kMaxThetas - 1))];
    int64_t delta_in = 0, pc_in = 0, target_in = 0;
    if (rot) {
        if (p.mode == MODE_DELTA) {
            delta_in = ld_uniform(p.delta + i);
        } else {
            pc_in = p.canon_pos ? ld_uniform(p.canon_pos + c) : 0;
            if (p.mode == MODE_RECALL) target_in = ld_uniform(p.target + i);
        }
    }

    // A operands of this wave's segment, resident for all tiles.  Every load
    // is issued (rank slices past the rank read a clamped in-range slice) and
    // the padding is zeroed once the loads have landed.
    u32x4 aop_raw[2][KS];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
        const int f = row_feature(sg, bb, col);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int k0 = min(16 * ks + 8 * hh, p.rank - 8);
            aop_raw[bb][ks] = ld_cached(V + (int64_t)f * p.rank + k0);
        }
    }
    bf16x8 aop[2][KS];  // set from aop_raw below

    const int chunks_per_row = 8 * W;

    // Every global load of a tile -- its canonical rows (coalesced: chunk
    // q = tid + k*64W -> row, 16-byte column), this lane's U row slice, and the
    // page-table entry / offset of one token -- goes into a TileBuf and is
    // issued DEPTH tiles ahead, so it is in flight while earlier tiles are
    // computed and stored.
    // per-thread, loop-invariant 32-bit element offsets of its 4 chunks inside a
    // tile (row * F + column) and inside the LDS tile; bases stay uniform
    int goff[4], loff[4], grow[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int q = tid + k * nthreads;
        const int qr = q / chunks_per_row;
        const int qc = q - qr * chunks_per_row;
        grow[k] = qr;
        goff[k] = qr * F + 8 * qc;
        loff[k] = qr * pitch + 16 * qc;
    }
    // The loads of a tile (U rows, then the rows) go straight into a TileBuf
    // and stay raw until the tile is processed: the memory counter retires
    // loads in issue order, so any arithmetic on a freshly issued load would
    // make the wave wait for everything issued before it.
    struct TileBuf {
        u32x4 v4[4];
        u32x4 bop[KS];
    };
    auto load_tile = [&](TileBuf& tb_, int t0) {
        // rows past the chunk's end re-read its last row (never stored)
        const int last = p.T - 1 - t0;
        const uint16_t* __restrict__ ub = U + (int64_t)t0 * p.rank;     // uniform
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int k0 = min(16 * ks + 8 * hh, p.rank - 8);
            tb_.bop[ks] = ld_cached(ub + (uint32_t)(min(col, last) * p.rank + k0));
        }
        const uint16_t* __restrict__ tb = src + (int64_t)t0 * F + fw0;  // uniform
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = min(grow[k], last);
            tb_.v4[k] = ld_stream(tb + (uint32_t)(goff[k] + (r - grow[k]) * F));
        }
    };

    // One tile: park the loaded rows in LDS, reload the buffer for a later
    // tile, then rotate + patch + round in place and store the tile.
    auto process_tile = [&](TileBuf& buf, int tile, int reload_tile) {
        const int t0 = tile * kTileTokens;
#pragma unroll
        for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x4*>(tile_lds + loff[k]) = buf.v4[k];
        bf16x8 bop[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 zero = {0u, 0u, 0u, 0u};
            bop[ks] = __builtin_bit_cast(bf16x8, 16 * ks + 8 * hh < p.rank ? buf.bop[ks] : zero);
        }
        if (reload_tile < tile_end) load_tile(buf, reload_tile * kTileTokens);
        __syncthreads();

        // this wave's segment in the MFMA layout, one MFMA block (run) at a time:
        // run b's values are rotated against their partners in run 1-b, the
        // patch is accumulated on the matrix cores and the rounded result goes
        // back to LDS before the next run is widened (half the live fp32 state)
        {
            uint8_t* rowp = tile_lds + col * pitch;
            const int a[2] = {2 * (sg.r0 - fw0 + 8 * hh), 2 * (sg.r1 - fw0 + 8 * hh)};
            u32x4 raw[4];
            raw[0] = *reinterpret_cast<const u32x4*>(rowp + a[0]);
            raw[1] = *reinterpret_cast<const u32x4*>(rowp + a[0] + 32);
            raw[2] = *reinterpret_cast<const u32x4*>(rowp + a[1]);
            raw[3] = *reinterpret_cast<const u32x4*>(rowp + a[1] + 32);
            const float2* cs_w = cs_lds[wave];
            const bool half_style = p.rope_style == KAMERA_ROPE_HALF;
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                f32x16 acc;
#pragma unroll
                for (int w = 0; w < 8; ++w) {
                    const uint32_t word = raw[2 * bb + (w >> 2)][w & 3];
                    acc[2 * w] = bf_lo(word);
                    acc[2 * w + 1] = bf_hi(word);
                }
                if (rot) {
                    if (half_style) {
                        // run 0 holds x_j (A' = A c - B s), run 1 holds x_{j+R/2} (B' = B c + A s)
                        const float sg_s = bb ? 1.0f : -1.0f;
#pragma unroll
                        for (int w = 0; w < 8; ++w) {
                            const uint32_t pw = raw[2 * (1 - bb) + (w >> 2)][w & 3];
                            const float2 t0 = cs_w[run_offset(2 * w, hh)];
                            const float2 t1 = cs_w[run_offset(2 * w + 1, hh)];
                            acc[2 * w] = fmaf(acc[2 * w], t0.x, sg_s * bf_lo(pw) * t0.y);
                            acc[2 * w + 1] = fmaf(acc[2 * w + 1], t1.x, sg_s * bf_hi(pw) * t1.y);
                        }
                    } else {
#pragma unroll
                        for (int w = 0; w < 8; ++w) {
                            const float2 t = cs_w[(32 * bb + run_offset(2 * w, hh)) >> 1];
                            const float A = acc[2 * w], B = acc[2 * w + 1];
                            acc[2 * w] = fmaf(A, t.x, -B * t.y);
                            acc[2 * w + 1] = fmaf(B, t.x, A * t.y);
                        }
                    }
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[bb][ks], bop[ks], acc, 0, 0, 0);
                u32x4 o0, o1;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    o0[k] = pack_bf16x2(acc[2 * k], acc[2 * k + 1]);
                    o1[k] = pack_bf16x2(acc[8 + 2 * k], acc[8 + 2 * k + 1]);
                }
                *reinterpret_cast<u32x4*>(rowp + a[bb]) = o0;
                *reinterpret_cast<u32x4*>(rowp + a[bb] + 32) = o1;
            }
        }
        __syncthreads();

        // coalesced stores of the finished tile
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (t0 + grow[k] >= p.T) continue;
            const int64_t slot = slot_lds[t0 - tile_begin * kTileTokens + grow[k]];
            if (slot < 0) continue;
            const u32x4 w = *reinterpret_cast<const u32x4*>(tile_lds + loff[k]);
            st_stream(dst + slot * F + fw0 + (goff[k] - grow[k] * F), w);
        }
        // the next tile's LDS writes must wait until every thread has read this one
        __syncthreads();
    };

    TileBuf bufA, bufB;
    load_tile(bufA, tile_begin * kTileTokens);
    if (DEPTH == 2 && tile_begin + 1 < tile_end) load_tile(bufB, (tile_begin + 1) * kTileTokens);

    // slots of the group's tokens, bounds-checked (out of range: row skipped)
#pragma unroll
    for (int k = 0; k < kSlotLoads; ++k) {
        const int r = tid + k * nthreads;
        if (r < ntok) {
            const int64_t slot = slot_from(p, tok0 + r, page_raw[k], off_raw, err);
            slot_lds[r] = slot;
        }
    }

    if (rot && lane < 32) {
        int64_t delta;
        if (p.mode == MODE_DELTA) {
            delta = delta_in;
        } else {
            delta = (p.mode == MODE_REORDER) ? p.base_pos + (int64_t)i * p.T - pc_in : target_in - pc_in;
        }
        cs_lds[wave][lane] = rope_phase_of(rope_theta(tt, theta_in, p.log2_base, p.rope_dim, jph), delta);
    }
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 zero = {0u, 0u, 0u, 0u};
            aop[bb][ks] = __builtin_bit_cast(bf16x8, 16 * ks + 8 * hh < p.rank ? aop_raw[bb][ks] : zero);
        }

    if (DEPTH == 1) {
        for (int tile = tile_begin; tile < tile_end; ++tile) process_tile(bufA, tile, tile + 1);
    } else {
        for (int tile = tile_begin; tile < tile_end; tile += 2) {
            process_tile(bufA, tile, tile + 2);
            if (tile + 1 < tile_end) process_tile(bufB, tile + 1, tile + 3);
        }
    }
    if (err && p.error_word) atomicOr(p.error_word, err);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

struct Tuning {
    int row_unroll = 2;          // relocate_rows_kernel: 16-byte vectors per thread (1 or 2)
    int tiles_per_wave = 0;      // relocate_patch_kernel; 0 = pick from the size
    int patch_kernel = 1;        // 1: LDS-staged patch kernel, 0: direct MFMA-layout kernel
    int window_waves = 0;        // LDS kernel: cap on waves per workgroup (0 = widest window)
    int patch_depth = 1;         // patch kernels: tiles prefetched ahead (1 or 2)
    int patch_nt = 0;            // relocate_patch_kernel: nontemporal row loads/stores
                                 // (measured: cached ones let L2 merge the partial-line
                                 // accesses of the MFMA layout; nontemporal ones do not)
    int min_waves = 16384;       // target wave count for the automatic pick
};

Tuning g_tuning;
std::once_flag g_tuning_once;

void load_tuning() {
    // Optional tuning knobs for measurements: KAMERA_ROW_UNROLL,
    // KAMERA_TILES_PER_WAVE (token tiles of 32 per wave), KAMERA_PATCH_DEPTH,
    // KAMERA_PATCH_NT.
    if (const char* e = getenv("KAMERA_ROW_UNROLL")) {
        int v = atoi(e);
        if (v == 1 || v == 2) g_tuning.row_unroll = v;
    }
    if (const char* e = getenv("KAMERA_PATCH_NT")) g_tuning.patch_nt = atoi(e) ? 1 : 0;
    if (const char* e = getenv("KAMERA_PATCH_KERNEL")) g_tuning.patch_kernel = atoi(e) ? 1 : 0;
    if (const char* e = getenv("KAMERA_WINDOW_WAVES")) g_tuning.window_waves = atoi(e);
    if (const char* e = getenv("KAMERA_PATCH_DEPTH")) g_tuning.patch_depth = atoi(e) >= 2 ? 2 : 1;
    if (const char* e = getenv("KAMERA_TILES_PER_WAVE")) {
        int v = atoi(e);
        if (v >= 1 && v <= 1024) g_tuning.tiles_per_wave = v;
    }
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

struct Span {
    uintptr_t lo, hi;
};

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// Elements -> byte span of a strided [outer][...][rows][F] region.
Span span_of(const void* base, int64_t elems) {
    uintptr_t lo = (uintptr_t)base;
    return Span{lo, lo + (uintptr_t)elems * 2u};
}

int build_segments(const kamera_layout& L, SegmentTable& st) {
    int n = 0;
    auto push = [&](int r0, int r1, int j0, int rot) {
        if (n >= kMaxSegments) return false;
        st.seg[n++] = Segment{(int16_t)r0, (int16_t)r1, (int16_t)j0, (int16_t)rot};
        return true;
    };
    const int D = L.head_dim, o = L.rope_offset, R = L.rope_dim;
    for (int h = 0; h < L.num_heads; ++h) {
        const int base = h * D;
        for (int a = 0; a < o; a += 64)
            if (!push(base + a, base + a + 32, 0, 0)) return -1;
        if (L.rope_style == KAMERA_ROPE_HALF) {
            // pair j joins element o + j and o + R/2 + j
            for (int j0 = 0; j0 < R / 2; j0 += 32)
                if (!push(base + o + j0, base + o + R / 2 + j0, j0, 1)) return -1;
        } else {
            // pair j joins elements o + 2j and o + 2j + 1
            for (int k = 0; k < R; k += 64)
                if (!push(base + o + k, base + o + k + 32, k / 2, 1)) return -1;
        }
        for (int a = o + R; a < D; a += 64)
            if (!push(base + a, base + a + 32, 0, 0)) return -1;
    }
    st.count = n;
    return n;
}

// Waves per workgroup of the LDS-staged patch kernel: the largest W <= 4 that
// divides the segment count and makes every window of W consecutive segments
// cover exactly the contiguous features [r0 of its first segment, + 64W).
int window_waves(const SegmentTable& st) {
    for (int W = kMaxWindowWaves; W > 1; --W) {
        if (st.count % W) continue;
        bool good = true;
        for (int w0 = 0; w0 < st.count && good; w0 += W) {
            const int lo = st.seg[w0].r0, hi = lo + 64 * W;
            for (int k = w0; k < w0 + W; ++k) {
                const Segment& sg = st.seg[k];
                if (sg.r0 < lo || sg.r0 + 32 > hi || sg.r1 < lo || sg.r1 + 32 > hi) good = false;
            }
        }
        if (good) return W;
    }
    return 1;
}

kamera_status check_layout(const kamera_layout* L) {
    if (!L) return KAMERA_ERR_NULL;
    if (L->num_layers < 1 || L->num_heads < 1 || L->head_dim < 1) return KAMERA_ERR_RANGE;
    if (L->num_streams < 1 || L->num_streams > 2) return KAMERA_ERR_RANGE;
    if (L->rope_style != KAMERA_ROPE_HALF && L->rope_style != KAMERA_ROPE_INTERLEAVED) return KAMERA_ERR_RANGE;
    if (L->rope_offset < 0 || L->rope_dim < 0 || L->rope_offset + L->rope_dim > L->head_dim) return KAMERA_ERR_RANGE;
    if (!(L->rope_base > 0.0) || !isfinite(L->rope_base)) return KAMERA_ERR_RANGE;
    if (L->head_dim % 64 || L->rope_offset % 64 || L->rope_dim % 64) return KAMERA_ERR_UNSUPPORTED;
    if (L->head_dim > 1024 || (int64_t)L->num_heads * L->head_dim > 4096) return KAMERA_ERR_UNSUPPORTED;
    return KAMERA_OK;
}

struct Call {
    Params p;
    bool patched = false;
};

// Everything the host can check, before any HIP call.
kamera_status prepare(const kamera_layout* layout, const kamera_src* src, int32_t n, const kamera_patch* patch,
                      const kamera_dst* dst, int mode, Call& call, bool& empty) {
    kamera_status st = check_layout(layout);
    if (st != KAMERA_OK) return st;
    if (!src || !dst) return KAMERA_ERR_NULL;
    const kamera_layout& L = *layout;
    const int S = L.num_streams;
    const int64_t F = (int64_t)L.num_heads * L.head_dim;
    if (n < 0 || src->n_tokens < 0 || src->n_store < 1) return KAMERA_ERR_RANGE;
    if (mode == MODE_DELTA && n > src->n_store) return KAMERA_ERR_RANGE;
    const int T = src->n_tokens;
    if ((int64_t)T * F > INT32_MAX) return KAMERA_ERR_RANGE;  // in-slice offsets are 32-bit
    const int m = patch ? patch->rank : 0;
    if (m < 0 || m > 64) return KAMERA_ERR_RANGE;
    if (m % 8) return KAMERA_ERR_UNSUPPORTED;
    if (src->chunk_stride < 0 || src->layer_stride < 0 || dst->layer_stride < 0) return KAMERA_ERR_RANGE;
    if (dst->num_slots < 0 || dst->page_size < 0) return KAMERA_ERR_RANGE;
    for (int s = 0; s < S; ++s) {
        if (!src->rows[s] || !dst->rows[s]) return KAMERA_ERR_NULL;
        if (!aligned16(src->rows[s]) || !aligned16(dst->rows[s])) return KAMERA_ERR_ALIGN;
        if (m > 0) {
            if (!patch->u[s] || !patch->v[s]) return KAMERA_ERR_NULL;
            if (!aligned16(patch->u[s]) || !aligned16(patch->v[s])) return KAMERA_ERR_ALIGN;
        }
    }
    if (src->chunk_stride % 8 || src->layer_stride % 8 || dst->layer_stride % 8) return KAMERA_ERR_ALIGN;
    if (dst->page_size > 0 && !dst->page_table && n > 0) return KAMERA_ERR_NULL;
    if (dst->page_size == 0 && !dst->dst_offset && n > 0) return KAMERA_ERR_NULL;

    empty = (n == 0 || T == 0);
    if (empty) return KAMERA_OK;

    // shapes: a chunk's rows must fit its strides, and the pool's layers must not overlap
    if (L.num_layers > 1 && src->layer_stride < (int64_t)T * F) return KAMERA_ERR_SHAPE;
    if (src->n_store > 1 && src->chunk_stride < (int64_t)T * F) return KAMERA_ERR_SHAPE;
    if (L.num_layers > 1 && dst->layer_stride < dst->num_slots * F) return KAMERA_ERR_SHAPE;
    if (dst->num_slots < T) return KAMERA_ERR_RANGE;
    if (dst->page_size > 0 && dst->num_slots / dst->page_size < 1) return KAMERA_ERR_RANGE;
    if ((int64_t)n * L.num_layers * S * ((T + 31) / 32) > (int64_t)1 << 40) return KAMERA_ERR_RANGE;

    // the destination must not overlap any input
    const int64_t src_elems =
        (int64_t)(src->n_store - 1) * src->chunk_stride + (int64_t)(L.num_layers - 1) * src->layer_stride + (int64_t)T * F;
    const int64_t dst_elems = (int64_t)(L.num_layers - 1) * dst->layer_stride + dst->num_slots * F;
    const int64_t u_elems = (int64_t)src->n_store * L.num_layers * T * m;
    const int64_t v_elems = (int64_t)src->n_store * L.num_layers * F * m;
    for (int s = 0; s < S; ++s) {
        const Span d = span_of(dst->rows[s], dst_elems);
        for (int s2 = 0; s2 < S; ++s2) {
            if (overlap(d, span_of(src->rows[s2], src_elems))) return KAMERA_ERR_ALIAS;
            if (m > 0 && (overlap(d, span_of(patch->u[s2], u_elems)) || overlap(d, span_of(patch->v[s2], v_elems))))
                return KAMERA_ERR_ALIAS;
            if (s2 != s && overlap(d, span_of(dst->rows[s2], dst_elems))) return KAMERA_ERR_ALIAS;
        }
    }

    Params& p = call.p;
    memset(&p, 0, sizeof(p));
    for (int s = 0; s < S; ++s) {
        p.src[s] = src->rows[s];
        p.dst[s] = dst->rows[s];
        if (m > 0) {
            p.u[s] = patch->u[s];
            p.v[s] = patch->v[s];
        }
    }
    p.src_chunk_stride = src->chunk_stride;
    p.src_layer_stride = src->layer_stride;
    p.canon_pos = src->canon_pos;
    p.dst_layer_stride = dst->layer_stride;
    p.num_slots = dst->num_slots;
    p.page_table = dst->page_table;
    p.dst_offset = dst->dst_offset;
    p.error_word = dst->error_word;
    p.log2_base = log2(L.rope_base);
    p.mode = mode;
    p.rank = m;
    p.page_size = dst->page_size;
    p.pages_per_chunk = dst->page_size > 0 ? (T + dst->page_size - 1) / dst->page_size : 0;
    p.page_shift = -1;
    if (dst->page_size > 0 && (dst->page_size & (dst->page_size - 1)) == 0) {
        p.page_shift = 0;
        while ((1 << p.page_shift) < dst->page_size) ++p.page_shift;
    }
    p.n = n;
    p.n_store = src->n_store;
    p.L = L.num_layers;
    p.S = S;
    p.T = T;
    p.F = (int32_t)F;
    p.D = L.head_dim;
    p.rope_offset = L.rope_offset;
    p.rope_dim = L.rope_dim;
    p.rope_style = L.rope_style;
    call.patched = m > 0;
    return KAMERA_OK;
}

kamera_status launch(const kamera_layout* layout, Call& call, void* stream) {
    std::call_once(g_tuning_once, load_tuning);
    Params& p = call.p;
    ThetaTable tt;
    memset(&tt, 0, sizeof(tt));
    if (p.rope_dim / 2 <= kMaxThetas) {
        tt.count = p.rope_dim / 2;
        for (int j = 0; j < tt.count; ++j) tt.theta[j] = pow(layout->rope_base, -2.0 * j / (double)p.rope_dim);
    }
    hipStream_t hs = (hipStream_t)stream;
    hipError_t e;
    if (!call.patched) {
        const int u = g_tuning.row_unroll;
        const int64_t nvec = (int64_t)p.T * (p.F >> 3);
        if (nvec > INT32_MAX / 2) return KAMERA_ERR_RANGE;
        const int per_slice = (int)((nvec + (int64_t)kThreads * u - 1) / ((int64_t)kThreads * u));
        const int64_t blocks = (int64_t)p.n * p.S * p.L * per_slice;
        if (blocks > INT32_MAX) return KAMERA_ERR_RANGE;
        const FastDiv dvr = make_fastdiv((uint32_t)(p.F >> 3));
        const FastDiv dhd = make_fastdiv((uint32_t)(p.D >> 3));
        const FastDiv dupr = make_fastdiv((uint32_t)(p.F >> 4));  // pair units per row
        const FastDiv duph = make_fastdiv((uint32_t)(p.D >> 4));  // pair units per head
        void* args[] = {&p, &tt, (void*)&per_slice, (void*)&dvr, (void*)&dhd, (void*)&dupr, (void*)&duph};
        const void* fn = u == 1 ? (const void*)relocate_rows_kernel<1> : (const void*)relocate_rows_kernel<2>;
        e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), args, 0, hs);
    } else {
        SegmentTable st;
        memset(&st, 0, sizeof(st));
        if (build_segments(*layout, st) <= 0) return KAMERA_ERR_UNSUPPORTED;
        const int ks = (p.rank + 15) / 16;
        const int tiles_total = (p.T + 31) / 32;
        if (g_tuning.patch_kernel == 1) {
            int W = window_waves(st);
            if (g_tuning.window_waves > 0 && g_tuning.window_waves < W && W % g_tuning.window_waves == 0)
                W = g_tuning.window_waves;
            const int windows = st.count / W;
            int tpg = g_tuning.tiles_per_wave > 0 ? g_tuning.tiles_per_wave : 2;
            tpg = std::min(std::min(tpg, kMaxTilesPerGroup), tiles_total);
            const int groups = (tiles_total + tpg - 1) / tpg;
            const int64_t blocks = (int64_t)p.n * p.S * p.L * windows * groups;
            if (blocks > INT32_MAX) return KAMERA_ERR_RANGE;
            void* args[] = {&p, &tt, &st, (void*)&W, (void*)&windows, (void*)&tiles_total, (void*)&tpg,
                            (void*)&groups};
            static const void* const kLds[2][4] = {
                {(const void*)relocate_patch_lds_kernel<1, 1>, (const void*)relocate_patch_lds_kernel<2, 1>,
                 (const void*)relocate_patch_lds_kernel<3, 1>, (const void*)relocate_patch_lds_kernel<4, 1>},
                {(const void*)relocate_patch_lds_kernel<1, 2>, (const void*)relocate_patch_lds_kernel<2, 2>,
                 (const void*)relocate_patch_lds_kernel<3, 2>, (const void*)relocate_patch_lds_kernel<4, 2>}};
            e = hipLaunchKernel(kLds[g_tuning.patch_depth - 1][ks - 1], dim3((unsigned)blocks), dim3(64 * W), args,
                                0, hs);
        } else {
            const int64_t units = (int64_t)p.n * p.S * p.L * st.count;
            int tpw = g_tuning.tiles_per_wave;
            if (tpw <= 0) {
                tpw = 8;
                while (tpw > 1 && units * ((tiles_total + tpw - 1) / tpw) < g_tuning.min_waves) tpw >>= 1;
            }
            tpw = std::min(tpw, tiles_total);
            const int groups = (tiles_total + tpw - 1) / tpw;
            const int64_t items64 = units * groups;
            const int64_t wgs = (items64 + kWaves - 1) / kWaves;
            const int64_t grid = (wgs + kXcds - 1) / kXcds * kXcds;
            if (grid * kWaves > INT32_MAX) return KAMERA_ERR_RANGE;
            const int items = (int)items64;
            const int per_xcd = (int)(grid / kXcds);
            void* args[] = {&p, &tt, &st, &tpw, (void*)&groups, (void*)&items, (void*)&per_xcd};
#define KAMERA_PATCH_ROW(NT, D)                                                                   \
    {(const void*)relocate_patch_kernel<1, NT, D>, (const void*)relocate_patch_kernel<2, NT, D>,     \
     (const void*)relocate_patch_kernel<3, NT, D>, (const void*)relocate_patch_kernel<4, NT, D>}
            static const void* const kPatch[2][2][4] = {{KAMERA_PATCH_ROW(0, 1), KAMERA_PATCH_ROW(0, 2)},
                                                        {KAMERA_PATCH_ROW(1, 1), KAMERA_PATCH_ROW(1, 2)}};
#undef KAMERA_PATCH_ROW
            const void* fn = kPatch[g_tuning.patch_nt][g_tuning.patch_depth - 1][ks - 1];
            e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kThreads), args, 0, hs);
        }
    }
    return e == hipSuccess ? KAMERA_OK : KAMERA_ERR_HIP;
}

kamera_status run(const kamera_layout* layout, const kamera_src* src, int32_t n, const kamera_patch* patch,
                  const kamera_dst* dst, int mode, const int64_t* delta, const int32_t* ids,
                  const int64_t* target, int64_t base_pos, void* stream) {
    Call call;
    bool empty = false;
    kamera_status st = prepare(layout, src, n, patch, dst, mode, call, empty);
    if (st != KAMERA_OK || empty) return st;
    if (mode == MODE_DELTA && !delta) return KAMERA_ERR_NULL;
    if (mode != MODE_DELTA && !ids) return KAMERA_ERR_NULL;
    if (mode == MODE_RECALL && !target) return KAMERA_ERR_NULL;
    call.p.delta = delta;
    call.p.ids = ids;
    call.p.target = target;
    call.p.base_pos = base_pos;
    return launch(layout, call, stream);
}

}  // namespace

extern "C" {

kamera_status kamera_relocate(const kamera_layout* layout, const kamera_src* src, int32_t n, const int64_t* delta,
                              const kamera_dst* dst, void* hip_stream) {
    return run(layout, src, n, nullptr, dst, MODE_DELTA, delta, nullptr, nullptr, 0, hip_stream);
}

kamera_status kamera_relocate_patch(const kamera_layout* layout, const kamera_src* src, int32_t n,
                                    const int64_t* delta, const kamera_patch* patch, const kamera_dst* dst,
                                    void* hip_stream) {
    if (!patch) return KAMERA_ERR_NULL;
    return run(layout, src, n, patch, dst, MODE_DELTA, delta, nullptr, nullptr, 0, hip_stream);
}

kamera_status kamera_reorder(const kamera_layout* layout, const kamera_src* src, int32_t n, const int32_t* perm,
                             int64_t base_pos, const kamera_patch* orbit, const kamera_dst* dst, void* hip_stream) {
    return run(layout, src, n, orbit, dst, MODE_REORDER, nullptr, perm, nullptr, base_pos, hip_stream);
}

kamera_status kamera_recall(const kamera_layout* layout, const kamera_src* src, int32_t n, const int32_t* chunk_ids,
                            const int64_t* target_pos, const kamera_patch* patch, const kamera_dst* dst,
                            void* hip_stream) {
    return run(layout, src, n, patch, dst, MODE_RECALL, nullptr, chunk_ids, target_pos, 0, hip_stream);
}

const char* kamera_status_string(kamera_status status) {
    switch (status) {
        case KAMERA_OK: return "ok";
        case KAMERA_ERR_NULL: return "a required pointer is NULL";
        case KAMERA_ERR_ALIGN: return "a row base, factor base or stride is not 16-byte aligned";
        case KAMERA_ERR_SHAPE: return "sizes are inconsistent with each other";
        case KAMERA_ERR_RANGE: return "a count or size is out of range";
        case KAMERA_ERR_ALIAS: return "the destination overlaps the source";
        case KAMERA_ERR_UNSUPPORTED: return "shape not supported by the kernels";
        case KAMERA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

int32_t kamera_version(void) { return 100; }

}  // extern "C"
