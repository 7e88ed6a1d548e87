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
//  * relocate_patch_lds_kernel (m > 0).  The rank-m patch is a dense
//    contraction over m, so it runs on the matrix cores.  A workgroup of W
//    waves stages a 32-token x 64W-feature tile of canonical rows in LDS with
//    coalesced loads; each wave rotates one 64-feature segment and keeps it in
//    the fp32 accumulator of v_mfma_f32_32x32x16_bf16, so that
//    D = R(delta) x + V_f U_t^T comes out of the MFMA in place.  The MFMA rows
//    (features) are relabelled so that each lane's accumulator values are
//    contiguous features of its token, and the rotate-half partner of every
//    value sits in the same lane.  The rounded tile goes back through LDS to
//    coalesced stores.
//
// Rounding: fp32 -> bf16 with v_cvt_pk_bf16_f32 (round to nearest even).

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <tuple>
#include <utility>

#include "kamera.h"
#include "kamera_common.h"

namespace {

constexpr int kMaxSegments = 64;       // 64 x 64 elements: rows up to 4096 wide
constexpr int kMaxHalfRope = 512;
constexpr int kThreads = 256;          // both kernels: 4 waves of 64
constexpr int kMaxBlockRows = 64;      // rows one block of the m = 0 kernel touches (<= one wave)
static_assert(kThreads * 2 / 8 <= kMaxBlockRows, "a block of 2 vectors per thread spans more rows than a wave");
constexpr int kMaxGridZ = 65535;       // grid y / z limit: layers on y, (chunk, stream) on z in batches
constexpr int64_t kRowUnrollOneVectors = int64_t(1) << 26;  // 1 GiB of rows: one vector per thread from here



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
    int64_t num_pages;   // num_slots / page_size (0 for a contiguous pool)
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
    FastDiv page_div;    // divides by page_size (by 1 for a contiguous pool)
    int32_t n, n_store, L, S, T, F;
    int32_t D, rope_offset, rope_dim, rope_style;
    int32_t partner_lanes;  // m = 0 kernel: rotate-half partner sits this many lanes away (xor), 0 = load it
    // Destination order (paged pools): page_order[r] is the page-table entry
    // (i * pages_per_chunk + j) of the r-th page in ascending page-id order
    // (within runs of kSortRun entries); the kernels' BY_PAGE variants walk
    // those entries instead of (chunk, token).
    const int32_t* page_order;
    int32_t entries;     // n * pages_per_chunk
    FastDiv unit_div;    // divides a block index by the blocks (or token groups) per page
    FastDiv ppc_div;     // divides an entry by pages_per_chunk
    // Variable-length chunks (the kernels' VARLEN variants): store chunk c has
    // vl_tokens[c] <= T tokens, its rows (and U rows) starting at row
    // vl_row_offset[c], layer by layer; the store holds vl_total_rows rows.
    const int64_t* vl_row_offset;
    const int32_t* vl_tokens;
    int64_t vl_total_rows;
};

enum { MODE_DELTA = 0, MODE_REORDER = 1, MODE_RECALL = 2 };

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------


// A readable zero: the address a select falls back to when an optional input
// (chunk ids, page table, offsets) does not apply, so that the read itself
// needs no branch.
__device__ int64_t kZeroWord = 0;  // never written

// Marker of a page-table or chunk entry the content checks removed (a repeat
// of an earlier entry): the kernels skip it as they skip an out-of-range
// value, without flagging a range error.
constexpr int32_t kSkipEntry = INT32_MIN;

// Chunk id of output chunk i: ids[i] when the call has ids, else i.
__device__ __forceinline__ int chunk_of(const Params& p, int i) {
    const bool has_ids = p.mode != MODE_DELTA;
    const int id = ld_uniform(has_ids ? p.ids + i : reinterpret_cast<const int32_t*>(&kZeroWord));
    return has_ids ? id : i;
}


// cos/sin of delta * theta_j for this call's base and rotary span.
__device__ __forceinline__ float2 rope_phase(const Params& p, int j, int64_t delta) {
    return rope_cos_sin(p.log2_base, p.rope_dim, j, delta);
}

// Page-table column of token t of a chunk.
__device__ __forceinline__ int page_of(const Params& p, int t) {
    return (int)fdiv((uint32_t)t, p.page_div);
}

// Pool slot of token t of output chunk i from its page id (paged pool; the id
// read from the page table) or from the chunk's offset (contiguous pool), or
// -1 when the id or the offset is out of range (then the row is skipped and
// the error bit recorded).  The reads happen in the caller, ahead of the bulk
// loads, so that no wait on them holds up the rows.
__device__ __forceinline__ int64_t slot_from(const Params& p, int t, int32_t page_id, int64_t offset, int T,
                                             uint32_t& err) {
    // selects only: a branch would let the compiler sink the id's load into it
    const bool paged = p.page_size > 0;
    const bool bad_page = paged && (page_id < 0 || (int64_t)page_id >= p.num_pages);
    const bool bad_off = !paged && (offset < 0 || offset + T > p.num_slots);
    err |= ((bad_page && page_id != kSkipEntry) ? (uint32_t)KAMERA_EW_PAGE : 0u) |
           (bad_off ? (uint32_t)KAMERA_EW_OFFSET : 0u);
    const int64_t in_page = (int64_t)page_id * p.page_size + (t - page_of(p, t) * p.page_size);
    return (bad_page || bad_off) ? -1 : (paged ? in_page : offset + t);
}

// ---------------------------------------------------------------------------
// Destination order: sort the call's page-table entries by page id
// ---------------------------------------------------------------------------

constexpr int kSortRun = 8192;    // entries one workgroup sorts (64 KiB of keys in LDS)
constexpr int kSortThreads = 1024;

// Bitonic sort of key[0, np) in LDS, ascending (np a power of two <= kSortRun);
// every thread of the workgroup takes part.
__device__ void bitonic_sort_lds(uint64_t* key, const int np) {
    for (int size = 2; size <= np; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = threadIdx.x; t < (np >> 1); t += kSortThreads) {
                const int lo = 2 * t - (t & (stride - 1));  // pair (lo, lo + stride), lo's stride bit clear
                const int hi = lo + stride;
                const bool ascending = (lo & size) == 0;
                const uint64_t a = key[lo], b = key[hi];
                if ((a > b) == ascending) {
                    key[lo] = b;
                    key[hi] = a;
                }
            }
            __syncthreads();
        }
    }
}

// Key of entry k of a run: the value (sign-flipped, so that the unsigned
// order is the signed one) above the entry's index, so equal values keep entry
// order.  Entries past the run's end sort last.
__device__ __forceinline__ uint64_t value_key(int32_t v, int k) {
    return ((uint64_t)((uint32_t)v ^ 0x80000000u) << 32) | (uint32_t)k;
}
__device__ __forceinline__ int32_t key_value(uint64_t key) { return (int32_t)((uint32_t)(key >> 32) ^ 0x80000000u); }

// Workgroup r sorts entries [r*kSortRun, min(total, (r+1)*kSortRun)) of the
// flattened page table by page id (keys as above) and writes the entry
// indices in that order.  A run is padded to a power of two with keys that
// sort last.
__global__ __launch_bounds__(kSortThreads) void sort_pages_kernel(const int32_t* __restrict__ page_table,
                                                                  int32_t* __restrict__ order, const int total) {
    __shared__ uint64_t key[kSortRun];
    const int r0 = (int)blockIdx.x * kSortRun;
    const int len = min(kSortRun, total - r0);
    int np = 1;
    while (np < len) np <<= 1;
    for (int k = threadIdx.x; k < np; k += kSortThreads)
        key[k] = k < len ? value_key(page_table[r0 + k], r0 + k) : ~0ull;
    __syncthreads();
    bitonic_sort_lds(key, np);
    for (int k = threadIdx.x; k < len; k += kSortThreads) order[r0 + k] = (int32_t)(uint32_t)key[k];
}

// Content check of one index array (page table or chunk entries): out[k] =
// vals[k], except that an entry whose value lies in [0, bound) and equals the
// value of an earlier entry becomes kSkipEntry, and `flag` is OR-ed into
// error_word if any did.  Workgroup r owns the run of kSortRun entries from
// r*kSortRun: it sorts the run's keys in LDS, marks every entry whose sorted
// predecessor has the same value (a repeat inside the run: equal values keep
// entry order), then, for every earlier run, looks each of its values up in
// the sorted run (binary search) and marks the first own entry of that value
// (an earlier run's entry precedes all of this run's).  Bit 31 of a key's low
// word marks a repeat (entry indices inside a run are < 2^13).
constexpr uint64_t kRepeatBit = 0x80000000ull;

__global__ __launch_bounds__(kSortThreads) void dedup_kernel(const int32_t* __restrict__ vals, int32_t* __restrict__ out,
                                                             const int len, const int bound,
                                                             uint32_t* __restrict__ error_word, const uint32_t flag) {
    __shared__ uint64_t key[kSortRun];
    __shared__ int any_repeat;
    const int r0 = (int)blockIdx.x * kSortRun;
    const int n = min(kSortRun, len - r0);
    int np = 1;
    while (np < n) np <<= 1;
    if (threadIdx.x == 0) any_repeat = 0;
    for (int k = threadIdx.x; k < np; k += kSortThreads) key[k] = k < n ? value_key(vals[r0 + k], k) : ~0ull;
    __syncthreads();
    bitonic_sort_lds(key, np);
    // repeats inside the run: decided for every entry first, then marked
    constexpr int kPer = kSortRun / kSortThreads;
    bool rep[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int k = (int)threadIdx.x + q * kSortThreads;
        rep[q] = false;
        if (k > 0 && k < n) {
            const int32_t v = key_value(key[k]);
            rep[q] = v >= 0 && v < bound && key_value(key[k - 1]) == v;
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kPer; ++q)
        if (rep[q]) key[threadIdx.x + q * kSortThreads] |= kRepeatBit;
    __syncthreads();
    // repeats of earlier runs' values
    for (int e = threadIdx.x; e < r0; e += kSortThreads) {
        const int32_t v = vals[e];
        if (v < 0 || v >= bound) continue;
        int lo = 0, hi = n;  // first sorted position whose value is >= v
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (key_value(key[mid]) < v) lo = mid + 1;
            else hi = mid;
        }
        if (lo < n && key_value(key[lo]) == v) atomicOr((unsigned long long*)&key[lo], (unsigned long long)kRepeatBit);
    }
    __syncthreads();
    bool mine = false;
    for (int k = threadIdx.x; k < n; k += kSortThreads) {
        const uint64_t kk = key[k];
        const int idx = (int)((uint32_t)kk & 0x7FFFFFFFu);
        const bool repeat = (kk & kRepeatBit) != 0;
        out[r0 + idx] = repeat ? kSkipEntry : key_value(kk);
        mine |= repeat;
    }
    if (mine) any_repeat = 1;
    __syncthreads();
    if (threadIdx.x == 0 && any_repeat && error_word) atomicOr(error_word, flag);
}

// Page-table entry of the r-th page in destination order, clamped to the table
// (the sort writes a permutation of [0, entries); the clamp only guards reads).
__device__ __forceinline__ int ordered_entry(const Params& p, int r) {
    const int e = ld_uniform(p.page_order + min(r, p.entries - 1));
    return min(max(e, 0), p.entries - 1);
}

// Length and first row of store chunk c of a variable-length call, or false
// when they do not fit the call's bounds (then the chunk is skipped whole).
// Scalar loads: c is uniform over the workgroup.
__device__ __forceinline__ bool varlen_chunk(const Params& p, int c, int& T, int64_t& row0) {
    const int tc = ld_uniform(p.vl_tokens + c);
    const int64_t r0 = ld_uniform(p.vl_row_offset + c);
    const bool good = tc >= 0 && tc <= p.T && r0 >= 0 && r0 <= p.vl_total_rows - (int64_t)p.L * tc;
    T = good ? tc : 0;
    row0 = good ? r0 : 0;
    return good;
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
//
// Grid: x = block of the slice, y = layer, z = z_base + (output chunk * S +
// stream), so a workgroup finds its slice without any division.
// What a stream of a call does to its rows; each kind is a separate
// straight-line body, chosen once per workgroup, so that no load crosses a
// branch join (a join would make the compiler wait for every load in flight).
enum RowKind {
    kCopy = 0,         // no rotation (value stream, or no rotary span): raw bits
    kPairs = 1,        // rotate-half over whole heads, pair units (U = 2)
    kPartner = 2,      // rotate-half, each rotated vector also reads its partner
    kInterleaved = 3,  // (2j, 2j+1) pairs, inside one vector
    kShuffle = 4,      // rotate-half, partner taken from lane ^ (R/16) of the same wave
};

// Vector of lane (lane ^ d) of the wave, d = 4, 8, 16 or 32 (d = 8: a DPP
// rotate by 8 inside each row of 16 lanes, which is the same permutation).
__device__ __forceinline__ u32x4 lane_xor(u32x4 v, int d) {
    u32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (d == 8)
            r[q] = (uint32_t)__builtin_amdgcn_mov_dpp((int)v[q], 0x128, 0xF, 0xF, false);  // row_ror:8
        else
            r[q] = (uint32_t)__shfl_xor((int)v[q], d);
    }
    return r;
}

template <int U, int KIND, bool VARLEN>
__device__ __forceinline__ bool rows_body(const Params& p, const int v0, const int l,
                                          const int s, const int i, const FastDiv& div_vr, const FastDiv& div_hd,
                                          const FastDiv& div_upr, const FastDiv& div_uph, float2* cs,
                                          int64_t* slot_of_row) {
    constexpr bool kRot = KIND != kCopy;
    vm_settled();  // no vector load has been issued yet
    const int c = chunk_of(p, i);
    bool ok = c >= 0 && c < p.n_store;
    // a rejected chunk id reads chunk 0 (in range) and stores nothing
    int T = p.T;
    int64_t sofs = (int64_t)(ok ? c : 0) * p.src_chunk_stride + (int64_t)l * p.src_layer_stride;
    if (VARLEN) {
        int64_t row0;
        ok = varlen_chunk(p, ok ? c : 0, T, row0) && ok;
        sofs = (row0 + (int64_t)l * T) * p.F;
    }
    uint32_t err = (ok || c == kSkipEntry) ? 0u : (uint32_t)KAMERA_EW_CHUNK;
    const int VR = p.F >> 3;
    const int VD = p.D >> 3;
    const int half = p.rope_dim >> 1;
    const int nvec = T * VR;
    if (VARLEN && v0 >= nvec) {  // past the chunk's rows (uniform over the workgroup)
        if (err && p.error_word && threadIdx.x == 0) atomicOr(p.error_word, err);
        return false;
    }
    const int r_first = (int)fdiv((uint32_t)v0, div_vr);
    const uint16_t* __restrict__ sb = p.src[s] + sofs;
    uint16_t* __restrict__ db = p.dst[s] + (int64_t)l * p.dst_layer_stride;

    // The small loads go first -- the page id (or offset) of the row this
    // thread resolves and theta of its frequency -- and stay raw until the row
    // loads are issued: loads retire in issue order, so a wait on them then
    // costs nothing.  Row loads are unconditional (addresses past the end are
    // clamped and their results not stored), so the waits stay exact.
    const int r_end = min(T, (int)fdiv((uint32_t)min(v0 + kThreads * U, nvec) - 1u, div_vr) + 1);
    const int nrows = r_end - r_first;
    // wave 0 resolves the block's rows: at most 64 (256*U <= 512 vectors, rows
    // of >= 8 vectors, blocks start on a row when rows are 8 vectors)
    const bool resolver = threadIdx.x < 64;
    const int t_own = r_first + min((int)threadIdx.x, nrows - 1);
    const bool paged = p.page_size > 0;
    int32_t page_raw = 0;
    if (resolver)
        page_raw = *(paged ? p.page_table + (int64_t)i * p.pages_per_chunk + page_of(p, t_own)
                           : reinterpret_cast<const int32_t*>(&kZeroWord));
    const int64_t off_raw = ld_uniform(paged ? &kZeroWord : p.dst_offset + i);

    int row[U], col[U], ecol[U];
    uint32_t so[U], yo[U];  // element offsets of the vector and of its rotate-half partner
#pragma unroll
    for (int k = 0; k < U; ++k) {
        row[k] = -1;
        ecol[k] = -1;
    }
    if (KIND == kPairs) {
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
        if (g == gc) {
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
            so[k] = (uint32_t)vc << 3;
            bool in_rope = false;
            int e = 0;
            if (kRot) {
                const int h = (int)fdiv((uint32_t)vec, div_hd);
                e = ((vec - h * VD) << 3) - p.rope_offset;
                in_rope = e >= 0 && e < p.rope_dim;
            }
            // vectors outside the rotary span re-read themselves
            if (KIND == kPartner) yo[k] = so[k] + (uint32_t)(in_rope ? ((e < half) ? half : -half) : 0);
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
    if (KIND == kPartner) {
        // the rotate-half partner, R/2 elements away (an L1 hit)
#pragma unroll
        for (int k = 0; k < U; ++k) y[k] = ld_stream(sb + yo[k]);
    }
    if (!ok) {
#pragma unroll
        for (int k = 0; k < U; ++k) row[k] = -1;
    }
    // Every lane of wave 0 resolves a row (lanes past the block's rows
    // re-resolve its last row into a spare entry), so the page-id load has a
    // use on every path of that wave and stays ahead of the row loads.
    if (resolver)
        slot_of_row[(int)threadIdx.x < nrows ? (int)threadIdx.x : kMaxBlockRows] =
            slot_from(p, t_own, page_raw, off_raw, T, err);
    if (kRot && ok) {
        int64_t delta;
        if (p.mode == MODE_DELTA) {
            delta = ld_uniform(p.delta + i);
        } else {
            const int64_t pc = p.canon_pos ? ld_uniform(p.canon_pos + c) : 0;
            delta = (p.mode == MODE_REORDER) ? p.base_pos + (int64_t)i * p.T - pc : ld_uniform(p.target + i) - pc;
        }
        for (int j = threadIdx.x; j < half; j += kThreads) cs[j] = rope_phase(p, j, delta);
    }
    __syncthreads();

    if (KIND == kShuffle) {
        // every lane is active here (no branch taken yet): fetch the partner
        // vector, R/2 elements = R/16 vectors away, from its lane
#pragma unroll
        for (int k = 0; k < U; ++k) y[k] = lane_xor(x[k], p.partner_lanes);
    }
    if (KIND == kPairs) {
        if (row[0] >= 0) {
            const int64_t slot = slot_of_row[row[0]];
            if (slot >= 0) {
                const int j0 = ecol[0];
                const u32x4 oa = rotate_half_vec(x[0], x[U - 1], cs, j0, true);
                const u32x4 ob = rotate_half_vec(x[U - 1], x[0], cs, j0, false);
                st_stream(db + slot * p.F + col[0], oa);
                st_stream(db + slot * p.F + col[U - 1], ob);
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            if (row[k] < 0) continue;
            const int64_t slot = slot_of_row[row[k]];
            if (slot < 0) continue;
            u32x4 out = x[k];
            const int e = ecol[k];
            if ((KIND == kPartner || KIND == kShuffle) && e >= 0) {
                const bool first = e < half;
                out = rotate_half_vec(x[k], y[k], cs, first ? e : e - half, first);
            }
            if (KIND == kInterleaved && e >= 0) out = rotate_pairs_vec(x[k], cs, e >> 1);
            st_stream(db + slot * p.F + col[k], out);
        }
    }
    if (err && p.error_word) atomicOr(p.error_word, err);
    return true;
}

template <int U, bool BY_PAGE, bool VARLEN>
__global__ __launch_bounds__(kThreads) void relocate_rows_kernel(const Params p,
                                                                 const int z_base,
                                                                 const FastDiv div_vr, const FastDiv div_hd,
                                                                 const FastDiv div_upr, const FastDiv div_uph) {
    __shared__ float2 cs[kMaxHalfRope];
    __shared__ int64_t slot_of_row[kMaxBlockRows + 1];  // + a spare entry
    const int bx = blockIdx.x;
    const int l = BY_PAGE ? (int)blockIdx.z : (int)blockIdx.y;
    const int z = z_base + (int)blockIdx.z;
    int s, i, v0;
    if (BY_PAGE) {
        // grid x = page rank * blocks per page + block of the page, y =
        // stream, z = layer: the pages of a (layer, stream) go out in
        // ascending page-id order, each block inside one page (P*F is a
        // multiple of 2048*U), and the streams alternate per layer.  (Streams
        // alternating per page between the two pools measured 9% slower on
        // MI355X, like scattered writes.)
        const int rank = (int)fdiv((uint32_t)bx, p.unit_div);
        const int e = ordered_entry(p, rank);
        i = (int)fdiv((uint32_t)e, p.ppc_div);
        const int j = e - i * p.pages_per_chunk;
        s = blockIdx.y;
        v0 = (j * p.page_size) * (p.F >> 3) + (bx - rank * (int)p.unit_div.d) * kThreads * U;
        if (v0 >= p.T * (p.F >> 3)) return;  // past a partial last page: no rows (uniform)
    } else {
        // grid x = block of the slice, z = output chunk * S + stream.  (Giving
        // each XCD a contiguous run of a slice's blocks instead of every 8th
        // one measured the same on MI355X.)
        s = p.S == 2 ? (z & 1) : 0;
        i = p.S == 2 ? (z >> 1) : z;
        v0 = bx * kThreads * U;
    }
    const bool rot = (s == 0) && (p.rope_dim > 0);
    auto body = [&](int vb) -> bool {
        if (!rot) return rows_body<U, kCopy, VARLEN>(p, vb, l, s, i, div_vr, div_hd, div_upr, div_uph, cs, slot_of_row);
        if (p.rope_style == KAMERA_ROPE_INTERLEAVED)
            return rows_body<U, kInterleaved, VARLEN>(p, vb, l, s, i, div_vr, div_hd, div_upr, div_uph, cs,
                                                      slot_of_row);
        if (U == 2 && p.rope_offset == 0 && p.rope_dim == p.D)
            return rows_body<U, U == 2 ? kPairs : kPartner, VARLEN>(p, vb, l, s, i, div_vr, div_hd, div_upr,
                                                                    div_uph, cs, slot_of_row);
        if (p.partner_lanes)
            return rows_body<U, kShuffle, VARLEN>(p, vb, l, s, i, div_vr, div_hd, div_upr, div_uph, cs, slot_of_row);
        return rows_body<U, kPartner, VARLEN>(p, vb, l, s, i, div_vr, div_hd, div_upr, div_uph, cs, slot_of_row);
    };
    // (variable lengths: the grid is sized by the longest chunk and the blocks
    // past a shorter chunk's end return at once; walking a chunk's blocks in a
    // loop from a grid sized by the mean length measured 45% slower on MI355X)
    body(v0);
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

// The U rows of a tile (the MFMA B operand, 32 tokens x 16*KS ranks) are
// loaded once per workgroup, a 16-byte chunk or two per thread, and parked in
// LDS next to the rows: chunk q = col * 2KS + 2ks + hh holds the operand of
// lane (col, hh) for k-step ks.  Every wave then reads its B operands from
// LDS instead of loading the whole U tile itself.
// 128 VGPRs (4 waves per SIMD) hold ranks up to 16, and ranks up to 32 with
// even windows, without spilling; the other shapes keep what they need.
template <int KS, int W, bool BY_PAGE, bool VARLEN>
__global__ __launch_bounds__(64 * W, (KS == 1 || (KS == 2 && W % 2 == 0)) ? 4 : 1) void relocate_patch_lds_kernel(
    const Params p, const SegmentTable st, const int z_base, const int tiles, const int tiles_per_wg,
    const FastDiv div_x) {
    constexpr int kRowBytes = 128 * W;
    constexpr int kPitch = kRowBytes + 16;               // bytes per LDS row (padded)
    constexpr int kUOffset = kTileTokens * kPitch;       // U chunks after the rows
    constexpr int kUChunks = 64 * KS;
    constexpr int kUPerThread = (kUChunks + 64 * W - 1) / (64 * W);
    __shared__ __attribute__((aligned(16))) uint8_t tile_lds[kUOffset + 16 * kUChunks];
    __shared__ float2 cs_lds[W][32];
    __shared__ int64_t slot_lds[kTileTokens * kMaxTilesPerGroup];  // pool slot of every token of the group
    constexpr int nthreads = 64 * W;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: segment reads are scalar
    const int hh = lane >> 5;
    const int col = lane & 31;
    constexpr int pitch = kPitch;

    // Grid: x = window * groups + token group (div_x divides by groups), y =
    // layer, z = z_base + (output chunk * S + stream).  Consecutive blocks go
    // round-robin over the 8 XCDs (block x on XCD x % 8); with a multiple of 8
    // groups, the windows of a group then share an XCD and its L2.  (A slice's
    // blocks spread over all XCDs; measured on MI355X, that beats keeping a
    // slice on one XCD even though each XCD's L2 then fetches the slice's V
    // rows.)
    // BY_PAGE: x = 8 * windows * (g / 8) + 8 * window + g % 8 (div_x divides by
    // 8 * windows), y = layer, z = stream: the windows of token group g run on
    // one XCD, which then fetches the group's U rows once, and within 8 *
    // windows consecutive blocks, so that a page is written out completely
    // before the pages after it.
    int win, g;
    if (BY_PAGE) {
        const uint32_t run = fdiv(blockIdx.x, div_x);
        win = (int)((blockIdx.x >> 3) - run * (div_x.d >> 3));
        g = (int)(run * 8u + (blockIdx.x & 7u));
    } else {
        win = (int)fdiv(blockIdx.x, div_x);
        g = (int)blockIdx.x - win * (int)div_x.d;
    }
    const int l = blockIdx.y;
    const int z = z_base + (int)blockIdx.z;
    int s, i, tile_begin;
    if (BY_PAGE) {
        // token groups walk the pages in ascending page-id order (z = stream);
        // a page holds a whole number of groups
        const int rank = (int)fdiv((uint32_t)g, p.unit_div);
        if (rank >= p.entries) return;  // padding of the last run of 8 groups (uniform)
        const int e = ordered_entry(p, rank);
        i = (int)fdiv((uint32_t)e, p.ppc_div);
        const int j = e - i * p.pages_per_chunk;
        s = z;
        tile_begin = j * (p.page_size / kTileTokens) + (g - rank * (int)p.unit_div.d) * tiles_per_wg;
        // groups past the end of a partial last page have no rows (uniform:
        // nobody reaches a barrier, and no clamped address goes negative)
        if (tile_begin >= tiles) return;
    } else {
        s = p.S == 2 ? (z & 1) : 0;
        i = p.S == 2 ? (z >> 1) : z;
        tile_begin = g * tiles_per_wg;
    }

    const int c = chunk_of(p, i);
    uint32_t err = 0;
    if (c < 0 || c >= p.n_store) {
        if (p.error_word && tid == 0 && c != kSkipEntry) atomicOr(p.error_word, (uint32_t)KAMERA_EW_CHUNK);
        return;  // uniform over the workgroup: nobody reaches a barrier
    }
    const Segment sg = st.seg[win * W + wave];
    const bool rot = sg.rot && s == 0;
    const int fw0 = st.seg[win * W].r0;  // first feature of the window
    const int F = p.F;
    const int64_t blk = (int64_t)c * p.L + l;
    // the block's first row: canonical rows by strides, U rows [T][m] per block
    int T = p.T;
    int64_t row0 = blk * p.T;
    int64_t sofs = (int64_t)c * p.src_chunk_stride + (int64_t)l * p.src_layer_stride;
    int ntiles = tiles;
    if (VARLEN) {
        int64_t r0;
        if (!varlen_chunk(p, c, T, r0)) {
            if (p.error_word && tid == 0) atomicOr(p.error_word, (uint32_t)KAMERA_EW_CHUNK);
            return;  // uniform
        }
        row0 = r0 + (int64_t)l * T;
        sofs = row0 * F;
        ntiles = (T + kTileTokens - 1) / kTileTokens;
        if (tile_begin >= ntiles) return;  // past the chunk's rows (uniform)
    }
    const uint16_t* __restrict__ U = p.u[s] + row0 * p.rank;
    const uint16_t* __restrict__ V = p.v[s] + blk * F * p.rank;
    const uint16_t* __restrict__ src = p.src[s] + sofs;
    uint16_t* __restrict__ dst = p.dst[s] + (int64_t)l * p.dst_layer_stride;

    const int tile_end = min(ntiles, tile_begin + tiles_per_wg);
    const int tok0 = tile_begin * kTileTokens;
    const int ntok = min(T, tile_end * kTileTokens) - tok0;

    // Pool slots of the group's tokens: the page ids (or the chunk's offset)
    // are loaded before anything else, with clamped indices, and turned into
    // slots only after the first tile's loads are issued.
    // Wave 0 alone resolves them: a group has at most 64 * kSlotLoads tokens.
    constexpr int kSlotLoads = (kTileTokens * kMaxTilesPerGroup + 63) / 64;
    const bool paged = p.page_size > 0;
    int32_t page_raw[kSlotLoads];
    if (wave == 0) {
#pragma unroll
        for (int k = 0; k < kSlotLoads; ++k) {
            const int t = tok0 + min(lane + 64 * k, ntok - 1);
            page_raw[k] = *(paged ? p.page_table + (int64_t)i * p.pages_per_chunk + page_of(p, t)
                                  : reinterpret_cast<const int32_t*>(&kZeroWord));
        }
    }
    const int64_t off_raw = ld_uniform(paged ? &kZeroWord : p.dst_offset + i);

    // the shift's inputs next (small loads ahead of the big ones)
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

    constexpr int chunks_per_row = 8 * W;

    // Every global load of a tile -- its canonical rows (coalesced: chunk
    // q = tid + k*64W -> row, 16-byte column) and this thread's U chunks -- goes
    // into a TileBuf and is issued one tile ahead, so it is in flight while the
    // current tile is computed and stored.
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
        u32x4 u[kUPerThread];
    };
    auto load_tile = [&](TileBuf& tb_, int t0) {
        // rows past the chunk's end re-read its last row (never stored)
        const int last = T - 1 - t0;
        const uint16_t* __restrict__ ub = U + (int64_t)t0 * p.rank;     // uniform
#pragma unroll
        for (int j = 0; j < kUPerThread; ++j) {
            // chunk q: token q / 2KS, ranks 8 * (q % 2KS) .. + 8 (padding chunks
            // past the rank re-read an in-range slice and are zeroed at use)
            const int q = min(tid + j * nthreads, kUChunks - 1);
            const int ut = q / (2 * KS);
            const int k0 = min(8 * (q - ut * 2 * KS), p.rank - 8);
            tb_.u[j] = ld_cached(ub + (uint32_t)(min(ut, last) * p.rank + k0));
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
#pragma unroll
        for (int j = 0; j < kUPerThread; ++j) {
            const int q = tid + j * nthreads;
            if (q < kUChunks) *reinterpret_cast<u32x4*>(tile_lds + kUOffset + 16 * q) = buf.u[j];
        }
        if (reload_tile < tile_end) load_tile(buf, reload_tile * kTileTokens);
        __syncthreads();

        bf16x8 bop[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 zero = {0u, 0u, 0u, 0u};
            const u32x4 w = *reinterpret_cast<const u32x4*>(tile_lds + kUOffset + 16 * (col * 2 * KS + 2 * ks + hh));
            bop[ks] = __builtin_bit_cast(bf16x8, 16 * ks + 8 * hh < p.rank ? w : zero);
        }

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
            if (t0 + grow[k] >= T) continue;
            const int64_t slot = slot_lds[t0 - tile_begin * kTileTokens + grow[k]];
            if (slot < 0) continue;
            const u32x4 w = *reinterpret_cast<const u32x4*>(tile_lds + loff[k]);
            st_stream(dst + slot * F + fw0 + (goff[k] - grow[k] * F), w);
        }
        // the next tile's LDS writes must wait until every thread has read this one
        __syncthreads();
    };

    TileBuf bufA;
    load_tile(bufA, tile_begin * kTileTokens);

    // slots of the group's tokens, bounds-checked (out of range: row skipped)
    if (wave == 0) {
#pragma unroll
        for (int k = 0; k < kSlotLoads; ++k) {
            const int r = lane + 64 * k;
            if (r < ntok) slot_lds[r] = slot_from(p, tok0 + r, page_raw[k], off_raw, T, err);
        }
    }

    if (rot && lane < 32) {
        int64_t delta;
        if (p.mode == MODE_DELTA) {
            delta = delta_in;
        } else {
            delta = (p.mode == MODE_REORDER) ? p.base_pos + (int64_t)i * p.T - pc_in : target_in - pc_in;
        }
        cs_lds[wave][lane] = rope_phase(p, sg.j0 + lane, delta);
    }
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 zero = {0u, 0u, 0u, 0u};
            aop[bb][ks] = __builtin_bit_cast(bf16x8, 16 * ks + 8 * hh < p.rank ? aop_raw[bb][ks] : zero);
        }

    for (int tile = tile_begin; tile < tile_end; ++tile) process_tile(bufA, tile, tile + 1);
    if (err && p.error_word) atomicOr(p.error_word, err);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

struct Tuning {
    int row_unroll = 0;          // relocate_rows_kernel: 16-byte vectors per thread (1, 2; 0 = by size)
    int tiles_per_group = 0;     // relocate_patch_lds_kernel: token tiles per workgroup (0 = by shape)
    int window_waves = 0;        // LDS kernel: cap on waves per workgroup (0 = widest window)
    int page_order = 1;          // paged pools: destination order when the call gives scratch (0 = off)
    int partner_lanes = 1;       // m = 0 kernel: rotate-half partners by cross-lane moves (0 = load them)
};

Tuning g_tuning;
std::once_flag g_tuning_once;

void load_tuning() {
    // Optional overrides of the shape-based picks, for measurements:
    // KAMERA_ROW_UNROLL (1 or 2), KAMERA_TILES_PER_GROUP (32-token tiles per
    // workgroup), KAMERA_WINDOW_WAVES.
    if (const char* e = getenv("KAMERA_ROW_UNROLL")) {
        int v = atoi(e);
        if (v == 1 || v == 2) g_tuning.row_unroll = v;
    }
    if (const char* e = getenv("KAMERA_WINDOW_WAVES")) g_tuning.window_waves = atoi(e);
    if (const char* e = getenv("KAMERA_PAGE_ORDER")) g_tuning.page_order = atoi(e) != 0;
    if (const char* e = getenv("KAMERA_PARTNER_LANES")) g_tuning.partner_lanes = atoi(e) != 0;
    if (const char* e = getenv("KAMERA_TILES_PER_GROUP")) {
        int v = atoi(e);
        if (v >= 1 && v <= 1024) g_tuning.tiles_per_group = v;
    }
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
    if (L->num_layers < 1 || L->num_layers > kMaxGridZ || L->num_heads < 1 || L->head_dim < 1)
        return KAMERA_ERR_RANGE;
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
    int32_t* check_scratch = nullptr;  // content checks on (error word and scratch given)
    int64_t check_entries = 0;         // page-table entries at the head of the scratch
};

// Everything the host can check, before any HIP call.
kamera_status prepare(const kamera_layout* layout, const kamera_src* src, const kamera_varlen* vl, int32_t n,
                      const kamera_patch* patch, const kamera_dst* dst, int mode, Call& call, bool& empty) {
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
    if (!vl && (src->chunk_stride < 0 || src->layer_stride < 0)) return KAMERA_ERR_RANGE;
    if (dst->layer_stride < 0) return KAMERA_ERR_RANGE;
    if (dst->num_slots < 0 || dst->page_size < 0) return KAMERA_ERR_RANGE;
    if (vl) {
        // variable-length chunks: per-chunk lengths and first rows on the device
        if (mode == MODE_REORDER) return KAMERA_ERR_UNSUPPORTED;
        if (!vl->row_offset || !vl->n_tokens) return KAMERA_ERR_NULL;
        if (((uintptr_t)vl->row_offset & 7u) != 0 || ((uintptr_t)vl->n_tokens & 3u) != 0) return KAMERA_ERR_ALIGN;
        if (vl->total_rows < 0 || vl->total_rows > ((int64_t)1 << 40)) return KAMERA_ERR_RANGE;
    }
    for (int s = 0; s < S; ++s) {
        if (!src->rows[s] || !dst->rows[s]) return KAMERA_ERR_NULL;
        if (!aligned16(src->rows[s]) || !aligned16(dst->rows[s])) return KAMERA_ERR_ALIGN;
        if (m > 0) {
            if (!patch->u[s] || !patch->v[s]) return KAMERA_ERR_NULL;
            if (!aligned16(patch->u[s]) || !aligned16(patch->v[s])) return KAMERA_ERR_ALIGN;
        }
    }
    if ((!vl && (src->chunk_stride % 8 || src->layer_stride % 8)) || dst->layer_stride % 8) return KAMERA_ERR_ALIGN;
    if (dst->page_size > 0 && !dst->page_table && n > 0) return KAMERA_ERR_NULL;
    if (dst->page_size == 0 && !dst->dst_offset && n > 0) return KAMERA_ERR_NULL;

    empty = (n == 0 || T == 0);
    if (empty) return KAMERA_OK;

    // shapes: a chunk's rows must fit its strides, and the pool's layers must not overlap
    if (!vl && L.num_layers > 1 && src->layer_stride < (int64_t)T * F) return KAMERA_ERR_SHAPE;
    if (!vl && src->n_store > 1 && src->chunk_stride < (int64_t)T * F) return KAMERA_ERR_SHAPE;
    if (L.num_layers > 1 && dst->layer_stride < dst->num_slots * F) return KAMERA_ERR_SHAPE;
    // (variable lengths: chunks shorter than T may fit a smaller pool; the
    // kernels check every chunk's slots)
    if (!vl && dst->num_slots < T) return KAMERA_ERR_RANGE;
    if (dst->page_size > 0 && dst->num_slots / dst->page_size < 1) return KAMERA_ERR_RANGE;
    if ((int64_t)n * L.num_layers * S * ((T + 31) / 32) > (int64_t)1 << 40) return KAMERA_ERR_RANGE;

    // the destination must not overlap any input
    const int64_t src_elems =
        vl ? vl->total_rows * F
           : (int64_t)(src->n_store - 1) * src->chunk_stride + (int64_t)(L.num_layers - 1) * src->layer_stride +
                 (int64_t)T * F;
    const int64_t dst_elems = (int64_t)(L.num_layers - 1) * dst->layer_stride + dst->num_slots * F;
    const int64_t u_elems = vl ? vl->total_rows * m : (int64_t)src->n_store * L.num_layers * T * m;
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

    // destination-order scratch: [n * pages per chunk] int32, disjoint from every
    // other argument (variable-length calls keep the page-table order and
    // ignore it)
    if (!vl && dst->page_size > 0 && dst->page_order) {
        if (((uintptr_t)dst->page_order & 3u) != 0) return KAMERA_ERR_ALIGN;
        const int64_t entries = (int64_t)n * ((T + dst->page_size - 1) / dst->page_size);
        const Span o{(uintptr_t)dst->page_order, (uintptr_t)dst->page_order + (uintptr_t)entries * 4u};
        if (overlap(o, Span{(uintptr_t)dst->page_table, (uintptr_t)dst->page_table + (uintptr_t)entries * 4u}))
            return KAMERA_ERR_ALIAS;
        for (int s = 0; s < S; ++s) {
            if (overlap(o, span_of(dst->rows[s], dst_elems)) || overlap(o, span_of(src->rows[s], src_elems)))
                return KAMERA_ERR_ALIAS;
            if (m > 0 && (overlap(o, span_of(patch->u[s], u_elems)) || overlap(o, span_of(patch->v[s], v_elems))))
                return KAMERA_ERR_ALIAS;
        }
    }

    // content-check scratch: [n * pages per chunk + n] int32 (paged) or [n]
    // (contiguous), used only with an error word; disjoint from every other
    // argument
    call.check_scratch = nullptr;
    if (dst->error_word && dst->check_scratch) {
        if (((uintptr_t)dst->check_scratch & 3u) != 0) return KAMERA_ERR_ALIGN;
        const int64_t ppc = dst->page_size > 0 ? (T + dst->page_size - 1) / dst->page_size : 0;
        const int64_t entries = (int64_t)n * ppc;
        if (entries + n > INT32_MAX / 2) return KAMERA_ERR_RANGE;
        const Span c{(uintptr_t)dst->check_scratch, (uintptr_t)dst->check_scratch + (uintptr_t)(entries + n) * 4u};
        if (dst->page_table &&
            overlap(c, Span{(uintptr_t)dst->page_table, (uintptr_t)dst->page_table + (uintptr_t)entries * 4u}))
            return KAMERA_ERR_ALIAS;
        if (dst->page_order && dst->page_size > 0 &&
            overlap(c, Span{(uintptr_t)dst->page_order, (uintptr_t)dst->page_order + (uintptr_t)entries * 4u}))
            return KAMERA_ERR_ALIAS;
        for (int s = 0; s < S; ++s) {
            if (overlap(c, span_of(dst->rows[s], dst_elems)) || overlap(c, span_of(src->rows[s], src_elems)))
                return KAMERA_ERR_ALIAS;
            if (m > 0 && (overlap(c, span_of(patch->u[s], u_elems)) || overlap(c, span_of(patch->v[s], v_elems))))
                return KAMERA_ERR_ALIAS;
        }
        call.check_scratch = dst->check_scratch;
        call.check_entries = entries;
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
    p.num_pages = dst->page_size > 0 ? dst->num_slots / dst->page_size : 0;
    p.page_table = dst->page_table;
    p.dst_offset = dst->dst_offset;
    p.error_word = dst->error_word;
    p.page_order = (dst->page_size > 0 && !vl) ? dst->page_order : nullptr;
    if (vl) {
        p.vl_row_offset = vl->row_offset;
        p.vl_tokens = vl->n_tokens;
        p.vl_total_rows = vl->total_rows;
    }
    p.log2_base = log2(L.rope_base);
    p.mode = mode;
    p.rank = m;
    p.page_size = dst->page_size;
    p.pages_per_chunk = dst->page_size > 0 ? (T + dst->page_size - 1) / dst->page_size : 0;
    p.page_div = make_fastdiv(dst->page_size > 0 ? (uint32_t)dst->page_size : 1u);
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
    // Rotate-half partners R/2 = 8d elements apart sit d lanes apart (xor) in
    // the m = 0 kernel when pairs never straddle a 2d-vector group: every
    // block starts on a multiple of 256 vectors, so lane and vector index agree
    // modulo 2d when 2d divides 256, the row (F/8), the head (D/8) and the span
    // offset (rope_offset/8).
    {
        const int d = L.rope_dim / 16;
        const bool fits = L.rope_style == KAMERA_ROPE_HALF && L.rope_dim > 0 && (d & (d - 1)) == 0 && d >= 4 &&
                          2 * d <= 64 && (L.head_dim / 8) % (2 * d) == 0 && (L.rope_offset / 8) % (2 * d) == 0 &&
                          (F / 8) % (2 * d) == 0;
        p.partner_lanes = fits ? d : 0;
    }
    call.patched = m > 0;
    return KAMERA_OK;
}


// Destination order applies to paged pools whose call brought scratch for it.
bool use_page_order(Params& p) {
    if (p.page_size <= 0 || !p.page_order || !g_tuning.page_order) return false;
    const int64_t entries = (int64_t)p.n * p.pages_per_chunk;
    if (entries < 1 || entries > INT32_MAX / 2) return false;
    p.entries = (int32_t)entries;
    p.ppc_div = make_fastdiv((uint32_t)p.pages_per_chunk);
    return true;
}

// Sorts the call's page-table entries into p.page_order (runs of kSortRun).
hipError_t sort_page_order(const Params& p, hipStream_t hs) {
    const int runs = (p.entries + kSortRun - 1) / kSortRun;
    return launch_kernel(sort_pages_kernel, dim3((unsigned)runs), dim3(kSortThreads), hs, p.page_table,
                         const_cast<int32_t*>(p.page_order), p.entries);
}

kamera_status launch(const kamera_layout* layout, Call& call, void* stream) {
    std::call_once(g_tuning_once, load_tuning);
    Params& p = call.p;
    hipStream_t hs = (hipStream_t)stream;
    hipError_t e;
    if (!call.patched) {
        // vectors per thread: 1 streams best on large calls, 2 on small ones
        // (measured on MI355X: 6.0 vs 5.7 TB/s on 9.7 GB, 23.3 vs 21.2 us on
        // 120 MB)
        // (variable lengths: the grid is sized by the longest chunk, and the
        // blocks past a shorter chunk's end exit at once; two vectors per
        // thread halve those blocks: 4.05 -> 3.25 ms on 64 chunks of
        // 256..1792 tokens, measured on MI355X)
        const bool vlen = p.vl_tokens != nullptr;
        const int64_t nvec = (int64_t)p.T * (p.F >> 3);
        if (nvec > INT32_MAX / 2) return KAMERA_ERR_RANGE;
        // destination order needs every block inside one page: one vector per
        // thread when two would straddle a page
        const int64_t page_elems = (int64_t)p.page_size * p.F;
        const bool by_page = page_elems % (8 * kThreads) == 0 && use_page_order(p);
        // (in page order two vectors per thread measured ~1% faster on the
        // 9.7 GB sliding-window shape: 5.56 vs 5.50-5.52 TB/s)
        int u = g_tuning.row_unroll > 0
                    ? g_tuning.row_unroll
                    : ((!vlen && !by_page && (int64_t)p.n * p.S * p.L * nvec >= kRowUnrollOneVectors) ? 1 : 2);
        if (by_page && page_elems % (8 * kThreads * u) != 0) u = 1;
        const int per_slice = (int)((nvec + (int64_t)kThreads * u - 1) / ((int64_t)kThreads * u));
        const FastDiv dvr = make_fastdiv((uint32_t)(p.F >> 3));
        const FastDiv dhd = make_fastdiv((uint32_t)(p.D >> 3));
        const FastDiv dupr = make_fastdiv((uint32_t)(p.F >> 4));  // pair units per row
        const FastDiv duph = make_fastdiv((uint32_t)(p.D >> 4));  // pair units per head
        if (!g_tuning.partner_lanes) p.partner_lanes = 0;
        if (by_page) {
            auto* fn = u == 1 ? relocate_rows_kernel<1, true, false> : relocate_rows_kernel<2, true, false>;
            const int64_t bpp = page_elems / (8 * kThreads * u);
            if ((int64_t)p.entries * bpp > INT32_MAX) return KAMERA_ERR_RANGE;
            p.unit_div = make_fastdiv((uint32_t)bpp);
            e = sort_page_order(p, hs);
            if (e == hipSuccess) {
                const dim3 grid((unsigned)(p.entries * bpp), (unsigned)p.S, (unsigned)p.L);
                e = launch_kernel(fn, grid, dim3(kThreads), hs, p, 0, dvr, dhd, dupr, duph);
            }
            return e == hipSuccess ? KAMERA_OK : KAMERA_ERR_HIP;
        }
        auto* fn = vlen ? (u == 1 ? relocate_rows_kernel<1, false, true> : relocate_rows_kernel<2, false, true>)
                        : (u == 1 ? relocate_rows_kernel<1, false, false> : relocate_rows_kernel<2, false, false>);
        e = hipSuccess;
        for (int zb = 0; zb < p.n * p.S && e == hipSuccess; zb += kMaxGridZ) {
            const dim3 grid((unsigned)per_slice, (unsigned)p.L, (unsigned)std::min(kMaxGridZ, p.n * p.S - zb));
            e = launch_kernel(fn, grid, dim3(kThreads), hs, p, zb, dvr, dhd, dupr, duph);
        }
    } else {
        SegmentTable st;
        memset(&st, 0, sizeof(st));
        if (build_segments(*layout, st) <= 0) return KAMERA_ERR_UNSUPPORTED;
        const int ks = (p.rank + 15) / 16;
        const int tiles_total = (p.T + 31) / 32;
        int W = window_waves(st);
        if (g_tuning.window_waves > 0 && g_tuning.window_waves < W && W % g_tuning.window_waves == 0)
            W = g_tuning.window_waves;
        const int windows = st.count / W;
        // token tiles per workgroup: enough for about 16 KB of rows (one
        // 32 x 256 tile at W = 4; measured best on MI355X)
        // (variable lengths: two tiles per workgroup halve the groups past a
        // shorter chunk's end; +1% on 32 chunks of 256..3840 tokens)
        int tpg = g_tuning.tiles_per_group > 0 ? g_tuning.tiles_per_group
                                               : (p.vl_tokens ? std::max(2, (4 + W - 1) / W) : (4 + W - 1) / W);
        tpg = std::min(std::min(tpg, kMaxTilesPerGroup), tiles_total);
        const int groups = (tiles_total + tpg - 1) / tpg;
        const FastDiv dgroups = make_fastdiv((uint32_t)groups);
        using LdsKernel = void (*)(Params, SegmentTable, int, int, int, FastDiv);
#define KAMERA_LDS_ROW(KS, BP, VL)                                                                        \
    {relocate_patch_lds_kernel<KS, 1, BP, VL>, relocate_patch_lds_kernel<KS, 2, BP, VL>,                   \
     relocate_patch_lds_kernel<KS, 3, BP, VL>, relocate_patch_lds_kernel<KS, 4, BP, VL>}
        // [page-table order, destination order, variable lengths][k-steps][waves]
        static const LdsKernel kLds[3][4][kMaxWindowWaves] = {
            {KAMERA_LDS_ROW(1, false, false), KAMERA_LDS_ROW(2, false, false), KAMERA_LDS_ROW(3, false, false),
             KAMERA_LDS_ROW(4, false, false)},
            {KAMERA_LDS_ROW(1, true, false), KAMERA_LDS_ROW(2, true, false), KAMERA_LDS_ROW(3, true, false),
             KAMERA_LDS_ROW(4, true, false)},
            {KAMERA_LDS_ROW(1, false, true), KAMERA_LDS_ROW(2, false, true), KAMERA_LDS_ROW(3, false, true),
             KAMERA_LDS_ROW(4, false, true)}};
#undef KAMERA_LDS_ROW
        // destination order: a page holds a whole number of token groups; the
        // windows of a group then run in consecutive blocks, so that every
        // page is written out completely before the next (measured on MI355X:
        // MLA 5.47 -> 5.72 TB/s with both, no gain from either alone; groups
        // spanning two 16-token pages keyed by their first page measured 3%
        // slower than the page-table order, so smaller pages keep that order)
        if (p.page_size % (kTileTokens * tpg) == 0 && use_page_order(p)) {
            const int gpu = p.page_size / (kTileTokens * tpg);  // token groups per page
            const int64_t all_groups = (int64_t)p.entries * gpu;
            const int64_t runs = (all_groups + 7) / 8;             // of 8 groups, one per XCD
            if (runs * 8 * windows > INT32_MAX / 2) return KAMERA_ERR_RANGE;
            p.unit_div = make_fastdiv((uint32_t)gpu);
            e = sort_page_order(p, hs);
            if (e == hipSuccess) {
                const dim3 grid((unsigned)(runs * 8 * windows), (unsigned)p.L, (unsigned)p.S);
                e = launch_kernel(kLds[1][ks - 1][W - 1], grid, dim3(64 * W), hs, p, st, 0, tiles_total, tpg,
                                  make_fastdiv((uint32_t)(8 * windows)));
            }
            return e == hipSuccess ? KAMERA_OK : KAMERA_ERR_HIP;
        }
        e = hipSuccess;
        for (int zb = 0; zb < p.n * p.S && e == hipSuccess; zb += kMaxGridZ) {
            const dim3 grid((unsigned)(windows * groups), (unsigned)p.L,
                            (unsigned)std::min(kMaxGridZ, p.n * p.S - zb));
            e = launch_kernel(kLds[p.vl_tokens ? 2 : 0][ks - 1][W - 1], grid, dim3(64 * W), hs, p, st, zb,
                              tiles_total, tpg, dgroups);
        }
    }
    return e == hipSuccess ? KAMERA_OK : KAMERA_ERR_HIP;
}

// Content checks (kamera_dst.check_scratch): copies of the page table and of
// the chunk entries with every repeat of an earlier entry replaced by the skip
// marker; the call then reads the copies.  Variable-length calls check their
// chunk entries only (their page-table rows are ragged: entries past a chunk's
// own pages are never read and may hold anything).
hipError_t run_content_checks(Call& call, bool check_pages, hipStream_t hs) {
    Params& p = call.p;
    int32_t* scratch = call.check_scratch;
    hipError_t e = hipSuccess;
    const int64_t entries = call.check_entries;
    if (check_pages && p.page_size > 0 && entries > 0) {
        const int runs = (int)((entries + kSortRun - 1) / kSortRun);
        const int bound = (int)std::min<int64_t>(p.num_pages, INT32_MAX);
        e = launch_kernel(dedup_kernel, dim3((unsigned)runs), dim3(kSortThreads), hs, p.page_table, scratch,
                          (int)entries, bound, p.error_word, (uint32_t)KAMERA_EW_DUP_PAGE);
        p.page_table = scratch;
    }
    if (e == hipSuccess && p.mode != MODE_DELTA) {
        const int runs = (p.n + kSortRun - 1) / kSortRun;
        e = launch_kernel(dedup_kernel, dim3((unsigned)runs), dim3(kSortThreads), hs, p.ids, scratch + entries, p.n,
                          p.n_store, p.error_word, (uint32_t)KAMERA_EW_DUP_CHUNK);
        p.ids = scratch + entries;
    }
    return e;
}

kamera_status run(const kamera_layout* layout, const kamera_src* src, const kamera_varlen* vl, int32_t n,
                  const kamera_patch* patch, const kamera_dst* dst, int mode, const int64_t* delta,
                  const int32_t* ids, const int64_t* target, int64_t base_pos, void* stream) {
    Call call;
    bool empty = false;
    kamera_status st = prepare(layout, src, vl, n, patch, dst, mode, call, empty);
    if (st != KAMERA_OK || empty) return st;
    if (mode == MODE_DELTA && !delta) return KAMERA_ERR_NULL;
    if (mode != MODE_DELTA && !ids) return KAMERA_ERR_NULL;
    if (mode == MODE_RECALL && !target) return KAMERA_ERR_NULL;
    if (call.check_scratch && mode != MODE_DELTA) {
        const Span c{(uintptr_t)call.check_scratch, (uintptr_t)(call.check_scratch + call.check_entries + n)};
        if (overlap(c, Span{(uintptr_t)ids, (uintptr_t)(ids + n)})) return KAMERA_ERR_ALIAS;
    }
    call.p.delta = delta;
    call.p.ids = ids;
    call.p.target = target;
    call.p.base_pos = base_pos;
    if (call.check_scratch && run_content_checks(call, vl == nullptr, (hipStream_t)stream) != hipSuccess)
        return KAMERA_ERR_HIP;
    return launch(layout, call, stream);
}

// ---------------------------------------------------------------------------
// Scratch for the allocation-free entry point
// ---------------------------------------------------------------------------

// kamera_relocate_patch_noalloc keeps the page-order scratch and the
// content-check scratch of a call in this array instead of caller memory.
// Each device the library runs on holds its own copy until the process ends;
// host code never uses the array's name as an address: the device address is
// resolved once per device (hipGetSymbolAddress) and kept.
constexpr int64_t kStaticScratchInts = (int64_t)1 << 18;  // 1 MiB
__device__ __align__(256) int32_t scratch[kStaticScratchInts];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
int32_t* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the current device (nullptr on failure).
int32_t* static_scratch(kamera_status& st) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        st = KAMERA_ERR_HIP;
        return nullptr;
    }
    std::call_once(g_scratch_once[dev], [dev] {
        void* ptr = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? (int32_t*)ptr : nullptr;
    });
    if (!g_scratch_ptr[dev]) {
        st = KAMERA_ERR_HIP;
        return nullptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

kamera_status kamera_relocate(const kamera_layout* layout, const kamera_src* src, int32_t n, const int64_t* delta,
                              const kamera_dst* dst, void* hip_stream) {
    return run(layout, src, nullptr, n, nullptr, dst, MODE_DELTA, delta, nullptr, nullptr, 0, hip_stream);
}

kamera_status kamera_relocate_patch(const kamera_layout* layout, const kamera_src* src, int32_t n,
                                    const int64_t* delta, const kamera_patch* patch, const kamera_dst* dst,
                                    void* hip_stream) {
    if (!patch) return KAMERA_ERR_NULL;
    return run(layout, src, nullptr, n, patch, dst, MODE_DELTA, delta, nullptr, nullptr, 0, hip_stream);
}

kamera_status kamera_relocate_patch_noalloc(const kamera_layout* layout, const kamera_src* src, int32_t n,
                                            const int64_t* delta, const kamera_patch* patch, const kamera_dst* dst,
                                            void* hip_stream) {
    if (!patch || !src || !dst) return KAMERA_ERR_NULL;
    if (n < 0 || src->n_tokens < 0 || dst->page_size < 0) return KAMERA_ERR_RANGE;
    // what the call would keep in caller scratch: the page order (paged
    // pools) and, with an error word, the content checks' copies
    const int64_t ppc = dst->page_size > 0 ? ((int64_t)src->n_tokens + dst->page_size - 1) / dst->page_size : 0;
    const int64_t entries = (int64_t)n * ppc;
    const int64_t need = entries + (dst->error_word ? entries + n : 0);
    if (need > kStaticScratchInts) return KAMERA_ERR_RANGE;
    kamera_dst d = *dst;
    d.page_order = nullptr;
    d.check_scratch = nullptr;
    if (need > 0 && n > 0 && src->n_tokens > 0) {
        kamera_status st = KAMERA_OK;
        int32_t* ptr = static_scratch(st);
        if (!ptr) return st;
        if (dst->page_size > 0) d.page_order = ptr;
        if (dst->error_word) d.check_scratch = ptr + entries;
    }
    return run(layout, src, nullptr, n, patch, &d, MODE_DELTA, delta, nullptr, nullptr, 0, hip_stream);
}

kamera_status kamera_reorder(const kamera_layout* layout, const kamera_src* src, int32_t n, const int32_t* perm,
                             int64_t base_pos, const kamera_patch* orbit, const kamera_dst* dst, void* hip_stream) {
    return run(layout, src, nullptr, n, orbit, dst, MODE_REORDER, nullptr, perm, nullptr, base_pos, hip_stream);
}

kamera_status kamera_recall(const kamera_layout* layout, const kamera_src* src, int32_t n, const int32_t* chunk_ids,
                            const int64_t* target_pos, const kamera_patch* patch, const kamera_dst* dst,
                            void* hip_stream) {
    return run(layout, src, nullptr, n, patch, dst, MODE_RECALL, nullptr, chunk_ids, target_pos, 0, hip_stream);
}

kamera_status kamera_relocate_patch_varlen(const kamera_layout* layout, const kamera_src* src,
                                           const kamera_varlen* varlen, int32_t n, const int64_t* delta,
                                           const kamera_patch* patch, const kamera_dst* dst, void* hip_stream) {
    if (!varlen) return KAMERA_ERR_NULL;
    return run(layout, src, varlen, n, patch, dst, MODE_DELTA, delta, nullptr, nullptr, 0, hip_stream);
}

kamera_status kamera_recall_varlen(const kamera_layout* layout, const kamera_src* src, const kamera_varlen* varlen,
                                   int32_t n, const int32_t* chunk_ids, const int64_t* target_pos,
                                   const kamera_patch* patch, const kamera_dst* dst, void* hip_stream) {
    if (!varlen) return KAMERA_ERR_NULL;
    return run(layout, src, varlen, n, patch, dst, MODE_RECALL, nullptr, chunk_ids, target_pos, 0, hip_stream);
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

int32_t kamera_version(void) { return 200; }

}  // extern "C"
