// kamera_host.cpp — relocation from a canonical store in pinned host memory
// (include/kamera.h, kamera_relocate_patch_host).
//
// Kamera summary, section 3, "Three cheap window operations", Recall: evicted
// chunks come back from the canonical store with a fresh patch, without
// re-encoding.  Here the store lives in host memory, so the rows must cross
// the host link first.  The call pipelines that crossing with the relocation:
//
//   copy stream:    [copy chunk 0 -> slot 0][copy 1 -> slot 1][wait done 0][copy 2 -> slot 0] ...
//   compute stream:            [wait][relocate slot 0][wait][relocate slot 1][wait] ...
//
// Each chunk's rows (every layer and stream) go into one slot of the
// caller's device staging buffer with one strided 2-D copy per stream; an
// event tells the compute stream the slot is filled, and the relocation of
// that slot (kamera_relocate_patch on a one-chunk store) records another event
// that frees the slot for the chunk `slots` places later.  With two or more
// slots the copies run back to back and the relocations hide behind them:
// the call is bound by the host link.

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "kamera.h"

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Span {
    uintptr_t lo, hi;
};
inline bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

int64_t slot_bytes(const kamera_layout& L, int T) {
    const int64_t b = (int64_t)L.num_streams * L.num_layers * T * L.num_heads * L.head_dim * 2;
    return (b + 255) & ~(int64_t)255;
}

// Pinned (page-locked) host memory that the device can copy from directly.
bool is_pinned_host(const void* p) {
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();  // pageable memory reports an error: clear it
        return false;
    }
    return a.type == hipMemoryTypeHost;
}

}  // namespace

extern "C" {

int64_t kamera_host_staging_bytes(const kamera_layout* layout, int32_t n_tokens, int32_t slots) {
    if (!layout || n_tokens < 0 || slots < 1 || layout->num_streams < 1 || layout->num_streams > 2 ||
        layout->num_layers < 1 || layout->num_heads < 1 || layout->head_dim < 1)
        return -1;
    return slot_bytes(*layout, n_tokens) * slots;
}

}  // extern "C"

namespace {

// Both host-store calls.  vl == nullptr: a fixed-length store (strides, one
// T); otherwise a packed store whose chunk lengths and first rows are the
// HOST arrays vl->n_tokens / vl->row_offset, and whose output factors are
// packed in output order.
kamera_status relocate_host(const kamera_layout* layout, const kamera_src* host_src, const kamera_varlen* vl,
                            int32_t n, const int32_t* chunk_ids, const int64_t* delta, const kamera_patch* patch,
                            const kamera_dst* dst, void* staging, int64_t staging_bytes, void* copy_stream,
                            void* compute_stream) {
    if (!layout || !host_src || !dst) return KAMERA_ERR_NULL;
    const kamera_layout& L = *layout;
    if (L.num_streams < 1 || L.num_streams > 2 || L.num_layers < 1 || L.num_heads < 1 || L.head_dim < 1)
        return KAMERA_ERR_RANGE;
    const int S = L.num_streams;
    const int T = host_src->n_tokens;  // T_max for a packed store
    const int64_t F = (int64_t)L.num_heads * L.head_dim;
    if (n < 0 || T < 0 || host_src->n_store < 1) return KAMERA_ERR_RANGE;
    if (host_src->canon_pos) return KAMERA_ERR_UNSUPPORTED;  // shifts come in `delta`
    const int m = patch ? patch->rank : 0;
    if (m < 0 || m > 64) return KAMERA_ERR_RANGE;
    if (n == 0 || T == 0) return KAMERA_OK;
    if (!chunk_ids || !delta) return KAMERA_ERR_NULL;
    if (vl) {
        if (!vl->row_offset || !vl->n_tokens) return KAMERA_ERR_NULL;
        if (vl->total_rows < 0) return KAMERA_ERR_RANGE;
    } else {
        if (host_src->chunk_stride < 0 || host_src->layer_stride < 0) return KAMERA_ERR_RANGE;
        if (L.num_layers > 1 && host_src->layer_stride < (int64_t)T * F) return KAMERA_ERR_SHAPE;
        if (host_src->n_store > 1 && host_src->chunk_stride < (int64_t)T * F) return KAMERA_ERR_SHAPE;
    }
    for (int s = 0; s < S; ++s) {
        if (!host_src->rows[s]) return KAMERA_ERR_NULL;
        if (!aligned16(host_src->rows[s])) return KAMERA_ERR_ALIGN;
    }
    for (int s = 0; s < S; ++s)
        if (!is_pinned_host(host_src->rows[s])) return KAMERA_ERR_UNSUPPORTED;
    for (int i = 0; i < n; ++i)
        if (chunk_ids[i] < 0 || chunk_ids[i] >= host_src->n_store) return KAMERA_ERR_RANGE;
    // a packed store's lengths and rows are host data: all checked here
    int64_t out_rows = 0;  // rows of every output chunk (the packed factors' length)
    for (int i = 0; i < n; ++i) {
        const int c = chunk_ids[i];
        if (vl) {
            const int tc = vl->n_tokens[c];
            const int64_t r0 = vl->row_offset[c];
            if (tc < 0 || tc > T || r0 < 0 || r0 > vl->total_rows - (int64_t)L.num_layers * tc)
                return KAMERA_ERR_RANGE;
            out_rows += (int64_t)L.num_layers * tc;
        } else {
            out_rows += (int64_t)L.num_layers * T;
        }
    }
    const int64_t sb = slot_bytes(L, T);
    if (!staging) return KAMERA_ERR_NULL;
    if (((uintptr_t)staging & 255u) != 0) return KAMERA_ERR_ALIGN;
    if (staging_bytes < sb) return KAMERA_ERR_RANGE;
    const int slots = (int)(staging_bytes / sb < n ? staging_bytes / sb : n);
    // the staging buffer must not overlap the pool, the factors or the index data
    {
        const Span st{(uintptr_t)staging, (uintptr_t)staging + (uintptr_t)(sb * slots)};
        const int64_t dst_el = (int64_t)(L.num_layers - 1) * dst->layer_stride + dst->num_slots * F;
        for (int s = 0; s < S; ++s) {
            if (dst->rows[s] && overlap(st, Span{(uintptr_t)dst->rows[s], (uintptr_t)dst->rows[s] + (uintptr_t)dst_el * 2}))
                return KAMERA_ERR_ALIAS;
            if (m > 0 && patch->u[s] &&
                overlap(st, Span{(uintptr_t)patch->u[s], (uintptr_t)patch->u[s] + (uintptr_t)(out_rows * m * 2)}))
                return KAMERA_ERR_ALIAS;
            if (m > 0 && patch->v[s] &&
                overlap(st, Span{(uintptr_t)patch->v[s], (uintptr_t)patch->v[s] + (uintptr_t)((int64_t)n * L.num_layers * F * m * 2)}))
                return KAMERA_ERR_ALIAS;
        }
        if (overlap(st, Span{(uintptr_t)delta, (uintptr_t)delta + (uintptr_t)n * 8u})) return KAMERA_ERR_ALIAS;
        const int ppc = dst->page_size > 0 ? (T + dst->page_size - 1) / dst->page_size : 0;
        if (dst->page_table && overlap(st, Span{(uintptr_t)dst->page_table, (uintptr_t)dst->page_table + (uintptr_t)((int64_t)n * ppc * 4)}))
            return KAMERA_ERR_ALIAS;
        if (dst->dst_offset && overlap(st, Span{(uintptr_t)dst->dst_offset, (uintptr_t)dst->dst_offset + (uintptr_t)n * 8u}))
            return KAMERA_ERR_ALIAS;
    }

    // per-chunk arguments: the staging slot as a one-chunk store of the
    // chunk's own length, output i's page-table row (or first slot) and
    // patch factors
    uint8_t* stg = (uint8_t*)staging;
    auto tokens_of = [&](int c) { return vl ? vl->n_tokens[c] : T; };
    auto one_src = [&](int k, int tc) {
        const int64_t stream_el = (int64_t)L.num_layers * tc * F;
        kamera_src o;
        memset(&o, 0, sizeof(o));
        for (int s = 0; s < S; ++s) o.rows[s] = (const uint16_t*)(stg + k * sb + s * stream_el * 2);
        o.chunk_stride = stream_el;
        o.layer_stride = (int64_t)tc * F;
        o.n_tokens = tc;
        o.n_store = 1;
        return o;
    };
    const int ppc = dst->page_size > 0 ? (T + dst->page_size - 1) / dst->page_size : 0;
    auto one_dst = [&](int i) {
        kamera_dst d = *dst;
        d.page_order = nullptr;     // one chunk: nothing to sort
        d.check_scratch = nullptr;  // one chunk per call: nothing to compare
        if (dst->page_size > 0) {
            if (dst->page_table) d.page_table = dst->page_table + (int64_t)i * ppc;
        } else if (dst->dst_offset) {
            d.dst_offset = dst->dst_offset + i;
        }
        return d;
    };
    // output i's factors: U from its first row (row0), V block i
    auto one_patch = [&](int i, int64_t row0) {
        kamera_patch q;
        memset(&q, 0, sizeof(q));
        q.rank = m;
        for (int s = 0; s < S && m > 0; ++s) {
            q.u[s] = patch->u[s] ? patch->u[s] + row0 * m : nullptr;
            q.v[s] = patch->v[s] ? patch->v[s] + (int64_t)i * L.num_layers * F * m : nullptr;
        }
        return q;
    };
    auto relocate_one = [&](int i, int k, int64_t row0, int tc, hipStream_t hs) {
        const kamera_src o = one_src(k, tc);
        const kamera_dst d = one_dst(i);
        if (m > 0) {
            const kamera_patch q = one_patch(i, row0);
            return kamera_relocate_patch(layout, &o, 1, delta + i, &q, &d, hs);
        }
        return kamera_relocate(layout, &o, 1, delta + i, &d, hs);
    };
    {
        // the device path's argument checks (with n = 0 it returns before any
        // launch); the shape checks that need n > 0 run on chunk 0's call,
        // before its relocation and after only its copy into the staging slot
        const kamera_src o = one_src(0, T);
        const kamera_dst d = one_dst(0);
        kamera_status st;
        if (m > 0) {
            const kamera_patch q = one_patch(0, 0);
            st = kamera_relocate_patch(layout, &o, 0, delta, &q, &d, compute_stream);
        } else {
            st = kamera_relocate(layout, &o, 0, delta, &d, compute_stream);
        }
        if (st != KAMERA_OK) return st;
    }

    hipStream_t cs = (hipStream_t)copy_stream, ks = (hipStream_t)compute_stream;
    hipEvent_t copied[64], done[64], entry = nullptr;
    const int ne = slots < 64 ? slots : 64;
    int made = 0;
    kamera_status result = KAMERA_OK;
    for (; made < ne; ++made) {
        if (hipEventCreateWithFlags(&copied[made], hipEventDisableTiming) != hipSuccess) break;
        if (hipEventCreateWithFlags(&done[made], hipEventDisableTiming) != hipSuccess) {
            (void)hipEventDestroy(copied[made]);
            break;
        }
    }
    if (made < ne) result = KAMERA_ERR_HIP;
    // The staging slots may still be read by work queued earlier on the
    // compute stream (the relocations of a previous call that used the same
    // buffer): no copy of this call starts before that work is done.
    if (result == KAMERA_OK && cs != ks) {
        if (hipEventCreateWithFlags(&entry, hipEventDisableTiming) != hipSuccess || hipEventRecord(entry, ks) != hipSuccess ||
            hipStreamWaitEvent(cs, entry, 0) != hipSuccess)
            result = KAMERA_ERR_HIP;
    }
    int64_t row0 = 0;  // first factor row of output i
    int j = 0;         // non-empty chunks so far: they take the slots in turn
    for (int i = 0; i < n && result == KAMERA_OK; ++i) {
        const int c = chunk_ids[i];
        const int tc = tokens_of(c);
        const int64_t rows_i = (int64_t)L.num_layers * tc;
        if (tc == 0) continue;  // an empty chunk writes nothing
        const int k = j % ne;
        if (j >= ne && hipStreamWaitEvent(cs, done[k], 0) != hipSuccess) {
            result = KAMERA_ERR_HIP;
            break;
        }
        for (int s = 0; s < S && result == KAMERA_OK; ++s) {
            uint8_t* to = stg + k * sb + s * rows_i * F * 2;
            const size_t width = (size_t)tc * F * 2;
            hipError_t e;
            if (vl) {
                // a packed chunk's rows are contiguous: one copy
                const uint16_t* src = host_src->rows[s] + vl->row_offset[c] * F;
                e = hipMemcpyAsync(to, src, width * (size_t)L.num_layers, hipMemcpyHostToDevice, cs);
            } else {
                const uint16_t* src = host_src->rows[s] + (int64_t)c * host_src->chunk_stride;
                const size_t spitch = L.num_layers > 1 ? (size_t)host_src->layer_stride * 2 : width;
                e = hipMemcpy2DAsync(to, width, src, spitch, width, (size_t)L.num_layers, hipMemcpyHostToDevice, cs);
            }
            if (e != hipSuccess) result = KAMERA_ERR_HIP;
        }
        if (result != KAMERA_OK) break;
        if (hipEventRecord(copied[k], cs) != hipSuccess || hipStreamWaitEvent(ks, copied[k], 0) != hipSuccess) {
            result = KAMERA_ERR_HIP;
            break;
        }
        const kamera_status st = relocate_one(i, k, vl ? row0 : (int64_t)i * L.num_layers * T, tc, ks);
        if (st != KAMERA_OK) {
            result = st;
            break;
        }
        if (hipEventRecord(done[k], ks) != hipSuccess) result = KAMERA_ERR_HIP;
        row0 += rows_i;
        ++j;
    }
    // the compute stream's last relocation follows every copy: nothing the
    // caller waits on depends on the copy stream beyond it
    for (int k = 0; k < made; ++k) {
        (void)hipEventDestroy(copied[k]);
        (void)hipEventDestroy(done[k]);
    }
    if (entry) (void)hipEventDestroy(entry);
    return result;
}

}  // namespace

extern "C" {

kamera_status kamera_relocate_patch_host(const kamera_layout* layout, const kamera_src* host_src, int32_t n,
                                         const int32_t* chunk_ids, const int64_t* delta,
                                         const kamera_patch* patch, const kamera_dst* dst, void* staging,
                                         int64_t staging_bytes, void* copy_stream, void* compute_stream) {
    return relocate_host(layout, host_src, nullptr, n, chunk_ids, delta, patch, dst, staging, staging_bytes,
                         copy_stream, compute_stream);
}

kamera_status kamera_relocate_patch_host_varlen(const kamera_layout* layout, const kamera_src* host_src,
                                                const kamera_varlen* host_varlen, int32_t n,
                                                const int32_t* chunk_ids, const int64_t* delta,
                                                const kamera_patch* patch, const kamera_dst* dst, void* staging,
                                                int64_t staging_bytes, void* copy_stream, void* compute_stream) {
    if (!host_varlen) return KAMERA_ERR_NULL;
    return relocate_host(layout, host_src, host_varlen, n, chunk_ids, delta, patch, dst, staging, staging_bytes,
                         copy_stream, compute_stream);
}

}  // extern "C"
