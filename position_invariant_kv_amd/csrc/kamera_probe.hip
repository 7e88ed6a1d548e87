// kamera_probe.hip — copy-ceiling probe (include/kamera_probe.h): the same
// bytes a relocation call moves, copied in the same block pattern with no
// arithmetic, so that a kernel's rate can be read against what a plain
// 16-byte copy reaches on this GPU in that pattern.
//
// Shape: 256-thread workgroups, one or two 16-byte vectors per thread, each
// workgroup used once (no grid-stride loop), nontemporal loads and stores.
// Measured on MI355X, that is the fastest plain streaming copy (more vectors
// per thread stream slower).

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "kamera_common.h"
#include "kamera_probe.h"

namespace {

constexpr int kProbeThreads = 256;

// Vector v of the pattern lies in block b = v / vpb, at byte 16 * (v % vpb) of
// it.  A block whose source or destination range leaves its buffer is skipped.
template <int U>
__global__ __launch_bounds__(kProbeThreads) void copy_blocks_kernel(
    const uint8_t* __restrict__ src, const int64_t src_bytes, uint8_t* __restrict__ dst, const int64_t dst_bytes,
    const int64_t* __restrict__ src_off, const int64_t* __restrict__ dst_off, const uint32_t total_vec,
    const FastDiv vpb, const int64_t block_bytes) {
    const uint32_t v0 = blockIdx.x * (uint32_t)(kProbeThreads * U) + threadIdx.x;
    u32x4 x[U];
    int64_t d[U];
    bool ok[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const uint32_t v = v0 + (uint32_t)(k * kProbeThreads);
        const uint32_t vc = v < total_vec ? v : total_vec - 1u;
        const uint32_t b = fdiv(vc, vpb);
        const int64_t w = (int64_t)(vc - b * vpb.d) * 16;
        const int64_t sb = src_off ? src_off[b] : (int64_t)b * block_bytes;
        const int64_t db = dst_off ? dst_off[b] : (int64_t)b * block_bytes;
        ok[k] = v < total_vec && sb >= 0 && sb <= src_bytes - block_bytes && db >= 0 &&
                db <= dst_bytes - block_bytes;
        d[k] = db + w;
        if (ok[k]) x[k] = ld_stream(reinterpret_cast<const uint16_t*>(src + sb + w));
    }
#pragma unroll
    for (int k = 0; k < U; ++k)
        if (ok[k]) st_stream(reinterpret_cast<uint16_t*>(dst + d[k]), x[k]);
}

}  // namespace

extern "C" {

int32_t kamera_probe_copy_blocks(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes,
                                 const int64_t* src_off, const int64_t* dst_off, int64_t nblocks,
                                 int64_t block_bytes, int32_t vectors_per_thread, void* hip_stream) {
    if (!src || !dst) return KAMERA_PROBE_ERR_NULL;
    if (!aligned16(src) || !aligned16(dst) || block_bytes % 16 != 0) return KAMERA_PROBE_ERR_ALIGN;
    if ((src_off && ((uintptr_t)src_off & 7u)) || (dst_off && ((uintptr_t)dst_off & 7u)))
        return KAMERA_PROBE_ERR_ALIGN;
    if (nblocks < 0 || block_bytes < 16 || (vectors_per_thread != 1 && vectors_per_thread != 2))
        return KAMERA_PROBE_ERR_RANGE;
    if (src_bytes < 0 || dst_bytes < 0) return KAMERA_PROBE_ERR_RANGE;
    if (nblocks == 0) return KAMERA_PROBE_OK;
    const int64_t vpb = block_bytes / 16;
    if (vpb >= ((int64_t)1 << 31) || nblocks >= ((int64_t)1 << 31) / vpb) return KAMERA_PROBE_ERR_RANGE;
    const uint32_t total = (uint32_t)(nblocks * vpb);
    const uint32_t per_wg = (uint32_t)(kProbeThreads * vectors_per_thread);
    const dim3 grid((total + per_wg - 1) / per_wg);
    const FastDiv div = make_fastdiv((uint32_t)vpb);
    hipStream_t hs = (hipStream_t)hip_stream;
    const uint8_t* s = (const uint8_t*)src;
    uint8_t* d = (uint8_t*)dst;
    const hipError_t e =
        vectors_per_thread == 1
            ? launch_kernel(copy_blocks_kernel<1>, grid, dim3(kProbeThreads), hs, s, src_bytes, d, dst_bytes, src_off,
                            dst_off, total, div, block_bytes)
            : launch_kernel(copy_blocks_kernel<2>, grid, dim3(kProbeThreads), hs, s, src_bytes, d, dst_bytes, src_off,
                            dst_off, total, div, block_bytes);
    return e == hipSuccess ? KAMERA_PROBE_OK : KAMERA_PROBE_ERR_HIP;
}

}  // extern "C"
