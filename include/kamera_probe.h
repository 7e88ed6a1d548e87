/*
 * kamera_probe.h — copy-ceiling probe for measuring the Kamera reuse kernels
 * on AMD Instinct MI355X (gfx950).  Not part of the operator: a measurement
 * helper, shipped as its own library (libkamera_probe.so).
 *
 * Why it exists.  The Kamera pages place the cost of reuse on memory
 * bandwidth once the forward pass is gone (Kamera technical summary on
 * gist.science, paper 2606.23581, section 5 "Significance", and section 4,
 * efficiency and memory).  The relocation kernels read every canonical row
 * once and write it once into a paged pool, so the fastest they could ever
 * run is the rate at which the same bytes can be copied in the same access
 * pattern.  This probe is that copy: 16-byte nontemporal loads and stores, one
 * or two vectors per thread, single-shot 256-thread workgroups (the shape
 * that streams fastest on MI355X), and no arithmetic.
 *
 * The copy is described as a list of equal-sized blocks: block b copies
 * block_bytes bytes from src + src_off[b] to dst + dst_off[b].  A NULL offset
 * array means block b sits at b * block_bytes on that side (a sequential
 * stream).  Workgroups take the blocks in list order, so the list order is
 * the order in which the pattern is walked (a relocation kernel's page-table
 * order, or ascending destination pages).
 *
 * Ownership and ordering: src, dst and the offset arrays are DEVICE memory
 * owned by the caller; the call allocates nothing, enqueues one kernel on
 * `hip_stream` (a hipStream_t; NULL = the default stream) and returns without
 * synchronising.
 *
 * Errors (checked on the host before any HIP call): NULL src/dst (or a NULL
 * offset array with nblocks > 0 is fine: see above) -> KAMERA_PROBE_ERR_NULL;
 * src, dst, the offset arrays or block_bytes not 16-byte aligned ->
 * KAMERA_PROBE_ERR_ALIGN; nblocks < 0, block_bytes < 16, vectors_per_thread
 * not 1 or 2, or nblocks * block_bytes / 16 >= 2^31 -> KAMERA_PROBE_ERR_RANGE.
 * Offsets live in device memory, so the host cannot see them: the kernel
 * checks every block against src_bytes and dst_bytes and skips a block that
 * would leave either buffer.  A HIP launch failure -> KAMERA_PROBE_ERR_HIP.
 */
#ifndef KAMERA_PROBE_H
#define KAMERA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    KAMERA_PROBE_OK = 0,
    KAMERA_PROBE_ERR_NULL = 1,
    KAMERA_PROBE_ERR_ALIGN = 2,
    KAMERA_PROBE_ERR_RANGE = 4,
    KAMERA_PROBE_ERR_HIP = 7
};

/* Copies nblocks blocks of block_bytes bytes (see above).
 *   src, src_bytes: source buffer and its size in bytes (device);
 *   dst, dst_bytes: destination buffer and its size in bytes (device);
 *   src_off, dst_off: int64 [nblocks] byte offsets of each block, or NULL;
 *   vectors_per_thread: 16-byte vectors each thread moves (1 or 2).
 * Returns KAMERA_PROBE_OK or one of the errors above. */
int32_t kamera_probe_copy_blocks(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes,
                                 const int64_t* src_off, const int64_t* dst_off, int64_t nblocks,
                                 int64_t block_bytes, int32_t vectors_per_thread, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* KAMERA_PROBE_H */
