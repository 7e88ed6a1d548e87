/*
 * kamera.h — C ABI of the Kamera position-invariant KV reuse operator on
 * AMD Instinct MI355X (gfx950).
 *
 * The operator (Kamera: Unified Position-Invariant Multimodal KV Cache for
 * Training-Free Reuse; technical summaries on gist.science, paper 2606.23581,
 * section 2 "Methodology: the Kamera operator", reuse equation):
 *
 *     KV^(B|A) = R(delta) . KV(B|empty) + U_m V_m^T
 *
 * R(delta) re-rotates the canonical keys of a cached chunk by the RoPE phase
 * shift delta of its new position (section 2, "Relocation"); U_m V_m^T is the
 * rank-m conditioning patch, added after the relocation (section 2, "Patch
 * application").  GQA/MHA rotate the whole key; MLA rotates only the decoupled
 * k_rope and keeps c_KV byte for byte; both families patch every channel
 * (section 2, "Unified architecture support").  The result of every output
 * chunk is scattered into a paged (or contiguous) KV pool.
 *
 * Data model (all counts in elements unless stated):
 *   - a ROW is one token of one layer of one stream: F = num_heads*head_dim
 *     bfloat16 values, stored as uint16 bit patterns, contiguous;
 *   - stream 0 carries RoPE inside every head at [rope_offset,
 *     rope_offset+rope_dim); stream 1 (if present: GQA/MHA values) never does;
 *     MLA is one stream whose row is c_KV followed by k_rope;
 *   - the canonical store holds n_store chunks of T rows per layer and stream;
 *     rows of chunk c, layer l start at rows[s] + c*chunk_stride + l*layer_stride;
 *   - the pool holds, per stream and layer, num_slots rows starting at
 *     rows[s] + l*layer_stride; token t of output chunk i goes to slot
 *       page_table[i*ceil(T/P) + t/P]*P + t%P   (paged, P = page_size > 0)
 *       dst_offset[i] + t                       (contiguous, P = 0).
 *
 * Arithmetic: inputs are widened to fp32.  For cos/sin of phi = delta*theta_j,
 * theta_j = rope_base^(-2j/rope_dim), the angle phi and its reduction
 * r = phi - k*pi/2 (|r| <= pi/4, two-term Cody-Waite) are computed in fp64;
 * sin r and cos r then come from their Taylor series evaluated in fp32 (error
 * <= 1e-7 in absolute value for |delta| <= 1e7), and k mod 4 picks the signs.
 * The rank-m product accumulates in fp32 (matrix cores); every element the
 * rotation or the patch touches is rounded once to bfloat16 (nearest-even).
 * Elements touched by neither (values and c_KV when m = 0) are copied bit for
 * bit.
 *
 * Ownership and ordering (every entry point):
 *   - every pointer inside the structs and every array argument is DEVICE
 *     memory owned by the caller, except the struct pointers themselves, which
 *     point to HOST memory read during the call only;
 *   - the library allocates nothing, keeps no pointer after returning, and
 *     enqueues its work on `hip_stream` (a hipStream_t; NULL = the default
 *     stream) without synchronising; buffers must stay valid until that work
 *     completes;
 *   - calls are thread-safe; two calls whose destinations overlap race.
 *
 * Errors: every argument check below runs on the host BEFORE any HIP call, so a
 * rejected call touches no device state.  Checks: NULL pointers; 16-byte
 * alignment of row bases, factor bases and strides; supported shapes; counts
 * in range; destination overlapping the source.  Indices that live in device
 * memory (page ids, destination offsets, chunk ids, permutations) cannot be
 * seen by the host: the kernels check every one against its bound and skip the
 * rows that would go out of range; if `error_word` is non-NULL they OR the
 * KAMERA_EW_* bits into it.  Repeated page ids and repeated chunk entries are
 * detected when the call also brings `check_scratch` (see "Content checks"
 * below); otherwise they are not, and the last writer wins.  A HIP launch
 * failure returns KAMERA_ERR_HIP.  n = 0 or T = 0 is a valid empty call and
 * returns KAMERA_OK without launching.
 */
#ifndef KAMERA_H
#define KAMERA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KAMERA_OK = 0,
    KAMERA_ERR_NULL = 1,        /* a required pointer is NULL                      */
    KAMERA_ERR_ALIGN = 2,       /* a row base, factor base or stride is not 16-B aligned */
    KAMERA_ERR_SHAPE = 3,       /* sizes are inconsistent with each other          */
    KAMERA_ERR_RANGE = 4,       /* a count or size is out of its range             */
    KAMERA_ERR_ALIAS = 5,       /* the destination overlaps the source            */
    KAMERA_ERR_UNSUPPORTED = 6, /* well-formed, but outside what the kernels cover */
    KAMERA_ERR_HIP = 7          /* the HIP runtime reported an error               */
} kamera_status;

/* Bits OR-ed into kamera_dst.error_word by the kernels. */
#define KAMERA_EW_PAGE   1u   /* a page id was outside [0, num_slots/page_size)      */
#define KAMERA_EW_OFFSET 2u   /* a contiguous chunk did not fit in [0, num_slots)   */
#define KAMERA_EW_CHUNK  4u   /* a permutation entry or chunk id was outside [0, n_store) */
#define KAMERA_EW_DUP_PAGE  8u   /* a page id repeated an earlier page-table entry's  */
#define KAMERA_EW_DUP_CHUNK 16u  /* a perm / chunk_ids entry repeated an earlier one  */

#define KAMERA_ROPE_HALF        0  /* element j pairs with j + rope_dim/2 (rotate-half) */
#define KAMERA_ROPE_INTERLEAVED 1  /* element 2j pairs with 2j + 1                       */

/* Shape of one row.  Supported: 1 <= num_streams <= 2, head_dim % 64 == 0,
 * head_dim <= 1024, rope_offset % 64 == 0, rope_dim % 64 == 0,
 * rope_offset + rope_dim <= head_dim, rope_base > 0, F = H*D <= 4096.
 * Other shapes return KAMERA_ERR_UNSUPPORTED. */
typedef struct {
    int32_t num_layers;   /* L, 1 <= L <= 65535                                 */
    int32_t num_heads;    /* KV heads H (1 for MLA)                             */
    int32_t head_dim;     /* D, elements per head (MLA: 512 + 64 = 576)         */
    int32_t rope_offset;  /* first rotated element inside a head (MLA: 512)     */
    int32_t rope_dim;     /* R, rotated elements per head (GQA: D, MLA: 64)     */
    int32_t rope_style;   /* KAMERA_ROPE_HALF or KAMERA_ROPE_INTERLEAVED        */
    double  rope_base;    /* theta_j = rope_base^(-2j/R)                        */
    int32_t num_streams;  /* 2 = K and V; 1 = one joint row (MLA)               */
} kamera_layout;

/* Canonical store KV(B|empty) (section 2, "Canonical KV"). */
typedef struct {
    const uint16_t* rows[2];     /* per stream: bfloat16 bits, see the data model     */
    int64_t chunk_stride;        /* elements between store chunks (multiple of 8)     */
    int64_t layer_stride;        /* elements between layers (multiple of 8)           */
    int32_t n_tokens;            /* T, rows per chunk, 0 <= T, T * F < 2^31           */
    int32_t n_store;             /* chunks in the store, >= 1                          */
    const int64_t* canon_pos;    /* [n_store] first position of each chunk's cached
                                    frame, used by reorder/recall; NULL = all 0        */
} kamera_src;

/* Rank-m factors, indexed by store chunk id (section 2, "Rank-m conditioning
 * patch").  u[s]: [n_store][L][T][m], v[s]: [n_store][L][F][m], contiguous.
 * MLA: one stream whose V holds the c_KV rows then the k_rope rows. */
typedef struct {
    int32_t rank;                /* m: 0, 8, 16, ..., 64                              */
    const uint16_t* u[2];
    const uint16_t* v[2];
} kamera_patch;

/* Destination pool. */
typedef struct {
    uint16_t* rows[2];           /* per stream: [L][num_slots][F] with layer_stride  */
    int64_t layer_stride;        /* elements between layers, >= num_slots*F, mult. of 8 */
    int64_t num_slots;           /* rows per layer                                    */
    int32_t page_size;           /* P > 0 paged; 0 contiguous                         */
    const int32_t* page_table;   /* paged: [n][ceil(T/P)] page ids                    */
    const int64_t* dst_offset;   /* contiguous: [n] first slot of each output chunk   */
    uint32_t* error_word;        /* optional: KAMERA_EW_* bits are OR-ed in           */
    int32_t* page_order;         /* optional scratch, paged pools only: [n*ceil(T/P)]
                                    int32 that the call overwrites (see below)         */
    int32_t* check_scratch;      /* optional scratch for the content checks, used only
                                    with error_word: [n*ceil(T/P) + n] int32 (paged) or
                                    [n] int32 (contiguous) that the call overwrites     */
} kamera_dst;

/* Content checks (kamera_dst.check_scratch).  A page id that appears twice
 * in one call's page table would make two chunks write one page, and a store
 * chunk that appears twice in a reorder's perm is not a permutation of the
 * cached set (section 3, "Reorder"), nor is a chunk recalled twice a single
 * rehydration (section 3, "Recall").  When error_word AND check_scratch are
 * non-NULL, the call first copies the page table and the perm / chunk_ids
 * array into check_scratch (page table first, then the n chunk entries) with
 * every entry that repeats the value of an EARLIER entry (in row-major
 * entry order) replaced by a skip marker, ORs KAMERA_EW_DUP_PAGE /
 * KAMERA_EW_DUP_CHUNK into error_word if it replaced any, and runs the
 * operator on those copies: the first occurrence is written, the repeats
 * write nothing.  Values outside their range are left for the range checks
 * (KAMERA_EW_PAGE / KAMERA_EW_CHUNK) and are not compared.  The checks sort
 * the entries in runs of 8192 per workgroup and compare every run with each
 * earlier one, so they cost O(E^2 / 8192 * log 8192) for E entries: tens of
 * microseconds up to ~16K entries.  Not checked: variable-length calls' page
 * tables (their rows are ragged; their chunk_ids are checked), overlapping
 * contiguous offsets, and the host-store entry points.  The scratch must not
 * overlap any other argument or be shared by calls that may run at the same
 * time. */

/* Destination order (kamera_dst.page_order).  The pool rows of one call form a
 * permutation of pages; HBM takes scattered 32 KiB writes markedly slower than
 * scattered 32 KiB reads, so when page_order is non-NULL the call first sorts
 * its page-table entries by page id (in runs of 8192 entries, one workgroup
 * each) into page_order, then processes the pages in that order, writing each
 * layer's pool in ascending address order, one whole page after another, and
 * reading the canonical rows in whatever order that implies.  The output is
 * identical either way.  The scratch must hold n*ceil(T/P) int32, must not
 * overlap any other argument and must not be shared by calls that may run at
 * the same time.  Pages are processed this way when a workgroup's rows stay
 * inside one page (m = 0: P*F a multiple of 2048; m > 0: P a multiple of the
 * workgroup's token span, 32 or 64); other shapes, contiguous pools and
 * page_order = NULL keep the page-table order. */

/*
 * Relocation only, m = 0 (section 3, "Sliding-Window Survival": chunks that
 * survive an eviction only need the exact re-rotation; no patch).  Output chunk
 * i is store chunk i (n <= n_store) shifted by delta[i].
 *   delta: [n] int64, device.
 */
kamera_status kamera_relocate(const kamera_layout* layout, const kamera_src* src, int32_t n,
                              const int64_t* delta, const kamera_dst* dst, void* hip_stream);

/*
 * Relocation plus the rank-m patch (section 2, reuse equation).  Output chunk i
 * is store chunk i shifted by delta[i] with the factors of chunk i added.
 * patch->rank = 0 is allowed and equals kamera_relocate.
 */
kamera_status kamera_relocate_patch(const kamera_layout* layout, const kamera_src* src, int32_t n,
                                    const int64_t* delta, const kamera_patch* patch,
                                    const kamera_dst* dst, void* hip_stream);

/*
 * kamera_relocate_patch with no allocation and no caller scratch.  For callers
 * that cannot allocate device memory or hand the library a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, checks and outputs as kamera_relocate_patch,
 * except that dst->page_order and dst->check_scratch are ignored: the call
 * keeps its page order (paged pools) and, with an error word, its content
 * checks in a fixed static array of the library on the current device (1 MiB:
 * 262,144 int32), so it needs n*ceil(T/P) int32 (paged) plus n*ceil(T/P) + n
 * more with an error word (contiguous: n), and returns KAMERA_ERR_RANGE before
 * any HIP call when that exceeds 262,144.  The array's device address is
 * looked up once per device on the first call there (KAMERA_ERR_HIP if that
 * fails); nothing is allocated, by the call or by that lookup.  Every call on
 * one GPU shares the array and leaves its contents behind (each call writes
 * every entry it reads first): calls on one GPU that may overlap in time
 * (different streams, host threads) race and must be ordered by the caller.
 */
kamera_status kamera_relocate_patch_noalloc(const kamera_layout* layout, const kamera_src* src, int32_t n,
                                            const int64_t* delta, const kamera_patch* patch,
                                            const kamera_dst* dst, void* hip_stream);

/*
 * Reorder (section 3, "Reorder": one orbit patch per chunk serves every order
 * of the cached set).  Output slot k holds store chunk c = perm[k], placed at
 * positions base_pos + k*T ...; its shift is delta = base_pos + k*T - canon_pos[c]
 * and its orbit patch is the factors of chunk c.  orbit may be NULL (m = 0).
 *   perm: [n] int32, device.
 */
kamera_status kamera_reorder(const kamera_layout* layout, const kamera_src* src, int32_t n,
                             const int32_t* perm, int64_t base_pos, const kamera_patch* orbit,
                             const kamera_dst* dst, void* hip_stream);

/*
 * Recall / reversible eviction (section 3, "Recall"): evicted store chunk
 * c = chunk_ids[i] is rehydrated at target_pos[i] from the canonical store with
 * its fresh patch; delta = target_pos[i] - canon_pos[c].  patch may be NULL.
 *   chunk_ids: [n] int32, target_pos: [n] int64, device.
 */
kamera_status kamera_recall(const kamera_layout* layout, const kamera_src* src, int32_t n,
                            const int32_t* chunk_ids, const int64_t* target_pos,
                            const kamera_patch* patch, const kamera_dst* dst, void* hip_stream);

/*
 * Variable-length chunks.  The cached chunks are whatever content an agent
 * revisits -- frames, screenshots, document pages (section 1, "Problem
 * definition"), long video segments (section 4, latency) -- and the window
 * operations act on whole chunks (section 3); nothing fixes a chunk's length,
 * so a store may hold chunks of different lengths.  Such a store keeps each chunk's rows back
 * to back: store chunk c has T_c = n_tokens[c] tokens, and its rows, layer by
 * layer, are
 *     rows[s][(row_offset[c] + l*T_c + t) * F + f]        (l < L, t < T_c)
 * with its U factor rows at u[s][(row_offset[c] + l*T_c + t) * m + k]; V stays
 * [n_store][L][F][m].  (A fixed-length store is the case T_c = T,
 * row_offset[c] = c*L*T.)
 *
 * In these calls kamera_src is read as: rows, n_store and canon_pos as above;
 * n_tokens = T_max, an upper bound of every T_c the call uses (it sizes the
 * launch and the page-table pitch); chunk_stride and layer_stride are ignored.
 * The page table keeps one row of ceil(T_max/P) entries per output chunk, of
 * which chunk i uses the first ceil(T_i/P); dst->page_order is ignored.  The
 * host checks row_offset and n_tokens for NULL and alignment (8 and 4 bytes);
 * the kernels check their values: a store chunk whose T_c is outside
 * [0, T_max] or whose rows leave [0, total_rows) is skipped whole and sets
 * KAMERA_EW_CHUNK; a contiguous chunk with dst_offset[i] + T_i > num_slots is
 * skipped and sets KAMERA_EW_OFFSET.  A chunk with T_c = 0 writes nothing.
 */
typedef struct {
    const int64_t* row_offset;   /* [n_store] device: first row of each store chunk   */
    const int32_t* n_tokens;     /* [n_store] device: T_c                              */
    int64_t total_rows;          /* host: rows in each stream's store (u[s]: rows x m)  */
} kamera_varlen;

/*
 * kamera_relocate_patch over variable-length chunks: output chunk i is store
 * chunk i (n <= n_store), shifted by delta[i] (device int64 [n]), with its
 * factors added.  patch may be NULL or of rank 0: relocation only (section 3,
 * "Sliding-Window Survival", for chunks of any length).  varlen: host struct.
 */
kamera_status kamera_relocate_patch_varlen(const kamera_layout* layout, const kamera_src* src,
                                           const kamera_varlen* varlen, int32_t n, const int64_t* delta,
                                           const kamera_patch* patch, const kamera_dst* dst,
                                           void* hip_stream);

/*
 * kamera_recall over variable-length chunks (section 3, "Recall"): output chunk
 * i is store chunk c = chunk_ids[i] placed at target_pos[i], delta =
 * target_pos[i] - canon_pos[c], with the factors of chunk c (patch may be
 * NULL).  A reorder of variable-length chunks (section 3, "Reorder") is this
 * call with chunk_ids = the new order and target_pos[k] = the first position
 * plus the lengths of the chunks placed before slot k; kamera_reorder itself
 * takes fixed-length chunks only.
 */
kamera_status kamera_recall_varlen(const kamera_layout* layout, const kamera_src* src,
                                   const kamera_varlen* varlen, int32_t n, const int32_t* chunk_ids,
                                   const int64_t* target_pos, const kamera_patch* patch,
                                   const kamera_dst* dst, void* hip_stream);

/*
 * Patch formation (section 2, "Patch application": the rank-m patch is made
 * once, by a forward pass on [A, B] and an SVD that keeps the top-m factors).
 * The forward pass is the caller's: `target` holds its output KV(B|A), chunk
 * i's rows at their positions in that context, in the same layout as the
 * canonical store.  For every output chunk i, layer and stream the call forms
 * the deficit in the destination frame, the reuse equation solved for the
 * patch,
 *     Delta = KV(B|A) - R(delta[i]) KV(B|empty)        (stream 0 rotated only),
 * and writes its rank-m factors U = U_m Sigma_m, V = V_m into `out` (the layout
 * kamera_relocate_patch reads: u[s] [n][L][T][m], v[s] [n][L][F][m], bfloat16),
 * so that relocate_patch(canon, delta, U, V) restores KV(B|A) up to the rank-m
 * truncation.  Conventions: each V column's largest-magnitude entry is
 * positive; directions whose singular value is <= 1e-6 sigma_1 give zero
 * columns.
 *
 * Method: randomized subspace iteration (Halko, Martinsson, Tropp, SIAM Review
 * 2011, Algorithms 4.4 and 5.1) with k = rank + oversample sketch columns and
 * power_iters passes; Delta is split into bfloat16 high and low parts for the
 * matrix cores; orthonormalization and the small k x k eigenproblems are fp64.
 * The result approaches the exact truncated SVD as the gap sigma_m/sigma_k
 * and power_iters grow; with rank(Delta) <= k it is exact up to rounding.
 *
 * canon, target: [n_store >= n][L][T][F] rows per stream (n_tokens equal).
 * delta: [n] int64, device.  sketch->omega: [k][F] bfloat16 test matrix the
 * caller draws (e.g. Gaussian), device, 16-byte aligned.  out->rank = m: even,
 * 2 <= m, m + oversample <= 64.  workspace: device, 256-byte aligned, at least
 * kamera_form_patch_workspace(...) bytes, overwritten; the call allocates
 * nothing.  Errors: as for the other entry points (checks before any HIP call;
 * outputs may not overlap the inputs or the workspace).
 */
typedef struct {
    int32_t oversample;          /* p >= 0 extra sketch columns                      */
    int32_t power_iters;         /* q, 0 ..16                                        */
    const uint16_t* omega;       /* [m + p][F] bfloat16 test matrix                  */
} kamera_sketch;

typedef struct {
    int32_t rank;                /* m                                                */
    uint16_t* u[2];              /* written: [n][L][T][m]                            */
    uint16_t* v[2];              /* written: [n][L][F][m]                            */
} kamera_factors;

/* Workspace bytes kamera_form_patch needs for this shape, or -1 if the shape
 * is outside what it supports. */
int64_t kamera_form_patch_workspace(const kamera_layout* layout, int32_t n, int32_t n_tokens,
                                    int32_t rank, int32_t oversample);

kamera_status kamera_form_patch(const kamera_layout* layout, const kamera_src* canon,
                                const kamera_src* target, int32_t n, const int64_t* delta,
                                const kamera_sketch* sketch, const kamera_factors* out,
                                void* workspace, int64_t workspace_bytes, void* hip_stream);

/*
 * Orbit patch formation (section 3, "Three cheap window operations", Reorder:
 * one patch, averaged over orderings, serves every ordering of a cached set).
 * Each chunk i is given `views` rows prefilled in different orderings:
 * targets chunk i * views + v holds KV_v(B_i | A_v), the rows of chunk i
 * after the context of ordering v, at shift deltas[i * views + v] from the
 * canonical rows.  The patch is added after the relocation in every ordering,
 * so the call decomposes the mean of the per-ordering deficits,
 *     Delta_orbit = (1 / views) sum_v [ KV_v(B|A_v) - R(delta_v) KV(B|empty) ],
 * with the same sketch, precision and conventions as kamera_form_patch (which
 * is this call with views = 1; the results are bit-identical).  targets holds
 * n * views chunks (n_store >= n * views); deltas has n * views entries.
 * Workspace: kamera_form_patch_workspace(layout, n, ...) bytes, the same as
 * for n chunks of the plain patch.  Errors: as for kamera_form_patch, and
 * KAMERA_ERR_RANGE for views < 1.
 */
kamera_status kamera_form_orbit_patch(const kamera_layout* layout, const kamera_src* canon,
                                      const kamera_src* targets, int32_t n, int32_t views,
                                      const int64_t* deltas, const kamera_sketch* sketch,
                                      const kamera_factors* out, void* workspace,
                                      int64_t workspace_bytes, void* hip_stream);

/*
 * Decode attention over a reused context, relocating on read (section 3,
 * "Production deployment": the engine's attention reads the reconstructed
 * cache; section 4: the reuse cost moves to memory bandwidth, the bound of
 * decoding).  The keys and values are the reuse equation applied to the
 * canonical store; nothing is written to a pool.
 *
 * Context: sequence b (0 <= b < num_seqs) attends entries
 * seq_entries[b] .. seq_entries[b+1]-1 (device int32 [num_seqs + 1],
 * non-decreasing, within [0, num_entries]).  Entry e is store chunk
 * chunk_ids[e] (device int32 [num_entries]) placed with shift delta[e]
 * (device int64): its T rows at layer `layer` are
 *     K = R(delta) K(B|empty) + U_K V_K^T,   V = V(B|empty) + U_V V_V^T
 * with the factors of patch (NULL or rank 0: no patch; u/v indexed by store
 * chunk as for kamera_relocate_patch).  The entries of a sequence are
 * concatenated in order; all of them precede the query.
 *
 * Query head h of sequence b (q: device bfloat16 [num_seqs][num_q_heads][D],
 * already rotated to the query's own position) reads KV head h / G,
 * G = num_q_heads / H:
 *     s_t = scale * q . k_t,  out = softmax(s) V,  lse = log sum_t exp(s_t).
 * MLA (num_streams = 1): every query head reads the one joint row as its key
 * (all D = 576 columns; q holds the absorbed queries) and the row's c_KV
 * part (its first rope_offset = 512 columns) as its value.
 * out: device float32 [num_seqs][num_q_heads][Dv] with Dv = D (two streams)
 * or rope_offset (MLA); lse: device float32 [num_seqs][num_q_heads] or NULL
 * (natural logarithm).  A sequence with no entries (or T = 0) gets out = 0
 * and lse = -inf.
 *
 * Arithmetic: fp32.  The shift turns the query by R(-delta) once per entry
 * (exact in real arithmetic, since R is orthogonal); the key patch enters as
 * U_K[t] . (V_K^T q) and the value patch as V_V (sum_t p_t U_V[t]).  Nothing
 * is rounded to bfloat16 between the store and the output.
 *
 * Supported: two streams (GQA/MHA) with D in {64, 128, 256} and
 * 1 <= G <= 16; one stream (MLA) with one KV head, D = 576, rope_offset = 512,
 * rope_dim = 64 and up to 16 query heads; rank 0..64 in steps of 8.  Other
 * layouts return KAMERA_ERR_UNSUPPORTED.
 * A chunk id outside [0, n_store) contributes nothing and, when error_word
 * is non-NULL, ORs KAMERA_EW_CHUNK into it.  workspace: device memory of
 * kamera_decode_attention_workspace(...) bytes, 256-byte aligned,
 * overwritten; the call allocates nothing.  Outputs may not overlap each
 * other, the workspace or any input.  Calls on one stream are ordered;
 * calls that share a workspace on different streams race.
 */
int64_t kamera_decode_attention_workspace(const kamera_layout* layout, int32_t num_q_heads,
                                          int32_t num_entries, int32_t n_tokens);

kamera_status kamera_decode_attention(const kamera_layout* layout, int32_t layer,
                                      const kamera_src* canon, const kamera_patch* patch,
                                      int32_t num_seqs, const int32_t* seq_entries,
                                      int32_t num_entries, const int32_t* chunk_ids,
                                      const int64_t* delta, int32_t num_q_heads,
                                      const uint16_t* q, float scale, float* out, float* lse,
                                      uint32_t* error_word, void* workspace,
                                      int64_t workspace_bytes, void* hip_stream);

/*
 * Decode attention over a reused context AND a paged pool (the engine's own KV
 * cache: section 3, "Production deployment", the engine's attention reads the
 * cache in its pool).  Sequence b attends the union of
 *   - its reused entries, relocated and patched on read exactly as in
 *     kamera_decode_attention, and
 *   - its first seq_tokens[b] pooled tokens: token t's row sits in pool slot
 *     block_table[b][t / P] * P + t % P (P = page_size), read as stored (keys
 *     already in their own frame: no shift, no patch);
 * the order of the two parts does not change the result.  Everything else --
 * query, scale, heads, MLA rows, outputs, errors -- as kamera_decode_attention.
 *
 * kamera_attn_pool: rows[s] per stream [L][num_slots][F], layer_stride apart
 * (the layout kamera_dst writes); page_size a multiple of 16 (else
 * KAMERA_ERR_UNSUPPORTED); block_table device int32 [num_seqs][max_pages];
 * seq_tokens device int32 [num_seqs], clamped to [0, max_pages * P].  A page
 * id outside [0, num_slots / P) masks its tokens out of the softmax and, when
 * error_word is non-NULL, ORs KAMERA_EW_PAGE into it.  max_pages = 0: no
 * pooled tokens.  workspace: kamera_decode_attention_paged_workspace(layout,
 * num_q_heads, num_entries, n_tokens, num_seqs, max_pages * page_size) bytes.
 */
typedef struct {
    const uint16_t* rows[2];     /* per stream: [L][num_slots][F] bfloat16 bits        */
    int64_t layer_stride;        /* elements between layers, >= num_slots*F, mult. of 8 */
    int64_t num_slots;           /* rows per layer                                     */
    int32_t page_size;           /* P, a multiple of 16                                 */
    int32_t max_pages;           /* entries per block-table row                         */
    const int32_t* block_table;  /* device [num_seqs][max_pages] page ids               */
    const int32_t* seq_tokens;   /* device [num_seqs] pooled tokens of each sequence   */
} kamera_attn_pool;

int64_t kamera_decode_attention_paged_workspace(const kamera_layout* layout, int32_t num_q_heads,
                                                int32_t num_entries, int32_t n_tokens, int32_t num_seqs,
                                                int32_t pool_max_tokens);

kamera_status kamera_decode_attention_paged(const kamera_layout* layout, int32_t layer,
                                            const kamera_src* canon, const kamera_patch* patch,
                                            const kamera_attn_pool* pool, int32_t num_seqs,
                                            const int32_t* seq_entries, int32_t num_entries,
                                            const int32_t* chunk_ids, const int64_t* delta,
                                            int32_t num_q_heads, const uint16_t* q, float scale,
                                            float* out, float* lse, uint32_t* error_word,
                                            void* workspace, int64_t workspace_bytes, void* hip_stream);

/*
 * Relocation (and patch) from a canonical store in pinned host memory
 * (section 3, "Three cheap window operations", Recall: evicted chunks are
 * rehydrated from the canonical store with a fresh patch, without
 * re-encoding).  Output chunk i is store chunk chunk_ids[i] relocated by
 * delta[i] plus patch i, written to the pool exactly as kamera_relocate_patch
 * writes output i (kamera_relocate when patch is NULL or rank 0); the result
 * is bit-identical to that call on a device copy of the same store.
 *
 * host_src: rows[s] in page-locked host memory (hipHostMalloc or a pinned
 *   torch tensor; pageable memory returns KAMERA_ERR_UNSUPPORTED), strides
 *   and n_tokens as for a device store; canon_pos must be NULL (the shifts
 *   are given).
 * chunk_ids: HOST int32 [n], each in [0, n_store) (checked).
 * delta: device int64 [n].
 * patch: NULL, or device factors indexed by OUTPUT index i:
 *   u[s] [n][L][T][m], v[s] [n][L][F][m].
 * dst: as for kamera_relocate_patch (page_table / dst_offset rows per output).
 * staging: device memory, 256-byte aligned, of at least
 *   kamera_host_staging_bytes(layout, T, 1) bytes; it holds
 *   staging_bytes / kamera_host_staging_bytes(layout, T, 1) chunk slots
 *   (at most 64 are used).  Two or more let copies and relocations overlap.
 * copy_stream, compute_stream: the H2D copies run on copy_stream, the
 *   relocations on compute_stream, ordered by events; they may be the same
 *   stream (then nothing overlaps).  Ordering across calls: the call's first
 *   copy waits for all work enqueued on compute_stream before the call (so a
 *   previous call's relocations are done reading a shared staging buffer),
 *   and every later copy into a slot waits for the relocation that last read
 *   it.  Back-to-back calls that share one staging buffer and one
 *   compute_stream are therefore safe without host synchronisation.  Work
 *   the caller enqueues on copy_stream itself is not waited for.  When the
 *   work on compute_stream is complete, the pool is written and the staging
 *   buffer is free.
 * Errors: argument errors return before any copy or launch, except shape
 * errors that only chunk 0's relocation detects: those return after chunk
 * 0's copy into the staging buffer (the pool is untouched).
 */
int64_t kamera_host_staging_bytes(const kamera_layout* layout, int32_t n_tokens, int32_t slots);

kamera_status kamera_relocate_patch_host(const kamera_layout* layout, const kamera_src* host_src,
                                         int32_t n, const int32_t* chunk_ids, const int64_t* delta,
                                         const kamera_patch* patch, const kamera_dst* dst,
                                         void* staging, int64_t staging_bytes, void* copy_stream,
                                         void* compute_stream);

/*
 * kamera_relocate_patch_host over variable-length chunks (the store layout of
 * kamera_varlen above, in pinned host memory).  Here host_varlen->row_offset
 * and host_varlen->n_tokens are HOST arrays [n_store] -- the host issues one
 * copy per chunk -- and are checked before any copy: every recalled chunk needs
 * 0 <= T_c <= T_max = host_src->n_tokens and its rows inside [0, total_rows)
 * (else KAMERA_ERR_RANGE).  Each recalled chunk's rows cross the host link in
 * one copy per stream.  patch: NULL, or device factors indexed by OUTPUT
 * index: u[s] packed in output order (output i's U rows start at row
 * sum over j < i of L*T_{chunk_ids[j]}), v[s] [n][L][F][m].  dst: page-table
 * rows of ceil(T_max/P) entries, output i using the first ceil(T_i/P), or
 * dst_offset.  staging: kamera_host_staging_bytes(layout, T_max, slots).
 * Chunks with T_c = 0 write nothing.  Output i is bit-identical to
 * kamera_recall_varlen's output i on a device copy of the same store with the
 * same factors.  Everything else as kamera_relocate_patch_host.
 */
kamera_status kamera_relocate_patch_host_varlen(const kamera_layout* layout, const kamera_src* host_src,
                                                const kamera_varlen* host_varlen, int32_t n,
                                                const int32_t* chunk_ids, const int64_t* delta,
                                                const kamera_patch* patch, const kamera_dst* dst,
                                                void* staging, int64_t staging_bytes, void* copy_stream,
                                                void* compute_stream);

/* Static text for a status code (never NULL). */
const char* kamera_status_string(kamera_status status);

/* Library version, as major*10000 + minor*100 + patch. */
int32_t kamera_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KAMERA_H */
