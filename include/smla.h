/*
 * smla.h -- C ABI of the sparse MLA decode library (libsmla.so, AMD gfx950).
 *
 * One decode step of sparse Multi-head Latent Attention: every query token
 * (one per sequence) attends, with all of this GPU's heads, over the latent KV
 * rows that the sequence's top-k list selects.  Keys and values are the same
 * 512-wide latent row: 448 "nope" columns stored as fp8 e4m3fn codes with one
 * scale per 64-column group (fp32, or an exponent byte), and 64 "rope" columns
 * stored as bf16.
 * Sources: "The Moment of Compilation", section "The Context: A Kernel
 * Optimization Campaign" (one KV read shared by all heads in a batched
 * matrix product); "The Power-of-Two Trap", sections "The Scene", "The Scale
 * Indexing Complication" and "Input Knowledge Required" (448 + 64 latent
 * split, per-64-column group scales, 7 groups plus one padding slot);
 * "The 80KB Mystery", section "The Context: Optimizing Attention on
 * Blackwell" (split-K over the selected tokens).
 *
 * All entry points are host functions.  Pointers to tensors are device
 * pointers owned by the caller; the library allocates nothing per call and
 * never synchronises the stream, so a call can be captured in a HIP graph.
 * Invalid host-visible arguments return an error status before anything is
 * launched and leave all outputs untouched.  Device-resident contents
 * (indices, sequence lengths, cache bytes) are never inspected by the host.
 */
#ifndef SMLA_H
#define SMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Cache row formats: one token's latent row, a fixed number of bytes apart.
 *
 * SMLA_ROW_FP32_SCALES (0), SMLA_ROW_BYTES = 640 bytes per row:
 *   bytes   0..447  nope, 448 fp8 e4m3fn codes (OCP, largest finite 448)
 *   bytes 448..479  8 fp32 group scales; slot g scales nope columns 64g..64g+63
 *                   for g < 7; slot 7 is padding, its value is never used
 *   bytes 480..607  rope, 64 bf16 values
 *   bytes 608..639  padding, never read
 *
 * SMLA_ROW_UE8M0_SCALES (1), SMLA_ROW_BYTES_UE8M0 = 584 bytes per row: the
 * exponent-only scale format ("The Power-of-Two Trap", section "Input
 * Knowledge Required": unsigned 8-bit scale exponents, one per 64 columns):
 *   bytes   0..447  nope, 448 fp8 e4m3fn codes
 *   bytes 448..454  7 group scale bytes; byte e stands for 2^(e - 127)
 *                   (e = 255 is NaN)
 *   byte  455       padding, never read
 *   bytes 456..583  rope, 64 bf16 values
 *
 * Dequantised row (both formats): K[i] = e4m3(code[i]) * scale[i / 64] for
 * i < 448, K[448 + k] = rope[k]. */
#define SMLA_ROW_FP32_SCALES 0
#define SMLA_ROW_UE8M0_SCALES 1
#define SMLA_ROW_BYTES 640
#define SMLA_ROW_BYTES_UE8M0 584
#define SMLA_NOPE_DIM 448
#define SMLA_ROPE_DIM 64
#define SMLA_LATENT_DIM 512
#define SMLA_GROUP 64
#define SMLA_SCALE_OFFSET 448
#define SMLA_ROPE_OFFSET 480
#define SMLA_ROPE_OFFSET_UE8M0 456

typedef enum {
    SMLA_OK = 0,
    SMLA_ERR_NULL = 1,         /* a required pointer is NULL */
    SMLA_ERR_SHAPE = 2,        /* bad batch/heads/topk/splits/stride/row format */
    SMLA_ERR_UNSUPPORTED = 3,  /* current device is not gfx950 */
    SMLA_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required */
    SMLA_ERR_HIP = 5,          /* a HIP runtime call or launch failed */
    SMLA_ERR_ALIGN = 6,        /* a pointer violates its alignment rule */
    SMLA_ERR_NO_DEVICE = 7,    /* no HIP device is available */
    SMLA_ERR_SCRATCH = 8       /* sparse_mla_decode_noalloc: the shape's split partials
                                  exceed SMLA_NOALLOC_SCRATCH_BYTES */
} smla_status;

/* Largest top-k list a call accepts (larger: SMLA_ERR_SHAPE).  The pages'
 * lists are 64 to 2048 entries; the bound keeps every byte offset into a list
 * and the split search far inside 32 bits. */
#define SMLA_MAX_TOPK (1 << 20)

typedef struct {
    int32_t batch;          /* B >= 0: query tokens, one per sequence */
    int32_t num_heads;      /* H >= 0, multiple of 16, <= 256: this GPU's heads */
    int32_t topk;           /* 0 .. SMLA_MAX_TOPK: entries in each top-k list */
    int32_t num_splits;     /* >= 0: split-K chunks per list; 0 = library's choice */
    int64_t kv_seq_stride;  /* >= 1: cache rows between sequence b and b + 1;
                               kv_seq_stride * row bytes must be below 2^31 */
    int32_t row_format;     /* SMLA_ROW_FP32_SCALES (0) or SMLA_ROW_UE8M0_SCALES (1) */
} smla_shape;

/* Split count a call with this shape uses (num_splits == 0 resolved by the
 * launch heuristic, larger requests clamped to the number of 32-token tiles).
 * Returns -1 for a NULL or invalid shape. */
int32_t smla_num_splits(const smla_shape* shape);

/* Workspace bytes sparse_mla_decode needs for this shape: 0 when one split is
 * used, otherwise room for the split partials (see sparse_mla_combine).
 * Returns 0 for a NULL or invalid shape. */
size_t smla_workspace_bytes(const smla_shape* shape);

/*
 * sparse_mla_decode -- one decode step.
 *
 *   q         bf16 [B][H][512], 16-byte aligned; columns 0..447 nope, 448..511 rope
 *   kv_cache  bytes [B][kv_seq_stride][R] in shape->row_format (R = 640 or
 *             584, formats above), 16-byte aligned; row t of sequence b
 *             starts at (b * kv_seq_stride + t) * R
 *   topk_idx  int32 [B][topk], 4-byte aligned: cache row of each list entry.
 *             An entry is skipped when it is < 0, >= seqlens[b] or >=
 *             kv_seq_stride (-1 pads short lists), so no device contents can
 *             make a sequence read outside its own rows; entries may come in
 *             any order; a repeated entry is counted once per occurrence
 *   seqlens   int32 [B], 4-byte aligned (normally <= kv_seq_stride)
 *   scale     softmax scale applied to q . K (e.g. 1/sqrt(512))
 *   out       bf16 [B][H][512], 16-byte aligned:
 *             out = sum_j softmax_j(scale * q . K_j) * K_j over the kept entries;
 *             all zeros when a list keeps no entry
 *   lse       fp32 [B][H]: natural-log sum of exp(scale * q . K_j); -inf when a
 *             list keeps no entry
 *   shape     sizes, see smla_shape
 *   workspace device memory of smla_workspace_bytes(shape) bytes, 256-byte
 *             aligned (may be NULL when that size is 0); its contents on entry
 *             do not matter and are overwritten
 *   stream    hipStream_t to launch on (NULL: the default stream)
 *
 * When batch or num_heads is 0 the call does nothing (tensor pointers may be
 * NULL); when topk is 0, kv_cache and topk_idx may be NULL and every output
 * row is 0 with lse -inf.
 *
 * Numerical contract: q . K is accumulated in fp32 from the exact bf16 query
 * and exact fp8/bf16 key values, with the group scales applied in fp32; the
 * softmax weights enter the value product in fp16 (value codes exact): a
 * weight is p * scale with p <= 2^8, so group scales must be finite with
 * magnitude at most 255 (UE8M0 bytes at most 134, i.e. 2^7), and rope values
 * below 65504 in magnitude.  Scales below 2^-14 give subnormal fp16 weights
 * (fewer significant bits, on values that small in absolute terms).  NaN
 * inputs propagate to the affected outputs.
 */
smla_status sparse_mla_decode(const void* q, const void* kv_cache, const int32_t* topk_idx,
                              const int32_t* seqlens, float scale, void* out, float* lse,
                              const smla_shape* shape, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * sparse_mla_decode_partials -- the decode kernel of sparse_mla_decode alone:
 * every split writes its normalised partial output and log-sum-exp instead of
 * the final result (also when the shape resolves to one split).
 *
 *   q, kv_cache, topk_idx, seqlens, scale, shape: as for sparse_mla_decode
 *   o_part    fp32 [B][H][S][512], 16-byte aligned, S = smla_num_splits(shape);
 *             split i covers list entries [i*C, min((i+1)*C, topk)) with
 *             C = smla_split_size(shape); an empty split writes 0
 *   lse_part  fp32 [B][H][S]: the split's log-sum-exp, -inf when it keeps no entry
 * sparse_mla_combine(o_part, lse_part, ...) then yields sparse_mla_decode's
 * result.
 */
smla_status sparse_mla_decode_partials(const void* q, const void* kv_cache,
                                       const int32_t* topk_idx, const int32_t* seqlens,
                                       float scale, const smla_shape* shape, float* o_part,
                                       float* lse_part, void* stream);

/*
 * Paged cache: the rows of all sequences live in one pool of pages of
 * page_size rows each (row bytes per shape->row_format), and
 * block_table[b][p] (int32 [B][pages_per_seq]) is the pool page that holds
 * positions p * page_size .. (p + 1) * page_size - 1 of sequence b: list entry
 * t of sequence b is pool row block_table[b][t / page_size] * page_size +
 * t % page_size.  The pages describe the deployed cache as paged ("The
 * Power-of-Two Trap", section "Input Knowledge Required") without giving a
 * block size or table; this is the usual block-table pool.
 */
typedef struct {
    int32_t page_size;      /* rows per page: a power of two, 1 .. 2^20 */
    int32_t pages_per_seq;  /* 1 .. 2^29: entries per block-table row */
    int64_t num_pages;      /* >= 1: pages in the pool; num_pages * page_size < 2^32 */
} smla_paged;

/*
 * sparse_mla_decode_paged -- sparse_mla_decode over a paged pool.
 *
 *   kv_pool     bytes [num_pages * page_size][R], 16-byte aligned (R = row bytes
 *               of shape->row_format); may exceed 4 GB
 *   block_table int32 [B][pages_per_seq], 4-byte aligned
 *   paged       page geometry, see smla_paged
 *   shape       as for sparse_mla_decode; kv_seq_stride is not used (pass 1)
 *   all other arguments as for sparse_mla_decode.
 * A list entry is skipped when it is < 0 or >= seqlens[b] (as before), when
 * t / page_size >= pages_per_seq, or when its block-table slot is negative or
 * >= num_pages.  The result is that of sparse_mla_decode on a contiguous
 * cache holding the same rows.  Invalid page geometry returns SMLA_ERR_SHAPE;
 * a NULL paged or (topk > 0) block_table returns SMLA_ERR_NULL.
 */
smla_status sparse_mla_decode_paged(const void* q, const void* kv_pool, const int32_t* block_table,
                                    const int32_t* topk_idx, const int32_t* seqlens, float scale,
                                    void* out, float* lse, const smla_shape* shape,
                                    const smla_paged* paged, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* The decode kernel of sparse_mla_decode_paged alone: split partials as for
 * sparse_mla_decode_partials. */
smla_status sparse_mla_decode_partials_paged(const void* q, const void* kv_pool,
                                             const int32_t* block_table, const int32_t* topk_idx,
                                             const int32_t* seqlens, float scale,
                                             const smla_shape* shape, const smla_paged* paged,
                                             float* o_part, float* lse_part, void* stream);

/*
 * sparse_mla_decode_single_launch -- sparse_mla_decode (or, with paged set,
 * sparse_mla_decode_paged) as one kernel launch.  The pages deploy the kernel
 * under CUDA-graph capture ("The Power-of-Two Trap", section "The Aftermath:
 * Validation and Deployment"); with the list split, the combine of the split
 * partials then runs inside the decode kernel instead of as a second launch:
 * the last of a (sequence, 16-head block)'s splits to finish merges every
 * split's partial (as sparse_mla_combine does) into out and lse.
 *
 *   q, topk_idx, seqlens, scale, out, lse, shape: as for sparse_mla_decode
 *   kv_cache    the contiguous cache, or with paged != NULL the pool
 *   block_table with paged != NULL, as for sparse_mla_decode_paged (ignored
 *               otherwise)
 *   paged       NULL for a contiguous cache, else as for sparse_mla_decode_paged
 *   workspace, workspace_bytes: as for sparse_mla_decode (the split partials)
 *   counters    uint32 [B][H / 16], 4-byte aligned device memory: one arrival
 *               counter per (sequence, 16-head block); may be NULL when the
 *               shape resolves to one split.  Every counter a call uses must be
 *               zero when it starts (e.g. allocate the array zeroed once, for
 *               the largest B x H / 16 it will serve); every call that runs to
 *               completion leaves them zero, so one array serves any later
 *               call, shape and graph replay.  Calls that share counters or a
 *               workspace must not run at the same time.
 *   stream      as for sparse_mla_decode
 *
 * With shape->num_splits 0 the split count is smla_num_splits_single_launch
 * (shape) (-1 for a NULL or invalid shape): at most sparse_mla_decode's, as the in-kernel merge costs more
 * than the combine kernel (32 sequences x 64 heads x top-512 runs as one
 * split), so the workspace sparse_mla_decode needs always suffices.
 *
 * Errors as for sparse_mla_decode / sparse_mla_decode_paged, plus
 * SMLA_ERR_NULL / SMLA_ERR_ALIGN for the counters of a split shape.  The
 * results are bitwise those of sparse_mla_decode with the same split count
 * (the same partials, merged by the same arithmetic); a shape that resolves
 * to one split is the same launch as sparse_mla_decode's.
 */
int32_t smla_num_splits_single_launch(const smla_shape* shape);
smla_status sparse_mla_decode_single_launch(const void* q, const void* kv_cache,
                                            const int32_t* block_table, const int32_t* topk_idx,
                                            const int32_t* seqlens, float scale, void* out,
                                            float* lse, const smla_shape* shape,
                                            const smla_paged* paged, void* workspace,
                                            size_t workspace_bytes, uint32_t* counters, void* stream);

/*
 * sparse_mla_decode_per_head -- the same step computed the way the production
 * kernel that the shared-read design replaced did it ("The Moment of
 * Compilation", section "The Context: A Kernel Optimization Campaign"): one
 * program (wave) per (sequence, head), fp32 vector arithmetic, every selected
 * row read again for every head, no split of the list.  An ablation baseline
 * for measuring the shared read; not the fast path.
 *
 *   arguments as for sparse_mla_decode; shape->num_splits is ignored and no
 *   workspace is used.  Same numerical contract (fp32 logits from exact
 *   operands; the value sum in fp32) and the same results up to rounding.
 */
smla_status sparse_mla_decode_per_head(const void* q, const void* kv_cache, const int32_t* topk_idx,
                                       const int32_t* seqlens, float scale, void* out, float* lse,
                                       const smla_shape* shape, void* stream);

/*
 * sparse_mla_decode_noalloc -- sparse_mla_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the split partials go to a fixed scratch
 * array that the library holds on each GPU (SMLA_NOALLOC_SCRATCH_BYTES, a
 * device array in the library's code object, kept until the process ends)
 * instead of a caller workspace.  The call itself allocates nothing.
 *
 *   arguments as for sparse_mla_decode, without workspace and workspace_bytes
 *
 * Returns SMLA_ERR_SCRATCH, before anything is launched, when
 * smla_workspace_bytes(shape) exceeds SMLA_NOALLOC_SCRATCH_BYTES (the split
 * partials are 2052 bytes per (sequence, head, split), so e.g. 32 sequences x
 * 64 heads x 2 splits fit).  Every call on one GPU uses that GPU's single
 * scratch array: calls that may run at the same time on one GPU (different
 * streams, or host threads) race and must be serialised by the caller.  The
 * scratch needs no clearing: each call overwrites every partial it reads.
 * Results are bitwise those of sparse_mla_decode with the same shape.
 */
#define SMLA_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
smla_status sparse_mla_decode_noalloc(const void* q, const void* kv_cache, const int32_t* topk_idx,
                                      const int32_t* seqlens, float scale, void* out, float* lse,
                                      const smla_shape* shape, void* stream);

/* List entries per split (C above, a multiple of 32); -1 for an invalid shape. */
int32_t smla_split_size(const smla_shape* shape);

/*
 * sparse_mla_combine -- the log-sum-exp merge of split partials (the second
 * kernel of sparse_mla_decode, exposed on its own).
 *
 *   o_part    fp32 [B][H][num_splits][512]: each split's normalised output
 *   lse_part  fp32 [B][H][num_splits]: each split's log-sum-exp (-inf = empty)
 *   out       bf16 [B][H][512]: sum_i exp(lse_i - LSE) * o_part_i
 *   lse       fp32 [B][H]: LSE = log(sum_i exp(lse_i)); -inf and out = 0 when
 *             every split is empty
 * o_part and out must be 16-byte aligned.  sparse_mla_decode places o_part at
 * offset 0 of its workspace and lse_part right after it.
 */
smla_status sparse_mla_combine(const float* o_part, const float* lse_part, int32_t batch,
                               int32_t num_heads, int32_t num_splits, void* out, float* lse,
                               void* stream);

/* Static description of a status code. */
const char* smla_status_str(smla_status status);

/*
 * Environment overrides, read once when the library is loaded:
 *
 *   SMLA_NSPLIT=n          the split count used when a shape leaves it to the
 *                          library (num_splits == 0), 1 <= n <= 4096; clamped
 *                          to the number of 32-token tiles like an explicit
 *                          request.  smla_num_splits and smla_workspace_bytes
 *                          follow it.  Other values are ignored.
 *   SMLA_DEBUG_VALIDATE=1  (any value other than "" and "0") every decode call
 *                          first launches, on the same stream, a scan of its
 *                          device-resident inputs (seqlens, topk_idx and the
 *                          block table), which the library otherwise never
 *                          inspects.  Conditions found are OR-ed into a
 *                          per-device word that smla_debug_flags reads.  The
 *                          decode results do not change; the scan costs
 *                          O(batch * topk^2) comparisons, so it is for debugging.
 *
 * The 16-head block and the four waves per workgroup are fixed by the kernel's
 * matrix-instruction shape and are not configurable.
 */
#define SMLA_DBG_SEQLEN    1u  /* a seqlens[b] < 0 or above the rows a sequence can address
                                  (kv_seq_stride; pages_per_seq * page_size when paged) */
#define SMLA_DBG_INDEX     2u  /* an entry < -1 or >= seqlens[b] (skipped) */
#define SMLA_DBG_PAGE      4u  /* paged: an entry below seqlens[b] whose block-table slot is
                                  < 0 or >= num_pages (skipped) */
#define SMLA_DBG_DUPLICATE 8u  /* a list holds the same kept entry twice (counted twice) */

/* 1 when SMLA_DEBUG_VALIDATE was set at load, else 0. */
int32_t smla_debug_validate_enabled(void);

/* Waits for the current device to finish (hipDeviceSynchronize), stores in
 * *flags the SMLA_DBG_* bits found by the scans run on it since the library
 * was loaded or the word was last cleared, and clears the word when clear is
 * non-zero.  0 when no scan ran.  Not for use under stream capture.
 * Errors: SMLA_ERR_NULL, SMLA_ERR_NO_DEVICE, SMLA_ERR_UNSUPPORTED, SMLA_ERR_HIP. */
smla_status smla_debug_flags(uint32_t* flags, int32_t clear);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H */
