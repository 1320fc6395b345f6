/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) paged MLA decode library.
 *
 * The operation (restated from the FlashInfer API docs page
 * "flashinfer.attention.prims_ts.prims_ts_batch_decode_with_kv_cache_mla",
 * signature and the layout/mask and contract paragraphs; scale semantics from
 * FlashInfer PR #1248 "update cubins for dynamic scale factor interface and
 * one-copy kvcache on trtllm-gen mla", Highlights; one-copy K/V from FlashInfer
 * issue #3131 "Support cum_seq_lens_q in trtllm_batch_decode_with_kv_cache_mla
 * trtllm-gen backend", run_func excerpt; natural-log LSE from the vLLM docs page
 * "FlashInferMLAImpl", class attributes):
 *
 *   For request b with live KV length L = seq_lens[b] and query rows
 *   i = 0 .. q_b-1, and every head h:
 *     s[j]   = bmm1_scale * dot(q[r_b+i, h, 0:576], K[j, 0:576]),  j < n
 *     out[r_b+i, h, 0:512] = bmm2_scale * sum_j softmax(s)[j] * K[j, 0:512]
 *     lse[r_b+i, h]        = ln(sum_j exp(s[j]))          (no bmm2 inside)
 *   K[j] is cache row (block_tables[b, j / page_size], j % page_size); the same
 *   rows serve as values (their first 512 dims).  n = L - q_b + i + 1 when
 *   causal (bottom-right aligned), n = L otherwise.
 *
 * Everything here is asynchronous on the caller's HIP stream; nothing reads
 * device memory back to the host, nothing allocates, nothing synchronises.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Any code other than MLA_OK means nothing was enqueued. */
enum {
  MLA_OK = 0,
  MLA_ERR_NULL_POINTER = 1,      /* a required pointer is NULL */
  MLA_ERR_BAD_HEADS = 2,         /* num_heads <= 0 or not a multiple of 16 */
  MLA_ERR_BAD_PAGE_SIZE = 3,     /* page_size not in {16, 32, 64} */
  MLA_ERR_BAD_HEAD_DIMS = 4,     /* kv_lora_rank != 512 or qk_rope_head_dim != 64 */
  MLA_ERR_BAD_DTYPE = 5,         /* kv_dtype not MLA_KV_BF16 / MLA_KV_FP8_E4M3FN */
  MLA_ERR_MISALIGNED = 6,        /* q, kv_cache, out or workspace not 16-byte aligned; lse or an option pointer not 4-byte aligned */
  MLA_ERR_WORKSPACE_TOO_SMALL = 7,
  MLA_ERR_BAD_Q_LEN = 8,         /* max_q_len < 1, fixed launch with q_len_fixed != max_q_len,
                                    or total_q inconsistent with a fixed launch */
  MLA_ERR_BAD_BLOCK_TABLE = 9,   /* block_table_stride * page_size < max_seq_len */
  MLA_ERR_BAD_SHAPE = 10,        /* batch out of [1, MLA_MAX_BATCH], max_seq_len < 1, num_pages < 1,
                                    total_q * num_heads >= 2^31 - 4 */
  MLA_ERR_HIP = 11,              /* the HIP runtime reported an error at launch */
  MLA_ERR_NO_DEVICE = 12,        /* no usable gfx950 device is current */
  MLA_ERR_SCRATCH_TOO_SMALL = 13 /* mla_decode_paged_noalloc: the launch needs more than
                                    MLA_NOALLOC_SCRATCH_BYTES of workspace */
};

enum { MLA_KV_BF16 = 0, MLA_KV_FP8_E4M3FN = 1 };

/* Largest batch one launch accepts (the work plan lives in LDS); in the
   sparse top-k layout, the largest number of query rows. */
#define MLA_MAX_BATCH 1024

/* Largest sparse top-k list length. */
#define MLA_MAX_TOP_K (1 << 20)

/* Static shape of a launch.  All fields are host integers. */
typedef struct mla_decode_dims {
  int32_t batch;              /* B: requests */
  int32_t num_heads;          /* H: query heads (all share the one latent KV head) */
  int32_t q_len_fixed;        /* SQ for a fixed [B, SQ, H, 576] query; ignored when packed */
  int32_t total_q;            /* rows of q / out / lse (B*SQ, or qo_indptr[B] when packed) */
  int32_t page_size;          /* rows per cache page: 16, 32 or 64 */
  int64_t num_pages;          /* pages in kv_cache (page ids must be < num_pages) */
  int32_t block_table_stride; /* W: int32 entries per block_tables row */
  int32_t kv_dtype;           /* MLA_KV_BF16 or MLA_KV_FP8_E4M3FN */
  int32_t kv_lora_rank;       /* must be 512 */
  int32_t qk_rope_head_dim;   /* must be 64 */
} mla_decode_dims_t;

/*
 * mla_decode_paged -- enqueue one batched paged MLA decode on `stream`.
 *
 * q            device, bf16 [total_q, H, 576] row-major (a fixed [B, SQ, H, 576]
 *              query is the same bytes).  Dims 0..511 latent, 512..575 RoPE.
 * kv_cache     device, [num_pages, page_size, 576] (bf16, or fp8 E4M3FN bytes);
 *              a [num_pages, 1, page_size, 576] view is the same bytes.  Row j of
 *              request b is read only for j < seq_lens[b]; other slots may hold
 *              anything, NaN included, and never affect the result.
 * block_tables device, int32 [B, block_table_stride] row-major.  Only entries
 *              0 .. ceil(seq_lens[b]/page_size)-1 of row b are read.
 * seq_lens     device, int32 [B]; each in [1, max_seq_len] (0 allowed in the
 *              sequence-sharded mode of mla_decode_paged_ex).
 * qo_indptr    device, int32 [B+1] cumulative query offsets (starts at 0, strictly
 *              increasing, ends at total_q, deltas <= max_q_len), or NULL for a
 *              fixed launch where every request has q_len_fixed rows.
 * max_seq_len  static bound on seq_lens (sizes only; never changes results).
 * max_q_len    static bound on per-request query length (sizes only).
 * bmm1_scale   complete logit multiplier (softmax scale x q/k dequant scales).
 * bmm2_scale   output multiplier (v dequant scale x output scale).
 * causal       nonzero: bottom-right causal mask; zero: every row sees all L rows.
 *              Causal launches need q_b <= seq_lens[b].
 * out          device, bf16 [total_q, H, 512], written completely.
 * lse          device, float32 [total_q, H] natural-log LSE, or NULL for none.
 * workspace    device scratch of at least mla_decode_paged_workspace_size() bytes,
 *              16-byte aligned, exclusive to this launch until it completes, and
 *              not overlapping any other argument.  It needs no initialisation
 *              and holds nothing between launches.
 * dims         host pointer to the static shape above (read during the call only).
 * stream       hipStream_t to enqueue on (NULL = default stream).
 *
 * Ownership: every pointer stays owned by the caller; the library keeps none
 * after the enqueued work completes and allocates nothing per call.  The first
 * call on a device caches its compute-unit count; call once before capturing
 * a HIP graph.  Device-resident contract violations (lengths, offsets, page
 * ids out of range) are not checked and give undefined results.
 * Returns MLA_OK or an MLA_ERR_* code (then nothing was enqueued, except
 * MLA_ERR_HIP, which reports a launch failure).
 */
int mla_decode_paged(const void* q, const void* kv_cache, const int32_t* block_tables,
                     const int32_t* seq_lens, const int32_t* qo_indptr, int32_t max_seq_len,
                     int32_t max_q_len, float bmm1_scale, float bmm2_scale, int causal, void* out,
                     float* lse, void* workspace, size_t workspace_bytes,
                     const mla_decode_dims_t* dims, void* stream);

/*
 * Device-resident options of mla_decode_paged_ex.  Each pointer may be NULL.
 *
 * bmm1_scale  device float32 scalar.  When set it replaces the bmm1_scale
 *             argument, read by the kernels at run time (FlashInfer PR #1248,
 *             "dynamic scale factor interface"; issue #3131, Python API:
 *             bmm1_scale / bmm2_scale may be a tensor), so a captured HIP
 *             graph follows scale updates made between its replays.
 * bmm2_scale  device float32 scalar, likewise for bmm2_scale.
 * sinks       device float32 [num_heads]: per-head attention-sink logits, in
 *             natural-log units on the scale of bmm1_scale * q.k (issue #3131,
 *             launcher excerpt: attention_sinks).  Each (row, head) softmax
 *             gains one term exp(sinks[h]) in its denominator and none in its
 *             numerator; lse, when requested, is ln of that whole denominator.
 * seq_lens_global
 *             device int32 [B], or NULL: sequence-sharded (DCP) partial mode
 *             (vLLM docs, "FlashInferMLAImpl", forward_mqa: cp_world, cp_rank,
 *             causal_seqlens_kv_global).  The cache given to this call holds
 *             rank cp_rank's share of each request: global positions
 *             t = cp_rank (mod cp_world), in order, so local row j is global
 *             position j * cp_world + cp_rank and seq_lens[b] counts the local
 *             rows (0 allowed).  Causal limits come from the global lengths:
 *             query row i sees global positions below
 *             seq_lens_global[b] - q_b + i + 1.  out and lse are then this
 *             rank's partial: bmm2 * the softmax-normalised P.V over the visible
 *             local rows and ln of their exponent sum; a (row, head) with no
 *             visible local row gets out = 0 and lse = -inf.  mla_merge_partials
 *             combines the ranks' partials (lse is required in this mode).
 *             Sinks, when given, enter rank 0's partial only (on other ranks
 *             they are ignored), so the merge counts each sink once; a rank-0
 *             (row, head) with no visible local row then has out = 0 and
 *             lse = sinks[h].
 * cp_world, cp_rank
 *             1 <= cp_world, 0 <= cp_rank < cp_world; read only in DCP mode.
 * sparse_top_k
 *             0: the paged layout above.  K > 0: sparse top-k layout
 *             (FlashInfer issue #3131: the trtllm_batch_decode_with_kv_cache_mla
 *             and trtllm_paged_attention_decode signatures carry
 *             sparse_mla_top_k; the pages give no index layout, so this is the
 *             library's reading).  block_tables is then a device int32 array
 *             [total_q, block_table_stride] (stride >= K)
 *             whose row r lists, in its first K entries, the cache rows query
 *             row r attends to: entry e >= 0 is cache row e of the cache seen as
 *             [num_pages * page_size, 576] (page e / page_size, slot
 *             e % page_size; e < num_pages * page_size is the caller's contract,
 *             unchecked); a negative entry is empty.  Every head of row r
 *             attends to exactly the listed rows (a repeated entry counts once
 *             per listing); no causal or length mask applies, and seq_lens,
 *             qo_indptr, max_seq_len, max_q_len and causal are not read (seq_lens
 *             may be NULL).  A (row, head) with no live entry gets out = 0 and
 *             lse = -inf (lse = sinks[h] with a sink).  total_q <= MLA_MAX_BATCH,
 *             K <= MLA_MAX_TOP_K; not combinable with DCP mode.  The workspace
 *             size comes from mla_decode_paged_ex_workspace_size().
 * q_fp8       0: q holds bf16.  Nonzero: q holds OCP E4M3FN codes (uint8,
 *             same [rows, H, 576] layout), a query quantised to fp8 whose
 *             q_scale the caller folds into bmm1_scale (FlashInfer PR #1248:
 *             q_scale / k_scale enter through bmm1; vLLM forward_mqa
 *             multiplies bmm1 by q_scale * k_scale); QK^T then runs on the
 *             fp8 matrix cores with fp32 accumulation (P.V stays bf16).  Needs
 *             the fp8 cache (MLA_ERR_BAD_DTYPE otherwise) and the paged layout
 *             (MLA_ERR_BAD_SHAPE with sparse_top_k).
 * All pointers must be 4-byte aligned and stay valid until the enqueued work
 * completes; the library only reads them.
 */
typedef struct {
  const float* bmm1_scale;
  const float* bmm2_scale;
  const float* sinks;
  const int32_t* seq_lens_global;
  int32_t cp_world;
  int32_t cp_rank;
  int32_t sparse_top_k;
  int32_t q_fp8;
} mla_decode_options_t;

/*
 * mla_decode_paged_ex -- mla_decode_paged with device-resident options.
 * Arguments as mla_decode_paged; opts may be NULL (then identical to it).
 * Same workspace, same errors, plus MLA_ERR_MISALIGNED for an option pointer
 * that is not 4-byte aligned, MLA_ERR_BAD_SHAPE for cp_world < 1 or cp_rank
 * outside [0, cp_world), a negative sparse_top_k, sparse_top_k above
 * MLA_MAX_TOP_K, total_q above MLA_MAX_BATCH in the sparse layout, or DCP and
 * sparse together, MLA_ERR_BAD_BLOCK_TABLE for block_table_stride <
 * sparse_top_k, and MLA_ERR_NULL_POINTER for DCP mode without lse.
 */
int mla_decode_paged_ex(const void* q, const void* kv_cache, const int32_t* block_tables,
                        const int32_t* seq_lens, const int32_t* qo_indptr, int32_t max_seq_len,
                        int32_t max_q_len, float bmm1_scale, float bmm2_scale, int causal, void* out,
                        float* lse, void* workspace, size_t workspace_bytes,
                        const mla_decode_dims_t* dims, void* stream, const mla_decode_options_t* opts);

/*
 * mla_merge_partials -- combine G partial results of the same (row, head)
 * items, e.g. the sequence shards of DCP mode after an all-to-all:
 * M = max_g lse_g, w_g = exp(lse_g - M), out = sum_g w_g out_g / sum_g w_g and
 * lse = M + ln sum_g w_g (vLLM docs, "FlashInferMLAImpl": the natural-log LSE
 * DCP consumes).  Items whose partials all have lse = -inf get out = 0 and
 * lse = -inf.  The order of summation is fixed (g ascending).
 *
 * outs     device bf16 [G][items][512], 16-byte aligned (items = rows x heads)
 * lses     device float32 [G][items], 4-byte aligned
 * out      device bf16 [items][512], 16-byte aligned; written completely
 * lse      device float32 [items], or NULL
 * Asynchronous on `stream`; allocates nothing.  Returns MLA_OK,
 * MLA_ERR_NULL_POINTER, MLA_ERR_MISALIGNED, MLA_ERR_BAD_SHAPE (G < 1 or
 * items < 1) or MLA_ERR_HIP.
 */
int mla_merge_partials(const void* outs, const float* lses, int32_t num_partials, int64_t items, void* out,
                       float* lse, void* stream);

/*
 * Bytes of workspace mla_decode_paged needs for this shape on the current
 * device (depends on its compute-unit count).  Returns 0 for a shape that
 * mla_decode_paged would reject.  want_lse is accepted for symmetry; the size
 * does not depend on it.
 */
size_t mla_decode_paged_workspace_size(const mla_decode_dims_t* dims, int32_t max_seq_len,
                                       int32_t max_q_len, int want_lse);

/*
 * Bytes of workspace mla_decode_paged_ex needs with these options: the same as
 * mla_decode_paged_workspace_size() unless opts selects the sparse top-k
 * layout, where the size depends on dims (total_q, num_heads) and
 * opts->sparse_top_k only.  Returns 0 for a shape the call would reject.
 */
size_t mla_decode_paged_ex_workspace_size(const mla_decode_dims_t* dims, int32_t max_seq_len, int32_t max_q_len,
                                          int want_lse, const mla_decode_options_t* opts);

/*
 * Bits of the word mla_decode_check_contract writes; 0 means the checked part
 * of the contract holds.
 */
#define MLA_CONTRACT_SEQ_LEN (1u << 0)  /* some seq_lens[b] < 1 or > max_seq_len */
#define MLA_CONTRACT_QO_START (1u << 1) /* qo_indptr[0] != 0 */
#define MLA_CONTRACT_QO_ORDER (1u << 2) /* some qo_indptr[b + 1] <= qo_indptr[b] */
#define MLA_CONTRACT_QO_END (1u << 3)   /* qo_indptr[B] != total_q */
#define MLA_CONTRACT_Q_LEN (1u << 4)    /* some request has more than max_q_len query rows */
#define MLA_CONTRACT_CAUSAL (1u << 5)   /* causal, and some request has more query rows than seq_lens[b] */
#define MLA_CONTRACT_PAGE_ID (1u << 6)  /* a block-table entry a launch would read is < 0 or >= num_pages */

/*
 * mla_decode_check_contract -- a test and debugging aid, not part of the
 * decode path: checks on the device the part of a launch's contract that
 * lives in device memory (FlashInfer docs,
 * "prims_ts_batch_decode_with_kv_cache_mla", contract paragraph: positive
 * lengths no larger than the static bound, query offsets that start at 0,
 * increase strictly and end at total_q with steps no larger than max_q_len,
 * causal requests with no more query rows than cached rows, page ids inside
 * the cache).  mla_decode_paged never checks these; a violation there gives
 * undefined results.
 *
 * Arguments are those of mla_decode_paged with the same meaning (dims: batch,
 * q_len_fixed, total_q, page_size, num_pages and block_table_stride are used).
 * Reads seq_lens[0 .. B), qo_indptr[0 .. B] (if not NULL) and, of row b of
 * block_tables, entries 0 .. min(ceil(seq_lens[b] / page_size),
 * block_table_stride) - 1 only (the entries a launch reads).  Writes
 * result[0] = the OR of the MLA_CONTRACT_* bits violated and result[1] = 1 +
 * the lowest request index with a violation (0 if none); result is device
 * memory, 4-byte aligned, owned by the caller.  In the sequence-sharded mode
 * of mla_decode_paged_ex a local length of 0 is allowed but reads here as
 * MLA_CONTRACT_SEQ_LEN.  One workgroup, asynchronous on `stream`, allocates
 * nothing.  Returns MLA_OK, MLA_ERR_NULL_POINTER, MLA_ERR_MISALIGNED,
 * MLA_ERR_BAD_SHAPE (batch out of [1, MLA_MAX_BATCH], num_pages < 1,
 * block_table_stride < 1 or max_seq_len < 1), MLA_ERR_BAD_PAGE_SIZE,
 * MLA_ERR_BAD_Q_LEN (max_q_len < 1, total_q < 1, or a fixed launch with
 * q_len_fixed < 1) or MLA_ERR_HIP.
 */
int mla_decode_check_contract(const int32_t* block_tables, const int32_t* seq_lens, const int32_t* qo_indptr,
                              int32_t max_seq_len, int32_t max_q_len, int causal, const mla_decode_dims_t* dims,
                              uint32_t* result, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* mla_status_string(int status);

/* Size of the library's own per-device workspace used by mla_decode_paged_noalloc. */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * mla_decode_paged_noalloc -- mla_decode_paged for callers that cannot
 * allocate: code under HIP graph capture that may not call hipMalloc, tight
 * serving loops, harnesses that forbid allocation.  Same arguments, meaning,
 * layouts, kernels and results as mla_decode_paged, minus the workspace: the
 * call uses instead a workspace the library holds in device memory, a
 * MLA_NOALLOC_SCRATCH_BYTES array on each device it runs on, kept until the
 * process ends.  It allocates nothing and frees nothing.
 *
 * The first call on a device looks up that device's copy of the array (call
 * once before capturing a graph).  Every call on one device shares that
 * device's array: calls that overlap on one device (concurrent streams,
 * graphs replayed concurrently) race and give undefined results; calls
 * ordered on one stream are safe.  The array needs no initialisation and
 * holds nothing between calls.
 * Returns what mla_decode_paged returns, or MLA_ERR_SCRATCH_TOO_SMALL (nothing
 * enqueued) when mla_decode_paged_workspace_size() for this shape exceeds
 * MLA_NOALLOC_SCRATCH_BYTES.
 */
int mla_decode_paged_noalloc(const void* q, const void* kv_cache, const int32_t* block_tables,
                             const int32_t* seq_lens, const int32_t* qo_indptr, int32_t max_seq_len,
                             int32_t max_q_len, float bmm1_scale, float bmm2_scale, int causal, void* out,
                             float* lse, const mla_decode_dims_t* dims, void* stream);

/*
 * Test hook, not part of the serving interface: override the persistent grid
 * size (workgroups) used to split work, 0 restores the default (one workgroup
 * per compute unit).  Changes how KV ranges are split and merged, never the
 * result beyond rounding.  Affects later calls and workspace sizes on every
 * device; not thread-safe against concurrent launches.
 */
void mla_decode_internal_set_grid_override(int32_t grid);

/*
 * Tuning hook, not part of the serving interface: the work split gives every
 * workgroup an equal share of (tiles + segment starts x cost), where a segment
 * is one workgroup's contiguous run of 32-row KV tiles of one 128-pair unit and
 * its start (query load, first tiles in flight, partial-output store) is
 * charged `tiles` tile-equivalents.  Negative restores the defaults (8; 4 in
 * the sparse top-k layout); values are capped at 256.  Changes how KV ranges are split and merged, never the
 * result beyond rounding.  Affects later calls on every device; not thread-safe
 * against concurrent launches.
 */
void mla_decode_internal_set_segment_cost(int32_t tiles);

/*
 * Tuning hook, not part of the serving interface: with enable != 0 (the
 * default), a launch whose requests all hold the same number U = 2, 4 or 8 of
 * 128-pair units (ceil(q_b x num_heads / 128); fixed-shape or packed), on a
 * grid whose workgroups per XCD are a multiple of U, hands each request's
 * tiles to a group of U workgroups on one XCD that walk them together, one
 * unit each, so that a KV tile is fetched from memory once per group and the
 * other reads hit L2.  The kernel decides this on the device from the
 * lengths.  0 always splits unit by unit; the sparse top-k layout never
 * groups.  Changes how KV ranges are split and merged, never the result
 * beyond rounding.  Affects later calls on every device; not thread-safe
 * against concurrent launches.
 */
void mla_decode_internal_set_work_groups(int32_t enable);

/*
 * Measurement hook, not part of the serving interface: when start_event and
 * stop_event are non-NULL, later mla_decode_paged calls record start_event (a
 * hipEvent_t) on their stream right before their first kernel and stop_event
 * right after their last one, so a caller can time the whole launch on the
 * stream it runs on; decode_event, if non-NULL, is recorded right after the
 * decode kernel (before a separate split merge, where there is one).  NULL
 * start or stop turns it off.  The events stay owned by the caller.
 */
void mla_decode_internal_set_kernel_events(void* start_event, void* decode_event, void* stop_event);

/*
 * Test hook, not part of the serving interface: widen n_groups x 8 fp8 E4M3FN
 * codes (device, 8-byte aligned) to bf16 (device, 16-byte aligned) with the
 * exact conversion the decode kernel applies to an fp8 cache, on `stream`.
 * Returns MLA_OK, MLA_ERR_NULL_POINTER, MLA_ERR_MISALIGNED or MLA_ERR_HIP.
 */
int mla_decode_internal_fp8_to_bf16(const void* in, void* out, int64_t n_groups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
