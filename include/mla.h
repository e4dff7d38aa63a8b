/*
 * mla.h — C ABI of the MI355X (gfx950) MLA decode library.
 *
 * Multi-head Latent Attention decode in its absorbed, MQA-like form over a paged latent KV cache
 * (vLLM mla_attention.py module docstring, "Data-Movement Friendly Approach": every head's query
 * [ql_nope, q_pe] attends over rows [kv_c, k_pe] shared by all heads, and kv_c also serves as V).
 * Three calls run in stream order, as in the FlashMLA wrapper (get_mla_metadata, then
 * flash_mla_with_kvcache) and HALOps (mla_attention_plan, mla_attention, then the split-KV
 * log-sum-exp combine of mla_output_proj):
 *
 *   mla_decode_plan  per-query-group split and work-unit metadata, computed on the device
 *   mla_decode       paged gather, QK^T, online softmax, PV; final O/LSE for groups processed in
 *                    one piece, split partials (bf16 O, fp32 LSE) for the others
 *   mla_combine      log-sum-exp merge of the partials (and the sink), final O/LSE
 *
 * and, before them in a layer, the write of the new tokens' rows into the cache:
 *
 *   mla_kv_write     each new token's [kv_c, k_pe] row written in place into its cache slot,
 *                    quantised to the fp8 row format when the cache holds fp8 rows
 *
 * and the per-head weight absorption on either side of the decode:
 *
 *   mla_q_absorb     the decode's query [q_nope x W_UK, q_pe] from the per-head query parts
 *   mla_v_up         the per-head output o x W_UV from the decode's latent output
 *
 * and, for caches whose sliding windows are given as lists of slots, their run-compressed form:
 *
 *   mla_swa_runs     each token's window of slots as at most two runs of consecutive slots
 *
 * and, for the chunked-context prefill, the gather of context rows into a bf16 workspace:
 *
 *   mla_plan_context_chunks  (host) the requests' context rows packed into workspace chunks
 *   mla_gather_context       rows of the requests of one context chunk, widened to bf16
 *
 * and the sparse prefill over index lists into a flat latent buffer, with each row's max logit:
 *
 *   mla_sparse_prefill       plan, decode and combine of the prefill tokens in one call
 *
 * Conventions shared by every call
 * - All pointers are device pointers unless a parameter says "host". The caller owns every buffer;
 *   the library never allocates, frees or synchronises. `stream` is a hipStream_t (NULL = default
 *   stream); all work is enqueued asynchronously on it, so the calls may be graph-captured.
 * - Return value: MLA_OK (0) or a positive mla_status. Argument checks run on the host before any
 *   launch; a failed check enqueues nothing. Launch failures are reported as MLA_ERR_LAUNCH.
 * - Query groups: without index lists a group is one request (R = q_len * num_heads stacked query
 *   rows, row r = t * num_heads + h); with index lists (topk > 0) a group is one (request, token)
 *   pair g = b * q_len + t (R = num_heads rows).
 * - Positions (vLLM MLACommonMetadata: seq_len = context_len + query_len): the q_len new tokens of
 *   request b are its last positions, token t at pos_t = seqlens[b] - q_len + t.
 * - Data contract (not checked): block-table entries of pages a request uses lie in
 *   [0, num_pages) — entries outside that range are read as zero rows instead of faulting, and the
 *   result is then unspecified; seqlens[b] <= max_pages_per_seq * page_size.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,       /* a required pointer is NULL                                      */
  MLA_ERR_SHAPE = 2,      /* batch/q_len/heads/dims out of range or unsupported              */
  MLA_ERR_FORMAT = 3,     /* kv_format unknown or inconsistent with the dims                 */
  MLA_ERR_PAGE = 4,       /* page_size not a power of two, or page stride too small/unaligned */
  MLA_ERR_MODE = 5,       /* unsupported mode combination (index lists with causal/window)   */
  MLA_ERR_WORKSPACE = 6,  /* plan or partial buffer smaller than mla_get_workspace_size says  */
  MLA_ERR_ALIGN = 7,      /* a pointer is not 16-byte aligned                                */
  MLA_ERR_DEVICE = 8,     /* HIP device query failed                                         */
  MLA_ERR_LAUNCH = 9,     /* a kernel launch failed                                          */
  MLA_ERR_SCRATCH = 10    /* mla_decode_noalloc: plan + partials exceed the static scratch   */
} mla_status;

typedef enum mla_kv_format {
  MLA_KV_BF16 = 0, /* page = page_size rows of d_qk bfloat16                                     */
  MLA_KV_FP8 = 1   /* page = page_size rows of [d_qk - d_rope e4m3fn][d_rope bfloat16], then
                      page_size 8-byte slots of ue8m0 scales, one per 64 NoPE values (HALOps
                      mla_attention kv_cache layout; 640-byte rows for d_qk 576, 576 for 512)   */
} mla_kv_format;

/* The problem statement (FlashMLA wrapper I/O contract: q [B, Sq, Hq, d], k_cache
 * (num_blocks, page_size, 1, d), block_table (B, max_blocks), cache_seqlens (B,), indices
 * (B, Sq, topk); HALOps: head dims 512/512 with 448 NoPE + 64 RoPE, sink, windows). */
typedef struct mla_problem {
  int32_t batch;             /* B >= 1                                                        */
  int32_t q_len;             /* Sq >= 1 query tokens per request                              */
  int32_t num_heads;         /* H >= 1 query heads (one shared latent KV head)                */
  int32_t d_qk;              /* 576 (DeepSeek-V3: 512 latent + 64 RoPE) or 512 (V4)            */
  int32_t d_v;               /* 512: V is the first 512 columns of each (dequantised) row      */
  int32_t d_rope;            /* 64                                                            */
  int32_t kv_format;         /* mla_kv_format                                                 */
  int32_t page_size;         /* rows per page, a power of two in [1, 4096]                    */
  int64_t page_stride_bytes; /* bytes between pages: multiple of 16, >= the page's used bytes */
  int64_t num_pages;         /* physical pages in kv_cache (>= 1)                             */
  int32_t max_pages_per_seq; /* row stride of block_table                                     */
  int32_t topk;              /* 0: dense; > 0: index lists of this width                      */
  int32_t causal;            /* 1: token t sees positions <= pos_t                            */
  int32_t window;            /* 0: none; W > 0: token t sees positions >= pos_t - W + 1       */
} mla_problem;

/* Buffer sizes for a problem planned over `num_cus` compute units (0: the current device's CU
 * count). plan_bytes (host out): the plan buffer for mla_decode_plan. partial_bytes (host out):
 * the split partials for mla_decode/mla_combine (bf16 [S_max][R][d_v] O, each split normalised by
 * its own softmax sum, then fp32 [S_max][R] LSE, S_max = groups + units). Either output pointer
 * may be NULL. */
int mla_get_workspace_size(const mla_problem* p, int32_t num_cus, size_t* plan_bytes,
                           size_t* partial_bytes);

/* Compute units of the current HIP device (host out). */
int mla_device_num_cus(int32_t* num_cus);

/* Plan (FlashMLA get_mla_metadata: tile scheduling metadata and split information; HALOps
 * mla_attention_plan: a per-forward work list shared by the layers of one kind). Reads seqlens
 * [B] int32 and, when topk > 0, the optional topk_lens [B * q_len] int32 (NULL: every token uses
 * topk entries) on the device and writes the int32 plan: a header, per-group split ranges,
 * per-unit split ranges, per-group (first row, row count), and split records (group, first block,
 * end block, unit), blocks being 64 consecutive effective rows; plus a zero row used for masked
 * rows and one 32-byte descriptor per split (group, request, first row, row count, request
 * length, range of 32-row steps, the group's split count) from which a decode workgroup starts
 * the split in one read. The plan stays valid until overwritten and may be reused by every layer
 * of a forward. */
int mla_decode_plan(const mla_problem* p, int32_t num_cus, const int32_t* seqlens,
                    const int32_t* topk_lens, void* plan, size_t plan_bytes, void* stream);

/* Decode (FlashMLA flash_mla_with_kvcache; HALOps mla_attention, attention part).
 *   q           bf16 [B, Sq, H, d_qk], contiguous (RoPE already applied to its last d_rope cols)
 *   kv_cache    paged rows in p->kv_format, page stride p->page_stride_bytes
 *   block_table int32 [B, max_pages_per_seq]
 *   seqlens     int32 [B] (the same array the plan read)
 *   sm_scale    softmax scale of the QK scores
 *   indices     int32 [B, Sq, topk] request-local positions when topk > 0, else NULL; entries
 *               outside [0, seqlens[b]) are skipped, repeats count once per occurrence
 *   sink        fp32 [H] per-head sink logits added once to each softmax denominator, or NULL
 *   plan        from mla_decode_plan with the same problem and num_cus
 *   partials    workspace of at least the partial_bytes mla_get_workspace_size gives
 *   out         bf16 [B, Sq, H, d_v]; lse fp32 [B, H, Sq] natural-log LSE of the scaled scores
 *               (sink included). Groups processed in one piece are written here; the rest are
 *               written by mla_combine, which must follow on the same stream. */
int mla_decode(const mla_problem* p, int32_t num_cus, const void* q, const void* kv_cache,
               const int32_t* block_table, const int32_t* seqlens, float sm_scale,
               const int32_t* indices, const float* sink, const void* plan, void* partials,
               size_t partial_bytes, void* out, float* lse, void* stream);

/* Combine (vLLM merge_attn_states; HALOps mla_output_proj, split-KV LSE combine): for every group
 * with a split count other than one, LSE = ln sum_i exp(LSE_i), O = sum_i exp(LSE_i - LSE) O_i,
 * then the sink; a group with no rows gets O = 0 and LSE = -inf (or LSE = sink_h). */
int mla_combine(const mla_problem* p, int32_t num_cus, const void* plan, const void* partials,
                size_t partial_bytes, const float* sink, void* out, float* lse, void* stream);

/* Allocation-free decode step, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): mla_decode_plan,
 * mla_decode and mla_combine enqueued in one call, with the plan and the split partials held in
 * the library's own static device scratch of 64 MiB per GPU (allocated with the library's code
 * object on each device it runs on, kept until the process ends) instead of caller buffers. The
 * arguments are those of the three calls it stands for (topk_lens as in mla_decode_plan); the
 * outputs equal theirs bit for bit. A problem whose plan (rounded up to 256 bytes) plus partial
 * bytes (mla_get_workspace_size) exceed 64 MiB is rejected with MLA_ERR_SCRATCH before anything is
 * enqueued. The call allocates and frees nothing. Every call on one GPU uses that GPU's one
 * scratch and the plan kernel rewrites all of it that the decode and combine read, so nothing has
 * to be cleared between calls; but calls whose work overlaps on one GPU (other streams, other
 * threads, or an earlier call's graph replay still running) race on the scratch and must be
 * ordered by the caller. */
int mla_decode_noalloc(const mla_problem* p, int32_t num_cus, const void* q, const void* kv_cache,
                       const int32_t* block_table, const int32_t* seqlens,
                       const int32_t* topk_lens, float sm_scale, const int32_t* indices,
                       const float* sink, void* out, float* lse, void* stream);

/* Cache write (vLLM mla_attention.py update_kv_cache(kv_c_normed, k_pe, kv_cache, slot_mapping,
 * ...); HALOps MLA API, mla_attention kv_cache: each token's new row is written in place).
 *   num_tokens   n >= 0 rows to write (0 enqueues nothing)
 *   kv_c         bf16 [n, d_qk - d_rope], contiguous: the latent (NoPE) part of each row
 *   k_pe         bf16 [n, d_rope], contiguous: the RoPE part (already rotated)
 *   slot_mapping int64 [n], 8-byte aligned: slot = physical page * page_size + row in the page;
 *                entries < 0 or >= num_pages * page_size are skipped. Slots must be distinct (two
 *                rows for one slot: which lands is unspecified).
 *   kv_cache     the paged cache in p->kv_format, p->page_stride_bytes, p->num_pages
 * Only the dims, format and page fields of p are used (the rest must still be valid).
 * bf16 rows are stored as given. fp8 rows: per 64-value group of kv_c, the ue8m0 scale byte is
 * 127 + k for the smallest integer k with max|x| <= 448 * 2^k (k clamped to [-127, 127]; 127 for an
 * all-zero group), and each code is x * 2^-k rounded to the nearest e4m3fn value, ties to even;
 * k_pe is stored as bf16; unused bytes of the row's 8-byte scale slot are written as zero. Inputs
 * must be finite. Other rows of the cache are not touched. */
int mla_kv_write(const mla_problem* p, int64_t num_tokens, const void* kv_c, const void* k_pe,
                 const int64_t* slot_mapping, void* kv_cache, void* stream);

/* Query absorption (vLLM mla_attention.py forward_mqa: ql_nope = q_nope x W_UK_T per head; module
 * docstring, "Data-Movement Friendly Approach"), fused with assembling the decode's query:
 *   q_out[t, h, 0:d_latent]              = sum_p q_nope[t, h, p] * w_uk[h, l, p]
 *   q_out[t, h, d_latent:d_latent+d_rope] = q_pe[t, h, :]
 *   tokens  T >= 0 query tokens (B * Sq of the decode; 0 enqueues nothing)
 *   q_nope  bf16 [T, H, d_nope]; d_nope a multiple of 32 (128 for DeepSeek-V3)
 *   q_pe    bf16 [T, H, d_rope] (already rotated), or NULL when d_rope = 0; d_rope a multiple of 8
 *   w_uk    bf16 [H, d_latent, d_nope]: per head, each latent column's d_nope weights contiguous
 *           (w_uk[h, l, p] = W_UK[l, h, p] of the (L, N, P) weight); d_latent a multiple of 64
 *   q_out   bf16 [T, H, d_latent + d_rope]: the q argument of mla_decode when T = B * Sq
 * All pointers 16-byte aligned. bf16 inputs, fp32 accumulation, bf16 output rounded to nearest even. */
int mla_q_absorb(int32_t tokens, int32_t num_heads, int32_t d_nope, int32_t d_latent,
                 int32_t d_rope, const void* q_nope, const void* q_pe, const void* w_uk, void* q_out,
                 void* stream);

/* Value up-projection (vLLM mla_attention.py _v_up_proj: (N, B, L) x (N, L, V) per head):
 *   out[t, h, v] = sum_l o[t, h, l] * w_uv[h, v, l]
 *   o     bf16 [T, H, d_latent] (the out argument of mla_decode); d_latent a multiple of 32
 *   w_uv  bf16 [H, d_v, d_latent]: per head, each value column's d_latent weights contiguous
 *         (w_uv[h, v, l] = W_UV[l, h, v] of the (L, N, V) weight); d_v a multiple of 64
 *   out   bf16 [T, H, d_v]
 * All pointers 16-byte aligned; fp32 accumulation, bf16 output rounded to nearest even. */
int mla_v_up(int32_t tokens, int32_t num_heads, int32_t d_latent, int32_t d_v, const void* o,
             const void* w_uv, void* out, void* stream);

/* Run-compressed sliding windows (HALOps MLA API, mla_attention_plan). With s_g the slot of window
 * row g, rows g - 1 and g belong to one run iff s_g == s_{g-1} + kv_run_step and
 * floor(s_g / page_size) == floor(s_{g-1} / page_size). A window is described by its runs when it
 * has at most two; otherwise (a padding or not yet written window) only by its row 0.
 *   tokens        T >= 0 (0 enqueues nothing); topk >= 1 columns per window
 *   kv_indices    int32 [T, topk]: the cache slots of each token's window rows, in row order;
 *                 columns past the token's length are ignored
 *   topk_lengths  int32 [T] rows per window (clamped to [0, topk]), or NULL for topk rows
 *   page_size     rows per cache page, a power of two; page of a slot = floor(slot / page_size)
 *   kv_run_step   1 or -1: the slot step between consecutive rows of a run
 *   runs          int32 [T, 4], 16-byte aligned (out): (slot0, len0, slot1, rows); rows g < len0 at
 *                 slot0 + kv_run_step * g, the others at slot1 + kv_run_step * (g - len0); slot1 = -1
 *                 when len0 = rows; an empty window gives (-1, 0, -1, 0) and a cut one
 *                 (slot of row 0, 1, -1, 1). */
int mla_swa_runs(int32_t tokens, int32_t topk, const int32_t* kv_indices,
                 const int32_t* topk_lengths, int32_t page_size, int32_t kv_run_step, int32_t* runs,
                 void* stream);

/* Chunked-context plan, on the host: this library's own packing of the requests' context rows into
 * chunks of at most W workspace rows (chunked context gathering is motivated by the vLLM
 * mla_attention.py module docstring, the chunked prefill approach; the planner that page prints
 * makes different plans and is not the one implemented here). Requests are packed in order, so a
 * chunk covers a contiguous run of requests and no empty span. A chunk takes whole remainders of requests while
 * they fit; when the next does not, it takes that remainder's longest prefix that fits and whose
 * length is a multiple of `alignment`, then closes. Requests without context rows are in no chunk.
 *   num_reqs, context_lens (host int32 [num_reqs]; values < 0 count as 0)
 *   workspace_rows W >= alignment >= 1 (e.g. page_size, so that every span starts page-aligned)
 *   max_chunks, max_spans   capacities of the outputs (num_reqs + total / (W - W mod alignment) + 1
 *                           chunks and num_reqs + chunks spans suffice)
 *   num_chunks (host out); chunk_ptr (host out, [num_chunks + 1]): the spans of chunk c are
 *   [chunk_ptr[c], chunk_ptr[c + 1]); span_req, span_start, span_len (host out): request, first
 *   context row and rows of each span, in request order (a chunk's requests are a run of the
 *   requests without the empty ones). A chunk's spans map to one mla_gather_context call:
 *   num_reqs = its span count, block_table = the block-table rows of the spans' requests in span
 *   order, seq_starts = span_start, cu_seq_lens = prefix sums of span_len.
 * Returns MLA_ERR_SHAPE for invalid sizes, MLA_ERR_WORKSPACE if a capacity is exceeded. */
int mla_plan_context_chunks(int32_t num_reqs, const int32_t* context_lens, int64_t workspace_rows,
                            int32_t alignment, int32_t max_chunks, int32_t max_spans,
                            int32_t* num_chunks, int32_t* chunk_ptr, int32_t* span_req,
                            int32_t* span_start, int32_t* span_len);

/* Context gather (vLLM mla_attention.py _compute_prefill_context: gather_and_maybe_dequant_cache
 * with cu_seq_lens, token_to_seq and seq_starts): output row i is row
 * j = seq_starts[r] + i - cu_seq_lens[r] of request r = token_to_seq[i], read through block_table
 * row r, as bf16. fp8 rows are widened exactly (e4m3 value times its group's ue8m0 scale; RoPE tail
 * as stored); bf16 rows are copied.
 *   p             the cache's problem (dims, format, page fields, max_pages_per_seq are used)
 *   num_reqs      requests of the chunk (rows of block_table, entries of seq_starts)
 *   num_rows      output rows n >= 0 (0 enqueues nothing)
 *   block_table   int32 [num_reqs, max_pages_per_seq]
 *   cu_seq_lens   int32 [num_reqs + 1]: output rows of request r are [cu_seq_lens[r], cu_seq_lens[r+1])
 *   seq_starts    int32 [num_reqs]: first logical row of each request's span, or NULL for 0
 *   token_to_seq  int32 [n]: request of each output row
 *   dst           bf16 [n, d_qk], 16-byte aligned
 * Rows whose position or page falls outside the block table or the cache are written as zeros.
 * Indices into cu_seq_lens / seq_starts / block_table must be valid (token_to_seq < num_reqs). */
int mla_gather_context(const mla_problem* p, int32_t num_reqs, int64_t num_rows,
                       const int32_t* block_table, const int32_t* cu_seq_lens,
                       const int32_t* seq_starts, const int32_t* token_to_seq, const void* kv_cache,
                       void* dst, void* stream);

/* Sparse prefill (FlashMLA wrapper, flash_mla_sparse_fwd(q, kv, indices, sm_scale, d_v = 512)
 * returning out, max_logits and lse): each of s_q prefill tokens attends, with all of its heads,
 * over the rows of one flat latent buffer that its own index list names. For token t and head h,
 * over the entries j of indices[t, :] in [0, s_kv) (repeats count once per occurrence):
 *   s_j = sm_scale * <q[t, h, :], kv[j, :]>,  max_logits = max s_j,  LSE = ln sum exp(s_j),
 *   out = sum exp(s_j - LSE) kv[j, 0:512];  no valid entry: out = 0, max_logits = LSE = -inf.
 *   s_q          1 <= s_q <= 8192 query tokens (larger prefills are issued in several calls)
 *   num_heads    H >= 1 query heads; every head of a token reads each gathered row once per
 *                64-head tile
 *   d_qk         576 (DeepSeek-V3: 512 latent + 64 RoPE) or 512 (V4)
 *   topk         >= 1 index entries per token; s_kv: 1 <= rows of kv <= INT32_MAX
 *   q            bf16 [s_q, H, d_qk]; kv bf16 [s_kv, d_qk] contiguous (one latent KV head)
 *   indices      int32 [s_q, topk]; entries outside [0, s_kv) (-1 padding) name no row
 *   workspace    at least mla_sparse_prefill_workspace_size bytes, 16-byte aligned, owned by the
 *                caller; it holds the request metadata, the plan and the split partials
 *   out          bf16 [s_q, H, 512]; max_logits and lse fp32 [H, s_q] (the decode's LSE layout
 *                [B, H, Sq] with one batch), natural-log units of the scaled scores
 * The call enqueues a metadata fill, mla_decode_plan, mla_decode and mla_combine on `stream`; it
 * runs the prefill as one request of q_len = s_q tokens whose positions are kv's rows (pages of
 * 4096 rows, page i at page i). q, kv, workspace and out 16-byte aligned. */
int mla_sparse_prefill_workspace_size(int32_t s_q, int32_t num_heads, int32_t d_qk, int32_t topk,
                                      int64_t s_kv, int32_t num_cus, size_t* workspace_bytes);
int mla_sparse_prefill(int32_t s_q, int32_t num_heads, int32_t d_qk, int32_t topk, int64_t s_kv,
                       int32_t num_cus, const void* q, const void* kv, const int32_t* indices,
                       float sm_scale, void* workspace, size_t workspace_bytes, void* out,
                       float* max_logits, float* lse, void* stream);

/* Static description of a status code. */
const char* mla_strerror(int status);

/* Static string identifying the sources the library was built from: 16 hex digits of the SHA-256
 * of the HIP sources, internal headers and this header, computed by the build ("unknown" when
 * built without it). A caller compares it with the same hash of the sources it expects. */
const char* mla_build_id(void);

/* Checked mode (the data contract of mla_decode made visible). With checks on, every mla_decode,
 * mla_decode_noalloc and mla_sparse_prefill call first runs a validation kernel on its stream that
 * sets bits of a per-device word, instead of the decode silently reading zero rows:
 *   MLA_CHECK_PAGE    a block-table entry outside [0, num_pages) for a page holding a row the
 *                     call attends to (dense: the request's rows or its window's; index lists:
 *                     a listed position in [0, L) within the token's row count)
 *   MLA_CHECK_LENGTH  such a row past the block table (page index >= max_pages_per_seq)
 *   MLA_CHECK_PLAN    a plan whose header does not describe the problem and CU count
 * The decode itself runs unchanged. mla_check_enable sets the process-wide switch (default off;
 * returns MLA_OK). mla_check_status waits for the stream's work, writes the current device's bits
 * to *bits (host pointer) and clears them when clear != 0; MLA_ERR_NULL for a NULL bits,
 * MLA_ERR_DEVICE if the read fails. Calls that overlap on one device share its word. */
enum { MLA_CHECK_PAGE = 1, MLA_CHECK_LENGTH = 2, MLA_CHECK_PLAN = 4 };
int mla_check_enable(int32_t on);
int mla_check_status(uint32_t* bits, int32_t clear, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
