/*
 * pa.h -- C ABI of libpa: paged GQA attention at head_dim 512 for MI355X (gfx950).
 *
 * Operations (each cites the page that defines it):
 *
 *  - Paged decode: one query token per request attends the request's KV, read through a
 *    page table from the combined HND cache [num_pages, 2, num_kv_heads, page_size,
 *    head_dim] ("[None][feat] Run Gemma4 head_dim 512 attention on Triton", TensorRT-LLM
 *    pull request 17772, section "Approach"), split along the key axis and merged by
 *    log-sum-exp (same page, section "Not covered": split-K workspaces), with sliding
 *    windows and FP8 KV cast on load (same page, sections "Approach" and "Test Coverage").
 *  - Paged prefill: causal attention of the new tokens over the cached prefix and
 *    themselves (same page, section "Approach"; section "Not covered" for the current
 *    tokens versus the prefix), including head_dim_qk = 512 with head_dim_vo = 256 over
 *    separately allocated K and V pools ("feat(attention): asymmetric VO-split NVFP4 paged
 *    prefill (qk=512/vo=256) for Gemma-4 on SM120/121", FlashInfer pull request 3684,
 *    sections "Summary" and "What's in it").
 *  - NVFP4 KV (decode and prefill): packed E2M1 pairs with one FP8 block scale per 16 head_dim
 *    elements of a token, the scales in a tensor of their own laid out like the data (the
 *    FlashInfer page, sections "Summary", "What's in it" and "NVFP4 split-KV correctness
 *    (added)"), dequantised on load.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless the parameter name ends in _host.  The library
 *    never allocates memory and never frees what it is given; every pointer is borrowed
 *    for the duration of the call (for enqueuing calls: until the stream reaches the
 *    enqueued work).
 *  - Every call returns a pa_status.  On an error nothing is enqueued and no output is
 *    written; pa_last_error() then returns a message naming the argument at fault
 *    (thread-local, valid until the next failing call on the same thread).  An input the
 *    library does not implement is refused with an error instead of being computed
 *    wrongly (the rule both pages follow: the Triton page's section "Not covered", and the
 *    FlashInfer page's commit on unequal K/V strides).
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.  Enqueuing
 *    calls do not synchronise.
 *  - Element strides are in elements of the stored type; the innermost (head_dim) stride
 *    is 1.  Base pointers and strides must keep every 16-byte vector load aligned.  NVFP4
 *    data and block-scale strides are in bytes (one data byte holds two elements).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,          /* malformed metadata, mismatched sizes, null pointers */
  PA_ERR_UNSUPPORTED = 2,          /* a valid request this library does not implement   */
  PA_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace or plan buffer below the planned size     */
  PA_ERR_HIP = 4                   /* a HIP runtime call failed                           */
} pa_status;

typedef enum {
  PA_DTYPE_BF16 = 0,
  PA_DTYPE_FP32 = 1,
  PA_DTYPE_FP8_E4M3FN = 2,         /* OCP E4M3FN: bias 7, max 448, NaN only at S.1111.111 */
  PA_DTYPE_NVFP4 = 3               /* KV only: two OCP E2M1 values per byte (element 2i in the
                                      low nibble, 2i+1 in the high one) and one E4M3FN block
                                      scale per 16 head_dim elements of a token            */
} pa_dtype;

/* One paged KV cache.  K and V may be two halves of the combined HND cache or two
 * separate pools with their own strides and widths (the FlashInfer page's commit that
 * tests the asymmetric prefill over separately allocated K and V pools whose strides
 * differ).  Element (page, head, slot, d) of K is at
 *   k + page*k_stride_page + head*k_stride_head + slot*k_stride_token + d
 * and likewise for V.  For FP8 the stored code c stands for e4m3fn(c) * k_scale (or
 * v_scale); bf16 caches use scales of 1.
 *
 * NVFP4: byte (page, head, slot, i) of K is at k + page*k_stride_page + head*k_stride_head
 * + slot*k_stride_token + i and holds elements 2i and 2i+1; the block scale of elements
 * 16j..16j+15 is byte k_sf + page*k_sf_stride_page + head*k_sf_stride_head +
 * slot*k_sf_stride_token + j, an E4M3FN code.  Element value = e2m1(nibble) *
 * e4m3fn(block scale) * k_scale (k_scale is the tensor-wide second-level scale); likewise
 * for V.  Data and scale tensors, and their strides, must be 16-byte aligned.  The block
 * scales are read through the same page table as the data, so a split of the key axis
 * never cuts a scale block (they run along head_dim).  Other dtypes leave the k_sf / v_sf
 * fields zero. */
typedef struct pa_kv_cache {
  const void* k;
  const void* v;
  int32_t kv_dtype;                /* PA_DTYPE_BF16, PA_DTYPE_FP8_E4M3FN or PA_DTYPE_NVFP4 */
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t page_size;               /* tokens per page, >= 1 */
  int32_t head_dim_qk;
  int32_t head_dim_vo;
  int64_t k_stride_page, k_stride_head, k_stride_token;
  int64_t v_stride_page, v_stride_head, v_stride_token;
  float k_scale;
  float v_scale;
  const void* k_sf;                /* NVFP4 block scales of K (uint8 E4M3FN), else NULL */
  const void* v_sf;
  int64_t k_sf_stride_page, k_sf_stride_head, k_sf_stride_token;  /* bytes */
  int64_t v_sf_stride_page, v_sf_stride_head, v_sf_stride_token;
} pa_kv_cache;

/* Page table, as the FlashInfer decode plan slices it (Triton page, section "Approach"):
 * request b owns pages kv_indices[kv_indptr[b] .. kv_indptr[b+1]) in logical order; all
 * are full except the last, which holds kv_last_page_len[b] tokens (1..page_size; an
 * exact multiple of the page size has a last page length of page_size).  Logical token t
 * of request b is slot t % page_size of page kv_indices[kv_indptr[b] + t / page_size].
 * All three arrays are device int32. */
typedef struct pa_page_table {
  const int32_t* kv_indptr;        /* [batch + 1], kv_indptr[0] == 0, non-decreasing */
  const int32_t* kv_indices;       /* [kv_indptr[batch]], each in [0, num_pages)      */
  const int32_t* kv_last_page_len; /* [batch]                                         */
  int32_t batch;
} pa_page_table;

typedef struct pa_attn_params {
  int32_t num_qo_heads;            /* multiple of num_kv_heads; query head h reads KV head
                                      h / (num_qo_heads / num_kv_heads)                  */
  float sm_scale;                  /* scores are sm_scale * q.k (e.g. 1/sqrt(head_dim_qk));
                                      any finite value: 0 weighs every visible key the same,
                                      a negative scale reverses the order of the scores   */
  int32_t window;                  /* > 0: a query at position p sees keys t > p - window;
                                      <= 0: no window                                      */
  int32_t causal;                  /* prefill: nonzero = causal; decode ignores it (the one
                                      query is the last position, so it is causal anyway) */
  int32_t q_dtype;                 /* PA_DTYPE_BF16 */
  int32_t out_dtype;               /* PA_DTYPE_FP32 or PA_DTYPE_BF16 (round to nearest even) */
} pa_attn_params;

/* Host-side plan: the partition of the work into items.  Plain data, owned by the
 * caller; filled by pa_decode_plan / pa_prefill_plan and read by the run calls, which
 * check that the sizes in it match their own arguments. */
typedef struct pa_plan {
  int32_t kind;                    /* 1 = decode, 2 = prefill                          */
  int32_t batch;
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t page_size;
  int32_t head_dim_qk;
  int32_t head_dim_vo;
  int32_t kv_dtype;
  int32_t window;
  int32_t causal;
  int32_t num_items;               /* decode: key segments; prefill: tiles and key chunks
                                      (one workgroup per (item, kv head))               */
  int32_t num_slots;               /* partial-result slots in the workspace             */
  int32_t num_merges;              /* decode: (request, kv head) pairs the merge writes;
                                      prefill: split tiles                              */
  int32_t block_tokens;            /* decode: key block of the partition (16)           */
  int32_t chunk_blocks;            /* decode: longest wave, in blocks; prefill: chunk
                                      length in 32-key stages (0: no split)             */
  int32_t num_splits;              /* decode: split-K chunk count (0 = no chunk cuts)    */
  int32_t tile_rows;               /* prefill: query rows (token, head) per tile        */
  int32_t total_q;                 /* prefill: number of query tokens                   */
  int32_t max_kv_len;
  int32_t num_workers;             /* decode: waves the partial kernel launches         */
  int32_t deferred_partials;       /* decode: 1 when a wave keeps the split result of a
                                      non-final segment in LDS and stores it after its
                                      last segment (the planner sets it when at least a
                                      quarter of the waves have such a segment); a speed
                                      choice only: either value gives the same bits      */
  int32_t short_tiles;             /* prefill: 1 when tiles too short to give each of the
                                      eight 16-row waves rows hold at least an eighth of
                                      the wave-stages (the planner sets it); the run then
                                      launches the kernel form whose waves without rows
                                      only copy stages; a speed choice only: either value
                                      gives the same bits                                */
  int32_t grouped_partials;        /* decode: 1 when the split results of neighbouring
                                      waves of one workgroup that belong to one (request,
                                      kv head) are combined in LDS into one slot (the
                                      planner sets it where the kernel can hold a split
                                      result per wave in LDS); changes rounding order only */
  int32_t staged_pages;            /* prefill, NVFP4 KV: page-table entries whose K and V
                                      pages the run first widens to bf16 in the workspace
                                      (0: none); the result is the same                  */
  int64_t plan_bytes;              /* bytes of the host plan buffer in use              */
  int64_t items_offset;            /* byte offset of the item array in the plan buffer  */
  int64_t merges_offset;           /* byte offset of the merge array in the plan buffer */
  int64_t workers_offset;          /* decode: byte offset of the further segments (the
                                      head segment of each wave comes first)            */
  int64_t partial_o_offset;        /* byte offset of partial outputs in the workspace   */
  int64_t partial_lse_offset;      /* byte offset of partial lse in the workspace       */
  int64_t workspace_bytes;         /* device workspace the run call needs               */
  int64_t staged_offset;           /* prefill: byte offset of the widened pages in the
                                      workspace (bf16 K, then bf16 V, [entry][kv head]
                                      [slot][head_dim], then one int32 per entry)        */
} pa_plan;

/* Fills *out for the combined HND cache [num_pages, 2, num_kv_heads, page_size, head_dim]
 * at `base` (K = index 0 of the "2" axis, V = index 1), contiguous, both widths equal to
 * head_dim.  Pure host arithmetic; `base` is not dereferenced. */
pa_status pa_kv_cache_hnd(const void* base, int32_t kv_dtype, int32_t num_pages,
                          int32_t num_kv_heads, int32_t page_size, int32_t head_dim,
                          float k_scale, float v_scale, pa_kv_cache* out);

/* Fills *out for two contiguous pools K [num_pages, num_kv_heads, page_size, head_dim_qk]
 * and V [num_pages, num_kv_heads, page_size, head_dim_vo] sharing one page table. */
pa_status pa_kv_cache_separate(const void* k, const void* v, int32_t kv_dtype,
                               int32_t num_pages, int32_t num_kv_heads, int32_t page_size,
                               int32_t head_dim_qk, int32_t head_dim_vo, float k_scale,
                               float v_scale, pa_kv_cache* out);

/* NVFP4 combined cache: data [num_pages, 2, num_kv_heads, page_size, head_dim / 2] at
 * `data` and block scales [num_pages, 2, num_kv_heads, page_size, head_dim / 16] at `sf`
 * (K = index 0 of the "2" axis, V = index 1), both contiguous uint8.  Pure host
 * arithmetic; no pointer is dereferenced. */
pa_status pa_kv_cache_nvfp4_hnd(const void* data, const void* sf, int32_t num_pages,
                                int32_t num_kv_heads, int32_t page_size, int32_t head_dim,
                                float k_scale, float v_scale, pa_kv_cache* out);

/* NVFP4 separate pools: K data [num_pages, num_kv_heads, page_size, head_dim_qk / 2] and
 * block scales [..., head_dim_qk / 16], likewise V with head_dim_vo, all contiguous. */
pa_status pa_kv_cache_nvfp4_separate(const void* k, const void* v, const void* k_sf,
                                     const void* v_sf, int32_t num_pages,
                                     int32_t num_kv_heads, int32_t page_size,
                                     int32_t head_dim_qk, int32_t head_dim_vo, float k_scale,
                                     float v_scale, pa_kv_cache* out);

/* Checks host copies of a page table: kv_indptr[0] == 0 and non-decreasing, every index
 * in [0, num_pages), every last page length in [1, page_size] for a non-empty request.
 * kv_indices_host may be NULL to skip the index range check.  Never calls HIP. */
pa_status pa_validate_page_table_host(const int32_t* kv_indptr_host,
                                      const int32_t* kv_indices_host,
                                      const int32_t* kv_last_page_len_host, int32_t batch,
                                      int32_t num_pages, int32_t page_size);

/* Plans a decode batch from host copies of kv_indptr and kv_last_page_len (the device
 * copies passed to pa_paged_decode must hold the same values).  The split of the key axis
 * into chunks merged by log-sum-exp is flash-decoding (the Triton page, sections
 * "Approach" and "Not covered"; the FlashInfer page, section "NVFP4 split-KV correctness
 * (added)", on split-KV for a short query over a long cache); a plan made once on the host
 * and run many times is the plan()/run() split of the FlashInfer page's commits.  The
 * result does not depend on the partition.  The work is the set of
 * (request, kv head, 16-token key block) units; each wave of the partial kernel runs one
 * piece of them: the units, flattened in (request, kv head, block) order, are cut into
 * P near-equal pieces, at most one wave per SIMD slot of the 256 CUs at two waves per SIMD
 * (2048): with P0 = min(2048, ceil(units / 8)) and m = ceil(units / P0) the largest piece,
 * P = ceil(units / m), so (nearly) every wave streams m blocks.  A piece is cut at
 * (request, kv head) boundaries into segments.  num_splits S > 0 (split-K S) also cuts
 * each (request, kv head) at the boundaries of its min(S, blocks) near-equal chunks, so
 * every chunk is computed by whole segments; S == 0 adds no cuts.  A (request, kv head)
 * with several segments is merged by log-sum-exp weights (the result does not depend on
 * the cuts).  Waves run longest first.  Call with plan_buf_host == NULL to
 * learn plan->plan_bytes (and plan->workspace_bytes); then call again with a buffer of
 * at least that size.
 * Supported: head dims (512,512), (256,256), (512,256); kv bf16, FP8 E4M3FN or NVFP4;
 * q bf16; out fp32 or bf16; 1 <= num_qo_heads / num_kv_heads <= 8; num_splits <= 64.
 * Never calls HIP. */
pa_status pa_decode_plan(const pa_attn_params* params, const pa_kv_cache* cache,
                         const int32_t* kv_indptr_host, const int32_t* kv_last_page_len_host,
                         int32_t batch, int32_t num_splits, void* plan_buf_host,
                         size_t plan_buf_bytes, pa_plan* plan);

/* Plans a prefill batch (the Triton page, section "Approach": causal attention of the new
 * tokens over the paged cache, in one branch with decode; section "Not covered": the new
 * tokens versus the cached prefix).  qo_indptr_host [batch + 1] gives each request's new
 * tokens, which must not outnumber its KV tokens; row i of request b sits at key position
 * L_b - q_len_b + i.  Query rows of one (request, KV head) are the (token, head) pairs of
 * its head group, tiled in plan->tile_rows; a tile sees the keys some of its rows see.
 * Split-K for short queries over long KV: when tiles x num_kv_heads < 512, every tile
 * whose keys span more than C 32-key stages, C = max(8, ceil(total stages x num_kv_heads
 * / 512)), is cut into ceil(stages / C) near-equal runs of whole stages; each such chunk
 * writes a partial (normalised output and log-sum-exps) to its own workspace slot and a
 * merge combines them (plan->num_merges split tiles, plan->num_slots slots,
 * plan->chunk_blocks = C, 0 without splitting).  Items run by key count, longest first;
 * without split-K, when the K and V bytes of the requests' key ranges (all KV heads) exceed
 * 256 MiB, the GPU's memory-side last-level cache, they run request by request instead
 * (requests in the order of their longest tile, longest first within each request).
 * NVFP4 without split-K, when the tiles read each key of the table at least four times
 * on average: the run first widens every K and V page the table lists into bf16 pages
 * in the workspace (exact: each E2M1 value times its E4M3 block scale) and runs the bf16
 * kernel over them (plan->staged_pages, plan->staged_offset; the workspace grows by
 * 2 (head_dim_qk + head_dim_vo) bytes per (entry, kv head, slot)).
 * The result does not depend on the split, the order or the widening.  Same two-call sizing as pa_decode_plan.
 * Supported: head dims (512,512), (256,256), (512,256); kv bf16, FP8 E4M3FN or NVFP4; q bf16;
 * out fp32 or bf16; num_qo_heads / num_kv_heads <= 16.  Never calls HIP. */
pa_status pa_prefill_plan(const pa_attn_params* params, const pa_kv_cache* cache,
                          const int32_t* qo_indptr_host, const int32_t* kv_indptr_host,
                          const int32_t* kv_last_page_len_host, int32_t batch,
                          void* plan_buf_host, size_t plan_buf_bytes, pa_plan* plan);

/* Copies plan->plan_bytes from plan_buf_host to the start of the device workspace
 * (stream-ordered hipMemcpyAsync).  The workspace is preallocated by the caller and reused
 * by every run of the plan (the Triton page, section "Not covered", names per-call
 * workspace allocation as the cost to avoid).  The host buffer must stay unchanged until the copy
 * has run.  The run calls read the work items from there, so upload once per plan. */
pa_status pa_plan_upload(const pa_plan* plan, const void* plan_buf_host, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Enqueues one decode step (the Triton page, sections "Approach" and "Test Coverage":
 * single-token paged decode over the HND cache, split-K, with sliding windows and FP8 KV
 * cast on load; the FlashInfer page, section "Summary": head_dim_vo may differ from
 * head_dim_qk, with V in its own pool): q [batch, num_qo_heads, head_dim_qk] bf16 (contiguous) ->
 * out [batch, num_qo_heads, head_dim_vo] in params->out_dtype, and, if lse != NULL,
 * lse [batch, num_qo_heads] fp32 (natural log; -inf for a request with no keys, whose
 * output row is zero).  workspace: device buffer of at least plan->workspace_bytes
 * holding the uploaded plan; it also receives the split partials.  Launches the
 * split-K partial kernel and, when a request was split, the log-sum-exp merge kernel.
 * Concurrent calls sharing one workspace race. */
pa_status pa_paged_decode(const pa_plan* plan, const void* q, const pa_kv_cache* cache,
                          const pa_page_table* table, const pa_attn_params* params,
                          void* out, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream);

/* pa_paged_decode for callers that cannot allocate device memory (code under graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels and
 * results, with the workspace taken from a device array inside the library (64 MiB per
 * GPU, held from the library's load until the process ends) instead of the caller's.
 * Each call first copies plan->plan_bytes from plan_buf_host into that array
 * (stream-ordered; the host buffer must stay unchanged until the stream has reached the
 * call), then launches the partial and merge kernels.  Calls no allocator.  A plan whose
 * workspace_bytes exceeds 64 MiB is refused with PA_ERR_WORKSPACE_TOO_SMALL.  Every call
 * on one GPU shares that GPU's array: calls that overlap on one GPU (other streams, other
 * threads) race; calls on one stream are ordered. */
pa_status pa_paged_decode_static(const pa_plan* plan, const void* plan_buf_host, const void* q,
                                 const pa_kv_cache* cache, const pa_page_table* table,
                                 const pa_attn_params* params, void* out, float* lse,
                                 void* stream);

/* The two phases of pa_paged_decode as separate calls, with the same arguments and
 * checks, for callers that schedule or time them apart: _partial launches the split-K
 * kernel (requests with a single chunk get their final out/lse from it), _merge launches
 * the log-sum-exp merge of the split requests (nothing when the plan split none).  Calling
 * _partial then _merge on one stream equals pa_paged_decode. */
pa_status pa_paged_decode_partial(const pa_plan* plan, const void* q, const pa_kv_cache* cache,
                                  const pa_page_table* table, const pa_attn_params* params,
                                  void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream);
pa_status pa_paged_decode_merge(const pa_plan* plan, const void* q, const pa_kv_cache* cache,
                                const pa_page_table* table, const pa_attn_params* params,
                                void* out, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Enqueues one prefill (the Triton page, section "Approach": causal paged prefill, FP8 KV
 * cast on load in both phases; the FlashInfer page, sections "Summary" and "What's in it":
 * head_dim_qk 512 with head_dim_vo 256 over separate pools, NVFP4 KV): q [total_q,
 * num_qo_heads, head_dim_qk] bf16 (contiguous, ragged by qo_indptr) -> out [total_q,
 * num_qo_heads, head_dim_vo] in params->out_dtype and optional lse [total_q, num_qo_heads]
 * fp32 (NULL: not written).  qo_indptr is the device copy of the array
 * given to pa_prefill_plan.  One kernel launch, or two when the plan splits tiles (the
 * chunk partials go to the workspace, then a merge kernel writes their rows), or, when
 * the plan widens NVFP4 pages (plan->staged_pages > 0), the widening kernel first and
 * then the bf16 prefill kernel over the widened pages.  NVFP4 at 512/512 without widening
 * runs the 512/256 form twice, once per half of head_dim_vo. */
pa_status pa_paged_prefill(const pa_plan* plan, const void* q, const int32_t* qo_indptr,
                           const pa_kv_cache* cache, const pa_page_table* table,
                           const pa_attn_params* params, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Copies the stored K and V elements of (request, kv_head) in logical token order, through
 * the same address path as the attention kernels (page-table semantics of the Triton page,
 * section "Approach"): k_out [kv_len, head_dim_qk] and v_out [kv_len, head_dim_vo] in the
 * cache's element type; for NVFP4 each row is the packed data (head_dim / 2 bytes)
 * followed by its block-scale codes (head_dim / 16 bytes).  kv_len must equal the
 * request's length.  For bit-exact checks of the page-table handling. */
pa_status pa_debug_gather_kv(const pa_kv_cache* cache, const pa_page_table* table,
                             int32_t request, int32_t kv_len, int32_t kv_head, void* k_out,
                             void* v_out, void* stream);

/* Converts n FP8 E4M3FN codes to fp32 with the decode kernels' conversion (prefill widens
 * codes to bf16 with the FP8-to-bf16 conversion instruction; both are exact). */
pa_status pa_debug_fp8_to_f32(const uint8_t* codes, float* out, int32_t n, void* stream);

const char* pa_last_error(void);        /* thread-local message of the last failing call */
uint64_t pa_launch_count(void);         /* kernels launched by this process so far         */
uint64_t pa_debug_launch_count(void);   /* the same count, under its introspection name    */
const char* pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
