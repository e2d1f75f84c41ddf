/*
 * pkb.h -- C ABI of libpkb.so: scaled-dot-product attention over a paged KV
 * cache on AMD Instinct MI355X (gfx950).
 *
 * Operations (each defined by a FlashInfer documentation page):
 *   - block-sparse attention with a paged KV cache
 *     (page "flashinfer.attention.prims_ts.block_sparse_attention_with_paged_kv_cache",
 *      signature and Parameters)                         -> bsa_plan / bsa_validate / bsa_run
 *   - packed-Q paged prefill
 *     (page "flashinfer.attention.prims_ts.batch_prefill_with_paged_kv_cache")
 *                                                        -> paged_prefill_validate / _plan / _plan_capacity / _run
 *   - single-token paged decode with caller scratch
 *     (page "flashinfer.attention.prims_ts.prims_ts_batch_decode_with_kv_cache")
 *                                                        -> paged_decode_validate / _workspace_size / _run
 *     multi-token (fixed SQ or packed qo_indptr) decode   -> paged_decode_q_validate / _workspace_size / _run
 *   - packed-query token-granular sparse attention
 *     (page "flashinfer.qsa.qsa_forward")                -> qsa_validate / qsa_run
 *   - prequantized Sage-style block-sparse attention
 *     (page "flashinfer.cute_dsl.sparse.bsa_attn_sm120.bsa_attn_sm120_blk64_sage_fwd")
 *                                                        -> bsa_sage_validate / bsa_sage_run
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership: every tensor, output, LSE buffer, work list and workspace is
 *   caller-owned device memory (host memory where a parameter name ends in _h).
 *   The library never allocates or frees device memory.  Plan structs are POD
 *   values owned by the caller; there is nothing to destroy.
 * Errors: every function returns an int status: PKB_OK (0) or a negative
 *   pkb_status code.  Nothing is thrown and nothing aborts.  *_run functions
 *   check static arguments and return before launching anything when they are
 *   wrong.  pkb_status_string() describes a code.
 * Synchronisation: *_run functions only enqueue work on the given HIP stream
 *   (hipStream_t passed as void*; NULL = the default stream).  They never copy
 *   device data to the host and never synchronise, so they may be captured in a
 *   HIP graph.  *_validate and paged_prefill_plan read HOST copies of metadata
 *   synchronously.
 * Trust: *_run trusts live metadata (page IDs, offsets, lengths) exactly as the
 *   pages state: callers that cannot guarantee it call *_validate first.
 * Layouts: all tensors are contiguous unless a stride argument says otherwise;
 *   strides are in ELEMENTS.  K/V page pools are HND: [P, Hkv, page_size, D].  A
 *   combined cache [P, 2, Hkv, page_size, D] is passed as k = base,
 *   v = base + Hkv*page_size*D with kv_page_stride = 2*Hkv*page_size*D.
 * Numerics: bf16 inputs, fp32 accumulation, online softmax in base 2, output
 *   rounded to bf16 (round-to-nearest-even) or written as fp32.  LSE is the
 *   natural-log softmax normaliser in fp32, laid out [tokens, Hq]; a query row
 *   with no admitted key gets an exact zero output and LSE = -inf.
 * Memory contract for K/V: every live token (position < seq_len) must hold
 *   finite values; slots at or past the live length and unreferenced pages are
 *   never read into the result and may hold anything (NaN included).
 */
#ifndef PKB_H_
#define PKB_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 3: a NaN softmax scale selects the default and other non-positive or
 * non-finite scales are rejected; paged_decode_run_noalloc; any page size >= 1
 * for block-sparse and decode pools. */
#define PKB_ABI_VERSION 3

/* Largest max_seq_len accepted: 2^31 - 128, so that a 128-token padded tile end
 * still fits in int32 (page "prims_ts_batch_decode_with_kv_cache", description of
 * max_seq_len). */
#define PKB_MAX_SEQ_LEN 2147483520

enum pkb_status {
  PKB_OK = 0,
  PKB_ERR_ARG = -1,         /* a static argument is out of range / inconsistent */
  PKB_ERR_SHAPE = -2,       /* a size or stride does not match the others */
  PKB_ERR_DTYPE = -3,       /* unsupported dtype or dtype combination */
  PKB_ERR_UNSUPPORTED = -4, /* valid request this library does not implement */
  PKB_ERR_METADATA = -5,    /* live metadata violates its contract (validate) */
  PKB_ERR_WORKSPACE = -6,   /* workspace / work list too small or missing */
  PKB_ERR_HIP = -7          /* a HIP runtime call or launch failed */
};

enum pkb_dtype { PKB_BF16 = 0, PKB_FP32 = 1, PKB_I8 = 2, PKB_FP8E4M3 = 3 };
enum pkb_mask { PKB_MASK_DENSE = 0, PKB_MASK_CAUSAL = 1 };

/* Which metadata array a validate failure refers to. */
enum pkb_field {
  PKB_FIELD_NONE = 0,
  PKB_FIELD_KV_INDPTR = 1,
  PKB_FIELD_KV_INDICES = 2,
  PKB_FIELD_SEQ_LENS = 3,
  PKB_FIELD_BLOCK_INDPTR = 4,
  PKB_FIELD_BLOCK_INDICES = 5,
  PKB_FIELD_QO_INDPTR = 6,
  PKB_FIELD_BLOCK_TABLES = 7,
  PKB_FIELD_Q2K_INDEX = 8,
  PKB_FIELD_Q2K_NUMS = 9,
  PKB_FIELD_BLOCK_SIZES = 10,
  PKB_FIELD_LO = 11,
  PKB_FIELD_HI = 12,
  PKB_FIELD_BLK_BASE = 13,
  PKB_FIELD_TOK_BASE = 14,
  PKB_FIELD_BLOCK_FIRST = 15,
  PKB_FIELD_BLOCK_LAST = 16
};

/* First contract violation found by a *_validate call: the array and the flat
 * element index inside it (-1 when the failure is not tied to one element). */
typedef struct {
  int32_t field;
  int64_t index;
} pkb_bad_t;

const char* pkb_status_string(int status);
int pkb_abi_version(void);
/* Text of the last HIP runtime error seen by a *_run call on this thread (the
 * detail behind PKB_ERR_HIP). */
const char* pkb_last_hip_error(void);

/* ======================================================================== */
/* Block-sparse attention with a paged KV cache                              */
/* (page "block_sparse_attention_with_paged_kv_cache": signature, Parameters) */
/* ======================================================================== */

/* Static (capacity-only) arguments.  The page plans from static capacities and
 * binds live metadata only at run time.
 *   B, Sq, Hq, Hkv, D      q is [B, Sq, Hq, D]; Hq % Hkv == 0; D in {128, 256}.
 *   num_pages, page_size   K/V pools [num_pages, Hkv, page_size, D]; page_size >= 1
 *                          (multiples of 8 take the fastest copy path; others copy
 *                          K/V row by row, since 8 tokens may then span pages).
 *   q_block_size           query tokens per BSR row; (q_block_size*Hq/Hkv) % 8 == 0.
 *   kv_block_size          KV tokens per logical block: 8, 16, 32 or a multiple of 64.
 *   max_seq_len_kv         static maximum live KV length, 1..PKB_MAX_SEQ_LEN.
 *   mask_type              PKB_MASK_DENSE or PKB_MASK_CAUSAL, applied per token
 *                          inside the selected blocks; causal aligns query i to
 *                          KV position seq_len - Sq + i.
 *   window_left            -1 (off) or w >= 0: admits keys p-w..p; needs causal.
 *   qkv_dtype, out_dtype   PKB_BF16 / (PKB_BF16 or PKB_FP32).
 *   num_cus                compute units of the target device (for the grid).  */
typedef struct {
  int32_t B, Sq, Hq, Hkv, D;
  int32_t num_pages, page_size;
  int32_t q_block_size, kv_block_size;
  int32_t max_seq_len_kv;
  int32_t mask_type, window_left;
  int32_t qkv_dtype, out_dtype;
  int32_t num_cus;
} bsa_static_args;

/* Plan: derived launch geometry.  POD; copy freely. */
typedef struct {
  bsa_static_args a;
  int32_t group;            /* Hq / Hkv */
  int32_t rows_per_brow;    /* q_block_size * group: packed rows of one BSR row */
  int32_t num_q_blocks;     /* ceil(Sq / q_block_size) */
  int32_t num_kv_blocks;    /* ceil(max_seq_len_kv / kv_block_size) */
  int32_t valid_words;      /* ceil(max_seq_len_kv / 32): row stride of kv_valid_bits */
  int32_t waves;            /* wavefronts per workgroup (32 packed rows each) */
  int32_t tile_m;           /* packed query rows per workgroup = 32 * waves */
  int32_t tiles_per_brow;   /* ceil(rows_per_brow / tile_m) */
  int32_t grid_x, grid_y, grid_z; /* work units: (query tile, KV head, request); the
                                      launch deals them over the XCDs as a 1-D grid */
  int32_t kernel_id;
} bsa_plan_t;

/* Checks the static arguments and fills *plan.  Host only, no device access. */
int bsa_plan(const bsa_static_args* args, bsa_plan_t* plan);

/* Host validation of live metadata (the page validates synchronously before the
 * trusted run).  All pointers are HOST copies:
 *   paged_kv_indptr_h [B+1]: starts at 0, strictly increasing, ends at n_indices.
 *   paged_kv_indices_h [n_indices]: the first ceil(seq_len/page_size) IDs of every
 *       request are in [0, num_pages) and there are enough of them.
 *   block_indptr_h [B, Hkv, num_q_blocks+1]: absolute offsets into block_indices,
 *       non-decreasing along each (b, kv head), every value in [0, n_block_indices].
 *   block_indices_h: logical KV block IDs in [0, num_kv_blocks), distinct per row.
 *   seq_lens_kv_h [B]: 0 <= seq_len <= max_seq_len_kv.
 * Returns PKB_OK or PKB_ERR_METADATA with *bad set to the first violation in the
 * order: kv_indptr, seq_lens, then per request the CSR sufficiency (reported on
 * kv_indptr[b+1]) and its live IDs, then block_indptr, then block_indices row by
 * row (each in increasing flat index).  bad may be NULL. */
int bsa_validate(const bsa_plan_t* plan,
                 const int32_t* paged_kv_indptr_h, const int32_t* paged_kv_indices_h,
                 int64_t n_indices,
                 const int32_t* block_indptr_h, const int32_t* block_indices_h,
                 int64_t n_block_indices,
                 const int32_t* seq_lens_kv_h, pkb_bad_t* bad);

/* Trusted run.  Device pointers:
 *   q [B, Sq, Hq, D] bf16;  k, v page pools (strides in elements: one page is
 *   kv_page_stride apart, one KV head kv_head_stride apart, tokens D apart);
 *   paged_kv_indptr/indices, block_indptr/indices, seq_lens_kv as in bsa_validate;
 *   kv_valid_bits [B, valid_words] uint32 or NULL (bit t%32 of word t/32, LSB
 *   first; 0 excludes token t);  sm_scale: NaN selects 1/sqrt(D), any other
 *   value must be finite and positive (else PKB_ERR_ARG);
 *   out [B, Sq, Hq, D] in plan->a.out_dtype;  lse [B*Sq, Hq] fp32 or NULL.
 * No workspace is needed. */
int bsa_run(const bsa_plan_t* plan, const void* q, const void* k, const void* v,
            int64_t kv_page_stride, int64_t kv_head_stride,
            const int32_t* paged_kv_indptr, const int32_t* paged_kv_indices,
            const int32_t* block_indptr, const int32_t* block_indices,
            const int32_t* seq_lens_kv, const uint32_t* kv_valid_bits, float sm_scale,
            void* out, float* lse, void* stream);

/* ======================================================================== */
/* Packed-Q paged prefill                                                     */
/* (page "batch_prefill_with_paged_kv_cache": description, Parameters)        */
/* ======================================================================== */

/*   B, Hq, Hkv, D   q/out are [total_q, Hq, D]; D in {128, 256}.
 *   num_pages, page_size  HND pools; page_size in {16, 32, 64, 128}.
 *   block_table_width     C: block_tables is [B, C] with row stride >= C.
 *   mask_type, window_left as for bsa; causal aligns query i of request b to
 *                         position seq_len[b] - qlen[b] + i.                */
typedef struct {
  int32_t B, Hq, Hkv, D;
  int32_t num_pages, page_size;
  int32_t total_q;
  int32_t block_table_width;
  int32_t mask_type, window_left;
  int32_t qkv_dtype, out_dtype;
  int32_t num_cus;
} prefill_static_args;

typedef struct {
  prefill_static_args a;
  int32_t group;
  int32_t waves, tile_m;
  int32_t n_work;           /* work items (= grid_x); each is (b, first packed row) */
  int32_t grid_x, grid_y;   /* (work item, KV head); launched as one 1-D grid of
                               grid_x * grid_y workgroups, KV head fastest */
  int32_t kernel_id;
  int64_t kv_tokens;        /* sum over work items of visited KV positions */
} pkb_prefill_plan_t;

/* Host validation of prefill metadata (host copies):
 *   qo_indptr_h [B+1]: starts at 0, strictly increasing, ends at total_q.
 *   seq_lens_kv_h [B]: >= 0; causal additionally needs qlen[b] <= seq_len[b].
 *   block_tables_h [B, row_stride]: ceil(seq_len/page_size) <= C (else the
 *       failure is reported on seq_lens[b]) and those leading entries are in
 *       [0, num_pages).
 * Order: qo_indptr, seq_lens, block_tables. */
int paged_prefill_validate(const prefill_static_args* args, const int32_t* qo_indptr_h,
                           const int32_t* seq_lens_kv_h, const int32_t* block_tables_h,
                           int64_t block_table_row_stride, pkb_bad_t* bad);

/* Reads host qo_indptr / seq_lens to build the work list (the page derives exact
 * plan bounds from host request metadata).  worklist_h receives 2*n_work int32:
 * (request, first packed query row of the tile within the request), sorted by
 * decreasing visited-KV span, ties by (request, row).  Returns PKB_ERR_WORKSPACE
 * (with *n_work set) when worklist_cap < n_work; worklist_h may then be NULL. */
int paged_prefill_plan(const prefill_static_args* args, const int32_t* qo_indptr_h,
                       const int32_t* seq_lens_kv_h, pkb_prefill_plan_t* plan,
                       int32_t* worklist_h, int64_t worklist_cap, int64_t* n_work);

/* Capacity plan for graph capture (prefill page, description: planning happens
 * outside a captured graph and replays only launch).  No request metadata is
 * read: the work list covers every request holding up to max_qlen query
 * rows, so one captured paged_prefill_run stays correct while qo_indptr /
 * seq_lens / block_tables change between replays within these bounds: every
 * qlen in [1, max_qlen],
 * qo_indptr starting at 0 and strictly increasing with qo_indptr[B] <= total_q
 * (rows past qo_indptr[B] of out / lse are not written), and the rest of the
 * paged_prefill_validate contract.  Tiles with no live rows exit at once.
 * Items: n_work = B * ceil(max_qlen * group / tile_m), ordered by tile index
 * from last to first and by request within a tile index; kv_tokens = 0.
 * max_qlen outside [1, total_q] -> PKB_ERR_ARG; worklist_cap < n_work (or a
 * NULL worklist_h) -> PKB_ERR_WORKSPACE with *n_work set. */
int paged_prefill_plan_capacity(const prefill_static_args* args, int32_t max_qlen,
                                pkb_prefill_plan_t* plan, int32_t* worklist_h,
                                int64_t worklist_cap, int64_t* n_work);

/* Trusted run.  worklist_d: device copy of the plan's work list.  sm_scale as
 * for bsa_run (NaN selects 1/sqrt(D); otherwise finite and positive);
 * output_scale (finite) multiplies the normalised output; out dtype from the
 * plan. */
int paged_prefill_run(const pkb_prefill_plan_t* plan, const int32_t* worklist_d,
                      const void* q, const void* k_cache, const void* v_cache,
                      int64_t kv_page_stride, int64_t kv_head_stride,
                      const int32_t* qo_indptr, const int32_t* block_tables,
                      int64_t block_table_row_stride, const int32_t* seq_lens_kv,
                      float sm_scale, float output_scale, void* out, float* lse,
                      void* stream);

/* ======================================================================== */
/* Single-token paged decode, split-KV with a merge pass                      */
/* (page "prims_ts_batch_decode_with_kv_cache": description, Parameters)      */
/* ======================================================================== */

/* Any page_size >= 1 is accepted (sizes that are not a multiple of 8 translate
 * every token's page on its own).
 * Static policy from max_seq_len (the page selects its policy from the static
 * maximum): each request's keys are cut into chunks of split_len tokens (at
 * most num_splits chunks); workspace bytes paged_decode_run needs (0 when one
 * chunk suffices): fp32 partials [B, Hq, num_splits, D+4] (O, running max,
 * running sum, pad).  Every live partial is written before it is read, so the
 * workspace needs no initialisation (zeroing it, as the page asks, is harmless). */
int paged_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                int32_t max_seq_len, int32_t page_size, int32_t num_cus,
                                size_t* bytes, int32_t* num_splits, int32_t* split_len);

/* Host validation (host copies): indptr starts at 0, strictly increasing, ends at
 * n_indices; 1 <= seq_len <= max_seq_len; each request owns
 * ceil(seq_len/page_size) CSR entries and those IDs are in [0, num_pages).
 * Order: kv_indptr, seq_lens, then per request the CSR sufficiency (reported on
 * kv_indptr[b+1]) and its live IDs. */
int paged_decode_validate(int32_t B, int32_t num_pages, int32_t page_size,
                          int32_t max_seq_len, const int32_t* paged_kv_indptr_h,
                          const int32_t* paged_kv_indices_h, int64_t n_indices,
                          const int32_t* seq_lens_h, pkb_bad_t* bad);

/* Trusted run.  query [B, Hq, D] bf16; k/v pools as above; bmm1_scale is the
 * softmax scale (NaN selects 1/sqrt(D); any other value must be finite and
 * positive, else PKB_ERR_ARG); bmm2_scale (finite) multiplies the output;
 * out [B, Hq, D] (out_dtype), lse [B, Hq] fp32 or NULL; workspace of at least
 * paged_decode_workspace_size() bytes, exclusive to this launch until it ends.
 * With more than one split a second, small kernel merges the partials. */
int paged_decode_run(const void* query, const void* k, const void* v,
                     int64_t kv_page_stride, int64_t kv_head_stride,
                     const int32_t* paged_kv_indptr, const int32_t* paged_kv_indices,
                     const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                     int32_t D, int32_t num_pages, int32_t page_size, int32_t max_seq_len,
                     int32_t mask_type, int32_t window_left, float bmm1_scale,
                     float bmm2_scale, int32_t out_dtype, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, int32_t num_cus,
                     void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * decode as paged_decode_run, with the split partials in a fixed scratch
 * array of PKB_DECODE_SCRATCH_BYTES (32 MiB) that the library holds on each
 * device it runs on until the process ends.  Nothing is allocated per call.
 * A call whose partials (paged_decode_workspace_size) exceed that size
 * returns PKB_ERR_WORKSPACE before anything is enqueued.  Every call on one
 * device shares that device's array: calls that overlap on one GPU (other
 * streams, or a second call before the first has finished on the device)
 * race and give undefined results.  The array needs no initialisation (every
 * partial is written before it is read).  Other arguments and errors as
 * paged_decode_run. */
#define PKB_DECODE_SCRATCH_BYTES (32u << 20)
int paged_decode_run_noalloc(const void* query, const void* k, const void* v,
                             int64_t kv_page_stride, int64_t kv_head_stride,
                             const int32_t* paged_kv_indptr, const int32_t* paged_kv_indices,
                             const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                             int32_t D, int32_t num_pages, int32_t page_size,
                             int32_t max_seq_len, int32_t mask_type, int32_t window_left,
                             float bmm1_scale, float bmm2_scale, int32_t out_dtype, void* out,
                             float* lse, int32_t num_cus, void* stream);

/* Multi-token decode (decode page, description: for seq_len_q > 1 query and
 * output are token-major [B, SQ, Hq, D]; with qo_indptr they are packed
 * [total_q, Hq, D] and request b owns rows qo_indptr[b]:qo_indptr[b+1];
 * max_seq_len_q is the static bound).  Query i of request b sits at position
 * seq_len - qlen + i (bottom-right); causal needs qlen <= seq_len.
 *
 * Split policy and workspace: the chunk policy of paged_decode_workspace_size,
 * except that with max_q > 1 the chunk length stops halving once the batch
 * holds 4 (not 8) chunks per persistent wave (longer chunks: fewer partials to
 * merge); fp32 partials [B, max_q, Hq, num_splits, D+4] (max_q = seq_len_q, or
 * max_seq_len_q when packed), written before they are read (no initialisation
 * needed). */
int paged_decode_q_workspace_size(int32_t B, int32_t max_q, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t max_seq_len, int32_t page_size, int32_t num_cus,
                                  size_t* bytes, int32_t* num_splits, int32_t* split_len);

/* Host validation (host copies).  Order: kv_indptr (CSR), seq_lens in
 * [1, max_seq_len], then if qo_indptr_h is given: qo_indptr[0] == 0 (index 0),
 * every delta in [1, max_seq_len_q] (index b+1), qo_indptr[B] == total_q
 * (index B); then, for causal, every query length <= seq_len (SEQ_LENS, b);
 * then each request's CSR sufficiency and live IDs as paged_decode_validate.
 * Static errors (PKB_ERR_ARG): seq_len_q < 1 without qo_indptr, or
 * max_seq_len_q < 1 / total_q < 1 with it. */
int paged_decode_q_validate(int32_t B, int32_t num_pages, int32_t page_size,
                            int32_t max_seq_len, const int32_t* paged_kv_indptr_h,
                            const int32_t* paged_kv_indices_h, int64_t n_indices,
                            const int32_t* seq_lens_h, const int32_t* qo_indptr_h,
                            int64_t total_q, int32_t seq_len_q, int32_t max_seq_len_q,
                            int32_t mask_type, pkb_bad_t* bad);

/* Trusted run.  query [B, seq_len_q, Hq, D] bf16 when qo_indptr is NULL, else
 * [total_q, Hq, D] with qo_indptr a device [B+1] int32 array satisfying the
 * packed-offset contract above (it is read on the device only); out in the
 * query's layout (out_dtype); lse [tokens, Hq] fp32 or NULL; other arguments as
 * paged_decode_run; workspace of at least paged_decode_q_workspace_size()
 * bytes for max_q = seq_len_q (fixed) or max_seq_len_q (packed). */
int paged_decode_q_run(const void* query, const void* k, const void* v,
                       int64_t kv_page_stride, int64_t kv_head_stride,
                       const int32_t* paged_kv_indptr, const int32_t* paged_kv_indices,
                       const int32_t* seq_lens, const int32_t* qo_indptr, int32_t B,
                       int32_t seq_len_q, int32_t max_seq_len_q, int32_t Hq, int32_t Hkv,
                       int32_t D, int32_t num_pages, int32_t page_size, int32_t max_seq_len,
                       int32_t mask_type, int32_t window_left, float bmm1_scale,
                       float bmm2_scale, int32_t out_dtype, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, int32_t num_cus,
                       void* stream);

/* ======================================================================== */
/* Sage-style prequantized block-sparse attention                            */
/* (page "bsa_attn_sm120_blk64_sage_fwd": signature, Parameters, Notes)       */
/* ======================================================================== */

/* Host validation: block_sparse_num in [0, capacity]; q2k_block_nums (if given
 * and not uniform) in [0, capacity]; the first n indices of every row in
 * [0, ceil(Sk/64)) and distinct; block_sizes (if given) in [0, 64].
 * Order: q2k_nums, q2k_index, block_sizes. */
int bsa_sage_validate(const int32_t* q2k_block_index_h, int32_t capacity,
                      int32_t block_sparse_num, const int32_t* block_sizes_h,
                      int32_t block_sizes_rank, const int32_t* q2k_block_nums_h,
                      int32_t uniform_block_count, int32_t B, int32_t H, int32_t Sq,
                      int32_t Sk, pkb_bad_t* bad);

/* Trusted run (MHA, D = 128, 64-token blocks).
 *   q [B,H,Sq,128] int8, k [B,H,Sk,128] int8,
 *   v_fp8 [B,H,128,ceil(Sk/64)*64] OCP E4M3FN in HDS layout (tokens contiguous);
 *   Sk above 2^25 returns PKB_ERR_UNSUPPORTED (32-bit offsets inside one head),
 *   q_scale [B,H,ceil(Sq/128)*4] (one per 32 rows), k_scale [B,H,ceil(Sk/64)],
 *   v_scale [B,H,128] fp32;
 *   q2k_block_index [B,H,ceil(Sq/64),capacity] int32;
 *   q2k_block_nums [B,H,ceil(Sq/64)] or NULL, used when non-NULL and
 *   uniform_block_count == 0, else every row uses block_sparse_num;
 *   block_sizes (NULL = 64) of rank 1 [nkb], 2 [B,nkb] or 3 [B,H,nkb]:
 *   valid-token count of each KV block (its first tokens);
 *   contiguous_block_indices (needs uniform_block_count, else PKB_ERR_ARG):
 *   the caller promises that each row's blocks are index[0], index[0] + 1, ...;
 *   only index[0] is read (Parameters: the promise is trusted, not checked).
 *   Block ids outside [0, ceil(Sk/64)) then count as empty blocks;
 *   softmax_scale: NaN selects 1/sqrt(128); otherwise it must be finite and
 *   positive (the page asks for a positive scale), else PKB_ERR_ARG;
 *   mask_type: PKB_MASK_DENSE as on the page, or PKB_MASK_CAUSAL, an addition
 *   that applies the block-sparse page's token-level causal rule to the
 *   selected tokens (query i at position Sk - Sq + i admits tokens j <= that);
 *   out [B,H,Sq,128] bf16; lse [B,H,Sq] fp32 natural-log LSE or NULL (an
 *   addition: the page's kernel returns no LSE).  A row with no admitted
 *   token is written as zeros (LSE -inf). */
int bsa_sage_run(const void* q_int8, const void* k_int8, const void* v_fp8,
                 const float* q_scale, const float* k_scale, const float* v_scale,
                 const int32_t* q2k_block_index, int32_t capacity,
                 int32_t block_sparse_num, const int32_t* block_sizes,
                 int32_t block_sizes_rank, const int32_t* q2k_block_nums,
                 int32_t uniform_block_count, int32_t contiguous_block_indices,
                 int32_t B, int32_t H, int32_t Sq, int32_t Sk, float softmax_scale,
                 int32_t mask_type, void* out, float* lse, void* stream);

/* ======================================================================== */
/* Packed-query token-granular sparse attention                              */
/* (page "qsa_forward": signature, Parameters, Returns, Notes)                */
/* ======================================================================== */

/* Host validation of the packed partition (host copies, all [T] or [NB] int32):
 *   tok_base: a token starting a sequence has tok_base[t] == t, every other
 *     token repeats its predecessor's value (TOK_BASE, t);
 *   blk_base: constant inside a sequence and, with the sequence's
 *     ceil(len/4) blocks, inside [0, NB) (BLK_BASE, t);
 *   block_first / block_last of block blk_base + m of a sequence starting at s0
 *     with length len: s0 + 4m and min(s0 + 4m + 3, s0 + len - 1)
 *     (BLOCK_FIRST / BLOCK_LAST, block index);
 *   lo / hi: when lo[t] <= hi[t], both inside t's sequence (LO / HI, t);
 *     lo[t] > hi[t] is an empty row.
 * Order: per token in order tok_base, blk_base; then blocks; then lo, hi.
 * Static errors: T < 1, NB < 1 or a NULL array -> PKB_ERR_ARG. */
int qsa_validate(int32_t T, int32_t NB, const int32_t* lo_h, const int32_t* hi_h,
                 const int32_t* blk_base_h, const int32_t* tok_base_h,
                 const int32_t* block_first_h, const int32_t* block_last_h, pkb_bad_t* bad);

/* Trusted run.  q [T, Hq, D] bf16, k / v [T, Hkv, D] bf16 (packed tokens, not
 * paged), sel_blocks [T, NB] uint8 (nonzero selects a global block), lo / hi /
 * blk_base / tok_base [T] int32 on the device, satisfying qsa_validate.
 * block_first / block_last need not be passed: under the partition contract a
 * block's span follows from tok_base and blk_base, which the kernel uses.
 * D in {128, 256} (the page: 256), Hq / Hkv <= 16 (the page: 12), block_size
 * must be 4, scale finite (used as given; the page's default is 1/sqrt(256)),
 * and each of k / v at most 4 GiB (T * Hkv * D * 2 bytes; else
 * PKB_ERR_UNSUPPORTED).
 * Outputs (each may be NULL, not all): out [T, Hq, D] bf16, out_f32
 * [T, Hq, D], lse [Hq, T] natural log (the page's layout).  Empty rows give
 * zeros and -inf. */
int qsa_run(const void* q, const void* k, const void* v, const uint8_t* sel_blocks,
            const int32_t* lo, const int32_t* hi, const int32_t* blk_base,
            const int32_t* tok_base, int32_t T, int32_t NB, int32_t Hq, int32_t Hkv,
            int32_t D, float scale, int32_t block_size, void* out, float* out_f32,
            float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKB_H_ */
