// api.cpp -- the *_run entry points of libpkb: check static arguments, fill the
// kernel parameter block and enqueue the kernels on the caller's stream.  No
// device memory is allocated, nothing is copied to the host, nothing waits.
#include <math.h>
#include <string.h>

#include <algorithm>

#include <hip/hip_runtime.h>

#include "../../include/pkb.h"
#include "pkb_internal.h"

using pkb::AttnParams;

namespace {

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

thread_local hipError_t g_last_hip = hipSuccess;

inline int hip_status(hipError_t e) {
  if (e == hipSuccess) return PKB_OK;
  g_last_hip = e;
  return PKB_ERR_HIP;
}

// Softmax scale: NaN selects the default 1/sqrt(D); any other value must be
// finite and positive.  Returns false for a scale the pages do not allow.
inline bool resolve_scale(float s, int D, float* out) {
  if (isnan(s)) {
    *out = 1.0f / sqrtf((float)D);
    return true;
  }
  if (!(s > 0.f) || !isfinite(s)) return false;
  *out = s;
  return true;
}

// Merge of split partials [B, maxq, Hq, S, D+4] into out / lse.
int launch_merge(float* part, const int32_t* seq_lens, const int32_t* qo_indptr, void* out,
                 float* lse, int B, int maxq, int Sq, int Hq, int S, int split_len,
                 int out_dtype, float out_scale, int D, hipStream_t s) {
  pkb::MergeParams mp;
  memset(&mp, 0, sizeof(mp));
  mp.part = part;
  mp.seq_lens = seq_lens;
  mp.qo_indptr = qo_indptr;
  mp.out = out;
  mp.lse = lse;
  mp.B = B;
  mp.Hq = Hq;
  mp.num_splits = S;
  mp.split_len = split_len;
  mp.maxq = maxq;
  mp.Sq = Sq;
  mp.out_f32 = out_dtype == PKB_FP32;
  mp.out_scale = out_scale;
  return hip_status(pkb::launch_decode_merge(mp, D, s));
}

}  // namespace

extern "C" {

const char* pkb_last_hip_error(void) { return hipGetErrorString(g_last_hip); }

int bsa_run(const bsa_plan_t* plan, const void* q, const void* k, const void* v,
            int64_t kv_page_stride, int64_t kv_head_stride, const int32_t* kv_indptr,
            const int32_t* kv_indices, const int32_t* block_indptr, const int32_t* block_indices,
            const int32_t* seq_lens, const uint32_t* kv_valid_bits, float sm_scale, void* out,
            float* lse, void* stream) {
  if (!plan) return PKB_ERR_ARG;
  bsa_plan_t chk;
  int st = bsa_plan(&plan->a, &chk);
  if (st) return st;
  if (memcmp(&chk, plan, sizeof(chk)) != 0) return PKB_ERR_ARG;   // stale or edited plan
  const bsa_static_args& a = plan->a;
  if (!q || !k || !v || !kv_indptr || !kv_indices || !block_indptr || !seq_lens || !out)
    return PKB_ERR_ARG;
  if (kv_page_stride < (int64_t)a.Hkv * a.page_size * a.D ||
      kv_head_stride < (int64_t)a.page_size * a.D)
    return PKB_ERR_SHAPE;
  float scale = 0.f;
  if (!resolve_scale(sm_scale, a.D, &scale)) return PKB_ERR_ARG;
  AttnParams p;
  memset(&p, 0, sizeof(p));
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.out = out;
  p.lse = lse;
  p.kv_indptr = kv_indptr;
  p.kv_indices = kv_indices;
  p.block_indptr = block_indptr;
  p.block_indices = block_indices;
  p.seq_lens = seq_lens;
  p.valid_bits = kv_valid_bits;
  p.kv_page_stride = kv_page_stride;
  p.kv_head_stride = kv_head_stride;
  p.B = a.B;
  p.Sq = a.Sq;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.G = plan->group;
  p.page_size = a.page_size;
  p.qbs = a.q_block_size;
  p.kvbs = a.kv_block_size;
  p.nqb = plan->num_q_blocks;
  p.tiles_per_brow = plan->tiles_per_brow;
  p.rows_per_brow = plan->rows_per_brow;
  p.valid_words = plan->valid_words;
  p.causal = a.mask_type == PKB_MASK_CAUSAL;
  p.window_left = a.window_left;
  p.num_splits = 1;
  p.split_len = 0;
  p.out_f32 = a.out_dtype == PKB_FP32;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.out_scale = 1.0f;
  const int64_t total = (int64_t)plan->grid_x * plan->grid_y * plan->grid_z;
  dim3 grid((unsigned)(((total + 7) / 8) * 8), 1, 1);
  return hip_status(pkb::launch_attn(p, a.D, plan->waves, pkb::kModeBsa, grid,
                                     (hipStream_t)stream));
}

int paged_prefill_run(const pkb_prefill_plan_t* plan, const int32_t* worklist_d, const void* q,
                      const void* k_cache, const void* v_cache, int64_t kv_page_stride,
                      int64_t kv_head_stride, const int32_t* qo_indptr,
                      const int32_t* block_tables, int64_t block_table_row_stride,
                      const int32_t* seq_lens, float sm_scale, float output_scale, void* out,
                      float* lse, void* stream) {
  if (!plan) return PKB_ERR_ARG;
  const prefill_static_args& a = plan->a;
  if (a.B < 1 || a.Hkv < 1 || a.Hq % a.Hkv || (a.D != 128 && a.D != 256) ||
      plan->waves != 4 || plan->group != a.Hq / a.Hkv)
    return PKB_ERR_ARG;
  if (a.mask_type != PKB_MASK_DENSE && a.mask_type != PKB_MASK_CAUSAL) return PKB_ERR_ARG;
  if (a.window_left < -1 || (a.window_left >= 0 && a.mask_type != PKB_MASK_CAUSAL))
    return PKB_ERR_ARG;
  if (a.out_dtype != PKB_BF16 && a.out_dtype != PKB_FP32) return PKB_ERR_DTYPE;
  if (!q || !k_cache || !v_cache || !qo_indptr || !block_tables || !seq_lens || !out)
    return PKB_ERR_ARG;
  if (block_table_row_stride < a.block_table_width) return PKB_ERR_SHAPE;
  if (kv_page_stride < (int64_t)a.Hkv * a.page_size * a.D ||
      kv_head_stride < (int64_t)a.page_size * a.D)
    return PKB_ERR_SHAPE;
  if (!isfinite(output_scale)) return PKB_ERR_ARG;
  float scale = 0.f;
  if (!resolve_scale(sm_scale, a.D, &scale)) return PKB_ERR_ARG;
  if (plan->n_work == 0) return PKB_OK;
  if (!worklist_d) return PKB_ERR_WORKSPACE;
  AttnParams p;
  memset(&p, 0, sizeof(p));
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k_cache;
  p.v = (const uint16_t*)v_cache;
  p.out = out;
  p.lse = lse;
  p.block_tables = block_tables;
  p.bt_stride = block_table_row_stride;
  p.qo_indptr = qo_indptr;
  p.seq_lens = seq_lens;
  p.worklist = worklist_d;
  p.kv_page_stride = kv_page_stride;
  p.kv_head_stride = kv_head_stride;
  p.B = a.B;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.G = plan->group;
  p.page_size = a.page_size;
  p.causal = a.mask_type == PKB_MASK_CAUSAL;
  p.window_left = a.window_left;
  p.num_splits = 1;
  p.out_f32 = a.out_dtype == PKB_FP32;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.out_scale = output_scale;
  dim3 grid(plan->grid_x * plan->grid_y, 1, 1);
  return hip_status(pkb::launch_attn(p, a.D, plan->waves, pkb::kModePrefill, grid,
                                     (hipStream_t)stream));
}

int paged_decode_run(const void* query, const void* k, const void* v, int64_t kv_page_stride,
                     int64_t kv_head_stride, const int32_t* kv_indptr, const int32_t* kv_indices,
                     const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                     int32_t num_pages, int32_t page_size, int32_t max_seq_len,
                     int32_t mask_type, int32_t window_left, float bmm1_scale,
                     float bmm2_scale, int32_t out_dtype, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, int32_t num_cus, void* stream) {
  size_t need = 0;
  int32_t S = 0, split_len = 0;
  int st = paged_decode_workspace_size(B, Hq, Hkv, D, max_seq_len, page_size, num_cus, &need,
                                       &S, &split_len);
  if (st) return st;
  if (num_pages < 1) return PKB_ERR_ARG;
  if (Hq / Hkv > 128) return PKB_ERR_UNSUPPORTED;   // one workgroup holds the GQA group
  if (mask_type != PKB_MASK_DENSE && mask_type != PKB_MASK_CAUSAL) return PKB_ERR_ARG;
  if (window_left < -1 || (window_left >= 0 && mask_type != PKB_MASK_CAUSAL)) return PKB_ERR_ARG;
  if (out_dtype != PKB_BF16 && out_dtype != PKB_FP32) return PKB_ERR_DTYPE;
  if (!query || !k || !v || !kv_indptr || !kv_indices || !seq_lens || !out) return PKB_ERR_ARG;
  if (kv_page_stride < (int64_t)Hkv * page_size * D || kv_head_stride < (int64_t)page_size * D)
    return PKB_ERR_SHAPE;
  if (!isfinite(bmm2_scale)) return PKB_ERR_ARG;
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKB_ERR_WORKSPACE;
  const hipStream_t s = (hipStream_t)stream;
  dim3 grid(S, Hkv, B);
  float* part = S > 1 ? (float*)workspace : nullptr;
  float scale = 0.f;
  if (!resolve_scale(bmm1_scale, D, &scale)) return PKB_ERR_ARG;
  const float sl2 = scale * 1.4426950408889634f;
  if (Hq / Hkv <= pkb::kDecodeMaxGroup) {
    pkb::DecodeParams d;
    memset(&d, 0, sizeof(d));
    d.q = (const uint16_t*)query;
    d.k = (const uint16_t*)k;
    d.v = (const uint16_t*)v;
    d.out = out;
    d.lse = lse;
    d.part = part;
    d.kv_indptr = kv_indptr;
    d.kv_indices = kv_indices;
    d.seq_lens = seq_lens;
    d.kv_page_stride = kv_page_stride;
    d.kv_head_stride = kv_head_stride;
    d.B = B;
    d.Hq = Hq;
    d.Hkv = Hkv;
    d.G = Hq / Hkv;
    d.page_size = page_size;
    d.window_left = window_left;
    d.num_splits = S;
    d.split_len = split_len;
    d.Sq = 1;
    d.maxq = 1;
    d.out_f32 = out_dtype == PKB_FP32;
    d.scale_log2 = sl2;
    d.out_scale = bmm2_scale;
    // wide batches: one pass, every (request, KV head) a whole item (S == 1)
    if (pkb::decode_coop(B, Hkv, Hq / Hkv, num_cus)) return hip_status(pkb::launch_decode_coop(d, D, num_cus, s));
    const int64_t items = (int64_t)B * Hkv * S;
    const int waves = (int)std::min<int64_t>(items, (int64_t)num_cus * pkb::decode_waves_per_cu(D));
    hipError_t e = pkb::launch_decode(d, D, waves, s);
    if (e != hipSuccess) return hip_status(e);
  } else {
    // Larger GQA groups: the general attention kernel in split-KV decode mode.
    AttnParams p;
    memset(&p, 0, sizeof(p));
    p.q = (const uint16_t*)query;
    p.k = (const uint16_t*)k;
    p.v = (const uint16_t*)v;
    p.out = out;
    p.lse = lse;
    p.part = part;
    p.kv_indptr = kv_indptr;
    p.kv_indices = kv_indices;
    p.seq_lens = seq_lens;
    p.kv_page_stride = kv_page_stride;
    p.kv_head_stride = kv_head_stride;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.G = Hq / Hkv;
    p.page_size = page_size;
    p.causal = mask_type == PKB_MASK_CAUSAL;
    p.window_left = window_left;
    p.num_splits = S;
    p.split_len = split_len;
    p.Sq = 1;
    p.maxq = 1;
    p.out_f32 = out_dtype == PKB_FP32;
    p.scale_log2 = sl2;
    p.out_scale = bmm2_scale;
    hipError_t e = pkb::launch_attn(p, D, 4, pkb::kModeDecode, grid, s);
    if (e != hipSuccess) return hip_status(e);
  }
  if (S > 1) return launch_merge(part, seq_lens, nullptr, out, lse, B, 1, 1, Hq, S, split_len,
                                 out_dtype, bmm2_scale, D, s);
  return PKB_OK;
}

int paged_decode_run_noalloc(const void* query, const void* k, const void* v,
                             int64_t kv_page_stride, int64_t kv_head_stride,
                             const int32_t* kv_indptr, const int32_t* kv_indices,
                             const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                             int32_t num_pages, int32_t page_size, int32_t max_seq_len,
                             int32_t mask_type, int32_t window_left, float bmm1_scale,
                             float bmm2_scale, int32_t out_dtype, void* out, float* lse,
                             int32_t num_cus, void* stream) {
  size_t need = 0;
  int32_t S = 0, split_len = 0;
  int st = paged_decode_workspace_size(B, Hq, Hkv, D, max_seq_len, page_size, num_cus, &need,
                                       &S, &split_len);
  if (st) return st;
  if (need > pkb::kDecodeScratchBytes) return PKB_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = pkb::decode_scratch(&ws);
    if (e != hipSuccess) return hip_status(e);
  }
  return paged_decode_run(query, k, v, kv_page_stride, kv_head_stride, kv_indptr, kv_indices,
                          seq_lens, B, Hq, Hkv, D, num_pages, page_size, max_seq_len, mask_type,
                          window_left, bmm1_scale, bmm2_scale, out_dtype, out, lse, ws, need,
                          num_cus, stream);
}

int paged_decode_q_run(const void* query, const void* k, const void* v, int64_t kv_page_stride,
                       int64_t kv_head_stride, const int32_t* kv_indptr,
                       const int32_t* kv_indices, const int32_t* seq_lens,
                       const int32_t* qo_indptr, int32_t B, int32_t seq_len_q,
                       int32_t max_seq_len_q, int32_t Hq, int32_t Hkv, int32_t D,
                       int32_t num_pages, int32_t page_size, int32_t max_seq_len,
                       int32_t mask_type, int32_t window_left, float bmm1_scale,
                       float bmm2_scale, int32_t out_dtype, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, int32_t num_cus, void* stream) {
  const int32_t maxq = qo_indptr ? max_seq_len_q : seq_len_q;
  size_t need = 0;
  int32_t S = 0, split_len = 0;
  int st = paged_decode_q_workspace_size(B, maxq, Hq, Hkv, D, max_seq_len, page_size, num_cus,
                                         &need, &S, &split_len);
  if (st) return st;
  if (num_pages < 1 || B > 65535) return PKB_ERR_ARG;
  if (mask_type != PKB_MASK_DENSE && mask_type != PKB_MASK_CAUSAL) return PKB_ERR_ARG;
  if (window_left < -1 || (window_left >= 0 && mask_type != PKB_MASK_CAUSAL)) return PKB_ERR_ARG;
  if (out_dtype != PKB_BF16 && out_dtype != PKB_FP32) return PKB_ERR_DTYPE;
  if (!query || !k || !v || !kv_indptr || !kv_indices || !seq_lens || !out) return PKB_ERR_ARG;
  if (kv_page_stride < (int64_t)Hkv * page_size * D || kv_head_stride < (int64_t)page_size * D)
    return PKB_ERR_SHAPE;
  if (!isfinite(bmm2_scale)) return PKB_ERR_ARG;
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKB_ERR_WORKSPACE;
  float* part = S > 1 ? (float*)workspace : nullptr;
  const hipStream_t s = (hipStream_t)stream;
  float scale = 0.f;
  if (!resolve_scale(bmm1_scale, D, &scale)) return PKB_ERR_ARG;
  const float sl2 = scale * 1.4426950408889634f;
  if ((int64_t)maxq * (Hq / Hkv) <= pkb::kDecodeMaxGroup) {
    // the query rows of a KV head fit the 16 MFMA columns of the decode kernel
    pkb::DecodeParams d;
    memset(&d, 0, sizeof(d));
    d.q = (const uint16_t*)query;
    d.k = (const uint16_t*)k;
    d.v = (const uint16_t*)v;
    d.out = out;
    d.lse = lse;
    d.part = part;
    d.kv_indptr = kv_indptr;
    d.kv_indices = kv_indices;
    d.seq_lens = seq_lens;
    d.qo_indptr = qo_indptr;
    d.kv_page_stride = kv_page_stride;
    d.kv_head_stride = kv_head_stride;
    d.B = B;
    d.Hq = Hq;
    d.Hkv = Hkv;
    d.G = Hq / Hkv;
    d.page_size = page_size;
    d.window_left = window_left;
    d.Sq = seq_len_q;
    d.maxq = maxq;
    d.causal = mask_type == PKB_MASK_CAUSAL;
    d.num_splits = S;
    d.split_len = split_len;
    d.out_f32 = out_dtype == PKB_FP32;
    d.scale_log2 = sl2;
    d.out_scale = bmm2_scale;
    if (pkb::decode_coop(B, Hkv, maxq * (Hq / Hkv), num_cus))
      return hip_status(pkb::launch_decode_coop(d, D, num_cus, s));
    const int64_t items = (int64_t)B * Hkv * S;
    const int waves = (int)std::min<int64_t>(items, (int64_t)num_cus * pkb::decode_waves_per_cu(D));
    hipError_t e = pkb::launch_decode(d, D, waves, s);
    if (e != hipSuccess) return hip_status(e);
    if (S > 1) return launch_merge(part, seq_lens, qo_indptr, out, lse, B, maxq, seq_len_q, Hq, S,
                                   split_len, out_dtype, bmm2_scale, D, s);
    return PKB_OK;
  }
  // larger row sets: the general kernel in decode mode (4 waves x 32 packed rows)
  const int64_t rtiles = cdiv((int64_t)maxq * (Hq / Hkv), 128);
  if (rtiles * S > 0x7fffffff) return PKB_ERR_UNSUPPORTED;
  AttnParams p;
  memset(&p, 0, sizeof(p));
  p.q = (const uint16_t*)query;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.out = out;
  p.lse = lse;
  p.part = part;
  p.kv_indptr = kv_indptr;
  p.kv_indices = kv_indices;
  p.qo_indptr = qo_indptr;
  p.seq_lens = seq_lens;
  p.kv_page_stride = kv_page_stride;
  p.kv_head_stride = kv_head_stride;
  p.B = B;
  p.Sq = seq_len_q;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.page_size = page_size;
  p.causal = mask_type == PKB_MASK_CAUSAL;
  p.window_left = window_left;
  p.num_splits = S;
  p.split_len = split_len;
  p.maxq = maxq;
  p.out_f32 = out_dtype == PKB_FP32;
  p.scale_log2 = sl2;
  p.out_scale = bmm2_scale;
  dim3 grid((unsigned)(rtiles * S), Hkv, B);
  hipError_t e = pkb::launch_attn(p, D, 4, pkb::kModeDecode, grid, s);
  if (e != hipSuccess) return hip_status(e);
  if (S > 1) return launch_merge(part, seq_lens, qo_indptr, out, lse, B, maxq, seq_len_q, Hq, S,
                                 split_len, out_dtype, bmm2_scale, D, s);
  return PKB_OK;
}

int bsa_sage_run(const void* q_int8, const void* k_int8, const void* v_fp8,
                 const float* q_scale, const float* k_scale, const float* v_scale,
                 const int32_t* q2k_block_index, int32_t capacity, int32_t block_sparse_num,
                 const int32_t* block_sizes, int32_t block_sizes_rank,
                 const int32_t* q2k_block_nums, int32_t uniform_block_count,
                 int32_t contiguous_block_indices, int32_t B, int32_t H, int32_t Sq, int32_t Sk,
                 float softmax_scale, int32_t mask_type, void* out, float* lse, void* stream) {
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || capacity < 0) return PKB_ERR_ARG;
  if (mask_type != PKB_MASK_DENSE && mask_type != PKB_MASK_CAUSAL) return PKB_ERR_ARG;
  if (block_sparse_num < 0 || block_sparse_num > capacity) return PKB_ERR_ARG;
  if (contiguous_block_indices && !uniform_block_count) return PKB_ERR_ARG;
  if (block_sizes && (block_sizes_rank < 1 || block_sizes_rank > 3)) return PKB_ERR_ARG;
  float scale = 0.f;
  if (!resolve_scale(softmax_scale, 128, &scale)) return PKB_ERR_ARG;
  if (!q_int8 || !k_int8 || !v_fp8 || !q_scale || !k_scale || !v_scale || !out)
    return PKB_ERR_ARG;
  if (capacity > 0 && !q2k_block_index) return PKB_ERR_ARG;
  if ((int64_t)B * H * cdiv(Sq, 64) > 0x7fffffff) return PKB_ERR_UNSUPPORTED;
  if (Sk > (1 << 25)) return PKB_ERR_UNSUPPORTED;   // V offsets inside one head fit 32 bits
  pkb::SageParams p;
  memset(&p, 0, sizeof(p));
  p.q = (const int8_t*)q_int8;
  p.k = (const int8_t*)k_int8;
  p.v = (const uint8_t*)v_fp8;
  p.q_scale = q_scale;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.index = q2k_block_index;
  p.nums = uniform_block_count ? nullptr : q2k_block_nums;
  p.block_sizes = block_sizes;
  p.out = (uint16_t*)out;
  p.lse = lse;
  p.causal = mask_type == PKB_MASK_CAUSAL;
  p.contig = contiguous_block_indices != 0;
  p.B = B;
  p.H = H;
  p.Sq = Sq;
  p.Sk = Sk;
  p.nqb = (int)cdiv(Sq, 64);
  p.nkb = (int)cdiv(Sk, 64);
  p.Skp = p.nkb * 64;
  p.capacity = capacity;
  p.block_sparse_num = block_sparse_num;
  p.bs_rank = block_sizes ? block_sizes_rank : 0;
  p.qs_len = (int)cdiv(Sq, 128) * 4;
  p.scale_log2 = scale * 1.4426950408889634f;
  return hip_status(pkb::launch_sage(p, (hipStream_t)stream));
}

int qsa_run(const void* q, const void* k, const void* v, const uint8_t* sel_blocks,
            const int32_t* lo, const int32_t* hi, const int32_t* blk_base,
            const int32_t* tok_base, int32_t T, int32_t NB, int32_t Hq, int32_t Hkv,
            int32_t D, float scale, int32_t block_size, void* out, float* out_f32, float* lse,
            void* stream) {
  if (T < 1 || NB < 1 || Hq < 1 || Hkv < 1) return PKB_ERR_ARG;
  if (Hq % Hkv) return PKB_ERR_SHAPE;
  if (block_size != 4 || (D != 128 && D != 256) || Hq / Hkv > 16) return PKB_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return PKB_ERR_ARG;
  if (!q || !k || !v || !sel_blocks || !lo || !hi || !blk_base || !tok_base) return PKB_ERR_ARG;
  if (!out && !out_f32 && !lse) return PKB_ERR_ARG;
  // the kernel addresses K / V rows with 32-bit byte offsets
  if ((int64_t)T * Hkv * D * 2 > 0xFFFFFFFFLL) return PKB_ERR_UNSUPPORTED;
  pkb::QsaParams p;
  memset(&p, 0, sizeof(p));
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.sel = sel_blocks;
  p.lo = lo;
  p.hi = hi;
  p.blk_base = blk_base;
  p.tok_base = tok_base;
  p.out = (uint16_t*)out;
  p.out_f32 = out_f32;
  p.lse = lse;
  p.T = T;
  p.NB = NB;
  p.sel16 = (NB % 16 == 0 && ((uintptr_t)sel_blocks & 15) == 0) ? 1 : 0;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.scale_log2 = scale * 1.4426950408889634f;
  return hip_status(pkb::launch_qsa(p, D, (hipStream_t)stream));
}

}  // extern "C"
