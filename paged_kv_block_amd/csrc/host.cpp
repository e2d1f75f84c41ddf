// host.cpp -- static-argument checks, plans and host-side metadata validation of
// libpkb.  No device access happens here, so every function in this file can be
// called on a machine without a GPU.
//
// The rules restate the contracts of the FlashInfer pages:
//  * "prims_ts_batch_decode_with_kv_cache" (description): CSR page-ID offsets
//    start at zero, increase strictly and end at the number of IDs; each request
//    owns ceil(seq_len / page_size) IDs and every live ID indexes the cache;
//    sequence lengths are positive and at most max_seq_len <= 2^31 - 128.
//  * "block_sparse_attention_with_paged_kv_cache" (Parameters): BSR offsets of
//    shape [B, Hkv, ceil(Sq/q_block_size)+1]; kv_block_size in {8,16,32} or a
//    multiple of 64; (q_block_size * Hq/Hkv) divisible by 8; the convenience
//    path validates live page and sparse metadata on the host first.
//  * "batch_prefill_with_paged_kv_cache": page size 16/32/64/128, D 128/256.
//  * "bsa_attn_sm120_blk64_sage_fwd": block_sparse_num within [0, capacity].
#include <string.h>

#include <algorithm>
#include <unordered_set>
#include <vector>

#include "../../include/pkb.h"
#include "policy.h"

namespace {

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int set_bad(pkb_bad_t* bad, int field, int64_t index) {
  if (bad) {
    bad->field = field;
    bad->index = index;
  }
  return PKB_ERR_METADATA;
}

inline void clear_bad(pkb_bad_t* bad) {
  if (bad) {
    bad->field = PKB_FIELD_NONE;
    bad->index = -1;
  }
}

int kernel_id(int D, int waves, int out_dtype) {
  return (D == 256 ? 100 : 0) + waves * 10 + (out_dtype == PKB_FP32 ? 1 : 0);
}

// CSR offsets: [0] == 0, strictly increasing, [B] == n.
int check_indptr(int B, const int32_t* indptr, int64_t n, int field, pkb_bad_t* bad) {
  if (indptr[0] != 0) return set_bad(bad, field, 0);
  for (int b = 1; b <= B; ++b)
    if (indptr[b] <= indptr[b - 1]) return set_bad(bad, field, b);
  if ((int64_t)indptr[B] != n) return set_bad(bad, field, B);
  return PKB_OK;
}

// Per request: enough CSR entries for the live length, live IDs in [0, P).
int check_live_pages(int B, int P, int ps, const int32_t* indptr, const int32_t* indices,
                     const int32_t* seq_lens, pkb_bad_t* bad) {
  for (int b = 0; b < B; ++b) {
    const int64_t need = cdiv(seq_lens[b], ps);
    if (need > (int64_t)indptr[b + 1] - indptr[b]) return set_bad(bad, PKB_FIELD_KV_INDPTR, b + 1);
    for (int64_t j = indptr[b]; j < indptr[b] + need; ++j)
      if (indices[j] < 0 || indices[j] >= P) return set_bad(bad, PKB_FIELD_KV_INDICES, j);
  }
  return PKB_OK;
}

int check_mask(int mask_type, int window_left) {
  if (mask_type != PKB_MASK_DENSE && mask_type != PKB_MASK_CAUSAL) return PKB_ERR_ARG;
  if (window_left < -1) return PKB_ERR_ARG;
  if (window_left >= 0 && mask_type != PKB_MASK_CAUSAL) return PKB_ERR_ARG;
  return PKB_OK;
}

}  // namespace

extern "C" {

const char* pkb_status_string(int status) {
  switch (status) {
    case PKB_OK: return "ok";
    case PKB_ERR_ARG: return "invalid static argument";
    case PKB_ERR_SHAPE: return "inconsistent shape or stride";
    case PKB_ERR_DTYPE: return "unsupported dtype";
    case PKB_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKB_ERR_METADATA: return "live metadata violates its contract";
    case PKB_ERR_WORKSPACE: return "workspace or work list too small";
    case PKB_ERR_HIP: return "HIP runtime or launch error";
    default: return "unknown status";
  }
}

int pkb_abi_version(void) { return PKB_ABI_VERSION; }

// ------------------------------------------------------------------ block-sparse

int bsa_plan(const bsa_static_args* a, bsa_plan_t* plan) {
  if (!a || !plan) return PKB_ERR_ARG;
  if (a->B < 1 || a->Sq < 1 || a->Hq < 1 || a->Hkv < 1 || a->num_pages < 1 ||
      a->q_block_size < 1 || a->num_cus < 1 || a->page_size < 1)
    return PKB_ERR_ARG;
  if (a->Hq % a->Hkv) return PKB_ERR_SHAPE;
  if (a->qkv_dtype != PKB_BF16 || (a->out_dtype != PKB_BF16 && a->out_dtype != PKB_FP32))
    return PKB_ERR_DTYPE;
  if (a->D != 128 && a->D != 256) return PKB_ERR_UNSUPPORTED;
  const int G = a->Hq / a->Hkv;
  if (((int64_t)a->q_block_size * G) % 8) return PKB_ERR_ARG;
  const int kvbs = a->kv_block_size;
  if (!(kvbs == 8 || kvbs == 16 || kvbs == 32 || (kvbs > 0 && kvbs % 64 == 0))) return PKB_ERR_ARG;
  if (a->max_seq_len_kv < 1 || a->max_seq_len_kv > PKB_MAX_SEQ_LEN) return PKB_ERR_ARG;
  if (check_mask(a->mask_type, a->window_left)) return PKB_ERR_ARG;
  const int64_t rows = (int64_t)a->q_block_size * G;
  if (rows > (1 << 30) || (int64_t)a->Sq * G > (1 << 30)) return PKB_ERR_UNSUPPORTED;
  memset(plan, 0, sizeof(*plan));
  plan->a = *a;
  plan->group = G;
  plan->rows_per_brow = (int)rows;
  plan->num_q_blocks = (int)cdiv(a->Sq, a->q_block_size);
  plan->num_kv_blocks = (int)cdiv(a->max_seq_len_kv, kvbs);
  plan->valid_words = (int)cdiv(a->max_seq_len_kv, 32);
  // 1-4 waves of 32 rows; wider rows take several workgroups (two 4-wave
  // workgroups per CU outran one 8-wave workgroup sharing a barrier)
  plan->waves = rows <= 32 ? 1 : (rows <= 64 ? 2 : 4);
  plan->tile_m = 32 * plan->waves;
  plan->tiles_per_brow = (int)cdiv(rows, plan->tile_m);
  const int64_t gx = (int64_t)plan->num_q_blocks * plan->tiles_per_brow;
  if (gx > 0x7fffffff || a->B > 65535 || a->Hkv > 65535) return PKB_ERR_UNSUPPORTED;
  plan->grid_x = (int)gx;
  plan->grid_y = a->Hkv;
  plan->grid_z = a->B;
  plan->kernel_id = kernel_id(a->D, plan->waves, a->out_dtype);
  return PKB_OK;
}

int bsa_validate(const bsa_plan_t* plan, const int32_t* kv_indptr, const int32_t* kv_indices,
                 int64_t n_indices, const int32_t* block_indptr, const int32_t* block_indices,
                 int64_t n_block_indices, const int32_t* seq_lens, pkb_bad_t* bad) {
  clear_bad(bad);
  if (!plan || !kv_indptr || !seq_lens || !block_indptr) return PKB_ERR_ARG;
  if ((n_indices > 0 && !kv_indices) || (n_block_indices > 0 && !block_indices)) return PKB_ERR_ARG;
  const bsa_static_args& a = plan->a;
  int st = check_indptr(a.B, kv_indptr, n_indices, PKB_FIELD_KV_INDPTR, bad);
  if (st) return st;
  for (int b = 0; b < a.B; ++b)
    if (seq_lens[b] < 0 || seq_lens[b] > a.max_seq_len_kv) return set_bad(bad, PKB_FIELD_SEQ_LENS, b);
  st = check_live_pages(a.B, a.num_pages, a.page_size, kv_indptr, kv_indices, seq_lens, bad);
  if (st) return st;
  const int nq1 = plan->num_q_blocks + 1;
  for (int b = 0; b < a.B; ++b)
    for (int h = 0; h < a.Hkv; ++h)
      for (int r = 0; r < nq1; ++r) {
        const int64_t f = ((int64_t)b * a.Hkv + h) * nq1 + r;
        const int32_t v = block_indptr[f];
        if (v < 0 || v > n_block_indices) return set_bad(bad, PKB_FIELD_BLOCK_INDPTR, f);
        if (r > 0 && v < block_indptr[f - 1]) return set_bad(bad, PKB_FIELD_BLOCK_INDPTR, f);
      }
  std::vector<int32_t> seen_at(plan->num_kv_blocks, -1);
  int32_t row_id = 0;
  for (int b = 0; b < a.B; ++b)
    for (int h = 0; h < a.Hkv; ++h)
      for (int r = 0; r < plan->num_q_blocks; ++r, ++row_id) {
        const int64_t f = ((int64_t)b * a.Hkv + h) * nq1 + r;
        for (int64_t k = block_indptr[f]; k < block_indptr[f + 1]; ++k) {
          const int32_t x = block_indices[k];
          if (x < 0 || x >= plan->num_kv_blocks || seen_at[x] == row_id)
            return set_bad(bad, PKB_FIELD_BLOCK_INDICES, k);
          seen_at[x] = row_id;
        }
      }
  return PKB_OK;
}

// ------------------------------------------------------------------ prefill

static int prefill_static_check(const prefill_static_args* a) {
  if (!a) return PKB_ERR_ARG;
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1 || a->num_pages < 1 || a->total_q < 1 ||
      a->block_table_width < 1 || a->num_cus < 1)
    return PKB_ERR_ARG;
  if (a->Hq % a->Hkv) return PKB_ERR_SHAPE;
  if (a->qkv_dtype != PKB_BF16 || (a->out_dtype != PKB_BF16 && a->out_dtype != PKB_FP32))
    return PKB_ERR_DTYPE;
  if ((a->D != 128 && a->D != 256) ||
      !(a->page_size == 16 || a->page_size == 32 || a->page_size == 64 || a->page_size == 128))
    return PKB_ERR_UNSUPPORTED;
  if (check_mask(a->mask_type, a->window_left)) return PKB_ERR_ARG;
  return PKB_OK;
}

int paged_prefill_validate(const prefill_static_args* a, const int32_t* qo_indptr,
                           const int32_t* seq_lens, const int32_t* block_tables,
                           int64_t row_stride, pkb_bad_t* bad) {
  clear_bad(bad);
  int st = prefill_static_check(a);
  if (st) return st;
  if (!qo_indptr || !seq_lens || !block_tables || row_stride < a->block_table_width)
    return PKB_ERR_ARG;
  st = check_indptr(a->B, qo_indptr, a->total_q, PKB_FIELD_QO_INDPTR, bad);
  if (st) return st;
  for (int b = 0; b < a->B; ++b) {
    const int32_t L = seq_lens[b];
    const int32_t qlen = qo_indptr[b + 1] - qo_indptr[b];
    if (L < 0 || (a->mask_type == PKB_MASK_CAUSAL && qlen > L))
      return set_bad(bad, PKB_FIELD_SEQ_LENS, b);
  }
  for (int b = 0; b < a->B; ++b) {
    const int64_t need = cdiv(seq_lens[b], a->page_size);
    if (need > a->block_table_width) return set_bad(bad, PKB_FIELD_SEQ_LENS, b);
    for (int64_t j = 0; j < need; ++j) {
      const int32_t x = block_tables[(int64_t)b * row_stride + j];
      if (x < 0 || x >= a->num_pages)
        return set_bad(bad, PKB_FIELD_BLOCK_TABLES, (int64_t)b * row_stride + j);
    }
  }
  return PKB_OK;
}

int paged_prefill_plan(const prefill_static_args* a, const int32_t* qo_indptr,
                       const int32_t* seq_lens, pkb_prefill_plan_t* plan, int32_t* worklist,
                       int64_t worklist_cap, int64_t* n_work) {
  int st = prefill_static_check(a);
  if (st) return st;
  if (!qo_indptr || !seq_lens || !plan) return PKB_ERR_ARG;
  const int G = a->Hq / a->Hkv;
  const int waves = 4;
  const int tile_m = 32 * waves;
  const bool causal = a->mask_type == PKB_MASK_CAUSAL;
  struct Item {
    int64_t span;
    int32_t b, row0;
  };
  std::vector<Item> items;
  for (int b = 0; b < a->B; ++b) {
    const int64_t qlen = (int64_t)qo_indptr[b + 1] - qo_indptr[b];
    const int64_t L = seq_lens[b];
    if (qlen < 0) return PKB_ERR_ARG;
    for (int64_t row0 = 0; row0 < qlen * G; row0 += tile_m) {
      const int64_t i0 = row0 / G;
      const int64_t i1 = (std::min(qlen * G, row0 + tile_m) - 1) / G;
      const int64_t p0 = L - qlen + i0, p1 = L - qlen + i1;
      const int64_t hi = causal ? std::min(L, p1 + 1) : L;
      int64_t lo = a->window_left >= 0 ? std::max<int64_t>(0, p0 - a->window_left) : 0;
      lo = (lo / 8) * 8;
      items.push_back({std::max<int64_t>(0, hi - lo), (int32_t)b, (int32_t)row0});
    }
  }
  std::stable_sort(items.begin(), items.end(), [](const Item& x, const Item& y) {
    if (x.span != y.span) return x.span > y.span;
    if (x.b != y.b) return x.b < y.b;
    return x.row0 < y.row0;
  });
  const int64_t n = (int64_t)items.size();
  if (n_work) *n_work = n;
  memset(plan, 0, sizeof(*plan));
  plan->a = *a;
  plan->group = G;
  plan->waves = waves;
  plan->tile_m = tile_m;
  plan->n_work = (int32_t)n;
  plan->grid_x = (int32_t)n;
  plan->grid_y = a->Hkv;
  plan->kernel_id = kernel_id(a->D, waves, a->out_dtype);
  int64_t tot = 0;
  for (const Item& it : items) tot += it.span;
  plan->kv_tokens = tot;
  if (n > 0x7fffffff) return PKB_ERR_UNSUPPORTED;
  if (worklist_cap < n || (n > 0 && !worklist)) return PKB_ERR_WORKSPACE;
  for (int64_t i = 0; i < n; ++i) {
    worklist[2 * i] = items[i].b;
    worklist[2 * i + 1] = items[i].row0;
  }
  return PKB_OK;
}

int paged_prefill_plan_capacity(const prefill_static_args* a, int32_t max_qlen,
                                pkb_prefill_plan_t* plan, int32_t* worklist,
                                int64_t worklist_cap, int64_t* n_work) {
  int st = prefill_static_check(a);
  if (st) return st;
  if (!plan || max_qlen < 1 || max_qlen > a->total_q) return PKB_ERR_ARG;
  const int G = a->Hq / a->Hkv;
  const int waves = 4;
  const int tile_m = 32 * waves;
  // every request may own up to max_qlen rows: ceil(max_qlen * G / tile_m) tiles
  // each, latest tiles first (under bottom-right causal alignment they admit
  // the most keys), requests in order within a tile index
  const int64_t T = cdiv((int64_t)max_qlen * G, tile_m);
  const int64_t n = T * a->B;
  if (n_work) *n_work = n;
  memset(plan, 0, sizeof(*plan));
  plan->a = *a;
  plan->group = G;
  plan->waves = waves;
  plan->tile_m = tile_m;
  plan->n_work = (int32_t)std::min<int64_t>(n, 0x7fffffff);
  plan->grid_x = plan->n_work;
  plan->grid_y = a->Hkv;
  plan->kernel_id = kernel_id(a->D, waves, a->out_dtype);
  plan->kv_tokens = 0;
  if (n > 0x7fffffff) return PKB_ERR_UNSUPPORTED;
  if (worklist_cap < n || !worklist) return PKB_ERR_WORKSPACE;
  int64_t i = 0;
  for (int64_t t = T - 1; t >= 0; --t)
    for (int b = 0; b < a->B; ++b, ++i) {
      worklist[2 * i] = b;
      worklist[2 * i + 1] = (int32_t)(t * tile_m);
    }
  return PKB_OK;
}

// ------------------------------------------------------------------ decode

// Single pass when the batch is wide enough (pkb::decode_coop): one chunk of
// max_seq_len tokens per request, no workspace.  Otherwise the chunk length CH
// (tokens per work item) starts at 1024 (grown while a request would need more
// than 4096 chunks), then halves down to 64 until the largest possible item
// count reaches per_wave items per persistent wave (4 waves per CU).
// Multi-token decode aims at 4 items per wave: its merge reads max_q times more
// partials, so fewer, longer chunks pay off there.
static int decode_split(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_seq_len,
                        int32_t page_size, int32_t num_cus, int max_q, int per_wave,
                        size_t* bytes, int32_t* num_splits, int32_t* split_len) {
  if (B < 1 || Hq < 1 || Hkv < 1 || num_cus < 1 || page_size < 1) return PKB_ERR_ARG;
  if (Hq % Hkv) return PKB_ERR_SHAPE;
  if (D != 128 && D != 256) return PKB_ERR_UNSUPPORTED;
  if (max_seq_len < 1 || max_seq_len > PKB_MAX_SEQ_LEN) return PKB_ERR_ARG;
  if (pkb::decode_coop(B, Hkv, (int)std::min<int64_t>((int64_t)max_q * (Hq / Hkv), 1 << 30), num_cus)) {
    if (num_splits) *num_splits = 1;
    if (split_len) *split_len = max_seq_len;
    if (bytes) *bytes = 0;
    return PKB_OK;
  }
  int64_t CH = 1024;
  while (cdiv(max_seq_len, CH) > 4096) CH *= 2;
  const int64_t waves = 4LL * num_cus;
  while (CH > 64 && (int64_t)B * Hkv * cdiv(max_seq_len, CH) < per_wave * waves) CH /= 2;
  const int64_t S = cdiv(max_seq_len, CH);
  if (num_splits) *num_splits = (int32_t)S;
  if (split_len) *split_len = (int32_t)CH;
  // fp32 partials [B, Hq, S, D+4]: unnormalised O, running max, running sum, pad.
  if (bytes) *bytes = S == 1 ? 0 : (size_t)B * Hq * S * (D + 4) * sizeof(float);
  return PKB_OK;
}

int paged_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                int32_t max_seq_len, int32_t page_size, int32_t num_cus,
                                size_t* bytes, int32_t* num_splits, int32_t* split_len) {
  return decode_split(B, Hq, Hkv, D, max_seq_len, page_size, num_cus, 1, 8, bytes, num_splits,
                      split_len);
}

int paged_decode_validate(int32_t B, int32_t num_pages, int32_t page_size, int32_t max_seq_len,
                          const int32_t* kv_indptr, const int32_t* kv_indices, int64_t n_indices,
                          const int32_t* seq_lens, pkb_bad_t* bad) {
  clear_bad(bad);
  if (B < 1 || num_pages < 1 || page_size < 1 || !kv_indptr || !seq_lens) return PKB_ERR_ARG;
  if (max_seq_len < 1 || max_seq_len > PKB_MAX_SEQ_LEN) return PKB_ERR_ARG;
  if (n_indices > 0 && !kv_indices) return PKB_ERR_ARG;
  int st = check_indptr(B, kv_indptr, n_indices, PKB_FIELD_KV_INDPTR, bad);
  if (st) return st;
  for (int b = 0; b < B; ++b)
    if (seq_lens[b] < 1 || seq_lens[b] > max_seq_len) return set_bad(bad, PKB_FIELD_SEQ_LENS, b);
  return check_live_pages(B, num_pages, page_size, kv_indptr, kv_indices, seq_lens, bad);
}

int paged_decode_q_workspace_size(int32_t B, int32_t max_q, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t max_seq_len, int32_t page_size, int32_t num_cus,
                                  size_t* bytes, int32_t* num_splits, int32_t* split_len) {
  if (max_q < 1) return PKB_ERR_ARG;
  size_t one = 0;
  int st = decode_split(B, Hq, Hkv, D, max_seq_len, page_size, num_cus, max_q, max_q > 1 ? 4 : 8,
                        &one, num_splits, split_len);
  if (st) return st;
  // fp32 partials [B, max_q, Hq, S, D+4]
  if (bytes) *bytes = one * (size_t)max_q;
  return PKB_OK;
}

int paged_decode_q_validate(int32_t B, int32_t num_pages, int32_t page_size, int32_t max_seq_len,
                            const int32_t* kv_indptr, const int32_t* kv_indices, int64_t n_indices,
                            const int32_t* seq_lens, const int32_t* qo_indptr, int64_t total_q,
                            int32_t seq_len_q, int32_t max_seq_len_q, int32_t mask_type,
                            pkb_bad_t* bad) {
  clear_bad(bad);
  if (B < 1 || num_pages < 1 || page_size < 1 || !kv_indptr || !seq_lens) return PKB_ERR_ARG;
  if (max_seq_len < 1 || max_seq_len > PKB_MAX_SEQ_LEN) return PKB_ERR_ARG;
  if (n_indices > 0 && !kv_indices) return PKB_ERR_ARG;
  if (mask_type != PKB_MASK_DENSE && mask_type != PKB_MASK_CAUSAL) return PKB_ERR_ARG;
  if (qo_indptr ? (max_seq_len_q < 1 || total_q < 1) : seq_len_q < 1) return PKB_ERR_ARG;
  int st = check_indptr(B, kv_indptr, n_indices, PKB_FIELD_KV_INDPTR, bad);
  if (st) return st;
  for (int b = 0; b < B; ++b)
    if (seq_lens[b] < 1 || seq_lens[b] > max_seq_len) return set_bad(bad, PKB_FIELD_SEQ_LENS, b);
  if (qo_indptr) {
    if (qo_indptr[0] != 0) return set_bad(bad, PKB_FIELD_QO_INDPTR, 0);
    for (int b = 0; b < B; ++b) {
      const int64_t d = (int64_t)qo_indptr[b + 1] - qo_indptr[b];
      if (d < 1 || d > max_seq_len_q) return set_bad(bad, PKB_FIELD_QO_INDPTR, b + 1);
    }
    if ((int64_t)qo_indptr[B] != total_q) return set_bad(bad, PKB_FIELD_QO_INDPTR, B);
  }
  if (mask_type == PKB_MASK_CAUSAL)
    for (int b = 0; b < B; ++b) {
      const int64_t qlen = qo_indptr ? (int64_t)qo_indptr[b + 1] - qo_indptr[b] : seq_len_q;
      if (qlen > seq_lens[b]) return set_bad(bad, PKB_FIELD_SEQ_LENS, b);
    }
  return check_live_pages(B, num_pages, page_size, kv_indptr, kv_indices, seq_lens, bad);
}

// ------------------------------------------------------------------ sage

int bsa_sage_validate(const int32_t* index, int32_t capacity, int32_t block_sparse_num,
                      const int32_t* block_sizes, int32_t block_sizes_rank, const int32_t* nums,
                      int32_t uniform, int32_t B, int32_t H, int32_t Sq, int32_t Sk,
                      pkb_bad_t* bad) {
  clear_bad(bad);
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || capacity < 0 || !index) return PKB_ERR_ARG;
  if (block_sparse_num < 0 || block_sparse_num > capacity) return PKB_ERR_ARG;
  if (block_sizes && (block_sizes_rank < 1 || block_sizes_rank > 3)) return PKB_ERR_ARG;
  const int64_t nqb = cdiv(Sq, 64), nkb = cdiv(Sk, 64);
  const bool use_nums = nums && !uniform;
  const int64_t rows = (int64_t)B * H * nqb;
  if (use_nums)
    for (int64_t f = 0; f < rows; ++f)
      if (nums[f] < 0 || nums[f] > capacity) return set_bad(bad, PKB_FIELD_Q2K_NUMS, f);
  std::vector<int64_t> seen_at(nkb, -1);
  for (int64_t row = 0; row < rows; ++row) {
    const int n = use_nums ? nums[row] : block_sparse_num;
    for (int k = 0; k < n; ++k) {
      const int64_t f = row * capacity + k;
      const int32_t x = index[f];
      if (x < 0 || x >= nkb || seen_at[x] == row) return set_bad(bad, PKB_FIELD_Q2K_INDEX, f);
      seen_at[x] = row;
    }
  }
  if (block_sizes) {
    const int64_t cnt = (block_sizes_rank == 1 ? 1 : (block_sizes_rank == 2 ? B : (int64_t)B * H)) * nkb;
    for (int64_t f = 0; f < cnt; ++f)
      if (block_sizes[f] < 0 || block_sizes[f] > 64) return set_bad(bad, PKB_FIELD_BLOCK_SIZES, f);
  }
  return PKB_OK;
}

// ------------------------------------------------------------------ QSA

int qsa_validate(int32_t T, int32_t NB, const int32_t* lo, const int32_t* hi,
                            const int32_t* blk_base, const int32_t* tok_base,
                            const int32_t* block_first, const int32_t* block_last,
                            pkb_bad_t* bad) {
  clear_bad(bad);
  if (T < 1 || NB < 1 || !lo || !hi || !blk_base || !tok_base || !block_first || !block_last)
    return PKB_ERR_ARG;
  // sequences: runs of tokens sharing tok_base, each starting at its own index
  std::vector<int32_t> seq_end(T);
  for (int32_t t = 0; t < T;) {
    if (tok_base[t] != t) return set_bad(bad, PKB_FIELD_TOK_BASE, t);
    int32_t e = t + 1;
    while (e < T && tok_base[e] == t) ++e;
    if (e < T && tok_base[e] != e) return set_bad(bad, PKB_FIELD_TOK_BASE, e);
    const int64_t nblk = cdiv(e - t, 4);
    for (int32_t u = t; u < e; ++u) {
      if (blk_base[u] != blk_base[t] || blk_base[t] < 0 || blk_base[t] + nblk > NB)
        return set_bad(bad, PKB_FIELD_BLK_BASE, u);
      seq_end[u] = e - 1;
    }
    t = e;
  }
  for (int32_t t = 0; t < T;) {
    const int32_t e = seq_end[t] + 1;
    for (int64_t m = 0; m < cdiv(e - t, 4); ++m) {
      const int64_t nb = blk_base[t] + m;
      if (block_first[nb] != t + 4 * m) return set_bad(bad, PKB_FIELD_BLOCK_FIRST, nb);
      if (block_last[nb] != std::min<int64_t>(t + 4 * m + 3, e - 1))
        return set_bad(bad, PKB_FIELD_BLOCK_LAST, nb);
    }
    t = e;
  }
  for (int32_t t = 0; t < T; ++t) {
    if (lo[t] > hi[t]) continue;
    if (lo[t] < tok_base[t] || lo[t] > seq_end[t]) return set_bad(bad, PKB_FIELD_LO, t);
    if (hi[t] > seq_end[t]) return set_bad(bad, PKB_FIELD_HI, t);
  }
  return PKB_OK;
}

}  // extern "C"
