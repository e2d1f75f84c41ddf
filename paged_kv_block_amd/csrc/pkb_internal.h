// pkb_internal.h -- kernel parameter blocks and launcher declarations shared by
// the host API (api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "policy.h"

namespace pkb {

enum AttnMode { kModeBsa = 0, kModePrefill = 1, kModeDecode = 2 };

// Keys per KV tile of the bf16 attention kernel (one LDS tile = 8 chunks of 8).
constexpr int kKvTile = 64;

// Everything the bf16 attention kernel needs, passed by value.
struct AttnParams {
  const uint16_t* q;          // bf16 bits; token-major [tokens, Hq, D]
  const uint16_t* k;          // page pools (element strides below)
  const uint16_t* v;
  void* out;                  // [tokens, Hq, D] bf16 or fp32
  float* lse;                 // [tokens, Hq] or null
  float* part;                // decode split partials [B, maxq, Hq, S, D+4] or null
  const int32_t* kv_indptr;   // CSR page IDs (bsa, decode)
  const int32_t* kv_indices;
  const int32_t* block_tables;  // row-strided table (prefill)
  const int32_t* seq_lens;
  const int32_t* qo_indptr;     // prefill; multi-token decode (null: Sq rows per request)
  const int32_t* block_indptr;  // bsa [B, Hkv, nqb+1]
  const int32_t* block_indices;
  const uint32_t* valid_bits;   // bsa [B, valid_words] or null
  const int32_t* worklist;      // prefill (request, first row) pairs
  int64_t kv_page_stride, kv_head_stride, bt_stride;
  int B, Sq, Hq, Hkv, G, page_size;
  int qbs, kvbs, nqb, tiles_per_brow, rows_per_brow, valid_words;
  int causal, window_left;
  int num_splits, split_len;
  int maxq;           // decode: query rows per request in the partials workspace
  int out_f32;
  float scale_log2;   // softmax scale * log2(e)
  float out_scale;
};

// Dedicated decode kernels (at most kDecodeMaxGroup query rows per KV head).
// The split kernel is a persistent grid of single-wave workgroups,
// decode_waves_per_cu(D) per CU (one per SIMD), each keeping one 32-key group
// of loads in flight while it computes the previous one; the cooperative
// kernel runs kCoopWaves such waves per workgroup, one workgroup per CU.
constexpr int decode_waves_per_cu(int) { return 4; }

struct DecodeParams {
  const uint16_t* q;          // [tokens, Hq, D]
  const uint16_t* k;
  const uint16_t* v;
  void* out;                  // [tokens, Hq, D]
  float* lse;                 // [tokens, Hq] or null
  float* part;                // [B, maxq, Hq, S, D+4] or null (O, m, l, pad)
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* seq_lens;
  const int32_t* qo_indptr;   // multi-token packed rows, or null: Sq rows per request
  int64_t kv_page_stride, kv_head_stride;
  int B, Hq, Hkv, G, page_size, window_left;
  int Sq, maxq, causal;       // query tokens per request (fixed), partial rows, mask
  int num_splits, split_len, out_f32;
  float scale_log2;
  float out_scale;
};

struct MergeParams {
  const float* part;            // [B, maxq, Hq, num_splits, D+4]
  const int32_t* seq_lens;
  const int32_t* qo_indptr;     // packed query rows, or null: Sq rows per request
  void* out;
  float* lse;
  int B, Hq, num_splits, split_len, out_f32;
  int maxq, Sq;
  float out_scale;
};

struct SageParams {
  const int8_t* q;
  const int8_t* k;
  const uint8_t* v;           // e4m3 HDS [B, H, 128, Skp]
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  const int32_t* index;
  const int32_t* nums;        // null => block_sparse_num
  const int32_t* block_sizes; // null => 64
  uint16_t* out;
  float* lse;                 // null => no LSE output; else [B, H, Sq] natural log
  int B, H, Sq, Sk, Skp, nqb, nkb, capacity, block_sparse_num;
  int bs_rank, qs_len;
  int causal;                 // token-level causal, query i at position Sk - Sq + i
  int contig;                 // selected blocks are idx[0], idx[0] + 1, ... (trusted)
  float scale_log2;
};

// Packed-query token-granular sparse attention (non-paged packed K/V).
struct QsaParams {
  const uint16_t* q;          // [T, Hq, D]
  const uint16_t* k;          // [T, Hkv, D]
  const uint16_t* v;
  const uint8_t* sel;         // [T, NB]
  const int32_t* lo;          // [T] inclusive key bounds
  const int32_t* hi;
  const int32_t* blk_base;    // [T] first global block / token of the token's sequence
  const int32_t* tok_base;
  uint16_t* out;              // [T, Hq, D] bf16 or null
  float* out_f32;             // [T, Hq, D] or null
  float* lse;                 // [Hq, T] or null
  int T, NB, Hq, Hkv, G;
  int sel16;                  // NB % 16 == 0 and sel 16-byte aligned: 16-byte bitmap loads
  float scale_log2;
};

hipError_t launch_attn(const AttnParams& p, int D, int waves, int mode, dim3 grid,
                       hipStream_t stream);
// page sizes that are not a multiple of 8 (launch_attn forwards them here)
hipError_t launch_attn_ragged(const AttnParams& p, int D, int waves, int mode, dim3 grid,
                              hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int D, int grid, hipStream_t stream);
hipError_t launch_decode_coop(const DecodeParams& p, int D, int grid, hipStream_t stream);
hipError_t launch_decode_merge(const MergeParams& p, int D, hipStream_t stream);

// Fixed per-device scratch for the split partials of paged_decode_run_noalloc:
// its device address on the current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
hipError_t decode_scratch(void** ptr);
hipError_t launch_sage(const SageParams& p, hipStream_t stream);
hipError_t launch_qsa(const QsaParams& p, int D, hipStream_t stream);

}  // namespace pkb
