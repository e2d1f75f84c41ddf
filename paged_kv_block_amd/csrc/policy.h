// policy.h -- launch-policy rules shared by the planner (host.cpp, no HIP) and
// the launchers (api.cpp).
#pragma once

namespace pkb {

// Query rows of one KV head that the decode kernels hold: the 16 columns of
// v_mfma_f32_16x16x32_bf16 (single-token decode: the GQA group; multi-token
// decode: query tokens x group).
constexpr int kDecodeMaxGroup = 16;
// Waves of one cooperative decode workgroup, and the most requests it orders in LDS.
constexpr int kCoopWaves = 4;
constexpr int kCoopMaxBatch = 256;

// Single-pass (cooperative) decode: every (request, KV head) pair is one work
// item, so the batch needs at least two of them per compute unit to keep the
// persistent grid balanced; the items' query rows must fit the MFMA columns and
// the batch the in-LDS ordering.
inline bool decode_coop(int B, int Hkv, int rows_per_kv_head, int num_cus) {
  return rows_per_kv_head <= kDecodeMaxGroup && B <= kCoopMaxBatch &&
         (long long)B * Hkv >= 2LL * num_cus;
}

}  // namespace pkb
