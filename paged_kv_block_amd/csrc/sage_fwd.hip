// sage_fwd.hip -- prequantized block-sparse attention (int8 Q/K, fp8 E4M3 V) for
// gfx950.
//
// What is computed (FlashInfer page "bsa_attn_sm120_blk64_sage_fwd", Parameters
// and Notes): for head (b, h) and query row i in query block r = i / 64, over
// the tokens of the selected 64-token KV blocks q2k_block_index[b,h,r,:n] (n from
// the per-row counts or the scalar block_sparse_num), block beta contributing
// its first block_sizes[..beta] tokens (< Sk):
//     s_j = softmax_scale * (q_int8[i] . k_int8[j]) * q_scale[i/32] * k_scale[j/64]
//     out[i, d] = sum_j softmax(s)_j * e4m3(v[d, j]) * v_scale[d]    (bf16)
// A row with no selected block is written as zeros.
//
// One workgroup = (b, h, query block of 64 rows): two waves of 32 rows.  Per
// selected KV block (64 tokens, one tile):
//   * K [64 keys x 128] int8 goes to LDS row-major; S^T = K Q^T runs on
//     v_mfma_i32_32x32x32_i8 (M = keys, N = query rows, K = 32 dims), so each
//     lane holds 16 keys of one query row per 32-key half;
//   * the int32 scores are scaled once per (wave, block): q_scale is constant
//     over a wave's 32 rows and k_scale over the block;
//   * online softmax in base 2; P (in [0, 1]) is scaled by 448 and packed to
//     OCP E4M3 (v_cvt_pk_fp8_f32) as a hi part plus the rounding residual;
//   * V arrives in HDS layout (tokens contiguous per head dim), which is already
//     the K-contiguous A operand of O^T += V^T P^T on v_mfma_f32_32x32x64_f8f6f4.
//     Its 64-byte rows are staged in LDS with the 4-key groups reordered
//     (even groups, then odd) so that lane half h reads, as 32 contiguous bytes,
//     exactly the keys {4h + 8a + c} its S^T accumulator holds;
//   * the epilogue applies v_scale[d] / (448 * l) and writes bf16.
// The next block's K and V are loaded into registers while the current block
// computes.
#include "device_common.h"
#include "pkb_internal.h"

namespace pkb {

namespace {
constexpr int kKRow = 128 + 16;  // LDS bytes per K row (pad: distinct banks for 8 rows)
constexpr int kVRow = 64 + 16;   // LDS bytes per V^T row (64 fp8 keys + pad)
constexpr int kLds = 64 * kKRow + 128 * kVRow;
constexpr float kP8 = 448.f;     // P is stored as P * 448 (the E4M3 maximum)
}  // namespace

__device__ __forceinline__ int sage_block_size(const SageParams& p, int b, int h, int beta) {
  if (p.bs_rank == 0) return 64;
  if (p.bs_rank == 1) return p.block_sizes[beta];
  if (p.bs_rank == 2) return p.block_sizes[(int64_t)b * p.nkb + beta];
  return p.block_sizes[((int64_t)b * p.H + h) * p.nkb + beta];
}

__global__ void __launch_bounds__(128) sage_kernel(const SageParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
  unsigned char* sK = smem;
  unsigned char* sV = smem + 64 * kKRow;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int hh = lane >> 5;
  const int ql = lane & 31;
  const int r = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * p.H + h;

  const int64_t row_base = (int64_t)r * p.capacity;
  const int32_t* idx = p.index + (bh * p.nqb) * p.capacity + row_base;
  const int n = p.nums ? p.nums[bh * p.nqb + r] : p.block_sparse_num;

  const int row = r * 64 + wave * 32 + ql;
  const bool row_ok = row < p.Sq;

  // Q^T fragments (B operand of S^T): k-step s covers dims 32s..32s+31; lane
  // half hh holds dims 32s + 16hh .. +15.
  i32x4 qf[4];
  {
    const int8_t* qrow = p.q + (bh * p.Sq + row) * 128 + 16 * hh;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row_ok) x = ld_global_16(qrow + 32 * s);
      qf[s] = __builtin_bit_cast(i32x4, x);
    }
  }
  const float qs = p.q_scale[bh * p.qs_len + (r * 64 + wave * 32) / 32];

  f32x16 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[d][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // staging: thread t loads K row t/2 half t%2 (64 B) and V^T row t (64 B)
  const int krow = tid >> 1, khalf = tid & 1;
  u32x4 kreg[4], vreg[4];
  auto load_block = [&](int beta, int kv) {
    const int8_t* kp = p.k + (bh * p.Sk + (int64_t)beta * 64 + krow) * 128 + 64 * khalf;
    const bool kok = krow < kv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (kok) x = ld_global_16(kp + 16 * i);
      kreg[i] = x;
    }
    const uint8_t* vp = p.v + (bh * 128 + tid) * p.Skp + (int64_t)beta * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) vreg[i] = ld_global_16(vp + 16 * i);
  };
  auto store_block = [&](int kv) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4*)(sK + krow * kKRow + 64 * khalf + 16 * i) = kreg[i];
    // zero the bytes of keys >= kv (their storage may hold anything), then put
    // even 4-key groups first and odd ones second
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) w[4 * i + e] = vreg[i][e];
#pragma unroll
    for (int gq = 0; gq < 16; ++gq) {
      const int keep = min(max(kv - 4 * gq, 0), 4);          // valid keys in this group
      const uint32_t mask = keep >= 4 ? 0xFFFFFFFFu : ((1u << (8 * keep)) - 1u);
      w[gq] &= mask;
    }
    u32x4 e0 = {w[0], w[2], w[4], w[6]}, e1 = {w[8], w[10], w[12], w[14]};
    u32x4 o0 = {w[1], w[3], w[5], w[7]}, o1 = {w[9], w[11], w[13], w[15]};
    unsigned char* vr = sV + tid * kVRow;
    *(u32x4*)(vr + 0) = e0;
    *(u32x4*)(vr + 16) = e1;
    *(u32x4*)(vr + 32) = o0;
    *(u32x4*)(vr + 48) = o1;
  };

  const float sl2 = p.scale_log2;
  int beta = n > 0 ? idx[0] : 0;
  int kv = 0;
  if (n > 0) {
    kv = min(sage_block_size(p, b, h, beta), p.Sk - beta * 64);
    load_block(beta, kv);
  }
  for (int t = 0; t < n; ++t) {
    const int cur_kv = kv;
    const int cur_beta = beta;
    __syncthreads();                 // previous block's LDS reads are done
    store_block(cur_kv);
    __syncthreads();
    if (t + 1 < n) {                 // next block in flight during this one
      beta = idx[t + 1];
      kv = min(sage_block_size(p, b, h, beta), p.Sk - beta * 64);
      load_block(beta, kv);
    }
    const float ks = p.k_scale[bh * p.nkb + cur_beta];
    const float sc = qs * ks * sl2;

    // ---- S^T = K Q^T, two 32-key halves ----
    i32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0;
      const unsigned char* kr = sK + (32 * kb + ql) * kKRow + 16 * hh;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const i32x4 a = *(const i32x4*)(kr + 32 * s);
        sacc[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qf[s], sacc[kb], 0, 0, 0);
      }
    }
    // ---- scale, mask keys >= kv, online softmax ----
    float sv[2][16];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3);
        const float x = key < cur_kv ? (float)sacc[kb][i] * sc : -INFINITY;
        sv[kb][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = half_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(sv[kb][i] - m_use);
        sv[kb][i] = e;
        psum += e;
      }
    if (m_new != m_run) {
      const float alpha = fast_exp2(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
    }
    l_run += psum;
    m_run = m_new;

    // ---- P^T -> fp8 (x448), as hi + lo parts: E4M3 alone keeps 3 mantissa
    // bits, too coarse for rows with only a few admitted keys; hi + lo gives
    // about 7.  Slot j < 16: first 32-key half, else second. ----
    i32x8 pb, pl;
#pragma unroll
    for (int wd = 0; wd < 8; ++wd) {
      const int kb = wd >> 2;
      const int i0 = 4 * (wd & 3);
      const float x0 = sv[kb][i0] * kP8, x1 = sv[kb][i0 + 1] * kP8;
      const float x2 = sv[kb][i0 + 2] * kP8, x3 = sv[kb][i0 + 3] * kP8;
      int hi = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, hi, true);
      const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
      const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - h01[0], x1 - h01[1], 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(x2 - h23[0], x3 - h23[1], lo, true);
      pb[wd] = hi;
      pl[wd] = lo;
    }
    // ---- O^T += V^T P^T: four 32-dim blocks, K = 64 keys ----
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const unsigned char* vrp = sV + (32 * d + ql) * kVRow + 32 * hh;
      const u32x4 a0 = *(const u32x4*)(vrp);
      const u32x4 a1 = *(const u32x4*)(vrp + 16);
      i32x8 a;
      a[0] = a0[0]; a[1] = a0[1]; a[2] = a0[2]; a[3] = a0[3];
      a[4] = a1[0]; a[5] = a1[1]; a[6] = a1[2]; a[7] = a1[3];
      oacc[d] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, oacc[d], 0, 0, 0, 0, 0, 0);
      oacc[d] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pl, oacc[d], 0, 0, 0, 0, 0, 0);
    }
  }

  // ---- epilogue: O = O^T * v_scale[d] / (448 l) -> bf16 [B, H, Sq, 128] ----
  const float l_tot = half_sum(l_run);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.f / (kP8 * l_tot) : 0.f;
  const float* vsc = p.v_scale + bh * 128;
  uint16_t* o = p.out + (bh * p.Sq + row) * 128;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * d + 8 * g4 + 4 * hh;
      const f32x4 s4 = *(const f32x4*)(vsc + d0);
      u32x2 w;
      w[0] = pack_bf16x2(oacc[d][4 * g4] * s4[0] * inv, oacc[d][4 * g4 + 1] * s4[1] * inv);
      w[1] = pack_bf16x2(oacc[d][4 * g4 + 2] * s4[2] * inv, oacc[d][4 * g4 + 3] * s4[3] * inv);
      *(u32x2*)(o + d0) = w;
    }
}

hipError_t launch_sage(const SageParams& p, hipStream_t stream) {
  SageParams arg = p;
  void* args[] = {(void*)&arg};
  return hipLaunchKernel((const void*)sage_kernel, dim3(p.nqb, p.H, p.B), dim3(128), args, 0,
                         stream);
}

}  // namespace pkb
