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
// A row with no selected block is written as zeros.  Two additions beyond the
// page: an optional token-level causal mask (the block-sparse page's rule,
// bottom-right aligned: query i at position Sk - Sq + i) and an optional LSE
// output (natural log of the sum of exp(s_j) over admitted keys).  With
// contiguous selections (the page's contiguous_block_indices promise) block t
// is the first selected index plus t.
//
// One workgroup = (b, h, query block of 64 rows): two waves of 32 rows.  Per
// selected KV block (64 tokens, one tile):
//   * K [64 keys x 128] int8 and V^T [128 dims x 64 keys] fp8 are copied HBM ->
//     LDS by direct-to-LDS loads (global_load_lds_dwordx4) into a ring of
//     kNStage blocks, kNStage - 1 blocks ahead of use;
//   * S^T = K Q^T runs on v_mfma_i32_32x32x32_i8 (M = keys, N = query rows,
//     K = 32 dims).  The K rows are stored permuted (sage_key_of_row) so that
//     lane half h's accumulator holds keys 32h .. 32h+31 in order;
//   * the int32 scores are scaled once per (wave, block): q_scale is constant
//     over a wave's 32 rows and k_scale over the block;
//   * online softmax in base 2 whose reference moves only when a row max
//     passes it by more than 2 (so the rescale of O is rare and P <= 4); the
//     exponent carries log2(112), so the exp returns P * 112 <= 448, inside
//     E4M3's range; blocks that no row of the wave cuts skip the key mask;
//     P * 112 is packed to OCP E4M3
//     (v_cvt_pk_fp8_f32) as a hi part plus the rounding residual -- E4M3 alone
//     keeps 3 mantissa bits, too coarse for rows with only a few admitted keys;
//   * V arrives in HDS layout (tokens contiguous per head dim), which is the
//     K-contiguous A operand of O^T += V^T P^T on v_mfma_f32_32x32x64_f8f6f4:
//     lane half h reads the 32 contiguous bytes of keys 32h .. 32h+31, the
//     same keys (in the same order) its P^T operand holds.  Keys at or past a
//     partial block's size are zeroed in LDS (their storage may hold NaN codes);
//   * the epilogue applies v_scale[d] / l (O and l both carry the factor 112)
//     and writes bf16.
// Workgroups are dealt round-robin over the 8 XCDs; each XCD gets a contiguous
// run of (head, query block) items so the K/V of the heads it works on stay in
// its L2.
#include "device_common.h"
#include "pkb_internal.h"

namespace pkb {

namespace {
constexpr int kKRowB = 128;                // LDS bytes per K row
constexpr int kVRowB = 64;                 // LDS bytes per V^T row (64 fp8 keys)
constexpr int kKTile = 64 * kKRowB;        // 8 KB
constexpr int kVTile = 128 * kVRowB;       // 8 KB
constexpr int kStage = kKTile + kVTile;
constexpr int kNStage = 2;
static_assert(kNStage >= 2 && kNStage <= 4, "wait counts cover up to two blocks in flight");
constexpr int kLA = kNStage - 1;           // blocks copied ahead of the one computed
constexpr int kLds = kNStage * kStage;     // 32 KB: four workgroups (two waves per SIMD) per CU
// The softmax reference only moves when a row max passes it by more than
// kSlack (log2 units), so P <= 2^kSlack; P * kP8 <= 448, the E4M3 maximum.
constexpr float kSlack = 2.f;
constexpr float kP8 = 112.f;
constexpr float kLog2P8 = 6.807354922057604f;   // log2(112)
constexpr int kXcds = 8;
}  // namespace

__device__ __forceinline__ int sage_block_size(const SageParams& p, int b, int h, int beta) {
  if (p.bs_rank == 0) return 64;
  if (p.bs_rank == 1) return ld_const(p.block_sizes, beta);
  if (p.bs_rank == 2) return ld_const(p.block_sizes, (int64_t)b * p.nkb + beta);
  return ld_const(p.block_sizes, ((int64_t)b * p.H + h) * p.nkb + beta);
}

// Key held by LDS K row rho: the S^T accumulator of lane half h holds rows
// 32kb + 8a + 4h + c (element 4a + c of block kb), which is made key
// 32h + 16kb + 4a + c.
__device__ __forceinline__ int sage_key_of_row(int rho) {
  const int kb = rho >> 5, a = (rho >> 3) & 3, h = (rho >> 2) & 1, c = rho & 3;
  return 32 * h + 16 * kb + 4 * a + c;
}

// 16 bytes per lane from the wave-uniform address base + byte offset off to
// LDS address lds_addr + 16 * lane (global_load_lds_dwordx4 in its scalar-base
// form; the LDS base is taken from M0, which needs one wait state after the
// SALU write).  Inline assembly keeps the compiler from ordering later LDS
// reads after every copy in flight: the kernel orders them itself.
__device__ __forceinline__ void sage_dma16(const void* base, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(lds_addr) : "m0");
}

template <int N>
__device__ __forceinline__ void sage_wait_vmcnt() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__global__ void __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2)))
sage_kernel(const SageParams p) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int hh = lane >> 5;
  const int ql = lane & 31;

  // XCD-aware item order: workgroup g runs on XCD g % 8 and is that XCD's
  // (g / 8)-th; XCD x takes items [x * per, (x + 1) * per), head-major.
  const int total = p.nqb * p.H * p.B;
  const int per = (total + kXcds - 1) / kXcds;
  const int item = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
  if (item >= total) return;
  const int r = item % p.nqb;
  const int64_t bh = item / p.nqb;
  const int b = (int)(bh / p.H), h = (int)(bh % p.H);

  const int32_t* idx = p.index + (bh * p.nqb + r) * p.capacity;
  const int n = p.nums ? ld_const(p.nums, bh * p.nqb + r) : p.block_sparse_num;
  // contiguous selections: block t is the first index + t (no index loads)
  const int beta0 = (p.contig && n > 0) ? ld_const(idx, 0) : 0;

  const int row = r * 64 + wave * 32 + ql;
  const bool row_ok = row < p.Sq;
  // causal: row i sits at position Sk - Sq + i; a block starting past the
  // workgroup's last position admits nothing
  const int p_row = p.Sk - p.Sq + row;
  const int p_last = p.Sk - p.Sq + min(r * 64 + 63, p.Sq - 1);

  // block metadata: id and valid-token count (0: nothing to do).  Ids outside
  // [0, nkb) count as empty, so even a wrong contiguity promise stays in bounds.
  struct BlockMeta { int beta, kv; };
  auto block_meta = [&](int t) -> BlockMeta {
    BlockMeta m;
    m.beta = p.contig ? beta0 + t : ld_const(idx, t);
    m.kv = 0;
    if ((unsigned)m.beta < (unsigned)p.nkb && !(p.causal && m.beta * 64 > p_last))
      m.kv = min(sage_block_size(p, b, h, m.beta), p.Sk - m.beta * 64);
    return m;
  };
  // this wave's share of block t's copies into ring stage t % kNStage: K rows
  // (permuted, pieces swizzled by (row >> 1) & 7) and V^T rows (pieces swizzled
  // by (row >> 2) & 3); K rows past Sk re-read the block's first row
  auto issue_block = [&](const BlockMeta& m, int t) {
    const uint32_t kst = lds_base + (t % kNStage) * kStage;
    const uint32_t vst = kst + kKTile;
    const int8_t* kb = p.k + (bh * p.Sk + m.beta * 64) * 128;
    const uint8_t* vb = p.v + bh * 128 * p.Skp + m.beta * 64;
    // the per-key test is needed only for a block that ends past Sk
    const bool whole = m.beta * 64 + 64 <= p.Sk;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = wave * 4 + ii;
      const int rho = 8 * i + (lane >> 3);
      const int kp = (lane & 7) ^ ((rho >> 1) & 7);
      int key = sage_key_of_row(rho);
      if (!whole && m.beta * 64 + key >= p.Sk) key = 0;
      sage_dma16(kb, (uint32_t)(key * 128 + kp * 16), kst + i * 1024);
      const int d = 16 * i + (lane >> 2);
      const int vp = (lane & 3) ^ ((d >> 2) & 3);
      sage_dma16(vb, (uint32_t)(d * p.Skp + vp * 16), vst + i * 1024);
    }
  };

  // ---- prologue: first blocks in flight, then Q ----
  BlockMeta bm[kLA + 1];
#pragma unroll
  for (int k = 0; k <= kLA; ++k) {
    bm[k].kv = 0;
    if (k < n) {
      bm[k] = block_meta(k);
      if (bm[k].kv > 0 && k < kLA) issue_block(bm[k], k);
    }
  }
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
  sage_wait_vmcnt<0>();   // no load issued before the loop is pending inside it

  f32x16 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[d][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale_log2;
  const int koff_row = ql * kKRowB;
  const int kswz = (ql >> 1) & 7;                    // rows 32kb + ql: same low bits
  const int vswz = (ql >> 2) & 3;                    // rows 32d + ql

  // P^T operands (fp8 hi and lo parts): kept across blocks, so that each
  // conversion's untouched half starts from the register it overwrites
  // rather than from a fresh copy
  i32x8 pb = {}, pl = {};
  for (int t = 0; t < n; ++t) {
    // block t landed in every wave's share; blocks t+1 .. t+kLA-1 may still fly
    int ahead = 0;
#pragma unroll
    for (int k = 1; k < kLA; ++k) ahead += (t + k < n && bm[k].kv > 0) ? 1 : 0;
    if (ahead == 0) sage_wait_vmcnt<0>();
    else if (ahead == 1) sage_wait_vmcnt<8>();
    else sage_wait_vmcnt<16>();
    __syncthreads();                 // ... and is visible; block t-1's stage is free
    if (bm[kLA].kv > 0) issue_block(bm[kLA], t + kLA);
    const int kv = bm[0].kv;
    const unsigned char* sK = smem + (t % kNStage) * kStage;
    const unsigned char* sV = sK + kKTile;
    if (kv > 0 && kv < 64) {
      // partial block: zero the V bytes of keys >= kv (row d = tid)
      unsigned char* vr = (unsigned char*)sV + tid * kVRowB;
#pragma unroll
      for (int lp = 0; lp < 4; ++lp) {
        if (16 * lp + 15 < kv) continue;
        const int pp = lp ^ ((tid >> 2) & 3);
        u32x4 x = *(u32x4*)(vr + pp * 16);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int k0 = 16 * lp + 4 * w;
          const int keep = min(max(kv - k0, 0), 4);
          x[w] &= keep >= 4 ? 0xFFFFFFFFu : ((1u << (8 * keep)) - 1u);
        }
        *(u32x4*)(vr + pp * 16) = x;
      }
      __syncthreads();
    }
    if (kv > 0) {
      const float ks = ld_const(p.k_scale, bh * p.nkb + bm[0].beta);
      const float sc = qs * ks * sl2;
      // ---- S^T = K Q^T, two 32-key blocks ----
      i32x4 kf[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          kf[kb][s] = *(const i32x4*)(sK + kb * 32 * kKRowB + koff_row + (((2 * s + hh) ^ kswz) * 16));
      __builtin_amdgcn_sched_barrier(0);
      i32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] = 0;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          sacc[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[kb][s], qf[s], sacc[kb], 0, 0, 0);
      // V^T fragments, read while the S MFMAs run
      i32x8 vf[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const unsigned char* vr = sV + (32 * d + ql) * kVRowB;
        const u32x4 a0 = *(const u32x4*)(vr + (((2 * hh) ^ vswz) * 16));
        const u32x4 a1 = *(const u32x4*)(vr + (((2 * hh + 1) ^ vswz) * 16));
        vf[d][0] = a0[0]; vf[d][1] = a0[1]; vf[d][2] = a0[2]; vf[d][3] = a0[3];
        vf[d][4] = a1[0]; vf[d][5] = a1[1]; vf[d][6] = a1[2]; vf[d][7] = a1[3];
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- scale, mask keys >= kv (element (kb, i) is key 32hh + 16kb + i) ----
      float sv[2][16];
      float mx = -INFINITY;
      int kvh = kv - 32 * hh;        // keys of this lane half below the block size
      if (p.causal) kvh = min(kvh, p_row - bm[0].beta * 64 - 32 * hh + 1);
      // sv * scl is the scaled score: the raw scores (scl = sc), with keys at
      // or past the block end (or the causal edge) replaced in place by a value
      // whose product with sc is -inf, so both paths leave the scores in the
      // same registers.  The row max is taken on the raw scores, |sc| times the
      // max of sign(sc) * score, exact since scaling keeps or reverses the
      // order; the scale then rides in the exponent's FMA.  A zero scale
      // (all-zero quantised block) takes the explicit path.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[kb][i] = (float)sacc[kb][i];
      float scl = sc;
      if (__builtin_amdgcn_ballot_w64(kvh < 32)) {
        if (sc != 0.f) {
          const float dead = sc > 0.f ? -INFINITY : INFINITY;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) sv[kb][i] = (16 * kb + i < kvh) ? sv[kb][i] : dead;
        } else {
          // every live score is 0
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) sv[kb][i] = (16 * kb + i < kvh) ? 0.f : -INFINITY;
          scl = 1.f;
        }
      }
      if (scl >= 0.f) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sv[kb][i]);
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, -sv[kb][i]);
      }
      mx *= fabsf(scl);
      mx = half_max(mx);
      const float m_ref = (mx > m_run + kSlack) ? mx : m_run;
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      // P * kP8 straight from the exponent: exp2(s - m + log2 kP8)
      const float m_p8 = m_use - kLog2P8;
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = fast_exp2(__builtin_fmaf(sv[kb][i], scl, -m_p8));
          sv[kb][i] = e;
          psum += e;
        }
      if (__builtin_amdgcn_ballot_w64(m_ref != m_run)) {
        const float alpha = fast_exp2(m_run - m_use);
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
      }
      l_run += psum;
      m_run = m_ref;
      // ---- P^T * kP8 -> fp8 as hi + lo parts, slot j = 16kb + i ----
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        const int kb = wd >> 2;
        const int i0 = 4 * (wd & 3);
        const float x0 = sv[kb][i0], x1 = sv[kb][i0 + 1];
        const float x2 = sv[kb][i0 + 2], x3 = sv[kb][i0 + 3];
        int hi = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, pb[wd], false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, hi, true);
        const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
        const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - h01[0], x1 - h01[1], pl[wd], false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(x2 - h23[0], x3 - h23[1], lo, true);
        pb[wd] = hi;
        pl[wd] = lo;
      }
      // ---- O^T += V^T P^T: four 32-dim blocks, K = 64 keys ----
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        oacc[d] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[d], pb, oacc[d], 0, 0, 0, 0, 0, 0);
        oacc[d] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[d], pl, oacc[d], 0, 0, 0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int k = 0; k < kLA; ++k) bm[k] = bm[k + 1];
    bm[kLA].kv = 0;
    if (t + 1 + kLA < n) bm[kLA] = block_meta(t + 1 + kLA);
  }

  // ---- epilogue: O = O^T * v_scale[d] / l -> bf16 [B, H, Sq, 128] ----
  const float l_tot = half_sum(l_run);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;   // O and l both carry kP8
  if (p.lse && hh == 0)
    p.lse[bh * p.Sq + row] = l_tot > 0.f ? (m_run + __log2f(l_tot) - kLog2P8) * kLn2 : -INFINITY;
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
  const int64_t total = (int64_t)p.nqb * p.H * p.B;
  const int64_t per = (total + kXcds - 1) / kXcds;
  if (per * kXcds > 0x7fffffff) return hipErrorInvalidValue;
  SageParams arg = p;
  void* args[] = {(void*)&arg};
  return hipLaunchKernel((const void*)sage_kernel, dim3((unsigned)(per * kXcds)), dim3(128), args,
                         kLds, stream);
}

}  // namespace pkb
