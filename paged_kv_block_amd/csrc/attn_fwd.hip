// attn_fwd.hip -- bf16 scaled-dot-product attention over a paged KV cache for
// gfx950: block-sparse rows, packed prefill and split-KV decode share one kernel.
//
// What is computed (FlashInfer pages "block_sparse_attention_with_paged_kv_cache",
// "batch_prefill_with_paged_kv_cache", "prims_ts_batch_decode_with_kv_cache"):
// for query row i of request b and head h, over the keys j < seq_len[b] that its
// BSR row selects (all keys for prefill/decode), that carry a set validity bit,
// and that pass the causal (j <= p) and left-window (j >= p - w) tests, with
// p = seq_len - qlen + i:  out = output_scale * softmax(scale * q.K^T) V, and the
// natural-log LSE.  Rows with no admitted key give 0 and -inf.
//
// Work decomposition.  One workgroup = (request, KV head, tile of packed query
// rows).  Query heads of one GQA group are packed into the row dimension
// (row = token * group + head_in_group), so a KV tile loaded once serves every
// head of the group.  Each wavefront owns 32 packed rows.
//
// Per 64-key tile:
//   * the tile is 8 chunks of 8 logical tokens; an 8-token run never crosses a
//     page (page and block sizes are multiples of 8), so each chunk is one
//     contiguous [8, D] slab of the HND pool, fetched with 16-byte loads;
//   * K goes to LDS row-major [key][D] (rows padded by 16 B so the MFMA reads of
//     32 consecutive keys hit distinct banks);
//   * V goes to LDS transposed, [D][key], with the keys of every 16-key group
//     stored in the order 0-3, 8-11, 4-7, 12-15 (explained at the PV step);
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (M = keys, N = query rows,
//     K = head dim): every lane then holds 16 keys of ONE query row, so the row
//     max needs one exchange between the two half-waves and the row sum none
//     until the epilogue;
//   * online softmax in base 2 (the scale is folded with log2 e);
//   * O^T += V^T P^T, again 32x32x16 MFMAs.  The B operand P^T is taken straight
//     from the S^T accumulator: lane (row n, half h) holds keys {4h..4h+3,
//     8+4h..8+4h+3} of every 16-key step, which is exactly what the permuted V^T
//     rows provide at positions 8h..8h+7, so no data moves between the two
//     products.
// The next tile's page translation and global loads are issued before the
// current tile's MFMAs so HBM traffic overlaps compute.
#include "device_common.h"
#include "pkb_internal.h"

namespace pkb {

template <int D>
struct AttnLayout {
  static constexpr int KT = kKvTile;          // keys per tile
  static constexpr int PPK = D / 8;           // 16-byte pieces per key row
  static constexpr int KROW = D * 2 + 16;     // bytes per K row in LDS
  static constexpr int VROW = KT * 2 + 16;    // bytes per V^T row in LDS
  static constexpr int K_BYTES = KT * KROW;
  static constexpr int V_BYTES = D * VROW;
  static constexpr int LDS = K_BYTES + V_BYTES;
};

size_t attn_lds_bytes(int D) {
  return D == 128 ? AttnLayout<128>::LDS : AttnLayout<256>::LDS;
}

// Position of key k (0..63) inside a permuted V^T row.
__device__ __forceinline__ int vt_pos(int k) {
  const int b4 = (k >> 2) & 3;
  const int nb4 = (b4 == 1) ? 2 : (b4 == 2 ? 1 : b4);
  return (k & ~15) + nb4 * 4 + (k & 3);
}

template <int D, int NW, int MODE>
__global__ void __launch_bounds__(NW * 64) attn_fwd_kernel(const AttnParams p) {
  using Lay = AttnLayout<D>;
  constexpr int NT = NW * 64;
  constexpr int TILE_M = 32 * NW;
  constexpr int PPK = Lay::PPK;
  constexpr int NKS = D / 16;           // S^T k-steps over the head dim
  constexpr int NDB = D / 32;           // 32-row blocks of O^T
  constexpr int K_PASSES = (Lay::KT * PPK) / NT;
  constexpr int V_PASSES = (16 * PPK) / NT;
  static_assert(K_PASSES >= 1 && V_PASSES >= 1, "tile too small for the workgroup");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* sK = smem;
  unsigned char* sV = smem + Lay::K_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int hh = lane >> 5;        // half-wave
  const int ql = lane & 31;        // query row inside the wave
  const int kvh = blockIdx.y;
  const int G = p.G;

  // ---------------- work item ----------------
  int b, qlen, tok_base, m_begin, m_end, split = 0;
  int bip_lo = 0, n_sel = 0;
  if (MODE == kModeBsa) {
    b = blockIdx.z;
    const int x = p.nqb * p.tiles_per_brow - 1 - (int)blockIdx.x;   // late rows first
    const int r = x / p.tiles_per_brow;
    const int t = x - r * p.tiles_per_brow;
    qlen = p.Sq;
    tok_base = b * p.Sq;
    const int row_lo = r * p.rows_per_brow;
    const int row_hi = min(row_lo + p.rows_per_brow, qlen * G);
    m_begin = row_lo + t * TILE_M;
    m_end = min(m_begin + TILE_M, row_hi);
    const int* bp = p.block_indptr + (int64_t)(b * p.Hkv + kvh) * (p.nqb + 1) + r;
    bip_lo = bp[0];
    n_sel = bp[1] - bip_lo;
  } else if (MODE == kModePrefill) {
    b = p.worklist[2 * blockIdx.x];
    m_begin = p.worklist[2 * blockIdx.x + 1];
    tok_base = p.qo_indptr[b];
    qlen = p.qo_indptr[b + 1] - tok_base;
    m_end = min(m_begin + TILE_M, qlen * G);
  } else {
    b = blockIdx.z;
    split = blockIdx.x;
    qlen = 1;
    tok_base = b;
    m_begin = 0;
    m_end = G;
  }
  const int L = p.seq_lens[b];
  const bool partial_out = (MODE == kModeDecode) && p.num_splits > 1;
  if (partial_out && split * p.split_len >= L) return;   // merge ignores this split
  if (m_begin >= m_end) return;

  // ---------------- rows of this wave ----------------
  const int wm0 = m_begin + wave * 32;
  const int my_m = wm0 + ql;
  const bool row_ok = my_m < m_end;
  const int my_i = my_m / G;
  const int my_hq = kvh * G + (my_m - my_i * G);
  const int my_p = L - qlen + my_i;
  const bool wave_rows = wm0 < m_end;
  const int wp_lo = L - qlen + wm0 / G;
  const int wp_hi = L - qlen + (min(wm0 + 32, m_end) - 1) / G;

  // KV positions any row of the workgroup may admit: [k_lo, k_hi)
  const int p_lo = L - qlen + m_begin / G;
  const int p_hi = L - qlen + (m_end - 1) / G;
  int k_lo = (p.window_left >= 0) ? max(0, p_lo - p.window_left) : 0;
  int k_hi = p.causal ? min(L, p_hi + 1) : L;
  if (partial_out) {
    k_lo = max(k_lo, split * p.split_len);
    k_hi = min(k_hi, (split + 1) * p.split_len);
  }

  int n_vchunks, lo8 = 0;
  if (MODE == kModeBsa) {
    n_vchunks = n_sel * (p.kvbs >> 3);
  } else {
    lo8 = k_lo & ~7;
    n_vchunks = (k_hi > k_lo) ? (k_hi - lo8 + 7) >> 3 : 0;
  }
  const int n_tiles = (n_vchunks + 7) >> 3;

  // ---------------- Q fragments (B operand of S^T) ----------------
  bf16x8 qf[NKS];
  {
    const uint16_t* qrow = p.q + ((int64_t)(tok_base + my_i) * p.Hq + my_hq) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row_ok) x = ld_global_16(qrow + 16 * s);
      qf[s] = as_bf16x8(x);
    }
  }

  // ---------------- chunk translation (lanes 0..7 of every wave) ----------------
  // ts: first logical token of the chunk, or -1 when the chunk is dead;
  // off: element offset of the chunk's [8, D] slab; bw: 8 live bits (validity
  // bit, inside [k_lo, k_hi) and < L), LSB = first token.
  auto chunk_info = [&](int j, int& ts, int64_t& off, int& bw) {
    const int c = lane & 7;
    const int v = j * 8 + c;
    ts = -1; off = 0; bw = 0;
    if (lane < 8 && v < n_vchunks) {
      int64_t t;
      if (MODE == kModeBsa) {
        const int cpb = p.kvbs >> 3;
        const int q = v / cpb;
        t = (int64_t)p.block_indices[bip_lo + q] * p.kvbs + (int64_t)(v - q * cpb) * 8;
      } else {
        t = lo8 + (int64_t)v * 8;
      }
      if (t < k_hi && t + 8 > k_lo) {
        const int ti = (int)t;
        const int pi = ti / p.page_size;
        const int slot = ti - pi * p.page_size;
        int page;
        if (MODE == kModePrefill) page = p.block_tables[(int64_t)b * p.bt_stride + pi];
        else page = p.kv_indices[p.kv_indptr[b] + pi];
        off = (int64_t)page * p.kv_page_stride + (int64_t)kvh * p.kv_head_stride +
              (int64_t)slot * D;
        ts = ti;
        uint32_t bits = 0xFFu;
        if (p.valid_bits) bits = (p.valid_bits[(int64_t)b * p.valid_words + (ti >> 5)] >> (ti & 31)) & 0xFFu;
        const int lo_cut = max(k_lo - ti, 0);                 // tokens below k_lo
        const int hi_cut = min(max(k_hi - ti, 0), 8);         // tokens >= k_hi dead
        uint32_t range = ((1u << hi_cut) - 1u) & ~((1u << lo_cut) - 1u);
        bw = (int)(bits & range);
      }
    }
  };

  // ---------------- global -> register staging ----------------
  u32x4 kreg[K_PASSES];
  u32x4 vreg[V_PASSES][4];
  const int kg = tid & 15;                 // V: 4-key group handled by this lane
  auto load_tile = [&](int ts_v, int64_t off_v) {
    // K: pass i covers keys tid/PPK + (NT/PPK)*i, piece tid%PPK (wave-uniform chunk)
#pragma unroll
    for (int i = 0; i < K_PASSES; ++i) {
      const int key = tid / PPK + (NT / PPK) * i;
      const int c = wave_uniform(key >> 3);
      const int tsc = readlane_i32(ts_v, c);
      const int64_t offc = readlane_i64(off_v, c);
      u32x4 x = {0u, 0u, 0u, 0u};
      if (tsc >= 0) x = ld_global_16(p.k + offc + (key & 7) * D + (tid % PPK) * 8);
      kreg[i] = x;
    }
    // V: lane handles keys 4kg..4kg+3 and d-piece (tid>>4) + (NT/16)*i
    const int c = kg >> 1;
    const int tsc = shfl_i32(ts_v, c);
    const int64_t offc = shfl_i64(off_v, c);
#pragma unroll
    for (int i = 0; i < V_PASSES; ++i) {
      const int dp = (tid >> 4) + (NT / 16) * i;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (tsc >= 0) x = ld_global_16(p.v + offc + (4 * (kg & 1) + e) * D + dp * 8);
        vreg[i][e] = x;
      }
    }
  };

  auto store_tile = [&](int bw_v) {
#pragma unroll
    for (int i = 0; i < K_PASSES; ++i) {
      const int key = tid / PPK + (NT / PPK) * i;
      *(u32x4*)(sK + key * Lay::KROW + (tid % PPK) * 16) = kreg[i];
    }
    // zero V rows of dead keys (never multiply 0 by non-finite data)
    const int bwc = shfl_i32(bw_v, kg >> 1) >> (4 * (kg & 1));
    const int pos = vt_pos(4 * kg);
#pragma unroll
    for (int i = 0; i < V_PASSES; ++i) {
      const int dp = (tid >> 4) + (NT / 16) * i;
      u32x4 r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool live = (bwc >> e) & 1;
        r[e] = live ? vreg[i][e] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        const uint32_t sel = (e8 & 1) ? 0x07060302u : 0x05040100u;
        const int w = e8 >> 1;
        u32x2 d2;
        d2[0] = __builtin_amdgcn_perm(r[1][w], r[0][w], sel);
        d2[1] = __builtin_amdgcn_perm(r[3][w], r[2][w], sel);
        *(u32x2*)(sV + (dp * 8 + e8) * Lay::VROW + pos * 2) = d2;
      }
    }
  };

  // ---------------- accumulators ----------------
  f32x16 oacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[d][i] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float sl2 = p.scale_log2;
  const int wl = p.window_left;
  const bool precise = p.out_f32 != 0;   // fp32 output requested

  int cur_ts = -1, cur_bw = 0;
  int64_t cur_off = 0;
  if (n_tiles > 0) {
    chunk_info(0, cur_ts, cur_off, cur_bw);
    load_tile(cur_ts, cur_off);
  }

  for (int j = 0; j < n_tiles; ++j) {
    int nxt_ts = -1, nxt_bw = 0;
    int64_t nxt_off = 0;
    const bool has_next = (j + 1) < n_tiles;
    if (has_next) chunk_info(j + 1, nxt_ts, nxt_off, nxt_bw);

    __syncthreads();                  // previous tile's LDS reads are done
    store_tile(cur_bw);
    __syncthreads();

    int tsu[8], bwu[8];
    int any_live = 0, all_full = 1, ts_min = 0x7fffffff, ts_max = -1;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      tsu[c] = readlane_i32(cur_ts, c);
      bwu[c] = readlane_i32(cur_bw, c);
      any_live |= bwu[c];
      all_full &= (bwu[c] == 0xFF);
      if (tsu[c] >= 0) { ts_min = min(ts_min, tsu[c]); ts_max = max(ts_max, tsu[c]); }
    }

    if (has_next) load_tile(nxt_ts, nxt_off);

    if (wave_rows && any_live) {
      // ---- S^T = K Q^T for two 32-key blocks ----
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
        const unsigned char* kr = sK + (32 * kb + ql) * Lay::KROW + 16 * hh;
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          const bf16x8 a = *(const bf16x8*)(kr + 32 * s);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb], 0, 0, 0);
        }
      }
      // ---- scale + mask ----
      const bool fast = all_full && (!p.causal || ts_max + 7 <= wp_lo) &&
                        (wl < 0 || ts_min >= wp_hi - wl);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float s = sacc[kb][i] * sl2;
          if (!fast) {
            const int c = 4 * kb + (i >> 2);
            const int e = 4 * hh + (i & 3);
            const int tok = tsu[c] + e;
            bool ok = (bwu[c] >> e) & 1;
            if (p.causal) ok = ok && tok <= my_p;
            if (wl >= 0) ok = ok && tok >= my_p - wl;
            s = ok ? s : -INFINITY;
          }
          sacc[kb][i] = s;
        }
      }
      // ---- online softmax ----
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      mx = half_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = fast_exp2(sacc[kb][i] - m_use);
          sacc[kb][i] = e;
          psum += e;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;

      // ---- O^T += V^T P^T ----
      bf16x8 pb[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 w;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          w[t] = pack_bf16x2(sacc[s >> 1][8 * (s & 1) + 2 * t], sacc[s >> 1][8 * (s & 1) + 2 * t + 1]);
        pb[s] = as_bf16x8(w);
      }
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        const unsigned char* vr = sV + (32 * d + ql) * Lay::VROW + 16 * hh;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 a = *(const bf16x8*)(vr + 32 * s);
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[s], oacc[d], 0, 0, 0);
        }
      }
      if (precise) {
        // fp32 output: add P - bf16(P) as a second bf16 operand, so the
        // probabilities enter the PV product with ~16 significant bits.
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4 hi = __builtin_bit_cast(u32x4, pb[s]);
          u32x4 w;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float p0 = sacc[s >> 1][8 * (s & 1) + 2 * t];
            const float p1 = sacc[s >> 1][8 * (s & 1) + 2 * t + 1];
            w[t] = pack_bf16x2(p0 - __uint_as_float(hi[t] << 16),
                               p1 - __uint_as_float(hi[t] & 0xFFFF0000u));
          }
          pb[s] = as_bf16x8(w);
        }
#pragma unroll
        for (int d = 0; d < NDB; ++d) {
          const unsigned char* vr = sV + (32 * d + ql) * Lay::VROW + 16 * hh;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const bf16x8 a = *(const bf16x8*)(vr + 32 * s);
            oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[s], oacc[d], 0, 0, 0);
          }
        }
      }
    }
    cur_ts = nxt_ts; cur_off = nxt_off; cur_bw = nxt_bw;
  }

  // ---------------- epilogue ----------------
  if (partial_out) {
    // Split-KV decode: this split's unnormalised partial (O, m, l); a separate
    // merge kernel combines the splits.
    if (!wave_rows) return;
    const float l_tot = half_sum(l_run);
    if (!row_ok) return;
    float* dst = p.part + (((int64_t)b * p.Hq + my_hq) * p.num_splits + split) * (D + 4);
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * d + 8 * g4 + 4 * hh;
        f32x4 v4 = {oacc[d][4 * g4], oacc[d][4 * g4 + 1], oacc[d][4 * g4 + 2], oacc[d][4 * g4 + 3]};
        *(f32x4*)(dst + d0) = v4;
      }
    if (hh == 0) {
      dst[D] = m_run;
      dst[D + 1] = l_tot;
    }
    return;
  }
  if (!wave_rows) return;
  const float l_tot = half_sum(l_run);
  if (!row_ok) return;
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : p.out_scale / l_tot;
  const int64_t orow = ((int64_t)(tok_base + my_i) * p.Hq + my_hq);
  if (p.out_f32) {
    float* o = (float*)p.out + orow * D;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * d + 8 * g4 + 4 * hh;
        f32x4 v4 = {oacc[d][4 * g4] * inv, oacc[d][4 * g4 + 1] * inv,
                    oacc[d][4 * g4 + 2] * inv, oacc[d][4 * g4 + 3] * inv};
        *(f32x4*)(o + d0) = v4;
      }
  } else {
    uint16_t* o = (uint16_t*)p.out + orow * D;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * d + 8 * g4 + 4 * hh;
        u32x2 w;
        w[0] = pack_bf16x2(oacc[d][4 * g4] * inv, oacc[d][4 * g4 + 1] * inv);
        w[1] = pack_bf16x2(oacc[d][4 * g4 + 2] * inv, oacc[d][4 * g4 + 3] * inv);
        *(u32x2*)(o + d0) = w;
      }
  }
  if (p.lse && hh == 0)
    p.lse[orow] = empty ? -INFINITY : (m_run + __log2f(l_tot)) * kLn2;
}

template <int D, int NW, int MODE>
static hipError_t launch_one(const AttnParams& p, dim3 grid, hipStream_t st) {
  const size_t lds = AttnLayout<D>::LDS;
  const void* kern = (const void*)attn_fwd_kernel<D, NW, MODE>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  AttnParams arg = p;
  void* args[] = {(void*)&arg};
  return hipLaunchKernel(kern, grid, dim3(NW * 64), args, lds, st);
}

template <int D>
static hipError_t launch_d(const AttnParams& p, int waves, int mode, dim3 grid, hipStream_t st) {
  if (mode == kModeBsa) {
    if (waves == 1) return launch_one<D, 1, kModeBsa>(p, grid, st);
    if (waves == 2) return launch_one<D, 2, kModeBsa>(p, grid, st);
    if (waves == 4) return launch_one<D, 4, kModeBsa>(p, grid, st);
  } else if (mode == kModePrefill) {
    if (waves == 4) return launch_one<D, 4, kModePrefill>(p, grid, st);
  } else if (mode == kModeDecode) {
    if (waves == 4) return launch_one<D, 4, kModeDecode>(p, grid, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn(const AttnParams& p, int D, int waves, int mode, dim3 grid,
                       hipStream_t stream) {
  if (D == 128) return launch_d<128>(p, waves, mode, grid, stream);
  if (D == 256) return launch_d<256>(p, waves, mode, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkb
