// decode_fwd.hip -- single-token paged decode (split-KV + merge) for gfx950.
//
// What is computed (FlashInfer page "prims_ts_batch_decode_with_kv_cache"): for
// request b and query head h, out = bmm2_scale * softmax(bmm1_scale * q.K^T) V
// over keys j < seq_len[b] (and j >= seq_len-1-w with a left window w >= 0),
// plus the natural-log LSE.  The same kernel serves multi-token decode when
// the query rows of one KV head (tokens x group heads) fit 16 MFMA columns:
// token i of qlen sits at position seq_len - qlen + i (causal: keys up to it).
//
// The path is bound by HBM bandwidth -- every live K/V byte is read once -- so
// the design is about keeping bytes in flight on every CU until the end:
//   * Work items are chunks: (request, chunk of CH tokens, KV head), every full
//     chunk first and the partial last chunks after them.
//     The grid is persistent (a fixed number of single-wave workgroups); wave w
//     takes items w, w + W, w + 2W, ... of the flattened list, which it derives
//     on the device from seq_lens (no host read), so long and short requests
//     spread evenly and no CU idles while a long request finishes.
//   * Inside an item, keys go in groups of 32.  S^T = K Q^T uses
//     v_mfma_f32_16x16x32_bf16 with M = 16 keys, N = the GQA group (up to 16
//     query heads), K = 32 head dims; the A operand (16 keys x 32 dims) is
//     loaded straight from the page pool into registers, each lane reading 16
//     contiguous bytes of one key row.
//   * V (32 keys x D) is copied row-major into the wave's LDS slab and read back
//     with ds_read_b64_tr_b16, which delivers a 4-key x 16-dim block column-wise:
//     the A operand of O^T += V^T P^T.  Lane group g then holds keys {4g..4g+3}
//     of the first 16-key unit and {16+4g..16+4g+3} of the second -- the key set
//     its S^T accumulator already holds -- so P^T feeds the MFMA directly.
//   * Software pipeline: group j+1's loads are in flight while group j computes
//     (two register buffers in ping-pong); page IDs are loaded two groups
//     ahead and translated one ahead.
// Each item writes a partial (O, m, l); a small second kernel merges the chunks
// of every (request, head).  A kernel boundary, not an in-kernel agent-scope
// fence, makes the partials visible: on this part such a fence writes back and
// invalidates the whole L2 of an XCD.
#include <atomic>
#include <mutex>

#include "device_common.h"
#include "pkb_internal.h"

namespace pkb {

typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));

template <int D>
struct DecLayout {
  static constexpr int KEYS = 32;              // keys per wave iteration
  static constexpr int VROW = D * 2 + 32;      // V row bytes in LDS; the pad puts the four
                                               // rows of one transpose read on distinct banks
  static constexpr int LDS = KEYS * VROW;
  static constexpr int PIECES = KEYS * D / 8;  // 16-byte pieces of V per group
};

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// One wave's share of a decode work item: the keys of request b, KV head kvh
// inside [r_lo, r_hi) (and inside the columns' causal / window bounds), for the
// MFMA columns of the request's query rows.  On return oacc holds the
// unnormalised O^T fragment relative to m_run (lane (qn, g): dims 16d + 4g + i
// of column qn), m_run the column's running max in scale * log2(e) units (-inf
// when no key was admitted) and l_run this lane's share of the column's sum of
// probabilities (quad_sum adds the four shares).  vs is the wave's V slab.
// RAGGED: the page size is not a multiple of 8, so an 8-token chunk may span
// pages and every token is translated on its own (lanes 0..31 hold the 32
// tokens of a group; the loads fetch their row offsets with a lane shuffle).
template <int D, bool F32, bool RAGGED>
__device__ __forceinline__ void decode_part(const DecodeParams& p, int b, int kvh, int L, int qlen,
                                            int tok0, int r_lo, int r_hi, unsigned char* vs,
                                            f32x4 (&oacc)[D / 16], float& m_run, float& l_run) {
  using Lay = DecLayout<D>;
  constexpr int KS = D / 32;             // MFMA k-steps over the head dim (S^T)
  constexpr int DB = D / 16;             // 16-row blocks of O^T
  constexpr int VP = Lay::PIECES / 64;   // V pieces per lane per group
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;               // lane group: 4 keys of each 16-key unit
  const int qn = lane & 15;              // MFMA column = query row of the request
  const int G = p.G;

  // MFMA column qn is query row (token i, head h) of the request: qlen tokens
  // (one for single-token decode) x G heads, at most 16 columns.  Token i sits
  // at position L - qlen + i and, causal, sees keys [lo_i, p_i]; otherwise
  // [lo_i, L).  The wave covers the union of those ranges inside [r_lo, r_hi).
  const int qi = qn / G, qh = qn - qi * G;
  const bool col_ok = qi < qlen;
  const int p_col = L - qlen + qi;
  const int hi_col = p.causal ? p_col + 1 : L;
  const int lo_col = p.window_left >= 0 ? max(0, p_col - p.window_left) : 0;
  int k_lo = p.window_left >= 0 ? max(0, L - qlen - p.window_left) : 0;
  k_lo = max(k_lo, r_lo);
  const int k_hi = min(L, r_hi);
  // keys every column admits (no per-column mask needed inside)
  const int k_lo_all = max(p.window_left >= 0 ? max(0, L - 1 - p.window_left) : 0, r_lo);
  const int k_hi_all = min(p.causal ? L - qlen + 1 : L, r_hi);
  const int t_base = k_lo & ~31;
  const int n_groups = k_hi > k_lo ? (k_hi - t_base + 31) >> 5 : 0;
  const int64_t head_off = (int64_t)kvh * p.kv_head_stride;
  const int32_t* ids = p.kv_indices + ld_const(p.kv_indptr, b);

  bf16x8 qf[KS];
  {
    const uint16_t* qrow = p.q + ((int64_t)(tok0 + qi) * p.Hq + kvh * G + qh) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (col_ok) x = ld_global_16(qrow + 32 * s);
      qf[s] = as_bf16x8(x);
    }
  }
#pragma unroll
  for (int d = 0; d < DB; ++d) oacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  m_run = -INFINITY;
  l_run = 0.f;

  // Page translation of a group's four 8-token chunks (lanes 0..3).  The page
  // ID load is issued two groups ahead and only used one group ahead: loads
  // retire in issue order, so waiting for it must not also wait for the K/V
  // loads issued after it.  Every lane loads (the index is clamped into the
  // request's live range), so no path skips a load.
  auto page_id = [&](int grp) -> int {
    const int t = min(t_base + grp * 32 + (RAGGED ? (lane & 31) : 8 * (lane & 3)), L - 1);
    return ids[t / p.page_size];
  };
  // element offset of the chunk (RAGGED: the token) from its page ID; dead
  // chunks get offset 0 (page 0, always in bounds) and their keys are masked
  auto chunk_off = [&](int grp, int id) -> int64_t {
    const int t = t_base + grp * 32 + (RAGGED ? (lane & 31) : 8 * (lane & 3));
    if (!((RAGGED || lane < 4) && grp < n_groups && t < L)) return 0;
    const int pi = t / p.page_size;
    return (int64_t)id * p.kv_page_stride + head_off + (int64_t)(t - pi * p.page_size) * D;
  };

  const char* kbase = (const char*)p.k;
  const char* vbase = (const char*)p.v;
  // Loads of one 32-key group.  K goes straight into the A operand of S^T;
  // V pieces are row-major (piece lane + 64i is key 4i + lane/16 at D = 128,
  // 2i + lane/32 at D = 256, so each load's chunk is wave-uniform).  Every
  // K/V byte is read once per launch, so the loads are non-temporal.
  auto load_group = [&](int64_t off_v, bf16x8 (&ka)[2][KS], u32x4 (&vr)[VP]) {
    if (RAGGED) {
      // row offset of key k of the group, held by lane k
      auto row_off = [&](int k) -> int64_t {
        const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)off_v, k);
        const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)((uint64_t)off_v >> 32), k);
        return (int64_t)(((uint64_t)hi << 32) | lo);
      };
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t off = row_off(16 * u + qn) * 2 + 16 * g;
#pragma unroll
        for (int s = 0; s < KS; ++s) ka[u][s] = as_bf16x8(ld_stream_16(kbase + off + 64 * s));
      }
#pragma unroll
      for (int i = 0; i < VP; ++i) {
        const int piece = lane + 64 * i;
        const int key = piece / (D / 8);
        const int dp = piece - key * (D / 8);
        vr[i] = ld_stream_16(vbase + row_off(key) * 2 + dp * 16);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t o0 = readlane_i64(off_v, 2 * u), o1 = readlane_i64(off_v, 2 * u + 1);
      const int64_t off = (qn < 8 ? o0 : o1) * 2 + ((qn & 7) * D + 8 * g) * 2;
#pragma unroll
      for (int s = 0; s < KS; ++s) ka[u][s] = as_bf16x8(ld_stream_16(kbase + off + 64 * s));
    }
#pragma unroll
    for (int i = 0; i < VP; ++i) {
      const int piece = lane + 64 * i;
      const int key = piece / (D / 8);
      const int dp = piece - key * (D / 8);
      const int64_t off = readlane_i64(off_v, (64 * i) / (D / 8) / 8) * 2 + ((key & 7) * D + dp * 8) * 2;
      vr[i] = ld_stream_16(vbase + off);
    }
  };

  // One group: S^T, masks, online softmax, V slab, O^T += V^T P^T.
  auto compute = [&](int grp, bf16x8 (&ka)[2][KS], u32x4 (&vr)[VP]) {
    const int t0 = t_base + grp * 32;
    const bool full = t0 >= k_lo_all && t0 + 32 <= k_hi_all;
    f32x4 sacc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      sacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        sacc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u][s], qf[s], sacc[u], 0, 0, 0);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sv = sacc[u][i] * p.scale_log2;
        if (!full) {
          const int t = t0 + 16 * u + 4 * g + i;
          sv = (t >= k_lo && t < k_hi && t >= lo_col && t < hi_col) ? sv : -INFINITY;
        }
        sacc[u][i] = sv;
        mx = fmaxf(mx, sv);
      }
    if (!full) {
      // dead keys contribute nothing: zero their V rows (no 0 * NaN)
#pragma unroll
      for (int i = 0; i < VP; ++i) {
        const int key = (lane + 64 * i) / (D / 8);
        const int t = t0 + key;
        if (!(t >= k_lo && t < k_hi)) vr[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    mx = quad_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    float ps = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = fast_exp2(sacc[u][i] - m_use);
        sacc[u][i] = e;
        ps += e;
      }
    if (m_new != m_run) {            // rescale only when some running max moved
      const float alpha = fast_exp2(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < DB; ++d) oacc[d] *= alpha;
    }
    l_run += ps;
    m_run = m_new;

    // V slab -> LDS, then O^T += V^T P^T
#pragma unroll
    for (int i = 0; i < VP; ++i) {
      const int piece = lane + 64 * i;
      const int key = piece / (D / 8);
      const int dp = piece - key * (D / 8);
      *(u32x4*)(vs + key * Lay::VROW + dp * 16) = vr[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    u32x4 pw;
    pw[0] = pack_bf16x2(sacc[0][0], sacc[0][1]);
    pw[1] = pack_bf16x2(sacc[0][2], sacc[0][3]);
    pw[2] = pack_bf16x2(sacc[1][0], sacc[1][1]);
    pw[3] = pack_bf16x2(sacc[1][2], sacc[1][3]);
    u32x4 plo = {0u, 0u, 0u, 0u};
    if (F32) {
      // fp32 output: P - bf16(P) enters as a second operand (~16-bit P)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f32x4& sa = sacc[t >> 1];
        const int i0 = 2 * (t & 1);
        plo[t] = pack_bf16x2(sa[i0] - __uint_as_float(pw[t] << 16),
                             sa[i0 + 1] - __uint_as_float(pw[t] & 0xFFFF0000u));
      }
    }
    // transpose-read addresses: lane (4r + c) of a 16-lane group reads row
    // 4g + r (unit 0) or 16 + 4g + r (unit 1), dims 16d + 4c .. +3
    const int rr = (lane & 15) >> 2, cc = lane & 3;
    const unsigned char* a0 = vs + (4 * g + rr) * Lay::VROW + 8 * cc;
    const unsigned char* a1 = vs + (16 + 4 * g + rr) * Lay::VROW + 8 * cc;
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(a0 + 32 * d));
      const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(a1 + 32 * d));
      const u32x2 w0 = __builtin_bit_cast(u32x2, x0);
      const u32x2 w1 = __builtin_bit_cast(u32x2, x1);
      u32x4 aw;
      aw[0] = w0[0]; aw[1] = w0[1]; aw[2] = w1[0]; aw[3] = w1[1];
      oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(aw), as_bf16x8(pw), oacc[d], 0, 0, 0);
      if (F32)
        oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(aw), as_bf16x8(plo), oacc[d], 0, 0, 0);
    }
    // the slab is rewritten next iteration: keep these reads before those writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  };

  // Software pipeline over two register buffers, the loop unrolled twice so
  // that no buffer is copied (a copy would wait for the loads in flight).
  // Phase of group j: issue group j+2's page-ID load, translate group j+1's
  // (loaded a phase earlier), issue group j+1's K/V loads, compute group j.
  // Loads past the last group read page 0 and are never used, so every phase
  // has the same loads in flight.
  bf16x8 kA[2][KS], kB[2][KS];
  u32x4 vA[VP], vB[VP];
  {
    const int id0 = page_id(0);
    load_group(chunk_off(0, id0), kA, vA);
  }
  int id_n = page_id(1);
  for (int grp = 0; grp < n_groups; grp += 2) {
    {
      const int id_nn = page_id(grp + 2);
      load_group(chunk_off(grp + 1, id_n), kB, vB);
      compute(grp, kA, vA);
      id_n = id_nn;
    }
    if (grp + 1 >= n_groups) break;
    {
      const int id_nn = page_id(grp + 3);
      load_group(chunk_off(grp + 2, id_n), kA, vA);
      compute(grp + 1, kB, vB);
      id_n = id_nn;
    }
  }
}

// Normalised output and LSE of one query row held as (O, m, l): bf16 or fp32
// row `orow` of out; an empty row (no admitted key) gives zeros and -inf.
template <int D, bool F32, int N>
__device__ __forceinline__ void store_row(const DecodeParams& p, int64_t orow, int d0,
                                          const float (&o)[N], float m, float l, bool write_lse) {
  const bool empty = !(l > 0.f);
  const float inv = empty ? 0.f : p.out_scale / l;
  if (F32) {
    float* dst = (float*)p.out + orow * D + d0;
#pragma unroll
    for (int t = 0; t < N; t += 4)
      *(f32x4*)(dst + t) = f32x4{o[t] * inv, o[t + 1] * inv, o[t + 2] * inv, o[t + 3] * inv};
  } else {
    uint16_t* dst = (uint16_t*)p.out + orow * D + d0;
#pragma unroll
    for (int t = 0; t < N; t += 4) {
      u32x2 w;
      w[0] = pack_bf16x2(o[t] * inv, o[t + 1] * inv);
      w[1] = pack_bf16x2(o[t + 2] * inv, o[t + 3] * inv);
      *(u32x2*)(dst + t) = w;
    }
  }
  if (p.lse && write_lse) p.lse[orow] = empty ? -INFINITY : (m + __log2f(l)) * kLn2;
}

template <int D, bool F32, bool RAGGED>
__global__ void __launch_bounds__(64) decode_kernel(const DecodeParams p) {
  constexpr int DB = D / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x;
  const int g = lane >> 4;
  const int qn = lane & 15;
  const int G = p.G;
  const int CH = p.split_len;
  const int S = p.num_splits;

  // Item order: every full CH-token chunk of the batch first, then each
  // request's partial last chunk.  Waves are dealt items round robin, so the
  // waves that get one item more than the others mostly get a short one.
  // Running position in the chosen (request, chunk) list:
  int phase = 0;          // 0: full chunks, 1: partial last chunks
  int blk = 0;            // current block of 64 requests
  int blk_base = 0;       // chunks before this block
  int n_b = 0, incl = 0;  // this lane's request: chunk count, inclusive prefix in block
  auto load_block = [&]() {
    const int bb = blk * 64 + lane;
    int nc = 0;
    if (bb < p.B) {
      const int len = p.seq_lens[bb];
      nc = phase == 0 ? len / CH : (len % CH != 0 ? 1 : 0);
    }
    n_b = nc;
    incl = wave_incl_scan(n_b);
  };
  int n_full = 0;         // full chunks over the batch
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int bb = b0 + lane;
    n_full += readlane_i32(wave_incl_scan(bb < p.B ? p.seq_lens[bb] / CH : 0), 63);
  }
  load_block();

  const int W = gridDim.x;
  for (int item = blockIdx.x;; item += W) {
    const int j = item / p.Hkv;              // position in the chunk list
    const int kvh = item - j * p.Hkv;
    if (phase == 0 && j >= n_full) {         // on to the partial chunks
      phase = 1;
      blk = 0;
      blk_base = n_full;
      load_block();
    }
    // advance to the block of requests that holds chunk j
    int tot = readlane_i32(incl, 63);
    while (j >= blk_base + tot && blk * 64 + 64 < p.B) {
      blk_base += tot;
      ++blk;
      load_block();
      tot = readlane_i32(incl, 63);
    }
    if (j >= blk_base + tot) break;          // past the last chunk: done
    const int local = j - blk_base;
    const unsigned long long msk = __ballot(incl > local);
    const int ln = __builtin_ctzll(msk);
    const int b = blk * 64 + ln;
    const int L = ld_const(p.seq_lens, b);
    const int c = phase == 0 ? local - (readlane_i32(incl, ln) - readlane_i32(n_b, ln)) : L / CH;
    const int qlen = p.qo_indptr ? ld_const(p.qo_indptr, b + 1) - ld_const(p.qo_indptr, b) : p.Sq;
    const int tok0 = p.qo_indptr ? ld_const(p.qo_indptr, b) : b * p.Sq;

    f32x4 oacc[DB];
    float m_run, l_run;
    decode_part<D, F32, RAGGED>(p, b, kvh, L, qlen, tok0, c * CH, (c + 1) * CH, smem, oacc, m_run,
                                l_run);

    // ---- item result: lane (qn, g) holds O^T rows 16d + 4g + i of head qn ----
    const float l_tot = quad_sum(l_run);
    const int qi = qn / G, qh = qn - qi * G;
    if (qi < qlen) {
      const int hq = kvh * G + qh;
      if (S > 1) {
        float* dst = p.part + ((((int64_t)b * p.maxq + qi) * p.Hq + hq) * S + c) * (D + 4);
#pragma unroll
        for (int d = 0; d < DB; ++d) *(f32x4*)(dst + 16 * d + 4 * g) = oacc[d];
        if (g == 0) {
          dst[D] = m_run;
          dst[D + 1] = l_tot;
        }
      } else {
        const int64_t orow = (int64_t)(tok0 + qi) * p.Hq + hq;
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          const float o4[4] = {oacc[d][0], oacc[d][1], oacc[d][2], oacc[d][3]};
          store_row<D, F32, 4>(p, orow, 16 * d + 4 * g, o4, m_run, l_tot, d == 0 && g == 0);
        }
      }
    }
  }
}

// Cooperative decode for batches with at least two (request, KV head) pairs
// per compute unit: a persistent grid of kCoopWaves-wave workgroups, one per
// CU.  A work item is a whole (request, KV head) pair.  Items are ordered by
// the number of 32-key groups they visit, most first (ties by request), and
// dealt to the workgroups in snake order (round r gives item r*W + w to
// workgroup w on even rounds, r*W + W-1-w on odd ones), so a workgroup that
// takes a long item in one round takes a short one in the next: the static
// counterpart of longest-processing-time-first scheduling.  The waves of a
// workgroup split an item's groups evenly, and their partial (O, m, l) are
// merged through LDS into the final output: no workspace, no merge launch.
template <int D, bool F32, bool RAGGED>
__global__ void __launch_bounds__(kCoopWaves * 64) decode_coop_kernel(const DecodeParams p) {
  using Lay = DecLayout<D>;
  constexpr int DB = D / 16;
  constexpr int NT = kCoopWaves * 64;
  constexpr int PER = D / 16;            // dims per thread in the merge (16 threads per column)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int* key = (int*)(smem + kCoopWaves * Lay::LDS);   // [kCoopMaxBatch]: groups visited
  int* perm = key + kCoopMaxBatch;                    // [kCoopMaxBatch]: b of sorted position

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int g = lane >> 4;
  const int qn = lane & 15;
  const int G = p.G;

  // ---- sorted request order (every workgroup derives the same one) ----
  auto range_of = [&](int b, int& L, int& qlen, int& tok0, int& k_lo) {
    L = ld_const(p.seq_lens, b);
    qlen = p.qo_indptr ? ld_const(p.qo_indptr, b + 1) - ld_const(p.qo_indptr, b) : p.Sq;
    tok0 = p.qo_indptr ? ld_const(p.qo_indptr, b) : b * p.Sq;
    k_lo = p.window_left >= 0 ? max(0, L - qlen - p.window_left) : 0;
  };
  for (int b = tid; b < p.B; b += NT) {
    const int L = p.seq_lens[b];
    const int qlen = p.qo_indptr ? p.qo_indptr[b + 1] - p.qo_indptr[b] : p.Sq;
    const int k_lo = p.window_left >= 0 ? max(0, L - qlen - p.window_left) : 0;
    key[b] = L > k_lo ? (L - (k_lo & ~31) + 31) >> 5 : 0;
  }
  __syncthreads();
  for (int b = tid; b < p.B; b += NT) {
    const int kb = key[b];
    int r = 0;
    for (int o = 0; o < p.B; ++o) {
      const int ko = key[o];
      r += (ko > kb) || (ko == kb && o < b);
    }
    perm[r] = b;
  }
  __syncthreads();

  const int W = gridDim.x;
  const int n_items = p.B * p.Hkv;
  unsigned char* slab = smem + wave * Lay::LDS;
  for (int round = 0;; ++round) {
    const int k = (round & 1) ? W - 1 - (int)blockIdx.x : (int)blockIdx.x;
    const int item = round * W + k;
    if (item >= n_items) break;                // workgroup-uniform exit
    const int j = item / p.Hkv;
    const int kvh = item - j * p.Hkv;
    const int b = perm[j];
    int L, qlen, tok0, k_lo;
    range_of(b, L, qlen, tok0, k_lo);
    // this wave's share of the item's 32-key groups
    const int t_base = k_lo & ~31;
    const int ng = L > k_lo ? (L - t_base + 31) >> 5 : 0;
    const int g0 = (ng * wave) / kCoopWaves, g1 = (ng * (wave + 1)) / kCoopWaves;
    const int r_lo = wave == 0 ? 0 : t_base + 32 * g0;
    const int r_hi = wave == kCoopWaves - 1 ? L : t_base + 32 * g1;

    f32x4 oacc[DB];
    float m_run, l_run;
    decode_part<D, F32, RAGGED>(p, b, kvh, L, qlen, tok0, r_lo, r_hi, slab, oacc, m_run, l_run);
    const float l_tot = quad_sum(l_run);

    // ---- merge of the waves' partials through LDS (the V slabs are free now) ----
    __syncthreads();
    float* mine = (float*)slab;                // [16][D] O^T by column, then m[16], l[16]
#pragma unroll
    for (int d = 0; d < DB; ++d) *(f32x4*)(mine + qn * D + 16 * d + 4 * g) = oacc[d];
    if (g == 0) {
      mine[16 * D + qn] = m_run;
      mine[16 * D + 16 + qn] = l_tot;
    }
    __syncthreads();
    {
      const int col = tid >> 4;                // 16 threads per column
      const int d0 = (tid & 15) * PER;
      const int qi = col / G, qh = col - qi * G;
      if (qi < qlen) {
        float mw[kCoopWaves], lw[kCoopWaves];
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kCoopWaves; ++w) {
          const float* src = (const float*)(smem + w * Lay::LDS);
          mw[w] = src[16 * D + col];
          lw[w] = src[16 * D + 16 + col];
          M = fmaxf(M, mw[w]);
        }
        float o[PER];
#pragma unroll
        for (int t = 0; t < PER; ++t) o[t] = 0.f;
        float lsum = 0.f;
        if (M != -INFINITY) {
#pragma unroll
          for (int w = 0; w < kCoopWaves; ++w) {
            const float wt = fast_exp2(mw[w] - M);   // 0 for a wave that admitted nothing
            lsum += wt * lw[w];
            const float* src = (const float*)(smem + w * Lay::LDS) + col * D + d0;
#pragma unroll
            for (int t = 0; t < PER; t += 4) {
              const f32x4 x = *(const f32x4*)(src + t);
              o[t] += wt * x[0];
              o[t + 1] += wt * x[1];
              o[t + 2] += wt * x[2];
              o[t + 3] += wt * x[3];
            }
          }
        }
        const int64_t orow = (int64_t)(tok0 + qi) * p.Hq + kvh * G + qh;
        store_row<D, F32, PER>(p, orow, d0, o, M, lsum, (tid & 15) == 0);
      }
    }
    __syncthreads();                           // merge reads done before the slabs are rewritten
  }
}

// Merge of one (request, query token, query head): LSE-weighted sum of its live
// splits' partials, each lane owning D/64 dims.  Up to kMergeFew splits, all
// loads go out in one round.  Beyond that, lane s holds split s's (m, l) (64
// splits per pass), so the max and the weights take one load round trip, and
// the O accumulation then issues the partial rows of eight splits at a time.
constexpr int kMergeFew = 16;   // split counts merged with a single round of loads

template <int D>
__global__ void __launch_bounds__(64) decode_merge_kernel(const MergeParams p) {
  constexpr int PER = D / 64;
  constexpr int ROW = D + 4;
  const int lane = threadIdx.x;
  const int hq = (int)blockIdx.x % p.Hq;
  const int i = ((int)blockIdx.x / p.Hq) % p.maxq;
  const int b = (int)blockIdx.x / (p.Hq * p.maxq);
  const int qlen = p.qo_indptr ? p.qo_indptr[b + 1] - p.qo_indptr[b] : p.Sq;
  if (i >= qlen) return;
  const int64_t bh = ((int64_t)(p.qo_indptr ? p.qo_indptr[b] : b * p.Sq) + i) * p.Hq + hq;
  const int L = p.seq_lens[b];
  const int n = min(p.num_splits, (L + p.split_len - 1) / p.split_len);
  const float* base = p.part + (int64_t)blockIdx.x * p.num_splits * ROW;
  float M = -INFINITY;
  float lsum = 0.f;
  float acc[PER];
#pragma unroll
  for (int t = 0; t < PER; ++t) acc[t] = 0.f;
  if (n <= kMergeFew) {
    // Few splits: every load is issued in one round (lane s < n reads split
    // s's (m, l); each lane reads its dims of every partial row), then the
    // max, the weights and the weighted sum follow from registers.
    float m = -INFINITY, l = 0.f;
    if (lane < n) {
      m = base[(int64_t)lane * ROW + D];
      l = base[(int64_t)lane * ROW + D + 1];
    }
    float x[kMergeFew][PER];
#pragma unroll
    for (int k = 0; k < kMergeFew; ++k)
#pragma unroll
      for (int t = 0; t < PER; ++t) x[k][t] = k < n ? base[(int64_t)k * ROW + lane * PER + t] : 0.f;
    M = m;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    if (M != -INFINITY) {
      const float w = lane < n ? fast_exp2(m - M) : 0.f;
      float wl = w * l;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) wl += __shfl_xor(wl, o);
      lsum = wl;
#pragma unroll
      for (int k = 0; k < kMergeFew; ++k) {
        const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
#pragma unroll
        for (int t = 0; t < PER; ++t) acc[t] += wk * x[k][t];
      }
    }
  } else {
    for (int s0 = 0; s0 < n; s0 += 64) {
      const int s = s0 + lane;
      float m = s < n ? base[(int64_t)s * ROW + D] : -INFINITY;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      M = fmaxf(M, m);
    }
    if (M != -INFINITY) {
      for (int s0 = 0; s0 < n; s0 += 64) {
        const int s = s0 + lane;
        float w = 0.f, wl = 0.f;
        if (s < n) {
          w = fast_exp2(base[(int64_t)s * ROW + D] - M);
          wl = w * base[(int64_t)s * ROW + D + 1];
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) wl += __shfl_xor(wl, o);
        lsum += wl;
        const int cnt = min(64, n - s0);
        for (int k0 = 0; k0 < cnt; k0 += 8) {
          float x[8][PER];
#pragma unroll
          for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int t = 0; t < PER; ++t)
              x[k][t] = (k0 + k < cnt) ? base[(int64_t)(s0 + k0 + k) * ROW + lane * PER + t] : 0.f;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            // k0 + k <= 63: k0 < cnt <= 64 steps by 8
            const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k0 + k));
#pragma unroll
            for (int t = 0; t < PER; ++t) acc[t] += wk * x[k][t];
          }
        }
      }
    }
  }
  const bool empty = !(lsum > 0.f);
  const float inv = empty ? 0.f : p.out_scale / lsum;
  if (p.out_f32) {
    float* o = (float*)p.out + (int64_t)bh * D + lane * PER;
#pragma unroll
    for (int t = 0; t < PER; ++t) o[t] = acc[t] * inv;
  } else {
    uint16_t* o = (uint16_t*)p.out + (int64_t)bh * D + lane * PER;
#pragma unroll
    for (int t = 0; t < PER; t += 2) *(uint32_t*)(o + t) = pack_bf16x2(acc[t] * inv, acc[t + 1] * inv);
  }
  if (p.lse && lane == 0) p.lse[bh] = empty ? -INFINITY : (M + __log2f(lsum)) * kLn2;
}

template <int D>
static hipError_t launch_dec(const DecodeParams& p, int grid, hipStream_t st) {
  DecodeParams arg = p;
  void* args[] = {(void*)&arg};
  const bool ragged = (p.page_size & 7) != 0;
  const void* kern = ragged ? (p.out_f32 ? (const void*)decode_kernel<D, true, true>
                                         : (const void*)decode_kernel<D, false, true>)
                            : (p.out_f32 ? (const void*)decode_kernel<D, true, false>
                                         : (const void*)decode_kernel<D, false, false>);
  return hipLaunchKernel(kern, dim3(grid), dim3(64), args, DecLayout<D>::LDS, st);
}

template <int D>
static hipError_t launch_coop(const DecodeParams& p, int grid, hipStream_t st) {
  const size_t lds = kCoopWaves * DecLayout<D>::LDS + 2 * kCoopMaxBatch * sizeof(int);
  const bool ragged = (p.page_size & 7) != 0;
  const void* kern = ragged ? (p.out_f32 ? (const void*)decode_coop_kernel<D, true, true>
                                         : (const void*)decode_coop_kernel<D, false, true>)
                            : (p.out_f32 ? (const void*)decode_coop_kernel<D, true, false>
                                         : (const void*)decode_coop_kernel<D, false, false>);
  if (lds > 65536) {
    // The LDS limit is an attribute of the function on one device: raise it on
    // the first launch there only, so later launches (and graph capture) make
    // no extra runtime calls.
    static std::atomic<uint64_t> raised[4];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev < 64 ? (1ull << dev) : 0;
    std::atomic<uint64_t>& flag = raised[(p.out_f32 ? 1 : 0) + (ragged ? 2 : 0)];
    if (!(flag.load(std::memory_order_acquire) & bit)) {
      e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      flag.fetch_or(bit, std::memory_order_release);
    }
  }
  DecodeParams arg = p;
  void* args[] = {(void*)&arg};
  return hipLaunchKernel(kern, dim3(grid), dim3(kCoopWaves * 64), args, lds, st);
}

hipError_t launch_decode(const DecodeParams& p, int D, int grid, hipStream_t stream) {
  if (D == 128) return launch_dec<128>(p, grid, stream);
  if (D == 256) return launch_dec<256>(p, grid, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_coop(const DecodeParams& p, int D, int grid, hipStream_t stream) {
  if (p.B > kCoopMaxBatch || p.G * p.maxq > kDecodeMaxGroup) return hipErrorInvalidValue;
  if (D == 128) return launch_coop<128>(p, grid, stream);
  if (D == 256) return launch_coop<256>(p, grid, stream);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- fixed scratch
// Split partials for callers that cannot allocate device memory: one
// file-scope array per device, kDecodeScratchBytes large, held until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it only stands for the symbol); it uses the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current and kept in decode_scratch_ptr[].
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

static std::mutex decode_scratch_mu;
static void* decode_scratch_ptr[kMaxDevices];

hipError_t decode_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(decode_scratch_mu);
  if (!decode_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    decode_scratch_ptr[dev] = p;
  }
  *ptr = decode_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_merge(const MergeParams& p, int D, hipStream_t stream) {
  const int64_t n = (int64_t)p.B * p.maxq * p.Hq;
  if (n > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)n);
  MergeParams arg = p;
  void* args[] = {(void*)&arg};
  if (D == 128) return hipLaunchKernel((const void*)decode_merge_kernel<128>, grid, dim3(64), args, 0, stream);
  if (D == 256) return hipLaunchKernel((const void*)decode_merge_kernel<256>, grid, dim3(64), args, 0, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkb
