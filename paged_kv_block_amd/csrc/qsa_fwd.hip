// qsa_fwd.hip -- packed-query token-granular sparse attention for gfx950.
//
// What is computed (FlashInfer page "qsa_forward", Parameters / Returns /
// Notes): the queries of T packed tokens attend to key tokens of the same packed
// arrays.  Token t admits key j when j lies in a 4-token block that t selects
// (sel_blocks[t, nb] != 0) and lo[t] <= j <= hi[t]; nothing else is added.
//     out[t, h]  = softmax_j(scale * q[t, h] . k[j, g]) v[j, g],  g = h / (Hq/Hkv)
//     lse[h, t]  = log sum_j exp(scale * q[t, h] . k[j, g])   (natural log)
// Empty rows give zeros and LSE = -inf.  out (bf16) is the rounding of out_fp32.
//
// Block spans: blocks are numbered globally and restart at each packed sequence,
// so under the packed-partition contract block nb of token t's sequence covers
// tokens tok_base[t] + 4 (nb - blk_base[t]) .. +3 (the last block of a sequence
// is cut by the sequence end, which no admitted key passes since hi[t] stays
// inside the sequence).  Only blocks nb_lo .. nb_hi whose span meets [lo, hi]
// can contribute; the kernel derives spans from (tok_base, blk_base) and host
// validation checks block_first / block_last against that partition.
//
// Each token's key set is its own, so keys are never shared between tokens:
// one wave handles one (token, KV head) and gathers exactly the keys it admits.
//   * candidate blocks go 1024 at a time into a per-wave LDS list of the
//     selected ones (bitmap bytes tested per lane, placed by a prefix sum);
//     groups of 4U selected blocks (16U keys: U = 2 at D = 128, 1 at D = 256)
//     are read from it;
//   * per group, S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (M = 16 keys, N = the
//     query heads of the KV head, at most 16); each lane loads its key row's 16
//     bytes straight into the A operand, and lane group g of the accumulator
//     holds exactly the 4 tokens of block 4u + g, so the key mask is per group;
//   * V rows go through a row-major LDS slab and come back with
//     ds_read_b64_tr_b16 as the A operand of O^T += V^T P^T, the same scheme as
//     the single-token decode kernel;
//   * group j + 1's loads are in flight while group j computes, and group
//     j + 2's block ids are extracted meanwhile.
// Workgroups are dealt round-robin over the 8 XCDs; each XCD takes a contiguous
// run of tokens, whose key sets overlap, so their K/V stay in its L2.
#include "device_common.h"
#include "pkb_internal.h"

namespace pkb {

namespace {
typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
constexpr int kQsaXcds = 8;
constexpr int kChunk = 1024;       // candidate blocks per selected-block list

// U 16-key units (4 blocks each) per group: two at D = 128; one at D = 256,
// which halves the K/V registers so that two waves fit per SIMD.
template <int D, int U>
struct QsaLayout {
  static constexpr int KEYS = 16 * U;          // keys per group
  static constexpr int NB = 4 * U;             // selected blocks per group
  static constexpr int VROW = D * 2 + 32;      // padded V row: transpose reads hit distinct banks
  static constexpr int LDS = KEYS * VROW;     // V slab; the block list follows it
  static constexpr int LDS_TOTAL = LDS + kChunk * 2;
  static constexpr int VP = KEYS * D / 8 / 64; // 16-byte V pieces per lane per group
};
}  // namespace

template <int D, int U>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2)))
qsa_kernel(const QsaParams p) {
  using Lay = QsaLayout<D, U>;
  constexpr int NB = Lay::NB;
  constexpr int KS = D / 32;       // k-steps of S^T over the head dim
  constexpr int DB = D / 16;       // 16-dim blocks of O^T
  constexpr int VP = Lay::VP;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* vs = smem;

  const int lane = threadIdx.x;
  const int g = lane >> 4;         // lane group
  const int qn = lane & 15;        // MFMA column: query head within the KV head's group

  const int total = p.T * p.Hkv;
  const int per = (total + kQsaXcds - 1) / kQsaXcds;
  const int item = (int)(blockIdx.x % kQsaXcds) * per + (int)(blockIdx.x / kQsaXcds);
  if (item >= total) return;
  const int t = item / p.Hkv;
  const int kvh = item - t * p.Hkv;
  const int G = p.G;

  const int lo = ld_const(p.lo, t), hi = ld_const(p.hi, t);
  const int tb = ld_const(p.tok_base, t), bb = ld_const(p.blk_base, t);
  // candidate blocks: those whose span meets [lo, hi], clamped to the bitmap
  int nb_lo = 0, nb_hi = -1;
  if (lo <= hi) {
    nb_lo = max(0, bb + ((lo - tb) >> 2));
    nb_hi = min(p.NB - 1, bb + ((hi - tb) >> 2));
  }
  const uint8_t* selrow = p.sel + (int64_t)t * p.NB;

  // ---- selected-block list ----
  // Candidates go kChunk at a time from a 16-aligned start: lane l tests blocks
  // cb + 16l .. cb + 16l + 15 (one 16-byte load of the bitmap row where the
  // row allows it, else 16 byte loads), keeps those inside [nb_lo, nb_hi], and
  // a wave-wide prefix sum of the counts places the selected ones, in order,
  // into this wave's LDS list (16-bit offsets from cb).  Groups then read 8
  // list entries from LDS, which never waits on the K/V loads in flight.
  uint16_t* list = (uint16_t*)(smem + Lay::LDS);
  int cb = nb_lo & ~15;    // first candidate of the current list
  int n_list = 0;          // entries in the current list
  int taken = 0;           // entries already handed out
  // 4 bits: which bytes of x are nonzero (bit 7 of each byte after the
  // carry-free test, then the four bits gathered by one multiply)
  auto nz_bytes = [](uint32_t x) -> uint32_t {
    const uint32_t t = (((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u;
    return ((t >> 7) * 0x00204081u >> 21) & 0xFu;
  };
  auto build = [&]() {
    const int first = cb + 16 * lane;
    uint32_t nz = 0;
    if (p.sel16) {
      // the row is 16-byte aligned and first is a multiple of 16: the load
      // stays inside the row whenever first <= NB - 16
      u32x4 w = {0u, 0u, 0u, 0u};
      if (first <= p.NB - 16) w = *(const u32x4*)(selrow + first);
#pragma unroll
      for (int d = 0; d < 4; ++d) nz |= nz_bytes(w[d]) << (4 * d);
    } else {
      // 16 unconditional byte loads (index clamped into the row) all in flight
      uint8_t x[16];
#pragma unroll
      for (int b = 0; b < 16; ++b) x[b] = selrow[min(first + b, p.NB - 1)];
#pragma unroll
      for (int b = 0; b < 16; ++b)
        if (x[b] != 0) nz |= 1u << b;
    }
    // keep the candidates inside [nb_lo, nb_hi]
    const int lo_cut = min(max(nb_lo - first, 0), 16);
    const int hi_cut = min(max(nb_hi + 1 - first, 0), 16);
    const int flags0 = (int)(nz & ((1u << hi_cut) - 1u) & ~((1u << lo_cut) - 1u));
    int flags = flags0;
    const int cnt = __builtin_popcount(flags);
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    int pos = incl - cnt;
    while (flags) {
      const int b = __builtin_ctz(flags);
      flags &= flags - 1;
      list[pos++] = (uint16_t)(16 * lane + b);
    }
    n_list = readlane_i32(incl, 63);
    taken = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // next NB selected blocks (id -1 past the end); returns how many are real
  auto take = [&](int (&id)[NB]) -> int {
    while (taken >= n_list) {
      if (n_list > 0 || taken > 0) cb += kChunk;   // the current list is used up
      if (cb > nb_hi) {
#pragma unroll
        for (int k = 0; k < NB; ++k) id[k] = -1;
        return 0;
      }
      build();
      if (n_list == 0) taken = 1;                   // empty chunk: move on
    }
    int e = -1;
    if (lane < NB && taken + lane < n_list) e = cb + (int)list[taken + lane];
#pragma unroll
    for (int k = 0; k < NB; ++k) id[k] = readlane_i32(e, k);
    const int n = min(NB, n_list - taken);
    taken += NB;
    return n;
  };

  // ---- Q^T fragments (B operand of S^T) ----
  bf16x8 qf[KS];
  {
    const uint16_t* qrow = p.q + ((int64_t)t * p.Hq + kvh * G + qn) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qn < G) x = ld_global_16(qrow + 32 * s);
      qf[s] = as_bf16x8(x);
    }
  }
  f32x4 oacc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) oacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int64_t tok_stride = (int64_t)p.Hkv * D;     // elements between tokens
  const uint16_t* kb = p.k + (int64_t)kvh * D;
  const uint16_t* vb = p.v + (int64_t)kvh * D;
  // first token of block id (any in-bounds token for id < 0)
  auto first_tok = [&](int id) -> int { return id >= 0 ? tb + 4 * (id - bb) : tb; };
  auto clamp_tok = [&](int x) -> int { return min(max(x, 0), p.T - 1); };
  // K / V pools are at most 4 GiB (checked at launch), so a row's byte offset
  // from the head's base fits 32 bits: the loads take the base from SGPRs and
  // one 32-bit offset per lane
  const uint32_t tok_bytes = (uint32_t)(tok_stride * 2);
  auto ld_row = [&](const uint16_t* base, uint32_t off) -> u32x4 {
    return *(const u32x4*)((const char*)base + off);
  };

  // V piece lane + 64i of a group is key 2i + lane/32 (D = 256) or 4i + lane/16
  // (D = 128): block v_block(i) (the same for the whole wave), token v_off(i)
  // inside it, 16-byte piece lane % (D/8) of the row
  auto v_block = [](int i) -> int { return D == 256 ? (i >> 1) : i; };
  auto v_off = [&](int i) -> int { return D == 256 ? 2 * (i & 1) + (lane >> 5) : (lane >> 4); };

  // Loads of one group: K rows straight into the A operand (lane key qn of unit u
  // is token first(id[4u + qn/4]) + qn%4); V pieces row-major, one block per load.
  auto load_group = [&](const int (&id)[NB], bf16x8 (&ka)[U][KS], u32x4 (&vr)[VP]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q4 = qn >> 2;
      const int f0 = first_tok(id[4 * u]), f1 = first_tok(id[4 * u + 1]);
      const int f2 = first_tok(id[4 * u + 2]), f3 = first_tok(id[4 * u + 3]);
      const int f = q4 == 0 ? f0 : (q4 == 1 ? f1 : (q4 == 2 ? f2 : f3));
      const uint32_t row = (uint32_t)clamp_tok(f + (qn & 3)) * tok_bytes + 16u * g;
#pragma unroll
      for (int s = 0; s < KS; ++s) ka[u][s] = as_bf16x8(ld_row(kb, row + 64u * s));
    }
#pragma unroll
    for (int i = 0; i < VP; ++i) {
      const int f = first_tok(id[v_block(i)]);
      vr[i] = ld_row(vb, (uint32_t)clamp_tok(f + v_off(i)) * tok_bytes + 16u * (lane & (D / 8 - 1)));
    }
  };

  // One group: S^T, masks, online softmax, V slab, O^T += V^T P^T.  The K/V
  // registers are consumed here; the caller's other buffer is loading meanwhile.
  auto compute = [&](bf16x8 (&ka)[U][KS], u32x4 (&vr)[VP], const int (&id_c)[NB]) {
    f32x4 sacc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      sacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        sacc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u][s], qf[s], sacc[u], 0, 0, 0);
    }
    // lane group g of unit u holds the 4 tokens of block id_c[4u + g]
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i0 = id_c[4 * u], i1 = id_c[4 * u + 1], i2 = id_c[4 * u + 2], i3 = id_c[4 * u + 3];
      const int id = g == 0 ? i0 : (g == 1 ? i1 : (g == 2 ? i2 : i3));
      const int f = first_tok(id);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = f + i;
        const bool ok = id >= 0 && tok >= lo && tok <= hi;
        const float sv = ok ? sacc[u][i] * p.scale_log2 : -INFINITY;
        sacc[u][i] = sv;
        mx = fmaxf(mx, sv);
      }
    }
    // dead keys' V rows are zeroed (no 0 * NaN)
#pragma unroll
    for (int i = 0; i < VP; ++i) {
      const int id = id_c[v_block(i)];
      const int tok = first_tok(id) + v_off(i);
      if (!(id >= 0 && tok >= lo && tok <= hi)) vr[i] = u32x4{0u, 0u, 0u, 0u};
    }
    mx = quad_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    float ps = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = fast_exp2(sacc[u][i] - m_use);
        sacc[u][i] = e;
        ps += e;
      }
    if (m_new != m_run) {
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

    // P^T as bf16 (B operand; lane group g holds keys 4g..4g+3 of each unit),
    // and for fp32 output the rounding residual as a second operand (~16-bit P)
    uint32_t pw[2 * U], plo[2 * U];
#pragma unroll
    for (int w = 0; w < 2 * U; ++w) {
      const f32x4& sa = sacc[w >> 1];
      const int i0 = 2 * (w & 1);
      pw[w] = pack_bf16x2(sa[i0], sa[i0 + 1]);
      plo[w] = 0u;
      if (p.out_f32)
        plo[w] = pack_bf16x2(sa[i0] - __uint_as_float(pw[w] << 16),
                             sa[i0 + 1] - __uint_as_float(pw[w] & 0xFFFF0000u));
    }
    // transpose-read addresses: lane (4r + c) of a 16-lane group reads row
    // 4g + r of each unit, dims 16d + 4c .. +3
    const int rr = (lane & 15) >> 2, cc = lane & 3;
    const unsigned char* a0 = vs + (4 * g + rr) * Lay::VROW + 8 * cc;
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(a0 + 32 * d));
      if constexpr (U == 2) {
        const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(a0 + 16 * Lay::VROW + 32 * d));
        const u32x2 w0 = __builtin_bit_cast(u32x2, x0);
        const u32x2 w1 = __builtin_bit_cast(u32x2, x1);
        const u32x4 aw = {w0[0], w0[1], w1[0], w1[1]};
        const u32x4 bw = {pw[0], pw[1], pw[2], pw[3]};
        oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(aw), as_bf16x8(bw), oacc[d], 0, 0, 0);
        if (p.out_f32) {
          const u32x4 bl = {plo[0], plo[1], plo[2], plo[3]};
          oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(aw), as_bf16x8(bl), oacc[d], 0, 0, 0);
        }
      } else {
        // one unit: K = 16 keys, v_mfma_f32_16x16x16_bf16 with the same lane layout
        const u32x2 bw = {pw[0], pw[1]};
        oacc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(x0, __builtin_bit_cast(i16x4, bw), oacc[d], 0, 0, 0);
        if (p.out_f32) {
          const u32x2 bl = {plo[0], plo[1]};
          oacc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(x0, __builtin_bit_cast(i16x4, bl), oacc[d], 0, 0, 0);
        }
      }
    }
    // the slab is rewritten next iteration: keep these reads before those writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  };

  // Two register buffers in ping-pong (the loop body is unrolled twice so no
  // buffer is ever copied: a copy would wait for the loads still in flight).
  // Per phase: enumerate the group after next (a list rebuild may wait, but
  // only for this phase's own group, which is needed right away), start the
  // next group's loads, compute this one.  The next group's loads are issued
  // even past the last group (all ids -1: in-bounds rows of the token's own
  // sequence, never used), so no phase merges paths with different numbers of
  // loads in flight -- such a merge would make the compute wait for all of them.
  int id_c[NB], id_n[NB], id_nn[NB];
  bf16x8 kA[U][KS], kB[U][KS];
  u32x4 vA[VP], vB[VP];
  int n_c = take(id_c);
  if (n_c > 0) load_group(id_c, kA, vA);
  int n_n = n_c > 0 ? take(id_n) : 0;
  auto rotate_ids = [&](int n_nn) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      id_c[k] = id_n[k];
      id_n[k] = id_nn[k];
    }
    n_c = n_n;
    n_n = n_nn;
  };
  while (n_c > 0) {
    {
      const int n_nn = n_n > 0 ? take(id_nn) : 0;
      load_group(id_n, kB, vB);
      compute(kA, vA, id_c);
      rotate_ids(n_nn);
    }
    if (n_c == 0) break;
    {
      const int n_nn = n_n > 0 ? take(id_nn) : 0;
      load_group(id_n, kA, vA);
      compute(kB, vB, id_c);
      rotate_ids(n_nn);
    }
  }

  // ---- epilogue: lane (qn, g) holds O^T rows 16d + 4g + i of head qn ----
  const float l_tot = quad_sum(l_run);
  if (qn >= G) return;
  const int hq = kvh * G + qn;
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  const int64_t orow = (int64_t)t * p.Hq + hq;
  if (p.out_f32) {
    float* o = p.out_f32 + orow * D;
#pragma unroll
    for (int d = 0; d < DB; ++d) *(f32x4*)(o + 16 * d + 4 * g) = oacc[d] * inv;
  }
  if (p.out) {
    uint16_t* o = p.out + orow * D;
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      u32x2 w;
      w[0] = pack_bf16x2(oacc[d][0] * inv, oacc[d][1] * inv);
      w[1] = pack_bf16x2(oacc[d][2] * inv, oacc[d][3] * inv);
      *(u32x2*)(o + 16 * d + 4 * g) = w;
    }
  }
  if (p.lse && g == 0)
    p.lse[(int64_t)hq * p.T + t] = empty ? -INFINITY : (m_run + __log2f(l_tot)) * kLn2;
}

template <int D, int U>
static hipError_t launch_qsa_d(const QsaParams& p, hipStream_t st) {
  const int64_t total = (int64_t)p.T * p.Hkv;
  const int64_t per = (total + kQsaXcds - 1) / kQsaXcds;
  if (per * kQsaXcds > 0x7fffffff) return hipErrorInvalidValue;
  QsaParams arg = p;
  void* args[] = {(void*)&arg};
  return hipLaunchKernel((const void*)qsa_kernel<D, U>, dim3((unsigned)(per * kQsaXcds)), dim3(64),
                         args, QsaLayout<D, U>::LDS_TOTAL, st);
}

hipError_t launch_qsa(const QsaParams& p, int D, hipStream_t stream) {
  if (D == 128) return launch_qsa_d<128, 2>(p, stream);
  if (D == 256) return launch_qsa_d<256, 1>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkb
