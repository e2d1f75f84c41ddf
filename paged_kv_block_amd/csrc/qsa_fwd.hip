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
//   * candidate blocks go 64 at a time: each lane loads one bitmap byte and a
//     ballot gives the window's selected blocks as a scalar mask; selected block
//     ids are peeled off 8 at a time (a group of 32 keys) with scalar bit scans;
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

template <int D>
struct QsaLayout {
  static constexpr int KEYS = 32;              // keys per group (8 blocks of 4)
  static constexpr int VROW = D * 2 + 32;      // padded V row: transpose reads hit distinct banks
  static constexpr int LDS = KEYS * VROW;
  static constexpr int VP = KEYS * D / 8 / 64; // 16-byte V pieces per lane per group
};
}  // namespace

template <int D>
__global__ void __launch_bounds__(64) qsa_kernel(const QsaParams p) {
  using Lay = QsaLayout<D>;
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

  // ---- selected-block enumeration (scalar) ----
  int win = nb_lo;                                   // first candidate of the loaded window
  uint64_t mask = 0;                                 // selected, not yet taken, in window win - 64
  int wb = 0;                                        // this lane's byte of window `win`
  auto load_window = [&]() {
    wb = 0;
    if (win + lane <= nb_hi) wb = selrow[win + lane];
  };
  int mbase = 0;                                     // first candidate of `mask`'s window
  auto refill = [&]() -> bool {                      // false: no candidates left
    while (mask == 0) {
      if (win > nb_hi) return false;
      mask = __ballot(wb != 0);
      mbase = win;
      win += 64;
      load_window();
    }
    return true;
  };
  // take the next 8 selected blocks (id -1 when exhausted); returns the count
  auto take8 = [&](int (&id)[8]) -> int {
    int n = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      id[k] = -1;
      if (refill()) {
        const int bit = __builtin_ctzll(mask);
        mask &= mask - 1;
        id[k] = mbase + bit;
        ++n;
      }
    }
    return n;
  };
  load_window();

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
  auto clamp_tok = [&](int x) -> int64_t { return (int64_t)min(max(x, 0), p.T - 1); };

  // V piece lane + 64i of a group is key 2i + lane/32 (D = 256) or 4i + lane/16
  // (D = 128): block v_block(i) (the same for the whole wave), token v_off(i)
  // inside it, 16-byte piece lane % (D/8) of the row
  auto v_block = [](int i) -> int { return D == 256 ? (i >> 1) : i; };
  auto v_off = [&](int i) -> int { return D == 256 ? 2 * (i & 1) + (lane >> 5) : (lane >> 4); };

  // Loads of one group: K rows straight into the A operand (lane key qn of unit u
  // is token first(id[4u + qn/4]) + qn%4); V pieces row-major, one block per load.
  auto load_group = [&](const int (&id)[8], bf16x8 (&ka)[2][KS], u32x4 (&vr)[VP]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q4 = qn >> 2;
      const int f0 = first_tok(id[4 * u]), f1 = first_tok(id[4 * u + 1]);
      const int f2 = first_tok(id[4 * u + 2]), f3 = first_tok(id[4 * u + 3]);
      const int f = q4 == 0 ? f0 : (q4 == 1 ? f1 : (q4 == 2 ? f2 : f3));
      const uint16_t* row = kb + clamp_tok(f + (qn & 3)) * tok_stride + 8 * g;
#pragma unroll
      for (int s = 0; s < KS; ++s) ka[u][s] = as_bf16x8(ld_global_16(row + 32 * s));
    }
#pragma unroll
    for (int i = 0; i < VP; ++i) {
      const int f = first_tok(id[v_block(i)]);
      vr[i] = ld_global_16(vb + clamp_tok(f + v_off(i)) * tok_stride + 8 * (lane & (D / 8 - 1)));
    }
  };

  int id_c[8], id_n[8], id_nn[8];
  int n_c = take8(id_c);
  int n_n = take8(id_n);
  bf16x8 ka[2][KS], ka_n[2][KS];
  u32x4 vr[VP], vr_n[VP];
  if (n_c > 0) load_group(id_c, ka, vr);

  while (n_c > 0) {
    // next group's loads fly while this one computes; the one after is enumerated
    if (n_n > 0) load_group(id_n, ka_n, vr_n);
    const int n_nn = n_n > 0 ? take8(id_nn) : 0;

    f32x4 sacc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      sacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        sacc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u][s], qf[s], sacc[u], 0, 0, 0);
    }
    // lane group g of unit u holds the 4 tokens of block id_c[4u + g]
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
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
    for (int u = 0; u < 2; ++u)
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

    u32x4 pw;
    pw[0] = pack_bf16x2(sacc[0][0], sacc[0][1]);
    pw[1] = pack_bf16x2(sacc[0][2], sacc[0][3]);
    pw[2] = pack_bf16x2(sacc[1][0], sacc[1][1]);
    pw[3] = pack_bf16x2(sacc[1][2], sacc[1][3]);
    u32x4 plo = {0u, 0u, 0u, 0u};
    if (p.out_f32) {
      // fp32 output: P - bf16(P) enters as a second operand (~16-bit P)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x4& sa = sacc[w >> 1];
        const int i0 = 2 * (w & 1);
        plo[w] = pack_bf16x2(sa[i0] - __uint_as_float(pw[w] << 16),
                             sa[i0 + 1] - __uint_as_float(pw[w] & 0xFFFF0000u));
      }
    }
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
      if (p.out_f32)
        oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(aw), as_bf16x8(plo), oacc[d], 0, 0, 0);
    }
    // the slab is rewritten next iteration: keep these reads before those writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();

    // rotate the pipeline
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int s = 0; s < KS; ++s) ka[u][s] = ka_n[u][s];
#pragma unroll
    for (int i = 0; i < VP; ++i) vr[i] = vr_n[i];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      id_c[k] = id_n[k];
      id_n[k] = id_nn[k];
    }
    n_c = n_n;
    n_n = n_nn;
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

template <int D>
static hipError_t launch_qsa_d(const QsaParams& p, hipStream_t st) {
  const int64_t total = (int64_t)p.T * p.Hkv;
  const int64_t per = (total + kQsaXcds - 1) / kQsaXcds;
  if (per * kQsaXcds > 0x7fffffff) return hipErrorInvalidValue;
  QsaParams arg = p;
  void* args[] = {(void*)&arg};
  return hipLaunchKernel((const void*)qsa_kernel<D>, dim3((unsigned)(per * kQsaXcds)), dim3(64),
                         args, QsaLayout<D>::LDS, st);
}

hipError_t launch_qsa(const QsaParams& p, int D, hipStream_t stream) {
  if (D == 128) return launch_qsa_d<128>(p, stream);
  if (D == 256) return launch_qsa_d<256>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkb
