// attn_fwd_kernel.h -- bf16 scaled-dot-product attention over a paged KV cache
// for gfx950: block-sparse rows, packed prefill and split-KV decode share one
// kernel template, instantiated by attn_fwd.hip (page sizes that are multiples
// of 8) and attn_ragged.hip (other page sizes) so the two compile in parallel.
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
// head of the group.  Each wavefront owns 32 packed rows; up to 4 waves share
// one KV tile, and two such workgroups run per CU (two waves per SIMD from
// independent workgroups: no barrier keeps them in step, which measured faster
// than one 8-wave workgroup).
//
// KV tiles are 64 keys = 8 chunks of 8 logical tokens.  When the page size is a
// multiple of 8 (always for prefill) an 8-token run never crosses a page, so
// each chunk is one contiguous [8, D] slab of the HND pool; other page sizes
// (block-sparse and decode pools) copy each row from its own page.  Tiles go HBM -> LDS through
// direct-to-LDS loads (global_load_lds_dwordx4: 1 KB per wave instruction, no
// registers) into a K ring and a V ring, one tile ahead of use, with
// one workgroup barrier per tile.  Each copy takes its chunk's pool address
// from SGPRs plus a per-lane 32-bit offset fixed per instruction, so issuing a
// tile's copies needs no vector ALU work.  Rows are stored unpadded with their 16-byte
// pieces permuted per row: K piece l sits at l ^ (key & 15), so the A-operand
// reads of 16 consecutive keys hit distinct banks; the V permutation (v_swz)
// spreads the four 16-lane groups of a transpose read over all 64 banks.
//
// A tile is described by a 64-bit mask of the keys that can be admitted (live,
// valid, inside the workgroup's causal/window band) and the first token of each
// chunk.  Where the visited keys are contiguous (prefill, decode, and sparse
// blocks of 64 or more keys) that is one start token and the mask comes from a
// few scalar operations; only the chunk a wave copies needs its page looked up,
// and that lookup is done one iteration early.  Dead chunks copy the tile's
// first live chunk and rows at or past the live length re-read their chunk's
// first row, so LDS never holds non-finite data.
//
// Per tile and 32-row block:
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (M = keys, N = query rows,
//     K = head dim): every lane holds 16 keys of ONE query row per 32 keys, so
//     the row max needs one exchange between the two half-waves;
//   * masks are applied only to tiles that need them (an invalid or cut key,
//     the causal diagonal, the window edge);
//   * online softmax in base 2: exp2(s * scale * log2 e - m) as one FMA and one
//     exp; the reference m only moves when a row max passes it by more than a
//     fixed slack, so the running output is rarely rescaled;
//   * O^T += V^T P^T: the V^T operand comes from ds_read_b64_tr_b16, which
//     returns a 4-key x 16-dim block of the row-major V tile column-wise; lane
//     half h then holds keys {4h..4h+3, 8+4h..8+4h+3} of each 16-key step --
//     exactly the keys its S^T accumulator holds, so P^T feeds the MFMA as is.
#ifndef PKB_ATTN_FWD_KERNEL_H_
#define PKB_ATTN_FWD_KERNEL_H_

#include <atomic>

#include "device_common.h"
#include "pkb_internal.h"

namespace pkb {

typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef float f32x2e __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2e __attribute__((ext_vector_type(2)));

template <int D, int NW>
struct AttnLayout {
  static constexpr int KT = kKvTile;             // keys per tile
  static constexpr int ROWB = D * 2;             // bytes per K / V row
  static constexpr int TILE_B = KT * ROWB;       // bytes of a K (or V) tile
  // Tiles of copy lookahead: tile t is copied LA = 1 iteration before it is
  // read, into the ring slot (of two per ring) whose previous tile every wave
  // has finished.  That keeps two workgroups per CU at D = 128 (64 KB each).
  static constexpr int LA = 1;
  static constexpr int NSK = LA + 1;
  static constexpr int NSV = LA + 1;
  static constexpr int V_BASE = NSK * TILE_B;
  static constexpr int LDS = (NSK + NSV) * TILE_B;
  static constexpr int INSTR = TILE_B / 1024;    // 1 KB DMA instructions per K (or V) tile
  static constexpr int KPI = 1024 / ROWB;        // key rows per DMA instruction
  static constexpr int LPK = 64 / KPI;           // lanes per key row in one instruction
  static constexpr int IPW = INSTR / NW;         // K (and V) instructions per wave per tile
};

// Waves per SIMD that the LDS footprint allows (160 KB per CU).  Telling the
// compiler keeps it from trimming registers for an occupancy it cannot reach.
template <int D, int NW>
constexpr int attn_waves_per_simd() {
  constexpr int wgs = (160 * 1024) / AttnLayout<D, NW>::LDS;
  constexpr int w = wgs * NW / 4;
  return w < 1 ? 1 : (w > 8 ? 8 : w);
}

// Physical 16-byte piece of logical piece lp in V row `key`, and its inverse.
// The XOR with 2*(key & 3) separates the four rows of one transpose read; the
// bit-3 flip by (bit 1 of lp) ^ (bit 2 of key) moves the 16-lane groups that
// read other dims or other rows of the same 16-key step to the other 32 banks.
__device__ __forceinline__ int v_swz(int key, int lp) {
  const int x = lp ^ (2 * (key & 3));
  return x ^ (8 * (((lp >> 1) & 1) ^ ((key >> 2) & 1)));
}
__device__ __forceinline__ int v_unswz(int key, int pp) {
  const int x = pp ^ (2 * (key & 3));
  return x ^ (8 * (((x >> 1) & 1) ^ ((key >> 2) & 1)));
}

// Two floats -> packed bf16 pair (round to nearest even) in one instruction.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  const f32x2e v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2e));
}

// Waits until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 16 bytes per lane from the wave-uniform address base + byte offset off to LDS
// address lds_a + lds_b + 16 * lane (global_load_lds_dwordx4 in its
// scalar-base form: the 64-bit base sits in SGPRs, each lane adds 32 bits; the
// LDS base is taken from M0, written by one SALU add, which needs one wait
// state before the copy).  Written as inline assembly so the compiler does not
// treat every later LDS read as depending on every copy in flight: the kernel
// orders copies and reads itself with s_waitcnt vmcnt and barriers (both
// ordered with volatile asm), and the data read here is never written.
__device__ __forceinline__ void lds_dma16_s(const void* base, uint32_t off, uint32_t lds_a, uint32_t lds_b) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(lds_a), "s"(lds_b) : "m0", "scc");
}

// The same copy from a per-lane 64-bit address (global_load_lds_dwordx4 with
// a VGPR address and no scalar base); LDS destination M0 + 16 * lane.
__device__ __forceinline__ void lds_dma16_v(const void* addr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(addr), "s"(lds_addr) : "m0");
}

// Lanes whose bit is set in the 64-bit scalar mask keep x, the others take y
// (one v_cndmask with the mask as its condition; written with the inverse
// ballot so that the compiler sees the read of x, which may be an MFMA result
// still in flight, and inserts the wait states it needs).
__device__ __forceinline__ float select_lanes(uint64_t mask, float x, float y) {
  return __builtin_amdgcn_inverse_ballot_w64(mask) ? x : y;
}

// Slack of the softmax reference max, in log2 units.
constexpr float kRescaleSlack = 8.0f;
constexpr float kSlackPow = 256.0f;   // 2^kRescaleSlack

// One KV tile, wave-uniform.  CPW = chunks this wave copies (8 / waves).
template <int CPW>
struct TileMeta {
  uint64_t M;       // bit k: key k may be admitted (live, valid, inside [k_lo, k_hi))
  int t0;           // first token (contiguous tiles)
  int tmin, tmax;   // token range of the tile's chunks with admissible keys
  int ts[8];        // first token of each chunk (tiles of small sparse blocks)
  int64_t src[CPW]; // pool offset of the chunk each of this wave's copies reads
  int tsrc[CPW];    // and its first token
};

template <int D, int NW, int MODE, bool F32, bool CONTIG, bool RAGGED>
__global__ void __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(attn_waves_per_simd<D, NW>(), attn_waves_per_simd<D, NW>())))
attn_fwd_kernel(const AttnParams p) {
  using Lay = AttnLayout<D, NW>;
  constexpr int TILE_M = 32 * NW;
  constexpr int NKS = D / 16;           // S^T k-steps over the head dim
  constexpr int NDB = D / 32;           // 32-row blocks of O^T
  constexpr int IPW = Lay::IPW;
  static_assert(Lay::INSTR % NW == 0, "tile instructions must split evenly over waves");

  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int hh = lane >> 5;        // half-wave
  const int ql = lane & 31;        // query row inside the wave
  int kvh = blockIdx.y;
  const int G = p.G;

  // ---------------- work item ----------------
  int b, qlen, tok_base, m_begin, m_end, split = 0;
  int bip_lo = 0, n_sel = 0;
  if (MODE == kModeBsa) {
    // XCD-aware order: the 1-D grid deals workgroups round-robin over the 8
    // XCDs; XCD c takes items [c * per, (c + 1) * per) of the (b, kvh, x) list
    const int nx = p.nqb * p.tiles_per_brow;
    const int total = nx * p.Hkv * p.B;
    const int per = (total + 7) >> 3;
    const int item = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (item >= total) return;
    const int xi = item % nx;
    kvh = (item / nx) % p.Hkv;
    b = item / (nx * p.Hkv);
    const int x = nx - 1 - xi;   // late rows first
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
    // 1-D grid, KV head fastest: the work list is longest-first, so the whole
    // launch is dealt longest-first, and with 8 KV heads each XCD keeps one
    // head's K/V in its L2
    const int w = (int)blockIdx.x / p.Hkv;
    kvh = (int)blockIdx.x - w * p.Hkv;
    b = p.worklist[2 * w];
    m_begin = p.worklist[2 * w + 1];
    tok_base = p.qo_indptr[b];
    qlen = p.qo_indptr[b + 1] - tok_base;
    m_end = min(m_begin + TILE_M, qlen * G);
  } else {
    // split-KV decode: blockIdx.x = row tile * splits + split, one request per z
    b = blockIdx.z;
    const int rt = (int)blockIdx.x / p.num_splits;
    split = (int)blockIdx.x - rt * p.num_splits;
    if (p.qo_indptr) {
      tok_base = p.qo_indptr[b];
      qlen = p.qo_indptr[b + 1] - tok_base;
    } else {
      qlen = p.Sq;
      tok_base = b * p.Sq;
    }
    m_begin = rt * TILE_M;
    m_end = min(m_begin + TILE_M, qlen * G);
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

  // Chunks (8 tokens) this wave copies per tile, and their token span.  When
  // every wave's span of a tile lies inside one page -- contiguous walks whose
  // tiles start on a multiple of the span, with page_size a multiple of it --
  // each tile's copy sources come from lane-parallel descriptors (below).
  constexpr int CPW = 8 / NW;
  constexpr int SPAN = 8 * CPW;
  const bool fast = CONTIG && p.page_size % SPAN == 0;
  // RAGGED: the page size is not a multiple of 8 (block-sparse and decode
  // pools), so an 8-token chunk may span pages and its rows are copied one by
  // one (issue_ragged below).
  constexpr bool ragged = RAGGED;
  // page sizes below 8: row quotients by multiply-high with ceil(2^32 / page_size)
  const bool small_pages = RAGGED && p.page_size < 8;
  const uint64_t ps_magic =
      small_pages ? ((1ull << 32) + (uint64_t)p.page_size - 1) / (uint64_t)p.page_size : 0ull;

  // visited KV: contiguous modes walk [lo8, k_hi) in 64-token tiles (lo8 a
  // multiple of 8, and of SPAN on the fast path); sparse rows walk their
  // selected blocks in order, 8-token chunks packed 8 per tile
  int n_tiles, lo8 = 0;
  if (MODE == kModeBsa) {
    n_tiles = CONTIG ? n_sel * (p.kvbs >> 6) : (n_sel * (p.kvbs >> 3) + 7) >> 3;
  } else {
    lo8 = k_lo & (fast ? -SPAN : -8);
    n_tiles = (k_hi > k_lo) ? (k_hi - lo8 + 63) >> 6 : 0;
  }

  // ---------------- tile metadata (scalar; identical in every wave) ----------------
  const int64_t head_off = (int64_t)kvh * p.kv_head_stride;
  const int32_t* ids = MODE == kModePrefill ? p.block_tables + (int64_t)b * p.bt_stride
                                            : p.kv_indices + p.kv_indptr[b];
  const int ps_sh = __builtin_ctz(p.page_size | 0x40000000);
  const bool ps_pow2 = (p.page_size & (p.page_size - 1)) == 0;
  const int blk_tiles = p.kvbs >> 6;                 // tiles per sparse block (>= 64 keys)
  const int bt_sh = __builtin_ctz(blk_tiles | 0x40000000);
  const bool bt_pow2 = (blk_tiles & (blk_tiles - 1)) == 0;
  const int cpb_sh = __builtin_ctz((p.kvbs >> 3) | 0x40000000);   // chunks per small block (1, 2, 4)

  // admissible bits of the 8 keys from token t (a multiple of 8)
  auto chunk_bits = [&](int t) -> uint32_t {
    const int lo_cut = min(max(k_lo - t, 0), 8);
    const int hi_cut = min(max(k_hi - t, 0), 8);
    uint32_t bits = ((1u << hi_cut) - 1u) & ~((1u << lo_cut) - 1u);
    if (MODE == kModeBsa && p.valid_bits && bits)
      bits &= ld_const(p.valid_bits, (int64_t)b * p.valid_words + (t >> 5)) >> (t & 31);
    return bits & 0xFFu;
  };
  // first token of chunk v of a row's small-block walk
  auto small_chunk_token = [&](int v) -> int {
    const int qq = v >> cpb_sh;
    return ld_const(p.block_indices, bip_lo + qq) * p.kvbs + (v - (qq << cpb_sh)) * 8;
  };

  using TM = TileMeta<CPW>;

  // Lane-parallel tile descriptors (fast path): lane l describes tile
  // j0 + l -- its first token, the pool offset of this wave's SPAN tokens (a
  // span at or past L, whose pages may not exist, is redirected to the last
  // live span; the copies of such rows are never used), and for block-sparse
  // tiles the two validity words of its 64 keys.  The tile loop reads them with
  // v_readlane instead of a chain of dependent scalar loads, divisions by the
  // page size and 64-bit products per tile.
  int d_t0 = 0;
  int64_t d_src = 0;
  uint32_t d_w0 = ~0u, d_w1 = ~0u;
  auto load_desc = [&](int j0) {
    const int j = j0 + lane;
    const bool live = j < n_tiles;
    int t0 = 0;
    if (live) {
      if (MODE == kModeBsa) {
        const int qq = bt_pow2 ? (j >> bt_sh) : j / blk_tiles;
        t0 = p.block_indices[bip_lo + qq] * p.kvbs + (j - qq * blk_tiles) * 64;
      } else {
        t0 = lo8 + 64 * j;
      }
    }
    d_t0 = t0;
    int tw = t0 + SPAN * wave;
    if (tw >= L) tw = max((L - 1) & -SPAN, 0);
    const int pi = ps_pow2 ? (tw >> ps_sh) : tw / p.page_size;
    const int id = live ? ids[pi] : 0;
    d_src = (int64_t)id * p.kv_page_stride + head_off + (int64_t)(tw - pi * p.page_size) * D;
    if (MODE == kModeBsa && p.valid_bits) {
      // keys t0..t0+63 are two whole words; the second is read only when it
      // exists in the row (its bits are used only when t0 + 32 < L)
      const int64_t w = (int64_t)b * p.valid_words + (t0 >> 5);
      d_w0 = live ? p.valid_bits[w] : 0u;
      d_w1 = (live && (t0 >> 5) + 1 < p.valid_words) ? p.valid_bits[w + 1] : 0u;
    }
  };
  if (fast && n_tiles > 0) load_desc(0);
  // pool offsets of the chunks this wave copies (tm.tsrc set)
  auto fill_src = [&](TM& tm) {
    int pi[CPW], id[CPW];
#pragma unroll
    for (int lc = 0; lc < CPW; ++lc) pi[lc] = ps_pow2 ? (tm.tsrc[lc] >> ps_sh) : tm.tsrc[lc] / p.page_size;
    // (consecutive chunks usually share a page: one load then serves both)
#pragma unroll
    for (int lc = 0; lc < CPW; ++lc) {
      if (lc > 0 && pi[lc] == pi[lc - 1]) id[lc] = id[lc - 1];
      else id[lc] = ld_const(ids, pi[lc]);
    }
#pragma unroll
    for (int lc = 0; lc < CPW; ++lc)
      tm.src[lc] = (int64_t)id[lc] * p.kv_page_stride + head_off +
                   (int64_t)(tm.tsrc[lc] - pi[lc] * p.page_size) * D;
  };
  auto tile_meta = [&](int j) -> TM {
    TM tm;
    if (CONTIG && fast) {
      const int jj = j & 63;
      if (jj == 0 && j > 0) load_desc(j);   // next 64 tiles (rare)
      const int t0 = readlane_i32(d_t0, jj);
      if (t0 >= k_lo && t0 + 64 <= k_hi) {
        // Interior tile (the common case): every key is inside [k_lo, k_hi)
        // and below L, so no range cut and no copy redirection.  The token
        // bounds cover the whole tile; they only decide whether the causal and
        // window masks run, which is exact either way.
        uint64_t M = ~0ull;
        if (MODE == kModeBsa && p.valid_bits) {
          const uint32_t w0 = (uint32_t)readlane_i32((int)d_w0, jj);
          const uint32_t w1 = (uint32_t)readlane_i32((int)d_w1, jj);
          M = (uint64_t)w0 | ((uint64_t)w1 << 32);
        }
        tm.M = M;
        tm.t0 = t0;
        tm.tmin = t0;
        tm.tmax = t0 + 63;
        const int tw = t0 + SPAN * wave;
        const int64_t src = readlane_i64(d_src, jj);
#pragma unroll
        for (int lc = 0; lc < CPW; ++lc) {
          tm.tsrc[lc] = tw + 8 * lc;
          tm.src[lc] = src + (int64_t)(8 * lc) * D;
        }
        return tm;
      }
      const int lo = min(max(k_lo - t0, 0), 64);
      const int hi = min(max(k_hi - t0, 0), 64);
      uint64_t M = (hi >= 64 ? ~0ull : ((1ull << hi) - 1ull)) & ~(lo >= 64 ? ~0ull : ((1ull << lo) - 1ull));
      if (MODE == kModeBsa && p.valid_bits && M) {
        const uint32_t w0 = (uint32_t)readlane_i32((int)d_w0, jj);
        const uint32_t w1 = (uint32_t)readlane_i32((int)d_w1, jj);
        M &= (uint64_t)w0 | ((t0 + 32 < L) ? (uint64_t)w1 << 32 : 0ull);
      }
      tm.M = M;
      tm.t0 = t0;
      const int c_first = M ? (__builtin_ctzll(M) >> 3) : 0;
      const int c_last = M ? ((63 - __builtin_clzll(M)) >> 3) : 0;
      tm.tmin = t0 + 8 * c_first;
      tm.tmax = t0 + 8 * c_last + 7;
      if (M) {
        // the span's first chunk is live (tw < L); a chunk at or past L copies
        // it instead, so LDS never holds what lies past the sequence
        int tw = t0 + SPAN * wave;
        if (tw >= L) tw = max((L - 1) & -SPAN, 0);
        const int64_t src = readlane_i64(d_src, jj);
#pragma unroll
        for (int lc = 0; lc < CPW; ++lc) {
          const bool live = tw + 8 * lc < L;
          tm.tsrc[lc] = live ? tw + 8 * lc : tw;
          tm.src[lc] = live ? src + (int64_t)(8 * lc) * D : src;
        }
      }
    } else if (CONTIG) {
      int t0;
      if (MODE == kModeBsa) {
        const int qq = bt_pow2 ? (j >> bt_sh) : j / blk_tiles;
        t0 = ld_const(p.block_indices, bip_lo + qq) * p.kvbs + (j - qq * blk_tiles) * 64;
      } else {
        t0 = lo8 + 64 * j;
      }
      const int lo = min(max(k_lo - t0, 0), 64);
      const int hi = min(max(k_hi - t0, 0), 64);
      uint64_t M = (hi >= 64 ? ~0ull : ((1ull << hi) - 1ull)) & ~(lo >= 64 ? ~0ull : ((1ull << lo) - 1ull));
      const uint64_t M_range = M;
      if (MODE == kModeBsa && p.valid_bits && M) {
        // t0 is a multiple of 64 here: keys t0..t0+63 are two whole words; the
        // second is used only when t0 + 32 < L (its index is clamped to the array)
        const int64_t w = (int64_t)b * p.valid_words + (t0 >> 5);
        const int64_t w_last = (int64_t)p.B * p.valid_words - 1;
        const uint32_t lo = ld_const(p.valid_bits, w);
        const uint32_t hi = ld_const(p.valid_bits, w + 1 < w_last ? w + 1 : w_last);
        M &= (uint64_t)lo | ((t0 + 32 < L) ? (uint64_t)hi << 32 : 0ull);
      }
      tm.M = M;
      tm.t0 = t0;
      const int c_first = M ? (__builtin_ctzll(M) >> 3) : 0;
      const int c_last = M ? ((63 - __builtin_clzll(M)) >> 3) : 0;
      tm.tmin = t0 + 8 * c_first;
      tm.tmax = t0 + 8 * c_last + 7;
      if (M) {
        // chunks outside [k_lo, k_hi) copy the first chunk inside it
        const int t_r = max(t0, k_lo & ~7);
#pragma unroll
        for (int lc = 0; lc < CPW; ++lc) {
          const int c = wave * CPW + lc;
          const bool in_range = (M_range >> (8 * c)) & 0xFFu;
          tm.tsrc[lc] = in_range ? t0 + 8 * c : t_r;
        }
        if (!ragged) fill_src(tm);
      }
    } else {
      uint64_t M = 0;
      int t_first = -1, tmin = 0x7fffffff, tmax = -1;
      const int nch = n_sel << cpb_sh;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int v = j * 8 + c;
        tm.ts[c] = 0;
        if (v < nch) {
          const int t = small_chunk_token(v);
          tm.ts[c] = t;
          const uint32_t bw = chunk_bits(t);
          M |= (uint64_t)bw << (8 * c);
          if (bw) {
            if (t_first < 0) t_first = t;
            tmin = min(tmin, t);
            tmax = max(tmax, t + 7);
          }
        }
      }
      tm.M = M;
      tm.t0 = 0;
      tm.tmin = tmin;
      tm.tmax = tmax;
      if (M) {
        // chunks without an admissible key copy the first chunk with one
#pragma unroll
        for (int lc = 0; lc < CPW; ++lc) {
          const int c = wave * CPW + lc;
          tm.tsrc[lc] = ((M >> (8 * c)) & 0xFFu) ? small_chunk_token(j * 8 + c) : t_first;
        }
        if (!ragged) fill_src(tm);
      }
    }
    return tm;
  };

  // This wave's share of tile j's copies into its K and V ring slots.  Lane l of K (V)
  // instruction i writes LDS bytes i*1024 + 16l: row i*KPI + l/LPK, physical
  // piece l%LPK, so it fetches the logical piece stored there.
  // rows past the sequence end read their chunk's first row instead; the
  // per-row test is needed only when one of this wave's chunks is partial
  auto tile_whole = [&](const TM& tm) -> bool {
    bool whole = true;
#pragma unroll
    for (int lc = 0; lc < CPW; ++lc) whole = whole && (tm.tsrc[lc] + 8 <= L);
    return whole;
  };
  // instruction ii of the copies of a whole tile j (no row of it past L): its
  // K copy (part bit 0) and V copy (bit 1)
  auto issue_whole = [&](const TM& tm, int j, int ii, int part = 3) {
    const uint32_t kst = lds_base + (j % Lay::NSK) * Lay::TILE_B;
    const uint32_t vst = lds_base + Lay::V_BASE + (j % Lay::NSV) * Lay::TILE_B;
    const int i = wave * IPW + ii;
    const int lc = (ii * Lay::KPI) >> 3;   // = chunk (i * KPI) / 8 - wave * CPW
    const int key = i * Lay::KPI + lane / Lay::LPK;
    const uint32_t row = (uint32_t)((key & 7) * D * 2);
    const int pp = lane % Lay::LPK;
    if (part & 1) lds_dma16_s(p.k + tm.src[lc], row + (uint32_t)((pp ^ (key & 15)) * 16), kst, i * 1024);
    if (part & 2) lds_dma16_s(p.v + tm.src[lc], row + (uint32_t)(v_unswz(key, pp) * 16), vst, i * 1024);
  };
  // Copies of tile j when chunks may span pages.  Each instruction still
  // copies KPI whole rows (1 KB), but from a per-lane address.  Per chunk, the
  // pool offsets of its 8 rows are computed in scalar registers: one division
  // gives the page and slot of the chunk's first token, and row r's slot
  // s0 + r crosses at most one page boundary when the page size is 8 or more
  // (else its quotient comes from a multiply by ceil(2^32 / page_size), exact
  // for these small operands); the 8 page-ID loads are independent and share
  // one wait.  Every lane then picks its row's offset.  Rows at or past L
  // re-read their chunk's first token, so the LDS layout and contents match
  // the paged path's.
  auto issue_ragged = [&](const TM& tm, int j) {
    const uint32_t kst = lds_base + (j % Lay::NSK) * Lay::TILE_B;
    const uint32_t vst = lds_base + Lay::V_BASE + (j % Lay::NSV) * Lay::TILE_B;
    const int lrow = lane / Lay::LPK;
    const int pp = lane % Lay::LPK;
    constexpr int IPC = 8 / Lay::KPI;          // instructions per chunk
#pragma unroll
    for (int lc = 0; lc < CPW; ++lc) {
      const int t = tm.tsrc[lc];
      const int pi0 = t / p.page_size;
      const int s0 = t - pi0 * p.page_size;
      int pidx[8], slot[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int x = s0 + (t + r < L ? r : 0);
        const int q = small_pages ? (int)(((uint64_t)x * ps_magic) >> 32) : (int)(x >= p.page_size);
        pidx[r] = pi0 + q;
        slot[r] = x - q * p.page_size;
      }
      int id[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) id[r] = ld_const(ids, pidx[r]);
      int64_t rs[8];
#pragma unroll
      for (int r = 0; r < 8; ++r)
        rs[r] = (int64_t)id[r] * p.kv_page_stride + head_off + (int64_t)slot[r] * D;
#pragma unroll
      for (int c = 0; c < IPC; ++c) {
        const int ii = lc * IPC + c;
        const int i = wave * IPW + ii;
        int64_t src = rs[c * Lay::KPI];
#pragma unroll
        for (int k = 1; k < Lay::KPI; ++k) src = lrow == k ? rs[c * Lay::KPI + k] : src;
        const int key = i * Lay::KPI + lrow;
        lds_dma16_v(p.k + src + (pp ^ (key & 15)) * 8, kst + i * 1024);
        lds_dma16_v(p.v + src + v_unswz(key, pp) * 8, vst + i * 1024);
      }
    }
  };
  auto issue_tile = [&](const TM& tm, int j) {
    const uint32_t kst = lds_base + (j % Lay::NSK) * Lay::TILE_B;
    const uint32_t vst = lds_base + Lay::V_BASE + (j % Lay::NSV) * Lay::TILE_B;
    if (ragged) {
      issue_ragged(tm, j);
    } else if (tile_whole(tm)) {
#pragma unroll
      for (int ii = 0; ii < IPW; ++ii) issue_whole(tm, j, ii);
    } else {
#pragma unroll
      for (int ii = 0; ii < IPW; ++ii) {
        const int i = wave * IPW + ii;
        const int lc = (ii * Lay::KPI) >> 3;
        const int t = tm.tsrc[lc];
        const int key = i * Lay::KPI + lane / Lay::LPK;
        const int r = key & 7;
        const int pp = lane % Lay::LPK;
        const uint32_t row = (t + r < L) ? (uint32_t)(r * D * 2) : 0u;
        lds_dma16_s(p.k + tm.src[lc], row + (uint32_t)((pp ^ (key & 15)) * 16), kst, i * 1024);
        lds_dma16_s(p.v + tm.src[lc], row + (uint32_t)(v_unswz(key, pp) * 16), vst, i * 1024);
      }
    }
  };

  // ---------------- prologue: Q, then the first tiles in flight ----------------
  // (Q depends on no load, so it goes out while the tile descriptors are still
  // arriving; the first tile's copies wait for them.)
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
  constexpr int LA = Lay::LA;
  TM tmr[LA + 1];   // tmr[k] = tile j + k
#pragma unroll
  for (int k = 0; k <= LA; ++k) {
    tmr[k].M = 0;
    if (k < n_tiles) {
      tmr[k] = tile_meta(k);
      if (tmr[k].M && k < LA) issue_tile(tmr[k], k);
    }
  }
  // Q and every copy issued so far complete here, so no load issued before the
  // tile loop is pending inside it.
  wait_vmcnt<0>();

  // ---------------- per-lane LDS offsets ----------------
  // K (A operand of S^T): lane (ql, hh) reads key ql (+32 for the second block),
  // logical piece 2s + hh; pieces 16.. of a 256-dim row add 256 bytes.
  int koff[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) koff[s] = ql * Lay::ROWB + (((2 * s + hh) ^ (ql & 15)) * 16);
  // V (transpose reads): 16-lane group q16 covers dims 16*(q16&1) of a 32-dim
  // block for key half hq = q16>>1; lane 4r + c of the group reads key row
  // k0 + r, dims +4c..+4c+3, with k0 = 16s + 4hq (+8 for the second read).
  const int q16 = lane >> 4, li = lane & 15;
  const int v_r = li >> 2, v_c = li & 3;
  const int v_hq = q16 >> 1, v_dsub = q16 & 1;
  int voff[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int key = 4 * v_hq + v_r;
    voff[d] = key * Lay::ROWB + v_swz(key, 4 * d + 2 * v_dsub + (v_c >> 1)) * 16 + 8 * (v_c & 1);
  }

  // ---------------- accumulators ----------------
  f32x16 oacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[d][i] = 0.f;
  float m_run = -INFINITY;   // softmax reference, scale*log2(e) units (row max <= m_run + slack)
  float l_run = 0.f;
  const float sl2 = p.scale_log2;
  const int wl = p.window_left;
  const int myp4 = my_p - 4 * hh;        // causal: lane admits tile token tk + 4hh iff tk <= myp4
  const int myw4 = my_p - wl - 4 * hh;   // window: ... iff tk >= myw4
  const float neg_inf = -INFINITY;

  // ---------------- phases of one tile ----------------
  // K fragment of key block kb, k-step s from the K ring slot
  auto k_frag = [&](int slot, int kb, int s) -> bf16x8 {
    const unsigned char* sK = smem + slot * Lay::TILE_B;
    return *(const bf16x8*)(sK + koff[s & 7] + (s >> 3) * 256 + kb * 32 * Lay::ROWB);
  };
  // V^T fragment of dim block d, 16-key step s from the V ring slot
  auto v_frag = [&](int slot, int d, int s) -> bf16x8 {
    const unsigned char* a = smem + Lay::V_BASE + slot * Lay::TILE_B + voff[d & 3] + (d >> 2) * 256 +
                             16 * s * Lay::ROWB;
    const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(a));
    const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(a + 8 * Lay::ROWB));
    const u32x2 y0 = __builtin_bit_cast(u32x2, x0), y1 = __builtin_bit_cast(u32x2, x1);
    u32x4 w;
    w[0] = y0[0]; w[1] = y0[1]; w[2] = y1[0]; w[3] = y1[1];
    return as_bf16x8(w);
  };
  // S^T for the tile whose K sits in ring slot `slot`
  // (K fragments are read kKPre k-steps ahead of their MFMAs.)
  // When `cp` is set, the copies of whole tile cj go out one instruction per
  // k-step, in the shadow of the MFMAs (the slot they fill is not read here);
  // K and V copies on different k-steps, so an MFMA separates any two (two
  // copies in a row need a wait state between the first's read of M0 and the
  // second's write).
  auto compute_s = [&](int slot, f32x16 (&acc)[2], const TM* cp, int cj) {
    constexpr int kKPre = 4;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[kb][i] = 0.f;
    bf16x8 kr[kKPre][2];
#pragma unroll
    for (int s = 0; s < kKPre; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kr[s][kb] = k_frag(slot, kb, s);
    // the order written here is kept: the scheduler would otherwise sink
    // each read to just before its MFMA and expose the LDS latency
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[s % kKPre][kb], qf[s], acc[kb], 0, 0, 0);
      if (s + kKPre < NKS) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) kr[s % kKPre][kb] = k_frag(slot, kb, s + kKPre);
      }
      if (cp) {
        if constexpr (2 * IPW <= NKS) {
          // K copies on the first IPW k-steps, V copies on the next IPW
          if (s < IPW) issue_whole(*cp, cj, s, 1);
          else if (s < 2 * IPW) issue_whole(*cp, cj, s - IPW, 2);
        } else {
          constexpr int per = (IPW + NKS - 1) / NKS;
#pragma unroll
          for (int u = 0; u < per; ++u)
            if (s * per + u < IPW) issue_whole(*cp, cj, s * per + u);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // masks (element i of block kb is key 32kb + 8(i>>2) + 4hh + (i&3) of the tile)
  auto mask_s = [&](const TM& tm, f32x16 (&acc)[2]) {
    auto chunk_t = [&](int c) { return CONTIG ? tm.t0 + 8 * c : tm.ts[c]; };
    if (tm.M != ~0ull) {
      // Only the 8-key chunks with an excluded key are touched (a few invalid
      // keys leave most chunks whole).  Chunk c holds elements 4(c&3) .. +3 of
      // block c>>2; lanes 0-31 take chunk bit r, lanes 32-63 bit r + 4: a
      // scalar lane mask whose halves are those bits sign-extended.
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t cb = (uint32_t)(tm.M >> (8 * c)) & 0xFFu;
        if (cb != 0xFFu) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t lo = (uint32_t)((int32_t)(cb << (31 - r)) >> 31);
            const uint32_t hi = (uint32_t)((int32_t)(cb << (27 - r)) >> 31);
            acc[c >> 2][4 * (c & 3) + r] =
                select_lanes((uint64_t)lo | ((uint64_t)hi << 32), acc[c >> 2][4 * (c & 3) + r], neg_inf);
          }
        }
      }
    }
    if (p.causal && tm.tmax > wp_lo) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (chunk_t(4 * kb + (i >> 2)) + (i & 3) > myp4) acc[kb][i] = -INFINITY;
    }
    if (wl >= 0 && tm.tmin < wp_hi - wl) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (chunk_t(4 * kb + (i >> 2)) + (i & 3) < myw4) acc[kb][i] = -INFINITY;
    }
  };
  // Online softmax of one masked S^T tile: probabilities packed as bf16 (P^T
  // operands; lo = P - bf16(P) for fp32 output) and their sum.  The reference
  // only moves when the row max passes it by more than kRescaleSlack (log2
  // units), so P <= 2^kRescaleSlack and the rescale of O is rare; O / l does
  // not depend on the reference.
  float m_ref, m_use, psum;
  bf16x8 pb[4], pl[4];
  // probabilities of the tile against reference mu, and this lane's sum
  auto probs = [&](f32x16 (&acc)[2], float mu) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 w, wl4;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float e0 = fast_exp2(__builtin_fmaf(acc[s >> 1][8 * (s & 1) + 2 * t], sl2, -mu));
        const float e1 = fast_exp2(__builtin_fmaf(acc[s >> 1][8 * (s & 1) + 2 * t + 1], sl2, -mu));
        psum = (s == 0 && t == 0) ? e0 + e1 : psum + (e0 + e1);   // (no add of a zero start)
        w[t] = cvt_pk_bf16(e0, e1);
        if (F32)
          wl4[t] = cvt_pk_bf16(e0 - __uint_as_float(w[t] << 16), e1 - __uint_as_float(w[t] & 0xFFFF0000u));
      }
      pb[s] = as_bf16x8(w);
      if (F32) pl[s] = as_bf16x8(wl4);
    }
  };
  auto softmax = [&](f32x16 (&acc)[2]) {
    // Against the current reference first: when no lane's probabilities sum
    // past 2^kRescaleSlack, none of them passes it, the reference stays and
    // the row max is not needed.  (A NaN sum, from a row without a reference,
    // fails the test as well.)
    if (!__builtin_amdgcn_ballot_w64(m_run == -INFINITY)) {
      probs(acc, m_run);
      if (!__builtin_amdgcn_ballot_w64(!(psum <= kSlackPow))) {
        m_ref = m_use = m_run;
        return;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc[kb][i]);
    mx = half_max(mx);
    const float m_new = mx * sl2;
    m_ref = (m_new > m_run + kRescaleSlack) ? m_new : m_run;
    m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    probs(acc, m_use);
  };
  // move every row's softmax reference to m_ref
  auto rescale = [&]() {
    if (__builtin_amdgcn_ballot_w64(m_ref != m_run)) {
      const float alpha = fast_exp2(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
    }
    l_run += psum;
    m_run = m_ref;
  };
  // Dim blocks go in groups of four, key step outermost: the four MFMAs of one
  // step write four different accumulators, so none waits for the previous
  // one's result (a chain of dependent MFMAs runs the matrix pipe at about
  // two thirds of its rate).  The V fragments of the next step are read while
  // the current step's MFMAs run.
  auto compute_pv = [&](int slot) {
    constexpr int GD = NDB < 4 ? NDB : 4;   // dim blocks per group
    constexpr int NST = (NDB / GD) * 4;     // (group, key step) pairs
    bf16x8 va[2][GD];
#pragma unroll
    for (int d = 0; d < GD; ++d) va[0][d] = v_frag(slot, d, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int g = st >> 2, s = st & 3;
      if (st + 1 < NST) {
        const int g1 = (st + 1) >> 2, s1 = (st + 1) & 3;
#pragma unroll
        for (int d = 0; d < GD; ++d) va[(st + 1) & 1][d] = v_frag(slot, g1 * GD + d, s1);
      }
#pragma unroll
      for (int d = 0; d < GD; ++d)
        oacc[g * GD + d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[st & 1][d], pb[s], oacc[g * GD + d], 0, 0, 0);
      if (F32) {
#pragma unroll
        for (int d = 0; d < GD; ++d)
          oacc[g * GD + d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[st & 1][d], pl[s], oacc[g * GD + d], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---------------- tile loop ----------------
  // Iteration j: S_j, masks, softmax and O += V_j P_j.
  for (int j = 0; j < n_tiles; ++j) {
    wait_vmcnt<0>();     // tile j landed in this wave's share ...
    __syncthreads();     // ... and is visible; every wave is done with tile j-1
    // copies into the slots of tile j-1: a whole tile's go out during S
    const bool run = wave_rows && tmr[0].M;
    const bool in_s = run && tmr[LA].M && !ragged && tile_whole(tmr[LA]);
    if (tmr[LA].M && !in_s) issue_tile(tmr[LA], j + LA);
    if (run) {
      // The SIMD's other wave belongs to another workgroup and is usually in a
      // different phase: raising this wave's priority while it issues MFMAs
      // keeps the matrix pipe fed while the other one runs its softmax.
      f32x16 sc[2];
      __builtin_amdgcn_s_setprio(1);
      if (in_s) compute_s(j % Lay::NSK, sc, &tmr[LA], j + LA);
      else compute_s(j % Lay::NSK, sc, nullptr, 0);
      __builtin_amdgcn_s_setprio(0);
      mask_s(tmr[0], sc);
      softmax(sc);
      rescale();
      __builtin_amdgcn_s_setprio(1);
      compute_pv(j % Lay::NSV);
      __builtin_amdgcn_s_setprio(0);
    }
#pragma unroll
    for (int k = 0; k < LA; ++k) tmr[k] = tmr[k + 1];
    // metadata of the tile copied next iteration: its scalar loads overlap the
    // MFMAs still in flight
    tmr[LA].M = 0;
    if (j + 1 + LA < n_tiles) tmr[LA] = tile_meta(j + 1 + LA);
  }

  // ---------------- epilogue ----------------
  if (!wave_rows) return;
  const float l_tot = half_sum(l_run);
  if (!row_ok) return;
  if (partial_out) {
    // Split-KV decode: this split's unnormalised partial (O, m, l); a separate
    // merge kernel combines the splits.
    float* dst = p.part + ((((int64_t)b * p.maxq + my_i) * p.Hq + my_hq) * p.num_splits + split) * (D + 4);
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
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : p.out_scale / l_tot;
  const int64_t orow = ((int64_t)(tok_base + my_i) * p.Hq + my_hq);
  if (F32) {
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
    // dims 32d + 16k .. +15 of a row are split over lanes l (hh = 0) and l + 32;
    // one swap across the half-waves gives each lane 16 contiguous bytes
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        uint32_t x[2], y[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          x[e] = cvt_pk_bf16(oacc[d][8 * k2 + 2 * e] * inv, oacc[d][8 * k2 + 2 * e + 1] * inv);
          y[e] = cvt_pk_bf16(oacc[d][8 * k2 + 4 + 2 * e] * inv, oacc[d][8 * k2 + 4 + 2 * e + 1] * inv);
        }
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          // The swap exchanges x of lanes 32-63 with y of lanes 0-31.  Afterwards
          // lanes 0-31 hold their own g4 = 2k2 data then the partner's, and lanes
          // 32-63 the partner's g4 = 2k2 + 1 data then their own: in every lane
          // the two results are the row's 16 bytes in order, with no select.
          const auto r = __builtin_amdgcn_permlane32_swap(x[e], y[e], false, false);
          w[e] = r[0];
          w[2 + e] = r[1];
        }
        *(u32x4*)(o + 32 * d + 16 * k2 + 8 * hh) = w;
      }
  }
  if (p.lse && hh == 0)
    p.lse[orow] = empty ? -INFINITY : (m_run + __log2f(l_tot)) * kLn2;
}

// Launch of one instantiation (the LDS limit raised once per function and device).
template <int D, int NW, int MODE, bool RAGGED>
static hipError_t launch_one(const AttnParams& p, dim3 grid, hipStream_t st) {
  const size_t lds = AttnLayout<D, NW>::LDS;
  const void* kern = p.out_f32 ? (const void*)attn_fwd_kernel<D, NW, MODE, true, true, RAGGED>
                               : (const void*)attn_fwd_kernel<D, NW, MODE, false, true, RAGGED>;
  int variant = p.out_f32 ? 1 : 0;
  if constexpr (MODE == kModeBsa) {
    if (p.kvbs % 64 != 0) {   // sparse blocks of 8, 16 or 32 keys: several per tile
      kern = p.out_f32 ? (const void*)attn_fwd_kernel<D, NW, MODE, true, false, RAGGED>
                       : (const void*)attn_fwd_kernel<D, NW, MODE, false, false, RAGGED>;
      variant += 2;
    }
  }
  if (lds > 65536) {
    // The LDS limit is an attribute of the function on one device: raise it on
    // the first launch there only, so later launches (and graph capture) make
    // no extra runtime calls.
    static std::atomic<uint64_t> raised[4];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev < 64 ? (1ull << dev) : 0;
    if (!(raised[variant].load(std::memory_order_acquire) & bit)) {
      e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      raised[variant].fetch_or(bit, std::memory_order_release);
    }
  }
  AttnParams arg = p;
  void* args[] = {(void*)&arg};
  return hipLaunchKernel(kern, grid, dim3(NW * 64), args, lds, st);
}

}  // namespace pkb

#endif  // PKB_ATTN_FWD_KERNEL_H_
