/*
 * pkb_peaks.h -- C ABI of libpkb_peaks.so: on-device ceilings of an MI355X
 * (gfx950) used as measured roofline denominators next to the published ones.
 * Measurement code only; nothing here is part of the attention path.
 *
 * Every function enqueues one kernel on `stream` (a hipStream_t passed as
 * void*; NULL = the default stream) and returns 0, or a negative HIP error
 * code when the arguments are out of range or the launch fails.  Buffers are
 * caller-owned device memory; the kernels only read them, apart from `sink`
 * (at least 16 bytes), which receives a value only when a checksum hits a
 * fixed constant (it exists so that no load or MFMA can be removed).
 * `grid` is the number of 256-thread workgroups.
 */
#ifndef PKB_PEAKS_H_
#define PKB_PEAKS_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` (a multiple of 4096) from `buf`: every byte once;
 * consecutive waves read consecutive 4 KiB chunks, each wave keeping four
 * chunks (16 loads of 16 bytes per lane) in flight.  `nontemporal` 1 marks
 * the loads non-temporal (the nt cache policy), 0 leaves them plain; any other
 * value is rejected. */
int pkb_peak_hbm_read(const void* buf, int64_t bytes, void* sink, int32_t grid, int32_t nontemporal,
                      void* stream);

/* Gather of `n_reads` slabs of 4096 bytes at pseudo-random slab indices of
 * `buf` (`bytes` a multiple of 4096, at least one slab): the access shape of
 * paged decode (one 16-token page of one KV head at D = 128).  Each wave keeps
 * four slabs in flight; n_reads is rounded up to whole wave iterations
 * (returned bytes = 4096 * reads actually made, written to *bytes_read).
 * `nontemporal` as for pkb_peak_hbm_read. */
int pkb_peak_hbm_gather(const void* buf, int64_t bytes, int64_t n_reads, void* sink,
                        int32_t grid, int32_t nontemporal, int64_t* bytes_read, void* stream);

/* Gather of 512-byte rows at pseudo-random row indices of a buffer small
 * enough to stay in each XCD's 4 MB L2 (`bytes` a multiple of 512, at most
 * 4 MiB): the access shape of the packed-query sparse kernel (one K or V row
 * of 256 bf16).  Reads `n_reads` rows in total (rounded up as above). */
int pkb_peak_l2_gather(const void* buf, int64_t bytes, int64_t n_reads, void* sink,
                       int32_t grid, int64_t* bytes_read, void* stream);

/* Dense MFMA loop: every wave issues `iters` rounds of 8 independent
 * accumulations.  kind 0: v_mfma_f32_32x32x16_bf16 (32768 flop each);
 * 1: v_mfma_i32_32x32x32_i8 (65536 op); 2: v_mfma_f32_32x32x64_f8f6f4 with
 * fp8 E4M3 operands (131072 op).  Total operations = grid * 4 waves * iters *
 * 8 * (operations per instruction). */
int pkb_peak_mfma(int32_t kind, int32_t iters, void* sink, int32_t grid, void* stream);

/* Instruction-issue probe (512-thread workgroups holding 96 KB of LDS each, so
 * one per CU; grid = number of CUs): in each
 * workgroup the first `waves` waves (4 = one per SIMD, 8 = two per SIMD) run
 * `iters` rounds of 8 independent instructions of one kind -- 0: v_fma_f32
 * with three VGPR sources, 1: v_exp_f32, 2: v_add_f32 each followed by an
 * independent s_add_u32 -- and the rest exit.  SIMD cycles per instruction =
 * duration x clock / (iters x 8 x waves / 4). */
int pkb_peak_issue(int32_t kind, int32_t iters, int32_t waves, void* sink, int32_t grid,
                   void* stream);

/* MFMA / VALU co-execution probe (512-thread workgroups, one per CU as above): waves
 * 0-3 run iters_m rounds of 4 independent v_mfma_f32_32x32x16_bf16 (mode 0
 * and 2), waves 4-7 -- on the same four SIMDs -- iters_v rounds of 8
 * independent v_fma_f32 (mode 1 and 2).  Mode 2's duration against modes 0
 * and 1 shows how far the two overlap. */
int pkb_peak_coexec(int32_t mode, int32_t iters_m, int32_t iters_v, void* sink, int32_t grid,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKB_PEAKS_H_ */
