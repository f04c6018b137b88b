/* mmq_peak.h -- measured ceilings: matrix-core rates and a read-only HBM
 * stream (libmmq_peak.so).
 *
 * A measurement aid for the benchmark's roofline, separate from the matmul
 * library: it runs the two 32x32 MFMA instructions a q8 matmul on gfx950 can
 * use (f16 32x32x16, on integer-valued operands, and int8 32x32x32) back to
 * back, so the achieved rate of the matmul can be set against what the
 * matrix pipe delivers on this device at its clock under load, beside the
 * published peaks.
 *
 * Each launch runs `blocks` workgroups of 256 threads (4 waves); every wave
 * issues `iters` rounds of mmq_peak_chains() independent MFMAs on register
 * operands and writes one value per thread to `out`, so a launch performs
 *   blocks * 4 * iters * mmq_peak_chains() * (2*32*32*16)   f16 operations, or
 *   blocks * 4 * iters * mmq_peak_chains() * (2*32*32*32)   int8 operations.
 * Time the launch with events on `stream`.
 *
 * Arguments: `out` is a caller-owned device buffer of blocks * 256 elements
 * (float for f16, int32 for int8; its contents are meaningless); blocks >= 1,
 * 1 <= iters <= 2^20; `stream` is the caller's HIP stream (0 for the null
 * stream).  Returns 0 on success, -1 for an invalid argument (nothing is
 * launched), or the HIP error code of the launch.
 */
#ifndef MMQ_PEAK_H
#define MMQ_PEAK_H

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int mmq_peak_chains(void);
int mmq_peak_mfma_f16(float* out, int blocks, int iters, hipStream_t stream);
int mmq_peak_mfma_i8(int* out, int blocks, int iters, hipStream_t stream);

/* The matmul's per-block instruction mix with no memory traffic, in its
 * launch shape (workgroups of 512 threads, 2 waves per SIMD): per 32-block
 * each wave issues 4 f16 32x32x16 MFMAs (two output tiles, two K-steps) and
 * the 32 FMAs of the previous block's rescale (a per-lane factor, so each
 * FMA reads three VGPRs).  mode 0 issues the MFMAs only,
 * 1 the FMAs only, 2 both in the matmul's order; comparing the three times
 * shows how far the matrix pipe and the VALU overlap on this device.  mode 3
 * runs the same per-block work on int8 MFMA: 2 v_mfma_i32_32x32x32_i8 per
 * block and wave and 3 VALU operations per output (convert, weight scale,
 * token-scale FMA).  A launch runs blocks * 8 * iters * 2 blocks of that mix:
 * mode 0, 2 and 3 perform blocks * 8 * iters * 8 * (2*32*32*16) operations.  out: caller-owned
 * device buffer of blocks * 512 floats; blocks >= 1, 1 <= iters <= 2^20.
 * Returns 0, -1 for an invalid argument (nothing launched), or the HIP error
 * code of the launch. */
int mmq_peak_mix(float* out, int blocks, int iters, int mode, hipStream_t stream);

/* Overlap probes: variants of the per-block mix above that show what lets the
 * matrix pipe and the VALU run at the same time.  Each probe is one kernel;
 * per 32-block every wave issues, per output tile, 2 f16 32x32x16 MFMAs and
 * 16 rescale FMAs, or only one of the two kinds, or (split probes) one wave
 * of each SIMD pair issues only the MFMAs and the other only the FMAs; the
 * FMAs read the previous block's MFMA results or registers no MFMA writes.
 * Each FMA reads three VGPRs (the rescale factor differs per lane, as the
 * matmul's token scale does).  Probes named r... run on random f16 operands
 * that change from block to block, as real data does (iters rounded up to
 * even); the others on small constant operands.
 * mmq_peak_probe_count() gives the number of probes; mmq_peak_probe_info(i,
 * ...) its name, threads per workgroup, output tiles per wave and MFMA-issuing
 * waves per workgroup (0..count-1, else -1); mmq_peak_probe(i, out, blocks,
 * iters, stream) launches probe i with `blocks` workgroups (one per CU gives
 * threads/256 waves per SIMD) running `iters` rounds of 2 blocks, writing
 * blocks * threads floats to the caller's device buffer `out`.  A launch
 * performs blocks * mfma_waves * iters * 2 * tiles * 2 * (2*32*32*16) f16
 * operations.  Returns 0, -1 for an invalid argument (nothing launched), or
 * the HIP error code of the launch. */
int mmq_peak_probe_count(void);
int mmq_peak_probe_info(int i, const char** name, int* threads, int* tiles, int* mfma_waves);
int mmq_peak_probe(int i, float* out, int blocks, int iters, hipStream_t stream);

/* Read-only HBM stream: reads `bytes` (a multiple of 16, > 0) of the device
 * buffer `src` once with 16-byte non-temporal loads, `blocks` workgroups of
 * 256 threads walking it grid-stride with `unroll` (4, 8 or 16) loads in
 * flight per thread, and writes one folded value per thread to `out`
 * (blocks * 256 uint32, caller-owned).  Time it with events on `stream`;
 * the best of a few (blocks, unroll) shapes is the chip's practical read
 * rate.  Returns 0, -1 for an invalid argument (nothing launched), or the
 * HIP error code of the launch. */
int mmq_peak_read(const void* src, int64_t bytes, unsigned* out, int blocks, int unroll,
                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MMQ_PEAK_H */
