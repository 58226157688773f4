/*
 * ix_peaks.h -- measured ceilings for the roofline fractions of libix.so (gfx950).
 *
 * Not part of the method: three microbenchmark kernels that say what the chip delivers
 * on the shapes of work the path is made of, so each kernel's time can be read against
 * a measured ceiling as well as the datasheet peak.  The caller times a call with events
 * on `stream`; every buffer is device memory owned by the caller, nothing is allocated,
 * and the statuses and ix_last_error() are those of ix.h.
 */
#ifndef IX_PEAKS_H
#define IX_PEAKS_H

#include "ix.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * ix_peak_mfma_fp8 -- blocks x 4 waves, each wave issuing 16 * iters FP8 MFMAs
 * (v_mfma_f32_16x16x128_f8f6f4, 65,536 flop each) against 16 register-resident B
 * operands, followed by valu_per_mfma fp32 VALU ops per MFMA (0, 4, 8 or 12; the
 * indexer's epilogue is 8: an integer max and an FMA per output element).
 * operands: >= 34 * 64 * 32 bytes of e4m3 codes (any finite codes).
 * out:      one float, ADDED TO (a checksum that keeps the work live).
 * Errors: IX_ERR_INVALID for NULL pointers, blocks < 1, iters < 1 or another
 * valu_per_mfma.
 */
ix_status ix_peak_mfma_fp8(const void *operands, int32_t valu_per_mfma, int32_t blocks,
                           int32_t iters, float *out, hipStream_t stream);

/* ix_peak_copy -- dst[0, bytes) = src[0, bytes) with 16-byte loads and stores.
 * bytes: a multiple of 16; src and dst 16-byte aligned, not overlapping. */
ix_status ix_peak_copy(const void *src, void *dst, size_t bytes, hipStream_t stream);

/*
 * ix_peak_gather -- reads the 256-byte rows table[rows[i]], i < n, each by 16
 * consecutive lanes with 16-byte loads, 16 loads in flight per lane.
 * table_bytes: <= 2 GiB, a multiple of 256; rows outside the table read as zero.
 * out: one uint32, XORed with a checksum of the bytes read.
 */
ix_status ix_peak_gather(const void *table, size_t table_bytes, const int32_t *rows, int64_t n,
                         uint32_t *out, hipStream_t stream);

/*
 * ix_peak_atomic_add -- for each i < n, adds 1.0f with fp32 atomics to all 128 floats of
 * row idx[i] of table (rows with idx outside [0, rows) are skipped): one row per wave,
 * lanes adding to consecutive floats, as the attention backward accumulates dK and dV.
 * table: fp32 [rows, 128], ADDED TO; rows <= 2^24.
 */
ix_status ix_peak_atomic_add(float *table, int64_t rows, const int32_t *idx, int64_t n,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* IX_PEAKS_H */
