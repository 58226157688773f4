/*
 * ix_peaks.h -- measured ceilings for the roofline fractions (libix_peaks.so, gfx950).
 *
 * Not part of the method and not in the path's library: microbenchmark kernels that say
 * what the chip delivers on the shapes of work the path is made of, so each kernel's time
 * can be read against a measured ceiling as well as the datasheet peak.  The caller times
 * a call with events on `stream`; every buffer is device memory owned by the caller,
 * nothing is allocated.  Statuses are those of ix.h; the message of the last non-OK status
 * on the calling thread is ix_peak_last_error().
 */
#ifndef IX_PEAKS_H
#define IX_PEAKS_H

#include "ix.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Message for the last non-OK status of an ix_peak_* call on this thread ("" if none). */
const char *ix_peak_last_error(void);

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

/* ix_peak_read -- reads src[0, bytes) once with 16-byte loads, four in flight per lane, over
 * `blocks` blocks of 256 threads (a read-only stream, as the decode indexer streams its keys;
 * the best grid depends on the machine, so the caller sweeps it).  nontemporal = 1 marks the
 * loads non-temporal (the faster stream; the data does not stay in the caches), 0 makes them
 * ordinary loads, which fill the caches (reading a buffer larger than the caches this way
 * evicts what they held).  out: uint32 [blocks], entry i written with the XOR of the 32-bit
 * words block i read (the XOR of all entries is the XOR of the bytes).  bytes: a multiple of
 * 16; src 16-byte aligned.  Errors: IX_ERR_INVALID for NULL pointers, misalignment, blocks
 * outside 1..65536 or nontemporal outside {0, 1}. */
ix_status ix_peak_read(const void *src, size_t bytes, int32_t blocks, int32_t nontemporal,
                       uint32_t *out, hipStream_t stream);

/*
 * ix_peak_gather -- reads the 256-byte rows table[rows[i]], i < n, each by 16
 * consecutive lanes with 16-byte loads, 8 loads in flight per lane, over
 * `blocks` blocks of 256 threads.
 * table_bytes: <= 2 GiB, a multiple of 256; rows outside the table read as zero.
 * out: uint32 [blocks], entry i written with the XOR of the words block i read.
 * Errors: IX_ERR_INVALID for NULL pointers, n < 0, a bad table size or alignment, or blocks
 * outside 1..65536.
 */
ix_status ix_peak_gather(const void *table, size_t table_bytes, const int32_t *rows, int64_t n,
                         int32_t blocks, uint32_t *out, hipStream_t stream);

/*
 * ix_peak_gather_wide -- ix_peak_gather over a table of n_seg segments of seg_bytes each
 * (a footprint of up to 64 GiB): load step i of wave w (8 rows per lane group) reads the rows
 * rows[r], counted within segment (w + i) mod n_seg.  seg_bytes: <= 1 GiB, a multiple of 256;
 * rows outside a segment read as zero.  n_seg: 1..64.  nontemporal = 1 marks the loads
 * non-temporal (as the decode attention's row loads), 0 makes them ordinary loads.
 * out: as for ix_peak_gather.
 * Errors: IX_ERR_INVALID for NULL pointers, n < 0, a bad segment size, count or alignment,
 * blocks outside 1..65536 or nontemporal outside {0, 1}.
 */
ix_status ix_peak_gather_wide(const void *table, size_t seg_bytes, int32_t n_seg,
                              const int32_t *rows, int64_t n, int32_t blocks, int32_t nontemporal,
                              uint32_t *out, hipStream_t stream);

/*
 * ix_peak_gather_selection -- reads, for every query and KV head, the K and V rows its
 * selection names, exactly as sparse_attn_fwd gathers them (one block of 4 waves per query,
 * KV head and split, 32-entry chunks, two chunks in flight per wave, the same block order),
 * and computes nothing with them: the memory system's rate for the attention's own access
 * pattern (the main kernel's, taken for 1024 query rows or more).  kc, vc, idx, kv_len, B, T, S_max, H_kv, d, k: as for sparse_attn_fwd (entries
 * < 0 or >= kv_len read nothing).  splits: blocks per (query, KV head), each taking a
 * contiguous share of the selection's chunks.  blocks_per_cu: 0, or 2 or 3 to hold the
 * launch to that many resident blocks per CU (through unused LDS), as the attention's LDS
 * holds it to 2.  out: uint32 [B * T * H_kv * splits], entry i
 * written with the XOR of the words block i read (each row read once per selection entry).
 * Errors: IX_ERR_INVALID for NULL pointers, sizes out of range or misaligned caches;
 * IX_ERR_UNSUPPORTED for d outside {64, 128} or a grid too large for one launch.
 */
ix_status ix_peak_gather_selection(const void *kc, const void *vc, const int32_t *idx,
                                   const int32_t *kv_len, int32_t B, int32_t T, int32_t S_max,
                                   int32_t H_kv, int32_t d, int32_t k, int32_t splits,
                                   int32_t blocks_per_cu, uint32_t *out, hipStream_t stream);

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
