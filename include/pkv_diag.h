/*
 * pkv_diag.h - measurement aids of libpkv: the read rate the device reaches
 * on a plain stream of bytes, the practical ceiling beside the HBM peak for
 * the bandwidth-bound decode kernels (which read their K/V rows with the
 * same 16-byte non-temporal loads), and the rate its bf16 matrix cores
 * reach on the MFMA instruction the prefill and the fused QKV projection
 * use, the practical ceiling beside the dense bf16 peak.
 *
 * Conventions (device pointers owned by the caller, streams, status codes)
 * are those of pkv.h.
 */
#ifndef PKV_DIAG_H
#define PKV_DIAG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroups of one pkv_read_probe launch; its sink holds one 16-byte slot each. */
#define PKV_READ_PROBE_WORKGROUPS 8192

/*
 * read_probe: read every byte of `data` once (16-byte non-temporal loads,
 * each workgroup instruction covering 4 KiB of consecutive bytes, the next
 * eight loads per lane issued before the current eight are folded) and fold
 * them with XOR; a workgroup writes its 16-byte slot of `sink` only when its
 * fold equals an arbitrary constant, so `sink` is practically never written
 * and the call moves `bytes` of reads and nothing else.
 *
 *   data        device buffer of `bytes` bytes, 16-byte aligned, bytes a
 *               positive multiple of 16
 *   sink        device buffer of sink_bytes >= 16 * PKV_READ_PROBE_WORKGROUPS
 *               bytes, 16-byte aligned; its contents are unspecified after
 *               the call
 *
 * Errors: PKV_ERR_NULL_POINTER, PKV_ERR_MISALIGNED, PKV_ERR_BAD_SHAPE
 * (bytes), PKV_ERR_WORKSPACE (sink too small), PKV_ERR_HIP.
 */
int32_t pkv_read_probe(const void* data, size_t bytes, void* sink, size_t sink_bytes, void* stream);

/* Workgroups (of 256 threads: 4 waves) of one pkv_mfma_probe launch, and its
 * largest iteration count. */
#define PKV_MFMA_PROBE_WORKGROUPS 512
#define PKV_MFMA_PROBE_MAX_ITERS (1 << 20)

/*
 * mfma_probe: every wave of PKV_MFMA_PROBE_WORKGROUPS x 4 runs `iters`
 * rounds of 8 v_mfma_f32_32x32x16_bf16 (two independent accumulator chains
 * on register operands; 2 x 32 x 32 x 16 = 32768 flop each), so a launch
 * performs PKV_MFMA_PROBE_WORKGROUPS x 4 x 8 x iters x 32768 flop and reads
 * no memory.  The operands are fixed hashed bit patterns (finite, |x| < 2).
 * A lane would write its 4-byte slot of `sink` only if its (finite) fold of
 * the results had a NaN's bit pattern, so `sink` is never written.
 *
 *   iters       1 .. PKV_MFMA_PROBE_MAX_ITERS
 *   sink        device buffer of sink_bytes >= 4 * 256 *
 *               PKV_MFMA_PROBE_WORKGROUPS bytes, 4-byte aligned; its contents
 *               are unspecified after the call
 *
 * Errors: PKV_ERR_NULL_POINTER, PKV_ERR_MISALIGNED, PKV_ERR_BAD_SHAPE
 * (iters), PKV_ERR_WORKSPACE (sink too small), PKV_ERR_HIP.
 */
int32_t pkv_mfma_probe(int32_t iters, void* sink, size_t sink_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_DIAG_H */
