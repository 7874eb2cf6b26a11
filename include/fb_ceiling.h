/*
 * fb_ceiling.h — measured ceilings of the GPU the attention library runs on.
 *
 * Plain kernels, in a library of their own (libfb_ceiling.so), that measure what this chip
 * reaches on the two resources the attention kernels are bound by, and how far one wave's
 * matrix work and another wave's vector work overlap on a SIMD.  A measurement helper: no
 * attention work runs here.
 *   - a streaming read of a device buffer (the HBM read rate a kernel can reach), for the
 *     prefix pass, whose roofline is HBM (the cached K/V is read once per fresh step:
 *     "Resumo Técnico: FlashBlock", §2 Mecanismo Central);
 *   - a loop of independent bf16 matrix FMAs (v_mfma_f32_32x32x16_bf16) with no memory
 *     traffic, for the long-block pass whose roofline is the matrix units.
 * Both run under the same power and clock limits as the attention kernels, so their rates
 * sit beside the published peaks (8 TB/s HBM, 2.5 PFLOP/s dense bf16) as the achievable
 * ones.  Each writes a result the caller can check exactly, so a reported rate comes from
 * work that was really done.
 *
 * Conventions: the caller allocates every buffer in device memory; the library allocates
 * nothing and keeps no state.  Work is enqueued on `stream`; nothing synchronises the host.
 * Arguments are checked on the host before any launch: an invalid argument returns 1 and
 * launches nothing, a failed launch returns 5, success returns 0 (the numbering of
 * fb_status in flashblock.h).
 */
#ifndef FB_CEILING_H
#define FB_CEILING_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of `buf` once, 16 bytes per load, with `workgroups` workgroups of 256
 * threads striding over the buffer.  Workgroup w writes to sink[16 w .. 16 w + 15] the
 * bitwise XOR of the 16-byte words it read, so the XOR of all `workgroups` sink entries is
 * the XOR of every 16-byte word of the buffer.
 *   buf         device, 16-byte aligned, `bytes` bytes (bytes > 0, bytes % 16 == 0)
 *   workgroups  1 .. 65536
 *   nontemporal 0: plain loads; 1: loads with the non-temporal hint, as the streaming
 *               attention pass issues its K/V loads
 *   sink        device, 16 * workgroups bytes, written
 */
int fbc_stream_read(const void* buf, int64_t bytes, int32_t workgroups, int32_t nontemporal, void* sink,
                    hipStream_t stream);

/* Run `iters` rounds of 4 independent v_mfma_f32_32x32x16_bf16 per wave on register
 * operands: `workgroups` workgroups of 4 waves, every element of A set to bf16(a) and of B
 * to bf16(b).  Work done: workgroups * 4 * iters * 4 * 32768 flops (2 per multiply-add).
 * Wave j of workgroup w writes to sink[4 w + j] the sum over its 4 accumulators of one
 * output element, which is exactly 4 * 16 * iters * bf16(a) * bf16(b) when that value and
 * every partial sum are exact in fp32 (for a = b = 1: iters <= 262144).
 *   workgroups 1 .. 65536; iters 1 .. 262144
 *   sink       device, 4 * workgroups floats, written
 */
int fbc_mfma_loop(int32_t workgroups, int64_t iters, float a, float b, float* sink, hipStream_t stream);

/* Matrix and vector work side by side on one SIMD.  `workgroups` workgroups; a round is 8
 * v_mfma_f32_32x32x16_bf16 (two on each of 4 accumulators) for a wave of the MFMA stream,
 * and 8 * valu_per_mfma vector operations (half v_exp_f32, half v_fma_f32, on 8
 * independent chains) for a wave of the vector stream.
 *   mode 0: 4 waves per workgroup, each the MFMA stream (valu_per_mfma ignored, may be 0)
 *   mode 1: 4 waves per workgroup, each the vector stream
 *   mode 2: 8 waves per workgroup; waves 0-3 the MFMA stream, waves 4-7 the vector stream
 *           (waves w and w + 4 share a SIMD)
 *   mode 3: 4 waves per workgroup, each interleaving the two (valu_per_mfma operations after
 *           every MFMA)
 * The launch time of mode 2 against modes 0 and 1 says how far the two overlap: the maximum
 * of the two when they overlap fully, their sum when they do not.
 *   valu_per_mfma 2, 4 or 8 (0 allowed for mode 0); rounds 1 .. 262144
 *   one          pass 1.0: the operands are built from it at run time, so nothing is folded
 *   sink         device, 8 * workgroups floats; the entry of wave j of workgroup w,
 *                sink[8 w + j], is written for every wave the mode runs: 128 * rounds for a
 *                wave that ran the MFMA stream (each vector chain ends at exactly 0), 0 for a
 *                wave that ran only the vector stream
 * Flops of the MFMA stream: waves_with_mfma * rounds * 8 * 32768.
 */
int fbc_mfma_valu(int32_t mode, int32_t valu_per_mfma, int32_t workgroups, int64_t rounds, float one, float* sink,
                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FB_CEILING_H */
