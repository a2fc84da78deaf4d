/*
 * hbm_probe.h -- streaming kernels that measure what HBM delivers on this device, the ceilings
 * the norm kernels are compared against, and matrix-core and LDS read probes for the bf16
 * products.
 *
 * The norm passes are streams: the forward reads one [M, N] tensor and writes one, the fused
 * backward reads two and writes one, the residual forward reads two and writes two. The share
 * of the theoretical bandwidth that such sequential access actually reaches depends on the mix
 * of reads and writes and on how many requests are in flight (web page "Otimização de
 * Performance de GPU: Maximizando Throughput para Treinamento e Inferência de LLM", section
 * "Gargalos de largura de banda de memória limitam a performance de LLM"). Each probe moves
 * nin input streams and nout output streams of `bytes` each, 16 bytes per access, and does no
 * arithmetic beyond an XOR: its rate is the ceiling for a kernel with that stream mix.
 *
 * Not part of the norm library's boundary (libnorm.so); built into libhbmprobe.so.
 */
#ifndef DLN_HBM_PROBE_H
#define DLN_HBM_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Queue one probe on `stream` (a hipStream_t; NULL = the null stream).
 *   nin, nout   input and output streams: (1, 0) read, (0, 1) write, (1, 1) copy, (2, 1) triad
 *               (two reads, one write), (2, 2) two reads and two writes. Others: -1.
 *   in0, in1    device inputs of `bytes` each (in1 only when nin == 2).
 *   out0, out1  device outputs of `bytes` each (out1 only when nout == 2). For the read probe
 *               out0 is a 16-byte sink written only if the XOR of everything read equals `key`
 *               (so the loads cannot be dropped); the write probe stores `key` patterns.
 *   bytes       multiple of 16, > 0; every pointer 16-byte aligned; buffers must not overlap.
 *   unroll      16-byte accesses per thread and stream in flight at once: 1, 2, 4 or 8.
 *   nt_loads    1: loads marked nontemporal; 0: ordinary loads. Stores are always nontemporal.
 *   grid        workgroups (256 threads): 0 = one per tile of 256 * unroll accesses (every
 *               workgroup short-lived), else a grid-stride loop over the tiles.
 *   start_event, stop_event: NULL, or two hipEvent_t that take the kernel's own start and end
 *               timestamps (both or neither).
 * Returns 0 once queued, -1 for invalid arguments, -2 if the launch failed.
 */
int hbm_probe(int nin, int nout, const void *in0, const void *in1, void *out0, void *out1,
              size_t bytes, int unroll, int nt_loads, int64_t grid, uint32_t key,
              void *start_event, void *stop_event, void *stream);

/*
 * Queue the matrix-core probe on `stream`: `grid` workgroups of 64 * 4 * waves_per_simd threads
 * (one or two wavefronts per SIMD), each wavefront running `iters` rounds of eight independent
 * bf16 matrix operations (fp32 accumulation) on register operands, with no memory traffic
 * beyond one float per thread written to out [grid * 64 * 4 * waves_per_simd] at the end. Its
 * rate is the ceiling for the bf16 products (the attention kernel, the projection product):
 *   shape   32: v_mfma_f32_32x32x16_bf16 (32768 flops per operation); 16:
 *           v_mfma_f32_16x16x32_bf16 (16384 flops).
 *   start_event, stop_event: NULL, or two hipEvent_t that take the kernel's timestamps.
 * Returns 0 once queued, -1 for invalid arguments, -2 if the launch failed.
 */
int mfma_probe(int shape, int waves_per_simd, int64_t grid, int iters, float *out,
               void *start_event, void *stop_event, void *stream);

/*
 * Queue the LDS read probe on `stream`: `grid` workgroups of 256 * waves_per_simd threads (1, 2
 * or 4 wavefronts per SIMD), each with a 64 KB LDS buffer; every thread makes `iters` x 8
 * reads of 16 bytes, each wavefront read one contiguous KB (conflict-free), and writes the XOR
 * of what it read to out [grid * 256 * waves_per_simd]. Bytes read per launch:
 * grid * 256 * waves_per_simd * iters * 8 * 16. Returns 0 once queued, -1 for invalid
 * arguments, -2 if the launch failed.
 */
int lds_probe(int waves_per_simd, int64_t grid, int iters, unsigned *out, void *start_event,
              void *stop_event, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DLN_HBM_PROBE_H */
