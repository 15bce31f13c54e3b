/* Hardware probes for MI355X (gfx950): measurement aids behind the rates the
 * design quotes (LDS read throughput, instruction issue rates, wave placement,
 * global atomic throughput, v_exp_f32 accuracy, HBM read rate).  Not part of the attention
 * ABI in attn.h; libattn.so exports them beside it.
 *
 * Common rules: every pointer is a device pointer owned by the caller, sized as
 * stated; each call launches one kernel on `stream` (0 = the null stream) and
 * returns at once.  Return codes: 0 launched; 1 an argument is out of range
 * (nothing launched); 2 the launch failed (hipGetLastError). */
#ifndef ATTN_PROBE_H
#define ATTN_PROBE_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* LDS read throughput.  `workgroups` workgroups of 256 threads each fill a
 * 32 KiB LDS array and then read it 2048 x 8 times per thread: mode 0 with
 * 16-byte reads (ds_read_b128), mode 1 with 8-byte transposing reads
 * (ds_read_b64_tr_b16).  cycles[workgroups] receives each workgroup's
 * s_memtime cycle count for the read loop; sink[workgroups * 256] a value per
 * thread that keeps the reads alive.  Bytes read per workgroup:
 * 256 * 2048 * 8 * (16 or 8). */
int attn_probe_lds_rate(int mode, int workgroups, unsigned* sink, unsigned long long* cycles, hipStream_t stream);

/* Instruction issue rates.  Workgroups of `waves` (1..8) waves; wave w runs
 * kinds[w] (device int array of `waves` entries): 0 nothing, 1 8 x 4096
 * v_exp_f32, 2 8 x 4096 v_fma_f32, 3 4096 v_mfma_f32_32x32x16_bf16 in four
 * independent accumulator chains.  cycles[workgroups * 8] receives each wave's
 * s_memtime cycle count (index workgroup * 8 + wave); sink[workgroups * 64 *
 * waves] keeps the results alive.  Waves w and w + 4 of one workgroup share a
 * SIMD (attn_probe_wave_simd shows it). */
int attn_probe_issue(const int* kinds, int waves, int workgroups, float* sink, unsigned long long* cycles,
                     hipStream_t stream);

/* Wave placement: `workgroups` workgroups of 8 waves; hwid[workgroups * 8]
 * receives each wave's HW_ID register (SIMD in bits 5:4, CU in bits 11:8). */
int attn_probe_wave_simd(int workgroups, unsigned* hwid, hipStream_t stream);

/* Global fp32 update throughput over target[n] (n a multiple of 16384): every
 * element gets +1.0 once, with atomicAdd (atomic != 0) or a plain load, add and
 * store (atomic == 0), 16384 elements per workgroup of 256 threads. */
int attn_probe_atomic(float* target, size_t n, int atomic, hipStream_t stream);

/* y[i] = v_exp_f32(x[i]) (the exp2 every kernel's softmax uses), i < n. */
int attn_probe_exp2(const float* x, float* y, size_t n, hipStream_t stream);

/* HBM read rate: `workgroups` workgroups of 256 threads read the `bytes` bytes
 * at src (a multiple of 16, 16-byte aligned) once, as 16-byte loads, each
 * thread keeping `unroll` (1, 2, 4 or 8) loads in flight; sink[workgroups *
 * 256] receives a value per thread that keeps the loads alive. */
int attn_probe_read_rate(const void* src, size_t bytes, int unroll, int workgroups, unsigned* sink,
                         hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBE_H */
