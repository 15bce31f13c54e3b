// Hardware probes behind the design's measured rates (MI355X, gfx950).  They
// are measurement aids, not part of the attention ABI: each launches one small
// kernel on the caller's stream and writes raw cycle counts or values into
// caller-owned device buffers, which the host turns into rates.
//
//   attn_probe_lds_rate   LDS read throughput of 16-byte reads (ds_read_b128)
//                         and of the transposing 8-byte read
//                         (ds_read_b64_tr_b16), per workgroup in s_memtime
//                         cycles.
//   attn_probe_issue      issue rates of v_exp_f32, v_fma_f32 and the
//                         32x32x16 bf16 MFMA, one kind per wave, so two kinds
//                         can share a SIMD.
//   attn_probe_wave_simd  the HW_ID register of every wave of 8-wave
//                         workgroups (which SIMD each wave lands on).
//   attn_probe_atomic     fp32 global atomic adds, or the same update as a
//                         plain load, add and store, over a region.
//   attn_probe_exp2       y = v_exp_f32(x) elementwise, for an accuracy sweep.
//   attn_probe_read_rate  a read-only stream over a device buffer (16-byte
//                         loads, a chosen number in flight per thread): the
//                         HBM read rate a bandwidth-bound kernel can reach.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "attn_probe.h"

namespace attn_probe {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kLdsBytes = 32768;  // per workgroup, so four fit on a CU
constexpr int kLdsIters = 2048, kLdsUnroll = 8;

// Every lane reads 16 (or 8) bytes per instruction; consecutive lanes read
// consecutive chunks, each unrolled read starts 2 KB further on, and every
// address is masked into the array.  `off` is 0 at run time but unknown to the
// compiler, so no read can be folded or hoisted.
template <int MODE>
__global__ void __launch_bounds__(256) lds_rate_kernel(unsigned* __restrict__ sink,
                                                       unsigned long long* __restrict__ cycles) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
  const int tid = threadIdx.x;
  for (int i = tid * 16; i < kLdsBytes; i += 256 * 16) *(u32x4*)(lds + i) = u32x4{(unsigned)i, 1u, 2u, 3u};
  __syncthreads();
  const unsigned off = *(volatile unsigned*)(lds + 4) - 1u;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  unsigned acc = 0;
  const unsigned base = (unsigned)tid * 16u;
  for (int it = 0; it < kLdsIters; ++it) {
#pragma unroll
    for (int u = 0; u < kLdsUnroll; ++u) {
      const unsigned a = (base + (unsigned)((it * kLdsUnroll + u) & 15) * 2048u + (unsigned)it * off * 16u) &
                         (unsigned)(kLdsBytes - 16);
      if constexpr (MODE == 0) {
        const u32x4 v = *(const u32x4*)(lds + a);
        acc ^= v[0] + v[3];
      } else {
        const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(lds + (a & (unsigned)(kLdsBytes - 8))));
        acc ^= __builtin_bit_cast(unsigned, __builtin_shufflevector(v, v, 0, 1)) +
               __builtin_bit_cast(unsigned, __builtin_shufflevector(v, v, 2, 3));
      }
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  sink[blockIdx.x * 256 + tid] = acc;
  if (tid == 0) cycles[blockIdx.x] = t1 - t0;
}

constexpr int kIssueIters = 4096;

__device__ __forceinline__ float issue_exp(float x) {
  float a0 = x, a1 = x + 1, a2 = x + 2, a3 = x + 3, a4 = x + 4, a5 = x + 5, a6 = x + 6, a7 = x + 7;
  for (int i = 0; i < kIssueIters; ++i) {
    a0 = __builtin_amdgcn_exp2f(a0); a1 = __builtin_amdgcn_exp2f(a1); a2 = __builtin_amdgcn_exp2f(a2);
    a3 = __builtin_amdgcn_exp2f(a3); a4 = __builtin_amdgcn_exp2f(a4); a5 = __builtin_amdgcn_exp2f(a5);
    a6 = __builtin_amdgcn_exp2f(a6); a7 = __builtin_amdgcn_exp2f(a7);
  }
  return a0 + a1 + a2 + a3 + a4 + a5 + a6 + a7;
}
__device__ __forceinline__ float issue_fma(float x, float y) {
  float a0 = x, a1 = x + 1, a2 = x + 2, a3 = x + 3, a4 = x + 4, a5 = x + 5, a6 = x + 6, a7 = x + 7;
  for (int i = 0; i < kIssueIters; ++i) {
    a0 = fmaf(a0, y, x); a1 = fmaf(a1, y, x); a2 = fmaf(a2, y, x); a3 = fmaf(a3, y, x);
    a4 = fmaf(a4, y, x); a5 = fmaf(a5, y, x); a6 = fmaf(a6, y, x); a7 = fmaf(a7, y, x);
  }
  return a0 + a1 + a2 + a3 + a4 + a5 + a6 + a7;
}
__device__ __forceinline__ float issue_mfma(float x) {
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(x + e);
    b[e] = (__bf16)(x - e);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < kIssueIters / 4; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  return s;
}

// wave w of every workgroup runs kinds[w] (0 idle, 1 exp, 2 fma, 3 mfma):
// 8 * 4096 instructions of exp or fma, 4096 MFMAs
__global__ void __launch_bounds__(512) issue_kernel(const int* __restrict__ kinds, float* __restrict__ sink,
                                                    unsigned long long* __restrict__ cycles) {
  const int wave = threadIdx.x >> 6;
  const int kind = __builtin_amdgcn_readfirstlane(kinds[wave]);
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  float r = 0.f;
  if (kind == 1) r = issue_exp(0.001f);
  else if (kind == 2) r = issue_fma(0.001f, 0.999f);
  else if (kind == 3) r = issue_mfma(0.001f);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  sink[blockIdx.x * blockDim.x + threadIdx.x] = r;
  if ((threadIdx.x & 63) == 0) cycles[blockIdx.x * 8 + wave] = t1 - t0;
}

__global__ void __launch_bounds__(512) wave_simd_kernel(unsigned* __restrict__ hwid) {
  const unsigned hw = __builtin_amdgcn_s_getreg(4 | (31 << 11));  // HW_ID
  if ((threadIdx.x & 63) == 0) hwid[blockIdx.x * 8 + (threadIdx.x >> 6)] = hw;
}

constexpr int kAtomicIters = 64;

// thread t of workgroup b updates element (b * 256 * iters + i * 256 + t), so
// every element of a region of grid * 256 * iters floats is updated once
template <bool ATOMIC>
__global__ void __launch_bounds__(256) atomic_kernel(float* __restrict__ target) {
  const size_t base = (size_t)blockIdx.x * 256 * kAtomicIters + threadIdx.x;
  for (int i = 0; i < kAtomicIters; ++i) {
    float* p = target + base + (size_t)i * 256;
    if constexpr (ATOMIC) atomicAdd(p, 1.0f);
    else *p = *p + 1.0f;
  }
}

__global__ void __launch_bounds__(256) exp2_kernel(const float* __restrict__ x, float* __restrict__ y, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] = __builtin_amdgcn_exp2f(x[i]);
}

// Thread t of the grid reads 16-byte words t, t + T, t + 2T, ... (T threads in
// all), U of them issued before any is used; the words are folded into one
// value per thread so the loads stay live.
template <int U>
__global__ void __launch_bounds__(256) read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                   unsigned* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  unsigned acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace
}  // namespace attn_probe

using namespace attn_probe;

extern "C" {

int attn_probe_lds_rate(int mode, int workgroups, unsigned* sink, unsigned long long* cycles, hipStream_t stream) {
  if ((mode != 0 && mode != 1) || workgroups <= 0 || workgroups > (1 << 16) || !sink || !cycles) return 1;
  if (mode == 0) hipLaunchKernelGGL(lds_rate_kernel<0>, dim3(workgroups), dim3(256), 0, stream, sink, cycles);
  else hipLaunchKernelGGL(lds_rate_kernel<1>, dim3(workgroups), dim3(256), 0, stream, sink, cycles);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int attn_probe_issue(const int* kinds, int waves, int workgroups, float* sink, unsigned long long* cycles,
                     hipStream_t stream) {
  if (waves <= 0 || waves > 8 || workgroups <= 0 || workgroups > (1 << 16) || !kinds || !sink || !cycles) return 1;
  hipLaunchKernelGGL(issue_kernel, dim3(workgroups), dim3(64 * waves), 0, stream, kinds, sink, cycles);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int attn_probe_wave_simd(int workgroups, unsigned* hwid, hipStream_t stream) {
  if (workgroups <= 0 || workgroups > (1 << 16) || !hwid) return 1;
  hipLaunchKernelGGL(wave_simd_kernel, dim3(workgroups), dim3(512), 0, stream, hwid);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int attn_probe_atomic(float* target, size_t n, int atomic, hipStream_t stream) {
  const size_t per_wg = (size_t)256 * kAtomicIters;
  if (!target || n < per_wg || n % per_wg != 0 || n / per_wg > (size_t)(1u << 31)) return 1;
  const unsigned grid = (unsigned)(n / per_wg);
  if (atomic) hipLaunchKernelGGL(atomic_kernel<true>, dim3(grid), dim3(256), 0, stream, target);
  else hipLaunchKernelGGL(atomic_kernel<false>, dim3(grid), dim3(256), 0, stream, target);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int attn_probe_exp2(const float* x, float* y, size_t n, hipStream_t stream) {
  if (!x || !y || n == 0 || (n + 255) / 256 > (size_t)(1u << 31)) return 1;
  hipLaunchKernelGGL(exp2_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, x, y, n);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int attn_probe_read_rate(const void* src, size_t bytes, int unroll, int workgroups, unsigned* sink,
                         hipStream_t stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || workgroups <= 0 || workgroups > (1 << 20)) return 1;
  const u32x4* p = static_cast<const u32x4*>(src);
  const size_t n16 = bytes / 16;
  switch (unroll) {
    case 1: hipLaunchKernelGGL(read_kernel<1>, dim3(workgroups), dim3(256), 0, stream, p, n16, sink); break;
    case 2: hipLaunchKernelGGL(read_kernel<2>, dim3(workgroups), dim3(256), 0, stream, p, n16, sink); break;
    case 4: hipLaunchKernelGGL(read_kernel<4>, dim3(workgroups), dim3(256), 0, stream, p, n16, sink); break;
    case 8: hipLaunchKernelGGL(read_kernel<8>, dim3(workgroups), dim3(256), 0, stream, p, n16, sink); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
