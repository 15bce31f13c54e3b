// Internal launchers behind the C ABI.  Arguments are already validated;
// BH = B * H.  Each returns hipGetLastError() after enqueueing on `stream`.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Optional block-sparse mask: one byte per 128 x 128 block, [heads][nb][nb]
// with nb = ceil(N / 128); head_stride is 0 when one mask serves every head
// and nb * nb otherwise.  ptr == nullptr means dense.
constexpr int kMaxSparseN = 65536;  // longest sequence the block-sparse entry points take

struct BlockMask {
  const uint8_t* ptr = nullptr;
  int head_stride = 0;
  int nb = 0;
};

// Optional dropout on P: an element is kept iff its generator byte is >= t
// (rate t / 256); kept entries are scaled by inv_keep = 1 / (1 - t / 256).
// seed_lo / seed_hi are the two halves of the 64-bit generator key.
struct DropParams {
  bool on = false;
  uint32_t t = 0;
  uint32_t seed_lo = 0, seed_hi = 0;
  float inv_keep = 1.f;
};

// The factor the kernels fold into their exponent FMA (c = |scale| log2 e,
// or log2 e when scale = 0) and how the sign of scale is applied to the
// operand held in registers (kSignPos / kSignNeg / kSignZero of attn_common.h).
struct ScoreScale {
  float c;
  uint32_t mode;
};
inline ScoreScale split_scale(float scale) {
  constexpr float kLog2eHost = 1.4426950408889634f;
  if (scale > 0.f) return {scale * kLog2eHost, 0u};
  if (scale < 0.f) return {-scale * kLog2eHost, 1u};
  return {kLog2eHost, 2u};
}

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N,
                      int d, bool bf16_in, float scale, bool causal, const BlockMask& mask, const DropParams& drop,
                      hipStream_t stream);

hipError_t launch_bwd_preprocess(const void* o, const void* dout, float* delta, int BH, int N, int d,
                                 hipStream_t stream);

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                           const void* dout, const float* delta, void* dk, void* dv, int BH, int N,
                           int d, float scale, bool causal, const BlockMask& mask, const DropParams& drop,
                           hipStream_t stream);

// o_fused != nullptr: the kernel forms delta~ = rowsum(dO * O) itself (bit for
// bit as launch_bwd_preprocess does) and ignores `delta`.
hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                         const void* dout, const float* delta, const void* o_fused, void* dq, float* delta_out,
                         int BH, int N, int d, float scale, bool causal, const BlockMask& mask,
                         const DropParams& drop, hipStream_t stream);

// FP8 forward: q, k, v are e4m3 codes, o bf16; S = scale dq dk Q K^T, O = dv P V.
hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, int d,
                          float scale, float dq, float dk, float dv, bool causal, hipStream_t stream);

// Decode against a KV cache: Nq <= decode_max_queries() queries per
// (batch, head), Nk cached keys, split into S = decode_chunks(BH, Nk) chunks
// (of 512, 256 or 128 keys, by the size of the call) whose partial results
// (m, l: BH*S*Nq floats each, then O: BH*S*Nq*d floats) live in the fp32
// workspace `ws`.
int decode_chunks(int BH, int Nk);
int decode_max_queries();
hipError_t launch_decode(const void* q, const void* k, const void* v, void* o, float* lse, float* ws, int BH,
                         int Nq, int Nk, int d, float scale, bool causal, hipStream_t stream);

}  // namespace attn
