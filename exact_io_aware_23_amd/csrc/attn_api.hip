// C ABI of the attention library: argument validation, then dispatch to the
// kernel launchers.  Validation runs before anything is enqueued; on error no
// work is launched and no output is touched.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/attn.h"
#include "attn_launch.h"

namespace {

bool sizes_ok(int B, int H, int N) {
  if (B <= 0 || H <= 0 || N <= 0) return false;
  const int64_t rows = (int64_t)B * H * N;
  return rows < ((int64_t)1 << 31);
}

// any finite scale: the kernels run the softmax with |scale| and apply its
// sign (or zero) to the operand they hold in registers
bool scale_ok(float scale) { return std::isfinite(scale); }
bool descale_ok(float x) { return std::isfinite(x) && x > 0.f; }

// the kernels address one (batch, head) slab with 32-bit byte offsets
constexpr int kMaxN = 1 << 22;

attn_status_t map_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

attn_status_t check_bf16_d(int d, attn_dtype_t dtype) {
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                       int N, int d, attn_dtype_t dtype, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_INVALID;
  if (!sizes_ok(B, H, N) || !scale_ok(scale) || (causal != 0 && causal != 1)) return ATTN_ERR_INVALID;
  if (N > kMaxN) return ATTN_ERR_UNSUPPORTED;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  return map_hip(attn::launch_fwd(q, k, v, o, lse, B * H, N, d, dtype == ATTN_BF16, scale, causal != 0,
                                  attn::BlockMask{}, attn::DropParams{}, (hipStream_t)stream));
}

namespace {
size_t delta_bytes(int B, int H, int N) {
  const size_t bytes = (size_t)B * H * N * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}
}  // namespace

size_t attn_bwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  if (!sizes_ok(B, H, N)) return 0;
  return delta_bytes(B, H, N);  // the exact delta, from the dq stage to the dkdv stage
}

attn_status_t attn_bwd_preprocess(const void* o, const void* dout, float* delta, int B, int H, int N, int d,
                                  attn_dtype_t dtype, void* stream) {
  if (!o || !dout || !delta) return ATTN_ERR_INVALID;
  if (!sizes_ok(B, H, N)) return ATTN_ERR_INVALID;
  if (N > kMaxN) return ATTN_ERR_UNSUPPORTED;
  const attn_status_t s = check_bf16_d(d, dtype);
  if (s != ATTN_OK) return s;
  return map_hip(attn::launch_bwd_preprocess(o, dout, delta, B * H, N, d, (hipStream_t)stream));
}

attn_status_t attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                            const float* delta, void* dk, void* dv, int B, int H, int N, int d,
                            attn_dtype_t dtype, float scale, int causal, void* stream) {
  if (!q || !k || !v || !lse || !dout || !delta || !dk || !dv) return ATTN_ERR_INVALID;
  if (!sizes_ok(B, H, N) || !scale_ok(scale) || (causal != 0 && causal != 1)) return ATTN_ERR_INVALID;
  if (N > kMaxN) return ATTN_ERR_UNSUPPORTED;
  const attn_status_t s = check_bf16_d(d, dtype);
  if (s != ATTN_OK) return s;
  return map_hip(attn::launch_bwd_dkdv(q, k, v, lse, dout, delta, dk, dv, B * H, N, d, scale, causal != 0,
                                       attn::BlockMask{}, attn::DropParams{}, (hipStream_t)stream));
}

attn_status_t attn_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                          const float* delta, void* dq, float* delta_out, int B, int H, int N, int d,
                          attn_dtype_t dtype, float scale, int causal, void* stream) {
  if (!q || !k || !v || !lse || !dout || !delta || !dq || !delta_out) return ATTN_ERR_INVALID;
  if (!sizes_ok(B, H, N) || !scale_ok(scale) || (causal != 0 && causal != 1)) return ATTN_ERR_INVALID;
  if (N > kMaxN) return ATTN_ERR_UNSUPPORTED;
  const attn_status_t s = check_bf16_d(d, dtype);
  if (s != ATTN_OK) return s;
  return map_hip(attn::launch_bwd_dq(q, k, v, lse, dout, delta, nullptr, dq, delta_out, B * H, N, d, scale,
                                     causal != 0, attn::BlockMask{}, attn::DropParams{}, (hipStream_t)stream));
}

attn_status_t attn_bwd_dq_fused(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                const void* dout, void* dq, float* delta_out, int B, int H, int N, int d,
                                attn_dtype_t dtype, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !delta_out) return ATTN_ERR_INVALID;
  if (!sizes_ok(B, H, N) || !scale_ok(scale) || (causal != 0 && causal != 1)) return ATTN_ERR_INVALID;
  if (N > kMaxN) return ATTN_ERR_UNSUPPORTED;
  const attn_status_t s = check_bf16_d(d, dtype);
  if (s != ATTN_OK) return s;
  return map_hip(attn::launch_bwd_dq(q, k, v, lse, dout, nullptr, o, dq, delta_out, B * H, N, d, scale,
                                     causal != 0, attn::BlockMask{}, attn::DropParams{}, (hipStream_t)stream));
}

namespace {
// dq (forms delta~ = rowsum(dO * O) itself, bit for bit as the preprocess
// stage does, and writes the exact delta) -> dkdv, with an optional block mask
attn_status_t bwd_all(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, void* workspace, int B, int H, int N,
                      int d, float scale, int causal, const attn::BlockMask& m, const attn::DropParams& dr,
                      void* stream) {
  float* delta_exact = static_cast<float*>(workspace);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = attn::launch_bwd_dq(q, k, v, lse, dout, nullptr, o, dq, delta_exact, B * H, N, d, scale,
                                     causal != 0, m, dr, st);
  if (e != hipSuccess) return ATTN_ERR_HIP;
  e = attn::launch_bwd_dkdv(q, k, v, lse, dout, delta_exact, dk, dv, B * H, N, d, scale, causal != 0, m, dr, st);
  return map_hip(e);
}

// the mask arguments of the block-sparse entry points; ATTN_OK when usable
attn_status_t check_mask(const uint8_t* mask, int mask_heads, int B, int H, int N) {
  if (!mask || (mask_heads != 1 && mask_heads != B * H)) return ATTN_ERR_INVALID;
  if (N > attn::kMaxSparseN) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// dropout rate -> byte threshold t = round(256 p); ATTN_OK when t is in [0, 255]
attn_status_t make_drop(float p_drop, uint64_t seed, attn::DropParams* dr) {
  if (!std::isfinite(p_drop) || p_drop < 0.f) return ATTN_ERR_INVALID;
  const double t = std::floor(256.0 * (double)p_drop + 0.5);
  if (t > 255.0) return ATTN_ERR_INVALID;
  dr->on = true;
  dr->t = (uint32_t)t;
  dr->seed_lo = (uint32_t)(seed & 0xFFFFFFFFu);
  dr->seed_hi = (uint32_t)(seed >> 32);
  dr->inv_keep = (float)(256.0 / (256.0 - t));
  return ATTN_OK;
}

attn::BlockMask make_mask(const uint8_t* mask, int mask_heads, int N) {
  attn::BlockMask m;
  m.ptr = mask;
  m.nb = (N + 127) / 128;
  m.head_stride = mask_heads == 1 ? 0 : m.nb * m.nb;
  return m;
}
}  // namespace

attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, void* workspace,
                       size_t workspace_bytes, int B, int H, int N, int d, attn_dtype_t dtype, float scale,
                       int causal, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace) return ATTN_ERR_INVALID;
  if (!sizes_ok(B, H, N) || !scale_ok(scale) || (causal != 0 && causal != 1)) return ATTN_ERR_INVALID;
  if (N > kMaxN) return ATTN_ERR_UNSUPPORTED;
  const attn_status_t s = check_bf16_d(d, dtype);
  if (s != ATTN_OK) return s;
  if (workspace_bytes < attn_bwd_workspace_bytes(B, H, N, d)) return ATTN_ERR_INVALID;
  return bwd_all(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, d, scale, causal, attn::BlockMask{},
                 attn::DropParams{}, stream);
}

}  // extern "C"

namespace {
// Scratch of attn_bwd_noalloc: the exact delta of the dq stage, one fp32 per
// query row, in a file-scope device array instead of a caller workspace.  Each
// GPU holds its own copy until the process ends.  In host code `scratch`
// names a host-side stand-in; kernels get the device address that
// hipGetSymbolAddress returns, looked up once per device.
constexpr size_t kScratchBytes = (size_t)16 << 20;  // 4M rows
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of this device's scratch array (the current device)
attn_status_t scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ATTN_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}
}  // namespace

extern "C" {

size_t attn_bwd_noalloc_max_rows(void) { return kScratchBytes / sizeof(float); }

attn_status_t attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                               const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                               attn_dtype_t dtype, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_INVALID;
  if (!sizes_ok(B, H, N) || !scale_ok(scale) || (causal != 0 && causal != 1)) return ATTN_ERR_INVALID;
  if (N > kMaxN) return ATTN_ERR_UNSUPPORTED;
  const attn_status_t s = check_bf16_d(d, dtype);
  if (s != ATTN_OK) return s;
  if (attn_bwd_workspace_bytes(B, H, N, d) > kScratchBytes) return ATTN_ERR_SCRATCH;
  void* ws = nullptr;
  const attn_status_t sa = scratch_address(&ws);
  if (sa != ATTN_OK) return sa;
  // every row of the delta array is written by the dq stage before the dkdv
  // stage reads it, so the previous call's contents need no clearing
  return bwd_all(q, k, v, o, lse, dout, dq, dk, dv, ws, B, H, N, d, scale, causal, attn::BlockMask{},
                 attn::DropParams{}, stream);
}

attn_status_t attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                                    const uint8_t* block_mask, int mask_heads, int B, int H, int N, int d,
                                    attn_dtype_t dtype, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_INVALID;
  if (!sizes_ok(B, H, N) || !scale_ok(scale) || (causal != 0 && causal != 1)) return ATTN_ERR_INVALID;
  if (N > kMaxN) return ATTN_ERR_UNSUPPORTED;
  attn_status_t s = check_mask(block_mask, mask_heads, B, H, N);
  if (s == ATTN_OK) s = check_bf16_d(d, dtype);
  if (s != ATTN_OK) return s;
  return map_hip(attn::launch_fwd(q, k, v, o, lse, B * H, N, d, true, scale, causal != 0,
                                  make_mask(block_mask, mask_heads, N), attn::DropParams{}, (hipStream_t)stream));
}

attn_status_t attn_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o,
                                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                    const uint8_t* block_mask, int mask_heads, void* workspace,
                                    size_t workspace_bytes, int B, int H, int N, int d, attn_dtype_t dtype,
                                    float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace) return ATTN_ERR_INVALID;
  if (!sizes_ok(B, H, N) || !scale_ok(scale) || (causal != 0 && causal != 1)) return ATTN_ERR_INVALID;
  if (N > kMaxN) return ATTN_ERR_UNSUPPORTED;
  attn_status_t s = check_mask(block_mask, mask_heads, B, H, N);
  if (s == ATTN_OK) s = check_bf16_d(d, dtype);
  if (s != ATTN_OK) return s;
  if (workspace_bytes < attn_bwd_workspace_bytes(B, H, N, d)) return ATTN_ERR_INVALID;
  return bwd_all(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, d, scale, causal,
                 make_mask(block_mask, mask_heads, N), attn::DropParams{}, stream);
}

attn_status_t attn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, float p_drop,
                               uint64_t seed, int B, int H, int N, int d, attn_dtype_t dtype, float scale,
                               int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_INVALID;
  if (!sizes_ok(B, H, N) || !scale_ok(scale) || (causal != 0 && causal != 1)) return ATTN_ERR_INVALID;
  if (N > kMaxN) return ATTN_ERR_UNSUPPORTED;
  attn::DropParams dr;
  attn_status_t s = make_drop(p_drop, seed, &dr);
  if (s == ATTN_OK) s = check_bf16_d(d, dtype);
  if (s != ATTN_OK) return s;
  return map_hip(attn::launch_fwd(q, k, v, o, lse, B * H, N, d, true, scale, causal != 0, attn::BlockMask{}, dr,
                                  (hipStream_t)stream));
}

attn_status_t attn_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                               const void* dout, void* dq, void* dk, void* dv, float p_drop, uint64_t seed,
                               void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                               attn_dtype_t dtype, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace) return ATTN_ERR_INVALID;
  if (!sizes_ok(B, H, N) || !scale_ok(scale) || (causal != 0 && causal != 1)) return ATTN_ERR_INVALID;
  if (N > kMaxN) return ATTN_ERR_UNSUPPORTED;
  attn::DropParams dr;
  attn_status_t s = make_drop(p_drop, seed, &dr);
  if (s == ATTN_OK) s = check_bf16_d(d, dtype);
  if (s != ATTN_OK) return s;
  if (workspace_bytes < attn_bwd_workspace_bytes(B, H, N, d)) return ATTN_ERR_INVALID;
  return bwd_all(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, d, scale, causal, attn::BlockMask{}, dr,
                 stream);
}

size_t attn_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || (d != 64 && d != 128)) return 0;
  if (Nq > attn::decode_max_queries() || Nk > (1 << 23) || (int64_t)B * H * Nk >= ((int64_t)1 << 31)) return 0;
  const size_t parts = (size_t)B * H * attn::decode_chunks(B * H, Nk) * Nq;
  const size_t bytes = parts * (2 + (size_t)d) * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

attn_status_t attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                          void* workspace, size_t workspace_bytes, int B, int H, int Nq, int Nk, int d,
                          attn_dtype_t dtype, float scale, int causal, void* stream) {
  if (!q || !k_cache || !v_cache || !o || !lse || !workspace) return ATTN_ERR_INVALID;
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || (int64_t)B * H * Nk >= ((int64_t)1 << 31)) return ATTN_ERR_INVALID;
  if (!scale_ok(scale) || (causal != 0 && causal != 1)) return ATTN_ERR_INVALID;
  if (causal && Nq > Nk) return ATTN_ERR_INVALID;
  if (Nq > attn::decode_max_queries() || Nk > (1 << 23)) return ATTN_ERR_UNSUPPORTED;  // 32-bit byte offsets
  const attn_status_t s = check_bf16_d(d, dtype);
  if (s != ATTN_OK) return s;
  if (workspace_bytes < attn_decode_workspace_bytes(B, H, Nq, Nk, d)) return ATTN_ERR_INVALID;
  return map_hip(attn::launch_decode(q, k_cache, v_cache, o, lse, static_cast<float*>(workspace), B * H, Nq, Nk,
                                     d, scale, causal != 0, (hipStream_t)stream));
}

attn_status_t attn_fwd_fp8(const void* q, const void* k, const void* v, float descale_q, float descale_k,
                           float descale_v, void* o, float* lse, int B, int H, int N, int d, float scale,
                           int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_INVALID;
  if (!sizes_ok(B, H, N) || !scale_ok(scale) || (causal != 0 && causal != 1)) return ATTN_ERR_INVALID;
  if (!descale_ok(descale_q) || !descale_ok(descale_k) || !descale_ok(descale_v)) return ATTN_ERR_INVALID;
  // |scale dq dk| must be a finite fp32 value, and not round to 0 unless scale is 0
  const float c = (float)((double)(scale < 0.f ? -scale : scale) * descale_q * descale_k);
  if (!std::isfinite(c) || (scale != 0.f && c == 0.f)) return ATTN_ERR_INVALID;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (N > kMaxN) return ATTN_ERR_UNSUPPORTED;
  return map_hip(attn::launch_fwd_fp8(q, k, v, o, lse, B * H, N, d, scale, descale_q, descale_k, descale_v,
                                      causal != 0, (hipStream_t)stream));
}

const char* attn_status_string(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dimension, dtype or sequence length";
    case ATTN_ERR_HIP: return "HIP launch error";
    case ATTN_ERR_SCRATCH: return "problem larger than the static scratch buffer of the allocation-free entry point";
  }
  return "unknown status";
}

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

}  // extern "C"
