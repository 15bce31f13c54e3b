// Decode attention against a KV cache for gfx950.
//
// What it computes (the pages, by title and section): "What is Flash
// Attention?" (iania.ai video page, English) lists memory-bound inference
// with long prompts among the uses (10:00) and names the KV cache for fast
// generation as the next step (11:02-11:33).  A few new queries (Nq <= 8)
// attend to the Nk keys and values held in a cache; with the causal flag
// query i is the (Nk - Nq + i)-th position and sees keys j <= Nk - Nq + i.
//
// Design (MI355X): decode reads every cached key and value once and does
// ~2 FLOPs per byte, so it is bound by HBM bandwidth, not by the matrix
// cores.  The work is split over the keys:
//   * decode_partial_kernel (one query) or decode_mma_kernel (two or more,
//     both products on the matrix cores; see there): one workgroup per
//     (batch*head, chunk of 512 keys, or 256 / 128 for small calls).  In the first, four threads per key form
//     the chunk's scores for every query (16-byte loads of K kept as bf16
//     pairs, v_dot2_f32_bf16 against q held in LDS as bf16 pairs, two DPP
//     adds); one wave per query takes the chunk max and exp-sum; then 16
//     (d=128) or 32 (d=64) key lanes accumulate
//     sum_j p_j V_j two keys at a time: the two V rows are interleaved into
//     bf16 pairs, p of both keys is rounded to one bf16 pair (as the forward
//     rounds P before its P V product; l sums the unrounded p), and one
//     v_dot2_f32_bf16 adds both keys' products to a column.  The lanes and
//     waves are reduced through cross-lane swaps and LDS.  The chunk's
//     (m, l, unnormalised O) go to the workspace.
//   * decode_merge_kernel: per (batch*head, query) it merges the chunks with
//     the online-softmax rule of the same page (04:46-05:17): m = max m_c,
//     l = sum 2^(m_c - m) l_c, O = sum 2^(m_c - m) O_c / l.
// Scores are kept in base-2 units (scale * log2 e folded in), as in the
// forward kernel.
#include <cstdint>
#include <type_traits>

#include "attn_common.h"
#include "attn_launch.h"

namespace attn {
namespace {

constexpr int kDecChunk = 512;       // keys per workgroup at most (small calls take 256 or 128)
constexpr int kDecMinChunk = 128;    // keys per workgroup at least
constexpr int kDecTargetWgs = 1024;  // workgroups a call should have to fill the GPU (four per CU)
constexpr int kDecTile = 64;         // keys per pass-1 tile (4 threads per key)
constexpr int kDecMaxQ = 8;          // most queries per call

// A chunk's unnormalised O column goes to the workspace for the merge kernel;
// when the whole cache is one chunk (S == 1) there is nothing to merge, and
// the kernel writes what the merge would form from that single chunk,
// O = O_c / l_c and L = (m_c + log2 l_c) ln 2 (O = 0 and L = -inf for a query
// with no allowed key), so the call needs one launch, not two.
__device__ __forceinline__ void emit(bf16* __restrict__ O, float* __restrict__ L, float* __restrict__ ws_o, int bh,
                                     int s, int S, int nq, int qi, int D, int dd, float o, float m, float l) {
  if (S > 1) {
    ws_o[(((size_t)bh * S + s) * nq + qi) * D + dd] = o;
    return;
  }
  const bool empty = l == 0.f;
  O[((size_t)bh * nq + qi) * D + dd] = (bf16)(empty ? 0.f : o / l);
  if (dd == 0) L[(size_t)bh * nq + qi] = empty ? -INFINITY : (m + log2f(l)) * kLn2;
}

// NQ: query capacity of the instantiation (>= nq); registers and LDS scale
// with it.  The launcher instantiates it for one query only (more go to
// decode_mma_kernel), which keeps many workgroups per CU in flight.  CH: keys
// per chunk (512, 256 or 128).
template <int D, int NQ, int CH>
__global__ void __launch_bounds__(256)
decode_partial_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                      float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o,
                      bf16* __restrict__ O, float* __restrict__ L, int Nk, int nq, int S, float c, int causal) {
  constexpr int DP = D / 4;          // dims per thread in pass 1
  constexpr int G8 = D / 8;          // 8-dim groups in pass 2
  constexpr int KL = 256 / G8;       // key lanes in pass 2
  static_assert(NQ >= 1 && NQ <= kDecMaxQ, "query capacity");
  __shared__ __attribute__((aligned(16))) uint32_t qs2[NQ][D / 2];  // q as packed bf16 pairs
  __shared__ float sc[NQ][CH];
  __shared__ __attribute__((aligned(16))) float red[4][NQ][D];
  __shared__ float cm[NQ], cl[NQ];  // the chunk's max and exp-sum per query

  const int bh = blockIdx.x / S;
  const int s = blockIdx.x % S;
  const int k0 = s * CH;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint32_t head_bytes = (uint32_t)Nk * D * 2;
  const rsrc_t rK = make_rsrc(K + (size_t)bh * Nk * D, head_bytes);
  const rsrc_t rV = make_rsrc(V + (size_t)bh * Nk * D, head_bytes);

  {
    const uint32_t* q2 = reinterpret_cast<const uint32_t*>(Q + (size_t)bh * nq * D);
    for (int idx = tid; idx < nq * D / 2; idx += 256) qs2[idx / (D / 2)][idx % (D / 2)] = q2[idx];
  }
  __syncthreads();

  // ---- pass 1: scores of the chunk, in base-2 units; masked keys get -inf
  {
    const int kl = tid >> 2, part = tid & 3;
#pragma unroll 2
    for (int kt = 0; kt < CH; kt += kDecTile) {
      const int key = k0 + kt + kl;
      // K stays packed: v_dot2_f32_bf16 takes two bf16 products per
      // instruction (each exact in fp32) and q comes from LDS as bf16 pairs
      u32x4 kw[DP / 8];
#pragma unroll
      for (int i = 0; i < DP / 8; ++i) kw[i] = bload16(rK, (key * D + part * DP + 8 * i) * 2, 0);
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi) {
        if (qi >= nq) break;
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < DP / 8; ++i) {
          const u32x4 qv = *reinterpret_cast<const u32x4*>(&qs2[qi][(part * DP + 8 * i) / 2]);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            // (vector elements go through plain words: a bit_cast of a
            // subscripted vector element read element 0 with this compiler)
            const uint32_t kx = kw[i][w], qx = qv[w];
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kx), __builtin_bit_cast(bf16x2, qx), acc,
                                                  false);
          }
        }
        acc += __builtin_bit_cast(float, quad_xor<1>(__builtin_bit_cast(uint32_t, acc)));
        acc += __builtin_bit_cast(float, quad_xor<2>(__builtin_bit_cast(uint32_t, acc)));
        const bool ok = key < Nk && (!causal || key <= Nk - nq + qi);
        if (part == 0) sc[qi][kt + kl] = ok ? acc * c : -INFINITY;
      }
    }
  }
  __syncthreads();

  // ---- chunk max and exp-sum per query (one wave per query); p in place
  for (int qi = wave; qi < nq; qi += 4) {
    float m = -INFINITY;
    for (int i = lane; i < CH; i += 64) m = fmaxf(m, sc[qi][i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float l = 0.f;
    for (int i = lane; i < CH; i += 64) {
      const float p = m == -INFINITY ? 0.f : fast_exp2(sc[qi][i] - m);
      sc[qi][i] = p;
      l += p;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
    if (lane == 0) {
      cm[qi] = m;
      cl[qi] = l;
      if (S > 1) {
        ws_m[((size_t)bh * S + s) * nq + qi] = m;
        ws_l[((size_t)bh * S + s) * nq + qi] = l;
      }
    }
  }
  __syncthreads();

  // ---- pass 2: unnormalised O_c = sum_j p_j V_j over the chunk
  const int g8 = tid % G8, kl2 = tid / G8;
  float acc[NQ][8];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[qi][e] = 0.f;
  // two keys per step: V rows kj and kj + KL are interleaved into bf16 pairs
  // (one v_perm per pair) and p of both keys is rounded to one bf16 pair, so
  // each v_dot2_f32_bf16 adds two keys' products to a column
#pragma unroll 2
  for (int kj = kl2; kj < CH; kj += 2 * KL) {
    const u32x4 va = bload16(rV, ((k0 + kj) * D + 8 * g8) * 2, 0);
    const u32x4 vb = bload16(rV, ((k0 + kj + KL) * D + 8 * g8) * 2, 0);
    uint32_t pr[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      pr[2 * w] = __builtin_amdgcn_perm(vb[w], va[w], 0x05040100u);      // element 2w of both keys
      pr[2 * w + 1] = __builtin_amdgcn_perm(vb[w], va[w], 0x07060302u);  // element 2w + 1
    }
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      if (qi >= nq) break;
      const bf16x2 pp = __builtin_bit_cast(bf16x2, pack_bf16x2(sc[qi][kj], sc[qi][kj + KL]));
#pragma unroll
      for (int e = 0; e < 8; ++e)
        acc[qi][e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pr[e]), pp, acc[qi][e], false);
    }
  }
  // lanes of one wave with the same g8 hold different keys: fold them
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    if (qi >= nq) break;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[qi][e];
#pragma unroll
      for (int off = G8; off < 64; off <<= 1) x += __shfl_xor(x, off);
      acc[qi][e] = x;
    }
  }
  if (lane < G8) {
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      if (qi >= nq) break;
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][qi][8 * g8 + e] = acc[qi][e];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < nq * D; idx += 256) {
    const int qi = idx / D, dd = idx % D;
    const float o = red[0][qi][dd] + red[1][qi][dd] + red[2][qi][dd] + red[3][qi][dd];
    emit(O, L, ws_o, bh, s, S, nq, qi, D, dd, o, cm[qi], cl[qi]);
  }
}

// v_mfma_f32_16x16x32_bf16 (wave64): lane l holds A[l % 16][8 * (l / 16) + e],
// B[8 * (l / 16) + e][l % 16] (e = 0..7) and C[4 * (l / 16) + i][l % 16]
// (i = 0..3).  As for the 32x32 product, only the pairing of the k slots of A
// and B matters.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The same partial results as decode_partial_kernel with both products on the
// matrix cores, for calls with several queries: with eight of them the two
// v_dot2 passes kept the vector ALUs about half busy and the loads waited on
// them.  Each wave owns 128 keys of the chunk in both products, and both are
// 16x16x32 products with the queries padded to 16 rows (zeros):
//   * scores: S = Q K^T, A = Q from registers, B = K^T loaded straight from
//     HBM (lane l holds key l % 16, dims 32 st + 8 (l / 16) + e, so one load
//     covers 64 contiguous bytes of 16 keys); C register i of lanes 0-31
//     holds query 4 (l / 16) + i of key l % 16.  The next 16 keys' loads are
//     issued before the current products;
//   * p V: O = P V.  B must hold 8 keys of one value column per lane, while V
//     rows run along the dims, so each lane loads D / 16 dims of 8 keys (keys
//     8 (l / 16) + e of the step, 8 or 16 contiguous bytes each) and regroups
//     them with v_perm into one operand per dim: column l % 16 of product t
//     is dim (D / 16) (l % 16) + t.  P comes from LDS as bf16, rounded as in
//     the forward kernel; l sums the unrounded p.
// The four waves' partial O meet in LDS in the space the scores used.  The
// launch bounds cap it at 80 registers, so six workgroups share a CU, as many
// as its 24 KB of LDS allow (1-2% faster than the uncapped 94 at d = 128; no
// spills).
template <int D, int CH>
__global__ void __launch_bounds__(256, 6)
decode_mma_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                  float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o, bf16* __restrict__ O,
                  float* __restrict__ L, int Nk, int nq, int S, float c, int causal) {
  constexpr int KS = D / 32;                 // 32-dim steps of the score product
  constexpr int KPW = CH / 4;         // keys per wave
  constexpr int DPL = D / 16;                // value dims per lane (= products per p V step)
  // the scores of the chunk, later the four waves' partial O
  constexpr int SBUF = kDecMaxQ * CH > 4 * kDecMaxQ * D ? kDecMaxQ * CH : 4 * kDecMaxQ * D;
  __shared__ __attribute__((aligned(16))) float sbuf[SBUF];
  __shared__ __attribute__((aligned(16))) bf16 p16[kDecMaxQ][CH];
  __shared__ float cm[kDecMaxQ], cl[kDecMaxQ];  // the chunk's max and exp-sum per query
  float (*sc)[CH] = reinterpret_cast<float (*)[CH]>(sbuf);

  const int bh = blockIdx.x / S;
  const int s = blockIdx.x % S;
  const int k0 = s * CH;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kw = KPW * wave;  // first key of this wave, relative to k0
  const uint32_t head_bytes = (uint32_t)Nk * D * 2;
  const rsrc_t rK = make_rsrc(K + (size_t)bh * Nk * D, head_bytes);
  const rsrc_t rV = make_rsrc(V + (size_t)bh * Nk * D, head_bytes);

  // ---- scores, in base-2 units; masked keys get -inf
  {
    const int n = lane & 15, g = lane >> 4;
    u32x4 qa[KS];
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const u32x4* qrow = reinterpret_cast<const u32x4*>(Q + ((size_t)bh * nq + (n < nq ? n : 0)) * D);
#pragma unroll
    for (int st = 0; st < KS; ++st) qa[st] = n < nq ? qrow[4 * st + g] : zero;
    constexpr int PF = 1;  // blocks of K loads issued ahead (more costs occupancy at d = 128)
    u32x4 kv[PF + 1][KS];
    auto kload = [&](int b, u32x4 (&dst)[KS]) {
      const uint32_t row = (uint32_t)(k0 + kw + 16 * b + n) * (D * 2) + 16u * g;
#pragma unroll
      for (int st = 0; st < KS; ++st) dst[st] = bload16(rK, (int)(row + 64u * st), 0);
    };
#pragma unroll
    for (int b = 0; b < PF; ++b) kload(b, kv[b]);
#pragma unroll
    for (int b = 0; b < KPW / 16; ++b) {
      if (b + PF < KPW / 16) kload(b + PF, kv[(b + PF) % (PF + 1)]);
      const int key = k0 + kw + 16 * b + n;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KS; ++st)
        acc = mfma16(__builtin_bit_cast(bf16x8, qa[st]), __builtin_bit_cast(bf16x8, kv[b % (PF + 1)][st]), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qi = 4 * g + i;
        if (qi < nq) {
          const bool ok = key < Nk && (!causal || key <= Nk - nq + qi);
          sc[qi][kw + 16 * b + n] = ok ? acc[i] * c : -INFINITY;
        }
      }
    }
  }
  __syncthreads();

  // ---- chunk max and exp-sum per query (one wave per query); P as bf16
  for (int qi = wave; qi < nq; qi += 4) {
    float m = -INFINITY;
    for (int i = lane; i < CH; i += 64) m = fmaxf(m, sc[qi][i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float l = 0.f;
    for (int i = lane; i < CH; i += 64) {
      const float p = m == -INFINITY ? 0.f : fast_exp2(sc[qi][i] - m);
      p16[qi][i] = to_bf16(p);
      l += p;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
    if (lane == 0) {
      cm[qi] = m;
      cl[qi] = l;
      if (S > 1) {
        ws_m[((size_t)bh * S + s) * nq + qi] = m;
        ws_l[((size_t)bh * S + s) * nq + qi] = l;
      }
    }
  }
  __syncthreads();

  // ---- unnormalised O_c = P V over the chunk (scores are dead: the partial
  // results of the waves reuse their space)
  {
    const int n = lane & 15, g = lane >> 4;
    f32x4 acc[DPL];
#pragma unroll
    for (int t = 0; t < DPL; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto pv_step = [&](int j) {
      const int kb = kw + 32 * j + 8 * g;  // first of this lane's 8 keys, relative to k0
      const uint32_t row = (uint32_t)(k0 + kb) * (D * 2) + (uint32_t)(DPL * 2) * n;
      uint32_t w[8][DPL / 2];  // w[e][x]: dims 2x, 2x + 1 (of this lane's DPL) of key kb + e
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (DPL == 8) {
          const u32x4 x = bload16(rV, (int)(row + (uint32_t)(D * 2) * e), 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) w[e][i] = x[i];
        } else {
          const u32x2 x = bload8(rV, (int)(row + (uint32_t)(D * 2) * e), 0);
          w[e][0] = x[0];
          w[e][1] = x[1];
        }
      }
      u32x4 a = {0u, 0u, 0u, 0u};
      if (n < nq) a = *reinterpret_cast<const u32x4*>(&p16[n][kb]);
#pragma unroll
      for (int t = 0; t < DPL; ++t) {
        const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;  // high or low bf16 of each word
        u32x4 bt;
#pragma unroll
        for (int x = 0; x < 4; ++x) bt[x] = __builtin_amdgcn_perm(w[2 * x + 1][t / 2], w[2 * x][t / 2], sel);
        acc[t] = mfma16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, bt), acc[t]);
      }
    };
    // two steps a loop iteration (loads of the next step in flight); with
    // only two steps in all that would hold both steps' loads at once
    if constexpr (KPW / 32 > 2) {
#pragma unroll 2
      for (int j = 0; j < KPW / 32; ++j) pv_step(j);
    } else {
#pragma unroll 1
      for (int j = 0; j < KPW / 32; ++j) pv_step(j);
    }
    float (*red)[kDecMaxQ][D] = reinterpret_cast<float (*)[kDecMaxQ][D]>(sbuf);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qi = 4 * g + i;
      if (qi < nq) {
#pragma unroll
        for (int t = 0; t < DPL; ++t) red[wave][qi][DPL * n + t] = acc[t][i];
      }
    }
  }
  __syncthreads();
  {
    float (*red)[kDecMaxQ][D] = reinterpret_cast<float (*)[kDecMaxQ][D]>(sbuf);
    for (int idx = tid; idx < nq * D; idx += 256) {
      const int qi = idx / D, dd = idx % D;
      const float o = red[0][qi][dd] + red[1][qi][dd] + red[2][qi][dd] + red[3][qi][dd];
      emit(O, L, ws_o, bh, s, S, nq, qi, D, dd, o, cm[qi], cl[qi]);
    }
  }
}

constexpr int kMergeBatch = 32;  // chunks whose loads the merge keeps in flight together

// The merge: a workgroup of G x D threads per (batch*head, query); thread
// (g, dd) sums column dd over the g-th G-th of the chunks, and the G partial
// sums are added through LDS.  The launcher takes G = 4 beyond 64 chunks, so a
// long cache (hundreds of chunks) needs a quarter of the sequential batches
// of loads, and G = 1 otherwise (measured: G = 2 at 64 chunks was 0.6 us
// slower than one group with two batches).
template <int D, int G>
__global__ void __launch_bounds__(D * G)
decode_merge_kernel(const float* __restrict__ ws_m, const float* __restrict__ ws_l, const float* __restrict__ ws_o,
                    bf16* __restrict__ O, float* __restrict__ L, int nq, int S) {
  constexpr int NB = kMergeBatch;
  __shared__ float lsh[G][D], osh[G][D];
  const int bh = blockIdx.x / nq, qi = blockIdx.x % nq;
  const int tid = threadIdx.x;
  const int dd = G == 1 ? tid : tid % D, grp = G == 1 ? 0 : tid / D;  // D >= 64: each wave lies in one group
  const int lane = tid & 63;
  const size_t base = (size_t)bh * S * nq + qi;  // partial s of this query sits at base + s * nq
  // buffer resources over this query's partials: chunk s is a scalar offset
  // of s * nq words (times D for O), and chunks past S read as zero
  const uint32_t span = (uint32_t)S * nq * 4;
  const rsrc_t rm = make_rsrc(ws_m + base, span);
  const rsrc_t rl = make_rsrc(ws_l + base, span);
  const rsrc_t ro = make_rsrc(ws_o + base * D, span * D);
  const int per = (S + G - 1) / G;
  const int sb = G == 1 ? 0 : grp * per, se = G == 1 ? S : min(S, sb + per);  // this group's chunks
  float ob[NB], mb[NB], lb[NB];
  const int step = nq * 4;  // bytes from one chunk's m (or l) to the next
  auto fetch = [&](int s0) {
    int so = s0 * step;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      ob[i] = __uint_as_float(bload4(ro, 4 * dd, so * D));
      mb[i] = __uint_as_float(bload4(rm, 0, so));
      lb[i] = __uint_as_float(bload4(rl, 0, so));
      so += step;
    }
  };
  // the group's first chunks are requested before the max is known; each
  // wave reduces the max over all chunks on its own, so both round trips overlap
  fetch(sb);
  float m = -INFINITY;
  for (int s = lane; s < S; s += 64) m = fmaxf(m, __uint_as_float(bload4(rm, 4 * s * nq, 0)));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float l = 0.f, o = 0.f;
  if (m != -INFINITY) {
    for (int s0 = sb; s0 < se; s0 += NB) {
      if (s0 > sb) fetch(s0);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        // (a chunk past this group's range weighs 0; its partials are finite, or 0 past S)
        const float a = (s0 + i >= se || mb[i] == -INFINITY) ? 0.f : fast_exp2(mb[i] - m);
        l = fmaf(a, lb[i], l);
        o = fmaf(a, ob[i], o);
      }
    }
  }
  if constexpr (G > 1) {
    if (grp > 0) {
      lsh[grp][dd] = l;
      osh[grp][dd] = o;
    }
    __syncthreads();
  }
  if (grp == 0) {
#pragma unroll
    for (int g = 1; g < G; ++g) {
      l += lsh[g][dd];
      o += osh[g][dd];
    }
    const bool empty = l == 0.f;
    O[((size_t)bh * nq + qi) * D + dd] = (bf16)(empty ? 0.f : o / l);
    if (dd == 0) L[(size_t)bh * nq + qi] = empty ? -INFINITY : (m + log2f(l)) * kLn2;
  }
}

}  // namespace

// Keys per chunk: the largest of 512, 256 and 128 that still gives the call
// kDecTargetWgs workgroups.  With 512 a call with few heads and a short cache
// (one batch of 8 heads and 8192 keys: 128 workgroups) would leave most of
// the 256 CUs idle.
int decode_chunk_keys(int BH, int Nk) {
  for (int ch = kDecChunk; ch > kDecMinChunk; ch /= 2)
    if ((int64_t)BH * ((Nk + ch - 1) / ch) >= kDecTargetWgs) return ch;
  return kDecMinChunk;
}
int decode_chunks(int BH, int Nk) {
  const int ch = decode_chunk_keys(BH, Nk);
  return (Nk + ch - 1) / ch;
}
int decode_max_queries() { return kDecMaxQ; }

hipError_t launch_decode(const void* q, const void* k, const void* v, void* o, float* lse, float* ws, int BH,
                         int Nq, int Nk, int d, float scale, bool causal, hipStream_t stream) {
  const int ch = decode_chunk_keys(BH, Nk);
  const int S = (Nk + ch - 1) / ch;
  const size_t parts = (size_t)BH * S * Nq;
  float* ws_m = ws;
  float* ws_l = ws + parts;
  float* ws_o = ws + 2 * parts;
  const float c = scale * kLog2e;
  auto partial = [&](auto dq, auto chc) {
    constexpr int D = decltype(dq)::value;
    constexpr int CH = decltype(chc)::value;
    // the matrix-core kernel measured faster from two queries up
    if (Nq == 1)
      hipLaunchKernelGGL((decode_partial_kernel<D, 1, CH>), dim3(BH * S), dim3(256), 0, stream, (const bf16*)q,
                         (const bf16*)k, (const bf16*)v, ws_m, ws_l, ws_o, (bf16*)o, lse, Nk, Nq, S, c, (int)causal);
    else
      hipLaunchKernelGGL((decode_mma_kernel<D, CH>), dim3(BH * S), dim3(256), 0, stream, (const bf16*)q,
                         (const bf16*)k, (const bf16*)v, ws_m, ws_l, ws_o, (bf16*)o, lse, Nk, Nq, S, c, (int)causal);
    // a single chunk wrote O and L itself
    if (S > 2 * kMergeBatch)
      hipLaunchKernelGGL((decode_merge_kernel<D, 4>), dim3(BH * Nq), dim3(D * 4), 0, stream, ws_m, ws_l, ws_o,
                         (bf16*)o, lse, Nq, S);
    else if (S > 1)
      hipLaunchKernelGGL((decode_merge_kernel<D, 1>), dim3(BH * Nq), dim3(D), 0, stream, ws_m, ws_l, ws_o,
                         (bf16*)o, lse, Nq, S);
  };
  auto by_chunk = [&](auto dq) {
    if (ch == 512) partial(dq, std::integral_constant<int, 512>{});
    else if (ch == 256) partial(dq, std::integral_constant<int, 256>{});
    else partial(dq, std::integral_constant<int, 128>{});
  };
  if (d == 64) by_chunk(std::integral_constant<int, 64>{});
  else by_chunk(std::integral_constant<int, 128>{});
  return hipGetLastError();
}

}  // namespace attn
