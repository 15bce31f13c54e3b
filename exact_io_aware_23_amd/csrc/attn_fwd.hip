// Fused exact attention forward for gfx950.
//
// What it computes (the pages, by title and section):
//   "What is Flash Attention?" (iania.ai video page), transcript 01:04: S = Q K^T
//   scaled, row softmax P, O = P V.  Transcript 02:38-03:44: one kernel, one Q
//   block kept on chip while K/V blocks stream through, only O written.
//   Transcript 04:15-05:17: the online softmax with a running max m and sum l,
//   the accumulator rescaled as each block arrives, and one division by l at
//   the end.  "Atencao exata ..." (mentria.ai), online-update formula: the
//   single-exponential form l_new = e^(m_old - m_new) l_old + sum e^(x - m_new)
//   used here.
//
// bf16 kernel design (MI355X, CDNA4):
//   * One workgroup = 4 waves = 128 query rows, 32 per wave; two workgroups
//     share a CU (229 VGPRs, two waves per SIMD), so one wave's softmax runs
//     while the other wave on the SIMD issues MFMAs.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T kept in
//     VGPRs for the whole loop).  In the S^T layout each lane owns one query
//     row, so the row max, the exp-sum and the O rescale stay lane-local; one
//     v_permlane32_swap joins the two lane halves for the max.
//   * O^T += V^T P^T: P^T comes straight from the S^T accumulators (rounded to
//     bf16); the V^T fragments come from the row-major V tile by transposing
//     LDS reads (ds_read_b64_tr_b16), so V needs no transpose on the way in.
//   * Softmax in base 2: p = exp2(s * scale * log2(e) - m) with one FMA and one
//     v_exp_f32 per score; L = (m + log2 l) ln 2 at the end.  The reference max
//     m moves only when a tile's max exceeds it by more than 2^8 (lazy
//     rescaling), so the O accumulators are rarely touched by the VALU.
//   * Global loads use raw buffer resources: per-lane offsets are
//     loop-invariant, the tile offset is a scalar, rows past N read as zero.
//   * K/V tiles of 64 keys are double-buffered in LDS and loaded by buffer ->
//     LDS transfers (no VGPRs, no LDS store instructions); the loads of tile
//     j+1 are in flight while tile j is computed.  One barrier per tile.
//   * Causal: key tiles past a query tile's last row are never loaded; a wave
//     skips the tiles past its own last row; only diagonal (and ragged tail)
//     tiles apply the mask.  Query tiles run longest first within a head, and
//     work items are renumbered so each XCD sweeps whole heads (L2 reuse).
#include "attn_common.h"
#include "attn_launch.h"

namespace attn {
namespace {

template <int D, int QB_>
struct FwdCfg {
  static constexpr int WAVES = 4;
  static constexpr int QB = QB_;             // 32-row query blocks per wave
  static constexpr int BR = WAVES * QB * 32; // query rows per workgroup
  static constexpr int BC = 64;              // keys per K/V tile
  static constexpr int NCH = D / 8;          // 16-byte chunks per K row
  static constexpr int KS = D / 16;          // k-steps of S^T = K Q^T
  static constexpr int DT = D / 32;          // 32-wide d tiles of O^T
  static constexpr int NKLD = BC * NCH / 256;
  static constexpr int K_ELEMS = BC * D;
  static constexpr int STAGE = 2 * BC * D;   // K and V, row-major
  // one wave per SIMD when a wave owns two query blocks (more VGPRs), two otherwise
  static constexpr int MIN_WAVES_PER_EU = QB == 1 ? 2 : 1;
};

// Lazy rescaling threshold (log2 units).  The running reference max m of a row
// is raised only when a tile's max exceeds it by more than this, so most
// tiles skip the O-accumulator rescale.  p = exp2(s*c - m) then stays below
// 2^kTau; the result is unchanged (the same m is used for O and l).
constexpr float kTau = 8.0f;

template <int D, bool CAUSAL, int QB>
__global__ void __launch_bounds__(256, (FwdCfg<D, QB>::MIN_WAVES_PER_EU))
fwd_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                bf16* __restrict__ O, float* __restrict__ L, int N, int n_qtiles, int total, float c) {
  using C = FwdCfg<D, QB>;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * C::STAGE];

  const int work = xcd_remap(blockIdx.x, total);
  const int bh = work / n_qtiles;
  const int qt = CAUSAL ? (n_qtiles - 1 - work % n_qtiles) : (work % n_qtiles);
  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const rsrc_t rQ = make_rsrc(Q + head, head_bytes);
  const rsrc_t rK = make_rsrc(K + head, head_bytes);
  const rsrc_t rV = make_rsrc(V + head, head_bytes);

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int q0w = qt * C::BR + wave * (C::QB * 32);

  // ---- tile ranges (all wave-uniform)
  const int kv_end = CAUSAL ? min(N, qt * C::BR + C::BR) : N;
  const int n_tiles = (kv_end + C::BC - 1) / C::BC;
  int wave_tiles = 0;
  if (q0w < N) {
    const int wend = CAUSAL ? min(N, q0w + C::QB * 32) : N;
    wave_tiles = (wend + C::BC - 1) / C::BC;
  }

  // ---- Q^T operand in registers: lane (l32, g) holds Q[q][16ks + 8g .. +7]
  bf16x8 qreg[C::QB][C::KS];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int qoff = ((q0w + 32 * qb + l32) * D + 8 * g) * 2;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qreg[qb][ks] = __builtin_bit_cast(bf16x8, bload16(rQ, qoff + 32 * ks, 0));
  }
  wait_vmem_all();  // Q is in registers before the loop: the loop never waits on it

  // K and V tiles go straight into LDS (row-major, XOR-swizzled 16-byte chunks):
  // wave `wave`, instruction i fills 1 KB block (wave * NKLD + i).
  int kvoff[C::NKLD];
#pragma unroll
  for (int i = 0; i < C::NKLD; ++i) {
    const int idx = (wave * C::NKLD + i) * 64 + lane;
    const int row = idx / C::NCH, cphys = idx % C::NCH;
    const int clog = cphys ^ (chunk_swz<C::NCH>(row));
    kvoff[i] = (row * D + 8 * clog) * 2;
  }
  auto load_tile = [&](int kv0, int stage) {
    const int soff = kv0 * D * 2;
    bf16* Ks = smem + stage * C::STAGE;
    bf16* Vs = Ks + C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::NKLD; ++i) {
      bload16_lds(rK, Ks + (wave * C::NKLD + i) * 512, kvoff[i], soff);
      bload16_lds(rV, Vs + (wave * C::NKLD + i) * 512, kvoff[i], soff);
    }
  };
  // V^T operand by transposing reads: lane l = 16 G + 4 r + c reads key row
  // 16 m + 8 g + r (+4 for the second half) at d columns 32 dt + 16 (G & 1) + 4 c;
  // with chunk_swz the element offset is (vbase[hh] ^ (32 dt)) + 16 m D
  int vbase[2];
  {
    const int li = lane & 15, G = lane >> 4;
    const int r = li >> 2, cc = li & 3;
    const int rr = D == 128 ? r : ((r >> 1) & 1);
    const int x = 2 * (G & 1) + (cc >> 1);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      vbase[hh] = (8 * g + r + 4 * hh) * D + 32 * rr + 8 * (x ^ (2 * g + hh)) + 4 * (cc & 1);
  }
  auto vt_tr = [&](const bf16* Vs, int dt, int m) {
    bf16x8 out;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4*)(Vs + ((vbase[hh] ^ (32 * dt)) + 16 * m * D)));
#pragma unroll
      for (int e = 0; e < 4; ++e) out[4 * hh + e] = v[e];
    }
    return out;
  };

  // per-lane LDS read offsets
  const int krow = swap23(l32);
  const int k_swz = chunk_swz<C::NCH>(krow);

  f32x16 oacc[C::QB][C::DT];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][dt][r] = 0.f;
  float m_run[C::QB], l_run[C::QB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    m_run[qb] = -1e30f;
    l_run[qb] = 0.f;
  }

  load_tile(0, 0);
  wait_vmem_all();
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int stage = j & 1;
    const int kv0 = j * C::BC;
    const bool has_next = j + 1 < n_tiles;
    if (has_next) load_tile(kv0 + C::BC, stage ^ 1);

    if (j < wave_tiles) {
      const bf16* Ks = smem + stage * C::STAGE;
      const bf16* Vs = Ks + C::K_ELEMS;
      // ---- S^T = K Q^T
      f32x16 st[C::QB][2];
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) st[qb][kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 a = lds_read16(Ks + (32 * kb + krow) * D, (2 * ks + g) ^ k_swz);
#pragma unroll
          for (int qb = 0; qb < C::QB; ++qb) st[qb][kb] = mfma32(a, qreg[qb][ks], st[qb][kb]);
        }
      }
      // ---- mask (diagonal / ragged tiles only)
      const bool need_mask = (kv0 + C::BC > N) || (CAUSAL && kv0 + C::BC - 1 > q0w);
      if (need_mask) {
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb) {
          const int q = q0w + 32 * qb + l32;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kv0 + 32 * kb + crow(r, g);
              const bool bad = (key >= N) || (CAUSAL && key > q);
              st[qb][kb][r] = bad ? -INFINITY : st[qb][kb][r];
            }
        }
      }
      // ---- online softmax (base 2), lane-local per query row, lazy rescale
      bf16x8 pop[C::QB][4];
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[qb][kb][r]);
        const float mt = pair_max(mx) * c;
        if (__builtin_amdgcn_ballot_w64(mt > m_run[qb] + kTau) != 0) {
          const float m_new = fmaxf(m_run[qb], mt);
          const float alpha = fast_exp2(m_run[qb] - m_new);
          m_run[qb] = m_new;
          l_run[qb] *= alpha;
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][dt][r] *= alpha;
        }
        const float mneg = -m_run[qb];
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(st[qb][kb][r], c, mneg));
            st[qb][kb][r] = p;
            rs += p;
          }
        l_run[qb] += rs;
#pragma unroll
        for (int m = 0; m < 4; ++m) pop[qb][m] = c_to_operand(st[qb][m >> 1], m & 1);
      }
      // ---- O^T += V^T P^T (V^T fragments by transposing LDS reads)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const bf16x8 a = vt_tr(Vs, dt, m);
#pragma unroll
          for (int qb = 0; qb < C::QB; ++qb) oacc[qb][dt] = mfma32(a, pop[qb][m], oacc[qb][dt]);
        }
      }
    }

    wait_vmem_all();
    __syncthreads();
  }

  // ---- epilogue: O = O_acc / l, L = (m + log2 l) ln 2
  bf16* Oh = O + head;
  float* Lh = L + (size_t)bh * N;
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int q = q0w + 32 * qb + l32;
    const float lt = pair_sum(l_run[qb]);
    if (q < N) {
      const float inv = 1.0f / lt;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int dcol = 32 * dt + 8 * a + 4 * g;
          u32x2 w;
          w[0] = pack_bf16x2(oacc[qb][dt][4 * a + 0] * inv, oacc[qb][dt][4 * a + 1] * inv);
          w[1] = pack_bf16x2(oacc[qb][dt][4 * a + 2] * inv, oacc[qb][dt][4 * a + 3] * inv);
          *reinterpret_cast<u32x2*>(Oh + (size_t)q * D + dcol) = w;
        }
      if (g == 0) Lh[q] = (m_run[qb] + log2f(lt)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 forward: the same online-softmax algorithm on plain fp32 VALU
// arithmetic.  One thread owns one query row (q and the O accumulator in
// VGPRs); 32-key K/V tiles are staged in LDS and read as broadcasts.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64)
fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
               float* __restrict__ O, float* __restrict__ L, int N, int n_qtiles, float c) {
  constexpr int BC = 32;
  __shared__ float Ks[BC][D];
  __shared__ float Vs[BC][D];
  const int bh = blockIdx.x / n_qtiles;
  const int qt = blockIdx.x % n_qtiles;
  const size_t head = (size_t)bh * N * D;
  const int q = qt * 64 + threadIdx.x;
  const bool qv = q < N;

  float qr[D], acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    qr[i] = qv ? Q[head + (size_t)q * D + i] : 0.f;
    acc[i] = 0.f;
  }
  float m_run = -1e30f, l_run = 0.f;
  const int kv_end = CAUSAL ? min(N, qt * 64 + 64) : N;
  for (int kv0 = 0; kv0 < kv_end; kv0 += BC) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < BC * D; idx += 64) {
      const int row = idx / D, col = idx % D;
      const int key = kv0 + row;
      Ks[row][col] = key < N ? K[head + (size_t)key * D + col] : 0.f;
      Vs[row][col] = key < N ? V[head + (size_t)key * D + col] : 0.f;
    }
    __syncthreads();
    float s[BC];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) dot = fmaf(qr[i], Ks[j][i], dot);
      const int key = kv0 + j;
      const bool bad = key >= N || (CAUSAL && key > q);
      s[j] = bad ? -INFINITY : dot;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) acc[i] *= alpha;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      const float p = exp2f(fmaf(s[j], c, -m_new));
      rs += p;
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] = fmaf(p, Vs[j][i], acc[i]);
    }
    l_run = l_run * alpha + rs;
  }
  if (qv) {
    const float inv = 1.0f / l_run;
#pragma unroll
    for (int i = 0; i < D; ++i) O[head + (size_t)q * D + i] = acc[i] * inv;
    L[(size_t)bh * N + q] = (m_run + log2f(l_run)) * kLn2;
  }
}

constexpr int kFwdQB = 1;  // query blocks of 32 rows per wave

template <int D, bool CAUSAL>
hipError_t launch_fwd_bf16_t(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                             int N, float scale, hipStream_t stream) {
  using C = FwdCfg<D, kFwdQB>;
  const int n_qtiles = (N + C::BR - 1) / C::BR;
  const int total = BH * n_qtiles;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, kFwdQB>), dim3(total), dim3(256), 0, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse, N, n_qtiles, total,
                     scale * kLog2e);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_f32_t(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                            int N, float scale, hipStream_t stream) {
  const int n_qtiles = (N + 63) / 64;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(BH * n_qtiles), dim3(64), 0, stream,
                     (const float*)q, (const float*)k, (const float*)v, (float*)o, lse, N, n_qtiles,
                     scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N,
                      int d, bool bf16_in, float scale, bool causal, hipStream_t stream) {
  if (bf16_in) {
    if (d == 64) return causal ? launch_fwd_bf16_t<64, true>(q, k, v, o, lse, BH, N, scale, stream)
                               : launch_fwd_bf16_t<64, false>(q, k, v, o, lse, BH, N, scale, stream);
    return causal ? launch_fwd_bf16_t<128, true>(q, k, v, o, lse, BH, N, scale, stream)
                  : launch_fwd_bf16_t<128, false>(q, k, v, o, lse, BH, N, scale, stream);
  }
  if (d == 64) return causal ? launch_fwd_f32_t<64, true>(q, k, v, o, lse, BH, N, scale, stream)
                             : launch_fwd_f32_t<64, false>(q, k, v, o, lse, BH, N, scale, stream);
  return causal ? launch_fwd_f32_t<128, true>(q, k, v, o, lse, BH, N, scale, stream)
                : launch_fwd_f32_t<128, false>(q, k, v, o, lse, BH, N, scale, stream);
}

}  // namespace attn
