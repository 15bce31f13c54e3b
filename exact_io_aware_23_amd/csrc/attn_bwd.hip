// Exact attention backward for gfx950: recompute P tile by tile from Q, K and
// the saved row logsumexp L; never store an N x N array.
//
// The pages: "What is Flash Attention?" (iania.ai video page), transcript
// 06:52-07:24: the forward keeps only O and per-row statistics, and the
// backward rebuilds P block by block with the same tiling loop.  Transcript
// 08:26: the gradients are those of the exact function.  The formulas below
// are the calculus of O = softmax(S) V, S = scale Q K^T + mask (the pages do
// not print them):
//   P = exp(S - L)            (L_i = logsumexp of row i, saved by the forward)
//   dV = P^T dO, dP = dO V^T, delta_i = sum_k dO_ik O_ik = sum_j P_ij dP_ij,
//   dS = P * (dP - delta),   dQ = scale dS K,   dK = scale dS^T Q.
//
// Three kernels on one stream:
//   preprocess : delta = rowsum(dO * O), fp32.
//   dkdv       : a workgroup owns 128 keys (32 per wave): K as MFMA operands in
//                VGPRs, V in LDS (read once from memory), and streams 32-query
//                blocks of Q and dO into LDS by buffer -> LDS copies.  Four
//                MFMA products per block: S, dP, dV^T += dO^T P and
//                dK^T += Q^T dS, the dO^T and Q^T operands coming from the
//                row-major tiles by transposing LDS reads.  dK, dV accumulate
//                in fp32 registers; two workgroups share a CU.
//   dq         : a workgroup keeps 128 queries (32 per wave) of Q and dO in
//                VGPRs and streams 32-key tiles of K and V into LDS by buffer
//                -> LDS copies.  Three products per tile: S^T = K Q^T,
//                dP^T = V dO^T and dQ^T += K^T dS^T, the K^T operand by
//                transposing LDS reads.  No atomics, so dQ is deterministic;
//                two workgroups per CU.  On the way it sums delta exactly.
// Precision of delta: rowsum(dO * O) with O as stored (bf16) differs from the
// exact sum_j P_ij dP_ij by about 2^-9 |dO| |O|, and dP - delta cancels when a
// row's P is nearly one-hot, so that error passes into dS almost unreduced.
// In dQ = scale dS K it is multiplied by K and stays well inside the bf16
// tolerance, so the dq kernel uses delta~ = rowsum(dO * O) as the backward
// defines it.  In dK = scale dS^T Q it is multiplied by Q, and a query row of
// large norm carries it into dK at full size; so the dq kernel also sums
// delta = sum_j P_ij dP_ij in fp32 from the same P and dP it forms, and dkdv
// runs after it with that exact delta.  Order: preprocess -> dq -> dkdv.
// Both recompute P with p = exp2(s * scale * log2 e - L * log2 e).
#include <mutex>
#include <type_traits>

#include "attn_common.h"
#include "attn_launch.h"

namespace attn {
namespace {


// ------------------------------------------------------------------ preprocess
template <int D>
__global__ void __launch_bounds__(256)
bwd_preprocess_kernel(const bf16* __restrict__ O, const bf16* __restrict__ dO, float* __restrict__ delta,
                      int rows) {
  constexpr int TPR = D / 8;  // threads per row, 16 bytes each
  const int row = blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float s = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(O + (size_t)row * D + 8 * part);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dO + (size_t)row * D + 8 * part);
    const bf16x8 av = __builtin_bit_cast(bf16x8, a);
    const bf16x8 bv = __builtin_bit_cast(bf16x8, b);
#pragma unroll
    for (int i = 0; i < 8; ++i) s = fmaf((float)av[i], (float)bv[i], s);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, TPR);
  if (row < rows && part == 0) delta[row] = s;
}

// ------------------------------------------------------------------ dK, dV
// QSPLIT: the four waves are two 32-key groups times two query halves (wave w
// owns keys 32 (w % 2).. of the workgroup's 64 and the query block of parity
// w / 2 in every 64-query step), and the two halves' partial dK, dV are added
// through LDS at the end.  Each wave runs half as many steps and there are
// twice as many waves, so a launch that would leave its last round of
// workgroups one per SIMD splits more evenly.
template <int D, bool QSPLIT = false>
struct DkdvCfg {
  static constexpr int KG = QSPLIT ? 2 : 4;          // key groups of 32 per workgroup
  static constexpr int QH = QSPLIT ? 2 : 1;          // 32-query blocks per step, one per wave row
  static constexpr int BKV = 32 * KG;                // keys per workgroup
  static constexpr int BQ = 32;                      // queries per wave per step
  static constexpr int NCH = D / 8;
  static constexpr int KS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int QTILE = QH * BQ * D;          // bf16 elements of one step's Q (or dO) rows
  static constexpr int NB = QTILE * 2 / 1024 / 4;    // 1 KB transfers per wave per tile
  static constexpr int NBV = BKV * D * 2 / 1024 / 4; // 1 KB transfers per wave for the V block
  // LDS (bf16 elements): V block [BKV][D] | 2 stages x (Q [QH BQ][D], dO [QH BQ][D]) | 2 stages x (L', D) fp32
  static constexpr int V_ELEMS = BKV * D;
  static constexpr int STAGE = 2 * QTILE;
  static constexpr int NSTAT = 2 * QH * BQ;          // floats of statistics per stage
  static constexpr int BYTES = (V_ELEMS + 2 * STAGE) * 2 + 2 * NSTAT * 4;
};

// A operand of a product contracting over rows of a row-major [rows][D] LDS
// tile (lane = d column 32 dt + l%32, k slots (l/32, e) = rows 16 h + 8 (l/32) + e),
// by two transposing reads.  Lane l = 16 G + 4 r + c reads row 16 h + 8 g + r
// (+4 for the second read) at columns 32 dt + 16 (G & 1) + 4 c .. +3.
// With chunk_swz the element offset of that read is
//   (base[hh] ^ (32 dt)) + 16 h D,
// base[hh] = (8 g + r + 4 hh) D + 32 r' + 8 ((2 (G & 1) + c / 2) ^ (2 g + hh)) + 4 (c & 1),
// r' = r (D = 128) or (r / 2) & 1 (D = 64): the column group term occupies bits
// the row offset leaves zero, so one v_xor per read addresses any dt.
template <int D>
struct TrBase {
  int b[2];
  __device__ __forceinline__ explicit TrBase(int lane) {
    const int li = lane & 15, G = lane >> 4, g = lane >> 5;
    const int r = li >> 2, c = li & 3;
    const int rr = D == 128 ? r : ((r >> 1) & 1);
    const int x = 2 * (G & 1) + (c >> 1);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) b[hh] = (8 * g + r + 4 * hh) * D + 32 * rr + 8 * (x ^ (2 * g + hh)) + 4 * (c & 1);
  }
};
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const bf16* tile, int dt, int h, const TrBase<D>& tb) {
  bf16x8 out;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4*)(tile + ((tb.b[hh] ^ (32 * dt)) + 16 * h * D)));
#pragma unroll
    for (int e = 0; e < 4; ++e) out[4 * hh + e] = v[e];
  }
  return out;
}

// PAIR: each workgroup runs two key blocks of one head, p and n - 1 - p
// (pair_work), so causal workgroups all do the same work.
template <int D, bool CAUSAL, bool SPARSE, bool DROP, bool PAIR = false, bool QSPLIT = false>
__global__ void __launch_bounds__(256, 2)
bwd_dkdv_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                const float* __restrict__ Lse, const bf16* __restrict__ dO, const float* __restrict__ Delta,
                bf16* __restrict__ dK, bf16* __restrict__ dV, int N, int n_ktiles, int total, float c,
                float scale, const uint8_t* __restrict__ Mask, int mask_hs, int nb, uint32_t drop_t,
                uint32_t seed_lo, uint32_t seed_hi, float inv_keep, uint32_t smode) {
  using C = DkdvCfg<D, QSPLIT>;
  static_assert(!(SPARSE && DROP), "block-sparse and dropout are separate entry points");
  static_assert(!QSPLIT || (!SPARSE && !DROP && !PAIR), "the query split serves the dense kernel");
  __shared__ __attribute__((aligned(16))) char smem[C::BYTES];
  // block-sparse: the query blocks of this key block whose 128 x 128 block is on
  __shared__ uint16_t qlist[SPARSE ? kMaxSparseN / C::BQ : 1];
  __shared__ int wcnt[SPARSE ? 4 : 1];
  bf16* Vs = reinterpret_cast<bf16*>(smem);
  bf16* Xs = Vs + C::V_ELEMS;                                          // stage s: Q at s*STAGE, dO after
  float* Fs = reinterpret_cast<float*>(smem + (C::V_ELEMS + 2 * C::STAGE) * 2);  // stage s: L' [32], delta [32]

#pragma nounroll
  for (int item = 0; item < (PAIR ? 2 : 1); ++item) {
  const int work = PAIR ? pair_work(blockIdx.x, total, n_ktiles, item) : xcd_remap(blockIdx.x, total);
  const int bh = work / n_ktiles;
  const int kt = work % n_ktiles;
  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const rsrc_t rQ = make_rsrc(Q + head, head_bytes);
  const rsrc_t rK = make_rsrc(K + head, head_bytes);
  const rsrc_t rV = make_rsrc(V + head, head_bytes);
  const rsrc_t rdO = make_rsrc(dO + head, head_bytes);
  const rsrc_t rL = make_rsrc(Lse + (size_t)bh * N, (uint32_t)N * 4);
  const rsrc_t rD = make_rsrc(Delta + (size_t)bh * N, (uint32_t)N * 4);

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int k0 = kt * C::BKV;
  const int kw0 = k0 + 32 * (wave % C::KG);
  const int qh = QSPLIT ? wave / C::KG : 0;  // this wave's query block within a step
  const int key = kw0 + l32;

  // ---- K^T operand in VGPRs (lane = key, 8 consecutive d per k-step); V block into LDS
  bf16x8 kreg[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    kreg[ks] = sign_bf16x8(__builtin_bit_cast(bf16x8, bload16(rK, (key * D + 16 * ks + 8 * g) * 2, 0)), smode);
  // buffer -> LDS copies: 1 KB block b of a [rows][D] tile gets 16-byte chunk
  // idx = 64 b + lane, stored at its swizzled position
  auto tile_off = [&](int b) {
    const int idx = b * 64 + lane;
    const int row = idx / C::NCH, cphys = idx % C::NCH;
    return (row * D + 8 * (cphys ^ chunk_swz<C::NCH>(row))) * 2;
  };
#pragma unroll
  for (int i = 0; i < C::NBV; ++i) {
    const int b = wave * C::NBV + i;
    bload16_lds(rV, Vs + b * 512, tile_off(b), k0 * D * 2);
  }
  int qoff[C::NB];
#pragma unroll
  for (int i = 0; i < C::NB; ++i) qoff[i] = tile_off(wave * C::NB + i);
  float stat = 0.f;  // tid < 32: L' of query q0 + tid; 32 <= tid < 64: delta
  auto load_q = [&](int q0, int stage) {
    bf16* Qs = Xs + stage * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::NB; ++i) {
      const int b = wave * C::NB + i;
      bload16_lds(rQ, Qs + b * 512, qoff[i], q0 * D * 2);
      bload16_lds(rdO, Qs + C::QTILE + b * 512, qoff[i], q0 * D * 2);
    }
    constexpr int R = C::QH * C::BQ;  // query rows per step
    if (tid < R) {
      // a row with no allowed key (L = -inf) gets p = exp2(-inf) = 0
      const float lrow = __uint_as_float(bload4(rL, (q0 + tid) * 4, 0));
      stat = lrow == -INFINITY ? INFINITY : lrow * kLog2e;
    }
    else if (tid < 2 * R) stat = __uint_as_float(bload4(rD, (q0 + tid - R) * 4, 0));
  };
  auto store_stat = [&](int stage) {
    if (tid < C::NSTAT) Fs[stage * C::NSTAT + tid] = stat;
  };

  const int a_row = swap23(l32);
  const int a_swz = chunk_swz<C::NCH>(a_row);
  const TrBase<D> trb(lane);
  const int v_row = 32 * (wave % C::KG) + l32;
  const int v_swz = chunk_swz<C::NCH>(v_row);

  f32x16 dk[C::DT], dv[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[dt][r] = 0.f;
      dv[dt][r] = 0.f;
    }

  const int n_qt = (N + C::BQ - 1) / C::BQ;
  const int qt_begin = CAUSAL ? (k0 / C::BQ) : 0;
  // the workgroup visits query blocks it_of(0), it_of(1), ... (n_it of them;
  // with QSPLIT, steps of two blocks)
  int n_it = max((n_qt - qt_begin + C::QH - 1) / C::QH, 0);
  if constexpr (SPARSE) {
    // query block t holds rows [32 t, 32 t + 32), in block row t / 4; this is block column kt
    const uint8_t* mcol = Mask + (size_t)bh * mask_hs + kt;
    n_it = uniform(compact_indices(qlist, wcnt, qt_begin, n_qt,
                                   [&](int t) { return mcol[(size_t)(t >> 2) * nb] != 0; }));
  }
  auto it_of = [&](int idx) -> int {
    if constexpr (SPARSE) return uniform((int)qlist[idx]);
    else return qt_begin + C::QH * idx;
  };
  // first rows of query blocks idx and idx+1, carried from iteration to
  // iteration; a block-sparse iteration reads the list entry for idx+2 early
  // and makes it scalar only after its barrier
  int q_cur = n_it > 0 ? it_of(0) * C::BQ : 0;
  int q_nxt = n_it > 1 ? it_of(1) * C::BQ : 0;
  if (n_it > 0) load_q(q_cur, 0);
  wait_vmem_all();
  store_stat(0);
  __syncthreads();

  for (int idx = 0; idx < n_it; ++idx) {
    int raw2 = 0;
    if constexpr (SPARSE) raw2 = qlist[min(idx + 2, kMaxSparseN / C::BQ - 1)];
    const int stage = idx & 1;
    const int q0 = q_cur + C::BQ * qh;  // this wave's query block
    const bool has_next = idx + 1 < n_it;
    if (has_next) load_q(q_nxt, stage ^ 1);

    const bool active = kw0 < N && (!QSPLIT || q0 < N) && !(CAUSAL && q0 < kw0);
    if (active) {
      const bf16* Qs = Xs + stage * C::STAGE + C::BQ * D * qh;
      const bf16* dOs = Qs + C::QTILE;
      const float* Ls = Fs + stage * C::NSTAT + C::BQ * qh;
      const float* Ds = Ls + C::QH * C::BQ;
      // ---- S = Q K^T and dP = dO V^T
      // Each MFMA's operands are read one MFMA ahead; sched_barrier fences
      // the steps so the compiler cannot pull the reads down to their use.
      f32x16 s, dp;
      bf16x8 aq = lds_read16(Qs + a_row * D, g ^ a_swz);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 ao = lds_read16(dOs + a_row * D, (2 * ks + g) ^ a_swz);
        const bf16x8 bv = lds_read16(Vs + v_row * D, (2 * ks + g) ^ v_swz);
        __builtin_amdgcn_sched_barrier(0);
        s = mfma32(aq, kreg[ks], ks == 0 ? f32x16{} : s);
        __builtin_amdgcn_sched_barrier(0);
        if (ks + 1 < C::KS) aq = lds_read16(Qs + a_row * D, (2 * ks + 2 + g) ^ a_swz);
        __builtin_amdgcn_sched_barrier(0);
        dp = mfma32(ao, bv, ks == 0 ? f32x16{} : dp);
        __builtin_amdgcn_sched_barrier(0);
      }
      // ---- P = exp2(s c - L'), dS = P (dP - delta); query of register r: crow(r, g)
      // masked scores become -inf, so exp2 gives exactly 0 (one branch per tile)
      const bool need_mask = (kw0 + 32 > N) || (CAUSAL && q0 == kw0);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = q0 + crow(r, g);
          const bool bad = (key >= N) || (CAUSAL && key > q);
          s[r] = bad ? -INFINITY : s[r];
        }
      }
      // dropout: dP = Z dO V^T / (1 - rate) and the dV operand is Z P / (1 - rate)
      bool kept[16];
      if constexpr (DROP) {
        uint32_t word[4];
        drop_words_col(key, q0, g, bh, seed_lo, seed_hi, word);
#pragma unroll
        for (int r = 0; r < 16; ++r) kept[r] = drop_keep(word, r, drop_t);
      }
      if constexpr (DROP) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int v4 = 0; v4 < 2; ++v4) {
            const f32x4 lv = *reinterpret_cast<const f32x4*>(Ls + 16 * h + 8 * g + 4 * v4);
            const f32x4 dv4 = *reinterpret_cast<const f32x4*>(Ds + 16 * h + 8 * g + 4 * v4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 8 * h + 4 * v4 + i;
              const float p = fast_exp2(fmaf(s[r], c, -lv[i]));
              const float dpr = kept[r] ? dp[r] * inv_keep : 0.f;
              s[r] = kept[r] ? p * inv_keep : 0.f;
              dp[r] = p * (dpr - dv4[i]);
            }
          }
        // ---- dV^T += dO^T P and dK^T += Q^T dS (A operands by transposing reads)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16x8 pop = c_to_operand(s, h);
          const bf16x8 dso = c_to_operand(dp, h);
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt) {
            dv[dt] = mfma32(tr_operand<D>(dOs, dt, h, trb), pop, dv[dt]);
            dk[dt] = mfma32(tr_operand<D>(Qs, dt, h, trb), dso, dk[dt]);
          }
        }
      } else {
        // The elementwise work of the first half (registers r < 8), then the
        // dV / dK MFMAs in a fixed order: each one's transposing reads are
        // issued one MFMA ahead, and the second half's elementwise work is
        // spread over the first half's MFMAs (sched_barrier fences the steps).
        auto stat4 = [&](const float* base, int r) {
          return *reinterpret_cast<const f32x4*>(base + 16 * (r / 8) + 8 * g + 4 * ((r / 4) % 2));
        };
        auto elem = [&](int r, const f32x4& lv, const f32x4& dl) {
          const float p = fast_exp2(fmaf(s[r], c, -lv[r % 4]));
          s[r] = p;
          dp[r] = p * (dp[r] - dl[r % 4]);
        };
        f32x4 la = stat4(Ls, 0), da = stat4(Ds, 0), lb = stat4(Ls, 4), db = stat4(Ds, 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) elem(r, la, da);
#pragma unroll
        for (int r = 4; r < 8; ++r) elem(r, lb, db);
        la = stat4(Ls, 8);
        da = stat4(Ds, 8);
        lb = stat4(Ls, 12);
        db = stat4(Ds, 12);
        bf16x8 pop = c_to_operand(s, 0), dso = c_to_operand(dp, 0);
        // MFMA i: dV (i even) or dK (i odd), d tile (i / 2) % DT, half i / (2 DT)
        constexpr int NM = 4 * C::DT;
        constexpr int EPM = 8 / (2 * C::DT);  // second-half elements per first-half MFMA
        auto operand = [&](int i) {
          return tr_operand<D>((i & 1) ? Qs : dOs, (i / 2) % C::DT, i / (2 * C::DT), trb);
        };
        bf16x8 nxt = operand(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          const bf16x8 cur = nxt;
          if (i + 1 < NM) nxt = operand(i + 1);
          __builtin_amdgcn_sched_barrier(0);
          if (i == 2 * C::DT) {
            pop = c_to_operand(s, 1);
            dso = c_to_operand(dp, 1);
          }
          const int dt = (i / 2) % C::DT;
          if (i & 1) dk[dt] = mfma32(cur, dso, dk[dt]);
          else dv[dt] = mfma32(cur, pop, dv[dt]);
          if (i < 2 * C::DT) {
#pragma unroll
            for (int e = 0; e < EPM; ++e) {
              const int r = 8 + EPM * i + e;
              if (r < 12) elem(r, la, da);
              else elem(r, lb, db);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    if (has_next) {
      wait_vmem_all();  // the next tile has landed in LDS and its statistics in `stat`
      store_stat(stage ^ 1);
    }
    __syncthreads();
    q_cur = q_nxt;
    if constexpr (SPARSE) q_nxt = idx + 2 < n_it ? uniform(raw2) * C::BQ : 0;
    else q_nxt = (qt_begin + C::QH * (idx + 2)) * C::BQ;
  }

  if constexpr (QSPLIT) {
    // the second query half hands its partial dK, dV to the first through LDS
    // (free after the loop's last barrier): chunk j of the 2 DT 4 float4s a lane
    // holds goes to float4 slot (kg (2 DT 4) + j) 64 + lane, conflict-free
    constexpr int NQ = 2 * C::DT * 4;
    f32x4* xch = reinterpret_cast<f32x4*>(smem) + (wave % C::KG) * NQ * 64 + lane;
    if (qh == 1) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          xch[(dt * 4 + a) * 64] = f32x4{dk[dt][4 * a], dk[dt][4 * a + 1], dk[dt][4 * a + 2], dk[dt][4 * a + 3]};
          xch[((C::DT + dt) * 4 + a) * 64] =
              f32x4{dv[dt][4 * a], dv[dt][4 * a + 1], dv[dt][4 * a + 2], dv[dt][4 * a + 3]};
        }
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 pk = xch[(dt * 4 + a) * 64], pv = xch[((C::DT + dt) * 4 + a) * 64];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dk[dt][4 * a + e] += pk[e];
            dv[dt][4 * a + e] += pv[e];
          }
        }
    }
  }

  // ---- epilogue: dK = scale * (dK^T)^T, dV = (dV^T)^T
  if (key < N && qh == 0) {
    bf16* dKh = dK + head + (size_t)key * D;
    bf16* dVh = dV + head + (size_t)key * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int dcol = 32 * dt + 8 * a + 4 * g;
        u32x2 wk, wv;
        wk[0] = pack_bf16x2(dk[dt][4 * a + 0] * scale, dk[dt][4 * a + 1] * scale);
        wk[1] = pack_bf16x2(dk[dt][4 * a + 2] * scale, dk[dt][4 * a + 3] * scale);
        wv[0] = pack_bf16x2(dv[dt][4 * a + 0], dv[dt][4 * a + 1]);
        wv[1] = pack_bf16x2(dv[dt][4 * a + 2], dv[dt][4 * a + 3]);
        *reinterpret_cast<u32x2*>(dKh + dcol) = wk;
        *reinterpret_cast<u32x2*>(dVh + dcol) = wv;
      }
  }
  if (PAIR) __syncthreads();  // every wave is done with this block's LDS before the next block's copies
  }
}

// ------------------------------------------------------------------ dQ
template <int D>
struct DqCfg {
  static constexpr int BRQ = 128;  // queries per workgroup, 32 per wave
  static constexpr int BC = 32;    // keys per tile
  static constexpr int NCH = D / 8;
  static constexpr int KS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int TILE = BC * D;                // bf16 elements of one K or V tile
  static constexpr int NB = TILE * 2 / 1024 / 4;     // 1 KB transfers per wave per tile
  static constexpr int STAGE = 2 * TILE;             // K then V, row-major, swizzled
};

// PAIR: each workgroup runs two query tiles of one head, p and n - 1 - p
// (pair_work), so causal workgroups all do the same work.
template <int D, bool CAUSAL, bool SPARSE, bool DROP, bool PAIR = false>
__global__ void __launch_bounds__(256, 2)
bwd_dq_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
              const float* __restrict__ Lse, const bf16* __restrict__ dO, const float* __restrict__ Delta,
              const bf16* __restrict__ Ofused, bf16* __restrict__ dQ, float* __restrict__ DeltaOut, int N, int n_qtiles, int total, float c,
              float scale, const uint8_t* __restrict__ Mask, int mask_hs, int nb, uint32_t drop_t,
              uint32_t seed_lo, uint32_t seed_hi, float inv_keep, uint32_t smode) {
  using C = DqCfg<D>;
  static_assert(!(SPARSE && DROP), "block-sparse and dropout are separate entry points");
  // one array per stage: the compiler then knows that reads of one stage do
  // not alias the buffer -> LDS copies into the other, and does not wait for
  // those copies before the reads
  __shared__ __attribute__((aligned(16))) bf16 kv_lds0[C::STAGE];
  __shared__ __attribute__((aligned(16))) bf16 kv_lds1[C::STAGE];
  auto stage_lds = [&](int stage) -> bf16* { return stage ? kv_lds1 : kv_lds0; };
  // block-sparse: the key tiles of this query block whose 128 x 128 block is on
  __shared__ uint16_t tlist[SPARSE ? kMaxSparseN / C::BC : 1];
  __shared__ int wcnt[SPARSE ? 4 : 1];

  for (int item = 0; item < (PAIR ? 2 : 1); ++item) {
  const int work = PAIR ? pair_work(blockIdx.x, total, n_qtiles, item) : xcd_remap(blockIdx.x, total);
  const int bh = work / n_qtiles;
  const int qt = CAUSAL ? (n_qtiles - 1 - work % n_qtiles) : (work % n_qtiles);
  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const rsrc_t rQ = make_rsrc(Q + head, head_bytes);
  const rsrc_t rK = make_rsrc(K + head, head_bytes);
  const rsrc_t rV = make_rsrc(V + head, head_bytes);
  const rsrc_t rdO = make_rsrc(dO + head, head_bytes);

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int q0w = qt * C::BRQ + 32 * wave;
  const int q = q0w + l32;

  // ---- Q^T and dO^T operands in VGPRs (lane = query, 8 consecutive d per k-step)
  bf16x8 qreg[C::KS], doreg[C::KS];
  const int qoff = (q * D + 8 * g) * 2;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    qreg[ks] = sign_bf16x8(__builtin_bit_cast(bf16x8, bload16(rQ, qoff + 32 * ks, 0)), smode);
    doreg[ks] = __builtin_bit_cast(bf16x8, bload16(rdO, qoff + 32 * ks, 0));
  }
  // rows past N, and rows with no allowed key (L = -inf), get p = exp2(-inf) = 0
  const float lrow = q < N ? Lse[(size_t)bh * N + q] : -INFINITY;
  const float lq = lrow == -INFINITY ? INFINITY : lrow * kLog2e;
  // delta~ = rowsum(dO * O) with O as stored: read from Delta (written by the
  // preprocess kernel) or, when O is passed, formed here in that kernel's
  // exact summation order (an FMA chain over each 16-byte chunk, then the same
  // pairwise tree over the chunks), so both routes give the same bits
  float dq_delta = 0.f;
  if (Ofused != nullptr) {
    const rsrc_t rO = make_rsrc(Ofused + head, head_bytes);
    float cs[C::KS];  // chunk 2 ks + g of the row
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 ov = __builtin_bit_cast(bf16x8, bload16(rO, qoff + 32 * ks, 0));
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf((float)ov[e], (float)doreg[ks][e], s);
      cs[ks] = s;
    }
    float half;  // this lane half's chunks (even or odd), in the preprocess kernel's tree
    if constexpr (D == 128) half = ((cs[0] + cs[4]) + (cs[2] + cs[6])) + ((cs[1] + cs[5]) + (cs[3] + cs[7]));
    else half = (cs[0] + cs[2]) + (cs[1] + cs[3]);
    const float full = pair_sum(half);
    dq_delta = q < N ? full : 0.f;
  } else {
    dq_delta = q < N ? Delta[(size_t)bh * N + q] : 0.f;
  }
  float d_exact = 0.f;  // this lane's share of sum_j P_qj dP_qj

  const int kv_end = CAUSAL ? min(N, qt * C::BRQ + C::BRQ) : N;
  int n_tiles = (kv_end + C::BC - 1) / C::BC;
  int wave_tiles = 0;
  if (q0w < N) wave_tiles = CAUSAL ? (min(N, q0w + 32) + C::BC - 1) / C::BC : n_tiles;
  if constexpr (SPARSE) {
    // key tile t holds keys [32 t, 32 t + 32), in block t / 4 of the block row qt
    const uint8_t* mrow = Mask + (size_t)bh * mask_hs + (size_t)qt * nb;
    n_tiles = uniform(compact_indices(tlist, wcnt, 0, n_tiles, [&](int t) { return mrow[t >> 2] != 0; }));
    wave_tiles = uniform(count_below(tlist, n_tiles, wave_tiles));
  }
  wait_vmem_all();  // Q, dO, L and delta are in registers (the mask loads overlapped them)
  auto kv0_of = [&](int j) -> int {
    if constexpr (SPARSE) return uniform((int)tlist[j]) * C::BC;
    else return j * C::BC;
  };

  // buffer -> LDS copies of the K and V tiles (1 KB block b gets chunk 64 b + lane)
  int toff[C::NB];
#pragma unroll
  for (int i = 0; i < C::NB; ++i) {
    const int idx = (wave * C::NB + i) * 64 + lane;
    const int row = idx / C::NCH, cphys = idx % C::NCH;
    toff[i] = (row * D + 8 * (cphys ^ chunk_swz<C::NCH>(row))) * 2;
  }
  auto load_tile = [&](int kv0, int stage) {
    bf16* Ks = stage_lds(stage);
#pragma unroll
    for (int i = 0; i < C::NB; ++i) {
      const int b = wave * C::NB + i;
      bload16_lds(rK, Ks + b * 512, toff[i], kv0 * D * 2);
      bload16_lds(rV, Ks + C::TILE + b * 512, toff[i], kv0 * D * 2);
    }
  };

  const int a_row = swap23(l32);
  const int a_swz = chunk_swz<C::NCH>(a_row);
  const TrBase<D> trb(lane);

  f32x16 dq[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dq[dt][r] = 0.f;
    }

  // first keys of tiles j and j+1, carried from iteration to iteration; a
  // block-sparse iteration reads the list entry for j+2 early and makes it
  // scalar only after its barrier, when no other LDS read is outstanding
  int kv_cur = n_tiles > 0 ? kv0_of(0) : 0;
  int kv_nxt = n_tiles > 1 ? kv0_of(1) : 0;
  if (n_tiles > 0) load_tile(kv_cur, 0);
  wait_vmem_all();
  __syncthreads();

  // iteration j works on stage j & 1, passed as a constant (the loop is
  // unrolled by two) so every LDS access names one array
  auto iter = [&](int j, auto stage_c) {
    constexpr int stage = decltype(stage_c)::value;
    int raw2 = 0;
    if constexpr (SPARSE) raw2 = tlist[min(j + 2, kMaxSparseN / C::BC - 1)];
    const int kv0 = kv_cur;
    if (j + 1 < n_tiles) load_tile(kv_nxt, stage ^ 1);

    if (j < wave_tiles) {
      const bf16* Ks = stage_lds(stage);
      const bf16* Vs = Ks + C::TILE;
      // ---- S^T = K Q^T and dP^T = V dO^T (K, V rows read in swap23 order)
      f32x16 st, dpt;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 ak = lds_read16(Ks + a_row * D, (2 * ks + g) ^ a_swz);
        st = mfma32(ak, qreg[ks], ks == 0 ? f32x16{} : st);
        const bf16x8 av = lds_read16(Vs + a_row * D, (2 * ks + g) ^ a_swz);
        dpt = mfma32(av, doreg[ks], ks == 0 ? f32x16{} : dpt);
      }
      // ---- P, the exact-delta partial sums and dS = P (dP - delta~); key of register r: crow(r, g)
      // masked scores become -inf, so exp2 gives exactly 0 (one branch per tile)
      const bool need_mask = (kv0 + C::BC > N) || (CAUSAL && kv0 + C::BC - 1 > q0w);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + crow(r, g);
          const bool bad = (key >= N) || (CAUSAL && key > q);
          st[r] = bad ? -INFINITY : st[r];
        }
      }
      if constexpr (DROP) {  // dP = Z dO V^T / (1 - rate)
        uint32_t word[4];
        drop_words_row(q, kv0, g, bh, seed_lo, seed_hi, word);
#pragma unroll
        for (int r = 0; r < 16; ++r) dpt[r] = drop_keep(word, r, drop_t) ? dpt[r] * inv_keep : 0.f;
      }
      // per half h of the tile's keys: P, the exact-delta partial sums and
      // dS = P (dP - delta~), then dQ^T += K^T dS^T for those 16 keys
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int r = 8 * h; r < 8 * h + 8; ++r) {
          const float p = fast_exp2(fmaf(st[r], c, -lq));
          d_exact = fmaf(p, dpt[r], d_exact);
          dpt[r] = p * (dpt[r] - dq_delta);
          st[r] = p;
        }
        const bf16x8 dso = c_to_operand(dpt, h);
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const bf16x8 akt = tr_operand<D>(Ks, dt, h, trb);  // K^T by transposing reads
          dq[dt] = mfma32(akt, dso, dq[dt]);
        }
      }
      if constexpr (!DROP) {
        // Instruction order: the first half's VALU work, then each dQ MFMA
        // with the transposing reads of the next one, the second half's
        // exponentials spread over the first half's MFMAs.
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, 44, 0);
#pragma unroll
        for (int i = 0; i < 2 * C::DT; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i < 2 * C::DT - 1) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          if (i < C::DT) __builtin_amdgcn_sched_group_barrier(0x402, 11, 0);
        }
      }
    }

    wait_vmem_all();  // the next tile has landed in LDS
    __syncthreads();
    kv_cur = kv_nxt;
    if constexpr (SPARSE) kv_nxt = j + 2 < n_tiles ? uniform(raw2) * C::BC : 0;
    else kv_nxt = (j + 2) * C::BC;
  };
  int j = 0;
  for (; j + 1 < n_tiles; j += 2) {
    iter(j, std::integral_constant<int, 0>{});
    iter(j + 1, std::integral_constant<int, 1>{});
  }
  if (j < n_tiles) iter(j, std::integral_constant<int, 0>{});

  // exact delta_q = sum_j P_qj dP_qj, handed to the dK/dV kernel
  d_exact = pair_sum(d_exact);
  if (q < N) {
    bf16* dQh = dQ + head + (size_t)q * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int dcol = 32 * dt + 8 * a + 4 * g;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = scale * dq[dt][4 * a + i];
        u32x2 w;
        w[0] = pack_bf16x2(v[0], v[1]);
        w[1] = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<u32x2*>(dQh + dcol) = w;
      }
    if (g == 0) DeltaOut[(size_t)bh * N + q] = d_exact;
  }
  if (PAIR) __syncthreads();  // every wave is done with this tile's LDS before the next tile's copies
  }
}

// Longest causal sequence, in 128-row query tiles, whose dq kernel runs two
// tiles per workgroup (measured: dq 1.3% faster at 64 tiles and 0.6% slower
// at 256).
constexpr int kBwdPairMaxTiles = 64;
// The same for dkdv, in 128-key blocks.  Its two-block loop spills 10 VGPRs
// (d = 128): 8% faster at 32 blocks, 0.5% slower at 64.
constexpr int kDkdvPairMaxTiles = 32;

// Resident workgroups of the unsplit dense non-causal d = 64 dkdv kernel on
// the current GPU (the occupancy query times the CU count), looked up once per
// device; 0 if unavailable.
constexpr int kMaxDevicesBwd = 64;
std::mutex g_dkdv_mu;
int g_dkdv_slots[kMaxDevicesBwd] = {};

int dkdv64_slots() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevicesBwd) {
    (void)hipGetLastError();
    return 0;
  }
  std::lock_guard<std::mutex> lock(g_dkdv_mu);
  if (g_dkdv_slots[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, (const void*)bwd_dkdv_kernel<64, false, false, false, false, false>, 256, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    g_dkdv_slots[dev] = per_cu > 0 && cus > 0 ? per_cu * cus : -1;
  }
  return g_dkdv_slots[dev];
}

// Whether dkdv runs with its query split (dense, d = 64, not causal: at d = 128
// the split kernel would not fit two waves per SIMD).  The split doubles the
// waves and the Q/dO copies; it pays when the unsplit launch takes few rounds
// of resident workgroups and leaves its last round at most half full (then
// that round runs one wave per SIMD): measured 6% faster at B=4 H=16 N=2048,
// 18% on a few heads, 4% slower at N=8192 and where everything fits in one
// round.
template <int D, bool CAUSAL>
bool dkdv_qsplit(int BH, int N) {
  if constexpr (D != 64 || CAUSAL) {
    return false;
  } else {
    const int slots = dkdv64_slots();
    if (slots <= 0) return false;
    const int64_t wgs = (int64_t)BH * ((N + DkdvCfg<64>::BKV - 1) / DkdvCfg<64>::BKV);
    const int64_t full = wgs / slots, rest = wgs % slots;
    return full < 4 && rest > 0 && 2 * rest <= slots;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv_t(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                         const float* delta, void* dk, void* dv, int BH, int N, float scale, const BlockMask& m,
                         const DropParams& dr, hipStream_t stream) {
  using C = DkdvCfg<D>;
  static_assert(C::BKV == kMaskBlock, "a workgroup owns one block column of the mask");
  const int n_kt = (N + C::BKV - 1) / C::BKV;
  const int total = BH * n_kt;
  const ScoreScale sc = split_scale(scale);
#define ATTN_DKDV_ARGS                                                                                         \
  dim3(total), dim3(256), 0, stream, (const bf16*)q, (const bf16*)k, (const bf16*)v, lse, (const bf16*)dout, delta, \
      (bf16*)dk, (bf16*)dv, N, n_kt, total, sc.c, scale
  if (m.ptr)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, true, false>), ATTN_DKDV_ARGS, m.ptr, m.head_stride, m.nb, 0u, 0u,
                       0u, 1.f, sc.mode);
  else if (dr.on)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, false, true>), ATTN_DKDV_ARGS, (const uint8_t*)nullptr, 0, 0,
                       dr.t, dr.seed_lo, dr.seed_hi, dr.inv_keep, sc.mode);
  else if (dkdv_qsplit<D, CAUSAL>(BH, N)) {
    if constexpr (D == 64 && !CAUSAL) {
      using CQ = DkdvCfg<D, true>;
      const int n_kq = (N + CQ::BKV - 1) / CQ::BKV;
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, false, false, false, true>), dim3(BH * n_kq), dim3(256), 0,
                         stream, (const bf16*)q, (const bf16*)k, (const bf16*)v, lse, (const bf16*)dout, delta,
                         (bf16*)dk, (bf16*)dv, N, n_kq, BH * n_kq, sc.c, scale, (const uint8_t*)nullptr, 0, 0, 0u, 0u,
                         0u, 1.f, sc.mode);
    }
  }
  else if (CAUSAL && BH % 8 == 0 && n_kt % 2 == 0 && n_kt <= kDkdvPairMaxTiles)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, false, false, true>), dim3(total / 2), dim3(256), 0, stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, lse, (const bf16*)dout, delta, (bf16*)dk,
                       (bf16*)dv, N, n_kt, total, sc.c, scale, (const uint8_t*)nullptr, 0, 0, 0u, 0u, 0u, 1.f, sc.mode);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, false, false>), ATTN_DKDV_ARGS, (const uint8_t*)nullptr, 0, 0,
                       0u, 0u, 0u, 1.f, sc.mode);
#undef ATTN_DKDV_ARGS
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dq_t(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                       const float* delta, const void* o_fused, void* dq, float* delta_out, int BH, int N,
                       float scale, const BlockMask& m, const DropParams& dr, hipStream_t stream) {
  using C = DqCfg<D>;
  static_assert(C::BRQ == kMaskBlock, "a workgroup owns one block row of the mask");
  const int n_qt = (N + C::BRQ - 1) / C::BRQ;
  const int total = BH * n_qt;
  const ScoreScale sc = split_scale(scale);
#define ATTN_DQ_ARGS                                                                                           \
  dim3(total), dim3(256), 0, stream, (const bf16*)q, (const bf16*)k, (const bf16*)v, lse, (const bf16*)dout, delta, \
      (const bf16*)o_fused, (bf16*)dq, delta_out, N, n_qt, total, sc.c, scale
  if (m.ptr)
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, true, false>), ATTN_DQ_ARGS, m.ptr, m.head_stride, m.nb, 0u, 0u, 0u,
                       1.f, sc.mode);
  else if (dr.on)
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, false, true>), ATTN_DQ_ARGS, (const uint8_t*)nullptr, 0, 0, dr.t,
                       dr.seed_lo, dr.seed_hi, dr.inv_keep, sc.mode);
  else if (CAUSAL && BH % 8 == 0 && n_qt % 2 == 0 && n_qt <= kBwdPairMaxTiles)
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, false, false, true>), dim3(total / 2), dim3(256), 0, stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, lse, (const bf16*)dout, delta,
                       (const bf16*)o_fused, (bf16*)dq, delta_out, N, n_qt, total, sc.c, scale,
                       (const uint8_t*)nullptr, 0, 0, 0u, 0u, 0u, 1.f, sc.mode);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, false, false>), ATTN_DQ_ARGS, (const uint8_t*)nullptr, 0, 0, 0u, 0u,
                       0u, 1.f, sc.mode);
#undef ATTN_DQ_ARGS
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_preprocess(const void* o, const void* dout, float* delta, int BH, int N, int d,
                                 hipStream_t stream) {
  const int rows = BH * N;
  if (d == 64) {
    hipLaunchKernelGGL((bwd_preprocess_kernel<64>), dim3((rows + 31) / 32), dim3(256), 0, stream,
                       (const bf16*)o, (const bf16*)dout, delta, rows);
  } else {
    hipLaunchKernelGGL((bwd_preprocess_kernel<128>), dim3((rows + 15) / 16), dim3(256), 0, stream,
                       (const bf16*)o, (const bf16*)dout, delta, rows);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                           const float* delta, void* dk, void* dv, int BH, int N, int d, float scale,
                           bool causal, const BlockMask& m, const DropParams& dr, hipStream_t stream) {
  if (d == 64)
    return causal ? launch_dkdv_t<64, true>(q, k, v, lse, dout, delta, dk, dv, BH, N, scale, m, dr, stream)
                  : launch_dkdv_t<64, false>(q, k, v, lse, dout, delta, dk, dv, BH, N, scale, m, dr, stream);
  return causal ? launch_dkdv_t<128, true>(q, k, v, lse, dout, delta, dk, dv, BH, N, scale, m, dr, stream)
                : launch_dkdv_t<128, false>(q, k, v, lse, dout, delta, dk, dv, BH, N, scale, m, dr, stream);
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                         const float* delta, const void* o_fused, void* dq, float* delta_out, int BH, int N, int d,
                         float scale, bool causal, const BlockMask& m, const DropParams& dr, hipStream_t stream) {
  if (d == 64)
    return causal ? launch_dq_t<64, true>(q, k, v, lse, dout, delta, o_fused, dq, delta_out, BH, N, scale, m, dr, stream)
                  : launch_dq_t<64, false>(q, k, v, lse, dout, delta, o_fused, dq, delta_out, BH, N, scale, m, dr,
                                           stream);
  return causal ? launch_dq_t<128, true>(q, k, v, lse, dout, delta, o_fused, dq, delta_out, BH, N, scale, m, dr, stream)
                : launch_dq_t<128, false>(q, k, v, lse, dout, delta, o_fused, dq, delta_out, BH, N, scale, m, dr,
                                          stream);
}

}  // namespace attn
