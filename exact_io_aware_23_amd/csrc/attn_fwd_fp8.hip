// FP8 (e4m3) fused attention forward for gfx950.
//
// What it computes (the pages, by title and section): "What is Flash
// Attention?" (iania.ai video page, English), 09:29: the third generation of
// the method adds an FP8 forward.  The format is OCP OFP8 E4M3 (bias 7, three
// mantissa bits, largest finite value 448, no infinities).  Q, K, V arrive as
// e4m3 codes with one fp32 scale per tensor (dq, dk, dv); the result is the
// attention of the dequantized tensors,
//   S = scale * (dq Q8) (dk K8)^T,  P = softmax(S),  O = P (dv V8),
// with O in bf16 and L = logsumexp(S) in fp32, exactly as the bf16 kernel
// defines them (transcript 01:04, 04:15-05:17 of the same page).
//
// Design (MI355X, CDNA4), the bf16 forward's pipeline on the fp8 matrix cores:
//   * S^T = K Q^T on v_mfma_f32_32x32x64_f8f6f4 (both operands e4m3): one
//     instruction contracts 64 head dims, so d = 128 takes two per 32 x 32
//     tile.  The scale dq dk scale log2(e) is folded into the exponent FMA, so
//     Q and K never leave their codes.
//   * O^T += V^T P^T on the same instruction, 64 keys per step: the 32 scores
//     a lane holds (two 32-key halves of its query row) are rounded to e4m3
//     (v_cvt_pk_fp8_f32, nearest-even) in register order and are the P^T
//     operand as they stand; V^T comes from the row-major V tile by four
//     transposing byte reads (ds_read_b64_tr_b8).  dv is applied with the
//     final division by l.
//   * The probabilities are p = 2^(s - m) with a lazily raised reference max
//     m (raised only when some p of a tile would pass 2^8, which each lane's
//     row sum of p shows, so no tile max is formed on the common path), so
//     p <= 256 stays inside the e4m3 range; l sums the unrounded p in fp32.
//   * Everything else is the bf16 kernel's: 4 waves x 32 query rows, 64-key
//     K/V tiles double-buffered in LDS through buffer -> LDS copies, one
//     barrier per tile, scores of tile j+1 interleaved with tile j's
//     exponentials and P V, causal tile skipping, XCD-aware work order.
#include <type_traits>

#include "attn_common.h"
#include "attn_launch.h"

namespace attn {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// 32 x 32 x 64 e4m3 product: lane l holds A[l % 32][32 (l / 32) + e] and
// B[32 (l / 32) + e][l % 32] for byte e = 0..31; C as in the bf16 product.
// (No block scales: with zero scale operands the unscaled instruction is emitted.)
__device__ __forceinline__ f32x16 mfma32_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int D>
struct Fp8Cfg {
  static constexpr int WAVES = 4;
  static constexpr int BR = WAVES * 32;       // query rows per workgroup
  static constexpr int BC = 64;               // keys per K/V tile
  static constexpr int NCH = D / 16;          // 16-byte chunks per row (one byte per element)
  static constexpr int KS = D / 64;           // MFMAs per 32 x 32 score tile
  static constexpr int DT = D / 32;           // 32-wide d tiles of O^T
  static constexpr int NKLD = BC * NCH / 256; // 1 KB buffer -> LDS copies per wave per tile
  static constexpr int TILE = BC * D;         // bytes of one K or V tile
  static constexpr int STAGE = 2 * TILE;      // one slot: a K tile then a V tile
};

// XOR swizzles of the 16-byte chunks of a row (physical = logical ^ swz(row)).
// K tile, read by ds_read_b128 of one chunk from 16 rows (any order of the
// low four row bits): the row bits above the bank window pick 8 (d = 128,
// 128-byte rows, 2 per 256-byte window) or 4 (d = 64) distinct chunks.
template <int NCH>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (NCH == 8) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}
// V tile, read by ds_read_b64_tr_b8 of chunks {2 dt, 2 dt + 1} from 8
// consecutive rows per half-wave: rows sharing a bank window position go to
// different chunk pairs.
template <int NCH>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (NCH == 8) return (((row >> 1) & 3) << 1) | ((row >> 3) & 1);
  else return (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
}

// 8 transposed bytes: within each 16-lane group, lane 2 e + h names the
// 8 bytes (row e, columns 8 h .. 8 h + 7) of an 8 x 16 byte block, and lane i
// receives column i (one byte of each row).
__device__ __forceinline__ i32x2 lds_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)p);
}
__device__ __forceinline__ i32x4 lds16b(const uint8_t* p) { return *reinterpret_cast<const i32x4*>(p); }

constexpr float kTau8Pow = 256.0f;  // lazy rescaling bound 2^8: every p <= 2^8 (fits e4m3)

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 2)
fwd_fp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
               bf16* __restrict__ O, float* __restrict__ L, int N, int n_qtiles, int total, float c,
               float dv, uint32_t smode) {
  using C = Fp8Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];

  const int work = xcd_remap(blockIdx.x, total);
  const int bh = work / n_qtiles;
  const int qt = CAUSAL ? (n_qtiles - 1 - work % n_qtiles) : (work % n_qtiles);
  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D;
  const rsrc_t rQ = make_rsrc(Q + head, head_bytes);
  const rsrc_t rK = make_rsrc(K + head, head_bytes);
  const rsrc_t rV = make_rsrc(V + head, head_bytes);

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int q0w = qt * C::BR + wave * 32;
  const int q = q0w + l32;

  const int kv_end = CAUSAL ? min(N, qt * C::BR + C::BR) : N;
  const int n_tiles = (kv_end + C::BC - 1) / C::BC;
  int wave_tiles = 0;
  if (q0w < N) wave_tiles = ((CAUSAL ? min(N, q0w + 32) : N) + C::BC - 1) / C::BC;
  auto needs_mask = [&](int kv0) { return kv0 + C::BC > N || (CAUSAL && kv0 + C::BC - 1 > q0w); };

  // ---- Q^T operand in registers: lane (l32, g) holds Q[q][64 ks + 32 g + e]
  i32x8 qreg[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const int off = q * D + 64 * ks + 32 * g;
    const i32x4 lo = __builtin_bit_cast(i32x4, bload16(rQ, off, 0));
    const i32x4 hi = __builtin_bit_cast(i32x4, bload16(rQ, off + 16, 0));
    qreg[ks] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    if (smode != kSignPos) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qreg[ks][e] = (int)sign_word_e4m3((uint32_t)qreg[ks][e], smode);
    }
  }

  // ---- buffer -> LDS copies: wave `wave`, copy i fills 1 KB block
  // (wave * NKLD + i) of a tile; each lane picks the global chunk that its
  // LDS position holds under the tile's swizzle
  int koff[C::NKLD], voff[C::NKLD];
#pragma unroll
  for (int i = 0; i < C::NKLD; ++i) {
    const int idx = (wave * C::NKLD + i) * 64 + lane;
    const int row = idx / C::NCH, cphys = idx % C::NCH;
    koff[i] = row * D + 16 * (cphys ^ swz_k<C::NCH>(row));
    voff[i] = row * D + 16 * (cphys ^ swz_v<C::NCH>(row));
  }
  auto load_k = [&](int kv0, int slot) {
    uint8_t* Ks = smem + slot * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::NKLD; ++i) bload16_lds(rK, Ks + (wave * C::NKLD + i) * 1024, koff[i], kv0 * D);
  };
  auto load_v = [&](int kv0, int slot) {
    uint8_t* Vs = smem + slot * C::STAGE + C::TILE;
#pragma unroll
    for (int i = 0; i < C::NKLD; ++i) bload16_lds(rV, Vs + (wave * C::NKLD + i) * 1024, voff[i], kv0 * D);
  };

  // K operand: row swap23(l32) of each 32-key half, logical chunks
  // 4 ks + 2 g + u (u = 0, 1); the ks term is an XOR of 64 ks on the offset
  const int krow = swap23(l32);
  int kofs[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) kofs[u] = krow * D + 16 * ((2 * g + u) ^ swz_k<C::NCH>(krow));
  // V^T operand: lane 16 G + i (g = G / 2) reads row 16 t + 8 g + i / 2,
  // logical chunk 2 dt + (G & 1), bytes 8 (i & 1) .. +7, for t = 0..3; it
  // receives V[16 t + 8 g + e][32 dt + l32], e = 0..7: the keys that its
  // P^T bytes 8 t .. 8 t + 7 hold
  int vofs;
  {
    const int i = lane & 15, G = lane >> 4;
    const int rl = 8 * g + (i >> 1);
    vofs = rl * D + 16 * ((G & 1) ^ swz_v<C::NCH>(rl)) + 8 * (i & 1);
  }
  auto vt_op = [&](const uint8_t* Vs, int dt) {
    i32x8 out;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const i32x2 x = lds_tr8(Vs + ((vofs ^ (32 * dt)) + 16 * t * D));
      out[2 * t] = x[0];
      out[2 * t + 1] = x[1];
    }
    return out;
  };

  f32x16 oacc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -1e30f, l_run = 0.f;

  auto scores = [&](int slot, f32x16 (&st)[2]) {
    const uint8_t* Ks = smem + slot * C::STAGE;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const i32x4 lo = lds16b(Ks + (kofs[0] ^ (64 * ks)) + 32 * kb * D);
        const i32x4 hi = lds16b(Ks + (kofs[1] ^ (64 * ks)) + 32 * kb * D);
        st[kb] = mfma32_fp8(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), qreg[ks],
                            ks == 0 ? f32x16{} : st[kb]);
      }
  };
  auto mask = [&](f32x16 (&st)[2], int kv0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 32 * kb + crow(r, g);
        const bool bad = (key >= N) || (CAUSAL && key > q);
        st[kb][r] = bad ? -INFINITY : st[kb][r];
      }
  };
  auto tile_max = [&](const f32x16 (&st)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kb][r]);
    return pair_max(mx) * c;
  };
  // raise the reference max to the tile's max (a no-op where it is not
  // above it), rescaling l and the O accumulators
  auto raise_max = [&](float mt) {
    const float m_new = fmaxf(m_run, mt);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
  };
  // p = 2^(s c - m) (the scores stay), this lane's sum of p into rs, and P^T
  // as e4m3 bytes: byte e of the operand is register e % 16 of half e / 16
  // (key 32 (e/16) + crow)
  auto exps = [&](const f32x16 (&st)[2], i32x8& pop, float& rs) {
    const float mneg = -m_run;
    f32x16 p[2];
    rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[kb][r] = fast_exp2(fmaf(st[kb][r], c, mneg));
        rs += p[kb][r];
      }
    // (the first conversion of a word writes its low half and keeps the high
    // half of its third operand, which the second overwrites: passing a
    // register that dies there instead of 0 saves a v_mov per word)
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kb = w >> 2, r = 4 * (w & 3);
      int x = __builtin_amdgcn_cvt_pk_fp8_f32(p[kb][r], p[kb][r + 1], __builtin_bit_cast(int, p[kb][r]), false);
      x = __builtin_amdgcn_cvt_pk_fp8_f32(p[kb][r + 2], p[kb][r + 3], x, true);
      pop[w] = x;
    }
    // formed here, not sunk past the check below
    asm volatile("" : "+v"(pop));
  };
  // The lazy rescale without a tile max on the common path (as in the bf16
  // forward): a lane's sum of p bounds every p it holds, so a sum of at most
  // 2^kTau8 lets m stay (p then fits e4m3); otherwise, or on inf / NaN, the
  // tile's max is formed, m raised to it, and p formed again from the scores.
  auto check_exps = [&](const f32x16 (&st)[2], i32x8& pop, float& rs) {
    if (__builtin_amdgcn_ballot_w64(!(rs <= kTau8Pow)) != 0) {
      raise_max(tile_max(st));
      exps(st, pop, rs);
    }
    l_run += rs;
  };
  auto pv = [&](int slot, const i32x8& pop) {
    const uint8_t* Vs = smem + slot * C::STAGE + C::TILE;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) oacc[dt] = mfma32_fp8(vt_op(Vs, dt), pop, oacc[dt]);
  };

  // Instruction order of a pipelined step.  Phase A: the score MFMAs of tile
  // j+1, each fed by two K reads issued one MFMA ahead, with tile j's
  // exponentials and rounding spread over them.  Phase B: tile j's P V
  // MFMAs, each fed by four transposing reads, with tile j+1's max.
  constexpr int SM = 2 * C::KS, PVM = C::DT;
  auto pin_a = [&]() {
    constexpr int VA = (120 + SM - 1) / SM;
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < SM - 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, VA, 0);
    }
  };
  auto pin_b = [&]() {
    constexpr int VB = (40 + PVM - 1) / PVM;
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < PVM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < PVM - 2) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, VB, 0);
    }
  };

  // ---- software pipeline (the slot discipline of the bf16 kernel)
  if (n_tiles > 0) {
    load_k(0, 0);
    load_v(0, 0);
  }
  if (n_tiles > 1) load_k(C::BC, 1);
  wait_vmem_all();
  __syncthreads();
  f32x16 sa[2], sb[2];
  if (wave_tiles > 0) {
    scores(0, sa);
    if (needs_mask(0)) mask(sa, 0);
    m_run = fmaxf(m_run, tile_max(sa));  // (l and O are still 0)
  }
  __syncthreads();  // every wave has read K(0) before K(2) is loaded over it

  // A step whose next tile needs no mask (MASKED = false) has no branch
  // between its MFMAs and the next tile's max, so the row sums and the max
  // stay in the instruction stream of the MFMAs instead of being moved past
  // a join.  Tiles 0 .. jm-1 of this wave need no mask.
  const int lim = CAUSAL ? min(N, q0w + 1) : N;
  const int jm = uniform(max(lim, 0) / C::BC);
  auto step = [&](int j, int par, f32x16 (&cur)[2], f32x16 (&nxt)[2], auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    const int kv_a = (j + 1) * C::BC;
    if (j + 2 < n_tiles) load_k((j + 2) * C::BC, par);
    if (j + 1 < n_tiles) load_v(kv_a, par ^ 1);
    if (!MASKED || j < wave_tiles) {
      // the scores of tile j+1 are formed even when this wave has no such
      // tile (the slot holds an in-bounds K tile whose keys the mask removes)
      i32x8 pop;
      float rs;
      scores(par ^ 1, nxt);
      exps(cur, pop, rs);
      pin_a();
      check_exps(cur, pop, rs);
      pv(par, pop);
      pin_b();
      if constexpr (MASKED) {
        if (needs_mask(kv_a)) mask(nxt, kv_a);
      }
    }
    wait_vmem_all();
    __syncthreads();
  };
  using Plain = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;
  int j = 0;
  for (; j + 2 < jm; j += 2) {  // tiles j+1 and j+2 need no mask
    step(j, 0, sa, sb, Plain{});
    step(j + 1, 1, sb, sa, Plain{});
  }
  for (; j + 1 < n_tiles; j += 2) {
    step(j, 0, sa, sb, Masked{});
    step(j + 1, 1, sb, sa, Masked{});
  }
  if (j < n_tiles) step(j, 0, sa, sb, Masked{});

  // ---- epilogue: O = dv O_acc / l, L = (m + log2 l) ln 2
  const float lt = pair_sum(l_run);
  if (q < N) {
    bf16* Oh = O + head + (size_t)q * D;
    const float inv = dv / lt;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int dcol = 32 * dt + 8 * a + 4 * g;
        u32x2 w;
        w[0] = pack_bf16x2(oacc[dt][4 * a + 0] * inv, oacc[dt][4 * a + 1] * inv);
        w[1] = pack_bf16x2(oacc[dt][4 * a + 2] * inv, oacc[dt][4 * a + 3] * inv);
        *reinterpret_cast<u32x2*>(Oh + dcol) = w;
      }
    if (g == 0) L[(size_t)bh * N + q] = (m_run + log2f(lt)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_fp8_t(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N,
                            float c, float dv, uint32_t smode, hipStream_t stream) {
  using C = Fp8Cfg<D>;
  const int n_qtiles = (N + C::BR - 1) / C::BR;
  const int total = BH * n_qtiles;
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), dim3(total), dim3(256), 0, stream, (const uint8_t*)q,
                     (const uint8_t*)k, (const uint8_t*)v, (bf16*)o, lse, N, n_qtiles, total, c, dv, smode);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, int d,
                          float scale, float dq, float dk, float dv, bool causal, hipStream_t stream) {
  // the exponent factor |scale dq dk| log2 e; the sign of scale goes into Q (kSignNeg / kSignZero)
  const uint32_t mode = scale > 0.f ? kSignPos : scale < 0.f ? kSignNeg : kSignZero;
  const double mag = scale == 0.f ? 1.0 : (double)(scale < 0.f ? -scale : scale) * dq * dk;
  const float c = (float)(mag * 1.4426950408889634);
  if (d == 64) return causal ? launch_fwd_fp8_t<64, true>(q, k, v, o, lse, BH, N, c, dv, mode, stream)
                             : launch_fwd_fp8_t<64, false>(q, k, v, o, lse, BH, N, c, dv, mode, stream);
  return causal ? launch_fwd_fp8_t<128, true>(q, k, v, o, lse, BH, N, c, dv, mode, stream)
                : launch_fwd_fp8_t<128, false>(q, k, v, o, lse, BH, N, c, dv, mode, stream);
}

}  // namespace attn
