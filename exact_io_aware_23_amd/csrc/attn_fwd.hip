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
//   * One workgroup = 4 waves = 128 query rows, 32 per wave; at d = 128 two
//     workgroups share a CU (up to 256 VGPRs, two waves per SIMD).
//   * Software pipeline inside each wave: the scores of tile j+1 are formed
//     while tile j's exponentials run, then tile j's P V, all in one basic
//     block whose instruction order is pinned (sched_group_barrier), so the
//     VALU work sits in the shadow of the MFMAs of the same wave.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T kept in
//     VGPRs for the whole loop).  In the S^T layout each lane owns one query
//     row, so the row max, the exp-sum and the O rescale stay lane-local; one
//     v_permlane32_swap joins the two lane halves for the max.
//   * O^T += V^T P^T: P^T comes straight from the S^T accumulators (rounded to
//     bf16); the V^T fragments come from the row-major V tile by transposing
//     LDS reads (ds_read_b64_tr_b16), so V needs no transpose on the way in.
//   * Softmax in base 2: p = exp2(s * scale * log2(e) - m) with one FMA and one
//     v_exp_f32 per score; L = (m + log2 l) ln 2 at the end.  The reference max
//     m moves only when some p of a tile would exceed 2^8 (lazy rescaling), so
//     the O accumulators are rarely touched by the VALU.  Each lane's row sum
//     of p shows whether that happened, so the tile max is formed only then.
//   * Global loads use raw buffer resources: per-lane offsets are
//     loop-invariant, the tile offset is a scalar, rows past N read as zero.
//   * K/V tiles of 64 keys are double-buffered in LDS and loaded by buffer ->
//     LDS transfers (no VGPRs, no LDS store instructions): while a wave works
//     on K(j+1) and V(j), K(j+2) and V(j+1) are in flight.  One barrier per
//     tile.
//   * Causal: key tiles past a query tile's last row are never loaded; a wave
//     skips the tiles past its own last row; only diagonal (and ragged tail)
//     tiles apply the mask.  Query tiles run longest first within a head, and
//     work items are renumbered so each XCD sweeps whole heads (L2 reuse).
//   * At d = 64 the non-causal forward (any length) and the causal one up to
//     N = 512 take a variant without the in-wave pipeline: one score tile in
//     registers, under 128 VGPRs, four workgroups per CU.  Short sequences
//     are HBM-latency bound, and more workgroups keep more loads in flight;
//     long ones are bound by the VALU softmax (at d = 64 a tile's exponentials
//     take more VALU cycles than its matrix products take MFMA cycles), and
//     four waves per SIMD keep that pipe busier than three pipelined ones.
#include "attn_common.h"
#include "attn_launch.h"

namespace attn {
namespace {

template <int D>
struct FwdCfg {
  static constexpr int WAVES = 4;
  static constexpr int BR = WAVES * 32;      // query rows per workgroup, 32 per wave
  static constexpr int BC = 64;              // keys per K/V tile
  static constexpr int NCH = D / 8;          // 16-byte chunks per K row
  static constexpr int KS = D / 16;          // k-steps of S^T = K Q^T
  static constexpr int DT = D / 32;          // 32-wide d tiles of O^T
  static constexpr int NKLD = BC * NCH / 256;
  static constexpr int K_ELEMS = BC * D;
  static constexpr int STAGE = 2 * BC * D;   // one slot: a K tile then a V tile, row-major
};

// Lazy rescaling bound (log2 units).  The running reference max m of a row
// is raised only when some p = exp2(s*c - m) of a tile would exceed 2^kTau,
// so most tiles skip the O-accumulator rescale; the result is unchanged (the
// same m is used for O and l).
constexpr float kTau = 8.0f;
constexpr float kTauPow = 256.0f;  // 2^kTau

// Longest causal sequence (d = 64, no block mask, no dropout) that the
// forward runs with the one-tile-at-a-time kernel: up to eight 64-key tiles
// per workgroup (the non-causal d = 64 forward takes it at every length).
constexpr int kShortSeqMaxN = 512;

// Fewest tiles per workgroup for which the one-tile loop lowers a wave's
// priority as it progresses (measured: 3-5% faster from 16 tiles up, 20%
// slower at 4).
constexpr int kPrioMinTiles = 16;

// One work item (query tile qt of head bh, work = bh * n_qtiles + index) of
// the forward, by one workgroup of 256 threads.
template <int D, bool CAUSAL, bool SPARSE, bool DROP, bool PIPE>
__device__ __forceinline__ void fwd_bf16_item(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                              const bf16* __restrict__ V, bf16* __restrict__ O,
                                              float* __restrict__ L, int N, int n_qtiles, float c,
                                              const uint8_t* __restrict__ Mask, int mask_hs, int nb,
                                              uint32_t drop_t, uint32_t seed_lo, uint32_t seed_hi, float inv_keep,
                                              uint32_t smode, int work) {
  using C = FwdCfg<D>;
  static_assert(!(SPARSE && DROP), "block-sparse and dropout are separate entry points");
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * C::STAGE];
  // block-sparse: the key tiles of this workgroup whose 128 x 128 block is on
  __shared__ uint16_t tlist[SPARSE ? kMaxSparseN / C::BC : 1];
  __shared__ int wcnt[SPARSE ? 4 : 1];

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
  const int q0w = qt * C::BR + wave * 32;
  const int q = q0w + l32;

  // ---- tile ranges (all wave-uniform): the workgroup loads n_tiles tiles,
  // this wave computes the first wave_tiles of them
  const int kv_end = CAUSAL ? min(N, qt * C::BR + C::BR) : N;
  int n_tiles = (kv_end + C::BC - 1) / C::BC;
  int wave_tiles = 0;
  if (q0w < N) wave_tiles = ((CAUSAL ? min(N, q0w + 32) : N) + C::BC - 1) / C::BC;

  // ---- Q^T operand in registers: lane (l32, g) holds Q[q][16ks + 8g .. +7]
  bf16x8 qreg[C::KS];
  {
    const int qoff = (q * D + 8 * g) * 2;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8, bload16(rQ, qoff + 32 * ks, 0));
    if (smode != kSignPos) {
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) qreg[ks] = sign_bf16x8(qreg[ks], smode);
    }
  }
  if constexpr (SPARSE) {
    // (after the Q loads are issued, so the two latencies overlap)
    // tile t holds keys [64 t, 64 t + 64), in block t / 2 of the block row qt
    const uint8_t* mrow = Mask + (size_t)bh * mask_hs + (size_t)qt * nb;
    n_tiles = uniform(compact_indices(tlist, wcnt, 0, n_tiles, [&](int t) { return mrow[t >> 1] != 0; }));
    wave_tiles = uniform(count_below(tlist, n_tiles, wave_tiles));
  }
  // first key of the j-th tile this workgroup visits (past the end: N, all masked)
  auto kv0_of = [&](int j) -> int {
    if constexpr (SPARSE) return j < n_tiles ? uniform((int)tlist[j]) * C::BC : N;
    else return j * C::BC;
  };
  // the tile at kv0 needs the mask when it holds keys past N or (causal) past this wave's first row
  auto needs_mask = [&](int kv0) { return kv0 + C::BC > N || (CAUSAL && kv0 + C::BC - 1 > q0w); };

  // K and V tiles go straight into LDS (row-major, XOR-swizzled 16-byte chunks):
  // wave `wave`, instruction i fills 1 KB block (wave * NKLD + i) of the tile.
  int kvoff[C::NKLD];
#pragma unroll
  for (int i = 0; i < C::NKLD; ++i) {
    const int idx = (wave * C::NKLD + i) * 64 + lane;
    const int row = idx / C::NCH, cphys = idx % C::NCH;
    kvoff[i] = (row * D + 8 * (cphys ^ chunk_swz<C::NCH>(row))) * 2;
  }
  // copy the K (V) tile whose first key is kv0 into LDS slot `slot`
  auto load_k = [&](int kv0, int slot) {
    bf16* Ks = smem + slot * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::NKLD; ++i) bload16_lds(rK, Ks + (wave * C::NKLD + i) * 512, kvoff[i], kv0 * D * 2);
  };
  auto load_v = [&](int kv0, int slot) {
    bf16* Vs = smem + slot * C::STAGE + C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::NKLD; ++i) bload16_lds(rV, Vs + (wave * C::NKLD + i) * 512, kvoff[i], kv0 * D * 2);
  };

  // S^T operand reads: K row swap23(l32) of each 32-key half
  const int krow = swap23(l32);
  const int k_swz = chunk_swz<C::NCH>(krow);
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

  f32x16 oacc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -1e30f, l_run = 0.f;

  // ---- the pieces of one tile
  // S^T = K Q^T for the K tile in `slot`
  auto scores = [&](int slot, f32x16 (&st)[2]) {
    const bf16* Ks = smem + slot * C::STAGE;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = lds_read16(Ks + (32 * kb + krow) * D, (2 * ks + g) ^ k_swz);
        st[kb] = mfma32(a, qreg[ks], ks == 0 ? f32x16{} : st[kb]);
      }
  };
  // masked scores become -inf (keys past N, and causal keys past the row)
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
  // this row's tile max in log2 units
  auto tile_max = [&](const f32x16 (&st)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kb][r]);
    return pair_max(mx) * c;
  };
  // raise the reference max to the tile's max (a no-op where the tile's max
  // is not above it), rescaling l and the O accumulators
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
  // p = exp2(s c - m) into the P^T operands (the scores stay), and this
  // lane's sum of p into rs.  With dropout, rs sums every p (L is the
  // logsumexp without dropout) and the dropped entries become 0 in the P V
  // operand; 1 / (1 - rate) is applied with the division by l at the end.
  auto exps = [&](const f32x16 (&st)[2], bf16x8 (&pop)[4], int kv0, float& rs) {
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
    if constexpr (DROP) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        uint32_t word[4];
        drop_words_row(q, kv0 + 32 * kb, g, bh, seed_lo, seed_hi, word);
#pragma unroll
        for (int r = 0; r < 16; ++r) p[kb][r] = drop_keep(word, r, drop_t) ? p[kb][r] : 0.f;
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      pop[m] = c_to_operand(p[m >> 1], m & 1);
      // formed here, not sunk past the check below, so p is dead before it
      asm volatile("" : "+v"(pop[m]));
    }
  };
  // Lazy rescaling without a tile max on the common path.  Every p of a lane
  // is at most that lane's sum, so a sum of at most 2^kTau shows that the
  // reference max may stay.  Otherwise (a p above 2^kTau, or an inf or NaN
  // sum) the tile's max is formed, m raised to it, and p recomputed; the
  // scores are still in registers for that.  Either way every p is at most
  // 2^kTau, and m changes only through raise_max, so O and l stay on one
  // reference.
  auto check_exps = [&](const f32x16 (&st)[2], bf16x8 (&pop)[4], int kv0, float& rs) {
    if (__builtin_amdgcn_ballot_w64(!(rs <= kTauPow)) != 0) {
      raise_max(tile_max(st));
      exps(st, pop, kv0, rs);
    }
    l_run += rs;
  };
  // O^T += V^T P^T for the V tile in `slot`
  auto pv = [&](int slot, const bf16x8 (&pop)[4]) {
    const bf16* Vs = smem + slot * C::STAGE + C::K_ELEMS;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) oacc[dt] = mfma32(vt_tr(Vs, dt, m), pop[m], oacc[dt]);
  };

  // Instruction order inside the two straight-line phases of a pipelined step.
  // Phase A, the scores of tile j+1 with tile j's exponentials: each score
  // MFMA takes one K read issued four ahead and a share of the VALU work.
  // Phase B, tile j's P V with tile j+1's max: each P V MFMA takes two
  // transposing reads and a little VALU.
  constexpr int SM = 2 * C::KS, PVM = 4 * C::DT;  // MFMAs per phase
  auto pin_a = [&]() {
    constexpr int VA = ((DROP ? 400 : 120) + SM - 1) / SM;  // dropout adds its generator calls
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < SM - 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, VA, 0);
    }
  };
  auto pin_b = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < PVM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < PVM - 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 3, 0);
    }
  };

  if constexpr (!PIPE) {
    // Short sequences (a few tiles per workgroup): one tile at a time, scores,
    // max, exponentials and P V, while the next tile's K and V are copied into
    // the other LDS slot.  One score tile instead of two keeps the kernel
    // under 128 VGPRs, so four workgroups share a CU and more of them have
    // loads in flight.
    if (n_tiles > 0) {
      load_k(kv0_of(0), 0);
      load_v(kv0_of(0), 0);
    }
    wait_vmem_all();
    __syncthreads();
    for (int j = 0; j < n_tiles; ++j) {
      // The four waves of a SIMD come from four workgroups, and the hardware
      // issues oldest first, so the first workgroup runs ahead and the CU
      // ends with one wave left.  On long loops a wave lowers its own
      // priority as it passes each quarter of its tiles, so waves that are
      // behind get the issue slots.
      if (n_tiles >= kPrioMinTiles) {
        const int band = (4 * j) / n_tiles;
        if (band == 0) __builtin_amdgcn_s_setprio(3);
        else if (band == 1) __builtin_amdgcn_s_setprio(2);
        else if (band == 2) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }
      const int slot = j & 1;
      const int kv0 = kv0_of(j);
      if (j + 1 < n_tiles) {
        load_k(kv0_of(j + 1), slot ^ 1);
        load_v(kv0_of(j + 1), slot ^ 1);
      }
      if (j < wave_tiles) {
        f32x16 st[2];
        bf16x8 pop[4];
        // The scores die as p is formed (this kernel stays under 128 VGPRs);
        // the rare slow path forms them again from the K tile, which stays in
        // its slot until the barrier below.
        float rs;
        scores(slot, st);
        if (needs_mask(kv0)) mask(st, kv0);
        if (j == 0) m_run = fmaxf(m_run, tile_max(st));  // (l and O are still 0)
        exps(st, pop, kv0, rs);
        if (__builtin_amdgcn_ballot_w64(!(rs <= kTauPow)) != 0) {
          scores(slot, st);
          if (needs_mask(kv0)) mask(st, kv0);
          raise_max(tile_max(st));
          exps(st, pop, kv0, rs);
        }
        l_run += rs;
        pv(slot, pop);
      }
      wait_vmem_all();  // tile j+1 has landed; every wave is done with slot j & 1
      __syncthreads();
    }
  } else {
  // ---- software pipeline.  Slot s of LDS holds K and V tiles of the same
    // parity.  Iteration j reads K(j+1) (scores of the next tile) and V(j) (this
    // tile's P V), and loads K(j+2) over K(j) and V(j+1) over V(j-1), both read
    // before the previous barrier.  The scores of tile j+1 are independent of
    // tile j's exponentials, and tile j's P V of tile j+1's max, so each pair
    // sits in one basic block for the scheduler to interleave.
    const int kv_first = kv0_of(0);
    if (n_tiles > 0) {
      load_k(kv_first, 0);
      load_v(kv_first, 0);
    }
    if (n_tiles > 1) load_k(kv0_of(1), 1);
    wait_vmem_all();
    __syncthreads();
    f32x16 sa[2], sb[2];
    if (wave_tiles > 0) {
      scores(0, sa);
      if (needs_mask(kv_first)) mask(sa, kv_first);
      m_run = fmaxf(m_run, tile_max(sa));  // (l and O are still 0)
    }
    // first keys of tiles j+1 and j+2 at the start of step j, carried from step
    // to step; a block-sparse step reads the entry for j+3 from the LDS list
    // early and makes it scalar only after its barrier, when no other LDS read
    // is outstanding
    int kv_a = kv0_of(1), kv_b = kv0_of(2);
    __syncthreads();  // every wave has read K(0) before K(2) is loaded over it
  
    // `par` = j & 1, passed as a literal so every LDS address is a constant
    // offset from one per-lane base
    auto step = [&](int j, int par, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
      int raw3 = 0;
      if constexpr (SPARSE) raw3 = tlist[min(j + 3, kMaxSparseN / C::BC - 1)];
      if (j + 2 < n_tiles) load_k(kv_b, par);
      if (j + 1 < n_tiles) load_v(kv_a, par ^ 1);
      if (j < wave_tiles) {
        // The scores of tile j+1 are formed even when this wave has no such
        // tile: the slot then holds another K tile (in bounds), every one of
        // its keys lies past this wave's rows or past N, so the mask sets them
        // all to -inf, and the rescale is skipped.  One code path per step.
        bf16x8 pop[4];
        float rs;
        scores(par ^ 1, nxt);
        exps(cur, pop, j * C::BC, rs);  // (dropout runs on dense tiles only, so tile j starts at key 64 j)
        pin_a();
        check_exps(cur, pop, j * C::BC, rs);
        pv(par, pop);
        pin_b();
        if (needs_mask(kv_a)) mask(nxt, kv_a);
      }
      wait_vmem_all();  // K(j+2) and V(j+1) have landed in LDS
      __syncthreads();
      kv_a = kv_b;
      if constexpr (SPARSE) kv_b = j + 3 < n_tiles ? uniform(raw3) * C::BC : N;
      else kv_b = (j + 3) * C::BC;
    };
    int j = 0;
    for (; j + 1 < n_tiles; j += 2) {
      step(j, 0, sa, sb);
      step(j + 1, 1, sb, sa);
    }
    if (j < n_tiles) step(j, 0, sa, sb);
  
  }

  // ---- epilogue: O = O_acc / l, L = (m + log2 l) ln 2; a row with no allowed
  // key (possible only under a block mask) gets O = 0 and L = -inf
  const float lt = pair_sum(l_run);
  const bool empty_row = SPARSE && lt == 0.f;
  if (q < N) {
    bf16* Oh = O + head + (size_t)q * D;
    const float inv = empty_row ? 0.f : (DROP ? inv_keep : 1.0f) / lt;
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
    if (g == 0) L[(size_t)bh * N + q] = empty_row ? -INFINITY : (m_run + log2f(lt)) * kLn2;
  }
}

// One work item per workgroup, in the XCD-aware order of xcd_remap.
template <int D, bool CAUSAL, bool SPARSE, bool DROP, bool PIPE = true>
__global__ void __launch_bounds__(256, PIPE ? 2 : 4)
fwd_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                bf16* __restrict__ O, float* __restrict__ L, int N, int n_qtiles, int total, float c,
                const uint8_t* __restrict__ Mask, int mask_hs, int nb, uint32_t drop_t, uint32_t seed_lo,
                uint32_t seed_hi, float inv_keep, uint32_t smode) {
  fwd_bf16_item<D, CAUSAL, SPARSE, DROP, PIPE>(Q, K, V, O, L, N, n_qtiles, c, Mask, mask_hs, nb, drop_t, seed_lo,
                                               seed_hi, inv_keep, smode, xcd_remap(blockIdx.x, total));
}

// Causal forward with one pair of query tiles per workgroup: tile p and tile
// n - 1 - p of the same head, one after the other, so every workgroup does
// the same work (n + 1 tiles' worth) and the hardware's turn-based dispatch
// over the XCDs never waits for a long tile.  Workgroup b runs on XCD b % 8
// and takes pair b / 8 of that XCD's heads (the xcd_remap order), the shorter
// tile first (measured within 0.5% of the other order).
template <int D>
__global__ void __launch_bounds__(256, 2)
fwd_bf16_pair_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                     bf16* __restrict__ O, float* __restrict__ L, int N, int n_qtiles, int total, float c,
                     uint32_t smode) {
  const int first = pair_work(blockIdx.x, total, n_qtiles, 0), second = pair_work(blockIdx.x, total, n_qtiles, 1);
  fwd_bf16_item<D, true, false, false, true>(Q, K, V, O, L, N, n_qtiles, c, nullptr, 0, 0, 0u, 0u, 0u, 1.f, smode,
                                             first);
  __syncthreads();  // every wave is done with the first tile's LDS before the second copies its own
  fwd_bf16_item<D, true, false, false, true>(Q, K, V, O, L, N, n_qtiles, c, nullptr, 0, 0, 0u, 0u, 0u, 1.f, smode,
                                             second);
}

// ---------------------------------------------------------------------------
// fp32 forward: the same online-softmax algorithm on plain fp32 VALU
// arithmetic.  Four threads share a query row, each holding a quarter of its
// d columns of q and of the O accumulator; a score is their four partial dot
// products joined by two lane swaps, so all four hold the same scores, max
// and sum.  32-key K/V tiles are staged in LDS and read as broadcasts.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256)
fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
               float* __restrict__ O, float* __restrict__ L, int N, int n_qtiles, float c, uint32_t smode) {
  constexpr int BC = 32;
  constexpr int DP = D / 4;  // columns per thread
  __shared__ float Ks[BC][D];
  __shared__ float Vs[BC][D];
  const int bh = blockIdx.x / n_qtiles;
  const int qt = blockIdx.x % n_qtiles;
  const size_t head = (size_t)bh * N * D;
  const int d0 = (threadIdx.x & 3) * DP;
  const int q = qt * 64 + (threadIdx.x >> 2);
  const bool qv = q < N;

  float qr[DP], acc[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) {
    qr[i] = sign_f32(qv ? Q[head + (size_t)q * D + d0 + i] : 0.f, smode);
    acc[i] = 0.f;
  }
  float m_run = -1e30f, l_run = 0.f;
  const int kv_end = CAUSAL ? min(N, qt * 64 + 64) : N;
  for (int kv0 = 0; kv0 < kv_end; kv0 += BC) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < BC * D; idx += 256) {
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
      for (int i = 0; i < DP; ++i) dot = fmaf(qr[i], Ks[j][d0 + i], dot);
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
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
    for (int i = 0; i < DP; ++i) acc[i] *= alpha;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      const float p = exp2f(fmaf(s[j], c, -m_new));
      rs += p;
#pragma unroll
      for (int i = 0; i < DP; ++i) acc[i] = fmaf(p, Vs[j][d0 + i], acc[i]);
    }
    l_run = l_run * alpha + rs;
  }
  if (qv) {
    const float inv = 1.0f / l_run;
#pragma unroll
    for (int i = 0; i < DP; ++i) O[head + (size_t)q * D + d0 + i] = acc[i] * inv;
    if (d0 == 0) L[(size_t)bh * N + q] = (m_run + log2f(l_run)) * kLn2;
  }
}


// fp32 forward for small problems: the same arithmetic, split further.  A
// workgroup owns 16 query rows; four threads share a row as above.  The
// kF32Waves waves split the keys: wave w takes the 16-key tiles w, w + 8,
// w + 16, ... of the row block's range, each staged in an LDS region of its
// own (its lanes write a tile and then read it, in program order, so the loop
// has no barrier), with its own running max, sum and accumulator.  At the end
// the partial results of each row are merged through LDS the way the online
// update merges blocks.  Small problems are latency bound: the time is the
// serial length of one wave's key loop, which the split of the keys cuts by
// the number of waves, and 16 rows per workgroup spread one head of 128 rows
// over eight workgroups instead of two.  On large problems the 64-row kernel
// is faster: each of its K/V tiles serves four times the rows, in a quarter
// of the LDS.
constexpr int kF32Waves = 8;
// The split kernel runs when the 64-row kernel would launch fewer workgroups
// than this (two per CU of a 256-CU GPU).  Measured: one head of N = 128,
// 34 -> 16 us; four heads of N = 2048, 0.50 -> 0.17 ms; and, past the limit,
// 2.4x slower than the 64-row kernel at 16 heads of N = 4096, d = 128.
constexpr int kF32SplitBelow = 512;
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64 * kF32Waves)
fwd_f32_split_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
                     float* __restrict__ O, float* __restrict__ L, int N, int n_qtiles, float c, uint32_t smode) {
  constexpr int BC = 16;     // keys per tile
  constexpr int RW = 16;     // query rows per workgroup
  constexpr int DP = D / 4;  // columns per thread
  constexpr int KW = kF32Waves;
  constexpr int NT = 64 * KW;  // threads
  // per wave: a K tile and a V tile; after the key loop, the merge area
  __shared__ float sm[KW][2][BC][D];
  static_assert((DP + 2) * NT <= KW * 2 * BC * D, "the merge area fits in the tile regions");
  const int bh = blockIdx.x / n_qtiles;
  const int qt = blockIdx.x % n_qtiles;
  const size_t head = (size_t)bh * N * D;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int d0 = (lane & 3) * DP;
  const int q = qt * RW + (lane >> 2);
  const bool qv = q < N;

  float qr[DP], acc[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) {
    qr[i] = sign_f32(qv ? Q[head + (size_t)q * D + d0 + i] : 0.f, smode);
    acc[i] = 0.f;
  }
  float m_run = -1e30f, l_run = 0.f;
  const int kv_end = CAUSAL ? min(N, qt * RW + RW) : N;
  const int n_tiles = (kv_end + BC - 1) / BC;
  float (*Ks)[D] = sm[wave][0];
  float (*Vs)[D] = sm[wave][1];
  for (int t = wave; t < n_tiles; t += KW) {
    const int kv0 = t * BC;
    for (int idx = lane; idx < BC * D; idx += 64) {
      const int row = idx / D, col = idx % D;
      const int key = kv0 + row;
      Ks[row][col] = key < N ? K[head + (size_t)key * D + col] : 0.f;
      Vs[row][col] = key < N ? V[head + (size_t)key * D + col] : 0.f;
    }
    float s[BC];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < DP; ++i) dot = fmaf(qr[i], Ks[j][d0 + i], dot);
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
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
    for (int i = 0; i < DP; ++i) acc[i] *= alpha;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      const float p = exp2f(fmaf(s[j], c, -m_new));
      rs += p;
#pragma unroll
      for (int i = 0; i < DP; ++i) acc[i] = fmaf(p, Vs[j][d0 + i], acc[i]);
    }
    l_run = l_run * alpha + rs;
  }

  // merge: slot (i, thread) of the area holds accumulator column i, then m and l
  __syncthreads();  // every wave is done with its tiles
  float* mg = &sm[0][0][0][0];
#pragma unroll
  for (int i = 0; i < DP; ++i) mg[i * NT + threadIdx.x] = acc[i];
  mg[DP * NT + threadIdx.x] = m_run;
  mg[(DP + 1) * NT + threadIdx.x] = l_run;
  __syncthreads();
  if (wave == 0 && qv) {
    // a wave that saw no allowed key has m = -1e30 and weight 0; wave 0 holds key 0
    float mw[KW], mmax = -INFINITY;
#pragma unroll
    for (int w = 0; w < KW; ++w) {
      mw[w] = mg[DP * NT + w * 64 + lane];
      mmax = fmaxf(mmax, mw[w]);
    }
    float wt[KW], lt = 0.f;
#pragma unroll
    for (int w = 0; w < KW; ++w) {
      wt[w] = exp2f(mw[w] - mmax);
      lt = fmaf(mg[(DP + 1) * NT + w * 64 + lane], wt[w], lt);
    }
    const float inv = 1.0f / lt;
#pragma unroll
    for (int i = 0; i < DP; ++i) {
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < KW; ++w) o = fmaf(mg[i * NT + w * 64 + lane], wt[w], o);
      O[head + (size_t)q * D + d0 + i] = o * inv;
    }
    if (d0 == 0) L[(size_t)bh * N + q] = (mmax + log2f(lt)) * kLn2;
  }
}

// Longest causal sequence, in 128-row query tiles, that runs as pairs of tiles
// per workgroup (measured: 2.6% faster at 64 tiles, 10% at 32; 1% slower at
// 256, where each workgroup is long anyway and a second head's keys and
// values compete for the XCD's L2).
constexpr int kPairMaxQtiles = 64;

template <int D, bool CAUSAL>
hipError_t launch_fwd_bf16_t(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                             int N, float scale, const BlockMask& m, const DropParams& dr, hipStream_t stream) {
  using C = FwdCfg<D>;
  static_assert(C::BR == kMaskBlock, "a workgroup owns one block row of the mask");
  const int n_qtiles = (N + C::BR - 1) / C::BR;
  const int total = BH * n_qtiles;
  // the one-tile-at-a-time kernel for short sequences exists for d = 64 only
  // (at d = 128 the pipelined kernel's state already limits a CU to two
  // workgroups by LDS as well as registers)
  constexpr bool kShortFwd = D == 64;
  const bool short_seq = kShortFwd && (!CAUSAL || N <= kShortSeqMaxN);
  const ScoreScale sc = split_scale(scale);
  if (m.ptr)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, true, false>), dim3(total), dim3(256), 0, stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse, N, n_qtiles, total,
                       sc.c, m.ptr, m.head_stride, m.nb, 0u, 0u, 0u, 1.f, sc.mode);
  else if (dr.on)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, false, true>), dim3(total), dim3(256), 0, stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse, N, n_qtiles, total,
                       sc.c, (const uint8_t*)nullptr, 0, 0, dr.t, dr.seed_lo, dr.seed_hi, dr.inv_keep, sc.mode);
  else if (short_seq)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, false, false, /*PIPE=*/!kShortFwd>), dim3(total), dim3(256), 0, stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse, N, n_qtiles, total,
                       sc.c, (const uint8_t*)nullptr, 0, 0, 0u, 0u, 0u, 1.f, sc.mode);
  else if (CAUSAL && !short_seq && BH % 8 == 0 && n_qtiles % 2 == 0 && n_qtiles <= kPairMaxQtiles)
    hipLaunchKernelGGL((fwd_bf16_pair_kernel<D>), dim3(total / 2), dim3(256), 0, stream, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, (bf16*)o, lse, N, n_qtiles, total, sc.c, sc.mode);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, false, false>), dim3(total), dim3(256), 0, stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse, N, n_qtiles, total,
                       sc.c, (const uint8_t*)nullptr, 0, 0, 0u, 0u, 0u, 1.f, sc.mode);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_f32_t(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                            int N, float scale, hipStream_t stream) {
  const ScoreScale sc = split_scale(scale);
  const int n_qtiles = (N + 63) / 64;
  if ((int64_t)BH * n_qtiles < kF32SplitBelow) {
    const int n_rt = (N + 15) / 16;
    hipLaunchKernelGGL((fwd_f32_split_kernel<D, CAUSAL>), dim3(BH * n_rt), dim3(64 * kF32Waves), 0, stream,
                       (const float*)q, (const float*)k, (const float*)v, (float*)o, lse, N, n_rt, sc.c, sc.mode);
  } else {
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(BH * n_qtiles), dim3(256), 0, stream, (const float*)q,
                       (const float*)k, (const float*)v, (float*)o, lse, N, n_qtiles, sc.c, sc.mode);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N,
                      int d, bool bf16_in, float scale, bool causal, const BlockMask& m, const DropParams& dr,
                      hipStream_t stream) {
  if (bf16_in) {
    if (d == 64) return causal ? launch_fwd_bf16_t<64, true>(q, k, v, o, lse, BH, N, scale, m, dr, stream)
                               : launch_fwd_bf16_t<64, false>(q, k, v, o, lse, BH, N, scale, m, dr, stream);
    return causal ? launch_fwd_bf16_t<128, true>(q, k, v, o, lse, BH, N, scale, m, dr, stream)
                  : launch_fwd_bf16_t<128, false>(q, k, v, o, lse, BH, N, scale, m, dr, stream);
  }
  if (d == 64) return causal ? launch_fwd_f32_t<64, true>(q, k, v, o, lse, BH, N, scale, stream)
                             : launch_fwd_f32_t<64, false>(q, k, v, o, lse, BH, N, scale, stream);
  return causal ? launch_fwd_f32_t<128, true>(q, k, v, o, lse, BH, N, scale, stream)
                : launch_fwd_f32_t<128, false>(q, k, v, o, lse, BH, N, scale, stream);
}

}  // namespace attn
