// Device-side building blocks shared by the attention kernels (gfx950 only).
//
// Matrix-core conventions (v_mfma_f32_32x32x16_bf16, wave64), checked on the
// hardware:
//   A operand (32 x 16): lane l holds A[l % 32][8 * (l / 32) + e], e = 0..7
//   B operand (16 x 32): lane l holds B[8 * (l / 32) + e][l % 32]
//   C/D       (32 x 32): lane l, register r holds C[8*(r/4) + 4*(l/32) + r%4][l % 32]
// Only the pairing of A's and B's k slots matters for the product, so any
// consistent assignment of the contraction index to (l / 32, e) is valid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max over the lane pair (l, l ^ 32): v_permlane32_swap gives each lane both halves
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Swap bits 2 and 3 of a lane/row index.  Reading operand rows in this order
// makes the C registers of a 32x32 tile line up with 8 consecutive indices per
// lane half when they are reused as the k operand of the next product.
__device__ __forceinline__ int swap23(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// XOR swizzle of the 16-byte chunks of a row-major LDS tile with NCH chunks
// per row.  Physical chunk = logical chunk ^ chunk_swz(row).  It serves both
// read patterns used on the tiles:
//   * ds_read_b128 of one chunk from 16 consecutive rows (any order of the
//     low 4 row bits): the swizzle is a bijection of those bits, so the 16
//     lanes hit 16 different 16-byte bank groups;
//   * ds_read_b64_tr_b16 of 4 adjacent chunks from rows {r, r+8} x r = 0..3
//     (+4): the 4 rows r land in 4 different groups of 4 chunks (2-way at
//     most, the minimum for the 512 bytes such a read moves).
// D = 128 (16 chunks, 256-byte rows): swap the two 2-bit fields of row & 15.
// D = 64 (8 chunks, two rows per 256-byte bank window): bit 2 = row bit 1,
// bits 0-1 = row bits 2-3.
template <int NCH>
__device__ __forceinline__ int chunk_swz(int row) {
  if constexpr (NCH == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Row index (within a 32-row tile whose A-operand rows were read in swap23
// order) held by C register r in lane half g:
//   swap23(8*(r/4) + 4*g + r%4) = 16*(r/8) + 8*g + r%8
__device__ __forceinline__ constexpr int crow(int r, int g) { return 16 * (r / 8) + 8 * g + (r % 8); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// s_waitcnt vmcnt(0) as a real instruction the compiler's wait tracking sees:
// after it no global load is outstanding, so loads issued before a loop do not
// make the loop body wait on loads issued inside it.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// wave-uniform copy of a value that is the same in every lane (lets the
// compiler use scalar branches instead of exec masking)
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Eight consecutive C registers [8h, 8h+8) of a 32x32 fp32 tile, as a bf16x8
// operand (the k = 8 * (l/32) + e slots of the next product).
__device__ __forceinline__ bf16x8 c_to_operand(const f32x16& c, int h) {
  u32x4 u;
  u[0] = pack_bf16x2(c[8 * h + 0], c[8 * h + 1]);
  u[1] = pack_bf16x2(c[8 * h + 2], c[8 * h + 3]);
  u[2] = pack_bf16x2(c[8 * h + 4], c[8 * h + 5]);
  u[3] = pack_bf16x2(c[8 * h + 6], c[8 * h + 7]);
  return __builtin_bit_cast(bf16x8, u);
}

// LDS access helpers (16-byte granularity)
__device__ __forceinline__ bf16x8 lds_read16(const bf16* base, int chunk16) {
  return *reinterpret_cast<const bf16x8*>(base + 8 * chunk16);
}
__device__ __forceinline__ void lds_write16(bf16* base, int chunk16, const u32x4& v) {
  *reinterpret_cast<u32x4*>(base + 8 * chunk16) = v;
}

// Buffer resources: raw (stride 0) descriptors over one head's rows.  Loads
// whose byte offset lies at or past `bytes` return zero, which gives the zero
// fill of ragged tiles without any per-lane compare, and the per-tile offset
// goes in a scalar register so the lane offsets stay loop-invariant.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ u32x2 bload8(rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// Buffer -> LDS direct load (buffer_load_dwordx4 ... lds): lane i of the wave
// writes its 16 bytes at lds_wave_base + 16 * i, bypassing VGPRs.  Tracked by
// vmcnt like any buffer load.
__device__ __forceinline__ void bload16_lds(rsrc_t r, void* lds_wave_base, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff,
                                           soff, 0, 0);
}

// 16-byte global load with zero fill when !valid
__device__ __forceinline__ u32x4 gload16(const bf16* p, bool valid) {
  u32x4 z = {0u, 0u, 0u, 0u};
  return valid ? *reinterpret_cast<const u32x4*>(p) : z;
}

// Select the 16-bit half `half` (0 = low) of two dwords and pack them: low from
// a, high from b.  Used to transpose 2x2 blocks of bf16 pairs in registers.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);  // [a.lo, b.lo]
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);  // [a.hi, b.hi]
}

// Sign of the score scale.  The tiled kernels take a tile's max over the
// unscaled scores and fold c = scale * log2(e) into the exponent FMA, which
// needs c > 0.  A negative or zero scale is applied to the operand a kernel
// holds in registers instead (Q, or K in the key-stationary backward), and
// the kernel runs with c = |scale| log2(e) (log2(e) itself when scale = 0):
//   kSignNeg : the operand's sign bits are flipped (exact), so every score
//              changes sign and |scale| s = scale (q . k);
//   kSignZero: every finite element becomes +0 and every non-finite one NaN,
//              so each score is 0 * (q . k): 0, or NaN where q . k is not finite.
// Products that multiply by the scale itself (dQ, dK) use the signed scale.
enum : uint32_t { kSignPos = 0, kSignNeg = 1, kSignZero = 2 };

// one dword of two packed bf16 values
__device__ __forceinline__ uint32_t sign_word_bf16(uint32_t u, uint32_t mode) {
  if (mode == kSignNeg) return u ^ 0x80008000u;
  if (mode == kSignZero) {
    const uint32_t lo = (u & 0x7F80u) == 0x7F80u ? 0x7FC0u : 0u;
    const uint32_t hi = (u & 0x7F800000u) == 0x7F800000u ? 0x7FC00000u : 0u;
    return lo | hi;
  }
  return u;
}
__device__ __forceinline__ bf16x8 sign_bf16x8(const bf16x8& v, uint32_t mode) {
  u32x4 u = __builtin_bit_cast(u32x4, v);
  u32x4 r;
  r[0] = sign_word_bf16(u[0], mode);
  r[1] = sign_word_bf16(u[1], mode);
  r[2] = sign_word_bf16(u[2], mode);
  r[3] = sign_word_bf16(u[3], mode);
  return __builtin_bit_cast(bf16x8, r);
}
// one fp32 element
__device__ __forceinline__ float sign_f32(float x, uint32_t mode) {
  if (mode == kSignNeg) return -x;
  if (mode == kSignZero) return __builtin_isfinite(x) ? 0.f : __builtin_nanf("");
  return x;
}
// one dword of four OCP e4m3 codes (S.1111.111 is NaN; there is no infinity)
__device__ __forceinline__ uint32_t sign_word_e4m3(uint32_t u, uint32_t mode) {
  if (mode == kSignNeg) return u ^ 0x80808080u;
  if (mode == kSignZero) {
    uint32_t r = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (((u >> (8 * b)) & 0x7Fu) == 0x7Fu) r |= 0x7Fu << (8 * b);
    return r;
  }
  return u;
}

// XCD-aware work index.  Workgroups are handed to the 8 XCDs round-robin by
// linear id; renumbering so that each XCD walks a contiguous range of work
// items keeps the tiles of one head (which share K/V, or Q/dO) in one L2.
__device__ __forceinline__ int xcd_remap(int wid, int total) {
  if ((total & 7) != 0) return wid;
  return (wid & 7) * (total >> 3) + (wid >> 3);
}

// Work item `item` (0 or 1) of workgroup b when each workgroup runs two
// tiles of one head: tile p and tile n - 1 - p (n tiles per head, item index
// i within a head, longest first).  Workgroup b runs on XCD b % 8 and takes
// pair b / 8 of that XCD's work items (whole heads, as in xcd_remap); the
// shorter tile comes first.  Needs (B H) % 8 == 0 and n even.
__device__ __forceinline__ int pair_work(int b, int total, int n, int item) {
  const int x = b & 7, j = b >> 3;
  const int half = n >> 1;
  const int base = x * (total >> 3) + (j / half) * n, p = j % half;
  return item == 0 ? base + n - 1 - p : base + p;
}

// ---- dropout decisions: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011)
// One call maps a 128-bit counter and a 64-bit key to 128 random bits: ten
// rounds of two 32 x 32 -> 64-bit products, with the key advanced by two Weyl
// increments before every round after the first.  Element (i, j) of head bh
// uses the call for counter (j / 4, i / 4, bh, 0), byte 4 (i % 4) + (j % 4)
// of its four little-endian words, and is kept iff that byte >= t.
struct Philox4 {
  uint32_t w[4];
};
__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// Lane i of every quad of lanes reads the value of lane i ^ K (DPP quad_perm).
template <int K>
__device__ __forceinline__ uint32_t quad_xor(uint32_t v) {
  constexpr int ctrl = K == 1 ? 0xB1 : K == 2 ? 0x4E : 0x1B;  // [1,0,3,2], [2,3,0,1], [3,2,1,0]
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t pick4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, int i) {
  return i == 0 ? a0 : i == 1 ? a1 : i == 2 ? a2 : a3;
}

// Dropout words for the 16 scores a lane holds in the S^T layout of one
// 32-key block: the lane owns query row q (q % 4 == lane % 4) and register r
// holds key kb0 + 16 (r / 8) + 8 g + r % 8.  On return word[c] is word q % 4
// of the generator call for keys kb0 + 16 (c / 2) + 8 g + 4 (c % 2) .. + 3, so
// register r is kept iff byte r % 4 of word[r / 4] is >= t.  The four lanes of
// a quad share query group q / 4 and need the same four calls: lane m makes
// call m and the quad exchanges words (lane n takes word n of each).  Every
// lane of the quad must be active.
__device__ __forceinline__ void drop_words_row(int q, int kb0, int g, int bh, uint32_t k0, uint32_t k1,
                                               uint32_t (&word)[4]) {
  const int m = threadIdx.x & 3;
  const uint32_t kg = (uint32_t)(kb0 + 16 * (m >> 1) + 8 * g + 4 * (m & 1)) >> 2;
  const Philox4 w = philox4x32_10(kg, (uint32_t)q >> 2, (uint32_t)bh, 0u, k0, k1);
  const uint32_t own = pick4(w.w[0], w.w[1], w.w[2], w.w[3], m);
  const uint32_t r1 = quad_xor<1>(pick4(w.w[0], w.w[1], w.w[2], w.w[3], m ^ 1));
  const uint32_t r2 = quad_xor<2>(pick4(w.w[0], w.w[1], w.w[2], w.w[3], m ^ 2));
  const uint32_t r3 = quad_xor<3>(pick4(w.w[0], w.w[1], w.w[2], w.w[3], m ^ 3));
#pragma unroll
  for (int c = 0; c < 4; ++c) word[c] = pick4(own, r1, r2, r3, c ^ m);  // call c came from lane c
}

// The same for the S layout of one 32-query block: the lane owns key column
// `key` (key % 4 == lane % 4) and register r holds query qb0 + 16 (r / 8) +
// 8 g + r % 8.  On return byte w of word[c] is byte key % 4 of word w of the
// call for queries qb0 + 16 (c / 2) + 8 g + 4 (c % 2) .. + 3, so register r
// is kept iff byte r % 4 of word[r / 4] is >= t.  Lane m makes call m and
// sends lane n the bytes n of its four words, packed by v_perm_b32.
__device__ __forceinline__ void drop_words_col(int key, int qb0, int g, int bh, uint32_t k0, uint32_t k1,
                                               uint32_t (&word)[4]) {
  const int m = threadIdx.x & 3;
  const uint32_t qg = (uint32_t)(qb0 + 16 * (m >> 1) + 8 * g + 4 * (m & 1)) >> 2;
  const Philox4 w = philox4x32_10((uint32_t)key >> 2, qg, (uint32_t)bh, 0u, k0, k1);
  // bytes n of w0, w1, w2, w3 -> one word (selector 12 gives a zero byte)
  auto gather = [&](int n) {
    const uint32_t sel = (uint32_t)n | ((uint32_t)(4 + n) << 8) | 0x0C0C0000u;
    const uint32_t lo = __builtin_amdgcn_perm(w.w[1], w.w[0], sel);
    const uint32_t hi = __builtin_amdgcn_perm(w.w[3], w.w[2], sel);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
  };
  const uint32_t own = gather(m);
  const uint32_t r1 = quad_xor<1>(gather(m ^ 1));
  const uint32_t r2 = quad_xor<2>(gather(m ^ 2));
  const uint32_t r3 = quad_xor<3>(gather(m ^ 3));
#pragma unroll
  for (int c = 0; c < 4; ++c) word[c] = pick4(own, r1, r2, r3, c ^ m);
}

// keep decision of register r from the words above
__device__ __forceinline__ bool drop_keep(const uint32_t (&word)[4], int r, uint32_t t) {
  return ((word[r >> 2] >> (8 * (r & 3))) & 0xFFu) >= t;
}

// ---- block-sparse masks: one byte per 128 x 128 block of (query, key) pairs
constexpr int kMaskBlock = 128;

// All 256 threads of a workgroup call this with the same arguments.  Writes
// the indices t in [t_begin, t_end) for which on(t) holds, in increasing
// order, to list[0 .. count) and returns count.  `wcnt` is 4 ints of LDS.
template <typename Pred>
__device__ __forceinline__ int compact_indices(uint16_t* list, int* wcnt, int t_begin, int t_end, Pred on) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int count = 0;
  for (int base = t_begin; base < t_end; base += 256) {
    const int t = base + tid;
    const bool act = t < t_end && on(t);
    const uint64_t bal = __builtin_amdgcn_ballot_w64(act);
    const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (lane == 0) wcnt[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int off = count;
    for (int w = 0; w < 4; ++w) off += w < wave ? wcnt[w] : 0;
    if (act) list[off + rank] = (uint16_t)t;
    count += wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
    __syncthreads();  // the list is complete and wcnt free for the next round
  }
  return count;
}

// Entries of the increasing list[0 .. n) that are below `bound` (one wave).
__device__ __forceinline__ int count_below(const uint16_t* list, int n, int bound) {
  const int lane = threadIdx.x & 63;
  int c = 0;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    c += __builtin_popcountll(__builtin_amdgcn_ballot_w64(i < n && (int)list[i] < bound));
  }
  return c;
}

}  // namespace attn
