/*
 * attn.h - C ABI of the exact fused attention library for AMD MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention
 *     O = softmax(scale * Q K^T + mask) V
 * per (batch, head) pair.  Sources for the operation (the pages, by title):
 *   - "What is Flash Attention?" (iania.ai video page), transcript 01:04:
 *     scores S = Q K^T / sqrt(D), row softmax P, output O = P V.
 *   - Same page, transcript 02:38-05:17: one fused kernel, Q kept on chip,
 *     K/V visited in blocks, online softmax with a running max and sum.
 *   - Same page, transcript 06:52-07:24: the backward keeps O and a small
 *     per-row statistic and recomputes P block by block.
 *   - "Atencao exata, acelerada por nunca escrever a grade gigante"
 *     (mentria.ai): block scores, safe softmax, online update, o_flash = o_exact.
 * The N x N score and probability matrices are never stored in device memory.
 *
 * Conventions shared by every entry point:
 *   - Q, K, V, O, dO, dQ, dK, dV are dense row-major [B, H, N, d] arrays
 *     (d fastest), all with the same B, H, N, d.  Pointers are device pointers
 *     aligned to at least 16 bytes.  `dtype` gives their element type.
 *   - lse (the per-row logsumexp L_i = m_i + ln l_i of the scaled, masked
 *     scores, natural log) and delta (D_i = sum_k dO_ik O_ik) are fp32 [B, H, N].
 *   - causal = 1 lets query i attend keys j <= i (square, top-left aligned);
 *     causal = 0 attends all N keys.
 *   - scale is any finite value (usually 1/sqrt(d)).  A negative scale is
 *     the same attention with the sign of every score flipped; scale = 0
 *     gives uniform attention over the allowed keys (L = ln of their count,
 *     dQ = dK = 0).  The kernels run the softmax with |scale| and apply the
 *     sign to an operand they hold in registers (exact for bf16 and e4m3).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; it never synchronises.  The caller owns
 *     all buffers and keeps them alive until the stream has passed the work.
 *   - The library allocates no device memory and keeps no device state, except
 *     the static scratch array of attn_bwd_noalloc (see there); calls of the
 *     other entry points on different streams may run concurrently.  On the
 *     host it caches, per device, two figures it queries once (resident
 *     workgroups of one backward kernel, and the address of the scratch array),
 *     under a lock.
 *   - Validation happens before anything is enqueued.  On any error nothing is
 *     launched and no output is written.  ATTN_OK means "enqueued"; a device
 *     fault shows up at the caller's next synchronisation.
 *   - Supported: dtype ATTN_BF16 with d in {64, 128} for every entry point;
 *     dtype ATTN_F32 with d in {64, 128} for attn_fwd only.  N >= 1 (any N,
 *     not only multiples of the tile size), B, H >= 1, B*H*N < 2^31
 *     (ATTN_ERR_INVALID otherwise), and N <= 2^22 (ATTN_ERR_UNSUPPORTED
 *     otherwise: one head is addressed with 32-bit byte offsets).
 */
#ifndef EXACT_ATTN_H
#define EXACT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 8

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID = 1,     /* null pointer, non-positive size, bad scale/causal, workspace too small */
  ATTN_ERR_UNSUPPORTED = 2, /* d, dtype or (block-sparse) N outside the supported set */
  ATTN_ERR_HIP = 3,         /* the HIP runtime refused a launch */
  ATTN_ERR_SCRATCH = 4      /* attn_bwd_noalloc: B*H*N above attn_bwd_noalloc_max_rows() */
} attn_status_t;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype_t;

/* Forward pass: O = softmax(scale Q K^T + mask) V and L = logsumexp of each
 * row of scale Q K^T + mask.  One fused kernel; per query tile it streams the
 * K/V blocks through on-chip memory with the online softmax (video page,
 * transcript 03:44-05:17; slides, online-update formula).
 *   q, k, v : inputs [B,H,N,d] of `dtype`.
 *   o       : output [B,H,N,d] of `dtype` (rounded to nearest even for bf16).
 *   lse     : output [B,H,N] fp32.  Must not alias any input. */
attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int N, int d, attn_dtype_t dtype, float scale, int causal,
                       void* stream);

/* Bytes of device workspace attn_bwd needs: one fp32 [B,H,N] array (the
 * exact delta, handed from the dq stage to the dkdv stage), B*H*N*4 bytes
 * rounded up to 256.  Pure host arithmetic; returns 0 for invalid sizes. */
size_t attn_bwd_workspace_bytes(int B, int H, int N, int d);

/* Backward pass: gradients of O with respect to Q, K and V for an upstream
 * gradient dO, given the forward's O and L.  P is recomputed tile by tile from
 * Q, K and L (video page, transcript 06:52-07:24); no N x N array is stored.
 * Enqueues the dq stage and then attn_bwd_dkdv.  The dq stage forms
 * delta~ = rowsum(dO * O) itself, bit for bit as attn_bwd_preprocess does,
 * so the result equals preprocess -> attn_bwd_dq -> attn_bwd_dkdv called one
 * by one; it hands the exact delta to the dkdv stage through the workspace.
 *   q, k, v, o, dout : inputs [B,H,N,d] of `dtype`; lse : input [B,H,N] fp32
 *   dq, dk, dv       : outputs [B,H,N,d] of `dtype`
 *   workspace        : device buffer of at least attn_bwd_workspace_bytes(...)
 *                      bytes, holding delta; its contents on entry are ignored. */
attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                       attn_dtype_t dtype, float scale, int causal, void* stream);

/* Backward pass that allocates nothing, for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, kernels
 * and results (bit for bit) as attn_bwd, without the workspace: the exact
 * delta the dq stage hands to the dkdv stage goes to a static device array of
 * 16 MiB that the library holds on each GPU until the process ends.
 *   - B*H*N must be at most attn_bwd_noalloc_max_rows() (4194304), else
 *     ATTN_ERR_SCRATCH and nothing is launched.
 *   - `stream` must belong to the current device; the first call on a device
 *     looks up that device's array (hipGetSymbolAddress) and keeps it.
 *   - Calls on one GPU share its array: two calls whose work overlaps in time
 *     on that GPU (different streams, no ordering between them) race and give
 *     wrong results.  Calls ordered on one stream are fine; the array keeps
 *     the last call's contents, and every entry is rewritten before it is read.
 *   - It calls no hipMalloc, hipFree or other allocating routine. */
attn_status_t attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv,
                               int B, int H, int N, int d, attn_dtype_t dtype, float scale,
                               int causal, void* stream);

/* Largest B*H*N attn_bwd_noalloc accepts. */
size_t attn_bwd_noalloc_max_rows(void);

/* Backward stage 1: delta~_i = sum_k dO_ik * O_ik in fp32.  Mathematically
 * equal to sum_j P_ij dP_ij (the row term of the softmax Jacobian); with O
 * rounded to bf16 it is an approximation: stage 2 uses it for dQ and sums the
 * exact value for stage 3.
 *   o, dout : inputs [B,H,N,d] of `dtype`; delta : output [B,H,N] fp32. */
attn_status_t attn_bwd_preprocess(const void* o, const void* dout, float* delta, int B, int H,
                                  int N, int d, attn_dtype_t dtype, void* stream);

/* Backward stage 3: dK and dV.  One workgroup per block of keys keeps K and V
 * on chip and visits the query blocks, recomputing S = scale Q K^T and
 * P = exp(S - L) per block, then dV += P^T dO, dP = dO V^T,
 * dS = P (dP - delta), dK += scale dS^T Q.
 *   q, k, v, dout : inputs of `dtype`; lse, delta : fp32 inputs [B,H,N]
 *                   (delta: the exact one written by attn_bwd_dq)
 *   dk, dv        : outputs [B,H,N,d] of `dtype`. */
attn_status_t attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                            const void* dout, const float* delta, void* dk, void* dv, int B,
                            int H, int N, int d, attn_dtype_t dtype, float scale, int causal,
                            void* stream);

/* Backward stage 2: dQ and the exact delta.  One workgroup per block of
 * queries keeps Q and dO on chip and visits the key blocks, recomputing
 * P = exp(S - L) and dP = dO V^T per block.  It returns
 * dQ = scale P (dP - delta~) K with delta~ from stage 1 (the rowsum of
 * dO * O as stored), and sums delta_i = sum_j P_ij dP_ij in fp32 from the same
 * P and dP for stage 3, whose dK multiplies delta's error by Q.  No atomics:
 * the result is deterministic.
 *   q, k, v, dout : inputs of `dtype`; lse, delta : fp32 inputs [B,H,N]
 *   dq            : output [B,H,N,d] of `dtype`
 *   delta_out     : output [B,H,N] fp32, the exact delta (may not alias delta). */
attn_status_t attn_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                          const void* dout, const float* delta, void* dq, float* delta_out, int B,
                          int H, int N, int d, attn_dtype_t dtype, float scale, int causal,
                          void* stream);

/* Backward stages 1 and 2 in one launch, the dq stage that attn_bwd runs: as
 * attn_bwd_preprocess followed by attn_bwd_dq, bit for bit, but delta~ is
 * formed from O and dO inside the dq kernel (each workgroup reads the O rows
 * of its queries once) instead of going through memory.
 *   q, k, v, o, dout : inputs [B,H,N,d] of `dtype`; lse : fp32 input [B,H,N]
 *   dq               : output [B,H,N,d] of `dtype`
 *   delta_out        : output [B,H,N] fp32, the exact delta for attn_bwd_dkdv. */
attn_status_t attn_bwd_dq_fused(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dout, void* dq, float* delta_out,
                                int B, int H, int N, int d, attn_dtype_t dtype, float scale,
                                int causal, void* stream);

/* Block-sparse attention.  The FlashAttention talk transcript
 * (youtube-distilled.com, FThvfkXWqtE), questions after the method part:
 * the tiled method also takes imposed sparsity, and skips the computation it
 * removes.  Here the sparsity is a block mask over 128 x 128 blocks of
 * (query, key) pairs: pair (i, j) takes part iff its block is on, j < N and,
 * when causal, j <= i.  Kernels skip the tiles of blocks that are off.
 *   block_mask : device array of uint8, [mask_heads, nb, nb] row-major with
 *                nb = ceil(N / 128); entry [h][r][c] != 0 switches on the pairs
 *                of query rows 128 r .. 128 r + 127 and keys 128 c .. 128 c + 127.
 *                Read only; caller-owned like every other buffer.
 *   mask_heads : 1 (one mask for every (batch, head) pair) or B * H (one per
 *                pair, in the [B, H] order of the tensors).
 * A query row with no allowed key gets O = 0, L = -inf, dQ = 0, and adds
 * nothing to dK or dV.  Other arguments, layouts and errors are those of
 * attn_fwd / attn_bwd.  Supported: dtype ATTN_BF16, d in {64, 128},
 * N <= 65536 (ATTN_ERR_UNSUPPORTED otherwise); a null block_mask or any other
 * mask_heads is ATTN_ERR_INVALID. */
attn_status_t attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                                    const uint8_t* block_mask, int mask_heads, int B, int H, int N, int d,
                                    attn_dtype_t dtype, float scale, int causal, void* stream);

/* Backward of attn_fwd_block_sparse, with the same mask: preprocess, dq and
 * dkdv stages as in attn_bwd, each skipping the tiles of blocks that are off.
 * Workspace: attn_bwd_workspace_bytes(B, H, N, d) bytes, as for attn_bwd. */
attn_status_t attn_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o,
                                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                    const uint8_t* block_mask, int mask_heads, void* workspace,
                                    size_t workspace_bytes, int B, int H, int N, int d, attn_dtype_t dtype,
                                    float scale, int causal, void* stream);

/* Attention with dropout on P.  The FlashAttention talk transcript
 * (youtube-distilled.com, FThvfkXWqtE): standard attention optionally applies
 * dropout to the softmax output before the product with V, and the fused
 * kernel drops entries without writing them out, while the gradients use the
 * same decisions.  Here O = (Z * P / (1 - rate)) V with Z_ij in {0, 1}; L is
 * the logsumexp without dropout.  Z is regenerated, never stored: element
 * (i, j) of head bh = b * H + h takes the Philox4x32-10 output (Salmon et
 * al., SC 2011) for counter (j / 4, i / 4, bh, 0) and key (seed mod 2^32,
 * seed / 2^32), byte 4 (i % 4) + (j % 4) of its four little-endian words, and
 * is kept iff that byte >= t with t = round(256 * p_drop); the rate applied
 * is exactly t / 256.
 *   p_drop : requested rate, finite, with round(256 p_drop) in [0, 255]
 *            (ATTN_ERR_INVALID otherwise); 0 gives plain attention.
 *   seed   : the 64-bit generator key; the backward must get the forward's.
 * Other arguments, layouts and errors are those of attn_fwd / attn_bwd.
 * Supported: dtype ATTN_BF16, d in {64, 128}. */
attn_status_t attn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, float p_drop,
                               uint64_t seed, int B, int H, int N, int d, attn_dtype_t dtype, float scale,
                               int causal, void* stream);

/* Backward of attn_fwd_dropout with the same p_drop and seed: dV = (Z P / (1 - rate))^T dO,
 * dP = Z dO V^T / (1 - rate), dS = P (dP - delta), dQ = scale dS K, dK = scale dS^T Q.
 * Workspace: attn_bwd_workspace_bytes(B, H, N, d) bytes, as for attn_bwd. */
attn_status_t attn_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                               const void* dout, void* dq, void* dk, void* dv, float p_drop, uint64_t seed,
                               void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                               attn_dtype_t dtype, float scale, int causal, void* stream);

/* Decode against a KV cache.  "What is Flash Attention?" (iania.ai video
 * page, English): memory-bound inference with long prompts (10:00) and the KV
 * cache for fast generation (11:02-11:33).  Nq new queries per (batch, head)
 * attend to the Nk keys and values held in the cache:
 *     O = softmax(scale q K^T + mask) V,  L = logsumexp per query row.
 * causal = 1 places the queries at the last Nq positions (query i sees keys
 * j <= Nk - Nq + i); causal = 0 lets every query see all Nk keys.  The keys
 * are split into chunks whose partial results are merged with the online
 * softmax rule of the same page (04:46-05:17).
 *   q          : [B, H, Nq, d] bf16        o   : output [B, H, Nq, d] bf16
 *   k/v_cache  : [B, H, Nk, d] bf16        lse : output [B, H, Nq] fp32
 *   workspace  : device buffer of attn_decode_workspace_bytes(B, H, Nq, Nk, d)
 *                bytes (partial results; contents on entry ignored)
 * Supported: dtype ATTN_BF16, d in {64, 128}, 1 <= Nq <= 8, Nk <= 2^23
 * (ATTN_ERR_UNSUPPORTED otherwise); causal needs Nq <= Nk; B*H*Nk < 2^31.
 * attn_decode_workspace_bytes returns 0 for arguments attn_decode rejects.
 * Other conventions as above (caller-owned buffers, enqueue only). */
size_t attn_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d);
attn_status_t attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                          void* workspace, size_t workspace_bytes, int B, int H, int Nq, int Nk, int d,
                          attn_dtype_t dtype, float scale, int causal, void* stream);

/* FP8 forward.  "What is Flash Attention?" (iania.ai video page, English),
 * 09:29: the third generation of the method adds an FP8 forward.  Q, K, V are
 * OCP OFP8 E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * S.1111.111 is NaN; largest finite 448; the bytes of torch.float8_e4m3fn)
 * with one fp32 scale per tensor: the value of code x of Q is descale_q * x.
 * Computes the attention of the dequantized tensors:
 *     S = scale * (descale_q Q)(descale_k K)^T,  O = softmax(S + mask) (descale_v V),
 *     L = logsumexp of each row of S + mask (natural log).
 * Accuracy: S and l are formed in fp32 from exact fp8 products; P is rounded
 * to e4m3 (nearest even, in units of a reference max within 2^8 of the row
 * max) before the product with V, so each O element carries an error of at
 * most [2^-4 sum_j p_j |v_j| + 2^-10 sum_{p_j < 2^-6} |v_j|] / sum_j p_j
 * (p_j = e^(S_j - max S) of its row) plus the bf16 rounding of O.
 *   q, k, v : [B, H, N, d] uint8 e4m3 codes, 16-byte aligned; NaN codes give NaN.
 *   descale_q, descale_k, descale_v : finite and > 0; scale is any finite
 *             value, and |scale * descale_q * descale_k| must be a finite
 *             fp32 value that is not 0 unless scale is 0.
 *   o   : output [B, H, N, d] bf16 (round to nearest even).
 *   lse : output [B, H, N] fp32.
 * Supported: d in {64, 128}, N <= 2^22 (ATTN_ERR_UNSUPPORTED otherwise);
 * causal as for attn_fwd.  Other conventions as above. */
attn_status_t attn_fwd_fp8(const void* q, const void* k, const void* v, float descale_q, float descale_k,
                           float descale_v, void* o, float* lse, int B, int H, int N, int d, float scale,
                           int causal, void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* attn_status_string(attn_status_t s);

/* ATTN_ABI_VERSION of the built library. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTN_H */
