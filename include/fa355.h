/*
 * fa355.h -- C ABI of libfa355: exact, IO-aware attention on AMD MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   "FA notes"  = the close-reading notes "精读笔记 08：FlashAttention"
 *                 (llm-papers-study.pages.dev) on the FlashAttention paper;
 *   "S12"       = chapter "S12 FlashAttention" of an LLM-inference course
 *                 (llminference.xinbetween.com/zh/s12).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The library
 *     allocates, frees and caches nothing, and keeps no state between calls
 *     (one exception: fa_decode_paged_noalloc uses a fixed device array that
 *     the library itself holds, see there).
 *   - Every call only enqueues work on `stream` (a hipStream_t passed as void*;
 *     NULL means the null stream) and returns without synchronising.  Calls are
 *     reentrant; calls that share output or workspace buffers must be ordered
 *     by the caller.
 *   - Arguments are validated before anything is launched.  An invalid argument
 *     returns a negative fa_status and has no side effect.  A launch failure
 *     reported by the HIP runtime returns FA_E_HIP.  The contents of device
 *     arrays (kv_len values, block-table entries, sequence lengths) are the
 *     caller's contract: the kernels clamp malformed values so that no access
 *     leaves the buffers, but the results are then unspecified.  The debug
 *     build of the library checks these contents (fa_debug_flags).
 *   - Tensors are contiguous, row-major, with the layouts stated per argument.
 *     bf16 means IEEE bfloat16 storage; results are rounded to nearest even.
 *   - The score scale is applied before the row max: S = scale * Q K^T.  S12's
 *     recurrence uses scale = 1/sqrt(d); FA notes §2.1 states the unscaled form.
 */
#ifndef FA355_H
#define FA355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F32 = 0, FA_BF16 = 1 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_E_NULLPTR = -1,     /* a required pointer is NULL                         */
  FA_E_SHAPE = -2,       /* a size is out of range or inconsistent             */
  FA_E_UNSUPPORTED = -3, /* a valid request the library does not implement     */
  FA_E_WORKSPACE = -4,   /* workspace missing or smaller than the query says   */
  FA_E_HIP = -5,         /* the HIP runtime reported an error at launch        */
  FA_E_SCRATCH = -6      /* request larger than the library's fixed scratch    */
} fa_status;

/* Human-readable name of a status code (static string, never NULL). */
const char *fa_status_str(int status);

/*
 * fa_last_hip_error -- the hipError_t value behind the calling thread's most
 * recent FA_E_HIP (hipSuccess = 0 if there has been none); it is not reset by
 * later successful calls.  fa_last_hip_error_str is HIP's own text for it
 * (static storage, never NULL).  Neither touches the device.
 */
int fa_last_hip_error(void);
const char *fa_last_hip_error_str(void);

/*
 * Debug build.  The library built with FA355_DEBUG defined (libfa355_debug.so
 * beside libfa355.so) runs, on the call's stream and ahead of the call's own
 * kernels, a small check of every device array whose contents the call
 * relies on, and ORs a bit per kind of violation into a word kept on each
 * device.  The call's kernels then run exactly as in the ordinary build, so
 * outputs are unchanged; the check adds one launch per contract array.
 *
 *   FA_CHECK_KV_LEN       a kv_len[b] outside [0, N].
 *   FA_CHECK_CU_SEQLENS   cu_seqlens not 0 = cu[0] <= cu[1] <= ... <= cu[B]
 *                         = total, or a sequence longer than max_seqlen
 *                         (max_q for fa_prefill_paged).
 *   FA_CHECK_SEQ_LENS     a seq_lens[b] outside [0, max_blocks_per_seq *
 *                         block_size], or (fa_prefill_paged) smaller than the
 *                         sequence's new-token count.
 *   FA_CHECK_BLOCK_TABLE  a block-table entry the call reads (t <
 *                         ceil(seq_len / block_size), seq_len clamped as the
 *                         kernels clamp it) outside [0, num_blocks).
 *
 * fa_debug_flags waits for all work on the current device, stores that
 * device's word in *flags and, if clear is nonzero, resets the word to 0.
 * The word is sticky: it keeps the bits of every call since the last clear.
 * Returns FA_E_NULLPTR for a NULL flags, FA_E_HIP if the runtime fails, and
 * FA_E_UNSUPPORTED (touching nothing) in the ordinary build, which checks
 * nothing.
 */
enum {
  FA_CHECK_KV_LEN = 1,
  FA_CHECK_CU_SEQLENS = 2,
  FA_CHECK_SEQ_LENS = 4,
  FA_CHECK_BLOCK_TABLE = 8
};
int fa_debug_flags(uint32_t *flags, int clear);

/*
 * fa_fwd -- exact attention forward, O = softmax(scale * Q K^T) V.
 *
 * Computes FA notes §2.1 (standard attention) with the tiled, fused method of
 * FA notes §3.2 / §3.4: key/value tiles stream through on-chip memory and the
 * online-softmax recurrence of FA notes §3.1 / S12 ("core idea") carries the
 * running max m and sum l, so the N x N score matrix never reaches HBM.
 *
 *   dtype   FA_BF16 (bf16 in and out, fp32 accumulation) or FA_F32 (fp32).
 *   B, H    batch and heads, >= 1.
 *   N       sequence length, 1 <= N <= 1<<20 (queries and keys alike).
 *   d       head dimension, 64 or 128.
 *   q,k,v   [B,H,N,d] of `dtype`.
 *   o       [B,H,N,d] of `dtype`, written.
 *   m, l    [B,H,N] fp32, written, or both NULL to skip.  m is the row max of
 *           the scaled visible scores (natural-log units) and l = sum over
 *           visible keys of exp(S - m): the statistics FA notes §3.3 keeps for
 *           the backward pass.  A row with no visible key gets o = 0, l = 0,
 *           m = -inf.
 *   kv_len  NULL (all N keys valid) or device int32 [B]: keys j >= kv_len[b]
 *           are masked for batch b (key padding).  Values must be in [0, N].
 *   causal  nonzero: key j is visible to query i only if j <= i.
 *   scale   score scale, finite and > 0 (1/sqrt(d) for standard attention).
 *   stream  hipStream_t.
 * Masked scores are excluded exactly (never a finite penalty); the running
 * max starts at a finite negative so a fully masked tile cannot produce NaN
 * (S12, box on exp(-inf - -inf)).
 */
int fa_fwd(int dtype, int B, int H, int N, int d,
           const void *q, const void *k, const void *v, void *o,
           float *m, float *l, const int32_t *kv_len, int causal, float scale,
           void *stream);

/*
 * fa_fwd_fp8 -- the forward of fa_fwd with FP8 operands.  The pages name FP8
 * support only as a FlashAttention-3 feature (S12, production-practice list)
 * and give no scaling convention; this entry point takes E4M3
 * codes (OCP "E4M3FN": bias 7, no infinities, max 448) with one fp32
 * descale per (batch, head) and tensor: the real inputs are code * descale.
 * Both products run on the FP8 matrix instructions.  The probabilities are
 * rounded to E4M3 before the P V product (after a 2^6 shift that keeps
 * them inside the format's range), so O carries a relative error of up to
 * 2^-4 per probability on top of the input quantisation; m and l are
 * computed in fp32 from the unrounded probabilities.
 *
 *   B, H, N, d, kv_len, causal, scale, stream   as for fa_fwd.
 *   q, k         [B,H,N,d] E4M3 codes (uint8), 16-byte aligned.
 *   v_t          V transposed: [B,H,d,ldv] E4M3 codes, 16-byte aligned
 *                (V's key axis is the contraction axis of P V, so it is the
 *                contiguous one; a quantisation pass can write it so).
 *                Columns >= N (and >= kv_len[b]) are ignored.
 *   ldv          row stride of v_t in bytes: >= N and a multiple of 16.
 *   q_descale,
 *   k_descale,
 *   v_descale    device fp32 [B*H] (index b*H + h), finite and > 0, or
 *                NULL for 1.
 *   o            [B,H,N,d] bf16, written.
 *   m, l         [B,H,N] fp32 as for fa_fwd (statistics of the scaled
 *                scores of the dequantised inputs), or both NULL.
 */
int fa_fwd_fp8(int B, int H, int N, int d, const void *q, const void *k,
               const void *v_t, int ldv, const float *q_descale,
               const float *k_descale, const float *v_descale, void *o,
               float *m, float *l, const int32_t *kv_len, int causal,
               float scale, void *stream);

/*
 * fa_bwd_workspace_bytes -- device workspace fa_bwd needs for this shape: two
 * fp32 row vectors [B,H,N] (D = rowsum(dO * O) and the log2-domain row
 * offset m*log2(e) + log2(l)), each padded to 256 bytes.  Returns 0 for
 * invalid sizes.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * fa_bwd -- gradients of exact attention by recomputation (FA notes §3.3):
 * score and probability tiles are rebuilt on chip from Q, K and the saved
 * statistics (m, l) instead of being stored.  The gradient formulas are the
 * softmax chain rule (the pages do not print them):
 *   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
 *   dQ = scale dS K,  dK = scale dS^T Q.
 *
 *   B, H, N, d, kv_len, causal, scale   as for fa_fwd (bf16 only).
 *   q, k, v, o, dout  [B,H,N,d] bf16: the forward inputs, its output and dL/dO.
 *   m, l              [B,H,N] fp32 as written by fa_fwd for the same inputs.
 *   dq, dk, dv        [B,H,N,d] bf16, all written.  Keys masked by kv_len get
 *                     dk = dv = 0 exactly.
 *   workspace         device memory of at least fa_bwd_workspace_bytes(...)
 *                     bytes, 256-byte aligned; contents on entry are ignored.
 */
int fa_bwd(int B, int H, int N, int d,
           const void *q, const void *k, const void *v, const void *o,
           const void *dout, const float *m, const float *l,
           const int32_t *kv_len, int causal, float scale,
           void *dq, void *dk, void *dv,
           void *workspace, size_t workspace_bytes, void *stream);

/*
 * fa_fwd_dropout -- fa_fwd (bf16) with dropout on the probability matrix,
 * fused into the kernel: FA notes §2.1 counts dropout on P among the
 * memory-bound element-wise steps of standard attention and §3.4 lists it
 * among the operations done on chip, so the dropped matrix never reaches HBM.
 * The pages fix no generator.  This library draws the keep decisions from
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
 * Easy as 1, 2, 3", SC 2011), a counter-based generator, so that the backward
 * pass regenerates the same mask instead of storing it:
 *   for head bh = b*H + h, query i, key j:
 *     g = 2*(j/32) + (j/8)%2,   t = 8*((j/16)%2) + j%8,
 *     words = Philox4x32-10(counter (i, g, bh, offset),
 *                           key (seed & 0xffffffff, seed >> 32)),
 *     byte  = bits 8*(t%4) .. 8*(t%4)+7 of words[t/4],
 *     keep(i, j) = byte >= T,   T = floor(256 p_drop + 1/2).
 *   O = (P * keep * 256/(256 - T)) V with P the softmax of the visible
 *   scores; so the drop probability is T/256 exactly (p_drop rounded to a
 *   multiple of 1/256) and the output is unbiased.
 *
 *   B, H, N, d, q, k, v, o, kv_len, causal, scale, stream   as for fa_fwd
 *                 (dtype bf16).
 *   m, l          as for fa_fwd: the statistics of the softmax BEFORE
 *                 dropout (what fa_bwd_dropout needs), or both NULL.
 *   p_drop        drop probability, 0 <= p_drop and T <= 255 (p_drop <
 *                 255.5/256); otherwise FA_E_SHAPE.  p_drop = 0 gives the
 *                 results of fa_fwd exactly.
 *   seed, offset  the generator's key and fourth counter word: calls that
 *                 differ in either draw independent masks.
 */
int fa_fwd_dropout(int B, int H, int N, int d, const void *q, const void *k,
                   const void *v, void *o, float *m, float *l,
                   const int32_t *kv_len, int causal, float scale,
                   float p_drop, uint64_t seed, uint32_t offset,
                   void *stream);

/*
 * fa_bwd_dropout -- gradients of fa_fwd_dropout with the same (p_drop, seed,
 * offset): the mask is regenerated on chip, not read.  With Z = keep *
 * 256/(256 - T):  dV = (P*Z)^T dO,  dP = (dO V^T) * Z,  D = rowsum(dO * O),
 * dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
 *   Arguments as for fa_bwd plus p_drop, seed, offset as for fa_fwd_dropout
 *   (o, m, l are what fa_fwd_dropout wrote).  Workspace:
 *   fa_bwd_workspace_bytes(B, H, N, d) bytes.
 */
int fa_bwd_dropout(int B, int H, int N, int d, const void *q, const void *k,
                   const void *v, const void *o, const void *dout,
                   const float *m, const float *l, const int32_t *kv_len,
                   int causal, float scale, float p_drop, uint64_t seed,
                   uint32_t offset, void *dq, void *dk, void *dv,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * fa_fwd_block_sparse -- block-sparse attention (FA notes §4.4): the score
 * matrix is cut into 128 x 128 blocks and only the blocks the mask allows
 * are computed; masked blocks are skipped, not loaded.  Exact attention
 * under the mask (an approximation of full attention).  bf16 only.
 *
 *   B, H, N, d, q, k, v, o, m, l, causal, scale, stream   as for fa_fwd
 *                (dtype bf16).
 *   block_mask   device uint8 [H, nb, nb], nb = ceil(N / 128), shared by
 *                the batch: nonzero at [h, i, j] lets queries 128i .. see
 *                keys 128j .. (also subject to the causal rule).  A query
 *                row left with no visible key gets o = 0, l = 0, m = -inf.
 */
int fa_fwd_block_sparse(int B, int H, int N, int d, const void *q,
                        const void *k, const void *v, void *o, float *m,
                        float *l, const uint8_t *block_mask, int causal,
                        float scale, void *stream);

/*
 * fa_bwd_block_sparse_workspace_bytes -- device workspace fa_bwd_block_sparse
 * needs: fa_bwd_workspace_bytes(B, H, N, d) plus two [2][H * ceil(N/128)]
 * int32 arrays (the work of each (head, 128-block) item of the two passes,
 * and the items ordered heaviest first), each padded to 256 bytes.  Returns
 * 0 for shapes fa_bwd_workspace_bytes rejects.
 */
size_t fa_bwd_block_sparse_workspace_bytes(int B, int H, int N, int d);

/*
 * fa_bwd_block_sparse -- gradients of fa_fwd_block_sparse (the chain rule
 * of fa_bwd under the mask; masked blocks are skipped).  Arguments as for
 * fa_bwd without kv_len, plus the same block_mask; the workspace (256-byte
 * aligned, contents on entry ignored) is at least
 * fa_bwd_block_sparse_workspace_bytes(B, H, N, d) bytes, else
 * FA_E_WORKSPACE.  Two small kernels first count the blocks each key
 * column and query row of the mask allows and sort the (head, block) items
 * by that count, so the items with most work start first (a column every
 * row allows can carry many times the average).  Keys no query sees get
 * dk = dv = 0; queries that see no key get dq = 0.
 */
int fa_bwd_block_sparse(int B, int H, int N, int d, const void *q,
                        const void *k, const void *v, const void *o,
                        const void *dout, const float *m, const float *l,
                        const uint8_t *block_mask, int causal, float scale,
                        void *dq, void *dk, void *dv, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * fa_fwd_varlen -- fa_fwd on a packed ragged batch (variable-length prefill).
 * S12's NaN box: under a causal mask on a ragged batch whole tiles are
 * routinely masked; the finite running-max start covers them.  The B
 * sequences lie back to back along one token axis per head: sequence b is
 * tokens cu_seqlens[b] .. cu_seqlens[b+1]-1, and a token attends only tokens
 * of its own sequence (and, when causal, only those at or before it).
 *
 *   dtype, d, causal, scale, stream   as for fa_fwd.
 *   B            sequences, >= 1.
 *   H            heads, >= 1.
 *   total        tokens per head, >= 0 (0: nothing to do, FA_OK; the
 *                buffers may then be NULL).
 *   max_seqlen   1 .. 1<<20, at least every sequence's length.
 *   cu_seqlens   device int32 [B+1]: 0 = cu[0] <= cu[1] <= ... <= cu[B] =
 *                total.  Boundaries outside [0, total] are clamped and
 *                lengths above max_seqlen are cut to it, so malformed values
 *                give unspecified results but no access outside the buffers.
 *   q, k, v, o   [H, total, d] of `dtype` (head-major packed: head h's
 *                tokens are rows h*total .. h*total+total-1); o written.
 *   m, l         [H, total] fp32, written, or both NULL.
 * Sequences of length 0 are allowed.  kv_len padding does not apply.
 */
int fa_fwd_varlen(int dtype, int B, int H, int total, int max_seqlen, int d,
                  const int32_t *cu_seqlens, const void *q, const void *k,
                  const void *v, void *o, float *m, float *l, int causal,
                  float scale, void *stream);

/*
 * fa_bwd_varlen_workspace_bytes -- device workspace fa_bwd_varlen needs: two
 * fp32 vectors [H, total], each padded to 256 bytes.  Returns 0 when total is
 * 0 (no workspace needed) and for invalid sizes.
 */
size_t fa_bwd_varlen_workspace_bytes(int H, int total, int d);

/*
 * fa_bwd_varlen -- fa_bwd on a packed ragged batch (the layout and masking
 * of fa_fwd_varlen; bf16 only).
 *
 *   B, H, total, max_seqlen, d, cu_seqlens, causal, scale   as for
 *                     fa_fwd_varlen.
 *   q, k, v, o, dout  [H, total, d] bf16; m, l [H, total] fp32 as written by
 *                     fa_fwd_varlen for the same inputs.
 *   dq, dk, dv        [H, total, d] bf16, written.
 *   workspace         at least fa_bwd_varlen_workspace_bytes(H, total, d)
 *                     bytes, 256-byte aligned (may be NULL when total = 0).
 */
int fa_bwd_varlen(int B, int H, int total, int max_seqlen, int d,
                  const int32_t *cu_seqlens, const void *q, const void *k,
                  const void *v, const void *o, const void *dout,
                  const float *m, const float *l, int causal, float scale,
                  void *dq, void *dk, void *dv, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * fa_prefill_paged -- exact attention of a packed chunk of new tokens per
 * sequence against a paged KV cache (prefill / chunked prefill with a
 * cached prefix).  S12's paged loop (logical block t of a sequence is
 * physical block block_table[t]; the last block holds n = min(block_size,
 * seq_len - t*block_size) tokens) with GQA head sharing (S12 production
 * paragraph), run by the tiled forward of fa_fwd.
 *
 *   B              sequences (>= 1).
 *   Hq, Hkv        query and KV heads; Hq % Hkv == 0, query head h reads KV
 *                  head h / (Hq/Hkv).
 *   d              64 or 128.
 *   total_q        new tokens of all sequences (>= 0; 0: nothing to do).
 *   max_q          1 .. 1<<20, at least every sequence's new-token count.
 *   cu_seqlens_q   device int32 [B+1]: sequence b's new tokens are packed rows
 *                  cu[b] .. cu[b+1]-1 (malformed values are clamped as for
 *                  fa_fwd_varlen).
 *   q, o           [Hq, total_q, d] bf16 (head-major packed); o written.
 *   m, l           [Hq, total_q] fp32 written, or both NULL.
 *   v_cache        [num_blocks, Hkv, block_size, d] bf16, holding the V of
 *                  every token of each sequence, its new tokens included.
 *   k_cache        the same blocks of K, stored in 32-element groups as for
 *                  fa_decode_paged: [num_blocks, Hkv, d/32, block_size, 32].
 *   block_size     16.
 *   max_blocks_per_seq  >= 1, with B * max_blocks_per_seq and
 *                  max_blocks_per_seq * 16 below 2^31 (else FA_E_SHAPE).
 *   block_table    device int32 [B, max_blocks_per_seq]; entries for t <
 *                  ceil(seq_len/16) must be in [0, num_blocks) (others are
 *                  clamped into that range, giving unspecified results).
 *   seq_lens       device int32 [B]: cached tokens of sequence b, new ones
 *                  included (clamped to max_blocks_per_seq * 16).  The new
 *                  tokens are its last qlen_b = cu[b+1]-cu[b] positions: new
 *                  token i sits at position seq_lens[b] - qlen_b + i.
 *   causal         nonzero: a new token sees cached positions <= its own.
 *   scale          finite, > 0.
 */
int fa_prefill_paged(int B, int Hq, int Hkv, int d, int total_q, int max_q,
                     const int32_t *cu_seqlens_q, const void *q,
                     const void *k_cache, const void *v_cache, int num_blocks,
                     int block_size, const int32_t *block_table,
                     int max_blocks_per_seq, const int32_t *seq_lens,
                     int causal, float scale, void *o, float *m, float *l,
                     void *stream);

/*
 * fa_decode_workspace_bytes -- device workspace fa_decode_paged needs: the
 * per-split partial triples (m, l, o) in fp32.  Returns 0 for invalid sizes.
 */
size_t fa_decode_workspace_bytes(int B, int Hq, int d, int num_splits);

/*
 * fa_decode_paged -- one decode step: each sequence's single query token
 * attends to its whole paged KV cache.
 *
 * S12 ("implement it") gives the paged loop: logical block t of sequence b
 * lives in physical block block_table[b*max_blocks_per_seq + t] and the last
 * block holds n = min(block_size, seq_len - t*block_size) valid slots.  S12's
 * production-practice paragraph adds GQA head sharing and its "unlocks"
 * paragraph gives flash-decoding: the key range is split over workers whose
 * partial (m, l, o) triples are merged with the FA notes §3.1 rule.
 *
 *   B            sequences (>= 1).
 *   Hq, Hkv      query and KV heads; Hq % Hkv == 0, query head h reads KV head
 *                h / (Hq / Hkv).  Every group size Hq / Hkv from 1 to 16 is
 *                supported (one that is not a power of two runs on the
 *                kernel of the next power of two, its extra matrix columns
 *                unused); above 16, FA_E_UNSUPPORTED.
 *   d            head dimension, 64 or 128.
 *   q            [B,Hq,d] bf16.
 *   v_cache      [num_blocks, Hkv, block_size, d] bf16 (head-major within a
 *                block: one KV head's block_size x d tile is contiguous).
 *   k_cache      [num_blocks, Hkv, d/32, block_size, 32] bf16: the same
 *                tiles of K stored in 32-element groups, element 32g + j of
 *                token u of a head's block at [.., g, u, j], so that group g
 *                of the block's 16 tokens is 1 KiB contiguous (a layout of
 *                this library; the pages index a block by token).  A head's
 *                tile sits at the same offset in both caches.
 *                Slots past a sequence's length are never read into the
 *                arithmetic (they may hold anything, NaN included).
 *   block_size   tokens per block; 16.
 *   max_blocks_per_seq  >= 1; B * max_blocks_per_seq and
 *                max_blocks_per_seq * block_size must stay below 2^31
 *                (else FA_E_SHAPE).
 *   block_table  device int32 [B, max_blocks_per_seq]; entries for t <
 *                ceil(seq_len/block_size) must be in [0, num_blocks).  An
 *                entry outside that range is skipped (its tokens are treated
 *                as masked) rather than read.
 *   seq_lens     device int32 [B], each in [0, max_blocks_per_seq*block_size].
 *                A sequence of length 0 gets out = 0.
 *   num_splits   1..64: each sequence's blocks are cut into num_splits
 *                contiguous ranges of ceil(blocks/num_splits) blocks.
 *   scale        finite, > 0 (1/sqrt(d) for standard attention).
 *   out          [B,Hq,d] bf16, written.
 *   workspace    at least fa_decode_workspace_bytes(B,Hq,d,num_splits) bytes.
 */
int fa_decode_paged(int B, int Hq, int Hkv, int d,
                    const void *q, const void *k_cache, const void *v_cache,
                    int num_blocks, int block_size,
                    const int32_t *block_table, int max_blocks_per_seq,
                    const int32_t *seq_lens, int num_splits, float scale,
                    void *out, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * fa_decode_paged_noalloc -- fa_decode_paged for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments, kernels and results (bitwise),
 * without the workspace.  The per-split partial triples live instead in a
 * fixed array of FA_DECODE_SCRATCH_BYTES bytes that the library holds on
 * each GPU it runs on until the process ends.  The call itself allocates
 * nothing: no hipMalloc, hipFree or allocating library routine.
 *
 *   Limit     fa_decode_workspace_bytes(B, Hq, d, num_splits) must not exceed
 *             FA_DECODE_SCRATCH_BYTES (8 MiB: e.g. B * Hq * num_splits up to
 *             16,128 at d = 128), else FA_E_SCRATCH, touching nothing.
 *   Sharing   every call on one GPU uses that GPU's one array.  Calls that
 *             may overlap on one GPU (other streams, other threads, other
 *             processes' contexts excepted) race and must be ordered by the
 *             caller, e.g. by issuing them on one stream.  The array keeps
 *             the last call's partials; nothing in it needs to start at zero,
 *             since each call writes every partial it reads.
 *   Set-up    the first call on a device (with that device current) looks up
 *             the device address of that GPU's copy of the array; a failure
 *             there returns FA_E_HIP.
 * Other arguments and errors: as fa_decode_paged.
 */
#define FA_DECODE_SCRATCH_BYTES ((size_t)8 << 20)
int fa_decode_paged_noalloc(int B, int Hq, int Hkv, int d,
                            const void *q, const void *k_cache,
                            const void *v_cache, int num_blocks,
                            int block_size, const int32_t *block_table,
                            int max_blocks_per_seq, const int32_t *seq_lens,
                            int num_splits, float scale, void *out,
                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FA355_H */
