// fa_kernels.h -- argument blocks and launchers of the gfx950 kernels
// (internal to libfa355; the public C ABI is include/fa355.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa355 {

// Dropout on the probabilities (keep iff a Philox byte >= thr; see
// fa_device.h).  thr = 0 means no dropout.
struct Dropout {
  uint32_t thr;       // 0..255
  float keep_scale;   // 256 / (256 - thr)
  uint32_t seed_lo, seed_hi, offset;
};

// Dense problems use [B,H,N,d] matrices.  Packed variable-length problems
// (cu_seqlens non-null) use [H,total,d]: sequence b of head h is rows
// h*total + cu_seqlens[b] .. of those matrices, and N is the longest
// sequence (it sizes the grid).
struct FwdArgs {
  const void *q, *k, *v;   // [B,H,N,d] or [H,total,d], bf16 or fp32
  void *o;
  float *m, *l;            // [B,H,N] or [H,total], or both null
  const int32_t *kv_len;   // [B] or null (dense only)
  const int32_t *cu_seqlens;  // [B+1] or null
  int total;               // packed rows per head (varlen)
  // Paged prefill: keys and values come from a paged cache (V
  // [num_blocks, Hkv, 16, d], K [num_blocks, Hkv, d/32, 16, 32]) through
  // block_table [B, max_blocks]; sequence b's queries are the last
  // positions of its seq_lens[b] cached tokens.
  const void *k_cache, *v_cache;
  const int32_t *block_table, *seq_lens;
  int max_blocks, num_blocks, Hkv;
  // Block-sparse: block_mask [H, nb, nb] uint8 over 128 x 128 blocks
  // (nb = ceil(N / 128)); nonzero = query block i attends key block j.
  const uint8_t *block_mask;
  Dropout drop;            // dense bf16 only
  int B, H, N, BH;
  float scale;             // natural-units score scale
  float c;                 // scale * log2(e): scores enter exp2 in log2 units
};

hipError_t launch_fwd_bf16(const FwdArgs &a, int d, bool causal,
                           hipStream_t s);
hipError_t launch_prefill_paged(const FwdArgs &a, int d, bool causal,
                                hipStream_t s);
hipError_t launch_fwd_block_sparse(const FwdArgs &a, int d, bool causal,
                                   hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs &a, int d, bool causal,
                          hipStream_t s);

// FP8 forward: Q, K [B,H,N,d] and V^T [B,H,d,ldv] as E4M3 codes with
// per-(batch, head) fp32 descales (null = 1); O bf16 [B,H,N,d].
struct Fp8FwdArgs {
  const uint8_t *q, *k, *vt;
  int ldv;                 // V^T row stride in bytes, >= N, multiple of 16
  const float *q_descale, *k_descale, *v_descale;  // [B*H] or null
  uint16_t *o;
  float *m, *l;            // [B,H,N] or both null
  const int32_t *kv_len;   // [B] or null
  int B, H, N, BH;
  float scale;
};

hipError_t launch_fwd_fp8(const Fp8FwdArgs &a, int d, bool causal,
                          hipStream_t s);

struct BwdArgs {
  const uint16_t *q, *k, *v, *o, *dout;  // [B,H,N,d] or [H,total,d] bf16
  const float *m, *l;                    // [B,H,N] or [H,total]
  const int32_t *kv_len;                 // [B] or null (dense only)
  const int32_t *cu_seqlens;             // [B+1] or null
  int total;                             // packed rows per head (varlen)
  long long rows;                        // rows of the [rows, d] matrices
  const uint8_t *block_mask;             // [H, nb, nb] or null (see FwdArgs)
  Dropout drop;                          // dense only (see FwdArgs)
  uint16_t *dq, *dk, *dv;                // [B,H,N,d] bf16
  float *lse2;                           // [B,H,N] workspace: log2-domain row offset
  float *delta;                          // [B,H,N] workspace: rowsum(dO*O)
  // Block-sparse only (else null), workspace [2][H*nb] each, nb = N/128
  // rounded up: the work of every (head, block) item of the two passes
  // (dK/dV items, then dQ items), and the items of each pass heaviest first.
  int32_t *sp_work, *sp_order;
  int sp_causal;                         // the mask is causal (block-sparse)
  int B, H, N, BH;
  float scale, c;
};

hipError_t launch_bwd(const BwdArgs &a, int d, bool causal, hipStream_t s);
// The non-causal d = 128 case of launch_bwd, built in its own unit.
hipError_t launch_bwd_nc128(const BwdArgs &a, hipStream_t s);

struct DecodeArgs {
  const uint16_t *q;            // [B,Hq,d]
  const uint16_t *k_cache;      // [num_blocks, Hkv, d/32, block_size, 32]
  const uint16_t *v_cache;
  const int32_t *block_table;   // [B, max_blocks]
  const int32_t *seq_lens;      // [B]
  uint16_t *out;                // [B,Hq,d]
  float *part_m, *part_l;       // [B,Hq,S]
  float *part_o;                // [B,Hq,S,d]
  int B, Hq, Hkv, max_blocks, num_blocks, num_splits;
  int deal;                     // compute units of the device
  float scale, c;
};

hipError_t launch_decode(const DecodeArgs &a, int d, hipStream_t s);

// Contract checks of the debug build (fa_check.hip).  Each launches one small
// kernel on `s` that reads the named device arrays (and nothing else) and ORs
// FA_CHECK_* bits into the current device's contract word.  cu_q may be NULL
// (decode: no new-token counts to compare seq_lens against).
hipError_t check_kv_len(const int32_t *kv_len, int B, int N, hipStream_t s);
hipError_t check_cu_seqlens(const int32_t *cu, int B, int total, int max_len,
                            hipStream_t s);
hipError_t check_paged(const int32_t *seq_lens, const int32_t *cu_q,
                       const int32_t *block_table, int B, int max_blocks,
                       int block_size, int num_blocks, hipStream_t s);
// Waits for the device, returns its contract word, and zeroes it if asked.
hipError_t read_contract_word(uint32_t *word, bool clear);

}  // namespace fa355
