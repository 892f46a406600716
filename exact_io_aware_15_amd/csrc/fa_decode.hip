// fa_decode.hip -- paged, GQA, split-K attention decode for gfx950.
//
// S12 "implement it": the key loop reads each tile through the block table
// (logical block t -> physical block block_table[t]; the last block holds
// n = min(block_size, seq_len - t*block_size) valid slots).  S12's
// production-practice paragraph: one loop does the recurrence, the paged
// lookup and GQA head sharing -- every query head of a group reads the
// group's one KV head, so each K/V byte is loaded once for G heads.  S12's
// "unlocks" paragraph (flash-decoding): with one query token there is no
// parallelism along queries, so the key range is split over workgroups and
// their (m, l, o) triples are merged (FA notes §3.1 merge rule).
//
// Split kernel: grid (num_splits, Hkv, B), 4 waves.  Each wave walks its share
// of the split's blocks; a block's 16 tokens are taken D/8 lanes per token
// (one 16-byte chunk each), 64/(D/8) tokens per round.  Scores for a block are
// reduced across the token's lanes with DPP, then one running-max update per
// block and head.  Slots past the sequence length are never loaded: their V
// registers hold zero and their scores -inf.  The 4 x (64/(D/8)) partial
// states of the workgroup are merged through LDS into the split's triple.
// Merge kernel: grid (Hq, B): out = sum_p w_p o_p / sum_p w_p l_p with
// w_p = exp2(m_p - max m).  All maxima are kept in log2 units (q is
// pre-multiplied by scale * log2(e)).
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa355 {

namespace {

constexpr int kBlock = 16;  // tokens per cache block

__device__ __forceinline__ float dpp_add(float x, int ctrl_sel) {
  int v = __builtin_bit_cast(int, x);
  int y;
  switch (ctrl_sel) {  // constant-folded after inlining
    case 0: y = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false); break;
    case 1: y = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false); break;
    case 2: y = __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false); break;
    default: y = __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false); break;
  }
  return x + __builtin_bit_cast(float, y);
}

// Sum over aligned groups of LPT lanes (LPT = 8 or 16); every lane of the
// group receives the total.  quad_perm [1,0,3,2] and [2,3,0,1] sum quads,
// row_half_mirror pairs the two quads of 8 lanes, row_mirror the two halves
// of a 16-lane row.
template <int LPT>
__device__ __forceinline__ float group_sum(float x) {
  x = dpp_add(x, 0);
  x = dpp_add(x, 1);
  x = dpp_add(x, 2);
  if (LPT == 16) x = dpp_add(x, 3);
  return x;
}

template <int D, int G>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int LPT = D / 8;          // lanes per token
  constexpr int TPR = 64 / LPT;       // tokens per round per wave
  constexpr int ROUNDS = kBlock / TPR;
  constexpr int NST = 4 * TPR;        // partial states per workgroup
  __shared__ float sm_m[G][NST];
  __shared__ float sm_l[G][NST];
  __shared__ float sm_o[G][NST][D];

  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane / LPT, lig = lane % LPT;
  const int S = a.num_splits;
  const int Hkv = a.Hkv;

  // Lengths beyond the table's capacity are clamped to it.
  const int len = min(max(a.seq_lens[b], 0), a.max_blocks * kBlock);
  const int nblk = (len + kBlock - 1) / kBlock;
  const int per = (nblk + S - 1) / S;
  const int t_begin = min(nblk, split * per);
  const int t_end = min(nblk, t_begin + per);

  // q for the G heads of this group, pre-scaled into log2 units.
  float qf[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int hq = hk * G + g;
    const u32x4 x = ldg128(a.q + ((size_t)b * a.Hq + hq) * D + lig * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      qf[g][e] = a.c * bf16_to_f32((uint16_t)(x[e >> 1] >> (16 * (e & 1))));
  }

  float m_run[G], l_run[G], o[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = kMaxInit;
    l_run[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = 0.f;
  }

  const int32_t *table = a.block_table + (size_t)b * a.max_blocks;
  const size_t tok_stride = (size_t)Hkv * D;  // elements between tokens
  for (int t = t_begin + wave; t < t_end; t += 4) {
    const int phys = table[t];
    if (phys < 0 || phys >= a.num_blocks) continue;  // never read outside the cache
    const size_t base = ((size_t)phys * kBlock * Hkv + hk) * D + lig * 8;
    u32x4 kr[ROUNDS], vr[ROUNDS];
    bool ok[ROUNDS];
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const int slot = r * TPR + grp;
      ok[r] = t * kBlock + slot < len;
      kr[r] = u32x4{0u, 0u, 0u, 0u};
      vr[r] = u32x4{0u, 0u, 0u, 0u};
      if (ok[r]) {
        kr[r] = ldg128(a.k_cache + base + slot * tok_stride);
        vr[r] = ldg128(a.v_cache + base + slot * tok_stride);
      }
    }
    float sc[ROUNDS][G];
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      float kf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        kf[e] = bf16_to_f32((uint16_t)(kr[r][e >> 1] >> (16 * (e & 1))));
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(qf[g][e], kf[e], acc);
        acc = group_sum<LPT>(acc);
        sc[r][g] = ok[r] ? acc : -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = sc[0][g];
#pragma unroll
      for (int r = 1; r < ROUNDS; ++r) mx = fmaxf(mx, sc[r][g]);
      const float m_new = fmaxf(m_run[g], mx);
      const float alpha = fast_exp2(m_run[g] - m_new);
      m_run[g] = m_new;
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] *= alpha;
#pragma unroll
      for (int r = 0; r < ROUNDS; ++r) {
        const float p = fast_exp2(sc[r][g] - m_new);
        ps += p;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          o[g][e] = fmaf(
              p, bf16_to_f32((uint16_t)(vr[r][e >> 1] >> (16 * (e & 1)))),
              o[g][e]);
      }
      l_run[g] = fmaf(l_run[g], alpha, ps);
    }
  }

  // Merge the workgroup's partial states (one per wave and token group).
  const int st = wave * TPR + grp;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (lig == 0) {
      sm_m[g][st] = m_run[g];
      sm_l[g][st] = l_run[g];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_o[g][st][lig * 8 + e] = o[g][e];
  }
  __syncthreads();
  const size_t pbase = ((size_t)b * a.Hq + hk * G) * S + split;
  for (int x = tid; x < G * D; x += 256) {
    const int g = x / D, col = x % D;
    float mx = sm_m[g][0];
    for (int s2 = 1; s2 < NST; ++s2) mx = fmaxf(mx, sm_m[g][s2]);
    float acc = 0.f, lsum = 0.f;
    for (int s2 = 0; s2 < NST; ++s2) {
      const float w = fast_exp2(sm_m[g][s2] - mx);
      acc = fmaf(w, sm_o[g][s2][col], acc);
      lsum = fmaf(w, sm_l[g][s2], lsum);
    }
    const size_t pi = pbase + (size_t)g * S;
    a.part_o[pi * D + col] = acc;
    if (col == 0) {
      a.part_m[pi] = mx;
      a.part_l[pi] = lsum;
    }
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeArgs a) {
  const int hq = blockIdx.x, b = blockIdx.y, col = threadIdx.x;
  const int S = a.num_splits;
  const size_t pbase = ((size_t)b * a.Hq + hq) * S;
  float mx = a.part_m[pbase];
  for (int s = 1; s < S; ++s) mx = fmaxf(mx, a.part_m[pbase + s]);
  float acc = 0.f, lsum = 0.f;
  for (int s = 0; s < S; ++s) {
    const float w = fast_exp2(a.part_m[pbase + s] - mx);
    acc = fmaf(w, a.part_o[(pbase + s) * D + col], acc);
    lsum = fmaf(w, a.part_l[pbase + s], lsum);
  }
  const float out = lsum > 0.f ? acc / lsum : 0.f;
  const __bf16 ob = (__bf16)out;
  a.out[((size_t)b * a.Hq + hq) * D + col] = __builtin_bit_cast(uint16_t, ob);
}

template <int D, int G>
hipError_t decode_dispatch_g(const DecodeArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((decode_split_kernel<D, G>),
                     dim3(a.num_splits, a.Hkv, a.B), dim3(256), 0, s, a);
  hipLaunchKernelGGL(decode_merge_kernel<D>, dim3(a.Hq, a.B), dim3(D), 0, s,
                     a);
  return hipGetLastError();
}

template <int D>
hipError_t decode_dispatch(const DecodeArgs &a, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: return decode_dispatch_g<D, 1>(a, s);
    case 2: return decode_dispatch_g<D, 2>(a, s);
    case 4: return decode_dispatch_g<D, 4>(a, s);
    case 8: return decode_dispatch_g<D, 8>(a, s);
    case 16: return decode_dispatch_g<D, 16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int d, hipStream_t s) {
  return d == 64 ? decode_dispatch<64>(a, s) : decode_dispatch<128>(a, s);
}

}  // namespace fa355
