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

// Issues the DMA of one cache block (one KV head: 16 tokens x D) into an
// LDS tile (rows in row_perm order, swizzled).  Slots past the sequence read
// its last valid token instead (finite data the caller masks).
template <int D>
__device__ __forceinline__ void dma_block(uint16_t *tile, const uint16_t *blk,
                                          size_t tok_stride, int n_valid) {
  constexpr int CPR = D / 8;
  constexpr int SEG = kBlock * D * 2 / 1024;  // 1 KB segments
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < SEG; ++i) {
    const int p = i * 64 + lane;
    const int r = p / CPR, phys_c = p % CPR;
    const int swz = ((r & 3) << 1) | ((r >> 2) & 1);
    const int tok = min(row_perm(r), n_valid - 1);
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void *)(
            blk + (size_t)tok * tok_stride + (phys_c ^ swz) * 8),
        (__attribute__((address_space(3))) void *)(tile + i * 512), 16, 0, 0);
  }
}

template <int D, int G, int NW>
__global__ __launch_bounds__(64 * NW) void decode_split_kernel(DecodeArgs a) {
  constexpr int TILE = kBlock * D;                 // bf16 per K or V tile
  constexpr int SEG = kBlock * D * 2 / 1024;       // DMA ops per tile
  constexpr int TCH = 256;                         // table entries per chunk
  static_assert(G <= 32, "a query group must fit the 32 MFMA columns");
  // Per wave: two buffers, each a K tile and a V tile.
  __shared__ __attribute__((aligned(16))) uint16_t KVs[NW][2][2][TILE];
  __shared__ int tab[TCH];
  __shared__ float sm_m[NW][G], sm_l[NW][G];
  __shared__ float sm_o[NW][G][D];

  // KV heads vary fastest: the Hkv workgroups of one (split, sequence) are
  // dispatched together and read the same cache blocks at once.
  const int hk = blockIdx.x, split = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, hh = lane >> 5;
  const int S = a.num_splits;
  const int Hkv = a.Hkv;

  // Lengths beyond the table's capacity are clamped to it.
  const int len = min(max(a.seq_lens[b], 0), a.max_blocks * kBlock);
  const int nblk = (len + kBlock - 1) / kBlock;
  const int per = (nblk + S - 1) / S;
  const int t_begin = min(nblk, split * per);
  const int t_end = min(nblk, t_begin + per);

  // Scores are S^T = K Q^T on v_mfma_f32_32x32x16_bf16: MFMA rows are the
  // block's 16 tokens (rows 16..31 are zero), columns the G query heads of
  // this KV head's group (columns G..31 are zero).  Q as the B operand:
  // lane = head column, slots = head dim.
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (ln < G)
      x = ldg128(a.q + ((size_t)b * a.Hq + hk * G + ln) * D + ks * 16 + 8 * hh);
    qf[ks] = __builtin_bit_cast(bf16x8, x);
  }

  // O^T accumulator: lane = head column, register r of cb holds head-dim row
  // cb*32 + 8*(r/4) + 4*hh + (r%4).
  f32x16 oacc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.f;
  float m_run = kMaxInit, l_run = 0.f;  // raw score units; l over this half
  const float c = a.c;

  const int32_t *table = a.block_table + (size_t)b * a.max_blocks;
  const size_t tok_stride = (size_t)Hkv * D;  // elements between tokens
  const size_t head_off = (size_t)hk * D;

  for (int c0 = t_begin; c0 < t_end; c0 += TCH) {
    const int c1 = min(t_end, c0 + TCH);
    __syncthreads();  // previous chunk's table entries are no longer read
    for (int x = tid; x < c1 - c0; x += 64 * NW) {
      const int ph = table[c0 + x];
      tab[x] = (ph >= 0 && ph < a.num_blocks) ? ph : -1;  // never read outside
    }
    __syncthreads();

    // This wave's blocks: c0 + wave, +NW, ...; block i+1's DMA is issued
    // before block i is computed (double buffer per wave).
    auto issue = [&](int t, int buf) {
      const int ph = tab[t - c0];
      if (ph < 0) return;
      const int n_valid = min(kBlock, len - t * kBlock);  // >= 1
      const size_t boff = (size_t)ph * kBlock * tok_stride + head_off;
      dma_block<D>(KVs[wave][buf][0], a.k_cache + boff, tok_stride, n_valid);
      dma_block<D>(KVs[wave][buf][1], a.v_cache + boff, tok_stride, n_valid);
    };
    int buf = 0;
    int t = c0 + wave;
    if (t < c1) issue(t, 0);
    for (; t < c1; t += NW, buf ^= 1) {
      const bool has_next = t + NW < c1;
      if (has_next) {
        issue(t + NW, buf ^ 1);
        // wait for this block's tiles; the next block's may stay in flight
        if (tab[t + NW - c0] >= 0)
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * SEG) : "memory");
        else
          wait_dma();
      } else {
        wait_dma();
      }
      if (tab[t - c0] < 0) continue;
      const int n_valid = min(kBlock, len - t * kBlock);
      const uint16_t *Kt = KVs[wave][buf][0];
      const uint16_t *Vt = KVs[wave][buf][1];
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        bf16x8 kf = {};
        if (ln < kBlock) kf = lds_row_frag<D>(Kt, ln, ks * 16 + 8 * hh);
        s = mfma32(kf, qf[ks], s);
      }
      // Registers 0..7 hold tokens 8*hh + r of this lane's head.
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const bool ok = 8 * hh + r < n_valid;
        s[r] = ok ? s[r] : -INFINITY;
        mx = fmaxf(mx, s[r]);
      }
      const float m_new = fmaxf(m_run, max_xor32(mx));
      const float alpha = fast_exp2((m_run - m_new) * c);
      const float mc = m_new * c;
      m_run = m_new;
      u32x4 pb;
      float lsum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = fast_exp2(fmaf(s[2 * i], c, -mc));
        const float p1 = fast_exp2(fmaf(s[2 * i + 1], c, -mc));
        pb[i] = pack_bf16x2(p0, p1);
        lsum = dot2_ones(pb[i], lsum);
      }
      l_run = fmaf(l_run, alpha, lsum);
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
        oacc[cb] = mfma32(lds_tr_frag<D>(Vt, 0, cb * 32),
                          __builtin_bit_cast(bf16x8, pb), oacc[cb]);
      }
    }
    wait_dma();
  }

  // Merge the waves' states, then write the split's triple.
  const float l_tot = sum_xor32(l_run);
  if (ln < G) {
    if (hh == 0) {
      sm_m[wave][ln] = m_run;
      sm_l[wave][ln] = l_tot;
    }
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sm_o[wave][ln][cb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3)] =
            oacc[cb][r];
  }
  __syncthreads();
  const size_t pbase = ((size_t)b * a.Hq + hk * G) * S + split;
  for (int x = tid; x < G * D; x += 64 * NW) {
    const int g = x / D, col = x % D;
    float mx = sm_m[0][g];
#pragma unroll
    for (int w = 1; w < NW; ++w) mx = fmaxf(mx, sm_m[w][g]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = fast_exp2((sm_m[w][g] - mx) * c);
      acc = fmaf(wt, sm_o[w][g][col], acc);
      lsum = fmaf(wt, sm_l[w][g], lsum);
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
    const float w = fast_exp2((a.part_m[pbase + s] - mx) * a.c);
    acc = fmaf(w, a.part_o[(pbase + s) * D + col], acc);
    lsum = fmaf(w, a.part_l[pbase + s], lsum);
  }
  const float out = lsum > 0.f ? acc / lsum : 0.f;
  const __bf16 ob = (__bf16)out;
  a.out[((size_t)b * a.Hq + hq) * D + col] = __builtin_bit_cast(uint16_t, ob);
}

template <int D, int G>
hipError_t decode_dispatch_g(const DecodeArgs &a, hipStream_t s) {
  // Four waves per workgroup: two workgroups fit a CU's LDS at d = 128,
  // and measured faster than one 8-wave workgroup.
  constexpr int NW = 4;
  hipLaunchKernelGGL((decode_split_kernel<D, G, NW>),
                     dim3(a.Hkv, a.num_splits, a.B), dim3(64 * NW), 0, s, a);
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
