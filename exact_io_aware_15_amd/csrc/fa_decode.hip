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
// Split kernel: one workgroup of NW waves per (sequence, split, KV head).
// The G = Hq / Hkv query heads of a group are MFMA columns 0 .. G-1 of a
// 16-column tile; GP >= G is the group width the kernel is built for (a
// power of two, which sizes only the LDS merge area), so every G <= 16 runs
// on the kernel of the next power of two, the extra columns computing on
// zero queries and never stored.  Wave w of a split takes the split's blocks
// w, w + NW, ...; their table entries sit one per lane.  The wave works on
// them two at a time: it issues both blocks' K (straight from HBM into
// registers) and V (into its two LDS slots by direct DMA), waits once, and
// then, on 16 x 16 matrix-core tiles (tokens x query heads of the group),
// computes S^T = K Q^T for both, one online-softmax update per head over
// their 32 tokens, and O^T += V^T P^T with V read back transposed.  The
// kernel is bound by the bytes in flight (each wave waits on its own loads
// while the other waves' loads stream), so the pair doubles what a wave has
// outstanding over one block at a time, without more registers or LDS.  The
// NW per-wave states are merged through LDS into the split's triple.
// Merge kernel: one workgroup per (sequence, query head):
// out = sum_p w_p o_p / sum_p w_p l_p with
// w_p = exp2((m_p - max m) * scale * log2 e).
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa355 {

namespace {

constexpr int kBlock = 16;  // tokens per cache block

// Cache-policy operand of the direct-to-LDS loads: non-temporal.  Each cache
// byte is read once per call, so the K and V streams are marked as such
// (with both loads non-temporal the decode measured 7% faster).
constexpr int kNonTemporal = 2;

// Chunk permutation of a 16-row V tile (row r, bits r0..r2): the 16 x 16
// transposing reads (4 rows x 2 adjacent chunks per 16 lanes) are free of
// bank conflicts whether the LDS serves 128 or 256 bytes per cycle.
//   D = 64:  (r0^r2) << 1 | r1 << 2
//   D = 128: r0 << 1 | r1 << 2 | r2 << 3
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  if (D == 64) return (((r ^ (r >> 2)) & 1) << 1) | (((r >> 1) & 1) << 2);
  return ((r & 1) << 1) | (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 3);
}

// Issues the DMA of one block's V tile (16 tokens x D of one KV head) into
// an LDS slot: row r holds token r, its 16-byte chunk c at position
// c ^ v_swz(r).  Slots past the sequence read its last valid token instead
// (finite data that gets probability 0).  Non-temporal: read once.
template <int D>
__device__ __forceinline__ void dma_v_block(uint16_t *slot, const uint16_t *blk,
                                            size_t tok_stride, int n_valid) {
  constexpr int CPR = D / 8;
  constexpr int SEG = kBlock * D * 2 / 1024;  // 1 KB per operation
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < SEG; ++i) {
    const int p = i * 64 + lane;
    const int r = p / CPR, phys = p % CPR;
    const int tok = min(r, n_valid - 1);
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void *)(
            blk + (size_t)tok * tok_stride + (phys ^ v_swz<D>(r)) * 8),
        (__attribute__((address_space(3))) void *)(slot + i * 512), 16, 0,
        kNonTemporal);
  }
}

// The sequence whose length ranks z-th in descending order (ties by index),
// lengths clamped as the split kernel clamps them.  Workgroups take their
// sequence through this map from blockIdx.z, so the longest sequences are
// dispatched first (longest-processing-time-first; every split of one
// sequence carries the same number of blocks) and the hardware's deal of
// consecutive workgroups over the CUs gives each CU one workgroup of every
// length quartile (measured 4% faster than the sequences' own order).  One
// lane per sequence, so batches of up to 64 sequences are ordered; larger
// ones keep their own order.  Returns the sequence (uniform) and its
// clamped length.
__device__ __forceinline__ int seq_by_length(const DecodeArgs &a, int z,
                                             int &len) {
  const int cap = a.max_blocks * kBlock;
  if (a.B > 64) {
    len = min(max(a.seq_lens[z], 0), cap);
    return z;
  }
  const int lane = threadIdx.x & 63;
  const int mine = lane < a.B ? min(max(a.seq_lens[lane], 0), cap) : -1;
  int rank = 0;
  for (int i = 0; i < a.B; ++i) {
    const int li = __builtin_amdgcn_readlane(mine, i);
    rank += (li > mine) || (li == mine && i < lane);
  }
  const uint64_t hit = __ballot(lane < a.B && rank == z);
  const int b = hit ? (int)__builtin_ctzll(hit) : 0;  // ranks are a permutation
  len = __builtin_amdgcn_readlane(mine, b);
  return b;
}

// The work item of workgroup i.  The hardware deals consecutive workgroups
// to different compute units, one per unit per round of `deal`, and every
// workgroup of this launch is resident at once, so each unit's share is
// fixed at dispatch; items come longest first, and odd rounds take them in
// reverse, so that each unit's long and short items pair up (boustrophedon
// order: for the 16-sequence decode the busiest unit's share drops from
// 1.17 to 1.04 times the mean).  A permutation of 0 .. n-1.
__device__ __forceinline__ int deal_order(int i, int n, int deal) {
  const int r = i / deal, base = r * deal;
  if (!(r & 1)) return i;
  return base + min(deal, n - base) - 1 - (i - base);
}

// Four waves per SIMD (at most 128 registers per lane): with four-wave
// workgroups a CU holds four of them, so a launch of up to 1024 workgroups
// is resident at once and every wave keeps its next block's K and V in
// flight from the start (measured 3-5% faster than the two waves per SIMD
// the register allocation otherwise settles on).
template <int D, int GP, int NW>
__global__ __launch_bounds__(64 * NW, 4) void decode_split_kernel(
    DecodeArgs a) {
  constexpr int TILE = kBlock * D;  // bf16 per V slot
  constexpr int KS = D / 32;        // k-steps of S^T = K Q^T
  constexpr int NC = D / 16;        // 16-row blocks of O^T
  static_assert(GP <= 16, "a query group must fit the 16 MFMA columns");
  // One LDS object (the V slots, reused for the final merge), so that the
  // compiler does not make LDS reads wait for DMA into other slots.
  union Smem {
    uint16_t v[NW][2][TILE];
    struct {
      float m[NW][GP], l[NW][GP];
      float o[NW][GP][D];
    } red;
  };
  __shared__ __attribute__((aligned(16))) Smem sm;

  // One-dimensional grid of Hkv * S * B, walked through deal_order: KV heads
  // vary fastest, so the Hkv workgroups of one (split, sequence) are
  // dispatched together and read neighbouring tiles of the same blocks;
  // then splits; sequences go longest first.
  const int item = deal_order(blockIdx.x, gridDim.x, a.deal);
  const int hk = item % a.Hkv;
  const int rest = item / a.Hkv;
  const int split = rest % a.num_splits;
  int len;  // clamped to the table's capacity
  const int b = seq_by_length(a, rest / a.num_splits, len);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;  // MFMA column / lane group
  const int S = a.num_splits;
  const int Hkv = a.Hkv;
  const int G = a.Hq / Hkv;  // 1 .. GP (validated by the caller)

  const int nblk = (len + kBlock - 1) / kBlock;
  const int per = (nblk + S - 1) / S;
  const int t_begin = min(nblk, split * per);
  const int t_end = min(nblk, t_begin + per);
  const int tw0 = t_begin + wave;  // this wave's blocks: tw0 + NW*j
  const int cnt = tw0 < t_end ? (t_end - tw0 + NW - 1) / NW : 0;

  // Q as the B operand of S^T = K Q^T: column = head, k = head dim
  // 32*ks + 8*grp + e.
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (col < G)
      x = ldg128(a.q + ((size_t)b * a.Hq + hk * G + col) * D + ks * 32 + 8 * grp);
    qf[ks] = __builtin_bit_cast(bf16x8, x);
  }

  // O^T accumulator: lane = head column, register r of block cb holds
  // head-dim row 16*cb + 4*grp + r.
  f32x4 oacc[NC];
#pragma unroll
  for (int cb = 0; cb < NC; ++cb) oacc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kMaxInit, l_run = 0.f;  // raw score units; l over 4 tokens
  const float c = a.c;

  const int32_t *table = a.block_table + (size_t)b * a.max_blocks;
  // Cache layouts: V [num_blocks][Hkv][16][D] (one head's block tile is 16
  // contiguous rows of D); K [num_blocks][Hkv][D/32][16][32] (the same tile
  // in 32-element groups: group g of the 16 tokens is 1 KiB contiguous).
  // Both tiles of a head are 16*D elements at the same offset.
  constexpr size_t tok_stride = D;
  const size_t blk_stride = (size_t)Hkv * kBlock * D;
  const size_t head_off = (size_t)hk * kBlock * D;
  uint16_t(*slots)[TILE] = sm.v[wave];

  // Transposing reads of V^T block cb: lane (grp, 4e + j) addresses token
  // 4*grp + e, head-dim columns 16*cb + 4j .. +3 (slot 0; slot 1 is TILE
  // elements further).
  uint32_t va[NC];
  {
    const int e = col >> 2, j = col & 3;
    const int r = 4 * grp + e;
    const int swz = v_swz<D>(r);
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      const int ch = 2 * cb + (j >> 1);
      va[cb] = lds_addr(slots[0] + r * D + ((ch ^ swz) << 3) + 4 * (j & 1));
    }
  }

  for (int p0 = 0; p0 < cnt; p0 += 64) {
    const int n = min(64, cnt - p0);
    // Lane j holds the physical block of this pass's j-th block; entries
    // outside [0, num_blocks) become -1: such a block is fetched from
    // physical block 0 (always valid memory) and then skipped.
    int ent = -1;
    if (lane < n) {
      const int ph = table[tw0 + NW * (p0 + lane)];
      ent = (ph >= 0 && ph < a.num_blocks) ? ph : -1;
    }
    // K of block j: lane (grp, col) loads token col (clamped to the valid
    // ones), head dims 32*ks + 8*grp .. +7, i.e. part grp of the token's
    // group ks, so each load instruction reads one contiguous 1 KiB group;
    // V of block j goes to slot j % 2.
    auto fetch = [&](int j, bf16x8 (&kf)[KS]) {
      const int ph = __builtin_amdgcn_readlane(ent, j);
      const int t = tw0 + NW * (p0 + j);
      const int n_valid = min(kBlock, len - t * kBlock);  // >= 1
      const size_t boff = (size_t)max(ph, 0) * blk_stride + head_off;
      const uint16_t *kb =
          a.k_cache + boff + (size_t)min(col, n_valid - 1) * 32 + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)  // read once: non-temporal
        kf[ks] = __builtin_bit_cast(
            bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                        kb + ks * kBlock * 32)));
      dma_v_block<D>(slots[j & 1], a.v_cache + boff, tok_stride, n_valid);
    };
    // Valid tokens of block j (0 for a block that is absent, j >= n, or
    // whose table entry is out of range: fetched from block 0 if at all,
    // and never used).
    auto valid_tokens = [&](int j) {
      if (j >= n || __builtin_amdgcn_readlane(ent, j) < 0) return 0;
      return min(kBlock, len - (tw0 + NW * (p0 + j)) * kBlock);
    };
    bf16x8 k0[KS], k1[KS];
    for (int j = 0; j < n; j += 2) {
      const bool two = j + 1 < n;
      fetch(j, k0);
      if (two) fetch(j + 1, k1);
      wait_dma();  // both blocks' K and V have landed
      const int nv0 = valid_tokens(j), nv1 = valid_tokens(j + 1);
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s0 = mfma16k32(k0[ks], qf[ks], s0);
      if (two) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s1 = mfma16k32(k1[ks], qf[ks], s1);
      }
      // Register r holds token 4*grp + r of head col, in each block.
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s0[r] = 4 * grp + r < nv0 ? s0[r] : -INFINITY;
        s1[r] = 4 * grp + r < nv1 ? s1[r] : -INFINITY;
        mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
      }
      const float m_new = fmaxf(m_run, max_xor32(max_xor16(mx)));
      const float alpha = fast_exp2((m_run - m_new) * c);
      const float mc = m_new * c;
      m_run = m_new;
      u32x2 pb0, pb1;
      pb0[0] = pack_bf16x2(fast_exp2(fmaf(s0[0], c, -mc)),
                           fast_exp2(fmaf(s0[1], c, -mc)));
      pb0[1] = pack_bf16x2(fast_exp2(fmaf(s0[2], c, -mc)),
                           fast_exp2(fmaf(s0[3], c, -mc)));
      pb1[0] = pack_bf16x2(fast_exp2(fmaf(s1[0], c, -mc)),
                           fast_exp2(fmaf(s1[1], c, -mc)));
      pb1[1] = pack_bf16x2(fast_exp2(fmaf(s1[2], c, -mc)),
                           fast_exp2(fmaf(s1[3], c, -mc)));
      l_run = fmaf(l_run, alpha,
                   dot2_ones(pb1[1], dot2_ones(pb1[0], dot2_ones(
                       pb0[1], dot2_ones(pb0[0], 0.f)))));
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) oacc[cb] = oacc[cb] * alpha;
      // O^T += V^T P^T for each block that holds tokens (an absent block's
      // slot is stale, a skipped one's may hold anything: neither is read
      // into the arithmetic).
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if ((h ? nv1 : nv0) <= 0) continue;
        const u32x2 pb = h ? pb1 : pb0;
        uint32_t vaj[NC];
#pragma unroll
        for (int cb = 0; cb < NC; ++cb)
          vaj[cb] = va[cb] + (uint32_t)(h * TILE * 2);
        bf16x8 vf[NC / 2];  // two 16 x 16 V^T blocks per fragment
        lds_tr_frags(vf, vaj);
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) {
          const u32x4 w = __builtin_bit_cast(u32x4, vf[cb >> 1]);
          const u32x2 vb = (cb & 1) ? u32x2{w[2], w[3]} : u32x2{w[0], w[1]};
          oacc[cb] = mfma16k16(vb, pb, oacc[cb]);
        }
      }
    }
  }
  wait_dma();

  // Merge the waves' states, then write the split's triple.  The merge area
  // overlays the V slots: every wave must be done with its slots first.
  __syncthreads();
  const float l_tot = sum_xor32(sum_xor16(l_run));
  if (col < G) {
    if (grp == 0) {
      sm.red.m[wave][col] = m_run;
      sm.red.l[wave][col] = l_tot;
    }
#pragma unroll
    for (int cb = 0; cb < NC; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sm.red.o[wave][col][16 * cb + 4 * grp + r] = oacc[cb][r];
  }
  __syncthreads();
  const size_t pbase = ((size_t)b * a.Hq + hk * G) * S + split;
  for (int x = tid; x < G * D; x += 64 * NW) {
    const int g = x / D, dcol = x % D;
    float mx = sm.red.m[0][g];
#pragma unroll
    for (int w = 1; w < NW; ++w) mx = fmaxf(mx, sm.red.m[w][g]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = fast_exp2((sm.red.m[w][g] - mx) * c);
      acc = fmaf(wt, sm.red.o[w][g][dcol], acc);
      lsum = fmaf(wt, sm.red.l[w][g], lsum);
    }
    const size_t pi = pbase + (size_t)g * S;
    a.part_o[pi * D + dcol] = acc;
    if (dcol == 0) {
      a.part_m[pi] = mx;
      a.part_l[pi] = lsum;
    }
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeArgs a) {
  // Partitions are read eight at a time with all of a chunk's loads in
  // flight together (one memory latency per chunk rather than per
  // partition); chunks are merged online, the running sums rescaled to each
  // chunk's new max.  For up to eight partitions this is the plain merge:
  // m = max_p m_p, w_p = exp(m_p - m), out = sum w_p o_p / sum w_p l_p.
  constexpr int CH = 8;
  const int hq = blockIdx.x % a.Hq, b = blockIdx.x / a.Hq;
  const int col = threadIdx.x;
  const int S = a.num_splits;
  const size_t pbase = ((size_t)b * a.Hq + hq) * S;
  float mx = -INFINITY, acc = 0.f, lsum = 0.f;
  for (int s0 = 0; s0 < S; s0 += CH) {
    float pm[CH], pl[CH], po[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const bool ok = s0 + j < S;
      const size_t p = pbase + s0 + j;
      pm[j] = ok ? a.part_m[p] : -INFINITY;  // weight exp2(-inf) = 0
      pl[j] = ok ? a.part_l[p] : 0.f;
      po[j] = ok ? a.part_o[p * D + col] : 0.f;
    }
    float cm = mx;
#pragma unroll
    for (int j = 0; j < CH; ++j) cm = fmaxf(cm, pm[j]);
    const float r = fast_exp2((mx - cm) * a.c);  // 0 on the first chunk
    acc *= r;
    lsum *= r;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const float w = fast_exp2((pm[j] - cm) * a.c);
      acc = fmaf(w, po[j], acc);
      lsum = fmaf(w, pl[j], lsum);
    }
    mx = cm;
  }
  const float out = lsum > 0.f ? acc / lsum : 0.f;
  const __bf16 ob = (__bf16)out;
  a.out[((size_t)b * a.Hq + hq) * D + col] = __builtin_bit_cast(uint16_t, ob);
}

template <int D, int GP>
hipError_t decode_dispatch_g(const DecodeArgs &a, hipStream_t s) {
  // Four waves per workgroup (32.5 KB of LDS at d = 128: four workgroups
  // per CU).
  constexpr int NW = 4;
  hipLaunchKernelGGL((decode_split_kernel<D, GP, NW>),
                     dim3((unsigned)(a.Hkv * a.num_splits * a.B)),
                     dim3(64 * NW), 0, s, a);
  hipLaunchKernelGGL(decode_merge_kernel<D>, dim3((unsigned)(a.Hq * a.B)),
                     dim3(D), 0, s, a);
  return hipGetLastError();
}

// Every group size 1 .. 16 (the caller rejects larger ones) runs on the
// kernel built for the next power of two.
template <int D>
hipError_t decode_dispatch(const DecodeArgs &a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  if (G <= 1) return decode_dispatch_g<D, 1>(a, s);
  if (G <= 2) return decode_dispatch_g<D, 2>(a, s);
  if (G <= 4) return decode_dispatch_g<D, 4>(a, s);
  if (G <= 8) return decode_dispatch_g<D, 8>(a, s);
  return decode_dispatch_g<D, 16>(a, s);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int d, hipStream_t s) {
  return d == 64 ? decode_dispatch<64>(a, s) : decode_dispatch<128>(a, s);
}

}  // namespace fa355
