// fa_fwd.hip -- exact attention forward for gfx950.
//
// The method is FA notes §3.2/§3.4 (tiled, fused forward) with S12's
// deferred-normalisation recurrence ("core idea"): for each key tile
//   m_new = max(m, rowmax S),  alpha = exp(m - m_new),
//   p = exp(S - m_new),  l = alpha*l + rowsum p,  o = alpha*o + p V,
// and o / l at the end.  The loop order is query-outer (one workgroup owns a
// query tile and streams every key tile past it), which gives the same result
// as the notes' key-outer listing without round-tripping O, l, m through HBM.
//
// bf16 kernel: 4 waves x 32 queries, 64-key tiles.  Scores are computed as
// S^T = K Q^T on the 32x32x16 bf16 MFMA so each lane owns one query (see
// fa_device.h); exponentials are taken as exp2 with scale*log2(e) folded into
// one FMA; p is rounded to bf16 once and that same value feeds both the P V
// MFMA and the row sum.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa355 {

namespace {

// Rescale threshold, log2 units: the accumulator keeps the running max it was
// last rescaled to (m_ref) until a row's true max exceeds it by more than
// this, so p = exp2(c*s - c*m_ref) stays below 2^8 while most tiles skip the
// O *= alpha multiply.  The result is unchanged: O and l share the same
// reference, and l is converted to the true max at the end.
constexpr float kRescaleLog2 = 8.0f;

// One key tile of the forward for the calling wave's QB 32-query blocks
// (queries qw .. qw + 32*QB - 1) against the 64 keys k0 .. k0+63 staged in
// Kt / Vt: S^T = K Q^T, the mask (diagonal and tail tiles only), the
// running-max update, p = exp2(c*s - c*m_ref) rounded to bf16 once, l += sum p
// and O^T += V^T P^T.  A tile wholly above the causal diagonal is skipped.
template <int D, int QB, bool CAUSAL, bool DROP, bool LMF>
__device__ __forceinline__ void fwd_tile(
    const uint16_t *Kt, const uint16_t *Vt, int k0, int qw, int kv_valid,
    int qoff, int bh, float c, const Dropout &drop,
    const bf16x8 (&qf)[QB][D / 16], f32x16 (&oacc)[QB][D / 32],
    float (&m_ref)[QB], float (&m_max)[QB], f32x4 (&l_acc)[QB],
    const bf16x8 &lsel) {
  constexpr int QPW = 32 * QB;
  constexpr int BC = 64;
  const int lane = threadIdx.x & 63;
  const int ln = lane & 31, hh = lane >> 5;
  if (CAUSAL && k0 > qw + QPW - 1 + qoff) return;  // above the diagonal
  // S^T = K Q^T for every (key block, query block).
  f32x16 s[QB][2];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
  // ks outer: the two key blocks' accumulations alternate, so each
  // MFMA's predecessor in the pipe is independent of it.
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 kf = lds_row_frag<D>(Kt, kb * 32 + ln, ks * 16 + 8 * hh);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        s[qb][kb] = mfma32(kf, qf[qb][ks], s[qb][kb]);
    }

  // Online softmax per query block.  Register r of key block kb holds
  // key k0 + 32*kb + 16*(r/8) + 8*hh + (r%8) of this lane's query.
  // pv[qb][kb][s2] is the B operand (8 consecutive keys) of P V.
  u32x4 pv[QB][2][2];
  u32x4 pl[QB][2][2];  // the undropped p (the same as pv without dropout)
  float mcs[QB];
  u32x4 rnd[QB][2];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qbase = qw + 32 * qb;
    const int qi = qbase + ln;
    const bool tail = k0 + BC > kv_valid;
    const bool diag = CAUSAL && k0 + BC - 1 > qbase + qoff;
    if (CAUSAL && diag && !tail) {
      // Causal diagonal tile wholly inside kv_valid: register r's key is
      // k0 + 8*hh + off(r) with off(r) a constant, so "key > qi + qoff" is
      // one compare of that constant against a per-lane threshold.
      const int thr_k = qi + qoff - k0 - 8 * hh;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = kb * 32 + 16 * (r >> 3) + (r & 7);
          s[qb][kb][r] = off > thr_k ? -INFINITY : s[qb][kb][r];
        }
    } else if (tail || diag) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 16 * (r >> 3) + 8 * hh + (r & 7);
          const bool masked =
              key >= kv_valid || (CAUSAL && key > qi + qoff);
          s[qb][kb][r] = masked ? -INFINITY : s[qb][kb][r];
        }
    }
    // A chain max(max(mx, a), b) per pair: one v_max3_f32 per two scores.
    float mx = fmaxf(s[qb][0][0], s[qb][0][1]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = (kb == 0 ? 2 : 0); r < 16; r += 2)
        mx = fmaxf(fmaxf(mx, s[qb][kb][r]), s[qb][kb][r + 1]);
    mx = max_xor32(mx);
    m_max[qb] = fmaxf(m_max[qb], mx);
    // Move the reference only when some row's max outgrew it by more than
    // kRescaleLog2 in log2 units (a wave-uniform branch; the empty asm keeps
    // it a branch).
    if (__any((m_max[qb] - m_ref[qb]) * c > kRescaleLog2)) {
      asm volatile("" ::: "memory");
      const float alpha = fast_exp2((m_ref[qb] - m_max[qb]) * c);
      m_ref[qb] = m_max[qb];
      l_acc[qb] *= alpha;
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[qb][cb][r] *= alpha;
    }
    mcs[qb] = m_ref[qb] * c;
    // Dropout: this lane's 16 random bytes per key block (its query,
    // group 2*(key block) + hh); l keeps the undropped sum.
    if (DROP) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        rnd[qb][kb] = drop_bytes(drop, qi, 2 * ((k0 >> 5) + kb) + hh, bh);
    }
  }

  // Per 32-key block: p = exp2(c*s - c*m_ref) rounded to bf16 (the same
  // values feed l and the product), then O^T += V^T P^T for that block.  The
  // block-0 products are issued before block 1's exponentials, so the
  // matrix cores work on them while the VALU computes block 1.  The V^T
  // fragment is read once (transposing LDS load) and used for every query
  // block; a query block whose keys are all masked contributes p = 0.
  float lsum[QB];  // row sums by dot products (when !LMF)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) lsum[qb] = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 8 * s2 + 2 * i;
          const float p0 = fast_exp2(fmaf(s[qb][kb][r], c, -mcs[qb]));
          const float p1 = fast_exp2(fmaf(s[qb][kb][r + 1], c, -mcs[qb]));
          const uint32_t pu = pack_bf16x2(p0, p1);
          if (!LMF) lsum[qb] = dot2_ones(pu, lsum[qb]);
          if (DROP) {
            const uint32_t keep =
                (drop_keep(rnd[qb][kb], r, drop.thr) ? 0xffffu : 0u) |
                (drop_keep(rnd[qb][kb], r + 1, drop.thr) ? 0xffff0000u : 0u);
            pv[qb][kb][s2][i] = pu & keep;
          } else {
            pv[qb][kb][s2][i] = pu;
          }
          if (DROP && LMF) pl[qb][kb][s2][i] = pu;
        }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        const bf16x8 vf = lds_tr_frag<D>(Vt, kb * 32 + 16 * s2, cb * 32);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[qb][cb] = mfma32(vf, __builtin_bit_cast(bf16x8, pv[qb][kb][s2]),
                                oacc[qb][cb]);
      }
    // Row sums on the matrix cores: l += (selector) x P for each 16-key
    // group (the selector picks, per output row, the lanes of this lane's
    // query).  Undropped p: l is the softmax normaliser.
    if (LMF) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          l_acc[qb] = mfma16k32(
              lsel, __builtin_bit_cast(bf16x8, DROP ? pl[qb][kb][s2]
                                                    : pv[qb][kb][s2]),
              l_acc[qb]);
    }
  }
  if (!LMF) {  // per lane half; both halves are summed by the caller
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_acc[qb][0] += lsum[qb];
  }
}

// Epilogue for one lane's query qi: O = o / l (0 for a row with no visible
// key) for the 32-column blocks cb_lo .. cb_hi-1 of the accumulator, and, if
// stats, m in natural units and l referred to the true max.  l_ref is the
// row's full sum (both lane halves) against the reference max m_ref.
template <int D, bool DROP>
__device__ __forceinline__ void fwd_store_rows(const FwdArgs &a, size_t hoff,
                                               size_t row0, int qi, int N,
                                               float l_ref, float m_ref,
                                               float m_max,
                                               const f32x16 (&oacc)[D / 32],
                                               int cb_lo, int cb_hi,
                                               bool stats) {
  if (qi >= N) return;
  const int hh = (threadIdx.x & 63) >> 5;
  // Kept probabilities carry the factor 256 / (256 - thr).
  const float num = DROP ? a.drop.keep_scale : 1.0f;
  const float inv = l_ref > 0.f ? num / l_ref : 0.f;
  uint16_t *og = (uint16_t *)a.o + hoff + (size_t)qi * D;
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) {
    if (cb < cb_lo || cb >= cb_hi) continue;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c0 = cb * 32 + 8 * g + 4 * hh;
      u32x2 w2;
      w2[0] = pack_bf16x2(oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv);
      w2[1] =
          pack_bf16x2(oacc[cb][4 * g + 2] * inv, oacc[cb][4 * g + 3] * inv);
      *reinterpret_cast<u32x2 *>(og + c0) = w2;
    }
  }
  if (stats && a.m != nullptr) {
    const size_t ri = row0 + qi;
    const float l_true = l_ref * fast_exp2((m_ref - m_max) * a.c);
    a.m[ri] = l_ref > 0.f ? m_max * a.scale : -INFINITY;
    a.l[ri] = l_ref > 0.f ? l_true : 0.f;
  }
}

// MINW: waves per SIMD the register allocation must allow (4 caps a lane at
// 128 VGPRs; 2 lets the compiler take what it needs).
// Sequence with the z-th largest cached length (ties by index), for up to
// 64 sequences; larger batches keep their own order.  Uniform in the wave.
__device__ __forceinline__ int paged_seq_by_length(const FwdArgs &a, int z) {
  if (a.B > 64) return z;
  const int cap = a.max_blocks * 16;
  const int lane = threadIdx.x & 63;
  const int mine = lane < a.B ? min(max(a.seq_lens[lane], 0), cap) : -1;
  int rank = 0;
  for (int i = 0; i < a.B; ++i) {
    const int li = __builtin_amdgcn_readlane(mine, i);
    rank += (li > mine) || (li == mine && i < lane);
  }
  const uint64_t hit = __ballot(lane < a.B && rank == z);
  return hit ? (int)__builtin_ctzll(hit) : 0;  // ranks are a permutation
}

template <int D, int QPW, bool CAUSAL, bool PADDED, bool PAGED = false,
          bool SPARSE = false, bool DROP = false, int MINW = 2>
__global__ __launch_bounds__(256, MINW) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int QB = QPW / 32;                    // 32-query blocks per wave
  // Row sums on the matrix cores (a 16x16x32 product per 16 keys, taking
  // 16 VALU dot products off each tile) in the causal kernels, which keep
  // their waves per SIMD with it.  The non-causal ones schedule a tile as
  // one block and would need 4-50 more registers (losing a wave per SIMD or
  // spilling), so they sum with dot products.
  constexpr bool LMF = CAUSAL;
  constexpr int BR = 4 * QPW;                     // queries per workgroup
  constexpr int BC = 64;                          // keys per tile
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BC * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, hh = lane >> 5;

  // Query tiles in descending order (heaviest causal tiles first, dealt so
  // each CU's resident workgroups carry equal work); heads vary fastest, so
  // workgroups dealt round-robin to the 8 XCDs keep one head's tiles on one
  // XCD's L2 when B*H is a multiple of 8 (or divides 8).  With a
  // paged cache the G query heads of one KV head read the same K/V tiles:
  // their workgroups get block indices of equal residue mod 8 (one XCD, one
  // L2).  Unit u = (sequence rank, query tile, KV head), G heads each, the
  // sequences ranked by cached length, longest first (a workgroup's work
  // grows with it); the grid is rounded up to whole groups of eight units.
  const int nqt = (a.N + BR - 1) / BR;
  int bh, qt;
  if (PAGED) {
    const int G = a.H / a.Hkv;
    // Dealt like the dense grid (the deal keeps each block's residue mod 8).
    const int bi = CAUSAL ? causal_deal_order<MINW == 4 ? 4 : (D == 64 ? 3 : 2)>(blockIdx.x)
                          : (int)blockIdx.x;
    const int sx = bi >> 3;
    const int g = sx % G;
    const int u = (sx / G) * 8 + (bi & 7);
    const int per_seq = nqt * a.Hkv;
    if (u >= per_seq * a.B) return;  // rounding of the grid
    // Sequences by decreasing cached length (a workgroup's work grows with
    // it), then query tiles from the last, then KV heads.
    const int rk = u / per_seq, rem = u - rk * per_seq;
    qt = nqt - 1 - rem / a.Hkv;
    const int bb = paged_seq_by_length(a, rk);
    bh = bb * a.H + (rem % a.Hkv) * G + g;
  } else {
    // Resident workgroups per CU: 4 (MINW = 4), 3 (other d = 64), 2 (d = 128).
    const int i =
        (CAUSAL && !SPARSE)
            ? causal_deal_order<MINW == 4 ? 4 : (D == 64 ? 3 : 2)>(blockIdx.x)
            : (int)blockIdx.x;
    bh = i % a.BH;
    qt = nqt - 1 - i / a.BH;
  }
  const int b = bh / a.H;
  const SliceRows sr = slice_rows(a.cu_seqlens, a.total, a.N, a.H, bh);
  const int N = sr.n;  // queries of this slice
  const size_t hoff = sr.row0 * D;
  const uint16_t *__restrict__ qg = (const uint16_t *)a.q + hoff;
  const uint16_t *kg, *vg;
  // Keys: the slice's own rows, or (paged prefill) the KV head's tiles in
  // the cache, in which case the N queries are the last N of the kv_valid
  // cached positions: query i sits at position i + qoff (causal offset).
  int kv_valid, qoff = 0;
  size_t blk_stride = 0;
  const int32_t *btab = nullptr;
  if (PAGED) {
    const int h = bh - b * a.H, hk = h / (a.H / a.Hkv);
    kv_valid = min(max(a.seq_lens[b], 0), a.max_blocks * 16);
    qoff = kv_valid - N;
    blk_stride = (size_t)a.Hkv * 16 * D;
    kg = (const uint16_t *)a.k_cache + (size_t)hk * 16 * D;
    vg = (const uint16_t *)a.v_cache + (size_t)hk * 16 * D;
    btab = a.block_table + (size_t)b * a.max_blocks;
  } else {
    kg = (const uint16_t *)a.k + hoff;
    vg = (const uint16_t *)a.v + hoff;
    kv_valid = N;
    if (PADDED) kv_valid = min(max(a.kv_len[b], 0), N);
  }

  const int q0 = qt * BR;
  if (q0 >= N) return;  // a packed sequence shorter than the longest one
  const int qw = q0 + wave * QPW;
  int kend = kv_valid;
  if (CAUSAL) kend = max(0, min(kend, q0 + BR + qoff));
  const int ntiles = (kend + BC - 1) / BC;

  // Q as the B operand of S^T = K Q^T: lane holds Q[q][16*ks + 8*hh + e] for
  // its query q = qw + 32*qb + ln of each query block.
  bf16x8 qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int qi = qw + 32 * qb + ln;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qi < N) x = ldg128(qg + (size_t)qi * D + ks * 16 + 8 * hh);
      qf[qb][ks] = __builtin_bit_cast(bf16x8, x);
    }

  f32x16 oacc[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][cb][r] = 0.f;
  float m_ref[QB], m_max[QB];
  // Row sum of this lane's query: in all four registers (LMF), or in
  // register 0 over this lane's half of the keys (dot products).
  f32x4 l_acc[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = kMaxInit;  // raw (unscaled) score units
    m_max[qb] = kMaxInit;
    l_acc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Selector A operand of the row-sum product (16 x 16 x 32): output row
  // group j (rows 4j..4j+3) takes the contraction slots 8k..8k+7 with
  // k % 2 == j % 2, i.e. the lanes that hold this lane's query, so lane l
  // receives the row sum of query l % 32 (see fwd_tile).
  bf16x8 lsel;
  {
    const __bf16 sel =
        (__bf16)((((lane & 15) >> 2) & 1) == ((lane >> 4) & 1) ? 1.0f : 0.0f);
#pragma unroll
    for (int e = 0; e < 8; ++e) lsel[e] = sel;
  }
  const float c = a.c;

  // Global -> LDS staging by direct DMA; keys past kv_valid read the last
  // valid key instead (finite data that the mask then excludes).  A paged
  // tile takes its four cache blocks from the table (entries loaded one
  // tile ahead of their use, clamped to valid block indices).
  const int nb_used = (kv_valid + 15) / 16;
  size_t eo_next[4] = {0, 0, 0, 0};  // e_next as element offsets
  auto table_entries = [&](int t, int (&e)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = 4 * t + i;
      e[i] = __builtin_amdgcn_readfirstlane(
          idx < nb_used ? min(max(btab[idx], 0), a.num_blocks - 1) : 0);
      eo_next[i] = (size_t)e[i] * blk_stride;
    }
  };
  int e_next[4] = {0, 0, 0, 0};
  const DmaOffsets<D, BC> doff;
  const PagedDmaOffsets<D, true> pk_off;
  const PagedDmaOffsets<D, false> pv_off;
  // Whole tiles of a dense or packed slice go through buffer resources over
  // the slice's N rows (N <= 2^20, d <= 128: under 2^28 bytes).
  const uint32_t slice_bytes = PAGED ? 0u : (uint32_t)N * D * 2;
  auto load_tile = [&](int k0, int buf) {
    if (PAGED && k0 + BC <= kv_valid) {  // whole tile: uniform block bases
      dma_tile_paged_at<D, true>(Ks[buf], kg, eo_next, pk_off);
      dma_tile_paged_at<D, false>(Vs[buf], vg, eo_next, pv_off);
    } else if (PAGED) {
      dma_tile_paged<D, true>(Ks[buf], kg, blk_stride, e_next, k0,
                              kv_valid - 1);
      dma_tile_paged<D, false>(Vs[buf], vg, blk_stride, e_next, k0,
                               kv_valid - 1);
    } else if (k0 + BC <= kv_valid) {  // whole tile valid: uniform base
      dma_tile_at<D, BC>(Ks[buf], kg, slice_bytes, (uint32_t)k0 * D * 2,
                         doff);
      dma_tile_at<D, BC>(Vs[buf], vg, slice_bytes, (uint32_t)k0 * D * 2,
                         doff);
    } else {
      dma_tile_tail<D, BC>(Ks[buf], kg, k0, kv_valid - 1);
      dma_tile_tail<D, BC>(Vs[buf], vg, k0, kv_valid - 1);
    }
  };

  // Tiles to visit: all of [0, ntiles), or (block-sparse) those whose
  // 128-key block the mask row of this 128-query block allows.
  MaskWalk walk;
  if (SPARSE) {
    const int nb = (a.N + 127) / 128;
    const int h = bh - b * a.H;
    walk.mask = a.block_mask + ((size_t)h * nb + qt) * nb;
    walk.stride = 1;
    walk.per = 128 / BC;
    walk.n = ntiles;
  }
  auto next_tile = [&](int t) { return SPARSE ? walk.next(t) : t; };

  int t = next_tile(0);
  if (t < ntiles) {
    if (PAGED) table_entries(t, e_next);
    load_tile(t * BC, 0);
    if (PAGED) table_entries(t + 1, e_next);
  }
  wait_dma();
  __syncthreads();
  // One tile; the loop below instantiates it for buffer 0 and buffer 1 so
  // that every LDS address is a per-lane base plus a constant offset.
  auto step = [&](auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int k0 = t * BC;
    const int tn = next_tile(t + 1);
    // The other buffer was last read before the previous barrier.
    if (tn < ntiles) {
      load_tile(tn * BC, buf ^ 1);
      if (PAGED) table_entries(tn + 1, e_next);
    }
    const uint16_t *Kt = Ks[buf];
    const uint16_t *Vt = Vs[buf];

    fwd_tile<D, QB, CAUSAL, DROP, LMF>(Kt, Vt, k0, qw, kv_valid, qoff, bh, c,
                                  a.drop, qf, oacc, m_ref, m_max, l_acc,
                                  lsel);

    wait_dma();  // the next tile has landed
    __syncthreads();
    t = tn;
  };
  while (t < ntiles) {
    step(std::integral_constant<int, 0>{});
    if (t >= ntiles) break;
    step(std::integral_constant<int, 1>{});
  }

  // Epilogue: O = o / l (0 for a row with no visible key); m in natural
  // units and l referred to the true max.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
    fwd_store_rows<D, DROP>(a, hoff, sr.row0, qw + 32 * qb + ln, N,
                            LMF ? l_acc[qb][0] : sum_xor32(l_acc[qb][0]),
                            m_ref[qb], m_max[qb], oacc[qb], 0, D / 32,
                            hh == 0);
}

// fp32 path: one thread per query, 16-key tiles staged in LDS, the same
// recurrence in plain fp32 arithmetic.  A correctness path for fp32 inputs.
template <int D, bool CAUSAL, bool PADDED>
__global__ __launch_bounds__(64, 1) void fwd_f32_kernel(FwdArgs a) {
  constexpr int T = 16;
  __shared__ float Ks[T][D];
  __shared__ float Vs[T][D];
  const int tid = threadIdx.x;
  const int nqt = (a.N + 63) / 64;
  const int bh = blockIdx.x % a.BH;
  const int qt = blockIdx.x / a.BH;
  const int b = bh / a.H;
  const SliceRows sr = slice_rows(a.cu_seqlens, a.total, a.N, a.H, bh);
  const int N = sr.n;
  const size_t hoff = sr.row0 * D;
  const float *qg = (const float *)a.q + hoff;
  const float *kg = (const float *)a.k + hoff;
  const float *vg = (const float *)a.v + hoff;
  (void)nqt;
  const int qi = qt * 64 + tid;
  if (qt * 64 >= N) return;  // a packed sequence shorter than the longest one
  int kv_valid = N;
  if (PADDED) kv_valid = min(max(a.kv_len[b], 0), N);
  int kend = kv_valid;
  if (CAUSAL) kend = min(kend, qt * 64 + 64);

  float q[D], o[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    q[i] = qi < N ? qg[(size_t)qi * D + i] : 0.f;
    o[i] = 0.f;
  }
  float m_run = kMaxInit, l_run = 0.f;
  const float c = a.c;
  for (int k0 = 0; k0 < kend; k0 += T) {
    __syncthreads();
    for (int x = tid; x < T * D; x += 64) {
      const int j = x / D, i = x % D;
      const bool ok = k0 + j < kv_valid;
      Ks[j][i] = ok ? kg[(size_t)(k0 + j) * D + i] : 0.f;
      Vs[j][i] = ok ? vg[(size_t)(k0 + j) * D + i] : 0.f;
    }
    __syncthreads();
    float s[T];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < T; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) acc = fmaf(q[i], Ks[j][i], acc);
      const int key = k0 + j;
      const bool masked = key >= kv_valid || (CAUSAL && key > qi);
      s[j] = masked ? -INFINITY : acc;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f((m_run - m_new) * c);
    const float mc = m_new * c;
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < T; ++j) {
      s[j] = exp2f(fmaf(s[j], c, -mc));
      lsum += s[j];
    }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int i = 0; i < D; ++i) {
      float acc = o[i] * alpha;
#pragma unroll
      for (int j = 0; j < T; ++j) acc = fmaf(s[j], Vs[j][i], acc);
      o[i] = acc;
    }
  }
  if (qi < N) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    float *og = (float *)a.o + hoff + (size_t)qi * D;
#pragma unroll
    for (int i = 0; i < D; ++i) og[i] = o[i] * inv;
    if (a.m != nullptr) {
      a.m[sr.row0 + qi] = l_run > 0.f ? m_run * a.scale : -INFINITY;
      a.l[sr.row0 + qi] = l_run;
    }
  }
}

template <int D, bool CAUSAL>
hipError_t fwd_bf16_dispatch_pad(const FwdArgs &a, hipStream_t s) {
  // 32 queries per wave (one 32-query block), 4 waves per workgroup.
  constexpr int QPW = 32;
  const int nqt = (a.N + 4 * QPW - 1) / (4 * QPW);
  dim3 grid((unsigned)(nqt * a.BH)), block(256);
  if (a.drop.thr != 0) {
    // Dropout needs more registers (three waves per SIMD at d = 64).
    if (a.kv_len)
      hipLaunchKernelGGL(
          (fwd_bf16_kernel<D, QPW, CAUSAL, true, false, false, true>), grid,
          block, 0, s, a);
    else
      hipLaunchKernelGGL(
          (fwd_bf16_kernel<D, QPW, CAUSAL, false, false, false, true>), grid,
          block, 0, s, a);
    return hipGetLastError();
  }
  // Without dropout the d = 64 forward runs 4 waves per SIMD (128 VGPRs):
  // the extra resident workgroup per CU hides more latency (measured 1-9%
  // faster than 3 waves from N = 1K to 64K once causal tiles are dealt
  // evenly); d = 128 needs more registers and runs 2.
  constexpr int MINW = D == 64 ? 4 : 2;
  if (a.kv_len)
    hipLaunchKernelGGL(
        (fwd_bf16_kernel<D, QPW, CAUSAL, true, false, false, false, MINW>),
        grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(
        (fwd_bf16_kernel<D, QPW, CAUSAL, false, false, false, false, MINW>),
        grid, block, 0, s, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t fwd_f32_dispatch_pad(const FwdArgs &a, hipStream_t s) {
  const int nqt = (a.N + 63) / 64;
  dim3 grid((unsigned)(nqt * a.BH)), block(64);
  if (a.kv_len)
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, true>), grid, block, 0, s,
                       a);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, false>), grid, block, 0, s,
                       a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, int d, bool causal,
                           hipStream_t s) {
  if (d == 64)
    return causal ? fwd_bf16_dispatch_pad<64, true>(a, s)
                  : fwd_bf16_dispatch_pad<64, false>(a, s);
  return causal ? fwd_bf16_dispatch_pad<128, true>(a, s)
                : fwd_bf16_dispatch_pad<128, false>(a, s);
}

hipError_t launch_fwd_block_sparse(const FwdArgs &a, int d, bool causal,
                                   hipStream_t s) {
  const int nqt = (a.N + 127) / 128;
  dim3 grid((unsigned)(nqt * a.BH)), block(256);
  if (d == 64) {
    if (causal)
      hipLaunchKernelGGL((fwd_bf16_kernel<64, 32, true, false, false, true>),
                         grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<64, 32, false, false, false, true>),
                         grid, block, 0, s, a);
  } else {
    if (causal)
      hipLaunchKernelGGL((fwd_bf16_kernel<128, 32, true, false, false, true>),
                         grid, block, 0, s, a);
    else
      hipLaunchKernelGGL(
          (fwd_bf16_kernel<128, 32, false, false, false, true>), grid, block,
          0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_paged(const FwdArgs &a, int d, bool causal,
                                hipStream_t s) {
  // Units of (query tile, sequence, KV head) in groups of eight, each unit's
  // G = H / Hkv query heads on one XCD (see fwd_bf16_kernel).
  const int nqt = (a.N + 127) / 128;
  const long long units = (long long)nqt * a.B * a.Hkv;
  const long long blocks = 8LL * (a.H / a.Hkv) * ((units + 7) / 8);
  dim3 grid((unsigned)blocks), block(256);
  if (d == 64) {
    if (causal)
      hipLaunchKernelGGL((fwd_bf16_kernel<64, 32, true, false, true>), grid,
                         block, 0, s, a);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<64, 32, false, false, true>), grid,
                         block, 0, s, a);
  } else {
    if (causal)
      hipLaunchKernelGGL((fwd_bf16_kernel<128, 32, true, false, true>), grid,
                         block, 0, s, a);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<128, 32, false, false, true>), grid,
                         block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const FwdArgs &a, int d, bool causal,
                          hipStream_t s) {
  if (d == 64)
    return causal ? fwd_f32_dispatch_pad<64, true>(a, s)
                  : fwd_f32_dispatch_pad<64, false>(a, s);
  return causal ? fwd_f32_dispatch_pad<128, true>(a, s)
                : fwd_f32_dispatch_pad<128, false>(a, s);
}

}  // namespace fa355
