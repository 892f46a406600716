// fa_bwd.hip -- exact attention backward for gfx950 by recomputation.
//
// FA notes §3.3: the backward pass keeps only O and the row statistics (m, l)
// from the forward pass and rebuilds the score and probability tiles on chip.
// The gradient formulas are the softmax chain rule (the pages do not print
// them):  dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
// dQ = scale dS K,  dK = scale dS^T Q.
//
// Three passes, none using atomics:
//   1. pre:   D_i = sum_c dO_ic O_ic, and the log2-domain row offset
//             lse2_i = m_i log2(e) + log2(l_i), so that P = exp2(c S - lse2)
//             with c = scale log2(e).
//   2. dkdv:  key-stationary.  One workgroup per 128-key tile (4 waves x 32
//             keys) keeps its K, V fragments and dK, dV accumulators in
//             registers while 64-query blocks of Q and dO stream through LDS:
//             S = Q K^T, dP = dO V^T, P, dS, then dV += P^T dO, dK += dS^T Q.
//   3. dq:    query-stationary, laid out like the forward: one workgroup per
//             128-query tile (4 waves x 32 queries) keeps Q, dO, lse2 and D in
//             registers while 64-key tiles of K and V stream through LDS:
//             S^T = K Q^T, dP^T = V dO^T, dS^T, then dQ^T += K^T dS^T.
// At d = 64 (without dropout) passes 2 and 3 share one launch, their
// workgroups interleaved (bwd_fused_kernel); otherwise they are two launches.
// The non-causal d = 128 kernels are instantiated only in fa_bwd_nc128.hip
// (this file built with FA355_BWD_NC128_UNIT defined), so that they can be
// compiled with other scheduler options than the rest.
// Recomputing S and dP in the dq pass costs two extra contractions; it
// replaces the per-key-tile dQ partial sums that would otherwise need
// device-wide float atomics, which are far slower on this part than the
// matrix cores.
//
// Operand tiles in LDS are row-major with their rows in row_perm order, so
// score registers come out as 8 consecutive rows per lane (see fa_device.h);
// operands that contract over a tile's rows are read with transposing LDS
// loads (lds_tr_frag) instead of being stored transposed.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa355 {

namespace {

// Rows are handled by groups of d/8 lanes (16 bytes of O and of dO each),
// kPreRows rows per group with every load (O, dO, and the row's m and l)
// issued before any arithmetic, so each lane keeps 2 * kPreRows loads in
// flight and a workgroup makes one round trip.  O is read only here, so its
// loads are non-temporal; dO stays cached for the passes that follow.
constexpr int kPreRows = 4;

// Block-sparse work of item t = (h, j): the dK/dV item of key block j of
// head h visits the query blocks that mask column j allows (causal: i >= j),
// the dQ item of query block j the key blocks that mask row j allows
// (causal: i <= j).
__device__ __forceinline__ void sparse_work(const BwdArgs &a, int t) {
  const int nb = (a.N + 127) / 128;
  const int n = a.H * nb;
  if (t >= n) return;
  const int h = t / nb, j = t - h * nb;
  const uint8_t *m = a.block_mask + (size_t)h * nb * nb;
  int col = 0, row = 0;
  for (int i = 0; i < nb; ++i) {
    col += (m[(size_t)i * nb + j] != 0) && (!a.sp_causal || i >= j);
    row += (m[(size_t)j * nb + i] != 0) && (!a.sp_causal || i <= j);
  }
  a.sp_work[t] = col;
  a.sp_work[n + t] = row;
}

template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  constexpr int CPR = D / 8;
  constexpr int GPB = 256 / CPR;  // row groups per block
  const int tid = threadIdx.x;
  const long long total = a.rows;
  const long long r0 = ((long long)blockIdx.x * GPB + tid / CPR) * kPreRows;
  const int cc = tid % CPR;
  u32x4 o4[kPreRows], d4[kPreRows];
  float mv[kPreRows], lv[kPreRows];
#pragma unroll
  for (int k = 0; k < kPreRows; ++k) {
    const long long r = r0 + k;
    o4[k] = d4[k] = u32x4{0u, 0u, 0u, 0u};
    mv[k] = lv[k] = 0.f;
    if (r < total) {
      o4[k] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4 *>(a.o + r * D + cc * 8));
      d4[k] = ldg128(a.dout + r * D + cc * 8);
      if (cc == 0) {
        mv[k] = a.m[r];
        lv[k] = a.l[r];
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kPreRows; ++k) {
    const long long r = r0 + k;
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float ov =
          bf16_to_f32((uint16_t)(o4[k][e >> 1] >> (16 * (e & 1))));
      const float dv =
          bf16_to_f32((uint16_t)(d4[k][e >> 1] >> (16 * (e & 1))));
      part = fmaf(ov, dv, part);
    }
#pragma unroll
    for (int off = CPR / 2; off > 0; off >>= 1)
      part += __shfl_xor(part, off, 64);
    if (cc == 0 && r < total) {
      a.delta[r] = part;
      a.lse2[r] = lv[k] > 0.f ? fmaf(mv[k], kLog2e, __log2f(lv[k])) : INFINITY;
    }
  }
  // Block-sparse: one thread per (head, block) item counts its work (the
  // grid has at least 2 H N threads, H * ceil(N / 128) are needed).
  if (a.sp_work) sparse_work(a, blockIdx.x * 256 + tid);
}

template <int D, bool CAUSAL, bool PADDED, bool SPARSE, bool DROP>
__device__ __forceinline__ void bwd_dkdv_body(const BwdArgs &a, int i) {
  constexpr int BC = 128;    // keys per workgroup, 32 per wave
  constexpr int BR = 64;     // queries per step
  constexpr int CPR = D / 8;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][BR * D];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[2][BR * D];
  // Row statistics of the staged queries, interleaved (lse2, D) per query,
  // and -D by query: the start value of the dP accumulator, so the matrix
  // cores return dP - D (not with dropout, where D stays outside the mask).
  __shared__ __attribute__((aligned(16))) float LDs[2][2 * BR];
  __shared__ __attribute__((aligned(16))) float NDs[2][BR];
  // -lse2 / c by query: the start value of the S accumulator (without
  // dropout), so the matrix cores return S - lse2 / c and p = exp2(c s);
  // each lane fetches its 16 queries' start values of S and dP in eight
  // 16-byte reads, straight into the accumulators.
  __shared__ __attribute__((aligned(16))) float LSs[2][BR];

  const int tid = threadIdx.x;
  // The wave index is uniform: readfirstlane lets the compiler see it, so
  // per-wave conditions (diagonal tiles) become scalar branches.
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, hh = lane >> 5;
  const int bh = i % a.BH;
  const int kt = i / a.BH;
  const int b = bh / a.H;
  const SliceRows sr = slice_rows(a.cu_seqlens, a.total, a.N, a.H, bh);
  const int N = sr.n;
  const size_t hoff = sr.row0 * D;
  const int j0 = kt * BC;
  const int kw = j0 + 32 * wave;
  const int key = kw + ln;
  int kv_valid = N;
  if (PADDED) kv_valid = min(max(a.kv_len[b], 0), N);

  uint16_t *dkg = a.dk + hoff;
  uint16_t *dvg = a.dv + hoff;

  if (j0 >= kv_valid) {  // every key of the tile is masked: zero gradients
    for (int x = tid; x < BC * CPR; x += 256) {
      const int row = j0 + x / CPR, cc = x % CPR;
      if (row < N) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4 *>(dkg + (size_t)row * D + cc * 8) = z;
        *reinterpret_cast<u32x4 *>(dvg + (size_t)row * D + cc * 8) = z;
      }
    }
    return;
  }

  const uint16_t *qg = a.q + hoff;
  const uint16_t *kg = a.k + hoff;
  const uint16_t *vg = a.v + hoff;
  const uint16_t *dog = a.dout + hoff;
  const float *lse2 = a.lse2 + sr.row0;
  const float *dlt = a.delta + sr.row0;

  // This wave's 32 keys as B operands (lane = key, slots = head dim).
  bf16x8 kb[D / 16], vb[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (key < kv_valid) {
      x = ldg128(kg + (size_t)key * D + ks * 16 + 8 * hh);
      y = ldg128(vg + (size_t)key * D + ks * 16 + 8 * hh);
    }
    kb[ks] = __builtin_bit_cast(bf16x8, x);
    vb[ks] = __builtin_bit_cast(bf16x8, y);
  }

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[cb][r] = dv[cb][r] = 0.f;

  const float c = a.c;
  const float inv_c = 1.0f / c;
  const int q_begin = CAUSAL ? j0 : 0;

  // Double-buffered Q / dO blocks (DMA) and their row statistics; rows past
  // N read row N-1 and get lse2 = +inf, so their P is exactly 0.
  auto load_stats = [&](int q0, float &lv, float &dv2) {
    const bool ok = q0 + tid < N;
    lv = ok ? lse2[q0 + tid] : INFINITY;
    dv2 = ok ? dlt[q0 + tid] : 0.f;
  };
  // Query steps to visit: all from q_begin, or (block-sparse) those whose
  // 128-query block the mask column of this 128-key block allows.
  const int nsteps = (N + BR - 1) / BR;
  MaskWalk walk;
  if (SPARSE) {
    const int nb = (a.N + 127) / 128;
    const int h = bh - b * a.H;
    walk.mask = a.block_mask + (size_t)h * nb * nb + kt;
    walk.stride = nb;
    walk.per = 128 / BR;
    walk.n = nsteps;
  }
  auto next_step = [&](int st) { return SPARSE ? walk.next(st) : st; };

  // Q / dO step fills: uniform-base DMA for whole steps, the clamped
  // (out-of-line) fill for the ragged last one.
  const DmaOffsets<D, BR> doff;
  const uint32_t slice_bytes = (uint32_t)N * D * 2;  // N <= 2^20, d <= 128
  auto load_step = [&](int q1, int b2) {
    if (q1 + BR <= N) {
      dma_tile_at<D, BR>(Qs[b2], qg, slice_bytes, (uint32_t)q1 * D * 2, doff);
      dma_tile_at<D, BR>(dOs[b2], dog, slice_bytes, (uint32_t)q1 * D * 2, doff);
    } else {
      dma_tile_tail<D, BR>(Qs[b2], qg, q1, N - 1);
      dma_tile_tail<D, BR>(dOs[b2], dog, q1, N - 1);
    }
  };

  float l_nx = 0.f, d_nx = 0.f;
  int st = next_step(q_begin / BR);
  if (st < nsteps) {
    const int q1 = st * BR;
    load_step(q1, 0);
    if (tid < BR) {
      load_stats(q1, l_nx, d_nx);
      LDs[0][2 * tid] = l_nx;
      LDs[0][2 * tid + 1] = d_nx;
      NDs[0][tid] = -d_nx;
      LSs[0][tid] = -l_nx * inv_c;
    }
  }
  wait_dma();
  __syncthreads();

  // One step; instantiated for buffer 0 and buffer 1 so that every LDS
  // address is a per-lane base plus a constant offset.
  auto step = [&](auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int q0 = st * BR;
    const int sn = next_step(st + 1);
    const bool has_next = sn < nsteps;
    if (has_next) {  // the other buffers were last read before the barrier
      load_step(sn * BR, buf ^ 1);
      if (tid < BR) load_stats(sn * BR, l_nx, d_nx);
    }
    const uint16_t *Qt = Qs[buf];
    const uint16_t *dOt = dOs[buf];
    const float *LDt = LDs[buf];
    const float *NDt = NDs[buf];
    const float *LSt = LSs[buf];

#pragma unroll
    for (int qb = 0; qb < BR / 32; ++qb) {
      const int qs = q0 + 32 * qb;
      if (CAUSAL && qs + 31 < kw) continue;  // every query precedes every key
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
      if (!DROP) {  // s starts at -lse2/c, dp at -D of register r's query
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int qo = 32 * qb + 16 * (j >> 1) + 8 * hh + 4 * (j & 1);
          const f32x4 nd = *reinterpret_cast<const f32x4 *>(&NDt[qo]);
          const f32x4 ls = *reinterpret_cast<const f32x4 *>(&LSt[qo]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dp[4 * j + e] = nd[e];
            s[4 * j + e] = ls[e];
          }
        }
      }
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 qf = lds_row_frag<D>(Qt, 32 * qb + ln, ks * 16 + 8 * hh);
        const bf16x8 df = lds_row_frag<D>(dOt, 32 * qb + ln, ks * 16 + 8 * hh);
        s = mfma32(qf, kb[ks], s);
        dp = mfma32(df, vb[ks], dp);
      }
      // Register r holds query qs + 16*(r/8) + 8*hh + (r%8) of this key.
      // The mask test is wave-uniform: a scalar branch picks the variant.
      const bool need_mask =
          (kw + 32 > kv_valid) || (CAUSAL && qs < kw + 31);
      // Dropout keep bits of this key's 16 queries (bit 16*(r/8) + r%8).
      uint32_t kbits = 0;
      if (DROP)
        kbits = drop_keep_transposed(
            drop_bytes(a.drop, qs + ln, 2 * (kw >> 5) + hh, bh), a.drop.thr,
            ln, hh);
      uint32_t pp[8], ps[8];
      auto probs = [&](auto masked_tile) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // registers 2i, 2i+1 hold two consecutive queries: one 16-byte
          // read gives both (lse2, D) pairs
          const int qo0 = 32 * qb + 16 * (i >> 2) + 8 * hh + 2 * (i & 3);
          f32x4 st;
          if (DROP) st = *reinterpret_cast<const f32x4 *>(&LDt[2 * qo0]);
          float pv[2], dsv[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int r = 2 * i + t;
            // without dropout s already holds S - lse2 / c
            float p = DROP ? fast_exp2(fmaf(s[r], c, -st[2 * t]))
                           : fast_exp2(s[r] * c);
            if (decltype(masked_tile)::value) {
              const bool masked =
                  key >= kv_valid || (CAUSAL && key > q0 + qo0 + t);
              p = masked ? 0.f : p;
            }
            if (DROP) {
              // dV takes the kept P (scaled in the epilogue); dP passes
              // through the same mask and scale before the softmax rule.
              const bool kp = (kbits >> (16 * (r >> 3) + (r & 7))) & 1u;
              pv[t] = kp ? p : 0.f;
              dsv[t] = p * fmaf(dp[r], kp ? a.drop.keep_scale : 0.f,
                                -st[2 * t + 1]);
            } else {
              pv[t] = p;
              dsv[t] = p * dp[r];  // dp already holds dP - D
            }
          }
          pp[i] = pack_bf16x2(pv[0], pv[1]);
          ps[i] = pack_bf16x2(dsv[0], dsv[1]);
        }
      };
      if (need_mask)
        probs(std::true_type{});
      else
        probs(std::false_type{});
      // dV += P^T dO, dK += dS^T Q: A = this lane's registers (lane = key,
      // slots = 8 consecutive queries), B = transposed Q / dO fragments.
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const u32x4 pa = {pp[4 * s2], pp[4 * s2 + 1], pp[4 * s2 + 2],
                          pp[4 * s2 + 3]};
        const u32x4 sa = {ps[4 * s2], ps[4 * s2 + 1], ps[4 * s2 + 2],
                          ps[4 * s2 + 3]};
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) {
          const bf16x8 dof = lds_tr_frag<D>(dOt, 32 * qb + 16 * s2, cb * 32);
          const bf16x8 qtf = lds_tr_frag<D>(Qt, 32 * qb + 16 * s2, cb * 32);
          dv[cb] = mfma32(__builtin_bit_cast(bf16x8, pa), dof, dv[cb]);
          dk[cb] = mfma32(__builtin_bit_cast(bf16x8, sa), qtf, dk[cb]);
        }
      }
    }
    if (has_next && tid < BR) {
      LDs[buf ^ 1][2 * tid] = l_nx;
      LDs[buf ^ 1][2 * tid + 1] = d_nx;
      NDs[buf ^ 1][tid] = -d_nx;
      LSs[buf ^ 1][tid] = -l_nx * inv_c;
    }
    wait_dma();
    __syncthreads();
    st = sn;
  };
  while (st < nsteps) {
    step(std::integral_constant<int, 0>{});
    if (st >= nsteps) break;
    step(std::integral_constant<int, 1>{});
  }

  // Epilogue: dK = scale * dK_acc, dV (times the dropout keep scale);
  // lane = column, registers = key rows.
  const float vscale = DROP ? a.drop.keep_scale : 1.0f;
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = kw + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (kr < N) {
        const size_t idx = (size_t)kr * D + cb * 32 + ln;
        const __bf16 kv = (__bf16)(dk[cb][r] * a.scale);
        const __bf16 vv = (__bf16)(DROP ? dv[cb][r] * vscale : dv[cb][r]);
        dkg[idx] = __builtin_bit_cast(uint16_t, kv);
        dvg[idx] = __builtin_bit_cast(uint16_t, vv);
      }
    }
}

template <int D, bool CAUSAL, bool PADDED, bool SPARSE, bool DROP>
__device__ __forceinline__ void bwd_dq_body(const BwdArgs &a, int i) {
  constexpr int BR = 128;    // queries per workgroup, 32 per wave
  constexpr int BC = 64;     // keys per tile
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BC * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, hh = lane >> 5;
  const int nqt = (a.N + BR - 1) / BR;
  const int bh = i % a.BH;
  const int qt = nqt - 1 - i / a.BH;
  const int b = bh / a.H;
  const SliceRows sr = slice_rows(a.cu_seqlens, a.total, a.N, a.H, bh);
  const int N = sr.n;
  const size_t hoff = sr.row0 * D;
  const int q0 = qt * BR;
  if (q0 >= N) return;  // a packed sequence shorter than the longest one
  const int qw = q0 + 32 * wave;
  const int qi = qw + ln;
  int kv_valid = N;
  if (PADDED) kv_valid = min(max(a.kv_len[b], 0), N);
  int kend = kv_valid;
  if (CAUSAL) kend = min(kend, q0 + BR);
  const int ntiles = (kend + BC - 1) / BC;

  const uint16_t *qg = a.q + hoff;
  const uint16_t *kg = a.k + hoff;
  const uint16_t *vg = a.v + hoff;
  const uint16_t *dog = a.dout + hoff;

  // Q and dO as B operands (lane = query, slots = head dim), and this lane's
  // row statistics.
  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (qi < N) {
      x = ldg128(qg + (size_t)qi * D + ks * 16 + 8 * hh);
      y = ldg128(dog + (size_t)qi * D + ks * 16 + 8 * hh);
    }
    qf[ks] = __builtin_bit_cast(bf16x8, x);
    df[ks] = __builtin_bit_cast(bf16x8, y);
  }
  const float lrow = qi < N ? a.lse2[sr.row0 + qi] : INFINITY;
  const float drow = qi < N ? a.delta[sr.row0 + qi] : 0.f;
  // -D of this lane's query in every register: the start value of each
  // tile's dP^T accumulation, so the matrix cores return dP - D (not with
  // dropout, where D stays outside the keep mask).
  f32x16 negd;
#pragma unroll
  for (int r = 0; r < 16; ++r) negd[r] = DROP ? 0.f : -drow;

  f32x16 dq[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[cb][r] = 0.f;
  const float c = a.c;

  // Double-buffered K / V tiles (DMA); keys past kv_valid read the last
  // valid key (finite data that the mask excludes).
  // Key tiles to visit: all, or (block-sparse) those whose 128-key block
  // the mask row of this 128-query block allows.
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

  // K / V tile fills: uniform-base DMA for whole tiles, the clamped
  // (out-of-line) fill for the tail.
  const DmaOffsets<D, BC> doff;
  const uint32_t slice_bytes = (uint32_t)N * D * 2;  // N <= 2^20, d <= 128
  auto load_tile = [&](int k0, int b2) {
    if (k0 + BC <= kv_valid) {
      dma_tile_at<D, BC>(Ks[b2], kg, slice_bytes, (uint32_t)k0 * D * 2, doff);
      dma_tile_at<D, BC>(Vs[b2], vg, slice_bytes, (uint32_t)k0 * D * 2, doff);
    } else {
      dma_tile_tail<D, BC>(Ks[b2], kg, k0, kv_valid - 1);
      dma_tile_tail<D, BC>(Vs[b2], vg, k0, kv_valid - 1);
    }
  };
  int t = next_tile(0);
  if (t < ntiles) load_tile(t * BC, 0);
  wait_dma();
  __syncthreads();
  // One tile, instantiated per buffer (see bwd_dkdv_kernel).
  auto step = [&](auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int k0 = t * BC;
    const int tn = next_tile(t + 1);
    if (tn < ntiles)  // the other buffer was last read before the barrier
      load_tile(tn * BC, buf ^ 1);
    const uint16_t *Kt = Ks[buf];
    const uint16_t *Vt = Vs[buf];
    if (!(CAUSAL && k0 > qw + 31)) {  // else: tile above the diagonal
      uint32_t ps[2][8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 s, dp = negd;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8 kf = lds_row_frag<D>(Kt, 32 * kb + ln, ks * 16 + 8 * hh);
          const bf16x8 vf = lds_row_frag<D>(Vt, 32 * kb + ln, ks * 16 + 8 * hh);
          s = mfma32(kf, qf[ks], s);
          dp = mfma32(vf, df[ks], dp);
        }
        // Register r holds key k0 + 32*kb + 16*(r/8) + 8*hh + (r%8).  The
        // mask test is wave-uniform: a scalar branch picks the variant.
        const bool need_mask =
            (k0 + BC > kv_valid) || (CAUSAL && k0 + BC - 1 > qw);
        // Dropout: register r uses byte r of this lane's call for (query,
        // group 2*(key block) + hh).
        u32x4 rnd = {0u, 0u, 0u, 0u};
        if (DROP) rnd = drop_bytes(a.drop, qi, 2 * ((k0 >> 5) + kb) + hh, bh);
        auto grads = [&](auto masked_tile) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            float dsv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int r = 2 * i + u;
              float p = fast_exp2(fmaf(s[r], c, -lrow));
              if (decltype(masked_tile)::value) {
                const int kk =
                    k0 + 32 * kb + 16 * (r >> 3) + 8 * hh + (r & 7);
                const bool masked = kk >= kv_valid || (CAUSAL && kk > qi);
                p = masked ? 0.f : p;
              }
              if (DROP)
                dsv[u] = p * fmaf(dp[r],
                                  drop_keep(rnd, r, a.drop.thr)
                                      ? a.drop.keep_scale
                                      : 0.f,
                                  -drow);
              else
                dsv[u] = p * dp[r];  // dp already holds dP - D
            }
            ps[kb][i] = pack_bf16x2(dsv[0], dsv[1]);
          }
        };
        if (need_mask)
          grads(std::true_type{});
        else
          grads(std::false_type{});
      }
      // dQ^T += K^T dS^T: A = transposed K fragments, B = this lane's dS^T.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const u32x4 sb = {ps[kb][4 * s2], ps[kb][4 * s2 + 1],
                            ps[kb][4 * s2 + 2], ps[kb][4 * s2 + 3]};
#pragma unroll
          for (int cb = 0; cb < D / 32; ++cb) {
            const bf16x8 ktf = lds_tr_frag<D>(Kt, 32 * kb + 16 * s2, cb * 32);
            dq[cb] = mfma32(ktf, __builtin_bit_cast(bf16x8, sb), dq[cb]);
          }
        }
    }
    wait_dma();  // the next tile has landed
    __syncthreads();
    t = tn;
  };
  while (t < ntiles) {
    step(std::integral_constant<int, 0>{});
    if (t >= ntiles) break;
    step(std::integral_constant<int, 1>{});
  }

  if (qi < N) {
    uint16_t *out = a.dq + hoff + (size_t)qi * D;
    const float sc = a.scale;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = cb * 32 + 8 * g + 4 * hh;
        u32x2 w2;
        w2[0] = pack_bf16x2(dq[cb][4 * g] * sc, dq[cb][4 * g + 1] * sc);
        w2[1] = pack_bf16x2(dq[cb][4 * g + 2] * sc, dq[cb][4 * g + 3] * sc);
        *reinterpret_cast<u32x2 *>(out + c0) = w2;
      }
  }
}

// The items of each pass in decreasing work, by a counting sort over the
// work values 0 .. nb (nb <= 8192: N <= kMaxN = 2^20): workgroup 0 orders the
// dK/dV items, workgroup 1 the dQ items.  Items of equal work come in any
// order (each item's result does not depend on when it runs).
__global__ __launch_bounds__(1024) void sparse_order_kernel(BwdArgs a) {
  constexpr int kMaxBins = 8193;
  __shared__ int start[kMaxBins];
  __shared__ int part[1024];
  const int nb = (a.N + 127) / 128;
  const int n = a.H * nb;
  const int bins = nb + 1;
  const int32_t *work = a.sp_work + (size_t)blockIdx.x * n;
  int32_t *order = a.sp_order + (size_t)blockIdx.x * n;
  const int tid = threadIdx.x;
  for (int c = tid; c < bins; c += 1024) start[c] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += 1024) atomicAdd(&start[work[i]], 1);
  __syncthreads();
  // Bin c starts after every item of larger work.  Thread tid owns the
  // bins at positions [tid * per, (tid + 1) * per) of the descending order.
  const int per = (bins + 1023) / 1024;
  const int r0 = min(bins, tid * per), r1 = min(bins, r0 + per);
  int sum = 0;
  for (int r = r0; r < r1; ++r) sum += start[bins - 1 - r];
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan of part[]
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = tid ? part[tid - 1] : 0;
  for (int r = r0; r < r1; ++r) {
    const int c = bins - 1 - r;
    const int cnt = start[c];
    start[c] = run;
    run += cnt;
  }
  __syncthreads();
  for (int i = tid; i < n; i += 1024) order[atomicAdd(&start[work[i]], 1)] = i;
}

// Block-sparse: the index, in the bodies' numbering, of pass `kind`'s item
// at position idx of the heaviest-first order (positions r * B + b: the
// r-th heaviest (head, block), batch b).
__device__ __forceinline__ int sparse_item(const BwdArgs &a, int kind,
                                           int idx) {
  const int nb = (a.N + 127) / 128;
  const int r = idx / a.B, b = idx - r * a.B;
  const int it = a.sp_order[(size_t)kind * a.H * nb + r];
  const int h = it / nb, blk = it - h * nb;
  const int bh = b * a.H + h;
  return kind == 0 ? blk * a.BH + bh : (nb - 1 - blk) * a.BH + bh;
}

// Causal: low key tiles carry most work; dealt so each CU's two resident
// workgroups (d = 64) carry equal work.  Block-sparse: heaviest items first.
template <int D, bool CAUSAL, bool PADDED, bool SPARSE = false,
          bool DROP = false>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dkdv_kernel(
    BwdArgs a) {
  const int i = SPARSE ? sparse_item(a, 0, blockIdx.x)
                : CAUSAL ? causal_deal_order<D == 64 ? 2 : 1>(blockIdx.x)
                         : (int)blockIdx.x;
  bwd_dkdv_body<D, CAUSAL, PADDED, SPARSE, DROP>(a, i);
}

// Heaviest first, dealt so each CU's three resident workgroups (d = 64)
// carry equal work.
template <int D, bool CAUSAL, bool PADDED, bool SPARSE = false,
          bool DROP = false>
__global__ __launch_bounds__(256, D == 64 ? 3 : 1) void bwd_dq_kernel(
    BwdArgs a) {
  const int i = SPARSE ? sparse_item(a, 1, blockIdx.x)
                : CAUSAL ? causal_deal_order<D == 64 ? 3 : 1>(blockIdx.x)
                         : (int)blockIdx.x;
  bwd_dq_body<D, CAUSAL, PADDED, SPARSE, DROP>(a, i);
}

// Both passes in one launch of 2n workgroups (n of each kind): the grid
// alternates rounds of 256 workgroups between the two kinds, so a CU's two
// resident workgroups are one of each (their instruction mixes differ) and
// the tail of one pass overlaps the other.  Heaviest first within a kind
// (block-sparse: in the order of the items' work counts).
template <int D, bool CAUSAL, bool PADDED, bool SPARSE = false,
          bool DROP = false>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_fused_kernel(
    BwdArgs a, int n) {
  const int i = blockIdx.x;
  const int full = n / 256;
  int kind, idx;
  if (i < 512 * full) {
    const int r = i / 256;
    kind = r & 1;
    idx = (r >> 1) * 256 + (i & 255);
  } else {
    const int j = i - 512 * full, rem = n - 256 * full;
    kind = j >= rem;
    idx = 256 * full + (kind ? j - rem : j);
  }
  if (SPARSE) idx = sparse_item(a, kind, idx);
  if (kind == 0)
    bwd_dkdv_body<D, CAUSAL, PADDED, SPARSE, DROP>(a, idx);
  else
    bwd_dq_body<D, CAUSAL, PADDED, SPARSE, DROP>(a, idx);
}

template <int D, bool CAUSAL, bool PADDED, bool SPARSE = false,
          bool DROP = false>
void bwd_launch_main(const BwdArgs &a, hipStream_t st) {
  const int nkt = (a.N + 127) / 128;
  // d = 64 without dropout: one launch for both passes (measured 2-7%
  // faster than two; the dropout kernels would spill registers there).
  if constexpr (D == 64 && !DROP) {
    const int n = nkt * a.BH;
    hipLaunchKernelGGL((bwd_fused_kernel<D, CAUSAL, PADDED, SPARSE, DROP>),
                       dim3((unsigned)(2 * n)), dim3(256), 0, st, a, n);
  } else {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, PADDED, SPARSE, DROP>),
                       dim3((unsigned)(nkt * a.BH)), dim3(256), 0, st, a);
    const int nqt = (a.N + 127) / 128;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, PADDED, SPARSE, DROP>),
                       dim3((unsigned)(nqt * a.BH)), dim3(256), 0, st, a);
  }
}

template <int D, bool CAUSAL>
hipError_t bwd_dispatch(const BwdArgs &a, hipStream_t st) {
  const long long rows = a.rows;
  const long long rpb = 256 / (D / 8) * kPreRows;
  hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)((rows + rpb - 1) / rpb)),
                     dim3(256), 0, st, a);
  if (a.block_mask) {
    // Items heaviest first: the work of a (head, block) item, counted by
    // bwd_pre_kernel above, is the number of blocks its mask column (dK/dV)
    // or row (dQ) allows, and a column that every row allows can carry
    // many times the average.
    hipLaunchKernelGGL(sparse_order_kernel, dim3(2), dim3(1024), 0, st, a);
    bwd_launch_main<D, CAUSAL, false, true>(a, st);
  }
  else if (a.drop.thr != 0 && a.kv_len)
    bwd_launch_main<D, CAUSAL, true, false, true>(a, st);
  else if (a.drop.thr != 0)
    bwd_launch_main<D, CAUSAL, false, false, true>(a, st);
  else if (a.kv_len)
    bwd_launch_main<D, CAUSAL, true>(a, st);
  else
    bwd_launch_main<D, CAUSAL, false>(a, st);
  return hipGetLastError();
}

}  // namespace

#ifdef FA355_BWD_NC128_UNIT
hipError_t launch_bwd_nc128(const BwdArgs &a, hipStream_t s) {
  return bwd_dispatch<128, false>(a, s);
}
#else
hipError_t launch_bwd(const BwdArgs &a, int d, bool causal, hipStream_t s) {
  if (d == 64)
    return causal ? bwd_dispatch<64, true>(a, s) : bwd_dispatch<64, false>(a, s);
  return causal ? bwd_dispatch<128, true>(a, s) : launch_bwd_nc128(a, s);
}
#endif

}  // namespace fa355
