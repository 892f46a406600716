// fa_bwd.hip -- exact attention backward for gfx950 by recomputation.
//
// FA notes §3.3: the backward pass keeps only O and the row statistics (m, l)
// from the forward pass and rebuilds the score and probability tiles on chip.
// The gradient formulas are the softmax chain rule (the pages do not print
// them):  dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
// dQ = scale dS K,  dK = scale dS^T Q.
//
// Three launches:
//   1. pre:   D_i = sum_c dO_ic O_ic; the log2-domain row offset
//             lse2_i = m_i log2(e) + log2(l_i) so that P = exp2(c S - lse2);
//             the fp32 dQ accumulator rows are cleared.
//   2. main:  one workgroup per 128-key tile (4 waves x 32 keys), keeping its
//             K and V fragments and its dK, dV accumulators in registers while
//             32-query blocks of Q and dO stream through LDS.  Five bf16 MFMA
//             contractions per block; dQ partials go to the fp32 accumulator
//             with hardware float atomics.
//   3. conv:  dQ = scale * accumulator, rounded to bf16.
//
// Fragment layout (see fa_device.h): S = Q K^T is computed with keys as MFMA
// columns, so a lane owns one key and its registers hold 16 queries.  Rows of
// the Q / dO operands are stored in LDS in the order key_of_row() gives, which
// makes each lane's registers 8 consecutive queries: directly the A operand
// (P^T, dS^T) of the dV and dK products.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa355 {

namespace {

__device__ __forceinline__ int row_order(int p) {
  return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1);
}

template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  constexpr int CPR = D / 8;
  constexpr int RPB = 256 / CPR;  // rows per block
  const int tid = threadIdx.x;
  const long long total = (long long)a.BH * a.N;
  const long long r = (long long)blockIdx.x * RPB + tid / CPR;
  const int cc = tid % CPR;
  float part = 0.f;
  if (r < total) {
    const u32x4 o4 = ldg128(a.o + r * D + cc * 8);
    const u32x4 d4 = ldg128(a.dout + r * D + cc * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float ov = bf16_to_f32((uint16_t)(o4[e >> 1] >> (16 * (e & 1))));
      const float dv = bf16_to_f32((uint16_t)(d4[e >> 1] >> (16 * (e & 1))));
      part = fmaf(ov, dv, part);
    }
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4 *>(a.dq_acc + r * D + cc * 8) = z;
    *reinterpret_cast<f32x4 *>(a.dq_acc + r * D + cc * 8 + 4) = z;
  }
#pragma unroll
  for (int off = CPR / 2; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
  if (cc == 0 && r < total) {
    a.delta[r] = part;
    const float l = a.l[r];
    a.lse2[r] = l > 0.f ? fmaf(a.m[r], kLog2e, __log2f(l)) : INFINITY;
  }
}

template <int D, bool CAUSAL, bool PADDED>
__global__ __launch_bounds__(256, (D == 64 ? 2 : 1)) void bwd_main_kernel(
    BwdArgs a) {
  constexpr int BC = 128;        // keys per workgroup, 32 per wave
  constexpr int BR = 32;         // queries per step
  constexpr int QP = D + 8;      // row-major Q / dO pitch (bf16)
  constexpr int TP = BR + 8;     // transposed Q^T / dO^T pitch (bf16)
  constexpr int SP = 32 + 8;     // per-wave dS pitch (bf16)
  constexpr int CPR = D / 8;
  constexpr int NPAIR = (BR / 2) * CPR;  // row-pair chunks per tile
  static_assert(NPAIR <= 256, "one row-pair chunk per thread at most");
  __shared__ __attribute__((aligned(16))) uint16_t Qs[BR * QP];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[BR * QP];
  __shared__ __attribute__((aligned(16))) uint16_t QT[D * TP];
  __shared__ __attribute__((aligned(16))) uint16_t dOT[D * TP];
  __shared__ __attribute__((aligned(16))) uint16_t dSs[4][32 * SP];
  __shared__ float L2s[BR], Dls[BR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, hh = lane >> 5;
  const int N = a.N;
  const int bh = blockIdx.x % a.BH;
  const int kt = blockIdx.x / a.BH;  // causal: low key tiles carry most work
  const int b = bh / a.H;
  const size_t hoff = (size_t)bh * N * D;
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
  float *dqa = a.dq_acc + hoff;
  const float *lse2 = a.lse2 + (size_t)bh * N;
  const float *dlt = a.delta + (size_t)bh * N;

  // Resident fragments of this wave's 32 keys.
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
  // K as the B operand of dQ = dS K: lane (column c) holds keys 16s+8hh+e.
  bf16x8 ktb[D / 32][2];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      uint32_t w[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int k0 = kw + 16 * s2 + 8 * hh + 2 * e2;
        const int col = cb * 32 + ln;
        const uint32_t lo = k0 < kv_valid ? kg[(size_t)k0 * D + col] : 0u;
        const uint32_t hi =
            k0 + 1 < kv_valid ? kg[(size_t)(k0 + 1) * D + col] : 0u;
        w[e2] = lo | (hi << 16);
      }
      const u32x4 x = {w[0], w[1], w[2], w[3]};
      ktb[cb][s2] = __builtin_bit_cast(bf16x8, x);
    }

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[cb][r] = dv[cb][r] = 0.f;

  const float c = a.c;
  uint16_t *dsw = dSs[wave];
  const int q_begin = CAUSAL ? j0 : 0;

  for (int q0 = q_begin; q0 < N; q0 += BR) {
    __syncthreads();  // previous block's LDS operands are no longer in use
    if (tid < NPAIR) {
      const int rp = tid / CPR, cc = tid % CPR;
      const int r0 = 2 * rp, r1 = 2 * rp + 1;
      u32x4 qa = {0u, 0u, 0u, 0u}, qb = qa, da = qa, db = qa;
      if (q0 + r0 < N) {
        qa = ldg128(qg + (size_t)(q0 + r0) * D + cc * 8);
        da = ldg128(dog + (size_t)(q0 + r0) * D + cc * 8);
      }
      if (q0 + r1 < N) {
        qb = ldg128(qg + (size_t)(q0 + r1) * D + cc * 8);
        db = ldg128(dog + (size_t)(q0 + r1) * D + cc * 8);
      }
      *reinterpret_cast<u32x4 *>(&Qs[row_order(r0) * QP + cc * 8]) = qa;
      *reinterpret_cast<u32x4 *>(&Qs[row_order(r1) * QP + cc * 8]) = qb;
      *reinterpret_cast<u32x4 *>(&dOs[row_order(r0) * QP + cc * 8]) = da;
      *reinterpret_cast<u32x4 *>(&dOs[row_order(r1) * QP + cc * 8]) = db;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int col = cc * 8 + e;
        const int sh = 16 * (e & 1);
        const uint32_t q2 = ((qa[e >> 1] >> sh) & 0xffffu) |
                            (((qb[e >> 1] >> sh) & 0xffffu) << 16);
        const uint32_t d2 = ((da[e >> 1] >> sh) & 0xffffu) |
                            (((db[e >> 1] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<uint32_t *>(&QT[col * TP + r0]) = q2;
        *reinterpret_cast<uint32_t *>(&dOT[col * TP + r0]) = d2;
      }
    }
    if (tid >= 256 - BR) {
      const int i = tid - (256 - BR);
      const bool ok = q0 + i < N;
      L2s[i] = ok ? lse2[q0 + i] : INFINITY;
      Dls[i] = ok ? dlt[q0 + i] : 0.f;
    }
    __syncthreads();

    if (CAUSAL && q0 + BR - 1 < kw) continue;  // every query precedes every key

    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const u32x4 qf =
          *reinterpret_cast<const u32x4 *>(&Qs[ln * QP + ks * 16 + 8 * hh]);
      const u32x4 df =
          *reinterpret_cast<const u32x4 *>(&dOs[ln * QP + ks * 16 + 8 * hh]);
      s = mfma32(__builtin_bit_cast(bf16x8, qf), kb[ks], s);
      dp = mfma32(__builtin_bit_cast(bf16x8, df), vb[ks], dp);
    }

    // Register r of this lane holds query q0 + 16*(r/8) + 8*hh + (r%8).
    const bool need_mask =
        (kw + 32 > kv_valid) || (CAUSAL && q0 < kw + 31);
    uint32_t pp[8], ps[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float pv[2], dsv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int r = 2 * i + t;
        const int qo = 16 * (r >> 3) + 8 * hh + (r & 7);
        float p = fast_exp2(fmaf(s[r], c, -L2s[qo]));
        if (need_mask) {
          const bool masked =
              key >= kv_valid || (CAUSAL && key > q0 + qo);
          p = masked ? 0.f : p;
        }
        pv[t] = p;
        dsv[t] = p * (dp[r] - Dls[qo]);
      }
      pp[i] = pack_bf16x2(pv[0], pv[1]);
      ps[i] = pack_bf16x2(dsv[0], dsv[1]);
    }

    // dV += P^T dO and dK += dS^T Q: this lane's registers are the A operand.
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const u32x4 pa = {pp[4 * s2], pp[4 * s2 + 1], pp[4 * s2 + 2],
                        pp[4 * s2 + 3]};
      const u32x4 sa = {ps[4 * s2], ps[4 * s2 + 1], ps[4 * s2 + 2],
                        ps[4 * s2 + 3]};
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        const int col = cb * 32 + ln;
        const u32x4 dof = *reinterpret_cast<const u32x4 *>(
            &dOT[col * TP + 16 * s2 + 8 * hh]);
        const u32x4 qtf = *reinterpret_cast<const u32x4 *>(
            &QT[col * TP + 16 * s2 + 8 * hh]);
        dv[cb] = mfma32(__builtin_bit_cast(bf16x8, pa),
                        __builtin_bit_cast(bf16x8, dof), dv[cb]);
        dk[cb] = mfma32(__builtin_bit_cast(bf16x8, sa),
                        __builtin_bit_cast(bf16x8, qtf), dk[cb]);
      }
    }

    // dQ = dS K: transpose dS through this wave's private LDS slice so that
    // lanes own queries, then accumulate the partial into fp32 with atomics.
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int r = 2 * i + t;
        const int qo = 16 * (r >> 3) + 8 * hh + (r & 7);
        dsw[qo * SP + ln] = (uint16_t)(ps[i] >> (16 * t));
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    bf16x8 dsa[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
      dsa[s2] = __builtin_bit_cast(
          bf16x8,
          *reinterpret_cast<const u32x4 *>(&dsw[ln * SP + 16 * s2 + 8 * hh]));
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
      f32x16 dq;
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[r] = 0.f;
      dq = mfma32(dsa[0], ktb[cb][0], dq);
      dq = mfma32(dsa[1], ktb[cb][1], dq);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = q0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (qr < N)
          atomicAdd(dqa + (size_t)qr * D + cb * 32 + ln, dq[r]);
      }
    }
  }

  // Epilogue: dK = scale * dK_acc, dV; lane = column, registers = key rows.
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = kw + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (kr < N) {
        const size_t idx = (size_t)kr * D + cb * 32 + ln;
        const __bf16 kv = (__bf16)(dk[cb][r] * a.scale);
        const __bf16 vv = (__bf16)dv[cb][r];
        dkg[idx] = __builtin_bit_cast(uint16_t, kv);
        dvg[idx] = __builtin_bit_cast(uint16_t, vv);
      }
    }
}

__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(BwdArgs a,
                                                             long long n8) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 x0 = *reinterpret_cast<const f32x4 *>(a.dq_acc + i * 8);
  const f32x4 x1 = *reinterpret_cast<const f32x4 *>(a.dq_acc + i * 8 + 4);
  const float s = a.scale;
  u32x4 w;
  w[0] = pack_bf16x2(x0[0] * s, x0[1] * s);
  w[1] = pack_bf16x2(x0[2] * s, x0[3] * s);
  w[2] = pack_bf16x2(x1[0] * s, x1[1] * s);
  w[3] = pack_bf16x2(x1[2] * s, x1[3] * s);
  *reinterpret_cast<u32x4 *>(a.dq + i * 8) = w;
}

template <int D, bool CAUSAL>
hipError_t bwd_dispatch(const BwdArgs &a, hipStream_t st) {
  const long long rows = (long long)a.BH * a.N;
  const int rpb = 256 / (D / 8);
  hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)((rows + rpb - 1) / rpb)),
                     dim3(256), 0, st, a);
  const int nkt = (a.N + 127) / 128;
  dim3 grid((unsigned)(nkt * a.BH));
  if (a.kv_len)
    hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL, true>), grid, dim3(256), 0,
                       st, a);
  else
    hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL, false>), grid, dim3(256), 0,
                       st, a);
  const long long n8 = rows * D / 8;
  hipLaunchKernelGGL(bwd_dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)),
                     dim3(256), 0, st, a, n8);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, int d, bool causal, hipStream_t s) {
  if (d == 64)
    return causal ? bwd_dispatch<64, true>(a, s) : bwd_dispatch<64, false>(a, s);
  return causal ? bwd_dispatch<128, true>(a, s)
                : bwd_dispatch<128, false>(a, s);
}

}  // namespace fa355
