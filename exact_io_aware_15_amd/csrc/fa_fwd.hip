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
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa355 {

namespace {

// MFMA row p of the K operand holds key key_of_row(p) of its 32-key block
// (bits 2 and 3 of p exchanged).  With the C-operand row order 8*(r/4)+4h+r%4
// this puts key 16*(r/8) + 8*h + (r%8) in score register r of lane half h, so
// each lane's eight consecutive registers are eight consecutive keys: exactly
// the B-operand slots of the following P V MFMA, and V^T can be read with one
// 16-byte LDS load per fragment.
__device__ __forceinline__ int key_of_row(int p) {
  return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1);
}

template <int D, bool CAUSAL, bool PADDED>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int BR = 128;                         // queries per workgroup
  constexpr int BC = 64;                          // keys per tile
  constexpr int KP = D + 8;                       // K row pitch (bf16)
  constexpr int VP = BC + 8;                      // V^T row pitch (bf16)
  constexpr int CPR = D / 8;                      // 16-byte chunks per row
  constexpr int KCH = BC * CPR / 256;             // K chunks per thread
  constexpr int VCH = (BC / 2) * CPR / 256;       // V row-pair chunks per thread
  static_assert(KCH >= 1 && VCH >= 1, "tile too small for 256 threads");
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BC * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, hh = lane >> 5;

  // Query tiles in descending order (heaviest causal tiles first); heads vary
  // fastest, so workgroups dealt round-robin to the 8 XCDs keep one head's
  // tiles on one XCD's L2 when B*H is a multiple of 8 (or divides 8).
  const int nqt = (a.N + BR - 1) / BR;
  const int bh = blockIdx.x % a.BH;
  const int qt = nqt - 1 - (int)(blockIdx.x / a.BH);
  const int b = bh / a.H;
  const int N = a.N;
  const size_t hoff = (size_t)bh * N * D;
  const uint16_t *__restrict__ qg = (const uint16_t *)a.q + hoff;
  const uint16_t *__restrict__ kg = (const uint16_t *)a.k + hoff;
  const uint16_t *__restrict__ vg = (const uint16_t *)a.v + hoff;

  const int q0 = qt * BR;
  const int qw = q0 + wave * 32;
  const int qi = qw + ln;
  int kv_valid = N;
  if (PADDED) kv_valid = min(max(a.kv_len[b], 0), N);
  int kend = kv_valid;
  if (CAUSAL) kend = min(kend, q0 + BR);
  const int ntiles = (kend + BC - 1) / BC;

  // Q as the B operand of S^T = K Q^T: lane holds Q[qi][16*ks + 8*hh + e].
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qi < N) x = ldg128(qg + (size_t)qi * D + ks * 16 + 8 * hh);
    qf[ks] = __builtin_bit_cast(bf16x8, x);
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.f;
  float m_run = kMaxInit;  // running max of raw (unscaled) scores
  float l_run = 0.f;       // running sum over this lane's half of the keys
  const float c = a.c;

  u32x4 kreg[KCH];
  u32x4 vreg[VCH][2];

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int ci = tid + 256 * u;
      const int row = ci / CPR, cc = ci % CPR;
      const int key = k0 + row;
      kreg[u] = u32x4{0u, 0u, 0u, 0u};
      if (key < kv_valid) kreg[u] = ldg128(kg + (size_t)key * D + cc * 8);
    }
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int pi = tid + 256 * u;
      const int rp = pi / CPR, cc = pi % CPR;
      const int key = k0 + 2 * rp;
      vreg[u][0] = u32x4{0u, 0u, 0u, 0u};
      vreg[u][1] = u32x4{0u, 0u, 0u, 0u};
      if (key < kv_valid) vreg[u][0] = ldg128(vg + (size_t)key * D + cc * 8);
      if (key + 1 < kv_valid)
        vreg[u][1] = ldg128(vg + (size_t)(key + 1) * D + cc * 8);
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int ci = tid + 256 * u;
      const int row = ci / CPR, cc = ci % CPR;
      const int prow = (row & ~31) | key_of_row(row & 31);
      *reinterpret_cast<u32x4 *>(&Ks[prow * KP + cc * 8]) = kreg[u];
    }
    // V^T[c][key]: key chunks of 8 are XOR-swizzled by (c / 8) % 8 so the
    // transposing stores and the 16-byte fragment loads avoid bank conflicts.
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int pi = tid + 256 * u;
      const int rp = pi / CPR, cc = pi % CPR;
      const int jc = (2 * rp) >> 3, jo = (2 * rp) & 7;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int col = cc * 8 + e;
        const int jcs = jc ^ (cc & 7);
        const uint32_t lo = (vreg[u][0][e >> 1] >> (16 * (e & 1))) & 0xffffu;
        const uint32_t hi = (vreg[u][1][e >> 1] >> (16 * (e & 1))) & 0xffffu;
        *reinterpret_cast<uint32_t *>(&Vt[col * VP + jcs * 8 + jo]) =
            lo | (hi << 16);
      }
    }
  };

  if (ntiles > 0) load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * BC;
    __syncthreads();  // every wave is done reading the previous tile
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) load_tile(k0 + BC);  // in flight during compute

    if (CAUSAL && k0 > qw + 31) continue;  // tile entirely above the diagonal

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 kf = *reinterpret_cast<const u32x4 *>(
            &Ks[(kb * 32 + ln) * KP + ks * 16 + 8 * hh]);
        s[kb] = mfma32(__builtin_bit_cast(bf16x8, kf), qf[ks], s[kb]);
      }
    }

    const bool need_mask =
        (k0 + BC > kv_valid) || (CAUSAL && k0 + BC - 1 > qw);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 16 * (r >> 3) + 8 * hh + (r & 7);
          const bool masked = key >= kv_valid || (CAUSAL && key > qi);
          s[kb][r] = masked ? -INFINITY : s[kb][r];
        }
    }

    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2((m_run - m_new) * c);
    const float mc = m_new * c;
    m_run = m_new;

    uint32_t pk[2][8];
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p0 = fast_exp2(fmaf(s[kb][2 * i], c, -mc));
        const float p1 = fast_exp2(fmaf(s[kb][2 * i + 1], c, -mc));
        pk[kb][i] = pack_bf16x2(p0, p1);
        lsum = dot2_ones(pk[kb][i], lsum);
      }
    l_run = fmaf(l_run, alpha, lsum);

#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;

#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const u32x4 pb = {pk[kb][4 * s2], pk[kb][4 * s2 + 1],
                          pk[kb][4 * s2 + 2], pk[kb][4 * s2 + 3]};
        const int jc = kb * 4 + 2 * s2 + hh;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) {
          const int col = cb * 32 + ln;
          const int jcs = jc ^ ((col >> 3) & 7);
          const u32x4 vf =
              *reinterpret_cast<const u32x4 *>(&Vt[col * VP + jcs * 8]);
          oacc[cb] = mfma32(__builtin_bit_cast(bf16x8, vf),
                            __builtin_bit_cast(bf16x8, pb), oacc[cb]);
        }
      }
  }

  // Epilogue: O = o / l (0 for a row with no visible key), m in natural units.
  const float l_tot = l_run + xor32(l_run);
  if (qi < N) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    uint16_t *og = (uint16_t *)a.o + hoff + (size_t)qi * D;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = cb * 32 + 8 * g + 4 * hh;
        u32x2 w2;
        w2[0] = pack_bf16x2(oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv);
        w2[1] = pack_bf16x2(oacc[cb][4 * g + 2] * inv,
                            oacc[cb][4 * g + 3] * inv);
        *reinterpret_cast<u32x2 *>(og + c0) = w2;
      }
    if (hh == 0 && a.m != nullptr) {
      const size_t ri = (size_t)bh * N + qi;
      a.m[ri] = l_tot > 0.f ? m_run * a.scale : -INFINITY;
      a.l[ri] = l_tot;
    }
  }
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
  const int N = a.N;
  const size_t hoff = (size_t)bh * N * D;
  const float *qg = (const float *)a.q + hoff;
  const float *kg = (const float *)a.k + hoff;
  const float *vg = (const float *)a.v + hoff;
  (void)nqt;
  const int qi = qt * 64 + tid;
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
      a.m[(size_t)bh * N + qi] = l_run > 0.f ? m_run * a.scale : -INFINITY;
      a.l[(size_t)bh * N + qi] = l_run;
    }
  }
}

template <int D, bool CAUSAL>
hipError_t fwd_bf16_dispatch_pad(const FwdArgs &a, hipStream_t s) {
  const int nqt = (a.N + 127) / 128;
  dim3 grid((unsigned)(nqt * a.BH)), block(256);
  if (a.kv_len)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, true>), grid, block, 0, s,
                       a);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, false>), grid, block, 0, s,
                       a);
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

hipError_t launch_fwd_f32(const FwdArgs &a, int d, bool causal,
                          hipStream_t s) {
  if (d == 64)
    return causal ? fwd_f32_dispatch_pad<64, true>(a, s)
                  : fwd_f32_dispatch_pad<64, false>(a, s);
  return causal ? fwd_f32_dispatch_pad<128, true>(a, s)
                : fwd_f32_dispatch_pad<128, false>(a, s);
}

}  // namespace fa355
