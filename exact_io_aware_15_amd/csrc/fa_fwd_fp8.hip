// fa_fwd_fp8.hip -- exact-attention forward with FP8 (E4M3) operands.
//
// The same tiled, fused forward as fa_fwd.hip (FA notes §3.2 / §3.4; S12's
// deferred-normalisation recurrence), with both contractions on gfx950's
// 32x32x64 FP8 matrix instruction, which runs at twice the bf16 rate.  The
// pages mention FP8 only as a FlashAttention-3 feature (S12, production-
// practice list) and fix no scaling convention.  Here Q, K and V arrive as
// E4M3 codes with one fp32 descale per (batch, head) each: the real inputs
// are code * descale.  The Q and K
// descales fold into the score scale, the V descale into the epilogue.  P is
// rounded to E4M3 to feed the second contraction: p' = 2^6 * exp2(c (s -
// m_ref)) with the reference max moved whenever the row max outgrows it by
// more than 2 log2 units, so p' <= 2^8 stays inside E4M3's range (448) and
// values down to 2^-15 of the reference keep a representation.  The row sum l
// is taken from p' before rounding, in fp32.
//
// Layout of one workgroup: 4 waves x 32 queries, 64-key tiles double
// buffered in LDS by direct DMA.  S^T = K Q^T leaves one query per lane; the
// K tile's rows are stored so that register r of key block kb holds key
// 32*kb + 16*hh + r, which makes a lane's 32 probabilities the 32 contraction
// slots (keys 16*hh .. of each 32-key block) of the P operand, and the V^T
// operand the matching two 16-byte chunks of each V^T row.  V is therefore
// taken transposed, [B,H,d,ldv]: its key axis is the contraction axis.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa355 {

namespace {

constexpr float kRescaleLog2F8 = 2.0f;  // reference max slack, log2 units
constexpr float kBiasLog2F8 = 6.0f;     // p' = 2^6 exp2(c (s - m_ref))

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // FP8 (E4M3) x FP8 (E4M3), fp32 accumulate; block scales 127 = 2^0.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127,
                                                         0, 127);
}

// Storage row p of each 32-row block of the K tile holds logical key
// key_perm8(p): with the C-operand row order 8*(r/4) + 4*hh + r%4 this puts
// key 16*hh + r in register r.
__device__ __forceinline__ int key_perm8(int p) {
  return (p & ~31) | (p & 3) | (((p >> 3) & 3) << 2) | (((p >> 2) & 1) << 4);
}

// 16-byte chunk permutations (XOR by row bits) that make the 16-lane passes
// of the operand reads hit 16 distinct bank groups: K rows of D bytes, V^T
// rows of 64 bytes.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  return D == 64 ? ((r >> 2) & 3) : ((r >> 1) & 7);
}
__device__ __forceinline__ int vt_swz(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ void dma16(const uint8_t *src, uint8_t *dst) {
  __builtin_amdgcn_global_load_lds(
      (const __attribute__((address_space(1))) void *)src,
      (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
}

// Whole-tile fill through a raw buffer resource over the `bytes` bytes of a
// slice at `base`: each wave issues SEGS/4 16-byte-per-lane loads at byte
// offset off[u] (per lane) + tile_off (uniform) into its 1 KB segments.
template <int SEGS>
__device__ __forceinline__ void dma16_rows(uint8_t *tile, const uint8_t *base,
                                           uint32_t bytes, uint32_t tile_off,
                                           const uint32_t (&off)[SEGS / 4]) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto src = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(base), (short)0, (int)bytes, 0x00020000);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t soff = __builtin_amdgcn_readfirstlane(tile_off);
#pragma unroll
  for (int u = 0; u < SEGS / 4; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        src,
        (__attribute__((address_space(3))) void *)(tile + (wave + 4 * u) *
                                                              1024),
        16, off[u], soff, 0, 0);
#endif
}

__device__ __forceinline__ i32x8 cat8(u32x4 lo, u32x4 hi) {
  const i32x8 v = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  return v;
}

// Keeps the first n (0..16) bytes of a 16-byte chunk, zeroing the rest.
__device__ __forceinline__ u32x4 keep_bytes(u32x4 x, int n) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int k = n - 4 * w;
    const uint32_t m = k >= 4 ? 0xffffffffu
                              : (k <= 0 ? 0u : (1u << (8 * k)) - 1u);
    x[w] &= m;
  }
  return x;
}

// Clamped fill of a tile that reaches past the valid keys or past ldv (kept
// out of line: it runs at most once per workgroup).
template <int D>
__device__ __attribute__((noinline)) void fp8_tail_tile(
    uint8_t *ks, uint8_t *vs, const uint8_t *kg, const uint8_t *vtg, int k0,
    int kv_valid, int ldv) {
  constexpr int KCH = D / 16;
  constexpr int SEGS = 64 * D / 1024;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < SEGS / 4; ++u) {
    const int seg = wave + 4 * u;
    const int p = seg * 64 + lane;
    const int r = p / KCH, phys = p % KCH;
    const int key = min(k0 + key_perm8(r), kv_valid - 1);
    dma16(kg + (size_t)key * D + (phys ^ k_swz<D>(r)) * 16, ks + seg * 1024);
  }
#pragma unroll
  for (int u = 0; u < SEGS / 4; ++u) {
    const int seg = wave + 4 * u;
    const int p = seg * 64 + lane;
    const int r = p >> 2, phys = p & 3;
    const int kc = min(k0 + 16 * (phys ^ vt_swz(r)), ldv - 16);
    dma16(vtg + (size_t)r * ldv + kc, vs + seg * 1024);
  }
}

template <int D, bool CAUSAL, bool PADDED>
__global__ __launch_bounds__(256, 2) void fwd_fp8_kernel(Fp8FwdArgs a) {
  constexpr int BR = 128;        // queries per workgroup
  constexpr int BC = 64;         // keys per tile
  constexpr int KCH = D / 16;    // 16-byte chunks per K row
  constexpr int SEGS = BC * D / 1024;  // 1 KB DMA segments per tile (each)
  static_assert(SEGS % 4 == 0, "tile shape");
  // One LDS object for both tiles of both buffers.
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * BC * D];
  auto Ks = [&](int buf) { return smem + buf * BC * D; };
  auto Vs = [&](int buf) { return smem + (2 + buf) * BC * D; };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, hh = lane >> 5;
  const int N = a.N;
  const int nqt = (N + BR - 1) / BR;
  const int bh = blockIdx.x % a.BH;
  const int qt = nqt - 1 - (int)(blockIdx.x / a.BH);
  const int b = bh / a.H;

  const float qd = a.q_descale ? a.q_descale[bh] : 1.0f;
  const float kd = a.k_descale ? a.k_descale[bh] : 1.0f;
  const float vd = a.v_descale ? a.v_descale[bh] : 1.0f;
  const float sscale = a.scale * qd * kd;  // natural units per raw score
  const float c = sscale * kLog2e;         // log2 units per raw score

  const size_t hoff = (size_t)bh * N * D;
  const uint8_t *qg = a.q + hoff;
  const uint8_t *kg = a.k + hoff;
  const uint8_t *vtg = a.vt + (size_t)bh * D * a.ldv;
  const int ldv = a.ldv;
  int kv_valid = N;
  if (PADDED) kv_valid = min(max(a.kv_len[b], 0), N);

  const int q0 = qt * BR;
  const int qw = q0 + 32 * wave;
  const int qi = qw + ln;
  int kend = kv_valid;
  if (CAUSAL) kend = max(0, min(kend, q0 + BR));
  const int ntiles = (kend + BC - 1) / BC;

  // Q as the B operand: lane holds bytes 64*mi + 32*hh .. +31 of its query.
  i32x8 qf[D / 64];
#pragma unroll
  for (int mi = 0; mi < D / 64; ++mi) {
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (qi < N) {
      const uint8_t *p = qg + (size_t)qi * D + 64 * mi + 32 * hh;
      lo = ldg128(p);
      hi = ldg128(p + 16);
    }
    qf[mi] = cat8(lo, hi);
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.f;
  float m_ref = kMaxInit, m_max = kMaxInit, l_run = 0.f;

  // K tile: storage row r holds key k0 + key_perm8(r) (clamped to the last
  // valid key), chunks permuted by k_swz.  V^T tile: row = head dimension,
  // 64 key bytes, chunks permuted by vt_swz; chunks starting at or past ldv
  // read the row's last chunk instead (its keys are masked).
  // Per-lane source offsets of a whole tile (relative to its first key),
  // computed once: tiles inside the valid keys are fetched from a uniform
  // base; the tail tile takes the clamped path.
  uint32_t koff[SEGS / 4], voff[SEGS / 4];
#pragma unroll
  for (int u = 0; u < SEGS / 4; ++u) {
    const int p = (wave + 4 * u) * 64 + lane;
    const int rk = p / KCH, pk = p % KCH;
    koff[u] = (uint32_t)(key_perm8(rk) * D + (pk ^ k_swz<D>(rk)) * 16);
    const int rv = p >> 2, pv = p & 3;
    voff[u] = (uint32_t)(rv * ldv + 16 * (pv ^ vt_swz(rv)));
  }
  // Whole tiles go through buffer resources over the (b, h) slices (K:
  // N*d <= 2^27 bytes; V^T: d*ldv bytes, used while that fits in 2^31), so
  // a tile costs no vector address arithmetic.
  const bool vt_buf = (size_t)D * ldv < ((size_t)1 << 31);
  auto load_tile = [&](int k0, int buf) {
    if (k0 + BC <= kv_valid && k0 + BC <= ldv) {
      if (vt_buf) {
        dma16_rows<SEGS>(Ks(buf), kg, (uint32_t)N * D, (uint32_t)k0 * D,
                         koff);
        dma16_rows<SEGS>(Vs(buf), vtg, (uint32_t)(D * ldv), (uint32_t)k0,
                         voff);
        return;
      }
#pragma unroll
      for (int u = 0; u < SEGS / 4; ++u) {
        const int seg = wave + 4 * u;
        dma16(kg + (size_t)k0 * D + koff[u], Ks(buf) + seg * 1024);
        dma16(vtg + k0 + voff[u], Vs(buf) + seg * 1024);
      }
      return;
    }
    fp8_tail_tile<D>(Ks(buf), Vs(buf), kg, vtg, k0, kv_valid, ldv);
  };

  if (ntiles > 0) load_tile(0, 0);
  wait_dma();
  __syncthreads();
  for (int t = 0, buf = 0; t < ntiles; ++t, buf ^= 1) {
    const int k0 = t * BC;
    if (t + 1 < ntiles) load_tile(k0 + BC, buf ^ 1);
    const uint8_t *Kt = Ks(buf);
    const uint8_t *Vt = Vs(buf);

    if (!(CAUSAL && k0 > qw + 31)) {  // else: above the diagonal
      // S^T = K Q^T; register r of block kb: key k0 + 32*kb + 16*hh + r.
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
        const int row = 32 * kb + ln;
#pragma unroll
        for (int mi = 0; mi < D / 64; ++mi) {
          const int c0 = 4 * mi + 2 * hh;
          const u32x4 lo = *reinterpret_cast<const u32x4 *>(
              Kt + row * D + ((c0 ^ k_swz<D>(row)) << 4));
          const u32x4 hi = *reinterpret_cast<const u32x4 *>(
              Kt + row * D + (((c0 + 1) ^ k_swz<D>(row)) << 4));
          s[kb] = mfma_fp8(cat8(lo, hi), qf[mi], s[kb]);
        }
      }
      const bool tail_keys = k0 + BC > kv_valid;
      const bool diag = CAUSAL && k0 + BC - 1 > qw;
      if (CAUSAL && diag && !tail_keys) {
        // Causal diagonal tile inside kv_valid: register r's key is
        // k0 + 16*hh + 32*kb + r, masked iff that offset exceeds qi - k0 - 16*hh.
        const int thr_k = qi - k0 - 16 * hh;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[kb][r] = 32 * kb + r > thr_k ? -INFINITY : s[kb][r];
      } else if (tail_keys || diag) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kb + 16 * hh + r;
            const bool masked = key >= kv_valid || (CAUSAL && key > qi);
            s[kb][r] = masked ? -INFINITY : s[kb][r];
          }
      }
      // A chain max(max(mx, a), b) per pair: one v_max3_f32 per two scores.
      float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = (kb == 0 ? 2 : 0); r < 16; r += 2)
          mx = fmaxf(fmaxf(mx, s[kb][r]), s[kb][r + 1]);
      mx = max_xor32(mx);
      m_max = fmaxf(m_max, mx);
      if (__any((m_max - m_ref) * c > kRescaleLog2F8)) {
        asm volatile("" ::: "memory");
        const float alpha = fast_exp2((m_ref - m_max) * c);
        m_ref = m_max;
        l_run *= alpha;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
      }
      // p' = 2^6 exp2(c (s - m_ref)), rounded to E4M3 into the P operand:
      // slot 16*kb + r = byte (r % 4) of word 4*kb + r/4.
      const float mc = fmaf(m_ref, c, -kBiasLog2F8);
      i32x8 pf;
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int r = 4 * w;
          const float p0 = fast_exp2(fmaf(s[kb][r], c, -mc));
          const float p1 = fast_exp2(fmaf(s[kb][r + 1], c, -mc));
          const float p2 = fast_exp2(fmaf(s[kb][r + 2], c, -mc));
          const float p3 = fast_exp2(fmaf(s[kb][r + 3], c, -mc));
          lsum += (p0 + p1) + (p2 + p3);
          int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
          word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
          pf[4 * kb + w] = word;
        }
      l_run += lsum;

      // O^T += V^T P^T: lane (dim cb*32 + ln, hh) supplies V^T bytes of keys
      // 32*kb + 16*hh .. +15, i.e. chunk 2*kb + hh of its row.  In a tile
      // that crosses kv_valid the bytes of keys past it are zeroed (finite
      // data for p = 0).
      const bool tail = k0 + BC > kv_valid;
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        const int row = cb * 32 + ln;
        u32x4 ch[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          ch[kb] = *reinterpret_cast<const u32x4 *>(
              Vt + row * 64 + (((2 * kb + hh) ^ vt_swz(row)) << 4));
          if (tail)
            ch[kb] = keep_bytes(ch[kb], kv_valid - (k0 + 32 * kb + 16 * hh));
        }
        oacc[cb] = mfma_fp8(cat8(ch[0], ch[1]), pf, oacc[cb]);
      }
    }

    wait_dma();  // the next tile has landed
    __syncthreads();
  }

  // Epilogue: O = vd * o / l (0 for a row with no visible key); m in natural
  // units, l referred to the true max (the 2^6 bias removed).
  const float l_ref = sum_xor32(l_run);
  if (qi < N) {
    const float inv = l_ref > 0.f ? vd / l_ref : 0.f;
    uint16_t *og = a.o + hoff + (size_t)qi * D;
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
      const float l_true =
          l_ref * fast_exp2((m_ref - m_max) * c - kBiasLog2F8);
      a.m[ri] = l_ref > 0.f ? m_max * sscale : -INFINITY;
      a.l[ri] = l_ref > 0.f ? l_true : 0.f;
    }
  }
}

template <int D, bool CAUSAL>
void fp8_dispatch(const Fp8FwdArgs &a, hipStream_t s) {
  const int nqt = (a.N + 127) / 128;
  dim3 grid((unsigned)(nqt * a.BH)), block(256);
  if (a.kv_len)
    hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, true>), grid, block, 0, s,
                       a);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, false>), grid, block, 0, s,
                       a);
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8FwdArgs &a, int d, bool causal,
                          hipStream_t s) {
  if (d == 64) {
    if (causal) fp8_dispatch<64, true>(a, s);
    else fp8_dispatch<64, false>(a, s);
  } else {
    if (causal) fp8_dispatch<128, true>(a, s);
    else fp8_dispatch<128, false>(a, s);
  }
  return hipGetLastError();
}

}  // namespace fa355
