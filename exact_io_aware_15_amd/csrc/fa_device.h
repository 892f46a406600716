// fa_device.h -- device-side helpers shared by the gfx950 attention kernels.
//
// MFMA fragment conventions used throughout (v_mfma_f32_32x32x16_bf16, one
// 64-lane wavefront computes D[32x32] += A[32x16] * B[16x32]):
//   * A operand: lane l supplies 8 bf16 of row (l % 32); the lane half
//     h = l / 32 and the element index e (0..7) select the k index.  B operand:
//     lane l supplies 8 bf16 of column (l % 32) with the same (h, e) -> k
//     assignment.  Because A and B share that assignment, any consistent
//     placement of the contraction index into (h, e) slots gives the right
//     sum; the kernels choose placements that make LDS reads contiguous.
//   * C/D operand (16 fp32 per lane): lane l holds column (l % 32); register r
//     holds row 8*(r/4) + 4*h + (r%4).
//
// The forward pass computes S^T = K Q^T so that every lane owns one query
// column: the softmax row max / row sum become in-lane reductions plus one
// exchange between the two lane halves, and the output is kept as
// O^T = V^T P^T, whose columns are again queries, so the online-softmax
// rescale (FA notes §3.1; S12 "core idea": alpha = exp(m_old - m_new)) is a
// per-lane scalar multiply.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa355 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Finite stand-in for -inf as the running max's start value: a first tile
// whose scores are all masked (-inf) then gives exp2(-inf - finite) = 0
// instead of exp(-inf - -inf) = NaN (S12, box on the fully masked tile).
constexpr float kMaxInit = -1.0e30f;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}

// Round two fp32 to bf16 (nearest even) and pack them into one dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __builtin_bit_cast(float, (uint32_t)x << 16);
}

// Sum of the two bf16 halves of a packed dword, accumulated in fp32.
__device__ __forceinline__ float dot2_ones(uint32_t packed, float acc) {
  bf16x2 v = __builtin_bit_cast(bf16x2, packed);
  bf16x2 one;
  one[0] = (__bf16)1.0f;
  one[1] = (__bf16)1.0f;
  return __builtin_amdgcn_fdot2_f32_bf16(v, one, acc, false);
}

// Value of lane (l ^ 32): exchange between the two 32-lane halves.
__device__ __forceinline__ float xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

__device__ __forceinline__ u32x4 ldg128(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

// Row order of a 32-row block of an MFMA operand tile held in LDS: storage
// row p holds logical row row_perm(p) (bits 2 and 3 exchanged; the map is its
// own inverse).  With the C-operand row order 8*(r/4)+4h+r%4, a product whose
// A-operand rows are stored this way leaves logical row 16*(r/8)+8*h+(r%8) in
// register r of lane half h: eight consecutive registers hold eight
// consecutive logical rows, i.e. exactly the (h, e) contraction slots of a
// following MFMA that consumes those registers as an operand.
__device__ __forceinline__ int row_perm(int p) {
  return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1);
}

// Transposed MFMA fragment from a row-major bf16 tile in LDS, with the tile's
// rows in row_perm order within each 32-row block.  Returns, for lane l, the
// 8 values T[kbase + 8*h + e][cbase + l%32] (e = 0..7, h = l/32): the operand
// of a product that contracts over the tile's rows (V^T P^T, dS^T Q, ...).
// Uses ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// i%4 of the 8-byte chunk addressed by lane 4*e + i/4, for e = 0..3.  So source
// lane 4*e + j points at row (kbase + 8*h + e [+4]), columns cbase + 16*(g%2)
// + 4*j, where g = l/16.
__device__ __forceinline__ bf16x8 lds_tr_frag(const uint16_t *tile, int pitch,
                                              int kbase, int cbase) {
  typedef short shortx4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, t = lane & 15;
  const int h = g >> 1;
  const int esrc = t >> 2, j = t & 3;
  const int col = cbase + 16 * (g & 1) + 4 * j;
  const int k0 = kbase + 8 * h + esrc;
  const int k1 = k0 + 4;
  const int r0 = (k0 & ~31) | row_perm(k0 & 31);
  const int r1 = (k1 & ~31) | row_perm(k1 & 31);
  const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4 *)(tile + r0 * pitch + col));
  const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4 *)(tile + r1 * pitch + col));
  typedef short shortx8 __attribute__((ext_vector_type(8)));
  const shortx8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace fa355
