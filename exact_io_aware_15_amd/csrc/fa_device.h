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

#include "fa_kernels.h"

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

// Max / sum of x over lanes l and l ^ 32.  v_permlane32_swap(x, x) hands
// each lane the pair {x[l], x[l ^ 32]} (lanes 0-31 get (x[l], x[l+32]),
// lanes 32-63 get (x[l-32], x[l])), so no LDS traffic is involved.
__device__ __forceinline__ float max_xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]),
               __builtin_bit_cast(float, (uint32_t)r[1]));
}

__device__ __forceinline__ float sum_xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) +
         __builtin_bit_cast(float, (uint32_t)r[1]);
}

// x combined with the value of lane l ^ 16 (v_permlane16_swap exchanges the
// odd 16-lane rows of its first operand with the even rows of its second).
__device__ __forceinline__ float max_xor16(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]),
               __builtin_bit_cast(float, (uint32_t)r[1]));
}

__device__ __forceinline__ float sum_xor16(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) +
         __builtin_bit_cast(float, (uint32_t)r[1]);
}

// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] B[32x16].  Lane l supplies
// row (A) / column (B) l % 16 with k = 8*(l/16) + e; D: lane l holds column
// l % 16, register r row 4*(l/16) + r.
__device__ __forceinline__ f32x4 mfma16k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x16_bf16: as above with k = 4*(l/16) + e, e = 0..3 (each
// operand is 4 bf16 packed in two dwords).
__device__ __forceinline__ f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 c) {
  typedef short shortx4 __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
      __builtin_bit_cast(shortx4, a), __builtin_bit_cast(shortx4, b), c, 0, 0,
      0);
}

// The rows of one (batch, head) slice in the [rows, d] operand matrices: n
// rows starting at row0.  Dense [B,H,N,d]: slice bh is rows bh*N ...  Packed
// [H,total,d] (cu non-null): sequence b = bh / H of head h = bh % H starts at
// row h*total + cu[b].  Boundaries are clamped into [0, total] and the
// length to N (the longest sequence), so malformed boundaries cannot make a
// kernel touch rows outside its head.
struct SliceRows {
  int n;
  size_t row0;
};

__device__ __forceinline__ SliceRows slice_rows(const int32_t *cu, int total,
                                                int N, int H, int bh) {
  if (cu == nullptr) return {N, (size_t)bh * N};
  const int b = bh / H, h = bh - b * H;
  const int s = min(max(cu[b], 0), total);
  const int e = min(max(cu[b + 1], s), total);
  return {min(e - s, N), (size_t)h * total + s};
}

// Dispatch order of a causal grid whose blocks are sorted heaviest first.
// Model of the dispatcher this is built for: a launch's blocks go to the 8
// XCDs in turn and, within an XCD, to its 32 CUs in turn, so blocks i,
// i + 256, i + 512, ... become the successive resident workgroups of one CU
// (the speed-ups measured with this order fit the model; results never
// depend on it, since the order is a bijection).  Reversing every odd round
// of 256 blocks (in groups of eight, so each block keeps its XCD and a head
// its L2) pairs the heaviest tiles of one round with the lightest of the next:
// the ROUNDS rounds resident at once then carry about equal work on every
// CU, instead of the CUs that hold the long causal rows finishing last.
// Later rounds keep the heaviest-first order for the dynamic dispatch.  A
// bijection on [0, grid) for any grid size (a partial last round is not
// reversed).
template <int ROUNDS>
__device__ __forceinline__ int causal_deal_order(int i) {
  constexpr int kRound = 256;
  const int r = i / kRound;
  if ((r & 1) && r < ROUNDS && (r + 1) * kRound <= (int)gridDim.x) {
    const int p = i - r * kRound;
    i = r * kRound + (kRound - 8 - (p & ~7)) + (p & 7);
  }
  return i;
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

// LDS operand tiles hold rows of W bf16 with no padding; the 16-byte chunks
// of row r are stored XOR-permuted by lds_swz<W>(r) (r0..r3 = bits of r):
//   W = 64  (8 chunks):  r2 | (r0^r3) << 1 | r1 << 2
//   W = 128 (16 chunks): r2 | r1 << 1 | r0 << 2 | (r1^r3) << 3
// Either way both kinds of operand read are free of bank conflicts whether
// the LDS serves 128 or 256 bytes per cycle: a 16-byte row-fragment read
// (one chunk of 8 or 16 consecutive rows per pass) and an 8-byte transposing
// read (4 consecutive rows x 2 or 4 adjacent chunks per pass, lds_tr_frag).
// Every access computes its slot from the logical (row, column), so the
// permutation is invisible to the arithmetic.
template <int W>
__device__ __forceinline__ int lds_swz(int r) {
  static_assert(W == 64 || W == 128, "tile width");
  if (W == 64)
    return ((r >> 2) & 1) | (((r ^ (r >> 3)) & 1) << 1) | (((r >> 1) & 1) << 2);
  return ((r >> 2) & 1) | (((r >> 1) & 1) << 1) | ((r & 1) << 2) |
         ((((r >> 1) ^ (r >> 3)) & 1) << 3);
}

template <int W>
__device__ __forceinline__ int lds_index(int row, int col) {
  return row * W + (((col >> 3) ^ lds_swz<W>(row)) << 3) + (col & 7);
}

// Transposed MFMA fragment from a swizzled bf16 tile in LDS (row width W),
// whose rows are in row_perm order within each 32-row block.  Returns, for
// lane l, the 8 values T[kbase + 8*h + e][cbase + l%32] (e = 0..7,
// h = l/32): the operand of a product that contracts over the tile's rows
// (V^T P^T, dS^T Q, ...).  Uses ds_read_b64_tr_b16: within each 16-lane
// group, lane i receives element i%4 of the 8-byte chunk addressed by lane
// 4*e + i/4, for e = 0..3.  So source lane 4*e + j points at row
// (kbase + 8*h + e [+4]), columns cbase + 16*(g%2) + 4*j, where g = l/16.
template <int W>
__device__ __forceinline__ bf16x8 lds_tr_frag(const uint16_t *tile, int kbase,
                                              int cbase) {
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
      (__attribute__((address_space(3))) shortx4 *)(tile +
                                                    lds_index<W>(r0, col)));
  const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4 *)(tile +
                                                    lds_index<W>(r1, col)));
  typedef short shortx8 __attribute__((ext_vector_type(8)));
  const shortx8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// LDS byte addresses of the two 8-byte transposing reads (rows k and k + 4)
// that make up lds_tr_frag<W>(tile, kbase, cbase) for the calling lane.
template <int W>
__device__ __forceinline__ void lds_tr_addr(const uint16_t *tile, int kbase,
                                            int cbase, uint32_t &a0,
                                            uint32_t &a1) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, t = lane & 15;
  const int col = cbase + 16 * (g & 1) + 4 * (t & 3);
  const int k0 = kbase + 8 * (g >> 1) + (t >> 2);
  const int k1 = k0 + 4;
  const int r0 = (k0 & ~31) | row_perm(k0 & 31);
  const int r1 = (k1 & ~31) | row_perm(k1 & 31);
  a0 = lds_addr(tile + lds_index<W>(r0, col));
  a1 = lds_addr(tile + lds_index<W>(r1, col));
}

__device__ __forceinline__ bf16x8 tr_pair(u32x2 lo, u32x2 hi) {
  const u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, v);
}

// Two / four transposed fragments (addresses from lds_tr_addr, in the order
// a[2f], a[2f+1] for fragment f), read by one inline-asm statement that also
// waits for them.  Unlike the compiler builtin, whose reads the compiler makes
// wait for every outstanding direct-to-LDS DMA (vmcnt(0)), these leave DMA
// into other buffers in flight.  The wait inside also drains any other LDS or
// scalar-memory operation in flight, which is harmless.
__device__ __forceinline__ void lds_tr_frags(bf16x8 (&f)[2],
                                             const uint32_t (&a)[4]) {
  u32x2 r0, r1, r2, r3;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
  f[0] = tr_pair(r0, r1);
  f[1] = tr_pair(r2, r3);
}

__device__ __forceinline__ void lds_tr_frags(bf16x8 (&f)[4],
                                             const uint32_t (&a)[8]) {
  u32x2 r0, r1, r2, r3, r4, r5, r6, r7;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5),
        "=&v"(r6), "=&v"(r7)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]),
        "v"(a[6]), "v"(a[7])
      : "memory");
  f[0] = tr_pair(r0, r1);
  f[1] = tr_pair(r2, r3);
  f[2] = tr_pair(r4, r5);
  f[3] = tr_pair(r6, r7);
}

// 16-byte row fragment T[row][col .. col+7] from a swizzled tile (col % 8 == 0).
template <int W>
__device__ __forceinline__ bf16x8 lds_row_frag(const uint16_t *tile, int row,
                                               int col) {
  return __builtin_bit_cast(
      bf16x8, *reinterpret_cast<const u32x4 *>(tile + lds_index<W>(row, col)));
}

// Stores a 16-byte chunk of logical row `row` (any row order) at column col.
template <int W>
__device__ __forceinline__ void lds_store_chunk(uint16_t *tile, int row,
                                                int col, u32x4 x) {
  *reinterpret_cast<u32x4 *>(tile + lds_index<W>(row, col)) = x;
}

// Fills an LDS operand tile of ROWS x W bf16 (swizzled, rows in row_perm
// order) from rows row0 .. row0+ROWS-1 of a row-major [*, W] bf16 matrix by
// direct DMA (global_load_lds_dwordx4), issued by four waves.  One wave instruction fills 1 KB of
// LDS with lane i writing bytes 16i..16i+15, so each lane fetches the global
// chunk that belongs at its slot.  Rows past last_row read row last_row
// instead (finite data the caller masks); last_row must be >= 0.  The loads
// complete asynchronously: wait for vmcnt(0) and a barrier before reading.
template <int W, int ROWS>
__device__ __forceinline__ void dma_tile(uint16_t *tile, const uint16_t *src,
                                         int row0, int last_row) {
  constexpr int CPR = W / 8;
  constexpr int SEGS = ROWS * W * 2 / 1024;
  static_assert(SEGS % 4 == 0 && ROWS % 32 == 0, "tile shape");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < SEGS / 4; ++u) {
    const int seg = wave + 4 * u;
    const int p = seg * 64 + lane;          // 16-byte slot in the tile
    const int r = p / CPR, phys = p % CPR;  // storage row, chunk slot
    const int row = min(row0 + ((r & ~31) | row_perm(r & 31)), last_row);
    const size_t goff = (size_t)row * W + (phys ^ lds_swz<W>(r)) * 8;
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void *)(src + goff),
        (__attribute__((address_space(3))) void *)(tile + seg * 512), 16, 0,
        0);
  }
}

// Per-lane byte offsets of dma_tile's sources relative to the tile's first
// row: they depend only on the lane and the segment, so a kernel computes
// them once and every tile that lies wholly inside the valid rows is filled
// by dma_tile_at with a uniform base address (no per-tile address arithmetic).
template <int W, int ROWS>
struct DmaOffsets {
  static constexpr int SEGS = ROWS * W * 2 / 1024;
  uint32_t off[SEGS / 4];
  __device__ __forceinline__ DmaOffsets() {
    constexpr int CPR = W / 8;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int u = 0; u < SEGS / 4; ++u) {
      const int p = (wave + 4 * u) * 64 + lane;
      const int r = p / CPR, phys = p % CPR;
      const int row = (r & ~31) | row_perm(r & 31);
      off[u] = (uint32_t)((row * W + (phys ^ lds_swz<W>(r)) * 8) * 2);
    }
  }
};

// dma_tile for rows row0 .. row0+ROWS-1 all valid, through a raw buffer
// resource over the `bytes` bytes of the matrix slice at `base` (word 3 =
// 32-bit data format, no stride): each load names a byte offset as a per-lane
// register (o) plus a scalar (row0_bytes = row0 * W * 2), so filling a tile
// costs no vector address arithmetic, and an offset past `bytes` would read
// zeros instead of leaving the slice.  The LDS destination of each wave
// instruction is wave-uniform and set up by scalar instructions.
template <int W, int ROWS>
__device__ __forceinline__ void dma_tile_at(uint16_t *tile, const void *base,
                                            uint32_t bytes,
                                            uint32_t row0_bytes,
                                            const DmaOffsets<W, ROWS> &o) {
  // The resource type exists only for the GPU target; the host pass of the
  // compilation (which never runs device code) sees an empty body.
#if defined(__HIP_DEVICE_COMPILE__)
  const auto src = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // The tile offset is the same in every lane; stating so keeps it in a
  // scalar register (a vector one would wrap each load in a waterfall loop).
  const uint32_t soff = __builtin_amdgcn_readfirstlane(row0_bytes);
#pragma unroll
  for (int u = 0; u < DmaOffsets<W, ROWS>::SEGS / 4; ++u) {
    const int seg = wave + 4 * u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        src, (__attribute__((address_space(3))) void *)(tile + seg * 512), 16,
        o.off[u], soff, 0, 0);
  }
#endif
}

// dma_tile kept out of line, for the rare tail tile of a loop whose other
// tiles use dma_tile_at (its address arithmetic then stays out of the loop's
// register budget).
template <int W, int ROWS>
__device__ __attribute__((noinline)) void dma_tile_tail(uint16_t *tile,
                                                        const uint16_t *src,
                                                        int row0,
                                                        int last_row) {
  dma_tile<W, ROWS>(tile, src, row0, last_row);
}

// The same fill for a 64-row key or value tile of a paged cache: logical
// row t of the tile is token t % 16 of cache block blk[t / 16], whose 16 x W
// tile for this KV head starts at base + blk * blk_stride (base already
// points at the head's tile inside block 0).  The block tile is row-major
// (16 rows of W) or, with GROUPED, in 32-element groups (W/32 runs of 16
// tokens x 32 elements: element 32 g + j of token u at (16 g + u) * 32 + j).
// Rows past last_row read row last_row.  blk[] holds valid block indices.
template <int W, bool GROUPED>
__device__ __forceinline__ void dma_tile_paged(uint16_t *tile,
                                               const uint16_t *base,
                                               size_t blk_stride,
                                               const int (&blk)[4], int row0,
                                               int last_row) {
  constexpr int ROWS = 64;
  constexpr int CPR = W / 8;
  constexpr int SEGS = ROWS * W * 2 / 1024;
  static_assert(SEGS % 4 == 0, "tile shape");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < SEGS / 4; ++u) {
    const int seg = wave + 4 * u;
    const int p = seg * 64 + lane;
    const int r = p / CPR, phys = p % CPR;
    const int t = min(row0 + ((r & ~31) | row_perm(r & 31)), last_row) - row0;
    const int bi = t >> 4;
    const int b = bi == 0 ? blk[0] : bi == 1 ? blk[1] : bi == 2 ? blk[2]
                                                                 : blk[3];
    const int c = phys ^ lds_swz<W>(r);
    const size_t goff =
        (size_t)b * blk_stride +
        (GROUPED ? (size_t)(16 * (c >> 2) + (t & 15)) * 32 + (c & 3) * 8
                 : (size_t)(t & 15) * W + c * 8);
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void *)(base + goff),
        (__attribute__((address_space(3))) void *)(tile + seg * 512), 16, 0,
        0);
  }
}

// The same fill for a 64-row paged tile whose rows are all valid, with no
// per-tile vector arithmetic.  One wave instruction fills 64 / (W / 8) storage
// rows (4 at W = 128, 8 at W = 64) of one 16-row group, and row_perm moves
// rows only inside such a group, so every instruction reads a single cache
// block: its base is a scalar (blk_off[] holds the tile's four blocks as
// wave-uniform element offsets, block index x block stride) and each lane's
// byte offset inside the block's 16 x W tile is fixed.  The offsets are
// computed once (PagedDmaOffsets); a tile then costs a scalar address and a
// buffer resource per instruction.
template <int W, bool GROUPED>
struct PagedDmaOffsets {
  static constexpr int SEGS = 64 * W * 2 / 1024;
  static constexpr int ROWS_PER_SEG = 512 / W;
  static_assert(16 % ROWS_PER_SEG == 0, "an instruction spans one block");
  uint32_t off[SEGS / 4];
  __device__ __forceinline__ PagedDmaOffsets() {
    constexpr int CPR = W / 8;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int u = 0; u < SEGS / 4; ++u) {
      const int p = (wave + 4 * u) * 64 + lane;
      const int r = p / CPR, phys = p % CPR;
      const int tok = ((r & ~31) | row_perm(r & 31)) & 15;
      const int c = phys ^ lds_swz<W>(r);
      off[u] = (uint32_t)(GROUPED ? ((16 * (c >> 2) + tok) * 32 + (c & 3) * 8) * 2
                                  : (tok * W + c * 8) * 2);
    }
  }
};

template <int W, bool GROUPED>
__device__ __forceinline__ void dma_tile_paged_at(
    uint16_t *tile, const uint16_t *base, const size_t (&blk_off)[4],
    const PagedDmaOffsets<W, GROUPED> &o) {
#if defined(__HIP_DEVICE_COMPILE__)
  // Segment wave + 4u of a 256-thread workgroup lies in block u (W = 128,
  // 4 rows per segment) or 2u + wave / 2 (W = 64, 8 rows per segment).
  // Constant indices keep blk_off[] in scalar registers.
  constexpr int RPS = PagedDmaOffsets<W, GROUPED>::ROWS_PER_SEG;
  static_assert(RPS == 4 || RPS == 8, "rows per segment");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int u = 0; u < PagedDmaOffsets<W, GROUPED>::SEGS / 4; ++u) {
    const int seg = wave + 4 * u;
    size_t bo;
    if (RPS == 4) {
      bo = blk_off[u];
    } else {
      bo = wave >= 2 ? blk_off[2 * u + 1] : blk_off[2 * u];
    }
    const auto src = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(base + bo), (short)0, 16 * W * 2, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        src, (__attribute__((address_space(3))) void *)(tile + seg * 512), 16,
        o.off[u], 0, 0, 0);
  }
#endif
}

// Walks the allowed 128-wide blocks of one row (or column) of a block mask
// in order.  The wave loads 64 mask bytes at once, one per lane, and keeps
// them as a 64-bit ballot; next(t) is then a scalar bit scan except when a
// 64-block window is crossed.  Block b's byte is at mask[b * stride]; units
// (tiles or steps) of `per` per block, n units in all.  Uniform control flow.
struct MaskWalk {
  const uint8_t *mask;
  int stride, per, n;
  int win0 = -1;
  uint64_t bits = 0;

  __device__ __forceinline__ int next(int t) {
    while (t < n) {
      const int b = t / per, w0 = b & ~63;
      if (w0 != win0) {
        const int bl = w0 + (int)(threadIdx.x & 63);
        const bool ok = bl * per < n && mask[(size_t)bl * stride] != 0;
        bits = __ballot(ok);
        win0 = w0;
      }
      const uint64_t rest = bits >> (b - w0);
      if (rest) {
        const int nb = b + __builtin_ctzll(rest);
        return max(nb * per, t);
      }
      t = (w0 + 64) * per;
    }
    return n;
  }
};

// ---------------------------------------------------------------------------
// Dropout on P.  The pages fuse it into the kernel but give no generator; the
// keep decision of element (query i, key j) of head bh comes from Philox4x32
// with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers:
// As Easy as 1, 2, 3", SC 2011).  One call per (row, 16-key group):
//   counter (i, g, bh, offset), key (seed low word, seed high word),
//   g = 2*(j/32) + (j/8)%2, and j uses byte t = 8*((j/16)%2) + j%8 of the
// 16 output bytes (byte t = bits 8*(t%4).. of word t/4).  The element is kept
// iff that byte >= thr; kept values are scaled by 256/(256 - thr).  In the
// 32x32 score layout where a lane owns one query and, for key block kb, the
// keys 16*(r/8) + 8*hh + r%8 (r = 0..15), register r uses byte r of the
// lane's call for group 2*kb + hh.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1,
                                               uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;  // Weyl key increments
    k1 += 0xBB67AE85u;
  }
  return u32x4{c0, c1, c2, c3};
}

// The 16 random bytes of (row, group) for head bh.
__device__ __forceinline__ u32x4 drop_bytes(const Dropout &dr, int row,
                                            int group, int bh) {
  return philox4x32_10((uint32_t)row, (uint32_t)group, (uint32_t)bh,
                       dr.offset, dr.seed_lo, dr.seed_hi);
}

// Keep decision of byte r (0..15) of a call's output.
__device__ __forceinline__ bool drop_keep(const u32x4 &w, int r,
                                          uint32_t thr) {
  return ((w[r >> 2] >> (8 * (r & 3))) & 0xffu) >= thr;
}

// Transposed keep bits for a lane that owns one KEY of a 32x32 block and, in
// register r, the query 16*(r/8) + 8*hh + r%8 (the key-stationary layout).
// Every lane first draws the call its lane would own in the query-per-lane
// layout (query ln, group half hh: w); the 16 keep bits are then exchanged
// across the wave with ballots.  Ballot t has bit L = keep(query L%32, key
// 16*(t/8) + 8*(L/32) + t%8).  Key kl needs ballot t(kl) = 8*((kl/16)%2) +
// kl%8, word half (kl/8)%2, which each lane selects for itself.  Returns a
// word whose bit 16*(r/8) + r%8 is the keep decision of register r.  Call
// with all 64 lanes active.
__device__ __forceinline__ uint32_t drop_keep_transposed(const u32x4 &w,
                                                         uint32_t thr, int ln,
                                                         int hh) {
  const int my_t = 8 * ((ln >> 4) & 1) + (ln & 7);
  const bool high = (ln >> 3) & 1;
  uint32_t word = 0;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const uint64_t bt = __ballot(drop_keep(w, t, thr));
    const uint32_t half = high ? (uint32_t)(bt >> 32) : (uint32_t)bt;
    word = my_t == t ? half : word;
  }
  return word >> (8 * hh);
}

__device__ __forceinline__ void wait_dma() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace fa355
