// fa_check.hip -- device-side contract checks of the debug build.
//
// Some entry points read small integer arrays whose contents the caller
// guarantees: key-padding lengths, packed-sequence boundaries, and the paged
// cache's sequence lengths and block tables (S12's paged loop maps logical
// block t of a sequence to physical block block_table[t]).  The attention
// kernels clamp malformed values, so nothing is accessed outside the buffers,
// but the results are then meaningless.  The debug build launches these
// checks ahead of a call's kernels, on the same stream; each kind of
// violation becomes a bit of a per-device word that the host reads back.
// A thread gathers its bits in a register and issues at most one atomic OR.
#include "fa355.h"
#include "fa_kernels.h"

namespace fa355 {

// Sticky per-device record of violations (FA_CHECK_* bits).
__device__ uint32_t contract_word;

namespace {

constexpr int kThreads = 256;
constexpr int kMaxGrid = 1024;

int grid_for(long long items) {
  const long long g = (items + kThreads - 1) / kThreads;
  return (int)(g < 1 ? 1 : g > kMaxGrid ? kMaxGrid : g);
}

__device__ void report(uint32_t bits) {
  if (bits) atomicOr(&contract_word, bits);
}

__global__ void __launch_bounds__(kThreads)
    kv_len_kernel(const int32_t *kv_len, int B, int N) {
  uint32_t bad = 0;
  for (int b = blockIdx.x * kThreads + threadIdx.x; b < B;
       b += gridDim.x * kThreads) {
    const int x = kv_len[b];
    if (x < 0 || x > N) bad |= FA_CHECK_KV_LEN;
  }
  report(bad);
}

// Entry i of cu[0..B] is compared with its predecessor (0 for i = 0), so the
// boundaries must start at 0, never decrease, step by at most max_len, and
// end at total.
__global__ void __launch_bounds__(kThreads)
    cu_seqlens_kernel(const int32_t *cu, int B, int total, int max_len) {
  uint32_t bad = 0;
  for (int i = blockIdx.x * kThreads + threadIdx.x; i <= B;
       i += gridDim.x * kThreads) {
    const long long hi = cu[i];
    const long long lo = i == 0 ? 0 : cu[i - 1];
    if (i == 0 && hi != 0) bad |= FA_CHECK_CU_SEQLENS;
    if (hi < lo || hi - lo > max_len) bad |= FA_CHECK_CU_SEQLENS;
    if (i == B && hi != total) bad |= FA_CHECK_CU_SEQLENS;
  }
  report(bad);
}

// One workgroup per sequence (grid-strided): the length against the cache
// capacity and, for a prefill, against the sequence's new-token count; then
// every table entry the kernels read, with the length clamped as they clamp
// it (so t < max_blocks and the row is never overrun).
__global__ void __launch_bounds__(kThreads)
    paged_kernel(const int32_t *seq_lens, const int32_t *cu_q,
                 const int32_t *table, int B, int max_blocks, int block_size,
                 int num_blocks) {
  uint32_t bad = 0;
  const long long cap = (long long)max_blocks * block_size;
  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    const long long len = seq_lens[b];
    if (threadIdx.x == 0) {
      if (len < 0 || len > cap) bad |= FA_CHECK_SEQ_LENS;
      if (cu_q && len < (long long)cu_q[b + 1] - cu_q[b])
        bad |= FA_CHECK_SEQ_LENS;
    }
    const long long used_len = len < 0 ? 0 : len > cap ? cap : len;
    const int used = (int)((used_len + block_size - 1) / block_size);
    const int32_t *row = table + (size_t)b * max_blocks;
    for (int t = threadIdx.x; t < used; t += kThreads) {
      const int e = row[t];
      if (e < 0 || e >= num_blocks) bad |= FA_CHECK_BLOCK_TABLE;
    }
  }
  report(bad);
}

}  // namespace

hipError_t check_kv_len(const int32_t *kv_len, int B, int N, hipStream_t s) {
  hipLaunchKernelGGL(kv_len_kernel, dim3(grid_for(B)), dim3(kThreads), 0, s,
                     kv_len, B, N);
  return hipGetLastError();
}

hipError_t check_cu_seqlens(const int32_t *cu, int B, int total, int max_len,
                            hipStream_t s) {
  hipLaunchKernelGGL(cu_seqlens_kernel, dim3(grid_for((long long)B + 1)),
                     dim3(kThreads), 0, s, cu, B, total, max_len);
  return hipGetLastError();
}

hipError_t check_paged(const int32_t *seq_lens, const int32_t *cu_q,
                       const int32_t *block_table, int B, int max_blocks,
                       int block_size, int num_blocks, hipStream_t s) {
  hipLaunchKernelGGL(paged_kernel, dim3(B < kMaxGrid ? B : kMaxGrid),
                     dim3(kThreads), 0, s, seq_lens, cu_q, block_table, B,
                     max_blocks, block_size, num_blocks);
  return hipGetLastError();
}

hipError_t read_contract_word(uint32_t *word, bool clear) {
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess)
    e = hipMemcpyFromSymbol(word, HIP_SYMBOL(contract_word), sizeof *word);
  if (e == hipSuccess && clear) {
    const uint32_t zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(contract_word), &zero, sizeof zero);
  }
  return e;
}

}  // namespace fa355
