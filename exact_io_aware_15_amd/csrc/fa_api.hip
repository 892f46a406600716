// fa_api.hip -- the C ABI of libfa355 (declared in include/fa355.h):
// argument validation, workspace sizing and dispatch to the gfx950 kernels.
// Validation touches no device memory and calls no HIP function, so an invalid
// call returns its status with no side effect (also on a machine with no GPU).
#include <math.h>

#include <atomic>
#include <mutex>

#include "fa355.h"
#include "fa_kernels.h"

using namespace fa355;

namespace {

constexpr int kMaxN = 1 << 20;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool valid_scale(float s) { return isfinite(s) && s > 0.f; }

// Element counts must fit the kernels' int row indices and size_t offsets.
bool attn_shape_ok(int B, int H, int N) {
  if (B < 1 || H < 1 || N < 1 || N > kMaxN) return false;
  return (long long)B * H * N <= (1LL << 31) - 1;
}

// The HIP error behind the calling thread's most recent FA_E_HIP.
thread_local hipError_t last_hip_error = hipSuccess;

// Packed variable-length problems: B sequences of at most max_seqlen tokens
// in [H, total, d] matrices.  The grids span ceil(max_seqlen / 64) tiles per
// (sequence, head).
bool varlen_shape_ok(int B, int H, int total, int max_seqlen) {
  if (B < 1 || H < 1 || total < 0 || max_seqlen < 1 || max_seqlen > kMaxN)
    return false;
  if ((long long)H * total > (1LL << 31) - 1) return false;
  return (long long)((max_seqlen + 63) / 64) * B * H <= (1LL << 31) - 1;
}

int from_hip(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  last_hip_error = e;
  return FA_E_HIP;
}

// Dropout parameters: thr = floor(256 p + 1/2), exact in double (256 p is
// exact for a float p); valid for p >= 0 with thr <= 255.
bool drop_setup(float p, uint64_t seed, uint32_t offset, Dropout &dr) {
  if (!(p >= 0.f)) return false;  // also rejects NaN
  const double t = floor((double)p * 256.0 + 0.5);
  if (t > 255.0) return false;
  dr.thr = (uint32_t)t;
  dr.keep_scale = (float)(256.0 / (256.0 - t));
  dr.seed_lo = (uint32_t)seed;
  dr.seed_hi = (uint32_t)(seed >> 32);
  dr.offset = offset;
  return true;
}

// The debug build (FA355_DEBUG defined) puts the contract checks of
// fa_check.hip on the stream ahead of each call's kernels.
#ifdef FA355_DEBUG
constexpr bool kChecks = true;
#else
constexpr bool kChecks = false;
#endif

int fwd_dense(int dtype, int B, int H, int N, int d, const void *q,
              const void *k, const void *v, void *o, float *m, float *l,
              const int32_t *kv_len, int causal, float scale,
              const Dropout &dr, void *stream) {
  FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.m = m; a.l = l; a.kv_len = kv_len;
  a.cu_seqlens = nullptr; a.total = 0;
  a.drop = dr;
  a.B = B; a.H = H; a.N = N; a.BH = B * H;
  a.scale = scale;
  a.c = (float)((double)scale * 1.4426950408889634);
  hipStream_t s = (hipStream_t)stream;
  if (kChecks && kv_len)
    if (hipError_t e = check_kv_len(kv_len, B, N, s)) return from_hip(e);
  if (dtype == FA_BF16) return from_hip(launch_fwd_bf16(a, d, causal != 0, s));
  return from_hip(launch_fwd_f32(a, d, causal != 0, s));
}

int bwd_dense(int B, int H, int N, int d, const void *q, const void *k,
              const void *v, const void *o, const void *dout, const float *m,
              const float *l, const int32_t *kv_len, int causal, float scale,
              const Dropout &dr, void *dq, void *dk, void *dv,
              void *workspace, void *stream) {
  const size_t rows = (size_t)B * H * N;
  BwdArgs a{};
  a.q = (const uint16_t *)q; a.k = (const uint16_t *)k;
  a.v = (const uint16_t *)v; a.o = (const uint16_t *)o;
  a.dout = (const uint16_t *)dout; a.m = m; a.l = l; a.kv_len = kv_len;
  a.cu_seqlens = nullptr; a.total = 0; a.rows = (long long)rows;
  a.drop = dr;
  a.dq = (uint16_t *)dq; a.dk = (uint16_t *)dk; a.dv = (uint16_t *)dv;
  char *ws = (char *)workspace;
  a.lse2 = (float *)ws;
  a.delta = (float *)(ws + align_up(rows * sizeof(float)));
  a.B = B; a.H = H; a.N = N; a.BH = B * H;
  a.scale = scale;
  a.c = (float)((double)scale * 1.4426950408889634);
  hipStream_t s = (hipStream_t)stream;
  if (kChecks && kv_len)
    if (hipError_t e = check_kv_len(kv_len, B, N, s)) return from_hip(e);
  return from_hip(launch_bwd(a, d, causal != 0, s));
}

size_t fa_decode_workspace_bytes_impl(int B, int Hq, int d, int num_splits) {
  if (B < 1 || Hq < 1 || (d != 64 && d != 128) || num_splits < 1 ||
      num_splits > 64)
    return 0;
  const size_t parts = (size_t)B * Hq * num_splits;
  return 2 * align_up(parts * sizeof(float)) +
         align_up(parts * d * sizeof(float));
}

// Arguments of a paged decode, checked without touching the device.
int decode_validate(int B, int Hq, int Hkv, int d, const void *q,
                    const void *k_cache, const void *v_cache, int num_blocks,
                    int block_size, const int32_t *block_table,
                    int max_blocks_per_seq, const int32_t *seq_lens,
                    int num_splits, float scale, const void *out) {
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out)
    return FA_E_NULLPTR;
  if (B < 1 || Hq < 1 || Hkv < 1 || num_blocks < 1 ||
      max_blocks_per_seq < 1 || num_splits < 1 || num_splits > 64 ||
      !valid_scale(scale))
    return FA_E_SHAPE;
  if (Hq % Hkv != 0) return FA_E_SHAPE;
  if (Hq / Hkv > 16) return FA_E_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_E_UNSUPPORTED;
  if (block_size != 16) return FA_E_UNSUPPORTED;
  if ((long long)B * max_blocks_per_seq > (1LL << 31) - 1 ||
      (long long)max_blocks_per_seq * 16 > (1LL << 31) - 1 ||
      (long long)B * num_splits * Hq > (1LL << 31) - 1 ||
      (long long)num_blocks * block_size * Hkv * d > (1LL << 40))
    return FA_E_SHAPE;
  return FA_OK;
}

// Compute units of the current device, queried once per device.
hipError_t compute_units(int *n) {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev >= 0 && dev < 64 && (*n = cached[dev].load()) > 0) return hipSuccess;
  if (hipError_t e = hipDeviceGetAttribute(
          n, hipDeviceAttributeMultiprocessorCount, dev))
    return e;
  if (*n < 1) *n = 1;
  if (dev >= 0 && dev < 64) cached[dev].store(*n);
  return hipSuccess;
}

// Enqueues a validated decode whose partial triples live at ws (laid out as
// fa_decode_workspace_bytes counts them).
int decode_launch(int B, int Hq, int Hkv, int d, const void *q,
                  const void *k_cache, const void *v_cache, int num_blocks,
                  int block_size, const int32_t *block_table,
                  int max_blocks_per_seq, const int32_t *seq_lens,
                  int num_splits, float scale, void *out, char *ws,
                  void *stream) {
  const size_t parts = (size_t)B * Hq * num_splits;
  DecodeArgs a{};
  a.q = (const uint16_t *)q;
  a.k_cache = (const uint16_t *)k_cache;
  a.v_cache = (const uint16_t *)v_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out = (uint16_t *)out;
  a.part_m = (float *)ws;
  a.part_l = (float *)(ws + align_up(parts * sizeof(float)));
  a.part_o = (float *)(ws + 2 * align_up(parts * sizeof(float)));
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.num_splits = num_splits;
  if (hipError_t e = compute_units(&a.deal)) return from_hip(e);
  a.scale = scale;
  a.c = (float)((double)scale * 1.4426950408889634);
  hipStream_t s = (hipStream_t)stream;
  if (kChecks)
    if (hipError_t e = check_paged(seq_lens, nullptr, block_table, B,
                                   max_blocks_per_seq, block_size, num_blocks,
                                   s))
      return from_hip(e);
  return from_hip(launch_decode(a, d, s));
}

// Fixed scratch of fa_decode_paged_noalloc: one array per GPU, held until the
// process ends.  In host code `scratch` names a host-side stand-in, never
// the device memory: the device address of each GPU's copy comes from
// hipGetSymbolAddress, called once per device with that device current, and
// only that address is handed to kernels.  The split kernel writes every
// partial triple of a call before the merge kernel reads it, so nothing in
// the array has to start at zero.
constexpr size_t kScratchBytes = FA_DECODE_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
char *scratch_dev[kMaxDevices];  // device address per device, once known

int scratch_on_current_device(char **ptr) {
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev)) return from_hip(e);
  if (dev < 0 || dev >= kMaxDevices) return FA_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_dev[dev] == nullptr) {
    void *p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)))
      return from_hip(e);
    scratch_dev[dev] = (char *)p;
  }
  *ptr = scratch_dev[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

const char *fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_E_NULLPTR: return "FA_E_NULLPTR: a required pointer is NULL";
    case FA_E_SHAPE: return "FA_E_SHAPE: size out of range or inconsistent";
    case FA_E_UNSUPPORTED: return "FA_E_UNSUPPORTED: not implemented by the library";
    case FA_E_WORKSPACE: return "FA_E_WORKSPACE: workspace missing or too small";
    case FA_E_HIP: return "FA_E_HIP: HIP runtime error at launch";
    case FA_E_SCRATCH:
      return "FA_E_SCRATCH: request larger than the library's fixed scratch";
    default: return "unknown fa_status";
  }
}

int fa_last_hip_error(void) { return (int)last_hip_error; }

const char *fa_last_hip_error_str(void) {
  return hipGetErrorString(last_hip_error);
}

int fa_fwd(int dtype, int B, int H, int N, int d, const void *q,
           const void *k, const void *v, void *o, float *m, float *l,
           const int32_t *kv_len, int causal, float scale, void *stream) {
  if (!q || !k || !v || !o) return FA_E_NULLPTR;
  if ((m == nullptr) != (l == nullptr)) return FA_E_NULLPTR;
  if (!attn_shape_ok(B, H, N) || !valid_scale(scale)) return FA_E_SHAPE;
  if (d != 64 && d != 128) return FA_E_UNSUPPORTED;
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_E_UNSUPPORTED;
  return fwd_dense(dtype, B, H, N, d, q, k, v, o, m, l, kv_len, causal, scale,
                   Dropout{}, stream);
}

int fa_fwd_dropout(int B, int H, int N, int d, const void *q, const void *k,
                   const void *v, void *o, float *m, float *l,
                   const int32_t *kv_len, int causal, float scale,
                   float p_drop, uint64_t seed, uint32_t offset,
                   void *stream) {
  if (!q || !k || !v || !o) return FA_E_NULLPTR;
  if ((m == nullptr) != (l == nullptr)) return FA_E_NULLPTR;
  Dropout dr{};
  if (!attn_shape_ok(B, H, N) || !valid_scale(scale) ||
      !drop_setup(p_drop, seed, offset, dr))
    return FA_E_SHAPE;
  if (d != 64 && d != 128) return FA_E_UNSUPPORTED;
  return fwd_dense(FA_BF16, B, H, N, d, q, k, v, o, m, l, kv_len, causal,
                   scale, dr, stream);
}

int fa_fwd_fp8(int B, int H, int N, int d, const void *q, const void *k,
               const void *v_t, int ldv, const float *q_descale,
               const float *k_descale, const float *v_descale, void *o,
               float *m, float *l, const int32_t *kv_len, int causal,
               float scale, void *stream) {
  if (!q || !k || !v_t || !o) return FA_E_NULLPTR;
  if ((m == nullptr) != (l == nullptr)) return FA_E_NULLPTR;
  if (!attn_shape_ok(B, H, N) || !valid_scale(scale)) return FA_E_SHAPE;
  if (ldv < N || ldv % 16 != 0) return FA_E_SHAPE;
  if ((long long)B * H * ldv > (1LL << 40)) return FA_E_SHAPE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v_t) % 16) return FA_E_SHAPE;
  if (d != 64 && d != 128) return FA_E_UNSUPPORTED;
  Fp8FwdArgs a{};
  a.q = (const uint8_t *)q; a.k = (const uint8_t *)k;
  a.vt = (const uint8_t *)v_t; a.ldv = ldv;
  a.q_descale = q_descale; a.k_descale = k_descale; a.v_descale = v_descale;
  a.o = (uint16_t *)o; a.m = m; a.l = l; a.kv_len = kv_len;
  a.B = B; a.H = H; a.N = N; a.BH = B * H;
  a.scale = scale;
  hipStream_t s = (hipStream_t)stream;
  if (kChecks && kv_len)
    if (hipError_t e = check_kv_len(kv_len, B, N, s)) return from_hip(e);
  return from_hip(launch_fwd_fp8(a, d, causal != 0, s));
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (!attn_shape_ok(B, H, N) || (d != 64 && d != 128)) return 0;
  const size_t rows = (size_t)B * H * N;
  return 2 * align_up(rows * sizeof(float));
}

// The dense workspace, then the block-sparse items' work and order, each
// [2][H * nb] int32.
size_t fa_bwd_block_sparse_workspace_bytes(int B, int H, int N, int d) {
  const size_t dense = fa_bwd_workspace_bytes(B, H, N, d);
  if (!dense) return 0;
  const size_t items = (size_t)H * ((N + 127) / 128);
  return dense + 2 * align_up(2 * items * sizeof(int32_t));
}

int fa_bwd(int B, int H, int N, int d, const void *q, const void *k,
           const void *v, const void *o, const void *dout, const float *m,
           const float *l, const int32_t *kv_len, int causal, float scale,
           void *dq, void *dk, void *dv, void *workspace,
           size_t workspace_bytes, void *stream) {
  if (!q || !k || !v || !o || !dout || !m || !l || !dq || !dk || !dv)
    return FA_E_NULLPTR;
  if (!attn_shape_ok(B, H, N) || !valid_scale(scale)) return FA_E_SHAPE;
  if (d != 64 && d != 128) return FA_E_UNSUPPORTED;
  const size_t need = fa_bwd_workspace_bytes(B, H, N, d);
  if (!workspace || workspace_bytes < need) return FA_E_WORKSPACE;
  if (((uintptr_t)workspace) % kAlign) return FA_E_WORKSPACE;
  return bwd_dense(B, H, N, d, q, k, v, o, dout, m, l, kv_len, causal, scale,
                   Dropout{}, dq, dk, dv, workspace, stream);
}

int fa_bwd_dropout(int B, int H, int N, int d, const void *q, const void *k,
                   const void *v, const void *o, const void *dout,
                   const float *m, const float *l, const int32_t *kv_len,
                   int causal, float scale, float p_drop, uint64_t seed,
                   uint32_t offset, void *dq, void *dk, void *dv,
                   void *workspace, size_t workspace_bytes, void *stream) {
  if (!q || !k || !v || !o || !dout || !m || !l || !dq || !dk || !dv)
    return FA_E_NULLPTR;
  Dropout dr{};
  if (!attn_shape_ok(B, H, N) || !valid_scale(scale) ||
      !drop_setup(p_drop, seed, offset, dr))
    return FA_E_SHAPE;
  if (d != 64 && d != 128) return FA_E_UNSUPPORTED;
  const size_t need = fa_bwd_workspace_bytes(B, H, N, d);
  if (!workspace || workspace_bytes < need) return FA_E_WORKSPACE;
  if (((uintptr_t)workspace) % kAlign) return FA_E_WORKSPACE;
  return bwd_dense(B, H, N, d, q, k, v, o, dout, m, l, kv_len, causal, scale,
                   dr, dq, dk, dv, workspace, stream);
}

int fa_fwd_block_sparse(int B, int H, int N, int d, const void *q,
                        const void *k, const void *v, void *o, float *m,
                        float *l, const uint8_t *block_mask, int causal,
                        float scale, void *stream) {
  if (!q || !k || !v || !o || !block_mask) return FA_E_NULLPTR;
  if ((m == nullptr) != (l == nullptr)) return FA_E_NULLPTR;
  if (!attn_shape_ok(B, H, N) || !valid_scale(scale)) return FA_E_SHAPE;
  if (d != 64 && d != 128) return FA_E_UNSUPPORTED;
  FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.m = m; a.l = l;
  a.block_mask = block_mask;
  a.B = B; a.H = H; a.N = N; a.BH = B * H;
  a.scale = scale;
  a.c = (float)((double)scale * 1.4426950408889634);
  return from_hip(launch_fwd_block_sparse(a, d, causal != 0,
                                          (hipStream_t)stream));
}

int fa_bwd_block_sparse(int B, int H, int N, int d, const void *q,
                        const void *k, const void *v, const void *o,
                        const void *dout, const float *m, const float *l,
                        const uint8_t *block_mask, int causal, float scale,
                        void *dq, void *dk, void *dv, void *workspace,
                        size_t workspace_bytes, void *stream) {
  if (!q || !k || !v || !o || !dout || !m || !l || !dq || !dk || !dv ||
      !block_mask)
    return FA_E_NULLPTR;
  if (!attn_shape_ok(B, H, N) || !valid_scale(scale)) return FA_E_SHAPE;
  if (d != 64 && d != 128) return FA_E_UNSUPPORTED;
  const size_t need = fa_bwd_block_sparse_workspace_bytes(B, H, N, d);
  if (!workspace || workspace_bytes < need) return FA_E_WORKSPACE;
  if (((uintptr_t)workspace) % kAlign) return FA_E_WORKSPACE;
  const size_t rows = (size_t)B * H * N;
  const size_t items = (size_t)H * ((N + 127) / 128);
  BwdArgs a{};
  a.q = (const uint16_t *)q; a.k = (const uint16_t *)k;
  a.v = (const uint16_t *)v; a.o = (const uint16_t *)o;
  a.dout = (const uint16_t *)dout; a.m = m; a.l = l;
  a.block_mask = block_mask; a.rows = (long long)rows;
  a.dq = (uint16_t *)dq; a.dk = (uint16_t *)dk; a.dv = (uint16_t *)dv;
  char *ws = (char *)workspace;
  a.lse2 = (float *)ws;
  a.delta = (float *)(ws + align_up(rows * sizeof(float)));
  char *sp = ws + 2 * align_up(rows * sizeof(float));
  a.sp_work = (int32_t *)sp;
  a.sp_order = (int32_t *)(sp + align_up(2 * items * sizeof(int32_t)));
  a.sp_causal = causal != 0;
  a.B = B; a.H = H; a.N = N; a.BH = B * H;
  a.scale = scale;
  a.c = (float)((double)scale * 1.4426950408889634);
  return from_hip(launch_bwd(a, d, causal != 0, (hipStream_t)stream));
}

int fa_fwd_varlen(int dtype, int B, int H, int total, int max_seqlen, int d,
                  const int32_t *cu_seqlens, const void *q, const void *k,
                  const void *v, void *o, float *m, float *l, int causal,
                  float scale, void *stream) {
  if (!varlen_shape_ok(B, H, total, max_seqlen) || !valid_scale(scale))
    return FA_E_SHAPE;
  if (d != 64 && d != 128) return FA_E_UNSUPPORTED;
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_E_UNSUPPORTED;
  if (total == 0) return FA_OK;  // no rows (empty buffers may be NULL)
  if (!cu_seqlens || !q || !k || !v || !o) return FA_E_NULLPTR;
  if ((m == nullptr) != (l == nullptr)) return FA_E_NULLPTR;
  FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.m = m; a.l = l; a.kv_len = nullptr;
  a.cu_seqlens = cu_seqlens; a.total = total;
  a.B = B; a.H = H; a.N = max_seqlen; a.BH = B * H;
  a.scale = scale;
  a.c = (float)((double)scale * 1.4426950408889634);
  hipStream_t s = (hipStream_t)stream;
  if (kChecks)
    if (hipError_t e = check_cu_seqlens(cu_seqlens, B, total, max_seqlen, s))
      return from_hip(e);
  if (dtype == FA_BF16) return from_hip(launch_fwd_bf16(a, d, causal != 0, s));
  return from_hip(launch_fwd_f32(a, d, causal != 0, s));
}

size_t fa_bwd_varlen_workspace_bytes(int H, int total, int d) {
  if (H < 1 || total < 0 || (long long)H * total > (1LL << 31) - 1 ||
      (d != 64 && d != 128))
    return 0;
  return 2 * align_up((size_t)H * total * sizeof(float));
}

int fa_bwd_varlen(int B, int H, int total, int max_seqlen, int d,
                  const int32_t *cu_seqlens, const void *q, const void *k,
                  const void *v, const void *o, const void *dout,
                  const float *m, const float *l, int causal, float scale,
                  void *dq, void *dk, void *dv, void *workspace,
                  size_t workspace_bytes, void *stream) {
  if (!varlen_shape_ok(B, H, total, max_seqlen) || !valid_scale(scale))
    return FA_E_SHAPE;
  if (d != 64 && d != 128) return FA_E_UNSUPPORTED;
  if (total == 0) return FA_OK;  // no rows (empty buffers may be NULL)
  if (!cu_seqlens || !q || !k || !v || !o || !dout || !m || !l || !dq ||
      !dk || !dv)
    return FA_E_NULLPTR;
  const size_t need = fa_bwd_varlen_workspace_bytes(H, total, d);
  if (!workspace || workspace_bytes < need) return FA_E_WORKSPACE;
  if (((uintptr_t)workspace) % kAlign) return FA_E_WORKSPACE;
  const size_t rows = (size_t)H * total;
  BwdArgs a{};
  a.q = (const uint16_t *)q; a.k = (const uint16_t *)k;
  a.v = (const uint16_t *)v; a.o = (const uint16_t *)o;
  a.dout = (const uint16_t *)dout; a.m = m; a.l = l; a.kv_len = nullptr;
  a.cu_seqlens = cu_seqlens; a.total = total; a.rows = (long long)rows;
  a.dq = (uint16_t *)dq; a.dk = (uint16_t *)dk; a.dv = (uint16_t *)dv;
  char *ws = (char *)workspace;
  a.lse2 = (float *)ws;
  a.delta = (float *)(ws + align_up(rows * sizeof(float)));
  a.B = B; a.H = H; a.N = max_seqlen; a.BH = B * H;
  a.scale = scale;
  a.c = (float)((double)scale * 1.4426950408889634);
  hipStream_t s = (hipStream_t)stream;
  if (kChecks)
    if (hipError_t e = check_cu_seqlens(cu_seqlens, B, total, max_seqlen, s))
      return from_hip(e);
  return from_hip(launch_bwd(a, d, causal != 0, s));
}

int fa_prefill_paged(int B, int Hq, int Hkv, int d, int total_q, int max_q,
                     const int32_t *cu_seqlens_q, const void *q,
                     const void *k_cache, const void *v_cache, int num_blocks,
                     int block_size, const int32_t *block_table,
                     int max_blocks_per_seq, const int32_t *seq_lens,
                     int causal, float scale, void *o, float *m, float *l,
                     void *stream) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || num_blocks < 1 ||
      max_blocks_per_seq < 1 || !valid_scale(scale))
    return FA_E_SHAPE;
  if (!varlen_shape_ok(B, Hq, total_q, max_q)) return FA_E_SHAPE;
  if ((long long)B * max_blocks_per_seq > (1LL << 31) - 1 ||
      (long long)max_blocks_per_seq * 16 > (1LL << 31) - 1 ||
      (long long)num_blocks * block_size * Hkv * d > (1LL << 40))
    return FA_E_SHAPE;
  if (d != 64 && d != 128) return FA_E_UNSUPPORTED;
  if (block_size != 16) return FA_E_UNSUPPORTED;
  if (total_q == 0) return FA_OK;  // no new tokens (empty buffers may be NULL)
  if (!cu_seqlens_q || !q || !k_cache || !v_cache || !block_table ||
      !seq_lens || !o)
    return FA_E_NULLPTR;
  if ((m == nullptr) != (l == nullptr)) return FA_E_NULLPTR;
  FwdArgs a{};
  a.q = q; a.k = nullptr; a.v = nullptr; a.o = o; a.m = m; a.l = l;
  a.kv_len = nullptr;
  a.cu_seqlens = cu_seqlens_q; a.total = total_q;
  a.k_cache = k_cache; a.v_cache = v_cache;
  a.block_table = block_table; a.seq_lens = seq_lens;
  a.max_blocks = max_blocks_per_seq; a.num_blocks = num_blocks; a.Hkv = Hkv;
  a.B = B; a.H = Hq; a.N = max_q; a.BH = B * Hq;
  a.scale = scale;
  a.c = (float)((double)scale * 1.4426950408889634);
  hipStream_t s = (hipStream_t)stream;
  if (kChecks) {
    if (hipError_t e = check_cu_seqlens(cu_seqlens_q, B, total_q, max_q, s))
      return from_hip(e);
    if (hipError_t e = check_paged(seq_lens, cu_seqlens_q, block_table, B,
                                   max_blocks_per_seq, block_size, num_blocks,
                                   s))
      return from_hip(e);
  }
  return from_hip(launch_prefill_paged(a, d, causal != 0, s));
}

size_t fa_decode_workspace_bytes(int B, int Hq, int d, int num_splits) {
  return fa_decode_workspace_bytes_impl(B, Hq, d, num_splits);
}

int fa_decode_paged(int B, int Hq, int Hkv, int d, const void *q,
                    const void *k_cache, const void *v_cache, int num_blocks,
                    int block_size, const int32_t *block_table,
                    int max_blocks_per_seq, const int32_t *seq_lens,
                    int num_splits, float scale, void *out, void *workspace,
                    size_t workspace_bytes, void *stream) {
  if (int st = decode_validate(B, Hq, Hkv, d, q, k_cache, v_cache, num_blocks,
                               block_size, block_table, max_blocks_per_seq,
                               seq_lens, num_splits, scale, out))
    return st;
  const size_t need = fa_decode_workspace_bytes(B, Hq, d, num_splits);
  if (!workspace || workspace_bytes < need) return FA_E_WORKSPACE;
  if (((uintptr_t)workspace) % kAlign) return FA_E_WORKSPACE;
  return decode_launch(B, Hq, Hkv, d, q, k_cache, v_cache, num_blocks,
                       block_size, block_table, max_blocks_per_seq, seq_lens,
                       num_splits, scale, out, (char *)workspace, stream);
}

int fa_decode_paged_noalloc(int B, int Hq, int Hkv, int d, const void *q,
                            const void *k_cache, const void *v_cache,
                            int num_blocks, int block_size,
                            const int32_t *block_table,
                            int max_blocks_per_seq, const int32_t *seq_lens,
                            int num_splits, float scale, void *out,
                            void *stream) {
  if (int st = decode_validate(B, Hq, Hkv, d, q, k_cache, v_cache, num_blocks,
                               block_size, block_table, max_blocks_per_seq,
                               seq_lens, num_splits, scale, out))
    return st;
  if (fa_decode_workspace_bytes(B, Hq, d, num_splits) > kScratchBytes)
    return FA_E_SCRATCH;
  char *ws = nullptr;
  if (int st = scratch_on_current_device(&ws)) return st;
  return decode_launch(B, Hq, Hkv, d, q, k_cache, v_cache, num_blocks,
                       block_size, block_table, max_blocks_per_seq, seq_lens,
                       num_splits, scale, out, ws, stream);
}

int fa_debug_flags(uint32_t *flags, int clear) {
  if (!kChecks) return FA_E_UNSUPPORTED;
  if (!flags) return FA_E_NULLPTR;
  return from_hip(read_contract_word(flags, clear != 0));
}

}  // extern "C"
