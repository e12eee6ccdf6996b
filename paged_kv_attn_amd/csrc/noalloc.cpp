// attn_fwd_paged_noalloc: attn_fwd_paged with the split-KV partials kept in a
// device array that the library owns, for callers that cannot allocate (code
// under HIP graph capture, tight serving loops, harnesses that forbid it).
//
// The array `scratch` is a file-scope __device__ array: every GPU the library
// runs on holds its own copy, at its own address, until the process ends. In
// host code the name `scratch` is only a host-side handle, not a device
// address, so its address is looked up once per device (with that device
// current) through hipGetSymbolAddress and kept in g_scratch[device]; that
// pointer, never the name, is what the kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/attn.h"

namespace attn {
attn_status_t set_error(attn_status_t st, const char* fmt, ...);
}

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;   // 64 MiB per GPU
constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of each device's copy of `scratch`

}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

// Device address of `scratch` on device dev: looked up on the first call for
// that device, with dev current (the caller's current device is restored).
hipError_t scratch_on(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev]) {
    *out = g_scratch[dev];
    return hipSuccess;
  }
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (cur != dev) {
    const hipError_t e2 = hipSetDevice(cur);
    if (e == hipSuccess) e = e2;
  }
  if (e != hipSuccess) return e;
  if (!ptr) return hipErrorInvalidSymbol;
  g_scratch[dev] = ptr;
  *out = ptr;
  return hipSuccess;
}

}  // namespace

extern "C" {

attn_status_t attn_fwd_paged_noalloc(const attn_params_t* p, const void* q, const void* k_pool, const void* v_pool,
                                     void* o, float* lse, const int32_t* block_table, int block_table_stride,
                                     const int32_t* seqlens_k, int B, int sq, int Hq, int Hkv, int d, int page_size,
                                     int num_pages, const int64_t q_stride[3], const int64_t kv_stride[3],
                                     const int64_t o_stride[3], void* stream) {
  // Scratch the split-KV partials of this shape need (0: the prefill path, or
  // a shape that attn_fwd_paged refuses and reports itself). Host arithmetic
  // only: nothing is allocated, here or below.
  size_t need = 0;
  const int64_t max_len = (int64_t)block_table_stride * page_size;
  if (p && B > 0 && sq > 0 && block_table_stride > 0 && page_size > 0 && max_len <= ((int64_t)1 << 30))
    need = attn_workspace_bytes(p, B, Hq, Hkv, sq, d, (int)max_len);
  if (need > kScratchBytes)
    return attn::set_error(ATTN_EWORKSPACE,
                           "attn_fwd_paged_noalloc: this shape needs %zu bytes of split-KV scratch, more than the "
                           "library's %zu-byte array (use attn_fwd_paged with a workspace)",
                           need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
    if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
    if (e == hipSuccess) e = scratch_on(dev, &ws);
    if (e != hipSuccess)
      return attn::set_error(ATTN_ELAUNCH, "attn_fwd_paged_noalloc: cannot locate the scratch array: %s",
                             hipGetErrorString(e));
  }
  return attn_fwd_paged(p, q, k_pool, v_pool, o, lse, block_table, block_table_stride, seqlens_k, B, sq, Hq, Hkv, d,
                        page_size, num_pages, q_stride, kv_stride, o_stride, ws, ws ? kScratchBytes : 0, stream);
}

}  // extern "C"
