// C ABI of libattn: argument validation, path selection and launch set-up.
//
// Every check runs on the host before any launch, so a rejected call touches
// no device state. Errors follow the convention of the FlashAttention-2 mma
// page's torch entry point (unsupported head dims / dtypes are refused up
// front) and of the Composable Kernel page's MakeKargs (strides, head ratio,
// page-block size are arguments, not assumptions).
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <cmath>
#include <vector>

#include "../../include/attn.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

bool log_on();

// Records the failure for attn_last_error(); under ATTN_LOG also one stderr line.
attn_status_t fail(attn_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  if (log_on()) fprintf(stderr, "attn: error %d: %s\n", (int)st, g_err);
  return st;
}

int elem_bytes(int t) { return t == ATTN_F32 ? 4 : (t == ATTN_BF16 ? 2 : 1); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Decode-path choice: the packed query block (positions x q-heads of one
// kv-head) fits the 16 columns of one MFMA tile.
bool takes_decode_path(int in_dtype, int sq, int ratio) {
  return in_dtype != ATTN_F32 && (int64_t)sq * ratio <= 16;
}

// Keys per split-KV work unit (one wave each): unless the caller fixes it, the
// largest power of two in [256, 2048] that still gives the (request, kv-head,
// split) grid at least 4096 units, about three waves for each resident slot of
// the chip. Long units stream longer; the kv-heads of one split run side by side.
int plan_split_tokens(const attn_params_t* p, int B, int Hkv, int max_len) {
  if (p->kv_split_tokens > 0) return p->kv_split_tokens;
  const int64_t units = (int64_t)B * Hkv;
  // fp8 keys carry half the bytes, and the fp8 variant fits 10 waves per CU
  // (bf16: 5), so it wants more units in flight: 1024-key splits measured
  // 415 us against 434 us for 2048 on 64 requests of 1K-32K keys (bf16: 2048
  // is fastest, 731 us against 748 us for 1024)
  int c = p->in_dtype == ATTN_FP8_E4M3 ? 1024 : 2048;
  while (c > 256 && units * ((max_len + c - 1) / c) < 4096) c /= 2;
  return c;
}

int n_splits_for(int split, int max_len) { return max_len > 0 ? (max_len + split - 1) / split : 1; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// factor applied to the normalised O before it is stored: the value descale of
// fp8 inputs, times o_scale for fp8 output
float out_mul(const attn_params_t* p) {
  return (p->in_dtype == ATTN_FP8_E4M3 ? p->v_descale : 1.0f) * (p->out_dtype == ATTN_FP8_E4M3 ? p->o_scale : 1.0f);
}

// Bias in the kernels' logit units: the kernels compare and exponentiate
// x * c_exp2 in base 2, so a natural-log bias b enters as b * log2(e) / c_exp2.
void set_bias(const attn_params_t* p, float c_exp2, attn::PrefillArgs* a) {
  a->bias_type = p->bias_type;
  a->bias = p->bias;
  a->bias_sb = p->bias_stride[0]; a->bias_sh = p->bias_stride[1]; a->bias_sr = p->bias_stride[2];
  a->bias_mul = 1.4426950408889634f / c_exp2;
}
void set_bias(const attn_params_t* p, float c_exp2, attn::DecodeArgs* a) {
  a->alibi = p->bias_type == ATTN_BIAS_ALIBI ? p->bias : nullptr;
  a->alibi_sb = p->bias_stride[0];
  a->bias = p->bias_type == ATTN_BIAS_ELEMENTWISE ? p->bias : nullptr;
  a->bias_sb = p->bias_stride[0]; a->bias_sh = p->bias_stride[1]; a->bias_sr = p->bias_stride[2];
  a->bias_mul = 1.4426950408889634f / c_exp2;
}

// the V pool's strides: its own when any is set, else the K pool's
const int64_t* v_pool_strides(const attn_params_t* p, const int64_t* kv_stride) {
  const bool own = p->v_pool_stride[0] || p->v_pool_stride[1] || p->v_pool_stride[2];
  return own ? p->v_pool_stride : kv_stride;
}

size_t decode_ws_bytes(int B, int Hkv, int n_splits, int m_rows, int d) {
  const size_t units = (size_t)B * Hkv * n_splits * m_rows;
  return align256(units * d * sizeof(float)) + align256(units * sizeof(float));
}

attn_status_t check_params(const attn_params_t* p, int d) {
  if (!p) return fail(ATTN_EINVAL, "params is NULL");
  const bool pair_ok = (p->in_dtype == ATTN_F32 && p->out_dtype == ATTN_F32) ||
                       ((p->in_dtype == ATTN_BF16 || p->in_dtype == ATTN_FP8_E4M3) &&
                        (p->out_dtype == ATTN_BF16 || p->out_dtype == ATTN_FP8_E4M3));
  if (!pair_ok) return fail(ATTN_ENOTSUP, "unsupported (in_dtype, out_dtype) = (%d, %d)", p->in_dtype, p->out_dtype);
  if (d != 64 && d != 128) return fail(ATTN_ENOTSUP, "head dim %d not supported (64 or 128)", d);
  if (!(p->scale > 0.0f) || !std::isfinite(p->scale)) return fail(ATTN_EINVAL, "scale must be finite and > 0");
  if (!std::isfinite(p->softcap)) return fail(ATTN_EINVAL, "softcap must be finite");
  if (p->window_left < -1 || p->window_right < -1) return fail(ATTN_EINVAL, "window bounds must be >= -1");
  if (p->in_dtype == ATTN_FP8_E4M3) {
    const float ds[3] = {p->q_descale, p->k_descale, p->v_descale};
    for (float x : ds)
      if (!(x > 0.0f) || !std::isfinite(x)) return fail(ATTN_EINVAL, "fp8 descales must be finite and > 0");
  }
  if (p->kv_split_tokens < 0 || p->kv_split_tokens % 64 != 0 || p->kv_split_tokens > 2048)
    return fail(ATTN_EINVAL, "kv_split_tokens must be 0 or a multiple of 64 in [64, 2048]");
  if (p->out_dtype == ATTN_FP8_E4M3 && (!(p->o_scale > 0.0f) || !std::isfinite(p->o_scale)))
    return fail(ATTN_EINVAL, "o_scale must be finite and > 0 for fp8 output");
  if (p->sink_size < 0) return fail(ATTN_EINVAL, "sink_size must be >= 0");
  if (p->sink_logits && ((uintptr_t)p->sink_logits & 3u)) return fail(ATTN_EINVAL, "sink_logits is not 4-byte aligned");
  if (p->in_dtype == ATTN_F32 && (p->sink_size > 0 || p->sink_logits))
    return fail(ATTN_ENOTSUP, "attention sinks need bf16 or fp8 inputs");
  if (p->bias_type < ATTN_BIAS_NONE || p->bias_type > ATTN_BIAS_ALIBI)
    return fail(ATTN_EINVAL, "unknown bias_type %d", p->bias_type);
  if (p->bias_type != ATTN_BIAS_NONE) {
    if (p->in_dtype == ATTN_F32) return fail(ATTN_ENOTSUP, "a logit bias needs bf16 or fp8 inputs");
    if (!p->bias) return fail(ATTN_EINVAL, "bias is NULL");
    if (p->bias_stride[0] < 0 || p->bias_stride[1] < 0 || p->bias_stride[2] < 0)
      return fail(ATTN_EINVAL, "bias strides must be >= 0");
    if ((uintptr_t)p->bias & 3u) return fail(ATTN_EINVAL, "bias is not 4-byte aligned");
    if (p->bias_type == ATTN_BIAS_ELEMENTWISE &&
        (((uintptr_t)p->bias & 15u) || p->bias_stride[0] % 4 || p->bias_stride[1] % 4 || p->bias_stride[2] % 4))
      return fail(ATTN_EINVAL, "an elementwise bias needs a 16-byte aligned base and strides that are multiples of 4");
  }
  if (p->min_seqlen_q < 0) return fail(ATTN_EINVAL, "min_seqlen_q must be >= 0");
  if (p->head_dim_v != 0 && p->head_dim_v != 64 && p->head_dim_v != 128)
    return fail(ATTN_ENOTSUP, "head_dim_v %d not supported (0, 64 or 128)", p->head_dim_v);
  if (p->head_dim_v != 0 && p->head_dim_v != d && p->in_dtype == ATTN_F32)
    return fail(ATTN_ENOTSUP, "head_dim_v != d needs bf16 or fp8 inputs");
  if (p->v_layout != ATTN_V_ROW_MAJOR && p->v_layout != ATTN_V_COL_MAJOR)
    return fail(ATTN_EINVAL, "unknown v_layout %d", p->v_layout);
  return ATTN_OK;
}

// head dim of V and O
int dim_v(const attn_params_t* p, int d) { return p->head_dim_v ? p->head_dim_v : d; }

// The cache batch index (batch mode only) and min_seqlen_q (varlen only).
attn_status_t check_mode_fields(const attn_params_t* p, bool batch_mode, bool varlen_mode) {
  if (p->cache_batch_idx) {
    if (!batch_mode) return fail(ATTN_EINVAL, "cache_batch_idx applies to attn_fwd (batch mode) only");
    if (p->in_dtype == ATTN_F32) return fail(ATTN_ENOTSUP, "cache_batch_idx needs bf16 or fp8 inputs");
    if ((uintptr_t)p->cache_batch_idx & 3u) return fail(ATTN_EINVAL, "cache_batch_idx is not 4-byte aligned");
    if (p->cache_batch_count < 1) return fail(ATTN_EINVAL, "cache_batch_count must be >= 1 with cache_batch_idx");
  }
  if (p->min_seqlen_q != 0 && !varlen_mode)
    return fail(ATTN_EINVAL, "min_seqlen_q applies to attn_fwd_varlen only");
  return ATTN_OK;
}

attn_status_t check_strides(const char* name, const int64_t* st, int n, int eb) {
  if (!st) return fail(ATTN_EINVAL, "%s stride array is NULL", name);
  for (int i = 0; i < n; ++i) {
    if (st[i] < 0) return fail(ATTN_EINVAL, "%s stride[%d] is negative", name, i);
    if ((st[i] * eb) % 16 != 0) return fail(ATTN_EINVAL, "%s stride[%d] is not a multiple of 16 bytes", name, i);
  }
  return ATTN_OK;
}

attn_status_t check_ptr(const char* name, const void* ptr) {
  if (!ptr) return fail(ATTN_EINVAL, "%s is NULL", name);
  if (!aligned16(ptr)) return fail(ATTN_EINVAL, "%s is not 16-byte aligned", name);
  return ATTN_OK;
}

// Column-major V (keys contiguous, `row_stride` elements between head-dim
// rows): head_dim_v = d; the keys of one row come in 16-byte chunks (8 bf16 or
// 16 fp8 keys), so the row length (sk, or page_size) must be a multiple of
// that chunk; a tile's span of rows is addressed with 32-bit offsets.
attn_status_t check_colmajor_v(const attn_params_t* p, int d, int len, const char* what, int64_t row_stride) {
  if (p->in_dtype == ATTN_F32) return fail(ATTN_ENOTSUP, "column-major V needs bf16 or fp8 inputs");
  if (dim_v(p, d) != d) return fail(ATTN_ENOTSUP, "column-major V needs head_dim_v = d");
  const int eb = elem_bytes(p->in_dtype), chunk = 16 / eb;
  if (len >= 0 && len % chunk)  // len < 0: the row lengths are device metadata (varlen)
    return fail(ATTN_EINVAL, "column-major V needs %s a multiple of %d (got %d)", what, chunk, len);
  if ((int64_t)(d - 1) * row_stride * eb + 64 * eb >= ((int64_t)1 << 31))
    return fail(ATTN_EINVAL, "column-major V: head-dim row stride too large");
  return ATTN_OK;
}

// exp2-domain constants shared by all paths
void logit_consts(const attn_params_t* p, float* c_exp2, float* pre, float* post) {
  double s = p->scale;
  if (p->in_dtype == ATTN_FP8_E4M3) s *= (double)p->q_descale * (double)p->k_descale;
  if (p->softcap > 0.0f) {
    *pre = (float)(s / p->softcap);
    *post = (float)(p->softcap * 1.4426950408889634);
    *c_exp2 = 1.0f;
  } else {
    *pre = 0.0f;
    *post = 0.0f;
    *c_exp2 = (float)(s * 1.4426950408889634);
  }
}

// In-tile byte offsets are 32-bit in the kernels (buffer-load offsets and
// ranges): the rows of one tile (64 keys in the prefill kernel, a 32-key
// granule in the split-KV kernel) must span less than 2 GiB.
attn_status_t check_row_span(const char* name, int64_t row_stride, int eb, int rows) {
  if ((int64_t)rows * row_stride * eb >= ((int64_t)1 << 31))
    return fail(ATTN_EINVAL, "%s row stride %lld (x %d rows of a tile) spans 2 GiB or more; 32-bit in-tile offsets",
                name, (long long)row_stride, rows);
  return ATTN_OK;
}
constexpr int kPrefillTileRows = 64;
constexpr int kDecodeGranRows = 32;

// ---- ATTN_LOG: one stderr line per accepted call (entry point, path, types,
// shape, mask, launch grid, split plan) and one per refused or failed call
// (status and message), read per call like ATTN_VALIDATE ----
bool log_on() {
  const char* e = getenv("ATTN_LOG");
  return e && *e && strcmp(e, "0") != 0;
}

const char* dtype_name(int t) { return t == ATTN_F32 ? "f32" : (t == ATTN_BF16 ? "bf16" : "fp8_e4m3"); }

void log_call(const char* entry, const char* path, const attn_params_t* p, int d, int dv, int nz, int Hq, int Hkv,
              int sq, int sk, const char* launch) {
  if (!log_on()) return;
  fprintf(stderr,
          "attn: %s path=%s in=%s out=%s d=%d dv=%d batch=%d Hq=%d Hkv=%d sq=%d sk=%d window=(%d,%d) softcap=%g "
          "bias=%d sink_size=%d sink_logits=%d v_layout=%d %s\n",
          entry, path, dtype_name(p->in_dtype), dtype_name(p->out_dtype), d, dv, nz, Hq, Hkv, sq, sk, p->window_left,
          p->window_right, (double)p->softcap, p->bias_type, p->sink_size, p->sink_logits ? 1 : 0, p->v_layout,
          launch);
}

void log_prefill(const char* entry, const attn_params_t* p, const attn::PrefillArgs& a, int d, int dv, int nz,
                 int sq, int sk) {
  if (!log_on()) return;
  char g[160];
  snprintf(g, sizeof(g), "grid=%lld workgroups x 256 threads (%d query tiles of %d packed rows per unit)",
           (long long)attn::prefill_workgroups(a, nz), a.n_qtiles, attn::prefill_rows_per_tile(p->in_dtype));
  log_call(entry, "prefill", p, d, dv, nz, a.hq, a.hkv, sq, sk, g);
}

void log_decode(const char* entry, const attn_params_t* p, const attn::DecodeArgs& a, int d, int dv, int B,
                int sk) {
  if (!log_on()) return;
  char g[200];
  snprintf(g, sizeof(g), "grid=(%d,%d,%d) x 64 threads, splits=%d of %d keys; combine grid=%lld x 256 threads",
           a.hkv, a.n_splits, B, a.n_splits, a.split_tokens, (long long)(((int64_t)B * a.hq * a.sq + 3) / 4));
  log_call(entry, "split-kv decode", p, d, dv, B, a.hq, a.hkv, a.sq, sk, g);
}

attn_status_t launched(hipError_t e) {
  if (e != hipSuccess) return fail(ATTN_ELAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ATTN_OK;
}

#define TRY(x)                       \
  do {                               \
    attn_status_t st_ = (x);         \
    if (st_ != ATTN_OK) return st_;  \
  } while (0)

// ---- optional host-side check of device-resident metadata (ATTN_VALIDATE) ----
// Read per call, so a process can switch it on and off. It synchronises the
// stream, so it is a debugging aid, not for graph capture or serving loops.
bool validate_on() {
  const char* e = getenv("ATTN_VALIDATE");
  return e && *e && strcmp(e, "0") != 0;
}

// Waits for the stream (whose earlier work may still write the array), then
// copies count int32 from dev (device or host memory) into out.
attn_status_t fetch_i32(const char* name, const int32_t* dev, size_t count, hipStream_t s, std::vector<int32_t>& out) {
  out.assign(count, 0);
  if (count == 0) return ATTN_OK;
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(out.data(), dev, count * sizeof(int32_t), hipMemcpyDefault);
  if (e != hipSuccess) return fail(ATTN_EINVAL, "ATTN_VALIDATE: cannot read %s: %s", name, hipGetErrorString(e));
  return ATTN_OK;
}

// per-entry values 0 <= x <= hi (an absent array: nothing to check); the values are returned in h
attn_status_t validate_range(const char* name, const int32_t* dev, int count, int hi, hipStream_t s,
                             std::vector<int32_t>& h) {
  if (!dev) return ATTN_OK;
  TRY(fetch_i32(name, dev, (size_t)count, s, h));
  for (int i = 0; i < count; ++i)
    if (h[i] < 0 || h[i] > hi) return fail(ATTN_EINVAL, "ATTN_VALIDATE: %s[%d] = %d is outside [0, %d]", name, i, h[i], hi);
  return ATTN_OK;
}

// cu[0] >= 0, non-decreasing, every length <= max_len, cu[n] <= total (total < 0: unbounded)
attn_status_t validate_cu(const char* name, const int32_t* dev, int n, int max_len, int64_t total, hipStream_t s,
                          int multiple = 1) {
  std::vector<int32_t> h;
  TRY(fetch_i32(name, dev, (size_t)n + 1, s, h));
  if (h[0] < 0) return fail(ATTN_EINVAL, "ATTN_VALIDATE: %s[0] = %d is negative", name, h[0]);
  for (int i = 0; i <= n; ++i)
    if (h[i] % multiple)
      return fail(ATTN_EINVAL, "ATTN_VALIDATE: %s[%d] = %d is not a multiple of %d (column-major V)", name, i, h[i],
                  multiple);
  for (int i = 0; i < n; ++i) {
    const int64_t l = (int64_t)h[i + 1] - h[i];
    if (l < 0) return fail(ATTN_EINVAL, "ATTN_VALIDATE: %s decreases at entry %d (%d -> %d)", name, i, h[i], h[i + 1]);
    if (l > max_len)
      return fail(ATTN_EINVAL, "ATTN_VALIDATE: sequence %d of %s has length %lld > its maximum %d", i, name, (long long)l,
                  max_len);
  }
  if (total >= 0 && h[n] > total)
    return fail(ATTN_EINVAL, "ATTN_VALIDATE: %s[%d] = %d exceeds %lld", name, n, h[n], (long long)total);
  return ATTN_OK;
}

// page ids of the tokens [first[r], first[r] + count[r]) of each table row r
// lie in [0, num_pages); a row with count 0, or first < 0 (not computed), uses no entry
attn_status_t validate_pages(const int32_t* table_dev, int rows, int stride, int page_size, int num_pages,
                             const std::vector<int32_t>& first, const std::vector<int32_t>& count, hipStream_t s) {
  std::vector<int32_t> t;
  TRY(fetch_i32("block_table", table_dev, (size_t)rows * stride, s, t));
  for (int r = 0; r < rows; ++r) {
    if (count[r] <= 0 || first[r] < 0) continue;
    const int64_t end = (int64_t)first[r] + count[r];
    for (int64_t i = first[r] / page_size; i < (end + page_size - 1) / page_size; ++i) {
      const int32_t id = t[(size_t)r * stride + i];
      if (id < 0 || id >= num_pages)
        return fail(ATTN_EINVAL, "ATTN_VALIDATE: block_table[%d][%lld] = %d is not a page id in [0, %d)", r,
                    (long long)i, id, num_pages);
    }
  }
  return ATTN_OK;
}

}  // namespace

namespace attn {
// Sets the calling thread's attn_last_error() text (for entry points defined
// in other sources of the library) and returns st.
attn_status_t set_error(attn_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}
}  // namespace attn

extern "C" {

const char* attn_last_error(void) { return g_err; }

const char* attn_version(void) { return "libattn 0.1 (gfx950)"; }

void attn_params_init(attn_params_t* p, float scale) {
  if (!p) return;
  memset(p, 0, sizeof(*p));
  p->in_dtype = ATTN_BF16;
  p->out_dtype = ATTN_BF16;
  p->scale = scale;
  p->softcap = 0.0f;
  p->window_left = -1;
  p->window_right = -1;
  p->q_descale = p->k_descale = p->v_descale = 1.0f;
  p->kv_split_tokens = 0;
  p->sink_size = 0;
  p->sink_logits = nullptr;
  p->bias_type = ATTN_BIAS_NONE;
  p->bias = nullptr;
  p->bias_stride[0] = p->bias_stride[1] = p->bias_stride[2] = 0;
  p->o_scale = 1.0f;
  p->cache_batch_idx = nullptr;
  p->cache_batch_count = 0;
  p->min_seqlen_q = 0;
  p->head_dim_v = 0;
  p->v_layout = ATTN_V_ROW_MAJOR;
  p->v_pool_stride[0] = p->v_pool_stride[1] = p->v_pool_stride[2] = 0;
}

size_t attn_workspace_bytes(const attn_params_t* p, int B, int Hq, int Hkv, int sq, int d, int max_seqlen_k) {
  if (!p || B <= 0 || Hq <= 0 || Hkv <= 0 || sq <= 0 || max_seqlen_k < 0 || Hq % Hkv) return 0;
  const int ratio = Hq / Hkv;
  if (!takes_decode_path(p->in_dtype, sq, ratio)) return 0;
  const int split = plan_split_tokens(p, B, Hkv, max_seqlen_k);
  return decode_ws_bytes(B, Hkv, n_splits_for(split, max_seqlen_k), sq * ratio, dim_v(p, d));
}

int attn_num_splits(const attn_params_t* p, int B, int Hq, int Hkv, int sq, int max_seqlen_k) {
  if (!p || B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || sq <= 0) return 1;
  if (!takes_decode_path(p->in_dtype, sq, Hq / Hkv)) return 1;
  return n_splits_for(plan_split_tokens(p, B, Hkv, max_seqlen_k), max_seqlen_k);
}

attn_status_t attn_fwd(const attn_params_t* p, const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int Hq, int Hkv, int sq, int sk, int d, const int64_t q_stride[3],
                       const int64_t k_stride[3], const int64_t v_stride[3], const int64_t o_stride[3],
                       const int32_t* seqused_q, const int32_t* seqused_k, void* workspace,
                       size_t workspace_bytes, void* stream) {
  TRY(check_params(p, d));
  TRY(check_mode_fields(p, true, false));
  if (B < 0 || Hq <= 0 || Hkv <= 0 || sq < 0 || sk < 0) return fail(ATTN_EINVAL, "bad sizes B=%d Hq=%d Hkv=%d sq=%d sk=%d", B, Hq, Hkv, sq, sk);
  if (Hq % Hkv) return fail(ATTN_EINVAL, "Hq (%d) is not a multiple of Hkv (%d)", Hq, Hkv);
  const int eb = elem_bytes(p->in_dtype), ob = elem_bytes(p->out_dtype);
  TRY(check_ptr("q", q));
  if (sk > 0 || k) TRY(check_ptr("k", k));   // no keys: K and V may be NULL (nothing is read)
  if (sk > 0 || v) TRY(check_ptr("v", v));
  TRY(check_ptr("o", o));
  if (lse && ((uintptr_t)lse & 3u)) return fail(ATTN_EINVAL, "lse is not 4-byte aligned");
  TRY(check_strides("q", q_stride, 3, eb));
  TRY(check_strides("k", k_stride, 3, eb));
  TRY(check_strides("v", v_stride, 3, eb));
  TRY(check_strides("o", o_stride, 3, ob));
  if (p->v_layout == ATTN_V_COL_MAJOR) TRY(check_colmajor_v(p, d, sk, "sk", v_stride[2]));
  if (B == 0 || sq == 0) return ATTN_OK;
  const int ratio = Hq / Hkv;
  hipStream_t s = (hipStream_t)stream;
  if (validate_on()) {
    std::vector<int32_t> h;
    TRY(validate_range("seqused_q", seqused_q, B, sq, s, h));
    TRY(validate_range("seqused_k", seqused_k, B, sk, s, h));
  }
  float c_exp2, pre, post;
  logit_consts(p, &c_exp2, &pre, &post);

  if (p->in_dtype == ATTN_F32) {
    attn::F32Args a{};
    a.q = (const float*)q; a.k = (const float*)k; a.v = (const float*)v; a.o = (float*)o; a.lse = lse;
    a.q_sb = q_stride[0]; a.q_sh = q_stride[1]; a.q_sr = q_stride[2];
    a.k_sb = k_stride[0]; a.k_sh = k_stride[1]; a.k_sr = k_stride[2];
    a.v_sb = v_stride[0]; a.v_sh = v_stride[1]; a.v_sr = v_stride[2];
    a.o_sb = o_stride[0]; a.o_sh = o_stride[1]; a.o_sr = o_stride[2];
    a.seqused_q = seqused_q; a.seqused_k = seqused_k;
    a.B = B; a.sq = sq; a.sk = sk; a.hq = Hq; a.hkv = Hkv; a.ratio = ratio;
    a.c_exp2 = c_exp2; a.softcap_pre = pre; a.softcap_post = post;
    a.wl = p->window_left; a.wr = p->window_right;
    if (log_on()) {
      char g[96];
      snprintf(g, sizeof(g), "grid=%lld workgroups x 256 threads", (long long)attn::f32_workgroups(a));
      log_call("attn_fwd", "f32", p, d, d, B, Hq, Hkv, sq, sk, g);
    }
    return launched(attn::launch_f32(a, d, s));
  }

  if (takes_decode_path(p->in_dtype, sq, ratio)) {
    TRY(check_row_span("k", k_stride[2], eb, kDecodeGranRows));
    if (p->v_layout == ATTN_V_ROW_MAJOR) TRY(check_row_span("v", v_stride[2], eb, kDecodeGranRows));
    const int dv = dim_v(p, d);
    const int split = plan_split_tokens(p, B, Hkv, sk);
    const int nsp = n_splits_for(split, sk);
    const int m_rows = sq * ratio;
    const size_t need = decode_ws_bytes(B, Hkv, nsp, m_rows, dv);
    if (!workspace || workspace_bytes < need)
      return fail(ATTN_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
    TRY(check_ptr("workspace", workspace));
    attn::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v;
    a.q_sb = q_stride[0]; a.q_sh = q_stride[1]; a.q_sr = q_stride[2];
    a.k_sb = k_stride[0]; a.k_sh = k_stride[1]; a.k_sr = k_stride[2];
    a.v_sb = v_stride[0]; a.v_sh = v_stride[1]; a.v_sr = v_stride[2];
    a.seqlens_k = seqused_k; a.seqused_q = seqused_q; a.block_table = nullptr; a.bt_stride = 0; a.page_size = 0;
    a.v_colmajor = p->v_layout == ATTN_V_COL_MAJOR;
    a.sk = sk; a.sq = sq; a.hq = Hq; a.hkv = Hkv; a.ratio = ratio; a.m_rows = m_rows;
    a.split_tokens = split; a.n_splits = nsp;
    a.c_exp2 = c_exp2; a.softcap_pre = pre; a.softcap_post = post;
    a.wl = p->window_left; a.wr = p->window_right;
    a.sink_size = p->sink_size;
    a.fp8 = p->in_dtype == ATTN_FP8_E4M3;
    a.cache_idx = p->cache_batch_idx; a.cache_count = p->cache_batch_count;
    set_bias(p, c_exp2, &a);
    const size_t units = (size_t)B * Hkv * nsp * m_rows;
    a.part_o = (float*)workspace;
    a.part_lse = (float*)((char*)workspace + align256(units * dv * sizeof(float)));
    attn::CombineArgs c{};
    c.part_o = a.part_o; c.part_lse = a.part_lse; c.o = o; c.lse = lse;
    c.o_sb = o_stride[0]; c.o_sh = o_stride[1]; c.o_sr = o_stride[2];
    c.seqlens_k = seqused_k; c.seqused_q = seqused_q; c.sk = sk;
    c.no_keys = !k || !v;
    c.cache_idx = p->cache_batch_idx; c.cache_count = p->cache_batch_count;
    c.B = B; c.sq = sq; c.hq = Hq; c.hkv = Hkv; c.ratio = ratio; c.m_rows = m_rows;
    c.split_tokens = split; c.n_splits = nsp; c.o_mul = out_mul(p);
  c.out_fp8 = p->out_dtype == ATTN_FP8_E4M3;
    c.sink_logits = p->sink_logits;
    log_decode("attn_fwd", p, a, d, dv, B, sk);
    return launched(attn::launch_decode(a, c, d, dv, false, B, s));
  }

  TRY(check_row_span("k", k_stride[2], eb, kPrefillTileRows));
  if (p->v_layout == ATTN_V_ROW_MAJOR) TRY(check_row_span("v", v_stride[2], eb, kPrefillTileRows));
  attn::PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.q_sb = q_stride[0]; a.q_sh = q_stride[1]; a.q_sr = q_stride[2];
  a.k_sb = k_stride[0]; a.k_sh = k_stride[1]; a.k_sr = k_stride[2];
  a.v_sb = v_stride[0]; a.v_sh = v_stride[1]; a.v_sr = v_stride[2];
  a.o_sb = o_stride[0]; a.o_sh = o_stride[1]; a.o_sr = o_stride[2];
  a.lse_sb = (int64_t)Hq * sq; a.lse_sh = sq;
  a.seqused_q = seqused_q; a.seqused_k = seqused_k;
  a.cache_idx = p->cache_batch_idx; a.cache_count = p->cache_batch_count;
  a.v_colmajor = p->v_layout == ATTN_V_COL_MAJOR;
  a.sq = sq; a.sk = sk; a.hq = Hq; a.hkv = Hkv; a.ratio = ratio;
  const int rows_tile = attn::prefill_rows_per_tile(p->in_dtype);
  a.n_qtiles = (int)(((int64_t)sq * ratio + rows_tile - 1) / rows_tile);
  a.c_exp2 = c_exp2; a.softcap_pre = pre; a.softcap_post = post;
  a.o_mul = out_mul(p);
  a.out_fp8 = p->out_dtype == ATTN_FP8_E4M3;
  a.wl = p->window_left; a.wr = p->window_right;
  a.sink_size = p->sink_size; a.sink_logits = p->sink_logits;
  set_bias(p, c_exp2, &a);
  log_prefill("attn_fwd", p, a, d, dim_v(p, d), B, sq, sk);
  return launched(attn::launch_prefill(a, d, dim_v(p, d), p->in_dtype, attn::kPrefillBatch, B, s));
}

attn_status_t attn_fwd_varlen(const attn_params_t* p, const void* q, const void* k, const void* v, void* o,
                              float* lse, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int n,
                              int total_q, int max_seqlen_q, int max_seqlen_k, int Hq, int Hkv, int d,
                              const int64_t q_stride[2], const int64_t k_stride[2], const int64_t v_stride[2],
                              const int64_t o_stride[2], void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  (void)max_seqlen_k;
  TRY(check_params(p, d));
  TRY(check_mode_fields(p, false, true));
  if (p->in_dtype == ATTN_F32) return fail(ATTN_ENOTSUP, "fp32 inputs are supported in batch mode only");
  if (n < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || Hq <= 0 || Hkv <= 0)
    return fail(ATTN_EINVAL, "bad sizes n=%d total_q=%d max_q=%d max_k=%d Hq=%d Hkv=%d", n, total_q, max_seqlen_q,
                max_seqlen_k, Hq, Hkv);
  if (Hq % Hkv) return fail(ATTN_EINVAL, "Hq (%d) is not a multiple of Hkv (%d)", Hq, Hkv);
  if (!cu_seqlens_q || !cu_seqlens_k) return fail(ATTN_EINVAL, "cu_seqlens_q / cu_seqlens_k is NULL");
  const int eb = elem_bytes(p->in_dtype), ob = elem_bytes(p->out_dtype);
  TRY(check_ptr("q", q));
  if (max_seqlen_k > 0 || k) TRY(check_ptr("k", k));   // no keys anywhere: K and V may be NULL
  if (max_seqlen_k > 0 || v) TRY(check_ptr("v", v));
  TRY(check_ptr("o", o));
  if (lse && ((uintptr_t)lse & 3u)) return fail(ATTN_EINVAL, "lse is not 4-byte aligned");
  TRY(check_strides("q", q_stride, 2, eb));
  TRY(check_strides("k", k_stride, 2, eb));
  TRY(check_strides("v", v_stride, 2, eb));
  TRY(check_strides("o", o_stride, 2, ob));
  TRY(check_row_span("k", k_stride[0], eb, kPrefillTileRows));
  // column-major V: v_stride[0] is the stride between head-dim rows, keys run
  // along the packed token axis; every cu_seqlens_k entry a multiple of one
  // 16-byte chunk of keys (refused under ATTN_VALIDATE; otherwise a sequence
  // off that grid reads no key and gets NaN rows)
  const bool v_cm = p->v_layout == ATTN_V_COL_MAJOR;
  if (v_cm) TRY(check_colmajor_v(p, d, -1, "", v_stride[0]));
  else TRY(check_row_span("v", v_stride[0], eb, kPrefillTileRows));
  if (n == 0 || max_seqlen_q == 0) return ATTN_OK;
  if (validate_on()) {
    TRY(validate_cu("cu_seqlens_q", cu_seqlens_q, n, max_seqlen_q, total_q, (hipStream_t)stream));
    TRY(validate_cu("cu_seqlens_k", cu_seqlens_k, n, max_seqlen_k, -1, (hipStream_t)stream, v_cm ? 16 / eb : 1));
  }
  float c_exp2, pre, post;
  logit_consts(p, &c_exp2, &pre, &post);
  const int ratio = Hq / Hkv;
  attn::PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.q_sb = 0; a.q_sh = q_stride[1]; a.q_sr = q_stride[0];
  a.k_sb = 0; a.k_sh = k_stride[1]; a.k_sr = k_stride[0];
  a.v_sb = 0; a.v_sh = v_stride[1]; a.v_sr = v_stride[0];
  a.o_sb = 0; a.o_sh = o_stride[1]; a.o_sr = o_stride[0];
  a.lse_sb = 0; a.lse_sh = total_q;
  a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
  a.min_seqlen_q = p->min_seqlen_q;
  a.v_colmajor = v_cm;
  a.hq = Hq; a.hkv = Hkv; a.ratio = ratio;
  const int rows_tile = attn::prefill_rows_per_tile(p->in_dtype);
  a.n_qtiles = (int)(((int64_t)max_seqlen_q * ratio + rows_tile - 1) / rows_tile);
  a.c_exp2 = c_exp2; a.softcap_pre = pre; a.softcap_post = post;
  a.o_mul = out_mul(p);
  a.out_fp8 = p->out_dtype == ATTN_FP8_E4M3;
  a.wl = p->window_left; a.wr = p->window_right;
  a.sink_size = p->sink_size; a.sink_logits = p->sink_logits;
  set_bias(p, c_exp2, &a);
  log_prefill("attn_fwd_varlen", p, a, d, dim_v(p, d), n, max_seqlen_q, max_seqlen_k);
  return launched(attn::launch_prefill(a, d, dim_v(p, d), p->in_dtype, attn::kPrefillVarlen, n, (hipStream_t)stream));
}

attn_status_t attn_fwd_paged(const attn_params_t* p, const void* q, const void* k_pool, const void* v_pool, void* o,
                             float* lse, const int32_t* block_table, int block_table_stride,
                             const int32_t* seqlens_k, int B, int sq, int Hq, int Hkv, int d, int page_size,
                             int num_pages, const int64_t q_stride[3], const int64_t kv_stride[3],
                             const int64_t o_stride[3], void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_params(p, d));
  TRY(check_mode_fields(p, false, false));
  const int dv = dim_v(p, d);
  const int64_t* v_st = v_pool_strides(p, kv_stride);
  if (dv != d && v_st == kv_stride)
    return fail(ATTN_EINVAL, "head_dim_v != d in paged mode needs v_pool_stride (the V pool's strides)");
  const bool v_cm = p->v_layout == ATTN_V_COL_MAJOR;
  if (v_cm && v_st == kv_stride)
    return fail(ATTN_EINVAL, "column-major V pages need v_pool_stride ({page, head, head-dim row})");
  if (B < 0 || sq < 0 || Hq <= 0 || Hkv <= 0 || block_table_stride <= 0 || num_pages <= 0)
    return fail(ATTN_EINVAL, "bad sizes B=%d sq=%d Hq=%d Hkv=%d table_stride=%d num_pages=%d", B, sq, Hq, Hkv,
                block_table_stride, num_pages);
  if (Hq % Hkv) return fail(ATTN_EINVAL, "Hq (%d) is not a multiple of Hkv (%d)", Hq, Hkv);
  if (page_size <= 0 || page_size % 32) return fail(ATTN_ENOTSUP, "page_size %d is not a positive multiple of 32", page_size);
  if (p->in_dtype == ATTN_F32) return fail(ATTN_ENOTSUP, "paged KV supports bf16 and fp8 inputs");
  const int ratio = Hq / Hkv;
  const bool decode_shape = takes_decode_path(p->in_dtype, sq, ratio);
  if (!decode_shape && page_size % 64)
    return fail(ATTN_ENOTSUP, "paged prefill (sq*Hq/Hkv > 16) needs page_size a multiple of 64 (got %d)", page_size);
  if (!block_table || !seqlens_k) return fail(ATTN_EINVAL, "block_table / seqlens_k is NULL");
  TRY(check_ptr("q", q));
  TRY(check_ptr("k_pool", k_pool));
  TRY(check_ptr("v_pool", v_pool));
  TRY(check_ptr("o", o));
  if (lse && ((uintptr_t)lse & 3u)) return fail(ATTN_EINVAL, "lse is not 4-byte aligned");
  const int eb = elem_bytes(p->in_dtype);
  TRY(check_strides("q", q_stride, 3, eb));
  TRY(check_strides("kv", kv_stride, 3, eb));
  TRY(check_strides("v_pool_stride", v_st, 3, eb));
  TRY(check_strides("o", o_stride, 3, elem_bytes(p->out_dtype)));
  TRY(check_row_span("k_pool", kv_stride[2], eb, decode_shape ? kDecodeGranRows : kPrefillTileRows));
  if (v_cm) TRY(check_colmajor_v(p, d, page_size, "page_size", v_st[2]));
  else TRY(check_row_span("v_pool", v_st[2], eb, decode_shape ? kDecodeGranRows : kPrefillTileRows));
  if (B == 0 || sq == 0) return ATTN_OK;
  const int64_t max_len64 = (int64_t)block_table_stride * page_size;
  if (max_len64 > (1 << 30)) return fail(ATTN_EINVAL, "block_table_stride * page_size is too large");
  const int max_len = (int)max_len64;
  if (validate_on()) {
    std::vector<int32_t> lk;
    TRY(validate_range("seqlens_k", seqlens_k, B, max_len, (hipStream_t)stream, lk));
    TRY(validate_pages(block_table, B, block_table_stride, page_size, num_pages, std::vector<int32_t>(B, 0), lk,
                       (hipStream_t)stream));
  }
  float c_exp2, pre, post;
  logit_consts(p, &c_exp2, &pre, &post);

  if (!decode_shape) {
    // paged prefill: the prefill kernel, with each 64-key tile's rows found
    // through the block table
    attn::PrefillArgs a{};
    a.q = q; a.k = k_pool; a.v = v_pool; a.o = o; a.lse = lse;
    a.q_sb = q_stride[0]; a.q_sh = q_stride[1]; a.q_sr = q_stride[2];
    a.k_sb = kv_stride[0]; a.k_sh = kv_stride[1]; a.k_sr = kv_stride[2];
    a.v_sb = v_st[0]; a.v_sh = v_st[1]; a.v_sr = v_st[2];
    a.o_sb = o_stride[0]; a.o_sh = o_stride[1]; a.o_sr = o_stride[2];
    a.lse_sb = (int64_t)Hq * sq; a.lse_sh = sq;
    a.seqused_q = nullptr; a.seqused_k = seqlens_k;
    a.block_table = block_table; a.bt_stride = block_table_stride; a.page_size = page_size;
    a.v_colmajor = v_cm;
    a.sq = sq; a.sk = max_len; a.hq = Hq; a.hkv = Hkv; a.ratio = ratio;
    const int rows_tile = attn::prefill_rows_per_tile(p->in_dtype);
    a.n_qtiles = (int)(((int64_t)sq * ratio + rows_tile - 1) / rows_tile);
    a.c_exp2 = c_exp2; a.softcap_pre = pre; a.softcap_post = post;
    a.o_mul = out_mul(p);
  a.out_fp8 = p->out_dtype == ATTN_FP8_E4M3;
    a.wl = p->window_left; a.wr = p->window_right;
    a.sink_size = p->sink_size; a.sink_logits = p->sink_logits;
    set_bias(p, c_exp2, &a);
    log_prefill("attn_fwd_paged", p, a, d, dv, B, sq, max_len);
    return launched(attn::launch_prefill(a, d, dv, p->in_dtype, attn::kPrefillPaged, B, (hipStream_t)stream));
  }

  const int split = plan_split_tokens(p, B, Hkv, max_len);
  const int nsp = n_splits_for(split, max_len);
  const int m_rows = sq * ratio;
  const size_t need = decode_ws_bytes(B, Hkv, nsp, m_rows, dv);
  if (!workspace || workspace_bytes < need)
    return fail(ATTN_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
  TRY(check_ptr("workspace", workspace));
  attn::DecodeArgs a{};
  a.q = q; a.k = k_pool; a.v = v_pool;
  a.q_sb = q_stride[0]; a.q_sh = q_stride[1]; a.q_sr = q_stride[2];
  a.k_sb = kv_stride[0]; a.k_sh = kv_stride[1]; a.k_sr = kv_stride[2];
  a.v_sb = v_st[0]; a.v_sh = v_st[1]; a.v_sr = v_st[2];
  a.seqlens_k = seqlens_k; a.block_table = block_table; a.bt_stride = block_table_stride; a.page_size = page_size;
  a.v_colmajor = v_cm;
  a.sk = max_len; a.sq = sq; a.hq = Hq; a.hkv = Hkv; a.ratio = ratio; a.m_rows = m_rows;
  a.split_tokens = split; a.n_splits = nsp;
  a.c_exp2 = c_exp2; a.softcap_pre = pre; a.softcap_post = post;
  a.wl = p->window_left; a.wr = p->window_right;
  a.sink_size = p->sink_size;
  a.fp8 = p->in_dtype == ATTN_FP8_E4M3;
  set_bias(p, c_exp2, &a);
  const size_t units = (size_t)B * Hkv * nsp * m_rows;
  a.part_o = (float*)workspace;
  a.part_lse = (float*)((char*)workspace + align256(units * dv * sizeof(float)));
  attn::CombineArgs c{};
  c.part_o = a.part_o; c.part_lse = a.part_lse; c.o = o; c.lse = lse;
  c.o_sb = o_stride[0]; c.o_sh = o_stride[1]; c.o_sr = o_stride[2];
  c.seqlens_k = seqlens_k; c.sk = max_len;
  c.B = B; c.sq = sq; c.hq = Hq; c.hkv = Hkv; c.ratio = ratio; c.m_rows = m_rows;
  c.split_tokens = split; c.n_splits = nsp; c.o_mul = out_mul(p);
  c.out_fp8 = p->out_dtype == ATTN_FP8_E4M3;
  c.sink_logits = p->sink_logits;
  log_decode("attn_fwd_paged", p, a, d, dv, B, max_len);
  return launched(attn::launch_decode(a, c, d, dv, true, B, (hipStream_t)stream));
}

attn_status_t attn_fwd_varlen_paged(const attn_params_t* p, const void* q, const void* k_pool, const void* v_pool,
                                    void* o, float* lse, const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                                    const int32_t* kv_start, const int32_t* block_table, int block_table_stride,
                                    int n, int total_q, int max_seqlen_q, int Hq, int Hkv, int d, int page_size,
                                    int num_pages, const int64_t q_stride[2], const int64_t kv_stride[3],
                                    const int64_t o_stride[2], void* stream) {
  TRY(check_params(p, d));
  TRY(check_mode_fields(p, false, true));
  if (p->v_layout == ATTN_V_COL_MAJOR)
    return fail(ATTN_ENOTSUP, "column-major V is supported by attn_fwd, attn_fwd_varlen and attn_fwd_paged");
  const int dv = dim_v(p, d);
  const int64_t* v_st = v_pool_strides(p, kv_stride);
  if (dv != d && v_st == kv_stride)
    return fail(ATTN_EINVAL, "head_dim_v != d in paged mode needs v_pool_stride (the V pool's strides)");
  if (p->in_dtype == ATTN_F32) return fail(ATTN_ENOTSUP, "paged KV supports bf16 and fp8 inputs");
  if (n < 0 || total_q < 0 || max_seqlen_q < 0 || Hq <= 0 || Hkv <= 0 || block_table_stride <= 0 || num_pages <= 0)
    return fail(ATTN_EINVAL, "bad sizes n=%d total_q=%d max_q=%d Hq=%d Hkv=%d table_stride=%d num_pages=%d", n,
                total_q, max_seqlen_q, Hq, Hkv, block_table_stride, num_pages);
  if (Hq % Hkv) return fail(ATTN_EINVAL, "Hq (%d) is not a multiple of Hkv (%d)", Hq, Hkv);
  if (page_size <= 0 || page_size % 64)
    return fail(ATTN_ENOTSUP, "page_size %d is not a positive multiple of 64", page_size);
  if (!cu_seqlens_q || !seqlens_k || !block_table)
    return fail(ATTN_EINVAL, "cu_seqlens_q / seqlens_k / block_table is NULL");
  if (kv_start && ((uintptr_t)kv_start & 3u)) return fail(ATTN_EINVAL, "kv_start is not 4-byte aligned");
  TRY(check_ptr("q", q));
  TRY(check_ptr("k_pool", k_pool));
  TRY(check_ptr("v_pool", v_pool));
  TRY(check_ptr("o", o));
  if (lse && ((uintptr_t)lse & 3u)) return fail(ATTN_EINVAL, "lse is not 4-byte aligned");
  const int eb = elem_bytes(p->in_dtype);
  TRY(check_strides("q", q_stride, 2, eb));
  TRY(check_strides("kv", kv_stride, 3, eb));
  TRY(check_strides("v_pool_stride", v_st, 3, eb));
  TRY(check_strides("o", o_stride, 2, elem_bytes(p->out_dtype)));
  TRY(check_row_span("k_pool", kv_stride[2], eb, kPrefillTileRows));
  TRY(check_row_span("v_pool", v_st[2], eb, kPrefillTileRows));
  if (n == 0 || max_seqlen_q == 0) return ATTN_OK;
  const int64_t max_len64 = (int64_t)block_table_stride * page_size;
  if (max_len64 > (1 << 30)) return fail(ATTN_EINVAL, "block_table_stride * page_size is too large");
  if (validate_on()) {
    hipStream_t vs = (hipStream_t)stream;
    std::vector<int32_t> lk, st;
    TRY(validate_cu("cu_seqlens_q", cu_seqlens_q, n, max_seqlen_q, total_q, vs));
    TRY(validate_range("seqlens_k", seqlens_k, n, (int)max_len64, vs, lk));
    if (kv_start) {
      TRY(fetch_i32("kv_start", kv_start, (size_t)n, vs, st));
    } else {
      st.assign(n, 0);
    }
    for (int i = 0; i < n; ++i)
      if (st[i] >= 0 && (int64_t)st[i] + lk[i] > max_len64)
        return fail(ATTN_EINVAL, "ATTN_VALIDATE: kv_start[%d] + seqlens_k[%d] = %lld exceeds the table row (%lld tokens)",
                    i, i, (long long)st[i] + lk[i], (long long)max_len64);
    TRY(validate_pages(block_table, n, block_table_stride, page_size, num_pages, st, lk, vs));
  }
  float c_exp2, pre, post;
  logit_consts(p, &c_exp2, &pre, &post);
  const int ratio = Hq / Hkv;
  attn::PrefillArgs a{};
  a.q = q; a.k = k_pool; a.v = v_pool; a.o = o; a.lse = lse;
  a.q_sb = 0; a.q_sh = q_stride[1]; a.q_sr = q_stride[0];
  a.k_sb = kv_stride[0]; a.k_sh = kv_stride[1]; a.k_sr = kv_stride[2];
  a.v_sb = v_st[0]; a.v_sh = v_st[1]; a.v_sr = v_st[2];
  a.o_sb = 0; a.o_sh = o_stride[1]; a.o_sr = o_stride[0];
  a.lse_sb = 0; a.lse_sh = total_q;
  a.cu_q = cu_seqlens_q; a.cu_k = nullptr;
  a.seqused_q = nullptr; a.seqused_k = seqlens_k; a.kv_start = kv_start;
  a.block_table = block_table; a.bt_stride = block_table_stride; a.page_size = page_size;
  a.min_seqlen_q = p->min_seqlen_q;
  a.sq = 0; a.sk = (int)max_len64; a.hq = Hq; a.hkv = Hkv; a.ratio = ratio;
  const int rows_tile = attn::prefill_rows_per_tile(p->in_dtype);
  a.n_qtiles = (int)(((int64_t)max_seqlen_q * ratio + rows_tile - 1) / rows_tile);
  a.c_exp2 = c_exp2; a.softcap_pre = pre; a.softcap_post = post;
  a.o_mul = out_mul(p);
  a.out_fp8 = p->out_dtype == ATTN_FP8_E4M3;
  a.wl = p->window_left; a.wr = p->window_right;
  a.sink_size = p->sink_size; a.sink_logits = p->sink_logits;
  set_bias(p, c_exp2, &a);
  log_prefill("attn_fwd_varlen_paged", p, a, d, dv, n, max_seqlen_q, (int)max_len64);
  return launched(attn::launch_prefill(a, d, dv, p->in_dtype, attn::kPrefillVarlenPaged, n, (hipStream_t)stream));
}

}  // extern "C"
