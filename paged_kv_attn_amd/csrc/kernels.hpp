// Launch-side view of the attention kernels: argument blocks and launchers.
// Host code (api.cpp) fills these after validating the C-ABI arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

enum InType : int { kInF32 = 0, kInBF16 = 1, kInFP8 = 2 };
// prefill addressing modes: batch [B, H, S, d]; varlen (cu_seqlens); paged
// (K/V rows through a block table, Lq = sq, Lk = seqlens_k)
enum PrefillMode : int { kPrefillBatch = 0, kPrefillVarlen = 1, kPrefillPaged = 2, kPrefillVarlenPaged = 3 };
// logit bias kinds (the values of attn_bias_t)
enum BiasKind : int { kBiasNone = 0, kBiasElem = 1, kBiasAlibi = 2 };

// Prefill (one workgroup = 128 packed query rows of one sequence and kv-head).
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;                 // nullable
  // element strides: batch (0 in varlen mode), head, row/token
  int64_t q_sb, q_sh, q_sr;
  int64_t k_sb, k_sh, k_sr;   // paged mode: page, head, slot
  int64_t v_sb, v_sh, v_sr;
  int64_t o_sb, o_sh, o_sr;
  int64_t lse_sb, lse_sh;     // lse index = b*lse_sb + h*lse_sh + token
  const int32_t* seqused_q;   // batch mode, nullable
  const int32_t* seqused_k;   // batch mode, nullable; paged mode: seqlens_k (required)
  const int32_t* block_table; // paged mode: [nz][bt_stride] page ids
  int64_t bt_stride;
  int page_size;              // paged mode: a multiple of 64 (one page per 64-key tile)
  const int32_t* cu_q;        // varlen mode (non-null selects varlen)
  const int32_t* cu_k;
  int sq, sk;                 // batch-mode extents
  int hq, hkv, ratio;
  int n_qtiles;               // packed-row tiles per (sequence, kv-head)
  int nz;                     // batch entries (batch mode) or sequences (varlen); set by the launcher
  int items_x;                // workgroups per XCD of the launch; set by the launcher
  int cu_per_xcd;             // CUs per XCD of the device; set by the launcher
  float c_exp2;               // multiplier taking the kernel's logit domain to log2 units
  float softcap_pre;          // softcap: raw dot * softcap_pre = (scaled logit) / cap
  float softcap_post;         // softcap: cap * log2(e)
  float o_mul;                // applied to the normalised O: fp8 value descale, fp8-output scale
  int out_fp8;                // O stored as saturated E4M3FN (else bf16)
  int wl, wr;                 // window (-1 = unbounded)
  int sink_size;              // keys j < sink_size ignore the left bound
  const float* sink_logits;   // nullable [hq]: extra softmax-denominator term per q-head
  int bias_type;              // attn_bias_t
  const float* bias;          // ALiBi slopes or elementwise values (see attn.h)
  int64_t bias_sb, bias_sh, bias_sr;  // elementwise: batch (group mode: unused), head, query row
  float bias_mul;             // natural-log logit units -> the kernel's logit units
  const int32_t* cache_idx;   // batch mode, nullable: K/V batch entry of each batch entry
  int cache_count;            // K/V batch entries (indices outside [0, cache_count) read no keys)
  int min_seqlen_q;           // varlen mode: sequences with Lq <= min_seqlen_q are skipped
  int v_colmajor;             // batch or paged mode, equal head dims: V keys contiguous (within a page),
                              // v_sr = head-dim row stride
  const int32_t* kv_start;    // varlen-paged mode, nullable: logical position of each sequence's first key
};

// Split-KV decode (one workgroup = one split of one request and kv-head).
struct DecodeArgs {
  const void* q;
  const void* k;              // contiguous K, or the page pool
  const void* v;
  int64_t q_sb, q_sh, q_sr;
  int64_t k_sb, k_sh, k_sr;   // contiguous: batch, head, row. paged: page, head, slot
  int64_t v_sb, v_sh, v_sr;
  const int32_t* seqlens_k;   // per-request Lk (paged: required; contiguous: nullable)
  const int32_t* seqused_q;   // contiguous only, nullable: per-request used query rows Lq <= sq
  int v_colmajor;             // V keys contiguous (paged: within a page), v_sr = head-dim row stride
  const int32_t* block_table; // paged only
  int64_t bt_stride;
  int page_size;
  int sk;                     // contiguous: Lk when seqlens_k is null
  int sq, hq, hkv, ratio, m_rows;  // m_rows = sq * ratio (<= 16)
  int split_tokens, n_splits;
  float c_exp2;
  float softcap_pre, softcap_post;
  int wl, wr;
  int sink_size;              // keys j < sink_size ignore the left bound
  const float* alibi;         // nullable: ALiBi slope of (b, q-head) at alibi[b*alibi_sb + hq]
  int64_t alibi_sb;
  const float* bias;          // nullable: elementwise bias of (b, q-head, query row, key) at
  int64_t bias_sb, bias_sh, bias_sr;  // bias[b*bias_sb + hq*bias_sh + row*bias_sr + key]
  float bias_mul;             // natural-log logit units -> the kernel's logit units
  float* part_o;              // [B][hkv][n_splits][m_rows][dv] fp32
  float* part_lse;            // [B][hkv][n_splits][m_rows]
  int fp8;                    // Q/K/V stored as E4M3FN (descales folded into c_exp2 and the combine)
  const int32_t* cache_idx;   // contiguous K/V only, nullable: K/V batch entry of each request
  int cache_count;
};

struct CombineArgs {
  const float* part_o;
  const float* part_lse;
  void* o;
  float* lse;                 // nullable, [B, hq, sq]
  int64_t o_sb, o_sh, o_sr;
  const int32_t* seqlens_k;   // nullable (then sk)
  const int32_t* seqused_q;   // nullable (then sq): rows at or past it are not written
  int sk;
  int B, sq, hq, hkv, ratio, m_rows, split_tokens, n_splits;
  float o_mul;                // applied to the normalised O (fp8-output scale)
  int out_fp8;                // O stored as saturated E4M3FN (else bf16)
  const float* sink_logits;   // nullable [hq]: extra softmax-denominator term per q-head
  const int32_t* cache_idx;   // as DecodeArgs (an out-of-range entry has no keys)
  int cache_count;
  int no_keys;                // K or V is NULL: every row has no keys
};

// fp32 path (batch mode).
struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int64_t q_sb, q_sh, q_sr;
  int64_t k_sb, k_sh, k_sr;
  int64_t v_sb, v_sh, v_sr;
  int64_t o_sb, o_sh, o_sr;
  const int32_t* seqused_q;
  const int32_t* seqused_k;
  int B, sq, sk, hq, hkv, ratio;
  float c_exp2, softcap_pre, softcap_post;
  int wl, wr;
};

int prefill_rows_per_tile(int in_type);  // packed query rows per prefill workgroup
int64_t prefill_workgroups(const PrefillArgs& a, int nz);  // workgroups of launch_prefill(a, .., nz, ..)
// d: head dim of Q and K; dv: head dim of V and O ({64, 128} each; paged mode: dv == d)
hipError_t launch_prefill(const PrefillArgs& a, int d, int dv, int in_type, int mode, int batch_or_seqs,
                          hipStream_t stream);
// d: head dim of Q and K; dv: head dim of V and O
hipError_t launch_decode(const DecodeArgs& a, const CombineArgs& c, int d, int dv, bool paged, int B,
                         hipStream_t stream);
hipError_t launch_f32(const F32Args& a, int d, hipStream_t stream);
int64_t f32_workgroups(const F32Args& a);  // workgroups of launch_f32(a, ..)

}  // namespace attn
