/*
 * attn.h - C ABI of the MI355X (gfx950) fused attention forward library
 * (libattn.so).
 *
 * One operation, four entry points: batch (attn_fwd), packed sequences
 * (attn_fwd_varlen), a paged KV cache (attn_fwd_paged) and packed sequences
 * over a paged KV cache (attn_fwd_varlen_paged). For every query row i of
 * sequence b and q-head h, with kv-head g = h / (Hq / Hkv) and used lengths
 * Lq, Lk:
 *
 *     S[i,j]   = scale * dot(Q[b,h,i,:], K[b,g,j,:])            (0 <= j < Lk)
 *     S[i,j]   = softcap * tanh(S[i,j] / softcap)               if softcap > 0
 *     visible  = (wl < 0 || j >= i + Lk - Lq - wl) && (wr < 0 || j <= i + Lk - Lq + wr)
 *     O[b,h,i] = sum_j softmax_j(S[i, visible]) * V[b,g,j,:]
 *     LSE[b,h,i] = ln sum_{visible j} exp(S[i,j])
 *
 * This is the math contract printed at the top of the Composable Kernel page
 * "fmha_fwd_pagedkv_kernel.hpp Source File" (S = Q K^T, S' = S * scale,
 * P = softmax, O = P V), with the logit soft-cap and window-mask arguments of the
 * same page's kernel-argument structs (FmhaFwdLogitsSoftCapKargs, FmhaFwdMaskKargs),
 * its grouped-query head map (kv head = q head / nhead_ratio_qk), and the LSE
 * output and empty-row convention of the flash-attention page
 * "hopper/epilogue_fwd.hpp" (CollectiveEpilogueFwd::store / store_zero: a row
 * with no visible key gets O = 0 and LSE = -inf). The mask diagonal is aligned
 * bottom-right (offset Lk - Lq), so causal = (wl, wr) = (-1, 0) and a single
 * decode query sees every key.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers; every buffer is allocated and
 *     owned by the caller. The library never allocates, frees or synchronises:
 *     a call validates its arguments on the host, enqueues kernels on `stream`
 *     (a hipStream_t; NULL = the legacy default stream) and returns.
 *   - Strides are in ELEMENTS of the stored type; the head dimension d is
 *     contiguous (unit stride). Every tensor base pointer must be 16-byte
 *     aligned and every stride a multiple of 16 bytes. K and V may be NULL
 *     when there are no keys (attn_fwd with sk = 0, attn_fwd_varlen with
 *     max_seqlen_k = 0): every row then gets O = 0 and LSE = -inf (or the sink
 *     logit).
 *   - Supported: d (the head dim of Q and K) in {64, 128}, head_dim_v (of V
 *     and O; attn_params_t) in {64, 128}; (in_dtype, out_dtype) in {(F32, F32),
 *     (BF16, BF16), (BF16, FP8_E4M3), (FP8_E4M3, BF16), (FP8_E4M3, FP8_E4M3)}.
 *     FP8 output is E4M3FN with a per-tensor scale (o_scale). F32 runs in batch
 *     mode only (a plain vector-ALU kernel). The split-KV decode path (short
 *     query blocks: sq * Hq / Hkv <= 16 in attn_fwd and attn_fwd_paged) takes
 *     BF16 or FP8_E4M3 (FP8: Q K^T on fp8 matrix cores, V widened exactly to
 *     bf16 for P V). FP8 means OCP E4M3FN; the value of a stored byte x is
 *     e4m3(x) * descale of its tensor.
 *   - lse may be NULL (not stored). LSE is fp32, natural log.
 *   - Rows at or beyond a sequence's used query length are never written, in O
 *     or LSE (the predicated stores of the flash-attention epilogue page).
 *     K/V rows at or beyond the used key length, block-table entries past
 *     ceil(Lk / page_size) and slots past Lk in the last page are never read as
 *     keys.
 *   - Device-resident metadata (seqused, cu_seqlens, seqlens_k, block tables)
 *     is a precondition: monotone, in range, page ids < num_pages. Violating it
 *     is undefined behaviour (it is not checked on the device).
 *     With the environment variable ATTN_VALIDATE set (to anything but "" or
 *     "0", read on every call) each call first waits for its stream, copies
 *     that metadata to the host and checks it:
 *       seqused_q/k within [0, sq] / [0, sk] (cache_batch_idx may hold any
 *       index, see attn_params_t);
 *       cu_seqlens starting >= 0 and non-decreasing, every length within
 *       max_seqlen_q / max_seqlen_k, cu_seqlens_q[n] <= total_q;
 *       seqlens_k, and kv_start + seqlens_k, within block_table_stride *
 *       page_size;
 *       every block-table entry that a used key falls in within [0, num_pages).
 *     A violation returns ATTN_EINVAL with no launch. The check synchronises,
 *     so it is a debugging aid, not for graph capture.
 *   - Results are deterministic: the same call gives the same bits. Calls that
 *     differ only in addressing (paged vs contiguous KV with the same logical
 *     contents and the same split size; varlen vs padded batch with seqused)
 *     give bit-identical results on every valid row.
 *   - Return value: ATTN_OK, or an error status with no kernel launched (except
 *     ATTN_ELAUNCH, reported when the runtime rejects a launch). attn_last_error()
 *     then describes it.
 *   - In-tile byte offsets are 32-bit: 64 rows of K or V (the prefill tile), or
 *     32 rows (a split-KV granule), must span less than 2 GiB, i.e.
 *     64 * row stride * element size < 2^31 (32 * ... on the decode path);
 *     a larger row stride is ATTN_EINVAL.
 *   - With the environment variable ATTN_LOG set (to anything but "" or "0",
 *     read on every call) each accepted call writes one line to stderr: the
 *     entry point, the path taken (prefill, split-KV decode, f32), the types,
 *     shape and mask, the launch grid and the split plan (the analogue of the
 *     Composable Kernel page's GetName / PrintParameters of a kernel instance);
 *     each refused or failed call writes "attn: error <status>: <message>".
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_F32 = 0,      /* IEEE binary32 */
  ATTN_BF16 = 1,     /* bfloat16 */
  ATTN_FP8_E4M3 = 2  /* OCP FP8 E4M3FN, per-tensor descale */
} attn_dtype_t;

typedef enum {
  ATTN_BIAS_NONE = 0,
  ATTN_BIAS_ELEMENTWISE = 1, /* per (batch, q-head, query, key) values */
  ATTN_BIAS_ALIBI = 2        /* per (batch, q-head) slopes */
} attn_bias_t;

/* Layout of V (the page's VLayout: row-major [.., seqlen_k, hdim_v] or
 * column-major [.., hdim_v, seqlen_k]). */
typedef enum {
  ATTN_V_ROW_MAJOR = 0,      /* V[b, h, j, c] at b*stride[0] + h*stride[1] + j*stride[2] + c */
  ATTN_V_COL_MAJOR = 1       /* V[b, h, j, c] at b*stride[0] + h*stride[1] + c*stride[2] + j */
} attn_v_layout_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_EINVAL = 1,     /* bad argument: NULL pointer, bad size, stride, alignment */
  ATTN_ENOTSUP = 2,    /* valid but not implemented (head dim, dtype pair, mode) */
  ATTN_EWORKSPACE = 3, /* workspace smaller than attn_workspace_bytes() */
  ATTN_ELAUNCH = 4     /* the HIP runtime reported an error at launch */
} attn_status_t;

typedef struct {
  int in_dtype;        /* attn_dtype_t of Q, K and V */
  int out_dtype;       /* attn_dtype_t of O */
  float scale;         /* multiplies q.k (scale_s of the Composable Kernel page) */
  float softcap;       /* > 0 enables cap * tanh(s / cap); <= 0 disables */
  int window_left;     /* -1 = unbounded; causal = (-1, 0) */
  int window_right;
  float q_descale;     /* FP8 only: stored value * descale = real value; else ignored */
  float k_descale;
  float v_descale;
  int kv_split_tokens; /* decode path: keys per split-KV work unit, a multiple of 64
                          in [64, 2048]; 0 = choose from the shape and input type (the largest
                          power of two up to 2048, 1024 for FP8, that still gives >= 4096 units).
                          Calls that must agree bit for bit pass the same value (or the same shape
                          and type with 0). */
  int sink_size;       /* streaming sink keys (sink_size of the Composable Kernel page's
                          mask): keys j < sink_size are visible to every row whose right
                          bound reaches them, whatever window_left says; 0 = none */
  const float* sink_logits; /* nullable DEVICE fp32 [Hq]: per-q-head sink logit (the page's
                          sink_ptr), in the units of the scaled, soft-capped logits. It adds
                          exp(sink) to every row's softmax denominator with no value row, so
                          a row with no visible key gets O = 0, LSE = sink. Not capped.
                          BF16 / FP8 only (F32: ATTN_ENOTSUP), as is sink_size > 0. */
  int bias_type;       /* attn_bias_t: an additive logit bias S'' = S' + Bias (the math
                          contract of the Composable Kernel page), added after the scale and
                          the soft-cap, before the mask. BF16 / FP8 only. */
  const float* bias;   /* DEVICE fp32. ALIBI: the slope of (b, q-head h) at
                          bias[b*bias_stride[0] + h] (bias_stride[0] = 0: one slope per head
                          for every b); the bias of key j for query row i is
                          -slope * |i + Lk - Lq - j| (bottom-right aligned). In varlen mode b
                          is the sequence index. ELEMENTWISE (every entry point and path,
                          the bias kernel arguments of the Composable Kernel page): in batch
                          and paged modes the bias of (b, h, i, j) is at
                          bias[b*bias_stride[0] + h*bias_stride[1] + i*bias_stride[2] + j],
                          j the logical key index (its token position; paged: whatever page
                          holds it); in the varlen modes (group mode) the bias of q-head h,
                          packed query token t and the sequence's key j is at
                          bias[h*bias_stride[1] + t*bias_stride[2] + j] (the page's
                          query_start * stride_bias row offset; bias_stride[0] unused). Only
                          elements of used rows (i < Lq) and keys (j < Lk) are read, as
                          aligned 16-byte blocks of 4 keys: the base must be 16-byte aligned
                          and every stride a multiple of 4 (0 broadcasts that index). */
  int64_t bias_stride[3];
  float o_scale;       /* FP8 output only: O is stored as the saturating E4M3FN conversion
                          (round to nearest even, clamped to +-448) of O * o_scale, the
                          page's scale_o with its saturating O conversion; else ignored */
  const int32_t* cache_batch_idx; /* attn_fwd only (batch mode), nullable DEVICE int32 [B]: the
                          K/V batch entry that batch entry b reads (the cache_batch_idx of the
                          Composable Kernel page's batch-mode arguments), so K and V are
                          [cache_batch_count, Hkv, sk, d] caches and Q, O, LSE, seqused_q/k
                          and the bias keep index b. An index outside [0, cache_batch_count)
                          gives entry b no keys (O = 0, LSE = -inf or its sink logit): it is
                          never dereferenced. BF16 / FP8 only. */
  int cache_batch_count; /* K/V batch entries when cache_batch_idx is set (>= 1) */
  int min_seqlen_q;    /* attn_fwd_varlen only: a sequence with Lq <= min_seqlen_q is skipped
                          and its O and LSE rows are left untouched (the page's min_seqlen_q
                          of group mode); 0 skips only empty sequences, i.e. nothing. */
  int head_dim_v;      /* head dim of V and O (the page's hdim_v); 0 = the d argument (hdim_q).
                          64 or 128. A value different from d is supported by attn_fwd (prefill
                          and split-KV decode shapes alike) and by attn_fwd_varlen, BF16 / FP8
                          only; V's rows then have head_dim_v elements and O's rows too. The
                          paged entry points need v_pool_stride for it (the pools' rows differ). */
  int v_layout;        /* attn_v_layout_t. ATTN_V_COL_MAJOR (keys contiguous, the V stride[2]
                          the stride between head-dim rows; the page's non-row-major VLayout)
                          is supported by attn_fwd (prefill and split-KV decode shapes) and by
                          attn_fwd_paged (prefill and decode shapes: each V page of each
                          kv-head is [head_dim_v, page_size], keys contiguous, addressed as
                          pool + page*v_pool_stride[0] + head*v_pool_stride[1] +
                          c*v_pool_stride[2] + slot; v_pool_stride is required), with BF16 or
                          FP8_E4M3 inputs and head_dim_v = d. The row length (sk, or
                          page_size) must be a multiple of 8 keys (BF16) or 16 keys (FP8),
                          and (head_dim_v - 1) * row stride * elem + 64 * elem < 2^31. Keys
                          past the used length may hold any bits: they are never used.
                          attn_fwd_varlen takes it too: V is then [Hkv, head_dim_v, total_k],
                          keys contiguous along the packed token axis, addressed as
                          v + head*v_stride[1] + c*v_stride[0] + token; every cu_seqlens_k entry
                          must be a multiple of 8 keys (BF16) or 16 keys (FP8), so that each
                          16-byte chunk of keys belongs to one sequence. These are device
                          metadata: ATTN_VALIDATE refuses a call that breaks the rule, and
                          without it a sequence whose key offset or count is off that grid
                          reads no key and gets NaN rows of O and LSE. Not supported by
                          attn_fwd_varlen_paged (ATTN_ENOTSUP). */
  int64_t v_pool_stride[3]; /* attn_fwd_paged / attn_fwd_varlen_paged: the V pool's {page, head,
                          slot} element strides when they differ from the K pool's (required with
                          head_dim_v != d); all zero = kv_stride for both pools. Same rules as
                          kv_stride (multiples of 16 bytes, d contiguous). */
} attn_params_t;

/* Fill *p with defaults: BF16 in/out, the given scale, no soft-cap, no mask,
 * descales 1, automatic split size, no sinks, no bias, o_scale 1, no cache
 * batch index, min_seqlen_q 0, head_dim_v 0 (= d), row-major V. */
void attn_params_init(attn_params_t* p, float scale);

/*
 * Batch mode. Q [B, Hq, sq, d], K [B, Hkv, sk, d], V [B, Hkv, sk, dv] and
 * O [B, Hq, sq, dv] (dv = head_dim_v, default d), each addressed as
 * base + b*stride[0] + head*stride[1] + row*stride[2] + c (column-major V: see
 * v_layout).
 * lse (nullable) is a dense fp32 [B, Hq, sq] array.
 * seqused_q / seqused_k (nullable, int32 [B] on the device) give per-batch used
 * lengths Lq <= sq, Lk <= sk; NULL means Lq = sq, Lk = sk. Both the prefill and
 * the split-KV decode paths honour them (the mask diagonal sits on the used
 * rows; rows at or past Lq are not written).
 * Short query blocks (sq * Hq / Hkv <= 16) run the split-KV decode path, which
 * needs `workspace` of attn_workspace_bytes() bytes (else workspace may be NULL).
 * (Batch-mode arguments of the Composable Kernel page's MakeKargs; the
 * [B, H, N, d] tensors of the FlashAttention-2 mma page's entry point.)
 */
attn_status_t attn_fwd(const attn_params_t* p,
                       const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int Hq, int Hkv, int sq, int sk, int d,
                       const int64_t q_stride[3], const int64_t k_stride[3],
                       const int64_t v_stride[3], const int64_t o_stride[3],
                       const int32_t* seqused_q, const int32_t* seqused_k,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Varlen (group) mode. n sequences packed along the token axis:
 * Q [total_q, Hq, d], K [total_k, Hkv, d], V [total_k, Hkv, dv], O [total_q, Hq, dv]
 * (dv = head_dim_v, default d), addressed as base + token*stride[0] + head*stride[1] + c (column-major V:
 * see v_layout). Sequence s owns query tokens
 * cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 and key tokens likewise
 * (int32 [n+1] device arrays, the seqstart_q/k pointers of the Composable Kernel
 * page's group-mode MakeKargs). max_seqlen_q / max_seqlen_k bound every
 * sequence's lengths (they size the grid). lse (nullable) is fp32 [Hq, total_q].
 * Needs no workspace.
 */
attn_status_t attn_fwd_varlen(const attn_params_t* p,
                              const void* q, const void* k, const void* v, void* o, float* lse,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int n, int total_q, int max_seqlen_q, int max_seqlen_k,
                              int Hq, int Hkv, int d,
                              const int64_t q_stride[2], const int64_t k_stride[2],
                              const int64_t v_stride[2], const int64_t o_stride[2],
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Paged-KV mode. Q [B, Hq, sq, d] and O [B, Hq, sq, dv] strided as in attn_fwd;
 * K and V live in page pools of num_pages pages of page_size tokens,
 * addressed as pool + page*kv_stride[0] + head*kv_stride[1] + slot*kv_stride[2] + c
 * (64-bit offsets; the V pool with v_pool_stride instead when that is set). Token t of request b is slot t % page_size of page
 * block_table[b*block_table_stride + t / page_size] (the page-block navigator
 * of the Composable Kernel page: block_table_ptr, batch_stride_block_table,
 * page_block_size). seqlens_k (int32 [B], device) gives Lk per request;
 * Lq = sq (bottom-right aligned mask). block_table_stride * page_size bounds
 * every Lk. lse (nullable) is fp32 [B, Hq, sq].
 *   - Decode shapes (sq * Hq / Hkv <= 16): BF16 or FP8_E4M3, page_size a multiple of
 *     32, split-KV kernel + combine; needs a workspace of attn_workspace_bytes()
 *     bytes with max_seqlen_k = block_table_stride * page_size.
 *   - Longer query blocks (paged prefill, e.g. chunked prefill into a cache):
 *     BF16 or FP8_E4M3 (with descales), page_size a multiple of 64 (one page per
 *     64-key tile), the prefill kernel; no workspace.
 */
attn_status_t attn_fwd_paged(const attn_params_t* p,
                             const void* q, const void* k_pool, const void* v_pool,
                             void* o, float* lse,
                             const int32_t* block_table, int block_table_stride,
                             const int32_t* seqlens_k,
                             int B, int sq, int Hq, int Hkv, int d,
                             int page_size, int num_pages,
                             const int64_t q_stride[3], const int64_t kv_stride[3],
                             const int64_t o_stride[3],
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Group (varlen) mode over a paged KV cache, with optional per-sequence key
 * offsets ("gappy" group mode of the Composable Kernel page: with is_gappy,
 * seqstart_k[b] is the logical position of the sequence's first key in its
 * page list, kv_l2p_offset, and seqlen_k_ptr[b] its key count).
 * Q [total_q, Hq, d] and O [total_q, Hq, d] as in attn_fwd_varlen, sequence s
 * owning query tokens cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1; lse (nullable)
 * fp32 [Hq, total_q]. The pools are addressed as in attn_fwd_paged. Sequence s
 * has Lk = seqlens_k[s] keys; key j is token kv_start[s] + j of block table row
 * s (kv_start NULL: 0), i.e. slot (kv_start[s] + j) % page_size of page
 * block_table[s*block_table_stride + (kv_start[s] + j) / page_size];
 * kv_start[s] + Lk <= block_table_stride * page_size. Bottom-right aligned mask
 * per sequence. page_size must be a multiple of 64; kv_start[s] may be any
 * non-negative position (a 64-key tile then spans at most two pages). A
 * sequence whose kv_start is negative is not computed: its O and LSE rows are
 * set to NaN and no key of it is read. BF16 or FP8_E4M3 inputs, the
 * prefill kernel for every query length; no workspace. Not supported with
 * cache_batch_idx or column-major V. head_dim_v != d needs v_pool_stride.
 */
attn_status_t attn_fwd_varlen_paged(const attn_params_t* p,
                                    const void* q, const void* k_pool, const void* v_pool,
                                    void* o, float* lse,
                                    const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                                    const int32_t* kv_start,
                                    const int32_t* block_table, int block_table_stride,
                                    int n, int total_q, int max_seqlen_q,
                                    int Hq, int Hkv, int d, int page_size, int num_pages,
                                    const int64_t q_stride[2], const int64_t kv_stride[3],
                                    const int64_t o_stride[2], void* stream);

/*
 * attn_fwd_paged without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Arguments, layouts, results and errors are those of
 * attn_fwd_paged (the same kernels, bit-identical results). The split-KV
 * partials go to a 64 MiB array that the library keeps on each GPU it runs on
 * until the process ends (its address is looked up on the first call on a
 * device, so make one call on a device before capturing calls in a graph);
 * the call itself allocates nothing. A shape whose partials need more
 * than 64 MiB (attn_workspace_bytes() > 64 MiB) is refused with
 * ATTN_EWORKSPACE before any launch. Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (work queued on two streams, or from
 * two threads) race on it and must be serialised by the caller. The array
 * keeps the last call's contents; each call writes every partial it reads.
 */
attn_status_t attn_fwd_paged_noalloc(const attn_params_t* p,
                                     const void* q, const void* k_pool, const void* v_pool,
                                     void* o, float* lse,
                                     const int32_t* block_table, int block_table_stride,
                                     const int32_t* seqlens_k,
                                     int B, int sq, int Hq, int Hkv, int d,
                                     int page_size, int num_pages,
                                     const int64_t q_stride[3], const int64_t kv_stride[3],
                                     const int64_t o_stride[3], void* stream);

/*
 * Workspace bytes needed by attn_fwd / attn_fwd_paged for this shape (0 when
 * the shape takes the prefill path). max_seqlen_k is sk for attn_fwd and
 * block_table_stride * page_size for attn_fwd_paged. Returns 0 for invalid
 * shapes as well; the entry point then reports the error.
 * The workspace holds the split-KV partials: an fp32 O of [B, Hkv, n_splits,
 * sq * Hq / Hkv, dv] and an fp32 LSE of [B, Hkv, n_splits, sq * Hq / Hkv], the
 * num_splits axis that the O and LSE tensors of the flash-attention epilogue
 * page "hopper/epilogue_fwd.hpp" carry (CollectiveEpilogueFwd: its shapes and
 * strides have a split dimension indexed by split_idx), reduced here by the
 * library's own combine kernel. Owned by the caller; contents are scratch.
 */
size_t attn_workspace_bytes(const attn_params_t* p, int B, int Hq, int Hkv, int sq, int d,
                            int max_seqlen_k);

/* Number of split-KV work units per (request, kv-head) the decode path uses for
 * this shape (1 if it takes the prefill path): the extent of the num_splits
 * axis of the partial O / LSE described above (CollectiveEpilogueFwd of the
 * flash-attention epilogue page). */
int attn_num_splits(const attn_params_t* p, int B, int Hq, int Hkv, int sq, int max_seqlen_k);

/* Text describing the last non-OK status returned on the calling thread. The
 * FlashAttention-2 mma page's entry point refuses unsupported input (head dim,
 * dtype) by throwing with a message; a C ABI cannot throw, so each entry point
 * returns a status and leaves the message here (thread-local, overwritten by
 * the next failing call on the same thread). */
const char* attn_last_error(void);

/* Library version string. */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
