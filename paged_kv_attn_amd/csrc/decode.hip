// Split-KV decode for short query blocks (sq * Hq/Hkv <= 16 packed rows), with
// the keys either contiguous or in a paged pool, plus the split combine.
//
// Work unit = (split, kv-head, request). A split is a fixed, key-aligned range
// of split_tokens keys, so a paged call and a contiguous call with the same
// logical keys and the same split size perform identical arithmetic in the same
// order and give identical bits. Inside a workgroup, wave w takes the 32-key
// granules w, w+4, w+8, ... of its split; every granule lies in one page
// (page_size is a multiple of 32), whose physical id is read once per granule
// from the block table (the page-block navigator of the Composable Kernel page
// "fmha_fwd_pagedkv_kernel.hpp Source File": one table row per request,
// page_block_size tokens per page, 64-bit page base + in-page offset).
//
// Math per granule, on v_mfma_f32_16x16x32_bf16 with the <= 16 packed query
// rows (request position x q-heads of this kv-head) as the MFMA column
// dimension: S^T = K Q^T with K fed straight from global memory in A-operand
// layout (128-bit loads along d), online softmax over keys (max / sum across
// the four 16-lane groups), O^T += V^T P^T with V staged row-major in the
// wave's own LDS slice and read back transposed (ds_read_b64_tr_b16).
//
// The four waves' (m, l, O) are merged through LDS into one partial per split,
// stored normalised with its log-sum-exp (the num_splits axis of O / LSE in the
// flash-attention epilogue page "hopper/epilogue_fwd.hpp"). The combine kernel
// then forms, per query row and in a fixed split order,
//     LSE = log sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s,
// which equals attention over the union of the splits' keys.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kGran = 32;        // keys per wave step
constexpr int kVPitch = 144;     // bf16 elements per V row in LDS (72 dwords)
constexpr int kVStage = kGran * kVPitch * 2;  // bytes per wave

template <int D>
struct DTr {
  static constexpr int kSteps = D / 32;       // k-steps of S^T = K Q^T (32 d each)
  static constexpr int kDBlocks = D / 16;     // 16-row blocks of O^T
  static constexpr int kChunks = D / 8;       // 16-byte chunks per K/V row
  static constexpr int kVLoads = kGran * kChunks / 64;
  static constexpr int kKeyStep = 64 / kChunks;
  static constexpr int kMergeBytes = kWaves * (16 * D * 4 + 2 * 16 * 4);
  static constexpr int kSmem = (kWaves * kVStage > kMergeBytes) ? kWaves * kVStage : kMergeBytes;
};

__device__ __forceinline__ float xor_shfl(float x, int mask) {
  const int lane = threadIdx.x & 63;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(((lane ^ mask) << 2), __builtin_bit_cast(int, x)));
}

template <int D, bool PAGED, bool MASK, bool SOFTCAP>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  using Tr = DTr<D>;
  __shared__ __attribute__((aligned(16))) char smem[Tr::kSmem];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int Lk = a.seqlens_k ? a.seqlens_k[b] : a.sk;
  const int t0 = split * a.split_tokens;
  if (t0 >= Lk) return;  // empty split: the combine reads only ceil(Lk / split_tokens) partials
  const int t1 = min(Lk, t0 + a.split_tokens);

  // packed query row of this lane's MFMA column
  const int qc = lane & 15;
  const int j4 = lane >> 4;
  const int ratio = a.ratio;
  const bool row_ok = qc < a.m_rows;
  const int pos = qc / ratio;
  const int hq = g * ratio + qc % ratio;
  const int off = Lk - a.sq;
  int lim_lo = 0, lim_hi = Lk - 1;
  if (MASK) {
    if (a.wr >= 0) lim_hi = min(Lk - 1, pos + off + a.wr);
    if (a.wl >= 0) lim_lo = pos + off - a.wl;
  }

  // Q^T as the B operand: lane (column qc, group j4) holds Q[qc][32s + 8 j4 .. +7]
  U128 qf[Tr::kSteps];
  {
    const char* qp = (const char*)a.q + ((int64_t)b * a.q_sb + (int64_t)hq * a.q_sh + (int64_t)pos * a.q_sr) * 2;
#pragma unroll
    for (int s = 0; s < Tr::kSteps; ++s) qf[s] = row_ok ? *(const U128*)(qp + (32 * s + 8 * j4) * 2) : U128{0, 0, 0, 0};
  }

  char* vstage = smem + wave * kVStage;
  const int L = lane & 15;
  const int v_lane = ((4 * j4 + (L >> 2)) * kVPitch + 4 * (L & 3)) * 2;
  const int vch = lane % Tr::kChunks;
  const int vkey = lane / Tr::kChunks;

  const float c = a.c_exp2;
  float m_run = kNegInf;
  float l_run = 0.0f;
  f32x4 acc[Tr::kDBlocks];
#pragma unroll
  for (int i = 0; i < Tr::kDBlocks; ++i) acc[i] = f32x4{};

  for (int gs = t0 + wave * kGran; gs < t1; gs += kWaves * kGran) {
    // base of this granule's 32 key rows (64-bit page base + in-page offset)
    const char* kbase;
    const char* vbase;
    if (PAGED) {
      const int page = a.block_table[(int64_t)b * a.bt_stride + gs / a.page_size];
      const int slot = gs % a.page_size;
      kbase = (const char*)a.k + ((int64_t)page * a.k_sb + (int64_t)g * a.k_sh + (int64_t)slot * a.k_sr) * 2;
      vbase = (const char*)a.v + ((int64_t)page * a.v_sb + (int64_t)g * a.v_sh + (int64_t)slot * a.v_sr) * 2;
    } else {
      kbase = (const char*)a.k + ((int64_t)b * a.k_sb + (int64_t)g * a.k_sh + (int64_t)gs * a.k_sr) * 2;
      vbase = (const char*)a.v + ((int64_t)b * a.v_sb + (int64_t)g * a.v_sh + (int64_t)gs * a.v_sr) * 2;
    }
    const int nvalid = t1 - gs;  // keys of this granule below Lk (may exceed 32)

    // K as the A operand: lane (key 16kb + L, group j4) holds K[key][32s + 8 j4 .. +7]
    U128 kf[2][Tr::kSteps];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = 16 * kb + L;
#pragma unroll
      for (int s = 0; s < Tr::kSteps; ++s)
        kf[kb][s] = key < nvalid ? *(const U128*)(kbase + (int64_t)key * a.k_sr * 2 + (32 * s + 8 * j4) * 2)
                                 : U128{0, 0, 0, 0};
    }
    // V rows (zero past Lk), staged row-major in this wave's LDS slice
    U128 vf[Tr::kVLoads];
#pragma unroll
    for (int i = 0; i < Tr::kVLoads; ++i) {
      const int key = vkey + i * Tr::kKeyStep;
      vf[i] = key < nvalid ? *(const U128*)(vbase + (int64_t)key * a.v_sr * 2 + vch * 16) : U128{0, 0, 0, 0};
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // previous granule's LDS reads stay before these writes
#pragma unroll
    for (int i = 0; i < Tr::kVLoads; ++i) {
      const int key = vkey + i * Tr::kKeyStep;
      *(U128*)(vstage + (key * kVPitch + vch * 8) * 2) = vf[i];
    }

    // S^T = K Q^T: lane (column qc, group j4) gets keys 16kb + 4 j4 + r
    f32x4 st[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      st[kb] = f32x4{};
#pragma unroll
      for (int s = 0; s < Tr::kSteps; ++s) st[kb] = mfma16_bf16(as_bf16x8(kf[kb][s]), as_bf16x8(qf[s]), st[kb]);
    }
    float mt = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = st[kb][r];
        if (SOFTCAP) x = a.softcap_post * tanh_fast(x * a.softcap_pre);
        const int j = gs + 16 * kb + 4 * j4 + r;
        x = (j >= lim_lo && j <= lim_hi) ? x : kNegInf;
        st[kb][r] = x;
        mt = fmaxf(mt, x);
      }
    }
    mt = fmaxf(mt, xor_shfl(mt, 16));
    mt = fmaxf(mt, xor_shfl(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = fast_exp2((m_run - m_use) * c);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int i = 0; i < Tr::kDBlocks; ++i) acc[i] *= alpha;
    }
    l_run *= alpha;
    m_run = m_new;
    const float mc = m_use * c;
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = fast_exp2(__builtin_fmaf(st[i >> 2][i & 3], c, -mc));
      l_run += p[i];
    }
    // P^T as the B operand: slot 4kb + r <-> key 16kb + 4 j4 + r
    const U128 pu{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
    const bf16x8 pb = as_bf16x8(pu);
    // O^T += V^T P^T: transpose reads give lane (d, j4) V[16kb + 4 j4 + r][d]
#pragma unroll
    for (int dblk = 0; dblk < Tr::kDBlocks; ++dblk) {
      const char* vp = vstage + v_lane + 16 * dblk * 2;
      const U64 v0 = lds_read_tr16(vp);
      const U64 v1 = lds_read_tr16(vp + 16 * kVPitch * 2);
      acc[dblk] = mfma16_bf16(as_bf16x8(v0, v1), pb, acc[dblk]);
    }
  }

  // ---- merge the four waves' running states through LDS ----
  l_run += xor_shfl(l_run, 16);
  l_run += xor_shfl(l_run, 32);
  __syncthreads();  // all waves done with their V slices
  float* mo = (float*)smem;                           // [wave][16][D]
  float* mm = mo + kWaves * 16 * D;                   // [wave][16]
  float* ml = mm + kWaves * 16;                       // [wave][16]
#pragma unroll
  for (int dblk = 0; dblk < Tr::kDBlocks; ++dblk)
    *(f32x4*)(mo + (wave * 16 + qc) * D + 16 * dblk + 4 * j4) = acc[dblk];
  if (j4 == 0) {
    mm[wave * 16 + qc] = m_run;
    ml[wave * 16 + qc] = l_run;
  }
  __syncthreads();
  const int64_t unit = ((int64_t)b * a.hkv + g) * a.n_splits + split;
  for (int e = threadIdx.x; e < a.m_rows * D; e += kThreads) {
    const int r = e / D, d = e % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mm[w * 16 + r]);
    float o = 0.0f, lsum = 0.0f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float wt = fast_exp2((mm[w * 16 + r] - M) * c);
        o += wt * mo[(w * 16 + r) * D + d];
        lsum += wt * ml[w * 16 + r];
      }
      o /= lsum;
    }
    a.part_o[(unit * a.m_rows + r) * D + d] = o;
    if (d == 0) a.part_lse[unit * a.m_rows + r] = (M == kNegInf) ? kNegInf : (M * c + __builtin_log2f(lsum)) * kLn2;
  }
}

// One wave per output row (request, q-head, position).
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nrows = (int64_t)a.B * a.hq * a.sq;
  if (row >= nrows) return;
  const int pos = (int)(row % a.sq);
  const int hq = (int)((row / a.sq) % a.hq);
  const int b = (int)(row / ((int64_t)a.sq * a.hq));
  const int g = hq / a.ratio;
  const int r = pos * a.ratio + hq % a.ratio;  // packed row
  const int Lk = a.seqlens_k ? a.seqlens_k[b] : a.sk;
  const int n = Lk > 0 ? (Lk + a.split_tokens - 1) / a.split_tokens : 0;
  const int64_t unit0 = ((int64_t)b * a.hkv + g) * a.n_splits;
  constexpr int kPer = D / 64;
  float M = kNegInf;
  for (int s = 0; s < n; ++s) M = fmaxf(M, a.part_lse[(unit0 + s) * a.m_rows + r]);
  float o[kPer] = {};
  float wsum = 0.0f;
  if (M != kNegInf) {
    for (int s = 0; s < n; ++s) {
      const float ls = a.part_lse[(unit0 + s) * a.m_rows + r];
      const float w = fast_exp2((ls - M) * kLog2e);
      wsum += w;
      const float* po = a.part_o + ((unit0 + s) * a.m_rows + r) * D;
#pragma unroll
      for (int i = 0; i < kPer; ++i) o[i] += w * po[lane * kPer + i];
    }
  }
  const float inv = (M == kNegInf) ? 0.0f : a.o_mul / wsum;
  __bf16* op = (__bf16*)a.o + (int64_t)b * a.o_sb + (int64_t)hq * a.o_sh + (int64_t)pos * a.o_sr;
  if (kPer == 2) {
    *(uint32_t*)(op + 2 * lane) = pack_bf16x2(o[0] * inv, o[1] * inv);
  } else {
    op[lane] = (__bf16)(o[0] * inv);
  }
  if (a.lse && lane == 0)
    a.lse[((int64_t)b * a.hq + hq) * a.sq + pos] = (M == kNegInf) ? kNegInf : M + __builtin_log2f(wsum) * kLn2;
}

template <int D, bool PAGED, bool MASK, bool SOFTCAP>
hipError_t launch_t(const DecodeArgs& a, const CombineArgs& c, int B, hipStream_t s) {
  dim3 grid(a.n_splits, a.hkv, B);
  hipLaunchKernelGGL((decode_kernel<D, PAGED, MASK, SOFTCAP>), grid, dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)B * c.hq * c.sq;
  hipLaunchKernelGGL((combine_kernel<D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, c);
  return hipGetLastError();
}

template <int D, bool PAGED>
hipError_t launch_p(const DecodeArgs& a, const CombineArgs& c, int B, bool mask, bool softcap, hipStream_t s) {
  if (mask) return softcap ? launch_t<D, PAGED, true, true>(a, c, B, s) : launch_t<D, PAGED, true, false>(a, c, B, s);
  return softcap ? launch_t<D, PAGED, false, true>(a, c, B, s) : launch_t<D, PAGED, false, false>(a, c, B, s);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, const CombineArgs& c, int d, bool paged, int B, hipStream_t s) {
  const bool mask = a.wl >= 0 || a.wr >= 0;
  const bool softcap = a.softcap_pre != 0.0f;
  if (B <= 0 || a.hkv <= 0 || c.sq <= 0) return hipSuccess;
  if (d == 128) return paged ? launch_p<128, true>(a, c, B, mask, softcap, s) : launch_p<128, false>(a, c, B, mask, softcap, s);
  return paged ? launch_p<64, true>(a, c, B, mask, softcap, s) : launch_p<64, false>(a, c, B, mask, softcap, s);
}

}  // namespace attn
