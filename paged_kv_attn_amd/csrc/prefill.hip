// Fused attention forward, prefill shapes, for gfx950.
//
// One workgroup = 4 waves = 128 "packed" query rows of one sequence and one
// kv-head. With grouped-query attention the ratio = Hq/Hkv q-heads that share a
// kv-head are packed into the row tile, packed row r <-> (position r / ratio,
// q-head kv*ratio + r % ratio), so every K/V tile staged in LDS serves all of
// them (the PackGQA row packing of the flash-attention epilogue page
// "hopper/epilogue_fwd.hpp"; the head map kv = q / nhead_ratio_qk of the
// Composable Kernel page "fmha_fwd_pagedkv_kernel.hpp Source File").
//
// Per 64-key tile (the FlashAttention-2 loop of the CUDA-Learn-Notes page
// "flash_attn_mma_share_kv_F32F16F16F32.cu": load K/V tile, S = Q K^T, row max,
// P = exp(S - m), rescale, O += P V), each wave computes the TRANSPOSED scores
// S^T = K Q^T with v_mfma_f32_32x32x16 so that every lane owns one query row
// (lane % 32) and half of the tile's keys. Row max and row sum are then
// in-register reductions plus one exchange between the two lane halves
// (v_permlane32_swap). O^T = V^T P^T is accumulated the same way: P^T is fed
// straight from the score registers (no LDS round trip), V^T comes from the
// row-major V tile through the LDS transpose read ds_read_b64_tr_b16, and
// each lane again owns one output row, so the rescale by
// alpha = exp(m_old - m_new) is a per-lane scalar multiply.
//
// K and V tiles are double-buffered in LDS; the next tile's global loads
// (128-bit, coalesced along d) are issued before the current tile's math.
// Softmax runs in the exp2 domain with scale * log2(e) folded into one FMA
// (the FAST_EXP2 folding of the Composable Kernel page's MakeKargs).
#include "common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kBlockM = 128;
constexpr int kBlockN = 64;
constexpr int kThreads = 256;

template <int D, bool FP8>
struct Traits {
  static constexpr int kElem = FP8 ? 1 : 2;              // stored bytes per Q/K/V element
  static constexpr int kQkSteps = D / 16;                // k-steps of S^T = K Q^T
  static constexpr int kDBlocks = D / 32;                // 32-row blocks of O^T
  static constexpr int kKPitch = D * kElem + 16;         // bytes per K row in LDS
  static constexpr int kVPitch = 160;                    // bf16 elements per V row in LDS (80 dwords)
  static constexpr int kKTile = kBlockN * kKPitch;
  static constexpr int kVTile = kBlockN * kVPitch * 2;
  static constexpr int kBuf = kKTile + kVTile;
  static constexpr int kChunks = D * kElem / 16;         // 16-byte chunks per K/V row
  static constexpr int kLoads = kBlockN * kChunks / kThreads;
  static constexpr int kRowStep = kThreads / kChunks;
  static_assert(kLoads >= 1 && kBlockN * kChunks == kLoads * kThreads, "tile/threads mismatch");
  static_assert(D <= 128, "V pitch assumes d <= 128");
};

template <bool FP8> struct QFrag;
template <> struct QFrag<false> { using T = U128; };
template <> struct QFrag<true> { using T = U64; };

template <int D, bool FP8, bool VARLEN, bool MASK, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a) {
  using Tr = Traits<D, FP8>;
  using QT = typename QFrag<FP8>::T;
  __shared__ __attribute__((aligned(16))) char smem[2 * Tr::kBuf];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;          // which half of the key / d sub-blocks this lane holds
  const int g = blockIdx.y;         // kv-head
  const int z = blockIdx.z;         // batch entry or sequence
  int qt = blockIdx.x;
  if (MASK) qt = a.n_qtiles - 1 - qt;  // heaviest (latest) query tiles launch first

  // ---- sequence geometry (batch: seqused; varlen: cumulative offsets) ----
  int Lq, Lk;
  int64_t q_off, k_off, v_off, o_off, lse_off;
  if (VARLEN) {
    const int q0 = a.cu_q[z], k0 = a.cu_k[z];
    Lq = a.cu_q[z + 1] - q0;
    Lk = a.cu_k[z + 1] - k0;
    q_off = (int64_t)q0 * a.q_sr;
    k_off = (int64_t)k0 * a.k_sr;
    v_off = (int64_t)k0 * a.v_sr;
    o_off = (int64_t)q0 * a.o_sr;
    lse_off = q0;
  } else {
    Lq = a.seqused_q ? a.seqused_q[z] : a.sq;
    Lk = a.seqused_k ? a.seqused_k[z] : a.sk;
    q_off = (int64_t)z * a.q_sb;
    k_off = (int64_t)z * a.k_sb;
    v_off = (int64_t)z * a.v_sb;
    o_off = (int64_t)z * a.o_sb;
    lse_off = (int64_t)z * a.lse_sb;
  }
  const int ratio = a.ratio;
  const int rows_total = Lq * ratio;
  const int r0 = qt * kBlockM;
  if (r0 >= rows_total) return;  // tile past this sequence's end (whole workgroup)

  const int off = Lk - Lq;       // bottom-right alignment of the mask diagonal
  const int p_lo = r0 / ratio;
  const int p_hi = (min(r0 + kBlockM, rows_total) - 1) / ratio;
  int j_lo = 0, j_hi = Lk;
  if (MASK) {
    if (a.wl >= 0) j_lo = max(0, p_lo + off - a.wl);
    if (a.wr >= 0) j_hi = min(Lk, p_hi + off + a.wr + 1);
  }
  const int t_begin = j_lo / kBlockN;
  const int t_end = (j_hi > j_lo) ? (j_hi + kBlockN - 1) / kBlockN : t_begin;

  // ---- this lane's query row ----
  const int row = r0 + wave * 32 + (lane & 31);
  const bool row_ok = row < rows_total;
  const int pos = row / ratio;
  const int hq = g * ratio + row % ratio;
  const int wr0 = r0 + wave * 32;
  const bool wave_active = wr0 < rows_total;
  const int pw_lo = wr0 / ratio;
  const int pw_hi = (min(wr0 + 32, rows_total) - 1) / ratio;
  int lim_lo = 0, lim_hi = Lk - 1;  // visible keys of this row: lim_lo <= j <= lim_hi
  if (MASK) {
    if (a.wr >= 0) lim_hi = min(Lk - 1, pos + off + a.wr);
    if (a.wl >= 0) lim_lo = pos + off - a.wl;
  }

  // ---- Q fragment, resident in registers for the whole key loop ----
  // B operand of S^T = K Q^T: lane (row lane%32, half h) holds Q[row][16s + 8h .. +7].
  QT qf[Tr::kQkSteps];
  {
    const char* qp = (const char*)a.q + (q_off + (int64_t)hq * a.q_sh + (int64_t)pos * a.q_sr) * Tr::kElem;
#pragma unroll
    for (int s = 0; s < Tr::kQkSteps; ++s) {
      if (row_ok) qf[s] = *(const QT*)(qp + (16 * s + 8 * h) * Tr::kElem);
      else qf[s] = QT{};
    }
  }

  // ---- K/V staging: thread -> (row, 16-byte chunk) ----
  const int tid = threadIdx.x;
  const int ch = tid % Tr::kChunks;
  const int rb = tid / Tr::kChunks;
  const char* kg = (const char*)a.k + (k_off + (int64_t)g * a.k_sh) * Tr::kElem + ch * 16;
  const char* vg = (const char*)a.v + (v_off + (int64_t)g * a.v_sh) * Tr::kElem + ch * 16;
  U128 kreg[Tr::kLoads], vreg[Tr::kLoads];

  auto load_tile = [&](int t) {
    const int j0 = t * kBlockN;
#pragma unroll
    for (int i = 0; i < Tr::kLoads; ++i) {
      const int key = j0 + rb + i * Tr::kRowStep;
      if (key < Lk) {  // rows past the used length are zero-filled, never read
        kreg[i] = *(const U128*)(kg + (int64_t)key * a.k_sr * Tr::kElem);
        vreg[i] = *(const U128*)(vg + (int64_t)key * a.v_sr * Tr::kElem);
      } else {
        kreg[i] = U128{0, 0, 0, 0};
        vreg[i] = U128{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
    char* kt = smem + buf * Tr::kBuf;
    char* vt = kt + Tr::kKTile;
#pragma unroll
    for (int i = 0; i < Tr::kLoads; ++i) {
      const int r = rb + i * Tr::kRowStep;
      *(U128*)(kt + r * Tr::kKPitch + ch * 16) = kreg[i];
      if (FP8) {
        // V goes to LDS as bf16 (exact widening of E4M3FN); P V runs on bf16 MFMA.
        U128 lo = fp8x8_to_bf16x8(U64{vreg[i].x, vreg[i].y});
        U128 hi = fp8x8_to_bf16x8(U64{vreg[i].z, vreg[i].w});
        *(U128*)(vt + (r * Tr::kVPitch + ch * 16) * 2) = lo;
        *(U128*)(vt + (r * Tr::kVPitch + ch * 16 + 8) * 2) = hi;
      } else {
        *(U128*)(vt + (r * Tr::kVPitch + ch * 8) * 2) = vreg[i];
      }
    }
  };

  // lane-constant LDS offsets
  const int k_lane = (lane & 31) * Tr::kKPitch + 8 * h * Tr::kElem;
  const int L = lane & 15;
  const int v_lane = ((4 * h + (L >> 2)) * Tr::kVPitch + 16 * ((lane >> 4) & 1) + 4 * (L & 3)) * 2;

  const float c = a.c_exp2;
  float m_run = kNegInf;
  float l_run = 0.0f;
  f32x16 acc[Tr::kDBlocks];
#pragma unroll
  for (int i = 0; i < Tr::kDBlocks; ++i) acc[i] = f32x16{};

  auto compute = [&](int t, int buf) {
    const char* kt = smem + buf * Tr::kBuf;
    const char* vt = kt + Tr::kKTile;
    const int j0 = t * kBlockN;

    // S^T = K Q^T, two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < Tr::kQkSteps; ++kk) {
        const char* p = kt + k_lane + 32 * b * Tr::kKPitch + 16 * kk * Tr::kElem;
        if (FP8) s[b] = mfma32_fp8(*(const U64*)p, *(const U64*)&qf[kk], s[b]);
        else s[b] = mfma32_bf16(as_bf16x8(*(const U128*)p), as_bf16x8(*(const U128*)&qf[kk]), s[b]);
      }
    }

    // logit transform (soft-cap) and mask; register r of block b is key
    // j0 + 32b + 8(r/4) + 4h + r%4 of this lane's row
    bool need_mask = j0 + kBlockN > Lk;
    if (MASK) {
      if (a.wr >= 0 && j0 + kBlockN - 1 > pw_lo + off + a.wr) need_mask = true;
      if (a.wl >= 0 && j0 < pw_hi + off - a.wl) need_mask = true;
    }
    float mt = kNegInf;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[b][r];
        if (SOFTCAP) x = a.softcap_post * tanh_fast(x * a.softcap_pre);
        if (need_mask) {
          const int j = j0 + 32 * b + 8 * (r >> 2) + 4 * h + (r & 3);
          x = (j >= lim_lo && j <= lim_hi) ? x : kNegInf;
        }
        s[b][r] = x;
        mt = fmaxf(mt, x);
      }
    }
    mt = max_across_halves(mt);
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = fast_exp2((m_run - m_use) * c);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int i = 0; i < Tr::kDBlocks; ++i) acc[i] *= alpha;
    }
    l_run *= alpha;
    m_run = m_new;

    // P = exp2(x c - m c), packed to bf16 pairs in MFMA B-operand order
    const float mc = m_use * c;
    float lsum = 0.0f;
    uint32_t pk[2][8];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s[b][r], c, -mc));
        const float p1 = fast_exp2(__builtin_fmaf(s[b][r + 1], c, -mc));
        lsum += p0 + p1;
        pk[b][r >> 1] = pack_bf16x2(p0, p1);
      }
    }
    l_run += lsum;

    // O^T += V^T P^T over four 16-key steps
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int gm = 0; gm < 2; ++gm) {
        const U128 pu{pk[b][4 * gm], pk[b][4 * gm + 1], pk[b][4 * gm + 2], pk[b][4 * gm + 3]};
        const bf16x8 pb = as_bf16x8(pu);
        const int kb = 32 * b + 16 * gm;
#pragma unroll
        for (int dblk = 0; dblk < Tr::kDBlocks; ++dblk) {
          const char* p = vt + v_lane + (kb * Tr::kVPitch + 32 * dblk) * 2;
          const U64 v0 = lds_read_tr16(p);
          const U64 v1 = lds_read_tr16(p + 8 * Tr::kVPitch * 2);
          acc[dblk] = mfma32_bf16(as_bf16x8(v0, v1), pb, acc[dblk]);
        }
      }
    }
  };

  if (t_begin < t_end) {
    load_tile(t_begin);
    store_tile(0);
    __syncthreads();
    for (int t = t_begin; t < t_end; ++t) {
      const int buf = (t - t_begin) & 1;
      const bool more = t + 1 < t_end;
      if (more) load_tile(t + 1);
      const int j0 = t * kBlockN;
      bool skip = !wave_active;
      if (MASK) {
        if (a.wr >= 0 && j0 > pw_hi + off + a.wr) skip = true;
        if (a.wl >= 0 && j0 + kBlockN - 1 < pw_lo + off - a.wl) skip = true;
      }
      if (!skip) compute(t, buf);
      if (more) store_tile(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: normalise, LSE, predicated stores (rows < Lq only) ----
  const float l_tot = sum_across_halves(l_run);
  if (row_ok) {
    const bool empty = !(l_tot > 0.0f);  // no visible key: O = 0, LSE = -inf
    const float inv = empty ? 0.0f : a.o_mul / l_tot;
    char* op = (char*)a.o + (o_off + (int64_t)hq * a.o_sh + (int64_t)pos * a.o_sr) * 2;
#pragma unroll
    for (int dblk = 0; dblk < Tr::kDBlocks; ++dblk) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * dblk + 8 * q4 + 4 * h;
        U64 w;
        w.x = pack_bf16x2(acc[dblk][4 * q4 + 0] * inv, acc[dblk][4 * q4 + 1] * inv);
        w.y = pack_bf16x2(acc[dblk][4 * q4 + 2] * inv, acc[dblk][4 * q4 + 3] * inv);
        *(U64*)(op + d * 2) = w;
      }
    }
    if (a.lse && h == 0) {
      a.lse[lse_off + (int64_t)hq * a.lse_sh + pos] =
          empty ? kNegInf : (m_run * c + __builtin_log2f(l_tot)) * kLn2;
    }
  }
}

template <int D, bool FP8, bool VARLEN, bool MASK, bool SOFTCAP>
hipError_t launch_t(const PrefillArgs& a, int nz, hipStream_t stream) {
  dim3 grid(a.n_qtiles, a.hkv, nz);
  hipLaunchKernelGGL((prefill_kernel<D, FP8, VARLEN, MASK, SOFTCAP>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool FP8, bool VARLEN>
hipError_t launch_m(const PrefillArgs& a, int nz, bool mask, bool softcap, hipStream_t s) {
  if (mask) return softcap ? launch_t<D, FP8, VARLEN, true, true>(a, nz, s) : launch_t<D, FP8, VARLEN, true, false>(a, nz, s);
  return softcap ? launch_t<D, FP8, VARLEN, false, true>(a, nz, s) : launch_t<D, FP8, VARLEN, false, false>(a, nz, s);
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, int in_type, bool varlen, int nz, bool mask, bool softcap,
                    hipStream_t s) {
  if (in_type == kInFP8)
    return varlen ? launch_m<D, true, true>(a, nz, mask, softcap, s) : launch_m<D, true, false>(a, nz, mask, softcap, s);
  return varlen ? launch_m<D, false, true>(a, nz, mask, softcap, s) : launch_m<D, false, false>(a, nz, mask, softcap, s);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int d, int in_type, bool varlen, int nz, hipStream_t stream) {
  const bool mask = a.wl >= 0 || a.wr >= 0;
  const bool softcap = a.softcap_pre != 0.0f;
  if (a.n_qtiles <= 0 || nz <= 0 || a.hkv <= 0) return hipSuccess;
  if (d == 128) return launch_d<128>(a, in_type, varlen, nz, mask, softcap, stream);
  return launch_d<64>(a, in_type, varlen, nz, mask, softcap, stream);
}

}  // namespace attn
