// fp32 attention forward (batch mode), for small problems where fp32 inputs
// and an fp32 result are wanted (the FP32 data type of the Composable Kernel
// page "fmha_fwd_pagedkv_kernel.hpp Source File").
//
// Vector-ALU kernel: one wave per query row, four rows per workgroup. The 64
// lanes of a wave form four 16-lane DPP rows (key groups); key j of a tile
// belongs to group j % 4, so each group walks a quarter of the keys. A lane
// holds D/16 d-values of q and of its group's O accumulator. K/V tiles of 64
// keys are staged in LDS with 128-bit loads while the previous tile is
// computed (the next tile's loads are in flight in registers). Per key, the
// lanes' partial dot products are summed across the 16 lanes of the group by
// four DPP adds (every lane ends with the same bits). Per tile and group: the
// logits, soft-cap and mask, the group's tile max, one rescale of its O and l
// by alpha = exp(m_old - m_new), then O += p_j V_j (the FlashAttention-2 loop of
// the CUDA-Learn-Notes page "flash_attn_mma_share_kv_F32F16F16F32.cu", without
// matrix cores). At the end the four groups' (m, l, O) are merged like split-KV
// partials: M = max m_g, l = sum 2^(m_g - M) l_g, O = sum 2^(m_g - M) O_g.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kTileN = 64;
constexpr int kLPR = 16;                  // lanes per key group: one DPP row
constexpr int kGroups = 64 / kLPR;        // key groups per wave
constexpr int kRows = kThreads / 64;      // query rows per workgroup (one per wave)

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; each step adds a symmetric partner, so
// every lane of the row holds the same bits afterwards.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1, 0, 3, 2]: lane i ^ 1
  x += dpp_mov<0x4E>(x);   // quad_perm [2, 3, 0, 1]: lane i ^ 2
  x += dpp_mov<0x141>(x);  // row_half_mirror: lane 7 - i within 8
  x += dpp_mov<0x140>(x);  // row_mirror: lane 15 - i within 16
  return x;
}

__device__ __forceinline__ float lane_xor(float x, int m) { return __shfl_xor(x, m); }

template <int D, bool MASK, bool SOFTCAP>
__global__ __launch_bounds__(kThreads) void f32_kernel(F32Args a) {
  constexpr int DPL = D / kLPR;                        // d-values per lane
  constexpr int NL = kTileN * D / 4 / kThreads;        // 16-byte K (and V) loads per thread per tile
  __shared__ __attribute__((aligned(16))) float ks[kTileN * D];
  __shared__ __attribute__((aligned(16))) float vs[kTileN * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int part = lane % kLPR;
  const int grp = lane / kLPR;
  const int bh = blockIdx.y;
  const int b = bh / a.hq, hq = bh % a.hq;
  const int g = hq / a.ratio;
  const int Lq = a.seqused_q ? a.seqused_q[b] : a.sq;
  // NULL K or V: no keys, whatever seqused_k says (nothing is dereferenced)
  const int Lk = (!a.k || !a.v) ? 0 : (a.seqused_k ? a.seqused_k[b] : a.sk);
  const int r0 = blockIdx.x * kRows;
  if (r0 >= Lq) return;
  const int row = r0 + tid / 64;
  const bool row_ok = row < Lq;
  const int off = Lk - Lq;
  const int rmax = min(r0 + kRows, Lq) - 1;
  int j_lo = 0, j_hi = Lk;
  int lim_lo = 0, lim_hi = Lk - 1;
  if (MASK) {
    if (a.wl >= 0) { j_lo = max(0, r0 + off - a.wl); lim_lo = row + off - a.wl; }
    if (a.wr >= 0) { j_hi = min(Lk, rmax + off + a.wr + 1); lim_hi = min(Lk - 1, row + off + a.wr); }
  }

  float q[DPL], o[DPL];
  const float* qp = a.q + (int64_t)b * a.q_sb + (int64_t)hq * a.q_sh + (int64_t)row * a.q_sr + part * DPL;
#pragma unroll
  for (int c = 0; c < DPL; c += 4) {
    const f32x4 v = row_ok ? *(const f32x4*)(qp + c) : f32x4{};
    q[c] = v[0]; q[c + 1] = v[1]; q[c + 2] = v[2]; q[c + 3] = v[3];
  }
#pragma unroll
  for (int c = 0; c < DPL; ++c) o[c] = 0.0f;
  const float* kg = a.k + (int64_t)b * a.k_sb + (int64_t)g * a.k_sh;
  const float* vg = a.v + (int64_t)b * a.v_sb + (int64_t)g * a.v_sh;
  const float c2 = a.c_exp2;
  float m_run = kNegInf, l_run = 0.0f;   // this group's running max and sum

  // the next tile's K and V rows, in flight in registers while a tile is computed
  f32x4 kr[NL], vr[NL];
  auto fetch = [&](int j0) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = tid + kThreads * i;
      const int key = j0 + e / (D / 4), cc = (e % (D / 4)) * 4;
      kr[i] = key < Lk ? *(const f32x4*)(kg + (int64_t)key * a.k_sr + cc) : f32x4{};
      vr[i] = key < Lk ? *(const f32x4*)(vg + (int64_t)key * a.v_sr + cc) : f32x4{};
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = tid + kThreads * i;
      *(f32x4*)(ks + (e / (D / 4)) * D + (e % (D / 4)) * 4) = kr[i];
      *(f32x4*)(vs + (e / (D / 4)) * D + (e % (D / 4)) * 4) = vr[i];
    }
  };

  const int j_first = (j_lo / kTileN) * kTileN;
  if (j_first < j_hi) fetch(j_first);
  for (int j0 = j_first; j0 < j_hi; j0 += kTileN) {
    __syncthreads();   // every wave is done with the previous tile
    stash();
    __syncthreads();
    if (j0 + kTileN < j_hi) fetch(j0 + kTileN);
    constexpr int KPG = kTileN / kGroups;   // keys of this group in the tile: grp, grp + 4, ...
    float s[KPG];
    float mt = kNegInf;
#pragma unroll
    for (int jj = 0; jj < KPG; ++jj) {
      const int j = kGroups * jj + grp;
      float dot = 0.0f;
#pragma unroll
      for (int c = 0; c < DPL; ++c) dot = __builtin_fmaf(q[c], ks[j * D + part * DPL + c], dot);
      dot = row16_sum(dot);
      float x = SOFTCAP ? a.softcap_post * tanh_fast(dot * a.softcap_pre) : dot;
      const int key = j0 + j;
      x = (key >= lim_lo && key <= lim_hi) ? x : kNegInf;
      s[jj] = x;
      mt = fmaxf(mt, x);
    }
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = fast_exp2((m_run - m_use) * c2);
    l_run *= alpha;
#pragma unroll
    for (int c = 0; c < DPL; ++c) o[c] *= alpha;
    m_run = m_new;
#pragma unroll
    for (int jj = 0; jj < KPG; ++jj) {
      const int j = kGroups * jj + grp;
      const float p = fast_exp2(__builtin_fmaf(s[jj], c2, -m_use * c2));
      l_run += p;
#pragma unroll
      for (int c = 0; c < DPL; ++c) o[c] = __builtin_fmaf(p, vs[j * D + part * DPL + c], o[c]);
    }
  }

  // merge the four key groups (lanes part, part + 16, part + 32, part + 48)
  float M = fmaxf(m_run, lane_xor(m_run, 16));
  M = fmaxf(M, lane_xor(M, 32));
  const float f = (M == kNegInf) ? 0.0f : fast_exp2((m_run - M) * c2);   // 0 for a group with no key
  float l = l_run * f;
  l += lane_xor(l, 16);
  l += lane_xor(l, 32);
#pragma unroll
  for (int c = 0; c < DPL; ++c) {
    float x = o[c] * f;
    x += lane_xor(x, 16);
    x += lane_xor(x, 32);
    o[c] = x;
  }

  if (!row_ok || grp != 0) return;
  const bool empty = !(l > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / l;
  float* op = a.o + (int64_t)b * a.o_sb + (int64_t)hq * a.o_sh + (int64_t)row * a.o_sr + part * DPL;
#pragma unroll
  for (int c = 0; c < DPL; c += 4) *(f32x4*)(op + c) = f32x4{o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv};
  if (a.lse && part == 0)
    a.lse[((int64_t)b * a.hq + hq) * a.sq + row] = empty ? kNegInf : (M * c2 + __builtin_log2f(l)) * kLn2;
}

template <int D, bool MASK, bool SOFTCAP>
hipError_t launch_t(const F32Args& a, hipStream_t s) {
  dim3 grid((a.sq + kRows - 1) / kRows, a.B * a.hq);
  hipLaunchKernelGGL((f32_kernel<D, MASK, SOFTCAP>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const F32Args& a, bool mask, bool softcap, hipStream_t s) {
  if (mask) return softcap ? launch_t<D, true, true>(a, s) : launch_t<D, true, false>(a, s);
  return softcap ? launch_t<D, false, true>(a, s) : launch_t<D, false, false>(a, s);
}

}  // namespace

int64_t f32_workgroups(const F32Args& a) { return (int64_t)a.B * a.hq * ((a.sq + kRows - 1) / kRows); }

hipError_t launch_f32(const F32Args& a, int d, hipStream_t s) {
  const bool mask = a.wl >= 0 || a.wr >= 0;
  const bool softcap = a.softcap_pre != 0.0f;
  if (a.B <= 0 || a.hq <= 0 || a.sq <= 0) return hipSuccess;
  return d == 128 ? launch_d<128>(a, mask, softcap, s) : launch_d<64>(a, mask, softcap, s);
}

}  // namespace attn
