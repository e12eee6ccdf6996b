// Split-KV decode for short query blocks (sq * Hq/Hkv <= 16 packed rows), with
// the keys either contiguous or in a paged pool, plus the split combine.
//
// Work unit = (split, kv-head, request), one wave each. A split is a fixed,
// key-aligned range of split_tokens keys, so a paged call and a contiguous call
// with the same logical keys and the same split size perform identical
// arithmetic in the same order and give identical bits. The wave walks its
// split in 32-key granules; every granule lies in one page (page_size is a
// multiple of 32), whose physical id comes from the block table (the
// page-block navigator of the Composable Kernel page "fmha_fwd_pagedkv_kernel.hpp
// Source File": one table row per request, page_block_size tokens per page,
// 64-bit page base + in-page offset).
//
// Math per granule, on v_mfma_f32_16x16x32_bf16 (fp8: _fp8_fp8) with the <= 16
// packed query rows (request position x q-heads of this kv-head) as the MFMA
// column dimension: S^T = K Q^T, online softmax over keys (max / sum across
// the four 16-lane groups), O^T += V^T P^T. K and V travel HBM -> LDS as whole
// rows through the buffer unit's direct-to-LDS loads with the non-temporal
// policy (every row is read once); K is read back into A-operand registers
// (ds_read_b128, swizzled), V transposed (ds_read_b64_tr_b16). fp8 V goes
// through registers instead and is widened exactly to bf16 on its way into
// LDS; column-major V arrives as V^T rows and is read with plain 8-byte reads.
//
// Software pipeline: the next granule's K and V (the other LDS buffers, or
// registers for fp8 V) are in flight while the current one is computed; fp8,
// whose granules carry half the bytes, keeps the next two in flight. There
// is no barrier anywhere: all data a wave touches is its own.
//
// Each unit stores its (O, LSE) normalised (the num_splits axis of O / LSE in
// the flash-attention epilogue page "hopper/epilogue_fwd.hpp"). The combine
// kernel then forms, per query row and in a fixed split order,
//     LSE = log sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s,
// which equals attention over the union of the splits' keys.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kGran = 32;  // keys per pipeline step

// K rows sit in LDS in their stored type (bf16 or fp8); V rows always as bf16
// (fp8 V is widened on its way through registers, so P V stays a bf16 product).
// D: head dim of Q and K; DV: head dim of V and O.
template <int D, int DV, bool FP8>
struct DTr {
  static constexpr int kElem = FP8 ? 1 : 2;      // stored bytes per Q/K/V element
  static constexpr int kSteps = D / 32;          // k-steps of S^T = K Q^T (32 d each)
  static constexpr int kDBlocks = DV / 16;       // 16-row blocks of O^T
  static constexpr int kRow = D * kElem;         // bytes per K row in LDS
  static constexpr int kCh = kRow / 16;          // 16-byte chunks per K row
  static constexpr int kBuf = kGran * kRow;      // one K granule in LDS
  static constexpr int kBlocks = kBuf / 1024;    // direct-to-LDS loads per K granule
  static constexpr int kRowsPer256 = 256 / kRow;
  static constexpr int kVRow = DV * 2;           // bytes per V row in LDS (bf16)
  static constexpr int kVCh = kVRow / 16;
  static constexpr int kVBuf = kGran * kVRow;
  static constexpr int kVBlocks = kVBuf / 1024;  // direct-to-LDS loads per V granule (bf16)
  static constexpr int kVRowsPer256 = 256 / kVRow;
  static constexpr int kV8 = kGran * DV / 16 / 64;  // fp8 V: 16-byte register loads per lane per granule
  static constexpr int kOps = kBlocks + (FP8 ? kV8 : kVBlocks);  // vector-memory ops per granule
  static_assert(kBlocks >= 1 && kVBlocks >= 1 && (!FP8 || kV8 >= 1), "granule too small");
};

// Chunk swizzles of the LDS rows (chunk c of row R lives in slot c ^ swz(R));
// 64 banks of 4 bytes, so rows of the same residue modulo 256 bytes share bank
// offsets. K: the 16 lanes of an A-operand read (ds_read_b128) take one chunk
// of 16 consecutive rows; the swizzle spreads them over all 64 banks. V: a
// transpose read (ds_read_b64_tr_b16) of two 16-lane groups takes 8
// consecutive rows x 2 adjacent chunks; the swizzle (bit 0 clear, so the pair
// stays adjacent) gives the 8 rows 8 different chunk pairs.
template <int D, bool FP8>
__device__ __forceinline__ int kswz(int row) {
  return (row / DTr<D, D, FP8>::kRowsPer256) & (DTr<D, D, FP8>::kCh - 1);
}
template <int DV>
__device__ __forceinline__ int vswz(int row) {
  return ((row / DTr<DV, DV, false>::kVRowsPer256) & (DTr<DV, DV, false>::kVCh / 2 - 1)) << 1;
}

__device__ __forceinline__ f32x4 mfma16_fp8(const U64& a, const U64& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, a), __builtin_bit_cast(long, b), c, 0,
                                                    0, 0);
}

__device__ __forceinline__ float xor_shfl(float x, int mask) {
  const int lane = threadIdx.x & 63;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(((lane ^ mask) << 2), __builtin_bit_cast(int, x)));
}

// Column-major V (keys contiguous): the granule's V^T sits in LDS as DV rows of
// 32 keys (64 B); 16-byte chunk c of row R lives in slot c ^ vt_sw(R), so the 8-byte
// operand reads of 16 rows x 2 halves fall in 32 different bank pairs.
__device__ __forceinline__ int vt_sw(int row) { return (row >> 2) & 3; }

template <int D, int DV, bool PAGED, bool MASK, bool SOFTCAP, bool FP8, bool VT>
__global__ __launch_bounds__(64) void decode_kernel(DecodeArgs a) {
  static_assert(!VT || D == DV, "column-major V: equal head dims");
  using Tr = DTr<D, DV, FP8>;
  // One LDS object per pipeline buffer, so the compiler can tell the
  // HBM->LDS copies into one buffer from the reads of the other.
  __shared__ __attribute__((aligned(1024))) char kbuf0[Tr::kBuf];
  __shared__ __attribute__((aligned(1024))) char vbuf0[Tr::kVBuf];
  __shared__ __attribute__((aligned(1024))) char kbuf1[Tr::kBuf];
  __shared__ __attribute__((aligned(1024))) char vbuf1[Tr::kVBuf];
  __shared__ __attribute__((aligned(1024))) char kbuf2[FP8 ? Tr::kBuf : 16];  // fp8's third K stage
  lds_char* const k0 = (lds_char*)kbuf0;
  lds_char* const v0 = (lds_char*)vbuf0;
  lds_char* const k1 = (lds_char*)kbuf1;
  // fp8 V is in flight in registers and widened into LDS just before its
  // granule's products, so one bf16 V buffer serves every stage: this wave's
  // LDS accesses stay in program order, and the widening of granule g+1 comes
  // after the reads of granule g. Three K stages and one V buffer take 20 KB
  // per wave (8 waves per CU), with two 8 KB granules in flight per wave while
  // a third is computed.
  lds_char* const v1 = (lds_char*)vbuf1;  // bf16 only
  lds_char* const k2 = (lds_char*)kbuf2;

  const int lane = threadIdx.x;
  const int g = blockIdx.x;      // kv-heads fastest: the units running together read the
  const int split = blockIdx.y;  // same token rows (shared DRAM pages in a [page, slot, head] pool)
  const int b = blockIdx.z;
  // K/V batch entry of contiguous K/V (cache batch index; out of range: no keys)
  const int kb = PAGED ? b : kv_entry(a.cache_idx, a.cache_count, b);
  // an out-of-range cache entry, or NULL K or V, has no keys
  const int Lk = (kb < 0 || !a.k || !a.v) ? 0 : (a.seqlens_k ? a.seqlens_k[b] : a.sk);
  const int t0 = split * a.split_tokens;
  if (t0 >= Lk) return;  // empty split: the combine reads only ceil(Lk / split_tokens) partials
  const int t1 = min(Lk, t0 + a.split_tokens);

  // packed query row of this lane's MFMA column
  const int qc = lane & 15;
  const int j4 = lane >> 4;
  const int ratio = a.ratio;
  const int Lq = a.seqused_q ? a.seqused_q[b] : a.sq;  // used query rows of this request
  if (Lq <= 0) return;  // no row of this request is written (the combine skips them too)
  const int pos = qc / ratio;
  const bool row_ok = qc < a.m_rows && pos < Lq;
  const int hq = g * ratio + qc % ratio;
  const int off = Lk - Lq;                             // bottom-right alignment on the used rows
  int lim_lo = 0, lim_hi = Lk - 1;
  // keys any row of the unit can see (bottom-right aligned window)
  int t_lo = t0, t_hi = t1;
  if (MASK) {
    if (a.wr >= 0) {
      lim_hi = min(Lk - 1, pos + off + a.wr);
      t_hi = min(t1, (Lq - 1) + off + a.wr + 1);
    }
    if (a.wl >= 0) {
      lim_lo = pos + off - a.wl;
      t_lo = a.sink_size > t0 ? t0 : max(t0, off - a.wl);  // sink keys ignore the left bound
    }
    t_lo = t0 + (max(0, t_lo - t0) / kGran) * kGran;  // keep granules aligned to the split
  }

  // ALiBi slope of this lane's (request, q-head), in kernel logit units
  const float alibi_k = a.alibi ? a.alibi[(int64_t)b * a.alibi_sb + hq] * a.bias_mul : 0.0f;
  // elementwise bias: this lane's row (lanes past the used rows read row 0 of
  // their head, never stored); keys are read as aligned 16-byte blocks of 4,
  // clamped to the block holding key Lk - 1
  const float* bias_row =
      a.bias ? a.bias + (int64_t)b * a.bias_sb + (int64_t)hq * a.bias_sh + (int64_t)(row_ok ? pos : 0) * a.bias_sr
             : nullptr;
  const int bias_last = (Lk - 1) & ~3;

  // The split's page ids, one per lane (a split spans at most 64 pages).
  const int p_first = PAGED ? t0 / a.page_size : 0;
  int pg = 0;
  if (PAGED) {
    const int n_pg = (t1 - 1) / a.page_size - p_first + 1;
    if (lane < n_pg) pg = a.block_table[(int64_t)b * a.bt_stride + p_first + lane];
  }

  // Q^T as the B operand: lane (column qc, group j4) holds Q[qc][32s + 8 j4 .. +7]
  // (16 bytes of bf16, or 8 bytes of fp8)
  U128 qf[FP8 ? 1 : Tr::kSteps];
  U64 qf8[FP8 ? Tr::kSteps : 1];
  {
    const char* qp =
        (const char*)a.q + ((int64_t)b * a.q_sb + (int64_t)hq * a.q_sh + (int64_t)pos * a.q_sr) * Tr::kElem;
#pragma unroll
    for (int s = 0; s < Tr::kSteps; ++s) {
      if (FP8) qf8[s] = row_ok ? *(const U64*)(qp + 32 * s + 8 * j4) : U64{0, 0};
      else qf[s] = row_ok ? *(const U128*)(qp + (32 * s + 8 * j4) * 2) : U128{0, 0, 0, 0};
    }
  }

  const int64_t krow = a.k_sr * Tr::kElem, vrow = a.v_sr * Tr::kElem;   // bytes per key row
  const int L = lane & 15;
  // K and V granules -> LDS, whole rows per load: block q, lane l covers LDS
  // bytes 1024 q + 16 l = (row R, slot sl) and fetches chunk sl ^ swz(R) of row R.
  int koff[Tr::kBlocks], voff[FP8 ? Tr::kV8 : Tr::kVBlocks];
#pragma unroll
  for (int q = 0; q < Tr::kBlocks; ++q) {
    const int B = 1024 * q + 16 * lane;
    const int R = B / Tr::kRow, sl = (B % Tr::kRow) / 16;
    koff[q] = (int)(R * krow) + 16 * (sl ^ kswz<D, FP8>(R));
  }
  // V: bf16 rows straight to LDS; fp8 rows as 16-byte chunks into registers
  // (load i of lane l: chunk 64 i + l = row R, fp8 chunk c8 of the row; column-major
  // fp8 V: head-dim row ch / 2, keys 16 (ch % 2) .. of the granule)
#pragma unroll
  for (int q = 0; q < (FP8 ? Tr::kV8 : Tr::kVBlocks); ++q) {
    if (FP8 && VT) {
      const int ch = 64 * q + lane;
      voff[q] = (int)((ch >> 1) * vrow) + 16 * (ch & 1);
    } else if (FP8) {
      const int ch = 64 * q + lane, R = ch / (DV / 16), c8 = ch % (DV / 16);
      voff[q] = (int)(R * vrow) + 16 * c8;
    } else if (VT) {  // block q: V^T rows 16 q .. 16 q + 15, lane l: row 16 q + l / 4, slot l % 4
      const int R = 16 * q + (lane >> 2), kc = (lane & 3) ^ vt_sw(R);
      voff[q] = (int)(R * vrow) + 16 * kc;
    } else {
      const int B = 1024 * q + 16 * lane;
      const int R = B / Tr::kVRow, sl = (B % Tr::kVRow) / 16;
      voff[q] = (int)(R * vrow) + 16 * (sl ^ vswz<DV>(R));
    }
  }
  // column-major V: keys of chunk (lane & 3) ^ vt_sw(row) of this lane's load rows
  const int vt_kc = VT ? (lane & 3) ^ vt_sw(lane >> 2) : 0;   // vt_sw(16 q + l / 4) = vt_sw(l / 4)
  const char* const vt_head =
      VT ? (const char*)a.v + ((int64_t)(PAGED ? 0 : kb) * a.v_sb + (int64_t)g * a.v_sh) * Tr::kElem : nullptr;
  // K A-operand reads: lane (key 16 kb + L, group j4) takes K[key][32 st + 8 j4 .. +7],
  // chunk 4 st + j4 of row 16 kb + L, whose swizzle kswz(16 kb + L) = kswz(L) = ksw:
  // slot (4 st + j4) ^ ksw = ((4 st) ^ (ksw & ~3)) + ((j4 ^ ksw) & 3).
  const int ksw = kswz<D, FP8>(L);
  const int k_lane0 = L * Tr::kRow + 16 * ((j4 ^ ksw) & 3);
  const int k_hi = 16 * (ksw & ~3);
  // fp8 K: the 8 bytes K[key][32 st + 8 j4 ..] are half h8 = j4 & 1 of chunk 2 st + j4 / 2
  // of row 16 kb + L, whose swizzle is kswz(L) for both kb
  auto k8_addr = [&](int kb, int st) -> int {
    return (16 * kb + L) * Tr::kRow + 16 * ((2 * st + (j4 >> 1)) ^ ksw) + 8 * (j4 & 1);
  };
  // transpose reads: group j4 (16 lanes) reads rows 16 kb + 4 j4 + L / 4, bf16
  // columns 16 dblk + 4 (L & 3) .. +3 = byte 8 (L & 1) of chunk 2 dblk + (L & 3) / 2;
  // those rows' swizzle vs = vswz(4 j4 + L / 4) has bit 0 clear, so the slot is
  // (2 dblk ^ vs) + (L & 3) / 2.
  const int v_sw = vswz<DV>(4 * j4 + (L >> 2));
  const int v_base0 = (4 * j4 + (L >> 2)) * Tr::kVRow + 16 * ((L & 3) >> 1) + 8 * (L & 1);
  const int v_swhi = 16 * v_sw;

  // base of the 32 keys starting at key gs (64-bit page base + in-page offset)
  auto rows_base = [&](int gs, const void* pool, int64_t sb, int64_t sh, int64_t sr) -> const char* {
    if (PAGED) {
      const int page = __builtin_amdgcn_readlane(pg, gs / a.page_size - p_first);
      return (const char*)pool +
             ((int64_t)page * sb + (int64_t)g * sh + (int64_t)(gs % a.page_size) * sr) * Tr::kElem;
    }
    return (const char*)pool + ((int64_t)kb * sb + (int64_t)g * sh + (int64_t)gs * sr) * Tr::kElem;
  };
  // issue the loads of granule gs into the LDS buffers kb / vb (whole rows,
  // non-temporal: every K and V row is read once). A granule at or past t_hi is
  // issued with an empty range: no memory traffic, zeros everywhere.
  U128 v8a[FP8 ? Tr::kV8 : 1], v8b[FP8 ? Tr::kV8 : 1], v8c[FP8 ? Tr::kV8 : 1];  // fp8 V of the pipeline stages
  auto issue = [&](int gs, lds_char* kb, lds_char* vb, U128 (&v8)[FP8 ? Tr::kV8 : 1]) {
    // readfirstlane keeps the clamp (a vector med3) from making the
    // descriptor look divergent
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(kGran, t_hi - gs)));
    const int gp = rows > 0 ? gs : t0;  // any valid page for an empty range
    const __amdgpu_buffer_rsrc_t kr =
        make_rsrc(rows_base(gp, a.k, a.k_sb, a.k_sh, a.k_sr), (uint32_t)(rows * krow));
    // column-major V: the granule's 32-key span of every head-dim row (paged: in
    // the granule's page, keys contiguous as in the page's [hdim_v, page_block_size]
    // view of a V page); chunks of keys at or past the range get an offset beyond
    // it and arrive as zeros
    const char* vt_base = nullptr;
    if (VT) {
      if (PAGED) {
        const int page = __builtin_amdgcn_readlane(pg, gp / a.page_size - p_first);
        vt_base = vt_head + ((int64_t)page * a.v_sb + gp % a.page_size) * Tr::kElem;
      } else {
        vt_base = vt_head + (int64_t)gp * Tr::kElem;
      }
    }
    const __amdgpu_buffer_rsrc_t vr =
        VT ? make_rsrc(vt_base, (uint32_t)((DV - 1) * vrow + Tr::kElem * kGran))
           : make_rsrc(rows_base(gp, a.v, a.v_sb, a.v_sh, a.v_sr), (uint32_t)(rows * vrow));
#pragma unroll
    for (int q = 0; q < Tr::kBlocks; ++q) buf_load16_lds_stream(kr, kb + 1024 * q, koff[q]);
    if (FP8) {
#pragma unroll
      for (int q = 0; q < Tr::kV8; ++q)
        v8[q] = buf_load16(vr, (!VT || 16 * (lane & 1) < rows) ? voff[q] : 0x7FFFFFF0);
    } else {
#pragma unroll
      for (int q = 0; q < Tr::kVBlocks; ++q)
        buf_load16_lds_stream(vr, vb + 1024 * q, (!VT || 8 * vt_kc < rows) ? voff[q] : 0x7FFFFFF0);
    }
  };
  // fp8 V of one granule: widen (exactly) to bf16 into the LDS layout of bf16 V
  // (column-major: of bf16 V^T; keys at or past min(t_hi, gs + 32) in the chunk
  // holding the last one, any bits, are zeroed here)
  auto store_v8 = [&](lds_char* vb, const U128 (&v8)[FP8 ? Tr::kV8 : 1], int gs) {
    if (VT) {
      const int rows = min(kGran, t_hi - gs);
#pragma unroll
      for (int q = 0; q < (FP8 ? Tr::kV8 : 0); ++q) {
        const int ch = 64 * q + lane, R = ch >> 1, c = ch & 1;
        U128 lo = fp8x8_to_bf16x8(U64{v8[q].x, v8[q].y}), hi = fp8x8_to_bf16x8(U64{v8[q].z, v8[q].w});
        const int nv = rows - 16 * c;
        if (nv < 16) {
          uint32_t* w = &lo.x;
#pragma unroll
          for (int e = 0; e < 8; e += 2) w[e / 2] &= (e < nv ? 0xFFFFu : 0u) | (e + 1 < nv ? 0xFFFF0000u : 0u);
          w = &hi.x;
#pragma unroll
          for (int e = 0; e < 8; e += 2) w[e / 2] &= (8 + e < nv ? 0xFFFFu : 0u) | (9 + e < nv ? 0xFFFF0000u : 0u);
        }
        // a 16-byte LDS store resolves bank conflicts per 8 lanes over 128 bytes:
        // rows 4m + 2, 4m + 3 store their high chunk first, so that the 8 lanes
        // (rows 4m .. 4m + 3, two 64-byte rows per 128 bytes) hit 8 distinct slots
        lds_char* row = vb + R * (2 * kGran);
        const int f = (R >> 1) & 1;
        lds_store16(row + 16 * ((2 * c + f) ^ vt_sw(R)), f ? hi : lo);
        lds_store16(row + 16 * ((2 * c + 1 - f) ^ vt_sw(R)), f ? lo : hi);
      }
      return;
    }
#pragma unroll
    for (int q = 0; q < (FP8 ? Tr::kV8 : 0); ++q) {
      const int ch = 64 * q + lane, R = ch / (DV / 16), c0 = 2 * (ch % (DV / 16));
      const U128 lo = fp8x8_to_bf16x8(U64{v8[q].x, v8[q].y}), hi = fp8x8_to_bf16x8(U64{v8[q].z, v8[q].w});
      // a 16-byte LDS store resolves bank conflicts per 8 lanes over 128 bytes;
      // lanes 4 .. 7 of each 8 store their high chunk first, so the 8 lanes' 32-byte
      // chunk pairs (256 contiguous bytes before the swizzle, which XORs the slot
      // with a constant per 8 lanes) hit 8 distinct slots modulo 128 bytes
      const int f = (ch >> 2) & 1;
      lds_store16(vb + R * Tr::kVRow + 16 * ((c0 + f) ^ vswz<DV>(R)), f ? hi : lo);
      lds_store16(vb + R * Tr::kVRow + 16 * ((c0 + 1 - f) ^ vswz<DV>(R)), f ? lo : hi);
    }
  };

  const float c = a.c_exp2;
  float m_run = kNegInf;
  float l_run = 0.0f;
  f32x4 acc[Tr::kDBlocks];
#pragma unroll
  for (int i = 0; i < Tr::kDBlocks; ++i) acc[i] = f32x4{};

  // one 32-key granule: S^T = K Q^T, online softmax, O^T += V^T P^T
  auto compute = [&](int gs, const lds_char* kbuf, const lds_char* vb) {
    f32x4 st[2];
    int k_lane = k_lane0, k_x = k_hi;
    asm volatile("" : "+v"(k_lane), "+v"(k_x));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      st[kb] = f32x4{};
      if (FP8) {
        // an opaque block offset keeps the compiler from pairing the two key
        // blocks' reads into one two-address read, whose halves (2 KB apart) hit
        // the same banks
        int kofs = 16 * kb * Tr::kRow;
        asm volatile("" : "+v"(kofs));
        U64 kf[Tr::kSteps];
#pragma unroll
        for (int s = 0; s < Tr::kSteps; ++s) kf[s] = lds_load8(kbuf + kofs + k8_addr(0, s));
#pragma unroll
        for (int s = 0; s < Tr::kSteps; ++s) st[kb] = mfma16_fp8(kf[s], qf8[s], st[kb]);
      } else {
        U128 kf[Tr::kSteps];
#pragma unroll
        for (int s = 0; s < Tr::kSteps; ++s)
          kf[s] = lds_load16(kbuf + k_lane + 16 * kb * Tr::kRow + ((64 * s) ^ k_x));
#pragma unroll
        for (int s = 0; s < Tr::kSteps; ++s) st[kb] = mfma16_bf16(as_bf16x8(kf[s]), as_bf16x8(qf[s]), st[kb]);
      }
    }
    // lane (column qc, group j4) holds keys gs + 16 kb + 4 j4 + r
    U128 bv[2] = {};
    if (bias_row) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) bv[kb] = *(const U128*)(bias_row + min(gs + 16 * kb + 4 * j4, bias_last));
    }
    float mt = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = st[kb][r];
        if (SOFTCAP) x = softcap_logit(x, 2.0f * kLog2e * a.softcap_pre, a.softcap_post);
        const int j = gs + 16 * kb + 4 * j4 + r;
        if (a.alibi) x = __builtin_fmaf(-alibi_k, __builtin_fabsf((float)(pos + off - j)), x);
        if (bias_row) x = __builtin_fmaf(__builtin_bit_cast(float, (&bv[kb].x)[r]), a.bias_mul, x);
        x = ((j >= lim_lo || j < a.sink_size) && j <= lim_hi) ? x : kNegInf;
        st[kb][r] = x;
        mt = __builtin_fmaxf(mt, x);
      }
    }
    mt = __builtin_fmaxf(mt, xor_shfl(mt, 16));
    mt = __builtin_fmaxf(mt, xor_shfl(mt, 32));
    // lazy rescale, as in the prefill kernel: the reference max only moves when
    // the granule max exceeds it by more than 8 in log2 units
    const bool raise = (mt - m_run) * c > 8.0f;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float alpha = raise ? fast_exp2((m_run - mt) * c) : 1.0f;
#pragma unroll
      for (int i = 0; i < Tr::kDBlocks; ++i) acc[i] *= alpha;
      l_run *= alpha;
      m_run = raise ? mt : m_run;
    }
    const float mc = (m_run == kNegInf) ? 0.0f : m_run * c;
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = fast_exp2(__builtin_fmaf(st[i >> 2][i & 3], c, -mc));
      l_run += p[i];
    }
    // P^T as the B operand: slot 4 kb + r <-> key 16 kb + 4 j4 + r
    const U128 pu{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
    const bf16x8 pb = as_bf16x8(pu);
    if (VT) {
      // V^T row 16 dblk + L holds the keys; slot 4 kb + r of the operand is key
      // 16 kb + 4 j4 + r: bytes 32 kb + 8 j4 of the row, i.e. half j4 & 1 of chunk
      // 2 kb + j4 / 2 (swizzle vt_sw(16 dblk + L) = vt_sw(L))
      const int sw = vt_sw(L);
      const int c0 = 16 * ((j4 >> 1) ^ sw) + 8 * (j4 & 1), c1 = 16 * ((2 + (j4 >> 1)) ^ sw) + 8 * (j4 & 1);
#pragma unroll
      for (int dblk = 0; dblk < Tr::kDBlocks; ++dblk) {
        const lds_char* row = vb + (16 * dblk + L) * (2 * kGran);
        acc[dblk] = mfma16_bf16(as_bf16x8(lds_load8(row + c0), lds_load8(row + c1)), pb, acc[dblk]);
      }
      return;
    }
    int v_base = v_base0, v_hi = v_swhi;
    asm volatile("" : "+v"(v_base), "+v"(v_hi));
#pragma unroll
    for (int dblk = 0; dblk < Tr::kDBlocks; ++dblk) {
      const lds_char* vp = vb + v_base + ((32 * dblk) ^ v_hi);
      const U64 v0 = lds_read_tr16(vp);
      const U64 v1 = lds_read_tr16(vp + 16 * Tr::kVRow);
      acc[dblk] = mfma16_bf16(as_bf16x8(v0, v1), pb, acc[dblk]);
    }
  };
  // column-major V: the chunk holding key Lk - 1 also brought keys Lk .. (past the
  // used length, possibly not finite); zero them in LDS before the products read them
  auto vt_zero_tail = [&](int gs, lds_char* vb) {
    const int cs = Lk & ~7;
    if (VT && !FP8 && (Lk & 7) && cs >= gs && cs < gs + kGran && cs < t_hi) {
      const int kc = (cs - gs) >> 3;
      for (int R = lane; R < DV; R += 64) {
        lds_char* row = vb + R * (2 * kGran) + 16 * (kc ^ vt_sw(R));
        for (int e = Lk & 7; e < 8; ++e) *(__attribute__((address_space(3))) uint16_t*)(row + 2 * e) = 0;
      }
    }
  };

  int gs = t_lo;
  if (FP8 && gs < t_hi) {
    // three stages: granules g + 1 and g + 2 in flight while g is widened and
    // computed (a granule at or past t_hi is issued empty)
    issue(gs, k0, v0, v8a);
    issue(gs + kGran, k1, v0, v8b);
    for (;;) {
      issue(gs + 2 * kGran, k2, v0, v8c);
      wait_vmem_le<2 * Tr::kOps>();
      store_v8(v0, v8a, gs);
      compute(gs, k0, v0);
      gs += kGran;
      if (gs >= t_hi) break;
      issue(gs + 2 * kGran, k0, v0, v8a);
      wait_vmem_le<2 * Tr::kOps>();
      store_v8(v0, v8b, gs);
      compute(gs, k1, v0);
      gs += kGran;
      if (gs >= t_hi) break;
      issue(gs + 2 * kGran, k1, v0, v8b);
      wait_vmem_le<2 * Tr::kOps>();
      store_v8(v0, v8c, gs);
      compute(gs, k2, v0);
      gs += kGran;
      if (gs >= t_hi) break;
    }
    wait_vmem_le<0>();
  } else if (gs < t_hi) {  // bf16: two stages
    issue(gs, k0, v0, v8a);
    for (;;) {
      issue(gs + kGran, k1, v1, v8b);
      wait_vmem_le<Tr::kOps>();
      vt_zero_tail(gs, v0);
      compute(gs, k0, v0);
      gs += kGran;
      if (gs >= t_hi) break;
      issue(gs + kGran, k0, v0, v8a);
      wait_vmem_le<Tr::kOps>();
      vt_zero_tail(gs, v1);
      compute(gs, k1, v1);
      gs += kGran;
      if (gs >= t_hi) break;
    }
    wait_vmem_le<0>();
  }

  // normalised partial: lane (qc, j4) holds O^T[16 dblk + 4 j4 + r][qc]
  l_run += xor_shfl(l_run, 16);
  l_run += xor_shfl(l_run, 32);
  const int64_t unit = ((int64_t)b * a.hkv + g) * a.n_splits + split;
  if (row_ok) {
    const bool live = m_run != kNegInf;
    const float inv = live ? 1.0f / l_run : 0.0f;
    float* po = a.part_o + (unit * a.m_rows + qc) * DV + 4 * j4;
#pragma unroll
    for (int dblk = 0; dblk < Tr::kDBlocks; ++dblk) *(f32x4*)(po + 16 * dblk) = acc[dblk] * inv;
    if (j4 == 0) a.part_lse[unit * a.m_rows + qc] = live ? (m_run * c + __builtin_log2f(l_run)) * kLn2 : kNegInf;
  }
}

// One wave per output row (request, q-head, position). The split LSEs are
// read 64 at a time (one per lane) for the max and the weights; the partial
// rows are then summed in split order with 8 loads in flight.
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
  if (a.seqused_q && pos >= a.seqused_q[b]) return;  // row past the used query length: not written
  const int Lk = (a.no_keys || kv_entry(a.cache_idx, a.cache_count, b) < 0) ? 0 : (a.seqlens_k ? a.seqlens_k[b] : a.sk);
  const int n = Lk > 0 ? (Lk + a.split_tokens - 1) / a.split_tokens : 0;
  const int64_t unit0 = ((int64_t)b * a.hkv + g) * a.n_splits;
  const float* lse_p = a.part_lse + unit0 * a.m_rows + r;   // split s at lse_p[s * m_rows]
  const float* o_p = a.part_o + unit0 * a.m_rows * D + (int64_t)r * D;  // split s at o_p[s * m_rows * D]
  const int64_t o_stride = (int64_t)a.m_rows * D;
  constexpr int kPer = D / 64;

  float M = kNegInf;
  for (int s0 = 0; s0 < n; s0 += 64)
    if (s0 + lane < n) M = fmaxf(M, lse_p[(int64_t)(s0 + lane) * a.m_rows]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m));
  // the sink logit: one more denominator term exp(sink), no value row
  const float sink = a.sink_logits ? a.sink_logits[hq] : kNegInf;
  M = fmaxf(M, sink);

  float o[kPer] = {};
  float wsum = 0.0f;
  if (M != kNegInf) {
    for (int s0 = 0; s0 < n; s0 += 64) {
      const int cnt = min(64, n - s0);
      // this lane's split weight exp(LSE_s - M)
      const float w_l = lane < cnt ? fast_exp2((lse_p[(int64_t)(s0 + lane) * a.m_rows] - M) * kLog2e) : 0.0f;
      wsum += w_l;
      int s = 0;
      for (; s + 8 <= cnt; s += 8) {
        float v[8][kPer];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int i = 0; i < kPer; ++i) v[u][i] = o_p[(int64_t)(s0 + s + u) * o_stride + lane * kPer + i];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_l), s + u));
#pragma unroll
          for (int i = 0; i < kPer; ++i) o[i] += w * v[u][i];
        }
      }
      for (; s < cnt; ++s) {
        const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_l), s));
#pragma unroll
        for (int i = 0; i < kPer; ++i) o[i] += w * o_p[(int64_t)(s0 + s) * o_stride + lane * kPer + i];
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) wsum += __shfl_xor(wsum, m);
    if (sink > kNegInf) wsum += fast_exp2((sink - M) * kLog2e);
  }
  const float inv = (M == kNegInf) ? 0.0f : a.o_mul / wsum;
  const int64_t o_elem = (int64_t)b * a.o_sb + (int64_t)hq * a.o_sh + (int64_t)pos * a.o_sr;
  if (a.out_fp8) {  // saturated E4M3FN
    uint8_t* op = (uint8_t*)a.o + o_elem;
    const uint32_t w = pack_fp8x4_sat(o[0] * inv, kPer == 2 ? o[1] * inv : 0.0f, 0.0f, 0.0f);
    if (kPer == 2) {
      *(uint16_t*)(op + 2 * lane) = (uint16_t)w;
    } else {
      op[lane] = (uint8_t)w;
    }
  } else {
    __bf16* op = (__bf16*)a.o + o_elem;
    if (kPer == 2) {
      *(uint32_t*)(op + 2 * lane) = pack_bf16x2(o[0] * inv, o[1] * inv);
    } else {
      op[lane] = (__bf16)(o[0] * inv);
    }
  }
  if (a.lse && lane == 0)
    a.lse[((int64_t)b * a.hq + hq) * a.sq + pos] = (M == kNegInf) ? kNegInf : M + __builtin_log2f(wsum) * kLn2;
}

template <int D, int DV, bool PAGED, bool MASK, bool SOFTCAP>
hipError_t launch_t(const DecodeArgs& a, const CombineArgs& c, int B, hipStream_t s) {
  dim3 grid(a.hkv, a.n_splits, B);
  if constexpr (D == DV) {
    if (a.v_colmajor && a.fp8) {
      hipLaunchKernelGGL((decode_kernel<D, DV, PAGED, MASK, SOFTCAP, true, true>), grid, dim3(64), 0, s, a);
    } else if (a.v_colmajor) {
      hipLaunchKernelGGL((decode_kernel<D, DV, PAGED, MASK, SOFTCAP, false, true>), grid, dim3(64), 0, s, a);
    } else if (a.fp8) {
      hipLaunchKernelGGL((decode_kernel<D, DV, PAGED, MASK, SOFTCAP, true, false>), grid, dim3(64), 0, s, a);
    } else {
      hipLaunchKernelGGL((decode_kernel<D, DV, PAGED, MASK, SOFTCAP, false, false>), grid, dim3(64), 0, s, a);
    }
  } else {
    if (a.v_colmajor) return hipErrorInvalidValue;  // head_dim_v = d only
    if (a.fp8) hipLaunchKernelGGL((decode_kernel<D, DV, PAGED, MASK, SOFTCAP, true, false>), grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL((decode_kernel<D, DV, PAGED, MASK, SOFTCAP, false, false>), grid, dim3(64), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)B * c.hq * c.sq;
  hipLaunchKernelGGL((combine_kernel<DV>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, c);
  return hipGetLastError();
}

template <int D, int DV, bool PAGED>
hipError_t launch_p(const DecodeArgs& a, const CombineArgs& c, int B, bool mask, bool softcap, hipStream_t s) {
  if (mask)
    return softcap ? launch_t<D, DV, PAGED, true, true>(a, c, B, s) : launch_t<D, DV, PAGED, true, false>(a, c, B, s);
  return softcap ? launch_t<D, DV, PAGED, false, true>(a, c, B, s) : launch_t<D, DV, PAGED, false, false>(a, c, B, s);
}

template <int D>
hipError_t launch_dv(const DecodeArgs& a, const CombineArgs& c, int dv, bool paged, int B, bool mask, bool softcap,
                     hipStream_t s) {
  if (paged) return dv == 64 ? launch_p<D, 64, true>(a, c, B, mask, softcap, s) : launch_p<D, 128, true>(a, c, B, mask, softcap, s);
  if (dv == 64) return launch_p<D, 64, false>(a, c, B, mask, softcap, s);
  return launch_p<D, 128, false>(a, c, B, mask, softcap, s);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, const CombineArgs& c, int d, int dv, bool paged, int B, hipStream_t s) {
  const bool mask = a.wl >= 0 || a.wr >= 0;
  const bool softcap = a.softcap_pre != 0.0f;
  if (B <= 0 || a.hkv <= 0 || c.sq <= 0) return hipSuccess;
  if (d == 128) return launch_dv<128>(a, c, dv, paged, B, mask, softcap, s);
  return launch_dv<64>(a, c, dv, paged, B, mask, softcap, s);
}

}  // namespace attn
