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
// K and V tiles travel from HBM straight into LDS (buffer_load_dwordx4 ... lds,
// 128-bit per lane, coalesced along d; rows past the sequence end arrive as
// zeros from the buffer range check), so no registers are spent on staging.
// Two LDS slots (separate LDS objects, so the compiler can order reads of one
// slot against the copies into the other without waiting for them): while
// tile t is computed from one slot, tile t+1 is in flight into the other; one
// wait + barrier per tile. Within LDS each 16-byte chunk of a row is
// XOR-swizzled by the row index, which keeps the K operand reads and the V
// transpose reads free of bank conflicts. Tiles that no row of a wave can see
// are skipped by that wave; the mask is evaluated only on tiles that cut
// through some row's visible range.
// Softmax runs in the exp2 domain with scale * log2(e) folded into one FMA
// (the FAST_EXP2 folding of the Composable Kernel page's MakeKargs).
#include "common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kBlockM = 128;
constexpr int kBlockN = 64;
constexpr int kThreads = 256;
constexpr int kXcds = 8;         // accelerator complex dies on MI355X

// D: head dim of Q and K; DV: head dim of V and O
template <int D, int DV, bool FP8>
struct Traits {
  static constexpr int kElem = FP8 ? 1 : 2;              // stored bytes per Q/K/V element
  static constexpr int kQkSteps = D / 16;                // k-steps of S^T = K Q^T
  static constexpr int kDBlocks = DV / 32;               // 32-row blocks of O^T
  static constexpr int kKRow = D * kElem;                // bytes per K row in LDS (no padding)
  static constexpr int kKCh = kKRow / 16;                // 16-byte chunks per K row
  static constexpr int kVRow = DV * 2;                   // bytes per V row in LDS (bf16)
  static constexpr int kVCh = kVRow / 16;
  static constexpr int kKTile = kBlockN * kKRow;
  static constexpr int kVTile = kBlockN * kVRow;
  static constexpr int kKInstr = kKTile / 1024 / 4;      // direct-to-LDS instructions per wave per K tile
  static constexpr int kVInstr = kVTile / 1024 / 4;
  static constexpr int kSmem = 2 * kKTile + 2 * kVTile;
  // fp8 V goes through registers (to widen to bf16): 16-byte fp8 chunks per thread
  static constexpr int kV8Ch = DV / 16;
  static constexpr int kV8Loads = kBlockN * kV8Ch / kThreads;
  static_assert(kKInstr >= 1 && kVInstr >= 1, "tile too small for 4 waves");
  static_assert(!FP8 || kV8Loads >= 1, "fp8 V staging needs >= 1 chunk per thread");
};

// Chunk swizzle of LDS row R: chunk c of the row is stored in slot c ^ swz(R).
// swz is a bijection on 0..15 over any 16 consecutive rows (K operand reads)
// and its top two bits differ across any 4 rows 4m..4m+3 (V transpose reads).
__device__ __forceinline__ int swz(int row, int nchunks) {
  return (((row & 3) << 2) | ((row >> 2) & 3)) & (nchunks - 1);
}

template <bool B> struct BoolTag { static constexpr bool value = B; };

// Column-major V (keys contiguous in memory): the V^T tile sits in LDS as DV
// rows of 64 keys (128 B), 16-byte chunk c of row R in slot c ^ vt_swz(R), so
// the 32 rows x 2 chunks that one operand read touches fall in distinct banks.
__device__ __forceinline__ int vt_swz(int row) { return (row >> 1) & 7; }
// With column-major V the K tile's rows are loaded permuted within each 16-key
// block (rows 4-7 <-> 8-11), so that the 8 P values a lane feeds to one PV
// product belong to 8 consecutive keys, i.e. one 16-byte chunk of a V^T row.
__device__ __forceinline__ int k_row_perm(int r) {
  const int y = r & 15;
  return (r & ~15) | ((y >= 4 && y < 12) ? (y ^ 12) : y);
}

// Query tiles per dispatch group: two rounds of an XCD's resident workgroups
// (32 CUs, two workgroups each). Two rounds give the longest-first order room
// to pair heavy and light tiles; 64 (one round) measured 4% slower on causal
// B=4 H=16 s=2048, 32 slower still.
constexpr int kGroupTiles = 128;
// Units (sequence, kv-head) per dispatch group (at least one).
__host__ __device__ inline int group_units(int n_qtiles) {
  return n_qtiles >= kGroupTiles ? 1 : kGroupTiles / n_qtiles;
}

// Mask kinds (a template parameter, so the common causal mask costs one
// compare per score on the tiles it cuts): none; a right bound only (causal,
// or any window with window_left < 0); a window with a left bound (and sinks).
enum MaskKind : int { kMaskNone = 0, kMaskRight = 1, kMaskWindow = 2 };

template <int D, int DV, bool FP8, int MODE, int MK, bool SOFTCAP, int BIAS, bool VT>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a) {
  static_assert(!VT || (D == DV && MODE != kPrefillVarlenPaged),
                "column-major V: equal head dims, batch, varlen or paged mode");
  constexpr bool MASK = MK != kMaskNone;
  constexpr bool TWO_SIDED = MK == kMaskWindow;   // the host guarantees a.wl >= 0
  using Tr = Traits<D, DV, FP8>;
  // Separate LDS objects per slot: the compiler can then prove that reads of
  // one slot do not alias the HBM->LDS loads in flight into the other, and
  // does not wait for those loads before reading.
  __shared__ __attribute__((aligned(1024))) char k_lds0[Tr::kKTile];
  __shared__ __attribute__((aligned(1024))) char k_lds1[Tr::kKTile];
  __shared__ __attribute__((aligned(1024))) char v_lds0[Tr::kVTile];
  __shared__ __attribute__((aligned(1024))) char v_lds1[Tr::kVTile];

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int h = lane >> 5;          // which half of the key / d sub-blocks this lane holds
  // XCD-aware work order. Workgroups are dispatched round-robin over the 8
  // XCDs (hardware id w goes to XCD w % 8), each with its own L2. A unit is one
  // (sequence, kv-head): all its query tiles read the same K/V, so they run on
  // one XCD and share its L2. Units are dealt to the XCDs round-robin, so with
  // sequences of different lengths every XCD still gets a similar share of the
  // work (with Hkv a multiple of 8, XCD x takes kv-heads x, x+8, ... of every
  // sequence). Each XCD takes its units G at a time (G = group_units), G just
  // large enough for one group's query tiles to fill two rounds of the XCD's
  // slots, so the K/V of only about one group is live in L2. Inside a group, tiles go out
  // by rank across its units, heaviest (latest, under a causal mask) first:
  // the next group's heavy tiles then land on the slots that the previous
  // group's light tiles free first (longest-processing-time-first order),
  // instead of the last unit's heavy tiles starting when most slots are done.
  const int n_units = a.hkv * a.nz;
  const int xcd = (int)(blockIdx.x % kXcds);
  const int k_x = (int)(blockIdx.x / kXcds);       // position in this XCD's list
  const int G = group_units(a.n_qtiles);
  const int gsz = G * a.n_qtiles;
  // Balanced CU pairs. The dispatcher places positions c and c + C of an XCD's
  // list (C = its CU count) on CU c, two workgroups per CU, and the older
  // workgroup of a CU gets issue priority. Within every block of 4C positions
  // (two rounds of the XCD's slots) the second quarter is taken in reverse, so
  // each CU's first pair is (heavy, light) ranks, the heavier one older, and
  // every CU carries about the same number of key tiles. Measured on causal
  // B=4 H=16 s=2048: 82.7 -> 78.0 us; fewer than 256 of the 512 slots busy
  // for 6 us of the end instead of 12.
  int kk = k_x;
  {
    const int cx = a.cu_per_xcd, q = k_x % (4 * cx), b = k_x - q;
    if (q >= cx && q < 2 * cx && b + 2 * cx <= a.items_x) kk = b + 3 * cx - 1 - q;
  }
  const int qt_i = (kk % gsz) / G;                 // rank: 0 = heaviest
  const int unit = xcd + kXcds * ((kk / gsz) * G + (kk % gsz) % G);
  if (unit >= n_units) return;
  const int g = unit % a.hkv;                      // kv-head
  const int z = unit / a.hkv;                      // batch entry or sequence
  const int qt = MASK ? a.n_qtiles - 1 - qt_i : qt_i;

  // ---- sequence geometry (batch: seqused; varlen: cumulative offsets; paged:
  // Lq = sq, Lk = seqlens_k, K/V rows found through the block table) ----
  constexpr bool VARLEN = MODE == kPrefillVarlen;
  constexpr bool VPAGED = MODE == kPrefillVarlenPaged;        // varlen queries over a paged pool
  constexpr bool PAGED = MODE == kPrefillPaged || VPAGED;     // K/V rows through the block table
  int Lq, Lk;
  int64_t q_off, k_off, v_off, o_off, lse_off;
  int64_t bias_off = 0;  // elementwise bias: element offset of this sequence's row 0 (all heads)
  int kv0 = 0;       // logical position of key 0 in the sequence's page list
  // varlen-paged: a negative key start; varlen with column-major V: a key offset
  // or count off the 16-byte chunk grid -> NaN rows, no key read
  bool bad = false;
  if (VARLEN) {
    const int q0 = a.cu_q[z], k0 = a.cu_k[z];
    Lq = a.cu_q[z + 1] - q0;
    Lk = a.cu_k[z + 1] - k0;
    if (Lq <= a.min_seqlen_q) return;  // skipped sequence: its rows stay untouched
    q_off = (int64_t)q0 * a.q_sr;
    k_off = (int64_t)k0 * a.k_sr;
    // column-major V: keys run along the packed token axis, so the sequence's
    // keys start k0 elements into each head-dim row (a.v_sr is the row stride);
    // each 16-byte chunk of keys must belong to one sequence
    v_off = VT ? (int64_t)k0 : (int64_t)k0 * a.v_sr;
    if (VT && ((k0 | Lk) & (16 / Tr::kElem - 1))) {
      bad = true;
      Lk = 0;
    }
    o_off = (int64_t)q0 * a.o_sr;
    lse_off = q0;
    bias_off = (int64_t)q0 * a.bias_sr;  // group mode: rows follow the packed query tokens
  } else if (VPAGED) {
    const int q0 = a.cu_q[z];
    Lq = a.cu_q[z + 1] - q0;
    Lk = a.seqused_k[z];
    if (Lq <= a.min_seqlen_q) return;  // skipped sequence: its rows stay untouched
    kv0 = a.kv_start ? a.kv_start[z] : 0;
    if (kv0 < 0) {
      bad = true;
      kv0 = 0;
      Lk = 0;
    }
    q_off = (int64_t)q0 * a.q_sr;
    k_off = 0;  // pool base; pages are found per tile
    v_off = 0;
    o_off = (int64_t)q0 * a.o_sr;
    lse_off = q0;
    bias_off = (int64_t)q0 * a.bias_sr;
  } else if (PAGED) {
    Lq = a.sq;
    Lk = a.seqused_k[z];
    q_off = (int64_t)z * a.q_sb;
    k_off = 0;  // pool base; pages are found per tile
    v_off = 0;
    o_off = (int64_t)z * a.o_sb;
    lse_off = (int64_t)z * a.lse_sb;
    bias_off = (int64_t)z * a.bias_sb;
  } else {
    Lq = a.seqused_q ? a.seqused_q[z] : a.sq;
    Lk = a.seqused_k ? a.seqused_k[z] : a.sk;
    // K/V batch entry (cache batch index); an out-of-range index reads no keys
    int kz = kv_entry(a.cache_idx, a.cache_count, z);
    if (kz < 0) {
      kz = 0;
      Lk = 0;
    }
    q_off = (int64_t)z * a.q_sb;
    k_off = (int64_t)kz * a.k_sb;
    v_off = (int64_t)kz * a.v_sb;
    o_off = (int64_t)z * a.o_sb;
    lse_off = (int64_t)z * a.lse_sb;
    bias_off = (int64_t)z * a.bias_sb;
  }
  if (!a.k || !a.v) Lk = 0;  // NULL K or V: no keys, whatever the length arrays say
  const int ratio = a.ratio;
  const int rows_total = Lq * ratio;
  const int r0 = qt * kBlockM;
  if (r0 >= rows_total) return;  // tile past this sequence's end (whole workgroup)

  const int off = Lk - Lq;       // bottom-right alignment of the mask diagonal
  const int p_lo = r0 / ratio;
  const int p_hi = (min(r0 + kBlockM, rows_total) - 1) / ratio;
  int j_lo = 0, j_hi = Lk;
  if (MASK) {
    if (a.wl >= 0 && a.sink_size <= 0) j_lo = max(0, p_lo + off - a.wl);  // sink keys start at 0
    if (a.wr >= 0) j_hi = min(Lk, p_hi + off + a.wr + 1);
  }
  const int t_begin = j_lo / kBlockN;
  const int t_end = (j_hi > j_lo) ? (j_hi + kBlockN - 1) / kBlockN : t_begin;

  // ---- this lane's query row; the wave's row range (scalar) ----
  const int row = r0 + wave * 32 + (lane & 31);
  const bool row_ok = row < rows_total;
  const int pos = row / ratio;
  const int hq = g * ratio + row % ratio;
  const int wr0 = r0 + wave * 32;
  const int pw_lo = wr0 / ratio;
  const int pw_hi = (min(wr0 + 32, rows_total) - 1) / ratio;
  int lim_lo = 0, lim_hi = Lk - 1;  // visible keys of this row: lim_lo <= j <= lim_hi
  if (MASK) {
    if (a.wr >= 0) lim_hi = min(Lk - 1, pos + off + a.wr);
    if (a.wl >= 0) lim_lo = pos + off - a.wl;
  }
  // ALiBi slope of this row's (batch entry or sequence, q-head), in kernel logit units
  const float alibi_k = BIAS == kBiasAlibi ? a.bias[(int64_t)z * a.bias_sb + hq] * a.bias_mul : 0.0f;
  // elementwise bias: this lane's row (64-bit address). Lanes past the tile's
  // used rows read row 0 of their head (in the tensor; never stored). Keys are
  // read as aligned 16-byte blocks of 4, clamped to the block holding key
  // Lk - 1, so every load lies in a block that holds a used element.
  const float* bias_row = BIAS == kBiasElem
                              ? a.bias + bias_off + (int64_t)hq * a.bias_sh + (int64_t)(row_ok ? pos : 0) * a.bias_sr
                              : nullptr;
  const int bias_last = (Lk - 1) & ~3;

  // ---- Q fragment, resident in registers for the whole key loop ----
  // B operand of S^T = K Q^T. bf16: lane (row lane%32, half h) holds Q[row][16s + 8h .. +7] for step s of
  // 32x32x16 products. fp8: it holds Q[row][64s + 32h .. +31] (chunks 2s, 2s + 1 of
  // qf) for step s of 32x32x64 products.
  U128 qf[FP8 ? D / 32 : Tr::kQkSteps];
  {
    const char* qp = (const char*)a.q + (q_off + (int64_t)hq * a.q_sh + (int64_t)pos * a.q_sr) * Tr::kElem;
#pragma unroll
    for (int s = 0; s < (FP8 ? D / 32 : Tr::kQkSteps); ++s) {
      const int byte = FP8 ? 64 * (s >> 1) + 32 * h + 16 * (s & 1) : (16 * s + 8 * h) * 2;
      qf[s] = row_ok ? *(const U128*)(qp + byte) : U128{0, 0, 0, 0};
    }
  }

  // ---- K/V staging: HBM -> LDS directly; rows past Lk arrive as zeros ----
  const char* kh = (const char*)a.k + (k_off + (int64_t)g * a.k_sh) * Tr::kElem;
  const char* vh = (const char*)a.v + (v_off + (int64_t)g * a.v_sh) * Tr::kElem;
  // start of the 64 rows of tile j0 / 64: contiguous, or (paged) the tile's page
  // plus the in-page offset, as in the page-block navigator of the Composable
  // Kernel page (page_size is a multiple of 64, so with a key start that is a
  // multiple of 64 a tile lies in one page; other tiles are split below)
  auto tile_rows = [&](const char* head_base, int64_t page_stride, int64_t row_bytes, int j0) -> const char* {
    if (PAGED) {
      const int jl = kv0 + j0;  // logical token position in the page list
      const int page = a.block_table[(int64_t)z * a.bt_stride + jl / a.page_size];
      return head_base + (int64_t)page * page_stride * Tr::kElem + (int64_t)(jl % a.page_size) * row_bytes;
    }
    return head_base + j0 * row_bytes;
  };
  const int64_t krow = a.k_sr * Tr::kElem, vrow = a.v_sr * Tr::kElem;  // global bytes per key row
  // Varlen over a paged pool with a key start that is not a multiple of 64: a
  // 64-key tile can straddle two pages. Rows 0 .. na-1 of tile j0 lie at the end
  // of one page, rows na .. at the start of the next; such a tile is loaded in
  // two lane-masked parts, each through its own page's buffer range.
  auto rows_in_first_page = [&](int j0) -> int {
    return VPAGED ? a.page_size - (kv0 + j0) % a.page_size : kBlockN;
  };
  auto page_base = [&](const char* head_base, int64_t page_stride, int jl) -> const char* {
    const int page = a.block_table[(int64_t)z * a.bt_stride + jl / a.page_size];
    return head_base + (int64_t)page * page_stride * Tr::kElem;
  };
  // LDS addresses stay in the LDS address space (a generic pointer converted
  // back would cost a null check per use)
  lds_char* const kl0 = (lds_char*)k_lds0;
  lds_char* const kl1 = (lds_char*)k_lds1;
  lds_char* const vl0 = (lds_char*)v_lds0;
  lds_char* const vl1 = (lds_char*)v_lds1;
  auto kslot = [&](int slot) -> lds_char* { return slot ? kl1 : kl0; };
  auto vslot = [&](int slot) -> lds_char* { return slot ? vl1 : vl0; };
  // K row swizzle. bf16 rows (256 B) use swz; fp8 rows (128 or 64 B) rotate
  // their chunks by the row's index among the rows sharing a 256-byte bank
  // window, so the 16 rows of a 16-byte operand read hit 16 different banks.
  auto kswz = [](int R) -> int {
    return FP8 ? (R / (256 / Tr::kKRow)) & (Tr::kKCh - 1) : swz(R, Tr::kKCh);
  };
  // Wave w fills LDS blocks w, w+4, ... (1 KiB each) of a tile; lane l of block q
  // covers LDS bytes 1024 q + 16 l = (row R, slot s), fetching global chunk s ^ kswz(R) of
  // a K row (s ^ swz(R) of a V row).
  int koff[Tr::kKInstr], voff[Tr::kVInstr];
#pragma unroll
  for (int i = 0; i < Tr::kKInstr; ++i) {
    const int B = 1024 * (wave + 4 * i) + 16 * lane;
    const int R = B / Tr::kKRow, sl = (B % Tr::kKRow) / 16;
    koff[i] = (int)((VT ? k_row_perm(R) : R) * krow) + 16 * (sl ^ kswz(R));
  }
#pragma unroll
  for (int i = 0; i < Tr::kVInstr; ++i) {
    const int B = 1024 * (wave + 4 * i) + 16 * lane;
    const int R = B / Tr::kVRow, sl = (B % Tr::kVRow) / 16;
    voff[i] = (int)(R * vrow) + 16 * (sl ^ swz(R, Tr::kVCh));
  }
  // column-major V: lane l of block q fetches row R = 8 q + l / 8 (a head-dim
  // index), global chunk kc = (l % 8) ^ vt_swz(R) (keys 8 kc .. 8 kc + 7 of the tile)
  int vt_kc[VT ? Tr::kVInstr : 1];
#pragma unroll
  for (int i = 0; i < (VT ? Tr::kVInstr : 0); ++i) {
    const int R = 8 * (wave + 4 * i) + (lane >> 3);
    vt_kc[i] = (lane & 7) ^ vt_swz(R);
    voff[i] = (int)(R * vrow) + 16 * vt_kc[i];
  }
  auto load_k = [&](int t, int slot) {
    const int j0 = t * kBlockN;
    const int rows = min(kBlockN, Lk - j0);
    lds_char* base = kslot(slot);
    const int na = rows_in_first_page(j0);
    if (VPAGED && na < rows) {
      const int jl = kv0 + j0;
      const __amdgpu_buffer_rsrc_t ra =
          make_rsrc(page_base(kh, a.k_sb, jl) + (int64_t)(jl % a.page_size) * krow, (uint32_t)(na * krow));
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(page_base(kh, a.k_sb, jl + na), (uint32_t)((rows - na) * krow));
#pragma unroll
      for (int i = 0; i < Tr::kKInstr; ++i) {
        const int R = (1024 * (wave + 4 * i) + 16 * lane) / Tr::kKRow;   // tile row of this lane's chunk
        if (R < na) buf_load16_lds(ra, base + 1024 * (wave + 4 * i), koff[i]);
        else buf_load16_lds(rb, base + 1024 * (wave + 4 * i), koff[i] - na * (int)krow);
      }
      return;
    }
    const __amdgpu_buffer_rsrc_t r = make_rsrc(tile_rows(kh, a.k_sb, krow, j0), (uint32_t)(rows * krow));
#pragma unroll
    for (int i = 0; i < Tr::kKInstr; ++i) buf_load16_lds(r, base + 1024 * (wave + 4 * i), koff[i]);
  };
  // fp8 V: through registers, widened to bf16 on the way into LDS
  U128 v8[FP8 ? Tr::kV8Loads : 1];
  const int v8ch = threadIdx.x % Tr::kV8Ch, v8row = threadIdx.x / Tr::kV8Ch;
  // column-major V: the tile's 64 keys of every head-dim row start here (batch:
  // key j0 of the head; paged: the tile's page, keys contiguous within it as in
  // the page's non-row-major V view [hdim_v, page_block_size])
  auto vt_tile_base = [&](int j0) -> const char* {
    if (PAGED) {
      const int page = a.block_table[(int64_t)z * a.bt_stride + j0 / a.page_size];
      return vh + ((int64_t)page * a.v_sb + (j0 % a.page_size)) * Tr::kElem;
    }
    return vh + (int64_t)j0 * Tr::kElem;
  };
  auto load_v = [&](int t, int slot) {
    const int j0 = t * kBlockN;
    if (VT) {
      // rows are head-dim indices (row stride vrow); chunks of keys at or past Lk
      // get an offset beyond the range and arrive as zeros
      const __amdgpu_buffer_rsrc_t r =
          make_rsrc(vt_tile_base(j0), (uint32_t)((DV - 1) * vrow + Tr::kElem * kBlockN));
      if (FP8) {
        // 16-key fp8 chunks into registers (chunk i of this thread: head-dim row
        // ci / 4, keys 16 (ci % 4) .., ci = threadIdx.x + 256 i)
#pragma unroll
        for (int i = 0; i < Tr::kV8Loads; ++i) {
          const int ci = threadIdx.x + kThreads * i;
          const int c = ci & 3;
          v8[i] = buf_load16(r, j0 + 16 * c < Lk ? (int)((ci >> 2) * vrow) + 16 * c : 0x7FFFFFF0);
        }
        return;
      }
      lds_char* base = vslot(slot);
#pragma unroll
      for (int i = 0; i < Tr::kVInstr; ++i)
        buf_load16_lds(r, base + 1024 * (wave + 4 * i), j0 + 8 * vt_kc[i] < Lk ? voff[i] : 0x7FFFFFF0);
      return;
    }
    const int rows = min(kBlockN, Lk - j0);
    const int na = rows_in_first_page(j0);
    if (VPAGED && na < rows) {
      const int jl = kv0 + j0;
      const __amdgpu_buffer_rsrc_t ra =
          make_rsrc(page_base(vh, a.v_sb, jl) + (int64_t)(jl % a.page_size) * vrow, (uint32_t)(na * vrow));
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(page_base(vh, a.v_sb, jl + na), (uint32_t)((rows - na) * vrow));
      if (FP8) {
#pragma unroll
        for (int i = 0; i < Tr::kV8Loads; ++i) {
          const int R = v8row + i * (kThreads / Tr::kV8Ch);
          const int off = (int)(R * vrow) + 16 * v8ch;
          v8[i] = R < na ? buf_load16(ra, off) : buf_load16(rb, off - na * (int)vrow);
        }
      } else {
        lds_char* base = vslot(slot);
#pragma unroll
        for (int i = 0; i < Tr::kVInstr; ++i) {
          const int R = (1024 * (wave + 4 * i) + 16 * lane) / Tr::kVRow;
          if (R < na) buf_load16_lds(ra, base + 1024 * (wave + 4 * i), voff[i]);
          else buf_load16_lds(rb, base + 1024 * (wave + 4 * i), voff[i] - na * (int)vrow);
        }
      }
      return;
    }
    const __amdgpu_buffer_rsrc_t r = make_rsrc(tile_rows(vh, a.v_sb, vrow, j0), (uint32_t)(rows * vrow));
    if (FP8) {
#pragma unroll
      for (int i = 0; i < Tr::kV8Loads; ++i)
        v8[i] = buf_load16(r, (int)((v8row + i * (kThreads / Tr::kV8Ch)) * vrow) + 16 * v8ch);
    } else {
      lds_char* base = vslot(slot);
#pragma unroll
      for (int i = 0; i < Tr::kVInstr; ++i) buf_load16_lds(r, base + 1024 * (wave + 4 * i), voff[i]);
    }
  };
  auto store_v8 = [&](int slot, int t) {  // fp8 only: widen tile t's V into LDS slot `slot`
    lds_char* base = vslot(slot);
    if (VT) {
      // V^T rows of 64 keys as bf16 (the bf16 column-major layout); keys at or
      // past Lk in the chunk holding key Lk - 1 (any bits) are zeroed here
      const int j0 = t * kBlockN;
#pragma unroll
      for (int i = 0; i < (FP8 ? Tr::kV8Loads : 0); ++i) {
        const int ci = threadIdx.x + kThreads * i;
        const int R = ci >> 2, c = ci & 3;
        U128 lo = fp8x8_to_bf16x8(U64{v8[i].x, v8[i].y}), hi = fp8x8_to_bf16x8(U64{v8[i].z, v8[i].w});
        const int nv = Lk - (j0 + 16 * c);  // keys of this chunk below Lk
        if (nv < 16) {
          uint32_t* w = &lo.x;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            w[e / 2] &= (e < nv ? 0xFFFFu : 0u) | (e + 1 < nv ? 0xFFFF0000u : 0u);
          }
          w = &hi.x;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            w[e / 2] &= (8 + e < nv ? 0xFFFFu : 0u) | (9 + e < nv ? 0xFFFF0000u : 0u);
          }
        }
        // a 16-byte LDS store resolves bank conflicts per 8 lanes over 128 bytes:
        // odd rows store their high chunk first, so the 8 lanes (rows 2m, 2m + 1,
        // 128 bytes each, same swizzle) hit 8 distinct slots
        const int f = R & 1;
        lds_store16(base + R * (2 * kBlockN) + 16 * ((2 * c + f) ^ vt_swz(R)), f ? hi : lo);
        lds_store16(base + R * (2 * kBlockN) + 16 * ((2 * c + 1 - f) ^ vt_swz(R)), f ? lo : hi);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < (FP8 ? Tr::kV8Loads : 0); ++i) {
      const int R = v8row + i * (kThreads / Tr::kV8Ch);
      const int c0 = 2 * v8ch;  // bf16 chunks 2c, 2c+1 of the row
      const U128 lo = fp8x8_to_bf16x8(U64{v8[i].x, v8[i].y}), hi = fp8x8_to_bf16x8(U64{v8[i].z, v8[i].w});
      // a 16-byte LDS store resolves bank conflicts per 8 lanes over 128 bytes;
      // threads 4 .. 7 of each 8 store their high chunk first, so the 8 threads'
      // 32-byte chunk pairs (256 contiguous bytes before the swizzle, which XORs
      // the slot with a constant per 8 threads) hit 8 distinct slots modulo 128 bytes
      const int f = (threadIdx.x >> 2) & 1;
      lds_store16(base + R * Tr::kVRow + 16 * ((c0 + f) ^ swz(R, Tr::kVCh)), f ? hi : lo);
      lds_store16(base + R * Tr::kVRow + 16 * ((c0 + 1 - f) ^ swz(R, Tr::kVCh)), f ? lo : hi);
    }
  };

  // lane-constant LDS read offsets. K operand: row lane%32 (+32 for the second
  // block, same swizzle), chunk (16 kk + 8 h) * elem / 16.
  const int kR = lane & 31;
  const int k_swz = kswz(kR);
  auto k_addr = [&](int kk) -> int {
    const int byte = (16 * kk + 8 * h) * Tr::kElem;
    return kR * Tr::kKRow + 16 * ((byte >> 4) ^ k_swz) + (byte & 15);
  };
  // V transpose read of group (lanes 16 gi .. 16 gi + 15, L = lane & 15): rows
  // kb + 8 a + 4 (gi >> 1) + L / 4, bf16 columns 32 dblk + 16 (gi & 1) + 4 (L & 3).
  const int L = lane & 15;
  const int gi = lane >> 4;
  auto v_addr = [&](int kb, int aa, int dblk) -> int {
    const int R = kb + 8 * aa + 4 * (gi >> 1) + (L >> 2);
    const int byte = 2 * (32 * dblk + 16 * (gi & 1) + 4 * (L & 3));
    return R * Tr::kVRow + 16 * ((byte >> 4) ^ swz(R, Tr::kVCh)) + (byte & 15);
  };

  const float c = a.c_exp2;
  // Soft-capped logits without an additive bias never exceed post = cap log2(e)
  // (kernel units, where c = 1). For caps up to ~41 (2 post <= 120) the fixed
  // reference m = post then needs no row max and no rescale: every p =
  // 2^(s' - post) lies in [2^-(2 post), 1], far from fp32 and bf16 underflow.
  const bool capped = SOFTCAP && BIAS == kBiasNone && a.softcap_post <= 60.0f;
  float m_run = capped ? a.softcap_post : kNegInf;   // reference max (raised lazily, see below)
  float l_run = 0.0f;      // this lane's partial row sum (its half of the keys)
  float mc_run = 0.0f;     // m_run c (general softmax path; 0 until a key is visible)
  f32x16 acc[Tr::kDBlocks];
#pragma unroll
  for (int i = 0; i < Tr::kDBlocks; ++i) acc[i] = f32x16{};

  // K operand addresses of the bf16 steps, kept in registers (an XOR with the
  // lane's swizzle, so not an immediate offset): one add less per step and tile
  int kaddr[Tr::kQkSteps];
#pragma unroll
  for (int kk = 0; kk < Tr::kQkSteps; ++kk) {
    kaddr[kk] = k_addr(kk);
    asm volatile("" : "+v"(kaddr[kk]));  // keep the value, do not rematerialise it per tile
  }
  // S^T = K Q^T for the tile in K slot `slot`: two interleaved 32-key chains
  auto qk = [&](int slot, f32x16& s0, f32x16& s1) {
    const lds_char* kt = kslot(slot);
    s0 = f32x16{};
    s1 = f32x16{};
    if (FP8) {
      // 32x32x64 products: lane (key lane%32, half h) reads K[key][64 kk + 32 h .. +31],
      // chunks 4 kk + 2 h and 4 kk + 2 h + 1 of its LDS row
#pragma unroll
      for (int kk = 0; kk < D / 64; ++kk) {
        const lds_char* r = kt + kR * Tr::kKRow;
        const int c0 = 16 * ((4 * kk + 2 * h) ^ k_swz), c1 = 16 * ((4 * kk + 2 * h + 1) ^ k_swz);
        s0 = mfma32x64_fp8(lds_load16(r + c0), lds_load16(r + c1), qf[2 * kk], qf[2 * kk + 1], s0);
        s1 = mfma32x64_fp8(lds_load16(r + 32 * Tr::kKRow + c0), lds_load16(r + 32 * Tr::kKRow + c1),
                           qf[2 * kk], qf[2 * kk + 1], s1);
      }
    } else {
      // operands of step kk+1 are read while step kk's products run
      U128 a0 = lds_load16(kt + kaddr[0]);
      U128 a1 = lds_load16(kt + kaddr[0] + 32 * Tr::kKRow);
#pragma unroll
      for (int kk = 0; kk < Tr::kQkSteps; ++kk) {
        U128 n0 = a0, n1 = a1;
        if (kk + 1 < Tr::kQkSteps) {
          n0 = lds_load16(kt + kaddr[kk + 1]);
          n1 = lds_load16(kt + kaddr[kk + 1] + 32 * Tr::kKRow);
        }
        __builtin_amdgcn_sched_barrier(0);
        s0 = mfma32_bf16(as_bf16x8(a0), as_bf16x8(*(const U128*)&qf[kk]), s0);
        s1 = mfma32_bf16(as_bf16x8(a1), as_bf16x8(*(const U128*)&qf[kk]), s1);
        a0 = n0;
        a1 = n1;
      }
    }
  };

  // Softmax of tile t's scores (s0, s1) into bf16 P, with the lazy rescale of O.
  // Register r of block b is key j0 + 32b + 8(r/4) + 4h + r%4 of this lane's row.
  // Score register r of block b in lane half h is key j0 + kHStep h + key_rel(b, r)
  // (the S^T row of the register, through the K row permutation with column-major V).
  constexpr int kHStep = VT ? 8 : 4;
  auto key_rel = [](int b, int r) -> int {
    return VT ? 32 * b + 16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3) : 32 * b + 8 * (r >> 2) + (r & 3);
  };
  auto softmax = [&](auto masked_tag, int t, f32x16 s0, f32x16 s1, uint32_t (&pk)[2][8]) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    const int j0 = t * kBlockN;
    f32x16 s[2] = {s0, s1};
    if (SOFTCAP && BIAS == kBiasNone && capped) {
      // p = 2^(s' - post) with s' = post (1 - 2 r), r = 1 / (1 + e^(2y)): p = 2^(-2 post r)
      // q2 r = q2 / (1 + e) = 1 / fma(e, 1/q2, 1/q2): one FMA instead of an add and a multiply
      const float k2 = 2.0f * kLog2e * a.softcap_pre, iq2 = -0.5f / a.softcap_post;
      const int hi = lim_hi - j0 - kHStep * h;
      const int lo = lim_lo - j0 - kHStep * h;
      const int sk = a.sink_size - j0 - kHStep * h;
      constexpr bool two_sided = TWO_SIDED;
      float ls[4];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float e0 = fast_rcp(__builtin_fmaf(fast_exp2(s[b][r] * k2), iq2, iq2));
          float e1 = fast_rcp(__builtin_fmaf(fast_exp2(s[b][r + 1] * k2), iq2, iq2));
          if (kMasked) {
            const int j0r = key_rel(b, r), j1r = key_rel(b, r + 1);
            e0 = ((j0r <= hi) && (!two_sided || j0r >= lo || j0r < sk)) ? e0 : kNegInf;
            e1 = ((j1r <= hi) && (!two_sided || j1r >= lo || j1r < sk)) ? e1 : kNegInf;
          }
          const float p0 = fast_exp2(e0), p1 = fast_exp2(e1);
          if (b == 0 && r < 8) ls[r >> 1] = p0 + p1;  // first pair of each partial sum (0 + x is not folded)
          else ls[(r >> 1) & 3] += p0 + p1;
          pk[b][r >> 1] = pack_bf16x2(p0, p1);
        }
      }
      l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
      return 1.0f;
    }
    if (SOFTCAP) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[b][r] = softcap_logit(s[b][r], 2.0f * kLog2e * a.softcap_pre, a.softcap_post);
    }
    // additive bias (after the soft-cap, before the mask); register r of block b
    // is key j0 + 4h + 32b + 8(r/4) + r%4
    if (BIAS == kBiasAlibi) {
      const float dbase = (float)(pos + off - j0 - kHStep * h);  // distance to key j0 + kHStep h
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float jr = (float)key_rel(b, r);
          s[b][r] = __builtin_fmaf(-alibi_k, __builtin_fabsf(dbase - jr), s[b][r]);
        }
    }
    if (BIAS == kBiasElem) {
      // 16-byte loads of 4 consecutive keys (keys at or past Lk are masked below)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        U128 bv[4];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          bv[g4] = *(const U128*)(bias_row + min(j0 + kHStep * h + key_rel(b, 4 * g4), bias_last));
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t w = (&bv[r >> 2].x)[r & 3];
          s[b][r] = __builtin_fmaf(__builtin_bit_cast(float, w), a.bias_mul, s[b][r]);
        }
      }
    }
    if (kMasked) {
      const int hi = lim_hi - j0 - kHStep * h;
      const int lo = lim_lo - j0 - kHStep * h;
      const int sk = a.sink_size - j0 - kHStep * h;  // sink keys ignore the left bound
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jr = key_rel(b, r);
          const bool vis = (jr <= hi) && (!TWO_SIDED || jr >= lo || jr < sk);
          s[b][r] = vis ? s[b][r] : kNegInf;
        }
    }
    // row max: four independent chains (each starting at -inf, which lets the
    // compiler use v_max3 without NaN canonicalisation), then the lane halves
    float mx[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      mx[q] = kNegInf;
#pragma unroll
      for (int i = 0; i < 4; ++i) mx[q] = __builtin_fmaxf(mx[q], s[q >> 1][8 * (q & 1) + i]);
#pragma unroll
      for (int i = 4; i < 8; ++i) mx[q] = __builtin_fmaxf(mx[q], s[q >> 1][8 * (q & 1) + i]);
    }
    float mrow = kNegInf;
#pragma unroll
    for (int q = 0; q < 4; ++q) mrow = __builtin_fmaxf(mrow, mx[q]);
    const float mt = max_across_halves(mrow);

    // Lazy rescale: the reference max only moves when the tile max exceeds it
    // by more than 8 in log2 units, so P <= 2^8 and the rescale of O and l is
    // rare. O / l and m + log2(l) are unchanged by the choice of reference.
    const float dc = (mt - m_run) * c;   // +inf when m_run = -inf and mt is finite; NaN when both are -inf
    const bool raise = dc > 8.0f;
    const float alpha = raise ? fast_exp2(-dc) : 1.0f;   // 0 when m_run = -inf
    m_run = raise ? mt : m_run;
    mc_run = raise ? mt * c : mc_run;    // m_run c, or 0 while every key seen so far is masked
    l_run *= alpha;
    const float mc = mc_run;

    // P = exp2(x c - m c), packed to bf16 pairs in MFMA B-operand order;
    // four independent partial sums
    float ls[4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s[b][r], c, -mc));
        const float p1 = fast_exp2(__builtin_fmaf(s[b][r + 1], c, -mc));
        if (b == 0 && r < 8) ls[r >> 1] = p0 + p1;  // first pair of each partial sum (0 + x is not folded)
        else ls[(r >> 1) & 3] += p0 + p1;
        pk[b][r >> 1] = pack_bf16x2(p0, p1);
      }
    }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    return alpha;
  };

  // O^T = alpha O^T + V^T P^T over four 16-key steps (V slot `vslot`)
  auto pv = [&](int vs, float alpha, const uint32_t (&pk)[2][8]) {
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int i = 0; i < Tr::kDBlocks; ++i) acc[i] *= alpha;
    }
    const lds_char* vt = vslot(vs);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int gm = 0; gm < 2; ++gm) {
        const U128 pu{pk[b][4 * gm], pk[b][4 * gm + 1], pk[b][4 * gm + 2], pk[b][4 * gm + 3]};
        const bf16x8 pb = as_bf16x8(pu);
        const int kb = 32 * b + 16 * gm;
#pragma unroll
        for (int dblk = 0; dblk < Tr::kDBlocks; ++dblk) {
          if (VT) {  // keys kb + 8h .. +7 of head-dim row 32 dblk + lane % 32: one chunk
            const int R = 32 * dblk + (lane & 31);
            const U128 vv = lds_load16(vt + R * (2 * kBlockN) + 16 * (((kb >> 3) + h) ^ vt_swz(R)));
            acc[dblk] = mfma32_bf16(as_bf16x8(vv), pb, acc[dblk]);
          } else {
            const U64 v0 = lds_read_tr16(vt + v_addr(kb, 0, dblk));
            const U64 v1 = lds_read_tr16(vt + v_addr(kb, 1, dblk));
            acc[dblk] = mfma32_bf16(as_bf16x8(v0, v1), pb, acc[dblk]);
          }
        }
      }
    }
  };

  using MaskedT = BoolTag<true>;
  using PlainT = BoolTag<false>;

  // does no row of this wave see any key of tile t?
  auto tile_skipped = [&](int t) {
    const int j0 = t * kBlockN;
    bool skip = wr0 >= rows_total;
    if (MASK) {
      if (a.wr >= 0 && j0 > pw_hi + off + a.wr) skip = true;
      if (a.wl >= 0 && j0 + kBlockN - 1 < pw_lo + off - a.wl && j0 >= a.sink_size) skip = true;
    }
    return skip;
  };
  // does some row of this wave see only part of tile t (mask edge or Lk tail)?
  auto tile_needs_mask = [&](int t) {
    const int j0 = t * kBlockN;
    bool need = j0 + kBlockN > Lk;
    if (MASK) {
      if (a.wr >= 0 && j0 + kBlockN - 1 > pw_lo + off + a.wr) need = true;
      if (a.wl >= 0 && j0 < pw_hi + off - a.wl) need = true;
    }
    return need;
  };

  if (t_begin < t_end) {
    // Tile t lives in LDS slot (t - t0) % 2; the loads of tile t+1 into the
    // other slot are in flight (HBM -> LDS) while tile t is computed.
    load_k(t_begin, 0);
    load_v(t_begin, 0);
    if (FP8) store_v8(0, t_begin);
    wait_vmem();
    __syncthreads();
    auto step = [&](auto parity_tag, int t) {
      constexpr int P = decltype(parity_tag)::value ? 1 : 0;
      const bool has1 = t + 1 < t_end;
      if (VT && !FP8 && !has1) {
        // the chunk holding key Lk - 1 also brought keys Lk .. (past the used
        // length, possibly not finite): zero them before any product reads them
        const int rem = Lk - t * kBlockN;
        if (rem > 0 && rem < kBlockN && (rem & 7)) {
          if ((int)threadIdx.x < DV) {
            const int R = threadIdx.x;
            lds_char* row = vslot(P) + R * (2 * kBlockN) + 16 * ((rem >> 3) ^ vt_swz(R));
            for (int e = rem & 7; e < 8; ++e) *(__attribute__((address_space(3))) uint16_t*)(row + 2 * e) = 0;
          }
          __syncthreads();
        }
      }
      if (has1) {
        load_k(t + 1, 1 - P);
        load_v(t + 1, 1 - P);
      }
      if (!tile_skipped(t)) {
        f32x16 s0, s1;
        qk(P, s0, s1);
        uint32_t pk[2][8];
        const float alpha =
            tile_needs_mask(t) ? softmax(MaskedT{}, t, s0, s1, pk) : softmax(PlainT{}, t, s0, s1, pk);
        pv(P, alpha, pk);
      }
      if (FP8 && has1) store_v8(1 - P, t + 1);
      wait_vmem();
      __syncthreads();
    };
    for (int t = t_begin; t < t_end; t += 2) {
      step(BoolTag<false>{}, t);
      if (t + 1 >= t_end) break;
      step(BoolTag<true>{}, t + 1);
    }
  }

  // ---- epilogue: normalise, LSE, stores (rows < Lq only) ----
  const float l_tot = sum_across_halves(l_run);
  const bool empty = !(l_tot > 0.0f);  // no visible key: O = 0, LSE = -inf (or the sink logit)
  float inv = empty ? 0.0f : a.o_mul / l_tot;
  float lse2 = empty ? kNegInf : m_run * c + __builtin_log2f(l_tot);  // log2 units
  if (a.sink_logits) {
    // one more denominator term 2^sk2 (the sink logit in log2 units), no value row
    const float sk2 = a.sink_logits[hq] * kLog2e;
    if (empty) {
      lse2 = sk2;
    } else if (sk2 > kNegInf) {
      const float mc = m_run * c;
      if (sk2 <= mc) {
        const float l2 = l_tot + fast_exp2(sk2 - mc);
        inv = a.o_mul / l2;
        lse2 = mc + __builtin_log2f(l2);
      } else {  // scale by 2^(mc - sk2) <= 1 so nothing overflows
        const float f = fast_exp2(mc - sk2);
        const float l2 = l_tot * f + 1.0f;
        inv = a.o_mul * f / l2;
        lse2 = sk2 + __builtin_log2f(l2);
      }
    }
  }
  if ((VPAGED || (VARLEN && VT)) && bad) {  // not computed: NaN rows
    inv = __builtin_nanf("");
    lse2 = __builtin_nanf("");
  }
  if (!a.out_fp8) {
    // bf16 O through LDS: each lane holds 4-element pieces of its own row, so
    // direct stores would touch 64 rows per instruction. The wave stages its
    // 32 x DV tile (row-major, 16-byte chunks XOR-swizzled by row) in a slice of
    // the V buffers, which no wave reads after the key loop's last barrier,
    // and writes it back 16 bytes per lane, whole rows per instruction.
    constexpr int kPitch = DV * 2;            // bytes per staged row
    constexpr int kNch = DV / 8;              // 16-byte chunks per row
    constexpr int kRowsPer = 64 / kNch;       // rows per wave store
    lds_char* const st = (wave < 2 ? vl0 : vl1) + (wave & 1) * 32 * kPitch;
    const int ri = lane & 31;
#pragma unroll
    for (int dblk = 0; dblk < Tr::kDBlocks; ++dblk) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        U64 w;
        w.x = pack_bf16x2(acc[dblk][4 * q4 + 0] * inv, acc[dblk][4 * q4 + 1] * inv);
        w.y = pack_bf16x2(acc[dblk][4 * q4 + 2] * inv, acc[dblk][4 * q4 + 3] * inv);
        const int ch = 4 * dblk + q4;  // columns 8 ch .. 8 ch + 7; this lane's half at + 4 h
        lds_store8(st + ri * kPitch + 16 * (ch ^ (ri & (kNch - 1))) + 8 * h, w);
      }
    }
#pragma unroll
    for (int k = 0; k < 32 / kRowsPer; ++k) {
      const int r = k * kRowsPer + lane / kNch;
      const int cc = lane % kNch;
      const U128 v = lds_load16(st + r * kPitch + 16 * (cc ^ (r & (kNch - 1))));
      const int grow = wr0 + r;
      if (grow < rows_total) {
        const int pr = grow / ratio;
        const int hr = g * ratio + grow % ratio;
        *(U128*)((char*)a.o + (o_off + (int64_t)hr * a.o_sh + (int64_t)pr * a.o_sr) * 2 + 16 * cc) = v;
      }
    }
  } else if (row_ok) {
    char* op = (char*)a.o + (o_off + (int64_t)hq * a.o_sh + (int64_t)pos * a.o_sr);
#pragma unroll
    for (int dblk = 0; dblk < Tr::kDBlocks; ++dblk) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * dblk + 8 * q4 + 4 * h;
        if ((VPAGED || (VARLEN && VT)) && bad) {  // the E4M3FN NaN byte
          *(uint32_t*)(op + d) = 0x7F7F7F7Fu;
        } else {
          *(uint32_t*)(op + d) = pack_fp8x4_sat(acc[dblk][4 * q4 + 0] * inv, acc[dblk][4 * q4 + 1] * inv,
                                                acc[dblk][4 * q4 + 2] * inv, acc[dblk][4 * q4 + 3] * inv);
        }
      }
    }
  }
  if (row_ok && a.lse && h == 0) a.lse[lse_off + (int64_t)hq * a.lse_sh + pos] = lse2 * kLn2;
}

// workgroups of a launch: every XCD's list padded to whole dispatch groups
int64_t grid_size(const PrefillArgs& a, int nz) {
  const int64_t n_units = (int64_t)a.hkv * nz;
  const int64_t units_x = (n_units + kXcds - 1) / kXcds;   // units per XCD
  const int64_t G = group_units(a.n_qtiles);
  return kXcds * ((units_x + G - 1) / G) * G * a.n_qtiles;
}

// CUs per XCD of the current device (queried once per device; 32 on MI355X)
int cus_per_xcd() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 32;
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < kXcds) n = 256;
    cache[dev] = n / kXcds;
  }
  return cache[dev];
}

template <int D, int DV, bool FP8, int MODE, int MK, bool SOFTCAP, int BIAS, bool VT>
hipError_t launch_t(const PrefillArgs& a, int nz, hipStream_t stream) {
  PrefillArgs b = a;
  b.nz = nz;
  const int64_t grid = grid_size(a, nz);
  b.items_x = (int)(grid / kXcds);
  b.cu_per_xcd = cus_per_xcd();
  hipLaunchKernelGGL((prefill_kernel<D, DV, FP8, MODE, MK, SOFTCAP, BIAS, VT>), dim3((unsigned)grid), dim3(kThreads), 0,
                     stream, b);
  return hipGetLastError();
}

template <int D, int DV, bool FP8, int MODE, int MK, int BIAS, bool VT>
hipError_t launch_s(const PrefillArgs& a, int nz, bool softcap, hipStream_t s) {
  return softcap ? launch_t<D, DV, FP8, MODE, MK, true, BIAS, VT>(a, nz, s)
                 : launch_t<D, DV, FP8, MODE, MK, false, BIAS, VT>(a, nz, s);
}

template <int D, int DV, bool FP8, int MODE, int BIAS, bool VT>
hipError_t launch_b(const PrefillArgs& a, int nz, bool mask, bool softcap, hipStream_t s) {
  if (!mask) return launch_s<D, DV, FP8, MODE, kMaskNone, BIAS, VT>(a, nz, softcap, s);
  if (a.wl >= 0) return launch_s<D, DV, FP8, MODE, kMaskWindow, BIAS, VT>(a, nz, softcap, s);
  return launch_s<D, DV, FP8, MODE, kMaskRight, BIAS, VT>(a, nz, softcap, s);
}

template <int D, int DV, bool FP8, int MODE, bool VT>
hipError_t launch_v(const PrefillArgs& a, int nz, bool mask, bool softcap, hipStream_t s) {
  if (a.bias_type == kBiasAlibi) return launch_b<D, DV, FP8, MODE, kBiasAlibi, VT>(a, nz, mask, softcap, s);
  if (a.bias_type == kBiasElem) return launch_b<D, DV, FP8, MODE, kBiasElem, VT>(a, nz, mask, softcap, s);
  return launch_b<D, DV, FP8, MODE, kBiasNone, VT>(a, nz, mask, softcap, s);
}

template <int D, int DV, bool FP8, int MODE>
hipError_t launch_m(const PrefillArgs& a, int nz, bool mask, bool softcap, hipStream_t s) {
  if constexpr ((MODE == kPrefillBatch || MODE == kPrefillPaged || MODE == kPrefillVarlen) && D == DV) {
    if (a.v_colmajor) return launch_v<D, DV, FP8, MODE, true>(a, nz, mask, softcap, s);
  } else {
    if (a.v_colmajor) return hipErrorInvalidValue;  // batch, varlen or paged mode with equal head dims only
  }
  return launch_v<D, DV, FP8, MODE, false>(a, nz, mask, softcap, s);
}

template <int D, int DV, bool FP8>
hipError_t launch_f(const PrefillArgs& a, int mode, int nz, bool mask, bool softcap, hipStream_t s) {
  if (mode == kPrefillVarlen) return launch_m<D, DV, FP8, kPrefillVarlen>(a, nz, mask, softcap, s);
  if (mode == kPrefillPaged) return launch_m<D, DV, FP8, kPrefillPaged>(a, nz, mask, softcap, s);
  if (mode == kPrefillVarlenPaged) return launch_m<D, DV, FP8, kPrefillVarlenPaged>(a, nz, mask, softcap, s);
  return launch_m<D, DV, FP8, kPrefillBatch>(a, nz, mask, softcap, s);
}


// One (input type, d, head_dim_v) combination per part. The build compiles
// this file once per part (ATTN_PREFILL_PART = 0..7: bit 2 fp8, bit 1 d = 64,
// bit 0 head_dim_v = 64) so the instantiations compile in parallel; without
// the macro one object holds all.
template <int D, int DV, bool FP8>
hipError_t launch_part(const PrefillArgs& a, int mode, int nz, hipStream_t s) {
  const bool mask = a.wl >= 0 || a.wr >= 0;
  const bool softcap = a.softcap_pre != 0.0f;
  return launch_f<D, DV, FP8>(a, mode, nz, mask, softcap, s);
}

}  // namespace

#if !defined(ATTN_PREFILL_PART)
#define ATTN_PREFILL_ALL 1
#define ATTN_PREFILL_PART -1
#endif

#define ATTN_PREFILL_PART_FN(K, NAME, D, DV, FP8)                                      \
  hipError_t NAME(const PrefillArgs& a, int mode, int nz, hipStream_t s);                \
  hipError_t NAME(const PrefillArgs& a, int mode, int nz, hipStream_t s) {               \
    return launch_part<D, DV, FP8>(a, mode, nz, s);                                      \
  }

#if defined(ATTN_PREFILL_ALL) || ATTN_PREFILL_PART == 0
ATTN_PREFILL_PART_FN(0, launch_prefill_bf16_d128_dv128, 128, 128, false)
#endif
#if defined(ATTN_PREFILL_ALL) || ATTN_PREFILL_PART == 1
ATTN_PREFILL_PART_FN(1, launch_prefill_bf16_d128_dv64, 128, 64, false)
#endif
#if defined(ATTN_PREFILL_ALL) || ATTN_PREFILL_PART == 2
ATTN_PREFILL_PART_FN(2, launch_prefill_bf16_d64_dv128, 64, 128, false)
#endif
#if defined(ATTN_PREFILL_ALL) || ATTN_PREFILL_PART == 3
ATTN_PREFILL_PART_FN(3, launch_prefill_bf16_d64_dv64, 64, 64, false)
#endif
#if defined(ATTN_PREFILL_ALL) || ATTN_PREFILL_PART == 4
ATTN_PREFILL_PART_FN(4, launch_prefill_fp8_d128_dv128, 128, 128, true)
#endif
#if defined(ATTN_PREFILL_ALL) || ATTN_PREFILL_PART == 5
ATTN_PREFILL_PART_FN(5, launch_prefill_fp8_d128_dv64, 128, 64, true)
#endif
#if defined(ATTN_PREFILL_ALL) || ATTN_PREFILL_PART == 6
ATTN_PREFILL_PART_FN(6, launch_prefill_fp8_d64_dv128, 64, 128, true)
#endif
#if defined(ATTN_PREFILL_ALL) || ATTN_PREFILL_PART == 7
ATTN_PREFILL_PART_FN(7, launch_prefill_fp8_d64_dv64, 64, 64, true)
#endif

#if defined(ATTN_PREFILL_ALL) || ATTN_PREFILL_PART == 0
hipError_t launch_prefill_bf16_d128_dv64(const PrefillArgs& a, int mode, int nz, hipStream_t s);
hipError_t launch_prefill_bf16_d64_dv128(const PrefillArgs& a, int mode, int nz, hipStream_t s);
hipError_t launch_prefill_bf16_d64_dv64(const PrefillArgs& a, int mode, int nz, hipStream_t s);
hipError_t launch_prefill_fp8_d128_dv128(const PrefillArgs& a, int mode, int nz, hipStream_t s);
hipError_t launch_prefill_fp8_d128_dv64(const PrefillArgs& a, int mode, int nz, hipStream_t s);
hipError_t launch_prefill_fp8_d64_dv128(const PrefillArgs& a, int mode, int nz, hipStream_t s);
hipError_t launch_prefill_fp8_d64_dv64(const PrefillArgs& a, int mode, int nz, hipStream_t s);

int prefill_rows_per_tile(int) { return kBlockM; }

int64_t prefill_workgroups(const PrefillArgs& a, int nz) {
  return (a.n_qtiles <= 0 || nz <= 0 || a.hkv <= 0) ? 0 : grid_size(a, nz);
}

hipError_t launch_prefill(const PrefillArgs& a, int d, int dv, int in_type, int mode, int nz, hipStream_t stream) {
  if (a.n_qtiles <= 0 || nz <= 0 || a.hkv <= 0) return hipSuccess;
  typedef hipError_t (*Fn)(const PrefillArgs&, int, int, hipStream_t);
  static const Fn fns[8] = {launch_prefill_bf16_d128_dv128, launch_prefill_bf16_d128_dv64,
                            launch_prefill_bf16_d64_dv128,  launch_prefill_bf16_d64_dv64,
                            launch_prefill_fp8_d128_dv128,  launch_prefill_fp8_d128_dv64,
                            launch_prefill_fp8_d64_dv128,   launch_prefill_fp8_d64_dv64};
  const int part = (in_type == kInFP8 ? 4 : 0) | (d == 64 ? 2 : 0) | (dv == 64 ? 1 : 0);
  return fns[part](a, mode, nz, stream);
}
#endif

}  // namespace attn
