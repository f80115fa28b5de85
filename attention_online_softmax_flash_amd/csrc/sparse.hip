// Shared-KV sparse attention (KvQuantSparseAttnSharedkv; sparse_flash_mla SWA,
// CSA and HCA modes): O = softmax(Q K~^T * scale) V~ with K~ = V~ = the window
// rows of the original KV followed by the selected rows of the compressed KV,
// plus an optional per-head sink logit.
//
// Row list of query token t of batch b (the S1 tokens of the entry are the
// last S1 positions of its KV sequence: p = Lk - S1 + t; with the TND layout
// S1 is the entry's own count cu_seqlens_q[b + 1] - cu_seqlens_q[b]), as
// fixed slots so a result never depends on the other batch entries:
//   slots [0, n_win_slots): window row j = p - win_left + s, used when
//     0 <= j <= min(Lk - 1, p + win_right) (band);
//   slots [n_win_slots, n_win_slots + K2): compressed row c = idx[b][t][s - n_win]
//     (compressed-sparse) or c = s - n_win (heavily compressed: the whole
//     compressed sequence, no indices), used when 0 <= c < Lc - (S1 - 1 - t),
//     Lc = floor(Lk / cmp_ratio) (right-down causal over the compressed rows).
// Row formats: packed 640-byte rows (bf16 rope x64 | e4m3fn nope x448 | fp32
// scale x7, one per 64-wide nope tile; the logical 512-vector is
// [rope | nope * scale]), or plain bf16 / fp16 rows of 512 values.
//
// Work split.  A workgroup of 8 waves takes one query row, a block of HB
// heads (32, or 64 when the launch would not fit the CUs otherwise) and one
// chunk of its slots (sub_per_chunk sub-chunks of 64 slots), so every
// gathered row is converted once for the heads of the block (the workgroups
// of the other head blocks of the row run on the same XCD and find the rows
// in its L2).  It
//   1. loads its query rows into registers and caches the batch entry's block
//      table rows and its index entries in LDS (all in flight together);
//   2. resolves a sub-chunk's 64 slots to row addresses from those LDS copies
//      (the row loads are then the only dependent trip to memory);
//   3. loads the rows (the next sub-chunk's loads are in flight while the
//      current one is computed), converts them to bf16 / fp16 in LDS
//      row-major, runs S^T = X Q^T and O^T = X^T P^T on 32x32x16 MFMA (the
//      value product reads its transposed operand with LDS transpose reads)
//      with an online softmax across the sub-chunks;
//   4. writes the final output (and LSE) when the row has one chunk, else a
//      normalised fp32 partial with its log2-sum-exp, which the merge kernel
//      folds in chunk order together with the sink.
#include "fia_device.h"

namespace fia {

namespace {

constexpr int kThreads = 512;
// Bytes per row-major row in LDS: consecutive rows start 32 bytes (8 banks)
// apart, so the 4 rows x 32 bytes one 16-lane group of transposed value
// reads touches fall in distinct banks.
constexpr int X_PITCH = kSparseD * 2 + 32;
constexpr int X_BYTES = kSparseSub * X_PITCH;        // 67584
constexpr int RP_BYTES = 2 * kSparseSub * 8;         // row addresses, two sub-chunks
constexpr int BT_BYTES = 2 * kSparseBtCache * 4;     // ori / cmp block-table rows
constexpr int IX_BYTES = kSparseMaxSub * kSparseSub * 4;
constexpr int ST_BYTES = 4 * 64 * 4;                 // row max / sum per (slot half, head)
constexpr int LM_BYTES = 2 * 8;                      // live-slot masks, two sub-chunks
// LDS layout of a workgroup of HB heads (32 or 64).  HQ 32-head halves; the
// score product is split over DS d ranges, whose partial sums meet through
// the exchange area SX.
template <int HB>
struct SparseLds {
  static constexpr int HQ = HB / 32;
  static constexpr int DS = 4 / HQ;
  static constexpr int Q_BYTES = HB * X_PITCH;                        // query rows, row-major
  static constexpr int SX_BYTES = (DS - 1) * 2 * HQ * 64 * 16 * 4;    // score partials
  static constexpr int OFF_Q = X_BYTES;
  static constexpr int OFF_SX = OFF_Q + Q_BYTES;
  // The probabilities [head half][k step][lane] (HQ x 4 KB) share the score
  // exchange area: they are written after its last read in a step.
  static constexpr int OFF_P = OFF_SX;
  static constexpr int OFF_RP = OFF_SX + SX_BYTES;
  static constexpr int OFF_BT = OFF_RP + RP_BYTES;
  static constexpr int OFF_IX = OFF_BT + BT_BYTES;
  static constexpr int OFF_ST = OFF_IX + IX_BYTES;
  static constexpr int OFF_LM = OFF_ST + ST_BYTES;
  static constexpr int TOTAL = OFF_LM + LM_BYTES;
  static_assert(HQ * 4 * 64 * 16 <= SX_BYTES, "probabilities fit the exchange area");
};

}  // namespace

// Four OCP e4m3fn codes (one dword) -> floats, by the hardware conversion
// (v_cvt_pk_f32_fp8; exact: subnormals m * 2^-9, 0x7f / 0xff are NaN).
__device__ __forceinline__ void e4m3fn_x4(uint32_t w, float* f) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = lo[0];
  f[1] = lo[1];
  f[2] = hi[0];
  f[3] = hi[1];
}

// Loads through a row address that was kept in LDS: the address is known to
// be global memory, so the load is a global (not a generic / flat) load, which
// would otherwise also hold up every later wait for LDS traffic.
typedef const __attribute__((address_space(1))) u32x4* gptr_u32x4;
typedef const __attribute__((address_space(1))) float* gptr_f32;
__device__ __forceinline__ u32x4 ld16_global(const uint8_t* p) {
  return *(gptr_u32x4)(p);
}
__device__ __forceinline__ float ldf_global(const uint8_t* p) {
  return *(gptr_f32)(p);
}

// 32x32x16 MFMA on bf16 or fp16 operands (the 16-bit type of the rows).
template <bool F16>
__device__ __forceinline__ f32x16 mfma32h(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (F16) {
    typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return mfma32(a, b, c);
  }
}

// Two floats -> one packed pair of the 16-bit type (round to nearest even).
template <bool F16>
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  if constexpr (F16) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  } else {
    return pack_bf16x2(lo, hi);
  }
}

// Batch entry, token position and query count of row r.  BSND: b = r / S1.
// TND: the entry b with cu_q[b] <= r < cu_q[b + 1], by binary search over the
// cumulative counts (values as read; a row outside every entry, possible
// only with inconsistent counts, is dead: no key rows, output 0).  tq is the
// token index the query, output and index rows are addressed with (their
// batch strides are 0 with TND).
struct SparseRow {
  int b, t, s1, tq;
  bool live;
};
__device__ __forceinline__ SparseRow sparse_row(const SparseArgs& a, int r) {
  SparseRow w;
  if (a.cu_q == nullptr) {
    w.b = r / a.S1;
    w.t = r - w.b * a.S1;
    w.s1 = a.S1;
    w.tq = w.t;
    w.live = true;
    return w;
  }
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu_q[mid] <= r) {
      lo = mid;
    } else {
      hi = mid - 1;
    }
  }
  const int c0 = a.cu_q[lo], c1 = a.cu_q[lo + 1];
  w.b = lo;
  w.tq = r;
  w.live = c0 <= r && r < c1;
  w.t = w.live ? r - c0 : 0;
  w.s1 = w.live ? c1 - c0 : 1;
  return w;
}

// Same, for a row index r that is uniform over the calling wave (every
// lane active): with B + 1 <= 64 the wave loads the cumulative counts in one
// vector load (lane i: cu_q[i]) and counts the entries that start at or
// before r, instead of a chain of dependent loads.
__device__ __forceinline__ SparseRow sparse_row_wave(const SparseArgs& a, int r, int lane) {
  if (a.cu_q == nullptr || a.B + 1 > 64) return sparse_row(a, r);
  const int v = a.cu_q[min(lane, a.B)];
  const int lo = __popcll(__ballot(lane >= 1 && lane < a.B && v <= r));
  const int c0 = __builtin_amdgcn_readlane(v, lo), c1 = __builtin_amdgcn_readlane(v, lo + 1);
  SparseRow w;
  w.b = lo;
  w.tq = r;
  w.live = c0 <= r && r < c1;
  w.t = w.live ? r - c0 : 0;
  w.s1 = w.live ? c1 - c0 : 1;
  return w;
}

// KV length of the row's entry, clamped to what its pool can address.
__device__ __forceinline__ int sparse_len(const SparseArgs& a, const SparseRow& w) {
  if (!w.live) return 0;
  const int Lk = a.seqused[w.b];
  const int64_t cap = a.ori.paged ? (int64_t)a.ori.bt_cols * a.ori.bs : a.ori.n_rows;
  return Lk < 0 ? 0 : (int)((int64_t)Lk > cap ? cap : Lk);
}

// Row rr of pool `pd` for batch entry b.  `bt(col)` returns the raw block id
// of block-table column col of the entry (col < bt_cols); `off` is the
// entry's first row in a packed (TND) pool.
template <class BT>
__device__ __forceinline__ const uint8_t* pool_row(const SparsePool& pd, int b, int rr, int64_t off,
                                                   BT bt) {
  if (pd.paged) {
    const int page = rr / pd.bs;
    const int slot = rr - page * pd.bs;
    const int blk = clamp_block(bt(min(page, pd.bt_cols - 1)), pd.nb);
    return pd.base + (int64_t)blk * pd.sb + (int64_t)slot * pd.ss;
  }
  int64_t row = off + rr;
  row = row < 0 ? 0 : (row >= pd.n_rows ? pd.n_rows - 1 : row);
  return pd.base + (int64_t)b * pd.sb + row * pd.ss;
}

// What a query row needs to resolve its slots.
struct SlotCtx {
  int b, p, jmax, n_cmp;
  int64_t ori_off, cmp_off;   // first row of the entry in packed (TND) pools
  bool live;
};
__device__ __forceinline__ SlotCtx slot_ctx(const SparseArgs& a, const SparseRow& w, int Lk) {
  SlotCtx c;
  c.b = w.b;
  c.live = w.live;
  c.p = Lk - w.s1 + w.t;
  c.jmax = min(Lk - 1, c.p + a.win_right);
  c.n_cmp = Lk / a.cmp_ratio - (w.s1 - 1 - w.t);
  c.ori_off = a.ori.cu ? a.ori.cu[w.b] : 0;
  c.cmp_off = (a.has_cmp && a.cmp.cu) ? a.cmp.cu[w.b] : 0;
  return c;
}

// Slot s of a query row -> packed row address (nullptr for an unused slot)
// and id: j for window row j, (1 << 30) | c for compressed row c, -1 if
// unused.  `ori_bt` / `cmp_bt` read block-table columns of the entry and
// `idx(k)` index entry k of the row (the kernel reads them from its LDS
// copies, the test export from global memory).
template <class OBT, class CBT, class IDX>
__device__ __forceinline__ const uint8_t* slot_row(const SparseArgs& a, const SlotCtx& c, int s,
                                                   OBT ori_bt, CBT cmp_bt, IDX idx, int32_t* id) {
  *id = -1;
  if (!c.live || s < 0 || s >= a.n_slots) return nullptr;
  if (s < a.n_win_slots) {
    const int j = c.p - a.win_left + s;
    if (s > a.win_left + a.win_right || j < 0 || j > c.jmax) return nullptr;
    *id = j;
    return pool_row(a.ori, c.b, j, c.ori_off, ori_bt);
  }
  const int k = s - a.n_win_slots;
  if (!a.has_cmp || k >= a.K2) return nullptr;
  const int cr = a.cmp_direct ? k : idx(k);
  if (cr < 0 || cr >= c.n_cmp) return nullptr;
  *id = (1 << 30) | cr;
  return pool_row(a.cmp, c.b, cr, c.cmp_off, cmp_bt);
}

// Grid: n_rows * n_hb * n_chunks workgroups of 512 threads (8 waves).
template <int FMT, int HB>
__global__ __launch_bounds__(kThreads, 1) void sparse_attn(SparseArgs a) {
  constexpr bool F16 = FMT == SF_FP16;
  using SL = SparseLds<HB>;
  constexpr int HQ = SL::HQ;
  constexpr int DS = SL::DS;
  constexpr int DSW = kSparseD / DS;       // d values per score split (128 or 256)
  constexpr int DVW = kSparseD * HQ / 8;   // d values per wave in the value product (64 or 128)
  constexpr int NOB = DVW / 32;            // its 32-wide d blocks
  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t* xs = lds;                                                   // [64][X_PITCH]
  u32x4* ps = reinterpret_cast<u32x4*>(lds + SL::OFF_P);                   // [HQ][4][64]
  float* sx = reinterpret_cast<float*>(lds + SL::OFF_SX);                  // [DS - 1][2][HQ][4][64][4]
  const uint8_t** rowp = reinterpret_cast<const uint8_t**>(lds + SL::OFF_RP);   // [2][64]
  int32_t* bt_o = reinterpret_cast<int32_t*>(lds + SL::OFF_BT);            // [kSparseBtCache]
  int32_t* bt_c = bt_o + kSparseBtCache;                               // [kSparseBtCache]
  int32_t* ixc = reinterpret_cast<int32_t*>(lds + SL::OFF_IX);             // [64 * sub_per_chunk]
  float* mx_s = reinterpret_cast<float*>(lds + SL::OFF_ST);                // [2][HB]
  float* l_s = mx_s + 128;                                             // [2][HB]
  uint64_t* live_m = reinterpret_cast<uint64_t*>(lds + SL::OFF_LM);       // [2]: bit s = slot s used

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int n = lane & 31;
  const int hh = lane >> 5;

  // Workgroup -> (row, head block, chunk).
  const int parts = a.n_hb * a.n_chunks;
  int r, part;
  {
    const int L = blockIdx.x;
    if (a.xcd_rows) {
      const int k = L >> 3;
      r = (L & 7) + 8 * (k / parts);
      part = k % parts;
    } else {
      r = L / parts;
      part = L - r * parts;
    }
  }
  const int hb = part / a.n_chunks;
  const int chunk = part - hb * a.n_chunks;
  const int sub_n = a.sub_per_chunk;
  const int s_begin = chunk * kSparseSub * sub_n;

  // Roles.  Scores: slot half sb, head half hq, d range ds (DSW values).
  // Values: head half hq, d block dv (DVW values).  Lane (n, hh) owns head
  // HB hb + 32 hq + n.
  const int sb = wave & 1;
  const int hq = HQ == 2 ? ((wave >> 1) & 1) : 0;
  const int ds = HQ == 2 ? (wave >> 2) : (wave >> 1);
  const int dv = HQ == 2 ? ((wave & 1) + 2 * (wave >> 2)) : wave;
  const int head = HB * hb + 32 * hq + n;
  const bool head_ok = head < a.N1;

  const SparseRow qr = sparse_row_wave(a, r, lane);
  const int b = qr.b;

  // 1. The workgroup's 64 query rows into LDS (row-major; heads past N1 are
  // zero), and LDS copies of the entry's block-table rows and of the chunk's
  // index entries.  Every load is issued before the first store: each is
  // unconditional (positions are clamped into range, absent tables lie
  // outside their empty buffer resources and read as zero), so they are in
  // flight together, one trip to memory.
  uint8_t* qs = lds + SL::OFF_Q;
  const uint16_t* qrow = a.q + (int64_t)b * a.q_sb + (int64_t)qr.tq * a.q_ss;
  constexpr int QV = HB * 64 / kThreads;   // 16-byte query pieces per thread
  u32x4 qv[QV];
#pragma unroll
  for (int v = 0; v < QV; ++v) {
    // 16-byte piece p % 64 of head p / 64; heads past N1 load the last head
    // (a valid address) and are zeroed.
    const int p = tid + kThreads * v;
    const int hd = HB * hb + (p >> 6);
    const u32x4 w = ld16(qrow + (int64_t)min(hd, a.N1 - 1) * a.q_sh + 8 * (p & 63));
    qv[v] = hd < a.N1 ? w : u32x4{0u, 0u, 0u, 0u};
  }
  const bool cache_o = a.ori.paged && a.ori.bt_cols <= kSparseBtCache;
  const bool cache_c = a.has_cmp && a.cmp.paged && a.cmp.bt_cols <= kSparseBtCache;
  // One entry per thread: the caches hold at most kThreads entries, the
  // index slice 64 * sub_per_chunk <= kThreads.
  static_assert(kSparseBtCache <= kThreads && kSparseSub * kSparseMaxSub <= kThreads, "one entry per thread");
  const int k_begin = s_begin - a.n_win_slots;   // index entry of the chunk's first slot
  const bool use_idx = a.has_cmp && !a.cmp_direct;
  const int k_own = k_begin + tid;
  const __amdgpu_buffer_rsrc_t r_bto =
      make_rsrc(cache_o ? a.ori.bt + (int64_t)b * a.ori.bt_sb : nullptr, cache_o ? (uint32_t)a.ori.bt_cols * 4u : 0u);
  const __amdgpu_buffer_rsrc_t r_btc =
      make_rsrc(cache_c ? a.cmp.bt + (int64_t)b * a.cmp.bt_sb : nullptr, cache_c ? (uint32_t)a.cmp.bt_cols * 4u : 0u);
  const __amdgpu_buffer_rsrc_t r_ix =
      make_rsrc(use_idx ? a.idx + (int64_t)b * a.idx_sb + (int64_t)qr.tq * a.idx_ss : nullptr,
                use_idx ? (uint32_t)a.K2 * 4u : 0u);
  const int32_t bto = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(r_bto, (uint32_t)tid * 4u, 0, 0);
  const int32_t btc = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(r_btc, (uint32_t)tid * 4u, 0, 0);
  const int32_t ixv = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(r_ix, (uint32_t)max(k_own, 0) * 4u, 0, 0);
  const int Lk = sparse_len(a, qr);
  const SlotCtx ctx = slot_ctx(a, qr, Lk);
#pragma unroll
  for (int v = 0; v < QV; ++v) {
    const int p = tid + kThreads * v;
    *reinterpret_cast<u32x4*>(qs + (p >> 6) * X_PITCH + 16 * (p & 63)) = qv[v];
  }
  if (cache_o && tid < a.ori.bt_cols) bt_o[tid] = bto;
  if (cache_c && tid < a.cmp.bt_cols) bt_c[tid] = btc;
  if (use_idx && tid < kSparseSub * sub_n) ixc[tid] = (k_own >= 0 && k_own < a.K2) ? ixv : -1;
  __syncthreads();

  auto ori_bt = [&](int col) FIA_INLINE {
    return cache_o ? bt_o[col] : a.ori.bt[(int64_t)b * a.ori.bt_sb + col];
  };
  auto cmp_bt = [&](int col) FIA_INLINE {
    return cache_c ? bt_c[col] : a.cmp.bt[(int64_t)b * a.cmp.bt_sb + col];
  };
  auto idx_at = [&](int k) FIA_INLINE { return ixc[k - k_begin]; };
  // Row addresses of sub-chunk u and the mask of its used slots into buffer
  // u & 1 (wave 0: one slot per lane).
  auto resolve = [&](int u) FIA_INLINE {
    if (wave == 0) {
      int32_t id;
      const uint8_t* src = slot_row(a, ctx, s_begin + kSparseSub * u + lane, ori_bt, cmp_bt, idx_at, &id);
      rowp[(u & 1) * kSparseSub + lane] = src;
      const uint64_t m = __ballot(src != nullptr);
      if (lane == 0) live_m[u & 1] = m;
    }
  };

  // Row pieces of one sub-chunk in registers.  Packed rows: piece p = tid +
  // 512 v (p < 64 * 36) is 16 bytes of row p / 36: pieces 0..7 rope, 8..35
  // 16 nope codes each (with their tile scale).  16-bit rows: piece p = tid +
  // 512 v is 16 bytes (8 values) of row p / 64.
  constexpr int NP = FMT == SF_FP8_PACKED ? 5 : 8;
  constexpr int PPR = FMT == SF_FP8_PACKED ? 36 : 64;   // pieces per row
  u32x4 raw[NP];
  float scl[NP];
  auto load_rows = [&](int u) FIA_INLINE {
    const uint8_t* const* rp = rowp + (u & 1) * kSparseSub;
#pragma unroll
    for (int v = 0; v < NP; ++v) {
      const int p = tid + kThreads * v;
      raw[v] = u32x4{0u, 0u, 0u, 0u};
      scl[v] = 0.f;
      if (p < kSparseSub * PPR) {
        const int row = p / PPR;
        const int pc = p - row * PPR;
        const uint8_t* src = rp[row];
        if (src != nullptr) {
          raw[v] = ld16_global(src + 16 * pc);
          if (FMT == SF_FP8_PACKED && pc >= 8) scl[v] = ldf_global(src + 576 + 4 * ((pc - 8) >> 2));
        }
      }
    }
  };
  auto store_rows = [&]() FIA_INLINE {
#pragma unroll
    for (int v = 0; v < NP; ++v) {
      const int p = tid + kThreads * v;
      if (p < kSparseSub * PPR) {
        const int row = p / PPR;
        const int pc = p - row * PPR;
        uint8_t* xr = xs + row * X_PITCH;
        if (FMT != SF_FP8_PACKED || pc < 8) {
          *reinterpret_cast<u32x4*>(xr + 16 * pc) = raw[v];
        } else {
          const float sc = scl[v];
          float f[16];
          e4m3fn_x4(raw[v].x, f);
          e4m3fn_x4(raw[v].y, f + 4);
          e4m3fn_x4(raw[v].z, f + 8);
          e4m3fn_x4(raw[v].w, f + 12);
          u32x4* dst = reinterpret_cast<u32x4*>(xr + 128 + 32 * (pc - 8));
          dst[0] = u32x4{pack_bf16x2(f[0] * sc, f[1] * sc), pack_bf16x2(f[2] * sc, f[3] * sc),
                         pack_bf16x2(f[4] * sc, f[5] * sc), pack_bf16x2(f[6] * sc, f[7] * sc)};
          dst[1] = u32x4{pack_bf16x2(f[8] * sc, f[9] * sc), pack_bf16x2(f[10] * sc, f[11] * sc),
                         pack_bf16x2(f[12] * sc, f[13] * sc), pack_bf16x2(f[14] * sc, f[15] * sc)};
        }
      }
    }
  };

  // Transposed value operand: in 16-lane group g, lane j addresses slot
  // 16 kk + 8 r + 4 (g / 2) + j / 4 at columns 16 (g % 2) + 4 (j % 4) .. + 3
  // of the 32-wide d block (the order of the score accumulators).
  const uint8_t* tb;
  {
    const int g16 = lane >> 4;
    const int j = lane & 15;
    tb = xs + (4 * (g16 >> 1) + (j >> 2)) * X_PITCH + (DVW * dv + 16 * (g16 & 1) + 4 * (j & 3)) * 2;
  }

  float m_run = kNegInf;   // running max (log2 domain) of this lane's head
  float l_run = 0.f;
  f32x16 o[NOB];
#pragma unroll
  for (int mb = 0; mb < NOB; ++mb) {
#pragma unroll
    for (int q = 0; q < 16; ++q) o[mb][q] = 0.f;
  }

  int n_sub = 0;
  while (n_sub < sub_n && s_begin + kSparseSub * n_sub < a.n_slots) ++n_sub;
  if (n_sub > 0) {
    resolve(0);
    __syncthreads();
    load_rows(0);
  }
  for (int u = 0; u < n_sub; ++u) {
    store_rows();
    const bool has_next = u + 1 < n_sub;
    if (has_next) resolve(u + 1);
    __syncthreads();
    if (has_next) load_rows(u + 1);
    const uint64_t live = live_m[u & 1];

    // 2. Scores S^T[slot][head] for slots 32 sb + (0..31), heads of hq, d
    // range ds; ranges 1 .. DS - 1 hand their partial sums to the range-0
    // wave through LDS.
    f32x16 s;
#pragma unroll
    for (int q = 0; q < 16; ++q) s[q] = 0.f;
#pragma unroll
    for (int c = 0; c < DSW / 16; ++c) {
      const int off = (DSW * ds + 16 * c + 8 * hh) * 2;
      const u32x4 av = *reinterpret_cast<const u32x4*>(xs + (32 * sb + n) * X_PITCH + off);
      const u32x4 bv = *reinterpret_cast<const u32x4*>(qs + (32 * hq + n) * X_PITCH + off);
      s = mfma32h<F16>(av, bv, s);
    }
    // Element q of the partial of d range k >= 1, this (sb, hq, lane): four
    // floats per lane and quarter, lanes adjacent (16-byte stores, no bank
    // conflicts).
    auto part = [&](int k, int q) FIA_INLINE -> float& {
      return sx[(((((k - 1) * 2 + sb) * HQ + hq) * 4 + (q >> 2)) * 64 + lane) * 4 + (q & 3)];
    };
    if (ds > 0) {
#pragma unroll
      for (int q = 0; q < 16; ++q) part(ds, q) = s[q];
    }
    __syncthreads();
    if (ds == 0) {
      float m_loc = kNegInf;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int slot = 32 * sb + 8 * (q >> 2) + 4 * hh + (q & 3);
        float sum;
        if constexpr (DS == 2) {
          sum = s[q] + part(1, q);
        } else {
          sum = (s[q] + part(1, q)) + (part(2, q) + part(3, q));
        }
        const float x = sum * a.scale_log2;
        s[q] = ((live >> slot) & 1u) ? x : kNegInf;
        m_loc = fmaxf(m_loc, s[q]);
      }
      m_loc = pair32_max(m_loc);
      if (hh == 0) mx_s[sb * HB + 32 * hq + n] = m_loc;
    }
    __syncthreads();
    const float m_new = fmaxf(m_run, fmaxf(mx_s[32 * hq + n], mx_s[HB + 32 * hq + n]));
    const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    m_run = m_new;
    if (ds == 0) {
      float l = 0.f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float pr[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          pr[t] = fast_exp2(s[8 * kk + t] - m_use);
          l += pr[t];
        }
        ps[(hq * 4 + 2 * sb + kk) * 64 + lane] =
            u32x4{pack_h2<F16>(pr[0], pr[1]), pack_h2<F16>(pr[2], pr[3]),
                  pack_h2<F16>(pr[4], pr[5]), pack_h2<F16>(pr[6], pr[7])};
      }
      l = pair32_sum(l);
      if (hh == 0) l_s[sb * HB + 32 * hq + n] = l;
    }
    __syncthreads();
    l_run = l_run * alpha + l_s[32 * hq + n] + l_s[HB + 32 * hq + n];

    // 3. O^T[d][head] += X^T P^T for d in [DVW dv, DVW dv + DVW).
#pragma unroll
    for (int mb = 0; mb < NOB; ++mb) {
      o[mb] *= alpha;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint8_t* vp = tb + 16 * kk * X_PITCH + 64 * mb;
        const u32x2 lo2 = lds_tr16(vp);
        const u32x2 hi2 = lds_tr16(vp + 8 * X_PITCH);
        o[mb] = mfma32h<F16>(u32x4{lo2.x, lo2.y, hi2.x, hi2.y}, ps[(hq * 4 + kk) * 64 + lane], o[mb]);
      }
    }
    __syncthreads();   // every wave is done with xs, ps and the statistics
  }

  // 4. Lane (n, hh) holds O^T[d][head] at d = DVW dv + 32 mb + 8 (q / 4) +
  // 4 hh + q % 4.
  if (!head_ok) return;
  if (a.n_chunks == 1) {
    float m = m_run, L = l_run, osc = 1.f;
    bool has = L > 0.f;
    if (a.sinks != nullptr && qr.live) {
      // The sink: one more softmax term with a zero value vector.
      const float z = a.sinks[head] * kLog2e;
      const float mf = fmaxf(m, z);
      osc = (m == kNegInf) ? 0.f : fast_exp2(m - mf);
      L = L * osc + fast_exp2(z - mf);
      m = mf;
      has = true;
    }
    const float inv = has ? osc / L : 0.f;
    uint16_t* op = a.o + (int64_t)b * a.o_sb + (int64_t)qr.tq * a.o_ss + (int64_t)head * a.o_sh +
                   DVW * dv + 4 * hh;
#pragma unroll
    for (int mb = 0; mb < NOB; ++mb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        st8(op + 32 * mb + 8 * q4,
            u32x2{pack_h2<F16>(o[mb][4 * q4] * inv, o[mb][4 * q4 + 1] * inv),
                  pack_h2<F16>(o[mb][4 * q4 + 2] * inv, o[mb][4 * q4 + 3] * inv)});
      }
    }
    if (a.lse != nullptr && dv == 0 && hh == 0) {
      a.lse[(int64_t)b * a.lse_sb + (int64_t)qr.tq * a.lse_ss + (int64_t)head * a.lse_sh] =
          has ? (m + fast_log2(L)) * kLn2 : kPosInf;
    }
    return;
  }
  // Partial of chunk `chunk`: part_o[row][chunk][d / 4][head][d % 4] (four
  // consecutive d values of a head per 16-byte store, heads adjacent, so a
  // store writes whole runs of 32 heads), part_lse[row][chunk][head].
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  const int64_t rc = (int64_t)r * a.n_chunks + chunk;
  f32x4* pp = reinterpret_cast<f32x4*>(a.part_o) + (rc * (kSparseD / 4) + (DVW * dv) / 4 + hh) * a.N1 + head;
#pragma unroll
  for (int mb = 0; mb < NOB; ++mb) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      pp[(int64_t)(8 * mb + 2 * q4) * a.N1] = f32x4{o[mb][4 * q4] * inv, o[mb][4 * q4 + 1] * inv,
                                                    o[mb][4 * q4 + 2] * inv, o[mb][4 * q4 + 3] * inv};
    }
  }
  if (dv == 0 && hh == 0) a.part_lse[rc * a.N1 + head] = l_run > 0.f ? m_run + fast_log2(l_run) : kNegInf;
}

// Fold the chunk partials of one query row in chunk order with the sink
// logit.  Workgroup (row, 16-wide d block, 64-head block): the 64 threads of
// each wave take consecutive heads (coalesced partial reads), the 4 waves 4 d
// values each.  Chunks are folded in groups of G: every log-sum-exp and
// partial of a group is requested before the first is used (addresses
// clamped to the last chunk, so the loads are unconditional), and the group
// is folded into the running sum with the usual rescale by the new maximum;
// the sink's term joins at the end.
constexpr int kMergeD = 4;   // d values per thread (one 16-byte partial load)
constexpr int kMergeHeads = 64;   // heads per merge workgroup (one per lane)
template <bool F16>
__global__ __launch_bounds__(256) void sparse_merge(SparseArgs a) {
  constexpr int G = 8;   // chunks per group of loads in flight
  const int tid = threadIdx.x;
  const int hl = tid & 63;
  const int r = blockIdx.x;
  const int d0 = 4 * kMergeD * blockIdx.y + kMergeD * (tid >> 6);
  const int h = kMergeHeads * blockIdx.z + hl;
  const SparseRow qr = sparse_row_wave(a, r, hl);   // every lane still active
  if (h >= a.N1) return;
  const int nc = a.n_chunks;
  const int64_t rc0 = (int64_t)r * nc;
  const f32x4* base = reinterpret_cast<const f32x4*>(a.part_o) + (rc0 * (kSparseD / 4) + d0 / 4) * a.N1 + h;
  const float* lp = a.part_lse + rc0 * a.N1 + h;
  const int64_t cstride = (int64_t)(kSparseD / 4) * a.N1;   // in 4-float units
  // The sink logit (a buffer load, zero without sinks: no branch, so the
  // load stays in flight through the fold that follows).
  const bool sink_on = a.sinks != nullptr && qr.live;
  const __amdgpu_buffer_rsrc_t r_sink = make_rsrc(a.sinks, a.sinks != nullptr ? (uint32_t)a.N1 * 4u : 0u);
  const float z = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_sink, (uint32_t)h * 4u, 0, 0)) * kLog2e;
  // Running maximum M and sum L of 2^(lse_c - M) over the chunks so far.
  float M = kNegInf;
  float L = 0.f;
  float acc[kMergeD];
#pragma unroll
  for (int u = 0; u < kMergeD; ++u) acc[u] = 0.f;
  for (int c0 = 0; c0 < nc; c0 += G) {
    float lv[G];
    float x[G][kMergeD];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int64_t c = min(c0 + i, nc - 1);
      lv[i] = lp[c * a.N1];
      const f32x4 v4 = base[c * cstride];
#pragma unroll
      for (int u = 0; u < kMergeD; ++u) x[i][u] = v4[u];
    }
    // Branch-free from here (a branch would let the compiler sink the
    // partial loads past the wait for the log-sum-exps).
    float gm = M;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (c0 + i >= nc) lv[i] = kNegInf;
      gm = fmaxf(gm, lv[i]);
    }
    const float gmu = (gm == kNegInf) ? 0.f : gm;
    const float sc = (M == kNegInf) ? 0.f : fast_exp2(M - gmu);
    L *= sc;
#pragma unroll
    for (int u = 0; u < kMergeD; ++u) acc[u] *= sc;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float wc = (lv[i] == kNegInf) ? 0.f : fast_exp2(lv[i] - gmu);
      L += wc;
#pragma unroll
      for (int u = 0; u < kMergeD; ++u) acc[u] = __builtin_fmaf(wc, x[i][u], acc[u]);
    }
    M = gm;
  }
  if (sink_on) {
    const float mf = fmaxf(M, z);
    const float sc = (M == kNegInf) ? 0.f : fast_exp2(M - mf);
    L = L * sc + fast_exp2(z - mf);
#pragma unroll
    for (int u = 0; u < kMergeD; ++u) acc[u] *= sc;
    M = mf;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* op = a.o + (int64_t)qr.b * a.o_sb + (int64_t)qr.tq * a.o_ss + (int64_t)h * a.o_sh + d0;
  st8(op, u32x2{pack_h2<F16>(acc[0] * inv, acc[1] * inv), pack_h2<F16>(acc[2] * inv, acc[3] * inv)});
  if (a.lse != nullptr && blockIdx.y == 0 && tid < 64) {
    a.lse[(int64_t)qr.b * a.lse_sb + (int64_t)qr.tq * a.lse_ss + (int64_t)h * a.lse_sh] =
        L > 0.f ? (M + fast_log2(L)) * kLn2 : kPosInf;
  }
}

template <int FMT, int HB>
static hipError_t launch_hb(const SparseArgs& a, hipStream_t s) {
  // Dynamic LDS above the default limit must be enabled for the kernel (on
  // the current device); the call is cheap, so it is made on every launch.
  constexpr int lds = SparseLds<HB>::TOTAL;
  const hipError_t attr = hipFuncSetAttribute(
      (const void*)sparse_attn<FMT, HB>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const unsigned grid = (unsigned)a.n_rows * a.n_hb * a.n_chunks;
  sparse_attn<FMT, HB><<<grid, kThreads, lds, s>>>(a);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_fmt(const SparseArgs& a, hipStream_t s) {
  if (a.hb_heads == 32) return launch_hb<FMT, 32>(a, s);
  if (a.hb_heads == 64) return launch_hb<FMT, 64>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_sparse(const SparseArgs& a, hipStream_t s) {
  if (a.n_rows == 0) return hipSuccess;
  switch (a.fmt) {
    case SF_FP8_PACKED: return launch_fmt<SF_FP8_PACKED>(a, s);
    case SF_BF16: return launch_fmt<SF_BF16>(a, s);
    case SF_FP16: return launch_fmt<SF_FP16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_sparse_merge(const SparseArgs& a, hipStream_t s) {
  if (a.n_rows == 0 || a.n_chunks <= 1) return hipSuccess;
  const dim3 grid(a.n_rows, kSparseD / (4 * kMergeD), (a.N1 + kMergeHeads - 1) / kMergeHeads);
  if (a.fmt == SF_FP16) {
    sparse_merge<true><<<grid, 256, 0, s>>>(a);
  } else {
    sparse_merge<false><<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

// Test support: slot ids and raw row bytes, through slot_row with the block
// tables and index rows read from global memory.
__global__ __launch_bounds__(256) void debug_sparse_rows(SparseArgs a, int32_t* ids, uint8_t* rows,
                                                         int row_bytes) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.n_rows * a.n_slots;
  if (t >= total) return;
  const int r = (int)(t / a.n_slots);   // query row
  const int s = (int)(t % a.n_slots);
  const SparseRow qr = sparse_row(a, r);
  const SlotCtx ctx = slot_ctx(a, qr, sparse_len(a, qr));
  const int b = qr.b;
  auto ori_bt = [&](int col) { return a.ori.bt[(int64_t)b * a.ori.bt_sb + col]; };
  auto cmp_bt = [&](int col) { return a.cmp.bt[(int64_t)b * a.cmp.bt_sb + col]; };
  auto idx_at = [&](int k) { return a.idx[(int64_t)b * a.idx_sb + (int64_t)qr.tq * a.idx_ss + k]; };
  int32_t id;
  const uint8_t* row = slot_row(a, ctx, s, ori_bt, cmp_bt, idx_at, &id);
  ids[t] = id;
  uint32_t* dst = reinterpret_cast<uint32_t*>(rows + t * row_bytes);
  for (int w = 0; w < row_bytes / 4; ++w) {
    dst[w] = row ? reinterpret_cast<const uint32_t*>(row)[w] : 0u;
  }
}

hipError_t launch_debug_sparse_rows(const SparseArgs& a, int32_t* ids, uint8_t* rows,
                                    hipStream_t s) {
  const int64_t total = (int64_t)a.n_rows * a.n_slots;
  const int row_bytes = a.fmt == SF_FP8_PACKED ? kRowBytes : 2 * kSparseD;
  if (total > 0) {
    debug_sparse_rows<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(a, ids, rows, row_bytes);
  }
  return hipGetLastError();
}

}  // namespace fia
