// Prompt (prefill) branch: flash attention with an online softmax.
//
// One workgroup (4 waves) computes a 128-row query tile of one (batch, query
// head); each wave owns 32 query rows.  Key / value tiles of 64 rows are
// staged through LDS, double-buffered: the global loads of tile t+1 are in
// flight while tile t is consumed.  Both products run on the gfx950
// 32x32x16 bf16 MFMA with fp32 accumulation:
//
//   S^T[key][query] = K Q^T   (A = key rows from LDS, B = the wave's query
//                              rows held in registers for the whole loop)
//   O^T[d][query]  += V^T P^T (A = V^T from LDS, B = P taken straight from
//                              the S^T accumulators)
//
// With queries on the MFMA column axis, lane l owns query row l%32 of its
// wave: its running max and sum live in that lane plus its partner l^32, so a
// row reduction is one cross-lane step.  The key order inside each 16-key
// k-step follows the accumulator layout of S^T; V^T is read from the
// row-major value tile in LDS in the same order by transposing 8-byte LDS
// reads, so P needs no shuffling.
//
// Masks (aclnnFusedInferAttentionScoreV5 Attention Mask group): per query row
// i the visible keys are [lo(i), hi(i)); tiles wholly inside every row's range
// of a wave skip the per-element test, tiles outside are skipped.  ALiBi
// (pse type 2) adds slope * ((kv_start + j) - (q_start + i)) after scaling
// (aclnnFusedInferAttentionScoreV4 formula); it enters the score product as
// the accumulators' initial value.  Rows with no visible key and
// rows past the actual query length are written as 0 with LSE +inf.
#include <type_traits>

#include "fia_device.h"

namespace fia {

namespace {

constexpr int BM = kPrefillRows;  // 128
constexpr int BN = kPrefillKeys;  // 64

template <int D>
struct PrefillLds {
  static constexpr int ROW = D * 2;             // bytes per key / value row (swizzled, no padding)
  static constexpr int BYTES = BN * ROW;        // one stage of one tile
};

template <int D>
struct TileRegs {
  static constexpr int NK = BN * D / 8 / 256;   // 16-byte pieces of a tile per thread
  u32x4 k[NK];
  u32x4 v[NK];
};

// XOR swizzle of value rows in LDS: 16-byte piece q of row r sits in slot
// q ^ val_swz<PR>(r).  The value product reads them with 8-byte transpose
// reads in which one group of 16 lanes touches four consecutive rows
// (r % 4 = 0..3) and 32 contiguous bytes of each, and two neighbouring
// groups the next 32 bytes: the swizzle sends those 4 x 2 (or 4 x 4) pieces
// to distinct slots of the 128-byte (or 256-byte) bank window.
template <int PR>
__device__ __forceinline__ int val_swz(int r) {
  if constexpr (PR == 16) {
    constexpr int f = (0 << 0) | (6 << 4) | (10 << 8) | (12 << 12);
    return (f >> (4 * (r & 3))) & 15;
  } else {
    return 2 * (r & 3);
  }
}

}  // namespace

// KVM selects how key / value rows are addressed: 0 dense or TND (a tile is
// one strided run, its base advances by pointer arithmetic), 1 paged with
// block_size a multiple of 64 (a tile lies in one page, one table lookup per
// tile), 2 any paged layout (per-row lookup).
//
// Key and value tiles go global -> LDS by buffer-to-LDS loads (KVM 0 / 1) or
// through registers (KVM 2), row-major with an XOR swizzle.  Each stage is
// its own LDS array, so the compiler's wait for an outstanding buffer-to-LDS
// load only guards reads of that stage.
//
// EXT: an explicit mask tensor (modes 0 / 1) and / or a bias tensor (pse
// type 0).  Both enter through the
// initial value of the score accumulators: -inf for a masked key, bias /
// scale otherwise (the scaled score is then q.k * scale + bias).  Their
// loads for tile t + 1 go out at the end of step t, so they are in
// registers only between the steps.
template <int D, bool ALIBI, int KVM, bool EXT>
__global__ __launch_bounds__(256, 2) void prefill_bf16(AttnArgs a) {
  using L = PrefillLds<D>;
  constexpr int NQ = D / 16;   // 16-wide d chunks of the score product
  constexpr int NMB = D / 32;  // 32-wide d blocks of the output
  constexpr int DCH = D / 8;   // 16-byte pieces per row
  constexpr int NK = TileRegs<D>::NK;
  constexpr int RPI = 64 / DCH;   // key rows per 64-lane buffer-to-LDS load
  constexpr bool DMA_K = KVM != 2;
  // PIPE: the score product of tile t+1 is issued together with the softmax
  // of tile t (needs a second score buffer; too many registers with the ALiBi
  // bias, mask / bias tensors or per-row paging, which compute each tile's
  // scores up front).
  constexpr bool PIPE = !ALIBI && !EXT && KVM != 2;
  constexpr bool INTERLEAVE = PIPE;
  __shared__ __attribute__((aligned(16))) uint8_t lds_k0[L::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_k1[L::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v0[L::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v1[L::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;

  const int w0 = a.work[2 * blockIdx.x];
  const int w1 = a.work[2 * blockIdx.x + 1];
  const int b = w0;
  const int h = w1 & 0xff;
  const int qt = w1 >> 8;
  const int kvh = h / a.G;
  const int32_t* bm = a.meta + (int64_t)b * BF_COUNT;
  const int Lq = bm[BF_QLEN];
  // Key length: the plan's, or read on the device and clamped into [0, bound].
  const int Lk = a.dev_kvlen != nullptr ? min(max(a.dev_kvlen[b], 0), a.kvlen_bound) : bm[BF_KVLEN];
  const int q_off = bm[BF_QOFF], kv_off = bm[BF_KVOFF];
  const int write_rows = a.tnd ? Lq : a.Sq;

  const int i0 = qt * BM;
  const int iw0 = i0 + 32 * wave;
  const int i = iw0 + n;
  const bool row_live = i < Lq;

  // Key range of the whole tile and of this wave (monotone in the row).
  const int rows_end = min(i0 + BM, Lq);
  int klo = 0, khi = 0;
  if (rows_end > i0) {
    int l0, h0, l1, h1;
    visible_range(a, i0, Lq, Lk, l0, h0);
    visible_range(a, rows_end - 1, Lq, Lk, l1, h1);
    klo = l0;
    khi = h1;
  }
  int my_lo = 0, my_hi = 0;
  if (row_live) visible_range(a, i, Lq, Lk, my_lo, my_hi);
  int wlo_min = 0, wlo_max = 0, whi_min = 0, whi_max = 0;
  const int wrows_end = min(iw0 + 32, Lq);
  if (wrows_end > iw0) {
    visible_range(a, iw0, Lq, Lk, wlo_min, whi_min);
    visible_range(a, wrows_end - 1, Lq, Lk, wlo_max, whi_max);
  }

  float m_run = kNegInf;
  float l_run = 0.f;
  f32x16 o[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;
  }

  if (khi > klo) {
    // The wave's query rows, B operand of the score product.
    u32x4 qreg[NQ];
    const uint16_t* qp = (const uint16_t*)a.q + (int64_t)b * a.q_sb +
                         (int64_t)(q_off + i) * a.q_ss + (int64_t)h * a.q_sh + 8 * hh;
    // ALiBi enters through the initial value of the score accumulators,
    // slope ((kv_start + j) - (q_start + i)) / scale, so that the scaled
    // score q.k scale + bias comes out of the product; the softmax is then
    // the plain one.  With scale 0 the score is the bias alone: the query
    // operand is zero and the accumulators start at the bias in log2 units
    // (scaled by 1).
    const bool alibi_s0 = ALIBI && !(a.scale_log2 > 0.f);
    const float scl = alibi_s0 ? 1.f : a.scale_log2;
    const float c_al = ALIBI ? (alibi_s0 ? a.slopes[h] * kLog2e : a.slopes[h] / a.scale) : 0.f;
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      qreg[c] = (row_live && !alibi_s0) ? ld16(qp + 16 * c) : u32x4{0, 0, 0, 0};
    }

    // Explicit mask and bias rows of this lane's query row (rows past Q_S
    // are dead; their index is clamped into the tensor).
    const bool has_mask = EXT && a.mask != nullptr;
    const bool has_pse = EXT && a.pse != nullptr;
    const uint8_t* mrow = has_mask ? a.mask + (int64_t)b * a.mask_sb +
                                         (int64_t)min(i, a.mask_rows - 1) * a.mask_ss
                                   : nullptr;
    const uint16_t* prow = has_pse ? (const uint16_t*)a.pse + (int64_t)b * a.pse_sb +
                                         (int64_t)h * a.pse_sh +
                                         (int64_t)min(i, a.pse_rows - 1) * a.pse_ss
                                   : nullptr;
    uint32_t mw[8];
    u32x2 pw[8];
    const float inv_scale = EXT ? a.inv_scale : 0.f;
    // Mask bytes and bias values of keys j0 + 4 hh + 32 k2 + 8 g .. + 3
    // (4-aligned; a group past the tensor's width lies past every visible
    // key: address clamped, values unused).
    auto load_ext = [&](int kt) FIA_INLINE {
      if constexpr (EXT) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int j = kt * BN + 4 * hh + 32 * k2 + 8 * g4;
            mw[4 * k2 + g4] = has_mask ? *reinterpret_cast<const uint32_t*>(mrow + min(j, a.mask_cols - 4)) : 0u;
            pw[4 * k2 + g4] = has_pse ? *reinterpret_cast<const u32x2*>(prow + min(j, a.pse_cols - 4))
                                      : u32x2{0u, 0u};
          }
        }
      }
    };
    const uint16_t* kg = (const uint16_t*)a.k;
    const uint16_t* vg = (const uint16_t*)a.v;
    const uint16_t* kbase0 = kg + (int64_t)b * a.k_sb + (int64_t)kv_off * a.k_ss + (int64_t)kvh * a.k_sh;
    const uint16_t* vbase0 = vg + (int64_t)b * a.v_sb + (int64_t)kv_off * a.v_ss + (int64_t)kvh * a.v_sh;

    // Key / value staging.  Buffer-to-LDS load q of wave w fills rows
    // RPI (4 q + w) .. + RPI - 1 of the tile (1 KiB, lane l -> slot l % DCH
    // of row l / DCH), fetching the global piece that belongs in that slot.
    // With registers (KVM 2), thread u = tid + 256 q holds piece u % DCH of
    // row u / DCH and stores it into its slot.  Keys and values differ only
    // in their swizzle.
    // Consecutive q differ by a fixed number of rows with the same swizzle,
    // so one offset per lane plus a uniform step per q covers them.
    constexpr int QROWS = 256 / DCH;   // tile rows per q
    uint32_t koff, voff;
    if constexpr (DMA_K) {
      const int r = RPI * wave + lane / DCH;
      koff = (uint32_t)(r * a.k_ss + 8 * ((lane % DCH) ^ key_swz<DCH>(r))) * 2u;
      voff = (uint32_t)(r * a.v_ss + 8 * ((lane % DCH) ^ val_swz<DCH>(r))) * 2u;
    } else {
      const int r = tid / DCH;
      koff = (uint32_t)(r * L::ROW + 16 * ((tid % DCH) ^ key_swz<DCH>(r)));
      voff = (uint32_t)(r * L::ROW + 16 * ((tid % DCH) ^ val_swz<DCH>(r)));
    }
    const uint32_t kq_step = (uint32_t)(QROWS * a.k_ss) * 2u;
    const uint32_t vq_step = (uint32_t)(QROWS * a.v_ss) * 2u;
    // Score-operand reads: lane (n, hh) reads piece 2 c + hh of key rows
    // 32 k2 + n, which all share the swizzle of row n.
    uint32_t kr_addr[NQ];
    {
      const int sw = key_swz<DCH>(n);
#pragma unroll
      for (int c = 0; c < NQ; ++c) kr_addr[c] = (uint32_t)(n * L::ROW + 16 * ((2 * c + hh) ^ sw));
    }
    // Value-operand reads (transpose reads of row-major value rows).  For
    // k-step kk of the value product, lane (m, hh) needs V[key][32 mb + m]
    // for the keys whose probabilities it holds in the score accumulators:
    // 16 kk + 4 hh + (0..3), then 16 kk + 8 + 4 hh + (0..3).  In one
    // transpose read, lane 4 t + r' of a 16-lane group addresses row
    // 16 kk + 8 h + 4 hh + t at 8-byte column 8 mb + 4 (m / 16) + r', so
    // lane i of the group receives V[row t][32 mb + 16 (m / 16) + i].
    uint32_t vr_addr[NMB];
    {
      const int gi = lane & 15;
      const int t = gi >> 2, rp = gi & 3;
      const int half = (lane >> 4) & 1;
      const int r = 4 * hh + t;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const int c8 = 8 * mb + 4 * half + rp;
        vr_addr[mb] = (uint32_t)(r * L::ROW + 16 * ((c8 >> 1) ^ val_swz<DCH>(r)) + 8 * (c8 & 1));
      }
    }
    TileRegs<D> regs;

    // Resources (or, for KVM 2, register loads) of key / value tile kt.
    // Rows >= Lk fall outside the resources and read as zero.
    auto tile_rsrc = [&](int kt, __amdgpu_buffer_rsrc_t& rk, __amdgpu_buffer_rsrc_t& rv) FIA_INLINE {
      const int j0 = kt * BN;
      const uint16_t* kp;
      const uint16_t* vp;
      if constexpr (KVM == 0) {
        kp = kbase0 + (int64_t)j0 * a.k_ss;
        vp = vbase0 + (int64_t)j0 * a.v_ss;
      } else {
        const uint32_t page = fast_div((uint32_t)j0, a.bs_div);
        const int blk = clamp_block(a.block_table[(int64_t)b * a.bt_sb + page], a.n_blocks);
        const int slot = j0 - (int)page * a.block_size;
        kp = kg + paged_row_offset(blk, slot, kvh, a.k_sb, a.k_ss, a.k_sh);
        vp = vg + paged_row_offset(blk, slot, kvh, a.v_sb, a.v_ss, a.v_sh);
      }
      const int nvalid = min(BN, Lk - j0);
      rk = make_rsrc(kp, (uint32_t)((nvalid - 1) * a.k_ss + D) * 2u);
      rv = make_rsrc(vp, (uint32_t)((nvalid - 1) * a.v_ss + D) * 2u);
    };
    // Keys (or values) of tile kt straight into stage `dst` by buffer-to-LDS
    // loads (KVM 0 / 1).
    auto load_k_lds = [&](int kt, uint8_t* dst) FIA_INLINE {
      __amdgpu_buffer_rsrc_t rk, rv;
      tile_rsrc(kt, rk, rv);
#pragma unroll
      for (int q = 0; q < NK; ++q) buf_ld16_lds(rk, dst + 1024 * (4 * q + wave), koff + q * kq_step);
    };
    auto load_v_lds = [&](int kt, uint8_t* dst) FIA_INLINE {
      __amdgpu_buffer_rsrc_t rk, rv;
      tile_rsrc(kt, rk, rv);
#pragma unroll
      for (int q = 0; q < NK; ++q) buf_ld16_lds(rv, dst + 1024 * (4 * q + wave), voff + q * vq_step);
    };
    // KVM 2: keys and values of tile kt into registers (per-row page
    // lookups; rows >= Lk read as zero), then into their stages.
    auto load_regs = [&](int kt) FIA_INLINE {
      const int j0 = kt * BN;
#pragma unroll
      for (int q = 0; q < NK; ++q) {
        const int u = tid + 256 * q;
        const int j = j0 + u / DCH;
        u32x4 val = {0, 0, 0, 0};
        if (j < Lk) val = ld16(kg + kv_row_offset(a, a.k_sb, a.k_ss, a.k_sh, b, j, kvh, kv_off) + 8 * (u % DCH));
        regs.k[q] = val;
      }
#pragma unroll
      for (int q = 0; q < NK; ++q) {
        const int u = tid + 256 * q;
        const int j = j0 + u / DCH;
        u32x4 val = {0, 0, 0, 0};
        if (j < Lk) val = ld16(vg + kv_row_offset(a, a.v_sb, a.v_ss, a.v_sh, b, j, kvh, kv_off) + 8 * (u % DCH));
        regs.v[q] = val;
      }
    };
    auto store_regs = [&](uint8_t* kst, uint8_t* vst) FIA_INLINE {
#pragma unroll
      for (int q = 0; q < NK; ++q) {
        *reinterpret_cast<u32x4*>(kst + koff + q * QROWS * L::ROW) = regs.k[q];
        *reinterpret_cast<u32x4*>(vst + voff + q * QROWS * L::ROW) = regs.v[q];
      }
    };

    // Initial score accumulators of tile kt: the mask and bias tensors
    // (from the mask words / bias values loaded by load_ext) and the ALiBi
    // bias.  Accumulator r of key block k2 holds key 32 k2 + 8 (r / 4) +
    // r % 4 of the lane's 4 hh group; the ALiBi term is an fma with that
    // constant offset (an fma is not split, so no 32 loop-invariant products
    // are kept in registers).
    auto init_acc = [&](int kt, f32x16* sv) FIA_INLINE {
      const float cb = ALIBI ? c_al * (float)(kt * BN + 4 * hh - i + a.alibi_delta) : 0.f;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = 0.f;
          if constexpr (ALIBI) x = __builtin_fmaf(c_al, (float)(32 * k2 + 8 * (r >> 2) + (r & 3)), cb);
          if constexpr (EXT) {
            const uint32_t pv = pw[4 * k2 + (r >> 2)][(r >> 1) & 1];
            const float bias = __builtin_bit_cast(float, (r & 1) ? (pv & 0xffff0000u) : (pv << 16));
            const bool off = ((mw[4 * k2 + (r >> 2)] >> (8 * (r & 3))) & 0xffu) != 0u;
            x = off ? kNegInf : __builtin_fmaf(bias, inv_scale, x);
          }
          sv[k2][r] = x;
        }
      }
    };
    // S^T of one tile for this wave: 2 key blocks x 32 query rows, added to
    // the accumulators' initial value with ACC (else from zero).
    auto compute_s = [&](auto acc_tag, const uint8_t* kst, f32x16* sv) FIA_INLINE {
      constexpr bool ACC = decltype(acc_tag)::value;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        sv[k2] = mfma32(*reinterpret_cast<const u32x4*>(kst + kr_addr[0] + 32 * k2 * L::ROW), qreg[0],
                        ACC ? sv[k2] : f32x16{});
      }
#pragma unroll
      for (int c = 1; c < NQ; ++c) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          sv[k2] = mfma32(*reinterpret_cast<const u32x4*>(kst + kr_addr[c] + 32 * k2 * L::ROW),
                          qreg[c], sv[k2]);
        }
      }
    };
    // Scores of tile kt into sv (keys in stage kst).
    auto scores = [&](int kt, const uint8_t* kst, f32x16* sv) FIA_INLINE {
      if constexpr (ALIBI || EXT) {
        init_acc(kt, sv);
        compute_s(std::true_type{}, kst, sv);
      } else {
        compute_s(std::false_type{}, kst, sv);
      }
    };
    auto wave_skip = [&](int kt) FIA_INLINE {
      const int j0 = kt * BN;
      return (wrows_end <= iw0) || (j0 + BN <= wlo_min) || (j0 >= whi_max);
    };

    // Softmax of tile kt (scores in sc), then O += V^T P^T from `vst`.  With
    // DO_NEXT the score product of the next tile (keys in stage `knx`) is
    // issued inside the same straight-line block, so its MFMAs overlap this
    // tile's VALU work.
    auto tile_body = [&](auto masked_tag, int kt, const uint8_t* vst, f32x16* sc,
                         auto next_tag, const uint8_t* knx, f32x16* sn) FIA_INLINE {
      constexpr bool MASKED = decltype(masked_tag)::value;
      constexpr bool DO_NEXT = decltype(next_tag)::value;
      constexpr bool PLAIN = !MASKED;
      const int j0 = kt * BN;
      float mx = kNegInf;
      if constexpr (PLAIN) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[k2][r]);
        }
        mx *= scl;
      } else {
        const int jb = j0 + 4 * hh;
        // visible iff rel_lo <= koff < rel_hi, tested as one unsigned compare
        const uint32_t nlo = (uint32_t)(jb - my_lo);
        const uint32_t span = (uint32_t)(my_hi - my_lo);
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int koff = 32 * k2 + 8 * (r >> 2) + (r & 3);
            float x = sc[k2][r] * scl;
            if constexpr (MASKED) {
              bool keep = (uint32_t)koff + nlo < span;
              if constexpr (EXT) keep = keep && sc[k2][r] != kNegInf;   // masked-out key
              x = keep ? x : kNegInf;
            }
            sc[k2][r] = x;
            mx = fmaxf(mx, x);
          }
        }
      }
      mx = pair32_max(mx);
      // Lazy rescale: keep the running max m_run unless a row's new max
      // exceeds it by more than 8 (probabilities stay <= 2^8).
      const bool grow = mx > m_run + 8.f;
      if (__any(grow)) {
        const float m_new = grow ? mx : m_run;
        const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) o[mb] *= alpha;
      }
      const float m_sub = (m_run == kNegInf) ? 0.f : m_run;
      // Raised wave priority from here to the end of the value product: the
      // arbiter then favours this wave's MFMA / LDS stream over the softmax
      // VALU work of the other wave on the SIMD.
      __builtin_amdgcn_s_setprio(1);
      if constexpr (PIPE) {
        if constexpr (DO_NEXT) scores(kt + 1, knx, sn);
      }
      float psum = 0.f;
      u32x4 pb[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int k2 = kk >> 1;
        const int rb = 8 * (kk & 1);
        float p[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          p[t] = PLAIN ? fast_exp2(__builtin_fmaf(sc[k2][rb + t], scl, -m_sub))
                       : fast_exp2(sc[k2][rb + t] - m_sub);
          psum += p[t];
        }
        pb[kk] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                       pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
      }
      l_run += psum;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          const uint8_t* vp = vst + vr_addr[mb] + 16 * kk * L::ROW;
          const u32x2 lo = lds_tr16(vp);
          const u32x2 hi = lds_tr16(vp + 8 * L::ROW);
          o[mb] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[kk], o[mb]);
        }
      }
      // Order of the block's instructions (the hints have to come before the
      // priority change: the scheduler does not move instructions across
      // it).  The first key-operand reads of the next score product go out
      // ahead; then each score MFMA is followed by one LDS read and a few
      // softmax VALU instructions, and each value MFMA by two transpose reads
      // and more VALU work, so no MFMA waits for a read issued just before it.
      if constexpr (INTERLEAVE) {
        constexpr int SM = DO_NEXT ? 2 * NQ : 0;   // score MFMAs in the block
        constexpr int VM = 4 * NMB;                // value MFMAs
        if constexpr (DO_NEXT) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
        for (int g = 0; g < SM; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
#pragma unroll
        for (int g = 0; g < VM; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    };

    // Software pipeline over key tiles, two stages (stage of tile kt:
    // (kt - kt0) & 1).  Step kt holds the scores of tile kt in registers
    // (with PIPE) and computes softmax(kt) + PV(kt) together with the score
    // product of tile kt + 1; one barrier ends it.  Buffer-to-LDS loads
    // (KVM 0 / 1) go out at the start of a step into stages no wave reads in
    // that step: the values of tile kt + 1, and the keys of tile kt + 2
    // (with PIPE the keys of tile kt were consumed one step earlier) or of
    // tile kt + 1.  The barrier ending the step waits for them.  With
    // registers (KVM 2) tile kt + 2 is loaded at the start of step kt and
    // stored after its barrier into the stages tile kt used.
    const int kt0 = klo / BN;
    const int kt1 = (khi + BN - 1) / BN;
    const bool has1 = kt0 + 1 < kt1;
    if constexpr (DMA_K) {
      load_k_lds(kt0, lds_k0);
      load_v_lds(kt0, lds_v0);
      if (PIPE && has1) load_k_lds(kt0 + 1, lds_k1);
      barrier_after_loads();
    } else {
      load_regs(kt0);
      store_regs(lds_k0, lds_v0);
      if (has1) {
        load_regs(kt0 + 1);
        store_regs(lds_k1, lds_v1);
      }
      __syncthreads();
    }
    f32x16 s_a[2], s_b[2];
    bool cur_skip = wave_skip(kt0);
    if (PIPE && !cur_skip) scores(kt0, lds_k0, s_a);
    if (EXT && !cur_skip) load_ext(kt0);
    if (PIPE) __syncthreads();   // step kt0 refills lds_k0

    auto step = [&](auto stage_tag, int kt, f32x16* sc, f32x16* sn) FIA_INLINE {
      constexpr int S = decltype(stage_tag)::value;
      uint8_t* kst = S ? lds_k1 : lds_k0;
      uint8_t* vst = S ? lds_v1 : lds_v0;
      uint8_t* knx = S ? lds_k0 : lds_k1;
      uint8_t* vnx = S ? lds_v0 : lds_v1;
      const bool has_next = kt + 1 < kt1;
      const bool has_next2 = kt + 2 < kt1;
      if constexpr (DMA_K) {
        if constexpr (PIPE) {
          if (has_next2) load_k_lds(kt + 2, kst);
        } else {
          if (has_next) load_k_lds(kt + 1, knx);
        }
        if (has_next) load_v_lds(kt + 1, vnx);
      } else {
        if (has_next2) load_regs(kt + 2);
      }
      const bool next_skip = has_next ? wave_skip(kt + 1) : true;
      // The next tile's keys are always read from the other stage array
      // itself (not through a pointer chosen at run time), so the compiler
      // sees that they cannot alias this step's buffer-to-LDS loads.
      const bool do_next = PIPE && !next_skip;
      if (!PIPE && !cur_skip) scores(kt, kst, sc);
      if (!cur_skip) {
        const int j0 = kt * BN;
        // Tiles inside every row's visible range skip the per-element test;
        // with a mask / bias tensor too: masked keys already hold -inf in the
        // score accumulators, which the plain path maps to probability 0 as
        // long as the scale is positive.  With scale 0 the plain path would
        // form -inf * 0 = NaN, so such calls keep the per-element test, which
        // replaces a masked key's score by -inf after scaling.
        const bool need_mask = !(j0 >= wlo_max && j0 + BN <= whi_min) ||
                               (EXT && !(scl > 0.f));
        if (need_mask) {
          if (do_next) {
            tile_body(std::true_type{}, kt, vst, sc, std::true_type{}, knx, sn);
          } else {
            tile_body(std::true_type{}, kt, vst, sc, std::false_type{}, knx, sn);
          }
        } else {
          if (do_next) {
            tile_body(std::false_type{}, kt, vst, sc, std::true_type{}, knx, sn);
          } else {
            tile_body(std::false_type{}, kt, vst, sc, std::false_type{}, knx, sn);
          }
        }
      } else if (do_next) {
        scores(kt + 1, knx, sn);
      }
      cur_skip = next_skip;
      barrier_after_loads();   // this step's loads landed; every wave is done with tile kt
      if constexpr (!DMA_K) {
        if (has_next2) store_regs(kst, vst);
      }
      if (EXT && !next_skip) load_ext(kt + 1);
    };
    for (int kt = kt0; kt < kt1; kt += 2) {
      step(std::integral_constant<int, 0>{}, kt, s_a, s_b);
      if (kt + 1 < kt1) step(std::integral_constant<int, 1>{}, kt + 1, s_b, s_a);
    }
  }

  // Epilogue: normalise and write this lane's row.
  float l_tot = pair32_sum(l_run);
  bool has = row_live && m_run != kNegInf && l_tot > 0.f;
  float o_scale = 1.f;
  if (a.sink != nullptr && row_live) {
    // The sink: one more softmax term with a zero value vector.
    const float z = bf16_to_f32(a.sink[h]) * kLog2e;
    const float m_new = fmaxf(m_run, z);
    o_scale = (m_run == kNegInf) ? 0.f : fast_exp2(m_run - m_new);
    l_tot = l_tot * o_scale + fast_exp2(z - m_new);
    m_run = m_new;
    has = true;
  }
  const float inv = has ? o_scale / l_tot : 0.f;
  if (i < write_rows) {
    uint16_t* op = (uint16_t*)a.o + (int64_t)b * a.o_sb + (int64_t)(q_off + i) * a.o_ss +
                   (int64_t)h * a.o_sh;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * mb + 8 * q4 + 4 * hh;
        const u32x2 w = {pack_bf16x2(o[mb][4 * q4 + 0] * inv, o[mb][4 * q4 + 1] * inv),
                         pack_bf16x2(o[mb][4 * q4 + 2] * inv, o[mb][4 * q4 + 3] * inv)};
        st8(op + d0, w);
      }
    }
    if (a.write_lse && hh == 0) {
      a.lse[(int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)(q_off + i) * a.lse_ss] =
          has ? (m_run + fast_log2(l_tot)) * kLn2 : kPosInf;
    }
  }

  // Padded query layouts: tiles wholly past the actual query length get no
  // work item; the items of the live tiles write their rows (0, LSE +inf),
  // item qt taking tiles nl + qt, nl + qt + nl, ... (nl live tiles, at
  // least 1).
  if (!a.tnd) {
    const int nqt = (a.Sq + BM - 1) / BM;
    const int nl = max((Lq + BM - 1) / BM, 1);
    const int dp = tid % DCH;
    for (int t = nl + qt; t < nqt; t += nl) {
#pragma unroll
      for (int r0 = 0; r0 < BM; r0 += 256 / DCH) {
        const int row = t * BM + r0 + tid / DCH;
        if (row < a.Sq) {
          uint16_t* op = (uint16_t*)a.o + (int64_t)b * a.o_sb + (int64_t)row * a.o_ss +
                         (int64_t)h * a.o_sh + 8 * dp;
          st16(op, u32x4{0u, 0u, 0u, 0u});
          if (a.write_lse && dp == 0) {
            a.lse[(int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)row * a.lse_ss] = kPosInf;
          }
        }
      }
    }
  }
}

template <int D, bool ALIBI, int KVM>
static hipError_t launch_one(const AttnArgs& a, hipStream_t s) {
  if (a.mask != nullptr || a.pse != nullptr) {
    prefill_bf16<D, ALIBI, KVM, true><<<a.n_work, 256, 0, s>>>(a);
  } else {
    prefill_bf16<D, ALIBI, KVM, false><<<a.n_work, 256, 0, s>>>(a);
  }
  return hipSuccess;
}

template <int D, bool ALIBI>
static hipError_t launch_kvm(const AttnArgs& a, hipStream_t s) {
  if (!a.paged) return launch_one<D, ALIBI, 0>(a, s);
  if (a.tile_contig) return launch_one<D, ALIBI, 1>(a, s);
  return launch_one<D, ALIBI, 2>(a, s);
}

hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.n_work <= 0) return hipSuccess;
  const bool alibi = a.slopes != nullptr;
  hipError_t e;
  if (a.D == 128) {
    e = alibi ? launch_kvm<128, true>(a, s) : launch_kvm<128, false>(a, s);
  } else {
    e = alibi ? launch_kvm<64, true>(a, s) : launch_kvm<64, false>(a, s);
  }
  return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace fia
