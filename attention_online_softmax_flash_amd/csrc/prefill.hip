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
// k-step follows the accumulator layout of S^T; V^T is read from LDS in the
// same order, so P needs no shuffling.  V is transposed into LDS on the way in.
//
// Masks (aclnnFusedInferAttentionScoreV5 Attention Mask group): per query row
// i the visible keys are [lo(i), hi(i)); tiles wholly inside every row's range
// of a wave skip the per-element test, tiles outside are skipped.  ALiBi
// (pse type 2) adds slope * ((kv_start + j) - (q_start + i)) after scaling
// (aclnnFusedInferAttentionScoreV4 formula).  Rows with no visible key and
// rows past the actual query length are written as 0 with LSE +inf.
#include "fia_device.h"

namespace fia {

namespace {

constexpr int BM = kPrefillRows;  // 128
constexpr int BN = kPrefillKeys;  // 64

template <int D>
struct PrefillLds {
  static constexpr int K_PITCH = D * 2 + 16;    // bytes per key row
  static constexpr int V_PITCH = BN * 2 + 8;    // bytes per transposed value row
  static constexpr int K_BYTES = BN * K_PITCH;
  static constexpr int V_BYTES = D * V_PITCH;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int TOTAL = 2 * STAGE;
};

template <int D>
struct TileRegs {
  static constexpr int NK = BN * D / 8 / 256;   // 16-byte key pieces per thread
  u32x4 k[NK];
  u32x4 v[4];
};

}  // namespace

template <int D, bool ALIBI>
__global__ __launch_bounds__(256, 2) void prefill_bf16(AttnArgs a) {
  using L = PrefillLds<D>;
  constexpr int NQ = D / 16;   // 16-wide d chunks of the score product
  constexpr int NMB = D / 32;  // 32-wide d blocks of the output
  constexpr int DCH = D / 8;   // 16-byte pieces per row
  extern __shared__ __align__(16) uint8_t lds[];

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
  const int Lq = bm[BF_QLEN], Lk = bm[BF_KVLEN];
  const int q_off = bm[BF_QOFF], kv_off = bm[BF_KVOFF];
  const int write_rows = a.tnd ? Lq : a.Sq;

  const int i0 = qt * BM;
  const int iw0 = i0 + 32 * wave;
  const int i = iw0 + n;
  const bool row_live = i < Lq;

  // Key range of the whole tile and of this wave.
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
#pragma unroll
    for (int c = 0; c < NQ; ++c) qreg[c] = row_live ? ld16(qp + 16 * c) : u32x4{0, 0, 0, 0};

    const float c_al = ALIBI ? a.slopes[h] * kLog2e : 0.f;
    const uint16_t* kg = (const uint16_t*)a.k;
    const uint16_t* vg = (const uint16_t*)a.v;

    // Thread roles for staging one tile.
    const int va = tid & 15;   // keys 4 va .. 4 va + 3
    const int vq = tid >> 4;   // 16-byte value column piece
    TileRegs<D> regs;

    auto load_tile = [&](int kt) {
      const int j0 = kt * BN;
#pragma unroll
      for (int q = 0; q < TileRegs<D>::NK; ++q) {
        const int u = tid + 256 * q;
        const int key = u / DCH;
        const int dch = u % DCH;
        const int j = j0 + key;
        u32x4 val = {0, 0, 0, 0};
        if (j < Lk) {
          const int64_t off = kv_row_offset(a, a.k_sb, a.k_ss, a.k_sh, b, j, kvh, kv_off);
          val = ld16(kg + off + 8 * dch);
        }
        regs.k[q] = val;
      }
      if (vq < DCH) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = j0 + 4 * va + q;
          u32x4 val = {0, 0, 0, 0};
          if (j < Lk) {
            const int64_t off = kv_row_offset(a, a.v_sb, a.v_ss, a.v_sh, b, j, kvh, kv_off);
            val = ld16(vg + off + 8 * vq);
          }
          regs.v[q] = val;
        }
      }
    };
    auto store_tile = [&](int stage) {
      uint8_t* kb = lds + stage * L::STAGE;
      uint8_t* vb = kb + L::K_BYTES;
#pragma unroll
      for (int q = 0; q < TileRegs<D>::NK; ++q) {
        const int u = tid + 256 * q;
        const int key = u / DCH;
        const int dch = u % DCH;
        *reinterpret_cast<u32x4*>(kb + key * L::K_PITCH + dch * 16) = regs.k[q];
      }
      if (vq < DCH) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          u32x2 pr;
          if (e & 1) {
            pr = u32x2{pick_hi(regs.v[0][w], regs.v[1][w]), pick_hi(regs.v[2][w], regs.v[3][w])};
          } else {
            pr = u32x2{pick_lo(regs.v[0][w], regs.v[1][w]), pick_lo(regs.v[2][w], regs.v[3][w])};
          }
          *reinterpret_cast<u32x2*>(vb + (8 * vq + e) * L::V_PITCH + va * 8) = pr;
        }
      }
    };

    const int kt0 = klo / BN;
    const int kt1 = (khi + BN - 1) / BN;
    load_tile(kt0);
    store_tile(0);
    __syncthreads();

    for (int kt = kt0; kt < kt1; ++kt) {
      const int stage = (kt - kt0) & 1;
      const bool more = kt + 1 < kt1;
      if (more) load_tile(kt + 1);

      const int j0 = kt * BN;
      const bool wave_skip = (wrows_end <= iw0) || (j0 + BN <= wlo_min) || (j0 >= whi_max);
      if (!wave_skip) {
        const bool need_mask = !(j0 >= wlo_max && j0 + BN <= whi_min);
        const uint8_t* kb = lds + stage * L::STAGE;
        const uint8_t* vb = kb + L::K_BYTES;
        f32x16 s[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[k2][r] = 0.f;
#pragma unroll
          for (int c = 0; c < NQ; ++c) {
            const u32x4 av = *reinterpret_cast<const u32x4*>(
                kb + (32 * k2 + n) * L::K_PITCH + (16 * c + 8 * hh) * 2);
            s[k2] = mfma32(av, qreg[c], s[k2]);
          }
        }
        // Scale, bias, mask.  Key of slot (k2, r): j0 + 32 k2 + 8 (r/4) + 4 hh + r%4.
        float mx = kNegInf;
        const int jb = j0 + 4 * hh;
        const float cb = ALIBI ? c_al * (float)(jb - i + a.alibi_delta) : 0.f;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int koff = 32 * k2 + 8 * (r >> 2) + (r & 3);
            float x = s[k2][r] * a.scale_log2;
            if (ALIBI) x += __builtin_fmaf(c_al, (float)koff, cb);
            if (need_mask) {
              const int j = jb + koff;
              x = (j >= my_lo && j < my_hi) ? x : kNegInf;
            }
            s[k2][r] = x;
            mx = fmaxf(mx, x);
          }
        }
        mx = fmaxf(mx, shfl_xor_f(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        float psum = 0.f;
        u32x4 pb[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int k2 = kk >> 1;
          const int rb = 8 * (kk & 1);
          float p[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            p[t] = fast_exp2(s[k2][rb + t] - m_use);
            psum += p[t];
          }
          pb[kk] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                         pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          o[mb] *= alpha;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const uint8_t* vp = vb + (32 * mb + n) * L::V_PITCH + (16 * kk + 4 * hh) * 2;
            const u32x2 lo2 = *reinterpret_cast<const u32x2*>(vp);
            const u32x2 hi2 = *reinterpret_cast<const u32x2*>(vp + 16);
            const u32x4 av = {lo2.x, lo2.y, hi2.x, hi2.y};
            o[mb] = mfma32(av, pb[kk], o[mb]);
          }
        }
      }
      if (more) store_tile(stage ^ 1);
      __syncthreads();
    }
  }

  // Epilogue: normalise and write this lane's row.
  const float l_tot = l_run + shfl_xor_f(l_run, 32);
  const bool has = row_live && m_run != kNegInf && l_tot > 0.f;
  const float inv = has ? 1.f / l_tot : 0.f;
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
}

hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.n_work <= 0) return hipSuccess;
  const bool alibi = a.slopes != nullptr;
  if (a.D == 128) {
    constexpr int lds = PrefillLds<128>::TOTAL;
    if (alibi) {
      hipFuncSetAttribute((const void*)prefill_bf16<128, true>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      prefill_bf16<128, true><<<a.n_work, 256, lds, s>>>(a);
    } else {
      hipFuncSetAttribute((const void*)prefill_bf16<128, false>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      prefill_bf16<128, false><<<a.n_work, 256, lds, s>>>(a);
    }
  } else {
    constexpr int lds = PrefillLds<64>::TOTAL;
    if (alibi) {
      prefill_bf16<64, true><<<a.n_work, 256, lds, s>>>(a);
    } else {
      prefill_bf16<64, false><<<a.n_work, 256, lds, s>>>(a);
    }
  }
  return hipGetLastError();
}

}  // namespace fia
