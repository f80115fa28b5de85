// Incremental decode over a fake-quantised KV cache (aclnnFusedInferAttentionScoreV5,
// quantisation parameter group, fake-quant scenario): key and value rows are
// int8 or float8 e4m3fn codes, the query bf16.  A value is dequantised as
// scale * (code + offset), with the scale / offset either per channel
// ([KV_N, D], or one value for the whole tensor) or per token ([B, S2],
// shared by the KV heads).
//
// Same chunking, wave combine and partial format as the bf16 split-KV
// kernel, so the bf16 merge kernel folds the partials; work items run over
// KV heads, or over pairs of adjacent KV heads (one wave takes both: NH = 2).
// The scales and offsets are moved out of the MFMA operands:
//   * key, per channel:  s_j = sum_d (q_d ks_d) c_jd + sum_d q_d ks_d ko_d.  The
//     first term is a product of the raw codes against q * ks carried with
//     about 16 bits: int8 codes go into the int8 MFMA as loaded, against
//     q * ks = sq (qi + qj / 256) with int8 qi, qj; e4m3fn codes are
//     converted to bf16 (exact) against a bf16 high and low part of q * ks.
//     The second term is one constant per head.
//   * key, per token:    s_j = ks_j (q . c_j + ko_j sum_d q_d), q . c_j the same
//     product with ks = 1.
//   * value, per channel: o_d = vs_d (sum_j p_j c_jd / l + vo_d), applied to the
//     normalised chunk result (the merge is a convex combination, so it
//     commutes with this per-channel affine map).
//   * value, per token:  o_d = (sum_j (p_j vs_j) c_jd + sum_j p_j vs_j vo_j) / l;
//     p_j vs_j is the bf16 operand, the offset sum one fp32 value per head.
// Lane (n, g) of the score product holds d = (D / 4) g + 8 cc + e of both the
// key codes and the query (one permutation of d on both operands), so each
// lane loads D / 4 contiguous bytes of its key row.
#include "fia_device.h"

namespace fia {

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Elements i0 .. i0 + N - 1 of a per-channel scale / offset table (bf16 or
// fp32; every element is element 0 when `scalar`; zero without a table),
// every load issued before any is used: one trip to memory.  `count` is the
// table's element count (KV_N * D, or 1 when scalar).
template <int N>
__device__ __forceinline__ void chan_run(const void* p, int is_f32, int scalar, int64_t count, int i0,
                                         float (&out)[N]) {
  const uint32_t esz = is_f32 ? 4u : 2u;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(p, p != nullptr ? (uint32_t)(count * esz) : 0u);
  if (is_f32) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const uint32_t i = scalar ? 0u : (uint32_t)(i0 + k);
      out[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, i * 4u, 0, 0));
    }
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const uint32_t i = scalar ? 0u : (uint32_t)(i0 + k);
      out[k] = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, i * 2u, 0, 0));
    }
  }
}

// Byte K of the 4-byte word w as a float (int8 or e4m3fn code, exact).
template <bool FP8, int K>
__device__ __forceinline__ float code_byte(uint32_t w) {
  if constexpr (FP8) {
    return __builtin_amdgcn_cvt_f32_fp8((int)w, K);
  } else {
    return (float)(int8_t)(w >> (8 * K));
  }
}
// Same with the byte index known after unrolling.
template <bool FP8>
__device__ __forceinline__ float code_f32(uint32_t w, int k) {
  switch (k) {
    case 0: return code_byte<FP8, 0>(w);
    case 1: return code_byte<FP8, 1>(w);
    case 2: return code_byte<FP8, 2>(w);
    default: return code_byte<FP8, 3>(w);
  }
}

// Bytes 2 i and 2 i + 1 of w as a packed bf16 pair (e4m3fn codes; the
// conversion is exact).
template <int I>
__device__ __forceinline__ uint32_t fp8_pair_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, I == 1));
}

// Key operand: 8 e4m3fn codes (words w0, w1, bytes in order) as 8 bf16.
template <bool FP8>
__device__ __forceinline__ u32x4 codes8_bf16(uint32_t w0, uint32_t w1) {
  static_assert(FP8, "int8 key codes feed the int8 MFMA directly");
  return u32x4{fp8_pair_bf16<0>(w0), fp8_pair_bf16<1>(w0), fp8_pair_bf16<0>(w1), fp8_pair_bf16<1>(w1)};
}

// Byte k of x and byte k of y as a packed bf16 pair (x low).
template <bool FP8>
__device__ __forceinline__ uint32_t pair_bf16(uint32_t x, uint32_t y, int k) {
  if constexpr (FP8) {
    const uint32_t sel = (uint32_t)k | ((uint32_t)(4 + k) << 8) | 0x0c0c0000u;
    return fp8_pair_bf16<0>(__builtin_amdgcn_perm(y, x, sel));
  } else {
    return pack_bf16x2(code_f32<false>(x, k), code_f32<false>(y, k));
  }
}

// Split x into a bf16 high part and a bf16 low part (x - hi), as bits.
__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
  const uint32_t h = pack_bf16x2(x, 0.f) & 0xffffu;
  hi = h;
  lo = pack_bf16x2(x - bf16_to_f32((uint16_t)h), 0.f) & 0xffffu;
}

}  // namespace

// KPT / VPT: key / value scales per token (else per channel).  NH: KV heads
// per wave.  With NH = 2 (heads of a token adjacent in memory, G <= 8) a wave
// takes KV heads kvh and kvh + 1 of the same keys: their codes are one
// 2 D-byte run per token, loaded as a whole, and the G query heads of each
// fill columns [0, G) and [G, 2 G) of the 16-column MFMA tiles, so the
// softmax work of a column serves a real head twice as often.
template <int D, bool FP8, bool KPT, bool VPT, int NH>
__global__ __launch_bounds__(256, (KPT || VPT || FP8 || NH == 2) ? 3 : 4) void decode_split_q8(AttnArgs a) {
  constexpr int NC = D / 32;   // 32-wide k-steps of the score product per 16-key half
  constexpr int DPL = D / 16;  // value columns per lane column
  constexpr int KB = D / 4;    // key bytes per lane and row
  constexpr int NSUB = 2 / NH; // 32-key steps per load round (64 D bytes of key codes)
  constexpr int RB = NH * D;   // staged bytes per key row
  static_assert(NH == 1 || NH == 2, "one or two KV heads per wave");
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;

  int item = blockIdx.x;
  int hb = 0, kvh;
  if constexpr (NH == 1) {
    hb = item % a.n_head_blocks;
    item /= a.n_head_blocks;
    kvh = item % a.KVn;
    item /= a.KVn;
  } else {
    const int npair = a.KVn / 2;
    kvh = 2 * (item % npair);
    item /= npair;
  }
  const int cg = item;
  if (a.n_chunks_dev != nullptr && cg >= *a.n_chunks_dev) return;   // past the device plan's chunks
  const int b = a.work[2 * cg];
  const int c = a.work[2 * cg + 1];
  const int32_t* bm = a.meta + (int64_t)b * BF_COUNT;
  const int lo = bm[BF_LO], hi = bm[BF_HI];
  const int nchunk = bm[BF_NCHUNK], chunk0 = bm[BF_CHUNK0];
  const int kv_off = bm[BF_KVOFF], q_off = bm[BF_QOFF];

  const int C = a.chunk;
  const int wlen = C >> 2;
  const int cbase = (lo / C + c) * C;
  const int ws = cbase + wave * wlen;
  const int t_lo = max(ws, lo);
  const int t_hi = min(ws + wlen, hi);

  // Column n: query head hl of KV head kvl (with NH = 2 columns [G, 2 G)
  // belong to kvh + 1; columns past the heads are dead and carry a zero query).
  const int hs = (NH == 2 && n >= a.G) ? 1 : 0;
  const int hl = NH == 2 ? n - hs * a.G : hb * 16 + n;
  const bool hvalid = hl < a.G;
  const int kvl = kvh + hs;
  const int h = kvl * a.G + (hvalid ? hl : 0);

  // Query of head n at d = KB g + i (i < KB) -- the same permutation of d as
  // the key codes -- times the per-channel key scale (key per channel).  qc:
  // sum_d q_d ks_d ko_d (key per channel), or sum_d q_d (key per token).
  const uint16_t* qp = (const uint16_t*)a.q + (int64_t)b * a.q_sb + (int64_t)q_off * a.q_ss +
                       (int64_t)h * a.q_sh + KB * g;
  float qf[KB];
  float qc = 0.f;
  // Key per channel: the lane's KB scales and offsets (channels kvh D +
  // KB g ..), all requested together.
  float kcs[KPT ? 1 : KB], kco[KPT ? 1 : KB];
  if constexpr (!KPT) {
    const int64_t cnt = a.kq_scalar ? 1 : (int64_t)a.KVn * D;
    chan_run(a.kq_scale, a.kq_f32, a.kq_scalar, cnt, kvl * D + KB * g, kcs);
    chan_run(a.kq_off, a.kq_f32, a.kq_scalar, cnt, kvl * D + KB * g, kco);
  }
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    const u32x4 raw = hvalid ? ld16(qp + 8 * cc) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w = raw[e >> 1];
      const float qd = bf16_to_f32((uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu)));
      if constexpr (KPT) {
        qf[8 * cc + e] = qd;
        qc += qd;
      } else {
        qf[8 * cc + e] = qd * kcs[8 * cc + e];
        qc += qf[8 * cc + e] * kco[8 * cc + e];
      }
    }
  }
  // Sum over the four lanes of head n (lanes n, n + 16, n + 32, n + 48).
  qc += shfl_xor_f(qc, 16);
  qc += shfl_xor_f(qc, 32);
  // B operand of the score product.
  //  e4m3fn keys: bf16 MFMA; the query (scaled query: high and low bf16
  //    parts) as 8 bf16 per k-step cc.
  //  int8 keys: int8 MFMA on the raw codes; the query as sq * (qi + qj / 256)
  //    with int8 qi, qj (sq = max |q| / 127 per head), i.e. about 16 bits.
  u32x4 qh[NC], ql[NC];
  u32x4 qi[KB / 16], qj[KB / 16];
  float sq = 0.f;
  if constexpr (FP8) {
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      uint32_t hbits[8], lbits[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (KPT) {
          hbits[e] = pack_bf16x2(qf[8 * cc + e], 0.f) & 0xffffu;   // the bf16 query itself
          lbits[e] = 0u;
        } else {
          split_bf16(qf[8 * cc + e], hbits[e], lbits[e]);
        }
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        qh[cc][w] = hbits[2 * w] | (hbits[2 * w + 1] << 16);
        ql[cc][w] = lbits[2 * w] | (lbits[2 * w + 1] << 16);
      }
    }
  } else {
    float mabs = 0.f;
#pragma unroll
    for (int i = 0; i < KB; ++i) mabs = fmaxf(mabs, fabsf(qf[i]));
    mabs = fmaxf(mabs, shfl_xor_f(mabs, 16));
    mabs = fmaxf(mabs, shfl_xor_f(mabs, 32));
    sq = mabs > 0.f ? mabs * (1.f / 127.f) : 1.f;
    const float rq = 1.f / sq;
#pragma unroll
    for (int c4 = 0; c4 < KB / 16; ++c4) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t hw = 0u, lw = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x = qf[16 * c4 + 4 * w + k] * rq;
          const float xh = __builtin_rintf(x);
          const float xl = fminf(fmaxf(__builtin_rintf((x - xh) * 256.f), -127.f), 127.f);
          hw |= ((uint32_t)(int32_t)xh & 0xffu) << (8 * k);
          lw |= ((uint32_t)(int32_t)xl & 0xffu) << (8 * k);
        }
        qi[c4][w] = hw;
        qj[c4][w] = lw;
      }
    }
  }
  const float c_shift = KPT ? 0.f : qc * a.scale_log2;

  float m_run = kNegInf;
  float l_run = 0.f;
  float t_run = 0.f;   // value per token: sum_j p_j vs_j vo_j
  f32x4 o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint8_t* kbase = (const uint8_t*)a.k;
  const uint8_t* vbase = (const uint8_t*)a.v;
  const float* ksp = KPT ? (const float*)a.kq_scale + (int64_t)b * a.kq_sb : nullptr;
  const float* kop = KPT && a.kq_off ? (const float*)a.kq_off + (int64_t)b * a.kq_sb : nullptr;
  const float* vsp = VPT ? (const float*)a.vq_scale + (int64_t)b * a.vq_sb : nullptr;
  const float* vop = VPT && a.vq_off ? (const float*)a.vq_off + (int64_t)b * a.vq_sb : nullptr;

  // Per-wave staging inside the combine buffer (used after the loop): one
  // iteration's key rows (64 rows of D bytes, or 32 rows of the two heads'
  // 2 D bytes; row-major, 16-byte pieces XOR-swizzled so that the 16 rows
  // one operand read touches fall in distinct bank groups) and its
  // per-token tables (64 keys each).  All loads of an iteration -- keys,
  // values and tables of its 32-key steps -- go out before its first wait.
  constexpr int PR = RB / 16;                // 16-byte pieces per staged row
  constexpr int RPI = 64 / PR;               // rows per 64-lane buffer-to-LDS load
  constexpr int STAGE = 64 * D + 1024;       // bytes of one wave's stage
  constexpr int COMBINE = 4 * 16 * (D + 4) * 4;
  __shared__ __attribute__((aligned(16))) uint8_t sm_raw[COMBINE > 4 * STAGE ? COMBINE : 4 * STAGE];
  float(*sm_o)[16][D + 4] = reinterpret_cast<float(*)[16][D + 4]>(sm_raw);
  uint8_t* kst = sm_raw + wave * STAGE;
  float* tst = reinterpret_cast<float*>(kst + 64 * D);   // [4 tables][64 keys]
  // Lane l of buffer-to-LDS load `inst` fills slot l % PR of row
  // RPI inst + l / PR of a 32-key step, fetching the global piece that
  // belongs in that slot.
  uint32_t k_lds_off[PR / 2];
#pragma unroll
  for (int inst = 0; inst < PR / 2; ++inst) {
    const int r = RPI * inst + lane / PR;
    k_lds_off[inst] = (uint32_t)((r % 16) * a.k_ss + 16 * ((lane % PR) ^ key_swz<PR>(r)));
  }
  // Score operand reads: lane (n, g) reads piece (D / 16) x + (KB / 16) g + c4
  // of row 16 hf + n of a step (head x of the row).
  uint32_t k_rd[NH][2][KB / 16];
#pragma unroll
  for (int x = 0; x < NH; ++x) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int c4 = 0; c4 < KB / 16; ++c4) {
        const int r = 16 * hf + n;
        k_rd[x][hf][c4] = (uint32_t)(r * RB + 16 * (((D / 16) * x + (KB / 16) * g + c4) ^ key_swz<PR>(r)));
      }
    }
  }
  // Per-token table rows of the batch (no table: empty range, reads zero).
  const __amdgpu_buffer_rsrc_t r_ks = make_rsrc(ksp, ksp ? (uint32_t)a.kq_cols * 4u : 0u);
  const __amdgpu_buffer_rsrc_t r_ko = make_rsrc(kop, kop ? (uint32_t)a.kq_cols * 4u : 0u);
  const __amdgpu_buffer_rsrc_t r_vs = make_rsrc(vsp, vsp ? (uint32_t)a.vq_cols * 4u : 0u);
  const __amdgpu_buffer_rsrc_t r_vo = make_rsrc(vop, vop ? (uint32_t)a.vq_cols * 4u : 0u);
  auto lds_ptr = [](void* p) FIA_INLINE { return (__attribute__((address_space(3))) void*)p; };

  if (t_hi > t_lo) {
    const int first = ws + ((t_lo - ws) & ~31);
    const WavePages wp = wave_pages(a, b, first, hi - 1, lane);
    for (int ti = first; ti < t_hi; ti += NSUB * kDecodeStep) {
      // The 16-key quarters each lie inside one page (block sizes are
      // multiples of 32); rows at or past `hi` read as zero.
      __amdgpu_buffer_rsrc_t rk[2 * NSUB], rv[2 * NSUB];
#pragma unroll
      for (int qq = 0; qq < 2 * NSUB; ++qq) {
        const int jb = ti + 16 * qq;
        const int nv = min(16, hi - jb);
        int64_t ko = 0, vo = 0;
        uint32_t kbytes = 0, vbytes = 0;
        if (nv > 0) {
          ko = kv_row_offset_w(a, wp, a.k_sb, a.k_ss, a.k_sh, b, jb, kvh, kv_off);
          vo = kv_row_offset_w(a, wp, a.v_sb, a.v_ss, a.v_sh, b, jb, kvh, kv_off);
          kbytes = (uint32_t)((nv - 1) * a.k_ss + RB);
          vbytes = (uint32_t)((nv - 1) * a.v_ss + RB);
        }
        rk[qq] = make_rsrc(kbase + ko, kbytes);
        rv[qq] = make_rsrc(vbase + vo, vbytes);
      }
      // Key codes of the iteration's steps, whole rows, into this wave's
      // stage (the previous iteration's reads of it were consumed by its
      // products).
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub) {
#pragma unroll
        for (int inst = 0; inst < PR / 2; ++inst) {
          buf_ld16_lds_nt(rk[2 * sub + (RPI * inst) / 16], kst + 32 * RB * sub + 1024 * inst,
                          k_lds_off[inst]);
        }
      }
      // Value codes for step sub, head x, k-slot s: key 32 sub + 16 (s / 4) +
      // 4 g + s % 4, columns DPL n ..
      uint32_t vr[NSUB][NH][8][DPL / 4];
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub) {
#pragma unroll
        for (int x = 0; x < NH; ++x) {
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const int qq = 2 * sub + (s >> 2);
            const int t = 4 * g + (s & 3);
            const uint32_t off = (uint32_t)(t * a.v_ss + x * D + DPL * n);
            if constexpr (DPL == 8) {
              const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv[qq], off, 0, 2));
              vr[sub][x][s][0] = w.x;
              vr[sub][x][s][1] = w.y;
            } else {
              vr[sub][x][s][0] = __builtin_amdgcn_raw_buffer_load_b32(rv[qq], off, 0, 2);
            }
          }
        }
      }
      // Per-token scales / offsets of keys ti .. ti + 63: one 4-byte load per
      // key and table straight into the stage; keys past a table's width
      // read as zero (they lie past every visible key).
      if constexpr (KPT || VPT) {
        const uint32_t toff = (uint32_t)(ti + lane) * 4u;
        if constexpr (KPT) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r_ks, lds_ptr(tst), 4, toff, 0, 0, 0);
          if (kop != nullptr) __builtin_amdgcn_raw_ptr_buffer_load_lds(r_ko, lds_ptr(tst + 64), 4, toff, 0, 0, 0);
        }
        if constexpr (VPT) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r_vs, lds_ptr(tst + 128), 4, toff, 0, 0, 0);
          if (vop != nullptr) __builtin_amdgcn_raw_ptr_buffer_load_lds(r_vo, lds_ptr(tst + 192), 4, toff, 0, 0, 0);
        }
      }
      // The stage is complete once this wave's loads have landed (only this
      // wave reads its stage).
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub) {
        const int ts = ti + 32 * sub;
        if (ts >= t_hi) break;
        const uint8_t* ks_rows = kst + 32 * RB * sub;
        // Key operand pieces of head x, half hf (read where they are used).
        auto kwr = [&](int x, int hf, int c4) FIA_INLINE {
          return *reinterpret_cast<const u32x4*>(ks_rows + k_rd[x][hf][c4]);
        };
        // Tables of the lane's keys 16 hf + 4 g + r of this step.
        f32x4 ks[2], kq[2], vs[2], vq[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int j4 = 32 * sub + 16 * hf + 4 * g;
          ks[hf] = kq[hf] = vs[hf] = vq[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
          if constexpr (KPT) {
            ks[hf] = *reinterpret_cast<const f32x4*>(tst + j4);
            if (kop != nullptr) kq[hf] = *reinterpret_cast<const f32x4*>(tst + 64 + j4);
          }
          if constexpr (VPT) {
            vs[hf] = *reinterpret_cast<const f32x4*>(tst + 128 + j4);
            if (vop != nullptr) vq[hf] = *reinterpret_cast<const f32x4*>(tst + 192 + j4);
          }
        }

        // Scores S^T[key 16 hf + 4 g + r][column n]: one product per head of
        // the row against every column's query; a column keeps its own
        // head's.
        f32x4 sc[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          if constexpr (FP8) {
            f32x4 sx[NH];
#pragma unroll
            for (int x = 0; x < NH; ++x) {
              sx[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int cc = 0; cc < NC; ++cc) {
                // bytes 8 cc .. 8 cc + 7 of the lane's KB key bytes
                const u32x4 kp = kwr(x, hf, cc >> 1);
                const uint32_t w0 = kp[2 * (cc & 1)];
                const uint32_t w1 = kp[2 * (cc & 1) + 1];
                const u32x4 kop8 = codes8_bf16<true>(w0, w1);
                sx[x] = mfma16(kop8, qh[cc], sx[x]);
                if constexpr (!KPT) sx[x] = mfma16(kop8, ql[cc], sx[x]);
              }
            }
            sc[hf] = (NH == 2 && hs) ? sx[NH - 1] : sx[0];
          } else {
            // 16 key bytes per lane and product: the loaded pieces as they are.
            i32x4 ah[NH], al[NH];
#pragma unroll
            for (int x = 0; x < NH; ++x) {
              ah[x] = i32x4{0, 0, 0, 0};
              al[x] = i32x4{0, 0, 0, 0};
#pragma unroll
              for (int c4 = 0; c4 < KB / 16; ++c4) {
                const i32x4 kc = __builtin_bit_cast(i32x4, kwr(x, hf, c4));
                ah[x] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kc, __builtin_bit_cast(i32x4, qi[c4]), ah[x], 0, 0, 0);
                al[x] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kc, __builtin_bit_cast(i32x4, qj[c4]), al[x], 0, 0, 0);
              }
            }
            const i32x4 ahs = (NH == 2 && hs) ? ah[NH - 1] : ah[0];
            const i32x4 als = (NH == 2 && hs) ? al[NH - 1] : al[0];
#pragma unroll
            for (int r = 0; r < 4; ++r) sc[hf][r] = sq * __builtin_fmaf((float)als[r], 1.f / 256.f, (float)ahs[r]);
          }
        }
        float x[8];
        float mx = kNegInf;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int hf = s >> 2, r = s & 3;
          const int j = ts + 16 * hf + 4 * g + r;
          const bool ok = j >= t_lo && j < t_hi;
          float v;
          if constexpr (KPT) {
            v = ks[hf][r] * __builtin_fmaf(kq[hf][r], qc, sc[hf][r]) * a.scale_log2;
          } else {
            v = __builtin_fmaf(sc[hf][r], a.scale_log2, c_shift);
          }
          x[s] = ok ? v : kNegInf;
          mx = fmaxf(mx, x[s]);
        }
        mx = pair32_max(pair16_max(mx));
        // Lazy rescale: the running max moves only when a head's new max
        // exceeds it by more than 8 (probabilities stay <= 2^8).
        const bool grow = mx > m_run + 8.f;
        if (__any(grow)) {
          const float m_new = grow ? mx : m_run;
          const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
          t_run *= alpha;
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[e] *= alpha;
        }
        const float m_use = (m_run == kNegInf) ? 0.f : m_run;
        float p[8];
        float psum = 0.f, tsum = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          p[s] = fast_exp2(x[s] - m_use);
          psum += p[s];
        }
        if constexpr (VPT) {
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const float pv = p[s] * vs[s >> 2][s & 3];
            tsum = __builtin_fmaf(pv, vq[s >> 2][s & 3], tsum);
            p[s] = pv;
          }
        }
        l_run += psum;
        t_run += tsum;
        const u32x4 pb = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                          pack_bf16x2(p[6], p[7])};
        // Head x's values against the probabilities of its own columns only
        // (the other head's columns enter as zero), into the shared output.
#pragma unroll
        for (int x = 0; x < NH; ++x) {
          const u32x4 pbx = (NH == 1 || hs == x) ? pb : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
          for (int e = 0; e < DPL; ++e) {
            // byte e of the lane's DPL value bytes of each of the 8 keys
            const int w = e >> 2, k = e & 3;
            const uint32_t(&v8)[8][DPL / 4] = vr[sub][x];
            const u32x4 av = {pair_bf16<FP8>(v8[0][w], v8[1][w], k), pair_bf16<FP8>(v8[2][w], v8[3][w], k),
                              pair_bf16<FP8>(v8[4][w], v8[5][w], k), pair_bf16<FP8>(v8[6][w], v8[7][w], k)};
            o[e] = mfma16(av, pbx, o[e]);
          }
        }
      }
    }
  }
  l_run = pair32_sum(pair16_sum(l_run));
  t_run = pair32_sum(pair16_sum(t_run));

  // Combine the four waves through LDS in wave order (every wave is done
  // with its stage first).
  __shared__ float sm_m[4][16];
  __shared__ float sm_l[4][16];
  __shared__ float sm_t[4][16];
  __syncthreads();
  if (g == 0) {
    sm_m[wave][n] = m_run;
    sm_l[wave][n] = l_run;
    sm_t[wave][n] = t_run;
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
#pragma unroll
    for (int r = 0; r < 4; ++r) sm_o[wave][n][DPL * (4 * g + r) + e] = o[e][r];
  }
  __syncthreads();

  constexpr int PER = 16 * D / 256;  // outputs per thread
  const int hh = threadIdx.x / (D / PER);
  const int d0 = (threadIdx.x % (D / PER)) * PER;
  int hout, kvo;
  if constexpr (NH == 1) {
    if (hb * 16 + hh >= a.G) return;
    hout = kvh * a.G + hb * 16 + hh;
    kvo = kvh;
  } else {
    if (hh >= 2 * a.G) return;
    const int hso = hh >= a.G ? 1 : 0;
    kvo = kvh + hso;
    hout = kvo * a.G + hh - hso * a.G;
  }
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][hh]);
  float wgt[4];
  float L = 0.f, T = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wgt[w] = (sm_m[w][hh] == kNegInf) ? 0.f : fast_exp2(sm_m[w][hh] - M);
    L += sm_l[w][hh] * wgt[w];
    T += sm_t[w][hh] * wgt[w];
  }
  const bool any = L > 0.f;
  const float inv = any ? 1.f / L : 0.f;
  const float lse2 = any ? M + fast_log2(L) : kNegInf;
  float val[PER];
  // Value per channel: this thread's PER scales and offsets, requested
  // together.
  float vcs[VPT ? 1 : PER], vco[VPT ? 1 : PER];
  if constexpr (!VPT) {
    const int64_t cnt = a.vq_scalar ? 1 : (int64_t)a.KVn * D;
    chan_run(a.vq_scale, a.vq_f32, a.vq_scalar, cnt, kvo * D + d0, vcs);
    chan_run(a.vq_off, a.vq_f32, a.vq_scalar, cnt, kvo * D + d0, vco);
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) s += sm_o[w][hh][d0 + u] * wgt[w];
    if constexpr (VPT) {
      val[u] = (s + T) * inv;
    } else {
      val[u] = any ? vcs[u] * (s * inv + vco[u]) : 0.f;
    }
  }
  if (nchunk == 1) {
    uint16_t* op = (uint16_t*)a.o + (int64_t)b * a.o_sb + (int64_t)q_off * a.o_ss +
                   (int64_t)hout * a.o_sh + d0;
#pragma unroll
    for (int u = 0; u < PER; u += 2) {
      *reinterpret_cast<uint32_t*>(op + u) = pack_bf16x2(val[u], val[u + 1]);
    }
    if (a.write_lse && d0 == 0) {
      a.lse[(int64_t)b * a.lse_sb + (int64_t)hout * a.lse_sh + (int64_t)q_off * a.lse_ss] =
          any ? lse2 * kLn2 : kPosInf;
    }
  } else {
    const int64_t pi = (int64_t)(chunk0 + c) * a.Qn + hout;
    float* pp = a.part_o + pi * D + d0;
#pragma unroll
    for (int u = 0; u < PER; ++u) pp[u] = val[u];
    if (d0 == 0) a.part_lse[pi] = lse2;
  }
}

template <int D, bool FP8, int NH>
static void launch_q8_modes(const AttnArgs& a, int32_t n_items, hipStream_t s) {
  if (a.kq_mode == 1) {
    decode_split_q8<D, FP8, true, true, NH><<<n_items, 256, 0, s>>>(a);
  } else if (a.vq_mode == 1) {
    decode_split_q8<D, FP8, false, true, NH><<<n_items, 256, 0, s>>>(a);
  } else {
    decode_split_q8<D, FP8, false, false, NH><<<n_items, 256, 0, s>>>(a);
  }
}

hipError_t launch_decode_q8(const AttnArgs& a, int32_t n_items, hipStream_t s) {
  if (n_items > 0) {
    const bool fp8 = a.kvq == 2;
    if (a.D == 128 && a.kv_pair) {
      if (fp8) launch_q8_modes<128, true, 2>(a, n_items, s);
      else launch_q8_modes<128, false, 2>(a, n_items, s);
    } else if (a.D == 128) {
      if (fp8) launch_q8_modes<128, true, 1>(a, n_items, s);
      else launch_q8_modes<128, false, 1>(a, n_items, s);
    } else {
      if (fp8) launch_q8_modes<64, true, 1>(a, n_items, s);
      else launch_q8_modes<64, false, 1>(a, n_items, s);
    }
  }
  return hipGetLastError();
}

}  // namespace fia
