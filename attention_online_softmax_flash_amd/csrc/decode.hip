// Incremental-decode branch (query length 1): split-KV attention over a
// dense, TND or paged KV cache, and the second-pass LSE merge.
//
// Work item = (batch b, KV head, block of up to 16 query heads of that KV
// head's group, chunk of `chunk` keys).  Chunk boundaries sit at multiples of
// `chunk` in absolute key position, so how a row is split depends only on that
// row's own visible range: the result of one batch entry never depends on the
// rest of the batch.  Four waves split the chunk in four equal key ranges,
// combine through LDS in a fixed order and either write the final row (the
// row has one chunk) or a partial (normalised output + log2-sum-exp) that the
// merge kernel folds in chunk order (aclnnFusedInferAttentionScoreV2,
// softmaxLse restrictions: partials compose through their max / sum / LSE).
//
// Per 32-key wave step, the 16x16x32 bf16 MFMA computes S^T[key][head] with
// keys on the M axis (lane n reads 16-byte pieces of key row n) and heads on
// the N axis, so lane (n, g) owns query head n: the running max / sum of the
// online softmax stay in that lane.  The value product is O^T = V^T P^T; each
// lane loads 16 bytes of 8 value rows and re-packs them in registers into the
// MFMA operand (d = 8n + e for product e), so no LDS transpose is needed.
#include "fia_device.h"

namespace fia {

// EXT: an explicit mask tensor (modes 0 / 1) removes keys whose mask byte
// (query row 0 of the batch) is non-zero; a bias tensor (pse type 0) adds
// row 0 of the head's bias to the scaled scores.
template <int D, bool EXT>
__global__ __launch_bounds__(256, 4) void decode_split_bf16(AttnArgs a) {
  constexpr int NC = D / 32;   // 32-wide d chunks of the score product
  constexpr int DPL = D / 16;  // value columns per lane column (8 for D = 128)
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);   // wave-uniform: scalar bookkeeping
  const int n = lane & 15;
  const int g = lane >> 4;

  int item = blockIdx.x;
  const int hb = item % a.n_head_blocks;
  item /= a.n_head_blocks;
  const int kvh = item % a.KVn;
  const int cg = item / a.KVn;
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

  const int hl = hb * 16 + n;
  const bool hvalid = hl < a.G;
  const int h = kvh * a.G + (hvalid ? hl : 0);

  const uint16_t* qp = (const uint16_t*)a.q + (int64_t)b * a.q_sb + (int64_t)q_off * a.q_ss +
                       (int64_t)h * a.q_sh;
  u32x4 qv[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    qv[cc] = hvalid ? ld16(qp + 32 * cc + 8 * g) : u32x4{0, 0, 0, 0};
  }
  const float c_alibi = (a.slopes != nullptr && hvalid) ? a.slopes[h] * kLog2e : 0.f;

  float m_run = kNegInf;
  float l_run = 0.f;
  f32x4 o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Each wave stages its 32-key step of K in its own slice of the combine
  // buffer (free until the loop ends).  The XOR swizzle makes the operand
  // reads (16 rows, one piece each) hit 16 distinct 16-byte bank groups.
  constexpr int PR = D / 8;       // 16-byte pieces per key row
  constexpr int RPI = 64 / PR;    // key rows per 64-lane load
  constexpr int NDMA = 32 / RPI;  // loads per 32-key step
  __shared__ __attribute__((aligned(16))) float sm_o[4][16][D + 4];
  static_assert(sizeof(sm_o[0]) >= 32 * 2 * D, "key slot does not fit");
  char* kbuf = reinterpret_cast<char*>(&sm_o[wave][0][0]);

  const bool has_mask = EXT && a.mask != nullptr;
  const bool has_pse = EXT && a.pse != nullptr;
  const uint8_t* mrow = has_mask ? a.mask + (int64_t)b * a.mask_sb : nullptr;
  const uint16_t* prow = has_pse ? (const uint16_t*)a.pse + (int64_t)b * a.pse_sb + (int64_t)h * a.pse_sh
                                 : nullptr;
  const uint16_t* kbase = (const uint16_t*)a.k;
  const uint16_t* vbase = (const uint16_t*)a.v;

  if (t_hi > t_lo) {
    const int first = ws + ((t_lo - ws) & ~31);
    const WavePages wp = wave_pages(a, b, first, hi - 1, lane);
    for (int ts = first; ts < t_hi; ts += kDecodeStep) {
      // The two 16-key halves each lie inside one page (block sizes are
      // multiples of 16 and halves are 16-aligned): one bounds-checked
      // resource per half and operand; rows at or past `hi` (possibly the
      // unwritten tail of the last page) read as zero.
      __amdgpu_buffer_rsrc_t rk[2], rv[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int jb = ts + 16 * hf;
        const int nv = min(16, hi - jb);
        int64_t ko = 0, vo = 0;
        uint32_t kbytes = 0, vbytes = 0;
        if (nv > 0) {
          ko = kv_row_offset_w(a, wp, a.k_sb, a.k_ss, a.k_sh, b, jb, kvh, kv_off);
          vo = kv_row_offset_w(a, wp, a.v_sb, a.v_ss, a.v_sh, b, jb, kvh, kv_off);
          kbytes = (uint32_t)((nv - 1) * a.k_ss + D) * 2u;
          vbytes = (uint32_t)((nv - 1) * a.v_ss + D) * 2u;
        }
        rk[hf] = make_rsrc(kbase + ko, kbytes);
        rv[hf] = make_rsrc(vbase + vo, vbytes);
      }
      // The 32 key rows go to the wave's LDS slot, whole rows per load
      // (RPI rows of 16 * PR bytes), piece q of row r stored at q ^ key_swz<PR>(r).
#pragma unroll
      for (int i = 0; i < NDMA; ++i) {
        const int r = RPI * i + lane / PR;
        const int gp = (lane % PR) ^ key_swz<PR>(r);
        buf_ld16_lds_nt(rk[(RPI * i) >> 4], kbuf + 1024 * i,
                        (uint32_t)((r & 15) * a.k_ss + 8 * gp) * 2u);
      }
      // Value rows for k-slot s: key 16 (s/4) + 4 g + s%4, columns DPL n ..
      u32x4 vr[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int hf = s >> 2;
        const int t = 4 * g + (s & 3);
        const uint32_t off = (uint32_t)(t * a.v_ss + DPL * n) * 2u;
        if constexpr (DPL == 8) {
          vr[s] = buf_ld16_nt(rv[hf], off);
        } else {
          const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv[hf], off, 0, 2));
          vr[s] = u32x4{w.x, w.y, 0, 0};
        }
      }
      // Every load of the step is in flight before the first staged-key read,
      // so one wait (the value loads still outstanding) covers the key rows.
      __builtin_amdgcn_sched_barrier(0);
      // Scores S^T[key 16 hf + 4 g + r][head n]; key operand: row 16 hf + n,
      // d = 32 cc + 8 g .. +7 (piece 4 cc + g).
      f32x4 sc[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        sc[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int r = 16 * hf + n;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          const u32x4 kr = *reinterpret_cast<const u32x4*>(kbuf + 16 * PR * r +
                                                           16 * ((4 * cc + g) ^ key_swz<PR>(r)));
          sc[hf] = mfma16(kr, qv[cc], sc[hf]);
        }
      }
      // Mask bytes and bias values of keys ts + 16 hf + 4 g .. + 3
      // (4-aligned; a group past the tensor's width lies past every visible
      // key, so its address is clamped and its values unused).
      uint32_t mw[2] = {0u, 0u};
      u32x2 pw[2] = {u32x2{0u, 0u}, u32x2{0u, 0u}};
      if constexpr (EXT) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int j = ts + 16 * hf + 4 * g;
          if (has_mask) mw[hf] = *reinterpret_cast<const uint32_t*>(mrow + min(j, a.mask_cols - 4));
          if (has_pse) pw[hf] = *reinterpret_cast<const u32x2*>(prow + min(j, a.pse_cols - 4));
        }
      }
      float x[8];
      float mx = kNegInf;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int j = ts + 16 * (s >> 2) + 4 * g + (s & 3);
        bool ok = j >= t_lo && j < t_hi;
        if constexpr (EXT) ok = ok && ((mw[s >> 2] >> (8 * (s & 3))) & 0xffu) == 0u;
        float v = sc[s >> 2][s & 3] * a.scale_log2;
        v += c_alibi * (float)(j + a.alibi_delta);
        if constexpr (EXT) {
          const uint32_t pv = pw[s >> 2][(s >> 1) & 1];
          v = __builtin_fmaf(__builtin_bit_cast(float, (s & 1) ? (pv & 0xffff0000u) : (pv << 16)), kLog2e, v);
        }
        x[s] = ok ? v : kNegInf;
        mx = fmaxf(mx, x[s]);
      }
      mx = pair32_max(pair16_max(mx));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float p[8];
      float psum = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        p[s] = fast_exp2(x[s] - m_use);
        psum += p[s];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      u32x4 pb = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                  pack_bf16x2(p[6], p[7])};
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        o[e] *= alpha;
        const int w = e >> 1;
        u32x4 av;
        if (e & 1) {
          av = u32x4{pick_hi(vr[0][w], vr[1][w]), pick_hi(vr[2][w], vr[3][w]),
                     pick_hi(vr[4][w], vr[5][w]), pick_hi(vr[6][w], vr[7][w])};
        } else {
          av = u32x4{pick_lo(vr[0][w], vr[1][w]), pick_lo(vr[2][w], vr[3][w]),
                     pick_lo(vr[4][w], vr[5][w]), pick_lo(vr[6][w], vr[7][w])};
        }
        o[e] = mfma16(av, pb, o[e]);
      }
    }
  }
  l_run = pair32_sum(pair16_sum(l_run));

  // Combine the four waves through LDS in wave order.
  __shared__ float sm_m[4][16];
  __shared__ float sm_l[4][16];
  if (g == 0) {
    sm_m[wave][n] = m_run;
    sm_l[wave][n] = l_run;
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
  if (hb * 16 + hh >= a.G) return;
  const int hout = kvh * a.G + hb * 16 + hh;
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][hh]);
  float wgt[4];
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wgt[w] = (sm_m[w][hh] == kNegInf) ? 0.f : fast_exp2(sm_m[w][hh] - M);
    L += sm_l[w][hh] * wgt[w];
  }
  float acc[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) s += sm_o[w][hh][d0 + u] * wgt[w];
    acc[u] = s;
  }
  // A chunk can hold no visible key under an explicit mask: output 0 and a
  // log2-sum-exp of -inf (the row's LSE +inf when it is the only chunk).
  bool any = L > 0.f;
  float inv = any ? 1.f / L : 0.f;
  float lse2 = any ? M + fast_log2(L) : kNegInf;
  if (nchunk == 1 && a.sink != nullptr) {
    // The sink: one more softmax term with a zero value vector.
    const float z = bf16_to_f32(a.sink[hout]) * kLog2e;
    const float m_new = fmaxf(M, z);
    const float w = any ? fast_exp2(M - m_new) : 0.f;
    const float Ls = L * w + fast_exp2(z - m_new);
    inv = w / Ls;
    lse2 = m_new + fast_log2(Ls);
    any = true;
  }
  if (nchunk == 1) {
    uint16_t* op = (uint16_t*)a.o + (int64_t)b * a.o_sb + (int64_t)q_off * a.o_ss +
                   (int64_t)hout * a.o_sh + d0;
#pragma unroll
    for (int u = 0; u < PER; u += 2) {
      *reinterpret_cast<uint32_t*>(op + u) = pack_bf16x2(acc[u] * inv, acc[u + 1] * inv);
    }
    if (a.write_lse && d0 == 0) {
      a.lse[(int64_t)b * a.lse_sb + (int64_t)hout * a.lse_sh + (int64_t)q_off * a.lse_ss] =
          any ? lse2 * kLn2 : kPosInf;
    }
  } else {
    const int64_t pi = (int64_t)(chunk0 + c) * a.Qn + hout;
    float* pp = a.part_o + pi * D + d0;
#pragma unroll
    for (int u = 0; u < PER; ++u) pp[u] = acc[u] * inv;
    if (d0 == 0) a.part_lse[pi] = lse2;
  }
}

// One wave per output row (b, h): fold the row's partials in chunk order, or
// write the empty-row result (0, LSE +inf) when the row has no visible key.
// Lanes read the chunk LSEs in parallel (64 at a time); the weighted sum then
// runs over chunks in order with every load independent of the others.
template <int D>
__global__ __launch_bounds__(256) void decode_merge(AttnArgs a) {
  constexpr int PL = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + uniform(threadIdx.x >> 6);   // one row per wave
  if (row >= a.B * a.Qn) return;
  const int b = row / a.Qn;
  const int h = row - b * a.Qn;
  // The batch record, read whole (one scalar load).
  const int32_t* bm = a.meta + (int64_t)b * BF_COUNT;
  int32_t rec[BF_COUNT];
#pragma unroll
  for (int f = 0; f < BF_COUNT; ++f) rec[f] = bm[f];
  const int nchunk = rec[BF_NCHUNK];
  if (nchunk == 1) return;
  // A TND batch entry without a query token owns no output row (its offset
  // is the next entry's first row): nothing to write.
  if (a.tnd && rec[BF_QLEN] == 0) return;
  const int q_off = rec[BF_QOFF];
  uint16_t* op = (uint16_t*)a.o + (int64_t)b * a.o_sb + (int64_t)q_off * a.o_ss +
                 (int64_t)h * a.o_sh + lane * PL;
  float* lp = a.lse + (int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)q_off * a.lse_ss;
  // Learnable sink (log2 units): one more term with a zero value vector.
  // Loaded through a buffer resource (reads zero without a sink), so no
  // branch holds the chunk loads below behind it.
  const __amdgpu_buffer_rsrc_t r_sink =
      make_rsrc(a.sink, a.sink != nullptr ? (uint32_t)a.Qn * 2u : 0u);
  const float z = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r_sink, (uint32_t)h * 2u, 0, 0)) * kLog2e;
  // A row with no chunk (no visible key) takes the same path: the fold
  // leaves M = -inf and L = 0, and the end writes 0 with LSE +inf (or the
  // sink's).
  const int chunk0 = rec[BF_CHUNK0];
  // Chunks are folded in fixed order, in groups of G: every log-sum-exp and
  // partial of a group is requested before the first is used (addresses
  // clamped to the last chunk, so the loads are unconditional and nothing
  // branches before they are used), with a running-maximum rescale.
  constexpr int G = 8;
  float M = kNegInf;
  float L = 0.f;
  float acc[PL];
#pragma unroll
  for (int u = 0; u < PL; ++u) acc[u] = 0.f;
  for (int c0 = 0; c0 < nchunk; c0 += G) {
    // Lane i < G loads the log-sum-exp of chunk c0 + i (a vector load: the
    // address is wave-uniform per chunk, and scalar loads would each be
    // waited for on their own); every lane loads its d values of all G.
    const float lvl = a.part_lse[((int64_t)chunk0 + min(c0 + (lane & (G - 1)), nchunk - 1)) * a.Qn + h];
    float x[G][PL];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int64_t pc = (int64_t)chunk0 + min(c0 + i, nchunk - 1);
      const float* pp = a.part_o + (pc * a.Qn + h) * D + lane * PL;
#pragma unroll
      for (int u = 0; u < PL; ++u) x[i][u] = pp[u];
    }
    float lv[G];
    float gm = M;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      lv[i] = (c0 + i < nchunk) ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lvl), i))
                                : kNegInf;
      gm = fmaxf(gm, lv[i]);
    }
    const float gmu = (gm == kNegInf) ? 0.f : gm;
    const float sc = (M == kNegInf) ? 0.f : fast_exp2(M - gmu);
    L *= sc;
#pragma unroll
    for (int u = 0; u < PL; ++u) acc[u] *= sc;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float wc = (lv[i] == kNegInf) ? 0.f : fast_exp2(lv[i] - gmu);
      L += wc;
#pragma unroll
      for (int u = 0; u < PL; ++u) acc[u] = __builtin_fmaf(wc, x[i][u], acc[u]);
    }
    M = gm;
  }
  if (a.sink != nullptr) {
    // every chunk empty: output 0, LSE the sink's
    const float mf = fmaxf(M, z);
    const float sc = (M == kNegInf) ? 0.f : fast_exp2(M - mf);
    L = L * sc + fast_exp2(z - mf);
#pragma unroll
    for (int u = 0; u < PL; ++u) acc[u] *= sc;
    M = mf;
  }
  // every chunk empty and no sink: output 0, LSE +inf
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if constexpr (PL == 2) {
    *reinterpret_cast<uint32_t*>(op) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  } else {
#pragma unroll
    for (int u = 0; u < PL; ++u) {
      op[u] = (uint16_t)(pack_bf16x2(acc[u] * inv, 0.f) & 0xffffu);
    }
  }
  if (a.write_lse && lane == 0) *lp = L > 0.f ? (M + fast_log2(L)) * kLn2 : kPosInf;
}

hipError_t launch_decode_bf16(const AttnArgs& a, int32_t n_items, hipStream_t s) {
  if (n_items > 0) {
    const bool m = a.mask != nullptr || a.pse != nullptr;
    if (a.D == 128) {
      if (m) decode_split_bf16<128, true><<<n_items, 256, 0, s>>>(a);
      else decode_split_bf16<128, false><<<n_items, 256, 0, s>>>(a);
    } else {
      if (m) decode_split_bf16<64, true><<<n_items, 256, 0, s>>>(a);
      else decode_split_bf16<64, false><<<n_items, 256, 0, s>>>(a);
    }
  }
  return hipGetLastError();
}

// Device-side partitioner (the device counterpart of the host planner's
// decode branch, for KV lengths that live on the device): one workgroup
// walks the batch entries 1024 at a time.  Entry b gets Lk = its length
// clamped into [0, kvlen_bound], its visible range for query row 0 (the same
// rule as the kernels), nch = the 0-aligned chunks that range touches, and
// its first chunk index from an exclusive prefix sum of nch in batch order;
// the chunk list holds (b, c) for c < nch in that order, and the total goes
// to meta[B * BF_COUNT].  The result is the plan the host would build for
// the same lengths, so results are bitwise the same.
__global__ __launch_bounds__(1024) void decode_partition(AttnArgs a, int32_t* meta, int32_t* work) {
  __shared__ int32_t scan[1024];
  const int tid = threadIdx.x;
  int carry = 0;
  for (int base = 0; base < a.B; base += 1024) {
    const int b = base + tid;
    int Lk = 0, lo = 0, hi = 0, nch = 0;
    if (b < a.B) {
      Lk = a.dev_kvlen[b];
      Lk = Lk < 0 ? 0 : (Lk > a.kvlen_bound ? a.kvlen_bound : Lk);
      visible_range(a, 0, 1, Lk, lo, hi);
      nch = hi > lo ? (hi + a.chunk - 1) / a.chunk - lo / a.chunk : 0;
    }
    scan[tid] = nch;
    __syncthreads();
    // inclusive scan over the 1024 entries of this round
    for (int off = 1; off < 1024; off <<= 1) {
      const int add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const int first = carry + scan[tid] - nch;
    if (b < a.B) {
      int32_t* r = meta + (int64_t)b * BF_COUNT;
      r[BF_QLEN] = 1;
      r[BF_KVLEN] = Lk;
      r[BF_QOFF] = 0;
      r[BF_KVOFF] = 0;
      r[BF_LO] = lo;
      r[BF_HI] = hi;
      r[BF_NCHUNK] = nch;
      r[BF_CHUNK0] = first;
      for (int c = 0; c < nch; ++c) {
        work[2 * (first + c)] = b;
        work[2 * (first + c) + 1] = c;
      }
    }
    carry += scan[1023];
    __syncthreads();
  }
  if (tid == 0) meta[(int64_t)a.B * BF_COUNT] = carry;
}

hipError_t launch_decode_partition(const AttnArgs& a, int32_t* meta, int32_t* work, hipStream_t s) {
  if (a.B > 0) decode_partition<<<1, 1024, 0, s>>>(a, meta, work);
  return hipGetLastError();
}

hipError_t launch_decode_merge(const AttnArgs& a, hipStream_t s) {
  const int rows = a.B * a.Qn;
  if (rows > 0) {
    if (a.D == 128) {
      decode_merge<128><<<(rows + 3) / 4, 256, 0, s>>>(a);
    } else {
      decode_merge<64><<<(rows + 3) / 4, 256, 0, s>>>(a);
    }
  }
  return hipGetLastError();
}

}  // namespace fia
