// fp32 attention (full-precision inputs), the empty-input fill and the
// gather used by the bit-exact address tests.
#include "fia_device.h"

namespace fia {

// fp32 inputs: T = D/32 lanes cooperate on one query row; each holds 32
// elements of the row's query and output.  Keys / values are staged through
// LDS 32 rows at a time; the online softmax update runs per key in fp32.
// Handles every mask mode, ALiBi, TND and paged KV through the same row
// address function as the bf16 kernels.  Grid: (row tiles, Q_N, B).
template <int T>
__global__ __launch_bounds__(256) void attn_fp32(AttnArgs a) {
  constexpr int D = 32 * T;
  constexpr int RPW = 256 / T;
  constexpr int KT = 32;
  extern __shared__ __align__(16) uint8_t lds_raw[];
  float* ks = reinterpret_cast<float*>(lds_raw);
  float* vs = ks + KT * D;

  const int b = blockIdx.z;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int r = tid / T;
  const int part = tid % T;
  const int32_t* bm = a.meta + (int64_t)b * BF_COUNT;
  const int Lq = bm[BF_QLEN], Lk = bm[BF_KVLEN];
  const int q_off = bm[BF_QOFF], kv_off = bm[BF_KVOFF];
  const int write_rows = a.tnd ? Lq : a.Sq;
  const int i0 = blockIdx.x * RPW;
  if (i0 >= write_rows) return;
  const int i = i0 + r;
  const bool live = i < Lq;
  const int kvh = h / a.G;

  float q[32], o[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    q[e] = 0.f;
    o[e] = 0.f;
  }
  if (live) {
    const float* qp = (const float*)a.q + (int64_t)b * a.q_sb + (int64_t)(q_off + i) * a.q_ss +
                      (int64_t)h * a.q_sh + 32 * part;
#pragma unroll
    for (int e = 0; e < 32; ++e) q[e] = qp[e];
  }
  int lo = 0, hi = 0;
  if (live) visible_range(a, i, Lq, Lk, lo, hi);
  const int rows_end = min(i0 + RPW, Lq);
  int klo = 0, khi = 0;
  if (rows_end > i0) {
    int l0, h0, l1, h1;
    visible_range(a, i0, Lq, Lk, l0, h0);
    visible_range(a, rows_end - 1, Lq, Lk, l1, h1);
    klo = l0;
    khi = h1;
  }
  const float slope = a.slopes != nullptr ? a.slopes[h] * kLog2e : 0.f;
  // Explicit mask row (modes 0 / 1); rows i < Lq <= mask_rows when live.
  const uint8_t* mrow = a.mask != nullptr
                            ? a.mask + (int64_t)b * a.mask_sb + (int64_t)min(i, a.mask_rows - 1) * a.mask_ss
                            : nullptr;
  // Bias row (pse type 0), fp32 like the query.
  const float* prow = a.pse != nullptr ? (const float*)a.pse + (int64_t)b * a.pse_sb + (int64_t)h * a.pse_sh +
                                             (int64_t)min(i, a.pse_rows - 1) * a.pse_ss
                                       : nullptr;
  float m_run = kNegInf, l_run = 0.f;
  const float* kg = (const float*)a.k;
  const float* vg = (const float*)a.v;

  for (int j0 = (klo / KT) * KT; j0 < khi; j0 += KT) {
    __syncthreads();
    for (int u = tid; u < KT * D / 4; u += 256) {
      const int jj = u / (D / 4);
      const int c4 = u % (D / 4);
      const int j = j0 + jj;
      f32x4 kv4 = {0.f, 0.f, 0.f, 0.f}, vv4 = {0.f, 0.f, 0.f, 0.f};
      if (j < Lk) {
        kv4 = *reinterpret_cast<const f32x4*>(
            kg + kv_row_offset(a, a.k_sb, a.k_ss, a.k_sh, b, j, kvh, kv_off) + 4 * c4);
        vv4 = *reinterpret_cast<const f32x4*>(
            vg + kv_row_offset(a, a.v_sb, a.v_ss, a.v_sh, b, j, kvh, kv_off) + 4 * c4);
      }
      *reinterpret_cast<f32x4*>(ks + jj * D + 4 * c4) = kv4;
      *reinterpret_cast<f32x4*>(vs + jj * D + 4 * c4) = vv4;
    }
    __syncthreads();
    for (int jj = 0; jj < KT; ++jj) {
      const int j = j0 + jj;
      const float* kr = ks + jj * D + 32 * part;
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) dot = __builtin_fmaf(q[e], kr[e], dot);
#pragma unroll
      for (int msk = 1; msk < T; msk <<= 1) dot += __shfl_xor(dot, msk, 64);
      if (j < lo || j >= hi) continue;
      if (mrow != nullptr && mrow[j] != 0) continue;
      float x = dot * a.scale_log2 + slope * (float)(j - i + a.alibi_delta);
      if (prow != nullptr) x = __builtin_fmaf(prow[j], kLog2e, x);
      const float m_new = fmaxf(m_run, x);
      const float alpha = fast_exp2(m_run - m_new);
      const float p = fast_exp2(x - m_new);
      l_run = l_run * alpha + p;
      m_run = m_new;
      const float* vr = vs + jj * D + 32 * part;
#pragma unroll
      for (int e = 0; e < 32; ++e) o[e] = __builtin_fmaf(p, vr[e], o[e] * alpha);
    }
  }
  if (i >= write_rows) return;
  const bool has = live && l_run > 0.f;
  const float inv = has ? 1.f / l_run : 0.f;
  float* op = (float*)a.o + (int64_t)b * a.o_sb + (int64_t)(q_off + i) * a.o_ss +
              (int64_t)h * a.o_sh + 32 * part;
#pragma unroll
  for (int e = 0; e < 32; ++e) op[e] = o[e] * inv;
  if (a.write_lse && part == 0) {
    a.lse[(int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)(q_off + i) * a.lse_ss] =
        has ? (m_run + fast_log2(l_run)) * kLn2 : kPosInf;
  }
}

hipError_t launch_attn_fp32(const AttnArgs& a, hipStream_t s) {
  const int T = a.D / 32;
  const int rpw = 256 / T;
  if (a.B == 0 || a.Qn == 0 || a.Sq == 0) return hipSuccess;
  dim3 grid((a.Sq + rpw - 1) / rpw, a.Qn, a.B);
  const size_t lds = 2 * 32 * a.D * sizeof(float);
  switch (T) {
    case 1: attn_fp32<1><<<grid, 256, lds, s>>>(a); break;
    case 2: attn_fp32<2><<<grid, 256, lds, s>>>(a); break;
    case 4: attn_fp32<4><<<grid, 256, lds, s>>>(a); break;
    case 8: {
      const hipError_t attr = hipFuncSetAttribute(
          (const void*)attn_fp32<8>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (attr != hipSuccess) return attr;
      attn_fp32<8><<<grid, 256, lds, s>>>(a);
      break;
    }
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Empty input (no key at all): output rows 0, LSE +inf.  One thread per row.
__global__ __launch_bounds__(256) void fill_empty(AttnArgs a, int esz) {
  const int64_t rows = (int64_t)a.B * a.Sq * a.Qn;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= rows) return;
  const int h = (int)(t % a.Qn);
  const int64_t bi = t / a.Qn;
  const int i = (int)(bi % a.Sq);
  const int b = (int)(bi / a.Sq);
  int q_off = 0;
  if (a.tnd) {
    const int32_t* bm = a.meta + (int64_t)b * BF_COUNT;
    if (i >= bm[BF_QLEN]) return;
    q_off = bm[BF_QOFF];
  }
  uint8_t* op = (uint8_t*)a.o +
                ((int64_t)b * a.o_sb + (int64_t)(q_off + i) * a.o_ss + (int64_t)h * a.o_sh) * esz;
  for (int e = 0; e < a.D * esz; ++e) op[e] = 0;
  if (a.write_lse) {
    a.lse[(int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)(q_off + i) * a.lse_ss] = kPosInf;
  }
}

hipError_t launch_fill_empty(const AttnArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.Sq * a.Qn;
  if (rows > 0) {
    fill_empty<<<(unsigned)((rows + 255) / 256), 256, 0, s>>>(a, a.esz);
  }
  return hipGetLastError();
}

// Test support: copy key (which = 0) or value rows j < Lk of every batch into
// dst [B, s2max, KV_N, D] through kv_row_offset, the function the prefill,
// decode and fp32 kernels address rows with.  One thread per 4-byte word.
__global__ __launch_bounds__(256) void debug_gather(AttnArgs a, int which, uint8_t* dst,
                                                    int s2max, int esz) {
  const int words = a.D * esz / 4;
  const int64_t total = (int64_t)a.B * s2max * a.KVn * words;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const int w = (int)(t % words);
  int64_t rest = t / words;
  const int g = (int)(rest % a.KVn);
  rest /= a.KVn;
  const int j = (int)(rest % s2max);
  const int b = (int)(rest / s2max);
  const int32_t* bm = a.meta + (int64_t)b * BF_COUNT;
  if (j >= bm[BF_KVLEN]) return;
  const int64_t off = which == 0
                          ? kv_row_offset(a, a.k_sb, a.k_ss, a.k_sh, b, j, g, bm[BF_KVOFF])
                          : kv_row_offset(a, a.v_sb, a.v_ss, a.v_sh, b, j, g, bm[BF_KVOFF]);
  const uint8_t* src = (const uint8_t*)(which == 0 ? a.k : a.v) + off * esz;
  reinterpret_cast<uint32_t*>(dst + (((int64_t)b * s2max + j) * a.KVn + g) * a.D * esz)[w] =
      reinterpret_cast<const uint32_t*>(src)[w];
}

hipError_t launch_debug_gather(const AttnArgs& a, int32_t which, void* dst, int32_t s2max,
                               hipStream_t s) {
  const int esz = a.kvq ? 1 : a.esz;   // bytes per key / value element (1: fake-quant codes)
  const int64_t total = (int64_t)a.B * s2max * a.KVn * (a.D * esz / 4);
  if (total > 0) {
    debug_gather<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(a, which, (uint8_t*)dst, s2max, esz);
  }
  return hipGetLastError();
}

// Read-only pass over a split-KV decode plan's key / value rows, the
// measured ceiling of its access pattern: every visible key and value row of
// every chunk is loaded once (16-byte non-temporal loads through per-run
// buffer resources, 8 KB of keys and 8 KB of values per wave and step, all in
// flight before one wait) and folded by XOR; nothing else.
//   ORDER 0: a workgroup per (chunk, KV head), its waves over quarters of
//     the chunk, SPAN = D * esz bytes per key and request: the order the
//     decode kernels read in.
//   ORDER 1: a workgroup per (chunk, eighth of it), its waves over 32 keys,
//     SPAN = KV_N * D * esz contiguous bytes of a token row per request
//     (pools whose heads of one token are adjacent: PA_ND, BSND).
// out[blockIdx.x] receives the workgroup's XOR of every 32-bit word read.
template <int ORDER, int SPAN>
__global__ __launch_bounds__(256) void decode_read(AttnArgs a, uint32_t* out) {
  constexpr int KS = 8192 / SPAN;   // keys per step (64, 32, 8 or 4)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int parts = ORDER == 0 ? a.KVn : 8;
  const int cg = blockIdx.x / parts;
  const int part = blockIdx.x - cg * parts;
  const int b = a.work[2 * cg], c = a.work[2 * cg + 1];
  const int32_t* bm = a.meta + (int64_t)b * BF_COUNT;
  const int lo = bm[BF_LO], hi = bm[BF_HI], kv_off = bm[BF_KVOFF];
  const int C = a.chunk;
  const int cbase = (lo / C + c) * C;
  const int wlen = ORDER == 0 ? C / 4 : C / 32;
  const int ws = ORDER == 0 ? cbase + wave * wlen : cbase + (4 * part + wave) * wlen;
  const int t_lo = max(ws, lo), t_hi = min(ws + wlen, hi);
  const int kvh = ORDER == 0 ? part : 0;
  const int esz = a.kvq ? 1 : a.esz;   // bytes per key / value element
  const uint8_t* kb = (const uint8_t*)a.k;
  const uint8_t* vb = (const uint8_t*)a.v;
  u32x4 acc = {0u, 0u, 0u, 0u};
  if (t_hi > t_lo) {
    const int first = ws + ((t_lo - ws) & ~(KS - 1));
    const WavePages wp = wave_pages(a, b, first, hi - 1, lane);
    for (int ti = first; ti < t_hi; ti += KS) {
      // The step's keys in 16-key runs (each inside one page); keys at or
      // past t_hi lie outside a run's resources and read as zero.
      constexpr int NR = KS > 16 ? KS / 16 : 1;
      constexpr int RK = KS > 16 ? 16 : KS;   // keys per run
      __amdgpu_buffer_rsrc_t rk[NR], rv[NR];
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        const int jb = ti + RK * q;
        const int nv = min(RK, t_hi - jb);
        int64_t ko = 0, vo = 0;
        uint32_t kbytes = 0, vbytes = 0;
        if (nv > 0) {
          ko = kv_row_offset_w(a, wp, a.k_sb, a.k_ss, a.k_sh, b, jb, kvh, kv_off) * esz;
          vo = kv_row_offset_w(a, wp, a.v_sb, a.v_ss, a.v_sh, b, jb, kvh, kv_off) * esz;
          kbytes = (uint32_t)((int64_t)(nv - 1) * a.k_ss * esz + SPAN);
          vbytes = (uint32_t)((int64_t)(nv - 1) * a.v_ss * esz + SPAN);
        }
        rk[q] = make_rsrc(kb + ko, kbytes);
        rv[q] = make_rsrc(vb + vo, vbytes);
      }
      // Load i, lane l: byte 1024 i + 16 l of the step's KS x SPAN bytes.
      u32x4 v[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int byte = 1024 * i + 16 * lane;
        const int kk = byte / SPAN;            // key within the step
        const int q = (1024 * i / SPAN) / RK;  // its run (the same for every lane)
        const int kr = kk - RK * q;            // key within the run
        const int pc = byte - kk * SPAN;
        v[2 * i] = buf_ld16_nt(rk[q], (uint32_t)((int64_t)kr * a.k_ss * esz + pc));
        v[2 * i + 1] = buf_ld16_nt(rv[q], (uint32_t)((int64_t)kr * a.v_ss * esz + pc));
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) acc ^= v[i];
    }
  }
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m, 64);
  __shared__ uint32_t red[4];
  if (lane == 0) red[wave] = x;
  __syncthreads();
  if (tid == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

hipError_t launch_decode_read(const AttnArgs& a, int32_t order, uint32_t* out, hipStream_t s) {
  const int64_t grid = decode_read_grid(a, order);
  if (grid <= 0) return hipSuccess;
  const int64_t row = (int64_t)a.D * (a.kvq ? 1 : a.esz);
  const unsigned g = (unsigned)grid;
  if (order == 0) {
    if (row == 128) decode_read<0, 128><<<g, 256, 0, s>>>(a, out);
    else decode_read<0, 256><<<g, 256, 0, s>>>(a, out);
  } else {
    if (row * a.KVn == 1024) decode_read<1, 1024><<<g, 256, 0, s>>>(a, out);
    else decode_read<1, 2048><<<g, 256, 0, s>>>(a, out);
  }
  return hipGetLastError();
}

}  // namespace fia
