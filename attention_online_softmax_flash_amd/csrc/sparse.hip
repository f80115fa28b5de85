// Shared-KV sparse decode (KvQuantSparseAttnSharedkv; sparse_flash_mla CSA
// and HCA modes): O = softmax(Q K~^T * scale) V~ with K~ = V~ = the window rows of the
// original KV followed by the top-k selected rows of the compressed KV, plus a
// per-head sink logit.
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
// Each packed 640-byte row holds bf16 rope x64 | e4m3fn nope x448 | fp32
// scale x7 (one per 64-wide nope tile); the logical 512-vector is
// [rope | nope * scale].
//
// One workgroup takes 64 slots x 32 heads of one batch entry: it gathers the
// rows through the block tables, dequantises them into LDS once (row-major),
// runs both products on 32x32x16 bf16 MFMA (the value product reads its
// transposed operand with LDS transpose reads) and writes a normalised
// partial with its log2-sum-exp.  The merge kernel folds the chunks in slot order together with
// the sink: an extra logit sigma_h whose value vector is zero.
#include "fia_device.h"

namespace fia {

namespace {

constexpr int X_PITCH = kSparseD * 2 + 16;   // bytes per row-major row
constexpr int X_BYTES = kSparseChunk * X_PITCH;
constexpr int P_BYTES = 4 * 64 * 16;
constexpr int SX_BYTES = 2 * 64 * 16 * 4;
constexpr int LDS_TOTAL = X_BYTES + P_BYTES + SX_BYTES + 64 * 4 + 2 * 32 * 4 * 2;

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

// Slots s[0..N) of query row w -> packed row addresses (nullptr for an unused
// slot) and ids: j for window row j, (1 << 30) | c for compressed row c, -1
// if unused.  Compressed slot k holds row idx[b][k] (compressed-sparse) or
// row k itself (heavily compressed, no indices).  No read depends on a branch: every table read goes to an
// in-bounds address (a clamped position), so the N index reads, then the N
// block-table reads, are each in flight together.
template <int N>
__device__ __forceinline__ void sparse_slot_rows(const SparseArgs& a, const SparseRow& w, const int* s,
                                                 int Lk, const uint8_t** row, int32_t* id) {
  const int b = w.b;
  const int t = w.t;
  const int p = Lk - w.s1 + t;
  const int jmax = min(Lk - 1, p + a.win_right);
  const int n_cmp = Lk / a.cmp_ratio - (w.s1 - 1 - t);
  const bool cmp_on = a.has_cmp && a.K2 > 0;
  int c[N];
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int k = min(max(s[u] - a.n_win_slots, 0), a.K2 > 0 ? a.K2 - 1 : 0);
    if (a.cmp_direct) {
      c[u] = cmp_on ? s[u] - a.n_win_slots : -1;
    } else {
      c[u] = cmp_on ? a.idx[(int64_t)b * a.idx_sb + (int64_t)w.tq * a.idx_ss + k] : -1;
    }
  }
  int raw[N], slot[N];
  bool win[N], ok[N];
#pragma unroll
  for (int u = 0; u < N; ++u) {
    win[u] = s[u] < a.n_win_slots;
    const int j = p - a.win_left + s[u];
    const int k = s[u] - a.n_win_slots;
    const bool wok = s[u] <= a.win_left + a.win_right && j >= 0 && j <= jmax;
    const bool cok = cmp_on && k < a.K2 && c[u] >= 0 && c[u] < n_cmp;
    ok[u] = win[u] ? wok : cok;
    const int rr = ok[u] ? (win[u] ? j : c[u]) : 0;
    const int bs = win[u] ? a.bs1 : a.bs2;
    const int page = rr / bs;
    slot[u] = rr - page * bs;
    // Compressed slots read the compressed table only when there is one.
    const bool use_cmp = !win[u] && cmp_on;
    const int cols = use_cmp ? a.cmp_bt_cols : a.ori_bt_cols;
    const int32_t* bt = use_cmp ? a.cmp_bt + (int64_t)b * a.cmp_bt_sb : a.ori_bt + (int64_t)b * a.ori_bt_sb;
    raw[u] = bt[min(page, cols - 1)];
    id[u] = ok[u] ? (win[u] ? j : ((1 << 30) | c[u])) : -1;
  }
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const uint8_t* rp;
    if (win[u]) {
      rp = a.ori + (int64_t)clamp_block(raw[u], a.nb1) * a.ori_sb + (int64_t)slot[u] * a.ori_ss;
    } else {
      rp = a.cmp + (int64_t)clamp_block(raw[u], a.nb2) * a.cmp_sb + (int64_t)slot[u] * a.cmp_ss;
    }
    row[u] = ok[u] ? rp : nullptr;
  }
}

__device__ __forceinline__ int sparse_len(const SparseArgs& a, const SparseRow& w) {
  if (!w.live) return 0;
  int Lk = a.seqused[w.b];
  const int cap = a.ori_bt_cols * a.bs1;
  return Lk < 0 ? 0 : (Lk > cap ? cap : Lk);
}

// Grid: (n_slots / 64, N1 / 32, n_rows); 256 threads.
__global__ __launch_bounds__(256, 2) void sparse_chunk(SparseArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t* xs = lds;                         // [64][X_PITCH]
  u32x4* ps = reinterpret_cast<u32x4*>(xs + X_BYTES);        // [4][64]
  float* sx = reinterpret_cast<float*>(xs + X_BYTES + P_BYTES);  // [2][64][16]
  int32_t* ids = reinterpret_cast<int32_t*>(xs + X_BYTES + P_BYTES + SX_BYTES);  // [64]
  float* mx_s = reinterpret_cast<float*>(ids + 64);          // [2][32]
  float* l_s = mx_s + 64;                                    // [2][32]

  const int chunk = blockIdx.x;
  const int hb = blockIdx.y;
  const int r = blockIdx.z;   // query row
  const SparseRow qr = sparse_row(a, r);
  const int b = qr.b;
  const int n_chunks = gridDim.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);   // wave-uniform: scalar bookkeeping
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int Lk = sparse_len(a, qr);
  const int s0 = chunk * kSparseChunk;
  const int sb = wave & 1;
  const int dh = wave >> 1;
  const int head = hb * kSparseHeads + n;

  // Query operand for the score product, loaded first so its latency overlaps
  // the row gather: head n, d = 256 dh + 16 c + 8 hh .. +7.
  u32x4 qv[16];
  {
    const uint16_t* qp = a.q + (int64_t)b * a.q_sb + (int64_t)qr.tq * a.q_ss + (int64_t)head * a.q_sh +
                         256 * dh + 8 * hh;
#pragma unroll
    for (int c = 0; c < 16; ++c) qv[c] = ld16(qp + 16 * c);
  }

  // 1. Gather and dequantise: thread owns rows 4 rg .. 4 rg + 3 and the
  // 16-byte pieces pc = tid/16 + 16 q of their bf16 form (pieces 0..7 rope,
  // 8..63 nope: 8 fp8 codes and their tile scale).  Every load is issued
  // before the first conversion; unused slots read row 0 of the original KV
  // (in bounds) and are zeroed.
  {
    const int rg = tid & 15;
    const int pc0 = tid >> 4;
    const bool rope0 = pc0 < 8;   // wave-uniform: waves 0, 1
    int sl[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) sl[u] = s0 + 4 * rg + u;
    const uint8_t* rows[4];
    int32_t rid[4];
    sparse_slot_rows<4>(a, qr, sl, Lk, rows, rid);
    if (pc0 == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) ids[4 * rg + u] = rid[u];
    }
    u32x4 raw0[4];
    float sc0[4];
    u32x2 codes[3][4];
    float scl[3][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint8_t* rp = rows[u] != nullptr ? rows[u] : a.ori;
      if (rope0) {
        raw0[u] = ld16(rp + 16 * pc0);
        sc0[u] = 0.f;
      } else {
        const u32x2 cw = ld8(rp + 128 + 8 * (pc0 - 8));
        raw0[u] = u32x4{cw.x, cw.y, 0u, 0u};
        sc0[u] = *reinterpret_cast<const float*>(rp + 576 + 4 * ((pc0 - 8) >> 3));
      }
#pragma unroll
      for (int q = 1; q < 4; ++q) {
        const int np = pc0 + 16 * q - 8;
        codes[q - 1][u] = ld8(rp + 128 + 8 * np);
        scl[q - 1][u] = *reinterpret_cast<const float*>(rp + 576 + 4 * (np >> 3));
      }
    }
    auto dequant = [&](u32x2 cw, float sc) FIA_INLINE {
      float f[8];
      e4m3fn_x4(cw.x, f);
      e4m3fn_x4(cw.y, f + 4);
      return u32x4{pack_bf16x2(f[0] * sc, f[1] * sc), pack_bf16x2(f[2] * sc, f[3] * sc),
                   pack_bf16x2(f[4] * sc, f[5] * sc), pack_bf16x2(f[6] * sc, f[7] * sc)};
    };
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint8_t* xr = xs + (4 * rg + u) * X_PITCH;
      const bool live = rows[u] != nullptr;
      const u32x4 w0 = rope0 ? raw0[u] : dequant(u32x2{raw0[u].x, raw0[u].y}, sc0[u]);
      *reinterpret_cast<u32x4*>(xr + 16 * pc0) = live ? w0 : zero;
#pragma unroll
      for (int q = 1; q < 4; ++q) {
        const u32x4 w = dequant(codes[q - 1][u], scl[q - 1][u]);
        *reinterpret_cast<u32x4*>(xr + 16 * (pc0 + 16 * q)) = live ? w : zero;
      }
    }
  }
  __syncthreads();

  // 2. Scores S^T[slot][head]: wave (sb, dh) = slot block 32 sb, d half dh.
  f32x16 s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const u32x4 av = *reinterpret_cast<const u32x4*>(xs + (32 * sb + n) * X_PITCH +
                                                     (256 * dh + 16 * c + 8 * hh) * 2);
    s = mfma32(av, qv[c], s);
  }
  if (dh == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sx[(sb * 64 + lane) * 16 + r] = s[r];
  }
  __syncthreads();
  float m_loc = kNegInf;
  if (dh == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int slot = 32 * sb + 8 * (r >> 2) + 4 * hh + (r & 3);
      const float x = (s[r] + sx[(sb * 64 + lane) * 16 + r]) * a.scale_log2;
      s[r] = ids[slot] >= 0 ? x : kNegInf;
      m_loc = fmaxf(m_loc, s[r]);
    }
    m_loc = pair32_max(m_loc);
    if (hh == 0) mx_s[sb * 32 + n] = m_loc;
  }
  __syncthreads();
  const float m_all = fmaxf(mx_s[n], mx_s[32 + n]);
  const float m_use = (m_all == kNegInf) ? 0.f : m_all;
  if (dh == 0) {
    float l = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float p[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        p[t] = fast_exp2(s[8 * kk + t] - m_use);
        l += p[t];
      }
      ps[(2 * sb + kk) * 64 + lane] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                           pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
    }
    l = pair32_sum(l);
    if (hh == 0) l_s[sb * 32 + n] = l;
  }
  __syncthreads();

  // 3. O^T[d][head] for d in [128 wave, 128 wave + 128).  Lane (n, hh)
  // feeds k-step kk the slots 16 kk + 8 r + 4 hh + (0..3), r = 0, 1 (the
  // order of the score accumulators) of column d = n: in 16-lane group g,
  // lane j addresses slot 16 kk + 8 r + 4 (g / 2) + j / 4 at columns
  // 16 (g % 2) + 4 (j % 4) .. + 3 of the 32-wide d block.
  f32x16 o[4];
  {
    const int g16 = lane >> 4;
    const int j = lane & 15;
    const uint8_t* tb = xs + (4 * (g16 >> 1) + (j >> 2)) * X_PITCH +
                        (128 * wave + 16 * (g16 & 1) + 4 * (j & 3)) * 2;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint8_t* vp = tb + 16 * kk * X_PITCH + 64 * mb;
        const u32x2 lo2 = lds_tr16(vp);
        const u32x2 hi2 = lds_tr16(vp + 8 * X_PITCH);
        o[mb] = mfma32(u32x4{lo2.x, lo2.y, hi2.x, hi2.y}, ps[kk * 64 + lane], o[mb]);
      }
    }
  }
  const float l_tot = l_s[n] + l_s[32 + n];
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t pi = ((int64_t)r * n_chunks + chunk) * a.N1 + head;
  float* pp = a.part_o + pi * kSparseD + 128 * wave + 4 * hh;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      *reinterpret_cast<f32x4*>(pp + 32 * mb + 8 * q4) =
          f32x4{o[mb][4 * q4] * inv, o[mb][4 * q4 + 1] * inv, o[mb][4 * q4 + 2] * inv,
                o[mb][4 * q4 + 3] * inv};
    }
  }
  if (wave == 0 && hh == 0) a.part_lse[pi] = l_tot > 0.f ? m_use + fast_log2(l_tot) : kNegInf;
}

// One wave per (row, head): fold the chunks in slot order with the sink logit.
// Lanes read the chunk log2-sum-exps in parallel; the weighted sum runs over
// chunks in order.
__global__ __launch_bounds__(256) void sparse_merge(SparseArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.n_rows * a.N1) return;
  const int r = row / a.N1;   // query row
  const int h = row - r * a.N1;
  const SparseRow qr = sparse_row(a, r);
  const int n_chunks = a.n_slots / kSparseChunk;   // <= 64 (K2 <= 1024)
  const float sink = a.sinks[h] * kLog2e;
  const float lc = lane < n_chunks ? a.part_lse[((int64_t)r * n_chunks + lane) * a.N1 + h] : kNegInf;
  float M = fmaxf(lc, sink);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, shfl_xor_f(M, m));
  const float m_use = (M == kNegInf) ? 0.f : M;
  const float w = (lc == kNegInf) ? 0.f : fast_exp2(lc - m_use);
  float L = fast_exp2(sink - m_use);
  float acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = 0.f;
  int c = 0;
  for (; c + 2 <= n_chunks; c += 2) {
    const float w0 = __shfl(w, c, 64), w1 = __shfl(w, c + 1, 64);
    const f32x4* p0 = reinterpret_cast<const f32x4*>(
        a.part_o + (((int64_t)r * n_chunks + c) * a.N1 + h) * kSparseD + 8 * lane);
    const f32x4* p1 = reinterpret_cast<const f32x4*>(
        a.part_o + (((int64_t)r * n_chunks + c + 1) * a.N1 + h) * kSparseD + 8 * lane);
    const f32x4 x0 = p0[0], x1 = p0[1], y0 = p1[0], y1 = p1[1];
    L += w0;
    L += w1;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[u] += w0 * x0[u];
      acc[4 + u] += w0 * x1[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[u] += w1 * y0[u];
      acc[4 + u] += w1 * y1[u];
    }
  }
  for (; c < n_chunks; ++c) {
    const float w0 = __shfl(w, c, 64);
    const f32x4* p0 = reinterpret_cast<const f32x4*>(
        a.part_o + (((int64_t)r * n_chunks + c) * a.N1 + h) * kSparseD + 8 * lane);
    const f32x4 x0 = p0[0], x1 = p0[1];
    L += w0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[u] += w0 * x0[u];
      acc[4 + u] += w0 * x1[u];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* op = a.o + (int64_t)qr.b * a.o_sb + (int64_t)qr.tq * a.o_ss + (int64_t)h * a.o_sh + 8 * lane;
  st16(op, u32x4{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                 pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)});
}

hipError_t launch_sparse(const SparseArgs& a, hipStream_t s) {
  if (a.n_rows == 0) return hipSuccess;
  // Dynamic LDS above the default limit must be enabled for the kernel (on
  // the current device); the call is cheap, so it is made on every launch.
  const hipError_t attr = hipFuncSetAttribute(
      (const void*)sparse_chunk, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_TOTAL);
  if (attr != hipSuccess) return attr;
  dim3 grid(a.n_slots / kSparseChunk, a.N1 / kSparseHeads, a.n_rows);
  sparse_chunk<<<grid, 256, LDS_TOTAL, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_sparse_merge(const SparseArgs& a, hipStream_t s) {
  const int rows = a.n_rows * a.N1;
  if (rows > 0) sparse_merge<<<(rows + 3) / 4, 256, 0, s>>>(a);
  return hipGetLastError();
}

// Test support: slot ids and raw row bytes, through sparse_slot_rows.
__global__ __launch_bounds__(256) void debug_sparse_rows(SparseArgs a, int32_t* ids, uint8_t* rows) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.n_rows * a.n_slots;
  if (t >= total) return;
  const int r = (int)(t / a.n_slots);   // query row
  const int s = (int)(t % a.n_slots);
  int32_t id;
  const uint8_t* row;
  const SparseRow qr = sparse_row(a, r);
  sparse_slot_rows<1>(a, qr, &s, sparse_len(a, qr), &row, &id);
  ids[t] = id;
  uint32_t* dst = reinterpret_cast<uint32_t*>(rows + t * kRowBytes);
  for (int w = 0; w < kRowBytes / 4; ++w) {
    dst[w] = row ? reinterpret_cast<const uint32_t*>(row)[w] : 0u;
  }
}

hipError_t launch_debug_sparse_rows(const SparseArgs& a, int32_t* ids, uint8_t* rows,
                                    hipStream_t s) {
  const int64_t total = (int64_t)a.n_rows * a.n_slots;
  if (total > 0) debug_sparse_rows<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(a, ids, rows);
  return hipGetLastError();
}

}  // namespace fia
