// Device helpers shared by the gfx950 kernels: vector types, MFMA wrappers,
// key/value row addressing and small wave-level utilities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fia_internal.h"

// Helper lambdas inside kernels are force-inlined: their captures then stay
// in registers instead of going through private memory.
#define FIA_INLINE __attribute__((always_inline))

namespace fia {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_inff();

// D(32x32) += A(32x16) * B(16x32), bf16 in, fp32 accumulate.
// Lane l supplies A[l%32][8(l/32)+0..7] and B[8(l/32)+0..7][l%32]; it holds
// C[8(r/4) + 4(l/32) + r%4][l%32] in accumulator slot r.
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D(16x16) += A(16x32) * B(32x16).  Lane l supplies A[l%16][8(l/16)+0..7] and
// B[8(l/16)+0..7][l%16]; it holds C[4(l/16) + r][l%16] in slot r.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __builtin_bit_cast(float, (uint32_t)u << 16);
}

// Two floats -> packed bf16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Select the low (sel = 0) or high (sel = 1) bf16 halves of two words into one
// packed pair {a.half, b.half}.
__device__ __forceinline__ uint32_t pick_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pick_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Max / sum over lane pairs (l, l ^ 32) and (l, l ^ 16) by register lane swaps
// (v_permlane32_swap / v_permlane16_swap) instead of an LDS permute: with the
// same value in both operands, lane l ends up with its own value in one result
// and its partner's in the other.
__device__ __forceinline__ float pair32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv& f) {
  return (uint32_t)(((uint64_t)n * f.mul) >> (32 + f.shift));
}

__device__ __forceinline__ int32_t uniform(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// Base of the contiguous head-dim vector of key (or value) row j of batch b,
// KV head g.  Dense / TND rows are addressed with batch, token and head
// strides; paged rows through block_table[b][j / block_size], with the block
// id clamped into [0, n_blocks).  Returns an element offset.
__device__ __forceinline__ int64_t kv_row_offset(const AttnArgs& a, int64_t sb, int64_t ss,
                                                 int64_t sh, int b, int j, int g, int kv_off) {
  if (a.paged) {
    uint32_t page = fast_div((uint32_t)j, a.bs_div);
    int slot = j - (int)page * a.block_size;
    int blk = a.block_table[(int64_t)b * a.bt_sb + page];
    blk = blk < 0 ? 0 : (blk >= a.n_blocks ? a.n_blocks - 1 : blk);
    return (int64_t)blk * sb + (int64_t)slot * ss + (int64_t)g * sh;
  }
  return (int64_t)b * sb + (int64_t)(kv_off + j) * ss + (int64_t)g * sh;
}

// Paged key / value, decode: the block ids of the pages a wave reads, looked
// up once before its key loop.  Lane l holds the block id of page p0 + l
// (p0 = page of key j0), the column clamped to the page of key jmax (the
// batch's last visible key) and the id into [0, n_blocks).  The wave's keys
// must span fewer than 64 pages.  Zero when not paged.
struct WavePages {
  int btv;
  int p0;
};

__device__ __forceinline__ WavePages wave_pages(const AttnArgs& a, int b, int j0, int jmax, int lane) {
  WavePages w{0, 0};
  if (a.paged) {
    w.p0 = (int)fast_div((uint32_t)j0, a.bs_div);
    const int pmax = (int)fast_div((uint32_t)jmax, a.bs_div);
    const int col = min(w.p0 + lane, pmax);
    const int blk = a.block_table[(int64_t)b * a.bt_sb + col];
    w.btv = blk < 0 ? 0 : (blk >= a.n_blocks ? a.n_blocks - 1 : blk);
  }
  return w;
}

// kv_row_offset with the page's block id taken from the wave's WavePages
// (no memory access): j must lie in pages p0 .. p0 + 63, at most jmax.
__device__ __forceinline__ int64_t kv_row_offset_w(const AttnArgs& a, const WavePages& w, int64_t sb,
                                                   int64_t ss, int64_t sh, int b, int j, int g,
                                                   int kv_off) {
  if (a.paged) {
    const uint32_t page = fast_div((uint32_t)j, a.bs_div);
    const int slot = j - (int)page * a.block_size;
    const int blk = __builtin_amdgcn_readlane(w.btv, (int)page - w.p0);
    return (int64_t)blk * sb + (int64_t)slot * ss + (int64_t)g * sh;
  }
  return (int64_t)b * sb + (int64_t)(kv_off + j) * ss + (int64_t)g * sh;
}

// Same, for a run of rows known to share one page (paged) -- the block id is
// looked up once by the caller.
__device__ __forceinline__ int64_t paged_row_offset(int blk, int slot, int g, int64_t sb,
                                                    int64_t ss, int64_t sh) {
  return (int64_t)blk * sb + (int64_t)slot * ss + (int64_t)g * sh;
}

__device__ __forceinline__ int clamp_block(int blk, int n_blocks) {
  return blk < 0 ? 0 : (blk >= n_blocks ? n_blocks - 1 : blk);
}

// Buffer resource over [base, base + nbytes): loads past nbytes return zero,
// so rows past a sequence end need no branch.  The base is made wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(nbytes),
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Same, with the non-temporal hint (data read once: streamed past the caches).
__device__ __forceinline__ u32x4 buf_ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}

// 16 bytes per lane from a buffer straight into LDS (no staging registers):
// lane l's bytes land at lds + 16 l.  Kept out of kernel templates: the
// address-space cast is device-only.
__device__ __forceinline__ void buf_ld16_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off,
                                           0, 0, 0);
}
// Same, with the non-temporal hint.
__device__ __forceinline__ void buf_ld16_lds_nt(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off,
                                           0, 0, 2);
}

// XOR swizzle of key rows staged in LDS without padding: 16-byte piece q of
// row r sits in slot q ^ key_swz<PR>(r), PR = pieces per row.  The 16 rows
// that one 16-lane group of an MFMA operand read touches (same piece) then
// land in 16 distinct 16-byte groups of the 256-byte bank window.
template <int PR>
__device__ __forceinline__ int key_swz(int r) {
  return (r / (16 / PR)) % PR;
}

// Four 16-bit values by an LDS transpose read (ds_read_b64_tr_b16).  Within
// each group of 16 lanes, lane i receives value t from position i % 4 of the
// 8-byte piece addressed by lane 4 t + i / 4 of the group.
__device__ __forceinline__ u32x2 lds_tr16(const void* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Workgroup barrier that also publishes buffer-to-LDS loads: each wave first
// waits for all of its own outstanding vector-memory operations.  The
// workgroup-scope fence of __syncthreads does not reliably wait for them, so
// another wave could otherwise read LDS rows whose load is still in flight.
__device__ __forceinline__ void barrier_after_loads() {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt unconstrained
  __syncthreads();
}

// Global loads/stores of 16 and 8 bytes.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// Visible key range [lo, hi) of query row i given Lq, Lk and the mask mode
// (mode 0: all keys; 2: j <= i; 3: j <= i + Lk - Lq; 4: band around i + Lk - Lq).
__device__ __forceinline__ void visible_range(const AttnArgs& a, int i, int Lq, int Lk, int& lo,
                                              int& hi) {
  int64_t d = (int64_t)Lk - Lq;
  int64_t l = 0, h = Lk;
  if (a.mode == 2) {
    h = (int64_t)i + 1;
  } else if (a.mode == 3) {
    h = (int64_t)i + d + 1;
  } else if (a.mode == 4) {
    l = (int64_t)i + d - a.pre;
    h = (int64_t)i + d + a.next + 1;
  }
  if (l < 0) l = 0;
  if (l > Lk) l = Lk;
  if (h > Lk) h = Lk;
  if (h < l) h = l;
  lo = (int)l;
  hi = (int)h;
}

}  // namespace fia
