// Internal interface between the host planner (fia_api.cpp) and the HIP
// kernels (*.hip).  Plain structs passed by value as kernel arguments.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace fia {

// Per-batch record in the device metadata (int32 each).
enum BatchField {
  BF_QLEN = 0,      // actual query length Lq
  BF_KVLEN = 1,     // actual key/value length Lk
  BF_QOFF = 2,      // TND: first query token of the batch (else 0)
  BF_KVOFF = 3,     // TND: first key token of the batch (else 0)
  BF_LO = 4,        // decode: first visible key
  BF_HI = 5,        // decode: one past the last visible key
  BF_NCHUNK = 6,    // decode: number of split-KV chunks
  BF_CHUNK0 = 7,    // decode: global index of the batch's first chunk
  BF_COUNT = 8
};

// Unsigned division by a runtime constant through a 64-bit multiply:
// n / d == (n * mul) >> (32 + shift) for every n < 2^31 (mul < 2^33).
struct FastDiv {
  uint64_t mul;
  uint32_t shift;
  uint32_t d;
};

// Dense / paged attention arguments (prefill, decode and fp32 kernels).
struct AttnArgs {
  const void* q;
  void* o;
  float* lse;
  const void* k;
  const void* v;
  // strides in elements.  Query / output: batch, token, head.  For TND the
  // batch stride is 0 and the token index is offset by BF_QOFF.
  int64_t q_sb, q_ss, q_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t lse_sb, lse_sh, lse_ss;   // lse[b, h, i] (TND: lse[t, h])
  // key / value: dense -> batch, token, head; paged -> block, slot, head.
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  const int32_t* block_table;       // paged only
  int64_t bt_sb;                    // row stride of the block table
  int32_t block_size;
  int32_t n_blocks;
  FastDiv bs_div;
  int32_t paged;
  int32_t tnd;
  int32_t tile_contig;              // 64-key tiles never straddle a page (dense, or block % 64 == 0)
  const int32_t* meta;              // [B * BF_COUNT] then the work list
  const int32_t* work;              // prefill: 2 ints per item; decode: 2 ints per chunk
  int32_t n_work;
  int32_t B, Sq, Skv, Qn, KVn, G, D;
  int32_t esz;                      // bytes per element of q / k / v / o
  float scale;                      // softmax scale
  float scale_log2;                 // scale * log2(e)
  int32_t mode;                     // mask mode 0, 2, 3, 4
  int64_t pre, next;                // band (mode 4)
  const float* slopes;              // ALiBi slopes [Qn] or nullptr
  int32_t alibi_delta;              // kv_start_idx - q_start_idx
  // Explicit mask (modes 0 / 1) or nullptr: key j of query row i of batch b
  // is masked out when mask[b * mask_sb + i * mask_ss + j] != 0.  Rows and
  // mask_sb are multiples of 4 bytes; mask_cols >= the KV extent.
  const uint8_t* mask;
  int64_t mask_sb, mask_ss;
  int32_t mask_rows, mask_cols;
  // Bias tensor (pse type 0) or nullptr, in the element type of q: added to
  // the scaled score of (b, h, i, j) at pse[b * pse_sb + h * pse_sh +
  // i * pse_ss + j] (pse_ss = 0: one row for every query row).  Strides in
  // elements, multiples of 4; pse_cols >= the KV extent.
  const void* pse;
  int64_t pse_sb, pse_sh, pse_ss;
  int32_t pse_rows, pse_cols;
  float inv_scale;                  // 1 / scale (> 0 whenever pse is set)
  // Fake-quantised key / value (decode only): rows of int8 (kvq 1) or e4m3fn
  // (kvq 2) codes, dequantised as scale * (code + offset).  Mode 0: per
  // channel, element kvh * D + d of a bf16 (or fp32, *_f32) tensor, or its
  // only element (*_scalar); mode 1: per token, fp32 element b * *_sb + j
  // (j < *_cols, *_cols and *_sb multiples of 4).  Offsets (nullable) share
  // the scale's layout.
  int32_t kvq;
  int32_t kq_mode, vq_mode;
  const void* kq_scale;
  const void* kq_off;
  const void* vq_scale;
  const void* vq_off;
  int32_t kq_f32, kq_scalar, vq_f32, vq_scalar;
  int64_t kq_sb, vq_sb;
  int32_t kq_cols, vq_cols;
  // Learnable sink: bf16 logit per query head or nullptr; one more softmax
  // term with a zero value vector, not scaled.
  const uint16_t* sink;
  int32_t write_lse;
  // decode split-KV
  int32_t chunk;                    // tokens per chunk (multiple of 128)
  int32_t n_head_blocks;            // ceil(G / 16); 1 with kv_pair
  // Fake-quantised decode: two adjacent KV heads per wave (heads of a token
  // adjacent in memory, G <= 8, KV_N even, D = 128); work items then run
  // over KV head pairs.
  int32_t kv_pair;
  float* part_o;                    // [total_chunks * Qn * D]
  float* part_lse;                  // [total_chunks * Qn]
  // Decode with KV lengths on the device: dev_kvlen int32 [B] is read by
  // decode_partition, which writes the per-batch records, the chunk count
  // (*n_chunks_dev) and the chunk list into the workspace (meta / work point
  // there); lengths are clamped into [0, kvlen_bound].  The split kernels are
  // launched for the bound's chunk count and return early past *n_chunks_dev.
  const int32_t* dev_kvlen;         // nullptr: the plan was built on the host
  int32_t kvlen_bound;
  const int32_t* n_chunks_dev;
};

// One key / value pool of the sparse operators (ori_kv or cmp_kv).  Row rr
// of batch entry b lives at
//   paged: base + clamp(bt[b * bt_sb + min(rr / bs, bt_cols - 1)]) * sb + (rr % bs) * ss
//   dense: base + b * sb + clamp(off_b + rr) * ss, off_b = cu[b] (packed TND
//          rows, sb = 0) or 0 (BSND), clamped into [0, n_rows)
// (block ids clamped into [0, nb)).  Strides in bytes.
struct SparsePool {
  const uint8_t* base;
  int64_t sb, ss;
  const int32_t* bt;                // paged: block table [B, bt_cols]
  int64_t bt_sb;
  int32_t bt_cols, bs, nb;
  int32_t paged;
  const int32_t* cu;                // dense TND: first row of each entry [B + 1]
  int64_t n_rows;                   // dense: rows per batch (BSND) or in total (TND)
};

// Row formats of the sparse operators.
enum SparseFmt {
  SF_FP8_PACKED = 0,   // 640-byte rows: bf16 rope x64 | e4m3fn nope x448 | fp32 scale x7
  SF_BF16 = 1,         // 512 bf16 values
  SF_FP16 = 2          // 512 fp16 values
};

// Shared-KV sparse attention arguments (both sparse operators).
struct SparseArgs {
  // BSND: row r = b * S1 + t is query token t of batch entry b.  TND: row r
  // is token r of [T1, N1, 512]; its batch entry b satisfies
  // cu_q[b] <= r < cu_q[b + 1] (batch strides are 0, token strides address
  // the row).  Partials and the grid run over the n_rows rows.
  int32_t fmt;                      // SparseFmt (query / output are fp16 with SF_FP16, else bf16)
  const uint16_t* q;                // [B, S1, N1, 512] or [T1, N1, 512]
  int64_t q_sb, q_ss, q_sh;
  uint16_t* o;                      // the shape of q
  int64_t o_sb, o_ss, o_sh;
  float* lse;                       // nullptr, or fp32 at b * lse_sb + tq * lse_ss + h * lse_sh
  int64_t lse_sb, lse_ss, lse_sh;
  const int32_t* cu_q;              // TND: int32 [B + 1] on the device; BSND: nullptr
  int32_t n_rows;                   // B * S1 (BSND) or T1 (TND)
  SparsePool ori, cmp;
  const int32_t* idx;               // [B, S1, 1, K2] or [T1, 1, K2]
  int64_t idx_sb, idx_ss;
  const int32_t* seqused;           // [B]
  const float* sinks;               // [N1] or nullptr
  int32_t B, S1, N1, K2;
  int32_t cmp_ratio, win_left, win_right;
  int32_t n_win_slots;              // window slots (multiple of 64)
  int32_t n_slots;                  // window slots + K2
  int32_t has_cmp;
  int32_t cmp_direct;               // no indices: compressed slot k is row k
  float scale_log2;
  // Work split: every query row's slots are cut into n_chunks chunks of
  // sub_per_chunk 64-slot sub-chunks; head blocks of 64 heads.  A workgroup
  // takes one (row, head block, chunk).  xcd_rows: the workgroups of one
  // row run on one XCD (row r on XCD r % 8; needs n_rows % 8 == 0).
  int32_t sub_per_chunk, n_chunks, n_hb, xcd_rows;
  int32_t hb_heads;                 // heads per workgroup (kSparseHeadsSmall or kSparseHeadsLarge)
  float* part_o;                    // [n_rows * n_chunks * N1 * 512] (n_chunks > 1)
  float* part_lse;                  // [n_rows * n_chunks * N1], log2 domain
};

// Launchers (defined next to their kernels).  Return hipGetLastError().
hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_decode_bf16(const AttnArgs& a, int32_t n_items, hipStream_t s);
hipError_t launch_decode_merge(const AttnArgs& a, hipStream_t s);
hipError_t launch_decode_partition(const AttnArgs& a, int32_t* meta, int32_t* work, hipStream_t s);
hipError_t launch_decode_q8(const AttnArgs& a, int32_t n_items, hipStream_t s);
hipError_t launch_attn_fp32(const AttnArgs& a, hipStream_t s);
hipError_t launch_fill_empty(const AttnArgs& a, hipStream_t s);
hipError_t launch_sparse(const SparseArgs& a, hipStream_t s);
hipError_t launch_sparse_merge(const SparseArgs& a, hipStream_t s);
hipError_t launch_debug_gather(const AttnArgs& a, int32_t which, void* dst, int32_t s2max,
                               hipStream_t s);
hipError_t launch_decode_read(const AttnArgs& a, int32_t order, uint32_t* out, hipStream_t s);
hipError_t launch_debug_sparse_rows(const SparseArgs& a, int32_t* ids, uint8_t* rows,
                                    hipStream_t s);

// Workgroups of the decode read pass (the length of its output), or -1 when
// the plan's shape has no instantiation: order 0 needs rows of D * esz bytes
// in {128, 256} (esz: bytes per key / value element, 1 for fake-quant
// codes), order 1 KV_N * D * esz in {1024, 2048} with the heads of a token
// adjacent.
inline int64_t decode_read_grid(const AttnArgs& a, int32_t order) {
  const int64_t esz = a.kvq ? 1 : a.esz;   // bytes per key / value element
  const int64_t row = (int64_t)a.D * esz;
  if (order == 0) {
    if (row != 128 && row != 256) return -1;
    return (int64_t)a.n_work * a.KVn;
  }
  const int64_t span = row * a.KVn;
  if ((span != 1024 && span != 2048) || a.k_sh * esz != row || a.v_sh * esz != row) return -1;
  return (int64_t)a.n_work * 8;
}

// Constants shared by planner and kernels.
constexpr int kPrefillRows = 128;   // query rows per prefill workgroup
constexpr int kPrefillKeys = 64;    // keys per prefill tile
constexpr int kDecodeStep = 32;     // keys per decode wave step
constexpr int kSparseSub = 64;      // row slots per sparse sub-chunk
// Heads per sparse workgroup: 32, or 64 when the launch with 32 would need
// more workgroups than the CUs of a 256-CU MI355X (one workgroup per CU).
constexpr int kSparseHeadsSmall = 32;
constexpr int kSparseHeadsLarge = 64;
constexpr int kSparseCUs = 256;
constexpr int kSparseMaxSub = 8;    // sub-chunks per sparse workgroup, at most
constexpr int kSparseMaxChunks = 64;  // chunks per sparse query row, at most
constexpr int kSparseBtCache = 512;   // block-table entries a sparse workgroup caches in LDS
constexpr int kSparseD = 512;       // logical row width (64 rope + 448 nope)
constexpr int kRowBytes = 640;

}  // namespace fia
