// Host side of libfia: argument validation (the constraint tiers of the
// fused-inference-attention pages), branch dispatch, work planning, workspace
// layout and the C entry points declared in include/fia.h.
//
// Phase 1 (fia_get_workspace_size / fia_sparse_get_workspace_size) is pure
// host code: it never calls into HIP, so it runs without a GPU.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <string>
#include <vector>

#include "fia.h"
#include "fia_internal.h"

using fia::AttnArgs;
using fia::SparseArgs;

namespace {

thread_local std::string g_last_error;

fia_status fail(fia_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

enum Kind { KIND_FILL = 0, KIND_PREFILL = 1, KIND_DECODE = 2, KIND_SPARSE = 3, KIND_FP32 = 4 };

constexpr int kDecodeChunk = 1024;    // keys per split-KV chunk (multiple of 128)
constexpr int64_t kMaxLen = 20971520; // S <= 20M (V2 restrictions when Q_S > 1)
constexpr size_t kAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int dtype_size(int dt) {
  switch (dt) {
    case FIA_DT_BF16:
    case FIA_DT_FP16: return 2;
    case FIA_DT_FP32:
    case FIA_DT_INT32: return 4;
    case FIA_DT_INT64: return 8;
    case FIA_DT_FP8_E4M3FN:
    case FIA_DT_UINT8:
    case FIA_DT_INT8:
    case FIA_DT_BOOL: return 1;
    default: return 0;
  }
}

const char* dtype_name(int dt) {
  static const char* names[] = {"bf16", "fp16", "fp32", "fp8_e4m3fn", "int32",
                                "int64", "uint8", "int8", "bool"};
  return (dt >= 0 && dt <= 8) ? names[dt] : "unknown";
}

int64_t numel(const fia_tensor* t) {
  int64_t n = 1;
  for (int d = 0; d < t->ndim; ++d) n *= t->shape[d];
  return n;
}

std::string shape_str(const fia_tensor* t) {
  std::string s = "[";
  for (int d = 0; d < t->ndim; ++d) {
    if (d) s += ",";
    s += std::to_string(t->shape[d]);
  }
  return s + "]";
}

fia_status check_tensor(const fia_tensor* t, const char* name, bool allow_empty_null = true) {
  if (t->ndim < 1 || t->ndim > 5) {
    return fail(FIA_ERR_PARAM_INVALID, std::string(name) + ": ndim must be 1..5");
  }
  if (dtype_size(t->dtype) == 0) {
    return fail(FIA_ERR_PARAM_INVALID, std::string(name) + ": unknown dtype");
  }
  for (int d = 0; d < t->ndim; ++d) {
    if (t->shape[d] < 0) return fail(FIA_ERR_PARAM_INVALID, std::string(name) + ": negative dim");
  }
  if (numel(t) > 0) {
    if (t->data == nullptr) return fail(FIA_ERR_NULLPTR, std::string(name) + ": data is NULL");
    if (t->stride[t->ndim - 1] != 1 && t->shape[t->ndim - 1] > 1) {
      return fail(FIA_ERR_UNSUPPORTED, std::string(name) + ": innermost dim must be contiguous");
    }
  } else if (!allow_empty_null && t->data == nullptr) {
    return fail(FIA_ERR_NULLPTR, std::string(name) + ": data is NULL");
  }
  return FIA_SUCCESS;
}

// Canonical (batch, seq, head, dim) view of a query-like tensor.
struct Canon {
  int64_t B = 0, S = 0, N = 0, D = 0;
  int64_t sb = 0, ss = 0, sh = 0;
};

fia_status canon(const fia_tensor* t, const std::string& layout, int64_t heads, const char* name,
                 Canon* c) {
  if (layout == "BSND") {
    if (t->ndim != 4) return fail(FIA_ERR_PARAM_INVALID, std::string(name) + ": BSND needs 4 dims");
    *c = {t->shape[0], t->shape[1], t->shape[2], t->shape[3], t->stride[0], t->stride[1], t->stride[2]};
  } else if (layout == "BNSD") {
    if (t->ndim != 4) return fail(FIA_ERR_PARAM_INVALID, std::string(name) + ": BNSD needs 4 dims");
    *c = {t->shape[0], t->shape[2], t->shape[1], t->shape[3], t->stride[0], t->stride[2], t->stride[1]};
  } else if (layout == "BSH") {
    if (t->ndim != 3) return fail(FIA_ERR_PARAM_INVALID, std::string(name) + ": BSH needs 3 dims");
    if (heads <= 0 || t->shape[2] % heads != 0) {
      return fail(FIA_ERR_PARAM_INVALID, std::string(name) + ": H must be a multiple of N");
    }
    const int64_t D = t->shape[2] / heads;
    *c = {t->shape[0], t->shape[1], heads, D, t->stride[0], t->stride[1], D};
  } else if (layout == "TND") {
    if (t->ndim != 3) return fail(FIA_ERR_PARAM_INVALID, std::string(name) + ": TND needs 3 dims");
    *c = {1, t->shape[0], t->shape[1], t->shape[2], 0, t->stride[0], t->stride[1]};
  } else {
    return fail(FIA_ERR_PARAM_INVALID, "input_layout must be BSND, BSH, BNSD or TND");
  }
  return FIA_SUCCESS;
}

fia::FastDiv make_fastdiv(uint32_t d) {
  fia::FastDiv f{};
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  const unsigned __int128 num = (unsigned __int128)1 << (32 + s);
  f.mul = (uint64_t)((num + d - 1) / d);
  f.shift = s;
  return f;
}

}  // namespace

struct fia_executor {
  int kind = KIND_FILL;
  AttnArgs a{};
  SparseArgs sp{};
  std::vector<int32_t> meta;  // uploaded to the start of the workspace
  size_t meta_bytes = 0;
  size_t work_off = 0;        // offset (ints) of the work list inside meta
  size_t part_o_off = 0, part_lse_off = 0;
  size_t ws_size = 0;
  int32_t n_items = 0;        // decode workgroups
  int32_t s2max = 0;
  // Decode with KV lengths on the device: the plan (per-batch records, the
  // chunk count and the chunk list) is written into the workspace at
  // dev_meta_off by the partitioner kernel on every run.
  bool dev_len = false;
  size_t dev_meta_off = 0, dev_work_off = 0;
  bool noop = false;
  // Device copy of `meta`, made by the first run on a device and reused by
  // every later run there (the plan never changes after phase 1).
  void* dplan = nullptr;
  int dplan_device = -1;
};

namespace {

fia_status upload_plan(fia_executor* e) {
  if (e->meta_bytes == 0) return FIA_SUCCESS;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(FIA_ERR_HIP, "hipGetDevice failed");
  if (e->dplan != nullptr && e->dplan_device == dev) return FIA_SUCCESS;
  if (e->dplan != nullptr) {
    (void)hipFree(e->dplan);
    e->dplan = nullptr;
  }
  if (hipMalloc(&e->dplan, e->meta_bytes) != hipSuccess) {
    e->dplan = nullptr;
    return fail(FIA_ERR_HIP, "hipMalloc of the device plan failed");
  }
  if (hipMemcpy(e->dplan, e->meta.data(), e->meta_bytes, hipMemcpyHostToDevice) != hipSuccess) {
    return fail(FIA_ERR_HIP, "upload of the device plan failed");
  }
  e->dplan_device = dev;
  return FIA_SUCCESS;
}

void bind_workspace(fia_executor* e, void* ws) {
  uint8_t* base = static_cast<uint8_t*>(ws);
  if (e->dev_len) {
    int32_t* m = reinterpret_cast<int32_t*>(base + e->dev_meta_off);
    e->a.meta = m;
    e->a.work = reinterpret_cast<const int32_t*>(base + e->dev_work_off);
    e->a.n_chunks_dev = m + (size_t)e->a.B * fia::BF_COUNT;
  } else {
    e->a.meta = static_cast<const int32_t*>(e->dplan);
    e->a.work = static_cast<const int32_t*>(e->dplan) + e->work_off;
  }
  e->a.part_o = reinterpret_cast<float*>(base + e->part_o_off);
  e->a.part_lse = reinterpret_cast<float*>(base + e->part_lse_off);
  e->sp.part_o = reinterpret_cast<float*>(base + e->part_o_off);
  e->sp.part_lse = reinterpret_cast<float*>(base + e->part_lse_off);
}

fia_status check_ws(const fia_executor* e, void* ws, size_t ws_size) {
  if (ws_size < e->ws_size) {
    return fail(FIA_ERR_WORKSPACE, "workspace of " + std::to_string(ws_size) +
                                       " bytes is smaller than the required " +
                                       std::to_string(e->ws_size));
  }
  if (e->ws_size > 0 && ws == nullptr) return fail(FIA_ERR_WORKSPACE, "workspace is NULL");
  if (e->ws_size > 0 && (reinterpret_cast<uintptr_t>(ws) % 16) != 0) {
    return fail(FIA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  }
  return FIA_SUCCESS;
}

// Per-batch lengths from a host array (V2 actualSeqLengths rule).
fia_status lengths_from(const int64_t* arr, int64_t len, int64_t B, int64_t def, bool tnd,
                        int64_t total, const char* name, std::vector<int64_t>* out) {
  out->assign(B, def);
  if (arr == nullptr) {
    if (tnd) return fail(FIA_ERR_PARAM_INVALID, std::string(name) + " is required for TND");
    return FIA_SUCCESS;
  }
  if (tnd) {
    if (len != B) return fail(FIA_ERR_PARAM_INVALID, std::string(name) + ": TND needs exactly B entries");
    int64_t prev = 0;
    for (int64_t b = 0; b < B; ++b) {
      if (arr[b] < prev) {
        return fail(FIA_ERR_PARAM_INVALID, std::string(name) + ": TND entries must be non-decreasing");
      }
      (*out)[b] = arr[b] - prev;
      prev = arr[b];
    }
    if (B > 0 && prev != total) {
      return fail(FIA_ERR_PARAM_INVALID, std::string(name) + ": last TND entry must equal T");
    }
    return FIA_SUCCESS;
  }
  if (len != 1 && len < B) {
    return fail(FIA_ERR_PARAM_INVALID, std::string(name) + ": length must be 1 or >= B");
  }
  for (int64_t b = 0; b < B; ++b) {
    const int64_t v = (len == 1) ? arr[0] : arr[b];
    if (v < 0) return fail(FIA_ERR_PARAM_INVALID, std::string(name) + ": negative length");
    if (v > def) {
      return fail(FIA_ERR_PARAM_INVALID, std::string(name) + ": length " + std::to_string(v) +
                                             " exceeds the tensor's S " + std::to_string(def));
    }
    (*out)[b] = v;
  }
  return FIA_SUCCESS;
}

// Heads per decode work item: blocks of 16 query heads of one KV head, or
// (fake-quantised codes, D = 128, G <= 8, KV_N even, the heads of a token
// adjacent in both caches) two KV heads per wave, whose codes then form one
// 2 D-byte run per token.
void set_head_split(AttnArgs& a, int64_t KVn) {
  a.kv_pair = (a.kvq != 0 && a.D == 128 && a.G <= 8 && KVn % 2 == 0 && a.k_sh == a.D &&
               a.v_sh == a.D) ? 1 : 0;
  a.n_head_blocks = a.kv_pair ? 1 : (a.G + 15) / 16;
}

void visible(int mode, int64_t i, int64_t Lq, int64_t Lk, int64_t pre, int64_t next, int64_t* lo,
             int64_t* hi) {
  const int64_t d = Lk - Lq;
  int64_t l = 0, h = Lk;
  if (mode == 2) {
    h = i + 1;
  } else if (mode == 3) {
    h = i + d + 1;
  } else if (mode == 4) {
    l = i + d - pre;
    h = i + d + next + 1;
  }
  l = std::max<int64_t>(0, std::min(l, Lk));
  h = std::min(h, Lk);
  if (h < l) h = l;
  *lo = l;
  *hi = h;
}

}  // namespace

extern "C" {

const char* fia_last_error(void) { return g_last_error.c_str(); }

int32_t fia_executor_kind(const fia_executor* e) { return e ? e->kind : -1; }

void fia_executor_destroy(fia_executor* e) {
  if (e == nullptr) return;
  if (e->dplan) (void)hipFree(e->dplan);
  delete e;
}

fia_status fia_get_workspace_size(const fia_params* p, const fia_tensor* query,
                                  const fia_tensor* key, const fia_tensor* value,
                                  const fia_tensor* pse_shift, const fia_tensor* atten_mask,
                                  const fia_tensor* block_table, const fia_tensor* attention_out,
                                  const fia_tensor* softmax_lse, size_t* workspace_size,
                                  fia_executor** executor) {
  if (!p || !query || !key || !value || !attention_out || !workspace_size || !executor) {
    return fail(FIA_ERR_NULLPTR, "params, query, key, value, attention_out, workspace_size and "
                                 "executor must not be NULL");
  }
  *executor = nullptr;
  *workspace_size = 0;
  fia_status st;
  if ((st = check_tensor(query, "query")) != FIA_SUCCESS) return st;
  if ((st = check_tensor(key, "key")) != FIA_SUCCESS) return st;
  if ((st = check_tensor(value, "value")) != FIA_SUCCESS) return st;
  if ((st = check_tensor(attention_out, "attention_out")) != FIA_SUCCESS) return st;
  const std::string layout = p->input_layout ? p->input_layout : "BSND";
  const bool tnd = layout == "TND";
  const bool paged = block_table != nullptr;
  const int64_t Qn = p->num_heads;
  const int64_t KVn = p->num_key_value_heads == 0 ? Qn : p->num_key_value_heads;
  if (Qn < 1 || Qn > 256) return fail(FIA_ERR_PARAM_INVALID, "num_heads must be in [1, 256]");
  if (KVn < 1 || Qn % KVn != 0) {
    return fail(FIA_ERR_PARAM_INVALID, "num_heads must be a multiple of num_key_value_heads");
  }
  if (Qn / KVn > 64) return fail(FIA_ERR_PARAM_INVALID, "num_heads / num_key_value_heads must be <= 64");

  Canon cq, co;
  if ((st = canon(query, layout, Qn, "query", &cq)) != FIA_SUCCESS) return st;
  if ((st = canon(attention_out, layout, Qn, "attention_out", &co)) != FIA_SUCCESS) return st;
  if (cq.N != Qn) return fail(FIA_ERR_PARAM_INVALID, "query N axis must equal num_heads");
  if (co.B != cq.B || co.S != cq.S || co.N != cq.N || co.D != cq.D) {
    return fail(FIA_ERR_PARAM_INVALID, "attention_out shape must match query " + shape_str(query));
  }
  if (query->dtype != FIA_DT_BF16 && query->dtype != FIA_DT_FP32) {
    return fail(FIA_ERR_UNSUPPORTED, std::string("query dtype ") + dtype_name(query->dtype) +
                                         " is not supported (bf16, fp32)");
  }
  // Fake-quantised key / value: int8 or e4m3fn codes with a bf16 query.
  const bool kvq = query->dtype == FIA_DT_BF16 &&
                   (key->dtype == FIA_DT_INT8 || key->dtype == FIA_DT_FP8_E4M3FN);
  if (kvq) {
    if (value->dtype != key->dtype) {
      return fail(FIA_ERR_PARAM_INVALID, "fake-quantised key and value must have the same dtype");
    }
  } else if (key->dtype != query->dtype || value->dtype != query->dtype) {
    return fail(FIA_ERR_PARAM_INVALID, "key and value must have the query dtype");
  }
  if (attention_out->dtype != query->dtype) {
    return fail(FIA_ERR_PARAM_INVALID, "attention_out must have the query dtype");
  }
  const int64_t D = cq.D;
  const bool f32 = query->dtype == FIA_DT_FP32;

  // Query batch size and lengths.
  std::vector<int64_t> qlen, kvlen;
  int64_t B;
  std::vector<int64_t> q_cum;
  if (tnd) {
    if (!p->actual_seq_lengths) return fail(FIA_ERR_PARAM_INVALID, "TND requires actual_seq_lengths");
    B = p->actual_seq_lengths_len;
  } else {
    B = cq.B;
  }
  if (B > 65536) return fail(FIA_ERR_PARAM_INVALID, "B must be <= 65536");
  if (D > 512) return fail(FIA_ERR_PARAM_INVALID, "D must be <= 512");
  if (cq.S > kMaxLen) return fail(FIA_ERR_PARAM_INVALID, "S must be <= 20971520");

  // Empty-tensor rule (V4 public constraints): query / output empty -> nothing
  // to do, and validation is skipped.
  if (numel(query) == 0 || numel(attention_out) == 0) {
    fia_executor* e = new fia_executor();
    e->noop = true;
    *executor = e;
    return FIA_SUCCESS;
  }

  if ((st = lengths_from(p->actual_seq_lengths, p->actual_seq_lengths_len, B, cq.S, tnd, cq.S,
                         "actual_seq_lengths", &qlen)) != FIA_SUCCESS) {
    return st;
  }
  // KV lengths on the device: an int32 [B] tensor read by the partitioner
  // kernel at run time; the host sizes everything for the bound.
  const bool dev_len = p->actual_seq_lengths_kv_device != nullptr;
  const int64_t len_bound = p->max_actual_seq_length_kv;
  if (dev_len) {
    const fia_tensor* t = p->actual_seq_lengths_kv_device;
    if ((st = check_tensor(t, "actual_seq_lengths_kv_device")) != FIA_SUCCESS) return st;
    if (t->dtype != FIA_DT_INT32 || t->ndim != 1 || t->shape[0] != B || t->stride[0] != 1) {
      return fail(FIA_ERR_PARAM_INVALID, "actual_seq_lengths_kv_device must be contiguous int32 [B]");
    }
    if (p->actual_seq_lengths_kv != nullptr) {
      return fail(FIA_ERR_PARAM_INVALID, "give actual_seq_lengths_kv or actual_seq_lengths_kv_device, not both");
    }
    if (tnd) return fail(FIA_ERR_PARAM_INVALID, "actual_seq_lengths_kv_device is not supported with TND");
    if (p->pse_type == 2) {
      return fail(FIA_ERR_UNSUPPORTED, "actual_seq_lengths_kv_device does not take ALiBi (its equal-length "
                                       "rule cannot be checked on the host)");
    }
    if (len_bound < 0 || len_bound > kMaxLen) {
      return fail(FIA_ERR_PARAM_INVALID, "max_actual_seq_length_kv must be in [0, 20971520]");
    }
  }
  int64_t max_q = 0;
  for (auto v : qlen) max_q = std::max(max_q, v);

  // Key / value views.
  Canon ck{}, cv{};
  int64_t n_blocks = 0, bs = p->block_size, bt_cols = 0;
  if (paged) {
    if ((st = check_tensor(block_table, "block_table")) != FIA_SUCCESS) return st;
    if (block_table->dtype != FIA_DT_INT32) return fail(FIA_ERR_PARAM_INVALID, "block_table must be int32");
    if (block_table->ndim != 2 || block_table->shape[0] == 0 || block_table->shape[1] == 0) {
      return fail(FIA_ERR_PARAM_INVALID, "block_table must be 2-D with non-zero dims");
    }
    if (block_table->shape[0] != B) return fail(FIA_ERR_PARAM_INVALID, "block_table dim 0 must equal B");
    bt_cols = block_table->shape[1];
    if (bs <= 0) return fail(FIA_ERR_PARAM_INVALID, "block_size must be > 0");
    const bool d_64_128 = (D == 64 || D == 128);
    if (bs % 16 != 0 || bs > 1024) {
      return fail(FIA_ERR_PARAM_INVALID, "block_size must be a multiple of 16 and <= 1024");
    }
    if (!d_64_128 && max_q == 1 && bs > 512) {
      return fail(FIA_ERR_PARAM_INVALID, "block_size must be <= 512 when Q_S == 1");
    }
    if (!p->actual_seq_lengths_kv && !dev_len) {
      return fail(FIA_ERR_PARAM_INVALID, "paged attention requires actual_seq_lengths_kv");
    }
    const std::string kvl = p->kv_layout ? p->kv_layout : "PA_ND";
    const bool bnnbsd = kvl == "BnNBsD";
    if (!bnnbsd && kvl != "PA_ND" && kvl != "BnBsH") {
      return fail(FIA_ERR_PARAM_INVALID, "kv_layout must be PA_ND, BnBsH or BnNBsD");
    }
    for (const fia_tensor* t : {key, value}) {
      if (bnnbsd) {
        if (!(t->ndim == 4 && t->shape[1] == KVn && t->shape[2] == bs && t->shape[3] == D)) {
          return fail(FIA_ERR_PARAM_INVALID, "BnNBsD key/value must be [n_blocks, KV_N, block_size, D], "
                                             "got " + shape_str(t));
        }
        continue;
      }
      const bool four = t->ndim == 4 && t->shape[1] == bs && t->shape[2] == KVn && t->shape[3] == D;
      const bool three = t->ndim == 3 && t->shape[1] == bs && t->shape[2] == KVn * D;
      if (!four && !three) {
        return fail(FIA_ERR_PARAM_INVALID, "paged key/value must be [n_blocks, block_size, KV_N, D] "
                                           "or [n_blocks, block_size, KV_N*D], got " + shape_str(t));
      }
    }
    if (key->shape[0] != value->shape[0]) {
      return fail(FIA_ERR_PARAM_INVALID, "paged key and value must have the same shape");
    }
    n_blocks = key->shape[0];
    auto pool_view = [&](const fia_tensor* t, Canon* c) {
      c->B = n_blocks;
      c->S = bs;
      c->N = KVn;
      c->D = D;
      c->sb = t->stride[0];
      if (bnnbsd) {
        c->ss = t->stride[2];
        c->sh = t->stride[1];
      } else {
        c->ss = t->stride[1];
        c->sh = t->ndim == 4 ? t->stride[2] : D;
      }
    };
    pool_view(key, &ck);
    pool_view(value, &cv);
    std::vector<int64_t> kl;
    if (dev_len) {
      if (len_bound > bt_cols * bs) {
        return fail(FIA_ERR_PARAM_INVALID, "max_actual_seq_length_kv exceeds block_table cols * block_size");
      }
      kl.assign((size_t)B, len_bound);
    } else if ((st = lengths_from(p->actual_seq_lengths_kv, p->actual_seq_lengths_kv_len, B,
                                  bt_cols * bs, false, 0, "actual_seq_lengths_kv", &kl)) != FIA_SUCCESS) {
      return st;
    }
    kvlen = kl;
    int64_t max_kv = 0;
    for (auto v : kvlen) max_kv = std::max(max_kv, v);
    if (bt_cols < (max_kv + bs - 1) / bs) {
      return fail(FIA_ERR_PARAM_INVALID, "block_table dim 1 is smaller than the largest "
                                         "actual_seq_lengths_kv needs");
    }
    if (n_blocks == 0 && max_kv > 0) return fail(FIA_ERR_PARAM_INVALID, "paged key/value pool is empty");
  } else {
    if ((st = canon(key, layout, KVn, "key", &ck)) != FIA_SUCCESS) return st;
    if ((st = canon(value, layout, KVn, "value", &cv)) != FIA_SUCCESS) return st;
    if (ck.N != KVn || cv.N != KVn) {
      return fail(FIA_ERR_PARAM_INVALID, "key/value N axis must equal num_key_value_heads");
    }
    if (ck.D != D || cv.D != D) {
      return fail(FIA_ERR_UNSUPPORTED, "query, key and value head dims must be equal");
    }
    if (ck.S != cv.S || ck.B != cv.B) return fail(FIA_ERR_PARAM_INVALID, "key and value shapes differ");
    if (!tnd && ck.B != B) return fail(FIA_ERR_PARAM_INVALID, "key batch must equal query batch");
    if (dev_len) {
      if (len_bound > ck.S) return fail(FIA_ERR_PARAM_INVALID, "max_actual_seq_length_kv exceeds KV_S");
      kvlen.assign((size_t)B, len_bound);
    } else if ((st = lengths_from(p->actual_seq_lengths_kv, p->actual_seq_lengths_kv_len, B, ck.S, tnd,
                                  ck.S, "actual_seq_lengths_kv", &kvlen)) != FIA_SUCCESS) {
      return st;
    }
  }
  if (ck.S > kMaxLen) return fail(FIA_ERR_PARAM_INVALID, "KV S must be <= 20971520");

  // Mask group.
  const int mode = p->sparse_mode;
  if (mode < 0 || mode > 4) return fail(FIA_ERR_PARAM_INVALID, "sparse_mode must be in [0, 4]");
  if (mode == 1 && atten_mask == nullptr) {
    return fail(FIA_ERR_PARAM_INVALID, "sparse_mode 1 needs an explicit atten_mask tensor");
  }
  // Explicit mask (modes 0 / 1): [B or 1, >= Q_S, >= KV_S], [B or 1, 1, >= Q_S,
  // >= KV_S] or [>= Q_S, >= KV_S]; element != 0 masks the key out.
  const bool explicit_mask = atten_mask != nullptr && (mode == 0 || mode == 1);
  int64_t mask_sb = 0, mask_ss = 0, mask_rows = 0, mask_cols = 0;
  if (explicit_mask) {
    if ((st = check_tensor(atten_mask, "atten_mask")) != FIA_SUCCESS) return st;
    const int dt = atten_mask->dtype;
    if (dt != FIA_DT_BOOL && dt != FIA_DT_INT8 && dt != FIA_DT_UINT8) {
      return fail(FIA_ERR_PARAM_INVALID, "atten_mask dtype must be bool, int8 or uint8");
    }
    if (tnd) return fail(FIA_ERR_UNSUPPORTED, "an explicit atten_mask with TND is not supported");
    const int nd = atten_mask->ndim;
    if (nd < 2 || nd > 4) return fail(FIA_ERR_PARAM_INVALID, "atten_mask must have 2, 3 or 4 dims");
    if (nd == 4 && atten_mask->shape[1] != 1) {
      return fail(FIA_ERR_PARAM_INVALID, "a 4-dim atten_mask must be [B or 1, 1, Q_S, KV_S]");
    }
    const int64_t mb = nd >= 3 ? atten_mask->shape[0] : 1;
    if (mb != 1 && mb != B) return fail(FIA_ERR_PARAM_INVALID, "atten_mask dim 0 must be B or 1");
    mask_rows = atten_mask->shape[nd - 2];
    mask_cols = atten_mask->shape[nd - 1];
    const int64_t S2m = paged ? bt_cols * bs : ck.S;
    if (mask_rows < cq.S || mask_cols < S2m) {
      return fail(FIA_ERR_PARAM_INVALID, "atten_mask must cover [Q_S, KV_S]");
    }
    if (atten_mask->stride[nd - 1] != 1) {
      return fail(FIA_ERR_PARAM_INVALID, "atten_mask rows must be contiguous");
    }
    mask_ss = atten_mask->stride[nd - 2];
    mask_sb = (nd >= 3 && mb > 1) ? atten_mask->stride[0] : 0;
    if (mask_ss % 4 || mask_sb % 4 || mask_cols % 4 ||
        reinterpret_cast<uintptr_t>(atten_mask->data) % 4) {
      return fail(FIA_ERR_UNSUPPORTED, "atten_mask rows must be 4-byte aligned (pad KV_S to a "
                                       "multiple of 4)");
    }
  } else if (atten_mask != nullptr) {
    const int dt = atten_mask->dtype;
    if (dt != FIA_DT_BOOL && dt != FIA_DT_INT8 && dt != FIA_DT_UINT8) {
      return fail(FIA_ERR_PARAM_INVALID, "atten_mask dtype must be bool, int8 or uint8");
    }
    const int nd = atten_mask->ndim;
    bool ok = nd >= 2 && nd <= 4 && atten_mask->shape[nd - 1] == 2048 && atten_mask->shape[nd - 2] == 2048;
    for (int d = 0; ok && d < nd - 2; ++d) ok = atten_mask->shape[d] == 1;
    if (!ok) {
      return fail(FIA_ERR_PARAM_INVALID, "sparse_mode 2/3/4 needs atten_mask of shape (2048,2048), "
                                         "(1,2048,2048) or (1,1,2048,2048)");
    }
  }
  if (mode == 4 && -p->next_tokens > p->pre_tokens) {
    return fail(FIA_ERR_PARAM_INVALID, "pre_tokens and next_tokens must satisfy -next_tokens <= pre_tokens");
  }

  // PSE group.
  const int pse = p->pse_type;
  if (pse != 0 && pse != 1 && pse != 2 && pse != 3) {
    return fail(FIA_ERR_PARAM_INVALID, "pse_type must be 0, 2 or 3");
  }
  if (pse == 1) return fail(FIA_ERR_PARAM_INVALID, "pse_type 1 is for training only");
  if (pse == 3) return fail(FIA_ERR_UNSUPPORTED, "pse_type 3 is not supported");
  // pseType 0 with a tensor: bias [B or 1, Q_N, >= Q_S or 1, >= KV_S] in the
  // query's dtype, added to the scaled scores (V5 PSE group).
  int64_t pse_sb = 0, pse_sh = 0, pse_ss = 0, pse_rows = 0, pse_cols = 0;
  const bool pse_tensor = pse == 0 && pse_shift != nullptr;
  if (pse_tensor) {
    if ((st = check_tensor(pse_shift, "pse_shift")) != FIA_SUCCESS) return st;
    // The prefill kernel folds the bias into its score accumulators as
    // bias / scale.
    if (!(p->scale_value > 0.0)) {
      return fail(FIA_ERR_UNSUPPORTED, "a pse_shift tensor needs scale_value > 0");
    }
    if (pse_shift->dtype != query->dtype) {
      return fail(FIA_ERR_PARAM_INVALID, "pse_shift must have the query's dtype");
    }
    if (tnd) return fail(FIA_ERR_UNSUPPORTED, "a pse_shift tensor with TND is not supported");
    if (pse_shift->ndim != 4) return fail(FIA_ERR_PARAM_INVALID, "pse_shift must have 4 dims");
    const int64_t pb = pse_shift->shape[0];
    pse_rows = pse_shift->shape[2];
    pse_cols = pse_shift->shape[3];
    const int64_t S2p = paged ? bt_cols * bs : ck.S;
    if ((pb != 1 && pb != B) || pse_shift->shape[1] != Qn || (pse_rows != 1 && pse_rows < cq.S) ||
        pse_cols < S2p) {
      return fail(FIA_ERR_PARAM_INVALID, "pse_shift must be [B or 1, Q_N, >= Q_S or 1, >= KV_S]");
    }
    if (pse_shift->stride[3] != 1) return fail(FIA_ERR_PARAM_INVALID, "pse_shift rows must be contiguous");
    pse_sb = pb > 1 ? pse_shift->stride[0] : 0;
    pse_sh = pse_shift->stride[1];
    pse_ss = pse_rows > 1 ? pse_shift->stride[2] : 0;
    const int64_t esz = query->dtype == FIA_DT_FP32 ? 4 : 2;
    if (pse_sb % 4 || pse_sh % 4 || pse_ss % 4 || pse_cols % 4 ||
        reinterpret_cast<uintptr_t>(pse_shift->data) % (4 * esz)) {
      return fail(FIA_ERR_UNSUPPORTED, "pse_shift rows must be aligned to 4 elements (pad KV_S to a "
                                       "multiple of 4)");
    }
  }
  // LearnableSink group (V5): [Q_N] in the query's dtype (bf16 / fp16 only).
  const fia_tensor* sink = p->learnable_sink;
  if (sink != nullptr) {
    if ((st = check_tensor(sink, "learnable_sink")) != FIA_SUCCESS) return st;
    if (sink->dtype != FIA_DT_BF16 && sink->dtype != FIA_DT_FP16) {
      return fail(FIA_ERR_PARAM_INVALID, "learnable_sink dtype must be float16 or bfloat16");
    }
    if (sink->dtype != query->dtype) {
      return fail(FIA_ERR_PARAM_INVALID, "learnable_sink must have the query's dtype");
    }
    if (sink->ndim != 1 || sink->shape[0] != Qn) {
      return fail(FIA_ERR_PARAM_INVALID, "learnable_sink shape must be (Q_N)");
    }
    if (sink->stride[0] != 1) return fail(FIA_ERR_PARAM_INVALID, "learnable_sink must be contiguous");
    if (p->inner_precise != 0) {
      return fail(FIA_ERR_PARAM_INVALID, "learnable_sink requires inner_precise 0");
    }
    if (pse == 2 || pse_tensor) {
      return fail(FIA_ERR_PARAM_INVALID, "learnable_sink does not combine with pse or ALiBi");
    }
  }
  // Fake-quant group (V5 quantisation parameters, fake-quant scenario).
  struct AqView {
    const void* scale = nullptr;
    const void* off = nullptr;
    int32_t f32 = 0, scalar = 0, cols = 0;
    int64_t sb = 0;
  } aqk, aqv;
  const int kmode = p->key_antiquant_mode, vmode = p->value_antiquant_mode;
  if (kvq) {
    if (kmode < 0 || kmode > 6 || vmode < 0 || vmode > 6) {
      return fail(FIA_ERR_PARAM_INVALID, "key/value_antiquant_mode must be in [0, 6]");
    }
    if (kmode != vmode && !(kmode == 0 && vmode == 1)) {
      return fail(FIA_ERR_PARAM_INVALID, "key and value antiquant modes must be equal, or key per "
                                         "channel (0) with value per token (1)");
    }
    if (kmode > 1 || vmode > 1) {
      return fail(FIA_ERR_UNSUPPORTED, "antiquant modes 2-6 are not supported");
    }
    if (max_q > 1 || (!tnd && cq.S != 1)) {
      return fail(FIA_ERR_UNSUPPORTED, "fake-quantised key/value are supported for query length 1");
    }
    if (D != 64 && D != 128) return fail(FIA_ERR_UNSUPPORTED, "fake-quantised key/value need D 64 or 128");
    if (pse == 2 || pse_tensor || explicit_mask || sink != nullptr) {
      return fail(FIA_ERR_UNSUPPORTED, "fake-quantised key/value do not combine with pse, an explicit "
                                       "mask or a learnable sink");
    }
    if (paged && (bs % 32 != 0 || bs > 512)) {
      return fail(FIA_ERR_PARAM_INVALID, "fake-quant paged attention needs block_size % 32 == 0, <= 512");
    }
    const fia_tensor* ksc = p->key_antiquant_scale;
    const fia_tensor* vsc = p->value_antiquant_scale;
    const fia_tensor* kof = p->key_antiquant_offset;
    const fia_tensor* vof = p->value_antiquant_offset;
    if (ksc == nullptr || vsc == nullptr) {
      return fail(FIA_ERR_PARAM_INVALID, "fake quant needs key_antiquant_scale and value_antiquant_scale");
    }
    if ((kof == nullptr) != (vof == nullptr)) {
      return fail(FIA_ERR_PARAM_INVALID, "key_antiquant_offset and value_antiquant_offset go together");
    }
    if (kof != nullptr && key->dtype != FIA_DT_INT8) {
      return fail(FIA_ERR_PARAM_INVALID, "antiquant offsets are for int8 key/value only");
    }
    // Key length of the per-token tables: the padded S2, or with TND the
    // longest actual key length.
    int64_t S2q = paged ? bt_cols * bs : ck.S;
    if (tnd) {
      S2q = 0;
      for (auto v : kvlen) S2q = std::max(S2q, v);
    }
    auto view = [&](const fia_tensor* sc, const fia_tensor* of, int m, bool f32_chan, const char* what,
                    AqView* out) -> fia_status {
      fia_status s2;
      for (const fia_tensor* t : {sc, of}) {
        if (t == nullptr) continue;
        if ((s2 = check_tensor(t, what)) != FIA_SUCCESS) return s2;
        if (of != nullptr && (t->dtype != sc->dtype || t->ndim != sc->ndim)) {
          return fail(FIA_ERR_PARAM_INVALID, std::string(what) + ": offset must match the scale");
        }
        for (int d = 0; of != nullptr && d < t->ndim; ++d) {
          if (of->shape[d] != sc->shape[d] || of->stride[d] != sc->stride[d]) {
            return fail(FIA_ERR_PARAM_INVALID, std::string(what) + ": offset must match the scale");
          }
        }
      }
      out->scale = sc->data;
      out->off = of ? of->data : nullptr;
      if (m == 0) {
        const int want = f32_chan ? FIA_DT_FP32 : FIA_DT_BF16;
        if (sc->dtype != want) {
          return fail(FIA_ERR_PARAM_INVALID, std::string(what) + ": per-channel scale dtype must be " +
                                                 (f32_chan ? "fp32" : "the query's"));
        }
        if (numel(sc) == 1 && sc->ndim == 1) {
          if (key->dtype != FIA_DT_INT8 || f32_chan) {
            return fail(FIA_ERR_PARAM_INVALID, std::string(what) + ": per-tensor scale is for int8 "
                                                                   "with equal modes");
          }
          out->scalar = 1;
        } else {
          // (1, N, 1, D), (1, N, D), (1, H), (N, 1, D), (N, D), (H): N * D
          // contiguous values.
          bool ok = numel(sc) == KVn * D && sc->shape[sc->ndim - 1] % D == 0;
          if (sc->ndim == 4) ok = ok && sc->shape[0] == 1 && sc->shape[2] == 1 && sc->shape[3] == D;
          if (sc->ndim == 3) ok = ok && sc->shape[2] == D && (sc->shape[0] == 1 || sc->shape[1] == 1);
          int64_t acc = 1;
          for (int d = sc->ndim - 1; ok && d >= 0; --d) {
            if (sc->shape[d] > 1 && sc->stride[d] != acc) ok = false;
            acc *= sc->shape[d];
          }
          if (!ok) {
            return fail(FIA_ERR_PARAM_INVALID, std::string(what) + ": per-channel scale must be (1, N, 1, D), "
                                                   "(1, N, D), (1, H), (N, 1, D), (N, D) or (H), contiguous");
          }
        }
        out->f32 = f32_chan ? 1 : 0;
      } else {
        if (sc->dtype != FIA_DT_FP32) {
          return fail(FIA_ERR_PARAM_INVALID, std::string(what) + ": per-token scale must be fp32");
        }
        const bool two = sc->ndim == 2 && sc->shape[0] == B;
        const bool three = sc->ndim == 3 && sc->shape[0] == 1 && sc->shape[1] == B;
        if ((!two && !three) || sc->shape[sc->ndim - 1] < S2q) {
          return fail(FIA_ERR_PARAM_INVALID, std::string(what) + ": per-token scale must be (B, >= S2) or "
                                                                 "(1, B, >= S2)");
        }
        out->sb = sc->stride[sc->ndim - 2];
        const int64_t cols = sc->shape[sc->ndim - 1];
        if (cols > INT32_MAX) return fail(FIA_ERR_PARAM_INVALID, std::string(what) + ": too long");
        out->cols = (int32_t)cols;
        if (out->sb % 4 || cols % 4 || reinterpret_cast<uintptr_t>(sc->data) % 16 ||
            (of && reinterpret_cast<uintptr_t>(of->data) % 16)) {
          return fail(FIA_ERR_UNSUPPORTED, std::string(what) + ": per-token rows must be 16-byte aligned "
                                                               "(pad S2 to a multiple of 4)");
        }
      }
      return FIA_SUCCESS;
    };
    const bool mixed = kmode == 0 && vmode == 1;
    if ((st = view(ksc, kof, kmode, mixed, "key_antiquant_scale", &aqk)) != FIA_SUCCESS) return st;
    if ((st = view(vsc, vof, vmode, false, "value_antiquant_scale", &aqv)) != FIA_SUCCESS) return st;
  } else if (p->key_antiquant_scale || p->value_antiquant_scale || p->key_antiquant_offset ||
             p->value_antiquant_offset) {
    return fail(FIA_ERR_PARAM_INVALID, "antiquant scales / offsets need int8 or fp8 key/value");
  }
  if (pse == 2) {
    if (pse_shift == nullptr) return fail(FIA_ERR_PARAM_INVALID, "pse_type 2 requires pse_shift");
    if ((st = check_tensor(pse_shift, "pse_shift")) != FIA_SUCCESS) return st;
    if (pse_shift->dtype != FIA_DT_FP32) return fail(FIA_ERR_PARAM_INVALID, "ALiBi pse_shift must be fp32");
    if (pse_shift->ndim != 1 || pse_shift->shape[0] != Qn) {
      return fail(FIA_ERR_PARAM_INVALID, "ALiBi pse_shift shape must be (Q_N)");
    }
    const int64_t dlt = p->kv_start_idx - p->q_start_idx;
    if (dlt < -1048576 || dlt > 1048576) {
      return fail(FIA_ERR_PARAM_INVALID, "kv_start_idx - q_start_idx must be in [-1048576, 1048576]");
    }
    const int64_t S2 = paged ? bt_cols * bs : ck.S;
    if (!paged && !tnd && cq.S != S2) return fail(FIA_ERR_PARAM_INVALID, "ALiBi requires Q_S == KV_S");
    for (int64_t b = 0; b < B; ++b) {
      if (qlen[b] != kvlen[b]) {
        return fail(FIA_ERR_PARAM_INVALID, "ALiBi requires equal actual query and key lengths");
      }
    }
  }

  // SoftmaxLSE group.
  if (p->softmax_lse_flag) {
    if (softmax_lse == nullptr) return fail(FIA_ERR_PARAM_INVALID, "softmax_lse_flag needs softmax_lse");
    if ((st = check_tensor(softmax_lse, "softmax_lse")) != FIA_SUCCESS) return st;
    if (softmax_lse->dtype != FIA_DT_FP32) return fail(FIA_ERR_PARAM_INVALID, "softmax_lse must be fp32");
    if (tnd) {
      if (softmax_lse->ndim != 3 || softmax_lse->shape[0] != cq.S || softmax_lse->shape[1] != Qn ||
          softmax_lse->shape[2] != 1) {
        return fail(FIA_ERR_PARAM_INVALID, "softmax_lse must be [T, Q_N, 1] for TND");
      }
    } else if (softmax_lse->ndim != 4 || softmax_lse->shape[0] != B || softmax_lse->shape[1] != Qn ||
               softmax_lse->shape[2] != cq.S || softmax_lse->shape[3] != 1) {
      return fail(FIA_ERR_PARAM_INVALID, "softmax_lse must be [B, Q_N, Q_S, 1]");
    }
  }
  if (!(p->scale_value >= 0.0) || std::isinf(p->scale_value)) {
    return fail(FIA_ERR_UNSUPPORTED, "scale_value must be a finite non-negative number");
  }
  if (p->inner_precise < 0 || p->inner_precise > 3) {
    return fail(FIA_ERR_PARAM_INVALID, "inner_precise must be in [0, 3]");
  }

  // Kernel-specific requirements.
  if (f32) {
    if (D != 32 && D != 64 && D != 128 && D != 256) {
      return fail(FIA_ERR_UNSUPPORTED, "fp32 path needs D in {32, 64, 128, 256}");
    }
  } else if (D != 64 && D != 128) {
    return fail(FIA_ERR_UNSUPPORTED, "bf16 kernels support head dim 64 and 128");
  }
  const bool kv_empty = numel(key) == 0 || numel(value) == 0 || (!paged && ck.S == 0);
  {
    // Key / value of an empty input are never read; their strides do not matter.
    const int64_t vec = f32 ? 4 : 8;  // elements per 16-byte access
    const int64_t kv_vec = kvq ? 16 : vec;
    const int64_t strides[] = {cq.ss, cq.sh, co.ss, co.sh, tnd ? 0 : cq.sb, tnd ? 0 : co.sb};
    const int64_t kv_strides[] = {ck.ss, ck.sh, cv.ss, cv.sh, ck.sb, cv.sb};
    for (int64_t s : strides) {
      if (s % vec != 0) return fail(FIA_ERR_UNSUPPORTED, "row strides must be multiples of 16 bytes");
    }
    const void* ptrs[] = {query->data, attention_out->data};
    for (const void* ptr : ptrs) {
      if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0) {
        return fail(FIA_ERR_UNSUPPORTED, "tensor data must be 16-byte aligned");
      }
    }
    if (!kv_empty) {
      for (int64_t s : kv_strides) {
        if (s % kv_vec != 0) return fail(FIA_ERR_UNSUPPORTED, "row strides must be multiples of 16 bytes");
      }
      if (ck.ss < D || cv.ss < D) {
        return fail(FIA_ERR_UNSUPPORTED, "key/value rows must not overlap (token stride >= D)");
      }
      if (reinterpret_cast<uintptr_t>(key->data) % 16 != 0 ||
          reinterpret_cast<uintptr_t>(value->data) % 16 != 0) {
        return fail(FIA_ERR_UNSUPPORTED, "tensor data must be 16-byte aligned");
      }
    }
  }
  for (int64_t b = 0; b < B; ++b) {
    if (qlen[b] > INT32_MAX || kvlen[b] > INT32_MAX) return fail(FIA_ERR_PARAM_INVALID, "length too large");
  }

  // Build the executor.
  if (dev_len) {
    if (f32) return fail(FIA_ERR_UNSUPPORTED, "actual_seq_lengths_kv_device needs a bf16 query (fp32 is not taken)");
    if (explicit_mask || pse_tensor) {
      return fail(FIA_ERR_UNSUPPORTED, "actual_seq_lengths_kv_device does not take atten_mask or pse_shift tensors");
    }
  }
  fia_executor* e = new fia_executor();
  AttnArgs& a = e->a;
  a.q = query->data;
  a.o = attention_out->data;
  a.k = key->data;
  a.v = value->data;
  a.lse = p->softmax_lse_flag ? static_cast<float*>(softmax_lse->data) : nullptr;
  a.write_lse = p->softmax_lse_flag ? 1 : 0;
  a.q_sb = cq.sb; a.q_ss = cq.ss; a.q_sh = cq.sh;
  a.o_sb = co.sb; a.o_ss = co.ss; a.o_sh = co.sh;
  a.k_sb = ck.sb; a.k_ss = ck.ss; a.k_sh = ck.sh;
  a.v_sb = cv.sb; a.v_ss = cv.ss; a.v_sh = cv.sh;
  if (a.write_lse) {
    if (tnd) {
      a.lse_sb = 0; a.lse_ss = softmax_lse->stride[0]; a.lse_sh = softmax_lse->stride[1];
    } else {
      a.lse_sb = softmax_lse->stride[0]; a.lse_sh = softmax_lse->stride[1]; a.lse_ss = softmax_lse->stride[2];
    }
  }
  a.paged = paged ? 1 : 0;
  a.tnd = tnd ? 1 : 0;
  if (paged) {
    a.block_table = static_cast<const int32_t*>(block_table->data);
    a.bt_sb = block_table->stride[0];
    a.block_size = (int32_t)bs;
    a.n_blocks = (int32_t)n_blocks;
    a.bs_div = make_fastdiv((uint32_t)bs);
  }
  a.B = (int32_t)B;
  a.Sq = (int32_t)cq.S;
  a.Skv = (int32_t)(paged ? bt_cols * bs : ck.S);
  a.Qn = (int32_t)Qn;
  a.KVn = (int32_t)KVn;
  a.G = (int32_t)(Qn / KVn);
  a.D = (int32_t)D;
  a.esz = f32 ? 4 : 2;
  a.tile_contig = (!paged || bs % fia::kPrefillKeys == 0) ? 1 : 0;
  a.scale = (float)p->scale_value;
  a.scale_log2 = (float)(p->scale_value * 1.4426950408889634);
  a.inv_scale = p->scale_value > 0.0 ? (float)(1.0 / p->scale_value) : 0.f;
  a.mode = mode;
  a.pre = p->pre_tokens;
  a.next = p->next_tokens;
  a.slopes = pse == 2 ? static_cast<const float*>(pse_shift->data) : nullptr;
  a.alibi_delta = (int32_t)(p->kv_start_idx - p->q_start_idx);
  a.pse = pse_tensor ? pse_shift->data : nullptr;
  a.sink = sink != nullptr ? static_cast<const uint16_t*>(sink->data) : nullptr;
  a.kvq = kvq ? (key->dtype == FIA_DT_INT8 ? 1 : 2) : 0;
  a.kq_mode = kmode;
  a.vq_mode = vmode;
  a.kq_scale = aqk.scale; a.kq_off = aqk.off; a.kq_f32 = aqk.f32; a.kq_scalar = aqk.scalar;
  a.kq_sb = aqk.sb; a.kq_cols = aqk.cols;
  a.vq_scale = aqv.scale; a.vq_off = aqv.off; a.vq_f32 = aqv.f32; a.vq_scalar = aqv.scalar;
  a.vq_sb = aqv.sb; a.vq_cols = aqv.cols;
  a.pse_sb = pse_sb;
  a.pse_sh = pse_sh;
  a.pse_ss = pse_ss;
  a.pse_rows = (int32_t)pse_rows;
  a.pse_cols = (int32_t)pse_cols;
  a.mask = explicit_mask ? static_cast<const uint8_t*>(atten_mask->data) : nullptr;
  a.mask_sb = mask_sb;
  a.mask_ss = mask_ss;
  a.mask_rows = (int32_t)mask_rows;
  a.mask_cols = (int32_t)mask_cols;

  // Per-batch records.
  e->meta.assign((size_t)B * fia::BF_COUNT, 0);
  int64_t qo = 0, ko = 0, max_kv = 0;
  for (int64_t b = 0; b < B; ++b) {
    int32_t* r = &e->meta[(size_t)b * fia::BF_COUNT];
    r[fia::BF_QLEN] = (int32_t)qlen[b];
    r[fia::BF_KVLEN] = (int32_t)kvlen[b];
    r[fia::BF_QOFF] = tnd ? (int32_t)qo : 0;
    r[fia::BF_KVOFF] = tnd ? (int32_t)ko : 0;
    qo += qlen[b];
    ko += kvlen[b];
    max_kv = std::max(max_kv, kvlen[b]);
  }
  e->s2max = (int32_t)max_kv;
  e->work_off = e->meta.size();

  if (kv_empty) {
    e->kind = KIND_FILL;
  } else if (f32) {
    e->kind = KIND_FP32;
  } else if (max_q <= 1 && (tnd || cq.S == 1)) {
    e->kind = KIND_DECODE;
  } else {
    e->kind = KIND_PREFILL;
  }

  if (e->kind == KIND_PREFILL) {
    if (dev_len) {
      // KV lengths on the device: the items are planned (and costed) for the
      // bound; the kernel reads each entry's length, clamped into
      // [0, bound], and derives its visible key ranges from it.
      a.dev_kvlen = static_cast<const int32_t*>(p->actual_seq_lengths_kv_device->data);
      a.kvlen_bound = (int32_t)len_bound;
    }
    struct Item { int64_t cost; int32_t b, h, qt; };
    std::vector<Item> items;
    for (int64_t b = 0; b < B; ++b) {
      const int64_t rows = tnd ? qlen[b] : cq.S;
      const int64_t nqt = (rows + fia::kPrefillRows - 1) / fia::kPrefillRows;
      // Padded layouts: the tiles wholly past the actual query length get
      // no item; item qt of the nl live tiles (at least one) also writes the
      // rows of tiles nl + qt, nl + qt + nl, ... (zeros, LSE +inf).
      const int64_t nl = tnd ? nqt
                             : std::min(nqt, std::max<int64_t>(
                                                 (qlen[b] + fia::kPrefillRows - 1) / fia::kPrefillRows, 1));
      for (int64_t qt = 0; qt < nl; ++qt) {
        int64_t cost = 0;
        if (!tnd && nl + qt < nqt) cost += ((nqt - 1 - (nl + qt)) / nl + 1 + 3) / 4;
        const int64_t i0 = qt * fia::kPrefillRows;
        const int64_t i1 = std::min(i0 + fia::kPrefillRows, qlen[b]);
        if (i1 > i0) {
          int64_t l0, h0, l1, h1;
          visible(mode, i0, qlen[b], kvlen[b], p->pre_tokens, p->next_tokens, &l0, &h0);
          visible(mode, i1 - 1, qlen[b], kvlen[b], p->pre_tokens, p->next_tokens, &l1, &h1);
          if (h1 > l0) {
            cost += (h1 + fia::kPrefillKeys - 1) / fia::kPrefillKeys - l0 / fia::kPrefillKeys;
          }
        }
        for (int64_t h = 0; h < Qn; ++h) items.push_back({cost, (int32_t)b, (int32_t)h, (int32_t)qt});
      }
    }
    if (items.size() > (size_t)INT32_MAX / 2) {
      delete e;
      return fail(FIA_ERR_UNSUPPORTED, "too many prefill work items");
    }
    // Longest first: the hardware dispatcher hands workgroups out in index
    // order, so this is a greedy longest-processing-time schedule.
    std::stable_sort(items.begin(), items.end(),
                     [](const Item& x, const Item& y) { return x.cost > y.cost; });
    // Workgroups go round-robin to the 8 XCDs, each with its own L2.  Inside
    // each run of one (batch, query tile) (Qn items of equal cost, adjacent
    // after the stable sort), the query heads of one KV head are moved to
    // positions congruent mod 8, so they run on one XCD and share its L2
    // copy of the key / value tiles.
    {
      const int64_t G = Qn / KVn;
      std::vector<Item> run;
      std::vector<std::vector<Item>> lanes(8);
      for (size_t k0 = 0; k0 < items.size();) {
        size_t k1 = k0;
        while (k1 < items.size() && items[k1].b == items[k0].b && items[k1].qt == items[k0].qt) ++k1;
        if ((int64_t)(k1 - k0) == Qn) {
          for (auto& l : lanes) l.clear();
          for (size_t k = k0; k < k1; ++k) lanes[(size_t)((items[k].h / G) % 8)].push_back(items[k]);
          run.clear();
          for (size_t pos = 0; run.size() < (size_t)Qn; ++pos) {
            // take the next item of lane pos % 8, or of the next non-empty lane
            for (size_t t = 0; t < 8; ++t) {
              std::vector<Item>& l = lanes[(pos + t) % 8];
              if (!l.empty()) {
                run.push_back(l.front());
                l.erase(l.begin());
                break;
              }
            }
          }
          std::copy(run.begin(), run.end(), items.begin() + (int64_t)k0);
        }
        k0 = k1;
      }
    }
    for (const Item& it : items) {
      e->meta.push_back(it.b);
      e->meta.push_back(it.h | (it.qt << 8));
    }
    a.n_work = (int32_t)items.size();
    for (const Item& it : items) {
      if (it.qt >= (1 << 23)) {
        delete e;
        return fail(FIA_ERR_UNSUPPORTED, "query too long for the prefill work encoding");
      }
    }
  } else if (e->kind == KIND_DECODE && dev_len) {
    // Lengths on the device: size the grid and the workspace for the bound
    // (every entry at the bound, plus one chunk for a band that starts
    // inside a chunk); the partitioner kernel writes the real plan into the
    // workspace on every run.
    const int64_t chunk = kDecodeChunk;
    const int64_t per_b = (len_bound + chunk - 1) / chunk + (mode == 4 ? 1 : 0);
    const int64_t total_max = B * per_b;
    a.chunk = (int32_t)chunk;
    set_head_split(a, KVn);
    const int64_t n_items = total_max * (a.kv_pair ? KVn / 2 : KVn) * a.n_head_blocks;
    if (n_items > INT32_MAX) {
      delete e;
      return fail(FIA_ERR_UNSUPPORTED, "too many decode work items");
    }
    e->dev_len = true;
    e->n_items = (int32_t)n_items;
    a.n_work = (int32_t)total_max;
    a.dev_kvlen = static_cast<const int32_t*>(p->actual_seq_lengths_kv_device->data);
    a.kvlen_bound = (int32_t)len_bound;
    e->meta_bytes = 0;   // nothing to upload
    e->dev_meta_off = 0;
    e->dev_work_off = align_up(((size_t)B * fia::BF_COUNT + 4) * sizeof(int32_t), kAlign);
    e->part_o_off = align_up(e->dev_work_off + (size_t)total_max * 2 * sizeof(int32_t), kAlign);
    e->part_lse_off = align_up(e->part_o_off + (size_t)total_max * Qn * D * sizeof(float), kAlign);
    e->ws_size = align_up(e->part_lse_off + (size_t)total_max * Qn * sizeof(float), kAlign);
  } else if (e->kind == KIND_DECODE) {
    // Keys per chunk (the same for one-byte codes, which measured best at
    // this length too).
    const int64_t chunk = kDecodeChunk;
    int64_t total_chunks = 0;
    for (int64_t b = 0; b < B; ++b) {
      int32_t* r = &e->meta[(size_t)b * fia::BF_COUNT];
      int64_t lo = 0, hi = 0;
      if (qlen[b] >= 1) visible(mode, 0, qlen[b], kvlen[b], p->pre_tokens, p->next_tokens, &lo, &hi);
      const int64_t nch = hi > lo ? (hi + chunk - 1) / chunk - lo / chunk : 0;
      r[fia::BF_LO] = (int32_t)lo;
      r[fia::BF_HI] = (int32_t)hi;
      r[fia::BF_NCHUNK] = (int32_t)nch;
      r[fia::BF_CHUNK0] = (int32_t)total_chunks;
      total_chunks += nch;
    }
    for (int64_t b = 0; b < B; ++b) {
      const int32_t nch = e->meta[(size_t)b * fia::BF_COUNT + fia::BF_NCHUNK];
      for (int32_t c = 0; c < nch; ++c) {
        e->meta.push_back((int32_t)b);
        e->meta.push_back(c);
      }
    }
    a.chunk = (int32_t)chunk;
    set_head_split(a, KVn);
    const int64_t n_items = total_chunks * (a.kv_pair ? KVn / 2 : KVn) * a.n_head_blocks;
    if (n_items > INT32_MAX) {
      delete e;
      return fail(FIA_ERR_UNSUPPORTED, "too many decode work items");
    }
    e->n_items = (int32_t)n_items;
    a.n_work = (int32_t)total_chunks;
    e->meta_bytes = e->meta.size() * sizeof(int32_t);
    e->part_o_off = 0;
    e->part_lse_off = align_up((size_t)total_chunks * Qn * D * sizeof(float), kAlign);
    e->ws_size = align_up(e->part_lse_off + (size_t)total_chunks * Qn * sizeof(float), kAlign);
  }
  if (e->kind != KIND_DECODE) {
    e->meta_bytes = e->meta.size() * sizeof(int32_t);
    e->part_o_off = e->part_lse_off = 0;
    e->ws_size = 0;
  }
  *workspace_size = e->ws_size;
  *executor = e;
  return FIA_SUCCESS;
}

namespace {

// Sub-chunks of 64 slots per sparse workgroup.  Fixed (not derived from the
// batch), so that a row's chunk boundaries, and with them its result, depend
// only on its own slot count.
constexpr int kSparseSubPerChunk = 2;

// Query, output and index checks shared by both sparse operators.  Fills the
// query / output / index / length fields of `a`.
struct SparseShape {
  bool tnd = false;
  int64_t B = 0, S1 = 0, n_rows = 0, N1 = 0;
};

fia_status sparse_query(const fia_tensor* q, const fia_tensor* attention_out,
                        const fia_tensor* cu_seqlens_q, const fia_tensor* seqused_kv, bool tnd,
                        int want_dtype, SparseShape* sh, SparseArgs* a) {
  fia_status st;
  // TND packs the query tokens of all batch entries into T1 rows; the batch
  // count then comes from seqused_kv and the row split from cu_seqlens_q.
  if (q->ndim != (tnd ? 3 : 4)) {
    return fail(FIA_ERR_PARAM_INVALID, tnd ? "q must be [T1, N1, 512] for TND" : "q must be [B, S1, N1, 512]");
  }
  if (seqused_kv->dtype != FIA_DT_INT32 || seqused_kv->ndim != 1) {
    return fail(FIA_ERR_PARAM_INVALID, "seqused_kv must be int32 [B]");
  }
  sh->tnd = tnd;
  sh->B = tnd ? seqused_kv->shape[0] : q->shape[0];
  sh->S1 = tnd ? 1 : q->shape[1];
  sh->n_rows = tnd ? q->shape[0] : sh->B * sh->S1;
  sh->N1 = q->shape[tnd ? 1 : 2];
  if (q->shape[q->ndim - 1] != fia::kSparseD) return fail(FIA_ERR_PARAM_INVALID, "q head dim must be 512");
  if (sh->B < 1) return fail(FIA_ERR_PARAM_INVALID, "batch must be >= 1");
  if (!tnd && sh->S1 < 1) return fail(FIA_ERR_PARAM_INVALID, "query length must be >= 1");
  if (sh->n_rows > 65535) return fail(FIA_ERR_UNSUPPORTED, "B * S1 (or T1) must be <= 65535");
  if (seqused_kv->shape[0] != sh->B) return fail(FIA_ERR_PARAM_INVALID, "seqused_kv must be int32 [B]");
  bool out_ok = attention_out->dtype == want_dtype && attention_out->ndim == q->ndim;
  for (int d = 0; out_ok && d < q->ndim; ++d) out_ok = attention_out->shape[d] == q->shape[d];
  if (!out_ok) {
    return fail(FIA_ERR_PARAM_INVALID, std::string("attention_out must be ") + dtype_name(want_dtype) +
                                           " with the shape of q");
  }
  if (tnd) {
    if (cu_seqlens_q == nullptr) return fail(FIA_ERR_PARAM_INVALID, "TND requires cu_seqlens_q");
    if ((st = check_tensor(cu_seqlens_q, "cu_seqlens_q")) != FIA_SUCCESS) return st;
    if (cu_seqlens_q->dtype != FIA_DT_INT32 || cu_seqlens_q->ndim != 1 ||
        cu_seqlens_q->shape[0] != sh->B + 1 || cu_seqlens_q->stride[0] != 1) {
      return fail(FIA_ERR_PARAM_INVALID, "cu_seqlens_q must be contiguous int32 [B + 1]");
    }
  } else if (cu_seqlens_q != nullptr) {
    return fail(FIA_ERR_PARAM_INVALID, "cu_seqlens_q is only for layout_q TND");
  }
  for (int d = 0; d + 1 < q->ndim; ++d) {
    if (q->stride[d] % 8 || attention_out->stride[d] % 8) {
      return fail(FIA_ERR_UNSUPPORTED, "q / attention_out rows must be 16-byte aligned");
    }
  }
  if (q->stride[q->ndim - 1] != 1 || attention_out->stride[q->ndim - 1] != 1 ||
      reinterpret_cast<uintptr_t>(q->data) % 16 || reinterpret_cast<uintptr_t>(attention_out->data) % 16) {
    return fail(FIA_ERR_UNSUPPORTED, "q / attention_out rows must be 16-byte aligned");
  }
  a->q = static_cast<const uint16_t*>(q->data);
  a->q_sb = tnd ? 0 : q->stride[0];
  a->q_ss = q->stride[tnd ? 0 : 1];
  a->q_sh = q->stride[tnd ? 1 : 2];
  a->o = static_cast<uint16_t*>(attention_out->data);
  a->o_sb = tnd ? 0 : attention_out->stride[0];
  a->o_ss = attention_out->stride[tnd ? 0 : 1];
  a->o_sh = attention_out->stride[tnd ? 1 : 2];
  a->cu_q = tnd ? static_cast<const int32_t*>(cu_seqlens_q->data) : nullptr;
  a->n_rows = (int32_t)sh->n_rows;
  a->seqused = static_cast<const int32_t*>(seqused_kv->data);
  a->B = (int32_t)sh->B;
  a->S1 = (int32_t)sh->S1;
  a->N1 = (int32_t)sh->N1;
  return FIA_SUCCESS;
}

// cmp_sparse_indices: int32 [B, S1, 1, K2] (BSND) or [T1, 1, K2] (TND), rows
// contiguous.  Returns K2 through *K2.
fia_status sparse_indices(const fia_tensor* t, const SparseShape& sh, int64_t* K2, SparseArgs* a) {
  fia_status st = check_tensor(t, "cmp_sparse_indices");
  if (st != FIA_SUCCESS) return st;
  const bool shape_ok = sh.tnd ? (t->ndim == 3 && t->shape[0] == sh.n_rows && t->shape[1] == 1)
                               : (t->ndim == 4 && t->shape[0] == sh.B && t->shape[1] == sh.S1 &&
                                  t->shape[2] == 1);
  if (t->dtype != FIA_DT_INT32 || !shape_ok) {
    return fail(FIA_ERR_PARAM_INVALID, sh.tnd ? "cmp_sparse_indices must be int32 [T1, 1, K2]"
                                              : "cmp_sparse_indices must be int32 [B, S1, 1, K2]");
  }
  if (t->stride[t->ndim - 1] != 1) {
    return fail(FIA_ERR_PARAM_INVALID, "cmp_sparse_indices rows must be contiguous");
  }
  *K2 = t->shape[t->ndim - 1];
  a->idx = static_cast<const int32_t*>(t->data);
  a->idx_sb = sh.tnd ? 0 : t->stride[0];
  a->idx_ss = sh.tnd ? t->stride[0] : t->stride[1];
  return FIA_SUCCESS;
}

// Block table of a paged pool: int32 [B, cols], cols >= `need`.
fia_status sparse_block_table(const fia_tensor* t, const char* name, int64_t B, int64_t need,
                              fia::SparsePool* pd) {
  fia_status st = check_tensor(t, name);
  if (st != FIA_SUCCESS) return st;
  if (t->dtype != FIA_DT_INT32 || t->ndim != 2 || t->shape[0] != B || t->shape[1] == 0) {
    return fail(FIA_ERR_PARAM_INVALID, std::string(name) + " must be int32 [B, cols]");
  }
  if (t->shape[1] < need) {
    return fail(FIA_ERR_PARAM_INVALID, std::string(name) + " has fewer columns than the longest "
                                                          "sequence needs");
  }
  if (t->shape[1] > INT32_MAX) return fail(FIA_ERR_UNSUPPORTED, std::string(name) + " too wide");
  pd->bt = static_cast<const int32_t*>(t->data);
  pd->bt_sb = t->stride[0];
  pd->bt_cols = (int32_t)t->shape[1];
  return FIA_SUCCESS;
}

// Slots, work split and workspace of a planned sparse executor (the
// per-row slot count is n_win_slots + K2).
fia_status sparse_finish(fia_executor* e, int64_t K2, size_t* workspace_size, fia_executor** executor) {
  SparseArgs& a = e->sp;
  a.K2 = (int32_t)K2;
  a.n_win_slots = (int32_t)align_up((size_t)(a.win_left + a.win_right + 1), fia::kSparseSub);
  a.n_slots = a.n_win_slots + a.K2;
  a.sub_per_chunk = kSparseSubPerChunk;
  const int64_t per_chunk = (int64_t)fia::kSparseSub * a.sub_per_chunk;
  const int64_t n_chunks = (a.n_slots + per_chunk - 1) / per_chunk;
  if (n_chunks > fia::kSparseMaxChunks) {
    delete e;
    return fail(FIA_ERR_UNSUPPORTED, "too many key rows per query token (window + K2 must be <= " +
                                         std::to_string(fia::kSparseMaxChunks * per_chunk) + ")");
  }
  a.n_chunks = (int32_t)n_chunks;
  {
    const int64_t hs = fia::kSparseHeadsSmall;
    const int64_t wg_small = (int64_t)a.n_rows * n_chunks * ((a.N1 + hs - 1) / hs);
    a.hb_heads = (a.N1 <= hs || wg_small <= fia::kSparseCUs) ? fia::kSparseHeadsSmall : fia::kSparseHeadsLarge;
  }
  a.n_hb = (a.N1 + a.hb_heads - 1) / a.hb_heads;
  a.xcd_rows = (a.n_rows % 8 == 0) ? 1 : 0;
  if ((int64_t)a.n_rows * a.n_hb * a.n_chunks > INT32_MAX) {
    delete e;
    return fail(FIA_ERR_UNSUPPORTED, "too many sparse work items");
  }
  const size_t rows = (size_t)a.n_rows;
  e->part_o_off = 0;
  e->part_lse_off = 0;
  e->ws_size = 0;
  if (n_chunks > 1) {
    e->part_lse_off = align_up(rows * n_chunks * a.N1 * fia::kSparseD * sizeof(float), kAlign);
    e->ws_size = align_up(e->part_lse_off + rows * n_chunks * a.N1 * sizeof(float), kAlign);
  }
  *workspace_size = e->ws_size;
  *executor = e;
  return FIA_SUCCESS;
}

}  // namespace

fia_status fia_sparse_get_workspace_size(const fia_sparse_params* p, const fia_tensor* q,
                                         const fia_tensor* ori_kv, const fia_tensor* cmp_kv,
                                         const fia_tensor* ori_sparse_indices,
                                         const fia_tensor* cmp_sparse_indices,
                                         const fia_tensor* ori_block_table,
                                         const fia_tensor* cmp_block_table,
                                         const fia_tensor* cu_seqlens_q,
                                         const fia_tensor* seqused_kv, int64_t max_seqused_kv,
                                         const fia_tensor* sinks, const fia_tensor* metadata,
                                         const fia_tensor* attention_out, size_t* workspace_size,
                                         fia_executor** executor) {
  (void)metadata;
  if (!p || !q || !ori_kv || !ori_block_table || !seqused_kv || !sinks || !attention_out ||
      !workspace_size || !executor) {
    return fail(FIA_ERR_NULLPTR, "params, q, ori_kv, ori_block_table, seqused_kv, sinks, "
                                 "attention_out, workspace_size and executor must not be NULL");
  }
  *executor = nullptr;
  *workspace_size = 0;
  fia_status st;
  const fia_tensor* must[] = {q, ori_kv, ori_block_table, seqused_kv, sinks, attention_out};
  const char* names[] = {"q", "ori_kv", "ori_block_table", "seqused_kv", "sinks", "attention_out"};
  for (int i = 0; i < 6; ++i) {
    if ((st = check_tensor(must[i], names[i])) != FIA_SUCCESS) return st;
  }
  const std::string lq = p->layout_q ? p->layout_q : "BSND";
  const std::string lkv = p->layout_kv ? p->layout_kv : "PA_ND";
  if (lq != "BSND" && lq != "TND") return fail(FIA_ERR_PARAM_INVALID, "layout_q must be BSND or TND");
  const bool tnd = lq == "TND";
  if (lkv != "PA_ND") return fail(FIA_ERR_PARAM_INVALID, "layout_kv must be PA_ND");
  if (p->kv_quant_mode != 1) return fail(FIA_ERR_PARAM_INVALID, "kv_quant_mode must be 1 (per-tile)");
  if (p->tile_size != 64) return fail(FIA_ERR_PARAM_INVALID, "tile_size must be 64");
  if (p->rope_head_dim != 64) return fail(FIA_ERR_PARAM_INVALID, "rope_head_dim must be 64");
  if (p->ori_mask_mode != 4) return fail(FIA_ERR_PARAM_INVALID, "ori_mask_mode must be 4 (band)");
  if (p->ori_win_left != 127 || p->ori_win_right != 0) {
    return fail(FIA_ERR_PARAM_INVALID, "ori_win_left must be 127 and ori_win_right 0");
  }
  if (p->return_softmax_lse) return fail(FIA_ERR_PARAM_INVALID, "return_softmax_lse is reserved");
  if (ori_sparse_indices != nullptr) return fail(FIA_ERR_PARAM_INVALID, "ori_sparse_indices is reserved");
  if (q->dtype != FIA_DT_BF16) return fail(FIA_ERR_PARAM_INVALID, "q must be bf16");
  SparseArgs a{};
  SparseShape sh;
  if ((st = sparse_query(q, attention_out, cu_seqlens_q, seqused_kv, tnd, FIA_DT_BF16, &sh, &a)) !=
      FIA_SUCCESS) {
    return st;
  }
  if (sh.N1 != 64 && sh.N1 != 128) return fail(FIA_ERR_PARAM_INVALID, "q heads must be 64 or 128");
  auto check_pool = [&](const fia_tensor* t, const char* name, fia::SparsePool* pd) -> fia_status {
    if (t->dtype != FIA_DT_UINT8 && t->dtype != FIA_DT_FP8_E4M3FN && t->dtype != FIA_DT_INT8) {
      return fail(FIA_ERR_PARAM_INVALID, std::string(name) + " must be a byte tensor (fp8 packed rows)");
    }
    const bool four = t->ndim == 4 && t->shape[2] == 1 && t->shape[3] == fia::kRowBytes;
    const bool three = t->ndim == 3 && t->shape[2] == fia::kRowBytes;
    if (!four && !three) {
      return fail(FIA_ERR_PARAM_INVALID, std::string(name) + " must be [n_blocks, block_size, 1, 640]");
    }
    if (t->shape[1] % 16 != 0 || t->shape[1] > 1024 || t->shape[1] <= 0) {
      return fail(FIA_ERR_PARAM_INVALID, std::string(name) + ": block_size must be a multiple of 16, <= 1024");
    }
    if (t->stride[0] % 16 != 0 || t->stride[1] % 16 != 0 || reinterpret_cast<uintptr_t>(t->data) % 16 != 0) {
      return fail(FIA_ERR_UNSUPPORTED, std::string(name) + ": rows must be 16-byte aligned");
    }
    if (t->shape[0] < 1 || t->shape[0] > INT32_MAX) {
      return fail(FIA_ERR_PARAM_INVALID, std::string(name) + ": bad block count");
    }
    pd->base = static_cast<const uint8_t*>(t->data);
    pd->paged = 1;
    pd->nb = (int32_t)t->shape[0];
    pd->bs = (int32_t)t->shape[1];
    pd->sb = t->stride[0];
    pd->ss = t->stride[1];
    return FIA_SUCCESS;
  };
  if ((st = check_pool(ori_kv, "ori_kv", &a.ori)) != FIA_SUCCESS) return st;
  const bool has_cmp = cmp_kv != nullptr;
  if (has_cmp) {
    if ((st = check_tensor(cmp_kv, "cmp_kv")) != FIA_SUCCESS) return st;
    if ((st = check_pool(cmp_kv, "cmp_kv", &a.cmp)) != FIA_SUCCESS) return st;
    if (cmp_kv->dtype != ori_kv->dtype) return fail(FIA_ERR_PARAM_INVALID, "ori_kv and cmp_kv dtypes differ");
    // CSA: top-k indices into a ratio-4 compressed sequence; HCA: no indices,
    // every row of a ratio-128 compressed sequence.
    if (cmp_sparse_indices != nullptr && p->cmp_ratio != 4) {
      return fail(FIA_ERR_PARAM_INVALID, "cmp_ratio must be 4 with cmp_sparse_indices (compressed-sparse)");
    }
    if (cmp_sparse_indices == nullptr && p->cmp_ratio != 128) {
      return fail(FIA_ERR_PARAM_INVALID, "cmp_ratio must be 128 without cmp_sparse_indices "
                                         "(heavily compressed)");
    }
    if (p->cmp_mask_mode != 3) return fail(FIA_ERR_PARAM_INVALID, "cmp_mask_mode must be 3");
    if (cmp_block_table == nullptr) return fail(FIA_ERR_PARAM_INVALID, "cmp_kv needs cmp_block_table");
  } else {
    if (cmp_sparse_indices != nullptr) return fail(FIA_ERR_PARAM_INVALID, "cmp_sparse_indices needs cmp_kv");
    if (p->cmp_ratio != 1) return fail(FIA_ERR_PARAM_INVALID, "cmp_ratio must be 1 without compressed KV");
  }
  int64_t K2 = 0;
  if (cmp_sparse_indices != nullptr) {
    if ((st = sparse_indices(cmp_sparse_indices, sh, &K2, &a)) != FIA_SUCCESS) return st;
    if (K2 != 512 && K2 != 1024) return fail(FIA_ERR_PARAM_INVALID, "K2 must be 512 or 1024");
  }
  if (max_seqused_kv < 0) return fail(FIA_ERR_PARAM_INVALID, "max_seqused_kv must be >= 0");
  if ((st = sparse_block_table(ori_block_table, "ori_block_table", sh.B,
                               (max_seqused_kv + a.ori.bs - 1) / a.ori.bs, &a.ori)) != FIA_SUCCESS) {
    return st;
  }
  const bool hca = has_cmp && cmp_sparse_indices == nullptr;
  if (has_cmp) {
    const int64_t ncmp = max_seqused_kv / p->cmp_ratio;
    if ((st = sparse_block_table(cmp_block_table, "cmp_block_table", sh.B,
                                 (ncmp + a.cmp.bs - 1) / a.cmp.bs, &a.cmp)) != FIA_SUCCESS) {
      return st;
    }
    // Heavily compressed: one slot per compressed row of the longest sequence.
    if (hca) K2 = (int64_t)align_up((size_t)ncmp, fia::kSparseSub);
  }
  if (sinks->dtype != FIA_DT_FP32 || sinks->ndim != 1 || sinks->shape[0] != sh.N1) {
    return fail(FIA_ERR_PARAM_INVALID, "sinks must be fp32 [N1]");
  }
  fia_executor* e = new fia_executor();
  e->kind = KIND_SPARSE;
  a.fmt = fia::SF_FP8_PACKED;
  a.sinks = static_cast<const float*>(sinks->data);
  a.cmp_ratio = p->cmp_ratio;
  a.win_left = p->ori_win_left;
  a.win_right = p->ori_win_right;
  a.has_cmp = has_cmp ? 1 : 0;
  a.cmp_direct = hca ? 1 : 0;
  a.scale_log2 = (float)(p->softmax_scale * 1.4426950408889634);
  e->sp = a;
  return sparse_finish(e, K2, workspace_size, executor);
}

fia_status fia_sparse_flash_mla_get_workspace_size(
    const fia_sfmla_params* p, const fia_tensor* q, const fia_tensor* ori_kv,
    const fia_tensor* cmp_kv, const fia_tensor* ori_sparse_indices,
    const fia_tensor* cmp_sparse_indices, const fia_tensor* ori_block_table,
    const fia_tensor* cmp_block_table, const fia_tensor* cu_seqlens_q,
    const fia_tensor* cu_seqlens_ori_kv, const fia_tensor* cu_seqlens_cmp_kv,
    const fia_tensor* seqused_q, const fia_tensor* seqused_kv, int64_t max_seqused_kv,
    const fia_tensor* sinks, const fia_tensor* metadata, const fia_tensor* attention_out,
    const fia_tensor* softmax_lse, size_t* workspace_size, fia_executor** executor) {
  (void)metadata;
  if (!p || !q || !ori_kv || !seqused_kv || !attention_out || !workspace_size || !executor) {
    return fail(FIA_ERR_NULLPTR, "params, q, ori_kv, seqused_kv, attention_out, workspace_size "
                                 "and executor must not be NULL");
  }
  *executor = nullptr;
  *workspace_size = 0;
  fia_status st;
  const fia_tensor* must[] = {q, ori_kv, seqused_kv, attention_out};
  const char* names[] = {"q", "ori_kv", "seqused_kv", "attention_out"};
  for (int i = 0; i < 4; ++i) {
    if ((st = check_tensor(must[i], names[i])) != FIA_SUCCESS) return st;
  }
  const std::string lq = p->layout_q ? p->layout_q : "BSND";
  const std::string lkv = p->layout_kv ? p->layout_kv : "PA_BBND";
  if (lq != "BSND" && lq != "TND") return fail(FIA_ERR_PARAM_INVALID, "layout_q must be BSND or TND");
  const bool tnd = lq == "TND";
  // Layout pairs: BSND / BSND, TND / TND, BSND / PA_BBND, TND / PA_BBND.
  const bool paged = lkv == "PA_BBND";
  if (!paged && lkv != lq) {
    return fail(FIA_ERR_PARAM_INVALID, "layout_kv must be PA_BBND or equal layout_q");
  }
  if (p->ori_mask_mode != 4) return fail(FIA_ERR_PARAM_INVALID, "ori_mask_mode must be 4 (band)");
  if (p->ori_win_left != 127 || p->ori_win_right != 0) {
    return fail(FIA_ERR_PARAM_INVALID, "ori_win_left must be 127 and ori_win_right 0");
  }
  if (ori_sparse_indices != nullptr) return fail(FIA_ERR_PARAM_INVALID, "ori_sparse_indices is reserved");
  if (seqused_q != nullptr) return fail(FIA_ERR_PARAM_INVALID, "seqused_q is reserved");
  if (q->dtype != FIA_DT_BF16 && q->dtype != FIA_DT_FP16) {
    return fail(FIA_ERR_PARAM_INVALID, "q must be fp16 or bf16");
  }
  SparseArgs a{};
  SparseShape sh;
  if ((st = sparse_query(q, attention_out, cu_seqlens_q, seqused_kv, tnd, q->dtype, &sh, &a)) !=
      FIA_SUCCESS) {
    return st;
  }
  if (sh.N1 < 1 || sh.N1 > 128 || (sh.N1 & (sh.N1 - 1)) != 0) {
    return fail(FIA_ERR_PARAM_INVALID, "q heads must be a power of two in 1..128");
  }
  const bool has_cmp = cmp_kv != nullptr;
  // Modes (sparse_flash_mla SWA / CSA / HCA constraints).
  if (!has_cmp) {
    if (p->cmp_ratio != 1) return fail(FIA_ERR_PARAM_INVALID, "SWA (no cmp_kv) needs cmp_ratio 1");
    if (cmp_sparse_indices || cmp_block_table || cu_seqlens_cmp_kv) {
      return fail(FIA_ERR_PARAM_INVALID, "SWA takes no cmp_sparse_indices, cmp_block_table or "
                                         "cu_seqlens_cmp_kv");
    }
    if (p->cmp_mask_mode != 0) return fail(FIA_ERR_PARAM_INVALID, "SWA needs cmp_mask_mode 0");
  } else {
    if (p->cmp_mask_mode != 3) return fail(FIA_ERR_PARAM_INVALID, "cmp_mask_mode must be 3");
    if (cmp_sparse_indices != nullptr && p->cmp_ratio != 4) {
      return fail(FIA_ERR_PARAM_INVALID, "CSA (cmp_sparse_indices) needs cmp_ratio 4");
    }
    if (cmp_sparse_indices == nullptr && p->cmp_ratio != 128) {
      return fail(FIA_ERR_PARAM_INVALID, "HCA (cmp_kv without indices) needs cmp_ratio 128");
    }
  }
  // One pool: PA_BBND [n_blocks, block_size, 1, 512], BSND [B, S2, 1, 512]
  // or TND [T2, 1, 512] (cumulative row offsets in cu).
  auto check_pool = [&](const fia_tensor* t, const fia_tensor* bt, const fia_tensor* cu,
                        const char* name, int64_t max_rows, fia::SparsePool* pd) -> fia_status {
    fia_status s2 = check_tensor(t, name);
    if (s2 != FIA_SUCCESS) return s2;
    const std::string nm = name;
    if (t->dtype != q->dtype) return fail(FIA_ERR_PARAM_INVALID, nm + " must have the dtype of q");
    const int nd = tnd && !paged ? 3 : 4;
    if (t->ndim != nd || t->shape[nd - 2] != 1 || t->shape[nd - 1] != fia::kSparseD) {
      return fail(FIA_ERR_PARAM_INVALID,
                  nm + (paged ? " must be [n_blocks, block_size, 1, 512]"
                              : (tnd ? " must be [T2, 1, 512]" : " must be [B, S2, 1, 512]")));
    }
    for (int d = 0; d + 2 < nd; ++d) {
      if (t->stride[d] % 8 != 0) return fail(FIA_ERR_UNSUPPORTED, nm + ": rows must be 16-byte aligned");
    }
    if (reinterpret_cast<uintptr_t>(t->data) % 16 != 0) {
      return fail(FIA_ERR_UNSUPPORTED, nm + ": rows must be 16-byte aligned");
    }
    pd->base = static_cast<const uint8_t*>(t->data);
    pd->paged = paged ? 1 : 0;
    if (paged) {
      if (bt == nullptr) return fail(FIA_ERR_PARAM_INVALID, nm + " in PA_BBND needs its block table");
      if (cu != nullptr) return fail(FIA_ERR_PARAM_INVALID, "cu_seqlens_*_kv is only for layout_kv TND");
      if (t->shape[1] < 1 || t->shape[1] > 1024) {
        return fail(FIA_ERR_PARAM_INVALID, nm + ": block_size must be 1..1024");
      }
      if (t->shape[0] < 1 || t->shape[0] > INT32_MAX) return fail(FIA_ERR_PARAM_INVALID, nm + ": bad block count");
      pd->nb = (int32_t)t->shape[0];
      pd->bs = (int32_t)t->shape[1];
      pd->sb = t->stride[0] * 2;
      pd->ss = t->stride[1] * 2;
      return sparse_block_table(bt, (nm == "ori_kv") ? "ori_block_table" : "cmp_block_table", sh.B,
                                (max_rows + pd->bs - 1) / pd->bs, pd);
    }
    if (bt != nullptr) return fail(FIA_ERR_PARAM_INVALID, "block tables are only for layout_kv PA_BBND");
    if (tnd) {
      if (cu == nullptr) return fail(FIA_ERR_PARAM_INVALID, nm + " in TND needs its cu_seqlens");
      if ((s2 = check_tensor(cu, "cu_seqlens_kv")) != FIA_SUCCESS) return s2;
      if (cu->dtype != FIA_DT_INT32 || cu->ndim != 1 || cu->shape[0] != sh.B + 1 || cu->stride[0] != 1) {
        return fail(FIA_ERR_PARAM_INVALID, "cu_seqlens_ori_kv / cu_seqlens_cmp_kv must be contiguous "
                                           "int32 [B + 1]");
      }
      if (t->shape[0] < 1) return fail(FIA_ERR_PARAM_INVALID, nm + " holds no rows");
      pd->cu = static_cast<const int32_t*>(cu->data);
      pd->sb = 0;
      pd->ss = t->stride[0] * 2;
      pd->n_rows = t->shape[0];
      return FIA_SUCCESS;
    }
    if (cu != nullptr) return fail(FIA_ERR_PARAM_INVALID, "cu_seqlens_*_kv is only for layout_kv TND");
    if (t->shape[0] != sh.B || t->shape[1] < 1) {
      return fail(FIA_ERR_PARAM_INVALID, nm + " must be [B, S2, 1, 512] with S2 >= 1");
    }
    pd->sb = t->stride[0] * 2;
    pd->ss = t->stride[1] * 2;
    pd->n_rows = t->shape[1];
    return FIA_SUCCESS;
  };
  if (max_seqused_kv < 0) return fail(FIA_ERR_PARAM_INVALID, "max_seqused_kv must be >= 0");
  if ((st = check_pool(ori_kv, ori_block_table, cu_seqlens_ori_kv, "ori_kv", max_seqused_kv, &a.ori)) !=
      FIA_SUCCESS) {
    return st;
  }
  int64_t K2 = 0;
  if (has_cmp) {
    const int64_t ncmp = max_seqused_kv / p->cmp_ratio;
    if ((st = check_pool(cmp_kv, cmp_block_table, cu_seqlens_cmp_kv, "cmp_kv", ncmp, &a.cmp)) !=
        FIA_SUCCESS) {
      return st;
    }
    if (cmp_sparse_indices != nullptr) {
      if ((st = sparse_indices(cmp_sparse_indices, sh, &K2, &a)) != FIA_SUCCESS) return st;
      if (K2 < 1) return fail(FIA_ERR_PARAM_INVALID, "K2 must be >= 1");
    } else {
      K2 = (int64_t)align_up((size_t)ncmp, fia::kSparseSub);
    }
  }
  if (sinks != nullptr) {
    if ((st = check_tensor(sinks, "sinks")) != FIA_SUCCESS) return st;
    if (sinks->dtype != FIA_DT_FP32 || sinks->ndim != 1 || sinks->shape[0] != sh.N1 || sinks->stride[0] != 1) {
      return fail(FIA_ERR_PARAM_INVALID, "sinks must be contiguous fp32 [N1]");
    }
    a.sinks = static_cast<const float*>(sinks->data);
  }
  if (p->return_softmax_lse) {
    if (softmax_lse == nullptr) return fail(FIA_ERR_NULLPTR, "return_softmax_lse needs softmax_lse");
    if ((st = check_tensor(softmax_lse, "softmax_lse")) != FIA_SUCCESS) return st;
    // softmax_lse [B, N2, S1, N1 / N2] (BSND) or [N2, T1, N1 / N2] (TND), N2 = 1.
    const fia_tensor* t = softmax_lse;
    const bool ok = t->dtype == FIA_DT_FP32 &&
                    (tnd ? (t->ndim == 3 && t->shape[0] == 1 && t->shape[1] == sh.n_rows && t->shape[2] == sh.N1)
                         : (t->ndim == 4 && t->shape[0] == sh.B && t->shape[1] == 1 && t->shape[2] == sh.S1 &&
                            t->shape[3] == sh.N1));
    if (!ok) {
      return fail(FIA_ERR_PARAM_INVALID, tnd ? "softmax_lse must be fp32 [1, T1, N1]"
                                             : "softmax_lse must be fp32 [B, 1, S1, N1]");
    }
    a.lse = static_cast<float*>(t->data);
    a.lse_sb = tnd ? 0 : t->stride[0];
    a.lse_ss = tnd ? t->stride[1] : t->stride[2];
    a.lse_sh = t->stride[t->ndim - 1];
  }
  fia_executor* e = new fia_executor();
  e->kind = KIND_SPARSE;
  a.fmt = q->dtype == FIA_DT_FP16 ? fia::SF_FP16 : fia::SF_BF16;
  a.cmp_ratio = p->cmp_ratio;
  a.win_left = p->ori_win_left;
  a.win_right = p->ori_win_right;
  a.has_cmp = has_cmp ? 1 : 0;
  a.cmp_direct = (has_cmp && cmp_sparse_indices == nullptr) ? 1 : 0;
  a.scale_log2 = (float)(p->softmax_scale * 1.4426950408889634);
  e->sp = a;
  return sparse_finish(e, K2, workspace_size, executor);
}

namespace {

// Enqueue the kernels of a bound executor (plan and workspace pointers set).
fia_status launch_all(fia_executor* e, void* workspace, hipStream_t s) {
  hipError_t err = hipSuccess;
  switch (e->kind) {
    case KIND_FILL: err = fia::launch_fill_empty(e->a, s); break;
    case KIND_FP32: err = fia::launch_attn_fp32(e->a, s); break;
    case KIND_PREFILL: err = fia::launch_prefill_bf16(e->a, s); break;
    case KIND_DECODE:
      if (e->dev_len) {
        uint8_t* base = static_cast<uint8_t*>(workspace);
        err = fia::launch_decode_partition(e->a, reinterpret_cast<int32_t*>(base + e->dev_meta_off),
                                           reinterpret_cast<int32_t*>(base + e->dev_work_off), s);
        if (err != hipSuccess) break;
      }
      err = e->a.kvq ? fia::launch_decode_q8(e->a, e->n_items, s)
                     : fia::launch_decode_bf16(e->a, e->n_items, s);
      if (err == hipSuccess) err = fia::launch_decode_merge(e->a, s);
      break;
    case KIND_SPARSE:
      err = fia::launch_sparse(e->sp, s);
      if (err == hipSuccess) err = fia::launch_sparse_merge(e->sp, s);
      break;
    default: return fail(FIA_ERR_PARAM_INVALID, "corrupt executor");
  }
  if (err != hipSuccess) return fail(FIA_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(err));
  return FIA_SUCCESS;
}

}  // namespace

fia_status fia_run(void* workspace, size_t workspace_size, fia_executor* e, void* stream) {
  if (e == nullptr) return fail(FIA_ERR_NULLPTR, "executor is NULL");
  if (e->noop) return FIA_SUCCESS;
  fia_status st = check_ws(e, workspace, workspace_size);
  if (st != FIA_SUCCESS) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = upload_plan(e)) != FIA_SUCCESS) return st;
  bind_workspace(e, workspace);
  return launch_all(e, workspace, s);
}


fia_status fia_debug_gather_kv(fia_executor* e, void* workspace, size_t workspace_size,
                               int32_t which, void* dst, void* stream) {
  if (e == nullptr || dst == nullptr) return fail(FIA_ERR_NULLPTR, "executor and dst must not be NULL");
  if (e->noop || e->kind == KIND_SPARSE || e->kind == KIND_FILL) {
    return fail(FIA_ERR_PARAM_INVALID, "executor has no key/value rows to gather");
  }
  if (e->dev_len) return fail(FIA_ERR_PARAM_INVALID, "executor reads its KV lengths on the device");
  if (which != 0 && which != 1) return fail(FIA_ERR_PARAM_INVALID, "which must be 0 or 1");
  fia_status st = check_ws(e, workspace, workspace_size);
  if (st != FIA_SUCCESS) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = upload_plan(e)) != FIA_SUCCESS) return st;
  bind_workspace(e, workspace);
  hipError_t err = fia::launch_debug_gather(e->a, which, dst, e->s2max, s);
  if (err != hipSuccess) return fail(FIA_ERR_HIP, std::string("gather launch failed: ") + hipGetErrorString(err));
  return FIA_SUCCESS;
}

fia_status fia_debug_read_kv(fia_executor* e, void* workspace, size_t workspace_size, int32_t order,
                             uint32_t* out, int64_t* out_len, void* stream) {
  if (e == nullptr || out_len == nullptr) return fail(FIA_ERR_NULLPTR, "executor and out_len must not be NULL");
  if (e->noop || e->kind != KIND_DECODE || e->dev_len) {
    return fail(FIA_ERR_PARAM_INVALID, "fia_debug_read_kv needs a split-KV decode executor planned on the host");
  }
  if (order != 0 && order != 1) return fail(FIA_ERR_PARAM_INVALID, "order must be 0 or 1");
  const int64_t grid = fia::decode_read_grid(e->a, order);
  if (grid < 0) {
    return fail(FIA_ERR_UNSUPPORTED, order == 0 ? "read order 0 needs D * element size of 128 or 256 bytes"
                                                : "read order 1 needs adjacent heads and KV_N * D * element "
                                                  "size of 1024 or 2048 bytes");
  }
  if (out == nullptr) {
    *out_len = grid;
    return FIA_SUCCESS;
  }
  if (*out_len < grid) return fail(FIA_ERR_PARAM_INVALID, "out holds fewer words than the read writes");
  fia_status st = check_ws(e, workspace, workspace_size);
  if (st != FIA_SUCCESS) return st;
  if ((st = upload_plan(e)) != FIA_SUCCESS) return st;
  bind_workspace(e, workspace);
  hipError_t err = fia::launch_decode_read(e->a, order, out, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(FIA_ERR_HIP, std::string("read launch failed: ") + hipGetErrorString(err));
  *out_len = grid;
  return FIA_SUCCESS;
}

fia_status fia_debug_sparse_rows(fia_executor* e, void* workspace, size_t workspace_size,
                                 int32_t* ids_out, uint8_t* rows_out, int32_t* n_slots_out,
                                 void* stream) {
  if (e == nullptr) return fail(FIA_ERR_NULLPTR, "executor is NULL");
  if (e->kind != KIND_SPARSE) return fail(FIA_ERR_PARAM_INVALID, "not a sparse executor");
  if (n_slots_out) *n_slots_out = e->sp.n_slots;
  if (ids_out == nullptr) return FIA_SUCCESS;
  if (rows_out == nullptr) return fail(FIA_ERR_NULLPTR, "rows_out must not be NULL");
  fia_status st = check_ws(e, workspace, workspace_size);
  if (st != FIA_SUCCESS) return st;
  bind_workspace(e, workspace);
  hipError_t err = fia::launch_debug_sparse_rows(e->sp, ids_out, rows_out, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(FIA_ERR_HIP, std::string("launch failed: ") + hipGetErrorString(err));
  return FIA_SUCCESS;
}

}  // extern "C"

namespace fia {

void set_last_error(const char* msg) { g_last_error = msg; }

// fia_run with the plan and the workspace in caller-given device scratch:
// the plan (per-batch records and work list) is copied to `plan` on the
// stream, the workspace is `ws`.  Nothing is allocated.
fia_status run_on_scratch(fia_executor* e, void* plan, size_t plan_cap, void* ws, size_t ws_cap,
                          void* stream) {
  if (e == nullptr) return fail(FIA_ERR_NULLPTR, "executor is NULL");
  if (e->noop) return FIA_SUCCESS;
  if (e->meta_bytes > plan_cap) {
    return fail(FIA_ERR_UNSUPPORTED, "the executor's plan (" + std::to_string(e->meta_bytes) +
                                         " bytes) exceeds the no-allocation plan area of " +
                                         std::to_string(plan_cap) + " bytes");
  }
  if (e->ws_size > ws_cap) {
    return fail(FIA_ERR_UNSUPPORTED, "the executor's workspace (" + std::to_string(e->ws_size) +
                                         " bytes) exceeds the no-allocation scratch of " +
                                         std::to_string(ws_cap) + " bytes");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (e->meta_bytes > 0) {
    if (hipMemcpyAsync(plan, e->meta.data(), e->meta_bytes, hipMemcpyHostToDevice, s) != hipSuccess) {
      return fail(FIA_ERR_HIP, "copy of the plan into the scratch failed");
    }
  }
  bind_workspace(e, ws);
  if (!e->dev_len) {
    e->a.meta = static_cast<const int32_t*>(plan);
    e->a.work = static_cast<const int32_t*>(plan) + e->work_off;
  }
  const fia_status st = launch_all(e, ws, s);
  // Later fia_run calls bind their own plan copy again.
  return st;
}

}  // namespace fia
