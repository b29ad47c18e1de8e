// C ABI of libmsa: argument validation, workspace layout and the launch
// sequence of each entry point.  Every check runs on the host before any
// work is enqueued; nothing here allocates device memory or synchronises.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <string>

#include "../../include/msa.h"
#include "msa_internal.h"

namespace {

thread_local std::string g_err;
// Tuning knobs.  Each entry point reads them once, when it starts, and
// uses that snapshot throughout; no workspace size depends on them.
std::atomic<int64_t> g_opt_fused{1};
std::atomic<int64_t> g_opt_chunk{1024};

constexpr int kB = 128;
constexpr size_t kAlign = 256;
// Smallest accepted KV-outer work item: work lists are sized for it, so a
// workspace fits every item size the option can take.
constexpr int kMinItem = 128;

struct Opts {
  bool fused;  // Index Branch as one fused kernel
  int item;    // query positions per KV-outer work item
};

Opts opts_now() {
  return Opts{g_opt_fused.load(std::memory_order_relaxed) != 0,
              (int)g_opt_chunk.load(std::memory_order_relaxed)};
}

msa_status fail(msa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

msa_status ok() {
  g_err.clear();
  return MSA_OK;
}

msa_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MSA_OK;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Sub-allocator over a caller-provided workspace.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* p) : base(static_cast<char*>(p)) {}
  template <typename T>
  T* take(size_t bytes) {
    T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
    off = align_up(off + bytes);
    return p;
  }
};

int64_t nnz_of(int64_t q_start, int64_t Nq, int H_kv, int B_k, int k) {
  // sum over i of min(k, i/B_k + 1): positions with lb < k-1 contribute
  // lb+1, the rest k.
  int64_t tot = 0;
  const int64_t q_end = q_start + Nq;
  const int64_t full_from = (int64_t)(k - 1) * B_k;  // first i with lb >= k-1
  for (int64_t b = q_start / B_k; b * B_k < min(q_end, full_from); ++b) {
    const int64_t lo = max(q_start, b * B_k), hi = min(q_end, min((b + 1) * B_k, full_from));
    if (hi > lo) tot += (hi - lo) * (b + 1);
  }
  if (q_end > full_from) tot += (q_end - max(q_start, full_from)) * k;
  return tot * H_kv;
}

msa_status check_common(int64_t q_start, int64_t Nq, int H_kv, int B_k, int k) {
  if (q_start < 0 || Nq < 1) return fail(MSA_ERR_INVALID_ARG, "need q_start >= 0 and Nq >= 1");
  if (H_kv < 1) return fail(MSA_ERR_INVALID_ARG, "H_kv must be >= 1");
  if (H_kv > 64) return fail(MSA_ERR_UNSUPPORTED, "H_kv > 64 is not supported");
  if (B_k != kB) return fail(MSA_ERR_UNSUPPORTED, "only B_k = 128 is supported (got %d)", B_k);
  if (k < 1 || k > 32) return fail(MSA_ERR_UNSUPPORTED, "k must be in [1, 32] (got %d)", k);
  const int64_t nblk = cdiv(q_start + Nq, B_k);
  if (nblk > 16384) return fail(MSA_ERR_UNSUPPORTED, "more than 16384 key blocks");
  if (nnz_of(q_start, Nq, H_kv, B_k, k) >= (int64_t)1 << 31)
    return fail(MSA_ERR_UNSUPPORTED, "selection nnz >= 2^31: use smaller query chunks");
  return MSA_OK;
}

// ---------------------------------------------------------------- index
size_t index_ws(int64_t q_start, int64_t Nq, int H_kv) {
  const int64_t nblk = cdiv(q_start + Nq, kB);
  const int64_t ldp = cdiv(nblk, 4) * 4;
  return align_up(sizeof(float) * (size_t)(H_kv * Nq * ldp));
}

msa_status run_index_topk(const void* q_idx, const void* k_idx, int64_t q_start, int64_t Nq,
                          int H_kv, int d_idx, int k, int32_t* sel, void* ws, bool fused,
                          hipStream_t s) {
  if (fused)
    return hip_status(
        msa::launch_index_topk_fused(q_idx, k_idx, q_start, Nq, H_kv, d_idx, k, sel, s),
        "index/top-k (fused) launch");
  const int64_t nblk = cdiv(q_start + Nq, kB);
  const int64_t ldp = cdiv(nblk, 4) * 4;
  float* P = static_cast<float*>(ws);
  msa_status st = hip_status(
      msa::launch_index_pool(q_idx, k_idx, q_start, Nq, H_kv, d_idx, P, ldp, s),
      "index score launch");
  if (st) return st;
  return hip_status(msa::launch_topk_prefill(P, ldp, q_start, Nq, H_kv, k, sel, s),
                    "top-k launch");
}

// ---------------------------------------------------------------- invert
size_t invert_ws(int64_t q_start, int64_t Nq, int H_kv) {
  const int nblk = (int)cdiv(q_start + Nq, kB);
  return align_up(msa::invert_scratch_bytes(Nq, H_kv, nblk));
}

// ---------------------------------------------------------------- attention
struct AttnWs {
  int4* items;
  int32_t* n_items;
  void* Os;      // bf16 non-local partials [Nq*(k-1) + 1][H_kv][d_h/4][G][4]
  float* lse_s;  // their log-sum-exps [Nq*(k-1) + 1][H_q]
  int64_t max_items;
  size_t bytes;
};

AttnWs attn_layout(void* ws, int64_t q_start, int64_t Nq, int H_q, int H_kv, int d_h, int k) {
  const int64_t nblk = cdiv(q_start + Nq, kB);
  const int64_t nnz = nnz_of(q_start, Nq, H_kv, kB, k);
  AttnWs w;
  Carve c(ws);
  w.max_items = msa::attn_max_items((int64_t)H_kv * nblk, nnz, kMinItem);
  w.items = c.take<int4>(sizeof(int4) * (size_t)w.max_items);
  w.n_items = c.take<int32_t>(2 * sizeof(int32_t));  // count, fetch counter
  // Nq * (k-1) slots plus one spare that rows past a work item's end write.
  w.Os = c.take<void>(2 * ((size_t)Nq * (k - 1) + 1) * H_q * d_h);
  w.lse_s = c.take<float>(sizeof(float) * ((size_t)Nq * (k - 1) + 1) * H_q);
  w.bytes = c.off;
  return w;
}

msa_status check_attn_shapes(int H_q, int H_kv, int d_h) {
  if (H_q < 1 || H_q % H_kv) return fail(MSA_ERR_INVALID_ARG, "H_q must be a positive multiple of H_kv");
  if (H_q / H_kv > 64)
    return fail(MSA_ERR_UNSUPPORTED, "at most 64 query heads per KV head (got %d)", H_q / H_kv);
  if (d_h != 64 && d_h != 128) return fail(MSA_ERR_UNSUPPORTED, "d_h must be 64 or 128 (got %d)", d_h);
  return MSA_OK;
}

msa_status run_attn(const void* Q, const void* K, const void* V, const int32_t* row_ptr,
                    const int32_t* col, const uint8_t* slot, int64_t q_start, int64_t Nq,
                    int64_t Nk, int H_q, int H_kv, int d_h, int k, float scale, float* O,
                    float* lse, void* ws, int item, hipStream_t s) {
  const int nblk = (int)cdiv(q_start + Nq, kB);
  AttnWs w = attn_layout(ws, q_start, Nq, H_q, H_kv, d_h, k);
  msa_status st = hip_status(msa::launch_build_items(row_ptr, (int64_t)H_kv * nblk, nblk,
                                                     q_start, Nq, item, false, w.items,
                                                     w.n_items, s),
                             "work-list launch");
  if (st) return st;
  st = hip_status(msa::launch_attn(Q, K, V, col, slot, w.items, w.n_items, w.max_items, q_start,
                                   Nq, Nk, H_q, H_kv, d_h, nblk, k, scale, w.Os, w.lse_s, s),
                  "attention launch");
  if (st) return st;
  return hip_status(msa::launch_combine(Q, K, V, w.Os, w.lse_s, q_start, Nq, Nk, H_q, H_kv, d_h,
                                        k, scale, O, lse, s),
                    "combine launch");
}

msa_status check_index_dims(int d_idx) {
  if (d_idx != 32 && d_idx != 64 && d_idx != 128)
    return fail(MSA_ERR_UNSUPPORTED, "d_idx must be 32, 64 or 128 (got %d)", d_idx);
  return MSA_OK;
}

// ---------------------------------------------------------------- prefill
struct PrefillWs {
  int32_t* sel;  // chunk buffer when the caller passes no sel
  int32_t* row_ptr;
  int32_t* col;
  uint8_t* slot;
  void* shared;
  size_t bytes;
};

// Workspace for the query positions [q_begin, q_end) of one sequence, in
// chunks of `chunk` positions.
PrefillWs prefill_layout(void* ws, int64_t q_begin, int64_t q_end, int64_t chunk, int H_q,
                         int H_kv, int d_h, int k, bool own_sel) {
  const int64_t nblk = cdiv(q_end, kB);
  int64_t nnz_max = 0;
  size_t shared = 0;
  for (int64_t q0 = q_begin; q0 < q_end; q0 += chunk) {
    const int64_t nq = std::min(chunk, q_end - q0);
    nnz_max = std::max(nnz_max, nnz_of(q0, nq, H_kv, kB, k));
    shared = std::max(shared, index_ws(q0, nq, H_kv));
    shared = std::max(shared, invert_ws(q0, nq, H_kv));
    shared = std::max(shared, attn_layout(nullptr, q0, nq, H_q, H_kv, d_h, k).bytes);
  }
  PrefillWs w;
  Carve c(ws);
  w.sel = own_sel ? c.take<int32_t>(sizeof(int32_t) * (size_t)chunk * H_kv * k) : nullptr;
  w.row_ptr = c.take<int32_t>(sizeof(int32_t) * (size_t)(H_kv * nblk + 1));
  w.col = c.take<int32_t>(sizeof(int32_t) * (size_t)nnz_max);
  w.slot = c.take<uint8_t>((size_t)nnz_max);
  w.shared = c.take<void>(shared);
  w.bytes = c.off;
  return w;
}

// The three stages over query positions [q_begin, q_end) of one sequence
// whose keys are rows 0..Nk-1.  Q and q_idx are bases addressed by absolute
// position (rows below q_begin are never touched); sel, O and lse point at
// the row of position q_begin.
msa_status prefill_span(const void* Q, const void* K, const void* V, const void* q_idx,
                        const void* k_idx, int64_t q_begin, int64_t q_end, int64_t Nk,
                        int64_t chunk, int H_q, int H_kv, int d_h, int d_idx, int k, float scale,
                        int32_t* sel, float* O, float* lse, const PrefillWs& w, const Opts& o,
                        hipStream_t s) {
  // The fused Index Branch keeps no per-chunk state, so when the caller's
  // sel holds the whole span it runs once over all of it: its work-groups,
  // heaviest first, then balance across what would be separate chunk
  // launches (the early chunks alone leave most of the GPU idle).
  const bool whole_index = o.fused && sel != nullptr;
  if (whole_index) {
    msa_status st = run_index_topk(q_idx, k_idx, q_begin, q_end - q_begin, H_kv, d_idx, k, sel,
                                   nullptr, true, s);
    if (st) return st;
  }
  for (int64_t q0 = q_begin; q0 < q_end; q0 += chunk) {
    const int64_t nq = std::min(chunk, q_end - q0), off = q0 - q_begin;
    int32_t* sel_c = sel ? sel + off * H_kv * k : w.sel;
    if (!whole_index) {
      msa_status st =
          run_index_topk(q_idx, k_idx, q0, nq, H_kv, d_idx, k, sel_c, w.shared, o.fused, s);
      if (st) return st;
    }
    msa_status st;
    const int nblk = (int)cdiv(q0 + nq, kB);
    st = hip_status(msa::launch_invert(sel_c, q0, nq, H_kv, k, nblk, w.row_ptr, w.col, w.slot,
                                       w.shared, s),
                    "inverted-index launch");
    if (st) return st;
    st = run_attn(Q, K, V, w.row_ptr, w.col, w.slot, q0, nq, Nk, H_q, H_kv, d_h, k, scale,
                  O + off * H_q * d_h, lse ? lse + off * H_q : nullptr, w.shared, o.item, s);
    if (st) return st;
  }
  return MSA_OK;
}

// A base pointer for rows addressed by absolute position when the buffer
// starts at row `first` (only rows >= first are ever read through it).
const void* row_base(const void* p, int64_t first, int64_t row_elems, size_t elem) {
  return static_cast<const char*>(p) - first * row_elems * (int64_t)elem;
}

// ---------------------------------------------------------------- decode
struct DecodeWs {
  float* P;
  int64_t ldp;
  float* Opart;
  float* lse_part;
  size_t bytes;
};

DecodeWs decode_layout(void* ws, int B, int64_t N, int H_q, int H_kv, int d_h, int k) {
  const int64_t nblk = cdiv(N, kB);
  DecodeWs w;
  Carve c(ws);
  w.ldp = cdiv(nblk, 4) * 4;
  w.P = c.take<float>(sizeof(float) * (size_t)B * H_kv * w.ldp);
  w.Opart = c.take<float>(sizeof(float) * (size_t)B * H_q * k * d_h);
  w.lse_part = c.take<float>(sizeof(float) * (size_t)B * H_q * k);
  w.bytes = c.off;
  return w;
}

}  // namespace

extern "C" {

const char* msa_last_error(void) { return g_err.c_str(); }

int64_t msa_selection_nnz(int64_t q_start, int64_t Nq, int H_kv, int B_k, int k) {
  if (q_start < 0 || Nq < 0 || H_kv < 1 || B_k < 1 || k < 1) return -1;
  return nnz_of(q_start, Nq, H_kv, B_k, k);
}

size_t msa_index_topk_workspace_bytes(int64_t q_start, int64_t Nq, int H_kv, int B_k, int k) {
  if (check_common(q_start, Nq, H_kv, B_k, k)) return 0;
  return index_ws(q_start, Nq, H_kv);
}

msa_status msa_index_topk(const void* q_idx, const void* k_idx, int64_t q_start, int64_t Nq,
                          int64_t Nk, int H_kv, int d_idx, int B_k, int k, int32_t* sel,
                          void* ws, size_t ws_bytes, void* stream) {
  if (msa_status st = check_common(q_start, Nq, H_kv, B_k, k)) return st;
  if (msa_status st = check_index_dims(d_idx)) return st;
  if (!q_idx || !k_idx || !sel) return fail(MSA_ERR_INVALID_ARG, "null q_idx, k_idx or sel");
  if (Nk < q_start + Nq) return fail(MSA_ERR_INVALID_ARG, "Nk must be >= q_start + Nq");
  const Opts o = opts_now();
  if (!o.fused && (!ws || ws_bytes < index_ws(q_start, Nq, H_kv)))
    return fail(MSA_ERR_WORKSPACE, "workspace needs %zu bytes", index_ws(q_start, Nq, H_kv));
  msa_status st = run_index_topk(q_idx, k_idx, q_start, Nq, H_kv, d_idx, k, sel, ws, o.fused,
                                 static_cast<hipStream_t>(stream));
  return st ? st : ok();
}

size_t msa_invert_index_workspace_bytes(int64_t q_start, int64_t Nq, int H_kv, int B_k, int k) {
  if (check_common(q_start, Nq, H_kv, B_k, k)) return 0;
  return invert_ws(q_start, Nq, H_kv);
}

msa_status msa_invert_index(const int32_t* sel, int64_t q_start, int64_t Nq, int H_kv, int B_k,
                            int k, int32_t* row_ptr, int32_t* col, uint8_t* slot, void* ws,
                            size_t ws_bytes, void* stream) {
  if (msa_status st = check_common(q_start, Nq, H_kv, B_k, k)) return st;
  if (!sel || !row_ptr || !col || !slot)
    return fail(MSA_ERR_INVALID_ARG, "null sel, row_ptr, col or slot");
  if (!ws || ws_bytes < invert_ws(q_start, Nq, H_kv))
    return fail(MSA_ERR_WORKSPACE, "workspace needs %zu bytes", invert_ws(q_start, Nq, H_kv));
  const int nblk = (int)cdiv(q_start + Nq, B_k);
  msa_status st = hip_status(msa::launch_invert(sel, q_start, Nq, H_kv, k, nblk, row_ptr, col,
                                                slot, ws, static_cast<hipStream_t>(stream)),
                             "inverted-index launch");
  return st ? st : ok();
}

size_t msa_sparse_attn_fwd_workspace_bytes(int64_t q_start, int64_t Nq, int H_q, int H_kv,
                                           int d_h, int B_k, int k) {
  if (check_common(q_start, Nq, H_kv, B_k, k) || check_attn_shapes(H_q, H_kv, d_h)) return 0;
  return attn_layout(nullptr, q_start, Nq, H_q, H_kv, d_h, k).bytes;
}

msa_status msa_sparse_attn_fwd(const void* Q, const void* K, const void* V,
                               const int32_t* row_ptr, const int32_t* col, const uint8_t* slot,
                               int64_t q_start, int64_t Nq, int64_t Nk, int H_q, int H_kv,
                               int d_h, int B_k, int k, float scale, float* O, float* lse,
                               void* ws, size_t ws_bytes, void* stream) {
  if (msa_status st = check_common(q_start, Nq, H_kv, B_k, k)) return st;
  if (msa_status st = check_attn_shapes(H_q, H_kv, d_h)) return st;
  if (!Q || !K || !V || !row_ptr || !col || !slot || !O)
    return fail(MSA_ERR_INVALID_ARG, "null Q, K, V, row_ptr, col, slot or O");
  if (Nk < q_start + Nq) return fail(MSA_ERR_INVALID_ARG, "Nk must be >= q_start + Nq");
  if (!(scale > 0.f)) return fail(MSA_ERR_INVALID_ARG, "scale must be > 0");
  const size_t need = attn_layout(nullptr, q_start, Nq, H_q, H_kv, d_h, k).bytes;
  if (!ws || ws_bytes < need) return fail(MSA_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  msa_status st = run_attn(Q, K, V, row_ptr, col, slot, q_start, Nq, Nk, H_q, H_kv, d_h, k,
                           scale, O, lse, ws, opts_now().item, static_cast<hipStream_t>(stream));
  return st ? st : ok();
}

// ---------------------------------------------------------------- backward
struct BwdWs {
  int4* units;
  int32_t* n_units;
  int4* splits;
  int32_t* n_splits;
  float* D;       // dO . O per (row, head)
  void* dq_part;  // bf16 dQ partials [Nq*k + 1][H_kv][d_h/4][G][4]
  float* kvpart;  // fp32 dK/dV partials of split buckets [slice][2][B_k][d_h]
  msa::BwdBounds bounds;
  size_t bytes;
};

BwdWs bwd_layout(void* ws, int64_t q_start, int64_t Nq, int H_q, int H_kv, int d_h, int k) {
  const int64_t nblk = cdiv(q_start + Nq, kB);
  const int64_t nnz = nnz_of(q_start, Nq, H_kv, kB, k);
  BwdWs w;
  Carve c(ws);
  w.bounds = msa::bwd_bounds((int64_t)H_kv * nblk, nnz, H_q / H_kv);
  w.units = c.take<int4>(sizeof(int4) * (size_t)w.bounds.max_units);
  w.n_units = c.take<int32_t>(2 * sizeof(int32_t));
  w.splits = c.take<int4>(sizeof(int4) * (size_t)w.bounds.max_splits);
  w.n_splits = c.take<int32_t>(sizeof(int32_t));
  w.D = c.take<float>(sizeof(float) * (size_t)Nq * H_q);
  w.dq_part = c.take<void>(2 * ((size_t)Nq * k + 1) * H_q * d_h);
  w.kvpart = c.take<float>(sizeof(float) * 2 * kB * (size_t)d_h * w.bounds.max_slices);
  w.bytes = c.off;
  return w;
}

size_t msa_sparse_attn_bwd_workspace_bytes(int64_t q_start, int64_t Nq, int H_q, int H_kv,
                                           int d_h, int B_k, int k) {
  if (check_common(q_start, Nq, H_kv, B_k, k) || check_attn_shapes(H_q, H_kv, d_h)) return 0;
  return bwd_layout(nullptr, q_start, Nq, H_q, H_kv, d_h, k).bytes;
}

msa_status msa_sparse_attn_bwd(const void* Q, const void* K, const void* V, const float* O,
                               const float* lse, const void* dO, const int32_t* row_ptr,
                               const int32_t* col, const uint8_t* slot, int64_t q_start,
                               int64_t Nq, int64_t Nk, int H_q, int H_kv, int d_h, int B_k,
                               int k, float scale, float* dQ, float* dK, float* dV, void* ws,
                               size_t ws_bytes, void* stream) {
  if (msa_status st = check_common(q_start, Nq, H_kv, B_k, k)) return st;
  if (msa_status st = check_attn_shapes(H_q, H_kv, d_h)) return st;
  if (!Q || !K || !V || !O || !lse || !dO || !row_ptr || !col || !slot || !dQ || !dK || !dV)
    return fail(MSA_ERR_INVALID_ARG, "null Q, K, V, O, lse, dO, row_ptr, col, slot, dQ, dK or dV");
  if (Nk < q_start + Nq) return fail(MSA_ERR_INVALID_ARG, "Nk must be >= q_start + Nq");
  if (!(scale > 0.f)) return fail(MSA_ERR_INVALID_ARG, "scale must be > 0");
  const size_t need = bwd_layout(nullptr, q_start, Nq, H_q, H_kv, d_h, k).bytes;
  if (!ws || ws_bytes < need) return fail(MSA_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  BwdWs w = bwd_layout(ws, q_start, Nq, H_q, H_kv, d_h, k);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nblk = (int)cdiv(q_start + Nq, kB);
  msa_status st = hip_status(
      msa::launch_attn_bwd(Q, K, V, O, lse, dO, row_ptr, col, slot, w.units, w.n_units,
                           w.splits, w.n_splits, w.bounds, q_start, Nq, Nk, H_q, H_kv, d_h, nblk,
                           k, scale, w.D, w.dq_part, w.kvpart, dQ, dK, dV, s),
      "backward launch");
  return st ? st : ok();
}

// ---------------------------------------------------------------- index KL
struct KlWs {
  int4* items;
  int32_t* n_items;
  float* part;   // per (query, group, slot): sum t ln t, sum t s, ln sum exp s
  double* sums;  // per 4096 (query, group) values, for the deterministic total
  int64_t max_items;
  size_t bytes;
};

KlWs kl_layout(void* ws, int64_t q_start, int64_t Nq, int H_kv, int k) {
  const int64_t nblk = cdiv(q_start + Nq, kB);
  const int64_t nnz = nnz_of(q_start, Nq, H_kv, kB, k);
  KlWs w;
  Carve c(ws);
  w.max_items = msa::attn_max_items((int64_t)H_kv * nblk, nnz, kMinItem);
  w.items = c.take<int4>(sizeof(int4) * (size_t)w.max_items);
  w.n_items = c.take<int32_t>(2 * sizeof(int32_t));
  w.part = c.take<float>(sizeof(float) * 3 * (size_t)Nq * H_kv * k);
  w.sums = c.take<double>(sizeof(double) * (size_t)msa::kl_sum_partials(Nq * H_kv));
  w.bytes = c.off;
  return w;
}

size_t msa_index_kl_workspace_bytes(int64_t q_start, int64_t Nq, int H_kv, int B_k, int k) {
  if (check_common(q_start, Nq, H_kv, B_k, k)) return 0;
  return kl_layout(nullptr, q_start, Nq, H_kv, k).bytes;
}

msa_status msa_index_kl(const void* Q, const void* K, const void* q_idx, const void* k_idx,
                        const float* lse, const int32_t* row_ptr, const int32_t* col,
                        const uint8_t* slot, int64_t q_start, int64_t Nq, int64_t Nk, int H_q,
                        int H_kv, int d_h, int d_idx, int B_k, int k, float scale, float* kl,
                        double* kl_sum, void* ws, size_t ws_bytes, void* stream) {
  if (msa_status st = check_common(q_start, Nq, H_kv, B_k, k)) return st;
  if (msa_status st = check_attn_shapes(H_q, H_kv, d_h)) return st;
  if (msa_status st = check_index_dims(d_idx)) return st;
  if (!Q || !K || !q_idx || !k_idx || !lse || !row_ptr || !col || !slot || !kl)
    return fail(MSA_ERR_INVALID_ARG, "null Q, K, q_idx, k_idx, lse, row_ptr, col, slot or kl");
  if (Nk < q_start + Nq) return fail(MSA_ERR_INVALID_ARG, "Nk must be >= q_start + Nq");
  if (!(scale > 0.f)) return fail(MSA_ERR_INVALID_ARG, "scale must be > 0");
  const size_t need = kl_layout(nullptr, q_start, Nq, H_kv, k).bytes;
  if (!ws || ws_bytes < need) return fail(MSA_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  KlWs w = kl_layout(ws, q_start, Nq, H_kv, k);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nblk = (int)cdiv(q_start + Nq, kB);
  msa_status st = hip_status(msa::launch_build_items(row_ptr, (int64_t)H_kv * nblk, nblk, q_start,
                                                     Nq, opts_now().item, true, w.items,
                                                     w.n_items, s),
                             "work-list launch");
  if (st) return st;
  st = hip_status(msa::launch_index_kl(Q, K, q_idx, k_idx, lse, col, slot, w.items, w.n_items,
                                       w.max_items, q_start, Nq, Nk, H_q, H_kv, d_h, d_idx, nblk,
                                       k, scale, w.part, kl, w.sums, kl_sum, s),
                  "index KL launch");
  return st ? st : ok();
}

// ---------------------------------------------------------------- front-end
msa_status msa_index_frontend(const void* hidden, const void* Wq, const void* Wk,
                              const float* gq, const float* gk, int64_t N, int64_t pos0,
                              int d_model, int H_kv, int d_idx, int rope_dim, float rope_theta,
                              float eps, void* q_idx, void* k_idx, void* stream) {
  if (!hidden || !Wq || !Wk || !gq || !gk || !q_idx || !k_idx)
    return fail(MSA_ERR_INVALID_ARG, "null hidden, Wq, Wk, gq, gk, q_idx or k_idx");
  if (N < 1 || pos0 < 0) return fail(MSA_ERR_INVALID_ARG, "need N >= 1 and pos0 >= 0");
  if (N > ((int64_t)1 << 31) / 128) return fail(MSA_ERR_UNSUPPORTED, "N too large");
  if (H_kv < 1 || H_kv > 64) return fail(MSA_ERR_INVALID_ARG, "H_kv must be in [1, 64]");
  if (d_model < 64 || d_model % 64)
    return fail(MSA_ERR_UNSUPPORTED, "d_model must be a positive multiple of 64 (got %d)", d_model);
  if (d_idx != 32 && d_idx != 64 && d_idx != 128)
    return fail(MSA_ERR_UNSUPPORTED, "d_idx must be 32, 64 or 128 (got %d)", d_idx);
  if ((rope_dim != 0 && rope_dim != 32 && rope_dim != 64) || rope_dim > d_idx)
    return fail(MSA_ERR_UNSUPPORTED, "rope_dim must be 0, 32 or 64 and <= d_idx (got %d)", rope_dim);
  if (!(rope_theta > 1.f)) return fail(MSA_ERR_INVALID_ARG, "rope_theta must be > 1");
  if (!(eps >= 0.f)) return fail(MSA_ERR_INVALID_ARG, "eps must be >= 0");
  msa_status st = hip_status(
      msa::launch_index_frontend(hidden, Wq, Wk, gq, gk, N, pos0, d_model, H_kv, d_idx,
                                 rope_dim, std::log2((double)rope_theta), eps, q_idx, k_idx,
                                 static_cast<hipStream_t>(stream)),
      "front-end launch");
  return st ? st : ok();
}

size_t msa_prefill_workspace_bytes(int64_t N, int64_t chunk, int H_q, int H_kv, int d_h,
                                   int d_idx, int B_k, int k) {
  (void)d_idx;
  if (N < 1) return 0;
  if (chunk <= 0 || chunk > N) chunk = N;
  if (check_common(0, N, H_kv, B_k, k) || check_attn_shapes(H_q, H_kv, d_h)) return 0;
  return prefill_layout(nullptr, 0, N, chunk, H_q, H_kv, d_h, k, true).bytes;
}

msa_status msa_prefill(const void* Q, const void* K, const void* V, const void* q_idx,
                       const void* k_idx, int64_t N, int64_t chunk, int H_q, int H_kv, int d_h,
                       int d_idx, int B_k, int k, float scale, int32_t* sel, float* O,
                       float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (N < 1) return fail(MSA_ERR_INVALID_ARG, "N must be >= 1");
  if (chunk < 0) return fail(MSA_ERR_INVALID_ARG, "chunk must be >= 0");
  if (chunk == 0 || chunk > N) chunk = N;
  if (msa_status st = check_common(0, N, H_kv, B_k, k)) return st;
  if (msa_status st = check_attn_shapes(H_q, H_kv, d_h)) return st;
  if (msa_status st = check_index_dims(d_idx)) return st;
  if (!Q || !K || !V || !q_idx || !k_idx || !O)
    return fail(MSA_ERR_INVALID_ARG, "null Q, K, V, q_idx, k_idx or O");
  if (!(scale > 0.f)) return fail(MSA_ERR_INVALID_ARG, "scale must be > 0");
  const bool own_sel = sel == nullptr;
  const size_t need = prefill_layout(nullptr, 0, N, chunk, H_q, H_kv, d_h, k, true).bytes;
  if (!ws || ws_bytes < need) return fail(MSA_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  PrefillWs w = prefill_layout(ws, 0, N, chunk, H_q, H_kv, d_h, k, own_sel);
  msa_status st = prefill_span(Q, K, V, q_idx, k_idx, 0, N, N, chunk, H_q, H_kv, d_h, d_idx, k,
                               scale, sel, O, lse, w, opts_now(), static_cast<hipStream_t>(stream));
  return st ? st : ok();
}

size_t msa_prefill_cached_workspace_bytes(int64_t q_start, int64_t Nq, int64_t chunk, int H_q,
                                          int H_kv, int d_h, int d_idx, int B_k, int k) {
  (void)d_idx;
  if (chunk < 0 || check_common(q_start, Nq, H_kv, B_k, k) || check_attn_shapes(H_q, H_kv, d_h))
    return 0;
  if (chunk == 0 || chunk > Nq) chunk = Nq;
  return prefill_layout(nullptr, q_start, q_start + Nq, chunk, H_q, H_kv, d_h, k, true).bytes;
}

msa_status msa_prefill_cached(const void* Q, const void* K, const void* V, const void* q_idx,
                              const void* k_idx, int64_t q_start, int64_t Nq, int64_t chunk,
                              int H_q, int H_kv, int d_h, int d_idx, int B_k, int k, float scale,
                              int32_t* sel, float* O, float* lse, void* ws, size_t ws_bytes,
                              void* stream) {
  if (chunk < 0) return fail(MSA_ERR_INVALID_ARG, "chunk must be >= 0");
  if (msa_status st = check_common(q_start, Nq, H_kv, B_k, k)) return st;
  if (msa_status st = check_attn_shapes(H_q, H_kv, d_h)) return st;
  if (msa_status st = check_index_dims(d_idx)) return st;
  if (!Q || !K || !V || !q_idx || !k_idx || !O)
    return fail(MSA_ERR_INVALID_ARG, "null Q, K, V, q_idx, k_idx or O");
  if (!(scale > 0.f)) return fail(MSA_ERR_INVALID_ARG, "scale must be > 0");
  if (chunk == 0 || chunk > Nq) chunk = Nq;
  const int64_t q_end = q_start + Nq;
  const bool own_sel = sel == nullptr;
  const size_t need = prefill_layout(nullptr, q_start, q_end, chunk, H_q, H_kv, d_h, k, true).bytes;
  if (!ws || ws_bytes < need) return fail(MSA_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  PrefillWs w = prefill_layout(ws, q_start, q_end, chunk, H_q, H_kv, d_h, k, own_sel);
  msa_status st = prefill_span(row_base(Q, q_start, (int64_t)H_q * d_h, 2), K, V,
                               row_base(q_idx, q_start, (int64_t)H_kv * d_idx, 2), k_idx,
                               q_start, q_end, q_end, chunk, H_q, H_kv, d_h, d_idx, k, scale,
                               sel, O, lse, w, opts_now(), static_cast<hipStream_t>(stream));
  return st ? st : ok();
}

// Sequences of a varlen batch, validated: lengths from the host prefix sums.
msa_status check_cu_seqlens(const int64_t* cu, int B) {
  if (!cu || B < 1) return fail(MSA_ERR_INVALID_ARG, "need cu_seqlens and B >= 1");
  if (cu[0] != 0) return fail(MSA_ERR_INVALID_ARG, "cu_seqlens[0] must be 0");
  for (int b = 0; b < B; ++b)
    if (cu[b + 1] < cu[b]) return fail(MSA_ERR_INVALID_ARG, "cu_seqlens must be nondecreasing");
  if (cu[B] < 1) return fail(MSA_ERR_INVALID_ARG, "the batch holds no tokens");
  return MSA_OK;
}

size_t varlen_bytes(const int64_t* cu, int B, int64_t chunk, int H_q, int H_kv, int d_h, int k) {
  size_t need = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t L = cu[b + 1] - cu[b];
    if (L < 1) continue;
    const int64_t c = (chunk == 0 || chunk > L) ? L : chunk;
    need = std::max(need, prefill_layout(nullptr, 0, L, c, H_q, H_kv, d_h, k, true).bytes);
  }
  return need;
}

size_t msa_prefill_varlen_workspace_bytes(const int64_t* cu_seqlens, int B, int64_t chunk,
                                          int H_q, int H_kv, int d_h, int d_idx, int B_k, int k) {
  (void)d_idx;
  if (chunk < 0 || check_cu_seqlens(cu_seqlens, B)) return 0;
  for (int b = 0; b < B; ++b) {
    const int64_t L = cu_seqlens[b + 1] - cu_seqlens[b];
    if (L > 0 && check_common(0, L, H_kv, B_k, k)) return 0;
  }
  if (check_attn_shapes(H_q, H_kv, d_h)) return 0;
  return varlen_bytes(cu_seqlens, B, chunk, H_q, H_kv, d_h, k);
}

msa_status msa_prefill_varlen(const void* Q, const void* K, const void* V, const void* q_idx,
                              const void* k_idx, const int64_t* cu_seqlens, int B, int64_t chunk,
                              int H_q, int H_kv, int d_h, int d_idx, int B_k, int k, float scale,
                              int32_t* sel, float* O, float* lse, void* ws, size_t ws_bytes,
                              void* stream) {
  if (chunk < 0) return fail(MSA_ERR_INVALID_ARG, "chunk must be >= 0");
  if (msa_status st = check_cu_seqlens(cu_seqlens, B)) return st;
  for (int b = 0; b < B; ++b) {
    const int64_t L = cu_seqlens[b + 1] - cu_seqlens[b];
    if (L < 1) continue;
    if (msa_status st = check_common(0, L, H_kv, B_k, k)) return st;
  }
  if (msa_status st = check_attn_shapes(H_q, H_kv, d_h)) return st;
  if (msa_status st = check_index_dims(d_idx)) return st;
  if (!Q || !K || !V || !q_idx || !k_idx || !O)
    return fail(MSA_ERR_INVALID_ARG, "null Q, K, V, q_idx, k_idx or O");
  if (!(scale > 0.f)) return fail(MSA_ERR_INVALID_ARG, "scale must be > 0");
  const size_t need = varlen_bytes(cu_seqlens, B, chunk, H_q, H_kv, d_h, k);
  if (!ws || ws_bytes < need) return fail(MSA_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool own_sel = sel == nullptr;
  const Opts o = opts_now();
  auto at = [](const void* p, int64_t row, int64_t row_elems) {
    return static_cast<const char*>(p) + row * row_elems * 2;
  };
  for (int b = 0; b < B; ++b) {
    const int64_t t0 = cu_seqlens[b], L = cu_seqlens[b + 1] - t0;
    if (L < 1) continue;
    const int64_t c = (chunk == 0 || chunk > L) ? L : chunk;
    PrefillWs w = prefill_layout(ws, 0, L, c, H_q, H_kv, d_h, k, own_sel);
    msa_status st = prefill_span(
        at(Q, t0, (int64_t)H_q * d_h), at(K, t0, (int64_t)H_kv * d_h),
        at(V, t0, (int64_t)H_kv * d_h), at(q_idx, t0, (int64_t)H_kv * d_idx),
        at(k_idx, t0, (int64_t)H_kv * d_idx), 0, L, L, c, H_q, H_kv, d_h, d_idx, k, scale,
        own_sel ? nullptr : sel + t0 * H_kv * k, O + t0 * H_q * d_h,
        lse ? lse + t0 * H_q : nullptr, w, o, s);
    if (st) return st;
  }
  return ok();
}

// The split index scan reads whole tokens per KiB load: H_kv * d_idx must
// divide 512.
msa_status check_decode_index(int H_kv, int d_idx) {
  if (msa_status st = check_index_dims(d_idx)) return st;
  if (512 % (H_kv * d_idx))
    return fail(MSA_ERR_UNSUPPORTED, "decode needs H_kv * d_idx to divide 512 (got %d * %d)",
                H_kv, d_idx);
  return MSA_OK;
}

size_t msa_decode_workspace_bytes(int B, int64_t N, int H_q, int H_kv, int d_h, int d_idx,
                                  int B_k, int k) {
  if (B < 1 || N < 1 || check_common(0, N, H_kv, B_k, k) || check_attn_shapes(H_q, H_kv, d_h) ||
      check_decode_index(H_kv, d_idx))
    return 0;
  return decode_layout(nullptr, B, N, H_q, H_kv, d_h, k).bytes;
}

}  // extern "C"

namespace {

msa_status check_decode(const void* q, const void* q_idx, const void* K, const void* V,
                        const void* k_idx, int B, int64_t N, int H_q, int H_kv, int d_h,
                        int d_idx, int B_k, int k, float scale, const int32_t* sel,
                        const float* O) {
  if (B < 1 || N < 1) return fail(MSA_ERR_INVALID_ARG, "need B >= 1 and N >= 1");
  if (msa_status st = check_common(0, N, H_kv, B_k, k)) return st;
  if (msa_status st = check_attn_shapes(H_q, H_kv, d_h)) return st;
  if (msa_status st = check_decode_index(H_kv, d_idx)) return st;
  if (!q || !q_idx || !K || !V || !k_idx || !sel || !O)
    return fail(MSA_ERR_INVALID_ARG, "null q, q_idx, K, V, k_idx, sel or O");
  if (!(scale > 0.f)) return fail(MSA_ERR_INVALID_ARG, "scale must be > 0");
  return MSA_OK;
}

// The decode launches over a validated shape and a large-enough workspace.
// Every scratch value a kernel reads was written earlier in the same call
// (pooled scores of the scanned blocks, partials of the selected slots), so
// the workspace needs no clearing.
msa_status run_decode(const void* q, const void* q_idx, const void* K, const void* V,
                      const void* k_idx, int B, int64_t N, int H_q, int H_kv, int d_h, int d_idx,
                      int k, float scale, int32_t* sel, float* O, float* lse, void* ws,
                      hipStream_t s) {
  DecodeWs w = decode_layout(ws, B, N, H_q, H_kv, d_h, k);
  const int nblk = (int)cdiv(N, kB);
  msa_status st = MSA_OK;
  if (nblk > 1)
    st = hip_status(msa::launch_decode_scan(q_idx, k_idx, B, N, H_kv, d_idx, nblk, w.P, w.ldp, s),
                    "decode scan launch");
  if (st) return st;
  st = hip_status(msa::launch_topk_decode(w.P, w.ldp, B, H_kv, nblk, k, sel, s),
                  "decode top-k launch");
  if (st) return st;
  st = hip_status(msa::launch_decode_attn(q, K, V, sel, B, N, H_q, H_kv, d_h, k, scale, w.Opart,
                                          w.lse_part, s),
                  "decode attention launch");
  if (st) return st;
  return hip_status(msa::launch_decode_merge(w.Opart, w.lse_part, B, H_q, d_h, k,
                                            std::min(k, nblk), O, lse, s),
                    "decode merge launch");
}

// Scratch of msa_decode_static: one copy per GPU, resident until the process
// ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: kernels and copies take the address that
// hipGetSymbolAddress returns for the current device.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up once per device
// with that device current.
msa_status static_scratch(void** out) {
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess)
    return fail(MSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MSA_ERR_UNSUPPORTED, "device %d is beyond the %d the library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess || !p)
      return fail(MSA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

}  // namespace

extern "C" {

msa_status msa_decode(const void* q, const void* q_idx, const void* K, const void* V,
                      const void* k_idx, int B, int64_t N, int H_q, int H_kv, int d_h, int d_idx,
                      int B_k, int k, float scale, int32_t* sel, float* O, float* lse, void* ws,
                      size_t ws_bytes, void* stream) {
  if (msa_status st = check_decode(q, q_idx, K, V, k_idx, B, N, H_q, H_kv, d_h, d_idx, B_k, k,
                                   scale, sel, O))
    return st;
  const size_t need = decode_layout(nullptr, B, N, H_q, H_kv, d_h, k).bytes;
  if (!ws || ws_bytes < need) return fail(MSA_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  msa_status st = run_decode(q, q_idx, K, V, k_idx, B, N, H_q, H_kv, d_h, d_idx, k, scale, sel,
                             O, lse, ws, static_cast<hipStream_t>(stream));
  return st ? st : ok();
}

size_t msa_decode_static_scratch_bytes(void) { return kStaticScratchBytes; }

msa_status msa_decode_static(const void* q, const void* q_idx, const void* K, const void* V,
                             const void* k_idx, int B, int64_t N, int H_q, int H_kv, int d_h,
                             int d_idx, int B_k, int k, float scale, int32_t* sel, float* O,
                             float* lse, void* stream) {
  if (msa_status st = check_decode(q, q_idx, K, V, k_idx, B, N, H_q, H_kv, d_h, d_idx, B_k, k,
                                   scale, sel, O))
    return st;
  const size_t need = decode_layout(nullptr, B, N, H_q, H_kv, d_h, k).bytes;
  if (need > kStaticScratchBytes)
    return fail(MSA_ERR_WORKSPACE,
                "decode needs %zu bytes of scratch, more than the fixed %zu of the static "
                "entry point: use msa_decode with a workspace",
                need, kStaticScratchBytes);
  void* ws = nullptr;
  if (msa_status st = static_scratch(&ws)) return st;
  msa_status st = run_decode(q, q_idx, K, V, k_idx, B, N, H_q, H_kv, d_h, d_idx, k, scale, sel,
                             O, lse, ws, static_cast<hipStream_t>(stream));
  return st ? st : ok();
}

msa_status msa_set_option(int option, int64_t value) {
  switch (option) {
    case MSA_OPT_INDEX_FUSED:
      if (value != 0 && value != 1) return fail(MSA_ERR_INVALID_ARG, "fused must be 0 or 1");
      g_opt_fused.store(value, std::memory_order_relaxed);
      return ok();
    case MSA_OPT_ATTN_CHUNK:
      if (value < kMinItem || value > msa::attn_max_chunk())
        return fail(MSA_ERR_INVALID_ARG, "chunk must be in [%d, %d]", kMinItem,
                    msa::attn_max_chunk());
      g_opt_chunk.store(value, std::memory_order_relaxed);
      return ok();
    default:
      return fail(MSA_ERR_INVALID_ARG, "unknown option %d", option);
  }
}

int64_t msa_get_option(int option) {
  switch (option) {
    case MSA_OPT_INDEX_FUSED:
      return g_opt_fused.load(std::memory_order_relaxed);
    case MSA_OPT_ATTN_CHUNK:
      return g_opt_chunk.load(std::memory_order_relaxed);
    default:
      return -1;
  }
}

}  // extern "C"
