// Host-side launchers shared between the libmsa translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

// attn.hip: compute units of the current device (cached per device)
int device_cus();

// index_topk.hip
hipError_t launch_index_pool(const void* q_idx, const void* k_idx, int64_t q_start, int64_t Nq,
                             int H_kv, int d_idx, float* P, int64_t ldp, hipStream_t stream);
hipError_t launch_topk_prefill(const float* P, int64_t ldp, int64_t q_start, int64_t Nq,
                               int H_kv, int k, int32_t* sel, hipStream_t stream);
hipError_t launch_topk_decode(const float* P, int64_t ldp, int B, int H_kv, int nblk, int k,
                              int32_t* sel, hipStream_t stream);
hipError_t launch_index_topk_fused(const void* q_idx, const void* k_idx, int64_t q_start,
                                   int64_t Nq, int H_kv, int d_idx, int k, int32_t* sel,
                                   hipStream_t stream);

// csr.hip
size_t invert_scratch_bytes(int64_t Nq, int H_kv, int nblk);
hipError_t launch_invert(const int32_t* sel, int64_t q_start, int64_t Nq, int H_kv, int k,
                         int nblk, int32_t* row_ptr, int32_t* col, uint8_t* slot,
                         void* scratch, hipStream_t stream);

// attn.hip
int attn_max_chunk();
int64_t attn_max_items(int64_t nb, int64_t nnz, int chunk);
hipError_t launch_build_items(const int32_t* row_ptr, int64_t nb, int nblk, int64_t q_start,
                              int64_t Nq, int chunk, bool with_local, int4* items,
                              int32_t* n_items, hipStream_t stream);
hipError_t launch_attn(const void* Q, const void* K, const void* V, const int32_t* col,
                       const uint8_t* slot, const int4* items, int32_t* n_items,
                       int64_t max_items, int64_t q_start, int64_t Nq, int64_t Nk, int H_q,
                       int H_kv, int d_h, int nblk, int k, float scale, void* Os, float* lse_s,
                       hipStream_t stream);
hipError_t launch_combine(const void* Q, const void* K, const void* V, const void* Os,
                          const float* lse_s, int64_t q_start, int64_t Nq, int64_t Nk, int H_q,
                          int H_kv, int d_h, int k, float scale, float* O, float* lse,
                          hipStream_t stream);

// attn_bwd.hip
struct BwdBounds {
  int64_t max_units;   // work units (bucket slices)
  int64_t max_splits;  // buckets split over several units
  int64_t max_slices;  // fp32 dK/dV partials of split buckets
};
int bwd_unit_positions(int G);
BwdBounds bwd_bounds(int64_t nb, int64_t nnz, int G);
hipError_t launch_attn_bwd(const void* Q, const void* K, const void* V, const float* O,
                           const float* lse, const void* dO, const int32_t* row_ptr,
                           const int32_t* col, const uint8_t* slot, int4* units,
                           int32_t* n_units, int4* splits, int32_t* n_splits,
                           const BwdBounds& bounds, int64_t q_start, int64_t Nq, int64_t Nk,
                           int H_q, int H_kv, int d_h, int nblk, int k, float scale,
                           float* Dbuf, void* dq_part, float* kvpart, float* dQ, float* dK,
                           float* dV, hipStream_t stream);

// frontend.hip
hipError_t launch_index_frontend(const void* hidden, const void* Wq, const void* Wk,
                                 const float* gq, const float* gk, int64_t N, int64_t pos0,
                                 int d_model, int H_kv, int d_idx, int rope_dim,
                                 double log2_theta, float eps, void* q_idx, void* k_idx,
                                 hipStream_t stream);

// kl.hip
int64_t kl_sum_partials(int64_t n);
hipError_t launch_index_kl(const void* Q, const void* K, const void* q_idx, const void* k_idx,
                           const float* lse, const int32_t* col, const uint8_t* slot,
                           const int4* items, int32_t* n_items, int64_t max_items,
                           int64_t q_start, int64_t Nq, int64_t Nk, int H_q, int H_kv, int d_h,
                           int d_idx, int nblk, int k, float scale, float* part, float* kl,
                           double* sums, double* kl_sum, hipStream_t stream);

// decode.hip
hipError_t launch_decode_scan(const void* q_idx, const void* k_idx, int B, int64_t N, int H_kv,
                              int d_idx, int nblk, float* P, int64_t ldp, hipStream_t stream);
hipError_t launch_decode_attn(const void* q, const void* K, const void* V, const int32_t* sel,
                              int B, int64_t N, int H_q, int H_kv, int d_h, int k, float scale,
                              float* Opart, float* lse_part, hipStream_t stream);
hipError_t launch_decode_merge(const float* Opart, const float* lse_part, int B, int H_q,
                               int d_h, int k, int n_sel, float* O, float* lse,
                               hipStream_t stream);

}  // namespace msa
