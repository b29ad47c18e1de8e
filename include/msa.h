/*
 * msa.h -- C ABI of libmsa, the MiniMax Sparse Attention (MSA) forward path
 * for AMD Instinct MI355X (gfx950).
 *
 * Method: "MiniMax Sparse Attention" explainer
 * (minimax-sparse-attention-danialwang.pages.dev) and the paper abstract
 * (arXiv 2606.13392).  Attention is split into an Index Branch, which
 * picks for every query position i and GQA group r a set of k key blocks
 * of B_k tokens (always including the query's own "local" block), and a
 * Main Branch, which runs exact softmax attention over the tokens of
 * those blocks only (section 02; Figure 1 caption).
 *
 * Notation (section 01, section 04): N tokens, H_q query heads, H_kv KV
 * heads (= GQA groups), G = H_q / H_kv adjacent query heads per group
 * (head h is in group floor(h / G)), head dim d_h, index dim d_idx, block
 * size B_k, k blocks per (query, group).  Positions are 0-based; query i
 * sees keys j <= i; its local block is floor(i / B_k).
 *
 * Layouts: every tensor is dense, row-major, token-major:
 *   Q [N, H_q, d_h] bf16           K, V [N, H_kv, d_h] bf16
 *   q_idx, k_idx [N, H_kv, d_idx] bf16 (one index head per group)
 *   sel [Nq, H_kv, k] int32: ascending block ids, -1 padded
 *   O [Nq, H_q, d_h] fp32          lse [Nq, H_q] fp32 (natural log)
 * All pointers are device pointers unless stated otherwise.
 *
 * Ownership: the caller owns every buffer, including the workspaces sized
 * by the *_workspace_bytes functions.  The library allocates and frees
 * nothing, never synchronises, and keeps no per-call device state; all
 * work is enqueued on `stream` (a hipStream_t; NULL = default stream).
 *
 * Errors: arguments are checked on the host before anything is enqueued.
 * A bad argument returns MSA_ERR_INVALID_ARG, an unsupported shape
 * MSA_ERR_UNSUPPORTED, a short workspace MSA_ERR_WORKSPACE, all without
 * touching the device; a failed launch returns MSA_ERR_HIP.  The reason is
 * kept per thread and read with msa_last_error().
 *
 * Supported shapes: B_k = 128; d_h in {64, 128}; d_idx in {32, 64, 128};
 * 1 <= k <= 32; H_q a multiple of H_kv with G = H_q / H_kv <= 64;
 * H_kv <= 64; every block count ceil(N / B_k) <= 16384; every selection
 * nnz < 2^31.  Row counts (Nq, N, B) are at least 1 and q_start >= 0: an
 * empty chunk is MSA_ERR_INVALID_ARG (msa_prefill_varlen alone accepts
 * empty sequences within its batch).
 *
 * Determinism: every output is bitwise identical from run to run.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int msa_status;
#define MSA_OK 0
#define MSA_ERR_INVALID_ARG (-1)
#define MSA_ERR_UNSUPPORTED (-2)
#define MSA_ERR_WORKSPACE (-3)
#define MSA_ERR_HIP (-4)

/* Message for the last non-OK status returned on this thread ("" if none).
 * The string stays valid until the next libmsa call on the thread. */
const char *msa_last_error(void);

/* Number of (query, group, selected block) entries of a selection table
 * for query positions q_start .. q_start+Nq-1: H_kv * sum_i min(k, i/B_k+1).
 * (Section 04: every query reads a fixed budget of k blocks, fewer only
 * while fewer are visible.)  Returns -1 on bad arguments. */
int64_t msa_selection_nnz(int64_t q_start, int64_t Nq, int H_kv, int B_k, int k);

/*
 * Index Branch (section 02; Figure 1 caption; section 05 part 1).
 * For each query position i in [q_start, q_start+Nq) and group r:
 *   token score   S[j] = q_idx[i,r,:] . k_idx[j,r,:]   for j <= i
 *   block score   P[b] = max of S over block b          (block max pooling)
 *   selection     sel[i-q_start, r, :] = {lb(i)} plus the k-1 earlier
 *                 blocks with the largest P, ties to the lower block id;
 *                 all visible blocks if there are at most k.
 * Selection uses the raw scores (softmax keeps their order).
 *   q_idx, k_idx: bases of full-sequence tensors [>= q_start+Nq, H_kv, d_idx]
 *   Nk:           rows available in k_idx (must be >= q_start+Nq)
 *   sel:          out, [Nq, H_kv, k] int32
 *   ws:           device workspace of >= msa_index_topk_workspace_bytes()
 */
size_t msa_index_topk_workspace_bytes(int64_t q_start, int64_t Nq, int H_kv,
                                      int B_k, int k);
msa_status msa_index_topk(const void *q_idx, const void *k_idx, int64_t q_start,
                          int64_t Nq, int64_t Nk, int H_kv, int d_idx, int B_k,
                          int k, int32_t *sel, void *ws, size_t ws_bytes,
                          void *stream);

/*
 * Inverted index (section 05 part 2: KV-outer execution gathers, for each
 * KV block, the queries that selected it).  CSR over buckets (r, b) in
 * r-major order, nblk = ceil((q_start+Nq)/B_k):
 *   row_ptr [H_kv*nblk + 1] int32: bucket start offsets, row_ptr[0] = 0
 *   col     [nnz] int32: absolute query positions, ascending in a bucket
 *   slot    [nnz] uint8: rank of b inside sel[i-q_start, r, :]
 * nnz = msa_selection_nnz(q_start, Nq, H_kv, B_k, k).  sel must be a
 * well-formed selection (as msa_index_topk writes it).
 */
size_t msa_invert_index_workspace_bytes(int64_t q_start, int64_t Nq, int H_kv,
                                        int B_k, int k);
msa_status msa_invert_index(const int32_t *sel, int64_t q_start, int64_t Nq,
                            int H_kv, int B_k, int k, int32_t *row_ptr,
                            int32_t *col, uint8_t *slot, void *ws,
                            size_t ws_bytes, void *stream);

/*
 * Main Branch, KV-outer (section 02; section 05 part 2).  For each query
 * position i in the chunk and head h (group r = h / G):
 *   O[i-q_start, h, :] = softmax over the tokens j <= i of the selected
 *   blocks of scale * Q[i,h,:].K[j,r,:], applied to V[j,r,:]
 *   lse[i-q_start, h]  = ln sum_j exp(scale * Q[i,h,:].K[j,r,:])
 * Each selected KV block is read once per work item and the queries that
 * hit it are gathered through the inverted index; per-block partial
 * results go to pre-assigned slots and a combine step merges them through
 * their log-sum-exp in ascending block order (section 05 part 2,
 * two-phase forward).
 *   Q, K, V:  bases of full-sequence tensors; Nk rows of K/V available
 *   row_ptr, col, slot: from msa_invert_index for the same chunk
 *   O:        out [Nq, H_q, d_h] fp32; lse: out [Nq, H_q] fp32, nullable
 */
size_t msa_sparse_attn_fwd_workspace_bytes(int64_t q_start, int64_t Nq, int H_q,
                                           int H_kv, int d_h, int B_k, int k);
msa_status msa_sparse_attn_fwd(const void *Q, const void *K, const void *V,
                               const int32_t *row_ptr, const int32_t *col,
                               const uint8_t *slot, int64_t q_start, int64_t Nq,
                               int64_t Nk, int H_q, int H_kv, int d_h, int B_k,
                               int k, float scale, float *O, float *lse,
                               void *ws, size_t ws_bytes, void *stream);

/*
 * Whole prefill: Index Branch, inverted index and Main Branch over query
 * chunks of `chunk` positions, each against its full causal prefix.  Each
 * query row depends only on its own prefix, so the result does not depend
 * on `chunk` (0 = one chunk).  Outputs cover the whole sequence:
 *   sel [N, H_kv, k] int32 (nullable), O [N, H_q, d_h] fp32,
 *   lse [N, H_q] fp32 (nullable).
 */
size_t msa_prefill_workspace_bytes(int64_t N, int64_t chunk, int H_q, int H_kv,
                                   int d_h, int d_idx, int B_k, int k);
msa_status msa_prefill(const void *Q, const void *K, const void *V,
                       const void *q_idx, const void *k_idx, int64_t N,
                       int64_t chunk, int H_q, int H_kv, int d_h, int d_idx,
                       int B_k, int k, float scale, int32_t *sel, float *O,
                       float *lse, void *ws, size_t ws_bytes, void *stream);

/*
 * Chunked prefill against a KV cache (section 02: each query row's
 * selection and attention range over its own causal prefix only, so a
 * sequence can be prefilled piece by piece against the keys already
 * cached): the Nq new tokens at positions q_start .. q_start+Nq-1 attend
 * causally to the cached tokens and to each other, exactly as rows
 * q_start.. of msa_prefill over the whole sequence.
 *   Q [Nq, H_q, d_h], q_idx [Nq, H_kv, d_idx]: the new tokens only
 *   K, V [q_start+Nq, H_kv, d_h], k_idx [q_start+Nq, H_kv, d_idx]: the
 *     cache with the new tokens' keys already appended
 *   sel out [Nq, H_kv, k] int32 (nullable), O out [Nq, H_q, d_h] fp32,
 *   lse out [Nq, H_q] fp32 (nullable)
 * chunk: query positions per internal pass (0 = all Nq at once).
 */
size_t msa_prefill_cached_workspace_bytes(int64_t q_start, int64_t Nq, int64_t chunk,
                                          int H_q, int H_kv, int d_h, int d_idx,
                                          int B_k, int k);
msa_status msa_prefill_cached(const void *Q, const void *K, const void *V,
                              const void *q_idx, const void *k_idx, int64_t q_start,
                              int64_t Nq, int64_t chunk, int H_q, int H_kv, int d_h,
                              int d_idx, int B_k, int k, float scale, int32_t *sel,
                              float *O, float *lse, void *ws, size_t ws_bytes,
                              void *stream);

/*
 * Varlen batched prefill (section 02, as above: sequences share nothing,
 * so each is its own causal prefill): B independent sequences packed
 * token-major.
 * Sequence b is rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of every tensor,
 * with its own positions 0..L_b-1 and its own causal prefix; it gets the
 * msa_prefill result of that sequence alone.  Sequences run one after
 * another on the stream, each in query chunks of `chunk` (0 = whole).
 *   cu_seqlens: HOST array of B+1 prefix sums, cu_seqlens[0] = 0,
 *     nondecreasing (empty sequences are skipped), cu_seqlens[B] >= 1
 *   Q [T, H_q, d_h], K, V [T, H_kv, d_h], q_idx, k_idx [T, H_kv, d_idx]
 *   bf16, T = cu_seqlens[B]; sel out [T, H_kv, k] (nullable), O out
 *   [T, H_q, d_h] fp32, lse out [T, H_q] (nullable)
 */
size_t msa_prefill_varlen_workspace_bytes(const int64_t *cu_seqlens, int B, int64_t chunk,
                                          int H_q, int H_kv, int d_h, int d_idx,
                                          int B_k, int k);
msa_status msa_prefill_varlen(const void *Q, const void *K, const void *V,
                              const void *q_idx, const void *k_idx,
                              const int64_t *cu_seqlens, int B, int64_t chunk, int H_q,
                              int H_kv, int d_h, int d_idx, int B_k, int k, float scale,
                              int32_t *sel, float *O, float *lse, void *ws,
                              size_t ws_bytes, void *stream);

/*
 * Main Branch backward (section 02: exact softmax attention over the
 * selected blocks, so its gradients are those of softmax attention on each
 * row's token set; section 03: the selection is not differentiable, so no
 * gradient reaches the Index Branch from this loss).  For query positions
 * i in [q_start, q_start+Nq), head h (group r), T = the tokens j <= i of the
 * row's selected blocks, p = the forward's probabilities (rebuilt from lse),
 * D = dO[i,h].O[i,h]:
 *   ds_j = p_j (dO[i,h].V[j,r] - D)
 *   dQ[i,h]  = scale * sum_j ds_j K[j,r]
 *   dK[j,r] += scale * ds_j Q[i,h]      dV[j,r] += p_j dO[i,h]
 * dQ rows are written; dK and dV are ADDED to (zero them before the first
 * chunk), so calling this chunk by chunk over a sequence accumulates the
 * whole sequence's gradients.  Per-(i, h, block) dQ partials are bf16 and
 * summed in ascending slot order; each key's dK/dV sums are formed in one
 * work-group, or for a block selected by many rows in fixed-size slices
 * whose fp32 partials are summed in slice order: the result is
 * deterministic.
 *   Q [., H_q, d_h], K, V [Nk, H_kv, d_h]: bf16 full-sequence bases
 *   O [Nq, H_q, d_h] fp32, lse [Nq, H_q] fp32: this chunk's forward outputs
 *   dO [Nq, H_q, d_h] bf16
 *   row_ptr, col, slot: msa_invert_index output for the same chunk
 *   dQ out [Nq, H_q, d_h] fp32; dK, dV in/out [Nk, H_kv, d_h] fp32
 */
size_t msa_sparse_attn_bwd_workspace_bytes(int64_t q_start, int64_t Nq, int H_q,
                                           int H_kv, int d_h, int B_k, int k);
msa_status msa_sparse_attn_bwd(const void *Q, const void *K, const void *V,
                               const float *O, const float *lse, const void *dO,
                               const int32_t *row_ptr, const int32_t *col,
                               const uint8_t *slot, int64_t q_start, int64_t Nq,
                               int64_t Nk, int H_q, int H_kv, int d_h, int B_k, int k,
                               float scale, float *dQ, float *dK, float *dV, void *ws,
                               size_t ws_bytes, void *stream);

/*
 * Index-alignment KL, forward value (section 03, "KL Loss"; section 05
 * part 2: the forward keeps the LSE, so the KL needs no softmax pass of its
 * own).  For query i and group r over the token set T of its selection
 * (tokens j <= i of the selected blocks):
 *   teacher t_j = (1/G) sum over the group's heads h of
 *                 exp(scale * Q[i,h,:].K[j,r,:] - lse[i,h])
 *   student u_j = softmax over T of q_idx[i,r,:].k_idx[j,r,:]
 *   kl[i-q_start, r] = sum_{j in T} t_j (ln t_j - ln u_j)
 * The teacher is normalised by the forward's lse, so pass the lse that
 * msa_sparse_attn_fwd / msa_prefill wrote for the same Q, K and selection.
 * Partials are merged per (i, r) in ascending slot order, so the result is
 * deterministic.
 *   Q [>= q_start+Nq, H_q, d_h], K [Nk, H_kv, d_h], q_idx, k_idx
 *     [., H_kv, d_idx]: full-sequence bases, bf16
 *   lse:     [Nq, H_q] fp32 (natural log), this chunk's rows
 *   row_ptr, col, slot: msa_invert_index output for the same chunk
 *   kl:      out [Nq, H_kv] fp32
 *   kl_sum:  out, nullable: one double, the sum of kl over the chunk
 *            (fixed-order reduction; divide by the row count for the mean)
 */
size_t msa_index_kl_workspace_bytes(int64_t q_start, int64_t Nq, int H_kv, int B_k, int k);
msa_status msa_index_kl(const void *Q, const void *K, const void *q_idx, const void *k_idx,
                        const float *lse, const int32_t *row_ptr, const int32_t *col,
                        const uint8_t *slot, int64_t q_start, int64_t Nq, int64_t Nk,
                        int H_q, int H_kv, int d_h, int d_idx, int B_k, int k,
                        float scale, float *kl, double *kl_sum, void *ws,
                        size_t ws_bytes, void *stream);

/*
 * Decode: one new query per sequence at the last cache row (position N-1,
 * so it sees the whole cache and its local block is the last one).  Same
 * selection and attention as that prefill row, computed Q-outer: the
 * index scan of k_idx is split over the cache, then every (sequence,
 * group, selected block) is one attention piece whose partial results are
 * merged through their log-sum-exp in ascending block order.
 *   q [B, H_q, d_h], q_idx [B, H_kv, d_idx] bf16
 *   K, V [B, N, H_kv, d_h], k_idx [B, N, H_kv, d_idx] bf16
 *   sel out [B, H_kv, k] int32; O out [B, H_q, d_h] fp32;
 *   lse out [B, H_q] fp32, nullable
 * Besides the common limits, decode needs H_kv * d_idx to divide 512 (the
 * index scan reads whole tokens per KiB): other shapes return
 * MSA_ERR_UNSUPPORTED, and the workspace query returns 0 for them.
 */
size_t msa_decode_workspace_bytes(int B, int64_t N, int H_q, int H_kv, int d_h,
                                  int d_idx, int B_k, int k);
msa_status msa_decode(const void *q, const void *q_idx, const void *K,
                      const void *V, const void *k_idx, int B, int64_t N,
                      int H_q, int H_kv, int d_h, int d_idx, int B_k, int k,
                      float scale, int32_t *sel, float *O, float *lse, void *ws,
                      size_t ws_bytes, void *stream);

/*
 * msa_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, kernels and
 * results as msa_decode; the scratch lives in a fixed device array of
 * msa_decode_static_scratch_bytes() bytes (64 MiB) that the library holds
 * on each GPU it runs on until the process ends.  The call allocates and
 * frees nothing.
 *   Limit: msa_decode_workspace_bytes() of the shape must not exceed the
 *   fixed size, else MSA_ERR_WORKSPACE before anything is enqueued (32
 *   sequences of 1M tokens at H_q 64, H_kv 4, d_h 128, k 16 take 20 MiB).
 *   Sharing: every call on one GPU uses that GPU's one array.  Calls that
 *   overlap on one GPU (concurrent streams, or threads enqueueing on
 *   different streams) race on it; serialise them, e.g. on one stream.
 *   Nothing in the array needs clearing between calls.
 */
size_t msa_decode_static_scratch_bytes(void);
msa_status msa_decode_static(const void *q, const void *q_idx, const void *K,
                             const void *V, const void *k_idx, int B, int64_t N,
                             int H_q, int H_kv, int d_h, int d_idx, int B_k,
                             int k, float scale, int32_t *sel, float *O,
                             float *lse, void *stream);

/*
 * Index Branch front-end (Figure 1 caption: the hidden states pass a
 * linear projection and "Norm & RoPE" to give Q^idx and K^idx; section 06:
 * RoPE width 64).  For token i at position pos0 + i and group r, with
 * y = hidden[i] . W[r*d_idx : (r+1)*d_idx]^T (fp32 accumulation):
 *   y <- y * gamma / sqrt(mean(y^2) + eps)           (RMS norm per group)
 *   (y_j, y_{j+R/2}) <- rotation by (pos0+i) * theta^(-2j/R), j < R/2
 * with R = rope_dim (rotate-half pairing; entries past R unchanged), then
 * rounded to bf16.  Run once per projection (Wq -> q_idx, Wk -> k_idx).
 *   hidden [N, d_model] bf16; Wq, Wk [H_kv*d_idx, d_model] bf16 (row r*d_idx+c
 *   is output column c of group r); gq, gk [d_idx] fp32 norm scales
 *   q_idx, k_idx out [N, H_kv, d_idx] bf16 (the Index Branch's inputs)
 * d_model: a positive multiple of 64; d_idx in {32, 64, 128}; rope_dim in
 * {0, 32, 64} and <= d_idx; rope_theta > 1; eps >= 0.  No workspace.
 */
msa_status msa_index_frontend(const void *hidden, const void *Wq, const void *Wk,
                              const float *gq, const float *gk, int64_t N,
                              int64_t pos0, int d_model, int H_kv, int d_idx,
                              int rope_dim, float rope_theta, float eps,
                              void *q_idx, void *k_idx, void *stream);

/*
 * Tuning knobs (process-wide; they change speed, never results).
 *   MSA_OPT_INDEX_FUSED: 1 (default) = Index Branch as one kernel that
 *     keeps a running Top-k per query next to the score GEMM (it uses no
 *     workspace, and msa_prefill runs it once over the whole sequence when
 *     the caller passes sel); 0 = GEMM writes the block scores, a separate
 *     wavefront-per-row Top-k reads them.  Both give identical sel.
 *   MSA_OPT_ATTN_CHUNK: max query positions per KV-outer work item,
 *     128..2048, default 1024 (section 05 part 2: hot blocks are cut along
 *     the query dimension).
 * Thread safety: the values are atomics.  Every entry point reads them
 * once, when it starts, and runs the whole call with that snapshot; a
 * change made while a call runs on another thread takes effect from the
 * next call.  No *_workspace_bytes result depends on them, so a workspace
 * sized before a change stays large enough after it.
 * Returns MSA_ERR_INVALID_ARG for an unknown option or value.
 */
#define MSA_OPT_INDEX_FUSED 1
#define MSA_OPT_ATTN_CHUNK 2
msa_status msa_set_option(int option, int64_t value);
int64_t msa_get_option(int option);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
