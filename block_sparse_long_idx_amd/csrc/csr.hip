// Inverted index: selection table (query -> blocks) turned into a CSR over
// (group, block) buckets (block -> queries), as KV-outer execution needs
// ("MiniMax Sparse Attention" explainer, section 05 part 2: each KV block
// gathers the queries that selected it).
//
// A deterministic counting sort in three launches, no ordering atomics.
// The query range is cut into tiles of kTile positions:
//   (1) per tile and group, an LDS histogram over blocks -> hist[tile][bucket];
//   (2) per bucket, an exclusive scan over the tiles (in place), and an
//       exclusive scan of the bucket totals inside each 256-bucket work-group
//       -> lp[bucket], plus the work-group's total -> agg[wg];
//   (3) per tile and group, the cursor of every block is
//       hist[tile][bucket] + lp[bucket] + (sum of agg before the bucket's
//       work-group), and one wavefront walks the tile's queries in
//       ascending order, appending each (query, slot) at its block's cursor.
//       The tile-0 work-groups also write row_ptr.  Each XCD takes a
//       contiguous range of tiles, so the short runs that neighbouring
//       tiles append to one bucket are merged in one L2 (1M step: 1.97 ->
//       1.65 ms).
// Inside a bucket, positions therefore come out ascending.  Every global
// read of a tile's selection rows is issued before the first use, so each
// launch costs about one memory round trip per work-group.
#include "common.h"
#include "msa_internal.h"


namespace msa {

constexpr int kTile = 512;    // query positions per tile
constexpr int kScanWg = 256;  // buckets per scan work-group

// (1) hist[tile][r][b] = number of queries of the tile whose group-r row
//     selects block b.
__global__ __launch_bounds__(256) void csr_hist_kernel(const int32_t* __restrict__ sel,
                                                       int64_t Nq, int H_kv, int k, int nblk,
                                                       int32_t* __restrict__ hist) {
  extern __shared__ int32_t cnt[];
  const int tile = blockIdx.x, r = blockIdx.y, t = threadIdx.x;
  for (int b = t; b < nblk; b += 256) cnt[b] = 0;
  const int64_t iq0 = (int64_t)tile * kTile;
  const int n = (int)(min(Nq - iq0, (int64_t)kTile) * k);  // entries of this tile
  __syncthreads();
  // entry e = (query e / k, slot e % k); sixteen loads in flight per thread
  for (int e0 = 0; e0 < n; e0 += 16 * 256) {
    int32_t v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = e0 + 256 * u + t;
      v[u] = e < n ? sel[((iq0 + e / k) * H_kv + r) * k + e % k] : -1;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (v[u] >= 0) atomicAdd(&cnt[v[u]], 1);
  }
  __syncthreads();
  int32_t* dst = hist + ((int64_t)tile * H_kv + r) * nblk;
  for (int b = t; b < nblk; b += 256) dst[b] = cnt[b];
}

// (2) One thread per bucket: exclusive prefix over the tiles (in place),
//     then an exclusive scan of the bucket totals across the work-group.
__global__ __launch_bounds__(kScanWg) void csr_scan_kernel(int32_t* __restrict__ hist,
                                                           int ntiles, int64_t nb,
                                                           int32_t* __restrict__ lp,
                                                           int32_t* __restrict__ agg) {
  __shared__ int32_t part[kScanWg];
  const int t = threadIdx.x;
  const int64_t x = (int64_t)blockIdx.x * kScanWg + t;
  int32_t run = 0;
  if (x < nb) {
    for (int t0 = 0; t0 < ntiles; t0 += 8) {
      int32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = t0 + u < ntiles ? hist[(int64_t)(t0 + u) * nb + x] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (t0 + u < ntiles) hist[(int64_t)(t0 + u) * nb + x] = run;
        run += v[u];
      }
    }
  }
  part[t] = run;
  __syncthreads();
  for (int o = 1; o < kScanWg; o <<= 1) {  // Hillis-Steele inclusive scan
    const int32_t v = t >= o ? part[t - o] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  if (x < nb) lp[x] = t ? part[t - 1] : 0;
  if (t == kScanWg - 1) agg[blockIdx.x] = part[kScanWg - 1];
}

// (3) Scatter, work-group per (tile, group r).  LDS: the block cursors, the
//     exclusive prefix of the scan work-groups' totals and the tile's
//     selection rows of group r.
__global__ __launch_bounds__(256) void csr_scatter_kernel(
    const int32_t* __restrict__ sel, int64_t q_start, int64_t Nq, int H_kv, int k, int nblk,
    const int32_t* __restrict__ hist, const int32_t* __restrict__ lp,
    const int32_t* __restrict__ agg, int nwg, int ntiles, int32_t* __restrict__ row_ptr,
    int32_t* __restrict__ col, uint8_t* __restrict__ slot) {
  extern __shared__ int32_t smem[];
  int32_t* cur = smem;               // [nblk + 1]: the last one absorbs padding
  int32_t* aggp = cur + nblk + 1;    // [nwg + 1]
  int32_t* selt = aggp + nwg + 1;    // [kTile][k]
  int32_t* posq = selt + kTile * k;  // [8][32]: a walk step's positions
  // work-group L runs on XCD L % 8; each XCD takes a contiguous range of
  // tiles, so the runs that neighbouring tiles append to one bucket meet in
  // that XCD's L2 instead of being written back from several
  const int L = blockIdx.x, xcd = L & 7, j = L >> 3;
  const int tx = (ntiles + 7) >> 3;
  const int r = j / tx, tile = xcd * tx + j % tx;
  if (tile >= ntiles || r >= H_kv) return;
  const int t = threadIdx.x;
  const int64_t iq0 = (int64_t)tile * kTile;
  const int nq = (int)min(Nq - iq0, (int64_t)kTile);
  const int n = nq * k;
  // the tile's selection rows of group r, all loads in flight
  for (int e0 = 0; e0 < n; e0 += 16 * 256) {
    int32_t v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = e0 + 256 * u + t;
      v[u] = e < n ? sel[((iq0 + e / k) * H_kv + r) * k + e % k] : -1;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = e0 + 256 * u + t;
      if (e < n) selt[e] = v[u];
    }
  }
  // exclusive prefix of agg: per-thread sums of consecutive runs, then a
  // scan of the 256 run sums
  {
    const int per = (nwg + 255) / 256;
    const int lo = min(nwg, per * t), hi = min(nwg, per * (t + 1));
    int32_t s = 0;
    for (int w = lo; w < hi; ++w) s += agg[w];
    aggp[nwg] = 0;
    __shared__ int32_t part[256];
    part[t] = s;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int32_t v = t >= o ? part[t - o] : 0;
      __syncthreads();
      part[t] += v;
      __syncthreads();
    }
    int32_t run = t ? part[t - 1] : 0;
    for (int w = lo; w < hi; ++w) {
      aggp[w] = run;
      run += agg[w];
    }
    if (t == 255) aggp[nwg] = part[255];
  }
  __syncthreads();
  const int32_t* hrow = hist + ((int64_t)tile * H_kv + r) * nblk;
  const int64_t x0 = (int64_t)r * nblk;
  // the cursors: eight blocks per thread per batch, every load issued first
  for (int b0 = 0; b0 < nblk; b0 += 8 * 256) {
    int32_t hv[8], lv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int b = b0 + 256 * u + t;
      hv[u] = b < nblk ? hrow[b] : 0;
      lv[u] = b < nblk ? lp[x0 + b] : 0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int b = b0 + 256 * u + t;
      if (b < nblk) {
        const int32_t start = lv[u] + aggp[(x0 + b) / kScanWg];
        cur[b] = hv[u] + start;
        if (tile == 0) row_ptr[x0 + b] = start;
      }
    }
  }
  if (tile == 0 && r == H_kv - 1 && t == 0) row_ptr[(int64_t)H_kv * nblk] = aggp[nwg];
  __syncthreads();
  if (t >= kWave) return;
  // Lanes 0..k-1 of the first wavefront walk the tile's queries in order;
  // lane s takes slot s (the k blocks of one query are distinct, so the
  // lanes of one instruction never share a cursor).  Each query's cursor
  // updates are one LDS atomic add with return, and the LDS executes one
  // wavefront's instructions in issue order, so eight queries' updates go
  // out back to back and still take their positions in query order.
  // Padding entries (-1) and rows past the tile add to the spare cursor
  // cur[nblk], so no atomic is behind a branch.  The eight queries'
  // positions then pass through LDS so that every lane of the wave stores:
  // a store instruction covers 64 / KS queries (KS = k rounded up to 16 or
  // 32 lanes) instead of one, which keeps fewer stores in flight per entry.
  const int KS = k <= 16 ? 16 : 32, QS = kWave / KS;
  const int g = t / KS, sl = t % KS;
  if (t == 0) cur[nblk] = 0;
  for (int iq = 0; iq < nq; iq += 8) {
    if (t < k) {
      int32_t bb[8], pos[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) bb[u] = iq + u < nq ? selt[(iq + u) * k + t] : -1;
#pragma unroll
      for (int u = 0; u < 8; ++u) pos[u] = atomicAdd(&cur[bb[u] >= 0 ? bb[u] : nblk], 1);
#pragma unroll
      for (int u = 0; u < 8; ++u) posq[u * KS + t] = bb[u] >= 0 ? pos[u] : -1;
    }
    // the wave's LDS accesses complete in order; the fences keep the
    // compiler from moving the reads above the writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int j = 0; j < 8; j += QS) {
      const int qq = j + g;
      const int32_t p = sl < k ? posq[qq * KS + sl] : -1;
      if (p >= 0) {
        col[p] = (int32_t)(q_start + iq0 + iq + qq);
        slot[p] = (uint8_t)sl;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

static int64_t scan_wgs(int64_t nb) { return ceil_div(nb, kScanWg); }

size_t invert_scratch_bytes(int64_t Nq, int H_kv, int nblk) {
  const int64_t ntiles = ceil_div(Nq, kTile);
  const int64_t nb = (int64_t)H_kv * nblk;
  return sizeof(int32_t) * (size_t)(ntiles * nb + nb + scan_wgs(nb));
}

hipError_t launch_invert(const int32_t* sel, int64_t q_start, int64_t Nq, int H_kv, int k,
                         int nblk, int32_t* row_ptr, int32_t* col, uint8_t* slot,
                         void* scratch, hipStream_t stream) {
  const int ntiles = (int)ceil_div(Nq, kTile);
  const int64_t nb = (int64_t)H_kv * nblk;
  const int nwg = (int)scan_wgs(nb);
  int32_t* hist = static_cast<int32_t*>(scratch);
  int32_t* lp = hist + (int64_t)ntiles * nb;
  int32_t* agg = lp + nb;
  // scatter LDS: nblk + 1 + nwg + 1 + kTile * k + 256 ints, at most 16385 +
  // 4097 + 16384 + 256 (H_kv <= 64, nblk <= 16384, k <= 32): 145 KiB
  const size_t lds_hist = sizeof(int32_t) * (size_t)nblk;
  const size_t lds_scatter =
      sizeof(int32_t) * ((size_t)nblk + 1 + nwg + 1 + (size_t)kTile * k + 8 * 32);
  static bool lds_ready = false;
  if (!lds_ready) {
    const int most = (int)(sizeof(int32_t) * (16385 + 4097 + kTile * 32 + 8 * 32));
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&csr_scatter_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, most);
    if (e != hipSuccess) return e;
    lds_ready = true;
  }
  csr_hist_kernel<<<dim3(ntiles, H_kv), 256, lds_hist, stream>>>(sel, Nq, H_kv, k, nblk, hist);
  csr_scan_kernel<<<(unsigned)nwg, kScanWg, 0, stream>>>(hist, ntiles, nb, lp, agg);
  const int tx = (ntiles + 7) / 8;
  csr_scatter_kernel<<<(unsigned)(8 * tx * H_kv), 256, lds_scatter, stream>>>(
      sel, q_start, Nq, H_kv, k, nblk, hist, lp, agg, nwg, ntiles, row_ptr, col, slot);
  return hipGetLastError();
}

}  // namespace msa
