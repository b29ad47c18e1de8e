// Main Branch backward ("MiniMax Sparse Attention" explainer, section 02:
// the Main Branch is exact softmax attention over the selected blocks, so
// its gradients are those of softmax attention restricted to each row's
// token set T; section 03: the selection is not differentiable, so nothing
// flows back into the Index Branch from here).
//
// Per row (query i, head h of group r), with p the forward's probabilities
// (recomputed from the saved lse), D = dO . O:
//   dp_j = dO . V_j,  ds_j = p_j (dp_j - D)
//   dQ = scale * sum_j ds_j K_j,  dK_j += scale * ds_j Q,  dV_j += p_j dO
// One KV-outer pass over the forward's inverted index (local positions
// included, with the causal mask).  A work unit is one bucket (group r,
// block b), or a fixed-size slice of a large one.  Its work-group keeps
// the block's K and V in registers and sweeps the unit's rows -- (position,
// head) pairs -- in 32-row tiles staged row-major in LDS: S^T = K Q^T and
// dP^T = V dO^T read them as plain fragments, dV += P^T dO and
// dK += dS^T Q (the contractions over rows) through the transpose read, so
// no transposed copy is made.  Each tile's P and dS go through LDS; dS
// also feeds dQ^T = K^T dS^T over all 128 keys, formed by waves owning 32
// d each and stored as a bf16 partial per (i, h, slot), which a second
// kernel sums per (i, h) in ascending slot order.  A whole bucket adds its dK/dV sums to the outputs at
// the end; the slices of a split bucket write fp32 partials that a third
// kernel sums in slice order.  Deterministic, no atomics on the outputs.
#include "common.h"
#include "msa_internal.h"

#include <algorithm>

namespace msa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kUnitRows = 16384;  // rows per work unit, at most
constexpr int kUnitPos = 1024;    // positions per work unit, at most

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8) that wait for the vector memory counter alone.
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitVm0 = wait_vm(0);

// The Q and dO rows of a 32-row tile sit row-major in LDS, their 16-byte
// chunks XOR-swizzled by qsw(row).  Two kinds of read hit them: a fragment
// read (16 lanes on 16 consecutive rows, one chunk each) and a transpose
// read (each 16-lane group on 4 consecutive rows, 32 bytes of each).  For
// d = 128 a row spans all 64 banks and qsw spreads the low two row bits
// over the chunk index's high bits and the next two over its low bits, so
// both kinds land on distinct banks; for d = 64 two rows share a bank row.
template <int D>
__device__ __forceinline__ int qsw(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3))
                  : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}
template <int D>
__device__ __forceinline__ int qoff(int row, int col) {
  return row * D + 8 * ((col >> 3) ^ qsw<D>(row)) + (col & 7);
}

// MFMA A/B fragment of a row tile: 32 rows x 16 d at k-step s, lane half h
// covering d in [h*D/2, (h+1)*D/2).
template <int D>
__device__ __forceinline__ bf16x8 qr_frag(const __bf16* blk, int row, int s, int h) {
  return *reinterpret_cast<const bf16x8*>(&blk[row * D + 8 * (((D / 16) * h + s) ^ qsw<D>(row))]);
}

typedef __bf16 bf16v4 __attribute__((ext_vector_type(4)));

// LDS transpose read (gfx950): in each group of 16 lanes, lane m reads 4
// consecutive 16-bit values at its own address, and lane i receives, as
// its value j, value i%4 of lane 4j + i/4.  So if the group's lanes read a
// 4-row x 16-column block row by row (lane m: row m/4, columns 4(m%4)..),
// each lane ends up holding its own column over the 4 rows.
__device__ __forceinline__ bf16x4 ld_tr(const __bf16* p) {
  const bf16v4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (bf16v4 __attribute__((address_space(3)))*)p);
  return bf16x4{v[0], v[1], v[2], v[3]};
}

// Operand with the contraction over tile rows c0..c0+15 of a row tile:
// lane (n, h) gets column d0 + n at rows c0 + 4h + {0..3} and
// c0 + 8 + 4h + {0..3}, the order in which an accumulator's registers
// 8u..8u+7 hold rows 16u.. (so an accumulator can be the other operand).
template <int D>
__device__ __forceinline__ bf16x8 qtr_frag(const __bf16* blk, int d0, int c0, int h, int n) {
  const int row = c0 + 4 * h + ((n >> 2) & 3), col = d0 + (n & 16) + 4 * (n & 3);
  const bf16x4 lo = ld_tr(blk + qoff<D>(row, col));
  const bf16x4 hi = ld_tr(blk + qoff<D>(row + 8, col));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// P and dS tiles [32 rows][128 keys] (256-byte rows): 8-byte pieces (4
// keys) XOR-swizzled by psw(row).  Measured on gfx950, 8-byte LDS writes
// are served 16 lanes at a time over 32 banks (the piece index mod 16
// decides the banks) and reads 32 lanes at a time over 64 banks (mod 32).
// psw puts the row's low two bits on the piece's top two bits and its
// next two bits on the bottom two, with bit 1 of the row (flipped by bit
// 4) in between, so that
//  - 16 consecutive rows storing one piece differ mod 16 (producer stores),
//  - 32 rows reading one piece differ mod 32 (the dQ operand reads),
//  - a transpose read over 4 rows x 32 keys covers 32 distinct pieces.
// (Without the middle bit, the stores took ~4 conflict cycles each.)
__device__ __forceinline__ int psw(int row) {
  return ((row & 3) << 3) | ((((row >> 1) ^ (row >> 4)) & 1) << 2) | ((row >> 2) & 3);
}
__device__ __forceinline__ int poff(int row, int key) {
  return row * kBlock + 4 * ((key >> 2) ^ psw(row)) + (key & 3);
}
// Operand holding tile row `row` at keys c0 + 4h + {0..3}, c0 + 8 + 4h + {0..3}.
__device__ __forceinline__ bf16x8 pr_frag(const __bf16* t, int row, int c0, int h) {
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(&t[poff(row, c0 + 4 * h)]);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(&t[poff(row, c0 + 8 + 4 * h)]);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// Operand with the contraction over tile rows c0..c0+15: lane (n, h) gets
// key k0 + n at rows c0 + 4h + {0..3} and c0 + 8 + 4h + {0..3} (transpose
// read).
__device__ __forceinline__ bf16x8 ptr_frag(const __bf16* t, int k0, int c0, int h, int n) {
  const int row = c0 + 4 * h + ((n >> 2) & 3), key = k0 + (n & 16) + 4 * (n & 3);
  const bf16x4 lo = ld_tr(t + poff(row, key));
  const bf16x4 hi = ld_tr(t + poff(row + 8, key));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Work-group barrier that waits for this wave's LDS operations only.  A
// __syncthreads also waits for every direct global->LDS load in flight
// (its fence covers their LDS writes); the producers instead wait for the
// loads of the next tile alone, with an explicit counter wait, and leave
// the tile after it in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace

int bwd_unit_positions(int G) { return std::min(kUnitPos, std::max(1, kUnitRows / G)); }

// ---------------------------------------------------------------------------
// D = dO . O per (row, head): 16 lanes per row, one 8-wide chunk each.
__global__ __launch_bounds__(256) void bwd_delta_kernel(const __bf16* __restrict__ dO,
                                                        const float* __restrict__ O,
                                                        int64_t rows, int d_h,
                                                        float* __restrict__ D) {
  const int cpr = d_h / 8;  // 8 or 16 lanes per row
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / cpr;
  const int c = (int)(gid % cpr);
  float s = 0.f;
  if (row < rows) {
    const bf16x8 g = *reinterpret_cast<const bf16x8*>(dO + row * d_h + 8 * c);
    const f32x4 o0 = *reinterpret_cast<const f32x4*>(O + row * d_h + 8 * c);
    const f32x4 o1 = *reinterpret_cast<const f32x4*>(O + row * d_h + 8 * c + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) s = fmaf(bf2f(g[e]), o0[e], s);
#pragma unroll
    for (int e = 0; e < 4; ++e) s = fmaf(bf2f(g[4 + e]), o1[e], s);
  }
  for (int o = 1; o < cpr; o <<= 1) s += __shfl_xor(s, o, kWave);
  if (row < rows && c == 0) D[row] = s;
}

// ---------------------------------------------------------------------------
// Work units: every non-empty bucket, split into slices of at most `upos`
// positions when larger.  Units of split buckets and buckets of at least
// upos/2 entries come first.  A split bucket also gets a record (bucket,
// first partial, slices) for the dK/dV partial sum.
__global__ __launch_bounds__(1024) void build_bwd_units_kernel(
    const int32_t* __restrict__ row_ptr, int64_t nb, int upos, int4* __restrict__ units,
    int32_t* __restrict__ n_units, int4* __restrict__ splits, int32_t* __restrict__ n_splits) {
  __shared__ int4 sc[1024];
  const int t = threadIdx.x;
  const int64_t per = ceil_div(nb, (int64_t)1024);
  const int64_t lo = min(nb, per * t), hi = min(nb, per * (t + 1));
  int4 c = make_int4(0, 0, 0, 0);  // large units, small units, split buckets, slices
  for (int64_t x = lo; x < hi; ++x) {
    const int32_t cnt = row_ptr[x + 1] - row_ptr[x];
    const int32_t nu = (cnt + upos - 1) / upos;
    if (nu > 1) {
      c.x += nu;
      c.z += 1;
      c.w += nu;
    } else if (2 * cnt >= upos) {
      c.x += 1;
    } else if (cnt > 0) {
      c.y += 1;
    }
  }
  sc[t] = c;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int4 v = t >= o ? sc[t - o] : make_int4(0, 0, 0, 0);
    __syncthreads();
    const int4 m = sc[t];
    sc[t] = make_int4(m.x + v.x, m.y + v.y, m.z + v.z, m.w + v.w);
    __syncthreads();
  }
  const int4 tot = sc[1023];
  const int4 ex = t ? sc[t - 1] : make_int4(0, 0, 0, 0);
  int32_t ub = ex.x, us = tot.x + ex.y, sp = ex.z, pi = ex.w;
  for (int64_t x = lo; x < hi; ++x) {
    const int32_t s0 = row_ptr[x], cnt = row_ptr[x + 1] - s0;
    const int32_t nu = (cnt + upos - 1) / upos;
    if (nu > 1) {
      splits[sp++] = make_int4((int)x, pi, nu, 0);
      for (int32_t s = 0; s < nu; ++s)
        units[ub++] = make_int4((int)x, s0 + s * upos, min(upos, cnt - s * upos), pi + s);
      pi += nu;
    } else if (2 * cnt >= upos) {
      units[ub++] = make_int4((int)x, s0, cnt, -1);
    } else if (cnt > 0) {
      units[us++] = make_int4((int)x, s0, cnt, -1);
    }
  }
  if (t == 1023) {
    n_units[0] = tot.x + tot.y;
    n_units[1] = 0;
    n_splits[0] = tot.z;
  }
}

template <int DH>
struct BwdSmem {
  __bf16 qr[4][32 * DH];         // the tile's Q rows, row-major swizzled (ring of four)
  __bf16 gr[4][32 * DH];         // the tile's dO rows
  __bf16 pb[2][32 * kBlock];     // P [row][key], for dV
  __bf16 db[2][32 * kBlock];     // dS [row][key], for dK and dQ
  float ld[4][64];           // per tile row: lse, then D = dO . O
  int32_t lim[2][32];       // per tile row: last visible key of the block (-1: none)
  int32_t pos[kUnitPos];    // the unit's query positions
  uint8_t sl[kUnitPos];     // and the block's slot in each one's selection
};

// Eight waves per work-group, two per SIMD, producers and consumers, each
// role in its own tile loop:
//  - waves 0-3 (keys kw = 32w ..) fetch the row tiles (direct global -> LDS
//    loads, two tiles ahead), form S^T = K Q^T and dP^T = V dO^T, the
//    softmax and dS for tile T (the row on the lane), and leave P and dS
//    in LDS;
//  - waves 4-7 take tile T-1 from LDS after the barrier: dV += P^T dO and
//    dK += dS^T Q for a 64-key x 64-d quarter (d = 128; 32 keys x all of
//    d for d = 64), and dQ^T = K^T dS^T for a 32-wide d-slice (K^T in
//    registers).
// No MFMA or softmax is done twice, and each SIMD holds one wave of each
// kind, so one's softmax and LDS waits overlap the other's MFMAs.  The
// producers do no transpose read: the compiler waits for every direct
// load in flight before one, which would cut the prefetch to nothing.
template <int DH>
__global__ __launch_bounds__(512) void bwd_fused_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ D,
    const int32_t* __restrict__ col, const uint8_t* __restrict__ slot,
    const int4* __restrict__ units, int32_t* __restrict__ n_units, int64_t q_start, int64_t Nk,
    int H_q, int H_kv, int G, float inv_G, int nblk, int k, int64_t spare, float scale,
    float scale_log2, __bf16* __restrict__ part, float* __restrict__ kvpart,
    float* __restrict__ dK, float* __restrict__ dV) {
  constexpr int S = DH / 16, NDG = DH / 32, NDH = NDG / 2, CH = DH / 8;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  BwdSmem<DH>& sm = *reinterpret_cast<BwdSmem<DH>*>(smem_raw);
  __shared__ int32_t next;
  const int t = threadIdx.x, wave = t >> 6;
  const int32_t total = n_units[0];
  for (;;) {
    if (t == 0) next = atomicAdd(&n_units[1], 1);
    __syncthreads();
    const int32_t unit_id = next;
    if (unit_id >= total) return;
    const int4 un = units[unit_id];
    const int bucket = un.x, start = un.y, count = un.z, pidx = un.w;
    const int r = bucket / nblk, b = bucket % nblk;
    int tl = t;  // per-unit addresses are rebuilt, not hoisted and spilled
    asm volatile("" : "+v"(tl));
    {
      // count <= kUnitPos = 2 * 512: all loads first, then the LDS stores
      int32_t pv[kUnitPos / 512];
      uint8_t sv[kUnitPos / 512];
#pragma unroll
      for (int u = 0; u < kUnitPos / 512; ++u) {
        const int p = tl + 512 * u;
        pv[u] = col[start + min(p, count - 1)];
        sv[u] = slot[start + min(p, count - 1)];
      }
#pragma unroll
      for (int u = 0; u < kUnitPos / 512; ++u) {
        const int p = tl + 512 * u;
        if (p < count) {
          sm.pos[p] = pv[u];
          sm.sl[p] = sv[u];
        }
      }
    }
    const int lane = tl & 63, h = lane >> 5, n = lane & 31;
    const int kq = wave & 3, dh = wave >> 2;
    const int kw = 32 * kq;  // this wave's keys kw .. kw+31; its d-slice for dQ
    const int64_t key0 = (int64_t)b * kBlock;
    // Static operands in one register array, by role: producers hold the
    // wave's keys as the B operand of S (fr[0..S)) and dP (fr[S..2S)), d
    // split by lane half; consumers hold K^T of their d-slice over all 128
    // keys as the A operand of dQ^T (fr[0..8)).
    bf16x8 fr[2 * S];
#pragma unroll
    for (int s = 0; s < 2 * S; ++s) fr[s] = bf16x8{};
    if (dh == 0) {
      const int64_t key = key0 + kw + n;
      const bool in = key < Nk;
      const int64_t off = ((in ? key : key0) * H_kv + r) * DH + (DH / 2) * h;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        fr[s] = *reinterpret_cast<const bf16x8*>(K + off + 8 * s);
        fr[S + s] = *reinterpret_cast<const bf16x8*>(V + off + 8 * s);
      }
#pragma unroll
      for (int s = 0; s < 2 * S; ++s) fr[s] = in ? fr[s] : bf16x8{};
    } else if (kw < DH) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int64_t key = key0 + 16 * u + (e < 4 ? 4 * h + e : 8 + 4 * h + (e - 4));
          const __bf16 xv = K[((key < Nk ? key : key0) * H_kv + r) * DH + kw + n];
          fr[u][e] = key < Nk ? xv : f2bf(0.f);
        }
    }
    // every fragment load of the unit has landed before the tile loop, so no
    // wait inside the loop has to cover them
    __builtin_amdgcn_s_waitcnt(0);

    const int nrows = count * G;
    const int ntile = (nrows + 31) / 32;
    const int hq0 = r * G;
    // unit row R -> its position and query head (rows past the end take the
    // unit's first row, so every load stays valid)
    auto row_of = [&](int R, int64_t& pos, int& hq) {
      const bool ok = R < nrows;
      const int pp = ok ? (int)__fmul_rn(__fadd_rn((float)R, 0.5f), inv_G) : 0;
      pos = sm.pos[pp];
      hq = hq0 + (ok ? R - pp * G : 0);
    };
    // Tile T's Q and dO rows go global -> LDS by direct loads (no registers),
    // issued by the producer waves two tiles ahead into a ring of four: each
    // wave-instruction fills one contiguous KiB, lane i writing bytes
    // 16i..16i+15 (rows v*RPI.., chunk slot i % CH), and a lane fetches the
    // global chunk that the swizzle keeps at its slot.  The tile's lse and D
    // follow the same way, issued last by producer wave 0 (lane i < 32: lse
    // of row i; lane 32 + i: D of row i).
    constexpr int RPI = 1024 / (2 * DH);  // rows per wave-instruction
    constexpr int NI = 32 / RPI;          // wave-instructions per tensor and tile
    constexpr int PW = NI / 2;            // per producer wave (Q and dO together)
    // the wave index in a scalar register: the LDS destination must be
    // wave-uniform
    const int kqs = __builtin_amdgcn_readfirstlane(kq);
    auto dma = [&](int T) {
      const int b4 = T & 3;
#pragma unroll
      for (int u = 0; u < PW; ++u) {
        const int v = kqs * PW + u, tens = v / NI, vi = v % NI;
        const int row = vi * RPI + lane / CH, cs = lane % CH;
        int64_t pos;
        int hq;
        row_of(32 * T + row, pos, hq);
        const __bf16* src = (tens == 0 ? Q + (pos * H_q + hq) * DH
                                       : dO + ((pos - q_start) * H_q + hq) * DH) +
                            8 * (cs ^ qsw<DH>(row));
        __builtin_amdgcn_global_load_lds(
            static_cast<const void*>(src),
            static_cast<void*>((tens == 0 ? sm.qr[b4] : sm.gr[b4]) + vi * RPI * DH), 16, 0, 0);
      }
      if (kqs == 0) {
        int64_t pos;
        int hq;
        row_of(32 * T + (lane & 31), pos, hq);
        const int64_t ih = (pos - q_start) * H_q + hq;
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(lane < 32 ? lse + ih : D + ih),
                                         static_cast<void*>(sm.ld[b4]), 4, 0, 0);
      }
    };
    // last visible key of each row of tile T (wave 0, lanes 0..31)
    auto put_lim = [&](int T) {
      if (tl < 32) {
        const int R = 32 * T + tl;
        int64_t pos;
        int hq;
        row_of(R, pos, hq);
        sm.lim[T & 1][tl] = R < nrows ? (int)(pos - key0) : -1;
      }
    };
    // A producer wave's only memory-counter operations in the tile loop are
    // these loads, so "all but its last loads (those of tile T+2) done"
    // means tile T+1 has landed.
    auto wait_tile = [&](bool more) {
      if (!more)
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
      else if (kqs == 0)
        __builtin_amdgcn_s_waitcnt(wait_vm(PW + 1));
      else
        __builtin_amdgcn_s_waitcnt(wait_vm(PW));
    };
    __syncthreads();  // positions staged
    if (dh == 0) {
      // ---- producer waves: S^T, dP^T, softmax, dS; P and dS into LDS ----
      dma(0);
      if (ntile > 1) dma(1);
      put_lim(0);
      wait_tile(ntile > 1);
      lds_barrier();
      for (int T = 0; T < ntile; ++T) {
        const int b2 = T & 1, b4 = T & 3;
        // LDS indices go through an opaque copy of n so that the fragment
        // reads stay inside the loop rather than being hoisted into registers
        int nn = n;
        asm volatile("" : "+v"(nn));
        const bool more = T + 2 < ntile;
        if (more) dma(T + 2);
        // S^T = K Q^T and dP^T = V dO^T for the wave's 32 keys: the row on
        // the lane, keys in the registers, so each lane needs the row's lse,
        // D and mask bound only.  Each k-step's Q and dO fragments are read
        // while the previous step's two MFMAs run.
        f32x16 sa = {}, pa = {};
        bf16x8 qa = qr_frag<DH>(sm.qr[b4], nn, 0, h), ga = qr_frag<DH>(sm.gr[b4], nn, 0, h);
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const bf16x8 qn = s + 1 < S ? qr_frag<DH>(sm.qr[b4], nn, s + 1, h) : qa;
          const bf16x8 gn = s + 1 < S ? qr_frag<DH>(sm.gr[b4], nn, s + 1, h) : ga;
          sa = mfma32(fr[s], qa, sa);
          pa = mfma32(fr[S + s], ga, pa);
          qa = qn;
          ga = gn;
        }
        bf16x8 pA[2], dA[2];
        const int lm = sm.lim[b2][nn];
        const float l2 = sm.ld[b4][nn] * kLog2e, dv = sm.ld[b4][32 + nn];
        // the causal mask only bites in tiles holding the block's own
        // positions: elsewhere every row sees all of the wave's 32 keys
        if (__builtin_amdgcn_ballot_w64(lm < kw + 31) == 0) {
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float p = __builtin_amdgcn_exp2f(sa[8 * u + e] * scale_log2 - l2);
              pA[u][e] = f2bf(p);
              dA[u][e] = f2bf(p * (pa[8 * u + e] - dv));
            }
        } else
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int key = kw + acc_row(8 * u + e, h);
            const float ex = __builtin_amdgcn_exp2f(sa[8 * u + e] * scale_log2 - l2);
            const float p = key <= lm ? ex : 0.f;
            pA[u][e] = f2bf(p);
            dA[u][e] = f2bf(p * (pa[8 * u + e] - dv));
          }
        // P and dS [row][key] for the consumers: registers 8u + 4q' .. +3
        // hold keys kw + 16u + 8q' + 4h .. +3
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int qh = 0; qh < 2; ++qh) {
            const int kc = kw + 16 * u + 8 * qh + 4 * h;
            *reinterpret_cast<bf16x4*>(&sm.pb[b2][poff(nn, kc)]) =
                bf16x4{pA[u][4 * qh], pA[u][4 * qh + 1], pA[u][4 * qh + 2], pA[u][4 * qh + 3]};
            *reinterpret_cast<bf16x4*>(&sm.db[b2][poff(nn, kc)]) =
                bf16x4{dA[u][4 * qh], dA[u][4 * qh + 1], dA[u][4 * qh + 2], dA[u][4 * qh + 3]};
          }
        }
        if (T + 1 < ntile) put_lim(T + 1);
        wait_tile(more);  // tile T+1 is in LDS
        lds_barrier();
      }
    } else {
      // ---- consumer waves, one tile behind: dV += P^T dO and dK += dS^T Q
      // for the wave's share of keys and d, and dQ^T = K^T dS^T for its
      // 32-wide d-slice, stored as the rows' bf16 partials ----
      // dV/dK split: the wave owns KG 32-key groups x DG 32-d groups (64 x 64
      // for d = 128, so each operand fragment read feeds two MFMAs)
      constexpr int KG = NDG >= 4 ? 2 : 1, DG = NDG / KG;
      const int kb0 = 32 * KG * (kq / KG), db0 = 32 * DG * (kq % KG);
      f32x16 ak[KG][DG], av[KG][DG];
#pragma unroll
      for (int a = 0; a < KG; ++a)
#pragma unroll
        for (int i = 0; i < DG; ++i) ak[a][i] = av[a][i] = f32x16{};
      auto consume = [&](int T, int nn) {
        const int b2 = T & 1, b4 = T & 3;
        bf16x8 pf[KG][2], sf[KG][2];
#pragma unroll
        for (int a = 0; a < KG; ++a)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            pf[a][u] = ptr_frag(sm.pb[b2], kb0 + 32 * a, 16 * u, h, nn);
            sf[a][u] = ptr_frag(sm.db[b2], kb0 + 32 * a, 16 * u, h, nn);
          }
#pragma unroll
        for (int dg = 0; dg < DG; ++dg) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const bf16x8 gq = qtr_frag<DH>(sm.gr[b4], db0 + 32 * dg, 16 * u, h, nn);
            const bf16x8 qq = qtr_frag<DH>(sm.qr[b4], db0 + 32 * dg, 16 * u, h, nn);
#pragma unroll
            for (int a = 0; a < KG; ++a) {
              av[a][dg] = mfma32(pf[a][u], gq, av[a][dg]);
              ak[a][dg] = mfma32(sf[a][u], qq, ak[a][dg]);
            }
          }
        }
        if (kw < DH) {
          f32x16 acc = {};
#pragma unroll
          for (int u = 0; u < 8; ++u) acc = mfma32(fr[u], pr_frag(sm.db[b2], nn, 16 * u, h), acc);
          // rows past the end store zeros to the spare slot
          const int R = 32 * T + n;
          const bool ok = R < nrows;
          const int pp = ok ? (int)__fmul_rn(__fadd_rn((float)R, 0.5f), inv_G) : 0;
          const int64_t ps = ok ? (sm.pos[pp] - q_start) * k + sm.sl[pp] : spare;
          const int hl = ok ? R - pp * G : 0;
          __bf16* dstp = part + (ps * H_kv + r) * (DH / 4) * G * 4 + hl * 4;
          // accumulator rows are d = kw + 8qd + 4h + {0..3}: d-quad 8kq + 2qd + h
          const int dq0 = ok ? 8 * kq : 0;
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            *reinterpret_cast<bf16x4*>(dstp + (int64_t)(dq0 + 2 * qd + h) * G * 4) =
                bf16x4{f2bf(acc[4 * qd]), f2bf(acc[4 * qd + 1]), f2bf(acc[4 * qd + 2]),
                       f2bf(acc[4 * qd + 3])};
        }
      };
      __syncthreads();  // the producers' first tile is staged
      for (int T = 0; T < ntile; ++T) {
        int nn = n;
        asm volatile("" : "+v"(nn));
        if (T > 0) consume(T - 1, nn);
        __syncthreads();
      }
      consume(ntile - 1, n);
      // the unit's dK/dV sums: accumulator rows are keys, the lane is d
      if (pidx < 0) {
#pragma unroll
        for (int a = 0; a < KG; ++a)
#pragma unroll
          for (int i = 0; i < DG; ++i)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int64_t key = key0 + kb0 + 32 * a + acc_row(j, h);
              if (key < Nk) {
                const int64_t off = (key * H_kv + r) * DH + db0 + 32 * i + n;
                dK[off] += scale * ak[a][i][j];
                dV[off] += av[a][i][j];
              }
            }
      } else {
        float* pk = kvpart + (int64_t)pidx * 2 * kBlock * DH;
#pragma unroll
        for (int a = 0; a < KG; ++a)
#pragma unroll
          for (int i = 0; i < DG; ++i)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int kr = kb0 + 32 * a + acc_row(j, h), d = db0 + 32 * i + n;
              pk[kr * DH + d] = ak[a][i][j];
              pk[(kBlock + kr) * DH + d] = av[a][i][j];
            }
      }
    }
  }
}

// dQ[i, h] = scale * sum over the row's slots (ascending) of the partials.
// Thread -> (row i, group r, d-quad, head in group), head fastest: a
// partial row group [d_h/4][G][4] is then read contiguously by consecutive
// threads, and each head's dQ row gets whole 64-byte runs.
template <int DH>
__global__ __launch_bounds__(256) void bwd_dq_reduce_kernel(const __bf16* __restrict__ part,
                                                            int64_t q_start, int64_t Nq,
                                                            int H_q, int H_kv, int k,
                                                            float scale, float* __restrict__ dQ) {
  const int G = H_q / H_kv;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= Nq * H_q * (DH / 4)) return;
  const int hl = (int)(gid % G);
  const int64_t rest = gid / G;
  const int dq = (int)(rest % (DH / 4));
  const int64_t ir = rest / (DH / 4);
  const int r = (int)(ir % H_kv);
  const int64_t iq = ir / H_kv;
  const int n_sel = (int)min((int64_t)k, (q_start + iq) / kBlock + 1);
  const __bf16* src = part + ((iq * k) * H_kv + r) * (DH / 4) * G * 4 + ((int64_t)dq * G + hl) * 4;
  const int64_t slot_stride = (int64_t)H_kv * (DH / 4) * G * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // each partial is read once: non-temporal loads, four slots in flight
#pragma unroll 4
  for (int s = 0; s < n_sel; ++s) {
    const bf16x4 x =
        __builtin_nontemporal_load(reinterpret_cast<const bf16x4*>(src + s * slot_stride));
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += bf2f(x[e]);
  }
  // d-quad dq holds d = 4*dq .. 4*dq+3
  *reinterpret_cast<f32x4*>(dQ + (iq * H_q + r * G + hl) * DH + 4 * dq) =
      f32x4{acc[0] * scale, acc[1] * scale, acc[2] * scale, acc[3] * scale};
}

// dK/dV of split buckets: the slices' partials summed in slice order.
template <int DH>
__global__ __launch_bounds__(256) void bwd_kv_reduce_kernel(
    const int4* __restrict__ splits, const int32_t* __restrict__ n_splits,
    const float* __restrict__ kvpart, int H_kv, int nblk, int64_t Nk, float scale,
    float* __restrict__ dK, float* __restrict__ dV) {
  const int32_t ns = n_splits[0];
  for (int32_t si = blockIdx.x; si < ns; si += gridDim.x) {
    const int4 sp = splits[si];
    const int r = sp.x / nblk, b = sp.x % nblk;
    for (int e = 4 * (int)threadIdx.x; e < kBlock * DH; e += 4 * 256) {
      f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < sp.z; ++s) {
        const float* pk = kvpart + (int64_t)(sp.y + s) * 2 * kBlock * DH;
        const f32x4 a = *reinterpret_cast<const f32x4*>(pk + e);
        const f32x4 v = *reinterpret_cast<const f32x4*>(pk + kBlock * DH + e);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          sk[q] += a[q];
          sv[q] += v[q];
        }
      }
      const int64_t key = (int64_t)b * kBlock + e / DH;
      if (key < Nk) {
        const int64_t off = (key * H_kv + r) * DH + e % DH;
        f32x4 ok = *reinterpret_cast<const f32x4*>(dK + off);
        f32x4 ov = *reinterpret_cast<const f32x4*>(dV + off);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          ok[q] += scale * sk[q];
          ov[q] += sv[q];
        }
        *reinterpret_cast<f32x4*>(dK + off) = ok;
        *reinterpret_cast<f32x4*>(dV + off) = ov;
      }
    }
  }
}

// ---------------------------------------------------------------------------
static bool bwd_lds_ready = false;

template <typename Kern>
static hipError_t bwd_allow(Kern* kern, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

static hipError_t bwd_prepare() {
  if (bwd_lds_ready) return hipSuccess;
  hipError_t e = bwd_allow(&bwd_fused_kernel<128>, sizeof(BwdSmem<128>));
  if (e == hipSuccess) e = bwd_allow(&bwd_fused_kernel<64>, sizeof(BwdSmem<64>));
  if (e == hipSuccess) bwd_lds_ready = true;
  return e;
}

BwdBounds bwd_bounds(int64_t nb, int64_t nnz, int G) {
  const int64_t upos = bwd_unit_positions(G);
  BwdBounds w;
  w.max_units = nb + nnz / upos + 1;
  w.max_splits = nnz / (upos + 1) + 1;
  w.max_slices = 2 * (nnz / upos) + 1;
  return w;
}

hipError_t launch_attn_bwd(const void* Q, const void* K, const void* V, const float* O,
                           const float* lse, const void* dO, const int32_t* row_ptr,
                           const int32_t* col, const uint8_t* slot, int4* units,
                           int32_t* n_units, int4* splits, int32_t* n_splits,
                           const BwdBounds& bounds, int64_t q_start, int64_t Nq, int64_t Nk,
                           int H_q, int H_kv, int d_h, int nblk, int k, float scale,
                           float* Dbuf, void* dq_part, float* kvpart, float* dQ, float* dK,
                           float* dV, hipStream_t stream) {
  hipError_t e = bwd_prepare();
  if (e != hipSuccess) return e;
  const int G = H_q / H_kv;
  const float inv_G = 1.f / (float)G;
  const float scale_log2 = scale * kLog2e;
  auto* q = static_cast<const __bf16*>(Q);
  auto* kk = static_cast<const __bf16*>(K);
  auto* v = static_cast<const __bf16*>(V);
  auto* g = static_cast<const __bf16*>(dO);
  auto* part = static_cast<__bf16*>(dq_part);
  const int64_t rows = Nq * H_q;
  const int cpr = d_h / 8;
  bwd_delta_kernel<<<(unsigned)ceil_div(rows * cpr, (int64_t)256), 256, 0, stream>>>(
      g, O, rows, d_h, Dbuf);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t spare = Nq * k;
  const int nb = H_kv * nblk;
  build_bwd_units_kernel<<<1, 1024, 0, stream>>>(row_ptr, nb, bwd_unit_positions(G), units,
                                                 n_units, splits, n_splits);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dim3 grid((unsigned)std::min<int64_t>(bounds.max_units, device_cus()));
  dim3 rgrid((unsigned)ceil_div(rows * (d_h / 4), (int64_t)256));
  dim3 sgrid((unsigned)std::min<int64_t>(bounds.max_splits, 2 * device_cus()));
  if (d_h == 128) {
    bwd_fused_kernel<128><<<grid, 512, sizeof(BwdSmem<128>), stream>>>(
        q, kk, v, g, lse, Dbuf, col, slot, units, n_units, q_start, Nk, H_q, H_kv, G, inv_G,
        nblk, k, spare, scale, scale_log2, part, kvpart, dK, dV);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_dq_reduce_kernel<128><<<rgrid, 256, 0, stream>>>(part, q_start, Nq, H_q, H_kv, k,
                                                         scale, dQ);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_kv_reduce_kernel<128><<<sgrid, 256, 0, stream>>>(splits, n_splits, kvpart, H_kv, nblk,
                                                         Nk, scale, dK, dV);
  } else if (d_h == 64) {
    bwd_fused_kernel<64><<<grid, 512, sizeof(BwdSmem<64>), stream>>>(
        q, kk, v, g, lse, Dbuf, col, slot, units, n_units, q_start, Nk, H_q, H_kv, G, inv_G,
        nblk, k, spare, scale, scale_log2, part, kvpart, dK, dV);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_dq_reduce_kernel<64><<<rgrid, 256, 0, stream>>>(part, q_start, Nq, H_q, H_kv, k, scale,
                                                        dQ);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_kv_reduce_kernel<64><<<sgrid, 256, 0, stream>>>(splits, n_splits, kvpart, H_kv, nblk,
                                                        Nk, scale, dK, dV);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace msa
