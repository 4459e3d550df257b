// Non-refresh step: fused momentum + RowNorm + weight update.
//
// PaperDaily post on "Scaling Muon for Diffusion Transformers", section
// "Periodic Row-wise Muon": on steps with t mod K != 0 the update direction
// is gamma * RowNorm_eps(M) of the current momentum, where (blog fig. 4)
// every row is divided by max(||row||_2, eps).  For tall matrices the slices
// are columns: the post's section "distributed co-design", paper Eq. (8),
// normalises them by column sums of squares over the rows.
//
// The row and column kernels are HBM-bound: per element they read G (2 or
// 4 B), M (4 B) and W (4 B) and write M (4 B) and W (4 B).  Each thread issues
// its loads in batches ahead of the stores that may alias them, so a memory
// round trip serves many rows.  Reductions run in a fixed order, so results
// are bitwise reproducible from run to run.
#include <hip/hip_runtime.h>

#include "muon_internal.h"

namespace muon {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Four consecutive gradient values starting at element idx (16-B aligned for
// f32, 8-B aligned for bf16).
__device__ __forceinline__ float4 load_g4(const void* g, int gdt, int64_t idx) {
  if (gdt == 1) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(g) + idx);
    return make_float4(bf16_to_f32(u.x & 0xffffu), bf16_to_f32(u.x >> 16),
                       bf16_to_f32(u.y & 0xffffu), bf16_to_f32(u.y >> 16));
  }
  return *reinterpret_cast<const float4*>(static_cast<const float*>(g) + idx);
}

#define GLOBAL __attribute__((address_space(1)))
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef unsigned u32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float4 ld4(const GLOBAL float* p) {
  const f32x4v v = *(const GLOBAL f32x4v*)(p);
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st4(GLOBAL float* p, float4 v) {
  *(GLOBAL f32x4v*)(p) = f32x4v{v.x, v.y, v.z, v.w};
}

// Same, with the gradient dtype fixed (0 = f32, 1 = bf16) and global-memory
// loads (FLAT loads would also count against the LDS/scalar counter).
template <int GDT>
__device__ __forceinline__ float4 load_g4t(const void* g, int64_t idx) {
  if constexpr (GDT == 1) {
    const u32x2v u = *(const GLOBAL u32x2v*)(static_cast<const uint16_t*>(g) + idx);
    return make_float4(bf16_to_f32(u.x & 0xffffu), bf16_to_f32(u.x >> 16),
                       bf16_to_f32(u.y & 0xffffu), bf16_to_f32(u.y >> 16));
  } else {
    return ld4((const GLOBAL float*)(static_cast<const float*>(g) + idx));
  }
}

__device__ __forceinline__ float load_g1(const void* g, int gdt, int64_t idx) {
  if (gdt == 1) return bf16_to_f32(static_cast<const uint16_t*>(g)[idx]);
  return static_cast<const float*>(g)[idx];
}

__device__ __forceinline__ float4 fma4(float s, float4 a, float4 b) {  // s*a + b
  return make_float4(fmaf(s, a.x, b.x), fmaf(s, a.y, b.y), fmaf(s, a.z, b.z), fmaf(s, a.w, b.w));
}

__device__ __forceinline__ float dot4(float4 a) {
  return a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
}

// Sum over the 256-thread block in a fixed order; every thread gets the total.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

__device__ __forceinline__ int find_mat(const int64_t* prefix, int nmat, int64_t gid) {
  int lo = 0, hi = nmat - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= gid) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// One row (n <= MAXCH * 1024, n % 4 == 0) of a wide matrix held in
// registers: M <- beta M + G, then W <- W (1 - lr wd) - coef M with coef from
// the row's norm.  Loads are issued ahead of the stores that may alias them
// (as far as the compiler knows): G, M and, for rows of up to 8 chunks, W
// all before the reduction; longer rows load W after it, in batches of 8
// chunks.  Chunks past the row end re-read its last chunk and are not used.
template <int MAXCH, int GDT>
__device__ __forceinline__ void rows_in_registers(const void* g, int64_t goff, float* M, float* W,
                                                  int64_t n, const StepScalars& sc, float* red) {
  constexpr int WB = MAXCH < 8 ? MAXCH : 8;      // W chunks per batch
  constexpr bool W_EARLY = MAXCH <= 8;
  GLOBAL float* gM = (GLOBAL float*)(M);
  GLOBAL float* gW = (GLOBAL float*)(W);
  const int tid = threadIdx.x;
  const float wkeep = 1.0f - sc.lr * sc.wd;
  float4 gv[MAXCH], mv[MAXCH], wv[WB];
#pragma unroll
  for (int ch = 0; ch < MAXCH; ++ch) {
    const int64_t e = min((int64_t(ch) * kThreads + tid) * 4, n - 4);
    gv[ch] = load_g4t<GDT>(g, goff + e);
    mv[ch] = ld4(gM + e);
  }
  if constexpr (W_EARLY) {
#pragma unroll
    for (int ch = 0; ch < WB; ++ch) wv[ch] = ld4(gW + min((int64_t(ch) * kThreads + tid) * 4, n - 4));
  }
  float ss = 0.f;
#pragma unroll
  for (int ch = 0; ch < MAXCH; ++ch) {
    mv[ch] = fma4(sc.beta, mv[ch], gv[ch]);
    if ((int64_t(ch) * kThreads + tid) * 4 < n) ss += dot4(mv[ch]);
  }
  const float tot = block_sum(ss, red);
  const float coef = sc.lr * sc.gamma / fmaxf(sqrtf(tot), sc.eps_row);
#pragma unroll
  for (int b = 0; b < MAXCH; b += WB) {
    if constexpr (!W_EARLY) {
#pragma unroll
      for (int u = 0; u < WB; ++u)
        wv[u] = ld4(gW + min((int64_t(b + u) * kThreads + tid) * 4, n - 4));
    }
#pragma unroll
    for (int u = 0; u < WB; ++u) {
      const int64_t e = (int64_t(b + u) * kThreads + tid) * 4;
      if (e < n) {
        st4(gM + e, mv[b + u]);
        const float4 w = wv[u];
        st4(gW + e, fma4(-coef, mv[b + u],
                         make_float4(w.x * wkeep, w.y * wkeep, w.z * wkeep, w.w * wkeep)));
      }
    }
  }
}

// One workgroup per row.  MAXCH > 0: the row (<= MAXCH * 1024 elements)
// stays in registers between the norm and the update.  MAXCH == 0: any
// length, the updated momentum is re-read for the second pass.
template <int MAXCH>
__global__ __launch_bounds__(kThreads) void rownorm_rows_kernel(
    const MatDev* __restrict__ mats, const int32_t* __restrict__ mat_ids,
    const int64_t* __restrict__ row_prefix, int32_t nmat, StepScalars sc) {
  __shared__ float red[4];
  const int64_t gid = blockIdx.x;
  const int k = find_mat(row_prefix, nmat, gid);
  const MatDev d = mats[mat_ids[k]];
  const int64_t row = gid - row_prefix[k];
  const int64_t n = d.cols;
  float* __restrict__ M = d.mom + row * n;
  float* __restrict__ W = d.w + row * n;
  const int64_t goff = row * n;
  const int tid = threadIdx.x;
  const float wkeep = 1.0f - sc.lr * sc.wd;
  float ss = 0.f;

  if ((n & 3) == 0) {
    if constexpr (MAXCH > 0) {
      if (d.gdt == 1) rows_in_registers<MAXCH, 1>(d.g, goff, M, W, n, sc, red);
      else rows_in_registers<MAXCH, 0>(d.g, goff, M, W, n, sc, red);
    } else {
      for (int64_t e = int64_t(tid) * 4; e < n; e += kThreads * 4) {
        const float4 g = load_g4(d.g, d.gdt, goff + e);
        const float4 m = fma4(sc.beta, *reinterpret_cast<const float4*>(M + e), g);
        *reinterpret_cast<float4*>(M + e) = m;
        ss += dot4(m);
      }
      const float tot = block_sum(ss, red);
      const float coef = sc.lr * sc.gamma / fmaxf(sqrtf(tot), sc.eps_row);
      for (int64_t e = int64_t(tid) * 4; e < n; e += kThreads * 4) {
        const float4 m = *reinterpret_cast<const float4*>(M + e);
        float4 w = *reinterpret_cast<const float4*>(W + e);
        w = make_float4(w.x * wkeep, w.y * wkeep, w.z * wkeep, w.w * wkeep);
        *reinterpret_cast<float4*>(W + e) = fma4(-coef, m, w);
      }
    }
  } else {
    // Ragged row length: scalar, two passes.
    for (int64_t e = tid; e < n; e += kThreads) {
      const float m = fmaf(sc.beta, M[e], load_g1(d.g, d.gdt, goff + e));
      M[e] = m;
      ss += m * m;
    }
    const float tot = block_sum(ss, red);
    const float coef = sc.lr * sc.gamma / fmaxf(sqrtf(tot), sc.eps_row);
    for (int64_t e = tid; e < n; e += kThreads) W[e] = fmaf(-coef, M[e], W[e] * wkeep);
  }
}

// Tall-matrix row loops, four adjacent columns per thread.  A thread visits
// rows rb, rb + 4, rb + 8, ... of its tile, in batches of kColBatch such
// rows: all loads of a batch are issued before any of its stores, so one
// memory round trip serves the whole batch (the stores may alias the loads as
// far as the compiler knows, so it would not reorder them itself).  Loads of
// rows at or past r1 re-read row r1 - 1 (no branch around a load); their
// stores and sums are skipped.  Sums of squares accumulate in row order.
constexpr int kColBatch = 8;

template <int GDT>
__device__ __forceinline__ void cols_fetch_gm(const void* g, const GLOBAL float* mom, int64_t n,
                                              int64_t col, int64_t rb, int64_t r1,
                                              float4 (&gv)[kColBatch], float4 (&mv)[kColBatch]) {
#pragma unroll
  for (int u = 0; u < kColBatch; ++u) {
    const int64_t e = min(rb + 4 * u, r1 - 1) * n + col;
    gv[u] = load_g4t<GDT>(g, e);
    mv[u] = ld4(mom + e);
  }
}

__device__ __forceinline__ void cols_momentum(GLOBAL float* mom, int64_t n, int64_t col, int64_t rb,
                                              int64_t r1, float beta,
                                              const float4 (&gv)[kColBatch],
                                              const float4 (&mv)[kColBatch], float (&ss)[4]) {
#pragma unroll
  for (int u = 0; u < kColBatch; ++u) {
    const int64_t r = rb + 4 * u;
    if (r < r1) {
      const float4 mm = fma4(beta, mv[u], gv[u]);
      st4(mom + r * n + col, mm);
      ss[0] += mm.x * mm.x; ss[1] += mm.y * mm.y; ss[2] += mm.z * mm.z; ss[3] += mm.w * mm.w;
    }
  }
}

// Phase 1: M <- beta M + G over the thread's rows, sums of squares per column.
template <int GDT>
__device__ __forceinline__ void cols_phase1_vec(const MatDev& d, int64_t n, int64_t col,
                                                int64_t rb, int64_t r1, float beta,
                                                float (&ss)[4]) {
  GLOBAL float* mom = (GLOBAL float*)(d.mom);
  float4 gv[kColBatch], mv[kColBatch];
  for (; rb < r1; rb += 4 * kColBatch) {
    cols_fetch_gm<GDT>(d.g, mom, n, col, rb, r1, gv, mv);
    cols_momentum(mom, n, col, rb, r1, beta, gv, mv, ss);
  }
}

__device__ __forceinline__ void cols_fetch_mw(const GLOBAL float* mom, const GLOBAL float* w,
                                              int64_t n, int64_t col, int64_t rb, int64_t r1,
                                              float4 (&mv)[kColBatch], float4 (&wv)[kColBatch]) {
#pragma unroll
  for (int u = 0; u < kColBatch; ++u) {
    const int64_t e = min(rb + 4 * u, r1 - 1) * n + col;
    mv[u] = ld4(mom + e);
    wv[u] = ld4(w + e);
  }
}

__device__ __forceinline__ void cols_update(GLOBAL float* w, int64_t n, int64_t col, int64_t rb,
                                            int64_t r1, const float (&coef)[4], float wkeep,
                                            const float4 (&mv)[kColBatch],
                                            const float4 (&wv)[kColBatch]) {
#pragma unroll
  for (int u = 0; u < kColBatch; ++u) {
    const int64_t r = rb + 4 * u;
    if (r < r1) {
      const float4 mm = mv[u], ww = wv[u];
      st4(w + r * n + col,
          make_float4(fmaf(-coef[0], mm.x, ww.x * wkeep), fmaf(-coef[1], mm.y, ww.y * wkeep),
                      fmaf(-coef[2], mm.z, ww.z * wkeep), fmaf(-coef[3], mm.w, ww.w * wkeep)));
    }
  }
}

// Phase 2: W <- W (1 - lr wd) - coef M over the thread's rows.
__device__ __forceinline__ void cols_phase2_vec(const MatDev& d, int64_t n, int64_t col,
                                                int64_t rb, int64_t r1, const float (&coef)[4],
                                                float wkeep) {
  const GLOBAL float* mom = (const GLOBAL float*)(d.mom);
  GLOBAL float* w = (GLOBAL float*)(d.w);
  float4 mv[kColBatch], wv[kColBatch];
  for (; rb < r1; rb += 4 * kColBatch) {
    cols_fetch_mw(mom, w, n, col, rb, r1, mv, wv);
    cols_update(w, n, col, rb, r1, coef, wkeep, mv, wv);
  }
}

// Tall matrices, slices = columns.  A tile is kColTileRows x kColTileCols;
// thread (rg = tid / 64, ct = tid % 64) owns 4 columns and rows rg, rg+4, ...
// Phase 1 writes the new momentum and one partial column sum of squares per
// (row tile, column); rownorm_coef_kernel adds each column's partials over
// the row tiles in order and leaves lr * gamma / max(||column||, eps) in the
// first partial row; phase 2 scales and updates W.
// Phase 2 visits the tiles in reverse order, so the momentum phase 1 wrote
// last (most likely still in the Infinity Cache) is read first.
template <int PHASE>
__global__ __launch_bounds__(kThreads) void rownorm_cols_kernel(
    const MatDev* __restrict__ mats, const TileItem* __restrict__ tiles, StepScalars sc) {
  __shared__ float red[4][kColTileCols];
  const TileItem it = tiles[PHASE == 1 ? blockIdx.x : gridDim.x - 1 - blockIdx.x];
  const MatDev d = mats[it.id];
  const int64_t m = d.rows, n = d.cols;
  const int64_t r0 = int64_t(it.ti) * kColTileRows;
  const int64_t r1 = min(m, r0 + kColTileRows);
  const int64_t c0 = int64_t(it.tj) * kColTileCols;
  const int rg = threadIdx.x >> 6, ct = threadIdx.x & 63;
  const bool vec = (n & 3) == 0;
  // local column offsets owned by this thread (vector: 4 adjacent; scalar: strided)
  int lc[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) lc[v] = vec ? ct * 4 + v : ct + 64 * v;
  const int64_t nchunk = (m + kColTileRows - 1) / kColTileRows;

  if constexpr (PHASE == 1) {
    float ss[4] = {0.f, 0.f, 0.f, 0.f};
    if (vec) {
      const int64_t col = c0 + ct * 4;
      if (col < n) {
        if (d.gdt == 1) cols_phase1_vec<1>(d, n, col, r0 + rg, r1, sc.beta, ss);
        else cols_phase1_vec<0>(d, n, col, r0 + rg, r1, sc.beta, ss);
      }
    } else {
      for (int64_t r = r0 + rg; r < r1; r += 4) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t col = c0 + lc[v];
          if (col < n) {
            const int64_t e = r * n + col;
            const float mm = fmaf(sc.beta, d.mom[e], load_g1(d.g, d.gdt, e));
            d.mom[e] = mm;
            ss[v] += mm * mm;
          }
        }
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) red[rg][lc[v]] = ss[v];
    __syncthreads();
    if (rg == 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t col = c0 + lc[v];
        if (col < n)
          d.part[int64_t(it.ti) * n + col] =
              (red[0][lc[v]] + red[1][lc[v]]) + (red[2][lc[v]] + red[3][lc[v]]);
      }
    }
  } else {
    (void)nchunk;
    float coef[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t col = c0 + lc[v];
      coef[v] = col < n ? d.part[col] : 0.f;
    }
    const float wkeep = 1.0f - sc.lr * sc.wd;
    if (vec) {
      const int64_t col = c0 + ct * 4;
      if (col < n) cols_phase2_vec(d, n, col, r0 + rg, r1, coef, wkeep);
    } else {
      for (int64_t r = r0 + rg; r < r1; r += 4) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t col = c0 + lc[v];
          if (col < n) {
            const int64_t e = r * n + col;
            d.w[e] = fmaf(-coef[v], d.mom[e], d.w[e] * wkeep);
          }
        }
      }
    }
  }
}

// One workgroup per column strip (kColTileCols columns) of a tall matrix:
// each column's partial sums of squares over the row tiles, added in row
// order, become its update coefficient, stored in the first partial row.
__global__ __launch_bounds__(kThreads) void rownorm_coef_kernel(
    const MatDev* __restrict__ mats, const TileItem* __restrict__ strips, StepScalars sc) {
  const TileItem it = strips[blockIdx.x];
  const MatDev d = mats[it.id];
  const int64_t n = d.cols;
  const int64_t nchunk = (d.rows + kColTileRows - 1) / kColTileRows;
  const int64_t col = int64_t(it.tj) * kColTileCols + threadIdx.x;
  if (col >= n) return;
  float s = 0.f;
  for (int64_t k = 0; k < nchunk; ++k) s += d.part[k * n + col];
  d.part[col] = sc.lr * sc.gamma / fmaxf(sqrtf(s), sc.eps_row);
}


// ---- Tall matrices in one pass ------------------------------------------
//
// The same column normalisation as above without the second read of M: a
// workgroup keeps its tile's new momentum in registers while the column
// sums of squares of the whole strip are formed, then updates W from those
// registers.  Per element this is G, M and W read once and M, W written
// once (18 B with bf16 gradients), where the two-pass form re-reads M.
//
// Tiles are kTallRows x kTallCols; thread (rg = tid / 64, ct = tid % 64)
// owns two adjacent columns of the strip and rows rg, rg + 8, ... of the
// tile.  A strip's 128 columns are four runs of 32, 512 columns apart, so
// that the rows of one tile, a power-of-two pitch apart in DiT shapes
// (n = 2048: 8 KB), do not all fall in the same few DRAM channels:
// contiguous strips streamed about 10% slower at 8 KB and 16 KB pitches than
// at their neighbours, and runs a quarter of the row apart are 4 KB apart at
// n = 4096, which lost again.
// Workgroup b takes tile b, and the tile table lists each strip's row chunks
// consecutively.  Each workgroup stores its column partials and arrives at
// the strip; the last to arrive adds the strip's partials in a fixed order
// (8 waves over consecutive chunk ranges, then a fixed tree), writes
// lr * gamma / max(||column||, eps) behind the partials and raises the
// strip's ready word, which the others wait on.  While they wait, their
// first rows of W are already loading.
//
// Why every wait ends: the device deals workgroup ids round-robin to its 8
// XCDs, and each XCD starts its share in id order.  Take the first strip
// (by id) still missing an arrival.  Every earlier strip has all arrived, so
// its workgroups leave; an XCD that has not yet started all of its
// workgroups of this strip therefore holds no others that stay, and a strip
// of <= kTallMaxChunks workgroups has at most kTallMaxChunks / 8 on one XCD,
// which the host checks is at most half of what an XCD holds at once.  So
// the strip's workgroups all start and arrive, and by induction every strip
// does.  (Ids claimed at run time from a counter would not do: near the end
// of a launch the XCD with workgroups left would have to hold whole strips.)
// A wait still gives up after a poll limit (kTallPollLimit by default): the
// workgroup then leaves W alone and lists its tile, and a repair launch on
// the same stream writes the listed tiles once every strip's coefficients
// are published (they always are by the end of the launch, since arrivals
// never wait).  The result is the same either way, bit for bit.
//
// Partials and coefficients cross workgroups, and with them the XCDs'
// separate L2 caches, within the launch.  Each strip owns padded rows of its
// own (kTallCols floats: nchunk partial rows, then the coefficient row), so
// no cache line holds two strips' values, and both sides access them with
// agent-scope atomic stores and loads.  A writer waits until its wave's
// stores have completed before touching the strip's counter, and a reader
// loads them only after the counter it polled has changed; no L2 write-back
// or invalidate is needed (agent-scope fences, which do both, cost more than
// the second pass this kernel saves).
// Every counter is back at zero when the launch ends (the reducer resets the
// arrivals, the last workgroup to leave a strip its ready word and
// departures), so launches need no clearing between them and replay
// unchanged from a captured graph.
constexpr int kTallThreads = 512;
constexpr int kTallRowsPerThread = kTallRows / (kTallThreads / 64);   // 32
constexpr int kTallBatch = 8;                                         // rows per load batch
static_assert(kTallCols == 2 * 64, "two columns per lane");
constexpr unsigned kTallRunGap = 512;   // columns between a strip's runs
static_assert(kTallRunGap % 32 == 0, "whole runs");

// Counter words are only touched by agent-scope atomics: adds, exchanges
// and (for polling) loads.
__device__ __forceinline__ uint32_t rd_counter(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void set_counter(uint32_t* p, uint32_t v) {
  (void)__hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float2 ld2_agent(const float* p) {
  GLOBAL float* q = (GLOBAL float*)(p);
  return make_float2(__hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                     __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void st2_agent(float* p, float2 v) {
  GLOBAL float* q = (GLOBAL float*)(p);
  __hip_atomic_store(q, v.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, v.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until this wave's memory operations have completed (vmcnt(0) on
// gfx950: expcnt and lgkmcnt left at their no-wait maxima).  The values
// that cross workgroups are only stored and loaded with agent-scope atomics,
// which complete at the agent's coherence point; waiting for them orders
// them against the counter atomics without an L2 write-back or invalidate.
__device__ __forceinline__ void wait_vmem() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0f70);
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float2 add2(float2 a, float2 b) {
  return make_float2(a.x + b.x, a.y + b.y);
}
__device__ __forceinline__ float2 sum8(const float2 (&r)[kTallThreads / 64][64], int ct) {
  return add2(add2(add2(r[0][ct], r[1][ct]), add2(r[2][ct], r[3][ct])),
              add2(add2(r[4][ct], r[5][ct]), add2(r[6][ct], r[7][ct])));
}

// Rows of a tile are addressed through raw buffer resources based at the
// tile's first row and sized to its valid rows.  A lane's offset holds only
// its columns; the row, the same across a wave, is a scalar offset.  Lanes
// past the last column carry an offset beyond the buffer, so their loads
// return zeros and their stores are dropped.  Rows past the tile's end are
// clamped to its last row for loads, and skipped (a wave-uniform branch)
// for sums and stores.
typedef float f32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* p, int64_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, int(nbytes), 0x00020000);
}
__device__ __forceinline__ float2 bld2(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  const f32x2v v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return make_float2(v.x, v.y);
}

// A store whose data registers the next instructions may reuse, with three
// wait states after it.  The compiler has left none when a 16-byte store
// ended a conditional block and the join block began by writing its data
// registers (a 64-bit move, gfx950): the store's last lanes then took the
// new values.  These stores are 8 bytes; the guard costs three cycles.
__device__ __forceinline__ void bst2_guarded(__amdgpu_buffer_rsrc_t r, unsigned voff,
                                             unsigned soff, float2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(f32x2v{v.x, v.y}, r, voff, soff, 0);
  asm volatile("s_nop 2" ::: "memory");
}

// Byte offset of row rg + 8u of the tile (clamped to its last row), es
// bytes per element; 32-bit scalar arithmetic (a tile buffer is < 2 GiB).
__device__ __forceinline__ unsigned tall_row(int rg, int u, int rows, unsigned n, unsigned es) {
  return unsigned(min(rg + 8 * u, rows - 1)) * n * es;
}

// Momentum update of a thread's rows (row rg + 8u of the tile, columns
// col, col + 1 at lane offset vcol = 4 col, or past the buffer).  All M
// loads are issued first, then the gradients in batches of 8 rows, which
// keeps the kernel within 128 registers (two workgroups per CU).
template <int GDT>
__device__ __forceinline__ void tall_momentum(const void* g, __amdgpu_buffer_rsrc_t rm,
                                              int64_t r0, int rows, unsigned n, unsigned vcol,
                                              int rg, float beta,
                                              float2 (&mv)[kTallRowsPerThread]) {
  constexpr int RPT = kTallRowsPerThread;
  constexpr unsigned GES = GDT == 1 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t rgr =
      tile_rsrc(static_cast<const char*>(g) + r0 * n * GES, int64_t(rows) * n * GES);
  const unsigned vg = GDT == 1 ? vcol / 2 : vcol;   // the out-of-range mark stays out of range
#pragma unroll
  for (int u = 0; u < RPT; ++u) mv[u] = bld2(rm, vcol, tall_row(rg, u, rows, n, 4));
#pragma unroll
  for (int b = 0; b < RPT; b += kTallBatch) {
    float2 gv[kTallBatch];
#pragma unroll
    for (int u = 0; u < kTallBatch; ++u) {
      const unsigned so = tall_row(rg, b + u, rows, n, GES);
      if constexpr (GDT == 1) {
        const unsigned q = __builtin_amdgcn_raw_buffer_load_b32(rgr, vg, so, 0);
        gv[u] = make_float2(bf16_to_f32(q & 0xffffu), bf16_to_f32(q >> 16));
      } else {
        gv[u] = bld2(rgr, vg, so);
      }
    }
#pragma unroll
    for (int u = 0; u < kTallBatch; ++u)
      mv[b + u] = make_float2(fmaf(beta, mv[b + u].x, gv[u].x), fmaf(beta, mv[b + u].y, gv[u].y));
  }
}

// Column of lane ct (0..63, two columns col and col + 1) in column strip tj
// of an n-column matrix: four runs of 32 (one per group of 16 lanes, a
// 128-byte line per row), kTallRunGap columns apart within groups of
// 4 kTallRunGap columns when n allows; else a quarter of the row apart when
// n % 128 == 0; else 128 contiguous columns.  Every form covers each column
// once, and a lane keeps its columns in every chunk of the strip.
__device__ __forceinline__ int64_t tall_col(unsigned tj, int ct, unsigned n) {
  constexpr unsigned SPG = kTallRunGap / 32;   // strips per group
  if (n % (4u * kTallRunGap) == 0)
    return int64_t(tj / SPG) * (4 * kTallRunGap) + (ct >> 4) * kTallRunGap +
           int64_t(tj % SPG) * 32 + 2 * (ct & 15);
  if (n % 128u == 0) return int64_t(ct >> 4) * (n / 4) + int64_t(tj) * 32 + 2 * (ct & 15);
  return int64_t(tj) * kTallCols + 2 * ct;
}

__global__ __launch_bounds__(kTallThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void rownorm_tall_kernel(const MatDev* __restrict__ mats, const TileItem* __restrict__ tiles,
                         TallSync* __restrict__ sync, TallCtl* __restrict__ ctl,
                         uint32_t* __restrict__ repair, uint32_t ntiles, uint32_t poll_limit,
                         StepScalars sc) {
  constexpr int RPT = kTallRowsPerThread;
  constexpr int B = kTallBatch;
  __shared__ float2 red[kTallThreads / 64][64];
  __shared__ float2 cf[64];
  __shared__ uint32_t s_reducer, s_gaveup;
  const int tid = threadIdx.x;
  const TileItem it = tiles[blockIdx.x];
  const MatDev d = mats[it.id];
  TallSync* sy = sync + d.sync0 + it.tj;
  const int64_t m = d.rows;
  const unsigned n = unsigned(d.cols);   // tall: n < m <= kTallMaxChunks * kTallRows
  const uint32_t nchunk = static_cast<uint32_t>((m + kTallRows - 1) / kTallRows);
  const int64_t r0 = int64_t(it.ti) * kTallRows;
  const int rows = int(min(m, r0 + kTallRows) - r0);
  const int rg = __builtin_amdgcn_readfirstlane(tid >> 6), ct = tid & 63;
  const int64_t col = tall_col(unsigned(it.tj), ct, n);
  const bool act = col < n;
  const unsigned voff = act ? unsigned(col * 4) : 0x80000000u;   // beyond any tile buffer
  const __amdgpu_buffer_rsrc_t rm = tile_rsrc(d.mom + r0 * n, int64_t(rows) * n * 4);
  const __amdgpu_buffer_rsrc_t rw = tile_rsrc(d.w + r0 * n, int64_t(rows) * n * 4);
  // this strip's partial rows 0 .. nchunk - 1, then its coefficient row
  float* const sp = d.part + int64_t(it.tj) * (nchunk + 1) * kTallCols + 2 * ct;

  // 1. momentum, kept in registers; column sums of squares in row order
  //    (the new momentum is stored in step 2).
  float2 mv[RPT];
  {
    if (d.gdt == 1) tall_momentum<1>(d.g, rm, r0, rows, n, voff, rg, sc.beta, mv);
    else tall_momentum<0>(d.g, rm, r0, rows, n, voff, rg, sc.beta, mv);
    float2 ss = make_float2(0.f, 0.f);
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      if (rg + 8 * u < rows) {
        const float2 q = mv[u];
        ss = make_float2(fmaf(q.x, q.x, ss.x), fmaf(q.y, q.y, ss.y));
      }
    }
    red[rg][ct] = ss;
  }
  __syncthreads();
  // 2. the tile's column partials (wave 0), then arrival at the strip.
  if (rg == 0) {
    if (act) st2_agent(sp + int64_t(it.ti) * kTallCols, sum8(red, ct));
    if (tid == 0) {
      wait_vmem();   // wave 0's partial stores are complete
      s_reducer = atomicAdd(&sy->arrive, 1u) == nchunk - 1;
    }
  }
  // the first rows of W load during the wait, then the new momentum is
  // stored (after those loads: measured 1-2% faster than storing it before
  // the arrival)
  float2 wv[B];
#pragma unroll
  for (int u = 0; u < B; ++u) wv[u] = bld2(rw, voff, tall_row(rg, u, rows, n, 4));
#pragma unroll
  for (int u = 0; u < RPT; ++u)
    if (rg + 8 * u < rows) bst2_guarded(rm, voff, tall_row(rg, u, rows, n, 4), mv[u]);
  __syncthreads();
  float2 coef;
  bool skip_w = false;
  if (__builtin_amdgcn_readfirstlane(s_reducer)) {
    // 3a. last arrival: every partial of the strip is published.
    __syncthreads();
    const uint32_t q = (nchunk + 7) / 8;
    const uint32_t k0 = min(nchunk, rg * q), k1 = min(nchunk, k0 + q);
    float2 s = make_float2(0.f, 0.f);
    for (uint32_t k = k0; k < k1; k += 8) {
      float2 pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) pv[u] = ld2_agent(sp + int64_t(min(k + u, k1 - 1)) * kTallCols);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (k + u < k1) s = add2(s, pv[u]);
    }
    __syncthreads();   // red is reused
    red[rg][ct] = s;
    __syncthreads();
    if (rg == 0) {
      const float2 t = sum8(red, ct);
      const float lg = sc.lr * sc.gamma;
      const float2 c = make_float2(lg / fmaxf(sqrtf(t.x), sc.eps_row),
                                   lg / fmaxf(sqrtf(t.y), sc.eps_row));
      cf[ct] = c;
      if (act) st2_agent(sp + int64_t(nchunk) * kTallCols, c);
      if (tid == 0) {
        wait_vmem();   // wave 0's coefficient stores are complete
        set_counter(&sy->arrive, 0u);
        set_counter(&sy->ready, 1u);
      }
    }
    __syncthreads();
    coef = cf[ct];
  } else {
    // 3b. wait for the strip's coefficients; a wait that gives up lists the
    //     tile for the repair launch instead of writing W.
    if (tid == 0) {
      uint32_t spins = 0, gave_up = 0;
      while (rd_counter(&sy->ready) == 0u) {
        if (++spins > poll_limit) { gave_up = 1; break; }
        __builtin_amdgcn_s_sleep(10);   // about 640 clocks between polls
      }
      if (gave_up) {
        atomicAdd(&ctl->giveups, 1u);
        const uint32_t slot = atomicAdd(&ctl->repair_count, 1u);
        if (slot < ntiles) repair[slot] = blockIdx.x;
      }
      s_gaveup = gave_up;
    }
    __syncthreads();
    skip_w = __builtin_amdgcn_readfirstlane(s_gaveup) != 0;
    coef = skip_w ? make_float2(0.f, 0.f) : ld2_agent(sp + int64_t(nchunk) * kTallCols);
  }
  // 4. W <- W (1 - lr wd) - coef M, loads of 8 rows ahead of their stores
  //    (skipped by a workgroup whose wait gave up: the repair launch does it).
  const float wkeep = 1.0f - sc.lr * sc.wd;
  if (!skip_w) {
#pragma unroll
  for (int b = 0; b < RPT; b += B) {
    if (b > 0) {
#pragma unroll
      for (int u = 0; u < B; ++u) wv[u] = bld2(rw, voff, tall_row(rg, b + u, rows, n, 4));
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const float2 mm = mv[b + u], ww = wv[u];
      if (rg + 8 * (b + u) < rows)
        bst2_guarded(rw, voff, tall_row(rg, b + u, rows, n, 4),
                     make_float2(fmaf(-coef.x, mm.x, ww.x * wkeep),
                                 fmaf(-coef.y, mm.y, ww.y * wkeep)));
    }
  }
  }
  // 5. leave the strip; the last one out clears it for the next launch.
  __syncthreads();   // every thread holds its coefficients
  if (tid == 0) {
    if (atomicAdd(&sy->depart, 1u) == nchunk - 1) {
      set_counter(&sy->depart, 0u);
      set_counter(&sy->ready, 0u);
    }
  }
}

// Repair launch of the single-pass tall RowNorm, enqueued right after it:
// the tiles whose workgroup gave up waiting get W <- W (1 - lr wd) - coef M
// from the strip's published coefficients and the momentum that workgroup
// stored, with the arithmetic of the normal path, so the result is the
// same bit for bit.  Every workgroup reads the list length first; the last
// one to finish resets it (and its own counter) for the next launch, so no
// launch needs clearing.  With nothing listed each workgroup exits after a
// load and an atomic.
__global__ __launch_bounds__(kTallThreads) void rownorm_tall_repair_kernel(
    const MatDev* __restrict__ mats, const TileItem* __restrict__ tiles,
    TallCtl* __restrict__ ctl, const uint32_t* __restrict__ repair, uint32_t ntiles,
    StepScalars sc) {
  __shared__ uint32_t s_count;
  const int tid = threadIdx.x;
  if (tid == 0) s_count = min(rd_counter(&ctl->repair_count), ntiles);
  __syncthreads();
  const uint32_t count = s_count;
  const int rg = tid >> 6, ct = tid & 63;
  const float wkeep = 1.0f - sc.lr * sc.wd;
  for (uint32_t k = blockIdx.x; k < count; k += gridDim.x) {
    const TileItem it = tiles[repair[k]];
    const MatDev d = mats[it.id];
    const int64_t m = d.rows;
    const unsigned n = unsigned(d.cols);
    const uint32_t nchunk = static_cast<uint32_t>((m + kTallRows - 1) / kTallRows);
    const int64_t r0 = int64_t(it.ti) * kTallRows;
    const int rows = int(min(m, r0 + kTallRows) - r0);
    const int64_t col = tall_col(unsigned(it.tj), ct, n);
    if (col >= n) continue;
    const float2 coef = ld2_agent(d.part + int64_t(it.tj) * (nchunk + 1) * kTallCols + 2 * ct +
                                  int64_t(nchunk) * kTallCols);
    for (int r = rg; r < rows; r += kTallThreads / 64) {
      const int64_t e = (r0 + r) * n + col;
      const float2 mm = make_float2(d.mom[e], d.mom[e + 1]);
      const float2 ww = make_float2(d.w[e], d.w[e + 1]);
      d.w[e] = fmaf(-coef.x, mm.x, ww.x * wkeep);
      d.w[e + 1] = fmaf(-coef.y, mm.y, ww.y * wkeep);
    }
  }
  __syncthreads();   // every thread is done with the list
  if (tid == 0 && atomicAdd(&ctl->repair_done, 1u) == gridDim.x - 1) {
    set_counter(&ctl->repair_count, 0u);
    set_counter(&ctl->repair_done, 0u);
  }
}

}  // namespace

hipError_t launch_rownorm_coef(hipStream_t s, const MatDev* mats, const TileItem* strips,
                               int64_t nstrips, StepScalars sc) {
  if (nstrips <= 0) return hipSuccess;
  static_assert(kColTileCols == kThreads, "one thread per strip column");
  rownorm_coef_kernel<<<dim3(static_cast<unsigned>(nstrips)), dim3(kThreads), 0, s>>>(mats, strips,
                                                                                     sc);
  return hipGetLastError();
}

hipError_t launch_rownorm_rows(hipStream_t s, const MatDev* mats, const int32_t* mat_ids,
                               const int64_t* row_prefix, int32_t nmat, int64_t total_rows,
                               int max_chunks, StepScalars sc) {
  if (total_rows <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(total_rows)), block(kThreads);
  switch (max_chunks) {
    case 1: rownorm_rows_kernel<1><<<grid, block, 0, s>>>(mats, mat_ids, row_prefix, nmat, sc); break;
    case 2: rownorm_rows_kernel<2><<<grid, block, 0, s>>>(mats, mat_ids, row_prefix, nmat, sc); break;
    case 4: rownorm_rows_kernel<4><<<grid, block, 0, s>>>(mats, mat_ids, row_prefix, nmat, sc); break;
    case 8: rownorm_rows_kernel<8><<<grid, block, 0, s>>>(mats, mat_ids, row_prefix, nmat, sc); break;
    case 16: rownorm_rows_kernel<16><<<grid, block, 0, s>>>(mats, mat_ids, row_prefix, nmat, sc); break;
    case 32: rownorm_rows_kernel<32><<<grid, block, 0, s>>>(mats, mat_ids, row_prefix, nmat, sc); break;
    default: rownorm_rows_kernel<0><<<grid, block, 0, s>>>(mats, mat_ids, row_prefix, nmat, sc); break;
  }
  return hipGetLastError();
}

hipError_t launch_rownorm_cols(hipStream_t s, const MatDev* mats, const TileItem* tiles,
                               int64_t ntiles, int phase, StepScalars sc) {
  if (ntiles <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(ntiles)), block(kThreads);
  if (phase == 1)
    rownorm_cols_kernel<1><<<grid, block, 0, s>>>(mats, tiles, sc);
  else
    rownorm_cols_kernel<2><<<grid, block, 0, s>>>(mats, tiles, sc);
  return hipGetLastError();
}

hipError_t launch_rownorm_tall(hipStream_t s, const MatDev* mats, const TileItem* tiles,
                               int64_t ntiles, TallSync* sync, TallCtl* ctl, uint32_t* repair,
                               uint32_t poll_limit, StepScalars sc) {
  if (ntiles <= 0) return hipSuccess;
  rownorm_tall_kernel<<<dim3(static_cast<unsigned>(ntiles)), dim3(kTallThreads), 0, s>>>(
      mats, tiles, sync, ctl, repair, static_cast<uint32_t>(ntiles), poll_limit, sc);
  return hipGetLastError();
}

hipError_t launch_rownorm_repair(hipStream_t s, const MatDev* mats, const TileItem* tiles,
                                 int64_t ntiles, TallCtl* ctl, const uint32_t* repair,
                                 StepScalars sc) {
  if (ntiles <= 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>(ntiles < 256 ? ntiles : 256);
  rownorm_tall_repair_kernel<<<dim3(grid), dim3(kTallThreads), 0, s>>>(
      mats, tiles, ctl, repair, static_cast<uint32_t>(ntiles), sc);
  return hipGetLastError();
}

hipError_t rownorm_tall_resident(int* workgroups_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(workgroups_per_cu, rownorm_tall_kernel,
                                                      kTallThreads, 0);
}

}  // namespace muon
