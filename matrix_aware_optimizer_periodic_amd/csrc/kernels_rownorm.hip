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

}  // namespace muon
