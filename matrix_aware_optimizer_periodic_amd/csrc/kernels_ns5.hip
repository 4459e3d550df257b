// Refresh step: momentum, Frobenius pre-normalisation and the Newton-Schulz
// iteration as batched MFMA GEMMs.
//
// "Scaling Muon for Diffusion Transformers" (abstract) and the PaperDaily
// post's section "Periodic Row-wise Muon" (text under blog fig. 3): on steps
// with t mod K == 0 the direction is NS5(M), five rounds of matrix products
// that push M towards its polar factor without an SVD.  Per round, on the
// wide orientation X (r x c, r <= c):
//
//     A = X X^T          (r x r x c, symmetric: upper tiles only, mirrored)
//     B = b A + c A A    (r x r x r, symmetric)
//     X = a X + B X      (r x c x r)
//
// and the last round writes W -= lr * X straight into the stored layout.
//
// Layout.  Every product is of the form C[i][j] = sum_k P[i][k] Q[j][k]:
// Gram P = Q = X; poly P = Q = A (symmetric); product P = B, Q = X^T.  bf16
// keeps X once (r x c), in two buffers that alternate between rounds; the
// product stages its Q operand as rows of X and reads it transposed from
// LDS.  bf16 X, A and B are k-block-major (ws_at): per block of 32 columns,
// all rows' 64 bytes one after another, so that every stage of every operand
// is read as whole 128-byte lines (row-major rows of 64 bytes per stage would
// be half lines, which cost the L2 as much as whole ones).  fp32 keeps X (r x c, updated in place) and X^T
// (c x r, two alternating buffers) and stages both operands along k.  A tall
// stored matrix (m > n) is X^T: the prep kernel forms X from it through an
// LDS transpose, and the last product writes W through its transposed
// mirror pass, so no separate transpose kernel runs.
// All workspace dims are padded to the tile size with zeros; zero padding is
// preserved exactly by the three products, so the GEMMs need no bounds
// checks and ragged shapes cost only the padded tiles.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "muon_internal.h"

namespace muon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef short bf16x4_raw_t __attribute__((ext_vector_type(4)));

// Pointers into global memory.  The workspace pointers come out of launch
// tables, so the compiler cannot tell they are global; without the address
// space it emits flat loads, which also count against the LDS wait counter
// and would make every LDS fragment wait also wait for in-flight global loads.
#define GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ GLOBAL T* as_global(T* p) {
  return (GLOBAL T*)(p);
}
template <typename T>
__device__ __forceinline__ const GLOBAL T* as_global(const T* p) {
  return (const GLOBAL T*)(p);
}

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16 with the hardware conversion (v_cvt_pk_bf16_f32: round to
// nearest even, NaN stays NaN), one value or a packed pair.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

__device__ __forceinline__ float load_g(const void* g, int gdt, int64_t idx) {
  if (gdt == 1) return bf16_to_f32(static_cast<const uint16_t*>(g)[idx]);
  return static_cast<const float*>(g)[idx];
}

// The four rows p0 + tr + 16 pass (pass = 0..3) of a prep tile, four columns
// each (whole, 16-byte aligned runs): M <- beta M + G, the new values in v.
// All loads go out before any store; rows at or past `rows` re-read row
// rows - 1 (no branch around a load), are not stored, and give zeros.  FULL:
// the whole tile is inside the block, so no row needs those checks (and the
// stores need no branches, which would make the compiler wait for every
// load before each of them).
template <int GDT, bool FULL>
__device__ __forceinline__ void prep_rows_vec(const MatDev& mt, int64_t ld, int64_t e0,
                                              int64_t p0, int64_t rows, float beta,
                                              float (&v)[4][4]) {
  f32x4_t g[4], m[4];
  float* mom = mt.mom;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int64_t e = (FULL ? p0 + 16 * pass : min(p0 + 16 * pass, rows - 1)) * ld + e0;
    if constexpr (GDT == 1) {
      const u32x2_t u = *as_global(reinterpret_cast<const u32x2_t*>(
          static_cast<const uint16_t*>(mt.g) + e));
      g[pass] = f32x4_t{bf16_to_f32(u[0] & 0xffffu), bf16_to_f32(u[0] >> 16),
                        bf16_to_f32(u[1] & 0xffffu), bf16_to_f32(u[1] >> 16)};
    } else {
      g[pass] = *as_global(reinterpret_cast<const f32x4_t*>(static_cast<const float*>(mt.g) + e));
    }
    m[pass] = *as_global(reinterpret_cast<const f32x4_t*>(mom + e));
  }
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int64_t p = p0 + 16 * pass;
    f32x4_t mm;
#pragma unroll
    for (int u = 0; u < 4; ++u) mm[u] = fmaf(beta, m[pass][u], g[pass][u]);
    if (FULL || p < rows) *as_global(reinterpret_cast<f32x4_t*>(mom + p * ld + e0)) = mm;
#pragma unroll
    for (int u = 0; u < 4; ++u) v[pass][u] = (FULL || p < rows) ? mm[u] : 0.f;
  }
}

// Offset of element (i, j) of a workspace array with `rows` rows.  bf16
// arrays (X, its remainder, A, B) are k-block-major: blocks of 32 columns,
// each holding every row's 32 values (64 bytes) one after another, so that
// one k-stage of any set of consecutive rows is a contiguous run of whole
// 128-byte lines, and 8 consecutive values of a row stay contiguous.  fp32
// arrays are row-major with leading dimension ld.
template <typename T>
__device__ __forceinline__ int64_t ws_at(int64_t i, int64_t j, int64_t rows, int64_t ld) {
  if constexpr (sizeof(T) == 2) return ((j >> 5) * rows + i) * 32 + (j & 31);
  return i * ld + j;
}

// The bf16 rounding remainders v - bf16(v) of four values whose bf16 pairs
// are packed in lo, hi, stored as bf16 (the second half of a two-term split
// of v: X = hi + remainder to about 16 significant bits).
__device__ __forceinline__ void store_rem4(uint16_t* o, const float v[4], uint32_t lo, uint32_t hi) {
  const float r0 = v[0] - bf16_to_f32(lo & 0xffffu), r1 = v[1] - bf16_to_f32(lo >> 16);
  const float r2 = v[2] - bf16_to_f32(hi & 0xffffu), r3 = v[3] - bf16_to_f32(hi >> 16);
  *as_global(reinterpret_cast<u32x2_t*>(o)) = u32x2_t{pack_bf16x2(r0, r1), pack_bf16x2(r2, r3)};
}

// ---------------------------------------------------------------------------
// Refresh-step preparation, one 64 x 64 tile of the padded stored block per
// workgroup: M <- beta M + G for the tile's valid elements, the tile's sum of
// squares (one partial per tile), and the new M, unscaled, cast to the
// workspace type: X = M (wide) or M^T (tall, through an LDS transpose) into
// x[0], and for fp32 also X^T into xt[0]; padding is written as 0.  Where
// the problem has xlo (bf16 with the remainder), X's bf16 rounding remainder
// X - bf16(X) goes there in the same layout.
// The pre-normalisation factor s = 1 / (||M||_F + eps) is applied by the
// first Newton-Schulz round instead (A = s^2 X X^T, X_1 = s (a X + B X)),
// which saves a second pass over M.
template <typename T>
__global__ __launch_bounds__(kThreads) void ns_prep_kernel(
    const MatDev* __restrict__ mats, const NsDev* __restrict__ ns,
    const TileItem* __restrict__ items, float beta) {
  __shared__ float tile[kPrepTile][kPrepTile + 1];
  __shared__ float red[4];
  const TileItem it = items[blockIdx.x];
  const NsDev d = ns[it.id];
  const MatDev mt = mats[d.mat];
  const int64_t p0 = int64_t(it.ti) * kPrepTile, q0 = int64_t(it.tj) * kPrepTile;
  // stored orientation and its transpose; bf16 keeps only X itself
  T* dst = static_cast<T*>(d.tall ? d.xt[0] : d.x[0]);
  const int64_t ldd = d.tall ? d.rp : d.cp;
  T* dstt = static_cast<T*>(d.tall ? d.x[0] : d.xt[0]);
  const int64_t ldt = d.tall ? d.cp : d.rp;
  const int tr = threadIdx.x >> 4, tc = (threadIdx.x & 15) * 4;
  const bool vec = ((d.ld | d.col0) & 3) == 0 && q0 + kPrepTile <= d.cols;
  float ss = 0.f;
  float vt[4][4];
  if (vec) {
    const int64_t e0 = d.col0 + q0 + tc;
    const bool full = p0 + kPrepTile <= d.rows;
    if (mt.gdt == 1) {
      if (full) prep_rows_vec<1, true>(mt, d.ld, e0, p0 + tr, d.rows, beta, vt);
      else prep_rows_vec<1, false>(mt, d.ld, e0, p0 + tr, d.rows, beta, vt);
    } else {
      if (full) prep_rows_vec<0, true>(mt, d.ld, e0, p0 + tr, d.rows, beta, vt);
      else prep_rows_vec<0, false>(mt, d.ld, e0, p0 + tr, d.rows, beta, vt);
    }
  } else {
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int64_t p = p0 + tr + 16 * pass;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        vt[pass][u] = 0.f;
        const int64_t e = p * d.ld + d.col0 + q0 + tc + u;
        if (p < d.rows && q0 + tc + u < d.cols) {
          const float m = fmaf(beta, mt.mom[e], load_g(mt.g, mt.gdt, e));
          mt.mom[e] = m;
          vt[pass][u] = m;
        }
      }
    }
  }
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int lr = tr + 16 * pass;
    const int64_t p = p0 + lr;
    const float* v = vt[pass];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ss += v[u] * v[u];
      tile[lr][tc + u] = v[u];
    }
    if (dst == nullptr) continue;
    T* o = dst + ws_at<T>(p, q0 + tc, d.rp, ldd);   // bf16: X itself (rp rows)
    if constexpr (sizeof(T) == 2) {
      const uint32_t lo = pack_bf16x2(v[0], v[1]);
      const uint32_t hi = pack_bf16x2(v[2], v[3]);
      *as_global(reinterpret_cast<u32x2_t*>(o)) = u32x2_t{lo, hi};
      if (d.xlo) store_rem4(static_cast<uint16_t*>(d.xlo) + ws_at<T>(p, q0 + tc, d.rp, ldd), v, lo, hi);
    } else {
      *as_global(reinterpret_cast<f32x4_t*>(o)) = f32x4_t{v[0], v[1], v[2], v[3]};
    }
  }
  const float tot = block_sum(ss, red);   // contains the barrier the transpose needs
  if (threadIdx.x == 0) d.part[int64_t(it.ti) * (d.tall ? d.rp : d.cp) / kPrepTile + it.tj] = tot;
  if (dstt == nullptr) return;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int lq = tr + 16 * pass;
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = tile[tc + u][lq];
    T* o = dstt + ws_at<T>(q0 + lq, p0 + tc, d.rp, ldt);   // bf16: X itself (rp rows)
    if constexpr (sizeof(T) == 2) {
      const uint32_t lo = pack_bf16x2(v[0], v[1]);
      const uint32_t hi = pack_bf16x2(v[2], v[3]);
      *as_global(reinterpret_cast<u32x2_t*>(o)) = u32x2_t{lo, hi};
      if (d.xlo) store_rem4(static_cast<uint16_t*>(d.xlo) + ws_at<T>(q0 + lq, p0 + tc, d.rp, ldt), v, lo, hi);
    } else {
      *as_global(reinterpret_cast<f32x4_t*>(o)) = f32x4_t{v[0], v[1], v[2], v[3]};
    }
  }
}

// s = 1 / (||M||_F + eps) per NS problem, partials added in a fixed order.
__global__ __launch_bounds__(kThreads) void ns_scale_kernel(NsDev* __restrict__ ns, float eps) {
  __shared__ float red[4];
  const NsDev d = ns[blockIdx.x];
  float s = 0.f;
  for (int k = threadIdx.x; k < d.nparts; k += kThreads) s += d.part[k];
  const float tot = block_sum(s, red);
  if (threadIdx.x == 0) d.scale[0] = 1.0f / (sqrtf(tot) + eps);
}

// ---------------------------------------------------------------------------
// Eight consecutive workspace values as fp32 (16 bytes of bf16 or 32 of fp32,
// always aligned: workspace rows are padded to the tile size).
template <typename T>
__device__ __forceinline__ void load8(const T* p, float v[8]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4_t u = *as_global(reinterpret_cast<const u32x4_t*>(p));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = bf16_to_f32(u[k] & 0xffffu);
      v[2 * k + 1] = bf16_to_f32(u[k] >> 16);
    }
  } else {
    const f32x4_t a = as_global(reinterpret_cast<const f32x4_t*>(p))[0];
    const f32x4_t b = as_global(reinterpret_cast<const f32x4_t*>(p))[1];
#pragma unroll
    for (int k = 0; k < 4; ++k) { v[k] = a[k]; v[4 + k] = b[k]; }
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float v[8]) {
  if constexpr (sizeof(T) == 2) {
    u32x4_t u;
#pragma unroll
    for (int k = 0; k < 4; ++k) u[k] = pack_bf16x2(v[2 * k], v[2 * k + 1]);
    *as_global(reinterpret_cast<u32x4_t*>(p)) = u;
  } else {
    as_global(reinterpret_cast<f32x4_t*>(p))[0] = f32x4_t{v[0], v[1], v[2], v[3]};
    as_global(reinterpret_cast<f32x4_t*>(p))[1] = f32x4_t{v[4], v[5], v[6], v[7]};
  }
}

// Eight values W[e0 .. e0 + 7] of a weight matrix for the update of the last
// Newton-Schulz round, W <- W keep - lr v, for the first nv of them:
// vectorised when the run is whole and aligned, else value by value (zeros
// past nv).  Loading and storing are separate calls, so that a batch of loads
// can be in flight while an earlier batch is stored.
struct W8 {
  f32x4_t a, b;
  __device__ __forceinline__ void load(const float* w, int64_t e0, int nv) {
    const GLOBAL float* gw = as_global(w) + e0;
    if (nv == 8 && (e0 & 3) == 0) {
      a = reinterpret_cast<const GLOBAL f32x4_t*>(gw)[0];
      b = reinterpret_cast<const GLOBAL f32x4_t*>(gw)[1];
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = (u < nv) ? gw[u] : 0.f;
        b[u] = (u + 4 < nv) ? gw[u + 4] : 0.f;
      }
    }
  }
  __device__ __forceinline__ void update_store(float* w, int64_t e0, int nv, const float v[8],
                                               float lr, float keep) const {
    float o[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      o[u] = fmaf(-lr, v[u], a[u] * keep);
      o[4 + u] = fmaf(-lr, v[4 + u], b[u] * keep);
    }
    GLOBAL float* gw = as_global(w) + e0;
    if (nv == 8 && (e0 & 3) == 0) {
      reinterpret_cast<GLOBAL f32x4_t*>(gw)[0] = f32x4_t{o[0], o[1], o[2], o[3]};
      reinterpret_cast<GLOBAL f32x4_t*>(gw)[1] = f32x4_t{o[4], o[5], o[6], o[7]};
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (u < nv) gw[u] = o[u];
    }
  }
};

// Eight workspace values kept as loaded (bf16 stays packed) until used.
template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> {
  u32x4_t u;
  __device__ __forceinline__ void load(const uint16_t* p) {
    u = *as_global(reinterpret_cast<const u32x4_t*>(p));
  }
  __device__ __forceinline__ void unpack(float v[8]) const {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = bf16_to_f32(u[k] & 0xffffu);
      v[2 * k + 1] = bf16_to_f32(u[k] >> 16);
    }
  }
};
template <> struct Raw8<float> {
  f32x4_t a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = as_global(reinterpret_cast<const f32x4_t*>(p))[0];
    b = as_global(reinterpret_cast<const f32x4_t*>(p))[1];
  }
  __device__ __forceinline__ void unpack(float v[8]) const {
#pragma unroll
    for (int k = 0; k < 4; ++k) { v[k] = a[k]; v[4 + k] = b[k]; }
  }
};

// GEMM tile C[i0.., j0..] = sum_k P[i][k] Q[j][k] on MFMA, BM x BN per
// workgroup of 2 x 2 waves (one per SIMD), each wave (BM/2) x (BN/2) built
// from MFMA blocks (16 x 16 x 32 for bf16 256-tiles, 32 x 32 otherwise); a
// 256-tile wave holds its 128 x 128 fp32 accumulators in the 256 AGPRs.
// BN = BM except for the 128 x 256 bf16 product tiles of short-K problems.
//
// Operand staging.  The k loop runs over stages of 64 bytes of k (32 bf16 or
// 16 fp32; in bf16 one k-block of the operand's layout) for all BM + BN rows
// of P and Q, NSTAGE stages deep in LDS (4 for
// 256-tiles, 5 for 128-tiles, 3 for 128 x 256).  Global data goes straight to LDS (MUBUF
// buffer_load ... lds: each lane's 16 bytes land at the wave's LDS base +
// 16 * lane), issued NSTAGE - 1 stages ahead of its use, so no registers
// hold operands in flight.  A 64-byte LDS row holds four 16-byte chunks,
// placed by a row swizzle (the DMA mapping below) so that the rows a 128-bit
// fragment read takes at once fall on distinct bank groups.  The bf16
// product stages its X operand as rows of X instead (see QT below) and
// reads it transposed.
//
// MFMA operand layout of the 32 x 32 variants (the 16 x 16 x 32 one is given
// with the fragment reads below): lane l supplies row
// (l & 31) of P and of Q; its k values are the 16-byte chunk 2g + (l >> 5) of
// k-group g.  bf16 32x32x16 consumes the chunk's 8 values at once; fp32
// 32x32x2 consumes its 4 values over 4 instructions.  Any pairing of k
// between the two operands is valid as long as it is the same for both.
// Accumulator element v of lane l is C[8 (v/4) + 4 (l/32) + (v%4)][l & 31].
//
// Epilogue.  A bf16 product before the last round stores the next X straight
// from the accumulators (two 64-byte row runs per accumulator register in the
// k-block-major layout).  Every other epilogue works per pass over rows of
// the tile (as many as the workgroup's LDS share holds in fp32): the waves
// owning them park their accumulators in LDS, then all threads write the
// outputs in 16-byte chunks, first along rows (C, or W of a wide matrix),
// then along columns (the mirrored half of a symmetric A or B, X^T in fp32,
// or W of a tall matrix).
//
// Rounding.  The diagonal of A stays in fp32 (adiag), and the A_ii^2 term of
// (A A)_ii and the b A_ii term use it.  B's diagonal a + B_ii (the product
// applies aI + B) is kept to about 2^-18: fp32 stores 0 in B and applies
// (a + B_ii) X_i in fp32 in the epilogue; bf16 stores bf16(a + B_ii) in B and
// adds the remainder with extra diagonal MFMAs.  This is the same arithmetic,
// rounded later: it avoids the cancellation between a and B_ii that plain
// bf16 storage of B_ii would amplify when the short side r is small.
#define LOCAL __attribute__((address_space(3)))

// s_waitcnt vmcnt(N) for the DMA counts the GEMM pipeline uses.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16 bytes per lane from a raw buffer straight into LDS (lane l lands at
// lds_addr + 16 l).  Issued as inline asm so that the compiler does not
// model these LDS writes: it cannot tell them apart from the transposed LDS
// reads, and would otherwise drain every DMA in flight before each such
// read.  The GEMM pipeline orders them itself (explicit vmcnt waits and
// barriers).
__device__ __forceinline__ void dma16(u32x4_t rsrc, unsigned lds_addr, unsigned voff,
                                      unsigned soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
      : "m0");
}

// 4 bytes per lane from a raw buffer straight into LDS (lane l lands at
// lds_addr + 4 l); same conventions as dma16.
__device__ __forceinline__ void dma4(u32x4_t rsrc, unsigned lds_addr, unsigned voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(lds_addr), "v"(voff), "s"(rsrc)
      : "m0");
}

// Raw buffer resource: base, stride 0, byte size (reads past it return 0).
__device__ __forceinline__ u32x4_t buffer_rsrc(const void* p, int64_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return u32x4_t{unsigned(a), unsigned(a >> 32) & 0xffffu, unsigned(nbytes), 0x00020000u};
}

template <typename T, int BM, int WGM, int WGN, int OP, int BN = BM, bool XLO = false>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void ns_gemm_kernel(
    const MatDev* __restrict__ mats, const NsDev* __restrict__ ns,
    const GemmItem* __restrict__ items, int iter, float ca, float cb, float cc,
    float wd) {
  // OP kGemmProductLast is the product of the last round (updates W).
  constexpr bool PROD = OP == kGemmProduct || OP == kGemmProductLast;
  constexpr bool last = OP == kGemmProductLast;
  // bf16 product: the X operand is staged as rows of X (32 rows of k by the
  // tile's BN columns) and read with transposed LDS loads.
  constexpr bool QT = PROD && sizeof(T) == 2;
  // XLO (bf16 products with X's remainder): the a X term also takes a xlo,
  // and a round before the last stores its output's remainder back to xlo.
  static_assert(!XLO || QT, "the remainder is a bf16 product option");
  constexpr int NW = WGM * WGN;
  constexpr int NT = 64 * NW;                // threads
  // Output tiles are BM x BN: square except for the bf16 product, which may
  // take wider tiles (more flops per staged byte).
  static_assert(BN == BM || (OP == kGemmProduct && sizeof(T) == 2), "wide tiles: bf16 product");
  constexpr int WM = BM / WGM, WN = BN / WGN;
  // MFMA block: 16 x 16 x 32 for bf16 256-tiles, 32 x 32 x 16 (bf16) or
  // 32 x 32 x 2 (fp32) otherwise.  At the package power limit the 16 x 16 x
  // 32 form runs the same flops at a higher clock; the 128-tile kernels,
  // two workgroups per CU, lack the registers for its fragment buffers.
  constexpr int MF = sizeof(T) == 2 && BM >= 256 ? 16 : 32;
  constexpr int FM = WM / MF, FN = WN / MF;
  constexpr int NV = MF * MF / 64;           // accumulators per lane per block
  constexpr int ROWS = BM + BN;              // P rows then Q rows (64 bytes each)
  // Stages in the LDS ring: 4 for 256-tiles (of 160 KB), 5 for 128-tiles
  // and 3 for 128 x 256 (within 80 KB: two workgroups per CU); deeper rings
  // measured no faster.
  constexpr int NSTAGE = BM >= 256 ? 4 : BN > BM ? 3 : 5;
  constexpr int STAGE = ROWS * 64;           // bytes per stage
  constexpr int BLOCKS = ROWS / 16;          // 16-row (1 KB) DMA blocks per stage
  constexpr int DMA = BLOCKS / NW;           // DMA instructions per wave per stage
  constexpr int DMAP = BM / 16 / NW;         // of which for P
  constexpr int KT = 64 / int(sizeof(T));    // k elements per stage
  constexpr int SLD = BN + 4;                // epilogue stage row stride (floats)
  // Epilogue rows per pass: as many as the fp32 stage fits in the workgroup's
  // LDS share (160 KB for 256-tiles, 80 KB for 128-tiles, two per CU).
  constexpr int LDS_MAX = (BM >= 256 ? 160 : 80) * 1024;
  constexpr int NPASS = BM * SLD * 4 <= LDS_MAX ? 1 : (BM / 2) * SLD * 4 <= LDS_MAX ? 2 : 4;
  constexpr int HALF = BM / NPASS;
  constexpr int MAIN_BYTES = NSTAGE * STAGE;
  constexpr int STAGE_BYTES = HALF * SLD * 4;
  constexpr int SMEM = MAIN_BYTES > STAGE_BYTES ? MAIN_BYTES : STAGE_BYTES;
  static_assert(HALF % 32 == 0 && MAIN_BYTES <= LDS_MAX, "whole 32-row blocks per pass");
  static_assert((BM / 16) % NW == 0 && (BN / 16) % NW == 0, "whole DMA blocks per wave");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM];
  const u32x4_t* lds = reinterpret_cast<const u32x4_t*>(smem);

  const GemmItem it = items[blockIdx.x];
  const NsDev d = ns[it.ns];
  const int cur = iter & 1;
  // X of this round: bf16 alternates x[0] / x[1]; fp32 keeps it in x[0].
  const T* xcur = static_cast<const T*>(sizeof(T) == 2 && cur ? d.x[1] : d.x[0]);
  const T* P;
  const T* Q;
  int64_t ld, ldq, K;
  if constexpr (OP == kGemmGram) {
    P = Q = xcur; ld = ldq = d.cp; K = d.cp;
  } else if constexpr (OP == kGemmPoly) {
    P = Q = static_cast<const T*>(d.a); ld = ldq = d.rp; K = d.rp;
  } else {
    static_assert(PROD, "unknown op");
    P = static_cast<const T*>(d.b);
    ld = d.rp;
    K = d.rp;
    if constexpr (QT) {
      Q = xcur; ldq = d.cp;                  // X itself, rows k
    } else {
      Q = static_cast<const T*>(cur ? d.xt[1] : d.xt[0]); ldq = d.rp;   // X^T, rows j
    }
  }
  const int64_t i0 = int64_t(it.ti) * BM, j0 = int64_t(it.tj) * BN;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WGN, wn = wid % WGN;
  const int nk = int(K / KT);

  // DMA mapping.  Instruction q of wave w fills LDS rows 16 b .. 16 b + 15 of
  // the stage, b = w + NW q; lane l brings row r = 16 b + (l >> 2), logical
  // chunk (l & 3) ^ sw(r), which lands at physical chunk l & 3.  The row
  // swizzle sw(r) is (r >> 2) & 3 for 32 x 32 fragments (a 128-bit read then
  // takes 32 rows at one logical chunk) and (r >> 1) & 3 for 16 x 16
  // fragments (16 rows at each of the four chunks): measured on gfx950, each
  // keeps its fragment reads free of bank conflicts, and the other would
  // double their LDS cycles.
  // Blocks q < DMAP are P rows, the others Q rows.  The loads are MUBUF
  // buffer loads into LDS: unlike the FLAT form they count only against the
  // vector-memory counter, so waiting for LDS fragment reads does not also
  // wait for the prefetch in flight.  Offsets past a buffer's end read 0.
  //
  // QT: the Q part of a stage is X rows k .. k + 31, columns j0 .. j0 + BN - 1
  // (2 BN bytes per row in LDS, CPRQ 16-byte chunks; in memory, BN / 32
  // k-blocks of 32 rows x 64 bytes, 2 KB each); DMA block b holds rows
  // RPB b .. RPB b + RPB - 1 and lane l brings row RPB b + l / CPRQ, logical
  // chunk (l % CPRQ) ^ ((row & 3) << 2), which lands at physical chunk
  // l % CPRQ.  The XOR puts the four rows a transposed read touches in four
  // distinct 64-byte bank groups.
  const int drow = 16 * wid + (lane >> 2);
  const int dchunk = (lane & 3) ^ (MF == 16 ? (lane >> 3) & 3 : (lane >> 4) & 3);
  constexpr int CPRQ = BN / 8, RPB = 64 / CPRQ;
  static_assert(!QT || (RPB * CPRQ == 64 && (RPB * NW) % 4 == 0),
                "whole rows per DMA block; row phase of a lane fixed across its blocks");
  // With 16 x 16 x 32 MFMAs the four lane groups of a transposed read take
  // rows 8 apart (k 0-7, 8-15, ...) of the same columns; bit 3 of the row
  // then also flips bit 1 of the chunk, so that two groups served together
  // land in different banks.  A wave's blocks are 8 rows apart there, so
  // that bit alternates with the block.
  constexpr bool QSW8 = QT && MF == 16;
  static_assert(!QSW8 || RPB * NW == 8, "QT swizzle: row bit 3 alternates with the DMA block");
  const int qtrow = RPB * wid + lane / CPRQ;
  const int qtchunk = (lane % CPRQ) ^ ((qtrow & 3) << 2);
  const int qtchunk1 = qtchunk ^ (QSW8 ? 2 : 0);   // odd blocks (QSW8)
  const int64_t prow = d.rp;   // P is X, A or B: rp rows
  const int64_t qrow = QT ? d.rp : (PROD ? d.cp : d.rp);
  const u32x4_t rP = buffer_rsrc(P, prow * ld * int64_t(sizeof(T)));
  const u32x4_t rQ = buffer_rsrc(Q, qrow * ldq * int64_t(sizeof(T)));
  // bf16 operands are k-block-major (ws_at): a stage of P or Q rows is one
  // contiguous run (64 B per row), and QT's 32 rows of X are, per 32
  // columns, 2 KB contiguous.  fp32 operands are row-major.
  constexpr bool BLK = sizeof(T) == 2;
  const unsigned offP = BLK ? unsigned((i0 + drow) * 64 + dchunk * 16)
                            : unsigned((i0 + drow) * ld * int64_t(sizeof(T))) + unsigned(dchunk * 16);
  const unsigned rstride = BLK ? unsigned(16 * NW * 64) : unsigned(int64_t(16 * NW) * ld * int64_t(sizeof(T)));
  const unsigned offQ =
      QT ? unsigned((j0 / 32 + qtchunk / 4) * qrow * 64 + qtrow * 64 + (qtchunk % 4) * 16)
         : BLK ? unsigned((j0 + drow) * 64 + dchunk * 16)
               : unsigned((j0 + drow) * ldq * int64_t(sizeof(T))) + unsigned(dchunk * 16);
  const unsigned offQ1 =
      QSW8 ? unsigned((j0 / 32 + qtchunk1 / 4) * qrow * 64 + qtrow * 64 + (qtchunk1 % 4) * 16) : offQ;
  const unsigned rstrideQ = BLK ? unsigned((QT ? RPB * NW : 16 * NW) * 64)
                                : unsigned(int64_t(16 * NW) * ldq * int64_t(sizeof(T)));
  // bytes per stage along k: P, one k-block of all prow rows (bf16) or 64;
  // Q, likewise, or (QT) KT rows of one k-block
  const int64_t kstepP = BLK ? prow * 64 : 64;
  const int64_t kstepQ = QT ? int64_t(KT) * 64 : BLK ? qrow * 64 : 64;
  // Stages past the end are issued as a reload of the last stage: the loop
  // body then has no branches (exact wait counts), and the buffer such a
  // reload lands in is one no wave reads any more.
  // The per-lane byte offsets do not change along k: they stay in VGPRs, and
  // the stage's k offset goes in the scalar offset.  The LDS destination
  // (M0) is wave-uniform scalar arithmetic too, so a DMA costs two scalar
  // instructions and the load.
  // (A local array of these offsets captured by the lambda below makes the
  // host compilation pass drop this kernel's launch stub, silently.)
  const int swid = __builtin_amdgcn_readfirstlane(wid);
  auto issue_one = [&](int kt, int q) {
    const int kc = min(kt, nk - 1);
    LOCAL unsigned char* base =
        (LOCAL unsigned char*)(smem + (kt % NSTAGE) * STAGE + swid * 1024);
    const unsigned kb = q < DMAP ? unsigned(kc * kstepP) : unsigned(kc * kstepQ);
    const unsigned voff = q < DMAP ? offP + unsigned(q) * rstride
                                   : ((q - DMAP) & 1 ? offQ1 : offQ) + unsigned(q - DMAP) * rstrideQ;
    dma16(q < DMAP ? rP : rQ, unsigned(uintptr_t(base + q * NW * 1024)), voff, unsigned(kb));
  };
  auto issue = [&](int kt) {
#pragma unroll
    for (int q = 0; q < DMA; ++q) issue_one(kt, q);
  };

  using AccV = std::conditional_t<MF == 16, f32x4_t, f32x16_t>;
  AccV acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b) {
      acc[a][b] = (AccV)(0.0f);
      // Gram and polynomial: give every accumulator its AGPRs from the start;
      // otherwise the allocator keeps one block in VGPRs across the main loop
      // and rotates others through a spare AGPR tuple, some 90 moves a stage.
      if constexpr (MF == 16 && !PROD) asm volatile("" : "+a"(acc[a][b]));
    }
  // Row and column within an MFMA block of accumulator v of this lane.
  auto acc_row = [&](int v) { return MF == 16 ? 4 * (lane >> 4) + v : 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); };
  const int acc_col = lane & (MF - 1);

  // QT: the remainders lo_i of this wave's output rows (WM values from
  // bdiag) come by DMA too, into the ring slot of stage NSTAGE - 1, which is
  // not filled before the first loop iteration; issued ahead of the stages,
  // the prologue's wait covers them.  (A plain load here would make the
  // compiler wait for every DMA in flight before its first use.)
  constexpr int DLO_SLOT = (NSTAGE - 1) * STAGE;
  static_assert(!QT || (WM % 64 == 0 && NW * WM * 4 <= STAGE), "dlo staging");
  if constexpr (QT) {
    const u32x4_t rD = buffer_rsrc(d.bdiag, d.rp * int64_t(sizeof(float)));
#pragma unroll
    for (int h = 0; h < WM / 64; ++h)
      dma4(rD, unsigned(uintptr_t(smem + DLO_SLOT + (swid * WM + 64 * h) * 4)),
           unsigned((i0 + wm * WM + 64 * h + lane) * int64_t(sizeof(float))));
  }
  for (int s0 = 0; s0 < NSTAGE - 1; ++s0) issue(s0);

  // MFMA operand fragments: lane l holds 8 consecutive k (16 bytes) of row
  // (or column) l % MF of the fragment, k = 8 (l / MF) .. + 7 within the
  // k-group (16 k for 32 x 32 x 16, the stage's 32 for 16 x 16 x 32).
  const int frow = lane & (MF - 1), fhalf = lane / MF;
  const int fsw = MF == 16 ? (frow >> 1) & 3 : (frow >> 2) & 3;   // sw(row) of the lane's row
  // QT fragments.  ds_read_b64_tr_b16 works on groups of 16 lanes: lane i of
  // a group receives element i & 3 of the 8 bytes addressed by lane
  // 4 e + (i >> 2), for e = 0..3.  Lane s of a group therefore addresses row
  // k0 + (s >> 2), columns c0 + 4 (s & 3) .. + 3, and lane i receives column
  // c0 + i of rows k0 .. k0 + 3: four consecutive k of one column of X, as
  // the MFMA operand wants them.  Two such reads (h = 0, 1) give a lane its
  // 8 k values: k = 16 g + 8 (l >> 5) + 4 h + e, column (l & 31) of the
  // fragment (32 x 32 x 16); k = 8 (l >> 4) + 4 h + e, column (l & 15)
  // (16 x 16 x 32).
  const int trow = 8 * fhalf + ((lane & 15) >> 2);                 // + 16 g + 4 h
  const int tcol = (MF == 32 ? 16 * ((lane >> 4) & 1) : 0) + 4 * (lane & 3);   // + fragment column
  const int tsw = ((trow & 3) << 2) ^ (QSW8 ? ((trow >> 3) & 1) << 1 : 0);
  auto qtr = [&](const u32x4_t* sQ, int g, int f, int h, u32x4_t& out) {
    const int row = 16 * g + 4 * h + trow;
    const int col = wn * WN + f * MF + tcol;
    const int byte = row * (2 * BN) + (((col >> 3) ^ tsw) << 4) + ((col & 7) << 1);
    const LOCAL bf16x4_raw_t* p =
        (const LOCAL bf16x4_raw_t*)((const LOCAL unsigned char*)sQ + byte);
    const u32x2_t w = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                          (LOCAL bf16x4_raw_t*)p));
    out[2 * h] = w[0];
    out[2 * h + 1] = w[1];
  };
  // Fragments of k-group g (16 k values) of one stage.
  auto frag = [&](const u32x4_t* sP, const u32x4_t* sQ, int g, u32x4_t* fa, u32x4_t* fb) {
    const int ch = (2 * g + fhalf) ^ fsw;
#pragma unroll
    for (int f = 0; f < FM; ++f) fa[f] = sP[(wm * WM + f * MF + frow) * 4 + ch];
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      if constexpr (QT) {
        qtr(sQ, g, f, 0, fb[f]);
        qtr(sQ, g, f, 1, fb[f]);
      } else {
        fb[f] = sQ[(wn * WN + f * MF + frow) * 4 + ch];
      }
    }
  };
  // One LDS read of k-group g: index f < FM is P fragment f; after that Q
  // fragments, one read each, or (QT) two transposed reads each.
  auto frag_one = [&](const u32x4_t* sP, const u32x4_t* sQ, int g, int f, u32x4_t* fa,
                      u32x4_t* fb) {
    const int ch = (2 * g + fhalf) ^ fsw;
    if (f < FM) {
      fa[f] = sP[(wm * WM + f * MF + frow) * 4 + ch];
    } else if constexpr (QT) {
      qtr(sQ, g, (f - FM) >> 1, (f - FM) & 1, fb[(f - FM) >> 1]);
    } else {
      fb[f - FM] = sQ[(wn * WN + (f - FM) * MF + frow) * 4 + ch];
    }
  };
  // MFMAs of one k-group over the flattened fragment pairs [lo, hi).
  auto mma = [&](const u32x4_t* fa, const u32x4_t* fb, int lo, int hi) {
#pragma unroll
    for (int xy = 0; xy < FM * FN; ++xy) {
      if (xy < lo || xy >= hi) continue;
      const int x = xy / FN, y = xy % FN;
      if constexpr (MF == 16) {
        acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, fa[x]), __builtin_bit_cast(bf16x8_t, fb[y]), acc[x][y],
            0, 0, 0);
      } else if constexpr (sizeof(T) == 2) {
        acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, fa[x]), __builtin_bit_cast(bf16x8_t, fb[y]), acc[x][y],
            0, 0, 0);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x2f32(
              __uint_as_float(fa[x][s]), __uint_as_float(fb[y][s]), acc[x][y], 0, 0, 0);
      }
    }
  };
  // Software pipeline, two k-groups (g0, g1) per stage.  With one wave per
  // SIMD the matrix core idles whenever its wave issues anything but MFMAs,
  // so the other instructions are spread between MFMAs in fixed slots (one
  // MFMA pair, then at most one DMA and one LDS fragment read; sched_barrier
  // keeps each slot together), and the workgroup barrier sits behind MFMAs
  // already issued.
  //
  // Iteration kt starts with the g0 fragments of stage kt in registers.
  //   part 1: MFMAs of g0, with the LDS reads of the g1 fragments of stage kt
  //           (landed and visible since the barrier of iteration kt - 1)
  //           between them; then the first PRE MFMAs of g1.
  //   wait for this wave's DMA of stage kt + 1, then the barrier: every part
  //   of stage kt + 1 is in LDS, and every wave has finished reading stage
  //   kt - 1, whose buffer the DMA of stage kt + NSTAGE - 1 refills.
  //   part 2: the rest of g1's MFMAs, with the DMA of stage kt + NSTAGE - 1 and the
  //           LDS reads of the g0 fragments of stage kt + 1 between them.
  // The barrier is a bare s_barrier: __syncthreads() would add a release
  // fence that waits for every DMA in flight, i.e. for the stages
  // prefetched ahead.
  auto stage_ptrs = [&](int kt, const u32x4_t*& sP, const u32x4_t*& sQ) {
    sP = lds + (kt % NSTAGE) * (STAGE / 16);
    sQ = sP + BM * 4;
  };
  auto bar = [&]() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  if constexpr (MF == 16) {
    // One k-group per stage: its 32 k feed the FM x FN 16 x 16 x 32 MFMAs,
    // in two halves by column (y < HB, then y >= HB), each row by row.  One
    // set of fragments, a[] and b[], is refilled with the next stage's as the
    // current one frees up: b[y] after its last MFMA (in the last row of its
    // half), a[x] after row x of the second half.  Each refill then has about
    // half a stage (30-36 MFMAs) before the next stage needs it.  The reads
    // of stage kt + 1 may start after the barrier, which comes after the
    // first PRE MFMAs: by then every wave has issued all its reads of stage
    // kt (during stage kt - 1), so the DMA may refill stage kt - 1's buffer.
    constexpr int NXY = FM * FN;
    constexpr int HB = FN / 2;                   // columns per half
    constexpr int PRE = 2;                       // MFMAs issued before the barrier
    constexpr int NBR = QT ? 2 : 1;              // LDS reads per B fragment
    const int fch = fhalf ^ fsw;                 // the lane's 16-byte chunk of a P or Q row
    u32x4_t a[FM], b[FN];
    float dlo[FM];
    const int kf0 = int(it.ti) * (BM / 32) + (swid / WGN) * (WM / 32);
    auto rd_a = [&](const u32x4_t* sP, int x) { a[x] = sP[(wm * WM + x * 16 + frow) * 4 + fch]; };
    auto rd_b = [&](const u32x4_t* sQ, int y, int h) {
      if constexpr (QT) qtr(sQ, 0, y, h, b[y]);
      else b[y] = sQ[(wn * WN + y * 16 + frow) * 4 + fch];
    };
    // MFMA i of a stage: half i / (FM HB), row, then column within the half.
    auto ix = [&](int i) { return (i % (FM * HB)) / HB; };
    auto iy = [&](int i) { return (i / (FM * HB)) * HB + i % HB; };
    auto mma16 = [&](int i) {
      const int x = ix(i), y = iy(i);
      acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8_t, a[x]), __builtin_bit_cast(bf16x8_t, b[y]), acc[x][y], 0, 0, 0);
    };
    {
      wait_vmcnt<(NSTAGE - 2) * DMA>();   // stage 0 is in; stages 1 .. NSTAGE-2 may be in flight
      bar();
      if constexpr (QT) {
        const float* sd = reinterpret_cast<const float*>(smem + DLO_SLOT) + wid * WM;
#pragma unroll
        for (int fa = 0; fa < FM; ++fa) dlo[fa] = sd[fa * 16 + (lane & 15)];
      }
      const u32x4_t *sP, *sQ;
      stage_ptrs(0, sP, sQ);
#pragma unroll
      for (int x = 0; x < FM; ++x) rd_a(sP, x);
#pragma unroll
      for (int y = 0; y < FN; ++y)
#pragma unroll
        for (int h = 0; h < NBR; ++h) rd_b(sQ, y, h);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    // Every iteration issues exactly DMA loads, so after the wait below the
    // DMAs in flight are those of stages kt + 2 .. kt + NSTAGE - 2.  The
    // fragment reads of stage nk (past the end) read a reloaded buffer and
    // are never used.  DM >= 0: stage kf0 + DM, which also takes the
    // diagonal remainder MFMAs of fragment rows 2 DM and 2 DM + 1.  Those four
    // stages are peeled out of the loop (QT): conditional MFMA blocks inside
    // it cost the product about 5% (measured).
    auto body = [&](int kt, auto dmv) {
      constexpr int DM = decltype(dmv)::value;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < PRE; ++i) {
        mma16(i);
        __builtin_amdgcn_sched_barrier(0);
      }
      wait_vmcnt<(NSTAGE - 3) * DMA>();
      bar();
      __builtin_amdgcn_sched_barrier(0);
      const u32x4_t *sP, *sQ;
      if constexpr (QT) {
        // Stage kt = kf0 + DM holds rows 32 kt .. 32 kt + 31 of X: for
        // fa = 2 DM, 2 DM + 1 the X_i of this wave's output rows.  Add lo_i X_i
        // with MFMAs whose A operand is diag(lo) over those 16 rows (B
        // itself carries bf16(a + B_ii) on its diagonal).
        // fragment rows 2 m and 2 m + 1 (m static after unrolling)
        auto diag = [&](int m) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int fa = 2 * m + hh;
            const uint32_t bits = f32_to_bf16(dlo[fa]);
            const int e = 16 * hh + (lane & 15) - 8 * (lane >> 4);
            u32x4_t f = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2)
              f[w2] = (e >= 0 && e < 8 && (e >> 1) == w2) ? bits << (16 * (e & 1)) : 0u;
#pragma unroll
            for (int y = 0; y < FN; ++y)
              acc[fa][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, f), __builtin_bit_cast(bf16x8_t, b[y]),
                  acc[fa][y], 0, 0, 0);
          }
        };
        if constexpr (DM >= 0) {
          diag(DM);
        } else if constexpr (DM == -2) {   // the stage decides at run time
#pragma unroll
          for (int m = 0; m < FM / 2; ++m)
            if (kt == kf0 + m) diag(m);
        }
      }
      stage_ptrs(kt + 1, sP, sQ);
      // After MFMA i: the DMAs of stage kt + NSTAGE - 1 in the first slots,
      // the reads of stage kt + 1's b[y] once MFMA (FM - 1, y) is issued, and
      // of its a[x] once row x of the second half is.
      int nd = 0;
#pragma unroll
      for (int i = PRE; i < NXY; ++i) {
        mma16(i);
        const int x = ix(i), y = iy(i);
        if (nd < DMA && i % 2 == 0) { issue_one(kt + NSTAGE - 1, nd); ++nd; }
        if (x == FM - 1) {
#pragma unroll
          for (int h = 0; h < NBR; ++h) rd_b(sQ, y, h);
        }
        if (y == FN - 1) rd_a(sP, x);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (; nd < DMA; ++nd) issue_one(kt + NSTAGE - 1, nd);
      __builtin_amdgcn_sched_barrier(0);
    };
    using NoDiag = std::integral_constant<int, -1>;
    if constexpr (QT && !last) {
      static_assert(FM == 8, "four diagonal stages of two fragment rows each");
      // the wave's output rows are rows of X inside K, so kf0 + 3 < nk
      int kt = 0;
      for (; kt < kf0; ++kt) body(kt, NoDiag{});
      body(kt, std::integral_constant<int, 0>{});
      body(kt + 1, std::integral_constant<int, 1>{});
      body(kt + 2, std::integral_constant<int, 2>{});
      body(kt + 3, std::integral_constant<int, 3>{});
      for (kt += 4; kt < nk; ++kt) body(kt, NoDiag{});
    } else if constexpr (QT) {
      // The last product keeps the test inside its loop: peeled, the
      // diagonal stages cost its weight-update epilogue registers (a spill).
      for (int kt = 0; kt < nk; ++kt) body(kt, std::integral_constant<int, -2>{});
    } else {
      for (int kt = 0; kt < nk; ++kt) body(kt, NoDiag{});
    }
  } else {
    constexpr int NXY = FM * FN;                       // fragment pairs per k-group
    constexpr int PRE = NXY >= 16 ? 2 : 1;             // g1 pairs issued before the barrier
    constexpr int NRD = FM + (QT ? 2 : 1) * FN;        // LDS reads per k-group
    u32x4_t a0[FM], b0[FN], a1[FM], b1[FN];
    // QT: remainder lo_i of the diagonal a + B_ii for row (lane & 31) of each
    // fragment row fa, and the stage that holds those rows of X for fa = 0.
    float dlo[FM];
    const int kf0 = int(it.ti) * (BM / 32) + (swid / WGN) * FM;   // scalar: a uniform branch
    {
      wait_vmcnt<(NSTAGE - 2) * DMA>();   // stage 0 is in; stages 1 .. NSTAGE-2 may be in flight
      bar();
      if constexpr (QT) {
        const float* sd = reinterpret_cast<const float*>(smem + DLO_SLOT) + wid * WM;
  #pragma unroll
        for (int fa = 0; fa < FM; ++fa) dlo[fa] = sd[fa * 32 + (lane & 31)];
      }
      const u32x4_t *sP, *sQ;
      stage_ptrs(0, sP, sQ);
      frag(sP, sQ, 0, a0, b0);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    // Every iteration issues exactly DMA loads, so after the waits below the
    // DMAs in flight are those of stages kt + 2 .. kt + NSTAGE - 2.  The fragment reads of stage
    // nk (past the end) read a reloaded buffer and are never used.
    for (int kt = 0; kt < nk; ++kt) {
      __builtin_amdgcn_sched_barrier(0);
      {
        const u32x4_t *sP, *sQ;
        stage_ptrs(kt, sP, sQ);
  #pragma unroll
        for (int i = 0; i < NXY; ++i) {
          mma(a0, b0, i, i + 1);
          if (i < NRD) frag_one(sP, sQ, 1, i, a1, b1);
          __builtin_amdgcn_sched_barrier(0);
        }
  #pragma unroll
        for (int i = NXY; i < NRD; ++i) frag_one(sP, sQ, 1, i, a1, b1);
  #pragma unroll
        for (int i = 0; i < PRE; ++i) {
          mma(a1, b1, i, i + 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (QT) {
          // Stage kt holds rows 32 kt .. 32 kt + 31 of X, i.e. (for one fa)
          // X_i of this wave's output rows: add lo_i X_i with MFMAs whose P
          // operand is diag(lo) over those 32 rows (B itself carries bf16(a +
          // B_ii) on its diagonal).
  #pragma unroll
          for (int fa = 0; fa < FM; ++fa) {
            if (kt == kf0 + fa) {
              const uint32_t bits = f32_to_bf16(dlo[fa]);
  #pragma unroll
              for (int g = 0; g < 2; ++g) {
                const int e = (lane & 31) - 16 * g - 8 * (lane >> 5);
                u32x4_t f = {0u, 0u, 0u, 0u};
  #pragma unroll
                for (int w2 = 0; w2 < 4; ++w2)
                  f[w2] = (e >= 0 && (e >> 1) == w2) ? bits << (16 * (e & 1)) : 0u;
  #pragma unroll
                for (int y = 0; y < FN; ++y)
                  acc[fa][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                      __builtin_bit_cast(bf16x8_t, f),
                      __builtin_bit_cast(bf16x8_t, g ? b1[y] : b0[y]), acc[fa][y], 0, 0, 0);
              }
            }
          }
        }
      }
      wait_vmcnt<(NSTAGE - 3) * DMA>();
      bar();
      __builtin_amdgcn_sched_barrier(0);
      {
        const u32x4_t *sP, *sQ;
        stage_ptrs(kt + 1, sP, sQ);
        // Each slot carries up to two of the DMAs and LDS reads, alternating
        // while both remain.
        int nd = 0, nr = 0;
  #pragma unroll
        for (int i = PRE; i < NXY; ++i) {
          mma(a1, b1, i, i + 1);
  #pragma unroll
          for (int u = 0; u < 2; ++u) {
            if (nd < DMA && (nr >= NRD || nd <= nr)) { issue_one(kt + NSTAGE - 1, nd); ++nd; }
            else if (nr < NRD) { frag_one(sP, sQ, 0, nr, a0, b0); ++nr; }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
  #pragma unroll
        for (; nd < DMA; ++nd) issue_one(kt + NSTAGE - 1, nd);
  #pragma unroll
        for (; nr < NRD; ++nr) frag_one(sP, sQ, 0, nr, a0, b0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmcnt<0>();

  // ---- epilogue -----------------------------------------------------------
  // bf16 product of a round before the last: the next X straight from the
  // accumulators.  In the k-block-major layout, accumulator v of a 32 x 32
  // MFMA block holds across lanes 0-31 (and 32-63) 32 consecutive values of
  // one row (and of the row 4 below), 64 contiguous bytes each: a 2-byte
  // store per lane writes whole 128-byte lines, with no LDS staging and no
  // barrier.  In a 16 x 16 block each group of 16 lanes holds 16 values (32
  // bytes) of one row, and the neighbouring block the other half of the
  // row's 64 bytes.
  if constexpr (QT && !last) {
    // Buffer stores: the lane's offset in a VGPR, the block's (wave-uniform)
    // in an SGPR, the row within the block as the instruction's immediate.
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        cur ? d.x[0] : d.x[1], 0, int(d.rp * d.cp * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
        d.xlo, 0, XLO ? int(d.rp * d.cp * 2) : 0, 0x00020000);
    const float s0 = iter == 0 ? d.scale[0] : 1.0f;   // round 0 works on the unscaled M
    const int voff = (acc_row(0) * 32 + acc_col) * 2;
    const int swm = swid / WGN, swn = swid % WGN;     // wave-uniform
#pragma unroll
    for (int fa = 0; fa < FM; ++fa) {
      const int64_t ib = i0 + swm * WM + fa * MF;
#pragma unroll
      for (int fb = 0; fb < FN; ++fb) {
        const int64_t jb = j0 + swn * WN + fb * MF;   // MF columns of one 32-column block
        const int soff = int(((jb >> 5) * d.rp + ib) * 64 + (jb & 31) * 2);
        // Keeps this block's accumulators in AGPRs up to here: otherwise the
        // compiler copies every accumulator to VGPRs at the loop exit, and a
        // 128 x 256 tile no longer fits two workgroups per CU.
        asm volatile("" : "+a"(acc[fa][fb]));
        if constexpr (MF == 16 && !XLO) {
          // Lanes 2k and 2k + 1 hold columns c and c + 1 of the same four rows:
          // a swap of two values each (DPP within groups of four lanes) gives
          // the even lane rows 0 and 2, the odd lane rows 1 and 3, of both
          // columns: two 4-byte stores per lane instead of four 2-byte ones.
          const bool odd = lane & 1;
          const float x0 = s0 * acc[fa][fb][0], x1 = s0 * acc[fa][fb][1];
          const float x2 = s0 * acc[fa][fb][2], x3 = s0 * acc[fa][fb][3];
          auto swap = [](float v) {
            return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
          };
          const float r1 = swap(odd ? x0 : x1), r2 = swap(odd ? x2 : x3);
          const uint32_t p1 = odd ? pack_bf16x2(r1, x1) : pack_bf16x2(x0, r1);
          const uint32_t p2 = odd ? pack_bf16x2(r2, x3) : pack_bf16x2(x2, r2);
          const int vo = voff - (odd ? 2 : 0) + (odd ? 64 : 0);   // column c & ~1, row 0 or 1
          __builtin_amdgcn_raw_buffer_store_b32(p1, rx, vo, soff, 0);
          __builtin_amdgcn_raw_buffer_store_b32(p2, rx, vo + 128, soff, 0);   // row 2 or 3
          __builtin_amdgcn_sched_barrier(0);
          continue;
        }
        float lo[NV];
        // bytes from the lane's first row to that of accumulator v
        auto vrow = [&](int v) { return (acc_row(v) - acc_row(0)) * 64; };
        if constexpr (XLO) {
#pragma unroll
          for (int v = 0; v < NV; ++v)
            lo[v] = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rl, voff + vrow(v), soff, 0));
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int row = vrow(v);
          const float x = XLO ? s0 * fmaf(ca, lo[v], acc[fa][fb][v]) : s0 * acc[fa][fb][v];
          const uint32_t hi = f32_to_bf16(x);
          __builtin_amdgcn_raw_buffer_store_b16(uint16_t(hi), rx, voff + row, soff, 0);
          if constexpr (XLO)
            __builtin_amdgcn_raw_buffer_store_b16(uint16_t(f32_to_bf16(x - bf16_to_f32(hi))), rl,
                                                  voff + row, soff, 0);
        }
        // one block at a time: the compiler would otherwise copy every
        // accumulator out of the AGPRs at once and run out of VGPRs
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    return;
  }
  __syncthreads();

  // Stage layout: value (r, c) of a half tile sits at r * SLD + (c ^ sw(r)),
  // sw(r) = ((r >> 4) & 7) << 2.  The transposed pass reads a column run
  // r = 8 ch + u (ch = 0..15) at fixed c; with the swizzle those 16 reads hit
  // 16 distinct banks.  A row run of 8 values starting at a multiple of 8
  // stays inside one aligned group of 8, with its two 4-value halves swapped
  // when bit 2 of sw(r) is set.
  float* stage = reinterpret_cast<float*>(smem);
  const bool diag_tile = it.ti == it.tj;
  const T* xin = xcur;                                              // X of this round
  T* xout = static_cast<T*>(QT ? (cur ? d.x[0] : d.x[1]) : d.x[0]);  // next X (fp32: in place)
  T* xtn = static_cast<T*>(cur ? d.xt[0] : d.xt[1]);                // fp32: next X^T
  float* w = mats[d.mat].w;
  const float wkeep = 1.0f - d.lr * wd;
  bool mirror;
  if constexpr (PROD) mirror = QT ? (last && d.tall) : (!last || d.tall);
  else mirror = !diag_tile;
  auto sw = [](int r) { return ((r >> 4) & 7) << 2; };
  // Round 0 works on the unscaled M: A = s^2 (M M^T), X_1 = s (a M + B M).
  const float s0 = iter == 0 ? d.scale[0] : 1.0f;
  const float gscale = s0 * s0, pscale = s0;
  constexpr int CPR = BN / 8;                  // 8-value chunks per tile row
  constexpr int DIT = HALF * CPR / NT;         // direct-pass chunks per thread
  constexpr int CPC = HALF / 8;                // 8-value chunks per mirrored row
  constexpr int MIT = BN * CPC / NT;           // mirror-pass chunks per thread
  static_assert(DIT * NT == HALF * CPR && MIT * NT == BN * CPC, "whole passes");
  // The direct pass needs operand reads per chunk (A for B; X for the
  // product, plus W for the last product of a wide matrix).  They are issued in
  // batches of PB chunks, double-buffered: batch bt + 1 is in flight while
  // batch bt is computed and stored, and the first batch is issued before the
  // accumulators are parked, so its latency overlaps the staging and its
  // barrier.  The last product of a tall matrix updates W in the mirror pass,
  // in batches of MB chunks, double-buffered the same way, its first batch
  // issued before the direct pass.
  const bool aux_is_w = last && !d.tall;     // also the W values to update
  const bool need_aux = OP == kGemmPoly || (PROD && (!QT || XLO || aux_is_w));
  const bool mirror_w = last && d.tall;
  // Batch sizes: as many chunks in flight as registers allow without spills
  // (the two W paths share one double buffer of 4-chunk batches).
  constexpr int PBMAX = sizeof(T) == 4 ? (last ? 1 : 2) : (XLO && last ? 1 : last && MF == 16 ? 2 : 4);
  constexpr int PB = DIT < PBMAX ? DIT : PBMAX;
  constexpr int NB = DIT / PB;
  static_assert(NB * PB == DIT, "whole batches");
  constexpr int MBMAX = sizeof(T) == 4 || (XLO && last && MF == 16) ? 2 : 4;
  constexpr int MB = MIT < MBMAX ? MIT : MBMAX;
  constexpr int MNB = MIT / MB;
  static_assert(MNB * MB == MIT, "whole mirror batches");

#pragma unroll 1
  for (int half = 0; half < NPASS; ++half) {
    const int64_t ib0 = i0 + int64_t(half) * HALF;
    Raw8<T> ra[2][PB];
    W8 wb[2][4];
    static_assert(PB <= 4 && MB <= 4, "W batches fit the shared buffer");
    // values of a W row run that exist (wide: row i of X is row i of W)
    auto wide_nv = [&](int64_t i, int64_t j) {
      return (i < d.r) ? int(max<int64_t>(0, min<int64_t>(8, d.c - j))) : 0;
    };
    auto prefetch = [&](int bt) {
#pragma unroll
      for (int q = 0; q < PB; ++q) {
        const int idx = tid + (bt * PB + q) * NT;
        const int r = idx / CPR, ch = idx % CPR;
        const int64_t i = ib0 + r, j = j0 + ch * 8;
        if constexpr (OP == kGemmPoly) ra[bt & 1][q].load(static_cast<const T*>(d.a) + ws_at<T>(i, j, d.rp, d.rp));
        else if constexpr (!QT) ra[bt & 1][q].load(xin + ws_at<T>(i, j, d.rp, d.cp));
        else if constexpr (XLO) ra[bt & 1][q].load(static_cast<const T*>(d.xlo) + ws_at<T>(i, j, d.rp, d.cp));
        if (aux_is_w) wb[bt & 1][q].load(w, i * d.ld + d.col0 + j, wide_nv(i, j));
      }
    };
    // Mirror chunk: column jj of the tile, rows 8 ch .. 8 ch + 7 of this pass,
    // i.e. a run of row j of X^T (tall: of W).
    auto mirror_nv = [&](int64_t i, int64_t j) {
      return (j < d.c) ? int(max<int64_t>(0, min<int64_t>(8, d.r - i))) : 0;
    };
    auto mprefetch = [&](int mb) {
#pragma unroll
      for (int q = 0; q < MB; ++q) {
        const int idx = tid + (mb * MB + q) * NT;
        const int jj = idx / CPC, ch = idx % CPC;
        const int64_t j = j0 + jj, i = ib0 + ch * 8;
        wb[mb & 1][q].load(w, j * d.ld + d.col0 + i, mirror_nv(i, j));
      }
    };
    if (need_aux) prefetch(0);
    if (mirror_w) mprefetch(0);
    if constexpr (WM <= HALF) {
      // a wave's rows sit in one pass: one test per wave
      if (wm * WM >= half * HALF && wm * WM < (half + 1) * HALF) {
        const int rbase = wm * WM - half * HALF;
#pragma unroll
        for (int fa = 0; fa < FM; ++fa)
#pragma unroll
          for (int fb = 0; fb < FN; ++fb)
#pragma unroll
            for (int v = 0; v < NV; ++v) {
              const int r = rbase + fa * MF + acc_row(v);
              const int c = wn * WN + fb * MF + acc_col;
              stage[r * SLD + (c ^ sw(r))] = acc[fa][fb][v];
            }
      }
    } else {
#pragma unroll
      for (int fa = 0; fa < FM; ++fa) {
        const int rb = wm * WM + fa * MF - half * HALF;   // block row fa, first row in this pass
        if (rb >= 0 && rb < HALF) {
#pragma unroll
          for (int fb = 0; fb < FN; ++fb)
#pragma unroll
            for (int v = 0; v < NV; ++v) {
              const int r = rb + acc_row(v);
              const int c = wn * WN + fb * MF + acc_col;
              stage[r * SLD + (c ^ sw(r))] = acc[fa][fb][v];
            }
        }
      }
    }
    __syncthreads();
    // rows of the tile: C[i][j .. j+7].  The bf16 last product of a tall
    // matrix has nothing to do here (its W update reads the stage in the
    // mirror pass, which applies the round's scale itself).
    const bool skip_direct = QT && last && !XLO && d.tall;
#pragma unroll
    for (int bt = 0; bt < (skip_direct ? 0 : NB); ++bt) {
      if (bt + 1 < NB && need_aux) prefetch(bt + 1);
#pragma unroll
      for (int q = 0; q < PB; ++q) {
        const int idx = tid + (bt * PB + q) * NT;
        const int r = idx / CPR, ch = idx % CPR;
        const int64_t i = ib0 + r, j = j0 + ch * 8;
        const int swz = sw(r);
        f32x4_t* sv = reinterpret_cast<f32x4_t*>(stage + r * SLD + ((ch * 8) ^ (swz & ~7)));
        const bool flip = (swz & 4) != 0;
        const f32x4_t lo = flip ? sv[1] : sv[0], hi = flip ? sv[0] : sv[1];
        float v[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) { v[u] = lo[u]; v[4 + u] = hi[u]; }
        const bool has_diag = diag_tile && i >= j && i < j + 8;
        const int du = int(i - j);
        bool writeback = false;
        if constexpr (OP == kGemmGram) {
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] *= gscale;
          if (has_diag) {
            float dv = 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) dv = (u == du) ? v[u] : dv;
            d.adiag[i] = dv;
          }
          store8(static_cast<T*>(d.a) + ws_at<T>(i, j, d.rp, d.rp), v);
        } else if constexpr (OP == kGemmPoly) {
          float av[8];
          ra[bt & 1][q].unpack(av);
          float dval = 0.f;          // stored diagonal (bf16: a + B_ii; fp32: 0)
          if (has_diag) {
            float acc_ii = 0.f, a_ii = 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              acc_ii = (u == du) ? v[u] : acc_ii;
              a_ii = (u == du) ? av[u] : a_ii;
            }
            const float ad = d.adiag[i];
            const float aa = acc_ii + ad * ad - a_ii * a_ii;
            const float bii = fmaf(cb, ad, cc * aa);
            if constexpr (sizeof(T) == 2) {
              // stored B_ii = bf16(a + B_ii); the remainder goes to the product
              // as an extra diagonal MFMA operand
              const float dsum = ca + bii;
              dval = dsum;
              d.bdiag[i] = dsum - bf16_to_f32(f32_to_bf16(dsum));
            } else {
              d.bdiag[i] = bii;
            }
          }
#pragma unroll
          for (int u = 0; u < 8; ++u)
            v[u] = (has_diag && u == du) ? dval : fmaf(cc, v[u], cb * av[u]);
          store8(static_cast<T*>(d.b) + ws_at<T>(i, j, d.rp, d.rp), v);
          writeback = true;
        } else {
          // fp32: add (a + B_ii) X_i here; bf16: the MFMAs already did, on
          // bf16(X), and XLO adds a times X's remainder
          float mlt = 0.f, xv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          if constexpr (!QT) {
            mlt = ca + d.bdiag[i];
            ra[bt & 1][q].unpack(xv);
          } else if constexpr (XLO) {
            mlt = ca;
            ra[bt & 1][q].unpack(xv);
          }
          if constexpr (!last) {
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = pscale * fmaf(mlt, xv[u], v[u]);
            store8(xout + ws_at<T>(i, j, d.rp, d.cp), v);
            if constexpr (XLO) {
              float rem[8];
#pragma unroll
              for (int u = 0; u < 8; ++u) rem[u] = v[u] - bf16_to_f32(f32_to_bf16(v[u]));
              store8(static_cast<T*>(d.xlo) + ws_at<T>(i, j, d.rp, d.cp), rem);
            }
            writeback = !QT;                // fp32 also writes X^T from the stage
          } else if (!d.tall) {
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = pscale * fmaf(mlt, xv[u], v[u]);
            wb[bt & 1][q].update_store(w, i * d.ld + d.col0 + j, wide_nv(i, j), v, d.lr, wkeep);
          } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = pscale * fmaf(mlt, xv[u], v[u]);
            writeback = true;
          }
        }
        if (writeback) {
          const f32x4_t a4 = {v[0], v[1], v[2], v[3]}, b4 = {v[4], v[5], v[6], v[7]};
          sv[flip ? 1 : 0] = a4;
          sv[flip ? 0 : 1] = b4;
        }
      }
    }
    __syncthreads();
    // columns of the tile: C[i .. i+7][j] written as row j of the transpose
    auto mirror_vals = [&](int idx, float v[8]) {
      const int jj = idx / CPC, ch = idx % CPC;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = ch * 8 + u;
        v[u] = stage[r * SLD + (jj ^ sw(r))];
      }
    };
    if (mirror_w) {
#pragma unroll
      for (int mb = 0; mb < MNB; ++mb) {
        if (mb + 1 < MNB) mprefetch(mb + 1);
#pragma unroll
        for (int q = 0; q < MB; ++q) {
          const int idx = tid + (mb * MB + q) * NT;
          const int64_t j = j0 + idx / CPC, i = ib0 + (idx % CPC) * 8;
          float v[8];
          mirror_vals(idx, v);
          if (skip_direct) {
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] *= pscale;
          }
          wb[mb & 1][q].update_store(w, j * d.ld + d.col0 + i, mirror_nv(i, j), v, d.lr, wkeep);
        }
      }
    } else if (mirror) {
#pragma unroll
      for (int q = 0; q < MIT; ++q) {
        const int idx = tid + q * NT;
        const int64_t j = j0 + idx / CPC, i = ib0 + (idx % CPC) * 8;
        float v[8];
        mirror_vals(idx, v);
        if constexpr (OP == kGemmGram) {
          // the direct pass does not write its scaled values back to the stage
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] *= gscale;
          store8(static_cast<T*>(d.a) + ws_at<T>(j, i, d.rp, d.rp), v);
        } else if constexpr (OP == kGemmPoly) {
          store8(static_cast<T*>(d.b) + ws_at<T>(j, i, d.rp, d.rp), v);
        } else if constexpr (!last) {
          store8(xtn + j * d.rp + i, v);
        }
      }
    }
    __syncthreads();
  }
}

// Wave grids, chosen by timing on gfx950 (18 problems of 2048 x 8192): all
// tiles run 4 waves in a 2 x 2 grid, one wave per SIMD; a 256-tile wave
// holds its 128 x 128 accumulators in the 256 AGPRs.
template <int BM, int OP> struct WaveGrid { static constexpr int M = 2, N = 2; };

template <typename T, int BM, int OP, int BN = BM, bool XLO = false>
void launch_gemm_op(hipStream_t s, const MatDev* mats, const NsDev* ns, const GemmItem* items,
                    int64_t nitems, int iter, float a, float b, float c, float wd) {
  constexpr int GM = WaveGrid<BM, OP>::M, GN = WaveGrid<BM, OP>::N;
  ns_gemm_kernel<T, BM, GM, GN, OP, BN, XLO>
      <<<dim3(static_cast<unsigned>(nitems)), dim3(64 * GM * GN), 0, s>>>(mats, ns, items, iter, a,
                                                                          b, c, wd);
}

template <typename T, int BM, bool XLO = false>
hipError_t launch_gemm_t(hipStream_t s, const MatDev* mats, const NsDev* ns,
                         const GemmItem* items, int64_t nitems, int op, int iter, int last,
                         float a, float b, float c, float wd) {
  switch (op) {
    case kGemmGram:
      launch_gemm_op<T, BM, kGemmGram>(s, mats, ns, items, nitems, iter, a, b, c, wd);
      break;
    case kGemmPoly:
      launch_gemm_op<T, BM, kGemmPoly>(s, mats, ns, items, nitems, iter, a, b, c, wd);
      break;
    default:
      if (last)
        launch_gemm_op<T, BM, kGemmProductLast, BM, XLO>(s, mats, ns, items, nitems, iter, a, b, c, wd);
      else
        launch_gemm_op<T, BM, kGemmProduct, BM, XLO>(s, mats, ns, items, nitems, iter, a, b, c, wd);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ns_prep(hipStream_t s, const MatDev* mats, const NsDev* ns,
                          const TileItem* items, int64_t nitems, int prec, float beta) {
  if (nitems <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(nitems)), block(kThreads);
  if (prec != 1)   // bf16, with or without the remainder (its pointer tells)
    ns_prep_kernel<uint16_t><<<grid, block, 0, s>>>(mats, ns, items, beta);
  else
    ns_prep_kernel<float><<<grid, block, 0, s>>>(mats, ns, items, beta);
  return hipGetLastError();
}

hipError_t launch_ns_scale(hipStream_t s, NsDev* ns_dev, int32_t count, float eps) {
  if (count <= 0) return hipSuccess;
  ns_scale_kernel<<<dim3(count), dim3(kThreads), 0, s>>>(ns_dev, eps);
  return hipGetLastError();
}

hipError_t launch_ns_gemm(hipStream_t s, const MatDev* mats, const NsDev* ns,
                          const GemmItem* items, int64_t nitems, int op, int tile, int tile_n,
                          int prec, int iter, int last, float a, float b, float c, float wd) {
  if (nitems <= 0) return hipSuccess;
  if (tile_n != tile) {
    // the one wide tile: 128 x 256 for the bf16 product of the rounds
    // before the last (short K: twice the work per tile prologue/epilogue
    // and a third fewer staged bytes per flop than 128 x 128)
    if (prec == 1 || tile != 128 || tile_n != 256 || op != kGemmProduct || last)
      return hipErrorInvalidValue;
    if (prec == 2)
      launch_gemm_op<uint16_t, 128, kGemmProduct, 256, true>(s, mats, ns, items, nitems, iter, a, b, c, wd);
    else
      launch_gemm_op<uint16_t, 128, kGemmProduct, 256>(s, mats, ns, items, nitems, iter, a, b, c, wd);
    return hipGetLastError();
  }
  if (prec == 2 && op == kGemmProduct) {   // the Gram and polynomial do not read X's remainder
    if (tile == 256) return launch_gemm_t<uint16_t, 256, true>(s, mats, ns, items, nitems, op, iter, last, a, b, c, wd);
    return launch_gemm_t<uint16_t, 128, true>(s, mats, ns, items, nitems, op, iter, last, a, b, c, wd);
  }
  if (prec != 1) {
    if (tile == 256) return launch_gemm_t<uint16_t, 256>(s, mats, ns, items, nitems, op, iter, last, a, b, c, wd);
    return launch_gemm_t<uint16_t, 128>(s, mats, ns, items, nitems, op, iter, last, a, b, c, wd);
  }
  if (tile == 256) return launch_gemm_t<float, 256>(s, mats, ns, items, nitems, op, iter, last, a, b, c, wd);
  return launch_gemm_t<float, 128>(s, mats, ns, items, nitems, op, iter, last, a, b, c, wd);
}

}  // namespace muon
