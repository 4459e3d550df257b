// Gram A = X X^T of a Newton-Schulz round (the first of the three products
// per round; "Scaling Muon for Diffusion Transformers", PaperDaily post,
// section "Periodic Row-wise Muon", blog fig. 3) for problems whose padded
// short side is 384, in one workgroup per problem.
//
// Such problems are the column blocks of MuonBP ("MuonBP: Faster Muon via
// Block-Periodic Orthogonalization", abstract) on DiT widths of 3072: X is
// 384 x c with c from 3072 to 18432.  Tiled, the upper triangle of A is six
// 128-tiles, and each stages 2 x 128 rows of X per k-step for 128 x 128
// outputs: 64 flops per staged byte, where under full load the global->LDS
// path delivers 20 to 29 bytes per clock per CU for such rows (64 bytes of
// each, half a cache line), a third of what the matrix cores consume.  Here
// the workgroup stages the 384 rows of X once per k-step and computes all 78
// blocks (32 x 32) of the upper triangle from them: 213 flops per staged
// byte.
//
// Work split.  Eight waves, two per SIMD (a wave's accumulators must fit
// the 256 AGPRs; at 320 the compiler spills inside the loop).  Fragment f is
// rows 32 f .. 32 f + 31 of X, and G_k the fragments 3 k .. 3 k + 2.  The
// upper triangle is 4 diagonal super-blocks G_k x G_k (6 blocks each) and 6
// off-diagonal ones G_k x G_l (9 blocks).  Wave 0 takes the diagonal ones of
// G_0 and G_1, wave 1 G_0 x G_1, wave 2 the diagonal ones of G_2 and G_3,
// wave 3 G_2 x G_3, waves 4 .. 7 the other four; blocks (5, 5) and (11, 11)
// move from waves 0 and 2 to waves 1 and 3, which hold those fragments.
// Every wave reads 6 fragments per k-group and holds 9 to 11 blocks; waves
// w and w + 4 hold 19 or 20 together.
//
// Staging is the tiled kernel's: a ring of k-steps of 64 bytes per row
// (32 bf16 values; X and A are k-block-major, so a k-step of all 384 rows is
// one contiguous 24 KB run), filled by buffer_load ... lds issued ring - 1 steps ahead,
// 16-byte chunk c of row r at position c ^ ((r >> 2) & 3), MFMA
// v_mfma_f32_32x32x16_bf16 with the same operand layout.  Each wave
// interleaves its MFMAs with its fragment reads and DMAs in fixed slots.
// Fragments are not double buffered (a wave has 256 registers): each one is
// re-read for the next k-group (16 values of k) as soon as the current
// k-group's last MFMA that reads it has issued.
//
// Epilogue: each wave writes its blocks through a 32 x 32 fp32 stage in its
// own part of LDS: rows of block (i, j) as rows of A, its columns as rows of
// the mirrored block (j, i), and the fp32 diagonal of the diagonal blocks.
#include <hip/hip_runtime.h>

#include "gram_tri.h"
#include "muon_internal.h"

namespace muon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

#define LOCAL __attribute__((address_space(3)))
#define GLOBAL __attribute__((address_space(1)))

constexpr int kNF = kTriRows / 32;      // fragments (12)
constexpr int kWaves = 8;
constexpr int kThreadsTri = 64 * kWaves;
constexpr int kStageBytes = kTriRows * 64;   // one k-step of all rows
constexpr int kRing = 5;                      // k-steps in the LDS ring (120 KB)
constexpr int kDma = kTriRows / 16 / kWaves;  // 1 KB DMA blocks per wave per k-step
constexpr int kPre = 2;                       // g1 MFMAs issued before the barrier
constexpr int kMaxBlocks = 12;
constexpr int kEpiPitch = 36;                 // epilogue stage row pitch (floats)
static_assert(kNF == 12, "the work split below is written for 12 fragments");
static_assert(kRing * kStageBytes <= 160 * 1024, "ring fits the LDS");
static_assert(kWaves * 32 * kEpiPitch * 4 <= kRing * kStageBytes, "epilogue stages fit the ring");

// Which wave computes block (i, j), i <= j.
constexpr int tri_owner(int i, int j) {
  if (i == 5 && j == 5) return 1;
  if (i == 11 && j == 11) return 3;
  const int gi = i / 3, gj = j / 3;
  if (gi == gj) return gi < 2 ? 0 : 2;
  if (gi == 0 && gj == 1) return 1;
  if (gi == 2 && gj == 3) return 3;
  if (gi == 0) return gj == 2 ? 4 : 5;
  return gj == 2 ? 6 : 7;
}

// A wave's share: its fragments (frag[0 .. nf)) and blocks, block n being
// (frag[a[n]], frag[b[n]]); last[p] is the last block that reads fragment p.
struct TriPlan {
  int nf = 0, nb = 0;
  int frag[kNF] = {};
  int a[kMaxBlocks] = {}, b[kMaxBlocks] = {};
  int last[kNF] = {};
};

constexpr TriPlan tri_plan(int w) {
  TriPlan p;
  int pos[kNF] = {};
  for (int f = 0; f < kNF; ++f) pos[f] = -1;
  for (int i = 0; i < kNF; ++i)
    for (int j = i; j < kNF; ++j) {
      if (tri_owner(i, j) != w) continue;
      if (pos[i] < 0) { pos[i] = p.nf; p.frag[p.nf++] = i; }
      if (pos[j] < 0) { pos[j] = p.nf; p.frag[p.nf++] = j; }
      p.a[p.nb] = pos[i];
      p.b[p.nb] = pos[j];
      p.last[pos[i]] = p.last[pos[j]] = p.nb;
      ++p.nb;
    }
  return p;
}

constexpr bool tri_plans_cover() {
  int blocks = 0;
  for (int w = 0; w < kWaves; ++w) {
    const TriPlan p = tri_plan(w);
    if (p.nb > 11 || p.nf != 6) return false;   // 176 accumulator registers
    blocks += p.nb;
  }
  return blocks == kNF * (kNF + 1) / 2;
}
static_assert(tri_plans_cover(), "every upper block belongs to exactly one wave");

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16 bytes per lane from a raw buffer into LDS (lane l lands at lds_addr +
// 16 l).  Inline asm, so that the compiler does not model the LDS writes
// (it would otherwise drain every DMA in flight before each fragment read);
// the pipeline orders them with explicit vmcnt waits and barriers.
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

// Raw buffer resource: base, stride 0, byte size (reads past it return 0).
__device__ __forceinline__ u32x4_t buffer_rsrc(const void* p, int64_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return u32x4_t{unsigned(a), unsigned(a >> 32) & 0xffffu, unsigned(nbytes), 0x00020000u};
}

// Round to nearest even with the hardware packed conversion.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ void store8_bf16(uint16_t* p, const float v[8]) {
  u32x4_t u;
#pragma unroll
  for (int k = 0; k < 4; ++k) u[k] = pack_bf16x2(v[2 * k], v[2 * k + 1]);
  *(GLOBAL u32x4_t*)(p) = u;
}

template <int W>
__device__ __forceinline__ void tri_wave(const NsDev& d, unsigned char* smem, int lane, int iter) {
  constexpr TriPlan P = tri_plan(W);
  constexpr int NF = P.nf, NB = P.nb;
  static_assert(NB - kPre >= kDma, "every DMA has an MFMA slot");

  const int cur = iter & 1;
  const uint16_t* x = static_cast<const uint16_t*>(cur ? d.x[1] : d.x[0]);
  const int nk = int(d.cp / 32);                // k-steps
  // X is k-block-major: k-step kc is rows 0 .. kTriRows - 1 of 64 bytes
  // each, one contiguous run at kc * kStageBytes.
  const u32x4_t rX = buffer_rsrc(x, int64_t(kTriRows) * d.cp * 2);
  // DMA block q of this wave: rows 16 (W + 8 q) .. + 15; lane l brings row
  // + (l >> 2), logical chunk (l & 3) ^ ((l >> 4) & 3), which lands at
  // physical chunk l & 3 (the row's swizzle).
  const unsigned offX =
      unsigned((16 * W + (lane >> 2)) * 64) + unsigned(((lane & 3) ^ ((lane >> 4) & 3)) * 16);
  constexpr unsigned rstride = 16 * kWaves * 64;
  auto issue_one = [&](int kt, int q) {
    const int kc = min(kt, nk - 1);   // past the end: reload the last step
    LOCAL unsigned char* base =
        (LOCAL unsigned char*)(smem + (kt % kRing) * kStageBytes + (W + kWaves * q) * 1024);
    dma16(rX, unsigned(uintptr_t(base)), offX + unsigned(q) * rstride, unsigned(kc * kStageBytes));
  };

  f32x16_t acc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) acc[n] = (f32x16_t)(0.0f);
  u32x4_t f[NF];
  const int frow = lane & 31, fsw = (lane >> 2) & 3, fhalf = lane >> 5;
  const u32x4_t* lds = reinterpret_cast<const u32x4_t*>(smem);
  auto step = [&](int kt) { return lds + (kt % kRing) * (kStageBytes / 16); };
  // fragment p of k-group g: row frag*32 + (l & 31), chunk 2 g + (l >> 5)
  auto rd = [&](const u32x4_t* s, int g, int p) {
    f[p] = s[(P.frag[p] * 32 + frow) * 4 + ((2 * g + fhalf) ^ fsw)];
  };
  auto mm = [&](int n) {
    acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, f[P.a[n]]),
                                                     __builtin_bit_cast(bf16x8_t, f[P.b[n]]),
                                                     acc[n], 0, 0, 0);
  };
  auto bar = [&]() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

#pragma unroll
  for (int s0 = 0; s0 < kRing - 1; ++s0)
#pragma unroll
    for (int q = 0; q < kDma; ++q) issue_one(s0, q);
  wait_vmcnt<(kRing - 2) * kDma>();   // step 0 is in
  bar();
#pragma unroll
  for (int p = 0; p < NF; ++p) rd(step(0), 0, p);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

  // Iteration kt starts with the k-group 0 fragments of step kt in f.
  //   k-group 0: MFMA n, then the k-group 1 reads of the fragments whose
  //              last reader n is;
  //   k-group 1: the first kPre MFMAs; wait for this wave's DMA of step
  //              kt + 1 and the barrier: step kt + 1 is in, and every wave is
  //              done with step kt - 1, whose buffer the DMA of step
  //              kt + kRing - 1 refills; then the other MFMAs, each followed
  //              by the step kt + 1, k-group 0 reads of the fragments it was
  //              the last reader of, and by one DMA.
  // (cp >= 256, so nk >= 8: a loop without a zero-trip path.)
  int kt = 0;
  do {
    __builtin_amdgcn_sched_barrier(0);
    {
      const u32x4_t* s = step(kt);
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        mm(n);
#pragma unroll
        for (int p = 0; p < NF; ++p)
          if (P.last[p] == n) rd(s, 1, p);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int n = 0; n < kPre; ++n) {
        mm(n);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_vmcnt<(kRing - 3) * kDma>();
    bar();
    __builtin_amdgcn_sched_barrier(0);
    {
      const u32x4_t* s = step(kt + 1);
#pragma unroll
      for (int p = 0; p < NF; ++p)
        if (P.last[p] < kPre) rd(s, 0, p);
      int nd = 0;
#pragma unroll
      for (int n = kPre; n < NB; ++n) {
        mm(n);
#pragma unroll
        for (int p = 0; p < NF; ++p)
          if (P.last[p] == n) rd(s, 0, p);
        if (nd < kDma) { issue_one(kt + kRing - 1, nd); ++nd; }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (; nd < kDma; ++nd) issue_one(kt + kRing - 1, nd);
    }
    __builtin_amdgcn_sched_barrier(0);
  } while (++kt < nk);
  wait_vmcnt<0>();
  __syncthreads();

  // ---- epilogue: blocks through this wave's 32 x 32 stage ------------------
  // Accumulator element v of lane l is C[8 (v / 4) + 4 (l / 32) + v % 4][l % 32];
  // the stage holds the transpose, S[col][row] at col * kEpiPitch + row.
  const float s0 = iter == 0 ? d.scale[0] : 1.0f;
  const float gscale = s0 * s0;
  float* S = reinterpret_cast<float*>(smem) + W * 32 * kEpiPitch;
  // rp is kTriRows: every block's offset from a lane's two row bases is a
  // constant.
  constexpr int rp = kTriRows;
  uint16_t* A = static_cast<uint16_t*>(d.a);
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    __builtin_amdgcn_sched_barrier(0);
    const int bi = P.frag[P.a[n]], bj = P.frag[P.b[n]];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const f32x4_t v4 = {acc[n][4 * a] * gscale, acc[n][4 * a + 1] * gscale,
                          acc[n][4 * a + 2] * gscale, acc[n][4 * a + 3] * gscale};
      *reinterpret_cast<f32x4_t*>(S + frow * kEpiPitch + 8 * a + 4 * fhalf) = v4;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // 128 runs of 8 values per block, two per lane: run c is row c / 4 of
    // the block, values 8 (c % 4) .. + 7 along it.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = lane + 64 * h, row = c >> 2, q = c & 3;
      float v[8];
      // block (bi, bj), row `row`: C[row][8 q + u] = S[8 q + u][row]
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = S[(8 * q + u) * kEpiPitch + row];
      // A is k-block-major too: (i, j) at ((j / 32) rp + i) 32 + j % 32
      store8_bf16(A + (int64_t(bj) * rp + bi * 32 + row) * 32 + 8 * q, v);
      if (bi != bj) {
        // mirrored block (bj, bi), row `row`: C[8 q + u][row] = S[row][8 q + u]
        const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(S + row * kEpiPitch + 8 * q);
        const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(S + row * kEpiPitch + 8 * q + 4);
        const float m[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        store8_bf16(A + (int64_t(bi) * rp + bj * 32 + row) * 32 + 8 * q, m);
      }
    }
    if (bi == bj && lane < 32) d.adiag[bi * 32 + lane] = S[lane * kEpiPitch + lane];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

__global__ __launch_bounds__(kThreadsTri, 1) void ns_gram_tri_kernel(
    const NsDev* __restrict__ ns, const GemmItem* __restrict__ items, int iter) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kRing * kStageBytes];
  const NsDev d = ns[items[blockIdx.x].ns];
  const int lane = threadIdx.x & 63;
  switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
    case 0: tri_wave<0>(d, smem, lane, iter); break;
    case 1: tri_wave<1>(d, smem, lane, iter); break;
    case 2: tri_wave<2>(d, smem, lane, iter); break;
    case 3: tri_wave<3>(d, smem, lane, iter); break;
    case 4: tri_wave<4>(d, smem, lane, iter); break;
    case 5: tri_wave<5>(d, smem, lane, iter); break;
    case 6: tri_wave<6>(d, smem, lane, iter); break;
    default: tri_wave<7>(d, smem, lane, iter); break;
  }
}

}  // namespace

hipError_t launch_ns_gram_tri(hipStream_t s, const NsDev* ns, const GemmItem* items,
                              int64_t nitems, int iter) {
  if (nitems <= 0) return hipSuccess;
  ns_gram_tri_kernel<<<dim3(static_cast<unsigned>(nitems)), dim3(kThreadsTri), 0, s>>>(ns, items,
                                                                                      iter);
  return hipGetLastError();
}

}  // namespace muon
