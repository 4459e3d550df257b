// Internal structures shared by the host planner and the gfx950 kernels.
//
// Every table here lives in the caller's state buffer; the planner fills
// host copies and uploads them once in muon_init.  Pointers to the caller's
// W / G tensors are patched by a small kernel when a step passes new ones.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace muon {

// One Muon weight.
struct MatDev {
  float* w;          // stored W, rows x cols, row-major (caller-owned)
  const void* g;     // gradient, same shape (caller-owned), dtype = gdt
  float* mom;        // momentum, rows x cols fp32 (state buffer)
  int64_t rows, cols;
  float* part;       // RowNorm column partial sums (tall kernels).  Two-pass:
                     // one row of cols per row chunk.  Single pass: per
                     // column strip, one row of kTallCols per row chunk,
                     // then the strip's coefficient row.
  int32_t gdt;       // 0 = f32, 1 = bf16
  int32_t sync0;     // single-pass tall RowNorm: first TallSync of this matrix
};

// Cross-workgroup state of one column strip of the single-pass tall RowNorm
// kernel, one 128-byte cache line per strip (waiting workgroups poll it).
// All words are zero between launches.
struct TallSync {
  uint32_t arrive;   // workgroups that have published their partials
  uint32_t depart;   // workgroups done with the coefficients
  uint32_t ready;    // 1 once the coefficients are published
  uint32_t pad[29];
};

// Control line of the single-pass tall RowNorm, followed in the state
// buffer by its repair list (one uint32 per tile).  A workgroup whose wait
// for its strip gives up does not write W: it appends its tile index to the
// list, and the repair launch that follows on the same stream applies the
// W update of the listed tiles (the strip's coefficients are published by
// then).  repair_count and repair_done are zero between launch pairs.
struct TallCtl {
  uint32_t repair_count;   // tiles listed in this launch
  uint32_t giveups;        // waits that gave up since init (never reset)
  uint32_t repair_done;    // repair workgroups finished
  uint32_t pad[29];
};

// One AdamW tensor (flattened).
struct AdamDev {
  float* p;
  const void* g;
  float* m;
  float* v;
  int64_t numel;
  int32_t gdt;
  int32_t pad;
};

// A contiguous piece of one AdamW tensor handled by one workgroup.
struct AdamChunk {
  int32_t tensor;
  int32_t len;
  int64_t off;
};

// One Newton-Schulz problem: a whole matrix, or one MuonBP column block.
// X orientation is wide: r = min(rows, cols) rows, c = max columns.  The
// stored block (rows x cols at column col0 of a row-major matrix with row
// stride ld) equals X when wide and X^T when tall.
struct NsDev {
  int32_t mat;       // MatDev index
  int32_t tall;      // stored block is c x r
  int64_t rows, cols, col0, ld;
  int64_t r, c, rp, cp;   // logical and padded X dims
  // X (rp x cp).  bf16: x[0], x[1] ping-pong between rounds, and the
  // product reads its X operand from x through transposed LDS reads; bf16
  // X, xlo, A and B are k-block-major (element (i, j) at
  // ((j / 32) * rp + i) * 32 + j % 32).  fp32: row-major, x[0] only, updated
  // in place, plus X^T (cp x rp) in xt[0], xt[1] ping-pong as the product's
  // operand.
  void* x[2];
  void* xt[2];       // null in bf16
  void* a;           // rp x rp, X X^T
  void* b;           // rp x rp, b A + c A A
  float* part;       // Frobenius partial sums, one per prep tile (nparts)
  float* scale;      // s = 1 / (||M||_F + eps), one float
  float* adiag;      // rp: diagonal of A kept in fp32
  float* bdiag;      // rp, fp32: B_ii (stored B has 0 there); bf16: stored B
                     // holds bf16(a + B_ii) and this the rounding remainder
  void* xlo;         // MUON_NS_BF16_COMP: bf16(X - bf16(X)), rp x cp like
                     // x[0], updated in place by each round's product; else null
  int32_t nparts;
  float lr;          // learning rate applied by the final product
};

// A GEMM output tile of one NsDev.
struct GemmItem {
  int32_t ns;
  int16_t ti, tj;
};

// A prep tile of one NsDev (64 x 64 in stored coordinates of the padded
// block) or a RowNorm tile of one matrix.
struct TileItem {
  int32_t id;
  int16_t ti, tj;
};

// Pointer patch applied when a step passes new W / G pointers.
constexpr int kPatchMax = 24;
struct PatchArgs {
  int32_t count;
  int32_t adam;           // 0: MatDev table, 1: AdamDev table
  int32_t idx[kPatchMax];
  void* w[kPatchMax];
  const void* g[kPatchMax];
};

struct StepScalars {
  float lr, beta, gamma, eps_row, wd;
};

// ---- launchers (kernels_*.hip); all return hipGetLastError() -------------
// Rows of the matrices mat_ids[0..nmat) (one workgroup per row); row_prefix
// has nmat + 1 entries.  Every row must have <= max_chunks * kRowChunkElems
// elements, or max_chunks == 0 selects the streaming two-pass variant.
hipError_t launch_rownorm_rows(hipStream_t s, const MatDev* mats, const int32_t* mat_ids,
                               const int64_t* row_prefix, int32_t nmat, int64_t total_rows,
                               int max_chunks, StepScalars sc);
// Column-normalised (tall) matrices, phase 1 (momentum + column partials) or
// phase 2 (norms + weight update), one workgroup per tile.
hipError_t launch_rownorm_coef(hipStream_t s, const MatDev* mats, const TileItem* strips,
                               int64_t nstrips, StepScalars sc);
hipError_t launch_rownorm_cols(hipStream_t s, const MatDev* mats, const TileItem* tiles,
                               int64_t ntiles, int phase, StepScalars sc);
// Column-normalised (tall) matrices in one pass: tiles kTallRows x
// kTallCols listed strip by strip (row chunks of a strip consecutive),
// one workgroup per tile.  A wait gives up after poll_limit polls (that
// happens only when the residency bound is broken, or in tests that set a
// small limit) and lists its tile in `repair` instead of writing W;
// launch_rownorm_repair, enqueued right after, writes those tiles.
hipError_t launch_rownorm_tall(hipStream_t s, const MatDev* mats, const TileItem* tiles,
                               int64_t ntiles, TallSync* sync, TallCtl* ctl, uint32_t* repair,
                               uint32_t poll_limit, StepScalars sc);
hipError_t launch_rownorm_repair(hipStream_t s, const MatDev* mats, const TileItem* tiles,
                                 int64_t ntiles, TallCtl* ctl, const uint32_t* repair,
                                 StepScalars sc);
// Workgroups of the single-pass tall kernel that fit on one CU at once.
hipError_t rownorm_tall_resident(int* workgroups_per_cu);
// Refresh prep: momentum, Frobenius partials, unscaled X0 in both layouts
// (and its bf16 remainder where the problem has xlo).  prec: 0 bf16, 1 fp32,
// 2 bf16 with the remainder (muon_ns_precision).
hipError_t launch_ns_prep(hipStream_t s, const MatDev* mats, const NsDev* ns,
                          const TileItem* items, int64_t nitems, int prec, float beta);
hipError_t launch_ns_scale(hipStream_t s, NsDev* ns_dev, int32_t count, float eps);
// tile x tile_n output tiles (tile_n != tile only for 128 x 256 bf16
// products of the rounds before the last).
hipError_t launch_ns_gemm(hipStream_t s, const MatDev* mats, const NsDev* ns,
                          const GemmItem* items, int64_t nitems, int op, int tile, int tile_n,
                          int prec, int iter, int last, float a, float b, float c, float wd);
hipError_t launch_adamw(hipStream_t s, const AdamDev* t, const AdamChunk* chunks,
                        int64_t nchunks, float lr, float b1, float b2, float eps,
                        float wd, float bc1, float bc2);
hipError_t launch_patch(hipStream_t s, MatDev* mats, AdamDev* adams, const PatchArgs& args);
// Zero `bytes` (a multiple of 4) at the device address p with a kernel (no
// memset node, so a captured launch replays it unchanged).
hipError_t launch_fill_zero(hipStream_t s, void* p, size_t bytes);
// Device address of the no-alloc scratch array on the current device
// (kNoallocScratchBytes bytes), looked up once per device.
hipError_t noalloc_scratch(void** ptr);

constexpr int kGemmGram = 0, kGemmPoly = 1, kGemmProduct = 2;
constexpr int kGemmProductLast = 3;  // kernel variant only: product that updates W
constexpr int kRowChunkElems = 1024;   // elements per row-kernel chunk (256 thr x 4)
constexpr int kColTileRows = 512;      // tall RowNorm tile rows
constexpr int kColTileCols = 256;      // tall RowNorm tile columns
constexpr int kTallRows = 256;         // single-pass tall RowNorm tile rows
constexpr int kTallCols = 128;         // single-pass tall RowNorm strip width
constexpr int kTallMaxChunks = 128;    // single pass only for rows <= 128 * 256
constexpr uint32_t kTallPollLimit = 1u << 18;   // default polls before a wait gives up
constexpr int kPrepTile = 64;          // NS5 cast/transpose tile
constexpr int kAdamChunk = 4096;       // elements per AdamW workgroup
constexpr size_t kNoallocScratchBytes = size_t(128) << 20;   // muon_step_noalloc scratch

}  // namespace muon
