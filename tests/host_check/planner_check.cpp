// Host-only check of the launch planner and the per-step launch sequence.
//
// runtime.cpp is compiled for the CPU (under ASan/UBSan by
// tests/test_host_sanitized.py) with the HIP runtime calls and every kernel
// launcher replaced by stubs.  "Device" memory is host memory; each
// buffer the kernels may touch is registered, and every stubbed launch checks
// that each access its kernel would make - table entries, the rows and
// columns of W, G and M, partial sums, counters, Newton-Schulz workspaces and
// tiles - lies inside one registered buffer, and that tile indices fit the
// padded shapes.  Parameter lists too large to hold in host memory (DiT-15B)
// are checked on the host copies of the plan, at a fake base address.
#include "../../matrix_aware_optimizer_periodic_amd/csrc/runtime.cpp"

#include <cstdlib>
#include <map>

namespace chk {

struct Range {
  uintptr_t lo, hi;
  std::string what;
};
std::vector<Range> g_ranges;      // registered buffers
std::vector<Range> g_sorted;      // the same, sorted by start (rebuilt on demand)
bool g_dirty = true;
long g_fail = 0, g_checks = 0, g_launches = 0;
std::string g_scenario;

void reg(const void* p, size_t n, const std::string& what) {
  g_ranges.push_back({reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + n, what});
  g_dirty = true;
}
void unreg_all() { g_ranges.clear(); g_dirty = true; }

void fail(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::fprintf(stderr, "CHECK FAILED [%s]: ", g_scenario.c_str());
  std::vfprintf(stderr, fmt, ap);
  std::fprintf(stderr, "\n");
  va_end(ap);
  if (++g_fail > 20) std::abort();
}

// [p, p + n) lies inside one registered buffer.
// Zero bytes touch nothing and always pass.
void need(const void* p, double n, const char* what) {
  ++g_checks;
  if (n == 0) return;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if (!p || n < 0) { fail("%s: null pointer or negative size", what); return; }
  if (g_dirty) {
    g_sorted = g_ranges;
    std::sort(g_sorted.begin(), g_sorted.end(), [](const Range& x, const Range& y) { return x.lo < y.lo; });
    g_dirty = false;
  }
  // registered buffers do not overlap (a buffer registered twice aside), so
  // only the nearest ones starting at or below a can hold the access
  auto it = std::upper_bound(g_sorted.begin(), g_sorted.end(), a,
                             [](uintptr_t v, const Range& r) { return v < r.lo; });
  for (int k = 0; k < 4 && it != g_sorted.begin(); ++k) {
    --it;
    if (double(a) + n <= double(it->hi)) return;
  }
  fail("%s: [%#lx, +%.0f) is outside every registered buffer", what, (unsigned long)a, n);
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- footprints of each kernel, given its tables (host-readable) ----------
void mat_tensors(const muon::MatDev& d, const char* k) {
  const double e = double(d.rows) * double(d.cols);
  need(d.w, 4 * e, k);
  need(d.mom, 4 * e, k);
  need(d.g, (d.gdt == 1 ? 2 : 4) * e, k);
}

void check_rows(const muon::MatDev* mats, const int32_t* ids, const int64_t* prefix, int32_t nmat,
                int64_t total_rows, int max_chunks) {
  need(ids, 4.0 * nmat, "rows: ids");
  need(prefix, 8.0 * (nmat + 1), "rows: prefix");
  if (prefix[0] != 0 || prefix[nmat] != total_rows) fail("rows: prefix ends");
  for (int32_t k = 0; k < nmat; ++k) {
    need(&mats[ids[k]], sizeof(muon::MatDev), "rows: mat entry");
    const muon::MatDev& d = mats[ids[k]];
    if (prefix[k + 1] - prefix[k] != d.rows) fail("rows: prefix step %d != rows", k);
    if (max_chunks > 0 && (d.cols % 4 || d.cols > int64_t(max_chunks) * muon::kRowChunkElems))
      fail("rows: %lld columns in chunk class %d", (long long)d.cols, max_chunks);
    mat_tensors(d, "rows: tensors");
  }
}

int64_t g_tall_limit = 0;   // the planner's residency bound for the single pass

void check_tall(const muon::MatDev* mats, const muon::TileItem* tiles, int64_t ntiles,
                const muon::TallSync* sync, const muon::TallCtl* ctl, const uint32_t* repair) {
  need(tiles, 8.0 * ntiles, "tall: tiles");
  need(ctl, sizeof(muon::TallCtl), "tall: control");
  need(repair, 4.0 * ntiles, "tall: repair list");
  // Every wait ends if each strip's tiles lie within a window of at most
  // g_tall_limit consecutive workgroups (a workgroup still waiting then holds
  // one of at most window / 8 slots of its XCD), in chunk order; the planner
  // lists each strip as one run of consecutive workgroups.
  std::map<std::pair<int32_t, int32_t>, std::pair<int64_t, int32_t>> first_next;
  for (int64_t b = 0; b < ntiles; ++b) {
    const muon::TileItem it = tiles[b];
    auto& fn = first_next[{it.id, it.tj}];
    if (it.ti == 0) fn.first = b;
    if (it.ti != fn.second) fail("tall: strip (%d, %d) chunk %d out of order", it.id, it.tj, it.ti);
    fn.second = it.ti + 1;
    if (b - fn.first + 1 > g_tall_limit)
      fail("tall: strip (%d, %d) spans more than %lld workgroups", it.id, it.tj, (long long)g_tall_limit);
  }
  for (int64_t b = 0; b < ntiles; ++b) {
    const muon::TileItem it = tiles[b];
    need(&mats[it.id], sizeof(muon::MatDev), "tall: mat entry");
    const muon::MatDev& d = mats[it.id];
    const int64_t nchunk = cdiv(d.rows, muon::kTallRows), nstrip = cdiv(d.cols, muon::kTallCols);
    if (d.rows <= d.cols || d.cols % 2 || nchunk > muon::kTallMaxChunks)
      fail("tall: matrix %d (%lld x %lld) cannot take the single pass", it.id, (long long)d.rows,
           (long long)d.cols);
    if (it.ti < 0 || it.ti >= nchunk || it.tj < 0 || it.tj >= nstrip) fail("tall: tile index");
    mat_tensors(d, "tall: tensors");
    need(d.part, 4.0 * nstrip * (nchunk + 1) * muon::kTallCols, "tall: partial rows");
    need(&sync[d.sync0 + it.tj], sizeof(muon::TallSync), "tall: strip counters");
  }
}

void check_cols(const muon::MatDev* mats, const muon::TileItem* tiles, int64_t ntiles) {
  need(tiles, 8.0 * ntiles, "cols: tiles");
  for (int64_t b = 0; b < ntiles; ++b) {
    const muon::TileItem it = tiles[b];
    need(&mats[it.id], sizeof(muon::MatDev), "cols: mat entry");
    const muon::MatDev& d = mats[it.id];
    if (int64_t(it.ti) * muon::kColTileRows >= d.rows || int64_t(it.tj) * muon::kColTileCols >= d.cols)
      fail("cols: tile index");
    mat_tensors(d, "cols: tensors");
    need(d.part, 4.0 * cdiv(d.rows, muon::kColTileRows) * d.cols, "cols: partials");
  }
}

void check_ns_dev(const muon::NsDev& d, int prec, const char* k) {
  const double es = prec == 1 ? 4 : 2;
  need(d.x[0], es * d.rp * d.cp, k);
  if (prec == 2) need(d.xlo, 2.0 * d.rp * d.cp, k);
  else if (d.xlo) fail("%s: remainder buffer without the remainder precision", k);
  if (prec == 1) {
    need(d.xt[0], es * d.rp * d.cp, k);
    need(d.xt[1], es * d.rp * d.cp, k);
  } else {
    need(d.x[1], es * d.rp * d.cp, k);
  }
  need(d.a, es * d.rp * d.rp, k);
  need(d.b, es * d.rp * d.rp, k);
  need(d.part, 4.0 * d.nparts, k);
  need(d.scale, 4, k);
  need(d.adiag, 4.0 * d.rp, k);
  need(d.bdiag, 4.0 * d.rp, k);
  if (d.r != std::min(d.rows, d.cols) || d.c != std::max(d.rows, d.cols) || d.rp < d.r ||
      d.cp < d.c || d.rp % 128 || d.cp % 128)
    fail("%s: padded dims", k);
  if (double(d.rp) * d.cp * es >= 4294967296.0) fail("%s: workspace over 4 GiB", k);
}

void stored_block(const muon::MatDev* mats, const muon::NsDev& d, bool w_too, const char* k) {
  need(&mats[d.mat], sizeof(muon::MatDev), k);
  const muon::MatDev& mt = mats[d.mat];
  if (d.col0 + d.cols > d.ld || d.ld != mt.cols || d.rows != mt.rows) fail("%s: block geometry", k);
  const double span = double(d.rows - 1) * d.ld + d.col0 + d.cols;
  need(mt.mom, 4 * span, k);
  need(mt.g, (mt.gdt == 1 ? 2 : 4) * span, k);
  if (w_too) need(mt.w, 4 * span, k);
}

void check_prep(const muon::MatDev* mats, const muon::NsDev* ns, const muon::TileItem* items,
                int64_t nitems, int prec) {
  need(items, 8.0 * nitems, "prep: items");
  for (int64_t b = 0; b < nitems; ++b) {
    const muon::TileItem it = items[b];
    need(&ns[it.id], sizeof(muon::NsDev), "prep: ns entry");
    const muon::NsDev& d = ns[it.id];
    check_ns_dev(d, prec, "prep: workspace");
    stored_block(mats, d, false, "prep: stored block");
    const int64_t sp = d.tall ? d.cp : d.rp, sq = d.tall ? d.rp : d.cp;
    if (it.ti < 0 || int64_t(it.ti) * 64 >= sp || it.tj < 0 || int64_t(it.tj) * 64 >= sq)
      fail("prep: tile index");
    if (int64_t(it.ti) * (sq / 64) + it.tj >= d.nparts) fail("prep: partial index");
  }
}

void check_gemm(const muon::MatDev* mats, const muon::NsDev* ns, const muon::GemmItem* items,
                int64_t nitems, int op, int tile, int tile_n, int prec, int last) {
  need(items, 8.0 * nitems, "gemm: items");
  for (int64_t b = 0; b < nitems; ++b) {
    const muon::GemmItem it = items[b];
    need(&ns[it.ns], sizeof(muon::NsDev), "gemm: ns entry");
    const muon::NsDev& d = ns[it.ns];
    check_ns_dev(d, prec, "gemm: workspace");
    const int64_t i0 = int64_t(it.ti) * tile, j0 = int64_t(it.tj) * tile_n;
    const int64_t jmax = op == muon::kGemmProduct ? d.cp : d.rp;
    if (it.ti < 0 || it.tj < 0 || i0 + tile > d.rp || j0 + tile_n > jmax)
      fail("gemm op %d: tile (%d, %d) of %d x %d outside %lld x %lld", op, it.ti, it.tj, tile,
           tile_n, (long long)d.rp, (long long)jmax);
    if (op != muon::kGemmProduct && it.ti > it.tj) fail("gemm op %d: lower-triangle tile", op);
    if (d.rp % tile || (op == muon::kGemmProduct && d.cp % tile_n)) fail("gemm: padding vs tile");
    if (op == muon::kGemmProduct && last) stored_block(mats, d, true, "gemm: weight update");
  }
}

// Whole-triangle Gram: one workgroup per listed bf16 problem with rp ==
// kTriRows, reading X (rp x cp, whole 32-column k-steps) and writing A and
// adiag; listed longest first.
void check_gram_tri(const muon::NsDev* ns, const muon::GemmItem* items, int64_t nitems) {
  need(items, 8.0 * nitems, "gram_tri: items");
  int64_t prev = INT64_MAX;
  for (int64_t b = 0; b < nitems; ++b) {
    const muon::GemmItem it = items[b];
    need(&ns[it.ns], sizeof(muon::NsDev), "gram_tri: ns entry");
    const muon::NsDev& d = ns[it.ns];
    check_ns_dev(d, d.xlo ? 2 : 0, "gram_tri: workspace");   // reads X's bf16 part only
    if (d.rp != muon::kTriRows) fail("gram_tri: problem %d has rp %lld", it.ns, (long long)d.rp);
    if (d.cp < 256 || d.cp % 256) fail("gram_tri: cp %lld", (long long)d.cp);
    if (d.cp > prev) fail("gram_tri: not listed longest first");
    prev = d.cp;
  }
}

void check_adam(const muon::AdamDev* t, const muon::AdamChunk* chunks, int64_t n) {
  need(chunks, 16.0 * n, "adamw: chunks");
  for (int64_t b = 0; b < n; ++b) {
    const muon::AdamChunk ck = chunks[b];
    need(&t[ck.tensor], sizeof(muon::AdamDev), "adamw: entry");
    const muon::AdamDev& a = t[ck.tensor];
    if (ck.off < 0 || ck.len < 1 || ck.off + ck.len > a.numel) fail("adamw: chunk range");
    need(a.p, 4.0 * a.numel, "adamw: p");
    need(a.m, 4.0 * a.numel, "adamw: m");
    need(a.v, 4.0 * a.numel, "adamw: v");
    need(a.g, (a.gdt == 1 ? 2.0 : 4.0) * a.numel, "adamw: g");
  }
}

// ---- no-alloc scratch stand-in --------------------------------------------
void* scratch_buffer() {
  static void* p = nullptr;
  if (!p) p = std::aligned_alloc(256, muon::kNoallocScratchBytes);
  return p;
}

}  // namespace chk

// ---- stubbed HIP runtime --------------------------------------------------
extern "C" {
hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) { *v = 256; return hipSuccess; }
hipError_t hipMemsetAsync(void* p, int v, size_t n, hipStream_t) {
  chk::need(p, double(n), "hipMemsetAsync");
  if (!chk::g_fail) std::memset(p, v, n);
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind kind, hipStream_t) {
  if (kind == hipMemcpyHostToDevice) chk::need(dst, double(n), "hipMemcpyAsync(H2D)");
  if (!chk::g_fail) std::memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind kind) {
  if (kind == hipMemcpyDeviceToHost) chk::need(src, double(n), "hipMemcpy(D2H)");
  if (!chk::g_fail) std::memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "stub"; }
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipEventCreate(hipEvent_t* e) { *e = reinterpret_cast<hipEvent_t>(new int(0)); return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) { *ms = 0.f; return hipSuccess; }
hipError_t hipEventDestroy(hipEvent_t e) { delete reinterpret_cast<int*>(e); return hipSuccess; }
}

// ---- stubbed launchers (muon_internal.h) -----------------------------------
namespace muon {
hipError_t rownorm_tall_resident(int* w) { *w = 2; return hipSuccess; }
hipError_t noalloc_scratch(void** p) { *p = chk::scratch_buffer(); return hipSuccess; }
hipError_t launch_fill_zero(hipStream_t, void* p, size_t bytes) {
  ++chk::g_launches;
  if (bytes % 4) chk::fail("fill_zero: %zu bytes", bytes);
  chk::need(p, double(bytes), "fill_zero");
  if (!chk::g_fail) std::memset(p, 0, bytes);
  return hipSuccess;
}
hipError_t launch_ns_gram_tri(hipStream_t, const NsDev* ns, const GemmItem* items, int64_t nitems,
                              int) {
  ++chk::g_launches;
  chk::check_gram_tri(ns, items, nitems);
  return hipSuccess;
}
hipError_t launch_rownorm_rows(hipStream_t, const MatDev* mats, const int32_t* ids,
                               const int64_t* prefix, int32_t nmat, int64_t total_rows,
                               int max_chunks, StepScalars) {
  ++chk::g_launches;
  chk::check_rows(mats, ids, prefix, nmat, total_rows, max_chunks);
  return hipSuccess;
}
hipError_t launch_rownorm_coef(hipStream_t, const MatDev* mats, const TileItem* strips,
                               int64_t nstrips, StepScalars) {
  ++chk::g_launches;
  chk::check_cols(mats, strips, nstrips);
  return hipSuccess;
}
hipError_t launch_rownorm_cols(hipStream_t, const MatDev* mats, const TileItem* tiles,
                               int64_t ntiles, int, StepScalars) {
  ++chk::g_launches;
  chk::check_cols(mats, tiles, ntiles);
  return hipSuccess;
}
hipError_t launch_rownorm_tall(hipStream_t, const MatDev* mats, const TileItem* tiles,
                               int64_t ntiles, TallSync* sync, TallCtl* ctl, uint32_t* repair,
                               uint32_t, StepScalars) {
  ++chk::g_launches;
  chk::check_tall(mats, tiles, ntiles, sync, ctl, repair);
  return hipSuccess;
}
hipError_t launch_rownorm_repair(hipStream_t, const MatDev* mats, const TileItem* tiles,
                                 int64_t ntiles, TallCtl* ctl, const uint32_t* repair,
                                 StepScalars) {
  ++chk::g_launches;
  chk::need(ctl, sizeof(TallCtl), "repair: control");
  chk::need(repair, 4.0 * ntiles, "repair: list");
  chk::need(tiles, 8.0 * ntiles, "repair: tiles");
  (void)mats;
  return hipSuccess;
}
hipError_t launch_ns_prep(hipStream_t, const MatDev* mats, const NsDev* ns, const TileItem* items,
                          int64_t nitems, int prec, float) {
  ++chk::g_launches;
  chk::check_prep(mats, ns, items, nitems, prec);
  return hipSuccess;
}
hipError_t launch_ns_scale(hipStream_t, NsDev* ns, int32_t count, float) {
  ++chk::g_launches;
  for (int32_t k = 0; k < count; ++k) {
    chk::need(&ns[k], sizeof(NsDev), "scale: ns entry");
    chk::need(ns[k].part, 4.0 * ns[k].nparts, "scale: partials");
    chk::need(ns[k].scale, 4, "scale: scale");
  }
  return hipSuccess;
}
hipError_t launch_ns_gemm(hipStream_t, const MatDev* mats, const NsDev* ns, const GemmItem* items,
                          int64_t nitems, int op, int tile, int tile_n, int prec, int, int last,
                          float, float, float, float) {
  ++chk::g_launches;
  if (tile_n != tile && (prec == 1 || tile != 128 || tile_n != 256 || op != kGemmProduct || last))
    chk::fail("gemm: tile %d x %d not built for op %d prec %d last %d", tile, tile_n, op, prec, last);
  chk::check_gemm(mats, ns, items, nitems, op, tile, tile_n, prec, last);
  return hipSuccess;
}
hipError_t launch_adamw(hipStream_t, const AdamDev* t, const AdamChunk* chunks, int64_t n, float,
                        float, float, float, float, float, float) {
  ++chk::g_launches;
  chk::check_adam(t, chunks, n);
  return hipSuccess;
}
hipError_t launch_patch(hipStream_t, MatDev* mats, AdamDev* adams, const PatchArgs& a) {
  ++chk::g_launches;
  if (a.count < 0 || a.count > kPatchMax) chk::fail("patch: count %d", a.count);
  for (int k = 0; k < a.count; ++k) {
    if (a.adam) {
      chk::need(&adams[a.idx[k]], sizeof(AdamDev), "patch: adam entry");
      adams[a.idx[k]].p = static_cast<float*>(a.w[k]);
      adams[a.idx[k]].g = a.g[k];
    } else {
      chk::need(&mats[a.idx[k]], sizeof(MatDev), "patch: mat entry");
      mats[a.idx[k]].w = static_cast<float*>(a.w[k]);
      mats[a.idx[k]].g = a.g[k];
    }
  }
  return hipSuccess;
}
}  // namespace muon

// ---- whole-plan structure ----------------------------------------------------
namespace chk {

struct Region {
  size_t lo, hi;
  std::string what;
};

// Every carved region inside [0, total), pairwise disjoint; every tile set
// covers its grid exactly once.
void check_plan(const Plan& pl, const muon_config& cfg, const muon_tensor* params,
                const int32_t* kinds, int32_t n, bool ext_mom, int64_t tall_limit) {
  std::vector<Region> rg;
  auto add = [&](size_t off, size_t bytes, const std::string& w) {
    if (bytes) rg.push_back({off, off + bytes, w});
  };
  for (int32_t i = 0; i < n; ++i) {
    const size_t e = size_t(params[i].rows) * size_t(params[i].cols);
    if (kinds[i] == MUON_KIND_MATRIX) {
      if (!ext_mom) add(pl.mom_off[i], 4 * e, "momentum " + std::to_string(i));
    } else {
      add(pl.m_off[i], 4 * e, "adam m " + std::to_string(i));
      add(pl.v_off[i], 4 * e, "adam v " + std::to_string(i));
    }
  }
  add(pl.off_mats, pl.mats.size() * sizeof(MatDev), "mats");
  add(pl.off_adams, pl.adams.size() * sizeof(AdamDev), "adams");
  add(pl.off_col_tiles, size_t(pl.n_col_tiles_max) * sizeof(TileItem), "col tiles");
  add(pl.off_col_strips, size_t(pl.n_col_strips_max) * sizeof(TileItem), "col strips");
  add(pl.off_tall_tiles, size_t(pl.n_tall_tiles_max) * sizeof(TileItem), "tall tiles");
  add(pl.off_tall_sync, pl.tall_sync_bytes, "tall control");
  add(pl.off_adam_chunks, pl.adam_chunks.size() * sizeof(AdamChunk), "adam chunks");
  for (const RowGroup& g : pl.row_groups) {
    add(g.off_ids, g.ids.size() * 4, "row ids");
    add(g.off_prefix, g.prefix.size() * 8, "row prefix");
  }
  for (const auto* plan : {&pl.ns_full, &pl.ns_block})
    for (const NsChunk& ch : *plan) {
      add(ch.off_ns, ch.ns.size() * sizeof(NsDev), "ns table");
      add(ch.off_prep, ch.prep_items.size() * sizeof(TileItem), "prep items");
      for (const auto& op : ch.gemm)
        for (const auto& gl : op) add(gl.off, gl.items.size() * sizeof(GemmItem), "gemm items");
      add(ch.prod_wide.off, ch.prod_wide.items.size() * sizeof(GemmItem), "wide product items");
      add(ch.gram_tri.off, ch.gram_tri.items.size() * sizeof(GemmItem), "whole-triangle gram items");
      if (ch.ws_bytes > pl.ws_bytes) fail("chunk workspace over the reserved workspace");
    }
  add(pl.ws_base, pl.ws_bytes, "workspace");
  // partial rows of tall matrices (inside the zeroed prefix)
  for (int32_t i = 0; i < n; ++i)
    if (kinds[i] == MUON_KIND_MATRIX && pl.part_off[i] >= pl.zero_end && params[i].rows > params[i].cols &&
        cfg.rownorm_axis == 0)
      fail("partials of matrix %d are not in the zeroed prefix", i);
  std::sort(rg.begin(), rg.end(), [](const Region& a, const Region& b) { return a.lo < b.lo; });
  for (size_t k = 0; k < rg.size(); ++k) {
    ++g_checks;
    if (rg[k].hi > pl.total) fail("region %s ends past the buffer", rg[k].what.c_str());
    if (k && rg[k].lo < rg[k - 1].hi)
      fail("regions %s and %s overlap", rg[k - 1].what.c_str(), rg[k].what.c_str());
  }
  // RowNorm coverage: each matrix in exactly one of rows / tall / two-pass
  std::vector<int> seen(pl.mats.size(), 0);
  for (const RowGroup& g : pl.row_groups)
    for (int32_t id : g.ids) seen[id] += 1;
  std::vector<std::vector<int>> tall_hits(pl.mats.size());
  for (const TileItem& t : pl.tall_tiles) {
    const MatDev& d = pl.mats[t.id];
    auto& h = tall_hits[t.id];
    if (h.empty()) { h.assign(cdiv(d.rows, kTallRows) * cdiv(d.cols, kTallCols), 0); seen[t.id] += 1; }
    h[t.tj * cdiv(d.rows, kTallRows) + t.ti] += 1;
    if (cdiv(d.rows, kTallRows) > tall_limit) fail("tall: matrix %d over the residency limit", t.id);
  }
  for (auto& h : tall_hits)
    for (int c : h)
      if (c != 1) fail("tall: a tile listed %d times", c);
  std::vector<int> two(pl.mats.size(), 0);
  for (const TileItem& t : pl.col_tiles) two[t.id] += 1;
  for (size_t k = 0; k < pl.mats.size(); ++k) {
    const MatDev& d = pl.mats[k];
    if (two[k]) {
      seen[k] += 1;
      if (two[k] != cdiv(d.rows, kColTileRows) * cdiv(d.cols, kColTileCols)) fail("cols: tile count");
    }
    if (seen[k] != 1) fail("RowNorm: matrix %zu planned %d times", k, seen[k]);
  }
  // NS coverage per chunk
  for (const auto* plan : {&pl.ns_full, &pl.ns_block})
    for (const NsChunk& ch : *plan) {
      // workgroup p runs on XCD p mod 8: the K summed per XCD is balanced
      for (int op = 0; op < 3; ++op)
        for (const auto& gl : ch.gemm[op]) {
          if (gl.items.size() < 1024) continue;
          double c[8] = {0};
          for (size_t q = 0; q < gl.items.size(); ++q)
            c[q % 8] += double(op == kGemmGram ? ch.ns[gl.items[q].ns].cp : ch.ns[gl.items[q].ns].rp);
          const double lo = *std::min_element(c, c + 8), hi = *std::max_element(c, c + 8);
          ++g_checks;
          if (hi > 1.03 * lo) fail("gemm op %d: XCD cost imbalance %.3f", op, hi / lo);
        }
      const size_t es = cfg.ns_precision == MUON_NS_F32 ? 4 : 2;
      for (int32_t k = 0; k < int32_t(ch.ns.size()); ++k) {
        const NsDev& d = ch.ns[k];
        const int tile = d.r >= 1024 ? 256 : 128;
        const int64_t nr = d.rp / tile, nc = d.cp / tile;
        int64_t gram = 0, prod = 0, prep = 0, wide = 0, tri = 0;
        for (const GemmItem& g : ch.gemm[kGemmGram][tile == 256].items) gram += g.ns == k;
        for (const GemmItem& g : ch.gram_tri.items) tri += g.ns == k;
        for (const GemmItem& g : ch.gemm[kGemmProduct][tile == 256].items) prod += g.ns == k;
        for (const GemmItem& g : ch.prod_wide.items) wide += g.ns == k;
        for (const TileItem& t : ch.prep_items) prep += t.id == k;
        const bool whole = es == 2 && d.rp == kTriRows;
        if (gram != (whole ? 0 : nr * (nr + 1) / 2) || tri != (whole ? 1 : 0))
          fail("gram of problem %d: %lld tiles, %lld whole", k, (long long)gram, (long long)tri);
        if (prod != nr * nc) fail("product tiles of problem %d", k);
        if (es == 2 && tile == 128 && wide != nr * (d.cp / 256)) fail("wide product tiles");
        if (prep != (d.rp / 64) * (d.cp / 64)) fail("prep tiles of problem %d", k);
      }
    }
}

int64_t fake_tall_limit() {
  int per = 0;
  muon::rownorm_tall_resident(&per);
  return std::min<int64_t>(kTallMaxChunks, 256 * per / 2);
}

// A DiT-shaped set (5 matrices per block) plus its bias vectors.
std::vector<std::pair<int64_t, int64_t>> dit(int64_t d, int blocks) {
  std::vector<std::pair<int64_t, int64_t>> s;
  for (int b = 0; b < blocks; ++b)
    for (auto mn : {std::make_pair(3 * d, d), std::make_pair(d, d), std::make_pair(4 * d, d),
                    std::make_pair(d, 4 * d), std::make_pair(6 * d, d)})
      s.push_back(mn);
  return s;
}

// Plan-only: no memory behind the buffer or the tensors.
void plan_only(const char* name, const std::vector<std::pair<int64_t, int64_t>>& shapes,
               const muon_config& cfg) {
  g_scenario = std::string("plan ") + name;
  const int32_t n = int32_t(shapes.size());
  std::vector<muon_tensor> p(n), g(n);
  std::vector<int32_t> kinds(n, MUON_KIND_MATRIX);
  uintptr_t fake = uintptr_t(1) << 44;
  unreg_all();
  for (int32_t i = 0; i < n; ++i) {
    const double e = double(shapes[i].first) * shapes[i].second;
    p[i] = {reinterpret_cast<void*>(fake), shapes[i].first, shapes[i].second, shapes[i].second, MUON_F32, 0};
    reg(p[i].ptr, size_t(4 * e), "W");
    fake += (size_t(4 * e) + 4095) / 4096 * 4096 + 4096;
    g[i] = {reinterpret_cast<void*>(fake), shapes[i].first, shapes[i].second, shapes[i].second, MUON_BF16, 0};
    reg(g[i].ptr, size_t(2 * e), "G");
    fake += (size_t(2 * e) + 4095) / 4096 * 4096 + 4096;
  }
  size_t bytes = 0;
  if (muon_state_bytes(&cfg, p.data(), kinds.data(), n, &bytes) != MUON_OK) {
    fail("%s: muon_state_bytes: %s", name, muon_last_error(nullptr));
    return;
  }
  char* base = reinterpret_cast<char*>(uintptr_t(1) << 46);
  reg(base, bytes, "state");
  Plan pl;
  std::string err;
  const int64_t lim = fake_tall_limit();
  if (build_plan(cfg, p.data(), kinds.data(), n, base, pl, err, lim) != MUON_OK) {
    fail("%s: build_plan: %s", name, err.c_str());
    return;
  }
  if (pl.total != bytes) fail("%s: plan size differs from muon_state_bytes", name);
  bind_tensors(pl, p.data(), g.data(), kinds.data(), n);
  check_plan(pl, cfg, p.data(), kinds.data(), n, false, lim);
  // the launches of every branch, on the host copies of the tables
  reg(pl.mats.data(), pl.mats.size() * sizeof(MatDev), "host mats");
  for (const RowGroup& rgp : pl.row_groups) {
    reg(rgp.ids.data(), rgp.ids.size() * 4, "host ids");
    reg(rgp.prefix.data(), rgp.prefix.size() * 8, "host prefix");
    check_rows(pl.mats.data(), rgp.ids.data(), rgp.prefix.data(), int32_t(rgp.ids.size()),
               rgp.prefix.back(), rgp.max_chunks);
  }
  char* tb = base + pl.off_tall_sync;
  reg(pl.tall_tiles.data(), pl.tall_tiles.size() * sizeof(TileItem), "host tall tiles");
  check_tall(pl.mats.data(), pl.tall_tiles.data(), int64_t(pl.tall_tiles.size()),
             reinterpret_cast<TallSync*>(tb + sizeof(TallCtl) + pl.tall_list_bytes),
             reinterpret_cast<TallCtl*>(tb), reinterpret_cast<uint32_t*>(tb + sizeof(TallCtl)));
  reg(pl.col_tiles.data(), pl.col_tiles.size() * sizeof(TileItem), "host col tiles");
  check_cols(pl.mats.data(), pl.col_tiles.data(), int64_t(pl.col_tiles.size()));
  const int prec = cfg.ns_precision;
  size_t nchunks = 0;
  for (const auto* plan : {&pl.ns_full, &pl.ns_block})
    for (const NsChunk& ch : *plan) {
      ++nchunks;
      reg(ch.ns.data(), ch.ns.size() * sizeof(NsDev), "host ns");
      reg(ch.prep_items.data(), ch.prep_items.size() * sizeof(TileItem), "host prep");
      check_prep(pl.mats.data(), ch.ns.data(), ch.prep_items.data(), int64_t(ch.prep_items.size()), prec);
      for (int op = 0; op < 3; ++op)
        for (int t = 0; t < 2; ++t) {
          const auto& gl = ch.gemm[op][t];
          if (gl.items.empty()) continue;
          reg(gl.items.data(), gl.items.size() * sizeof(GemmItem), "host items");
          check_gemm(pl.mats.data(), ch.ns.data(), gl.items.data(), int64_t(gl.items.size()), op,
                     t ? 256 : 128, t ? 256 : 128, prec, 1);
        }
      if (!ch.prod_wide.items.empty()) {
        reg(ch.prod_wide.items.data(), ch.prod_wide.items.size() * sizeof(GemmItem), "host wide");
        check_gemm(pl.mats.data(), ch.ns.data(), ch.prod_wide.items.data(),
                   int64_t(ch.prod_wide.items.size()), kGemmProduct, 128, 256, prec, 0);
      }
      if (!ch.gram_tri.items.empty()) {
        reg(ch.gram_tri.items.data(), ch.gram_tri.items.size() * sizeof(GemmItem), "host tri");
        check_gram_tri(ch.ns.data(), ch.gram_tri.items.data(), int64_t(ch.gram_tri.items.size()));
      }
    }
  // no chunk of a plan is a small remainder
  double ws_lo = 0, ws_hi = 0;
  for (const auto* plan : {&pl.ns_full, &pl.ns_block}) {
    if (plan->size() < 2) continue;
    double lo = 1e300, hi = 0;
    for (const NsChunk& ch : *plan) {
      lo = std::min(lo, double(ch.ws_bytes));
      hi = std::max(hi, double(ch.ws_bytes));
    }
    ++g_checks;
    if (lo < 0.5 * hi) fail("NS chunks of %.2f to %.2f GB", lo / 1e9, hi / 1e9);
    ws_lo = lo; ws_hi = hi;
  }
  std::printf("plan %-28s %4d matrices  %6.1f GB  %zu NS chunks (%.2f-%.2f GB)  %zu tall tiles\n",
              name, n, bytes / 1e9, nchunks, ws_lo / 1e9, ws_hi / 1e9, pl.tall_tiles.size());
}

// Full: host memory behind everything, through the public entry points.
struct HostSet {
  std::vector<std::vector<char>> bufs;
  std::vector<muon_tensor> p, g, m;
  std::vector<int32_t> kinds;
  void* add(size_t bytes, const char* what) {
    bufs.emplace_back(bytes + 256);
    char* q = bufs.back().data();
    q += (256 - reinterpret_cast<uintptr_t>(q) % 256) % 256;
    reg(q, bytes, what);
    return q;
  }
};

void fill(void* p, size_t floats, uint32_t seed) {
  float* f = static_cast<float*>(p);
  for (size_t i = 0; i < floats; ++i) {
    seed = seed * 1664525u + 1013904223u;
    f[i] = float(int32_t(seed >> 8) % 2001 - 1000) * 1e-3f;
  }
}

void full(const char* name, const std::vector<std::pair<int64_t, int64_t>>& shapes, int n_adam,
          const muon_config& cfg, int steps, bool noalloc) {
  g_scenario = std::string("full ") + name;
  unreg_all();
  reg(scratch_buffer(), kNoallocScratchBytes, "no-alloc scratch");
  HostSet hs;
  const int32_t n = int32_t(shapes.size()) + n_adam;
  for (int32_t i = 0; i < n; ++i) {
    const bool adam = i >= int32_t(shapes.size());
    const int64_t r = adam ? 1 : shapes[i].first, c = adam ? 1000 + 37 * i : shapes[i].second;
    const int gdt = (i % 2) ? MUON_BF16 : MUON_F32;
    void* w = hs.add(size_t(4 * r * c), "W");
    void* gg = hs.add(size_t((gdt == MUON_BF16 ? 2 : 4) * r * c), "G");
    void* mm = hs.add(size_t(4 * r * c), "M");
    fill(w, size_t(r * c), 7u * i + 1);
    std::memset(mm, 0, size_t(4 * r * c));
    hs.p.push_back({w, r, c, c, MUON_F32, 0});
    hs.g.push_back({gg, r, c, c, gdt, 0});
    hs.m.push_back({mm, r, c, c, MUON_F32, 0});
    hs.kinds.push_back(adam ? MUON_KIND_ADAMW : MUON_KIND_MATRIX);
  }
  size_t bytes = 0;
  if (muon_state_bytes(&cfg, hs.p.data(), hs.kinds.data(), n, &bytes) != MUON_OK) {
    fail("%s: muon_state_bytes: %s", name, muon_last_error(nullptr));
    return;
  }
  void* state = hs.add(bytes, "state");
  muon_ctx* ctx = nullptr;
  if (muon_init(&ctx, &cfg, hs.p.data(), hs.g.data(), hs.kinds.data(), n, state, bytes, nullptr) != MUON_OK) {
    fail("%s: muon_init: %s", name, muon_last_error(nullptr));
    return;
  }
  check_plan(ctx->plan, cfg, hs.p.data(), hs.kinds.data(), n, false, fake_tall_limit());
  muon_timing_enable(ctx, 1);
  for (int t = 0; t < steps; ++t) {
    std::vector<muon_tensor> p = hs.p, g = hs.g;
    if (t == 2 && n > 0) {   // new buffers for the first tensor: the patch path
      p[0].ptr = hs.add(size_t(4 * p[0].rows * p[0].cols), "W'");
      g[0].ptr = hs.add(size_t((g[0].dtype == MUON_BF16 ? 2 : 4) * g[0].rows * g[0].cols), "G'");
    }
    if (muon_step(ctx, p.data(), g.data(), t) != MUON_OK) fail("%s: muon_step %d: %s", name, t, muon_last_error(ctx));
  }
  double ms[MUON_K_COUNT];
  int64_t cnt[MUON_K_COUNT];
  uint64_t gave = 1;
  if (muon_timing_read(ctx, ms, cnt) != MUON_OK || muon_sync(ctx) != MUON_OK ||
      muon_tall_giveups(ctx, &gave) != MUON_OK || gave != 0)
    fail("%s: timing / sync / give-up count", name);
  for (int32_t i = 0; i < n; ++i) {
    muon_tensor v{};
    if (muon_state(ctx, i, 0, &v) != MUON_OK) fail("%s: muon_state %d", name, i);
    need(v.ptr, 4.0 * v.rows * v.cols, "muon_state view");
  }
  muon_free(ctx);
  if (noalloc) {
    const int32_t nm = int32_t(shapes.size());
    for (int t = 0; t < steps; ++t)
      if (muon_step_noalloc(&cfg, hs.p.data(), hs.g.data(), hs.m.data(), nm, t, nullptr) != MUON_OK)
        fail("%s: muon_step_noalloc %d: %s", name, t, muon_last_error(nullptr));
  }
  std::printf("full %-28s %4d tensors  %8.1f MB state  noalloc %d\n", name, n, bytes / 1e6, int(noalloc));
}

}  // namespace chk

int main() {
  using namespace chk;
  g_tall_limit = fake_tall_limit();
  muon_config def;
  muon_config_default(&def);
  muon_config f32 = def, two = def, rows = def, bp = def, cap = def, comp = def;
  f32.ns_precision = MUON_NS_F32;
  comp.ns_precision = MUON_NS_BF16_COMP;
  two.tall_single_pass = 0;
  rows.rownorm_axis = 1;
  bp.bp_blocks = 8;
  cap.ns_workspace_max = uint64_t(1) << 30;
  // DiT sets, plan only
  plan_only("dit-1.3b", dit(2048, 18), def);
  plan_only("dit-1.3b fp32 NS5", dit(2048, 18), f32);
  plan_only("dit-1.3b two-pass", dit(2048, 18), two);
  plan_only("dit-1.3b stored rows", dit(2048, 18), rows);
  plan_only("dit-4b", dit(3072, 24), def);
  plan_only("dit-4b muonbp", dit(3072, 24), bp);
  plan_only("dit-15b", dit(5120, 32), def);
  plan_only("dit-15b 1 GiB workspace cap", dit(5120, 32), cap);
  plan_only("dit-15b bf16 with X's remainder", dit(5120, 32), comp);
  plan_only("dit-15b muonbp", dit(5120, 32), bp);
  // ragged and edge shapes, through the entry points
  const std::vector<std::pair<int64_t, int64_t>> ragged = {
      {300, 700}, {700, 300}, {128, 128}, {1, 64}, {64, 1}, {260, 260}, {33, 2050}, {2050, 33},
      {1200, 1030}, {1000, 300}, {129, 4}, {520, 516}, {2200, 2048}, {33000, 40}, {700, 301},
      {3, 9000}, {2, 20000}, {5, 16388}, {4, 40000}, {3, 33001}, {32768, 256}};
  muon_config small_cap = def;
  small_cap.ns_workspace_max = uint64_t(8) << 20;
  for (auto [nm, c] : {std::make_pair("ragged", def), std::make_pair("ragged fp32", f32),
                       std::make_pair("ragged two-pass", two), std::make_pair("ragged stored rows", rows),
                       std::make_pair("ragged 8 MiB cap", small_cap),
                       std::make_pair("ragged bf16 with X's remainder", comp)}) {
    full(nm, ragged, 3, c, 4, true);
  }
  // (384 x 3072: blocks with r = 384, and 3072 x 384: r = 384 on the full steps; their Gram runs
  // one workgroup per problem)
  full("muonbp", {{512, 1024}, {1024, 512}, {384, 384}, {96, 4096}, {384, 3072}, {3072, 384}}, 1, bp,
       4, true);
  muon_config bp_comp = bp;
  bp_comp.ns_precision = MUON_NS_BF16_COMP;
  full("muonbp bf16 with X's remainder", {{512, 1024}, {384, 3072}, {3072, 384}}, 1, bp_comp, 4, true);
  // the no-alloc entry point refuses a matrix whose workspace does not fit
  {
    g_scenario = "no-alloc refusal";
    HostSet hs;
    void* w = hs.add(4, "W");
    muon_tensor p{w, 3072, 18432, 18432, MUON_F32, 0};
    muon_tensor g{w, 3072, 18432, 18432, MUON_BF16, 0};
    const long before = g_launches;
    if (muon_step_noalloc(&def, &p, &g, &p, 1, 0, nullptr) != MUON_E_WORKSPACE || g_launches != before)
      fail("no-alloc: a matrix beyond the scratch was not refused before any launch");
  }
  std::printf("checks %ld  launches %ld  failures %ld\n", g_checks, g_launches, g_fail);
  return g_fail ? 1 : 0;
}
