// Host side of the C ABI: validation, planning, state-buffer carving, and the
// per-step launch sequence.  No device memory is ever allocated here: every
// device byte comes from the caller's state buffer.
//
// Schedule (PaperDaily post on "Scaling Muon for Diffusion Transformers",
// section "Periodic Row-wise Muon", blog fig. 3): refresh when t mod K == 0,
// RowNorm otherwise; with MuonBP ("MuonBP: Faster Muon via Block-Periodic
// Orthogonalization", abstract) full NS5 every bp_period steps and per-block
// NS5 in between, with its own step size.
//
// The pages' distributed design gathers momentum in buckets so only a
// bounded number of full matrices is materialised at a time (the post's
// section "distributed co-design").  On one GPU that becomes NS5 "chunks":
// problems are grouped so that one chunk's workspace stays under
// ns_workspace_max, and each chunk runs all its matrices through every
// Newton-Schulz round with one grouped launch per product.
#include "../../include/muon.h"
#include "gram_tri.h"
#include "muon_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

using namespace muon;

namespace {

thread_local std::string g_last_error;

constexpr size_t kAlign = 256;
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct RowGroup {
  int max_chunks = 0;
  std::vector<int32_t> ids;
  std::vector<int64_t> prefix;
  size_t off_ids = 0, off_prefix = 0;
};

struct GemmList {
  std::vector<GemmItem> items;
  size_t off = 0;
};

struct NsChunk {
  std::vector<NsDev> ns;          // device pointers filled once base is known
  std::vector<size_t> ws_off;     // per problem: workspace offset (relative to ws base)
  std::vector<TileItem> prep_items;
  GemmList gemm[3][2];            // [op][tile == 256]
  GemmList prod_wide;             // bf16, 128-tile problems: 128 x 256 product tiles
                                  // for the rounds before the last
  GemmList gram_tri;              // bf16 problems with rp == kTriRows: their whole
                                  // Gram in one workgroup (ti, tj unused), largest cp first
  size_t off_ns = 0, off_prep = 0;
  size_t ws_bytes = 0;
};

struct Plan {
  // per parameter
  std::vector<int32_t> table_index;      // index into mats or adams
  std::vector<MatDev> mats;
  std::vector<AdamDev> adams;
  std::vector<size_t> mom_off, part_off, m_off, v_off;
  std::vector<RowGroup> row_groups;
  std::vector<TileItem> col_tiles;
  std::vector<TileItem> col_strips;   // (matrix, 0, column strip) of the tall matrices
  std::vector<TileItem> tall_tiles;   // single-pass tall tiles, strip by strip
  int64_t n_col_tiles_max = 0, n_col_strips_max = 0, n_tall_tiles_max = 0, n_tall_sync_max = 0;
  int32_t n_tall_sync = 0;
  std::vector<AdamChunk> adam_chunks;
  std::vector<NsChunk> ns_full, ns_block;
  size_t off_mats = 0, off_adams = 0, off_col_tiles = 0, off_col_strips = 0, off_adam_chunks = 0;
  size_t off_tall_tiles = 0, off_tall_sync = 0, tall_sync_bytes = 0, tall_list_bytes = 0;
  size_t ws_base = 0, ws_bytes = 0;
  size_t zero_end = 0;                    // bytes [0, zero_end) are zeroed at init
  size_t total = 0;
};

struct Bump {
  size_t cur = 0;
  size_t take(size_t bytes) {
    const size_t o = cur;
    cur = align_up(cur + bytes, kAlign);
    return o;
  }
};

bool finite(float x) { return std::isfinite(x); }

muon_status check_config(const muon_config* c, std::string& err) {
  if (!c) { err = "config is NULL"; return MUON_E_ARG; }
  if (c->K < 1) { err = "K must be >= 1"; return MUON_E_ARG; }
  if (c->ns_iters < 1 || c->ns_iters > 64) { err = "ns_iters must be in [1, 64]"; return MUON_E_ARG; }
  if (!finite(c->lr) || !finite(c->beta) || !finite(c->gamma) || !finite(c->ns_a) ||
      !finite(c->ns_b) || !finite(c->ns_c) || !finite(c->muon_wd) || !finite(c->adam_lr) ||
      !finite(c->adam_wd) || !finite(c->bp_lr_ratio)) {
    err = "non-finite config value"; return MUON_E_ARG;
  }
  if (!(c->eps_row >= 0.f) || !(c->ns_eps >= 0.f) || !(c->adam_eps >= 0.f)) {
    err = "eps values must be >= 0"; return MUON_E_ARG;
  }
  if (c->ns_precision != MUON_NS_BF16 && c->ns_precision != MUON_NS_F32 &&
      c->ns_precision != MUON_NS_BF16_COMP) {
    err = "ns_precision must be MUON_NS_BF16, MUON_NS_F32 or MUON_NS_BF16_COMP"; return MUON_E_ARG;
  }
  if (c->rownorm_axis != 0 && c->rownorm_axis != 1) { err = "rownorm_axis must be 0 or 1"; return MUON_E_ARG; }
  if (c->tall_single_pass != 0 && c->tall_single_pass != 1) { err = "tall_single_pass must be 0 or 1"; return MUON_E_ARG; }
  if (c->reserved0 != 0) { err = "reserved0 must be 0"; return MUON_E_ARG; }
  if (c->bp_blocks < 0) { err = "bp_blocks must be >= 0"; return MUON_E_ARG; }
  if (c->bp_blocks > 0 && c->bp_period < 1) { err = "bp_period must be >= 1"; return MUON_E_ARG; }
  if (!(c->adam_b1 >= 0.f && c->adam_b1 < 1.f) || !(c->adam_b2 >= 0.f && c->adam_b2 < 1.f)) {
    err = "adam betas must be in [0, 1)"; return MUON_E_ARG;
  }
  return MUON_OK;
}

muon_status check_tensor(const muon_tensor& t, bool need_f32, const char* what, int32_t i,
                         std::string& err) {
  char buf[160];
  if (t.rows < 1 || t.cols < 1 || t.ld != t.cols || t.reserved != 0) {
    snprintf(buf, sizeof buf, "%s %d: need rows, cols >= 1, ld == cols, reserved == 0", what, i);
    err = buf;
    return (t.ld != t.cols && t.rows >= 1 && t.cols >= 1) ? MUON_E_ALIGN : MUON_E_SHAPE;
  }
  if (t.rows > (int64_t(1) << 40) / t.cols) {
    snprintf(buf, sizeof buf, "%s %d: tensor too large", what, i); err = buf; return MUON_E_SHAPE;
  }
  if (t.dtype != MUON_F32 && t.dtype != MUON_BF16) {
    snprintf(buf, sizeof buf, "%s %d: unknown dtype %d", what, i, t.dtype); err = buf; return MUON_E_DTYPE;
  }
  if (need_f32 && t.dtype != MUON_F32) {
    snprintf(buf, sizeof buf, "%s %d: must be F32", what, i); err = buf; return MUON_E_DTYPE;
  }
  return MUON_OK;
}

muon_status check_ptr(const void* p, const char* what, int32_t i, std::string& err) {
  char buf[128];
  if (!p) { snprintf(buf, sizeof buf, "%s %d: NULL pointer", what, i); err = buf; return MUON_E_ARG; }
  if (reinterpret_cast<uintptr_t>(p) % 16) {
    snprintf(buf, sizeof buf, "%s %d: pointer not 16-byte aligned", what, i); err = buf; return MUON_E_ALIGN;
  }
  return MUON_OK;
}

int row_chunk_class(int64_t cols) {
  if (cols % 4) return 0;
  const int64_t need = ceil_div(cols, kRowChunkElems);
  for (int c : {1, 2, 4, 8, 16, 32})
    if (need <= c) return c;
  return 0;
}

// Reorder a natural-order work list (each problem's tiles consecutive) for
// the hardware's round-robin dispatch of workgroups to its 8 XCDs
// (workgroup i -> XCD i mod 8), so that each XCD gets an equal share of the
// work and neighbouring tiles, which share operand strips, meet in one XCD's
// L2.
//
// When every tile costs the same (the product and polynomial of same-sized
// problems), each XCD takes one contiguous eighth of the list: its ~32
// concurrent tiles then form whole super-blocks.  When costs differ (the
// Gram's K is the long side, from d to 6d), equal counts per XCD would not
// be equal work: each problem's tiles are cut into parts of up to kXcdPart
// consecutive tiles (a small problem stays whole), and the parts, most
// expensive tiles first, go to the least-loaded XCD that still has room
// (split where one fills up).  Every XCD holds exactly n / 8 tiles, the
// first n % 8 one more, so position p of the result goes to XCD p mod 8.
// Each XCD's list is ordered longest tile first (stable): a launch then
// ends on short tiles instead of leaving most CUs idle behind a few long
// ones.
constexpr int64_t kXcdPart = 8;    // tiles: fine enough to balance to about 1%

// part_size: the parts a problem's tiles are cut into when costs differ.
// Larger parts keep more of an XCD's concurrent tiles on shared operand
// strips (a Gram super-block); if they leave the per-XCD costs more than 2%
// apart, the parts are cut to kXcdPart tiles instead.
template <typename T, typename Key, typename Cost>
void xcd_interleave(std::vector<T>& v, Key key, Cost cost, int64_t part_size = kXcdPart) {
  const int64_t n = static_cast<int64_t>(v.size());
  if (n < 16) return;
  bool uniform = true;
  for (const T& t : v) uniform = uniform && cost(t) == cost(v[0]);
  std::vector<std::vector<T>> part(8);
  if (uniform) {
    const int64_t q = n / 8, rem = n % 8;
    for (int64_t x = 0, o = 0; x < 8; ++x) {
      const int64_t take = q + (x < rem ? 1 : 0);
      part[x].assign(v.begin() + o, v.begin() + o + take);
      o += take;
    }
  } else {
    // Parts of up to `ps` consecutive tiles of one problem, most expensive
    // first, each to the least-loaded XCD that still has room (split where
    // one fills up); returns the largest per-XCD cost over the smallest.
    auto assign = [&](int64_t ps) {
      for (auto& pl : part) pl.clear();
      struct Part { int64_t b, e; double c; };
      std::vector<Part> parts;
      for (int64_t b = 0; b < n;) {
        int64_t e = b + 1;
        while (e < n && key(v[e]) == key(v[b])) ++e;
        for (int64_t o = b; o < e; o += ps)
          parts.push_back(Part{o, std::min(e, o + ps), double(cost(v[o]))});
        b = e;
      }
      std::stable_sort(parts.begin(), parts.end(), [](const Part& l, const Part& r) { return l.c > r.c; });
      const int64_t q = n / 8, rem = n % 8;
      double load[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (const Part& pt : parts)
        for (int64_t o = pt.b; o < pt.e;) {
          int best = -1;
          for (int x = 0; x < 8; ++x)
            if (int64_t(part[x].size()) < q + (x < rem ? 1 : 0) && (best < 0 || load[x] < load[best]))
              best = x;
          const int64_t take = std::min(pt.e - o, q + (best < rem ? 1 : 0) - int64_t(part[best].size()));
          part[best].insert(part[best].end(), v.begin() + o, v.begin() + o + take);
          load[best] += double(take) * pt.c;
          o += take;
        }
      return *std::max_element(load, load + 8) / *std::min_element(load, load + 8);
    };
    if (assign(part_size) > 1.02 && part_size > kXcdPart) assign(kXcdPart);
    for (auto& pl : part)
      std::stable_sort(pl.begin(), pl.end(), [&](const T& l, const T& r) { return cost(l) > cost(r); });
  }
  std::vector<T> out;
  out.reserve(v.size());
  for (size_t local = 0; local < part[0].size(); ++local)
    for (int64_t x = 0; x < 8; ++x)
      if (local < part[x].size()) out.push_back(part[x][local]);
  v.swap(out);
}

// One NS problem (a whole matrix or one MuonBP block).
struct Problem {
  int32_t mat;
  int64_t rows, cols, col0, ld;
  float lr;
};

// Column padding of X: the tile, or 256 for bf16 128-tile problems, whose
// products before the last round use 128 x 256 tiles.
int col_tile(int tile, size_t es) { return tile == 128 && es == 2 ? 256 : tile; }

size_t problem_ws_bytes(const Problem& p, int tile, size_t es, bool xlo, int64_t* rp_out,
                        int64_t* cp_out, int32_t* nparts_out) {
  const int64_t r = std::min(p.rows, p.cols), c = std::max(p.rows, p.cols);
  const int ct = col_tile(tile, es);
  const int64_t rp = ceil_div(r, tile) * tile, cp = ceil_div(c, ct) * ct;
  const int32_t nparts = static_cast<int32_t>((rp / kPrepTile) * (cp / kPrepTile));
  *rp_out = rp; *cp_out = cp; *nparts_out = nparts;
  size_t b = 0;
  b += 2 * align_up(size_t(rp) * cp * es, kAlign);      // bf16: x[0], x[1]; fp32: x[0], xt[0]
  if (xlo) b += align_up(size_t(rp) * cp * 2, kAlign);   // bf16 remainder of X
  if (es == 4) b += align_up(size_t(cp) * rp * es, kAlign);   // fp32: xt[1]
  b += 2 * align_up(size_t(rp) * rp * es, kAlign);      // a, b
  b += align_up(size_t(nparts) * 4, kAlign);            // partials
  b += kAlign;                                          // scale
  b += 2 * align_up(size_t(rp) * 4, kAlign);            // adiag, bdiag
  return b;
}

int tile_for(int64_t r) { return r >= 1024 ? 256 : 128; }

constexpr int64_t kSuperRows = 8, kSuperCols = 4;

// Upper-triangle tiles (i <= j) of an nr x nr tile grid, in blocks whose
// tiles share few operand strips (tile (i, j) reads strips i and j): bands of
// kSuperRows tile rows; each band's own triangle (up to 36 tiles on 8
// strips), and its rectangle with each later band in halves of kSuperRows x
// kSuperCols tiles (32 tiles on 12 strips).  Listed column band by column
// band, so that consecutive blocks share strips too.
template <typename Emit> void upper_tiles_banded(int64_t nr, Emit emit) {
  for (int64_t jb = 0; jb < nr; jb += kSuperRows)
    for (int64_t ib = 0; ib <= jb; ib += kSuperRows) {
      const int64_t je = std::min(nr, jb + kSuperRows);
      if (ib == jb) {
        for (int64_t i = ib; i < je; ++i)
          for (int64_t j = i; j < je; ++j) emit(i, j);
        continue;
      }
      for (int64_t jh = jb; jh < je; jh += kSuperCols)
        for (int64_t i = ib; i < ib + kSuperRows; ++i)
          for (int64_t j = jh; j < std::min(je, jh + kSuperCols); ++j) emit(i, j);
    }
}

std::vector<NsChunk> plan_ns(const std::vector<Problem>& probs, const muon_config& cfg) {
  const size_t es = cfg.ns_precision == MUON_NS_F32 ? 4 : 2;
  const bool xlo = cfg.ns_precision == MUON_NS_BF16_COMP;
  std::vector<NsChunk> chunks;
  NsChunk cur;
  // Chunks are filled up to the cap, unless that leaves a last chunk under
  // half the cap: its launches would hold a few CUs for about as long as a
  // full chunk's (the r = 384 Gram runs one workgroup per problem).  Then
  // chunk k ends near k * total / count, the fewest chunks the cap allows
  // (boundaries on the running total, so that per-chunk shortfalls do not
  // add up to an extra chunk).
  const uint64_t cap = cfg.ns_workspace_max;
  size_t total = 0, fill = 0;
  for (const Problem& p : probs) {
    int64_t rp, cp;
    int32_t np;
    const size_t wb = problem_ws_bytes(p, tile_for(std::min(p.rows, p.cols)), es, xlo, &rp, &cp, &np);
    total += wb;
    fill = fill && cap && fill + wb > cap ? wb : fill + wb;
  }
  const bool balance = cap && total > cap && fill < cap / 2;
  const size_t target = balance ? total / size_t((total + cap - 1) / cap) : SIZE_MAX;
  size_t pos = 0;   // bytes of the problems before this one
  for (const Problem& p : probs) {
    int64_t rp, cp;
    int32_t nparts;
    const int64_t r = std::min(p.rows, p.cols);
    const int tile = tile_for(r);
    const size_t wb = problem_ws_bytes(p, tile, es, xlo, &rp, &cp, &nparts);
    if (!cur.ns.empty() && cap &&
        (cur.ws_bytes + wb > cap ||
         (balance && pos + wb / 2 > (chunks.size() + 1) * target))) {
      chunks.push_back(std::move(cur));
      cur = NsChunk();
    }
    pos += wb;
    NsDev d{};
    d.mat = p.mat;
    d.tall = p.rows > p.cols ? 1 : 0;
    d.rows = p.rows; d.cols = p.cols; d.col0 = p.col0; d.ld = p.ld;
    d.r = r; d.c = std::max(p.rows, p.cols); d.rp = rp; d.cp = cp;
    d.nparts = nparts;
    d.lr = p.lr;
    cur.ws_off.push_back(cur.ws_bytes);
    cur.ws_bytes += wb;
    cur.ns.push_back(d);
  }
  if (!cur.ns.empty()) chunks.push_back(std::move(cur));

  for (NsChunk& ch : chunks) {
    for (int32_t k = 0; k < static_cast<int32_t>(ch.ns.size()); ++k) {
      const NsDev& d = ch.ns[k];
      const int tile = tile_for(d.r);
      const int t256 = tile == 256 ? 1 : 0;
      // prep tiles over the padded stored block; tile (a, b) owns partial
      // a * (stored padded cols / 64) + b
      const int64_t sp = d.tall ? d.cp : d.rp, sq = d.tall ? d.rp : d.cp;
      for (int64_t a = 0; a < sp / kPrepTile; ++a)
        for (int64_t b = 0; b < sq / kPrepTile; ++b)
          ch.prep_items.push_back(TileItem{k, int16_t(a), int16_t(b)});
      const int64_t nr = d.rp / tile, nc = d.cp / tile;
      const bool tri = es == 2 && d.rp == kTriRows;
      if (tri) ch.gram_tri.items.push_back(GemmItem{k, 0, 0});
      // Polynomial: upper tiles in banded blocks.  Its tiles all cost the
      // same when the problems do, so each XCD's contiguous share runs in
      // step and its concurrent tiles share strips in its L2.
      upper_tiles_banded(nr, [&](int64_t i, int64_t j) {
        ch.gemm[kGemmPoly][t256].items.push_back(GemmItem{k, int16_t(i), int16_t(j)});
      });
      // Gram: upper tiles in 4 x 4 super-blocks, each one XCD part below
      // (its up to 16 tiles read 8 strips of X where single rows of tiles
      // would read 17), so an XCD's concurrent tiles share strips in its L2.
      if (!tri)
        for (int64_t jb = 0; jb < nr; jb += 4)
          for (int64_t ib = 0; ib < std::min(nr, jb + 4); ib += 4)
            for (int64_t i = ib; i < std::min(nr, ib + 4); ++i)
              for (int64_t j = std::max(jb, i); j < std::min(nr, jb + 4); ++j)
                ch.gemm[kGemmGram][t256].items.push_back(GemmItem{k, int16_t(i), int16_t(j)});
      // Product tiles in super-blocks of kSuperRows x kSuperCols tiles: the
      // ~32 tiles one XCD runs at a time then share a few B and X panels in
      // its L2 instead of streaming one B panel against 32 X panels.
      for (int64_t jb = 0; jb < nc; jb += kSuperCols)
        for (int64_t ib = 0; ib < nr; ib += kSuperRows)
          for (int64_t i = ib; i < std::min(nr, ib + kSuperRows); ++i)
            for (int64_t j = jb; j < std::min(nc, jb + kSuperCols); ++j)
              ch.gemm[kGemmProduct][t256].items.push_back(GemmItem{k, int16_t(i), int16_t(j)});
      if (col_tile(tile, es) != tile) {
        const int64_t ncw = d.cp / col_tile(tile, es);
        for (int64_t jb = 0; jb < ncw; jb += kSuperCols)
          for (int64_t ib = 0; ib < nr; ib += kSuperRows)
            for (int64_t i = ib; i < std::min(nr, ib + kSuperRows); ++i)
              for (int64_t j = jb; j < std::min(ncw, jb + kSuperCols); ++j)
                ch.prod_wide.items.push_back(GemmItem{k, int16_t(i), int16_t(j)});
      }
    }
    // A tile costs its K: cp for the Gram, rp for the polynomial and product.
    // Gram parts are whole super-blocks when that keeps the XCDs balanced.
    const auto prob = [](const GemmItem& g) { return g.ns; };
    for (int op = 0; op < 3; ++op)
      for (auto& gl : ch.gemm[op])
        xcd_interleave(gl.items, prob, [&](const GemmItem& g) {
          return op == kGemmGram ? ch.ns[g.ns].cp : ch.ns[g.ns].rp;
        }, op == kGemmGram ? 16 : kXcdPart);
    xcd_interleave(ch.prod_wide.items, prob, [&](const GemmItem& g) { return ch.ns[g.ns].rp; });
    // One workgroup per problem, each as long as its cp: longest first, so
    // that the ones handed out last are short.
    std::stable_sort(ch.gram_tri.items.begin(), ch.gram_tri.items.end(),
                     [&](const GemmItem& x, const GemmItem& y) { return ch.ns[x.ns].cp > ch.ns[y.ns].cp; });
  }
  return chunks;
}

// tall_limit: the largest number of row chunks (kTallRows each) a tall
// matrix may have to take the single-pass RowNorm kernel, set by how many of
// its workgroups the device holds at once.  Table and buffer sizes are
// reserved for every eligible matrix either way, so the state size does not
// depend on it.
//
// ext_mom: when given (the no-alloc entry point), the momentum of matrix i is
// the caller's ext_mom[i] instead of a region of the buffer.
muon_status build_plan(const muon_config& cfg, const muon_tensor* params, const int32_t* kinds,
                       int32_t n, char* base, Plan& pl, std::string& err,
                       int64_t tall_limit = kTallMaxChunks,
                       const muon_tensor* ext_mom = nullptr) {
  pl = Plan();
  Bump bump;
  pl.table_index.assign(n, -1);
  pl.mom_off.assign(n, 0); pl.part_off.assign(n, 0); pl.m_off.assign(n, 0); pl.v_off.assign(n, 0);
  // 1. optimizer state (zeroed at init)
  for (int32_t i = 0; i < n; ++i) {
    const muon_tensor& t = params[i];
    const size_t numel = size_t(t.rows) * size_t(t.cols);
    if (kinds[i] == MUON_KIND_MATRIX) {
      pl.table_index[i] = static_cast<int32_t>(pl.mats.size());
      if (!ext_mom) pl.mom_off[i] = bump.take(numel * 4);
      MatDev d{};
      d.rows = t.rows; d.cols = t.cols;
      pl.mats.push_back(d);
    } else {
      pl.table_index[i] = static_cast<int32_t>(pl.adams.size());
      pl.m_off[i] = bump.take(numel * 4);
      pl.v_off[i] = bump.take(numel * 4);
      AdamDev a{};
      a.numel = int64_t(numel);
      pl.adams.push_back(a);
    }
  }
  // 2. RowNorm plan (its partial rows are zeroed at init with the state, so
  //    no launch ever reads a value no kernel wrote)
  const bool cols_mode = cfg.rownorm_axis == 0;
  std::vector<RowGroup> groups(7);
  const int classes[7] = {0, 1, 2, 4, 8, 16, 32};
  for (int g = 0; g < 7; ++g) groups[g].max_chunks = classes[g];
  for (int32_t i = 0; i < n; ++i) {
    if (kinds[i] != MUON_KIND_MATRIX) continue;
    const muon_tensor& t = params[i];
    const int32_t mi = pl.table_index[i];
    if (cols_mode && t.rows > t.cols) {
      const int64_t nchunk = ceil_div(t.rows, kColTileRows);
      const int64_t nstrip = ceil_div(t.cols, kColTileCols);
      if (nchunk > 32767 || nstrip > 32767) {
        err = "param " + std::to_string(i) + ": too large for the tile index range";
        return MUON_E_SHAPE;
      }
      const int64_t tchunk = ceil_div(t.rows, kTallRows);
      const int64_t tstrip = ceil_div(t.cols, kTallCols);
      const bool eligible = cfg.tall_single_pass != 0 && t.cols % 2 == 0 && tchunk <= kTallMaxChunks;
      // single pass: per strip, tchunk partial rows and a coefficient row of
      // kTallCols floats each (no cache line shared between strips)
      pl.part_off[i] = bump.take(std::max(eligible ? size_t(tchunk + 1) * tstrip * kTallCols * 4 : 0,
                                          size_t(nchunk) * t.cols * 4));
      pl.n_col_tiles_max += nchunk * nstrip;
      pl.n_col_strips_max += nstrip;
      if (eligible) {
        pl.n_tall_tiles_max += tchunk * tstrip;
        pl.n_tall_sync_max += tstrip;
      }
      if (eligible && tchunk <= tall_limit) {
        pl.mats[mi].sync0 = pl.n_tall_sync;
        pl.n_tall_sync += int32_t(tstrip);
        for (int64_t b = 0; b < tstrip; ++b)
          for (int64_t a = 0; a < tchunk; ++a)
            pl.tall_tiles.push_back(TileItem{mi, int16_t(a), int16_t(b)});
      } else {
        for (int64_t a = 0; a < nchunk; ++a)
          for (int64_t b = 0; b < nstrip; ++b)
            pl.col_tiles.push_back(TileItem{mi, int16_t(a), int16_t(b)});
        for (int64_t b = 0; b < nstrip; ++b)
          pl.col_strips.push_back(TileItem{mi, 0, int16_t(b)});
      }
    } else {
      const int cls = row_chunk_class(t.cols);
      RowGroup& g = groups[std::find(classes, classes + 7, cls) - classes];
      if (g.prefix.empty()) g.prefix.push_back(0);
      g.ids.push_back(mi);
      g.prefix.push_back(g.prefix.back() + t.rows);
    }
  }
  pl.zero_end = bump.cur;
  for (RowGroup& g : groups)
    if (!g.ids.empty()) pl.row_groups.push_back(std::move(g));
  // 3. AdamW chunks
  for (int32_t i = 0; i < n; ++i) {
    if (kinds[i] != MUON_KIND_ADAMW) continue;
    const int64_t numel = params[i].rows * params[i].cols;
    for (int64_t o = 0; o < numel; o += kAdamChunk)
      pl.adam_chunks.push_back(AdamChunk{pl.table_index[i],
                                         int32_t(std::min<int64_t>(kAdamChunk, numel - o)), o});
  }
  // 4. NS plans
  std::vector<Problem> full, block;
  for (int32_t i = 0; i < n; ++i) {
    if (kinds[i] != MUON_KIND_MATRIX) continue;
    const muon_tensor& t = params[i];
    full.push_back(Problem{pl.table_index[i], t.rows, t.cols, 0, t.cols, cfg.lr});
    if (cfg.bp_blocks > 0) {
      if (t.cols % cfg.bp_blocks) {
        char buf[160];
        snprintf(buf, sizeof buf, "param %d: %lld columns do not split into %d MuonBP blocks", i,
                 (long long)t.cols, cfg.bp_blocks);
        err = buf;
        return MUON_E_SHAPE;
      }
      const int64_t w = t.cols / cfg.bp_blocks;
      for (int32_t b = 0; b < cfg.bp_blocks; ++b)
        block.push_back(Problem{pl.table_index[i], t.rows, w, b * w, t.cols, cfg.lr * cfg.bp_lr_ratio});
    }
  }
  pl.ns_full = plan_ns(full, cfg);
  pl.ns_block = plan_ns(block, cfg);
  // The GEMM kernels address X (rp x cp) and A, B (rp x rp) through raw
  // buffer descriptors with 32-bit byte sizes and offsets.
  const int64_t ns_es = cfg.ns_precision == MUON_NS_F32 ? 4 : 2;
  for (auto* plan : {&pl.ns_full, &pl.ns_block})
    for (NsChunk& ch : *plan)
      for (const NsDev& d : ch.ns) {
        if (d.rp / 128 > 32767 || d.cp / 64 > 32767) {
          err = "matrix too large for the tile index range"; return MUON_E_SHAPE;
        }
        if (d.rp * d.cp * ns_es >= (int64_t(1) << 32)) {
          err = "matrix too large: its Newton-Schulz workspace copy exceeds 4 GiB";
          return MUON_E_SHAPE;
        }
      }
  // 5. tables
  pl.off_mats = bump.take(pl.mats.size() * sizeof(MatDev));
  pl.off_adams = bump.take(pl.adams.size() * sizeof(AdamDev));
  pl.off_col_tiles = bump.take(size_t(pl.n_col_tiles_max) * sizeof(TileItem));
  pl.off_col_strips = bump.take(size_t(pl.n_col_strips_max) * sizeof(TileItem));
  pl.off_tall_tiles = bump.take(size_t(pl.n_tall_tiles_max) * sizeof(TileItem));
  // the control line, the repair list (one word per tile), then one
  // TallSync per strip
  pl.tall_list_bytes = align_up(size_t(pl.n_tall_tiles_max) * 4, sizeof(TallSync));
  pl.tall_sync_bytes = pl.n_tall_tiles_max ? sizeof(TallCtl) + pl.tall_list_bytes +
                                                 size_t(pl.n_tall_sync_max) * sizeof(TallSync)
                                           : 0;
  pl.off_tall_sync = bump.take(pl.tall_sync_bytes);
  pl.off_adam_chunks = bump.take(pl.adam_chunks.size() * sizeof(AdamChunk));
  for (RowGroup& g : pl.row_groups) {
    g.off_ids = bump.take(g.ids.size() * 4);
    g.off_prefix = bump.take(g.prefix.size() * 8);
  }
  size_t ws = 0;
  for (auto* plan : {&pl.ns_full, &pl.ns_block})
    for (NsChunk& ch : *plan) {
      ch.off_ns = bump.take(ch.ns.size() * sizeof(NsDev));
      ch.off_prep = bump.take(ch.prep_items.size() * sizeof(TileItem));
      for (auto& op : ch.gemm)
        for (auto& gl : op) gl.off = bump.take(gl.items.size() * sizeof(GemmItem));
      ch.prod_wide.off = bump.take(ch.prod_wide.items.size() * sizeof(GemmItem));
      ch.gram_tri.off = bump.take(ch.gram_tri.items.size() * sizeof(GemmItem));
      ws = std::max(ws, ch.ws_bytes);
    }
  // 6. NS workspace, shared by all chunks of both plans
  pl.ws_base = bump.take(ws);
  pl.ws_bytes = ws;
  pl.total = bump.cur;

  // Device pointers (meaningful only when base is the real buffer).
  auto at = [&](size_t off) { return static_cast<void*>(base + off); };
  for (int32_t i = 0; i < n; ++i) {
    const int32_t k = pl.table_index[i];
    if (kinds[i] == MUON_KIND_MATRIX) {
      MatDev& d = pl.mats[k];
      d.mom = ext_mom ? static_cast<float*>(ext_mom[i].ptr) : static_cast<float*>(at(pl.mom_off[i]));
      d.part = static_cast<float*>(at(pl.part_off[i]));
    } else {
      AdamDev& a = pl.adams[k];
      a.m = static_cast<float*>(at(pl.m_off[i]));
      a.v = static_cast<float*>(at(pl.v_off[i]));
    }
  }
  const size_t es = cfg.ns_precision == MUON_NS_F32 ? 4 : 2;
  const bool xlo = cfg.ns_precision == MUON_NS_BF16_COMP;
  for (auto* plan : {&pl.ns_full, &pl.ns_block})
    for (NsChunk& ch : *plan)
      for (size_t k = 0; k < ch.ns.size(); ++k) {
        NsDev& d = ch.ns[k];
        size_t o = pl.ws_base + ch.ws_off[k];
        const size_t xb = align_up(size_t(d.rp) * d.cp * es, kAlign);
        if (es == 2) {
          d.x[0] = at(o); o += xb;
          d.x[1] = at(o); o += xb;
          d.xt[0] = d.xt[1] = nullptr;
          d.xlo = nullptr;
          if (xlo) { d.xlo = at(o); o += xb; }
        } else {
          d.x[0] = at(o); o += xb;
          d.x[1] = nullptr;
          d.xt[0] = at(o); o += xb;
          d.xt[1] = at(o); o += xb;
          d.xlo = nullptr;
        }
        d.a = at(o); o += align_up(size_t(d.rp) * d.rp * es, kAlign);
        d.b = at(o); o += align_up(size_t(d.rp) * d.rp * es, kAlign);
        d.part = static_cast<float*>(at(o)); o += align_up(size_t(d.nparts) * 4, kAlign);
        d.scale = static_cast<float*>(at(o)); o += kAlign;
        d.adiag = static_cast<float*>(at(o)); o += align_up(size_t(d.rp) * 4, kAlign);
        d.bdiag = static_cast<float*>(at(o));
      }
  return MUON_OK;
}

muon_status validate_list(const muon_config* cfg, const muon_tensor* params,
                          const muon_tensor* grads, const int32_t* kinds, int32_t n,
                          bool check_ptrs, std::string& err) {
  muon_status st = check_config(cfg, err);
  if (st != MUON_OK) return st;
  if (n < 0) { err = "n must be >= 0"; return MUON_E_ARG; }
  if (n > 0 && (!params || !kinds)) { err = "params/kinds is NULL"; return MUON_E_ARG; }
  if (n > 0 && check_ptrs && !grads) { err = "grads is NULL"; return MUON_E_ARG; }
  for (int32_t i = 0; i < n; ++i) {
    if (kinds[i] != MUON_KIND_MATRIX && kinds[i] != MUON_KIND_ADAMW) {
      err = "param " + std::to_string(i) + ": unknown kind";
      return MUON_E_ARG;
    }
    st = check_tensor(params[i], true, "param", i, err);
    if (st != MUON_OK) return st;
    if (check_ptrs) {
      st = check_tensor(grads[i], false, "grad", i, err);
      if (st != MUON_OK) return st;
      if (grads[i].rows != params[i].rows || grads[i].cols != params[i].cols) {
        err = "grad " + std::to_string(i) + ": shape differs from its param";
        return MUON_E_SHAPE;
      }
      if ((st = check_ptr(params[i].ptr, "param", i, err)) != MUON_OK) return st;
      if ((st = check_ptr(grads[i].ptr, "grad", i, err)) != MUON_OK) return st;
    }
  }
  return MUON_OK;
}

}  // namespace

struct muon_ctx {
  muon_config cfg{};
  hipStream_t stream = nullptr;
  int device = 0;
  char* base = nullptr;
  int32_t n = 0;
  std::vector<muon_tensor> params, grads;  // init-time descriptors + current pointers
  std::vector<int32_t> kinds;
  Plan plan;
  std::string err;
  bool broken = false;
  uint32_t poll_limit = kTallPollLimit;   // single-pass tall RowNorm waits
  // measurement hook
  bool timing = false;
  std::vector<hipEvent_t> events;            // pool, two per recorded launch
  std::vector<int32_t> event_class;          // class of each recorded pair
  size_t events_used = 0;                    // pairs recorded since last read
  ~muon_ctx() {
    for (hipEvent_t e : events) (void)hipEventDestroy(e);
  }
};

namespace {

muon_status hip_fail(muon_ctx* ctx, hipError_t e, const char* what) {
  char buf[256];
  snprintf(buf, sizeof buf, "%s: %s", what, hipGetErrorString(e));
  ctx->err = buf;
  return MUON_E_HIP;
}

template <typename T>
hipError_t upload(hipStream_t s, char* base, size_t off, const std::vector<T>& v) {
  if (v.empty()) return hipSuccess;
  return hipMemcpyAsync(base + off, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice, s);
}

// Enqueue the copies of every launch table of pl to base + its offsets.  The
// host vectors must stay alive until the stream has passed the copies.
hipError_t upload_plan(hipStream_t s, char* base, const Plan& pl, const char** what) {
  *what = "hipMemcpyAsync(tables)";
  hipError_t e = hipSuccess;
  auto up = [&](size_t off, const auto& v) {
    if (e == hipSuccess) e = upload(s, base, off, v);
  };
  up(pl.off_mats, pl.mats);
  up(pl.off_adams, pl.adams);
  up(pl.off_col_tiles, pl.col_tiles);
  up(pl.off_col_strips, pl.col_strips);
  up(pl.off_tall_tiles, pl.tall_tiles);
  up(pl.off_adam_chunks, pl.adam_chunks);
  for (const RowGroup& g : pl.row_groups) {
    up(g.off_ids, g.ids);
    up(g.off_prefix, g.prefix);
  }
  for (const auto* plan : {&pl.ns_full, &pl.ns_block})
    for (const NsChunk& ch : *plan) {
      up(ch.off_ns, ch.ns);
      up(ch.off_prep, ch.prep_items);
      for (const auto& op : ch.gemm)
        for (const auto& gl : op) up(gl.off, gl.items);
      up(ch.prod_wide.off, ch.prod_wide.items);
      up(ch.gram_tri.off, ch.gram_tri.items);
    }
  return e;
}

// Records a start event for kernel class cls when timing is on; close()
// records the stop event after the launch.
struct Timed {
  muon_ctx* ctx;
  size_t pair = SIZE_MAX;
  Timed(muon_ctx* c, int32_t cls) : ctx(c) {
    if (!ctx->timing) return;
    if (ctx->events.size() < 2 * (ctx->events_used + 1)) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess) return;
      if (hipEventCreate(&b) != hipSuccess) { (void)hipEventDestroy(a); return; }
      ctx->events.push_back(a);
      ctx->events.push_back(b);
      ctx->event_class.push_back(cls);
    }
    pair = ctx->events_used++;
    ctx->event_class[pair] = cls;
    (void)hipEventRecord(ctx->events[2 * pair], ctx->stream);
  }
  hipError_t close(hipError_t e) {
    if (pair != SIZE_MAX) (void)hipEventRecord(ctx->events[2 * pair + 1], ctx->stream);
    return e;
  }
};

#define MUON_TIMED(ctx, cls, expr) Timed((ctx), (cls)).close(expr)

#define MUON_HIP(ctx, expr)                                   \
  do {                                                        \
    const hipError_t e_ = (expr);                             \
    if (e_ != hipSuccess) return hip_fail((ctx), e_, #expr);  \
  } while (0)

muon_status run_ns(muon_ctx* ctx, std::vector<NsChunk>& chunks) {
  const muon_config& c = ctx->cfg;
  const Plan& pl = ctx->plan;
  const MatDev* mats = reinterpret_cast<const MatDev*>(ctx->base + pl.off_mats);
  const int prec = c.ns_precision;   // 0 bf16, 1 fp32, 2 bf16 with X's remainder
  for (NsChunk& ch : chunks) {
    NsDev* ns = reinterpret_cast<NsDev*>(ctx->base + ch.off_ns);
    const TileItem* prep = reinterpret_cast<const TileItem*>(ctx->base + ch.off_prep);
    MUON_HIP(ctx, MUON_TIMED(ctx, MUON_K_NS_PREP,
                             launch_ns_prep(ctx->stream, mats, ns, prep,
                                            int64_t(ch.prep_items.size()), prec, c.beta)));
    MUON_HIP(ctx, MUON_TIMED(ctx, MUON_K_NS_SCALE,
                             launch_ns_scale(ctx->stream, ns, int32_t(ch.ns.size()), c.ns_eps)));
    for (int it = 0; it < c.ns_iters; ++it) {
      const int last = it == c.ns_iters - 1;
      for (int op = 0; op < 3; ++op) {
        if (op == kGemmGram && !ch.gram_tri.items.empty()) {
          const GemmItem* items = reinterpret_cast<const GemmItem*>(ctx->base + ch.gram_tri.off);
          MUON_HIP(ctx, MUON_TIMED(ctx, MUON_K_NS_GRAM,
                                   launch_ns_gram_tri(ctx->stream, ns, items,
                                                      int64_t(ch.gram_tri.items.size()), it)));
        }
        for (int t = 0; t < 2; ++t) {
          // before the last round, bf16 128-tile products run on 128 x 256 tiles
          const bool wide = op == kGemmProduct && t == 0 && !last && !ch.prod_wide.items.empty();
          const GemmList& gl = wide ? ch.prod_wide : ch.gemm[op][t];
          if (gl.items.empty()) continue;
          const GemmItem* items = reinterpret_cast<const GemmItem*>(ctx->base + gl.off);
          MUON_HIP(ctx, MUON_TIMED(ctx, op == 2 && last ? MUON_K_NS_PRODUCT_LAST : MUON_K_NS_GRAM + op,
                                   launch_ns_gemm(ctx->stream, mats, ns, items,
                                                  int64_t(gl.items.size()), op, t ? 256 : 128,
                                                  wide ? 256 : (t ? 256 : 128), prec, it, last, c.ns_a, c.ns_b, c.ns_c,
                                                  c.muon_wd)));
        }
      }
    }
  }
  return MUON_OK;
}

// The caller's weights and gradients in the plan's tables (build_plan fills
// everything else).
void bind_tensors(Plan& pl, const muon_tensor* params, const muon_tensor* grads,
                  const int32_t* kinds, int32_t n) {
  for (int32_t i = 0; i < n; ++i) {
    const int32_t k = pl.table_index[i];
    if (kinds[i] == MUON_KIND_MATRIX) {
      pl.mats[k].w = static_cast<float*>(params[i].ptr);
      pl.mats[k].g = grads[i].ptr;
      pl.mats[k].gdt = grads[i].dtype;
    } else {
      pl.adams[k].p = static_cast<float*>(params[i].ptr);
      pl.adams[k].g = grads[i].ptr;
      pl.adams[k].gdt = grads[i].dtype;
    }
  }
}

// The single-pass tall RowNorm kernel needs every workgroup of a column
// strip resident at once; strips of up to half the current device's
// capacity (so up to half of each XCD's, as a strip's workgroups are dealt
// round-robin to the XCDs) take it, the rest the two-pass kernels.  0 when
// the device cannot be queried.
int64_t device_tall_limit() {
  int dev = 0, cus = 0, per_cu = 0;
  int64_t lim = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      rownorm_tall_resident(&per_cu) == hipSuccess)
    lim = std::min<int64_t>(kTallMaxChunks, int64_t(cus) * per_cu / 2);
  (void)hipGetLastError();
  return lim;
}

// The launches of one step t on ctx's stream, from its plan: the branch's
// kernels over every matrix, then AdamW over the other tensors.
muon_status enqueue_step(muon_ctx* ctx, int64_t step) {
  Plan& pl = ctx->plan;
  // Host copies of the tables: every tensor pointer must be bound before a
  // kernel may use it.
  for (const MatDev& d : pl.mats)
    if (!d.w || !d.g || !d.mom) { ctx->err = "internal: unbound matrix tensor"; return MUON_E_STATE; }
  for (const AdamDev& a : pl.adams)
    if (!a.p || !a.g) { ctx->err = "internal: unbound AdamW tensor"; return MUON_E_STATE; }
  MatDev* mats = reinterpret_cast<MatDev*>(ctx->base + pl.off_mats);
  AdamDev* adams = reinterpret_cast<AdamDev*>(ctx->base + pl.off_adams);
  const muon_config& c = ctx->cfg;
  const int32_t br = muon_branch(&c, step);
  muon_status st = MUON_OK;
  if (!pl.mats.empty()) {
    if (br == MUON_BRANCH_ROWNORM) {
      StepScalars sc{c.lr, c.beta, c.gamma, c.eps_row, c.muon_wd};
      for (RowGroup& g : pl.row_groups) {
        const hipError_t e = MUON_TIMED(ctx, MUON_K_ROWNORM_ROWS, launch_rownorm_rows(
            ctx->stream, mats, reinterpret_cast<const int32_t*>(ctx->base + g.off_ids),
            reinterpret_cast<const int64_t*>(ctx->base + g.off_prefix), int32_t(g.ids.size()),
            g.prefix.back(), g.max_chunks, sc));
        if (e != hipSuccess) { ctx->broken = true; return hip_fail(ctx, e, "rownorm_rows"); }
      }
      if (!pl.tall_tiles.empty()) {
        char* tb = ctx->base + pl.off_tall_sync;
        TallCtl* ctl = reinterpret_cast<TallCtl*>(tb);
        uint32_t* list = reinterpret_cast<uint32_t*>(tb + sizeof(TallCtl));
        TallSync* sync = reinterpret_cast<TallSync*>(tb + sizeof(TallCtl) + pl.tall_list_bytes);
        const TileItem* tt = reinterpret_cast<const TileItem*>(ctx->base + pl.off_tall_tiles);
        const int64_t nt = int64_t(pl.tall_tiles.size());
        hipError_t e = MUON_TIMED(ctx, MUON_K_ROWNORM_TALL, launch_rownorm_tall(
            ctx->stream, mats, tt, nt, sync, ctl, list, ctx->poll_limit, sc));
        if (e != hipSuccess) { ctx->broken = true; return hip_fail(ctx, e, "rownorm_tall"); }
        e = MUON_TIMED(ctx, MUON_K_ROWNORM_REPAIR,
                       launch_rownorm_repair(ctx->stream, mats, tt, nt, ctl, list, sc));
        if (e != hipSuccess) { ctx->broken = true; return hip_fail(ctx, e, "rownorm_repair"); }
      }
      const TileItem* tiles = reinterpret_cast<const TileItem*>(ctx->base + pl.off_col_tiles);
      const TileItem* strips = reinterpret_cast<const TileItem*>(ctx->base + pl.off_col_strips);
      for (int phase = 1; phase <= 2 && !pl.col_tiles.empty(); ++phase) {
        if (phase == 2) {
          const hipError_t e = MUON_TIMED(ctx, MUON_K_ROWNORM_COEF,
                                          launch_rownorm_coef(ctx->stream, mats, strips,
                                                              int64_t(pl.col_strips.size()), sc));
          if (e != hipSuccess) { ctx->broken = true; return hip_fail(ctx, e, "rownorm_coef"); }
        }
        const hipError_t e = MUON_TIMED(ctx, MUON_K_ROWNORM_COLS1 + phase - 1,
                                        launch_rownorm_cols(ctx->stream, mats, tiles,
                                                            int64_t(pl.col_tiles.size()), phase, sc));
        if (e != hipSuccess) { ctx->broken = true; return hip_fail(ctx, e, "rownorm_cols"); }
      }
    } else {
      st = run_ns(ctx, br == MUON_BRANCH_NS5 ? pl.ns_full : pl.ns_block);
      if (st != MUON_OK) { ctx->broken = true; return st; }
    }
  }
  if (!pl.adams.empty()) {
    const double n1 = double(step) + 1.0;
    const float bc1 = float(1.0 - std::pow(double(c.adam_b1), n1));
    const float bc2 = float(1.0 - std::pow(double(c.adam_b2), n1));
    const hipError_t e = MUON_TIMED(ctx, MUON_K_ADAMW, launch_adamw(
        ctx->stream, adams, reinterpret_cast<const AdamChunk*>(ctx->base + pl.off_adam_chunks),
        int64_t(pl.adam_chunks.size()), c.adam_lr, c.adam_b1, c.adam_b2, c.adam_eps, c.adam_wd,
        bc1, bc2));
    if (e != hipSuccess) { ctx->broken = true; return hip_fail(ctx, e, "adamw"); }
  }
  return MUON_OK;
}

}  // namespace

extern "C" {

muon_status muon_config_default(muon_config* out) {
  if (!out) return MUON_E_ARG;
  std::memset(out, 0, sizeof *out);
  out->lr = 0.02f;
  out->beta = 0.95f;
  out->gamma = 0.15f;
  out->eps_row = 1e-8f;
  out->K = 3;
  out->ns_iters = 5;
  out->ns_a = 3.4445f;
  out->ns_b = -4.7750f;
  out->ns_c = 2.0315f;
  out->ns_eps = 1e-7f;
  out->ns_precision = MUON_NS_BF16;
  out->rownorm_axis = 0;
  out->bp_blocks = 0;
  out->bp_period = 3;
  out->bp_lr_ratio = 0.5f;
  out->muon_wd = 0.f;
  out->adam_lr = 1e-3f;
  out->adam_b1 = 0.9f;
  out->adam_b2 = 0.999f;
  out->adam_eps = 1e-8f;
  out->adam_wd = 0.f;
  out->ns_workspace_max = uint64_t(16) << 30;
  out->tall_single_pass = 1;
  return MUON_OK;
}

muon_status muon_state_bytes(const muon_config* cfg, const muon_tensor* params,
                             const int32_t* kinds, int32_t n, size_t* bytes) {
  std::string err;
  if (!bytes) { g_last_error = "bytes is NULL"; return MUON_E_ARG; }
  muon_status st = validate_list(cfg, params, nullptr, kinds, n, false, err);
  if (st != MUON_OK) { g_last_error = err; return st; }
  Plan pl;
  st = build_plan(*cfg, params, kinds, n, nullptr, pl, err);
  if (st != MUON_OK) { g_last_error = err; return st; }
  *bytes = pl.total;
  return MUON_OK;
}

muon_status muon_init(muon_ctx** out, const muon_config* cfg, const muon_tensor* params,
                      const muon_tensor* grads, const int32_t* kinds, int32_t n, void* state_buf,
                      size_t state_bytes, void* hip_stream) {
  std::string err;
  if (!out) { g_last_error = "out is NULL"; return MUON_E_ARG; }
  *out = nullptr;
  muon_status st = validate_list(cfg, params, grads, kinds, n, true, err);
  if (st != MUON_OK) { g_last_error = err; return st; }
  Plan probe;
  st = build_plan(*cfg, params, kinds, n, nullptr, probe, err);
  if (st != MUON_OK) { g_last_error = err; return st; }
  if (probe.total > 0 && (!state_buf || reinterpret_cast<uintptr_t>(state_buf) % kAlign)) {
    g_last_error = "state buffer is NULL or not 256-byte aligned";
    return state_buf ? MUON_E_ALIGN : MUON_E_WORKSPACE;
  }
  if (state_bytes < probe.total) {
    g_last_error = "state buffer too small: need " + std::to_string(probe.total) + " bytes";
    return MUON_E_WORKSPACE;
  }
  muon_ctx* ctx = new (std::nothrow) muon_ctx();
  if (!ctx) { g_last_error = "out of host memory"; return MUON_E_STATE; }
  ctx->cfg = *cfg;
  ctx->stream = static_cast<hipStream_t>(hip_stream);
  ctx->base = static_cast<char*>(state_buf);
  ctx->n = n;
  ctx->params.assign(params, params + n);
  ctx->grads.assign(grads, grads + n);
  ctx->kinds.assign(kinds, kinds + n);
  const int64_t tall_limit = probe.n_tall_tiles_max > 0 ? device_tall_limit() : 0;
  build_plan(*cfg, params, kinds, n, ctx->base, ctx->plan, err, tall_limit);
  Plan& pl = ctx->plan;
  bind_tensors(pl, params, grads, kinds, n);
  hipError_t e = hipGetDevice(&ctx->device);
  if (e == hipSuccess && pl.zero_end) e = hipMemsetAsync(ctx->base, 0, pl.zero_end, ctx->stream);
  if (e == hipSuccess && pl.tall_sync_bytes)
    e = hipMemsetAsync(ctx->base + pl.off_tall_sync, 0, pl.tall_sync_bytes, ctx->stream);
  const char* what = "muon_init: zeroing the state";
  if (e == hipSuccess) e = upload_plan(ctx->stream, ctx->base, pl, &what);
  // The host copies of the tables must outlive the transfers.
  if (e == hipSuccess) e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) {
    char buf[256];
    snprintf(buf, sizeof buf, "%s: %s", what, hipGetErrorString(e));
    g_last_error = buf;
    delete ctx;
    return MUON_E_HIP;
  }
  *out = ctx;
  return MUON_OK;
}

muon_status muon_step(muon_ctx* ctx, const muon_tensor* params, const muon_tensor* grads,
                      int64_t step) {
  if (!ctx) return MUON_E_ARG;
  if (ctx->broken) { ctx->err = "context unusable after an earlier HIP failure"; return MUON_E_STATE; }
  if (step < 0) { ctx->err = "step must be >= 0"; return MUON_E_ARG; }
  if (ctx->n > 0 && (!params || !grads)) { ctx->err = "params/grads is NULL"; return MUON_E_ARG; }
  // validate everything before enqueueing anything
  for (int32_t i = 0; i < ctx->n; ++i) {
    const muon_tensor &p = params[i], &g = grads[i];
    const muon_tensor &p0 = ctx->params[i], &g0 = ctx->grads[i];
    std::string err;
    muon_status st;
    if ((st = check_ptr(p.ptr, "param", i, err)) != MUON_OK ||
        (st = check_ptr(g.ptr, "grad", i, err)) != MUON_OK) {
      ctx->err = err;
      return st;
    }
    if (p.rows != p0.rows || p.cols != p0.cols || g.rows != g0.rows || g.cols != g0.cols) {
      ctx->err = "tensor " + std::to_string(i) + ": shape differs from the init-time plan";
      return MUON_E_SHAPE;
    }
    if (p.ld != p.cols || g.ld != g.cols) {
      ctx->err = "tensor " + std::to_string(i) + ": ld must equal cols";
      return MUON_E_ALIGN;
    }
    if (p.dtype != p0.dtype || g.dtype != g0.dtype) {
      ctx->err = "tensor " + std::to_string(i) + ": dtype differs from the init-time plan";
      return MUON_E_DTYPE;
    }
  }
  Plan& pl = ctx->plan;
  MatDev* mats = reinterpret_cast<MatDev*>(ctx->base + pl.off_mats);
  AdamDev* adams = reinterpret_cast<AdamDev*>(ctx->base + pl.off_adams);
  // patch moved pointers
  PatchArgs pa[2]{};
  pa[1].adam = 1;
  for (int32_t i = 0; i < ctx->n; ++i) {
    if (params[i].ptr == ctx->params[i].ptr && grads[i].ptr == ctx->grads[i].ptr) continue;
    PatchArgs& a = pa[ctx->kinds[i] == MUON_KIND_ADAMW ? 1 : 0];
    a.idx[a.count] = ctx->plan.table_index[i];
    a.w[a.count] = params[i].ptr;
    a.g[a.count] = grads[i].ptr;
    ++a.count;
    ctx->params[i].ptr = params[i].ptr;
    ctx->grads[i].ptr = grads[i].ptr;
    if (a.count == kPatchMax) {
      const hipError_t e = launch_patch(ctx->stream, mats, adams, a);
      if (e != hipSuccess) { ctx->broken = true; return hip_fail(ctx, e, "patch"); }
      a.count = 0;
    }
  }
  for (PatchArgs& a : pa) {
    const hipError_t e = launch_patch(ctx->stream, mats, adams, a);
    if (e != hipSuccess) { ctx->broken = true; return hip_fail(ctx, e, "patch"); }
  }

  return enqueue_step(ctx, step);
}

muon_status muon_state(const muon_ctx* ctx, int32_t i, int32_t which, muon_tensor* view) {
  if (!ctx || !view) return MUON_E_ARG;
  if (i < 0 || i >= ctx->n) return MUON_E_STATE;
  const bool adam = ctx->kinds[i] == MUON_KIND_ADAMW;
  if (which < 0 || which > (adam ? 1 : 0)) return MUON_E_ARG;
  const Plan& pl = ctx->plan;
  const size_t off = adam ? (which ? pl.v_off[i] : pl.m_off[i]) : pl.mom_off[i];
  view->ptr = ctx->base + off;
  view->rows = ctx->params[i].rows;
  view->cols = ctx->params[i].cols;
  view->ld = view->cols;
  view->dtype = MUON_F32;
  view->reserved = 0;
  return MUON_OK;
}

int32_t muon_branch(const muon_config* cfg, int64_t step) {
  if (!cfg || step < 0) return -1;
  if (cfg->bp_blocks > 0) {
    if (cfg->bp_period < 1) return -1;
    return step % cfg->bp_period == 0 ? MUON_BRANCH_NS5 : MUON_BRANCH_BLOCK_NS5;
  }
  if (cfg->K < 1) return -1;
  return step % cfg->K == 0 ? MUON_BRANCH_NS5 : MUON_BRANCH_ROWNORM;
}

muon_status muon_timing_enable(muon_ctx* ctx, int32_t enable) {
  if (!ctx) return MUON_E_ARG;
  ctx->timing = enable != 0;
  return MUON_OK;
}

muon_status muon_timing_read(muon_ctx* ctx, double* ms, int64_t* launches) {
  if (!ctx) return MUON_E_ARG;
  double acc[MUON_K_COUNT] = {0};
  int64_t cnt[MUON_K_COUNT] = {0};
  for (size_t p = 0; p < ctx->events_used; ++p) {
    hipError_t e = hipEventSynchronize(ctx->events[2 * p + 1]);
    float dt = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&dt, ctx->events[2 * p], ctx->events[2 * p + 1]);
    if (e != hipSuccess) {
      ctx->events_used = 0;
      return hip_fail(ctx, e, "muon_timing_read");
    }
    const int32_t k = ctx->event_class[p];
    acc[k] += dt;
    cnt[k] += 1;
  }
  ctx->events_used = 0;
  for (int k = 0; k < MUON_K_COUNT; ++k) {
    if (ms) ms[k] = acc[k];
    if (launches) launches[k] = cnt[k];
  }
  return MUON_OK;
}

muon_status muon_sync(muon_ctx* ctx) {
  if (!ctx) return MUON_E_ARG;
  const hipError_t e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) { ctx->broken = true; return hip_fail(ctx, e, "muon_sync"); }
  return MUON_OK;
}

muon_status muon_tall_poll_limit(muon_ctx* ctx, uint32_t polls) {
  if (!ctx) return MUON_E_ARG;
  ctx->poll_limit = polls;
  return MUON_OK;
}

muon_status muon_tall_giveups(muon_ctx* ctx, uint64_t* count) {
  if (!ctx || !count) return MUON_E_ARG;
  *count = 0;
  hipError_t e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) { ctx->broken = true; return hip_fail(ctx, e, "muon_tall_giveups"); }
  const Plan& pl = ctx->plan;
  if (!pl.tall_sync_bytes) return MUON_OK;
  TallCtl ctl{};
  e = hipMemcpy(&ctl, ctx->base + pl.off_tall_sync, sizeof ctl, hipMemcpyDeviceToHost);
  if (e != hipSuccess) { ctx->broken = true; return hip_fail(ctx, e, "muon_tall_giveups"); }
  *count = ctl.giveups;
  return MUON_OK;
}

muon_status muon_step_noalloc(const muon_config* cfg, const muon_tensor* params,
                              const muon_tensor* grads, const muon_tensor* moms, int32_t n,
                              int64_t step, void* hip_stream) {
  std::string err;
  if (step < 0) { g_last_error = "step must be >= 0"; return MUON_E_ARG; }
  if (n > 0 && !moms) { g_last_error = "moms is NULL"; return MUON_E_ARG; }
  std::vector<int32_t> kinds(size_t(std::max(n, 0)), MUON_KIND_MATRIX);
  muon_status st = validate_list(cfg, params, grads, kinds.data(), n, true, err);
  if (st != MUON_OK) { g_last_error = err; return st; }
  for (int32_t i = 0; i < n; ++i) {
    if ((st = check_tensor(moms[i], true, "momentum", i, err)) != MUON_OK ||
        (st = check_ptr(moms[i].ptr, "momentum", i, err)) != MUON_OK) {
      g_last_error = err;
      return st;
    }
    if (moms[i].rows != params[i].rows || moms[i].cols != params[i].cols) {
      g_last_error = "momentum " + std::to_string(i) + ": shape differs from its param";
      return MUON_E_SHAPE;
    }
  }
  if (n == 0) return MUON_OK;
  // Plan into the scratch array: tables, partials and counters first, then
  // the Newton-Schulz workspace of one chunk, its cap set to what is left.
  Plan probe;
  st = build_plan(*cfg, params, kinds.data(), n, nullptr, probe, err, kTallMaxChunks, moms);
  if (st != MUON_OK) { g_last_error = err; return st; }
  void* sp = nullptr;
  hipError_t e = noalloc_scratch(&sp);
  if (e != hipSuccess) {
    g_last_error = std::string("muon_step_noalloc: scratch address: ") + hipGetErrorString(e);
    return MUON_E_HIP;
  }
  const int64_t tall_limit = probe.n_tall_tiles_max > 0 ? device_tall_limit() : 0;
  muon_config c = *cfg;
  Plan pl;
  size_t cap = kNoallocScratchBytes;
  for (int attempt = 0; attempt < 4; ++attempt) {
    c.ns_workspace_max = cfg->ns_workspace_max ? std::min<uint64_t>(cfg->ns_workspace_max, cap) : cap;
    st = build_plan(c, params, kinds.data(), n, static_cast<char*>(sp), pl, err, tall_limit, moms);
    if (st != MUON_OK) { g_last_error = err; return st; }
    const size_t other = pl.total - pl.ws_bytes;
    if (pl.total <= kNoallocScratchBytes || other + kAlign >= kNoallocScratchBytes) break;
    cap = kNoallocScratchBytes - other - kAlign;
  }
  if (pl.total > kNoallocScratchBytes) {
    g_last_error = "muon_step_noalloc: this step needs " + std::to_string(pl.total) +
                   " bytes of device scratch (launch tables, partial sums and the largest "
                   "matrix's Newton-Schulz workspace); the array holds " +
                   std::to_string(kNoallocScratchBytes);
    return MUON_E_WORKSPACE;
  }
  bind_tensors(pl, params, grads, kinds.data(), n);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  char* base = static_cast<char*>(sp);
  const char* what = "muon_step_noalloc: clearing the scratch counters";
  // The array keeps the last call's contents: clear the partial rows and the
  // tall RowNorm counters, which must start at zero.
  e = launch_fill_zero(s, base, pl.zero_end);
  if (e == hipSuccess && pl.tall_sync_bytes)
    e = launch_fill_zero(s, base + pl.off_tall_sync, pl.tall_sync_bytes);
  if (e == hipSuccess) e = upload_plan(s, base, pl, &what);
  // The host copies of the tables must outlive the transfers.
  if (e == hipSuccess) {
    what = "muon_step_noalloc: hipStreamSynchronize";
    e = hipStreamSynchronize(s);
  }
  if (e != hipSuccess) {
    g_last_error = std::string(what) + ": " + hipGetErrorString(e);
    return MUON_E_HIP;
  }
  muon_ctx tmp;
  tmp.cfg = c;
  tmp.stream = s;
  tmp.base = base;
  tmp.n = n;
  tmp.plan = std::move(pl);
  (void)hipGetDevice(&tmp.device);
  st = enqueue_step(&tmp, step);
  if (st != MUON_OK) g_last_error = tmp.err;
  return st;
}

void muon_free(muon_ctx* ctx) { delete ctx; }

const char* muon_status_str(int32_t s) {
  switch (s) {
    case MUON_OK: return "ok";
    case MUON_E_ARG: return "invalid argument";
    case MUON_E_SHAPE: return "shape mismatch";
    case MUON_E_DTYPE: return "dtype mismatch";
    case MUON_E_ALIGN: return "misaligned or strided tensor";
    case MUON_E_WORKSPACE: return "state buffer missing or too small";
    case MUON_E_STATE: return "invalid context state";
    case MUON_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* muon_last_error(const muon_ctx* ctx) {
  return ctx ? ctx->err.c_str() : g_last_error.c_str();
}

}  // extern "C"
