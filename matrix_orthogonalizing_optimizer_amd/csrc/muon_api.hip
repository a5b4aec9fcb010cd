// C ABI of the Muon optimizer step (declared in include/muon.h).
//
// Host side: argument validation (all-or-nothing), grouping of matrices by
// oriented shape, tile choice, workspace layout, the descriptor table, and
// the launch sequence of one step:
//   per shape group ("bin"), per chunk of matrices that fits the workspace:
//     prep (momentum, Nesterov input, norm partials, X_0 in the oriented layout)
//     norm (r = 1 / (||N||_F + eps))
//     N x { Gram, Poly, Update }   -- the last Update applies the step
//     rms (optional update RMS)
// The method is that of "Muon is Scalable for LLM Training" (section 2.1,
// Eq. 1 and 2; section 2.2, Eq. 4; section 2.3, Algorithm 1's RMS).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "muon.h"
#include "mo_internal.h"
#include "mo_host.h"

namespace mo {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

bool debug_sync() {
  static const bool on = [] {
    const char* e = std::getenv("MO_DEBUG_SYNC");
    return e && *e && std::strcmp(e, "0") != 0;
  }();
  return on;
}

// ------------------------------------------------------------------ profiling
struct ProfEntry {
  hipEvent_t start, stop;
  double work;
};
struct ProfClass {
  int64_t launches = 0;
  double ms = 0.0, work = 0.0;
  std::vector<ProfEntry> pending;
};
std::mutex g_prof_mu;
unsigned g_prof_mask = 0;
ProfClass g_prof[MO_K_COUNT];

ProfScope::ProfScope(int c, hipStream_t st, double w) {
  if (!(g_prof_mask & (1u << c))) return;
  if (hipEventCreate(&start_) != hipSuccess || hipEventCreate(&stop_) != hipSuccess) return;
  cls_ = c;
  s_ = st;
  work_ = w;
  (void)hipEventRecord(start_, s_);
}

ProfScope::~ProfScope() {
  if (cls_ < 0) return;
  (void)hipEventRecord(stop_, s_);
  std::lock_guard<std::mutex> g(g_prof_mu);
  g_prof[cls_].pending.push_back({start_, stop_, work_});
}

// Launch bookkeeping: checks the launch status and optionally syncs.
int checked(hipError_t e, hipStream_t s, const char* what) {
  if (e != hipSuccess) return fail(MO_EHIP, "%s launch failed: %s", what, hipGetErrorString(e));
  if (debug_sync()) {
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(MO_EHIP, "%s failed: %s", what, hipGetErrorString(e));
  }
  return MO_OK;
}

int validate_dtype(int dt, const char* what) {
  if (dt != MO_F32 && dt != MO_BF16) return fail(MO_EINVAL, "%s must be MO_F32 or MO_BF16 (got %d)", what, dt);
  return MO_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_workspace(void* ws, size_t ws_bytes, size_t min_bytes) {
  if (!ws) return fail(MO_EWORKSPACE, "workspace is NULL (need %zu bytes)", min_bytes);
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(MO_EWORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < min_bytes)
    return fail(MO_EWORKSPACE, "workspace has %zu bytes, need at least %zu", ws_bytes, min_bytes);
  return MO_OK;
}

}  // namespace mo

namespace {

using namespace mo;

int64_t ru(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

bool finite(float x) { return std::isfinite(x); }

// ------------------------------------------------------------------ planning
struct Bin {
  int m, n, m_pad, n_pad;
  TileCfg cfg;
  int first, count;        // range in the plan's descriptor order
};

struct HostPlan {
  int grad_dt = BF16, mom_dt = BF16, ns_dt = BF16;
  int64_t count = 0;
  std::vector<MatDesc> descs;   // grouped by bin
  std::vector<Bin> bins;
  int esz() const { return ns_dt == F32 ? 4 : 2; }
};

int dt_size(int dt) { return dt == F32 ? 4 : 2; }

// Tile choice for a shape group: the estimated time of its padded work at
// each tile size.  The symmetric products (Gram and polynomial, lower tiles
// only) and the update (all tiles) are separate launches, so each is charged
// for how well its own tile count fills 256 CUs.  Per-tile efficiencies are
// measured: with the chip filled, a 128 tile delivers about 0.75 and a 64
// tile about 0.5 of a 256 tile's rate (Newton-Schulz alone, bf16, N = 5, 15
// shapes from [64, 2048] to [2048, 5632] and batches of 8 to 64, every tile
// size forced in turn); these constants pick the fastest size on 13 of the
// 15 and lose 1.6% and 4.9% on the other two.  Groups of small matrices
// (m <= 128, bf16, at least kSmallMinCount of them) take 128 tiles: the
// fused small-matrix kernel works on 128-row panels.
constexpr int kSmallMinCount = 32;
TileCfg choose_tile(int m, int n, int count, int ns_dt) {
  if (const char* e = std::getenv("MO_TILE")) {
    const int t = std::atoi(e);
    if (t == 256 && ns_dt == BF16) return TILE_256;
    if (t == 128) return TILE_128;
    if (t == 64) return TILE_64;
  }
  if (ns_dt == BF16 && m <= 128 && count >= kSmallMinCount) return TILE_128;
  const TileCfg cands_bf[] = {TILE_256, TILE_128, TILE_64};
  const TileCfg cands_f[] = {TILE_128, TILE_64};
  const TileCfg* c = ns_dt == BF16 ? cands_bf : cands_f;
  const int nc = ns_dt == BF16 ? 3 : 2;
  auto filled = [](double tiles) { return tiles / (std::ceil(tiles / 256.0) * 256.0); };
  double best = 1e300;
  TileCfg pick = c[nc - 1];
  for (int i = 0; i < nc; ++i) {
    const int T = tile_size(c[i]);
    const double eff = T == 256 ? 1.0 : (T == 128 ? 0.75 : 0.5);
    const double mp = static_cast<double>(ru(m, T)), np = static_cast<double>(ru(n, T));
    const double tm = mp / T, tn = np / T;
    const double sym_work = (mp * mp * np + mp * mp * mp) * count;
    const double upd_work = 2.0 * mp * mp * np * count;
    const double cost = (sym_work / filled(count * tm * (tm + 1) / 2) + upd_work / filled(count * tm * tn)) / eff;
    if (cost < best * 0.999) {
      best = cost;
      pick = c[i];
    }
  }
  return pick;
}

struct Range {
  uintptr_t lo, hi;
  int64_t idx;
  const char* what;
};

int check_overlap(std::vector<Range>& r) {
  std::sort(r.begin(), r.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < r.size(); ++i)
    if (r[i].lo < r[i - 1].hi)
      return fail(MO_EINVAL, "tensor %lld %s overlaps tensor %lld %s", static_cast<long long>(r[i].idx),
                  r[i].what, static_cast<long long>(r[i - 1].idx), r[i - 1].what);
  return MO_OK;
}

constexpr int64_t kMaxDim = 1 << 24;
constexpr int64_t kMaxPadded = (int64_t{1} << 31) - 1;

int build_plan(const mo_tensor* t, int64_t count, int grad_dt, int mom_dt, int ns_dt, bool check_ptrs,
               HostPlan& plan) {
  int rc;
  if ((rc = validate_dtype(grad_dt, "grad_dtype")) || (rc = validate_dtype(mom_dt, "mom_dtype")) ||
      (rc = validate_dtype(ns_dt, "ns_dtype")))
    return rc;
  if (count < 0) return fail(MO_EINVAL, "count must be >= 0");
  if (count > 0 && !t) return fail(MO_EINVAL, "tensors is NULL");
  if (count > (int64_t{1} << 30)) return fail(MO_EINVAL, "too many tensors");
  plan = HostPlan{};
  plan.grad_dt = grad_dt;
  plan.mom_dt = mom_dt;
  plan.ns_dt = ns_dt;
  plan.count = count;
  std::vector<Range> ranges;
  struct Item {
    int m, n;
    int64_t idx;
  };
  std::vector<Item> items;
  items.reserve(count);
  for (int64_t i = 0; i < count; ++i) {
    const mo_tensor& x = t[i];
    if (x.rows < 1 || x.cols < 1 || x.rows > kMaxDim || x.cols > kMaxDim)
      return fail(MO_EINVAL, "tensor %lld: rows and cols must be in [1, 2^24]", static_cast<long long>(i));
    const int m = static_cast<int>(std::min(x.rows, x.cols)), n = static_cast<int>(std::max(x.rows, x.cols));
    if (ru(m, 256) * ru(n, 256) > kMaxPadded)
      return fail(MO_EINVAL, "tensor %lld: %lld x %lld exceeds 2^31 padded elements", static_cast<long long>(i),
                  static_cast<long long>(x.rows), static_cast<long long>(x.cols));
    if (check_ptrs) {
      if (!x.param || !x.grad || !x.state0)
        return fail(MO_EINVAL, "tensor %lld: param, grad and state0 must be non-NULL", static_cast<long long>(i));
      if (x.state1) return fail(MO_EINVAL, "tensor %lld: state1 must be NULL for Muon", static_cast<long long>(i));
      if (!aligned16(x.param) || !aligned16(x.grad) || !aligned16(x.state0))
        return fail(MO_EINVAL, "tensor %lld: pointers must be 16-byte aligned", static_cast<long long>(i));
      const uintptr_t ne = static_cast<uintptr_t>(x.rows * x.cols);
      ranges.push_back({reinterpret_cast<uintptr_t>(x.param), reinterpret_cast<uintptr_t>(x.param) + ne * 4, i, "param"});
      ranges.push_back({reinterpret_cast<uintptr_t>(x.grad),
                        reinterpret_cast<uintptr_t>(x.grad) + ne * dt_size(grad_dt), i, "grad"});
      ranges.push_back({reinterpret_cast<uintptr_t>(x.state0),
                        reinterpret_cast<uintptr_t>(x.state0) + ne * dt_size(mom_dt), i, "momentum"});
    }
    items.push_back({m, n, i});
  }
  if (check_ptrs && (rc = check_overlap(ranges))) return rc;
  std::stable_sort(items.begin(), items.end(), [](const Item& a, const Item& b) {
    return a.m != b.m ? a.m > b.m : a.n > b.n;
  });
  for (size_t i = 0; i < items.size();) {
    size_t j = i;
    while (j < items.size() && items[j].m == items[i].m && items[j].n == items[i].n) ++j;
    Bin b{};
    b.m = items[i].m;
    b.n = items[i].n;
    b.count = static_cast<int>(j - i);
    b.first = static_cast<int>(plan.descs.size());
    b.cfg = choose_tile(b.m, b.n, b.count, ns_dt);
    const int T = tile_size(b.cfg);
    b.m_pad = static_cast<int>(ru(b.m, T));
    b.n_pad = static_cast<int>(ru(b.n, T));
    for (size_t k = i; k < j; ++k) {
      const mo_tensor& x = t[items[k].idx];
      MatDesc d{};
      d.param = static_cast<float*>(x.param);
      d.grad = x.grad;
      d.mom = x.state0;
      d.oriented = x.rows > x.cols ? 1 : 0;
      d.out_index = static_cast<int32_t>(items[k].idx);
      plan.descs.push_back(d);
    }
    plan.bins.push_back(b);
    i = j;
  }
  return MO_OK;
}

// Workspace layout ---------------------------------------------------------
// [descriptor table (one-shot calls only)] [rscale: count floats]
// [step: count floats (update-norm scaling)]
// then, reused by every bin in turn, for a chunk of `cap` matrices:
// [norm partials] [rms partials] [X][X'][S][P]
struct BinLayout {
  int64_t x_elems, s_elems;
  int prep_tiles, upd_tiles, x0_tiles, rms_tiles;
};

BinLayout bin_layout(const Bin& b, int esz) {
  BinLayout L{};
  const int T = tile_size(b.cfg);
  L.x_elems = static_cast<int64_t>(b.m_pad) * b.n_pad;
  L.s_elems = static_cast<int64_t>(b.m_pad) * b.m_pad;
  L.prep_tiles = (b.m_pad / 64) * (b.n_pad / 64);
  L.upd_tiles = (b.m_pad / T) * (b.n_pad / T);
  L.x0_tiles = static_cast<int>(((b.m + 63) / 64) * static_cast<int64_t>((b.n + 63) / 64));
  L.rms_tiles = std::max(L.upd_tiles, L.x0_tiles);
  return L;
}

size_t fixed_bytes(const HostPlan& p, bool with_table) {
  size_t f = 0;
  if (with_table) f += align_up(p.descs.size() * sizeof(MatDesc));
  f += 2 * align_up(static_cast<size_t>(p.count) * 4);
  return f;
}

// Bytes of an item's region (every piece rounded up to kAlign).
size_t item_bytes(const BinLayout& L, int chunk, int esz) {
  const size_t c = static_cast<size_t>(chunk);
  return align_up(c * L.prep_tiles * 4) + align_up(c * L.rms_tiles * 4) +
         2 * align_up(c * L.x_elems * esz) + 2 * align_up(c * L.s_elems * esz);
}

// full: every shape group resident at once (grouped launches); min: one
// matrix of the largest group at a time.
void ws_sizes(const HostPlan& p, bool with_table, size_t* full, size_t* mn) {
  size_t sum_full = 0, mx_min = 0;
  for (const Bin& b : p.bins) {
    const BinLayout L = bin_layout(b, p.esz());
    sum_full += item_bytes(L, b.count, p.esz());
    mx_min = std::max(mx_min, item_bytes(L, 1, p.esz()));
  }
  const size_t f = fixed_bytes(p, with_table);
  if (full) *full = f + sum_full;
  if (mn) *mn = f + mx_min;
}

struct Hyper {
  float lr, wd, mu, a, b, c, rms_scale, eps;
  int nesterov, ns_steps;
  bool has_mom;
  int scaling;      // MO_SCALE_*
  float hidden;     // H of MO_SCALE_HIDDEN
};

int validate_hyper(const Hyper& h) {
  if (!finite(h.lr) || !finite(h.wd) || !finite(h.mu) || !finite(h.rms_scale))
    return fail(MO_EINVAL, "lr, wd, mu and rms_scale must be finite");
  if (!finite(h.eps) || h.eps < 0.0f) return fail(MO_EINVAL, "eps must be finite and >= 0");
  if (!finite(h.a) || !finite(h.b) || !finite(h.c)) return fail(MO_EINVAL, "abc must be finite");
  if (h.ns_steps < 0 || h.ns_steps > 16) return fail(MO_EINVAL, "ns_steps must be in [0, 16]");
  return MO_OK;
}

// The matrices of one shape group (or a chunk of them) and their carved
// workspace: [norm partials] [rms partials] [X] [X'] [S] [P].
struct Item {
  const Bin* bin;
  BinLayout L;
  int c0, chunk;
  const MatDesc* desc;
  float* rscale;
  float* step;        // per matrix step of the update-norm scaling
  float* norm_part;
  float* rms_part;
  char* x[2];
  char* S;
  char* P;
};

char* carve(Item& it, char* q, int esz) {
  auto take = [&](size_t bytes) {
    char* r = q;
    q += align_up(bytes);
    return r;
  };
  const size_t c = static_cast<size_t>(it.chunk);
  it.norm_part = reinterpret_cast<float*>(take(c * it.L.prep_tiles * 4));
  it.rms_part = reinterpret_cast<float*>(take(c * it.L.rms_tiles * 4));
  it.x[0] = take(c * it.L.x_elems * esz);
  it.x[1] = take(c * it.L.x_elems * esz);
  it.S = take(c * it.L.s_elems * esz);
  it.P = take(c * it.L.s_elems * esz);
  return q;
}

struct StepCtx {
  const HostPlan& plan;
  const Hyper& h;
  float* update_rms;
  hipStream_t s;
  void* store_out;
  int64_t store_stride;
  int esz;
  float lrwd;
};

// lr times the scale of X_N in the update: Eq. 4 / Eq. 7 rms_scale
// sqrt(max(A, B)), or Eq. 5 rms_scale sqrt(H).  (Eq. 6 scales per matrix on
// the device: Item::step.)
float item_step(const StepCtx& c, const Item& it) {
  const double root = c.h.scaling == MO_SCALE_HIDDEN ? std::sqrt(static_cast<double>(c.h.hidden))
                                                     : std::sqrt(static_cast<double>(it.bin->n));
  const double scale = static_cast<double>(c.h.rms_scale) * root;
  return static_cast<float>(static_cast<double>(c.h.lr) * scale);
}

// Waves per workgroup of a GEMM launch: bf16 256-wide tiles run 8 waves
// (two per SIMD, so one wave's memory waits are covered by the other's
// MFMAs; measured faster on every product), everything else 4.  The 8-wave
// polynomial product folds b S into the accumulators as (b / c) S, so a
// polynomial without the S^2 term (c = 0) runs 4 waves.
int gemm_waves(int ns_dt, TileCfg cfg, Epi epi, float c) {
  if (ns_dt != BF16 || cfg != TILE_256) return 4;
  if (epi == EPI_POLY && c == 0.0f) return 4;
  if (const char* e = std::getenv("MO_WAVES")) {
    const int w = std::atoi(e);
    if (w == 4 || w == 8) return w;
  }
  return 8;
}

// One Newton-Schulz product over a set of items: launches grouped by tile
// configuration, up to kMaxGroup shape groups per launch.
// rms_only (EPI_APPLY): the scale pass of the update-norm scaling, which
// only writes the partial sums of squares of X_N.
int gemm_phase(const StepCtx& c, std::vector<Item>& items, Epi epi, int k, int cls, const char* what,
               bool rms_only = false) {
  int rc;
  const int N = c.h.ns_steps;
  std::vector<int> order(items.size());
  for (size_t i = 0; i < items.size(); ++i) order[i] = static_cast<int>(i);
  // same tile configuration together
  std::stable_sort(order.begin(), order.end(),
                   [&](int x, int y) { return items[x].bin->cfg < items[y].bin->cfg; });
  size_t i0 = 0;
  while (i0 < order.size()) {
    const TileCfg cfg = items[order[i0]].bin->cfg;
    size_t i1 = i0;
    while (i1 < order.size() && items[order[i1]].bin->cfg == cfg && i1 - i0 < static_cast<size_t>(kMaxGroup)) ++i1;
    GemmArgs g{};
    g.nbins = static_cast<int>(i1 - i0);
    g.use_rscale = (k == 0 && (epi == EPI_GRAM || epi == EPI_UPDATE || epi == EPI_APPLY || epi == EPI_STORE)) ? 1 : 0;
    g.alpha = c.h.c; g.beta = c.h.b; g.gamma = c.h.a;
    g.lrwd = c.lrwd;
    g.rms_only = rms_only ? 1 : 0;
    const bool unorm = c.h.scaling == MO_SCALE_UPDATE_NORM && c.store_out == nullptr;
    double work = 0.0;
    int per_xcd = 0;
    bool all_super = true;
    const bool want_rms = c.update_rms != nullptr && c.store_out == nullptr;
    const int bk = 64 / c.esz;              // K elements per stage (64 bytes)
    for (size_t j = i0; j < i1; ++j) {
      const Item& it = items[order[j]];
      const Bin& bin = *it.bin;
      GemmBin& gb = g.bin[j - i0];
      const int T = tile_size(bin.cfg);
      const int tm = bin.m_pad / T, tn = bin.n_pad / T;
      const double m = bin.m, n = bin.n;
      char* xc = it.x[k & 1];
      char* xn = it.x[(k + 1) & 1];
      gb.rscale = it.rscale;
      gb.batch = it.chunk;
      if (epi == EPI_GRAM) {            // S = X X^T
        gb.A = xc; gb.sA = it.L.x_elems;
        gb.B = xc; gb.sB = it.L.x_elems;
        gb.C = it.S; gb.sC = it.L.s_elems;
        gb.M = bin.m_pad; gb.N = bin.m_pad; gb.K = bin.n_pad;
        gb.k_loop = gb.K / bk;
        gb.tiles_m = tm; gb.tiles_n = tm; gb.tiles_per_mat = tm * (tm + 1) / 2;
        work += it.chunk * m * m * n;
      } else if (epi == EPI_POLY) {     // P' = a I + b S + c S S
        gb.A = it.S; gb.sA = it.L.s_elems;
        gb.B = it.S; gb.sB = it.L.s_elems;
        gb.D = it.S; gb.sD = it.L.s_elems;
        gb.C = it.P; gb.sC = it.L.s_elems;
        gb.M = bin.m_pad; gb.N = bin.m_pad; gb.K = bin.m_pad;
        // K runs over S's columns: stages past the true m multiply its zero
        // padding only
        gb.k_loop = (bin.m + bk - 1) / bk;
        gb.tiles_m = tm; gb.tiles_n = tm; gb.tiles_per_mat = tm * (tm + 1) / 2;
        work += it.chunk * m * m * m;
      } else {                          // X' = P' X, X read K-major from its own layout
        gb.A = it.P; gb.sA = it.L.s_elems;
        gb.B = xc; gb.sB = it.L.x_elems;
        gb.M = bin.m_pad; gb.N = bin.n_pad; gb.K = bin.m_pad;
        // K runs over the rows of X: stages past the true m multiply the
        // zero padding of P' and X only
        gb.k_loop = (bin.m + bk - 1) / bk;
        gb.tiles_m = tm; gb.tiles_n = tn; gb.tiles_per_mat = tm * tn;
        if (epi == EPI_UPDATE) {
          gb.C = xn; gb.sC = it.L.x_elems;
        } else {
          gb.desc = it.desc;
          gb.m_true = bin.m; gb.n_true = bin.n;
          gb.step = item_step(c, it);
          gb.step_dev = unorm ? it.step : nullptr;
          gb.rms_part = rms_only ? it.rms_part : (want_rms && !unorm ? it.rms_part : nullptr);
          if (epi == EPI_STORE) {
            gb.out = static_cast<char*>(c.store_out) + static_cast<size_t>(it.c0) * c.store_stride * c.esz;
            gb.s_out = c.store_stride;
          }
        }
        if (!rms_only) work += 2.0 * it.chunk * m * m * n;
      }
      const bool sym = (epi == EPI_GRAM || epi == EPI_POLY);
      gb.super_order = (tm >= 16 && tm % 16 == 0 && (sym || tn % 16 == 0)) ? 1 : 0;
      all_super = all_super && gb.super_order;
      const int total = gb.tiles_per_mat * gb.batch;
      per_xcd += (total + 7) / 8;
    }
    g.per_xcd = per_xcd;
    // super-blocks need every XCD on the same block at a time
    g.rotate = all_super ? 0 : 1;
    (void)N;
    ProfScope ps(cls, c.s, work);
    const int waves = gemm_waves(c.plan.ns_dt, cfg, epi, g.alpha);
    if ((rc = checked(launch_gemm(c.plan.ns_dt, cfg, epi, waves, g, c.s), c.s, what))) return rc;
    i0 = i1;
  }
  return MO_OK;
}

// The fused small-matrix kernel takes a shape group when its matrices sit
// on one 128-row panel (m <= 128, bf16) and are numerous enough to fill the
// chip with one workgroup each; it applies with the shape or hidden scaling
// (the update-norm scaling and the Newton-Schulz-only entry point take the
// general kernels).  It iterates on the m x m Gram matrix, where rounding
// can push the eigenvalues of directions with tiny singular values below
// zero; the polynomial then amplifies them by about a^2 = 11.9 per step
// without the bound that the odd polynomial keeps on singular values.  Up
// to 5 steps this stays at or below the error of bf16 iterates even on
// rank-deficient inputs; from 8 steps on it can overflow, so longer
// iterations take the general kernels.  The choice depends on the whole
// group, not on the chunk a smaller workspace processes at a time, so
// results do not depend on the workspace size.
constexpr int kSmallMaxSteps = 5;
bool small_eligible(const StepCtx& c, const Item& it) {
  const char* e = std::getenv("MO_NO_SMALL");
  const bool off = e && std::atoi(e) != 0;
  return !off && c.plan.ns_dt == BF16 && it.bin->cfg == TILE_128 && it.bin->m_pad == 128 &&
         it.bin->count >= kSmallMinCount && c.store_out == nullptr && c.h.scaling != MO_SCALE_UPDATE_NORM &&
         c.h.ns_steps <= kSmallMaxSteps;
}

// Momentum, norm, Newton-Schulz and apply for a set of items processed
// together (all shape groups at once when the workspace allows).
int run_round(const StepCtx& c, std::vector<Item>& items) {
  int rc;
  const HostPlan& plan = c.plan;
  const Hyper& h = c.h;
  const bool want_rms = c.update_rms != nullptr && c.store_out == nullptr;
  for (Item& it : items) {
    const Bin& bin = *it.bin;
    PrepArgs a{};
    a.desc = it.desc;
    a.x = it.x[0];
    a.x_stride = it.L.x_elems;
    a.tile = tile_size(bin.cfg);
    a.m = bin.m; a.n = bin.n; a.m_pad = bin.m_pad; a.n_pad = bin.n_pad;
    a.tiles_per_mat = it.L.prep_tiles;
    a.mu = h.mu;
    a.nesterov = h.nesterov;
    a.has_mom = h.has_mom ? 1 : 0;
    a.grad_dt = plan.grad_dt; a.mom_dt = plan.mom_dt; a.ns_dt = plan.ns_dt;
    a.norm_part = it.norm_part;
    const double elems = static_cast<double>(it.chunk) * bin.m * bin.n;
    const double bytes = elems * (dt_size(plan.grad_dt) + (h.has_mom ? 2 * dt_size(plan.mom_dt) : 0) + c.esz);
    {
      ProfScope ps(MO_K_MOMENTUM, c.s, bytes);
      if ((rc = checked(launch_prep(a, it.chunk, c.s), c.s, "prep"))) return rc;
    }
    NormArgs na{it.norm_part, it.L.prep_tiles, h.eps, it.rscale};
    ProfScope ps(MO_K_NORM, c.s, static_cast<double>(it.chunk) * it.L.prep_tiles * 4);
    if ((rc = checked(launch_norm(na, it.chunk, c.s), c.s, "norm"))) return rc;
  }
  // Eq. 6 (update-norm scaling): the per-matrix step lr rms_scale / RMS(X_N)
  // is computed on the device before the apply; it also yields update_rms
  const bool unorm = h.scaling == MO_SCALE_UPDATE_NORM && c.store_out == nullptr;
  auto scale_pass = [&](Item& it, const float* part, int tiles, const float* rscale) {
    RmsArgs a{};
    a.desc = it.desc;
    a.part = part;
    a.tiles = tiles;
    a.inv_count = 1.0 / (static_cast<double>(it.bin->m) * it.bin->n);
    a.update_rms = want_rms ? c.update_rms : nullptr;
    a.rscale = rscale;
    a.step = it.step;
    a.lr_scale = static_cast<float>(static_cast<double>(h.lr) * h.rms_scale);
    ProfScope ps(MO_K_RMS, c.s, static_cast<double>(it.chunk) * tiles * 4);
    return checked(launch_rms(a, it.chunk, c.s), c.s, "scale");
  };
  if (h.ns_steps == 0) {
    for (Item& it : items) {
      if (unorm && (rc = scale_pass(it, it.norm_part, it.L.prep_tiles, it.rscale))) return rc;
      const Bin& bin = *it.bin;
      ApplyX0Args a{};
      a.desc = it.desc;
      a.x = it.x[0];
      a.x_stride = it.L.x_elems;
      a.tile = tile_size(bin.cfg);
      a.m = bin.m; a.n = bin.n; a.m_pad = bin.m_pad; a.n_pad = bin.n_pad;
      a.tiles_per_mat = it.L.x0_tiles;
      a.rscale = it.rscale;
      a.lrwd = c.lrwd;
      a.step = item_step(c, it);
      a.step_dev = unorm ? it.step : nullptr;
      a.ns_dt = plan.ns_dt;
      a.out = c.store_out ? static_cast<char*>(c.store_out) + static_cast<size_t>(it.c0) * c.store_stride * c.esz
                          : nullptr;
      a.s_out = c.store_stride;
      a.rms_part = want_rms && !unorm ? it.rms_part : nullptr;
      const double elems = static_cast<double>(it.chunk) * bin.m * bin.n;
      ProfScope ps(MO_K_APPLY_X0, c.s, elems * (c.esz + (c.store_out ? c.esz : 8)));
      if ((rc = checked(launch_apply_x0(a, it.chunk, c.s), c.s, "apply_x0"))) return rc;
    }
  } else {
    // shape groups of many small matrices (m <= 128 on 128-row panels) run
    // the whole iteration and the apply in one fused kernel
    std::vector<Item> small, rest;
    for (Item& it : items) (small_eligible(c, it) ? small : rest).push_back(it);
    for (size_t i0 = 0; i0 < small.size(); i0 += kMaxGroup) {
      SmallArgs a{};
      a.ns_steps = h.ns_steps;
      a.a = h.a; a.b = h.b; a.c = h.c;
      a.lrwd = c.lrwd;
      int total = 0;
      double work = 0.0;
      for (size_t j = i0; j < std::min(small.size(), i0 + kMaxGroup); ++j) {
        const Item& it = small[j];
        SmallBin& sb = a.bin[a.nbins++];
        sb.desc = it.desc;
        sb.x0 = it.x[0];
        sb.x_stride = it.L.x_elems;
        sb.rscale = it.rscale;
        sb.rms_part = want_rms ? it.rms_part : nullptr;
        sb.n_pad = it.bin->n_pad; sb.m_true = it.bin->m; sb.n_true = it.bin->n;
        sb.count = it.chunk;
        sb.step = item_step(c, it);
        total += it.chunk;
        const double m = it.bin->m, n = it.bin->n;
        work += static_cast<double>(it.chunk) * h.ns_steps * (3.0 * m * m * n + m * m * m);
      }
      ProfScope ps(MO_K_UPDATE, c.s, work);
      if ((rc = checked(launch_small(a, total, c.s), c.s, "ns_small"))) return rc;
    }
    for (int k = 0; k < h.ns_steps && !rest.empty(); ++k) {
      const bool last = (k + 1 == h.ns_steps);
      if ((rc = gemm_phase(c, rest, EPI_GRAM, k, MO_K_GRAM, "gram"))) return rc;
      if ((rc = gemm_phase(c, rest, EPI_POLY, k, MO_K_POLY, "poly"))) return rc;
      const Epi ue = !last ? EPI_UPDATE : (c.store_out ? EPI_STORE : EPI_APPLY);
      if (last && unorm) {
        if ((rc = gemm_phase(c, rest, EPI_APPLY, k, MO_K_UPDATE, "update norm", true))) return rc;
        for (Item& it : rest)
          if ((rc = scale_pass(it, it.rms_part, it.L.upd_tiles, nullptr))) return rc;
      }
      if ((rc = gemm_phase(c, rest, ue, k, last ? MO_K_APPLY : MO_K_UPDATE, "update"))) return rc;
    }
  }
  if (want_rms && !unorm) {
    for (Item& it : items) {
      RmsArgs a{};
      a.desc = it.desc;
      a.part = it.rms_part;
      a.tiles = h.ns_steps == 0 ? it.L.x0_tiles : it.L.upd_tiles;
      a.inv_count = 1.0 / (static_cast<double>(it.bin->m) * it.bin->n);
      a.update_rms = c.update_rms;
      ProfScope ps(MO_K_RMS, c.s, static_cast<double>(it.chunk) * a.tiles * 4);
      if ((rc = checked(launch_rms(a, it.chunk, c.s), c.s, "rms"))) return rc;
    }
  }
  return MO_OK;
}

// Enqueues the whole step.  `d_desc` is the device copy of plan.descs.
// `store_out`: Newton-Schulz-only mode, writing X_N into store_out.
// With a workspace of the full size every shape group is resident at once
// and each Newton-Schulz product is one launch over all groups; otherwise
// the groups (in chunks that fit) are processed one after another.
int run_step(const HostPlan& plan, const MatDesc* d_desc, const Hyper& h, float* update_rms, char* ws,
             size_t ws_bytes, size_t fixed_used, hipStream_t s, void* store_out, int64_t store_stride) {
  const int esz = plan.esz();
  float* rscale_all = reinterpret_cast<float*>(ws + fixed_used);
  float* step_all = reinterpret_cast<float*>(ws + fixed_used + align_up(static_cast<size_t>(plan.count) * 4));
  char* region = ws + fixed_used + 2 * align_up(static_cast<size_t>(plan.count) * 4);
  const size_t region_bytes = ws_bytes - static_cast<size_t>(region - ws);
  StepCtx c{plan, h, update_rms, s, store_out, store_stride, esz,
            static_cast<float>(static_cast<double>(h.lr) * h.wd)};
  auto make_item = [&](const Bin& bin, int c0, int chunk) {
    Item it{};
    it.bin = &bin;
    it.L = bin_layout(bin, esz);
    it.c0 = c0;
    it.chunk = chunk;
    it.desc = d_desc + bin.first + c0;
    it.rscale = rscale_all + bin.first + c0;
    it.step = step_all + bin.first + c0;
    return it;
  };
  size_t all = 0;
  for (const Bin& bin : plan.bins) all += item_bytes(bin_layout(bin, esz), bin.count, esz);
  if (all <= region_bytes) {
    std::vector<Item> items;
    char* q = region;
    for (const Bin& bin : plan.bins) {
      items.push_back(make_item(bin, 0, bin.count));
      q = carve(items.back(), q, esz);
    }
    return run_round(c, items);
  }
  int rc;
  for (const Bin& bin : plan.bins) {
    const BinLayout L = bin_layout(bin, esz);
    int cap = bin.count;
    while (cap > 0 && item_bytes(L, cap, esz) > region_bytes) --cap;
    if (cap < 1) return fail(MO_EWORKSPACE, "workspace too small for a %d x %d matrix", bin.m, bin.n);
    for (int c0 = 0; c0 < bin.count; c0 += cap) {
      std::vector<Item> items{make_item(bin, c0, std::min(cap, bin.count - c0))};
      carve(items.back(), region, esz);
      if ((rc = run_round(c, items))) return rc;
    }
  }
  return MO_OK;
}

// One-shot calls copy the descriptor table into the workspace with small
// kernels that carry it in their arguments (launch_desc_copy): the host
// neither stages it in pinned memory nor waits on an earlier call's upload.
int upload_descs(const HostPlan& plan, void* dst, hipStream_t s) {
  if (plan.descs.empty()) return MO_OK;
  return checked(launch_desc_copy(plan.descs.data(), static_cast<int64_t>(plan.descs.size()),
                                  static_cast<MatDesc*>(dst), s),
                 s, "descriptor upload");
}

Hyper make_hyper(float lr, float wd, float mu, int nesterov, int ns_steps, const float* abc, float rms_scale,
                 float eps, bool has_mom) {
  Hyper h{};
  h.lr = lr; h.wd = wd; h.mu = mu; h.nesterov = nesterov ? 1 : 0; h.ns_steps = ns_steps;
  h.a = abc ? abc[0] : 3.4445f;
  h.b = abc ? abc[1] : -4.7750f;
  h.c = abc ? abc[2] : 2.0315f;
  h.rms_scale = rms_scale; h.eps = eps; h.has_mom = has_mom;
  h.scaling = MO_SCALE_SHAPE; h.hidden = 0.0f;
  return h;
}

}  // namespace

namespace mo {

int one_shot_step(const mo_tensor* tensors, int64_t count, int grad_dtype, int mom_dtype, int ns_dtype, float lr,
                  float wd, float mu, int nesterov, int ns_steps, const float* abc, float rms_scale, float eps,
                  float* update_rms, void* workspace, size_t workspace_bytes, void* stream,
                  const char* ws_name) {
  HostPlan p;
  int rc = build_plan(tensors, count, grad_dtype, mom_dtype, ns_dtype, true, p);
  if (rc) return rc;
  const Hyper h = make_hyper(lr, wd, mu, nesterov, ns_steps, abc, rms_scale, eps, true);
  if ((rc = validate_hyper(h))) return rc;
  if (update_rms && (reinterpret_cast<uintptr_t>(update_rms) & 3u))
    return fail(MO_EINVAL, "update_rms must be 4-byte aligned");
  if (count == 0) return MO_OK;
  size_t full = 0, mn = 0;
  ws_sizes(p, true, &full, &mn);
  if (ws_name && mn > workspace_bytes)
    return fail(MO_EWORKSPACE, "these matrices need %zu bytes of %s, more than its %zu bytes", mn, ws_name,
                workspace_bytes);
  if ((rc = check_workspace(workspace, workspace_bytes, mn))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if ((rc = upload_descs(p, ws, s))) return rc;
  const size_t table = align_up(p.descs.size() * sizeof(MatDesc));
  return run_step(p, reinterpret_cast<const MatDesc*>(ws), h, update_rms, ws, workspace_bytes, table, s, nullptr, 0);
}

}  // namespace mo

struct mo_muon_plan {
  HostPlan plan;
  MatDesc* d_desc = nullptr;
  int device = 0;
  int scaling = MO_SCALE_SHAPE;
  float hidden = 0.0f;
};

extern "C" {

int mo_abi_version(void) { return MO_ABI_VERSION; }

const char* mo_last_error(void) { return g_err.c_str(); }

int mo_muon_workspace_size(const mo_tensor* tensors, int64_t count, int ns_dtype, size_t* full_bytes,
                           size_t* min_bytes) {
  if (!full_bytes) return fail(MO_EINVAL, "full_bytes is NULL");
  HostPlan p;
  int rc = build_plan(tensors, count, MO_F32, MO_F32, ns_dtype, false, p);
  if (rc) return rc;
  ws_sizes(p, true, full_bytes, min_bytes);
  return MO_OK;
}

int mo_muon_step(const mo_tensor* tensors, int64_t count, int grad_dtype, int mom_dtype, int ns_dtype, float lr,
                 float wd, float mu, int nesterov, int ns_steps, const float* abc, float rms_scale, float eps,
                 float* update_rms, void* workspace, size_t workspace_bytes, void* stream) {
  return mo::one_shot_step(tensors, count, grad_dtype, mom_dtype, ns_dtype, lr, wd, mu, nesterov, ns_steps, abc,
                           rms_scale, eps, update_rms, workspace, workspace_bytes, stream, nullptr);
}

int mo_muon_plan_create(const mo_tensor* tensors, int64_t count, int grad_dtype, int mom_dtype, int ns_dtype,
                        mo_muon_plan** out) {
  if (!out) return fail(MO_EINVAL, "plan is NULL");
  *out = nullptr;
  auto* pl = new mo_muon_plan();
  int rc = build_plan(tensors, count, grad_dtype, mom_dtype, ns_dtype, true, pl->plan);
  if (rc) {
    delete pl;
    return rc;
  }
  hipError_t e = hipGetDevice(&pl->device);
  if (e != hipSuccess) {
    delete pl;
    return fail(MO_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  }
  const size_t bytes = pl->plan.descs.size() * sizeof(MatDesc);
  if (bytes) {
    if ((e = hipMalloc(&pl->d_desc, bytes)) != hipSuccess) {
      delete pl;
      return fail(MO_EHIP, "descriptor table allocation failed: %s", hipGetErrorString(e));
    }
    if ((e = hipMemcpy(pl->d_desc, pl->plan.descs.data(), bytes, hipMemcpyHostToDevice)) != hipSuccess) {
      (void)hipFree(pl->d_desc);
      delete pl;
      return fail(MO_EHIP, "descriptor upload failed: %s", hipGetErrorString(e));
    }
  }
  *out = pl;
  return MO_OK;
}

int mo_muon_plan_workspace_size(const mo_muon_plan* plan, size_t* full_bytes, size_t* min_bytes) {
  if (!plan || !full_bytes) return fail(MO_EINVAL, "plan and full_bytes must be non-NULL");
  ws_sizes(plan->plan, false, full_bytes, min_bytes);
  return MO_OK;
}

int mo_muon_plan_step(mo_muon_plan* plan, float lr, float wd, float mu, int nesterov, int ns_steps,
                      const float* abc, float rms_scale, float eps, float* update_rms, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (!plan) return fail(MO_EINVAL, "plan is NULL");
  Hyper h = make_hyper(lr, wd, mu, nesterov, ns_steps, abc, rms_scale, eps, true);
  h.scaling = plan->scaling;
  h.hidden = plan->hidden;
  int rc;
  if ((rc = validate_hyper(h))) return rc;
  if (update_rms && (reinterpret_cast<uintptr_t>(update_rms) & 3u))
    return fail(MO_EINVAL, "update_rms must be 4-byte aligned");
  if (plan->plan.count == 0) return MO_OK;
  size_t full = 0, mn = 0;
  ws_sizes(plan->plan, false, &full, &mn);
  if ((rc = check_workspace(workspace, workspace_bytes, mn))) return rc;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan->device)
    return fail(MO_EINVAL, "plan was created on device %d, current device is %d", plan->device, dev);
  return run_step(plan->plan, plan->d_desc, h, update_rms, static_cast<char*>(workspace), workspace_bytes, 0,
                  static_cast<hipStream_t>(stream), nullptr, 0);
}

int mo_muon_plan_set_scaling(mo_muon_plan* plan, int scaling, float hidden) {
  if (!plan) return fail(MO_EINVAL, "plan is NULL");
  if (scaling != MO_SCALE_SHAPE && scaling != MO_SCALE_HIDDEN && scaling != MO_SCALE_UPDATE_NORM)
    return fail(MO_EINVAL, "scaling must be MO_SCALE_SHAPE, MO_SCALE_HIDDEN or MO_SCALE_UPDATE_NORM (got %d)",
                scaling);
  if (scaling == MO_SCALE_HIDDEN && !(finite(hidden) && hidden >= 1.0f))
    return fail(MO_EINVAL, "hidden must be finite and >= 1 for MO_SCALE_HIDDEN");
  plan->scaling = scaling;
  plan->hidden = scaling == MO_SCALE_HIDDEN ? hidden : 0.0f;
  return MO_OK;
}

int mo_muon_plan_set_grads(mo_muon_plan* plan, const void* const* grads, int64_t count, void* stream) {
  if (!plan) return fail(MO_EINVAL, "plan is NULL");
  HostPlan& hp = plan->plan;
  if (count != hp.count) return fail(MO_EINVAL, "count %lld does not match the plan's %lld tensors",
                                      static_cast<long long>(count), static_cast<long long>(hp.count));
  if (count > 0 && !grads) return fail(MO_EINVAL, "grads is NULL");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan->device)
    return fail(MO_EINVAL, "plan was created on device %d, current device is %d", plan->device, dev);
  // validate in full against the plan's other buffers before changing anything
  std::vector<Range> ranges;
  std::vector<const void*> by_desc(hp.descs.size());
  bool same = true;
  for (const Bin& b : hp.bins) {
    const uintptr_t ne = static_cast<uintptr_t>(b.m) * static_cast<uintptr_t>(b.n);
    for (int k = b.first; k < b.first + b.count; ++k) {
      const MatDesc& d = hp.descs[k];
      const void* g = grads[d.out_index];
      if (!g) return fail(MO_EINVAL, "grad %d is NULL", d.out_index);
      if (!aligned16(g)) return fail(MO_EINVAL, "grad %d must be 16-byte aligned", d.out_index);
      by_desc[k] = g;
      same = same && g == d.grad;
      ranges.push_back({reinterpret_cast<uintptr_t>(d.param), reinterpret_cast<uintptr_t>(d.param) + ne * 4,
                        d.out_index, "param"});
      ranges.push_back({reinterpret_cast<uintptr_t>(g), reinterpret_cast<uintptr_t>(g) + ne * dt_size(hp.grad_dt),
                        d.out_index, "grad"});
      ranges.push_back({reinterpret_cast<uintptr_t>(d.mom),
                        reinterpret_cast<uintptr_t>(d.mom) + ne * dt_size(hp.mom_dt), d.out_index, "momentum"});
    }
  }
  if (same) return MO_OK;
  int rc;
  if ((rc = check_overlap(ranges))) return rc;
  for (size_t k = 0; k < hp.descs.size(); ++k) hp.descs[k].grad = by_desc[k];
  hipStream_t s = static_cast<hipStream_t>(stream);
  return checked(launch_desc_copy(hp.descs.data(), static_cast<int64_t>(hp.descs.size()), plan->d_desc, s), s,
                 "descriptor upload");
}

int mo_muon_plan_destroy(mo_muon_plan* plan) {
  if (!plan) return MO_OK;
  int rc = MO_OK;
  if (plan->d_desc) {
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipFree(plan->d_desc);
    if (e != hipSuccess) rc = fail(MO_EHIP, "plan destroy failed: %s", hipGetErrorString(e));
  }
  delete plan;
  return rc;
}

int mo_adamw_step(const mo_tensor* tensors, int64_t count, int grad_dtype, float lr, float wd, double beta1,
                  double beta2, float eps, int64_t step, void* stream) {
  int rc;
  if ((rc = validate_dtype(grad_dtype, "grad_dtype"))) return rc;
  if (count < 0) return fail(MO_EINVAL, "count must be >= 0");
  if (count > 0 && !tensors) return fail(MO_EINVAL, "tensors is NULL");
  if (!finite(lr) || !finite(wd) || !finite(eps) || eps < 0.0f)
    return fail(MO_EINVAL, "lr, wd must be finite; eps finite and >= 0");
  if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0))
    return fail(MO_EINVAL, "beta1 and beta2 must be in [0, 1)");
  if (step < 1) return fail(MO_EINVAL, "step must be >= 1");
  std::vector<Range> ranges;
  for (int64_t i = 0; i < count; ++i) {
    const mo_tensor& x = tensors[i];
    if (x.rows < 1 || x.cols < 1 || x.rows > (int64_t{1} << 40) / x.cols)
      return fail(MO_EINVAL, "tensor %lld: rows and cols must be >= 1", static_cast<long long>(i));
    if (!x.param || !x.grad || !x.state0 || !x.state1)
      return fail(MO_EINVAL, "tensor %lld: param, grad, state0 and state1 must be non-NULL",
                  static_cast<long long>(i));
    if (!aligned16(x.param) || !aligned16(x.grad) || !aligned16(x.state0) || !aligned16(x.state1))
      return fail(MO_EINVAL, "tensor %lld: pointers must be 16-byte aligned", static_cast<long long>(i));
    const uintptr_t ne = static_cast<uintptr_t>(x.rows * x.cols);
    ranges.push_back({reinterpret_cast<uintptr_t>(x.param), reinterpret_cast<uintptr_t>(x.param) + ne * 4, i, "param"});
    ranges.push_back({reinterpret_cast<uintptr_t>(x.grad),
                      reinterpret_cast<uintptr_t>(x.grad) + ne * dt_size(grad_dtype), i, "grad"});
    ranges.push_back({reinterpret_cast<uintptr_t>(x.state0), reinterpret_cast<uintptr_t>(x.state0) + ne * 4, i, "m"});
    ranges.push_back({reinterpret_cast<uintptr_t>(x.state1), reinterpret_cast<uintptr_t>(x.state1) + ne * 4, i, "v"});
  }
  if ((rc = check_overlap(ranges))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  AdamArgs a{};
  a.grad_dt = grad_dtype;
  a.lr = lr; a.wd = wd; a.eps = eps;
  a.beta1 = static_cast<float>(beta1);
  a.beta2 = static_cast<float>(beta2);
  a.one_m_beta1 = static_cast<float>(1.0 - beta1);
  a.one_m_beta2 = static_cast<float>(1.0 - beta2);
  a.bc1 = static_cast<float>(1.0 / (1.0 - std::pow(beta1, static_cast<double>(step))));
  a.bc2_rsqrt = static_cast<float>(1.0 / std::sqrt(1.0 - std::pow(beta2, static_cast<double>(step))));
  for (int64_t i0 = 0; i0 < count; i0 += kAdamMaxTensors) {
    const int nt = static_cast<int>(std::min<int64_t>(kAdamMaxTensors, count - i0));
    int64_t blocks = 0;
    double bytes = 0;
    for (int k = 0; k < nt; ++k) {
      const mo_tensor& x = tensors[i0 + k];
      AdamTensor& T = a.t[k];
      T.p = static_cast<float*>(x.param);
      T.g = x.grad;
      T.m = static_cast<float*>(x.state0);
      T.v = static_cast<float*>(x.state1);
      T.n = x.rows * x.cols;
      T.block0 = blocks;
      blocks += (T.n + kAdamElemsPerBlock - 1) / kAdamElemsPerBlock;
      bytes += static_cast<double>(T.n) * (dt_size(grad_dtype) + 24);
    }
    a.count = nt;
    if (blocks > 0x7fffffff) return fail(MO_EINVAL, "AdamW launch too large");
    ProfScope ps(MO_K_ADAMW, s, bytes);
    if ((rc = checked(launch_adamw(a, blocks, s), s, "adamw"))) return rc;
  }
  return MO_OK;
}

int mo_newton_schulz_workspace_size(int64_t batch, int64_t rows, int64_t cols, int dtype, size_t* bytes) {
  if (!bytes) return fail(MO_EINVAL, "bytes is NULL");
  if (batch < 0) return fail(MO_EINVAL, "batch must be >= 0");
  std::vector<mo_tensor> t(static_cast<size_t>(batch));
  for (auto& x : t) {
    x.rows = rows;
    x.cols = cols;
  }
  HostPlan p;
  int rc = build_plan(t.data(), batch, dtype, MO_F32, dtype, false, p);
  if (rc) return rc;
  ws_sizes(p, true, bytes, nullptr);
  return MO_OK;
}

int mo_newton_schulz(const void* input, void* output, int64_t batch, int64_t rows, int64_t cols, int dtype,
                     int ns_steps, const float* abc, float eps, void* workspace, size_t workspace_bytes,
                     void* stream) {
  int rc;
  if ((rc = validate_dtype(dtype, "dtype"))) return rc;
  if (batch < 0) return fail(MO_EINVAL, "batch must be >= 0");
  if (batch > 0 && (!input || !output)) return fail(MO_EINVAL, "input and output must be non-NULL");
  if (!aligned16(input) || !aligned16(output)) return fail(MO_EINVAL, "input and output must be 16-byte aligned");
  const int64_t esz = dtype == MO_F32 ? 4 : 2;
  std::vector<mo_tensor> t(static_cast<size_t>(batch));
  for (int64_t i = 0; i < batch; ++i) {
    t[i].rows = rows;
    t[i].cols = cols;
    t[i].grad = static_cast<const char*>(input) + i * rows * cols * esz;
    t[i].param = static_cast<char*>(output) + i * rows * cols * esz;   // placeholder for the table
    t[i].state0 = nullptr;
    t[i].state1 = nullptr;
  }
  HostPlan p;
  if ((rc = build_plan(t.data(), batch, dtype, MO_F32, dtype, false, p))) return rc;
  if (batch > 0) {
    const uintptr_t in0 = reinterpret_cast<uintptr_t>(input), out0 = reinterpret_cast<uintptr_t>(output);
    const uintptr_t nb = static_cast<uintptr_t>(batch * rows * cols * esz);
    if (in0 < out0 + nb && out0 < in0 + nb) return fail(MO_EINVAL, "input and output overlap");
  }
  const Hyper h = make_hyper(0.0f, 0.0f, 0.0f, 0, ns_steps, abc, 0.0f, eps, false);
  if ((rc = validate_hyper(h))) return rc;
  if (batch == 0) return MO_OK;
  // every matrix has the same shape: one bin whose descriptors keep the
  // caller's order, so output b lands at output + b * rows * cols
  size_t full = 0, mn = 0;
  ws_sizes(p, true, &full, &mn);
  if ((rc = check_workspace(workspace, workspace_bytes, mn))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if ((rc = upload_descs(p, ws, s))) return rc;
  const size_t table = align_up(p.descs.size() * sizeof(MatDesc));
  return run_step(p, reinterpret_cast<const MatDesc*>(ws), h, nullptr, ws, workspace_bytes, table, s, output,
                  rows * cols);
}

int mo_profile_enable(unsigned int class_mask) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  g_prof_mask = class_mask & ((1u << MO_K_COUNT) - 1);
  return MO_OK;
}

int mo_profile_read(int kernel_class, int64_t* launches, double* total_ms, double* total_work) {
  if (kernel_class < 0 || kernel_class >= MO_K_COUNT) return fail(MO_EINVAL, "bad kernel class %d", kernel_class);
  std::lock_guard<std::mutex> g(g_prof_mu);
  ProfClass& c = g_prof[kernel_class];
  for (ProfEntry& e : c.pending) {
    float ms = 0.0f;
    hipError_t err = hipEventSynchronize(e.stop);
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e.start, e.stop);
    (void)hipEventDestroy(e.start);
    (void)hipEventDestroy(e.stop);
    if (err != hipSuccess) {
      c.pending.clear();
      return fail(MO_EHIP, "profile event failed: %s", hipGetErrorString(err));
    }
    c.launches += 1;
    c.ms += ms;
    c.work += e.work;
  }
  c.pending.clear();
  if (launches) *launches = c.launches;
  if (total_ms) *total_ms = c.ms;
  if (total_work) *total_work = c.work;
  return MO_OK;
}

int mo_profile_reset(void) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  for (ProfClass& c : g_prof) {
    for (ProfEntry& e : c.pending) {
      (void)hipEventSynchronize(e.stop);
      (void)hipEventDestroy(e.start);
      (void)hipEventDestroy(e.stop);
    }
    c = ProfClass{};
  }
  return MO_OK;
}

}  // extern "C"
