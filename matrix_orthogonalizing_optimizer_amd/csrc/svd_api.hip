// C ABI of the SVD-entropy diagnostic (declared in include/muon.h).
//
// "Muon is Scalable for LLM Training", section 3.4 and appendix F: the SVD
// entropy and sorted singular values of weight matrices.  Host side:
// validation (all-or-nothing), grouping by m = min(rows, cols), workspace
// layout and chunking, and the launch sequence of svd_entropy.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <vector>

#include "muon.h"
#include "mo_host.h"
#include "svd_internal.h"

namespace {

using namespace mo;

// ------------------------------------------------------- SVD entropy (host)
// Matrices are grouped by m = min(rows, cols) (then by shape, so that one
// Gram launch covers equal shapes); a group is processed in chunks that fit
// the workspace, each chunk as one batch of launches.
struct SvdItem {
  int64_t idx;            // position in the caller's list
  int64_t rows, cols;
  const void* data;
  int64_t sigma_off;      // offset of its singular values in the packed output
  int m, n;
};

size_t svd_chunk_bytes(int m, int64_t cnt) {
  const int64_t nb = (m + kSvdTile - 1) / kSvdTile;
  const size_t v = static_cast<size_t>(m) * sizeof(double) * static_cast<size_t>(cnt);
  return align_up(v * static_cast<size_t>(m))           // working matrices
         + align_up(2 * v)                                // Householder vectors (two steps)
         + 2 * align_up(v * kSvdPanel)                    // the panel's v and w
         + align_up(static_cast<size_t>(cnt) * nb * 2 * kSvdPanel * sizeof(double))   // panel dots
         + align_up(v * static_cast<size_t>(nb))          // partial products
         + 3 * align_up(v);                               // d, e, eigenvalues
}

int svd_validate(const mo_matrix* mats, int64_t count, int dtype, std::vector<SvdItem>& items,
                 int64_t* sigma_total) {
  int rc;
  if ((rc = validate_dtype(dtype, "dtype"))) return rc;
  if (count < 0) return fail(MO_EINVAL, "count must be >= 0");
  if (count > 0 && !mats) return fail(MO_EINVAL, "mats is NULL");
  if (count > (int64_t{1} << 30)) return fail(MO_EINVAL, "too many matrices");
  items.clear();
  items.reserve(static_cast<size_t>(count));
  int64_t off = 0;
  for (int64_t i = 0; i < count; ++i) {
    const mo_matrix& x = mats[i];
    if (x.rows < 1 || x.cols < 1) return fail(MO_EINVAL, "matrix %lld: rows and cols must be >= 1", static_cast<long long>(i));
    const int64_t m = std::min(x.rows, x.cols), n = std::max(x.rows, x.cols);
    if (m > kSvdMaxM) return fail(MO_EINVAL, "matrix %lld: min(rows, cols) = %lld exceeds %d", static_cast<long long>(i),
                                  static_cast<long long>(m), kSvdMaxM);
    if (n > (int64_t{1} << 31) / m || n > INT32_MAX)
      return fail(MO_EINVAL, "matrix %lld: more than 2^31 elements, or a side of 2^31", static_cast<long long>(i));
    if (!x.data) return fail(MO_EINVAL, "matrix %lld: data is NULL", static_cast<long long>(i));
    if (!aligned16(x.data)) return fail(MO_EINVAL, "matrix %lld: data must be 16-byte aligned", static_cast<long long>(i));
    items.push_back({i, x.rows, x.cols, x.data, off, static_cast<int>(m), static_cast<int>(n)});
    off += m;
  }
  *sigma_total = off;
  std::stable_sort(items.begin(), items.end(), [](const SvdItem& a, const SvdItem& b) {
    if (a.m != b.m) return a.m < b.m;
    if (a.rows != b.rows) return a.rows < b.rows;
    return a.cols < b.cols;
  });
  return MO_OK;
}

void svd_sizes(const std::vector<SvdItem>& items, size_t* full, size_t* mn) {
  size_t f = 0, lo = 0;
  for (size_t g = 0; g < items.size();) {
    size_t h = g;
    while (h < items.size() && items[h].m == items[g].m) ++h;
    const int64_t cnt = std::min<int64_t>(static_cast<int64_t>(h - g), 65535);
    f = std::max(f, svd_chunk_bytes(items[g].m, cnt));
    lo = std::max(lo, svd_chunk_bytes(items[g].m, 1));
    g = h;
  }
  *full = f;
  *mn = lo;
}

// Launches for one chunk: items [b, e) share m.
int svd_chunk(const std::vector<SvdItem>& items, size_t b, size_t e, int dtype, double* entropy, double* sigma,
              char* ws, hipStream_t s) {
  int rc;
  const int m = items[b].m, cnt = static_cast<int>(e - b);
  const int nb = (m + kSvdTile - 1) / kSvdTile;
  const size_t v = static_cast<size_t>(m) * sizeof(double) * static_cast<size_t>(cnt);
  char* q = ws;
  auto take = [&](size_t bytes) { char* r = q; q += align_up(bytes); return reinterpret_cast<double*>(r); };
  SvdTrdArgs t{};
  t.a = take(v * static_cast<size_t>(m));
  t.v = take(2 * v);
  t.pv = take(v * kSvdPanel);
  t.pw = take(v * kSvdPanel);
  t.pdot = take(static_cast<size_t>(cnt) * nb * 2 * kSvdPanel * sizeof(double));
  t.part = take(v * static_cast<size_t>(nb));
  t.d = take(v);
  t.e = take(v);
  double* lam = take(v);
  t.m = m;
  t.nb = nb;
  t.batch = cnt;

  // 1. Gram matrices, equal shapes per launch
  for (size_t i = b; i < e;) {
    SvdGramArgs g{};
    g.ld = items[i].cols;
    g.m = m;
    g.n = items[i].n;
    g.trans = items[i].rows > items[i].cols ? 1 : 0;
    const size_t first = i;
    int c = 0;
    while (i < e && c < kSvdGramBatch && items[i].rows == items[first].rows && items[i].cols == items[first].cols) {
      g.src[c] = items[i].data;
      g.dst[c] = t.a + static_cast<int64_t>(i - b) * m * m;
      ++c;
      ++i;
    }
    ProfScope ps(MO_K_SVD_GRAM, s, static_cast<double>(c) * m * m * g.n);
    if ((rc = checked(launch_svd_gram(dtype, g, c, s), s, "svd gram"))) return rc;
  }
  // 2. Householder reduction to tridiagonal, rank-2 updates applied in
  //    panels of kSvdPanel steps
  const int kend = std::max(m - 3, -1);
  int k0 = 0;
  for (int k = -1; k <= kend; ++k) {
    {
      const double rows = m - (k + 1), slots = nb - (k + 1) / kSvdTile;
      ProfScope ps(MO_K_SVD_COLUMN, s, k >= 0 ? static_cast<double>(cnt) * rows * slots * 8.0 : 0.0);
      if ((rc = checked(launch_svd_trd_col(t, k, k0, s), s, "svd column"))) return rc;
    }
    const int j = k + 1;
    if (j > m - 3) continue;
    if (k >= 0 && k - k0 + 1 == kSvdPanel) {
      const double tr = m - (j + 1);
      ProfScope ps(MO_K_SVD_PANEL, s, static_cast<double>(cnt) * tr * (tr + 1) / 2 * 16.0);
      if ((rc = checked(launch_svd_trd_panel(t, j + 1, s), s, "svd panel"))) return rc;
      k0 = j;
    }
    const double tr = m - (j + 1);
    ProfScope ps(MO_K_SVD_REDUCE, s, static_cast<double>(cnt) * tr * (tr + 1) / 2 * 8.0);
    if ((rc = checked(launch_svd_trd_pass(t, j, j - k0, s), s, "svd reduce"))) return rc;
  }
  // 3. eigenvalues, 4. entropy and singular values
  {
    SvdEigArgs ea{t.d, t.e, lam, m};
    ProfScope ps(MO_K_SVD_EIG, s, static_cast<double>(cnt) * m * m);
    if ((rc = checked(launch_svd_eig(ea, cnt, s), s, "svd eigenvalues"))) return rc;
  }
  for (int f = 0; f < cnt; f += kSvdOutBatch) {
    SvdOutArgs o{};
    o.lam = lam;
    o.entropy = entropy;
    o.sigma = sigma;
    o.first = f;
    o.m = m;
    const int c = std::min(kSvdOutBatch, cnt - f);
    for (int i = 0; i < c; ++i) {
      o.out_index[i] = items[b + f + i].idx;
      o.sigma_off[i] = items[b + f + i].sigma_off;
    }
    ProfScope ps(MO_K_SVD_EIG, s, 0.0);
    if ((rc = checked(launch_svd_out(o, c, s), s, "svd entropy"))) return rc;
  }
  return MO_OK;
}

}  // namespace

extern "C" {

int mo_svd_entropy_workspace_size(const mo_matrix* mats, int64_t count, size_t* full_bytes, size_t* min_bytes) {
  int rc;
  if (!full_bytes) return fail(MO_EINVAL, "full_bytes is NULL");
  std::vector<SvdItem> items;
  int64_t total = 0;
  if ((rc = svd_validate(mats, count, MO_F32, items, &total))) return rc;
  size_t f = 0, mn = 0;
  svd_sizes(items, &f, &mn);
  *full_bytes = f;
  if (min_bytes) *min_bytes = mn;
  return MO_OK;
}

int mo_svd_entropy(const mo_matrix* mats, int64_t count, int dtype, double* entropy, double* sigma, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int rc;
  std::vector<SvdItem> items;
  int64_t total = 0;
  if ((rc = svd_validate(mats, count, dtype, items, &total))) return rc;
  if (count == 0) return MO_OK;
  if (!entropy) return fail(MO_EINVAL, "entropy is NULL");
  if ((reinterpret_cast<uintptr_t>(entropy) & 7u) || (reinterpret_cast<uintptr_t>(sigma) & 7u))
    return fail(MO_EINVAL, "entropy and sigma must be 8-byte aligned");
  size_t full = 0, mn = 0;
  svd_sizes(items, &full, &mn);
  if ((rc = check_workspace(workspace, workspace_bytes, mn))) return rc;
  // outputs may not overlap each other, an input or the workspace
  const int64_t esz = dtype == MO_F32 ? 4 : 2;
  auto overlap = [](const void* a, size_t na, const void* b, size_t nb2) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na && nb2 && x < y + nb2 && y < x + na;
  };
  const size_t ent_bytes = static_cast<size_t>(count) * sizeof(double);
  const size_t sig_bytes = sigma ? static_cast<size_t>(total) * sizeof(double) : 0;
  if (overlap(entropy, ent_bytes, sigma, sig_bytes)) return fail(MO_EINVAL, "entropy and sigma overlap");
  if (overlap(entropy, ent_bytes, workspace, workspace_bytes) || overlap(sigma, sig_bytes, workspace, workspace_bytes))
    return fail(MO_EINVAL, "an output overlaps the workspace");
  for (const SvdItem& it : items) {
    const size_t nbytes = static_cast<size_t>(it.rows * it.cols * esz);
    if (overlap(entropy, ent_bytes, it.data, nbytes) || overlap(sigma, sig_bytes, it.data, nbytes))
      return fail(MO_EINVAL, "an output overlaps matrix %lld", static_cast<long long>(it.idx));
    if (overlap(workspace, workspace_bytes, it.data, nbytes))
      return fail(MO_EINVAL, "the workspace overlaps matrix %lld", static_cast<long long>(it.idx));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  for (size_t g = 0; g < items.size();) {
    size_t h = g;
    while (h < items.size() && items[h].m == items[g].m) ++h;
    // largest chunk that fits (the minimum size guarantees one matrix)
    int64_t cap = std::min<int64_t>(static_cast<int64_t>(h - g), 65535);
    while (cap > 1 && svd_chunk_bytes(items[g].m, cap) > workspace_bytes) {
      const int64_t lo = static_cast<int64_t>(workspace_bytes / svd_chunk_bytes(items[g].m, 1));
      cap = std::max<int64_t>(1, std::min(cap - 1, lo));
    }
    for (size_t c = g; c < h; c += static_cast<size_t>(cap)) {
      const size_t e = std::min(h, c + static_cast<size_t>(cap));
      if ((rc = svd_chunk(items, c, e, dtype, entropy, sigma, ws, s))) return rc;
    }
    g = h;
  }
  return MO_OK;
}

}  // extern "C"
