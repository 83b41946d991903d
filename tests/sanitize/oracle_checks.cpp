// The oracle run under AddressSanitizer and UndefinedBehaviorSanitizer on
// small seeded inputs and on the edge cases (empty inputs, repeated and
// out-of-range coordinates, negative coordinates, capacities smaller than the
// result), checking identities that hold for any input along the way:
//   * forward, dgrad and wgrad are adjoint: <y, g> = <x, dgrad(g)> = <w, wgrad(x, g)>;
//   * a submanifold relation pairs (i, j, o) with (j, i, kvol-1-o);
//   * the transposed relation of a stride-s map is the strided relation with
//     input and output swapped;
//   * generated and strided supports hold distinct coordinates.
// Exit status 0 when every identity holds; a sanitizer report aborts.
#include "../../oracle/oracle.cpp"

#include <algorithm>
#include <cstdio>
#include <set>
#include <tuple>

static int g_fail = 0;
#define EXPECT(cond)                                                                  \
  do {                                                                                \
    if (!(cond)) {                                                                    \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                                       \
    }                                                                                 \
  } while (0)

struct Rng {
  uint64_t s;
  explicit Rng(uint64_t seed) : s(seed * 0x9E3779B97F4A7C15ull + 1) {}
  uint32_t next() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return static_cast<uint32_t>(s >> 33);
  }
  int32_t range(int32_t lo, int32_t hi) { return lo + static_cast<int32_t>(next() % static_cast<uint32_t>(hi - lo + 1)); }
  double unit() { return (next() >> 8) * (1.0 / 8388608.0) - 1.0; }
};

// n rows (batch, x, y[, z]) in a small box so that neighbours exist; a few rows
// repeat an earlier coordinate and, with `bad`, a few leave the range.
static std::vector<int32_t> coords(Rng& r, int64_t n, int ndim, int lo, int hi, bool bad) {
  std::vector<int32_t> c(static_cast<size_t>(n) * (ndim + 1));
  for (int64_t i = 0; i < n; ++i) {
    int32_t* row = &c[static_cast<size_t>(i) * (ndim + 1)];
    row[0] = r.range(0, 1);
    for (int d = 1; d <= ndim; ++d) row[d] = r.range(lo, hi);
    if (i > 4 && r.next() % 9 == 0) std::copy(row - (ndim + 1) * 3, row - (ndim + 1) * 2, row);
    if (bad && r.next() % 13 == 0) row[1 + r.next() % ndim] = (r.next() & 1) ? 40000 : -40000;
    if (bad && r.next() % 29 == 0) row[0] = -1;
  }
  return c;
}

static std::vector<double> values(Rng& r, size_t n) {
  std::vector<double> v(n);
  for (auto& x : v) x = r.unit();
  return v;
}

static double dot(const std::vector<double>& a, const std::vector<double>& b) {
  double s = 0;
  for (size_t k = 0; k < a.size(); ++k) s += a[k] * b[k];
  return s;
}

struct Rel {
  std::vector<int32_t> in, out, off;
};

static Rel kmap(const std::vector<int32_t>& ci, int64_t n_in, const std::vector<int32_t>& co, int64_t n_out, int ndim,
                int ks, int s, int target) {
  const int kvol = ipow(ks, ndim);
  const int64_t cap = std::max<int64_t>(1, n_out * kvol);
  Rel r;
  r.in.resize(cap);
  r.out.resize(cap);
  r.off.resize(cap);
  const int64_t n = oracle_kmap(ci.data(), n_in, co.data(), n_out, ndim, ks, s, target, r.in.data(), r.out.data(),
                                r.off.data(), cap);
  EXPECT(n <= cap);
  r.in.resize(n);
  r.out.resize(n);
  r.off.resize(n);
  return r;
}

static void adjoint(Rng& rng, const Rel& r, int64_t n_in, int64_t n_out, int kvol, int cin, int cout) {
  const auto x = values(rng, static_cast<size_t>(n_in) * cin);
  const auto w = values(rng, static_cast<size_t>(kvol) * cin * cout);
  const auto g = values(rng, static_cast<size_t>(n_out) * cout);
  std::vector<double> y(static_cast<size_t>(n_out) * cout), dx(x.size()), dw(w.size());
  const int64_t np = static_cast<int64_t>(r.in.size());
  oracle_conv_fwd(r.in.data(), r.out.data(), r.off.data(), np, x.data(), cin, w.data(), cout, y.data(), n_out);
  oracle_conv_dgrad(r.in.data(), r.out.data(), r.off.data(), np, g.data(), cout, w.data(), cin, dx.data(), n_in);
  oracle_conv_wgrad(r.in.data(), r.out.data(), r.off.data(), np, x.data(), cin, g.data(), cout, dw.data(), kvol);
  const double a = dot(y, g), b = dot(x, dx), c = dot(w, dw);
  const double tol = 1e-9 * (1.0 + std::fabs(a));
  EXPECT(std::fabs(a - b) <= tol);
  EXPECT(std::fabs(a - c) <= tol);
  // pooling and graph convolution over the same relation
  std::vector<double> p(static_cast<size_t>(n_out) * cin);
  oracle_pool(r.in.data(), r.out.data(), np, x.data(), cin, 0, p.data(), n_out);
  oracle_pool(r.in.data(), r.out.data(), np, x.data(), cin, 1, p.data(), n_out);
  // CSR by output row: sparse convolution is graph convolution with
  // edges = triples and relations = offsets
  std::vector<int64_t> indptr(static_cast<size_t>(n_out) + 1, 0);
  for (int64_t k = 0; k < np; ++k) ++indptr[static_cast<size_t>(r.out[k]) + 1];
  for (int64_t j = 0; j < n_out; ++j) indptr[j + 1] += indptr[j];
  std::vector<int64_t> fill(indptr.begin(), indptr.end() - 1);
  std::vector<int32_t> src(static_cast<size_t>(np)), rel(static_cast<size_t>(np));
  for (int64_t k = 0; k < np; ++k) {
    const int64_t e = fill[r.out[k]]++;
    src[e] = r.in[k];
    rel[e] = r.off[k];
  }
  std::vector<double> yg(y.size());
  oracle_graph_conv(indptr.data(), src.data(), rel.data(), n_out, x.data(), cin, w.data(), cout, yg.data());
  for (size_t k = 0; k < y.size(); ++k) EXPECT(std::fabs(y[k] - yg[k]) <= 1e-12 * (1.0 + std::fabs(y[k])));
}

static void distinct(const std::vector<int32_t>& c, int64_t n, int ndim) {
  std::set<std::vector<int32_t>> s;
  for (int64_t i = 0; i < n; ++i) s.emplace(c.begin() + i * (ndim + 1), c.begin() + (i + 1) * (ndim + 1));
  EXPECT(static_cast<int64_t>(s.size()) == n);
}

static void one_case(uint64_t seed, int64_t n, int ndim, int ks) {
  Rng rng(seed);
  const int kvol = ipow(ks, ndim);
  auto c = coords(rng, n, ndim, -6, 6, true);
  // hash query: every row finds the lowest row of its coordinate, or -1
  std::vector<int32_t> rows(static_cast<size_t>(std::max<int64_t>(n, 1)));
  uint32_t flags = 0;
  oracle_hash_query(c.data(), n, ndim, c.data(), n, rows.data(), &flags);
  for (int64_t i = 0; i < n; ++i) EXPECT(rows[i] <= i);
  // submanifold relation and its mirror symmetry
  Rel sub = kmap(c, n, c, n, ndim, ks, 1, 0);
  std::set<std::tuple<int32_t, int32_t, int32_t>> t;
  for (size_t k = 0; k < sub.in.size(); ++k) t.emplace(sub.in[k], sub.out[k], sub.off[k]);
  if (ks & 1)  // an odd kernel is centred, so its offsets pair up
    for (size_t k = 0; k < sub.in.size(); ++k) EXPECT(t.count({sub.out[k], sub.in[k], kvol - 1 - sub.off[k]}) == 1);
  adjoint(rng, sub, n, n, kvol, 3, 5);
  // strided support, relation and its transposed reading
  std::vector<int32_t> so(static_cast<size_t>(std::max<int64_t>(n, 1)) * (ndim + 1));
  const int64_t n_s = oracle_strided_support(c.data(), n, ndim, 2, so.data());
  EXPECT(n_s <= n);
  distinct(so, n_s, ndim);
  Rel st = kmap(c, n, so, n_s, ndim, 2, 2, 0);
  adjoint(rng, st, n, n_s, ipow(2, ndim), 4, 2);
  {
    const int64_t cap = std::max<int64_t>(1, n * ipow(2, ndim));
    Rel tr;
    tr.in.resize(cap);
    tr.out.resize(cap);
    tr.off.resize(cap);
    const int64_t nt = oracle_kmap_transposed(so.data(), n_s, c.data(), n, ndim, 2, 2, tr.in.data(), tr.out.data(),
                                              tr.off.data(), cap);
    std::set<std::tuple<int32_t, int32_t, int32_t>> a, b;
    for (size_t k = 0; k < st.in.size(); ++k) a.emplace(st.out[k], st.in[k], st.off[k]);
    for (int64_t k = 0; k < std::min(nt, cap); ++k) b.emplace(tr.in[k], tr.out[k], tr.off[k]);
    EXPECT(a == b);
  }
  // generative support, once with a capacity below the site count
  const int64_t gcap = std::max<int64_t>(1, n * kvol);
  std::vector<int32_t> go(static_cast<size_t>(gcap) * (ndim + 1));
  const int64_t n_g = oracle_generative_support(c.data(), n, ndim, ks, go.data(), gcap);
  EXPECT(n_g <= gcap);
  distinct(go, n_g, ndim);
  std::vector<int32_t> go_small(static_cast<size_t>(3) * (ndim + 1));
  EXPECT(oracle_generative_support(c.data(), n, ndim, ks, go_small.data(), 3) == n_g);
  Rel tg = kmap(c, n, go, n_g, ndim, ks, 1, 1);
  adjoint(rng, tg, n, n_g, kvol, 2, 3);
  // transposed support
  const int64_t tcap = std::max<int64_t>(1, n * ipow(2, ndim));
  std::vector<int32_t> to(static_cast<size_t>(tcap) * (ndim + 1));
  const int64_t n_t = oracle_transposed_support(so.data(), n_s, ndim, 2, 2, to.data(), tcap);
  EXPECT(n_t <= tcap);
  distinct(to, n_t, ndim);
  // voxelization: points in and out of range, with and without a batch
  std::vector<float> pos(static_cast<size_t>(n) * ndim);
  std::vector<int32_t> batch(static_cast<size_t>(n));
  for (int64_t i = 0; i < n; ++i) {
    batch[i] = rng.range(0, 2);
    for (int d = 0; d < ndim; ++d) pos[i * ndim + d] = static_cast<float>(rng.unit() * (i % 17 == 3 ? 1e6 : 2.0));
  }
  const float size[3] = {0.25f, 0.5f, 0.125f}, origin[3] = {-0.5f, 0.f, 0.25f};
  const auto f = values(rng, static_cast<size_t>(n) * 2);
  std::vector<int32_t> vc(static_cast<size_t>(std::max<int64_t>(n, 1)) * (ndim + 1)), vof(static_cast<size_t>(std::max<int64_t>(n, 1)));
  std::vector<double> vf(static_cast<size_t>(std::max<int64_t>(n, 1)) * 2);
  for (int with_batch = 0; with_batch < 2; ++with_batch) {
    const int64_t nv = oracle_voxelize(with_batch ? batch.data() : nullptr, pos.data(), n, ndim, size, origin, f.data(),
                                       2, vc.data(), vof.data(), vf.data());
    EXPECT(nv <= n);
    distinct(vc, nv, ndim);
    for (int64_t i = 0; i < n; ++i) EXPECT(vof[i] >= -1 && vof[i] < nv);
  }
}

int main() {
  // empty inputs
  one_case(1, 0, 3, 3);
  one_case(2, 0, 2, 3);
  // one row, two rows
  one_case(3, 1, 3, 3);
  one_case(4, 2, 2, 5);
  // small seeded clouds with repeats, out-of-range rows and negative coordinates
  for (uint64_t s = 10; s < 16; ++s) one_case(s, 40 + 23 * static_cast<int64_t>(s), 3, (s & 1) ? 3 : 1);
  for (uint64_t s = 20; s < 24; ++s) one_case(s, 60 + 11 * static_cast<int64_t>(s), 2, (s & 1) ? 5 : 3);
  one_case(30, 300, 3, 4);  // even kernel as a target map
  if (g_fail) std::fprintf(stderr, "%d expectation(s) failed\n", g_fail);
  else std::printf("oracle checks: all passed\n");
  return g_fail ? 1 : 0;
}
