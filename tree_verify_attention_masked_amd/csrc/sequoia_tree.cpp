// Sequoia tree construction (host code, no GPU): the draft-tree shape of a
// given size and depth bound that maximises the expected number of tokens one
// verification step generates, by dynamic programming ("Sequoia: Scalable and
// Robust Speculative Decoding" summary, "Scalable Speculative Decoding" and
// "Dynamic Programming"; the objective and recurrence are those of the
// published Sequoia paper, which the summary names without stating them).
//
// Positional acceptance: the k-th child of an accepted node (in the order the
// verifier tries siblings) is the accepted one with probability p_k.  A node is
// accepted with the product of p_rank along its path, and a tree T generates
// F(T) = sum of those products (root: 1) tokens in expectation.
//   c(m, d) = best F over trees of m nodes, depth <= d:  c(1, d) = 1,
//             c(m > 1, 0) infeasible, c(m, d) = 1 + g(m - 1, 1, d - 1);
//   g(m, k, e) = best split of m nodes over children of ranks k, k+1, ...
//             with subtrees of depth <= e: g(0, k, e) = 0,
//             g(m, k, e) = max_{a=1..m} p_k c(a, e) + g(m - a, k + 1, e),
//             and g(m, k, e) = 0 for ranks past the vector (p = 0).
// Ties keep the smallest subtree for the lower rank.  The tree comes out
// numbered breadth first with siblings in rank order.
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <deque>
#include <vector>

#include "spectree.h"

namespace {

constexpr int kMaxTreeNodes = 4096;
constexpr double kMaxEntries = 16.0 * 1024 * 1024;    // 12 bytes each: about 200 MB of tables at most
constexpr double kMaxSteps = 4.0 * 1024 * 1024 * 1024;  // a few seconds of one host core at most

struct SequoiaTables {
  int n, D, K;  // nodes, depth bound, ranks that carry probability (<= n - 1)
  std::vector<double> c;      // [(D + 1) * (n + 1)], NaN = infeasible
  std::vector<double> g;      // [D * (K + 2) * (n + 1)] for e < D
  std::vector<int32_t> pick;  // same shape: rank k's subtree size
  double& C(int m, int d) { return c[static_cast<size_t>(d) * (n + 1) + m]; }
  size_t gi(int m, int k, int e) const { return (static_cast<size_t>(e) * (K + 2) + k) * (n + 1) + m; }
};

#pragma clang fp contract(off)
// Fills every c(m, d) for m <= n, d <= D and the g tables they need.
void fill_tables(SequoiaTables& t, const double* p) {
  const int n = t.n, D = t.D, K = t.K;
  const double none = std::nan("");
  t.c.assign(static_cast<size_t>(D + 1) * (n + 1), none);
  t.g.assign(static_cast<size_t>(std::max(D, 1)) * (K + 2) * (n + 1), none);
  t.pick.assign(t.g.size(), 0);
  for (int d = 0; d <= D; ++d) {
    t.C(1, d) = 1.0;
    if (d >= 1)
      for (int m = 2; m <= n; ++m) {
        const double rest = t.g[t.gi(m - 1, 1, d - 1)];
        if (!std::isnan(rest)) t.C(m, d) = 1.0 + rest;
      }
    if (d == D) break;
    const int e = d;  // g at child depth bound e uses c(., e), complete now
    for (int m = 0; m <= n; ++m) {  // ranks past the vector: m leaves, nothing added
      t.g[t.gi(m, K + 1, e)] = 0.0;
      t.pick[t.gi(m, K + 1, e)] = m > 0 ? 1 : 0;
    }
    for (int k = K; k >= 1; --k) {
      t.g[t.gi(0, k, e)] = 0.0;
      for (int m = 1; m <= n; ++m) {
        double best = none;
        int best_a = 0;
        for (int a = 1; a <= m; ++a) {
          const double sub = t.C(a, e);
          const double tail = t.g[t.gi(m - a, k + 1, e)];
          if (std::isnan(sub) || std::isnan(tail)) continue;
          const double prod = p[k - 1] * sub;
          const double v = prod + tail;
          if (std::isnan(best) || v > best) {
            best = v;
            best_a = a;
          }
        }
        t.g[t.gi(m, k, e)] = best;
        t.pick[t.gi(m, k, e)] = best_a;
      }
    }
  }
}
#pragma clang fp contract(on)

}  // namespace

extern "C" int spec_sequoia_tree(const double* accept, int K, int n, int max_depth, int32_t* parent,
                                 double* expected) {
  if (n < 1 || K < 0 || max_depth < 0 || parent == nullptr || (K > 0 && accept == nullptr))
    return SPEC_ERR_INVALID_ARG;
  if (n > kMaxTreeNodes) return SPEC_ERR_UNSUPPORTED;
  for (int k = 0; k < K; ++k)
    if (!(accept[k] >= 0.0 && accept[k] <= 1.0)) return SPEC_ERR_INVALID_ARG;
  if (n > 1 && max_depth == 0) return SPEC_ERR_INVALID_ARG;  // no tree of that size fits
  SequoiaTables t;
  t.n = n;
  t.D = std::min(max_depth, n - 1);  // a deeper bound changes nothing
  t.K = std::min(K, std::max(n - 1, 0));
  // table entries and inner-loop steps: about D (K + 2) n and D K n^2 / 2
  const double entries = static_cast<double>(std::max(t.D, 1)) * (t.K + 2) * (n + 1);
  const double steps = static_cast<double>(t.D) * t.K * n * (n + 1) / 2.0;
  if (entries > kMaxEntries || steps > kMaxSteps) return SPEC_ERR_UNSUPPORTED;
  fill_tables(t, accept);
  const double value = t.C(n, t.D);
  if (std::isnan(value)) return SPEC_ERR_INVALID_ARG;
  // rebuild breadth first: (node, subtree size, depth bound)
  struct Item {
    int node, m, d;
  };
  std::deque<Item> queue{{0, n, t.D}};
  int next = 1;
  parent[0] = -1;
  while (!queue.empty()) {
    const Item it = queue.front();
    queue.pop_front();
    int left = it.m - 1, k = 1;
    while (left > 0) {
      const int a = t.pick[t.gi(left, std::min(k, t.K + 1), it.d - 1)];
      parent[next] = it.node;
      queue.push_back({next, a, it.d - 1});
      ++next;
      left -= a;
      ++k;
    }
  }
  if (expected != nullptr) *expected = value;
  return SPEC_OK;
}
