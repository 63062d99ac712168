// Schedule of the blocked inverse factor (host code, no HIP types).
//
// The same factor as the recursion in prep.hip (page "量化", section GPTQ, Cholesky
// reformulation: A = H + lambda I = U U^T with U upper, G = U^-1), taken in 128-column
// blocks from the bottom right.  For block k (columns [c_k, c_{k+1})):
//   leaf    A_kk -> G_kk = U_kk^-1                                   (one workgroup)
//   panel   U[0:c_k, k] = A[0:c_k, k] G_kk^T, into a scratch matrix at U's own place
//   column  A[0:c_k, k-1] -= U[0:c_k, k] U[k-1, k]^T                (next block's column)
//   rest    A[0:c_{k-1}, 0:c_{k-1}] -= U[0:c_{k-1}, k] U[0:c_{k-1}, k]^T (upper triangle)
// G's blocks above the diagonal come from a binary tree over the block range: a node
// [a, b) split at m, once its right half is complete, forms Q = U[a:m, m:b] G[m:b, m:b],
// and once its left half is complete, G[a:m, m:b] = -G[a:m, a:m] Q, written over entries of
// A that the panels of blocks m..b-1 have consumed.
//
// Everything runs on the caller's stream, three launches per block.  The leaf of block k is
// one workgroup of a launch whose other workgroups run 64 x 64 tiles of the trailing update
// of block k + 1 and of the tree products whose inputs earlier launches completed (large
// products spread over several launches), so that the one-CU leaf does not leave the chip
// idle; then the panel and the column update.  The parts of one launch touch disjoint
// entries.  Every product has the operand forms of the recursion's (op(A) = A; op(B) = B or
// B^T; triangular masks on G blocks; an upper-only output).
//
// When the block is the left half A11 of a recursion node whose right half (r columns) is
// already factored, the schedule can also carry that node's Q = P G22 (P = A12 G22^T, n x r;
// G22 the r x r upper factor right below and right of the block), which the node needs only
// after this block: its tiles run beside the leaves, split along K into chunks that start on
// G22's diagonal, Q[:, k0:r] += P[:, k0:k0+kc] G22[k0:k0+kc, k0:r] (upper again from its own
// corner), each chunk in a later launch than the one before.
//
// Operations are described by offsets into five buffers: 0 the matrix (upper triangle A,
// then G; row-major with leading dimension ld, offsets from the block's top-left corner),
// 1 the n x n scratch matrix of U's blocks above the diagonal (leading dimension n), 2 the
// Q scratch of the tree (one region per tree node), 3 the node's P and 4 its Q (n x r,
// leading dimension r).
#pragma once

#include <stdint.h>

#include <climits>

#include <vector>

namespace gptq {
namespace plan {

constexpr int64_t PB = 128;   // block size (the leaf size)

struct Mat { int buf; int64_t off, ld; };
struct Gemm {
  int64_t M, N, K;
  Mat A; int transA, triA;
  Mat B; int transB, triB;
  Mat C; int triC;
  float alpha, beta;
};
constexpr int FUSED_TASKS = 6;          // products beside the leaf in one launch
constexpr int64_t TREE_BUDGET = 1 << 19; // tree tiles x K per launch (512 tiles of K 1024)
constexpr int64_t NODE_Q_K = 512;        // k per chunk of the parent node's Q
constexpr int64_t NODE_Q_TILES = 192;    // its tiles per launch beside a leaf

enum Kind { FUSED = 0, GEMM = 1 };
struct Task {
  Gemm g;
  int64_t t0, t1;       // the 64 x 64 tiles [t0, t1) of the product, in the GEMM's tile order
};
struct Op {
  int kind;             // FUSED: the leaf (if n > 0) and up to FUSED_TASKS tile ranges in
                        // one launch; GEMM: one whole product by the GEMM dispatcher
  int64_t off, n;       // the leaf: diagonal offset and size of the block (n = 0: none)
  std::vector<Task> t;
};

struct Plan {
  int64_t n, ld, nb, r;   // r: columns of the parent node's Q carried along (0: none)
  int64_t panel_floats; // buffer 1 (n * n)
  int64_t q_floats;     // buffer 2
  std::vector<Op> ops;
};

inline int64_t col_of(int64_t n, int64_t k) { return k * PB < n ? k * PB : n; }
inline int64_t up64(int64_t x) { return (x + 63) / 64 * 64; }
inline int64_t tiles_of(const Gemm& g) { return ((g.M + 63) / 64) * ((g.N + 63) / 64); }

struct Node { int64_t a, m, b, q_off; };

// Binary tree over blocks [a, b): a node splits at its midpoint; single blocks are leaves
// (not stored).  Q offsets are assigned in creation order; `q_total` gets the scratch size.
inline void build_tree(int64_t n, int64_t a, int64_t b, std::vector<Node>& out, int64_t& q_total) {
  if (b - a < 2) return;
  const int64_t m = a + (b - a) / 2;
  const int64_t rows = col_of(n, m) - col_of(n, a), cols = col_of(n, b) - col_of(n, m);
  out.push_back(Node{a, m, b, q_total});
  q_total += up64(rows * cols);
  build_tree(n, a, m, out, q_total);
  build_tree(n, m, b, out, q_total);
}

inline Mat matA(int64_t ld, int64_t r, int64_t c) { return Mat{0, r * ld + c, ld}; }

inline Plan blocked_plan(int64_t n, int64_t ld, int64_t r = 0) {
  Plan p;
  p.n = n;
  p.ld = ld;
  p.r = r;
  p.nb = (n + PB - 1) / PB;
  const int64_t nb = p.nb;
  auto col = [&](int64_t k) { return col_of(n, k); };
  p.panel_floats = n * n;
  std::vector<Node> tree;
  int64_t q_total = 0;
  build_tree(n, 0, nb, tree, q_total);
  p.q_floats = q_total;
  const int nt = (int)tree.size();
  const int nq = r > 0 ? (int)((r + NODE_Q_K - 1) / NODE_Q_K) : 0;   // chunks of the node's Q
  const int ns = 2 * nt + nq;                                        // steps off the chain

  // Positions of the chain's launches: for k = nb-1 .. 0 the fused launch of leaf k, then
  // (k > 0) the panel and the column update.
  auto pos_leaf = [&](int64_t k) { return 3 * (nb - 1 - k); };
  auto pos_panel = [&](int64_t k) { return 3 * (nb - 1 - k) + 1; };

  // Tree steps: 2 t (Q of node t) and 2 t + 1 (G block of node t), each done in chunks of
  // 64 x 64 tiles.  A step may start in a launch after the one that completes its inputs:
  // the leaves and panels of its half (`after`) and the G steps of the nodes inside that half.
  std::vector<Gemm> step(ns);
  std::vector<std::vector<int>> deps(ns);
  std::vector<int64_t> after(ns, -1);
  for (int t = 0; t < nt; ++t) {
    const Node& x = tree[t];
    const int64_t ca = col(x.a), cm = col(x.m), cb = col(x.b);
    Gemm q{};
    q.M = cm - ca; q.N = cb - cm; q.K = cb - cm;
    q.A = Mat{1, ca * n + cm, n};                      // U[a:m, m:b]
    q.B = matA(ld, cm, cm); q.triB = 1;                // G[m:b, m:b], upper
    q.C = Mat{2, x.q_off, cb - cm};
    q.alpha = 1.0f; q.beta = 0.0f;
    Gemm g{};
    g.M = cm - ca; g.N = cb - cm; g.K = cm - ca;
    g.A = matA(ld, ca, ca); g.triA = 1;                // G[a:m, a:m], upper
    g.B = Mat{2, x.q_off, cb - cm};
    g.C = matA(ld, ca, cm);
    g.alpha = -1.0f; g.beta = 0.0f;
    step[2 * t] = q;
    step[2 * t + 1] = g;
    after[2 * t] = pos_panel(x.m);                     // leaf m, then panel m: the last of [m, b)
    after[2 * t + 1] = pos_leaf(x.a);                  // leaf a: the last of [a, m)
    deps[2 * t + 1].push_back(2 * t);
    for (int u = 0; u < nt; ++u) {
      if (u == t) continue;
      const Node& y = tree[u];
      if (y.a >= x.m && y.b <= x.b) deps[2 * t].push_back(2 * u + 1);
      if (y.a >= x.a && y.b <= x.m) deps[2 * t + 1].push_back(2 * u + 1);
    }
  }
  for (int c = 0; c < nq; ++c) {                     // the node's Q, chunk by chunk
    const int64_t k0 = c * NODE_Q_K, kc = r - k0 < NODE_Q_K ? r - k0 : NODE_Q_K;
    Gemm q{};
    q.M = n; q.N = r - k0; q.K = kc;                   // Q[:, k0:r] (+)= P[:, k0:k0+kc] G22[..]
    q.A = Mat{3, k0, r};
    q.B = matA(ld, n + k0, n + k0); q.triB = 1;        // G22 from its diagonal entry (k0, k0)
    q.C = Mat{4, k0, r};
    q.alpha = 1.0f; q.beta = c == 0 ? 0.0f : 1.0f;
    step[2 * nt + c] = q;
    if (c > 0) deps[2 * nt + c].push_back(2 * nt + c - 1);
  }
  std::vector<int64_t> done_at(ns, -1);               // launch holding each step's last tiles
  std::vector<int64_t> next_tile(ns, 0);
  int64_t n_left = ns;
  // Tiles of ready steps for the launch at `pos`, within the budget (none: no limit).
  auto take_ready = [&](int64_t pos, int room, int64_t budget, std::vector<Task>& out) {
    int64_t q_room = budget > 0 ? NODE_Q_TILES : INT64_MAX;   // the node's Q: a budget of its own
    for (int s = 0; s < ns && room > 0; ++s) {
      if (done_at[s] >= 0 || after[s] >= pos) continue;
      bool ok = true;
      for (int d : deps[s])
        if (done_at[d] < 0 || done_at[d] >= pos) { ok = false; break; }
      if (!ok) continue;
      const int64_t total = tiles_of(step[s]);
      const int64_t k = step[s].K > 0 ? step[s].K : 1;
      int64_t cnt = total - next_tile[s];
      if (s >= 2 * nt) {
        if (q_room <= 0) continue;
        if (cnt > q_room) cnt = q_room;
        q_room -= cnt;
      } else if (budget > 0) {
        const int64_t fit = budget / k;
        if (fit <= 0) break;
        if (cnt > fit) cnt = fit;
        budget -= cnt * k;
      }
      out.push_back(Task{step[s], next_tile[s], next_tile[s] + cnt});
      next_tile[s] += cnt;
      if (next_tile[s] == total) {
        done_at[s] = pos;
        --n_left;
      }
      --room;
    }
  };

  int64_t pos = 0;
  for (int64_t k = nb - 1; k >= 0; --k) {
    const int64_t ck = col(k), nk = col(k + 1) - ck;
    Op f{};
    f.kind = FUSED;
    f.off = ck;
    f.n = nk;
    if (k + 1 <= nb - 1 && k + 1 >= 2) {               // rest of block k + 1
      const int64_t c1 = col(k + 1), n1 = col(k + 2) - c1;
      Gemm r{};
      r.M = ck; r.N = ck; r.K = n1;                    // A[0:c_k, 0:c_k] -= U U^T
      r.A = Mat{1, c1, n};
      r.B = Mat{1, c1, n}; r.transB = 1;
      r.C = matA(ld, 0, 0); r.triC = 1;
      r.alpha = -1.0f; r.beta = 1.0f;
      f.t.push_back(Task{r, 0, tiles_of(r)});
    }
    take_ready(pos, FUSED_TASKS - (int)f.t.size(), TREE_BUDGET, f.t);
    p.ops.push_back(f);
    ++pos;
    if (k > 0) {
      const int64_t cp = col(k - 1);
      Op u{};
      u.kind = GEMM;
      Gemm g{};
      g.M = ck; g.N = nk; g.K = nk;                    // U[0:c_k, k] = A[0:c_k, k] G_kk^T
      g.A = matA(ld, 0, ck);
      g.B = matA(ld, ck, ck); g.transB = 1; g.triB = 2;
      g.C = Mat{1, ck, n};
      g.alpha = 1.0f; g.beta = 0.0f;
      u.t.push_back(Task{g, 0, tiles_of(g)});
      p.ops.push_back(u);
      ++pos;
      Op c{};
      c.kind = GEMM;
      Gemm h{};
      h.M = ck; h.N = ck - cp; h.K = nk;               // A[0:c_k, k-1] -= U[:, k] U[k-1, k]^T
      h.A = Mat{1, ck, n};
      h.B = Mat{1, cp * n + ck, n}; h.transB = 1;
      h.C = matA(ld, 0, cp);
      h.alpha = -1.0f; h.beta = 1.0f;
      c.t.push_back(Task{h, 0, tiles_of(h)});
      p.ops.push_back(c);
      ++pos;
    }
  }
  // The tree steps left after the last leaf, a launch per dependency level.
  while (n_left > 0) {
    Op f{};
    f.kind = FUSED;
    f.off = 0;
    f.n = 0;
    take_ready(pos, FUSED_TASKS, 0, f.t);
    if (f.t.empty()) break;                            // unreachable for a well-formed tree
    p.ops.push_back(f);
    ++pos;
  }
  return p;
}

}  // namespace plan
}  // namespace gptq
