// Inverse factor G = Cholesky((H + lambda I)^-1)^T (page "量化", section GPTQ: the
// Cholesky reformulation; damping lambda = frac * mean(diag H) is not on the pages).
//
// G is computed without forming an inverse.  With A = H + lambda I = U U^T, U upper,
// G = U^-1 is upper with G^T G = A^-1 and positive diagonal, hence the same unique
// factor.  A recursion on the 2x2 block split A = [[A11, A12], [A12^T, A22]]:
//     G22 = factor(A22)                     (recursion)
//     P   = A12 G22^T                       (= U12)
//     Q   = P G22,  A11 <- A11 - P P^T      (one launch; Schur complement, upper triangle)
//     G11 = factor(A11)                     (recursion)
//     G12 = -G11 Q                          (written over A12)
// All products run on the fp32 MFMA GEMM; blocks of at most 128 are factored and
// inverted by one workgroup in LDS.  Blocks of 1024 to 2048 columns are factored by the
// blocked schedule of prep_plan.h instead, whose launches run each one-workgroup leaf
// beside the previous block's trailing update and the tree products that form G's
// off-diagonal blocks.  Everything happens in the upper triangle of G; the strictly lower
// triangle is zeroed at the end.

#include <climits>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>
#include <vector>

#include "gemm_tile.h"
#include "gptq_internal.h"
#include "prep_plan.h"

namespace gptq {

namespace {

constexpr int NB = 128;           // leaf size

struct PrepWs {
  double* lambda;
  int* flag;
  float* tmp;
};

PrepWs carve(void* ws, int64_t d) {
  char* p = static_cast<char*>(ws);
  PrepWs w;
  w.lambda = reinterpret_cast<double*>(p);
  w.flag = reinterpret_cast<int*>(p + 8);
  w.tmp = reinterpret_cast<float*>(p + 256);
  return w;
}

// lambda = frac * mean(diag H) in double with a fixed reduction order; flag reset.
__global__ void __launch_bounds__(256)
damp_lambda(const float* __restrict__ H, int64_t d, float frac, double* lambda, int* flag) {
  __shared__ double s[256];
  // thread t adds H_ii for i = t, t + 256, ... in that order; eight loads go out before their
  // additions (the order, and so the sum, is that of one load at a time)
  double acc = 0.0;
  int64_t i = threadIdx.x;
  for (; i + 7 * 256 < d; i += 8 * 256) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = H[(i + 256 * u) * d + i + 256 * u];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += (double)v[u];
  }
  for (; i < d; i += 256) acc += (double)H[i * d + i];
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) s[threadIdx.x] += s[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double mean = s[0] / (double)d;
    *lambda = (double)frac * mean;
    *flag = (mean > 0.0 && mean < 1e300) ? INT_MAX : 1;
  }
}

// Upper triangle of G <- upper triangle of H, diagonal + lambda (safe when G == H).
// Row-wise helpers: rows stride over gridDim.y, columns over gridDim.x * 256.
__global__ void __launch_bounds__(256)
copy_damp(const float* H, float* G, int64_t d, const double* lambda) {
  const float lam = (float)*lambda;
  for (int64_t i = blockIdx.y; i < d; i += gridDim.y)
    for (int64_t j = i + blockIdx.x * 256 + threadIdx.x; j < d; j += (int64_t)gridDim.x * 256) {
      float v = H[i * d + j];
      if (j == i) v += lam;
      G[i * d + j] = v;
    }
}

__global__ void __launch_bounds__(256) zero_lower(float* __restrict__ G, int64_t d) {
  for (int64_t i = blockIdx.y; i < d; i += gridDim.y)
    for (int64_t j = blockIdx.x * 256 + threadIdx.x; j < i; j += (int64_t)gridDim.x * 256)
      G[i * d + j] = 0.0f;
}

// The same two passes with 16-byte accesses (d % 4 == 0, H and G 16-byte aligned): rows
// stride over the workgroups, four columns per thread; the quad that holds the diagonal is
// written element by element, so nothing left of the diagonal (copy) or right of it (zero)
// is touched.
__global__ void __launch_bounds__(256)
copy_damp4(const float* H, float* G, int64_t d, const double* lambda) {
  const float lam = (float)*lambda;
  const int64_t nq = d / 4;
  for (int64_t i = blockIdx.x; i < d; i += gridDim.x) {
    const floatx4* hr = reinterpret_cast<const floatx4*>(H + i * d);
    floatx4* gr = reinterpret_cast<floatx4*>(G + i * d);
    const int64_t qd = i / 4;
    for (int64_t q = qd + threadIdx.x; q < nq; q += 256) {
      const floatx4 v = hr[q];
      if (q == qd) {
        const int k = (int)(i - 4 * qd);   // the diagonal's place in the quad
        float* g = G + i * d + 4 * qd;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (c >= k) g[c] = c == k ? v[c] + lam : v[c];
      } else {
        gr[q] = v;
      }
    }
  }
}

__global__ void __launch_bounds__(256) zero_lower4(float* __restrict__ G, int64_t d) {
  const floatx4 z = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t i = blockIdx.x; i < d; i += gridDim.x) {
    floatx4* gr = reinterpret_cast<floatx4*>(G + i * d);
    const int64_t qd = i / 4;
    for (int64_t q = threadIdx.x; q <= qd; q += 256) {
      if (q < qd) {
        gr[q] = z;
      } else {
        for (int64_t j = 4 * qd; j < i; ++j) G[i * d + j] = 0.0f;
      }
    }
  }
}

dim3 rows_grid(int64_t rows, int64_t cols) {
  const int64_t gx = (cols + 255) / 256;
  return dim3((unsigned)(gx < 1 ? 1 : gx > 64 ? 64 : gx), (unsigned)(rows > 32768 ? 32768 : rows));
}

// Factor the n x n diagonal block at (off, off) (n <= 128) as U U^T (U upper) and
// overwrite its upper triangle with G = U^-1.  One workgroup of 4 waves; the block, padded
// with the identity to 128, lives in LDS as its ten upper 32 x 32 sub-blocks.
//
// Sub-block p = 3, 2, 1, 0 (from the bottom right):
//   diag   one wave factors the 32 x 32 Schur block S_pp and writes G_pp = U_pp^-1;
//   row    G_pr = -G_pp T_pr for r > p, where T_pr = sum_{p<t<=r} U_pt G_tr;
//   panel  U_qp = S_qp G_pp^T for q < p;
//   update T_qp = U_qp G_pp, T_qr += U_qp G_pr (r > p), S_qt -= U_qp U_tp^T (q <= t < p).
// Every product is one 32 x 32 x 32 v_mfma_f32_32x32x2_f32 sequence of one wave; the
// products of a phase are spread over the four waves and phases are separated by
// barriers.  Slot (q, r) holds S_qr, then T_qr, then G_qr; the panel U_qp has slots of
// its own because the update phase reads it while overwriting slot (q, p).
constexpr int LB = 32;              // sub-block
constexpr int LS = LB + 1;          // LDS row stride: rows and columns both conflict-free
constexpr int NLB = NB / LB;        // sub-blocks per side
constexpr int NSLOT = NLB * (NLB + 1) / 2;
constexpr int SLOT = LB * LS;

__device__ __forceinline__ int slot_of(int q, int r) { return q * NLB - q * (q - 1) / 2 + (r - q); }

// C = op(X) op(Y), C += op(X) op(Y) (ACC) or the same with the product negated (NEG),
// for 32 x 32 blocks in LDS, one wave.
//   op(X)[m][k] = TX ? X[k][m] : X[m][k],  op(Y)[k][n] = TY ? Y[n][k] : Y[k][n].
// All operands are read into registers before the first MFMA (one LDS wait per product),
// so C may alias X or Y.
template <bool TX, bool TY, bool ACC, bool NEG>
__device__ __forceinline__ void block_prod(float* C, const float* X, const float* Y, int lane) {
  const int l32 = lane & 31, hi = lane >> 5;
  float a[LB / 2], b[LB / 2], c[16];
#pragma unroll
  for (int kk = 0; kk < LB / 2; ++kk) {
    const int k = 2 * kk + hi;
    a[kk] = TX ? X[k * LS + l32] : X[l32 * LS + k];
    b[kk] = TY ? Y[l32 * LS + k] : Y[k * LS + l32];
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) c[r] = ACC ? C[(8 * (r >> 2) + 4 * hi + (r & 3)) * LS + l32] : 0.0f;
  __builtin_amdgcn_sched_barrier(0);   // keep every read ahead of the MFMA chain
  floatx16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = NEG ? -c[r] : c[r];   // -(-C + XY) = C - XY
#pragma unroll
  for (int kk = 0; kk < LB / 2; ++kk)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[kk], b[kk], acc, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r)
    C[(8 * (r >> 2) + 4 * hi + (r & 3)) * LS + l32] = NEG ? -acc[r] : acc[r];
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
// v of lane (lane % 32) + 32 hs: one half of the wave copied to both.  v_permlane32_swap with
// both operands v returns the low half in both halves of its first result and the high half
// in both halves of its second.
__device__ __forceinline__ float half_bcast(float v, int hs) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, hs ? p[1] : p[0]);
}

// One wave: S (symmetric 32 x 32 at sp, only its upper triangle is read) = U U^T, U upper;
// sp <- G = U^-1 (full block, zeros below the diagonal).  Reverse Gaussian elimination:
// pivot k removes column k from rows i < k of S (rank-1 Schur update) and the same row
// operation is applied to R (starting from I), so that R = L^-1 for S = L D L^T with L
// unit upper; then G = D^-1/2 R.  Pivots are taken in pairs (k, k - 1): with
// beta = S[k][k-1] / S[k][k], column k - 1 after the first update is
// u2 = S[:, k-1] - beta S[:, k] and its pivot S[k-1][k-1] - beta S[k][k-1], so the pair is
// one rank-2 update
//     S -= S[:, k] S[k, :] / p1 + u2 u2^T / p2,   R -= S[:, k] R[k, :] / p1 + u2 R'[k-1, :] / p2
// on rows and columns below k - 1 (R' = row k - 1 of R after the first pivot).  S and R are
// kept in the accumulator layout of v_mfma_f32_32x32x2_f32 (lane (j, h) holds column j,
// rows 8 (c / 4) + 4 h + c % 4 in register c), so each rank-2 update is one MFMA whose
// A operand (32 x 2) and B operand (2 x 32) are built per lane from rows k and k - 1.
// Those two rows sit in one half of the wave; v_permlane32_swap copies them to the other.
// When u is given, the last Schur update S -= U U^T (U = the 32 x 32 block at u) is applied
// in registers first, by the same MFMA sequence as block_prod: its result is symmetric bit for
// bit (entries (i, j) and (j, i) sum the same products in the same order), so the mirrored
// upper triangle plus this update equals updating S in LDS and mirroring afterwards.
// Returns the smallest k < k_valid whose pivot was not positive and finite, else -1.
__device__ int diag_factor(float* sp, const float* u, int lane, int k_valid) {
  const int j = lane & 31, h = lane >> 5;
  floatx16 s, r;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const int i = 8 * (c >> 2) + 4 * h + (c & 3);
    s[c] = i <= j ? sp[i * LS + j] : sp[j * LS + i];
    r[c] = (i == j) ? 1.0f : 0.0f;
  }
  if (u) {
    float uv[LB / 2];
#pragma unroll
    for (int kk = 0; kk < LB / 2; ++kk) uv[kk] = u[j * LS + 2 * kk + h];
#pragma unroll
    for (int kk = 0; kk < LB / 2; ++kk)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(-uv[kk], uv[kk], s, 0, 0, 0);
  }
  floatx16 pv;    // D^-1/2 of the row of register c
  int bad = -1;
#pragma unroll
  for (int t = LB / 2 - 1; t >= 0; --t) {
    const int k = 2 * t + 1;
    const int hs = (t >> 1) & 1;                     // half holding rows k and k - 1
    const int c1 = 4 * (k >> 3) + (k & 3), c2 = c1 - 1;   // their registers
    const float p1 = readlane_f(s[c1], k + 32 * hs);      // S[k][k]
    const float bk = readlane_f(s[c1], k - 1 + 32 * hs);  // S[k][k-1]
    const float p2 = readlane_f(s[c2], k - 1 + 32 * hs);  // S[k-1][k-1]
    const float sk = half_bcast(s[c1], hs), sk1 = half_bcast(s[c2], hs);   // S[k][j], S[k-1][j]
    const float rk = half_bcast(r[c1], hs), rk1 = half_bcast(r[c2], hs);   // R[k][j], R[k-1][j]
    const float rp1 = __builtin_amdgcn_rcpf(p1);
    const float beta = bk * rp1;
    const float p2s = fmaf(-beta, bk, p2);
    const float rp2 = __builtin_amdgcn_rcpf(p2s);
    if (k < k_valid && !(p1 > 0.0f && p1 < 3.0e38f)) bad = k;
    if (k - 1 < k_valid && !(p2s > 0.0f && p2s < 3.0e38f)) bad = k - 1;
    const float rk1n = fmaf(-beta, rk, rk1);          // R'[k-1][j]
    if (h == hs) {
      pv[c1] = __builtin_amdgcn_rsqf(p1);
      pv[c2] = __builtin_amdgcn_rsqf(p2s);
      r[c2] = rk1n;
    }
    if (t == 0) break;
    const float u2 = fmaf(-beta, sk, sk1);
    const bool act = j < k - 1;
    const float a = act ? -(h ? u2 * rp2 : sk * rp1) : 0.0f;   // -A[j][h]
    const float bs = act ? (h ? u2 : sk) : 0.0f;                // B[h][j] for S
    const float br = h ? rk1n : rk;                             // B[h][j] for R
    s = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bs, s, 0, 0, 0);
    r = __builtin_amdgcn_mfma_f32_32x32x2f32(a, br, r, 0, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < 16; ++c) sp[(8 * (c >> 2) + 4 * h + (c & 3)) * LS + j] = r[c] * pv[c];
  return bad;
}

// Load order of the ten upper sub-blocks (row block, column block): the one factored first,
// then the panels it feeds, then the rest.
__host__ __device__ constexpr int unit_q(int e) {
  return e == 0 ? 3 : e == 1 ? 2 : e == 2 ? 1 : e == 3 ? 0 : e == 4 ? 2 : e == 5 ? 1 : e == 6 ? 0
       : e == 7 ? 1 : 0;
}
__host__ __device__ constexpr int unit_r(int e) { return e <= 3 ? 3 : e <= 6 ? 2 : e <= 8 ? 1 : 0; }

// Unit E of this thread into its slot; entries beyond n are the identity.
template <int E>
__device__ __forceinline__ void put_unit(float* slot, const floatx4& v, int rho, int kap, int n) {
  constexpr int q = unit_q(E), r = unit_r(E);
  const int i = LB * q + rho;
  float* d = slot + slot_of(q, r) * SLOT + rho * LS + 4 * kap;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int jj = LB * r + 4 * kap + c;
    d[c] = (i < n && jj < n) ? v[c] : (i == jj ? 1.0f : 0.0f);
  }
}

struct LeafSmem {
  float slot[NSLOT * SLOT];
  float ubuf[(NLB - 1) * SLOT];
  int bad_at;
};

__device__ __forceinline__ void leaf_body(float* __restrict__ A, int64_t ld, int64_t off, int n,
                                          int* flag, LeafSmem& sm) {
  float* slot = sm.slot;
  float* ubuf = sm.ubuf;
  int& bad_at = sm.bad_at;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  float* blk = A + off * ld + off;

  // Load the ten upper sub-blocks: unit e of every thread is row tid / 8, columns 4 (tid % 8)
  // .. +3 of sub-block (unit_q(e), unit_r(e)), all loads issued at once (addresses clamped into the
  // block, then selected; the padding beyond n is the identity).  Sub-block (3, 3) comes
  // first: it is written to LDS before the first barrier so that its factorization starts
  // while the other nine are still in flight; they are written during that iteration.
  const bool vec = ((reinterpret_cast<uintptr_t>(blk) | (uintptr_t)(ld * 4)) & 15) == 0 &&
                   (n & 3) == 0;
  const int rho = tid >> 3, kap = tid & 7;
  floatx4 v[NSLOT];
#pragma unroll
  for (int e = 0; e < NSLOT; ++e) {
    const int i = LB * unit_q(e) + rho, j0 = LB * unit_r(e) + 4 * kap;
    const int ic = i < n ? i : n - 1;
    if (vec) {
      const int jc = j0 < n ? j0 : n - 4;
      v[e] = *reinterpret_cast<const floatx4*>(blk + (ic * (int)ld + jc));
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int jc = j0 + c < n ? j0 + c : n - 1;
        v[e][c] = blk[ic * (int)ld + jc];
      }
    }
  }
  put_unit<0>(slot, v[0], rho, kap, n);
  if (tid == 0) bad_at = INT_MAX;
  __syncthreads();

  // Iteration p: wave 0 applies the last Schur update of S_pp (from the panel of p + 1) and
  // factors it while waves 1-3 run the other update products of p + 1; then all waves form
  // row p of G and the panel of p.
  for (int p = NLB - 1; p >= 0; --p) {
    const float* gpp = slot + slot_of(p, p) * SLOT;
    if (wave == 0) {
      float* spp = slot + slot_of(p, p) * SLOT;
      // S_pp -= U_p U_p^T (from the panel of p + 1), then the factorization
      const int b = diag_factor(spp, p + 1 < NLB ? ubuf + p * SLOT : nullptr, lane, n - LB * p);
      if (b >= 0 && lane == 0) bad_at = min(bad_at, LB * p + b);
    } else if (p + 1 < NLB) {
      const int pp = p + 1;                               // update products of step p + 1
      const float* gq = slot + slot_of(pp, pp) * SLOT;
      int task = 0;
      for (int q = 0; q < pp; ++q) {
        const float* u = ubuf + q * SLOT;
        if (task++ % 3 == wave - 1)                      // T_q,pp = U_q G_pp,pp
          block_prod<false, false, false, false>(slot + slot_of(q, pp) * SLOT, u, gq, lane);
        for (int r = pp + 1; r < NLB; ++r)               // T_qr += U_q G_pp,r
          if (task++ % 3 == wave - 1)
            block_prod<false, false, true, false>(slot + slot_of(q, r) * SLOT, u,
                                                  slot + slot_of(pp, r) * SLOT, lane);
        for (int t = q; t < pp; ++t)                     // S_qt -= U_q U_t^T (but S_pp)
          if (!(q == p && t == p) && task++ % 3 == wave - 1)
            block_prod<false, true, true, true>(slot + slot_of(q, t) * SLOT, u, ubuf + t * SLOT,
                                                lane);
      }
    }
    if (p == NLB - 1) {   // the other nine sub-blocks (wave 0 after its factorization)
      put_unit<1>(slot, v[1], rho, kap, n);
      put_unit<2>(slot, v[2], rho, kap, n);
      put_unit<3>(slot, v[3], rho, kap, n);
      put_unit<4>(slot, v[4], rho, kap, n);
      put_unit<5>(slot, v[5], rho, kap, n);
      put_unit<6>(slot, v[6], rho, kap, n);
      put_unit<7>(slot, v[7], rho, kap, n);
      put_unit<8>(slot, v[8], rho, kap, n);
      put_unit<9>(slot, v[9], rho, kap, n);
    }
    __syncthreads();
    int task = 0;
    for (int r = p + 1; r < NLB; ++r, ++task)            // G_pr = -G_pp T_pr
      if (task % 4 == wave) {
        float* c = slot + slot_of(p, r) * SLOT;
        block_prod<false, false, false, true>(c, gpp, c, lane);
      }
    for (int q = 0; q < p; ++q, ++task)                  // U_qp = S_qp G_pp^T
      if (task % 4 == wave)
        block_prod<false, true, false, false>(ubuf + q * SLOT, slot + slot_of(q, p) * SLOT, gpp,
                                              lane);
    __syncthreads();
    // Row block p of G is final (later iterations only read it): store its sub-blocks
    // (p, r >= p) while the next iterations run.  The sub-blocks left of the diagonal ones
    // are strictly lower entries, which every later product masks and the final pass clears.
#pragma unroll
    for (int r = 0; r < NLB; ++r) {
      if (r < p) continue;
      const int i = LB * p + rho, j0 = LB * r + 4 * kap;
      const float* s = slot + slot_of(p, r) * SLOT + rho * LS + 4 * kap;
      const floatx4 g = floatx4{s[0], s[1], s[2], s[3]};
      float* dst = blk + (i * (int)ld + j0);
      if (vec) {
        if (i < n && j0 < n) *reinterpret_cast<floatx4*>(dst) = g;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (i < n && j0 + c < n) dst[c] = g[c];
      }
    }
  }

  if (tid == 0 && bad_at != INT_MAX) atomicMin(flag, (int)(off + bad_at) + 1);
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
leaf_factor_invert(float* __restrict__ A, int64_t ld, int64_t off, int n, int* flag) {
  __shared__ LeafSmem sm;
  leaf_body(A, ld, off, n, flag, sm);
}

// One launch of the blocked schedule: workgroup 0 factors a leaf (when leaf_n > 0) while
// the others run 64 x 64 tiles of up to FUSED_TASKS independent products (tile ranges, with
// the tile code of the GEMM launches), all sharing one LDS allocation.
struct FusedArgs {
  float* A;
  int64_t ld, leaf_off;
  int* flag;
  int leaf_n, ntask;
  Dev g[plan::FUSED_TASKS];
  int64_t t0[plan::FUSED_TASKS], cnt[plan::FUSED_TASKS];
  int tb[plan::FUSED_TASKS];
};
union FusedSmem {
  LeafSmem leaf;
  Smem<64, 64> gm;
};

__global__ void __launch_bounds__(256, 2) prep_fused(FusedArgs a) {
  __shared__ __attribute__((aligned(16))) FusedSmem sm;
  int64_t b = blockIdx.x;
  if (a.leaf_n > 0) {
    if (b == 0) {
      leaf_body(a.A, a.ld, a.leaf_off, a.leaf_n, a.flag, sm.leaf);
      return;
    }
    --b;
  }
  for (int i = 0; i < a.ntask; ++i) {
    if (b < a.cnt[i]) {
      const int64_t t = a.t0[i] + b;
      if (a.tb[i]) gemm_tile<64, 64, false, true>(a.g[i], t, sm.gm);
      else gemm_tile<64, 64, false, false>(a.g[i], t, sm.gm);
      return;
    }
    b -= a.cnt[i];
  }
}

// Blocks factored by the blocked schedule (prep_plan.h) instead of the recursion below.
// Measured on MI355X (prepare at d = 1024 ... 11008): from 1024 it beats the recursion; up to
// 2048 its trailing updates and tree products fit beside the leaves, while at 4096 the
// early trailing updates (rank 128 over a 3840-square triangle) outlast the leaf and the
// recursion's one split into two 2048 halves with large products is faster.
constexpr int64_t BLK_MIN = 1024, BLK_MAX = 2048;
bool blocked(int64_t n) { return n > NB && n >= BLK_MIN && n <= BLK_MAX; }

// Plans by (n, ld, r), built once (the ones a process uses are few).
const plan::Plan& plan_of(int64_t n, int64_t ld, int64_t r) {
  static std::mutex mu;
  static std::map<std::tuple<int64_t, int64_t, int64_t>, plan::Plan> cache;
  std::lock_guard<std::mutex> lk(mu);
  const auto key = std::make_tuple(n, ld, r);
  auto it = cache.find(key);
  if (it == cache.end()) it = cache.emplace(key, plan::blocked_plan(n, ld, r)).first;
  return it->second;
}

// Split of an n-block: the leading m columns (a multiple of the leaf size) and the rest.
int64_t split_of(int64_t n) {
  int64_t m = (n / 2) / NB * NB;
  return m == 0 ? n - NB : m;
}
// Floats of the Q stack needed by factor_rec on an n-block (see below).
int64_t q_stack(int64_t n) {
  if (n <= NB || blocked(n)) return 0;
  const int64_t m = split_of(n), r = n - m;
  const int64_t own = align_up((size_t)(m * r), 64);
  const int64_t right = q_stack(r), left = own + q_stack(m);
  return right > left ? right : left;
}
// Floats of the blocked schedule's scratch (U and the tree's Q blocks) for the largest
// block the recursion hands to it; the blocked calls run one after another.
int64_t blk_floats(int64_t n) {
  if (n <= NB) return 0;
  if (blocked(n)) {
    const plan::Plan& p = plan_of(n, n, 0);
    return align_up((size_t)p.panel_floats, 64) + p.q_floats;
  }
  const int64_t m = split_of(n), a = blk_floats(m), b = blk_floats(n - m);
  return a > b ? a : b;
}

GemmArgs args_of(const plan::Gemm& g, float* const* bufs) {
  return GemmArgs{g.M, g.N, g.K, bufs[g.A.buf] + g.A.off, g.A.ld, g.transA, g.triA,
                  bufs[g.B.buf] + g.B.off, g.B.ld, g.transB, g.triB,
                  bufs[g.C.buf] + g.C.off, g.C.ld, g.triC, g.alpha, g.beta};
}

// The n-block at (off, off) by the blocked schedule, on the caller's stream; with r > 0 it
// also forms the enclosing node's Q = P G22 (P, Q: n x r, G22 the r-block at (off + n,
// off + n)).
hipError_t factor_blocked(float* A, int64_t ld, int64_t off, int64_t n, float* scratch, int* flag,
                          hipStream_t s, float* P = nullptr, float* Q = nullptr, int64_t r = 0) {
  if (ld >= ((int64_t)1 << 24)) return hipErrorInvalidValue;   // 32-bit in-tile offsets
  const plan::Plan& p = plan_of(n, ld, r);
  float* bufs[5] = {A + off * ld + off, scratch, scratch + align_up((size_t)p.panel_floats, 64),
                    P, Q};
  for (const plan::Op& o : p.ops) {
    hipError_t e;
    if (o.kind == plan::GEMM) {
      e = gemm_f32(args_of(o.t[0].g, bufs), s, "prep_gemm");
    } else {
      FusedArgs fa{};
      fa.A = A;
      fa.ld = ld;
      fa.leaf_off = off + o.off;
      fa.flag = flag;
      fa.leaf_n = (int)o.n;
      fa.ntask = (int)o.t.size();
      int64_t grid = o.n > 0 ? 1 : 0;
      for (int i = 0; i < fa.ntask; ++i) {
        const plan::Task& t = o.t[i];
        const GemmArgs ga = args_of(t.g, bufs);
        fa.g[i] = make_dev(ga);
        fa.t0[i] = t.t0;
        fa.cnt[i] = t.t1 - t.t0;
        fa.tb[i] = ga.transB;
        grid += fa.cnt[i];
      }
      ProfScope ps(o.n > 0 ? "prep_leaf" : "prep_gemm", s);
      hipLaunchKernelGGL(prep_fused, dim3((unsigned)grid), dim3(256), 0, s, fa);
      e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// P (m x r) is scratch shared by all nodes (it is dead once Q and the Schur update are
// formed); Q = P G22 must survive the recursion on A11, so each node takes its Q from a
// stack above the ones of its ancestors.
hipError_t factor_rec(float* A, int64_t ld, int64_t off, int64_t n, float* P, float* qstack,
                      float* blk, int* flag, hipStream_t s) {
  hipError_t e;
  if (blocked(n)) return factor_blocked(A, ld, off, n, blk, flag, s);
  if (n <= NB) {
    ProfScope ps("prep_leaf", s);
    hipLaunchKernelGGL(leaf_factor_invert, dim3(1), dim3(256), 0, s, A, ld, off, (int)n, flag);
    return hipGetLastError();
  }
  const int64_t m = split_of(n), r = n - m;
  float* A11 = A + off * ld + off;
  float* A12 = A11 + m;
  float* A22 = A + (off + m) * ld + off + m;
  float* Q = qstack;

  if ((e = factor_rec(A, ld, off + m, r, P, qstack, blk, flag, s)) != hipSuccess) return e;
  // P = A12 G22^T   (op(B)[k][j] = G22[j][k], zero for k < j)
  if ((e = gemm_f32({m, r, r, A12, ld, 0, 0, A22, ld, 1, 2, P, r, 0, 1.0f, 0.0f}, s,
                    "prep_gemm")) != hipSuccess)
    return e;
  if (blocked(m)) {
    // A11 <- A11 - P P^T (upper triangle); Q = P G22 runs beside A11's leaves
    if ((e = gemm_f32({m, m, r, P, r, 0, 0, P, r, 1, 0, A11, ld, 1, -1.0f, 1.0f}, s,
                      "prep_gemm")) != hipSuccess)
      return e;
    if ((e = factor_blocked(A, ld, off, m, blk, flag, s, P, Q, r)) != hipSuccess) return e;
    return gemm_f32({m, r, m, A11, ld, 0, 1, Q, r, 0, 0, A12, ld, 0, -1.0f, 0.0f}, s, "prep_gemm");
  }
  // Q = P G22 (G22 upper: zero for k > j), and A11 <- A11 - P P^T (upper triangle)
  if ((e = gemm_f32_pair({m, r, r, P, r, 0, 0, A22, ld, 0, 1, Q, r, 0, 1.0f, 0.0f},
                         {m, m, r, P, r, 0, 0, P, r, 1, 0, A11, ld, 1, -1.0f, 1.0f}, s,
                         "prep_gemm")) != hipSuccess)
    return e;
  if ((e = factor_rec(A, ld, off, m, P, qstack + align_up((size_t)(m * r), 64), blk, flag, s)) !=
      hipSuccess)
    return e;
  // G12 = -G11 Q   (G11 upper: zero for k < i), straight into A12
  return gemm_f32({m, r, m, A11, ld, 0, 1, Q, r, 0, 0, A12, ld, 0, -1.0f, 0.0f}, s, "prep_gemm");
}

}  // namespace

// Floats of the recursion's P scratch (its largest product), none when the whole matrix
// goes to the blocked schedule.
int64_t p_floats(int64_t d) { return d > NB && !blocked(d) ? split_of(d) * (d - split_of(d)) : 0; }

size_t prepare_ws_bytes(int64_t d) {
  const int64_t p = p_floats(d);
  return 256 + (align_up((size_t)p, 64) + align_up((size_t)q_stack(d), 64) +
                (size_t)blk_floats(d) + 64) * sizeof(float);
}

int* prepare_flag_ptr(void* ws, int64_t d) { return carve(ws, d).flag; }

hipError_t prepare_launch(const float* H, float* G, int64_t d, float damp_frac, void* ws,
                          hipStream_t stream) {
  hipError_t e;
  PrepWs w = carve(ws, d);
  const bool vec4 = d % 4 == 0 && ((reinterpret_cast<uintptr_t>(H) | reinterpret_cast<uintptr_t>(G)) & 15) == 0;
  {
    ProfScope ps("prep_damp", stream);
    hipLaunchKernelGGL(damp_lambda, dim3(1), dim3(256), 0, stream, H, d, damp_frac, w.lambda,
                       w.flag);
    if (vec4)
      hipLaunchKernelGGL(copy_damp4, dim3((unsigned)(d < 16384 ? d : 16384)), dim3(256), 0, stream, H,
                         G, d, w.lambda);
    else
      hipLaunchKernelGGL(copy_damp, rows_grid(d, d), dim3(256), 0, stream, H, G, d, w.lambda);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  float* qs = w.tmp + align_up((size_t)p_floats(d), 64);
  float* blk = qs + align_up((size_t)q_stack(d), 64);
  if ((e = factor_rec(G, d, 0, d, w.tmp, qs, blk, w.flag, stream)) != hipSuccess) return e;
  if (vec4)
    hipLaunchKernelGGL(zero_lower4, dim3((unsigned)(d < 16384 ? d : 16384)), dim3(256), 0, stream, G,
                       d);
  else
    hipLaunchKernelGGL(zero_lower, rows_grid(d, d), dim3(256), 0, stream, G, d);
  return hipGetLastError();
}

}  // namespace gptq
