// Inverse-Hessian factor for GPTQ: U upper triangular, positive diagonal,
// U^T U = Hd^-1, with Hd the damped Hessian.
//
// GPTQ (Frantar et al., ICLR 2023, section "Cholesky reformulation") drives its
// column-sequential updates from the rows of the upper Cholesky factor of the
// inverse Hessian; the CLHA summary (section 2.2, step 3) runs that standard
// GPTQ on H_comb.
//
// Route (no explicit inverse): with J the index reversal, factor the reversed
// matrix J Hd J = L L^T (ordinary lower Cholesky).  Then Hd = R R^T with
// R = J L J upper triangular, Hd^-1 = R^-T R^-1, and U = R^-1 = J L^-1 J.
// Cost: c^3/3 flops for the factorisation and c^3/3 for the triangular inverse.
//
// Precision: the factorisation and the inverse run in fp64 (the fp64 matrix
// cores, v_mfma_f64_16x16x4f64, run at half the fp32 rate on MI355X).  A
// right-looking fp32 factorisation rounds each diagonal entry once per block
// step while it shrinks from H_jj to its Schur complement, which costs about a
// decimal digit on ill-conditioned Hessians; GPTQ's code decisions inherit that
// error.  U is rounded to fp32 once, at the end.
//
// Every step is batched over all distinct Hessians of one call:
//   diag_stats      dead columns (H_ii == 0) and lambda = damp * mean(diag),
//                   taking H_ii := 1 on dead columns first
//   build_reversed  A = J (H + fixes + lambda I) J, lower triangle, fp64
//   left-looking Cholesky, per 64-column block step k:
//     chol_left     T_i = A[i][k] - sum_{m<k} L[i][m] L[k][m]^T for block rows i >= k
//                   (a chunked fp64 MFMA product, next chunk prefetched)
//     chol_diag     L_kk = chol(T_k) and its inverse Dinv_k (one wavefront per matrix,
//                   rows in registers)
//     chol_panel    L[i][k] = T_i Dinv_k^T for i > k
//   triangular inverse X = L^-1 (fp64), merged bottom-up over block ranges:
//     trtri_leaf    X[i][i] = Dinv_i
//     trtri_merge   X21 = -X22 L21 X11 per merge (two batched GEMMs per level),
//                   U = J X J and U^T written in fp32 as X becomes final
// The Hessians of one call are split into groups, one stream each, started one
// block step apart (see launch_factor_group).
#include "kernels.h"

namespace clha {

typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void tri_of(int t, int& i, int& j) {
  int a = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((a + 1) * (a + 2) / 2 <= t) ++a;
  while (a * (a + 1) / 2 > t) --a;
  i = a;
  j = t - a * (a + 1) / 2;
}

// 64x64 tile product on the fp64 matrix cores: each of the 4 waves owns a 32x32
// quarter as 2x2 blocks of 16x16.  acc[bi][bj][r] is element
// (wm*32 + bi*16 + 4*(lane/16) + r, wn*32 + bj*16 + lane%16) of the tile.
// Operand lanes of v_mfma_f64_16x16x4f64 (measured on gfx950): lane l holds
// B[k = l/16][j = l%16] and A[i = 4*(l%4) + (l%16)/4][k = l/16].
struct Tile64 {
  f64x4 acc[2][2];
  __device__ void zero() {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
  }
  // acc += sign * Am[row][k] * Bm[k][col]; Am indexed [row][k], Bm given by
  // `bk(k, col)` through a [k][col] array or a [col][k] array (transposed)
  template <bool BT>
  __device__ void mac(const double (*Am)[kNb + 1], const double (*Bm)[kNb + 1], double sign) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int li = lane & 15, lk = lane >> 4;
    const int ai = 4 * (li & 3) + (li >> 2);
#pragma unroll 4
    for (int k = 0; k < kNb; k += 4) {
      double a[2], b[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        a[x] = sign * Am[wm * 32 + x * 16 + ai][k + lk];
        b[x] = BT ? Bm[wn * 32 + x * 16 + li][k + lk] : Bm[k + lk][wn * 32 + x * 16 + li];
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[x], b[y], acc[x][y], 0, 0, 0);
    }
  }
  __device__ static int row(int x, int r) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    return (wave >> 1) * 32 + x * 16 + 4 * (lane >> 4) + r;
  }
  __device__ static int col(int y) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    return (wave & 1) * 32 + y * 16 + (lane & 15);
  }
};

// ---------------------------------------------------------------- damping

__global__ __launch_bounds__(256) void diag_stats_kernel(const float* const* __restrict__ mats,
                                                         int c, float damp,
                                                         uint8_t* __restrict__ dead,
                                                         double* __restrict__ lamd,
                                                         float* __restrict__ lam_out) {
  __shared__ double red[256];
  const int m = blockIdx.x;
  const float* H = mats[m];
  double sum = 0.0;
  for (int i = threadIdx.x; i < c; i += 256) {
    const float h = H[(int64_t)i * c + i];
    const bool z = h == 0.0f;
    dead[(int64_t)m * c + i] = z;
    sum += z ? 1.0 : (double)h;
  }
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double l = (double)damp * (red[0] / (double)c);
    lamd[m] = l;
    if (lam_out) lam_out[m] = (float)l;
  }
}

__global__ __launch_bounds__(256) void build_reversed_kernel(const float* const* __restrict__ mats,
                                                             int c, const uint8_t* __restrict__ dead,
                                                             const double* __restrict__ lamd,
                                                             double* __restrict__ Aall) {
  const int m = blockIdx.y;
  int bi, bj;
  tri_of(blockIdx.x, bi, bj);
  const float* H = mats[m];
  double* A = Aall + (int64_t)m * c * c;
  const double l = lamd[m];
  for (int idx = threadIdx.x; idx < kNb * kNb; idx += 256) {
    const int r = idx >> 6, cc = idx & 63;
    const int i = bi * kNb + r, j = bj * kNb + cc;
    if (j > i) continue;
    const int hi = c - 1 - i, hj = c - 1 - j;
    double v = (double)H[(int64_t)hi * c + hj];
    if (i == j) v = (dead[(int64_t)m * c + hi] ? 1.0 : v) + l;
    A[(int64_t)i * c + j] = v;
  }
}

// ---------------------------------------------------------------- chunked 64x64 products
// Sum over chunks m of P_m Q_m (64x64 fp64 blocks read from global memory):
// each thread prefetches its 16+16 elements of the next chunk into registers
// while the matrix cores work on the current chunk in LDS.
struct ChunkPipe {
  double ra[16], rb[16];
  __device__ __forceinline__ void fetch(const double* P, int64_t ldp, const double* Q, int64_t ldq) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int idx = threadIdx.x + 256 * u, r = idx >> 6, cc = idx & 63;
      ra[u] = P[r * ldp + cc];
      rb[u] = Q[r * ldq + cc];
    }
  }
  __device__ __forceinline__ void stage(double (*As)[kNb + 1], double (*Bs)[kNb + 1]) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int idx = threadIdx.x + 256 * u, r = idx >> 6, cc = idx & 63;
      As[r][cc] = ra[u];
      Bs[r][cc] = rb[u];
    }
  }
};

// ---------------------------------------------------------------- left-looking Cholesky
// Step k, block row i >= k:  T_i = A[i][k] - sum_{m<k} L[i][m] L[k][m]^T, stored over A[i][k].
__global__ __launch_bounds__(256) void chol_left_kernel(double* __restrict__ Aall, int c, int k) {
  __shared__ double As[kNb][kNb + 1];
  __shared__ double Bs[kNb][kNb + 1];
  const int m = blockIdx.y, i = k + blockIdx.x;
  const bool diag = i == k;
  double* A = Aall + (int64_t)m * c * c;
  const int64_t i0 = (int64_t)i * kNb, k0 = (int64_t)k * kNb;
  Tile64 t;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = Tile64::row(x, r), col = Tile64::col(y);
        t.acc[x][y][r] = (!diag || col <= row) ? A[(i0 + row) * c + k0 + col] : 0.0;
      }
  if (k > 0) {
    ChunkPipe pipe;
    pipe.fetch(A + i0 * c, c, A + k0 * c, c);
    for (int mm = 0; mm < k; ++mm) {
      __syncthreads();
      pipe.stage(As, Bs);
      __syncthreads();
      if (mm + 1 < k) pipe.fetch(A + i0 * c + (mm + 1) * kNb, c, A + k0 * c + (mm + 1) * kNb, c);
      t.mac<true>(As, Bs, -1.0);
    }
  }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = Tile64::row(x, r), col = Tile64::col(y);
        if (!diag || col <= row) A[(i0 + row) * c + k0 + col] = t.acc[x][y][r];
      }
}

// Step k: L_kk = chol(T_k) and Dinv_k = L_kk^-1, one wavefront per matrix.
// Lane r holds row r of the 64x64 block in registers; a pivot or a column
// value is broadcast with readlane, so no step needs a barrier.  The template
// recursion keeps every register index a compile-time constant.
__device__ __forceinline__ double lane_value(double v, int src) {
  const uint64_t b = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)b, src);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(b >> 32), src);
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

// Cholesky column J: a[] is this lane's row of the block being factored.
template <int J>
__device__ __forceinline__ void chol_cols(double (&a)[kNb], double (&piv)[kNb], int r, bool& bad) {
  double d = lane_value(a[J], J);
  if (!(d > 0.0)) {
    bad = true;
    d = 1.0;
  }
  const double ljj = sqrt(d);
  piv[J] = ljj;
  if (r == J) a[J] = ljj;
  if (r > J) a[J] = a[J] / ljj;
#pragma unroll
  for (int cc = J + 1; cc < kNb; ++cc) a[cc] = fma(-a[J], lane_value(a[J], cc), a[cc]);
  if constexpr (J + 1 < kNb) chol_cols<J + 1>(a, piv, r, bad);
}

// Forward elimination on L X = I, pivot row J: x[] is this lane's row of X.
template <int J>
__device__ __forceinline__ void inv_rows(const double (&a)[kNb], const double (&piv)[kNb],
                                         double (&x)[kNb], int r) {
  const double inv = 1.0 / piv[J];
  if (r == J) {
#pragma unroll
    for (int cc = 0; cc <= J; ++cc) x[cc] *= inv;
  }
#pragma unroll
  for (int cc = 0; cc <= J; ++cc) {
    const double xj = lane_value(x[cc], J);
    if (r > J) x[cc] = fma(-a[J], xj, x[cc]);
  }
  if constexpr (J + 1 < kNb) inv_rows<J + 1>(a, piv, x, r);
}

__global__ __launch_bounds__(64) void chol_diag_kernel(const double* __restrict__ Aall, int c, int k,
                                                       double* __restrict__ dinv,
                                                       int* __restrict__ status) {
  const int m = blockIdx.x, r = threadIdx.x;
  const double* A = Aall + (int64_t)m * c * c;
  const int64_t k0 = (int64_t)k * kNb;
  double a[kNb], x[kNb], piv[kNb];
  const double* row = A + (k0 + r) * c + k0;
#pragma unroll
  for (int cc = 0; cc < kNb; cc += 2) {
    const double2 v = *reinterpret_cast<const double2*>(row + cc);
    a[cc] = cc <= r ? v.x : 0.0;
    a[cc + 1] = cc + 1 <= r ? v.y : 0.0;
  }
  bool bad = false;
  chol_cols<0>(a, piv, r, bad);
  if (bad && r == 0) atomicOr(status, kStatusNotPd);
#pragma unroll
  for (int cc = 0; cc < kNb; ++cc) x[cc] = cc == r ? 1.0 : 0.0;
  inv_rows<0>(a, piv, x, r);
  double* D = dinv + ((int64_t)m * (c / kNb) + k) * kNb * kNb + (int64_t)r * kNb;
#pragma unroll
  for (int cc = 0; cc < kNb; cc += 2) *reinterpret_cast<double2*>(D + cc) = make_double2(x[cc], x[cc + 1]);
}

// Step k, block row i > k:  L[i][k] = T_i Dinv_k^T.
__global__ __launch_bounds__(256) void chol_panel_kernel(double* __restrict__ Aall, int c, int k,
                                                         const double* __restrict__ dinv) {
  __shared__ double Ts[kNb][kNb + 1];
  __shared__ double Ds[kNb][kNb + 1];
  const int m = blockIdx.y, i = k + 1 + blockIdx.x;
  double* A = Aall + (int64_t)m * c * c;
  const double* D = dinv + ((int64_t)m * (c / kNb) + k) * kNb * kNb;
  const int64_t i0 = (int64_t)i * kNb, k0 = (int64_t)k * kNb;
  for (int idx = threadIdx.x; idx < kNb * kNb; idx += 256) {
    const int r = idx >> 6, cc = idx & 63;
    Ts[r][cc] = A[(i0 + r) * c + k0 + cc];
    Ds[r][cc] = D[idx];
  }
  __syncthreads();
  Tile64 t;
  t.zero();
  t.mac<true>(Ts, Ds, 1.0);
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        A[(i0 + Tile64::row(x, r)) * c + k0 + Tile64::col(y)] = t.acc[x][y][r];
}

// ---------------------------------------------------------------- triangular inverse
// X = L^-1, merged bottom-up over ranges of 64-column blocks.  For a range
// [a, b) split at mid, with X11 the inverse over [a, mid) and X22 over [mid, b):
//   X21 = -X22 L21 X11,   L21 = L[mid:b, a:mid]
// (the inverse of a 2x2 block lower-triangular matrix).  Level s merges ranges
// of 2s blocks (s = 1, 2, 4, ...); merges of one level are independent.  The
// leaves are the diagonal blocks' inverses Dinv from the factorisation.  Each
// merge is two batched fp64 GEMMs on the matrix cores:
//   phase 0:  T = L21 X11     (X11 lower triangular: only k >= column counts)
//   phase 1:  X21 = -X22 T    (X22 lower triangular: only k <= row counts)
// T is kept transposed in the strictly upper triangle of A, which the
// factorisation leaves unused: T[row][col] at A[col][row].  Every X element is
// final when written, so U = J X J (and U^T) get their fp32 values at once.

// Leaves: X[i][i] = Dinv_i (zeros above the diagonal), and U, U^T there.
__global__ __launch_bounds__(256) void trtri_leaf_kernel(int c, const double* __restrict__ dinv,
                                                         double* __restrict__ Xall,
                                                         float* __restrict__ Uall,
                                                         float* __restrict__ UTall) {
  const int m = blockIdx.y, i = blockIdx.x;
  double* X = Xall + (int64_t)m * c * c;
  float* U = Uall + (int64_t)m * c * c;
  float* UT = UTall ? UTall + (int64_t)m * c * c : nullptr;
  const double* Di = dinv + ((int64_t)m * (c / kNb) + i) * kNb * kNb;
  const int64_t i0 = (int64_t)i * kNb;
  for (int idx = threadIdx.x; idx < kNb * kNb; idx += 256) {
    const int r = idx >> 6, cc = idx & 63;
    const double v = cc <= r ? Di[idx] : 0.0;
    X[(i0 + r) * c + i0 + cc] = v;
    if (cc <= r) U[(c - 1 - (i0 + r)) * c + (c - 1 - (i0 + cc))] = (float)v;
    // U^T: element (c-1-(i0+cc), c-1-(i0+r)); consecutive threads step r
    const int rr = idx & 63, c2 = idx >> 6;
    if (UT && c2 <= rr) UT[(c - 1 - (i0 + c2)) * c + (c - 1 - (i0 + rr))] = (float)Di[rr * kNb + c2];
  }
}

constexpr int kTT = 128;          // merge tile: rows and columns
constexpr int kTK = 16;           // K chunk
constexpr int kTPa = kTK + 2;     // pitch of [row][k] LDS tiles (doubles): conflict-free lane reads
constexpr int kTPb = kTT + 16;    // pitch of the [k][col] LDS tile (doubles)
constexpr int kTBuf = kTT * kTPa; // one operand buffer (== kTK * kTPb)
static_assert(kTT * kTPa == kTK * kTPb, "operand buffers share one size");

// One 128x128 tile of one merge.  256 threads = 4 waves of 64x64 (4x4 blocks
// of v_mfma_f64_16x16x4f64; lane layout as in Tile64).  Operands are staged
// through LDS in chunks of 16 along K, double-buffered with two register
// stages.  Tiles of one merge are mapped to one XCD (workgroup b runs on XCD
// b % 8) so its operands are shared through one L2.
template <int PHASE>
__global__ __launch_bounds__(256, 2) void trtri_merge_kernel(double* __restrict__ Aall,
                                                             double* __restrict__ Xall,
                                                             float* __restrict__ Uall,
                                                             float* __restrict__ UTall, int c, int s,
                                                             int n_merge, int tc, int n_mats) {
  __shared__ __attribute__((aligned(16))) double lds[4 * kTBuf];   // A0 B0 A1 B1
  const int nbk = c / kNb, tmax = tc * tc;
  const int total = n_mats * n_merge * tmax;
  const int per = (total + kXcds - 1) / kXcds;
  const int L = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
  if (L >= total) return;
  const int t = L % tmax, rest = L / tmax;
  const int pm = rest % n_merge, m = rest / n_merge;
  const int ti = t / tc, tj = t - (t / tc) * tc;
  const int a = 2 * s * pm, mid = a + s, b = min(a + 2 * s, nbk);
  const int r0 = mid * kNb + ti * kTT, c0 = a * kNb + tj * kTT;
  const int nr = min(kTT, b * kNb - r0), nc = min(kTT, mid * kNb - c0);
  if (nr <= 0 || nc <= 0) return;
  // K range of the tile (64-aligned; masked elements contribute zero)
  const int k0 = PHASE == 0 ? c0 : mid * kNb;
  const int k1 = PHASE == 0 ? mid * kNb : min(r0 + kTT, b * kNb);
  const int nch = (k1 - k0) / kTK;
  double* A = Aall + (int64_t)m * c * c;
  double* X = Xall + (int64_t)m * c * c;
  // A operand rows (K-contiguous): phase 0 L[r0 + i][k], phase 1 X[r0 + i][k]
  const double* Ar = (PHASE == 0 ? A : X) + (int64_t)r0 * c;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const bool active = wm * 64 < nr && wn * 64 < nc;
  const int li = lane & 15, lk = lane >> 4, ai = 4 * (li & 3) + (li >> 2);

  struct Stage {
    double2 a[4], b[4];
  };
  // Phase 0 walks K downwards from the merge's common end, phase 1 upwards from
  // its common start: the tiles of one merge then read the same K chunks at
  // about the same time, so one L2 serves them all.
  auto fetch = [&](Stage& rg, int ch) {
    const int kb = PHASE == 0 ? k1 - (ch + 1) * kTK : k0 + ch * kTK;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = tid + 256 * u;
      {  // A operand: row q/8, k pair 2(q%8)
        const int row = q >> 3, kc = 2 * (q & 7), kk = kb + kc;
        double2 v = make_double2(0.0, 0.0);
        if (row < nr) {
          v = *reinterpret_cast<const double2*>(Ar + (int64_t)row * c + kk);
          if (PHASE == 1) {   // X22 lower triangular
            if (kk > r0 + row) v.x = 0.0;
            if (kk + 1 > r0 + row) v.y = 0.0;
          }
        }
        rg.a[u] = v;
      }
      if (PHASE == 0) {  // B = X11[k][c0 + j]: k row q/64, column pair 2(q%64)
        const int krow = q >> 6, jc = 2 * (q & 63), kk = kb + krow;
        double2 v = make_double2(0.0, 0.0);
        if (jc < nc) {
          v = *reinterpret_cast<const double2*>(X + (int64_t)kk * c + c0 + jc);
          if (kk < c0 + jc) v.x = 0.0;
          if (kk < c0 + jc + 1) v.y = 0.0;
        }
        rg.b[u] = v;
      } else {           // B^T = T^T[c0 + j][k] stored at A[c0 + j][k]: row q/8, k pair 2(q%8)
        const int row = q >> 3, kc = 2 * (q & 7);
        rg.b[u] = row < nc ? *reinterpret_cast<const double2*>(A + (int64_t)(c0 + row) * c + kb + kc)
                           : make_double2(0.0, 0.0);
      }
    }
  };
  auto stage = [&](const Stage& rg, int buf) {
    double* As = lds + (2 * buf) * kTBuf;
    double* Bs = lds + (2 * buf + 1) * kTBuf;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = tid + 256 * u;
      *reinterpret_cast<double2*>(As + (q >> 3) * kTPa + 2 * (q & 7)) = rg.a[u];
      if (PHASE == 0)
        *reinterpret_cast<double2*>(Bs + (q >> 6) * kTPb + 2 * (q & 63)) = rg.b[u];
      else
        *reinterpret_cast<double2*>(Bs + (q >> 3) * kTPa + 2 * (q & 7)) = rg.b[u];
    }
  };
  f64x4 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f64x4{0.0, 0.0, 0.0, 0.0};
  auto multiply = [&](int buf) {
    if (!active) return;
    const double* As = lds + (2 * buf) * kTBuf + (wm * 64 + ai) * kTPa + lk;
    const double* Bs = lds + (2 * buf + 1) * kTBuf;
#pragma unroll
    for (int kk = 0; kk < kTK; kk += 4) {
      double av[4], bv[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) av[x] = As[x * 16 * kTPa + kk];
#pragma unroll
      for (int y = 0; y < 4; ++y)
        bv[y] = PHASE == 0 ? Bs[(kk + lk) * kTPb + wn * 64 + y * 16 + li]
                           : Bs[(wn * 64 + y * 16 + li) * kTPa + kk + lk];
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[x], bv[y], acc[x][y], 0, 0, 0);
    }
  };

  // nch is a multiple of 4
  Stage g0, g1;
  fetch(g0, 0);
  stage(g0, 0);
  fetch(g1, 1);
  if (nch > 2) fetch(g0, 2);
  __syncthreads();
#pragma unroll 1
  for (int st = 0; st < nch; st += 2) {
    multiply(0);
    stage(g1, 1);
    if (st + 3 < nch) fetch(g1, st + 3);
    __syncthreads();
    multiply(1);
    if (st + 2 < nch) stage(g0, 0);
    if (st + 4 < nch) fetch(g0, st + 4);
    __syncthreads();
  }
  if (!active) return;
  // element (row, col) of the tile: row = wm*64 + 16x + 4(lane/16) + r, col = wn*64 + 16y + lane%16
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int row = r0 + wm * 64 + 16 * x + 4 * lk, col = c0 + wn * 64 + 16 * y + li;
      const f64x4 v = acc[x][y];
      if (PHASE == 0) {
        // T^T[col][row .. row+3], contiguous
        double* tp = A + (int64_t)col * c + row;
        *reinterpret_cast<double2*>(tp) = make_double2(v[0], v[1]);
        *reinterpret_cast<double2*>(tp + 2) = make_double2(v[2], v[3]);
      } else {
        float* U = Uall + (int64_t)m * c * c;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          X[(int64_t)(row + r) * c + col] = -v[r];
          U[(int64_t)(c - 1 - (row + r)) * c + (c - 1 - col)] = (float)(-v[r]);
        }
        if (UTall) {
          // U^T row c-1-col, columns c-1-row-3 .. c-1-row (ascending)
          float* ut = UTall + (int64_t)m * c * c + (int64_t)(c - 1 - col) * c + (c - 4 - row);
          *reinterpret_cast<float4*>(ut) =
              make_float4((float)(-v[3]), (float)(-v[2]), (float)(-v[1]), (float)(-v[0]));
        }
      }
    }
}

// One group of Hessians [m0, m1) on one stream: the block-step chain of the
// factorisation, then the merge levels of the inverse.  Groups on separate
// streams interleave one group's latency-bound diagonal steps with the others'
// wide products.  step0_done (optional) is recorded after block step 0.
void launch_factor_group(const GptqPlan& p, int m0, int m1, hipStream_t s, hipEvent_t step0_done) {
  const int c = p.cols, nbk = c / kNb, n = m1 - m0;
  if (n <= 0) return;
  const int64_t cc = (int64_t)c * c;
  const float* const* mats = p.mats + m0;
  uint8_t* dead = p.dead + (int64_t)m0 * c;
  double* lamd = p.lamd + m0;
  float* lam = p.lam ? p.lam + m0 : nullptr;
  double* A = p.A + m0 * cc;
  double* X = p.X + m0 * cc;
  double* dinv = p.dinv + (int64_t)m0 * c * kNb;
  float* U = p.U + m0 * cc;
  float* UT = p.UT ? p.UT + m0 * cc : nullptr;
  hipLaunchKernelGGL(diag_stats_kernel, dim3(n), dim3(256), 0, s, mats, c, p.damp, dead, lamd, lam);
  hipLaunchKernelGGL(build_reversed_kernel, dim3(nbk * (nbk + 1) / 2, n), dim3(256), 0, s, mats, c, dead,
                     lamd, A);
  for (int k = 0; k < nbk; ++k) {
    hipLaunchKernelGGL(chol_left_kernel, dim3(nbk - k, n), dim3(256), 0, s, A, c, k);
    hipLaunchKernelGGL(chol_diag_kernel, dim3(n), dim3(64), 0, s, A, c, k, dinv, p.status);
    if (k == 0 && step0_done) hipEventRecord(step0_done, s);
    if (k + 1 < nbk)
      hipLaunchKernelGGL(chol_panel_kernel, dim3(nbk - k - 1, n), dim3(256), 0, s, A, c, k, dinv);
  }
  hipLaunchKernelGGL(trtri_leaf_kernel, dim3(nbk, n), dim3(256), 0, s, c, dinv, X, U, UT);
  for (int sz = 1; sz < nbk; sz *= 2) {
    const int n_merge = (nbk - sz + 2 * sz - 1) / (2 * sz);
    const int tc = (sz * kNb + kTT - 1) / kTT;
    const int total = n * n_merge * tc * tc;
    const dim3 grid(((total + kXcds - 1) / kXcds) * kXcds);
    hipLaunchKernelGGL(trtri_merge_kernel<0>, grid, dim3(256), 0, s, A, X, U, UT, c, sz, n_merge, tc, n);
    hipLaunchKernelGGL(trtri_merge_kernel<1>, grid, dim3(256), 0, s, A, X, U, UT, c, sz, n_merge, tc, n);
  }
}

}  // namespace clha
