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
//   per block row i:
//     trtri_row     X[i][j] = -Linv_ii sum_m L[i][m] X[m][j] (X = L^-1, fp64),
//                   and U at the reversed position in fp32
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
// Block row i of X = L^-1:  X[i][j] = -Dinv_i sum_{m=j}^{i-1} L[i][m] X[m][j]  (j < i),
// X[i][i] = Dinv_i.  X is kept in fp64; U (and U^T) receive the fp32 values at
// the reversed position.
__global__ __launch_bounds__(256) void trtri_row_kernel(const double* __restrict__ Aall, int c, int i,
                                                        const double* __restrict__ dinv,
                                                        double* __restrict__ Xall,
                                                        float* __restrict__ Uall,
                                                        float* __restrict__ UTall) {
  __shared__ double Ls[kNb][kNb + 1];
  __shared__ double Xs[kNb][kNb + 1];
  const int m = blockIdx.y, j = blockIdx.x;
  const double* A = Aall + (int64_t)m * c * c;
  double* X = Xall + (int64_t)m * c * c;
  float* U = Uall + (int64_t)m * c * c;
  float* UT = UTall ? UTall + (int64_t)m * c * c : nullptr;
  const double* Di = dinv + ((int64_t)m * (c / kNb) + i) * kNb * kNb;
  const int64_t i0 = (int64_t)i * kNb, j0 = (int64_t)j * kNb;
  if (j == i) {
    for (int idx = threadIdx.x; idx < kNb * kNb; idx += 256) {
      const int r = idx >> 6, cc = idx & 63;
      const double v = cc <= r ? Di[idx] : 0.0;
      X[(i0 + r) * c + j0 + cc] = v;
      if (cc <= r) U[(c - 1 - (i0 + r)) * c + (c - 1 - (j0 + cc))] = (float)v;
      // U^T: element (c-1-(j0+cc), c-1-(i0+r)); consecutive threads step r
      const int rr = idx & 63, c2 = idx >> 6;
      if (UT && c2 <= rr) UT[(c - 1 - (j0 + c2)) * c + (c - 1 - (i0 + rr))] = (float)Di[rr * kNb + c2];
    }
    return;
  }
  Tile64 t;
  t.zero();
  {
    ChunkPipe pipe;
    pipe.fetch(A + i0 * c + j0, c, X + j0 * c + j0, c);
    for (int mm = j; mm < i; ++mm) {
      __syncthreads();
      pipe.stage(Ls, Xs);
      __syncthreads();
      if (mm + 1 < i) pipe.fetch(A + i0 * c + (mm + 1) * kNb, c, X + (int64_t)(mm + 1) * kNb * c + j0, c);
      t.mac<false>(Ls, Xs, 1.0);
    }
  }
  // Xs <- T (the sum), Ls <- Linv_ii; then X[i][j] = -Linv_ii T
  __syncthreads();
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) Xs[Tile64::row(x, r)][Tile64::col(y)] = t.acc[x][y][r];
  for (int idx = threadIdx.x; idx < kNb * kNb; idx += 256) Ls[idx >> 6][idx & 63] = Di[idx];
  __syncthreads();
  t.zero();
  t.mac<false>(Ls, Xs, -1.0);
  __syncthreads();
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = Tile64::row(x, r), col = Tile64::col(y);
        const double v = t.acc[x][y][r];
        X[(i0 + row) * c + j0 + col] = v;
        U[(c - 1 - (i0 + row)) * c + (c - 1 - (j0 + col))] = (float)v;
        Xs[row][col] = v;
      }
  if (UT) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < kNb * kNb; idx += 256) {
      const int rr = idx & 63, cc = idx >> 6;   // consecutive threads step the U^T column
      UT[(c - 1 - (j0 + cc)) * c + (c - 1 - (i0 + rr))] = (float)Xs[rr][cc];
    }
  }
}

void launch_inverse_cholesky(const GptqPlan& p, hipStream_t s) {
  const int c = p.cols, nbk = c / kNb;
  hipLaunchKernelGGL(diag_stats_kernel, dim3(p.n_mats), dim3(256), 0, s, p.mats, c, p.damp,
                     p.dead, p.lamd, p.lam);
  hipLaunchKernelGGL(build_reversed_kernel, dim3(nbk * (nbk + 1) / 2, p.n_mats), dim3(256), 0, s,
                     p.mats, c, p.dead, p.lamd, p.A);
  for (int k = 0; k < nbk; ++k) {
    hipLaunchKernelGGL(chol_left_kernel, dim3(nbk - k, p.n_mats), dim3(256), 0, s, p.A, c, k);
    hipLaunchKernelGGL(chol_diag_kernel, dim3(p.n_mats), dim3(64), 0, s, p.A, c, k, p.dinv, p.status);
    if (k + 1 < nbk)
      hipLaunchKernelGGL(chol_panel_kernel, dim3(nbk - k - 1, p.n_mats), dim3(256), 0, s, p.A, c, k,
                         p.dinv);
  }
  for (int i = 0; i < nbk; ++i)
    hipLaunchKernelGGL(trtri_row_kernel, dim3(i + 1, p.n_mats), dim3(256), 0, s, p.A, c, i, p.dinv,
                       p.X, p.U, p.UT);
}

}  // namespace clha
