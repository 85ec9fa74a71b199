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
// Precision: the factorisation keeps fp64 values.  A right-looking fp32
// factorisation rounds each diagonal entry once per block step while it
// shrinks from H_jj to its Schur complement, which costs about a decimal digit
// on ill-conditioned Hessians; GPTQ's code decisions inherit that error.  Its
// long products (the left-looking updates) run exactly on the int8 matrix
// cores over 42-bit digit expansions of L (see "sliced factor" below): about
// five times the sustained fp64 matrix rate, within 2^-36 of the fp64 product.
// The triangular inverse then runs at fp32 precision on the bf16 matrix cores:
// each fp32 operand is split into three bf16 parts and a product is the sum of
// the six part products above 2^-24 of it, each exact, accumulated in fp32
// (v_mfma_f32_32x32x16_bf16; see "triangular inverse" below).  Its error is
// governed by cond(L) = sqrt(cond(Hd)): against the fp64 oracle U moves by
// 1.7e-7 to 2.6e-7 relative at c = 256..2048 and cond(Hd) up to 2.4e3, about
// what fp32 matrix-core products gave (1.8e-7 to 3.2e-7).
//
// Every step is batched over all distinct Hessians of one call:
//   diag_stats      dead columns (H_ii == 0) and lambda = damp * mean(diag),
//                   taking H_ii := 1 on dead columns first; row exponents of the
//                   sliced factor (below)
//   The reversed damped matrix A = J (H + fixes + lambda I) J is never formed:
//   each entry is read from H (fp32, exact in fp64) once, by the block step
//   that first needs it.
//   left-looking Cholesky, per 64-column block step k:
//     chol_left     T_i = A[i][k] - sum_{m<k} L[i][m] L[k][m]^T for block rows i >= k
//                   (int8 digit-pair products accumulated exactly, next chunk prefetched);
//                   the diagonal tile's workgroup then forms L_kk = chol(T_k) and its
//                   inverse Dinv_k (one wave factors, one inverts, sharing each column
//                   through LDS)
//     chol_panel    L[i][k] = T_i Dinv_k^T for i > k, and its digit planes
//   triangular inverse X = L^-1, merged bottom-up over block ranges in fp32:
//     trtri_leaf    X[i][i] = Dinv_i
//     trtri_merge   X21 = -X22 L21 X11 per merge (two batched GEMMs per level),
//                   U = J X J and U^T written as X becomes final
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

// Also starts the Hessian's status bits (mstat[m]): kStatusNonfinite when a
// diagonal entry is NaN or infinite; the factor adds kStatusNotPd on a pivot
// that is not positive.  A failing Hessian is recorded in the context's status
// record by its index m_base + m.
__global__ __launch_bounds__(256) void diag_stats_kernel(const float* const* __restrict__ mats,
                                                         int c, float damp,
                                                         uint8_t* __restrict__ dead,
                                                         double* __restrict__ lamd,
                                                         float* __restrict__ lam_out,
                                                         int* __restrict__ lexp,
                                                         int* __restrict__ mstat,
                                                         int* __restrict__ status, int m_base) {
  __shared__ double red[256];
  __shared__ int nonfinite;
  const int m = blockIdx.x;
  const float* H = mats[m];
  if (threadIdx.x == 0) nonfinite = 0;
  __syncthreads();
  double sum = 0.0;
  bool bad = false;
  for (int i = threadIdx.x; i < c; i += 256) {
    const float h = H[(int64_t)i * c + i];
    const bool z = h == 0.0f;
    dead[(int64_t)m * c + i] = z;
    sum += z ? 1.0 : (double)h;
    bad |= !isfinite(h);
  }
  if (bad) nonfinite = 1;   // any writer, the same value
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const double l = (double)damp * (red[0] / (double)c);
  if (threadIdx.x == 0) {
    lamd[m] = l;
    if (lam_out) lam_out[m] = (float)l;
    mstat[m] = nonfinite ? kStatusNonfinite : 0;
    if (nonfinite) {
      atomicOr(status, kStatusNonfinite);
      atomicMax(reinterpret_cast<unsigned*>(status) + kStatusMat, 0xffffffffu - (unsigned)(m_base + m));
    }
  }
  // Row exponents of the factor of the reversed matrix A = J Hd J: every entry
  // of row i of the factor is at most sqrt(A_ii) in magnitude, and 2^e >=
  // sqrt(A_ii) (1 + 1/64) scales the row's digits so that a scaled entry
  // times 128 stays within 126.1 and its first digit fits int8.
  for (int hi = threadIdx.x; hi < c; hi += 256) {
    const float h = H[(int64_t)hi * c + hi];
    const double v = (h == 0.0f ? 1.0 : (double)h) + l;
    int e = 0;
    if (v > 0.0) frexp(sqrt(v) * (1.0 + 1.0 / 64.0), &e);
    lexp[(int64_t)m * c + (c - 1 - hi)] = e;
  }
}

// ---------------------------------------------------------------- sliced factor
// The off-diagonal blocks of L are also kept as kSlices signed 7-bit digit
// planes, so that the left-looking products run exactly on the int8 matrix
// cores (the splitting scheme of Ozaki, Ogita, Oishi and Rump, Numerical
// Algorithms 2012, with integer slices): row i has a power-of-two scale 2^e_i
// bounding its entries, and
//   L_im ~ 2^e_i * sum_p d_p(i,m) 2^-7(p+1),   |d_0| <= 126, |d_p| <= 64 after,
// a base-128 expansion of L_im 2^-e_i whose digits are each rounded to the
// nearest integer (so the dropped remainder is at most half the last digit's
// weight and carries no bias across a long sum).  A product sum_m L_im L_jm is
// then a sum over digit pairs (p, q) of integer dot products, exact in int32,
// weighted by 2^(e_i + e_j - 7(p + q + 2)).  Pairs with p + q >= kSlices are
// dropped: their weight is below the expansion's own remainder.  With
// kSlices = 6 each entry carries 42 bits relative to its row bound; products
// over 2048 terms come out within about 2^-35 sqrt(A_ii A_jj), against 2^-24
// for an fp32 product and far below the fp32 precision of everything
// downstream of the factor.
//
// Storage: per Hessian, tile (I, K) of 64x64 is kSlices contiguous 4 KB
// planes, row-major, at ((I * nbk + K) * kSlices) * 4096 bytes; the planes
// occupy the inverse's buffer (8 c^2 bytes per Hessian), which is free until
// the factorisation has finished.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
constexpr int kLqTile = kSlices * kNb * kNb;   // bytes of one sliced 64x64 tile
constexpr int kLqPitch = 80;                    // LDS row pitch (bytes): conflict-free 16-byte reads

__device__ __forceinline__ int64_t lq_offset(int c, int m, int I, int K) {
  return (int64_t)m * c * c * 8 + ((int64_t)I * (c / kNb) + K) * kLqTile;
}

// Step k: L_kk = chol(T_k) and Dinv_k = L_kk^-1, by the workgroup of the
// left-looking step that has just written T_k (its diagonal tile), so the
// factorisation overlaps the off-diagonal tiles still in progress.  Wave 0
// factors (lane r holds row r of T_k); wave 1 inverts (lane r holds column r
// of X = L_kk^-1, eliminated forward on L X = I, starting from the identity);
// waves 2 and 3 repeat wave 1's arithmetic on private registers and write
// nothing, so that every wave of the workgroup takes the same barriers.  At
// step J wave 0 finishes column J of L and puts it in LDS with 1 / L_JJ; then
// the waves apply the same rank-one update with that column, read as
// broadcasts: wave 0 to the later columns of its row, wave 1 to the rows of
// its column below J once X_Jr is final.  The column is double-buffered, so
// one barrier per step orders everything.  The template recursion keeps every
// register index a compile-time constant.
__device__ __forceinline__ double lane_value(double v, int src) {
  const uint64_t b = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)b, src);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(b >> 32), src);
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

template <int J>
__device__ __forceinline__ void diag_step(double (&v)[kNb], int r, bool factor, bool& bad,
                                          double (*col)[kNb + 2]) {
  double* cj = col[J & 1];
  if (factor) {
    double d = lane_value(v[J], J);
    if (!(d > 0.0)) {
      bad = true;
      d = 1.0;
    }
    const double ljj = sqrt(d);
    if (r == J) v[J] = ljj;
    if (r > J) v[J] = v[J] / ljj;
    cj[r] = v[J];
    if (r == 0) cj[kNb] = 1.0 / ljj;
  }
  __syncthreads();
  if (!factor) v[J] *= cj[kNb];   // X_Jr is final (zero for r > J)
  // rows above J of the factoring wave hold nothing of L: leave them alone
  const double mult = (factor && r <= J) ? 0.0 : v[J];
#pragma unroll
  for (int cc = J + 1; cc < kNb; ++cc) v[cc] = fma(-mult, cj[cc], v[cc]);
  if constexpr (J + 1 < kNb) diag_step<J + 1>(v, r, factor, bad, col);
}

__device__ __forceinline__ void diag_block(const double* __restrict__ A, int c, int k, int m,
                                           double* __restrict__ dinv, int* __restrict__ status,
                                           int* __restrict__ mstat, int m_base,
                                           double (*col)[kNb + 2]) {
  const int r = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool factor = wave == 0;
  const int64_t k0 = (int64_t)k * kNb;
  double v[kNb];
  if (factor) {
    const double* row = A + (k0 + r) * c + k0;
#pragma unroll
    for (int cc = 0; cc < kNb; cc += 2) {
      const double2 t = *reinterpret_cast<const double2*>(row + cc);
      v[cc] = cc <= r ? t.x : 0.0;
      v[cc + 1] = cc + 1 <= r ? t.y : 0.0;
    }
  } else {
#pragma unroll
    for (int cc = 0; cc < kNb; ++cc) v[cc] = cc == r ? 1.0 : 0.0;
  }
  bool bad = false;
  diag_step<0>(v, r, factor, bad, col);
  if (factor) {
    if (bad && r == 0) {
      atomicOr(status, kStatusNotPd);
      atomicOr(&mstat[m], kStatusNotPd);
      atomicMax(reinterpret_cast<unsigned*>(status) + kStatusMat, 0xffffffffu - (unsigned)(m_base + m));
    }
  } else if (wave == 1) {
    // Dinv_k row-major: lane r writes column r, each store one coalesced row
    double* D = dinv + ((int64_t)m * (c / kNb) + k) * kNb * kNb + r;
#pragma unroll
    for (int kk = 0; kk < kNb; ++kk) D[kk * kNb] = v[kk];
  }
}

// ---------------------------------------------------------------- left-looking Cholesky
// Step k, block row i >= k:  T_i = A[i][k] - sum_{m<k} L[i][m] L[k][m]^T, stored over A[i][k].
// Four waves each own a 32x32 quarter (v_mfma_i32_32x32x32_i8: lane l holds
// row l%32, bytes 16(l/32)..+15 of each 32-byte K step; result row
// 8(r/4) + 4(l/32) + r%4, column l%32).  The digit planes of chunks m+1 and
// m+2 are in flight in two register sets while the matrix cores work on chunk
// m in LDS.
__global__ __launch_bounds__(256, 2) void chol_left_kernel(double* __restrict__ Aall,
                                                           const int8_t* __restrict__ Lq,
                                                           const int* __restrict__ lexp,
                                                           const float* const* __restrict__ mats,
                                                           const uint8_t* __restrict__ dead,
                                                           const double* __restrict__ lamd, int c, int k,
                                                           double* __restrict__ dinv,
                                                           int* __restrict__ status,
                                                           int* __restrict__ mstat, int m_base,
                                                           int n_mats) {
  __shared__ __align__(16) int8_t As[kSlices][kNb][kLqPitch];
  __shared__ __align__(16) int8_t Bs[kSlices][kNb][kLqPitch];
  __shared__ __align__(16) double dcol[2][kNb + 2];
  // the tiles of one Hessian run on one XCD (workgroup b runs on XCD b % 8), so
  // its B panel, read by all of them, is fetched into one L2
  const int nt = c / kNb - k, total = nt * n_mats;
  const int per = (total + kXcds - 1) / kXcds;
  const int L = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
  if (L >= total) return;   // the whole workgroup, before any barrier
  const int m = L / nt, i = k + L % nt;
  const bool diag = i == k;
  double* A = Aall + (int64_t)m * c * c;
  const int64_t i0 = (int64_t)i * kNb, k0 = (int64_t)k * kNb;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  i32x16 acc[kSlices];
#pragma unroll
  for (int w = 0; w < kSlices; ++w) acc[w] = i32x16{};
  if (k > 0) {
    const int8_t* Pa = Lq + lq_offset(c, m, i, 0) + 16 * threadIdx.x;
    const int8_t* Pb = Lq + lq_offset(c, m, k, 0) + 16 * threadIdx.x;
    const int pr = threadIdx.x >> 2, pc = 16 * (threadIdx.x & 3);   // this thread's piece of a plane
    const int fa = 32 * wm + (lane & 31), fb = 32 * wn + (lane & 31), fk = 16 * (lane >> 5);
    i32x4 ra0[kSlices], rb0[kSlices], ra1[kSlices], rb1[kSlices];
    auto load = [&](i32x4 (&ra)[kSlices], i32x4 (&rb)[kSlices], int ch) {
      const int64_t nx = (int64_t)min(ch, k - 1) * kLqTile;
#pragma unroll
      for (int p = 0; p < kSlices; ++p) {
        ra[p] = *reinterpret_cast<const i32x4*>(Pa + nx + p * kNb * kNb);
        rb[p] = *reinterpret_cast<const i32x4*>(Pb + nx + p * kNb * kNb);
      }
    };
    load(ra0, rb0, 0);
    load(ra1, rb1, 1);
    auto step = [&](i32x4 (&ra)[kSlices], i32x4 (&rb)[kSlices], int mm) {
      __syncthreads();
#pragma unroll
      for (int p = 0; p < kSlices; ++p) {
        *reinterpret_cast<i32x4*>(&As[p][pr][pc]) = ra[p];
        *reinterpret_cast<i32x4*>(&Bs[p][pr][pc]) = rb[p];
      }
      __syncthreads();
      load(ra, rb, mm + 2);
      i32x4 a[kSlices][2], b[kSlices][2];
#pragma unroll
      for (int p = 0; p < kSlices; ++p)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          a[p][h] = *reinterpret_cast<const i32x4*>(&As[p][fa][fk + 32 * h]);
          b[p][h] = *reinterpret_cast<const i32x4*>(&Bs[p][fb][fk + 32 * h]);
        }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int p = 0; p < kSlices; ++p)
#pragma unroll
          for (int q = 0; q + p < kSlices; ++q)
            acc[p + q] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[p][h], b[q][h], acc[p + q], 0, 0, 0);
    };
    int mm = 0;
    for (; mm + 1 < k; mm += 2) {
      step(ra0, rb0, mm);
      step(ra1, rb1, mm + 1);
    }
    if (mm < k) step(ra0, rb0, mm);
  }
  // A[i][j] = Hd[c-1-i][c-1-j], read from H: its diagonal takes the dead-column
  // fix (H_jj := 1) and lambda
  const int* ex = lexp + (int64_t)m * c;
  const float* H = mats[m];
  const int col = 32 * wn + (lane & 31);
  const int ecol = ex[k0 + col];
  const int64_t hj = c - 1 - (k0 + col);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 32 * wm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (diag && col > row) continue;
    double sum = 0.0;
#pragma unroll
    for (int w = kSlices - 1; w >= 0; --w) sum += ldexp((double)acc[w][r], -7 * (w + 2));
    const int64_t hi = c - 1 - (i0 + row);
    double a = (double)H[hi * c + hj];
    if (hi == hj) a = (dead[(int64_t)m * c + hi] ? 1.0 : a) + lamd[m];
    A[(i0 + row) * c + k0 + col] = a - ldexp(sum, ex[i0 + row] + ecol);
  }
  if (diag) {
    // the whole workgroup: T_k is written, then factored and inverted
    __threadfence_block();
    __syncthreads();
    diag_block(A, c, k, m, dinv, status, mstat, m_base, dcol);
  }
}

// Step k, block row i > k:  L[i][k] = T_i Dinv_k^T.
__global__ __launch_bounds__(256) void chol_panel_kernel(double* __restrict__ Aall, int c, int k,
                                                         const double* __restrict__ dinv,
                                                         int8_t* __restrict__ Lq,
                                                         const int* __restrict__ lexp, int n_mats) {
  __shared__ double Ts[kNb][kNb + 1];
  __shared__ double Ds[kNb][kNb + 1];
  // the tiles of one Hessian run on one XCD, so its Dinv_k is fetched into one L2
  const int nt = c / kNb - k - 1, total = nt * n_mats;
  const int per = (total + kXcds - 1) / kXcds;
  const int L = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
  if (L >= total) return;   // the whole workgroup, before any barrier
  const int m = L / nt, i = k + 1 + L % nt;
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
  // digit planes of the tile: thread t writes 16 consecutive entries of row t/4
  __syncthreads();
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) Ts[Tile64::row(x, r)][Tile64::col(y)] = t.acc[x][y][r];
  __syncthreads();
  const int pr = threadIdx.x >> 2, pc = 16 * (threadIdx.x & 3);
  const int e = lexp[(int64_t)m * c + i0 + pr];
  uint32_t packed[kSlices][4];
#pragma unroll
  for (int p = 0; p < kSlices; ++p)
#pragma unroll
    for (int u = 0; u < 4; ++u) packed[p][u] = 0;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    // |x| <= 0.985, so the first digit is at most 126 and each later one, a
    // rounded remainder times 128, at most 64; the clamp only guards a factor
    // that has already failed (status not positive definite)
    double x = fmin(fmax(ldexp(Ts[pr][pc + u], -e), -0.984375), 0.984375);
#pragma unroll
    for (int p = 0; p < kSlices; ++p) {
      x *= 128.0;
      const double d = rint(x);
      x -= d;
      packed[p][u >> 2] |= ((uint32_t)(int)d & 0xffu) << (8 * (u & 3));
    }
  }
  int8_t* out = Lq + lq_offset(c, m, i, k) + 16 * threadIdx.x;
#pragma unroll
  for (int p = 0; p < kSlices; ++p)
    *reinterpret_cast<uint4*>(out + p * kNb * kNb) = make_uint4(packed[p][0], packed[p][1], packed[p][2], packed[p][3]);
}

// ---------------------------------------------------------------- triangular inverse
// X = L^-1, merged bottom-up over ranges of 64-column blocks.  For a range
// [a, b) split at mid, with X11 the inverse over [a, mid) and X22 over [mid, b):
//   X21 = -X22 L21 X11,   L21 = L[mid:b, a:mid]
// (the inverse of a 2x2 block lower-triangular matrix).  Level s merges ranges
// of 2s blocks (s = 1, 2, 4, ...); merges of one level are independent.  The
// leaves are the fp64 diagonal-block inverses Dinv of the factorisation.
// The factor L is fp64; the merges run at fp32 precision on the bf16 matrix
// cores: every operand x is split into three bf16 parts, x = x1 + x2 + x3 to
// within 2^-25 |x| (x1 = bf16(x), x2 = bf16(x - x1), x3 = bf16(x - x1 - x2)), and
// a product is the sum of the six part products above 2^-24 of it (x1y1, x1y2,
// x2y1, x1y3, x3y1, x2y2), each exact in fp32 and accumulated in fp32
// (v_mfma_f32_32x32x16_bf16, about 2.7 times the fp32 matrix rate).  The
// inverse is well conditioned relative to the factor (cond(L) = sqrt(cond(Hd))),
// and U is stored in fp32 in any case.
// Each merge is two batched GEMMs:
//   phase 0:  T = L21 X11     (X11 lower triangular: only k >= column counts)
//   phase 1:  X21 = -X22 T    (X22 lower triangular: only k <= row counts)
// fp32 storage, in the (fp64-sized) X buffer of each Hessian:
//   X32  [c][c]  X row-major (lower triangle); its strictly upper triangle holds
//                T^T during a level: T[row][col] at X32[col][row]
//   XT32 [c][c]  X^T row-major (upper triangle)
// so every GEMM operand is a K-contiguous row.  Every X element is final when
// written, so U = J X J and U^T get their values at once.

// Leaves: X[i][i] = Dinv_i (zeros above the diagonal), in X32, XT32, U and U^T.
__global__ __launch_bounds__(256) void trtri_leaf_kernel(int c, const double* __restrict__ dinv,
                                                         double* __restrict__ Xall,
                                                         float* __restrict__ Uall,
                                                         float* __restrict__ UTall) {
  const int m = blockIdx.y, i = blockIdx.x;
  float* X32 = reinterpret_cast<float*>(Xall + (int64_t)m * c * c);
  float* XT32 = X32 + (int64_t)c * c;
  float* U = Uall + (int64_t)m * c * c;
  float* UT = UTall ? UTall + (int64_t)m * c * c : nullptr;
  const double* Di = dinv + ((int64_t)m * (c / kNb) + i) * kNb * kNb;
  const int64_t i0 = (int64_t)i * kNb;
  for (int idx = threadIdx.x; idx < kNb * kNb; idx += 256) {
    const int r = idx >> 6, cc = idx & 63;
    const float v = cc <= r ? (float)Di[idx] : 0.0f;
    X32[(i0 + r) * c + i0 + cc] = v;
    if (cc <= r) U[(c - 1 - (i0 + r)) * c + (c - 1 - (i0 + cc))] = v;
    // transposed element (consecutive threads step its column)
    const int rr = idx & 63, c2 = idx >> 6;
    const float vt = c2 <= rr ? (float)Di[rr * kNb + c2] : 0.0f;
    XT32[(i0 + c2) * c + i0 + rr] = vt;
    if (UT && c2 <= rr) UT[(c - 1 - (i0 + c2)) * c + (c - 1 - (i0 + rr))] = vt;
  }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kTT = 128;          // merge tile: rows and columns
constexpr int kTK = 16;           // K chunk (one MFMA step)
constexpr int kTRow = 48;         // LDS row pitch (bytes) of one bf16 part: 16 k + padding,
                                  // so the 16-byte fragment reads of 16 lanes hit distinct banks
constexpr int kTPart = kTT * kTRow;     // one part of one operand (bytes)
constexpr int kTBuf = 6 * kTPart;       // one stage: three parts of A, three of B

// bf16 round to nearest even of an fp32 value (finite inputs), as raw bits
__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// One 128x128 tile of one merge.  256 threads = 4 waves of 64x64 (2x2 blocks of
// v_mfma_f32_32x32x16_bf16, six part products each).  Both operands are
// K-contiguous rows staged through LDS in chunks of 16 as three bf16 parts,
// double-buffered with two register stages; a lane's operand fragment of a
// block is one 16-byte LDS read per part (row l%32, k 8(l/32) .. +7).  Phase 0
// walks K downwards from the merge's common end, phase 1 upwards from its
// common start, so the tiles of a merge read the same chunks at about the same
// time; tiles of one merge are mapped to one XCD (workgroup b runs on XCD b % 8).
template <int PHASE>
__global__ __launch_bounds__(256, 2) void trtri_merge_kernel(const double* __restrict__ Aall,
                                                             double* __restrict__ Xall,
                                                             float* __restrict__ Uall,
                                                             float* __restrict__ UTall, int c, int s,
                                                             int n_merge, int tc, int n_mats) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kTBuf];   // stage 0, stage 1
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
  const int k0 = PHASE == 0 ? c0 : mid * kNb;
  const int k1 = PHASE == 0 ? mid * kNb : min(r0 + kTT, b * kNb);
  const int nch = (k1 - k0) / kTK;   // a multiple of 4: K ranges are multiples of 64
  const double* A = Aall + (int64_t)m * c * c;
  float* X32 = reinterpret_cast<float*>(Xall + (int64_t)m * c * c);
  float* XT32 = X32 + (int64_t)c * c;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, li = lane & 31;
  const bool active = wm * 64 < nr && wn * 64 < nc;

  // MFMA A operand rows (tile row i):  phase 0 L21[r0+i][k] (fp64), phase 1 X22[r0+i][k]
  // MFMA B operand rows (tile column j): phase 0 X11^T[c0+j][k] = XT32, phase 1 T^T[c0+j][k] = X32
  // A fetch only issues loads (raw values in registers); conversion and the
  // triangular masks happen when the stage is written to LDS, so a prefetch
  // is never waited for before its turn.
  struct Stage {
    double2 alo[2], ahi[2];   // phase 0: fp64 A operand
    float4 a[2], b[2];
  };
  // thread t moves 16-byte chunks q = t + 256u: row q/4, k = 4(q%4) .. +3.
  // Every fetch is unconditional (chunk and row indices are clamped into
  // range), so the compiler counts outstanding loads exactly; clamped rows
  // (past nr or nc) only feed waves that are inactive for this tile.
  auto chunk_base = [&](int ch) {
    ch = ch < nch ? ch : nch - 1;
    return PHASE == 0 ? k1 - (ch + 1) * kTK : k0 + ch * kTK;
  };
  auto fetch = [&](Stage& rg, int ch) {
    const int kb = chunk_base(ch);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = tid + 256 * u, row = q >> 2, kk = kb + 4 * (q & 3);
      const int ra = min(row, nr - 1), rb = min(row, nc - 1);
      if (PHASE == 0) {
        const double* src = A + (int64_t)(r0 + ra) * c + kk;
        rg.alo[u] = *reinterpret_cast<const double2*>(src);
        rg.ahi[u] = *reinterpret_cast<const double2*>(src + 2);
        rg.b[u] = *reinterpret_cast<const float4*>(XT32 + (int64_t)(c0 + rb) * c + kk);
      } else {
        rg.a[u] = *reinterpret_cast<const float4*>(X32 + (int64_t)(r0 + ra) * c + kk);
        rg.b[u] = *reinterpret_cast<const float4*>(X32 + (int64_t)(c0 + rb) * c + kk);
      }
    }
  };
  // four values -> three bf16 parts, each four consecutive k (8 bytes) of one row
  auto put_parts = [&](char* base, int row, int kc, const float (&v)[4]) {
    uint32_t w[3][2];
    float r[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      uint32_t hb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hb[e] = bf16_bits_rne(r[e]);
        r[e] = r[e] - __uint_as_float(hb[e] << 16);   // exact: the remainder of a rounding
      }
      w[p][0] = hb[0] | (hb[1] << 16);
      w[p][1] = hb[2] | (hb[3] << 16);
    }
#pragma unroll
    for (int p = 0; p < 3; ++p)
      *reinterpret_cast<uint2*>(base + p * kTPart + row * kTRow + 2 * kc) = make_uint2(w[p][0], w[p][1]);
  };
  auto stage = [&](const Stage& rg, int buf, int ch) {
    const int kb = chunk_base(ch);
    char* As = lds + buf * kTBuf;
    char* Bs = As + 3 * kTPart;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = tid + 256 * u, row = q >> 2, kc = 4 * (q & 3), kk = kb + kc;
      float4 va, vb = rg.b[u];
      if (PHASE == 0) {
        va = make_float4((float)rg.alo[u].x, (float)rg.alo[u].y, (float)rg.ahi[u].x, (float)rg.ahi[u].y);
        // X11^T row cc: X11[k][cc] is nonzero for k >= cc
        const int cc = c0 + min(row, nc - 1);
        vb.x = kk < cc ? 0.f : vb.x;
        vb.y = kk + 1 < cc ? 0.f : vb.y;
        vb.z = kk + 2 < cc ? 0.f : vb.z;
        vb.w = kk + 3 < cc ? 0.f : vb.w;
      } else {
        // X22 lower triangular: k <= row
        va = rg.a[u];
        const int rr = r0 + min(row, nr - 1);
        va.x = kk > rr ? 0.f : va.x;
        va.y = kk + 1 > rr ? 0.f : va.y;
        va.z = kk + 2 > rr ? 0.f : va.z;
        va.w = kk + 3 > rr ? 0.f : va.w;
      }
      const float fa[4] = {va.x, va.y, va.z, va.w}, fb[4] = {vb.x, vb.y, vb.z, vb.w};
      put_parts(As, row, kc, fa);
      put_parts(Bs, row, kc, fb);
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f32x16{};
  auto multiply = [&](int buf) {
    if (!active) return;
    const char* As = lds + buf * kTBuf + (wm * 64 + li) * kTRow + 16 * h;
    const char* Bs = lds + buf * kTBuf + 3 * kTPart + (wn * 64 + li) * kTRow + 16 * h;
    bf16x8 av[2][3], bv[2][3];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        av[x][p] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(As + p * kTPart + 32 * x * kTRow));
        bv[x][p] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Bs + p * kTPart + 32 * x * kTRow));
      }
    // smallest part products first; x1 y1 last
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[x][1], bv[y][1], acc[x][y], 0, 0, 0);
        acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[x][0], bv[y][2], acc[x][y], 0, 0, 0);
        acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[x][2], bv[y][0], acc[x][y], 0, 0, 0);
        acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[x][0], bv[y][1], acc[x][y], 0, 0, 0);
        acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[x][1], bv[y][0], acc[x][y], 0, 0, 0);
        acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[x][0], bv[y][0], acc[x][y], 0, 0, 0);
      }
  };

  Stage g0, g1;
  fetch(g0, 0);
  stage(g0, 0, 0);
  fetch(g1, 1);
  fetch(g0, 2);
  __syncthreads();
#pragma unroll 1
  for (int st = 0; st < nch; st += 2) {
    multiply(0);
    stage(g1, 1, st + 1);
    fetch(g1, st + 3);
    __syncthreads();
    multiply(1);
    stage(g0, 0, st + 2);
    fetch(g0, st + 4);
    __syncthreads();
  }
  if (!active) return;
  // element (i, j) of the tile: i = wm*64 + 32x + 8(r/4) + 4h + r%4, j = wn*64 + 32y + li
  float* U = Uall + (int64_t)m * c * c;
  float* UT = UTall ? UTall + (int64_t)m * c * c : nullptr;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int col = c0 + wn * 64 + 32 * y + li;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = r0 + wm * 64 + 32 * x + 8 * q + 4 * h;   // rows row .. row+3
        const f32x16& v = acc[x][y];
        if (PHASE == 0) {
          // T^T[col][row .. row+3] in X32's strictly upper triangle
          *reinterpret_cast<float4*>(X32 + (int64_t)col * c + row) =
              make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        } else {
          const float e0 = -v[4 * q], e1 = -v[4 * q + 1], e2 = -v[4 * q + 2], e3 = -v[4 * q + 3];
          *reinterpret_cast<float4*>(XT32 + (int64_t)col * c + row) = make_float4(e0, e1, e2, e3);
          const float ev[4] = {e0, e1, e2, e3};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            X32[(int64_t)(row + r) * c + col] = ev[r];
            U[(int64_t)(c - 1 - (row + r)) * c + (c - 1 - col)] = ev[r];
          }
          // U^T row c-1-col, columns c-1-row-3 .. c-1-row (ascending)
          if (UT)
            *reinterpret_cast<float4*>(UT + (int64_t)(c - 1 - col) * c + (c - 4 - row)) =
                make_float4(e3, e2, e1, e0);
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
  int* lexp = p.lexp + (int64_t)m0 * c;
  int8_t* Lq = reinterpret_cast<int8_t*>(X);   // free until the inverse starts
  int* mstat = p.mstat + m0;
  hipLaunchKernelGGL(diag_stats_kernel, dim3(n), dim3(256), 0, s, mats, c, p.damp, dead, lamd, lam, lexp,
                     mstat, p.status, m0);
  for (int k = 0; k < nbk; ++k) {
    const int per = ((nbk - k) * n + kXcds - 1) / kXcds;
    hipLaunchKernelGGL(chol_left_kernel, dim3(per * kXcds), dim3(256), 0, s, A, Lq, lexp, mats, dead, lamd, c, k,
                       dinv, p.status, mstat, m0, n);
    if (k == 0 && step0_done) hipEventRecord(step0_done, s);
    if (k + 1 < nbk) {
      const int pper = ((nbk - k - 1) * n + kXcds - 1) / kXcds;
      hipLaunchKernelGGL(chol_panel_kernel, dim3(pper * kXcds), dim3(256), 0, s, A, c, k, dinv, Lq, lexp, n);
    }
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
