// Quantization phase: GPTQ column-sequential quantize-and-propagate with lazy
// block updates and per-group asymmetric grids.
//
// CLHA summary, section 2.2 step 3: standard GPTQ updates on H_comb; section
// 2.3 (CLHA-MP): b+1 bits for always-active shared experts, b for routed ones
// (the bit width is per job).  The GPTQ steps follow Frantar et al. (ICLR 2023):
// for column j, with U the upper Cholesky factor of Hd^-1,
//   err_j = (w_j - dequant(quant(w_j))) / U_jj,   w_k -= err_j U_jk  (k > j),
// applied eagerly inside a block of columns and lazily (one rank-64 product)
// to the columns after the block.  The grid of each (row, group) is fitted at
// the group's first column on the weights updated so far.
//
// Work decomposition.  Rows are independent given U.  Columns are processed
// in superblocks of kSuper (256) columns, each in two launches:
//   * the panel kernel: one wavefront owns a slab of 64 rows, one thread one
//     row.  The row's current 64-column block lives in 64 registers; the column
//     loop is fully unrolled, so quantization, the error and the rank-1 update
//     of the rest of the block are register arithmetic with no barrier (the U
//     values of column j are the same for every row: LDS broadcasts).  Codes,
//     scales and zero points are decided in fp32 with IEEE division and
//     round-half-to-even.  After each 64-column block its errors update the
//     later columns of the same superblock (fp32 matrix cores,
//     v_mfma_f32_32x32x2f32, 64-row x 32-column tiles) and are stored for the
//     next launch;
//   * the trailing kernel: Wf[:, later] -= E U[superblock, later] for every row
//     of every job at once, a batched GEMM with K = 256 in 128x128 tiles, run
//     exactly on the int8 matrix cores over 28-bit digit expansions of E and U
//     (see "trailing update"), so each later weight is read and written once per
//     superblock instead of once per 64 columns.
// Options (GPTQ's activation order and static groups).  Activation order
// processes the columns by decreasing H_ii (a dead column counts as 1, ties by
// column index): the Hessian is permuted once (H[perm][:, perm]) and factored
// as usual, the working copy holds the permuted columns, and after the last
// superblock each row's codes are moved back to their natural columns; a grid
// then belongs to a run of `group` processed columns, and g_idx gives each
// column's grid.  Static groups fit every natural group's grid once, before
// any update, on the weights with dead columns zeroed; the column loop loads
// a column's grid instead of fitting it.
// The loss uses the OBS identity: sum_j err_j^2 = tr[(Wq - W) Hd (Wq - W)^T],
// so the undamped loss is sum err^2 - lambda ||Wq - W||^2 (W after zeroing
// dead columns); ||Wq - W||^2 is a separate coalesced pass over the outputs.
#include "kernels.h"

namespace clha {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int kRB = 64;             // register block: columns held per thread

// Four consecutive weights (16-byte aligned fp32 or 8-byte aligned bf16).
__device__ __forceinline__ float4 load_w4(const void* W, int dtype, int64_t i) {
  if (dtype == 1) {
    const uint2 b = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(W) + i);
    return make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xffff0000u),
                       __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xffff0000u));
  }
  return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(W) + i);
}

__device__ __forceinline__ float load_w1(const void* W, int dtype, int64_t i) {
  if (dtype == 1) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(W)[i] << 16);
  return reinterpret_cast<const float*>(W)[i];
}

__device__ __forceinline__ void fit_grid(float xmin, float xmax, float fmaxq, float& s, float& z) {
  xmin = fminf(xmin, 0.0f);
  xmax = fmaxf(xmax, 0.0f);
  if (xmin == 0.0f && xmax == 0.0f) {
    xmin = -1.0f;
    xmax = 1.0f;
  }
  s = __fdiv_rn(__fsub_rn(xmax, xmin), fmaxq);
  z = rintf(__fdiv_rn(-xmin, s));
}

// U is read-only while the GPTQ kernel runs; reading it through the constant
// address space lets the compiler fetch the per-column U values (identical for
// every row of the wave) with scalar loads into SGPRs.
typedef const __attribute__((address_space(4))) float* const_fptr;

struct ColCtx {
  const float* ublk;                // the block's diagonal 64x64 U block in LDS, row stride 64
  const float* urcp;                // 1 / U_jj of the block's columns, in LDS
  int c;
  float fmaxq;
  float* scales;
  uint8_t* zeros;
  bool live;
  // static grids: the block's first natural group, the natural column of each
  // of the block's processed columns (activation order), and the index of this
  // row's first grid in scales/zeros.  Rows past the matrix use row 0's grids
  // (their weights are zero, so their errors stay zero and no code is stored).
  int gfirst;
  const int* gperm;
  uint32_t rowg;
};

// Grid modes of the column loop: fitted at each group's first column (dynamic),
// loaded at each group's first column (static, natural order), or loaded for
// every column, kLook columns ahead (static under activation order, where
// consecutive processed columns belong to unrelated natural groups).
enum { kGridFit = 0, kGridStatic = 1, kGridStaticPerm = 2 };
constexpr int kLook = 4;

// Column JJ of the register block (the recursion makes every register index a
// compile-time constant, so the block stays in registers).
// Grids fitted inside a register block, stored after it (a store inside the
// column chain would be a branch on the row's liveness, and the compiler would
// then hoist and spill the U block).
constexpr int grids_per_block(int G) { return G <= kRB ? kRB / G : 1; }

template <int G, int MODE, int JJ>
__device__ __forceinline__ void column_steps(float (&w)[kRB], uint32_t (&packed)[kRB / 4], float& s,
                                             float& z, float (&sq)[kLook], float (&zq)[kLook],
                                             float (&sb)[grids_per_block(G)], float (&zb)[grids_per_block(G)],
                                             double& obs, const ColCtx& cx) {
  if constexpr (MODE == kGridStaticPerm) {
    s = sq[JJ % kLook];
    z = zq[JJ % kLook];
    if constexpr (JJ + kLook < kRB) {
      // unconditional (rows past the matrix read row 0's grids, see ColCtx):
      // a branch here would split the column and let the compiler hoist and
      // spill the whole U block
      const uint32_t gi = cx.rowg + (uint32_t)(cx.gperm[JJ + kLook] / G);
      sq[JJ % kLook] = cx.scales[gi];
      zq[JJ % kLook] = (float)cx.zeros[gi];
    }
  } else if constexpr (MODE == kGridStatic) {
    if constexpr (G <= kRB && (JJ % G) == 0) {
      const uint32_t gi = cx.rowg + (uint32_t)(cx.gfirst + JJ / G);
      s = cx.scales[gi];
      z = (float)cx.zeros[gi];
    }
  } else {
    if constexpr (G <= kRB && (JJ % G) == 0) {
      float mn = w[JJ], mx = w[JJ];
#pragma unroll
      for (int u = 1; u < G; ++u) {
        mn = fminf(mn, w[JJ + u]);
        mx = fmaxf(mx, w[JJ + u]);
      }
      fit_grid(mn, mx, cx.fmaxq, s, z);
      sb[JJ / G] = s;
      zb[JJ / G] = z;
    }
  }
  const float* urow = cx.ublk + JJ * kRB;
  const float x = w[JJ];
  float q = rintf(__fdiv_rn(x, s)) + z;
  q = fminf(fmaxf(q, 0.0f), cx.fmaxq);
  const float what = __fmul_rn(s, __fsub_rn(q, z));
  // the error is propagation arithmetic, not a decision: multiplied by 1/U_jj,
  // rounded once per block (within an ulp of the quotient)
  const float e = __fmul_rn(__fsub_rn(x, what), cx.urcp[JJ]);
  packed[JJ >> 2] |= (uint32_t)q << (8 * (JJ & 3));
  obs += (double)e * (double)e;
  w[JJ] = e;
#pragma unroll
  for (int kk = JJ + 1; kk < kRB; ++kk) w[kk] = fmaf(-e, urow[kk], w[kk]);
  // keep each look-ahead load in its own column instead of all at the top
  if constexpr (MODE == kGridStaticPerm) __builtin_amdgcn_sched_barrier(0);
  if constexpr (JJ + 1 < kRB) column_steps<G, MODE, JJ + 1>(w, packed, s, z, sq, zq, sb, zb, obs, cx);
}

// One 64-row x 32-column tile of the far update: the A operands (U) and the
// current W values, loaded ahead of use.
struct TileBuf {
  float4 u[kRB / 8];          // A operands: U^T row jt+lc, columns i1+32kh .. +31
  float4 wa[4], wb[4];        // W rows lc and 32+lc, columns jt+8q+4kh .. +3
  __device__ __forceinline__ void load(const float* UT, const float* wr0, const float* wr1, int c,
                                       int jt, int ucol) {
    const float* ut = UT + (int64_t)jt * c + ucol;
#pragma unroll
    for (int m = 0; m < kRB / 8; ++m) u[m] = *reinterpret_cast<const float4*>(ut + 4 * m);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      wa[q] = *reinterpret_cast<const float4*>(wr0 + jt + 8 * q);
      wb[q] = *reinterpret_cast<const float4*>(wr1 + jt + 8 * q);
    }
  }
  // eb: the block's negated errors in B-operand order in LDS, eb[st*128 + mb*64 + lane]
  __device__ __forceinline__ void apply(const float* eb, float* wr0, float* wr1, int jt, int lane) {
    f32x16 acc0, acc1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc0[4 * q] = wa[q].x; acc0[4 * q + 1] = wa[q].y; acc0[4 * q + 2] = wa[q].z; acc0[4 * q + 3] = wa[q].w;
      acc1[4 * q] = wb[q].x; acc1[4 * q + 1] = wb[q].y; acc1[4 * q + 2] = wb[q].z; acc1[4 * q + 3] = wb[q].w;
    }
    // an opaque zero keeps the 64 LDS reads inside the tile loop instead of
    // holding them in registers for the whole update
    int opaque;
    asm volatile("v_mov_b32 %0, 0" : "=v"(opaque));
    const float* e = eb + lane + opaque;
#pragma unroll
    for (int st = 0; st < kRB / 2; ++st) {
      const float a = (&u[st >> 2].x)[st & 3];
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, e[st * 128], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, e[st * 128 + 64], acc1, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<float4*>(wr0 + jt + 8 * q) =
          make_float4(acc0[4 * q], acc0[4 * q + 1], acc0[4 * q + 2], acc0[4 * q + 3]);
      *reinterpret_cast<float4*>(wr1 + jt + 8 * q) =
          make_float4(acc1[4 * q], acc1[4 * q + 1], acc1[4 * q + 2], acc1[4 * q + 3]);
    }
  }
};

// Wf[:, jt0:cend] -= E U[i1:i1+64, jt0:cend] for one 64-row slab, E = the block's
// errors (thread-per-row in e[]).  Transposed product on the fp32 matrix cores:
// C[i][j] = sum_k U[i1+k][jt+i] E[j][k] is the update of W[row j][column jt+i].
// With U as the A operand (read from U^T, so a lane's operands are contiguous)
// and -E as the B operand, each lane's 16 results are 4 runs of 4 consecutive
// columns of one row.  MFMA step st contracts k = st (lanes 0..31) and
// k = st+32 (lanes 32..63); the B operands come from the row-owner registers by
// one cross-half shuffle per step and are staged in LDS.  Tiles are
// double-buffered: the next tile's U and W load while the current tile's
// products run.
__device__ __forceinline__ void far_update(const float (&e)[kRB], float* Wf, const float* UT, int c,
                                           int i1, int jt0, int cend, int lane, float* eb) {
  const int kh = lane >> 5, lc = lane & 31;
  // B operands for rows 0..31 (mb 0) and 32..63 (mb 1), negated, into LDS
#pragma unroll
  for (int st = 0; st < kRB / 2; ++st) {
    const float lo = e[st], hi = e[st + kRB / 2];
    const float lo_x = __shfl_xor(lo, 32), hi_x = __shfl_xor(hi, 32);
    eb[st * 128 + lane] = -(kh == 0 ? lo : hi_x);        // row lc:    k = st / st+32
    eb[st * 128 + 64 + lane] = -(kh == 0 ? lo_x : hi);   // row 32+lc
  }
  __syncthreads();
  const float* utl = UT + (int64_t)lc * c;            // U^T row jt+lc
  const int ucol = i1 + (kRB / 2) * kh;
  float* wr0 = Wf + (int64_t)lc * c + 4 * kh;          // rows lc and 32+lc, columns jt+8q+4kh
  float* wr1 = wr0 + (int64_t)32 * c;
  TileBuf x, y;
  x.load(utl, wr0, wr1, c, jt0, ucol);
#pragma unroll 1
  for (int jt = jt0; jt < cend; jt += 64) {
    const bool second = jt + 32 < cend;
    if (second) y.load(utl, wr0, wr1, c, jt + 32, ucol);
    x.apply(eb, wr0, wr1, jt, lane);
    if (!second) break;
    if (jt + 64 < cend) x.load(utl, wr0, wr1, c, jt + 64, ucol);
    y.apply(eb, wr0, wr1, jt + 32, lane);
  }
}

// Columns [c0, min(c, c0 + kSuper)) of every slab.
template <int G, int MODE>
__global__ __launch_bounds__(64, 2) void gptq_panel_kernel(GptqPlan p, int c0, JobRange jr) {
  __shared__ float eb[kRB * 64];   // the block's errors as MFMA B operands
  __shared__ float urcp[kRB];      // 1 / U_jj of the current block
  const int c = p.cols;
  const int cend = min(c, c0 + kSuper);
  const int gslab = jr.slab0 + (int)blockIdx.x;
  int lo = jr.j0, hi = jr.j1;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.jobs[mid].slab_base <= gslab) lo = mid; else hi = mid;
  }
  const GJob job = p.jobs[lo];
  const int slab = gslab - job.slab_base;
  const int row0 = slab * kGptqRows;
  const int nrows = min(kGptqRows, job.rows - row0);
  const float* __restrict__ U = p.U + (int64_t)job.mat * c * c;
  const float* __restrict__ UT = p.UT + (int64_t)job.mat * c * c;
  const uint8_t* __restrict__ dead = p.dead + (int64_t)job.mat * c;
  float* Wf = p.wf + job.wf_off + (int64_t)row0 * c;
  const float fmaxq = (float)((1 << job.bits) - 1);
  const int ngroups_row = c / G;
  const int lane = threadIdx.x;
  const bool live = lane < nrows;

  // first superblock: its columns of the fp32 working copy (rows past the
  // matrix are zero, dead columns zeroed); the first trailing update fills the
  // later columns straight from W.  With an option on, the preparation pass
  // has written the whole working copy.
  if (c0 == 0 && !(p.act_order | p.static_groups)) {
    for (int r = 0; r < kGptqRows; ++r) {
      for (int col = 4 * lane; col < cend; col += 256) {
        const float4 v = r < nrows ? load_w4(job.W, job.dtype, (int64_t)(row0 + r) * c + col)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
        const uchar4 dd = *reinterpret_cast<const uchar4*>(dead + col);
        *reinterpret_cast<float4*>(Wf + (int64_t)r * c + col) =
            make_float4(dd.x ? 0.f : v.x, dd.y ? 0.f : v.y, dd.z ? 0.f : v.z, dd.w ? 0.f : v.w);
      }
    }
    __threadfence_block();
    __syncthreads();
  }
  // this row's errors of the superblock, for the trailing update
  float* erow = cend < c ? p.ebuf + (job.wf_off / c + row0 + lane) * kSuper : nullptr;

  double obs = 0.0;
  float s = 1.0f, z = 0.0f;
  float* myrow = Wf + (int64_t)lane * c;
  const int64_t rowg = (int64_t)(row0 + lane) * ngroups_row;   // this row's first grid
  const int* perm = p.perm ? p.perm + (int64_t)job.mat * c : nullptr;

  for (int i1 = c0; i1 < cend; i1 += kRB) {
    // U's diagonal block of these 64 columns into LDS (coalesced, all loads in
    // flight together); every lane then reads the same U values (broadcast)
    __syncthreads();
    {
      // lane moves rows lane/16 + 4m, columns 4 (lane % 16) .. +3; an opaque
      // zero keeps the addresses from being hoisted out of the block loop
      int opaque;
      asm volatile("v_mov_b32 %0, 0" : "=v"(opaque));
      const int r0 = (lane >> 4) + opaque, q4 = 4 * (lane & 15);
      const float* ug = U + (int64_t)(i1 + r0) * c + i1 + q4;
      float* ul = eb + r0 * kRB + q4;
      const int64_t step = 4 * (int64_t)c;
      float4 ub[kRB * kRB / 4 / 64];
#pragma unroll
      for (int m = 0; m < kRB * kRB / 4 / 64; ++m) ub[m] = *reinterpret_cast<const float4*>(ug + m * step);
#pragma unroll
      for (int m = 0; m < kRB * kRB / 4 / 64; ++m) *reinterpret_cast<float4*>(ul + 4 * m * kRB) = ub[m];
    }
    __syncthreads();
    urcp[lane] = __fdiv_rn(1.0f, eb[lane * kRB + lane]);
    __syncthreads();
    float w[kRB];
#pragma unroll
    for (int q = 0; q < kRB / 4; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(myrow + i1 + 4 * q);
      w[4 * q] = v.x;
      w[4 * q + 1] = v.y;
      w[4 * q + 2] = v.z;
      w[4 * q + 3] = v.w;
    }
    if (MODE == kGridStatic && G > kRB && (i1 % G) == 0) {
      s = job.scales[(live ? rowg : 0) + i1 / G];
      z = (float)job.zeros[(live ? rowg : 0) + i1 / G];
    } else if (MODE == kGridFit && G > kRB && (i1 % G) == 0) {
      // group wider than the register block: its other columns are current in Wf
      float mn = INFINITY, mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < kRB; ++u) {
        mn = fminf(mn, w[u]);
        mx = fmaxf(mx, w[u]);
      }
      for (int u = kRB; u < G; u += 4) {
        const float4 v = *reinterpret_cast<const float4*>(myrow + i1 + u);
        mn = fminf(fminf(mn, v.x), fminf(fminf(v.y, v.z), v.w));
        mx = fmaxf(fmaxf(mx, v.x), fmaxf(fmaxf(v.y, v.z), v.w));
      }
      fit_grid(mn, mx, fmaxq, s, z);
      if (live) {
        const int64_t o = (int64_t)(row0 + lane) * ngroups_row + i1 / G;
        job.scales[o] = s;
        job.zeros[o] = (uint8_t)z;
      }
    }
    uint32_t packed[kRB / 4];
#pragma unroll
    for (int q = 0; q < kRB / 4; ++q) packed[q] = 0u;
    const uint32_t grow = live ? (uint32_t)rowg : 0u;
    ColCtx cx{eb, urcp, c, fmaxq, job.scales, job.zeros, live, i1 / G, perm ? perm + i1 : nullptr, grow};
    float sq[kLook], zq[kLook];
#pragma unroll
    for (int k = 0; k < kLook; ++k) {
      sq[k] = 1.0f;
      zq[k] = 0.0f;
      if (MODE == kGridStaticPerm) {
        const uint32_t gi = grow + (uint32_t)(perm[i1 + k] / G);
        sq[k] = job.scales[gi];
        zq[k] = (float)job.zeros[gi];
      }
    }
    float sb[grids_per_block(G)], zb[grids_per_block(G)];
    column_steps<G, MODE, 0>(w, packed, s, z, sq, zq, sb, zb, obs, cx);
    if (MODE == kGridFit && G <= kRB && live) {
#pragma unroll
      for (int k = 0; k < grids_per_block(G); ++k) {
        job.scales[rowg + i1 / G + k] = sb[k];
        job.zeros[rowg + i1 / G + k] = (uint8_t)zb[k];
      }
    }
    if (live) {
      uint8_t* cp = job.codes + (int64_t)(row0 + lane) * c + i1;
#pragma unroll
      for (int q = 0; q < kRB / 16; ++q)
        *reinterpret_cast<uint4*>(cp + 16 * q) =
            make_uint4(packed[4 * q], packed[4 * q + 1], packed[4 * q + 2], packed[4 * q + 3]);
    }

    // rows past the matrix have zero weights and so zero errors
    if (erow) {
#pragma unroll
      for (int q = 0; q < kRB / 4; ++q)
        *reinterpret_cast<float4*>(erow + (i1 - c0) + 4 * q) =
            make_float4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
    }
    // lazy update of the superblock's later columns: Wf[:, i2:cend] -= E U[i1:i2, i2:cend]
    const int i2 = i1 + kRB;
    if (i2 < cend) {
      far_update(w, Wf, UT, c, i1, i2, cend, lane, eb);
      __threadfence_block();
      __syncthreads();
    }
  }
  double* part = reinterpret_cast<double*>(p.partials) + 2 * (int64_t)gslab;
  // sum of err^2 over the slab's live rows, reduced in a fixed lane order and
  // added to the earlier superblocks' sum (launches run in order)
  double v = live ? obs : 0.0;
  for (int off = 32; off > 0; off >>= 1) v += __shfl_down(v, off);
  if (lane == 0) part[0] = c0 == 0 ? v : part[0] + v;
}

// ---------------------------------------------------------------- trailing update
// Trailing update after the superblock at c0, for all jobs:
//   Wf[:, n0:] -= E U[c0:c0+kSuper, n0:],   n0 = c0 + kSuper.
// The product runs exactly on the int8 matrix cores over digit expansions of
// its operands (the splitting scheme of Ozaki, Ogita, Oishi and Rump, with
// integer slices, as in the factorisation): each row of E (over the
// superblock) and each column of U (over the superblock's rows) has a
// power-of-two bound 2^e >= max |.| (1 + 1/64) and kTS base-128 digits, each
// rounded to nearest, so an operand is carried to 28 bits relative to its
// row's (column's) largest entry.  Digit pairs p + q < kTS are multiplied
// (v_mfma_i32_32x32x32_i8, exact int32 sums over K = 256) and combined in
// fp32: sum_w acc_w 2^-7w by Horner, then scaled by 2^(e_row + e_col - 14).
// The fp32 products this replaces carry 24 bits per operand and round at
// every accumulation step; the code decisions downstream see no difference.
constexpr int kTS = 4;                  // digits per operand entry
constexpr int kTK = 32;                 // K chunk of one MFMA step
constexpr float kDigitBound = 0.984375f;  // 1 / (1 + 1/64): |scaled entry| * 128 <= 126

// Digit planes of U for the trailing products, once per Hessian after the
// factor: for superblock sb and column col >= (sb + 1) kSuper, with the 256
// values U[sb*kSuper + k][col] (contiguous in U^T).  Layout in the Hessian's
// inverse buffer (free once U is written): plane p at byte p c^2; in a plane,
// the 32 digits of K step kc (k = 32 kc .. +31) of column col at byte
// ((sb * 8 + kc) * c + col) * 32, so that the operands of one K step for 32
// consecutive columns are 1 KB of consecutive bytes; the exponents follow at
// byte kTS c^2 as int eU[sb][col].  Four threads share a column, 64 values
// (two K steps) each.
__global__ __launch_bounds__(256) void u_digits_kernel(const float* __restrict__ UTall, double* Xall, int c) {
  const int sb = blockIdx.y, m = blockIdx.z;
  const int col = 64 * blockIdx.x + (threadIdx.x >> 2), part = threadIdx.x & 3;
  if (64 * (int)blockIdx.x < (sb + 1) * kSuper) return;   // whole block at or before the superblock
  const int64_t cc = (int64_t)c * c;
  const float* src = UTall + m * cc + (int64_t)col * c + sb * kSuper + 64 * part;
  int8_t* X8 = reinterpret_cast<int8_t*>(Xall + m * cc);
  float v[64];
  float mx = 0.0f;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const float4 t = *reinterpret_cast<const float4*>(src + 4 * q);
    v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(t.x), fabsf(t.y)), fmaxf(fabsf(t.z), fabsf(t.w))));
  }
  mx = fmaxf(mx, __shfl_xor(mx, 1));
  mx = fmaxf(mx, __shfl_xor(mx, 2));
  int e = 0;
  if (mx > 0.0f) frexpf(mx * (1.0f + 1.0f / 64.0f), &e);
  if (part == 0) reinterpret_cast<int*>(X8 + kTS * cc)[(int64_t)sb * c + col] = e;
  uint32_t packed[kTS][16];
#pragma unroll
  for (int p = 0; p < kTS; ++p)
#pragma unroll
    for (int u = 0; u < 16; ++u) packed[p][u] = 0u;
#pragma unroll
  for (int u = 0; u < 64; ++u) {
    float x = fminf(fmaxf(ldexpf(v[u], -e), -kDigitBound), kDigitBound);
#pragma unroll
    for (int p = 0; p < kTS; ++p) {
      x *= 128.0f;
      const float d = rintf(x);
      x -= d;
      packed[p][u >> 2] |= ((uint32_t)(int)d & 0xffu) << (8 * (u & 3));
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int8_t* dst = X8 + (((int64_t)sb * (kSuper / kTK) + 2 * part + h) * c + col) * kTK;
#pragma unroll
    for (int p = 0; p < kTS; ++p)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int u4 = 8 * h + 4 * q;
        *reinterpret_cast<uint4*>(dst + p * cc + 16 * q) =
            make_uint4(packed[p][u4], packed[p][u4 + 1], packed[p][u4 + 2], packed[p][u4 + 3]);
      }
  }
}

// One workgroup per slab (64 padded rows of one job) and superblock, sweeping
// all of the job's trailing column tiles of 128: the slab's error digits are
// made once, into LDS, and every column tile reuses them.  512 threads = 8
// waves in two roles, so that the matrix-core work and the Wf traffic overlap
// (a wave's memory counter retires in issue order, so one wave doing both
// would wait for its Wf loads and stores at every U-digit wait):
//   * waves 0-3 (products): wave w owns columns 32w..32w+31 of a tile for all
//     64 rows, as two 32x32 blocks.  The product is transposed, C[col][row] =
//     sum_k U^T[col][k] E[row][k], so each lane's 16 results of a block are 4
//     runs of 4 consecutive columns of one row.  Operand lanes of
//     v_mfma_i32_32x32x32_i8: lane l holds row l%32, K bytes 16(l/32)..+15 of
//     the 32-byte step; result r of lane l is row 8(r/4) + 4(l/32) + r%4,
//     column l%32.  Each wave streams its own U digits from global memory two
//     K steps ahead in registers, so the K loop has no barrier.  A tile's
//     digit sums, combined in fp32 (Horner), go to one of two LDS buffers;
//   * waves 4-7 (weights): load the next tile's weights and column exponents
//     while the products run, then apply Wf -= f 2^(e_row + e_col - 14) and
//     store, coalesced by rows.
// One barrier per tile hands a buffer from the first role to the second; the
// buffers alternate, so a buffer is rewritten only after the second role has
// read it (it reads before it reaches the next barrier).  Slabs of one job are
// mapped to one XCD (workgroup b runs on XCD b % 8), so the job's U digits are
// shared through one L2.
constexpr int kRPitch = kGemmTile + 4;   // result buffer row pitch (floats): rows 4 banks apart

// global-address-space views of the weights (the job table holds generic pointers)
typedef const __attribute__((address_space(1))) uint16_t g_u16;
typedef const __attribute__((address_space(1))) float g_f32;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x2 g_u32x2;
typedef const __attribute__((address_space(1))) f32x4 g_f32x4;

// Barrier over the workgroup's LDS only: s_waitcnt lgkmcnt(0) (vmcnt and expcnt
// at their maxima), so this wave's LDS accesses have completed while its global
// loads and stores stay in flight, then s_barrier.  The empty asm statements
// keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(512, 1) void gptq_trail_kernel(GptqPlan p, int c0, JobRange jr) {
  // error digits: row r's 16-byte chunk ch at slot ch ^ (r % 16) (conflict-free lane reads)
  __shared__ __attribute__((aligned(16))) int8_t Eq[kTS][kGptqRows][kSuper];
  __shared__ int eE[kGptqRows];
  __shared__ __attribute__((aligned(16))) float R[2][kGptqRows * kRPitch];
  const int c = p.cols, n0 = c0 + kSuper, sb = c0 / kSuper;
  const int total = jr.n_slabs;
  const int per = (total + kXcds - 1) / kXcds;
  const int L = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
  if (L >= total) return;
  const int gslab = jr.slab0 + L;
  int lo = jr.j0, hi = jr.j1;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.jobs[mid].slab_base <= gslab) lo = mid; else hi = mid;
  }
  const GJob job = p.jobs[lo];
  const int prow0 = (gslab - job.slab_base) * kGptqRows;
  const int64_t grow = job.wf_off / c + prow0;     // first padded row of the slab (all jobs)
  const int64_t cc = (int64_t)c * c;
  const int8_t* UTq = reinterpret_cast<const int8_t*>(p.X + (int64_t)job.mat * cc);
  const int* eU = reinterpret_cast<const int*>(UTq + kTS * cc) + (int64_t)sb * c;
  const int tid = threadIdx.x;
  const int n_ct = (c - n0 + kGemmTile - 1) / kGemmTile;

  // ---- error digits of the slab's rows (first role)
  if (tid < 256) {
    const int row = tid >> 2, part = tid & 3;
    const float* er = p.ebuf + (grow + row) * kSuper + 64 * part;
    float v[64];
    float mx = 0.0f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float4 t = *reinterpret_cast<const float4*>(er + 4 * q);
      v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(t.x), fabsf(t.y)), fmaxf(fabsf(t.z), fabsf(t.w))));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    int e = 0;
    if (mx > 0.0f) frexpf(mx * (1.0f + 1.0f / 64.0f), &e);
    if (part == 0) eE[row] = e;
    uint32_t packed[kTS][16];
#pragma unroll
    for (int pp = 0; pp < kTS; ++pp)
#pragma unroll
      for (int u = 0; u < 16; ++u) packed[pp][u] = 0u;
#pragma unroll
    for (int u = 0; u < 64; ++u) {
      float x = fminf(fmaxf(ldexpf(v[u], -e), -kDigitBound), kDigitBound);
#pragma unroll
      for (int pp = 0; pp < kTS; ++pp) {
        x *= 128.0f;
        const float d = rintf(x);
        x -= d;
        packed[pp][u >> 2] |= ((uint32_t)(int)d & 0xffu) << (8 * (u & 3));
      }
    }
#pragma unroll
    for (int pp = 0; pp < kTS; ++pp)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ch = 4 * part + q;
        *reinterpret_cast<uint4*>(&Eq[pp][row][16 * (ch ^ (row & 15))]) =
            make_uint4(packed[pp][4 * q], packed[pp][4 * q + 1], packed[pp][4 * q + 2], packed[pp][4 * q + 3]);
      }
  }
  __syncthreads();

  if (tid < 256) {
    // ---------------------------------------------------------- products
    const int lane = tid & 63, wc = tid >> 6, hh = lane >> 5, li = lane & 31;
    const int last = n_ct * (kSuper / kTK) - 1;
    const int lcol = wc * 32 + li;                    // the lane's operand column in a tile
    auto fetch = [&](i32x4 (&a)[kTS], int g) {
      g = min(g, last);
      const int t = g / (kSuper / kTK), kc = g % (kSuper / kTK);
      const int col = min(n0 + t * kGemmTile + lcol, c - 1);
      const int8_t* src = UTq + (((int64_t)sb * (kSuper / kTK) + kc) * c + col) * kTK + 16 * hh;
#pragma unroll
      for (int pp = 0; pp < kTS; ++pp) a[pp] = *reinterpret_cast<const i32x4*>(src + pp * cc);
    };
    i32x4 a0[kTS], a1[kTS];
    fetch(a0, 0);
    fetch(a1, 1);
    const int cl = wc * 32 + 4 * hh;                  // lane's first result column in a tile
    // The error digits of K step kc (the same for every tile) are read one step
    // ahead of their products, into two register sets, so the LDS latency
    // overlaps the previous step's products; the read after a tile's last
    // step is step 0 of the next tile.
    auto read_e = [&](i32x4 (&bq)[2][kTS], int kc) {
      const int ch = 2 * kc + hh;
#pragma unroll
      for (int pp = 0; pp < kTS; ++pp)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int row = 32 * b + li;
          bq[b][pp] = *reinterpret_cast<const i32x4*>(&Eq[pp][row][16 * (ch ^ (row & 15))]);
        }
    };
    i32x4 e0[2][kTS], e1[2][kTS];
    read_e(e0, 0);
    int g = 0;
    for (int t = 0; t < n_ct; ++t) {
      const int ncols = min(kGemmTile, c - (n0 + t * kGemmTile));   // 64 or 128
      i32x16 acc[2][kTS];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int w = 0; w < kTS; ++w) acc[b][w] = i32x16{};
      auto mul = [&](const i32x4 (&a)[kTS], const i32x4 (&bq)[2][kTS]) {
        // the two blocks alternate, so products into one accumulator are never adjacent
#pragma unroll
        for (int pp = 0; pp < kTS; ++pp)
#pragma unroll
          for (int q = 0; pp + q < kTS; ++q)
#pragma unroll
            for (int b = 0; b < 2; ++b)
              acc[b][pp + q] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[pp], bq[b][q], acc[b][pp + q], 0, 0, 0);
      };
      // K steps in pairs: even steps use a0 and e0, odd ones a1 and e1; the U
      // digits are refilled two steps ahead, the error digits one.  Unrolled,
      // so that the waits for the U digits count the loads issued after them
      // (across a loop edge the compiler waits for every load in flight).
#pragma unroll
      for (int kc = 0; kc < kSuper / kTK; kc += 2) {
        read_e(e1, kc + 1);
        __builtin_amdgcn_sched_barrier(0);
        mul(a0, e0);
        fetch(a0, g + kc + 2);
        __builtin_amdgcn_sched_barrier(0);
        read_e(e0, (kc + 2) % (kSuper / kTK));
        __builtin_amdgcn_sched_barrier(0);
        mul(a1, e1);
        fetch(a1, g + kc + 3);
        __builtin_amdgcn_sched_barrier(0);
      }
      g += kSuper / kTK;
      if (wc * 32 < ncols) {
        // results r = 4q .. 4q+3 are columns cl + 8q .. +3 of row 32b + li
        float* Rt = R[t & 1];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float f4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int r = 4 * q + u;
              float f = (float)acc[b][kTS - 1][r];
#pragma unroll
              for (int w = kTS - 2; w >= 0; --w) f = fmaf(f, 1.0f / 128.0f, (float)acc[b][w][r]);
              f4[u] = f;
            }
            *reinterpret_cast<float4*>(Rt + (32 * b + li) * kRPitch + cl + 8 * q) =
                make_float4(f4[0], f4[1], f4[2], f4[3]);
          }
      }
      lds_barrier();
    }
  } else {
    // ---------------------------------------------------------- weights
    // thread m: columns 4 (m % 32) .. +3 of rows m / 32 + 8 i, i = 0..7
    const int m = tid - 256, col4 = 4 * (m & 31), rsub = m >> 5;
    const bool fill = c0 == 0 && !(p.act_order | p.static_groups);
    const uint8_t* dead = p.dead + (int64_t)job.mat * c;
    float4 wv[kGptqRows / 8];
    int4 e4;
    auto load = [&](int t) {
      const int col0 = n0 + t * kGemmTile;
      const int ncols = min(kGemmTile, c - col0);
      if (col4 >= ncols) return;
      e4 = *reinterpret_cast<const int4*>(eU + col0 + col4);
      if (fill) {
        // first trailing update: the working copy of these columns does not exist
        // yet; start from W (rows past the matrix zero, dead columns zeroed).  The
        // loads are unconditional (row index clamped) and through global-space
        // pointers: a flat load would also count against the LDS counter, which
        // the barrier waits for.
        const uchar4 dd = *reinterpret_cast<const uchar4*>(dead + col0 + col4);
        if (job.dtype == 1) {
          g_u16* Wb = (g_u16*)job.W;   // a C cast: reinterpret_cast cannot change address spaces
#pragma unroll
          for (int i = 0; i < kGptqRows / 8; ++i) {
            const int64_t r = min(prow0 + rsub + 8 * i, job.rows - 1);
            const u32x2 b = *(g_u32x2*)(Wb + r * c + col0 + col4);
            wv[i] = make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xffff0000u),
                                __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xffff0000u));
          }
        } else {
          g_f32* Wq = (g_f32*)job.W;
#pragma unroll
          for (int i = 0; i < kGptqRows / 8; ++i) {
            const int64_t r = min(prow0 + rsub + 8 * i, job.rows - 1);
            const f32x4 v = *(g_f32x4*)(Wq + r * c + col0 + col4);
            wv[i] = make_float4(v.x, v.y, v.z, v.w);
          }
        }
#pragma unroll
        for (int i = 0; i < kGptqRows / 8; ++i) {
          const bool live = prow0 + rsub + 8 * i < job.rows;
          wv[i] = make_float4(dd.x || !live ? 0.f : wv[i].x, dd.y || !live ? 0.f : wv[i].y,
                              dd.z || !live ? 0.f : wv[i].z, dd.w || !live ? 0.f : wv[i].w);
        }
      } else {
        const float* W = p.wf + grow * c + col0 + col4;
#pragma unroll
        for (int i = 0; i < kGptqRows / 8; ++i)
          wv[i] = *reinterpret_cast<const float4*>(W + (int64_t)(rsub + 8 * i) * c);
      }
    };
    load(0);
    for (int t = 0; t < n_ct; ++t) {
      // the barrier also retires this wave's reads of the buffer of tile t - 1
      lds_barrier();
      const int col0 = n0 + t * kGemmTile;
      const int ncols = min(kGemmTile, c - col0);
      if (col4 < ncols) {
        const float* Rt = R[t & 1];
        float* W = p.wf + grow * c + col0 + col4;
        const int ec[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
        for (int i = 0; i < kGptqRows / 8; ++i) {
          const int row = rsub + 8 * i;
          const float4 f = *reinterpret_cast<const float4*>(Rt + row * kRPitch + col4);
          const int er = eE[row] - 14;
          const float fv[4] = {f.x, f.y, f.z, f.w};
          const float w4[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
          float out[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) out[u] = w4[u] - ldexpf(fv[u], er + ec[u]);
          *reinterpret_cast<float4*>(W + (int64_t)row * c) = make_float4(out[0], out[1], out[2], out[3]);
        }
      }
      if (t + 1 < n_ct) load(t + 1);
    }
  }
}

// ||Wq - W||^2 per slab (W with dead columns zeroed), coalesced over the outputs.
__global__ __launch_bounds__(256) void gptq_dist_kernel(GptqPlan p, JobRange jr) {
  __shared__ double red[256];
  __shared__ __attribute__((aligned(4))) uint8_t deadn[8192];
  const int c = p.cols, group = p.group;
  const int gslab = jr.slab0 + (int)blockIdx.x;
  int lo = jr.j0, hi = jr.j1;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.jobs[mid].slab_base <= gslab) lo = mid; else hi = mid;
  }
  const GJob job = p.jobs[lo];
  const int row0 = (gslab - job.slab_base) * kGptqRows;
  const int nrows = min(kGptqRows, job.rows - row0);
  const uint8_t* dead = p.dead + (int64_t)job.mat * c;
  const int ng = c / group;
  // with activation order the dead flags are in processing order: use the
  // natural ones (H_ii == 0 of the caller's Hessian) instead
  if (p.act_order) {
    const float* Hsrc = p.src_mats[job.mat];
    for (int i = threadIdx.x; i < c; i += 256) deadn[i] = Hsrc[(int64_t)i * c + i] == 0.0f;
    __syncthreads();
    dead = deadn;
  }
  const int* gidx = p.gidx ? p.gidx + (int64_t)job.mat * c : nullptr;
  // four consecutive columns per step (without g_idx they share one grid: group >= 4)
  double acc = 0.0;
  for (int r = 0; r < nrows; ++r) {
    const int64_t row = row0 + r;
    for (int col = 4 * (int)threadIdx.x; col < c; col += 1024) {
      const int4 g4 = gidx ? *reinterpret_cast<const int4*>(gidx + col) : make_int4(0, 0, 0, 0);
      const int gq[4] = {g4.x, g4.y, g4.z, g4.w};
      const uchar4 q = *reinterpret_cast<const uchar4*>(job.codes + row * c + col);
      const uchar4 dd = *reinterpret_cast<const uchar4*>(dead + col);
      const float4 w = load_w4(job.W, job.dtype, row * c + col);
      const float qv[4] = {(float)q.x, (float)q.y, (float)q.z, (float)q.w};
      const float wv[4] = {dd.x ? 0.f : w.x, dd.y ? 0.f : w.y, dd.z ? 0.f : w.z, dd.w ? 0.f : w.w};
      if (gidx) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t gi = row * ng + gq[u];
          const float sc = job.scales[gi], zp = (float)job.zeros[gi];
          const float what = __fmul_rn(sc, __fsub_rn(qv[u], zp));
          const double dv = (double)what - (double)wv[u];
          acc += dv * dv;
        }
      } else {
        const int64_t gi = row * ng + col / group;     // one grid for the four columns
        const float sc = job.scales[gi], zp = (float)job.zeros[gi];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float what = __fmul_rn(sc, __fsub_rn(qv[u], zp));
          const double dv = (double)what - (double)wv[u];
          acc += dv * dv;
        }
      }
    }
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) reinterpret_cast<double*>(p.partials)[2 * (int64_t)gslab + 1] = red[0];
}

// ---------------------------------------------------------------- options
// Processing position and grid of every column of Hessian m0 + blockIdx.y,
// 256 columns per workgroup.  Activation order ranks the keys k_i = H_ii (1 for
// a dead column) by decreasing value, ties by index: position(i) = #{j : k_j >
// k_i, or k_j = k_i and j < i}.  The keys are compared as integers that order
// like the floats (sign-magnitude to offset binary), a strict total order with
// the index tie break, so the positions are a permutation for any input.
__global__ __launch_bounds__(256) void order_kernel(GptqPlan p, int m0) {
  __shared__ uint32_t key[8192];
  const int m = m0 + (int)blockIdx.y, c = p.cols;
  const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
  if (p.act_order) {
    const float* H = p.src_mats[m];
    for (int t = threadIdx.x; t < c; t += 256) {
      float d = H[(int64_t)t * c + t];
      if (d == 0.0f) d = 1.0f;
      const uint32_t u = __float_as_uint(d);
      key[t] = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    }
    __syncthreads();
  }
  if (i >= c) return;
  int pos = i;
  if (p.act_order) {
    const uint32_t ki = key[i];
    pos = 0;
    for (int j = 0; j < c; ++j) {
      const uint32_t kj = key[j];
      pos += (kj > ki) | ((kj == ki) & (j < i));
    }
    p.perm[(int64_t)m * c + pos] = i;
  }
  p.ipos[(int64_t)m * c + i] = pos;
  p.gidx[(int64_t)m * c + i] = (p.act_order && !p.static_groups ? pos : i) / p.group;
}

// Hp[i][j] = H[perm[i]][perm[j]]: row i of Hessian m0 + blockIdx.y per workgroup.
__global__ __launch_bounds__(256) void permute_h_kernel(GptqPlan p, int m0) {
  const int c = p.cols, i = blockIdx.x, m = m0 + (int)blockIdx.y;
  const int* perm = p.perm + (int64_t)m * c;
  const float* Hr = p.src_mats[m] + (int64_t)perm[i] * c;
  float* out = p.hperm + (int64_t)m * c * c + (int64_t)i * c;
  for (int j = 4 * (int)threadIdx.x; j < c; j += 1024) {
    const int4 pj = *reinterpret_cast<const int4*>(perm + j);
    *reinterpret_cast<float4*>(out + j) = make_float4(Hr[pj.x], Hr[pj.y], Hr[pj.z], Hr[pj.w]);
  }
}

// One slab per workgroup: the whole fp32 working copy in processing order
// (rows past the matrix zero, dead columns zeroed) and, with static groups,
// the grid of every (row, natural group) fitted on the same weights.  A row is
// read once, coalesced (thread t holds natural columns 4t .. 4t+3); its static
// grids are reduced from those registers across the group's lanes; the row
// then goes through LDS to be written in processing order.
__global__ __launch_bounds__(256) void gptq_prep_kernel(GptqPlan p, JobRange jr) {
  __shared__ uint8_t deadn[8192];
  __shared__ __attribute__((aligned(16))) float rowbuf[8192];
  const int c = p.cols;
  const int gslab = jr.slab0 + (int)blockIdx.x;
  int lo = jr.j0, hi = jr.j1;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.jobs[mid].slab_base <= gslab) lo = mid; else hi = mid;
  }
  const GJob job = p.jobs[lo];
  const int row0 = (gslab - job.slab_base) * kGptqRows;
  const int nrows = min(kGptqRows, job.rows - row0);
  const float* H = p.src_mats[job.mat];
  for (int i = threadIdx.x; i < c; i += 256) deadn[i] = H[(int64_t)i * c + i] == 0.0f;
  __syncthreads();
  const int* perm = p.perm ? p.perm + (int64_t)job.mat * c : nullptr;
  float* Wf = p.wf + job.wf_off + (int64_t)row0 * c;
  const int G = p.group, ng = c / G;
  const float fmaxq = (float)((1 << job.bits) - 1);
  for (int r = 0; r < kGptqRows; ++r) {
    const bool live = r < nrows;
    const int64_t wrow = (int64_t)(row0 + r) * c;
    // the lanes with columns in a pass are a multiple of 16 (32 when g = 128,
    // since then c is a multiple of 128), so a group's g/4 lanes are all active
    for (int j = 4 * (int)threadIdx.x; j < c; j += 1024) {
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (live) {
        const float4 t = load_w4(job.W, job.dtype, wrow + j);
        v[0] = deadn[j] ? 0.f : t.x;
        v[1] = deadn[j + 1] ? 0.f : t.y;
        v[2] = deadn[j + 2] ? 0.f : t.z;
        v[3] = deadn[j + 3] ? 0.f : t.w;
      }
      if (perm) {
        *reinterpret_cast<float4*>(rowbuf + j) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        *reinterpret_cast<float4*>(Wf + (int64_t)r * c + j) = make_float4(v[0], v[1], v[2], v[3]);
      }
      if (p.static_groups && live) {
        // the G/4 lanes of a group are consecutive and aligned (G <= 128, so at
        // most 32 lanes, within one wave)
        float mn = fminf(fminf(v[0], v[1]), fminf(v[2], v[3]));
        float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
        for (int off = 1; off < G / 4; off <<= 1) {
          mn = fminf(mn, __shfl_xor(mn, off));
          mx = fmaxf(mx, __shfl_xor(mx, off));
        }
        if ((j % G) == 0) {
          float sc, zp;
          fit_grid(mn, mx, fmaxq, sc, zp);
          job.scales[(int64_t)(row0 + r) * ng + j / G] = sc;
          job.zeros[(int64_t)(row0 + r) * ng + j / G] = (uint8_t)zp;
        }
      }
    }
    if (perm) {
      __syncthreads();
      for (int j = 4 * (int)threadIdx.x; j < c; j += 1024) {
        const int4 pj = *reinterpret_cast<const int4*>(perm + j);
        *reinterpret_cast<float4*>(Wf + (int64_t)r * c + j) =
            make_float4(rowbuf[pj.x], rowbuf[pj.y], rowbuf[pj.z], rowbuf[pj.w]);
      }
      __syncthreads();
    }
  }
}

// Activation order: each row's codes, written in processing order, back to
// their natural columns (code of column i = the one at position ipos[i]).
__global__ __launch_bounds__(256) void unpermute_codes_kernel(GptqPlan p, JobRange jr) {
  __shared__ __attribute__((aligned(16))) uint8_t rowc[8192];
  const int c = p.cols;
  const int gslab = jr.slab0 + (int)blockIdx.x;
  int lo = jr.j0, hi = jr.j1;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.jobs[mid].slab_base <= gslab) lo = mid; else hi = mid;
  }
  const GJob job = p.jobs[lo];
  const int row0 = (gslab - job.slab_base) * kGptqRows;
  const int nrows = min(kGptqRows, job.rows - row0);
  const int* ipos = p.ipos + (int64_t)job.mat * c;
  for (int r = 0; r < nrows; ++r) {
    uint8_t* cr = job.codes + (int64_t)(row0 + r) * c;
    for (int j = 16 * (int)threadIdx.x; j < c; j += 4096)
      *reinterpret_cast<uint4*>(rowc + j) = *reinterpret_cast<const uint4*>(cr + j);
    __syncthreads();
    for (int j = 4 * (int)threadIdx.x; j < c; j += 1024) {
      const int4 q = *reinterpret_cast<const int4*>(ipos + j);
      *reinterpret_cast<uchar4*>(cr + j) = make_uchar4(rowc[q.x], rowc[q.y], rowc[q.z], rowc[q.w]);
    }
    __syncthreads();
  }
}

void launch_gptq_prep(const GptqPlan& p, const JobRange& jr, hipStream_t s) {
  if (!(p.act_order | p.static_groups)) return;
  const int nm = jr.m1 - jr.m0;
  if (nm > 0) {
    hipLaunchKernelGGL(order_kernel, dim3((p.cols + 255) / 256, nm), dim3(256), 0, s, p, jr.m0);
    if (p.act_order) hipLaunchKernelGGL(permute_h_kernel, dim3(p.cols, nm), dim3(256), 0, s, p, jr.m0);
  }
  if (jr.j1 > jr.j0) hipLaunchKernelGGL(gptq_prep_kernel, dim3(jr.n_slabs), dim3(256), 0, s, p, jr);
}

__global__ void natural_gidx_kernel(int32_t* g, int cols, int group) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < cols) g[i] = i / group;
}

void launch_natural_gidx(int32_t* g, int cols, int group, hipStream_t s) {
  hipLaunchKernelGGL(natural_gidx_kernel, dim3((cols + 255) / 256), dim3(256), 0, s, g, cols, group);
}

// Per job: the loss by the OBS identity, the job's numerical status from its
// Hessian's factor (NONFINITE before NOT_PD; a failing job is also recorded in
// the context's status record by its caller index), and its Hessian's dead
// columns in natural order (H_ii == 0 of the caller's Hessian).
__global__ void gptq_finish_kernel(GptqPlan p, JobRange jr) {
  const GJob job = p.jobs[jr.j0 + blockIdx.x];
  const int c = p.cols;
  if (job.dead_out) {
    const float* H = p.src_mats ? p.src_mats[job.mat] : p.mats[job.mat];
    for (int i = threadIdx.x; i < c; i += blockDim.x) job.dead_out[i] = H[(int64_t)i * c + i] == 0.0f;
  }
  if (threadIdx.x != 0) return;
  const int ms = p.mstat[job.mat];
  if (job.status) job.status[0] = (ms & kStatusNonfinite) ? 6 : (ms & kStatusNotPd) ? 5 : 0;   // clha_status
  if (ms) atomicMax(reinterpret_cast<unsigned*>(p.status) + kStatusJob, 0xffffffffu - (unsigned)job.user_index);
  if (job.loss == nullptr) return;
  const double* part = reinterpret_cast<const double*>(p.partials);
  double obs = 0.0, d2 = 0.0;
  for (int s = 0; s < job.n_slabs; ++s) {
    obs += part[2 * (int64_t)(job.slab_base + s)];
    d2 += part[2 * (int64_t)(job.slab_base + s) + 1];
  }
  job.loss[0] = (float)(obs - p.lamd[job.mat] * d2);
}

bool gptq_group_supported(int group) {
  return group == 4 || group == 8 || group == 16 || group == 32 || group == 64 || group == 128;
}

template <int MODE>
void launch_panel(const GptqPlan& p, int c0, const JobRange& jr, dim3 grid, dim3 blk, hipStream_t s) {
  switch (p.group) {
    case 4: hipLaunchKernelGGL((gptq_panel_kernel<4, MODE>), grid, blk, 0, s, p, c0, jr); break;
    case 8: hipLaunchKernelGGL((gptq_panel_kernel<8, MODE>), grid, blk, 0, s, p, c0, jr); break;
    case 16: hipLaunchKernelGGL((gptq_panel_kernel<16, MODE>), grid, blk, 0, s, p, c0, jr); break;
    case 32: hipLaunchKernelGGL((gptq_panel_kernel<32, MODE>), grid, blk, 0, s, p, c0, jr); break;
    case 64: hipLaunchKernelGGL((gptq_panel_kernel<64, MODE>), grid, blk, 0, s, p, c0, jr); break;
    default: hipLaunchKernelGGL((gptq_panel_kernel<128, MODE>), grid, blk, 0, s, p, c0, jr); break;
  }
}

void launch_gptq(const GptqPlan& p, const JobRange& jr, hipStream_t s) {
  if (jr.j1 <= jr.j0) return;
  if (p.cols > kSuper) {
    const int64_t cc = (int64_t)p.cols * p.cols;
    // superblocks followed by trailing columns: all but the last (full ones)
    const int nsb = (p.cols + kSuper - 1) / kSuper - 1;
    hipLaunchKernelGGL(u_digits_kernel, dim3(p.cols / 64, nsb, jr.m1 - jr.m0), dim3(256), 0, s,
                       p.UT + jr.m0 * cc, p.X + jr.m0 * cc, p.cols);
  }
  const dim3 grid(jr.n_slabs), blk(64);
  for (int c0 = 0; c0 < p.cols; c0 += kSuper) {
    if (p.static_groups && p.perm) launch_panel<kGridStaticPerm>(p, c0, jr, grid, blk, s);
    else if (p.static_groups) launch_panel<kGridStatic>(p, c0, jr, grid, blk, s);
    else launch_panel<kGridFit>(p, c0, jr, grid, blk, s);
    const int n0 = c0 + kSuper;
    if (n0 < p.cols) {
      const int per = (jr.n_slabs + kXcds - 1) / kXcds;
      hipLaunchKernelGGL(gptq_trail_kernel, dim3(per * kXcds), dim3(512), 0, s, p, c0, jr);
    }
  }
  if (p.perm) hipLaunchKernelGGL(unpermute_codes_kernel, dim3(jr.n_slabs), dim3(256), 0, s, p, jr);
  hipLaunchKernelGGL(gptq_dist_kernel, dim3(jr.n_slabs), dim3(256), 0, s, p, jr);
  hipLaunchKernelGGL(gptq_finish_kernel, dim3(jr.j1 - jr.j0), dim3(64), 0, s, p, jr);
}

}  // namespace clha
