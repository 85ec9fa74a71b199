// Quantization phase: GPTQ column-sequential quantize-and-propagate with lazy
// block updates and per-group asymmetric grids.
//
// CLHA summary, section 2.2 step 3: standard GPTQ updates on H_comb; section
// 2.3 (CLHA-MP): b+1 bits for always-active shared experts, b for routed ones
// (the bit width is per job).  The GPTQ steps follow Frantar et al. (ICLR 2023):
// for column j, with U the upper Cholesky factor of Hd^-1,
//   err_j = (w_j - dequant(quant(w_j))) / U_jj,   w_k -= err_j U_jk  (k > j),
// applied eagerly inside a block of B columns and lazily (one rank-B product)
// to the columns after the block.  The grid of each (row, group) is fitted at
// the group's first column on the weights updated so far.
//
// Work decomposition: one workgroup per (job, slab of 64 rows); rows are
// independent given U, so slabs never communicate.  Per block:
//   * the slab's B columns are staged column-major in LDS (pitch 65), U's
//     diagonal block in LDS;
//   * column loop: 64 threads quantize the column (one row each; codes, scale
//     and zero are decided in fp32 with IEEE division and rint), all 256
//     threads apply the rank-1 update to the rest of the block;
//   * the block's errors then update every later column of the slab's fp32
//     working copy through U[block, later] on the fp32 matrix cores
//     (v_mfma_f32_32x32x2f32), 64 columns at a time.
// The loss is assembled from the OBS identity: sum_j err_j^2 equals
// tr[(Wq - W) Hd (Wq - W)^T], so the undamped loss is
// sum err^2 - lambda ||Wq - W||^2 (W after zeroing dead columns).
#include "kernels.h"

namespace clha {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kP = kGptqRows + 1;    // LDS pitch of a staged column
constexpr int kCodePitch = 68;       // bytes per staged code column

struct GptqSmem {
  static size_t bytes(int B, int group) {
    return (size_t)B * kP * 4            // W1 / errors
         + (size_t)B * B * 4             // U diagonal block, later a U tile [B][64]
         + (size_t)B * kCodePitch        // codes
         + 2 * 4 * kGptqRows * 4         // group min/max partials
         + 2 * (size_t)(B / group) * kGptqRows * 4;  // grids of the block's groups
  }
};

__device__ __forceinline__ float load_w(const void* W, int dtype, int64_t i) {
  if (dtype == 1) {
    const uint32_t b = reinterpret_cast<const uint16_t*>(W)[i];
    return __uint_as_float(b << 16);
  }
  return reinterpret_cast<const float*>(W)[i];
}

__global__ __launch_bounds__(256) void gptq_kernel(GptqPlan p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int B = p.block, c = p.cols, group = p.group;
  float* W1 = reinterpret_cast<float*>(smem);
  float* Ub = W1 + B * kP;
  unsigned char* cs = reinterpret_cast<unsigned char*>(Ub + B * B);
  float* redmn = reinterpret_cast<float*>(cs + B * kCodePitch);
  float* redmx = redmn + 4 * kGptqRows;
  float* gs = redmx + 4 * kGptqRows;
  float* gz = gs + (B / group) * kGptqRows;

  // job of this slab
  int lo = 0, hi = p.n_jobs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.jobs[mid].slab_base <= (int)blockIdx.x) lo = mid; else hi = mid;
  }
  const GJob job = p.jobs[lo];
  const int slab = blockIdx.x - job.slab_base;
  const int row0 = slab * kGptqRows;
  const int nrows = min(kGptqRows, job.rows - row0);
  const float* U = p.U + (int64_t)job.mat * c * c;
  const uint8_t* dead = p.dead + (int64_t)job.mat * c;
  float* Wf = p.wf + job.wf_off + (int64_t)row0 * c;
  const int maxq = (1 << job.bits) - 1;
  const float fmaxq = (float)maxq;
  const int ngroups_row = c / group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // fp32 working copy of the slab, dead columns zeroed
  for (int64_t idx = tid; idx < (int64_t)nrows * c; idx += 256) {
    const int col = (int)(idx % c);
    const float v = load_w(job.W, job.dtype, (int64_t)row0 * c + idx);
    Wf[idx] = dead[col] ? 0.0f : v;
  }
  __threadfence_block();
  __syncthreads();

  double obs = 0.0, d2 = 0.0;
  float s = 1.0f, z = 0.0f;   // grid of the current group (threads < 64, row = tid)

  for (int i1 = 0; i1 < c; i1 += B) {
    for (int idx = tid; idx < kGptqRows * B; idx += 256) {
      const int r = idx / B, col = idx - r * B;
      W1[col * kP + r] = r < nrows ? Wf[(int64_t)r * c + i1 + col] : 0.0f;
    }
    for (int idx = tid; idx < B * B; idx += 256) {
      const int a = idx / B, b = idx - a * B;
      Ub[idx] = b >= a ? U[(int64_t)(i1 + a) * c + i1 + b] : 0.0f;
    }
    __syncthreads();

    for (int jj = 0; jj < B; ++jj) {
      const int j = i1 + jj;
      if (j % group == 0) {
        const int r = lane, part = wave, q = group / 4;
        float mn = INFINITY, mx = -INFINITY;
        for (int u = 0; u < q; ++u) {
          const float v = W1[(jj + part * q + u) * kP + r];
          mn = fminf(mn, v);
          mx = fmaxf(mx, v);
        }
        redmn[part * kGptqRows + r] = mn;
        redmx[part * kGptqRows + r] = mx;
        __syncthreads();
        if (tid < kGptqRows) {
          float xmin = fminf(fminf(redmn[r], redmn[kGptqRows + r]),
                             fminf(redmn[2 * kGptqRows + r], redmn[3 * kGptqRows + r]));
          float xmax = fmaxf(fmaxf(redmx[r], redmx[kGptqRows + r]),
                             fmaxf(redmx[2 * kGptqRows + r], redmx[3 * kGptqRows + r]));
          xmin = fminf(xmin, 0.0f);
          xmax = fmaxf(xmax, 0.0f);
          if (xmin == 0.0f && xmax == 0.0f) {
            xmin = -1.0f;
            xmax = 1.0f;
          }
          s = __fdiv_rn(__fsub_rn(xmax, xmin), fmaxq);
          z = rintf(__fdiv_rn(-xmin, s));
          const int gb = jj / group;
          gs[gb * kGptqRows + r] = s;
          gz[gb * kGptqRows + r] = z;
          if (r < nrows) {
            const int64_t o = (int64_t)(row0 + r) * ngroups_row + j / group;
            job.scales[o] = s;
            job.zeros[o] = (uint8_t)z;
          }
        }
      }
      if (tid < kGptqRows) {
        const float w = W1[jj * kP + tid];
        float q = rintf(__fdiv_rn(w, s)) + z;
        q = fminf(fmaxf(q, 0.0f), fmaxq);
        const float what = __fmul_rn(s, __fsub_rn(q, z));
        const float e = __fdiv_rn(__fsub_rn(w, what), Ub[jj * B + jj]);
        cs[jj * kCodePitch + tid] = (unsigned char)q;
        W1[jj * kP + tid] = e;
        obs += (double)e * (double)e;
      }
      __syncthreads();
      {
        const int r = lane;
        const float e = W1[jj * kP + r];
        const float* urow = Ub + jj * B;
        for (int kk = jj + 1 + wave; kk < B; kk += 4) W1[kk * kP + r] -= e * urow[kk];
      }
      __syncthreads();
    }

    // codes of the block, and ||Wq - W||^2 over it
    for (int idx = tid; idx < kGptqRows * (B / 4); idx += 256) {
      const int r = idx / (B / 4), c4 = (idx - r * (B / 4)) * 4;
      if (r < nrows) {
        uint32_t packed = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int col = c4 + u;
          const unsigned q = cs[col * kCodePitch + r];
          packed |= q << (8 * u);
          const int gb = col / group;
          const float what = __fmul_rn(gs[gb * kGptqRows + r], __fsub_rn((float)q, gz[gb * kGptqRows + r]));
          const float w0 = dead[i1 + col] ? 0.0f : load_w(job.W, job.dtype, (int64_t)(row0 + r) * c + i1 + col);
          const double dd = (double)what - (double)w0;
          d2 += dd * dd;
        }
        *reinterpret_cast<uint32_t*>(job.codes + (int64_t)(row0 + r) * c + i1 + c4) = packed;
      }
    }

    // lazy update of the later columns: Wf[:, i2:] -= E1 U[i1:i2, i2:]
    const int i2 = i1 + B;
    const int wm = wave >> 1, wn = wave & 1;
    const int arow = wm * 32 + (lane & 31), kh = lane >> 5;
    for (int jt = i2; jt < c; jt += 64) {
      __syncthreads();
      for (int idx = tid; idx < B * 64; idx += 256) {
        const int k = idx >> 6, jc = idx & 63;
        Ub[idx] = U[(int64_t)(i1 + k) * c + jt + jc];
      }
      __syncthreads();
      const int col = jt + wn * 32 + (lane & 31);
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
        acc[r] = row < nrows ? Wf[(int64_t)row * c + col] : 0.0f;
      }
      for (int k = 0; k < B; k += 2) {
        const float a = -W1[(k + kh) * kP + arow];
        const float b = Ub[(k + kh) * 64 + wn * 32 + (lane & 31)];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
        if (row < nrows) Wf[(int64_t)row * c + col] = acc[r];
      }
    }
    __threadfence_block();
    __syncthreads();
  }

  // per-slab partial sums, reduced in a fixed order
  __shared__ double red[2][256];
  red[0][tid] = (tid < nrows) ? obs : 0.0;
  red[1][tid] = d2;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) {
      red[0][tid] += red[0][tid + st];
      red[1][tid] += red[1][tid + st];
    }
    __syncthreads();
  }
  if (tid == 0) {
    double* part = reinterpret_cast<double*>(p.partials) + 2 * (int64_t)blockIdx.x;
    part[0] = red[0][0];
    part[1] = red[1][0];
  }
}

__global__ void gptq_finish_kernel(GptqPlan p) {
  const GJob job = p.jobs[blockIdx.x];
  if (threadIdx.x != 0 || job.loss == nullptr) return;
  const double* part = reinterpret_cast<const double*>(p.partials);
  double obs = 0.0, d2 = 0.0;
  for (int s = 0; s < job.n_slabs; ++s) {
    obs += part[2 * (int64_t)(job.slab_base + s)];
    d2 += part[2 * (int64_t)(job.slab_base + s) + 1];
  }
  job.loss[0] = (float)(obs - p.lamd[job.mat] * d2);
}

void launch_gptq(const GptqPlan& p, hipStream_t s) {
  const size_t smem = GptqSmem::bytes(p.block, p.group);
  hipFuncSetAttribute(reinterpret_cast<const void*>(gptq_kernel),
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  hipLaunchKernelGGL(gptq_kernel, dim3(p.total_slabs), dim3(256), smem, s, p);
  hipLaunchKernelGGL(gptq_finish_kernel, dim3(p.n_jobs), dim3(64), 0, s, p);
}

size_t gptq_smem_bytes(int block, int group) { return GptqSmem::bytes(block, group); }

}  // namespace clha
