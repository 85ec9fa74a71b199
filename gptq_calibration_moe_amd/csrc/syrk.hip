// Collection phase, second half: per-slot Gram sums S[e] += X_e^T X_e.
//
// CLHA summary, section 2.1: the Hessian of a layer for a weight fed by
// activations x is the (uncentred) activation second moment; section 2.2
// accumulates it per layer and per active expert over the calibration data.
// Products of bf16 values are exact in fp32; they are accumulated in fp32 on
// the matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Work decomposition.  S is symmetric, so only the lower-triangular 128x128
// tiles (ti >= tj) of each slot are computed: nt(nt+1)/2 tiles for nt = d/128.
// Workgroup b takes slot slot_order[b / tiles_per_slot] -- slots are ordered
// longest token list first, so the long shared-expert and heavily loaded
// experts start first -- and tile b % tiles_per_slot.  One workgroup owns one
// (slot, tile) for the whole token range, so every element of S is summed in a
// fixed order by a single workgroup: results are bit-identical run to run.
// The running sum is added into S every kFlushSteps token steps (two-level
// summation keeps fp32 error independent of the expert's size).
//
// Tile pipeline: 256 threads (4 waves, 2x2), 64 output rows x 64 columns per
// wave as 2x2 MFMA 32x32 blocks; tokens advance 64 at a time through LDS.  The
// operand tiles are feature-major [128 features][64 tokens] so each lane's
// MFMA fragment (8 consecutive tokens of one feature) is one 16-byte LDS read;
// the LDS row pitch of 72 bf16 (144 B) keeps those reads bank-conflict free.
#include "kernels.h"

namespace clha {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kSK = 64;              // tokens per step
constexpr int kPitch = kSK + 8;      // LDS row pitch (bf16 elements)
constexpr int kFlushSteps = 128;     // 8192 tokens between partial-sum flushes

__device__ __forceinline__ void tile_of(int t, int& ti, int& tj) {
  int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  while (i * (i + 1) / 2 > t) --i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

__device__ __forceinline__ void flush_acc(f32x16 (&acc)[2][2], float* __restrict__ Sslot, int d,
                                          int row0, int col0, bool diag, int lane) {
#pragma unroll
  for (int im = 0; im < 2; ++im)
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
      const int j = col0 + jn * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = row0 + im * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (!diag || i >= j) Sslot[(int64_t)i * d + j] += acc[im][jn][r];
        acc[im][jn][r] = 0.0f;
      }
    }
}

__global__ __launch_bounds__(256) void syrk_kernel(const uint16_t* __restrict__ xgT,
                                                   const int64_t* __restrict__ pad_off,
                                                   const int32_t* __restrict__ slot_order, int d,
                                                   int tiles_per_slot, float* __restrict__ S) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kSyrkTile * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kSyrkTile * kPitch];

  const int rank = blockIdx.x / tiles_per_slot;
  const int tile = blockIdx.x - rank * tiles_per_slot;
  const int slot = slot_order[rank];
  const int64_t npad = pad_off[slot + 1] - pad_off[slot];
  if (npad == 0) return;
  int ti, tj;
  tile_of(tile, ti, tj);
  const bool diag = ti == tj;
  const uint16_t* base = xgT + pad_off[slot] * d;
  const uint16_t* Ag = base + (int64_t)ti * kSyrkTile * npad;
  const uint16_t* Bg = base + (int64_t)tj * kSyrkTile * npad;
  const uint16_t* Bsrc = diag ? As : Bs;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[2][2];
#pragma unroll
  for (int im = 0; im < 2; ++im)
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) acc[im][jn] = f32x16{};

  int steps = 0;
  for (int64_t k0 = 0; k0 < npad; k0 += kSK) {
    uint4 ra[4], rb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int c = tid + 256 * m;
      const int row = c >> 3, ch = c & 7;
      ra[m] = *reinterpret_cast<const uint4*>(Ag + (int64_t)row * npad + k0 + ch * 8);
      if (!diag) rb[m] = *reinterpret_cast<const uint4*>(Bg + (int64_t)row * npad + k0 + ch * 8);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int c = tid + 256 * m;
      const int row = c >> 3, ch = c & 7;
      *reinterpret_cast<uint4*>(&As[row * kPitch + ch * 8]) = ra[m];
      if (!diag) *reinterpret_cast<uint4*>(&Bs[row * kPitch + ch * 8]) = rb[m];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kSK / 16; ++kk) {
      const int kcol = kk * 16 + (lane >> 5) * 8;
      bf16x8 a[2], b[2];
#pragma unroll
      for (int im = 0; im < 2; ++im) {
        const int row = wm * 64 + im * 32 + (lane & 31);
        a[im] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&As[row * kPitch + kcol]));
      }
#pragma unroll
      for (int jn = 0; jn < 2; ++jn) {
        const int row = wn * 64 + jn * 32 + (lane & 31);
        b[jn] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&Bsrc[row * kPitch + kcol]));
      }
#pragma unroll
      for (int im = 0; im < 2; ++im)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
          acc[im][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[im], b[jn], acc[im][jn], 0, 0, 0);
    }
    __syncthreads();
    if (++steps == kFlushSteps) {
      steps = 0;
      flush_acc(acc, S + (int64_t)slot * d * d, d, ti * kSyrkTile + wm * 64,
                tj * kSyrkTile + wn * 64, diag, lane);
    }
  }
  if (steps) flush_acc(acc, S + (int64_t)slot * d * d, d, ti * kSyrkTile + wm * 64,
                       tj * kSyrkTile + wn * 64, diag, lane);
}

void launch_syrk(const CollectPlan& p, float* S, hipStream_t s) {
  const int nt = p.d / kSyrkTile;
  const int tiles = nt * (nt + 1) / 2;
  const int slots = p.E + p.has_shared;
  hipLaunchKernelGGL(syrk_kernel, dim3(tiles * slots), dim3(256), 0, s, p.xgT, p.pad_off,
                     p.slot_order, p.d, tiles, S);
}

}  // namespace clha
