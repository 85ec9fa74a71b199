// Collection phase, second half: per-slot Gram sums S[e] += X_e^T X_e.
//
// CLHA summary, section 2.1: the Hessian of a layer for a weight fed by
// activations x is the (uncentred) activation second moment; section 2.2
// accumulates it per layer and per active expert over the calibration data.
// Products of bf16 values are exact in fp32; they are accumulated in fp32 on
// the matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Work decomposition.  S is symmetric, so only the lower-triangular 256x256
// tiles (ti >= tj) of each slot are computed: nt(nt+1)/2 tiles for nt = d/256.
// The (slot, tile) items are dealt to per-XCD lists by the bucketing scan (a
// slot's tiles stay on one die, so its activations stream through one L2;
// longest slots first).  Persistent workgroups pull items from their die's
// list.  One workgroup owns one item for the whole token range, so every
// element of S is summed in a fixed order: results are bit-identical run to
// run whichever workgroup takes the item.
// The running sum is added into S every kFlushSteps token steps (two-level
// summation keeps the fp32 error independent of the expert's size).
//
// Tile pipeline: 512 threads = 8 waves in a 2x4 arrangement, each wave owns a
// 128x64 part as 4x2 MFMA blocks of 32x32 (128 fp32 accumulators per lane).
// Tokens advance 32 at a time through two LDS buffers and two register stages:
// while the matrix cores consume one buffer, the other buffer is filled from
// the register stage loaded a step earlier, and the register stage is refilled
// with the step after that -- each global load has a full step to arrive.  Operand tiles are feature-major
// [256 features][32 tokens]; a lane's MFMA fragment (8 consecutive tokens of one
// feature) is one 16-byte LDS read, and the row pitch of 40 bf16 (80 bytes)
// keeps those reads bank-conflict free.  On diagonal tiles the two waves whose
// parts lie entirely above the diagonal skip their products, and the B operand
// is the A operand.
#include "kernels.h"

namespace clha {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kT = 256;              // output tile
constexpr int kSK = 32;              // tokens per step
constexpr int kPitch = kSK + 8;      // LDS row pitch (bf16 elements, 80 bytes)
constexpr int kFlushSteps = 256;     // 8192 tokens between partial-sum flushes (even)
constexpr int kBuf = kT * kPitch;    // one operand buffer (bf16 elements)

__device__ __forceinline__ void tile_of(int t, int& ti, int& tj) {
  int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  while (i * (i + 1) / 2 > t) --i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

// Adds the running sums into S and clears them.  One 32x32 block at a time
// (scheduling barriers keep at most 16 loads of S in flight per lane).
__device__ __forceinline__ void flush_acc(f32x16 (&acc)[4][2], float* __restrict__ Sslot, int d,
                                          int row0, int col0, bool diag, int lane) {
  // An opaque zero keeps the 128 element addresses from being hoisted out of
  // the token loop (where they would occupy registers for the whole kernel).
  int opaque;
  asm volatile("v_mov_b32 %0, 0" : "=v"(opaque));
  const int lc = (lane & 31) + opaque, kh = lane >> 5;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const int j = col0 + bj * 32 + lc;
      float* p = Sslot + (int64_t)(row0 + bi * 32 + 4 * kh) * d + j;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = row0 + bi * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
        if ((!diag || i >= j) && i < d && j < d) p[(int64_t)(8 * (r >> 2) + (r & 3)) * d] += acc[bi][bj][r];
        acc[bi][bj][r] = 0.0f;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
}

// One (slot, tile) item: S[slot] tile (ti, tj) += X_slot^T X_slot over the slot's tokens.
__device__ __forceinline__ void syrk_tile(const uint16_t* __restrict__ xgT,
                                          const int64_t* __restrict__ pad_off, int slot, int tile,
                                          int d, float* __restrict__ S, uint16_t* lds) {
  const int64_t npad = pad_off[slot + 1] - pad_off[slot];
  if (npad == 0) return;
  int ti, tj;
  tile_of(tile, ti, tj);
  const bool diag = ti == tj;
  const uint16_t* base = xgT + pad_off[slot] * d;
  const uint16_t* Ag = base + (int64_t)ti * kT * npad;
  const uint16_t* Bg = base + (int64_t)tj * kT * npad;
  const int arows = min(kT, d - ti * kT), brows = min(kT, d - tj * kT);   // d % 256 may be 128

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const bool idle = diag && wm * 128 + 127 < wn * 64;   // part strictly above the diagonal

  f32x16 acc[4][2];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) acc[bi][bj] = f32x16{};

  // thread t moves 16-byte chunks q = t + 512u: row q/4, token chunk q%4.
  // Two register stages: the loads for step st+2 are issued while step st is
  // multiplied, so each load has a full step of products to arrive.
  struct Stage {
    uint4 a[2], b[2];
  };
  auto fetch = [&](Stage& r, int64_t k0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = tid + 512 * u, row = q >> 2, ch = q & 3;
      r.a[u] = row < arows ? *reinterpret_cast<const uint4*>(Ag + (int64_t)row * npad + k0 + ch * 8)
                           : make_uint4(0, 0, 0, 0);
      if (!diag)
        r.b[u] = row < brows ? *reinterpret_cast<const uint4*>(Bg + (int64_t)row * npad + k0 + ch * 8)
                             : make_uint4(0, 0, 0, 0);
    }
  };
  auto stage = [&](const Stage& r, int buf) {
    uint16_t* As = lds + (2 * buf) * kBuf;
    uint16_t* Bs = lds + (2 * buf + 1) * kBuf;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = tid + 512 * u, row = q >> 2, ch = q & 3;
      *reinterpret_cast<uint4*>(&As[row * kPitch + ch * 8]) = r.a[u];
      if (!diag) *reinterpret_cast<uint4*>(&Bs[row * kPitch + ch * 8]) = r.b[u];
    }
  };
  auto multiply = [&](int buf) {
    if (idle) return;
    const uint16_t* As = lds + (2 * buf) * kBuf;
    const uint16_t* Bs = diag ? As : lds + (2 * buf + 1) * kBuf;
#pragma unroll
    for (int kk = 0; kk < kSK / 16; ++kk) {
      const int kcol = kk * 16 + (lane >> 5) * 8;
      bf16x8 a[4], b[2];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        const int row = wm * 128 + bi * 32 + (lane & 31);
        a[bi] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&As[row * kPitch + kcol]));
      }
#pragma unroll
      for (int bj = 0; bj < 2; ++bj) {
        const int row = wn * 64 + bj * 32 + (lane & 31);
        b[bj] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&Bs[row * kPitch + kcol]));
      }
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
          acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi], b[bj], acc[bi][bj], 0, 0, 0);
    }
  };

  // nsteps is even (token lists are padded to 64); steps 2s and 2s+1 form a pair
  const int64_t nsteps = npad / kSK;
  Stage r0, r1;
  fetch(r0, 0);
  stage(r0, 0);
  fetch(r1, kSK);
  if (nsteps > 2) fetch(r0, 2 * kSK);
  __syncthreads();
  float* Sslot = S + (int64_t)slot * d * d;
  for (int64_t c0 = 0; c0 < nsteps; c0 += kFlushSteps) {
    const int64_t c1 = c0 + kFlushSteps < nsteps ? c0 + kFlushSteps : nsteps;
    for (int64_t st = c0; st < c1; st += 2) {
      // step st: LDS buffer 0 holds it, r1 holds st+1, r0 holds st+2 (if any)
      multiply(0);
      stage(r1, 1);
      if (st + 3 < nsteps) fetch(r1, (st + 3) * kSK);
      __syncthreads();
      // step st+1 from buffer 1; r0 (step st+2) goes to buffer 0
      multiply(1);
      if (st + 2 < nsteps) stage(r0, 0);
      if (st + 4 < nsteps) fetch(r0, (st + 4) * kSK);
      __syncthreads();
    }
    if (!idle) flush_acc(acc, Sslot, d, ti * kT + wm * 128, tj * kT + wn * 64, diag, lane);
  }
}

// Persistent workgroups, kSyrkWgPerXcd per die: workgroup b runs on die b % 8
// and takes items from that die's list until the list is exhausted, so all
// tiles of a slot read the slot's activations through one L2.
__global__ __launch_bounds__(512) void syrk_kernel(const uint16_t* __restrict__ xgT,
                                                   const int64_t* __restrict__ pad_off,
                                                   const int32_t* __restrict__ work,
                                                   const int32_t* __restrict__ work_len,
                                                   int32_t* __restrict__ work_next, int cap, int d,
                                                   float* __restrict__ S) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * kBuf];   // A0 B0 A1 B1
  __shared__ int item;
  const int x = blockIdx.x % kXcds;
  const int len = work_len[x];
  for (;;) {
    if (threadIdx.x == 0) item = atomicAdd(&work_next[x], 1);
    __syncthreads();
    const int it = item;
    __syncthreads();
    if (it >= len) break;
    const int code = work[x * cap + it];
    syrk_tile(xgT, pad_off, code >> 10, code & 1023, d, S, lds);
  }
}

void launch_syrk(const CollectPlan& p, float* S, hipStream_t s) {
  const int slots = p.E + p.has_shared;
  hipLaunchKernelGGL(syrk_kernel, dim3(kXcds * kSyrkWgPerXcd), dim3(512), 0, s, p.xgT, p.pad_off,
                     p.work, p.work_len, p.work_next, slots * p.syrk_tiles, p.d, S);
}

int syrk_tiles_per_slot(int d) {
  const int nt = (d + kT - 1) / kT;
  return nt * (nt + 1) / 2;
}

}  // namespace clha
