// Collection phase, second half: per-slot Gram sums S[e] += X_e^T X_e.
//
// CLHA summary, section 2.1: the Hessian of a layer for a weight fed by
// activations x is the (uncentred) activation second moment; section 2.2
// accumulates it per layer and per active expert over the calibration data.
// Products of bf16 values are exact in fp32; they are accumulated in fp32 on
// the matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Work decomposition.  S is symmetric, so only its lower triangle is computed,
// in 256-row panels (nt = d/256 rounded up).  The items of one slot are the
// nt(nt-1)/2 off-diagonal 256x256 tiles and the nt diagonal tiles taken in
// pairs (p, nt-1-p): a diagonal tile's lower triangle is 36 of 64 32x32 blocks,
// a pair is 72 blocks, 9 per wave, so every item is about one tile of work
// (d = 2048: 28 + 4 = 32 items per slot, one per CU of an XCD).
// The bucketing scan deals segments (token ranges of one slot) to per-XCD
// lists, a segment's items consecutive, the diagonal pairs first.  Persistent
// workgroups pull items from their die's list; since a segment's items take
// about equally long, the 32 workgroups of a die run one segment's items side
// by side and read its activations through one L2.  Every element of S is
// summed in a fixed order whichever workgroup takes the item, so results are
// bit-identical run to run.  The running sum is added into S every
// kFlushSteps token steps (two-level summation keeps the fp32 error
// independent of the expert's size); for the later token ranges of a split
// slot it goes to a partial buffer, added into S in part order afterwards.
//
// Tile pipeline: 512 threads = 8 waves.  Tokens advance 32 at a time through
// two LDS buffers and two register stages: while the matrix cores consume one
// buffer, the other buffer is filled from the register stage loaded a step
// earlier, and the register stage is refilled with the step after that -- each
// global load has a full step to arrive.  Operand tiles are feature-major
// [256 features][32 tokens]; a lane's MFMA fragment (8 consecutive tokens of
// one feature) is one 16-byte LDS read, and the row pitch of 40 bf16 (80 bytes)
// keeps those reads bank-conflict free.
//   off-diagonal tile (ti, tj): waves in 2x4, each 128x64 as 4x2 32x32 blocks;
//   diagonal pair (p, q): waves 0-3 take panel p, waves 4-7 panel q; wave k of a
//     panel owns block rows 7-k and k (9 blocks), both operands from that panel.
#include "kernels.h"

namespace clha {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kT = 256;              // output tile
constexpr int kSK = 32;              // tokens per step
constexpr int kPitch = kSK + 8;      // LDS row pitch (bf16 elements, 80 bytes)
constexpr int kFlushSteps = 256;     // 8192 tokens between partial-sum flushes (even)
constexpr int kBuf = kT * kPitch;    // one operand buffer (bf16 elements)

// The token pipeline shared by both item kinds.  Ag / Bg: feature-major rows of
// the two panels (row stride npad); Bg unused when !loadB.  multiply(buf) runs
// one 32-token step from LDS buffer buf; flush(first) adds the running sums.
template <class Mul, class Flush>
__device__ __forceinline__ void token_loop(const uint16_t* __restrict__ Ag, const uint16_t* __restrict__ Bg,
                                           int64_t npad, int64_t t0, int64_t nsteps, int arows, int brows,
                                           bool loadB, uint16_t* lds, Mul&& multiply, Flush&& flush) {
  const int tid = threadIdx.x;
  // thread t moves 16-byte chunks q = t + 512u: row q/4, token chunk q%4
  struct Stage {
    uint4 a[2], b[2];
  };
  auto fetch = [&](Stage& r, int64_t k0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = tid + 512 * u, row = q >> 2, ch = q & 3;
      r.a[u] = row < arows ? *reinterpret_cast<const uint4*>(Ag + (int64_t)row * npad + t0 + k0 + ch * 8)
                           : make_uint4(0, 0, 0, 0);
      if (loadB)
        r.b[u] = row < brows ? *reinterpret_cast<const uint4*>(Bg + (int64_t)row * npad + t0 + k0 + ch * 8)
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
      if (loadB) *reinterpret_cast<uint4*>(&Bs[row * kPitch + ch * 8]) = r.b[u];
    }
  };
  // nsteps is even (token ranges are multiples of 64); steps 2s and 2s+1 form a pair
  Stage r0, r1;
  fetch(r0, 0);
  stage(r0, 0);
  fetch(r1, kSK);
  if (nsteps > 2) fetch(r0, 2 * kSK);
  __syncthreads();
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
    flush(c0 == 0);
  }
}

// Adds (or, for the first flush into a partial buffer, stores) one 32x32
// accumulator block at (row0, col0) of Sd; lower triangle and i, j < d only.
__device__ __forceinline__ void flush_block(f32x16& acc, float* __restrict__ Sd, int d, int row0, int col0,
                                            bool diag, bool store, int lane) {
  // An opaque zero keeps the element addresses from being hoisted out of the
  // token loop (where they would occupy registers for the whole item).
  int opaque;
  asm volatile("v_mov_b32 %0, 0" : "=v"(opaque));
  const int lc = (lane & 31) + opaque, kh = lane >> 5;
  const int j = col0 + lc;
  float* p = Sd + (int64_t)(row0 + 4 * kh) * d + j;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = row0 + 8 * (r >> 2) + 4 * kh + (r & 3);
    float* e = p + (int64_t)(8 * (r >> 2) + (r & 3)) * d;
    if ((!diag || i >= j) && i < d && j < d) *e = store ? acc[r] : *e + acc[r];
    acc[r] = 0.0f;
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Off-diagonal tile (ti, tj), ti > tj: waves 2x4, each 128x64.
__device__ __forceinline__ void syrk_offdiag(const uint16_t* base, int64_t npad, int64_t t0, int64_t nsteps,
                                             int d, int ti, int tj, float* Sd, bool partial, uint16_t* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  f32x16 acc[4][2];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) acc[bi][bj] = f32x16{};
  auto multiply = [&](int buf) {
    const uint16_t* As = lds + (2 * buf) * kBuf;
    const uint16_t* Bs = lds + (2 * buf + 1) * kBuf;
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
  auto flush = [&](bool first) {
    const bool store = partial && first;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
        flush_block(acc[bi][bj], Sd, d, ti * kT + wm * 128 + bi * 32, tj * kT + wn * 64 + bj * 32, false,
                    store, lane);
  };
  token_loop(base + (int64_t)ti * kT * npad, base + (int64_t)tj * kT * npad, npad, t0, nsteps,
             min(kT, d - ti * kT), min(kT, d - tj * kT), true, lds, multiply, flush);
}

// Diagonal pair: this wave's share of panel P's diagonal tile -- block rows
// 7-K (columns 0..7-K) and K (columns 0..K) -- read from LDS buffer half `pb`.
template <int K>
__device__ __forceinline__ void syrk_diag_wave(const uint16_t* Ag, const uint16_t* Bg, bool loadB, int64_t npad,
                                               int64_t t0, int64_t nsteps, int d, int P, int pb, bool active,
                                               float* Sd, bool partial, int arows, int brows, uint16_t* lds) {
  constexpr int R1 = 7 - K, R2 = K, NA = 8 - K;   // NA fragments: panel blocks 0..7-K
  const int lane = threadIdx.x & 63;
  f32x16 acc[9];
#pragma unroll
  for (int x = 0; x < 9; ++x) acc[x] = f32x16{};
  auto multiply = [&](int buf) {
    if (!active) return;
    const uint16_t* Ps = lds + (2 * buf + pb) * kBuf;
#pragma unroll
    for (int kk = 0; kk < kSK / 16; ++kk) {
      const int kcol = kk * 16 + (lane >> 5) * 8;
      bf16x8 f[NA];
#pragma unroll
      for (int cb = 0; cb < NA; ++cb)
        f[cb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&Ps[(cb * 32 + (lane & 31)) * kPitch + kcol]));
#pragma unroll
      for (int cb = 0; cb <= R1; ++cb)
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[R1], f[cb], acc[cb], 0, 0, 0);
#pragma unroll
      for (int cb = 0; cb <= R2; ++cb)
        acc[NA + cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[R2], f[cb], acc[NA + cb], 0, 0, 0);
    }
  };
  auto flush = [&](bool first) {
    if (!active) return;
    const bool store = partial && first;
#pragma unroll
    for (int cb = 0; cb <= R1; ++cb)
      flush_block(acc[cb], Sd, d, P * kT + R1 * 32, P * kT + cb * 32, cb == R1, store, lane);
#pragma unroll
    for (int cb = 0; cb <= R2; ++cb)
      flush_block(acc[NA + cb], Sd, d, P * kT + R2 * 32, P * kT + cb * 32, cb == R2, store, lane);
  };
  token_loop(Ag, Bg, npad, t0, nsteps, arows, brows, loadB, lds, multiply, flush);
}

__device__ __forceinline__ void tile_of(int t, int& ti, int& tj) {
  int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  while (i * (i + 1) / 2 > t) --i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

// One item of one segment.
__device__ __forceinline__ void syrk_item(const uint16_t* __restrict__ xgT, const int64_t* __restrict__ pad_off,
                                          const int32_t* __restrict__ seg, int sg, int item, int d,
                                          float* __restrict__ S, float* __restrict__ partials, uint16_t* lds) {
  const int slot = seg[4 * sg], dest = seg[4 * sg + 1];
  const int64_t t0 = seg[4 * sg + 2], ntok = seg[4 * sg + 3];
  const int64_t npad = pad_off[slot + 1] - pad_off[slot];
  const uint16_t* base = xgT + pad_off[slot] * d;
  const int64_t dd = (int64_t)d * d;
  float* Sd = dest < 0 ? S + (int64_t)slot * dd : partials + (int64_t)dest * dd;
  const bool partial = dest >= 0;
  const int64_t nsteps = ntok / kSK;
  const int nt = (d + kT - 1) / kT, nd = (nt + 1) / 2;
  if (item >= nd) {
    int a, b;
    tile_of(item - nd, a, b);
    syrk_offdiag(base, npad, t0, nsteps, d, a + 1, b, Sd, partial, lds);
    return;
  }
  const int p = item, q = nt - 1 - item;
  const bool single = p == q;
  const int wave = threadIdx.x >> 6, hp = wave >> 2, k = wave & 3;
  const int P = hp ? q : p;
  const bool active = !(hp && single);
  const uint16_t* Ag = base + (int64_t)p * kT * npad;
  const uint16_t* Bg = base + (int64_t)q * kT * npad;
  const int arows = min(kT, d - p * kT), brows = min(kT, d - q * kT);
  switch (k) {
    case 0: syrk_diag_wave<0>(Ag, Bg, !single, npad, t0, nsteps, d, P, hp, active, Sd, partial, arows, brows, lds); break;
    case 1: syrk_diag_wave<1>(Ag, Bg, !single, npad, t0, nsteps, d, P, hp, active, Sd, partial, arows, brows, lds); break;
    case 2: syrk_diag_wave<2>(Ag, Bg, !single, npad, t0, nsteps, d, P, hp, active, Sd, partial, arows, brows, lds); break;
    default: syrk_diag_wave<3>(Ag, Bg, !single, npad, t0, nsteps, d, P, hp, active, Sd, partial, arows, brows, lds); break;
  }
}

// Persistent workgroups, kSyrkWgPerXcd per die: workgroup b runs on die b % 8
// and takes items from that die's list until the list is exhausted.
__global__ __launch_bounds__(512) void syrk_kernel(const uint16_t* __restrict__ xgT,
                                                   const int64_t* __restrict__ pad_off,
                                                   const int32_t* __restrict__ work,
                                                   const int32_t* __restrict__ work_len,
                                                   int32_t* __restrict__ work_next,
                                                   const int32_t* __restrict__ seg, int cap, int d,
                                                   float* __restrict__ S, float* __restrict__ partials) {
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
    syrk_item(xgT, pad_off, seg, code >> 10, code & 1023, d, S, partials, lds);
  }
}

// S[slot] (lower triangle) += the partial sums of each token-split slot, in
// part order.  Row i per block row, four columns per thread.
__global__ __launch_bounds__(256) void syrk_reduce_kernel(const int32_t* __restrict__ split,
                                                          const float* __restrict__ partials,
                                                          float* __restrict__ S, int d) {
  const int nsplit = split[0];
  const int i = blockIdx.y, j = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (nsplit == 0 || j > i || j >= d) return;
  const int64_t dd = (int64_t)d * d, off = (int64_t)i * d + j;
  for (int sp = 0; sp < nsplit; ++sp) {
    const int slot = split[1 + 3 * sp], p0 = split[2 + 3 * sp], np = split[3 + 3 * sp];
    float* o = S + (int64_t)slot * dd + off;
    float4 v = *reinterpret_cast<const float4*>(o);
    for (int k = 0; k < np; ++k) {
      const float4 w = *reinterpret_cast<const float4*>(partials + (int64_t)(p0 + k) * dd + off);
      v.x += w.x;
      v.y += w.y;
      v.z += w.z;
      v.w += w.w;
    }
    // columns above the diagonal keep their value (S's upper triangle is never written)
    if (j + 1 > i) v.y = o[1];
    if (j + 2 > i) v.z = o[2];
    if (j + 3 > i) v.w = o[3];
    *reinterpret_cast<float4*>(o) = v;
  }
}

void launch_syrk(const CollectPlan& p, float* S, hipStream_t s) {
  hipLaunchKernelGGL(syrk_kernel, dim3(kXcds * kSyrkWgPerXcd), dim3(512), 0, s, p.xgT, p.pad_off, p.work,
                     p.work_len, p.work_next, p.seg, kMaxSegs * p.syrk_items, p.d, S, p.partials);
  hipLaunchKernelGGL(syrk_reduce_kernel, dim3((p.d + 1023) / 1024, p.d), dim3(256), 0, s, p.split,
                     p.partials, S, p.d);
}

int syrk_items_per_slot(int d) {
  const int nt = (d + kT - 1) / kT;
  return nt * (nt - 1) / 2 + (nt + 1) / 2;
}

}  // namespace clha
