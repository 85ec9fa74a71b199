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
// The bucketing scan deals segments (token ranges of one slot, at most
// kSegTokens = one flush interval long) to per-XCD lists, a segment's items
// consecutive, the diagonal pairs first.  Persistent workgroups pull items
// from their die's list, so the 32 workgroups of a die start a segment's items
// together, run them side by side and read its activations through one L2;
// short segments keep them from drifting apart (a diagonal pair takes 9/8 of
// an off-diagonal tile's time, which over a long token range would leave the
// pairs reading panels the die's L2 no longer holds).  Every element of S is
// summed in a fixed order whichever workgroup takes the item, so results are
// bit-identical run to run.  The running sum is added into S every
// kFlushSteps token steps (two-level summation keeps the fp32 error
// independent of the expert's size); for the later segments of a slot it goes
// to a partial buffer, added into S in part order afterwards.
//
// Tile pipeline: 512 threads = 8 waves.  Tokens advance 32 at a time through
// four LDS stages filled by direct global-to-LDS loads (global_load_lds_dwordx4)
// issued three steps ahead (after each step's products), so no registers stage
// the operands and each load has three steps of products to arrive.  Each wave waits for its own loads of
// the step (vmcnt) and one barrier per step publishes them.  The activations
// are stored in blocks of 32 tokens, each block [d features][32 tokens], so a
// step's operand panel (256 features x 32 tokens) is one contiguous 16 KB run
// and every 128-byte line fetched is used whole in the step that fetches it.
// Operand tiles are [256 features][32 tokens] with 64-byte rows; a lane's MFMA
// fragment (8 consecutive tokens of one feature) is one 16-byte chunk, and the
// four chunks of row r sit at slots c ^ ((r >> 2) & 3), which makes the
// fragment reads bank-conflict free.
//   off-diagonal tile (ti, tj): waves in 2x4, each 128x64 as 4x2 32x32 blocks;
//   diagonal pair (p, q): waves 0-3 take panel p, waves 4-7 panel q; wave k of a
//     panel owns block rows 7-k and k (9 blocks), both operands from that panel.
#include "kernels.h"

namespace clha {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kT = 256;              // output tile
constexpr int kSK = 32;              // tokens per step
constexpr int kFlushSteps = 256;     // 8192 tokens between partial-sum flushes (multiple of kStages)
constexpr int kStages = 4;           // LDS stages; loads run kStages - 1 steps ahead
constexpr int kPanel = kT * kSK;     // one operand stage: 256 rows x 32 tokens (bf16 elements)

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef const __attribute__((address_space(1))) void* glb_ptr;

// The LDS stages, one array each so that the compiler can tell a stage being
// loaded from a stage being read.
struct Stages {
  uint16_t* a[kStages];
  uint16_t* b[kStages];
};

// s_waitcnt with vmcnt <= N and lgkmcnt == 0: this wave's global loads up to
// the N most recent have landed, and its LDS reads have all returned (so a
// barrier after it also means the wave is done reading the stages it read).
template <int N>
__device__ __forceinline__ void wait_loads() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | (((N >> 4) & 3) << 14));
}

// Byte offset in a stage of 16-byte chunk c (0..3) of row r.
__device__ __forceinline__ int chunk_off(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }

// The token pipeline shared by both item kinds.  Ag / Bg: the two panels' first
// rows in a 32-token block (row stride kSK, block stride bstride = d * kSK);
// t0, a multiple of kSK, is the first token; when !loadB only Ag is used.
// multiply(stage) runs one 32-token step from LDS stage `stage`; flush(first)
// adds the running sums.  Steps past nsteps are padding: their loads re-read
// the last step (clamped, always in range) and they run no products, so every
// wave issues the same loads, waits and barriers.
template <class Mul, class Flush>
__device__ __forceinline__ void token_loop(const uint16_t* __restrict__ Ag, const uint16_t* __restrict__ Bg,
                                           int64_t bstride, int64_t t0, int64_t nsteps, int arows, int brows,
                                           bool loadB, const Stages& sb, Mul&& multiply, Flush&& flush) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (!loadB) {
    Bg = Ag;
    brows = arows;
  }
  // wave w loads 1 KB blocks 2w and 2w+1 of each panel: 16 rows x 4 chunks,
  // lane l -> row 16 blk + l/4, LDS slot l%4 (holding chunk slot ^ ((row>>2)&3))
  const uint16_t* pa[2];
  const uint16_t* pb[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 16 * (2 * wave + j) + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    pa[j] = Ag + (int64_t)min(row, arows - 1) * kSK + (t0 / kSK) * bstride + c * 8;
    pb[j] = Bg + (int64_t)min(row, brows - 1) * kSK + (t0 / kSK) * bstride + c * 8;
  }
  auto issue = [&](int stage, int64_t st) {
    const int64_t k0 = (st < nsteps ? st : nsteps - 1) * bstride;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      __builtin_amdgcn_global_load_lds((glb_ptr)(pa[j] + k0), (lds_ptr)(sb.a[stage] + (2 * wave + j) * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((glb_ptr)(pb[j] + k0), (lds_ptr)(sb.b[stage] + (2 * wave + j) * 512), 16, 0, 0);
    }
  };
  // one step: this wave's loads for stage `stage` are done once at most the
  // loads of the (kStages - 2) later steps are outstanding.  The loads for
  // kStages - 1 steps ahead go into the stage every wave finished reading
  // before this step's barrier, and are issued after this step's products:
  // issued first, a wave waits for the address unit to take them before it
  // starts its products (measured: 8.38 to 8.05 ms per full-depth launch)
  auto step = [&](auto stage_c, int64_t st) {
    constexpr int stage = decltype(stage_c)::value;
    wait_loads<4 * (kStages - 2)>();
    __builtin_amdgcn_s_barrier();
    if (st < nsteps) multiply(stage);
    issue((stage + kStages - 1) % kStages, st + kStages - 1);
  };
  for (int64_t c0 = 0; c0 < nsteps; c0 += kFlushSteps) {
    // restart the pipeline (all earlier loads and stores drained)
    wait_loads<0>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int j = 0; j < kStages - 1; ++j) issue(j, c0 + j);
    const int64_t c1 = c0 + kFlushSteps < nsteps ? c0 + kFlushSteps : nsteps;
    for (int64_t st = c0; st < c1; st += kStages) {
      step(std::integral_constant<int, 0>{}, st);
      step(std::integral_constant<int, 1>{}, st + 1);
      step(std::integral_constant<int, 2>{}, st + 2);
      step(std::integral_constant<int, 3>{}, st + 3);
    }
    wait_loads<0>();
    __builtin_amdgcn_s_barrier();
    flush(c0 == 0);
  }
}

// Adds (or, for the first flush into a partial buffer, stores) one 32x32
// accumulator block at (row0, col0) of Sd; lower triangle and i, j < d only.
// S is touched once per flush, so its loads and stores are non-temporal: they
// stream past the L2, which keeps the activation panels other workgroups of
// the die are still reading.
__device__ __forceinline__ void flush_block(f32x16& acc, float* __restrict__ Sd, int d, int row0, int col0,
                                            bool diag, bool store, int lane) {
  // An opaque zero keeps the element addresses from being hoisted out of the
  // token loop (where they would occupy registers for the whole item).
  int opaque;
  asm volatile("v_mov_b32 %0, 0" : "=v"(opaque));
  const int lc = (lane & 31) + opaque, kh = lane >> 5;
  const int j = col0 + lc;
  float* p = Sd + (int64_t)(row0 + 4 * kh) * d + j;
  if (!diag && row0 + 32 <= d && col0 + 32 <= d) {
    // a block inside S and off the diagonal (the same for the whole wave): no
    // per-element tests, and the 16 loads are in flight together
    float old[16];
    if (!store) {
#pragma unroll
      for (int r = 0; r < 16; ++r) old[r] = __builtin_nontemporal_load(p + (int64_t)(8 * (r >> 2) + (r & 3)) * d);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      __builtin_nontemporal_store(store ? acc[r] : old[r] + acc[r], p + (int64_t)(8 * (r >> 2) + (r & 3)) * d);
      acc[r] = 0.0f;
    }
    __builtin_amdgcn_sched_barrier(0);
    return;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = row0 + 8 * (r >> 2) + 4 * kh + (r & 3);
    float* e = p + (int64_t)(8 * (r >> 2) + (r & 3)) * d;
    if ((!diag || i >= j) && i < d && j < d)
      __builtin_nontemporal_store(store ? acc[r] : __builtin_nontemporal_load(e) + acc[r], e);
    acc[r] = 0.0f;
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Off-diagonal tile (ti, tj), ti > tj: waves 2x4, each 128x64.
__device__ __forceinline__ void syrk_offdiag(const uint16_t* base, int64_t t0, int64_t nsteps,
                                             int d, int ti, int tj, float* Sd, bool partial, const Stages& sb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  f32x16 acc[4][2];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) acc[bi][bj] = f32x16{};
  auto multiply = [&](int stage) {
    const char* As = reinterpret_cast<const char*>(sb.a[stage]);
    const char* Bs = reinterpret_cast<const char*>(sb.b[stage]);
#pragma unroll
    for (int kk = 0; kk < kSK / 16; ++kk) {
      const int c = 2 * kk + (lane >> 5);
      bf16x8 a[4], b[2];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
        a[bi] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(As + chunk_off(wm * 128 + bi * 32 + (lane & 31), c)));
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
        b[bj] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Bs + chunk_off(wn * 64 + bj * 32 + (lane & 31), c)));
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
  token_loop(base + (int64_t)ti * kT * kSK, base + (int64_t)tj * kT * kSK, (int64_t)d * kSK, t0, nsteps,
             min(kT, d - ti * kT), min(kT, d - tj * kT), true, sb, multiply, flush);
}

// Diagonal pair: this wave's share of panel P's diagonal tile -- block rows
// 7-K (columns 0..7-K) and K (columns 0..K) -- read from LDS buffer half `pb`.
template <int K>
__device__ __forceinline__ void syrk_diag_wave(const uint16_t* Ag, const uint16_t* Bg, bool loadB, int64_t bstride,
                                               int64_t t0, int64_t nsteps, int d, int P, int pb, bool active,
                                               float* Sd, bool partial, int arows, int brows, const Stages& sb) {
  constexpr int R1 = 7 - K, R2 = K, NA = 8 - K;   // NA fragments: panel blocks 0..7-K
  const int lane = threadIdx.x & 63;
  f32x16 acc[9];
#pragma unroll
  for (int x = 0; x < 9; ++x) acc[x] = f32x16{};
  auto multiply = [&](int stage) {
    if (!active) return;
    const char* Ps = reinterpret_cast<const char*>(pb ? sb.b[stage] : sb.a[stage]);
#pragma unroll
    for (int kk = 0; kk < kSK / 16; ++kk) {
      const int c = 2 * kk + (lane >> 5);
      bf16x8 f[NA];
#pragma unroll
      for (int cb = 0; cb < NA; ++cb)
        f[cb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Ps + chunk_off(cb * 32 + (lane & 31), c)));
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
  token_loop(Ag, Bg, bstride, t0, nsteps, arows, brows, loadB, sb, multiply, flush);
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
                                          float* __restrict__ S, float* __restrict__ partials, bool overwrite,
                                          const Stages& sb) {
  const int slot = seg[4 * sg], dest = seg[4 * sg + 1];
  const int64_t t0 = seg[4 * sg + 2], ntok = seg[4 * sg + 3];
  const uint16_t* base = xgT + pad_off[slot] * d;
  const int64_t dd = (int64_t)d * d;
  float* Sd = dest < 0 ? S + (int64_t)slot * dd : partials + (int64_t)dest * dd;
  // the first flush of a partial buffer stores; so does the first flush into S
  // when this collection overwrites the layer's sums
  const bool partial = dest >= 0 || overwrite;
  const int64_t nsteps = ntok / kSK;
  const int nt = (d + kT - 1) / kT, nd = (nt + 1) / 2;
  if (item >= nd) {
    int a, b;
    tile_of(item - nd, a, b);
    syrk_offdiag(base, t0, nsteps, d, a + 1, b, Sd, partial, sb);
    return;
  }
  const int p = item, q = nt - 1 - item;
  const bool single = p == q;
  const int wave = threadIdx.x >> 6, hp = wave >> 2, k = wave & 3;
  const int P = hp ? q : p;
  const bool active = !(hp && single);
  const uint16_t* Ag = base + (int64_t)p * kT * kSK;
  const uint16_t* Bg = base + (int64_t)q * kT * kSK;
  const int64_t bstride = (int64_t)d * kSK;
  const int arows = min(kT, d - p * kT), brows = min(kT, d - q * kT);
  switch (k) {
    case 0: syrk_diag_wave<0>(Ag, Bg, !single, bstride, t0, nsteps, d, P, hp, active, Sd, partial, arows, brows, sb); break;
    case 1: syrk_diag_wave<1>(Ag, Bg, !single, bstride, t0, nsteps, d, P, hp, active, Sd, partial, arows, brows, sb); break;
    case 2: syrk_diag_wave<2>(Ag, Bg, !single, bstride, t0, nsteps, d, P, hp, active, Sd, partial, arows, brows, sb); break;
    default: syrk_diag_wave<3>(Ag, Bg, !single, bstride, t0, nsteps, d, P, hp, active, Sd, partial, arows, brows, sb); break;
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
                                                   float* __restrict__ S, float* __restrict__ partials,
                                                   int overwrite) {
  __shared__ __attribute__((aligned(16))) uint16_t a0[kPanel], a1[kPanel], a2[kPanel], a3[kPanel];
  __shared__ __attribute__((aligned(16))) uint16_t b0[kPanel], b1[kPanel], b2[kPanel], b3[kPanel];
  __shared__ int item;
  const Stages sb{{a0, a1, a2, a3}, {b0, b1, b2, b3}};
  const int x = blockIdx.x % kXcds;
  const int len = work_len[x];
  for (;;) {
    if (threadIdx.x == 0) item = atomicAdd(&work_next[x], 1);
    __syncthreads();
    const int it = item;
    __syncthreads();
    if (it >= len) break;
    const int code = work[x * cap + it];
    syrk_item(xgT, pad_off, seg, code >> 10, code & 1023, d, S, partials, overwrite != 0, sb);
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
    const float* pp = partials + (int64_t)p0 * dd + off;
    auto add = [&](const float4& w) {
      v.x += w.x;
      v.y += w.y;
      v.z += w.z;
      v.w += w.w;
    };
    // four parts' loads in flight together; the sums stay in part order
    int k = 0;
    for (; k + 4 <= np; k += 4) {
      float4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = *reinterpret_cast<const float4*>(pp + (int64_t)(k + u) * dd);
#pragma unroll
      for (int u = 0; u < 4; ++u) add(w[u]);
    }
    for (; k < np; ++k) add(*reinterpret_cast<const float4*>(pp + (int64_t)k * dd));
    // columns above the diagonal keep their value (S's upper triangle is never written)
    if (j + 1 > i) v.y = o[1];
    if (j + 2 > i) v.z = o[2];
    if (j + 3 > i) v.w = o[3];
    *reinterpret_cast<float4*>(o) = v;
  }
}

// When a collection overwrites the layer's sums, a slot that received no
// token has no Gram-sum item: its lower triangle is zeroed here instead.
// One workgroup per slot; slots with tokens return at once.
__global__ __launch_bounds__(256) void zero_empty_slots_kernel(const int64_t* __restrict__ counts,
                                                               float* __restrict__ S, int d) {
  const int slot = blockIdx.x;
  if (counts[slot] != 0) return;
  float* Ss = S + (int64_t)slot * d * d;
  for (int i = 0; i < d; ++i)
    for (int j = 4 * (int)threadIdx.x; j <= i; j += 1024) {
      float* o = Ss + (int64_t)i * d + j;
      if (j + 3 <= i) {
        *reinterpret_cast<float4*>(o) = make_float4(0.f, 0.f, 0.f, 0.f);
      } else {
        for (int u = 0; j + u <= i; ++u) o[u] = 0.0f;
      }
    }
}

void launch_syrk(const CollectPlan& p, float* S, hipStream_t s) {
  hipLaunchKernelGGL(syrk_kernel, dim3(kXcds * kSyrkWgPerXcd), dim3(512), 0, s, p.xgT, p.pad_off, p.work,
                     p.work_len, p.work_next, p.seg, p.max_segs * p.syrk_items, p.d, S, p.partials,
                     p.overwrite);
}

// After the Gram-sum kernel.  The slots zeroed here received no token, so no
// Gram-sum item or partial buffer touches them.
void launch_syrk_reduce(const CollectPlan& p, float* S, const int64_t* layer_counts, hipStream_t s) {
  hipLaunchKernelGGL(syrk_reduce_kernel, dim3((p.d + 1023) / 1024, p.d), dim3(256), 0, s, p.split,
                     p.partials, S, p.d);
  if (p.overwrite)
    hipLaunchKernelGGL(zero_empty_slots_kernel, dim3(p.E + p.has_shared), dim3(256), 0, s, layer_counts, S,
                       p.d);
}

int syrk_items_per_slot(int d) {
  const int nt = (d + kT - 1) / kT;
  return nt * (nt - 1) / 2 + (nt + 1) / 2;
}

}  // namespace clha
