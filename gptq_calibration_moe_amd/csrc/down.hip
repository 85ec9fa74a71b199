// Inputs of the experts' second matrix (down_proj): the SwiGLU intermediate.
//
// CLHA summary, section 2.2: the collection phase accumulates, per layer and
// per active expert, the Hessian of every shared weight over that weight's own
// input.  The input of an expert's down_proj is its intermediate activation
//   h = bf16( silu(x Wg^T) * (x Wu^T) ),   silu(g) = g / (1 + e^-g),
// computed from the full-precision gate and up weights, so each routed expert
// (over its routed tokens) and each shared expert (over all tokens, with its
// own weights) has its own down_proj Hessian, summed by the same Gram-sum
// kernel at width f (the intermediate size).
//
// Grouped GEMM: for every slot, C = [Wg; Wu] X_e^T with K = d_model, in tiles
// of 128 features (their 128 gate and 128 up rows) x 128 tokens.  256 threads
// = 4 waves; wave (wf, wt) owns features 64wf.. and tokens 64wt.. as 2x2
// blocks of 32x32 for gate and the same for up (v_mfma_f32_32x32x16_bf16), so
// each lane holds the gate and up value of the same (feature, token) and the
// SwiGLU product is formed in registers.  Both operands are K-contiguous rows
// (weight rows; token rows of x, gathered through the routing's token lists),
// staged through two LDS buffers in chunks of 32 from two register stages;
// rows are 64 bytes with the four 16-byte chunks of row r at slots
// c ^ ((r >> 2) & 3); each chunk is fetched two products ahead of its
// staging.  The output is bf16 with zeros for the padding tokens, in the
// layout the Gram-sum kernel reads: per slot, blocks of 32 tokens, each block
// [f][32] (element (feature, t) at ((t/32)*f + feature)*32 + t%32).
#include "kernels.h"

namespace clha {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kDF = 128;   // features per tile
constexpr int kDT = 128;   // tokens per tile
constexpr int kDK = 32;    // model dimension per chunk (64-byte rows)
constexpr int kDG = 2;     // feature tiles per group of the tile order (see the kernel)

__device__ __forceinline__ int down_off(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }

__device__ __forceinline__ uint16_t bf16_rne(float v) {
  uint32_t b = __float_as_uint(v);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__global__ __launch_bounds__(256, 2) void down_gemm_kernel(const uint16_t* __restrict__ x, int dm,
                                                           const int32_t* __restrict__ token_ids,
                                                           const int64_t* __restrict__ roff, int E, int64_t n,
                                                           const uint16_t* const* __restrict__ wgu,
                                                           const int64_t* __restrict__ pad_off,
                                                           const int32_t* __restrict__ tile_off, int slots,
                                                           int f, uint16_t* __restrict__ hT, int64_t grid_tiles) {
  __shared__ __attribute__((aligned(16))) char As[2][2 * kDF * 64];   // gate rows 0..127, up rows 128..255
  __shared__ __attribute__((aligned(16))) char Bs[2][kDT * 64];
  const int nft = f / kDF;
  const int64_t total = (int64_t)tile_off[slots] * nft;
  // tiles of one slot run on one XCD (workgroup b runs on XCD b % 8)
  const int64_t per = (grid_tiles + kXcds - 1) / kXcds;
  const int64_t L = (int64_t)(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (L >= total) return;
  // the slot owns workgroups [tile_off[e] nft, tile_off[e+1] nft); inside it the
  // order is kDG feature tiles at a time, all token tiles per group, the kDG
  // tiles of one token tile adjacent: the workgroups an XCD runs together share
  // kDG weight slices (2 MB at kDG = 2) and read each x panel once per group,
  // where a token-tile-major order cycled through the expert's whole 11.5 MB of
  // weights, more than an XCD's L2 holds
  const int ttg = (int)(L / nft);
  int lo = 0, hi = slots;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_off[mid] <= ttg) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int T = tile_off[e + 1] - tile_off[e];
  const int64_t l = L - (int64_t)tile_off[e] * nft;
  const int g = (int)(l / ((int64_t)kDG * T));
  const int gs = min(kDG, nft - g * kDG);
  const int within = (int)(l - (int64_t)g * kDG * T);
  const int tt = within / gs, ft = g * kDG + within % gs;
  const int t0 = tt * kDT;
  const int64_t cnt = e < E ? roff[e + 1] - roff[e] : n;
  const int64_t npad = pad_off[e + 1] - pad_off[e];
  const int f0 = ft * kDF;
  const uint16_t* W = wgu[e];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wf = wave >> 1, wt = wave & 1;

  // this thread's 16-byte pieces of a chunk: A rows q/4 for q = tid + 256u
  // (u < 4), B rows q/4 for q = tid + 256u (u < 2); chunk q % 4 of the row
  const uint16_t* ap[4];
  const uint16_t* bp[2];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = (tid + 256 * u) >> 2, c = tid & 3;
    const int wrow = r < kDF ? f0 + r : f + f0 + (r - kDF);
    ap[u] = W + (int64_t)wrow * dm + 8 * c;
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = (tid + 256 * u) >> 2, c = tid & 3;
    int64_t tok = t0 + r;
    tok = tok < cnt ? tok : (cnt > 0 ? cnt - 1 : 0);   // padding rows read a valid row; their h is zeroed
    const int64_t src = e < E ? (int64_t)token_ids[roff[e] + tok] : tok;
    bp[u] = x + src * dm + 8 * c;
  }
  const int nk = dm / kDK;   // even (d_model is a multiple of 64)
  struct Stage {
    i32x4 a[4], b[2];
  };
  auto fetch = [&](Stage& r, int kc) {
    kc = kc < nk ? kc : nk - 1;   // unconditional: clamped past the end
#pragma unroll
    for (int u = 0; u < 4; ++u) r.a[u] = *reinterpret_cast<const i32x4*>(ap[u] + kDK * kc);
#pragma unroll
    for (int u = 0; u < 2; ++u) r.b[u] = *reinterpret_cast<const i32x4*>(bp[u] + kDK * kc);
  };
  auto stage = [&](const Stage& r, int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<i32x4*>(As[buf] + down_off((tid + 256 * u) >> 2, tid & 3)) = r.a[u];
#pragma unroll
    for (int u = 0; u < 2; ++u) *reinterpret_cast<i32x4*>(Bs[buf] + down_off((tid + 256 * u) >> 2, tid & 3)) = r.b[u];
  };
  f32x16 acc[2][2][2];   // [gate/up][feature block][token block]
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[g][a][b] = f32x16{};
  auto multiply = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < kDK / 16; ++kk) {
      const int c = 2 * kk + (lane >> 5);
      bf16x8 af[2][2], bf[2];
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int a = 0; a < 2; ++a)
          af[g][a] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const i32x4*>(As[buf] + down_off(g * kDF + 64 * wf + 32 * a + (lane & 31), c)));
#pragma unroll
      for (int b = 0; b < 2; ++b)
        bf[b] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(Bs[buf] + down_off(64 * wt + 32 * b + (lane & 31), c)));
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b)
            acc[g][a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[g][a], bf[b], acc[g][a][b], 0, 0, 0);
    }
  };
  // two register stages: a chunk is fetched two products ahead of its staging
  Stage g0, g1;
  fetch(g0, 0);
  stage(g0, 0);
  fetch(g1, 1);
  fetch(g0, 2);
  __syncthreads();
#pragma unroll 1
  for (int kc = 0; kc < nk; kc += 2) {
    // chunk kc in buffer 0, kc+1 in g1, kc+2 in g0
    multiply(0);
    stage(g1, 1);
    fetch(g1, kc + 3);
    __syncthreads();
    multiply(1);
    stage(g0, 0);
    fetch(g0, kc + 4);
    __syncthreads();
  }
  // h = silu(g) * u, zero for padding tokens; rows past the slot's padded range are not written
  uint16_t* out = hT + pad_off[e] * f;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t tok = t0 + 64 * wt + 32 * b + (lane & 31);
      if (tok >= npad) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int feat = f0 + 64 * wf + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const float g = acc[0][a][b][r], u = acc[1][a][b][r];
        const float h = tok < cnt ? g / (1.0f + expf(-g)) * u : 0.0f;
        out[((tok >> 5) * f + feat) * 32 + (tok & 31)] = bf16_rne(h);
      }
    }
}

void launch_down_gemm(const uint16_t* x, int d_model, const int32_t* token_ids, const int64_t* routed_offsets,
                      int E, int64_t n, const uint16_t* const* wgu, const CollectPlan& p, const int32_t* tile_off,
                      int64_t max_tiles, hipStream_t s) {
  const int64_t tiles = max_tiles * (p.d / kDF);
  const int64_t grid = (tiles + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL(down_gemm_kernel, dim3((unsigned)grid), dim3(256), 0, s, x, d_model, token_ids,
                     routed_offsets, E, n, wgu, p.pad_off, tile_off, p.E, p.d, p.xgT, grid);
}

}  // namespace clha
