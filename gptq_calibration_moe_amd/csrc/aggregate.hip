// Aggregation phase: combined Hessian of every shared expert slot.
//
// CLHA summary, section 2.1 (Proposition 1): minimising the shared weight's
// total reconstruction error over the layers that use it is GPTQ on
// H_comb = sum_i alpha_i H_i.  Section 2.2 gives two weightings: routing
// frequency alpha_i = n_i / sum n ("CLHA-rt") and equal alpha = 0.5 ("CLHA-eq");
// PLIC (one primary layer) is alpha = (1, 0).
//
// With H_i = S_i / n_i, routing-frequency weighting is (sum_i S_i)/(sum_i n_i);
// that form is used here.  Equal and explicit weights form sum_i a_i (S_i / n_i)
// with separately rounded products and sums, in layer order, so that a = (1, 0)
// returns S_a/n_a bit for bit and two identical layers return S/n bit for bit.
// Any number of layers up to kMaxLayers combine the same way (Proposition 1 is
// stated for n layers); explicit weights may also differ per expert slot.
//
// Each workgroup reads one 64x64 lower-triangular tile of every layer's S and
// writes the tile and its mirror image, so H comes out full and symmetric.  A
// thread's four 16-byte positions of a layer are loaded together before they
// are summed, which keeps four loads in flight per thread.
#include "kernels.h"

namespace clha {

struct SlotWeights {
  float a[kMaxLayers];
  float inv_total;   // routing frequency: 1 / sum n (unused otherwise)
  int identity;      // no tokens at all: H = I
  int rt;
};

__device__ SlotWeights slot_weights(const AggArgs& g, int slot) {
  SlotWeights w;
  int64_t n[kMaxLayers];
  int64_t total = 0;
  int nonempty = 0;
  for (int l = 0; l < g.n_layers; ++l) {
    n[l] = g.counts[l][slot];
    total += n[l];
    nonempty += n[l] > 0;
  }
  w.identity = total == 0;
  w.rt = g.mode == 0;
  w.inv_total = 0.0f;
  for (int l = 0; l < kMaxLayers; ++l) w.a[l] = 0.0f;
  if (w.identity) return w;
  if (g.mode == 0) {
    for (int l = 0; l < g.n_layers; ++l) w.a[l] = (float)n[l] / (float)total;
  } else if (g.mode == 1) {
    const float a = 1.0f / (float)nonempty;
    for (int l = 0; l < g.n_layers; ++l) w.a[l] = n[l] > 0 ? a : 0.0f;
  } else {
    // explicit weights: one set for every slot (mode 2) or one per slot (mode 3)
    const float* al = g.mode == 3 ? g.alpha_slot + (int64_t)slot * g.n_layers : g.alpha;
    bool lost = false;
    float sum = 0.0f;
    for (int l = 0; l < g.n_layers; ++l) {
      lost |= (al[l] != 0.0f) && n[l] == 0;
      w.a[l] = n[l] > 0 ? al[l] : 0.0f;
      sum += w.a[l];
    }
    if (lost) {
      if (sum == 0.0f) {
        w.identity = 1;
        for (int l = 0; l < kMaxLayers; ++l) w.a[l] = 0.0f;
        return w;
      }
      for (int l = 0; l < g.n_layers; ++l) w.a[l] = w.a[l] / sum;
    }
  }
  return w;
}

__global__ __launch_bounds__(256) void aggregate_kernel(AggArgs g, float* __restrict__ H,
                                                        float* __restrict__ alpha_out) {
  __shared__ float T[64][65];
  const int slot = blockIdx.y;
  const int d = g.d;
  int t = blockIdx.x;
  int ti = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((ti + 1) * (ti + 2) / 2 <= t) ++ti;
  while (ti * (ti + 1) / 2 > t) --ti;
  const int tj = t - ti * (ti + 1) / 2;
  const bool diag = ti == tj;
  const SlotWeights w = slot_weights(g, slot);
  if (blockIdx.x == 0 && threadIdx.x < g.n_layers && alpha_out)
    alpha_out[slot * g.n_layers + threadIdx.x] = w.a[threadIdx.x];

  int64_t n[kMaxLayers];
  int64_t total = 0;
  for (int l = 0; l < g.n_layers; ++l) {
    n[l] = g.counts[l][slot];
    total += n[l];
  }
  const float ftotal = (float)total;
  float* Hs = H + (int64_t)slot * d * d;
  const int64_t soff = (int64_t)slot * d * d;
  // four 16-byte positions per thread (row r = idx / 16, columns c .. c+3, idx =
  // tid + 256k); every layer's loads of the four are issued before their sums.
  // On a diagonal tile the positions above the diagonal are loaded and summed
  // as well (in range, never stored), so all threads issue the same loads.
  float v[4][4];
  if (w.identity) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = threadIdx.x + 256 * k, r = idx >> 4, c = 4 * (idx & 15);
#pragma unroll
      for (int u = 0; u < 4; ++u) v[k][u] = (ti * 64 + r == tj * 64 + c + u) ? 1.0f : 0.0f;
    }
  } else {
    float acc[4][4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[k][u] = 0.0f;
    for (int l = 0; l < g.n_layers; ++l) {
      // a layer without tokens for this slot drops out (and, with explicit or
      // equal weights, so does a layer of weight zero)
      if (n[l] == 0 || (!w.rt && w.a[l] == 0.0f)) continue;
      float4 x[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int idx = threadIdx.x + 256 * k, r = idx >> 4, c = 4 * (idx & 15);
        x[k] = *reinterpret_cast<const float4*>(g.S[l] + soff + (int64_t)(ti * 64 + r) * d + tj * 64 + c);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float xs[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc[k][u] = w.rt ? __fadd_rn(acc[k][u], xs[u])
                           : __fadd_rn(acc[k][u], __fmul_rn(w.a[l], __fdiv_rn(xs[u], (float)n[l])));
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int u = 0; u < 4; ++u) v[k][u] = w.rt ? __fdiv_rn(acc[k][u], ftotal) : acc[k][u];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = threadIdx.x + 256 * k, r = idx >> 4, c = 4 * (idx & 15);
#pragma unroll
    for (int u = 0; u < 4; ++u) T[r][c + u] = v[k][u];
    // an off-diagonal tile is written here and mirrored below; a diagonal tile
    // is written whole below (its upper half from the mirror of its lower half:
    // S is not written above the diagonal)
    if (!diag)
      *reinterpret_cast<float4*>(Hs + (int64_t)(ti * 64 + r) * d + tj * 64 + c) =
          make_float4(v[k][0], v[k][1], v[k][2], v[k][3]);
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 64 * 16; idx += 256) {
    const int r = idx >> 4, c = 4 * (idx & 15);   // writes row tj*64 + r, columns ti*64 + c ..
    float* o = Hs + (int64_t)(tj * 64 + r) * d + ti * 64 + c;
    float4 t;
    if (!diag) {
      t = make_float4(T[c][r], T[c + 1][r], T[c + 2][r], T[c + 3][r]);
    } else {
      t.x = c <= r ? T[r][c] : T[c][r];
      t.y = c + 1 <= r ? T[r][c + 1] : T[c + 1][r];
      t.z = c + 2 <= r ? T[r][c + 2] : T[c + 2][r];
      t.w = c + 3 <= r ? T[r][c + 3] : T[c + 3][r];
    }
    *reinterpret_cast<float4*>(o) = t;
  }
}

void launch_aggregate(const AggArgs& a, float* H, float* alpha_out, hipStream_t s) {
  const int nt = a.d / 64;
  hipLaunchKernelGGL(aggregate_kernel, dim3(nt * (nt + 1) / 2, a.slots), dim3(256), 0, s, a, H,
                     alpha_out);
}

}  // namespace clha
