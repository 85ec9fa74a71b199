// Collection phase, first half: top-K routing, per-expert bucketing and the
// gather of each expert's rows into a token-blocked, feature-major layout.
//
// CLHA summary, section 2.2 (collection): per calibration batch, every layer
// accumulates a Hessian and a token count for each expert that is active for
// its tokens; section 2.3: routed experts see the K/E fraction of tokens the
// router sends them, shared experts see all N tokens.
//
// Layout produced here (all in the caller's workspace):
//   topk        int32 [N][K]        experts of each token, larger logit first
//   offsets     int64 [E+1]         exclusive prefix sum of per-expert counts
//   token_ids   int32 [N*K]         tokens of expert e at offsets[e].., ascending
//   pad_off     int64 [slots+1]     start of slot e's token columns in xgT,
//                                   each slot padded to a multiple of 64 tokens;
//                                   slot E (if the block has shared experts) holds
//                                   all N tokens in order
//   xgT         bf16  per slot e, at xgT + pad_off[e]*d: npad_e/32 blocks of
//                     32 tokens, each block [d][32] (feature-major inside the
//                     block); element (f, t) at ((t/32)*d + f)*32 + t%32;
//                     padding tokens are zero
// Inside a block the Gram sum's contraction index (tokens) is contiguous, which
// is the operand layout the matrix cores read, and the 32-token step of 256
// features that one Gram-sum workgroup reads is one contiguous 16 KB run, so
// every 128-byte line it fetches is used whole in one step.
#include "kernels.h"

namespace clha {

// ------------------------------------------------------------------ routing

__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int64_t n,
                                                    int E, int K, int32_t* __restrict__ topk,
                                                    int* __restrict__ status) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  const float* row = logits + t * E;
  float val[kMaxTopK];
  int idx[kMaxTopK];
#pragma unroll
  for (int p = 0; p < kMaxTopK; ++p) {
    val[p] = -INFINITY;
    idx[p] = 0x7fffffff;
  }
  bool bad = false;
  for (int e = 0; e < E; ++e) {
    float cv = row[e];
    int ci = e;
    bad |= !isfinite(cv);
    // insertion into the list ordered by (logit descending, index ascending);
    // an element pushed down keeps moving past entries it precedes, so equal
    // logits always end up in index order
#pragma unroll
    for (int p = 0; p < kMaxTopK; ++p) {
      if (p < K) {
        const bool gt = cv > val[p] || (cv == val[p] && ci < idx[p]) || idx[p] == 0x7fffffff;
        const float tv = val[p];
        const int ti = idx[p];
        val[p] = gt ? cv : tv;
        idx[p] = gt ? ci : ti;
        cv = gt ? tv : cv;
        ci = gt ? ti : ci;
      }
    }
  }
#pragma unroll
  for (int p = 0; p < kMaxTopK; ++p)
    if (p < K) topk[t * K + p] = idx[p];
  if (bad) atomicOr(status, kStatusNonfinite);
}

void launch_route(const float* logits, const CollectPlan& p, hipStream_t s) {
  const unsigned grid = (unsigned)((p.n_tokens + 255) / 256);
  hipLaunchKernelGGL(route_kernel, dim3(grid), dim3(256), 0, s, logits, p.n_tokens, p.E, p.K,
                     p.topk, p.status);
}

// ------------------------------------------------------------------ bucketing
// A workgroup owns kBucketTokens consecutive tokens as 16 groups of 64.  For
// each (group, expert) a 64-bit mask records which tokens of the group chose
// the expert; popcounts of the masks give per-workgroup counts, and the rank of
// a token inside its expert list is a popcount of the lower mask bits plus the
// counts of the earlier groups -- no ordering atomics, so the lists come out
// sorted by token and identical on every run.

__device__ __forceinline__ void build_masks(const int32_t* __restrict__ topk, int64_t n, int K,
                                            int E, unsigned long long* mask) {
  for (int i = threadIdx.x; i < 16 * E; i += 256) mask[i] = 0ull;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t base = (int64_t)blockIdx.x * kBucketTokens;
  for (int g = wave; g < 16; g += 4) {
    const int64_t t = base + g * 64 + lane;
    if (t < n) {
      for (int k = 0; k < K; ++k) {
        const int e = topk[t * K + k];
        atomicOr(&mask[g * E + e], 1ull << lane);
      }
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void bucket_count_kernel(const int32_t* __restrict__ topk,
                                                           int64_t n, int K, int E,
                                                           int32_t* __restrict__ blockcounts) {
  __shared__ unsigned long long mask[16 * kMaxExperts];
  build_masks(topk, n, K, E, mask);
  for (int e = threadIdx.x; e < E; e += 256) {
    int c = 0;
#pragma unroll
    for (int g = 0; g < 16; ++g) c += __popcll(mask[g * E + e]);
    blockcounts[(int64_t)blockIdx.x * E + e] = c;
  }
}

// Gram-sum plan of `slots` slots whose token counts are in cnt[] (LDS, complete
// before the call; every thread of the workgroup calls this): padded counts,
// padded slot offsets, the longest-first slot order, the layer's running token
// counts, and the per-XCD Gram-sum work lists.  A segment is a token range of
// one slot; every item of a segment reads the same activations, so a segment
// stays on one XCD and its items are consecutive in the list.  Slots far
// longer than the average XCD share are split into up to 8 token ranges (the
// parts after the first go to partial buffers, added back in part order
// afterwards).  Longest slots first, each segment onto the least-loaded XCD.
struct PlanLds {
  int64_t padc[kMaxSlots];
  int32_t order[kMaxSlots];
  int32_t seg_x[kMaxSegs];      // XCD of each segment
  int32_t seg_pos[kMaxSegs];    // first list position of its items
  int32_t nseg;
};

__device__ void plan_gram(const int64_t* cnt, PlanLds& L, int slots, int64_t* __restrict__ pad_off,
                          int32_t* __restrict__ slot_order, int64_t* __restrict__ layer_counts, int overwrite,
                          int items, int32_t* __restrict__ work, int32_t* __restrict__ work_len,
                          int32_t* __restrict__ work_next, int32_t* __restrict__ seg, int32_t* __restrict__ split) {
  for (int e = threadIdx.x; e < slots; e += blockDim.x) {
    L.padc[e] = (cnt[e] + kTokPad - 1) / kTokPad * kTokPad;
    if (layer_counts) layer_counts[e] = overwrite ? cnt[e] : layer_counts[e] + cnt[e];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t po = 0;
    for (int e = 0; e < slots; ++e) {
      pad_off[e] = po;
      po += L.padc[e];
    }
    pad_off[slots] = po;
  }
  // rank of each slot by (padded length descending, slot ascending)
  for (int e = threadIdx.x; e < slots; e += blockDim.x) {
    int r = 0;
    for (int o = 0; o < slots; ++o) r += (L.padc[o] > L.padc[e]) || (L.padc[o] == L.padc[e] && o < e);
    slot_order[r] = e;
    L.order[r] = e;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t total = 0;
    for (int e = 0; e < slots; ++e) total += L.padc[e];
    // segment target length in 64-token chunks; the splitting below runs in
    // 32-bit chunk counts (64-bit division is a long instruction sequence)
    const int target = (int)((total / (8 * kXcds)) / kTokPad + 1);
    int64_t load[kXcds];
    int32_t len[kXcds];
    for (int x = 0; x < kXcds; ++x) {
      load[x] = 0;
      len[x] = 0;
    }
    int nseg = 0, nsplit = 0, used = 0;
    for (int r = 0; r < slots; ++r) {
      const int e = L.order[r];
      const int chunks = (int)(L.padc[e] / kTokPad);
      if (chunks == 0) continue;
      int k = (chunks + target - 1) / target;
      k = k < kXcds ? k : kXcds;
      k = k < 1 + kMaxPartials - used ? k : 1 + kMaxPartials - used;
      k = k < chunks ? k : chunks;
      if (k > 1) {
        split[1 + 3 * nsplit] = e;
        split[2 + 3 * nsplit] = used;
        split[3 + 3 * nsplit] = (int32_t)(k - 1);
        ++nsplit;
      }
      const int per = chunks / k, rem = chunks - per * k;
      int b = 0;
      for (int j = 0; j < k; ++j) {
        const int nc = per + (j < rem ? 1 : 0);
        seg[4 * nseg] = e;
        seg[4 * nseg + 1] = j == 0 ? -1 : used + j - 1;
        seg[4 * nseg + 2] = (int32_t)(b * kTokPad);
        seg[4 * nseg + 3] = (int32_t)(nc * kTokPad);
        int best = 0;
        for (int x = 1; x < kXcds; ++x) best = load[x] < load[best] ? x : best;
        L.seg_x[nseg] = best;
        L.seg_pos[nseg] = len[best];
        len[best] += items;
        load[best] += nc;
        b += nc;
        ++nseg;
      }
      used += (int)k - 1;
    }
    split[0] = nsplit;
    L.nseg = nseg;
    for (int x = 0; x < kXcds; ++x) {
      work_len[x] = len[x];
      work_next[x] = 0;
    }
  }
  __syncthreads();
  const int cap = kMaxSegs * items;
  for (int it = threadIdx.x; it < L.nseg * items; it += blockDim.x) {
    const int sg = it / items, t = it - sg * items;
    work[L.seg_x[sg] * cap + L.seg_pos[sg] + t] = sg * 1024 + t;
  }
}

// One workgroup: per-expert exclusive scan over bucketing workgroups, expert
// offsets, then the Gram-sum plan of the layer's slots (routed experts, and the
// shared-expert slot with all tokens).
__global__ __launch_bounds__(256) void bucket_scan_kernel(
    const int32_t* __restrict__ blockcounts, int nblk, int64_t n, int E, int has_shared,
    int32_t* __restrict__ blockbase, int64_t* __restrict__ offsets, int64_t* __restrict__ pad_off,
    int32_t* __restrict__ slot_order, int64_t* __restrict__ layer_counts, int overwrite, int items,
    int32_t* __restrict__ work, int32_t* __restrict__ work_len, int32_t* __restrict__ work_next,
    int32_t* __restrict__ seg, int32_t* __restrict__ split) {
  __shared__ int64_t cnt[kMaxSlots];
  __shared__ PlanLds L;
  const int slots = E + has_shared;
  // 16 blocks' counts are loaded together, so a thread waits for memory once
  // per 16 blocks rather than once per block
  constexpr int kScanBatch = 16;
  for (int e = threadIdx.x; e < E; e += 256) {
    int64_t run = 0;
    for (int b0 = 0; b0 < nblk; b0 += kScanBatch) {
      int c[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j)
        c[j] = b0 + j < nblk ? blockcounts[(int64_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        if (b0 + j < nblk) blockbase[(int64_t)(b0 + j) * E + e] = (int32_t)run;
        run += c[j];
      }
    }
    cnt[e] = run;
  }
  if (threadIdx.x == 0 && has_shared) cnt[E] = n;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t o = 0;
    for (int e = 0; e < E; ++e) {
      offsets[e] = o;
      o += cnt[e];
    }
    offsets[E] = o;
  }
  plan_gram(cnt, L, slots, pad_off, slot_order, layer_counts, overwrite, items, work, work_len, work_next, seg,
            split);
}

// Plan of the down_proj inputs of one layer: slot e < E takes expert e's routed
// tokens (offsets of the layer's routing), every slot from E on (one per shared
// expert) all n tokens; then the Gram-sum plan, and the grouped GEMM's tile
// offsets: ceil(padded count / 128) token tiles per slot.
__global__ __launch_bounds__(256) void down_scan_kernel(
    const int64_t* __restrict__ routed_offsets, int64_t n, int E, int slots, int64_t* __restrict__ pad_off,
    int32_t* __restrict__ slot_order, int64_t* __restrict__ layer_counts, int overwrite, int items,
    int32_t* __restrict__ work, int32_t* __restrict__ work_len, int32_t* __restrict__ work_next,
    int32_t* __restrict__ seg, int32_t* __restrict__ split, int32_t* __restrict__ tile_off) {
  __shared__ int64_t cnt[kMaxSlots];
  __shared__ PlanLds L;
  for (int e = threadIdx.x; e < slots; e += 256)
    cnt[e] = e < E ? routed_offsets[e + 1] - routed_offsets[e] : n;
  __syncthreads();
  plan_gram(cnt, L, slots, pad_off, slot_order, layer_counts, overwrite, items, work, work_len, work_next, seg,
            split);
  if (threadIdx.x == 0) {
    int32_t t = 0;
    for (int e = 0; e < slots; ++e) {
      tile_off[e] = t;
      t += (int32_t)((L.padc[e] + 127) / 128);
    }
    tile_off[slots] = t;
  }
}

void launch_down_scan(const int64_t* routed_offsets, int64_t n, int E, const CollectPlan& p,
                      int64_t* layer_counts, int32_t* tile_off, hipStream_t s) {
  hipLaunchKernelGGL(down_scan_kernel, dim3(1), dim3(256), 0, s, routed_offsets, n, E, p.E, p.pad_off,
                     p.slot_order, layer_counts, p.overwrite, p.syrk_items, p.work, p.work_len, p.work_next,
                     p.seg, p.split, tile_off);
}

__global__ __launch_bounds__(256) void bucket_scatter_kernel(
    const int32_t* __restrict__ topk, int64_t n, int K, int E,
    const int32_t* __restrict__ blockbase, const int64_t* __restrict__ offsets,
    int32_t* __restrict__ token_ids) {
  __shared__ unsigned long long mask[16 * kMaxExperts];
  __shared__ int32_t pre[16 * kMaxExperts];
  build_masks(topk, n, K, E, mask);
  for (int e = threadIdx.x; e < E; e += 256) {
    int run = blockbase[(int64_t)blockIdx.x * E + e];
    for (int g = 0; g < 16; ++g) {
      pre[g * E + e] = run;
      run += __popcll(mask[g * E + e]);
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t base = (int64_t)blockIdx.x * kBucketTokens;
  for (int g = wave; g < 16; g += 4) {
    const int64_t t = base + g * 64 + lane;
    if (t < n) {
      for (int k = 0; k < K; ++k) {
        const int e = topk[t * K + k];
        const int r = pre[g * E + e] + __popcll(mask[g * E + e] & below);
        token_ids[offsets[e] + r] = (int32_t)t;
      }
    }
  }
}

__global__ void zero_counts_kernel(int64_t* __restrict__ counts, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) counts[i] = 0;
}

// A fill kernel rather than a memset, so that the reset can be captured in a graph.
void launch_zero_counts(int64_t* counts, int n, hipStream_t s) {
  hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(256), 0, s, counts, n);
}

void launch_bucket(const CollectPlan& p, int64_t* layer_counts, hipStream_t s) {
  hipLaunchKernelGGL(bucket_count_kernel, dim3(p.nblk), dim3(256), 0, s, p.topk, p.n_tokens, p.K,
                     p.E, p.blockcounts);
  hipLaunchKernelGGL(bucket_scan_kernel, dim3(1), dim3(256), 0, s, p.blockcounts, p.nblk,
                     p.n_tokens, p.E, p.has_shared, p.blockbase, p.offsets, p.pad_off,
                     p.slot_order, layer_counts, p.overwrite, p.syrk_items, p.work, p.work_len, p.work_next,
                     p.seg, p.split);
  hipLaunchKernelGGL(bucket_scatter_kernel, dim3(p.nblk), dim3(256), 0, s, p.topk, p.n_tokens,
                     p.K, p.E, p.blockbase, p.offsets, p.token_ids);
}

// ------------------------------------------------------------------ gather
// One workgroup of 128 threads moves a 64-token x 128-feature tile, i.e. two
// 32-token blocks of 128 features, each 8 KB contiguous in xgT.  Thread
// (q, fc) = (tid / 16, tid % 16) reads 8 token rows x 8 features (16 B per row,
// 256 B contiguous per row across the 16 threads of a token group), transposes
// the 8x8 bf16 block in registers and puts each feature's 8 tokens (16 B) into
// an LDS copy of the two blocks; the workgroup then writes the blocks out in
// order, 16 B per thread, so each wave stores 1 KB contiguous.  In LDS a
// feature row is 64 B with 16 B of padding after every 8 features, which keeps
// both the transposed writes and the in-order reads free of bank conflicts.
// Tiles past the last slot exit at once.

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

constexpr int kGatherBlk = 128 * 64 + 16 * 16;   // LDS bytes of one 32-token block of 128 features

// LDS byte offset of the 16 B holding tokens 8*qq .. 8*qq+7 of feature f in block b.
__device__ __forceinline__ int gather_lds_off(int b, int f, int qq) {
  return b * kGatherBlk + f * 64 + (f >> 3) * 16 + qq * 16;
}

__global__ __launch_bounds__(128) void gather_kernel(
    const uint16_t* __restrict__ x, int64_t n, int d, int E, int has_shared,
    const int64_t* __restrict__ offsets, const int64_t* __restrict__ pad_off,
    const int32_t* __restrict__ token_ids, uint16_t* __restrict__ xgT) {
  __shared__ __attribute__((aligned(16))) char tile[2 * kGatherBlk];
  const int slots = E + has_shared;
  const int64_t p0 = (int64_t)blockIdx.x * kTokPad;
  const int64_t total = pad_off[slots];
  if (p0 >= total) return;
  int lo = 0, hi = slots;  // pad_off[lo] <= p0 < pad_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pad_off[mid] <= p0) lo = mid; else hi = mid;
  }
  const int s = lo;
  const int64_t i0 = p0 - pad_off[s];    // a multiple of 64
  const bool routed = s < E;
  const int64_t cnt = routed ? offsets[s + 1] - offsets[s] : n;
  const int32_t* ids = token_ids + (routed ? offsets[s] : 0);
  const int q = threadIdx.x >> 4;        // token group of 8 (0..7)
  const int fc = threadIdx.x & 15;       // feature group of 8 (0..15)
  const int fbase = blockIdx.y * 128;

  uint4 in[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t i = i0 + q * 8 + u;
    in[u] = make_uint4(0, 0, 0, 0);
    if (i < cnt) {
      const int64_t tok = routed ? (int64_t)ids[i] : i;
      in[u] = *reinterpret_cast<const uint4*>(x + tok * d + fbase + fc * 8);
    }
  }
#pragma unroll
  for (int fp = 0; fp < 4; ++fp) {       // feature pair (2fp, 2fp+1) inside the 8
    uint32_t a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = (&in[u].x)[fp];
    uint4 e, o;
    e.x = lo_pair(a[0], a[1]); e.y = lo_pair(a[2], a[3]);
    e.z = lo_pair(a[4], a[5]); e.w = lo_pair(a[6], a[7]);
    o.x = hi_pair(a[0], a[1]); o.y = hi_pair(a[2], a[3]);
    o.z = hi_pair(a[4], a[5]); o.w = hi_pair(a[6], a[7]);
    *reinterpret_cast<uint4*>(tile + gather_lds_off(q >> 2, fc * 8 + 2 * fp, q & 3)) = e;
    *reinterpret_cast<uint4*>(tile + gather_lds_off(q >> 2, fc * 8 + 2 * fp + 1, q & 3)) = o;
  }
  __syncthreads();
  // block b of the tile is 32-token block i0/32 + b of the slot: 128 features x 64 B
  uint16_t* out = xgT + pad_off[s] * d + (i0 >> 5) * ((int64_t)d * 32) + (int64_t)fbase * 32;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int c = r * 128 + threadIdx.x;   // 16-byte chunk of the tile in output order
    const int b = c >> 9, w = c & 511;
    const uint4 v = *reinterpret_cast<const uint4*>(tile + gather_lds_off(b, w >> 2, w & 3));
    *reinterpret_cast<uint4*>(out + (int64_t)b * d * 32 + w * 8) = v;
  }
}

void launch_gather(const uint16_t* x, const CollectPlan& p, hipStream_t s) {
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)p.xg_tiles, p.d / 128), dim3(128), 0, s, x,
                     p.n_tokens, p.d, p.E, p.has_shared, p.offsets, p.pad_off, p.token_ids,
                     p.xgT);
}

}  // namespace clha
