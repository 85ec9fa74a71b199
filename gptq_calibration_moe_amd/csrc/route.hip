// Collection phase, first half: top-K routing, per-expert bucketing and the
// Gram-sum plan.
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
//   iota        int32 [N]           0 .. N-1, the shared slot's token list
//   zero_row    bf16  [d]           zeros, the Gram sums' operand at padding positions
//   pad_off     int64 [slots+1]     padded start of each slot's positions (each
//                                   slot padded to a multiple of 64 tokens; slot E,
//                                   if the block has shared experts, holds all N
//                                   tokens in order), the Gram-sum segments and the
//                                   per-XCD work lists
// The Gram sums read each slot's rows of x straight through its token list.
#include "kernels.h"

namespace clha {

// ------------------------------------------------------------------ routing

// Also writes iota[t] = t, the shared slot's token list for the Gram sums.
// KC >= K is the list length the insertion runs over (a compile-time bound, so
// the list stays in registers with no per-entry test of K); VEC reads the row
// 16 bytes at a time (E a multiple of 4 and the logits 16-byte aligned).
template <int KC, bool VEC>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int64_t n,
                                                    int E, int K, int32_t* __restrict__ topk,
                                                    int* __restrict__ status, int layer,
                                                    int32_t* __restrict__ iota) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  iota[t] = (int32_t)t;
  const float* row = logits + t * E;
  float val[KC];
  int idx[KC];
#pragma unroll
  for (int p = 0; p < KC; ++p) {
    val[p] = -INFINITY;
    idx[p] = 0x7fffffff;
  }
  bool bad = false;
  // insertion into the list ordered by (logit descending, index ascending);
  // an element pushed down keeps moving past entries it precedes, so equal
  // logits always end up in index order.  Entries past K only ever hold
  // elements pushed out of the first K, so the first K are the top K.
  auto insert = [&](float cv, int ci) {
    bad |= !isfinite(cv);
#pragma unroll
    for (int p = 0; p < KC; ++p) {
      const bool gt = cv > val[p] || (cv == val[p] && ci < idx[p]) || idx[p] == 0x7fffffff;
      const float tv = val[p];
      const int ti = idx[p];
      val[p] = gt ? cv : tv;
      idx[p] = gt ? ci : ti;
      cv = gt ? tv : cv;
      ci = gt ? ti : ci;
    }
  };
  if constexpr (VEC) {
    for (int e = 0; e < E; e += 4) {
      const float4 q = *reinterpret_cast<const float4*>(row + e);
      insert(q.x, e);
      insert(q.y, e + 1);
      insert(q.z, e + 2);
      insert(q.w, e + 3);
    }
  } else {
    for (int e = 0; e < E; ++e) insert(row[e], e);
  }
#pragma unroll
  for (int p = 0; p < KC; ++p)
    if (p < K) topk[t * K + p] = idx[p];
  if (bad) {
    atomicOr(status, kStatusNonfinite);
    // the first collection with a non-finite logit names its layer
    atomicCAS(reinterpret_cast<unsigned long long*>(status + kStatusLayer), 0ull,
              (1ull << 32) | (unsigned long long)(uint32_t)layer);
  }
}

template <int KC>
static void launch_route_k(const float* logits, const CollectPlan& p, hipStream_t s) {
  const unsigned grid = (unsigned)((p.n_tokens + 255) / 256);
  if (p.E % 4 == 0 && reinterpret_cast<uintptr_t>(logits) % 16 == 0)
    hipLaunchKernelGGL((route_kernel<KC, true>), dim3(grid), dim3(256), 0, s, logits, p.n_tokens, p.E, p.K,
                       p.topk, p.status, p.layer, p.iota);
  else
    hipLaunchKernelGGL((route_kernel<KC, false>), dim3(grid), dim3(256), 0, s, logits, p.n_tokens, p.E, p.K,
                       p.topk, p.status, p.layer, p.iota);
}

void launch_route(const float* logits, const CollectPlan& p, hipStream_t s) {
  if (p.K <= 2) launch_route_k<2>(logits, p, s);
  else if (p.K <= 4) launch_route_k<4>(logits, p, s);
  else if (p.K <= 8) launch_route_k<8>(logits, p, s);
  else launch_route_k<kMaxTopK>(logits, p, s);
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
// stays on one XCD and its items are consecutive in the list, the diagonal
// pairs (the longest items) first.  Segments are at most kSegTokens long: the
// workgroups of a die then start each segment's items together and run them
// side by side, so the activation panels they all read stay in the die's L2
// (over a long token range the items would drift apart and each fetch its
// panels again).  The parts of a slot after its first go to partial buffers,
// added into S in part order afterwards; when the buffers run short the
// segments grow.  Longest slots first, each segment onto the least-loaded XCD.
// Slot `derived` (or none, -1) keeps its counts but gets no Gram-sum items.
struct PlanLds {
  int64_t padc[kMaxSlots];
  int32_t order[kMaxSlots];
  int32_t seg_x[kMaxSegsCap];   // XCD of each segment
  int32_t seg_pos[kMaxSegsCap]; // first list position of its items
  int32_t nseg;
};

__device__ void plan_gram(const int64_t* cnt, PlanLds& L, int slots, int64_t* __restrict__ pad_off,
                          int32_t* __restrict__ slot_order, int64_t* __restrict__ layer_counts, int overwrite,
                          int items, int32_t* __restrict__ work, int32_t* __restrict__ work_len,
                          int32_t* __restrict__ work_next, int32_t* __restrict__ seg, int32_t* __restrict__ split,
                          int max_partials, int derived) {
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
    for (int e = 0; e < slots; ++e) total += e == derived ? 0 : L.padc[e];
    // In 64-token chunks (32-bit counts: 64-bit division is a long instruction
    // sequence).  The slots, longest first, are laid end to end and cut into
    // kXcds runs of per_x chunks, one run per die, so every die gets the same
    // work whatever the load shape; each run is cut further into segments of at
    // most seg_max chunks (kSegTokens, longer only when the partial buffers
    // would run short: every segment of a slot after its first takes one).
    const int total_chunks = (int)(total / kTokPad);
    const int per_x = (total_chunks + kXcds - 1) / kXcds;
    const int spare = max_partials > kXcds ? max_partials - (kXcds - 1) : 1;
    int seg_max = kSegTokens / kTokPad;
    const int need = (total_chunks + spare - 1) / spare;
    seg_max = seg_max > need ? seg_max : need;
    int32_t len[kXcds];
    for (int x = 0; x < kXcds; ++x) len[x] = 0;
    int x = 0, xload = 0, nseg = 0, nsplit = 0, used = 0;
    for (int r = 0; r < slots; ++r) {
      const int e = L.order[r];
      const int chunks = e == derived ? 0 : (int)(L.padc[e] / kTokPad);
      if (chunks == 0) continue;
      const int first_part = used;
      int pos = 0, parts = 0;
      while (pos < chunks) {
        if (parts > 0 && used >= max_partials) {
          // no partial buffer left: the slot's last segment takes the rest
          seg[4 * (nseg - 1) + 3] += (int32_t)((chunks - pos) * kTokPad);
          xload += chunks - pos;
          break;
        }
        if (xload >= per_x && x < kXcds - 1) {
          ++x;
          xload = 0;
        }
        int n = chunks - pos;
        n = n < seg_max ? n : seg_max;
        if (x < kXcds - 1 && n > per_x - xload) n = per_x - xload;
        seg[4 * nseg] = e;
        seg[4 * nseg + 1] = parts == 0 ? -1 : used++;
        seg[4 * nseg + 2] = (int32_t)(pos * kTokPad);
        seg[4 * nseg + 3] = (int32_t)(n * kTokPad);
        L.seg_x[nseg] = x;
        L.seg_pos[nseg] = len[x];
        len[x] += items;
        xload += n;
        pos += n;
        ++parts;
        ++nseg;
      }
      if (parts > 1) {
        split[1 + 3 * nsplit] = e;
        split[2 + 3 * nsplit] = first_part;
        split[3 + 3 * nsplit] = parts - 1;
        ++nsplit;
      }
    }
    split[0] = nsplit;
    L.nseg = nseg;
    for (int x = 0; x < kXcds; ++x) {
      work_len[x] = len[x];
      work_next[x] = 0;
    }
  }
  __syncthreads();
  const int cap = (slots + max_partials) * items;
  for (int it = threadIdx.x; it < L.nseg * items; it += blockDim.x) {
    const int sg = it / items, t = it - sg * items;
    work[L.seg_x[sg] * cap + L.seg_pos[sg] + t] = sg * 1024 + t;
  }
}

// One workgroup: per-expert exclusive scan over bucketing workgroups, expert
// offsets, then the Gram-sum plan of the layer's slots (routed experts, and the
// shared-expert slot with all tokens).
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void bucket_scan_kernel(
    const int32_t* __restrict__ blockcounts, int nblk, int64_t n, int E, int has_shared,
    int32_t* __restrict__ blockbase, int64_t* __restrict__ offsets, int64_t* __restrict__ pad_off,
    int32_t* __restrict__ slot_order, int64_t* __restrict__ layer_counts, int overwrite, int items,
    int32_t* __restrict__ work, int32_t* __restrict__ work_len, int32_t* __restrict__ work_next,
    int32_t* __restrict__ seg, int32_t* __restrict__ split, int max_partials, uint16_t* __restrict__ zero_row,
    int d, int derived) {
  __shared__ int64_t cnt[kMaxSlots];
  __shared__ int64_t part[kScanThreads];
  __shared__ PlanLds L;
  const int slots = E + has_shared;
  // the Gram sums' operand for padding positions
  for (int f = threadIdx.x; f < d; f += blockDim.x) zero_row[f] = 0;
  // tpe threads per expert (a power of two, E * tpe <= the block), each over one
  // run of consecutive token blocks: the runs' sums, an exclusive scan over an
  // expert's runs, then each run's block bases.  16 blocks' counts are loaded
  // together, so a thread waits for memory once per 16 blocks.
  constexpr int kScanBatch = 16;
  int tpe = 1;
  while (tpe < 64 && 2 * tpe * E <= (int)blockDim.x) tpe *= 2;
  const bool mine = (int)threadIdx.x < E * tpe;
  const int e = threadIdx.x / tpe, t = threadIdx.x % tpe;
  const int run_len = (nblk + tpe - 1) / tpe;
  const int b_lo = min(t * run_len, nblk), b_hi = min(b_lo + run_len, nblk);
  int64_t sum = 0;
  if (mine) {
    for (int b0 = b_lo; b0 < b_hi; b0 += kScanBatch) {
      int c[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) c[j] = b0 + j < b_hi ? blockcounts[(int64_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) sum += c[j];
    }
  }
  part[threadIdx.x] = sum;
  __syncthreads();
  if (mine) {
    int64_t run = 0;
    for (int u = 0; u < t; ++u) run += part[e * tpe + u];
    if (t == tpe - 1) cnt[e] = run + sum;
    for (int b0 = b_lo; b0 < b_hi; b0 += kScanBatch) {
      int c[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) c[j] = b0 + j < b_hi ? blockcounts[(int64_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        if (b0 + j < b_hi) blockbase[(int64_t)(b0 + j) * E + e] = (int32_t)run;
        run += c[j];
      }
    }
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
            split, max_partials, derived);
}

// Plan of the down_proj inputs of one layer: slot e < E takes expert e's routed
// tokens (offsets of the layer's routing), every slot from E on (one per shared
// expert) all n tokens; then the Gram-sum plan, and the grouped GEMM's tile
// offsets: ceil(padded count / 128) token tiles per slot.
__global__ __launch_bounds__(256) void down_scan_kernel(
    const int64_t* __restrict__ routed_offsets, int64_t n, int E, int slots, int64_t* __restrict__ pad_off,
    int32_t* __restrict__ slot_order, int64_t* __restrict__ layer_counts, int overwrite, int items,
    int32_t* __restrict__ work, int32_t* __restrict__ work_len, int32_t* __restrict__ work_next,
    int32_t* __restrict__ seg, int32_t* __restrict__ split, int32_t* __restrict__ tile_off, int max_partials) {
  __shared__ int64_t cnt[kMaxSlots];
  __shared__ PlanLds L;
  for (int e = threadIdx.x; e < slots; e += 256)
    cnt[e] = e < E ? routed_offsets[e + 1] - routed_offsets[e] : n;
  __syncthreads();
  plan_gram(cnt, L, slots, pad_off, slot_order, layer_counts, overwrite, items, work, work_len, work_next, seg,
            split, max_partials, -1);
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
                     p.seg, p.split, tile_off, p.max_partials);
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
  hipLaunchKernelGGL(bucket_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, p.blockcounts, p.nblk,
                     p.n_tokens, p.E, p.has_shared, p.blockbase, p.offsets, p.pad_off,
                     p.slot_order, layer_counts, p.overwrite, p.syrk_items, p.work, p.work_len, p.work_next,
                     p.seg, p.split, p.max_partials, p.zero_row, p.d, p.derive_shared ? p.E : -1);
  hipLaunchKernelGGL(bucket_scatter_kernel, dim3(p.nblk), dim3(256), 0, s, p.topk, p.n_tokens,
                     p.K, p.E, p.blockbase, p.offsets, p.token_ids);
}

}  // namespace clha

namespace clha {
int max_partials(int d, int64_t max_tokens, int top_k, int slots) {
  // segments past each slot's first: at most rows / kSegTokens from the length
  // cap, plus one at each boundary between two dies' runs
  const int64_t rows = max_tokens * (top_k + 1) + (int64_t)kTokPad * slots;
  int64_t need = rows / kSegTokens + kXcds;
  const int64_t fit = ((int64_t)4 << 30) / ((int64_t)4 * d * d);
  need = need < fit ? need : fit;
  need = need < kMaxPartialsCap ? need : kMaxPartialsCap;
  return (int)(need > 8 ? need : 8);
}
}  // namespace clha
