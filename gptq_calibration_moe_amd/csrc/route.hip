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
//   tilebase    int32 [ceil(N/256)][E] rank in expert e's list of the first
//                                   token of each 256-token gather tile
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
                                                    int* __restrict__ status, int layer) {
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
  if (bad) {
    atomicOr(status, kStatusNonfinite);
    // the first collection with a non-finite logit names its layer
    atomicCAS(reinterpret_cast<unsigned long long*>(status + kStatusLayer), 0ull,
              (1ull << 32) | (unsigned long long)(uint32_t)layer);
  }
}

void launch_route(const float* logits, const CollectPlan& p, hipStream_t s) {
  const unsigned grid = (unsigned)((p.n_tokens + 255) / 256);
  hipLaunchKernelGGL(route_kernel, dim3(grid), dim3(256), 0, s, logits, p.n_tokens, p.E, p.K,
                     p.topk, p.status, p.layer);
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
                          int max_partials) {
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
      const int chunks = (int)(L.padc[e] / kTokPad);
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
__global__ __launch_bounds__(256) void bucket_scan_kernel(
    const int32_t* __restrict__ blockcounts, int nblk, int64_t n, int E, int has_shared,
    int32_t* __restrict__ blockbase, int64_t* __restrict__ offsets, int64_t* __restrict__ pad_off,
    int32_t* __restrict__ slot_order, int64_t* __restrict__ layer_counts, int overwrite, int items,
    int32_t* __restrict__ work, int32_t* __restrict__ work_len, int32_t* __restrict__ work_next,
    int32_t* __restrict__ seg, int32_t* __restrict__ split, int max_partials) {
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
            split, max_partials);
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
            split, max_partials);
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

// Also the rank, in each expert's list, of the first token of every gather
// tile (kGatherTok tokens: every fourth 64-token group) for the gather.
__global__ __launch_bounds__(256) void bucket_scatter_kernel(
    const int32_t* __restrict__ topk, int64_t n, int K, int E,
    const int32_t* __restrict__ blockbase, const int64_t* __restrict__ offsets,
    int32_t* __restrict__ token_ids, int32_t* __restrict__ tilebase, int ntile) {
  __shared__ unsigned long long mask[16 * kMaxExperts];
  __shared__ int32_t pre[16 * kMaxExperts];
  constexpr int kGroupsPerTile = kGatherTok / 64;
  build_masks(topk, n, K, E, mask);
  for (int e = threadIdx.x; e < E; e += 256) {
    int run = blockbase[(int64_t)blockIdx.x * E + e];
    for (int g = 0; g < 16; ++g) {
      if (g % kGroupsPerTile == 0) {
        const int64_t tl = (int64_t)blockIdx.x * (kBucketTokens / kGatherTok) + g / kGroupsPerTile;
        if (tl < ntile) tilebase[tl * E + e] = run;
      }
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
                     p.seg, p.split, p.max_partials);
  hipLaunchKernelGGL(bucket_scatter_kernel, dim3(p.nblk), dim3(256), 0, s, p.topk, p.n_tokens,
                     p.K, p.E, p.blockbase, p.offsets, p.token_ids, p.tilebase, p.ntile);
}

// ------------------------------------------------------------------ gather
// Token-major: each activation row is read from memory once.  A workgroup of
// 512 threads takes a tile of kGatherTok consecutive tokens and a slice of
// kGatherFeat features: it reads the slice of the tile's rows (256 B of each
// row, 16 B per thread) into LDS, then writes that slice of every slot's rows
// for those tokens.  Expert lists are sorted by token, so a tile's tokens form
// one run [lo, hi) of each slot's positions; the bucketing gives lo and hi
// (tilebase), and the shared slot's run is the tile itself.  Output is written
// in 16-byte chunks, 8 consecutive positions of one feature, and every chunk
// belongs to exactly one tile: the one holding its first position.  A tile
// therefore writes the chunks that start in its run; the last of them may
// reach past the run, and those few positions (at most 7 per slot) are read
// straight from the activations through their token ids.  The tile that holds
// a slot's last position also writes the slot's padding chunks as zeros.  A
// wave takes one 32-token block at a time: lane (q, g) reads the 16-byte
// pieces (features 8g .. 8g+7) of chunk q's 8 positions, transposes the 8x8
// block in registers and stores 8 chunks, so each store instruction of the
// wave writes 16 whole 64-byte feature rows where the block lies inside the
// run.  Workgroups are dealt to the dies as contiguous runs of tiles taken
// slice by slice, so the two tiles that share a 64-byte row run on one die at
// the same time and its halves meet in that die's L2.

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

constexpr int kGatherFeat = 128;                    // features per gather tile
constexpr int kGatherPitch = 2 * kGatherFeat + 16;  // LDS bytes per token row (16 B of padding)
constexpr int kGatherThreads = 512;
constexpr int kHalo = 7;                            // most positions of a chunk past the run
constexpr uint16_t kFromHalo = 0x8000;              // entry: position past the run (halo index below)
constexpr uint16_t kZeroPos = 0xffff;               // entry: padding position

template <int SCAP, int KCAP>
__global__ __launch_bounds__(kGatherThreads) void gather_kernel(
    const uint16_t* __restrict__ x, int64_t n, int d, int E, int has_shared,
    const int64_t* __restrict__ offsets, const int64_t* __restrict__ pad_off,
    const int32_t* __restrict__ token_ids, const int32_t* __restrict__ tilebase, int ntile, int tpx,
    uint16_t* __restrict__ xgT) {
  __shared__ __attribute__((aligned(16))) char xt[kGatherTok * kGatherPitch];
  // per slot: data run [lo, hi), position count, owned chunks [c0, c1), and
  // exclusive prefixes of the blocks written and of the position entries
  __shared__ int s_lo[SCAP], s_hi[SCAP], s_cnt[SCAP], s_c0[SCAP], s_c1[SCAP], s_pblk[SCAP + 1],
      s_ppos[SCAP + 1];
  __shared__ int s_halo[SCAP * kHalo];   // token ids of the positions hi .. hi + 6 (routed slots)
  // one entry per position of a routed slot's owned chunks up to hi rounded up
  // to 8 (at most hi - lo + 14 per slot): the local token index, or a halo
  // index | kFromHalo, or kZeroPos; slot s's entries start at s_ppos[s] with
  // position 8 c0, so every chunk's entries are one aligned 16-byte read
  __shared__ __attribute__((aligned(16))) uint16_t ent[kGatherTok * KCAP + 16 * SCAP];
  const int slots = E + has_shared;
  const int xcd = (int)(blockIdx.x % kXcds), j = (int)(blockIdx.x / kXcds);
  const int slice = j / tpx, tile = xcd * tpx + j % tpx;
  if (tile >= ntile) return;
  const int64_t t0 = (int64_t)tile * kGatherTok;
  const int nt = (int)(n - t0 < kGatherTok ? n - t0 : kGatherTok);
  const int fbase = slice * kGatherFeat;
  const int tid = threadIdx.x;

  // the tile's slice: kGatherTok rows x 16 chunks of 16 B
  constexpr int kLoads = kGatherTok * 16 / kGatherThreads;
  uint4 v[kLoads];
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int ch = u * kGatherThreads + tid, r = ch >> 4, c = ch & 15;
    v[u] = make_uint4(0u, 0u, 0u, 0u);
    if (r < nt) v[u] = *reinterpret_cast<const uint4*>(x + (t0 + r) * d + fbase + 8 * c);
  }

  for (int s = tid; s < slots; s += kGatherThreads) {
    int lo, hi, cnt;
    if (s < E) {
      cnt = (int)(offsets[s + 1] - offsets[s]);
      lo = tilebase[(int64_t)tile * E + s];
      hi = tile + 1 < ntile ? tilebase[(int64_t)(tile + 1) * E + s] : cnt;
    } else {
      cnt = (int)n;
      lo = (int)t0;
      hi = (int)t0 + nt;
    }
    const int c0 = (lo + 7) >> 3;
    int c1 = lo < hi ? ((hi - 1) >> 3) + 1 : c0;
    if (lo < hi && hi == cnt) c1 = (int)((pad_off[s + 1] - pad_off[s]) >> 3);   // the slot's last tile
    if (c1 < c0) c1 = c0;
    s_lo[s] = lo;
    s_hi[s] = hi;
    s_cnt[s] = cnt;
    s_c0[s] = c0;
    s_c1[s] = c1;
    s_pblk[s] = c0 < c1 ? ((c1 - 1) >> 2) - (c0 >> 2) + 1 : 0;
    s_ppos[s] = (s < E && c0 < c1 && hi > 8 * c0) ? ((hi + 7) & ~7) - 8 * c0 : 0;
    if (s < E)
      for (int u = 0; u < kHalo; ++u)
        s_halo[s * kHalo + u] = (c0 < c1 && hi + u < cnt && hi + u < 8 * c1) ? token_ids[offsets[s] + hi + u] : 0;
  }
  __syncthreads();
  if (tid < 64) {
    // exclusive prefix sums over the slots: lane l takes `per` consecutive slots
    const int per = (slots + 63) / 64, s0 = tid * per;
    int sb = 0, sp = 0;
    for (int k = 0; k < per; ++k)
      if (s0 + k < slots) {
        sb += s_pblk[s0 + k];
        sp += s_ppos[s0 + k];
      }
    int ib = sb, ip = sp;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int ob = __shfl_up(ib, off), op = __shfl_up(ip, off);
      if (tid >= off) {
        ib += ob;
        ip += op;
      }
    }
    int eb = ib - sb, ep = ip - sp;
    for (int k = 0; k < per; ++k)
      if (s0 + k < slots) {
        const int b = s_pblk[s0 + k], q = s_ppos[s0 + k];
        s_pblk[s0 + k] = eb;
        s_ppos[s0 + k] = ep;
        eb += b;
        ep += q;
      }
    if (tid == 63) {
      s_pblk[slots] = ib;
      s_ppos[slots] = ip;
    }
  }
  __syncthreads();
  // position entries of the routed slots
  const int ntot = s_ppos[slots];
  for (int i = tid; i < ntot; i += kGatherThreads) {
    int a = 0, b = slots;   // s_ppos[a] <= i < s_ppos[b]
    while (b - a > 1) {
      const int m = (a + b) >> 1;
      if (s_ppos[m] <= i) a = m; else b = m;
    }
    const int p = 8 * s_c0[a] + (i - s_ppos[a]);
    uint16_t e = kZeroPos;
    if (p < s_hi[a]) e = (uint16_t)(token_ids[offsets[a] + p] - t0);
    else if (p < s_cnt[a]) e = (uint16_t)(kFromHalo | (p - s_hi[a]));
    ent[i] = e;
  }
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int ch = u * kGatherThreads + tid, r = ch >> 4, c = ch & 15;
    *reinterpret_cast<uint4*>(xt + r * kGatherPitch + 16 * c) = v[u];
  }
  __syncthreads();

  // wave w writes blocks w, w + 8, ... of the list (slot-major).  Lane
  // (q, g) = (lane % 4, lane / 4) takes chunk q of the block for features
  // 8g .. 8g+7: it reads the 8 positions' 16-byte pieces of those features (from
  // the LDS tile, or from memory for positions past the run), transposes the
  // 8x8 block in registers and stores 8 chunks; for each of them the wave
  // writes 16 feature rows of 64 B.
  const int lane = tid & 63, wv = tid >> 6;
  const int q = lane & 3, g = lane >> 2;
  const int nb = s_pblk[slots];
  for (int bi = wv; bi < nb; bi += kGatherThreads / 64) {
    int s = 0, b = slots;   // s_pblk[s] <= bi < s_pblk[b]
    while (b - s > 1) {
      const int m = (s + b) >> 1;
      if (s_pblk[m] <= bi) s = m; else b = m;
    }
    const int hi = s_hi[s], c0 = s_c0[s], c1 = s_c1[s];
    const int blk = (c0 >> 2) + (bi - s_pblk[s]);
    const int chunk = 4 * blk + q;
    if (chunk < c0 || chunk >= c1) continue;
    const int p0 = 8 * chunk;
    uint4 rv[8];
    if (s < E) {
      const int pend = 8 * c0 + (s_ppos[s + 1] - s_ppos[s]);   // entries cover positions [8 c0, pend)
      uint4 w = make_uint4(0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu);
      if (p0 < pend) w = *reinterpret_cast<const uint4*>(ent + s_ppos[s] + (p0 - 8 * c0));
      const int* halo = s_halo + s * kHalo;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t e = ((&w.x)[u >> 1] >> (16 * (u & 1))) & 0xffffu;
        rv[u] = make_uint4(0u, 0u, 0u, 0u);
        if (e < kFromHalo)
          rv[u] = *reinterpret_cast<const uint4*>(xt + e * kGatherPitch + 16 * g);
        else if (e != kZeroPos)
          rv[u] = *reinterpret_cast<const uint4*>(x + (int64_t)halo[e & 7] * d + fbase + 8 * g);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int p = p0 + u;
        rv[u] = make_uint4(0u, 0u, 0u, 0u);
        if (p < hi) rv[u] = *reinterpret_cast<const uint4*>(xt + (p - (int)t0) * kGatherPitch + 16 * g);
      }
    }
    uint16_t* dst = xgT + (pad_off[s] + 32 * (int64_t)blk) * d + (int64_t)(fbase + 8 * g) * 32 + 8 * q;
#pragma unroll
    for (int fp = 0; fp < 4; ++fp) {       // feature pair (2fp, 2fp+1) of the group
      uint32_t a[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] = (&rv[u].x)[fp];
      *reinterpret_cast<uint4*>(dst + (2 * fp) * 32) =
          make_uint4(lo_pair(a[0], a[1]), lo_pair(a[2], a[3]), lo_pair(a[4], a[5]), lo_pair(a[6], a[7]));
      *reinterpret_cast<uint4*>(dst + (2 * fp + 1) * 32) =
          make_uint4(hi_pair(a[0], a[1]), hi_pair(a[2], a[3]), hi_pair(a[4], a[5]), hi_pair(a[6], a[7]));
    }
  }
}

void launch_gather(const uint16_t* x, const CollectPlan& p, hipStream_t s) {
  const int tpx = (p.ntile + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(kXcds * tpx * (p.d / kGatherFeat)));
  // the common shapes (up to 64 routed experts + 1 shared, top-8) get the small
  // LDS tables, so two workgroups fit on a CU
  if (p.E + p.has_shared <= 65 && p.K <= 8)
    hipLaunchKernelGGL((gather_kernel<65, 8>), grid, dim3(kGatherThreads), 0, s, x, p.n_tokens, p.d, p.E,
                       p.has_shared, p.offsets, p.pad_off, p.token_ids, p.tilebase, p.ntile, tpx, p.xgT);
  else
    hipLaunchKernelGGL((gather_kernel<kMaxSlots, kMaxTopK>), grid, dim3(kGatherThreads), 0, s, x, p.n_tokens,
                       p.d, p.E, p.has_shared, p.offsets, p.pad_off, p.token_ids, p.tilebase, p.ntile, tpx,
                       p.xgT);
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
