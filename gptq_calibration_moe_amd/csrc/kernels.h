// Internal declarations shared by the C-ABI layer (api.cpp) and the HIP kernel
// sources.  Host-side launchers only; every launcher enqueues on `stream` and
// returns without synchronising.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace clha {

// ---------------------------------------------------------------- constants
constexpr int kBucketTokens = 1024;   // tokens per bucketing workgroup (16 groups of 64)
constexpr int kTokPad = 64;           // expert token lists are padded to this multiple
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 16;
constexpr int kMaxLayers = 8;
constexpr int kSyrkTile = 256;        // Gram-sum output tile
constexpr int kMaxPartialsCap = 512;  // most partial Gram-sum buffers of token-split slots
constexpr int kSegTokens = 16384;     // longest Gram-sum segment (one flush interval)
constexpr int kMaxSlots = kMaxExperts + 1;                // Hessian slots of one layer
constexpr int kMaxSegsCap = kMaxSlots + kMaxPartialsCap;  // most Gram-sum segments per call
// Partial buffers of a context: enough for every segment past each slot's first
// at max_tokens, at most 4 GiB of them (and at least 8).
int max_partials(int d, int64_t max_tokens, int top_k, int slots);
constexpr int kXcds = 8;              // accelerator complex dies; workgroup b runs on die b % 8
constexpr int kSyrkWgPerXcd = 32;     // persistent Gram-sum workgroups per die (one per CU)
constexpr int kNb = 64;               // Cholesky / triangular-inverse block
constexpr int kGptqRows = 64;         // rows per GPTQ workgroup
constexpr int kSuper = 256;           // GPTQ columns between trailing GEMM updates
constexpr int kGemmTile = 128;        // rows and columns of a trailing-update tile

// Status record of a context: 16 32-bit words of device memory (latched; see
// clha_sync), held in a file-scope device array so that no context allocates.
//   word 0       flag bits (kStatusNonfinite | kStatusNotPd)
//   word 1       0, or 0xffffffff - i for the lowest caller index i of a GPTQ job
//                whose Hessian failed (atomicMax keeps the lowest index)
//   word 2       the same for the lowest failing Hessian of the call
//   words 4, 5   0, or (1 << 32 | layer) of the first collection with a
//                non-finite router logit (the first writer wins)
constexpr int kStatusNonfinite = 1;
constexpr int kStatusNotPd = 2;
constexpr int kStatusWords = 16;
constexpr int kStatusJob = 1;
constexpr int kStatusMat = 2;
constexpr int kStatusLayer = 4;
constexpr int kMaxContexts = 1024;    // live contexts per device (status records)
// A free status record of `device` (the current device), cleared, and its slot;
// nullptr when all kMaxContexts records are taken or the lookup fails.
int* status_acquire(int device, int* slot);
void status_release(int device, int slot);
constexpr int kSlices = 6;            // signed 7-bit digits per sliced fp64 factor entry

// ---------------------------------------------------------------- collection
struct CollectPlan {
  int64_t n_tokens;
  int d, E, K, has_shared;
  int nblk;              // bucketing workgroups
  // device buffers (from the caller's workspace or outputs)
  int32_t* topk;         // [n][K]
  int32_t* blockcounts;  // [nblk][E]
  int32_t* blockbase;    // [nblk][E]
  int64_t* offsets;      // [E+1]
  int64_t* pad_off;      // [slots+1] padded starts of each slot's token list
  int32_t* slot_order;   // [slots] slots sorted by padded length, longest first
  int32_t* work;         // [kXcds][max_segs*items] Gram-sum items (segment*1024 + item) per XCD
  int32_t* work_len;     // [kXcds] items per XCD
  int32_t* work_next;    // [kXcds] queue heads (reset by the bucketing scan)
  int32_t* seg;          // [max_segs][4] slot, destination (-1: S, else partial buffer),
                         //   first token and token count within the slot's padded list
  int32_t* split;        // [1 + 3*max_partials] count, then (slot, first partial, partials)
  float* partials;       // [max_partials][d][d] partial sums of token-split slots
  int max_partials;      // partial buffers in the workspace
  int max_segs;          // slots + max_partials
  int syrk_items;        // Gram-sum items per segment
  int overwrite;         // first collection after a reset: S and counts are stored, not added
  int32_t* token_ids;    // [n*K]
  uint16_t* xgT;         // gathered activations: per slot, 32-token blocks of [d][32]
  // Gram sums straight from the activations (non-null): x [n][d], the shared
  // slot's token list 0 .. n-1 and d zero elements for padding positions
  const uint16_t* x_rows;
  int32_t* iota;
  uint16_t* zero_row;
  int* status;           // the context's status record
  int layer;             // the collected layer (named by a non-finite logit)
  // the shared slot's sums follow from the routed slots' (S_E = sum_e S_e / K):
  // it gets no Gram-sum items and is formed after the partial-sum reduce
  int derive_shared = 0;
};

void launch_route(const float* logits, const CollectPlan& p, hipStream_t s);
void launch_bucket(const CollectPlan& p, int64_t* layer_counts, hipStream_t s);
void launch_syrk(const CollectPlan& p, float* S, hipStream_t s);
// partial sums of token-split slots into S; with p.overwrite, slots without tokens zeroed
void launch_syrk_reduce(const CollectPlan& p, float* S, const int64_t* layer_counts, hipStream_t s);
// down_proj inputs: plan from a layer's routing, and the grouped SwiGLU GEMM
// writing each slot's h^T (in the gathered activations' 32-token blocks)
void launch_down_scan(const int64_t* routed_offsets, int64_t n, int E, const CollectPlan& p,
                      int64_t* layer_counts, int32_t* tile_off, hipStream_t s);
void launch_down_gemm(const uint16_t* x, int d_model, const int32_t* token_ids, const int64_t* routed_offsets,
                      int E, int64_t n, const uint16_t* const* wgu, const CollectPlan& p, const int32_t* tile_off,
                      int64_t max_tiles, hipStream_t s);
void launch_zero_counts(int64_t* counts, int n, hipStream_t s);
int syrk_items_per_slot(int d);

// ---------------------------------------------------------------- aggregation
struct AggArgs {
  const float* S[kMaxLayers];
  const int64_t* counts[kMaxLayers];
  float alpha[kMaxLayers];
  const float* alpha_slot;   // per-slot explicit weights, device [slots][n_layers] (mode 3)
  int n_layers;
  int mode;              // clha_alpha_mode
  int d;
  int slots;
};
void launch_aggregate(const AggArgs& a, float* H, float* alpha_out, hipStream_t s);

// ---------------------------------------------------------------- GPTQ
struct GJob {
  const void* W;
  uint8_t* codes;
  float* scales;
  uint8_t* zeros;
  float* loss;
  int64_t wf_off;        // offset of the job's fp32 working copy (elements)
  int32_t dtype;
  int32_t rows;
  int32_t bits;
  int32_t mat;           // index of the job's distinct Hessian
  int32_t slab_base;     // first global slab of this job
  int32_t n_slabs;
  int32_t tile_base;     // first global row tile (kGemmTile rows) of the trailing update
  int32_t n_tiles;
  int32_t user_index;    // the job's index in the caller's array
  int32_t* status;       // optional: the job's numerical status (clha_status code)
  uint8_t* dead_out;     // optional: dead-column flags of the job's Hessian, natural order
};

struct GptqPlan {
  int n_jobs, n_mats, cols, group, block, total_slabs, total_tiles;
  float damp;
  const GJob* jobs;          // device [n_jobs]
  const float* const* mats;  // device [n_mats] Hessian pointers
  double* A;                 // device [n_mats][cols][cols]  reversed damped H, then its Cholesky factor
  double* X;                 // device [n_mats][cols][cols]  inverse of that factor
  float* U;                  // device [n_mats][cols][cols]  upper factor of Hd^-1 (fp32)
  float* UT;                 // device [n_mats][cols][cols]  its transpose (may be null when only U is wanted)
  double* dinv;              // device [n_mats][cols/kNb][kNb][kNb] inverses of L's diagonal blocks
  uint8_t* dead;             // device [n_mats][cols]
  double* lamd;              // device [n_mats] damping lambda
  int* lexp;                 // device [n_mats][cols] row exponents of the sliced factor
  float* lam;                // device [n_mats] lambda as float (optional output, may be null)
  float* wf;                 // device fp32 working copies of all jobs' weights
  float* ebuf;               // device [padded rows][kSuper] a superblock's negated errors
  float* partials;           // device [total_slabs][2]
  int* status;               // the context's status record
  int* mstat;                // device [n_mats] status bits of each distinct Hessian's factor
  // GPTQ options (zero / null when off)
  int act_order;             // columns processed by decreasing H_ii
  int static_groups;         // grids fitted once per natural group before any update
  const float* const* src_mats;  // device [n_mats] the callers' Hessians (mats may point at hperm)
  float* hperm;              // device [n_mats][cols][cols] H[perm][:, perm] (activation order)
  int* perm;                 // device [n_mats][cols] column processed j-th (activation order, else null)
  int* ipos;                 // device [n_mats][cols] processing position of each column
  int* gidx;                 // device [n_mats][cols] grid of each column (any option)
};
constexpr int kFactorStreams = 4;     // Hessian groups factored on separate streams
void launch_factor_group(const GptqPlan& p, int m0, int m1, hipStream_t s, hipEvent_t step0_done);
// A contiguous range of jobs [j0, j1) with their global slabs and row tiles.
struct JobRange {
  int j0, j1, slab0, n_slabs, tile0, n_tiles;
  int m0, m1;   // the Hessians of these jobs
};
void launch_gptq(const GptqPlan& p, const JobRange& r, hipStream_t s);
// Before the factorisation of Hessians [m0, m1) and the GPTQ of their jobs,
// when an option is on: processing order and grid index per column, the
// permuted Hessians, the jobs' working copies and their static grids.
void launch_gptq_prep(const GptqPlan& p, const JobRange& r, hipStream_t s);
// g_idx of the natural order: g[i] = i / group
void launch_natural_gidx(int32_t* g, int cols, int group, hipStream_t s);

// ---------------------------------------------------------------- loss
// gidx (optional, device int32 [cols]) names each column's grid; null means column k / group
void launch_loss(int rows, int cols, int group, const void* W, int dtype, const uint8_t* codes,
                 const float* scales, const uint8_t* zeros, const float* H, const int* gidx,
                 float* partials, float* loss_out, hipStream_t s);
int64_t loss_partial_count(int rows, int cols);
// The allocation-free loss entry point's scratch: kLossScratchPartials fp64
// partials (1 MiB) per device, in a file-scope device array of loss.hip.
constexpr int64_t kLossScratchPartials = 131072;
bool loss_scratch_init(int device);      // looks the array up on `device` (current); false on failure
double* loss_scratch(int device);        // its address on `device`, or null before init

// ---------------------------------------------------------------- packed codes
void launch_pack_codes(const uint8_t* codes, uint8_t* packed, int64_t n_codes, int bits, hipStream_t s);
void launch_unpack_codes(const uint8_t* packed, uint8_t* codes, int64_t n_codes, int bits, hipStream_t s);

}  // namespace clha
