// Host side of the CLHA C ABI: argument validation, the layer registry that keeps
// per-layer accumulators apart, workspace carving and the device status record.
// All compute is enqueued through the launchers in kernels.h.
#include "clha.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <map>
#include <string>
#include <vector>

#include "kernels.h"

using clha::AggArgs;
using clha::CollectPlan;
using clha::GJob;
using clha::GptqPlan;

namespace clha {
bool gptq_group_supported(int group);
int syrk_items_per_slot(int d);
}

struct LayerBufs {
  float* S;
  int64_t* counts;
  bool fresh;   // reset since the last collection with tokens: the next one overwrites
};

struct clha_ctx {
  clha_moe_desc desc;
  int slots;
  int device;
  int* status_dev;               // this context's status record (kernels.h), from the pool
  int status_slot = -1;
  std::map<int32_t, LayerBufs> layers;
  std::string err;
  void* pinned = nullptr;        // staging for job tables (host, page-locked)
  size_t pinned_bytes = 0;
  hipEvent_t pinned_done = nullptr;
  bool pinned_pending = false;
  // optional per-stage timers
  bool timing = false;
  struct Rec {
    int stage;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> free_events;
  // extra streams of the factorisation (default priority) and their events
  hipStream_t aux[clha::kFactorStreams - 1] = {};
  hipEvent_t stagger[clha::kFactorStreams] = {};
  hipEvent_t join[clha::kFactorStreams] = {};
  bool aux_ready = false;
};

namespace {

constexpr uint32_t kGptqFlags = CLHA_GPTQ_ACT_ORDER | CLHA_GPTQ_STATIC_GROUPS;

clha_status fail(clha_ctx* ctx, clha_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (ctx) ctx->err = buf;
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

// Sequential carve-up of one workspace allocation.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += up256(count * sizeof(T));
    return p;
  }
};

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

hipEvent_t take_event(clha_ctx* ctx) {
  if (!ctx->free_events.empty()) {
    hipEvent_t e = ctx->free_events.back();
    ctx->free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Records a hipEvent pair around one stage's launches when timing is enabled.
struct StageTimer {
  clha_ctx* ctx;
  int stage;
  hipStream_t s;
  hipEvent_t a = nullptr;
  StageTimer(clha_ctx* c, int st, hipStream_t stream) : ctx(c), stage(st), s(stream) {
    if (!ctx->timing) return;
    a = take_event(ctx);
    if (a) hipEventRecord(a, s);
  }
  ~StageTimer() {
    if (!a) return;
    hipEvent_t b = take_event(ctx);
    if (!b) {
      ctx->free_events.push_back(a);
      return;
    }
    hipEventRecord(b, s);
    ctx->recs.push_back({stage, a, b});
  }
};

clha_status hip_check(clha_ctx* ctx, const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ctx, CLHA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return CLHA_OK;
}

// Copies `bytes` of host data to `dst` on `stream` through the context's pinned
// staging buffer; waits for the previous staged copy before reusing the buffer.
clha_status stage_to_device(clha_ctx* ctx, void* dst, const void* src, size_t bytes,
                            hipStream_t stream) {
  if (ctx->pinned_pending) {
    if (hipEventSynchronize(ctx->pinned_done) != hipSuccess)
      return fail(ctx, CLHA_ERR_HIP, "staging wait failed");
    ctx->pinned_pending = false;
  }
  if (bytes > ctx->pinned_bytes) {
    if (ctx->pinned) hipHostFree(ctx->pinned);
    ctx->pinned = nullptr;
    size_t nb = bytes < 65536 ? 65536 : bytes * 2;
    if (hipHostMalloc(&ctx->pinned, nb, hipHostMallocDefault) != hipSuccess) {
      ctx->pinned_bytes = 0;
      return fail(ctx, CLHA_ERR_HIP, "pinned staging allocation failed");
    }
    ctx->pinned_bytes = nb;
  }
  std::memcpy(ctx->pinned, src, bytes);
  if (hipMemcpyAsync(dst, ctx->pinned, bytes, hipMemcpyHostToDevice, stream) != hipSuccess)
    return fail(ctx, CLHA_ERR_HIP, "staging copy failed");
  if (hipEventRecord(ctx->pinned_done, stream) != hipSuccess)
    return fail(ctx, CLHA_ERR_HIP, "staging event failed");
  ctx->pinned_pending = true;
  return CLHA_OK;
}

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bn && y < x + an;
}

// ---------------------------------------------------------------- collection layout
struct CollectLayout {
  int32_t* topk;
  int32_t* blockcounts;
  int32_t* blockbase;
  int64_t* offsets;
  int64_t* pad_off;
  int32_t* slot_order;
  int32_t* work;
  int32_t* work_len;
  int32_t* work_next;
  int32_t* seg;
  int32_t* split;
  float* partials;
  int max_partials;
  int32_t* token_ids;
  int32_t* iota;
  uint16_t* zero_row;
  size_t bytes;
};

CollectLayout collect_layout(const clha_ctx* ctx, void* ws) {
  const clha_moe_desc& d = ctx->desc;
  const int64_t n = d.max_tokens;
  const int64_t nblk = (n + clha::kBucketTokens - 1) / clha::kBucketTokens;
  Carver c(ws);
  CollectLayout L;
  L.topk = c.take<int32_t>((size_t)n * d.top_k);
  L.blockcounts = c.take<int32_t>((size_t)nblk * d.n_routed);
  L.blockbase = c.take<int32_t>((size_t)nblk * d.n_routed);
  L.offsets = c.take<int64_t>((size_t)d.n_routed + 1);
  L.pad_off = c.take<int64_t>((size_t)ctx->slots + 1);
  L.slot_order = c.take<int32_t>((size_t)ctx->slots);
  L.max_partials = clha::max_partials(d.d, n, d.top_k, ctx->slots);
  const int max_segs = ctx->slots + L.max_partials;
  L.work = c.take<int32_t>((size_t)clha::kXcds * max_segs * clha::syrk_items_per_slot(d.d));
  L.work_len = c.take<int32_t>(clha::kXcds);
  L.work_next = c.take<int32_t>(clha::kXcds);
  L.seg = c.take<int32_t>((size_t)4 * max_segs);
  L.split = c.take<int32_t>((size_t)1 + 3 * L.max_partials);
  L.partials = c.take<float>((size_t)L.max_partials * d.d * d.d);
  L.token_ids = c.take<int32_t>((size_t)n * d.top_k);
  L.iota = c.take<int32_t>((size_t)n);
  L.zero_row = c.take<uint16_t>((size_t)d.d);
  L.bytes = c.off;
  return L;
}

// ---------------------------------------------------------------- down_proj layout
// The down_proj context has d = f (the intermediate size) and one slot per
// routed expert and per shared expert; its collection reads the model-width
// activations through the routing of the block's main context.
struct DownLayout {
  const uint16_t** wgu;
  int64_t* pad_off;
  int32_t* slot_order;
  int32_t* tile_off;
  int32_t* work;
  int32_t* work_len;
  int32_t* work_next;
  int32_t* seg;
  int32_t* split;
  float* partials;
  int max_partials;
  uint16_t* hT;
  size_t bytes;
};

DownLayout down_layout(const clha_ctx* ctx, int n_routed, void* ws) {
  const clha_moe_desc& d = ctx->desc;
  const int64_t n = d.max_tokens;
  const int slots = ctx->slots;
  const int64_t h_tokens = n * d.top_k + (int64_t)(slots - n_routed) * n + (int64_t)clha::kTokPad * slots;
  Carver c(ws);
  DownLayout L;
  L.wgu = c.take<const uint16_t*>((size_t)slots);
  L.pad_off = c.take<int64_t>((size_t)slots + 1);
  L.slot_order = c.take<int32_t>((size_t)slots);
  L.tile_off = c.take<int32_t>((size_t)slots + 1);
  L.max_partials = clha::max_partials(d.d, n, d.top_k, slots);
  const int max_segs = slots + L.max_partials;
  L.work = c.take<int32_t>((size_t)clha::kXcds * max_segs * clha::syrk_items_per_slot(d.d));
  L.work_len = c.take<int32_t>(clha::kXcds);
  L.work_next = c.take<int32_t>(clha::kXcds);
  L.seg = c.take<int32_t>((size_t)4 * max_segs);
  L.split = c.take<int32_t>((size_t)1 + 3 * L.max_partials);
  L.partials = c.take<float>((size_t)L.max_partials * d.d * d.d);
  L.hT = c.take<uint16_t>((size_t)h_tokens * d.d);
  L.bytes = c.off;
  return L;
}

// ---------------------------------------------------------------- GPTQ layout
struct GptqLayout {
  GJob* jobs;
  const float** mats;
  double* A;
  double* X;
  float* U;
  float* UT;
  double* dinv;
  uint8_t* dead;
  double* lamd;
  int* lexp;
  float* wf;
  float* ebuf;
  double* partials;
  const float** src_mats;
  float* hperm;
  int* perm;
  int* ipos;
  int* gidx;
  int* mstat;
  double* eval_part;
  size_t bytes;
};

GptqLayout gptq_layout(void* ws, int n_jobs, int n_mats, int cols, int64_t wf_elems,
                       int64_t total_slabs, bool need_u, bool need_wf, uint32_t flags = 0,
                       int64_t eval_parts = 0) {
  Carver c(ws);
  GptqLayout L;
  const bool act = flags & CLHA_GPTQ_ACT_ORDER;
  L.jobs = c.take<GJob>((size_t)(n_jobs > 0 ? n_jobs : 1));
  L.mats = c.take<const float*>((size_t)n_mats);
  // the callers' Hessians, staged with the job and Hessian tables in one copy
  L.src_mats = flags ? c.take<const float*>((size_t)n_mats) : nullptr;
  L.A = c.take<double>((size_t)n_mats * cols * cols);
  L.X = c.take<double>((size_t)n_mats * cols * cols);
  L.U = need_u ? c.take<float>((size_t)n_mats * cols * cols) : nullptr;
  L.UT = need_u ? c.take<float>((size_t)n_mats * cols * cols) : nullptr;
  L.dinv = c.take<double>((size_t)n_mats * cols * clha::kNb);
  L.dead = c.take<uint8_t>((size_t)n_mats * cols);
  L.lamd = c.take<double>((size_t)n_mats);
  L.lexp = c.take<int>((size_t)n_mats * cols);
  L.wf = need_wf ? c.take<float>((size_t)wf_elems) : nullptr;
  L.ebuf = need_wf && cols > clha::kSuper ? c.take<float>((size_t)(wf_elems / cols) * clha::kSuper) : nullptr;
  L.partials = need_wf ? c.take<double>((size_t)2 * (total_slabs > 0 ? total_slabs : 1)) : nullptr;
  L.hperm = act ? c.take<float>((size_t)n_mats * cols * cols) : nullptr;
  L.perm = act ? c.take<int>((size_t)n_mats * cols) : nullptr;
  L.ipos = flags ? c.take<int>((size_t)n_mats * cols) : nullptr;
  L.gidx = flags ? c.take<int>((size_t)n_mats * cols) : nullptr;
  L.mstat = c.take<int>((size_t)n_mats);
  L.eval_part = eval_parts > 0 ? c.take<double>((size_t)eval_parts) : nullptr;
  L.bytes = c.off;
  return L;
}

struct JobScan {
  std::vector<const float*> mats;
  std::vector<int> mat_of;
  std::vector<int64_t> eval_off;   // each job's loss partials under H_eval (-1: none)
  int64_t wf_elems = 0;
  int64_t total_slabs = 0;
  int64_t eval_parts = 0;
};

JobScan scan_jobs(int n_jobs, const clha_gptq_job* jobs, int cols) {
  JobScan s;
  std::map<const float*, int> ids;
  for (int i = 0; i < n_jobs; ++i) {
    auto it = ids.find(jobs[i].H);
    int id;
    if (it == ids.end()) {
      id = (int)s.mats.size();
      ids[jobs[i].H] = id;
      s.mats.push_back(jobs[i].H);
    } else {
      id = it->second;
    }
    s.mat_of.push_back(id);
    s.eval_off.push_back(jobs[i].H_eval ? s.eval_parts : -1);
    if (jobs[i].H_eval) s.eval_parts += clha::loss_partial_count(jobs[i].rows, cols);
    const int64_t slabs = (jobs[i].rows + clha::kGptqRows - 1) / clha::kGptqRows;
    s.wf_elems += slabs * clha::kGptqRows * cols;   // whole 64-row slabs
    s.total_slabs += slabs;
  }
  return s;
}

}  // namespace

extern "C" {

CLHA_API clha_status clha_create(const clha_moe_desc* desc, clha_ctx** out) {
  if (!desc || !out) return CLHA_ERR_INVALID_ARG;
  *out = nullptr;
  const clha_moe_desc& d = *desc;
  if (d.d < 128 || d.d > 8192 || d.d % 128 != 0) return CLHA_ERR_SHAPE;
  if (d.n_routed < 1 || d.n_routed > clha::kMaxExperts) return CLHA_ERR_SHAPE;
  if (d.top_k < 1 || d.top_k > d.n_routed || d.top_k > clha::kMaxTopK) return CLHA_ERR_SHAPE;
  if (d.n_shared < 0) return CLHA_ERR_SHAPE;
  if (d.max_tokens < 1 || d.max_tokens > (int64_t)INT32_MAX / d.top_k) return CLHA_ERR_SHAPE;
  clha_ctx* ctx = new (std::nothrow) clha_ctx();
  if (!ctx) return CLHA_ERR_INVALID_ARG;
  ctx->desc = d;
  ctx->slots = d.n_routed + (d.n_shared > 0 ? 1 : 0);
  if (hipGetDevice(&ctx->device) != hipSuccess || !clha::loss_scratch_init(ctx->device) ||
      !(ctx->status_dev = clha::status_acquire(ctx->device, &ctx->status_slot)) ||
      hipEventCreateWithFlags(&ctx->pinned_done, hipEventDisableTiming) != hipSuccess) {
    if (ctx->status_dev) clha::status_release(ctx->device, ctx->status_slot);
    delete ctx;
    return CLHA_ERR_HIP;
  }
  *out = ctx;
  return CLHA_OK;
}

CLHA_API clha_status clha_destroy(clha_ctx* ctx) {
  if (!ctx) return CLHA_OK;
  if (ctx->pinned_pending) hipEventSynchronize(ctx->pinned_done);
  if (ctx->pinned) hipHostFree(ctx->pinned);
  if (ctx->pinned_done) hipEventDestroy(ctx->pinned_done);
  for (auto& r : ctx->recs) {
    hipEventSynchronize(r.b);
    hipEventDestroy(r.a);
    hipEventDestroy(r.b);
  }
  for (auto e : ctx->free_events) hipEventDestroy(e);
  for (auto& a : ctx->aux)
    if (a) {
      hipStreamSynchronize(a);
      hipStreamDestroy(a);
    }
  for (int g = 0; g < clha::kFactorStreams; ++g) {
    if (ctx->stagger[g]) hipEventDestroy(ctx->stagger[g]);
    if (ctx->join[g]) hipEventDestroy(ctx->join[g]);
  }
  if (ctx->status_dev) {
    // kernels of this context may still write its record: wait for its device first
    int cur = -1;
    hipGetDevice(&cur);
    if (cur != ctx->device) hipSetDevice(ctx->device);
    hipDeviceSynchronize();
    if (cur >= 0 && cur != ctx->device) hipSetDevice(cur);
    clha::status_release(ctx->device, ctx->status_slot);
  }
  delete ctx;
  return CLHA_OK;
}

CLHA_API const char* clha_last_error(const clha_ctx* ctx) {
  return ctx ? ctx->err.c_str() : "null context";
}

CLHA_API int32_t clha_num_slots(const clha_ctx* ctx) { return ctx ? ctx->slots : 0; }

CLHA_API clha_status clha_register_layer(clha_ctx* ctx, int32_t layer, float* S, int64_t* counts) {
  if (!ctx) return CLHA_ERR_INVALID_ARG;
  if (!S || !counts) return fail(ctx, CLHA_ERR_INVALID_ARG, "register_layer: null buffer");
  if (!aligned16(S) || !aligned4(counts)) return fail(ctx, CLHA_ERR_ALIGN, "register_layer: misaligned");
  const size_t sb = (size_t)ctx->slots * ctx->desc.d * ctx->desc.d * sizeof(float);
  const size_t cb = (size_t)ctx->slots * sizeof(int64_t);
  for (const auto& kv : ctx->layers) {
    if (kv.first == layer) continue;
    const LayerBufs& o = kv.second;
    if (overlaps(S, sb, o.S, sb) || overlaps(counts, cb, o.counts, cb) ||
        overlaps(S, sb, o.counts, cb) || overlaps(counts, cb, o.S, sb))
      return fail(ctx, CLHA_ERR_INVALID_ARG,
                  "register_layer: layer %d's buffers overlap layer %d's; every layer needs "
                  "its own Hessian accumulator", layer, kv.first);
  }
  if (overlaps(S, sb, counts, cb))
    return fail(ctx, CLHA_ERR_INVALID_ARG, "register_layer: S and counts overlap");
  ctx->layers[layer] = LayerBufs{S, counts, false};
  return CLHA_OK;
}

CLHA_API clha_status clha_reset_layer(clha_ctx* ctx, int32_t layer, void* stream) {
  if (!ctx) return CLHA_ERR_INVALID_ARG;
  auto it = ctx->layers.find(layer);
  if (it == ctx->layers.end())
    return fail(ctx, CLHA_ERR_INVALID_ARG, "reset_layer: layer %d is not registered", layer);
  clha::launch_zero_counts(it->second.counts, ctx->slots, as_stream(stream));
  it->second.fresh = true;
  return hip_check(ctx, "reset_layer");
}

CLHA_API size_t clha_collect_workspace_bytes(const clha_ctx* ctx) {
  if (!ctx) return 0;
  return collect_layout(ctx, nullptr).bytes;
}

CLHA_API clha_status clha_collect_hessians(clha_ctx* ctx, int32_t layer, int64_t n_tokens,
                                           const uint16_t* x, const float* logits,
                                           int32_t* topk_out, int64_t* offsets_out,
                                           int32_t* token_ids_out, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  if (!ctx) return CLHA_ERR_INVALID_ARG;
  auto it = ctx->layers.find(layer);
  if (it == ctx->layers.end())
    return fail(ctx, CLHA_ERR_INVALID_ARG, "collect_hessians: layer %d is not registered", layer);
  if (n_tokens < 0 || n_tokens > ctx->desc.max_tokens)
    return fail(ctx, CLHA_ERR_SHAPE, "collect_hessians: n_tokens %lld outside 0..%lld",
                (long long)n_tokens, (long long)ctx->desc.max_tokens);
  if (n_tokens == 0) return CLHA_OK;   // an empty batch adds nothing; its pointers are not read
  if (!x || !logits || !workspace)
    return fail(ctx, CLHA_ERR_INVALID_ARG, "collect_hessians: null x, logits or workspace");
  if (!aligned16(x) || !aligned4(logits) || !aligned16(workspace) ||
      (topk_out && !aligned4(topk_out)) || (offsets_out && !aligned16(offsets_out)) ||
      (token_ids_out && !aligned4(token_ids_out)))
    return fail(ctx, CLHA_ERR_ALIGN, "collect_hessians: misaligned pointer");
  const CollectLayout need = collect_layout(ctx, nullptr);
  if (workspace_bytes < need.bytes)
    return fail(ctx, CLHA_ERR_WORKSPACE, "collect_hessians: workspace %zu < %zu bytes",
                workspace_bytes, need.bytes);
  const CollectLayout L = collect_layout(ctx, workspace);
  const clha_moe_desc& d = ctx->desc;
  CollectPlan p;
  p.n_tokens = n_tokens;
  p.d = d.d;
  p.E = d.n_routed;
  p.K = d.top_k;
  p.has_shared = d.n_shared > 0;
  p.nblk = (int)((n_tokens + clha::kBucketTokens - 1) / clha::kBucketTokens);
  p.topk = topk_out ? topk_out : L.topk;
  p.blockcounts = L.blockcounts;
  p.blockbase = L.blockbase;
  p.offsets = offsets_out ? offsets_out : L.offsets;
  p.pad_off = L.pad_off;
  p.slot_order = L.slot_order;
  p.work = L.work;
  p.work_len = L.work_len;
  p.work_next = L.work_next;
  p.seg = L.seg;
  p.split = L.split;
  p.partials = L.partials;
  p.max_partials = L.max_partials;
  p.max_segs = ctx->slots + L.max_partials;
  p.syrk_items = clha::syrk_items_per_slot(d.d);
  p.overwrite = it->second.fresh ? 1 : 0;
  p.token_ids = token_ids_out ? token_ids_out : L.token_ids;
  p.xgT = nullptr;
  p.x_rows = x;
  p.iota = L.iota;
  p.zero_row = L.zero_row;
  p.status = ctx->status_dev;
  p.layer = layer;
  // the shared slot's sums are derived from the routed ones (every token goes
  // to exactly top_k routed experts): no Gram-sum items for it
  p.derive_shared = p.has_shared ? 1 : 0;
  const hipStream_t s = as_stream(stream);
  {
    StageTimer t(ctx, CLHA_STAGE_ROUTE, s);
    clha::launch_route(logits, p, s);
  }
  {
    StageTimer t(ctx, CLHA_STAGE_BUCKET, s);
    clha::launch_bucket(p, it->second.counts, s);
  }
  {
    StageTimer t(ctx, CLHA_STAGE_SYRK, s);
    clha::launch_syrk(p, it->second.S, s);
  }
  {
    StageTimer t(ctx, CLHA_STAGE_SYRK_REDUCE, s);
    clha::launch_syrk_reduce(p, it->second.S, it->second.counts, s);
  }
  it->second.fresh = false;
  return hip_check(ctx, "collect_hessians");
}

CLHA_API clha_status clha_aggregate(clha_ctx* ctx, int32_t n_layers, const int32_t* layers,
                                    clha_alpha_mode mode, const float* alpha, float* H_out,
                                    float* alpha_out, void* stream) {
  if (!ctx) return CLHA_ERR_INVALID_ARG;
  if (n_layers < 1 || n_layers > clha::kMaxLayers || !layers)
    return fail(ctx, CLHA_ERR_SHAPE, "aggregate: n_layers must be 1..%d", clha::kMaxLayers);
  if (mode != CLHA_ALPHA_ROUTING_FREQ && mode != CLHA_ALPHA_EQUAL && mode != CLHA_ALPHA_EXPLICIT &&
      mode != CLHA_ALPHA_EXPLICIT_PER_SLOT)
    return fail(ctx, CLHA_ERR_INVALID_ARG, "aggregate: unknown alpha mode %d", (int)mode);
  if (mode == CLHA_ALPHA_EXPLICIT_PER_SLOT && (!alpha || !aligned4(alpha)))
    return fail(ctx, CLHA_ERR_INVALID_ARG, "aggregate: per-slot mode needs a device alpha table");
  if (!H_out) return fail(ctx, CLHA_ERR_INVALID_ARG, "aggregate: null H_out");
  if (!aligned16(H_out) || (alpha_out && !aligned4(alpha_out)))
    return fail(ctx, CLHA_ERR_ALIGN, "aggregate: misaligned output");
  AggArgs a;
  std::memset(&a, 0, sizeof a);
  for (int i = 0; i < n_layers; ++i) {
    auto it = ctx->layers.find(layers[i]);
    if (it == ctx->layers.end())
      return fail(ctx, CLHA_ERR_INVALID_ARG, "aggregate: layer %d is not registered", layers[i]);
    for (int j = 0; j < i; ++j)
      if (layers[j] == layers[i])
        return fail(ctx, CLHA_ERR_INVALID_ARG, "aggregate: layer %d listed twice", layers[i]);
    a.S[i] = it->second.S;
    a.counts[i] = it->second.counts;
    if (mode == CLHA_ALPHA_EXPLICIT) {
      if (!alpha) return fail(ctx, CLHA_ERR_INVALID_ARG, "aggregate: explicit mode needs alpha");
      if (!std::isfinite(alpha[i]) || alpha[i] < 0.0f)
        return fail(ctx, CLHA_ERR_INVALID_ARG, "aggregate: alpha[%d] must be finite and >= 0", i);
      a.alpha[i] = alpha[i];
    }
  }
  const size_t hb = (size_t)ctx->slots * ctx->desc.d * ctx->desc.d * sizeof(float);
  for (const auto& kv : ctx->layers)
    if (overlaps(H_out, hb, kv.second.S, hb))
      return fail(ctx, CLHA_ERR_INVALID_ARG, "aggregate: H_out overlaps layer %d's S", kv.first);
  a.alpha_slot = mode == CLHA_ALPHA_EXPLICIT_PER_SLOT ? alpha : nullptr;
  a.n_layers = n_layers;
  a.mode = (int)mode;
  a.d = ctx->desc.d;
  a.slots = ctx->slots;
  {
    StageTimer t(ctx, CLHA_STAGE_AGGREGATE, as_stream(stream));
    clha::launch_aggregate(a, H_out, alpha_out, as_stream(stream));
  }
  return hip_check(ctx, "aggregate");
}

// Factorisation of all distinct Hessians (and, when `jobs` is given, the GPTQ
// of their jobs): groups of Hessians on up to kFactorStreams streams forked
// from and joined back to the caller's stream; group g starts once group g-1
// has finished its first block step.  A group's GPTQ jobs follow its own
// factorisation on its stream, so they overlap the later groups' factors.
// `jobs` (host copy of the device job table) must be sorted by Hessian; `evals`
// (same order, may be null) holds each job's optional second-Hessian loss,
// computed on the job's stream once its GPTQ is done.
struct EvalJob {
  const float* H = nullptr;
  float* out = nullptr;
  float* partials = nullptr;
};

static clha_status run_factor(clha_ctx* ctx, const GptqPlan& p, hipStream_t s, const GJob* jobs,
                              const EvalJob* evals = nullptr) {
  if (!ctx->aux_ready) {
    for (auto& a : ctx->aux)
      if (hipStreamCreateWithFlags(&a, hipStreamNonBlocking) != hipSuccess)
        return fail(ctx, CLHA_ERR_HIP, "factor: stream creation failed");
    for (int g = 0; g < clha::kFactorStreams; ++g)
      if (hipEventCreateWithFlags(&ctx->stagger[g], hipEventDisableTiming) != hipSuccess ||
          hipEventCreateWithFlags(&ctx->join[g], hipEventDisableTiming) != hipSuccess)
        return fail(ctx, CLHA_ERR_HIP, "factor: event creation failed");
    ctx->aux_ready = true;
  }
  const int groups = p.n_mats < clha::kFactorStreams ? p.n_mats : clha::kFactorStreams;
  int j = 0;
  for (int g = 0; g < groups; ++g) {
    const int m0 = (int)((int64_t)p.n_mats * g / groups), m1 = (int)((int64_t)p.n_mats * (g + 1) / groups);
    hipStream_t gs = g == 0 ? s : ctx->aux[g - 1];
    if (g > 0) hipStreamWaitEvent(gs, ctx->stagger[g - 1], 0);
    clha::JobRange r{};
    r.j0 = j;
    r.m0 = m0;
    r.m1 = m1;
    if (jobs) {
      while (j < p.n_jobs && jobs[j].mat < m1) ++j;
      r.j1 = j;
      if (r.j1 > r.j0) {
        const GJob& first = jobs[r.j0];
        const GJob& last = jobs[r.j1 - 1];
        r.slab0 = first.slab_base;
        r.n_slabs = last.slab_base + last.n_slabs - first.slab_base;
        r.tile0 = first.tile_base;
        r.n_tiles = last.tile_base + last.n_tiles - first.tile_base;
      }
      clha::launch_gptq_prep(p, r, gs);
    }
    clha::launch_factor_group(p, m0, m1, gs, g + 1 < groups ? ctx->stagger[g] : nullptr);
    if (jobs && r.j1 > r.j0) clha::launch_gptq(p, r, gs);
    for (int k = r.j0; evals && k < r.j1; ++k) {
      const GJob& jb = jobs[k];
      if (!evals[k].H) continue;
      clha::launch_loss(jb.rows, p.cols, p.group, jb.W, jb.dtype, jb.codes, jb.scales, jb.zeros, evals[k].H,
                        p.gidx ? p.gidx + (size_t)jb.mat * p.cols : nullptr, evals[k].partials, evals[k].out, gs);
    }
  }
  for (int g = 1; g < groups; ++g) {
    hipEventRecord(ctx->join[g], ctx->aux[g - 1]);
    hipStreamWaitEvent(s, ctx->join[g], 0);
  }
  return CLHA_OK;
}

static clha_status check_gptq_args(clha_ctx* ctx, int32_t n_jobs, const clha_gptq_job* jobs,
                                   int32_t cols, int32_t group, int32_t block, float damp) {
  if (n_jobs < 1 || !jobs) return fail(ctx, CLHA_ERR_INVALID_ARG, "gptq: no jobs");
  if (block != 64 && block != 128) return fail(ctx, CLHA_ERR_SHAPE, "gptq: block must be 64 or 128");
  if (cols < block || cols > 8192 || cols % block != 0)
    return fail(ctx, CLHA_ERR_SHAPE, "gptq: cols %d must be a multiple of block %d, <= 8192", cols, block);
  if (!clha::gptq_group_supported(group) || block % group != 0)
    return fail(ctx, CLHA_ERR_SHAPE, "gptq: group %d must be one of 4, 8, 16, 32, 64, 128 and divide block %d",
                group, block);
  if (!std::isfinite(damp) || damp < 0.0f) return fail(ctx, CLHA_ERR_INVALID_ARG, "gptq: bad damp");
  for (int i = 0; i < n_jobs; ++i) {
    const clha_gptq_job& j = jobs[i];
    if (!j.H || !j.W || !j.codes || !j.scales || !j.zeros)
      return fail(ctx, CLHA_ERR_INVALID_ARG, "gptq: job %d has a null pointer", i);
    if (j.w_dtype != CLHA_F32 && j.w_dtype != CLHA_BF16)
      return fail(ctx, CLHA_ERR_INVALID_ARG, "gptq: job %d has an unknown dtype", i);
    if (j.rows < 1 || j.bits < 2 || j.bits > 8)
      return fail(ctx, CLHA_ERR_SHAPE, "gptq: job %d needs rows >= 1 and bits in 2..8", i);
    if (!j.H_eval != !j.loss_eval)
      return fail(ctx, CLHA_ERR_INVALID_ARG, "gptq: job %d needs loss_eval exactly when H_eval is given", i);
    if (!aligned16(j.H) || !aligned16(j.W) || !aligned16(j.codes) || !aligned4(j.scales) ||
        (j.loss && !aligned4(j.loss)) || (j.H_eval && !aligned16(j.H_eval)) ||
        (j.loss_eval && !aligned4(j.loss_eval)) || (j.status && !aligned4(j.status)))
      return fail(ctx, CLHA_ERR_ALIGN, "gptq: job %d has a misaligned pointer", i);
  }
  return CLHA_OK;
}

CLHA_API size_t clha_gptq_workspace_bytes_ex(const clha_ctx* ctx, int32_t n_jobs,
                                             const clha_gptq_job* jobs, int32_t cols, uint32_t flags) {
  if (!ctx || n_jobs < 1 || !jobs || cols < 1) return 0;
  const JobScan js = scan_jobs(n_jobs, jobs, cols);
  return gptq_layout(nullptr, n_jobs, (int)js.mats.size(), cols, js.wf_elems, js.total_slabs, true,
                     true, flags & kGptqFlags, js.eval_parts).bytes;
}

CLHA_API size_t clha_gptq_workspace_bytes(const clha_ctx* ctx, int32_t n_jobs,
                                          const clha_gptq_job* jobs, int32_t cols) {
  return clha_gptq_workspace_bytes_ex(ctx, n_jobs, jobs, cols, 0);
}

CLHA_API clha_status clha_gptq_quantize_ex(clha_ctx* ctx, int32_t n_jobs, const clha_gptq_job* jobs,
                                           int32_t cols, int32_t group, int32_t block, float damp,
                                           uint32_t flags, int32_t* const* g_idx, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  if (!ctx) return CLHA_ERR_INVALID_ARG;
  clha_status st = check_gptq_args(ctx, n_jobs, jobs, cols, group, block, damp);
  if (st != CLHA_OK) return st;
  if (flags & ~kGptqFlags) return fail(ctx, CLHA_ERR_INVALID_ARG, "gptq: unknown flags 0x%x", flags);
  if (g_idx)
    for (int i = 0; i < n_jobs; ++i)
      if (g_idx[i] && !aligned4(g_idx[i]))
        return fail(ctx, CLHA_ERR_ALIGN, "gptq: g_idx[%d] is misaligned", i);
  if (!workspace || !aligned16(workspace))
    return fail(ctx, CLHA_ERR_ALIGN, "gptq: workspace null or misaligned");
  const JobScan js = scan_jobs(n_jobs, jobs, cols);
  const int n_mats = (int)js.mats.size();
  const GptqLayout need = gptq_layout(nullptr, n_jobs, n_mats, cols, js.wf_elems, js.total_slabs,
                                      true, true, flags, js.eval_parts);
  if (workspace_bytes < need.bytes)
    return fail(ctx, CLHA_ERR_WORKSPACE, "gptq: workspace %zu < %zu bytes", workspace_bytes, need.bytes);
  if (js.total_slabs > INT32_MAX) return fail(ctx, CLHA_ERR_SHAPE, "gptq: too many rows");
  const GptqLayout L = gptq_layout(workspace, n_jobs, n_mats, cols, js.wf_elems, js.total_slabs,
                                   true, true, flags, js.eval_parts);
  const bool act = flags & CLHA_GPTQ_ACT_ORDER;
  // host tables: jobs, the Hessian pointers the factorisation reads, and (with
  // an option) the callers' Hessians, staged in one copy
  const size_t mats_bytes = sizeof(float*) * n_mats;
  std::vector<char> host(up256(sizeof(GJob) * n_jobs) + (flags ? up256(mats_bytes) : 0) + mats_bytes);
  GJob* hj = reinterpret_cast<GJob*>(host.data());
  // device job table ordered by Hessian (stable), so the jobs of each
  // factorisation group are contiguous
  std::vector<int> order(n_jobs);
  for (int i = 0; i < n_jobs; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return js.mat_of[a] < js.mat_of[b]; });
  int64_t wf_off = 0;
  int slab_base = 0, tile_base = 0;
  std::vector<EvalJob> evals(n_jobs);
  for (int k = 0; k < n_jobs; ++k) {
    const int i = order[k];
    const clha_gptq_job& j = jobs[i];
    if (j.H_eval) {
      evals[k].H = j.H_eval;
      evals[k].out = j.loss_eval;
      evals[k].partials = reinterpret_cast<float*>(L.eval_part + js.eval_off[i]);
    }
    GJob g;
    g.W = j.W;
    g.codes = j.codes;
    g.scales = j.scales;
    g.zeros = j.zeros;
    g.loss = j.loss;
    g.wf_off = wf_off;
    g.dtype = j.w_dtype;
    g.rows = j.rows;
    g.bits = j.bits;
    g.mat = js.mat_of[i];
    g.slab_base = slab_base;
    g.n_slabs = (j.rows + clha::kGptqRows - 1) / clha::kGptqRows;
    g.tile_base = tile_base;
    g.n_tiles = (g.n_slabs * clha::kGptqRows + clha::kGemmTile - 1) / clha::kGemmTile;
    g.user_index = i;
    g.status = j.status;
    g.dead_out = j.dead;
    hj[k] = g;
    wf_off += (int64_t)g.n_slabs * clha::kGptqRows * cols;
    slab_base += g.n_slabs;
    tile_base += g.n_tiles;
  }
  {
    char* hm = host.data() + up256(sizeof(GJob) * n_jobs);
    std::vector<const float*> fmats(js.mats);
    if (act)   // the factorisation reads the permuted copies
      for (int m = 0; m < n_mats; ++m) fmats[m] = L.hperm + (size_t)m * cols * cols;
    std::memcpy(hm, fmats.data(), mats_bytes);
    if (flags) std::memcpy(hm + up256(mats_bytes), js.mats.data(), mats_bytes);
  }
  const hipStream_t s = as_stream(stream);
  // jobs, mats and src_mats are adjacent in the layout (carved first)
  if (reinterpret_cast<char*>(L.mats) != reinterpret_cast<char*>(L.jobs) + up256(sizeof(GJob) * n_jobs) ||
      (flags && reinterpret_cast<char*>(L.src_mats) != reinterpret_cast<char*>(L.mats) + up256(mats_bytes)))
    return fail(ctx, CLHA_ERR_WORKSPACE, "gptq: internal layout mismatch");
  st = stage_to_device(ctx, L.jobs, host.data(), host.size(), s);
  if (st != CLHA_OK) return st;
  GptqPlan p;
  std::memset(&p, 0, sizeof p);
  p.act_order = act;
  p.static_groups = (flags & CLHA_GPTQ_STATIC_GROUPS) != 0;
  p.src_mats = flags ? L.src_mats : L.mats;
  p.hperm = L.hperm;
  p.perm = L.perm;
  p.ipos = L.ipos;
  p.gidx = L.gidx;
  p.n_jobs = n_jobs;
  p.n_mats = n_mats;
  p.cols = cols;
  p.group = group;
  p.block = block;
  p.total_slabs = (int)js.total_slabs;
  p.total_tiles = tile_base;
  p.damp = damp;
  p.jobs = L.jobs;
  p.mats = L.mats;
  p.A = L.A;
  p.X = L.X;
  p.U = L.U;
  p.UT = L.UT;
  p.dinv = L.dinv;
  p.dead = L.dead;
  p.lamd = L.lamd;
  p.lexp = L.lexp;
  p.lam = nullptr;
  p.wf = L.wf;
  p.ebuf = L.ebuf;
  p.partials = reinterpret_cast<float*>(L.partials);
  p.status = ctx->status_dev;
  p.mstat = L.mstat;
  {
    // the factorisation and the quantization overlap: both are timed as GPTQ
    StageTimer t(ctx, CLHA_STAGE_GPTQ, s);
    st = run_factor(ctx, p, s, hj, evals.data());
  }
  if (st != CLHA_OK) return st;
  if (g_idx) {
    for (int i = 0; i < n_jobs; ++i) {
      if (!g_idx[i]) continue;
      if (p.gidx) {
        hipMemcpyAsync(g_idx[i], p.gidx + (size_t)js.mat_of[i] * cols, sizeof(int32_t) * cols,
                       hipMemcpyDeviceToDevice, s);
      } else {
        clha::launch_natural_gidx(g_idx[i], cols, group, s);
      }
    }
  }
  return hip_check(ctx, "gptq_quantize");
}

CLHA_API clha_status clha_gptq_quantize(clha_ctx* ctx, int32_t n_jobs, const clha_gptq_job* jobs,
                                        int32_t cols, int32_t group, int32_t block, float damp,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  return clha_gptq_quantize_ex(ctx, n_jobs, jobs, cols, group, block, damp, 0, nullptr, workspace,
                               workspace_bytes, stream);
}

CLHA_API size_t clha_inverse_cholesky_workspace_bytes(const clha_ctx* ctx, int32_t n, int32_t cols) {
  if (!ctx || n < 1 || cols < 1) return 0;
  return gptq_layout(nullptr, 0, n, cols, 0, 0, false, false).bytes;
}

CLHA_API clha_status clha_inverse_cholesky(clha_ctx* ctx, int32_t n, const float* const* H,
                                           int32_t cols, float damp, float* U_out,
                                           float* lambda_out, uint8_t* dead_out, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  if (!ctx) return CLHA_ERR_INVALID_ARG;
  if (n < 1 || !H || !U_out) return fail(ctx, CLHA_ERR_INVALID_ARG, "inverse_cholesky: bad arguments");
  if (cols < clha::kNb || cols > 8192 || cols % clha::kNb != 0)
    return fail(ctx, CLHA_ERR_SHAPE, "inverse_cholesky: cols must be a multiple of %d, <= 8192", clha::kNb);
  if (!std::isfinite(damp) || damp < 0.0f) return fail(ctx, CLHA_ERR_INVALID_ARG, "inverse_cholesky: bad damp");
  for (int i = 0; i < n; ++i)
    if (!H[i] || !aligned16(H[i])) return fail(ctx, CLHA_ERR_ALIGN, "inverse_cholesky: H[%d] null or misaligned", i);
  if (!aligned16(U_out) || !workspace || !aligned16(workspace))
    return fail(ctx, CLHA_ERR_ALIGN, "inverse_cholesky: misaligned output or workspace");
  const GptqLayout need = gptq_layout(nullptr, 0, n, cols, 0, 0, false, false);
  if (workspace_bytes < need.bytes)
    return fail(ctx, CLHA_ERR_WORKSPACE, "inverse_cholesky: workspace %zu < %zu bytes", workspace_bytes, need.bytes);
  const GptqLayout L = gptq_layout(workspace, 0, n, cols, 0, 0, false, false);
  const hipStream_t s = as_stream(stream);
  clha_status st = stage_to_device(ctx, L.mats, H, sizeof(float*) * n, s);
  if (st != CLHA_OK) return st;
  GptqPlan p;
  std::memset(&p, 0, sizeof p);
  p.n_mats = n;
  p.cols = cols;
  p.damp = damp;
  p.mats = L.mats;
  p.A = L.A;
  p.X = L.X;
  p.U = U_out;
  p.UT = nullptr;
  p.dinv = L.dinv;
  p.dead = dead_out ? dead_out : L.dead;
  p.lamd = L.lamd;
  p.lexp = L.lexp;
  p.lam = lambda_out;
  p.status = ctx->status_dev;
  p.mstat = L.mstat;
  {
    StageTimer t(ctx, CLHA_STAGE_FACTOR, s);
    st = run_factor(ctx, p, s, nullptr);
  }
  if (st != CLHA_OK) return st;
  return hip_check(ctx, "inverse_cholesky");
}

CLHA_API size_t clha_loss_workspace_bytes(const clha_ctx* ctx, int32_t rows, int32_t cols) {
  if (!ctx || rows < 1 || cols < 64) return 0;
  return up256((size_t)clha::loss_partial_count(rows, cols) * sizeof(double));
}

CLHA_API clha_status clha_loss(clha_ctx* ctx, int32_t rows, int32_t cols, int32_t group,
                               const void* W, int32_t w_dtype, const uint8_t* codes,
                               const float* scales, const uint8_t* zeros, const float* H,
                               float* loss_out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (!ctx) return CLHA_ERR_INVALID_ARG;
  if (rows < 1 || cols < 64 || cols > 8192 || cols % 64 != 0 || group < 1 || cols % group != 0)
    return fail(ctx, CLHA_ERR_SHAPE, "loss: bad shape");
  if (!W || !codes || !scales || !zeros || !H || !loss_out || !workspace)
    return fail(ctx, CLHA_ERR_INVALID_ARG, "loss: null pointer");
  if (w_dtype != CLHA_F32 && w_dtype != CLHA_BF16) return fail(ctx, CLHA_ERR_INVALID_ARG, "loss: bad dtype");
  if (!aligned16(W) || !aligned16(H) || !aligned4(scales) || !aligned4(loss_out) || !aligned16(workspace))
    return fail(ctx, CLHA_ERR_ALIGN, "loss: misaligned pointer");
  if (workspace_bytes < clha_loss_workspace_bytes(ctx, rows, cols))
    return fail(ctx, CLHA_ERR_WORKSPACE, "loss: workspace too small");
  {
    StageTimer t(ctx, CLHA_STAGE_LOSS, as_stream(stream));
    clha::launch_loss(rows, cols, group, W, w_dtype, codes, scales, zeros, H, nullptr,
                      static_cast<float*>(workspace), loss_out, as_stream(stream));
  }
  return hip_check(ctx, "loss");
}

CLHA_API clha_status clha_loss_static(clha_ctx* ctx, int32_t rows, int32_t cols, int32_t group,
                                      const void* W, int32_t w_dtype, const uint8_t* codes,
                                      const float* scales, const uint8_t* zeros, const float* H,
                                      float* loss_out, void* stream) {
  if (!ctx) return CLHA_ERR_INVALID_ARG;
  if (rows < 1 || cols < 64 || cols > 8192 || cols % 64 != 0 || group < 1 || cols % group != 0)
    return fail(ctx, CLHA_ERR_SHAPE, "loss_static: bad shape");
  if (!W || !codes || !scales || !zeros || !H || !loss_out)
    return fail(ctx, CLHA_ERR_INVALID_ARG, "loss_static: null pointer");
  if (w_dtype != CLHA_F32 && w_dtype != CLHA_BF16)
    return fail(ctx, CLHA_ERR_INVALID_ARG, "loss_static: bad dtype");
  if (!aligned16(W) || !aligned16(H) || !aligned4(scales) || !aligned4(loss_out))
    return fail(ctx, CLHA_ERR_ALIGN, "loss_static: misaligned pointer");
  const int64_t parts = clha::loss_partial_count(rows, cols);
  if (parts > clha::kLossScratchPartials)
    return fail(ctx, CLHA_ERR_WORKSPACE,
                "loss_static: %lld tile partials (rows %d, cols %d) exceed the static scratch of %lld "
                "(rows/64 rounded up times cols/64); use clha_loss with a workspace",
                (long long)parts, rows, cols, (long long)clha::kLossScratchPartials);
  double* scratch_ptr = clha::loss_scratch(ctx->device);
  if (!scratch_ptr) return fail(ctx, CLHA_ERR_HIP, "loss_static: no scratch address for device %d", ctx->device);
  {
    StageTimer t(ctx, CLHA_STAGE_LOSS, as_stream(stream));
    clha::launch_loss(rows, cols, group, W, w_dtype, codes, scales, zeros, H, nullptr,
                      reinterpret_cast<float*>(scratch_ptr), loss_out, as_stream(stream));
  }
  return hip_check(ctx, "loss_static");
}

CLHA_API clha_status clha_set_timing(clha_ctx* ctx, int32_t enable) {
  if (!ctx) return CLHA_ERR_INVALID_ARG;
  ctx->timing = enable != 0;
  return CLHA_OK;
}

CLHA_API clha_status clha_read_timing(clha_ctx* ctx, double* ms_out, int64_t* calls_out, int32_t n) {
  if (!ctx) return CLHA_ERR_INVALID_ARG;
  if (n < 0 || n > CLHA_NUM_STAGES) return fail(ctx, CLHA_ERR_SHAPE, "read_timing: n must be 0..%d", CLHA_NUM_STAGES);
  clha_status st = CLHA_OK;
  for (auto& r : ctx->recs) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      st = fail(ctx, CLHA_ERR_HIP, "read_timing: event query failed");
    if (r.stage < n) {
      if (ms_out) ms_out[r.stage] += ms;
      if (calls_out) calls_out[r.stage] += 1;
    }
    ctx->free_events.push_back(r.a);
    ctx->free_events.push_back(r.b);
  }
  ctx->recs.clear();
  return st;
}

CLHA_API clha_status clha_sync(clha_ctx* ctx, void* stream) {
  if (!ctx) return CLHA_ERR_INVALID_ARG;
  const hipStream_t s = as_stream(stream);
  uint32_t rec[clha::kStatusWords] = {};
  if (hipMemcpyAsync(rec, ctx->status_dev, sizeof rec, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return fail(ctx, CLHA_ERR_HIP, "sync: %s", hipGetErrorString(hipGetLastError()));
  if (ctx->pinned_pending) {
    hipEventSynchronize(ctx->pinned_done);
    ctx->pinned_pending = false;
  }
  if (rec[0] == 0) return CLHA_OK;
  if (hipMemsetAsync(ctx->status_dev, 0, sizeof rec, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess)
    return fail(ctx, CLHA_ERR_HIP, "sync: could not clear the status record");
  std::string where;
  char buf[96];
  if (rec[clha::kStatusJob]) {
    snprintf(buf, sizeof buf, "GPTQ job %u", 0xffffffffu - rec[clha::kStatusJob]);
    where += buf;
  }
  if (rec[clha::kStatusMat]) {
    snprintf(buf, sizeof buf, "%sHessian %u", where.empty() ? "" : ", ", 0xffffffffu - rec[clha::kStatusMat]);
    where += buf;
  }
  const uint64_t lay = (uint64_t)rec[clha::kStatusLayer] | ((uint64_t)rec[clha::kStatusLayer + 1] << 32);
  if (rec[0] & clha::kStatusNonfinite) {
    if (lay >> 32)
      return fail(ctx, CLHA_ERR_NONFINITE, "layer %d: a router logit was NaN or infinite%s%s",
                  (int32_t)(uint32_t)lay, where.empty() ? "" : "; also ", where.c_str());
    return fail(ctx, CLHA_ERR_NONFINITE, "%s: a Hessian diagonal entry was NaN or infinite", where.c_str());
  }
  return fail(ctx, CLHA_ERR_NOT_PD, "%s: the damped Hessian is not positive definite", where.c_str());
}

static clha_status check_pack(clha_ctx* ctx, const char* what, int64_t n_codes, int32_t bits, const void* a,
                              const void* b) {
  if (n_codes < 0 || n_codes % 8 != 0)
    return fail(ctx, CLHA_ERR_SHAPE, "%s: n_codes %lld must be a multiple of 8", what, (long long)n_codes);
  if (bits < 2 || bits > 8) return fail(ctx, CLHA_ERR_SHAPE, "%s: bits %d outside 2..8", what, bits);
  if (n_codes == 0) return CLHA_OK;
  if (!a || !b) return fail(ctx, CLHA_ERR_INVALID_ARG, "%s: null pointer", what);
  return CLHA_OK;
}

CLHA_API clha_status clha_pack_codes(clha_ctx* ctx, int64_t n_codes, int32_t bits, const uint8_t* codes,
                                     uint8_t* packed, void* stream) {
  if (!ctx) return CLHA_ERR_INVALID_ARG;
  const clha_status st = check_pack(ctx, "pack_codes", n_codes, bits, codes, packed);
  if (st != CLHA_OK || n_codes == 0) return st;
  if (!aligned16(codes)) return fail(ctx, CLHA_ERR_ALIGN, "pack_codes: codes not 16-byte aligned");
  clha::launch_pack_codes(codes, packed, n_codes, bits, as_stream(stream));
  return hip_check(ctx, "pack_codes");
}

CLHA_API clha_status clha_unpack_codes(clha_ctx* ctx, int64_t n_codes, int32_t bits, const uint8_t* packed,
                                       uint8_t* codes, void* stream) {
  if (!ctx) return CLHA_ERR_INVALID_ARG;
  const clha_status st = check_pack(ctx, "unpack_codes", n_codes, bits, packed, codes);
  if (st != CLHA_OK || n_codes == 0) return st;
  if (!aligned16(codes)) return fail(ctx, CLHA_ERR_ALIGN, "unpack_codes: codes not 16-byte aligned");
  clha::launch_unpack_codes(packed, codes, n_codes, bits, as_stream(stream));
  return hip_check(ctx, "unpack_codes");
}

CLHA_API size_t clha_down_workspace_bytes(const clha_ctx* ctx, int32_t n_routed) {
  if (!ctx || n_routed < 1 || n_routed > ctx->slots) return 0;
  return down_layout(ctx, n_routed, nullptr).bytes;
}

CLHA_API clha_status clha_collect_down_hessians(clha_ctx* ctx, int32_t layer, int64_t n_tokens, int32_t d_model,
                                                int32_t n_routed, const uint16_t* x, const int32_t* token_ids,
                                                const int64_t* offsets, const uint16_t* const* wgu,
                                                void* workspace, size_t workspace_bytes, void* stream) {
  if (!ctx) return CLHA_ERR_INVALID_ARG;
  auto it = ctx->layers.find(layer);
  if (it == ctx->layers.end())
    return fail(ctx, CLHA_ERR_INVALID_ARG, "collect_down_hessians: layer %d is not registered", layer);
  const clha_moe_desc& d = ctx->desc;
  if (d.n_shared != 0)
    return fail(ctx, CLHA_ERR_INVALID_ARG, "collect_down_hessians: a down_proj context has no shared slot "
                "(one slot per routed and per shared expert)");
  if (n_routed < 1 || n_routed > ctx->slots)
    return fail(ctx, CLHA_ERR_SHAPE, "collect_down_hessians: n_routed %d outside 1..%d", n_routed, ctx->slots);
  if (d_model < 64 || d_model > 8192 || d_model % 64 != 0)
    return fail(ctx, CLHA_ERR_SHAPE, "collect_down_hessians: d_model %d must be a multiple of 64, <= 8192", d_model);
  if (n_tokens < 0 || n_tokens > d.max_tokens)
    return fail(ctx, CLHA_ERR_SHAPE, "collect_down_hessians: n_tokens %lld outside 0..%lld",
                (long long)n_tokens, (long long)d.max_tokens);
  if (n_tokens == 0) return CLHA_OK;   // an empty batch adds nothing; its pointers are not read
  if (!x || !token_ids || !offsets || !wgu || !workspace)
    return fail(ctx, CLHA_ERR_INVALID_ARG, "collect_down_hessians: null pointer");
  if (!aligned16(x) || !aligned4(token_ids) || !aligned16(offsets) || !aligned16(workspace))
    return fail(ctx, CLHA_ERR_ALIGN, "collect_down_hessians: misaligned pointer");
  for (int e = 0; e < ctx->slots; ++e)
    if (!wgu[e] || !aligned16(wgu[e]))
      return fail(ctx, CLHA_ERR_ALIGN, "collect_down_hessians: weights of slot %d null or misaligned", e);
  const DownLayout need = down_layout(ctx, n_routed, nullptr);
  if (workspace_bytes < need.bytes)
    return fail(ctx, CLHA_ERR_WORKSPACE, "collect_down_hessians: workspace %zu < %zu bytes", workspace_bytes,
                need.bytes);
  const DownLayout L = down_layout(ctx, n_routed, workspace);
  const hipStream_t s = as_stream(stream);
  clha_status st = stage_to_device(ctx, L.wgu, wgu, sizeof(const uint16_t*) * ctx->slots, s);
  if (st != CLHA_OK) return st;
  CollectPlan p;
  std::memset(&p, 0, sizeof p);
  p.n_tokens = n_tokens;
  p.d = d.d;
  p.E = ctx->slots;
  p.K = d.top_k;
  p.has_shared = 0;
  p.pad_off = L.pad_off;
  p.slot_order = L.slot_order;
  p.work = L.work;
  p.work_len = L.work_len;
  p.work_next = L.work_next;
  p.seg = L.seg;
  p.split = L.split;
  p.partials = L.partials;
  p.max_partials = L.max_partials;
  p.max_segs = ctx->slots + L.max_partials;
  p.syrk_items = clha::syrk_items_per_slot(d.d);
  p.overwrite = it->second.fresh ? 1 : 0;
  p.xgT = L.hT;
  p.status = ctx->status_dev;
  p.layer = layer;
  // token tiles of 128 over all slots, at most one partial tile per slot
  const int64_t max_tiles = (n_tokens * d.top_k + (int64_t)(ctx->slots - n_routed) * n_tokens +
                             (int64_t)clha::kTokPad * ctx->slots) / 128 + ctx->slots + 1;
  {
    StageTimer t(ctx, CLHA_STAGE_BUCKET, s);
    clha::launch_down_scan(offsets, n_tokens, n_routed, p, it->second.counts, L.tile_off, s);
  }
  {
    StageTimer t(ctx, CLHA_STAGE_GATHER, s);
    clha::launch_down_gemm(x, d_model, token_ids, offsets, n_routed, n_tokens, L.wgu, p, L.tile_off, max_tiles, s);
  }
  {
    StageTimer t(ctx, CLHA_STAGE_SYRK, s);
    clha::launch_syrk(p, it->second.S, s);
  }
  {
    StageTimer t(ctx, CLHA_STAGE_SYRK_REDUCE, s);
    clha::launch_syrk_reduce(p, it->second.S, it->second.counts, s);
  }
  it->second.fresh = false;
  return hip_check(ctx, "collect_down_hessians");
}

}  // extern "C"
