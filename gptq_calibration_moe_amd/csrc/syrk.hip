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
// the operands and each load has three steps of products to arrive.  Each wave
// waits for its own loads of the step (vmcnt) and one barrier per step
// publishes them.  Two operand sources:
//   rows (the collection): a step's operand panel is 32 token rows of x, 512
//     bytes each (256 features), fetched through the slot's token list, so
//     the activations are read where they lie, with no gathered copy; the
//     fragments come from transposing LDS reads (see the rows layout below);
//   blocked (the down_proj inputs, which a GEMM writes in this form): 32-token
//     blocks [d features][32 tokens], so a panel (256 features x 32 tokens) is
//     one contiguous 16 KB run; a lane's MFMA fragment (8 consecutive tokens of
//     one feature) is one 16-byte chunk, and the four chunks of row r sit at
//     slots c ^ ((r >> 2) & 3), which makes the fragment reads bank-conflict
//     free.
//   off-diagonal tile (ti, tj): waves in 2x4, each 128x64 as 4x2 32x32 blocks;
//   diagonal pair (p, q): waves 0-3 take panel p, waves 4-7 panel q; wave k of a
//     panel owns block rows 7-k and k (9 blocks), both operands from that panel.
#include "kernels.h"

namespace clha {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kT = 256;              // output tile
constexpr int kSK = 32;              // tokens per step
constexpr int kFlushSteps = 512;     // 16384 tokens between partial-sum flushes (multiple of kStages)
constexpr int kStages = 4;           // LDS stages; loads run kStages - 1 steps ahead
constexpr int kPanel = kT * kSK;     // one operand stage: 256 rows x 32 tokens (bf16 elements)

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef const __attribute__((address_space(1))) void* glb_ptr;

// The LDS stages, one array each so that the compiler can tell a stage being
// loaded from a stage being read.
struct Stages {
  uint16_t* a[kStages];
  uint16_t* b[kStages];
  int32_t* ids;          // rows layout: tokens of 8 steps (ring), 32 per step
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

// Where a segment's operands come from.  Blocked: the slot's gathered 32-token
// blocks ([d][32] each, see the layout note above).  Rows: the activations
// themselves, row t of x for token t, through the slot's token list.
struct Src {
  const uint16_t* blocks;   // blocked layout: the slot's first block (nullptr: rows)
  const uint16_t* x;        // rows: [n][d]
  const int32_t* ids;       // rows: the slot's token list (the shared slot: 0, 1, .., n-1)
  const uint16_t* zero;     // rows: d zeros, the operand of a padding position
  int64_t cnt;              // rows: tokens of the slot; positions from cnt on are padding
};

// Rows layout of a stage: 32 token rows of 512 bytes (256 features); the
// 16-byte slot of features 8s .. 8s+7 of row r sits at s ^ 4(r % 4).  A lane's
// MFMA fragment (8 consecutive tokens of one feature) comes from two
// transposing LDS reads, ds_read_b64_tr_b16: within each 16-lane group, lane i
// reads 4 consecutive bf16 at its own address and lane j receives element j % 4
// of the reads of lanes j/4, 4 + j/4, 8 + j/4, 12 + j/4 (measured on gfx950).
// So lane i = 4k + a of group G points at token row 16kk + 8(G/2) + 4h + k,
// features fr + 16(G%2) + 4a; lane 16G + j then holds feature fr + 16(G%2) + j
// of tokens 16kk + 8(G/2) + 4h .. +3, which is half (h) of the fragment of
// MFMA lane 16G + j for token step kk.  The eight rows one read touches fall on
// four distinct 64-byte bank windows, two rows each (the swizzle), which is the
// least the 512 bytes allow.
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s* lds_v4s;

// This lane's part of the address of its first transposing read: token row
// 8(G/2) + k, byte 32(G%2) + 16((i%4)/2) + 8(i%2) of the 64-byte group, and
// the group swizzle k in bits 6..8.  The read of features fr .. fr+31 (fr a
// multiple of 32) for token step kk in a stage at LDS byte address B (a
// multiple of 512) is at (B + lane part + 8192 kk) ^ 2fr: 2fr = 64(fr/32)
// sets the group, and the XOR with k's bits gives its swizzled place.
__device__ __forceinline__ uint32_t tr_lane(int lane) {
  const int G = lane >> 4, i = lane & 15, k = i >> 2;
  return (uint32_t)((8 * (G >> 1) + k) * 512 + 64 * k + 32 * (G & 1) + 16 * ((i & 3) >> 1) + 8 * (i & 1));
}

// Batched transposing reads: fragment f (features of one 32-block, one token
// step) from the LDS byte address addr[f] (its first read; the second is 4
// rows, 2048 bytes, further).  All reads of a batch are issued together and
// waited for in the same asm statement.  (The compiler's own form of this read
// is not known to stay clear of the stages the direct global-to-LDS loads are
// filling, so before each one it waits for every load in flight.)
typedef int v2i __attribute__((ext_vector_type(2)));
template <int N>
__device__ __forceinline__ void tr_batch(bf16x8 (&out)[N], const uint32_t (&addr)[N]);
template <>
__device__ __forceinline__ void tr_batch<5>(bf16x8 (&out)[5], const uint32_t (&addr)[5]) {
  v2i r[10];
  asm volatile(
        "ds_read_b64_tr_b16 %0, %10\n"
        "ds_read_b64_tr_b16 %1, %10 offset:2048\n"
        "ds_read_b64_tr_b16 %2, %11\n"
        "ds_read_b64_tr_b16 %3, %11 offset:2048\n"
        "ds_read_b64_tr_b16 %4, %12\n"
        "ds_read_b64_tr_b16 %5, %12 offset:2048\n"
        "ds_read_b64_tr_b16 %6, %13\n"
        "ds_read_b64_tr_b16 %7, %13 offset:2048\n"
        "ds_read_b64_tr_b16 %8, %14\n"
        "ds_read_b64_tr_b16 %9, %14 offset:2048\n"
        "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4])
      : "memory");
#pragma unroll
  for (int f = 0; f < 5; ++f) {
    const v2i v[2] = {r[2 * f], r[2 * f + 1]};
    out[f] = __builtin_bit_cast(bf16x8, v);
  }
}
template <>
__device__ __forceinline__ void tr_batch<6>(bf16x8 (&out)[6], const uint32_t (&addr)[6]) {
  v2i r[12];
  asm volatile(
        "ds_read_b64_tr_b16 %0, %12\n"
        "ds_read_b64_tr_b16 %1, %12 offset:2048\n"
        "ds_read_b64_tr_b16 %2, %13\n"
        "ds_read_b64_tr_b16 %3, %13 offset:2048\n"
        "ds_read_b64_tr_b16 %4, %14\n"
        "ds_read_b64_tr_b16 %5, %14 offset:2048\n"
        "ds_read_b64_tr_b16 %6, %15\n"
        "ds_read_b64_tr_b16 %7, %15 offset:2048\n"
        "ds_read_b64_tr_b16 %8, %16\n"
        "ds_read_b64_tr_b16 %9, %16 offset:2048\n"
        "ds_read_b64_tr_b16 %10, %17\n"
        "ds_read_b64_tr_b16 %11, %17 offset:2048\n"
        "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5])
      : "memory");
#pragma unroll
  for (int f = 0; f < 6; ++f) {
    const v2i v[2] = {r[2 * f], r[2 * f + 1]};
    out[f] = __builtin_bit_cast(bf16x8, v);
  }
}
template <>
__device__ __forceinline__ void tr_batch<7>(bf16x8 (&out)[7], const uint32_t (&addr)[7]) {
  v2i r[14];
  asm volatile(
        "ds_read_b64_tr_b16 %0, %14\n"
        "ds_read_b64_tr_b16 %1, %14 offset:2048\n"
        "ds_read_b64_tr_b16 %2, %15\n"
        "ds_read_b64_tr_b16 %3, %15 offset:2048\n"
        "ds_read_b64_tr_b16 %4, %16\n"
        "ds_read_b64_tr_b16 %5, %16 offset:2048\n"
        "ds_read_b64_tr_b16 %6, %17\n"
        "ds_read_b64_tr_b16 %7, %17 offset:2048\n"
        "ds_read_b64_tr_b16 %8, %18\n"
        "ds_read_b64_tr_b16 %9, %18 offset:2048\n"
        "ds_read_b64_tr_b16 %10, %19\n"
        "ds_read_b64_tr_b16 %11, %19 offset:2048\n"
        "ds_read_b64_tr_b16 %12, %20\n"
        "ds_read_b64_tr_b16 %13, %20 offset:2048\n"
        "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6])
      : "memory");
#pragma unroll
  for (int f = 0; f < 7; ++f) {
    const v2i v[2] = {r[2 * f], r[2 * f + 1]};
    out[f] = __builtin_bit_cast(bf16x8, v);
  }
}
template <>
__device__ __forceinline__ void tr_batch<8>(bf16x8 (&out)[8], const uint32_t (&addr)[8]) {
  v2i r[16];
  asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n"
        "ds_read_b64_tr_b16 %1, %16 offset:2048\n"
        "ds_read_b64_tr_b16 %2, %17\n"
        "ds_read_b64_tr_b16 %3, %17 offset:2048\n"
        "ds_read_b64_tr_b16 %4, %18\n"
        "ds_read_b64_tr_b16 %5, %18 offset:2048\n"
        "ds_read_b64_tr_b16 %6, %19\n"
        "ds_read_b64_tr_b16 %7, %19 offset:2048\n"
        "ds_read_b64_tr_b16 %8, %20\n"
        "ds_read_b64_tr_b16 %9, %20 offset:2048\n"
        "ds_read_b64_tr_b16 %10, %21\n"
        "ds_read_b64_tr_b16 %11, %21 offset:2048\n"
        "ds_read_b64_tr_b16 %12, %22\n"
        "ds_read_b64_tr_b16 %13, %22 offset:2048\n"
        "ds_read_b64_tr_b16 %14, %23\n"
        "ds_read_b64_tr_b16 %15, %23 offset:2048\n"
        "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]), "v"(addr[7])
      : "memory");
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const v2i v[2] = {r[2 * f], r[2 * f + 1]};
    out[f] = __builtin_bit_cast(bf16x8, v);
  }
}

// LDS byte address of a stage pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One int from LDS, waited for in the same asm statement (for the same reason).
__device__ __forceinline__ int lds_read_i32(uint32_t addr) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n s_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(addr) : "memory");
  return v;
}

// The fragments of N 32-feature blocks (first features fr[f]) for token step
// kk from stage P: one 16-byte read each (blocked), or a batch of transposing
// reads (rows).
template <bool kRows, int N>
__device__ __forceinline__ void frags(const char* P, const int (&fr)[N], int kk, int lane, bf16x8 (&out)[N]) {
  if constexpr (kRows) {
    uint32_t x = lds_addr(P) + tr_lane(lane) + 8192 * kk;
    asm volatile("" : "+v"(x));   // formed here, not hoisted out of the token loop
    uint32_t addr[N];
#pragma unroll
    for (int f = 0; f < N; ++f) addr[f] = x ^ (uint32_t)(2 * fr[f]);
    tr_batch<N>(out, addr);
  } else {
#pragma unroll
    for (int f = 0; f < N; ++f)
      out[f] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(P + chunk_off(fr[f] + (lane & 31), 2 * kk + (lane >> 5))));
  }
}

// The off-diagonal tile's fragments: 4 blocks of stage A and 2 of stage B, one
// batch.
template <bool kRows>
__device__ __forceinline__ void frags2(const char* A, const int (&fa)[4], const char* B, const int (&fb)[2], int kk,
                                       int lane, bf16x8 (&a)[4], bf16x8 (&b)[2]) {
  if constexpr (kRows) {
    uint32_t xa = lds_addr(A) + tr_lane(lane) + 8192 * kk, xb = lds_addr(B) + tr_lane(lane) + 8192 * kk;
    asm volatile("" : "+v"(xa), "+v"(xb));   // formed here, not hoisted out of the token loop
    const uint32_t addr[6] = {xa ^ (uint32_t)(2 * fa[0]), xa ^ (uint32_t)(2 * fa[1]), xa ^ (uint32_t)(2 * fa[2]),
                              xa ^ (uint32_t)(2 * fa[3]), xb ^ (uint32_t)(2 * fb[0]), xb ^ (uint32_t)(2 * fb[1])};
    bf16x8 o[6];
    tr_batch<6>(o, addr);
#pragma unroll
    for (int f = 0; f < 4; ++f) a[f] = o[f];
    b[0] = o[4];
    b[1] = o[5];
  } else {
    frags<false, 4>(A, fa, kk, lane, a);
    frags<false, 2>(B, fb, kk, lane, b);
  }
}

// The token pipeline shared by both item kinds, for panels pa and pb (pb only
// when loadB); t0, a multiple of kSK, is the segment's first position.
// multiply(stage) runs one 32-token step from LDS stage `stage`; flush(first)
// adds the running sums.  Steps past nsteps are padding: their loads re-read
// the last step (clamped, always in range) and they run no products, so every
// wave issues the same loads, waits and barriers.
template <bool kRows, class Mul, class Flush>
__device__ __forceinline__ void token_loop(const Src& src, int pa, int pb, int d, int64_t t0, int64_t nsteps,
                                           bool loadB, const Stages& sb, Mul&& multiply, Flush&& flush) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (!loadB) pb = pa;
  // blocked: wave w loads 1 KB blocks 2w and 2w+1 of each panel: 16 rows x 4
  // chunks, lane l -> row 16 blk + l/4, LDS slot l%4 (holding chunk slot ^
  // ((row>>2)&3)).  rows: the same 1 KB blocks are token rows 4w + 2j and
  // 4w + 2j + 1, lane l -> row 4w + 2j + l/32, LDS slot l%32 (holding feature
  // slot (l%32) ^ 4(row % 4), clamped to the matrix).
  const uint16_t* pa_[2] = {nullptr, nullptr};
  const uint16_t* pb_[2] = {nullptr, nullptr};
  int col_a[2] = {0, 0}, col_b[2] = {0, 0};
  const int64_t bstride = (int64_t)d * kSK;
  if constexpr (kRows) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 2 * j + (lane >> 5);   // row within the wave's four (r % 4 = the row's swizzle)
      const int ls = (lane & 31) ^ (4 * r);
      const int fa = pa * kT, fb = pb * kT;
      col_a[j] = fa + 8 * min(ls, (d - fa) / 8 - 1);
      col_b[j] = fb + 8 * min(ls, (d - fb) / 8 - 1);
    }
  } else {
    const int arows = min(kT, d - pa * kT), brows = min(kT, d - pb * kT);
    const uint16_t* Ag = src.blocks + (int64_t)pa * kT * kSK;
    const uint16_t* Bg = src.blocks + (int64_t)pb * kT * kSK;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = 16 * (2 * wave + j) + (lane >> 2);
      const int c = (lane & 3) ^ ((row >> 2) & 3);
      pa_[j] = Ag + (int64_t)min(row, arows - 1) * kSK + (t0 / kSK) * bstride + c * 8;
      pb_[j] = Bg + (int64_t)min(row, brows - 1) * kSK + (t0 / kSK) * bstride + c * 8;
    }
  }
  // rows: the token of each row of a step comes from the slot's list, copied
  // by each wave for its own four rows straight into LDS (a ring of 8 steps,
  // 32 tokens each) seven steps ahead, with the same direct global-to-LDS loads
  // as the activations, and read back where the row address is formed.  (A
  // list load into registers would make the compiler wait for the whole memory
  // counter before its first use, draining the activation loads in flight.)
  // Positions from cnt on are padding; their list load is clamped into the list
  // and their activation row is `zero`.
  auto row_pos = [&](int64_t st, int j) {
    const int64_t s1 = st < nsteps ? st : nsteps - 1;
    return t0 + s1 * kSK + 4 * wave + 2 * j + (lane >> 5);
  };
  auto load_ids = [&](int64_t st) {
    if constexpr (kRows) {
      if (lane < 4) {
        const int64_t s1 = st < nsteps ? st : nsteps - 1;
        const int64_t pos = t0 + s1 * kSK + 4 * wave + lane;
        __builtin_amdgcn_global_load_lds((glb_ptr)(src.ids + (pos < src.cnt ? pos : src.cnt - 1)),
                                         (lds_ptr)(sb.ids + (st & 7) * kSK + 4 * wave), 4, 0, 0);
      }
    }
  };
  auto issue = [&](int stage, int64_t st) {
    if constexpr (kRows) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int tk = lds_read_i32(lds_addr(sb.ids + (st & 7) * kSK + 4 * wave + 2 * j + (lane >> 5)));
        const uint16_t* row = row_pos(st, j) < src.cnt ? src.x + (int64_t)tk * d : src.zero;
        __builtin_amdgcn_global_load_lds((glb_ptr)(row + col_a[j]), (lds_ptr)(sb.a[stage] + (2 * wave + j) * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((glb_ptr)(row + col_b[j]), (lds_ptr)(sb.b[stage] + (2 * wave + j) * 512), 16, 0, 0);
      }
    } else {
      const int64_t k0 = (st < nsteps ? st : nsteps - 1) * bstride;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        __builtin_amdgcn_global_load_lds((glb_ptr)(pa_[j] + k0), (lds_ptr)(sb.a[stage] + (2 * wave + j) * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((glb_ptr)(pb_[j] + k0), (lds_ptr)(sb.b[stage] + (2 * wave + j) * 512), 16, 0, 0);
      }
    }
  };
  // One step: this wave's loads for stage `stage` are done once at most the
  // memory operations issued after them are outstanding: the loads of the
  // (kStages - 2) later steps, 4 per step, and under the rows layout each
  // step's list copy as well (the batch after each step's products is: list of
  // step st + 7, then activations of step st + 3, so a step's list has landed
  // once the activations of the step before it have).  The loads for
  // kStages - 1 steps ahead go into the stage every wave finished reading
  // before this step's barrier, and are issued after this step's products:
  // issued first, a wave waits for the address unit to take them before it
  // starts its products (measured: 8.38 to 8.05 ms per full-depth launch)
  constexpr int kAfter = (kRows ? 5 : 4) * (kStages - 2);
  auto step = [&](auto stage_c, int64_t st) {
    constexpr int stage = decltype(stage_c)::value;
    wait_loads<kAfter>();
    __builtin_amdgcn_s_barrier();
    if (st < nsteps) multiply(stage);
    load_ids(st + 7);
    __builtin_amdgcn_sched_barrier(0);
    issue((stage + kStages - 1) % kStages, st + kStages - 1);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int64_t c0 = 0; c0 < nsteps; c0 += kFlushSteps) {
    // restart the pipeline (all earlier loads and stores drained)
    wait_loads<0>();
    __builtin_amdgcn_s_barrier();
    if constexpr (kRows) {
      // lists of steps c0 .. c0 + 3, then the batches of steps c0 - 3 .. c0 - 1
#pragma unroll
      for (int j = 0; j < 4; ++j) load_ids(c0 + j);
      wait_loads<0>();
#pragma unroll
      for (int j = 0; j < kStages - 1; ++j) {
        load_ids(c0 + 4 + j);
        __builtin_amdgcn_sched_barrier(0);
        issue(j, c0 + j);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kStages - 1; ++j) issue(j, c0 + j);
    }
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
template <bool kRows>
__device__ __forceinline__ void syrk_offdiag(const Src& src, int64_t t0, int64_t nsteps, int d, int ti, int tj,
                                             float* Sd, bool partial, const Stages& sb) {
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
      bf16x8 a[4], b[2];
      frags2<kRows>(As, {wm * 128, wm * 128 + 32, wm * 128 + 64, wm * 128 + 96}, Bs, {wn * 64, wn * 64 + 32}, kk,
                    lane, a, b);
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
  token_loop<kRows>(src, ti, tj, d, t0, nsteps, true, sb, multiply, flush);
}

// Diagonal pair: this wave's share of panel P's diagonal tile -- block rows
// 7-K (columns 0..7-K) and K (columns 0..K) -- read from LDS buffer half `pb`.
template <bool kRows, int K>
__device__ __forceinline__ void syrk_diag_wave(const Src& src, int p, int q, bool loadB, int64_t t0,
                                               int64_t nsteps, int d, int P, int pb, bool active, float* Sd,
                                               bool partial, const Stages& sb) {
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
      bf16x8 f[NA];
      int fr[NA];
#pragma unroll
      for (int cb = 0; cb < NA; ++cb) fr[cb] = cb * 32;
      frags<kRows, NA>(Ps, fr, kk, lane, f);
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
  token_loop<kRows>(src, p, q, d, t0, nsteps, loadB, sb, multiply, flush);
}

__device__ __forceinline__ void tile_of(int t, int& ti, int& tj) {
  int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  while (i * (i + 1) / 2 > t) --i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

// Operands of the Gram sums: the gathered blocks (xgT, pad_off), or the
// activations through the token lists (x, ids with offsets; the shared slot's
// list is `iota`; zero: d zeros).
struct GramIn {
  const uint16_t* xgT;
  const int64_t* pad_off;
  const uint16_t* x;
  const int32_t* token_ids;
  const int64_t* offsets;
  const int32_t* iota;
  const uint16_t* zero;
  int64_t n;
  int E;
};

// One item of one segment.
template <bool kRows>
__device__ __forceinline__ void syrk_item(const GramIn& in, const int32_t* __restrict__ seg, int sg, int item, int d,
                                          float* __restrict__ S, float* __restrict__ partials, bool overwrite,
                                          const Stages& sb) {
  const int slot = seg[4 * sg], dest = seg[4 * sg + 1];
  const int64_t t0 = seg[4 * sg + 2], ntok = seg[4 * sg + 3];
  Src src;
  if constexpr (kRows) {
    src.blocks = nullptr;
    src.x = in.x;
    src.zero = in.zero;
    if (slot < in.E) {
      src.ids = in.token_ids + in.offsets[slot];
      src.cnt = in.offsets[slot + 1] - in.offsets[slot];
    } else {
      src.ids = in.iota;
      src.cnt = in.n;
    }
  } else {
    src.blocks = in.xgT + in.pad_off[slot] * d;
  }
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
    syrk_offdiag<kRows>(src, t0, nsteps, d, a + 1, b, Sd, partial, sb);
    return;
  }
  const int p = item, q = nt - 1 - item;
  const bool single = p == q;
  const int wave = threadIdx.x >> 6, hp = wave >> 2, k = wave & 3;
  const int P = hp ? q : p;
  const bool active = !(hp && single);
  switch (k) {
    case 0: syrk_diag_wave<kRows, 0>(src, p, q, !single, t0, nsteps, d, P, hp, active, Sd, partial, sb); break;
    case 1: syrk_diag_wave<kRows, 1>(src, p, q, !single, t0, nsteps, d, P, hp, active, Sd, partial, sb); break;
    case 2: syrk_diag_wave<kRows, 2>(src, p, q, !single, t0, nsteps, d, P, hp, active, Sd, partial, sb); break;
    default: syrk_diag_wave<kRows, 3>(src, p, q, !single, t0, nsteps, d, P, hp, active, Sd, partial, sb); break;
  }
}

// Persistent workgroups, kSyrkWgPerXcd per die: workgroup b runs on die b % 8
// and takes items from that die's list until the list is exhausted.
template <bool kRows>
__global__ __launch_bounds__(512) void syrk_kernel(GramIn in, const int32_t* __restrict__ work,
                                                   const int32_t* __restrict__ work_len,
                                                   int32_t* __restrict__ work_next,
                                                   const int32_t* __restrict__ seg, int cap, int d,
                                                   float* __restrict__ S, float* __restrict__ partials,
                                                   int overwrite) {
  // (512-byte aligned: the transposing reads' addresses are formed by XOR below bit 9)
  __shared__ __attribute__((aligned(1024))) uint16_t a0[kPanel], a1[kPanel], a2[kPanel], a3[kPanel];
  __shared__ __attribute__((aligned(1024))) uint16_t b0[kPanel], b1[kPanel], b2[kPanel], b3[kPanel];
  __shared__ __attribute__((aligned(16))) int32_t ids[8 * kSK];
  __shared__ int item;
  const Stages sb{{a0, a1, a2, a3}, {b0, b1, b2, b3}, ids};
  const int x = blockIdx.x % kXcds;
  const int len = work_len[x];
  for (;;) {
    if (threadIdx.x == 0) item = atomicAdd(&work_next[x], 1);
    __syncthreads();
    const int it = item;
    __syncthreads();
    if (it >= len) break;
    const int code = work[x * cap + it];
    syrk_item<kRows>(in, seg, code >> 10, code & 1023, d, S, partials, overwrite != 0, sb);
  }
}

// S[slot] (lower triangle) += the partial sums of each token-split slot, in
// part order.  Workgroup (x, i, z): row i, columns 1024x .. +1023 (four per
// thread), split slots z, z + kReduceGroups, ...
constexpr int kReduceGroups = 8;
__global__ __launch_bounds__(256) void syrk_reduce_kernel(const int32_t* __restrict__ split,
                                                          const float* __restrict__ partials,
                                                          float* __restrict__ S, int d) {
  const int nsplit = split[0];
  const int i = blockIdx.y, j = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (j > i || j >= d) return;
  const int64_t dd = (int64_t)d * d, off = (int64_t)i * d + j;
  for (int sp = blockIdx.z; sp < nsplit; sp += kReduceGroups) {
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

// The shared slot's sums from the routed slots' (CLHA summary, section 2.2:
// a shared expert's Hessian is accumulated over every token).  Top-K routing
// sends each token to exactly K distinct routed experts, so
//   sum_e S_e = sum_e sum_{t -> e} x_t x_t^T = K sum_t x_t x_t^T = K S_shared:
// S_E = (sum_e S_e) / K, summed in fp64 in slot order and rounded once, for
// the lower triangle.  The routed sums are cumulative over a layer's batches,
// so S_E is formed anew after each batch.  Workgroup (x, i): row i, columns
// 1024x .. +1023, four per thread.
__global__ __launch_bounds__(256) void shared_from_routed_kernel(float* __restrict__ S, int E, int K, int d) {
  const int i = blockIdx.y, j = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (j > i || j >= d) return;
  const int64_t dd = (int64_t)d * d, off = (int64_t)i * d + j;
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  int e = 0;
  // eight slots' loads in flight together; the sums stay in slot order
  for (; e + 8 <= E; e += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4*>(S + (int64_t)(e + u) * dd + off);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a0 += (double)v[u].x;
      a1 += (double)v[u].y;
      a2 += (double)v[u].z;
      a3 += (double)v[u].w;
    }
  }
  for (; e < E; ++e) {
    const float4 v = *reinterpret_cast<const float4*>(S + (int64_t)e * dd + off);
    a0 += (double)v.x;
    a1 += (double)v.y;
    a2 += (double)v.z;
    a3 += (double)v.w;
  }
  float* o = S + (int64_t)E * dd + off;
  float4 r = make_float4((float)(a0 / K), (float)(a1 / K), (float)(a2 / K), (float)(a3 / K));
  // columns above the diagonal keep their value (S's upper triangle is never written)
  if (j + 1 > i) r.y = o[1];
  if (j + 2 > i) r.z = o[2];
  if (j + 3 > i) r.w = o[3];
  *reinterpret_cast<float4*>(o) = r;
}

void launch_syrk(const CollectPlan& p, float* S, hipStream_t s) {
  GramIn in{p.xgT, p.pad_off, p.x_rows, p.token_ids, p.offsets, p.iota, p.zero_row, p.n_tokens, p.E};
  if (p.x_rows)
    hipLaunchKernelGGL(syrk_kernel<true>, dim3(kXcds * kSyrkWgPerXcd), dim3(512), 0, s, in, p.work, p.work_len,
                       p.work_next, p.seg, p.max_segs * p.syrk_items, p.d, S, p.partials, p.overwrite);
  else
    hipLaunchKernelGGL(syrk_kernel<false>, dim3(kXcds * kSyrkWgPerXcd), dim3(512), 0, s, in, p.work, p.work_len,
                       p.work_next, p.seg, p.max_segs * p.syrk_items, p.d, S, p.partials, p.overwrite);
}

// After the Gram-sum kernel.  The slots zeroed here received no token, so no
// Gram-sum item or partial buffer touches them; the derived shared slot comes
// last, from the finished routed sums.
void launch_syrk_reduce(const CollectPlan& p, float* S, const int64_t* layer_counts, hipStream_t s) {
  hipLaunchKernelGGL(syrk_reduce_kernel, dim3((p.d + 1023) / 1024, p.d, kReduceGroups), dim3(256), 0, s, p.split,
                     p.partials, S, p.d);
  if (p.overwrite)
    hipLaunchKernelGGL(zero_empty_slots_kernel, dim3(p.E + p.has_shared), dim3(256), 0, s, layer_counts, S,
                       p.d);
  if (p.derive_shared)
    hipLaunchKernelGGL(shared_from_routed_kernel, dim3((p.d + 1023) / 1024, p.d), dim3(256), 0, s, S, p.E, p.K,
                       p.d);
}

int syrk_items_per_slot(int d) {
  const int nt = (d + kT - 1) / kT;
  return nt * (nt - 1) / 2 + (nt + 1) / 2;
}

}  // namespace clha
