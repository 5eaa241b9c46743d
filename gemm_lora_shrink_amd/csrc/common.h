// Internal definitions shared by the library's HIP sources: storage-type traits,
// the segment-record layout and the parameter blocks passed to the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lora.h"

namespace lora {

// ---------------------------------------------------------------------------
// Work decomposition constants
// ---------------------------------------------------------------------------
constexpr int kInfoWords = 16;
constexpr int kGroup = 16;  // tokens per gather (BGMV) work item
constexpr int kTile = 64;   // tokens per segmented (SGMV) work item
constexpr int kSgmvMinTokens = 48;  // AUTO: slots with this many tokens go to SGMV
constexpr int kFusedMaxTokens = 4096;  // lora_shrink_expand runs as one launch up to this T
constexpr int kF32FusedMaxTokens = 2048;  // ... and fp32 batches up to this T
constexpr int kFusedBuildMaxSlots = 256;  // ... and builds the record inside that launch up to this S
constexpr int kMaskMaxLanes = 128;  // the mask form takes adapters of at most this many stacked ranks (S * r_max)

enum InfoWord {
  kNumActive = 0,
  kNumSegments = 1,
  kMaxSegLen = 2,
  kStatus = 3,
  kNumGroups = 4,
  kNumTiles = 5,
  kBuiltT = 6,
  kBuiltS = 7,
};

// One work item: tokens perm[p0 .. p0 + cnt) all have slot `slot`.  In the
// record an item is this header followed by its token indices inline (padded
// to the list's item capacity with -1), so a kernel gets the header and the
// tokens in one memory round trip.
struct Item {
  int p0, cnt, slot, seg;
};
constexpr int kGroupItemWords = 4 + kGroup;  // 20
constexpr int kTileItemWords = 4 + kTile;    // 68

struct SegLayout {
  int64_t perm, seg_slot, seg_start, groups, tiles, words;
  int64_t cap_groups, cap_tiles;
};

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

__host__ __device__ inline SegLayout seg_layout(int64_t T, int64_t S) {
  SegLayout L;
  L.perm = kInfoWords;
  L.seg_slot = L.perm + T;
  L.seg_start = L.seg_slot + S;
  L.groups = (L.seg_start + S + 1 + 3) & ~int64_t(3);  // 16-byte aligned items
  int64_t minST = S < T ? S : T;
  L.cap_groups = ceil_div(T, kGroup) + minST;
  L.tiles = L.groups + kGroupItemWords * L.cap_groups;
  L.cap_tiles = ceil_div(T, kTile) + minST;
  L.words = L.tiles + kTileItemWords * L.cap_tiles;
  return L;
}

// ---------------------------------------------------------------------------
// Storage types
// ---------------------------------------------------------------------------
typedef _Float16 half_t;
typedef __bf16 bf16_t;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ inline float bf16_bits_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round-to-nearest-even conversions of one fp32 value to the 16-bit types,
// returned as the 16-bit pattern.
__device__ inline uint32_t float_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, static_cast<bf16_t>(f));
}
__device__ inline uint32_t float_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, static_cast<half_t>(f));
}

// Two fp32 values rounded to nearest-even into one word of two 16-bit lanes
// (a in the low half): one packed conversion instruction on gfx950.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack2_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ inline uint32_t pack2_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

// Reinterpret one 32-bit word as two 16-bit lanes.  The word is always passed
// by value: this compiler mis-lowers __builtin_bit_cast applied directly to an
// element of an ext_vector (it reads element 0 whatever the index), so vector
// elements are first copied into a scalar.
__device__ inline f16x2 as_f16x2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ inline bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its global loads and stores (__syncthreads also waits
// for those).
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Branch-free guarded loads.  A lane whose access is out of range reads 16
// bytes of zeros from a small constant array instead, so the select is on the
// address, before the load: no branch splits the code (the compiler would wait
// for every outstanding load at the merge) and no select on the loaded value
// forces a wait right after the load.
__device__ const u32x4 g_zero16[2] = {u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}};

// Both candidate addresses are global memory; saying so keeps the load a
// global_load (a generic flat_load would also hold the LDS wait counter).
typedef __attribute__((address_space(1))) const u32x4 global_u32x4;
typedef __attribute__((address_space(1))) const f32x4 global_f32x4;

__device__ inline u32x4 ld16_or0(const void* p, bool ok) {
  const global_u32x4* gp = (const global_u32x4*)(ok ? p : static_cast<const void*>(g_zero16));
  return *gp;
}
// The same with a non-temporal hint, for data streamed once (the y rows the
// expand reads, adds to and writes back): it is not kept in the caches.
__device__ inline u32x4 ld16_or0_nt(const void* p, bool ok) {
  const global_u32x4* gp = (const global_u32x4*)(ok ? p : static_cast<const void*>(g_zero16));
  return __builtin_nontemporal_load(gp);
}
__device__ inline f32x4 ldf4_or0(const float* p, bool ok) {
  const global_f32x4* gp =
      (const global_f32x4*)(ok ? static_cast<const void*>(p) : static_cast<const void*>(g_zero16));
  return *gp;
}

// Traits: Elem is the storage type; a "vec" is 16 bytes of it.
template <typename Elem> struct Traits;

template <> struct Traits<float> {
  static constexpr int kVec = 4;  // elements per 16 bytes
  static constexpr lora_dtype kDtype = LORA_F32;
  // dot of two 16-byte vectors accumulated into acc (fp32 FMA)
  __device__ static inline float dot(u32x4 a, u32x4 b, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ai = a[i], bi = b[i];
      acc = __builtin_fmaf(__uint_as_float(ai), __uint_as_float(bi), acc);
    }
    return acc;
  }
  __device__ static inline void to_float(u32x4 a, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ai = a[i];
      out[i] = __uint_as_float(ai);
    }
  }
  __device__ static inline float elem_to_float(uint32_t bits) { return __uint_as_float(bits); }
};

template <> struct Traits<half_t> {
  static constexpr int kVec = 8;
  static constexpr lora_dtype kDtype = LORA_F16;
  __device__ static inline float dot(u32x4 a, u32x4 b, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ai = a[i], bi = b[i];
      acc = __builtin_amdgcn_fdot2(as_f16x2(ai), as_f16x2(bi), acc, false);
    }
    return acc;
  }
  __device__ static inline void to_float(u32x4 a, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ai = a[i];
      const f16x2 h = as_f16x2(ai);
      out[2 * i] = (float)h[0];
      out[2 * i + 1] = (float)h[1];
    }
  }
  __device__ static inline float elem_to_float(uint32_t bits) {
    return (float)__builtin_bit_cast(half_t, (uint16_t)bits);
  }
};

template <> struct Traits<bf16_t> {
  static constexpr int kVec = 8;
  static constexpr lora_dtype kDtype = LORA_BF16;
  __device__ static inline float dot(u32x4 a, u32x4 b, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ai = a[i], bi = b[i];
      acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(ai), as_bf16x2(bi), acc, false);
    }
    return acc;
  }
  __device__ static inline void to_float(u32x4 a, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ai = a[i];
      out[2 * i] = __uint_as_float(ai << 16);
      out[2 * i + 1] = __uint_as_float(ai & 0xffff0000u);
    }
  }
  __device__ static inline float elem_to_float(uint32_t bits) { return bf16_bits_to_float(bits); }
};

// ---------------------------------------------------------------------------
// Kernel parameter blocks
// ---------------------------------------------------------------------------
struct ShrinkParams {
  const void* x;
  int64_t ldx;
  const void* A[LORA_MAX_SLICES];
  const int32_t* ranks;  // nullable
  const float* scale;    // nullable
  const int32_t* rec;    // segment record
  float* v;
  int64_t v_slice_stride;  // floats between slices of v (= T * r_max)
  int32_t D, S, r_max, n_slices, T;
};

struct ExpandParams {
  const float* v;
  int64_t v_slice_stride;  // 0: all slices share one v
  const void* B[LORA_MAX_SLICES];
  int64_t out_size[LORA_MAX_SLICES];
  int64_t out_off[LORA_MAX_SLICES];
  const int32_t* ranks;  // nullable
  const int32_t* rec;
  void* y;
  int64_t ldy;
  int32_t S, r_max, n_slices, T;
  int32_t b_row_unit;  // 0: B rows of r_max elements; else rows of the slot's rank rounded up to this
};

// A kernel's arguments are read from device memory through the scalar cache,
// one 64-byte line at a time on first use.  A large parameter block whose
// lines are first touched one after another puts one memory round trip per
// line on the kernel's critical path (measured: about 1.2 us between the
// grouping and the first producer unit of the one-launch kernel at decode
// size).  warm_args requests every line of the first kBytes of the kernel's
// argument segment (the parameter block is every kernel's first argument) at
// entry, all at once.  It reads through the segment pointer: taking the
// address of the by-value parameter instead makes the compiler copy it to
// scratch memory and read its fields from there.
template <typename P>
__device__ __forceinline__ void warm_args(const P&) {
  constexpr int kWords = (int)(sizeof(P) / 4);
  static_assert(kWords <= 8 * 16, "at most 8 lines");
  typedef const __attribute__((address_space(4))) uint32_t* KernargWords;  // the constant address space
  const KernargWords w = (KernargWords)__builtin_amdgcn_kernarg_segment_ptr();
  auto line = [&](int i) { return w[16 * i < kWords ? 16 * i : kWords - 1]; };
  // one statement takes every line's word, so that the loads are issued
  // together and waited for once
  asm volatile("" ::"s"(line(0)), "s"(line(1)), "s"(line(2)), "s"(line(3)), "s"(line(4)), "s"(line(5)),
               "s"(line(6)), "s"(line(7)));
}

// Elements between consecutive rows j, j + 1 of one slot's B (rank r): r_max
// in the padded layout, the rank rounded up to whole 16-byte pieces in the
// rank-rows layout (the slot's region keeps its [out][r_max] size either way).
__device__ inline int b_row_stride(const ExpandParams& p, int r) {
  return p.b_row_unit ? (r + p.b_row_unit - 1) / p.b_row_unit * p.b_row_unit : p.r_max;
}

// Persistent work loops.  A launch has a fixed number of workgroups (a
// multiple of 8, sized to what the chip holds at once) and walks a work list
// whose length is only known on the device.  The hardware hands workgroup b
// to XCD b % 8, and each of the 8 XCDs has its own L2, so XCD x is given the
// contiguous range [x N / 8, (x + 1) N / 8) of the list and its workgroups
// stride through it: consecutive work items (which share adapter rows or
// activation rows) then meet in the same L2.  Every workgroup leaves the loop
// after at most ceil(N / gridDim.x) + 1 items.
constexpr int kXcds = 8;

struct WorkRange {
  int64_t begin, end, step;
};

__device__ inline WorkRange xcd_work_range(int64_t n_work) {
  const int64_t xcd = blockIdx.x % kXcds, lb = blockIdx.x / kXcds, wgs = gridDim.x / kXcds;
  const int64_t per = n_work / kXcds, rem = n_work % kXcds;
  const int64_t start = xcd * per + (xcd < rem ? xcd : rem);
  const int64_t len = per + (xcd < rem ? 1 : 0);
  return WorkRange{start + lb, start + len, wgs};
}

// Number of items in a record's list, or 0 when the record does not match
// the call's sizes or its count is out of range.
__device__ inline int record_items(const int32_t* rec, int T, int S, bool tiles) {
  if (rec[kBuiltT] != T || rec[kBuiltS] != S) return 0;
  const int n = rec[tiles ? kNumTiles : kNumGroups];
  const SegLayout L = seg_layout(T, S);
  return (n < 0 || n > (tiles ? L.cap_tiles : L.cap_groups)) ? 0 : n;
}

// Word pointer to item `i` of a list (header, then inline tokens).
__device__ inline const int32_t* item_ptr(const int32_t* rec, int T, int S, bool tiles, int64_t i) {
  const SegLayout L = seg_layout(T, S);
  return rec + (tiles ? L.tiles + i * kTileItemWords : L.groups + i * kGroupItemWords);
}

// Header of item `i` (< record_items) of a list, with its fields checked
// against the sizes.
__device__ inline bool read_item(const int32_t* rec, int T, int S, bool tiles, int64_t i, Item& it) {
  // one 16-byte load (items are 16-byte aligned), so that the checks below
  // do not split the header into dependent loads
  const u32x4 h = *reinterpret_cast<const u32x4*>(item_ptr(rec, T, S, tiles, i));
  it = Item{(int)h[0], (int)h[1], (int)h[2], (int)h[3]};
  const int cap = tiles ? kTile : kGroup;
  return it.slot >= 0 && it.slot < S && it.p0 >= 0 && it.cnt > 0 && it.cnt <= cap && it.p0 + it.cnt <= T;
}

// Token k of item `i`, clamped into [0, T); -1 when k is past the item's count.
__device__ inline int item_token(const int32_t* rec, int T, int S, bool tiles, int64_t i, int k, int cnt) {
  const int t = item_ptr(rec, T, S, tiles, i)[4 + k];
  if (k >= cnt) return -1;
  return t < 0 ? 0 : (t >= T ? T - 1 : t);
}

__device__ inline int slot_rank(const int32_t* ranks, int s, int r_max) {
  if (!ranks) return r_max;
  int r = ranks[s];
  return r < 0 ? 0 : (r > r_max ? r_max : r);
}

// Workgroups of `kernel` the current device holds at once (occupancy x
// compute units), computed once per device and kernel.
int resident_workgroups(const void* kernel, int block, size_t dyn_lds);
// Workgroups of a persistent launch of `kernel`: what the chip holds at once
// rounded down to a multiple of 8, no more than `max_useful` rounded up to a
// multiple of 8, and at least 8.
int persistent_grid(const void* kernel, int block, size_t dyn_lds, int64_t max_useful);

// Host-side launchers (defined in the .hip files).
hipError_t launch_build_segments(const int32_t* idx, int32_t T, int32_t S, int32_t mode, int32_t* rec,
                                 hipStream_t stream);
// Shrink of every work item of the record (the gather groups and/or the
// segmented tiles) plus the clearing of the rows of tokens without an adapter,
// in one launch.
hipError_t launch_shrink(lora_dtype dt, const ShrinkParams& p, bool groups, bool tiles, hipStream_t stream);
// v[0 .. n) = 0
hipError_t launch_fill_zero(float* v, int64_t n, hipStream_t stream);
hipError_t launch_bgmv_expand(lora_dtype dt, const ExpandParams& p, bool tiles, hipStream_t stream);
// Matrix-core expand over the gather groups and/or the segmented tiles, in one
// launch (16-bit types only).
hipError_t launch_mfma_expand(lora_dtype dt, const ExpandParams& p, bool groups, bool tiles, hipStream_t stream);

// Shrink of an embedding adapter: v[t][k] = scale[s] * A_emb[s][tok[t]][k]
// for every token (zero rows for tokens without a valid slot or id).
hipError_t launch_embedding_shrink(lora_dtype dt, const int32_t* tok, const int32_t* idx, int32_t T, int64_t V,
                                   const void* A_emb, int32_t S, int32_t r_max, const int32_t* ranks,
                                   const float* scale, float* v, hipStream_t stream);

// dst[i][j] = M[i][j] inside M's rows and columns, 0 elsewhere, for
// i < dst_rows, j < dst_cols; M = src ([m_rows][m_cols], row stride src_ld)
// or, with transpose, src^T (src then [m_cols][m_rows]).
hipError_t launch_copy_padded(int elem_bytes, const void* src, int64_t src_ld, int transpose, int64_t m_rows,
                              int64_t m_cols, void* dst, int64_t dst_rows, int64_t dst_cols, int64_t dst_ld,
                              hipStream_t stream);

// Mask form of shrink + expand (S * r_max <= kMaskMaxLanes): the stacked
// rank lanes, the shrink's K parts and the workspace bytes it needs
// ([n_slices][parts][T][lanes] fp32 partial sums).
int32_t mask_lanes(lora_dtype dt, int32_t S, int32_t r_max);
int32_t mask_parts(int32_t T, int32_t D, int32_t n_slices);
int64_t mask_need_bytes(lora_dtype dt, int32_t T, int32_t D, int32_t S, int32_t n_slices, int32_t r_max);
hipError_t launch_mask(lora_dtype dt, const ShrinkParams& sp, const ExpandParams& ep, const int32_t* idx,
                       float* part, float* v, hipStream_t stream);

// Workspace of the fused shrink-expand call.  The layout depends only on the
// workspace's size: word 0 counts waits that gave up, the per-chunk counters
// fill [counters, counters + counter_bytes), the producer slabs (or v, when
// the call runs as two launches) start at `part`.
struct FusedLayout {
  int64_t counters, counter_bytes, part;
};
FusedLayout fused_layout(int64_t bytes);
// Smallest workspace for a call of this shape.
int64_t fused_need_bytes(int64_t T, int64_t S, int64_t n_slices, int64_t r_max);
// Shrink and expand of the batch's 16-token chunks in one launch (16-bit types
// only); v_out (nullable) receives v in full.
// idx (nullable): the batch's slots; when given, the kernel groups the tokens
// itself (T <= kFusedMaxTokens) and one of its workgroups builds the segment
// record into sp.rec (S <= kFusedBuildMaxSlots); the record is not read.
hipError_t launch_fused(lora_dtype dt, const ShrinkParams& sp, const ExpandParams& ep, const int32_t* idx, char* ws,
                        int64_t ws_bytes, float* v_out, hipStream_t stream);
// Whether every workgroup of the one-launch kernel for (dt, T, idx form) fits
// on the current device at once, which its waits need; when it does not, the
// call runs as separate launches.
bool fused_coresident(lora_dtype dt, int32_t T, bool from_idx);

}  // namespace lora
