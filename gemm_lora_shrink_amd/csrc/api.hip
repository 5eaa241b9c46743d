// C ABI entry points: host-side argument checks, the no-op gate and dispatch.
//
// Every check runs before anything is enqueued, so a rejected call leaves
// every buffer untouched.  The no-op gate follows "[LoRA] LoRA cuda graph
// specialization" (Purpose, Implementation): whether any adapter is active is
// a host-side fact, and when none is the call launches nothing at all; when
// the call does run, the intermediate is cleared inside the shrink call.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

#include "common.h"

#define LORA_EXPORT extern "C" __attribute__((visibility("default")))

namespace lora {
namespace {

thread_local char g_err[512];

lora_status fail(lora_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

lora_status hip_fail(hipError_t e, const char* what) {
  return fail(LORA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

void clear_error() { g_err[0] = 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int vec_of(lora_dtype dt) { return dt == LORA_F32 ? 4 : 8; }

bool valid_dtype(int dt) { return dt == LORA_F32 || dt == LORA_F16 || dt == LORA_BF16; }

// Kernel used for the expand of gather (decode) groups of 16-bit data.  The
// matrix-core kernel is the default; LORA_MI355X_GATHER_EXPAND=valu selects the
// VALU gather kernel instead (kept for comparison measurements).
bool gather_expand_on_valu() {
  static const bool valu = [] {
    const char* e = getenv("LORA_MI355X_GATHER_EXPAND");
    return e && strcmp(e, "valu") == 0;
  }();
  return valu;
}

lora_status check_common(int dt, int32_t T, int32_t n_slices, int32_t S, int32_t r_max, const void* seg) {
  if (!valid_dtype(dt)) return fail(LORA_ERR_INVALID_ARG, "unknown dtype %d", dt);
  if (T < 0) return fail(LORA_ERR_INVALID_ARG, "T = %d is negative", T);
  if (n_slices < 1) return fail(LORA_ERR_INVALID_ARG, "n_slices = %d must be >= 1", n_slices);
  if (n_slices > LORA_MAX_SLICES)
    return fail(LORA_ERR_UNSUPPORTED, "n_slices = %d exceeds %d", n_slices, LORA_MAX_SLICES);
  if (S < 1) return fail(LORA_ERR_INVALID_ARG, "S = %d must be >= 1", S);
  if (S > LORA_MAX_SLOTS) return fail(LORA_ERR_UNSUPPORTED, "S = %d exceeds %d", S, LORA_MAX_SLOTS);
  if (r_max < 1) return fail(LORA_ERR_INVALID_ARG, "r_max = %d must be >= 1", r_max);
  if (r_max > LORA_MAX_RANK) return fail(LORA_ERR_UNSUPPORTED, "r_max = %d exceeds %d", r_max, LORA_MAX_RANK);
  if (r_max % vec_of((lora_dtype)dt))
    return fail(LORA_ERR_UNSUPPORTED, "r_max = %d must be a multiple of %d for this dtype", r_max,
                vec_of((lora_dtype)dt));
  if (!seg) return fail(LORA_ERR_INVALID_ARG, "segment record is null");
  if (reinterpret_cast<uintptr_t>(seg) & 255u)
    return fail(LORA_ERR_INVALID_ARG, "segment record must be 256-byte aligned");
  return LORA_OK;
}

}  // namespace

int resident_workgroups(const void* kernel, int block, size_t dyn_lds) {
  // (device, kernel) -> workgroups resident at once, computed on first use
  struct Entry {
    int device;
    const void* kernel;
    int blocks;
  };
  static std::mutex mu;
  static std::vector<Entry> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  int resident = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry& e : cache)
      if (e.device == dev && e.kernel == kernel) resident = e.blocks;
  }
  if (resident == 0) {
    int occ = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, block, dyn_lds) != hipSuccess || occ < 1) occ = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    resident = occ * cus;
    std::lock_guard<std::mutex> lock(mu);
    cache.push_back(Entry{dev, kernel, resident});
  }
  return resident;
}

int persistent_grid(const void* kernel, int block, size_t dyn_lds, int64_t max_useful) {
  // a multiple of 8 (the XCD count) no larger than what is resident at once,
  // so that every workgroup of the launch can run at the same time (the
  // one-launch shrink-expand relies on it); at least 8
  int64_t g = resident_workgroups(kernel, block, dyn_lds) / kXcds * kXcds;
  const int64_t useful = ((max_useful > 0 ? max_useful : 1) + kXcds - 1) / kXcds * kXcds;
  if (g > useful) g = useful;
  if (g < kXcds) g = kXcds;
  return (int)g;
}

}  // namespace lora

using namespace lora;

LORA_EXPORT int32_t lora_abi_version(void) { return LORA_ABI_VERSION; }

LORA_EXPORT const char* lora_status_string(lora_status s) {
  switch (s) {
    case LORA_OK: return "LORA_OK";
    case LORA_ERR_INVALID_ARG: return "LORA_ERR_INVALID_ARG";
    case LORA_ERR_UNSUPPORTED: return "LORA_ERR_UNSUPPORTED";
    case LORA_ERR_INDEX: return "LORA_ERR_INDEX";
    case LORA_ERR_HIP: return "LORA_ERR_HIP";
  }
  return "LORA_ERR_UNKNOWN";
}

LORA_EXPORT const char* lora_last_error(void) { return g_err; }

LORA_EXPORT int32_t lora_sgmv_min_tokens(void) { return kSgmvMinTokens; }

LORA_EXPORT int32_t lora_fused_max_tokens(void) { return kFusedMaxTokens; }

LORA_EXPORT int32_t lora_fused_max_tokens_for(lora_dtype dt) {
  switch (dt) {
    case LORA_F32: return kF32FusedMaxTokens;
    case LORA_F16:
    case LORA_BF16: return kFusedMaxTokens;
  }
  return 0;
}

LORA_EXPORT size_t lora_segments_bytes(int32_t T, int32_t S) {
  if (T < 0 || S < 1 || S > LORA_MAX_SLOTS) return 0;
  const SegLayout L = seg_layout(T, S);
  return (size_t)(((L.words * 4) + 255) & ~int64_t(255));
}

LORA_EXPORT int64_t lora_segments_offset(int32_t T, int32_t S, lora_seg_field field) {
  if (T < 0 || S < 1 || S > LORA_MAX_SLOTS) return -1;
  const SegLayout L = seg_layout(T, S);
  switch (field) {
    case LORA_SEG_INFO: return 0;
    case LORA_SEG_PERM: return L.perm;
    case LORA_SEG_SLOT: return L.seg_slot;
    case LORA_SEG_START: return L.seg_start;
    case LORA_SEG_GROUPS: return L.groups;
    case LORA_SEG_TILES: return L.tiles;
  }
  return -1;
}

LORA_EXPORT lora_status lora_build_segments(const int32_t* idx, int32_t T, int32_t S, int32_t mode, void* seg,
                                            int32_t* info_host, hipStream_t stream) {
  clear_error();
  if (T < 0) return fail(LORA_ERR_INVALID_ARG, "T = %d is negative", T);
  if (S < 1) return fail(LORA_ERR_INVALID_ARG, "S = %d must be >= 1", S);
  if (S > LORA_MAX_SLOTS) return fail(LORA_ERR_UNSUPPORTED, "S = %d exceeds %d", S, LORA_MAX_SLOTS);
  if (mode != LORA_MODE_AUTO && mode != LORA_MODE_BGMV && mode != LORA_MODE_SGMV)
    return fail(LORA_ERR_INVALID_ARG, "unknown mode %d", mode);
  if (!seg) return fail(LORA_ERR_INVALID_ARG, "segment record is null");
  if (reinterpret_cast<uintptr_t>(seg) & 255u)
    return fail(LORA_ERR_INVALID_ARG, "segment record must be 256-byte aligned");
  if (T > 0 && !idx) return fail(LORA_ERR_INVALID_ARG, "idx is null");
  hipError_t e = launch_build_segments(idx, T, S, mode, static_cast<int32_t*>(seg), stream);
  if (e != hipSuccess) return hip_fail(e, "segment build launch");
  if (info_host) {
    e = hipMemcpyAsync(info_host, seg, kInfoWords * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (e != hipSuccess) return hip_fail(e, "info copy");
  }
  return LORA_OK;
}

namespace lora {
namespace {

// Host checks of the shrink arguments; fills p (everything but the v pointer
// check happens here; v is checked by the caller).
lora_status prep_shrink(lora_dtype dt, const void* x, int64_t ldx, int32_t T, int32_t D, int32_t n_slices,
                        const void* const* A, int32_t S, int32_t r_max, const int32_t* ranks, const float* scale,
                        const void* seg, float* v, ShrinkParams& p) {
  lora_status st = check_common(dt, T, n_slices, S, r_max, seg);
  if (st != LORA_OK) return st;
  const int vec = vec_of(dt);
  if (D < 1) return fail(LORA_ERR_INVALID_ARG, "D = %d must be >= 1", D);
  if (T == 0) return LORA_OK;  // empty batch: nothing to read or write
  if (ldx < D) return fail(LORA_ERR_INVALID_ARG, "ldx = %lld is smaller than D = %d", (long long)ldx, D);
  if (D % vec || ldx % vec)
    return fail(LORA_ERR_UNSUPPORTED, "D and ldx must be multiples of %d elements for this dtype", vec);
  if (!x || !v) return fail(LORA_ERR_INVALID_ARG, "x or v is null");
  // the shrink kernels address x and one slot's A rows with 32-bit byte offsets
  const uint64_t esize = dt == LORA_F32 ? 4 : 2;
  if (((uint64_t)(T - 1) * (uint64_t)ldx + (uint64_t)D) * esize > 0xFFFFFFFFull)
    return fail(LORA_ERR_UNSUPPORTED, "x spans more than 4 GiB");
  if ((uint64_t)r_max * (uint64_t)D * esize > 0xFFFFFFFFull)
    return fail(LORA_ERR_UNSUPPORTED, "one slot's A rows span more than 4 GiB");
  if (!aligned16(x) || !aligned16(v)) return fail(LORA_ERR_UNSUPPORTED, "x and v must be 16-byte aligned");
  if (!A) return fail(LORA_ERR_INVALID_ARG, "A pointer array is null");
  p = ShrinkParams{};
  for (int i = 0; i < n_slices; ++i) {
    if (!A[i]) return fail(LORA_ERR_INVALID_ARG, "A[%d] is null", i);
    if (!aligned16(A[i])) return fail(LORA_ERR_UNSUPPORTED, "A[%d] must be 16-byte aligned", i);
    p.A[i] = A[i];
  }
  p.x = x;
  p.ldx = ldx;
  p.ranks = ranks;
  p.scale = scale;
  p.rec = static_cast<const int32_t*>(seg);
  p.v = v;
  p.v_slice_stride = (int64_t)T * r_max;
  p.D = D;
  p.S = S;
  p.r_max = r_max;
  p.n_slices = n_slices;
  p.T = T;
  return LORA_OK;
}

// Host checks of the expand arguments; fills p.
lora_status prep_expand(lora_dtype dt, const float* v, int64_t v_slice_stride, int32_t T, int32_t n_slices,
                        const void* const* B, const int64_t* out_sizes, const int64_t* out_offsets, int32_t S,
                        int32_t r_max, const int32_t* ranks, int32_t b_layout, const void* seg, void* y,
                        int64_t ldy, ExpandParams& p) {
  lora_status st = check_common(dt, T, n_slices, S, r_max, seg);
  if (st != LORA_OK) return st;
  if (b_layout != LORA_B_PADDED && b_layout != LORA_B_RANK_ROWS)
    return fail(LORA_ERR_INVALID_ARG, "unknown B layout %d", b_layout);
  const int vec = vec_of(dt);
  if (T == 0) return LORA_OK;  // empty batch: nothing to read or write
  if (!v || !y) return fail(LORA_ERR_INVALID_ARG, "v or y is null");
  if (!aligned16(v) || !aligned16(y)) return fail(LORA_ERR_UNSUPPORTED, "v and y must be 16-byte aligned");
  if (!B || !out_sizes || !out_offsets) return fail(LORA_ERR_INVALID_ARG, "B, out_sizes or out_offsets is null");
  if (v_slice_stride < 0) return fail(LORA_ERR_INVALID_ARG, "v_slice_stride is negative");
  if (v_slice_stride % 4) return fail(LORA_ERR_UNSUPPORTED, "v_slice_stride must be a multiple of 4 floats");
  if (v_slice_stride != 0 && v_slice_stride < (int64_t)T * r_max)
    return fail(LORA_ERR_INVALID_ARG, "v_slice_stride is smaller than T * r_max");
  if (ldy < 1 || ldy % vec) return fail(LORA_ERR_UNSUPPORTED, "ldy must be a positive multiple of %d", vec);
  p = ExpandParams{};
  std::vector<std::pair<int64_t, int64_t>> cols;
  for (int i = 0; i < n_slices; ++i) {
    if (!B[i]) return fail(LORA_ERR_INVALID_ARG, "B[%d] is null", i);
    if (!aligned16(B[i])) return fail(LORA_ERR_UNSUPPORTED, "B[%d] must be 16-byte aligned", i);
    if (out_sizes[i] < 1) return fail(LORA_ERR_INVALID_ARG, "out_sizes[%d] must be >= 1", i);
    if (out_offsets[i] < 0) return fail(LORA_ERR_INVALID_ARG, "out_offsets[%d] is negative", i);
    if (out_sizes[i] % vec || out_offsets[i] % vec)
      return fail(LORA_ERR_UNSUPPORTED, "out_sizes[%d] and out_offsets[%d] must be multiples of %d", i, i, vec);
    if (out_offsets[i] + out_sizes[i] > ldy)
      return fail(LORA_ERR_INVALID_ARG, "slice %d ends past ldy", i);
    if (out_sizes[i] > (int64_t)1 << 30) return fail(LORA_ERR_UNSUPPORTED, "out_sizes[%d] too large", i);
    p.B[i] = B[i];
    p.out_size[i] = out_sizes[i];
    p.out_off[i] = out_offsets[i];
    cols.emplace_back(out_offsets[i], out_offsets[i] + out_sizes[i]);
  }
  std::sort(cols.begin(), cols.end());
  for (size_t i = 1; i < cols.size(); ++i)
    if (cols[i].first < cols[i - 1].second) return fail(LORA_ERR_INVALID_ARG, "output slices overlap");
  p.v = v;
  p.v_slice_stride = v_slice_stride;
  p.ranks = ranks;
  p.rec = static_cast<const int32_t*>(seg);
  p.y = y;
  p.ldy = ldy;
  p.S = S;
  p.r_max = r_max;
  p.n_slices = n_slices;
  p.T = T;
  p.b_row_unit = b_layout == LORA_B_RANK_ROWS ? vec : 0;
  return LORA_OK;
}

// The expand launches of the record's items.
hipError_t run_expand(lora_dtype dt, const ExpandParams& p, hipStream_t stream) {
  hipError_t e;
  if (dt == LORA_F32) {
    e = launch_bgmv_expand(dt, p, /*tiles=*/false, stream);
    if (e == hipSuccess) e = launch_bgmv_expand(dt, p, /*tiles=*/true, stream);
  } else if (gather_expand_on_valu()) {
    e = launch_bgmv_expand(dt, p, /*tiles=*/false, stream);
    if (e == hipSuccess) e = launch_mfma_expand(dt, p, /*groups=*/false, /*tiles=*/true, stream);
  } else {
    e = launch_mfma_expand(dt, p, /*groups=*/true, /*tiles=*/true, stream);
  }
  return e;
}

}  // namespace
}  // namespace lora

LORA_EXPORT lora_status lora_shrink(lora_dtype dt, const void* x, int64_t ldx, int32_t T, int32_t D,
                                    int32_t n_slices, const void* const* A, int32_t S, int32_t r_max,
                                    const int32_t* ranks, const float* scale, const void* seg,
                                    int32_t active_hint, float* v, hipStream_t stream) {
  clear_error();
  ShrinkParams p;
  const lora_status st = prep_shrink(dt, x, ldx, T, D, n_slices, A, S, r_max, ranks, scale, seg, v, p);
  if (st != LORA_OK || T == 0) return st;
  if (active_hint == 0) return LORA_OK;  // base-only batch: nothing is enqueued
  // One launch shrinks every work item and leaves v fully written (preceded by
  // a clearing launch when items are cut into parts summed with atomics).
  const hipError_t e = launch_shrink(dt, p, /*groups=*/true, /*tiles=*/true, stream);
  if (e != hipSuccess) return hip_fail(e, "shrink launch");
  return LORA_OK;
}

LORA_EXPORT lora_status lora_expand(lora_dtype dt, const float* v, int64_t v_slice_stride, int32_t T,
                                    int32_t n_slices, const void* const* B, const int64_t* out_sizes,
                                    const int64_t* out_offsets, int32_t S, int32_t r_max, const int32_t* ranks,
                                    int32_t b_layout, const void* seg, int32_t active_hint, void* y, int64_t ldy,
                                    hipStream_t stream) {
  clear_error();
  ExpandParams p;
  const lora_status st = prep_expand(dt, v, v_slice_stride, T, n_slices, B, out_sizes, out_offsets, S, r_max, ranks,
                                     b_layout, seg, y, ldy, p);
  if (st != LORA_OK || T == 0) return st;
  if (active_hint == 0) return LORA_OK;  // base-only batch: nothing is enqueued
  const hipError_t e = run_expand(dt, p, stream);
  if (e != hipSuccess) return hip_fail(e, "expand launch");
  return LORA_OK;
}

LORA_EXPORT size_t lora_shrink_expand_workspace_bytes(int32_t T, int32_t S, int32_t n_slices, int32_t r_max) {
  if (T < 0 || S < 1 || S > LORA_MAX_SLOTS || n_slices < 1 || n_slices > LORA_MAX_SLICES || r_max < 1 ||
      r_max > LORA_MAX_RANK)
    return 0;
  return (size_t)fused_need_bytes(T, S, n_slices, r_max);
}

namespace lora {
namespace {

// The body of lora_shrink_expand and of its allocation-free variant: checks,
// the no-op gate, then the launches on the workspace ws of ws_bytes bytes.
// clear_first: enqueue a clearing of the workspace's header and counters
// before the launches (the variant's first call on a device).
lora_status shrink_expand_impl(lora_dtype dt, const void* x, int64_t ldx, int32_t T, int32_t D, int32_t n_slices,
                               const void* const* A, const void* const* B, const int64_t* out_sizes,
                               const int64_t* out_offsets, int32_t S, int32_t r_max, const int32_t* ranks,
                               int32_t b_layout, const float* scale, const void* seg, const int32_t* idx,
                               int32_t active_hint, float* v, void* y, int64_t ldy, char* ws, int64_t ws_bytes,
                               bool clear_first, bool* ran, hipStream_t stream) {
  *ran = false;
  // without a caller v, the two-launch form keeps v in the workspace's data
  // region (never in the header or the counters)
  const FusedLayout W = fused_layout(ws_bytes);
  float* v_eff = v ? v : reinterpret_cast<float*>(ws + W.part);
  ShrinkParams sp;
  lora_status st = prep_shrink(dt, x, ldx, T, D, n_slices, A, S, r_max, ranks, scale, seg, v_eff, sp);
  if (st != LORA_OK) return st;
  ExpandParams ep;
  st = prep_expand(dt, v_eff, (int64_t)T * r_max, T, n_slices, B, out_sizes, out_offsets, S, r_max, ranks, b_layout,
                   seg, y, ldy, ep);
  if (st != LORA_OK || T == 0) return st;
  if (active_hint == 0) return LORA_OK;  // base-only batch: nothing is enqueued
  hipError_t e = hipSuccess;
  if (clear_first) e = launch_fill_zero(reinterpret_cast<float*>(ws), W.part / 4, stream);
  *ran = e == hipSuccess;
  // one launch only where all of its workgroups are resident at once (its
  // consumers wait for its producers); otherwise the separate launches
  const bool one_launch = T <= lora_fused_max_tokens_for(dt) &&
                          fused_coresident(dt, T, idx != nullptr && S <= kFusedBuildMaxSlots);
  if (e != hipSuccess) {
  } else if (one_launch && idx && S <= kFusedBuildMaxSlots) {
    // the launch builds the record itself, beside the layer
    e = launch_fused(dt, sp, ep, idx, ws, ws_bytes, v, stream);
  } else {
    // with idx and no room for the build inside the launch: the build kernel first
    if (idx) e = launch_build_segments(idx, T, S, LORA_MODE_AUTO, static_cast<int32_t*>(const_cast<void*>(seg)), stream);
    if (e == hipSuccess && one_launch) {
      e = launch_fused(dt, sp, ep, nullptr, ws, ws_bytes, v, stream);
    } else if (e == hipSuccess) {
      // larger batches stream enough bytes per launch that the launch and the
      // round trips no longer dominate: the shrink launch then the expand launch
      e = launch_shrink(dt, sp, /*groups=*/true, /*tiles=*/true, stream);
      if (e == hipSuccess) e = run_expand(dt, ep, stream);
    }
  }
  if (e != hipSuccess) return hip_fail(e, "shrink-expand launch");
  return LORA_OK;
}

// Scratch of the allocation-free variant: a file-scope device array, one copy
// per device the library runs on, held until the process ends.  Host code
// never uses the array's name as an address: the device address of each
// device's copy comes from hipGetSymbolAddress, once per device, with that
// device current.
static __device__ __align__(256) char scratch[LORA_NOALLOC_SCRATCH_BYTES];

struct ScratchOfDevice {
  int device;
  char* ptr;     // device address of this device's copy of `scratch`
  bool cleared;  // its header and counters have been cleared in stream order
};
std::mutex g_scratch_mu;
std::vector<ScratchOfDevice> g_scratch;

}  // namespace
}  // namespace lora

LORA_EXPORT lora_status lora_shrink_expand(lora_dtype dt, const void* x, int64_t ldx, int32_t T, int32_t D,
                                           int32_t n_slices, const void* const* A, const void* const* B,
                                           const int64_t* out_sizes, const int64_t* out_offsets, int32_t S,
                                           int32_t r_max, const int32_t* ranks, int32_t b_layout, const float* scale,
                                           const void* seg, const int32_t* idx, int32_t active_hint, float* v, void* y,
                                           int64_t ldy, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  lora_status st = check_common(dt, T, n_slices, S, r_max, seg);
  if (st != LORA_OK) return st;
  if (!workspace) return fail(LORA_ERR_INVALID_ARG, "workspace is null");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(LORA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const int64_t need = fused_need_bytes(T, S, n_slices, r_max);
  if ((int64_t)workspace_bytes < need)
    return fail(LORA_ERR_INVALID_ARG, "workspace has %zu bytes, the call needs %lld", workspace_bytes,
                (long long)need);
  bool ran;
  return shrink_expand_impl(dt, x, ldx, T, D, n_slices, A, B, out_sizes, out_offsets, S, r_max, ranks, b_layout,
                            scale, seg, idx, active_hint, v, y, ldy, static_cast<char*>(workspace),
                            (int64_t)workspace_bytes, /*clear_first=*/false, &ran, stream);
}

LORA_EXPORT lora_status lora_shrink_expand_noalloc(lora_dtype dt, const void* x, int64_t ldx, int32_t T, int32_t D,
                                                   int32_t n_slices, const void* const* A, const void* const* B,
                                                   const int64_t* out_sizes, const int64_t* out_offsets, int32_t S,
                                                   int32_t r_max, const int32_t* ranks, int32_t b_layout,
                                                   const float* scale, const void* seg, const int32_t* idx,
                                                   int32_t active_hint, float* v, void* y, int64_t ldy,
                                                   int32_t* errors_host, hipStream_t stream) {
  clear_error();
  lora_status st = check_common(dt, T, n_slices, S, r_max, seg);
  if (st != LORA_OK) return st;
  const int64_t need = fused_need_bytes(T, S, n_slices, r_max);
  if (need > (int64_t)LORA_NOALLOC_SCRATCH_BYTES)
    return fail(LORA_ERR_UNSUPPORTED,
                "the call needs %lld bytes of scratch, more than the %lld of the allocation-free variant "
                "(use lora_shrink_expand with a workspace)",
                (long long)need, (long long)LORA_NOALLOC_SCRATCH_BYTES);
  // the device address of this device's scratch (no allocation: the array is
  // part of the loaded code object)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  char* ptr = nullptr;
  bool cleared = false;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    for (const ScratchOfDevice& sd : g_scratch)
      if (sd.device == dev) {
        ptr = sd.ptr;
        cleared = sd.cleared;
      }
    if (!ptr) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
      ptr = static_cast<char*>(p);
      g_scratch.push_back(ScratchOfDevice{dev, ptr, false});
    }
  }
  // The first call on a device clears the scratch's header and counters, in
  // stream order before its launches.  A call made while the stream is being
  // captured records that clearing in the graph (replayed with it) and does
  // not count as the first call.
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  bool ran = false;
  st = shrink_expand_impl(dt, x, ldx, T, D, n_slices, A, B, out_sizes, out_offsets, S, r_max, ranks, b_layout, scale,
                          seg, idx, active_hint, v, y, ldy, ptr, (int64_t)LORA_NOALLOC_SCRATCH_BYTES, !cleared, &ran,
                          stream);
  if (ran && !cleared && cap == hipStreamCaptureStatusNone) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    for (ScratchOfDevice& sd : g_scratch)
      if (sd.device == dev) sd.cleared = true;
  }
  if (st != LORA_OK || !errors_host) return st;
  e = hipMemcpyAsync(errors_host, ptr, sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return hip_fail(e, "scratch error count copy");
  return LORA_OK;
}

LORA_EXPORT lora_status lora_workspace_errors(const void* workspace, int32_t* host_out, hipStream_t stream) {
  clear_error();
  if (!workspace || !host_out) return fail(LORA_ERR_INVALID_ARG, "workspace or host_out is null");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(LORA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const hipError_t e = hipMemcpyAsync(host_out, workspace, sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return hip_fail(e, "workspace error count copy");
  return LORA_OK;
}

LORA_EXPORT lora_status lora_embedding_shrink(lora_dtype dt, const int32_t* tok, int32_t T, int64_t V,
                                              const void* A_emb, int32_t S, int32_t r_max, const int32_t* ranks,
                                              const float* scale, const int32_t* idx, int32_t active_hint, float* v,
                                              hipStream_t stream) {
  clear_error();
  if (!valid_dtype(dt)) return fail(LORA_ERR_INVALID_ARG, "unknown dtype %d", dt);
  if (T < 0) return fail(LORA_ERR_INVALID_ARG, "T = %d is negative", T);
  if (V < 1) return fail(LORA_ERR_INVALID_ARG, "V = %lld must be >= 1", (long long)V);
  if (S < 1) return fail(LORA_ERR_INVALID_ARG, "S = %d must be >= 1", S);
  if (S > LORA_MAX_SLOTS) return fail(LORA_ERR_UNSUPPORTED, "S = %d exceeds %d", S, LORA_MAX_SLOTS);
  if (r_max < 1) return fail(LORA_ERR_INVALID_ARG, "r_max = %d must be >= 1", r_max);
  if (r_max > LORA_MAX_RANK) return fail(LORA_ERR_UNSUPPORTED, "r_max = %d exceeds %d", r_max, LORA_MAX_RANK);
  if (r_max % vec_of(dt))
    return fail(LORA_ERR_UNSUPPORTED, "r_max = %d must be a multiple of %d for this dtype", r_max, vec_of(dt));
  if (T == 0) return LORA_OK;
  if (!tok || !idx || !A_emb || !v) return fail(LORA_ERR_INVALID_ARG, "tok, idx, A_emb or v is null");
  if (!aligned16(A_emb) || !aligned16(v)) return fail(LORA_ERR_UNSUPPORTED, "A_emb and v must be 16-byte aligned");
  if (V > ((int64_t)1 << 40) / ((int64_t)S * r_max)) return fail(LORA_ERR_UNSUPPORTED, "the stacked table is too large");
  if (active_hint == 0) return LORA_OK;  // base-only batch: nothing is enqueued
  const hipError_t e = launch_embedding_shrink(dt, tok, idx, T, V, A_emb, S, r_max, ranks, scale, v, stream);
  if (e != hipSuccess) return hip_fail(e, "embedding shrink launch");
  return LORA_OK;
}

LORA_EXPORT lora_status lora_copy_padded(lora_dtype dt, const void* src, int64_t m_rows, int64_t m_cols, int64_t src_ld,
                                         int32_t transpose, void* dst, int64_t dst_rows, int64_t dst_cols,
                                         int64_t dst_ld, hipStream_t stream) {
  clear_error();
  if (!valid_dtype(dt)) return fail(LORA_ERR_INVALID_ARG, "unknown dtype %d", dt);
  if (m_rows < 0 || m_cols < 0 || dst_rows < 0 || dst_cols < 0)
    return fail(LORA_ERR_INVALID_ARG, "negative size");
  if (m_rows > dst_rows || m_cols > dst_cols)
    return fail(LORA_ERR_INVALID_ARG, "the matrix (%lld x %lld) does not fit the slot (%lld x %lld)",
                (long long)m_rows, (long long)m_cols, (long long)dst_rows, (long long)dst_cols);
  if (dst_ld < dst_cols) return fail(LORA_ERR_INVALID_ARG, "dst_ld is smaller than dst_cols");
  if (m_rows > 0 && m_cols > 0) {
    if (!src) return fail(LORA_ERR_INVALID_ARG, "src is null");
    if (src_ld < (transpose ? m_rows : m_cols)) return fail(LORA_ERR_INVALID_ARG, "src_ld is too small");
  }
  if (dst_rows * dst_cols == 0) return LORA_OK;
  if (!dst) return fail(LORA_ERR_INVALID_ARG, "dst is null");
  const int esize = dt == LORA_F32 ? 4 : 2;
  const hipError_t e = launch_copy_padded(esize, src, src_ld, transpose ? 1 : 0, m_rows, m_cols, dst, dst_rows,
                                          dst_cols, dst_ld, stream);
  if (e != hipSuccess) return hip_fail(e, "padded copy launch");
  return LORA_OK;
}

LORA_EXPORT size_t lora_mask_workspace_bytes(lora_dtype dt, int32_t T, int32_t D, int32_t S, int32_t n_slices,
                                             int32_t r_max) {
  if (!valid_dtype(dt) || T < 0 || D < 1 || S < 1 || n_slices < 1 || n_slices > LORA_MAX_SLICES || r_max < 1 ||
      (int64_t)S * r_max > kMaskMaxLanes)
    return 0;
  const int64_t b = mask_need_bytes(dt, T, D, S, n_slices, r_max);
  return (size_t)((b + 255) & ~int64_t(255));
}

LORA_EXPORT lora_status lora_shrink_expand_mask(lora_dtype dt, const void* x, int64_t ldx, int32_t T, int32_t D,
                                                int32_t n_slices, const void* const* A, const void* const* B,
                                                const int64_t* out_sizes, const int64_t* out_offsets, int32_t S,
                                                int32_t r_max, const int32_t* ranks, const float* scale,
                                                const int32_t* idx, int32_t active_hint, float* v, void* y,
                                                int64_t ldy, void* workspace, size_t workspace_bytes,
                                                hipStream_t stream) {
  clear_error();
  // the checks shared with lora_shrink and lora_expand; this form reads no
  // segment record, so the workspace (256-byte aligned as a record must be)
  // stands in for it there, and for v when the caller passes none
  if (!workspace) return fail(LORA_ERR_INVALID_ARG, "workspace is null");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(LORA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  float* v_chk = v ? v : static_cast<float*>(workspace);
  ShrinkParams sp;
  lora_status st = prep_shrink(dt, x, ldx, T, D, n_slices, A, S, r_max, ranks, scale, workspace, v_chk, sp);
  if (st != LORA_OK) return st;
  ExpandParams ep;
  st = prep_expand(dt, v_chk, (int64_t)T * r_max, T, n_slices, B, out_sizes, out_offsets, S, r_max, ranks,
                   LORA_B_PADDED, workspace, y, ldy, ep);
  if (st != LORA_OK) return st;
  if ((int64_t)S * r_max > kMaskMaxLanes)
    return fail(LORA_ERR_UNSUPPORTED, "S * r_max = %lld exceeds the %d lanes of the mask form",
                (long long)S * r_max, kMaskMaxLanes);
  if (T == 0) return LORA_OK;
  if (!idx) return fail(LORA_ERR_INVALID_ARG, "idx is null");
  const int64_t need = mask_need_bytes(dt, T, D, S, n_slices, r_max);
  if ((int64_t)workspace_bytes < need)
    return fail(LORA_ERR_INVALID_ARG, "workspace has %zu bytes, the call needs %lld", workspace_bytes,
                (long long)need);
  if (active_hint == 0) return LORA_OK;  // base-only batch: nothing is enqueued
  const hipError_t e = launch_mask(dt, sp, ep, idx, static_cast<float*>(workspace), v, stream);
  if (e != hipSuccess) return hip_fail(e, "mask shrink-expand launch");
  return LORA_OK;
}
