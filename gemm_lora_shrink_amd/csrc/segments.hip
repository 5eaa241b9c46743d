// Segment build: group a batch's active tokens by adapter slot and plan the
// kernel work items.  The token index vector is built on the host and moved to
// the device once per batch ("[Hardware][TPU][V1] Better tpu multilora
// compilation", review of the token index buffer); every LoRA layer of the
// batch then reuses this record.
//
// One workgroup of 1024 threads (16 waves of 64) does everything, so the result
// is bit-exact and deterministic:
//   1. per-slot token counts (LDS atomics: counts do not depend on order);
//   2. a block-wide exclusive scan over slots giving each slot's start in perm,
//      its segment number and the offsets of its work items;
//   3. the segment tables, the info words and the work items;
//   4. a stable scatter of the tokens into perm, 1024 tokens per chunk: inside a
//      wave, lanes holding the same slot find each other with ballots; across
//      the 16 waves a per-(wave, slot) count table gives each wave its offset in
//      wave order.  No atomics touch the order.  Tokens without a valid slot
//      are placed as if they had slot S, after all active tokens, so perm ends
//      with them in ascending order (the shrink clears their v rows);
//   5. the work items, each followed by its token indices, read back from an
//      LDS mirror of perm (from global memory past 8192 tokens).
// The first 8192 slot indices are loaded once, all at the same time, and kept
// in registers.
#include "common.h"

namespace lora {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ inline int lane_id() { return __lane_id(); }

// Inclusive scan of one int across the wave.
__device__ inline int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  return v;
}

// Block-wide exclusive scan of four ints per thread (thread order), returning
// the exclusive prefixes and writing the four totals to `total`.
__device__ inline void block_exclusive_scan4(int4& v, int4* wave_sums, int4& total) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  int4 inc;
  inc.x = wave_inclusive_scan(v.x);
  inc.y = wave_inclusive_scan(v.y);
  inc.z = wave_inclusive_scan(v.z);
  inc.w = wave_inclusive_scan(v.w);
  if (lane == 63) wave_sums[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    int4 w = lane < kWaves ? wave_sums[lane] : make_int4(0, 0, 0, 0);
    int4 wi;
    wi.x = wave_inclusive_scan(w.x);
    wi.y = wave_inclusive_scan(w.y);
    wi.z = wave_inclusive_scan(w.z);
    wi.w = wave_inclusive_scan(w.w);
    if (lane < kWaves) wave_sums[lane] = make_int4(wi.x - w.x, wi.y - w.y, wi.z - w.z, wi.w - w.w);
    if (lane == kWaves - 1) wave_sums[kWaves] = wi;
  }
  __syncthreads();
  int4 base = wave_sums[wave];
  total = wave_sums[kWaves];
  v = make_int4(base.x + inc.x - v.x, base.y + inc.y - v.y, base.z + inc.z - v.z, base.w + inc.w - v.w);
}

// Largest s in [0, n) with arr[s] <= key, for a non-decreasing arr with arr[0] <= key.
__device__ inline int upper_slot(const int* arr, int n, int key) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (arr[mid] <= key) lo = mid; else hi = mid - 1;
  }
  return lo;
}

constexpr int kRegChunks = 8;                  // idx chunks held in registers (T <= 8192)
constexpr int kLdsPerm = kRegChunks * kThreads;  // perm positions mirrored in LDS

// Stable placement of one chunk of 1024 tokens (t = c0 + tid, slot index s).
// A token whose s is not a valid slot takes key S: those tokens follow every
// active token in perm.  Lanes with t >= T place nothing.
__device__ inline void scatter_chunk(int t, int s, int T, int S, int32_t* __restrict__ perm, int* s_perm, int* s_run,
                                     uint8_t (*s_wtab)[LORA_MAX_SLOTS + 1], int* s_leader_base) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const bool valid = t < T;
  s = (s >= 0 && s < S) ? s : S;
  // lanes of this wave with the same key
  uint64_t remaining = __ballot(valid);
  uint64_t peers = 0;
  while (remaining) {
    const int leader = __builtin_ctzll(remaining);
    const int ls = __shfl(s, leader, 64);
    const uint64_t m = __ballot(valid && s == ls);
    if (valid && s == ls) peers = m;
    remaining &= ~m;
  }
  const bool is_leader = valid && (peers & lt_mask) == 0;
  const int wcount = __popcll(peers);
  if (is_leader) s_wtab[wave][s] = (uint8_t)wcount;
  __syncthreads();
  int base = 0;
  bool last_wave = false;
  if (is_leader) {
    int pre = 0, post = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int c = s_wtab[w][s];
      if (w < wave) pre += c;
      if (w > wave) post += c;
    }
    base = s_run[s] + pre;
    last_wave = (post == 0);
    s_leader_base[tid] = base;
  }
  __syncthreads();
  if (valid) {
    const int pos = s_leader_base[(wave << 6) + __builtin_ctzll(peers)] + __popcll(peers & lt_mask);
    perm[pos] = t;
    if (pos < kLdsPerm) s_perm[pos] = t;
  }
  if (is_leader) {
    s_wtab[wave][s] = 0;
    if (last_wave) s_run[s] = base + wcount;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void build_segments_kernel(const int32_t* __restrict__ idx, int T, int S,
                                                                  int mode, int32_t* __restrict__ rec) {
  __shared__ int s_count[LORA_MAX_SLOTS];
  __shared__ int s_start[LORA_MAX_SLOTS];
  __shared__ int s_run[LORA_MAX_SLOTS + 1];  // [S]: the tokens without a slot
  __shared__ int s_seg[LORA_MAX_SLOTS];
  __shared__ int s_gofs[LORA_MAX_SLOTS + 1];
  __shared__ int s_tofs[LORA_MAX_SLOTS + 1];
  __shared__ uint8_t s_wtab[kWaves][LORA_MAX_SLOTS + 1];
  __shared__ int s_leader_base[kThreads];
  __shared__ int s_perm[kLdsPerm];
  __shared__ int4 s_wave_sums[kWaves + 1];
  __shared__ int s_bad, s_maxlen;

  const int tid = threadIdx.x;
  const SegLayout L = seg_layout(T, S);
  int32_t* perm = rec + L.perm;

  // the first 8192 slot indices stay in registers; all loads are issued at once
  int my_idx[kRegChunks];
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) {
    const int t = c * kThreads + tid;
    const int32_t* src = t < T ? idx + t : reinterpret_cast<const int32_t*>(g_zero16);  // idx may be null when T = 0
    my_idx[c] = *src;
    if (t >= T) my_idx[c] = -1;
  }

  for (int s = tid; s <= S; s += kThreads) {
    if (s < S) s_count[s] = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s_wtab[w][s] = 0;
  }
  if (tid == 0) {
    s_bad = 0;
    s_maxlen = 0;
  }
  __syncthreads();

  // 1. counts
  int bad = 0;
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) {
    const int s = my_idx[c];
    if (s >= 0 && s < S) atomicAdd(&s_count[s], 1);
    else if (s != -1) bad = 1;
  }
  for (int t = kRegChunks * kThreads + tid; t < T; t += kThreads) {
    const int s = idx[t];
    if (s >= 0 && s < S) atomicAdd(&s_count[s], 1);
    else if (s != -1) bad = 1;
  }
  if (bad) s_bad = 1;  // benign: every writer stores 1
  __syncthreads();

  // 2. scans over slots; thread tid owns slot tid (S <= 1024 = kThreads)
  const int n = tid < S ? s_count[tid] : 0;
  int ng = 0, nt = 0;
  if (n > 0) {
    const bool to_tiles = (mode == LORA_MODE_SGMV) || (mode == LORA_MODE_AUTO && n >= kSgmvMinTokens);
    if (to_tiles) nt = (int)ceil_div(n, kTile);
    else ng = (int)ceil_div(n, kGroup);
    atomicMax(&s_maxlen, n);
  }
  int4 sc = make_int4(n, n > 0 ? 1 : 0, ng, nt);
  int4 tot;
  block_exclusive_scan4(sc, s_wave_sums, tot);
  if (tid < S) {
    s_start[tid] = sc.x;
    s_run[tid] = sc.x;
    s_seg[tid] = sc.y;
    s_gofs[tid] = sc.z;
    s_tofs[tid] = sc.w;
  }
  if (tid == 0) {
    s_gofs[S] = tot.z;
    s_tofs[S] = tot.w;
    s_run[S] = tot.x;  // tokens without a slot start after the active ones
  }
  const int num_active = tot.x, num_seg = tot.y, n_groups = tot.z, n_tiles = tot.w;

  // 3. tables and info
  if (n > 0) {
    rec[L.seg_slot + sc.y] = tid;
    rec[L.seg_start + sc.y] = sc.x;
  }
  __syncthreads();
  if (tid == 0) {
    rec[L.seg_start + num_seg] = num_active;
    rec[kNumActive] = num_active;
    rec[kNumSegments] = num_seg;
    rec[kMaxSegLen] = s_maxlen;
    rec[kStatus] = s_bad ? LORA_ERR_INDEX : LORA_OK;
    rec[kNumGroups] = n_groups;
    rec[kNumTiles] = n_tiles;
    rec[kBuiltT] = T;
    rec[kBuiltS] = S;
    for (int w = 8; w < kInfoWords; ++w) rec[w] = 0;
  }

  // 4. stable scatter into perm (and its LDS mirror)
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c)
    if (c * kThreads < T)
      scatter_chunk(c * kThreads + tid, my_idx[c], T, S, perm, s_perm, s_run, s_wtab, s_leader_base);
  for (int c0 = kRegChunks * kThreads; c0 < T; c0 += kThreads) {
    const int t = c0 + tid;
    scatter_chunk(t, t < T ? idx[t] : -1, T, S, perm, s_perm, s_run, s_wtab, s_leader_base);
  }
  if (T > kLdsPerm) __threadfence();  // the items below read perm back from global memory
  __syncthreads();

  // 5. work items: header, then the item's tokens inline (-1 past the count)
  auto perm_at = [&](int pos) -> int {
    if (pos < kLdsPerm) return s_perm[pos];
    return __hip_atomic_load(perm + pos, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  for (int e = tid; e < n_groups * kGroupItemWords; e += kThreads) {
    const int i = e / kGroupItemWords, wd = e - i * kGroupItemWords;
    const int s = upper_slot(s_gofs, S, i);
    const int g = i - s_gofs[s];
    const int p0 = s_start[s] + g * kGroup;
    const int cnt = min(kGroup, s_count[s] - g * kGroup);
    int v;
    if (wd == 0) v = p0;
    else if (wd == 1) v = cnt;
    else if (wd == 2) v = s;
    else if (wd == 3) v = s_seg[s];
    else v = (wd - 4 < cnt) ? perm_at(p0 + wd - 4) : -1;
    rec[L.groups + e] = v;
  }
  for (int e = tid; e < n_tiles * kTileItemWords; e += kThreads) {
    const int i = e / kTileItemWords, wd = e - i * kTileItemWords;
    const int s = upper_slot(s_tofs, S, i);
    const int g = i - s_tofs[s];
    const int p0 = s_start[s] + g * kTile;
    const int cnt = min(kTile, s_count[s] - g * kTile);
    int v;
    if (wd == 0) v = p0;
    else if (wd == 1) v = cnt;
    else if (wd == 2) v = s;
    else if (wd == 3) v = s_seg[s];
    else v = (wd - 4 < cnt) ? perm_at(p0 + wd - 4) : -1;
    rec[L.tiles + e] = v;
  }
}

}  // namespace

hipError_t launch_build_segments(const int32_t* idx, int32_t T, int32_t S, int32_t mode, int32_t* rec,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(build_segments_kernel, dim3(1), dim3(kThreads), 0, stream, idx, T, S, mode, rec);
  return hipGetLastError();
}

}  // namespace lora
