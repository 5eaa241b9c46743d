// The segment build kernels.
//
// Batches of fewer than 512 tokens: one workgroup runs the block-level build
// of segments_block.h -- 1024 threads in general, 256 for small batches
// (T <= kSmallT, S <= 256), where fewer waves mean shorter per-key table walks
// and cheaper barriers.
//
// From 512 tokens: the wide build below.  On one workgroup the build is bound
// by instruction issue on one compute unit (the per-chunk ballots and the
// per-word arithmetic of the item pass: about 10 us at 8192 tokens, 7 us of
// it measured inside the kernel; the wide build takes 7 us in all at 8192
// tokens, 5 us at 1024, and the same 4.5 us at 256).  The
// wide build runs one workgroup per 1024 tokens, and no workgroup waits for
// another: each counts every token of the batch itself (the index vector is
// small and its chunks are counted with LDS adds, one add for a chunk whose
// tokens share a slot), so each knows every slot's total and how many tokens
// of each slot lie before its own range.  Each then runs the same scan over
// slots, and places only its own 1024 tokens:
//   - a token's perm position is its slot's start, plus the slot's tokens
//     before this range, plus those in earlier waves of this range, plus its
//     rank among the lanes of its chunk with its slot (one ballot per key bit);
//   - the token is also written straight into its work item (item = the
//     slot's first item + position in the slot / item capacity), so no pass
//     reads perm back;
//   - each workgroup writes the headers and -1 padding of a share of the
//     items, and workgroup 0 the segment tables and the info words.
// Ranges, waves and lanes are in token order, so the placement is stable and
// the record is the block build's, word for word.
#include <stdlib.h>

#include <type_traits>

#include "segments_block.h"

namespace lora {

namespace {

constexpr int kThreadsLarge = 1024;
constexpr int kThreadsSmall = 256;
constexpr int kSmallT = 1024;
constexpr int kLdsPerm = 8192;  // perm positions mirrored in LDS

template <int kThreads>
__global__ __launch_bounds__(kThreads) void build_segments_kernel(const int32_t* __restrict__ idx, int T, int S,
                                                                  int mode, int32_t* __restrict__ rec) {
  __shared__ SegShared<kThreads, kLdsPerm> sh;
  build_segments_block<kThreads, kLdsPerm>(idx, T, S, mode, rec, sh);
}

// ---------------------------------------------------------------------------
// Wide build
// ---------------------------------------------------------------------------
constexpr int kWThreads = 1024;
constexpr int kWWaves = kWThreads / 64;
constexpr int kWTokens = kWThreads;  // tokens per workgroup: one 64-token chunk per wave
constexpr int kWBatch = 16;          // chunks per wave whose indices are loaded together

struct WideShared {
  int tot[LORA_MAX_SLOTS + 1];           // per key (slot, or S for no slot): tokens in the batch
  int pre[LORA_MAX_SLOTS + 1];           // ... in the ranges of earlier workgroups
  int tab[kWWaves][LORA_MAX_SLOTS + 1];  // ... per wave of this range, then each wave's run start
  int start[LORA_MAX_SLOTS];
  int seg[LORA_MAX_SLOTS];
  int gofs[LORA_MAX_SLOTS + 1];
  int tofs[LORA_MAX_SLOTS + 1];
  int4 wave_sums[kWWaves + 1];
  int bad, maxlen;
};

__global__ __launch_bounds__(kWThreads) void build_segments_wide_kernel(const int32_t* __restrict__ idx, int T,
                                                                        int S, int mode,
                                                                        int32_t* __restrict__ rec) {
  __shared__ WideShared sh;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const SegLayout L = seg_layout(T, S);
  const int P = gridDim.x, b = blockIdx.x;
  int32_t* perm = rec + L.perm;
  const int nbits = 32 - __builtin_clz((unsigned)S);  // keys 0 .. S
  const int n_chunks = (int)ceil_div(T, 64);
  const int own_first = b * kWWaves;  // this workgroup's first chunk
  auto key_of = [&](int v) { return (v >= 0 && v < S) ? v : S; };
  auto to_tiles = [&](int n) { return mode == LORA_MODE_SGMV || (mode == LORA_MODE_AUTO && n >= kSgmvMinTokens); };

  // every load of the first batch is in flight before the tables are cleared:
  // this wave's own chunk, then its chunks of the whole batch
  const int t_own = b * kWTokens + wave * 64 + lane;
  const bool own_valid = t_own < T;
  // unconditional loads: a guarded load becomes a branch, and the compiler
  // waits for every load in flight at the merge; lanes past the batch read its
  // last token and are masked afterwards
  const int own_ld = idx[own_valid ? t_own : T - 1];
  const int own_raw = own_valid ? own_ld : -1;
  int raw[kWBatch];
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int u = 0; u < kWBatch; ++u) {
      const int t = (c0 + u * kWWaves) * 64 + lane;
      raw[u] = idx[t < T ? t : T - 1];
    }
  };
  load_batch(wave);
  for (int k = tid; k <= S; k += kWThreads) {
    sh.tot[k] = 0;
    sh.pre[k] = 0;
  }
  for (int k = lane; k <= S; k += 64) sh.tab[wave][k] = 0;
  if (tid == 0) {
    sh.bad = 0;
    sh.maxlen = 0;
  }
  lds_barrier();

  // 1. every token of the batch: per-key totals, and the part before this range
  int bad = 0;
  for (int c0 = wave; c0 < n_chunks; c0 += kWWaves * kWBatch) {
    if (c0 != wave) load_batch(c0);
    // predicated rather than left early, so that the loop unrolls and each
    // chunk waits only for its own load
#pragma unroll
    for (int u = 0; u < kWBatch; ++u) {
      const int c = c0 + u * kWWaves;
      if (c >= n_chunks) continue;  // uniform
      const bool valid = c * 64 + lane < T;
      const int k = valid ? key_of(raw[u]) : S;
      if (valid && raw[u] != -1 && k == S) bad = 1;
      const bool before = c < own_first;  // uniform
      const uint64_t vmask = __ballot(valid);
      const int first = __builtin_amdgcn_readfirstlane(k);
      if (__ballot(valid && k == first) == vmask) {  // uniform: one key in the chunk
        if (lane == 0) {
          atomicAdd(&sh.tot[first], __popcll(vmask));
          if (before) atomicAdd(&sh.pre[first], __popcll(vmask));
        }
      } else if (valid) {
        atomicAdd(&sh.tot[k], 1);
        if (before) atomicAdd(&sh.pre[k], 1);
      }
    }
  }
  if (bad) sh.bad = 1;  // benign: every writer stores 1
  // this range: per-wave counts and each lane's peers
  const int own_key = key_of(own_raw);
  const uint64_t own_peers = wave_peers(own_key, own_valid, nbits);
  if (own_valid && (own_peers & lt_mask) == 0) sh.tab[wave][own_key] = __popcll(own_peers);
  lds_barrier();

  // 2. the scan over slots (thread tid owns slot tid), then run starts
  const int n_slot = tid < S ? sh.tot[tid] : 0;
  int ng = 0, nt = 0;
  if (n_slot > 0) {
    if (to_tiles(n_slot)) nt = (int)ceil_div(n_slot, kTile);
    else ng = (int)ceil_div(n_slot, kGroup);
  }
  if (wave * 64 < S) {  // uniform: one LDS atomic per wave
    const int wmax = wave_max_nonneg(n_slot);
    if (lane == 0) atomicMax(&sh.maxlen, wmax);
  }
  int4 sc = make_int4(n_slot, n_slot > 0 ? 1 : 0, ng, nt);
  int4 tot4;
  block_exclusive_scan4<kWWaves>(sc, sh.wave_sums, tot4, S);
  const int num_active = tot4.x, num_seg = tot4.y, n_groups = tot4.z, n_tiles = tot4.w;
  if (tid < S) {
    sh.start[tid] = sc.x;
    sh.seg[tid] = sc.y;
    sh.gofs[tid] = sc.z;
    sh.tofs[tid] = sc.w;
    if (b == 0 && n_slot > 0) {
      rec[L.seg_slot + sc.y] = tid;
      rec[L.seg_start + sc.y] = sc.x;
    }
  }
  if (tid == 0) {
    sh.gofs[S] = n_groups;
    sh.tofs[S] = n_tiles;
  }
  lds_barrier();
  for (int k = tid; k <= S; k += kWThreads) {
    int run = (k < S ? sh.start[k] : num_active) + sh.pre[k];
    int c[kWWaves];  // every count is read before any start is written
#pragma unroll
    for (int w = 0; w < kWWaves; ++w) c[w] = sh.tab[w][k];
#pragma unroll
    for (int w = 0; w < kWWaves; ++w) {
      sh.tab[w][k] = run;
      run += c[w];
    }
  }
  if (b == 0 && tid == 0) {
    rec[L.seg_start + num_seg] = num_active;
    rec[kNumActive] = num_active;
    rec[kNumSegments] = num_seg;
    rec[kMaxSegLen] = sh.maxlen;
    rec[kStatus] = sh.bad ? LORA_ERR_INDEX : LORA_OK;
    rec[kNumGroups] = n_groups;
    rec[kNumTiles] = n_tiles;
    rec[kBuiltT] = T;
    rec[kBuiltS] = S;
    for (int w = 8; w < kInfoWords; ++w) rec[w] = 0;
  }
  lds_barrier();

  // 3. this range's tokens into perm and into their items
  if (own_valid) {
    const int pos = sh.tab[wave][own_key] + __popcll(own_peers & lt_mask);
    perm[pos] = t_own;
    if (own_key < S) {
      const int r = pos - sh.start[own_key];
      if (to_tiles(sh.tot[own_key]))
        rec[L.tiles + (int64_t)(sh.tofs[own_key] + r / kTile) * kTileItemWords + 4 + r % kTile] = t_own;
      else
        rec[L.groups + (int64_t)(sh.gofs[own_key] + r / kGroup) * kGroupItemWords + 4 + r % kGroup] = t_own;
    }
  }

  // 4. headers and -1 padding of this workgroup's share of each item list,
  // one thread per item, in 16-byte stores where whole (items and their token
  // lists are 16-byte aligned)
  auto write_share = [&](int n_items, auto cap_c, const int* ofs, int64_t at) {
    constexpr int cap = decltype(cap_c)::value;
    constexpr int words = 4 + cap;
    const int i0 = (int)((int64_t)n_items * b / P), i1 = (int)((int64_t)n_items * (b + 1) / P);
    for (int i = i0 + tid; i < i1; i += kWThreads) {
      const int s = upper_slot(ofs, S, i);
      const int g = i - ofs[s];
      const int cnt = min(cap, sh.tot[s] - g * cap);
      int32_t* item = rec + at + (int64_t)i * words;
      *reinterpret_cast<int4*>(item) = make_int4(sh.start[s] + g * cap, cnt, s, sh.seg[s]);
      const int q = (cnt + 3) & ~3;  // first whole quad of padding
      for (int e = cnt; e < q && e < cap; ++e) item[4 + e] = -1;
      for (int e = q; e < cap; e += 4) *reinterpret_cast<int4*>(item + 4 + e) = make_int4(-1, -1, -1, -1);
    }
  };
  write_share(n_groups, std::integral_constant<int, kGroup>{}, sh.gofs, L.groups);
  write_share(n_tiles, std::integral_constant<int, kTile>{}, sh.tofs, L.tiles);
}

// Smallest T built by the wide build; LORA_SEG_WIDE_MIN_T overrides it.
constexpr int kWideMinT = 512;

int wide_min_t() {
  const char* s = getenv("LORA_SEG_WIDE_MIN_T");
  if (s && *s) {
    const long v = strtol(s, nullptr, 10);
    if (v >= 0 && v <= INT32_MAX) return (int)v;
  }
  return kWideMinT;
}

}  // namespace

hipError_t launch_build_segments(const int32_t* idx, int32_t T, int32_t S, int32_t mode, int32_t* rec,
                                 hipStream_t stream) {
  if (T > 0 && T >= wide_min_t()) {
    hipLaunchKernelGGL(build_segments_wide_kernel, dim3((unsigned)ceil_div(T, kWTokens)), dim3(kWThreads), 0,
                       stream, idx, T, S, mode, rec);
  } else if (T <= kSmallT && S <= kThreadsSmall) {
    hipLaunchKernelGGL(build_segments_kernel<kThreadsSmall>, dim3(1), dim3(kThreadsSmall), 0, stream, idx, T, S,
                       mode, rec);
  } else {
    hipLaunchKernelGGL(build_segments_kernel<kThreadsLarge>, dim3(1), dim3(kThreadsLarge), 0, stream, idx, T, S,
                       mode, rec);
  }
  return hipGetLastError();
}

}  // namespace lora
