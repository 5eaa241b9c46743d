// Segment build: group a batch's active tokens by adapter slot and plan the
// kernel work items.  The token index vector is built on the host and moved to
// the device once per batch ("[Hardware][TPU][V1] Better tpu multilora
// compilation", review of the token index buffer); every LoRA layer of the
// batch then reuses this record.
//
// One workgroup (16 waves; 4 for batches of at most 1024 tokens and 256
// slots) does everything, so the result is bit-exact and deterministic.  Wave w owns the contiguous token range
// [w R, (w + 1) R), walked in chunks of 64 (one token per lane).  The key of a
// token is its slot, or S for a token without a valid slot (those follow every
// active token in perm, ascending, and the shrink clears their v rows).
//   1. Counts: in each chunk the lanes with one key find each other with one
//      ballot per bit of the key; the lowest of them adds their number to the
//      wave's row of a per-(wave, key) count table.  No atomics.
//   2. One thread per key sums its column of the table, a block-wide scan over
//      slots gives each slot's start in perm, its segment number and the
//      offsets of its work items, and the column is turned into the start of
//      each wave's run of that key.  Segment tables and info words follow.
//   3. Scatter: each wave walks its range again; a token lands at its wave's
//      run start for its key plus its rank among the chunk's lanes with that
//      key, and the run start advances by their number.  Ranges, chunks and
//      lanes are all in token order, so the placement is stable, and since a
//      wave only touches its own row no barrier is needed.
//   4. Work items, each followed by its token indices, read back from an LDS
//      mirror of perm (from global memory past 8192 tokens).
// Chunks held in registers keep their keys and lane masks from step 1 to step
// 3.  Barriers that only order LDS traffic do not wait for the record's global
// stores.
#pragma once

#include <type_traits>

#include "common.h"

namespace lora {

namespace {

// The build is one workgroup of NT threads (a multiple of 64, at least S: a
// slot is owned by thread `slot` in the scan), with its tables in the LDS
// block SegShared.
constexpr int kRegChunks = 8;   // chunks per wave kept in registers
constexpr int kItemTab = 2048;  // items whose slot is tabulated in LDS

__device__ inline int lane_id() { return __lane_id(); }

// Barriers here are lds_barrier(): __syncthreads() would also wait for every
// outstanding global store (the perm and table writes).

// Lanes of this wave (valid ones only) whose key equals this lane's: one ballot
// per bit of the key, keys being below 2^nbits; a chunk whose valid lanes all
// hold one key (a prefill segment) needs a single ballot.
__device__ inline uint64_t wave_peers(int key, bool valid, int nbits) {
  uint64_t peers = __ballot(valid);
  const int first = __builtin_amdgcn_readlane(key, peers ? __builtin_ctzll(peers) : 0);
  if (__ballot(valid && key == first) == peers) return valid ? peers : 0;  // uniform
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return valid ? peers : 0;
}

// Cross-lane moves on the DPP network (no LDS round trip): lane i of a row of
// 16 takes lane i - n of its row (0 past the row's start); a row broadcast
// hands lane 15 (31) to the rows selected by the mask (rows 1 and 3 for lane
// 15, rows 2 and 3 for lane 31), the other rows receiving 0.
template <int kCtrl, int kRowMask = 0xf>
__device__ inline int dpp_or0(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, kRowMask, 0xf, true);
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// Inclusive scan of one int across the wave: within rows of 16 by shifts of
// 1, 2, 4, 8, then across rows by the two broadcasts.
__device__ inline int wave_inclusive_scan(int v) {
  v += dpp_or0<kRowShr1>(v);
  v += dpp_or0<kRowShr2>(v);
  v += dpp_or0<kRowShr4>(v);
  v += dpp_or0<kRowShr8>(v);
  v += dpp_or0<kRowBcast15, 0xa>(v);
  v += dpp_or0<kRowBcast31, 0xc>(v);
  return v;
}

// Maximum of one non-negative int over the wave (the same pattern with max;
// 0 is the identity), returned to every lane.
__device__ inline int wave_max_nonneg(int v) {
  v = max(v, dpp_or0<kRowShr1>(v));
  v = max(v, dpp_or0<kRowShr2>(v));
  v = max(v, dpp_or0<kRowShr4>(v));
  v = max(v, dpp_or0<kRowShr8>(v));
  v = max(v, dpp_or0<kRowBcast15, 0xa>(v));
  v = max(v, dpp_or0<kRowBcast31, 0xc>(v));
  return __builtin_amdgcn_readlane(v, 63);
}

// Block-wide exclusive scan of four ints per thread (thread order), returning
// the exclusive prefixes and writing the four totals to `total`.  Only threads
// below S hold nonzero values; with S <= 64 one wave's scan is the whole scan.
template <int kWaves>
__device__ inline void block_exclusive_scan4(int4& v, int4* wave_sums, int4& total, int S) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  int4 inc = v;  // waves past the slots hold zeros: their scan is the identity
  if (wave * 64 < S) {  // uniform
    inc.x = wave_inclusive_scan(v.x);
    inc.y = wave_inclusive_scan(v.y);
    inc.z = wave_inclusive_scan(v.z);
    inc.w = wave_inclusive_scan(v.w);
  }
  if (S <= 64) {  // uniform
    if (wave == 0 && lane == 63) wave_sums[0] = inc;
    lds_barrier();
    total = wave_sums[0];
    v = make_int4(inc.x - v.x, inc.y - v.y, inc.z - v.z, inc.w - v.w);
    return;
  }
  if (lane == 63) wave_sums[wave] = inc;
  lds_barrier();
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
  lds_barrier();
  int4 base = wave_sums[wave];
  total = wave_sums[kWaves];
  v = make_int4(base.x + inc.x - v.x, base.y + inc.y - v.y, base.z + inc.z - v.z, base.w + inc.w - v.w);
}

// Exclusive prefix sum of one int over a workgroup of kW waves (thread order),
// and the total.  Every thread calls it; scan holds kW ints of LDS.
template <int kW>
__device__ inline int block_exscan(int v, int* scan, int& total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int x = wave_inclusive_scan(v);  // DPP row shifts and broadcasts, no LDS round trips
  if (lane == 63) scan[wave] = x;
  lds_barrier();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    const int t = scan[w];
    before += w < wave ? t : 0;
    total += t;
  }
  lds_barrier();  // scan may be rewritten
  return before + x - v;
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

// The LDS tables of one build: per-(wave, key) counts (then run starts), the
// per-slot tables, the item-to-slot tables and a mirror of perm's first
// kPermLds positions.
template <int kThreads, int kPermLds>
struct SegShared {
  int tab[kThreads / 64][LORA_MAX_SLOTS + 1];
  int count[LORA_MAX_SLOTS];
  int start[LORA_MAX_SLOTS];
  int seg[LORA_MAX_SLOTS];
  int gofs[LORA_MAX_SLOTS + 1];
  int tofs[LORA_MAX_SLOTS + 1];
  int16_t gslot[kItemTab];  // slot of gather item i
  int16_t tslot[kItemTab];  // slot of segmented item i
  int perm[kPermLds];
  int4 wave_sums[kThreads / 64 + 1];
  int bad, maxlen;
};

// The whole build by one workgroup of kThreads threads (S <= kThreads), every
// thread calling it; the record is complete once the workgroup's stores are.
template <int kThreads, int kPermLds>
__device__ __forceinline__ void build_segments_block(const int32_t* __restrict__ idx, int T, int S, int mode,
                                                     int32_t* __restrict__ rec, SegShared<kThreads, kPermLds>& sh) {
  constexpr int kWaves = kThreads / 64;
  auto& s_tab = sh.tab;
  auto& s_count = sh.count;
  auto& s_start = sh.start;
  auto& s_seg = sh.seg;
  auto& s_gofs = sh.gofs;
  auto& s_tofs = sh.tofs;
  auto& s_gslot = sh.gslot;
  auto& s_tslot = sh.tslot;
  auto& s_perm = sh.perm;
  auto& s_wave_sums = sh.wave_sums;
  int& s_bad = sh.bad;
  int& s_maxlen = sh.maxlen;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const SegLayout L = seg_layout(T, S);
  int32_t* perm = rec + L.perm;
  const int R = (int)ceil_div(ceil_div(T, kWaves), 64) * 64;  // tokens per wave
  const int n_chunks = R / 64;
  const int t_begin = wave * R;
  const int nbits = 32 - __builtin_clz((unsigned)S);  // keys 0 .. S

  // the first kRegChunks chunks of the wave's slot indices are loaded at once
  int key[kRegChunks];
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) {
    const int t = t_begin + c * 64 + lane;
    const bool in = c < n_chunks && t < T;
    const int32_t* src = in ? idx + t : reinterpret_cast<const int32_t*>(g_zero16);  // idx may be null when T = 0
    key[c] = *src;
  }

  for (int e = tid; e < kWaves * (S + 1); e += kThreads) s_tab[e / (S + 1)][e % (S + 1)] = 0;
  if (tid == 0) {
    s_bad = 0;
    s_maxlen = 0;
  }
  lds_barrier();

  // 1. per-(wave, key) counts
  int bad = 0;
  uint64_t peers_reg[kRegChunks];
  // A chunk whose valid lanes all hold one key (a prefill segment) adds to a
  // pending run kept in registers, flushed when the key changes, so that long
  // segments do not chain one LDS read-modify-write per chunk.
  int run_key = -1, run_cnt = 0;
  auto flush_run = [&]() {
    if (run_cnt > 0 && lane == 0) s_tab[wave][run_key] += run_cnt;
    run_cnt = 0;
  };
  auto count_chunk = [&](int t, int& k) -> uint64_t {
    const bool valid = t < T;
    if (valid && !(k >= 0 && k < S)) {
      if (k != -1) bad = 1;
      k = S;
    }
    const uint64_t peers = wave_peers(k, valid, nbits);
    const uint64_t all = __ballot(valid);
    if (all != 0 && __ballot(valid && peers == all) == all) {  // uniform: one key in the whole chunk
      const int key0 = __builtin_amdgcn_readfirstlane(k);
      if (key0 != run_key) {
        flush_run();
        run_key = key0;
      }
      run_cnt += __popcll(all);
    } else if (valid && (peers & lt_mask) == 0) {
      s_tab[wave][k] += __popcll(peers);  // one lane per key
    }
    return peers;
  };
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) {
    peers_reg[c] = 0;
    if (c < n_chunks) peers_reg[c] = count_chunk(t_begin + c * 64 + lane, key[c]);  // uniform condition
  }
  for (int c = kRegChunks; c < n_chunks; ++c) {
    const int t = t_begin + c * 64 + lane;
    int k = t < T ? idx[t] : -1;
    count_chunk(t, k);
  }
  flush_run();
  if (bad) s_bad = 1;  // benign: every writer stores 1
  lds_barrier();

  // 2. scan over slots (thread tid owns slot tid; S <= 1024), then run starts
  int n_slot = 0;
  if (tid < S) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) n_slot += s_tab[w][tid];
  }
  int ng = 0, nt = 0;
  if (n_slot > 0) {
    const bool to_tiles = (mode == LORA_MODE_SGMV) || (mode == LORA_MODE_AUTO && n_slot >= kSgmvMinTokens);
    if (to_tiles) nt = (int)ceil_div(n_slot, kTile);
    else ng = (int)ceil_div(n_slot, kGroup);
  }
  if (wave * 64 < S) {  // uniform: one LDS atomic per wave, not one per slot
    const int wmax = wave_max_nonneg(n_slot);
    if (lane == 0) atomicMax(&s_maxlen, wmax);
  }
  int4 sc = make_int4(n_slot, n_slot > 0 ? 1 : 0, ng, nt);
  int4 tot;
  block_exclusive_scan4<kWaves>(sc, s_wave_sums, tot, S);
  const int num_active = tot.x, num_seg = tot.y, n_groups = tot.z, n_tiles = tot.w;
  // keys 0 .. S (key S, the tokens without a slot, starts after every active
  // token; with S = 1024 thread 0 also takes it)
  for (int k = tid; k <= S; k += kThreads) {
    int run = k < S ? sc.x : num_active;
    int c[kWaves];  // every count is read before any start is written
#pragma unroll
    for (int w = 0; w < kWaves; ++w) c[w] = s_tab[w][k];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      s_tab[w][k] = run;
      run += c[w];
    }
  }
  if (tid < S) {
    s_count[tid] = n_slot;
    s_start[tid] = sc.x;
    s_seg[tid] = sc.y;
    s_gofs[tid] = sc.z;
    s_tofs[tid] = sc.w;
    for (int g = 0; g < ng && sc.z + g < kItemTab; ++g) s_gslot[sc.z + g] = (int16_t)tid;
    for (int g = 0; g < nt && sc.w + g < kItemTab; ++g) s_tslot[sc.w + g] = (int16_t)tid;
    if (n_slot > 0) {
      rec[L.seg_slot + sc.y] = tid;
      rec[L.seg_start + sc.y] = sc.x;
    }
  }
  if (tid == 0) {
    s_gofs[S] = n_groups;
    s_tofs[S] = n_tiles;
    rec[L.seg_start + num_seg] = num_active;
    rec[kNumActive] = num_active;
    rec[kNumSegments] = num_seg;
    rec[kStatus] = s_bad ? LORA_ERR_INDEX : LORA_OK;
    rec[kNumGroups] = n_groups;
    rec[kNumTiles] = n_tiles;
    rec[kBuiltT] = T;
    rec[kBuiltS] = S;
    for (int w = 8; w < kInfoWords; ++w) rec[w] = 0;
  }
  lds_barrier();
  if (tid == 0) rec[kMaxSegLen] = s_maxlen;

  // 3. stable scatter: each wave only touches its own row of s_tab
  auto place_chunk = [&](int t, int k, uint64_t peers) {
    const bool valid = t < T;
    int base = 0;
    if (valid) base = s_tab[wave][k];  // every lane of the key reads before its first lane writes
    if (valid && (peers & lt_mask) == 0) s_tab[wave][k] = base + __popcll(peers);
    if (valid) {
      const int pos = base + __popcll(peers & lt_mask);
      perm[pos] = t;
      if (pos < kPermLds) s_perm[pos] = t;
    }
  };
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c)
    if (c < n_chunks) place_chunk(t_begin + c * 64 + lane, key[c], peers_reg[c]);
  for (int c = kRegChunks; c < n_chunks; ++c) {
    const int t = t_begin + c * 64 + lane;
    int k = t < T ? idx[t] : -1;
    if (!(k >= 0 && k < S)) k = S;
    place_chunk(t, k, wave_peers(k, t < T, nbits));
  }
  if (T > kPermLds) {
    __threadfence();  // the items below read perm back from global memory
    __syncthreads();
  } else {
    lds_barrier();
  }

  // 4. work items: header, then the item's tokens inline (-1 past the count)
  auto perm_at = [&](int pos) -> int {
    if (pos < kPermLds) return s_perm[pos];
    return __hip_atomic_load(perm + pos, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // Each thread takes four words at a time, so that their chains of LDS
  // lookups overlap.
  auto write_items = [&](int n_items, auto words_c, int cap, const int* s_ofs, const int16_t* s_islot, int64_t at) {
    constexpr int words = decltype(words_c)::value;  // a constant: the divisions below are multiplies
    const int total = n_items * words;
    for (int e0 = tid; e0 < total; e0 += 4 * kThreads) {
      int val[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * kThreads;
        const int ec = e < total ? e : 0;
        const int i = ec / words, wd = ec - i * words;
        const int s = i < kItemTab ? (int)s_islot[i] : upper_slot(s_ofs, S, i);
        const int g = i - s_ofs[s];
        const int p0 = s_start[s] + g * cap;
        const int cnt = min(cap, s_count[s] - g * cap);
        int v;
        if (wd == 0) v = p0;
        else if (wd == 1) v = cnt;
        else if (wd == 2) v = s;
        else if (wd == 3) v = s_seg[s];
        else v = (wd - 4 < cnt) ? perm_at(p0 + wd - 4) : -1;
        val[u] = v;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (e0 + u * kThreads < total) rec[at + e0 + u * kThreads] = val[u];
    }
  };
  write_items(n_groups, std::integral_constant<int, kGroupItemWords>{}, kGroup, s_gofs, s_gslot, L.groups);
  write_items(n_tiles, std::integral_constant<int, kTileItemWords>{}, kTile, s_tofs, s_tslot, L.tiles);
}

}  // namespace

}  // namespace lora
