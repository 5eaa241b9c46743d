// Fused shrink + expand of one LoRA layer in a single launch, for 16-bit data:
//   v[i][t][k]        = scale[s] * sum_d A_i[s][k][d] * x[t][d]
//   y[t][off_i + j]  += sum_k B_i[s][j][k] * v[i][t][k]
// (the shrink and expand of "Add multi-LoRA support"; the intermediate is fp32
// throughout, as that page's Limitations ask).
//
// Decode-shaped batches move a few MB per layer, and separate shrink and
// expand launches spend most of their time in launch, set-up and the chain of
// dependent memory round trips.  Here the work is cut into 16-token chunks (a
// gather group, or a quarter of a segmented tile) and one launch runs
//   - producer units (chunk, K part, slice): the chunk's [16 x D] by [D x r]
//     contraction over one range of K, on the matrix cores (shrink_unit.h),
//     stored raw into the part's slab of the caller's workspace;
//   - consumer units (chunk, slice, run of 256-column tiles): the expand of the
//     chunk (expand_unit.h), whose fp32 v is the sum of the chunk's slabs, in
//     part order, times the slot's scale.
// A producer stores its slab with device-coherent (agent scope) stores, which
// write through the XCD's L2, waits until they are complete, then increments
// the chunk's counter (a device-coherent atomic).  A consumer requests its
// first y and B rows, polls the counter with device-coherent loads until it
// shows every part, then reads the slabs with ordinary cached loads: no cache
// on the chip can hold a stale copy of a slab line, since every L2 and L1 is
// invalidated when a kernel starts, and in this launch nothing reads a slab
// line before its chunk's counter is complete (slabs are whole 128-byte
// lines, written by one producer unit).  The other consumers of the chunk then
// hit in L2.  (Release and acquire fences at agent scope would instead write
// back or invalidate a whole L2 per wave, which costs far more than the
// layer.)
//   Every workgroup runs all of its producer units before any consumer unit,
// and the grid is no larger than what the chip holds at once, so every
// producer runs while consumers wait; a wait still gives up after a bounded
// number of polls (and counts itself in the workspace's error word), so every
// wave exits.
//   The counters start at zero.  Consumers add their column tiles to the same
// counter, and the unit that brings it to its final value (every part and
// every column tile of the chunk) sets it back to zero, so the next call
// starts from zero again without a clearing pass -- also after a call in
// which a wait gave up.  The workspace layout
// depends only on its size (counters in its first quarter, after a 256-byte
// header), so calls of any shape on one workspace use the same counter region
// and never write their slabs over another call's counters.
//   The chunks come from the batch's segment record (record form) or, when
// the call is given idx (idx form), from a grouping every workgroup builds in
// LDS; in the idx form one workgroup with no unit of its own also builds the
// record (segments_block.h) for the batch's later layers.
#include <stdlib.h>

#include "common.h"
#include "expand_unit.h"
#include "segments_block.h"
#include "shrink_unit.h"

namespace lora {

namespace {

constexpr int kFThreads = kUnitThreads;
constexpr int kFRing = 16384;        // per-wave LDS ring: 64 KB per workgroup, two workgroups per CU
constexpr int kMaxParts = 4;         // K parts per chunk
constexpr int kSumBatch = 4;         // parts whose slabs a consumer loads at once
constexpr int kFusedUnits = 1024;    // at most this many producer slabs when chunks are cut into K parts
constexpr int kSpinLimit = 1 << 20;  // polls (about a microsecond each) before a wait gives up
constexpr int kZeroRowsF = 64;       // tail entries per zero unit
constexpr int kCounterStride = 32;   // int32 words between counters: one 128-byte line each

struct FusedParams {
  ShrinkParams sp;
  ExpandParams ep;
  float* part;        // producer slabs, [slab][16][r_max] fp32
  int32_t* counters;  // [n_slices * chunk_cap]
  int32_t* err;       // waits that gave up
  float* v_out;       // nullable: v written in full when given
  const int32_t* idx; // the batch's slots: grouped in each workgroup (idx mode)
  int spin_limit;     // polls before a wait gives up
  int32_t* rec_out;   // idx mode, nullable: the segment record one workgroup builds
};

// idx mode also builds the batch's segment record, in one workgroup on this
// kernel's four waves (so S <= kFThreads), its tables in that workgroup's
// ring LDS (the batch's T <= TPT x kFThreads positions of perm mirrored).
template <int TPT>
using BuildShared = SegShared<kFThreads, TPT * kFThreads>;

// idx mode: every workgroup groups the batch's tokens by slot itself, in LDS,
// from idx (T <= kFusedMaxTokens): tokens per slot and the first chunk of each
// slot.  A slot's chunks are its tokens, in token order, cut into runs of 16
// (the same pieces as the record's gather groups and tile quarters).
// The kernel's idx form is instantiated for at most 8 tokens per thread
// (T <= 2048) and at most 16 (T <= kFusedMaxTokens): the tokens' slots stay in
// registers through the whole kernel.
constexpr int kTokPerThreadSmall = 8;
constexpr int kTokPerThreadLarge = kFusedMaxTokens / kFThreads;
static_assert(kTokPerThreadLarge * kFThreads == kFusedMaxTokens, "tokens per thread");
struct IdxTables {
  int cnt[LORA_MAX_SLOTS];      // tokens per slot
  int cst[LORA_MAX_SLOTS + 1];  // first chunk of each slot; [S] = chunks
  int rank[LORA_MAX_SLOTS];     // each slot's rank, loaded beside idx
  int scan[kWaves];
  int slot;
};

// Chunk c of the record: gather group c, or for c >= n_g the 16-token quarter
// (c - n_g) % 4 of tile (c - n_g) / 4.  The chunk's token words start at
// `toks`; they can be loaded before the header is checked, so that header and
// tokens arrive in one memory round trip.
struct Chunk {
  bool tiles;
  int64_t item;
  int first;
  const int32_t* toks;
};
__device__ inline Chunk chunk_at(const int32_t* rec, int T, int S, int64_t n_g, int64_t c) {
  Chunk ch;
  ch.tiles = c >= n_g;
  ch.item = ch.tiles ? (c - n_g) >> 2 : c;
  ch.first = ch.tiles ? (int)((c - n_g) & 3) * 16 : 0;
  ch.toks = item_ptr(rec, T, S, ch.tiles, ch.item) + 4 + ch.first;
  return ch;
}
// The chunk's item header (false when it does not check out) and its token
// count (false when 0).
__device__ inline bool chunk_header(const int32_t* rec, int T, int S, const Chunk& ch, Item& it, int& cnt) {
  if (!read_item(rec, T, S, ch.tiles, ch.item, it)) return false;
  cnt = min(16, it.cnt - ch.first);
  return cnt > 0;
}

// TPT: 0 for the record form, else the idx form with at most TPT tokens per
// thread.
template <typename Elem, int TPT>
__global__ __launch_bounds__(kFThreads, 2) void fused_kernel(FusedParams f) {
  constexpr bool FROM_IDX = TPT > 0;
  constexpr int kTokPerThread = TPT > 0 ? TPT : 1;
  __shared__ __attribute__((aligned(1024))) char s_lds[kWaves * kFRing];
  __shared__ int s_tok[16];
  __shared__ IdxTables s_it;

  warm_args(f);
  const ShrinkParams& p = f.sp;
  const int32_t* rec = p.rec;
  const int T = p.T, S = p.S, r_max = p.r_max, ns = p.n_slices;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t G = gridDim.x;
  bool rec_ok = false;
  int na = 0;
  int64_t n_g = 0, n_chunks = 0;
  // idx mode: this thread's tokens t_first .. t_first + tpt - 1 (tpt =
  // ceil(T / threads), so that small batches spread over every thread) and
  // their slots (-1: no valid slot)
  const int tpt = (T + kFThreads - 1) / kFThreads;
  const int t_first = tid * tpt;
  int keys[kTokPerThread];
  if constexpr (FROM_IDX) {
#pragma unroll
    for (int i = 0; i < kTokPerThread; ++i) {
      // an unconditional load (a guarded one becomes a branch, and the
      // compiler waits for every load in flight at the merge), masked after
      const int t = t_first + i;
      const bool in = i < tpt && t < T;
      const int ld = f.idx[in ? t : 0];
      const int k = in ? ld : -1;
      keys[i] = k >= 0 && k < S ? k : -1;
    }
    // the slots' ranks are requested with idx, so that a unit's rank costs no
    // memory round trip of its own once its slot is known
    for (int s = tid; s < S; s += kFThreads) {
      s_it.cnt[s] = 0;
      s_it.rank[s] = slot_rank(p.ranks, s, r_max);
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < kTokPerThread; ++i)
      if (keys[i] >= 0) atomicAdd(&s_it.cnt[keys[i]], 1);
    lds_barrier();
    // chunks per slot, scanned over the slots (4 slots per thread)
    int local = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = 4 * tid + j;
      local += s < S ? (s_it.cnt[s] + 15) >> 4 : 0;
    }
    int total;
    int ex = block_exscan<kWaves>(local, s_it.scan, total);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = 4 * tid + j;
      if (s < S) {
        s_it.cst[s] = ex;
        ex += (s_it.cnt[s] + 15) >> 4;
      }
    }
    if (tid == 0) s_it.cst[S] = total;
    lds_barrier();
    n_chunks = total;
  } else {
    rec_ok = rec[kBuiltT] == T && rec[kBuiltS] == S;
    na = rec_ok ? rec[kNumActive] : 0;
    na = na < 0 ? 0 : (na > T ? T : na);
    n_g = record_items(rec, T, S, false);
    n_chunks = n_g + 4 * record_items(rec, T, S, true);
  }
  // idx mode: the slot, token count and tokens (into s_tok) of chunk c; every
  // thread calls it
  auto idx_chunk = [&](int64_t c, int& s, int& cnt) {
    lds_barrier();  // the previous chunk's s_tok and slot are no longer read
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = 4 * tid + j;
      if (q < S) {
        const int nch = (s_it.cnt[q] + 15) >> 4;
        if (nch > 0 && s_it.cst[q] <= c && c < s_it.cst[q] + nch) s_it.slot = q;
      }
    }
    if (tid < 16) s_tok[tid] = -1;
    lds_barrier();
    s = __builtin_amdgcn_readfirstlane(s_it.slot);
    const int piece = (int)(c - s_it.cst[s]);
    cnt = min(16, s_it.cnt[s] - 16 * piece);
    int m = 0;
#pragma unroll
    for (int i = 0; i < kTokPerThread; ++i) m += keys[i] == s ? 1 : 0;
    int tot;
    int rk = block_exscan<kWaves>(m, s_it.scan, tot) - 16 * piece;  // rank of this thread's first match in the chunk
#pragma unroll
    for (int i = 0; i < kTokPerThread; ++i)
      if (keys[i] == s) {
        if (rk >= 0 && rk < 16) s_tok[rk] = t_first + i;
        ++rk;
      }
    lds_barrier();
  };

  // K parts: enough producer units to cover the grid, at most kFusedUnits
  // slabs, and at least one batch of two K steps per wave in every part
  const int n_steps = (p.D + 4 * Traits<Elem>::kVec - 1) / (4 * Traits<Elem>::kVec);
  // (32-bit arithmetic: a 64-bit division is a long instruction sequence,
  // and these sit on the producers' path)
  int kp = 1;
  if (n_chunks > 0) {
    const int want = (int)min(G, (int64_t)kFusedUnits) / ((int)n_chunks * ns);
    kp = max(1, min(want, min(kMaxParts, max(1, n_steps / (2 * kWaves)))));
  }
  const int per_part = (n_steps + kp - 1) / kp;
  const int64_t n_su = n_chunks * kp * ns;
  const int64_t n_z = f.v_out ? ceil_div(FROM_IDX ? T : T - na, kZeroRowsF) * ns : 0;
  const int32_t* perm = rec + seg_layout(T, S).perm;
  const size_t slab_floats = (size_t)16 * r_max;

  // idx mode with a record to build: one workgroup builds it with the block
  // build of the segment kernel -- the first workgroup with neither producer
  // nor consumer units, else the last one (which then does its units after)
  if constexpr (FROM_IDX) {
    static_assert(sizeof(BuildShared<kTokPerThread>) <= sizeof(s_lds), "the build's tables fit the rings' LDS");
    if (f.rec_out) {
      const ExpandParams& eb = f.ep;
      int64_t pairs = 0;
      for (int i = 0; i < ns; ++i) pairs += n_chunks * ceil_div(eb.out_size[i], kExpandColsPerWG);
      const int64_t ge = min(G, max((int64_t)kXcds, ceil_div(pairs, kXcds) * kXcds));
      // (workgroup kXcds * ceil(units / kXcds) has no producer unit: see below)
      const int64_t bc = kXcds * ceil_div(n_su + n_z, kXcds);
      const int64_t builder = bc < G - ge ? bc : G - 1;
      if (blockIdx.x == builder) {
        build_segments_block<kFThreads, kTokPerThread * kFThreads>(
            f.idx, T, S, LORA_MODE_AUTO, f.rec_out, *reinterpret_cast<BuildShared<kTokPerThread>*>(s_lds));
        __syncthreads();  // the rings' LDS is used again below
      }
    }
  }

  // A chunk's counter returns to zero once every part and every column tile
  // of the chunk has been counted: whichever unit, producer or consumer,
  // brings it to that final value resets it.  Consumers normally come last;
  // a consumer whose wait gave up still counts its tiles, and then the last
  // producer resets, so the counters are zero after every call, even one
  // whose output was invalidated by a give-up.  A producer's returned count is
  // checked only when the workgroup next needs thread 0 idle (its next unit,
  // or its exit), so that the atomic's round trip is not waited for on the way
  // to the consumer units.
  int32_t* pend_ptr = nullptr;
  int pend_old = 0, pend_final = 0;
  auto settle = [&]() {
    if (pend_ptr != nullptr && pend_old + 1 == pend_final)
      __hip_atomic_store(pend_ptr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    pend_ptr = nullptr;
  };

  // ---- producer units (then zero units) on the first workgroups, which the
  // hardware dispatches first: a producer never waits, so the consumers below
  // (on the last workgroups) only ever wait for work that is running or done.
  // The list is cut into kXcds contiguous ranges, range x going to the
  // workgroups of XCD x (blockIdx % kXcds == x) in order, so that the chunks
  // of one slot, which read the same A rows, mostly share one L2 (zipf_many
  // 52.7 -> 51.3 us).  The workgroups holding units are still the first
  // kXcds * ceil(units / kXcds) or fewer.
  const WorkRange pw = xcd_work_range(n_su + n_z);
  for (int64_t u = pw.begin; u < pw.end; u += pw.step) {
    if (u >= n_su) {
      // rows of tokens without an adapter: v = 0
      const int64_t z = u - n_su;
      const int slice = (int)(z % ns);
      float* vb = f.v_out + (int64_t)slice * p.v_slice_stride;
      const int w4 = r_max / 4;
      const int64_t pos0 = na + (z / ns) * kZeroRowsF;
      for (int e = tid; e < kZeroRowsF * w4; e += kFThreads) {
        const int row = e / w4, c = e - row * w4;
        const int64_t pos = pos0 + row;
        if (FROM_IDX) {
          // idx mode: unit z covers token rows 64 z .. 64 z + 63; those
          // without a valid slot are cleared
          const int64_t t = (z / ns) * kZeroRowsF + row;
          if (t < T) {
            const int k = f.idx[t];
            if (k < 0 || k >= S)
              *reinterpret_cast<f32x4*>(vb + t * r_max + 4 * c) = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        } else if (pos < T) {
          const int t = rec_ok ? perm[pos] : (int)pos;
          if (t >= 0 && t < T) *reinterpret_cast<f32x4*>(vb + (int64_t)t * r_max + 4 * c) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      continue;
    }
    const uint32_t uu = (uint32_t)u, un = uu / (uint32_t)ns;  // 32-bit, as above
    const int slice = (int)(uu - un * (uint32_t)ns);
    const int part = (int)(un % (uint32_t)kp);
    const int64_t chunk = un / (uint32_t)kp;
    int s, cnt;
    if constexpr (FROM_IDX) {
      idx_chunk(chunk, s, cnt);
    } else {
      const Chunk ch = chunk_at(rec, T, S, n_g, chunk);
      const int tw = ch.toks[tid & 15];  // requested with the header
      Item it;
      if (!chunk_header(rec, T, S, ch, it, cnt)) continue;  // uniform
      s = __builtin_amdgcn_readfirstlane(it.slot);
      if (tid < 16) s_tok[tid] = tid < cnt ? (tw < 0 ? 0 : (tw >= T ? T - 1 : tw)) : -1;
      __syncthreads();
    }
    const int r = __builtin_amdgcn_readfirstlane(FROM_IDX ? s_it.rank[s] : slot_rank(p.ranks, s, r_max));
    if (r == 0) continue;  // consumers skip such chunks too
    const int s0 = min(n_steps, part * per_part), s1 = min(n_steps, s0 + per_part);
    float* slab = f.part + ((slice * n_chunks + chunk) * kp + part) * slab_floats;
    const int nb = (r + 15) / 16;
    if (ns == 1) contract_rb<Elem, 1, true, kFRing>(p, nb, cnt, s, r, slice, s0, s1, false, slab, s_lds, s_tok, 0, r_max);
    else contract_rb<Elem, 1, false, kFRing>(p, nb, cnt, s, r, slice, s0, s1, false, slab, s_lds, s_tok, 0, r_max);
    // publish: every wave's slab stores are complete before the unit's count
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();  // also: the next unit rewrites s_tok and the rings
    if (tid == 0) {
      settle();  // the previous unit's count has long returned
      pend_ptr = f.counters + (slice * n_chunks + chunk) * kCounterStride;
      pend_final = kp + (int)ceil_div(f.ep.out_size[slice], kExpandColsPerWG);
      pend_old = __hip_atomic_fetch_add(pend_ptr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // ---- consumer units: the pairs (slice, chunk, column tile), cut into equal
  // contiguous shares, the shares of one XCD adjacent.  Each slice's column
  // tiles are cut into blocks of C, and pairs are ordered by slice, block,
  // chunk, column tile.  C is a whole slice unless the B rows of the slots one
  // XCD sees would not stay in its L2; then C is about the pairs per share, so
  // that the chunks of one slot, which read the same B rows, are taken at
  // about the same time by workgroups of one XCD.
  float(*s_tr)[16][kTrRow] = reinterpret_cast<float(*)[16][kTrRow]>(s_lds);  // after the rings' last use
  const ExpandParams& e = f.ep;
  auto n_cols = [&](int i) { return (int)ceil_div(e.out_size[i], kExpandColsPerWG); };
  int64_t P = 0, max_out = 0;
  int max_cols = 1;
  for (int i = 0; i < ns; ++i) {
    P += n_chunks * n_cols(i);
    max_cols = max(max_cols, n_cols(i));
    max_out = max(max_out, e.out_size[i]);
  }
  int64_t Ge = min(G, max((int64_t)kXcds, ceil_div(P, kXcds) * kXcds));
  int64_t ci = G - 1 - blockIdx.x;  // consumer order: the last workgroup first
  if (TPT == kTokPerThreadLarge && f.rec_out && kXcds * ceil_div(n_su + n_z, kXcds) >= G - Ge && G >= 2 * kXcds) {
    // the record's builder is the last workgroup (the same test as above) and
    // the batch is large (T > 2048): the last row of kXcds workgroups takes no
    // share, so that the build, which then runs longer than a share, is not
    // followed by one (zipf_many 60 -> 54 us; at T = 1024 the build is
    // shorter and the row's shares are worth more)
    Ge = min(Ge, G - kXcds);
    ci -= kXcds;
    if (ci < 0) {  // uniform
      if (tid == 0) settle();
      return;
    }
  }
  const int64_t lb = ci / kXcds;
  if (lb >= Ge / kXcds) {  // uniform: no share
    if (tid == 0) settle();
    return;
  }
  const int64_t k = (ci % kXcds) * (Ge / kXcds) + lb;  // ci % 8 names the XCD (G is a multiple of 8)
  const int64_t w0 = P * k / Ge, w1 = P * (k + 1) / Ge;
  // distinct slots in the batch (idx mode: at most the chunks and the slots)
  const int64_t n_seg = FROM_IDX ? max((int64_t)1, min((int64_t)S, n_chunks)) : max(1, rec[kNumSegments]);
  const bool blocked = ceil_div(n_seg, kXcds) * max_out * r_max * (int64_t)sizeof(Elem) > (int64_t)(4 << 20);
  const int C = blocked ? (int)min((int64_t)max_cols, max((int64_t)1, ceil_div(P, Ge))) : max_cols;
  int sl = 0, c0 = 0;  // current block: slice sl, column tiles c0 .. c0 + width - 1
  int64_t base = 0;    // first pair of the block
  auto width = [&]() { return min(C, n_cols(sl) - c0); };
  auto next_block = [&]() {
    base += n_chunks * width();
    c0 += C;
    if (c0 >= n_cols(sl)) {
      c0 = 0;
      ++sl;
    }
  };
  const int n = lane & 15, kg = lane >> 4, yr = lane >> 3;
  for (int64_t pos = w0; pos < w1;) {
    while (sl < ns && pos >= base + n_chunks * width()) next_block();
    if (sl >= ns) break;
    const int nc = n_cols(sl), cb = width();
    const uint32_t rel = (uint32_t)(pos - base), rq = rel / (uint32_t)cb;  // 32-bit division
    const int64_t chunk = rq;
    const int ct_begin = c0 + (int)(rel - rq * (uint32_t)cb);
    const int ct_end = (int)min((int64_t)c0 + cb, ct_begin + (w1 - pos));
    pos += ct_end - ct_begin;
    int s, cnt, tok_n, ytok0, ytok1;
    if constexpr (FROM_IDX) {
      idx_chunk(chunk, s, cnt);
      tok_n = s_tok[n];
      ytok0 = s_tok[yr];
      ytok1 = s_tok[yr + 8];
    } else {
      const Chunk ch = chunk_at(rec, T, S, n_g, chunk);
      const int tw_n = ch.toks[n], tw_y0 = ch.toks[yr], tw_y1 = ch.toks[yr + 8];  // with the header
      Item it;
      if (!chunk_header(rec, T, S, ch, it, cnt)) continue;
      auto tok = [&](int q, int t) { return q < cnt ? (t < 0 ? 0 : (t >= T ? T - 1 : t)) : -1; };
      tok_n = tok(n, tw_n);
      ytok0 = tok(yr, tw_y0);
      ytok1 = tok(yr + 8, tw_y1);
      s = __builtin_amdgcn_readfirstlane(it.slot);
    }
    const int r = __builtin_amdgcn_readfirstlane(FROM_IDX ? s_it.rank[s] : slot_rank(e.ranks, s, r_max));
    const bool write_v = f.v_out && ct_begin == 0 && wave == 0;
    float* vrow = f.v_out ? f.v_out + (int64_t)sl * p.v_slice_stride + (int64_t)(tok_n >= 0 ? tok_n : 0) * r_max
                          : nullptr;
    if (r == 0) {
      // rank 0: no product, v rows are zero
      if (write_v && tok_n >= 0)
        for (int k0 = kg * 8; k0 < r_max; k0 += 32) {
          *reinterpret_cast<f32x4*>(vrow + k0) = f32x4{0.f, 0.f, 0.f, 0.f};
          // fp32 rows may end halfway through a piece of 8 (r_max a multiple of 4)
          if (k0 + 4 < r_max) *reinterpret_cast<f32x4*>(vrow + k0 + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      continue;
    }
    int32_t* cnt_ptr = f.counters + (sl * n_chunks + chunk) * kCounterStride;
    const float* slabs = f.part + (sl * n_chunks + chunk) * kp * slab_floats + n * r_max;
    const float sc = p.scale ? p.scale[s] : 1.0f;
    const int nks = r > 32 ? 2 : 1;
    const int need = kp, final_count = kp + nc, mine = ct_end - ct_begin;
    auto vsrc = [&](f32x4 (&vraw)[2][2]) {
      // one thread polls for the workgroup (every wave calls vsrc once per unit)
      if (tid == 0) {
        int spins = 0;
        while (__hip_atomic_load(cnt_ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
          if (++spins > f.spin_limit) {
            atomicAdd(f.err, 1);
            break;
          }
          __builtin_amdgcn_s_sleep(4);
        }
      }
      lds_barrier();  // the y and B loads stay in flight
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int k0 = ks * 32 + kg * 8;
        const bool ok = tok_n >= 0 && ks < nks && k0 < r;
        f32x4 a0 = f32x4{0.f, 0.f, 0.f, 0.f}, a1 = a0;
        if (ks < nks) {  // uniform
          // the parts' loads in flight kSumBatch at a time, summed in part
          // order (parts past kp read zeros)
          for (int q0 = 0; q0 < kp; q0 += kSumBatch) {
            f32x4 w[kSumBatch][2];
#pragma unroll
            for (int j = 0; j < kSumBatch; ++j) {
              // the second half of the piece only below the rank: an fp32
              // row (r_max a multiple of 4) may end after the first
              const bool okq = ok && q0 + j < kp, okq1 = okq && k0 + 4 < r;
              const float* src = slabs + (okq ? (q0 + j) * slab_floats + k0 : 0);
              w[j][0] = ldf4_or0(src, okq);
              w[j][1] = ldf4_or0(src + (okq1 ? 4 : 0), okq1);
            }
#pragma unroll
            for (int j = 0; j < kSumBatch; ++j) {
              a0 += w[j][0];
              a1 += w[j][1];
            }
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a0[i] = k0 + i < r ? a0[i] * sc : 0.f;
          a1[i] = k0 + 4 + i < r ? a1[i] * sc : 0.f;
        }
        vraw[ks][0] = a0;
        vraw[ks][1] = a1;
        if (write_v && tok_n >= 0 && k0 < r_max) {
          *reinterpret_cast<f32x4*>(vrow + k0) = a0;
          if (k0 + 4 < r_max) *reinterpret_cast<f32x4*>(vrow + k0 + 4) = a1;
        }
      }
    };
    if constexpr (sizeof(Elem) == 4)
      expand_group_f32(e, vsrc, tok_n, s_tr[wave], sl, s, r, (int)e.out_size[sl], ct_begin, ct_end);
    else
      expand_group_direct<Elem>(e, vsrc, ytok0, ytok1, s_tr, sl, s, r, (int)e.out_size[sl], ct_begin, ct_end);
    // this unit's column tiles are counted as consumed (after its y stores are
    // issued, so the atomic's round trip overlaps them); the last consumer of
    // the chunk sets the counter back to zero for the next call
    if (tid == 0) {
      const int old = __hip_atomic_fetch_add(cnt_ptr, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old + mine == final_count) __hip_atomic_store(cnt_ptr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (tid == 0) settle();
}

template <typename Elem, int TPT>
const void* fused_kernel_ptr() {
  return reinterpret_cast<const void*>(&fused_kernel<Elem, TPT>);
}

template <typename Elem, int TPT>
bool fused_fits() {
  // the grid (a multiple of 8, at least 8) must be resident at once, and the
  // consumer shares assume at least two rows of 8 workgroups
  const void* kernel = fused_kernel_ptr<Elem, TPT>();
  const int grid = persistent_grid(kernel, kFThreads, 0, INT64_MAX / 4);
  return grid >= 2 * kXcds && grid <= resident_workgroups(kernel, kFThreads, 0);
}

template <typename Elem, int TPT>
hipError_t fused_launch(const FusedParams& f, hipStream_t stream) {
  const void* kernel = fused_kernel_ptr<Elem, TPT>();
  // the grid is what the chip holds at once: consumers wait for producers
  const int grid = persistent_grid(kernel, kFThreads, 0, INT64_MAX / 4);
  if (!fused_fits<Elem, TPT>()) return hipErrorInvalidConfiguration;  // the caller checked fused_coresident
  hipLaunchKernelGGL((fused_kernel<Elem, TPT>), dim3(grid), dim3(kFThreads), 0, stream, f);
  return hipGetLastError();
}

}  // namespace

int64_t fused_need_bytes(int64_t T, int64_t S, int64_t n_slices, int64_t r_max) {
  const SegLayout L = seg_layout(T, S);
  const int64_t units = n_slices * (L.cap_groups + 4 * L.cap_tiles);  // counters
  const int64_t slabs = (units > kFusedUnits ? units : kFusedUnits) * 16 * r_max * 4;
  const int64_t v_bytes = n_slices * T * r_max * 4;  // v of the two-launch form
  const int64_t data = slabs > v_bytes ? slabs : v_bytes;
  // the counter region is a quarter of the whole, at least 128 bytes per
  // counter; the rest holds the data after 512 bytes of header and alignment
  int64_t b = ceil_div((data + 512) * 4, 3);
  if (b < 4 * 128 * (units + 1)) b = 4 * 128 * (units + 1);
  return (b + 255) & ~int64_t(255);
}

FusedLayout fused_layout(int64_t bytes) {
  FusedLayout W;
  W.counters = 256;
  W.counter_bytes = (bytes / 4) & ~int64_t(127);
  W.part = (W.counters + W.counter_bytes + 255) & ~int64_t(255);
  return W;
}

bool fused_coresident(lora_dtype dt, int32_t T, bool from_idx) {
  const int tpt = !from_idx ? 0 : (T <= kTokPerThreadSmall * kFThreads ? kTokPerThreadSmall : kTokPerThreadLarge);
  switch (dt) {
    case LORA_F32:  // fp32: the record form and the idx form of at most 8 tokens per thread
      return T <= kF32FusedMaxTokens &&
             (tpt == 0 ? fused_fits<float, 0>() : fused_fits<float, kTokPerThreadSmall>());
    case LORA_F16:
      return tpt == 0 ? fused_fits<half_t, 0>()
                      : tpt == kTokPerThreadSmall ? fused_fits<half_t, kTokPerThreadSmall>()
                                                  : fused_fits<half_t, kTokPerThreadLarge>();
    case LORA_BF16:
      return tpt == 0 ? fused_fits<bf16_t, 0>()
                      : tpt == kTokPerThreadSmall ? fused_fits<bf16_t, kTokPerThreadSmall>()
                                                  : fused_fits<bf16_t, kTokPerThreadLarge>();
    default: return false;
  }
}

hipError_t launch_fused(lora_dtype dt, const ShrinkParams& sp, const ExpandParams& ep, const int32_t* idx, char* ws,
                        int64_t ws_bytes, float* v_out, hipStream_t stream) {
  const FusedLayout W = fused_layout(ws_bytes);
  FusedParams f;
  f.sp = sp;
  f.ep = ep;
  f.part = reinterpret_cast<float*>(ws + W.part);
  f.counters = reinterpret_cast<int32_t*>(ws + W.counters);
  f.err = reinterpret_cast<int32_t*>(ws);
  f.v_out = v_out;
  f.idx = idx;
  f.rec_out = idx ? const_cast<int32_t*>(sp.rec) : nullptr;
  // LORA_MI355X_FUSED_SPIN_LIMIT (a count of polls >= 0) replaces the bound on
  // the consumers' waits, so that tests can force the give-up path from the host
  f.spin_limit = kSpinLimit;
  if (const char* e = getenv("LORA_MI355X_FUSED_SPIN_LIMIT")) {
    const long v = strtol(e, nullptr, 10);
    if (v >= 0 && v < kSpinLimit) f.spin_limit = (int)v;
  }
  // record form, or the idx form with at most 8 or 16 tokens per thread
  const int tpt = idx == nullptr ? 0 : (sp.T <= kTokPerThreadSmall * kFThreads ? kTokPerThreadSmall : kTokPerThreadLarge);
  switch (dt) {
    case LORA_F32:
      if (sp.T > kF32FusedMaxTokens) return hipErrorInvalidValue;
      return tpt == 0 ? fused_launch<float, 0>(f, stream) : fused_launch<float, kTokPerThreadSmall>(f, stream);
    case LORA_F16:
      return tpt == 0 ? fused_launch<half_t, 0>(f, stream)
                      : tpt == kTokPerThreadSmall ? fused_launch<half_t, kTokPerThreadSmall>(f, stream)
                                                  : fused_launch<half_t, kTokPerThreadLarge>(f, stream);
    case LORA_BF16:
      return tpt == 0 ? fused_launch<bf16_t, 0>(f, stream)
                      : tpt == kTokPerThreadSmall ? fused_launch<bf16_t, kTokPerThreadSmall>(f, stream)
                                                  : fused_launch<bf16_t, kTokPerThreadLarge>(f, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lora
