// Shrink: v[i][t][k] = scale[s] * sum_d A_i[s][k][d] * x[t][d] for every slice i
// ("Add multi-LoRA support", the shrink of the punica kernels; the scale is
// applied to the fp32 value), with the intermediate cleared inside the call
// ("[LoRA] LoRA cuda graph specialization", Implementation).
//
// One launch covers the whole segment record.  Its work units are
//   - the record's items, once per slice: a gather group (at most 16 tokens of
//     one slot) or a segmented tile (at most 64 tokens of one slot).  For the
//     item's tokens the unit computes D[token][rank] = X A_s^T, a [cnt x D] by
//     [D x r_s] contraction, on the matrix cores with fp32 accumulation;
//   - zero units: 64 consecutive entries of the record's tail of tokens without
//     an adapter, whose v rows are cleared.
// Every v row of the batch is written exactly once with plain stores: the rows
// of active tokens with their values (0 in rank columns k >= r_s), the others
// with zeros.  There is no separate clearing pass and no atomic, and the result
// does not depend on how the units are scheduled.
//
// Inside a unit the four waves split the contraction index d between them.  A
// K step is 64 bytes of every operand row: 32 elements of a 16-bit type (one
// v_mfma_f32_16x16x32) or 16 fp32 elements (four v_mfma_f32_16x16x4f32).  A
// batch is two steps, one 128-byte cache line of every row; wave w takes batches
// w, w + 4, w + 8, .. so that the workgroup reads 512 contiguous bytes of each
// row per round.  MFMA wants lane l to hold 16 bytes of row l % 16, so loading
// operands straight into registers makes every group of 16 lanes touch 16
// different rows, and a compute unit then streams only about a third of what it
// does with whole-line accesses.  Each wave therefore copies its batches into
// its own LDS ring with global-to-LDS loads in which 8 lanes fetch one whole
// row line, several batches ahead, and reads them back in MFMA layout.  The 16
// byte pieces of a row are stored XOR-swizzled by row so that those reads are
// free of bank conflicts.  Only the wave's own loads fill its ring, so the
// wave waits on its own load counter and no barrier is needed.  At the end the
// four waves' partial sums meet in LDS, where each 16 x 16 block is summed,
// scaled and stored by one wave.
#include "common.h"

namespace lora {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kZeroRows = 64;                                    // tail entries per zero unit

// One K step: one 16-byte operand per lane and 16-row block.
template <typename Elem> struct StepMma;
template <> struct StepMma<bf16_t> {
  __device__ static inline f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
};
template <> struct StepMma<half_t> {
  __device__ static inline f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
};
template <> struct StepMma<float> {
  // Element e of every lane's 4 values forms one 16x16x4 product whose K index
  // is the lane's 16-lane group: the four products together cover the 16
  // elements of the step.
  __device__ static inline f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t ae = a[e], be = b[e];
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(ae), __uint_as_float(be), c, 0, 0, 0);
    }
    return c;
  }
};

constexpr int kRingBytes = 32768;  // LDS ring of one wave (also holds its partial sums)
constexpr int kBlockBytes = 2048;  // one batch of one 16-row block: 16 rows x 128 bytes

// One global-to-LDS load: every lane fetches the 16 bytes at base + voff (base
// wave-uniform) and they land at LDS byte lds + 16 * lane.  Issued by hand: the
// compiler, which cannot tell the ring's slots apart, would otherwise wait for
// every load in flight before each LDS read.  M0 is saved and restored around
// it.
__device__ inline void load_to_lds(const char* base, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(base)
      : "memory");
}
// The same with a non-temporal hint, for rows read once.
__device__ inline void load_to_lds_nt(const char* base, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(base)
      : "memory");
}

// Wait until at most n (a multiple of `unit`, at most 7 units and at most 63,
// the counter's range) of this wave's vector memory operations are outstanding.
template <int k, int unit>
__device__ inline void wait_vm_const() {
  constexpr int n = k * unit < 63 ? k * unit : 63;  // larger cases never occur
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
}
template <int unit>
__device__ inline void wait_vm(int n) {
  switch (n / unit) {
    case 0: wait_vm_const<0, unit>(); break;
    case 1: wait_vm_const<1, unit>(); break;
    case 2: wait_vm_const<2, unit>(); break;
    case 3: wait_vm_const<3, unit>(); break;
    case 4: wait_vm_const<4, unit>(); break;
    case 5: wait_vm_const<5, unit>(); break;
    case 6: wait_vm_const<6, unit>(); break;
    default: wait_vm_const<7, unit>(); break;
  }
}

// Clear v columns [c0, c1) of the unit's token rows (s_tok, -1 = none),
// spread over the threads [first, first + count).
__device__ inline void clear_columns(float* vb, int r_max, const int* s_tok, int cnt, int c0, int c1, int first,
                                     int count) {
  const int w4 = (c1 - c0) / 4;  // r_max, c0 and c1 are multiples of 4
  if (w4 <= 0) return;
  for (int e = threadIdx.x - first; e < cnt * w4; e += count) {
    const int row = e / w4, c = e - row * w4;
    const int t = s_tok[row];
    if (t >= 0) *reinterpret_cast<f32x4*>(vb + (int64_t)t * r_max + c0 + 4 * c) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// One unit: RB blocks of 16 tokens by NB blocks of 16 ranks, over the K steps
// [s0, s1) of the contraction.  s_tok holds the unit's tokens, -1 past the
// count (written before a barrier); the ranks are c_lo .. c_lo + 16 NB - 1 of
// the slot (rank r), and the unit owns v columns [c_lo, c_hi).  s_lds is the
// workgroup's four rings.  With `partial` the unit is one of several parts of
// the contraction: it adds its sums to v with atomics (v was cleared
// beforehand) and leaves the other columns alone; otherwise it stores its
// columns whole (zeros past the rank).  XONCE: no other unit reads this
// unit's x rows (one slice, no rank pieces), so they are loaded with a
// non-temporal hint and do not displace reused data from the caches.
template <typename Elem, int RB, int NB, bool XONCE>
__device__ __forceinline__ void contract_unit(const ShrinkParams& p, int cnt, int s, int r, int slice, int s0,
                                              int s1, bool partial, char* s_lds, const int* s_tok, int c_lo,
                                              int c_hi) {
  using M = StepMma<Elem>;
  constexpr int kVec = Traits<Elem>::kVec;
  constexpr int kStep = 4 * kVec;  // elements per K step (64 bytes)
  constexpr int NBLK = RB + NB;
  constexpr int kSlot = NBLK * kBlockBytes;              // one batch of every block
  constexpr int DEPTH = kRingBytes / kSlot < 8 ? kRingBytes / kSlot : 8;
  constexpr int IPB = 2 * NBLK;                          // loads per batch
  static_assert((DEPTH - 1) * IPB <= 63, "the ring's loads must fit the wait counter");
  const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, kg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  char* ring = s_lds + wave * kRingBytes;

  // Operand rows.  Block bk < RB holds tokens bk * 16 .. of the item, block
  // RB + nb rank rows nb * 16 ..  Rows of a MFMA product do not mix, so a row
  // whose token or rank does not exist is read from one that does (the item's
  // first token, the slot's last rank row): its outputs are discarded, and its
  // loads hit addresses another lane loads too.  Addresses are a wave-uniform
  // base plus a 32-bit byte offset (the host checks that x and one slot's A rows
  // each span less than 4 GiB).
  //
  // Global-to-LDS load q (0, 1) of a block: lane l fetches row 8 q + l / 8, the
  // 16-byte piece (l % 8) ^ (l / 8) of the batch's line of that row, and lands
  // at byte 16 l of the load's 1 KB.
  const char* xb = reinterpret_cast<const char*>(p.x);
  const char* ab = reinterpret_cast<const char*>(p.A[slice]) +
                   ((int64_t)s * p.r_max + c_lo) * p.D * (int64_t)sizeof(Elem);
  const int r_loc = min(r, c_hi) - c_lo;  // rank rows of this unit, >= 1
  const int t0 = s_tok[0];  // cnt >= 1: a valid token
  const uint32_t piece = (uint32_t)(((lane & 7) ^ (lane >> 3)) * 16);
  uint32_t so[NBLK][2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = 8 * q + (lane >> 3);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int t = s_tok[rb * 16 + row];
      so[rb][q] = (uint32_t)((int64_t)(t >= 0 ? t : t0) * p.ldx * (int64_t)sizeof(Elem)) + piece;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int k = nb * 16 + row;
      so[RB + nb][q] = (uint32_t)((int64_t)(k < r_loc ? k : r_loc - 1) * p.D * (int64_t)sizeof(Elem)) + piece;
    }
  }
  // MFMA reads: step j of a batch gives K slot kg the piece 4 j + kg of row m
  uint32_t rd[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) rd[j] = (uint32_t)((m >> 3) * 1024 + (m & 7) * 128 + (((4 * j + kg) ^ (m & 7)) * 16));

  f32x4 acc[RB][NB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // batches of this unit: b covers steps s0 + 2 b, s0 + 2 b + 1; the full ones
  // lie wholly inside D and [s0, s1)
  const int full_end = min(s1, p.D / kStep);
  const int n_full = max(0, (full_end - s0) / 2);
  const int my_n = n_full > wave ? (n_full - wave + kWaves - 1) / kWaves : 0;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;  // LDS byte address of the ring
  auto issue = [&](int i) {  // the wave's i-th batch into ring slot i % DEPTH
    const uint32_t boff = (uint32_t)(s0 + 2 * (wave + kWaves * i)) * 64u;
    const uint32_t dst = ring_lds + (uint32_t)((i % DEPTH) * kSlot);
#pragma unroll
    for (int bk = 0; bk < NBLK; ++bk)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        if (XONCE && bk < RB) load_to_lds_nt(xb, so[bk][q] + boff, dst + (uint32_t)(bk * kBlockBytes + q * 1024));
        else load_to_lds(bk < RB ? xb : ab, so[bk][q] + boff, dst + (uint32_t)(bk * kBlockBytes + q * 1024));
  };
  int issued = 0;
  for (; issued < my_n && issued < DEPTH; ++issued) issue(issued);
  for (int i = 0; i < my_n; ++i) {
    wait_vm<IPB>((issued - i - 1) * IPB);  // batch i has landed
    // the whole batch moves to registers, so that its slot can be refilled
    // before the multiplications
    const char* slot = ring + (i % DEPTH) * kSlot;
    u32x4 op[2][NBLK];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int bk = 0; bk < NBLK; ++bk) op[j][bk] = *reinterpret_cast<const u32x4*>(slot + bk * kBlockBytes + rd[j]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (issued < my_n) {
      issue(issued);
      ++issued;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[rb][nb] = M::mma(op[j][rb], op[j][RB + nb], acc[rb][nb]);
  }

  // the batch that reaches past the end of D or of the part (at most one):
  // masked loads straight into registers
  if (n_full * 2 < s1 - s0 && n_full % kWaves == wave) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int step = s0 + 2 * n_full + j;
      const int d = step * kStep + kg * kVec;
      const bool ok = step < s1 && d < p.D;
      u32x4 op[NBLK];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int t = s_tok[rb * 16 + m];
        const char* row = xb + (int64_t)(t >= 0 ? t : t0) * p.ldx * (int64_t)sizeof(Elem);
        op[rb] = ld16_or0(row + (ok ? (int64_t)d * (int64_t)sizeof(Elem) : 0), ok);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int k = nb * 16 + m;
        const char* row = ab + (int64_t)(k < r_loc ? k : r_loc - 1) * p.D * (int64_t)sizeof(Elem);
        op[RB + nb] = ld16_or0(row + (ok ? (int64_t)d * (int64_t)sizeof(Elem) : 0), ok);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[rb][nb] = M::mma(op[rb], op[RB + nb], acc[rb][nb]);
    }
  }

  // Cross-wave sum: each wave leaves its blocks in its own ring (16 bytes per
  // lane, conflict-free); block b is then summed, scaled and stored by wave
  // b % 4, and the rank columns past the computed blocks are cleared.
  f32x4* red = reinterpret_cast<f32x4*>(ring);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) red[(rb * NB + nb) * 64 + lane] = acc[rb][nb];
  __syncthreads();
  float* vb = p.v + (int64_t)slice * p.v_slice_stride;
  const float sc = p.scale ? p.scale[s] : 1.0f;
#pragma unroll
  for (int b = 0; b < RB * NB; ++b) {
    if (b % kWaves != wave) continue;
    const int rb = b / NB, nb = b % NB;
    f32x4 a = reinterpret_cast<const f32x4*>(s_lds)[b * 64 + lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const f32x4 o = reinterpret_cast<const f32x4*>(s_lds + w * kRingBytes)[b * 64 + lane];
      a[0] += o[0];
      a[1] += o[1];
      a[2] += o[2];
      a[3] += o[3];
    }
    // lane (m, kg) holds D[token rb*16 + 4 kg + i][rank c_lo + nb*16 + m]
    const int k = c_lo + nb * 16 + m;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = s_tok[rb * 16 + 4 * kg + i];
      if (partial) {
        if (t >= 0 && k < r) atomicAdd(vb + (int64_t)t * p.r_max + k, a[i] * sc);
      } else if (t >= 0 && k < c_hi) {
        vb[(int64_t)t * p.r_max + k] = k < r ? a[i] * sc : 0.f;
      }
    }
  }
  if (!partial) clear_columns(vb, p.r_max, s_tok, cnt, min(c_lo + NB * 16, c_hi), c_hi, 0, kThreads);
}

// Token / rank pieces and K parts of every item of a list.
struct Split {
  int ts, rs, kp;  // token pieces, rank pieces, K parts
};

template <typename Elem, int RB, bool XONCE>
__device__ inline void contract_rb(const ShrinkParams& p, int nb, int cnt, int s, int r, int slice, int s0, int s1,
                                   bool partial, char* s_lds, const int* s_tok, int c_lo, int c_hi) {
  switch (nb) {
    case 1: contract_unit<Elem, RB, 1, XONCE>(p, cnt, s, r, slice, s0, s1, partial, s_lds, s_tok, c_lo, c_hi); break;
    case 2: contract_unit<Elem, RB, 2, XONCE>(p, cnt, s, r, slice, s0, s1, partial, s_lds, s_tok, c_lo, c_hi); break;
    case 3: contract_unit<Elem, RB, 3, XONCE>(p, cnt, s, r, slice, s0, s1, partial, s_lds, s_tok, c_lo, c_hi); break;
    default: contract_unit<Elem, RB, 4, XONCE>(p, cnt, s, r, slice, s0, s1, partial, s_lds, s_tok, c_lo, c_hi); break;
  }
}

template <typename Elem, bool XONCE>
__device__ inline void contract_any(const ShrinkParams& p, int rbs, int nb, int cnt, int s, int r, int slice, int s0,
                                    int s1, bool partial, char* s_lds, const int* s_tok, int c_lo, int c_hi) {
  if (rbs == 1) contract_rb<Elem, 1, XONCE>(p, nb, cnt, s, r, slice, s0, s1, partial, s_lds, s_tok, c_lo, c_hi);
  else if (rbs == 2) contract_rb<Elem, 2, XONCE>(p, nb, cnt, s, r, slice, s0, s1, partial, s_lds, s_tok, c_lo, c_hi);
  else contract_rb<Elem, 4, XONCE>(p, nb, cnt, s, r, slice, s0, s1, partial, s_lds, s_tok, c_lo, c_hi);
}

// use_tiles / use_groups: which lists of the record to work on.
// resident: the workgroups the chip holds at once (the grid).  From the
// record's actual item counts, items are cut into pieces while all units
// still fit one round of the grid: each step halves the pieces of the list
// whose units read the most rows (tokens + ranks), along the longer of the
// two (tokens only for tiles; down to 16 tokens and 16 ranks).  Pieces write
// disjoint v rows and columns, so they need no atomics; a token piece re-reads
// the slot's A rows and a rank piece the item's x rows, from L2.  Splitting
// stops short of a second round: every unit pays a fixed set-up and drain.
// cleared: v was cleared beforehand (tiny batches).  Then lists still short
// of about three quarters of the grid are also cut into K parts (units of
// their own, each with at least two K steps per wave) whose partial sums are
// added with atomics; otherwise zero units clear the rows of tokens without
// an adapter.
template <typename Elem>
__global__ __launch_bounds__(kThreads, 1) void shrink_kernel(ShrinkParams p, int use_tiles, int use_groups,
                                                            int resident, int cleared) {
  __shared__ __attribute__((aligned(1024))) char s_lds[kWaves * kRingBytes];
  __shared__ int s_tok[kTile];

  const int32_t* rec = p.rec;
  const bool rec_ok = rec[kBuiltT] == p.T && rec[kBuiltS] == p.S;
  int na = rec_ok ? rec[kNumActive] : 0;
  na = na < 0 ? 0 : (na > p.T ? p.T : na);
  const int64_t items_t = use_tiles ? record_items(rec, p.T, p.S, true) : 0;
  const int64_t items_g = use_groups ? record_items(rec, p.T, p.S, false) : 0;
  const int step_elems = 4 * Traits<Elem>::kVec;
  const int n_steps = (p.D + step_elems - 1) / step_elems;
  const int64_t ns = p.n_slices;
  Split sp_t{1, 1, 1}, sp_g{1, 1, 1};
  {
    int tok_t = kTile, rk_t = p.r_max, rk_g = p.r_max;  // tokens and ranks per piece
    int64_t u_t = items_t * ns, u_g = items_g * ns;
    for (;;) {
      // candidate cuts: tiles (tokens or ranks), groups (ranks)
      const bool t_tok = tok_t > 16 && (tok_t >= rk_t || rk_t % 32 != 0);
      const bool t_ok = u_t > 0 && (t_tok || rk_t % 32 == 0) && u_t * 2 + u_g <= resident;
      const bool g_ok = u_g > 0 && rk_g % 32 == 0 && u_t + u_g * 2 <= resident;
      if (t_ok && (!g_ok || tok_t + rk_t >= kGroup + rk_g)) {
        if (t_tok) {
          sp_t.ts *= 2;
          tok_t /= 2;
        } else {
          sp_t.rs *= 2;
          rk_t /= 2;
        }
        u_t *= 2;
      } else if (g_ok) {
        sp_g.rs *= 2;
        rk_g /= 2;
        u_g *= 2;
      } else {
        break;
      }
    }
    if (cleared) {
      const int64_t target = (int64_t)resident * 3 / 4, most = max(1, n_steps / (2 * kWaves));
      if (u_t > 0) sp_t.kp = (int)min(most, max((int64_t)1, ceil_div(target, u_t)));
      if (u_g > 0) sp_g.kp = (int)min(most, max((int64_t)1, ceil_div(target, u_g)));
    }
  }
  const int64_t n_t = items_t * sp_t.kp * sp_t.ts * sp_t.rs;
  const int64_t n_g = items_g * sp_g.kp * sp_g.ts * sp_g.rs;
  const int64_t n_z = cleared ? 0 : (p.T - na + kZeroRows - 1) / kZeroRows;
  const int32_t* perm = rec + seg_layout(p.T, p.S).perm;

  // Each of the three lists (tile units, group units, zero units; each unit
  // once per slice) is cut into 8 contiguous shares, one per XCD; the
  // workgroups of an XCD walk the concatenation of its three shares.  Within
  // an item the order is slice fastest, then rank piece (these units share
  // the item's x rows in one L2), then token piece, then K part.
  const int64_t xcd = blockIdx.x % kXcds, lb = blockIdx.x / kXcds, wgs = gridDim.x / kXcds;
  auto share = [&](int64_t n, int64_t& st, int64_t& ln) {
    const int64_t per = n / kXcds, rem = n % kXcds;
    st = xcd * per + (xcd < rem ? xcd : rem);
    ln = per + (xcd < rem ? 1 : 0);
  };
  int64_t st_t, ln_t, st_g, ln_g, st_z, ln_z;
  share(n_t * ns, st_t, ln_t);
  share(n_g * ns, st_g, ln_g);
  share(n_z * ns, st_z, ln_z);
  const int tid = threadIdx.x;

  for (int64_t w = lb; w < ln_t + ln_g + ln_z; w += wgs) {
    const int list = w < ln_t ? 0 : (w < ln_t + ln_g ? 1 : 2);
    int64_t unit = list == 0 ? st_t + w : (list == 1 ? st_g + (w - ln_t) : st_z + (w - ln_t - ln_g));
    const int slice = (int)(unit % ns);
    unit /= ns;
    float* vb = p.v + (int64_t)slice * p.v_slice_stride;

    if (list == 2) {
      // zero unit: tail entries na + 64 unit .. of perm
      const int w4 = p.r_max / 4;
      const int64_t pos0 = na + unit * kZeroRows;
      for (int e = tid; e < kZeroRows * w4; e += kThreads) {
        const int row = e / w4, c = e - row * w4;
        const int64_t pos = pos0 + row;
        if (pos < p.T) {
          const int t = rec_ok ? perm[pos] : (int)pos;
          if (t >= 0 && t < p.T)
            *reinterpret_cast<f32x4*>(vb + (int64_t)t * p.r_max + 4 * c) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      continue;  // no shared memory used: no barrier needed
    }

    const bool tiles = list == 0;
    const Split sp = tiles ? sp_t : sp_g;
    const int rp = (int)(unit % sp.rs);
    unit /= sp.rs;
    const int tp = (int)(unit % sp.ts);
    unit /= sp.ts;
    const int part = (int)(unit % sp.kp);
    const int64_t item = unit / sp.kp;

    // the item's header and its tokens arrive in one memory round trip
    const int cap = tiles ? kTile : kGroup;
    const int32_t* it = item_ptr(rec, p.T, p.S, tiles, item);
    const int tv = tid < cap ? it[4 + tid] : -1;
    Item hd;
    const bool ok = read_item(rec, p.T, p.S, tiles, item, hd);
    if (!ok) continue;  // uniform
    if (tid < kTile) s_tok[tid] = (tid < hd.cnt && tv >= 0 && tv < p.T) ? tv : -1;
    __syncthreads();
    // this unit's tokens and v columns
    const int per_tok = cap / sp.ts;
    const int tok0 = tp * per_tok;
    const int cnt = min(per_tok, hd.cnt - tok0);
    if (cnt <= 0) continue;  // an empty token piece; no thread reads s_tok here
    const int per_rk = p.r_max / sp.rs;
    const int c_lo = rp * per_rk, c_hi = c_lo + per_rk;
    const int s = __builtin_amdgcn_readfirstlane(hd.slot);
    const int r = __builtin_amdgcn_readfirstlane(slot_rank(p.ranks, s, p.r_max));
    const int nb = r > c_lo ? (min(r, c_hi) - c_lo + 15) / 16 : 0;
    // this part's K steps: parts take equal runs of whole steps
    const int per_part = (n_steps + sp.kp - 1) / sp.kp;
    const int s0 = min(n_steps, part * per_part), s1 = min(n_steps, s0 + per_part);
    const bool partial = sp.kp > 1;
    const int* utok = s_tok + tok0;
    const bool x_once = ns == 1 && sp.rs == 1;
    const int rbs = (cnt + 15) / 16;
    if (nb == 0) {
      if (!partial) clear_columns(vb, p.r_max, utok, cnt, c_lo, c_hi, 0, kThreads);
    } else if (x_once) {
      contract_any<Elem, true>(p, rbs, nb, cnt, s, r, slice, s0, s1, partial, s_lds, utok, c_lo, c_hi);
    } else {
      contract_any<Elem, false>(p, rbs, nb, cnt, s, r, slice, s0, s1, partial, s_lds, utok, c_lo, c_hi);
    }
    __syncthreads();  // the next unit rewrites s_tok and the rings
  }
}

template <typename Elem>
hipError_t launch(const ShrinkParams& p, bool groups, bool tiles, hipStream_t stream) {
  const void* kernel = reinterpret_cast<const void*>(&shrink_kernel<Elem>);
  // The kernel is persistent, aiming at about three quarters of the
  // workgroups the chip holds at once.  When even a batch of nothing but full
  // tiles, with every piece cut, would give fewer units, items may also be
  // cut along K: v is cleared first.
  const int resident = persistent_grid(kernel, kThreads, 0, INT64_MAX / 4);
  const bool cleared = ceil_div(p.T, kTile) * p.n_slices * (kTile / 16) * ceil_div(p.r_max, 16) < resident * 3 / 4;
  if (cleared) {
    hipError_t e = launch_fill_zero(p.v, (int64_t)p.n_slices * p.v_slice_stride, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(shrink_kernel<Elem>, dim3(resident), dim3(kThreads), 0, stream, p, tiles ? 1 : 0,
                     groups ? 1 : 0, resident, cleared ? 1 : 0);
  return hipGetLastError();
}

__global__ void fill_zero_kernel(float* __restrict__ v, int64_t n) {
  const int64_t n4 = n >> 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    reinterpret_cast<f32x4*>(v)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t i = (n4 << 2) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) v[i] = 0.f;
}

}  // namespace

hipError_t launch_fill_zero(float* v, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = ceil_div(ceil_div(n, 4), 256);
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, v, n);
  return hipGetLastError();
}

hipError_t launch_shrink(lora_dtype dt, const ShrinkParams& p, bool groups, bool tiles, hipStream_t stream) {
  switch (dt) {
    case LORA_F32: return launch<float>(p, groups, tiles, stream);
    case LORA_F16: return launch<half_t>(p, groups, tiles, stream);
    case LORA_BF16: return launch<bf16_t>(p, groups, tiles, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace lora
