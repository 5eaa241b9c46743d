// One shrink work unit on the matrix cores, shared by the shrink kernel and
// the fused shrink-expand kernel: for up to 64 tokens of one slot and up to 64
// of its ranks it computes D[token][rank] = X A_s^T over a range of K steps.
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
#pragma once

#include "common.h"

namespace lora {

namespace {

constexpr int kUnitThreads = 256;
constexpr int kWaves = kUnitThreads / 64;

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

constexpr int kBlockBytes = 2048;  // one batch of one 16-row block: 16 rows x 128 bytes

// One global-to-LDS load: every lane fetches the 16 bytes at base + voff (base
// wave-uniform) and they land at LDS byte lds + 16 * lane.  Issued by hand: the
// compiler, which cannot tell the ring's slots apart, would otherwise wait for
// every load in flight before each LDS read.  M0 is saved and restored around
// it.
// The base and the LDS address are wave-uniform at every call; they go through
// readfirstlane so that the compiler can prove it (free when it already can).
__device__ inline const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}
__device__ inline void load_to_lds(const char* base, uint32_t voff, uint32_t lds) {
  base = uniform_ptr(base);
  lds = __builtin_amdgcn_readfirstlane(lds);
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
  base = uniform_ptr(base);
  lds = __builtin_amdgcn_readfirstlane(lds);
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
// XSL: the rank blocks run across slices -- block nb is block g0 + nb of the
// slices' 16-rank blocks taken together (slice (g0 + nb) / (r_max / 16)),
// `slice`, c_lo and c_hi are unused, r >= 1, and the unit stores its blocks'
// columns whole (zeros past the rank); not with `partial` or `part`.
template <typename Elem, int RB, int NB, bool XONCE, int RING, bool XSL = false>
__device__ __forceinline__ void contract_unit(const ShrinkParams& p, int cnt, int s, int r, int slice, int s0,
                                              int s1, bool partial, float* part, char* s_lds, const int* s_tok,
                                              int c_lo, int c_hi, int g0 = 0) {
  using M = StepMma<Elem>;
  constexpr int kVec = Traits<Elem>::kVec;
  constexpr int kStep = 4 * kVec;  // elements per K step (64 bytes)
  constexpr int NBLK = RB + NB;
  constexpr int kSlot = NBLK * kBlockBytes;              // one batch of every block
  constexpr int DEPTH = RING / kSlot < 8 ? RING / kSlot : 8;
  constexpr int IPB = 2 * NBLK;                          // loads per batch
  static_assert((DEPTH - 1) * IPB <= 63, "the ring's loads must fit the wait counter");
  const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, kg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  char* ring = s_lds + wave * RING;

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
  const char* ab = reinterpret_cast<const char*>(p.A[XSL ? 0 : slice]) +
                   ((int64_t)s * p.r_max + (XSL ? 0 : c_lo)) * p.D * (int64_t)sizeof(Elem);
  const int r_loc = XSL ? r : min(r, c_hi) - c_lo;  // rank rows of this unit, >= 1
  // XSL: each rank block's slice, A base and first rank
  const int bps = p.r_max / 16;
  const char* abk[NB];
  int bsl[NB], bcol[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    bsl[nb] = XSL ? (g0 + nb) / bps : slice;
    bcol[nb] = XSL ? ((g0 + nb) % bps) * 16 : nb * 16;  // XSL: the slot's rank; else relative to c_lo
    abk[nb] = XSL ? reinterpret_cast<const char*>(p.A[bsl[nb]]) + (int64_t)s * p.r_max * p.D * (int64_t)sizeof(Elem)
                  : ab;
  }
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
      const int k = bcol[nb] + row;
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
        else load_to_lds(bk < RB ? xb : abk[bk < RB ? 0 : bk - RB], so[bk][q] + boff,
                         dst + (uint32_t)(bk * kBlockBytes + q * 1024));
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
        const int k = bcol[nb] + m;
        const char* row = abk[nb] + (int64_t)(k < r_loc ? k : r_loc - 1) * p.D * (int64_t)sizeof(Elem);
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
      const f32x4 o = reinterpret_cast<const f32x4*>(s_lds + w * RING)[b * 64 + lane];
      a[0] += o[0];
      a[1] += o[1];
      a[2] += o[2];
      a[3] += o[3];
    }
    // lane (m, kg) holds D[token rb*16 + 4 kg + i][rank c_lo + nb*16 + m]
    // (XSL: rank bcol[nb] + m of slice bsl[nb])
    const int k = (XSL ? 0 : c_lo) + bcol[nb] + m;
    if constexpr (XSL) {
      float* vs = p.v + (int64_t)bsl[nb] * p.v_slice_stride;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = s_tok[rb * 16 + 4 * kg + i];
        if (t >= 0) vs[(int64_t)t * p.r_max + k] = k < r ? a[i] * sc : 0.f;
      }
      continue;
    }
    if (part) {
      // raw sums (unscaled) into the unit's slab, row = token position, as
      // device-coherent stores (another workgroup, on any XCD, reads them)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (k < r)
          __hip_atomic_store(part + (rb * 16 + 4 * kg + i) * p.r_max + k, a[i], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      continue;
    }
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
  if (!XSL && !partial && !part)
    clear_columns(vb, p.r_max, s_tok, cnt, min(c_lo + NB * 16, c_hi), c_hi, 0, kUnitThreads);
}

template <typename Elem, int RB, bool XONCE, int RING>
__device__ __forceinline__ void contract_rb(const ShrinkParams& p, int nb, int cnt, int s, int r, int slice, int s0, int s1,
                                   bool partial, float* part, char* s_lds, const int* s_tok, int c_lo, int c_hi) {
  switch (nb) {
    case 1: contract_unit<Elem, RB, 1, XONCE, RING>(p, cnt, s, r, slice, s0, s1, partial, part, s_lds, s_tok, c_lo, c_hi); break;
    case 2: contract_unit<Elem, RB, 2, XONCE, RING>(p, cnt, s, r, slice, s0, s1, partial, part, s_lds, s_tok, c_lo, c_hi); break;
    case 3: contract_unit<Elem, RB, 3, XONCE, RING>(p, cnt, s, r, slice, s0, s1, partial, part, s_lds, s_tok, c_lo, c_hi); break;
    default: contract_unit<Elem, RB, 4, XONCE, RING>(p, cnt, s, r, slice, s0, s1, partial, part, s_lds, s_tok, c_lo, c_hi); break;
  }
}

// An XSL unit (rank blocks across slices, see contract_unit): rbs token blocks
// by nb rank blocks from block g0.
template <typename Elem, int RB, int RING>
__device__ __forceinline__ void contract_xsl_rb(const ShrinkParams& p, int nb, int cnt, int s, int r, int s0, int s1,
                                                char* s_lds, const int* s_tok, int g0) {
  switch (nb) {
    case 1: contract_unit<Elem, RB, 1, false, RING, true>(p, cnt, s, r, 0, s0, s1, false, nullptr, s_lds, s_tok, 0, 0, g0); break;
    case 2: contract_unit<Elem, RB, 2, false, RING, true>(p, cnt, s, r, 0, s0, s1, false, nullptr, s_lds, s_tok, 0, 0, g0); break;
    case 3: contract_unit<Elem, RB, 3, false, RING, true>(p, cnt, s, r, 0, s0, s1, false, nullptr, s_lds, s_tok, 0, 0, g0); break;
    default: contract_unit<Elem, RB, 4, false, RING, true>(p, cnt, s, r, 0, s0, s1, false, nullptr, s_lds, s_tok, 0, 0, g0); break;
  }
}
template <typename Elem, int RING>
__device__ __forceinline__ void contract_xsl(const ShrinkParams& p, int rbs, int nb, int cnt, int s, int r, int s0,
                                             int s1, char* s_lds, const int* s_tok, int g0) {
  if (rbs == 1) contract_xsl_rb<Elem, 1, RING>(p, nb, cnt, s, r, s0, s1, s_lds, s_tok, g0);
  else if (rbs == 2) contract_xsl_rb<Elem, 2, RING>(p, nb, cnt, s, r, s0, s1, s_lds, s_tok, g0);
  else contract_xsl_rb<Elem, 4, RING>(p, nb, cnt, s, r, s0, s1, s_lds, s_tok, g0);
}

template <typename Elem, bool XONCE, int RING>
__device__ __forceinline__ void contract_any(const ShrinkParams& p, int rbs, int nb, int cnt, int s, int r, int slice, int s0,
                                    int s1, bool partial, float* part, char* s_lds, const int* s_tok, int c_lo, int c_hi) {
  if (rbs == 1) contract_rb<Elem, 1, XONCE, RING>(p, nb, cnt, s, r, slice, s0, s1, partial, part, s_lds, s_tok, c_lo, c_hi);
  else if (rbs == 2) contract_rb<Elem, 2, XONCE, RING>(p, nb, cnt, s, r, slice, s0, s1, partial, part, s_lds, s_tok, c_lo, c_hi);
  else contract_rb<Elem, 4, XONCE, RING>(p, nb, cnt, s, r, slice, s0, s1, partial, part, s_lds, s_tok, c_lo, c_hi);
}


}  // namespace

}  // namespace lora
