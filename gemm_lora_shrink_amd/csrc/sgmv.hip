// Expand on the matrix cores, for the gather groups and the segmented tiles of
// 16-bit data: per item the expand is a dense [cnt x r] by [r x out]
// contraction, run on v_mfma_f32_16x16x32 (bf16 or fp16 inputs, fp32
// accumulation).  The earlier segmented kernel lost accuracy by keeping the
// intermediate in half precision ("Add multi-LoRA support", Limitations); here
// the intermediate stays fp32 end to end.
//
// The MFMA lane layout and the hi + lo form of the fp32 intermediate are
// described in expand_unit.h, which holds the gather-group path.
#include "common.h"
#include "expand_unit.h"

namespace lora {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Expand
// ---------------------------------------------------------------------------
// Work unit: (item of up to 64 tokens, slice, a run of 256-column tiles).  Per
// unit the workgroup reads the item's token list once and converts the item's
// fp32 v rows once into the 16-bit hi/lo operands, kept in LDS for the four
// waves.  Then, per column tile, wave w handles columns 64 w .. 64 w + 63:
// it issues its B-row loads and then its y loads (lane-contiguous: eight lanes
// cover one token's 64 columns, 128 bytes) -- loads complete in order, so the
// products, which need only B, start while y is still on its way from HBM
// (2 us of the fused-QKV prefill's expand) -- runs the MFMAs per 16-token
// sub-block, transposes the fp32 result through a wave-private LDS block and
// updates y with 16-byte accesses.  No workgroup barrier is needed inside a
// unit.
constexpr int kSubs = kTile / 16;                              // 16-token sub-blocks per item
constexpr int kVRow = LORA_MAX_RANK + 8;                       // padded 16-bit LDS row of v
constexpr int kTileRun = 2;              // column tiles per unit of a segmented tile (see the kernel)
constexpr int kGroupRun = 4 * kTileRun;  // ... of a gather group
constexpr int kBStage = kExpandColsPerWave * 8;  // 16-byte pieces of one wave's B rows of a tile (64 rows x 128 B)

// One tile unit: the column tiles [ct_begin, ct_end) of an item of up to 64
// tokens (NSUB 16-token sub-blocks; sub-blocks past the item's tokens hold no
// token and are skipped by their -1 entries).  tok_v is the token of this
// thread's v row (row tid / 4, -1 past the item's count).  The v rows, the
// first column tile's y and its B rows are all requested before any of them
// is waited for; the fp32 v rows are then converted into the 16-bit hi/lo
// operands in LDS.  A unit has at most RUN column tiles (a compile-time bound,
// so that no load is issued for a tile past the last one a unit can have).
template <typename Elem, int NSUB, int RUN>
__device__ inline void expand_tile(const ExpandParams& p, int tok_v, int n_sub, int* s_tok, float* s_unscale,
                                   Elem (*s_vhi)[kVRow], Elem (*s_vlo)[kVRow], float (*s_tr)[16][kTrRow],
                                   u32x4* s_bw, int slice, int s, int r, int out, int ct_begin, int ct_end) {
  using M = Mfma<Elem>;
  using V = typename M::vec;
  using Tr = Traits<Elem>;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, kg = lane >> 4;
  const int yr = lane >> 3, yc = (lane & 7) * 8;
  const Elem* yzero = reinterpret_cast<const Elem*>(g_zero16);
  const int nks = r > 32 ? 2 : 1;  // 32-wide rank steps
  const bool ragged_rank = (r & 7) != 0;
  const Elem* Bs = reinterpret_cast<const Elem*>(p.B[slice]) + (int64_t)s * out * p.r_max;
  const int ldb = b_row_stride(p, r);
  Elem* ybase = reinterpret_cast<Elem*>(p.y) + p.out_off[slice] + yc;

  // this thread's v row: token tid / 4, ranks 16 (tid % 4) .. +15
  const int tt = tid >> 2, kq = (tid & 3) * 16;
  if ((tid & 3) == 0) s_tok[tt] = tok_v;
  f32x4 vraw[4];
  {
    const float* src = p.v + (int64_t)slice * p.v_slice_stride + (int64_t)(tok_v >= 0 ? tok_v : 0) * p.r_max + kq;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool ok = tok_v >= 0 && kq + 4 * q < r;
      vraw[q] = ldf4_or0(src + (ok ? 4 * q : 0), ok);
    }
  }
  lds_barrier();  // s_tok is visible; the v loads stay in flight

  // y of every sub-block of column tile `ct`, lane-contiguous (zeros past the end)
  auto load_y = [&](int ct, u32x4 (&dst)[NSUB][2]) {
    const int jw = ct * kExpandColsPerWG + wave * kExpandColsPerWave;
    const bool ycol_ok = ct < ct_end && jw + yc < out;  // out is a multiple of 8
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = sb < n_sub ? s_tok[sb * 16 + h * 8 + yr] : -1;
        const bool ok = ycol_ok && t >= 0;
        dst[sb][h] = ld16_or0_nt(ok ? ybase + jw + (int64_t)t * p.ldy : yzero, ok);
      }
  };
  // A operand: this wave's 64 B rows of column tile `ct`, loaded in whole
  // lines -- lane l takes the 16-byte piece l % 8 of row 8 i + l / 8, i = 0..7
  // (the MFMA layout would have every 16 lanes touch 16 rows, which a compute
  // unit streams far more slowly) -- and moved into MFMA layout through the
  // wave's LDS block before the tile's products.  Pieces past the slot's rank
  // and rows past `out` are not read (zeros past ct_end: the last prefetch
  // issues only loads of the zero constant).
  const int bl_row = lane >> 3, bl_piece = lane & 7;
  auto load_b = [&](int ct, u32x4 (&bl)[8]) {
    const int jw = ct * kExpandColsPerWG + wave * kExpandColsPerWave;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = jw + 8 * i + bl_row;
      const int k0 = bl_piece * 8;
      const bool ok = ct < ct_end && row < out && k0 < r;
      bl[i] = ld16_or0(Bs + (ok ? (int64_t)row * ldb + k0 : 0), ok);
    }
  };
  u32x4 yold[NSUB][2];
  u32x4 bop[8];
  load_b(ct_begin, bop);
  load_y(ct_begin, yold);

  {
    float vv[16];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) vv[4 * q + e] = (kq + 4 * q + e < r) ? vraw[q][e] : 0.f;
    float unscale = 1.0f;
    if constexpr (Tr::kDtype == LORA_F16) {
      // scale the token's row by a power of two so that |v| < 2
      float mx = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fabsf(vv[e]));
      mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
      if (mx > 0.f) {
        int ex;
        frexpf(mx, &ex);  // mx = f * 2^ex, f in [0.5, 1)
        const float sc = ldexpf(1.0f, 1 - ex);
        unscale = ldexpf(1.0f, ex - 1);
#pragma unroll
        for (int e = 0; e < 16; ++e) vv[e] *= sc;
      }
    }
    if ((tid & 3) == 0) s_unscale[tt] = unscale;
    V hi0, hi1, lo0, lo1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const Elem h0 = static_cast<Elem>(vv[e]), h1 = static_cast<Elem>(vv[8 + e]);
      hi0[e] = h0;
      hi1[e] = h1;
      lo0[e] = static_cast<Elem>(vv[e] - static_cast<float>(h0));
      lo1[e] = static_cast<Elem>(vv[8 + e] - static_cast<float>(h1));
    }
    *reinterpret_cast<V*>(&s_vhi[tt][kq]) = hi0;
    *reinterpret_cast<V*>(&s_vhi[tt][kq + 8]) = hi1;
    *reinterpret_cast<V*>(&s_vlo[tt][kq]) = lo0;
    *reinterpret_cast<V*>(&s_vlo[tt][kq + 8]) = lo1;
  }
  lds_barrier();  // the v operands are visible; y and B loads stay in flight

  // one column tile with its y and B rows (loaded one tile ahead)
  auto compute_tile = [&](int ct, const u32x4 (&ycur)[NSUB][2], const u32x4 (&bcur)[8]) {
    const int jw = ct * kExpandColsPerWG + wave * kExpandColsPerWave;
    const bool ycol_ok = jw + yc < out;  // out is a multiple of 8
    // the B lines into MFMA layout: row q's piece c sits at piece c ^ (q % 8)
    // of the row's 128 bytes in the wave's block (conflict-free both ways)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = 8 * i + bl_row;
      s_bw[q * 8 + (bl_piece ^ (q & 7))] = bcur[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // a rank that is not a multiple of 8 ends inside one 16-byte piece: zero
    // the columns past it (loaded pieces past the rank are zeros already)
    V bv[4][2];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int q = cb * 16 + n, c = ks * 4 + kg;
        const u32x4 b = s_bw[q * 8 + (c ^ (q & 7))];
        bv[cb][ks] = as_vec<V>(ragged_rank ? mask_tail16(b, ks * 32 + kg * 8, r) : b);
      }
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) {
      if (sb >= n_sub) break;
      // B operand: v[tok 16 sb + n][32 ks + 8 kg .. +7], hi and lo
      V vhi[2], vlo[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        vhi[ks] = *reinterpret_cast<const V*>(&s_vhi[sb * 16 + n][ks * 32 + kg * 8]);
        vlo[ks] = *reinterpret_cast<const V*>(&s_vlo[sb * 16 + n][ks * 32 + kg * 8]);
      }
      const float unscale = s_unscale[sb * 16 + n];
      // D[column 4 kg + i][token n] of block cb -> s_tr[wave][n][16 cb + 4 kg + i]
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        acc = M::mma(bv[cb][0], vhi[0], acc);
        acc = M::mma(bv[cb][0], vlo[0], acc);
        if (nks > 1) {
          acc = M::mma(bv[cb][1], vhi[1], acc);
          acc = M::mma(bv[cb][1], vlo[1], acc);
        }
        if constexpr (Tr::kDtype == LORA_F16) acc *= unscale;  // bf16 rows are not scaled
        *reinterpret_cast<f32x4*>(&s_tr[wave][n][cb * 16 + kg * 4]) = acc;
      }
      // the block is written and read by this wave only
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = s_tok[sb * 16 + h * 8 + yr];
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(&s_tr[wave][h * 8 + yr][yc]);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(&s_tr[wave][h * 8 + yr][yc + 4]);
        if (ycol_ok && t >= 0) {
          const float add[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          u32x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t wd = ycur[sb][h][q];
            const float y0 = Tr::elem_to_float(wd & 0xffffu) + add[2 * q];
            const float y1 = Tr::elem_to_float(wd >> 16) + add[2 * q + 1];
            if constexpr (Tr::kDtype == LORA_BF16) o[q] = pack2_bf16(y0, y1);
            else o[q] = pack2_f16(y0, y1);
          }
          // y is streamed once: non-temporal, so that it does not sit dirty in
          // L2 for the kernels that follow
          __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(ybase + jw + (int64_t)t * p.ldy));
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  };

  // two tiles per iteration, so that the register buffers alternate without
  // copies; the next tile's y and B rows are in flight during each tile
  u32x4 ynext[NSUB][2], bnext[8];
#pragma unroll
  for (int i = 0; i < RUN; i += 2) {
    const int ct = ct_begin + i;
    if (ct >= ct_end) break;
    if (i + 1 < RUN) {
      load_b(ct + 1, bnext);
      load_y(ct + 1, ynext);
    }
    compute_tile(ct, yold, bop);
    if (i + 1 >= RUN || ct + 1 >= ct_end) break;
    if (i + 2 < RUN) {
      load_b(ct + 2, bop);
      load_y(ct + 2, yold);
    }
    compute_tile(ct + 1, ynext, bnext);
  }
}

// The words of an item a unit needs: its header and the token words of this
// thread (the token of its v row -- tile path: row tid / 4 -- and those of its
// MFMA column and y rows -- gather path).  The kernel requests them one unit
// ahead, so that they are in registers when the unit starts.
struct UnitWords {
  u32x4 head;
  int tw_v, tw_n, tw_y0, tw_y1;
};
__device__ inline UnitWords load_unit_words(const ExpandParams& p, bool tiles, int64_t li) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int32_t* ip = item_ptr(p.rec, p.T, p.S, tiles, li);
  UnitWords w;
  w.head = *reinterpret_cast<const u32x4*>(ip);  // items are 16-byte aligned
  w.tw_v = ip[4 + (tiles ? (tid >> 2) : ((tid >> 2) & (kGroup - 1)))];
  w.tw_n = ip[4 + (lane & 15)];
  w.tw_y0 = ip[4 + (lane >> 3)];
  w.tw_y1 = ip[4 + (lane >> 3) + 8];
  return w;
}

// One unit: the column tiles [ct_begin, ct_end) of item `li` of a list
// (tiles or gather groups) for one slice, from its words w; s_rank holds
// every slot's rank.
template <typename Elem>
__device__ inline void expand_unit(const ExpandParams& p, int slice, bool tiles, const UnitWords& w, int ct_begin,
                                   int ct_end, const int* s_rank, int* s_tok, float* s_unscale,
                                   Elem (*s_vhi)[kVRow], Elem (*s_vlo)[kVRow], float (*s_tr)[16][kTrRow],
                                   u32x4 (*s_b)[kBStage]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int n = lane & 15, yr = lane >> 3;
  const int out = (int)p.out_size[slice];
  const int tw_v = w.tw_v, tw_n = w.tw_n, tw_y0 = w.tw_y0, tw_y1 = w.tw_y1;
  const Item it{(int)w.head[0], (int)w.head[1], (int)w.head[2], (int)w.head[3]};
  const int cap = tiles ? kTile : kGroup;
  if (!(it.slot >= 0 && it.slot < p.S && it.p0 >= 0 && it.cnt > 0 && it.cnt <= cap && it.p0 + it.cnt <= p.T))
    return;
  const int s = __builtin_amdgcn_readfirstlane(it.slot);
  const int r = __builtin_amdgcn_readfirstlane(s_rank[s]);
  if (r == 0) return;
  // token k of the item, clamped into [0, T); -1 past its count
  auto tok = [&](int k, int t) { return k < it.cnt ? (t < 0 ? 0 : (t >= p.T ? p.T - 1 : t)) : -1; };
  if (it.cnt <= 16) {
    // uniform per unit; this path uses only wave-private LDS
    const int tok_n = tok(n, tw_n);
    const int kg = lane >> 4, nks = r > 32 ? 2 : 1;
    const float* vrow = p.v + (int64_t)slice * p.v_slice_stride + (int64_t)(tok_n >= 0 ? tok_n : 0) * p.r_max;
    auto vsrc = [&](f32x4 (&vraw)[2][2]) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int k0 = ks * 32 + kg * 8;
        // an fp32 row (r_max a multiple of 4) may end halfway through the piece
        const bool ok = tok_n >= 0 && ks < nks && k0 < r, ok1 = ok && k0 + 4 < r;
        vraw[ks][0] = ldf4_or0(vrow + (ok ? k0 : 0), ok);
        vraw[ks][1] = ldf4_or0(vrow + (ok1 ? k0 + 4 : 0), ok1);
      }
    };
    expand_group_direct<Elem>(p, vsrc, tok(yr, tw_y0), tok(yr + 8, tw_y1), s_tr, slice, s, r, out, ct_begin,
                              ct_end);
    return;
  }
  expand_tile<Elem, kSubs, kTileRun>(p, tok(tid >> 2, tw_v), (it.cnt + 15) >> 4, s_tok, s_unscale, s_vhi, s_vlo, s_tr,
                                     s_b[tid >> 6], slice, s, r, out, ct_begin, ct_end);
  lds_barrier();  // the next unit rewrites s_tok and the v operands
}

// The work is cut into units (item, slice, run of column tiles): a run of
// kTileRun 256-column tiles for a segmented tile (64 tokens), of kGroupRun for
// a gather group (16 tokens), so that every unit updates about the same bytes
// of y.  Units are ordered by slice, item (gather groups first), run, and
// taken window by window: round j of the kernel covers units [j G, (j + 1) G),
// unit j G + q going to the workgroup with position q.  All workgroups thus
// update y inside one compact window of rows at any time, which the HBM
// serves faster than the same read-modify-write traffic spread over the whole
// of y (a workgroup per contiguous share: 54 -> 50.5 us for the fused-QKV
// prefill at 8192 tokens).  Positions are XCD-major (the workgroups of XCD x,
// blockIdx % 8 == x, hold positions x G / 8 .. (x + 1) G / 8 - 1), so the
// consecutive units of one item -- which read the same v rows, and items of
// one slot the same B rows -- run on one XCD and share its L2.  Runs of two
// tiles keep the per-unit set-up (tokens, v operands) to one per 128 KB of y
// traffic; runs of one tile pay it twice as often, runs of four leave the last
// round short.  With fewer units than workgroups, G is the units rounded up
// to a multiple of kXcds.

template <typename Elem>
__global__ __launch_bounds__(kThreads, 2) void mfma_expand_kernel(ExpandParams p, int use_groups, int use_tiles) {
  warm_args(p);
  __shared__ int s_tok[kTile];
  __shared__ float s_unscale[kTile];
  __shared__ int s_rank[LORA_MAX_SLOTS];
  __shared__ __attribute__((aligned(16))) Elem s_vhi[kTile][kVRow];
  __shared__ __attribute__((aligned(16))) Elem s_vlo[kTile][kVRow];
  __shared__ __attribute__((aligned(16))) float s_tr[4][16][kTrRow];
  __shared__ u32x4 s_b[4][kBStage];  // per wave: one tile's B rows on their way to MFMA layout

  const int64_t n_g = use_groups ? record_items(p.rec, p.T, p.S, false) : 0;
  const int64_t n_t = use_tiles ? record_items(p.rec, p.T, p.S, true) : 0;
  auto n_cols = [&](int i) { return (int)ceil_div(p.out_size[i], kExpandColsPerWG); };
  int64_t units = 0;
  for (int i = 0; i < p.n_slices; ++i)
    units += n_g * ceil_div(n_cols(i), kGroupRun) + n_t * ceil_div(n_cols(i), kTileRun);
  // with fewer units than workgroups, the first workgroups of every XCD take
  // them (the hardware places those on distinct compute units)
  const int64_t G = min((int64_t)gridDim.x, max((int64_t)kXcds, ceil_div(units, kXcds) * kXcds));
  const int64_t lb = blockIdx.x / kXcds;
  if (lb >= G / kXcds) return;  // uniform: no unit for this workgroup
  const int64_t q = (blockIdx.x % kXcds) * (G / kXcds) + lb;
  // every slot's rank, in LDS: a unit's rank costs no memory round trip
  for (int i = threadIdx.x; i < p.S; i += kThreads) s_rank[i] = slot_rank(p.ranks, i, p.r_max);
  // unit u: its slice, list, item and column tiles
  struct Unit {
    bool ok, tiles;
    int slice, ct0, ct1;
    int64_t item;
  };
  auto decode = [&](int64_t u) {
    Unit d{false, false, 0, 0, 0, 0};
    for (int i = 0; i < p.n_slices; ++i) {
      const int gu = (int)ceil_div(n_cols(i), kGroupRun);  // units per gather group
      const int tu = (int)ceil_div(n_cols(i), kTileRun);   // units per segmented tile
      const int64_t nu = n_g * gu + n_t * tu;
      if (u < nu) {
        d.ok = true;
        d.slice = i;
        d.tiles = u >= n_g * gu;
        const int64_t rr = d.tiles ? u - n_g * gu : u;
        const int per = d.tiles ? tu : gu, run = d.tiles ? kTileRun : kGroupRun;
        d.item = rr / per;
        d.ct0 = (int)(rr % per) * run;
        d.ct1 = min(n_cols(i), d.ct0 + run);
        return d;
      }
      u -= nu;
    }
    return d;
  };
  lds_barrier();
  // this workgroup's units u = q, q + G, ..., each unit's words requested
  // while the unit before it runs
  Unit cur = decode(q);
  UnitWords cw{};
  if (cur.ok) cw = load_unit_words(p, cur.tiles, cur.item);
  for (int64_t u = q; cur.ok; u += G) {
    const Unit nxt = decode(u + G);
    UnitWords nw{};
    if (nxt.ok) nw = load_unit_words(p, nxt.tiles, nxt.item);
    expand_unit<Elem>(p, cur.slice, cur.tiles, cw, cur.ct0, cur.ct1, s_rank, s_tok, s_unscale, s_vhi, s_vlo, s_tr,
                      s_b);
    cur = nxt;
    cw = nw;
  }
}

template <typename Elem>
hipError_t expand_launch(const ExpandParams& p, bool groups, bool tiles, hipStream_t stream) {
  const SegLayout L = seg_layout(p.T, p.S);
  int64_t cols = 0;
  for (int i = 0; i < p.n_slices; ++i) cols += ceil_div(p.out_size[i], kExpandColsPerWG);
  const int64_t cap = (groups ? L.cap_groups : 0) + (tiles ? L.cap_tiles : 0);
  const int grid = persistent_grid(reinterpret_cast<const void*>(&mfma_expand_kernel<Elem>), kThreads, 0,
                                   cap * cols);
  hipLaunchKernelGGL(mfma_expand_kernel<Elem>, dim3(grid), dim3(kThreads), 0, stream, p, groups ? 1 : 0,
                     tiles ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_expand(lora_dtype dt, const ExpandParams& p, bool groups, bool tiles, hipStream_t stream) {
  switch (dt) {
    case LORA_F16: return expand_launch<half_t>(p, groups, tiles, stream);
    case LORA_BF16: return expand_launch<bf16_t>(p, groups, tiles, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lora
