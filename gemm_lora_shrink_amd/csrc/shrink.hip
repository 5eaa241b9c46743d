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
// Mostly, every v row of the batch is written exactly once with plain stores:
// the rows of active tokens with their values (0 in rank columns k >= r_s),
// the others with zeros, with no clearing pass and no atomic, so the result
// does not depend on how the units are scheduled.  The exception is a batch
// whose items are cut along K (batches too small to fill the chip, and
// mid-size batches with a contraction of at least kLongK): a clearing launch
// then precedes the shrink, and the K parts of an item add their partial sums
// into v with fp32 atomics in whatever order they finish, so the last bits of
// v can differ from run to run (always within fp32 accumulation error).
//
// The unit itself (how its four waves split the contraction and stream the
// operands through LDS) is in shrink_unit.h.
#include "common.h"
#include "shrink_unit.h"

namespace lora {

namespace {

constexpr int kThreads = kUnitThreads;
constexpr int kZeroRows = 64;  // tail entries per zero unit
constexpr int kRingBytes = 16384;  // LDS ring of one wave (also holds its partial sums)
constexpr int kLongK = 8192;       // contractions at least this long may be cut along K at mid sizes

// Token / rank pieces and K parts of every item of a list.
struct Split {
  int ts, rs, kp;  // token pieces, rank pieces, K parts
};

// use_tiles / use_groups: which lists of the record to work on.
// resident: the workgroups the chip holds at once (the grid).  From the
// record's actual item counts, items are cut into pieces while all units
// still fit one round of the grid: each step halves the pieces of the list
// whose units read the most rows (tokens + ranks), along the longer of the
// two (tokens only for tiles; down to 16 tokens and 16 ranks).  Pieces write
// disjoint v rows and columns, so they need no atomics; a token piece re-reads
// the slot's A rows and a rank piece the item's x rows, from L2.  Splitting
// stops short of a second round: every unit pays a fixed set-up and drain.
// cleared: v was cleared beforehand (tiny batches, or long contractions;
// 2 for the latter).  Then lists still short of about three quarters of the
// grid are also cut into K parts (units of their own, each with at least two
// K steps per wave) whose partial sums are added with atomics; otherwise zero
// units clear the rows of tokens without an adapter.  With long contractions
// gather groups are not cut into rank pieces: K parts fill the grid instead,
// without every rank piece re-reading the group's x rows.
// Tiles of several slices whose ranks are whole 16-rank blocks may instead be
// cut across the slices: the slices' blocks taken together (TB of them) go
// into P pieces of ceil(TB / P) blocks, P the most that fit one round of the
// grid beside the gather groups.  When P exceeds the slice count, every unit
// reads about the same bytes and the grid gets an even load, where per-slice
// units would leave two units on some compute units and one on others.  (A
// separate instance, XSL, carries this cut, so that the registers of the
// single-slice instance stay as they are.)
template <typename Elem, bool XSL>
__global__ __launch_bounds__(kThreads, 2) void shrink_kernel(ShrinkParams p, int use_tiles, int use_groups,
                                                            int resident, int cleared) {
  warm_args(p);
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
  // cut of the tiles across slices: xsl_p pieces of xsl_nb blocks (0: none)
  const int n_blk = p.r_max % 16 == 0 ? (int)ns * (p.r_max / 16) : 0;
  int xsl_p = 0, xsl_nb = 0;
  if (XSL && !cleared && ns >= 2 && n_blk > 0 && items_t > 0) {
    const int64_t fit = min((int64_t)n_blk, ((int64_t)resident - items_g * ns) / items_t);
    if (fit > ns) {
      xsl_nb = (int)ceil_div((int64_t)n_blk, fit);
      xsl_p = (int)ceil_div(n_blk, xsl_nb);
    }
  }
  {
    int tok_t = kTile, rk_t = p.r_max, rk_g = p.r_max;  // tokens and ranks per piece
    int64_t u_t = items_t * (xsl_p ? xsl_p : ns), u_g = items_g * ns;
    for (;;) {
      // candidate cuts: tiles (tokens or ranks), groups (ranks)
      const bool t_tok = tok_t > 16 && (tok_t >= rk_t || rk_t % 32 != 0);
      const bool t_ok = !xsl_p && u_t > 0 && (t_tok || rk_t % 32 == 0) && u_t * 2 + u_g <= resident;
      const bool g_ok = cleared != 2 && u_g > 0 && rk_g % 32 == 0 && u_t + u_g * 2 <= resident;
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
  share(n_t * (xsl_p ? xsl_p : ns), st_t, ln_t);
  share(n_g * ns, st_g, ln_g);
  share(n_z * ns, st_z, ln_z);
  const int tid = threadIdx.x;

  for (int64_t w = lb; w < ln_t + ln_g + ln_z; w += wgs) {
    const int list = w < ln_t ? 0 : (w < ln_t + ln_g ? 1 : 2);
    int64_t unit = list == 0 ? st_t + w : (list == 1 ? st_g + (w - ln_t) : st_z + (w - ln_t - ln_g));
    const bool xsl = xsl_p > 0 && list == 0;  // a tile unit cut across slices
    const int per = xsl ? xsl_p : (int)ns;
    const int slice = xsl ? 0 : (int)(unit % ns), xsl_piece = xsl ? (int)(unit % xsl_p) : 0;
    unit /= per;
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
    if (XSL && xsl) {
      const int g0 = xsl_piece * xsl_nb, nbk = min(xsl_nb, n_blk - g0), bps = p.r_max / 16;
      if (r > 0) {
        contract_xsl<Elem, kRingBytes>(p, (cnt + 15) / 16, nbk, cnt, s, r, s0, s1, s_lds, utok, g0);
      } else {
        for (int g = g0; g < g0 + nbk; ++g)
          clear_columns(p.v + (int64_t)(g / bps) * p.v_slice_stride, p.r_max, utok, cnt, (g % bps) * 16,
                        (g % bps) * 16 + 16, 0, kThreads);
      }
      __syncthreads();  // the next unit rewrites s_tok and the rings
      continue;
    }
    const bool x_once = ns == 1 && sp.rs == 1;
    const int rbs = (cnt + 15) / 16;
    if (nb == 0) {
      if (!partial) clear_columns(vb, p.r_max, utok, cnt, c_lo, c_hi, 0, kThreads);
    } else if (x_once) {
      contract_any<Elem, true, kRingBytes>(p, rbs, nb, cnt, s, r, slice, s0, s1, partial, nullptr, s_lds, utok, c_lo, c_hi);
    } else {
      contract_any<Elem, false, kRingBytes>(p, rbs, nb, cnt, s, r, slice, s0, s1, partial, nullptr, s_lds, utok, c_lo, c_hi);
    }
    __syncthreads();  // the next unit rewrites s_tok and the rings
  }
}

template <typename Elem>
hipError_t launch(const ShrinkParams& p, bool groups, bool tiles, hipStream_t stream) {
  const void* kernel = reinterpret_cast<const void*>(&shrink_kernel<Elem, false>);
  // The kernel is persistent: its grid is the workgroups the chip holds at
  // once (two per compute unit, each with four 16 KB LDS rings).  When even a
  // batch of nothing but full tiles, with every piece cut, would give fewer
  // units than about three quarters of the compute units, items may also be
  // cut along K: v is cleared first.  (Mid-size batches, which would fill the
  // compute units once, run faster without the atomics -- unless the
  // contraction is long, D >= kLongK: then a unit streams so many bytes that
  // one round of them is slower than K parts and their atomics.)
  const int resident = persistent_grid(kernel, kThreads, 0, INT64_MAX / 4);
  const int64_t pieces = ceil_div(p.T, kTile) * p.n_slices * (kTile / 16) * ceil_div(p.r_max, 16);
  const bool long_k = p.D >= kLongK && pieces <= resident;
  // (a contraction of at most 2 batches per wave is not worth cutting: the
  // clearing launch would cost more than the parts save -- tiny fp32 batches
  // at D = 256: shrink 7.6 -> 5.5 us)
  const int64_t steps = ceil_div(p.D, 4 * Traits<Elem>::kVec);
  const bool cleared = (pieces < resident * 3 / 8 && steps > 2 * 2 * kWaves) || long_k;
  if (cleared) {
    hipError_t e = launch_fill_zero(p.v, (int64_t)p.n_slices * p.v_slice_stride, stream);
    if (e != hipSuccess) return e;
  }
  // batches of several slices in whole 16-rank blocks, not cut along K: the
  // instance that may cut tiles across slices (same grid: same LDS and
  // occupancy)
  const bool xsl = tiles && !cleared && p.n_slices >= 2 && p.r_max % 16 == 0;
  if (xsl)
    hipLaunchKernelGGL((shrink_kernel<Elem, true>), dim3(resident), dim3(kThreads), 0, stream, p, 1, groups ? 1 : 0,
                       resident, 0);
  else
    hipLaunchKernelGGL((shrink_kernel<Elem, false>), dim3(resident), dim3(kThreads), 0, stream, p, tiles ? 1 : 0,
                       groups ? 1 : 0, resident, long_k ? 2 : (cleared ? 1 : 0));
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
