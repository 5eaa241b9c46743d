// The expand of a group of at most 16 tokens of one slot on the matrix
// cores, shared by the expand kernel and the fused shrink-expand kernel.
//
// MFMA 16x16x32 lane layout (checked on gfx950): for D = A(16x32) * B(32x16),
// lane l holds A[l%16][8*(l/16) + i], B[8*(l/16) + i][l%16] (i < 8) and
// D[4*(l/16) + i][l%16] (i < 4).
//
// The group computes y^T[j][token] += sum_k B[s][j][k] * v[token][k], the
// transposed product, so that each lane's four accumulators are four
// consecutive y columns of one token.  The fp32 intermediate enters the matrix
// core as v = hi + lo, both 16-bit (two MFMAs), which keeps about 16
// significant bits of v instead of re-rounding it to 8 or 11 (a
// half-precision intermediate loses accuracy: "Add multi-LoRA support",
// Limitations).  For fp16 each token row is first scaled by a power of two so
// that its largest value lies in [1, 2): hi and lo then stay in fp16's normal
// range whatever the magnitude of v, and the scale is undone exactly on the
// fp32 result.
#pragma once

#include "common.h"

namespace lora {

namespace {

template <typename Elem> struct Mfma;
template <> struct Mfma<bf16_t> {
  typedef bf16x8 vec;
  __device__ static inline f32x4 mma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<half_t> {
  typedef f16x8 vec;
  __device__ static inline f32x4 mma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

template <typename V> __device__ inline V as_vec(u32x4 u) { return __builtin_bit_cast(V, u); }

// Zero the 16-bit elements k0 + e (e < 8) that are >= r.  Selects only: a
// branch here would make the compiler wait for the load that produced u
// before issuing the loads that follow it.
__device__ inline u32x4 mask_tail16(u32x4 u, int k0, int r) {
  u32x4 o;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t keep = (k0 + 2 * w + 1 < r) ? 0xffffffffu : ((k0 + 2 * w < r) ? 0x0000ffffu : 0u);
    o[w] = u[w] & keep;
  }
  return o;
}

constexpr int kExpandColsPerWave = 64;                         // 4 MFMA blocks of 16
constexpr int kExpandColsPerWG = 4 * kExpandColsPerWave;       // 256
constexpr int kTrRow = kExpandColsPerWave + 4;                 // padded fp32 LDS row

// A gather group (at most 16 tokens) needs no shared staging: each wave gets
// its own v operands from vsrc, once per unit, right after requesting the
// first column tile's y and B rows, and then walks its column tiles with the
// next tile's y and B rows in flight while the current tile is multiplied --
// no workgroup barrier.
template <typename Elem, typename VSrc>
__device__ inline void expand_group_direct(const ExpandParams& p, const VSrc& vsrc, int ytok0, int ytok1,
                                           float (*s_tr)[16][kTrRow], int slice, int s, int r, int out,
                                           int ct_begin, int ct_end) {
  using M = Mfma<Elem>;
  using V = typename M::vec;
  using Tr = Traits<Elem>;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, kg = lane >> 4;
  const int yr = lane >> 3, yc = (lane & 7) * 8;
  const int nks = r > 32 ? 2 : 1;
  const bool ragged_rank = (r & 7) != 0;
  const Elem* Bs = reinterpret_cast<const Elem*>(p.B[slice]) + (int64_t)s * out * p.r_max;
  const int ldb = b_row_stride(p, r);
  const Elem* yzero = reinterpret_cast<const Elem*>(g_zero16);
  Elem* ybase = reinterpret_cast<Elem*>(p.y) + p.out_off[slice] + yc;

  // B rows and y pieces of column tile ct (zeros past ct_end: the last
  // prefetch issues only loads of the zero constant).  B first: loads complete
  // in order, so the products, which need only B (mostly from L2), start
  // while y is still on its way from HBM.
  auto load_tile = [&](int ct, u32x4 (&yd)[2], u32x4 (&bd)[4][2]) {
    const int jw = ct * kExpandColsPerWG + wave * kExpandColsPerWave;
    const bool ycol_ok = ct < ct_end && jw + yc < out;  // out is a multiple of 8
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int row = jw + cb * 16 + n;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int k0 = ks * 32 + kg * 8;
        const bool ok = ct < ct_end && ks < nks && row < out && k0 < r;
        bd[cb][ks] = ld16_or0(Bs + (ok ? (int64_t)row * ldb + k0 : 0), ok);
      }
    }
    yd[0] = ld16_or0_nt(ycol_ok && ytok0 >= 0 ? ybase + jw + (int64_t)ytok0 * p.ldy : yzero, ycol_ok && ytok0 >= 0);
    yd[1] = ld16_or0_nt(ycol_ok && ytok1 >= 0 ? ybase + jw + (int64_t)ytok1 * p.ldy : yzero, ycol_ok && ytok1 >= 0);
  };
  u32x4 ya[2], ba[4][2], yb[2], bb[4][2];
  load_tile(ct_begin, ya, ba);
  // A unit of one column tile requests its (zero-constant) second tile here,
  // before the v operands, rather than in the loop: measured 11.8 -> 11.3 us
  // on the decode call (its consumers hold one tile each) and 62.1 -> 61.7 us
  // on mixed_rank_mlp; units of several tiles keep the order of the loop
  // (requesting their second tile here too was slower for them).
  const bool early = ct_end - ct_begin == 1;
  if (early) load_tile(ct_begin + 1, yb, bb);

  // the group's v operands, once per unit: vsrc fills lane (n, kg)'s fp32
  // v[token n][32 ks + 8 kg .. + 7] (values past the rank are masked below)
  f32x4 vraw[2][2];
  vsrc(vraw);
  float vv[2][8];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int k0 = ks * 32 + kg * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      vv[ks][i] = (k0 + i < r) ? vraw[ks][0][i] : 0.f;
      vv[ks][4 + i] = (k0 + 4 + i < r) ? vraw[ks][1][i] : 0.f;
    }
  }
  float unscale = 1.0f;
  if constexpr (Tr::kDtype == LORA_F16) {
    float mx = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(vv[ks][i]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (mx > 0.f) {
      int ex;
      frexpf(mx, &ex);
      const float sc = ldexpf(1.0f, 1 - ex);
      unscale = ldexpf(1.0f, ex - 1);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 8; ++i) vv[ks][i] *= sc;
    }
  }
  V vhi[2], vlo[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const Elem h = static_cast<Elem>(vv[ks][i]);
      vhi[ks][i] = h;
      vlo[ks][i] = static_cast<Elem>(vv[ks][i] - static_cast<float>(h));
    }

  auto compute_tile = [&](int ct, const u32x4 (&yd)[2], const u32x4 (&bd)[4][2]) {
    const int jw = ct * kExpandColsPerWG + wave * kExpandColsPerWave;
    const bool ycol_ok = jw + yc < out;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      V b0 = as_vec<V>(ragged_rank ? mask_tail16(bd[cb][0], kg * 8, r) : bd[cb][0]);
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      acc = M::mma(b0, vhi[0], acc);
      acc = M::mma(b0, vlo[0], acc);
      if (nks > 1) {
        V b1 = as_vec<V>(ragged_rank ? mask_tail16(bd[cb][1], 32 + kg * 8, r) : bd[cb][1]);
        acc = M::mma(b1, vhi[1], acc);
        acc = M::mma(b1, vlo[1], acc);
      }
      if constexpr (Tr::kDtype == LORA_F16) acc *= unscale;
      *reinterpret_cast<f32x4*>(&s_tr[wave][n][cb * 16 + kg * 4]) = acc;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = h ? ytok1 : ytok0;
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(&s_tr[wave][h * 8 + yr][yc]);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(&s_tr[wave][h * 8 + yr][yc + 4]);
      if (ycol_ok && t >= 0) {
        const float add[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t wd = yd[h][q];
          const float y0 = Tr::elem_to_float(wd & 0xffffu) + add[2 * q];
          const float y1 = Tr::elem_to_float(wd >> 16) + add[2 * q + 1];
          if constexpr (Tr::kDtype == LORA_BF16) o[q] = pack2_bf16(y0, y1);
          else o[q] = pack2_f16(y0, y1);
        }
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(ybase + jw + (int64_t)t * p.ldy));
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // two tiles per iteration, so that the register buffers alternate without copies
  for (int ct = ct_begin; ct < ct_end; ct += 2) {
    if (!early || ct != ct_begin) load_tile(ct + 1, yb, bb);
    compute_tile(ct, ya, ba);
    if (ct + 1 >= ct_end) break;
    load_tile(ct + 2, ya, ba);
    compute_tile(ct + 1, yb, bb);
  }
}

// The same group expand for fp32 data, on the vector ALUs: v is fp32 already
// and the products are plain fp32 FMAs (a 16x16 block of rank 64 would take
// sixteen 16x16x4 fp32 matrix instructions).  The wave puts the group's v rows
// (from vsrc, in the lane layout above) and its tokens (lane n's tok_n) into
// its LDS block s_v; per 256-column tile each lane then owns one of the wave's
// 64 columns: it reads that column's B row over the rank, forms the 16 tokens'
// dot products against the v rows (LDS broadcasts) and read-modify-writes y
// once per element.
template <typename VSrc>
__device__ inline void expand_group_f32(const ExpandParams& p, const VSrc& vsrc, int tok_n, float (*s_v)[kTrRow],
                                        int slice, int s, int r, int out, int ct_begin, int ct_end) {
  static_assert(kTrRow >= LORA_MAX_RANK + 1, "a v row and a token word fit a block row");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, kg = lane >> 4;
  f32x4 vraw[2][2];
  vsrc(vraw);  // lane (n, kg): v[token n][32 ks + 8 kg .. + 7], zeros past the rank
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int h = 0; h < 2; ++h) *reinterpret_cast<f32x4*>(&s_v[n][ks * 32 + kg * 8 + 4 * h]) = vraw[ks][h];
  if (kg == 0) s_v[n][LORA_MAX_RANK] = __int_as_float(tok_n);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int tk[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) tk[t] = __float_as_int(s_v[t][LORA_MAX_RANK]);
  const float* Bs = reinterpret_cast<const float*>(p.B[slice]) + (int64_t)s * out * p.r_max;
  const int ldb = b_row_stride(p, r);
  float* ybase = reinterpret_cast<float*>(p.y) + p.out_off[slice];
  const float* yzero = reinterpret_cast<const float*>(g_zero16);
  for (int ct = ct_begin; ct < ct_end; ++ct) {
    const int col = ct * kExpandColsPerWG + wave * kExpandColsPerWave + lane;
    const bool col_ok = col < out;
    // the tile's y values first, so that their loads are in flight together
    float yv[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const bool ok = col_ok && tk[t] >= 0;
      yv[t] = *(ok ? ybase + (int64_t)tk[t] * p.ldy + col : yzero);
    }
    float acc[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) acc[t] = 0.f;
    const float* brow = Bs + (int64_t)(col_ok ? col : 0) * ldb;
    for (int k0 = 0; k0 < r; k0 += 4) {  // rows hold whole 16-byte pieces up to the rank
      f32x4 b = ldf4_or0(brow + k0, col_ok);
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = k0 + i < r ? b[i] : 0.f;  // padding past the rank is not read as data
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(&s_v[t][k0]);
        acc[t] = __builtin_fmaf(b[0], v4[0], acc[t]);
        acc[t] = __builtin_fmaf(b[1], v4[1], acc[t]);
        acc[t] = __builtin_fmaf(b[2], v4[2], acc[t]);
        acc[t] = __builtin_fmaf(b[3], v4[3], acc[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < 16; ++t)
      if (col_ok && tk[t] >= 0) ybase[(int64_t)tk[t] * p.ldy + col] = yv[t] + acc[t];
  }
  // the block is rewritten by the wave's next unit only after these reads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace

}  // namespace lora
