// Mask ("laning") form of shrink + expand, for batches whose adapters,
// stacked, have few rank lanes: S * r_max <= kMaskMaxLanes.
//
// "[Hardware][TPU][V1] Better tpu multilora compilation" reports, on TPU, a
// masked formulation beating the per-token gather, and LoRA laning -- several
// adapters packed side by side so that one matrix product serves them all --
// cutting the number of matrix products.  Here the stacked A tensor
// [S][r_max][D] is read as one matrix of L = S * r_max rows (the lanes), and
//   shrink:  W[t][c] = sum_d x[t][d] * A_all[c][d]       for every lane c
//            (a dense product of each 16-token tile with all lanes, no
//            grouping of tokens by slot and no segment record);
//   mask:    v[t][k] = scale[s] * W[t][s * r_max + k]    (s = idx[t], k < r_s)
//   expand:  y[t][j] += sum_c B_all[j][c] * vm[t][c], vm being v placed in
//            the token's own lanes and zero in every other lane, B_all[j][c] =
//            B[c / r_max][j][c % r_max].
// Both products run on the matrix cores; the expand takes the fp32 v as hi +
// lo 16-bit parts as the gather path does.  The shrink cuts the contraction
// into kp parts whose fp32 partial sums go to the caller's workspace
// [slice][part][T][L]; the expand sums a token's own lanes over the parts in
// part order (no atomics, no clearing pass), so the result is deterministic.
// Two launches; every token of the batch is read once per slice whatever its
// slot, and rows of tokens without a valid slot are left untouched in y.
#include "common.h"
#include "expand_unit.h"
#include "shrink_unit.h"

namespace lora {

namespace {

constexpr int kMaskThreads = 256;
constexpr int kMaskKChunk = 256;    // smallest contraction range of one shrink part
constexpr int kMaskMaxParts = 16;
constexpr int kMaskUnitsTarget = 256;

struct MaskParams {
  const void* x;
  int64_t ldx;
  const void* A[LORA_MAX_SLICES];
  const void* B[LORA_MAX_SLICES];
  int64_t out_size[LORA_MAX_SLICES];
  int64_t out_off[LORA_MAX_SLICES];
  const int32_t* idx;
  const int32_t* ranks;  // nullable
  const float* scale;    // nullable
  float* part;           // [n_slices][kp][T][L]
  float* v;              // nullable: [n_slices][T][r_max]
  void* y;
  int64_t ldy;
  int32_t T, D, S, r_max, n_slices, L, kp, k_per_part;
};

__device__ inline int slot_of(const MaskParams& p, int t) {
  if (t < 0 || t >= p.T) return -1;
  const int s = p.idx[t];
  return s >= 0 && s < p.S ? s : -1;
}

// Whether token t's row of y receives a delta: a valid slot of rank > 0
// (other rows are never written, so they stay bit-identical).
__device__ inline bool row_gets_delta(const MaskParams& p, int t) {
  const int s = slot_of(p, t);
  return s >= 0 && slot_rank(p.ranks, s, p.r_max) > 0;
}

// ---- shrink: unit (16-token tile, K part, slice); wave w computes the lane
// blocks w and w + 4 (16 lanes each) over the part's K steps.
template <typename Elem>
__global__ __launch_bounds__(kMaskThreads) void mask_shrink_kernel(MaskParams p) {
  warm_args(p);
  using M = StepMma<Elem>;
  constexpr int kVec = Traits<Elem>::kVec;
  constexpr int kStep = 4 * kVec;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, m = lane & 15, kg = lane >> 4;
  const int n_tiles = (p.T + 15) / 16;
  const int nblk = p.L / 16;
  const int lanes_real = p.S * p.r_max;
  const int64_t n_units = (int64_t)n_tiles * p.kp * p.n_slices;
  for (int64_t u = blockIdx.x; u < n_units; u += gridDim.x) {
    const int slice = (int)(u % p.n_slices);
    const int64_t rest = u / p.n_slices;
    const int part = (int)(rest % p.kp);
    const int tile = (int)(rest / p.kp);
    const int t = tile * 16 + m;
    const bool tok_ok = t < p.T;
    const int k0 = part * p.k_per_part, k1 = min(p.D, k0 + p.k_per_part);
    const Elem* xrow = reinterpret_cast<const Elem*>(p.x) + (int64_t)(tok_ok ? t : 0) * p.ldx;
    const Elem* Ab = reinterpret_cast<const Elem*>(p.A[slice]);
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    for (int k = k0; k < k1; k += kStep) {
      const int d = k + kg * kVec;  // D, k0, k1 are multiples of kVec
      const bool okd = d < k1;
      const u32x4 xa = ld16_or0(xrow + (okd ? d : 0), tok_ok && okd);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int blk = wave + 4 * b;
        const int row = blk * 16 + m;
        const bool ok = blk < nblk && row < lanes_real && okd;
        const u32x4 aa = ld16_or0(Ab + (ok ? (int64_t)row * p.D + d : 0), ok);
        acc[b] = M::mma(xa, aa, acc[b]);
      }
    }
    // lane (m, kg) holds W[token 4 kg + i][lane 16 blk + m]
    float* dst = p.part + (((int64_t)slice * p.kp + part) * p.T) * p.L;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int blk = wave + 4 * b;
      if (blk >= nblk) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t2 = tile * 16 + 4 * kg + i;
        if (t2 < p.T) dst[(int64_t)t2 * p.L + blk * 16 + m] = acc[b][i];
      }
    }
  }
}

// ---- expand: unit (16-token tile, slice, 256-column tile); wave w takes
// columns 64 w .. 64 w + 63 of the tile, as the gather path's group unit does.
template <typename Elem>
__global__ __launch_bounds__(kMaskThreads, 2) void mask_expand_kernel(MaskParams p) {
  warm_args(p);
  constexpr int kVec = Traits<Elem>::kVec;
  constexpr int kStep = 4 * kVec;
  constexpr int kMaxQ = kMaskMaxLanes / kStep;  // K steps over the lanes
  constexpr bool HALF = sizeof(Elem) == 2;
  using Tr = Traits<Elem>;
  __shared__ __attribute__((aligned(16))) float s_tr[4][16][kTrRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kg = lane >> 4;
  const int yr = lane >> 3, yc = (lane & 7) * 8 / (HALF ? 1 : 2);  // fp32: 4 columns per 16 bytes
  const int n_tiles = (p.T + 15) / 16;
  int ctot = 0;
  for (int i = 0; i < p.n_slices; ++i) ctot += (int)ceil_div(p.out_size[i], kExpandColsPerWG);
  const int nq = p.L / kStep;
  const int64_t n_units = (int64_t)n_tiles * ctot;
  for (int64_t u = blockIdx.x; u < n_units; u += gridDim.x) {
    const int tile = (int)(u / ctot);
    int ct = (int)(u % ctot), slice = 0;
    while (ct >= (int)ceil_div(p.out_size[slice], kExpandColsPerWG)) {
      ct -= (int)ceil_div(p.out_size[slice], kExpandColsPerWG);
      ++slice;
    }
    const int out = (int)p.out_size[slice];
    // this lane's MFMA token (column n of the v operand) and its slot
    const int tok_n = tile * 16 + n;
    const int s_n = slot_of(p, tok_n);
    const int r_n = s_n >= 0 ? slot_rank(p.ranks, s_n, p.r_max) : 0;
    const float sc_n = s_n >= 0 && p.scale ? p.scale[s_n] : 1.0f;

    // masked v operand: lane (n, kg) holds vm[token n][c .. c + kVec - 1] for
    // c = q kStep + kg kVec, the sum of the token's own lanes over the parts
    float vm[kMaxQ][kVec];
#pragma unroll
    for (int q = 0; q < kMaxQ; ++q) {
      const int c = q * kStep + kg * kVec;
      const int s_c = c / p.r_max, within = c - s_c * p.r_max;
      const bool on = q < nq && s_n >= 0 && s_c == s_n;
      float sum[kVec];
#pragma unroll
      for (int e = 0; e < kVec; ++e) sum[e] = 0.f;
      const float* src = p.part + (((int64_t)slice * p.kp) * p.T + (on ? tok_n : 0)) * p.L + (on ? c : 0);
      for (int pp = 0; pp < p.kp; ++pp) {
#pragma unroll
        for (int h = 0; h < kVec / 4; ++h) {
          const f32x4 w = ldf4_or0(src + (int64_t)pp * p.T * p.L + 4 * h, on);
          sum[4 * h] += w[0];
          sum[4 * h + 1] += w[1];
          sum[4 * h + 2] += w[2];
          sum[4 * h + 3] += w[3];
        }
      }
#pragma unroll
      for (int e = 0; e < kVec; ++e) vm[q][e] = on && within + e < r_n ? sum[e] * sc_n : 0.f;
      // v of the first column tile's unit: the token's own row (zeros for
      // tokens without a valid slot, written from the first r_max lanes)
      if (p.v && ct == 0 && wave == 0 && tok_n < p.T && q < nq) {
        float* vr = p.v + ((int64_t)slice * p.T + tok_n) * p.r_max;
        if (on) {
#pragma unroll
          for (int h = 0; h < kVec / 4; ++h)
            *reinterpret_cast<f32x4*>(vr + within + 4 * h) =
                f32x4{vm[q][4 * h], vm[q][4 * h + 1], vm[q][4 * h + 2], vm[q][4 * h + 3]};
        } else if (s_n < 0 && c < p.r_max) {
#pragma unroll
          for (int h = 0; h < kVec / 4; ++h) *reinterpret_cast<f32x4*>(vr + c + 4 * h) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    // fp16: scale each token's row by a power of two so that hi and lo stay
    // in the normal range (undone exactly on the fp32 result)
    float unscale = 1.0f;
    if constexpr (Tr::kDtype == LORA_F16) {
      float mx = 0.f;
#pragma unroll
      for (int q = 0; q < kMaxQ; ++q)
#pragma unroll
        for (int e = 0; e < kVec; ++e) mx = fmaxf(mx, fabsf(vm[q][e]));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (mx > 0.f) {
        int ex;
        frexpf(mx, &ex);
        const float scl = ldexpf(1.0f, 1 - ex);
        unscale = ldexpf(1.0f, ex - 1);
#pragma unroll
        for (int q = 0; q < kMaxQ; ++q)
#pragma unroll
          for (int e = 0; e < kVec; ++e) vm[q][e] *= scl;
      }
    }

    // y^T[j][token] = sum_c B_all[j][c] vm[token][c], per 16-column block cb
    const int jw = ct * kExpandColsPerWG + wave * kExpandColsPerWave;
    const Elem* Bb = reinterpret_cast<const Elem*>(p.B[slice]);
    f32x4 acc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < kMaxQ; ++q) {
      if (q >= nq) continue;  // uniform; predicated so that the loop unrolls
      const int c = q * kStep + kg * kVec;
      const int s_c = c / p.r_max, within = c - s_c * p.r_max;
      const int r_c = s_c < p.S ? slot_rank(p.ranks, s_c, p.r_max) : 0;
      u32x4 bq[4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int j = jw + cb * 16 + n;
        const bool ok = j < out && s_c < p.S && within < r_c;
        bq[cb] = ld16_or0(Bb + (ok ? ((int64_t)s_c * out + j) * p.r_max + within : 0), ok);
      }
      if constexpr (HALF) {
        using Mf = Mfma<Elem>;
        using V = typename Mf::vec;
        V hi, lo;
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
          const Elem h = static_cast<Elem>(vm[q][e]);
          hi[e] = h;
          lo[e] = static_cast<Elem>(vm[q][e] - static_cast<float>(h));
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const V bv = as_vec<V>(mask_tail16(bq[cb], within, r_c));  // B past the slot's rank is never used
          acc[cb] = Mf::mma(bv, hi, acc[cb]);
          acc[cb] = Mf::mma(bv, lo, acc[cb]);
        }
      } else {
        u32x4 vq;
#pragma unroll
        for (int e = 0; e < 4; ++e) vq[e] = __float_as_uint(vm[q][e]);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          u32x4 bv = bq[cb];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w = bv[e];
            bv[e] = within + e < r_c ? w : 0u;
          }
          acc[cb] = StepMma<float>::mma(bv, vq, acc[cb]);
        }
      }
    }
    if constexpr (Tr::kDtype == LORA_F16) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[cb] *= unscale;
    }
    // lane (n, kg) holds y^T[column 16 cb + 4 kg + i][token n]: through LDS to
    // lane-contiguous rows of y, one rounding per element
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) *reinterpret_cast<f32x4*>(&s_tr[wave][n][cb * 16 + kg * 4]) = acc[cb];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    Elem* ybase = reinterpret_cast<Elem*>(p.y) + p.out_off[slice];
    if constexpr (HALF) {
      // 8 lanes per token row: 64 columns of 16-bit y
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int tr = h * 8 + yr;
        const int t = tile * 16 + tr;
        const int col = jw + yc;
        if (t < p.T && row_gets_delta(p, t) && col < out) {
          const f32x4 a0 = *reinterpret_cast<const f32x4*>(&s_tr[wave][tr][yc]);
          const f32x4 a1 = *reinterpret_cast<const f32x4*>(&s_tr[wave][tr][yc + 4]);
          u32x4* yp = reinterpret_cast<u32x4*>(ybase + (int64_t)t * p.ldy + col);
          const u32x4 old = *yp;
          const float add[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          u32x4 o;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const uint32_t wd = old[qq];
            const float y0 = Tr::elem_to_float(wd & 0xffffu) + add[2 * qq];
            const float y1 = Tr::elem_to_float(wd >> 16) + add[2 * qq + 1];
            o[qq] = Tr::kDtype == LORA_BF16 ? pack2_bf16(y0, y1) : pack2_f16(y0, y1);
          }
          *yp = o;
        }
      }
    } else {
      // fp32 y: 16 lanes per token row (4 columns each), 4 token rows per pass
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int tr = h * 4 + (lane >> 4);
        const int cc = (lane & 15) * 4;
        const int t = tile * 16 + tr;
        const int col = jw + cc;
        if (t < p.T && row_gets_delta(p, t) && col < out) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(&s_tr[wave][tr][cc]);
          f32x4* yp = reinterpret_cast<f32x4*>(ybase + (int64_t)t * p.ldy + col);
          *yp = *yp + a;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

template <typename Elem>
hipError_t mask_launch(const MaskParams& p, hipStream_t stream) {
  const int64_t n_tiles = ceil_div(p.T, 16);
  int64_t ctot = 0;
  for (int i = 0; i < p.n_slices; ++i) ctot += ceil_div(p.out_size[i], kExpandColsPerWG);
  const int g1 = persistent_grid(reinterpret_cast<const void*>(&mask_shrink_kernel<Elem>), kMaskThreads, 0,
                                 n_tiles * p.kp * p.n_slices);
  hipLaunchKernelGGL(mask_shrink_kernel<Elem>, dim3(g1), dim3(kMaskThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int g2 = persistent_grid(reinterpret_cast<const void*>(&mask_expand_kernel<Elem>), kMaskThreads, 0,
                                 n_tiles * ctot);
  hipLaunchKernelGGL(mask_expand_kernel<Elem>, dim3(g2), dim3(kMaskThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// Lanes rounded up to whole 16-lane blocks and to whole K steps of the expand.
int32_t mask_lanes(lora_dtype dt, int32_t S, int32_t r_max) {
  const int step = dt == LORA_F32 ? 16 : 32;
  return (int32_t)ceil_div((int64_t)S * r_max, step) * step;
}

// K parts of the shrink: enough units to fill about a round of the chip, each
// part at least kMaskKChunk long, at most kMaskMaxParts.
int32_t mask_parts(int32_t T, int32_t D, int32_t n_slices) {
  const int64_t base = ceil_div(T, 16) * n_slices;
  int64_t kp = ceil_div(kMaskUnitsTarget, base > 0 ? base : 1);
  kp = kp < D / kMaskKChunk ? kp : D / kMaskKChunk;
  kp = kp < kMaskMaxParts ? kp : kMaskMaxParts;
  return (int32_t)(kp < 1 ? 1 : kp);
}

int64_t mask_need_bytes(lora_dtype dt, int32_t T, int32_t D, int32_t S, int32_t n_slices, int32_t r_max) {
  return (int64_t)n_slices * mask_parts(T, D, n_slices) * T * mask_lanes(dt, S, r_max) * 4;
}

hipError_t launch_mask(lora_dtype dt, const ShrinkParams& sp, const ExpandParams& ep, const int32_t* idx,
                       float* part, float* v, hipStream_t stream) {
  MaskParams p{};
  p.x = sp.x;
  p.ldx = sp.ldx;
  for (int i = 0; i < sp.n_slices; ++i) {
    p.A[i] = sp.A[i];
    p.B[i] = ep.B[i];
    p.out_size[i] = ep.out_size[i];
    p.out_off[i] = ep.out_off[i];
  }
  p.idx = idx;
  p.ranks = sp.ranks;
  p.scale = sp.scale;
  p.part = part;
  p.v = v;
  p.y = ep.y;
  p.ldy = ep.ldy;
  p.T = sp.T;
  p.D = sp.D;
  p.S = sp.S;
  p.r_max = sp.r_max;
  p.n_slices = sp.n_slices;
  p.L = mask_lanes(dt, sp.S, sp.r_max);
  p.kp = mask_parts(sp.T, sp.D, sp.n_slices);
  const int step = dt == LORA_F32 ? 16 : 32;
  p.k_per_part = (int32_t)(ceil_div(ceil_div(sp.D, p.kp), step) * step);
  switch (dt) {
    case LORA_F32: return mask_launch<float>(p, stream);
    case LORA_F16: return mask_launch<half_t>(p, stream);
    case LORA_BF16: return mask_launch<bf16_t>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace lora
