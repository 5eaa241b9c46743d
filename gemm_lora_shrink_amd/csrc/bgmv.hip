// Gather path (BGMV) for decode-shaped batches: each work item is a group of
// at most 16 tokens that share one adapter slot.  The gather semantics are
// those of the baseline in "[Hardware][TPU][V1] Better tpu multilora
// compilation" (review thread): a token multiplies the stacked matrix of its
// own slot.  Instead of materialising a per-token copy of the weights (the
// index_select that the same thread names as the slow part), a workgroup reads
// its slot's rows once for the whole group, with 16-byte coalesced loads.
//
// Shrink: a workgroup owns (group, slice, D-chunk).  The group's x rows for the
// chunk are staged in LDS; each of the 4 waves takes every 4th rank row, and
// each lane takes 16 bytes of D per step, accumulating fp32 dot products (dot2
// for 16-bit data).  The per-lane partial sums are then reduced across the
// wavefront with a halving butterfly (each step trades half of the remaining
// values with the partner lane), so 64 (rank, token) sums cost 63 shuffles
// instead of 384.  When D is split over several workgroups the partial results
// are added into v with fp32 atomics; v was cleared beforehand inside the same
// lora_shrink call.
//
// Expand: a workgroup owns (group, slice, column tile).  The group's v rows are
// staged in LDS (rank columns past the slot's rank read as 0); each lane owns 4
// consecutive output columns, forms the fp32 dot products over the rank with
// the slot's B rows, then read-modify-writes y with one rounding per element.
#include "common.h"

namespace lora {

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerWG = kThreads / 64;
constexpr int kRowsPerPass = 4;                       // rank rows per wave per pass
constexpr int kItemsPerPass = kRowsPerPass * kGroup;  // 64 (rank, token) sums per pass
constexpr int kXChunkBytes = 2048;                    // bytes of one x row staged per workgroup
constexpr int kColsPerLane = 4;
constexpr int kExpandCols = kThreads * kColsPerLane;  // 1024 output columns per workgroup
constexpr int kKChunk = 8;                            // rank elements per B load step

__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// One step of the halving butterfly: lanes whose bit HALF is set keep the upper
// half of their values, the others the lower half, and each adds what its
// partner lane sends.
template <int HALF>
__device__ inline void butterfly_step(float (&vals)[64], bool upper) {
#pragma unroll
  for (int j = 0; j < HALF; ++j) {
    const float send = upper ? vals[j] : vals[j + HALF];
    const float keep = upper ? vals[j + HALF] : vals[j];
    vals[j] = keep + __shfl_xor(send, HALF, 64);
  }
}

// Halving butterfly: on entry lane l holds 64 partial sums vals[0..63]; on exit
// vals[0] of lane l is the wave-wide sum of element l.
__device__ inline float wave_transpose_reduce64(float (&vals)[64]) {
  const int lane = __lane_id();
  butterfly_step<32>(vals, (lane & 32) != 0);
  butterfly_step<16>(vals, (lane & 16) != 0);
  butterfly_step<8>(vals, (lane & 8) != 0);
  butterfly_step<4>(vals, (lane & 4) != 0);
  butterfly_step<2>(vals, (lane & 2) != 0);
  butterfly_step<1>(vals, (lane & 1) != 0);
  return vals[0];
}

template <typename Elem>
__global__ __launch_bounds__(kThreads) void bgmv_shrink_kernel(ShrinkParams p, int use_tiles, int nsplit,
                                                               int d_chunk, int atomic_out) {
  using Tr = Traits<Elem>;
  constexpr int kVec = Tr::kVec;
  constexpr int kChunkElems = kXChunkBytes / sizeof(Elem);
  __shared__ __attribute__((aligned(16))) Elem s_x[kGroup][kChunkElems];
  __shared__ int s_tok[kGroup];

  // work list: (16-token unit, D split, slice), unit fastest, so that the
  // groups of one slot (adjacent in the list) read the same A rows in one L2.
  // A tile of 64 tokens is processed as four 16-token units.
  const SegLayout L = seg_layout(p.T, p.S);
  const int sub_per_item = use_tiles ? kTile / kGroup : 1;
  const int64_t n_units = (int64_t)record_items(p.rec, p.T, p.S, use_tiles != 0) * sub_per_item;
  const WorkRange R = xcd_work_range(n_units * nsplit * p.n_slices);
  const int tid = threadIdx.x;
  const int lane = __lane_id();
  const int wave = tid >> 6;

  for (int64_t w = R.begin; w < R.end; w += R.step) {
  const int64_t unit = w % n_units;
  const int64_t rest = w / n_units;
  const int split = (int)(rest % nsplit);
  const int slice = (int)(rest / nsplit);
  const int64_t item_id = unit / sub_per_item;
  const int sub = (int)(unit - item_id * sub_per_item);
  Item it;
  if (!read_item(p.rec, p.T, p.S, use_tiles != 0, item_id, it)) continue;
  const int cnt = min(kGroup, it.cnt - sub * kGroup);
  if (cnt <= 0) continue;
  const int s = it.slot;
  const int r = slot_rank(p.ranks, s, p.r_max);
  if (r == 0) continue;
  const int d0 = split * d_chunk;
  const int dlen = min(d_chunk, p.D - d0);
  if (dlen <= 0) continue;

  if (tid < kGroup) {
    const int t = item_token(p.rec, p.T, p.S, use_tiles != 0, item_id, sub * kGroup + tid, it.cnt);
    s_tok[tid] = t < 0 ? 0 : t;
  }
  __syncthreads();

  // stage the group's x rows for [d0, d0 + dlen): every load is issued before
  // the first LDS store, so the staging costs one memory round trip
  {
    constexpr int kPerThread = kGroup * kXChunkBytes / 16 / kThreads;  // 8
    const int vecs_per_row = dlen / kVec;
    const int total = cnt * vecs_per_row;
    const Elem* xb = reinterpret_cast<const Elem*>(p.x);
    u32x4 tmp[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int e = tid + j * kThreads;
      if (e < total) {
        const int g = e / vecs_per_row;
        const int c = e - g * vecs_per_row;
        tmp[j] = ld16(xb + (int64_t)s_tok[g] * p.ldx + d0 + c * kVec);
      }
    }
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int e = tid + j * kThreads;
      if (e < total) {
        const int g = e / vecs_per_row;
        const int c = e - g * vecs_per_row;
        *reinterpret_cast<u32x4*>(&s_x[g][c * kVec]) = tmp[j];
      }
    }
  }
  __syncthreads();

  const float sc = p.scale ? p.scale[s] : 1.0f;
  const Elem* Ab = reinterpret_cast<const Elem*>(p.A[slice]) + (int64_t)s * p.r_max * p.D;
  float* vout = p.v + (int64_t)slice * p.v_slice_stride;
  const int n_pass = (int)ceil_div(r, kRowsPerPass * kWavesPerWG);

  for (int pass = 0; pass < n_pass; ++pass) {
    float acc[kItemsPerPass];
#pragma unroll
    for (int j = 0; j < kItemsPerPass; ++j) acc[j] = 0.f;
    int krow[kRowsPerPass];
#pragma unroll
    for (int q = 0; q < kRowsPerPass; ++q) krow[q] = (pass * kRowsPerPass + q) * kWavesPerWG + wave;

    constexpr int kSteps = kChunkElems / (64 * kVec);  // 16-byte steps per lane per chunk
    u32x4 a[kSteps][kRowsPerPass];
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int dd = (st * 64 + lane) * kVec;
#pragma unroll
      for (int q = 0; q < kRowsPerPass; ++q) {
        const bool ok = krow[q] < r && dd < dlen;
        a[st][q] = ld16_or0(Ab + (ok ? (int64_t)krow[q] * p.D + d0 + dd : 0), ok);
      }
    }
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int dd = (st * 64 + lane) * kVec;
      if (dd < dlen) {
#pragma unroll
        for (int g = 0; g < kGroup; ++g) {
          if (g < cnt) {
            const u32x4 xv = *reinterpret_cast<const u32x4*>(&s_x[g][dd]);
#pragma unroll
            for (int q = 0; q < kRowsPerPass; ++q)
              acc[q * kGroup + g] = Tr::dot(a[st][q], xv, acc[q * kGroup + g]);
          }
        }
      }
    }
    const float sum = wave_transpose_reduce64(acc);
    const int q = lane / kGroup, g = lane % kGroup;
    const int k = (pass * kRowsPerPass + q) * kWavesPerWG + wave;
    if (g < cnt && k < r) {
      float* dst = vout + (int64_t)s_tok[g] * p.r_max + k;
      if (atomic_out) atomicAdd(dst, sum * sc);
      else *dst = sum * sc;
    }
  }
  __syncthreads();  // the next work item reuses s_tok and s_x
  }
}

// 4 consecutive y elements: 16 bytes of fp32 or 8 bytes of a 16-bit type.
template <typename Elem> struct YChunk { typedef u32x2 type; };
template <> struct YChunk<float> { typedef f32x4 type; };

// y += acc for 4 consecutive elements, one rounding per element.
template <typename Elem>
__device__ inline void store_y4(Elem* dst, const float* acc, typename YChunk<Elem>::type yv) {
  if constexpr (sizeof(Elem) == 4) {
    f32x4 y = yv;
    y[0] += acc[0];
    y[1] += acc[1];
    y[2] += acc[2];
    y[3] += acc[3];
    *reinterpret_cast<f32x4*>(dst) = y;
  } else {
    using Tr = Traits<Elem>;
    const uint32_t w0 = yv[0], w1 = yv[1];
    const float y0 = Tr::elem_to_float(w0 & 0xffffu) + acc[0];
    const float y1 = Tr::elem_to_float(w0 >> 16) + acc[1];
    const float y2 = Tr::elem_to_float(w1 & 0xffffu) + acc[2];
    const float y3 = Tr::elem_to_float(w1 >> 16) + acc[3];
    u32x2 o;
    if constexpr (Tr::kDtype == LORA_BF16) {
      o[0] = float_to_bf16_bits(y0) | (float_to_bf16_bits(y1) << 16);
      o[1] = float_to_bf16_bits(y2) | (float_to_bf16_bits(y3) << 16);
    } else {
      o[0] = float_to_f16_bits(y0) | (float_to_f16_bits(y1) << 16);
      o[1] = float_to_f16_bits(y2) | (float_to_f16_bits(y3) << 16);
    }
    *reinterpret_cast<u32x2*>(dst) = o;
  }
}


template <typename Elem>
__global__ __launch_bounds__(kThreads) void bgmv_expand_kernel(ExpandParams p, int use_tiles, int n_ct) {
  using Tr = Traits<Elem>;
  __shared__ __attribute__((aligned(16))) float s_v[kGroup][LORA_MAX_RANK];
  __shared__ int s_tok[kGroup];

  // work list: (16-token unit, column tile, slice), unit fastest
  const SegLayout L = seg_layout(p.T, p.S);
  const int sub_per_item = use_tiles ? kTile / kGroup : 1;
  const int64_t n_units = (int64_t)record_items(p.rec, p.T, p.S, use_tiles != 0) * sub_per_item;
  const WorkRange R = xcd_work_range(n_units * n_ct * p.n_slices);
  const int tid = threadIdx.x;

  for (int64_t w = R.begin; w < R.end; w += R.step) {
  const int64_t unit = w % n_units;
  const int64_t rest = w / n_units;
  const int ct = (int)(rest % n_ct);
  const int slice = (int)(rest / n_ct);
  const int64_t item_id = unit / sub_per_item;
  const int sub = (int)(unit - item_id * sub_per_item);
  Item it;
  if (!read_item(p.rec, p.T, p.S, use_tiles != 0, item_id, it)) continue;
  const int cnt = min(kGroup, it.cnt - sub * kGroup);
  if (cnt <= 0) continue;
  const int out = (int)p.out_size[slice];
  const int j0 = ct * kExpandCols;
  if (j0 >= out) continue;
  const int s = it.slot;
  const int r = slot_rank(p.ranks, s, p.r_max);
  if (r == 0) continue;

  if (tid < kGroup) {
    const int t = item_token(p.rec, p.T, p.S, use_tiles != 0, item_id, sub * kGroup + tid, it.cnt);
    s_tok[tid] = t < 0 ? 0 : t;
  }
  __syncthreads();
  const float* vb = p.v + (int64_t)slice * p.v_slice_stride;
  {
    constexpr int kPerThread = kGroup * LORA_MAX_RANK / kThreads;  // 4
    float tmp[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int e = tid + j * kThreads;
      const int g = e / LORA_MAX_RANK, k = e % LORA_MAX_RANK;
      tmp[j] = (g < cnt && k < r) ? vb[(int64_t)s_tok[g] * p.r_max + k] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int e = tid + j * kThreads;
      s_v[e / LORA_MAX_RANK][e % LORA_MAX_RANK] = tmp[j];
    }
  }
  __syncthreads();

  const int j = j0 + tid * kColsPerLane;
  if (j < out) {
  const Elem* Bb = reinterpret_cast<const Elem*>(p.B[slice]) + ((int64_t)s * out + j) * p.r_max;
  Elem* yb = reinterpret_cast<Elem*>(p.y) + p.out_off[slice] + j;
  // the group's y values are loaded before any store, so the loads of all
  // tokens are in flight together
  typedef typename YChunk<Elem>::type ychunk_t;
  ychunk_t ysave[kGroup];
#pragma unroll
  for (int g = 0; g < kGroup; ++g)
    if (g < cnt) ysave[g] = *reinterpret_cast<const ychunk_t*>(yb + (int64_t)s_tok[g] * p.ldy);
  float acc[kGroup][kColsPerLane];
#pragma unroll
  for (int g = 0; g < kGroup; ++g)
#pragma unroll
    for (int c = 0; c < kColsPerLane; ++c) acc[g][c] = 0.f;

  for (int k0 = 0; k0 < r; k0 += kKChunk) {
    float bf[kColsPerLane][kKChunk];
#pragma unroll
    for (int c = 0; c < kColsPerLane; ++c) {
      const Elem* row = Bb + (int64_t)c * p.r_max + k0;
      if constexpr (sizeof(Elem) == 4) {
        // 8 fp32 values = two 16-byte loads; r_max is a multiple of 4
        u32x4 lo = ld16(row);
        u32x4 hi = (k0 + 4 < p.r_max) ? ld16(row + 4) : u32x4{0, 0, 0, 0};
        Tr::to_float(lo, &bf[c][0]);
        Tr::to_float(hi, &bf[c][4]);
      } else {
        Tr::to_float(ld16(row), &bf[c][0]);  // r_max is a multiple of 8
      }
#pragma unroll
      for (int kk = 0; kk < kKChunk; ++kk)
        if (k0 + kk >= r) bf[c][kk] = 0.f;
    }
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      if (g < cnt) {
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(&s_v[g][k0]);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(&s_v[g][k0 + 4]);
#pragma unroll
        for (int c = 0; c < kColsPerLane; ++c) {
          float a = acc[g][c];
          a = __builtin_fmaf(bf[c][0], v0[0], a);
          a = __builtin_fmaf(bf[c][1], v0[1], a);
          a = __builtin_fmaf(bf[c][2], v0[2], a);
          a = __builtin_fmaf(bf[c][3], v0[3], a);
          a = __builtin_fmaf(bf[c][4], v1[0], a);
          a = __builtin_fmaf(bf[c][5], v1[1], a);
          a = __builtin_fmaf(bf[c][6], v1[2], a);
          a = __builtin_fmaf(bf[c][7], v1[3], a);
          acc[g][c] = a;
        }
      }
    }
  }

#pragma unroll
  for (int g = 0; g < kGroup; ++g)
    if (g < cnt) store_y4<Elem>(yb + (int64_t)s_tok[g] * p.ldy, acc[g], ysave[g]);
  }
  __syncthreads();  // the next work item reuses s_tok and s_v
  }
}

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t n4 = n >> 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    reinterpret_cast<f32x4*>(p)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t i = (n4 << 2) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.f;
}

template <typename Elem>
hipError_t shrink_launch(const ShrinkParams& p, bool tiles, hipStream_t stream) {
  const SegLayout L = seg_layout(p.T, p.S);
  const int sub = tiles ? kTile / kGroup : 1;
  const int64_t cap = tiles ? L.cap_tiles : L.cap_groups;
  const int chunk = kXChunkBytes / (int)sizeof(Elem);
  const int nsplit = (int)ceil_div(p.D, chunk);
  const int grid = persistent_grid(reinterpret_cast<const void*>(&bgmv_shrink_kernel<Elem>), kThreads, 0,
                                   cap * sub * nsplit * p.n_slices);
  hipLaunchKernelGGL(bgmv_shrink_kernel<Elem>, dim3(grid), dim3(kThreads), 0, stream, p, tiles ? 1 : 0, nsplit,
                     chunk, nsplit > 1 ? 1 : 0);
  return hipGetLastError();
}

template <typename Elem>
hipError_t expand_launch(const ExpandParams& p, bool tiles, hipStream_t stream) {
  const SegLayout L = seg_layout(p.T, p.S);
  const int sub = tiles ? kTile / kGroup : 1;
  const int64_t cap = tiles ? L.cap_tiles : L.cap_groups;
  int64_t max_out = 0;
  for (int i = 0; i < p.n_slices; ++i) max_out = p.out_size[i] > max_out ? p.out_size[i] : max_out;
  const int n_ct = (int)ceil_div(max_out, kExpandCols);
  const int grid = persistent_grid(reinterpret_cast<const void*>(&bgmv_expand_kernel<Elem>), kThreads, 0,
                                   cap * sub * n_ct * p.n_slices);
  hipLaunchKernelGGL(bgmv_expand_kernel<Elem>, dim3(grid), dim3(kThreads), 0, stream, p, tiles ? 1 : 0, n_ct);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = ceil_div(ceil_div(n, 4), 256);
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_bgmv_shrink(lora_dtype dt, const ShrinkParams& p, bool tiles, hipStream_t stream) {
  switch (dt) {
    case LORA_F32: return shrink_launch<float>(p, tiles, stream);
    case LORA_F16: return shrink_launch<half_t>(p, tiles, stream);
    case LORA_BF16: return shrink_launch<bf16_t>(p, tiles, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bgmv_expand(lora_dtype dt, const ExpandParams& p, bool tiles, hipStream_t stream) {
  switch (dt) {
    case LORA_F32: return expand_launch<float>(p, tiles, stream);
    case LORA_F16: return expand_launch<half_t>(p, tiles, stream);
    case LORA_BF16: return expand_launch<bf16_t>(p, tiles, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace lora
