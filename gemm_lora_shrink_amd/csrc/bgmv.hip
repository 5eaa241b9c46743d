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
__global__ __launch_bounds__(kThreads) void bgmv_shrink_kernel(ShrinkParams p, int which_list, int sub_per_item,
                                                               int d_chunk, int atomic_out) {
  using Tr = Traits<Elem>;
  constexpr int kVec = Tr::kVec;
  constexpr int kChunkElems = kXChunkBytes / sizeof(Elem);
  __shared__ __attribute__((aligned(16))) Elem s_x[kGroup][kChunkElems];
  __shared__ int s_tok[kGroup];

  const SegLayout L = seg_layout(p.T, p.S);
  const int item_id = blockIdx.x / sub_per_item;
  Item it;
  if (!load_item(p.rec, p.T, p.S, which_list != 0, item_id, it)) return;
  const int sub = blockIdx.x - item_id * sub_per_item;
  const int cnt = min(kGroup, it.cnt - sub * kGroup);
  if (cnt <= 0) return;
  const int s = it.slot;
  const int r = slot_rank(p.ranks, s, p.r_max);
  if (r == 0) return;
  const int slice = blockIdx.y;
  const int d0 = blockIdx.z * d_chunk;
  const int dlen = min(d_chunk, p.D - d0);
  if (dlen <= 0) return;

  const int tid = threadIdx.x;
  const int lane = __lane_id();
  const int wave = tid >> 6;
  if (tid < kGroup) s_tok[tid] = tid < cnt ? load_token(p.rec, p.T, L.perm, it.p0 + sub * kGroup + tid) : 0;
  __syncthreads();

  // stage the group's x rows for [d0, d0 + dlen)
  {
    const int vecs_per_row = dlen / kVec;
    const Elem* xb = reinterpret_cast<const Elem*>(p.x);
    for (int e = tid; e < cnt * vecs_per_row; e += kThreads) {
      const int g = e / vecs_per_row;
      const int c = e - g * vecs_per_row;
      const Elem* src = xb + (int64_t)s_tok[g] * p.ldx + d0 + c * kVec;
      *reinterpret_cast<u32x4*>(&s_x[g][c * kVec]) = ld16(src);
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

    for (int dd = lane * kVec; dd < dlen; dd += 64 * kVec) {
      u32x4 a[kRowsPerPass];
#pragma unroll
      for (int q = 0; q < kRowsPerPass; ++q)
        a[q] = krow[q] < r ? ld16(Ab + (int64_t)krow[q] * p.D + d0 + dd) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int g = 0; g < kGroup; ++g) {
        if (g < cnt) {
          const u32x4 xv = *reinterpret_cast<const u32x4*>(&s_x[g][dd]);
#pragma unroll
          for (int q = 0; q < kRowsPerPass; ++q) acc[q * kGroup + g] = Tr::dot(a[q], xv, acc[q * kGroup + g]);
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
}

template <typename Elem>
__device__ inline void store_y4(Elem* dst, const float* acc, const Elem* src);

template <>
__device__ inline void store_y4<float>(float* dst, const float* acc, const float* src) {
  f32x4 y = *reinterpret_cast<const f32x4*>(src);
  y[0] += acc[0];
  y[1] += acc[1];
  y[2] += acc[2];
  y[3] += acc[3];
  *reinterpret_cast<f32x4*>(dst) = y;
}

template <typename Elem>
__device__ inline void store_y4(Elem* dst, const float* acc, const Elem* src) {
  using Tr = Traits<Elem>;
  const u32x2 yv = *reinterpret_cast<const u32x2*>(src);
  float y0 = Tr::elem_to_float(yv[0] & 0xffffu) + acc[0];
  float y1 = Tr::elem_to_float(yv[0] >> 16) + acc[1];
  float y2 = Tr::elem_to_float(yv[1] & 0xffffu) + acc[2];
  float y3 = Tr::elem_to_float(yv[1] >> 16) + acc[3];
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

constexpr int kColsPerLane = 4;
constexpr int kExpandCols = kThreads * kColsPerLane;  // 1024 output columns per workgroup
constexpr int kKChunk = 8;                            // rank elements per B load step

template <typename Elem>
__global__ __launch_bounds__(kThreads) void bgmv_expand_kernel(ExpandParams p, int which_list, int sub_per_item) {
  using Tr = Traits<Elem>;
  __shared__ __attribute__((aligned(16))) float s_v[kGroup][LORA_MAX_RANK];
  __shared__ int s_tok[kGroup];

  const SegLayout L = seg_layout(p.T, p.S);
  const int item_id = blockIdx.x / sub_per_item;
  Item it;
  if (!load_item(p.rec, p.T, p.S, which_list != 0, item_id, it)) return;
  const int sub = blockIdx.x - item_id * sub_per_item;
  const int cnt = min(kGroup, it.cnt - sub * kGroup);
  if (cnt <= 0) return;
  const int slice = blockIdx.y;
  const int out = (int)p.out_size[slice];
  const int j0 = blockIdx.z * kExpandCols;
  if (j0 >= out) return;
  const int s = it.slot;
  const int r = slot_rank(p.ranks, s, p.r_max);
  if (r == 0) return;

  const int tid = threadIdx.x;
  if (tid < kGroup) s_tok[tid] = tid < cnt ? load_token(p.rec, p.T, L.perm, it.p0 + sub * kGroup + tid) : 0;
  __syncthreads();
  const float* vb = p.v + (int64_t)slice * p.v_slice_stride;
  for (int e = tid; e < kGroup * LORA_MAX_RANK; e += kThreads) {
    const int g = e / LORA_MAX_RANK, k = e % LORA_MAX_RANK;
    s_v[g][k] = (g < cnt && k < r) ? vb[(int64_t)s_tok[g] * p.r_max + k] : 0.f;
  }
  __syncthreads();

  const int j = j0 + tid * kColsPerLane;
  if (j >= out) return;
  const Elem* Bb = reinterpret_cast<const Elem*>(p.B[slice]) + ((int64_t)s * out + j) * p.r_max;
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

  Elem* yb = reinterpret_cast<Elem*>(p.y) + p.out_off[slice] + j;
#pragma unroll
  for (int g = 0; g < kGroup; ++g) {
    if (g < cnt) {
      Elem* row = yb + (int64_t)s_tok[g] * p.ldy;
      store_y4<Elem>(row, acc[g], row);
    }
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
  dim3 grid((unsigned)(cap * sub), (unsigned)p.n_slices, (unsigned)nsplit);
  hipLaunchKernelGGL(bgmv_shrink_kernel<Elem>, grid, dim3(kThreads), 0, stream, p, tiles ? 1 : 0, sub, chunk,
                     nsplit > 1 ? 1 : 0);
  return hipGetLastError();
}

template <typename Elem>
hipError_t expand_launch(const ExpandParams& p, bool tiles, hipStream_t stream) {
  const SegLayout L = seg_layout(p.T, p.S);
  const int sub = tiles ? kTile / kGroup : 1;
  const int64_t cap = tiles ? L.cap_tiles : L.cap_groups;
  int64_t max_out = 0;
  for (int i = 0; i < p.n_slices; ++i) max_out = p.out_size[i] > max_out ? p.out_size[i] : max_out;
  dim3 grid((unsigned)(cap * sub), (unsigned)p.n_slices, (unsigned)ceil_div(max_out, kExpandCols));
  hipLaunchKernelGGL(bgmv_expand_kernel<Elem>, grid, dim3(kThreads), 0, stream, p, tiles ? 1 : 0, sub);
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
