// Gather path (BGMV) expand on the vector ALUs, used for fp32 data (and, on
// request, for the gather groups of 16-bit data).  A work item is a group of at
// most 16 tokens that share one adapter slot.  The gather semantics are those of
// the baseline in "[Hardware][TPU][V1] Better tpu multilora compilation" (review
// thread): a token multiplies the stacked matrix of its own slot.  Instead of
// materialising a per-token copy of the weights (the index_select that the same
// thread names as the slow part), a workgroup reads its slot's rows once for the
// whole group, with 16-byte coalesced loads.
//
// A workgroup owns (group, slice, column tile).  The group's v rows are staged
// in LDS (rank columns past the slot's rank read as 0); each lane owns 4
// consecutive output columns, forms the fp32 dot products over the rank with
// the slot's B rows, then read-modify-writes y with one rounding per element.
#include "common.h"

namespace lora {

namespace {

constexpr int kThreads = 256;
constexpr int kColsPerLane = 4;
constexpr int kExpandCols = kThreads * kColsPerLane;  // 1024 output columns per workgroup
constexpr int kKChunk = 8;                            // rank elements per B load step

__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

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
      o[0] = pack2_bf16(y0, y1);
      o[1] = pack2_bf16(y2, y3);
    } else {
      o[0] = pack2_f16(y0, y1);
      o[1] = pack2_f16(y2, y3);
    }
    *reinterpret_cast<u32x2*>(dst) = o;
  }
}


template <typename Elem>
__global__ __launch_bounds__(kThreads) void bgmv_expand_kernel(ExpandParams p, int use_tiles, int n_ct) {
  warm_args(p);
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
  const int ldb = b_row_stride(p, r);
  const Elem* Bb = reinterpret_cast<const Elem*>(p.B[slice]) + (int64_t)s * out * p.r_max + (int64_t)j * ldb;
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
      const Elem* row = Bb + (int64_t)c * ldb + k0;
      if constexpr (sizeof(Elem) == 4) {
        // 8 fp32 values = two 16-byte loads; r_max is a multiple of 4
        u32x4 lo = ld16(row);
        u32x4 hi = (k0 + 4 < ldb) ? ld16(row + 4) : u32x4{0, 0, 0, 0};
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

hipError_t launch_bgmv_expand(lora_dtype dt, const ExpandParams& p, bool tiles, hipStream_t stream) {
  switch (dt) {
    case LORA_F32: return expand_launch<float>(p, tiles, stream);
    case LORA_F16: return expand_launch<half_t>(p, tiles, stream);
    case LORA_BF16: return expand_launch<bf16_t>(p, tiles, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace lora
