// Shrink of a LoRA on an embedding table ("Add multi-LoRA support",
// Features: adapters cover every linear layer and the embeddings, in PEFT
// format).  The layer's input for token id w is the one-hot vector e_w, so
// the shrink A_s e_w is one column of the adapter's A table; the tables are
// stacked transposed, A_emb [S][V][r_max], so that the column is one
// contiguous rank vector:
//   v[t][k] = scale[s] * A_emb[s][tok[t]][k]      (k < r_s; 0 otherwise)
// The expand that follows is the linear layers' expand (lora_expand).  Each
// token is one 16-lane group: lane q converts ranks 4q .. 4q + 3 to fp32 and
// stores them, so v is written in full (zero rows for tokens without a valid
// slot or with an id outside [0, V)).
#include "common.h"

namespace lora {

namespace {

struct EmbParams {
  const int32_t* tok;
  const int32_t* idx;
  const void* A;
  const int32_t* ranks;  // nullable
  const float* scale;    // nullable
  float* v;
  int64_t V;
  int32_t T, S, r_max;
};

template <typename Elem>
__global__ __launch_bounds__(256) void embedding_shrink_kernel(EmbParams p) {
  warm_args(p);
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t = g >> 4;
  const int k0 = (int)(g & 15) * 4;
  if (t >= p.T || k0 >= p.r_max) return;
  const int s = p.idx[t];
  const int64_t w = p.tok[t];
  f32x4 out = f32x4{0.f, 0.f, 0.f, 0.f};
  if (s >= 0 && s < p.S && w >= 0 && w < p.V) {
    const int r = slot_rank(p.ranks, s, p.r_max);
    const float sc = p.scale ? p.scale[s] : 1.0f;
    const Elem* row = reinterpret_cast<const Elem*>(p.A) + ((int64_t)s * p.V + w) * p.r_max + k0;
    float a[4];
    if constexpr (sizeof(Elem) == 4) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(row);
      a[0] = q[0];
      a[1] = q[1];
      a[2] = q[2];
      a[3] = q[3];
    } else {
      const u32x2 q = *reinterpret_cast<const u32x2*>(row);
      const uint32_t lo = q[0], hi = q[1];
      a[0] = Traits<Elem>::elem_to_float(lo & 0xffffu);
      a[1] = Traits<Elem>::elem_to_float(lo >> 16);
      a[2] = Traits<Elem>::elem_to_float(hi & 0xffffu);
      a[3] = Traits<Elem>::elem_to_float(hi >> 16);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = k0 + i < r ? a[i] * sc : 0.f;
  }
  *reinterpret_cast<f32x4*>(p.v + t * p.r_max + k0) = out;
}

template <typename Elem>
hipError_t launch(const EmbParams& p, hipStream_t stream) {
  const int64_t threads = (int64_t)p.T * 16;
  const unsigned blocks = (unsigned)ceil_div(threads, 256);
  hipLaunchKernelGGL(embedding_shrink_kernel<Elem>, dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_embedding_shrink(lora_dtype dt, const int32_t* tok, const int32_t* idx, int32_t T, int64_t V,
                                   const void* A_emb, int32_t S, int32_t r_max, const int32_t* ranks,
                                   const float* scale, float* v, hipStream_t stream) {
  const EmbParams p{tok, idx, A_emb, ranks, scale, v, V, T, S, r_max};
  switch (dt) {
    case LORA_F32: return launch<float>(p, stream);
    case LORA_F16: return launch<half_t>(p, stream);
    case LORA_BF16: return launch<bf16_t>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace lora
