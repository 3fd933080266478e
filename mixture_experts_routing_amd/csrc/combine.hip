// Top-k weighted combine: the direct slot-order gather of the b70 lab note
// "MTP1 M2 compact scheduler closure" (correctness paragraph), i.e. the
// FusedMoE "combine" step.
//
//   out[t, :] = sum_{k ascending, slot_to_row[t*K+k] >= 0} w[t,k] * y[row, :]
//
// A block covers one token and 2048 hidden elements; each thread owns 8
// consecutive elements (one 16-byte load of a bf16 row) and adds the token's
// K slots in ascending k, so the fp32 accumulation order is fixed.  Slot rows
// and weights are block-uniform and come through the scalar cache.
// HBM-bound: it reads R*H elements of y and writes T*H outputs.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

template <typename YT>
__device__ __forceinline__ void load8(const YT* p, float (&v)[8]) {
  if constexpr (sizeof(YT) == 2) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(p);
    v[0] = bf16_bits_to_f32(q.x & 0xFFFFu); v[1] = bf16_bits_to_f32(q.x >> 16);
    v[2] = bf16_bits_to_f32(q.y & 0xFFFFu); v[3] = bf16_bits_to_f32(q.y >> 16);
    v[4] = bf16_bits_to_f32(q.z & 0xFFFFu); v[5] = bf16_bits_to_f32(q.z >> 16);
    v[6] = bf16_bits_to_f32(q.w & 0xFFFFu); v[7] = bf16_bits_to_f32(q.w >> 16);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <typename OT>
__device__ __forceinline__ void store8(OT* p, const float (&v)[8]) {
  if constexpr (sizeof(OT) == 2) {
    u32x4 q;
    q.x = pack_bf16x2(v[0], v[1]); q.y = pack_bf16x2(v[2], v[3]);
    q.z = pack_bf16x2(v[4], v[5]); q.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<u32x4*>(p) = q;
  } else {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
}

template <typename YT>
__device__ __forceinline__ float load1(const YT* p) {
  if constexpr (sizeof(YT) == 2) return bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(p));
  else return *p;
}
template <typename OT>
__device__ __forceinline__ void store1(OT* p, float v) {
  if constexpr (sizeof(OT) == 2) *reinterpret_cast<uint16_t*>(p) = f32_to_bf16_bits(v);
  else *p = v;
}

// YT/OT: uint16_t (bf16 bits) or float.  Block (t, c): token t, hidden
// elements [c*kThreads*EPT, ...).  Slots are taken kSlotChunk at a time: the
// rows of the chunk are all requested before the first FMA, then added in
// ascending k, so K dependent memory round trips become one per chunk.
constexpr int kSlotChunk = 8;

template <typename YT, typename OT, bool VEC>
__global__ __launch_bounds__(kThreads) void combine_kernel(const YT* __restrict__ y, const float* __restrict__ w,
                                                          const int32_t* __restrict__ s2r, int64_t T, int K,
                                                          int H, OT* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const int32_t* rows = s2r + t * K;
  const float* wt = w + t * K;
  constexpr int EPT = VEC ? 8 : 1;  // elements per thread
  const int c = (blockIdx.y * kThreads + threadIdx.x) * EPT;
  if (c >= H) return;
  float acc[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) acc[i] = 0.0f;
  for (int k0 = 0; k0 < K; k0 += kSlotChunk) {
    int r[kSlotChunk];
    float wk[kSlotChunk], v[kSlotChunk][EPT];
#pragma unroll
    for (int j = 0; j < kSlotChunk; ++j) {
      r[j] = (k0 + j < K) ? rows[k0 + j] : -1;
      wk[j] = (k0 + j < K) ? wt[k0 + j] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kSlotChunk; ++j) {
      if (r[j] >= 0) {
        if constexpr (VEC) load8(y + (int64_t)r[j] * H + c, v[j]);
        else v[j][0] = load1(y + (int64_t)r[j] * H + c);
      }
    }
#pragma unroll
    for (int j = 0; j < kSlotChunk; ++j) {
      if (r[j] >= 0) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) acc[i] = fmaf(wk[j], v[j][i], acc[i]);
      }
    }
  }
  if constexpr (VEC) store8(out + t * H + c, acc);
  else store1(out + t * H + c, acc[0]);
}

template <typename YT, typename OT>
hipError_t launch_typed(const void* y, const float* w, const int32_t* s2r, int64_t T, int K, int H, void* out,
                        hipStream_t stream) {
  const YT* yp = static_cast<const YT*>(y);
  OT* op = static_cast<OT*>(out);
  const bool vec = (H % 8 == 0) && ((uintptr_t)y % 16 == 0) && ((uintptr_t)out % 16 == 0);
  const int per_block = kThreads * (vec ? 8 : 1);
  const dim3 grid((unsigned)T, (unsigned)((H + per_block - 1) / per_block));
  if (vec)
    hipLaunchKernelGGL((combine_kernel<YT, OT, true>), grid, dim3(kThreads), 0, stream, yp, w, s2r, T, K, H, op);
  else
    hipLaunchKernelGGL((combine_kernel<YT, OT, false>), grid, dim3(kThreads), 0, stream, yp, w, s2r, T, K, H, op);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const void* y, int y_dtype, const float* w, const int32_t* s2r, int64_t T, int K, int H,
                          void* out, int out_dtype, hipStream_t stream) {
  if (y_dtype == MOE_BF16 && out_dtype == MOE_BF16) return launch_typed<uint16_t, uint16_t>(y, w, s2r, T, K, H, out, stream);
  if (y_dtype == MOE_BF16 && out_dtype == MOE_F32) return launch_typed<uint16_t, float>(y, w, s2r, T, K, H, out, stream);
  if (y_dtype == MOE_F32 && out_dtype == MOE_BF16) return launch_typed<float, uint16_t>(y, w, s2r, T, K, H, out, stream);
  return launch_typed<float, float>(y, w, s2r, T, K, H, out, stream);
}

}  // namespace moe
