// Measurement probes: kernels of a known access pattern or instruction mix
// that measure what the chip achieves, next to the spec peaks the roofline
// uses (HBM bandwidth, bf16 matrix-core rate) and next to the gate kernel's
// own access pattern.  None of them is a step of the layer.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocks = 4096;  // 16 blocks per compute unit
constexpr int kProbeUnroll = 4;

// Streaming read: every 16-byte piece of src once (non-temporal loads,
// kProbeUnroll pieces in flight per thread); each thread folds what it read
// into one word, written to out[thread] so that no load is dead.
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4* __restrict__ src, int64_t n,
                                                                   uint32_t* __restrict__ out) {
  const int64_t tid = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  uint32_t acc = 0;
  int64_t i = tid;
  for (; i + (kProbeUnroll - 1) * stride < n; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[tid] = acc;
}

// Copy: every 16-byte piece of src to dst.
__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                                   int64_t n) {
  const int64_t tid = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = tid;
  for (; i + (kProbeUnroll - 1) * stride < n; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// bf16 matrix-core loop: every wave issues iters rounds of four independent
// v_mfma_f32_32x32x16_bf16 (4 x 32768 flops per round) on register operands;
// the accumulators are summed into out[thread].  TOGGLE: the operands start
// from hashed bf16 values in [0.5, 2) with random signs, and every round
// flips the sign and the 7 mantissa bits of each element (so half the
// operand bits change from one MFMA to the next, as with real data; the
// exponents stay, so every value stays finite); otherwise the operands are
// loop-invariant small constants.  clk (if not null) receives per wave the
// shader-clock cycles (s_memtime) and the 100 MHz reference-clock ticks
// (s_memrealtime) the loop took: clk[2w], clk[2w+1].
template <bool TOGGLE>
__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(int64_t iters, float* __restrict__ out,
                                                                   unsigned long long* __restrict__ clk) {
  const int lane = threadIdx.x & 63;
  const int64_t tid = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4 ua, ub;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (TOGGLE) {
      const uint32_t h = ((uint32_t)tid * 4u + (uint32_t)i) * 2654435761u;
      const uint32_t h2 = h * 2246822519u + 3266489917u;
      // two bf16 per word: exponent of 0.5 or 1 (0x3F00 | mantissa), sign from the hash
      ua[i] = ((0x3F00u | ((h >> 17) & 0xFFu)) << 16 | (0x3F00u | ((h >> 9) & 0xFFu))) ^ (h & 0x80008000u);
      ub[i] = ((0x3F00u | ((h2 >> 17) & 0xFFu)) << 16 | (0x3F00u | ((h2 >> 9) & 0xFFu))) ^ (h2 & 0x80008000u);
    } else {
      ua[i] = pack_bf16x2(0.001f * (float)((lane + 2 * i) & 7), 0.001f * (float)((lane + 2 * i + 1) & 7));
      ub[i] = pack_bf16x2(0.002f * (float)((lane * 3 + 2 * i) & 7), 0.002f * (float)((lane * 3 + 2 * i + 1) & 7));
    }
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t it = 0; it < iters; ++it) {
    if constexpr (TOGGLE) {
      ua ^= (u32x4){0x807F807Fu, 0x807F807Fu, 0x807F807Fu, 0x807F807Fu};
      ub ^= (u32x4){0x807F807Fu, 0x807F807Fu, 0x807F807Fu, 0x807F807Fu};
    }
    const bf16x8 a = __builtin_bit_cast(bf16x8, ua), b = __builtin_bit_cast(bf16x8, ub);
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[tid] = s;
  if (clk && lane == 0) {
    const int64_t w = tid >> 6;
    clk[2 * w] = t1 - t0;
    clk[2 * w + 1] = r1 - r0;
  }
}

// The bf16 gate's memory traffic without its selection: the same grid (8
// lanes per row, 32 rows per 256-thread block), the same per-lane
// non-temporal loads of the row's logits, and the same K stores of weight,
// id and token-expert index per row, fed by a fold of the loaded words.
template <int V>
__global__ __launch_bounds__(kProbeThreads) void probe_gate_loads_kernel(const uint16_t* __restrict__ logits,
                                                                         int64_t T, int K, float* __restrict__ w_out,
                                                                         int32_t* __restrict__ id_out,
                                                                         int32_t* __restrict__ tei_out) {
  constexpr int E = 8 * V, W = V / 2;
  const int64_t t = (int64_t)blockIdx.x * (kProbeThreads / 8) + (threadIdx.x >> 3);
  const int q = threadIdx.x & 7;
  if (t >= T) return;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(logits + t * E + q * V);
  uint32_t acc = 0;
  if constexpr (V % 8 == 0) {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + i);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < W / 2; ++i) {
      const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src) + i);
      acc ^= v.x ^ v.y;
    }
  }
  acc = (uint32_t)group_max_i32<8>((int)acc);
  if (q < K) {
    const int64_t o = t * K + q;
    w_out[o] = __uint_as_float(acc & 0x3FFFFFFFu);
    id_out[o] = (int32_t)(acc & 0xFF);
    if (tei_out) tei_out[o] = (int32_t)((int64_t)q * T + t);
  }
}

}  // namespace

hipError_t launch_probe_read(const void* src, int64_t bytes, uint32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(probe_read_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, out);
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  hipLaunchKernelGGL(probe_copy_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int64_t iters, int blocks, bool toggle, float* out, unsigned long long* clk,
                             hipStream_t stream) {
  if (toggle)
    hipLaunchKernelGGL(probe_mfma_kernel<true>, dim3((unsigned)blocks), dim3(kProbeThreads), 0, stream, iters, out, clk);
  else
    hipLaunchKernelGGL(probe_mfma_kernel<false>, dim3((unsigned)blocks), dim3(kProbeThreads), 0, stream, iters, out, clk);
  return hipGetLastError();
}

hipError_t launch_probe_gate_loads(const uint16_t* logits, int64_t T, int E, int K, float* w, int32_t* ids,
                                   int32_t* tei, hipStream_t stream) {
  const dim3 grid((unsigned)((T + kProbeThreads / 8 - 1) / (kProbeThreads / 8)));
  switch (E / 8) {
    case 8: hipLaunchKernelGGL((probe_gate_loads_kernel<8>), grid, dim3(kProbeThreads), 0, stream, logits, T, K, w, ids, tei); break;
    case 12: hipLaunchKernelGGL((probe_gate_loads_kernel<12>), grid, dim3(kProbeThreads), 0, stream, logits, T, K, w, ids, tei); break;
    case 16: hipLaunchKernelGGL((probe_gate_loads_kernel<16>), grid, dim3(kProbeThreads), 0, stream, logits, T, K, w, ids, tei); break;
    case 20: hipLaunchKernelGGL((probe_gate_loads_kernel<20>), grid, dim3(kProbeThreads), 0, stream, logits, T, K, w, ids, tei); break;
    default: hipLaunchKernelGGL((probe_gate_loads_kernel<24>), grid, dim3(kProbeThreads), 0, stream, logits, T, K, w, ids, tei); break;
  }
  return hipGetLastError();
}

int probe_read_out_words() { return kProbeBlocks * kProbeThreads; }

}  // namespace moe
