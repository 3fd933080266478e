// Expert-grouped SwiGLU FFN: expand -> GEMM1 -> silu_and_mul -> GEMM2.
//
// Sources: page "Upstream Reference: Deep-Spark xllm + vllm", section "File
// Index" (FusedMoE: expand -> gemm1 -> act -> gemm2, with silu_and_mul), and
// the b70 lab note "MTP1 M2 compact scheduler closure", design paragraph
// (expert-grouped activation layout, cross-row weight reuse, tiles derived on
// device from per-expert row counts, no host round trip).
//
// Work decomposition.  The grouped layout puts the R local rows expert by
// expert; expert e owns rows [offsets[e], offsets[e+1]).  An M-tile is BM
// consecutive rows of one expert; tile i is found on device from counts (a
// wave prefix over ceil(count/BM)), so the grid is sized by the host-known
// bound ceil(N/BM) + min(E_local, N) and surplus blocks exit at once.
//
// Streaming kernels (this file): every wavefront owns 16 output columns of one
// M-tile and walks the whole reduction dimension, reading each weight row of
// its 16 columns exactly once per M-tile and feeding 16x16x32 bf16 MFMAs for
// every 16-row block of the tile (cross-row reuse: one weight pass serves up
// to BM rows).  A and B fragments come straight from global memory in the
// MFMA lane layout (lane l: row/column l%16, a 32-element slice of each
// 128-wide K step chosen by l/16), so every weight row is read as 256
// contiguous bytes per step.  The gather of x rows (expand) happens in the A
// load; silu_and_mul runs in the GEMM1 epilogue on the two accumulators of a
// gate column and its up column.  MXFP4 weights are widened to bf16 in
// registers with v_cvt_scalef32_pk_bf16_fp4 (exact: every e2m1 value times a
// power-of-two scale in range is a bf16 value).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;  // 4 wavefronts
constexpr int kWaves = kThreads / 64;

// Tile i of height BM: expert e, first grouped row and number of valid rows.
// Wave-uniform; every lane of the wave must call it.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
                                          int El, int BM, int i, int& e, int& row0, int& nrows) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int c0 = 0; c0 < El; c0 += 64) {
    const int ee = c0 + lane;
    const int cnt = ee < El ? counts[ee] : 0;
    const int nt = (cnt + BM - 1) / BM;
    int inc = nt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(inc, d, 64);
      if (lane >= d) inc += o;
    }
    const int excl = inc - nt;
    const bool own = (i >= base + excl) && (i < base + inc);
    const unsigned long long m = __ballot(own);
    if (m) {
      const int src = __ffsll((long long)m) - 1;
      e = c0 + src;
      const int tile_in_e = i - base - __shfl(excl, src, 64);
      const int ce = __shfl(cnt, src, 64);
      row0 = offsets[e] + tile_in_e * BM;
      nrows = min(BM, ce - tile_in_e * BM);
      return true;
    }
    base += __shfl(inc, 63, 64);
  }
  return false;
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

// One lane's KS/4-element slice of a bf16 row, as KS/32 MFMA operands.
template <int KS>
__device__ __forceinline__ void load_bf16_slice(const uint16_t* __restrict__ p, bf16x8 (&v)[KS / 32]) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int j = 0; j < KS / 32; ++j) v[j] = __builtin_bit_cast(bf16x8, q[j]);
}

// MXFP4 slice of KS/4 elements (KS/8 bytes of codes, one e8m0 scale per 32
// elements) widened to bf16.
template <int KS>
__device__ __forceinline__ void load_mx_slice(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                              bf16x8 (&v)[KS / 32]) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  constexpr int NB = KS / 8;  // code bytes of this lane's slice
  uint32_t c[(NB + 3) / 4];
  if constexpr (NB == 16) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(codes);
    c[0] = q.x; c[1] = q.y; c[2] = q.z; c[3] = q.w;
  } else {
    c[0] = *reinterpret_cast<const uint32_t*>(codes);
  }
  // the slice never straddles a 32-element scale block: KS/4 is 32 or 8
  const uint32_t e8 = scales[0];
  const float s = e8 == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(e8 << 23);
#pragma unroll
  for (int j = 0; j < KS / 32; ++j) {
    const uint32_t w = c[j];
    bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
    bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
    bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
    bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
    v[j] = bf16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
  }
}

template <int KS, bool MX>
__device__ __forceinline__ void load_w_slice(const void* __restrict__ w, const uint8_t* __restrict__ ws,
                                             int64_t row, int64_t kdim, int k, bf16x8 (&v)[KS / 32]) {
  if constexpr (MX) {
    load_mx_slice<KS>(static_cast<const uint8_t*>(w) + row * (kdim / 2) + k / 2, ws + row * (kdim / 32) + k / 32, v);
  } else {
    load_bf16_slice<KS>(static_cast<const uint16_t*>(w) + row * kdim + k, v);
  }
}

// GEMM1 + silu_and_mul.  x [T,H] bf16; w1 [El, 2F, H] (bf16 or MXFP4);
// act [N, F] bf16 (grouped rows).  KS: K step (128, or 32 when H % 128 != 0).
template <int MB, int KS, bool MX>
__global__ __launch_bounds__(kThreads) void ffn1_stream_kernel(
    const uint16_t* __restrict__ x, int K, int H, int F, int El, const void* __restrict__ w1,
    const uint8_t* __restrict__ w1s, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ r2s, uint16_t* __restrict__ act) {
  constexpr int BM = 16 * MB;
  int e, row0, nrows;
  if (!find_tile(counts, offsets, El, BM, blockIdx.x, e, row0, nrows)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = (blockIdx.y * kWaves + wave) * 16;
  if (n0 >= F) return;
  const int kq = (lane >> 4) * (KS / 4);

  const uint16_t* xrow[MB];
  bool valid[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = mb * 16 + (lane & 15);
    valid[mb] = m < nrows;
    const int tok = valid[mb] ? r2s[row0 + m] / K : 0;
    xrow[mb] = x + (int64_t)tok * H;
  }
  const int64_t wrow_g = (int64_t)e * 2 * F + n0 + (lane & 15);
  const int64_t wrow_u = wrow_g + F;

  f32x4 acc_g[MB], acc_u[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) { acc_g[mb] = f32x4{0, 0, 0, 0}; acc_u[mb] = f32x4{0, 0, 0, 0}; }

  for (int k0 = 0; k0 < H; k0 += KS) {
    bf16x8 bg[KS / 32], bu[KS / 32];
    load_w_slice<KS, MX>(w1, w1s, wrow_g, H, k0 + kq, bg);
    load_w_slice<KS, MX>(w1, w1s, wrow_u, H, k0 + kq, bu);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      bf16x8 a[KS / 32];
      if (valid[mb]) {
        load_bf16_slice<KS>(xrow[mb] + k0 + kq, a);
      } else {
#pragma unroll
        for (int j = 0; j < KS / 32; ++j) a[j] = bf16x8{};
      }
#pragma unroll
      for (int j = 0; j < KS / 32; ++j) {
        acc_g[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], bg[j], acc_g[mb], 0, 0, 0);
        acc_u[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], bu[j], acc_u[mb], 0, 0, 0);
      }
    }
  }

  // lane holds D[(lane/16)*4 + i][lane%16]
  const int n = n0 + (lane & 15);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mb * 16 + (lane >> 4) * 4 + i;
      if (m < nrows) {
        const float a = silu_f32(acc_g[mb][i]) * acc_u[mb][i];
        act[(int64_t)(row0 + m) * F + n] = f32_to_bf16_bits(a);
      }
    }
  }
}

// GEMM2.  act [N, F] bf16; w2 [El, H, F]; y [N, H] (bf16 bits or f32).
template <int MB, int KS, bool MX, typename YT>
__global__ __launch_bounds__(kThreads) void ffn2_stream_kernel(
    const uint16_t* __restrict__ act, int H, int F, int El, const void* __restrict__ w2,
    const uint8_t* __restrict__ w2s, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    YT* __restrict__ y) {
  constexpr int BM = 16 * MB;
  int e, row0, nrows;
  if (!find_tile(counts, offsets, El, BM, blockIdx.x, e, row0, nrows)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = (blockIdx.y * kWaves + wave) * 16;
  if (n0 >= H) return;
  const int kq = (lane >> 4) * (KS / 4);

  const uint16_t* arow[MB];
  bool valid[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = mb * 16 + (lane & 15);
    valid[mb] = m < nrows;
    arow[mb] = act + (int64_t)(row0 + (valid[mb] ? m : 0)) * F;
  }
  const int64_t wrow = (int64_t)e * H + n0 + (lane & 15);

  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0, 0, 0, 0};

  for (int k0 = 0; k0 < F; k0 += KS) {
    bf16x8 b[KS / 32];
    load_w_slice<KS, MX>(w2, w2s, wrow, F, k0 + kq, b);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      bf16x8 a[KS / 32];
      if (valid[mb]) {
        load_bf16_slice<KS>(arow[mb] + k0 + kq, a);
      } else {
#pragma unroll
        for (int j = 0; j < KS / 32; ++j) a[j] = bf16x8{};
      }
#pragma unroll
      for (int j = 0; j < KS / 32; ++j) acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], b[j], acc[mb], 0, 0, 0);
    }
  }

  const int n = n0 + (lane & 15);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mb * 16 + (lane >> 4) * 4 + i;
      if (m < nrows) {
        if constexpr (sizeof(YT) == 2) y[(int64_t)(row0 + m) * H + n] = f32_to_bf16_bits(acc[mb][i]);
        else y[(int64_t)(row0 + m) * H + n] = acc[mb][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 weights (small problems): one thread per output element, VALU FMAs.

__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ offsets, int El, int r) {
  int lo = 0, hi = El;  // offsets[lo] <= r < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(kThreads) void ffn1_f32_kernel(const float* __restrict__ x, int K, int H, int F, int El,
                                                           const float* __restrict__ w1,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ r2s, float* __restrict__ act) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int r = (int)(idx / F), n = (int)(idx % F);
  if (r >= offsets[El]) return;
  const int e = expert_of_row(offsets, El, r);
  const float* xr = x + (int64_t)(r2s[r] / K) * H;
  const float* wg = w1 + ((int64_t)e * 2 * F + n) * H;
  const float* wu = wg + (int64_t)F * H;
  float g = 0.0f, u = 0.0f;
  for (int k = 0; k < H; ++k) {
    g = fmaf(xr[k], wg[k], g);
    u = fmaf(xr[k], wu[k], u);
  }
  act[(int64_t)r * F + n] = silu_f32(g) * u;
}

template <typename YT>
__global__ __launch_bounds__(kThreads) void ffn2_f32_kernel(const float* __restrict__ act, int H, int F, int El,
                                                           const float* __restrict__ w2,
                                                           const int32_t* __restrict__ offsets, YT* __restrict__ y) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int r = (int)(idx / H), n = (int)(idx % H);
  if (r >= offsets[El]) return;
  const int e = expert_of_row(offsets, El, r);
  const float* ar = act + (int64_t)r * F;
  const float* wr = w2 + ((int64_t)e * H + n) * F;
  float s = 0.0f;
  for (int f = 0; f < F; ++f) s = fmaf(ar[f], wr[f], s);
  if constexpr (sizeof(YT) == 2) y[(int64_t)r * H + n] = f32_to_bf16_bits(s);
  else y[(int64_t)r * H + n] = s;
}

template <int MB, int KS, bool MX>
hipError_t launch_stream(const uint16_t* x, int64_t N, int K, int H, int F, int El, const void* w1, const uint8_t* w1s,
                         const void* w2, const uint8_t* w2s, const int32_t* counts, const int32_t* offsets,
                         const int32_t* r2s, void* y, int y_dtype, uint16_t* act, hipStream_t stream) {
  constexpr int BM = 16 * MB;
  const int64_t mtiles = (N + BM - 1) / BM + (N < El ? N : (int64_t)El);
  const dim3 g1((unsigned)mtiles, (unsigned)((F + 16 * kWaves - 1) / (16 * kWaves)));
  hipLaunchKernelGGL((ffn1_stream_kernel<MB, KS, MX>), g1, dim3(kThreads), 0, stream, x, K, H, F, El, w1, w1s, counts,
                     offsets, r2s, act);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 g2((unsigned)mtiles, (unsigned)((H + 16 * kWaves - 1) / (16 * kWaves)));
  if (y_dtype == MOE_BF16)
    hipLaunchKernelGGL((ffn2_stream_kernel<MB, KS, MX, uint16_t>), g2, dim3(kThreads), 0, stream, act, H, F, El, w2,
                       w2s, counts, offsets, static_cast<uint16_t*>(y));
  else
    hipLaunchKernelGGL((ffn2_stream_kernel<MB, KS, MX, float>), g2, dim3(kThreads), 0, stream, act, H, F, El, w2, w2s,
                       counts, offsets, static_cast<float*>(y));
  return hipGetLastError();
}

template <bool MX>
hipError_t dispatch_stream(const uint16_t* x, int64_t N, int K, int H, int F, int El, const void* w1,
                           const uint8_t* w1s, const void* w2, const uint8_t* w2s, const int32_t* counts,
                           const int32_t* offsets, const int32_t* r2s, void* y, int y_dtype, uint16_t* act,
                           hipStream_t stream) {
  // rows per expert on average decides how many 16-row blocks share a weight pass
  const int64_t avg = N / (El > 0 ? El : 1);
  const bool k128 = (H % 128 == 0) && (F % 128 == 0);
#define MOE_FFN_CASE(MBV)                                                                                        \
  return k128 ? launch_stream<MBV, 128, MX>(x, N, K, H, F, El, w1, w1s, w2, w2s, counts, offsets, r2s, y, y_dtype, \
                                            act, stream)                                                         \
              : launch_stream<MBV, 32, MX>(x, N, K, H, F, El, w1, w1s, w2, w2s, counts, offsets, r2s, y, y_dtype,  \
                                           act, stream)
  if (avg >= 48) MOE_FFN_CASE(4);
  if (avg >= 24) MOE_FFN_CASE(2);
  MOE_FFN_CASE(1);
#undef MOE_FFN_CASE
}

}  // namespace

size_t grouped_ffn_workspace_bytes(int64_t N, int F, int w_dtype) {
  const size_t elt = (w_dtype == MOE_F32) ? sizeof(float) : sizeof(uint16_t);
  return (size_t)N * (size_t)F * elt;
}

hipError_t launch_grouped_ffn(const void* x, int x_dtype, int64_t T, int K, int H, int F, int El, const void* w1,
                              const uint8_t* w1s, const void* w2, const uint8_t* w2s, int w_dtype,
                              const int32_t* counts, const int32_t* offsets, const int32_t* r2s, void* y,
                              int y_dtype, void* workspace, hipStream_t stream) {
  const int64_t N = T * K;
  if (w_dtype == MOE_F32) {
    float* act = static_cast<float*>(workspace);
    const dim3 g1((unsigned)((N * F + kThreads - 1) / kThreads));
    hipLaunchKernelGGL(ffn1_f32_kernel, g1, dim3(kThreads), 0, stream, static_cast<const float*>(x), K, H, F, El,
                       static_cast<const float*>(w1), offsets, r2s, act);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const dim3 g2((unsigned)((N * H + kThreads - 1) / kThreads));
    if (y_dtype == MOE_BF16)
      hipLaunchKernelGGL((ffn2_f32_kernel<uint16_t>), g2, dim3(kThreads), 0, stream, act, H, F, El,
                         static_cast<const float*>(w2), offsets, static_cast<uint16_t*>(y));
    else
      hipLaunchKernelGGL((ffn2_f32_kernel<float>), g2, dim3(kThreads), 0, stream, act, H, F, El,
                         static_cast<const float*>(w2), offsets, static_cast<float*>(y));
    return hipGetLastError();
  }
  uint16_t* act = static_cast<uint16_t*>(workspace);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (w_dtype == MOE_BF16 && tiled_ffn_applicable(N, H, F, El))
    return launch_tiled_ffn(xb, T, N, K, H, F, El, static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w2),
                            counts, offsets, r2s, y, y_dtype, act, stream);
  if (w_dtype == MOE_MXFP4)
    return dispatch_stream<true>(xb, N, K, H, F, El, w1, w1s, w2, w2s, counts, offsets, r2s, y, y_dtype, act, stream);
  return dispatch_stream<false>(xb, N, K, H, F, El, w1, nullptr, w2, nullptr, counts, offsets, r2s, y, y_dtype, act,
                                stream);
}

}  // namespace moe
