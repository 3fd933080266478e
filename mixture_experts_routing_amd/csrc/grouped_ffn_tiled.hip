// LDS-tiled expert GEMMs for many rows per expert (prefill sizes).
//
// Same contract as the streaming kernels of grouped_ffn.hip (the
// expand -> gemm1 -> silu_and_mul -> gemm2 order of the FusedMoE pipeline on
// the "Upstream Reference: Deep-Spark xllm + vllm" page, "File Index"; the
// expert-grouped layout and cross-row weight reuse of the b70 lab note "MTP1
// M2 compact scheduler closure", design paragraph), tiled for MFMA
// throughput instead of pure weight streaming:
//
//   block tile   BM rows of one expert x 128 weight rows, K step 64, 4 waves
//                in a 2 x 2 grid; each wave owns (BM/2) x 64 and issues
//                v_mfma_f32_32x32x16_bf16 on (BM/64) x 2 accumulator tiles
//   LDS          double-buffered A and B tiles, rows padded by 16 bytes so the
//                16-byte fragment reads of 8 consecutive lanes hit distinct
//                banks; one barrier per K step; global loads of step k+1 are
//                in flight while step k runs on the matrix cores
//   GEMM1        A rows are gathered from x through row_to_slot (expand), the
//                128 weight rows are 64 gate rows and the matching 64 up rows
//                interleaved in 32-row groups, so each lane holds a gate value
//                and its up value and silu(g)*u is formed in registers
//   GEMM2        A rows are act rows; 128 output columns per block
//   rows         32-row MFMA blocks past the tile's last valid row are skipped
//
// One expert's whole row set usually fits one M-tile (BM = 320 >= the
// typical 256 +- 3 sigma rows at top-8 of 128), so each (expert, N-tile)
// weight panel is read from HBM once.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTThreads = 256;
constexpr int kBK = 64;
constexpr int kLds = kBK + 8;  // bf16 elements per LDS row: 128 B of data + 16 B pad
constexpr int kBN = 128;

__device__ __forceinline__ bool find_tile_t(const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
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
    const unsigned long long m = __ballot((i >= base + excl) && (i < base + inc));
    if (m) {
      const int src = __ffsll((long long)m) - 1;
      e = c0 + src;
      const int tile_in_e = i - base - __shfl(excl, src, 64);
      row0 = offsets[e] + tile_in_e * BM;
      nrows = min(BM, __shfl(cnt, src, 64) - tile_in_e * BM);
      return true;
    }
    base += __shfl(inc, 63, 64);
  }
  return false;
}


// Per-thread global->LDS chunk assignment: chunk i of a tile covers tile row
// (tid >> 3) + 32 * i and the 16-byte column (tid & 7) of the 128-byte K step.
template <int MBW>
struct Stage {
  u32x4 a[2 * MBW];
  u32x4 b[4];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw (unstructured) buffer: stride 0, byte-addressed, range-checked
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// The K loop of one block.  LDS holds two K steps (double buffer, one barrier
// per step); registers hold two more, so the global loads of step k+2 are
// issued while step k runs on the matrix cores and step k+1 is in flight.
// Loads are buffer loads: the lane's row offset is a per-lane byte offset
// fixed for the whole loop, the K position a scalar offset.
// Wave (wm, wn) owns the 32-row blocks b = 2*mb + wm (interleaved, so both
// wave rows get the same share of a ragged tile) and 64 weight rows of B.
// LIVE: blocks of this wave holding valid rows; the others issue no MFMAs.
template <int MBW, int LIVE>
__device__ __forceinline__ void kloop(__amdgpu_buffer_rsrc_t ra_rsrc, const uint32_t (&a_off)[2 * MBW],
                                      __amdgpu_buffer_rsrc_t rb_rsrc, const uint32_t (&b_off)[4],
                                      uint16_t (&As)[2][64 * MBW * kLds], uint16_t (&Bs)[2][kBN * kLds],
                                      f32x16 (&acc)[MBW][2], int K, int nrows, int tid, int lane, int wm, int wn) {
  constexpr int A_CH = 2 * MBW, B_CH = 4;
  const int kc = tid & 7;
  auto gload = [&](Stage<MBW>& st, int k0) {
    const int sk = k0 * 2;  // bytes
#pragma unroll
    for (int i = 0; i < A_CH; ++i) st.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ra_rsrc, a_off[i], sk, 0);
#pragma unroll
    for (int i = 0; i < B_CH; ++i) st.b[i] = __builtin_amdgcn_raw_buffer_load_b128(rb_rsrc, b_off[i], sk, 0);
  };
  auto lstore = [&](const Stage<MBW>& st, int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i)
      *reinterpret_cast<u32x4*>(&As[buf][((tid >> 3) + 32 * i) * kLds + kc * 8]) = st.a[i];
#pragma unroll
    for (int i = 0; i < B_CH; ++i)
      *reinterpret_cast<u32x4*>(&Bs[buf][((tid >> 3) + 32 * i) * kLds + kc * 8]) = st.b[i];
  };
  auto compute = [&](int buf) {
    const uint16_t* as = &As[buf][(wm * 32 + (lane & 31)) * kLds + (lane >> 5) * 8];
    const uint16_t* bs = &Bs[buf][(wn * 64 + (lane & 31)) * kLds + (lane >> 5) * 8];
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(bs + ks * 16);
      const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(bs + 32 * kLds + ks * 16);
      bf16x8 a[LIVE > 0 ? LIVE : 1];
#pragma unroll
      for (int mb = 0; mb < LIVE; ++mb) a[mb] = *reinterpret_cast<const bf16x8*>(as + mb * 64 * kLds + ks * 16);
#pragma unroll
      for (int mb = 0; mb < LIVE; ++mb) {
        acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], b0, acc[mb][0], 0, 0, 0);
        acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], b1, acc[mb][1], 0, 0, 0);
      }
    }
  };
  const int KT = K / kBK;
  Stage<MBW> s0, s1;
  // Every load in the steady state is unconditional so that the compiler's
  // vmcnt waits before each LDS store release only the older stage: step k+2
  // stays in flight while step k computes.  (A load count that differs
  // between control paths makes the wait pass fall back to waiting for the
  // newest loads too.)
  gload(s0, 0);
  gload(s1, (KT > 1 ? 1 : 0) * kBK);
  lstore(s0, 0);
  __syncthreads();
  // top of each pair: LDS[0] holds step kt, s1 holds step kt+1 (in flight)
  int kt = 0;
  for (; kt + 3 < KT; kt += 2) {
    gload(s0, (kt + 2) * kBK);
    compute(0);
    lstore(s1, 1);
    __syncthreads();
    gload(s1, (kt + 3) * kBK);
    compute(1);
    lstore(s0, 0);
    __syncthreads();
  }
  const int left = KT - kt;  // 1, 2 or 3 steps
  if (left == 3) {
    gload(s0, (kt + 2) * kBK);
    compute(0);
    lstore(s1, 1);
    __syncthreads();
    compute(1);
    lstore(s0, 0);
    __syncthreads();
    compute(0);
  } else if (left == 2) {
    compute(0);
    lstore(s1, 1);
    __syncthreads();
    compute(1);
  } else {
    compute(0);
  }
}

// Block -> (M-tile, N-tile).  Workgroups are dispatched to the 8 XCDs round
// robin (linear id % 8).  M-tiles are dealt to XCDs round robin too, and on
// each XCD consecutive blocks walk the N-tiles of one M-tile, so the blocks
// that share an A tile (the expert's gathered rows) run together on one XCD
// and find it in that XCD's L2; every weight panel is still read by exactly
// one block.
__device__ __forceinline__ void xcd_map(int L, int NT, int& mt, int& nt) {
  const int xcd = L & 7, local = L >> 3;
  mt = xcd + 8 * (local / NT);
  nt = local % NT;
}

// GATED = true : GEMM1 + silu_and_mul.  A = x [T, K] gathered by row_to_slot /
//                topk, W = W1 [El, 2*Fh, K], out = act [N, Fh] (bf16 bits).
// GATED = false: GEMM2.  A = act [N, K] (grouped rows), W = W2 [El, Nw, K],
//                out = y [N, Nw] (OT = bf16 bits or float).
template <int MBW, bool GATED, typename OT>
__global__ __launch_bounds__(kTThreads) void ffn_tiled_kernel(
    const uint16_t* __restrict__ A, int K, int topk, const int32_t* __restrict__ r2s, const uint16_t* __restrict__ W,
    int Nw, int Fh, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, int El,
    OT* __restrict__ out, int ldo, uint32_t a_bytes, int NT) {
  constexpr int BM = 64 * MBW;
  constexpr int A_CH = BM * 8 / kTThreads;   // 16-byte chunks of the A tile per thread
  constexpr int B_CH = kBN * 8 / kTThreads;  // ... of the B tile
  static_assert(A_CH == 2 * MBW && B_CH == 4, "thread/chunk mapping");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBN * kLds];

  int mt, ntile;
  xcd_map(blockIdx.x, NT, mt, ntile);
  int e, row0, nrows;
  if (!find_tile_t(counts, offsets, El, BM, mt, e, row0, nrows)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = ntile * (GATED ? kBN / 2 : kBN);  // first act column (GEMM1) / output column (GEMM2)

  // A: byte offsets of this thread's rows.  Rows past nrows get an offset
  // beyond the buffer's range (a_bytes < 2^31 and K offsets stay below 2^31):
  // the range-checked buffer load returns zeros for them without a memory
  // access, so every load is unconditional and the compiler can keep exact
  // vmcnt waits (two K steps in flight).
  const int kc = tid & 7;
  const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(A, a_bytes);
  uint32_t a_off[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int r = (tid >> 3) + 32 * i;
    if (r < nrows) {
      const uint32_t row = GATED ? (uint32_t)(r2s[row0 + r] / topk) : (uint32_t)(row0 + r);
      a_off[i] = (row * (uint32_t)K + kc * 8) * 2u;
    } else {
      a_off[i] = 0x80000000u;
    }
  }
  // B: this expert's weight rows, offsets relative to the expert's slab
  const int rows_e = GATED ? 2 * Fh : Nw;
  const __amdgpu_buffer_rsrc_t rb_rsrc = make_rsrc(W + (int64_t)e * rows_e * K, (uint32_t)rows_e * K * 2u);
  uint32_t b_off[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = (tid >> 3) + 32 * i;
    uint32_t wrow;
    if constexpr (GATED) wrow = (((c >> 5) & 1) ? Fh : 0) + n0 + (c >> 6) * 32 + (c & 31);
    else wrow = n0 + c;
    b_off[i] = (wrow * (uint32_t)K + kc * 8) * 2u;
  }

  f32x16 acc[MBW][2];
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mb][nb][j] = 0.0f;

  // blocks b = 2*mb + wm with b*32 < nrows
  int live = ((nrows + 31) / 32 - wm + 1) / 2;
  live = live < 0 ? 0 : (live > MBW ? MBW : live);

  switch (live) {
    case 0: kloop<MBW, 0>(ra_rsrc, a_off, rb_rsrc, b_off, As, Bs, acc, K, nrows, tid, lane, wm, wn); break;
    case 1: kloop<MBW, 1>(ra_rsrc, a_off, rb_rsrc, b_off, As, Bs, acc, K, nrows, tid, lane, wm, wn); break;
    case 2: kloop<MBW, (MBW >= 2 ? 2 : MBW)>(ra_rsrc, a_off, rb_rsrc, b_off, As, Bs, acc, K, nrows, tid, lane, wm, wn); break;
    case 3: kloop<MBW, (MBW >= 3 ? 3 : MBW)>(ra_rsrc, a_off, rb_rsrc, b_off, As, Bs, acc, K, nrows, tid, lane, wm, wn); break;
    case 4: kloop<MBW, (MBW >= 4 ? 4 : MBW)>(ra_rsrc, a_off, rb_rsrc, b_off, As, Bs, acc, K, nrows, tid, lane, wm, wn); break;
    default: kloop<MBW, MBW>(ra_rsrc, a_off, rb_rsrc, b_off, As, Bs, acc, K, nrows, tid, lane, wm, wn); break;
  }

  // Epilogue.  acc[mb][nb][j] is C[row (j/4)*8 + (lane/32)*4 + j%4][col lane%32]
  // of block b = 2*mb + wm.  bf16 results are staged through LDS (the K loop
  // is done with it) so that global stores are whole 16-byte row pieces.
  const int cl = lane & 31;
  if constexpr (GATED || sizeof(OT) == 2) {
    constexpr int OC = GATED ? kBN / 2 : kBN;  // output columns of the block
    constexpr int OS = OC + 8;                 // padded LDS row (bf16 elements)
    static_assert(BM * OS <= 2 * BM * kLds, "staging tile fits in the A buffers");
    uint16_t* st = &As[0][0];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
      if (mb >= live) continue;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = (2 * mb + wm) * 32 + (j >> 2) * 8 + (lane >> 5) * 4 + (j & 3);
        if constexpr (GATED) {
          const float g = acc[mb][0][j], u = acc[mb][1][j];
          st[r * OS + wn * 32 + cl] = f32_to_bf16_bits(g / (1.0f + expf(-g)) * u);
        } else {
          st[r * OS + wn * 64 + cl] = f32_to_bf16_bits(acc[mb][0][j]);
          st[r * OS + wn * 64 + 32 + cl] = f32_to_bf16_bits(acc[mb][1][j]);
        }
      }
    }
    __syncthreads();
    constexpr int CPR = OC / 8;  // 16-byte pieces per row
    uint16_t* ob = reinterpret_cast<uint16_t*>(out);
    for (int p = tid; p < nrows * CPR; p += kTThreads) {
      const int r = p / CPR, c8 = (p % CPR) * 8;
      *reinterpret_cast<u32x4*>(ob + (int64_t)(row0 + r) * ldo + n0 + c8) =
          *reinterpret_cast<const u32x4*>(st + r * OS + c8);
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
      if (mb >= live) continue;
      for (int j = 0; j < 16; ++j) {
        const int r = (2 * mb + wm) * 32 + (j >> 2) * 8 + (lane >> 5) * 4 + (j & 3);
        if (r >= nrows) continue;
        const int64_t orow = (int64_t)(row0 + r) * ldo;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) out[orow + n0 + wn * 64 + nb * 32 + cl] = acc[mb][nb][j];
      }
    }
  }
}

template <int MBW>
hipError_t launch_tiled_mbw(const uint16_t* x, int64_t T, int64_t N, int topk, int H, int F, int El,
                            const uint16_t* w1, const uint16_t* w2, const int32_t* counts, const int32_t* offsets,
                            const int32_t* r2s, void* y, int y_dtype, uint16_t* act, hipStream_t stream) {
  constexpr int BM = 64 * MBW;
  int64_t mtiles = (N + BM - 1) / BM + (N < El ? N : (int64_t)El);
  mtiles = (mtiles + 7) / 8 * 8;  // whole rounds of the 8 XCDs
  const int nt1 = F / (kBN / 2), nt2 = H / kBN;
  hipLaunchKernelGGL((ffn_tiled_kernel<MBW, true, uint16_t>), dim3((unsigned)(mtiles * nt1)), dim3(kTThreads), 0,
                     stream, x, H, topk, r2s, w1, 2 * F, F, counts, offsets, El, act, F, (uint32_t)(T * H * 2), nt1);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 g2((unsigned)(mtiles * nt2));
  const uint32_t act_bytes = (uint32_t)(N * F * 2);
  if (y_dtype == MOE_BF16)
    hipLaunchKernelGGL((ffn_tiled_kernel<MBW, false, uint16_t>), g2, dim3(kTThreads), 0, stream, act, F, topk, r2s,
                       w2, H, F, counts, offsets, El, static_cast<uint16_t*>(y), H, act_bytes, nt2);
  else
    hipLaunchKernelGGL((ffn_tiled_kernel<MBW, false, float>), g2, dim3(kTThreads), 0, stream, act, F, topk, r2s, w2,
                       H, F, counts, offsets, El, static_cast<float*>(y), H, act_bytes, nt2);
  return hipGetLastError();
}

}  // namespace

bool tiled_ffn_applicable(int64_t N, int H, int F, int El) {
  // K steps of 64 for both GEMMs, 64 act columns per GEMM1 block, 128 output
  // columns per GEMM2 block, and enough rows per expert to fill the tiles
  // buffer offsets are 32-bit byte offsets: x and act must stay below 2 GiB
  // (offsets from 2^31 up mark padding rows), one expert's weights below 4 GiB
  return (H % kBN == 0) && (F % 64 == 0) && (N / (El > 0 ? El : 1) >= 96) &&
         (N * (int64_t)(H > F ? H : F) * 2 < ((int64_t)1 << 31)) && ((int64_t)2 * F * H * 2 < ((int64_t)1 << 32));
}

hipError_t launch_tiled_ffn(const uint16_t* x, int64_t T, int64_t N, int topk, int H, int F, int El,
                            const uint16_t* w1, const uint16_t* w2, const int32_t* counts, const int32_t* offsets,
                            const int32_t* r2s, void* y, int y_dtype, uint16_t* act, hipStream_t stream) {
  const int64_t avg = N / El;
  if (avg >= 192)
    return launch_tiled_mbw<5>(x, T, N, topk, H, F, El, w1, w2, counts, offsets, r2s, y, y_dtype, act, stream);
  return launch_tiled_mbw<2>(x, T, N, topk, H, F, El, w1, w2, counts, offsets, r2s, y, y_dtype, act, stream);
}

}  // namespace moe
