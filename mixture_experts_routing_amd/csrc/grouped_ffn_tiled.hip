// LDS-tiled expert GEMMs for many rows per expert (prefill sizes).
//
// Same contract as the streaming kernels of grouped_ffn.hip (the
// expand -> gemm1 -> silu_and_mul -> gemm2 order of the FusedMoE pipeline on
// the "Upstream Reference: Deep-Spark xllm + vllm" page, "File Index"; the
// expert-grouped layout and cross-row weight reuse of the b70 lab note "MTP1
// M2 compact scheduler closure", design paragraph), tiled for the matrix
// cores:
//
//   tile         BM (320 or 128) rows of one expert x 256 weight rows; K is
//                walked in steps of 32.  8 waves (2 per SIMD) in a 2 x 4
//                grid; wave (wm, wn) owns the 32-row blocks b = 2*mb + wm and
//                64 weight rows, i.e. (BM/64) x 2 tiles of
//                v_mfma_f32_32x32x16_bf16 accumulators.
//   persistent   one block per compute unit walks a fixed sequence of tiles
//                of its XCD; the load pipeline runs on across tile borders,
//                so a tile's first K steps arrive while the previous tile
//                finishes, and the next tile's row lookup is done a tile
//                ahead.
//   loads        global -> LDS with buffer_load ... lds (no registers) into a
//                4-slot ring of K steps, two steps in flight while one is
//                computed; waves 0-3 move A rows, waves 4-7 weight rows.
//                LDS rows are 64 bytes with XOR-swizzled 16-byte pieces so the
//                fragment reads are free of bank conflicts.  One barrier per
//                K step.  Tile-packed weights (moe_pack_ffn_weights) arrive
//                as one contiguous 16 KB block per step.
//   GEMM1        A rows are gathered from x through row_to_slot (expand); the
//                256 weight rows are 128 gate rows and the matching 128 up
//                rows interleaved in 32-row groups, so each lane holds a gate
//                value and its up value and silu(g)*u is formed in registers
//   GEMM2        A rows are act rows; 256 output columns per tile
//   rows         32-row MFMA blocks past the tile's last valid row are skipped
//   epilogue     the weight fragment is the MFMA's first operand, so a lane
//                holds 4 consecutive output columns of one row; bf16 results
//                pass through a 2 KB LDS block per wave (beside the ring) and
//                leave as 16 contiguous bytes per lane
//
// One expert's whole row set usually fits one M-tile (BM = 320 >= the
// typical 256 +- 3 sigma rows at top-8 of 128), so each (expert, N-tile)
// weight panel is read from HBM once.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTThreads = 512;  // 8 waves: 2 per SIMD
constexpr int kBK = kPanelK;     // K elements per step: 64 bytes of every A and B row
constexpr int kBN = kPanelRows; // weight rows per block
constexpr int kStages = 4;      // LDS ring: steps k+1, k+2 in flight while step k computes
constexpr int kRowBytes = kBK * 2;
constexpr int kGrid = 256;       // persistent blocks: one per compute unit
constexpr int kEpiBytes = 2048;  // per-wave LDS block of the epilogue: 32 rows x 64 bytes
// cache policy of the weight loads: non-temporal (each weight panel is read
// by one block, once), so the streamed weights do not push the re-read A
// rows out of the caches
constexpr int kWeightCachePolicy = 2;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14)
constexpr int wait_vm(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14); }
constexpr int kWaitLgkm0 = 0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14);

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

// silu(g) = g * sigmoid(g) with the hardware base-2 exponential and
// reciprocal (about 1 ulp each): a few instructions per value instead of the
// libm expf and an IEEE divide, far below the bf16 rounding of the stored
// act value.  g = +-inf and NaN give what g / (1 + exp(-g)) gives.
__device__ __forceinline__ float silu_fast(float g) {
  constexpr float kLog2e = 1.4426950408889634f;
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -kLog2e));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw (unstructured) buffer: stride 0, byte-addressed, range-checked
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// LDS layout of one stage: BM A rows then kBN B rows, 64 bytes each (one K
// step), unpadded.  The four 16-byte pieces of row R are stored XOR-swizzled,
// piece p at p ^ swz(R): the fragment reads of 8 (or 16) consecutive lanes --
// consecutive rows, one logical piece -- then hit distinct 16-byte bank groups
// whether the LDS serves 8 or 16 lanes per cycle.
__device__ __forceinline__ int swz(int R) { return panel_swz(R); }

// 16-row units of a stage: waves 0-3 move the BM/16 A units (unit u = wave +
// 4*i), waves 4-7 the kBN/16 = 16 B units, so every load instruction of a
// wave uses one fixed buffer resource.
template <int MBW>
struct Units {
  static constexpr int BM = 64 * MBW;
  static constexpr int A = BM / 64;   // A units per A wave
  static constexpr int B = kBN / 64;  // B units per B wave
  static constexpr int MAXW = A > B ? A : B;
};

// Block -> tiles.  Workgroups are dispatched to the 8 XCDs round robin
// (linear id % 8); block b walks tiles L = b, b + G, b + 2G, ... (G, the
// grid, a multiple of 8), so all its tiles belong to XCD b % 8.  M-tiles are
// dealt to XCDs round robin and, within an XCD, neighbouring tile indices
// walk the N-tiles of one M-tile, so the blocks that share an A tile (the
// expert's gathered rows) run together on one XCD and find it in that XCD's
// L2; every weight panel is read by exactly one block.
__device__ __forceinline__ void xcd_map(int L, int NT, int& mt, int& nt) {
  const int xcd = L & 7, local = L >> 3;
  mt = xcd + 8 * (local / NT);
  nt = local % NT;
}

// What a block needs to stream one tile: the weight resource, this lane's
// DMA source offsets (A rows for waves 0-3, weight rows for waves 4-7) and
// the tile's rows.
struct Tile {
  __amdgpu_buffer_rsrc_t rb;
  uint32_t src[5];
  int row0, nrows, n0;
  bool valid;
};

template <int MBW, bool GATED, bool PACKED>
__device__ __forceinline__ void load_tile(Tile& t, int L, int NT, const uint16_t* __restrict__ W, int rows_e, int Fh,
                                          int K, int topk, const int32_t* __restrict__ r2s,
                                          const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
                                          int El, int wave, int lane) {
  using U = Units<MBW>;
  constexpr int BM = U::BM;
  int mt, nt, e = 0, row0 = 0, nrows = 0;
  xcd_map(L, NT, mt, nt);
  t.valid = find_tile_t(counts, offsets, El, BM, mt, e, row0, nrows);
  if (!t.valid) return;  // uniform
  t.row0 = row0;
  t.nrows = nrows;
  t.n0 = nt * (GATED ? kBN / 2 : kBN);
  t.rb = PACKED ? make_rsrc(W + ((int64_t)e * rows_e + (int64_t)nt * kBN) * K, (uint32_t)kBN * K * 2u)
                : make_rsrc(W + (int64_t)e * rows_e * K, (uint32_t)rows_e * K * 2u);
  // A rows past nrows get an offset beyond the A buffer's range (its size is
  // below 2^31 and K offsets stay below 2^31): the range-checked load reads
  // nothing for them.
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    uint32_t off = 0x80000000u;
    if (wave < 4) {
      const int R = (wave + 4 * i) * 16 + (lane >> 2);  // A row of the tile
      if (i < U::A && R < nrows) {
        const uint32_t row = GATED ? (uint32_t)(r2s[row0 + R] / topk) : (uint32_t)(row0 + R);
        off = row * (uint32_t)K * 2u + (uint32_t)((lane & 3) ^ swz(R)) * 16u;
      }
    } else if (i < U::B) {
      const int c = (wave - 4 + 4 * i) * 16 + (lane >> 2);  // weight row of the tile
      if constexpr (PACKED) {
        // a packed K-step block is the LDS image: unit u at u KB, lane at 16 B
        off = (uint32_t)((wave - 4 + 4 * i) * 1024 + lane * 16);
      } else {
        const uint32_t wrow = GATED ? (uint32_t)panel_w1_row(c, nt, Fh) : (uint32_t)panel_w2_row(c, nt);
        off = wrow * (uint32_t)K * 2u + (uint32_t)((lane & 3) ^ swz(BM + c)) * 16u;
      }
    }
    t.src[i] = off;
  }
}

// K loop of one tile: KT steps, global step counter g (ring slot g %
// kStages).  At each step the loads of global step g + kStages - 1 are
// issued: this tile's, the next tile's first steps, or (after the last tile)
// loads of an empty buffer (all out of range: no memory traffic) so that
// every step issues the same number of loads and each wave's vmcnt
// arithmetic holds.  LIVE: A blocks of this wave holding valid rows.
template <int MBW, int LIVE, bool PACKED>
__device__ __forceinline__ void tile_kloop(const Tile& cur, const Tile& nxt, __amdgpu_buffer_rsrc_t ra,
                                           __amdgpu_buffer_rsrc_t rz, uint8_t* __restrict__ lds,
                                           f32x16 (&acc)[MBW][2], int KT, int& g, int wave, int lane, int wm,
                                           int wn) {
  using U = Units<MBW>;
  constexpr int BM = U::BM;
  constexpr int STAGE = (BM + kBN) * kRowBytes;
  const bool a_wave = wave < 4;  // uniform
  auto dma = [&](int slot, const Tile& t, int kt, bool real) {
    const int sk = real ? kt * kRowBytes : 0;
    const int skb = real ? kt * (PACKED ? kBN * kRowBytes : kRowBytes) : 0;
    uint8_t* base = lds + slot * STAGE;
    if (a_wave) {
      const __amdgpu_buffer_rsrc_t r = real ? ra : rz;
#pragma unroll
      for (int i = 0; i < U::A; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(base + (wave + 4 * i) * 1024), 16, t.src[i], sk, 0,
                                                 0);
    } else {
      const __amdgpu_buffer_rsrc_t r = real ? t.rb : rz;
#pragma unroll
      for (int i = 0; i < U::B; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(base + BM * kRowBytes + (wave - 4 + 4 * i) * 1024),
                                                 16, t.src[i], skb, 0, kWeightCachePolicy);
    }
  };
  // fragment addresses (bytes within a stage): lane l reads row R, logical
  // piece 2*ks + l/32
  const int r32 = lane & 31, hi = lane >> 5, sw = swz(r32);
  int a_addr[LIVE > 0 ? LIVE : 1][2], b_addr[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int mb = 0; mb < LIVE; ++mb) a_addr[mb][ks] = ((2 * mb + wm) * 32 + r32) * kRowBytes + (((2 * ks + hi) ^ sw) * 16);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      b_addr[nb][ks] = (BM + wn * 64 + nb * 32 + r32) * kRowBytes + (((2 * ks + hi) ^ sw) * 16);
  }
  // The fragments of the step's first K half are requested first; its MFMAs
  // then alternate with the reads of the second half (one read after each
  // MFMA), so the first MFMAs do not queue behind the whole step's LDS reads.
  // mid() runs between the two halves' MFMAs: the step's loads are issued
  // there, while the MFMA unit still works through both waves' first halves,
  // instead of after the step, where the two waves of a SIMD would issue them
  // with nothing left in the MFMA pipe.
  auto compute = [&](int slot, auto&& mid) {
    const uint8_t* base = lds + slot * STAGE;
    bf16x8 a[2][LIVE > 0 ? LIVE : 1], b[2][2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) b[0][nb] = *reinterpret_cast<const bf16x8*>(base + b_addr[nb][0]);
#pragma unroll
    for (int mb = 0; mb < LIVE; ++mb) a[0][mb] = *reinterpret_cast<const bf16x8*>(base + a_addr[mb][0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) b[1][nb] = *reinterpret_cast<const bf16x8*>(base + b_addr[nb][1]);
#pragma unroll
    for (int mb = 0; mb < LIVE; ++mb) a[1][mb] = *reinterpret_cast<const bf16x8*>(base + a_addr[mb][1]);
#pragma unroll
    for (int mb = 0; mb < LIVE; ++mb) {
      acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[0][0], a[0][mb], acc[mb][0], 0, 0, 0);
      acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[0][1], a[0][mb], acc[mb][1], 0, 0, 0);
    }
    // scheduling groups (mask 0x008: MFMA, 0x100: LDS read)
#pragma unroll
    for (int i = 0; i < LIVE + 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (LIVE > 2) __builtin_amdgcn_sched_group_barrier(0x008, LIVE - 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    mid();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < LIVE; ++mb) {
      acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[1][0], a[1][mb], acc[mb][0], 0, 0, 0);
      acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[1][1], a[1][mb], acc[mb][1], 0, 0, 0);
    }
  };
  for (int kt = 0; kt < KT; ++kt, ++g) {
    // own loads of step g have landed once only the kStages-2 newer steps remain
    if (a_wave) __builtin_amdgcn_s_waitcnt(wait_vm((kStages - 2) * U::A));
    else __builtin_amdgcn_s_waitcnt(wait_vm((kStages - 2) * U::B));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // the slot read in step g-1 is free: every wave has passed the barrier
    const int ahead = kt + kStages - 1;
    const int fill = (g + kStages - 1) % kStages;
    compute(g % kStages, [&] {
      if (ahead < KT) dma(fill, cur, ahead, true);
      else dma(fill, nxt, ahead - KT, nxt.valid);
    });
    __builtin_amdgcn_sched_barrier(0);
  }
}

// GATED = true : GEMM1 + silu_and_mul.  A = x [T, K] gathered by row_to_slot /
//                topk, W = W1 [El, 2*Fh, K], out = act [N, Fh] (bf16 bits).
// GATED = false: GEMM2.  A = act [N, K] (grouped rows), W = W2 [El, Nw, K],
//                out = y [N, Nw] (OT = bf16 bits or float).
// PACKED: W is in the tile-packed layout (one contiguous 16 KB block per K
// step of a tile's panel), else row-major.  K / 32 >= kStages - 1.
template <int MBW, bool GATED, bool PACKED, typename OT>
__global__ __launch_bounds__(kTThreads) void ffn_tiled_kernel(
    const uint16_t* __restrict__ A, int K, int topk, const int32_t* __restrict__ r2s, const uint16_t* __restrict__ W,
    int Nw, int Fh, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, int El,
    OT* __restrict__ out, int ldo, uint32_t a_bytes, int NT) {
  using U = Units<MBW>;
  constexpr int BM = U::BM;
  constexpr int RING = kStages * (BM + kBN) * kRowBytes;
  static_assert(RING + (kTThreads / 64) * kEpiBytes <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[RING + (kTThreads / 64) * kEpiBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: resource choices stay scalar
  const int wm = wave >> 2, wn = wave & 3;
  const int rows_e = GATED ? 2 * Fh : Nw;
  const int KT = K / kBK;
  const int G = gridDim.x;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, a_bytes);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(A, 0u);

  Tile cur, nxt;
  int L = blockIdx.x;
  load_tile<MBW, GATED, PACKED>(cur, L, NT, W, rows_e, Fh, K, topk, r2s, counts, offsets, El, wave, lane);
  if (!cur.valid) return;  // uniform: the whole block has no tile
  load_tile<MBW, GATED, PACKED>(nxt, L + G, NT, W, rows_e, Fh, K, topk, r2s, counts, offsets, El, wave, lane);

  // prologue: the first kStages-1 steps of the first tile
  {
    constexpr int STAGE = (BM + kBN) * kRowBytes;
    const bool a_wave = wave < 4;
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) {
      uint8_t* base = lds + s * STAGE;
      if (a_wave) {
#pragma unroll
        for (int i = 0; i < U::A; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(base + (wave + 4 * i) * 1024), 16, cur.src[i],
                                                   s * kRowBytes, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < U::B; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(cur.rb, (lds_ptr_t)(base + BM * kRowBytes + (wave - 4 + 4 * i) * 1024),
                                                   16, cur.src[i], s * (PACKED ? kBN * kRowBytes : kRowBytes), 0,
                                                   kWeightCachePolicy);
      }
    }
  }

  int g = 0;
  while (true) {
    f32x16 acc[MBW][2];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[mb][nb][j] = 0.0f;
    // blocks b = 2*mb + wm with b*32 < nrows
    int live = ((cur.nrows + 31) / 32 - wm + 1) / 2;
    live = live < 0 ? 0 : (live > MBW ? MBW : live);
    switch (live) {
      case 0: tile_kloop<MBW, 0, PACKED>(cur, nxt, ra, rz, lds, acc, KT, g, wave, lane, wm, wn); break;
      case 1: tile_kloop<MBW, 1, PACKED>(cur, nxt, ra, rz, lds, acc, KT, g, wave, lane, wm, wn); break;
      case 2: tile_kloop<MBW, (MBW >= 2 ? 2 : MBW), PACKED>(cur, nxt, ra, rz, lds, acc, KT, g, wave, lane, wm, wn); break;
      case 3: tile_kloop<MBW, (MBW >= 3 ? 3 : MBW), PACKED>(cur, nxt, ra, rz, lds, acc, KT, g, wave, lane, wm, wn); break;
      case 4: tile_kloop<MBW, (MBW >= 4 ? 4 : MBW), PACKED>(cur, nxt, ra, rz, lds, acc, KT, g, wave, lane, wm, wn); break;
      default: tile_kloop<MBW, MBW, PACKED>(cur, nxt, ra, rz, lds, acc, KT, g, wave, lane, wm, wn); break;
    }

    // Epilogue (the LDS ring already holds the next tile's first steps).  The
    // weight fragment is the MFMA's first operand, so acc[mb][nb][4q + i] is
    // C[row lane%32 of block b = 2*mb + wm][column 8q + 4*(lane/32) + i of
    // the 32-column block nb]: four consecutive columns per lane.  bf16
    // results are packed to 8 bytes, written to this wave's own LDS block
    // (row m at 64 m bytes, its four 16-byte pieces XOR-swizzled by m/4) and
    // read back as 16 bytes of one row per lane, so each store instruction
    // writes 16 rows x 64 contiguous bytes.  f32 results are stored as 16
    // bytes per lane straight from the accumulators.
    {
      const int m = lane & 31, h = lane >> 5;
      uint8_t* stage = lds + RING + wave * kEpiBytes;
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb) {
        if (mb >= live) continue;
        const int rb = (2 * mb + wm) * 32;  // the block's first row in the tile
#pragma unroll
        for (int ob = 0; ob < (GATED ? 1 : 2); ++ob) {
          const int col0 = cur.n0 + (GATED ? wn * 32 : wn * 64 + ob * 32);
          if constexpr (!GATED && sizeof(OT) == 4) {
            if (rb + m < cur.nrows) {
              float* orow = reinterpret_cast<float*>(out) + (int64_t)(cur.row0 + rb + m) * ldo + col0 + 4 * h;
#pragma unroll
              for (int q = 0; q < 4; ++q)
                *reinterpret_cast<f32x4*>(orow + 8 * q) =
                    f32x4{acc[mb][ob][4 * q], acc[mb][ob][4 * q + 1], acc[mb][ob][4 * q + 2], acc[mb][ob][4 * q + 3]};
            }
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float v[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                if constexpr (GATED) v[i] = silu_fast(acc[mb][0][4 * q + i]) * acc[mb][1][4 * q + i];
                else v[i] = acc[mb][ob][4 * q + i];
              }
              *reinterpret_cast<u32x2*>(stage + m * 64 + ((q ^ ((m >> 2) & 3)) * 16) + h * 8) =
                  u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const int r = i * 16 + (lane >> 2), c = lane & 3;
              const u32x4 w = *reinterpret_cast<const u32x4*>(stage + r * 64 + ((c ^ ((r >> 2) & 3)) * 16));
              if (rb + r < cur.nrows)
                *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + (int64_t)(cur.row0 + rb + r) * ldo + col0 +
                                          c * 8) = w;
            }
          }
        }
      }
    }

    if (!nxt.valid) break;  // uniform
    cur = nxt;
    L += G;
    load_tile<MBW, GATED, PACKED>(nxt, L + G, NT, W, rows_e, Fh, K, topk, r2s, counts, offsets, El, wave, lane);
  }
  // drain the trailing (empty) loads before the block's LDS is released
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
}

template <int MBW, bool PACKED>
hipError_t launch_tiled_mbw(const uint16_t* x, int64_t T, int64_t N, int topk, int H, int F, int El,
                            const uint16_t* w1, const uint16_t* w2, const int32_t* counts, const int32_t* offsets,
                            const int32_t* r2s, void* y, int y_dtype, uint16_t* act, hipStream_t stream) {
  constexpr int BM = 64 * MBW;
  int64_t mtiles = (N + BM - 1) / BM + (N < El ? N : (int64_t)El);
  mtiles = (mtiles + 7) / 8 * 8;  // whole rounds of the 8 XCDs
  const int nt1 = F / (kBN / 2), nt2 = H / kBN;  // 128 act columns / 256 output columns per tile
  // persistent grid: one block per compute unit, fewer if there are fewer tiles
  auto grid = [&](int nt) {
    const int64_t tiles = mtiles * nt;
    return dim3((unsigned)(tiles < kGrid ? tiles : kGrid));
  };
  hipLaunchKernelGGL((ffn_tiled_kernel<MBW, true, PACKED, uint16_t>), grid(nt1), dim3(kTThreads), 0, stream, x, H,
                     topk, r2s, w1, 2 * F, F, counts, offsets, El, act, F, (uint32_t)(T * H * 2), nt1);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 g2 = grid(nt2);
  const uint32_t act_bytes = (uint32_t)(N * F * 2);
  if (y_dtype == MOE_BF16)
    hipLaunchKernelGGL((ffn_tiled_kernel<MBW, false, PACKED, uint16_t>), g2, dim3(kTThreads), 0, stream, act, F, topk,
                       r2s, w2, H, F, counts, offsets, El, static_cast<uint16_t*>(y), H, act_bytes, nt2);
  else
    hipLaunchKernelGGL((ffn_tiled_kernel<MBW, false, PACKED, float>), g2, dim3(kTThreads), 0, stream, act, F, topk, r2s,
                       w2, H, F, counts, offsets, El, static_cast<float*>(y), H, act_bytes, nt2);
  return hipGetLastError();
}

}  // namespace

bool tiled_shape_ok(int64_t N, int H, int F) {
  // 128 act columns per GEMM1 block, 256 output columns per GEMM2 block (so
  // both reduction lengths are multiples of the 32-wide step).  Buffer
  // offsets are 32-bit byte offsets: x and act must stay below 2 GiB (offsets
  // from 2^31 up mark padding rows), one expert's weights below 4 GiB.
  return (H % kBN == 0) && (F % (kBN / 2) == 0) && (N * (int64_t)(H > F ? H : F) * 2 < ((int64_t)1 << 31)) &&
         ((int64_t)2 * F * H * 2 < ((int64_t)1 << 32));
}

bool tiled_ffn_applicable(int64_t N, int H, int F, int El) {
  // row-major weights: worth it once experts hold enough rows to fill the tiles
  return tiled_shape_ok(N, H, F) && (N / (El > 0 ? El : 1) >= 96);
}

hipError_t launch_tiled_ffn(const uint16_t* x, int64_t T, int64_t N, int topk, int H, int F, int El,
                            const uint16_t* w1, const uint16_t* w2, bool packed, const int32_t* counts,
                            const int32_t* offsets, const int32_t* r2s, void* y, int y_dtype, uint16_t* act,
                            hipStream_t stream) {
  const bool big = N / El >= 192;
  if (packed)
    return big ? launch_tiled_mbw<5, true>(x, T, N, topk, H, F, El, w1, w2, counts, offsets, r2s, y, y_dtype, act, stream)
               : launch_tiled_mbw<2, true>(x, T, N, topk, H, F, El, w1, w2, counts, offsets, r2s, y, y_dtype, act, stream);
  return big ? launch_tiled_mbw<5, false>(x, T, N, topk, H, F, El, w1, w2, counts, offsets, r2s, y, y_dtype, act, stream)
             : launch_tiled_mbw<2, false>(x, T, N, topk, H, F, El, w1, w2, counts, offsets, r2s, y, y_dtype, act, stream);
}

// ---------------------------------------------------------------------------
// moe_pack_ffn_weights: row-major bf16 W1 / W2 -> tile-packed layout.  One
// thread per 16-byte piece of the destination (contiguous stores).

namespace {

__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ w, uint16_t* __restrict__ wt,
                                                   int64_t pieces, int rows, int K, int gated, int F) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= pieces) return;
  const int64_t per_expert = (int64_t)rows * K / 8;
  const int64_t e = q / per_expert;
  int64_t r = q - e * per_expert;
  const int64_t per_panel = (int64_t)kPanelRows * K / 8;
  const int nt = (int)(r / per_panel);
  r -= (int64_t)nt * per_panel;
  const int kt = (int)(r / (kPanelRows * 4));
  const int rem = (int)(r - (int64_t)kt * kPanelRows * 4);
  const int R = rem >> 2, p = rem & 3;
  const int row = gated ? panel_w1_row(R, nt, F) : panel_w2_row(R, nt);
  const int k = kt * kPanelK + ((p ^ panel_swz(R)) * 8);
  const u32x4 v = *reinterpret_cast<const u32x4*>(w + ((int64_t)e * rows + row) * K + k);
  *reinterpret_cast<u32x4*>(wt + q * 8) = v;
}

}  // namespace

hipError_t launch_pack_ffn_weights(const uint16_t* w1, const uint16_t* w2, int El, int H, int F, uint16_t* w1t,
                                   uint16_t* w2t, hipStream_t stream) {
  const int64_t p1 = (int64_t)El * 2 * F * H / 8, p2 = (int64_t)El * H * F / 8;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((p1 + 255) / 256)), dim3(256), 0, stream, w1, w1t, p1, 2 * F, H, 1,
                     F);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((p2 + 255) / 256)), dim3(256), 0, stream, w2, w2t, p2, H, F, 0, F);
  return hipGetLastError();
}

}  // namespace moe
