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
#include <atomic>

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

// Number of M-tiles of height BM over all experts (wave-uniform).
__device__ __forceinline__ int count_tiles(const int32_t* __restrict__ counts, int El, int BM) {
  const int lane = threadIdx.x & 63;
  int n = 0;
  for (int c0 = 0; c0 < El; c0 += 64) {
    const int ee = c0 + lane;
    n += ee < El ? (counts[ee] + BM - 1) / BM : 0;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) n += __shfl_xor(n, d, 64);
  return n;
}

// Tile table of up to 64 experts held in one wave's registers (lane = local
// expert): counts and offsets are read once, side by side, so looking up a
// tile costs no further memory round trip.
struct TileTab {
  int cnt, off, nt, incl, total;
};

// From each lane's own expert count and first row (lanes >= El: count 0).
__device__ __forceinline__ TileTab make_tile_tab(int cnt, int off, int BM) {
  const int lane = threadIdx.x & 63;
  TileTab t;
  t.cnt = cnt;
  t.off = off;
  t.nt = (t.cnt + BM - 1) / BM;
  int inc = t.nt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  t.incl = inc;
  t.total = __shfl(inc, 63, 64);
  return t;
}

__device__ __forceinline__ TileTab load_tile_tab(const int32_t* __restrict__ counts,
                                                 const int32_t* __restrict__ offsets, int El, int BM) {
  const int lane = threadIdx.x & 63;
  return make_tile_tab(lane < El ? counts[lane] : 0, lane < El ? offsets[lane] : 0, BM);
}

// Route compaction of at most 64 slots (one per lane) into at most 64 local
// experts, in one wave's registers -- the same stable counting sort as the
// one-wave compaction kernel: the row of slot s is the number of local slots
// with a smaller local id plus the number of earlier slots with the same id.
// Lane e also gets expert e's count and first row; lane r gets the slot of
// row r (-1 for r >= R).  N, Eg, El are wave-uniform.
struct WaveRoutes {
  int row;  // this lane's slot: its grouped row, -1 if remote or lane >= N
  int cnt;  // expert `lane`: routed rows
  int off;  // expert `lane`: first row (R for lanes >= El)
  int inv;  // row `lane`: its slot, -1 if lane >= R
  int R;    // local rows (uniform)
};

__device__ __forceinline__ WaveRoutes wave_routes(const int32_t* __restrict__ ids, int N,
                                                 const int32_t* __restrict__ emap, int Eg, int El) {
  const int lane = threadIdx.x & 63;
  const int l = lane < N ? local_expert(ids[lane], emap, Eg, El) : -1;
  WaveRoutes w;
  int row = 0, cnt = 0, off = 0;
  for (int j = 0; j < N; ++j) {
    const int lj = __builtin_amdgcn_readlane(l, j);
    const bool ok = lj >= 0;
    cnt += (lj == lane) ? 1 : 0;
    off += (ok && lj < lane) ? 1 : 0;
    row += (ok && (lj < l || (lj == l && j < lane))) ? 1 : 0;
  }
  w.row = l >= 0 ? row : -1;
  w.cnt = cnt;
  w.off = off;
  w.R = __popcll(__ballot(l >= 0));
  int inv = -1;
  for (int j = 0; j < N; ++j) inv = (__builtin_amdgcn_readlane(w.row, j) == lane) ? j : inv;
  w.inv = inv;
  return w;
}

// Tile i (< t.total): expert, first grouped row, valid rows (wave-uniform).
__device__ __forceinline__ void tab_find(const TileTab& t, int BM, int i, int& e, int& row0, int& nrows) {
  const bool own = (i >= t.incl - t.nt) && (i < t.incl);
  const unsigned long long m = __ballot(own);
  const int src = __ffsll((long long)m) - 1;
  e = src;
  const int tile_in_e = i - __shfl(t.incl - t.nt, src, 64);
  row0 = __shfl(t.off, src, 64) + tile_in_e * BM;
  nrows = min(BM, __shfl(t.cnt, src, 64) - tile_in_e * BM);
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
// One wave: act columns [n0, n0+16) of the rows [row0, row0+nrows) (nrows <=
// 16*MB) of expert e.
template <int MB, int KS, bool MX>
__device__ __forceinline__ void gemm1_cols(const uint16_t* __restrict__ x, int K, int H, int F,
                                           const void* __restrict__ w1, const uint8_t* __restrict__ w1s,
                                           const int32_t* __restrict__ r2s, uint16_t* __restrict__ act, int e,
                                           int row0, int nrows, int n0, int lane) {
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
  gemm1_cols<MB, KS, MX>(x, K, H, F, w1, w1s, r2s, act, e, row0, nrows, n0, lane);
}

// GEMM2.  act [N, F] bf16; w2 [El, H, F]; y [N, H] (bf16 bits or f32).
// One wave: output columns [n0, n0+16) of the rows [row0, row0+nrows) of expert e.
template <int MB, int KS, bool MX, typename YT>
__device__ __forceinline__ void gemm2_cols(const uint16_t* __restrict__ act, int H, int F,
                                           const void* __restrict__ w2, const uint8_t* __restrict__ w2s,
                                           YT* __restrict__ y, int e, int row0, int nrows, int n0, int lane) {
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
  gemm2_cols<MB, KS, MX, YT>(act, H, F, w2, w2s, y, e, row0, nrows, n0, lane);
}

// ---------------------------------------------------------------------------
// Few rows per expert (decode): 16-wave blocks with an in-block K split.
//
// With a handful of rows per expert the FFN is a weight stream.  One wave per
// 16 output columns of a 16-row M-tile leaves too few waves in flight to keep
// HBM busy when only one or two experts are hit, so each 1024-thread block
// takes an item -- one M-tile and 16/S column groups (16 output columns of
// GEMM2; 8 act columns, i.e. 8 gate and 8 up weight rows, of GEMM1) -- and
// its 16 waves split the reduction dimension S ways.  The partial accumulators meet
// in LDS and are summed in split order, so the result does not depend on
// timing.  S is derived on device from the actual tile count (decode_split),
// and the grid is persistent: a fixed number of blocks walks the item list,
// so nothing is launched for tiles that do not exist (an all-remote batch
// costs one pass over counts).
//
// K is walked in 32-wide units; in unit u, lane group g = lane/16 holds
// elements [32u + 8g, 32u + 8g + 8) of its A row and B row (the same K
// assignment on both operands, as the MFMA sum requires), so one load
// instruction reads 64 contiguous bytes of each of 16 weight rows.

constexpr int kDecThreads = 1024;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecGrid = 256;
// K units loaded before their MFMAs: 8 (512 bytes of each bf16 weight row);
// 4 for MXFP4 GEMM1, whose widened operands would not fit in 128 VGPRs at 8
template <bool MX>
constexpr int dec_unroll1() { return MX ? 4 : 8; }
constexpr int kDecUnroll = 8;

// K split S: a power of two <= 16 (the block's waves) with at least one K
// unit per split, chosen by an estimate of the kernel's time.  An item (one
// tile x 16/S column groups) keeps each wave busy for about
// max(units/S, kSplitLatencyUnits) unit loads -- past a few units a wave's
// time grows with the bytes it streams, below that the memory latency
// dominates -- and `grid` persistent blocks take ceil(items / grid) rounds.
// A split that leaves compute units idle (items just under a multiple of the
// grid) loses to one that keeps them all streaming.  Of two splits with the
// same estimate the larger wins if it needs no more rounds (its extra items
// land on otherwise idle compute units), else the smaller (fewer partial
// sums to add).  The latency floor is 8 KB of weights per wave: 8 units of
// bf16 (1 KB per wave each), 32 of MXFP4 codes (256 bytes).
constexpr int kSplitLatencyUnits = 8;     // bf16
constexpr int kSplitLatencyUnitsMX = 32;  // MXFP4

__device__ __forceinline__ int decode_split(int tiles, int col_groups, int units, int grid, unsigned lat) {
  // The inputs are wave-uniform: make that visible so the search runs on the
  // scalar unit with 32-bit divisions (a few hundred cycles at most).
  tiles = __builtin_amdgcn_readfirstlane(tiles);
  if (tiles <= 0 || (int64_t)tiles * col_groups >= ((int64_t)1 << 30)) return 1;  // nothing, or plenty, to spread
  const unsigned g = (unsigned)grid;
  int best = 1;
  uint64_t best_cost = ~(uint64_t)0;
  unsigned best_rounds = ~0u;
  for (int s = 1; s <= kDecWaves && s <= units; s <<= 1) {
    const unsigned cpb = (unsigned)(kDecWaves / s);
    const unsigned items = (unsigned)tiles * (((unsigned)col_groups + cpb - 1) / cpb);
    const unsigned rounds = (items + g - 1) / g;
    const unsigned per = ((unsigned)units + s - 1) / (unsigned)s;
    const uint64_t cost = (uint64_t)rounds * (per > lat ? per : lat);
    if (cost < best_cost || (cost == best_cost && rounds <= best_rounds)) {
      best = s;
      best_cost = cost;
      best_rounds = rounds;
    }
  }
  return best;
}

__device__ __forceinline__ bf16x8 widen_mx8(uint32_t w, uint32_t e8) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const float s = e8 == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(e8 << 23);
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
  return bf16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// MXFP4 K units in batches of four for the decode kernels.  Within a batch
// [u, u+4) the lanes of group g take unit u+g whole -- its 16 code bytes in
// one load and its one scale byte -- and feed its 32 elements to the batch's
// four MFMAs, 8 per MFMA (MFMA j: elements 8j..8j+7 of every group's unit).
// The x (or act) operand takes the same elements, so each K element meets its
// weight exactly once; only the order of the sum differs from unit by unit.
// The weight loads of all NB batches are issued before the first MFMA, so a
// wave keeps 1 KB of codes per batch in flight (up to 8 KB).  TWO (a 32-row
// tile): the A rows of the second 16-row half (xr1) meet the same widened
// weights, so one weight byte feeds two MFMAs.  Unit v of an A row starts at
// element 32 (v - ub) of xr0 / xr1.
template <int NB, bool TWO>
__device__ __forceinline__ void mx_batches(f32x4& acc0, f32x4& acc1, const uint16_t* __restrict__ xr0,
                                           const uint16_t* __restrict__ xr1, const uint8_t* __restrict__ wrow,
                                           const uint8_t* __restrict__ srow, int u, int ub, int g) {
  u32x4 cw[NB];
  uint32_t sc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    cw[b] = *reinterpret_cast<const u32x4*>(wrow + 16 * (u + 4 * b + g));
    sc[b] = srow[u + 4 * b + g];
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int xo = 32 * (u + 4 * b + g - ub);
    bf16x8 xa[4], xb[TWO ? 4 : 1];
#pragma unroll
    for (int j = 0; j < 4; ++j) xa[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xr0 + xo + 8 * j));
    if constexpr (TWO) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xb[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xr1 + xo + 8 * j));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 wv = widen_mx8(cw[b][j], sc[b]);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[j], wv, acc0, 0, 0, 0);
      if constexpr (TWO) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb[j], wv, acc1, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);  // the next batch's x loads stay after these MFMAs
  }
}

__device__ __forceinline__ bf16x8 unit_bf16(const uint16_t* __restrict__ row, int u, int g) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + 32 * u + 8 * g));
}

// Raw pieces of one K unit of a weight row: bf16 -> 16 bytes; MXFP4 -> the
// 4 code bytes of this lane and the unit's scale byte.
template <bool MX>
struct WUnit;
template <>
struct WUnit<false> {
  u32x4 v;
  __device__ __forceinline__ void load(const void* __restrict__ w, const uint8_t* __restrict__, int64_t row,
                                       int kdim, int u, int g) {
    v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(w) + row * kdim + 32 * u + 8 * g);
  }
  __device__ __forceinline__ bf16x8 get() const { return __builtin_bit_cast(bf16x8, v); }
};
template <>
struct WUnit<true> {
  uint32_t c, e8;
  __device__ __forceinline__ void load(const void* __restrict__ w, const uint8_t* __restrict__ ws, int64_t row,
                                       int kdim, int u, int g) {
    c = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(w) + row * (kdim / 2) + 16 * u + 4 * g);
    e8 = ws[row * (kdim / 32) + u];
  }
  __device__ __forceinline__ bf16x8 get() const { return widen_mx8(c, e8); }
};

// Workgroup barrier that orders LDS accesses only: global loads in flight
// stay in flight across it (a full __syncthreads waits for them too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One wave's share of a decode item: the dot products of the tile's A rows
// (xr0: this lane's row c; xr1: row 16 + c, used when TWO) with the 16 weight
// rows (rw: this lane's weight row) over K units [u, u_end), added to acc0 /
// acc1 in unit order.  Unit v of an A row starts at element 32 (v - ub): the
// rows may sit in LDS (a staged chunk that begins at unit ub) or in global
// memory (ub = 0).  A 32-row tile reads each weight byte once for both
// halves (the weight pass of a tile serves all its rows).
template <bool MX, int U, bool TWO>
__device__ __forceinline__ void tile_dot(f32x4& acc0, f32x4& acc1, const uint16_t* __restrict__ xr0,
                                         const uint16_t* __restrict__ xr1, int ub, const void* __restrict__ w,
                                         const uint8_t* __restrict__ ws, int64_t rw, int kdim, int u, int u_end,
                                         int g) {
  if constexpr (MX) {
    const uint8_t* wrow = static_cast<const uint8_t*>(w) + rw * (kdim / 2);
    const uint8_t* srow = ws + rw * (kdim / 32);
    // TWO: batches of at most 4 (the second A half needs the registers)
    if constexpr (!TWO)
      for (; u + 32 <= u_end; u += 32) mx_batches<8, TWO>(acc0, acc1, xr0, xr1, wrow, srow, u, ub, g);
    for (; u + 16 <= u_end; u += 16) mx_batches<4, TWO>(acc0, acc1, xr0, xr1, wrow, srow, u, ub, g);
    if (u + 8 <= u_end) {
      mx_batches<2, TWO>(acc0, acc1, xr0, xr1, wrow, srow, u, ub, g);
      u += 8;
    }
    if (u + 4 <= u_end) {
      mx_batches<1, TWO>(acc0, acc1, xr0, xr1, wrow, srow, u, ub, g);
      u += 4;
    }
  } else {
    constexpr int V = TWO ? U / 2 : U;  // the second A half takes the registers of half the batch
    for (; u + V <= u_end; u += V) {
      WUnit<MX> b[V];
      bf16x8 a[V], a1[TWO ? V : 1];
#pragma unroll
      for (int j = 0; j < V; ++j) b[j].load(w, ws, rw, kdim, u + j, g);
#pragma unroll
      for (int j = 0; j < V; ++j) a[j] = unit_bf16(xr0, u + j - ub, g);
      if constexpr (TWO) {
#pragma unroll
        for (int j = 0; j < V; ++j) a1[j] = unit_bf16(xr1, u + j - ub, g);
      }
#pragma unroll
      for (int j = 0; j < V; ++j) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], b[j].get(), acc0, 0, 0, 0);
        if constexpr (TWO) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[j], b[j].get(), acc1, 0, 0, 0);
      }
    }
  }
  for (; u < u_end; ++u) {
    WUnit<MX> b;
    b.load(w, ws, rw, kdim, u, g);
    const bf16x8 wv = b.get();
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(unit_bf16(xr0, u - ub, g), wv, acc0, 0, 0, 0);
    if constexpr (TWO) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(unit_bf16(xr1, u - ub, g), wv, acc1, 0, 0, 0);
  }
}

// The same for one 16-row tile whose rows are in global memory.
template <bool MX, int U>
__device__ __forceinline__ f32x4 tile_dot16(const uint16_t* __restrict__ xr, const void* __restrict__ w,
                                            const uint8_t* __restrict__ ws, int64_t rw, int kdim, int u, int u_end,
                                            int g) {
  f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  tile_dot<MX, U, false>(acc0, acc1, xr, xr, 0, w, ws, rw, kdim, u, u_end, g);
  return acc0;
}

// Tile height of the decode kernels: up to 32 rows of one expert share every
// weight byte an item streams (two 16-row MFMA halves), so an expert with up
// to 32 rows is one weight pass.
constexpr int kDecBM = 32;

// Staged A rows of a decode item.  When the splits leave several waves of a
// block on the same K range, those waves would each load the same A rows
// from global memory; instead the block copies the item's distinct rows (at
// most 32; rows past the tile's end use row 0) into LDS, with contiguous
// 16-byte loads, and every wave reads its fragments from there.  The copy
// and its barriers pay off with at least 4 waves per range (S <= 4), or 2 per
// range (S = 8) when the tile holds 8 rows or more.  Only the MXFP4 kernels
// stage: their A rows are 4x the bytes of the weight codes they meet, and
// the 128 KB block they need keeps a kernel's blocks from sharing a compute
// unit with the previous kernel's, which costs the bf16 decode kernels more
// than the staging saves them.
// Rows that do not fit whole (n rows x K elements above kXsBytes: 32 rows at
// K > 2048, 16 rows at K > 4096) are staged in chunks of whole K units; every
// split takes its share of each chunk (split ks: the ks-th of S equal parts),
// so no wave waits idle while a chunk is in LDS.  In a chunk of nu units, row
// r sits at r * (64 nu + kXsPad) bytes, an odd multiple of 16, so the 16 rows
// a quarter-wave reads (one piece each) start in 16 distinct 16-byte slots of
// the 256-byte bank period and hit distinct banks.
constexpr int kXsPad = 16;
constexpr int kXsBytes = 32 * (64 * 64 + kXsPad);  // 32 rows x 2048 elements (or 16 rows x 4096)
constexpr int kRedBytes = kDecWaves * 8 * 64 * 4;  // split partials: 2 x 4 floats per lane per wave
static_assert(kXsBytes >= kRedBytes, "the split partials reuse the staging buffer");

__device__ __forceinline__ bool stage_item(int S, int nrows) { return S <= 4 || (S <= 8 && nrows >= 8); }

// K units per staged chunk for n rows of `units` units: all of them if they
// fit, else the most that fit, a multiple of 4 (the MXFP4 batch).
__device__ __forceinline__ int stage_chunk_units(int n, int units) {
  const int kmax = (kXsBytes / n - kXsPad) / 64;
  return units <= kmax ? units : (kmax & ~3);
}

// Copy elements [e0, e0 + ne) of rows [0, n) (row r from src_row(r)) into xs
// at row stride 2 ne + kXsPad bytes, then a barrier (the rows are visible).
// Every thread of the block takes part; the caller has passed a barrier after
// the previous reads of xs.
template <typename SrcRow>
__device__ __forceinline__ void stage_rows(uint8_t* __restrict__ xs, int n, int e0, int ne, SrcRow src_row) {
  const int ppr = ne / 8;  // 16-byte pieces per row
  const int RS = 2 * ne + kXsPad;
  for (int p = threadIdx.x; p < n * ppr; p += kDecThreads) {
    const int r = p / ppr, q = p - r * ppr;
    const u32x4 v = *reinterpret_cast<const u32x4*>(src_row(r) + e0 + 8 * q);
    *reinterpret_cast<u32x4*>(xs + r * RS + 16 * q) = v;
  }
  lds_barrier();
}

// The dot products of one item over its staged rows: the block copies the
// rows chunk by chunk and each wave adds its split's share of every chunk.
// `active`, n and the split are wave-uniform.
template <bool MX, int U, bool TWO, typename SrcRow>
__device__ __forceinline__ void staged_dot(f32x4& acc0, f32x4& acc1, uint8_t* __restrict__ xs, int n, bool active,
                                           SrcRow src_row, const void* __restrict__ w,
                                           const uint8_t* __restrict__ ws, int64_t rw, int kdim, int ks, int S,
                                           int c, int g) {
  const int units = kdim / 32;
  const int kc = stage_chunk_units(n, units);
  for (int c0 = 0; c0 < units; c0 += kc) {
    const int nu = min(kc, units - c0);
    lds_barrier();  // every wave is done with the previous rows in xs
    stage_rows(xs, n, 32 * c0, 32 * nu, src_row);
    if (active) {
      const int pc = (nu + S - 1) / S;
      const int ub = c0 + min(nu, ks * pc), ue = c0 + min(nu, ks * pc + pc);
      const int RS = 64 * nu + kXsPad;
      const uint16_t* x0 = reinterpret_cast<const uint16_t*>(xs + (c < n ? c : 0) * RS);
      const uint16_t* x1 = reinterpret_cast<const uint16_t*>(xs + (16 + c < n ? 16 + c : 0) * RS);
      tile_dot<MX, U, TWO>(acc0, acc1, x0, x1, c0, w, ws, rw, kdim, ub, ue, g);
    }
  }
}

// ---------------------------------------------------------------------------
// MXFP4 on the CDNA4 block-scaled matrix cores (MOE_MXFP4_MMA_F8F6F4).
//
// v_mfma_scale_f32_16x16x128_f8f6f4 multiplies a 16 x 128 A block by a
// 128 x 16 B block with an e8m0 scale for every 32 K elements of each A row
// and each B column.  Operand layout (lane l: row or column l % 16, lane
// group g = l / 16; established with one-wave runs on inputs of known
// structure):
//   B, e2m1: the 32 nibbles of dwords 0-3 (low nibble first) are K
//     [32g, 32g + 32);
//   A, e4m3: bytes 0-15 are K [16g, 16g + 16), bytes 16-31 are K
//     [64 + 16g, 64 + 16g + 16);
//   scale_a / scale_b (byte 0): K block [32g, 32g + 32) of the lane's row or
//     column;
//   C: element q of lane l is row 4 (l / 16) + q, column l % 16.
// K block b of one MFMA is MXFP4 unit u + b, so a weight lane loads unit
// u + g whole (16 code bytes) and its scale byte, exactly as stored.  The
// activations (x for GEMM1, act for GEMM2) are bf16: every 32-element unit
// is split into two e4m3 terms with e8m0 scales, v = 2^e (hi + 2^-4 lo), where
// e is the least exponent with max|v| <= 448 * 2^e (no element rounds past
// e4m3's largest finite value, 448), hi = RNE(v 2^-e) and
// lo = RNE(16 (v 2^-e - hi)).  |v 2^-e - hi| is at most half a unit in the
// last place of hi (<= 16), so lo stays in range, and the two MFMAs (hi at
// scale 2^e, lo at 2^(e-4)) see v to about 2^-9 of the unit's largest
// element.  The split is made once per item while the rows are staged in
// LDS: per row the hi bytes, then the lo bytes (the 64 bytes per unit a bf16
// row takes), and the two scale bytes per unit in a small array beside them.

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kSxsMax = kXsBytes / 64;  // staged (row, unit) pairs: n x nu <= kXsBytes / 64

// Stage elements [e0, e0 + ne) of rows [0, n) as e4m3 hi / lo bytes (row r at
// xs + r (2 ne + kXsPad): hi at [0, ne), lo at [ne, 2 ne)) and their scale
// bytes (sxs[r * ne / 32 + unit]: hi exponent + 127 in the low byte, lo in
// the high byte), then a barrier.  The four 16-byte pieces of a unit fall on
// four adjacent lanes (ne / 8 pieces per row, a multiple of 4, and the block
// a multiple of 4 threads), which exchange their largest magnitude.
template <typename SrcRow>
__device__ __forceinline__ void stage_rows_f4(uint8_t* __restrict__ xs, uint16_t* __restrict__ sxs, int n, int e0,
                                              int ne, SrcRow src_row) {
  const int ppr = ne / 8, nu = ne / 32;
  const int RS = 2 * ne + kXsPad;
  for (int p = threadIdx.x; p < n * ppr; p += kDecThreads) {
    const int r = p / ppr, q = p - r * ppr;
    const u32x4 v = *reinterpret_cast<const u32x4*>(src_row(r) + e0 + 8 * q);
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    const uint32_t mb = __float_as_uint(m);
    // floor(log2 m) - 8, plus one where m's significand exceeds 1.75 (448 = 1.75 * 2^8)
    int e = (int)(mb >> 23) - 127 - 8 + ((mb & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    e = max(e, -123);  // lo's exponent e - 4 stays a valid e8m0 (zero rows: any)
    const float s = __uint_as_float((uint32_t)(127 - e) << 23);
    uint32_t hw[2], lw[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const float h0 = f[4 * w] * s, h1 = f[4 * w + 1] * s, h2 = f[4 * w + 2] * s, h3 = f[4 * w + 3] * s;
      int ph = __builtin_amdgcn_cvt_pk_fp8_f32(h0, h1, 0, false);
      ph = __builtin_amdgcn_cvt_pk_fp8_f32(h2, h3, ph, true);
      const float d0 = (h0 - __builtin_amdgcn_cvt_f32_fp8(ph, 0)) * 16.0f;
      const float d1 = (h1 - __builtin_amdgcn_cvt_f32_fp8(ph, 1)) * 16.0f;
      const float d2 = (h2 - __builtin_amdgcn_cvt_f32_fp8(ph, 2)) * 16.0f;
      const float d3 = (h3 - __builtin_amdgcn_cvt_f32_fp8(ph, 3)) * 16.0f;
      int pl = __builtin_amdgcn_cvt_pk_fp8_f32(d0, d1, 0, false);
      pl = __builtin_amdgcn_cvt_pk_fp8_f32(d2, d3, pl, true);
      hw[w] = (uint32_t)ph;
      lw[w] = (uint32_t)pl;
    }
    *reinterpret_cast<u32x2*>(xs + r * RS + 8 * q) = u32x2{hw[0], hw[1]};
    *reinterpret_cast<u32x2*>(xs + r * RS + ne + 8 * q) = u32x2{lw[0], lw[1]};
    if ((q & 3) == 0) sxs[r * nu + (q >> 2)] = (uint16_t)((e + 127) | ((e + 123) << 8));
  }
  lds_barrier();
}

// NB MFMA steps of 4 units from unit u (the last may hold fewer: units at or
// past u_end carry zero codes).  xr0 / xr1: the staged hi bytes of this
// lane's A rows (c and 16 + c), lo bytes lo_off further; sx0 / sx1 their
// scale pairs; ub: the chunk's first unit.  The code loads of all NB steps
// are issued before the first MFMA.
template <int NB, bool TWO>
__device__ __forceinline__ void f4_steps(f32x4& acc0, f32x4& acc1, const uint8_t* __restrict__ xr0,
                                         const uint8_t* __restrict__ xr1, const uint16_t* __restrict__ sx0,
                                         const uint16_t* __restrict__ sx1, int lo_off, const uint8_t* __restrict__ wrow,
                                         const uint8_t* __restrict__ srow, int u, int u_end, int ub, int g) {
  u32x4 cw[NB];
  uint32_t sb[NB];
#pragma unroll
  for (int s = 0; s < NB; ++s) {
    const int uw = u + 4 * s + g;
    const int ul = min(uw, u_end - 1);
    const u32x4 t = *reinterpret_cast<const u32x4*>(wrow + 16 * ul);
    cw[s] = uw < u_end ? t : u32x4{0u, 0u, 0u, 0u};
    sb[s] = srow[ul];
  }
#pragma unroll
  for (int s = 0; s < NB; ++s) {
    const int k0 = u + 4 * s - ub;                  // chunk unit of K block 0
    const int nl = min(4, u_end - (u + 4 * s));     // units in this step
    const int h = g >> 1;
    // K blocks past the step's units meet zero codes: read any staged bytes
    const int oa = 32 * (k0 + (h < nl ? h : 0)) + 16 * (g & 1);
    const int ob = 32 * (k0 + (2 + h < nl ? 2 + h : 0)) + 16 * (g & 1);
    const int us = k0 + (g < nl ? g : 0);
    const i32x8 bw = {(int)cw[s].x, (int)cw[s].y, (int)cw[s].z, (int)cw[s].w, 0, 0, 0, 0};
    {
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(xr0 + oa), a1 = *reinterpret_cast<const u32x4*>(xr0 + ob);
      const u32x4 l0 = *reinterpret_cast<const u32x4*>(xr0 + lo_off + oa);
      const u32x4 l1 = *reinterpret_cast<const u32x4*>(xr0 + lo_off + ob);
      const uint32_t sv = sx0[us];
      const i32x8 ah = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      const i32x8 al = {(int)l0.x, (int)l0.y, (int)l0.z, (int)l0.w, (int)l1.x, (int)l1.y, (int)l1.z, (int)l1.w};
      acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ah, bw, acc0, 0, 4, 0, (int)(sv & 0xFFu), 0, (int)sb[s]);
      acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(al, bw, acc0, 0, 4, 0, (int)(sv >> 8), 0, (int)sb[s]);
    }
    if constexpr (TWO) {
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(xr1 + oa), a1 = *reinterpret_cast<const u32x4*>(xr1 + ob);
      const u32x4 l0 = *reinterpret_cast<const u32x4*>(xr1 + lo_off + oa);
      const u32x4 l1 = *reinterpret_cast<const u32x4*>(xr1 + lo_off + ob);
      const uint32_t sv = sx1[us];
      const i32x8 ah = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      const i32x8 al = {(int)l0.x, (int)l0.y, (int)l0.z, (int)l0.w, (int)l1.x, (int)l1.y, (int)l1.z, (int)l1.w};
      acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ah, bw, acc1, 0, 4, 0, (int)(sv & 0xFFu), 0, (int)sb[s]);
      acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(al, bw, acc1, 0, 4, 0, (int)(sv >> 8), 0, (int)sb[s]);
    }
    __builtin_amdgcn_sched_barrier(0);  // the next step's LDS reads stay after these MFMAs
  }
}

// One wave's share of a decode item over staged e4m3 rows: units [u, u_end).
template <bool TWO>
__device__ __forceinline__ void tile_dot_f4(f32x4& acc0, f32x4& acc1, const uint8_t* __restrict__ xr0,
                                            const uint8_t* __restrict__ xr1, const uint16_t* __restrict__ sx0,
                                            const uint16_t* __restrict__ sx1, int lo_off, int ub,
                                            const void* __restrict__ w, const uint8_t* __restrict__ ws, int64_t rw,
                                            int kdim, int u, int u_end, int g) {
  const uint8_t* wrow = static_cast<const uint8_t*>(w) + rw * (kdim / 2);
  const uint8_t* srow = ws + rw * (kdim / 32);
  if constexpr (!TWO)
    for (; u + 32 <= u_end; u += 32) f4_steps<8, TWO>(acc0, acc1, xr0, xr1, sx0, sx1, lo_off, wrow, srow, u, u_end, ub, g);
  for (; u + 16 <= u_end; u += 16) f4_steps<4, TWO>(acc0, acc1, xr0, xr1, sx0, sx1, lo_off, wrow, srow, u, u_end, ub, g);
  if (u + 8 <= u_end) {
    f4_steps<2, TWO>(acc0, acc1, xr0, xr1, sx0, sx1, lo_off, wrow, srow, u, u_end, ub, g);
    u += 8;
  }
  for (; u < u_end; u += 4) f4_steps<1, TWO>(acc0, acc1, xr0, xr1, sx0, sx1, lo_off, wrow, srow, u, u_end, ub, g);
}

// The F4 counterpart of staged_dot: rows split into e4m3 terms chunk by
// chunk; every split's share of a chunk is a whole number of MFMA steps.
template <bool TWO, typename SrcRow>
__device__ __forceinline__ void staged_dot_f4(f32x4& acc0, f32x4& acc1, uint8_t* __restrict__ xs,
                                              uint16_t* __restrict__ sxs, int n, bool active, SrcRow src_row,
                                              const void* __restrict__ w, const uint8_t* __restrict__ ws, int64_t rw,
                                              int kdim, int ks, int S, int c, int g) {
  const int units = kdim / 32;
  const int kc = stage_chunk_units(n, units);
  for (int c0 = 0; c0 < units; c0 += kc) {
    const int nu = min(kc, units - c0);
    lds_barrier();  // every wave is done with the previous rows in xs
    stage_rows_f4(xs, sxs, n, 32 * c0, 32 * nu, src_row);
    if (active) {
      const int pc = ((nu + S - 1) / S + 3) & ~3;
      const int ub = c0 + min(nu, ks * pc), ue = c0 + min(nu, ks * pc + pc);
      const int RS = 64 * nu + kXsPad;
      const int r0 = c < n ? c : 0, r1 = 16 + c < n ? 16 + c : 0;
      tile_dot_f4<TWO>(acc0, acc1, xs + r0 * RS, xs + r1 * RS, sxs + r0 * nu, sxs + r1 * nu, 32 * nu, c0, w, ws, rw,
                       kdim, ub, ue, g);
    }
  }
}

// Sum of the S split partials of an item, in split order, into the waves of
// split 0 (red: kRedBytes of LDS; it may alias the staged rows, so the
// caller passes `staged` to wait for every wave's last read of them first).
template <bool TWO>
__device__ __forceinline__ void split_reduce(f32x4& acc0, f32x4& acc1, float* __restrict__ red, bool staged, int S,
                                             int ks, int wave, int lane) {
  if (S <= 1) return;
  if (staged) lds_barrier();
#pragma unroll
  for (int i = 0; i < 4; ++i) red[(wave * 8 + i) * 64 + lane] = acc0[i];
  if constexpr (TWO) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * 8 + 4 + i) * 64 + lane] = acc1[i];
  }
  __syncthreads();
  if (ks == 0) {
    for (int sp = 1; sp < S; ++sp) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc0[i] += red[((wave + sp) * 8 + i) * 64 + lane];
      if constexpr (TWO) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc1[i] += red[((wave + sp) * 8 + 4 + i) * 64 + lane];
      }
    }
  }
  __syncthreads();  // red is rewritten by the next item
}

// Where a decode item sits: its tile (expert, first grouped row, rows), this
// wave's column group and K split.  All fields are wave-uniform.
struct DecItem {
  int e, row0, nrows, cg, ks, S, u_begin, u_end;
  bool active, staged;
};

// Compaction inputs and outputs of the fused GEMM1 (ROUTES = true): every
// wave derives the route table itself from topk_ids and the expert map, and
// block 0 stores it for the kernels that follow and for the caller.
struct FusedRoutes {
  const int32_t* ids;
  const int32_t* emap;
  int N, Eg;
  int32_t* counts;
  int32_t* offsets;
  int32_t* s2r;
  int32_t* r2s;
};

// GEMM1 + silu_and_mul of one decode item (TWO: a tile of more than 16
// rows).  inv (ROUTES): lane r holds the slot of grouped row r.
template <bool MX, bool ROUTES, bool TWO, bool F4>
__device__ __forceinline__ void ffn1_item(const DecItem& d, const uint16_t* __restrict__ x, int K, int H, int F,
                                          const void* __restrict__ w1, const uint8_t* __restrict__ w1s,
                                          const int32_t* __restrict__ r2s, int inv, uint16_t* __restrict__ act,
                                          uint8_t* __restrict__ smem, uint16_t* __restrict__ sxs,
                                          int* __restrict__ xtok) {
  constexpr int U = dec_unroll1<MX>();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  // W1 row of this lane's MFMA column: gate row (c < 8) or up row
  const int64_t rw = (int64_t)d.e * 2 * F + (c >> 3) * F + d.cg * 8 + (c & 7);
  f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  if (d.staged) {
    if (wave == 0) {  // the x row (token) of each of the item's rows
      const int r = d.row0 + (lane < d.nrows ? lane : 0);
      int slot;
      if constexpr (ROUTES) slot = __shfl(inv, r, 64);
      else slot = r2s[r];
      if (lane < kDecBM) xtok[lane] = slot / K;
    }
    // the staging's first barrier makes xtok visible
    const auto xrow = [&](int r) { return x + (int64_t)xtok[r] * H; };
    if constexpr (F4) staged_dot_f4<TWO>(acc0, acc1, smem, sxs, d.nrows, d.active, xrow, w1, w1s, rw, H, d.ks, d.S, c, g);
    else staged_dot<MX, U, TWO>(acc0, acc1, smem, d.nrows, d.active, xrow, w1, w1s, rw, H, d.ks, d.S, c, g);
  } else if (d.active) {
    // rows past the tile's end reuse the first row; their results are dropped
    const int r0 = d.row0 + (c < d.nrows ? c : 0), r1 = d.row0 + (16 + c < d.nrows ? 16 + c : 0);
    int s0, s1;
    if constexpr (ROUTES) {
      s0 = __shfl(inv, r0, 64);
      s1 = __shfl(inv, r1, 64);
    } else {
      s0 = r2s[r0];
      s1 = TWO ? r2s[r1] : s0;
    }
    tile_dot<MX, U, TWO>(acc0, acc1, x + (int64_t)(s0 / K) * H, x + (int64_t)(s1 / K) * H, 0, w1, w1s, rw, H,
                         d.u_begin, d.u_end, g);
  }
  split_reduce<TWO>(acc0, acc1, reinterpret_cast<float*>(smem), d.staged, d.S, d.ks, wave, lane);
  if (d.ks == 0 && d.active) {
    const int n = d.cg * 8 + (c & 7);
#pragma unroll
    for (int h = 0; h < (TWO ? 2 : 1); ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * h + g * 4 + i;
        const float gate = h ? acc1[i] : acc0[i];
        const float up = __shfl_xor(gate, 8, 64);  // lane c ^ 8: the up value of the same column
        if (c < 8 && m < d.nrows) act[(int64_t)(d.row0 + m) * F + n] = f32_to_bf16_bits(silu_f32(gate) * up);
      }
    }
  }
}

// GEMM2 of one decode item.
template <bool MX, bool TWO, bool F4, typename YT>
__device__ __forceinline__ void ffn2_item(const DecItem& d, const uint16_t* __restrict__ act, int H, int F,
                                          const void* __restrict__ w2, const uint8_t* __restrict__ w2s,
                                          YT* __restrict__ y, uint8_t* __restrict__ smem, uint16_t* __restrict__ sxs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int64_t rw = (int64_t)d.e * H + d.cg * 16 + c;
  f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  if (d.staged) {
    const auto arow = [&](int r) { return act + (int64_t)(d.row0 + r) * F; };
    if constexpr (F4) staged_dot_f4<TWO>(acc0, acc1, smem, sxs, d.nrows, d.active, arow, w2, w2s, rw, F, d.ks, d.S, c, g);
    else staged_dot<MX, kDecUnroll, TWO>(acc0, acc1, smem, d.nrows, d.active, arow, w2, w2s, rw, F, d.ks, d.S, c, g);
  } else if (d.active) {
    // rows past the tile's end reuse the first row; their results are dropped
    const uint16_t* a0 = act + (int64_t)(d.row0 + (c < d.nrows ? c : 0)) * F;
    const uint16_t* a1 = act + (int64_t)(d.row0 + (16 + c < d.nrows ? 16 + c : 0)) * F;
    tile_dot<MX, kDecUnroll, TWO>(acc0, acc1, a0, a1, 0, w2, w2s, rw, F, d.u_begin, d.u_end, g);
  }
  split_reduce<TWO>(acc0, acc1, reinterpret_cast<float*>(smem), d.staged, d.S, d.ks, wave, lane);
  if (d.ks == 0 && d.active) {
    const int n = d.cg * 16 + c;
#pragma unroll
    for (int h = 0; h < (TWO ? 2 : 1); ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * h + g * 4 + i;
        const float v = h ? acc1[i] : acc0[i];
        if (m < d.nrows) {
          if constexpr (sizeof(YT) == 2) y[(int64_t)(d.row0 + m) * H + n] = f32_to_bf16_bits(v);
          else y[(int64_t)(d.row0 + m) * H + n] = v;
        }
      }
    }
  }
}

// GEMM1 + silu_and_mul for the decode regime.  Same operands as
// ffn1_stream_kernel; with ROUTES, counts/offsets/r2s are unused and the
// route table comes from `fr` (El <= 64, N <= 64).  A column group is 8 act
// columns: the 16 columns of one MFMA tile are their 8 gate rows of W1
// (lanes c < 8) and the matching 8 up rows (lanes c >= 8), so one MFMA
// yields both halves and a lane exchange (c <-> c + 8) pairs them for
// silu(gate) * up -- twice as many items as 16 gate + 16 up columns would
// give, which keeps every compute unit streaming when few tiles exist.
template <bool MX, bool ROUTES, bool F4>
__global__ __launch_bounds__(kDecThreads) void ffn1_decode_kernel(
    const uint16_t* __restrict__ x, int K, int H, int F, int El, const void* __restrict__ w1,
    const uint8_t* __restrict__ w1s, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ r2s, uint16_t* __restrict__ act, FusedRoutes fr) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[MX ? kXsBytes : kRedBytes];  // staged rows / partials
  __shared__ int xtok[kDecBM];
  __shared__ uint16_t sxs[F4 ? kSxsMax : 1];  // F4: scale bytes of the staged rows
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool small = ROUTES || El <= 64;  // uniform
  TileTab tab{};
  int inv = -1;  // ROUTES: slot of row `lane`
  if constexpr (ROUTES) {
    const WaveRoutes wr = wave_routes(fr.ids, fr.N, fr.emap, fr.Eg, El);
    tab = make_tile_tab(wr.cnt, wr.off, kDecBM);
    inv = wr.inv;
    if (blockIdx.x == 0 && wave == 0) {
      if (lane < El) {
        fr.counts[lane] = wr.cnt;
        fr.offsets[lane] = wr.off;
      }
      if (lane == 0) fr.offsets[El] = wr.R;
      if (lane < fr.N) {
        fr.s2r[lane] = wr.row;
        fr.r2s[lane] = wr.inv;
      }
    }
  } else if (small) {
    tab = load_tile_tab(counts, offsets, El, kDecBM);
  }
  const int tiles = small ? tab.total : count_tiles(counts, El, kDecBM);
  const int CG = F / 8, units = H / 32;  // column groups of 8 act columns
  DecItem d;
  d.S = decode_split(tiles, CG, units, gridDim.x, MX ? kSplitLatencyUnitsMX : kSplitLatencyUnits);
  const int cpb = kDecWaves / d.S;       // column groups per item
  const int ipt = (CG + cpb - 1) / cpb;  // items per tile
  const int items = tiles * ipt;
  d.ks = wave % d.S;
  const int cgl = wave / d.S;
  const int per = (units + d.S - 1) / d.S;
  d.u_begin = min(units, d.ks * per);
  d.u_end = min(units, d.u_begin + per);

  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int tile = it / ipt, cb = it % ipt;
    if (small) tab_find(tab, kDecBM, tile, d.e, d.row0, d.nrows);
    else find_tile(counts, offsets, El, kDecBM, tile, d.e, d.row0, d.nrows);
    d.cg = cb * cpb + cgl;
    d.active = d.cg < CG;
    d.staged = F4 || (MX && stage_item(d.S, d.nrows));  // uniform: one tile per item; F4 always stages
    if (d.nrows > 16) ffn1_item<MX, ROUTES, true, F4>(d, x, K, H, F, w1, w1s, r2s, inv, act, smem, sxs, xtok);
    else ffn1_item<MX, ROUTES, false, F4>(d, x, K, H, F, w1, w1s, r2s, inv, act, smem, sxs, xtok);
  }
}

// GEMM2 for the decode regime: y = W2[e] act over the grouped rows.
template <bool MX, typename YT, bool F4>
__global__ __launch_bounds__(kDecThreads) void ffn2_decode_kernel(
    const uint16_t* __restrict__ act, int H, int F, int El, const void* __restrict__ w2,
    const uint8_t* __restrict__ w2s, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    YT* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[MX ? kXsBytes : kRedBytes];  // staged rows / partials
  __shared__ uint16_t sxs[F4 ? kSxsMax : 1];  // F4: scale bytes of the staged rows
  const int wave = threadIdx.x >> 6;
  const bool small = El <= 64;  // uniform
  TileTab tab{};
  if (small) tab = load_tile_tab(counts, offsets, El, kDecBM);
  const int tiles = small ? tab.total : count_tiles(counts, El, kDecBM);
  const int CG = H / 16, units = F / 32;
  DecItem d;
  d.S = decode_split(tiles, CG, units, gridDim.x, MX ? kSplitLatencyUnitsMX : kSplitLatencyUnits);
  const int cpb = kDecWaves / d.S;
  const int ipt = (CG + cpb - 1) / cpb;
  const int items = tiles * ipt;
  d.ks = wave % d.S;
  const int cgl = wave / d.S;
  const int per = (units + d.S - 1) / d.S;
  d.u_begin = min(units, d.ks * per);
  d.u_end = min(units, d.u_begin + per);

  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int tile = it / ipt, cb = it % ipt;
    if (small) tab_find(tab, kDecBM, tile, d.e, d.row0, d.nrows);
    else find_tile(counts, offsets, El, kDecBM, tile, d.e, d.row0, d.nrows);
    d.cg = cb * cpb + cgl;
    d.active = d.cg < CG;
    d.staged = F4 || (MX && stage_item(d.S, d.nrows));  // uniform: one tile per item; F4 always stages
    if (d.nrows > 16) ffn2_item<MX, true, F4>(d, act, H, F, w2, w2s, y, smem, sxs);
    else ffn2_item<MX, false, F4>(d, act, H, F, w2, w2s, y, smem, sxs);
  }
}

// ---------------------------------------------------------------------------
// Generic persistent scheduler, kept as the A/B control of the b70 lab note
// "MTP1 M2 compact scheduler closure", timing paragraph (the generic path it
// measures against: a persistent grouped GEMM that scans every local expert
// and takes work from a global atomic counter, pinned to a 64-column N tile).
// Only the scheduling differs from the decode kernels above: the blocks are
// the same 16-wave blocks running the same item body (ffn1_item / ffn2_item:
// staging, K split, 32-row tiles, epilogue), but work item i is (local expert
// i / NT, 64-column N tile i % NT) for every local expert, routed or not,
// claimed from a global counter until none are left; an item walks its
// expert's rows tile by tile (none for an expert without rows).  The N tile
// fixes the split: 64 act columns are 8 GEMM1 column groups (S = 2), 64
// output columns 4 GEMM2 column groups (S = 4).  Results equal the decode
// kernels' within rounding (same tiles; the split may differ).

constexpr int kControlGrid = 256;  // persistent blocks: one per compute unit
constexpr int kControlCols = 64;   // the pinned N tile

__global__ void zero_counters_kernel(int32_t* __restrict__ w) { w[threadIdx.x] = 0; }

// One claim from *work, broadcast to the block (uniform).
__device__ __forceinline__ int claim_item(int32_t* __restrict__ work, int* __restrict__ slot) {
  if (threadIdx.x == 0) *slot = atomicAdd(work, 1);
  __syncthreads();
  const int it = *slot;
  __syncthreads();  // the slot is rewritten by the next claim
  return it;
}

template <bool MX>
__global__ __launch_bounds__(kDecThreads) void ffn1_control_kernel(
    const uint16_t* __restrict__ x, int K, int H, int F, int El, const void* __restrict__ w1,
    const uint8_t* __restrict__ w1s, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ r2s, uint16_t* __restrict__ act, int32_t* __restrict__ work) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[MX ? kXsBytes : kRedBytes];
  __shared__ int xtok[kDecBM];
  __shared__ int slot;
  const int wave = threadIdx.x >> 6;
  constexpr int cpb = kControlCols / 8;  // GEMM1 column groups per N tile
  const int CG = F / 8, units = H / 32, NT = F / kControlCols, total = El * NT;
  DecItem d;
  d.S = kDecWaves / cpb;
  d.ks = wave % d.S;
  const int cgl = wave / d.S;
  const int per = (units + d.S - 1) / d.S;
  d.u_begin = min(units, d.ks * per);
  d.u_end = min(units, d.u_begin + per);
  for (int it = claim_item(work, &slot); it < total; it = claim_item(work, &slot)) {
    d.e = it / NT;
    d.cg = (it % NT) * cpb + cgl;
    d.active = d.cg < CG;
    const int cnt = counts[d.e], base = offsets[d.e];
    for (int m0 = 0; m0 < cnt; m0 += kDecBM) {
      d.row0 = base + m0;
      d.nrows = min(kDecBM, cnt - m0);
      d.staged = MX && stage_item(d.S, d.nrows);
      if (d.nrows > 16) ffn1_item<MX, false, true, false>(d, x, K, H, F, w1, w1s, r2s, -1, act, smem, nullptr, xtok);
      else ffn1_item<MX, false, false, false>(d, x, K, H, F, w1, w1s, r2s, -1, act, smem, nullptr, xtok);
    }
  }
}

template <bool MX, typename YT>
__global__ __launch_bounds__(kDecThreads) void ffn2_control_kernel(
    const uint16_t* __restrict__ act, int H, int F, int El, const void* __restrict__ w2,
    const uint8_t* __restrict__ w2s, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    YT* __restrict__ y, int32_t* __restrict__ work) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[MX ? kXsBytes : kRedBytes];
  __shared__ int slot;
  const int wave = threadIdx.x >> 6;
  constexpr int cpb = kControlCols / 16;  // GEMM2 column groups per N tile
  const int CG = H / 16, units = F / 32, NT = H / kControlCols, total = El * NT;
  DecItem d;
  d.S = kDecWaves / cpb;
  d.ks = wave % d.S;
  const int cgl = wave / d.S;
  const int per = (units + d.S - 1) / d.S;
  d.u_begin = min(units, d.ks * per);
  d.u_end = min(units, d.u_begin + per);
  for (int it = claim_item(work, &slot); it < total; it = claim_item(work, &slot)) {
    d.e = it / NT;
    d.cg = (it % NT) * cpb + cgl;
    d.active = d.cg < CG;
    const int cnt = counts[d.e], base = offsets[d.e];
    for (int m0 = 0; m0 < cnt; m0 += kDecBM) {
      d.row0 = base + m0;
      d.nrows = min(kDecBM, cnt - m0);
      d.staged = MX && stage_item(d.S, d.nrows);
      if (d.nrows > 16) ffn2_item<MX, true, false>(d, act, H, F, w2, w2s, y, smem, nullptr);
      else ffn2_item<MX, false, false>(d, act, H, F, w2, w2s, y, smem, nullptr);
    }
  }
}

template <bool MX>
hipError_t launch_control(const uint16_t* x, int K, int H, int F, int El, const void* w1, const uint8_t* w1s,
                          const void* w2, const uint8_t* w2s, const int32_t* counts, const int32_t* offsets,
                          const int32_t* r2s, void* y, int y_dtype, uint16_t* act, int32_t* work,
                          hipStream_t stream) {
  hipLaunchKernelGGL(zero_counters_kernel, dim3(1), dim3(2), 0, stream, work);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((ffn1_control_kernel<MX>), dim3(kControlGrid), dim3(kDecThreads), 0, stream, x, K, H, F, El, w1,
                     w1s, counts, offsets, r2s, act, work);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (y_dtype == MOE_BF16)
    hipLaunchKernelGGL((ffn2_control_kernel<MX, uint16_t>), dim3(kControlGrid), dim3(kDecThreads), 0, stream, act, H,
                       F, El, w2, w2s, counts, offsets, static_cast<uint16_t*>(y), work + 1);
  else
    hipLaunchKernelGGL((ffn2_control_kernel<MX, float>), dim3(kControlGrid), dim3(kDecThreads), 0, stream, act, H, F,
                       El, w2, w2s, counts, offsets, static_cast<float*>(y), work + 1);
  return hipGetLastError();
}

template <bool MX, bool F4>
hipError_t launch_decode(const uint16_t* x, int K, int H, int F, int El, const void* w1, const uint8_t* w1s,
                         const void* w2, const uint8_t* w2s, const int32_t* counts, const int32_t* offsets,
                         const int32_t* r2s, void* y, int y_dtype, uint16_t* act, hipStream_t stream) {
  hipLaunchKernelGGL((ffn1_decode_kernel<MX, false, F4>), dim3(kDecGrid), dim3(kDecThreads), 0, stream, x, K, H, F,
                     El, w1, w1s, counts, offsets, r2s, act, FusedRoutes{});
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (y_dtype == MOE_BF16)
    hipLaunchKernelGGL((ffn2_decode_kernel<MX, uint16_t, F4>), dim3(kDecGrid), dim3(kDecThreads), 0, stream, act, H,
                       F, El, w2, w2s, counts, offsets, static_cast<uint16_t*>(y));
  else
    hipLaunchKernelGGL((ffn2_decode_kernel<MX, float, F4>), dim3(kDecGrid), dim3(kDecThreads), 0, stream, act, H, F,
                       El, w2, w2s, counts, offsets, static_cast<float*>(y));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Boundary fusion for decode batches (N = T*K <= kFusedMaxSlots slots, at
// most 64 local experts): the route compaction runs in the prologue of the
// GEMM1 kernel (ffn1_decode_kernel<MX, true>) and the combine in the tail of
// the GEMM2 kernel below, so the layer after the gate is two launches.

// One tile's operands for a wave of the fused GEMM2: the n (<= kFusedUnits)
// K units [u0, u0 + n) of its 16 weight rows and of the tile's act rows.
constexpr int kFusedUnits = 4;

template <bool MX>
struct TileOperands {
  WUnit<MX> b[kFusedUnits];
  bf16x8 a[kFusedUnits];
  int row0, nrows;

  // Every slot is loaded (units past the wave's range re-read unit
  // units - 1 and are not used), so no register keeps an older value.
  __device__ __forceinline__ void load(const TileTab& tab, int tile, const uint16_t* __restrict__ act,
                                       const void* __restrict__ w2, const uint8_t* __restrict__ w2s, int H, int F,
                                       int cg, int u0, int units, int c, int g) {
    int e = 0;
    tab_find(tab, 16, tile, e, row0, nrows);
    const uint16_t* ar = act + (int64_t)(row0 + (c < nrows ? c : 0)) * F;
    const int64_t rw = (int64_t)e * H + cg * 16 + c;
#pragma unroll
    for (int j = 0; j < kFusedUnits; ++j) b[j].load(w2, w2s, rw, F, min(u0 + j, units - 1), g);
#pragma unroll
    for (int j = 0; j < kFusedUnits; ++j) a[j] = unit_bf16(ar, min(u0 + j, units - 1), g);
  }

  __device__ __forceinline__ f32x4 mma(int n) const {
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < kFusedUnits; ++j)
      if (j < n) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], b[j].get(), acc, 0, 0, 0);
    return acc;
  }
};

// MXFP4: the batch layout of mx_batches for the (at most) four units
// [u0, u0 + n) of a wave: the lanes of group g hold unit u0 + g whole; a
// group past the wave's range (g >= n) loads a valid unit and feeds zeros.
template <>
struct TileOperands<true> {
  u32x4 cw;                // the 16 code bytes of this lane group's unit
  uint32_t sc;             // its scale byte
  bf16x8 a[kFusedUnits];   // its act elements, 8 per MFMA
  int row0, nrows;

  __device__ __forceinline__ void load(const TileTab& tab, int tile, const uint16_t* __restrict__ act,
                                       const void* __restrict__ w2, const uint8_t* __restrict__ w2s, int H, int F,
                                       int cg, int u0, int units, int c, int g) {
    int e = 0;
    tab_find(tab, 16, tile, e, row0, nrows);
    const uint16_t* ar = act + (int64_t)(row0 + (c < nrows ? c : 0)) * F;
    const int64_t rw = (int64_t)e * H + cg * 16 + c;
    const int u = min(u0 + g, units - 1);
    cw = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(w2) + rw * (F / 2) + 16 * u);
    sc = w2s[rw * (F / 32) + u];
#pragma unroll
    for (int j = 0; j < kFusedUnits; ++j) a[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ar + 32 * u + 8 * j));
  }

  __device__ __forceinline__ f32x4 mma(int n) const {
    const bool live = ((int)(threadIdx.x & 63) >> 4) < n;
    const bf16x8 zero = {};
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < kFusedUnits; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(live ? a[j] : zero, live ? widen_mx8(cw[j], sc) : zero, acc, 0, 0,
                                                    0);
    return acc;
  }
};

// GEMM2 with the combine in its tail.  Block b owns the 16 output columns
// [16 cg, 16 cg + 16), cg = b, b + grid, ..., across every tile: the 16 waves
// split the reduction 16 ways for one tile at a time, wave 0 adds the
// partials in split order and keeps the tile's y values, rounded to bf16, in
// LDS.  When all tiles are done the block forms
//   out[t, cols] = sum over k ascending, slot local, of w[t,k] * y[row, cols]
// from LDS -- the combine kernel's arithmetic -- so y never goes to memory.
// PIPE (at most kFusedUnits K units per wave, F <= 2048): the next tile's
// loads are in flight while the current tile is reduced.
template <bool MX, bool PIPE, typename OT>
__global__ __launch_bounds__(kDecThreads) void ffn2_combine_kernel(
    const uint16_t* __restrict__ act, int H, int F, int El, const void* __restrict__ w2,
    const uint8_t* __restrict__ w2s, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ s2r, const float* __restrict__ tw, int T, int K, OT* __restrict__ out) {
  __shared__ float red[kDecWaves][4][64];
  __shared__ float ys[kFusedMaxSlots][16];  // y[row, 16 cg + col]
  __shared__ int srow[kFusedMaxSlots];
  __shared__ float sw[kFusedMaxSlots];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int N = T * K;
  if ((int)threadIdx.x < N) {
    srow[threadIdx.x] = s2r[threadIdx.x];
    sw[threadIdx.x] = tw[threadIdx.x];
  }
  const TileTab tab = load_tile_tab(counts, offsets, El, 16);
  const int tiles = tab.total;
  const int CG = H / 16, units = F / 32;
  const int per = (units + kDecWaves - 1) / kDecWaves;
  const int u_begin = min(units, wave * per), u_end = min(units, u_begin + per);
  const int n = u_end - u_begin;  // this wave's K units (wave-uniform)
  __syncthreads();  // srow, sw

  // partial sums of one tile -> y values of its rows in ys
  auto finish_tile = [&](f32x4 acc, int row0, int nrows) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][i][lane] = acc[i];
    __syncthreads();
    if (wave == 0) {
      for (int sp = 1; sp < kDecWaves; ++sp) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += red[sp][i][lane];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = g * 4 + i;
        if (m < nrows) ys[row0 + m][c] = bf16_bits_to_f32(f32_to_bf16_bits(acc[i]));
      }
    }
    __syncthreads();  // red is rewritten by the next tile; ys complete
  };

  for (int cg = blockIdx.x; cg < CG; cg += gridDim.x) {
    if constexpr (PIPE) {
      // the operands of tile i + 1 are requested as soon as the MFMAs have
      // consumed those of tile i, so they arrive during tile i's reduction
      TileOperands<MX> op;
      if (tiles > 0) op.load(tab, 0, act, w2, w2s, H, F, cg, u_begin, units, c, g);
      for (int tile = 0; tile < tiles; ++tile) {
        const f32x4 acc = op.mma(n);
        const int row0 = op.row0, nrows = op.nrows;
        if (tile + 1 < tiles) op.load(tab, tile + 1, act, w2, w2s, H, F, cg, u_begin, units, c, g);
        finish_tile(acc, row0, nrows);
      }
    } else {
      for (int tile = 0; tile < tiles; ++tile) {
        int e = 0, row0 = 0, nrows = 0;
        tab_find(tab, 16, tile, e, row0, nrows);
        const uint16_t* ar = act + (int64_t)(row0 + (c < nrows ? c : 0)) * F;
        const int64_t rw = (int64_t)e * H + cg * 16 + c;
        finish_tile(tile_dot16<MX, kDecUnroll>(ar, w2, w2s, rw, F, u_begin, u_end, g), row0, nrows);
      }
    }
    for (int i = threadIdx.x; i < T * 16; i += kDecThreads) {
      const int t = i >> 4, col = i & 15;
      float a = 0.0f;
      for (int k = 0; k < K; ++k) {
        const int r = srow[t * K + k];
        if (r >= 0) a = fmaf(sw[t * K + k], ys[r][col], a);
      }
      const int64_t o = (int64_t)t * H + cg * 16 + col;
      if constexpr (sizeof(OT) == 2) out[o] = f32_to_bf16_bits(a);
      else out[o] = a;
    }
    __syncthreads();  // ys is rewritten for the next column group
  }
}

template <bool MX>
hipError_t launch_fused_k(const uint16_t* x, int64_t T, int K, int H, int F, const int32_t* ids, const float* tw,
                          const int32_t* emap, int Eg, int El, const void* w1, const uint8_t* w1s, const void* w2,
                          const uint8_t* w2s, int32_t* counts, int32_t* offsets, int32_t* s2r, int32_t* r2s,
                          void* out, int out_dtype, uint16_t* act, hipStream_t stream) {
  const FusedRoutes fr{ids, emap, (int)(T * K), Eg, counts, offsets, s2r, r2s};
  if (MX && mxfp4_mma_mode() == MOE_MXFP4_MMA_F8F6F4)
    hipLaunchKernelGGL((ffn1_decode_kernel<MX, true, MX>), dim3(kDecGrid), dim3(kDecThreads), 0, stream, x, K, H, F,
                       El, w1, w1s, static_cast<const int32_t*>(nullptr), static_cast<const int32_t*>(nullptr),
                       static_cast<const int32_t*>(nullptr), act, fr);
  else
    hipLaunchKernelGGL((ffn1_decode_kernel<MX, true, false>), dim3(kDecGrid), dim3(kDecThreads), 0, stream, x, K, H,
                       F, El, w1, w1s, static_cast<const int32_t*>(nullptr), static_cast<const int32_t*>(nullptr),
                       static_cast<const int32_t*>(nullptr), act, fr);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || T == 0) return err;  // T == 0: counts and offsets (zeros) are written
  const unsigned grid = (unsigned)min(kDecGrid, H / 16);
  const bool pipe = (F / 32 + kDecWaves - 1) / kDecWaves <= kFusedUnits;
  const dim3 g(grid), b(kDecThreads);
  if (out_dtype == MOE_BF16) {
    uint16_t* o = static_cast<uint16_t*>(out);
    if (pipe)
      hipLaunchKernelGGL((ffn2_combine_kernel<MX, true, uint16_t>), g, b, 0, stream, act, H, F, El, w2, w2s, counts,
                         offsets, s2r, tw, (int)T, K, o);
    else
      hipLaunchKernelGGL((ffn2_combine_kernel<MX, false, uint16_t>), g, b, 0, stream, act, H, F, El, w2, w2s, counts,
                         offsets, s2r, tw, (int)T, K, o);
  } else {
    float* o = static_cast<float*>(out);
    if (pipe)
      hipLaunchKernelGGL((ffn2_combine_kernel<MX, true, float>), g, b, 0, stream, act, H, F, El, w2, w2s, counts,
                         offsets, s2r, tw, (int)T, K, o);
    else
      hipLaunchKernelGGL((ffn2_combine_kernel<MX, false, float>), g, b, 0, stream, act, H, F, El, w2, w2s, counts,
                         offsets, s2r, tw, (int)T, K, o);
  }
  return hipGetLastError();
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
#undef MOE_FFN_CASE
  if constexpr (MX) {
    if (mxfp4_mma_mode() == MOE_MXFP4_MMA_F8F6F4)
      return launch_decode<true, true>(x, K, H, F, El, w1, w1s, w2, w2s, counts, offsets, r2s, y, y_dtype, act, stream);
  }
  return launch_decode<MX, false>(x, K, H, F, El, w1, w1s, w2, w2s, counts, offsets, r2s, y, y_dtype, act, stream);
}

}  // namespace

namespace {
std::atomic<int> g_mxfp4_mma{MOE_MXFP4_MMA_BF16};
}  // namespace

int mxfp4_mma_mode() { return g_mxfp4_mma.load(std::memory_order_relaxed); }
void set_mxfp4_mma_mode(int mode) { g_mxfp4_mma.store(mode, std::memory_order_relaxed); }

size_t grouped_ffn_workspace_bytes(int64_t N, int H, int F, int El, int w_dtype) {
  (void)H;
  (void)El;
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
  if (w_dtype == MOE_BF16_TILED || (w_dtype == MOE_BF16 && tiled_ffn_applicable(N, H, F, El)))
    return launch_tiled_ffn(xb, T, N, K, H, F, El, static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w2),
                            w_dtype == MOE_BF16_TILED, counts, offsets, r2s, y, y_dtype, act, stream);
  if (w_dtype == MOE_MXFP4)
    return dispatch_stream<true>(xb, N, K, H, F, El, w1, w1s, w2, w2s, counts, offsets, r2s, y, y_dtype, act, stream);
  return dispatch_stream<false>(xb, N, K, H, F, El, w1, nullptr, w2, nullptr, counts, offsets, r2s, y, y_dtype, act,
                                stream);
}

hipError_t launch_grouped_ffn_control(const void* x, int64_t T, int K, int H, int F, int El, const void* w1,
                                      const uint8_t* w1s, const void* w2, const uint8_t* w2s, int w_dtype,
                                      const int32_t* counts, const int32_t* offsets, const int32_t* r2s, void* y,
                                      int y_dtype, void* workspace, hipStream_t stream) {
  const int64_t N = T * K;
  uint16_t* act = static_cast<uint16_t*>(workspace);
  int32_t* work = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) +
                                             (grouped_ffn_workspace_bytes(N, H, F, El, w_dtype) + 255) / 256 * 256);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (w_dtype == MOE_MXFP4)
    return launch_control<true>(xb, K, H, F, El, w1, w1s, w2, w2s, counts, offsets, r2s, y, y_dtype, act, work, stream);
  return launch_control<false>(xb, K, H, F, El, w1, nullptr, w2, nullptr, counts, offsets, r2s, y, y_dtype, act, work,
                               stream);
}

size_t grouped_ffn_control_workspace_bytes(int64_t N, int H, int F, int El, int w_dtype) {
  return (grouped_ffn_workspace_bytes(N, H, F, El, w_dtype) + 255) / 256 * 256 + 256;
}

size_t fused_experts_workspace_bytes(int64_t N, int F) { return (size_t)N * (size_t)F * sizeof(uint16_t); }

hipError_t launch_fused_experts(const uint16_t* x, int64_t T, int K, int H, int F, const int32_t* ids,
                                const float* topk_weights, const int32_t* emap, int Eg, int El, const void* w1,
                                const uint8_t* w1s, const void* w2, const uint8_t* w2s, int w_dtype,
                                int32_t* counts, int32_t* offsets, int32_t* s2r, int32_t* r2s, void* out,
                                int out_dtype, void* workspace, hipStream_t stream) {
  uint16_t* act = static_cast<uint16_t*>(workspace);
  if (w_dtype == MOE_MXFP4)
    return launch_fused_k<true>(x, T, K, H, F, ids, topk_weights, emap, Eg, El, w1, w1s, w2, w2s, counts, offsets,
                                s2r, r2s, out, out_dtype, act, stream);
  return launch_fused_k<false>(x, T, K, H, F, ids, topk_weights, emap, Eg, El, w1, w1s, w2, w2s, counts, offsets,
                               s2r, r2s, out, out_dtype, act, stream);
}

}  // namespace moe
