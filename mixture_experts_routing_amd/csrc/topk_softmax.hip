// Fused softmax + top-k gate for gfx950.
//
// Source: page "Upstream Reference: Deep-Spark xllm + vllm", section "Call
// Chain: MoE topk_softmax on BI-V100": one fused op turns router logits into
// routing weights, expert ids and a token-expert index map.  The CUDA kernel
// named there (one warp-sized group per row, power-of-two expert counts
// favoured) is prior art only; this kernel is laid out for 64-wide CDNA
// wavefronts and handles any E up to 1280.
//
// Layout: a row of E logits is split over G adjacent lanes of a wavefront
// (G = 1..64), lane q holding V contiguous experts [q*V, q*V+V), so one
// wavefront serves 64/G rows and its loads are fully coalesced.  Each logit
// becomes one integer key that orders by (value desc, index asc):
//   bf16: int32  (two's-complement of the sign-magnitude value) << 16 | (0xFFFF - j)
//   f32 : int64  (two's-complement of the sign-magnitude value) << 32 | (0xFFFFFFFF - j)
// (-0 and +0 map to the same value field, so they tie and the lower index
// wins).  Keys are unique within a row, so "max" is a single integer max.
// Each lane sorts its keys (Batcher odd-even merge network, registers only);
// then K rounds of a DPP group max pick the row's best key and the winning
// lane pops its head.  The softmax denominator is a fixed-order tree sum of
// exp2 terms; the K chosen weights use the accurate expf and an IEEE divide.
#include "moe_internal.h"

#include <limits.h>

namespace moe {
namespace {

template <typename LT>
struct Keys;

template <>
struct Keys<uint16_t> {  // bf16 logits stored as raw bits
  using Key = int32_t;
  static constexpr Key kMin = INT32_MIN;  // below every real key
  __device__ __forceinline__ static Key make(uint32_t bits16, int j) {
    int32_t mag = (int32_t)(bits16 & 0x7FFFu);
    int32_t tc = (bits16 & 0x8000u) ? -mag : mag;
    return (Key)(((uint32_t)tc << 16) | (uint32_t)(0xFFFF - j));
  }
  __device__ __forceinline__ static float value(Key k) {
    int32_t tc = k >> 16;
    uint32_t bits = tc < 0 ? (0x8000u | (uint32_t)(-tc)) : (uint32_t)tc;
    return __uint_as_float(bits << 16);
  }
  __device__ __forceinline__ static int index(Key k) { return 0xFFFF - (int)(k & 0xFFFF); }
  __device__ __forceinline__ static float to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
};

template <>
struct Keys<float> {  // f32 logits, handled through their bits
  using Key = int64_t;
  static constexpr Key kMin = INT64_MIN;
  __device__ __forceinline__ static Key make(uint32_t bits, int j) {
    int64_t mag = (int64_t)(bits & 0x7FFFFFFFu);
    int64_t tc = (bits & 0x80000000u) ? -mag : mag;
    return (Key)(((uint64_t)tc << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j));
  }
  __device__ __forceinline__ static float value(Key k) {
    int64_t tc = k >> 32;
    uint32_t bits = tc < 0 ? (0x80000000u | (uint32_t)(-tc)) : (uint32_t)tc;
    return __uint_as_float(bits);
  }
  __device__ __forceinline__ static int index(Key k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }
  __device__ __forceinline__ static float to_f32(uint32_t bits) { return __uint_as_float(bits); }
};

template <int G, typename Key>
__device__ __forceinline__ Key group_max(Key k) {
  if constexpr (sizeof(Key) == 4) return group_max_i32<G>(k);
  else return group_max_i64<G>(k);
}

// Descending compare-exchange: larger key to the lower position.
template <typename Key>
__device__ __forceinline__ void cx(Key& a, Key& b) {
  Key hi = a > b ? a : b;
  Key lo = a > b ? b : a;
  a = hi;
  b = lo;
}

constexpr int pow2_ceil(int n) { int p = 1; while (p < n) p <<= 1; return p; }

// Batcher odd-even merge sort over n registers (padded to a power of two;
// comparators that touch a padding position are skipped, which is exact
// because every comparator of this network moves the larger key to the
// lower position and padding would hold the smallest key).
template <int N, typename Key>
__device__ __forceinline__ void sort_desc(Key (&k)[N]) {
  constexpr int P2 = pow2_ceil(N);
#pragma unroll
  for (int p = 1; p < P2; p <<= 1) {
#pragma unroll
    for (int kk = p; kk >= 1; kk >>= 1) {
#pragma unroll
      for (int j = kk % p; j + kk < P2; j += 2 * kk) {
#pragma unroll
        for (int i = 0; i < kk; ++i) {
          const int a = i + j, b = i + j + kk;
          if (b < N && (a / (2 * p)) == (b / (2 * p))) cx(k[a], k[b]);
        }
      }
    }
  }
}

// Loads the V raw logits [j0, j0+V) of row `row` (bits in uint32 lanes).
template <typename LT, int V>
__device__ __forceinline__ void load_row_chunk(const LT* __restrict__ row, int j0, int E, bool vec_ok,
                                               uint32_t (&raw)[V]) {
  if constexpr (sizeof(LT) == 2) {
    static_assert(V % 2 == 0, "bf16 chunks are loaded as pairs");
    if (vec_ok) {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(row + j0);
      if constexpr (V % 8 == 0) {
#pragma unroll
        for (int i = 0; i < V / 8; ++i) {
          u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + i);
          raw[8 * i + 0] = q.x & 0xFFFFu; raw[8 * i + 1] = q.x >> 16;
          raw[8 * i + 2] = q.y & 0xFFFFu; raw[8 * i + 3] = q.y >> 16;
          raw[8 * i + 4] = q.z & 0xFFFFu; raw[8 * i + 5] = q.z >> 16;
          raw[8 * i + 6] = q.w & 0xFFFFu; raw[8 * i + 7] = q.w >> 16;
        }
      } else {
#pragma unroll
        for (int i = 0; i < V / 4; ++i) {
          u32x2 q = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p) + i);
          raw[4 * i + 0] = q.x & 0xFFFFu; raw[4 * i + 1] = q.x >> 16;
          raw[4 * i + 2] = q.y & 0xFFFFu; raw[4 * i + 3] = q.y >> 16;
        }
        if constexpr (V % 4) {
          uint32_t q = __builtin_nontemporal_load(p + V / 2 - 1);
          raw[V - 2] = q & 0xFFFFu;
          raw[V - 1] = q >> 16;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) raw[i] = (j0 + i < E) ? (uint32_t)row[j0 + i] : 0u;
    }
  } else {
    if (vec_ok && V % 4 == 0) {
      const u32x4* p = reinterpret_cast<const u32x4*>(row + j0);
#pragma unroll
      for (int i = 0; i < V / 4; ++i) {
        u32x4 q = __builtin_nontemporal_load(p + i);
        raw[4 * i + 0] = q.x; raw[4 * i + 1] = q.y; raw[4 * i + 2] = q.z; raw[4 * i + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) raw[i] = (j0 + i < E) ? __float_as_uint(row[j0 + i]) : 0u;
    }
  }
}

constexpr int kBlock = 256;

// SIG: sigmoid scoring -- weight = sigmoid(logit), no softmax denominator.
template <typename LT, int G, int V, int KMAX, bool SIG>
__global__ __launch_bounds__(kBlock) void topk_softmax_kernel(
    const LT* __restrict__ logits, int64_t T, int E, int K, int renorm, int vec_ok,
    float* __restrict__ w_out, int32_t* __restrict__ id_out, int32_t* __restrict__ tei_out) {
  using Tr = Keys<LT>;
  using Key = typename Tr::Key;
  constexpr int L = V < KMAX ? V : KMAX;     // keys a lane can ever contribute
  constexpr int RPL = (KMAX + G - 1) / G;    // output ranks per lane
  constexpr int ROWS = kBlock / G;

  const int lane_g = threadIdx.x % G;
  const int64_t t = (int64_t)blockIdx.x * ROWS + threadIdx.x / G;
  const bool row_ok = t < T;
  const int j0 = lane_g * V;
  const bool full = row_ok && (j0 + V <= E);

  uint32_t raw[V];
  if (row_ok) {
    load_row_chunk<LT, V>(logits + t * (int64_t)E, j0, E, vec_ok && full, raw);
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) raw[i] = 0u;
  }

  Key k[V];
#pragma unroll
  for (int i = 0; i < V; ++i) k[i] = (row_ok && j0 + i < E) ? Tr::make(raw[i], j0 + i) : Tr::kMin;
  sort_desc<V>(k);

  // K rounds: the group max is the row's next-best key; its owner pops it.
  // After round r at most K-1-r more pops follow, so only the first
  // KMAX-1-r positions of a lane's list still matter.
  Key top[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    if (r < K) {
      const Key m = group_max<G>(k[0]);
      top[r] = m;
      const bool win = (k[0] == m);
#pragma unroll
      for (int i = 0; i < L; ++i) {
        if (i < KMAX - 1 - r) {
          const Key nxt = (i + 1 < L) ? k[i + 1] : Tr::kMin;
          k[i] = win ? nxt : k[i];
        }
      }
    } else {
      top[r] = Tr::kMin;
    }
  }

  // softmax denominator: fixed-order pairwise tree inside the lane, then the
  // DPP group sum
  const float mx = Tr::value(top[0]);
  float denom = 1.0f;
  if constexpr (!SIG) {
    constexpr float kLog2e = 1.4426950408889634f;
    float ex[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const float v = Tr::to_f32(raw[i]);
      ex[i] = (row_ok && j0 + i < E) ? __builtin_amdgcn_exp2f((v - mx) * kLog2e) : 0.0f;
    }
#pragma unroll
    for (int w = 1; w < V; w <<= 1) {
#pragma unroll
      for (int i = 0; i + w < V; i += 2 * w) ex[i] += ex[i + w];
    }
    denom = group_sum_f32<G>(ex[0]);
  }

  // each lane finishes ranks lane_g, lane_g + G, ...
  Key mine[RPL];
  float e_mine[RPL];
  float part = 0.0f;
#pragma unroll
  for (int c = 0; c < RPL; ++c) {
    Key kk = Tr::kMin;
#pragma unroll
    for (int r = c * G; r < (c + 1) * G && r < KMAX; ++r) kk = (lane_g + c * G == r) ? top[r] : kk;
    mine[c] = kk;
    const int q = lane_g + c * G;
    if constexpr (SIG) e_mine[c] = (q < K) ? 1.0f / (1.0f + expf(-Tr::value(kk))) : 0.0f;
    else e_mine[c] = (q < K) ? expf(Tr::value(kk) - mx) : 0.0f;
    part += e_mine[c];
  }
  float norm = denom;
  if (renorm) norm = group_sum_f32<G>(part);
  (void)mx;

  if (row_ok) {
#pragma unroll
    for (int c = 0; c < RPL; ++c) {
      const int q = lane_g + c * G;
      if (q < K) {
        const int64_t o = t * K + q;
        w_out[o] = (SIG && !renorm) ? e_mine[c] : e_mine[c] / norm;
        id_out[o] = Tr::index(mine[c]);
        if (tei_out) tei_out[o] = (int32_t)((int64_t)q * T + t);
      }
    }
  }
}

template <typename LT, int G, int V, int KMAX, bool SIG>
hipError_t launch_cfg(const LT* logits, int64_t T, int E, int K, int renorm, float* w, int32_t* ids,
                      int32_t* tei, hipStream_t stream) {
  constexpr int ROWS = kBlock / G;
  const int64_t blocks = (T + ROWS - 1) / ROWS;
  // vector loads need the lane's chunk start aligned: row stride and chunk
  // size multiples of the vector width, and an aligned base pointer
  const int elt = (int)sizeof(LT);
  const int vec_bytes = (elt == 2) ? ((V % 8 == 0) ? 16 : 8) : 16;
  const bool vec_ok = ((E * elt) % vec_bytes == 0) && ((V * elt) % vec_bytes == 0) &&
                      ((uintptr_t)logits % vec_bytes == 0);
  hipLaunchKernelGGL((topk_softmax_kernel<LT, G, V, KMAX, SIG>), dim3((unsigned)blocks), dim3(kBlock), 0,
                     stream, logits, T, E, K, renorm, (int)vec_ok, w, ids, tei);
  return hipGetLastError();
}

template <typename LT, int KMAX, bool SIG>
hipError_t dispatch_gv(const LT* logits, int64_t T, int E, int K, int renorm, float* w, int32_t* ids,
                       int32_t* tei, hipStream_t stream) {
#define MOE_GATE_CASE(GG, VV) return launch_cfg<LT, GG, VV, KMAX, SIG>(logits, T, E, K, renorm, w, ids, tei, stream)
  if (E <= 8) MOE_GATE_CASE(1, 8);
  if (E <= 16) MOE_GATE_CASE(1, 16);
  if (E <= 20) MOE_GATE_CASE(1, 20);
  int G = 1;
  while (G * 20 < E) G <<= 1;
  const int v = (E + G - 1) / G;  // in (10, 20]
  const bool v16 = v <= 16;
  switch (G) {
    case 2: if (v16) MOE_GATE_CASE(2, 16); MOE_GATE_CASE(2, 20);
    case 4: if (v16) MOE_GATE_CASE(4, 16); MOE_GATE_CASE(4, 20);
    case 8: if (v16) MOE_GATE_CASE(8, 16); MOE_GATE_CASE(8, 20);
    case 16: if (v16) MOE_GATE_CASE(16, 16); MOE_GATE_CASE(16, 20);
    case 32: if (v16) MOE_GATE_CASE(32, 16); MOE_GATE_CASE(32, 20);
    case 64: if (v16) MOE_GATE_CASE(64, 16); MOE_GATE_CASE(64, 20);
    default: return hipErrorInvalidValue;
  }
#undef MOE_GATE_CASE
}


// ---------------------------------------------------------------------------
// Fast path: bf16 logits, K <= 8, E = 8*V with V in {8, 12, 16, 20, 24}, rows
// 16-byte (V % 8 == 0) or 8-byte aligned.  Eight lanes per row (32 rows per
// 256-thread block), no bounds checks in the body, keys built two at a time
// with packed 16-bit ALU ops, and only each lane's top 8 keys kept (two or
// three sorting networks and bitonic merges instead of a full sort).

typedef short s16x2 __attribute__((ext_vector_type(2)));

// descending Batcher sort of 8 registers (19 comparators)
__device__ __forceinline__ void sort8_desc(int32_t* k) {
  cx(k[0], k[1]); cx(k[2], k[3]); cx(k[4], k[5]); cx(k[6], k[7]);
  cx(k[0], k[2]); cx(k[1], k[3]); cx(k[4], k[6]); cx(k[5], k[7]);
  cx(k[1], k[2]); cx(k[5], k[6]);
  cx(k[0], k[4]); cx(k[1], k[5]); cx(k[2], k[6]); cx(k[3], k[7]);
  cx(k[2], k[4]); cx(k[3], k[5]);
  cx(k[1], k[2]); cx(k[3], k[4]); cx(k[5], k[6]);
}
// descending sort of 4 registers (5 comparators)
__device__ __forceinline__ void sort4_desc(int32_t* k) {
  cx(k[0], k[1]); cx(k[2], k[3]); cx(k[0], k[2]); cx(k[1], k[3]); cx(k[1], k[2]);
}
// a[0..8) sorted desc <- top 8 of (a, b), b[0..nb) sorted desc (nb <= 8):
// max(a[i], b[7-i]) is a bitonic sequence holding the 8 largest; a
// half-cleaner network then sorts it.
__device__ __forceinline__ void merge_top8(int32_t* a, const int32_t* b, int nb) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = 7 - i;
    if (j < nb) a[i] = max(a[i], b[j]);
  }
  cx(a[0], a[4]); cx(a[1], a[5]); cx(a[2], a[6]); cx(a[3], a[7]);
  cx(a[0], a[2]); cx(a[1], a[3]); cx(a[4], a[6]); cx(a[5], a[7]);
  cx(a[0], a[1]); cx(a[2], a[3]); cx(a[4], a[5]); cx(a[6], a[7]);
}

// Row t of the bf16 fast gate on the 8-lane group of this thread (lane q =
// threadIdx.x % 8 holds experts [qV, qV+V) and finishes rank q).  Stores the
// row's outputs and returns this lane's chosen expert id, or -1 (q >= K or
// t >= T).
template <int V, bool SIG>
__device__ __forceinline__ int gate8_group(const uint16_t* __restrict__ logits, int64_t T, int K, int renorm,
                                           int64_t t, float* __restrict__ w_out, int32_t* __restrict__ id_out,
                                           int32_t* __restrict__ tei_out) {
  constexpr int G = 8, E = G * V, W = V / 2;  // W: 32-bit words per lane
  const int q = threadIdx.x & 7;
  const bool row_ok = t < T;
  const int64_t tc = row_ok ? t : 0;  // out-of-range rows read row 0, store nothing

  uint32_t wd[W];
  const uint32_t* src = reinterpret_cast<const uint32_t*>(logits + tc * E + q * V);
  if constexpr (V % 8 == 0) {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + i);
      wd[4 * i] = v.x; wd[4 * i + 1] = v.y; wd[4 * i + 2] = v.z; wd[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < W / 2; ++i) {
      const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src) + i);
      wd[2 * i] = v.x; wd[2 * i + 1] = v.y;
    }
  }

  // keys: (two's-complement value << 16) | (0xFFFF - index), two per word.
  // sign-magnitude -> two's complement per 16-bit half: (mag ^ s) - s with
  // s = 0 or -1; -0 becomes 0.
  int32_t key[V];
  const int j0 = q * V;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const s16x2 h = __builtin_bit_cast(s16x2, wd[i]);
    const s16x2 sg = h >> (s16x2){15, 15};
    const s16x2 mag = __builtin_bit_cast(s16x2, wd[i] & 0x7FFF7FFFu);
    const uint32_t tcv = __builtin_bit_cast(uint32_t, (s16x2)((mag ^ sg) - sg));
    key[2 * i] = (int32_t)((tcv << 16) | (uint32_t)(0xFFFF - (j0 + 2 * i)));
    key[2 * i + 1] = (int32_t)((tcv & 0xFFFF0000u) | (uint32_t)(0xFFFF - (j0 + 2 * i + 1)));
  }

  // this lane's 8 best keys, sorted
  int32_t k[8];
  if constexpr (V == 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) k[i] = key[i];
    sort8_desc(k);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) k[i] = key[i];
    sort8_desc(k);
    if constexpr (V >= 16) {
      sort8_desc(key + 8);
      merge_top8(k, key + 8, 8);
    }
    if constexpr (V == 12 || V == 20) {
      sort4_desc(key + V - 4);
      merge_top8(k, key + V - 4, 4);
    }
    if constexpr (V == 24) {
      sort8_desc(key + 16);
      merge_top8(k, key + 16, 8);
    }
  }

  // K rounds of an 8-lane max; the owner pops.  After round r only the first
  // 7-r entries can still be needed.
  int32_t top[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if (r < K) {
      const int32_t m = group_max_i32<G>(k[0]);
      top[r] = m;
      const bool win = (k[0] == m);
#pragma unroll
      for (int i = 0; i < 7 - r; ++i) k[i] = win ? k[i + 1] : k[i];
    } else {
      top[r] = INT32_MIN;
    }
  }

  // softmax denominator over the lane's V values, pairwise, then the group
  const float mx = Keys<uint16_t>::value(top[0]);
  float denom = 1.0f;
  if constexpr (!SIG) {
    constexpr float kLog2e = 1.4426950408889634f;
    float ex[V];
#pragma unroll
    for (int i = 0; i < W; ++i) {
      ex[2 * i] = __builtin_amdgcn_exp2f((__uint_as_float(wd[i] << 16) - mx) * kLog2e);
      ex[2 * i + 1] = __builtin_amdgcn_exp2f((__uint_as_float(wd[i] & 0xFFFF0000u) - mx) * kLog2e);
    }
#pragma unroll
    for (int w = 1; w < V; w <<= 1) {
#pragma unroll
      for (int i = 0; i + w < V; i += 2 * w) ex[i] += ex[i + w];
    }
    denom = group_sum_f32<G>(ex[0]);
  }

  // lane q finishes rank q
  int32_t mine = top[0];
#pragma unroll
  for (int r = 1; r < 8; ++r) mine = (q == r) ? top[r] : mine;
  const float v = Keys<uint16_t>::value(mine);
  float e;
  if constexpr (SIG) e = (q < K) ? 1.0f / (1.0f + expf(-v)) : 0.0f;
  else e = (q < K) ? expf(v - mx) : 0.0f;
  const float norm = renorm ? group_sum_f32<G>(e) : denom;
  if (row_ok && q < K) {
    const int64_t o = t * K + q;
    const int id = Keys<uint16_t>::index(mine);
    w_out[o] = (SIG && !renorm) ? e : e / norm;
    id_out[o] = id;
    if (tei_out) tei_out[o] = (int32_t)((int64_t)q * T + t);
    return id;
  }
  return -1;
}

template <int V, bool SIG>
__global__ __launch_bounds__(kBlock) void topk8_bf16_kernel(const uint16_t* __restrict__ logits, int64_t T, int K,
                                                            int renorm, float* __restrict__ w_out,
                                                            int32_t* __restrict__ id_out,
                                                            int32_t* __restrict__ tei_out) {
  const int64_t t = (int64_t)blockIdx.x * (kBlock / 8) + (threadIdx.x >> 3);
  gate8_group<V, SIG>(logits, T, K, renorm, t, w_out, id_out, tei_out);
}

// The gate with the count pass of the route compaction fused in (K = 8): a
// block of kCompactBlockSlots threads takes 128 rows, so thread i ends up
// holding slot b * kCompactBlockSlots + i -- the slot the compaction's count
// kernel gives that thread -- and does that kernel's work on it: the slot's
// rank among equal local ids of its block (in slot order) parked in s2r, and
// the block's per-expert counts in block_counts[b][El].  The compaction's
// scan/scatter phase follows as a separate launch.
template <int V, bool SIG>
__global__ __launch_bounds__(kCompactBlockSlots) void topk8_count_kernel(
    const uint16_t* __restrict__ logits, int64_t T, int renorm, float* __restrict__ w_out,
    int32_t* __restrict__ id_out, int32_t* __restrict__ tei_out, const int32_t* __restrict__ emap, int Eg, int El,
    int32_t* __restrict__ block_counts, int32_t* __restrict__ s2r) {
  extern __shared__ int run[];  // [kCompactWaves][El]: per-wave counts, then their prefix
  for (int i = threadIdx.x; i < kCompactWaves * El; i += kCompactBlockSlots) run[i] = 0;
  const int64_t t = (int64_t)blockIdx.x * (kCompactBlockSlots / 8) + (threadIdx.x >> 3);
  const int id = gate8_group<V, SIG>(logits, T, 8, renorm, t, w_out, id_out, tei_out);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l = id >= 0 ? local_expert(id, emap, Eg, El) : -1;
  int below, total;
  wave_group_rank(l, El, below, total);
  __syncthreads();  // run is zero
  int* runw = run + wave * El;
  if (l >= 0 && below == total - 1) runw[l] = total;  // one writer per distinct id of the wave
  __syncthreads();
  prefix_over_compact_waves(run, El, block_counts + (int64_t)blockIdx.x * El);
  __syncthreads();
  if (l >= 0) s2r[(int64_t)blockIdx.x * kCompactBlockSlots + threadIdx.x] = runw[l] + below;
}

template <int V, bool SIG>
hipError_t launch_fast(const uint16_t* logits, int64_t T, int K, int renorm, float* w, int32_t* ids, int32_t* tei,
                       hipStream_t stream) {
  const int64_t blocks = (T + (kBlock / 8) - 1) / (kBlock / 8);
  hipLaunchKernelGGL((topk8_bf16_kernel<V, SIG>), dim3((unsigned)blocks), dim3(kBlock), 0, stream, logits, T, K, renorm, w,
                     ids, tei);
  return hipGetLastError();
}

// E = 8*V with V in {8, 12, 16, 20, 24}, K <= 8, aligned rows: the fast kernel
template <bool SIG>
bool try_fast(const uint16_t* logits, int64_t T, int E, int K, int renorm, float* w, int32_t* ids, int32_t* tei,
              hipStream_t stream, hipError_t* err) {
  if (K > 8 || E % 8 != 0) return false;
  const int V = E / 8;
  const int align = (V % 8 == 0) ? 16 : 8;
  if ((uintptr_t)logits % align != 0 || (E * 2) % align != 0) return false;
  switch (V) {
    case 8: *err = launch_fast<8, SIG>(logits, T, K, renorm, w, ids, tei, stream); return true;
    case 12: *err = launch_fast<12, SIG>(logits, T, K, renorm, w, ids, tei, stream); return true;
    case 16: *err = launch_fast<16, SIG>(logits, T, K, renorm, w, ids, tei, stream); return true;
    case 20: *err = launch_fast<20, SIG>(logits, T, K, renorm, w, ids, tei, stream); return true;
    case 24: *err = launch_fast<24, SIG>(logits, T, K, renorm, w, ids, tei, stream); return true;
    default: return false;
  }
}
}  // namespace

namespace {
template <bool SIG>
hipError_t launch_gate(const void* logits, int logits_dtype, int64_t T, int E, int K, int renormalize, float* w,
                       int32_t* ids, int32_t* tei, hipStream_t stream) {
  if (logits_dtype == MOE_BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(logits);
    hipError_t err;
    if (try_fast<SIG>(p, T, E, K, renormalize, w, ids, tei, stream, &err)) return err;
    return K <= 8 ? dispatch_gv<uint16_t, 8, SIG>(p, T, E, K, renormalize, w, ids, tei, stream)
                  : dispatch_gv<uint16_t, 32, SIG>(p, T, E, K, renormalize, w, ids, tei, stream);
  }
  const float* p = static_cast<const float*>(logits);
  return K <= 8 ? dispatch_gv<float, 8, SIG>(p, T, E, K, renormalize, w, ids, tei, stream)
                : dispatch_gv<float, 32, SIG>(p, T, E, K, renormalize, w, ids, tei, stream);
}
}  // namespace

hipError_t launch_topk_softmax(const void* logits, int logits_dtype, int64_t T, int E, int K, int renormalize,
                               float* w, int32_t* ids, int32_t* tei, hipStream_t stream) {
  return launch_gate<false>(logits, logits_dtype, T, E, K, renormalize, w, ids, tei, stream);
}

hipError_t launch_topk_sigmoid(const void* logits, int logits_dtype, int64_t T, int E, int K, int renormalize,
                               float* w, int32_t* ids, int32_t* tei, hipStream_t stream) {
  return launch_gate<true>(logits, logits_dtype, T, E, K, renormalize, w, ids, tei, stream);
}

namespace {
template <int V, bool SIG>
hipError_t launch_count_fused(const uint16_t* logits, int64_t T, int renorm, float* w, int32_t* ids, int32_t* tei,
                              const int32_t* emap, int Eg, int El, int32_t* bc, int32_t* s2r, hipStream_t stream) {
  const int64_t blocks = (T + kCompactBlockSlots / 8 - 1) / (kCompactBlockSlots / 8);
  hipLaunchKernelGGL((topk8_count_kernel<V, SIG>), dim3((unsigned)blocks), dim3(kCompactBlockSlots),
                     sizeof(int) * (size_t)kCompactWaves * El, stream, logits, T, renorm, w, ids, tei, emap, Eg, El,
                     bc, s2r);
  return hipGetLastError();
}

template <bool SIG>
hipError_t dispatch_count_fused(int V, const uint16_t* logits, int64_t T, int renorm, float* w, int32_t* ids,
                                int32_t* tei, const int32_t* emap, int Eg, int El, int32_t* bc, int32_t* s2r,
                                hipStream_t stream) {
  switch (V) {
    case 8: return launch_count_fused<8, SIG>(logits, T, renorm, w, ids, tei, emap, Eg, El, bc, s2r, stream);
    case 12: return launch_count_fused<12, SIG>(logits, T, renorm, w, ids, tei, emap, Eg, El, bc, s2r, stream);
    case 16: return launch_count_fused<16, SIG>(logits, T, renorm, w, ids, tei, emap, Eg, El, bc, s2r, stream);
    case 20: return launch_count_fused<20, SIG>(logits, T, renorm, w, ids, tei, emap, Eg, El, bc, s2r, stream);
    default: return launch_count_fused<24, SIG>(logits, T, renorm, w, ids, tei, emap, Eg, El, bc, s2r, stream);
  }
}
}  // namespace

hipError_t launch_topk_compact(const void* logits, int logits_dtype, int64_t T, int E, int K, int renormalize,
                               int scoring, float* w, int32_t* ids, int32_t* tei, const int32_t* emap, int El,
                               int32_t* counts, int32_t* offsets, int32_t* s2r, int32_t* r2s, void* workspace,
                               hipStream_t stream) {
  const int64_t N = T * K;
  const int V = E / 8;
  const int align = (V % 8 == 0) ? 16 : 8;
  const bool fused = logits_dtype == MOE_BF16 && K == 8 && N > kCompactSingleMax && E % 8 == 0 &&
                     (V == 8 || V == 12 || V == 16 || V == 20 || V == 24) && (uintptr_t)logits % align == 0 &&
                     (E * 2) % align == 0;
  if (fused) {
    const uint16_t* p = static_cast<const uint16_t*>(logits);
    int32_t* bc = static_cast<int32_t*>(workspace);  // [B][El], as the compaction's count kernel uses it
    hipError_t err = scoring ? dispatch_count_fused<true>(V, p, T, renormalize, w, ids, tei, emap, E, El, bc, s2r,
                                                          stream)
                             : dispatch_count_fused<false>(V, p, T, renormalize, w, ids, tei, emap, E, El, bc, s2r,
                                                           stream);
    if (err != hipSuccess) return err;
    return launch_compact_scatter_phase(ids, N, emap, E, El, bc, counts, offsets, s2r, r2s, stream);
  }
  if (T > 0) {
    const hipError_t err = scoring ? launch_gate<true>(logits, logits_dtype, T, E, K, renormalize, w, ids, tei, stream)
                                   : launch_gate<false>(logits, logits_dtype, T, E, K, renormalize, w, ids, tei, stream);
    if (err != hipSuccess) return err;
  }
  return launch_route_compact(ids, N, emap, E, El, counts, offsets, s2r, r2s, workspace, stream);
}

}  // namespace moe
