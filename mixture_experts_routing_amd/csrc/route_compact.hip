// Route compaction for one expert-parallel rank (gfx950).
//
// Source: b70-optimization-lab note "MTP1 M2 compact scheduler closure"
// (2026-07-16), design paragraph: each local expert's row count and
// remapped-row prefix are derived on device from topk_ids plus expert_map,
// the expert-grouped activation layout is kept, duplicates are allowed and a
// rank whose routes are all remote is valid.
//
// Output is a stable counting sort of the slots by local expert id, so every
// position is fixed by the inputs (no atomics decide an order):
//   occurrence(s) = number of earlier slots with the same local id
//   slot_to_row[s] = offsets[l] + occurrence(s)
// A wavefront takes 64 consecutive slots; the rank of a slot among equal ids
// of its group comes from bit-sliced ballots (one per bit of the local id),
// and per-wave running counts per expert live in LDS.  A per-expert exclusive prefix over the
// waves (then over blocks) turns group ranks into occurrences.
//
//   N <= 64         : one wavefront does everything (decode batches)
//   N <= kSingleMax : one 1024-thread block does everything
//   larger N        : count kernel (per block counts + in-block ranks, which
//                     are parked in slot_to_row), then for up to 64 count
//                     blocks one fused kernel in which every block sums the
//                     block counts it needs itself and scatters, else a
//                     one-block scan kernel (per expert prefix over blocks,
//                     offsets) -> scatter
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = kCompactWaves;
constexpr int kThreads = kWaves * 64;
constexpr int kGroupsSingle = 4;                       // 64-slot groups per wave, single-block path
constexpr int kSingleMax = kCompactSingleMax;          // 4096 slots
constexpr int kBlockSlots = kCompactBlockSlots;        // slots per block, multi-block path
static_assert(kSingleMax == kWaves * kGroupsSingle * 64, "single-block capacity");

__device__ __forceinline__ int local_of(int id, const int32_t* __restrict__ emap, int Eg, int El) {
  return local_expert(id, emap, Eg, El);
}

__device__ __forceinline__ void group_rank(int l, int El, int& below, int& total) {
  wave_group_rank(l, El, below, total);
}

// Ranks the 64-slot groups [first_slot + 64*g, ...) of one wave; returns the
// rank of each lane's slot among equal local ids of this wave's slots (in
// slot order) and leaves the wave's per-expert totals in run[0..El).
template <int GPW>
__device__ __forceinline__ void wave_ranks(const int32_t* __restrict__ ids, int64_t N, int64_t first_slot,
                                           const int32_t* __restrict__ emap, int Eg, int El, int lane,
                                           int* __restrict__ run, int (&loc)[GPW], int (&rank)[GPW]) {
#pragma unroll
  for (int g = 0; g < GPW; ++g) {
    const int64_t s0 = first_slot + (int64_t)g * 64;
    loc[g] = -1;
    rank[g] = 0;
    if (s0 >= N) continue;  // uniform
    const int64_t s = s0 + lane;
    const int l = (s < N) ? local_of(ids[s], emap, Eg, El) : -1;
    int below, total;
    group_rank(l, El, below, total);
    if (l >= 0) rank[g] = run[l] + below;
    // one writer per distinct id: the last occurrence in this group
    if (l >= 0 && below == total - 1) run[l] += total;
    loc[g] = l;
  }
}

// Exclusive scan of v over the block's threads (kThreads of them); returns
// the prefix and writes the block total to *total.  tmp: kWaves+1 ints.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int ws = lane < kWaves ? tmp[lane] : 0;
    int wi = ws;
#pragma unroll
    for (int d = 1; d < kWaves; d <<= 1) {
      const int o = __shfl_up(wi, d, 64);
      if (lane >= d) wi += o;
    }
    if (lane < kWaves) tmp[lane] = wi - ws;
    if (lane == kWaves - 1) tmp[kWaves] = wi;
  }
  __syncthreads();
  const int r = tmp[wave] + inc - v;
  *total = tmp[kWaves];
  __syncthreads();
  return r;
}

__device__ __forceinline__ void prefix_over_waves(int* __restrict__ run, int El, int* __restrict__ cnt) {
  prefix_over_compact_waves(run, El, cnt);
}

// Exclusive scan of cnt[0..El) into offs[0..El]; El <= kThreads.
__device__ __forceinline__ void scan_counts(const int* __restrict__ cnt, int El, int* __restrict__ offs,
                                            int* tmp) {
  const int e = threadIdx.x;
  const int v = e < El ? cnt[e] : 0;
  int total;
  const int ex = block_exclusive_scan(v, tmp, &total);
  if (e < El) offs[e] = ex;
  if (e == 0) offs[El] = total;
  __syncthreads();
}

// ---------------------------------------------------------------------------
// one wave: N <= 64 (decode batches).  Every slot sits in one lane; an
// expert's count is the number of lanes holding its id, read lane by lane.

constexpr int kWaveMax = 64;
constexpr int kWaveMaxEl = 768;

__global__ __launch_bounds__(64) void compact_wave_kernel(
    const int32_t* __restrict__ ids, int N, const int32_t* __restrict__ emap, int Eg, int El,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ s2r,
    int32_t* __restrict__ r2s) {
  __shared__ int offs[kWaveMaxEl];
  const int lane = threadIdx.x;
  const int l = lane < N ? local_of(ids[lane], emap, Eg, El) : -1;
  int below, total;
  group_rank(l, El, below, total);
  int carry = 0;
  for (int c0 = 0; c0 < El; c0 += 64) {
    const int e = c0 + lane;
    int cnt = 0;
    for (int j = 0; j < N; ++j) cnt += (__builtin_amdgcn_readlane(l, j) == e) ? 1 : 0;
    int inc = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(inc, d, 64);
      if (lane >= d) inc += o;
    }
    if (e < El) {
      const int ex = carry + inc - cnt;
      counts[e] = cnt;
      offsets[e] = ex;
      offs[e] = ex;
    }
    carry += __shfl(inc, 63, 64);
  }
  if (lane == 0) offsets[El] = carry;
  __syncthreads();
  if (lane < N) {
    const int row = l >= 0 ? offs[l] + below : -1;
    s2r[lane] = row;
    if (row >= 0) r2s[row] = lane;
    if (lane >= carry) r2s[lane] = -1;
  }
}

// ---------------------------------------------------------------------------
// single block: N <= kSingleMax

__global__ __launch_bounds__(kThreads) void compact_single_kernel(
    const int32_t* __restrict__ ids, int N, const int32_t* __restrict__ emap, int Eg, int El,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ s2r,
    int32_t* __restrict__ r2s) {
  extern __shared__ int lds[];
  int* run = lds;                     // [kWaves][El]
  int* cnt = run + kWaves * El;       // [El]
  int* offs = cnt + El;               // [El + 1]
  int* tmp = offs + El + 1;           // [kWaves + 1]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  for (int i = threadIdx.x; i < kWaves * El; i += kThreads) run[i] = 0;
  __syncthreads();

  int loc[kGroupsSingle], rank[kGroupsSingle];
  const int64_t first = (int64_t)wave * kGroupsSingle * 64;
  wave_ranks<kGroupsSingle>(ids, N, first, emap, Eg, El, lane, run + wave * El, loc, rank);
  __syncthreads();
  prefix_over_waves(run, El, cnt);
  __syncthreads();
  scan_counts(cnt, El, offs, tmp);

  for (int e = threadIdx.x; e < El; e += kThreads) counts[e] = cnt[e];
  for (int e = threadIdx.x; e <= El; e += kThreads) offsets[e] = offs[e];

#pragma unroll
  for (int g = 0; g < kGroupsSingle; ++g) {
    const int64_t s = first + g * 64 + lane;
    if (s < N) {
      const int l = loc[g];
      const int row = l >= 0 ? offs[l] + run[wave * El + l] + rank[g] : -1;
      s2r[s] = row;
      if (row >= 0) r2s[row] = (int32_t)s;
    }
  }
  const int R = offs[El];
  for (int r = R + threadIdx.x; r < N; r += kThreads) r2s[r] = -1;
}

// ---------------------------------------------------------------------------
// multi block

__global__ __launch_bounds__(kThreads) void compact_count_kernel(
    const int32_t* __restrict__ ids, int64_t N, const int32_t* __restrict__ emap, int Eg, int El,
    int32_t* __restrict__ block_counts /*[B][El]*/, int32_t* __restrict__ s2r) {
  extern __shared__ int lds[];
  int* run = lds;  // [kWaves][El]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kWaves * El; i += kThreads) run[i] = 0;
  __syncthreads();
  int loc[1], rank[1];
  const int64_t first = (int64_t)blockIdx.x * kBlockSlots + wave * 64;
  wave_ranks<1>(ids, N, first, emap, Eg, El, lane, run + wave * El, loc, rank);
  __syncthreads();
  prefix_over_waves(run, El, block_counts + (int64_t)blockIdx.x * El);
  __syncthreads();
  const int64_t s = first + lane;
  if (s < N && loc[0] >= 0) s2r[s] = run[wave * El + loc[0]] + rank[0];  // rank inside this block
}

// Per-expert exclusive prefix over the B count blocks (each block's base row
// per expert), the expert totals and the offsets, in one block.  Thread t
// takes expert t % El and part t / El of the count blocks (P = kThreads / El
// parts of consecutive blocks), so a thread reads few counts and none of its
// loads waits on another: the part sums, a prefix over the parts per expert,
// the scan over experts, then each part writes its blocks' bases.
__global__ __launch_bounds__(kThreads) void compact_scan_kernel(
    int32_t* __restrict__ block_counts, int B, int El, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets) {
  extern __shared__ int lds[];
  const int P = kThreads / El;  // El <= kThreads
  int* cnt = lds;                  // [El]
  int* offs = cnt + El;            // [El + 1]
  int* tmp = offs + El + 1;        // [kWaves + 1]
  int* part = tmp + kWaves + 1;    // [P][El]
  const int e = (int)threadIdx.x % El, p = (int)threadIdx.x / El;
  const int per = (B + P - 1) / P;
  const int b0 = p < P ? min(B, p * per) : B, b1 = min(B, b0 + per);
  constexpr int kBatch = 8;
  int sum = 0;
  for (int b = b0; b < b1; b += kBatch) {
    int c[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) c[j] = (b + j < b1) ? block_counts[(int64_t)(b + j) * El + e] : 0;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) sum += c[j];
  }
  if (p < P) part[p * El + e] = sum;
  __syncthreads();
  for (int x = threadIdx.x; x < El; x += kThreads) {
    int acc = 0;
    for (int q = 0; q < P; ++q) {
      const int c = part[q * El + x];
      part[q * El + x] = acc;
      acc += c;
    }
    cnt[x] = acc;
  }
  __syncthreads();
  scan_counts(cnt, El, offs, tmp);
  if (p < P) {
    int acc = offs[e] + part[p * El + e];
    for (int b = b0; b < b1; b += kBatch) {
      int c[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) c[j] = (b + j < b1) ? block_counts[(int64_t)(b + j) * El + e] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (b + j < b1) block_counts[(int64_t)(b + j) * El + e] = acc;
        acc += c[j];
      }
    }
  }
  for (int x = threadIdx.x; x < El; x += kThreads) counts[x] = cnt[x];
  for (int x = threadIdx.x; x <= El; x += kThreads) offsets[x] = offs[x];
}

__global__ __launch_bounds__(256) void compact_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t N, const int32_t* __restrict__ emap, int Eg, int El,
    const int32_t* __restrict__ block_base /*[B][El]*/, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ s2r, int32_t* __restrict__ r2s) {
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (s >= N) return;
  const int l = local_of(ids[s], emap, Eg, El);
  int row = -1;
  if (l >= 0) {
    const int64_t b = s / kBlockSlots;
    row = block_base[b * El + l] + s2r[s];
    r2s[row] = (int32_t)s;
  }
  s2r[s] = row;
  const int R = offsets[El];
  if (s >= R) r2s[s] = -1;
}

// Fused scan + scatter for few count blocks (B <= kFusedMaxBlocks): block b
// (1024 threads, the same 1024 slots as count block b) sums every block's
// counts per expert itself -- the total (for the expert offsets) and the part
// of blocks before b (its base) -- so no separate scan pass is needed.
// Block 0 writes counts and offsets.
constexpr int kFusedMaxBlocks = 64;

__global__ __launch_bounds__(kThreads) void compact_scan_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t N, const int32_t* __restrict__ emap, int Eg, int El,
    const int32_t* __restrict__ block_counts /*[B][El]*/, int B, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ s2r, int32_t* __restrict__ r2s) {
  extern __shared__ int lds[];
  int* base = lds;          // [El]
  int* tmp = base + El;     // [kWaves + 1]
  const int b = blockIdx.x;
  const int e = threadIdx.x;  // El <= kThreads: one expert per thread
  int tot = 0, pre = 0;
  if (e < El) {
    // 8 count loads in flight at a time (independent, L2-resident)
    int bb = 0;
    for (; bb + 8 <= B; bb += 8) {
      int c[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = block_counts[(int64_t)(bb + j) * El + e];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        tot += c[j];
        pre += bb + j < b ? c[j] : 0;
      }
    }
    for (; bb < B; ++bb) {
      const int c = block_counts[(int64_t)bb * El + e];
      tot += c;
      pre += bb < b ? c : 0;
    }
  }
  int total;
  const int off = block_exclusive_scan(e < El ? tot : 0, tmp, &total);
  if (e < El) {
    base[e] = off + pre;
    if (b == 0) {
      counts[e] = tot;
      offsets[e] = off;
    }
  }
  if (b == 0 && e == 0) offsets[El] = total;
  __syncthreads();
  const int64_t s = (int64_t)b * kBlockSlots + threadIdx.x;
  if (s < N) {
    const int l = local_of(ids[s], emap, Eg, El);
    int row = -1;
    if (l >= 0) {
      row = base[l] + s2r[s];  // in-block rank parked by the count kernel
      r2s[row] = (int32_t)s;
    }
    s2r[s] = row;
    if (s >= total) r2s[s] = -1;
  }
}

// ---------------------------------------------------------------------------
// block-aligned layout, from the compaction's counts / offsets / permutation

// Expert e with off[e] <= x < off[e+1] (off ascending, off[0] = 0, x < off[El]).
__device__ __forceinline__ int expert_at(const int32_t* __restrict__ off, int El, int x) {
  int lo = 0, hi = El;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// One block: padded offsets (exclusive scan of the counts rounded up to the
// block size) and the expert of every block.
__global__ __launch_bounds__(kThreads) void align_offsets_kernel(const int32_t* __restrict__ counts, int El, int bs,
                                                                 int cap_blocks, int32_t* __restrict__ poff,
                                                                 int32_t* __restrict__ block_expert) {
  extern __shared__ int lds[];
  int* off = lds;        // [El + 1]
  int* tmp = off + El + 1;  // [kWaves + 1]
  const int e = threadIdx.x;  // El <= kThreads
  const int padded = e < El ? (counts[e] + bs - 1) / bs * bs : 0;
  int total;
  const int ex = block_exclusive_scan(padded, tmp, &total);
  if (e < El) {
    off[e] = ex;
    poff[e] = ex;
  }
  if (e == 0) {
    off[El] = total;
    poff[El] = total;
  }
  __syncthreads();
  const int nblocks = total / bs;
  for (int b = threadIdx.x; b < cap_blocks; b += kThreads)
    block_expert[b] = b < nblocks ? expert_at(off, El, b * bs) : -1;
}

// sorted_slots over the capacity and the padded row of every slot.
__global__ __launch_bounds__(256) void align_fill_kernel(const int32_t* __restrict__ counts,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ r2s,
                                                         const int32_t* __restrict__ s2r,
                                                         const int32_t* __restrict__ poff, int El, int64_t N,
                                                         int64_t cap_rows, int32_t* __restrict__ sorted_slots,
                                                         int32_t* __restrict__ slot_to_row) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < cap_rows) {
    const int p = (int)i;
    int v = -1;
    if (p < poff[El]) {
      const int e = expert_at(poff, El, p);
      const int o = p - poff[e];
      if (o < counts[e]) v = r2s[offsets[e] + o];
    }
    sorted_slots[p] = v;
  }
  if (i < N) {
    const int r = s2r[i];
    int v = -1;
    if (r >= 0) {
      const int e = expert_at(offsets, El, r);
      v = poff[e] + (r - offsets[e]);
    }
    slot_to_row[i] = v;
  }
}

}  // namespace

size_t route_align_workspace_bytes(int64_t N, int E_local) {
  // counts, offsets, slot_to_row, row_to_slot of the compaction, then its workspace
  const size_t own = ((size_t)(2 * E_local + 1) + 2 * (size_t)N) * sizeof(int32_t);
  return (own + 255) / 256 * 256 + route_compact_workspace_bytes(N, E_local);
}

hipError_t launch_route_align(const int32_t* ids, int64_t N, const int32_t* emap, int Eg, int El, int bs,
                              int32_t* poff, int32_t* sorted_slots, int32_t* block_expert, int32_t* slot_to_row,
                              void* workspace, hipStream_t stream) {
  int32_t* counts = static_cast<int32_t*>(workspace);
  int32_t* offsets = counts + El;
  int32_t* s2r = offsets + El + 1;
  int32_t* r2s = s2r + N;
  const size_t own = ((size_t)(2 * El + 1) + 2 * (size_t)N) * sizeof(int32_t);
  void* cws = static_cast<uint8_t*>(workspace) + (own + 255) / 256 * 256;
  hipError_t err = launch_route_compact(ids, N, emap, Eg, El, counts, offsets, s2r, r2s, cws, stream);
  if (err != hipSuccess) return err;
  const int64_t cap_rows = N + (int64_t)El * (bs - 1);
  const int64_t cap_blocks = (N + bs - 1) / bs + El;
  hipLaunchKernelGGL(align_offsets_kernel, dim3(1), dim3(kThreads), sizeof(int) * ((size_t)El + 1 + kWaves + 1),
                     stream, counts, El, bs, (int)cap_blocks, poff, block_expert);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int64_t n = cap_rows > N ? cap_rows : N;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(align_fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, counts, offsets, r2s,
                     s2r, poff, El, N, cap_rows, sorted_slots, slot_to_row);
  return hipGetLastError();
}

size_t route_compact_workspace_bytes(int64_t N, int E_local) {
  if (N <= kSingleMax) return 0;
  const int64_t B = (N + kBlockSlots - 1) / kBlockSlots;
  return (size_t)B * (size_t)E_local * sizeof(int32_t);
}

hipError_t launch_route_compact(const int32_t* ids, int64_t N, const int32_t* emap, int Eg, int El,
                                int32_t* counts, int32_t* offsets, int32_t* s2r, int32_t* r2s,
                                void* workspace, hipStream_t stream) {
  if (N <= kWaveMax && El <= kWaveMaxEl) {
    hipLaunchKernelGGL(compact_wave_kernel, dim3(1), dim3(64), 0, stream, ids, (int)N, emap, Eg, El, counts, offsets,
                       s2r, r2s);
    return hipGetLastError();
  }
  if (N <= kSingleMax) {
    const size_t lds = sizeof(int) * ((size_t)kWaves * El + El + El + 1 + kWaves + 1);
    hipLaunchKernelGGL(compact_single_kernel, dim3(1), dim3(kThreads), lds, stream, ids, (int)N, emap,
                       Eg, El, counts, offsets, s2r, r2s);
    return hipGetLastError();
  }
  const int64_t B = (N + kBlockSlots - 1) / kBlockSlots;
  int32_t* bc = static_cast<int32_t*>(workspace);
  hipLaunchKernelGGL(compact_count_kernel, dim3((unsigned)B), dim3(kThreads),
                     sizeof(int) * (size_t)kWaves * El, stream, ids, N, emap, Eg, El, bc, s2r);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_compact_scatter_phase(ids, N, emap, Eg, El, bc, counts, offsets, s2r, r2s, stream);
}

hipError_t launch_compact_scatter_phase(const int32_t* ids, int64_t N, const int32_t* emap, int Eg, int El,
                                        int32_t* bc, int32_t* counts, int32_t* offsets, int32_t* s2r, int32_t* r2s,
                                        hipStream_t stream) {
  const int64_t B = (N + kBlockSlots - 1) / kBlockSlots;
  hipError_t err;
  if (B <= kFusedMaxBlocks) {
    hipLaunchKernelGGL(compact_scan_scatter_kernel, dim3((unsigned)B), dim3(kThreads),
                       sizeof(int) * ((size_t)El + kWaves + 1), stream, ids, N, emap, Eg, El, bc, (int)B, counts,
                       offsets, s2r, r2s);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(compact_scan_kernel, dim3(1), dim3(kThreads),
                     sizeof(int) * ((size_t)El + El + 1 + kWaves + 1 + (size_t)(kThreads / El) * El), stream, bc,
                     (int)B, El, counts,
                     offsets);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(compact_scatter_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream,
                     ids, N, emap, Eg, El, bc, offsets, s2r, r2s);
  return hipGetLastError();
}

}  // namespace moe
