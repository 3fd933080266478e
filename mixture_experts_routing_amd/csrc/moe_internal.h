// Internal declarations shared by the library's translation units: device
// helpers (bf16 conversion, wave-level DPP reductions) and the host-side
// launchers that the C ABI layer calls after validating arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_routing.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// scalar conversions

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// ---------------------------------------------------------------------------
// DPP lane exchanges inside a wave.  Every pattern used here reads a lane of
// the same 16-lane row that always exists, so bound_ctrl never zero-fills; it
// is set so that the compiler folds the move into the consuming ALU op.
// Callers keep EXEC full around these helpers.

enum : int {
  DPP_QUAD_XOR1 = 0xB1,    // quad_perm [1,0,3,2]
  DPP_QUAD_XOR2 = 0x4E,    // quad_perm [2,3,0,1]
  DPP_ROW_HALF_MIRROR = 0x141,  // lane i <- lane 7-i within each 8
  DPP_ROW_MIRROR = 0x140,       // lane i <- lane 15-i within each 16
};

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, true);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Value of lane (lane ^ m) for m in {16, 32}: crosses 16-lane rows, so it
// goes through ds_swizzle/bpermute rather than DPP.
__device__ __forceinline__ int xor_lane_i32(int x, int m) { return __shfl_xor(x, m, 64); }
__device__ __forceinline__ float xor_lane_f32(float x, int m) { return __shfl_xor(x, m, 64); }

// Max over each aligned group of G lanes (G a power of two <= 64); every lane
// of the group receives the result.
template <int G>
__device__ __forceinline__ int group_max_i32(int x) {
  if constexpr (G >= 2) x = max(x, dpp_i32<DPP_QUAD_XOR1>(x));
  if constexpr (G >= 4) x = max(x, dpp_i32<DPP_QUAD_XOR2>(x));
  if constexpr (G >= 8) x = max(x, dpp_i32<DPP_ROW_HALF_MIRROR>(x));
  if constexpr (G >= 16) x = max(x, dpp_i32<DPP_ROW_MIRROR>(x));
  if constexpr (G >= 32) x = max(x, xor_lane_i32(x, 16));
  if constexpr (G >= 64) x = max(x, xor_lane_i32(x, 32));
  return x;
}

// 64-bit keys: exchange both halves, compare as signed 64-bit.
template <int CTRL>
__device__ __forceinline__ int64_t dpp_i64(int64_t x) {
  int lo = dpp_i32<CTRL>((int)(uint32_t)x);
  int hi = dpp_i32<CTRL>((int)(x >> 32));
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ int64_t xor_lane_i64(int64_t x, int m) {
  int lo = __shfl_xor((int)(uint32_t)x, m, 64);
  int hi = __shfl_xor((int)(x >> 32), m, 64);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
template <int G>
__device__ __forceinline__ int64_t group_max_i64(int64_t x) {
  if constexpr (G >= 2) { int64_t y = dpp_i64<DPP_QUAD_XOR1>(x); x = x > y ? x : y; }
  if constexpr (G >= 4) { int64_t y = dpp_i64<DPP_QUAD_XOR2>(x); x = x > y ? x : y; }
  if constexpr (G >= 8) { int64_t y = dpp_i64<DPP_ROW_HALF_MIRROR>(x); x = x > y ? x : y; }
  if constexpr (G >= 16) { int64_t y = dpp_i64<DPP_ROW_MIRROR>(x); x = x > y ? x : y; }
  if constexpr (G >= 32) { int64_t y = xor_lane_i64(x, 16); x = x > y ? x : y; }
  if constexpr (G >= 64) { int64_t y = xor_lane_i64(x, 32); x = x > y ? x : y; }
  return x;
}

// Sum over each aligned group of G lanes.  Each step adds a lane's partial to
// its partner's (a + b == b + a), so every lane of the group ends with the
// bit-identical sum, in a fixed order.
template <int G>
__device__ __forceinline__ float group_sum_f32(float x) {
  if constexpr (G >= 2) x += dpp_f32<DPP_QUAD_XOR1>(x);
  if constexpr (G >= 4) x += dpp_f32<DPP_QUAD_XOR2>(x);
  if constexpr (G >= 8) x += dpp_f32<DPP_ROW_HALF_MIRROR>(x);
  if constexpr (G >= 16) x += dpp_f32<DPP_ROW_MIRROR>(x);
  if constexpr (G >= 32) x += xor_lane_f32(x, 16);
  if constexpr (G >= 64) x += xor_lane_f32(x, 32);
  return x;
}

// Local expert of a global id on this rank: -1 for a remote expert (map
// value outside [0, El)) and for an id outside [0, Eg).  emap == nullptr is
// the identity map.
__device__ __forceinline__ int local_expert(int id, const int32_t* __restrict__ emap, int Eg, int El) {
  if (id < 0 || id >= Eg) return -1;
  const int l = emap ? emap[id] : id;
  return (l >= 0 && l < El) ? l : -1;
}

// ---------------------------------------------------------------------------
// stable counting sort of slots by local expert (route compaction), pieces
// shared by the compaction kernels and the gate kernel that fuses the count
// pass: the multi-block compaction cuts the slots into blocks of
// kCompactBlockSlots (thread i of block b holds slot b * kCompactBlockSlots + i)

constexpr int kCompactWaves = 16;
constexpr int kCompactBlockSlots = kCompactWaves * 64;  // 1024
constexpr int kCompactSingleMax = 4096;                 // one block handles up to this many slots

// For the 64 lanes of a wave holding local ids l (-1 = remote/absent,
// l < El): the number of lower lanes with the same id, and the number with
// that id.  Lane j holds this lane's id exactly when every bit of l+1 agrees,
// so the lanes of equal id are the AND over those bits of "the lanes where
// the bit is set" (one ballot) or its complement: ceil(log2(El+1)) ballots.
// Every lane of the wave must be active.
__device__ __forceinline__ void wave_group_rank(int l, int El, int& below, int& total) {
  const uint32_t u = (uint32_t)(l + 1);  // 0 .. El
  const int nbits = El > 0 ? 32 - __clz(El) : 0;
  uint64_t m = ~0ull;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (u >> b) & 1u;
    const uint64_t set = __ballot(bit);
    m &= bit ? set : ~set;
  }
  total = __popcll(m);
  below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Per-expert exclusive prefix over the kCompactWaves rows of run[w*El + e]
// (every thread of the block takes experts e = tid, tid + blockDim.x, ...);
// each expert's total goes to cnt[e].
__device__ __forceinline__ void prefix_over_compact_waves(int* __restrict__ run, int El, int* __restrict__ cnt) {
  for (int e = threadIdx.x; e < El; e += blockDim.x) {
    int acc = 0;
#pragma unroll
    for (int w = 0; w < kCompactWaves; ++w) {
      const int c = run[w * El + e];
      run[w * El + e] = acc;
      acc += c;
    }
    cnt[e] = acc;
  }
}

// ---------------------------------------------------------------------------
// host-side launchers (one per kernel family), called after validation

hipError_t launch_topk_softmax(const void* logits, int logits_dtype, int64_t T, int E, int K,
                               int renormalize, float* w, int32_t* ids, int32_t* tei,
                               hipStream_t stream);
hipError_t launch_topk_sigmoid(const void* logits, int logits_dtype, int64_t T, int E, int K,
                               int renormalize, float* w, int32_t* ids, int32_t* tei,
                               hipStream_t stream);

size_t route_compact_workspace_bytes(int64_t N, int E_local);
hipError_t launch_route_compact(const int32_t* topk_ids, int64_t N, const int32_t* expert_map,
                                int E_global, int E_local, int32_t* counts, int32_t* offsets,
                                int32_t* slot_to_row, int32_t* row_to_slot, void* workspace,
                                hipStream_t stream);

// second phase of the multi-block compaction: from the per-block counts
// block_counts [B][El] and the in-block ranks parked in s2r, the expert
// counts and offsets and both permutations (N > kCompactSingleMax)
hipError_t launch_compact_scatter_phase(const int32_t* topk_ids, int64_t N, const int32_t* expert_map, int E_global,
                                        int E_local, int32_t* block_counts, int32_t* counts, int32_t* offsets,
                                        int32_t* slot_to_row, int32_t* row_to_slot, hipStream_t stream);

// gate and route compaction in one call; the count pass of the compaction
// runs inside the gate kernel where the shape allows (scoring 0 softmax, 1
// sigmoid)
hipError_t launch_topk_compact(const void* logits, int logits_dtype, int64_t T, int E, int K, int renormalize,
                               int scoring, float* w, int32_t* ids, int32_t* tei, const int32_t* expert_map,
                               int E_local, int32_t* counts, int32_t* offsets, int32_t* slot_to_row,
                               int32_t* row_to_slot, void* workspace, hipStream_t stream);

size_t route_align_workspace_bytes(int64_t N, int E_local);
hipError_t launch_route_align(const int32_t* topk_ids, int64_t N, const int32_t* expert_map, int E_global,
                              int E_local, int block_size, int32_t* padded_offsets, int32_t* sorted_slots,
                              int32_t* block_expert, int32_t* slot_to_row, void* workspace, hipStream_t stream);

size_t grouped_ffn_workspace_bytes(int64_t N, int H, int F, int El, int w_dtype);
// MXFP4 decode arithmetic (a moe_mxfp4_mma value), process-wide
int mxfp4_mma_mode();
void set_mxfp4_mma_mode(int mode);
hipError_t launch_grouped_ffn(const void* x, int x_dtype, int64_t T, int K, int H, int F,
                              int E_local, const void* w1, const uint8_t* w1s, const void* w2,
                              const uint8_t* w2s, int w_dtype, const int32_t* counts,
                              const int32_t* offsets, const int32_t* row_to_slot, void* y,
                              int y_dtype, void* workspace, hipStream_t stream);

// Tile-packed bf16 weight layout (MOE_BF16_TILED), written by
// moe_pack_ffn_weights and read by the tiled FFN kernels.  Per expert, the
// weight rows are cut into panels of kPanelRows rows and the reduction
// dimension into chunks of kPanelK elements; chunk (panel, kt) is stored as
// one contiguous 16 KB block, kt fastest after the panel, holding panel row R
// (64 bytes) at R*64 with its four 16-byte pieces XOR-swizzled: stored piece
// p holds elements kt*32 + 8*(p ^ panel_swz(R)) .. +8.  The block is the
// byte image of the kernels' LDS stage, so it moves with contiguous loads.
// GEMM1 panels interleave 32 gate rows and the matching 32 up rows.
constexpr int kPanelRows = 256;
constexpr int kPanelK = 32;
__host__ __device__ constexpr int panel_swz(int R) { return ((R >> 1) ^ (R >> 2)) & 3; }
// W1 row held by row R of GEMM1 panel nt (gate rows [0,F), up rows [F,2F))
__host__ __device__ constexpr int panel_w1_row(int R, int nt, int F) {
  return (((R >> 5) & 1) ? F : 0) + nt * (kPanelRows / 2) + (R >> 6) * 32 + (R & 31);
}
// W2 row held by row R of GEMM2 panel nt
__host__ __device__ constexpr int panel_w2_row(int R, int nt) { return nt * kPanelRows + R; }

// generic persistent scheduler (atomic work counter over every local expert,
// 64-column N tiles), the A/B control of the compact one
size_t grouped_ffn_control_workspace_bytes(int64_t N, int H, int F, int El, int w_dtype);
hipError_t launch_grouped_ffn_control(const void* x, int64_t T, int K, int H, int F, int El, const void* w1,
                                      const uint8_t* w1s, const void* w2, const uint8_t* w2s, int w_dtype,
                                      const int32_t* counts, const int32_t* offsets, const int32_t* r2s, void* y,
                                      int y_dtype, void* workspace, hipStream_t stream);

// LDS-tiled MFMA path for many rows per expert (bf16 weights, row-major or
// tile-packed)
bool tiled_ffn_applicable(int64_t N, int H, int F, int El);
bool tiled_shape_ok(int64_t N, int H, int F);
hipError_t launch_tiled_ffn(const uint16_t* x, int64_t T, int64_t N, int topk, int H, int F, int El,
                            const uint16_t* w1, const uint16_t* w2, bool packed, const int32_t* counts,
                            const int32_t* offsets, const int32_t* r2s, void* y, int y_dtype, uint16_t* act,
                            hipStream_t stream);
hipError_t launch_pack_ffn_weights(const uint16_t* w1, const uint16_t* w2, int El, int H, int F, uint16_t* w1t,
                                   uint16_t* w2t, hipStream_t stream);

// boundary fusion for decode batches: route compaction inside the GEMM1
// kernel, combine inside the GEMM2 kernel (T*K <= kFusedMaxSlots, El <= 64)
constexpr int kFusedMaxSlots = 64;
constexpr int kFusedMaxExperts = 64;
size_t fused_experts_workspace_bytes(int64_t N, int F);
hipError_t launch_fused_experts(const uint16_t* x, int64_t T, int K, int H, int F, const int32_t* ids,
                                const float* topk_weights, const int32_t* emap, int Eg, int El, const void* w1,
                                const uint8_t* w1s, const void* w2, const uint8_t* w2s, int w_dtype,
                                int32_t* counts, int32_t* offsets, int32_t* s2r, int32_t* r2s, void* out,
                                int out_dtype, void* workspace, hipStream_t stream);

hipError_t launch_combine(const void* y, int y_dtype, const float* w, const int32_t* slot_to_row,
                          int64_t T, int K, int H, void* out, int out_dtype, hipStream_t stream);

// measurement probes (no step of the layer)
hipError_t launch_probe_read(const void* src, int64_t bytes, uint32_t* out, hipStream_t stream);
hipError_t launch_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);
hipError_t launch_probe_mfma(int64_t iters, int blocks, bool toggle, float* out, unsigned long long* clk,
                             hipStream_t stream);
hipError_t launch_probe_gate_loads(const uint16_t* logits, int64_t T, int E, int K, float* w, int32_t* ids,
                                   int32_t* tei, hipStream_t stream);
int probe_read_out_words();

}  // namespace moe
