// C ABI entry points: host-side argument checks, then the launchers.
// Every check runs before anything is enqueued, so an error leaves the
// outputs untouched and the stream unchanged.
#include <mutex>

#include "moe_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = (int)e;
  return MOE_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

extern "C" {

const char* moe_version(void) { return "moe_routing 0.1 (gfx950)"; }

moe_status moe_set_mxfp4_mma(int mode) {
  if (mode != MOE_MXFP4_MMA_BF16 && mode != MOE_MXFP4_MMA_F8F6F4) return MOE_ERR_INVALID_ARG;
  moe::set_mxfp4_mma_mode(mode);
  return MOE_OK;
}

int moe_get_mxfp4_mma(void) { return moe::mxfp4_mma_mode(); }

const char* moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_SCRATCH_LIMIT: return "MOE_ERR_SCRATCH_LIMIT";
    default: return "MOE_ERR_UNKNOWN";
  }
}

int moe_last_hip_error(void) { return g_last_hip_error; }

namespace {
int check_gate(const void* logits, int logits_dtype, int64_t T, int32_t E, int32_t K, const float* topk_weights,
               const int32_t* topk_ids) {
  if (T < 0 || E < 1 || K < 1 || K > E) return MOE_ERR_INVALID_ARG;
  if (logits_dtype != MOE_F32 && logits_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (E > 1280 || K > 32) return MOE_ERR_UNSUPPORTED;
  if (T > ((int64_t)1 << 31) / K) return MOE_ERR_UNSUPPORTED;  // k*T + t must fit int32
  if (T == 0) return -1;                                        // valid no-op
  if (!logits || !topk_weights || !topk_ids) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}
}  // namespace

int moe_topk_softmax(const void* logits, int logits_dtype, int64_t T, int32_t E, int32_t K, int32_t renormalize,
                     float* topk_weights, int32_t* topk_ids, int32_t* token_expert_indices, void* stream) {
  const int st = check_gate(logits, logits_dtype, T, E, K, topk_weights, topk_ids);
  if (st != MOE_OK) return st < 0 ? MOE_OK : st;
  return hip_status(moe::launch_topk_softmax(logits, logits_dtype, T, E, K, renormalize != 0, topk_weights, topk_ids,
                                             token_expert_indices, static_cast<hipStream_t>(stream)));
}

int moe_topk_sigmoid(const void* logits, int logits_dtype, int64_t T, int32_t E, int32_t K, int32_t renormalize,
                     float* topk_weights, int32_t* topk_ids, int32_t* token_expert_indices, void* stream) {
  const int st = check_gate(logits, logits_dtype, T, E, K, topk_weights, topk_ids);
  if (st != MOE_OK) return st < 0 ? MOE_OK : st;
  return hip_status(moe::launch_topk_sigmoid(logits, logits_dtype, T, E, K, renormalize != 0, topk_weights, topk_ids,
                                             token_expert_indices, static_cast<hipStream_t>(stream)));
}

int moe_topk_compact(const void* logits, int logits_dtype, int64_t T, int32_t E, int32_t K, int32_t renormalize,
                     int32_t scoring, float* topk_weights, int32_t* topk_ids, int32_t* token_expert_indices,
                     const int32_t* expert_map, int32_t E_local, int32_t* counts, int32_t* offsets,
                     int32_t* slot_to_row, int32_t* row_to_slot, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (scoring != 0 && scoring != 1) return MOE_ERR_UNSUPPORTED;
  const int st = check_gate(logits, logits_dtype, T, E, K, topk_weights, topk_ids);
  if (st > 0) return st;  // st < 0: T == 0, the compaction still defines counts and offsets
  if (E_local < 1 || E_local > E) return MOE_ERR_INVALID_ARG;
  if (!expert_map && E_local != E) return MOE_ERR_INVALID_ARG;
  if (E_local > 768) return MOE_ERR_UNSUPPORTED;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
  const int64_t N = T * K;
  if (N > 0 && (!slot_to_row || !row_to_slot)) return MOE_ERR_INVALID_ARG;
  const size_t need = moe::route_compact_workspace_bytes(N, E_local);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_topk_compact(logits, logits_dtype, T, E, K, renormalize != 0, scoring, topk_weights,
                                             topk_ids, token_expert_indices, expert_map, E_local, counts, offsets,
                                             slot_to_row, row_to_slot, workspace, static_cast<hipStream_t>(stream)));
}

size_t moe_route_compact_workspace_bytes(int64_t T, int32_t K, int32_t E_local) {
  if (T <= 0 || K <= 0 || E_local <= 0) return 0;
  return moe::route_compact_workspace_bytes(T * K, E_local);
}

int moe_route_compact(const int32_t* topk_ids, int64_t T, int32_t K, const int32_t* expert_map, int32_t E_global,
                      int32_t E_local, int32_t* counts, int32_t* offsets, int32_t* slot_to_row,
                      int32_t* row_to_slot, void* workspace, size_t workspace_bytes, void* stream) {
  if (T < 0 || K < 1 || E_local < 1 || E_global < 1 || E_local > E_global) return MOE_ERR_INVALID_ARG;
  if (!expert_map && E_local != E_global) return MOE_ERR_INVALID_ARG;
  if (E_local > 768) return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)K >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
  const int64_t N = T * K;
  if (N > 0 && (!topk_ids || !slot_to_row || !row_to_slot)) return MOE_ERR_INVALID_ARG;
  const size_t need = moe::route_compact_workspace_bytes(N, E_local);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MOE_ERR_WORKSPACE;
  // T == 0 still defines counts = 0 and offsets = 0: run the (cheap) kernel
  return hip_status(moe::launch_route_compact(topk_ids, N, expert_map, E_global, E_local, counts, offsets,
                                              slot_to_row, row_to_slot, workspace, static_cast<hipStream_t>(stream)));
}

size_t moe_route_align_workspace_bytes(int64_t T, int32_t K, int32_t E_local) {
  if (T < 0 || K <= 0 || E_local <= 0) return 0;
  return moe::route_align_workspace_bytes(T * K, E_local);
}

int moe_route_align(const int32_t* topk_ids, int64_t T, int32_t K, const int32_t* expert_map, int32_t E_global,
                    int32_t E_local, int32_t block_size, int32_t* padded_offsets, int32_t* sorted_slots,
                    int32_t* block_expert, int32_t* slot_to_row, void* workspace, size_t workspace_bytes,
                    void* stream) {
  if (T < 0 || K < 1 || E_local < 1 || E_global < 1 || E_local > E_global) return MOE_ERR_INVALID_ARG;
  if (block_size < 1) return MOE_ERR_INVALID_ARG;
  if (!expert_map && E_local != E_global) return MOE_ERR_INVALID_ARG;
  if (E_local > 768 || block_size > 4096) return MOE_ERR_UNSUPPORTED;
  const int64_t N = T * K;
  if (N + (int64_t)E_local * (block_size - 1) >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (!padded_offsets || !sorted_slots || !block_expert) return MOE_ERR_INVALID_ARG;
  if (N > 0 && (!topk_ids || !slot_to_row)) return MOE_ERR_INVALID_ARG;
  const size_t need = moe::route_align_workspace_bytes(N, E_local);
  if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_route_align(topk_ids, N, expert_map, E_global, E_local, block_size, padded_offsets,
                                            sorted_slots, block_expert, slot_to_row, workspace,
                                            static_cast<hipStream_t>(stream)));
}

size_t moe_grouped_ffn_workspace_bytes(int64_t T, int32_t K, int32_t H, int32_t F, int32_t E_local, int w_dtype) {
  if (T <= 0 || K <= 0 || F <= 0 || H <= 0 || E_local <= 0) return 0;
  return moe::grouped_ffn_workspace_bytes(T * K, H, F, E_local, w_dtype);
}

namespace {
// Checks shared by moe_grouped_ffn and moe_grouped_ffn_noalloc (everything but
// the workspace).  Returns MOE_OK, an error, or -1 for the valid no-op T == 0.
int check_grouped_ffn(const void* x, int x_dtype, int64_t T, int32_t K, int32_t H, int32_t F, int32_t E_local,
                      const void* w1, const uint8_t* w1_scale, const void* w2, const uint8_t* w2_scale, int w_dtype,
                      const int32_t* counts, const int32_t* offsets, const int32_t* row_to_slot, const void* y,
                      int y_dtype) {
  if (T < 0 || K < 1 || H < 1 || F < 1 || E_local < 1) return MOE_ERR_INVALID_ARG;
  if (y_dtype != MOE_F32 && y_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  const bool f32_pair = (x_dtype == MOE_F32 && w_dtype == MOE_F32);
  const bool bf16_pair = (x_dtype == MOE_BF16 && w_dtype == MOE_BF16);
  const bool mx_pair = (x_dtype == MOE_BF16 && w_dtype == MOE_MXFP4);
  const bool tiled_pair = (x_dtype == MOE_BF16 && w_dtype == MOE_BF16_TILED);
  if (!f32_pair && !bf16_pair && !mx_pair && !tiled_pair) return MOE_ERR_UNSUPPORTED;
  if (tiled_pair && !moe::tiled_shape_ok(T * (int64_t)K, H, F)) return MOE_ERR_UNSUPPORTED;
  if (!f32_pair && (H % 32 != 0 || F % 32 != 0)) return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)K >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (f32_pair && T * (int64_t)K * (int64_t)(H > F ? H : F) >= ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return -1;
  if (!x || !w1 || !w2 || !counts || !offsets || !row_to_slot || !y) return MOE_ERR_INVALID_ARG;
  if (mx_pair && (!w1_scale || !w2_scale)) return MOE_ERR_INVALID_ARG;
  if (!f32_pair) {
    // bf16 rows are read as 16-byte vectors
    if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16)) return MOE_ERR_INVALID_ARG;
    if (!aligned(y, 16)) return MOE_ERR_INVALID_ARG;  // rows are stored as 16-byte pieces
  }
  return MOE_OK;
}

// Scratch of moe_grouped_ffn_noalloc: the act rows that moe_grouped_ffn keeps
// in the caller's workspace.  Each GPU holds its own copy of the array from
// the time the library's code is loaded on it until the process ends.  The
// array's name is a host-side handle, not a device address: the address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is passed to the kernels.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

int moe_grouped_ffn(const void* x, int x_dtype, int64_t T, int32_t K, int32_t H, int32_t F, int32_t E_local,
                    const void* w1, const uint8_t* w1_scale, const void* w2, const uint8_t* w2_scale, int w_dtype,
                    const int32_t* counts, const int32_t* offsets, const int32_t* row_to_slot, void* y, int y_dtype,
                    void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_grouped_ffn(x, x_dtype, T, K, H, F, E_local, w1, w1_scale, w2, w2_scale, w_dtype, counts,
                                   offsets, row_to_slot, y, y_dtype);
  if (st != MOE_OK) return st < 0 ? MOE_OK : st;
  const size_t need = moe::grouped_ffn_workspace_bytes(T * K, H, F, E_local, w_dtype);
  if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_grouped_ffn(x, x_dtype, T, K, H, F, E_local, w1, w1_scale, w2, w2_scale, w_dtype,
                                            counts, offsets, row_to_slot, y, y_dtype, workspace,
                                            static_cast<hipStream_t>(stream)));
}

int moe_grouped_ffn_noalloc(const void* x, int x_dtype, int64_t T, int32_t K, int32_t H, int32_t F, int32_t E_local,
                            const void* w1, const uint8_t* w1_scale, const void* w2, const uint8_t* w2_scale,
                            int w_dtype, const int32_t* counts, const int32_t* offsets, const int32_t* row_to_slot,
                            void* y, int y_dtype, void* stream) {
  const int st = check_grouped_ffn(x, x_dtype, T, K, H, F, E_local, w1, w1_scale, w2, w2_scale, w_dtype, counts,
                                   offsets, row_to_slot, y, y_dtype);
  if (st != MOE_OK) return st < 0 ? MOE_OK : st;
  // the act rows must fit the scratch array; checked before any HIP call
  if (moe::grouped_ffn_workspace_bytes(T * K, H, F, E_local, w_dtype) > kScratchBytes) return MOE_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  const int sst = scratch_of_current_device(&ws);
  if (sst != MOE_OK) return sst;
  return hip_status(moe::launch_grouped_ffn(x, x_dtype, T, K, H, F, E_local, w1, w1_scale, w2, w2_scale, w_dtype,
                                            counts, offsets, row_to_slot, y, y_dtype, ws,
                                            static_cast<hipStream_t>(stream)));
}

size_t moe_grouped_ffn_control_workspace_bytes(int64_t T, int32_t K, int32_t H, int32_t F, int32_t E_local,
                                               int w_dtype) {
  if (T <= 0 || K <= 0 || F <= 0 || H <= 0 || E_local <= 0) return 0;
  return moe::grouped_ffn_control_workspace_bytes(T * K, H, F, E_local, w_dtype);
}

int moe_grouped_ffn_control(const void* x, int x_dtype, int64_t T, int32_t K, int32_t H, int32_t F,
                            int32_t E_local, const void* w1, const uint8_t* w1_scale, const void* w2,
                            const uint8_t* w2_scale, int w_dtype, const int32_t* counts, const int32_t* offsets,
                            const int32_t* row_to_slot, void* y, int y_dtype, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (T < 0 || K < 1 || H < 1 || F < 1 || E_local < 1) return MOE_ERR_INVALID_ARG;
  if (y_dtype != MOE_F32 && y_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (x_dtype != MOE_BF16 || (w_dtype != MOE_BF16 && w_dtype != MOE_MXFP4)) return MOE_ERR_UNSUPPORTED;
  if (H % 64 != 0 || F % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)K >= ((int64_t)1 << 31) || (int64_t)E_local * (H > F ? H : F) / 64 >= ((int64_t)1 << 31))
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w1 || !w2 || !counts || !offsets || !row_to_slot || !y) return MOE_ERR_INVALID_ARG;
  if (w_dtype == MOE_MXFP4 && (!w1_scale || !w2_scale)) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16) || !aligned(y, 16)) return MOE_ERR_INVALID_ARG;
  const size_t need = moe::grouped_ffn_control_workspace_bytes(T * K, H, F, E_local, w_dtype);
  if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_grouped_ffn_control(x, T, K, H, F, E_local, w1, w1_scale, w2, w2_scale, w_dtype,
                                                    counts, offsets, row_to_slot, y, y_dtype, workspace,
                                                    static_cast<hipStream_t>(stream)));
}

size_t moe_fused_experts_workspace_bytes(int64_t T, int32_t K, int32_t H, int32_t F, int32_t E_local,
                                         int w_dtype) {
  (void)H;
  (void)E_local;
  (void)w_dtype;
  if (T <= 0 || K <= 0 || F <= 0) return 0;
  return moe::fused_experts_workspace_bytes(T * K, F);
}

int moe_fused_experts(const void* x, int x_dtype, int64_t T, int32_t K, int32_t H, int32_t F,
                      const int32_t* topk_ids, const float* topk_weights, const int32_t* expert_map, int32_t E_global,
                      int32_t E_local, const void* w1, const uint8_t* w1_scale, const void* w2,
                      const uint8_t* w2_scale, int w_dtype, int32_t* counts, int32_t* offsets, int32_t* slot_to_row,
                      int32_t* row_to_slot, void* out, int out_dtype, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (T < 0 || K < 1 || H < 1 || F < 1 || E_local < 1 || E_global < 1 || E_local > E_global)
    return MOE_ERR_INVALID_ARG;
  if (!expert_map && E_local != E_global) return MOE_ERR_INVALID_ARG;
  if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (x_dtype != MOE_BF16 || (w_dtype != MOE_BF16 && w_dtype != MOE_MXFP4)) return MOE_ERR_UNSUPPORTED;
  if (H % 32 != 0 || F % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)K > moe::kFusedMaxSlots || E_local > moe::kFusedMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
  if (T > 0) {
    if (!x || !topk_ids || !topk_weights || !w1 || !w2 || !slot_to_row || !row_to_slot || !out)
      return MOE_ERR_INVALID_ARG;
    if (w_dtype == MOE_MXFP4 && (!w1_scale || !w2_scale)) return MOE_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16)) return MOE_ERR_INVALID_ARG;
    const size_t need = moe::fused_experts_workspace_bytes(T * K, F);
    if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return MOE_ERR_INVALID_ARG;
  }
  // T == 0 still defines counts = 0 and offsets = 0
  return hip_status(moe::launch_fused_experts(static_cast<const uint16_t*>(x), T, K, H, F, topk_ids, topk_weights,
                                              expert_map, E_global, E_local, w1, w1_scale, w2, w2_scale, w_dtype,
                                              counts, offsets, slot_to_row, row_to_slot, out, out_dtype, workspace,
                                              static_cast<hipStream_t>(stream)));
}

int moe_pack_ffn_weights(const void* w1, const void* w2, int32_t E_local, int32_t H, int32_t F, void* w1_tiled,
                         void* w2_tiled, void* stream) {
  if (E_local < 1 || H < 1 || F < 1) return MOE_ERR_INVALID_ARG;
  if (H % moe::kPanelRows != 0 || F % (moe::kPanelRows / 2) != 0) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)2 * F * H * 2 >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  if (!w1 || !w2 || !w1_tiled || !w2_tiled) return MOE_ERR_INVALID_ARG;
  if (!aligned(w1, 16) || !aligned(w2, 16) || !aligned(w1_tiled, 16) || !aligned(w2_tiled, 16))
    return MOE_ERR_INVALID_ARG;
  const uintptr_t b1 = (uintptr_t)E_local * 2 * F * H * 2, b2 = (uintptr_t)E_local * H * F * 2;
  auto overlap = [](const void* a, uintptr_t na, const void* b, uintptr_t nb) {
    return (uintptr_t)a < (uintptr_t)b + nb && (uintptr_t)b < (uintptr_t)a + na;
  };
  if (overlap(w1_tiled, b1, w1, b1) || overlap(w1_tiled, b1, w2, b2) || overlap(w2_tiled, b2, w1, b1) ||
      overlap(w2_tiled, b2, w2, b2) || overlap(w1_tiled, b1, w2_tiled, b2))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_pack_ffn_weights(static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w2),
                                                 E_local, H, F, static_cast<uint16_t*>(w1_tiled),
                                                 static_cast<uint16_t*>(w2_tiled), static_cast<hipStream_t>(stream)));
}

int moe_probe_read(const void* src, size_t bytes, uint32_t* out, size_t out_words, void* stream) {
  if (bytes == 0) return MOE_OK;
  if (!src || !out || bytes % 16 != 0 || !aligned(src, 16)) return MOE_ERR_INVALID_ARG;
  if (out_words < (size_t)moe::probe_read_out_words()) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_probe_read(src, (int64_t)bytes, out, static_cast<hipStream_t>(stream)));
}

int moe_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes == 0) return MOE_OK;
  if (!src || !dst || bytes % 16 != 0 || !aligned(src, 16) || !aligned(dst, 16)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_probe_copy(src, dst, (int64_t)bytes, static_cast<hipStream_t>(stream)));
}

int moe_probe_mfma(int64_t iters, int32_t blocks, float* out, void* stream) {
  if (iters < 1 || blocks < 1 || !out) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_probe_mfma(iters, blocks, false, out, nullptr, static_cast<hipStream_t>(stream)));
}

int moe_probe_mfma_clock(int64_t iters, int32_t blocks, int32_t toggle, float* out, uint64_t* clocks, void* stream) {
  if (iters < 1 || blocks < 1 || !out || (toggle != 0 && toggle != 1)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_probe_mfma(iters, blocks, toggle != 0, out,
                                           reinterpret_cast<unsigned long long*>(clocks),
                                           static_cast<hipStream_t>(stream)));
}

int moe_probe_gate_loads(const void* logits, int64_t T, int32_t E, int32_t K, float* topk_weights,
                         int32_t* topk_ids, int32_t* token_expert_indices, void* stream) {
  if (T < 0 || K < 1 || K > 8 || K > E) return MOE_ERR_INVALID_ARG;
  const int V = E / 8;
  if (E % 8 != 0 || (V != 8 && V != 12 && V != 16 && V != 20 && V != 24)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_weights || !topk_ids || !aligned(logits, 16)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_probe_gate_loads(static_cast<const uint16_t*>(logits), T, E, K, topk_weights,
                                                 topk_ids, token_expert_indices, static_cast<hipStream_t>(stream)));
}

int moe_combine(const void* y, int y_dtype, const float* topk_weights, const int32_t* slot_to_row, int64_t T,
                int32_t K, int32_t H, void* out, int out_dtype, void* stream) {
  if (T < 0 || K < 1 || H < 1) return MOE_ERR_INVALID_ARG;
  if ((y_dtype != MOE_F32 && y_dtype != MOE_BF16) || (out_dtype != MOE_F32 && out_dtype != MOE_BF16))
    return MOE_ERR_UNSUPPORTED;
  if (T >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!topk_weights || !slot_to_row || !out) return MOE_ERR_INVALID_ARG;
  // y may be NULL only if nothing is local; that cannot be known on the host
  if (!y) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_combine(y, y_dtype, topk_weights, slot_to_row, T, K, H, out, out_dtype,
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"
