/*
 * moe_routing.h -- C ABI of the MI355X (gfx950) MoE routing + expert-FFN hot path.
 *
 * The library runs one MoE layer's data path on one GPU, in the order of the
 * FusedMoE pipeline "gate -> topk -> expand -> gemm1 -> act -> gemm2 -> combine"
 * (page "Upstream Reference: Deep-Spark xllm + vllm", section "File Index"):
 *
 *   moe_topk_softmax   fused softmax + top-k over router logits
 *   moe_route_compact  per-local-expert row counts, row prefix and the
 *                      slot <-> row permutation of the expert-grouped layout
 *   moe_grouped_ffn    expand (gather) -> GEMM1 -> silu_and_mul -> GEMM2 per
 *                      local expert, weights read once per expert tile
 *   moe_combine        top-k weighted slot-order gather back to token order
 *
 * Conventions shared by every entry point
 *   - Every array argument is caller-owned DEVICE memory (hipMalloc'd or a
 *     torch tensor's data_ptr()), contiguous and row-major, unless stated.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *     enqueued on it; no call synchronises, allocates, frees, or reads device
 *     data on the host, so a sequence of calls can be captured in a graph.
 *   - A slot is s = t*K + k for token t and rank k.  N = T*K slots.
 *   - Return value: MOE_OK, or an error code.  Argument checks run on the
 *     host before anything is launched; on an error nothing is enqueued and
 *     the outputs are untouched.  MOE_ERR_HIP means a launch failed
 *     (moe_last_hip_error() gives the hipError_t).  T == 0 is a valid no-op.
 *   - Device-side preconditions (not checked on the host): logits are
 *     finite; topk_ids lie in [0, E_global); expert_map values lie in
 *     [-1, E_local).  Out-of-range ids or map values are treated as remote
 *     routes (memory-safe, deterministic), never read out of bounds.
 *   - Outputs are deterministic: identical inputs give bit-identical outputs.
 */
#ifndef MOE_ROUTING_H
#define MOE_ROUTING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, negative or inconsistent size */
  MOE_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels implement */
  MOE_ERR_HIP = 3,         /* a HIP launch or device query failed */
  MOE_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
  MOE_ERR_SCRATCH_LIMIT = 5 /* the call needs more than the library's fixed
                               scratch (moe_grouped_ffn_noalloc) */
} moe_status;

typedef enum moe_dtype {
  MOE_F32 = 0,   /* IEEE binary32 */
  MOE_BF16 = 1,  /* bfloat16, round-to-nearest-even on every store */
  MOE_MXFP4 = 2, /* OCP MX FP4 (E2M1) codes, 2 per byte, element 2i in the low
                    nibble, plus one E8M0 scale byte (2^(e-127)) per 32
                    consecutive elements of the reduction dimension.
                    Device-side precondition: no scale byte is 0xFF (NaN in
                    the OCP format); the kernels would read it as an infinite
                    scale */
  MOE_BF16_TILED = 3 /* expert weights in bfloat16, stored in the tile-packed
                        layout written by moe_pack_ffn_weights */
} moe_dtype;

/* Arithmetic of MXFP4 expert GEMMs in the few-rows-per-expert (decode)
 * kernels; see moe_set_mxfp4_mma. */
typedef enum moe_mxfp4_mma {
  MOE_MXFP4_MMA_BF16 = 0,  /* codes widened to bf16 in registers (exact), bf16
                              matrix cores; activations used as given */
  MOE_MXFP4_MMA_F8F6F4 = 1 /* CDNA4 block-scaled matrix cores on the e2m1 codes
                              and their e8m0 scales as stored; activations split
                              per 32 elements into two e4m3 terms (hi + lo) with
                              their own e8m0 scales, which carry them to about
                              2^-9 of the block's largest magnitude */
} moe_mxfp4_mma;

/*
 * moe_topk_softmax -- fused softmax + top-k gate.
 * Source: page "Upstream Reference: Deep-Spark xllm + vllm", section "Call
 * Chain: MoE topk_softmax on BI-V100" (a fused topk_softmax op returning the
 * routing weights, the expert ids and a token-expert index map).
 *
 *   logits               [T, E], MOE_F32 or MOE_BF16 (logits_dtype)
 *   topk_weights (out)   [T, K] float: softmax(logits[t])[topk_ids[t,k]];
 *                        with renormalize != 0 divided by the sum over the
 *                        row's K chosen experts (remote experts included)
 *   topk_ids (out)       [T, K] int32: the K largest logits of the row, best
 *                        first; equal logits rank the lower expert index first
 *   token_expert_indices [T, K] int32 (out, may be NULL): k*T + t, the slot's
 *                        source row in a k-major expanded layout
 * Limits: 1 <= E <= 1280, 1 <= K <= min(E, 32).  Weights are computed in
 * fp32 (max relative error vs exact softmax ~5e-7).
 */
int moe_topk_softmax(const void* logits, int logits_dtype, int64_t T, int32_t E, int32_t K,
                     int32_t renormalize, float* topk_weights, int32_t* topk_ids,
                     int32_t* token_expert_indices, void* stream);

/*
 * moe_topk_sigmoid -- the sigmoid-scoring variant of the gate.
 * Source: page "Upstream Reference: Deep-Spark xllm + vllm", section "File
 * Index" (a sigmoid/softmax top-k dispatcher and a sigmoid variant of the
 * kernel for DeepSeek-style routing).  The page names the variant without
 * defining it; this library's reading: every expert is scored independently
 * by s_j = 1 / (1 + exp(-logit_j)); the top-K experts are those with the
 * largest scores (the logit order, s being increasing; ties -> lower expert
 * index), in descending order; weight_k = s_{id_k}, or with renormalize
 * s_{id_k} / sum_k' s_{id_k'}.  No score bias and no expert groups.
 * Arguments, layout, limits and errors are exactly those of moe_topk_softmax.
 */
int moe_topk_sigmoid(const void* logits, int logits_dtype, int64_t T, int32_t E, int32_t K, int32_t renormalize,
                     float* topk_weights, int32_t* topk_ids, int32_t* token_expert_indices, void* stream);

/*
 * moe_route_compact -- route compaction for one expert-parallel rank.
 * Source: b70-optimization-lab note "MTP1 M2 compact scheduler closure"
 * (2026-07-16), design paragraph: derive each local expert's row count and
 * remapped-row prefix on device from topk_ids plus expert_map, keeping the
 * expert-grouped activation layout; duplicate routes and an all-remote rank
 * are valid inputs.
 *
 *   topk_ids     [T*K] int32 global expert ids
 *   expert_map   [E_global] int32 global -> local id, -1 = remote; NULL means
 *                identity (then E_local must equal E_global)
 *   counts (out)      [E_local] rows routed to each local expert
 *   offsets (out)     [E_local + 1] exclusive prefix of counts; offsets[E_local] = R
 *   slot_to_row (out) [T*K] row of each slot in the grouped layout, -1 if remote
 *   row_to_slot (out) [T*K] inverse: slot of row r for r < R, -1 for r >= R
 * Rows of one expert are in slot order (a stable counting sort by local id);
 * every slot gets its own row, duplicates included.
 * workspace: device scratch of moe_route_compact_workspace_bytes(T, K, E_local)
 * bytes (may be 0 bytes/NULL when that function returns 0).
 * Limits: 1 <= E_local <= 768, E_local <= E_global, T*K < 2^31.
 */
int moe_route_compact(const int32_t* topk_ids, int64_t T, int32_t K, const int32_t* expert_map,
                      int32_t E_global, int32_t E_local, int32_t* counts, int32_t* offsets,
                      int32_t* slot_to_row, int32_t* row_to_slot, void* workspace,
                      size_t workspace_bytes, void* stream);
size_t moe_route_compact_workspace_bytes(int64_t T, int32_t K, int32_t E_local);

/*
 * moe_topk_compact -- the gate and the route compaction of one rank in one
 * call, with the compaction's count pass inside the gate kernel.
 * Sources: page "Upstream Reference: Deep-Spark xllm + vllm", section "Call
 * Chain: MoE topk_softmax on BI-V100" (the gate); b70 lab note "MTP1 M2
 * compact scheduler closure", design paragraph (counts and row prefix on
 * device from topk_ids plus expert_map) and closing paragraph (remove the
 * remap boundary).
 *
 * Computes exactly what moe_topk_softmax (scoring 0) or moe_topk_sigmoid
 * (scoring 1) followed by moe_route_compact compute, bit for bit: the gate
 * outputs, then counts / offsets / slot_to_row / row_to_slot of topk_ids
 * under expert_map (E_global = E, the logits' expert count).  For bf16
 * logits with E in {64, 96, 128, 160, 192}, K = 8 and T*K > 4096 the gate
 * kernel also ranks each block's slots by local expert, so the separate
 * count pass of the compaction disappears; other shapes run the two steps
 * one after the other.
 * Arguments: those of the two calls; workspace as for moe_route_compact
 * (moe_route_compact_workspace_bytes(T, K, E_local)).  Limits and errors:
 * the union of theirs; scoring other than 0 or 1 is MOE_ERR_UNSUPPORTED.
 * T == 0 writes counts = 0 and offsets = 0 only.
 */
int moe_topk_compact(const void* logits, int logits_dtype, int64_t T, int32_t E, int32_t K, int32_t renormalize,
                     int32_t scoring, float* topk_weights, int32_t* topk_ids, int32_t* token_expert_indices,
                     const int32_t* expert_map, int32_t E_local, int32_t* counts, int32_t* offsets,
                     int32_t* slot_to_row, int32_t* row_to_slot, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * moe_route_align -- block-aligned (padded) variant of the expert-grouped
 * layout, for grouped GEMMs that work on fixed-height row blocks.
 * Source: page "Upstream Reference: Deep-Spark xllm + vllm", section "File
 * Index" (a block-alignment kernel for the scatter; named, not defined).
 * Reading: the rows of moe_route_compact, each local expert's rows starting
 * on a multiple of block_size, the unused tail rows of an expert's last block
 * being padding.  N = T*K slots;
 *   cap_rows   = N + E_local * (block_size - 1)
 *   cap_blocks = ceil(N / block_size) + E_local
 * Outputs (device, int32, caller-allocated):
 *   padded_offsets [E_local+1]  expert e owns padded rows
 *                               [padded_offsets[e], padded_offsets[e+1]),
 *                               = counts rounded up to block_size, scanned
 *   sorted_slots   [cap_rows]   slot of each padded row in slot order within
 *                               an expert; -1 for padding and past the end
 *   block_expert   [cap_blocks] local expert of each block; -1 past the end
 *   slot_to_row    [N]          padded row of each slot; -1 for remote slots
 * workspace: moe_route_align_workspace_bytes(T, K, E_local) bytes, 16-byte
 * aligned (the compaction's own arrays live there).
 * Limits: 1 <= block_size <= 4096, E_local <= 768, cap_rows < 2^31.
 */
int moe_route_align(const int32_t* topk_ids, int64_t T, int32_t K, const int32_t* expert_map,
                    int32_t E_global, int32_t E_local, int32_t block_size, int32_t* padded_offsets,
                    int32_t* sorted_slots, int32_t* block_expert, int32_t* slot_to_row, void* workspace,
                    size_t workspace_bytes, void* stream);
size_t moe_route_align_workspace_bytes(int64_t T, int32_t K, int32_t E_local);

/*
 * moe_grouped_ffn -- expert-grouped SwiGLU FFN over the compacted rows.
 * Sources: page "Upstream Reference: Deep-Spark xllm + vllm", section "File
 * Index" (expand -> gemm1 -> act (silu_and_mul) -> gemm2); b70 lab note
 * "MTP1 M2 compact scheduler closure", design paragraph (expert-grouped
 * layout, one weight pass shared by every row routed to the same expert).
 *
 * For every row r < R of the grouped layout, with e the local expert owning
 * r (offsets[e] <= r < offsets[e+1]) and t = row_to_slot[r] / K:
 *   h      = W1[e] x[t]                      (fp32 accumulation)
 *   act    = silu(h[0:F]) * h[F:2F]          silu(g) = g / (1 + exp(-g))
 *   y[r]   = W2[e] act                       (fp32 accumulation)
 *   x        [T, H]            MOE_F32 or MOE_BF16 (x_dtype)
 *   w1       [E_local, 2F, H]  gate rows [0,F), up rows [F,2F); MOE_F32/MOE_BF16,
 *                              or MXFP4 codes [E_local, 2F, H/2] with
 *                              w1_scale [E_local, 2F, H/32]
 *   w2       [E_local, H, F]   or MXFP4 codes [E_local, H, F/2] with
 *                              w2_scale [E_local, H, F/32]
 *   counts, offsets, row_to_slot: as produced by moe_route_compact
 *   y (out)  [T*K, H] (y_dtype MOE_F32 or MOE_BF16); rows >= R are not written
 * Supported (x, w) pairs: (F32, F32), (BF16, BF16), (BF16, MXFP4),
 * (BF16, BF16_TILED); BF16_TILED weights come from moe_pack_ffn_weights and
 * need H % 256 == 0 and F % 128 == 0.
 * The intermediate act is kept in the workspace in bf16 for bf16/MXFP4
 * weights and in fp32 for fp32 weights.  Every sum is taken in a fixed
 * order, so results are deterministic for a given input.
 * workspace: moe_grouped_ffn_workspace_bytes(...) bytes of device scratch,
 * 16-byte aligned.
 * Limits: H and F multiples of 32 for bf16/MXFP4 (of 1 for f32); H, F >= 1.
 */
int moe_grouped_ffn(const void* x, int x_dtype, int64_t T, int32_t K, int32_t H, int32_t F,
                    int32_t E_local, const void* w1, const uint8_t* w1_scale, const void* w2,
                    const uint8_t* w2_scale, int w_dtype, const int32_t* counts,
                    const int32_t* offsets, const int32_t* row_to_slot, void* y, int y_dtype,
                    void* workspace, size_t workspace_bytes, void* stream);
size_t moe_grouped_ffn_workspace_bytes(int64_t T, int32_t K, int32_t H, int32_t F, int32_t E_local,
                                       int w_dtype);

/*
 * moe_grouped_ffn_noalloc -- moe_grouped_ffn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation and the same
 * results, with the act rows kept in a fixed scratch array of the library
 * instead of a caller workspace.  No hipMalloc, hipFree or allocating call is
 * made.
 *
 * Arguments as for moe_grouped_ffn, without workspace and workspace_bytes.
 * Scratch: 64 MiB per GPU (a device array of the library, held by each GPU
 * it runs on until the process ends); the call needs
 * moe_grouped_ffn_workspace_bytes(...) of it -- T*K*F*2 bytes for bf16,
 * MXFP4 and tile-packed weights, T*K*F*4 for f32 -- and returns
 * MOE_ERR_SCRATCH_LIMIT, before anything is enqueued, when that exceeds
 * 64 MiB.  The scratch of the current device is used (the stream must belong
 * to it).  Every call on one GPU shares that GPU's scratch: calls that may
 * overlap on one GPU (different streams without ordering) race and must not
 * be issued.  Nothing in the scratch needs clearing between calls (every act
 * row is written before it is read).
 */
int moe_grouped_ffn_noalloc(const void* x, int x_dtype, int64_t T, int32_t K, int32_t H, int32_t F,
                            int32_t E_local, const void* w1, const uint8_t* w1_scale, const void* w2,
                            const uint8_t* w2_scale, int w_dtype, const int32_t* counts,
                            const int32_t* offsets, const int32_t* row_to_slot, void* y, int y_dtype,
                            void* stream);

/*
 * moe_grouped_ffn_control -- the same FFN as moe_grouped_ffn, run by the
 * generic persistent scheduler that the b70 lab note "MTP1 M2 compact
 * scheduler closure" measures its compact scheduler against (timing
 * paragraph): one block per compute unit claims work items (local expert, N
 * tile of 64 columns) from a global atomic counter, scanning every local
 * expert whether or not any route reached it.  Kept as an A/B control for
 * the compact path; the outputs agree with moe_grouped_ffn within rounding.
 * Arguments as for moe_grouped_ffn; pairs (BF16, BF16) and (BF16, MXFP4);
 * H % 64 == 0, F % 64 == 0.  workspace:
 * moe_grouped_ffn_control_workspace_bytes(...) (the act rows and the two
 * work counters, which the call resets itself).
 */
int moe_grouped_ffn_control(const void* x, int x_dtype, int64_t T, int32_t K, int32_t H, int32_t F,
                            int32_t E_local, const void* w1, const uint8_t* w1_scale, const void* w2,
                            const uint8_t* w2_scale, int w_dtype, const int32_t* counts,
                            const int32_t* offsets, const int32_t* row_to_slot, void* y, int y_dtype,
                            void* workspace, size_t workspace_bytes, void* stream);
size_t moe_grouped_ffn_control_workspace_bytes(int64_t T, int32_t K, int32_t H, int32_t F,
                                               int32_t E_local, int w_dtype);

/*
 * moe_fused_experts -- the layer after the gate for decode batches, with the
 * remap and final-gather boundaries removed: route compaction, grouped SwiGLU
 * FFN and top-k weighted combine in two kernel launches.
 * Source: b70 lab note "MTP1 M2 compact scheduler closure", closing paragraph
 * (next screen: remove the remap and the final permuted gather while keeping
 * compact scheduling and the grouped weight reuse).
 *
 * Computes exactly what moe_route_compact, then moe_grouped_ffn (y in bf16),
 * then moe_combine compute on the same inputs, with the grouped y rows never
 * stored: the first kernel derives the compaction itself from topk_ids and
 * expert_map (and stores it in counts/offsets/slot_to_row/row_to_slot, which
 * are bit-identical to moe_route_compact's), the second adds each token's
 * weighted rows, in ascending k, as soon as its columns are computed.  The
 * reduction of the second GEMM may be split differently from moe_grouped_ffn,
 * so out agrees with the three-call path within rounding (bit-identical when
 * all local rows fall in one 16-row tile).
 *   x [T, H] bf16; topk_ids, topk_weights [T, K]; expert_map as for
 *   moe_route_compact; w1, w2 (+ scales) as for moe_grouped_ffn with w_dtype
 *   MOE_BF16 or MOE_MXFP4; counts [E_local], offsets [E_local+1],
 *   slot_to_row [T*K], row_to_slot [T*K]: outputs as for moe_route_compact;
 *   out [T, H] (out_dtype MOE_BF16 or MOE_F32): partial sum over local routes.
 * workspace: moe_fused_experts_workspace_bytes(...) bytes (the act rows),
 * 16-byte aligned.
 * Limits: T*K <= 64, E_local <= 64, H % 32 == 0, F % 32 == 0
 * (MOE_ERR_UNSUPPORTED otherwise: larger batches take the separate calls).
 * T == 0 writes counts = 0 and offsets = 0 and nothing else.
 */
int moe_fused_experts(const void* x, int x_dtype, int64_t T, int32_t K, int32_t H, int32_t F,
                      const int32_t* topk_ids, const float* topk_weights, const int32_t* expert_map, int32_t E_global,
                      int32_t E_local, const void* w1, const uint8_t* w1_scale, const void* w2,
                      const uint8_t* w2_scale, int w_dtype, int32_t* counts, int32_t* offsets, int32_t* slot_to_row,
                      int32_t* row_to_slot, void* out, int out_dtype, void* workspace, size_t workspace_bytes,
                      void* stream);
size_t moe_fused_experts_workspace_bytes(int64_t T, int32_t K, int32_t H, int32_t F, int32_t E_local,
                                         int w_dtype);

/*
 * Measurement probes -- not steps of the layer.  Each runs one kernel of a
 * known access pattern or instruction mix, so that a benchmark can report
 * what this GPU achieves next to the spec peaks the roofline uses, and the
 * ceiling of the gate's own memory traffic.
 *
 * moe_probe_read: reads bytes of src once (16-byte non-temporal loads, 4096
 *   blocks x 256 threads, grid-stride); each thread folds what it read into
 *   out[thread], so out needs out_words >= 4096*256 (MOE_ERR_WORKSPACE
 *   otherwise).  bytes % 16 == 0, src 16-byte aligned.
 * moe_probe_copy: copies bytes from src to dst with the same loads and
 *   non-temporal stores.  bytes % 16 == 0, both 16-byte aligned.
 * moe_probe_mfma: blocks x 256 threads; every wave issues iters rounds of
 *   four independent v_mfma_f32_32x32x16_bf16 on register operands
 *   (4 x 32768 flops per round); out[blocks*256] receives the sums.  The
 *   operands are loop-invariant constants.
 * moe_probe_mfma_clock: the same loop; toggle = 1 starts the operands from
 *   hashed values in [0.5, 2) with random signs and flips the sign and the 7
 *   mantissa bits of every element each round (half the operand bits change
 *   from one MFMA to the next, as with real data), toggle = 0 keeps the
 *   constants of moe_probe_mfma.  If clocks is not null it receives, per
 *   wave w (blocks*4 waves), clocks[2w] = shader-clock cycles of the loop
 *   (s_memtime) and clocks[2w+1] = 100 MHz reference-clock ticks
 *   (s_memrealtime): their ratio x 100 MHz is the clock the loop ran at.
 *   MOE_ERR_INVALID_ARG for iters < 1, blocks < 1, a null out or toggle
 *   other than 0/1.
 * moe_probe_gate_loads: the memory traffic of moe_topk_softmax's bf16 kernel
 *   for E = 8V, V in {8, 12, 16, 20, 24}, K <= 8 (the same grid, per-lane
 *   loads of the row's logits and K stores of weight, id and token-expert
 *   index per row) without its sort, selection or softmax; the values it
 *   stores are not a gate's.  Source of the access pattern: page "Upstream
 *   Reference: Deep-Spark xllm + vllm", section "Call Chain: MoE topk_softmax
 *   on BI-V100" (the op's inputs and outputs).
 */
int moe_probe_read(const void* src, size_t bytes, uint32_t* out, size_t out_words, void* stream);
int moe_probe_copy(const void* src, void* dst, size_t bytes, void* stream);
int moe_probe_mfma(int64_t iters, int32_t blocks, float* out, void* stream);
int moe_probe_mfma_clock(int64_t iters, int32_t blocks, int32_t toggle, float* out, uint64_t* clocks, void* stream);
int moe_probe_gate_loads(const void* logits, int64_t T, int32_t E, int32_t K, float* topk_weights,
                         int32_t* topk_ids, int32_t* token_expert_indices, void* stream);

/*
 * moe_pack_ffn_weights -- store bf16 expert weights in the tile-packed layout
 * (MOE_BF16_TILED) that the many-rows-per-expert FFN kernels stream with
 * contiguous loads.  A one-time transform of the weights (model load), not
 * part of a layer's pass; the values are unchanged, only their order.
 * Source of the weights' role: page "Upstream Reference: Deep-Spark xllm +
 * vllm", section "File Index" (gemm1 / gemm2 of the FusedMoE pipeline); the
 * layout itself is this library's.
 *
 *   w1 [E_local, 2F, H] bf16, w2 [E_local, H, F] bf16 (row-major, as for
 *   moe_grouped_ffn) -> w1_tiled, w2_tiled: buffers of the same sizes.
 * Layout: per expert, rows are cut into panels of 256 and the reduction
 * dimension into chunks of 32 elements; the 256 x 32 block of (panel,
 * chunk) is stored as 16 KB, chunks of a panel consecutive, panels of an
 * expert consecutive.  Inside a block, panel row R occupies bytes
 * [64 R, 64 R + 64), its 16-byte piece p holding elements 8 (p ^ s(R)) .. +8
 * of the chunk, s(R) = ((R >> 1) ^ (R >> 2)) & 3.  W2 panel nt holds rows
 * 256 nt + R.  W1 panel nt holds, for R = 64 j + 32 g + r (g = 0 gate, 1 up),
 * row g F + 128 nt + 32 j + r.
 * Limits: H % 256 == 0, F % 128 == 0; 16-byte aligned buffers; the outputs
 * must not overlap the inputs.  MOE_ERR_UNSUPPORTED otherwise.
 */
int moe_pack_ffn_weights(const void* w1, const void* w2, int32_t E_local, int32_t H, int32_t F, void* w1_tiled,
                         void* w2_tiled, void* stream);

/*
 * moe_combine -- top-k weighted combine (direct slot-order gather).
 * Source: b70 lab note "MTP1 M2 compact scheduler closure", correctness
 * paragraph (direct slot-order gather as the reference combine) and its
 * next-screen paragraph (the final permuted gather boundary).
 *
 *   out[t, :] = sum over k = 0..K-1 (ascending) with slot_to_row[t*K+k] >= 0
 *               of topk_weights[t, k] * y[slot_to_row[t*K+k], :]
 * fp32 accumulation, one rounding to out_dtype.  Remote slots contribute
 * nothing: this is the partial sum of one expert-parallel rank, and a token
 * with only remote routes gets exact zeros.
 *   y [R, H] (y_dtype), topk_weights [T, K] float, slot_to_row [T*K] int32,
 *   out (out) [T, H] (out_dtype MOE_F32 or MOE_BF16)
 */
int moe_combine(const void* y, int y_dtype, const float* topk_weights, const int32_t* slot_to_row,
                int64_t T, int32_t K, int32_t H, void* out, int out_dtype, void* stream);

/* Human-readable name of a moe_status value (static string). */
/*
 * moe_set_mxfp4_mma / moe_get_mxfp4_mma -- which arithmetic the MXFP4 expert
 * GEMMs take in the decode kernels (fewer than 24 routed slots per local
 * expert: moe_grouped_ffn, moe_grouped_ffn_noalloc, and GEMM1 of
 * moe_fused_experts); larger batches always widen to bf16.  Source: b70 lab
 * note "MTP1 M2 compact scheduler closure", correctness paragraph (the routed
 * MXFP4 expert GEMMs), run here on the matrix-core formats of the target.
 *
 *   mode   a moe_mxfp4_mma value
 *
 * Process-wide; read on the host when a call is launched, so calls already
 * launched (or captured in a graph) keep the arithmetic they were launched
 * with.  Setting it from one thread while another launches MXFP4 calls
 * leaves which of the two those calls take unspecified.  Non-finite
 * activations give NaN outputs under MOE_MXFP4_MMA_F8F6F4.  Default:
 * MOE_MXFP4_MMA_BF16.  Errors: MOE_ERR_INVALID_ARG for another mode.
 */
moe_status moe_set_mxfp4_mma(int mode);
int moe_get_mxfp4_mma(void);

const char* moe_status_string(int status);

/* The hipError_t of the most recent MOE_ERR_HIP on the calling thread (0 if none). */
int moe_last_hip_error(void);

/* Library version string (static). */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTING_H */
