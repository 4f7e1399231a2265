/*
 * sgg_lora.h -- chunked SGMV (segmented gather matrix-vector / GEMM) LoRA
 * for AMD Instinct MI355X (gfx950).  Plain C ABI.
 *
 * The operations are the LoRA backend calls of sglang's chunked LoRA
 * backend, as described on the web pages about it:
 *   - the "chunked_backend.py" page, class ChunkedSgmvLoRABackend: the batch
 *     plan (prepare_lora_batch, _determine_chunk_size, _get_permutation,
 *     _get_segments_info, _build_req_seg_indptr) and the kernel calls
 *     (run_lora_a_sgemm, run_lora_b_sgemm, run_qkv_lora, run_gate_up_lora,
 *     run_lora_a_embedding);
 *   - the "base_backend.py" page, class BaseLoRABackend: the shape contract
 *     of every call;
 *   - the "lora_manager.py" page, LoRAManager.prepare_lora_batch: per-slot
 *     rank and scaling tables (rank 0 and scaling 0 mean "no adapter").
 *
 * Notation: s = number of tokens, K = in_dim, c = number of stacked slices,
 * R = padded LoRA rank (the rank dimension of the weight tensors), L =
 * number of adapter slots.  Token t belongs to adapter slot a(t); rho_a =
 * min(lora_ranks[a], R), sigma_a = scalings[a].
 *
 * Conventions shared by every call
 *   - Status: 0 on success, a negative SGG_ERR_* code otherwise;
 *     lora_last_error() then returns a message for the calling thread.
 *   - Ownership: the caller owns every buffer.  The library keeps no state
 *     between calls except the per-thread error message.
 *   - Element type: every floating-point tensor is bf16 (2 bytes, stored as
 *     raw bits) except `scalings` (float32).  Index arrays are int32, token
 *     ids int64.  Accumulation is float32; results are rounded to bf16 with
 *     round-to-nearest-even.
 *   - Layout: row-major.  Activation rows have a leading dimension (ld*, in
 *     elements); weight tensors are dense.  Vector loads need 16-byte
 *     aligned device pointers, K, R, ld* multiples of 8 (else
 *     SGG_ERR_UNSUPPORTED).
 *   - Device calls take device pointers (except where "host" is said),
 *     enqueue work on `stream` (a hipStream_t; NULL = the null stream),
 *     return without synchronising and never allocate memory.  Arguments
 *     are validated on the host before anything is enqueued.  Values that
 *     live in device memory (plan arrays, ranks, ids) are not read by the
 *     host: kernels skip tokens whose permutation entry lies outside
 *     [0, s), treat a segment slot outside [0, L) as rank 0, clamp ranks to
 *     [0, R] and give zeros for token ids outside [0, vocab_size).  A
 *     segment longer than `chunk_size` is still processed in full.
 *   - Row order: h, the output and every activation use the original token
 *     order; `permutation` (sorted position -> token) is only a gather /
 *     scatter index.
 */
#ifndef SGG_LORA_H_
#define SGG_LORA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SGG_OK 0
#define SGG_ERR_INVALID (-1)     /* bad argument: null pointer, bad size, stride, offsets */
#define SGG_ERR_UNSUPPORTED (-2) /* well-formed but not implemented (alignment, extra vocab) */
#define SGG_ERR_CAPACITY (-3)    /* output capacity too small, slot id out of range */
#define SGG_ERR_HIP (-4)         /* the HIP runtime reported an error at launch */

#define SGG_MIN_CHUNK_SIZE 16    /* smallest chunk the heuristic picks */
#define SGG_MAX_SLICES 8         /* most stacked slices one call takes */

/* Message describing the last non-zero status returned on this thread. */
const char* lora_last_error(void);

/*
 * lora_plan_segments -- the batch plan, on the host.
 * (chunked_backend.py page: _determine_chunk_size_for_tokens,
 *  _get_permutation, _get_segments_info, _build_req_seg_indptr, and the
 *  graph branch of prepare_lora_batch for padding.)
 *
 *   seq_lens[num_reqs]    host; tokens per request, >= 0.  May be NULL in
 *                         decode mode (one token per request); in decode
 *                         mode every length must be 1.
 *   req_slots[num_reqs]   host; adapter slot of each request, in [0, max_loras).
 *   is_decode             nonzero: the chunk rule keys on num_reqs;
 *                         zero (extend): it keys on the total token count.
 *   max_chunk_size        the server cap on the chunk size.
 *   chunk_size_override   > 0 forces that chunk size; 0 uses the rule.
 *   permutation[perm_capacity]  out: sorted position -> token index, a stable
 *                         ascending sort of tokens by slot (s entries).
 *   seg_indptr[seg_capacity+1], seg_slots[seg_capacity]  out: CSR segment
 *                         boundaries over sorted positions and each segment's
 *                         slot.  Runs of equal slots are cut into segments of
 *                         chunk tokens with the remainder last.  Entries past
 *                         the segment count are padded: slot 0 and zero
 *                         length (boundary = s).
 *   req_seg_indptr[num_reqs+1]  out (may be NULL): [0, cumsum(seq_lens)].
 *   out_num_segments, out_chunk_size, out_num_tokens  out (each may be NULL).
 * Errors: SGG_ERR_INVALID for bad lengths / sizes, SGG_ERR_CAPACITY when a
 * slot is outside [0, max_loras) or a capacity is too small.  Deterministic:
 * the same inputs always give the same arrays.  Thread-safe.
 */
int lora_plan_segments(const int32_t* seq_lens, const int32_t* req_slots, int32_t num_reqs,
                       int32_t max_loras, int32_t is_decode, int32_t max_chunk_size,
                       int32_t chunk_size_override,
                       int32_t* permutation, int64_t perm_capacity,
                       int32_t* seg_indptr, int32_t* seg_slots, int32_t seg_capacity,
                       int32_t* req_seg_indptr,
                       int32_t* out_num_segments, int32_t* out_chunk_size,
                       int64_t* out_num_tokens);

/*
 * Upper bound on the number of segments of any plan over num_tokens tokens
 * with at most max_loras distinct slots and chunks of at least min_chunk
 * tokens (SGG_MIN_CHUNK_SIZE unless an override is used).  Host only.
 */
int64_t lora_plan_max_segments(int64_t num_tokens, int32_t max_loras, int32_t min_chunk);

/*
 * Plan buffer layout used by lora_plan_upload: int32 regions, each starting
 * at a multiple of 64 elements, in this order:
 *   0 permutation [token_capacity]     1 seg_indptr [seg_capacity + 1]
 *   2 seg_slots [seg_capacity]         3 req_seg_indptr [req_capacity + 1]
 *   4 req_slots [req_capacity]         5 lora_ranks [max_loras]
 *   6 scalings [max_loras] (float32 bits)
 *   7 work_indptr [seg_capacity + 1]   8 work_slots [seg_capacity]
 *   9 work_permutation [token_capacity] (lm_head plans only)
 * lora_plan_layout writes the 10 element offsets to offsets[0..9] and returns
 * the total element count (host only; -1 for negative sizes).
 */
#define SGG_PLAN_REGIONS 10
/* Work segments (regions 7, 8): the plan's segments with consecutive
 * segments of one slot merged while the merged length stays within
 * max(chunk_size, SGG_WORK_SEGMENT_TOKENS).  They partition the same sorted
 * positions, so any kernel call gives the same result with them (and the
 * plan's permutation) as with the plan's segments; with short chunks they let
 * a workgroup reuse an adapter's weights across more tokens.  For an lm_head
 * plan they are built the same way from the pruned tokens sorted by slot (a
 * stable sort), whose permutation is region 9: kernels given region 9 as the
 * permutation and regions 7, 8 as the segments compute the same result as
 * over the lm_head plan itself, without re-reading an adapter's weights for
 * every short run of one adapter. */
#define SGG_WORK_SEGMENT_TOKENS 128
int64_t lora_plan_layout(int64_t token_capacity, int32_t seg_capacity, int32_t req_capacity,
                         int32_t max_loras, int64_t* offsets);

/*
 * lora_plan_upload -- the batch plan (as lora_plan_segments, segment arrays
 * padded to seg_capacity) written into a pinned host staging buffer in the
 * layout above, together with the per-request slots and the per-slot rank
 * and scaling tables, followed by ONE asynchronous host-to-device transfer of
 * the whole buffer to `device_plan` on `stream` (a copy kernel that reads the
 * pinned buffer through its device mapping; a runtime copy if it has none).
 * (chunked_backend.py page: prepare_lora_batch, which plans on the host and
 *  copies the plan arrays to the device without blocking.)
 *
 *   host_staging   pinned host memory (hipHostMalloc) of buffer_bytes bytes,
 *                  8-byte aligned.  The caller must not modify it until the
 *                  copy has read it: wait for done_flag, or for an event
 *                  recorded on `stream` after the call.
 *   device_plan    device memory of buffer_bytes bytes, 8-byte aligned.
 *   buffer_bytes   at least 4 * lora_plan_layout(...).
 *   lora_ranks, scalings  host arrays of max_loras entries.
 *   out_info[6]    host out: num_segments, chunk_size, longest segment,
 *                  num_tokens, number of work segments, longest work segment.
 *   done_flag      NULL, or one int32 of pinned host memory mapped for the
 *                  device: the copy writes done_value there (system scope)
 *                  once it has read the whole staging buffer, so a caller
 *                  that cycles through several staging buffers can tell when
 *                  one is free again by reading host memory, without an
 *                  event.  Not pinned and mapped: SGG_ERR_INVALID.
 * Segment and work-segment arrays are padded to seg_capacity with empty
 * segments of slot 0 (chunked_backend.py page: the CUDA-graph branch of
 * prepare_lora_batch pads the same way).
 * Errors as lora_plan_segments, plus SGG_ERR_CAPACITY when the batch exceeds
 * a capacity and SGG_ERR_HIP when the copy cannot be enqueued.
 */
int lora_plan_upload(const int32_t* seq_lens, const int32_t* req_slots, int32_t num_reqs,
                     const int32_t* lora_ranks, const float* scalings, int32_t max_loras,
                     int32_t is_decode, int32_t max_chunk_size, int32_t chunk_size_override,
                     int64_t token_capacity, int32_t seg_capacity, int32_t req_capacity,
                     void* host_staging, void* device_plan, int64_t buffer_bytes,
                     int32_t* out_info, int32_t* done_flag, int32_t done_value, void* stream);

/*
 * lora_plan_upload_embedding -- lora_plan_upload, then lora_a_embedding of
 * the uploaded batch, with the same results as those two calls: the plan in
 * device_plan, out_info and done_flag exactly as lora_plan_upload, and
 * out[t, j] = A_emb[a(t), j, input_ids[t]] for j < rho_a and in-vocabulary
 * ids (else 0) for the num_tokens tokens of the batch.
 * (chunked_backend.py page: prepare_lora_batch, then run_lora_a_embedding,
 *  the first LoRA call of a forward pass.)
 *
 * For a decode-shaped batch (decode mode, or every seq_lens[r] == 1) of at
 * most 3072 tokens with max_loras <= 64, both are one launch: one workgroup
 * copies the plan while the others do the lookup, taking each token's slot
 * (token t is request t) and the slots' ranks from the call's arguments
 * instead of the plan.  Any other batch gets the two launches of the
 * separate calls.
 *
 *   Plan arguments as lora_plan_upload (same ownership and the same staging
 *   rules: the done flag is raised once the staging buffer has been read).
 *   input_ids  (num_tokens,) int64 (device).
 *   A_emb      (max_loras, R, V) bf16 dense, V >= vocab_size.
 *   out        (num_tokens, R) bf16, row stride ldo >= R.
 *   Ranks above R are taken as R, negative ranks as 0.
 * Errors: as lora_plan_upload and lora_a_embedding; the embedding arguments
 * are checked before anything is planned or enqueued.
 */
int lora_plan_upload_embedding(const int32_t* seq_lens, const int32_t* req_slots,
                               int32_t num_reqs, const int32_t* lora_ranks,
                               const float* scalings, int32_t max_loras, int32_t is_decode,
                               int32_t max_chunk_size, int32_t chunk_size_override,
                               int64_t token_capacity, int32_t seg_capacity,
                               int32_t req_capacity, void* host_staging, void* device_plan,
                               int64_t buffer_bytes, int32_t* out_info, int32_t* done_flag,
                               int32_t done_value, const int64_t* input_ids, const void* A_emb,
                               int64_t V, void* out, int64_t ldo, int32_t R,
                               int64_t vocab_size, void* stream);

/*
 * lora_plan_device -- the batch plan computed on the GPU, as one kernel on
 * `stream`, from request lengths and slots already in device memory.
 * (chunked_backend.py page: the steps of lora_plan_upload -- chunk size,
 *  permutation, segments, request boundaries, graph-capacity padding of the
 *  CUDA-graph branch of prepare_lora_batch.)
 *
 * Writes regions 0-8 of the layout above into `device_plan` (bit for bit the
 * plan lora_plan_upload writes for the same batch and capacities) and
 * out_info's six values, then a status, to device_info[0..6].  Nothing goes
 * through the host and nothing synchronises, so the launch can be captured
 * in a graph with the kernels that read the plan; the caller updates the
 * lengths and slots in device memory between replays.
 *   seq_lens       device int32 [num_reqs]; ignored (one token each) when
 *                  is_decode.
 *   req_slots      device int32 [num_reqs]; lora_ranks, scalings: device
 *                  arrays of max_loras entries.
 *   device_info    device int32 [8].
 * Host-side errors as lora_plan_upload; SGG_ERR_UNSUPPORTED above
 * SGG_DEVICE_PLAN_MAX_REQS requests or SGG_DEVICE_PLAN_MAX_LORAS slots.  A
 * batch that is invalid on the device (slot outside [0, max_loras), negative
 * length, a decode request of other than one token, more tokens or segments
 * than the capacities) is not planned: device_info[6] holds a non-zero
 * status and every segment and work segment is written empty.
 */
#define SGG_DEVICE_PLAN_MAX_REQS 4096
#define SGG_DEVICE_PLAN_MAX_LORAS 1024
int lora_plan_device(const int32_t* seq_lens, const int32_t* req_slots, int32_t num_reqs,
                     const int32_t* lora_ranks, const float* scalings, int32_t max_loras,
                     int32_t is_decode, int32_t max_chunk_size, int32_t chunk_size_override,
                     int64_t token_capacity, int32_t seg_capacity, int32_t req_capacity,
                     void* device_plan, int64_t buffer_bytes, int32_t* device_info,
                     void* stream);

/*
 * lora_plan_lm_head -- plan of a pruned lm_head pass.
 * (chunked_backend.py page: _prepare_lm_head_batch_info and
 *  _build_lm_head_batch_info.)
 *
 * The pruned tokens (pruned_lens[r] of request r, r < num_reqs, requests
 * laid out one after another) stay in original order: permutation[t] = t.
 * Segments: the page's merge_and_chunk_segments, which it imports but does
 * not print, read plainly -- requests with no pruned token are dropped,
 * consecutive requests of one slot form a run, each run is cut into pieces
 * of `chunk` tokens, the remainder last.  The chunk follows the token-count
 * rule over the pruned total (as lora_plan_segments in extend mode), or
 * chunk_size_override when positive.  A per-pass plan (logprob chunking) is
 * this plan over the requests of one pass.  Arrays, capacities, padding and
 * errors as lora_plan_segments (a segment capacity of
 * lora_plan_max_segments(total, num_reqs, min_chunk) always suffices).
 * Host only, synchronous.
 */
int lora_plan_lm_head(const int32_t* pruned_lens, const int32_t* req_slots, int32_t num_reqs,
                      int32_t max_loras, int32_t max_chunk_size, int32_t chunk_size_override,
                      int32_t* permutation, int64_t perm_capacity,
                      int32_t* seg_indptr, int32_t* seg_slots, int32_t seg_capacity,
                      int32_t* out_num_segments, int32_t* out_chunk_size,
                      int64_t* out_num_tokens);

/*
 * lora_plan_lm_head_upload -- as lora_plan_upload, for the lm_head plan of
 * lora_plan_lm_head: the same buffer layout (req_seg_indptr holds the
 * boundaries of each request's pruned tokens), done flag and single transfer
 * on `stream`; the work segments and the work permutation (regions 7-9) come
 * from the pruned tokens sorted by slot.  lora_plan_upload leaves region 9
 * alone and does not transfer it.
 */
int lora_plan_lm_head_upload(const int32_t* pruned_lens, const int32_t* req_slots,
                             int32_t num_reqs, const int32_t* lora_ranks, const float* scalings,
                             int32_t max_loras, int32_t max_chunk_size,
                             int32_t chunk_size_override, int64_t token_capacity,
                             int32_t seg_capacity, int32_t req_capacity, void* host_staging,
                             void* device_plan, int64_t buffer_bytes, int32_t* out_info,
                             int32_t* done_flag, int32_t done_value, void* stream);

/*
 * lora_shrink -- LoRA-A segmented gather GEMM.
 * (chunked_backend.py page: run_lora_a_sgemm, and the shrink step of
 *  run_qkv_lora / run_gate_up_lora; base_backend.py page: run_lora_a_sgemm
 *  shape contract.)
 *
 *   h[t, k*R + j] = sum_{q<K} A[a(t), k*R + j, q] * x[t, q]   for j < rho_a
 *   h[t, k*R + j] = 0                                         for rho_a <= j < R
 * for every slice k < c (c = num_slices).  Rank padding of A is never read.
 *
 *   x          (s, K) bf16, row stride ldx >= K.
 *   A          (L, c*R, K) bf16, dense.
 *   h          (s, c*R) bf16 out, row stride ldh >= c*R.  Every row of every
 *              token covered by the plan is written.
 *   seg_indptr[num_segments+1], seg_slots[num_segments], permutation[s]:
 *              the plan (device memory), as lora_plan_segments makes it.
 *   lora_ranks[L] int32 (device).
 *   chunk_size the plan's chunk size (tiling hint; an upper bound on
 *              segment length for efficiency, not for correctness).
 *   workspace  device scratch of at least lora_shrink_workspace_bytes()
 *              bytes (may be NULL when that is 0).  Its first use must see
 *              it zero-filled; every call leaves it ready for the next one.
 *              Calls that share a workspace must not overlap in time.
 */
int64_t lora_shrink_workspace_bytes(int64_t s, int64_t in_dim, int32_t num_slices, int32_t R,
                                    int32_t num_segments, int32_t chunk_size);
int lora_shrink(const void* x, int64_t ldx, const void* A, void* h, int64_t ldh,
                int64_t s, int64_t in_dim, int32_t num_loras, int32_t num_slices, int32_t R,
                const int32_t* seg_indptr, const int32_t* seg_slots, int32_t num_segments,
                const int32_t* permutation, const int32_t* lora_ranks, int32_t chunk_size,
                void* workspace, int64_t workspace_bytes, void* stream);

/*
 * lora_expand -- LoRA-B segmented gather GEMM with scaling, added in place.
 * (chunked_backend.py page: run_lora_b_sgemm with slice offsets [0, out],
 *  and the expand step of run_qkv_lora / run_gate_up_lora; base_backend.py
 *  page: run_lora_b_sgemm shape contract.)
 *
 *   out[t, o_k + n] += sigma_a * sum_{j < rho_a} B[a, o_k + n, j] * h[t, k*R + j]
 * for slice k < c and n < o_{k+1} - o_k.  Columns at or past o_c and every
 * row of a rank-0 slot are left bit-for-bit unchanged.  Rank padding of B
 * and h never reaches the result (it may hold anything, NaN included): with
 * R <= 32 the B fragments are loaded before the slot's rank is known and
 * their columns past the rank discarded, h rows are staged whole, and only
 * the columns below the rank are used.
 *
 *   h          (s, c*R) bf16, row stride ldh >= c*R.
 *   B          (L, N, R) bf16 dense, N >= o_c.
 *   base_output (s, >= o_c) bf16, row stride ldo, read and written in place.
 *   slice_offsets[num_slices+1]  HOST int32, o_0 = 0, non-decreasing,
 *              1 <= num_slices <= SGG_MAX_SLICES.
 *   max_slice_size  >= the widest slice (a launch bound; results do not
 *              depend on it).
 *   scalings[L] float32 (device).
 */
int lora_expand(const void* h, int64_t ldh, const void* B, int64_t N, void* base_output,
                int64_t ldo, int64_t s, int32_t num_loras, int32_t R,
                const int32_t* slice_offsets, int32_t num_slices, int32_t max_slice_size,
                const int32_t* seg_indptr, const int32_t* seg_slots, int32_t num_segments,
                const int32_t* permutation, const int32_t* lora_ranks, const float* scalings,
                int32_t chunk_size, void* stream);

/*
 * lora_qkv -- stacked LoRA for qkv (c = 3) or gate_up (c = 2) projections:
 * shrink then expand with the same plan.
 * (chunked_backend.py page: run_qkv_lora, run_gate_up_lora;
 *  base_backend.py page: their shape contracts.  A plain projection is
 *  c = 1 with offsets [0, out].)
 *
 *   x (s, K), A (L, c*R, K), B (L, N, R), base_output (s, >= o_c) as in
 *   lora_shrink / lora_expand.  The intermediate h (bf16, s x c*R) lives in
 *   `workspace`, which must hold lora_qkv_workspace_bytes() bytes, zero-
 *   filled on first use, and is not shared by overlapping calls.
 *
 * The call makes two launches, and its result equals lora_shrink followed
 * by lora_expand bit for bit.  A one-launch form exists for small batches
 * (those whose shrink splits K across workgroups, e.g. decode) with
 * c*R <= 48: the expand's workgroups wait for the shrink's workgroups of
 * their segment inside one grid (bounded waits), taken when asked for with
 * lora_set_option("fused_stacked", 1) and when the grid fits on the device at
 * once.  It splits K its own way, so it agrees with the two-launch form to
 * rounding, not bit for bit.  Measured on MI355X it is slower on the decode
 * batch, and it is off by default.
 */
int64_t lora_qkv_workspace_bytes(int64_t s, int64_t in_dim, int32_t num_slices, int32_t R,
                                 int32_t num_segments, int32_t chunk_size);
/* Byte offset, in a lora_qkv workspace, of a 32-bit status word: bit 0 is set
 * (and stays set) once a one-launch stacked call had to give up waiting for
 * its shrink tiles and computed them again itself (the result is the same;
 * see lora_set_option "spin_limit"). */
#define SGG_WORKSPACE_STATUS_OFFSET 65532
int lora_qkv(const void* x, int64_t ldx, const void* A, const void* B, int64_t N,
             void* base_output, int64_t ldo, int64_t s, int64_t in_dim, int32_t num_loras,
             int32_t R, const int32_t* slice_offsets, int32_t num_slices,
             int32_t max_slice_size, const int32_t* seg_indptr, const int32_t* seg_slots,
             int32_t num_segments, const int32_t* permutation, const int32_t* lora_ranks,
             const float* scalings, int32_t chunk_size, void* workspace,
             int64_t workspace_bytes, void* stream);

/*
 * lora_moe_route -- the MoE LoRA add's routing (PR #24007 report page,
 * implementation breakdown items 2-4: the MoE layer takes each token's adapter
 * from the per-request fields req_seg_indptr / req_weight_indices, since the
 * chunked segments are cut per adapter across requests; the MoE LoRA kernel
 * combines adapter and expert into a "virtual expert").  The report names
 * that kernel but does not give its body; this library's reading: copy j of
 * token t goes to virtual expert a(t) * num_experts + topk_ids[t][j], where
 * a(t) = req_weight_indices[r] for the request r with
 * req_seg_indptr[r] <= t < req_seg_indptr[r + 1].
 *   req_seg_indptr      device int32 [num_reqs + 1], non-decreasing.
 *   req_weight_indices  device int32 [num_reqs] adapter slots.
 *   topk_ids            device int32 [num_tokens][top_k] expert ids.
 *   lora_ranks, scalings  device tables of the num_loras adapters.
 *   virtual_slots       device int32 [num_tokens * top_k] out: the copies'
 *                       virtual experts; num_loras * num_experts (a slot of
 *                       rank 0) for a token outside every request, an adapter
 *                       outside [0, num_loras) or an expert outside
 *                       [0, num_experts).
 *   virtual_ranks, virtual_scalings  device [num_loras * num_experts + 1] out:
 *                       adapter a's rank / scaling at every a * E + e, rank 0
 *                       and scaling 0 at the last entry.
 * Plan the copies with lora_plan_device (decode mode: one-token requests,
 * req_slots = virtual_slots, max_loras = num_loras * num_experts + 1) or with
 * the host planner, then call lora_moe_add.  Async on `stream`; errors:
 * SGG_ERR_INVALID (NULL pointers, non-positive counts), SGG_ERR_UNSUPPORTED
 * (sizes beyond int32 indexing), SGG_ERR_HIP.
 */
int lora_moe_route(const int32_t* req_seg_indptr, const int32_t* req_weight_indices,
                   int32_t num_reqs, const int32_t* topk_ids, int64_t num_tokens, int32_t top_k,
                   int32_t num_experts, const int32_t* lora_ranks, const float* scalings,
                   int32_t num_loras, int32_t* virtual_slots, int32_t* virtual_ranks,
                   float* virtual_scalings, void* stream);

/*
 * lora_moe_plan -- lora_moe_route and then lora_plan_device over the copies
 * (decode mode: one-token requests, max_loras = num_loras * num_experts + 1,
 * token and request capacity num_tokens * top_k, no chunk override), in one
 * launch of the device planner, with the same plan: regions 0-8 of the
 * lora_plan_layout(num_tokens * top_k, seg_capacity, num_tokens * top_k,
 * num_loras * num_experts + 1) layout in device_plan, the virtual rank and
 * scaling tables in regions 5 and 6 (no separate virtual arrays), and the
 * counts and status in device_info as lora_plan_device.  Routing inputs as
 * lora_moe_route.
 * (PR #24007 report page: the MoE layer's routing from the per-request
 *  fields; chunked_backend.py page: the plan of prepare_lora_batch.)
 * Limits of the device planner: num_tokens * top_k <= 4096 copies,
 * num_loras * num_experts + 1 <= 1024 (else SGG_ERR_UNSUPPORTED).  Errors
 * as lora_moe_route and lora_plan_device.
 */
int lora_moe_plan(const int32_t* req_seg_indptr, const int32_t* req_weight_indices,
                  int32_t num_reqs, const int32_t* topk_ids, int64_t num_tokens, int32_t top_k,
                  int32_t num_experts, const int32_t* lora_ranks, const float* scalings,
                  int32_t num_loras, int32_t max_chunk_size, int32_t seg_capacity,
                  void* device_plan, int64_t buffer_bytes, int32_t* device_info, void* stream);

/*
 * lora_moe_add -- the MoE LoRA add on a fused-MoE intermediate (reading as in
 * lora_moe_route): for every copy m = t * top_k + j of a plan over the
 * num_tokens * top_k copies (segments by virtual expert v),
 *     out[m, :N] += virtual_scalings[v] * B[v] (A[v] x[t])
 * over the first virtual_ranks[v] rank rows; rows of virtual slots of rank 0
 * (or at or past num_virtual) are unchanged.  It is lora_qkv with one slice
 * and x row t read for the copies t * top_k + j (same kernels, same two
 * launches, same workspace: lora_qkv_workspace_bytes(num_tokens * top_k,
 * in_dim, 1, R, num_segments, chunk_size)).
 *   x     device bf16 (num_tokens, in_dim), row stride ldx.
 *   A     device bf16 (num_virtual, R, in_dim): adapter a's expert e at a*E+e.
 *   B     device bf16 (num_virtual, N, R).
 *   out   device bf16 (num_tokens * top_k, >= N), row stride ldo; read and
 *         written in place.
 *   plan arrays   the device plan of the copies (seg_indptr, seg_slots,
 *         permutation over copies; virtual_ranks / virtual_scalings as
 *         written by lora_moe_route).
 * Errors as lora_qkv.
 */
int lora_moe_add(const void* x, int64_t ldx, int64_t num_tokens, int32_t top_k, const void* A,
                 const void* B, int64_t N, void* out, int64_t ldo, int64_t in_dim,
                 int32_t num_virtual, int32_t R, const int32_t* seg_indptr,
                 const int32_t* seg_slots, int32_t num_segments, const int32_t* permutation,
                 const int32_t* virtual_ranks, const float* virtual_scalings, int32_t chunk_size,
                 void* workspace, int64_t workspace_bytes, void* stream);

/*
 * lora_set_option -- process-wide settings of the device calls; returns the
 * previous value, or -1 for an unknown name.  Not needed for normal use.
 *   "fused_stacked"  0 (default): lora_qkv makes two launches;
 *                    1: one launch where it can (see lora_qkv).
 *   "spin_limit"     polls (about 128 cycles apart) before a one-launch
 *                    stacked call's wait gives up and recomputes (default
 *                    2^20; 0 gives up at once, which tests use to exercise
 *                    that path).
 *   "fused_ksplit"   K ranges of the one-launch call's shrink tiles (0, the
 *                    default: the most that fit; 2..16 forces that many when
 *                    they fit).
 *   "expand_deal_tiles"  1 (default): the expand deals column tiles to the
 *                    XCDs (an adapter's B columns stay in each L2 across its
 *                    segments); 0: it deals segments.  Same results.
 *   "shrink_valu"    0 (default): the shrink computes on the matrix cores;
 *                    1: its split-K kernel takes 16-token tiles and sums the
 *                    dot products of tiles with at most 4 tokens on the
 *                    vector ALU (cross-lane reductions).  Same bytes read,
 *                    results equal to rounding; measured slower, kept for
 *                    comparison.
 *   "shrink_pair_tiles"  0 (default); 1: long-segment batches with c*R
 *                    above 64 (prefill) take shrink tiles of 256 tokens over
 *                    pairs of consecutive same-slot work segments, with K
 *                    split in two (the shrink then needs a split-K workspace,
 *                    see lora_shrink_workspace_bytes).  Results equal to
 *                    rounding; measured slower, kept for comparison.
 *   "fused_trace"    a diagnostic: the device address (as an integer) of a
 *                    zeroed buffer of 32 * "fused_trace_blocks" bytes, or 0
 *                    (default, off).  While set, each one-launch stacked call
 *                    writes, for each of its first "fused_trace_blocks"
 *                    workgroups b, four 64-bit words at word 4b: start time,
 *                    wait-done time (shrink tiles: work-done time; 0 for a
 *                    workgroup with nothing to wait for), end time -- ticks
 *                    of the device's 100 MHz real-time counter -- and its role
 *                    (0 shrink tile, 1 expand tile, 2 expand tile that gave
 *                    up waiting).  One buffer for the process: set it only
 *                    while calls go to the device that holds it.
 *   "fused_trace_blocks"  capacity of the "fused_trace" buffer, in workgroups.
 */
int64_t lora_set_option(const char* name, int64_t value);

/*
 * lora_qkv_noalloc -- lora_qkv without a caller workspace, for callers that
 * cannot allocate device memory (code under graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments and results as
 * lora_qkv (bit for bit), minus the workspace: the library uses a device
 * array of SGG_NOALLOC_SCRATCH_BYTES bytes that each device holds from the
 * first call on it until the process ends.  It calls no allocating routine.
 *
 * Errors: SGG_ERR_CAPACITY when lora_qkv_workspace_bytes() of the call
 * exceeds SGG_NOALLOC_SCRATCH_BYTES (use lora_qkv with a workspace);
 * SGG_ERR_HIP when the array's device address cannot be found; otherwise as
 * lora_qkv.  All calls on one device share the array: calls that overlap in
 * time (other streams, other host threads) race and must not be issued.
 */
#define SGG_NOALLOC_SCRATCH_BYTES (16LL << 20)
int lora_qkv_noalloc(const void* x, int64_t ldx, const void* A, const void* B, int64_t N,
                     void* base_output, int64_t ldo, int64_t s, int64_t in_dim,
                     int32_t num_loras, int32_t R, const int32_t* slice_offsets,
                     int32_t num_slices, int32_t max_slice_size, const int32_t* seg_indptr,
                     const int32_t* seg_slots, int32_t num_segments,
                     const int32_t* permutation, const int32_t* lora_ranks,
                     const float* scalings, int32_t chunk_size, void* stream);

/*
 * lora_a_embedding -- LoRA-A embedding lookup.
 * (chunked_backend.py page: run_lora_a_embedding; base_backend.py page:
 *  run_lora_a_embedding shape contract.)
 *
 *   out[t, j] = A_emb[a(t), j, input_ids[t]]   for j < rho_a and
 *                                              0 <= input_ids[t] < vocab_size
 *   out[t, j] = 0                              otherwise.
 *
 *   input_ids  (s,) int64 (device).
 *   A_emb      (L, R, V) bf16 dense, V >= vocab_size.
 *   out        (s, R) bf16, row stride ldo >= R.
 *   has_extra_embeddings  must be 0: added-vocabulary embeddings are not
 *              supported by the chunked backend (SGG_ERR_UNSUPPORTED).
 */
int lora_a_embedding(const int64_t* input_ids, const void* A_emb, int64_t V, void* out,
                     int64_t ldo, int64_t s, int32_t num_loras, int32_t R,
                     int64_t vocab_size, const int32_t* seg_indptr, const int32_t* seg_slots,
                     int32_t num_segments, const int32_t* permutation,
                     const int32_t* lora_ranks, int32_t has_extra_embeddings, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SGG_LORA_H_ */
