/*
 * hs2.h -- C ABI of the HySparse2 hybrid-block attention hot path on MI355X (gfx950).
 *
 * Three operations, in the order a hybrid block runs them:
 *
 *   hs2_kv_bridge         KV Bridging: a cross-decoder full-attention layer builds its K/V cache
 *                         by projecting self-decoder hidden states with its own K and V
 *                         projections (lynxflow blog, "Two-Level KV Sharing"; agentik-os article,
 *                         section 2 "Two levels of KV sharing"; ainews page, mechanism paragraph).
 *   hs2_full_attn_select  The full-attention MQA layer (one shared KV head: ainews page,
 *                         experimental-setup paragraph) that, on completion, picks per query token
 *                         the 1,024 best-scoring earlier positions one by one plus a forced window
 *                         of the 128 most recent positions (kucoin news flash; lynxflow blog,
 *                         "Token-Level Sparse Selection"; agentik-os article, section 3).
 *   hs2_sparse_attn       A sparse layer of the same hybrid block: it reads the full layer's K/V
 *                         rows and picked positions as they are (KV Reuse: lynxflow "Two-Level KV Sharing";
 *                         agentik-os section 2) and attends over only the selected rows.
 *
 * The pages leave the selection score open (agentik-os, "What is not documented").  This
 * library uses: score(j) = sum over heads h of the full layer's softmax probability p_h(t, j),
 * the softmax running over every visible key 0..t (window included); ties go to the lower j.
 *
 * Conventions shared by every entry point
 *  - Every pointer argument except the stream is a DEVICE pointer unless stated otherwise.
 *    The caller owns all buffers; the library allocates no memory that outlives a call and
 *    never frees caller memory.  hs2_full_attn_select needs scratch memory, which the caller
 *    passes as `workspace` (size from hs2_full_attn_select_workspace_size).
 *  - Every call is asynchronous on `stream` (0 = the null stream) and performs no host/device
 *    synchronisation.  Calls that share a workspace must be ordered on one stream.
 *  - Arguments are validated on the host before any HIP call.  On a non-OK status nothing has
 *    been enqueued and no output was written; hs2_last_error() gives a message.  A failure of
 *    the HIP runtime at launch returns HS2_ERR_HIP.  Faults inside kernels surface at the
 *    caller's next synchronisation.
 *  - Values in device memory (positions, lengths, indices) are not validated on the host.
 *    Kernels never read outside [0, Nmax) rows for them: a query whose position is outside
 *    [0, min(kv_len, Nmax)) produces o = 0 and an all -1 index row; index entries outside
 *    [0, min(kv_len, Nmax)) are skipped like -1.
 *  - Alignment: q, k, v, o, hidden, w_k, w_v and the workspaces start on 16-byte boundaries;
 *    the int32 and fp32 arrays (q_pos, kv_len, idx, scores, k_scale, v_scale) on 4-byte and
 *    k_out / v_out on 2-byte boundaries.  Misaligned pointers return HS2_ERR_INVALID_ARG.
 *  - Layouts are dense and row-major in the order the dimensions are listed.
 *    q: [B, Tq, H, d]; k, v: [B, Nmax, d] (one KV head); k_scale, v_scale: [B, Nmax] fp32;
 *    q_pos: [B, Tq] int32 absolute positions; kv_len: [B] int32 valid cache rows;
 *    o: [B, Tq, H, d] fp32; idx: [B, Tq, k_global + window] int32.
 *  - Supported: d in {64, 128}; 1 <= H <= 32; (q, kv) dtypes (F32, F32), (BF16, BF16) and
 *    (BF16, FP8_E4M3).  Other combinations return HS2_ERR_UNSUPPORTED.  The calls that select
 *    (hs2_full_attn_select, hs2_full_attn_select_blocks, hs2_decode_block) take
 *    Nmax <= HS2_MAX_SELECT_NMAX (65535 selection segments of 4096 keys); larger values return
 *    HS2_ERR_UNSUPPORTED and their workspace-size queries return 0.
 *  - BF16/FP8 paths run on MFMA with fp32 accumulation.  Q.K^T uses the exact bf16 values
 *    (FP8 codes convert to bf16 exactly).  For P.V, calls with Tq < 8 query tokens per
 *    sequence (decode) and hs2_sparse_attn split the attention weights into a bf16 high and
 *    low part against bf16 V (weights kept to about 2^-16 relative); calls with Tq >= 8
 *    (query chunks) use fp16 weights against V converted to fp16 by truncation, which is exact
 *    for bf16 V with |v| in [2^-17, 65504] and 0 (smaller magnitudes lose less than 2^-24, larger
 *    ones clamp to 65504).  Query chunks whose cache rows span 2^31 bytes
 *    or more per sequence (Nmax >= 8M keys at d = 128 in bf16) run on the decode kernels
 *    instead, one query row per workgroup.  fp32 paths compute in fp32 throughout.
 */
#ifndef HS2_H
#define HS2_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

/* Largest cache length (rows per sequence) of the calls that select. */
#define HS2_MAX_SELECT_NMAX ((int64_t)65535 * 4096)

/* Bytes of the static per-GPU scratch that hs2_full_attn_select_noalloc works in (64 MiB). */
#define HS2_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HS2_OK = 0,
    HS2_ERR_INVALID_ARG = -1,   /* null pointer, non-positive or inconsistent size */
    HS2_ERR_UNSUPPORTED = -2,   /* valid but outside the supported set (dtype, d, H) */
    HS2_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required */
    HS2_ERR_HIP = -4            /* the HIP runtime reported an error */
} hs2_status;

typedef enum {
    HS2_F32 = 0,                /* IEEE binary32 */
    HS2_BF16 = 1,               /* bfloat16 */
    HS2_FP8_E4M3 = 2            /* OCP FP8 E4M3FN codes (max 448, no infinities) with a per-row
                                   fp32 scale: value = decode(code) * scale[row]
                                   (FP8 caches: ainews page, experimental-setup paragraph) */
} hs2_dtype;

/*
 * KV Bridging for one target layer (lynxflow "Two-Level KV Sharing": each target layer keeps its
 * own K/V projections; ainews mechanism paragraph).
 *   K[t, c] = bf16_rne( sum_i hidden[t, i] * w_k[i, c] ),  V likewise with w_v,
 * products and sums in fp32, one rounding to bf16 (nearest, ties to even) at the end.  Spans of
 * up to 64 rows (D <= 4096) run a vector-matrix kernel that reads the weights once per four rows;
 * longer spans run MFMA tiles of 256 rows.
 *   hidden : bf16 [T, D] row-major            w_k, w_v : bf16 [D, d] row-major
 *   k_out, v_out : bf16, row t at element offset t * out_row_stride (out_row_stride >= d), so
 *                  the rows can be written straight into a larger cache.
 * Requirements: T >= 0, D >= 1 and D % 64 == 0, d in {64, 128}.  T == 0 is a no-op.
 */
hs2_status hs2_kv_bridge(const void* hidden, int64_t T, int32_t D,
                         const void* w_k, const void* w_v, int32_t d,
                         void* k_out, void* v_out, int64_t out_row_stride,
                         hipStream_t stream);

/*
 * Multi-target KV Bridging into FP8 caches: every cross-decoder full-attention layer (target)
 * projects the same self-decoder hidden states with its own projections (lynxflow "Two-Level KV
 * Sharing"), and its cache is FP8 E4M3FN with a per-row fp32 scale (ainews experimental-setup
 * paragraph).  For each target l = 0..L-1 and row t:
 *   x[c] = sum_i hidden[t, i] * w_k[l][c, i]                     (fp32 accumulation)
 *   k_scale[l][t] = max_c |x[c]| / 448   (1 when the row is all zero)
 *   k_out[l][t * out_row_stride + c] = E4M3FN(x[c] / k_scale[l][t])   (nearest, ties to even,
 *                                                                      saturating at +-448)
 * and V likewise with w_v, v_out, v_scale.  The decoded cache row is code * scale.
 *   hidden : bf16 [T, D] row-major
 *   w_k, w_v : HOST arrays of L device pointers, each bf16 [d, D] (a linear layer's weight:
 *              output row c holds that column's D weights)
 *   k_out, v_out : HOST arrays of L device pointers to u8 codes; row t at byte t * out_row_stride
 *   k_scale, v_scale : HOST arrays of L device pointers to fp32 [T]
 * All targets are computed in one launch.  Targets whose hidden states differ (one source layer
 * each) take one call per hidden buffer.
 * Requirements: 1 <= L <= 8, T >= 0, D % 64 == 0, d in {64, 128}, out_row_stride >= d;
 *   hidden and weights 16-byte aligned, scales 4-byte aligned.  T == 0 is a no-op.
 *   Inputs are finite (a non-finite product gives unspecified codes).
 */
hs2_status hs2_kv_bridge_fp8(const void* hidden, int64_t T, int32_t D,
                             const void* const* w_k, const void* const* w_v, int32_t L, int32_t d,
                             void* const* k_out, void* const* v_out,
                             float* const* k_scale, float* const* v_scale,
                             int64_t out_row_stride, hipStream_t stream);

/*
 * Bytes of workspace hs2_full_attn_select needs for these sizes (0 on invalid sizes).
 * The same value is valid for every call with sizes no larger than these (B, Tq, H, d, Nmax,
 * k_global) and the same KV dtype, whichever kernels that call takes: a size queried for a
 * query chunk also covers decode calls with fewer query tokens.
 */
size_t hs2_full_attn_select_workspace_size(int32_t B, int32_t Tq, int32_t H, int32_t d,
                                           int64_t Nmax, int32_t k_global, int32_t window,
                                           hs2_dtype kv_dtype);

/*
 * Full-attention MQA layer with token-level selection.
 * For query (b, i) at position t = q_pos[b, i], visible keys j = 0..t:
 *   s_h(j) = sm_scale * q_h . k_j,  p_h(j) = softmax_j s_h(j),  o[b,i,h] = sum_j p_h(j) v_j
 *   score(j) = sum_h p_h(j) for the candidates j = 0..t-window (none when t < window)
 *   idx[b,i, 0:k_global]  = the min(k_global, #candidates) best candidates by (score desc,
 *                           j asc), in ascending order, then -1 padding;
 *   idx[b,i, k_global:k_global+window] = max(0, t-window+1) .. t ascending, then -1 padding.
 * scores_dbg (optional, NULL = off): fp32 [B, Tq, Nmax]; entry j holds score(j) for
 *   candidates and -1.0f elsewhere.
 * Requirements: 1 <= k_global <= 4096, 0 <= window <= 4096, sm_scale finite and > 0,
 *   workspace_bytes >= hs2_full_attn_select_workspace_size(...).  k_scale/v_scale are
 *   required for HS2_FP8_E4M3 and must be NULL otherwise.  B == 0 or Tq == 0 is a no-op.
 */
hs2_status hs2_full_attn_select(const void* q, hs2_dtype q_dtype,
                                const void* k, const void* v, hs2_dtype kv_dtype,
                                const float* k_scale, const float* v_scale,
                                const int32_t* q_pos, const int32_t* kv_len,
                                int32_t B, int32_t Tq, int32_t H, int32_t d, int64_t Nmax,
                                int32_t k_global, int32_t window, float sm_scale,
                                float* o, int32_t* idx, float* scores_dbg,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * hs2_full_attn_select for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, and harnesses that forbid hipMalloc.  It computes exactly what
 * hs2_full_attn_select computes (same kernels, same results) but works in a static scratch array
 * that the library holds on every GPU it runs on, HS2_NOALLOC_SCRATCH_BYTES bytes per GPU, from
 * module load until the process ends.  It calls no hipMalloc, hipFree or other allocating routine.
 *   Limit: the sizes must need at most HS2_NOALLOC_SCRATCH_BYTES of workspace
 *   (hs2_full_attn_select_workspace_size); larger ones return HS2_ERR_WORKSPACE before anything is
 *   enqueued (64 MiB covers decode batches up to 64 sequences at 131072 keys).
 *   Every call on one GPU shares that GPU's scratch, whose contents persist between calls: calls
 *   that may overlap on one GPU (different streams, or host threads without ordering) race and
 *   give undefined results; calls ordered on one stream are safe.  The kernels clear what must
 *   start at zero themselves.
 *   The stream must belong to the current device (otherwise HS2_ERR_INVALID_ARG).  The first call
 *   on a device looks up that device's copy of the scratch (a HIP runtime query, no allocation).
 * Other arguments, layouts, requirements and errors as for hs2_full_attn_select.
 */
hs2_status hs2_full_attn_select_noalloc(const void* q, hs2_dtype q_dtype,
                                        const void* k, const void* v, hs2_dtype kv_dtype,
                                        const float* k_scale, const float* v_scale,
                                        const int32_t* q_pos, const int32_t* kv_len,
                                        int32_t B, int32_t Tq, int32_t H, int32_t d, int64_t Nmax,
                                        int32_t k_global, int32_t window, float sm_scale,
                                        float* o, int32_t* idx, float* scores_dbg, hipStream_t stream);

/*
 * Bytes of workspace hs2_full_attn_select_blocks needs for these sizes (0 on invalid sizes);
 * valid for every call with no larger sizes and the same KV dtype, as above.
 */
size_t hs2_full_attn_select_blocks_workspace_size(int32_t B, int32_t Tq, int32_t H, int32_t d,
                                                  int64_t Nmax, int32_t k_blocks, int32_t block,
                                                  int32_t window, hs2_dtype kv_dtype);

/*
 * Full-attention MQA layer with block-level selection: the first-generation scheme that the
 * token-level selection replaces (kucoin news flash: groups of 64 tokens, a group kept whole
 * when any member is important; lynxflow "Token-Level Sparse Selection"), on the same score and
 * the same budget of k_blocks * block positions.
 *   o, score(j), the candidates j = 0..C-1 (C = t-window+1, or 0) and the window: as in
 *   hs2_full_attn_select.
 *   Block b holds the candidates b*block .. min(C, (b+1)*block) - 1; its score is the largest
 *   score(j) of its members.
 *   block_idx[b,i, 0:k_blocks] = the min(k_blocks, #blocks) best blocks by (block score desc,
 *                                block id asc), ascending, then -1 padding;
 *   idx[b,i, 0:k_blocks*block] = every member of those blocks, ascending, then -1 padding;
 *   idx[b,i, k_blocks*block : k_blocks*block+window] = the window, as in hs2_full_attn_select.
 * idx has the token-level layout with k_global = k_blocks * block, so hs2_sparse_attn and
 * hs2_sparse_attn_layers consume it unchanged (S = k_blocks * block + window).
 * Requirements: block a power of two in [1, 64]; 1 <= k_blocks, k_blocks * block <= 4096;
 *   ceil(Nmax / block) <= 16384 (otherwise HS2_ERR_UNSUPPORTED); 0 <= window <= 4096;
 *   workspace_bytes >= hs2_full_attn_select_blocks_workspace_size(...); other arguments as for
 *   hs2_full_attn_select.  block = 1 gives exactly the token-level selection.
 */
hs2_status hs2_full_attn_select_blocks(const void* q, hs2_dtype q_dtype,
                                       const void* k, const void* v, hs2_dtype kv_dtype,
                                       const float* k_scale, const float* v_scale,
                                       const int32_t* q_pos, const int32_t* kv_len,
                                       int32_t B, int32_t Tq, int32_t H, int32_t d, int64_t Nmax,
                                       int32_t k_blocks, int32_t block, int32_t window,
                                       float sm_scale, float* o, int32_t* block_idx, int32_t* idx,
                                       float* scores_dbg, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/*
 * Bytes of workspace hs2_decode_block needs for these sizes (0 on invalid sizes); valid for every
 * call with no larger sizes (B, Tq, H, d, Nmax, k_global, window, L) and the same KV dtype.
 */
size_t hs2_decode_block_workspace_size(int32_t B, int32_t Tq, int32_t H, int32_t d, int64_t Nmax,
                                       int32_t k_global, int32_t window, hs2_dtype kv_dtype, int32_t L);

/*
 * The decode hybrid block in one launch: the full-attention layer with token-level selection
 * (exactly hs2_full_attn_select) followed by L sparse layers on the indices it selected (exactly
 * hs2_sparse_attn_layers with a workspace), as one cooperative kernel launch whose phases are
 * separated by grid-wide barriers (lynxflow "Two-Level KV Sharing": the sparse layers reuse the
 * full layer's cache and indices; ainews page, closing paragraph: the compute saving on paper
 * becomes a wall-clock saving only through the kernels, the memory traffic and the launch order).
 *   q : bf16 [B, Tq, H, d] (the full layer's queries); q_sparse : HOST array of L device pointers
 *   to bf16 [B, Tq, H, d]; o : fp32 [B, Tq, H, d]; idx : int32 [B, Tq, k_global + window];
 *   o_sparse : HOST array of L device pointers to fp32 [B, Tq, H, d].  Everything else as for
 *   hs2_full_attn_select.
 * Results are bit-identical to the two separate calls.  On MI355X the separate calls are faster
 * (phase boundaries inside one launch need device-wide barriers and cache write-back and
 * invalidation that kernel boundaries provide for free); this entry point is for callers that
 * need the block as a single launch.
 * Requirements: bf16 queries, decode rows (Tq < 8), 1 <= L <= 8, k_global + window small enough
 *   for one sparse split (at most 1280 rows per split), workspace_bytes >=
 *   hs2_decode_block_workspace_size(...).  The launch needs every workgroup resident at once:
 *   the GPU must not be shared with work that holds compute units for the duration (the
 *   runtime rejects a cooperative launch that cannot fit, with HS2_ERR_HIP).
 */
hs2_status hs2_decode_block(const void* q, const void* const* q_sparse, int32_t L, hs2_dtype q_dtype,
                            const void* k, const void* v, hs2_dtype kv_dtype,
                            const float* k_scale, const float* v_scale,
                            const int32_t* q_pos, const int32_t* kv_len,
                            int32_t B, int32_t Tq, int32_t H, int32_t d, int64_t Nmax,
                            int32_t k_global, int32_t window, float sm_scale,
                            float* o, int32_t* idx, float* const* o_sparse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Sparse (index-reusing) attention layer (KV Reuse).
 *   o[b,i,h] = sum_{j in sel} softmax_j(sm_scale * q_h . k_j) v_j,
 *   sel = { idx[b,i,e] : 0 <= e < S, 0 <= idx[b,i,e] < min(kv_len[b], Nmax) }.
 * The order of idx entries does not matter; -1 entries are skipped; entries must be unique
 * (a repeated entry is counted once per occurrence).  A row with no valid entry gets o = 0.
 * kv_len may be NULL (then every row < Nmax is valid).  Same dtype rules as above.
 * workspace (optional, may be NULL): scratch of hs2_sparse_attn_workspace_size bytes.
 * Requirements: 1 <= S <= 8192.  B == 0 or Tq == 0 is a no-op.
 */
hs2_status hs2_sparse_attn(const void* q, hs2_dtype q_dtype,
                           const void* k, const void* v, hs2_dtype kv_dtype,
                           const float* k_scale, const float* v_scale,
                           const int32_t* idx, int32_t S, const int32_t* kv_len,
                           int32_t B, int32_t Tq, int32_t H, int32_t d, int64_t Nmax,
                           float sm_scale, float* o,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of optional workspace that let hs2_sparse_attn split each row's index list over
 * several workgroups (used when there are few rows, e.g. decode).  With a NULL or smaller
 * workspace each row is handled by one workgroup; results are the same up to fp32 rounding.
 * The value serves every call with no larger sizes (B, Tq, H, d, S).
 */
size_t hs2_sparse_attn_workspace_size(int32_t B, int32_t Tq, int32_t H, int32_t d, int32_t S);

/*
 * L sparse layers of one hybrid block in one call: every layer reuses the same KV cache and
 * index lists with its own queries (KV Reuse: lynxflow "Two-Level KV Sharing"; agentik-os
 * section 2, where several sparse layers follow one full layer).  Layer l computes exactly
 * what hs2_sparse_attn computes for q[l] into o[l]; on the MFMA paths all layers share one
 * launch of each kernel (the per-layer launches are what bound decode-sized sparse layers).
 * q, o: HOST arrays of L device pointers ([B, Tq, H, d] each); 1 <= L <= 8.
 * workspace (optional): hs2_sparse_attn_layers_workspace_size bytes (L times the per-layer
 * size); with a smaller one every row is handled by one workgroup per layer.
 * Other arguments, requirements and errors as for hs2_sparse_attn.
 */
hs2_status hs2_sparse_attn_layers(const void* const* q, int32_t L, hs2_dtype q_dtype,
                                  const void* k, const void* v, hs2_dtype kv_dtype,
                                  const float* k_scale, const float* v_scale,
                                  const int32_t* idx, int32_t S, const int32_t* kv_len,
                                  int32_t B, int32_t Tq, int32_t H, int32_t d, int64_t Nmax,
                                  float sm_scale, float* const* o,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes for hs2_sparse_attn_layers with L layers (0 if L is outside [1, 8]). */
size_t hs2_sparse_attn_layers_workspace_size(int32_t B, int32_t Tq, int32_t H, int32_t d, int32_t S,
                                             int32_t L);

/* Thread-local message describing the last non-OK status returned on this thread. */
const char* hs2_last_error(void);

/* Library version string. */
const char* hs2_version(void);

/*
 * Per-kernel timing for measurement.  While enabled, every kernel the library launches is
 * bracketed by HIP events recorded on the caller's stream; hs2_profile_read accumulates the
 * elapsed time of each kernel name (it synchronises on the recorded events).  Disabled by
 * default; enabling it adds two event records per launch.  Not thread-safe.
 *   hs2_profile_enable(1) clears earlier records.
 *   hs2_profile_read(i, ...) fills the i-th kernel name's totals; returns 0, or -1 past the end.
 */
void hs2_profile_enable(int enable);
int  hs2_profile_read(int i, const char** name, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* HS2_H */
