// Internal interfaces between the hs2 host code (abi.hip) and the kernel files.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "hs2.h"

namespace hs2 {

// Candidate list capacity per row for the in-LDS selection fast path.
constexpr int kSelCap = 4096;
// Radix digits of the fp32 score bit pattern: [31:21] [20:10] [9:0].
constexpr int kHistBins = 2048;
// Row segment handled by one select workgroup.
constexpr int kSelSeg = 4096;
constexpr int kSelDigitRows = 64;     // rows from which a launch finds each row's digit once
static_assert(HS2_MAX_SELECT_NMAX == (int64_t)65535 * kSelSeg, "one selection segment per grid row, at most 65535");
constexpr int kBlkMaxCand = 16384;   // candidate blocks per row of the block-level selection
// Query tokens per sequence from which a launch is a query chunk: the full layer takes the chunk
// kernels (8 queries sharing each K/V tile) instead of one row per workgroup, and the sparse layers
// gather with cached loads (the chunk's queries share window rows and often-chosen keys).
constexpr int kPrefillMinTq = 8;

// One attention problem: R = B*Tq query rows, each over a key set given either as the causal
// range [0, t] (list == nullptr) or as an index list idx[r, 0:S].
constexpr int kMaxLayers = 8;        // layers of one multi-layer sparse launch

struct AttnArgs {
    const void* q; int q_dtype;          // [R, H, d]
    const void* k; const void* v; int kv_dtype;
    const float* k_scale; const float* v_scale;
    const int32_t* q_pos;                // [R] (range mode)
    const int32_t* kv_len;               // [B] or nullptr
    const int32_t* list; int S;          // [R, S] (list mode)
    int B, Tq, H, d; int64_t Nmax;
    float scale_log2;                    // sm_scale * log2(e): logits are kept in base 2
    int nsplit; int64_t chunk;           // key entries per split
    // partial results of the splits.  VALU kernels: part [R, nsplit, H, d + 2] (o, m, l).
    // MFMA kernels: part [R, nsplit, H, d] (o) and part_ml [R, nsplit, H, 2] (m, l).
    float* part;
    float* part_ml;
    float* o;                            // [R, H, d]
    float* lse;                          // [R, H] base-2 log-sum-exp (nullptr: not needed)
    uint32_t* zero_hist;                 // [R, kHistBins] to clear (nullptr: none)
    uint32_t* zero_cnt;                  // [R, 4] to clear
    // Several layers over the same K/V and index lists in one launch (nlayer > 1): block row x
    // is row x % R of layer x / R, which takes its Q and O from ql / ol and its partial results
    // at part + layer * part_lstride and part_ml + layer * ml_lstride.
    int nlayer;
    const void* ql[kMaxLayers];
    float* ol[kMaxLayers];
    int64_t part_lstride, ml_lstride;
    // Query chunks: V of every sequence as fp16 V^T images of 32-key sub-tiles (the attention
    // kernel's LDS layout), vt_nsub per sequence, written by vt_prep_kernel before the attention.
    char* vt_img;
    int64_t vt_nsub;
};

struct ScoreArgs {
    const void* q; int q_dtype;
    const void* k; int kv_dtype; const float* k_scale;
    const int32_t* q_pos; const int32_t* kv_len;
    int B, Tq, H, d; int64_t Nmax; int window;
    float scale_log2;
    const float* lse;                    // [R, H]
    float* scores; int64_t cstride;      // [R, cstride]
    int nsplit; int64_t chunk;
    uint32_t* rowhist;                   // [R, kHistBins] or nullptr
    // block-level selection with blocks of one 64-key stage (query-chunk score pass only): the
    // maximum of each stage's scores goes to bscore [R, bstride] instead of the token scores and
    // the histogram (nullptr: token scores)
    float* bscore; int64_t bstride;
};

struct SelectArgs {
    const int32_t* q_pos; const int32_t* kv_len;
    int R, Tq; int64_t Nmax; int k_global, window;
    const float* scores; int64_t cstride;
    uint32_t* rowhist;                   // [R, kHistBins]
    uint32_t* counters;                  // [R, 4]: sure count, candidate count
    int32_t* sure;                       // [R, k_global]
    uint2* cand;                         // [R, kSelCap] (key bits, index)
    uint32_t* digits;                    // [R, 2]: the k-th's top digit and the count above it
    int nseg;
    int32_t* idx;                        // [R, k_global + window]
    float* scores_dbg;                   // [R, Nmax] or nullptr
    // block-level selection (k_global = k_blocks * block)
    int block, k_blocks;
    float* bscore; int64_t bstride;      // [R, bstride] block maxima
    int32_t* block_idx;                  // [R, k_blocks]
};

struct BridgeArgs {
    const uint16_t* hidden; int64_t T; int D;
    const uint16_t* wk; const uint16_t* wv; int d;
    uint16_t* k_out; uint16_t* v_out; int64_t stride;
};

constexpr int kMaxTargets = 8;       // target layers of one multi-target bridge launch

struct BridgeFp8Args {
    const uint16_t* hidden; int64_t T; int D; int d; int L;
    const uint16_t* wk[kMaxTargets]; const uint16_t* wv[kMaxTargets];    // [d, D] each
    uint8_t* k_out[kMaxTargets]; uint8_t* v_out[kMaxTargets];            // row t at t * stride bytes
    float* k_scale[kMaxTargets]; float* v_scale[kMaxTargets];            // [T]
    int64_t stride;
};

// The decode hybrid block in one launch: full layer, split merge, scores, selection, sparse layers.
struct DecodeBlockArgs {
    AttnArgs full;
    ScoreArgs score;
    SelectArgs sel;
    AttnArgs sparse;
};

// Kernel launchers (return the launch status).
hipError_t launch_attn_generic(const AttnArgs& a, const char* name, hipStream_t s);
hipError_t launch_attn_combine(const AttnArgs& a, const char* name, hipStream_t s);
hipError_t launch_score_generic(const ScoreArgs& a, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, bool hist_done, hipStream_t s);
hipError_t launch_select_blocks(const SelectArgs& a, bool maxima_done, hipStream_t s);
hipError_t launch_bridge_mfma(const BridgeArgs& a, hipStream_t s);
bool bridge_rows_fits(const BridgeArgs& a);
hipError_t launch_bridge_rows(const BridgeArgs& a, hipStream_t s);
hipError_t launch_bridge_fp8(const BridgeFp8Args& a, hipStream_t s);
hipError_t launch_decode_block(const DecodeBlockArgs& a, hipStream_t s);
hipError_t launch_attn_rows_mfma(const AttnArgs& a, const char* name, hipStream_t s);
hipError_t launch_attn_split_combine(const AttnArgs& a, const char* name, hipStream_t s);
hipError_t launch_score_rows_mfma(const ScoreArgs& a, hipStream_t s);
hipError_t launch_attn_prefill(const AttnArgs& a, hipStream_t s);
hipError_t launch_score_prefill(const ScoreArgs& a, hipStream_t s);

// Measurement hook: brackets a launch with events on `s` while profiling is enabled.
struct ProfScope {
    ProfScope(const char* name, hipStream_t s);
    ~ProfScope();
    int slot;
    hipStream_t stream;
};

}  // namespace hs2
