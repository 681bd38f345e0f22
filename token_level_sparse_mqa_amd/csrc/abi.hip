// Host side of the hs2 C ABI: argument validation, workspace planning, kernel dispatch,
// error reporting and the optional per-kernel timing hook.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>
#include <vector>

#include "hs2_internal.h"

namespace hs2 {
namespace {

thread_local std::string g_err;

hs2_status fail(hs2_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

hs2_status hip_fail(hipError_t e, const char* where) {
    return fail(HS2_ERR_HIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool dtype_pair_ok(int qd, int kd) {
    return (qd == HS2_F32 && kd == HS2_F32) || (qd == HS2_BF16 && kd == HS2_BF16) ||
           (qd == HS2_BF16 && kd == HS2_FP8_E4M3);
}

// ---- workspace plan of hs2_full_attn_select ----------------------------------------------------
enum Path { PATH_GENERIC = 0, PATH_MFMA_ROWS = 1, PATH_MFMA_PREFILL = 2 };
// The chunk kernels address a sequence's cache rows with 32-bit byte offsets: they take the
// chunk only when Nmax rows of K (or V) span less than 2^31 bytes (8M keys at d = 128 in bf16);
// longer caches take the row kernels, whose offsets are 64-bit.
bool chunk_offsets_fit(int64_t Nmax, int d, int kv_dtype) {
    const int64_t row_bytes = (int64_t)d * (kv_dtype == HS2_FP8_E4M3 ? 1 : 2);
    return Nmax * row_bytes < ((int64_t)1 << 31);
}

struct SelectPlan {
    Path path;
    int64_t R;
    int nsplit; int64_t chunk;         // attention pass over keys
    int score_nsplit; int64_t score_chunk;
    int nseg;
    size_t off_part, off_lse, off_scores, off_hist, off_cnt, off_sure, off_cand, off_digits, off_vt, total;
    int64_t vt_nsub;                    // query chunks: V^T images per sequence (whole 64-key stages)
};

// Split a key range of n entries over workgroups: at least `min_chunk` entries each (a multiple
// of `quant`), and about `target_wg` workgroups over all R rows.
void split_range(int64_t R, int64_t n, int64_t target_wg, int64_t min_chunk, int64_t quant,
                 int* nsplit, int64_t* chunk) {
    int64_t ns = ceil_div(target_wg, R);
    const int64_t ns_max = ceil_div(n, min_chunk);
    if (ns > ns_max) ns = ns_max;
    if (ns < 1) ns = 1;
    int64_t c = ceil_div(ceil_div(n, ns), quant) * quant;
    *chunk = c;
    *nsplit = (int)ceil_div(n, c);
}

SelectPlan plan_select(int B, int Tq, int H, int d, int64_t Nmax, int k_global, int kv_dtype) {
    SelectPlan p{};
    p.R = (int64_t)B * Tq;
    p.path = kv_dtype == HS2_F32 ? PATH_GENERIC
             : (Tq >= kPrefillMinTq && chunk_offsets_fit(Nmax, d, kv_dtype) ? PATH_MFMA_PREFILL : PATH_MFMA_ROWS);
    if (p.path == PATH_MFMA_PREFILL) {
        p.nsplit = 1; p.chunk = Nmax;
        p.score_nsplit = 1; p.score_chunk = Nmax;
    } else if (p.path == PATH_GENERIC) {
        split_range(p.R, Nmax, 4096, 256, 32, &p.nsplit, &p.chunk);
        p.score_nsplit = p.nsplit;
        p.score_chunk = p.chunk;
    } else {
        const int64_t min_chunk = kv_dtype == HS2_FP8_E4M3 ? 2048 : 512;
        // attention: about three workgroups per CU over the pass; score pass: about two (one
        // wave of workgroups, so no workgroup's start-up latency falls into the stream).
        // Both were chosen by measurement on the decode workloads.  The minimum chunk only binds
        // for a few rows (one sequence at 128K keys: 256 workgroups instead of 768).
        split_range(p.R, Nmax, 768, min_chunk, 128, &p.nsplit, &p.chunk);
        split_range(p.R, Nmax, 512, min_chunk, 128, &p.score_nsplit, &p.score_chunk);
    }
    p.nseg = (int)ceil_div(Nmax, kSelSeg);
    size_t off = 0;
    p.off_part = off;   off = align_up(off + (p.nsplit > 1 ? (size_t)p.R * p.nsplit * H * (d + 2) * 4 : 0));
    p.off_lse = off;    off = align_up(off + (size_t)p.R * H * 4);
    p.off_hist = off;   off = off + (size_t)p.R * kHistBins * 4;
    p.off_cnt = off;    off = align_up(off + (size_t)p.R * 4 * 4);
    p.off_sure = off;   off = align_up(off + (size_t)p.R * k_global * 4);
    p.off_cand = off;   off = align_up(off + (size_t)p.R * kSelCap * 8);
    p.off_scores = off; off = align_up(off + (size_t)p.R * Nmax * 4);
    p.off_digits = off; off = align_up(off + (size_t)p.R * 2 * 4);
    // query chunks: every sequence's V as fp16 V^T images of 32-key sub-tiles, d rows of 80 bytes
    p.vt_nsub = p.path == PATH_MFMA_PREFILL ? 2 * ceil_div(Nmax, 64) : 0;
    p.off_vt = off;     off = align_up(off + (size_t)B * p.vt_nsub * d * 80);
    p.total = off;
    return p;
}

// Splits of a sparse layer: about 256 workgroups over its rows, at least 128 list entries each.
// Decode launches (a few rows) reach the limit of 128 entries per split; batches large enough to
// be bandwidth-sized get long chunks and few splits to merge (measured on cold 1152-row
// gathers: 15% faster than planning for 1024 workgroups).  The plan depends on one layer's rows
// only, so a multi-layer launch gives every layer the bytes a one-layer launch gives it.
constexpr int64_t kSparseTargetGroups = 256;
void sparse_plan(int64_t R, int S, int q_dtype, int* nsplit, int64_t* chunk) {
    if (q_dtype == HS2_F32) split_range(R, S, 2048, 64, 32, nsplit, chunk);
    else split_range(R, S, kSparseTargetGroups, 128, 128, nsplit, chunk);
}

size_t sparse_ws_bytes(int64_t R, int H, int d, int S, int q_dtype) {
    int ns; int64_t c;
    sparse_plan(R, S, q_dtype, &ns, &c);
    return ns > 1 ? (size_t)R * ns * H * (d + 2) * 4 : 0;
}

// split_range gives R' rows at most min(ceil(target / R'), ceil(n / min_chunk)) splits each, so
// for every R' <= R and n' <= n the split records number at most
// min(target + R - 1, R * ceil(n / min_chunk)) (0 when no call can split).  The size queries
// use this bound so that one workspace serves every call with no larger sizes, whichever plan
// such a call takes.
int64_t split_records_bound(int64_t R, int64_t n, int64_t target, int64_t min_chunk) {
    const int64_t ns_max = ceil_div(n, min_chunk);
    if (R <= 0 || ns_max <= 1) return 0;
    const int64_t a = target + R - 1, b = R * ns_max;
    return a < b ? a : b;
}

// Workspace bytes of hs2_full_attn_select for every call with sizes no larger than these (same
// KV dtype): the exact plan's later buffers (linear in R, H, Nmax, k_global) after the largest
// split-partial buffer any smaller call can need.  Query chunks (Tq >= 8) plan no partials, but
// a call with fewer query tokens takes the row kernels, which do.
size_t select_ws_bound(int B, int Tq, int H, int d, int64_t Nmax, int k_global, int kv_dtype) {
    const SelectPlan p = plan_select(B, Tq, H, d, Nmax, k_global, kv_dtype);
    const size_t rest = p.total - p.off_lse;
    int64_t R_rows, target, min_chunk;
    if (kv_dtype == HS2_F32) {
        R_rows = p.R; target = 4096; min_chunk = 256;
    } else {
        const int64_t tq_rows = chunk_offsets_fit(Nmax, d, kv_dtype) ? (Tq < kPrefillMinTq ? Tq : kPrefillMinTq - 1) : Tq;
        R_rows = (int64_t)B * tq_rows; target = 1024; min_chunk = kv_dtype == HS2_FP8_E4M3 ? 2048 : 512;
    }
    const size_t part = (size_t)split_records_bound(R_rows, Nmax, target, min_chunk) * H * (d + 2) * 4;
    const size_t own = p.off_lse;
    return align_up(part > own ? part : own) + rest;
}

// Sparse-layer partials for every call with no larger sizes (one layer).
size_t sparse_ws_bound(int64_t R, int H, int d, int S) {
    const int64_t a = split_records_bound(R, S, 2048, 64), b = split_records_bound(R, S, kSparseTargetGroups, 128);
    return (size_t)(a > b ? a : b) * H * (d + 2) * 4;
}

// every kernel reads q/k/v rows, hidden states and weights in 16-byte vectors
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

hs2_status check_common(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype,
                        const float* k_scale, const float* v_scale, int B, int Tq, int H, int d,
                        int64_t Nmax, float sm_scale, const float* o) {
    if (B < 0 || Tq < 0) return fail(HS2_ERR_INVALID_ARG, "B and Tq must be >= 0 (got %d, %d)", B, Tq);
    if (H < 1 || Nmax < 1) return fail(HS2_ERR_INVALID_ARG, "H and Nmax must be >= 1 (got %d, %lld)", H, (long long)Nmax);
    if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return fail(HS2_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
    if (q_dtype < HS2_F32 || q_dtype > HS2_FP8_E4M3 || kv_dtype < HS2_F32 || kv_dtype > HS2_FP8_E4M3)
        return fail(HS2_ERR_INVALID_ARG, "unknown dtype (q %d, kv %d)", q_dtype, kv_dtype);
    if (d != 64 && d != 128) return fail(HS2_ERR_UNSUPPORTED, "head dim d=%d not supported (64 or 128)", d);
    if (H > 32) return fail(HS2_ERR_UNSUPPORTED, "H=%d query heads not supported (at most 32)", H);
    if (!dtype_pair_ok(q_dtype, kv_dtype)) return fail(HS2_ERR_UNSUPPORTED, "dtype pair (q %d, kv %d) not supported", q_dtype, kv_dtype);
    if (kv_dtype == HS2_FP8_E4M3) {
        if (!k_scale || !v_scale) return fail(HS2_ERR_INVALID_ARG, "FP8 KV needs k_scale and v_scale");
    } else if (k_scale || v_scale) {
        return fail(HS2_ERR_INVALID_ARG, "k_scale/v_scale must be NULL unless the KV dtype is FP8");
    }
    if ((int64_t)B * Tq > 0 && (!q || !k || !v || !o)) return fail(HS2_ERR_INVALID_ARG, "null q/k/v/o pointer");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
        return fail(HS2_ERR_INVALID_ARG, "q/k/v/o must be 16-byte aligned");
    if (!aligned(k_scale, 4) || !aligned(v_scale, 4)) return fail(HS2_ERR_INVALID_ARG, "k_scale/v_scale must be 4-byte aligned");
    return HS2_OK;
}

// the selection kernels run one grid row per 4096-key segment of a row
hs2_status check_select_nmax(int64_t Nmax) {
    if (Nmax > HS2_MAX_SELECT_NMAX)
        return fail(HS2_ERR_UNSUPPORTED, "Nmax=%lld: selection supports at most %lld rows per sequence", (long long)Nmax,
                    (long long)HS2_MAX_SELECT_NMAX);
    return HS2_OK;
}

}  // namespace

// ---- measurement hook ------------------------------------------------------------------------
namespace {
struct ProfEntry { std::string name; double ms = 0; int64_t launches = 0; };
struct ProfPending { int entry; hipEvent_t start, stop; };
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfEntry> g_prof;
std::vector<ProfPending> g_pending;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t get_event() {
    if (!g_event_pool.empty()) { hipEvent_t e = g_event_pool.back(); g_event_pool.pop_back(); return e; }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}
}  // namespace

ProfScope::ProfScope(const char* name, hipStream_t s) : slot(-1), stream(s) {
    if (!g_prof_on) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    int entry = -1;
    for (size_t i = 0; i < g_prof.size(); ++i) if (g_prof[i].name == name) entry = (int)i;
    if (entry < 0) { g_prof.push_back(ProfEntry{name}); entry = (int)g_prof.size() - 1; }
    hipEvent_t a = get_event(), b = get_event();
    if (a && b && hipEventRecord(a, s) == hipSuccess) {
        g_pending.push_back(ProfPending{entry, a, b});
        slot = (int)g_pending.size() - 1;
        return;
    }
    // no measurement for this launch (the launch itself is unaffected)
    if (a) g_event_pool.push_back(a);
    if (b) g_event_pool.push_back(b);
}

ProfScope::~ProfScope() {
    if (slot < 0) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (hipEventRecord(g_pending[slot].stop, stream) != hipSuccess) g_pending[slot].entry = -1;
}

}  // namespace hs2

// ---- the static scratch of hs2_full_attn_select_noalloc -------------------------------------------
// One copy per GPU, held from module load until the process ends.  Host code never passes the
// array's name to a kernel or a copy: in host code it is a host-side stand-in, not a device address.
// The address of each device's copy comes from hipGetSymbolAddress with that device current.
static __device__ __align__(256) unsigned char scratch[HS2_NOALLOC_SCRATCH_BYTES];

namespace hs2 {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_addr[kMaxDevices];

// This call's device (the stream's device must be the current one) and its copy of `scratch`,
// looked up on the first call on that device.
hs2_status device_scratch(hipStream_t stream, char** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(HS2_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    if (stream) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
        if (sdev != dev)
            return fail(HS2_ERR_INVALID_ARG, "the stream belongs to device %d but device %d is current", (int)sdev, dev);
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(HS2_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
        g_scratch_addr[dev] = (char*)p;
    }
    *out = g_scratch_addr[dev];
    return HS2_OK;
}
}  // namespace
}  // namespace hs2

using namespace hs2;

extern "C" {

const char* hs2_last_error(void) { return g_err.c_str(); }

const char* hs2_version(void) { return "hs2 0.1.0 (gfx950)"; }

void hs2_profile_enable(int enable) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (enable) {
        for (auto& p : g_pending) {
            if (p.entry >= 0) (void)hipEventSynchronize(p.stop);      // drain; the timings are discarded
            g_event_pool.push_back(p.start);
            g_event_pool.push_back(p.stop);
        }
        g_pending.clear();
        g_prof.clear();
    }
    g_prof_on = enable != 0;
}

int hs2_profile_read(int i, const char** name, double* total_ms, int64_t* launches) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (auto& p : g_pending) {
        float ms = 0.f;
        if (p.entry >= 0 && hipEventSynchronize(p.stop) == hipSuccess &&
            hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
            g_prof[p.entry].ms += ms;
            g_prof[p.entry].launches += 1;
        }
        g_event_pool.push_back(p.start);
        g_event_pool.push_back(p.stop);
    }
    g_pending.clear();
    if (i < 0 || i >= (int)g_prof.size()) return -1;
    if (name) *name = g_prof[i].name.c_str();
    if (total_ms) *total_ms = g_prof[i].ms;
    if (launches) *launches = g_prof[i].launches;
    return 0;
}

hs2_status hs2_kv_bridge(const void* hidden, int64_t T, int32_t D, const void* w_k, const void* w_v, int32_t d,
                         void* k_out, void* v_out, int64_t out_row_stride, hipStream_t stream) {
    if (T < 0) return fail(HS2_ERR_INVALID_ARG, "T must be >= 0");
    if (D < 1 || D % 64 != 0) return fail(HS2_ERR_INVALID_ARG, "D=%d must be a positive multiple of 64", D);
    if (d != 64 && d != 128) return fail(HS2_ERR_UNSUPPORTED, "d=%d not supported (64 or 128)", d);
    if (out_row_stride < d) return fail(HS2_ERR_INVALID_ARG, "out_row_stride %lld < d", (long long)out_row_stride);
    if (T == 0) return HS2_OK;
    if (!hidden || !w_k || !w_v || !k_out || !v_out) return fail(HS2_ERR_INVALID_ARG, "null pointer");
    if (!aligned(hidden, 16) || !aligned(w_k, 16) || !aligned(w_v, 16) || !aligned(k_out, 2) || !aligned(v_out, 2))
        return fail(HS2_ERR_INVALID_ARG, "hidden/w_k/w_v must be 16-byte and k_out/v_out 2-byte aligned");
    BridgeArgs a{(const uint16_t*)hidden, T, D, (const uint16_t*)w_k, (const uint16_t*)w_v, d,
                 (uint16_t*)k_out, (uint16_t*)v_out, out_row_stride};
    // a few rows (a decoded token's) take the vector-matrix kernel, longer spans the MFMA tiles
    hipError_t e = bridge_rows_fits(a) ? launch_bridge_rows(a, stream) : launch_bridge_mfma(a, stream);
    if (e != hipSuccess) return hip_fail(e, "kv_bridge launch");
    return HS2_OK;
}

hs2_status hs2_kv_bridge_fp8(const void* hidden, int64_t T, int32_t D, const void* const* w_k,
                             const void* const* w_v, int32_t L, int32_t d, void* const* k_out, void* const* v_out,
                             float* const* k_scale, float* const* v_scale, int64_t out_row_stride,
                             hipStream_t stream) {
    if (T < 0) return fail(HS2_ERR_INVALID_ARG, "T must be >= 0");
    if (L < 1 || L > kMaxTargets) return fail(HS2_ERR_INVALID_ARG, "L=%d outside [1, %d]", L, kMaxTargets);
    if (D < 1 || D % 64 != 0) return fail(HS2_ERR_INVALID_ARG, "D=%d must be a positive multiple of 64", D);
    if (d != 64 && d != 128) return fail(HS2_ERR_UNSUPPORTED, "d=%d not supported (64 or 128)", d);
    if (out_row_stride < d) return fail(HS2_ERR_INVALID_ARG, "out_row_stride %lld < d", (long long)out_row_stride);
    if (!w_k || !w_v || !k_out || !v_out || !k_scale || !v_scale)
        return fail(HS2_ERR_INVALID_ARG, "null pointer array");
    if (T == 0) return HS2_OK;
    if (!hidden || !aligned(hidden, 16)) return fail(HS2_ERR_INVALID_ARG, "hidden must be non-null and 16-byte aligned");
    BridgeFp8Args a{};
    a.hidden = (const uint16_t*)hidden; a.T = T; a.D = D; a.d = d; a.L = L; a.stride = out_row_stride;
    for (int l = 0; l < L; ++l) {
        if (!w_k[l] || !w_v[l] || !k_out[l] || !v_out[l] || !k_scale[l] || !v_scale[l])
            return fail(HS2_ERR_INVALID_ARG, "null pointer for target %d", l);
        if (!aligned(w_k[l], 16) || !aligned(w_v[l], 16) || !aligned(k_scale[l], 4) || !aligned(v_scale[l], 4))
            return fail(HS2_ERR_INVALID_ARG, "target %d: weights must be 16-byte and scales 4-byte aligned", l);
        a.wk[l] = (const uint16_t*)w_k[l]; a.wv[l] = (const uint16_t*)w_v[l];
        a.k_out[l] = (uint8_t*)k_out[l]; a.v_out[l] = (uint8_t*)v_out[l];
        a.k_scale[l] = k_scale[l]; a.v_scale[l] = v_scale[l];
    }
    for (int l = L; l < kMaxTargets; ++l) {      // unused slots repeat target 0 (never selected)
        a.wk[l] = a.wk[0]; a.wv[l] = a.wv[0]; a.k_out[l] = a.k_out[0]; a.v_out[l] = a.v_out[0];
        a.k_scale[l] = a.k_scale[0]; a.v_scale[l] = a.v_scale[0];
    }
    hipError_t e = launch_bridge_fp8(a, stream);
    if (e != hipSuccess) return hip_fail(e, "kv_bridge_fp8 launch");
    return HS2_OK;
}

size_t hs2_full_attn_select_workspace_size(int32_t B, int32_t Tq, int32_t H, int32_t d, int64_t Nmax,
                                           int32_t k_global, int32_t window, hs2_dtype kv_dtype) {
    (void)window;
    if (B < 0 || Tq < 0 || H < 1 || H > 32 || (d != 64 && d != 128) || Nmax < 1 || Nmax > HS2_MAX_SELECT_NMAX ||
        k_global < 1 || k_global > 4096)
        return 0;
    if ((int64_t)B * Tq == 0) return kAlign;
    return select_ws_bound(B, Tq, H, d, Nmax, k_global, kv_dtype);
}

namespace {

// The full layer up to the token scores: attention (o, per-head log-sum-exp) and the score pass.
// Shared by the token-level and the block-level selection.
hs2_status full_layer(const SelectPlan& p, const void* q, int q_dtype, const void* k, const void* v, int kv_dtype,
                      const float* k_scale, const float* v_scale, const int32_t* q_pos, const int32_t* kv_len,
                      int B, int Tq, int H, int d, int64_t Nmax, int window, float sm_scale, float* o, char* ws,
                      hipStream_t stream, float* bscore = nullptr, int64_t bstride = 0) {
    float* lse = (float*)(ws + p.off_lse);
    float* scores = (float*)(ws + p.off_scores);
    uint32_t* rowhist = (uint32_t*)(ws + p.off_hist);
    uint32_t* counters = (uint32_t*)(ws + p.off_cnt);
    const float scale_log2 = sm_scale * 1.4426950408889634f;

    hipError_t e;
    AttnArgs aa{};
    aa.q = q; aa.q_dtype = q_dtype; aa.k = k; aa.v = v; aa.kv_dtype = kv_dtype;
    aa.k_scale = k_scale; aa.v_scale = v_scale; aa.q_pos = q_pos; aa.kv_len = kv_len;
    aa.list = nullptr; aa.S = 0; aa.B = B; aa.Tq = Tq; aa.H = H; aa.d = d; aa.Nmax = Nmax;
    aa.scale_log2 = scale_log2; aa.nsplit = p.nsplit; aa.chunk = p.chunk;
    aa.part = p.nsplit > 1 ? (float*)(ws + p.off_part) : nullptr;
    aa.part_ml = aa.part ? aa.part + p.R * p.nsplit * H * d : nullptr;   // MFMA layout
    aa.o = o; aa.lse = lse;
    aa.zero_hist = rowhist; aa.zero_cnt = counters;     // cleared by the attention pass
    aa.vt_img = ws + p.off_vt; aa.vt_nsub = p.vt_nsub;
    if (p.path == PATH_GENERIC) {
        e = launch_attn_generic(aa, "full_attn_generic", stream);
        if (e != hipSuccess) return hip_fail(e, "attention launch");
        if (p.nsplit > 1) e = launch_attn_combine(aa, "full_attn_combine", stream);
    } else if (p.path == PATH_MFMA_PREFILL) {
        e = launch_attn_prefill(aa, stream);
    } else {
        e = launch_attn_rows_mfma(aa, "full_attn_mfma", stream);
        if (e != hipSuccess) return hip_fail(e, "attention launch");
        if (p.nsplit > 1) e = launch_attn_split_combine(aa, "full_attn_combine", stream);
    }
    if (e != hipSuccess) return hip_fail(e, "attention combine launch");

    ScoreArgs sa{};
    sa.q = q; sa.q_dtype = q_dtype; sa.k = k; sa.kv_dtype = kv_dtype; sa.k_scale = k_scale;
    sa.q_pos = q_pos; sa.kv_len = kv_len; sa.B = B; sa.Tq = Tq; sa.H = H; sa.d = d; sa.Nmax = Nmax;
    sa.window = window; sa.scale_log2 = scale_log2; sa.lse = lse; sa.scores = scores; sa.cstride = Nmax;
    sa.nsplit = p.score_nsplit; sa.chunk = p.score_chunk; sa.rowhist = bscore ? nullptr : rowhist;
    sa.bscore = bscore; sa.bstride = bstride;
    e = p.path == PATH_GENERIC ? launch_score_generic(sa, stream)
        : p.path == PATH_MFMA_PREFILL ? launch_score_prefill(sa, stream) : launch_score_rows_mfma(sa, stream);
    if (e != hipSuccess) return hip_fail(e, "score launch");
    return HS2_OK;
}

SelectArgs select_args(const SelectPlan& p, char* ws, const int32_t* q_pos, const int32_t* kv_len, int Tq,
                       int64_t Nmax, int k_global, int window, int32_t* idx, float* scores_dbg) {
    SelectArgs se{};
    se.q_pos = q_pos; se.kv_len = kv_len; se.R = (int)p.R; se.Tq = Tq; se.Nmax = Nmax;
    se.k_global = k_global; se.window = window; se.scores = (float*)(ws + p.off_scores); se.cstride = Nmax;
    se.rowhist = (uint32_t*)(ws + p.off_hist); se.counters = (uint32_t*)(ws + p.off_cnt);
    se.sure = (int32_t*)(ws + p.off_sure); se.cand = (uint2*)(ws + p.off_cand); se.nseg = p.nseg;
    se.digits = (uint32_t*)(ws + p.off_digits);
    se.idx = idx; se.scores_dbg = scores_dbg;
    return se;
}

// the block maxima follow the token-level plan's workspace
size_t block_ws_extra(int64_t R, int64_t Nmax, int block) {
    return align_up((size_t)R * (size_t)((Nmax + block - 1) / block) * 4);
}

}  // namespace

namespace {

// Host validation shared by hs2_full_attn_select and its variant that allocates nothing.
hs2_status check_full_attn_select(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype,
                                  const float* k_scale, const float* v_scale, const int32_t* q_pos,
                                  const int32_t* kv_len, int B, int Tq, int H, int d, int64_t Nmax, int k_global,
                                  int window, float sm_scale, const float* o, const int32_t* idx,
                                  const float* scores_dbg) {
    hs2_status st = check_common(q, q_dtype, k, v, kv_dtype, k_scale, v_scale, B, Tq, H, d, Nmax, sm_scale, o);
    if (st == HS2_OK) st = check_select_nmax(Nmax);
    if (st != HS2_OK) return st;
    if (k_global < 1 || k_global > 4096) return fail(HS2_ERR_INVALID_ARG, "k_global=%d outside [1, 4096]", k_global);
    if (window < 0 || window > 4096) return fail(HS2_ERR_INVALID_ARG, "window=%d outside [0, 4096]", window);
    if ((int64_t)B * Tq == 0) return HS2_OK;
    if (!q_pos || !kv_len || !idx) return fail(HS2_ERR_INVALID_ARG, "null q_pos/kv_len/idx pointer");
    if (!aligned(q_pos, 4) || !aligned(kv_len, 4) || !aligned(idx, 4) || !aligned(scores_dbg, 4))
        return fail(HS2_ERR_INVALID_ARG, "q_pos/kv_len/idx/scores_dbg must be 4-byte aligned");
    return HS2_OK;
}

// The full layer and the token-level selection on a validated call, with the plan's workspace at ws.
hs2_status run_full_attn_select(const SelectPlan& p, const void* q, int q_dtype, const void* k, const void* v,
                                int kv_dtype, const float* k_scale, const float* v_scale, const int32_t* q_pos,
                                const int32_t* kv_len, int B, int Tq, int H, int d, int64_t Nmax, int k_global,
                                int window, float sm_scale, float* o, int32_t* idx, float* scores_dbg, char* ws,
                                hipStream_t stream) {
    hs2_status st = full_layer(p, q, q_dtype, k, v, kv_dtype, k_scale, v_scale, q_pos, kv_len, B, Tq, H, d, Nmax,
                               window, sm_scale, o, ws, stream);
    if (st != HS2_OK) return st;
    const SelectArgs se = select_args(p, ws, q_pos, kv_len, Tq, Nmax, k_global, window, idx, scores_dbg);
    hipError_t e = launch_select(se, /*hist_done=*/true, stream);
    if (e != hipSuccess) return hip_fail(e, "select launch");
    return HS2_OK;
}

}  // namespace

hs2_status hs2_full_attn_select(const void* q, hs2_dtype q_dtype, const void* k, const void* v, hs2_dtype kv_dtype,
                                const float* k_scale, const float* v_scale, const int32_t* q_pos,
                                const int32_t* kv_len, int32_t B, int32_t Tq, int32_t H, int32_t d, int64_t Nmax,
                                int32_t k_global, int32_t window, float sm_scale, float* o, int32_t* idx,
                                float* scores_dbg, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    hs2_status st = check_full_attn_select(q, q_dtype, k, v, kv_dtype, k_scale, v_scale, q_pos, kv_len, B, Tq, H, d,
                                           Nmax, k_global, window, sm_scale, o, idx, scores_dbg);
    if (st != HS2_OK || (int64_t)B * Tq == 0) return st;
    if (!aligned(workspace, 16)) return fail(HS2_ERR_INVALID_ARG, "the workspace must be 16-byte aligned");
    const SelectPlan p = plan_select(B, Tq, H, d, Nmax, k_global, kv_dtype);
    if (!workspace || workspace_bytes < p.total)
        return fail(HS2_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", p.total, workspace ? workspace_bytes : (size_t)0);
    return run_full_attn_select(p, q, q_dtype, k, v, kv_dtype, k_scale, v_scale, q_pos, kv_len, B, Tq, H, d, Nmax,
                                k_global, window, sm_scale, o, idx, scores_dbg, (char*)workspace, stream);
}

hs2_status hs2_full_attn_select_noalloc(const void* q, hs2_dtype q_dtype, const void* k, const void* v,
                                        hs2_dtype kv_dtype, const float* k_scale, const float* v_scale,
                                        const int32_t* q_pos, const int32_t* kv_len, int32_t B, int32_t Tq, int32_t H,
                                        int32_t d, int64_t Nmax, int32_t k_global, int32_t window, float sm_scale,
                                        float* o, int32_t* idx, float* scores_dbg, hipStream_t stream) {
    hs2_status st = check_full_attn_select(q, q_dtype, k, v, kv_dtype, k_scale, v_scale, q_pos, kv_len, B, Tq, H, d,
                                           Nmax, k_global, window, sm_scale, o, idx, scores_dbg);
    if (st != HS2_OK || (int64_t)B * Tq == 0) return st;
    const SelectPlan p = plan_select(B, Tq, H, d, Nmax, k_global, kv_dtype);
    if (p.total > (size_t)HS2_NOALLOC_SCRATCH_BYTES)
        return fail(HS2_ERR_WORKSPACE, "these sizes need %zu bytes of scratch; the static scratch holds %zu "
                    "(use hs2_full_attn_select with a workspace)", p.total, (size_t)HS2_NOALLOC_SCRATCH_BYTES);
    char* ws = nullptr;
    st = device_scratch(stream, &ws);
    if (st != HS2_OK) return st;
    return run_full_attn_select(p, q, q_dtype, k, v, kv_dtype, k_scale, v_scale, q_pos, kv_len, B, Tq, H, d, Nmax,
                                k_global, window, sm_scale, o, idx, scores_dbg, ws, stream);
}

size_t hs2_full_attn_select_blocks_workspace_size(int32_t B, int32_t Tq, int32_t H, int32_t d, int64_t Nmax,
                                                  int32_t k_blocks, int32_t block, int32_t window,
                                                  hs2_dtype kv_dtype) {
    (void)window;
    if (block < 1 || block > 64 || (block & (block - 1)) || k_blocks < 1 || (int64_t)k_blocks * block > 4096)
        return 0;
    if (B < 0 || Tq < 0 || H < 1 || H > 32 || (d != 64 && d != 128) || Nmax < 1 || Nmax > HS2_MAX_SELECT_NMAX) return 0;
    if ((Nmax + block - 1) / block > kBlkMaxCand) return 0;
    if ((int64_t)B * Tq == 0) return kAlign;
    return select_ws_bound(B, Tq, H, d, Nmax, k_blocks * block, kv_dtype) +
           block_ws_extra((int64_t)B * Tq, Nmax, block);
}

hs2_status hs2_full_attn_select_blocks(const void* q, hs2_dtype q_dtype, const void* k, const void* v,
                                       hs2_dtype kv_dtype, const float* k_scale, const float* v_scale,
                                       const int32_t* q_pos, const int32_t* kv_len, int32_t B, int32_t Tq,
                                       int32_t H, int32_t d, int64_t Nmax, int32_t k_blocks, int32_t block,
                                       int32_t window, float sm_scale, float* o, int32_t* block_idx, int32_t* idx,
                                       float* scores_dbg, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
    hs2_status st = check_common(q, q_dtype, k, v, kv_dtype, k_scale, v_scale, B, Tq, H, d, Nmax, sm_scale, o);
    if (st == HS2_OK) st = check_select_nmax(Nmax);
    if (st != HS2_OK) return st;
    if (block < 1 || block > 64 || (block & (block - 1)))
        return fail(HS2_ERR_INVALID_ARG, "block=%d must be a power of two in [1, 64]", block);
    if (k_blocks < 1 || (int64_t)k_blocks * block > 4096)
        return fail(HS2_ERR_INVALID_ARG, "k_blocks=%d: need 1 <= k_blocks and k_blocks * block <= 4096", k_blocks);
    if (window < 0 || window > 4096) return fail(HS2_ERR_INVALID_ARG, "window=%d outside [0, 4096]", window);
    if ((Nmax + block - 1) / block > kBlkMaxCand)
        return fail(HS2_ERR_UNSUPPORTED, "Nmax=%lld: at most %d blocks per row", (long long)Nmax, kBlkMaxCand);
    if ((int64_t)B * Tq == 0) return HS2_OK;
    if (!q_pos || !kv_len || !idx || !block_idx) return fail(HS2_ERR_INVALID_ARG, "null q_pos/kv_len/idx/block_idx pointer");
    if (!aligned(q_pos, 4) || !aligned(kv_len, 4) || !aligned(idx, 4) || !aligned(block_idx, 4) ||
        !aligned(scores_dbg, 4) || !aligned(workspace, 16))
        return fail(HS2_ERR_INVALID_ARG, "q_pos/kv_len/idx/block_idx/scores_dbg must be 4-byte and the workspace 16-byte aligned");
    const int K = k_blocks * block;
    const SelectPlan p = plan_select(B, Tq, H, d, Nmax, K, kv_dtype);
    const size_t need = p.total + block_ws_extra(p.R, Nmax, block);
    if (!workspace || workspace_bytes < need)
        return fail(HS2_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
    char* ws = (char*)workspace;
    float* bscore = (float*)(ws + p.total);
    const int64_t bstride = (Nmax + block - 1) / block;
    // query chunks with blocks of 64 keys (one score-pass stage): the score pass writes the block
    // maxima itself, unless the token scores are asked for
    const bool stage_blocks = block == 64 && p.path == PATH_MFMA_PREFILL && !scores_dbg;
    st = full_layer(p, q, q_dtype, k, v, kv_dtype, k_scale, v_scale, q_pos, kv_len, B, Tq, H, d, Nmax, window,
                    sm_scale, o, ws, stream, stage_blocks ? bscore : nullptr, bstride);
    if (st != HS2_OK) return st;
    SelectArgs se = select_args(p, ws, q_pos, kv_len, Tq, Nmax, K, window, idx, scores_dbg);
    se.block = block; se.k_blocks = k_blocks;
    se.bscore = bscore; se.bstride = bstride;
    se.block_idx = block_idx;
    hipError_t e = launch_select_blocks(se, stage_blocks, stream);
    if (e != hipSuccess) return hip_fail(e, "block select launch");
    return HS2_OK;
}

// ---- the decode hybrid block in one launch ------------------------------------------------------

namespace {

struct DecodeBlockPlan {
    SelectPlan sel;
    int sp_nsplit; int64_t sp_chunk;
    size_t off_sparse, total;
};

DecodeBlockPlan plan_decode_block(int B, int Tq, int H, int d, int64_t Nmax, int k_global, int window,
                                  int kv_dtype, int L) {
    DecodeBlockPlan p{};
    p.sel = plan_select(B, Tq, H, d, Nmax, k_global, kv_dtype);
    const int64_t R = (int64_t)B * Tq;
    const int S = k_global + window;
    sparse_plan(R, S, HS2_BF16, &p.sp_nsplit, &p.sp_chunk);
    p.off_sparse = p.sel.total;
    const size_t sp = p.sp_nsplit > 1 ? (size_t)L * R * p.sp_nsplit * H * (d + 2) * 4 : 0;
    p.total = p.off_sparse + align_up(sp);
    return p;
}

}  // namespace

size_t hs2_decode_block_workspace_size(int32_t B, int32_t Tq, int32_t H, int32_t d, int64_t Nmax,
                                       int32_t k_global, int32_t window, hs2_dtype kv_dtype, int32_t L) {
    if (B < 0 || Tq < 0 || Tq >= kPrefillMinTq || H < 1 || H > 32 || (d != 64 && d != 128) || Nmax < 1 ||
        Nmax > HS2_MAX_SELECT_NMAX ||
        k_global < 1 || k_global > 4096 || window < 0 || window > 4096 || L < 1 || L > kMaxLayers)
        return 0;
    if ((int64_t)B * Tq == 0) return kAlign;
    // every smaller call's own plan fits: the selection bound, then L layers' sparse partials
    const int64_t R = (int64_t)B * Tq;
    return select_ws_bound(B, Tq, H, d, Nmax, k_global, kv_dtype) +
           align_up((size_t)L * split_records_bound(R, (int64_t)k_global + window, kSparseTargetGroups, 128) * H * (d + 2) * 4);
}

hs2_status hs2_decode_block(const void* q, const void* const* q_sparse, int32_t L, hs2_dtype q_dtype,
                            const void* k, const void* v, hs2_dtype kv_dtype, const float* k_scale,
                            const float* v_scale, const int32_t* q_pos, const int32_t* kv_len, int32_t B,
                            int32_t Tq, int32_t H, int32_t d, int64_t Nmax, int32_t k_global, int32_t window,
                            float sm_scale, float* o, int32_t* idx, float* const* o_sparse, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    hs2_status st = check_common(q, q_dtype, k, v, kv_dtype, k_scale, v_scale, B, Tq, H, d, Nmax, sm_scale, o);
    if (st == HS2_OK) st = check_select_nmax(Nmax);
    if (st != HS2_OK) return st;
    if (q_dtype != HS2_BF16) return fail(HS2_ERR_UNSUPPORTED, "the single-launch block takes bf16 queries");
    if (Tq >= kPrefillMinTq) return fail(HS2_ERR_UNSUPPORTED, "Tq=%d: the single-launch block is for decode rows (Tq < %d)", Tq, kPrefillMinTq);
    if (!q_sparse || !o_sparse) return fail(HS2_ERR_INVALID_ARG, "null q_sparse or o_sparse pointer array");
    if (L < 1 || L > kMaxLayers) return fail(HS2_ERR_INVALID_ARG, "L=%d outside [1, %d]", L, kMaxLayers);
    if (k_global < 1 || k_global > 4096) return fail(HS2_ERR_INVALID_ARG, "k_global=%d outside [1, 4096]", k_global);
    if (window < 0 || window > 4096) return fail(HS2_ERR_INVALID_ARG, "window=%d outside [0, 4096]", window);
    for (int l = 0; l < L; ++l) {
        st = check_common(q_sparse[l], q_dtype, k, v, kv_dtype, k_scale, v_scale, B, Tq, H, d, Nmax, sm_scale, o_sparse[l]);
        if (st != HS2_OK) return st;
    }
    if ((int64_t)B * Tq == 0) return HS2_OK;
    if (!q_pos || !kv_len || !idx) return fail(HS2_ERR_INVALID_ARG, "null q_pos/kv_len/idx pointer");
    if (!aligned(q_pos, 4) || !aligned(kv_len, 4) || !aligned(idx, 4) || !aligned(workspace, 16))
        return fail(HS2_ERR_INVALID_ARG, "q_pos/kv_len/idx must be 4-byte and the workspace 16-byte aligned");
    const DecodeBlockPlan p = plan_decode_block(B, Tq, H, d, Nmax, k_global, window, kv_dtype, L);
    if (p.sp_chunk > 1280)     // list entries one workgroup of the row kernel stages
        return fail(HS2_ERR_UNSUPPORTED, "k_global + window = %d: a sparse split holds at most 1280 rows", k_global + window);
    if (!workspace || workspace_bytes < p.total)
        return fail(HS2_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", p.total, workspace ? workspace_bytes : (size_t)0);
    char* ws = (char*)workspace;
    const int64_t R = (int64_t)B * Tq;
    const float scale_log2 = sm_scale * 1.4426950408889634f;
    DecodeBlockArgs a{};
    // full layer, as hs2_full_attn_select's row path
    AttnArgs& f = a.full;
    f.q = q; f.q_dtype = q_dtype; f.k = k; f.v = v; f.kv_dtype = kv_dtype; f.k_scale = k_scale; f.v_scale = v_scale;
    f.q_pos = q_pos; f.kv_len = kv_len; f.list = nullptr; f.S = 0; f.B = B; f.Tq = Tq; f.H = H; f.d = d; f.Nmax = Nmax;
    f.scale_log2 = scale_log2; f.nsplit = p.sel.nsplit; f.chunk = p.sel.chunk;
    f.part = p.sel.nsplit > 1 ? (float*)(ws + p.sel.off_part) : nullptr;
    f.part_ml = f.part ? f.part + R * p.sel.nsplit * H * d : nullptr;
    f.o = o; f.lse = (float*)(ws + p.sel.off_lse); f.nlayer = 1;
    f.zero_hist = (uint32_t*)(ws + p.sel.off_hist); f.zero_cnt = (uint32_t*)(ws + p.sel.off_cnt);
    ScoreArgs& sa = a.score;
    sa.q = q; sa.q_dtype = q_dtype; sa.k = k; sa.kv_dtype = kv_dtype; sa.k_scale = k_scale; sa.q_pos = q_pos;
    sa.kv_len = kv_len; sa.B = B; sa.Tq = Tq; sa.H = H; sa.d = d; sa.Nmax = Nmax; sa.window = window;
    sa.scale_log2 = scale_log2; sa.lse = f.lse; sa.scores = (float*)(ws + p.sel.off_scores); sa.cstride = Nmax;
    sa.nsplit = p.sel.score_nsplit; sa.chunk = p.sel.score_chunk; sa.rowhist = f.zero_hist;
    a.sel = select_args(p.sel, ws, q_pos, kv_len, Tq, Nmax, k_global, window, idx, nullptr);
    // sparse layers, as hs2_sparse_attn_layers' split MFMA path over the indices just written
    AttnArgs& sp = a.sparse;
    sp.q = q_sparse[0]; sp.q_dtype = q_dtype; sp.k = k; sp.v = v; sp.kv_dtype = kv_dtype; sp.k_scale = k_scale;
    sp.v_scale = v_scale; sp.q_pos = nullptr; sp.kv_len = kv_len; sp.list = idx; sp.S = k_global + window;
    sp.B = B; sp.Tq = Tq; sp.H = H; sp.d = d; sp.Nmax = Nmax; sp.scale_log2 = scale_log2;
    sp.nsplit = p.sp_nsplit; sp.chunk = p.sp_chunk; sp.nlayer = L;
    for (int l = 0; l < L; ++l) { sp.ql[l] = q_sparse[l]; sp.ol[l] = o_sparse[l]; }
    sp.o = o_sparse[0]; sp.lse = nullptr;
    sp.part_lstride = R * p.sp_nsplit * H * d;
    sp.ml_lstride = R * p.sp_nsplit * H * 2;
    sp.part = p.sp_nsplit > 1 ? (float*)(ws + p.off_sparse) : nullptr;
    sp.part_ml = sp.part ? sp.part + L * sp.part_lstride : nullptr;
    hipError_t e = launch_decode_block(a, stream);
    if (e != hipSuccess) return hip_fail(e, "decode block launch");
    return HS2_OK;
}

size_t hs2_sparse_attn_workspace_size(int32_t B, int32_t Tq, int32_t H, int32_t d, int32_t S) {
    if (B < 0 || Tq < 0 || H < 1 || H > 32 || (d != 64 && d != 128) || S < 1 || S > 8192) return 0;
    // the larger of the fp32 and bf16 plans of every call with no larger sizes
    const size_t n = sparse_ws_bound((int64_t)B * Tq, H, d, S);
    return n ? n : kAlign;
}

hs2_status hs2_sparse_attn(const void* q, hs2_dtype q_dtype, const void* k, const void* v, hs2_dtype kv_dtype,
                           const float* k_scale, const float* v_scale, const int32_t* idx, int32_t S,
                           const int32_t* kv_len, int32_t B, int32_t Tq, int32_t H, int32_t d, int64_t Nmax,
                           float sm_scale, float* o, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return hs2_sparse_attn_layers(&q, 1, q_dtype, k, v, kv_dtype, k_scale, v_scale, idx, S, kv_len, B, Tq, H, d,
                                  Nmax, sm_scale, &o, workspace, workspace_bytes, stream);
}

size_t hs2_sparse_attn_layers_workspace_size(int32_t B, int32_t Tq, int32_t H, int32_t d, int32_t S, int32_t L) {
    if (L < 1 || L > kMaxLayers) return 0;
    const size_t n = hs2_sparse_attn_workspace_size(B, Tq, H, d, S);
    return n ? n * (size_t)L : 0;
}

hs2_status hs2_sparse_attn_layers(const void* const* q, int32_t L, hs2_dtype q_dtype, const void* k, const void* v,
                                  hs2_dtype kv_dtype, const float* k_scale, const float* v_scale, const int32_t* idx,
                                  int32_t S, const int32_t* kv_len, int32_t B, int32_t Tq, int32_t H, int32_t d,
                                  int64_t Nmax, float sm_scale, float* const* o, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    if (!q || !o) return fail(HS2_ERR_INVALID_ARG, "null q or o pointer array");
    if (L < 1 || L > kMaxLayers) return fail(HS2_ERR_INVALID_ARG, "L=%d outside [1, %d]", L, kMaxLayers);
    for (int l = 0; l < L; ++l) {
        hs2_status st = check_common(q[l], q_dtype, k, v, kv_dtype, k_scale, v_scale, B, Tq, H, d, Nmax, sm_scale, o[l]);
        if (st != HS2_OK) return st;
    }
    if (S < 1 || S > 8192) return fail(HS2_ERR_INVALID_ARG, "S=%d outside [1, 8192]", S);
    if ((int64_t)B * Tq == 0) return HS2_OK;
    if (!idx) return fail(HS2_ERR_INVALID_ARG, "null idx pointer");
    if (!aligned(idx, 4) || !aligned(kv_len, 4) || !aligned(workspace, 16))
        return fail(HS2_ERR_INVALID_ARG, "idx/kv_len must be 4-byte and the workspace 16-byte aligned");
    const int64_t R = (int64_t)B * Tq;
    const size_t need = sparse_ws_bytes(R, H, d, S, q_dtype);        // per layer
    const bool split = workspace && need > 0 && workspace_bytes >= need * (size_t)L;

    AttnArgs aa{};
    aa.q = q[0]; aa.q_dtype = q_dtype; aa.k = k; aa.v = v; aa.kv_dtype = kv_dtype;
    aa.k_scale = k_scale; aa.v_scale = v_scale; aa.q_pos = nullptr; aa.kv_len = kv_len;
    aa.list = idx; aa.S = S; aa.B = B; aa.Tq = Tq; aa.H = H; aa.d = d; aa.Nmax = Nmax;
    aa.scale_log2 = sm_scale * 1.4426950408889634f;
    if (split) {
        sparse_plan(R, S, q_dtype, &aa.nsplit, &aa.chunk);
    } else {
        aa.nsplit = 1;
        aa.chunk = S;
    }
    // the MFMA kernel stages at most 1280 list entries per workgroup; longer unsplit lists
    // take the generic kernel
    const bool mfma = q_dtype != HS2_F32 && aa.chunk <= 1280;
    hipError_t e;
    if (!mfma) {
        // generic kernels: one layer per launch
        for (int l = 0; l < L; ++l) {
            aa.q = q[l];
            aa.o = o[l];
            aa.part = aa.nsplit > 1 ? (float*)workspace : nullptr;
            e = launch_attn_generic(aa, "sparse_attn_generic", stream);
            if (e != hipSuccess) return hip_fail(e, "sparse attention launch");
            if (aa.nsplit > 1) e = launch_attn_combine(aa, "sparse_attn_combine", stream);
            if (e != hipSuccess) return hip_fail(e, "sparse combine launch");
        }
        return HS2_OK;
    }
    // MFMA kernels: all layers in one launch of each kernel.  Partial results of layer l:
    // o at part + l * R * nsplit * H * d, (m, l) at part_ml + l * R * nsplit * H * 2.
    aa.nlayer = L;
    for (int l = 0; l < L; ++l) {
        aa.ql[l] = q[l];
        aa.ol[l] = o[l];
    }
    aa.o = o[0];
    aa.lse = nullptr;
    aa.part_lstride = R * aa.nsplit * H * d;
    aa.ml_lstride = R * aa.nsplit * H * 2;
    aa.part = aa.nsplit > 1 ? (float*)workspace : nullptr;
    aa.part_ml = aa.part ? aa.part + L * aa.part_lstride : nullptr;
    e = launch_attn_rows_mfma(aa, L > 1 ? "sparse_attn_layers_mfma" : "sparse_attn_mfma", stream);
    if (e != hipSuccess) return hip_fail(e, "sparse attention launch");
    if (aa.nsplit > 1) e = launch_attn_split_combine(aa, L > 1 ? "sparse_attn_layers_combine" : "sparse_attn_combine", stream);
    if (e != hipSuccess) return hip_fail(e, "sparse combine launch");
    return HS2_OK;
}

}  // extern "C"
