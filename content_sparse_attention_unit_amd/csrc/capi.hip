// capi.hip -- the C ABI (include/routed_attn.h): host-side argument checks,
// workspace carving and kernel launches.  Every check runs before anything is
// enqueued; no entry point allocates, synchronises or keeps state.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <initializer_list>
#include <cmath>
#include <mutex>

#include "routed_attn.h"
#include "rt_internal.hpp"

namespace {

thread_local char g_err[512] = "";

rt_status fail(rt_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

rt_status hip_fail(const char* where, hipError_t e) {
    return fail(RT_EHIP, "%s: kernel launch failed: %s", where, hipGetErrorString(e));
}

// Required tensor pointers: non-null and 16-byte aligned (the kernels move
// token rows, centroids and index lists in 16-byte vector accesses).
rt_status check_ptrs(const char* fn, std::initializer_list<const void*> ptrs) {
    int i = 0;
    for (const void* p : ptrs) {
        if (p == nullptr) return fail(RT_EINVAL, "%s: null tensor pointer (argument %d)", fn, i);
        if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
            return fail(RT_EINVAL, "%s: tensor pointer %p (argument %d) not 16-byte aligned", fn,
                        p, i);
        ++i;
    }
    return RT_OK;
}

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Checks shared by the entry points that take [B][H][n][d] token tensors.
rt_status check_tokens(const char* fn, int dtype, int B, int H, int n, int d) {
    if (B <= 0 || H <= 0 || n <= 0 || d <= 0)
        return fail(RT_EINVAL, "%s: sizes must be positive (B=%d H=%d n=%d d=%d)", fn, B, H, n, d);
    if (dtype != RT_F32 && dtype != RT_BF16)
        return fail(RT_EUNSUPPORTED, "%s: dtype %d is not RT_F32 or RT_BF16", fn, dtype);
    if (!dim_ok(d)) return fail(RT_EUNSUPPORTED, "%s: d=%d not in {16,32,64,128}", fn, d);
    if ((long long)B * H > 65535)
        return fail(RT_EUNSUPPORTED, "%s: B*H=%lld exceeds 65535", fn, (long long)B * H);
    if ((long long)n * d >= (1LL << 31))
        return fail(RT_EUNSUPPORTED, "%s: n*d=%lld exceeds 2^31-1", fn, (long long)n * d);
    return RT_OK;
}

rt_status check_clusters(const char* fn, int n, int k, int w) {
    if (k <= 0 || w <= 0) return fail(RT_EINVAL, "%s: k=%d and w=%d must be positive", fn, k, w);
    if (w > n) return fail(RT_EINVAL, "%s: w=%d exceeds n=%d", fn, w, n);
    if (k > 256) return fail(RT_EUNSUPPORTED, "%s: k=%d exceeds 256", fn, k);
    return RT_OK;
}

// Checks shared by the decode entry points.
rt_status check_decode(const char* fn, int B, int H, int d) {
    if (B <= 0 || H <= 0 || d <= 0)
        return fail(RT_EINVAL, "%s: sizes must be positive (B=%d H=%d d=%d)", fn, B, H, d);
    if (!dim_ok(d)) return fail(RT_EUNSUPPORTED, "%s: d=%d not in {16,32,64,128}", fn, d);
    if ((long long)B * H > 65535)
        return fail(RT_EUNSUPPORTED, "%s: B*H=%lld exceeds 65535", fn, (long long)B * H);
    return RT_OK;
}

rt_status check_entries(const char* fn, const char* what, int m) {
    if (m <= 0) return fail(RT_EINVAL, "%s: %s=%d must be positive", fn, what, m);
    if (m > rt::kDecodeMaxEntries)
        return fail(RT_EUNSUPPORTED, "%s: %s=%d exceeds %d", fn, what, m, rt::kDecodeMaxEntries);
    return RT_OK;
}

// rt_routed_attn_update's member sums (queries, then keys unless shared).
size_t update_sums_ws(int B, int H, int k, int d) {
    return align256((size_t)2 * B * H * k * d * sizeof(float));
}

// Splits of a weight-gradient product (M x N outputs, contraction over T
// tokens) that fill the chip (about two workgroups a compute unit) and fit in
// ws_bytes of float32 partial products; 1 when no split applies.
int weight_grad_splits(long M, long N, long T, size_t ws_bytes) {
    const long tiles = ((M + 127) / 128) * ((N + 127) / 128);
    long want = 512 / tiles;
    want = std::min(want, (T + 63) / 64 / 8);                   // at least 8 k-tiles a split
    want = std::min(want, (long)(ws_bytes / ((size_t)M * N * sizeof(float))));
    want = std::min(want, 8L);
    return want >= 2 ? (int)want : 1;
}

// Workspace that lets both weight gradients of a layer split (0 if neither would).
size_t proj_bwd_ws(int B, int n, int dm, int d, int R, int L) {
    const long T = (long)B * n, NO = (long)(R + L) * d, NC = (long)(2 * R + 3 * L) * d;
    const int so = weight_grad_splits(dm, NO, T, (size_t)-1);
    const int si = weight_grad_splits(NC, dm, T, (size_t)-1);
    const size_t bo = so > 1 ? (size_t)so * dm * NO * sizeof(float) : 0;
    const size_t bi = si > 1 ? (size_t)si * NC * dm * sizeof(float) : 0;
    return std::max(bo, bi);
}

size_t route_ws(int B, int H, int n, int k) { return (size_t)B * H * k * n * sizeof(float); }

// rt_routed_attn workspace: mask [B*H*n][KW] u32 | slots [B*H*n][kSlots][d] f32 |
// overflow [B*H*k*w][d] f32 | directory [B*H*n][k - kSlots] i32, each part
// 256-byte aligned.
size_t attn_ws_mask(int B, int H, int n, int k) {
    return align256((size_t)B * H * n * rt::mask_words(k) * sizeof(uint32_t));
}

size_t attn_ws_slots(int B, int H, int n, int d) {
    return align256((size_t)B * H * n * rt::kSlots * d * sizeof(float));
}

size_t attn_ws_ovf(int B, int H, int d, int k, int w) {
    return align256((size_t)B * H * k * w * d * sizeof(float));
}

// rt_route_partition workspace: label, best, grp, cl [B*H*n] (4 bytes each) | goff
// [B*H][k + 1] int32.
size_t partition_ws(int B, int H, int n, int k) {
    return (size_t)B * H * n * 4 * 4 + (size_t)B * H * (k + 1) * 4;
}

size_t attn_ws(int B, int H, int n, int d, int k, int w) {
    return attn_ws_mask(B, H, n, k) + attn_ws_slots(B, H, n, d) + attn_ws_ovf(B, H, d, k, w) +
           (size_t)B * H * n * rt::ovf_ranks(k) * sizeof(int32_t);
}

bool out_dtype_ok(int t) { return t == RT_F32 || t == RT_BF16; }

// rt_centroid_update_argmax workspace, for either side (q, then kk when given):
// inverse norms, labels, best scores [B*H*n] each, then the chunk partial sums
// [chunks][H][k][d] float32; sized for distinct q and kk.
size_t argmax_side_ws(int B, int H, int n, int d, int k) {
    return align256((size_t)B * H * n * 3 * 4) +
           align256((size_t)rt::label_chunks(B, n) * H * k * d * sizeof(float));
}
size_t argmax_ema_ws(int B, int H, int n, int d, int k) { return 2 * argmax_side_ws(B, H, n, d, k); }

}  // namespace

extern "C" {

int rt_version(void) { return 10000; }

const char* rt_last_error(void) { return g_err; }

const char* rt_status_string(int status) {
    switch (status) {
        case RT_OK: return "RT_OK";
        case RT_EINVAL: return "RT_EINVAL: invalid argument";
        case RT_EUNSUPPORTED: return "RT_EUNSUPPORTED: outside the supported shapes or types";
        case RT_EHIP: return "RT_EHIP: HIP runtime error";
        default: return "unknown rt_status";
    }
}

size_t rt_workspace_bytes(int op, int B, int H, int n, int d, int k, int w) {
    if (B <= 0 || H <= 0 || n <= 0 || d <= 0 || k <= 0 || w <= 0) return (size_t)-1;
    switch (op) {
        case RT_OP_ROUTE: return route_ws(B, H, n, k);
        case RT_OP_ROUTED_ATTN: return attn_ws(B, H, n, d, k, w);
        case RT_OP_LOCAL_ATTN: return 0;
        case RT_OP_CENTROID_UPDATE: return 0;
        case RT_OP_ROUTED_ATTN_BWD: return rt::bwd_workspace_bytes(B * H, n, d, k, w);
        case RT_OP_LOCAL_ATTN_BWD: return rt::local_bwd_workspace_bytes(B * H, n);
        case RT_OP_CENTROID_UPDATE_ARGMAX: return argmax_ema_ws(B, H, n, d, k);
        case RT_OP_ROUTE_PARTITION: return partition_ws(B, H, n, k);
        case RT_OP_ROUTED_ATTN_UPDATE: return attn_ws(B, H, n, d, k, w) + update_sums_ws(B, H, k, d);
        case RT_OP_ATTN_JS: return align256((size_t)B * H * n * d * 2) + align256((size_t)B * H * n * 4);
        default: return (size_t)-1;
    }
}

}  // extern "C"

namespace {

rt_status check_route(const char* fn, const void* qk, int dtype, const float* mu, int B, int H,
                      int n, int d, int k, int w, const float* inv_norm, const int32_t* idx) {
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {qk, mu, inv_norm, idx})) return st;
    rt_status st = check_tokens(fn, dtype, B, H, n, d);
    if (st != RT_OK) return st;
    if (k <= 0 || w <= 0) return fail(RT_EINVAL, "%s: k=%d and w=%d must be positive", fn, k, w);
    if (w > n) return fail(RT_EINVAL, "%s: w=%d exceeds n=%d", fn, w, n);
    if (n > rt::kMaxSeqTopw)
        return fail(RT_EUNSUPPORTED, "%s: n=%d exceeds %d", fn, n, rt::kMaxSeqTopw);
    if ((long long)B * H * k > 0x7fffffffLL)
        return fail(RT_EUNSUPPORTED, "%s: B*H*k too large", fn);
    return RT_OK;
}

// The score matrix of rt_route_noalloc: one copy per GPU the library runs on,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: kernels get the address from
// hipGetSymbolAddress (scratch_on_current_device) and never this name.
constexpr size_t kNoallocScores = (size_t)RT_ROUTE_NOALLOC_MAX_SCORES;
static __device__ __align__(256) float scratch[kNoallocScores];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr with g_err set on failure.
float* scratch_on_current_device(const char* fn) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        fail(RT_EHIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        fail(RT_EUNSUPPORTED, "%s: device %d beyond the %d this library tracks", fn, dev,
             kMaxDevices);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) {
            fail(RT_EHIP, "%s: hipGetSymbolAddress(scratch) failed: %s", fn,
                 hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev] = static_cast<float*>(ptr);
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

rt_status rt_route(const void* qk, int dtype, const float* mu, int B, int H, int n, int d, int k,
                   int w, float* inv_norm, int32_t* idx, uint32_t* member_mask, void* qk_hat,
                   float* scores, void* ws, size_t ws_bytes, void* stream) {
    static const char* fn = "rt_route";
    rt_status st = check_route(fn, qk, dtype, mu, B, H, n, d, k, w, inv_norm, idx);
    if (st != RT_OK) return st;
    float* sc = scores;
    if (sc == nullptr) {
        const size_t need = route_ws(B, H, n, k);
        if (ws == nullptr || ws_bytes < need)
            return fail(RT_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                        ws == nullptr ? (size_t)0 : ws_bytes);
        sc = static_cast<float*>(ws);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e =
        rt::launch_score(qk, dtype, mu, B, H, n, d, k, inv_norm, sc, qk_hat, member_mask, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    e = rt::launch_topw(sc, B * H, n, k, w, idx, member_mask, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

rt_status rt_route_noalloc(const void* qk, int dtype, const float* mu, int B, int H, int n, int d,
                           int k, int w, float* inv_norm, int32_t* idx, uint32_t* member_mask,
                           void* qk_hat, void* stream) {
    static const char* fn = "rt_route_noalloc";
    rt_status st = check_route(fn, qk, dtype, mu, B, H, n, d, k, w, inv_norm, idx);
    if (st != RT_OK) return st;
    const size_t nscores = (size_t)B * H * k * n;
    if (nscores > kNoallocScores)
        return fail(RT_EUNSUPPORTED, "%s: B*H*k*n=%zu scores exceed the static scratch of %zu",
                    fn, nscores, kNoallocScores);
    float* sc = scratch_on_current_device(fn);
    if (sc == nullptr) return RT_EHIP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // every score the selection reads is written first by the scoring kernel,
    // so the array needs no clearing between calls
    hipError_t e =
        rt::launch_score(qk, dtype, mu, B, H, n, d, k, inv_norm, sc, qk_hat, member_mask, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    e = rt::launch_topw(sc, B * H, n, k, w, idx, member_mask, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

}  // extern "C"

namespace {

// Which kernels routed_attn_impl launches: the in-cluster rows, the scatter
// of rows of tokens several clusters hold (and the update), or both.
constexpr int kRowsPhase = 1, kScatterPhase = 2, kBothPhases = 3;

// rt_routed_attn and rt_routed_attn_split: idx holds the clusters' keys and
// values, idx_q their queries (nullptr: idx).
rt_status routed_attn_impl(const char* fn, const void* q, const void* kk, const void* v, int dtype,
                           const float* q_inv, const float* k_inv, const int32_t* idx,
                           const int32_t* idx_q, const uint32_t* member_mask, int B, int H, int n,
                           int d, int k, int w, float scale, int causal, void* out, int out_dtype,
                           float* lse, float* sum_q, float* sum_k, void* ws, size_t ws_bytes,
                           void* stream, float* mu = nullptr, float lambda = 0.f,
                           int phases = kBothPhases, bool sums_in_ws = true) {
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {q, kk, v, idx, out})) return st;
    if (mu != nullptr && !(lambda >= 0.f && lambda <= 1.f))
        return fail(RT_EINVAL, "%s: lambda=%g outside [0, 1]", fn, (double)lambda);
    if ((q_inv == nullptr) != (k_inv == nullptr))
        return fail(RT_EINVAL, "%s: q_inv and k_inv must both be given or both be NULL", fn);
    rt_status st = check_tokens(fn, dtype, B, H, n, d);
    if (st != RT_OK) return st;
    st = check_clusters(fn, n, k, w);
    if (st != RT_OK) return st;
    if (out == q || out == kk || out == v) return fail(RT_EINVAL, "%s: out aliases an input", fn);
    if (!std::isfinite(scale)) return fail(RT_EINVAL, "%s: scale is not finite", fn);
    if (causal != 0 && causal != 1) return fail(RT_EINVAL, "%s: causal must be 0 or 1", fn);
    if (!out_dtype_ok(out_dtype))
        return fail(RT_EUNSUPPORTED, "%s: out_dtype %d is not RT_F32 or RT_BF16", fn, out_dtype);
    const bool shared = (q == kk) && (q_inv == k_inv) && (idx_q == nullptr || idx_q == idx);
    const int wmax = rt::max_cluster_rows(dtype, d, shared);
    if (w > wmax)
        return fail(RT_EUNSUPPORTED, "%s: w=%d exceeds %d for this dtype, d and q/k sharing", fn,
                    w, wmax);
    const size_t need = attn_ws(B, H, n, d, k, w) +
                        (mu != nullptr && sums_in_ws ? update_sums_ws(B, H, k, d) : 0);
    if (ws == nullptr || ws_bytes < need)
        return fail(RT_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    ws == nullptr ? (size_t)0 : ws_bytes);
    char* base = static_cast<char*>(ws);
    if (mu != nullptr && sums_in_ws) {   // the member sums of the update, after the attention's parts
        sum_q = reinterpret_cast<float*>(base + attn_ws(B, H, n, d, k, w));
        sum_k = shared ? nullptr : sum_q + (size_t)B * H * k * d;
    }
    uint32_t* mask_ws = reinterpret_cast<uint32_t*>(base);
    float* slots = reinterpret_cast<float*>(base + attn_ws_mask(B, H, n, k));
    float* ovf = reinterpret_cast<float*>(base + attn_ws_mask(B, H, n, k) + attn_ws_slots(B, H, n, d));
    int32_t* dir = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ovf) +
                                              attn_ws_ovf(B, H, d, k, w));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int BH = B * H;
    hipError_t e = hipSuccess;
    const uint32_t* mask = member_mask;             // the queries' memberships
    if (mask == nullptr) {
        if (phases != kBothPhases)
            return fail(RT_EINVAL, "%s: the membership bits are required", fn);
        e = rt::launch_mask(idx_q ? idx_q : idx, BH, n, k, w, mask_ws, s);
        if (e != hipSuccess) return hip_fail(fn, e);
        mask = mask_ws;
    }
    if (phases & kRowsPhase) {
        e = rt::launch_cluster_attn(q, kk, v, dtype, q_inv, k_inv, idx, idx_q, mask, BH, n, d, k,
                                    w, scale, causal, out, out_dtype, lse, slots, ovf, dir, sum_q,
                                    sum_k, s);
        if (e != hipSuccess) return hip_fail(fn, e);
    }
    if (phases & kScatterPhase) {
        e = rt::launch_combine(mask, slots, ovf, dir, out_dtype, BH, n, d, k, w, out, s, mu, sum_q,
                               sum_k, B, H, lambda);
        if (e != hipSuccess) return hip_fail(fn, e);
    }
    return RT_OK;
}

}  // namespace

extern "C" {

rt_status rt_routed_attn(const void* q, const void* kk, const void* v, int dtype,
                         const float* q_inv, const float* k_inv, const int32_t* idx,
                         const uint32_t* member_mask, int B, int H, int n, int d, int k, int w,
                         float scale, int causal, void* out, int out_dtype, float* lse,
                         float* sum_q, float* sum_k, void* ws, size_t ws_bytes, void* stream) {
    return routed_attn_impl("rt_routed_attn", q, kk, v, dtype, q_inv, k_inv, idx, nullptr,
                            member_mask, B, H, n, d, k, w, scale, causal, out, out_dtype, lse,
                            sum_q, sum_k, ws, ws_bytes, stream);
}

rt_status rt_routed_attn_update(const void* q, const void* kk, const void* v, int dtype,
                                const float* q_inv, const float* k_inv, const int32_t* idx,
                                const uint32_t* member_mask, int B, int H, int n, int d, int k,
                                int w, float scale, int causal, void* out, int out_dtype,
                                float* lse, float* mu, float lambda, void* ws, size_t ws_bytes,
                                void* stream) {
    static const char* fn = "rt_routed_attn_update";
    if (!mu || reinterpret_cast<uintptr_t>(mu) % 16 != 0) {
        g_err[0] = 0;
        return check_ptrs(fn, {mu});
    }
    return routed_attn_impl(fn, q, kk, v, dtype, q_inv, k_inv, idx, nullptr, member_mask, B, H, n,
                            d, k, w, scale, causal, out, out_dtype, lse, nullptr, nullptr, ws,
                            ws_bytes, stream, mu, lambda);
}

rt_status rt_cluster_attn(const void* q, const void* kk, const void* v, int dtype,
                          const float* q_inv, const float* k_inv, const int32_t* idx,
                          const uint32_t* member_mask, int B, int H, int n, int d, int k, int w,
                          float scale, int causal, void* out, int out_dtype, float* lse,
                          float* sum_q, float* sum_k, void* ws, size_t ws_bytes, void* stream) {
    static const char* fn = "rt_cluster_attn";
    if (!member_mask) {
        g_err[0] = 0;
        return fail(RT_EINVAL, "%s: null tensor pointer (member_mask)", fn);
    }
    return routed_attn_impl(fn, q, kk, v, dtype, q_inv, k_inv, idx, nullptr, member_mask, B, H, n,
                            d, k, w, scale, causal, out, out_dtype, lse, sum_q, sum_k, ws,
                            ws_bytes, stream, nullptr, 0.f, kRowsPhase);
}

rt_status rt_scatter_rows(const uint32_t* member_mask, int dtype, int B, int H, int n, int d,
                          int k, int w, void* out, int out_dtype, float* mu, const float* sum_q,
                          const float* sum_k, float lambda, void* ws, size_t ws_bytes,
                          void* stream) {
    static const char* fn = "rt_scatter_rows";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {member_mask, out})) return st;
    if (mu != nullptr && sum_q == nullptr)
        return fail(RT_EINVAL, "%s: the update needs sum_q", fn);
    if (B <= 0 || H <= 0 || n <= 0 || d <= 0)
        return fail(RT_EINVAL, "%s: sizes must be positive (B=%d H=%d n=%d d=%d)", fn, B, H, n, d);
    if (!dim_ok(d)) return fail(RT_EUNSUPPORTED, "%s: d=%d not in {16,32,64,128}", fn, d);
    rt_status st = check_clusters(fn, n, k, w);
    if (st != RT_OK) return st;
    if (mu != nullptr && !(lambda >= 0.f && lambda <= 1.f))
        return fail(RT_EINVAL, "%s: lambda=%g outside [0, 1]", fn, (double)lambda);
    if (!out_dtype_ok(out_dtype))
        return fail(RT_EUNSUPPORTED, "%s: out_dtype %d is not RT_F32 or RT_BF16", fn, out_dtype);
    if (dtype != RT_F32 && dtype != RT_BF16)
        return fail(RT_EUNSUPPORTED, "%s: dtype %d is not RT_F32 or RT_BF16", fn, dtype);
    if ((long long)B * H > 65535)
        return fail(RT_EUNSUPPORTED, "%s: B*H=%lld exceeds 65535", fn, (long long)B * H);
    const size_t need = attn_ws(B, H, n, d, k, w);
    if (ws == nullptr || ws_bytes < need)
        return fail(RT_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    ws == nullptr ? (size_t)0 : ws_bytes);
    char* base = static_cast<char*>(ws);
    float* slots = reinterpret_cast<float*>(base + attn_ws_mask(B, H, n, k));
    float* ovf = reinterpret_cast<float*>(base + attn_ws_mask(B, H, n, k) + attn_ws_slots(B, H, n, d));
    int32_t* dir = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ovf) +
                                              attn_ws_ovf(B, H, d, k, w));
    hipError_t e = rt::launch_combine(member_mask, slots, ovf, dir, out_dtype, B * H, n, d, k, w,
                                      out, static_cast<hipStream_t>(stream), mu, sum_q, sum_k, B,
                                      H, lambda);
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

rt_status rt_routed_attn_split(const void* q, const void* kk, const void* v, int dtype,
                               const float* q_inv, const float* k_inv, const int32_t* idx_q,
                               const int32_t* idx_k, const uint32_t* q_mask, int B, int H, int n,
                               int d, int k, int w, float scale, void* out, int out_dtype,
                               float* lse, float* sum_q, float* sum_k, void* ws, size_t ws_bytes,
                               void* stream) {
    static const char* fn = "rt_routed_attn_split";
    if (!idx_q || reinterpret_cast<uintptr_t>(idx_q) % 16 != 0) {
        g_err[0] = 0;
        return check_ptrs(fn, {idx_q});
    }
    return routed_attn_impl(fn, q, kk, v, dtype, q_inv, k_inv, idx_k, idx_q, q_mask, B, H, n, d,
                            k, w, scale, 0, out, out_dtype, lse, sum_q, sum_k, ws, ws_bytes,
                            stream);
}

rt_status rt_local_attn(const void* q, const void* kk, const void* v, int dtype, int B, int H,
                        int n, int d, int window, float scale, int causal, void* out,
                        int out_dtype, void* stream) {
    static const char* fn = "rt_local_attn";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {q, kk, v, out})) return st;
    rt_status st = check_tokens(fn, dtype, B, H, n, d);
    if (st != RT_OK) return st;
    if (window < 1) return fail(RT_EINVAL, "%s: window=%d must be >= 1", fn, window);
    if (out == q || out == kk || out == v) return fail(RT_EINVAL, "%s: out aliases an input", fn);
    if (!std::isfinite(scale)) return fail(RT_EINVAL, "%s: scale is not finite", fn);
    if (causal != 0 && causal != 1) return fail(RT_EINVAL, "%s: causal must be 0 or 1", fn);
    if (!out_dtype_ok(out_dtype))
        return fail(RT_EUNSUPPORTED, "%s: out_dtype %d is not RT_F32 or RT_BF16", fn, out_dtype);
    hipError_t e = rt::launch_local_attn(q, kk, v, dtype, B * H, n, d, window, -1, scale, causal, out,
                                         out_dtype, nullptr, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

rt_status rt_centroid_update(float* mu, const void* q, const float* q_inv, const void* kk,
                             const float* k_inv, int dtype, const int32_t* idx, int B, int H, int n,
                             int d, int k, int w, float lambda, void* stream) {
    static const char* fn = "rt_centroid_update";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {mu, q, q_inv, idx})) return st;
    if ((kk == nullptr) != (k_inv == nullptr))
        return fail(RT_EINVAL, "%s: kk and k_inv must both be given or both be NULL", fn);
    rt_status st = check_tokens(fn, dtype, B, H, n, d);
    if (st != RT_OK) return st;
    if (k <= 0 || w <= 0) return fail(RT_EINVAL, "%s: k=%d and w=%d must be positive", fn, k, w);
    if (w > n) return fail(RT_EINVAL, "%s: w=%d exceeds n=%d", fn, w, n);
    if (k > 65535) return fail(RT_EUNSUPPORTED, "%s: k=%d exceeds 65535", fn, k);
    if (!(lambda >= 0.f && lambda <= 1.f))
        return fail(RT_EINVAL, "%s: lambda=%g outside [0, 1]", fn, (double)lambda);
    if ((long long)B * w > 0x7fffffffLL) return fail(RT_EUNSUPPORTED, "%s: B*w too large", fn);
    hipError_t e = rt::launch_ema(mu, q, q_inv, kk, k_inv, dtype, idx, B, H, n, d, k, w, lambda,
                                  static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

namespace {

rt_status check_proj(const char* fn, int B, int n, int dm, int d, int R, int L) {
    if (B <= 0 || n <= 0 || dm <= 0 || d <= 0 || R <= 0 || L < 0)
        return fail(RT_EINVAL, "%s: sizes must be positive (B=%d n=%d dm=%d d=%d R=%d L=%d)", fn,
                    B, n, dm, d, R, L);
    if (!dim_ok(d)) return fail(RT_EUNSUPPORTED, "%s: d=%d not in {16,32,64,128}", fn, d);
    if (dm % 8 != 0) return fail(RT_EUNSUPPORTED, "%s: dm=%d is not a multiple of 8", fn, dm);
    const long long wide = std::max<long long>(dm, (long long)(2 * R + 3 * L) * d);
    if ((long long)B * n * wide >= (1LL << 31))
        return fail(RT_EUNSUPPORTED, "%s: B*n*width too large", fn);
    return RT_OK;
}

}  // namespace

rt_status rt_in_proj(const void* x, const void* w_in, int B, int n, int dm, int d, int R, int L,
                     void* qk, void* v, void* q_l, void* k_l, void* v_l, void* stream) {
    static const char* fn = "rt_in_proj";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {x, w_in, qk, v})) return st;
    if (L > 0 && (!q_l || !k_l || !v_l))
        return fail(RT_EINVAL, "%s: null local-head output with L=%d", fn, L);
    rt_status st = check_proj(fn, B, n, dm, d, R, L);
    if (st != RT_OK) return st;
    const void* outs[5] = {qk, v, q_l, k_l, v_l};
    for (int i = 0; i < (L > 0 ? 5 : 2); ++i) {
        if (outs[i] == x || outs[i] == w_in) return fail(RT_EINVAL, "%s: an output aliases an input", fn);
        for (int j = i + 1; j < (L > 0 ? 5 : 2); ++j)
            if (outs[i] == outs[j]) return fail(RT_EINVAL, "%s: outputs alias each other", fn);
    }
    rt::ProjArgs p{};
    p.a[0] = x;
    p.w = w_in;
    p.c[0] = qk;
    p.c[1] = v;
    p.c[2] = q_l;
    p.c[3] = k_l;
    p.c[4] = v_l;
    p.hc[0] = R;
    p.hc[1] = R;
    p.hc[2] = p.hc[3] = p.hc[4] = L;
    p.M = B * n;
    p.N = (2 * R + 3 * L) * d;
    p.K = dm;
    p.n = n;
    p.d = d;
    hipError_t e = rt::launch_proj(p, 0, 1, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

rt_status rt_out_proj(const void* o_r, const void* o_l, const void* w_o, const void* x, int B,
                      int n, int dm, int d, int R, int L, void* y, void* stream) {
    static const char* fn = "rt_out_proj";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {o_r, w_o, y})) return st;
    if (L > 0)
        if (rt_status st = check_ptrs(fn, {o_l})) return st;
    rt_status st = check_proj(fn, B, n, dm, d, R, L);
    if (st != RT_OK) return st;
    if (y == o_r || y == w_o || (L > 0 && y == o_l))
        return fail(RT_EINVAL, "%s: y aliases a head output or the weights", fn);
    rt::ProjArgs p{};
    p.a[0] = o_r;
    p.a[1] = o_l;
    p.ha[0] = R;
    p.ha[1] = L;
    p.w = w_o;
    p.c[0] = y;
    p.res = x;
    p.M = B * n;
    p.N = dm;
    p.K = (R + L) * d;
    p.n = n;
    p.d = d;
    hipError_t e = rt::launch_proj(p, 1, 0, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

rt_status rt_centroid_update_sums(float* mu, const float* sum_q, const float* sum_k, int B,
                                  int H, int k, int d, float lambda, void* stream) {
    static const char* fn = "rt_centroid_update_sums";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {mu, sum_q})) return st;
    if (B <= 0 || H <= 0 || k <= 0 || d <= 0)
        return fail(RT_EINVAL, "%s: sizes must be positive (B=%d H=%d k=%d d=%d)", fn, B, H, k, d);
    if (!(lambda >= 0.f && lambda <= 1.f))
        return fail(RT_EINVAL, "%s: lambda=%g outside [0, 1]", fn, (double)lambda);
    if ((long long)B * H * k * d >= (1LL << 31))
        return fail(RT_EUNSUPPORTED, "%s: B*H*k*d too large", fn);
    hipError_t e = rt::launch_ema_sums(mu, sum_q, sum_k, B, H, k, d, lambda,
                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

rt_status rt_routed_attn_bwd(const void* q, const void* kk, const void* v, int dtype,
                             const float* q_inv, const float* k_inv, const int32_t* idx,
                             const uint32_t* member_mask, const float* lse, const void* dout, int B, int H, int n, int d, int k,
                             int w, float scale, int causal, float* dq_hat, float* dk_hat,
                             float* dv, void* ws, size_t ws_bytes, void* stream) {
    static const char* fn = "rt_routed_attn_bwd";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {q, kk, v, idx, lse, dout, dq_hat, dv})) return st;
    if ((q_inv == nullptr) != (k_inv == nullptr))
        return fail(RT_EINVAL, "%s: q_inv and k_inv must both be given or both be NULL", fn);
    if (dk_hat == nullptr && !(q == kk && q_inv == k_inv))
        return fail(RT_EINVAL, "%s: dk_hat may be NULL only with shared q/k (q == kk)", fn);
    {
        const void* outs[3] = {dq_hat, dk_hat, dv};
        const void* ins[5] = {q, kk, v, dout, lse};
        for (int i = 0; i < 3; ++i) {
            if (outs[i] == nullptr) continue;
            for (int j = 0; j < 5; ++j)
                if (outs[i] == ins[j]) return fail(RT_EINVAL, "%s: a gradient aliases an input", fn);
            for (int j = i + 1; j < 3; ++j)
                if (outs[i] == outs[j]) return fail(RT_EINVAL, "%s: gradients alias each other", fn);
        }
    }
    rt_status st = check_tokens(fn, dtype, B, H, n, d);
    if (st != RT_OK) return st;
    st = check_clusters(fn, n, k, w);
    if (st != RT_OK) return st;
    if (!std::isfinite(scale)) return fail(RT_EINVAL, "%s: scale is not finite", fn);
    if (causal != 0 && causal != 1) return fail(RT_EINVAL, "%s: causal must be 0 or 1", fn);
    const bool shared = (q == kk) && (q_inv == k_inv);
    const int wmax = rt::max_cluster_rows_bwd(dtype, d, shared);
    if (w > wmax)
        return fail(RT_EUNSUPPORTED, "%s: w=%d exceeds %d for this dtype, d and q/k sharing", fn,
                    w, wmax);
    const size_t need = rt::bwd_workspace_bytes(B * H, n, d, k, w);
    if (need > 0 && (ws == nullptr || ws_bytes < need))
        return fail(RT_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    ws == nullptr ? (size_t)0 : ws_bytes);
    hipError_t e = rt::launch_cluster_attn_bwd(q, kk, v, dtype, q_inv, k_inv, idx, member_mask,
                                               lse, dout,
                                               B * H, n, d, k, w, scale, causal, dq_hat, dk_hat,
                                               dv, ws,
                                               static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported)
        return fail(RT_EUNSUPPORTED, "%s: this configuration has no backward kernel", fn);
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

rt_status rt_local_attn_bwd(const void* q, const void* kk, const void* v, const void* dout,
                            int dtype, int B, int H, int n, int d, int window, float scale,
                            int causal, float* dq, float* dk, float* dv, void* ws,
                            size_t ws_bytes, void* stream) {
    static const char* fn = "rt_local_attn_bwd";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {q, kk, v, dout, dq, dk, dv})) return st;
    {
        const void* outs[3] = {dq, dk, dv};
        const void* ins[4] = {q, kk, v, dout};
        for (int i = 0; i < 3; ++i) {
            for (int j = 0; j < 4; ++j)
                if (outs[i] == ins[j]) return fail(RT_EINVAL, "%s: a gradient aliases an input", fn);
            for (int j = i + 1; j < 3; ++j)
                if (outs[i] == outs[j]) return fail(RT_EINVAL, "%s: gradients alias each other", fn);
        }
    }
    rt_status st = check_tokens(fn, dtype, B, H, n, d);
    if (st != RT_OK) return st;
    if (window < 1) return fail(RT_EINVAL, "%s: window=%d must be >= 1", fn, window);
    if (!std::isfinite(scale)) return fail(RT_EINVAL, "%s: scale is not finite", fn);
    if (causal != 0 && causal != 1) return fail(RT_EINVAL, "%s: causal must be 0 or 1", fn);
    if (dtype != RT_BF16 || (d != 64 && d != 128))
        return fail(RT_EUNSUPPORTED, "%s: bf16 inputs with d in {64, 128} only", fn);
    const size_t need = rt::local_bwd_workspace_bytes(B * H, n);
    if (ws == nullptr || ws_bytes < need)
        return fail(RT_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    ws == nullptr ? (size_t)0 : ws_bytes);
    hipError_t e = rt::launch_local_attn_bwd(q, kk, v, dout, B * H, n, d, window, scale, causal,
                                             dq, dk, dv, ws, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

rt_status rt_normalize_bwd(const void* x, int dtype, const float* inv_norm, const float* g1,
                           const float* g2, long rows, int d, float* dx, void* stream) {
    static const char* fn = "rt_normalize_bwd";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {x, inv_norm, g1, dx})) return st;
    if (rows <= 0 || d <= 0) return fail(RT_EINVAL, "%s: rows=%ld and d=%d must be positive", fn,
                                         rows, d);
    if (dtype != RT_F32 && dtype != RT_BF16)
        return fail(RT_EUNSUPPORTED, "%s: dtype %d is not RT_F32 or RT_BF16", fn, dtype);
    if (!dim_ok(d)) return fail(RT_EUNSUPPORTED, "%s: d=%d not in {16,32,64,128}", fn, d);
    if (dx == x || dx == static_cast<const void*>(inv_norm))
        return fail(RT_EINVAL, "%s: dx aliases x or inv_norm", fn);
    if (rows * (long)d >= (1L << 40)) return fail(RT_EUNSUPPORTED, "%s: rows*d too large", fn);
    hipError_t e = rt::launch_norm_bwd(x, dtype, inv_norm, g1, g2, rows, d, dx,
                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

rt_status rt_out_proj_bwd(const void* dy, const void* o_r, const void* o_l, const void* w_o,
                          int B, int n, int dm, int d, int R, int L, void* do_r, void* do_l,
                          float* dw_o, void* ws, size_t ws_bytes, void* stream) {
    static const char* fn = "rt_out_proj_bwd";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {dy, o_r, w_o, do_r, dw_o})) return st;
    if (L > 0)
        if (rt_status st = check_ptrs(fn, {o_l, do_l})) return st;
    rt_status st = check_proj(fn, B, n, dm, d, R, L);
    if (st != RT_OK) return st;
    {
        const void* outs[3] = {do_r, L > 0 ? do_l : nullptr, dw_o};
        const void* ins[4] = {dy, o_r, o_l, w_o};
        for (int i = 0; i < 3; ++i) {
            if (outs[i] == nullptr) continue;
            for (int j = 0; j < 4; ++j)
                if (outs[i] == ins[j]) return fail(RT_EINVAL, "%s: an output aliases an input", fn);
            for (int j = i + 1; j < 3; ++j)
                if (outs[i] == outs[j]) return fail(RT_EINVAL, "%s: outputs alias each other", fn);
        }
    }
    const int T = B * n, NO = (R + L) * d;
    hipStream_t s = static_cast<hipStream_t>(stream);
    rt::GemmArgs p{};
    p.a.p[0] = dy;
    p.a.ld = dm;
    p.b.p[0] = w_o;
    p.b.ld = NO;
    p.c[0] = do_r;
    p.c[1] = do_l;
    p.hc[0] = R;
    p.hc[1] = L;
    p.M = T;
    p.N = NO;
    p.K = dm;
    p.n = n;
    p.d = d;
    hipError_t e = rt::launch_gemm_bwd(rt::GEMM_DO, p, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    rt::GemmArgs q{};
    q.a.p[0] = dy;
    q.a.ld = dm;
    q.b.p[0] = o_r;
    q.b.p[1] = o_l;
    q.b.hs[0] = R;
    q.b.hs[1] = L;
    q.c[0] = dw_o;
    q.M = dm;
    q.N = NO;
    q.K = T;
    q.n = n;
    q.d = d;
    q.ksplit = ws != nullptr ? weight_grad_splits(dm, NO, T, ws_bytes) : 1;
    q.part = static_cast<float*>(ws);
    e = rt::launch_gemm_bwd(rt::GEMM_DWO, q, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

rt_status rt_in_proj_bwd(const void* x, const void* w_in, const float* dqk, const float* dv,
                         const float* dq_l, const float* dk_l, const float* dv_l, const void* dres,
                         int B, int n, int dm, int d, int R, int L, float* dx, float* dw_in,
                         void* ws, size_t ws_bytes, void* stream) {
    static const char* fn = "rt_in_proj_bwd";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {x, w_in, dqk, dv, dx, dw_in})) return st;
    if (L > 0)
        if (rt_status st = check_ptrs(fn, {dq_l, dk_l, dv_l})) return st;
    rt_status st = check_proj(fn, B, n, dm, d, R, L);
    if (st != RT_OK) return st;
    {
        const void* outs[2] = {dx, dw_in};
        const void* ins[8] = {x, w_in, dqk, dv, dq_l, dk_l, dv_l, dres};
        if (dx == static_cast<const void*>(dw_in)) return fail(RT_EINVAL, "%s: outputs alias", fn);
        for (int i = 0; i < 2; ++i)
            for (int j = 0; j < 8; ++j)
                if (ins[j] != nullptr && outs[i] == ins[j])
                    return fail(RT_EINVAL, "%s: an output aliases an input", fn);
    }
    const int T = B * n, NC = (2 * R + 3 * L) * d;
    hipStream_t s = static_cast<hipStream_t>(stream);
    rt::GemmOperand dc{};
    dc.p[0] = dqk;
    dc.p[1] = dv;
    dc.p[2] = dq_l;
    dc.p[3] = dk_l;
    dc.p[4] = dv_l;
    dc.hs[0] = dc.hs[1] = R;
    dc.hs[2] = dc.hs[3] = dc.hs[4] = L;
    rt::GemmArgs p{};
    p.a = dc;
    p.b.p[0] = w_in;
    p.b.ld = dm;
    p.c[0] = dx;
    p.res = static_cast<const uint16_t*>(dres);
    p.M = T;
    p.N = dm;
    p.K = NC;
    p.n = n;
    p.d = d;
    hipError_t e = rt::launch_gemm_bwd(rt::GEMM_DX, p, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    rt::GemmArgs q{};
    q.a = dc;
    q.b.p[0] = x;
    q.b.ld = dm;
    q.c[0] = dw_in;
    q.M = NC;
    q.N = dm;
    q.K = T;
    q.n = n;
    q.d = d;
    q.ksplit = ws != nullptr ? weight_grad_splits(NC, dm, T, ws_bytes) : 1;
    q.part = static_cast<float*>(ws);
    e = rt::launch_gemm_bwd(rt::GEMM_DWIN, q, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

rt_status rt_local_attn_blocked(const void* q, const void* kk, const void* v, int dtype, int B,
                                int H, int n, int d, int block, int lookback, float scale,
                                void* out, int out_dtype, void* stream) {
    static const char* fn = "rt_local_attn_blocked";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {q, kk, v, out})) return st;
    rt_status st = check_tokens(fn, dtype, B, H, n, d);
    if (st != RT_OK) return st;
    if (block < 1) return fail(RT_EINVAL, "%s: block=%d must be >= 1", fn, block);
    if (lookback < 0) return fail(RT_EINVAL, "%s: lookback=%d must be >= 0", fn, lookback);
    if ((long long)block * (lookback + 1) > (1LL << 30))
        return fail(RT_EUNSUPPORTED, "%s: block*(lookback+1) too large", fn);
    if (out == q || out == kk || out == v) return fail(RT_EINVAL, "%s: out aliases an input", fn);
    if (!std::isfinite(scale)) return fail(RT_EINVAL, "%s: scale is not finite", fn);
    if (!out_dtype_ok(out_dtype))
        return fail(RT_EUNSUPPORTED, "%s: out_dtype %d is not RT_F32 or RT_BF16", fn, out_dtype);
    hipError_t e = rt::launch_local_attn(q, kk, v, dtype, B * H, n, d, block, lookback, scale, 1,
                                         out, out_dtype, nullptr, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

rt_status rt_centroid_update_argmax(float* mu, const void* q, const void* kk, int dtype, int B,
                                    int H, int n, int d, int k, float lambda, void* ws,
                                    size_t ws_bytes, void* stream) {
    static const char* fn = "rt_centroid_update_argmax";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {mu, q})) return st;
    rt_status st = check_tokens(fn, dtype, B, H, n, d);
    if (st != RT_OK) return st;
    if (k <= 0) return fail(RT_EINVAL, "%s: k=%d must be positive", fn, k);
    if (k > 65535) return fail(RT_EUNSUPPORTED, "%s: k=%d exceeds 65535", fn, k);
    if (!(lambda >= 0.f && lambda <= 1.f))
        return fail(RT_EINVAL, "%s: lambda=%g outside [0, 1]", fn, (double)lambda);
    const size_t need = argmax_ema_ws(B, H, n, d, k);
    if (ws == nullptr || ws_bytes < need)
        return fail(RT_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    ws == nullptr ? (size_t)0 : ws_bytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t BHn = (size_t)B * H * n, side = argmax_side_ws(B, H, n, d, k);
    const size_t part_off = align256(BHn * 3 * 4);
    float* inv[2];
    int32_t* lab[2];
    float* part[2];
    for (int i = 0; i < 2; ++i) {
        char* base = static_cast<char*>(ws) + i * side;
        inv[i] = reinterpret_cast<float*>(base);
        lab[i] = reinterpret_cast<int32_t*>(base + BHn * 4);
        part[i] = reinterpret_cast<float*>(base + part_off);
    }
    float* best[2] = {reinterpret_cast<float*>(static_cast<char*>(ws) + BHn * 8),
                      reinterpret_cast<float*>(static_cast<char*>(ws) + side + BHn * 8)};
    const bool shared = (kk == nullptr || kk == q);
    hipError_t e = rt::launch_nearest(q, dtype, mu, B, H, n, d, k, inv[0], lab[0], best[0],
                                      nullptr, s);
    if (e == hipSuccess && !shared)
        e = rt::launch_nearest(kk, dtype, mu, B, H, n, d, k, inv[1], lab[1], best[1], nullptr, s);
    if (e == hipSuccess)
        e = rt::launch_label_ema(mu, q, inv[0], lab[0], shared ? nullptr : kk, inv[1], lab[1],
                                 dtype, B, H, n, d, k, lambda, part[0], part[1], s);
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

rt_status rt_route_partition(const void* qk, int dtype, const float* mu, int B, int H, int n,
                             int d, int k, float* inv_norm, int32_t* idx, uint32_t* member_mask,
                             void* ws, size_t ws_bytes, void* stream) {
    static const char* fn = "rt_route_partition";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {qk, mu, inv_norm, idx})) return st;
    rt_status st = check_tokens(fn, dtype, B, H, n, d);
    if (st != RT_OK) return st;
    if (k <= 0) return fail(RT_EINVAL, "%s: k=%d must be positive", fn, k);
    if (k > 256) return fail(RT_EUNSUPPORTED, "%s: k=%d exceeds 256", fn, k);
    if (n % k != 0) return fail(RT_EINVAL, "%s: n=%d is not a multiple of k=%d", fn, n, k);
    if (n > rt::kPartitionMaxN)
        return fail(RT_EUNSUPPORTED, "%s: n=%d exceeds %d", fn, n, rt::kPartitionMaxN);
    const size_t need = partition_ws(B, H, n, k);
    if (ws == nullptr || ws_bytes < need)
        return fail(RT_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    ws == nullptr ? (size_t)0 : ws_bytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t tok = (size_t)B * H * n;
    int32_t* label = static_cast<int32_t*>(ws);
    float* best = reinterpret_cast<float*>(label + tok);
    int32_t* grp = label + 2 * tok;
    int32_t* cl = label + 3 * tok;
    int32_t* goff = label + 4 * tok;
    hipError_t e = rt::launch_nearest(qk, dtype, mu, B, H, n, d, k, inv_norm, label, best,
                                      member_mask, s);
    if (e == hipSuccess)
        e = rt::launch_partition(label, best, B * H, n, k, idx, member_mask, grp, cl, goff, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

// ---- decode -------------------------------------------------------------------------------

rt_status rt_decode_fill(const void* qk, const float* inv_norm, const void* v, const int32_t* idx,
                         int B, int H, int n, int d, int k, int w, int cap, void* cache_k,
                         float* cache_inv, void* cache_v, int32_t* cache_pos, int32_t* cache_len,
                         void* stream) {
    static const char* fn = "rt_decode_fill";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {qk, inv_norm, v, idx, cache_k, cache_inv, cache_v, cache_pos, cache_len})) return st;
    rt_status st = check_tokens(fn, RT_BF16, B, H, n, d);
    if (st == RT_OK) st = check_clusters(fn, n, k, w);
    if (st == RT_OK) st = check_entries(fn, "cap", cap);
    if (st != RT_OK) return st;
    if (cap < w) return fail(RT_EINVAL, "%s: cap=%d is below w=%d", fn, cap, w);
    if ((long long)B * H * k * cap * d >= (1LL << 40))
        return fail(RT_EUNSUPPORTED, "%s: cache too large", fn);
    hipError_t e = rt::launch_decode_fill(qk, inv_norm, v, idx, B * H, n, d, k, w, cap, cache_k,
                                          cache_inv, cache_v, cache_pos, cache_len,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

rt_status rt_decode_ring_fill(const void* kk, const void* v, int B, int H, int n, int d,
                              int window, void* ring_k, void* ring_v, void* stream) {
    static const char* fn = "rt_decode_ring_fill";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {kk, v, ring_k, ring_v})) return st;
    rt_status st = check_tokens(fn, RT_BF16, B, H, n, d);
    if (st == RT_OK) st = check_entries(fn, "window", window);
    if (st != RT_OK) return st;
    hipError_t e = rt::launch_decode_ring_fill(kk, v, B * H, n, d, window, ring_k, ring_v,
                                               static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

rt_status rt_decode_routed(const void* qk_t, const void* v_t, const float* mu, int B, int H, int d,
                           int k, int cap, void* cache_k, float* cache_inv, void* cache_v,
                           int32_t* cache_pos, int32_t* cache_len, int t, float scale, void* out,
                           int out_dtype, int32_t* label, void* stream) {
    static const char* fn = "rt_decode_routed";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {qk_t, v_t, mu, cache_k, cache_inv, cache_v, cache_pos, cache_len, out})) return st;
    rt_status st = check_decode(fn, B, H, d);
    if (st == RT_OK) st = check_entries(fn, "cap", cap);
    if (st != RT_OK) return st;
    if (k <= 0) return fail(RT_EINVAL, "%s: k=%d must be positive", fn, k);
    if (k > 256) return fail(RT_EUNSUPPORTED, "%s: k=%d exceeds 256", fn, k);
    if (t < 0) return fail(RT_EINVAL, "%s: position t=%d is negative", fn, t);
    if (!std::isfinite(scale)) return fail(RT_EINVAL, "%s: scale is not finite", fn);
    if (out_dtype != RT_F32 && out_dtype != RT_BF16)
        return fail(RT_EUNSUPPORTED, "%s: out_dtype %d is not RT_F32 or RT_BF16", fn, out_dtype);
    hipError_t e = rt::launch_decode_routed(qk_t, v_t, mu, B * H, H, d, k, cap, cache_k, cache_inv,
                                            cache_v, cache_pos, cache_len, t, scale, out,
                                            out_dtype, label, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

rt_status rt_decode_local(const void* q_t, const void* k_t, const void* v_t, int B, int H, int d,
                          int window, void* ring_k, void* ring_v, int t, float scale, void* out,
                          int out_dtype, void* stream) {
    static const char* fn = "rt_decode_local";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {q_t, k_t, v_t, ring_k, ring_v, out})) return st;
    rt_status st = check_decode(fn, B, H, d);
    if (st == RT_OK) st = check_entries(fn, "window", window);
    if (st != RT_OK) return st;
    if (t < 0) return fail(RT_EINVAL, "%s: position t=%d is negative", fn, t);
    if (!std::isfinite(scale)) return fail(RT_EINVAL, "%s: scale is not finite", fn);
    if (out_dtype != RT_F32 && out_dtype != RT_BF16)
        return fail(RT_EUNSUPPORTED, "%s: out_dtype %d is not RT_F32 or RT_BF16", fn, out_dtype);
    hipError_t e = rt::launch_decode_local(q_t, k_t, v_t, B * H, d, window, ring_k, ring_v, t,
                                           scale, out, out_dtype, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

rt_status rt_attn_js(const void* qk, const float* q_inv, const int32_t* idx, const void* q_l,
                     const void* k_l, int B, int H, int n, int d, int k, int w, int window,
                     float scale_r, float scale_l, int causal, float* js, void* ws,
                     size_t ws_bytes, void* stream) {
    static const char* fn = "rt_attn_js";
    g_err[0] = 0;
    if (rt_status st = check_ptrs(fn, {qk, q_inv, idx, q_l, k_l, js})) return st;
    rt_status st = check_tokens(fn, RT_BF16, B, H, n, d);
    if (st == RT_OK) st = check_clusters(fn, n, k, w);
    if (st != RT_OK) return st;
    if (w > rt::max_js_rows(d))
        return fail(RT_EUNSUPPORTED, "%s: w=%d exceeds %d at d=%d", fn, w, rt::max_js_rows(d), d);
    if (window < 1) return fail(RT_EINVAL, "%s: window=%d must be >= 1", fn, window);
    if (!std::isfinite(scale_r) || !std::isfinite(scale_l))
        return fail(RT_EINVAL, "%s: scale is not finite", fn);
    if (causal != 0 && causal != 1) return fail(RT_EINVAL, "%s: causal must be 0 or 1", fn);
    const size_t out_bytes = align256((size_t)B * H * n * d * 2);
    const size_t need = out_bytes + align256((size_t)B * H * n * 4);
    if (ws == nullptr || ws_bytes < need)
        return fail(RT_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    ws == nullptr ? (size_t)0 : ws_bytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    float* lse_l = reinterpret_cast<float*>(static_cast<char*>(ws) + out_bytes);
    // the local heads' log-denominators (their output, with the keys as values, is discarded)
    hipError_t e = rt::launch_local_attn(q_l, k_l, k_l, RT_BF16, B * H, n, d, window, -1, scale_l,
                                         causal, ws, RT_BF16, lse_l, s);
    if (e == hipSuccess)
        e = rt::launch_attn_js(qk, q_inv, idx, q_l, k_l, lse_l, B * H, n, d, k, w, window, scale_r,
                               scale_l, causal, js, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    return RT_OK;
}

size_t rt_proj_bwd_workspace_bytes(int B, int n, int dm, int d, int R, int L) {
    if (B <= 0 || n <= 0 || dm <= 0 || d <= 0 || R <= 0 || L < 0) return (size_t)-1;
    return proj_bwd_ws(B, n, dm, d, R, L);
}

}  // extern "C"
