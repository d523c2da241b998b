// decode.hip -- one generation step at a time (gfx950).
//
// The paperlayer.ai summary of "Efficient Content-Based Sparse Attention with
// Routing Transformers" (Appendix A) samples from the model one token at a
// time.  Routing attention (§4) groups queries and keys by their nearest
// shared centroid; for a single new token the balanced top-w of a whole
// sequence does not exist, so here the new token joins the one cluster whose
// centroid is nearest (largest inner product of the unit vectors, ties to the
// lower index), its raw key row, inverse norm and value are appended to that
// cluster's cache, and its query attends to every entry of that cache (all at
// earlier positions, or itself).  The local heads keep their last `window`
// keys and values in a ring (position p at slot p % window).
//
// Cluster cache per (batch, head, cluster): raw key rows [cap][d] bf16, their
// inverse norms [cap] fp32, values [cap][d] bf16, positions [cap] int32 and
// the fill count.  A prefill membership (rt_route's idx) fills it.
//
// Kernels (one workgroup of 256 threads per (batch, head): a decode step has
// B*H independent pieces of work, each a few microseconds long, so the step is
// bound by launch latency and the serial chain inside one workgroup, not by
// HBM):
//   decode_fill_kernel        cache rows from a prefill membership.
//   decode_ring_fill_kernel   the local ring from the last window positions.
//   decode_routed_kernel      norm, nearest centroid (one thread per centroid),
//                             append, logits (one thread per cache entry, 16-
//                             byte row loads), the softmax in LDS, output (one
//                             thread per dimension, coalesced value rows).
//   decode_local_kernel       the same over the ring.
#include "rt_common.hpp"
#include "rt_internal.hpp"

namespace rt {
namespace {

constexpr int kDecNT = 256;

__device__ __forceinline__ float block_sum(float x, float* red) {
    const int lane = lane_id(), wv = wave_id();
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    __syncthreads();
    if (lane == 0) red[wv] = x;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < kDecNT / kWave; ++i) t += red[i];
    return t;
}

__device__ __forceinline__ float block_max(float x, float* red) {
    const int lane = lane_id(), wv = wave_id();
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    __syncthreads();
    if (lane == 0) red[wv] = x;
    __syncthreads();
    float t = -INFINITY;
    for (int i = 0; i < kDecNT / kWave; ++i) t = fmaxf(t, red[i]);
    return t;
}

// Logit of one cached row against the query held in LDS (d % 8 == 0; rows
// are 16-byte aligned).
__device__ __forceinline__ float row_dot(const float* __restrict__ lq, const u16* __restrict__ row,
                                         int d) {
    const uint4* r = reinterpret_cast<const uint4*>(row);
    float acc = 0.f;
    for (int i = 0; i < d / 8; ++i) {
        const uint4 u = r[i];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = fmaf(lq[8 * i + j], u4_elem(u, j), acc);
    }
    return acc;
}

// Softmax over the L logits in lp (LDS, log2 units, in place) and
// out[i] = sum_e p_e v_e[i]; rowv(e) points at entry e's value row.
template <typename OutT, typename RowFn>
__device__ __forceinline__ void softmax_out(float* lp, int L, float* red, int d, RowFn rowv,
                                            OutT* out) {
    float m = -INFINITY;
    for (int e = threadIdx.x; e < L; e += kDecNT) m = fmaxf(m, lp[e]);
    m = block_max(m, red);
    float z = 0.f;
    for (int e = threadIdx.x; e < L; e += kDecNT) {
        const float p = exp2f(lp[e] - m);
        lp[e] = p;
        z += p;
    }
    z = block_sum(z, red);                            // its barriers also publish lp
    const float rz = 1.0f / z;
    for (int i = threadIdx.x; i < d; i += kDecNT) {
        float acc = 0.f;
        for (int e = 0; e < L; ++e) acc = fmaf(lp[e], bf2f(rowv(e)[i]), acc);
        Elem<OutT>::store(out, i, acc * rz);
    }
}

__global__ __launch_bounds__(256) void decode_fill_kernel(
    const u16* __restrict__ qk, const float* __restrict__ inv, const u16* __restrict__ v,
    const int32_t* __restrict__ idx, int n, int d, int k, int w, int cap, u16* __restrict__ ck,
    float* __restrict__ cinv, u16* __restrict__ cv, int32_t* __restrict__ cpos,
    int32_t* __restrict__ clen) {
    const int c = blockIdx.x;
    const long bh = blockIdx.y;
    const long cb = bh * k + c;                       // this cluster's cache
    for (int e = threadIdx.x; e < w * d; e += 256) {
        const int r = e / d, i = e % d;
        const int t = clamp_pos(idx[cb * w + r], n);
        ck[(cb * cap + r) * d + i] = qk[(bh * n + t) * d + i];
        cv[(cb * cap + r) * d + i] = v[(bh * n + t) * d + i];
    }
    for (int r = threadIdx.x; r < w; r += 256) {
        const int t = clamp_pos(idx[cb * w + r], n);
        cinv[cb * cap + r] = inv[bh * n + t];
        cpos[cb * cap + r] = t;
    }
    if (threadIdx.x == 0) clen[cb] = w;
}

// Slot s of the ring holds the last prefill position p < n with p % window == s.
__global__ __launch_bounds__(256) void decode_ring_fill_kernel(
    const u16* __restrict__ kk, const u16* __restrict__ v, int n, int d, int window,
    u16* __restrict__ rk, u16* __restrict__ rv) {
    const int s = blockIdx.x;
    const long bh = blockIdx.y;
    const int p = (n - 1) - (((n - 1 - s) % window) + window) % window;
    if (p < 0) return;
    for (int i = threadIdx.x; i < d; i += 256) {
        rk[(bh * window + s) * d + i] = kk[(bh * n + p) * d + i];
        rv[(bh * window + s) * d + i] = v[(bh * n + p) * d + i];
    }
}

template <typename OutT>
__global__ __launch_bounds__(256) void decode_routed_kernel(
    const u16* __restrict__ qk_t, const u16* __restrict__ v_t, const float* __restrict__ mu, int H,
    int d, int k, int cap, u16* __restrict__ ck, float* __restrict__ cinv, u16* __restrict__ cv,
    int32_t* __restrict__ cpos, int32_t* __restrict__ clen, int t, float scale,
    OutT* __restrict__ out, int32_t* __restrict__ label) {
    extern __shared__ float lp[];                     // cap logits
    __shared__ float lx[256];
    __shared__ float red[kDecNT / kWave];
    __shared__ float bestv[kDecNT / kWave];
    __shared__ int bestc[kDecNT / kWave];
    const long bh = blockIdx.x;
    const int h = (int)(bh % H);
    const int lane = lane_id(), wv = wave_id();
    u16 xraw = 0;
    if (threadIdx.x < d) xraw = qk_t[bh * d + threadIdx.x];
    const float xi = bf2f(xraw);
    lx[threadIdx.x] = xi;
    const float inv = 1.0f / fmaxf(sqrtf(block_sum(xi * xi, red)), 1e-12f);
    // nearest centroid: thread c scores centroid c; ties to the lower index
    float s = -INFINITY;
    int c = 0x7fffffff;
    if ((int)threadIdx.x < k) {
        c = threadIdx.x;
        const float* m = mu + ((long)h * k + c) * d;
        float acc = 0.f;
        for (int i = 0; i < d; ++i) acc = fmaf(lx[i], m[i], acc);
        s = acc * inv;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float os = __shfl_xor(s, off);
        const int oc = __shfl_xor(c, off);
        if (os > s || (os == s && oc < c)) {
            s = os;
            c = oc;
        }
    }
    if (lane == 0) {
        bestv[wv] = s;
        bestc[wv] = c;
    }
    __syncthreads();
    float bs = bestv[0];
    int bc = bestc[0];
    for (int i = 1; i < kDecNT / kWave; ++i)
        if (bestv[i] > bs || (bestv[i] == bs && bestc[i] < bc)) {
            bs = bestv[i];
            bc = bestc[i];
        }
    if (bc >= k) bc = 0;                              // non-finite scores everywhere: stay in bounds
    const long cb = bh * k + bc;
    const int j = clen[cb];                           // the new entry's slot
    if (j < 0 || j >= cap) {                          // a full (or corrupt) cache: report, change nothing
        if (threadIdx.x < d) Elem<OutT>::store(out, bh * d + threadIdx.x, NAN);
        if (threadIdx.x == 0 && label != nullptr) label[bh] = -1;
        return;
    }
    __syncthreads();                                  // every thread has read the fill count
    if (threadIdx.x < d) {
        ck[(cb * cap + j) * d + threadIdx.x] = xraw;
        cv[(cb * cap + j) * d + threadIdx.x] = v_t[bh * d + threadIdx.x];
    }
    if (threadIdx.x == 0) {
        cinv[cb * cap + j] = inv;
        cpos[cb * cap + j] = t;
        clen[cb] = j + 1;
        if (label != nullptr) label[bh] = bc;
    }
    __threadfence_block();
    __syncthreads();                                  // the appended row is visible to the block
    // logits over the cluster's L = j + 1 entries, log2 units
    const int L = j + 1;
    const float sl2 = scale * inv * 1.4426950408889634f;
    for (int e = threadIdx.x; e < L; e += kDecNT)
        lp[e] = row_dot(lx, ck + (cb * cap + e) * d, d) * cinv[cb * cap + e] * sl2;
    softmax_out<OutT>(lp, L, red, d, [&](int e) { return cv + (cb * cap + e) * d; }, out + bh * d);
}

template <typename OutT>
__global__ __launch_bounds__(256) void decode_local_kernel(
    const u16* __restrict__ q_t, const u16* __restrict__ k_t, const u16* __restrict__ v_t, int d,
    int window, u16* __restrict__ rk, u16* __restrict__ rv, int t, float scale,
    OutT* __restrict__ out) {
    extern __shared__ float lp[];                     // window logits
    __shared__ float lq[256];
    __shared__ float red[kDecNT / kWave];
    const long bh = blockIdx.x;
    const int slot = t % window;
    lq[threadIdx.x] = threadIdx.x < d ? bf2f(q_t[bh * d + threadIdx.x]) : 0.f;
    if (threadIdx.x < d) {
        rk[(bh * window + slot) * d + threadIdx.x] = k_t[bh * d + threadIdx.x];
        rv[(bh * window + slot) * d + threadIdx.x] = v_t[bh * d + threadIdx.x];
    }
    __threadfence_block();
    __syncthreads();
    const int p0 = max(0, t - window + 1), L = t - p0 + 1;
    const float sl2 = scale * 1.4426950408889634f;
    for (int e = threadIdx.x; e < L; e += kDecNT)
        lp[e] = row_dot(lq, rk + (bh * window + (p0 + e) % window) * d, d) * sl2;
    softmax_out<OutT>(lp, L, red, d,
                      [&](int e) { return rv + (bh * window + (p0 + e) % window) * d; },
                      out + bh * d);
}

}  // namespace

hipError_t launch_decode_fill(const void* qk, const float* inv, const void* v, const int32_t* idx,
                              int BH, int n, int d, int k, int w, int cap, void* ck, float* cinv,
                              void* cv, int32_t* cpos, int32_t* clen, hipStream_t s) {
    hipLaunchKernelGGL(decode_fill_kernel, dim3(k, BH), dim3(256), 0, s, (const u16*)qk, inv,
                       (const u16*)v, idx, n, d, k, w, cap, (u16*)ck, cinv, (u16*)cv, cpos, clen);
    return hipGetLastError();
}

hipError_t launch_decode_ring_fill(const void* kk, const void* v, int BH, int n, int d,
                                   int window, void* rk, void* rv, hipStream_t s) {
    hipLaunchKernelGGL(decode_ring_fill_kernel, dim3(window, BH), dim3(256), 0, s,
                       (const u16*)kk, (const u16*)v, n, d, window, (u16*)rk, (u16*)rv);
    return hipGetLastError();
}

hipError_t launch_decode_routed(const void* qk_t, const void* v_t, const float* mu, int BH, int H,
                                int d, int k, int cap, void* ck, float* cinv, void* cv,
                                int32_t* cpos, int32_t* clen, int t, float scale, void* out,
                                int out_dtype, int32_t* label, hipStream_t s) {
    const size_t lds = (size_t)cap * sizeof(float);
    if (out_dtype == 1)
        hipLaunchKernelGGL(decode_routed_kernel<u16>, dim3(BH), dim3(kDecNT), lds, s,
                           (const u16*)qk_t, (const u16*)v_t, mu, H, d, k, cap, (u16*)ck, cinv,
                           (u16*)cv, cpos, clen, t, scale, (u16*)out, label);
    else
        hipLaunchKernelGGL(decode_routed_kernel<float>, dim3(BH), dim3(kDecNT), lds, s,
                           (const u16*)qk_t, (const u16*)v_t, mu, H, d, k, cap, (u16*)ck, cinv,
                           (u16*)cv, cpos, clen, t, scale, (float*)out, label);
    return hipGetLastError();
}

hipError_t launch_decode_local(const void* q_t, const void* k_t, const void* v_t, int BH, int d,
                               int window, void* rk, void* rv, int t, float scale, void* out,
                               int out_dtype, hipStream_t s) {
    const size_t lds = (size_t)window * sizeof(float);
    if (out_dtype == 1)
        hipLaunchKernelGGL(decode_local_kernel<u16>, dim3(BH), dim3(kDecNT), lds, s,
                           (const u16*)q_t, (const u16*)k_t, (const u16*)v_t, d, window, (u16*)rk,
                           (u16*)rv, t, scale, (u16*)out);
    else
        hipLaunchKernelGGL(decode_local_kernel<float>, dim3(BH), dim3(kDecNT), lds, s,
                           (const u16*)q_t, (const u16*)k_t, (const u16*)v_t, d, window, (u16*)rk,
                           (u16*)rv, t, scale, (float*)out);
    return hipGetLastError();
}

}  // namespace rt
