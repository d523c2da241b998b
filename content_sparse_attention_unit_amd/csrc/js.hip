// js.hip -- the Jensen-Shannon divergence between local and routed attention
// (gfx950), a diagnostic.
//
// The paperlayer.ai summary of "Efficient Content-Based Sparse Attention with
// Routing Transformers" (§6) compares, per query, the attention distribution
// of a local head with that of a routing head by their Jensen-Shannon
// divergence (natural log, so at most ln 2).  For every row r of every cluster
// c (query i = idx[c][r]):
//   P = softmax over i's window of scale_l * <q_l,i, k_l,j>    (local head)
//   Q = softmax over the cluster's keys visible to row r of
//       scale_r * <x^_i, x^_s>                                  (routing head)
//   JS = 1/2 KL(P || M) + 1/2 KL(Q || M),  M = (P + Q) / 2.
// A position in only one of the two supports contributes half its mass times
// ln 2, so with I = the cluster keys inside i's window,
//   JS = ln2/2 (2 - P(I) - Q(I)) + 1/2 sum_I [p ln(2p/(p+q)) + q ln(2q/(p+q))],
// which needs P only on I: the local head's log-denominator (from the local
// attention kernel) and one logit per key of I.  Q's log-denominator comes from
// the cluster's keys, which are all here.
//
// One workgroup (four waves) per (batch, head, cluster): the members' routed
// rows and local query and key rows are staged in LDS (rows padded by 16
// bytes, so the rows that 16 lanes read together start in different banks);
// each wave takes every fourth row, a lane per key.  Not on the layer's path:
// plain FMA dot products.
#include "rt_common.hpp"
#include "rt_internal.hpp"

namespace rt {
namespace {

constexpr float kLn2 = 0.6931471805599453f;

// <a, b> over D bf16 of two LDS rows.
template <int D>
__device__ __forceinline__ float lds_row_dot(const u16* a, const u16* b) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
        const uint4 x = *reinterpret_cast<const uint4*>(a + 8 * i);
        const uint4 y = *reinterpret_cast<const uint4*>(b + 8 * i);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = fmaf(u4_elem(x, j), u4_elem(y, j), acc);
    }
    return acc;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

template <int D, int WMAX>
__global__ __launch_bounds__(256) void attn_js_kernel(
    const u16* __restrict__ qk, const float* __restrict__ q_inv, const int32_t* __restrict__ idx,
    const u16* __restrict__ q_l, const u16* __restrict__ k_l, const float* __restrict__ lse_l,
    int n, int k, int w, int window, float scale_r, float scale_l, int causal,
    float* __restrict__ js) {
    constexpr int LDX = D + 8;
    constexpr int SLOTS = WMAX / kWave;               // keys a lane
    __shared__ __attribute__((aligned(16))) u16 lx[WMAX * LDX];    // routed rows (raw)
    __shared__ __attribute__((aligned(16))) u16 lkl[WMAX * LDX];   // local key rows
    __shared__ __attribute__((aligned(16))) u16 lql[WMAX * LDX];   // local query rows
    __shared__ float linv[WMAX];
    __shared__ int lpos[WMAX];
    const int c = blockIdx.x;
    const long bh = blockIdx.y;
    const long tokbase = bh * n;
    const int32_t* irow = idx + (bh * k + c) * w;
    for (int e = threadIdx.x; e < w * (D / 8); e += 256) {
        const int r = e / (D / 8), ch = e % (D / 8);
        const long off = (tokbase + clamp_pos(irow[r], n)) * D + 8 * ch;
        *reinterpret_cast<uint4*>(&lx[r * LDX + 8 * ch]) = *reinterpret_cast<const uint4*>(qk + off);
        *reinterpret_cast<uint4*>(&lkl[r * LDX + 8 * ch]) = *reinterpret_cast<const uint4*>(k_l + off);
        *reinterpret_cast<uint4*>(&lql[r * LDX + 8 * ch]) = *reinterpret_cast<const uint4*>(q_l + off);
    }
    for (int r = threadIdx.x; r < w; r += 256) {
        const int t = clamp_pos(irow[r], n);
        lpos[r] = t;
        linv[r] = q_inv[tokbase + t];
    }
    __syncthreads();
    const int lane = lane_id(), wv = wave_id();
    for (int r = wv; r < w; r += 4) {
        const int i = lpos[r];
        const float sr = scale_r * linv[r];
        const float lsel = lse_l[tokbase + i];
        const int send = causal ? r + 1 : w;          // the routed keys row r sees
        float lr[SLOTS], ll[SLOTS];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < SLOTS; ++j) {
            const int s = lane + kWave * j;
            lr[j] = -INFINITY;
            ll[j] = -INFINITY;
            if (s < send) {
                lr[j] = sr * linv[s] * lds_row_dot<D>(&lx[r * LDX], &lx[s * LDX]);
                const int dp = i - lpos[s];
                const bool near = causal ? dp < window : (dp < window && -dp < window);
                if (near) ll[j] = scale_l * lds_row_dot<D>(&lql[r * LDX], &lkl[s * LDX]);
                mx = fmaxf(mx, lr[j]);
            }
        }
        mx = wave_max(mx);
        float z = 0.f;
#pragma unroll
        for (int j = 0; j < SLOTS; ++j)
            if (lane + kWave * j < send) z += expf(lr[j] - mx);
        const float lser = mx + logf(wave_sum(z));
        float pi = 0.f, qi = 0.f, t = 0.f;
#pragma unroll
        for (int j = 0; j < SLOTS; ++j) {
            if (lane + kWave * j < send && ll[j] != -INFINITY) {
                const float q = expf(lr[j] - lser), p = expf(ll[j] - lsel);
                const float h = 0.5f * (p + q);
                pi += p;
                qi += q;
                if (p > 0.f) t = fmaf(p, logf(p / h), t);
                if (q > 0.f) t = fmaf(q, logf(q / h), t);
            }
        }
        pi = wave_sum(pi);
        qi = wave_sum(qi);
        t = wave_sum(t);
        if (lane == 0) {
            const float v = 0.5f * kLn2 * (2.f - pi - qi) + 0.5f * t;
            js[(bh * k + c) * w + r] = fminf(fmaxf(v, 0.f), kLn2);
        }
    }
}

template <int D, int WMAX>
void launch_js_w(const void* qk, const float* q_inv, const int32_t* idx, const void* q_l,
                 const void* k_l, const float* lse_l, int BH, int n, int k, int w, int window,
                 float scale_r, float scale_l, int causal, float* js, hipStream_t s) {
    hipLaunchKernelGGL((attn_js_kernel<D, WMAX>), dim3(k, BH), dim3(256), 0, s, (const u16*)qk,
                       q_inv, idx, (const u16*)q_l, (const u16*)k_l, lse_l, n, k, w, window,
                       scale_r, scale_l, causal, js);
}

template <int D>
void launch_js_d(const void* qk, const float* q_inv, const int32_t* idx, const void* q_l,
                 const void* k_l, const float* lse_l, int BH, int n, int k, int w, int window,
                 float scale_r, float scale_l, int causal, float* js, hipStream_t s) {
#define RT_JS(WM)                                                                               \
    launch_js_w<D, WM>(qk, q_inv, idx, q_l, k_l, lse_l, BH, n, k, w, window, scale_r, scale_l, \
                       causal, js, s)
    if (w <= 64) RT_JS(64);
    else if (w <= 128) RT_JS(128);
    else if constexpr (D <= 64) {
        if (w <= 256) RT_JS(256);
        else if constexpr (D <= 32) RT_JS(512);
    }
#undef RT_JS
}

}  // namespace

int max_js_rows(int d) { return d >= 128 ? 128 : (d == 64 ? 256 : 512); }

hipError_t launch_attn_js(const void* qk, const float* q_inv, const int32_t* idx, const void* q_l,
                          const void* k_l, const float* lse_l, int BH, int n, int d, int k, int w,
                          int window, float scale_r, float scale_l, int causal, float* js,
                          hipStream_t s) {
    switch (d) {
        case 16: launch_js_d<16>(qk, q_inv, idx, q_l, k_l, lse_l, BH, n, k, w, window, scale_r, scale_l, causal, js, s); break;
        case 32: launch_js_d<32>(qk, q_inv, idx, q_l, k_l, lse_l, BH, n, k, w, window, scale_r, scale_l, causal, js, s); break;
        case 64: launch_js_d<64>(qk, q_inv, idx, q_l, k_l, lse_l, BH, n, k, w, window, scale_r, scale_l, causal, js, s); break;
        case 128: launch_js_d<128>(qk, q_inv, idx, q_l, k_l, lse_l, BH, n, k, w, window, scale_r, scale_l, causal, js, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rt
