// ema.hip -- online k-means update of the shared centroids (gfx950).
//
// The paperlayer.ai summary of "Efficient Content-Based Sparse Attention with
// Routing Transformers" (§2 and §4) says the centroids are shared by queries
// and keys and across sequences, and are learned online by mini-batch
// spherical k-means alongside the model.  The update applied here is the
// exponential moving average
//     mu_c <- lambda * mu_c + (1 - lambda)/2 * (S_Q[c] + S_K[c]),
// S_Q[c] the sum of the unit-normalised queries routed to c over the whole
// batch, S_K[c] likewise for the keys; no renormalisation.
//
// One workgroup per (head, centroid) owns mu[h][c] and sums its B*w member
// rows (raw bf16/f32 times the float32 inverse norm) in a fixed order, so the
// update is deterministic and needs no cross-workgroup reduction.
#include "rt_common.hpp"
#include "rt_internal.hpp"

namespace rt {
namespace {

template <typename T>
__device__ __forceinline__ float4 load4(const T* p, long off);
template <>
__device__ __forceinline__ float4 load4<float>(const float* p, long off) {
    return *reinterpret_cast<const float4*>(p + off);
}
template <>
__device__ __forceinline__ float4 load4<u16>(const u16* p, long off) {
    const uint2 v = *reinterpret_cast<const uint2*>(p + off);
    return make_float4(bf2f((u16)(v.x & 0xffffu)), bf2f((u16)(v.x >> 16)),
                       bf2f((u16)(v.y & 0xffffu)), bf2f((u16)(v.y >> 16)));
}

template <typename T>
__global__ __launch_bounds__(256) void ema_kernel(float* __restrict__ mu, const T* __restrict__ q,
                                                  const float* __restrict__ q_inv,
                                                  const T* __restrict__ kk,
                                                  const float* __restrict__ k_inv,
                                                  const int32_t* __restrict__ idx, int B, int H,
                                                  int n, int D, int k, int w, float lam) {
    __shared__ float4 red[256];
    const int c = blockIdx.x, h = blockIdx.y;
    const int DG = D / 4;               // threads per row (4 dims each)
    const int RPI = 256 / DG;           // rows in flight
    const int dg = threadIdx.x % DG, rg = threadIdx.x / DG;
    const bool shared = (kk == nullptr);
    float4 sq = make_float4(0.f, 0.f, 0.f, 0.f), sk = sq;
    const int members = B * w;
    for (int mi = rg; mi < members; mi += RPI) {
        const int b = mi / w, r = mi % w;
        const long bh = (long)b * H + h;
        const int t = clamp_pos(idx[(bh * k + c) * w + r], n);
        const long tok = bh * n + t;
        const float iq = q_inv[tok];
        const float4 x = load4<T>(q, tok * D + 4 * dg);
        sq.x = fmaf(x.x, iq, sq.x);
        sq.y = fmaf(x.y, iq, sq.y);
        sq.z = fmaf(x.z, iq, sq.z);
        sq.w = fmaf(x.w, iq, sq.w);
        if (!shared) {
            const float ik = k_inv[tok];
            const float4 y = load4<T>(kk, tok * D + 4 * dg);
            sk.x = fmaf(y.x, ik, sk.x);
            sk.y = fmaf(y.y, ik, sk.y);
            sk.z = fmaf(y.z, ik, sk.z);
            sk.w = fmaf(y.w, ik, sk.w);
        }
    }
    // S_Q + S_K per thread, then a fixed-order sum over the row groups.
    float4 s;
    if (shared) {
        s = make_float4(2.f * sq.x, 2.f * sq.y, 2.f * sq.z, 2.f * sq.w);
    } else {
        s = make_float4(sq.x + sk.x, sq.y + sk.y, sq.z + sk.z, sq.w + sk.w);
    }
    red[threadIdx.x] = s;
    __syncthreads();
    if (rg == 0) {
        float4 tot = red[dg];
        for (int g2 = 1; g2 < RPI; ++g2) {
            const float4 o = red[g2 * DG + dg];
            tot.x += o.x;
            tot.y += o.y;
            tot.z += o.z;
            tot.w += o.w;
        }
        float* m = mu + ((long)h * k + c) * D + 4 * dg;
        const float a = (1.0f - lam) * 0.5f;
        m[0] = fmaf(lam, m[0], a * tot.x);
        m[1] = fmaf(lam, m[1], a * tot.y);
        m[2] = fmaf(lam, m[2], a * tot.z);
        m[3] = fmaf(lam, m[3], a * tot.w);
    }
}

// mu <- lambda*mu + (1-lambda)/2 * (sum over b of sum_q + sum_k): one thread
// per centroid element, batch rows summed in ascending order.
__global__ __launch_bounds__(256) void ema_sums_kernel(float* __restrict__ mu,
                                                       const float* __restrict__ sum_q,
                                                       const float* __restrict__ sum_k, int B,
                                                       long HKD, float lam) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= HKD) return;
    float sq = 0.f, sk = 0.f;
    for (int b = 0; b < B; ++b) {
        sq += sum_q[b * HKD + i];
        if (sum_k != nullptr) sk += sum_k[b * HKD + i];
    }
    const float tot = (sum_k != nullptr) ? sq + sk : 2.f * sq;
    mu[i] = fmaf(lam, mu[i], (1.0f - lam) * 0.5f * tot);
}

// Nearest-centroid variant: the partial sums, over one chunk of CH tokens of a
// head (batch rows concatenated in ascending order), of the normalised rows
// whose label is c.  The chunk's matching tokens are listed in ascending
// order first (wave ballots), then summed in that order.
constexpr int kLabelChunk = 1024;

template <typename T>
__global__ __launch_bounds__(256) void label_sums_kernel(const T* __restrict__ x,
                                                         const float* __restrict__ inv,
                                                         const int32_t* __restrict__ label,
                                                         int B, int H, int n, int D, int k,
                                                         float* __restrict__ part) {
    __shared__ int32_t list[kLabelChunk];
    __shared__ uint32_t wcount[4];
    __shared__ float4 red[256];
    const int c = blockIdx.x, h = blockIdx.y, chunk = blockIdx.z;
    const long total = (long)B * n;
    const long t0 = (long)chunk * kLabelChunk;
    const int lane = lane_id(), wv = wave_id();
    // list the chunk's tokens labelled c, in ascending order
    bool hit[kLabelChunk / 256];
#pragma unroll
    for (int it = 0; it < kLabelChunk / 256; ++it) {
        const long f = t0 + 256 * it + threadIdx.x;     // flattened (b, t)
        bool is = false;
        if (f < total) {
            const long b = f / n, t = f - b * n;
            is = label[(b * H + h) * n + t] == c;
        }
        hit[it] = is;
    }
    uint32_t cnt_total = 0u;
#pragma unroll
    for (int it = 0; it < kLabelChunk / 256; ++it) {
        const uint64_t mb = __ballot(hit[it]);
        if (lane == 0) wcount[wv] = (uint32_t)__popcll(mb);
        __syncthreads();
        uint32_t off = cnt_total;
        for (int v = 0; v < wv; ++v) off += wcount[v];
        if (hit[it]) list[off + (uint32_t)lanes_below(mb)] = 256 * it + (int)threadIdx.x;
        for (int v = 0; v < 4; ++v) cnt_total += wcount[v];
        __syncthreads();
    }
    // sum the listed rows: DG threads per row (4 dims each), RPI rows in flight
    const int DG = D / 4, RPI = 256 / DG;
    const int dg = threadIdx.x % DG, rg = threadIdx.x / DG;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (uint32_t i = rg; i < cnt_total; i += RPI) {
        const long f = t0 + list[i];
        const long b = f / n, t = f - b * n;
        const long tok = (b * H + h) * n + t;
        const float a = inv[tok];
        const float4 v = load4<T>(x, tok * D + 4 * dg);
        acc.x = fmaf(v.x, a, acc.x);
        acc.y = fmaf(v.y, a, acc.y);
        acc.z = fmaf(v.z, a, acc.z);
        acc.w = fmaf(v.w, a, acc.w);
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    if (rg == 0) {
        float4 tot = red[dg];
        for (int g2 = 1; g2 < RPI; ++g2) {
            const float4 o = red[g2 * DG + dg];
            tot.x += o.x;
            tot.y += o.y;
            tot.z += o.z;
            tot.w += o.w;
        }
        *reinterpret_cast<float4*>(part + (((long)chunk * H + h) * k + c) * D + 4 * dg) = tot;
    }
}

// mu <- lambda*mu + (1-lambda)/2 (S_Q + S_K) from the chunk partials (summed in
// ascending chunk order); part_k == nullptr means shared q/k (S_K = S_Q).
__global__ __launch_bounds__(256) void label_ema_kernel(float* __restrict__ mu,
                                                        const float* __restrict__ part_q,
                                                        const float* __restrict__ part_k,
                                                        int nchunk, long HKD, float lam) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= HKD) return;
    float sq = 0.f, sk = 0.f;
    for (int j = 0; j < nchunk; ++j) {
        sq += part_q[j * HKD + i];
        if (part_k != nullptr) sk += part_k[j * HKD + i];
    }
    const float tot = (part_k != nullptr) ? sq + sk : 2.f * sq;
    mu[i] = fmaf(lam, mu[i], (1.0f - lam) * 0.5f * tot);
}

}  // namespace

int label_chunks(int B, int n) { return (int)(((long)B * n + kLabelChunk - 1) / kLabelChunk); }

hipError_t launch_label_ema(float* mu, const void* q, const float* q_inv, const int32_t* q_label,
                            const void* kk, const float* k_inv, const int32_t* k_label, int dtype,
                            int B, int H, int n, int d, int k, float lambda, float* part_q,
                            float* part_k, hipStream_t s) {
    const int nch = label_chunks(B, n);
    const dim3 grid(k, H, nch);
    for (int side = 0; side < (kk != nullptr ? 2 : 1); ++side) {
        const void* x = side == 0 ? q : kk;
        const float* iv = side == 0 ? q_inv : k_inv;
        const int32_t* lb = side == 0 ? q_label : k_label;
        float* part = side == 0 ? part_q : part_k;
        if (dtype == 1)
            hipLaunchKernelGGL(label_sums_kernel<u16>, grid, dim3(256), 0, s, (const u16*)x, iv, lb,
                               B, H, n, d, k, part);
        else
            hipLaunchKernelGGL(label_sums_kernel<float>, grid, dim3(256), 0, s, (const float*)x, iv,
                               lb, B, H, n, d, k, part);
    }
    const long HKD = (long)H * k * d;
    hipLaunchKernelGGL(label_ema_kernel, dim3((unsigned)((HKD + 255) / 256)), dim3(256), 0, s, mu,
                       part_q, kk != nullptr ? part_k : nullptr, nch, HKD, lambda);
    return hipGetLastError();
}

hipError_t launch_ema_sums(float* mu, const float* sum_q, const float* sum_k, int B, int H,
                           int k, int d, float lambda, hipStream_t s) {
    const long HKD = (long)H * k * d;
    hipLaunchKernelGGL(ema_sums_kernel, dim3((unsigned)((HKD + 255) / 256)), dim3(256), 0, s, mu,
                       sum_q, sum_k, B, HKD, lambda);
    return hipGetLastError();
}

hipError_t launch_ema(float* mu, const void* q, const float* q_inv, const void* kk,
                      const float* k_inv, int dtype, const int32_t* idx, int B, int H, int n,
                      int d, int k, int w, float lambda, hipStream_t s) {
    if (dtype == 1)
        hipLaunchKernelGGL(ema_kernel<u16>, dim3(k, H), dim3(256), 0, s, mu, (const u16*)q, q_inv,
                           (const u16*)kk, k_inv, idx, B, H, n, d, k, w, lambda);
    else
        hipLaunchKernelGGL(ema_kernel<float>, dim3(k, H), dim3(256), 0, s, mu, (const float*)q,
                           q_inv, (const float*)kk, k_inv, idx, B, H, n, d, k, w, lambda);
    return hipGetLastError();
}

}  // namespace rt
