// local_attn.hip -- sliding-window attention for the non-routed heads (gfx950).
//
// The arXiv abstract and §6 of the paperlayer.ai summary of "Efficient
// Content-Based Sparse Attention with Routing Transformers" pair routing
// heads with local attention over a window of recent positions (windows of
// 512 and 1024 are the ones reported).  Position i attends, with ordinary
// softmax attention, to positions [i - window + 1, i] (causal) or to the band
// |i - j| < window (non-causal).
//
// local_attn_bf16_kernel: one workgroup = 64 queries (4 waves x 16).  Key
// tiles of 64 rows (and the matching value rows, transposed) are staged in
// LDS and shared by the four waves; each wave computes S^T = K Q^T and
// O^T = V^T P^T with v_mfma_f32_16x16x32_bf16 and an online softmax, skipping
// key blocks that lie outside its own band.
#include "rt_common.hpp"
#include "rt_internal.hpp"

namespace rt {
namespace {

template <int D>
struct LocalCfg {
    static constexpr int DP = D < 32 ? 32 : D;
    static constexpr int LDX = DP + 8;
    static constexpr int KT = 64;
    static constexpr int LDV = KT + 8;
    static constexpr int NS = DP / 32;
    static constexpr int NJ = D / 16;
};

template <int D>
__global__ __launch_bounds__(256) void local_attn_bf16_kernel(const u16* __restrict__ q,
                                                              const u16* __restrict__ kk,
                                                              const u16* __restrict__ v, int n,
                                                              int window, float scale, int causal,
                                                              u16* __restrict__ out) {
    using C = LocalCfg<D>;
    __shared__ __attribute__((aligned(16))) u16 lk[C::KT * C::LDX];
    __shared__ __attribute__((aligned(16))) u16 lvt[D * C::LDV];

    const int bh = blockIdx.y;
    const int q0 = blockIdx.x * 64;
    const long base = (long)bh * n;
    const int lane = lane_id(), wv = threadIdx.x >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int qw0 = q0 + 16 * wv;      // first query of this wave
    const int qi = qw0 + r16;          // this lane's query

    uint4 qreg[C::NS];
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
        const int d0 = 32 * s + 8 * g;
        qreg[s] = (qi < n && d0 < D) ? *reinterpret_cast<const uint4*>(q + (base + qi) * D + d0)
                                     : zero_u4();
    }
    const float sl2 = scale * 1.4426950408889634f;

    // Keys needed by the whole workgroup, and by this wave.
    const int lo = max(0, q0 - window + 1);
    const int hi = causal ? min(n - 1, q0 + 63) : min(n - 1, q0 + 63 + window - 1);
    const int wlo = qw0 - window + 1;
    const int whi = causal ? qw0 + 15 : qw0 + 15 + window - 1;

    f32x4 o[C::NJ];
#pragma unroll
    for (int jb = 0; jb < C::NJ; ++jb) o[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, z = 0.f;

    constexpr int CPR = C::DP / 8;
    constexpr int DCH = D / 8;
    for (int kt = lo & ~(C::KT - 1); kt <= hi; kt += C::KT) {
        __syncthreads();
        for (int e = threadIdx.x; e < C::KT * CPR; e += 256) {
            const int r = e / CPR, ch = e % CPR;
            const int j = kt + r;
            uint4 x = zero_u4();
            if (j < n && 8 * ch < D) x = *reinterpret_cast<const uint4*>(kk + (base + j) * D + 8 * ch);
            *reinterpret_cast<uint4*>(&lk[r * C::LDX + 8 * ch]) = x;
        }
        for (int e = threadIdx.x; e < (C::KT / 2) * DCH; e += 256) {
            const int rp = e / DCH, ch = e % DCH;
            const int j0 = kt + 2 * rp;
            uint4 a = zero_u4(), b = zero_u4();
            if (j0 < n) a = *reinterpret_cast<const uint4*>(v + (base + j0) * D + 8 * ch);
            if (j0 + 1 < n) b = *reinterpret_cast<const uint4*>(v + (base + j0 + 1) * D + 8 * ch);
            const uint32_t* aw = reinterpret_cast<const uint32_t*>(&a);
            const uint32_t* bw = reinterpret_cast<const uint32_t*>(&b);
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const int jj = 8 * ch + 2 * e2;
                *reinterpret_cast<uint32_t*>(&lvt[jj * C::LDV + 2 * rp]) =
                    (aw[e2] & 0xffffu) | (bw[e2] << 16);
                *reinterpret_cast<uint32_t*>(&lvt[(jj + 1) * C::LDV + 2 * rp]) =
                    (aw[e2] >> 16) | (bw[e2] & 0xffff0000u);
            }
        }
        __syncthreads();
        if (kt + C::KT - 1 < wlo || kt > whi) continue;  // tile outside this wave's band

        f32x4 sv[4];
        float cmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int key0 = kt + 16 * kb;
            if (key0 + 15 < wlo || key0 > whi || key0 >= n) {
                sv[kb] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
                continue;
            }
            sv[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < C::NS; ++s) {
                const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(
                    &lk[(16 * kb + r16) * C::LDX + 32 * s + 8 * g]));
                sv[kb] = mfma16(a, as_bf16x8(qreg[s]), sv[kb]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = key0 + 4 * g + i;
                const bool ok = j < n && j > qi - window &&
                                (causal ? j <= qi : j < qi + window);
                sv[kb][i] = ok ? sv[kb][i] * sl2 : -INFINITY;
                cmax = fmaxf(cmax, sv[kb][i]);
            }
        }
        cmax = xor_max_16_32(cmax);
        const float mnew = fmaxf(m, cmax);
        const float msafe = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(m - msafe);
        z *= alpha;
#pragma unroll
        for (int jb = 0; jb < C::NJ; ++jb) o[jb] *= alpha;
        m = mnew;

        u16 pb[4][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u16 pv = f2bf(__builtin_amdgcn_exp2f(sv[kb][i] - msafe));
                pb[kb][i] = pv;
                z += bf2f(pv);
            }
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
            uint4 pw;
            pw.x = pack2(pb[2 * mm][0], pb[2 * mm][1]);
            pw.y = pack2(pb[2 * mm][2], pb[2 * mm][3]);
            pw.z = pack2(pb[2 * mm + 1][0], pb[2 * mm + 1][1]);
            pw.w = pack2(pb[2 * mm + 1][2], pb[2 * mm + 1][3]);
            if (__ballot((pw.x | pw.y | pw.z | pw.w) != 0u) == 0ull) continue;  // wave-uniform
            const bf16x8 pbv = as_bf16x8(pw);
#pragma unroll
            for (int jb = 0; jb < C::NJ; ++jb) {
                const u16* vr = &lvt[(16 * jb + r16) * C::LDV + 32 * mm + 4 * g];
                const uint2 l2 = *reinterpret_cast<const uint2*>(vr);
                const uint2 h2 = *reinterpret_cast<const uint2*>(vr + 16);
                o[jb] = mfma16(as_bf16x8(make_uint4(l2.x, l2.y, h2.x, h2.y)), pbv, o[jb]);
            }
        }
    }

    const float zt = xor_sum_16_32(z);
    const float rz = 1.0f / zt;
    if (qi < n) {
        u16* dst = out + (base + qi) * D + 4 * g;
#pragma unroll
        for (int jb = 0; jb < C::NJ; ++jb) {
            uint2 pk;
            pk.x = pack2(f2bf(o[jb][0] * rz), f2bf(o[jb][1] * rz));
            pk.y = pack2(f2bf(o[jb][2] * rz), f2bf(o[jb][3] * rz));
            *reinterpret_cast<uint2*>(dst + 16 * jb) = pk;
        }
    }
}

// float32 inputs: one wave per query, 64-key chunks, online softmax.
template <int D>
__global__ __launch_bounds__(64) void local_attn_f32_kernel(const float* __restrict__ q,
                                                            const float* __restrict__ kk,
                                                            const float* __restrict__ v, int n,
                                                            int window, float scale, int causal,
                                                            float* __restrict__ out) {
    __shared__ float lq[D];
    __shared__ float lp[64];
    const int i = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
    const long base = (long)bh * n;
    for (int e = lane; e < D; e += 64) lq[e] = q[(base + i) * D + e];
    __syncthreads();
    const int lo = max(0, i - window + 1);
    const int hi = causal ? i : min(n - 1, i + window - 1);
    constexpr int PER = (D + 63) / 64;
    float acc[PER];
    for (int u = 0; u < PER; ++u) acc[u] = 0.f;
    float m = -INFINITY, z = 0.f;
    for (int j0 = lo; j0 <= hi; j0 += 64) {
        const int j = j0 + lane;
        float s = -INFINITY;
        if (j <= hi) {
            float dot = 0.f;
            for (int e = 0; e < D; ++e) dot = fmaf(lq[e], kk[(base + j) * D + e], dot);
            s = dot * scale;
        }
        float cm = s;
        for (int off = 32; off >= 1; off >>= 1) cm = fmaxf(cm, __shfl_xor(cm, off));
        const float mnew = fmaxf(m, cm);
        const float alpha = expf(m - mnew);
        const float p = (j <= hi) ? expf(s - mnew) : 0.f;
        float ps = p;
        for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off);
        z = z * alpha + ps;
        m = mnew;
        __syncthreads();
        lp[lane] = p;
        __syncthreads();
        const int cnt = min(64, hi - j0 + 1);
        for (int u = 0; u < PER; ++u) {
            const int e = lane + 64 * u;
            if (e < D) {
                float a = acc[u] * alpha;
                for (int jj = 0; jj < cnt; ++jj) a = fmaf(lp[jj], v[(base + j0 + jj) * D + e], a);
                acc[u] = a;
            }
        }
    }
    for (int u = 0; u < PER; ++u) {
        const int e = lane + 64 * u;
        if (e < D) out[(base + i) * D + e] = acc[u] / z;
    }
}

template <int D>
void launch_local_d(const void* q, const void* kk, const void* v, int dtype, int BH, int n,
                    int window, float scale, int causal, void* out, hipStream_t s) {
    if (dtype == 1)
        hipLaunchKernelGGL(local_attn_bf16_kernel<D>, dim3((n + 63) / 64, BH), dim3(256), 0, s,
                           (const u16*)q, (const u16*)kk, (const u16*)v, n, window, scale, causal,
                           (u16*)out);
    else
        hipLaunchKernelGGL(local_attn_f32_kernel<D>, dim3(n, BH), dim3(64), 0, s, (const float*)q,
                           (const float*)kk, (const float*)v, n, window, scale, causal,
                           (float*)out);
}

}  // namespace

hipError_t launch_local_attn(const void* q, const void* kk, const void* v, int dtype, int BH,
                             int n, int d, int window, float scale, int causal, void* out,
                             hipStream_t s) {
    switch (d) {
        case 16: launch_local_d<16>(q, kk, v, dtype, BH, n, window, scale, causal, out, s); break;
        case 32: launch_local_d<32>(q, kk, v, dtype, BH, n, window, scale, causal, out, s); break;
        case 64: launch_local_d<64>(q, kk, v, dtype, BH, n, window, scale, causal, out, s); break;
        default: launch_local_d<128>(q, kk, v, dtype, BH, n, window, scale, causal, out, s); break;
    }
    return hipGetLastError();
}

}  // namespace rt
