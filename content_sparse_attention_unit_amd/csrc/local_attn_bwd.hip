// local_attn_bwd.hip -- backward of the sliding-window attention (gfx950).
//
// The local heads of the layer (arXiv abstract; §6 of the paperlayer.ai
// summary of "Efficient Content-Based Sparse Attention with Routing
// Transformers") attend with ordinary softmax attention (summary §3) to the
// positions [i - window + 1, i] (causal) or to the band |i - j| < window.  For
// the output gradient dO, with P the softmax rows and l = scale <q_i, k_j>:
//   dV_j = sum_i P_ij dO_i,   dP_ij = <dO_i, v_j>,
//   dl_ij = P_ij (dP_ij - D_i) with D_i = sum_j P_ij dP_ij,
//   dQ_i = scale sum_j dl_ij k_j,   dK_j = scale sum_i dl_ij q_i.
//
// Two kernels, no atomics (results do not depend on scheduling):
//   local_bwd_dq_kernel  one workgroup = 64 queries (four waves of 16, a lane
//                        owns a query).  Sweep 1 over the key tiles forms each
//                        query's log-sum-exp and D_i in one online pass
//                        (running maximum, denominator and sum of e^l dP, per
//                        lane, merged over the four lanes of a query at the
//                        end); sweep 2 recomputes P and dP and accumulates
//                        dQ^T = K^T dl^T.  It writes lse and D for the second
//                        kernel.
//   local_bwd_dkv_kernel one workgroup = 64 keys (a lane owns a key); over
//                        the query tiles that see them it recomputes P and dP
//                        from lse and D and accumulates dV^T = dO^T P and
//                        dK^T = Q^T dl.
// All products are v_mfma_f32_16x16x32_bf16: S^T = K Q^T and dP^T = V dO^T
// (or S = Q K^T and dP = dO V^T) from a row-major LDS tile and the lane's own
// rows in registers; the sums over the tile's rows take their transposed
// operand straight from the row-major tile (transposing LDS reads), with P and
// dl rounded to bf16 for those products.  Gradients are float32.
#include "rt_common.hpp"
#include "rt_internal.hpp"

namespace rt {
namespace {

template <int D>
struct LbCfg {
    static constexpr int LDX = D + 16;         // LDS row stride (bf16): an odd multiple of 16
    static constexpr int T = 64;               // rows per tile
    static constexpr int NS = D / 32;          // MFMA k-steps over the head dimension
    static constexpr int NJ = D / 16;          // 16-wide blocks of the head dimension
    static constexpr int CPR = D / 8;          // 16-byte chunks per row
    static constexpr int CPT = T * CPR / 256;  // chunks per thread per tile
};

__device__ __forceinline__ bool band_vis(int j, int i, int n, int window, int causal) {
    if (i >= n || j >= n) return false;
    return causal ? (j <= i && j > i - window) : (j > i - window && j < i + window);
}

// Rows [r0, r0 + 64) of a [n][D] bf16 tensor into LDS; rows past n are zeros.
template <int D>
__device__ __forceinline__ void stage_rows(u16* dst, buf_rsrc rs, int r0, int n) {
    using C = LbCfg<D>;
    uint4 t[C::CPT];
#pragma unroll
    for (int it = 0; it < C::CPT; ++it) {
        const int e = threadIdx.x + 256 * it;
        const int r = e / C::CPR, ch = e % C::CPR;
        const int row = r0 + r;
        t[it] = buffer_load16(rs, row < n ? (uint32_t)(row * D + 8 * ch) * 2u : kOutOfRange);
    }
#pragma unroll
    for (int it = 0; it < C::CPT; ++it) {
        const int e = threadIdx.x + 256 * it;
        *reinterpret_cast<uint4*>(&dst[(e / C::CPR) * C::LDX + 8 * (e % C::CPR)]) = t[it];
    }
}

// acc[rb] = (rows 16 rb + r16 of the tile) . (this lane's row, as B operand):
// element i of acc[rb] pairs tile row 16 rb + 4 g + i with the lane's column r16.
template <int D>
__device__ __forceinline__ void tile_dot(const u16* lt, const uint4 (&b)[LbCfg<D>::NS],
                                         f32x4 (&acc)[4], int r16, int g) {
    using C = LbCfg<D>;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
            const bf16x8 a = as_bf16x8(
                *reinterpret_cast<const uint4*>(&lt[(16 * rb + r16) * C::LDX + 32 * s + 8 * g]));
            acc[rb] = mfma16(a, as_bf16x8(b[s]), acc[rb]);
        }
    }
}

template <int D>
__device__ __forceinline__ void load_row_frags(const u16* x, long row, bool ok,
                                               uint4 (&r)[LbCfg<D>::NS], int g) {
#pragma unroll
    for (int s = 0; s < LbCfg<D>::NS; ++s)
        r[s] = ok ? *reinterpret_cast<const uint4*>(x + row * D + 32 * s + 8 * g) : zero_u4();
}

template <int D>
__global__ __launch_bounds__(256) void local_bwd_dq_kernel(
    const u16* __restrict__ q, const u16* __restrict__ kk, const u16* __restrict__ v,
    const u16* __restrict__ dout, int n, int window, float scale, int causal,
    float* __restrict__ dq, float* __restrict__ lse2_out, float* __restrict__ dd_out) {
    using C = LbCfg<D>;
    __shared__ __attribute__((aligned(16))) u16 lk[C::T * C::LDX];
    __shared__ __attribute__((aligned(16))) u16 lv[C::T * C::LDX];

    const int item = xcd_contiguous(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
    const int bh = item / gridDim.x;
    const int q0 = (item % gridDim.x) * C::T;
    const long base = (long)bh * n;
    const int lane = lane_id(), wv = wave_id();
    const int g = lane >> 4, r16 = lane & 15;
    const int qi = q0 + 16 * wv + r16;   // this lane's query
    const float sl2 = scale * 1.4426950408889634f;

    uint4 qreg[C::NS], oreg[C::NS];
    load_row_frags<D>(q, base + qi, qi < n, qreg, g);
    load_row_frags<D>(dout, base + qi, qi < n, oreg, g);
    const buf_rsrc krs = make_rsrc(kk + base * D, (uint32_t)n * D * 2u);
    const buf_rsrc vrs = make_rsrc(v + base * D, (uint32_t)n * D * 2u);

    const int lo = max(0, q0 - window + 1);
    const int hi = causal ? min(n - 1, q0 + C::T - 1) : min(n - 1, q0 + C::T - 1 + window - 1);
    const int t_first = (lo / C::T) * C::T;

    // Sweep 1: per lane, over its keys, the running maximum m (log2 units),
    // the denominator z and a = sum e^(l - m) dP.
    float m = -INFINITY, z = 0.f, a = 0.f;
    for (int t0 = t_first; t0 <= hi; t0 += C::T) {
        __syncthreads();
        stage_rows<D>(lk, krs, t0, n);
        stage_rows<D>(lv, vrs, t0, n);
        __syncthreads();
        f32x4 s[4], dp[4];
        tile_dot<D>(lk, qreg, s, r16, g);
        tile_dot<D>(lv, oreg, dp, r16, g);
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = t0 + 16 * kb + 4 * g + i;
                s[kb][i] = band_vis(j, qi, n, window, causal) ? s[kb][i] * sl2 : -INFINITY;
                tmax = fmaxf(tmax, s[kb][i]);
            }
        if (tmax == -INFINITY) continue;
        const float mn = fmaxf(m, tmax);
        const float f = __builtin_amdgcn_exp2f(m - mn);   // 0 when m = -inf
        z *= f;
        a *= f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = __builtin_amdgcn_exp2f(s[kb][i] - mn);
                z += e;
                a += e * dp[kb][i];
            }
        m = mn;
    }
    // merge the four lanes of each query (lanes r16, r16 + 16, r16 + 32, r16 + 48)
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
        const float m2 = __shfl_xor(m, off), z2 = __shfl_xor(z, off), a2 = __shfl_xor(a, off);
        const float mn = fmaxf(m, m2);
        const float f1 = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
        const float f2 = (m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
        z = z * f1 + z2 * f2;
        a = a * f1 + a2 * f2;
        m = mn;
    }
    // every query sees at least itself, so z > 0 for a query inside the row
    const float lse2 = (qi < n) ? m + log2f(z) : 0.f;
    const float ddq = (qi < n) ? a / z : 0.f;
    if (g == 0 && qi < n) {
        lse2_out[base + qi] = lse2;
        dd_out[base + qi] = ddq;
    }

    // Sweep 2: dl = P (dP - D) and dQ^T += K^T dl^T.
    f32x4 acc[C::NJ];
#pragma unroll
    for (int jb = 0; jb < C::NJ; ++jb) acc[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int t0 = t_first; t0 <= hi; t0 += C::T) {
        __syncthreads();
        stage_rows<D>(lk, krs, t0, n);
        stage_rows<D>(lv, vrs, t0, n);
        __syncthreads();
        f32x4 s[4], dp[4];
        tile_dot<D>(lk, qreg, s, r16, g);
        tile_dot<D>(lv, oreg, dp, r16, g);
        uint32_t pw[4][2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            float dl[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = t0 + 16 * kb + 4 * g + i;
                const float p = band_vis(j, qi, n, window, causal)
                                    ? __builtin_amdgcn_exp2f(s[kb][i] * sl2 - lse2)
                                    : 0.f;
                dl[i] = p * (dp[kb][i] - ddq);
            }
            pw[kb][0] = cvt_pk_bf16(dl[0], dl[1]);
            pw[kb][1] = cvt_pk_bf16(dl[2], dl[3]);
        }
        acc_xt_w<C::NJ, C::LDX>(pw, acc, lk, r16, g, 3);
    }
    if (qi < n) {
#pragma unroll
        for (int jb = 0; jb < C::NJ; ++jb)
            store4<float>(dq + (base + qi) * D + 16 * jb + 4 * g, scale * acc[jb][0],
                          scale * acc[jb][1], scale * acc[jb][2], scale * acc[jb][3]);
    }
}

template <int D>
__global__ __launch_bounds__(256) void local_bwd_dkv_kernel(
    const u16* __restrict__ q, const u16* __restrict__ kk, const u16* __restrict__ v,
    const u16* __restrict__ dout, int n, int window, float scale, int causal,
    const float* __restrict__ lse2_in, const float* __restrict__ dd_in, float* __restrict__ dk,
    float* __restrict__ dv) {
    using C = LbCfg<D>;
    __shared__ __attribute__((aligned(16))) u16 lq[C::T * C::LDX];
    __shared__ __attribute__((aligned(16))) u16 lo_[C::T * C::LDX];
    __shared__ float llse[C::T], ldd[C::T];

    const int item = xcd_contiguous(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
    const int bh = item / gridDim.x;
    const int k0 = (item % gridDim.x) * C::T;
    const long base = (long)bh * n;
    const int lane = lane_id(), wv = wave_id();
    const int g = lane >> 4, r16 = lane & 15;
    const int kj = k0 + 16 * wv + r16;   // this lane's key
    const float sl2 = scale * 1.4426950408889634f;

    uint4 kreg[C::NS], vreg[C::NS];
    load_row_frags<D>(kk, base + kj, kj < n, kreg, g);
    load_row_frags<D>(v, base + kj, kj < n, vreg, g);
    const buf_rsrc qrs = make_rsrc(q + base * D, (uint32_t)n * D * 2u);
    const buf_rsrc ors = make_rsrc(dout + base * D, (uint32_t)n * D * 2u);

    // queries that see the workgroup's keys
    const int lo = causal ? k0 : max(0, k0 - window + 1);
    const int hi = min(n - 1, k0 + C::T - 1 + window - 1);
    const int t_first = (lo / C::T) * C::T;

    f32x4 adk[C::NJ], adv[C::NJ];
#pragma unroll
    for (int jb = 0; jb < C::NJ; ++jb) {
        adk[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        adv[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int t0 = t_first; t0 <= hi; t0 += C::T) {
        __syncthreads();
        stage_rows<D>(lq, qrs, t0, n);
        stage_rows<D>(lo_, ors, t0, n);
        if (threadIdx.x < C::T) {
            const int qr = t0 + threadIdx.x;
            llse[threadIdx.x] = qr < n ? lse2_in[base + qr] : 0.f;
            ldd[threadIdx.x] = qr < n ? dd_in[base + qr] : 0.f;
        }
        __syncthreads();
        f32x4 s[4], dp[4];
        tile_dot<D>(lq, kreg, s, r16, g);     // S[query 16 qb + 4 g + i][key r16]
        tile_dot<D>(lo_, vreg, dp, r16, g);   // dP[query][key]
        uint32_t pp[4][2], pl[4][2];
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
            float p[4], dl[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * qb + 4 * g + i;
                p[i] = band_vis(kj, t0 + r, n, window, causal)
                           ? __builtin_amdgcn_exp2f(s[qb][i] * sl2 - llse[r])
                           : 0.f;
                dl[i] = p[i] * (dp[qb][i] - ldd[r]);
            }
            pp[qb][0] = cvt_pk_bf16(p[0], p[1]);
            pp[qb][1] = cvt_pk_bf16(p[2], p[3]);
            pl[qb][0] = cvt_pk_bf16(dl[0], dl[1]);
            pl[qb][1] = cvt_pk_bf16(dl[2], dl[3]);
        }
        acc_xt_w<C::NJ, C::LDX>(pp, adv, lo_, r16, g, 3);   // dV^T += dO^T P
        acc_xt_w<C::NJ, C::LDX>(pl, adk, lq, r16, g, 3);    // dK^T += Q^T dl
    }
    if (kj < n) {
#pragma unroll
        for (int jb = 0; jb < C::NJ; ++jb) {
            store4<float>(dk + (base + kj) * D + 16 * jb + 4 * g, scale * adk[jb][0],
                          scale * adk[jb][1], scale * adk[jb][2], scale * adk[jb][3]);
            store4<float>(dv + (base + kj) * D + 16 * jb + 4 * g, adv[jb][0], adv[jb][1],
                          adv[jb][2], adv[jb][3]);
        }
    }
}

template <int D>
void launch_local_bwd_d(const u16* q, const u16* kk, const u16* v, const u16* dout, int BH, int n,
                        int window, float scale, int causal, float* dq, float* dk, float* dv,
                        float* lse2, float* dd, hipStream_t s) {
    const dim3 grid((n + 63) / 64, BH);
    hipLaunchKernelGGL(local_bwd_dq_kernel<D>, grid, dim3(256), 0, s, q, kk, v, dout, n, window,
                       scale, causal, dq, lse2, dd);
    hipLaunchKernelGGL(local_bwd_dkv_kernel<D>, grid, dim3(256), 0, s, q, kk, v, dout, n, window,
                       scale, causal, lse2, dd, dk, dv);
}

}  // namespace

size_t local_bwd_workspace_bytes(int BH, int n) { return (size_t)BH * n * 2 * sizeof(float); }

hipError_t launch_local_attn_bwd(const void* q, const void* kk, const void* v, const void* dout,
                                 int BH, int n, int d, int window, float scale, int causal,
                                 float* dq, float* dk, float* dv, void* ws, hipStream_t s) {
    float* lse2 = static_cast<float*>(ws);
    float* dd = lse2 + (size_t)BH * n;
    const u16 *q16 = static_cast<const u16*>(q), *k16 = static_cast<const u16*>(kk),
              *v16 = static_cast<const u16*>(v), *o16 = static_cast<const u16*>(dout);
    if (d == 64)
        launch_local_bwd_d<64>(q16, k16, v16, o16, BH, n, window, scale, causal, dq, dk, dv, lse2,
                               dd, s);
    else if (d == 128)
        launch_local_bwd_d<128>(q16, k16, v16, o16, BH, n, window, scale, causal, dq, dk, dv, lse2,
                                dd, s);
    else
        return hipErrorNotSupported;
    return hipGetLastError();
}

}  // namespace rt
