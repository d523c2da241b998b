// proj.hip -- the projections around the attention layer (gfx950).
//
// The paperlayer.ai summary of "Efficient Content-Based Sparse Attention with
// Routing Transformers" (§3) describes a self-attention layer as three learned
// linear maps from n vectors of dimension d_model to queries, keys and values,
// and §5 reports a 22-layer model at sequence length 8192.  A layer of that
// stack here maps x [B, n, d_model] to the heads' inputs with one matrix
// product (shared query/key and values of the routed heads, queries, keys and
// values of the local heads, each written head-major [B, H, n, d]), runs the
// attention, and maps the heads' outputs back with a second product plus the
// residual: y = x + [routed | local] W_o.
//
// proj_kernel: C = A W^T with W stored [N][K] (k contiguous, like the rows of
// a linear layer's weight), bf16 operands, float32 accumulation on
// v_mfma_f32_16x16x32_bf16.  One workgroup = a BM x BN output tile of waves
// holding 64 x 64 blocks each (256 x 256 with sixteen waves, 128 x 256 with
// eight); K advances 64 at a time through double-buffered LDS tiles fed by
// register prefetch.  Each wave computes the transposed product
// (C^T = W A^T) so that every lane ends up holding four consecutive output
// columns of one row: one 8-byte store per block.
//   A layouts: row-major [M][K], or head-major segments (the concatenated
//   outputs of the routed and the local heads, [B, H_s, n, d] each).
//   C layouts: row-major [M][N] with an optional residual of the same layout
//   added in float32, or head-major segments (up to five tensors).
#include "rt_common.hpp"
#include "rt_internal.hpp"

namespace rt {
namespace {

constexpr int PBK = 64;                          // K step
constexpr int PLD = PBK + 8;                     // LDS row stride (bf16): 144 bytes
constexpr int PCH = PBK / 8;                     // 16-byte chunks per tile row

// Address of the 16-byte chunk holding elements (m, k .. k+7) of A.
template <int AMODE>
__device__ __forceinline__ const u16* a_chunk(const ProjArgs& p, int m, int k) {
    if constexpr (AMODE == 0) {
        return static_cast<const u16*>(p.a[0]) + (long)m * p.K + k;
    } else {
        const int hh = k / p.d, i = k % p.d;
        const int s = hh < p.ha[0] ? 0 : 1;
        const int hl = s == 0 ? hh : hh - p.ha[0];
        const int b = m / p.n, t = m % p.n;
        return static_cast<const u16*>(p.a[s]) + (((long)b * p.ha[s] + hl) * p.n + t) * p.d + i;
    }
}

// Tile shape: a BM x BN output tile per workgroup, WM x WN waves each holding
// a (BM / WM) x (BN / WN) block of 16 x 16 MFMA tiles.
template <int BM, int BN, int WM, int WN>
struct ProjCfg {
    static constexpr int NT = 64 * WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;   // one wave's block
    static constexpr int MI = TM / 16, NI = TN / 16;
    static constexpr int APT = BM * PCH / NT;          // A chunks per thread per K step
    static constexpr int WPT = BN * PCH / NT;          // W chunks per thread per K step
    static_assert(BM * PCH % NT == 0 && BN * PCH % NT == 0, "whole chunks per thread");
    static_assert(TM % 16 == 0 && TN % 16 == 0, "whole MFMA tiles per wave");
};

template <int AMODE, int CMODE, int BM, int BN, int WM, int WN, int MINB>
__global__ __launch_bounds__(64 * WM * WN, MINB) void proj_kernel(ProjArgs p) {
    using C = ProjCfg<BM, BN, WM, WN>;
    __shared__ __attribute__((aligned(16))) u16 la[2][BM * PLD];
    __shared__ __attribute__((aligned(16))) u16 lw[2][BN * PLD];

    const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
    const int lane = lane_id(), wv = wave_id();
    const int g = lane >> 4, r16 = lane & 15;
    const int wm = wv / WN, wn = wv % WN;
    const u16* w = static_cast<const u16*>(p.w);

    uint4 ra[C::APT], rw[C::WPT];
    auto load = [&](int k0) {
#pragma unroll
        for (int it = 0; it < C::APT; ++it) {
            const int e = threadIdx.x + C::NT * it;
            const int r = e / PCH, k = k0 + 8 * (e % PCH);
            ra[it] = (m0 + r < p.M && k < p.K)
                         ? *reinterpret_cast<const uint4*>(a_chunk<AMODE>(p, m0 + r, k))
                         : zero_u4();
        }
#pragma unroll
        for (int it = 0; it < C::WPT; ++it) {
            const int e = threadIdx.x + C::NT * it;
            const int r = e / PCH, k = k0 + 8 * (e % PCH);
            rw[it] = (n0 + r < p.N && k < p.K)
                         ? *reinterpret_cast<const uint4*>(w + (long)(n0 + r) * p.K + k)
                         : zero_u4();
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int it = 0; it < C::APT; ++it) {
            const int e = threadIdx.x + C::NT * it;
            *reinterpret_cast<uint4*>(&la[buf][(e / PCH) * PLD + 8 * (e % PCH)]) = ra[it];
        }
#pragma unroll
        for (int it = 0; it < C::WPT; ++it) {
            const int e = threadIdx.x + C::NT * it;
            *reinterpret_cast<uint4*>(&lw[buf][(e / PCH) * PLD + 8 * (e % PCH)]) = rw[it];
        }
    };

    // acc[ni][mi]: C^T rows n0 + TN wn + 16 ni + 4 g + i, column m0 + TM wm + 16 mi + r16
    f32x4 acc[C::NI][C::MI];
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi) acc[ni][mi] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (p.K + PBK - 1) / PBK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load((kt + 1) * PBK);
#pragma unroll
        for (int kk = 0; kk < PBK / 32; ++kk) {
            bf16x8 av[C::MI], wvv[C::NI];
#pragma unroll
            for (int i = 0; i < C::MI; ++i)
                av[i] = as_bf16x8(*reinterpret_cast<const uint4*>(
                    &la[buf][(C::TM * wm + 16 * i + r16) * PLD + 32 * kk + 8 * g]));
#pragma unroll
            for (int i = 0; i < C::NI; ++i)
                wvv[i] = as_bf16x8(*reinterpret_cast<const uint4*>(
                    &lw[buf][(C::TN * wn + 16 * i + r16) * PLD + 32 * kk + 8 * g]));
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
                for (int mi = 0; mi < C::MI; ++mi) acc[ni][mi] = mfma16(wvv[ni], av[mi], acc[ni][mi]);
        }
        if (kt + 1 < nk) {
            store(buf ^ 1);
            __syncthreads();
        }
    }

    // Epilogue: lane holds C[m][n .. n+3] for m = m0 + TM wm + 16 mi + r16,
    // n = n0 + TN wn + 16 ni + 4 g.  The residual's elements are all requested
    // first (addresses clamped into it, so no load sits under a branch), then
    // added: one memory round trip rather than one per block.
    const bool with_res = CMODE == 0 && p.res != nullptr;
    uint2 rres[C::MI][C::NI];
    if (with_res) {
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni) {
                const int m = min(m0 + C::TM * wm + 16 * mi + r16, p.M - 1);
                const int nn = min(n0 + C::TN * wn + 16 * ni + 4 * g, p.N - 4);
                rres[mi][ni] = *reinterpret_cast<const uint2*>(static_cast<const u16*>(p.res) +
                                                               (long)m * p.N + nn);
            }
    }
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
        const int m = m0 + C::TM * wm + 16 * mi + r16;
        if (m >= p.M) continue;
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni) {
            const int nn = n0 + C::TN * wn + 16 * ni + 4 * g;
            if (nn >= p.N) continue;
            float c0 = acc[ni][mi][0], c1 = acc[ni][mi][1], c2 = acc[ni][mi][2], c3 = acc[ni][mi][3];
            if constexpr (CMODE == 0) {
                const long off = (long)m * p.N + nn;
                if (with_res) {
                    const uint2 rr = rres[mi][ni];
                    c0 += bf2f((u16)(rr.x & 0xffffu));
                    c1 += bf2f((u16)(rr.x >> 16));
                    c2 += bf2f((u16)(rr.y & 0xffffu));
                    c3 += bf2f((u16)(rr.y >> 16));
                }
                store4<u16>(static_cast<u16*>(p.c[0]) + off, c0, c1, c2, c3);
            } else {
                const int hh = nn / p.d, i = nn % p.d;
                int s = 0, hl = hh;
                while (s < 4 && hl >= p.hc[s]) hl -= p.hc[s++];
                const int b = m / p.n, t = m % p.n;
                u16* dst = static_cast<u16*>(p.c[s]) + (((long)b * p.hc[s] + hl) * p.n + t) * p.d + i;
                store4<u16>(dst, c0, c1, c2, c3);
            }
        }
    }
}

template <int AMODE, int CMODE, int BM, int BN, int WM, int WN, int MINB>
void launch_proj_cfg(const ProjArgs& p, hipStream_t s) {
    const dim3 grid((p.M + BM - 1) / BM, (p.N + BN - 1) / BN);
    hipLaunchKernelGGL((proj_kernel<AMODE, CMODE, BM, BN, WM, WN, MINB>), grid, dim3(64 * WM * WN),
                       0, s, p);
}

}  // namespace

hipError_t launch_proj(const ProjArgs& p, int amode, int cmode, hipStream_t s) {
    // Measured at d_model = 1024, n = 8192, 8 + 4 heads of 128: the input
    // product (N = 3584) runs best on 256 x 256 tiles of sixteen waves (four a
    // SIMD hide the LDS and global latencies), the output product (N = 1024:
    // 256 x 256 tiles would leave half the CUs idle) on 128 x 256 tiles of
    // eight waves; 128 x 128 tiles of four waves were 19% and 14% slower.
    if (amode == 0 && cmode == 1) launch_proj_cfg<0, 1, 256, 256, 4, 4, 1>(p, s);
    else if (amode == 1 && cmode == 0) launch_proj_cfg<1, 0, 128, 256, 2, 4, 1>(p, s);
    else if (amode == 0 && cmode == 0) launch_proj_cfg<0, 0, 128, 256, 2, 4, 1>(p, s);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace rt
