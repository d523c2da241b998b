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
// v_mfma_f32_16x16x32_bf16.  One workgroup = a 128 x 128 output tile, four
// waves of 64 x 64; K advances 64 at a time through double-buffered LDS tiles
// fed by register prefetch.  Each wave computes the transposed product
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

constexpr int PBM = 128, PBN = 128, PBK = 64;   // tile sizes
constexpr int PLD = PBK + 8;                     // LDS row stride (bf16): 144 bytes
constexpr int PNT = 256;
constexpr int PCH = PBK / 8;                     // 16-byte chunks per tile row
constexpr int PPT = PBM * PCH / PNT;             // chunks per thread per tile (4)

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

template <int AMODE, int CMODE>
__global__ __launch_bounds__(PNT, 2) void proj_kernel(ProjArgs p) {
    __shared__ __attribute__((aligned(16))) u16 la[2][PBM * PLD];
    __shared__ __attribute__((aligned(16))) u16 lw[2][PBN * PLD];

    const int m0 = blockIdx.x * PBM, n0 = blockIdx.y * PBN;
    const int lane = lane_id(), wv = wave_id();
    const int g = lane >> 4, r16 = lane & 15;
    const int wm = wv >> 1, wn = wv & 1;
    const u16* w = static_cast<const u16*>(p.w);

    uint4 ra[PPT], rw[PPT];
    auto load = [&](int k0) {
#pragma unroll
        for (int it = 0; it < PPT; ++it) {
            const int e = threadIdx.x + PNT * it;
            const int r = e / PCH, k = k0 + 8 * (e % PCH);
            const bool ka = k < p.K;
            ra[it] = (m0 + r < p.M && ka) ? *reinterpret_cast<const uint4*>(a_chunk<AMODE>(p, m0 + r, k))
                                          : zero_u4();
            rw[it] = (n0 + r < p.N && ka)
                         ? *reinterpret_cast<const uint4*>(w + (long)(n0 + r) * p.K + k)
                         : zero_u4();
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int it = 0; it < PPT; ++it) {
            const int e = threadIdx.x + PNT * it;
            const int r = e / PCH, c = 8 * (e % PCH);
            *reinterpret_cast<uint4*>(&la[buf][r * PLD + c]) = ra[it];
            *reinterpret_cast<uint4*>(&lw[buf][r * PLD + c]) = rw[it];
        }
    };

    f32x4 acc[4][4];   // [n block][m block]: C^T rows n0 + 64wn + 16ni + 4g + i, col m0 + 64wm + 16mi + r16
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) acc[ni][mi] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (p.K + PBK - 1) / PBK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load((kt + 1) * PBK);
#pragma unroll
        for (int kk = 0; kk < PBK / 32; ++kk) {
            bf16x8 av[4], wvv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[i] = as_bf16x8(*reinterpret_cast<const uint4*>(
                    &la[buf][(64 * wm + 16 * i + r16) * PLD + 32 * kk + 8 * g]));
                wvv[i] = as_bf16x8(*reinterpret_cast<const uint4*>(
                    &lw[buf][(64 * wn + 16 * i + r16) * PLD + 32 * kk + 8 * g]));
            }
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) acc[ni][mi] = mfma16(wvv[ni], av[mi], acc[ni][mi]);
        }
        if (kt + 1 < nk) {
            store(buf ^ 1);
            __syncthreads();
        }
    }

    // Epilogue: lane holds C[m][n .. n+3] for m = m0 + 64wm + 16mi + r16,
    // n = n0 + 64wn + 16ni + 4g.
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int m = m0 + 64 * wm + 16 * mi + r16;
        if (m >= p.M) continue;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const int nn = n0 + 64 * wn + 16 * ni + 4 * g;
            if (nn >= p.N) continue;
            float c0 = acc[ni][mi][0], c1 = acc[ni][mi][1], c2 = acc[ni][mi][2], c3 = acc[ni][mi][3];
            if constexpr (CMODE == 0) {
                const long off = (long)m * p.N + nn;
                if (p.res != nullptr) {
                    const uint2 rr = *reinterpret_cast<const uint2*>(static_cast<const u16*>(p.res) + off);
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

}  // namespace

hipError_t launch_proj(const ProjArgs& p, int amode, int cmode, hipStream_t s) {
    const dim3 grid((p.M + PBM - 1) / PBM, (p.N + PBN - 1) / PBN);
    if (amode == 0 && cmode == 1) hipLaunchKernelGGL((proj_kernel<0, 1>), grid, dim3(PNT), 0, s, p);
    else if (amode == 1 && cmode == 0) hipLaunchKernelGGL((proj_kernel<1, 0>), grid, dim3(PNT), 0, s, p);
    else if (amode == 0 && cmode == 0) hipLaunchKernelGGL((proj_kernel<0, 0>), grid, dim3(PNT), 0, s, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace rt
