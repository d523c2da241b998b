// layer_bwd.hip -- gradients of the layer's projections and of the unit
// normalisation of the routed heads (gfx950).
//
// The paperlayer.ai summary of "Efficient Content-Based Sparse Attention with
// Routing Transformers" (§3) has a self-attention layer map its n input
// vectors to queries, keys and values with learned linear maps, and (§4) use
// queries and keys unit-normalised.  With [qk | v | q_l | k_l | v_l] = x W_in^T
// and y = x + O W_o^T (O the heads' outputs, concatenated per token):
//   dO = dy W_o,   dW_o = dy^T O,   dx = dy + dC W_in,   dW_in = dC^T x,
// dC being the heads' input gradients; and for x^ = x / max(||x||, 1e-12),
//   dx = (g - x^ <x^, g>) / ||x||   (g / 1e-12 where the clamp holds).
//
// gemm_kernel: C = A B^T over a contraction K for the four products above,
// bf16 operands (float32 gradients are rounded to bf16 as they are staged),
// float32 accumulation on v_mfma_f32_16x16x32_bf16.  Each operand X[idx][k]
// lives in memory either k-contiguous (row-major rows of k) or
// idx-contiguous (rows of idx for each k): the tile is copied to LDS in its
// memory orientation, and the fragments come from plain 8-byte reads in the
// first case and from transposing LDS reads (ds_read_b64_tr_b16) in the
// second, both giving the same order of the contraction index, so no operand
// is ever transposed in memory.  Operands can also be the head-major
// [B][H][n][d] tensors of the attention heads (several segments, concatenated
// over heads), so the layer needs no copies.  One workgroup = a 128 x 128
// output tile (eight waves of 64 x 32) or a 128 x 256 one (sixteen waves of
// 32 x 64), K in steps of 64 through
// double-buffered LDS tiles fed by register prefetch; each wave computes the
// transposed product so a lane holds four consecutive output columns.  The
// weight gradients have few output tiles and a long contraction (all tokens):
// they split the contraction over several workgroups per tile, write the
// partial products to a workspace and add them up in a fixed order
// (gemm_reduce_kernel), so results do not depend on scheduling.
//
// norm_bwd_kernel: one wave per row, the row and its gradients in registers.
#include "rt_common.hpp"
#include "rt_internal.hpp"

namespace rt {
namespace {

constexpr int GBK = 64;
constexpr int GPLD = GBK + 8;      // k-contiguous tile: row stride (bf16)
// idx-contiguous tile of ROWS rows: row stride (bf16), an odd multiple of 16
template <int ROWS>
constexpr int gldi() { return ROWS + 16; }

enum { OP_KC_RM = 0, OP_IC_RM = 1, OP_KC_HM = 2, OP_IC_HM = 3 };

// Address of element (idx, k) of an operand; `col` is the head-concatenated
// column and `tok` the token for the head-major modes.
template <int MODE, bool F32>
__device__ __forceinline__ const void* op_addr(const GemmOperand& o, int idx, int k, int n, int d) {
    const int esz = F32 ? 4 : 2;
    long off;
    int s = 0;
    if constexpr (MODE == OP_KC_RM) {
        off = (long)idx * o.ld + k;
    } else if constexpr (MODE == OP_IC_RM) {
        off = (long)k * o.ld + idx;
    } else {
        const int tok = MODE == OP_KC_HM ? idx : k;
        const int col = MODE == OP_KC_HM ? k : idx;
        int hl = col / d;
        const int i = col - hl * d;
        while (s < 4 && hl >= o.hs[s]) hl -= o.hs[s++];
        const int b = tok / n, t = tok - b * n;
        off = (((long)b * o.hs[s] + hl) * n + t) * d + i;
    }
    return static_cast<const char*>(o.p[s]) + off * esz;
}

// Eight consecutive elements along the operand's contiguous direction, as
// loaded: bf16 as they are, float32 kept whole until the tile is stored to LDS
// (rounding them at the load would make the load wait, before the products of
// the tile in LDS, for data that has a whole contraction step to arrive).
template <bool F32> struct Chunk8;
template <> struct Chunk8<false> { uint4 v; };
template <> struct Chunk8<true> { float4 a, b; };

template <bool F32>
__device__ __forceinline__ Chunk8<F32> load8(const void* p) {
    if constexpr (F32) {
        return Chunk8<true>{*reinterpret_cast<const float4*>(p),
                            *(reinterpret_cast<const float4*>(p) + 1)};
    } else {
        return Chunk8<false>{*reinterpret_cast<const uint4*>(p)};
    }
}

template <bool F32>
__device__ __forceinline__ uint4 as_bf16x8_bits(const Chunk8<F32>& c) {
    if constexpr (F32) {
        return make_uint4(cvt_pk_bf16(c.a.x, c.a.y), cvt_pk_bf16(c.a.z, c.a.w),
                          cvt_pk_bf16(c.b.x, c.b.y), cvt_pk_bf16(c.b.z, c.b.w));
    } else {
        return c.v;
    }
}

constexpr bool k_contig(int mode) { return mode == OP_KC_RM || mode == OP_KC_HM; }

// Element (idx, k) of chunk `it` of this thread in a ROWS x 64 operand tile.
template <int MODE, int ROWS, int NT>
__device__ __forceinline__ void chunk_pos(int it, int idx0, int k0, int& idx, int& k) {
    const int e = threadIdx.x + NT * it;
    if constexpr (k_contig(MODE)) {
        idx = idx0 + e / 8;
        k = k0 + 8 * (e % 8);
    } else {
        idx = idx0 + 8 * (e % (ROWS / 8));
        k = k0 + e / (ROWS / 8);
    }
}

// One ROWS x 64 operand tile (rows idx0.., contraction k0..) into registers,
// NT threads, CPT = ROWS * 8 / NT chunks of eight elements each.  Addresses
// are clamped into the operand so that every load is issued unconditionally;
// chunks outside it are zeroed by tile_store.
template <int MODE, bool F32, int ROWS, int NT, int CPT>
__device__ __forceinline__ void tile_load(const GemmOperand& o, int idx0, int nidx, int k0, int K,
                                          int n, int d, Chunk8<F32> (&r)[CPT]) {
    static_assert(ROWS * 8 == NT * CPT, "whole chunks per thread");
#pragma unroll
    for (int it = 0; it < CPT; ++it) {
        int idx, k;
        chunk_pos<MODE, ROWS, NT>(it, idx0, k0, idx, k);
        // the eight elements run along k (k-contiguous) or along idx
        const int ic = k_contig(MODE) ? min(idx, nidx - 1) : max(0, min(idx, nidx - 8));
        const int kc = k_contig(MODE) ? max(0, min(k, K - 8)) : min(k, K - 1);
        r[it] = load8<F32>(op_addr<MODE, F32>(o, ic, kc, n, d));
    }
}

template <int MODE, bool F32, int ROWS, int NT, int CPT>
__device__ __forceinline__ void tile_store(u16* t, const Chunk8<F32> (&r)[CPT], int idx0, int nidx,
                                           int k0, int K) {
#pragma unroll
    for (int it = 0; it < CPT; ++it) {
        const int e = threadIdx.x + NT * it;
        int idx, k;
        chunk_pos<MODE, ROWS, NT>(it, idx0, k0, idx, k);
        const uint4 v = idx < nidx && k < K ? as_bf16x8_bits<F32>(r[it]) : zero_u4();
        if constexpr (k_contig(MODE))
            *reinterpret_cast<uint4*>(&t[(e / 8) * GPLD + 8 * (e % 8)]) = v;
        else
            *reinterpret_cast<uint4*>(&t[(e / (ROWS / 8)) * gldi<ROWS>() + 8 * (e % (ROWS / 8))]) = v;
    }
}

// Fragment of 16 rows (block b of the tile's idx) for contraction step kk
// (32 k): element e holds k = 32 kk + 4 g + e (e < 4) or 32 kk + 16 + 4 g + e - 4.
template <int MODE, int ROWS>
__device__ __forceinline__ bf16x8 frag(const u16* t, int b, int kk, int r16, int g) {
    constexpr int GLDI = gldi<ROWS>();
    if constexpr (k_contig(MODE)) {
        const u16* p = t + (16 * b + r16) * GPLD + 32 * kk + 4 * g;
        const uint2 lo = *reinterpret_cast<const uint2*>(p);
        const uint2 hi = *reinterpret_cast<const uint2*>(p + 16);
        return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
    } else {
        const u16* p = t + (32 * kk + 4 * g + (r16 >> 2)) * GLDI + 4 * (r16 & 3) + 16 * b;
        const uint2 lo = lds_read_tr16(p);
        const uint2 hi = lds_read_tr16(p + 16 * GLDI);
        return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
    }
}

// Tile shape: a TBM x TBN output tile per workgroup, WM x WN waves each holding
// a (TBM / WM) x (TBN / WN) block of 16 x 16 MFMA tiles.
template <int TBM, int TBN, int WM, int WN>
struct GemmCfg {
    static constexpr int NT = 64 * WM * WN;
    static constexpr int TM = TBM / WM, TN = TBN / WN;
    static constexpr int MI = TM / 16, NI = TN / 16;
    static constexpr int ACPT = TBM * 8 / NT, BCPT = TBN * 8 / NT;
};

template <int AM, bool AF, int BM, bool BF, int CM, int TBM, int TBN, int WM, int WN, int MINB>
__global__ __launch_bounds__(64 * WM * WN, MINB) void gemm_kernel(GemmArgs p) {
    using G = GemmCfg<TBM, TBN, WM, WN>;
    constexpr int NT = G::NT;
    constexpr int ASZ = k_contig(AM) ? TBM * GPLD : GBK * gldi<TBM>();
    constexpr int BSZ = k_contig(BM) ? TBN * GPLD : GBK * gldi<TBN>();
    __shared__ __attribute__((aligned(16))) u16 la[2][ASZ];
    __shared__ __attribute__((aligned(16))) u16 lb[2][BSZ];

    const int m0 = blockIdx.x * TBM, n0 = blockIdx.y * TBN;
    const int lane = lane_id(), wv = wave_id();
    const int g = lane >> 4, r16 = lane & 15;
    const int wm = wv / WN, wn = wv % WN;

    Chunk8<AF> ra[G::ACPT];
    Chunk8<BF> rb[G::BCPT];
    // [n block][m block]: C^T rows n0 + TN wn + 16ni + 4g + i, col m0 + TM wm + 16mi + r16
    f32x4 acc[G::NI][G::MI];
#pragma unroll
    for (int ni = 0; ni < G::NI; ++ni)
#pragma unroll
        for (int mi = 0; mi < G::MI; ++mi) acc[ni][mi] = f32x4{0.f, 0.f, 0.f, 0.f};

    // this workgroup's range of contraction tiles (all of them unless split)
    const int nk_all = (p.K + GBK - 1) / GBK;
    const int per = (nk_all + p.ksplit - 1) / p.ksplit;
    const int kt0 = (int)blockIdx.z * per;
    const int nk = min(nk_all, kt0 + per);
    tile_load<AM, AF, TBM, NT>(p.a, m0, p.M, kt0 * GBK, p.K, p.n, p.d, ra);
    tile_load<BM, BF, TBN, NT>(p.b, n0, p.N, kt0 * GBK, p.K, p.n, p.d, rb);
    tile_store<AM, AF, TBM, NT>(la[0], ra, m0, p.M, kt0 * GBK, p.K);
    tile_store<BM, BF, TBN, NT>(lb[0], rb, n0, p.N, kt0 * GBK, p.K);
    __syncthreads();
    for (int kt = kt0; kt < nk; ++kt) {
        const int buf = (kt - kt0) & 1;
        if (kt + 1 < nk) {
            tile_load<AM, AF, TBM, NT>(p.a, m0, p.M, (kt + 1) * GBK, p.K, p.n, p.d, ra);
            tile_load<BM, BF, TBN, NT>(p.b, n0, p.N, (kt + 1) * GBK, p.K, p.n, p.d, rb);
        }
#pragma unroll
        for (int kk = 0; kk < GBK / 32; ++kk) {
            bf16x8 fa[G::MI], fb[G::NI];
#pragma unroll
            for (int i = 0; i < G::MI; ++i) fa[i] = frag<AM, TBM>(la[buf], G::MI * wm + i, kk, r16, g);
#pragma unroll
            for (int i = 0; i < G::NI; ++i) fb[i] = frag<BM, TBN>(lb[buf], G::NI * wn + i, kk, r16, g);
#pragma unroll
            for (int ni = 0; ni < G::NI; ++ni)
#pragma unroll
                for (int mi = 0; mi < G::MI; ++mi) acc[ni][mi] = mfma16(fb[ni], fa[mi], acc[ni][mi]);
        }
        if (kt + 1 < nk) {
            tile_store<AM, AF, TBM, NT>(la[buf ^ 1], ra, m0, p.M, (kt + 1) * GBK, p.K);
            tile_store<BM, BF, TBN, NT>(lb[buf ^ 1], rb, n0, p.N, (kt + 1) * GBK, p.K);
            __syncthreads();
        }
    }

    // Epilogue: lane holds C[m][n .. n+3] for m = m0 + TM wm + 16mi + r16,
    // n = n0 + TN wn + 16ni + 4g.  The residual's elements are all requested
    // first (addresses clamped into it, so no load sits under a branch), then
    // added: one memory round trip rather than one per block.
    const bool with_res = CM == 0 && p.ksplit <= 1 && p.res != nullptr;
    uint2 rres[G::MI][G::NI];
    if (with_res) {
#pragma unroll
        for (int mi = 0; mi < G::MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < G::NI; ++ni) {
                const int m = min(m0 + G::TM * wm + 16 * mi + r16, p.M - 1);
                const int nn = min(n0 + G::TN * wn + 16 * ni + 4 * g, p.N - 4);
                rres[mi][ni] = *reinterpret_cast<const uint2*>(p.res + (long)m * p.N + nn);
            }
    }
#pragma unroll
    for (int mi = 0; mi < G::MI; ++mi) {
        const int m = m0 + G::TM * wm + 16 * mi + r16;
        if (m >= p.M) continue;
#pragma unroll
        for (int ni = 0; ni < G::NI; ++ni) {
            const int nn = n0 + G::TN * wn + 16 * ni + 4 * g;
            if (nn >= p.N) continue;
            float c0 = acc[ni][mi][0], c1 = acc[ni][mi][1], c2 = acc[ni][mi][2], c3 = acc[ni][mi][3];
            if (CM == 0 && p.ksplit > 1) {          // a partial product: added up later
                store4<float>(p.part + ((long)blockIdx.z * p.M + m) * p.N + nn, c0, c1, c2, c3);
            } else if constexpr (CM == 0) {
                const long off = (long)m * p.N + nn;
                if (with_res) {
                    const uint2 rr = rres[mi][ni];
                    c0 += bf2f((u16)(rr.x & 0xffffu));
                    c1 += bf2f((u16)(rr.x >> 16));
                    c2 += bf2f((u16)(rr.y & 0xffffu));
                    c3 += bf2f((u16)(rr.y >> 16));
                }
                store4<float>(static_cast<float*>(p.c[0]) + off, c0, c1, c2, c3);
            } else {
                int hl = nn / p.d;
                const int i = nn - hl * p.d;
                int s = 0;
                while (s < 4 && hl >= p.hc[s]) hl -= p.hc[s++];
                const int b = m / p.n, t = m - b * p.n;
                u16* dst = static_cast<u16*>(p.c[s]) + (((long)b * p.hc[s] + hl) * p.n + t) * p.d + i;
                store4<u16>(dst, c0, c1, c2, c3);
            }
        }
    }
}

// C = sum over z of part[z] (in order of z) + the residual: four elements a
// thread (M * N is a multiple of 4: N is).
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float* __restrict__ part, int S,
                                                          long MN, const u16* __restrict__ res,
                                                          float* __restrict__ c) {
    const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= MN) return;
    float4 t = *reinterpret_cast<const float4*>(part + i);
    for (int z = 1; z < S; ++z) {
        const float4 u = *reinterpret_cast<const float4*>(part + (long)z * MN + i);
        t.x += u.x;
        t.y += u.y;
        t.z += u.z;
        t.w += u.w;
    }
    if (res != nullptr) {
        const uint2 rr = *reinterpret_cast<const uint2*>(res + i);
        t.x += bf2f((u16)(rr.x & 0xffffu));
        t.y += bf2f((u16)(rr.x >> 16));
        t.z += bf2f((u16)(rr.y & 0xffffu));
        t.w += bf2f((u16)(rr.y >> 16));
    }
    *reinterpret_cast<float4*>(c + i) = t;
}

// One wave per row of d elements (d <= 128: two per lane).
template <bool BF16>
__global__ __launch_bounds__(256) void norm_bwd_kernel(const void* __restrict__ x,
                                                       const float* __restrict__ inv_norm,
                                                       const float* __restrict__ g1,
                                                       const float* __restrict__ g2, long rows,
                                                       int d, float* __restrict__ dx) {
    const long row = (long)blockIdx.x * 4 + wave_id();
    if (row >= rows) return;
    const int lane = lane_id();
    float xv[2], gv[2];
    float ss = 0.f, xg = 0.f;
    const float inv = inv_norm[row];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = lane + 64 * u;
        xv[u] = 0.f;
        gv[u] = 0.f;
        if (i < d) {
            const long o = row * d + i;
            xv[u] = BF16 ? bf2f(static_cast<const u16*>(x)[o]) : static_cast<const float*>(x)[o];
            gv[u] = g1[o] + (g2 != nullptr ? g2[o] : 0.f);
        }
        ss = fmaf(xv[u], xv[u], ss);
        xg = fmaf(xv[u] * inv, gv[u], xg);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        ss += __shfl_xor(ss, off);
        xg += __shfl_xor(xg, off);
    }
    const bool clamped = sqrtf(ss) < 1e-12f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = lane + 64 * u;
        if (i < d)
            dx[row * d + i] = clamped ? gv[u] * inv : (gv[u] - xv[u] * inv * xg) * inv;
    }
}

template <int AM, bool AF, int BM, bool BF, int CM, int TBM, int TBN, int WM, int WN, int MINB>
hipError_t launch_gemm(const GemmArgs& p, hipStream_t s) {
    const int split = (CM == 0 && p.ksplit > 1 && p.part != nullptr) ? p.ksplit : 1;
    GemmArgs q = p;
    q.ksplit = split;
    const dim3 grid((p.M + TBM - 1) / TBM, (p.N + TBN - 1) / TBN, split);
    hipLaunchKernelGGL((gemm_kernel<AM, AF, BM, BF, CM, TBM, TBN, WM, WN, MINB>), grid,
                       dim3(64 * WM * WN), 0, s, q);
    if (split > 1) {
        const long MN = (long)p.M * p.N;
        hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)((MN / 4 + 255) / 256)), dim3(256),
                           0, s, p.part, split, MN, reinterpret_cast<const u16*>(p.res),
                           static_cast<float*>(p.c[0]));
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bwd(int which, const GemmArgs& p, hipStream_t s) {
    switch (which) {
        // Tile shapes measured at d_model = 1024, n = 8192 (8 + 4 heads of 128):
        // more waves per SIMD pay as long as each still holds a 64 x 64 or
        // 32 x 64 block.  dO and dW_o: 128 x 128 with eight waves (115 vs 130 µs
        // for both with four); dx and dW_in (float32 operand A): 128 x 256 with
        // sixteen (242 vs 350 µs with 128 x 128 and four).
        case GEMM_DO: return launch_gemm<OP_KC_RM, false, OP_IC_RM, false, 1, 128, 128, 2, 4, 2>(p, s);
        case GEMM_DWO: return launch_gemm<OP_IC_RM, false, OP_IC_HM, false, 0, 128, 128, 2, 4, 2>(p, s);
        case GEMM_DX: return launch_gemm<OP_KC_HM, true, OP_IC_RM, false, 0, 128, 256, 4, 4, 1>(p, s);
        case GEMM_DWIN: return launch_gemm<OP_IC_HM, true, OP_IC_RM, false, 0, 128, 256, 4, 4, 1>(p, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_norm_bwd(const void* x, int dtype, const float* inv_norm, const float* g1,
                           const float* g2, long rows, int d, float* dx, hipStream_t s) {
    const unsigned blocks = (unsigned)((rows + 3) / 4);
    if (dtype == 1)
        hipLaunchKernelGGL(norm_bwd_kernel<true>, dim3(blocks), dim3(256), 0, s, x, inv_norm, g1,
                           g2, rows, d, dx);
    else
        hipLaunchKernelGGL(norm_bwd_kernel<false>, dim3(blocks), dim3(256), 0, s, x, inv_norm, g1,
                           g2, rows, d, dx);
    return hipGetLastError();
}

}  // namespace rt
