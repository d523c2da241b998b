// local_attn.hip -- sliding-window attention for the non-routed heads (gfx950).
//
// The arXiv abstract and §6 of the paperlayer.ai summary of "Efficient
// Content-Based Sparse Attention with Routing Transformers" pair routing
// heads with local attention over a window of recent positions (windows of
// 512 and 1024 are the ones reported).  Position i attends, with ordinary
// softmax attention, to positions [i - window + 1, i] (causal) or to the band
// |i - j| < window (non-causal).  The blocked variant (lookback >= 0, causal):
// the sequence is cut into blocks of `window` positions and position i sees
// the positions of its own block and of the `lookback` blocks before it, not
// later than i; only the band's lower edge differs.
//
// local_attn_bf16_kernel: one workgroup = 128 queries in 8 blocks of 16 (64
// queries in 4 blocks at d <= 64), each block served by two waves: key/value tiles of 64 rows are staged
// row-major in LDS, and of every tile one wave of a pair takes the first 32
// keys, the other the last 32.  Each computes S^T = K Q^T and O^T = V^T P^T
// with v_mfma_f32_16x16x32_bf16 (the transposed value operand read straight
// from the row-major tile) and an online softmax over its keys; at the end the
// two partial softmax states of a block are merged through LDS.  Splitting the
// keys halves each wave's serial chain and doubles the waves per SIMD.  Key
// blocks outside a block's band are skipped.  A wave raises its priority
// while it issues a block of matrix products, so that its products go out
// back to back while the other waves of its SIMD do vector work.
#include "rt_common.hpp"
#include "rt_internal.hpp"

namespace rt {
namespace {

// softmax_pv_half on unscaled logits: the scale enters as one fma with the
// reference, exp2(s * sl2 - m), and the chunk maximum is scaled once (sl2 > 0).
// The fma does not round s * sl2 while m is the rounded product, so for the
// maximum the argument is the rounding error of m: harmless while |m| is
// moderate, but up to half an ulp of m (beyond the exponent range once |m|
// passes ~2^24).  Waves whose reference is that large take the rounded
// product first, as m was formed.
template <int NJ, int LDX>
__device__ __forceinline__ void softmax_pv_half_unscaled(f32x4 (&sv)[2], float sl2, float& m,
                                                         f32x4& zacc, f32x4 (&o)[NJ],
                                                         const u16* lv, int r16, int g) {
    const float r1 = max3_logits(sv[0][0], sv[0][1], sv[0][2]);
    const float r2 = max3_logits(sv[0][3], sv[1][0], sv[1][1]);
    const float lmax = sl2 * max3_logits(max3_logits(sv[1][2], sv[1][3], r1), r2, r2);
    lazy_rescale<NJ>(lmax, m, zacc, o);
    const float nm = (m == -INFINITY) ? 0.f : -m;
    uint32_t pw[2][2];
    if (__ballot(fabsf(m) > 4096.f) == 0ull) {   // wave-uniform
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            pw[kb][0] = cvt_pk_bf16(__builtin_amdgcn_exp2f(fmaf(sv[kb][0], sl2, nm)),
                                    __builtin_amdgcn_exp2f(fmaf(sv[kb][1], sl2, nm)));
            pw[kb][1] = cvt_pk_bf16(__builtin_amdgcn_exp2f(fmaf(sv[kb][2], sl2, nm)),
                                    __builtin_amdgcn_exp2f(fmaf(sv[kb][3], sl2, nm)));
        }
    } else {
#pragma clang fp contract(off)   // round the product, as m was rounded
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            pw[kb][0] = cvt_pk_bf16(__builtin_amdgcn_exp2f(sv[kb][0] * sl2 + nm),
                                    __builtin_amdgcn_exp2f(sv[kb][1] * sl2 + nm));
            pw[kb][1] = cvt_pk_bf16(__builtin_amdgcn_exp2f(sv[kb][2] * sl2 + nm),
                                    __builtin_amdgcn_exp2f(sv[kb][3] * sl2 + nm));
        }
    }
    const bf16x8 pbv = as_bf16x8(make_uint4(pw[0][0], pw[0][1], pw[1][0], pw[1][1]));
    const u16* vb = lv + (4 * g + (r16 >> 2)) * LDX + 4 * (r16 & 3);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) {
        const uint2 lo = lds_read_tr16(vb + 16 * jb);
        const uint2 hi = lds_read_tr16(vb + 16 * LDX + 16 * jb);
        o[jb] = mfma16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pbv, o[jb]);
    }
    zacc = mfma16(bf16_ones(), pbv, zacc);
    __builtin_amdgcn_s_setprio(0);
}

template <int D>
struct LocalCfg {
    static constexpr int DP = D < 32 ? 32 : D;
    // key/value row stride in LDS (bf16): an odd multiple of 16 elements, so 8
    // consecutive rows start in disjoint bank groups
    static constexpr int LDX = DP + 16;
    static constexpr int KT = 64;                // keys per tile
    static constexpr int NS = DP / 32;
    static constexpr int NJ = D / 16;
    // 16-query blocks per workgroup: eight (1024 threads) at d = 128, four at
    // d <= 64, where a workgroup's 79 VGPRs a lane let 24 waves share a CU in
    // 512-thread workgroups but only 16 in 1024-thread ones (window 256, 32K
    // tokens: 72 -> 53 us; at d = 128 four blocks spill and run slower)
    static constexpr int NQB = D <= 64 ? 4 : 8;
    static constexpr int NWV = 2 * NQB;          // two waves per block (key halves)
    static constexpr int NT = 64 * NWV;
    static constexpr int QT = 16 * NQB;          // queries per workgroup
    static constexpr int CPR = DP / 8;
    static constexpr int DCH = D / 8;
    static constexpr int KITEMS = KT * CPR;                // key row chunks per tile
    static constexpr int KPT = (KITEMS + NT - 1) / NT;     // ... per thread
    static constexpr int VITEMS = KT * DCH;                // value row chunks per tile
    static constexpr int VPT = (VITEMS + NT - 1) / NT;     // ... per thread
};

// Key/value tiles travel through registers: a tile's loads are issued two
// tiles ahead of its use and stored to LDS one tile ahead, so global-load
// latency overlaps two tiles of compute.  The loads are range-checked buffer
// loads (rows past the end read as zeros), issued unconditionally: the number
// in flight is fixed, so a store waits only for its own tile.
#define RT_LOAD_TILE(tk, tv, KT0)                                                           \
    do {                                                                                    \
        _Pragma("unroll") for (int it = 0; it < C::KPT; ++it) {                              \
            const int e = threadIdx.x + C::NT * it;                                         \
            const int r = e / C::CPR, ch = e % C::CPR;                                      \
            const bool in = (C::KITEMS % C::NT == 0 || e < C::KITEMS) && 8 * ch < D;        \
            tk[it] = buffer_load16(krs, in ? (uint32_t)(((KT0) + r) * D + 8 * ch) * 2u      \
                                           : kOutOfRange);                                  \
        }                                                                                   \
        _Pragma("unroll") for (int it = 0; it < C::VPT; ++it) {                              \
            const int e = threadIdx.x + C::NT * it;                                         \
            const int r = e / C::DCH, ch = e % C::DCH;                                      \
            const bool in = C::VITEMS % C::NT == 0 || e < C::VITEMS;                        \
            tv[it] = buffer_load16(vrs, in ? (uint32_t)(((KT0) + r) * D + 8 * ch) * 2u      \
                                           : kOutOfRange);                                  \
        }                                                                                   \
    } while (0)

#define RT_STORE_TILE(LK, LV, tk, tv)                                                       \
    do {                                                                                    \
        _Pragma("unroll") for (int it = 0; it < C::KPT; ++it) {                              \
            const int e = threadIdx.x + C::NT * it;                                         \
            if (C::KITEMS % C::NT == 0 || e < C::KITEMS)                                    \
                *reinterpret_cast<uint4*>(&(LK)[(e / C::CPR) * C::LDX + 8 * (e % C::CPR)]) = tk[it]; \
        }                                                                                   \
        _Pragma("unroll") for (int it = 0; it < C::VPT; ++it) {                              \
            const int e = threadIdx.x + C::NT * it;                                         \
            if (C::VITEMS % C::NT == 0 || e < C::VITEMS)                                    \
                *reinterpret_cast<uint4*>(&(LV)[(e / C::DCH) * C::LDX + 8 * (e % C::DCH)]) = tv[it]; \
        }                                                                                   \
    } while (0)

template <int D, typename OutT>
__global__ __launch_bounds__(1024) void local_attn_bf16_kernel(const u16* __restrict__ q,
                                                              const u16* __restrict__ kk,
                                                              const u16* __restrict__ v, int n,
                                                              int window, int lookback,
                                                              float scale, int causal,
                                                              OutT* __restrict__ out,
                                                              float* __restrict__ lse) {
    using C = LocalCfg<D>;
    __shared__ __attribute__((aligned(16))) u16 lk[2][C::KT * C::LDX];
    __shared__ __attribute__((aligned(16))) u16 lv[2][C::KT * C::LDX];

    // consecutive query tiles of a head read overlapping key windows: keep
    // them on one XCD
    const int item = xcd_contiguous(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
    const int bh = item / gridDim.x;
    const int q0 = (item % gridDim.x) * C::QT;
    const long base = (long)bh * n;
    const int lane = lane_id(), wv = wave_id();
    const int g = lane >> 4, r16 = lane & 15;
    // log2-unit scale, kept positive: a negative scale negates the queries
    // instead, and a zero scale becomes one too small to change any logit
    const float sl2s = scale * 1.4426950408889634f;
    const float sl2 = sl2s > 0.f ? sl2s : (sl2s < 0.f ? -sl2s : 1e-30f);
    const uint32_t qflip = sl2s < 0.f ? 0x80008000u : 0u;
    const int hf = wv / C::NQB;                  // key half of every tile: [32 hf, 32 hf + 32)
    const int qb0 = q0 + 16 * (wv % C::NQB);    // first query of this wave's block
    const int qi = qb0 + r16;                    // this lane's query

    uint4 qreg[C::NS];
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
        const int d0 = 32 * s + 8 * g;
        qreg[s] = (qi < n && d0 < D) ? *reinterpret_cast<const uint4*>(q + (base + qi) * D + d0)
                                     : zero_u4();
        qreg[s].x ^= qflip;
        qreg[s].y ^= qflip;
        qreg[s].z ^= qflip;
        qreg[s].w ^= qflip;
    }
    // keys needed by the workgroup / by this wave's block; keys in [clo, chi]
    // are visible to every query of the block
    // first key of position i's band (non-decreasing in i)
    auto band_lo = [&](int i) {
        return lookback < 0 ? i - window + 1 : max(0, (i / window - lookback) * window);
    };
    const int qlo = band_lo(qi);
    // this lane's visible keys as one unsigned range: key j is visible iff
    // (unsigned)(j - qlo_m) <= qspan (an empty band masks every key)
    const int qhi = min(n - 1, causal ? qi : qi + window - 1);
    const int qlo_m = qhi >= qlo ? qlo : -0x40000000;
    const uint32_t qspan = qhi >= qlo ? (uint32_t)(qhi - qlo) : 0u;
    const int lo = max(0, band_lo(q0));
    const int hi = causal ? min(n - 1, q0 + C::QT - 1) : min(n - 1, q0 + C::QT - 1 + window - 1);
    const int blo = band_lo(qb0);
    const int bhi = causal ? qb0 + 15 : qb0 + 15 + window - 1;
    const int clo = band_lo(qb0 + 15);
    const int chi = min(n - 1, causal ? qb0 : qb0 + window - 1);

    f32x4 o[C::NJ];
#pragma unroll
    for (int jb = 0; jb < C::NJ; ++jb) o[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;
    f32x4 zacc = {0.f, 0.f, 0.f, 0.f};   // the denominator (every element holds it)

    // This wave's half of tile [KT0, KT0 + 64) from LDS buffer BUF.
#define RT_COMPUTE_TILE(KT0, BUF)                                                            \
    do {                                                                                     \
        const int kh_ = (KT0) + 32 * hf;                   /* first key of the half */       \
        if (kh_ + 31 >= blo && kh_ <= bhi) {               /* half meets the band */         \
            const u16* LK = lk[BUF] + 32 * hf * C::LDX;                                      \
            f32x4 sv[2];                                                                     \
            __builtin_amdgcn_s_setprio(1);     /* products first, see the header */          \
            _Pragma("unroll") for (int kb = 0; kb < 2; ++kb) {                               \
                const int key0 = kh_ + 16 * kb;                                              \
                if (key0 + 15 < blo || key0 > bhi || key0 >= n) {                            \
                    sv[kb] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};              \
                    continue;                                                                \
                }                                                                            \
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};                                            \
                _Pragma("unroll") for (int s = 0; s < C::NS; ++s) {                          \
                    const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(              \
                        &LK[(16 * kb + r16) * C::LDX + 32 * s + 8 * g]));                    \
                    acc = mfma16(a, as_bf16x8(qreg[s]), acc);                                \
                }                                                                            \
                sv[kb] = acc;                          /* unscaled: sl2 enters in exp2 */  \
            }                                                                                \
            __builtin_amdgcn_s_setprio(0);                                                   \
            if (kh_ < clo || kh_ + 31 > chi) {     /* not inside every band: mask */         \
                const uint32_t rel0 = (uint32_t)(kh_ + 4 * g - qlo_m);                       \
                _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                             \
                    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                          \
                        const bool ok = rel0 + (uint32_t)(16 * kb + i) <= qspan;             \
                        sv[kb][i] = ok ? sv[kb][i] : -INFINITY;                              \
                    }                                                                        \
            }                                                                                \
            softmax_pv_half_unscaled<C::NJ, C::LDX>(sv, sl2, m, zacc, o,                      \
                                                   lv[BUF] + 32 * hf * C::LDX, r16, g);      \
        }                                                                                    \
    } while (0)

    const int kt_first = lo & ~(C::KT - 1);
    uint4 tka[C::KPT], tva[C::VPT], tkb[C::KPT], tvb[C::VPT];
    // this head's keys and values as range-checked buffers
    const buf_rsrc krs = make_rsrc(kk + base * D, (uint32_t)n * D * 2u);
    const buf_rsrc vrs = make_rsrc(v + base * D, (uint32_t)n * D * 2u);
    RT_LOAD_TILE(tka, tva, kt_first);
    RT_LOAD_TILE(tkb, tvb, kt_first + C::KT);
    RT_STORE_TILE(lk[0], lv[0], tka, tva);
    __syncthreads();

    // Two tiles per trip so that the two register sets keep static names: on
    // entry the tile at kt is in LDS buffer 0 and the next one in set b.
    for (int kt = kt_first;; kt += 2 * C::KT) {
        RT_LOAD_TILE(tka, tva, kt + 2 * C::KT);
        RT_COMPUTE_TILE(kt, 0);
        if (kt + C::KT > hi) break;
        RT_STORE_TILE(lk[1], lv[1], tkb, tvb);
        __syncthreads();
        RT_LOAD_TILE(tkb, tvb, kt + 3 * C::KT);
        RT_COMPUTE_TILE(kt + C::KT, 1);
        if (kt + 2 * C::KT > hi) break;
        RT_STORE_TILE(lk[0], lv[0], tka, tva);
        __syncthreads();
    }
#undef RT_COMPUTE_TILE

    // Merge the two key halves of each block: the second wave of a pair hands
    // its softmax state (max, partial denominator, accumulators) to the first
    // through LDS, reusing the tile buffers.
    constexpr int MS = 2 + 4 * C::NJ;            // floats per lane
    static_assert(C::NQB * 64 * MS * 4 <= (int)sizeof(lk) + (int)sizeof(lv), "merge area");
    float* lmerge = reinterpret_cast<float*>(&lk[0][0]);
    __syncthreads();                             // every wave is done with the tiles
    float* mine = lmerge + ((wv % C::NQB) * 64 + lane) * MS;
    if (hf == 1) {
        mine[0] = m;
        mine[1] = zacc[0];
#pragma unroll
        for (int jb = 0; jb < C::NJ; ++jb)
            *reinterpret_cast<float4*>(mine + 2 + 4 * jb) =
                make_float4(o[jb][0], o[jb][1], o[jb][2], o[jb][3]);
    }
    __syncthreads();
    if (hf == 0) {
        const float m2 = mine[0], z2 = mine[1];
        const float mt = fmaxf(m, m2);
        const float ms = (mt == -INFINITY) ? 0.f : mt;
        const float a1 = __builtin_amdgcn_exp2f(m - ms), a2 = __builtin_amdgcn_exp2f(m2 - ms);
        const float zt = zacc[0] * a1 + z2 * a2;
        const float rz = 1.0f / zt;
        if (qi < n) {
            if (lse != nullptr && g == 0)            // natural log of the denominator
                lse[base + qi] = (ms + __log2f(zt)) * 0.6931471805599453f;
            OutT* dst = out + (base + qi) * D + 4 * g;
#pragma unroll
            for (int jb = 0; jb < C::NJ; ++jb) {
                const float4 o2 = *reinterpret_cast<const float4*>(mine + 2 + 4 * jb);
                store4<OutT>(dst + 16 * jb, (o[jb][0] * a1 + o2.x * a2) * rz,
                             (o[jb][1] * a1 + o2.y * a2) * rz, (o[jb][2] * a1 + o2.z * a2) * rz,
                             (o[jb][3] * a1 + o2.w * a2) * rz);
            }
        }
    }
}

// float32 inputs: one wave per query, 64-key chunks, online softmax.
template <int D, typename OutT>
__global__ __launch_bounds__(64) void local_attn_f32_kernel(const float* __restrict__ q,
                                                            const float* __restrict__ kk,
                                                            const float* __restrict__ v, int n,
                                                            int window, int lookback,
                                                            float scale, int causal,
                                                            OutT* __restrict__ out,
                                                            float* __restrict__ lse) {
    __shared__ float lq[D];
    __shared__ float lp[64];
    const int i = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
    const long base = (long)bh * n;
    for (int e = lane; e < D; e += 64) lq[e] = q[(base + i) * D + e];
    __syncthreads();
    const int lo = lookback < 0 ? max(0, i - window + 1) : max(0, (i / window - lookback) * window);
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
        if (e < D) Elem<OutT>::store(out, (base + i) * D + e, acc[u] / z);
    }
    if (lse != nullptr && lane == 0) lse[base + i] = m + logf(z);
}

template <int D, typename OutT>
void launch_local_d(const void* q, const void* kk, const void* v, int dtype, int BH, int n,
                    int window, int lookback, float scale, int causal, void* out, float* lse,
                    hipStream_t s) {
    if (dtype == 1)
        hipLaunchKernelGGL((local_attn_bf16_kernel<D, OutT>),
                           dim3((n + LocalCfg<D>::QT - 1) / LocalCfg<D>::QT, BH),
                           dim3(LocalCfg<D>::NT), 0, s,
                           (const u16*)q, (const u16*)kk, (const u16*)v, n, window, lookback,
                           scale, causal, (OutT*)out, lse);
    else
        hipLaunchKernelGGL((local_attn_f32_kernel<D, OutT>), dim3(n, BH), dim3(64), 0, s,
                           (const float*)q, (const float*)kk, (const float*)v, n, window, lookback,
                           scale, causal, (OutT*)out, lse);
}

template <typename OutT>
void launch_local_outt(const void* q, const void* kk, const void* v, int dtype, int BH, int n,
                       int d, int window, int lookback, float scale, int causal, void* out,
                       float* lse, hipStream_t s) {
    switch (d) {
        case 16: launch_local_d<16, OutT>(q, kk, v, dtype, BH, n, window, lookback, scale, causal, out, lse, s); break;
        case 32: launch_local_d<32, OutT>(q, kk, v, dtype, BH, n, window, lookback, scale, causal, out, lse, s); break;
        case 64: launch_local_d<64, OutT>(q, kk, v, dtype, BH, n, window, lookback, scale, causal, out, lse, s); break;
        default: launch_local_d<128, OutT>(q, kk, v, dtype, BH, n, window, lookback, scale, causal, out, lse, s); break;
    }
}

}  // namespace

hipError_t launch_local_attn(const void* q, const void* kk, const void* v, int dtype, int BH,
                             int n, int d, int window, int lookback, float scale, int causal,
                             void* out, int out_dtype, float* lse, hipStream_t s) {
    if (out_dtype == 1)
        launch_local_outt<u16>(q, kk, v, dtype, BH, n, d, window, lookback, scale, causal, out,
                               lse, s);
    else
        launch_local_outt<float>(q, kk, v, dtype, BH, n, d, window, lookback, scale, causal, out,
                                 lse, s);
    return hipGetLastError();
}

}  // namespace rt
