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
    // key/value row stride in LDS (bf16): an odd multiple of 16 elements, so 8
    // consecutive rows start in disjoint bank groups
    static constexpr int LDX = DP + 16;
    static constexpr int KT = 64;                // keys per tile
    static constexpr int NS = DP / 32;
    static constexpr int NJ = D / 16;
    static constexpr int NWV = 8;                // waves per workgroup, 16 queries each
    static constexpr int NT = 64 * NWV;
    static constexpr int QT = 16 * NWV;          // queries per workgroup
    static constexpr int CPR = DP / 8;
    static constexpr int DCH = D / 8;
    static constexpr int KITEMS = KT * CPR;                // key row chunks per tile
    static constexpr int KPT = (KITEMS + NT - 1) / NT;     // ... per thread
    static constexpr int VITEMS = KT * DCH;                // value row chunks per tile
    static constexpr int VPT = (VITEMS + NT - 1) / NT;     // ... per thread
};

// Key/value tiles travel through registers: a tile's loads are issued two
// tiles ahead of its use and stored to LDS one tile ahead, so global-load
// latency overlaps two tiles of compute.
#define RT_LOAD_TILE(tk, tv, KT0)                                                           \
    do {                                                                                    \
        _Pragma("unroll") for (int it = 0; it < C::KPT; ++it) {                              \
            const int e = threadIdx.x + C::NT * it;                                         \
            const int r = e / C::CPR, ch = e % C::CPR;                                      \
            const int j = (C::KITEMS % C::NT == 0 || e < C::KITEMS) ? (KT0) + r : n;        \
            tk[it] = (j < n && 8 * ch < D)                                                  \
                         ? *reinterpret_cast<const uint4*>(kk + (base + j) * D + 8 * ch)   \
                         : zero_u4();                                                       \
        }                                                                                   \
        _Pragma("unroll") for (int it = 0; it < C::VPT; ++it) {                              \
            const int e = threadIdx.x + C::NT * it;                                         \
            const int r = e / C::DCH, ch = e % C::DCH;                                      \
            const int j = (C::VITEMS % C::NT == 0 || e < C::VITEMS) ? (KT0) + r : n;        \
            tv[it] = (j < n) ? *reinterpret_cast<const uint4*>(v + (base + j) * D + 8 * ch)\
                             : zero_u4();                                                   \
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
__global__ __launch_bounds__(512) void local_attn_bf16_kernel(const u16* __restrict__ q,
                                                              const u16* __restrict__ kk,
                                                              const u16* __restrict__ v, int n,
                                                              int window, float scale, int causal,
                                                              OutT* __restrict__ out) {
    using C = LocalCfg<D>;
    __shared__ __attribute__((aligned(16))) u16 lk[2][C::KT * C::LDX];
    __shared__ __attribute__((aligned(16))) u16 lv[2][C::KT * C::LDX];

    // consecutive query tiles of a head read overlapping key windows: keep
    // them on one XCD
    const int item = xcd_contiguous(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
    const int bh = item / gridDim.x;
    const int q0 = (item % gridDim.x) * C::QT;
    const long base = (long)bh * n;
    const int lane = lane_id(), wv = threadIdx.x >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const float sl2 = scale * 1.4426950408889634f;
    const int qb0 = q0 + 16 * wv;      // first query of this wave's block
    const int qi = qb0 + r16;          // this lane's query

    uint4 qreg[C::NS];
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
        const int d0 = 32 * s + 8 * g;
        qreg[s] = (qi < n && d0 < D) ? *reinterpret_cast<const uint4*>(q + (base + qi) * D + d0)
                                     : zero_u4();
    }
    // keys needed by the workgroup / by this wave's block; keys in [clo, chi]
    // are visible to every query of the block
    const int lo = max(0, q0 - window + 1);
    const int hi = causal ? min(n - 1, q0 + C::QT - 1) : min(n - 1, q0 + C::QT - 1 + window - 1);
    const int blo = qb0 - window + 1;
    const int bhi = causal ? qb0 + 15 : qb0 + 15 + window - 1;
    const int clo = qb0 + 15 - window + 1;
    const int chi = min(n - 1, causal ? qb0 : qb0 + window - 1);

    f32x4 o[C::NJ];
#pragma unroll
    for (int jb = 0; jb < C::NJ; ++jb) o[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, z = 0.f;

    // One tile of keys [KT0, KT0 + 64) from LDS buffer BUF against this wave's queries.
#define RT_COMPUTE_TILE(KT0, BUF)                                                            \
    do {                                                                                     \
        const int kt_ = (KT0);                                                               \
        if (kt_ + C::KT - 1 >= blo && kt_ <= bhi) {        /* tile meets this wave's band */ \
            const u16* LK = lk[BUF];                                                         \
            f32x4 sv[4];                                                                     \
            _Pragma("unroll") for (int kb = 0; kb < 4; ++kb) {                               \
                const int key0 = kt_ + 16 * kb;                                              \
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
                sv[kb] = acc * sl2;                                                          \
            }                                                                                \
            if (kt_ < clo || kt_ + C::KT - 1 > chi) { /* not inside every band: mask */      \
                _Pragma("unroll") for (int kb = 0; kb < 4; ++kb)                             \
                    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                          \
                        const int j = kt_ + 16 * kb + 4 * g + i;                             \
                        const bool ok = j < n && j > qi - window &&                          \
                                        (causal ? j <= qi : j < qi + window);                \
                        sv[kb][i] = ok ? sv[kb][i] : -INFINITY;                              \
                    }                                                                        \
            }                                                                                \
            const int halves = ((kt_ + 31 >= blo && kt_ <= bhi) ? 1 : 0) |                   \
                               ((kt_ + 63 >= blo && kt_ + 32 <= bhi) ? 2 : 0);               \
            softmax_pv_chunk<C::NJ, C::LDX>(sv, m, z, o, lv[BUF], r16, g, halves);           \
        }                                                                                    \
    } while (0)

    const int kt_first = lo & ~(C::KT - 1);
    uint4 tka[C::KPT], tva[C::VPT], tkb[C::KPT], tvb[C::VPT];
    RT_LOAD_TILE(tka, tva, kt_first);
    if (kt_first + C::KT <= hi) RT_LOAD_TILE(tkb, tvb, kt_first + C::KT);
    RT_STORE_TILE(lk[0], lv[0], tka, tva);
    __syncthreads();

    // Two tiles per trip so that the two register sets keep static names: on
    // entry the tile at kt is in LDS buffer 0 and the next one in set b.
    for (int kt = kt_first;; kt += 2 * C::KT) {
        if (kt + 2 * C::KT <= hi) RT_LOAD_TILE(tka, tva, kt + 2 * C::KT);
        RT_COMPUTE_TILE(kt, 0);
        if (kt + C::KT > hi) break;
        RT_STORE_TILE(lk[1], lv[1], tkb, tvb);
        __syncthreads();
        if (kt + 3 * C::KT <= hi) RT_LOAD_TILE(tkb, tvb, kt + 3 * C::KT);
        RT_COMPUTE_TILE(kt + C::KT, 1);
        if (kt + 2 * C::KT > hi) break;
        RT_STORE_TILE(lk[0], lv[0], tka, tva);
        __syncthreads();
    }
#undef RT_COMPUTE_TILE

    const float zt = xor_sum_16_32(z);
    const float rz = 1.0f / zt;
    if (qi < n) {
        OutT* dst = out + (base + qi) * D + 4 * g;
#pragma unroll
        for (int jb = 0; jb < C::NJ; ++jb)
            store4<OutT>(dst + 16 * jb, o[jb][0] * rz, o[jb][1] * rz, o[jb][2] * rz, o[jb][3] * rz);
    }
}

// float32 inputs: one wave per query, 64-key chunks, online softmax.
template <int D, typename OutT>
__global__ __launch_bounds__(64) void local_attn_f32_kernel(const float* __restrict__ q,
                                                            const float* __restrict__ kk,
                                                            const float* __restrict__ v, int n,
                                                            int window, float scale, int causal,
                                                            OutT* __restrict__ out) {
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
        if (e < D) Elem<OutT>::store(out, (base + i) * D + e, acc[u] / z);
    }
}

template <int D, typename OutT>
void launch_local_d(const void* q, const void* kk, const void* v, int dtype, int BH, int n,
                    int window, float scale, int causal, void* out, hipStream_t s) {
    if (dtype == 1)
        hipLaunchKernelGGL((local_attn_bf16_kernel<D, OutT>),
                           dim3((n + LocalCfg<D>::QT - 1) / LocalCfg<D>::QT, BH),
                           dim3(LocalCfg<D>::NT), 0, s,
                           (const u16*)q, (const u16*)kk, (const u16*)v, n, window, scale, causal,
                           (OutT*)out);
    else
        hipLaunchKernelGGL((local_attn_f32_kernel<D, OutT>), dim3(n, BH), dim3(64), 0, s,
                           (const float*)q, (const float*)kk, (const float*)v, n, window, scale,
                           causal, (OutT*)out);
}

template <typename OutT>
void launch_local_outt(const void* q, const void* kk, const void* v, int dtype, int BH, int n,
                       int d, int window, float scale, int causal, void* out, hipStream_t s) {
    switch (d) {
        case 16: launch_local_d<16, OutT>(q, kk, v, dtype, BH, n, window, scale, causal, out, s); break;
        case 32: launch_local_d<32, OutT>(q, kk, v, dtype, BH, n, window, scale, causal, out, s); break;
        case 64: launch_local_d<64, OutT>(q, kk, v, dtype, BH, n, window, scale, causal, out, s); break;
        default: launch_local_d<128, OutT>(q, kk, v, dtype, BH, n, window, scale, causal, out, s); break;
    }
}

}  // namespace

hipError_t launch_local_attn(const void* q, const void* kk, const void* v, int dtype, int BH,
                             int n, int d, int window, float scale, int causal, void* out,
                             int out_dtype, hipStream_t s) {
    if (out_dtype == 1)
        launch_local_outt<u16>(q, kk, v, dtype, BH, n, d, window, scale, causal, out, s);
    else
        launch_local_outt<float>(q, kk, v, dtype, BH, n, d, window, scale, causal, out, s);
    return hipGetLastError();
}

}  // namespace rt
