// route.hip -- routing: unit normalisation, centroid scores and balanced
// top-w selection (gfx950).
//
// Routing attention (paperlayer.ai summary of "Efficient Content-Based Sparse
// Attention with Routing Transformers", §4 "Routing attention with
// clustering"): queries/keys are unit-normalised and compared with k shared
// centroids (the O(nkd) routing comparisons); with balanced clusters every
// centroid holds the same number w of tokens, the top-w assignment costing
// far less than the attention itself.
//
// Kernels
//   score_bf16_kernel  one workgroup = 256 tokens x all centroids of a head.
//                      The raw bf16 token rows are the B operand of
//                      v_mfma_f32_16x16x32_bf16 straight from HBM; the fp32
//                      centroids are split into three bf16 terms in LDS
//                      (mu = hi + mid + lo, exact), so three MFMA passes give
//                      float32-accurate inner products.  Scores are scaled by
//                      the token's inverse norm in fp32 afterwards.
//   score_f32_kernel   the same on the vector ALUs for float32 inputs.
//   topw_kernel        one workgroup per (batch, head, centroid) row of n
//                      scores (a single wave for short rows when there are
//                      enough of them): an exact radix select of the w-th
//                      largest order-preserving key (8-bit digits, histograms
//                      in LDS, mostly over short lists of the candidates),
//                      then a position-ordered compaction with wave ballots,
//                      so the w members come out sorted by position with ties
//                      taken at the lowest positions.
//   part_group_kernel, part_rank_kernel, part_emit_kernel
//                      partition-style routing (every token in one cluster):
//                      group by nearest centroid, rank inside the group,
//                      list each cluster by position.
#include <type_traits>

#include "rt_common.hpp"
#include "rt_internal.hpp"

namespace rt {
namespace {

// rows up to this many tokens keep all their keys in registers in topw_kernel
constexpr int kTopwRegisterRow = 8192;
// rows of up to 1024 keys take one wave each from this many rows on (one per
// SIMD of the 256 CUs)
constexpr int kTopwOneWaveRows = 1024;

template <int D>
struct ScoreCfg {
    static constexpr int DP = D < 32 ? 32 : D;         // dims padded to the MFMA k-depth
    static constexpr int KC = (D == 128) ? 64 : 128;   // centroids per LDS chunk
    static constexpr int LD = DP + 8;                  // LDS row stride (bf16), 16 B aligned
    static constexpr int NS = DP / 32;                 // MFMA k-steps per token row
    static constexpr int NT = 512;                     // threads per workgroup (8 waves)
    static constexpr int TOK = 32 * NT / 64;           // tokens per workgroup (32 per wave)
};

// ARGMAX: instead of the scores, each token's nearest centroid (largest score,
// ties to the lower index) and that score go to label[] and best[].
template <int D, bool ARGMAX>
__global__ __launch_bounds__(ScoreCfg<D>::NT) void score_bf16_kernel(const u16* __restrict__ qk,
                                                         const float* __restrict__ mu, int H,
                                                         int n, int k,
                                                         float* __restrict__ inv_norm,
                                                         float* __restrict__ scores,
                                                         u16* __restrict__ qk_hat,
                                                         uint32_t* __restrict__ mask, int KW,
                                                         int32_t* __restrict__ label,
                                                         float* __restrict__ best) {
    using C = ScoreCfg<D>;
    __shared__ __attribute__((aligned(16))) u16 lmu[3][C::KC][C::LD];

    // the token tiles of one head share its centroids: keep them on one XCD
    const int item = xcd_contiguous(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
    const int bh = item / gridDim.x, tile = item % gridDim.x;
    const int h = bh % H;
    const int lane = lane_id(), wv = wave_id();
    const int g = lane >> 4, r16 = lane & 15;
    const long base = (long)bh * n;

    // Centroids of the first chunk: request them before the token rows so the
    // two latencies overlap.  Each thread takes MG groups of 8 consecutive
    // dims (two 16-byte loads) and stores each of the three bf16 terms of a
    // group with one 16-byte LDS write.
    constexpr int GPR = C::DP / 8;                   // 8-dim groups per centroid row
    constexpr int MG = (C::KC * GPR) / C::NT;        // groups per thread
    // Loads go through buffer resources (offsets out of range read zeros), so
    // none sits under a branch and the waits for them stay exact.
    const buf_rsrc mrs = make_rsrc(mu + (long)h * k * D, 4u * (uint32_t)k * D);
    float4 mreg[MG][2];
    auto load_mu = [&](int c0) {
#pragma unroll
        for (int j = 0; j < MG; ++j) {
            const int e = threadIdx.x + C::NT * j;
            const int c = e / GPR, dim0 = 8 * (e % GPR);
            const bool ok = c0 + c < k && dim0 < D;
            const uint32_t off = ok ? 4u * (uint32_t)((c0 + c) * D + dim0) : kOutOfRange;
            mreg[j][0] = __builtin_bit_cast(float4, buffer_load16(mrs, off));
            mreg[j][1] = __builtin_bit_cast(float4, buffer_load16(mrs, ok ? off + 16u : kOutOfRange));
        }
    };
    auto stage_mu = [&]() {
#pragma unroll
        for (int j = 0; j < MG; ++j) {
            const int e = threadIdx.x + C::NT * j;
            const int c = e / GPR, dim0 = 8 * (e % GPR);
            const float m8[8] = {mreg[j][0].x, mreg[j][0].y, mreg[j][0].z, mreg[j][0].w,
                                 mreg[j][1].x, mreg[j][1].y, mreg[j][1].z, mreg[j][1].w};
            uint32_t hw[4], mw[4], lw[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // mu = hi + mid + lo exactly: each term is the bf16 rounding of
                // what the previous ones leave
                const float a = m8[2 * q], b = m8[2 * q + 1];
                hw[q] = cvt_pk_bf16(a, b);
                const float ra = a - __uint_as_float(hw[q] << 16);
                const float rb = b - __uint_as_float(hw[q] & 0xffff0000u);
                mw[q] = cvt_pk_bf16(ra, rb);
                lw[q] = cvt_pk_bf16(ra - __uint_as_float(mw[q] << 16),
                                    rb - __uint_as_float(mw[q] & 0xffff0000u));
            }
            *reinterpret_cast<uint4*>(&lmu[0][c][dim0]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            *reinterpret_cast<uint4*>(&lmu[1][c][dim0]) = make_uint4(mw[0], mw[1], mw[2], mw[3]);
            *reinterpret_cast<uint4*>(&lmu[2][c][dim0]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        }
    };
    load_mu(0);

    const buf_rsrc xrs = make_rsrc(qk + base * D, 2u * (uint32_t)n * D);
    uint4 breg[2][C::NS];
    float inv[2];
    int tok[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int t = tile * C::TOK + wv * 32 + tb * 16 + r16;
        tok[tb] = t;
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
            const int d0 = 32 * s + 8 * g;
            breg[tb][s] = buffer_load16(xrs, t < n && d0 < D ? 2u * (uint32_t)(t * D + d0) : kOutOfRange);
        }
    }
    stage_mu();
    // every wave's terms are in LDS; the barrier comes before any wave waits
    // for its token rows, so that a wave starts its products once its own rows
    // are in, not once every wave's are (nothing that reads them is moved
    // above it)
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int t = tok[tb];
        float ss = 0.f;
#pragma unroll
        for (int s = 0; s < C::NS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = u4_elem(breg[tb][s], e);
                ss = fmaf(x, x, ss);
            }
        ss = xor_sum_16_32(ss);
        inv[tb] = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
        if (g == 0 && t < n) {
            inv_norm[base + t] = inv[tb];
            if (mask != nullptr)
                for (int i = 0; i < KW; ++i) mask[(base + t) * KW + i] = 0u;
        }
        if (qk_hat != nullptr && t < n) {
#pragma unroll
            for (int s = 0; s < C::NS; ++s) {
                const int d0 = 32 * s + 8 * g;
                if (d0 < D) {
                    uint4 o;
                    uint32_t* ow = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        ow[e] = cvt_pk_bf16(u4_elem(breg[tb][s], 2 * e) * inv[tb],
                                            u4_elem(breg[tb][s], 2 * e + 1) * inv[tb]);
                    *reinterpret_cast<uint4*>(qk_hat + (base + t) * D + d0) = o;
                }
            }
        }
    }

    float bs[2] = {-INFINITY, -INFINITY};   // ARGMAX: this lane's best score and centroid
    int bc[2] = {0, 0};
    for (int c0 = 0; c0 < k; c0 += C::KC) {
        if (c0 > 0) {
            __syncthreads();          // previous chunk's MFMAs are done with lmu
            load_mu(c0);
            stage_mu();
            __syncthreads();
        }
        const int cn = min(C::KC, k - c0);
        for (int cb = 0; cb * 16 < cn; ++cb) {
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 3; ++p) {
#pragma unroll
                for (int s = 0; s < C::NS; ++s) {
                    const bf16x8 a = as_bf16x8(
                        *reinterpret_cast<const uint4*>(&lmu[p][cb * 16 + r16][32 * s + 8 * g]));
                    acc0 = mfma16(a, as_bf16x8(breg[0][s]), acc0);
                    acc1 = mfma16(a, as_bf16x8(breg[1][s]), acc1);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = c0 + cb * 16 + 4 * g + i;
                if (c < k) {
                    const float s0 = acc0[i] * inv[0], s1 = acc1[i] * inv[1];
                    if constexpr (ARGMAX) {
                        // centroids arrive in ascending order for this lane
                        if (s0 > bs[0]) { bs[0] = s0; bc[0] = c; }
                        if (s1 > bs[1]) { bs[1] = s1; bc[1] = c; }
                    } else {
                        // Up to 8192 tokens the top-w selection reads every
                        // score once, in the next launch, after L2 has been
                        // written back and invalidated: the scores are
                        // streamed past it (kept dirty there they would only
                        // lengthen the write-back at the end of this launch).
                        // Longer rows re-read their candidates, and those
                        // re-reads find the scores written the ordinary way
                        // in the cache behind L2 (measured at n = 32768:
                        // streamed stores cost the route 13 us of 86).
                        float* row = scores + ((long)bh * k + c) * n;
                        if (n <= kTopwRegisterRow) {
                            if (tok[0] < n) __builtin_nontemporal_store(s0, &row[tok[0]]);
                            if (tok[1] < n) __builtin_nontemporal_store(s1, &row[tok[1]]);
                        } else {
                            if (tok[0] < n) row[tok[0]] = s0;
                            if (tok[1] < n) row[tok[1]] = s1;
                        }
                    }
                }
            }
        }
    }
    if constexpr (ARGMAX) {
        // the four lanes of a token (g = 0..3) hold disjoint centroids
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
            for (int off = 16; off <= 32; off <<= 1) {
                const float os = __shfl_xor(bs[tb], off);
                const int oc = __shfl_xor(bc[tb], off);
                if (os > bs[tb] || (os == bs[tb] && oc < bc[tb])) {
                    bs[tb] = os;
                    bc[tb] = oc;
                }
            }
            if (g == 0 && tok[tb] < n) {
                label[base + tok[tb]] = bc[tb];
                best[base + tok[tb]] = bs[tb];
            }
        }
    }
}

template <int D, bool ARGMAX>
__global__ __launch_bounds__(256) void score_f32_kernel(const float* __restrict__ qk,
                                                        const float* __restrict__ mu, int H, int n,
                                                        int k, float* __restrict__ inv_norm,
                                                        float* __restrict__ scores,
                                                        float* __restrict__ qk_hat,
                                                        uint32_t* __restrict__ mask, int KW,
                                                        int32_t* __restrict__ label,
                                                        float* __restrict__ best) {
    constexpr int KC = 8192 / D;  // 32 KB of centroids per chunk
    __shared__ float lmu[KC * D];
    const int bh = blockIdx.y, h = bh % H;
    const int t = blockIdx.x * 256 + threadIdx.x;
    const long base = (long)bh * n;
    float x[D];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) {
        x[i] = (t < n) ? qk[(base + t) * D + i] : 0.f;
        ss = fmaf(x[i], x[i], ss);
    }
    const float inv = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
    if (t < n) {
        inv_norm[base + t] = inv;
        if (mask != nullptr)
            for (int i = 0; i < KW; ++i) mask[(base + t) * KW + i] = 0u;
        if (qk_hat != nullptr)
            for (int i = 0; i < D; ++i) qk_hat[(base + t) * D + i] = x[i] * inv;
    }
    float bs = -INFINITY;
    int bc = 0;
    for (int c0 = 0; c0 < k; c0 += KC) {
        __syncthreads();
        const int cn = min(KC, k - c0);
        for (int e = threadIdx.x; e < cn * D; e += 256) lmu[e] = mu[((long)h * k + c0) * D + e];
        __syncthreads();
        if (t < n) {
            for (int c = 0; c < cn; ++c) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < D; ++i) acc = fmaf(x[i], lmu[c * D + i], acc);
                if constexpr (ARGMAX) {
                    if (acc * inv > bs) {
                        bs = acc * inv;
                        bc = c0 + c;
                    }
                } else {
                    scores[((long)bh * k + c0 + c) * n + t] = acc * inv;
                }
            }
        }
    }
    if constexpr (ARGMAX) {
        if (t < n) {
            label[base + t] = bc;
            best[base + t] = bs;
        }
    }
}

// Order-preserving map float -> uint32 (larger float, larger key); -0 and +0
// map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ uint32_t buffer_load4(buf_rsrc r, uint32_t byte_off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, 0);
}
#else
__device__ __forceinline__ uint32_t buffer_load4(buf_rsrc, uint32_t) { return 0u; }
#endif

// Wave reductions on the DPP network (no LDS traffic): partial results move
// along each row of 16 lanes, then across rows; the total lands in lane 63.
template <bool MAX>
__device__ __forceinline__ uint32_t dpp_step(uint32_t x, uint32_t y) {
    return MAX ? max(x, y) : x + y;
}
#define RT_DPP(x, ctrl, rmask) \
    (uint32_t) __builtin_amdgcn_update_dpp(0, (int)(x), ctrl, rmask, 0xf, true)
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t x) {
    x = dpp_step<MAX>(x, RT_DPP(x, 0x111, 0xf));   // row_shr:1
    x = dpp_step<MAX>(x, RT_DPP(x, 0x112, 0xf));   // row_shr:2
    x = dpp_step<MAX>(x, RT_DPP(x, 0x114, 0xf));   // row_shr:4
    x = dpp_step<MAX>(x, RT_DPP(x, 0x118, 0xf));   // row_shr:8
    x = dpp_step<MAX>(x, RT_DPP(x, 0x142, 0xa));   // row_bcast:15 into rows 1, 3
    x = dpp_step<MAX>(x, RT_DPP(x, 0x143, 0xc));   // row_bcast:31 into rows 2, 3
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
// The same over lanes 0..15 only.
template <bool MAX>
__device__ __forceinline__ uint32_t row16_reduce_u32(uint32_t x) {
    x = dpp_step<MAX>(x, RT_DPP(x, 0x111, 0xf));
    x = dpp_step<MAX>(x, RT_DPP(x, 0x112, 0xf));
    x = dpp_step<MAX>(x, RT_DPP(x, 0x114, 0xf));
    x = dpp_step<MAX>(x, RT_DPP(x, 0x118, 0xf));
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
}
#undef RT_DPP

// Inclusive prefix sum over the 64 lanes of a wave on the DPP network: a
// scan inside each row of 16 lanes, then the totals of the rows below added
// (read with readlane).  No LDS round trips.
__device__ __forceinline__ uint32_t wave_prefix_u32(uint32_t x, uint32_t& total) {
#define RT_DPP_SHR(v, n) (uint32_t) __builtin_amdgcn_update_dpp(0, (int)(v), 0x110 + (n), 0xf, 0xf, true)
    x += RT_DPP_SHR(x, 1);
    x += RT_DPP_SHR(x, 2);
    x += RT_DPP_SHR(x, 4);
    x += RT_DPP_SHR(x, 8);
#undef RT_DPP_SHR
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
    const int row = lane_id() >> 4;
    x += (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
    total = r0 + r1 + r2 + r3;
    return x;
}

// Each wave finds for itself, in a shared 256-bin histogram, the bin holding
// the `remaining`-th largest key: every lane gets the bin and the rank left
// inside it (no barrier needed after it).
// `remaining` must be between 1 and the histogram total.
__device__ __forceinline__ void find_bin_wave(const uint32_t* hist, uint32_t remaining,
                                              uint32_t& bin, uint32_t& rem) {
    const int lane = lane_id();
    const uint4 c4 = *reinterpret_cast<const uint4*>(hist + 4 * lane);
    const uint32_t cnt[4] = {c4.x, c4.y, c4.z, c4.w};
    const uint32_t tot = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    uint32_t all;
    const uint32_t incl = wave_prefix_u32(tot, all);
    uint32_t above = all - incl;   // keys in the bins of the lanes above this one
    int fb = -1;
    uint32_t fr = 0u;
#pragma unroll
    for (int b = 3; b >= 0; --b) {
        if (above < remaining && remaining <= above + cnt[b]) {
            fb = 4 * lane + b;
            fr = remaining - above;
        }
        above += cnt[b];
    }
    const uint64_t m = __ballot(fb >= 0);
    const int src = m ? __builtin_ctzll(m) : 0;
    bin = (uint32_t)__builtin_amdgcn_readlane(fb, src);
    rem = (uint32_t)__builtin_amdgcn_readlane((int)fr, src);
}

// Balanced top-w of one row of n scores; one workgroup per row.  Key j of
// lane l in wave v belongs to position v*64*KPT + 64*j + l, so that a wave's
// ballot over its key j is the membership bitmap of 64 consecutive positions.
//  1. Load the row as order-preserving keys (registers); each wave counts its
//     keys in its own four highest top bytes (sign and high exponent bits).
//  2. One exchange gives the row's counts of its four highest top bytes: the
//     top byte bin0 of the w-th largest key and its rank inside that byte.
//  3. Each wave lists its keys of top byte bin0 or above (fewer than w of
//     them above) with their positions, in position order: a few per cent of
//     the row.
//  4. Three 8-bit digit passes over the lists give the w-th largest key T and
//     how many keys equal to T belong to the top w.
//  5. The lists, read in position order, give the members: the keys above T
//     and, at the lowest positions, the keys equal to T.
// A row whose bin0 is not among its four highest top bytes, or whose lists
// overflow, finishes with the digit passes and the selection over all keys.
// Positions past the row hold key 0, below every key of a number: they rank
// last among equals and are never selected.
constexpr int kCandPerWave = 512;

// TOPB: only the keys' high halves stay in registers (two to a register, for
// 32 or 64 keys a lane).  The lists carry those halves; once the first digit
// pass over them has fixed the threshold's top 16 bits, the listed keys inside
// that 16-bit bucket (a few a wave) are re-read in full from the score row.
// The slow path re-reads every key it needs.
template <int NT, int KPT, bool TOPB>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8, 8))) void topw_kernel(const float* __restrict__ scores, int n, int w,
                                                  int32_t* __restrict__ idx, int k,
                                                  uint32_t* __restrict__ mask, int KW) {
    static_assert(NT % kWave == 0, "whole waves");
    // clears a 256-bin histogram (one bin a thread from 256 threads on)
    auto zero_hist = [&](uint32_t* h) {
#pragma unroll
        for (int i = 0; i < (256 + NT - 1) / NT; ++i)
            if (NT >= 256 ? threadIdx.x < 256 : true) h[threadIdx.x + NT * i] = 0u;
    };
    constexpr int NWV = NT / kWave;
    constexpr int CW = kCandPerWave;
    __shared__ __attribute__((aligned(16))) uint2 cand[NWV][CW];   // (key, position)
    __shared__ __attribute__((aligned(16))) uint32_t hist3[3][256];
    __shared__ __attribute__((aligned(16))) uint32_t wtop[NWV][8];  // per wave: highest top
                                         // byte, counts of it and the 3 below (padded)
    __shared__ uint32_t wcnt[NWV], wgt[NWV], weq[NWV];

    // the rows of one head on one XCD: the scoring kernel wrote that head's
    // scores from the same XCD
    const int row = xcd_contiguous(blockIdx.x, gridDim.x);
    const float* srow = scores + (long)row * n;
    const int lane = lane_id(), wv = wave_id();
    const int seg0 = wv * kWave * KPT;
    const int pl = seg0 + lane;   // position of key 0 of this lane; key j at pl + 64 j
    int32_t* out = idx + (long)row * w;
    const int bh = row / k, c = row - bh * k;
    uint32_t* mrow = mask == nullptr ? nullptr : mask + (long)bh * n * KW + (c >> 5);
    const uint32_t cbit = 1u << (c & 31);

    // 1. Keys.  Every load is issued unconditionally (a wave keeps them all in
    // flight); only a wave whose segment runs past the row checks positions.
    const buf_rsrc srs = make_rsrc(srow, 4u * (uint32_t)n);
    constexpr int NKR = TOPB ? (KPT + 1) / 2 : KPT;
    uint32_t key[NKR];   // the keys, or (TOPB) their high halves
    uint32_t mw = 0u;
    auto load = [&](auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int p = pl + kWave * j;
            const bool in = !TAIL || p < n;
            uint32_t kj =
                order_key(__uint_as_float(buffer_load4(srs, in ? 4u * (uint32_t)p : kOutOfRange)));
            kj = in ? kj : 0u;
            mw = max(mw, kj);
            if constexpr (TOPB) {
                if (j % 2 == 0) key[j / 2] = kj >> 16;
                else key[j / 2] |= kj & 0xffff0000u;
            } else {
                key[j] = kj;
            }
        }
    };
    if (seg0 + kWave * KPT <= n) load(std::false_type{});
    else load(std::true_type{});
    // (TOPB) key j with its low half zero
    auto hi16 = [&](int j) -> uint32_t {
        if constexpr (TOPB) return (j % 2 == 0) ? key[j / 2] << 16 : key[j / 2] & 0xffff0000u;
        else return key[j] & 0xffff0000u;
    };
    auto top8 = [&](int j) -> uint32_t { return hi16(j) >> 24; };
    mw = wave_reduce_u32<true>(mw) >> 24;
    // 7-bit counters of the top bytes mw, mw-1, mw-2, mw-3 (bits 28.. take the
    // rest and may wrap); a lane holds at most 64 keys
    uint32_t cf = 0u;
    const uint32_t mw7 = 7u * mw;
#pragma unroll
    for (int j = 0; j < KPT; ++j) cf += 1u << min(mw7 - 7u * top8(j), 28u);
    uint32_t c01 = (cf & 0x7fu) | (((cf >> 7) & 0x7fu) << 16);
    uint32_t c23 = ((cf >> 14) & 0x7fu) | (((cf >> 21) & 0x7fu) << 16);
    c01 = wave_reduce_u32<false>(c01);
    c23 = wave_reduce_u32<false>(c23);
    if (lane == 0) {
        wtop[wv][0] = mw;
        wtop[wv][1] = c01 & 0xffffu;
        wtop[wv][2] = c01 >> 16;
        wtop[wv][3] = c23 & 0xffffu;
        wtop[wv][4] = c23 >> 16;
    }
    zero_hist(hist3[0]);
    __syncthreads();

    // 2. The row's four highest top bytes: lane v < NWV holds wave v's entry.
    static_assert(NWV <= 16, "one DPP row holds every wave's entry");
    uint4 we = make_uint4(0u, 0u, 0u, 0u);
    uint32_t we4 = 0u;
    if (lane < NWV) {
        we = *reinterpret_cast<const uint4*>(&wtop[lane][0]);
        we4 = wtop[lane][4];
    }
    const uint32_t rtop = row16_reduce_u32<true>(we.x);
    uint32_t tot[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t b = rtop - (uint32_t)i, dv = we.x - b;
        const uint32_t cv = (lane < NWV && rtop >= (uint32_t)i && we.x >= b)
                                ? (dv == 0u ? we.y : dv == 1u ? we.z : dv == 2u ? we.w : we4)
                                : 0u;
        tot[i] = row16_reduce_u32<false>(cv);
    }
    uint32_t bin0 = rtop, remaining = (uint32_t)w;
    bool found = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (!found && rtop >= (uint32_t)i) {
            if (tot[i] >= remaining) {
                bin0 = rtop - (uint32_t)i;
                found = true;
            } else {
                remaining -= tot[i];
            }
        }
    }

    // 3. This wave's keys of top byte bin0 or above, in position order, and
    // the first digit's histogram of its keys of top byte bin0.
    uint32_t nl = 0u;
    if (found) {
        const uint32_t lo = bin0 << 24;
        uint32_t cnt = 0u;
        bool ovf = false;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const bool is = TOPB ? top8(j) >= bin0 : key[TOPB ? 0 : j] >= lo;
            const uint64_t mb = __ballot(is);
            const uint32_t pc = (uint32_t)__popcll(mb);
            if (cnt + pc <= (uint32_t)CW) {
                if (is)
                    cand[wv][cnt + (uint32_t)lanes_below(mb)] =
                        make_uint2(TOPB ? hi16(j) : key[TOPB ? 0 : j], (uint32_t)(pl + kWave * j));
            } else {
                ovf = true;
            }
            cnt += pc;
        }
        nl = min(cnt, (uint32_t)CW);
        for (uint32_t i = lane; i < nl; i += kWave) {
            const uint32_t kc = cand[wv][i].x;
            if ((kc >> 24) == bin0) atomicAdd(&hist3[0][(kc >> 16) & 255u], 1u);
        }
        if (lane == 0) wcnt[wv] = ovf ? 0xffffffffu : cnt;
        zero_hist(hist3[1]);
    }
    __syncthreads();
    bool slow = !found;
    if (found) {
#pragma unroll
        for (int v = 0; v < NWV; ++v) slow = slow || wcnt[v] == 0xffffffffu;
    }

    uint32_t prefix = bin0 << 24, himask = 0xff000000u;
    // 4. Digit passes over the lists (one barrier each), from digit pass0 on
    // (prefix, himask and remaining hold the digits before it), then 5.
    auto list_path = [&](int pass0) {
        for (int pass = pass0; pass < 3; ++pass) {
            const int shift = 16 - 8 * pass;
            if (pass > 0) {
                if (TOPB && pass == 1 && pass0 == 0) {
                    // lists of high halves: the entries in the threshold's
                    // 16-bit bucket get their keys in full from the score row
                    // (every load issued at once, out of range for the others)
                    const uint32_t p16 = prefix & 0xffff0000u;
                    static_assert(kCandPerWave <= 8 * kWave, "one round of loads covers a list");
                    uint32_t pp[8], kv[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const uint32_t i = (uint32_t)(u * kWave + lane);
                        const uint2 e = i < nl ? cand[wv][i] : make_uint2(0u, 0u);
                        pp[u] = (i < nl && (e.x & 0xffff0000u) == p16 && e.y < (uint32_t)n)
                                    ? e.y : 0xffffffffu;
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        kv[u] = order_key(__uint_as_float(
                            buffer_load4(srs, pp[u] != 0xffffffffu ? 4u * pp[u] : kOutOfRange)));
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        if (pp[u] != 0xffffffffu) cand[wv][(uint32_t)(u * kWave + lane)].x = kv[u];
                }
                for (uint32_t i = lane; i < nl; i += kWave) {
                    const uint32_t kc = cand[wv][i].x;
                    if ((kc & himask) == prefix) atomicAdd(&hist3[pass][(kc >> shift) & 255u], 1u);
                }
                zero_hist(hist3[(pass + 1) % 3]);
                __syncthreads();
            }
            uint32_t b, r;
            find_bin_wave(hist3[pass], remaining, b, r);
            prefix |= b << shift;
            himask |= 0xffu << shift;
            remaining = r;
        }
        // 5. Members from the lists: counts per wave, then position-ordered writes.
        const uint32_t T = prefix, need_eq = remaining;
        uint32_t gtc = 0u, eqc = 0u;
        for (uint32_t base = 0; base < nl; base += kWave) {
            const uint32_t i = base + lane;
            const uint32_t kc = i < nl ? cand[wv][i].x : 0u;
            gtc += (uint32_t)__popcll(__ballot(i < nl && kc > T));
            eqc += (uint32_t)__popcll(__ballot(i < nl && kc == T));
        }
        if (lane == 0) {
            wgt[wv] = gtc;
            weq[wv] = eqc;
        }
        __syncthreads();
        uint32_t eq_before = 0u, sel_before = 0u;
        for (int v = 0; v < wv; ++v) {
            const uint32_t take = (need_eq > eq_before) ? min(need_eq - eq_before, weq[v]) : 0u;
            sel_before += wgt[v] + take;
            eq_before += weq[v];
        }
        for (uint32_t base = 0; base < nl; base += kWave) {
            const uint32_t i = base + lane;
            const uint2 e = i < nl ? cand[wv][i] : make_uint2(0u, 0u);
            const bool gt = i < nl && e.x > T, eq = i < nl && e.x == T;
            const uint64_t eb = __ballot(eq);
            const bool sel = gt || (eq && eq_before + (uint32_t)lanes_below(eb) < need_eq);
            const uint64_t sb = __ballot(sel);
            const uint32_t slot = sel_before + (uint32_t)lanes_below(sb);
            if (sel && slot < (uint32_t)w && e.y < (uint32_t)n) {
                out[slot] = (int32_t)e.y;
                if (mrow != nullptr) atomicOr(mrow + (long)e.y * KW, cbit);
            }
            eq_before += (uint32_t)__popcll(eb);
            sel_before += (uint32_t)__popcll(sb);
        }
    };
    if (!slow) {
        list_path(0);
        return;
    }

    // Over all keys: the remaining digits (all four when bin0 is unknown) ...
    // fn(j, key j) for every key of this lane, in order; (TOPB) re-read from
    // the score row sixteen at a time
    auto for_keys = [&](auto&& fn) {
        if constexpr (!TOPB) {
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                fn(j, key[TOPB ? 0 : j]);
                if (j % 8 == 7) __builtin_amdgcn_sched_barrier(0);   // few ballots live
            }
        } else {
#pragma unroll 1
            for (int j0 = 0; j0 < KPT; j0 += 16) {
                uint32_t kk[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int p = pl + kWave * (j0 + u);
                    const uint32_t kj = order_key(
                        __uint_as_float(buffer_load4(srs, p < n ? 4u * (uint32_t)p : kOutOfRange)));
                    kk[u] = p < n ? kj : 0u;
                }
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    fn(j0 + u, kk[u]);
                    if (u % 8 == 7) __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };
    if (!found) {
        prefix = 0u;
        himask = 0u;
        remaining = (uint32_t)w;
    }
    zero_hist(hist3[0]);
    __syncthreads();
    for (int shift = found ? 16 : 24, it = 0; shift >= 0; shift -= 8, ++it) {
        uint32_t* h = hist3[it % 3];
        for_keys([&](int, uint32_t kj) {
            if ((kj & himask) == prefix) atomicAdd(&h[(kj >> shift) & 255u], 1u);
        });
        zero_hist(hist3[(it + 1) % 3]);
        __syncthreads();
        uint32_t b, r;
        find_bin_wave(h, remaining, b, r);
        prefix |= b << shift;
        himask |= 0xffu << shift;
        remaining = r;
        if (found && shift == 16) {
            // The top-byte lists overflowed (a top byte spans a factor of 4 in
            // score): list the keys at or above the 16-bit prefix instead, one
            // more pass over the keys, and finish on the lists if they fit.
            uint32_t cnt = 0u;
            bool ovf = false;
            for_keys([&](int j, uint32_t kj) {
                const bool is = kj >= prefix;
                const uint64_t mb = __ballot(is);
                const uint32_t pc = (uint32_t)__popcll(mb);
                if (cnt + pc <= (uint32_t)CW) {
                    if (is)
                        cand[wv][cnt + (uint32_t)lanes_below(mb)] =
                            make_uint2(kj, (uint32_t)(pl + kWave * j));
                } else {
                    ovf = true;
                }
                cnt += pc;
            });
            if (lane == 0) wcnt[wv] = ovf ? 0xffffffffu : cnt;   // read before the last barrier
            __syncthreads();
            bool again = false;
#pragma unroll
            for (int v = 0; v < NWV; ++v) again = again || wcnt[v] == 0xffffffffu;
            if (!again) {
                nl = cnt;
                list_path(1);
                return;
            }
        }
    }
    // ... and the members, in position order, from the keys.
    const uint32_t T = prefix, need_eq = remaining;
    uint32_t gtc = 0u, eqc = 0u;
    for_keys([&](int, uint32_t kj) {
        gtc += kj > T ? 1u : 0u;
        eqc += kj == T ? 1u : 0u;
    });
    gtc = wave_reduce_u32<false>(gtc);
    eqc = wave_reduce_u32<false>(eqc);
    if (lane == 0) {
        wgt[wv] = gtc;
        weq[wv] = eqc;
    }
    __syncthreads();
    uint32_t eq_before = 0u, sel_before = 0u;
    for (int v = 0; v < wv; ++v) {
        const uint32_t take = (need_eq > eq_before) ? min(need_eq - eq_before, weq[v]) : 0u;
        sel_before += wgt[v] + take;
        eq_before += weq[v];
    }
    // (a copy of T the compiler cannot identify with it: the comparisons
    // above are not kept alive, as scalar masks, until here)
    const uint32_t T2 = (uint32_t)__builtin_amdgcn_readfirstlane((int)T);
    for_keys([&](int j, uint32_t kj) {
        const int p = pl + kWave * j;
        const bool eq = kj == T2;
        const uint64_t eb = __ballot(eq);
        const bool sel = kj > T2 || (eq && eq_before + (uint32_t)lanes_below(eb) < need_eq);
        const uint64_t sb = __ballot(sel);
        const uint32_t slot = sel_before + (uint32_t)lanes_below(sb);
        if (sel && slot < (uint32_t)w && p < n) {
            out[slot] = p;
            if (mrow != nullptr) atomicOr(mrow + (long)p * KW, cbit);
        }
        eq_before += (uint32_t)__popcll(eb);
        sel_before += (uint32_t)__popcll(sb);
    });
}

// Partition-style balanced clusters: every token sits in exactly one cluster
// of w = n / k.  The tokens of a (batch, head) are ordered by (nearest
// centroid, descending score against it, position); rank r goes to cluster
// r / w, and each cluster is listed by ascending position.  Three launches:
//   part_group_kernel  one workgroup per (batch, head): the label histogram,
//                      its exclusive sums (group offsets), and every token
//                      placed in its label's group (in any order inside it);
//   part_rank_kernel   one workgroup per (batch, head, label): each member's
//                      rank inside its group is the number of members before
//                      it in (descending score, position), so the order the
//                      group was filled in does not matter; offset + rank
//                      gives the cluster and the token's membership bit;
//   part_emit_kernel   one workgroup per (batch, head, cluster): its members
//                      listed in ascending position with wave ballots.
// Each thread requests all its values before using any (kPartPerThread per
// thread, 1024 threads: n <= kPartitionMaxN).
constexpr int kPartThreads = 1024;
constexpr int kPartPerThread = kPartitionMaxN / kPartThreads;

__global__ __launch_bounds__(kPartThreads) void part_group_kernel(const int32_t* __restrict__ label,
                                                                  int n, int k,
                                                                  int32_t* __restrict__ grp,
                                                                  int32_t* __restrict__ goff) {
    __shared__ int hist[256], cursor[256];
    const long base = (long)blockIdx.x * n;
    const buf_rsrc lrs = make_rsrc(label + base, 4u * (uint32_t)n);
    int lab[kPartPerThread];
#pragma unroll
    for (int j = 0; j < kPartPerThread; ++j) {
        const int t = (int)threadIdx.x + kPartThreads * j;
        lab[j] = (int)buffer_load_u32(lrs, t < n ? 4u * t : kOutOfRange);
    }
    for (int c = threadIdx.x; c < k; c += kPartThreads) hist[c] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPartPerThread; ++j)
        if ((int)threadIdx.x + kPartThreads * j < n) atomicAdd(&hist[lab[j]], 1);
    __syncthreads();
    if (threadIdx.x < kWave) {
        // exclusive sums over the k <= 256 labels: four a lane, then across lanes
        const int lane = threadIdx.x;
        int v[4], tot = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = 4 * lane + i < k ? hist[4 * lane + i] : 0;
            tot += v[i];
        }
        int incl = tot;
#pragma unroll
        for (int dl = 1; dl < kWave; dl <<= 1) {
            const int o = __shfl_up(incl, dl);
            if (lane >= dl) incl += o;
        }
        int run = incl - tot;
        int32_t* go = goff + (long)blockIdx.x * (k + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 4 * lane + i;
            if (c < k) {
                cursor[c] = run;
                go[c] = run;
            }
            run += v[i];
        }
        if (lane == kWave - 1) go[k] = run;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPartPerThread; ++j) {
        const int t = (int)threadIdx.x + kPartThreads * j;
        if (t < n) grp[base + atomicAdd(&cursor[lab[j]], 1)] = t;
    }
}

constexpr int kRankThreads = 256;
constexpr int kRankTile = 1024;   // group members staged in LDS at a time

// A member's place in its group's order as one unsigned 64-bit number: the
// order-preserving score key above the complemented position, so that a
// larger number means a higher score, or an equal one at a lower position.
__device__ __forceinline__ unsigned long long rank_key(float score, int pos) {
    return ((unsigned long long)order_key(score) << 32) | (unsigned long long)(~(uint32_t)pos);
}

__global__ __launch_bounds__(kRankThreads) void part_rank_kernel(
    const float* __restrict__ best, const int32_t* __restrict__ grp,
    const int32_t* __restrict__ goff, int n, int k, int w, int KW, int32_t* __restrict__ cl,
    uint32_t* __restrict__ mask) {
    constexpr int PER = kRankTile / kRankThreads;
    __shared__ __attribute__((aligned(16))) unsigned long long skey[kRankTile + 2];
    const int c = blockIdx.x;
    const long bh = blockIdx.y, base = bh * n;
    const int32_t* go = goff + bh * (k + 1);
    const int g0 = go[c], m = go[c + 1] - g0;
    for (int i0 = 0; i0 < m; i0 += kRankThreads) {
        const int i = i0 + (int)threadIdx.x;
        // this member's key: from the first tile when the group fits one,
        // else read for itself
        unsigned long long mine = 0ull;
        if (m > kRankTile && i < m) {
            const int t = grp[base + g0 + i];
            mine = rank_key(best[base + t], t);
        }
        int before = 0;   // members with a larger key
        for (int j0 = 0; j0 < m; j0 += kRankTile) {
            const int jn = min(kRankTile, m - j0);
            __syncthreads();   // the previous tile is no longer read
            // (indices clamped into the tile, so that every load is issued
            // unconditionally and none waits for the one before it)
            int tj[PER];
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                const int j = min((int)threadIdx.x + kRankThreads * u, jn - 1);
                tj[u] = grp[base + g0 + j0 + j];
            }
            float bj[PER];
#pragma unroll
            for (int u = 0; u < PER; ++u) bj[u] = best[base + tj[u]];
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                const int j = (int)threadIdx.x + kRankThreads * u;
                if (j < jn) skey[j] = rank_key(bj[u], tj[u]);
            }
            // padding past the tile: 0 is below every member's key
            if (threadIdx.x < 2) skey[jn + threadIdx.x] = 0ull;
            __syncthreads();
            if (m <= kRankTile && i < m) mine = skey[i];
            if (i < m) {
                for (int j = 0; j < jn; j += 2) {
                    const ulonglong2 kj = *reinterpret_cast<const ulonglong2*>(&skey[j]);
                    before += (kj.x > mine ? 1 : 0) + (kj.y > mine ? 1 : 0);
                }
            }
        }
        if (i < m) {
            const int tok = (int)~(uint32_t)(mine & 0xffffffffull);
            const int clu = (g0 + before) / w;
            cl[base + tok] = clu;
            if (mask != nullptr) mask[(base + tok) * KW + (clu >> 5)] = 1u << (clu & 31);
        }
    }
}

__global__ __launch_bounds__(kPartThreads) void part_emit_kernel(const int32_t* __restrict__ cl,
                                                                 int n, int k, int w,
                                                                 int32_t* __restrict__ idx) {
    constexpr int NWV = kPartThreads / kWave;
    __shared__ int wcount[NWV];
    const int c = blockIdx.x;
    const long bh = blockIdx.y, base = bh * n;
    const int lane = lane_id(), wv = wave_id();
    // wave wv takes positions [wv * seg, (wv + 1) * seg), 64 at a time
    const int seg = kWave * kPartPerThread;
    const buf_rsrc crs = make_rsrc(cl + base, 4u * (uint32_t)n);
    int cv[kPartPerThread];
#pragma unroll
    for (int j = 0; j < kPartPerThread; ++j) {
        const int p = wv * seg + kWave * j + lane;
        cv[j] = (int)buffer_load_u32(crs, p < n ? 4u * p : kOutOfRange);
    }
    bool is[kPartPerThread];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kPartPerThread; ++j) {
        is[j] = wv * seg + kWave * j + lane < n && cv[j] == c;
        cnt += __popcll(__ballot(is[j]));
    }
    if (lane == 0) wcount[wv] = cnt;
    __syncthreads();
    int before = 0;
    for (int v2 = 0; v2 < wv; ++v2) before += wcount[v2];
    int32_t* out = idx + (bh * k + c) * (long)w;
#pragma unroll
    for (int j = 0; j < kPartPerThread; ++j) {
        const uint64_t b = __ballot(is[j]);
        const int slot = before + lanes_below(b);
        if (is[j] && slot < w) out[slot] = wv * seg + kWave * j + lane;
        before += __popcll(b);
    }
}

template <int D, bool ARGMAX>
void launch_score_d(const void* qk, int dtype, const float* mu, int BH, int H, int n, int k,
                    float* inv_norm, float* scores, void* qk_hat, uint32_t* mask, int32_t* label,
                    float* best, hipStream_t s) {
    if (dtype == 1) {
        dim3 grid((n + ScoreCfg<D>::TOK - 1) / ScoreCfg<D>::TOK, BH);
        hipLaunchKernelGGL((score_bf16_kernel<D, ARGMAX>), grid, dim3(ScoreCfg<D>::NT), 0, s,
                           (const u16*)qk, mu, H, n, k, inv_norm, scores, (u16*)qk_hat, mask,
                           mask_words(k), label, best);
    } else {
        dim3 grid((n + 255) / 256, BH);
        hipLaunchKernelGGL((score_f32_kernel<D, ARGMAX>), grid, dim3(256), 0, s, (const float*)qk,
                           mu, H, n, k, inv_norm, scores, (float*)qk_hat, mask, mask_words(k),
                           label, best);
    }
}

template <bool ARGMAX>
void launch_score_any(const void* qk, int dtype, const float* mu, int BH, int H, int n, int d,
                      int k, float* inv_norm, float* scores, void* qk_hat, uint32_t* mask,
                      int32_t* label, float* best, hipStream_t s) {
    switch (d) {
        case 16: launch_score_d<16, ARGMAX>(qk, dtype, mu, BH, H, n, k, inv_norm, scores, qk_hat, mask, label, best, s); break;
        case 32: launch_score_d<32, ARGMAX>(qk, dtype, mu, BH, H, n, k, inv_norm, scores, qk_hat, mask, label, best, s); break;
        case 64: launch_score_d<64, ARGMAX>(qk, dtype, mu, BH, H, n, k, inv_norm, scores, qk_hat, mask, label, best, s); break;
        default: launch_score_d<128, ARGMAX>(qk, dtype, mu, BH, H, n, k, inv_norm, scores, qk_hat, mask, label, best, s); break;
    }
}

template <int NT, int KPT, bool TOPB = false>
void launch_topw_k(const float* scores, int rows, int n, int w, int32_t* idx, int k,
                   uint32_t* mask, hipStream_t s) {
    hipLaunchKernelGGL((topw_kernel<NT, KPT, TOPB>), dim3(rows), dim3(NT), 0, s, scores, n, w, idx,
                       k, mask, mask_words(k));
}

}  // namespace

hipError_t launch_score(const void* qk, int dtype, const float* mu, int B, int H, int n, int d,
                        int k, float* inv_norm, float* scores, void* qk_hat, uint32_t* mask,
                        hipStream_t s) {
    launch_score_any<false>(qk, dtype, mu, B * H, H, n, d, k, inv_norm, scores, qk_hat, mask,
                            nullptr, nullptr, s);
    return hipGetLastError();
}

hipError_t launch_nearest(const void* qk, int dtype, const float* mu, int B, int H, int n, int d,
                          int k, float* inv_norm, int32_t* label, float* best, uint32_t* mask,
                          hipStream_t s) {
    launch_score_any<true>(qk, dtype, mu, B * H, H, n, d, k, inv_norm, nullptr, nullptr, mask,
                           label, best, s);
    return hipGetLastError();
}

hipError_t launch_partition(const int32_t* label, const float* best, int BH, int n, int k,
                            int32_t* idx, uint32_t* mask, int32_t* grp, int32_t* cl,
                            int32_t* goff, hipStream_t s) {
    const int w = n / k;
    hipLaunchKernelGGL(part_group_kernel, dim3(BH), dim3(kPartThreads), 0, s, label, n, k, grp,
                       goff);
    hipLaunchKernelGGL(part_rank_kernel, dim3(k, BH), dim3(kRankThreads), 0, s, best, grp, goff,
                       n, k, w, mask_words(k), cl, mask);
    hipLaunchKernelGGL(part_emit_kernel, dim3(k, BH), dim3(kPartThreads), 0, s, cl, n, k, w, idx);
    return hipGetLastError();
}

hipError_t launch_topw(const float* scores, int BH, int n, int k, int w, int32_t* idx,
                       uint32_t* mask, hipStream_t s) {
    const int rows = BH * k;
    // Up to 1024 keys a row and rows enough to give each of the chip's 1024
    // SIMDs one: a single wave a row, whose barriers cost next to nothing
    // (1024 rows of 1024 keys: route 12.0 -> 11.7 us).  Fewer rows keep four
    // waves a row, which spread each row's chain over more of the chip (512
    // rows: 10.1 us against 10.9 with one wave a row; 256 rows: 10.5 vs 11.0).
    const bool one_wave = rows >= kTopwOneWaveRows;
    if (one_wave && n <= 256) launch_topw_k<64, 4>(scores, rows, n, w, idx, k, mask, s);
    else if (one_wave && n <= 512) launch_topw_k<64, 8>(scores, rows, n, w, idx, k, mask, s);
    else if (one_wave && n <= 1024) launch_topw_k<64, 16>(scores, rows, n, w, idx, k, mask, s);
    else if (n <= 256) launch_topw_k<256, 1>(scores, rows, n, w, idx, k, mask, s);
    else if (n <= 512) launch_topw_k<256, 2>(scores, rows, n, w, idx, k, mask, s);
    else if (n <= 1024) launch_topw_k<256, 4>(scores, rows, n, w, idx, k, mask, s);
    else if (n <= 2048) launch_topw_k<256, 8>(scores, rows, n, w, idx, k, mask, s);
    else if (n <= 4096) launch_topw_k<256, 16>(scores, rows, n, w, idx, k, mask, s);
    else if (n <= kTopwRegisterRow) launch_topw_k<512, 16>(scores, rows, n, w, idx, k, mask, s);
    // beyond 8K keys a row, the keys' high halves only: fewer registers, two rows a CU
    else if (n <= 16384) launch_topw_k<512, 32, true>(scores, rows, n, w, idx, k, mask, s);
    else if (n <= 32768) launch_topw_k<1024, 32, true>(scores, rows, n, w, idx, k, mask, s);
    else launch_topw_k<1024, 64, true>(scores, rows, n, w, idx, k, mask, s);
    return hipGetLastError();
}

}  // namespace rt
