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
//   score_bf16_kernel  one workgroup = 128 tokens x all centroids of a head.
//                      The raw bf16 token rows are the B operand of
//                      v_mfma_f32_16x16x32_bf16 straight from HBM; the fp32
//                      centroids are split into three bf16 terms in LDS
//                      (mu = hi + mid + lo, exact), so three MFMA passes give
//                      float32-accurate inner products.  Scores are scaled by
//                      the token's inverse norm in fp32 afterwards.
//   score_f32_kernel   the same on the vector ALUs for float32 inputs.
//   topw_kernel        one workgroup per (batch, head, centroid) row of n
//                      scores: an exact radix select of the w-th largest
//                      order-preserving key (4 passes of 8 bits, histogram in
//                      LDS), then a position-ordered compaction with wave
//                      ballots, so the w members come out sorted by position
//                      with ties taken at the lowest positions.
#include "rt_common.hpp"
#include "rt_internal.hpp"

namespace rt {
namespace {

template <int D>
struct ScoreCfg {
    static constexpr int DP = D < 32 ? 32 : D;         // dims padded to the MFMA k-depth
    static constexpr int KC = (D == 128) ? 64 : 128;   // centroids per LDS chunk
    static constexpr int LD = DP + 8;                  // LDS row stride (bf16), 16 B aligned
    static constexpr int NS = DP / 32;                 // MFMA k-steps per token row
    static constexpr int TOK = 128;                    // tokens per workgroup (4 waves x 32)
};

template <int D>
__global__ __launch_bounds__(256) void score_bf16_kernel(const u16* __restrict__ qk,
                                                         const float* __restrict__ mu, int H,
                                                         int n, int k,
                                                         float* __restrict__ inv_norm,
                                                         float* __restrict__ scores,
                                                         u16* __restrict__ qk_hat,
                                                         uint32_t* __restrict__ mask, int KW) {
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
    constexpr int MG = (C::KC * GPR) / 256;          // groups per thread
    float4 mreg[MG][2];
    auto load_mu = [&](int c0) {
#pragma unroll
        for (int j = 0; j < MG; ++j) {
            const int e = threadIdx.x + 256 * j;
            const int c = e / GPR, dim0 = 8 * (e % GPR);
            const bool ok = c0 + c < k && dim0 < D;
            const float* src = mu + ((long)h * k + c0 + c) * D + dim0;
            mreg[j][0] = ok ? *reinterpret_cast<const float4*>(src) : make_float4(0.f, 0.f, 0.f, 0.f);
            mreg[j][1] = ok ? *reinterpret_cast<const float4*>(src + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto stage_mu = [&]() {
#pragma unroll
        for (int j = 0; j < MG; ++j) {
            const int e = threadIdx.x + 256 * j;
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
            breg[tb][s] = (t < n && d0 < D) ? *reinterpret_cast<const uint4*>(qk + (base + t) * D + d0)
                                           : zero_u4();
        }
    }
    stage_mu();
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

    for (int c0 = 0; c0 < k; c0 += C::KC) {
        if (c0 > 0) {
            __syncthreads();          // previous chunk's MFMAs are done with lmu
            load_mu(c0);
            stage_mu();
        }
        __syncthreads();
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
                    float* row = scores + ((long)bh * k + c) * n;
                    if (tok[0] < n) row[tok[0]] = acc0[i] * inv[0];
                    if (tok[1] < n) row[tok[1]] = acc1[i] * inv[1];
                }
            }
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void score_f32_kernel(const float* __restrict__ qk,
                                                        const float* __restrict__ mu, int H, int n,
                                                        int k, float* __restrict__ inv_norm,
                                                        float* __restrict__ scores,
                                                        float* __restrict__ qk_hat,
                                                        uint32_t* __restrict__ mask, int KW) {
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
                scores[((long)bh * k + c0 + c) * n + t] = acc * inv;
            }
        }
    }
}

// Order-preserving map float -> uint32 (larger float, larger key); -0 and +0
// map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += (uint32_t)__shfl_xor((int)x, off);
    return x;
}

// Wave 0 finds, in a 256-bin histogram (bins summed over `parts` copies laid
// out `stride` words apart), the bin holding the `remaining`-th largest key:
// writes the bin and the rank left inside it.
__device__ __forceinline__ void find_bin(const uint32_t* hist, int parts, int stride,
                                         uint32_t remaining, uint32_t* sel_bin,
                                         uint32_t* sel_rem) {
    const int lane = lane_id();
    uint32_t cnt[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        uint32_t t = 0u;
        for (int v = 0; v < parts; ++v) t += hist[v * stride + 4 * lane + b];
        cnt[b] = t;
    }
    const uint32_t tot = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    uint32_t suf = tot;  // inclusive suffix sum over lanes
#pragma unroll
    for (int dl = 1; dl < kWave; dl <<= 1) {
        const uint32_t o = __shfl_down(suf, dl);
        if (lane + dl < kWave) suf += o;
    }
    uint32_t above = suf - tot;
#pragma unroll
    for (int b = 3; b >= 0; --b) {
        if (above < remaining && remaining <= above + cnt[b]) {
            *sel_bin = (uint32_t)(4 * lane + b);
            *sel_rem = remaining - above;
        }
        above += cnt[b];
    }
}

// The same search done by each wave for itself on a shared histogram: every
// lane gets the bin and the rank left inside it (no barrier needed after it).
// `remaining` must be between 1 and the histogram total.
__device__ __forceinline__ void find_bin_wave(const uint32_t* hist, uint32_t remaining,
                                              uint32_t& bin, uint32_t& rem) {
    const int lane = lane_id();
    const uint4 c4 = *reinterpret_cast<const uint4*>(hist + 4 * lane);
    const uint32_t cnt[4] = {c4.x, c4.y, c4.z, c4.w};
    const uint32_t tot = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    uint32_t suf = tot;   // inclusive suffix sum over lanes
#pragma unroll
    for (int dl = 1; dl < kWave; dl <<= 1) {
        const uint32_t o = __shfl_down(suf, dl);
        if (lane + dl < kWave) suf += o;
    }
    uint32_t above = suf - tot;
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
    bin = (uint32_t)__shfl(fb, src);
    rem = (uint32_t)__shfl((int)fr, src);
}

// LDSK: the row's keys live in LDS instead of registers (long rows: 64K keys
// need 128 KiB, which LDS holds and registers do not).
template <int NT, int KPT, bool LDSK>
__global__ __launch_bounds__(NT) void topw_kernel(const float* __restrict__ scores, int n, int w,
                                                  int32_t* __restrict__ idx, int k,
                                                  uint32_t* __restrict__ mask, int KW) {
    constexpr int NWV = NT / kWave;
    constexpr int CAND = 4096;           // capacity of the candidate list
    // the candidate list, or before it (only when the first digit needs a full
    // histogram) the per-wave histograms of the top byte
    constexpr int CSZ = CAND > NWV * 256 ? CAND : NWV * 256;
    __shared__ __attribute__((aligned(16))) uint32_t cand[CSZ];
    uint32_t (*sub)[256] = reinterpret_cast<uint32_t (*)[256]>(cand);
    __shared__ __attribute__((aligned(16))) uint32_t lkeys[LDSK ? NT * KPT : 4];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sel_bin, sel_rem;
    __shared__ uint32_t wgt[NWV], weq[NWV];
    __shared__ __attribute__((aligned(16))) uint32_t wtop[NWV][8];   // per wave: highest top
                                         // byte, counts of it and the 3 below (padded)
    __shared__ __attribute__((aligned(16))) uint32_t hist3[3][256];

    const long row = blockIdx.x;
    const float* srow = scores + row * n;
    const int lane = lane_id(), wv = wave_id();
    const int seg0 = wv * kWave * KPT;
    // Wave wv owns positions [seg0, seg0 + 64*KPT); its key j sits at
    // seg0 + 64*VEC*(j / VEC) + VEC*lane + j % VEC: VEC consecutive positions
    // per lane, loaded as one 16-byte vector when VEC = 4.
    constexpr int VEC = (KPT % 4 == 0) ? 4 : 1;
    auto key_pos = [&](int j) { return seg0 + kWave * VEC * (j / VEC) + VEC * lane + j % VEC; };

    uint32_t key[LDSK ? 1 : KPT];
    // key j of this thread (in a register, or read back from LDS)
#define RT_KEY(j) (LDSK ? lkeys[key_pos(j)] : key[LDSK ? 0 : (j)])
    // loops over the keys: fully unrolled for registers, partly for LDS
    constexpr int UNR = LDSK ? 4 : KPT;
    constexpr int UNRG = LDSK ? 1 : KPT / VEC;
    uint32_t wtopb = 0u;   // highest top byte (sign and high exponent bits) in this lane
    const bool vec_ok = VEC == 4 && (n & 3) == 0;   // rows start 16-byte aligned
#pragma unroll
    for (int jg = 0; jg < KPT / VEC; ++jg) {
        const int p0 = key_pos(VEC * jg);
        uint32_t kv[VEC];
        if (vec_ok && p0 + VEC <= n) {
            const float4 f = *reinterpret_cast<const float4*>(srow + p0);
            const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
            for (int e = 0; e < VEC; ++e) kv[e] = order_key(fv[e]);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) kv[e] = (p0 + e < n) ? order_key(srow[p0 + e]) : 0u;
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            if (p0 + e < n) wtopb = max(wtopb, kv[e] >> 24);
            if constexpr (!LDSK) key[VEC * jg + e] = kv[e];
        }
        if constexpr (LDSK) {
            if constexpr (VEC == 4)
                *reinterpret_cast<uint4*>(&lkeys[p0]) = make_uint4(kv[0], kv[1], kv[2], kv[3]);
            else
                lkeys[p0] = kv[0];
        }
    }
    // The w-th largest key nearly always has one of the row's four highest top
    // bytes.  Each wave counts its keys in its own four highest top bytes with
    // per-lane counters (a row's scores share top bytes in large groups, which
    // makes an LDS histogram a hot spot of atomics); one exchange then gives
    // the exact counts of the row's four highest top bytes.
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) wtopb = max(wtopb, (uint32_t)__shfl_xor((int)wtopb, off));
    uint32_t c01 = 0u, c23 = 0u;
#pragma unroll UNR
    for (int j = 0; j < KPT; ++j) {
        const int pos = key_pos(j);
        const uint32_t dlt = wtopb - (RT_KEY(j) >> 24);   // >= 0 for every valid key
        if (pos < n && dlt < 4u) {
            if (dlt < 2u) c01 += 1u << (16 * dlt);
            else c23 += 1u << (16 * (dlt - 2u));
        }
    }
    c01 = wave_sum_u32(c01);
    c23 = wave_sum_u32(c23);
    if (lane == 0) {
        wtop[wv][0] = wtopb;
        wtop[wv][1] = c01 & 0xffffu;
        wtop[wv][2] = c01 >> 16;
        wtop[wv][3] = c23 & 0xffffu;
        wtop[wv][4] = c23 >> 16;
    }
    // the first histogram of the candidate passes starts cleared
    if (threadIdx.x < 256) hist3[0][threadIdx.x] = 0u;
    __syncthreads();
    uint32_t wt[NWV][5];   // every wave's entry, read at once (independent LDS loads)
#pragma unroll
    for (int v = 0; v < NWV; ++v) {
        const uint4 a = *reinterpret_cast<const uint4*>(&wtop[v][0]);
        wt[v][0] = a.x;
        wt[v][1] = a.y;
        wt[v][2] = a.z;
        wt[v][3] = a.w;
        wt[v][4] = wtop[v][4];
    }
    uint32_t rtop = 0u;
#pragma unroll
    for (int v = 0; v < NWV; ++v) rtop = max(rtop, wt[v][0]);
    uint32_t bin0 = rtop, remaining = (uint32_t)w, ncand = 0u, cand_off = 0u;
    bool found = false;
    for (uint32_t i = 0; i < 4u && i <= rtop; ++i) {
        const uint32_t b = rtop - i;
        uint32_t tot = 0u, before = 0u;
#pragma unroll
        for (int v = 0; v < NWV; ++v) {
            const uint32_t dv = wt[v][0] - b;   // wt[v][0] <= rtop, so dv <= i <= 3
            uint32_t cv = 0u;
            if (wt[v][0] >= b)
                cv = dv == 0u ? wt[v][1] : dv == 1u ? wt[v][2] : dv == 2u ? wt[v][3] : wt[v][4];
            if (v < wv) before += cv;
            tot += cv;
        }
        if (tot >= remaining) {
            bin0 = b;
            ncand = tot;
            cand_off = before;
            found = true;
            break;
        }
        remaining -= tot;
    }
    if (!found) {   // the threshold lies lower: full histogram of the top byte
        for (int e = threadIdx.x; e < NWV * 256; e += NT) (&sub[0][0])[e] = 0u;
        __syncthreads();
#pragma unroll UNR
        for (int j = 0; j < KPT; ++j) {
            const int pos = key_pos(j);
            if (pos < n) atomicAdd(&sub[wv][RT_KEY(j) >> 24], 1u);
        }
        __syncthreads();
        if (wv == 0) find_bin(&sub[0][0], NWV, 256, (uint32_t)w, &sel_bin, &sel_rem);
        __syncthreads();
        bin0 = sel_bin;
        remaining = sel_rem;
        ncand = 0u;
        for (int v = 0; v < NWV; ++v) {
            if (v == wv) cand_off = ncand;
            ncand += sub[v][bin0];
        }
        __syncthreads();   // the candidate list reuses the histograms' memory
    }

    // Radix select: after the four digits `prefix` is the w-th largest key and
    // `remaining` the number of keys equal to it that belong to the top w.
    uint32_t prefix = bin0 << 24, himask = 0xff000000u;
    if (ncand <= (uint32_t)CAND) {
        // The remaining digits only concern keys whose top byte is bin0: list
        // them (in position order) and finish on the short list.
#pragma unroll UNR
        for (int j = 0; j < KPT; ++j) {
            const int pos = key_pos(j);
            const uint32_t kj = RT_KEY(j);
            const bool is = pos < n && (kj >> 24) == bin0;
            const uint64_t mb = __ballot(is);
            if (is) cand[cand_off + (uint32_t)lanes_below(mb)] = kj;
            cand_off += (uint32_t)__popcll(mb);
        }
        __syncthreads();
        // One barrier per digit: every wave reads the histogram itself after
        // it, and the histogram of the next digit (not read by anyone since
        // the barrier before this one) is cleared while this one fills.
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = 16 - 8 * pass;
            for (uint32_t i = threadIdx.x; i < ncand; i += NT) {
                const uint32_t kc = cand[i];
                if ((kc & himask) == prefix) atomicAdd(&hist3[pass][(kc >> shift) & 255u], 1u);
            }
            if (threadIdx.x < 256) hist3[(pass + 1) % 3][threadIdx.x] = 0u;
            __syncthreads();
            uint32_t b, r;
            find_bin_wave(hist3[pass], remaining, b, r);
            prefix |= b << shift;
            himask |= 0xffu << shift;
            remaining = r;
        }
    } else {
        for (int shift = 16; shift >= 0; shift -= 8) {
            if (threadIdx.x < 256) hist[threadIdx.x] = 0u;
            __syncthreads();
#pragma unroll UNR
            for (int j = 0; j < KPT; ++j) {
                const int pos = key_pos(j);
                const uint32_t kj = RT_KEY(j);
                if (pos < n && (kj & himask) == prefix)
                    atomicAdd(&hist[(kj >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (wv == 0) find_bin(hist, 1, 0, remaining, &sel_bin, &sel_rem);
            __syncthreads();
            prefix |= sel_bin << shift;
            himask |= 0xffu << shift;
            remaining = sel_rem;
        }
    }
    const uint32_t T = prefix, need_eq = remaining;

    // Position-ordered compaction: wave wv's positions are visited in
    // ascending order (groups jg, then lanes, then the VEC keys of a lane).
    uint32_t gtc = 0u, eqc = 0u;
#pragma unroll UNR
    for (int j = 0; j < KPT; ++j) {
        const int pos = key_pos(j);
        const bool valid = pos < n;
        const uint32_t kj = RT_KEY(j);
        gtc += (valid && kj > T) ? 1u : 0u;
        eqc += (valid && kj == T) ? 1u : 0u;
    }
    gtc = wave_sum_u32(gtc);
    eqc = wave_sum_u32(eqc);
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
    int32_t* out = idx + row * w;
    const long bh = row / k;
    const int c = (int)(row % k);
#pragma unroll UNRG
    for (int jg = 0; jg < KPT / VEC; ++jg) {
        // positions of group jg in ascending order: (lane, e) lexicographic
        bool gt[VEC], eq[VEC], sel[VEC];
        uint64_t eb[VEC], sb[VEC];
        uint32_t eq_lanes = 0u, sel_lanes = 0u;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int j = VEC * jg + e;
            const bool valid = key_pos(j) < n;
            const uint32_t kj = RT_KEY(j);
            gt[e] = valid && kj > T;
            eq[e] = valid && kj == T;
            eb[e] = __ballot(eq[e]);
            eq_lanes += (uint32_t)lanes_below(eb[e]);
        }
        uint32_t own = 0u;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            sel[e] = gt[e] || (eq[e] && eq_before + eq_lanes + own < need_eq);
            own += eq[e] ? 1u : 0u;
            sb[e] = __ballot(sel[e]);
            sel_lanes += (uint32_t)lanes_below(sb[e]);
        }
        own = 0u;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const uint32_t slot = sel_before + sel_lanes + own;
            if (sel[e] && slot < (uint32_t)w) {
                const int pos = key_pos(VEC * jg + e);
                out[slot] = pos;
                if (mask != nullptr)
                    atomicOr(&mask[(bh * n + pos) * KW + (c >> 5)], 1u << (c & 31));
            }
            own += sel[e] ? 1u : 0u;
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            eq_before += (uint32_t)__popcll(eb[e]);
            sel_before += (uint32_t)__popcll(sb[e]);
        }
    }
}

template <int D>
void launch_score_d(const void* qk, int dtype, const float* mu, int BH, int H, int n, int k,
                    float* inv_norm, float* scores, void* qk_hat, uint32_t* mask, hipStream_t s) {
    if (dtype == 1) {
        dim3 grid((n + ScoreCfg<D>::TOK - 1) / ScoreCfg<D>::TOK, BH);
        hipLaunchKernelGGL(score_bf16_kernel<D>, grid, dim3(256), 0, s, (const u16*)qk, mu, H, n,
                           k, inv_norm, scores, (u16*)qk_hat, mask, mask_words(k));
    } else {
        dim3 grid((n + 255) / 256, BH);
        hipLaunchKernelGGL(score_f32_kernel<D>, grid, dim3(256), 0, s, (const float*)qk, mu, H, n,
                           k, inv_norm, scores, (float*)qk_hat, mask, mask_words(k));
    }
}

#undef RT_KEY

template <int NT, int KPT, bool LDSK = false>
void launch_topw_k(const float* scores, int rows, int n, int w, int32_t* idx, int k,
                   uint32_t* mask, hipStream_t s) {
    hipLaunchKernelGGL((topw_kernel<NT, KPT, LDSK>), dim3(rows), dim3(NT), 0, s, scores, n, w, idx,
                       k, mask, mask_words(k));
}

}  // namespace

hipError_t launch_score(const void* qk, int dtype, const float* mu, int B, int H, int n, int d,
                        int k, float* inv_norm, float* scores, void* qk_hat, uint32_t* mask,
                        hipStream_t s) {
    const int BH = B * H;
    switch (d) {
        case 16: launch_score_d<16>(qk, dtype, mu, BH, H, n, k, inv_norm, scores, qk_hat, mask, s); break;
        case 32: launch_score_d<32>(qk, dtype, mu, BH, H, n, k, inv_norm, scores, qk_hat, mask, s); break;
        case 64: launch_score_d<64>(qk, dtype, mu, BH, H, n, k, inv_norm, scores, qk_hat, mask, s); break;
        default: launch_score_d<128>(qk, dtype, mu, BH, H, n, k, inv_norm, scores, qk_hat, mask, s); break;
    }
    return hipGetLastError();
}

hipError_t launch_topw(const float* scores, int BH, int n, int k, int w, int32_t* idx,
                       uint32_t* mask, hipStream_t s) {
    const int rows = BH * k;
    const int per = (n + 511) / 512;
    if (per <= 1) launch_topw_k<512, 1>(scores, rows, n, w, idx, k, mask, s);
    else if (per <= 2) launch_topw_k<512, 2>(scores, rows, n, w, idx, k, mask, s);
    else if (per <= 4) launch_topw_k<512, 4>(scores, rows, n, w, idx, k, mask, s);
    else if (per <= 8) launch_topw_k<512, 8>(scores, rows, n, w, idx, k, mask, s);
    else if (per <= 16) launch_topw_k<512, 16>(scores, rows, n, w, idx, k, mask, s);
    else if (per <= 32) launch_topw_k<512, 32>(scores, rows, n, w, idx, k, mask, s);
    else if (per <= 64) launch_topw_k<1024, 32, true>(scores, rows, n, w, idx, k, mask, s);
    else launch_topw_k<1024, 64>(scores, rows, n, w, idx, k, mask, s);
    return hipGetLastError();
}

}  // namespace rt
