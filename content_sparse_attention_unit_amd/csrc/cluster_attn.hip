// cluster_attn.hip -- attention inside each routed cluster, and the
// scatter-add of the cluster rows back to token order (gfx950).
//
// Routing attention (paperlayer.ai summary of "Efficient Content-Based Sparse
// Attention with Routing Transformers", §4): only query-key pairs routed to
// the same cluster are attended to; with balanced clusters each query meets w
// keys, so the in-cluster dot products cost O(n w d).  Within a cluster the
// attention is the ordinary autoregressive softmax attention of §3: member s
// is visible to member r when its original position is not later.
//
// Membership bitmask: mask[b][h][t] holds one bit per centroid (KW = ceil(k/32)
// words per token).  For member row r of cluster c holding token t,
// cnt = popcount(mask[t]) and rank = number of set bits below c.  A token held
// by one cluster is written straight to `out`; otherwise its row goes to the
// partial buffer at slot `rank` (token-major, kSlots slots per token; higher
// ranks go to a cluster-major overflow buffer and are listed in a per-token
// directory), and combine_kernel sums the slots in rank order, i.e. ascending
// centroid order, so results are deterministic.
//
// Kernels
//   zero_u32_kernel / mask_kernel   build the bitmask from idx (skipped when
//                       the caller passes the mask rt_route produced).
//   cluster_attn_bf16   one workgroup per cluster.  Every member row of the
//                       keys (raw bf16) and values is requested from memory at
//                       once, in two round trips (all row indices, then all
//                       rows); keys are staged in LDS, values stay in flight
//                       while the first query block's logits are computed, then
//                       are stored transposed.  Each wave takes 16-row query blocks in a
//                       zig-zag order that balances the causal triangle,
//                       computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16
//                       (each lane owns one query, so the row statistics are
//                       per lane), applies the inverse norms and the scale in
//                       fp32, runs an online softmax over 64-key chunks and
//                       accumulates O^T = V^T P^T with the same MFMA.  It can
//                       also emit the per-cluster sums of the normalised rows
//                       that the centroid update needs.
//   cluster_attn_f32    a plain vector-ALU variant for float32 inputs.
//   combine_kernel      per token: zeros if no cluster holds it, the ordered
//                       sum of its slots if several do, nothing if one does.
#include <type_traits>

#include "rt_common.hpp"
#include "rt_internal.hpp"

namespace rt {
namespace {

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* __restrict__ p, long count) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i < count) p[i] = 0u;
}

// grid (ceil(w / 256), k, BH): one thread per membership.
__global__ __launch_bounds__(256) void mask_kernel(const int32_t* __restrict__ idx, int n, int k,
                                                   int w, int KW, uint32_t* __restrict__ mask) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    const int c = blockIdx.y, bh = blockIdx.z;
    if (r >= w) return;
    const int t = idx[((long)bh * k + c) * w + r];
    if (t < 0 || t >= n) return;
    atomicOr(&mask[((long)bh * n + t) * KW + (c >> 5)], 1u << (c & 31));
}

template <int D, int WMAX, bool SHARED>
struct AttnCfg {
    static constexpr int DP = D < 32 ? 32 : D;  // dims padded to the MFMA k-depth
    // key/query/value row stride in LDS (bf16): an odd multiple of 16 elements,
    // so 8 consecutive rows start in disjoint bank groups; DP + 8 from 256
    // rows on, which lets two workgroups share a CU at d = 64, w = 256 (twice
    // the waves in flight: 72 -> 57 us for the 32K-token stress call) and the
    // 512-row tile fit at all
    static constexpr int LDX = (WMAX >= 256) ? DP + 8 : DP + 16;
    static constexpr int NS = DP / 32;          // MFMA k-steps over d
    static constexpr int NJ = D / 16;           // 16-wide output column blocks
    static constexpr int QROWS = SHARED ? 1 : WMAX;
    // waves per workgroup: one or two 16-row query blocks each
    static constexpr int NW = WMAX <= 32 ? 2 : (WMAX <= 128 ? 4 : 8);
    static constexpr int NT = 64 * NW;
    static constexpr int CPR = DP / 8;          // 16-byte chunks per padded key row
    static constexpr int XPT = (WMAX * CPR + NT - 1) / NT;         // key chunks per thread
    static constexpr int DCH = D / 8;           // 16-byte chunks per value row
    static constexpr int VPT = (WMAX * DCH + NT - 1) / NT;         // value chunks per thread
};

template <int D, int WMAX, bool SHARED, typename OutT>
__global__ __launch_bounds__((AttnCfg<D, WMAX, SHARED>::NT), 2) void cluster_attn_bf16_kernel(
    const u16* __restrict__ q, const u16* __restrict__ kk, const u16* __restrict__ v,
    const float* __restrict__ q_inv, const float* __restrict__ k_inv,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ idx_q,
    const uint32_t* __restrict__ mask, int n, int k, int w,
    int KW, float scale, int causal, OutT* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ slots, float* __restrict__ ovf, int32_t* __restrict__ dir,
    float* __restrict__ sum_q, float* __restrict__ sum_k) {
    using C = AttnCfg<D, WMAX, SHARED>;
    __shared__ __attribute__((aligned(16))) u16 lx[WMAX * C::LDX];
    __shared__ __attribute__((aligned(16))) u16 lq[C::QROWS * C::LDX];
    __shared__ __attribute__((aligned(16))) u16 lv[WMAX * C::LDX];
    __shared__ __attribute__((aligned(16))) float linvk[WMAX];
    __shared__ __attribute__((aligned(16))) float linvq[C::QROWS];
    __shared__ int lpos[WMAX];    // position, or -1 for padding / invalid rows
    __shared__ int ldest[WMAX];   // see row_dest
    // partial member sums per wave (one side for shared q/k, else keys then queries)
    __shared__ float lsum[SHARED ? 1 : 2][C::NW][C::DP];

    // the clusters of one head on one XCD (they gather rows of the same head)
    const int item = xcd_contiguous(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
    const int cl = item % gridDim.x, bh = item / gridDim.x;
    const long tokbase = (long)bh * n;
    const long rowbase = ((long)bh * k + cl) * w;
    const int32_t* irow = idx + rowbase;              // the cluster's keys (and values)
    // its queries: the same rows unless the queries were routed on their own
    // (then only without causality: the mask below compares row indices)
    const int32_t* irowq = SHARED ? irow : idx_q + rowbase;

    // Request every member row at once.  First the row indices, all in flight
    // together with this thread's output row; then that row's inverse norms and
    // membership words and every key/query and value row the indices name.
    // The loads go through buffer resources (one per (batch, head) slice or
    // cluster row): rows past w and absent inverse norms read as zeros from an
    // offset out of range, so no load sits under a branch, and nothing loaded is
    // used before the last load is issued.  (A load under a branch, or one whose
    // address needs another load, makes the compiler wait for every load issued
    // before it: one memory round trip per row instead of two in all.)
    // Thread t holds the 16-byte chunk t % CPR of rows t / CPR + (NT / CPR) * it.
    static_assert(C::NT >= WMAX, "one output row per thread");
    const bool want_sums = sum_q != nullptr || sum_k != nullptr;
    const uint32_t slice = (uint32_t)n * D * 2u;   // bytes of one (batch, head) slice
    const buf_rsrc krs = make_rsrc(kk + tokbase * D, slice);
    const buf_rsrc qrs = make_rsrc(q + tokbase * D, slice);
    const buf_rsrc vrs = make_rsrc(v + tokbase * D, slice);
    const buf_rsrc irs = make_rsrc(irow, 4u * (uint32_t)w);
    const buf_rsrc iqrs = make_rsrc(irowq, 4u * (uint32_t)w);
    const buf_rsrc kinv_rs = make_rsrc(k_inv ? k_inv + tokbase : nullptr, k_inv ? 4u * n : 0u);
    const buf_rsrc qinv_rs = make_rsrc(q_inv ? q_inv + tokbase : nullptr, q_inv ? 4u * n : 0u);
    const buf_rsrc mrs = make_rsrc(mask + tokbase * KW, 4u * (uint32_t)n * KW);

    int tk[C::XPT], tq[SHARED ? 1 : C::XPT];
#pragma unroll
    for (int it = 0; it < C::XPT; ++it) {
        const int r = (int)(threadIdx.x + it * C::NT) / C::CPR;
        const uint32_t off = r < w ? 4u * r : kOutOfRange;
        tk[it] = (int)buffer_load_u32(irs, off);
        if (!SHARED) tq[it] = (int)buffer_load_u32(iqrs, off);
    }
    constexpr bool VROWS = C::DCH == C::CPR;   // value chunks lie on the key rows
    int tv[VROWS ? 1 : C::VPT];
    if constexpr (!VROWS) {
#pragma unroll
        for (int it = 0; it < C::VPT; ++it) {
            const int r = (int)(threadIdx.x + it * C::NT) / C::DCH;
            tv[it] = (int)buffer_load_u32(irs, r < w ? 4u * r : kOutOfRange);
        }
    }
    const int orow = threadIdx.x;
    const uint32_t ooff = orow < w ? 4u * orow : kOutOfRange;
    const int raw = (int)buffer_load_u32(iqrs, ooff);   // row orow's query token (if orow < w)
    const int kraw = SHARED ? raw : (int)buffer_load_u32(irs, ooff);  // and its key token

    // this thread's output row: inverse norms (0 when absent) and membership words
    const bool qok = orow < w && raw >= 0 && raw < n;
    const float ik_ld = __uint_as_float(
        buffer_load_u32(kinv_rs, orow < w ? 4u * clamp_pos(kraw, n) : kOutOfRange));
    const float iq_ld = SHARED ? ik_ld : __uint_as_float(
        buffer_load_u32(qinv_rs, orow < w ? 4u * clamp_pos(raw, n) : kOutOfRange));
    uint32_t wd[8];
    load_words(mrs, qok, clamp_pos(raw, n), KW, wd);

    uint4 xk[C::XPT], xq[SHARED ? 1 : C::XPT];
    float ikr[C::XPT], iqr[SHARED ? 1 : C::XPT];   // their inverse norms (0 when absent)
#pragma unroll
    for (int it = 0; it < C::XPT; ++it) {
        const int e = threadIdx.x + it * C::NT;
        const int r = e / C::CPR, ch = e % C::CPR;
        const bool ok = r < w && 8 * ch < D;
        xk[it] = buffer_load16(krs, ok ? 2u * (uint32_t)(clamp_pos(tk[it], n) * D + 8 * ch) : kOutOfRange);
        if (!SHARED)
            xq[it] = buffer_load16(qrs, ok ? 2u * (uint32_t)(clamp_pos(tq[it], n) * D + 8 * ch) : kOutOfRange);
        // (read as zeros unless the sums are wanted)
        ikr[it] = __uint_as_float(buffer_load_u32(
            kinv_rs, ok && want_sums ? 4u * clamp_pos(tk[it], n) : kOutOfRange));
        if (!SHARED)
            iqr[it] = __uint_as_float(buffer_load_u32(
                qinv_rs, ok && want_sums ? 4u * clamp_pos(tq[it], n) : kOutOfRange));
    }
    uint4 va[C::VPT];
#pragma unroll
    for (int it = 0; it < C::VPT; ++it) {
        const int e = threadIdx.x + it * C::NT;
        const int r = e / C::DCH, ch = e % C::DCH;
        const int t = clamp_pos(VROWS ? tk[VROWS ? it : 0] : tv[VROWS ? 0 : it], n);
        va[it] = buffer_load16(vrs, r < w ? 2u * (uint32_t)(t * D + 8 * ch) : kOutOfRange);
    }
    if (want_sums) {
        // absent inverse norms: the rows are unit vectors already
#pragma unroll
        for (int it = 0; it < C::XPT; ++it) {
            const int e = threadIdx.x + it * C::NT;
            const bool ok = e / C::CPR < w && 8 * (e % C::CPR) < D;
            if (k_inv == nullptr) ikr[it] = ok ? 1.f : 0.f;
            if (!SHARED && q_inv == nullptr) iqr[SHARED ? 0 : it] = ok ? 1.f : 0.f;
        }
    }
    {
        int pos = -1, dest = -2;
        if (qok) {
            pos = raw;
            dest = dest_from_words(wd, cl, KW);
            if (dest >= kSlots) dir[(tokbase + raw) * (k - kSlots) + (dest - kSlots)] = cl * w + orow;
        }
        if (orow < WMAX) {
            lpos[orow] = pos;
            ldest[orow] = dest;
            linvk[orow] = orow < w ? (k_inv ? ik_ld : 1.f) : 0.f;
            if (!SHARED) linvq[orow] = orow < w ? (q_inv ? iq_ld : 1.f) : 0.f;
        }
    }
#pragma unroll
    for (int it = 0; it < C::XPT; ++it) {
        const int e = threadIdx.x + it * C::NT;
        if (e < WMAX * C::CPR) {
            const int r = e / C::CPR, ch = e % C::CPR;
            *reinterpret_cast<uint4*>(&lx[r * C::LDX + 8 * ch]) = xk[it];
            if (!SHARED) *reinterpret_cast<uint4*>(&lq[r * C::LDX + 8 * ch]) = xq[it];
        }
    }
    // Per-cluster sums of the normalised member rows (for the centroid update):
    // each thread sums its own rows, then the lanes holding the same chunk, then
    // the waves (after the barrier below).  Fixed order, so deterministic.
    static_assert(C::NT % C::CPR == 0 && 64 % C::CPR == 0, "chunk per thread must be fixed");
    if (want_sums) {
        const int lane0 = lane_id(), wv0 = threadIdx.x >> 6;
#pragma unroll
        for (int side = 0; side < (SHARED ? 1 : 2); ++side) {
            float a[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) a[j] = 0.f;
#pragma unroll
            for (int it = 0; it < C::XPT; ++it) {
                const uint4 x = (side == 0) ? xk[it] : xq[SHARED ? 0 : it];
                const float iv = (side == 0) ? ikr[it] : iqr[SHARED ? 0 : it];
#pragma unroll
                for (int j = 0; j < 8; ++j) a[j] = fmaf(u4_elem(x, j), iv, a[j]);
            }
#pragma unroll
            for (int off = C::CPR; off < 64; off <<= 1)
#pragma unroll
                for (int j = 0; j < 8; ++j) a[j] += __shfl_xor(a[j], off);
            if (lane0 < C::CPR) {
#pragma unroll
                for (int j = 0; j < 8; ++j) lsum[side][wv0][8 * lane0 + j] = a[j];
            }
        }
    }
    __syncthreads();
    if (want_sums) {
        const long sbase = ((long)bh * k + cl) * D;
        for (int dcol = threadIdx.x; dcol < D; dcol += C::NT) {
            float tot[2] = {0.f, 0.f};
#pragma unroll
            for (int side = 0; side < (SHARED ? 1 : 2); ++side)
                for (int v2 = 0; v2 < C::NW; ++v2) tot[side] += lsum[side][v2][dcol];
            if (sum_k != nullptr) sum_k[sbase + dcol] = tot[0];
            if (sum_q != nullptr) sum_q[sbase + dcol] = tot[SHARED ? 0 : 1];
        }
    }

    const int lane = lane_id(), wv = wave_id();
    const int g = lane >> 4, r16 = lane & 15;
    const int nqb = (w + 15) / 16;
    const float sl2 = scale * 1.4426950408889634f;  // logits in log2 units
    const u16* qsrc = SHARED ? lx : lq;
    bool values_staged = false;

    for (int round = 0; round * C::NW < nqb; ++round) {
        const int qb = round * C::NW + ((round & 1) ? (C::NW - 1 - wv) : wv);
        const bool active = qb < nqb;
        const int qrow = qb * 16 + r16;
        uint4 qreg[C::NS];
        float qs = 0.f;
#pragma unroll
        for (int s = 0; s < C::NS; ++s) qreg[s] = zero_u4();
        if (active) {
#pragma unroll
            for (int s = 0; s < C::NS; ++s)
                qreg[s] = *reinterpret_cast<const uint4*>(&qsrc[qrow * C::LDX + 32 * s + 8 * g]);
            qs = sl2 * (SHARED ? linvk[qrow] : linvq[qrow]);
        }
        f32x4 o[C::NJ];
#pragma unroll
        for (int jb = 0; jb < C::NJ; ++jb) o[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m = -INFINITY;
        f32x4 zacc = {0.f, 0.f, 0.f, 0.f};
        const int kend = !active ? 0 : (causal ? min(w, qb * 16 + 16) : w);
        // keys below `clean` are visible to every query of the block
        const int clean = causal ? qb * 16 : w;
        // this lane's last visible key (the row's last, or its own under
        // causality), less the lane's key offset 4 g
        const int glim = (causal ? min(qrow, w - 1) : w - 1) - 4 * g;

        for (int kc = 0; kc < kend || !values_staged; kc += 64) {
            f32x4 sv[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int key0 = kc + 16 * kb;
                if (key0 < kend) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < C::NS; ++s) {
                        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(
                            &lx[(key0 + r16) * C::LDX + 32 * s + 8 * g]));
                        acc = mfma16(a, as_bf16x8(qreg[s]), acc);
                    }
                    const float4 ik = *reinterpret_cast<const float4*>(&linvk[key0 + 4 * g]);
                    sv[kb][0] = acc[0] * qs * ik.x;
                    sv[kb][1] = acc[1] * qs * ik.y;
                    sv[kb][2] = acc[2] * qs * ik.z;
                    sv[kb][3] = acc[3] * qs * ik.w;
                } else {
                    sv[kb] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
                }
            }
            if (!values_staged) {  // first chunk of the first round: values arrive now
#pragma unroll
                for (int it = 0; it < C::VPT; ++it) {
                    const int e = threadIdx.x + it * C::NT;
                    if (e < WMAX * C::DCH) {
                        const int r = e / C::DCH, ch = e % C::DCH;
                        *reinterpret_cast<uint4*>(&lv[r * C::LDX + 8 * ch]) = va[it];
                    }
                }
                __syncthreads();
                values_staged = true;
                if (kc >= kend) break;
            }
            if (kc + 64 > clean) {  // chunk reaches the diagonal or the tail: mask
                // key kc + 16 kb + 4 g + i is visible iff kc + 16 kb + i <= glim
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sv[kb][i] = (kc + 16 * kb + i <= glim) ? sv[kb][i] : -INFINITY;
            }
            const int halves = 1 | ((kc + 32 < kend) ? 2 : 0);
            softmax_pv_chunk<C::NJ, C::LDX>(sv, m, zacc, o, &lv[kc * C::LDX], r16, g, halves);
        }
        if (!active) continue;

        const float zt = zacc[0];   // the query's denominator (every element holds it)
        const float rz = 1.0f / zt;
        if (qrow < w) {
            if (g == 0 && lse != nullptr)
                lse[rowbase + qrow] = (m + __log2f(zt)) * 0.6931471805599453f;
            const int t = lpos[qrow];
            const int dest = ldest[qrow];
            if (t >= 0) {
                if (dest == -1) {
                    // a token only this cluster holds: its finished row,
                    // streamed past L2 (nothing reads it back here; rows for
                    // the scatter stay cached: 13.7 -> 13.4 us a call at 8192
                    // x 8 heads of 128, bit-identical)
                    OutT* dst = out + (tokbase + t) * D + 4 * g;
                    if constexpr (std::is_same<OutT, u16>::value && C::NJ % 2 == 0) {
                        // lanes g = 0..3 of this row hold dims 16 jb + 4 g; after
                        // four lane pulls per 32 dims lane g holds 32 p + 8 g .. +7
                        // (g < 2 from the o[2p] halves, g >= 2 from o[2p+1]), one
                        // 16-byte store each.  Round 0 reads lane s0, round 1 its
                        // partner s0 ^ 1; each source sends the word its reader needs.
                        // The four lanes share qrow, so they take this branch
                        // together.  Whole 64-byte pieces instead of 8-byte ones:
                        // 13.6 -> 13.4 us a call at the size above, counted writes
                        // 33.0 -> 29.2 MB, bit-identical.
                        const int s0 = 2 * (g & 1) + (g >> 1);
                        const int l0 = 16 * s0 + r16, l1 = 16 * (s0 ^ 1) + r16;
                        const bool odd = g & 1, hi = g >= 2;
                        u16* row = out + (tokbase + t) * D + 8 * g;
#pragma unroll
                        for (int p = 0; p < C::NJ / 2; ++p) {
                            const uint32_t a0 = cvt_pk_bf16(o[2 * p][0] * rz, o[2 * p][1] * rz);
                            const uint32_t a1 = cvt_pk_bf16(o[2 * p][2] * rz, o[2 * p][3] * rz);
                            const uint32_t b0 = cvt_pk_bf16(o[2 * p + 1][0] * rz, o[2 * p + 1][1] * rz);
                            const uint32_t b1 = cvt_pk_bf16(o[2 * p + 1][2] * rz, o[2 * p + 1][3] * rz);
                            const uint32_t r0 = __shfl(odd ? b0 : a0, l0);
                            const uint32_t r2 = __shfl(odd ? b1 : a1, l0);
                            const uint32_t r1 = __shfl(odd ? a0 : b0, l1);
                            const uint32_t r3 = __shfl(odd ? a1 : b1, l1);
                            typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
                            const u32x4v w4 = hi ? u32x4v{r1, r3, r0, r2} : u32x4v{r0, r2, r1, r3};
                            __builtin_nontemporal_store(w4, reinterpret_cast<u32x4v*>(row + 32 * p));
                        }
                    } else {
#pragma unroll
                    for (int jb = 0; jb < C::NJ; ++jb)
                        store4<OutT>(dst + 16 * jb, o[jb][0] * rz, o[jb][1] * rz, o[jb][2] * rz,
                                     o[jb][3] * rz);
                    }
                } else {
                    float* dst = (dest < kSlots ? slots + ((tokbase + t) * kSlots + dest) * D
                                                : ovf + (rowbase + qrow) * D) + 4 * g;
#pragma unroll
                    for (int jb = 0; jb < C::NJ; ++jb)
                        store4<float>(dst + 16 * jb, o[jb][0] * rz, o[jb][1] * rz, o[jb][2] * rz,
                                      o[jb][3] * rz);
                }
            }
        }
    }
}

// float32 inputs: one wave per cluster row, vector ALU only.
template <int D, typename OutT>
__global__ __launch_bounds__(64) void cluster_attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kk, const float* __restrict__ v,
    const float* __restrict__ q_inv, const float* __restrict__ k_inv,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ idx_q,
    const uint32_t* __restrict__ mask, int n, int k, int w,
    int KW, float scale, int causal, OutT* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ slots, float* __restrict__ ovf, int32_t* __restrict__ dir) {
    __shared__ float lg[1024];
    __shared__ float lqrow[D];
    const int r = blockIdx.x, cl = blockIdx.y, bh = blockIdx.z;
    const int lane = threadIdx.x;
    const long tokbase = (long)bh * n;
    const long rowbase = ((long)bh * k + cl) * w;
    const int32_t* irow = idx + rowbase;              // keys and values
    const int raw = idx_q[rowbase + r];               // this row's query token
    const int tc = clamp_pos(raw, n);
    for (int i = lane; i < D; i += 64) lqrow[i] = q[(tokbase + tc) * D + i];
    const float qs = scale * (q_inv ? q_inv[tokbase + tc] : 1.f);
    __syncthreads();
    float m = -INFINITY;
    for (int s = lane; s < w; s += 64) {
        const int ts = clamp_pos(irow[s], n);
        float val = -INFINITY;
        if (!causal || irow[s] <= raw) {
            float dot = 0.f;
            for (int i = 0; i < D; ++i) dot = fmaf(lqrow[i], kk[(tokbase + ts) * D + i], dot);
            val = dot * qs * (k_inv ? k_inv[tokbase + ts] : 1.f);
        }
        lg[s] = val;
        m = fmaxf(m, val);
    }
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    __syncthreads();
    float z = 0.f;
    for (int s = lane; s < w; s += 64) {
        const float p = (lg[s] == -INFINITY) ? 0.f : expf(lg[s] - m);
        lg[s] = p;
        z += p;
    }
    for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
    __syncthreads();
    const bool valid = raw >= 0 && raw < n;
    const int dest = valid ? row_dest(mask + (tokbase + raw) * KW, KW, cl) : -2;
    if (dest >= kSlots && lane == 0) dir[(tokbase + raw) * (k - kSlots) + (dest - kSlots)] = cl * w + r;
    for (int i = lane; i < D; i += 64) {
        float acc = 0.f;
        if (z > 0.f) {
            for (int s = 0; s < w; ++s)
                if (lg[s] != 0.f) acc = fmaf(lg[s], v[(tokbase + clamp_pos(irow[s], n)) * D + i], acc);
            acc /= z;
        }
        if (dest == -1) Elem<OutT>::store(out, (tokbase + raw) * D + i, acc);
        else if (dest >= 0 && dest < kSlots) slots[((tokbase + raw) * kSlots + dest) * D + i] = acc;
        else if (dest >= kSlots) ovf[(rowbase + r) * D + i] = acc;
    }
    if (lane == 0 && lse != nullptr) lse[rowbase + r] = (z > 0.f) ? m + logf(z) : -INFINITY;
}

// float32 inputs: per-cluster sums of the normalised member rows.
__global__ __launch_bounds__(128) void cluster_sums_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ x_inv, const int32_t* __restrict__ idx,
    int n, int D, int k, int w, float* __restrict__ sums) {
    const int cl = blockIdx.x, bh = blockIdx.y;
    const long tokbase = (long)bh * n;
    const int32_t* irow = idx + ((long)bh * k + cl) * w;
    for (int dcol = threadIdx.x; dcol < D; dcol += 128) {
        float acc = 0.f;
        for (int r = 0; r < w; ++r) {
            const int t = clamp_pos(irow[r], n);
            acc = fmaf(x[(tokbase + t) * D + dcol], x_inv ? x_inv[tokbase + t] : 1.f, acc);
        }
        sums[((long)bh * k + cl) * D + dcol] = acc;
    }
}

// One thread per (token, 4 * kCombineQV output dims), for NO outputs sharing one
// membership (the backward's three gradients): the slots hold the rows of
// ranks 0..kSlots-1 contiguously; higher ranks are read from the overflow
// buffer at the rows the directory lists.
constexpr int kCombineQV = 2;

template <int NO>
struct CombineSet {
    const float* slots[NO];
    const float* ovf[NO];
    void* out[NO];
};

// The centroid update folded into the same launch (the workgroups past the
// combine's): mu <- lambda*mu + (1-lambda)/2 * (sum over b of sum_q + sum_k),
// one thread per centroid element, as rt_centroid_update_sums computes it.
struct FoldedEma {
    float* mu;                 // nullptr: none
    const float* sum_q;
    const float* sum_k;        // nullptr: sum_q counts twice (shared q/k)
    int B;
    long HKD;
    float lam;
    unsigned first_block;      // first workgroup of the update
};

template <typename OutT, int D, int NO>
__global__ __launch_bounds__(256) void combine_kernel(const uint32_t* __restrict__ mask,
                                                      const int32_t* __restrict__ dir,
                                                      CombineSet<NO> cs, long BHn, int n, int k,
                                                      int w, int KW, FoldedEma ema) {
    constexpr int QV = kCombineQV;               // float4 per thread and row
    constexpr int DG = D / (4 * QV);
    if (ema.mu != nullptr && blockIdx.x >= ema.first_block) {
        const long i = (long)(blockIdx.x - ema.first_block) * 256 + threadIdx.x;
        if (i >= ema.HKD) return;
        float sq = 0.f, sk = 0.f;
        for (int b = 0; b < ema.B; ++b) {
            sq += ema.sum_q[b * ema.HKD + i];
            if (ema.sum_k != nullptr) sk += ema.sum_k[b * ema.HKD + i];
        }
        const float tot = (ema.sum_k != nullptr) ? sq + sk : 2.f * sq;
        ema.mu[i] = fmaf(ema.lam, ema.mu[i], (1.0f - ema.lam) * 0.5f * tot);
        return;
    }
    // tokens of one head on one XCD, as in the attention kernel
    const long gid = (long)xcd_contiguous(blockIdx.x, ema.first_block) * 256 + threadIdx.x;
    const long tok = gid / DG;
    if (tok >= BHn) return;
    const int d0 = 4 * QV * (int)(gid % DG);
    // the token's membership words, requested together (KW <= 8; the tests
    // on KW are the same for every thread), then counted
    const uint32_t* mrow = mask + tok * KW;
    uint32_t wd[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        wd[i] = 0u;
        if (i < KW) wd[i] = mrow[i];
    }
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) cnt += __popc(wd[i]);
    if (cnt == 1) return;
    const long bhkw = (tok / n) * k * (long)w;
    const int32_t* drow = dir + tok * (k - kSlots);
#pragma unroll
    for (int o = 0; o < NO; ++o) {
        float4 p[kSlots][QV];
        const float* sp = cs.slots[o] + tok * kSlots * D + d0;
#pragma unroll
        for (int j = 0; j < kSlots; ++j)
#pragma unroll
            for (int q = 0; q < QV; ++q)
                p[j][q] = (j < cnt) ? *reinterpret_cast<const float4*>(sp + (long)j * D + 4 * q)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
        float4 acc[QV];
#pragma unroll
        for (int q = 0; q < QV; ++q) {
            acc[q] = p[0][q];
#pragma unroll
            for (int j = 1; j < kSlots; ++j) {
                acc[q].x += p[j][q].x;
                acc[q].y += p[j][q].y;
                acc[q].z += p[j][q].z;
                acc[q].w += p[j][q].w;
            }
        }
        for (int j = kSlots; j < cnt; ++j) {
            const float* op = cs.ovf[o] + (bhkw + drow[j - kSlots]) * D + d0;
#pragma unroll
            for (int q = 0; q < QV; ++q) {
                const float4 v4 = *reinterpret_cast<const float4*>(op + 4 * q);
                acc[q].x += v4.x;
                acc[q].y += v4.y;
                acc[q].z += v4.z;
                acc[q].w += v4.w;
            }
        }
        OutT* dst = static_cast<OutT*>(cs.out[o]) + tok * D + d0;
#pragma unroll
        for (int q = 0; q < QV; ++q) {
            // the finished rows are streamed past L2: nothing in this launch
            // reads them back, and no dirty lines are left for the write-back
            // at its end (bf16: the call 6.5 -> 5.8 us at 8192 x 8 heads of
            // 128; float32 gradients: the 32K-token backward call 151 -> 141
            // us; bit-identical)
            if constexpr (std::is_same<OutT, u16>::value) {
                const unsigned long long pk =
                    (unsigned long long)cvt_pk_bf16(acc[q].x, acc[q].y) |
                    ((unsigned long long)cvt_pk_bf16(acc[q].z, acc[q].w) << 32);
                __builtin_nontemporal_store(pk, reinterpret_cast<unsigned long long*>(dst + 4 * q));
            } else {
                __builtin_nontemporal_store(f32x4{acc[q].x, acc[q].y, acc[q].z, acc[q].w},
                                            reinterpret_cast<f32x4*>(dst + 4 * q));
            }
        }
    }
}

struct AttnArgs {
    const void *q, *kk, *v;
    const float *q_inv, *k_inv;
    const int32_t* idx;
    const int32_t* idx_q;   // query rows (== idx unless the queries were routed on their own)
    const uint32_t* mask;
    int BH, n, k, w, KW;
    float scale;
    int causal;
    void* out;
    float *lse, *slots, *ovf;
    int32_t* dir;
    float *sum_q, *sum_k;
};

template <int D, int WMAX, bool SHARED, typename OutT>
void launch_bf16(const AttnArgs& a, hipStream_t s) {
    using C = AttnCfg<D, WMAX, SHARED>;
    hipLaunchKernelGGL((cluster_attn_bf16_kernel<D, WMAX, SHARED, OutT>), dim3(a.k, a.BH),
                       dim3(C::NT), 0, s, (const u16*)a.q, (const u16*)a.kk, (const u16*)a.v,
                       a.q_inv, a.k_inv, a.idx, a.idx_q, a.mask, a.n, a.k, a.w, a.KW, a.scale,
                       a.causal, (OutT*)a.out, a.lse, a.slots, a.ovf, a.dir, a.sum_q, a.sum_k);
}

template <int D, bool SHARED, typename OutT>
void dispatch_w(const AttnArgs& a, hipStream_t s) {
    const int w = a.w;
    if (w <= 32) launch_bf16<D, 32, SHARED, OutT>(a, s);
    else if (w <= 64) launch_bf16<D, 64, SHARED, OutT>(a, s);
    else if (w <= 128) launch_bf16<D, 128, SHARED, OutT>(a, s);
    else {
        if constexpr (SHARED || D <= 64) {
            if (w <= 256) launch_bf16<D, 256, SHARED, OutT>(a, s);
            else {
                if constexpr (SHARED && D <= 64) launch_bf16<D, 512, SHARED, OutT>(a, s);
            }
        }
    }
}

template <int D, typename OutT>
void launch_d(const AttnArgs& a, int dtype, hipStream_t s) {
    if (dtype == 0) {
        hipLaunchKernelGGL((cluster_attn_f32_kernel<D, OutT>), dim3(a.w, a.k, a.BH), dim3(64), 0,
                           s, (const float*)a.q, (const float*)a.kk, (const float*)a.v, a.q_inv,
                           a.k_inv, a.idx, a.idx_q, a.mask, a.n, a.k, a.w, a.KW, a.scale, a.causal,
                           (OutT*)a.out, a.lse, a.slots, a.ovf, a.dir);
        if (a.sum_q)
            hipLaunchKernelGGL(cluster_sums_f32_kernel, dim3(a.k, a.BH), dim3(128), 0, s,
                               (const float*)a.q, a.q_inv, a.idx_q, a.n, D, a.k, a.w, a.sum_q);
        if (a.sum_k)
            hipLaunchKernelGGL(cluster_sums_f32_kernel, dim3(a.k, a.BH), dim3(128), 0, s,
                               (const float*)a.kk, a.k_inv, a.idx, a.n, D, a.k, a.w, a.sum_k);
    } else if (a.q == a.kk && a.q_inv == a.k_inv && a.idx_q == a.idx) {
        dispatch_w<D, true, OutT>(a, s);
    } else {
        dispatch_w<D, false, OutT>(a, s);
    }
}

template <typename OutT>
void launch_outt(const AttnArgs& a, int dtype, int d, hipStream_t s) {
    switch (d) {
        case 16: launch_d<16, OutT>(a, dtype, s); break;
        case 32: launch_d<32, OutT>(a, dtype, s); break;
        case 64: launch_d<64, OutT>(a, dtype, s); break;
        default: launch_d<128, OutT>(a, dtype, s); break;
    }
}

}  // namespace

int max_cluster_rows(int dtype, int d, bool shared_qk) {
    if (dtype == 0) return 1024;
    if (shared_qk) return d == 128 ? 256 : 512;
    return d == 128 ? 128 : 256;
}

hipError_t launch_mask(const int32_t* idx, int BH, int n, int k, int w, uint32_t* mask,
                       hipStream_t s) {
    const int KW = mask_words(k);
    const long count = (long)BH * n * KW;
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s,
                       mask, count);
    hipLaunchKernelGGL(mask_kernel, dim3((w + 255) / 256, k, BH), dim3(256), 0, s, idx, n, k, w,
                       KW, mask);
    return hipGetLastError();
}

hipError_t launch_cluster_attn(const void* q, const void* kk, const void* v, int dtype,
                               const float* q_inv, const float* k_inv, const int32_t* idx,
                               const int32_t* idx_q, const uint32_t* mask, int BH, int n, int d,
                               int k, int w, float scale, int causal, void* out, int out_dtype,
                               float* lse, float* slots, float* ovf, int32_t* dir, float* sum_q,
                               float* sum_k, hipStream_t s) {
    const AttnArgs a{q, kk, v, q_inv, k_inv, idx, idx_q ? idx_q : idx, mask, BH, n, k, w,
                     mask_words(k), scale, causal, out, lse, slots, ovf, dir, sum_q, sum_k};
    if (out_dtype == 1) launch_outt<u16>(a, dtype, d, s);
    else launch_outt<float>(a, dtype, d, s);
    return hipGetLastError();
}

template <typename OutT, int D, int NO>
void launch_combine_d(const uint32_t* mask, const int32_t* dir, const CombineSet<NO>& cs, int BH,
                      int n, int k, int w, FoldedEma ema, hipStream_t s) {
    const long BHn = (long)BH * n;
    const long threads = BHn * (D / (4 * kCombineQV));
    const unsigned comb_blocks = (unsigned)((threads + 255) / 256);
    ema.first_block = comb_blocks;
    const unsigned ema_blocks = ema.mu != nullptr ? (unsigned)((ema.HKD + 255) / 256) : 0u;
    hipLaunchKernelGGL((combine_kernel<OutT, D, NO>), dim3(comb_blocks + ema_blocks), dim3(256), 0,
                       s, mask, dir, cs, BHn, n, k, w, mask_words(k), ema);
}

template <typename OutT, int NO>
void launch_combine_t(const uint32_t* mask, const int32_t* dir, const CombineSet<NO>& cs, int BH,
                      int n, int d, int k, int w, const FoldedEma& ema, hipStream_t s) {
    switch (d) {
        case 16: launch_combine_d<OutT, 16, NO>(mask, dir, cs, BH, n, k, w, ema, s); break;
        case 32: launch_combine_d<OutT, 32, NO>(mask, dir, cs, BH, n, k, w, ema, s); break;
        case 64: launch_combine_d<OutT, 64, NO>(mask, dir, cs, BH, n, k, w, ema, s); break;
        default: launch_combine_d<OutT, 128, NO>(mask, dir, cs, BH, n, k, w, ema, s); break;
    }
}

hipError_t launch_combine(const uint32_t* mask, const float* slots, const float* ovf,
                          const int32_t* dir, int out_dtype, int BH, int n, int d, int k, int w,
                          void* out, hipStream_t s, float* mu, const float* sum_q,
                          const float* sum_k, int B, int H, float lambda) {
    const CombineSet<1> cs{{slots}, {ovf}, {out}};
    const FoldedEma ema{mu, sum_q, sum_k, B, (long)H * k * d, lambda, 0u};
    if (out_dtype == 1) launch_combine_t<u16, 1>(mask, dir, cs, BH, n, d, k, w, ema, s);
    else launch_combine_t<float, 1>(mask, dir, cs, BH, n, d, k, w, ema, s);
    return hipGetLastError();
}

hipError_t launch_combine2_f32(const uint32_t* mask, const float* const slots[2],
                               const float* const ovf[2], const int32_t* dir, int BH, int n, int d,
                               int k, int w, float* const out[2], hipStream_t s) {
    const CombineSet<2> cs{{slots[0], slots[1]}, {ovf[0], ovf[1]}, {out[0], out[1]}};
    launch_combine_t<float, 2>(mask, dir, cs, BH, n, d, k, w, FoldedEma{}, s);
    return hipGetLastError();
}

hipError_t launch_combine3_f32(const uint32_t* mask, const float* const slots[3],
                               const float* const ovf[3], const int32_t* dir, int BH, int n, int d,
                               int k, int w, float* const out[3], hipStream_t s) {
    const CombineSet<3> cs{{slots[0], slots[1], slots[2]}, {ovf[0], ovf[1], ovf[2]},
                           {out[0], out[1], out[2]}};
    launch_combine_t<float, 3>(mask, dir, cs, BH, n, d, k, w, FoldedEma{}, s);
    return hipGetLastError();
}

}  // namespace rt
