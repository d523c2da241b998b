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
// Kernels (in launch order)
//   zero_u32_kernel     clears the per-token membership counters.
//   membership_kernel   one thread per membership (c, r): bumps the token's
//                       counter and appends c*w + r to the token's list.  The
//                       list order is arbitrary; readers sort it.
//   cluster_attn_bf16   one workgroup per cluster.  The w member rows of the
//                       keys (raw bf16) and of the values (transposed) are
//                       gathered into LDS once, with every load of a thread
//                       issued before the first LDS store; each wave takes
//                       16-row query blocks in a zig-zag order that balances
//                       the causal triangle, computes S^T = K Q^T with
//                       v_mfma_f32_16x16x32_bf16 (each lane owns one query,
//                       so row statistics are per lane), applies the inverse
//                       norms and the scale in fp32, runs an online softmax
//                       over 64-key chunks and accumulates O^T = V^T P^T with
//                       the same MFMA.  A row whose token belongs to this
//                       cluster only is written straight to `out`; otherwise
//                       the fp32 row goes to the partial buffer.
//   cluster_attn_f32    a plain vector-ALU variant for float32 inputs.
//   combine_kernel      per token: 0 if no cluster holds it; the sum of its
//                       fp32 partial rows in ascending centroid order if
//                       several do (deterministic); nothing if one does.
#include "rt_common.hpp"
#include "rt_internal.hpp"

namespace rt {
namespace {

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* __restrict__ p, long count) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i < count) p[i] = 0u;
}

// grid (ceil(w / 256), k, BH)
__global__ __launch_bounds__(256) void membership_kernel(const int32_t* __restrict__ idx, int n,
                                                         int k, int w,
                                                         uint32_t* __restrict__ cnt,
                                                         int32_t* __restrict__ list) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    const int c = blockIdx.y, bh = blockIdx.z;
    if (r >= w) return;
    const int t = idx[((long)bh * k + c) * w + r];
    if (t < 0 || t >= n) return;
    const long tok = (long)bh * n + t;
    const uint32_t slot = atomicAdd(&cnt[tok], 1u);
    if (slot < (uint32_t)k) list[tok * k + slot] = c * w + r;
}

template <typename OutT>
__device__ __forceinline__ void store4(OutT* dst, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<u16>(u16* dst, float a, float b, float c, float d) {
    uint2 pk;
    pk.x = pack2(f2bf(a), f2bf(b));
    pk.y = pack2(f2bf(c), f2bf(d));
    *reinterpret_cast<uint2*>(dst) = pk;
}
template <>
__device__ __forceinline__ void store4<float>(float* dst, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}

template <int D, int WMAX, bool SHARED>
struct AttnCfg {
    static constexpr int DP = D < 32 ? 32 : D;  // dims padded to the MFMA k-depth
    static constexpr int LDX = DP + 8;          // key/query row stride in LDS (bf16)
    static constexpr int LDV = WMAX + 8;        // transposed value row stride (bf16)
    static constexpr int NS = DP / 32;          // MFMA k-steps over d
    static constexpr int NJ = D / 16;           // 16-wide output column blocks
    static constexpr int QROWS = SHARED ? 1 : WMAX;
    static constexpr int NW = WMAX <= 32 ? 1 : (WMAX <= 64 ? 2 : 4);  // waves per workgroup
    static constexpr int NT = 64 * NW;
    static constexpr int CPR = DP / 8;          // 16-byte chunks per padded key row
    static constexpr int XPT = (WMAX * CPR + NT - 1) / NT;         // key chunks per thread
    static constexpr int DCH = D / 8;           // 16-byte chunks per value row
    static constexpr int VPT = ((WMAX / 2) * DCH + NT - 1) / NT;   // value row-pair chunks per thread
};

template <int D, int WMAX, bool SHARED, typename OutT>
__global__ __launch_bounds__((AttnCfg<D, WMAX, SHARED>::NT)) void cluster_attn_bf16_kernel(
    const u16* __restrict__ q, const u16* __restrict__ kk, const u16* __restrict__ v,
    const float* __restrict__ q_inv, const float* __restrict__ k_inv,
    const int32_t* __restrict__ idx, const uint32_t* __restrict__ cnt, int n, int k, int w,
    float scale, int causal, OutT* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part) {
    using C = AttnCfg<D, WMAX, SHARED>;
    __shared__ __attribute__((aligned(16))) u16 lx[WMAX * C::LDX];
    __shared__ __attribute__((aligned(16))) u16 lq[C::QROWS * C::LDX];
    __shared__ __attribute__((aligned(16))) u16 lvt[D * C::LDV];
    __shared__ __attribute__((aligned(16))) float linvk[WMAX];
    __shared__ __attribute__((aligned(16))) float linvq[C::QROWS];
    __shared__ int lposc[WMAX];   // clamped position (safe to dereference)
    __shared__ int lpos[WMAX];    // position, or -1 when the row is padding / invalid
    __shared__ int lsingle[WMAX]; // 1 when exactly one cluster holds the token

    const int cl = blockIdx.x, bh = blockIdx.y;
    const long tokbase = (long)bh * n;
    const long rowbase = ((long)bh * k + cl) * w;
    const int32_t* irow = idx + rowbase;

    for (int r = threadIdx.x; r < WMAX; r += C::NT) {
        int pos = -1, posc = 0, single = 0;
        float ik = 0.f, iq = 0.f;
        if (r < w) {
            const int raw = irow[r];
            posc = clamp_pos(raw, n);
            if (raw >= 0 && raw < n) {
                pos = raw;
                single = cnt[tokbase + raw] == 1u;
            }
            ik = k_inv ? k_inv[tokbase + posc] : 1.f;
            iq = q_inv ? q_inv[tokbase + posc] : 1.f;
        }
        lpos[r] = pos;
        lposc[r] = posc;
        lsingle[r] = single;
        linvk[r] = ik;
        if (!SHARED) linvq[r] = iq;
    }
    __syncthreads();

    // Gather the member rows (padding rows are zero): all loads first.
    {
        uint4 xk[C::XPT], xq[SHARED ? 1 : C::XPT];
#pragma unroll
        for (int it = 0; it < C::XPT; ++it) {
            const int e = threadIdx.x + it * C::NT;
            const int r = e / C::CPR, ch = e % C::CPR;
            xk[it] = zero_u4();
            if (!SHARED) xq[it] = zero_u4();
            if (r < w && 8 * ch < D) {
                const long off = (tokbase + lposc[r]) * D + 8 * ch;
                xk[it] = *reinterpret_cast<const uint4*>(kk + off);
                if (!SHARED) xq[it] = *reinterpret_cast<const uint4*>(q + off);
            }
        }
        uint4 va[C::VPT], vb[C::VPT];
#pragma unroll
        for (int it = 0; it < C::VPT; ++it) {
            const int e = threadIdx.x + it * C::NT;
            const int rp = e / C::DCH, ch = e % C::DCH;
            const int r0 = 2 * rp;
            va[it] = zero_u4();
            vb[it] = zero_u4();
            if (r0 < w) va[it] = *reinterpret_cast<const uint4*>(v + (tokbase + lposc[r0]) * D + 8 * ch);
            if (r0 + 1 < w)
                vb[it] = *reinterpret_cast<const uint4*>(v + (tokbase + lposc[r0 + 1]) * D + 8 * ch);
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
#pragma unroll
        for (int it = 0; it < C::VPT; ++it) {
            const int e = threadIdx.x + it * C::NT;
            if (e < (WMAX / 2) * C::DCH) {
                const int rp = e / C::DCH, ch = e % C::DCH;
                const int r0 = 2 * rp;
                const uint32_t* aw = reinterpret_cast<const uint32_t*>(&va[it]);
                const uint32_t* bw = reinterpret_cast<const uint32_t*>(&vb[it]);
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const int j = 8 * ch + 2 * e2;
                    *reinterpret_cast<uint32_t*>(&lvt[j * C::LDV + r0]) =
                        (aw[e2] & 0xffffu) | (bw[e2] << 16);
                    *reinterpret_cast<uint32_t*>(&lvt[(j + 1) * C::LDV + r0]) =
                        (aw[e2] >> 16) | (bw[e2] & 0xffff0000u);
                }
            }
        }
    }
    __syncthreads();

    const int lane = lane_id(), wv = threadIdx.x >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int nqb = (w + 15) / 16;
    const float sl2 = scale * 1.4426950408889634f;  // logits in log2 units
    const u16* qsrc = SHARED ? lx : lq;

    for (int round = 0; round * C::NW < nqb; ++round) {
        const int qb = round * C::NW + ((round & 1) ? (C::NW - 1 - wv) : wv);
        if (qb >= nqb) continue;
        const int qrow = qb * 16 + r16;
        uint4 qreg[C::NS];
#pragma unroll
        for (int s = 0; s < C::NS; ++s)
            qreg[s] = *reinterpret_cast<const uint4*>(&qsrc[qrow * C::LDX + 32 * s + 8 * g]);
        const float qs = sl2 * (SHARED ? linvk[qrow] : linvq[qrow]);

        f32x4 o[C::NJ];
#pragma unroll
        for (int jb = 0; jb < C::NJ; ++jb) o[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m = -INFINITY, z = 0.f;
        const int kend = causal ? min(w, qb * 16 + 16) : w;

        for (int kc = 0; kc < kend; kc += 64) {
            f32x4 sv[4];
            float cmax = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int key0 = kc + 16 * kb;
                sv[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (key0 < kend) {
#pragma unroll
                    for (int s = 0; s < C::NS; ++s) {
                        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(
                            &lx[(key0 + r16) * C::LDX + 32 * s + 8 * g]));
                        sv[kb] = mfma16(a, as_bf16x8(qreg[s]), sv[kb]);
                    }
                    const float4 ik = *reinterpret_cast<const float4*>(&linvk[key0 + 4 * g]);
                    const float ikv[4] = {ik.x, ik.y, ik.z, ik.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = key0 + 4 * g + i;
                        const bool ok = key < w && (!causal || key <= qrow);
                        sv[kb][i] = ok ? sv[kb][i] * qs * ikv[i] : -INFINITY;
                        cmax = fmaxf(cmax, sv[kb][i]);
                    }
                } else {
                    sv[kb] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
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
                if (kc + 32 * mm < kend) {
                    uint4 pw;
                    pw.x = pack2(pb[2 * mm][0], pb[2 * mm][1]);
                    pw.y = pack2(pb[2 * mm][2], pb[2 * mm][3]);
                    pw.z = pack2(pb[2 * mm + 1][0], pb[2 * mm + 1][1]);
                    pw.w = pack2(pb[2 * mm + 1][2], pb[2 * mm + 1][3]);
                    const bf16x8 pbv = as_bf16x8(pw);
#pragma unroll
                    for (int jb = 0; jb < C::NJ; ++jb) {
                        const u16* vr = &lvt[(16 * jb + r16) * C::LDV + kc + 32 * mm + 4 * g];
                        const uint2 lo = *reinterpret_cast<const uint2*>(vr);
                        const uint2 hi = *reinterpret_cast<const uint2*>(vr + 16);
                        o[jb] = mfma16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pbv, o[jb]);
                    }
                }
            }
        }

        const float zt = xor_sum_16_32(z);
        const float rz = 1.0f / zt;
        if (qrow < w) {
            if (g == 0 && lse != nullptr)
                lse[rowbase + qrow] = (m + __log2f(zt)) * 0.6931471805599453f;
            const int t = lpos[qrow];
            if (t >= 0) {
                if (lsingle[qrow]) {
                    OutT* dst = out + (tokbase + t) * D + 4 * g;
#pragma unroll
                    for (int jb = 0; jb < C::NJ; ++jb)
                        store4<OutT>(dst + 16 * jb, o[jb][0] * rz, o[jb][1] * rz, o[jb][2] * rz,
                                     o[jb][3] * rz);
                } else {
                    float* dst = part + (rowbase + qrow) * D + 4 * g;
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
    const int32_t* __restrict__ idx, const uint32_t* __restrict__ cnt, int n, int k, int w,
    float scale, int causal, OutT* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part) {
    __shared__ float lg[1024];
    __shared__ float lqrow[D];
    const int r = blockIdx.x, cl = blockIdx.y, bh = blockIdx.z;
    const int lane = threadIdx.x;
    const long tokbase = (long)bh * n;
    const long rowbase = ((long)bh * k + cl) * w;
    const int32_t* irow = idx + rowbase;
    const int raw = irow[r];
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
    const bool single = valid && cnt[tokbase + raw] == 1u;
    for (int i = lane; i < D; i += 64) {
        float acc = 0.f;
        if (z > 0.f) {
            for (int s = 0; s < w; ++s)
                if (lg[s] != 0.f) acc = fmaf(lg[s], v[(tokbase + clamp_pos(irow[s], n)) * D + i], acc);
            acc /= z;
        }
        if (valid) {
            if (single) Elem<OutT>::store(out, (tokbase + raw) * D + i, acc);
            else part[(rowbase + r) * D + i] = acc;
        }
    }
    if (lane == 0 && lse != nullptr) lse[rowbase + r] = (z > 0.f) ? m + logf(z) : -INFINITY;
}

// One thread per (token, 4 output dims).  The token's list entries c*w + r
// are visited in increasing order (selection over the short list), so the
// sum runs in ascending centroid order whatever order the list was filled in.
template <typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(const uint32_t* __restrict__ cnt,
                                                      const int32_t* __restrict__ list,
                                                      const float* __restrict__ part, long BHn,
                                                      int n, int D, int k, int w,
                                                      OutT* __restrict__ out) {
    const int DG = D / 4;
    const long gid = (long)blockIdx.x * 256 + threadIdx.x;
    const long tok = gid / DG;
    if (tok >= BHn) return;
    const int dg = (int)(gid % DG);
    const uint32_t c_tok = cnt[tok];
    if (c_tok == 1u) return;
    const int m = (int)min(c_tok, (uint32_t)k);
    const long bh = tok / n;
    const int32_t* lst = list + tok * k;
    const float* pbase = part + bh * (long)k * w * D + 4 * dg;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int prev = -1;
    for (int j = 0; j < m; ++j) {
        int best = 0x7fffffff;
        for (int i = 0; i < m; ++i) {
            const int e = lst[i];
            if (e > prev && e < best) best = e;
        }
        prev = best;
        const float4 p = *reinterpret_cast<const float4*>(pbase + (long)best * D);
        acc.x += p.x;
        acc.y += p.y;
        acc.z += p.z;
        acc.w += p.w;
    }
    store4<OutT>(out + tok * D + 4 * dg, acc.x, acc.y, acc.z, acc.w);
}

template <int D, int WMAX, bool SHARED, typename OutT>
void launch_bf16(const void* q, const void* kk, const void* v, const float* q_inv,
                 const float* k_inv, const int32_t* idx, const uint32_t* cnt, int BH, int n,
                 int k, int w, float scale, int causal, void* out, float* lse, float* part,
                 hipStream_t s) {
    using C = AttnCfg<D, WMAX, SHARED>;
    hipLaunchKernelGGL((cluster_attn_bf16_kernel<D, WMAX, SHARED, OutT>), dim3(k, BH),
                       dim3(C::NT), 0, s, (const u16*)q, (const u16*)kk, (const u16*)v, q_inv,
                       k_inv, idx, cnt, n, k, w, scale, causal, (OutT*)out, lse, part);
}

template <int D, bool SHARED, typename OutT>
void dispatch_w(const void* q, const void* kk, const void* v, const float* q_inv,
                const float* k_inv, const int32_t* idx, const uint32_t* cnt, int BH, int n, int k,
                int w, float scale, int causal, void* out, float* lse, float* part,
                hipStream_t s) {
#define RT_LAUNCH(WM)                                                                          \
    launch_bf16<D, WM, SHARED, OutT>(q, kk, v, q_inv, k_inv, idx, cnt, BH, n, k, w, scale,     \
                                     causal, out, lse, part, s)
    if (w <= 32) RT_LAUNCH(32);
    else if (w <= 64) RT_LAUNCH(64);
    else if (w <= 128) RT_LAUNCH(128);
    else {
        if constexpr (SHARED || D <= 64) {
            if (w <= 256) RT_LAUNCH(256);
            else {
                if constexpr (SHARED && D <= 64) RT_LAUNCH(512);
            }
        }
    }
#undef RT_LAUNCH
}

template <int D, typename OutT>
void launch_f32(const void* q, const void* kk, const void* v, const float* q_inv,
                const float* k_inv, const int32_t* idx, const uint32_t* cnt, int BH, int n, int k,
                int w, float scale, int causal, void* out, float* lse, float* part,
                hipStream_t s) {
    hipLaunchKernelGGL((cluster_attn_f32_kernel<D, OutT>), dim3(w, k, BH), dim3(64), 0, s,
                       (const float*)q, (const float*)kk, (const float*)v, q_inv, k_inv, idx,
                       cnt, n, k, w, scale, causal, (OutT*)out, lse, part);
}

template <int D, typename OutT>
void launch_d(const void* q, const void* kk, const void* v, int dtype, const float* q_inv,
              const float* k_inv, const int32_t* idx, const uint32_t* cnt, int BH, int n, int k,
              int w, float scale, int causal, void* out, float* lse, float* part,
              hipStream_t s) {
    if (dtype == 0) {
        launch_f32<D, OutT>(q, kk, v, q_inv, k_inv, idx, cnt, BH, n, k, w, scale, causal, out,
                            lse, part, s);
    } else if (q == kk && q_inv == k_inv) {
        dispatch_w<D, true, OutT>(q, kk, v, q_inv, k_inv, idx, cnt, BH, n, k, w, scale, causal,
                                  out, lse, part, s);
    } else {
        dispatch_w<D, false, OutT>(q, kk, v, q_inv, k_inv, idx, cnt, BH, n, k, w, scale, causal,
                                   out, lse, part, s);
    }
}

template <typename OutT>
void launch_outt(const void* q, const void* kk, const void* v, int dtype, const float* q_inv,
                 const float* k_inv, const int32_t* idx, const uint32_t* cnt, int BH, int n,
                 int d, int k, int w, float scale, int causal, void* out, float* lse,
                 float* part, hipStream_t s) {
    switch (d) {
        case 16: launch_d<16, OutT>(q, kk, v, dtype, q_inv, k_inv, idx, cnt, BH, n, k, w, scale, causal, out, lse, part, s); break;
        case 32: launch_d<32, OutT>(q, kk, v, dtype, q_inv, k_inv, idx, cnt, BH, n, k, w, scale, causal, out, lse, part, s); break;
        case 64: launch_d<64, OutT>(q, kk, v, dtype, q_inv, k_inv, idx, cnt, BH, n, k, w, scale, causal, out, lse, part, s); break;
        default: launch_d<128, OutT>(q, kk, v, dtype, q_inv, k_inv, idx, cnt, BH, n, k, w, scale, causal, out, lse, part, s); break;
    }
}

}  // namespace

int max_cluster_rows(int dtype, int d, bool shared_qk) {
    if (dtype == 0) return 1024;
    if (shared_qk) return d == 128 ? 256 : 512;
    return d == 128 ? 128 : 256;
}

hipError_t launch_membership(const int32_t* idx, int BH, int n, int k, int w, uint32_t* cnt,
                             int32_t* list, hipStream_t s) {
    const long count = (long)BH * n;
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s,
                       cnt, count);
    hipLaunchKernelGGL(membership_kernel, dim3((w + 255) / 256, k, BH), dim3(256), 0, s, idx, n,
                       k, w, cnt, list);
    return hipGetLastError();
}

hipError_t launch_cluster_attn(const void* q, const void* kk, const void* v, int dtype,
                               const float* q_inv, const float* k_inv, const int32_t* idx,
                               const uint32_t* cnt, int BH, int n, int d, int k, int w,
                               float scale, int causal, void* out, int out_dtype, float* lse,
                               float* part, hipStream_t s) {
    if (out_dtype == 1)
        launch_outt<u16>(q, kk, v, dtype, q_inv, k_inv, idx, cnt, BH, n, d, k, w, scale, causal,
                         out, lse, part, s);
    else
        launch_outt<float>(q, kk, v, dtype, q_inv, k_inv, idx, cnt, BH, n, d, k, w, scale,
                           causal, out, lse, part, s);
    return hipGetLastError();
}

hipError_t launch_combine(const uint32_t* cnt, const int32_t* list, const float* part,
                          int out_dtype, int BH, int n, int d, int k, int w, void* out,
                          hipStream_t s) {
    const long BHn = (long)BH * n;
    const long threads = BHn * (d / 4);
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (out_dtype == 1)
        hipLaunchKernelGGL(combine_kernel<u16>, grid, dim3(256), 0, s, cnt, list, part, BHn, n, d,
                           k, w, (u16*)out);
    else
        hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, s, cnt, list, part, BHn, n,
                           d, k, w, (float*)out);
    return hipGetLastError();
}

}  // namespace rt
