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
// Kernels
//   membership_kernel   per (batch, head, token chunk): a k-bit membership
//                       mask per token, built in LDS from the idx rows.
//   cluster_attn_bf16   one workgroup per cluster.  The w member rows of the
//                       keys (raw bf16) and of the values (transposed) are
//                       gathered into LDS once; each wave takes 16-row query
//                       blocks in a zig-zag order that balances the causal
//                       triangle, computes S^T = K Q^T with
//                       v_mfma_f32_16x16x32_bf16 (so each lane owns one query
//                       and the row statistics are per lane), applies the
//                       inverse norms and the scale in fp32, runs an online
//                       softmax over 64-key chunks, and accumulates
//                       O^T = V^T P^T with the same MFMA.
//   cluster_attn_f32    a plain vector-ALU variant for float32 inputs.
//   combine_kernel      per token: 0 if no cluster holds it; the sum of its
//                       float32 partial rows in ascending centroid order if
//                       several do.  A token held by exactly one cluster is
//                       written directly by the attention kernel.
#include "rt_common.hpp"
#include "rt_internal.hpp"

namespace rt {
namespace {

constexpr int kMaskLdsWords = 8192;  // 32 KB of membership bits per workgroup

__global__ __launch_bounds__(256) void membership_kernel(const int32_t* __restrict__ idx, int n,
                                                         int k, int w, int KW, int chunk,
                                                         uint32_t* __restrict__ mask) {
    __shared__ uint32_t lm[kMaskLdsWords];
    const int bh = blockIdx.y;
    const int t0 = blockIdx.x * chunk;
    const int tn = min(chunk, n - t0);
    for (int e = threadIdx.x; e < tn * KW; e += 256) lm[e] = 0u;
    __syncthreads();
    const int32_t* ib = idx + (long)bh * k * w;
    const int kw = k * w;
    for (int e = threadIdx.x; e < kw; e += 256) {
        const int t = ib[e];
        if (t >= t0 && t < t0 + tn) {
            const int c = e / w;
            atomicOr(&lm[(t - t0) * KW + (c >> 5)], 1u << (c & 31));
        }
    }
    __syncthreads();
    uint32_t* mb = mask + ((long)bh * n + t0) * KW;
    for (int e = threadIdx.x; e < tn * KW; e += 256) mb[e] = lm[e];
}

__device__ __forceinline__ int popcount_mask(const uint32_t* m, int KW) {
    int c = 0;
    for (int i = 0; i < KW; ++i) c += __popc(m[i]);
    return c;
}

template <int D, int WMAX, bool SHARED>
struct AttnCfg {
    static constexpr int DP = D < 32 ? 32 : D;  // dims padded to the MFMA k-depth
    static constexpr int LDX = DP + 8;          // key/query row stride in LDS (bf16)
    static constexpr int LDV = WMAX + 8;        // transposed value row stride (bf16)
    static constexpr int NS = DP / 32;          // MFMA k-steps over d
    static constexpr int NJ = D / 16;           // 16-wide output column blocks
    static constexpr int QROWS = SHARED ? 1 : WMAX;
};

template <int D, int WMAX, bool SHARED>
__global__ __launch_bounds__(256) void cluster_attn_bf16_kernel(
    const u16* __restrict__ q, const u16* __restrict__ kk, const u16* __restrict__ v,
    const float* __restrict__ q_inv, const float* __restrict__ k_inv,
    const int32_t* __restrict__ idx, const uint32_t* __restrict__ mask, int n, int k, int w,
    int KW, float scale, int causal, u16* __restrict__ out, float* __restrict__ lse,
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
    const int nthr = blockDim.x;
    const long tokbase = (long)bh * n;
    const long rowbase = ((long)bh * k + cl) * w;
    const int32_t* irow = idx + rowbase;

    for (int r = threadIdx.x; r < WMAX; r += nthr) {
        int pos = -1, posc = 0, single = 0;
        float ik = 0.f, iq = 0.f;
        if (r < w) {
            const int raw = irow[r];
            posc = clamp_pos(raw, n);
            if (raw >= 0 && raw < n) {
                pos = raw;
                single = popcount_mask(mask + (tokbase + raw) * KW, KW) == 1;
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

    // Gather the member rows (padding rows are zero).
    constexpr int CPR = C::DP / 8;
    for (int e = threadIdx.x; e < WMAX * CPR; e += nthr) {
        const int r = e / CPR, ch = e % CPR;
        uint4 xk = zero_u4(), xq = zero_u4();
        if (r < w && 8 * ch < D) {
            const long off = (tokbase + lposc[r]) * D + 8 * ch;
            xk = *reinterpret_cast<const uint4*>(kk + off);
            if (!SHARED) xq = *reinterpret_cast<const uint4*>(q + off);
        }
        *reinterpret_cast<uint4*>(&lx[r * C::LDX + 8 * ch]) = xk;
        if (!SHARED) *reinterpret_cast<uint4*>(&lq[r * C::LDX + 8 * ch]) = xq;
    }
    constexpr int DCH = D / 8;
    for (int e = threadIdx.x; e < (WMAX / 2) * DCH; e += nthr) {
        const int rp = e / DCH, ch = e % DCH;
        const int r0 = 2 * rp, r1 = r0 + 1;
        uint4 a = zero_u4(), b = zero_u4();
        if (r0 < w) a = *reinterpret_cast<const uint4*>(v + (tokbase + lposc[r0]) * D + 8 * ch);
        if (r1 < w) b = *reinterpret_cast<const uint4*>(v + (tokbase + lposc[r1]) * D + 8 * ch);
        const uint32_t* aw = reinterpret_cast<const uint32_t*>(&a);
        const uint32_t* bw = reinterpret_cast<const uint32_t*>(&b);
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            const int j = 8 * ch + 2 * e2;
            *reinterpret_cast<uint32_t*>(&lvt[j * C::LDV + r0]) =
                (aw[e2] & 0xffffu) | (bw[e2] << 16);
            *reinterpret_cast<uint32_t*>(&lvt[(j + 1) * C::LDV + r0]) =
                (aw[e2] >> 16) | (bw[e2] & 0xffff0000u);
        }
    }
    __syncthreads();

    const int lane = lane_id(), wv = threadIdx.x >> 6, NW = nthr >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int nqb = (w + 15) / 16;
    const float sl2 = scale * 1.4426950408889634f;  // logits in log2 units
    const u16* qsrc = SHARED ? lx : lq;

    for (int round = 0; round * NW < nqb; ++round) {
        const int qb = round * NW + ((round & 1) ? (NW - 1 - wv) : wv);
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
                    u16* dst = out + (tokbase + t) * D + 4 * g;
#pragma unroll
                    for (int jb = 0; jb < C::NJ; ++jb) {
                        uint2 pk;
                        pk.x = pack2(f2bf(o[jb][0] * rz), f2bf(o[jb][1] * rz));
                        pk.y = pack2(f2bf(o[jb][2] * rz), f2bf(o[jb][3] * rz));
                        *reinterpret_cast<uint2*>(dst + 16 * jb) = pk;
                    }
                } else {
                    float* dst = part + (rowbase + qrow) * D + 4 * g;
#pragma unroll
                    for (int jb = 0; jb < C::NJ; ++jb)
                        *reinterpret_cast<float4*>(dst + 16 * jb) =
                            make_float4(o[jb][0] * rz, o[jb][1] * rz, o[jb][2] * rz, o[jb][3] * rz);
                }
            }
        }
    }
}

// float32 inputs: one wave per cluster row, vector ALU only.
template <int D>
__global__ __launch_bounds__(64) void cluster_attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kk, const float* __restrict__ v,
    const float* __restrict__ q_inv, const float* __restrict__ k_inv,
    const int32_t* __restrict__ idx, const uint32_t* __restrict__ mask, int n, int k, int w,
    int KW, float scale, int causal, float* __restrict__ out, float* __restrict__ lse,
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
    const bool single = valid && popcount_mask(mask + (tokbase + raw) * KW, KW) == 1;
    for (int i = lane; i < D; i += 64) {
        float acc = 0.f;
        if (z > 0.f) {
            for (int s = 0; s < w; ++s)
                if (lg[s] != 0.f) acc = fmaf(lg[s], v[(tokbase + clamp_pos(irow[s], n)) * D + i], acc);
            acc /= z;
        }
        if (valid) {
            if (single) out[(tokbase + raw) * D + i] = acc;
            else part[(rowbase + r) * D + i] = acc;
        }
    }
    if (lane == 0 && lse != nullptr) lse[rowbase + r] = (z > 0.f) ? m + logf(z) : -INFINITY;
}

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const uint32_t* __restrict__ mask,
                                                      const int32_t* __restrict__ idx,
                                                      const float* __restrict__ part, long BHn,
                                                      int n, int D, int k, int w, int KW,
                                                      T* __restrict__ out) {
    const int DG = D / 4;
    const long gid = (long)blockIdx.x * 256 + threadIdx.x;
    const long tok = gid / DG;
    if (tok >= BHn) return;
    const int dg = (int)(gid % DG);
    const uint32_t* mrow = mask + tok * KW;
    int cnt = 0;
    for (int i = 0; i < KW; ++i) cnt += __popc(mrow[i]);
    if (cnt == 1) return;
    const int bh = (int)(tok / n), t = (int)(tok % n);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int wi = 0; wi < KW && cnt > 1; ++wi) {
        uint32_t bits = mrow[wi];
        while (bits) {
            const int c = 32 * wi + __ffs(bits) - 1;
            bits &= bits - 1u;
            const int32_t* ir = idx + ((long)bh * k + c) * w;
            int lo = 0, hi = w;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (ir[mid] < t) lo = mid + 1;
                else hi = mid;
            }
            if (lo < w && ir[lo] == t) {
                const float4 p =
                    *reinterpret_cast<const float4*>(part + (((long)bh * k + c) * w + lo) * D + 4 * dg);
                acc.x += p.x;
                acc.y += p.y;
                acc.z += p.z;
                acc.w += p.w;
            }
        }
    }
    T* dst = out + tok * D + 4 * dg;
    Elem<T>::store(dst, 0, acc.x);
    Elem<T>::store(dst, 1, acc.y);
    Elem<T>::store(dst, 2, acc.z);
    Elem<T>::store(dst, 3, acc.w);
}

template <int D, int WMAX, bool SHARED>
void launch_bf16(const void* q, const void* kk, const void* v, const float* q_inv,
                 const float* k_inv, const int32_t* idx, const uint32_t* mask, int BH, int n,
                 int k, int w, float scale, int causal, void* out, float* lse, float* part,
                 hipStream_t s) {
    const int nqb = (w + 15) / 16;
    int nw = nqb / 2;
    nw = nw < 1 ? 1 : (nw > 4 ? 4 : nw);
    hipLaunchKernelGGL((cluster_attn_bf16_kernel<D, WMAX, SHARED>), dim3(k, BH), dim3(64 * nw), 0,
                       s, (const u16*)q, (const u16*)kk, (const u16*)v, q_inv, k_inv, idx, mask,
                       n, k, w, mask_words(k), scale, causal, (u16*)out, lse, part);
}

template <int D, bool SHARED>
hipError_t dispatch_w(const void* q, const void* kk, const void* v, const float* q_inv,
                      const float* k_inv, const int32_t* idx, const uint32_t* mask, int BH, int n,
                      int k, int w, float scale, int causal, void* out, float* lse, float* part,
                      hipStream_t s) {
#define RT_LAUNCH(WM) \
    launch_bf16<D, WM, SHARED>(q, kk, v, q_inv, k_inv, idx, mask, BH, n, k, w, scale, causal, out, lse, part, s)
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
    return hipGetLastError();
}

template <int D>
void launch_f32(const void* q, const void* kk, const void* v, const float* q_inv,
                const float* k_inv, const int32_t* idx, const uint32_t* mask, int BH, int n, int k,
                int w, float scale, int causal, void* out, float* lse, float* part,
                hipStream_t s) {
    hipLaunchKernelGGL(cluster_attn_f32_kernel<D>, dim3(w, k, BH), dim3(64), 0, s,
                       (const float*)q, (const float*)kk, (const float*)v, q_inv, k_inv, idx,
                       mask, n, k, w, mask_words(k), scale, causal, (float*)out, lse, part);
}

}  // namespace

int max_cluster_rows(int dtype, int d, bool shared_qk) {
    if (dtype == 0) return 1024;
    if (shared_qk) return d == 128 ? 256 : 512;
    return d == 128 ? 128 : 256;
}

hipError_t launch_membership(const int32_t* idx, int BH, int n, int k, int w, uint32_t* mask,
                             hipStream_t s) {
    const int KW = mask_words(k);
    const int chunk = kMaskLdsWords / KW;
    hipLaunchKernelGGL(membership_kernel, dim3((n + chunk - 1) / chunk, BH), dim3(256), 0, s, idx,
                       n, k, w, KW, chunk, mask);
    return hipGetLastError();
}

hipError_t launch_cluster_attn(const void* q, const void* kk, const void* v, int dtype,
                               const float* q_inv, const float* k_inv, const int32_t* idx,
                               const uint32_t* mask, int BH, int n, int d, int k, int w,
                               float scale, int causal, void* out, float* lse, float* part,
                               hipStream_t s) {
    if (dtype == 0) {
        switch (d) {
            case 16: launch_f32<16>(q, kk, v, q_inv, k_inv, idx, mask, BH, n, k, w, scale, causal, out, lse, part, s); break;
            case 32: launch_f32<32>(q, kk, v, q_inv, k_inv, idx, mask, BH, n, k, w, scale, causal, out, lse, part, s); break;
            case 64: launch_f32<64>(q, kk, v, q_inv, k_inv, idx, mask, BH, n, k, w, scale, causal, out, lse, part, s); break;
            default: launch_f32<128>(q, kk, v, q_inv, k_inv, idx, mask, BH, n, k, w, scale, causal, out, lse, part, s); break;
        }
        return hipGetLastError();
    }
    const bool shared = (q == kk) && (q_inv == k_inv);
#define RT_DISPATCH(DD)                                                                                 \
    return shared ? dispatch_w<DD, true>(q, kk, v, q_inv, k_inv, idx, mask, BH, n, k, w, scale, causal, out, lse, part, s) \
                  : dispatch_w<DD, false>(q, kk, v, q_inv, k_inv, idx, mask, BH, n, k, w, scale, causal, out, lse, part, s)
    switch (d) {
        case 16: RT_DISPATCH(16);
        case 32: RT_DISPATCH(32);
        case 64: RT_DISPATCH(64);
        default: RT_DISPATCH(128);
    }
#undef RT_DISPATCH
}

hipError_t launch_combine(const uint32_t* mask, const int32_t* idx, const float* part, int dtype,
                          int BH, int n, int d, int k, int w, void* out, hipStream_t s) {
    const long BHn = (long)BH * n;
    const long threads = BHn * (d / 4);
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (dtype == 1)
        hipLaunchKernelGGL(combine_kernel<u16>, grid, dim3(256), 0, s, mask, idx, part, BHn, n, d,
                           k, w, mask_words(k), (u16*)out);
    else
        hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, s, mask, idx, part, BHn, n,
                           d, k, w, mask_words(k), (float*)out);
    return hipGetLastError();
}

}  // namespace rt
