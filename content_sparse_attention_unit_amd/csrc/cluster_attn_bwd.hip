// cluster_attn_bwd.hip -- backward of the in-cluster attention (gfx950).
//
// Routing attention (paperlayer.ai summary of "Efficient Content-Based Sparse
// Attention with Routing Transformers", §4) restricts the softmax attention of
// §3 to pairs of the same cluster.  For a fixed membership that layer is, per
// cluster c with members p_0 < ... < p_{w-1}, ordinary causal attention over
// the w gathered rows, so its gradient is the usual softmax-attention one:
//     P    = softmax_s(scale <q^_r, k^_s>)           (from the forward's lse)
//     dV_s = sum_r P_rs dO_r
//     dP_rs = <dO_r, v_s>,   D_r = sum_s P_rs dP_rs
//     dl_rs = P_rs (dP_rs - D_r)
//     dq^_r = scale sum_s dl_rs k^_s,   dk^_s = scale sum_r dl_rs q^_r
// and the rows of every cluster are summed back to token order.  Routing is a
// discrete choice and the centroids move by their moving average, so neither
// is differentiated.
//
// One workgroup per cluster keeps the whole cluster (raw keys/queries, values,
// output gradients) in LDS and works in two phases.
//   phase A (each lane owns a query, as in the forward): a first sweep over
//     the visible keys builds D_r; a second one forms dl^T and accumulates
//     dQ^T = K^T dl'^T with the key inverse norms folded into dl'.
//   phase B (each lane owns a key): the logits and dP are recomputed in the
//     transposed layout (S = Q K^T, dP = dO V^T) and dV^T = dO^T P,
//     dK^T = Q^T dl'' (query inverse norms folded into dl'') accumulate.
// Matrix products use v_mfma_f32_16x16x32_bf16 (P and dl rounded to bf16,
// float32 accumulation); the transposed operands come from row-major LDS
// tiles through ds_read_b64_tr_b16.  Output rows follow the forward's
// destinations: a token held by one cluster is written directly, otherwise
// its rank slot is, and the combine step sums the slots in centroid order.
// With shared queries and keys the caller may take dq^ + dk^ as one gradient
// (dk == nullptr): a wave keeps phase A's dq^ rows in registers and adds phase
// B's dk^ rows of the same block to them before the one store.
#include "rt_common.hpp"
#include "rt_internal.hpp"

namespace rt {
namespace {

template <int D, int WMAX, bool SHARED>
struct BwdCfg {
    static constexpr int DP = D < 32 ? 32 : D;
    static constexpr int LDX = DP + 16;          // odd multiple of 16 elements
    static constexpr int NS = DP / 32;
    static constexpr int NJ = D / 16;
    static constexpr int QROWS = SHARED ? 1 : WMAX;
    // waves per workgroup; sixteen from 256 rows on, where the LDS tiles allow
    // one workgroup a CU (d = 64, w = 256: 236 -> 211 us for the 32K-token call)
    static constexpr int NW = WMAX <= 32 ? 2 : (WMAX <= 64 ? 4 : (WMAX <= 128 ? 8 : 16));
    static constexpr int NT = 64 * NW;
    static constexpr int CPR = DP / 8;           // 16-byte chunks per padded row
    static constexpr int XPT = (WMAX * CPR + NT - 1) / NT;
};

// Gather the `w` member rows (row r = token irow[r]) of NX tensors into padded
// LDS tiles (rows >= w and dims >= D are zero).  The row indices are loaded
// first, all together, then every row of every tensor, through buffer
// resources of the (batch, head) slices: rows past w read as zeros from an
// offset out of range, so no load sits under a branch.  (A load under a
// branch, or one whose address needs another load, makes the compiler wait
// for every load issued before it: one memory round trip per row instead of
// two in all.)  `mid(raw)` runs before the rows are requested, with
// raw = irow[threadIdx.x] (any value when threadIdx.x >= w) loaded with the
// indices, so that its own loads join the rows' round trip; it returns a step
// that runs once every row is requested and before they are stored (the place
// to use what `mid` loaded).
template <int D, int WMAX, int NT, int LDX, int NX, typename Mid>
__device__ __forceinline__ void gather_tiles(const u16* const (&xs)[NX], long tokbase,
                                             const int32_t* __restrict__ irow, int n, int w,
                                             u16* const (&lxs)[NX], Mid&& mid) {
    constexpr int DP = D < 32 ? 32 : D;
    constexpr int CPR = DP / 8;
    constexpr int XPT = (WMAX * CPR + NT - 1) / NT;
    const buf_rsrc irs = make_rsrc(irow, 4u * (uint32_t)w);
    int tr[XPT];
#pragma unroll
    for (int it = 0; it < XPT; ++it) {
        const int r = (int)(threadIdx.x + it * NT) / CPR;
        tr[it] = (int)buffer_load_u32(irs, r < w ? 4u * r : kOutOfRange);
    }
    const int raw = (int)buffer_load_u32(irs, (int)threadIdx.x < w ? 4u * threadIdx.x : kOutOfRange);
    auto fin = mid(raw);
    uint4 t[NX][XPT];
#pragma unroll
    for (int x = 0; x < NX; ++x) {
        const buf_rsrc rs = make_rsrc(xs[x] + tokbase * D, (uint32_t)n * D * 2u);
#pragma unroll
        for (int it = 0; it < XPT; ++it) {
            const int e = threadIdx.x + it * NT;
            const int r = e / CPR, ch = e % CPR;
            t[x][it] = buffer_load16(
                rs, r < w && 8 * ch < D ? 2u * (uint32_t)(clamp_pos(tr[it], n) * D + 8 * ch) : kOutOfRange);
        }
    }
    fin();
#pragma unroll
    for (int x = 0; x < NX; ++x)
#pragma unroll
        for (int it = 0; it < XPT; ++it) {
            const int e = threadIdx.x + it * NT;
            if (e < WMAX * CPR) {
                const int r = e / CPR, ch = e % CPR;
                *reinterpret_cast<uint4*>(&lxs[x][r * LDX + 8 * ch]) = t[x][it];
            }
        }
}

// One 16 x 16 block of A B^T over d: rows of A from an LDS tile (row a0 + r16),
// B^T from this lane's registers.
template <int NS, int LDX>
__device__ __forceinline__ f32x4 block_dot(const u16* la, int a0, const uint4 (&b)[NS], int r16,
                                           int g) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(&la[(a0 + r16) * LDX + 32 * s + 8 * g]));
        acc = mfma16(a, as_bf16x8(b[s]), acc);
    }
    return acc;
}

// Write one output row (4 dims per lane per 16-dim block) to its destination.
template <int NJ>
__device__ __forceinline__ void store_row(const f32x4 (&o)[NJ], float mul, int dest, long tok,
                                          long row, int D, int g, float* __restrict__ out,
                                          float* __restrict__ slots, float* __restrict__ ovf) {
    if (dest == -2) return;
    float* dst = dest == -1 ? out + tok * D
                            : (dest < kSlots ? slots + (tok * kSlots + dest) * D : ovf + row * D);
    dst += 4 * g;
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb)
        store4<float>(dst + 16 * jb, o[jb][0] * mul, o[jb][1] * mul, o[jb][2] * mul,
                      o[jb][3] * mul);
}

struct BwdOut {
    // token order (rows of tokens held by one cluster); dk == nullptr (shared
    // q/k only): dq receives dq^ + dk^, the gradient of the shared vector
    float *dq, *dk, *dv;
    float *sq, *sk, *sv;           // rank slots
    float *oq, *ok, *ov;           // overflow ranks
    int32_t* dir;                  // overflow directory (shared by the three)
};

template <int D, int WMAX, bool SHARED>
__global__ __launch_bounds__((BwdCfg<D, WMAX, SHARED>::NT)) void cluster_attn_bwd_bf16_kernel(
    const u16* __restrict__ q, const u16* __restrict__ kk, const u16* __restrict__ v,
    const float* __restrict__ q_inv, const float* __restrict__ k_inv,
    const int32_t* __restrict__ idx, const float* __restrict__ lse,
    const u16* __restrict__ dout, const uint32_t* __restrict__ mask, int n, int k, int w,
    int KW, float scale, int causal, BwdOut out) {
    using C = BwdCfg<D, WMAX, SHARED>;
    __shared__ __attribute__((aligned(16))) u16 lk[WMAX * C::LDX];
    __shared__ __attribute__((aligned(16))) u16 lq[C::QROWS * C::LDX];
    __shared__ __attribute__((aligned(16))) u16 lv[WMAX * C::LDX];
    __shared__ __attribute__((aligned(16))) u16 ldo[WMAX * C::LDX];
    __shared__ __attribute__((aligned(16))) float linvk[WMAX];
    __shared__ __attribute__((aligned(16))) float linvq[C::QROWS];
    __shared__ __attribute__((aligned(16))) float llse[WMAX];   // log2 units; +inf on padding
    __shared__ __attribute__((aligned(16))) float lD[WMAX];
    __shared__ int ldest[WMAX];

    const int cl = blockIdx.x, bh = blockIdx.y;
    const long tokbase = (long)bh * n;
    const long rowbase = ((long)bh * k + cl) * w;
    const int32_t* irow = idx + rowbase;

    static_assert(C::NT >= WMAX, "one row per thread");
    // this thread's row: destination, inverse norms and log-denominator
    auto row_info = [&](int raw) {
        const int r = threadIdx.x;
        const bool rok = r < w, tok = rok && raw >= 0 && raw < n;
        const uint32_t toff = rok ? 4u * clamp_pos(raw, n) : kOutOfRange;
        const float ik = __uint_as_float(buffer_load_u32(
            make_rsrc(k_inv ? k_inv + tokbase : nullptr, k_inv ? 4u * n : 0u), toff));
        const float iq = __uint_as_float(buffer_load_u32(
            make_rsrc(q_inv ? q_inv + tokbase : nullptr, q_inv ? 4u * n : 0u), toff));
        const float lr = __uint_as_float(buffer_load_u32(
            make_rsrc(lse + rowbase, 4u * (uint32_t)w), rok ? 4u * r : kOutOfRange));
        uint32_t wd[8];
        load_words(make_rsrc(mask + tokbase * KW, 4u * (uint32_t)n * KW), tok, clamp_pos(raw, n),
                   KW, wd);
        return [=]() {
            int dest = -2;
            if (tok) {
                dest = dest_from_words(wd, cl, KW);
                if (dest >= kSlots)
                    out.dir[(tokbase + raw) * (k - kSlots) + (dest - kSlots)] = cl * w + r;
            }
            if (r < WMAX) {
                ldest[r] = dest;
                // absent inverse norms: the rows are unit vectors already
                linvk[r] = rok ? (k_inv ? ik : 1.f) : 0.f;
                if (!SHARED) linvq[r] = rok ? (q_inv ? iq : 1.f) : 0.f;
                llse[r] = rok ? lr * 1.4426950408889634f : INFINITY;
            }
        };
    };
    if constexpr (SHARED) {
        const u16* const xs[3] = {kk, v, dout};
        u16* const ls[3] = {lk, lv, ldo};
        gather_tiles<D, WMAX, C::NT, C::LDX, 3>(xs, tokbase, irow, n, w, ls, row_info);
    } else {
        const u16* const xs[4] = {kk, q, v, dout};
        u16* const ls[4] = {lk, lq, lv, ldo};
        gather_tiles<D, WMAX, C::NT, C::LDX, 4>(xs, tokbase, irow, n, w, ls, row_info);
    }
    __syncthreads();

    const u16* lqs = SHARED ? lk : lq;
    const float* linvqs = SHARED ? linvk : linvq;
    const int lane = lane_id(), wv = wave_id();
    const int g = lane >> 4, r16 = lane & 15;
    const int nb = (w + 15) / 16;
    const float sl2 = scale * 1.4426950408889634f;

    // With shared q/k a wave takes the same 16-row blocks in both phases, in
    // the same lane layout, so dq^ rows can wait in registers for dk^.
    const bool sum_qk = SHARED && out.dk == nullptr;
    constexpr int RMAX = (WMAX / 16 + C::NW - 1) / C::NW;   // rounds of blocks per wave
    f32x4 oa[RMAX][C::NJ];

    // ---- phase A: lanes own queries -------------------------------------------
#pragma unroll
    for (int round = 0; round < RMAX; ++round) {
        if (round * C::NW >= nb) break;
        const int qb = round * C::NW + ((round & 1) ? (C::NW - 1 - wv) : wv);
        if (qb >= nb) continue;
        const int qrow = qb * 16 + r16;
        uint4 qreg[C::NS], dreg[C::NS];
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
            qreg[s] = *reinterpret_cast<const uint4*>(&lqs[qrow * C::LDX + 32 * s + 8 * g]);
            dreg[s] = *reinterpret_cast<const uint4*>(&ldo[qrow * C::LDX + 32 * s + 8 * g]);
        }
        const float qs = sl2 * linvqs[qrow];
        const float l2 = llse[qrow];
        const int kend = causal ? min(w, qb * 16 + 16) : w;

        // sweep 1: D_r = sum_s P_rs dP_rs
        float dsum = 0.f;
        for (int kc = 0; kc < kend; kc += 64) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int key0 = kc + 16 * kb;
                if (key0 >= kend) continue;
                const f32x4 sacc = block_dot<C::NS, C::LDX>(lk, key0, qreg, r16, g);
                const f32x4 dacc = block_dot<C::NS, C::LDX>(lv, key0, dreg, r16, g);
                const float4 ik = *reinterpret_cast<const float4*>(&linvk[key0 + 4 * g]);
                const float ikv[4] = {ik.x, ik.y, ik.z, ik.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = key0 + 4 * g + i;
                    const bool ok = key < w && qrow < w && (!causal || key <= qrow);
                    const float p = ok ? __builtin_amdgcn_exp2f(sacc[i] * qs * ikv[i] - l2) : 0.f;
                    dsum = fmaf(p, dacc[i], dsum);
                }
            }
        }
        const float Dr = xor_sum_16_32(dsum);
        if (g == 0) lD[qrow] = Dr;

        // sweep 2: dQ^T += K^T (dl * k_inv)^T
        f32x4 o[C::NJ];
#pragma unroll
        for (int jb = 0; jb < C::NJ; ++jb) o[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int kc = 0; kc < kend; kc += 64) {
            uint32_t pw[4][2];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int key0 = kc + 16 * kb;
                if (key0 >= kend) {
                    pw[kb][0] = pw[kb][1] = 0u;
                    continue;
                }
                const f32x4 sacc = block_dot<C::NS, C::LDX>(lk, key0, qreg, r16, g);
                const f32x4 dacc = block_dot<C::NS, C::LDX>(lv, key0, dreg, r16, g);
                const float4 ik = *reinterpret_cast<const float4*>(&linvk[key0 + 4 * g]);
                const float ikv[4] = {ik.x, ik.y, ik.z, ik.w};
                float ds[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = key0 + 4 * g + i;
                    const bool ok = key < w && qrow < w && (!causal || key <= qrow);
                    const float p = ok ? __builtin_amdgcn_exp2f(sacc[i] * qs * ikv[i] - l2) : 0.f;
                    ds[i] = p * (dacc[i] - Dr) * ikv[i];
                }
                pw[kb][0] = cvt_pk_bf16(ds[0], ds[1]);
                pw[kb][1] = cvt_pk_bf16(ds[2], ds[3]);
            }
            acc_xt_w<C::NJ, C::LDX>(pw, o, &lk[kc * C::LDX], r16, g, 1 | ((kc + 32 < kend) ? 2 : 0));
        }
        if (sum_qk) {
#pragma unroll
            for (int jb = 0; jb < C::NJ; ++jb) oa[round][jb] = o[jb];
        } else if (qrow < w) {
            const int t = clamp_pos(irow[qrow], n);
            store_row<C::NJ>(o, scale, ldest[qrow], tokbase + t, rowbase + qrow, D, g, out.dq,
                             out.sq, out.oq);
        }
    }
    __syncthreads();   // D_r of every query is in lD

    // ---- phase B: lanes own keys ----------------------------------------------
#pragma unroll
    for (int round = 0; round < RMAX; ++round) {
        if (round * C::NW >= nb) break;
        const int kbk = round * C::NW + ((round & 1) ? (C::NW - 1 - wv) : wv);
        if (kbk >= nb) continue;
        const int key = kbk * 16 + r16;
        uint4 kreg[C::NS], vreg[C::NS];
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
            kreg[s] = *reinterpret_cast<const uint4*>(&lk[key * C::LDX + 32 * s + 8 * g]);
            vreg[s] = *reinterpret_cast<const uint4*>(&lv[key * C::LDX + 32 * s + 8 * g]);
        }
        const float ks = sl2 * linvk[key];
        f32x4 odv[C::NJ], odk[C::NJ];
#pragma unroll
        for (int jb = 0; jb < C::NJ; ++jb) {
            odv[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
            odk[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const int qstart = causal ? ((kbk * 16) & ~63) : 0;
        for (int qc = qstart; qc < w; qc += 64) {
            uint32_t pp[4][2], pd[4][2];
#pragma unroll
            for (int qb4 = 0; qb4 < 4; ++qb4) {
                const int q0 = qc + 16 * qb4;
                if (q0 >= w || (causal && q0 + 15 < kbk * 16)) {
                    pp[qb4][0] = pp[qb4][1] = pd[qb4][0] = pd[qb4][1] = 0u;
                    continue;
                }
                const f32x4 sacc = block_dot<C::NS, C::LDX>(lqs, q0, kreg, r16, g);
                const f32x4 dacc = block_dot<C::NS, C::LDX>(ldo, q0, vreg, r16, g);
                const float4 iq = *reinterpret_cast<const float4*>(&linvqs[q0 + 4 * g]);
                const float4 l4 = *reinterpret_cast<const float4*>(&llse[q0 + 4 * g]);
                const float4 d4 = *reinterpret_cast<const float4*>(&lD[q0 + 4 * g]);
                const float iqv[4] = {iq.x, iq.y, iq.z, iq.w};
                const float l4v[4] = {l4.x, l4.y, l4.z, l4.w};
                const float d4v[4] = {d4.x, d4.y, d4.z, d4.w};
                float p[4], ds[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int qi = q0 + 4 * g + i;
                    const bool ok = qi < w && key < w && (!causal || key <= qi);
                    p[i] = ok ? __builtin_amdgcn_exp2f(sacc[i] * ks * iqv[i] - l4v[i]) : 0.f;
                    ds[i] = p[i] * (dacc[i] - d4v[i]) * iqv[i];
                }
                pp[qb4][0] = cvt_pk_bf16(p[0], p[1]);
                pp[qb4][1] = cvt_pk_bf16(p[2], p[3]);
                pd[qb4][0] = cvt_pk_bf16(ds[0], ds[1]);
                pd[qb4][1] = cvt_pk_bf16(ds[2], ds[3]);
            }
            const int halves = 1 | ((qc + 32 < w) ? 2 : 0);
            acc_xt_w<C::NJ, C::LDX>(pp, odv, &ldo[qc * C::LDX], r16, g, halves);
            acc_xt_w<C::NJ, C::LDX>(pd, odk, &lqs[qc * C::LDX], r16, g, halves);
        }
        if (key < w) {
            const int t = clamp_pos(irow[key], n);
            const int dest = ldest[key];
            if (sum_qk) {        // this row's dq^ (phase A, same block, same lanes) + dk^
#pragma unroll
                for (int jb = 0; jb < C::NJ; ++jb) odk[jb] += oa[round][jb];
                store_row<C::NJ>(odk, scale, dest, tokbase + t, rowbase + key, D, g, out.dq,
                                 out.sq, out.oq);
            } else {
                store_row<C::NJ>(odk, scale, dest, tokbase + t, rowbase + key, D, g, out.dk,
                                 out.sk, out.ok);
            }
            store_row<C::NJ>(odv, 1.f, dest, tokbase + t, rowbase + key, D, g, out.dv, out.sv,
                             out.ov);
        }
    }
}

// float32 inputs (small clusters): one workgroup per cluster, vector ALU, the
// w x w probabilities and their gradients in LDS.
constexpr int kF32BwdMaxW = 64;

template <int D>
__global__ __launch_bounds__(256) void cluster_attn_bwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kk, const float* __restrict__ v,
    const float* __restrict__ q_inv, const float* __restrict__ k_inv,
    const int32_t* __restrict__ idx, const float* __restrict__ lse,
    const float* __restrict__ dout, const uint32_t* __restrict__ mask, int n, int k, int w,
    int KW, float scale, int causal, BwdOut out) {
    __shared__ float P[kF32BwdMaxW][kF32BwdMaxW];
    __shared__ float G[kF32BwdMaxW][kF32BwdMaxW];   // dP, then dl
    __shared__ float Dr[kF32BwdMaxW];
    __shared__ int tokr[kF32BwdMaxW];
    __shared__ float iqr[kF32BwdMaxW], ikr[kF32BwdMaxW];
    const int cl = blockIdx.x, bh = blockIdx.y;
    const long tokbase = (long)bh * n;
    const long rowbase = ((long)bh * k + cl) * w;
    const int32_t* irow = idx + rowbase;
    for (int r = threadIdx.x; r < w; r += 256) {
        const int t = clamp_pos(irow[r], n);
        tokr[r] = t;
        iqr[r] = q_inv ? q_inv[tokbase + t] : 1.f;
        ikr[r] = k_inv ? k_inv[tokbase + t] : 1.f;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < w * w; e += 256) {
        const int r = e / w, s = e % w;
        float p = 0.f, dp = 0.f;
        if (!causal || irow[s] <= irow[r]) {
            const float* qr = q + (tokbase + tokr[r]) * D;
            const float* ks = kk + (tokbase + tokr[s]) * D;
            const float* gr = dout + (tokbase + tokr[r]) * D;
            const float* vs = v + (tokbase + tokr[s]) * D;
            float dot = 0.f;
            for (int i = 0; i < D; ++i) {
                dot = fmaf(qr[i], ks[i], dot);
                dp = fmaf(gr[i], vs[i], dp);
            }
            p = expf(dot * scale * iqr[r] * ikr[s] - lse[rowbase + r]);
        }
        P[r][s] = p;
        G[r][s] = dp;
    }
    __syncthreads();
    for (int r = threadIdx.x; r < w; r += 256) {
        float acc = 0.f;
        for (int s = 0; s < w; ++s) acc = fmaf(P[r][s], G[r][s], acc);
        Dr[r] = acc;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < w * w; e += 256) {
        const int r = e / w, s = e % w;
        G[r][s] = P[r][s] * (G[r][s] - Dr[r]);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < w * D; e += 256) {
        const int r = e / D, i = e % D;
        const int raw = irow[r];
        if (raw < 0 || raw >= n) continue;
        float aq = 0.f, ak = 0.f, av = 0.f;
        for (int s = 0; s < w; ++s) {
            aq = fmaf(G[r][s], kk[(tokbase + tokr[s]) * D + i] * ikr[s], aq);
            ak = fmaf(G[s][r], q[(tokbase + tokr[s]) * D + i] * iqr[s], ak);
            av = fmaf(P[s][r], dout[(tokbase + tokr[s]) * D + i], av);
        }
        const int dest = row_dest(mask + (tokbase + raw) * KW, KW, cl);
        if (dest >= kSlots && i == 0)
            out.dir[(tokbase + raw) * (k - kSlots) + (dest - kSlots)] = cl * w + r;
        // dk == nullptr (shared q/k): dq receives dq^ + dk^
        const bool sum_qk = out.dk == nullptr;
        const float vals[3] = {sum_qk ? (aq + ak) * scale : aq * scale, ak * scale, av};
        float* direct[3] = {out.dq, out.dk, out.dv};
        float* slot[3] = {out.sq, out.sk, out.sv};
        float* over[3] = {out.oq, out.ok, out.ov};
        for (int j = 0; j < 3; ++j) {
            if (j == 1 && sum_qk) continue;
            if (dest == -1) direct[j][(tokbase + raw) * D + i] = vals[j];
            else if (dest < kSlots) slot[j][((tokbase + raw) * kSlots + dest) * D + i] = vals[j];
            else over[j][(rowbase + r) * D + i] = vals[j];
        }
    }
}

struct BwdArgs {
    const void *q, *kk, *v;
    const float *q_inv, *k_inv;
    const int32_t* idx;
    const float* lse;
    const void* dout;
    const uint32_t* mask;
    int BH, n, k, w, KW;
    float scale;
    int causal;
    BwdOut out;
};

template <int D, int WMAX, bool SHARED>
void launch_bwd_bf16(const BwdArgs& a, hipStream_t s) {
    using C = BwdCfg<D, WMAX, SHARED>;
    hipLaunchKernelGGL((cluster_attn_bwd_bf16_kernel<D, WMAX, SHARED>), dim3(a.k, a.BH),
                       dim3(C::NT), 0, s, (const u16*)a.q, (const u16*)a.kk, (const u16*)a.v,
                       a.q_inv, a.k_inv, a.idx, a.lse, (const u16*)a.dout, a.mask, a.n, a.k, a.w,
                       a.KW, a.scale, a.causal, a.out);
}

// Largest cluster kept in LDS (keys, [queries,] values and output gradients).
constexpr int bwd_max_rows(int D, bool shared) {
    return shared ? (D == 128 ? 128 : 256) : (D == 128 ? 64 : 128);
}

template <int D, bool SHARED>
void bwd_dispatch_w(const BwdArgs& a, hipStream_t s) {
    constexpr int kMax = bwd_max_rows(D, SHARED);
    if (a.w <= 32) launch_bwd_bf16<D, 32, SHARED>(a, s);
    else if (a.w <= 64) launch_bwd_bf16<D, 64, SHARED>(a, s);
    else {
        if constexpr (kMax >= 128) {
            if (a.w <= 128) launch_bwd_bf16<D, 128, SHARED>(a, s);
            else {
                if constexpr (kMax >= 256) launch_bwd_bf16<D, 256, SHARED>(a, s);
            }
        }
    }
}

template <int D>
void bwd_launch_d(const BwdArgs& a, int dtype, hipStream_t s) {
    if (dtype == 0) {
        hipLaunchKernelGGL((cluster_attn_bwd_f32_kernel<D>), dim3(a.k, a.BH), dim3(256), 0, s,
                           (const float*)a.q, (const float*)a.kk, (const float*)a.v, a.q_inv,
                           a.k_inv, a.idx, a.lse, (const float*)a.dout, a.mask, a.n, a.k, a.w,
                           a.KW, a.scale, a.causal, a.out);
    } else if (a.q == a.kk && a.q_inv == a.k_inv) {
        bwd_dispatch_w<D, true>(a, s);
    } else {
        bwd_dispatch_w<D, false>(a, s);
    }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
size_t bwd_mask_bytes(int BH, int n, int k) {
    return align256((size_t)BH * n * mask_words(k) * sizeof(uint32_t));
}
size_t bwd_slot_bytes(int BH, int n, int d) {
    return align256((size_t)BH * n * kSlots * d * sizeof(float));
}
size_t bwd_ovf_bytes(int BH, int d, int k, int w) {
    return align256((size_t)BH * k * w * d * sizeof(float));
}

}  // namespace

int max_cluster_rows_bwd(int dtype, int d, bool shared_qk) {
    if (dtype == 0) return kF32BwdMaxW;
    return bwd_max_rows(d, shared_qk);
}

size_t bwd_dir_bytes(int BH, int n, int k) {
    return align256((size_t)BH * n * ovf_ranks(k) * sizeof(int32_t));
}

// workspace: mask | directory | 3 x (slots | overflow)
size_t bwd_workspace_bytes(int BH, int n, int d, int k, int w) {
    return bwd_mask_bytes(BH, n, k) + bwd_dir_bytes(BH, n, k) +
           3 * (bwd_slot_bytes(BH, n, d) + bwd_ovf_bytes(BH, d, k, w));
}

hipError_t launch_cluster_attn_bwd(const void* q, const void* kk, const void* v, int dtype,
                                   const float* q_inv, const float* k_inv, const int32_t* idx,
                                   const uint32_t* member_mask, const float* lse,
                                   const void* dout, int BH, int n, int d,
                                   int k, int w, float scale, int causal, float* dq, float* dk,
                                   float* dv, void* ws, hipStream_t s) {
    char* base = static_cast<char*>(ws);
    uint32_t* mask_ws = reinterpret_cast<uint32_t*>(base);
    base += bwd_mask_bytes(BH, n, k);
    int32_t* dir = reinterpret_cast<int32_t*>(base);
    base += bwd_dir_bytes(BH, n, k);
    float* part[3][2];
    for (int j = 0; j < 3; ++j) {
        part[j][0] = reinterpret_cast<float*>(base);
        base += bwd_slot_bytes(BH, n, d);
        part[j][1] = reinterpret_cast<float*>(base);
        base += bwd_ovf_bytes(BH, d, k, w);
    }
    const uint32_t* mask = member_mask;   // the memberships rt_route produced, or built here
    if (mask == nullptr) {
        hipError_t e = launch_mask(idx, BH, n, k, w, mask_ws, s);
        if (e != hipSuccess) return e;
        mask = mask_ws;
    }
    const BwdOut out{dq, dk, dv, part[0][0], part[1][0], part[2][0],
                     part[0][1], part[1][1], part[2][1], dir};
    const BwdArgs a{q, kk, v, q_inv, k_inv, idx, lse, dout, mask, BH, n, k, w, mask_words(k),
                    scale, causal, out};
    switch (d) {
        case 16: bwd_launch_d<16>(a, dtype, s); break;
        case 32: bwd_launch_d<32>(a, dtype, s); break;
        case 64: bwd_launch_d<64>(a, dtype, s); break;
        default: bwd_launch_d<128>(a, dtype, s); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (dk == nullptr) {      // dq + dk in dq: two gradients to scatter
        float* const grads[2] = {dq, dv};
        const float* const sl[2] = {part[0][0], part[2][0]};
        const float* const ov[2] = {part[0][1], part[2][1]};
        return launch_combine2_f32(mask, sl, ov, dir, BH, n, d, k, w, grads, s);
    }
    float* const grads[3] = {dq, dk, dv};
    const float* const sl[3] = {part[0][0], part[1][0], part[2][0]};
    const float* const ov[3] = {part[0][1], part[1][1], part[2][1]};
    return launch_combine3_f32(mask, sl, ov, dir, BH, n, d, k, w, grads, s);
}

}  // namespace rt
