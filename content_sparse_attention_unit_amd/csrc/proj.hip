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
// v_mfma_f32_16x16x32_bf16.  One workgroup = a BM x BN output tile of waves
// holding 64 x 64 blocks each (256 x 256 with sixteen waves, 128 x 256 with
// eight); K advances 64 at a time through double-buffered LDS tiles fed by
// register prefetch.  Each wave computes the transposed product
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

constexpr int PBK = 64;                          // K step
constexpr int PLD = PBK + 8;                     // LDS row stride (bf16): 144 bytes
constexpr int PCH = PBK / 8;                     // 16-byte chunks per tile row

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

// Tile shape: a BM x BN output tile per workgroup, WM x WN waves each holding
// a (BM / WM) x (BN / WN) block of 16 x 16 MFMA tiles.
template <int BM, int BN, int WM, int WN>
struct ProjCfg {
    static constexpr int NT = 64 * WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;   // one wave's block
    static constexpr int MI = TM / 16, NI = TN / 16;
    static constexpr int APT = BM * PCH / NT;          // A chunks per thread per K step
    static constexpr int WPT = BN * PCH / NT;          // W chunks per thread per K step
    static_assert(BM * PCH % NT == 0 && BN * PCH % NT == 0, "whole chunks per thread");
    static_assert(TM % 16 == 0 && TN % 16 == 0, "whole MFMA tiles per wave");
};

template <int AMODE, int CMODE, int BM, int BN, int WM, int WN, int MINB>
__global__ __launch_bounds__(64 * WM * WN, MINB) void proj_kernel(ProjArgs p) {
    using C = ProjCfg<BM, BN, WM, WN>;
    __shared__ __attribute__((aligned(16))) u16 la[2][BM * PLD];
    __shared__ __attribute__((aligned(16))) u16 lw[2][BN * PLD];

    const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
    const int lane = lane_id(), wv = wave_id();
    const int g = lane >> 4, r16 = lane & 15;
    const int wm = wv / WN, wn = wv % WN;
    const u16* w = static_cast<const u16*>(p.w);

    uint4 ra[C::APT], rw[C::WPT];
    auto load = [&](int k0) {
#pragma unroll
        for (int it = 0; it < C::APT; ++it) {
            const int e = threadIdx.x + C::NT * it;
            const int r = e / PCH, k = k0 + 8 * (e % PCH);
            ra[it] = (m0 + r < p.M && k < p.K)
                         ? *reinterpret_cast<const uint4*>(a_chunk<AMODE>(p, m0 + r, k))
                         : zero_u4();
        }
#pragma unroll
        for (int it = 0; it < C::WPT; ++it) {
            const int e = threadIdx.x + C::NT * it;
            const int r = e / PCH, k = k0 + 8 * (e % PCH);
            rw[it] = (n0 + r < p.N && k < p.K)
                         ? *reinterpret_cast<const uint4*>(w + (long)(n0 + r) * p.K + k)
                         : zero_u4();
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int it = 0; it < C::APT; ++it) {
            const int e = threadIdx.x + C::NT * it;
            *reinterpret_cast<uint4*>(&la[buf][(e / PCH) * PLD + 8 * (e % PCH)]) = ra[it];
        }
#pragma unroll
        for (int it = 0; it < C::WPT; ++it) {
            const int e = threadIdx.x + C::NT * it;
            *reinterpret_cast<uint4*>(&lw[buf][(e / PCH) * PLD + 8 * (e % PCH)]) = rw[it];
        }
    };

    // acc[ni][mi]: C^T rows n0 + TN wn + 16 ni + 4 g + i, column m0 + TM wm + 16 mi + r16
    f32x4 acc[C::NI][C::MI];
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi) acc[ni][mi] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (p.K + PBK - 1) / PBK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load((kt + 1) * PBK);
#pragma unroll
        for (int kk = 0; kk < PBK / 32; ++kk) {
            bf16x8 av[C::MI], wvv[C::NI];
#pragma unroll
            for (int i = 0; i < C::MI; ++i)
                av[i] = as_bf16x8(*reinterpret_cast<const uint4*>(
                    &la[buf][(C::TM * wm + 16 * i + r16) * PLD + 32 * kk + 8 * g]));
#pragma unroll
            for (int i = 0; i < C::NI; ++i)
                wvv[i] = as_bf16x8(*reinterpret_cast<const uint4*>(
                    &lw[buf][(C::TN * wn + 16 * i + r16) * PLD + 32 * kk + 8 * g]));
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
                for (int mi = 0; mi < C::MI; ++mi) acc[ni][mi] = mfma16(wvv[ni], av[mi], acc[ni][mi]);
        }
        if (kt + 1 < nk) {
            store(buf ^ 1);
            __syncthreads();
        }
    }

    // Epilogue: lane holds C[m][n .. n+3] for m = m0 + TM wm + 16 mi + r16,
    // n = n0 + TN wn + 16 ni + 4 g.  The residual's elements are all requested
    // first (addresses clamped into it, so no load sits under a branch), then
    // added: one memory round trip rather than one per block.
    const bool with_res = CMODE == 0 && p.res != nullptr;
    uint2 rres[C::MI][C::NI];
    if (with_res) {
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni) {
                const int m = min(m0 + C::TM * wm + 16 * mi + r16, p.M - 1);
                const int nn = min(n0 + C::TN * wn + 16 * ni + 4 * g, p.N - 4);
                rres[mi][ni] = *reinterpret_cast<const uint2*>(static_cast<const u16*>(p.res) +
                                                               (long)m * p.N + nn);
            }
    }
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
        const int m = m0 + C::TM * wm + 16 * mi + r16;
        if (m >= p.M) continue;
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni) {
            const int nn = n0 + C::TN * wn + 16 * ni + 4 * g;
            if (nn >= p.N) continue;
            float c0 = acc[ni][mi][0], c1 = acc[ni][mi][1], c2 = acc[ni][mi][2], c3 = acc[ni][mi][3];
            if constexpr (CMODE == 0) {
                const long off = (long)m * p.N + nn;
                if (with_res) {
                    const uint2 rr = rres[mi][ni];
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

// proj_dl_kernel: the same product for K a multiple of 64 (and, with
// head-major A, heads of at least 64 dims, so that every 64-wide K step lies in
// one head).  Tiles go from global memory straight into LDS
// (global_load_lds_dwordx4: lane l of a wave writes bytes 16 l .. 16 l + 15
// of the 1 KB the instruction fills), two stages deep, so no registers stage
// them and the operand fragments of the next 16-wide K slice can be read while
// the current slice's products run.  A stage keeps the 64 K elements of a row
// as two groups of four 16-byte chunks, each group a [row][4 chunks] array
// with chunk j of row r at slot j ^ ((r >> 2) & 3): one load instruction
// fills 16 rows of a group (64 contiguous bytes of each row from global
// memory), the sixteen rows one ds_read_b128 pass touches fall in sixteen
// distinct groups of four banks, and the slices of a row sit at fixed offsets
// from two per-lane addresses.  Products on v_mfma_f32_32x32x16_bf16, each
// wave holding 2 x 2 blocks of 32 x 32 (the transposed product again, four
// consecutive output columns per lane and block row).  Rows past M or N read
// the last valid row; they feed only outputs that are never stored.
constexpr int DBK = 64;                          // K per stage
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int AMODE, int CMODE, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN, 1) void proj_dl_kernel(ProjArgs p) {
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;    // one wave's block of the output
    constexpr int MI = TM / 32, NI = TN / 32;
    // load instructions per wave and stage: 16 rows of one chunk group each
    constexpr int AI = 2 * BM / (16 * NW), WI = 2 * BN / (16 * NW);
    static_assert((2 * BM) % (16 * NW) == 0 && (2 * BN) % (16 * NW) == 0, "whole loads per wave");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "whole 32 x 32 blocks per wave");
    // two stages as four separate arrays: the compiler then sees that a
    // stage's reads cannot alias the other stage's loads in flight, and does
    // not wait for those loads before reading
    __shared__ __attribute__((aligned(1024))) u16 la0[BM * DBK];
    __shared__ __attribute__((aligned(1024))) u16 lw0[BN * DBK];
    __shared__ __attribute__((aligned(1024))) u16 la1[BM * DBK];
    __shared__ __attribute__((aligned(1024))) u16 lw1[BN * DBK];

    const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
    const int lane = lane_id(), wv = wave_id();
    const int wm = wv / WN, wn = wv % WN;

    // Load instruction i of this wave fills rows 16 (u % (ROWS / 16)) .. + 15
    // of chunk group u / (ROWS / 16), u = wv * (loads per wave) + i; lane l
    // takes row + l / 4 and slot l % 4, i.e. logical chunk 4 group +
    // ((l % 4) ^ ((row >> 2) & 3)).
    const int lr = lane >> 2, ls = lane & 3;
    long aoff[AI][2];     // AMODE 0: the row's start; AMODE 1: its (b, t) part per A segment
    int acol[AI], adst[AI];
#pragma unroll
    for (int i = 0; i < AI; ++i) {
        const int u = wv * AI + i, grp = u / (BM / 16);
        const int r = 16 * (u % (BM / 16)) + lr;
        acol[i] = 8 * (4 * grp + (ls ^ ((r >> 2) & 3)));
        adst[i] = grp * BM * 32 + (r - lr) * 32;          // elements: group, then 16-row block
        const int m = min(m0 + r, p.M - 1);
        if constexpr (AMODE == 0) {
            aoff[i][0] = (long)m * p.K;
            aoff[i][1] = 0;
        } else {
            const int b = m / p.n, t = m % p.n;
            aoff[i][0] = ((long)b * p.ha[0] * p.n + t) * p.d;
            aoff[i][1] = ((long)b * p.ha[1] * p.n + t) * p.d;
        }
    }
    long woff[WI];
    int wcol[WI], wdst[WI];
#pragma unroll
    for (int i = 0; i < WI; ++i) {
        const int u = wv * WI + i, grp = u / (BN / 16);
        const int r = 16 * (u % (BN / 16)) + lr;
        wcol[i] = 8 * (4 * grp + (ls ^ ((r >> 2) & 3)));
        wdst[i] = grp * BN * 32 + (r - lr) * 32;
        woff[i] = (long)min(n0 + r, p.N - 1) * p.K;
    }
    const u16* w = static_cast<const u16*>(p.w);

    auto issue = [&](u16* la, u16* lw, int k0) {
        const u16* abase;
        int sel = 0;
        long hoff = 0;
        if constexpr (AMODE == 0) {
            abase = static_cast<const u16*>(p.a[0]) + k0;
        } else {
            const int hh = k0 / p.d, i0 = k0 % p.d;
            sel = hh < p.ha[0] ? 0 : 1;
            const int hl = sel == 0 ? hh : hh - p.ha[0];
            abase = static_cast<const u16*>(p.a[sel]) + i0;
            hoff = (long)hl * p.n * p.d;
        }
#pragma unroll
        for (int i = 0; i < AI; ++i)
            __builtin_amdgcn_global_load_lds(
                (const void*)(abase + aoff[i][AMODE == 0 ? 0 : sel] + hoff + acol[i]),
                (__attribute__((address_space(3))) void*)&la[adst[i]], 16, 0, 0);
#pragma unroll
        for (int i = 0; i < WI; ++i)
            __builtin_amdgcn_global_load_lds(
                (const void*)(w + woff[i] + k0 + wcol[i]),
                (__attribute__((address_space(3))) void*)&lw[wdst[i]], 16, 0, 0);
    };

    f32x16 acc[NI][MI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[ni][mi][e] = 0.f;

    // Fragment reads: lane l takes row l % 32 of a 32-row block and logical
    // chunk 2 s + l / 32 of the 16-wide K slice s, i.e. group s / 2, chunk
    // j = 2 (s % 2) + l / 32 at slot j ^ q with q = ((l % 32) >> 2) & 3.
    const int fr = lane & 31, fh = lane >> 5;
    const int q = (fr >> 2) & 3;
    const int fa0 = (TM * wm + fr) * 32 + 8 * (fh ^ q);     // elements, slice parity 0
    const int fa1 = (TM * wm + fr) * 32 + 8 * (fh ^ q ^ 2); // slice parity 1
    const int fw0 = (TN * wn + fr) * 32 + 8 * (fh ^ q);
    const int fw1 = (TN * wn + fr) * 32 + 8 * (fh ^ q ^ 2);
    auto frags = [&](const u16* la, const u16* lw, int s, bf16x8 (&fa)[MI], bf16x8 (&fw)[NI]) {
        const int ga = (s >> 1) * BM * 32, gw = (s >> 1) * BN * 32;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
            fa[mi] = as_bf16x8(*reinterpret_cast<const uint4*>(
                &la[((s & 1) ? fa1 : fa0) + ga + 32 * 32 * mi]));
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
            fw[ni] = as_bf16x8(*reinterpret_cast<const uint4*>(
                &lw[((s & 1) ? fw1 : fw0) + gw + 32 * 32 * ni]));
    };
    // the products of one stage, the next slice's fragments read while the
    // current slice's products run
    auto compute = [&](const u16* la, const u16* lw) {
        bf16x8 fa[2][MI], fw[2][NI];
        frags(la, lw, 0, fa[0], fw[0]);
#pragma unroll
        for (int s = 0; s < DBK / 16; ++s) {
            if (s + 1 < DBK / 16) frags(la, lw, s + 1, fa[(s + 1) & 1], fw[(s + 1) & 1]);
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    acc[ni][mi] = mfma32(fw[s & 1][ni], fa[s & 1][mi], acc[ni][mi]);
        }
        // keep that order: the first slice's reads, then each slice's
        // products behind the next slice's reads (left alone, the scheduler
        // reuses one set of fragment registers and waits for every read)
        __builtin_amdgcn_sched_group_barrier(0x100, MI + NI, 0);
#pragma unroll
        for (int s = 0; s + 1 < DBK / 16; ++s) {
            __builtin_amdgcn_sched_group_barrier(0x100, MI + NI, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, MI * NI, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, MI * NI, 0);
    };

    // Two stages a trip so that each names its arrays statically; the wait
    // and barrier after a stage's products make the next stage's loads
    // visible and free the stage just read for the loads issued next.
    const int nk = p.K / DBK;
    issue(la0, lw0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0;; kt += 2) {
        if (kt + 1 < nk) issue(la1, lw1, (kt + 1) * DBK);
        compute(la0, lw0);
        if (kt + 1 >= nk) break;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kt + 2 < nk) issue(la0, lw0, (kt + 2) * DBK);
        compute(la1, lw1);
        if (kt + 2 >= nk) break;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // Epilogue through LDS, so that every global access is a 16-byte piece of
    // a contiguous row: acc[ni][mi][4 j + i] is C[m][nn + i] for m = TM wm +
    // 32 mi + lane % 32 and nn = TN wn + 32 ni + 8 j + 4 (lane / 32) inside the
    // tile.  The stage arrays are free once every wave is past its last
    // products.
    __syncthreads();
    const int tid = threadIdx.x;
    if constexpr (CMODE == 1) {
        // head-major outputs: the tile rounded to bf16 (nothing is added), 64
        // rows per stage array, 16-byte chunk c of row r at c ^ (r & 31)
        static_assert(BM == 256 && BN == 256 && NW == 16, "head-major epilogue geometry");
        auto rows4 = [&](int q4) -> u16* { return q4 == 0 ? la0 : q4 == 1 ? lw0 : q4 == 2 ? la1 : lw1; };
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int r = TM * wm + 32 * mi + fr;
            u16* const dst = rows4(r >> 6) + (r & 63) * BN;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = (TN * wn + 32 * ni + 8 * j) >> 3;
                    *reinterpret_cast<uint2*>(dst + 8 * (c ^ (r & 31)) + 4 * fh) =
                        make_uint2(cvt_pk_bf16(acc[ni][mi][4 * j], acc[ni][mi][4 * j + 1]),
                                   cvt_pk_bf16(acc[ni][mi][4 * j + 2], acc[ni][mi][4 * j + 3]));
                }
        }
        __syncthreads();
        const int dshift = __builtin_ctz(p.d);
#pragma unroll
        for (int it = 0; it < BM * BN / 8 / (64 * NW); ++it) {
            const int e = tid + 64 * NW * it;
            const int r = e / (BN / 8), c = e % (BN / 8);
            const int m = m0 + r, nn = n0 + 8 * c;
            if (m >= p.M || nn >= p.N) continue;
            const uint4 v = *reinterpret_cast<const uint4*>(rows4(r >> 6) + (r & 63) * BN +
                                                            8 * (c ^ (r & 31)));
            int sg = 0, hl = nn >> dshift;
            while (sg < 4 && hl >= p.hc[sg]) hl -= p.hc[sg++];
            const int b = m / p.n, t = m - b * p.n;
            u16* dst = static_cast<u16*>(p.c[sg]) + (((long)b * p.hc[sg] + hl) * p.n + t) * p.d +
                       (nn & (p.d - 1));
            *reinterpret_cast<uint4*>(dst) = v;
        }
    } else {
        // row-major output, the residual added in float32 before the one
        // rounding: two passes of 64 rows (the waves of one row of waves
        // each) staged as float32, 32 rows per stage array of the weights,
        // 16-byte chunk c of row r at c ^ (r & 63)
        static_assert(BM == 128 && BN == 256 && WM == 2, "row-major epilogue geometry");
        auto half2 = [&](int q2) -> float* { return reinterpret_cast<float*>(q2 == 0 ? lw0 : lw1); };
        const u16* res = static_cast<const u16*>(p.res);
        u16* out = static_cast<u16*>(p.c[0]);
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            if (wm == pass) {
#pragma unroll
                for (int mi = 0; mi < MI; ++mi) {
                    const int r = 32 * mi + fr;                   // row inside the pass
                    float* const dst = half2(r >> 5) + (r & 31) * BN;
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int c = ((TN * wn + 32 * ni + 8 * j) >> 2) + fh;
                            *reinterpret_cast<float4*>(dst + 4 * (c ^ (r & 63))) =
                                make_float4(acc[ni][mi][4 * j], acc[ni][mi][4 * j + 1],
                                            acc[ni][mi][4 * j + 2], acc[ni][mi][4 * j + 3]);
                        }
                }
            }
            __syncthreads();
#pragma unroll
            for (int it = 0; it < 64 * BN / 8 / (64 * NW); ++it) {
                const int e = tid + 64 * NW * it;
                const int r = e / (BN / 8), c = e % (BN / 8);   // 8 columns: float4 chunks 2c, 2c + 1
                const int m = m0 + 64 * pass + r, nn = n0 + 8 * c;
                if (m >= p.M || nn >= p.N) continue;
                const float* src = half2(r >> 5) + (r & 31) * BN;
                const float4 lo = *reinterpret_cast<const float4*>(src + 4 * ((2 * c) ^ (r & 63)));
                const float4 hi = *reinterpret_cast<const float4*>(src + 4 * ((2 * c + 1) ^ (r & 63)));
                float f[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                const long off = (long)m * p.N + nn;
                if (res != nullptr) {
                    const uint4 rr = *reinterpret_cast<const uint4*>(res + off);
#pragma unroll
                    for (int q2 = 0; q2 < 8; ++q2) f[q2] += u4_elem(rr, q2);
                }
                *reinterpret_cast<uint4*>(out + off) =
                    make_uint4(cvt_pk_bf16(f[0], f[1]), cvt_pk_bf16(f[2], f[3]),
                               cvt_pk_bf16(f[4], f[5]), cvt_pk_bf16(f[6], f[7]));
            }
            if (pass == 0) __syncthreads();             // the second pass reuses the arrays
        }
    }
}

template <int AMODE, int CMODE, int BM, int BN, int WM, int WN>
void launch_proj_dl(const ProjArgs& p, hipStream_t s) {
    const dim3 grid((p.M + BM - 1) / BM, (p.N + BN - 1) / BN);
    hipLaunchKernelGGL((proj_dl_kernel<AMODE, CMODE, BM, BN, WM, WN>), grid, dim3(64 * WM * WN),
                       0, s, p);
}

template <int AMODE, int CMODE, int BM, int BN, int WM, int WN, int MINB>
void launch_proj_cfg(const ProjArgs& p, hipStream_t s) {
    const dim3 grid((p.M + BM - 1) / BM, (p.N + BN - 1) / BN);
    hipLaunchKernelGGL((proj_kernel<AMODE, CMODE, BM, BN, WM, WN, MINB>), grid, dim3(64 * WM * WN),
                       0, s, p);
}

}  // namespace

hipError_t launch_proj(const ProjArgs& p, int amode, int cmode, hipStream_t s) {
    // Measured at d_model = 1024, n = 8192, 8 + 4 heads of 128: the input
    // product (N = 3584) runs best on 256 x 256 tiles of sixteen waves (four a
    // SIMD hide the LDS and global latencies), the output product (N = 1024:
    // 256 x 256 tiles would leave half the CUs idle) on 128 x 256 tiles of
    // eight waves; 128 x 128 tiles of four waves were 19% and 14% slower.
    const bool dl = p.K % DBK == 0 && (amode == 0 || p.d >= DBK);
    if (dl && amode == 0 && cmode == 1) launch_proj_dl<0, 1, 256, 256, 4, 4>(p, s);
    else if (dl && amode == 1 && cmode == 0) launch_proj_dl<1, 0, 128, 256, 2, 4>(p, s);
    else if (dl && amode == 0 && cmode == 0) launch_proj_dl<0, 0, 128, 256, 2, 4>(p, s);
    else if (amode == 0 && cmode == 1) launch_proj_cfg<0, 1, 256, 256, 4, 4, 1>(p, s);
    else if (amode == 1 && cmode == 0) launch_proj_cfg<1, 0, 128, 256, 2, 4, 1>(p, s);
    else if (amode == 0 && cmode == 0) launch_proj_cfg<0, 0, 128, 256, 2, 4, 1>(p, s);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace rt
