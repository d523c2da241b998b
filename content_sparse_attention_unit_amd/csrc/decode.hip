// decode.hip -- one generation step at a time (gfx950).
//
// The paperlayer.ai summary of "Efficient Content-Based Sparse Attention with
// Routing Transformers" (Appendix A) samples from the model one token at a
// time.  Routing attention (§4) groups queries and keys by their nearest
// shared centroid; for a single new token the balanced top-w of a whole
// sequence does not exist, so here the new token joins the one cluster whose
// centroid is nearest (largest inner product of the unit vectors, ties to the
// lower index), its raw key row, inverse norm and value are appended to that
// cluster's cache, and its query attends to every entry of that cache (all at
// earlier positions, or itself).  The local heads keep their last `window`
// keys and values in a ring (position p at slot p % window).
//
// Cluster cache per (batch, head, cluster): raw key rows [cap][d] bf16, their
// inverse norms [cap] fp32, values [cap][d] bf16, positions [cap] int32 and
// the fill count.  A prefill membership (rt_route's idx) fills it.
//
// A step has B*H independent pieces of work of a few hundred KB at most, so
// it is bound by launch latency and by the chain of dependent memory round
// trips inside one workgroup, not by HBM bandwidth.  One workgroup of 512 or
// 1024 threads per (batch, head) keeps that chain short:
//   routed: (token row, centroids, fill counts) -> (cached key rows, their
//           inverse norms, value rows) -> output: two round trips.  The new
//           entry's own logit and value come from registers and LDS, so the
//           appends are never read back inside the step.
//   local:  the ring's key and value rows do not depend on the query and are
//           loaded at once beside it: one round trip.
// The value sum runs over slots of D/4 lanes (8-byte row loads, 256/D rows a
// wave per instruction), whose partial rows are added in LDS in a fixed order.
//
// Kernels:
//   decode_fill_kernel        cache rows from a prefill membership.
//   decode_ring_fill_kernel   the local ring from the last window positions.
//   decode_routed_kernel      one routed step.
//   decode_local_kernel       one local step.
#include "rt_common.hpp"
#include "rt_internal.hpp"

namespace rt {
namespace {

// Threads a workgroup: 1024 for narrow heads; 512 from D = 64 on, where a
// thread's key row, value prefetch and query operands need more than the 128
// registers a 1024-thread workgroup leaves each thread.
template <int D>
struct Dec {
    static constexpr int kNT = D >= 64 ? 512 : 1024;
    static constexpr int kWaves = kNT / kWave;
};
constexpr float kLog2e = 1.4426950408889634f;

template <int NW>
__device__ __forceinline__ float block_sum(float x, float* red) {
    const int lane = lane_id(), wv = wave_id();
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    __syncthreads();
    if (lane == 0) red[wv] = x;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < NW; ++i) t += red[i];
    return t;
}

template <int NW>
__device__ __forceinline__ float block_max(float x, float* red) {
    const int lane = lane_id(), wv = wave_id();
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    __syncthreads();
    if (lane == 0) red[wv] = x;
    __syncthreads();
    float t = -INFINITY;
    for (int i = 0; i < NW; ++i) t = fmaxf(t, red[i]);
    return t;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// One cached key row (D bf16, 16-byte aligned) in registers.
template <int D>
struct KeyRow {
    uint4 u[D / 8];
    __device__ __forceinline__ void load(const u16* row) {
        const uint4* r = reinterpret_cast<const uint4*>(row);
#pragma unroll
        for (int i = 0; i < D / 8; ++i) u[i] = r[i];
    }
    // Row at element offset `off` from a workgroup-uniform base: a 32-bit byte
    // offset lets the loads use the scalar-base form (one address register).
    __device__ __forceinline__ void load(const u16* base, uint32_t off) {
        const char* b = reinterpret_cast<const char*>(base);
        const uint32_t byte = off * 2u;
#pragma unroll
        for (int i = 0; i < D / 8; ++i) u[i] = *reinterpret_cast<const uint4*>(b + (byte + 16u * i));
    }
    // <q, row> with q (float) in LDS.
    __device__ __forceinline__ float dot(const float* __restrict__ lq) const {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
            const float4 qa = *reinterpret_cast<const float4*>(lq + 8 * i);
            const float4 qb = *reinterpret_cast<const float4*>(lq + 8 * i + 4);
            acc = fmaf(qa.x, bf_lo(u[i].x), acc);
            acc = fmaf(qa.y, bf_hi(u[i].x), acc);
            acc = fmaf(qa.z, bf_lo(u[i].y), acc);
            acc = fmaf(qa.w, bf_hi(u[i].y), acc);
            acc = fmaf(qb.x, bf_lo(u[i].z), acc);
            acc = fmaf(qb.y, bf_hi(u[i].z), acc);
            acc = fmaf(qb.z, bf_lo(u[i].w), acc);
            acc = fmaf(qb.w, bf_hi(u[i].w), acc);
            // keep the query's LDS reads from all being hoisted into registers at once
            if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
        return acc;
    }
};

// Four bf16 at element offset `off` from a workgroup-uniform base (32-bit byte
// offset, as in KeyRow::load).
__device__ __forceinline__ uint2 load8(const u16* base, uint32_t off) {
    return *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(base) + off * 2u);
}

// The value sum over slots (see the file comment): slot `slot()` takes cached
// entries slot, slot + kSlots, ...  The first 2 * kUnroll of them are loaded
// ahead of the softmax in two halves: the first beside the key rows, the
// second once the key rows' registers are free.
template <int D, int U>
struct ValueSum {
    static constexpr int kLanes = D / 4;
    static constexpr int kPerWave = kWave / kLanes;
    static constexpr int kSlots = Dec<D>::kWaves * kPerWave;   // kSlots * D == 4 * kNT
    static constexpr int kUnroll = U;
    uint2 u[2 * kUnroll];
    __device__ __forceinline__ static int slot() { return wave_id() * kPerWave + lane_id() / kLanes; }
    __device__ __forceinline__ static int col() { return (lane_id() % kLanes) * 4; }

    // Rows are base + off(e) (element offsets below 2^32 from a base that is
    // the same for the whole workgroup).  Half h loads u[h*kUnroll ...].  The
    // loads are unconditional (entries past the last one re-read a valid row
    // and are weighted out later): predicated loads would split the code into
    // branches, at whose joins the compiler waits for every load in flight.
    template <int H, typename OffFn>
    __device__ __forceinline__ void prefetch(const u16* base, OffFn off, int Lc) {
        const int s0 = slot(), i0 = col(), last = max(Lc - 1, 0);
#pragma unroll
        for (int j = H * kUnroll; j < (H + 1) * kUnroll; ++j) {
            const int e = min(s0 + j * kSlots, last);
            u[j] = load8(base, off(e) + (uint32_t)i0);
        }
    }

    __device__ __forceinline__ static void fma4(float p, uint2 v, float& a0, float& a1, float& a2,
                                                float& a3) {
        a0 = fmaf(p, bf_lo(v.x), a0);
        a1 = fmaf(p, bf_hi(v.x), a1);
        a2 = fmaf(p, bf_lo(v.y), a2);
        a3 = fmaf(p, bf_hi(v.y), a3);
    }

    // Partial rows of sum_e p_e v_e over the cached entries into part[kSlots][D]
    // (both halves prefetched).
    template <typename OffFn>
    __device__ __forceinline__ void accumulate(const float* lp, const u16* base, OffFn off, int Lc,
                                               float* part) {
        const int s0 = slot(), i0 = col(), last = max(Lc - 1, 0);
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
        for (int j = 0; j < 2 * kUnroll; ++j) {
            const int e = s0 + j * kSlots;
            const bool ok = e < Lc;
            const float p = lp[min(e, last)];
            fma4(ok ? p : 0.f, ok ? u[j] : make_uint2(0u, 0u), a0, a1, a2, a3);
        }
        for (int e0 = s0 + 2 * kUnroll * kSlots; e0 < Lc; e0 += kUnroll * kSlots) {
#pragma unroll
            for (int j = 0; j < kUnroll; ++j) {
                const int e = e0 + j * kSlots;
                if (e < Lc) u[j] = load8(base, off(e) + (uint32_t)i0);
            }
#pragma unroll
            for (int j = 0; j < kUnroll; ++j) {
                const int e = e0 + j * kSlots;
                if (e < Lc) fma4(lp[e], u[j], a0, a1, a2, a3);
            }
        }
        *reinterpret_cast<float4*>(part + s0 * D + i0) = make_float4(a0, a1, a2, a3);
    }
};

// out[i] = (sum over slots of part[.][i] + p_new * vnew[i]) / z, slots added
// in a fixed order (four per thread, then kNT / D groups).
template <int D, typename OutT>
__device__ __forceinline__ void combine_out(float* part, float p_new, const float* vnew, float z,
                                            OutT* out) {
    constexpr int G = Dec<D>::kNT / D;
    const int i = threadIdx.x % D, g = threadIdx.x / D;
    __syncthreads();                                  // every slot's partial row is in part
    float acc = part[g * D + i];
#pragma unroll
    for (int r = 1; r < 4; ++r) acc += part[(g + r * G) * D + i];
    __syncthreads();
    part[g * D + i] = acc;
    __syncthreads();
    if (threadIdx.x < D) {
        float t = 0.f;
        for (int gg = 0; gg < G; ++gg) t += part[gg * D + i];
        t = fmaf(p_new, vnew[i], t);
        Elem<OutT>::store(out, i, t / z);
    }
}

// Softmax weights in place over lp[0..L): returns the denominator.
template <int NT>
__device__ __forceinline__ float softmax_weights(float* lp, int L, float* red) {
    float m = -INFINITY;
    for (int e = threadIdx.x; e < L; e += NT) m = fmaxf(m, lp[e]);
    m = block_max<NT / kWave>(m, red);
    float z = 0.f;
    for (int e = threadIdx.x; e < L; e += NT) {
        const float p = exp2f(lp[e] - m);
        lp[e] = p;
        z += p;
    }
    return block_sum<NT / kWave>(z, red);             // its barriers also publish lp
}

__global__ __launch_bounds__(256) void decode_fill_kernel(
    const u16* __restrict__ qk, const float* __restrict__ inv, const u16* __restrict__ v,
    const int32_t* __restrict__ idx, int n, int d, int k, int w, int cap, u16* __restrict__ ck,
    float* __restrict__ cinv, u16* __restrict__ cv, int32_t* __restrict__ cpos,
    int32_t* __restrict__ clen) {
    const int c = blockIdx.x;
    const long bh = blockIdx.y;
    const long cb = bh * k + c;                       // this cluster's cache
    for (int e = threadIdx.x; e < w * d; e += 256) {
        const int r = e / d, i = e % d;
        const int t = clamp_pos(idx[cb * w + r], n);
        ck[(cb * cap + r) * d + i] = qk[(bh * n + t) * d + i];
        cv[(cb * cap + r) * d + i] = v[(bh * n + t) * d + i];
    }
    for (int r = threadIdx.x; r < w; r += 256) {
        const int t = clamp_pos(idx[cb * w + r], n);
        cinv[cb * cap + r] = inv[bh * n + t];
        cpos[cb * cap + r] = t;
    }
    if (threadIdx.x == 0) clen[cb] = w;
}

// Slot s of the ring holds the last prefill position p < n with p % window == s.
__global__ __launch_bounds__(256) void decode_ring_fill_kernel(
    const u16* __restrict__ kk, const u16* __restrict__ v, int n, int d, int window,
    u16* __restrict__ rk, u16* __restrict__ rv) {
    const int s = blockIdx.x;
    const long bh = blockIdx.y;
    const int p = (n - 1) - (((n - 1 - s) % window) + window) % window;
    if (p < 0) return;
    for (int i = threadIdx.x; i < d; i += 256) {
        rk[(bh * window + s) * d + i] = kk[(bh * n + p) * d + i];
        rv[(bh * window + s) * d + i] = v[(bh * n + p) * d + i];
    }
}

// Arguments of one routed step (see the entry points for their layouts).
template <typename OutT>
struct RoutedStep {
    const u16* qk_t;
    const u16* v_t;
    const float* mu;
    int H, k, cap;
    u16* ck;
    float* cinv;
    u16* cv;
    int32_t* cpos;
    int32_t* clen;
    OutT* out;
    int32_t* label;
};

// Arguments of one local step.
template <typename OutT>
struct LocalStep {
    const u16* q_t;
    const u16* k_t;
    const u16* v_t;
    int window;
    u16* rk;
    u16* rv;
    OutT* out;
};

// One routed step of (batch, head) bh; lp: cap floats of LDS.
template <int D, typename OutT>
__device__ __forceinline__ void routed_step(const RoutedStep<OutT>& a, long bh, int t, float scale,
                                            float* lp) {
    const u16* __restrict__ qk_t = a.qk_t;
    const u16* __restrict__ v_t = a.v_t;
    const float* __restrict__ mu = a.mu;
    const int H = a.H, k = a.k, cap = a.cap;
    u16* __restrict__ ck = a.ck;
    float* __restrict__ cinv = a.cinv;
    u16* __restrict__ cv = a.cv;
    int32_t* __restrict__ cpos = a.cpos;
    int32_t* __restrict__ clen = a.clen;
    OutT* __restrict__ out = a.out;
    int32_t* __restrict__ label = a.label;
    constexpr int NT = Dec<D>::kNT, NW = Dec<D>::kWaves;
    constexpr int TPC = NT / 256, DPT = D / TPC;      // threads a centroid, dimensions a thread
    __shared__ __align__(16) float lx[D];
    __shared__ __align__(16) u16 lxr[D];
    __shared__ __align__(16) float lv[D];
    __shared__ __align__(16) float part[4 * NT];
    __shared__ float red[NW];
    __shared__ float bestv[NW];
    __shared__ int bestc[NW];
    __shared__ int lens[256];
    const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
    const int h = (int)(bh % H);
    // round trip 1: the token's rows, its quarter of a centroid, the fill counts
    // (every load unconditional, from in-bounds clamped indices: see ValueSum)
    const u16 xraw = qk_t[bh * D + tid % D];
    const u16 vraw = v_t[bh * D + tid % D];
    __builtin_amdgcn_sched_barrier(0);                // ahead of the loads below: LDS staging waits on them only
    const int c = tid / TPC, part_of_c = tid % TPC, cl = min(c, k - 1);
    float4 mv[DPT / 4];
    {
        const float4* m = reinterpret_cast<const float4*>(mu + ((long)h * k + cl) * D +
                                                          part_of_c * DPT);
#pragma unroll
        for (int i = 0; i < DPT / 4; ++i) mv[i] = m[i];
    }
    const int len_c = clen[bh * k + cl];
    const float xi = tid < D ? bf2f(xraw) : 0.f;
    if (tid < D) {
        lx[tid] = xi;
        lxr[tid] = xraw;
        lv[tid] = bf2f(vraw);
    }
    if (c < k && part_of_c == 0) lens[c] = len_c;
    const float inv = 1.0f / fmaxf(sqrtf(block_sum<NW>(xi * xi, red)), 1e-12f);
    // nearest centroid; ties to the lower index
    float s = -INFINITY;
    int cc = 0x7fffffff;
    if (c < k) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < DPT / 4; ++i) {
            const float4 xv = *reinterpret_cast<const float4*>(lx + part_of_c * DPT + 4 * i);
            acc = fmaf(xv.x, mv[i].x, acc);
            acc = fmaf(xv.y, mv[i].y, acc);
            acc = fmaf(xv.z, mv[i].z, acc);
            acc = fmaf(xv.w, mv[i].w, acc);
        }
#pragma unroll
        for (int off = 1; off < TPC; off <<= 1) acc += __shfl_xor(acc, off);
        s = acc * inv;
        cc = c;
    }
#pragma unroll
    for (int off = 32; off >= TPC; off >>= 1) {
        const float os = __shfl_xor(s, off);
        const int oc = __shfl_xor(cc, off);
        if (os > s || (os == s && oc < cc)) {
            s = os;
            cc = oc;
        }
    }
    if (lane == 0) {
        bestv[wv] = s;
        bestc[wv] = cc;
    }
    __syncthreads();
    float bs = bestv[0];
    int bc = bestc[0];
    for (int i = 1; i < NW; ++i)
        if (bestv[i] > bs || (bestv[i] == bs && bestc[i] < bc)) {
            bs = bestv[i];
            bc = bestc[i];
        }
    if (bc < 0 || bc >= k) bc = 0;                    // non-finite scores everywhere: stay in bounds
    const long cb = bh * k + bc;
    const int j = lens[bc];                           // the new entry's slot
    if (j < 0 || j >= cap) {                          // a full (or corrupt) cache: report, change nothing
        if (tid < D) Elem<OutT>::store(out, bh * D + tid, NAN);
        if (tid == 0 && label != nullptr) label[bh] = -1;
        return;
    }
    // round trip 2: cached value rows, key rows and their inverse norms
    const int Lc = j;                                 // cached entries; the new one is entry Lc
    const int last = max(Lc - 1, 0);
    const u16* cvb = cv + cb * cap * D;               // this cluster's value rows
    const u16* ckb = ck + cb * cap * D;
    const float* cib = cinv + cb * cap;
    auto off = [](int e) { return (uint32_t)e * D; };
    KeyRow<D> kr;
    kr.load(ckb, off(min(tid, last)));
    float kinv = cib[min(tid, last)];
    ValueSum<D, 8> vs;                                // 2 * 8 * kSlots entries ahead (256 at D = 128)
    vs.template prefetch<0>(cvb, off, Lc);
    const float sl2 = scale * inv * kLog2e;
    for (int e = tid; e <= Lc; e += NT) {             // clusters longer than NT take more passes
        // the query's LDS reads are loop-invariant: keep them from being hoisted
        // (and held, D registers) ahead of the loop
        asm volatile("" ::: "memory");
        if (e == Lc) {                                // the new entry: its row is in LDS
            kr.load(lxr);
            kinv = inv;
        }
        lp[e] = kr.dot(lx) * kinv * sl2;
        if (e + NT < Lc) {
            kr.load(ckb, off(e + NT));
            kinv = cib[e + NT];
        }
    }
    vs.template prefetch<1>(cvb, off, Lc);
    // the append (read by later steps only)
    if (tid < D) {
        ck[(cb * cap + j) * D + tid] = xraw;
        cv[(cb * cap + j) * D + tid] = vraw;
    }
    if (tid == 0) {
        cinv[cb * cap + j] = inv;
        cpos[cb * cap + j] = t;
        clen[cb] = j + 1;
        if (label != nullptr) label[bh] = bc;
    }
    const float z = softmax_weights<NT>(lp, Lc + 1, red);
    vs.accumulate(lp, cvb, off, Lc, part);
    combine_out<D, OutT>(part, lp[Lc], lv, z, out + bh * D);
}

// One local step of (batch, head) bh; lp: window floats of LDS.
template <int D, typename OutT>
__device__ __forceinline__ void local_step(const LocalStep<OutT>& a, long bh, int t, float scale,
                                           float* lp) {
    const u16* __restrict__ q_t = a.q_t;
    const u16* __restrict__ k_t = a.k_t;
    const u16* __restrict__ v_t = a.v_t;
    const int window = a.window;
    u16* __restrict__ rk = a.rk;
    u16* __restrict__ rv = a.rv;
    OutT* __restrict__ out = a.out;
    constexpr int NT = Dec<D>::kNT, NW = Dec<D>::kWaves;
    __shared__ __align__(16) float lq[D];
    __shared__ __align__(16) u16 lkr[D];
    __shared__ __align__(16) float lv[D];
    __shared__ __align__(16) float part[4 * NT];
    __shared__ float red[NW];
    const int tid = threadIdx.x;
    const int p0 = max(0, t - window + 1);
    const int Lc = t - p0;                            // ring entries before the new one
    const int s0 = p0 % window, last = max(Lc - 1, 0);
    const u16* rkb = rk + bh * window * D;            // this (batch, head)'s ring
    const u16* rvb = rv + bh * window * D;
    auto off = [&](int e) {                           // e < window: one wrap at most
        const int sl = s0 + e;
        return (uint32_t)(sl >= window ? sl - window : sl) * D;
    };
    // one round trip: the new rows, this thread's ring key row, the value prefetch
    // (every load unconditional, from in-bounds clamped indices: see ValueSum)
    const u16 qraw = q_t[bh * D + tid % D];
    const u16 kraw = k_t[bh * D + tid % D];
    const u16 vraw = v_t[bh * D + tid % D];
    __builtin_amdgcn_sched_barrier(0);                // ahead of the loads below: LDS staging waits on them only
    KeyRow<D> kr;
    kr.load(rkb, off(min(tid, last)));
    ValueSum<D, 16> vs;                               // 2 * 16 * kSlots entries ahead (512 at D = 128)
    vs.template prefetch<0>(rvb, off, Lc);
    if (tid < D) {
        lq[tid] = bf2f(qraw);
        lkr[tid] = kraw;
        lv[tid] = bf2f(vraw);
    }
    __syncthreads();
    const float sl2 = scale * kLog2e;
    for (int e = tid; e <= Lc; e += NT) {             // windows longer than NT take more passes
        asm volatile("" ::: "memory");                // as in the routed step
        if (e == Lc) kr.load(lkr);                    // the new entry: its row is in LDS
        lp[e] = kr.dot(lq) * sl2;
        if (e + NT < Lc) kr.load(rkb, off(e + NT));
    }
    vs.template prefetch<1>(rvb, off, Lc);
    // the ring write (slot t % window holds no entry of this step)
    if (tid < D) {
        rk[(bh * window + t % window) * D + tid] = kraw;
        rv[(bh * window + t % window) * D + tid] = vraw;
    }
    const float z = softmax_weights<NT>(lp, Lc + 1, red);
    vs.accumulate(lp, rvb, off, Lc, part);
    combine_out<D, OutT>(part, lp[Lc], lv, z, out + bh * D);
}

template <int D, typename OutT>
__global__ __launch_bounds__(Dec<D>::kNT) void decode_routed_kernel(RoutedStep<OutT> a, int t,
                                                                    float scale) {
    extern __shared__ float lp[];
    routed_step<D, OutT>(a, blockIdx.x, t, scale, lp);
}

template <int D, typename OutT>
__global__ __launch_bounds__(Dec<D>::kNT) void decode_local_kernel(LocalStep<OutT> a, int t,
                                                                   float scale) {
    extern __shared__ float lp[];
    local_step<D, OutT>(a, blockIdx.x, t, scale, lp);
}

}  // namespace

hipError_t launch_decode_fill(const void* qk, const float* inv, const void* v, const int32_t* idx,
                              int BH, int n, int d, int k, int w, int cap, void* ck, float* cinv,
                              void* cv, int32_t* cpos, int32_t* clen, hipStream_t s) {
    hipLaunchKernelGGL(decode_fill_kernel, dim3(k, BH), dim3(256), 0, s, (const u16*)qk, inv,
                       (const u16*)v, idx, n, d, k, w, cap, (u16*)ck, cinv, (u16*)cv, cpos, clen);
    return hipGetLastError();
}

hipError_t launch_decode_ring_fill(const void* kk, const void* v, int BH, int n, int d,
                                   int window, void* rk, void* rv, hipStream_t s) {
    hipLaunchKernelGGL(decode_ring_fill_kernel, dim3(window, BH), dim3(256), 0, s,
                       (const u16*)kk, (const u16*)v, n, d, window, (u16*)rk, (u16*)rv);
    return hipGetLastError();
}

namespace {

template <typename OutT>
RoutedStep<OutT> routed_args(const void* qk_t, const void* v_t, const float* mu, int H, int k,
                             int cap, void* ck, float* cinv, void* cv, int32_t* cpos,
                             int32_t* clen, void* out, int32_t* label) {
    return RoutedStep<OutT>{(const u16*)qk_t, (const u16*)v_t, mu, H, k, cap, (u16*)ck, cinv,
                            (u16*)cv, cpos, clen, (OutT*)out, label};
}

template <typename OutT>
LocalStep<OutT> local_args(const void* q_t, const void* k_t, const void* v_t, int window, void* rk,
                           void* rv, void* out) {
    return LocalStep<OutT>{(const u16*)q_t, (const u16*)k_t, (const u16*)v_t, window, (u16*)rk,
                           (u16*)rv, (OutT*)out};
}

// Expands LAUNCH(D, OutT) for the supported widths and output types.
#define RT_DECODE_DISPATCH(d, out_dtype, LAUNCH)                 \
    switch (d) {                                                 \
        case 16:                                                 \
            if (out_dtype == 1) LAUNCH(16, u16); else LAUNCH(16, float); \
            break;                                               \
        case 32:                                                 \
            if (out_dtype == 1) LAUNCH(32, u16); else LAUNCH(32, float); \
            break;                                               \
        case 64:                                                 \
            if (out_dtype == 1) LAUNCH(64, u16); else LAUNCH(64, float); \
            break;                                               \
        case 128:                                                \
            if (out_dtype == 1) LAUNCH(128, u16); else LAUNCH(128, float); \
            break;                                               \
        default:                                                 \
            return hipErrorInvalidValue;                         \
    }

}  // namespace

hipError_t launch_decode_routed(const void* qk_t, const void* v_t, const float* mu, int BH, int H,
                                int d, int k, int cap, void* ck, float* cinv, void* cv,
                                int32_t* cpos, int32_t* clen, int t, float scale, void* out,
                                int out_dtype, int32_t* label, hipStream_t s) {
    const size_t lds = (size_t)cap * sizeof(float);
#define RT_LAUNCH(D, O)                                                                         \
    hipLaunchKernelGGL((decode_routed_kernel<D, O>), dim3(BH), dim3(Dec<D>::kNT), lds, s,      \
                       routed_args<O>(qk_t, v_t, mu, H, k, cap, ck, cinv, cv, cpos, clen, out,  \
                                      label),                                                   \
                       t, scale)
    RT_DECODE_DISPATCH(d, out_dtype, RT_LAUNCH)
#undef RT_LAUNCH
    return hipGetLastError();
}

hipError_t launch_decode_local(const void* q_t, const void* k_t, const void* v_t, int BH, int d,
                               int window, void* rk, void* rv, int t, float scale, void* out,
                               int out_dtype, hipStream_t s) {
    const size_t lds = (size_t)window * sizeof(float);
#define RT_LAUNCH(D, O)                                                                         \
    hipLaunchKernelGGL((decode_local_kernel<D, O>), dim3(BH), dim3(Dec<D>::kNT), lds, s,       \
                       local_args<O>(q_t, k_t, v_t, window, rk, rv, out), t, scale)
    RT_DECODE_DISPATCH(d, out_dtype, RT_LAUNCH)
#undef RT_LAUNCH
    return hipGetLastError();
}

#undef RT_DECODE_DISPATCH

}  // namespace rt
