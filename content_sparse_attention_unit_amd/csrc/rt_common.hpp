// rt_common.hpp -- device helpers shared by the gfx950 kernels of the routed
// attention library.  Only this library includes it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int kWave = 64;

// ---- bfloat16 <-> float32 ----------------------------------------------------
__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float((uint32_t)b << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two float32 -> packed bf16 (a in the low half), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Round to nearest even (NaN stays NaN).
__device__ __forceinline__ u16 f2bf(float f) { return (u16)(cvt_pk_bf16(f, 0.f) & 0xffffu); }

// 8 bf16 values packed in a uint4 (16 bytes) <-> MFMA operand.
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint4 zero_u4() { return make_uint4(0u, 0u, 0u, 0u); }

// Unpack the i-th bf16 of a uint4 to float.
__device__ __forceinline__ float u4_elem(const uint4& v, int i) {
    uint32_t word = (i < 2) ? v.x : (i < 4) ? v.y : (i < 6) ? v.z : v.w;
    return bf2f((u16)((i & 1) ? (word >> 16) : (word & 0xffffu)));
}

__device__ __forceinline__ uint32_t pack2(u16 lo, u16 hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// ---- MFMA --------------------------------------------------------------------
// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] * B[32x16].
// Lane l (g = l / 16) supplies A[row = l % 16][k = 8g .. 8g+7] and
// B[k = 8g .. 8g+7][col = l % 16]; it receives D[row = 4g + i][col = l % 16],
// i = 0..3.  Since k is summed over, any permutation of k applied to both
// operands alike gives the same product.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane i receives
// element (i % 4) of the 4-element (8-byte) rows addressed by lanes
// i/4, i/4 + 4, i/4 + 8 and i/4 + 12, in that order.  With a row-major
// [key][dim] tile and source lane s pointing at key (k0 + s/4), dims
// (d0 + 4*(s%4)) .. +3, lane i receives V[k0 + m][d0 + i] for m = 0..3: the
// transposed operand an MFMA needs, without transposing the tile in memory.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const u16* p) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p));
#else
    (void)p;
    return make_uint2(0u, 0u);
#endif
}

// o^T += X^T W^T over the 64 rows of a row-major LDS tile: X is the tile
// (rows = the contraction index, row stride LDX, `lx` at its first row), o^T
// holds NJ 16 x 16 blocks of [column of X][this lane's column r16], and
// pw[kb] packs, as bf16 pairs, this lane's W values for rows 16*kb + 4*g + 0..3.
// X^T comes straight from the row-major tile through transposing LDS reads.
// `halves` says which 32-row halves to include (wave-uniform); rows outside
// them are never read.
template <int NJ, int LDX>
__device__ __forceinline__ void acc_xt_w(const uint32_t (&pw)[4][2], f32x4 (&o)[NJ],
                                         const u16* lx, int r16, int g, int halves) {
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
        if (!(halves & (1 << mm))) continue;
        // B operand: rows 32mm + 4g + (0..3) and 32mm + 16 + 4g + (0..3)
        const bf16x8 wv = as_bf16x8(make_uint4(pw[2 * mm][0], pw[2 * mm][1], pw[2 * mm + 1][0],
                                               pw[2 * mm + 1][1]));
        const u16* xb = lx + (32 * mm + 4 * g + (r16 >> 2)) * LDX + 4 * (r16 & 3);
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
            const uint2 lo = lds_read_tr16(xb + 16 * jb);
            const uint2 hi = lds_read_tr16(xb + 16 * LDX + 16 * jb);
            o[jb] = mfma16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), wv, o[jb]);
        }
    }
}

// Raw buffer loads (gfx9 buffer resource: base, byte range, stride 0).  An
// access past the range returns zeros without touching memory, so a load
// needs no branch around it and every load is issued unconditionally.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(buf_rsrc r, uint32_t byte_off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}
__device__ __forceinline__ uint32_t buffer_load_u32(buf_rsrc r, uint32_t byte_off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, 0);
}
#else
struct buf_rsrc {};
__device__ __forceinline__ buf_rsrc make_rsrc(const void*, uint32_t) { return buf_rsrc{}; }
__device__ __forceinline__ uint4 buffer_load16(buf_rsrc, uint32_t) { return make_uint4(0u, 0u, 0u, 0u); }
__device__ __forceinline__ uint32_t buffer_load_u32(buf_rsrc, uint32_t) { return 0u; }
#endif
// a byte offset no range reaches (loads from it return zeros)
constexpr uint32_t kOutOfRange = 0xfffffff0u;

// Online softmax with lazy rescaling.  The reference m (log2 units, shared by
// the four lanes of a query) moves, and the accumulators are rescaled, only
// when some lane's chunk maximum `lmax` exceeds m by more than kLazyRescale;
// otherwise the chunk's probabilities are taken against the old m and stay
// below 2^kLazyRescale (harmless in float32 and bf16).  o / z and m + log2 z
// come out the same either way; the common case needs neither the cross-lane
// maximum nor the NJ*4 multiplies.  The denominator is accumulated by the
// matrix cores too (`zacc` = ones^T P^T, every element the query's sum of the
// bf16 probabilities that weight the values), which also keeps it consistent
// with those weights.
constexpr float kLazyRescale = 8.0f;
template <int NJ>
__device__ __forceinline__ void lazy_rescale(float lmax, float& m, f32x4& zacc, f32x4 (&o)[NJ]) {
    if (__ballot(lmax > m + kLazyRescale) != 0ull) {   // wave-uniform branch
        float cmax = fmaxf(lmax, __shfl_xor(lmax, 16));
        cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
        const float mnew = fmaxf(m, cmax);
        const float alpha = __builtin_amdgcn_exp2f(m - ((mnew == -INFINITY) ? 0.f : mnew));
        zacc *= alpha;
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) o[jb] *= alpha;
        m = mnew;
    }
}

// bf16 ones, the A operand that turns P^T into its column sums.
__device__ __forceinline__ bf16x8 bf16_ones() {
    return as_bf16x8(make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
}

// Maximum of three floats in one v_max3_f32.  Written out because the
// compiler quiets every operand it cannot prove a non-signalling value (the
// logits come from MFMA results) with an extra v_max each; the logits here are
// finite or -inf.
__device__ __forceinline__ float max3_logits(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ __forceinline__ float max16(const f32x4 (&sv)[4]) {
    const float r1 = max3_logits(sv[0][0], sv[0][1], sv[0][2]);
    const float r2 = max3_logits(sv[0][3], sv[1][0], sv[1][1]);
    const float r3 = max3_logits(sv[1][2], sv[1][3], sv[2][0]);
    const float r4 = max3_logits(sv[2][1], sv[2][2], sv[2][3]);
    const float r5 = max3_logits(sv[3][0], sv[3][1], sv[3][2]);
    const float r6 = max3_logits(r1, r2, r3);
    const float r7 = max3_logits(r4, r5, sv[3][3]);
    return max3_logits(r6, r7, r7);
}

// Online-softmax step shared by the attention kernels.  `sv[kb][i]` holds the
// logits, in log2 units, of keys kc + 16*kb + 4*g + i for this lane's query
// (-inf where masked).  Updates the reference `m` and the denominator `zacc`,
// and accumulates O^T += V^T P^T (NJ 16 x 16 tiles, rows = value dims) for the
// 64 keys of the chunk; `lv` points at the chunk's first key row of the
// row-major value tile (row stride LDX), and `halves` says which 32-key halves
// hold any visible key (wave-uniform).
template <int NJ, int LDX>
__device__ __forceinline__ void softmax_pv_chunk(f32x4 (&sv)[4], float& m, f32x4& zacc,
                                                 f32x4 (&o)[NJ], const u16* lv, int r16, int g,
                                                 int halves) {
    lazy_rescale<NJ>(max16(sv), m, zacc, o);
    const float msafe = (m == -INFINITY) ? 0.f : m;
    uint32_t pw[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        pw[kb][0] = cvt_pk_bf16(__builtin_amdgcn_exp2f(sv[kb][0] - msafe),
                                __builtin_amdgcn_exp2f(sv[kb][1] - msafe));
        pw[kb][1] = cvt_pk_bf16(__builtin_amdgcn_exp2f(sv[kb][2] - msafe),
                                __builtin_amdgcn_exp2f(sv[kb][3] - msafe));
    }
    acc_xt_w<NJ, LDX>(pw, o, lv, r16, g, halves);
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
        if (!(halves & (1 << mm))) continue;
        zacc = mfma16(bf16_ones(), as_bf16x8(make_uint4(pw[2 * mm][0], pw[2 * mm][1],
                                                        pw[2 * mm + 1][0], pw[2 * mm + 1][1])),
                      zacc);
    }
}

// Four float32 values to 4 consecutive output elements (bf16: one 8-byte store).
template <typename OutT>
__device__ __forceinline__ void store4(OutT* dst, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<u16>(u16* dst, float a, float b, float c, float d) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(cvt_pk_bf16(a, b), cvt_pk_bf16(c, d));
}
template <>
__device__ __forceinline__ void store4<float>(float* dst, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}

// Membership bitmask of one token (KW words, bit c = member of cluster c):
// where that token's row of cluster c goes.  -1: straight to the output (the
// token has no other cluster); otherwise its rank, the number of the token's
// clusters below c (the combine step sums ranks in ascending order).
__device__ __forceinline__ int row_dest(const uint32_t* __restrict__ m, int KW, int c) {
    int cnt = 0, below = 0;
    for (int i = 0; i < KW; ++i) {
        const uint32_t word = m[i];
        cnt += __popc(word);
        if (i < (c >> 5)) below += __popc(word);
        else if (i == (c >> 5)) below += __popc(word & ((1u << (c & 31)) - 1u));
    }
    return cnt == 1 ? -1 : below;
}

// The same in two steps, so that the words can be requested together with
// other loads and counted only after all of them are issued: load_words reads
// token t's KW <= 8 words (k <= 256) from the resource of its (batch, head)
// slice of the mask, or zeros unless `ok`; dest_from_words counts them.
__device__ __forceinline__ void load_words(buf_rsrc mrs, bool ok, int t, int KW,
                                           uint32_t (&wd)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
        wd[i] = buffer_load_u32(mrs, ok && i < KW ? 4u * (uint32_t)(t * KW + i) : kOutOfRange);
}
__device__ __forceinline__ int dest_from_words(const uint32_t (&wd)[8], int c, int KW) {
    int cnt = 0, below = 0;
    if (KW <= 2) {   // k <= 64 (wave-uniform): only the first two words can be set
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            cnt += __popc(wd[i]);
            if (i < (c >> 5)) below += __popc(wd[i]);
            else if (i == (c >> 5)) below += __popc(wd[i] & ((1u << (c & 31)) - 1u));
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            cnt += __popc(wd[i]);
            if (i < (c >> 5)) below += __popc(wd[i]);
            else if (i == (c >> 5)) below += __popc(wd[i] & ((1u << (c & 31)) - 1u));
        }
    }
    return cnt == 1 ? -1 : below;
}

// The online-softmax step over 32 keys: `sv[kb][i]` holds the logits (log2
// units, -inf where masked) of keys 16*kb + 4*g + i of the half tile whose
// first value row `lv` points at (row stride LDX).
template <int NJ, int LDX>
__device__ __forceinline__ void softmax_pv_half(f32x4 (&sv)[2], float& m, f32x4& zacc,
                                                f32x4 (&o)[NJ], const u16* lv, int r16, int g) {
    const float lmax = fmaxf(fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3])),
                             fmaxf(fmaxf(sv[1][0], sv[1][1]), fmaxf(sv[1][2], sv[1][3])));
    lazy_rescale<NJ>(lmax, m, zacc, o);
    const float msafe = (m == -INFINITY) ? 0.f : m;
    uint32_t pw[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        pw[kb][0] = cvt_pk_bf16(__builtin_amdgcn_exp2f(sv[kb][0] - msafe),
                                __builtin_amdgcn_exp2f(sv[kb][1] - msafe));
        pw[kb][1] = cvt_pk_bf16(__builtin_amdgcn_exp2f(sv[kb][2] - msafe),
                                __builtin_amdgcn_exp2f(sv[kb][3] - msafe));
    }
    const bf16x8 pbv = as_bf16x8(make_uint4(pw[0][0], pw[0][1], pw[1][0], pw[1][1]));
    const u16* vb = lv + (4 * g + (r16 >> 2)) * LDX + 4 * (r16 & 3);
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) {
        const uint2 lo = lds_read_tr16(vb + 16 * jb);
        const uint2 hi = lds_read_tr16(vb + 16 * LDX + 16 * jb);
        o[jb] = mfma16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pbv, o[jb]);
    }
    zacc = mfma16(bf16_ones(), pbv, zacc);
}

// ---- wave helpers --------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// This thread's wave within the workgroup, as a wave-uniform (scalar) value, so
// that everything derived from it stays in scalar registers.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ float xor_max_16_32(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

__device__ __forceinline__ float xor_sum_16_32(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// exp(x) through the hardware base-2 exponential.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// The dispatcher hands workgroups to the 8 XCDs round-robin (linear workgroup
// id b goes to XCD b % 8), and each XCD has its own L2.  This renumbering
// gives every XCD one contiguous run of the nb work items, so neighbouring
// items that read overlapping rows share an L2.  It is a bijection on [0, nb).
__device__ __forceinline__ int xcd_contiguous(int b, int nb) {
    constexpr int kXcd = 8;
    const int per = nb / kXcd, rem = nb % kXcd;
    const int x = b % kXcd, s = b / kXcd;
    return x * per + (x < rem ? x : rem) + s;
}

__device__ __forceinline__ int clamp_pos(int t, int n) { return t < 0 ? 0 : (t >= n ? n - 1 : t); }

// Typed loads of one token element for the float32 and bf16 variants.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float* p, long i) { return p[i]; }
    static __device__ __forceinline__ void store(float* p, long i, float v) { p[i] = v; }
};
template <> struct Elem<u16> {
    static __device__ __forceinline__ float load(const u16* p, long i) { return bf2f(p[i]); }
    static __device__ __forceinline__ void store(u16* p, long i, float v) { p[i] = f2bf(v); }
};

}  // namespace rt
