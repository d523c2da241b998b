// rt_internal.hpp -- launchers behind the C ABI (host side).  Arguments are
// validated by the caller (capi.hip) before any launcher runs; launchers only
// pick kernel variants and enqueue them on `s`.  Each returns the HIP error
// of its launches (hipSuccess when all were accepted).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rt {

// Largest cluster the in-cluster kernels keep on chip.
int max_cluster_rows(int dtype, int d, bool shared_qk);

// Largest sequence the top-w kernel holds in registers.
constexpr int kMaxSeqTopw = 65536;

// mask (nullable) [B*H*n][mask_words(k)]: zeroed by the score kernel, filled
// by the top-w kernel.
// Each token's nearest centroid (largest score, ties to the lower index) and
// that score, with the inverse norms (and the zeroed bitmask when mask != null).
hipError_t launch_nearest(const void* qk, int dtype, const float* mu, int B, int H, int n, int d,
                          int k, float* inv_norm, int32_t* label, float* best, uint32_t* mask,
                          hipStream_t s);

// Partition-style balanced clusters from the nearest-centroid labels and
// scores (n a multiple of k, n <= kPartitionMaxN); mask (nullable) must be
// zeroed.  Scratch: grp and cl [BH][n] int32, goff [BH][k + 1] int32.
constexpr int kPartitionMaxN = 16384;
hipError_t launch_partition(const int32_t* label, const float* best, int BH, int n, int k,
                            int32_t* idx, uint32_t* mask, int32_t* grp, int32_t* cl,
                            int32_t* goff, hipStream_t s);

// The nearest-centroid EMA: per-chunk sums of each label's normalised rows
// (part_q / part_k: label_chunks(B, n) * H * k * d floats each; kk == nullptr
// for shared q/k), then the update.
int label_chunks(int B, int n);
hipError_t launch_label_ema(float* mu, const void* q, const float* q_inv, const int32_t* q_label,
                            const void* kk, const float* k_inv, const int32_t* k_label, int dtype,
                            int B, int H, int n, int d, int k, float lambda, float* part_q,
                            float* part_k, hipStream_t s);

hipError_t launch_score(const void* qk, int dtype, const float* mu, int B, int H, int n, int d,
                        int k, float* inv_norm, float* scores, void* qk_hat, uint32_t* mask,
                        hipStream_t s);

hipError_t launch_topw(const float* scores, int BH, int n, int k, int w, int32_t* idx,
                       uint32_t* mask, hipStream_t s);

// Words of the per-token membership bitmask (one bit per centroid).
inline int mask_words(int k) { return (k + 31) / 32; }

// Token-major partial-row slots per token; higher membership ranks overflow
// to a cluster-major buffer, found through a per-token directory
// dir[token][rank - kSlots] = c * w + r (cluster c, member row r).
constexpr int kSlots = 4;
inline int ovf_ranks(int k) { return k > kSlots ? k - kSlots : 0; }

// Zero the bitmask mask [BH*n][mask_words(k)] and set one bit per membership.
hipError_t launch_mask(const int32_t* idx, int BH, int n, int k, int w, uint32_t* mask,
                       hipStream_t s);

// idx: the clusters' keys and values; idx_q: their queries (nullptr: idx; a
// separate query membership only with causal == 0).
hipError_t launch_cluster_attn(const void* q, const void* kk, const void* v, int dtype,
                               const float* q_inv, const float* k_inv, const int32_t* idx,
                               const int32_t* idx_q, const uint32_t* mask, int BH, int n, int d,
                               int k, int w, float scale, int causal, void* out, int out_dtype,
                               float* lse, float* slots, float* ovf, int32_t* dir, float* sum_q,
                               float* sum_k, hipStream_t s);

// mu != nullptr: the centroid update from the member sums (sum_q, sum_k of B
// batch rows; sum_k nullptr counts sum_q twice) runs in the same launch.
hipError_t launch_combine(const uint32_t* mask, const float* slots, const float* ovf,
                          const int32_t* dir, int out_dtype, int BH, int n, int d, int k, int w,
                          void* out, hipStream_t s, float* mu = nullptr,
                          const float* sum_q = nullptr, const float* sum_k = nullptr, int B = 0,
                          int H = 0, float lambda = 0.f);

// The same for three float32 outputs sharing one membership (one pass over the
// bits).
hipError_t launch_combine3_f32(const uint32_t* mask, const float* const slots[3],
                               const float* const ovf[3], const int32_t* dir, int BH, int n, int d,
                               int k, int w, float* const out[3], hipStream_t s);
hipError_t launch_combine2_f32(const uint32_t* mask, const float* const slots[2],
                               const float* const ovf[2], const int32_t* dir, int BH, int n, int d,
                               int k, int w, float* const out[2], hipStream_t s);

// mu <- lambda*mu + (1-lambda)/2 * (sum_b sum_q[b] + sum_b sum_k[b]); sum_k may
// be NULL (keys are the queries: S_K = S_Q).  sums are [B][H][k][d].
hipError_t launch_ema_sums(float* mu, const float* sum_q, const float* sum_k, int B, int H,
                           int k, int d, float lambda, hipStream_t s);

hipError_t launch_ema(float* mu, const void* q, const float* q_inv, const void* kk,
                      const float* k_inv, int dtype, const int32_t* idx, int B, int H, int n,
                      int d, int k, int w, float lambda, hipStream_t s);

// lookback < 0: the sliding window [i - window + 1, i] (or the band when not
// causal); lookback >= 0: blocks of `window` positions, own block and the
// `lookback` before it (causal).
// lse: optional [BH][n] float32, the natural log of each query's denominator.
hipError_t launch_local_attn(const void* q, const void* kk, const void* v, int dtype, int BH,
                             int n, int d, int window, int lookback, float scale, int causal,
                             void* out, int out_dtype, float* lse, hipStream_t s);

hipError_t launch_cluster_attn_bwd(const void* q, const void* kk, const void* v, int dtype,
                                   const float* q_inv, const float* k_inv, const int32_t* idx,
                                   const uint32_t* member_mask, const float* lse,
                                   const void* dout, int BH, int n, int d,
                                   int k, int w, float scale, int causal, float* dq, float* dk,
                                   float* dv, void* ws, hipStream_t s);

size_t bwd_workspace_bytes(int BH, int n, int d, int k, int w);

// C = A W^T (+ residual), bf16 in and out, float32 accumulation.  A is
// row-major [M][K] (amode 0) or head-major segments a[s] [B][ha[s]][n][d]
// (amode 1, k = head * d + i over the concatenated heads); W is [N][K]; C is
// row-major [M][N] with an optional row-major residual (cmode 0) or head-major
// segments c[s] [B][hc[s]][n][d] (cmode 1, unused segments have hc = 0).
struct ProjArgs {
    const void* a[2];
    int ha[2];
    const void* w;
    void* c[5];
    int hc[5];
    const void* res;
    int M, N, K, n, d;
};
hipError_t launch_proj(const ProjArgs& p, int amode, int cmode, hipStream_t s);

// Backward of the local-window attention: two kernels (dq with the per-query
// log-sum-exp and D into ws, then dk and dv); bf16 inputs, d in {64, 128}.
size_t local_bwd_workspace_bytes(int BH, int n);
hipError_t launch_local_attn_bwd(const void* q, const void* kk, const void* v, const void* dout,
                                 int BH, int n, int d, int window, float scale, int causal,
                                 float* dq, float* dk, float* dv, void* ws, hipStream_t s);

// Gradient through the unit normalisation, one row of d <= 128 per wave.
hipError_t launch_norm_bwd(const void* x, int dtype, const float* inv_norm, const float* g1,
                           const float* g2, long rows, int d, float* dx, hipStream_t s);

// Operand X[idx][k] of the backward products: row-major with leading
// dimension ld, or head-major segments p[s] [B][hs[s]][n][d] over the
// concatenated heads (unused segments have hs = 0).
struct GemmOperand {
    const void* p[5];
    int hs[5];
    int ld;
};
// C[M][N] = sum_k A[m][k] B[n][k]: float32 row-major (+ bf16 residual res) or
// bf16 head-major segments c[s] (m = token, n = head * d + i).
struct GemmArgs {
    GemmOperand a, b;
    void* c[5];
    int hc[5];
    const uint16_t* res;
    int M, N, K, n, d;
    // float32 row-major C only: ksplit > 1 splits the contraction into that
    // many ranges, each product going to part[z][M][N], then added in order
    // of z (deterministic) into C, with the residual.
    int ksplit;
    float* part;
};
// The four products of the projections' backward:
//   GEMM_DO    dO = dy W_o        A = dy [T][dm] row-major, B = W_o [dm][N] (idx-contiguous), C head-major bf16
//   GEMM_DWO   dW_o = dy^T O      A = dy read idx-contiguous, B = O head-major (bf16), C fp32
//   GEMM_DX    dx = dC W_in + dy  A = dC head-major fp32 (k-contiguous), B = W_in [K][dm], C fp32 + res
//   GEMM_DWIN  dW_in = dC^T x     A = dC head-major fp32 (idx-contiguous), B = x [T][dm], C fp32
enum { GEMM_DO = 0, GEMM_DWO = 1, GEMM_DX = 2, GEMM_DWIN = 3 };
hipError_t launch_gemm_bwd(int which, const GemmArgs& p, hipStream_t s);

// Largest cluster the backward kernels keep on chip.
int max_cluster_rows_bwd(int dtype, int d, bool shared_qk);

// One decode step (bfloat16 rows; caches as described with the entry points).
constexpr int kDecodeMaxEntries = 16384;   // cap and window: their logits live in LDS
hipError_t launch_decode_fill(const void* qk, const float* inv, const void* v, const int32_t* idx,
                              int BH, int n, int d, int k, int w, int cap, void* ck, float* cinv,
                              void* cv, int32_t* cpos, int32_t* clen, hipStream_t s);
hipError_t launch_decode_ring_fill(const void* kk, const void* v, int BH, int n, int d,
                                   int window, void* rk, void* rv, hipStream_t s);
hipError_t launch_decode_routed(const void* qk_t, const void* v_t, const float* mu, int BH, int H,
                                int d, int k, int cap, void* ck, float* cinv, void* cv,
                                int32_t* cpos, int32_t* clen, int t, float scale, void* out,
                                int out_dtype, int32_t* label, hipStream_t s);
hipError_t launch_decode_local(const void* q_t, const void* k_t, const void* v_t, int BH, int d,
                               int window, void* rk, void* rv, int t, float scale, void* out,
                               int out_dtype, hipStream_t s);

// Jensen-Shannon divergence of each cluster row's routed distribution from its
// query's local one (bf16 rows; lse_l: the local heads' natural log-denominators).
int max_js_rows(int d);
hipError_t launch_attn_js(const void* qk, const float* q_inv, const int32_t* idx, const void* q_l,
                          const void* k_l, const float* lse_l, int BH, int n, int d, int k, int w,
                          int window, float scale_r, float scale_l, int causal, float* js,
                          hipStream_t s);

}  // namespace rt
