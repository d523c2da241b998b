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

hipError_t launch_score(const void* qk, int dtype, const float* mu, int B, int H, int n, int d,
                        int k, float* inv_norm, float* scores, void* qk_hat, hipStream_t s);

hipError_t launch_topw(const float* scores, int BH, int n, int k, int w, int32_t* idx,
                       hipStream_t s);

// Per-token membership counters cnt [BH*n] and lists list [BH*n][k] of
// c*w + r entries (unordered).
hipError_t launch_membership(const int32_t* idx, int BH, int n, int k, int w, uint32_t* cnt,
                             int32_t* list, hipStream_t s);

hipError_t launch_cluster_attn(const void* q, const void* kk, const void* v, int dtype,
                               const float* q_inv, const float* k_inv, const int32_t* idx,
                               const uint32_t* cnt, int BH, int n, int d, int k, int w,
                               float scale, int causal, void* out, int out_dtype, float* lse,
                               float* part, hipStream_t s);

hipError_t launch_combine(const uint32_t* cnt, const int32_t* list, const float* part,
                          int out_dtype, int BH, int n, int d, int k, int w, void* out,
                          hipStream_t s);

hipError_t launch_ema(float* mu, const void* q, const float* q_inv, const void* kk,
                      const float* k_inv, int dtype, const int32_t* idx, int B, int H, int n,
                      int d, int k, int w, float lambda, hipStream_t s);

hipError_t launch_local_attn(const void* q, const void* kk, const void* v, int dtype, int BH,
                             int n, int d, int window, float scale, int causal, void* out,
                             int out_dtype, hipStream_t s);

hipError_t launch_cluster_attn_bwd(const void* q, const void* kk, const void* v, int dtype,
                                   const float* q_inv, const float* k_inv, const int32_t* idx,
                                   const float* lse, const void* dout, int BH, int n, int d,
                                   int k, int w, float scale, int causal, float* dq, float* dk,
                                   float* dv, float* ws, hipStream_t s);

size_t bwd_workspace_bytes(int BH, int n, int d, int k, int w);

}  // namespace rt
