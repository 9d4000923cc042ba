// Internal launchers behind the C ABI.  Every launcher enqueues on `stream`,
// trusts that api.hip has validated its arguments, and returns
// hipGetLastError() of its last launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

hipError_t launch_gate(const float* logits, int T, int E, int k, int renormalize, int* topk_ids,
                       float* topk_w, hipStream_t stream);
hipError_t launch_gate_record(const float* logits, int T, int E, int k, int renormalize, int* topk_ids,
                              float* topk_w, int block_tokens, int layer, int L, int* block_counts,
                              hipStream_t stream);

// ---- router projection -------------------------------------------------------
hipError_t launch_router(const void* x, const void* w_router, int T, int d, int E, int bf16, float* logits,
                         hipStream_t stream);

// ---- permutation -----------------------------------------------------------
struct PermuteArgs {
  const int* topk_ids;
  int T, E, k, n_shared, n_priority;
  const void* x;
  int elem_bytes;  // 2 (bf16) or 4 (f32)
  int d;
  int* group_offsets;
  int* sorted_to_flat;
  int* flat_to_sorted;
  int* sorted_token;  // may be nullptr
  void* x_sorted;
};
size_t permute_workspace_bytes(int T, int E, int k, int n_shared, int n_priority);
hipError_t launch_permute(const PermuteArgs& a, void* workspace, hipStream_t stream);

// ---- grouped FFN -----------------------------------------------------------
struct FfnArgs {
  const void* x_sorted;
  const int* x_rows;  // nullptr: x_sorted is already in sorted order
  int n_x;            // rows of x_sorted when x_rows is given
  const int* group_offsets;
  int n_rows, E, n_shared, nseg, d, I;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  int bf16;  // 1: bf16 operands, 0: fp32
  void* h_sorted;
  // FP8-weight call only: one fp32 scale per weight row ([E+S][I], [E+S][I], [E+S][d])
  const float* s_gate = nullptr;
  const float* s_up = nullptr;
  const float* s_down = nullptr;
  // weights pre-packed in 1 KiB blocks of 16 rows: 32 K values for bf16
  // (moe_grouped_ffn_packed), 64 for FP8 codes (moe_grouped_ffn_fp8w_packed)
  bool packed = false;
  // per-tile timeline of the persistent queue (moe_grouped_ffn_traced): records
  // of 4 uint64, nullptr for none
  unsigned long long* trace = nullptr;
  int trace_capacity = 0;
  // combine folded into the down projection (moe_grouped_ffn_combine): y32 is
  // the [T][d] fp32 sums in the workspace, y the [T][d] bf16 result; nullptr
  // for the plain call
  float* y32 = nullptr;
  void* y = nullptr;
  const int* s2f = nullptr;
  const float* topk_w = nullptr;
  int T = 0, k = 0;
};
size_t ffn_workspace_bytes(int n_rows, int E, int n_shared, int nseg, int d, int I, int bf16);
// moe_grouped_ffn_combine: batches on the decode-shaped kernels only
bool ffn_fused_combine_supported(int n_rows, int E, int n_shared, int nseg, int d, int I);
hipError_t launch_ffn(const FfnArgs& a, void* workspace, hipStream_t stream);
size_t ffn_fp8w_workspace_bytes(int n_rows, int E, int n_shared, int nseg, int d, int I, bool packed);
// FP8 batches that run on the GEMM kernel (packed codes, groups averaging more
// than 48 rows, d and I multiples of 64 and at least 128, 16-byte aligned scales)
bool fp8w_uses_gemm(int n_rows, int G, int d, int I, bool packed, const void* s_gate, const void* s_up,
                    const void* s_down);
hipError_t launch_ffn_fp8w(const FfnArgs& a, void* workspace, hipStream_t stream);

// ---- combine ---------------------------------------------------------------
hipError_t launch_combine(const void* h_sorted, const int* flat_to_sorted, const float* topk_w, int T,
                          int k, int n_shared, int d, int bf16, void* y, hipStream_t stream);

// ---- statistics ------------------------------------------------------------
struct StatsArgs {
  const int* topk_ids;
  int L, T, k, E;
  const int* req_offsets;
  int R;
  const float* idf;
  int* counts;
  int* union_size;
  uint8_t* union_mask;
  int* affinity;
  int* req_counts;
  float* signature;
};
size_t stats_workspace_bytes(int L, int T, int k, int E, int R);
hipError_t launch_stats(const StatsArgs& a, void* workspace, hipStream_t stream);

// ---- continuous (softmax-probability) request signature ---------------------
hipError_t launch_prob_signature(const float* logits, int L, int T, int E, const int* req_offsets, int R,
                                 float* signature, hipStream_t stream);

}  // namespace moe
