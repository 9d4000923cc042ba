// libmoe C ABI: host-side argument checks, workspace queries and launches.
// Every check happens before anything is enqueued; no call synchronises or
// reads device memory on the host.
#include <stdint.h>

#include <mutex>

#include "libmoe.h"
#include "launch.h"

namespace {

// Scratch of moe_grouped_ffn_noalloc: the FFN workspace (SwiGLU intermediate,
// tile-queue flags, diagnostic word) in a device array that every GPU the
// library runs on holds until the process ends.  In host code `scratch` only
// names the symbol; its device address is looked up once per device (with that
// device current) and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// This device's copy of `scratch`.
moe_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return MOE_ERR_HIP;
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

constexpr long long kIntMax = 0x7fffffffLL;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool fits_int(long long v) { return v >= 0 && v <= kIntMax; }

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

int elem_bytes(moe_dtype dt) { return dt == MOE_BF16 ? 2 : 4; }

bool known_dtype(moe_dtype dt) { return dt == MOE_F32 || dt == MOE_BF16; }

// workspace protocol: NULL buffer -> report the size; else check it is enough
moe_status workspace_check(void* workspace, size_t* workspace_bytes, size_t need, bool* query) {
  *query = false;
  if (workspace_bytes == nullptr) return MOE_ERR_INVALID_ARG;
  if (workspace == nullptr) {
    *workspace_bytes = need;
    *query = true;
    return MOE_OK;
  }
  if (*workspace_bytes < need) return MOE_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// moe_grouped_ffn_fp8w and its packed-weight variant
moe_status ffn_fp8w_call(bool packed, const void* x_sorted, const int32_t* x_rows, int32_t n_x,
                                const int32_t* group_offsets, int32_t n_rows, int32_t E, int32_t n_shared,
                                int32_t nseg, int32_t d, int32_t I, const void* w_gate, const float* s_gate,
                                const void* w_up, const float* s_up, const void* w_down, const float* s_down,
                                void* h_sorted, void* workspace, size_t* workspace_bytes, hipStream_t stream) {
  if (n_rows < 0 || E < 1 || n_shared < 0 || (nseg != 1 && nseg != 2) || d < 1 || I < 1)
    return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || n_shared > MOE_MAX_SHARED) return MOE_ERR_UNSUPPORTED;
  if (d % 16 != 0 || I % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if (packed && (d % 64 != 0 || I % 64 != 0)) return MOE_ERR_UNSUPPORTED;
  if (!fits_int(static_cast<long long>(n_rows) * d) || !fits_int(static_cast<long long>(n_rows) * I))
    return MOE_ERR_UNSUPPORTED;
  bool query;
  moe_status st = workspace_check(workspace, workspace_bytes,
                                  moe::ffn_fp8w_workspace_bytes(n_rows, E, n_shared, nseg, d, I, packed), &query);
  if (st != MOE_OK || query) return st;
  if (n_rows == 0) return MOE_OK;
  if (!x_sorted || !group_offsets || !w_gate || !w_up || !w_down || !s_gate || !s_up || !s_down || !h_sorted)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_sorted) || !aligned4(group_offsets) || !aligned16(w_gate) || !aligned16(w_up) ||
      !aligned16(w_down) || !aligned16(s_gate) || !aligned16(s_up) || !aligned16(s_down) || !aligned16(h_sorted))
    return MOE_ERR_INVALID_ARG;
  if (x_rows && (!aligned4(x_rows) || n_x < 1)) return MOE_ERR_INVALID_ARG;
  if (x_rows && !fits_int(static_cast<long long>(n_x) * d)) return MOE_ERR_UNSUPPORTED;
  moe::FfnArgs a;
  a.x_sorted = x_sorted;
  a.x_rows = x_rows;
  a.n_x = x_rows ? n_x : n_rows;
  a.group_offsets = group_offsets;
  a.n_rows = n_rows;
  a.E = E;
  a.n_shared = n_shared;
  a.nseg = nseg;
  a.d = d;
  a.I = I;
  a.w_gate = w_gate;
  a.w_up = w_up;
  a.w_down = w_down;
  a.bf16 = 1;
  a.h_sorted = h_sorted;
  a.s_gate = s_gate;
  a.s_up = s_up;
  a.s_down = s_down;
  a.packed = packed;
  return hip_status(moe::launch_ffn_fp8w(a, workspace, stream));
}

// moe_grouped_ffn and its traced form
moe_status ffn_call(const void* x_sorted, const int32_t* x_rows, int32_t n_x, const int32_t* group_offsets,
                    int32_t n_rows, int32_t E, int32_t n_shared, int32_t nseg, int32_t d, int32_t I,
                    const void* w_gate, const void* w_up, const void* w_down, moe_dtype dtype, void* h_sorted,
                    void* workspace, size_t* workspace_bytes, uint64_t* trace, int32_t trace_capacity,
                    bool packed, hipStream_t stream) {
  if (n_rows < 0 || E < 1 || n_shared < 0 || (nseg != 1 && nseg != 2) || d < 1 || I < 1)
    return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || n_shared > MOE_MAX_SHARED) return MOE_ERR_UNSUPPORTED;
  if (!known_dtype(dtype) || d % 8 != 0 || I % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (packed && (dtype != MOE_BF16 || d % 32 != 0 || I % 32 != 0)) return MOE_ERR_UNSUPPORTED;
  if (!fits_int(static_cast<long long>(n_rows) * d) || !fits_int(static_cast<long long>(n_rows) * I))
    return MOE_ERR_UNSUPPORTED;
  bool query;
  moe_status st = workspace_check(
      workspace, workspace_bytes,
      moe::ffn_workspace_bytes(n_rows, E, n_shared, nseg, d, I, dtype == MOE_BF16 ? 1 : 0), &query);
  if (st != MOE_OK || query) return st;
  if (n_rows == 0) return MOE_OK;
  if (!x_sorted || !group_offsets || !w_gate || !w_up || !w_down || !h_sorted) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_sorted) || !aligned4(group_offsets) || !aligned16(w_gate) || !aligned16(w_up) ||
      !aligned16(w_down) || !aligned16(h_sorted))
    return MOE_ERR_INVALID_ARG;
  if (x_rows && (!aligned4(x_rows) || n_x < 1)) return MOE_ERR_INVALID_ARG;
  if (x_rows && !fits_int(static_cast<long long>(n_x) * d)) return MOE_ERR_UNSUPPORTED;
  moe::FfnArgs a;
  a.x_sorted = x_sorted;
  a.x_rows = x_rows;
  a.n_x = x_rows ? n_x : n_rows;
  a.group_offsets = group_offsets;
  a.n_rows = n_rows;
  a.E = E;
  a.n_shared = n_shared;
  a.nseg = nseg;
  a.d = d;
  a.I = I;
  a.w_gate = w_gate;
  a.w_up = w_up;
  a.w_down = w_down;
  a.bf16 = dtype == MOE_BF16 ? 1 : 0;
  a.h_sorted = h_sorted;
  a.trace = reinterpret_cast<unsigned long long*>(trace);
  a.trace_capacity = trace_capacity;
  a.packed = packed;
  return hip_status(moe::launch_ffn(a, workspace, stream));
}

}  // namespace

extern "C" {

moe_status moe_prob_signature(const float* logits, int32_t L, int32_t T, int32_t E, const int32_t* req_offsets,
                              int32_t R, float* signature, hipStream_t stream) {
  if (L < 1 || T < 0 || E < 1 || R < 0) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || L > 65535) return MOE_ERR_UNSUPPORTED;
  if (!fits_int(static_cast<long long>(L) * T * E) || !fits_int(static_cast<long long>(R) * L * E))
    return MOE_ERR_UNSUPPORTED;
  if (R == 0) return MOE_OK;
  if (!req_offsets || !signature || (T > 0 && !logits)) return MOE_ERR_INVALID_ARG;
  if (!aligned4(req_offsets) || !aligned4(signature) || (logits && !aligned4(logits))) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_prob_signature(logits, L, T, E, req_offsets, R, signature, stream));
}

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

moe_status moe_gate(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renormalize, int32_t* topk_ids,
                    float* topk_w, hipStream_t stream) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (renormalize != 0 && renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  if (!fits_int(static_cast<long long>(T) * E)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned4(logits) || !aligned4(topk_ids) || !aligned4(topk_w)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_gate(logits, T, E, k, renormalize, topk_ids, topk_w, stream));
}

moe_status moe_gate_record(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renormalize,
                           int32_t* topk_ids, float* topk_w, int32_t block_tokens, int32_t layer, int32_t L,
                           int32_t* block_counts, hipStream_t stream) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (renormalize != 0 && renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (block_tokens < 1 || L < 1 || layer < 0 || layer >= L) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  if (!fits_int(static_cast<long long>(T) * E)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w || !block_counts) return MOE_ERR_INVALID_ARG;
  if (!aligned4(logits) || !aligned4(topk_ids) || !aligned4(topk_w) || !aligned4(block_counts))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_gate_record(logits, T, E, k, renormalize, topk_ids, topk_w, block_tokens, layer, L,
                                            block_counts, stream));
}

moe_status moe_stage_to_host(const void* src, void* dst_host, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return MOE_OK;
  if (!src || !dst_host) return MOE_ERR_INVALID_ARG;
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, dst_host) != hipSuccess) {
    (void)hipGetLastError();   // pageable memory is an argument error, not a sticky one
    return MOE_ERR_INVALID_ARG;
  }
  if (a.type != hipMemoryTypeHost) return MOE_ERR_INVALID_ARG;
  hipPointerAttribute_t b{};
  if (hipPointerGetAttributes(&b, src) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_ERR_INVALID_ARG;
  }
  if (b.type != hipMemoryTypeDevice) return MOE_ERR_INVALID_ARG;
  return hip_status(hipMemcpyAsync(dst_host, src, bytes, hipMemcpyDeviceToHost, stream));
}

moe_status moe_router(const void* x, const void* w_router, int32_t T, int32_t d, int32_t E, moe_dtype dtype,
                      float* logits, hipStream_t stream) {
  if (T < 0 || E < 1 || d < 1) return MOE_ERR_INVALID_ARG;
  if (!known_dtype(dtype) || E > MOE_MAX_EXPERTS || d % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (!fits_int(static_cast<long long>(T) * d) || !fits_int(static_cast<long long>(T) * E) ||
      !fits_int(static_cast<long long>(E) * d))
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !logits) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(logits)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_router(x, w_router, T, d, E, dtype == MOE_BF16 ? 1 : 0, logits, stream));
}

moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t E, int32_t k, int32_t n_shared,
                       int32_t n_priority, const void* x, moe_dtype dtype, int32_t d, int32_t* group_offsets,
                       int32_t* sorted_to_flat, int32_t* flat_to_sorted, int32_t* sorted_token, void* x_sorted,
                       void* workspace, size_t* workspace_bytes, hipStream_t stream) {
  if (T < 0 || E < 1 || k < 1 || k > E || n_shared < 0 || n_priority < 0 || n_priority > T)
    return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || n_shared > MOE_MAX_SHARED) return MOE_ERR_UNSUPPORTED;
  const long long N = static_cast<long long>(T) * (k + n_shared);
  if (!fits_int(N)) return MOE_ERR_UNSUPPORTED;
  if (x != nullptr) {
    if (!known_dtype(dtype)) return MOE_ERR_UNSUPPORTED;
    if (d < 1) return MOE_ERR_INVALID_ARG;
    if (d % 8 != 0) return MOE_ERR_UNSUPPORTED;
  }
  bool query;
  moe_status st = workspace_check(workspace, workspace_bytes,
                                  moe::permute_workspace_bytes(T, E, k, n_shared, n_priority), &query);
  if (st != MOE_OK || query) return st;
  if (!group_offsets || !aligned4(group_offsets)) return MOE_ERR_INVALID_ARG;
  if (N > 0) {
    if (!topk_ids || !sorted_to_flat || !flat_to_sorted) return MOE_ERR_INVALID_ARG;
    if (!aligned4(topk_ids) || !aligned4(sorted_to_flat) || !aligned4(flat_to_sorted) ||
        (sorted_token && !aligned4(sorted_token)))
      return MOE_ERR_INVALID_ARG;
    if (x != nullptr && (!x_sorted || !aligned16(x) || !aligned16(x_sorted))) return MOE_ERR_INVALID_ARG;
  }
  moe::PermuteArgs a;
  a.topk_ids = topk_ids;
  a.T = T;
  a.E = E;
  a.k = k;
  a.n_shared = n_shared;
  a.n_priority = n_priority;
  a.x = N > 0 ? x : nullptr;
  a.elem_bytes = elem_bytes(dtype);
  a.d = d;
  a.group_offsets = group_offsets;
  a.sorted_to_flat = sorted_to_flat;
  a.flat_to_sorted = flat_to_sorted;
  a.sorted_token = sorted_token;
  a.x_sorted = x_sorted;
  return hip_status(moe::launch_permute(a, workspace, stream));
}

moe_status moe_grouped_ffn(const void* x_sorted, const int32_t* x_rows, int32_t n_x,
                           const int32_t* group_offsets, int32_t n_rows, int32_t E,
                           int32_t n_shared, int32_t nseg, int32_t d, int32_t I, const void* w_gate,
                           const void* w_up, const void* w_down, moe_dtype dtype, void* h_sorted, void* workspace,
                           size_t* workspace_bytes, hipStream_t stream) {
  return ffn_call(x_sorted, x_rows, n_x, group_offsets, n_rows, E, n_shared, nseg, d, I, w_gate, w_up, w_down, dtype,
                  h_sorted, workspace, workspace_bytes, nullptr, 0, false, stream);
}

moe_status moe_grouped_ffn_traced(const void* x_sorted, const int32_t* x_rows, int32_t n_x,
                                  const int32_t* group_offsets, int32_t n_rows, int32_t E, int32_t n_shared,
                                  int32_t nseg, int32_t d, int32_t I, const void* w_gate, const void* w_up,
                                  const void* w_down, moe_dtype dtype, void* h_sorted, void* workspace,
                                  size_t* workspace_bytes, uint64_t* trace, int32_t trace_capacity,
                                  int32_t weights_packed, hipStream_t stream) {
  if (trace_capacity < 0 || (trace_capacity > 0 && (!trace || !aligned16(trace)))) return MOE_ERR_INVALID_ARG;
  if (weights_packed != 0 && weights_packed != 1) return MOE_ERR_INVALID_ARG;
  return ffn_call(x_sorted, x_rows, n_x, group_offsets, n_rows, E, n_shared, nseg, d, I, w_gate, w_up, w_down, dtype,
                  h_sorted, workspace, workspace_bytes, trace_capacity > 0 ? trace : nullptr, trace_capacity,
                  weights_packed == 1, stream);
}

moe_status moe_grouped_ffn_noalloc(const void* x_sorted, const int32_t* x_rows, int32_t n_x,
                                   const int32_t* group_offsets, int32_t n_rows, int32_t E, int32_t n_shared,
                                   int32_t nseg, int32_t d, int32_t I, const void* w_gate, const void* w_up,
                                   const void* w_down, moe_dtype dtype, void* h_sorted, hipStream_t stream) {
  // the scalar checks of moe_grouped_ffn, and the workspace this call needs
  size_t need = 0;
  moe_status st = ffn_call(x_sorted, x_rows, n_x, group_offsets, n_rows, E, n_shared, nseg, d, I, w_gate, w_up,
                           w_down, dtype, h_sorted, nullptr, &need, nullptr, 0, false, stream);
  if (st != MOE_OK) return st;
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  if (n_rows == 0) return MOE_OK;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MOE_OK) return st;
  size_t have = MOE_NOALLOC_SCRATCH_BYTES;
  return ffn_call(x_sorted, x_rows, n_x, group_offsets, n_rows, E, n_shared, nseg, d, I, w_gate, w_up, w_down, dtype,
                  h_sorted, ws, &have, nullptr, 0, false, stream);
}

moe_status moe_grouped_ffn_combine(const void* x_sorted, const int32_t* x_rows, int32_t n_x,
                                   const int32_t* group_offsets, int32_t n_rows, int32_t E, int32_t n_shared,
                                   int32_t nseg, int32_t d, int32_t I, const void* w_gate, const void* w_up,
                                   const void* w_down, int32_t weights_packed, const int32_t* sorted_to_flat,
                                   const float* topk_w, int32_t T, int32_t k, void* y, void* workspace,
                                   size_t* workspace_bytes, hipStream_t stream) {
  if (n_rows < 0 || E < 1 || n_shared < 0 || (nseg != 1 && nseg != 2) || d < 1 || I < 1 || T < 0 || k < 1)
    return MOE_ERR_INVALID_ARG;
  if (weights_packed != 0 && weights_packed != 1) return MOE_ERR_INVALID_ARG;
  if (static_cast<long long>(T) * (k + n_shared) != n_rows) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || n_shared > MOE_MAX_SHARED || k > E) return MOE_ERR_UNSUPPORTED;
  if (d % 8 != 0 || I % 8 != 0 || (weights_packed && (d % 32 != 0 || I % 32 != 0))) return MOE_ERR_UNSUPPORTED;
  if (!fits_int(static_cast<long long>(n_rows) * d) || !fits_int(static_cast<long long>(n_rows) * I))
    return MOE_ERR_UNSUPPORTED;
  if (n_rows > 0 && !moe::ffn_fused_combine_supported(n_rows, E, n_shared, nseg, d, I)) return MOE_ERR_UNSUPPORTED;
  // workspace: the [T][d] fp32 combine sums, then moe_grouped_ffn's workspace
  const size_t ysum = (static_cast<size_t>(T) * d * 4 + 255) / 256 * 256;
  bool query;
  moe_status st = workspace_check(workspace, workspace_bytes,
                                  ysum + moe::ffn_workspace_bytes(n_rows, E, n_shared, nseg, d, I, 1), &query);
  if (st != MOE_OK || query) return st;
  if (n_rows == 0) return MOE_OK;
  if (!x_sorted || !group_offsets || !w_gate || !w_up || !w_down || !sorted_to_flat || !topk_w || !y)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_sorted) || !aligned4(group_offsets) || !aligned16(w_gate) || !aligned16(w_up) ||
      !aligned16(w_down) || !aligned4(sorted_to_flat) || !aligned4(topk_w) || !aligned16(y) || !aligned16(workspace))
    return MOE_ERR_INVALID_ARG;
  if (x_rows && (!aligned4(x_rows) || n_x < 1)) return MOE_ERR_INVALID_ARG;
  if (x_rows && !fits_int(static_cast<long long>(n_x) * d)) return MOE_ERR_UNSUPPORTED;
  moe::FfnArgs a;
  a.x_sorted = x_sorted;
  a.x_rows = x_rows;
  a.n_x = x_rows ? n_x : n_rows;
  a.group_offsets = group_offsets;
  a.n_rows = n_rows;
  a.E = E;
  a.n_shared = n_shared;
  a.nseg = nseg;
  a.d = d;
  a.I = I;
  a.w_gate = w_gate;
  a.w_up = w_up;
  a.w_down = w_down;
  a.bf16 = 1;
  a.h_sorted = nullptr;
  a.packed = weights_packed == 1;
  a.y32 = static_cast<float*>(workspace);
  a.y = y;
  a.s2f = sorted_to_flat;
  a.topk_w = topk_w;
  a.T = T;
  a.k = k;
  return hip_status(moe::launch_ffn(a, static_cast<char*>(workspace) + ysum, stream));
}

moe_status moe_grouped_ffn_packed(const void* x_sorted, const int32_t* x_rows, int32_t n_x,
                                  const int32_t* group_offsets, int32_t n_rows, int32_t E, int32_t n_shared,
                                  int32_t nseg, int32_t d, int32_t I, const void* w_gate, const void* w_up,
                                  const void* w_down, void* h_sorted, void* workspace, size_t* workspace_bytes,
                                  hipStream_t stream) {
  return ffn_call(x_sorted, x_rows, n_x, group_offsets, n_rows, E, n_shared, nseg, d, I, w_gate, w_up, w_down,
                  MOE_BF16, h_sorted, workspace, workspace_bytes, nullptr, 0, true, stream);
}

moe_status moe_grouped_ffn_fp8w(const void* x_sorted, const int32_t* x_rows, int32_t n_x,
                                const int32_t* group_offsets, int32_t n_rows, int32_t E, int32_t n_shared,
                                int32_t nseg, int32_t d, int32_t I, const void* w_gate, const float* s_gate,
                                const void* w_up, const float* s_up, const void* w_down, const float* s_down,
                                void* h_sorted, void* workspace, size_t* workspace_bytes, hipStream_t stream) {
  return ffn_fp8w_call(false, x_sorted, x_rows, n_x, group_offsets, n_rows, E, n_shared, nseg, d, I, w_gate, s_gate, w_up,
                       s_up, w_down, s_down, h_sorted, workspace, workspace_bytes, stream);
}

moe_status moe_grouped_ffn_fp8w_packed(const void* x_sorted, const int32_t* x_rows, int32_t n_x,
                                const int32_t* group_offsets, int32_t n_rows, int32_t E, int32_t n_shared,
                                int32_t nseg, int32_t d, int32_t I, const void* w_gate, const float* s_gate,
                                const void* w_up, const float* s_up, const void* w_down, const float* s_down,
                                void* h_sorted, void* workspace, size_t* workspace_bytes, hipStream_t stream) {
  return ffn_fp8w_call(true, x_sorted, x_rows, n_x, group_offsets, n_rows, E, n_shared, nseg, d, I, w_gate, s_gate, w_up,
                       s_up, w_down, s_down, h_sorted, workspace, workspace_bytes, stream);
}

moe_status moe_combine(const void* h_sorted, const int32_t* flat_to_sorted, const float* topk_w, int32_t T, int32_t k,
                       int32_t n_shared, int32_t d, moe_dtype dtype, void* y, hipStream_t stream) {
  if (T < 0 || k < 1 || n_shared < 0 || d < 1) return MOE_ERR_INVALID_ARG;
  if (!known_dtype(dtype) || d % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (!fits_int(static_cast<long long>(T) * (k + n_shared)) ||
      !fits_int(static_cast<long long>(T) * (k + n_shared) * (d / 8)))
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!h_sorted || !flat_to_sorted || !topk_w || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(h_sorted) || !aligned4(flat_to_sorted) || !aligned4(topk_w) || !aligned16(y))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_combine(h_sorted, flat_to_sorted, topk_w, T, k, n_shared, d,
                                        dtype == MOE_BF16 ? 1 : 0, y, stream));
}

moe_status moe_stats(const int32_t* topk_ids, int32_t L, int32_t T, int32_t k, int32_t E, const int32_t* req_offsets,
                     int32_t R, const float* idf, int32_t* counts, int32_t* union_size, uint8_t* union_mask,
                     int32_t* affinity, int32_t* req_counts, float* signature, void* workspace,
                     size_t* workspace_bytes, hipStream_t stream) {
  if (L < 0 || T < 0 || k < 1 || E < 1 || k > E || R < 0) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  if (!fits_int(static_cast<long long>(L) * T * k) || !fits_int(static_cast<long long>(L) * E * E) ||
      !fits_int(static_cast<long long>(R) * L * E))
    return MOE_ERR_UNSUPPORTED;
  if (L > 65535 || R > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  if ((req_counts || signature) && !req_offsets) return MOE_ERR_INVALID_ARG;
  bool query;
  moe_status st = workspace_check(workspace, workspace_bytes, moe::stats_workspace_bytes(L, T, k, E, R), &query);
  if (st != MOE_OK || query) return st;
  if (L == 0) return MOE_OK;
  if (!counts || !union_size) return MOE_ERR_INVALID_ARG;
  if (T > 0 && !topk_ids) return MOE_ERR_INVALID_ARG;
  if (!aligned4(counts) || !aligned4(union_size) || (topk_ids && !aligned4(topk_ids)) ||
      (affinity && !aligned4(affinity)) || (req_counts && !aligned4(req_counts)) ||
      (signature && !aligned4(signature)) || (req_offsets && !aligned4(req_offsets)) || (idf && !aligned4(idf)))
    return MOE_ERR_INVALID_ARG;
  moe::StatsArgs a;
  a.topk_ids = topk_ids;
  a.L = L;
  a.T = T;
  a.k = k;
  a.E = E;
  a.req_offsets = req_offsets;
  a.R = req_offsets ? R : 0;
  a.idf = idf;
  a.counts = counts;
  a.union_size = union_size;
  a.union_mask = union_mask;
  a.affinity = affinity;
  a.req_counts = req_counts;
  a.signature = signature;
  return hip_status(moe::launch_stats(a, workspace, stream));
}

}  // extern "C"
