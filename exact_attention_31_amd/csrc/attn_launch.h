// Host-side launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>

namespace attn {

// Tuning knobs (attn_set_tuning, or the ATTN_TUNING environment variable read
// once per process). Never needed for correctness: every setting gives the
// same results up to rounding. 0 = automatic.
enum TuneKnob {
  kTunePrefillVariant = 0,  // 1..5: alternative prefill kernel forms
  kTunePrefillSlots = 1,    // n > 0: persistent prefill grid with at most n workgroups
  kTuneDecodeChunk = 2,     // n > 0: keys per decode split (rounded up to 128), no device raise
  kTuneDecodeGroups = 3,    // 1, 2 or 4: query column groups per decode wavefront
  kTuneDecodeRowsMode = 4,  // 1: multi-token decode through the prefill kernel; 2: never
  kTuneCount = 5
};
int tuning(int knob);

// Resident workgroups of `kernel` (launched with `threads` threads) per compute
// unit of device `device`, cached per (kernel, device).
int occupancy_per_cu(const void* kernel, int threads, int device);

// Launches `kernel` with `args` converted to its parameter types and returns
// the status of this launch alone (no earlier error is picked up).
template <typename... P, typename... A>
hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, A... args) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> vals{static_cast<P>(args)...};
  return std::apply(
      [&](auto&... v) {
        void* ptrs[] = {(void*)&v...};
        return hipLaunchKernel((const void*)kernel, grid, block, ptrs, 0, stream);
      },
      vals);
}

constexpr int kDtypeF32 = 0;
constexpr int kDtypeF16 = 1;
constexpr int kDtypeBF16 = 2;

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H_q, H_kv, N_q, N_kv, d;
  int causal;
  float scale;
  int dtype;
  int num_cus;  // compute units of the device (sizes persistent grids)
  int device;   // HIP device index (occupancy cache)
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int* kv_lens;  // device pointer or null (all N_kv)
  void* o;
  float* lse;
  int B, H_q, H_kv, N_q, N_kv, d;
  int causal;
  float scale;
  int dtype;
  int chunk;      // keys per split (the plan's; sizes the workspace)
  int splits;     // splits per (request, KV head), = ceil(N_kv / chunk)
  int chunk_cap;  // the kernels may raise the split up to this many keys (>= chunk)
  int num_cus; // compute units of the device (sizes the persistent grid)
  float* part_u;   // [B, H_q, N_q, splits, d] un-normalised partial outputs
  float* part_ml;  // [B, H_q, N_q, splits, 2] partial (max in log2 units, denominator)
  // paged caches (block_table non-null): k and v are pools
  // [num_blocks, H_kv, block_size, d]; N_kv = max_blocks * block_size
  const int* block_table;  // [B, max_blocks]
  int max_blocks;
  int block_size_log2;
  int num_blocks;
  // FP8 E4M3 caches (kv_fp8 != 0): one byte per element, value = code * scale
  int kv_fp8;
  float k_scale, v_scale;
};

// Split plan shared by the workspace query and the launch.
struct DecodePlan {
  int chunk;
  int splits;
  int chunk_cap;  // largest split the kernels may choose from the actual lengths
  size_t workspace_bytes;
};
// max_workspace > 0: if the plan's partials would exceed that many bytes, the
// split is coarsened (contiguous caches) until they fit; a plan whose single
// split still does not fit keeps workspace_bytes > max_workspace.
DecodePlan decode_plan(int B, int H_q, int H_kv, int N_q, int N_kv, int d, bool paged,
                       size_t max_workspace = 0);
constexpr int kDecodeMaxNq = 64;  // query tokens per request the decode path takes

struct BackwardArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* d_o;
  const float* lse;  // [B, H_q, N_q] natural log, from the forward pass
  void* dq;
  void* dk;
  void* dv;
  int B, H_q, H_kv, N_q, N_kv, d;
  int causal;
  float scale;
  int dtype;
  float* lse2;   // workspace [B, H_q, N_q]: lse in log2 units (+inf for empty rows)
  float* delta;  // workspace [B, H_q, N_q]: rowsum(dO * O)
};

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// Prefill kernel in rows mode: a.N_q rows per "head" are row_period tokens of
// a.N_q / row_period query heads; kv_lens (nullable) bounds each request's keys.
hipError_t launch_prefill_rows(const PrefillArgs& a, const int* kv_lens, int row_period,
                               hipStream_t stream);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

}  // namespace attn
