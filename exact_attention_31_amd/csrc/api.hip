// C-ABI entry points: argument checks, device checks, dispatch to the kernels.
// Nothing is enqueued unless every check passes; no allocation, no sync.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <utility>

#include "../../include/attn.h"
#include "attn_launch.h"

namespace {

constexpr int kMaxDevices = 64;
int g_dev_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other
int g_dev_cus[kMaxDevices];
std::mutex g_dev_mu;

// ATTN_OK if the current device is a gfx950; cached per device.
int check_device() {
  int dev = -1;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return ATTN_ERR_NO_DEVICE;
  }
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return ATTN_ERR_NO_DEVICE;
  }
  if (dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) {
      (void)hipGetLastError();
      return ATTN_ERR_NO_DEVICE;
    }
    g_dev_ok[dev] = (strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    g_dev_cus[dev] = p.multiProcessorCount;
  }
  return g_dev_ok[dev] == 1 ? ATTN_OK : ATTN_ERR_UNSUPPORTED;
}

// ---- tuning knobs: defaults from ATTN_TUNING ("name=value,name=value"), read
// once per process; attn_set_tuning changes them afterwards.
std::atomic<int> g_tune[attn::kTuneCount];
std::once_flag g_tune_once;
const char* const kTuneNames[attn::kTuneCount] = {"prefill_variant", "prefill_slots", "decode_chunk",
                                                  "decode_groups", "decode_rows_mode"};

bool tune_valid(int knob, long v) {
  switch (knob) {
    case attn::kTunePrefillVariant: return v >= 0 && v <= 5;
    case attn::kTunePrefillSlots: return v >= 0 && v <= (1L << 20);
    case attn::kTuneDecodeChunk: return v >= 0 && v <= (1L << 24);
    case attn::kTuneDecodeGroups: return v == 0 || v == 1 || v == 2 || v == 4;
    case attn::kTuneDecodeRowsMode: return v >= 0 && v <= 2;
    default: return false;
  }
}

void tune_init() {
  const char* e = getenv("ATTN_TUNING");
  if (e == nullptr) return;
  // entries that do not parse, name no knob or hold an invalid value are ignored
  while (*e) {
    const char* end = strchr(e, ',');
    const size_t n = end ? (size_t)(end - e) : strlen(e);
    const char* eq = (const char*)memchr(e, '=', n);
    if (eq != nullptr) {
      for (int k = 0; k < attn::kTuneCount; ++k) {
        const size_t kl = strlen(kTuneNames[k]);
        if ((size_t)(eq - e) == kl && strncmp(e, kTuneNames[k], kl) == 0) {
          char* stop = nullptr;
          const long v = strtol(eq + 1, &stop, 10);
          if (stop == e + n && stop != eq + 1 && tune_valid(k, v)) g_tune[k].store((int)v);
        }
      }
    }
    e += n;
    if (*e == ',') ++e;
  }
}

// ---- occupancy per (kernel, device)
std::map<std::pair<const void*, int>, int> g_occ;
std::mutex g_occ_mu;

// ---- the no-allocation decode entry point's scratch: one array per device,
// held for the life of the process. Host code never uses the array's name as
// an address: the device address comes from hipGetSymbolAddress, once per
// device with that device current, and is kept in g_scratch.
constexpr size_t kScratchBytes = ATTN_DECODE_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
void* g_scratch[kMaxDevices];  // guarded by g_dev_mu

int scratch_of_device(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return ATTN_ERR_LAUNCH;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return ATTN_OK;
}

size_t elem_size(int dtype) { return dtype == ATTN_F32 ? 4 : 2; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const char* pa = (const char*)a;
  const char* pb = (const char*)b;
  return pa < pb + nb && pb < pa + na;
}

// Shared shape checks. Returns ATTN_OK or an error code.
int check_common(int B, int H_q, int H_kv, int N_q, int N_kv, int d, int dtype, float scale) {
  if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (B < 0 || H_q < 0 || H_kv < 0 || N_q < 0 || N_kv < 0 || d < 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (H_kv == 0 || H_q % H_kv != 0 || (H_q == 0 && B > 0 && N_q > 0)) return ATTN_ERR_GQA;
  if (B > 65535 || H_q > 65535) return ATTN_ERR_SHAPE;
  // the kernels take the running maximum of raw scores and mask with -inf, which
  // presumes a positive scale (the attention scale is 1/sqrt(d))
  if (!isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_VALUE;
  return ATTN_OK;
}

}  // namespace

namespace attn {

int tuning(int knob) {
  std::call_once(g_tune_once, tune_init);
  return (knob >= 0 && knob < kTuneCount) ? g_tune[knob].load(std::memory_order_relaxed) : 0;
}

int occupancy_per_cu(const void* kernel, int threads, int device) {
  std::lock_guard<std::mutex> lk(g_occ_mu);
  const auto key = std::make_pair(kernel, device);
  auto it = g_occ.find(key);
  if (it != g_occ.end()) return it->second;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    n = 1;
  }
  g_occ[key] = n;
  return n;
}

}  // namespace attn

extern "C" {

int attn_set_tuning(int knob, int value) {
  if (knob < 0 || knob >= attn::kTuneCount) return ATTN_ERR_VALUE;
  if (!tune_valid(knob, value)) return ATTN_ERR_VALUE;
  std::call_once(g_tune_once, tune_init);
  g_tune[knob].store(value, std::memory_order_relaxed);
  return ATTN_OK;
}

int attn_get_tuning(int knob) {
  if (knob < 0 || knob >= attn::kTuneCount) return -1;
  return attn::tuning(knob);
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid sizes";
    case ATTN_ERR_GQA: return "H_q must be a positive multiple of H_kv";
    case ATTN_ERR_UNSUPPORTED: return "unsupported dtype, head dim, query length or device";
    case ATTN_ERR_WORKSPACE: return "decode workspace missing or too small";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_NO_DEVICE: return "no HIP device available";
    case ATTN_ERR_ALIAS: return "an output overlaps an input";
    case ATTN_ERR_VALUE: return "scale is not positive and finite, or causal is not 0 or 1";
    default: return "unknown status";
  }
}

int attn_version(void) { return 100; }

int attn_prefill_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H_q, int H_kv, int N_q, int N_kv, int d, int causal, float scale,
                     int dtype, void* stream) {
  int st = check_common(B, H_q, H_kv, N_q, N_kv, d, dtype, scale);
  if (st != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_VALUE;
  // one workgroup per (batch, head, 128-row query block) on a 1-D grid
  if ((int64_t)((N_q + 127) / 128) * H_q * B > 0x7ffffff0LL) return ATTN_ERR_SHAPE;
  // per-head byte offsets are 32-bit (buffer addressing)
  if ((int64_t)N_q * d * elem_size(dtype) > 0xffffffffLL ||
      (int64_t)N_kv * d * elem_size(dtype) > 0xffffffffLL)
    return ATTN_ERR_SHAPE;
  if (B == 0 || H_q == 0 || N_q == 0) return ATTN_OK;
  if (q == nullptr || o == nullptr) return ATTN_ERR_NULL;
  if (N_kv > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_NULL;
  const size_t es = elem_size(dtype);
  const size_t nq = (size_t)B * H_q * N_q * d * es;
  const size_t nkv = (size_t)B * H_kv * N_kv * d * es;
  const size_t nl = (size_t)B * H_q * N_q * sizeof(float);
  if (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nkv) || overlaps(o, nq, v, nkv) ||
      overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nkv) || overlaps(lse, nl, v, nkv) ||
      overlaps(lse, nl, o, nq))
    return ATTN_ERR_ALIAS;
  st = check_device();
  if (st != ATTN_OK) return st;
  int dev = 0;
  (void)hipGetDevice(&dev);
  attn::PrefillArgs a{q, k, v, o, lse, B, H_q, H_kv, N_q, N_kv, d, causal, scale, dtype, g_dev_cus[dev],
                      dev};
  return attn::launch_prefill(a, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

size_t attn_decode_workspace_size(int B, int H_q, int H_kv, int N_q, int N_kv, int d, int dtype) {
  if (check_common(B, H_q, H_kv, N_q, N_kv, d, dtype, 1.f) != ATTN_OK) return 0;
  if (N_q < 1 || N_q > attn::kDecodeMaxNq) return 0;
  return attn::decode_plan(B, H_q, H_kv, N_q, N_kv, d, false).workspace_bytes;
}

namespace {

bool valid_block_size(int bs) { return bs >= 16 && bs <= 4096 && (bs & (bs - 1)) == 0; }

int log2_of(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

// Shared validation and launch of both decode entry points. For a paged cache
// (table != null) k and v are pools of kv_bytes each and N_kv = max_blocks *
// block_size; for a contiguous cache they are [B, H_kv, N_kv, d].
int decode_launch(const void* q, const void* k, const void* v, size_t kv_bytes, const int* table,
                  int max_blocks, int block_size, int num_blocks, const int* kv_lens, void* o,
                  float* lse, int B, int H_q, int H_kv, int N_q, int N_kv, int d, int causal,
                  float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream,
                  bool kv_fp8 = false, float k_scale = 1.f, float v_scale = 1.f,
                  bool use_scratch = false) {
  const bool paged = table != nullptr || block_size != 0;
  int st = check_common(B, H_q, H_kv, N_q, N_kv, d, dtype, scale);
  if (st != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_VALUE;
  if (dtype == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (kv_fp8) {
    if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (!isfinite(k_scale) || !(k_scale > 0.f) || !isfinite(v_scale) || !(v_scale > 0.f))
      return ATTN_ERR_VALUE;
  }
  if (N_q > attn::kDecodeMaxNq) return ATTN_ERR_UNSUPPORTED;
  if (B == 0 || H_q == 0 || N_q == 0) return ATTN_OK;
  if (q == nullptr || o == nullptr) return ATTN_ERR_NULL;
  if (paged) {
    if (max_blocks > 0 && table == nullptr) return ATTN_ERR_NULL;
    if (num_blocks > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_NULL;
  } else if (N_kv > 0 && (k == nullptr || v == nullptr)) {
    return ATTN_ERR_NULL;
  }
  const attn::DecodePlan plan =
      attn::decode_plan(B, H_q, H_kv, N_q, N_kv, d, paged, use_scratch ? kScratchBytes : 0);
  // partial rows and work units are indexed with 32-bit integers
  const int64_t groups = ((int64_t)(H_q / H_kv) * N_q + 15) / 16;
  if ((int64_t)B * H_q * N_q * plan.splits > 0x3fffffffLL ||
      (int64_t)B * H_kv * groups * plan.splits > 0x3fffffffLL)
    return ATTN_ERR_SHAPE;
  // contiguous caches: per-head byte offsets are 32-bit (buffer addressing)
  if (!paged && (int64_t)N_kv * d * (kv_fp8 ? 1 : elem_size(dtype)) > 0xffffffffLL)
    return ATTN_ERR_SHAPE;
  if (use_scratch) {
    if (plan.workspace_bytes > kScratchBytes) return ATTN_ERR_WORKSPACE;
  } else if (workspace == nullptr || workspace_bytes < plan.workspace_bytes) {
    return ATTN_ERR_WORKSPACE;
  }
  const size_t es = elem_size(dtype);
  const size_t nq = (size_t)B * H_q * N_q * d * es;
  const size_t nkv = kv_bytes;
  const size_t nl = (size_t)B * H_q * N_q * sizeof(float);
  const size_t nw = plan.workspace_bytes;
  const size_t nt = paged ? (size_t)B * max_blocks * sizeof(int) : 0;
  const size_t nlen = (size_t)B * sizeof(int);
  if (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nkv) || overlaps(o, nq, v, nkv) ||
      overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nkv) || overlaps(lse, nl, v, nkv) ||
      overlaps(lse, nl, o, nq) || overlaps(workspace, nw, q, nq) ||
      overlaps(workspace, nw, k, nkv) || overlaps(workspace, nw, v, nkv) ||
      overlaps(workspace, nw, o, nq) || overlaps(workspace, nw, lse, nl) ||
      overlaps(kv_lens, nlen, o, nq) || overlaps(kv_lens, nlen, workspace, nw) ||
      overlaps(kv_lens, nlen, lse, nl) || overlaps(table, nt, o, nq) ||
      overlaps(table, nt, lse, nl) || overlaps(table, nt, workspace, nw))
    return ATTN_ERR_ALIAS;
  st = check_device();
  if (st != ATTN_OK) return st;
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (use_scratch) {
    st = scratch_of_device(dev, &workspace);
    if (st != ATTN_OK) return st;
  }
  float* ws = (float*)workspace;
  // Many query rows per KV head (G * N_q, several new tokens) and enough
  // of them to fill the device: the rows are a tall product, better served by
  // the prefill kernel in rows mode (32x32 MFMA tiles, K/V shared through LDS)
  // than by the split-KV decode kernel. The decode_rows_mode knob forces it
  // on (1) or off (2) (contiguous 16-bit caches only).
  if (!paged && !kv_fp8) {
    const int rows = (H_q / H_kv) * N_q;
    const int bm = d == 128 ? 256 : 128;  // query rows per prefill workgroup
    const int64_t items = (int64_t)B * H_kv * ((rows + bm - 1) / bm);
    // at least half a workgroup's rows (padding rows cost as much as real ones)
    bool rows_mode = 2 * rows >= bm && items >= (g_dev_cus[dev] > 0 ? g_dev_cus[dev] : 256);
    const int forced = attn::tuning(attn::kTuneDecodeRowsMode);
    if (forced != 0) rows_mode = forced == 1;
    if (rows_mode) {
      attn::PrefillArgs pa{q, k, v, o, lse, B, H_kv, H_kv, rows, N_kv, d, causal, scale, dtype,
                           g_dev_cus[dev], dev};
      return attn::launch_prefill_rows(pa, kv_lens, N_q, (hipStream_t)stream) == hipSuccess
                 ? ATTN_OK
                 : ATTN_ERR_LAUNCH;
    }
  }
  attn::DecodeArgs a{q, k, v, kv_lens, o, lse, B, H_q, H_kv, N_q, N_kv, d, causal, scale, dtype,
                     plan.chunk, plan.splits, plan.chunk_cap, g_dev_cus[dev], ws,
                     ws + (size_t)B * H_q * N_q * plan.splits * d,
                     paged ? table : nullptr, max_blocks, paged ? log2_of(block_size) : 0,
                     num_blocks, kv_fp8 ? 1 : 0, k_scale, v_scale};
  return attn::launch_decode(a, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// Checks the paged sizes and returns N_kv = max_blocks * block_size, or -1.
int64_t paged_capacity(int max_blocks, int block_size, int num_blocks) {
  if (max_blocks < 0 || num_blocks < 0) return -1;
  if (!valid_block_size(block_size)) return -2;
  const int64_t n = (int64_t)max_blocks * block_size;
  return n > (1LL << 30) ? -1 : n;
}

}  // namespace

int attn_decode_fwd(const void* q, const void* k_cache, const void* v_cache, const int* kv_lens,
                    void* o, float* lse, int B, int H_q, int H_kv, int N_q, int N_kv, int d,
                    int causal, float scale, int dtype, void* workspace, size_t workspace_bytes,
                    void* stream) {
  const size_t nkv =
      (B > 0 && H_kv > 0 && N_kv > 0 && d > 0) ? (size_t)B * H_kv * N_kv * d * elem_size(dtype) : 0;
  return decode_launch(q, k_cache, v_cache, nkv, nullptr, 0, 0, 0, kv_lens, o, lse, B, H_q, H_kv,
                       N_q, N_kv, d, causal, scale, dtype, workspace, workspace_bytes, stream);
}

int attn_decode_fwd_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int* kv_lens, void* o, float* lse, int B, int H_q, int H_kv,
                            int N_q, int N_kv, int d, int causal, float scale, int dtype,
                            void* stream) {
  const size_t nkv =
      (B > 0 && H_kv > 0 && N_kv > 0 && d > 0) ? (size_t)B * H_kv * N_kv * d * elem_size(dtype) : 0;
  return decode_launch(q, k_cache, v_cache, nkv, nullptr, 0, 0, 0, kv_lens, o, lse, B, H_q, H_kv,
                       N_q, N_kv, d, causal, scale, dtype, nullptr, 0, stream, false, 1.f, 1.f, true);
}

size_t attn_decode_paged_workspace_size(int B, int H_q, int H_kv, int N_q, int max_blocks,
                                        int block_size, int d, int dtype) {
  const int64_t n = paged_capacity(max_blocks, block_size, 1);
  if (n < 0) return 0;
  if (check_common(B, H_q, H_kv, N_q, (int)n, d, dtype, 1.f) != ATTN_OK) return 0;
  if (N_q < 1 || N_q > attn::kDecodeMaxNq) return 0;
  return attn::decode_plan(B, H_q, H_kv, N_q, (int)n, d, true).workspace_bytes;
}

int attn_decode_paged_fwd(const void* q, const void* k_pool, const void* v_pool,
                          const int* block_table, const int* kv_lens, void* o, float* lse, int B,
                          int H_q, int H_kv, int N_q, int max_blocks, int block_size,
                          int num_blocks, int d, int causal, float scale, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
  const int64_t n = paged_capacity(max_blocks, block_size, num_blocks);
  if (n == -2) return ATTN_ERR_UNSUPPORTED;
  if (n < 0) return ATTN_ERR_SHAPE;
  const size_t npool = (num_blocks > 0 && H_kv > 0 && d > 0)
                           ? (size_t)num_blocks * H_kv * block_size * d * 2
                           : 0;
  return decode_launch(q, k_pool, v_pool, npool, block_table, max_blocks, block_size, num_blocks,
                       kv_lens, o, lse, B, H_q, H_kv, N_q, (int)n, d, causal, scale, dtype,
                       workspace, workspace_bytes, stream);
}

int attn_decode_fp8_fwd(const void* q, const void* k_cache, const void* v_cache, float k_scale,
                        float v_scale, const int* kv_lens, void* o, float* lse, int B, int H_q,
                        int H_kv, int N_q, int N_kv, int d, int causal, float scale, int dtype,
                        void* workspace, size_t workspace_bytes, void* stream) {
  const size_t nkv = (B > 0 && H_kv > 0 && N_kv > 0 && d > 0) ? (size_t)B * H_kv * N_kv * d : 0;
  return decode_launch(q, k_cache, v_cache, nkv, nullptr, 0, 0, 0, kv_lens, o, lse, B, H_q, H_kv,
                       N_q, N_kv, d, causal, scale, dtype, workspace, workspace_bytes, stream, true,
                       k_scale, v_scale);
}

int attn_decode_paged_fp8_fwd(const void* q, const void* k_pool, const void* v_pool,
                              float k_scale, float v_scale, const int* block_table,
                              const int* kv_lens, void* o, float* lse, int B, int H_q, int H_kv,
                              int N_q, int max_blocks, int block_size, int num_blocks, int d,
                              int causal, float scale, int dtype, void* workspace,
                              size_t workspace_bytes, void* stream) {
  const int64_t n = paged_capacity(max_blocks, block_size, num_blocks);
  if (n == -2) return ATTN_ERR_UNSUPPORTED;
  if (n < 0) return ATTN_ERR_SHAPE;
  const size_t npool =
      (num_blocks > 0 && H_kv > 0 && d > 0) ? (size_t)num_blocks * H_kv * block_size * d : 0;
  return decode_launch(q, k_pool, v_pool, npool, block_table, max_blocks, block_size, num_blocks,
                       kv_lens, o, lse, B, H_q, H_kv, N_q, (int)n, d, causal, scale, dtype,
                       workspace, workspace_bytes, stream, true, k_scale, v_scale);
}

size_t attn_backward_workspace_size(int B, int H_q, int H_kv, int N_q, int N_kv, int d, int dtype) {
  if (check_common(B, H_q, H_kv, N_q, N_kv, d, dtype, 1.f) != ATTN_OK) return 0;
  return (size_t)2 * B * H_q * N_q * sizeof(float);
}

int attn_backward(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                  const float* lse, void* dq, void* dk, void* dv, int B, int H_q, int H_kv,
                  int N_q, int N_kv, int d, int causal, float scale, int dtype, void* workspace,
                  size_t workspace_bytes, void* stream) {
  int st = check_common(B, H_q, H_kv, N_q, N_kv, d, dtype, scale);
  if (st != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_VALUE;
  if (dtype == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  // 1-D grids of 128-row / 128-key blocks; per-head byte offsets are 32-bit
  if ((int64_t)((N_q + 127) / 128) * H_q * B > 0x7ffffff0LL ||
      (int64_t)((N_kv + 127) / 128) * H_kv * B > 0x7ffffff0LL)
    return ATTN_ERR_SHAPE;
  if ((int64_t)N_q * d * 2 > 0xffffffffLL || (int64_t)N_kv * d * 2 > 0xffffffffLL)
    return ATTN_ERR_SHAPE;
  if (B == 0 || H_q == 0 || (N_q == 0 && N_kv == 0)) return ATTN_OK;
  if (N_q > 0 && (q == nullptr || o == nullptr || d_o == nullptr || lse == nullptr || dq == nullptr))
    return ATTN_ERR_NULL;
  if (N_kv > 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr))
    return ATTN_ERR_NULL;
  const size_t need = (size_t)2 * B * H_q * N_q * sizeof(float);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  const size_t es = elem_size(dtype);
  const size_t nq = (size_t)B * H_q * N_q * d * es;
  const size_t nkv = (size_t)B * H_kv * N_kv * d * es;
  const size_t nl = (size_t)B * H_q * N_q * sizeof(float);
  const void* ins[6] = {q, k, v, o, d_o, lse};
  const size_t in_sz[6] = {nq, nkv, nkv, nq, nq, nl};
  void* outs[4] = {dq, dk, dv, workspace};
  const size_t out_sz[4] = {nq, nkv, nkv, need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_sz[i], ins[j], in_sz[j])) return ATTN_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_sz[i], outs[j], out_sz[j])) return ATTN_ERR_ALIAS;
  }
  st = check_device();
  if (st != ATTN_OK) return st;
  float* ws = (float*)workspace;
  attn::BackwardArgs a{q, k, v, o, d_o, lse, dq, dk, dv, B, H_q, H_kv, N_q, N_kv, d, causal,
                       scale, dtype, ws, ws + (size_t)B * H_q * N_q};
  return attn::launch_backward(a, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // extern "C"
