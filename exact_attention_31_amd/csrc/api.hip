// C-ABI entry points: argument checks, device checks, dispatch to the kernels.
// Nothing is enqueued unless every check passes; no allocation, no sync.
#include <math.h>
#include <string.h>

#include <mutex>

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

extern "C" {

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
  attn::PrefillArgs a{q, k, v, o, lse, B, H_q, H_kv, N_q, N_kv, d, causal, scale, dtype};
  return attn::launch_prefill(a, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

size_t attn_decode_workspace_size(int B, int H_q, int H_kv, int N_q, int N_kv, int d, int dtype) {
  if (check_common(B, H_q, H_kv, N_q, N_kv, d, dtype, 1.f) != ATTN_OK) return 0;
  if (N_q < 1 || N_q > attn::kDecodeMaxNq) return 0;
  return attn::decode_plan(B, H_q, H_kv, N_q, N_kv, d).workspace_bytes;
}

int attn_decode_fwd(const void* q, const void* k_cache, const void* v_cache, const int* kv_lens,
                    void* o, float* lse, int B, int H_q, int H_kv, int N_q, int N_kv, int d,
                    int causal, float scale, int dtype, void* workspace, size_t workspace_bytes,
                    void* stream) {
  int st = check_common(B, H_q, H_kv, N_q, N_kv, d, dtype, scale);
  if (st != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_VALUE;
  if (dtype == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (N_q > attn::kDecodeMaxNq) return ATTN_ERR_UNSUPPORTED;
  if (B == 0 || H_q == 0 || N_q == 0) return ATTN_OK;
  if (q == nullptr || o == nullptr) return ATTN_ERR_NULL;
  if (N_kv > 0 && (k_cache == nullptr || v_cache == nullptr)) return ATTN_ERR_NULL;
  const attn::DecodePlan plan = attn::decode_plan(B, H_q, H_kv, N_q, N_kv, d);
  // partial rows and work units are indexed with 32-bit integers
  const int64_t groups = ((int64_t)(H_q / H_kv) * N_q + 15) / 16;
  if ((int64_t)B * H_q * N_q * plan.splits > 0x3fffffffLL ||
      (int64_t)B * H_kv * groups * plan.splits > 0x3fffffffLL)
    return ATTN_ERR_SHAPE;
  if ((int64_t)N_kv * d * elem_size(dtype) > 0xffffffffLL) return ATTN_ERR_SHAPE;
  if (workspace == nullptr || workspace_bytes < plan.workspace_bytes) return ATTN_ERR_WORKSPACE;
  const size_t es = elem_size(dtype);
  const size_t nq = (size_t)B * H_q * N_q * d * es;
  const size_t nkv = (size_t)B * H_kv * N_kv * d * es;
  const size_t nl = (size_t)B * H_q * N_q * sizeof(float);
  const size_t nw = plan.workspace_bytes;
  if (overlaps(o, nq, q, nq) || overlaps(o, nq, k_cache, nkv) || overlaps(o, nq, v_cache, nkv) ||
      overlaps(lse, nl, q, nq) || overlaps(lse, nl, k_cache, nkv) ||
      overlaps(lse, nl, v_cache, nkv) || overlaps(lse, nl, o, nq) ||
      overlaps(workspace, nw, q, nq) || overlaps(workspace, nw, k_cache, nkv) ||
      overlaps(workspace, nw, v_cache, nkv) || overlaps(workspace, nw, o, nq) ||
      overlaps(workspace, nw, lse, nl) || overlaps(kv_lens, (size_t)B * 4, o, nq) ||
      overlaps(kv_lens, (size_t)B * 4, workspace, nw) || overlaps(kv_lens, (size_t)B * 4, lse, nl))
    return ATTN_ERR_ALIAS;
  st = check_device();
  if (st != ATTN_OK) return st;
  float* ws = (float*)workspace;
  int dev = 0;
  (void)hipGetDevice(&dev);
  attn::DecodeArgs a{q, k_cache, v_cache, kv_lens, o, lse, B, H_q, H_kv, N_q, N_kv, d, causal,
                     scale, dtype, plan.chunk, plan.splits, g_dev_cus[dev], ws,
                     ws + (size_t)B * H_q * N_q * plan.splits * d};
  return attn::launch_decode(a, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // extern "C"
