// Device-side building blocks for the gfx950 (CDNA4) attention kernels.
//
// Matrix-core conventions used throughout (64-lane wavefront):
//   v_mfma_f32_32x32x16_{bf16,f16}: lane l supplies row (l % 32) of A and column
//   (l % 32) of B, each as 8 consecutive K-slots of half (l / 32); the 16
//   accumulators of lane l hold column (l % 32) of D at rows
//   8*(r/4) + 4*(l/32) + (r%4), r = 0..15.
//   v_mfma_f32_16x16x32_{bf16,f16}: lane l supplies row/column (l % 16) with
//   the 8 K-slots of quarter (l / 16); accumulator r of lane l is D[4*(l/16)+r][l%16].
//   v_mfma_f32_32x32x2_f32: lane l supplies A[l%32][l/32] and B[l/32][l%32].
// A and B always agree on which K index a (lane half, slot) pair carries, so a
// contraction may permute its K index freely as long as both operands use the
// same permutation; the kernels rely on this to feed softmax probabilities from
// the accumulator layout straight back into the next MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// 16-bit element traits: bf16 or fp16 storage, fp32 accumulation.
struct BF16 {
  static __device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  // Round two floats to nearest-even 16-bit values and pack (lo in bits 0..15).
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  // The low / high 16-bit value of a packed pair, exactly as a float.
  static __device__ __forceinline__ float lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return __builtin_bit_cast(float, w & 0xffff0000u);
  }
};

struct F16 {
  static __device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f16x2_t v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(f16x2_t, w)[0];
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(f16x2_t, w)[1];
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maxima that propagate NaN (v_maximum3_f32 / v_maximum_f32). Unlike fmaxf
// they need no quieting of their inputs, which costs an extra instruction per
// operand that the compiler cannot prove canonical (MFMA results, lane
// exchanges).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max3(float a, float b, float c) { return vmax(vmax(a, b), c); }

// Exchange with the lane 32 positions away (the other half of the wavefront).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

// Cross-half reductions without LDS: v_permlane32_swap(x, x) leaves, in every
// lane i, the values of lanes i % 32 and i % 32 + 32 in its two results.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return vmax(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Wait until every vector-memory load this wavefront issued has returned
// (s_waitcnt vmcnt(0); other counters untouched). Placed before a loop, it keeps
// the compiler from treating prologue loads as possibly in flight inside the
// loop, where in-order counting would otherwise stall on fresh prefetches.
__device__ __forceinline__ void vmem_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// True in every lane if `p` holds in any lane of the wavefront (uniform branch).
__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0; }

// Work order of a grid with one work item per workgroup. Items are (unit,
// block) pairs, a unit being a (batch, head) and block 0 the longest under a
// causal mask. The hardware hands workgroup ids to the 8 XCDs round-robin and,
// within an XCD, in increasing order, so workgroup k is the k-th item of that
// XCD's share. Items are numbered in groups of 32 units and, within a group,
// block-major (block 0 of each unit, then block 1, ...): every XCD gets the
// same mix of lengths and starts with its longest blocks, the short ones
// filling in at the end. When a group's unit count is a multiple of 8, the
// units an XCD receives are consecutive (adjacent heads: the query heads of a
// KV head), so what they share stays in that XCD's L2; otherwise they are
// dealt one by one.
struct GridItem {
  int unit, blk;
  bool valid;
};
__device__ __forceinline__ GridItem grid_item(int nblk, int nunit) {
  constexpr int GU = 32;  // units per group (a multiple of 8)
  const int k = blockIdx.x;
  GridItem w;
  w.valid = k < nblk * nunit;
  const int g = k / (GU * nblk);
  const int r = k - g * (GU * nblk);
  const int gu = min(GU, nunit - g * GU);  // units in this group
  w.blk = r / gu;
  const int u = r - w.blk * gu;             // lands on XCD u % 8 when gu % 8 == 0
  w.unit = g * GU + ((gu & 7) ? u : (u & 7) * (gu >> 3) + (u >> 3));
  return w;
}

// Raw buffer resource over [base, base + nbytes): loads past the end return
// zeros and stores past the end are dropped, with no branches in the kernel.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
}
__device__ __forceinline__ void buffer_store8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x2_t v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)byte_off, 0, 0);
}

// 16-byte load from a raw buffer straight into LDS (buffer_load_dwordx4 ...
// lds): lane j's 16 bytes land at lds_addr + 16*j, where lds_addr (a byte
// address in LDS) is wavefront-uniform. Out-of-range offsets read zeros. The
// compiler tracks the load like any other, so reads of that LDS region wait
// for it.
__device__ __forceinline__ void dma_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds_addr) {
  typedef __attribute__((address_space(3))) void lds_void_t;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(uintptr_t)lds_addr, 16, (int)voff, 0, 0, 0);
}

// LDS transposing read (gfx950 ds_read_b64_tr_b16). Within each group of 16
// lanes, lane i addresses 4 consecutive 16-bit elements of row i/4, columns
// 4*(i%4)..+3, of a 4 x 16 block; lane i receives column i of that block, i.e.
// the 4 elements of rows 0..3 at column i, packed low to high.
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

}  // namespace attn
