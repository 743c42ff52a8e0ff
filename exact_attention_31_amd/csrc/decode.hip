// Decode attention forward on gfx950: one query token per request against a
// KV cache, grouped-query (G = H_q / H_kv query heads share a KV head).
//
// Decode is the phase whose matrix product has only G rows and which is bound by
// HBM bandwidth (code-journey.com attention co-design summary, prefill/decode
// table and "Group Size(G)"): every cached key and value byte is read once and
// reused by the G query heads of its group. To give 256 compute units enough
// independent streams, the KV sequence is split into chunks; each chunk yields
// per-head partial statistics (max m_s, denominator l_s, un-normalised output
// u_s), and a second kernel merges them with weights exp(m_s - m), the same
// rescaling that the online softmax applies between blocks (auturnal.com
// transformer-attention guide, section 8), applied across partitions.
//
// gfx950 mapping: a persistent grid of wavefronts takes (request, KV head,
// chunk) units round-robin; a wavefront streams its chunk 32 keys per step with
// the next step's loads in flight. K rows go straight from HBM
// into the A operand of S^T = K Q^T (v_mfma_f32_16x16x32, 16-byte loads); the
// group's query heads form the B operand (padded to 16 columns). V rows are
// staged in LDS and read back transposed (ds_read_b64_tr_b16) as the A operand
// of O^T = V^T P^T, so each lane's accumulators belong to one query head.
#include <stdlib.h>

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr int kThreads = 256;
constexpr int kWaveKeys = 32;            // keys per wavefront step
constexpr int kStepKeys = 4 * kWaveKeys; // keys per workgroup step
constexpr int kQCols = 16;               // query rows per column group (MFMA N)
constexpr float kLazyRescale = 8.f;      // rescale threshold, log2 units

// Orders this wavefront's LDS writes before its later LDS reads (the lanes of a
// wavefront exchange V rows through LDS; no other wavefront touches them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D> struct DecLds {
  static constexpr int VST = D + 16;              // row stride of staged V rows
  static constexpr int kV = 4 * kWaveKeys * VST;  // V staging, 4 wavefronts (elements)
};

// Where one request's cached rows live. Contiguous caches are
// [B, H_kv, N_kv, d]. Paged caches are a pool of fixed-size blocks
// [num_blocks, H_kv, block_size, d] plus a per-request block table
// [B, max_blocks] that maps logical block i (positions i*block_size ..
// (i+1)*block_size - 1) to a physical block of the pool. Elements are 16-bit
// (the query's type) or FP8 E4M3 codes.
struct KvSrc {
  const uint8_t* k;
  const uint8_t* v;
  const int* table;     // paged only
  int max_blocks;       // paged only: table row length
  int bs_log2;          // paged only: log2(block_size), block_size >= 16
  int num_blocks;       // paged only: pool size in blocks
};

struct SplitParams {
  const uint16_t* q;
  KvSrc kv;
  const int* kv_lens;
  float* part_u;
  float* part_ml;
  int B, H_q, H_kv, N_q, N_kv, causal, chunk, chunk_cap;
  float scale_log2;  // softmax scale * log2(e) (times the K dequantisation scale for FP8)
};

// Keys per work unit, chosen on the device from the requests' actual lengths.
// The host plan's chunk sizes the workspace (ceil(N_kv / chunk) partials per
// query row); a larger chunk never needs more. The split grows from the
// batch's keys per wavefront (at least the plan's chunk, at most cap) until
// the units of the whole batch number at most one per wavefront of the grid:
// every wavefront still gets a unit (short requests in a long cache spread
// over the whole grid), no wavefront gets two (which would double its time),
// and the per-unit costs (start-up, the partial results and their merge) are
// paid as few times as possible. Each lane reads the lengths of requests
// lane, lane + 64, ... at once, and the sums are wavefront reductions; the
// unit counts use a float reciprocal (a heuristic needs no exact division).
// The result is a pure function of the arguments: the merge kernel evaluates
// it on the same inputs as the split kernel. Above kAdaptMaxB requests the
// plan's chunk is kept. Called by all 64 lanes of a wavefront.
constexpr int kAdaptMaxB = 1024;
__device__ int unit_chunk(const int* __restrict__ kv_lens, int B, int N_kv, int chunk, int cap,
                          int HG, int nwaves) {
  if (cap <= chunk || B > kAdaptMaxB || nwaves <= 0) return chunk;
  constexpr int PER = kAdaptMaxB / 64;
  const int lane = (int)threadIdx.x & 63;
  float len[PER];
  float total = 0.f, nb = 0.f;
  int lo = N_kv, hi = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int b = lane + 64 * i;
    const int n = b < B ? min(max(kv_lens ? kv_lens[b] : N_kv, 0), N_kv) : -1;
    len[i] = (float)max(n, 0);
    total += len[i];
    nb += n > 0 ? 1.f : 0.f;
    if (n >= 0) {
      lo = min(lo, n);
      hi = max(hi, n);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    total += __shfl_xor(total, o);
    nb += __shfl_xor(nb, o);
    lo = min(lo, __shfl_xor(lo, o));
    hi = max(hi, __shfl_xor(hi, o));
  }
  // every lane holds the reductions; taking lane 0's keeps the decisions (and
  // the result) in scalar registers
  total = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, total)));
  nb = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, nb)));
  lo = __builtin_amdgcn_readfirstlane(lo);
  hi = __builtin_amdgcn_readfirstlane(hi);
  if (total == 0.f) return chunk;
  // first guess: the batch's keys over the wavefronts; with unequal lengths
  // each request's last unit is on average half full, so the units of
  // nb / 2 requests' worth of wavefronts are set aside (usually no step of
  // the search below is then needed)
  const float wv = lo == hi ? (float)nwaves : fmaxf((float)nwaves - 0.5f * nb * (float)HG, 0.5f * (float)nwaves);
  const float cf = fminf(ceilf(total * (float)HG / wv), (float)cap);
  int c = ((int)cf + kStepKeys - 1) / kStepKeys * kStepKeys;
  c = c < chunk ? chunk : (c > cap ? cap : c);
  for (int it = 0; it < 32 && c < cap; ++it) {
    const float rc = 1.f / (float)c;
    float units = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) units += ceilf(len[i] * rc);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) units += __shfl_xor(units, o);
    units = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, units)));
    if (units * (float)HG <= (float)nwaves) break;
    const int step = (c / 16 + kStepKeys - 1) / kStepKeys * kStepKeys;
    c = c + step > cap ? cap : c + step;
  }
  return c;
}

// Four FP8 E4M3 codes (one dword) to four bf16 values (two dwords), exactly:
// every E4M3 value is a bf16 value.
__device__ __forceinline__ u32x2_t fp8x4_to_bf16(uint32_t w) {
  const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return u32x2_t{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// One work unit, done by one wavefront alone: keys [split*chunk,
// min((split+1)*chunk, len)) of request b for KV head hk and query column
// groups NG*qg .. NG*qg + NG-1 (16 columns each). Writes that chunk's partial
// (u, m, l) for the groups' query rows. The NG groups share every K register
// and every V operand read from LDS; only the matrix products are per group.
// FP8: K and V are E4M3 codes, widened to bf16 in registers (K) or on their way
// into LDS (V); the dequantisation scales are applied to the score scale and,
// in the merge, to the output.
template <class TT, int D, int NG, bool PAGED, bool FP8>
__device__ __forceinline__ void wave_unit(const SplitParams& P, int chunk, int nsplit, int b, int hk,
                                          int qg, int split, int len, uint16_t* sV) {
  constexpr int VST = DecLds<D>::VST;
  constexpr int KS = D / 32;        // k-steps of the score MFMA
  constexpr int DB = D / 16;        // 16-wide output blocks
  constexpr int EB = FP8 ? 1 : 2;   // bytes per cached element
  constexpr int RB = D * EB;        // bytes per cached row
  constexpr int CPR = RB / 16;      // 16-byte chunks per cached row
  constexpr int VL = kWaveKeys * CPR / 64;  // V loads per lane per step (half per 16 rows)
  constexpr int KL = FP8 ? D / 64 : KS;     // K loads per lane per 16 keys

  const int lane = threadIdx.x & 63;
  const int c16 = lane & 15;   // query column (S^T) / output row
  const int g = lane >> 4;     // 16-lane group
  const int H_kv = P.H_kv, N_q = P.N_q;
  const int G = P.H_q / H_kv;
  const int wbeg = split * chunk;
  const int wend = min(wbeg + chunk, len);
  const int nsteps = (wend - wbeg + kWaveKeys - 1) / kWaveKeys;
  const float scale_log2 = P.scale_log2;

  // ---- cache addressing. rows16(r0) is a buffer resource over rows r0 ..
  // r0 + 15 of this request and KV head (r0 a multiple of 16) bounded by the
  // request's length: rows past it read as zeros.
  const uint8_t* Kh = nullptr;
  const uint8_t* Vh = nullptr;
  int tb0 = -1, tb1 = -1, blk0 = 0;
  if constexpr (!PAGED) {
    Kh = P.kv.k + ((int64_t)b * H_kv + hk) * (int64_t)P.N_kv * RB;
    Vh = P.kv.v + ((int64_t)b * H_kv + hk) * (int64_t)P.N_kv * RB;
  } else {
    // this chunk's block-table entries, one per lane (a chunk spans at most
    // 128 blocks); entries of blocks past the request's length are not read
    const int bsl = P.kv.bs_log2;
    blk0 = wbeg >> bsl;
    const int nblk = (len + (1 << bsl) - 1) >> bsl;
    const int* trow = P.kv.table + (int64_t)b * P.kv.max_blocks;
    if (blk0 + lane < nblk) tb0 = trow[blk0 + lane];
    if (blk0 + 64 + lane < nblk) tb1 = trow[blk0 + 64 + lane];
  }
  auto rows16 = [&](const uint8_t* base, int r0) {
    if constexpr (!PAGED) {
      const int n = max(0, len - r0);
      return buffer_rsrc(base + (int64_t)min(r0, len) * RB, (uint32_t)n * RB);
    } else {
      const int bsl = P.kv.bs_log2;
      const int li = (r0 >> bsl) - blk0;   // wavefront-uniform
      const int pb = li < 64 ? __builtin_amdgcn_readlane(tb0, li) : __builtin_amdgcn_readlane(tb1, li - 64);
      const int off = r0 & ((1 << bsl) - 1);
      // a table entry outside the pool reads as zeros instead of faulting
      const bool ok = (unsigned)pb < (unsigned)P.kv.num_blocks && r0 < len;
      const int n = ok ? min((1 << bsl) - off, len - r0) : 0;
      const int64_t row = ok ? (((int64_t)pb * H_kv + hk) << bsl) + off : 0;
      return buffer_rsrc(base + row * RB, (uint32_t)n * RB);
    }
  };
  const uint8_t* kbase = PAGED ? P.kv.k : Kh;
  const uint8_t* vbase = PAGED ? P.kv.v : Vh;

  // The G query heads of KV head hk, N_q query rows each, are G*N_q contiguous
  // rows of Q; they are the MFMA's query columns, 16 per group.
  const int64_t qrow0 = ((int64_t)b * P.H_q + (int64_t)hk * G) * N_q;  // first row of the KV head's block
  int col0[NG], ncols[NG], lim[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    col0[j] = (qg * NG + j) * kQCols;   // first column of group j
    ncols[j] = max(0, min(kQCols, G * N_q - col0[j]));
    // keys below lim are visible to this lane's column (query row i = col % N_q,
    // aligned so that the last query row sees the last key)
    const int qi = (col0[j] + c16) % N_q;
    lim[j] = P.causal ? min(len, len - N_q + qi + 1) : len;
  }

  // Which head-dim slots lane group g feeds to k-step st. Any assignment works
  // if Q and K agree; 16-bit K uses d = 32*st + 8*g + 0..7, FP8 K gives each
  // lane group one contiguous run of D/4 codes (d = (D/4)*g + 8*st + 0..7) so
  // that its bytes come in whole 16-byte loads.
  auto dslot = [&](int st) { return FP8 ? (D / 4) * g + 8 * st : 32 * st + 8 * g; };

  // Q^T operands: column c16 of group j = row col0[j] + c16 of the block
  u32x4_t qreg[NG][KS];
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const auto rQ = buffer_rsrc(P.q + (qrow0 + min(col0[j], G * N_q)) * D, (uint32_t)ncols[j] * D * 2);
#pragma unroll
    for (int st = 0; st < KS; ++st)
      qreg[j][st] = buffer_load16(rQ, (uint32_t)(c16 * D + dslot(st)) * 2);
  }

  f32x4_t oacc[NG][DB];
#pragma unroll
  for (int j = 0; j < NG; ++j)
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[j][i] = f32x4_t{0, 0, 0, 0};
  float m[NG], l[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    m[j] = kNegInf;
    l[j] = 0.f;
  }

  // K rows feed the A operand directly: key = w0 + 16*kb + c16. V rows: lane
  // takes 16-byte chunk c = lane + 64*i of the step's rows (row c / CPR, chunk
  // c % CPR); the first VL/2 chunks are rows 0..15. The lane offsets are fixed;
  // each 16-row half has its own wavefront-uniform resource.
  const uint32_t koff = FP8 ? (uint32_t)(c16 * RB + (D / 4) * g) : (uint32_t)(c16 * D + 8 * g) * 2;
  const uint32_t voff = (uint32_t)lane * 16;
  u32x4_t ka[2][2][KL], va[2][VL];
  auto issue = [&](int w0, u32x4_t (&kk)[2][KL], u32x4_t (&vv)[VL]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const auto rK = rows16(kbase, w0 + 16 * h);
      const auto rV = rows16(vbase, w0 + 16 * h);
#pragma unroll
      for (int st = 0; st < KL; ++st) kk[h][st] = buffer_load16(rK, koff + (FP8 ? 16 : 64) * st);
#pragma unroll
      for (int i = 0; i < VL / 2; ++i) vv[h * (VL / 2) + i] = buffer_load16(rV, voff + 1024 * i);
    }
  };
  auto step = [&](int w0, const u32x4_t (&kraw)[2][KL], const u32x4_t (&vv)[VL]) {
    // V rows into LDS as 16-bit values
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int c = lane + 64 * i;
      if constexpr (FP8) {
        const u32x2_t a = fp8x4_to_bf16(vv[i][0]), b2 = fp8x4_to_bf16(vv[i][1]);
        const u32x2_t c2 = fp8x4_to_bf16(vv[i][2]), d2 = fp8x4_to_bf16(vv[i][3]);
        uint16_t* dst = sV + (c / CPR) * VST + (c % CPR) * 16;
        *(u32x4_t*)dst = u32x4_t{a[0], a[1], b2[0], b2[1]};
        *(u32x4_t*)(dst + 8) = u32x4_t{c2[0], c2[1], d2[0], d2[1]};
      } else {
        *(u32x4_t*)(sV + (c / CPR) * VST + (c % CPR) * 8) = vv[i];
      }
    }
    // K operands: 16-bit rows as loaded; FP8 codes widened (8 per k-step)
    u32x4_t kk[2][KS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (FP8) {
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          const u32x4_t& w = kraw[kb][st / 2];
          const u32x2_t x = fp8x4_to_bf16(w[(st & 1) * 2]);
          const u32x2_t y = fp8x4_to_bf16(w[(st & 1) * 2 + 1]);
          kk[kb][st] = u32x4_t{x[0], x[1], y[0], y[1]};
        }
      } else {
#pragma unroll
        for (int st = 0; st < KS; ++st) kk[kb][st] = kraw[kb][st];
      }
    }
    u32x4_t bop[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      f32x4_t s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x4_t{0, 0, 0, 0};
#pragma unroll
        for (int st = 0; st < KS; ++st) s[kb] = TT::mfma16(kk[kb][st], qreg[j][st], s[kb]);
      }
      // mask keys past the chunk or after the column's aligned diagonal; running
      // max over the step's 32 keys
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = w0 + kb * 16 + 4 * g + r;
          s[kb][r] = (key < wend && key < lim[j]) ? s[kb][r] : kNegInf;
          mx = fmaxf(mx, s[kb][r]);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = half_max(mx) * scale_log2;
      // lazy rescale: a column's reference maximum moves only when the step's
      // maximum exceeds it by more than kLazyRescale (probabilities stay below
      // 2^kLazyRescale; l and u keep a common reference, so u / l is unchanged)
      const bool need = mx > m[j] + kLazyRescale;
      if (wave_any(need)) {
        const float alpha = need ? ((m[j] == kNegInf) ? 0.f : fast_exp2(m[j] - mx)) : 1.f;
        m[j] = need ? mx : m[j];
        l[j] *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) oacc[j][i] *= alpha;
      }
      const float nm = (m[j] == kNegInf) ? 0.f : -m[j];
      float p[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], scale_log2, nm));
          l[j] += p[kb][r];
        }
      // K-slots of lane group g: keys 4g+0..3 (block 0) then 16+4g+0..3 (block 1)
      bop[j] = u32x4_t{TT::pack2(p[0][0], p[0][1]), TT::pack2(p[0][2], p[0][3]),
                       TT::pack2(p[1][0], p[1][1]), TT::pack2(p[1][2], p[1][3])};
    }
    wave_lds_sync();  // V rows of this step are in LDS
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int dcol = 16 * db + 4 * (c16 & 3);
      const u32x2_t lo = lds_read_tr16(sV + (4 * g + (c16 >> 2)) * VST + dcol);
      const u32x2_t hi = lds_read_tr16(sV + (16 + 4 * g + (c16 >> 2)) * VST + dcol);
      const u32x4_t aop = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int j = 0; j < NG; ++j) oacc[j][db] = TT::mfma16(aop, bop[j], oacc[j][db]);
    }
    wave_lds_sync();  // reads done before the next step overwrites the rows
  };

  issue(wbeg, ka[0], va[0]);
  for (int i = 0; i < nsteps; i += 2) {
    const int w0 = wbeg + i * kWaveKeys;
    if (i + 1 < nsteps) issue(w0 + kWaveKeys, ka[1], va[1]);
    step(w0, ka[0], va[0]);
    if (i + 1 < nsteps) {
      if (i + 2 < nsteps) issue(w0 + 2 * kWaveKeys, ka[0], va[0]);
      step(w0 + kWaveKeys, ka[1], va[1]);
    }
  }

  // ---- this chunk's partials: column c16 of group j (query row col0[j] + c16)
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    float lj = l[j] + __shfl_xor(l[j], 16);
    lj = half_sum(lj);
    if (c16 < ncols[j]) {
      const int64_t row = (qrow0 + col0[j] + c16) * nsplit + split;
      float* pu = P.part_u + row * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *(f32x4_t*)(pu + 16 * db + 4 * g) = oacc[j][db];
      if (g == 0) {
        P.part_ml[row * 2 + 0] = m[j];
        P.part_ml[row * 2 + 1] = lj;
      }
    }
  }
}

// Persistent split kernel with a static, balanced schedule. Work units are
// (request b, KV-head group hg, chunk c of request b), numbered chunk-major over
// the concatenated requests: unit u covers global chunk u / HG and head group
// u % HG. Every unit holds `chunk` keys except the last chunk of a request, so
// handing units out round-robin to the wavefronts of the grid balances ragged
// lengths without atomics or barriers. Each wavefront walks the requests
// forward as its unit index grows, reading kv_lens as it goes.
template <class TT, int D, int NG, int OCC, bool PAGED, bool FP8>
__global__ __launch_bounds__(kThreads, OCC) void decode_split_kernel(const SplitParams P) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[DecLds<D>::kV];
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  uint16_t* sV = smem + wave * kWaveKeys * DecLds<D>::VST;
  const int G = P.H_q / P.H_kv;
  const int ngroups = (G * P.N_q + NG * kQCols - 1) / (NG * kQCols);  // units of NG column groups
  const int HG = P.H_kv * ngroups;
  const int nw = (int)gridDim.x * 4;
  const int B = P.B;
  const int chunk = unit_chunk(P.kv_lens, B, P.N_kv, P.chunk, P.chunk_cap, HG, nw);
  // partials of a query row sit in consecutive slots, one per split of the
  // chosen chunk (never more than the plan's splits: the chunk only grows)
  const int nsplit = (P.N_kv + chunk - 1) / chunk;
  auto len_of = [&](int b) {
    const int n = P.kv_lens ? P.kv_lens[b] : P.N_kv;
    return min(max(n, 0), P.N_kv);
  };
  int cb = 0;                 // request holding the current global chunk
  int cstart = 0;             // its first global chunk index
  int lb = B > 0 ? len_of(0) : 0;
  int cnt = (lb + chunk - 1) / chunk;
  for (int u = (int)blockIdx.x * 4 + wave;; u += nw) {
    const int c = u / HG, hg = u - (u / HG) * HG;
    while (cb < B && c >= cstart + cnt) {
      cstart += cnt;
      ++cb;
      if (cb < B) {
        lb = len_of(cb);
        cnt = (lb + chunk - 1) / chunk;
      }
    }
    if (cb >= B) break;
    wave_unit<TT, D, NG, PAGED, FP8>(P, chunk, nsplit, cb, hg / ngroups, hg - (hg / ngroups) * ngroups,
                                     c - cstart, lb, sV);
  }
}

// Merge of the split partials: out = sum_s w_s u_s / sum_s w_s l_s with
// w_s = exp2(m_s - max_s m_s), times out_scale (the V dequantisation scale
// of an FP8 cache, else 1). One 64-lane wavefront per query row (request,
// query head, query index); lane i owns output column i (d = 64) or columns
// 2i, 2i+1 (d = 128).
template <class TT, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float* __restrict__ part_u, const float* __restrict__ part_ml,
    const int* __restrict__ kv_lens, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int rows_per_b, int N_kv, int chunk, int chunk_cap, int HG, int nwaves, int BH,
    float out_scale) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int PER = D / 64;  // columns per lane
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);  // ((b * H_q + h) * N_q + i)
  if (bh >= BH) return;
  const int b = bh / rows_per_b;
  int len = kv_lens ? kv_lens[b] : N_kv;
  len = min(max(len, 0), N_kv);
  // the split kernel's units: the same function of the same inputs
  const int ce = unit_chunk(kv_lens, BH / rows_per_b, N_kv, chunk, chunk_cap, HG, nwaves);
  const int ns = (len + ce - 1) / ce;
  const int64_t row0 = (int64_t)bh * ((N_kv + ce - 1) / ce);
  float M = kNegInf;
  for (int s = lane; s < ns; s += 64) M = fmaxf(M, part_ml[(row0 + s) * 2]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  const float Mref = (M == kNegInf) ? 0.f : M;
  float L = 0.f, U0 = 0.f, U1 = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const int s = s0 + lane;
    const float w = (s < ns) ? fast_exp2(part_ml[(row0 + s) * 2] - Mref) : 0.f;
    L += (s < ns) ? w * part_ml[(row0 + s) * 2 + 1] : 0.f;
    const int cnt = min(64, ns - s0);
    const float* ub = part_u + (row0 + s0) * D + PER * lane;
    // eight splits per batch: all loads issued before the accumulation
    for (int j0 = 0; j0 < cnt; j0 += 8) {
      float a0[8], a1[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int jj = min(j0 + j, cnt - 1);
        if constexpr (PER == 2) {
          const float2 v = *(const float2*)(ub + (int64_t)jj * D);
          a0[j] = v.x;
          a1[j] = v.y;
        } else {
          a0[j] = ub[(int64_t)jj * D];
          a1[j] = 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float wj = (j0 + j < cnt) ? __shfl(w, j0 + j) : 0.f;
        U0 += wj * a0[j];
        U1 += wj * a1[j];
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
  const float inv = (L > 0.f) ? out_scale / L : 0.f;
  uint16_t* out = O + (int64_t)bh * D + PER * lane;
  if constexpr (PER == 2) {
    *(uint32_t*)out = TT::pack2(U0 * inv, U1 * inv);
  } else {
    *out = (uint16_t)(TT::pack2(U0 * inv, 0.f) & 0xffffu);
  }
  if (LSE != nullptr && lane == 0) LSE[bh] = (L > 0.f) ? (M + log2f(L)) * kLn2 : kNegInf;
}

template <class TT, int D, int NG, int OCC, bool FP8>
hipError_t launch_t(const DecodeArgs& a, hipStream_t st) {
  const int G = a.H_q / a.H_kv;
  const int ngroups = (G * a.N_q + NG * kQCols - 1) / (NG * kQCols);
  // OCC resident workgroups per compute unit (one for FP8 caches, whose units
  // carry half the bytes: measured faster with half the wavefronts and twice
  // the keys per unit); never more than the units there can be
  const int64_t units = (int64_t)a.B * a.H_kv * ngroups * a.splits;
  const int64_t slots = (int64_t)(FP8 ? 1 : OCC) * (a.num_cus > 0 ? a.num_cus : 256);
  const int64_t wgs = (units + 3) / 4;
  dim3 grid((unsigned)(wgs < slots ? wgs : slots));
  SplitParams P;
  P.q = (const uint16_t*)a.q;
  P.kv = KvSrc{(const uint8_t*)a.k, (const uint8_t*)a.v, a.block_table, a.max_blocks,
               a.block_size_log2, a.num_blocks};
  P.kv_lens = a.kv_lens;
  P.part_u = a.part_u;
  P.part_ml = a.part_ml;
  P.B = a.B;
  P.H_q = a.H_q;
  P.H_kv = a.H_kv;
  P.N_q = a.N_q;
  P.N_kv = a.N_kv;
  P.causal = a.causal;
  P.chunk = a.chunk;
  P.chunk_cap = a.chunk_cap;
  P.scale_log2 = a.scale * (FP8 ? a.k_scale : 1.f) * kLog2e;
  const hipError_t e =
      a.block_table != nullptr
          ? launch_kernel(decode_split_kernel<TT, D, NG, OCC, true, FP8>, grid, dim3(kThreads), st, P)
          : launch_kernel(decode_split_kernel<TT, D, NG, OCC, false, FP8>, grid, dim3(kThreads), st, P);
  if (e != hipSuccess) return e;
  const int BH = a.B * a.H_q * a.N_q;
  return launch_kernel(decode_merge_kernel<TT, D>, dim3((BH + 3) / 4), dim3(256), st, a.part_u,
                       a.part_ml, a.kv_lens, (uint16_t*)a.o, a.lse, a.H_q * a.N_q, a.N_kv, a.chunk,
                       a.chunk_cap, a.H_kv * ngroups, (int)grid.x * 4, BH, FP8 ? a.v_scale : 1.f);
}

template <class TT, bool FP8>
hipError_t launch_dtype(const DecodeArgs& a, hipStream_t st) {
  // more than 16 query rows per KV head: each wavefront serves two or four
  // column groups, so K and V are read once per 32 or 64 rows
  // (the decode_groups knob forces 1, 2 or 4)
  const int cols = (a.H_q / a.H_kv) * a.N_q;
  int ng = cols <= kQCols ? 1 : (cols <= 2 * kQCols ? 2 : 4);
  if (const int f = tuning(kTuneDecodeGroups)) ng = f;
  if (a.d == 64) {
    if (ng == 1) return launch_t<TT, 64, 1, 2, FP8>(a, st);
    return ng == 2 ? launch_t<TT, 64, 2, 2, FP8>(a, st) : launch_t<TT, 64, 4, 2, FP8>(a, st);
  }
  if (ng == 1) return launch_t<TT, 128, 1, 2, FP8>(a, st);
  return ng == 2 ? launch_t<TT, 128, 2, 1, FP8>(a, st) : launch_t<TT, 128, 4, 1, FP8>(a, st);
}

}  // namespace

DecodePlan decode_plan(int B, int H_q, int H_kv, int N_q, int N_kv, int d, bool paged,
                       size_t max_workspace) {
  // The persistent kernel hands chunks out round-robin to wavefronts. The
  // plan's chunk is the finest split the kernels may use (they raise it from
  // the actual lengths, unit_chunk): about N_kv / 64 keys for one new token
  // per request, so that short requests in a long cache still spread over the
  // grid, and N_kv / 16 for more tokens, whose partials are N_q times larger;
  // at least 128 keys and at most 2048 (1 MB of K and V at d = 128).
  const int64_t target = N_q <= 1 ? 64 : 16;
  int64_t chunk = ((int64_t)N_kv + target - 1) / target;
  chunk = ((chunk + kWaveKeys * 4 - 1) / (kWaveKeys * 4)) * (kWaveKeys * 4);
  if (chunk < 128) chunk = 128;
  if (chunk > 2048) chunk = 2048;
  // The kernels may raise the split on the device, from the actual lengths
  // (unit_chunk), up to one chunk per request for contiguous caches; paged
  // caches keep at most 2048 keys per chunk, whose block-table entries sit in
  // one register pair per lane.
  int64_t cap = paged ? 2048 : ((int64_t)N_kv + kStepKeys - 1) / kStepKeys * kStepKeys;
  // tuning override (the decode_chunk knob: keys per split, rounded up to a
  // multiple of 128, used as given: no raise on the device)
  if (const int v = tuning(kTuneDecodeChunk)) {
    chunk = ((v + kStepKeys - 1) / kStepKeys) * kStepKeys;
    if (paged && chunk > 2048) chunk = 2048;
    cap = chunk;
  }
  if (cap < chunk) cap = chunk;
  DecodePlan p;
  p.chunk = (int)chunk;
  p.chunk_cap = (int)cap;
  p.splits = N_kv > 0 ? (int)((N_kv + chunk - 1) / chunk) : 1;
  const size_t per_split = (size_t)B * H_q * N_q * (size_t)(d + 2) * sizeof(float);
  p.workspace_bytes = per_split * p.splits;
  if (max_workspace > 0 && p.workspace_bytes > max_workspace && !paged && per_split > 0 &&
      per_split <= max_workspace && N_kv > 0) {
    // fewer, longer splits: the most that fit, each a multiple of the step
    const int64_t smax = (int64_t)(max_workspace / per_split);
    int64_t c = ((int64_t)N_kv + smax - 1) / smax;
    c = (c + kStepKeys - 1) / kStepKeys * kStepKeys;
    p.chunk = (int)c;
    if (p.chunk_cap < p.chunk) p.chunk_cap = p.chunk;
    p.splits = (int)(((int64_t)N_kv + c - 1) / c);
    p.workspace_bytes = per_split * p.splits;
  }
  return p;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  // FP8 caches are widened to bf16, so they pair with bf16 queries only
  if (a.kv_fp8) return launch_dtype<BF16, true>(a, st);
  if (a.dtype == kDtypeBF16) return launch_dtype<BF16, false>(a, st);
  return launch_dtype<F16, false>(a, st);
}

}  // namespace attn
