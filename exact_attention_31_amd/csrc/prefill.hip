// Prefill attention forward on gfx950: O = softmax(scale * Q K^T) V, block by
// block, without writing the score matrix to HBM.
//
// The method (marketmaker.cc "Flash Attention und die Frage nach der
// Sequenzlaenge", sections on the algorithm, the online-softmax recurrence and
// FA2; auturnal.com transformer-attention guide, section 8): each query block
// keeps, per row, a running maximum m, a denominator l and an un-normalised
// output u; a new key block raises the maximum to m', rescales l and u by
// exp(m - m'), adds its own exponentials, and the row's output is u / l, divided
// once at the end (FA2's first change). Query blocks are spread over the grid
// (FA2's second change) and each wavefront owns whole query rows, so row
// statistics never cross wavefronts (FA2's third change). Key blocks that lie
// entirely after a causal query block are never loaded (causal skipping).
//
// gfx950 mapping (one workgroup = 4 wavefronts = 128 query rows):
//   * Q rows stay in VGPRs for the whole loop, laid out as the B operand of
//     S^T = K Q^T (v_mfma_f32_32x32x16): each lane owns one query row, and the
//     accumulator layout then gives each lane 16 of the 32 scores of its row,
//     so the row max/sum needs one exchange with the opposite half-wave only.
//   * K and V tiles (64 keys) are staged through LDS with 16-byte coalesced
//     loads; all four wavefronts read them.
//   * The probabilities, rounded to the input type, are reused in registers as
//     the B operand of O^T = V^T P^T; V^T comes from LDS through the gfx950
//     transposing read, so each lane's output accumulators belong to its own
//     query row and the rescale by exp2(m - m') is lane-local.
//   * exp is evaluated as exp2 with scale*log2(e) folded into one multiply.
// fp32 inputs use v_mfma_f32_32x32x2_f32 in the same arrangement (no LDS
// transpose is needed there because each lane feeds one K-slot).
#include <stdlib.h>

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr int kBM = 128;  // query rows per workgroup (4 wavefronts x 32)
constexpr int kBN = 64;   // keys per tile
constexpr int kThreads = 256;

// Row stride (elements) of the K and V tiles in LDS. The padding keeps the
// 16-byte row reads of K and the 4-row transposing reads of V spread over banks.
template <int D> struct Lds16 {
  static constexpr int kK = D + 8;
  static constexpr int kV = D + 16;
};

// Rescale threshold (log2 units): a row's reference maximum is only raised when
// a block's maximum exceeds it by more than this, so most blocks skip the
// rescale of l and u. Probabilities then stay below 2^8, and l and u keep one
// common reference point, so u / l is unchanged.
constexpr float kLazyRescale = 8.f;

// QB query blocks of 32 rows per wavefront (QB = 1: 128 rows per workgroup,
// QB = 2: 256). Each K or V operand read from LDS feeds QB MFMAs, so QB = 2
// halves the LDS bytes per FLOP at the price of twice the registers.
// Workgroup -> (batch, head, query block). Workgroups are handed to the 8
// XCDs (each with its own L2) round-robin by linear id, so XCD x runs ids
// x, x+8, x+16, ... Work items (head-major, longest query block first within a
// head) are cut into 8 contiguous ranges and XCD x takes range x in order: the
// query blocks of a head, and heads sharing a KV head, then run on one XCD and
// reuse its L2, while every XCD gets the same number of items.
struct WorkItem {
  int b, h, qblk;
  bool valid;
};
__device__ __forceinline__ WorkItem map_work(int nqb, int H_q, int B, bool longest_first) {
  const int id = blockIdx.x;
  const int per_xcd = (int)gridDim.x >> 3;
  const int item = (id & 7) * per_xcd + (id >> 3);
  WorkItem w;
  const int total = nqb * H_q * B;
  w.valid = item < total;
  const int unit = item / nqb;
  const int qi = item - unit * nqb;
  w.qblk = longest_first ? (nqb - 1 - qi) : qi;
  w.b = unit / H_q;
  w.h = unit - w.b * H_q;
  return w;
}

template <int QB, int D> struct Occ {
  static constexpr int kWaves = (QB == 2 && D == 128) ? 1 : 2;  // wavefronts per SIMD
};

template <class TT, int D, bool CAUSAL, int QB>
__global__ __launch_bounds__(kThreads, (Occ<QB, D>::kWaves)) void prefill16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int H_q, int H_kv, int N_q, int N_kv,
    float scale_log2, int nqb, int nbatch) {
  constexpr int KST = Lds16<D>::kK;
  constexpr int VST = Lds16<D>::kV;
  constexpr int KS = D / 16;   // k-steps of the score MFMA
  constexpr int DB = D / 32;   // 32-wide blocks of the output
  constexpr int CPR = D / 8;   // 16-byte chunks per K/V row
  constexpr int LPT = kBN * CPR / kThreads;  // 16-byte loads per thread per tile, per tensor
  constexpr int BM = 4 * 32 * QB;            // query rows per workgroup
  static_assert(LPT * kThreads == kBN * CPR, "tile load must split evenly");
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kBN * KST];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][kBN * VST];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // scalar, so that every per-wavefront decision below is a uniform branch
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31;
  const int lh = lane >> 5;
  // causal: longest query blocks first
  const WorkItem wi = map_work(nqb, H_q, nbatch, CAUSAL);
  if (!wi.valid) return;
  const int qblk = wi.qblk, h = wi.h, b = wi.b;
  const int hk = h / (H_q / H_kv);

  const uint32_t head_q_bytes = (uint32_t)N_q * D * 2;
  const uint32_t head_kv_bytes = (uint32_t)N_kv * D * 2;
  const auto rQ = buffer_rsrc(Q + ((int64_t)b * H_q + h) * (int64_t)N_q * D, head_q_bytes);
  const auto rK = buffer_rsrc(K + ((int64_t)b * H_kv + hk) * (int64_t)N_kv * D, head_kv_bytes);
  const auto rV = buffer_rsrc(V + ((int64_t)b * H_kv + hk) * (int64_t)N_kv * D, head_kv_bytes);

  const int q0 = qblk * BM + wave * 32 * QB;  // first row of this wavefront
  const int off = N_kv - N_q;                 // bottom-right causal alignment
  int qrow[QB], lim[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    qrow[j] = q0 + 32 * j + lr;  // this lane's row in query block j
    // keys below lim[j] are visible to that row
    lim[j] = CAUSAL ? min(N_kv, max(qrow[j] + off + 1, 0)) : N_kv;
  }

  // Q^T operand: lane holds row qrow[j], d = 16*s + 8*lh + 0..7 (rows past N_q read as 0)
  u32x4_t qreg[QB][KS];
#pragma unroll
  for (int j = 0; j < QB; ++j)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qreg[j][s] = buffer_load16(rQ, (uint32_t)(qrow[j] * D + 16 * s + 8 * lh) * 2);

  int kv_end = N_kv;
  if (CAUSAL) {
    const int qlast = min(qblk * BM + BM - 1, N_q - 1);
    kv_end = min(N_kv, qlast + off + 1);
  }
  const int ntiles = kv_end > 0 ? (kv_end + kBN - 1) / kBN : 0;

  // this thread's share of each tile: chunk c = tid + kThreads*i -> row c / CPR, column c % CPR
  uint32_t ld_off[LPT];
  int st_k[LPT], st_v[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int c = tid + kThreads * i;
    const int r = c / CPR, cc = c % CPR;
    ld_off[i] = (uint32_t)(r * D + cc * 8) * 2;
    st_k[i] = r * KST + cc * 8;
    st_v[i] = r * VST + cc * 8;
  }
  // per-lane LDS offsets of the MFMA operands (elements):
  //   K: row lr (+32 for the second key block), columns 16*st + 8*lh
  //   V (transposing read): lane i of 16-lane group g reads row 4*(g/2) + i/4,
  //   columns 16*(g%2) + 4*(i%4)
  const int k_lane = lr * KST + 8 * lh;
  const int v_lane = (4 * ((lane >> 4) >> 1) + ((lane & 15) >> 2)) * VST + 16 * ((lane >> 4) & 1) +
                     4 * (lane & 3);
  u32x4_t kbuf[LPT], vbuf[LPT];
  auto load_tile = [&](int t) {
    const uint32_t base = (uint32_t)(t * kBN) * D * 2;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      kbuf[i] = buffer_load16(rK, base + ld_off[i]);
      vbuf[i] = buffer_load16(rV, base + ld_off[i]);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      *(u32x4_t*)(&sK[buf][st_k[i]]) = kbuf[i];
      *(u32x4_t*)(&sV[buf][st_v[i]]) = vbuf[i];
    }
  };

  f32x16_t oacc[QB][DB];
  float m[QB], l[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[j][i] = f32x16_t{0};
    m[j] = kNegInf;  // reference maximum, in units of log2 (scores * scale * log2 e)
    l[j] = 0.f;      // this half-wave's part of the denominator
  }

  // Tile 0 is staged unconditionally (loads past the end read zeros): with no
  // branch here every load issued so far has completed when the loop starts,
  // so the loop only ever waits for its own prefetch, at the LDS store.
  load_tile(0);
  store_tile(0);
  vmem_wait_all();
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);  // in flight during this tile's math
    const int kv0 = t * kBN;
    // wavefront-uniform: does this tile hold any key visible to this wavefront?
    const bool live = !CAUSAL || kv0 <= q0 + 32 * QB - 1 + off;
    if (live) {
      const uint16_t* tK = &sK[0][0] + buf * (kBN * KST) + k_lane;
      const uint16_t* tV = &sV[0][0] + buf * (kBN * VST) + v_lane;
      // ---- S^T = K Q^T: two 32-key blocks x QB query blocks; each K read feeds QB MFMAs
      f32x16_t s[QB][2];
#pragma unroll
      for (int j = 0; j < QB; ++j) s[j][0] = s[j][1] = f32x16_t{0};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const u32x4_t a0 = *(const u32x4_t*)(tK + 16 * st);
        const u32x4_t a1 = *(const u32x4_t*)(tK + 32 * KST + 16 * st);
#pragma unroll
        for (int j = 0; j < QB; ++j) {
          s[j][0] = TT::mfma32(a0, qreg[j][st], s[j][0]);
          s[j][1] = TT::mfma32(a1, qreg[j][st], s[j][1]);
        }
      }
      // ---- mask (tail and causal diagonal tiles only), branch-free per element
      const bool need_mask = (kv0 + kBN > N_kv) || (CAUSAL && kv0 + kBN - 1 > q0 + off);
      if (need_mask) {
        const int kvb = kv0 + 4 * lh;
#pragma unroll
        for (int j = 0; j < QB; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kv = kvb + 8 * (r >> 2) + (r & 3);
            s[j][0][r] = (kv < lim[j]) ? s[j][0][r] : kNegInf;
            s[j][1][r] = (kv + 32 < lim[j]) ? s[j][1][r] : kNegInf;
          }
      }
      uint32_t pk[QB][16];
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        // ---- row max of the raw scores (scale > 0 commutes with max)
        float mx = max3(s[j][0][0], s[j][0][1], s[j][1][0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = max3(mx, s[j][0][r], s[j][1][r]);
        mx = fmaxf(mx, s[j][1][0]);
        const float mxs = half_max(mx) * scale_log2;
        // The branch is wavefront-uniform, but each lane moves only its own
        // reference (alpha = 1 is an exact multiply), so a row's arithmetic never
        // depends on the other rows of the wavefront.
        const bool need = mxs > m[j] + kLazyRescale;
        if (wave_any(need)) {
          const float alpha = need ? ((m[j] == kNegInf) ? 0.f : fast_exp2(m[j] - mxs)) : 1.f;
          m[j] = need ? mxs : m[j];
          l[j] *= alpha;
#pragma unroll
          for (int i = 0; i < DB; ++i) oacc[j][i] *= alpha;
        }
        const float nm = (m[j] == kNegInf) ? 0.f : -m[j];
        // ---- P = exp2(S * scale*log2e - m), packed to 16-bit as the B operand
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(__builtin_fmaf(s[j][0][r], scale_log2, nm));
          const float p1 = fast_exp2(__builtin_fmaf(s[j][0][r + 1], scale_log2, nm));
          const float p2 = fast_exp2(__builtin_fmaf(s[j][1][r], scale_log2, nm));
          const float p3 = fast_exp2(__builtin_fmaf(s[j][1][r + 1], scale_log2, nm));
          l[j] += (p0 + p1) + (p2 + p3);
          pk[j][r >> 1] = TT::pack2(p0, p1);
          pk[j][8 + (r >> 1)] = TT::pack2(p2, p3);
        }
      }
      // ---- O^T += V^T P^T, four 16-key steps; V^T through the transposing LDS read,
      // each V operand feeding QB MFMAs
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          // key rows 16*t4 + 4*lh + {0..3} (then + 8), columns db*32 + this lane's 16-group
          const u32x2_t lo = lds_read_tr16(tV + 16 * t4 * VST + db * 32);
          const u32x2_t hi = lds_read_tr16(tV + (16 * t4 + 8) * VST + db * 32);
          const u32x4_t aop = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
          for (int j = 0; j < QB; ++j) {
            const u32x4_t bop = {pk[j][4 * t4 + 0], pk[j][4 * t4 + 1], pk[j][4 * t4 + 2],
                                 pk[j][4 * t4 + 3]};
            oacc[j][db] = TT::mfma32(aop, bop, oacc[j][db]);
          }
        }
      }
    }
    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: combine half-wave denominators, normalise, store (rows past N_q dropped)
  const auto rO = buffer_rsrc(O + ((int64_t)b * H_q + h) * (int64_t)N_q * D, head_q_bytes);
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const float lt = half_sum(l[j]);
    const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d = db * 32 + 8 * rg + 4 * lh;
        const u32x2_t w = {TT::pack2(oacc[j][db][4 * rg + 0] * inv, oacc[j][db][4 * rg + 1] * inv),
                           TT::pack2(oacc[j][db][4 * rg + 2] * inv, oacc[j][db][4 * rg + 3] * inv)};
        buffer_store8(rO, (uint32_t)(qrow[j] * D + d) * 2, w);
      }
    }
    if (LSE != nullptr && lh == 0 && qrow[j] < N_q) {
      LSE[((int64_t)b * H_q + h) * N_q + qrow[j]] = (lt > 0.f) ? (m[j] + log2f(lt)) * kLn2 : kNegInf;
    }
  }
}

// Software-pipelined form (32 rows per wavefront). While the matrix cores
// compute the scores of key tile t+1, the vector ALUs turn the scores of tile t
// into probabilities; the products with V follow. K is staged in LDS one tile
// ahead of V, so the same two buffers per tensor suffice:
//   iteration t reads K(t+1) from K buffer (t+1)%2 and V(t) from V buffer t%2,
//   and at its end stores K(t+2) into K buffer t%2 and V(t+1) into V buffer
//   (t+1)%2, both loaded from HBM while the tile's math runs.
template <class TT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void prefill16_pipe_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int H_q, int H_kv, int N_q, int N_kv,
    float scale_log2, int nqb, int nbatch) {
  constexpr int KST = Lds16<D>::kK;
  constexpr int VST = Lds16<D>::kV;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int CPR = D / 8;
  constexpr int LPT = kBN * CPR / kThreads;
  static_assert(LPT * kThreads == kBN * CPR, "tile load must split evenly");
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kBN * KST];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][kBN * VST];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const WorkItem wi = map_work(nqb, H_q, nbatch, CAUSAL);
  if (!wi.valid) return;
  const int qblk = wi.qblk, h = wi.h, b = wi.b;
  const int hk = h / (H_q / H_kv);

  const uint32_t head_q_bytes = (uint32_t)N_q * D * 2;
  const uint32_t head_kv_bytes = (uint32_t)N_kv * D * 2;
  const auto rQ = buffer_rsrc(Q + ((int64_t)b * H_q + h) * (int64_t)N_q * D, head_q_bytes);
  const auto rK = buffer_rsrc(K + ((int64_t)b * H_kv + hk) * (int64_t)N_kv * D, head_kv_bytes);
  const auto rV = buffer_rsrc(V + ((int64_t)b * H_kv + hk) * (int64_t)N_kv * D, head_kv_bytes);

  const int q0 = qblk * kBM + wave * 32;
  const int qrow = q0 + lr;
  const int off = N_kv - N_q;
  const int lim = CAUSAL ? min(N_kv, max(qrow + off + 1, 0)) : N_kv;

  u32x4_t qreg[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) qreg[st] = buffer_load16(rQ, (uint32_t)(qrow * D + 16 * st + 8 * lh) * 2);

  int kv_end = N_kv;
  if (CAUSAL) kv_end = min(N_kv, min(qblk * kBM + kBM - 1, N_q - 1) + off + 1);
  const int ntiles = kv_end > 0 ? (kv_end + kBN - 1) / kBN : 0;
  // tiles holding a key visible to some row of this wavefront (a prefix of the tiles)
  int wtiles = ntiles;
  if (CAUSAL) wtiles = min(ntiles, max(0, (q0 + 31 + off + kBN) / kBN));

  uint32_t ld_off[LPT];
  int st_k[LPT], st_v[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int c = tid + kThreads * i;
    const int r = c / CPR, cc = c % CPR;
    ld_off[i] = (uint32_t)(r * D + cc * 8) * 2;
    st_k[i] = r * KST + cc * 8;
    st_v[i] = r * VST + cc * 8;
  }
  const int k_lane = lr * KST + 8 * lh;
  const int v_lane = (4 * ((lane >> 4) >> 1) + ((lane & 15) >> 2)) * VST + 16 * ((lane >> 4) & 1) +
                     4 * (lane & 3);
  u32x4_t kbuf[LPT], vbuf[LPT];
  auto load_k = [&](int t) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) kbuf[i] = buffer_load16(rK, (uint32_t)(t * kBN) * D * 2 + ld_off[i]);
  };
  auto load_v = [&](int t) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) vbuf[i] = buffer_load16(rV, (uint32_t)(t * kBN) * D * 2 + ld_off[i]);
  };
  auto store_k = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) *(u32x4_t*)(&sK[buf][st_k[i]]) = kbuf[i];
  };
  auto store_v = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) *(u32x4_t*)(&sV[buf][st_v[i]]) = vbuf[i];
  };
  auto gemm_s = [&](int buf, f32x16_t& s0, f32x16_t& s1) {
    const uint16_t* tK = &sK[0][0] + buf * (kBN * KST) + k_lane;
    s0 = f32x16_t{0};
    s1 = f32x16_t{0};
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const u32x4_t a0 = *(const u32x4_t*)(tK + 16 * st);
      const u32x4_t a1 = *(const u32x4_t*)(tK + 32 * KST + 16 * st);
      s0 = TT::mfma32(a0, qreg[st], s0);
      s1 = TT::mfma32(a1, qreg[st], s1);
    }
  };

  // prologue: K(0), V(0) into buffers 0 and K(1) into K buffer 1 (past-the-end
  // loads read zeros, so this needs no branch)
  load_k(0);
  load_v(0);
  store_k(0);
  store_v(0);
  load_k(1);
  store_k(1);
  vmem_wait_all();
  __syncthreads();

  f32x16_t oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16_t{0};
  float m = kNegInf, l = 0.f;
  f32x16_t sa0, sa1, sb0, sb1;
  gemm_s(0, sa0, sa1);

  auto step = [&](int t, f32x16_t& c0, f32x16_t& c1, f32x16_t& n0, f32x16_t& n1) {
    const bool pre_k = t + 2 < ntiles;
    const bool pre_v = t + 1 < ntiles;
    if (pre_k) load_k(t + 2);
    if (pre_v) load_v(t + 1);
    if (t < wtiles) {
      const int kv0 = t * kBN;
      // ---- mask, row max and rescale decision for S(t)
      const bool need_mask = (kv0 + kBN > N_kv) || (CAUSAL && kv0 + kBN - 1 > q0 + off);
      if (need_mask) {
        const int kvb = kv0 + 4 * lh;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kv = kvb + 8 * (r >> 2) + (r & 3);
          c0[r] = (kv < lim) ? c0[r] : kNegInf;
          c1[r] = (kv + 32 < lim) ? c1[r] : kNegInf;
        }
      }
      float mx = max3(c0[0], c0[1], c1[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = max3(mx, c0[r], c1[r]);
      const float mxs = half_max(mx) * scale_log2;
      const bool need = mxs > m + kLazyRescale;
      if (wave_any(need)) {
        const float alpha = need ? ((m == kNegInf) ? 0.f : fast_exp2(m - mxs)) : 1.f;
        m = need ? mxs : m;
        l *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
      }
      const float nm = (m == kNegInf) ? 0.f : -m;
      // ---- S(t+1) on the matrix cores while S(t) becomes P(t)
      gemm_s((t + 1) & 1, n0, n1);
      uint32_t pk[16];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(c0[r], scale_log2, nm));
        const float p1 = fast_exp2(__builtin_fmaf(c0[r + 1], scale_log2, nm));
        const float p2 = fast_exp2(__builtin_fmaf(c1[r], scale_log2, nm));
        const float p3 = fast_exp2(__builtin_fmaf(c1[r + 1], scale_log2, nm));
        l += (p0 + p1) + (p2 + p3);
        pk[r >> 1] = TT::pack2(p0, p1);
        pk[8 + (r >> 1)] = TT::pack2(p2, p3);
      }
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads of K
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two score MFMAs
        __builtin_amdgcn_sched_group_barrier(0x002, 56 / KS * 2, 0);  // exp / convert / sum
      }
      // ---- O^T += V^T P^T
      const uint16_t* tV = &sV[0][0] + (t & 1) * (kBN * VST) + v_lane;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const u32x4_t bop = {pk[4 * t4 + 0], pk[4 * t4 + 1], pk[4 * t4 + 2], pk[4 * t4 + 3]};
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x2_t lo = lds_read_tr16(tV + 16 * t4 * VST + db * 32);
          const u32x2_t hi = lds_read_tr16(tV + (16 * t4 + 8) * VST + db * 32);
          const u32x4_t aop = {lo[0], lo[1], hi[0], hi[1]};
          oacc[db] = TT::mfma32(aop, bop, oacc[db]);
        }
      }
    }
    if (pre_k) store_k(t & 1);
    if (pre_v) store_v((t + 1) & 1);
    __syncthreads();
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, sa0, sa1, sb0, sb1);
    if (t + 1 < ntiles) step(t + 1, sb0, sb1, sa0, sa1);
  }

  l = half_sum(l);
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  const auto rO = buffer_rsrc(O + ((int64_t)b * H_q + h) * (int64_t)N_q * D, head_q_bytes);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d = db * 32 + 8 * rg + 4 * lh;
      const u32x2_t w = {TT::pack2(oacc[db][4 * rg + 0] * inv, oacc[db][4 * rg + 1] * inv),
                         TT::pack2(oacc[db][4 * rg + 2] * inv, oacc[db][4 * rg + 3] * inv)};
      buffer_store8(rO, (uint32_t)(qrow * D + d) * 2, w);
    }
  }
  if (LSE != nullptr && lh == 0 && qrow < N_q) {
    LSE[((int64_t)b * H_q + h) * N_q + qrow] = (l > 0.f) ? (m + log2f(l)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------- fp32 inputs
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void prefill32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int H_q, int H_kv, int N_q, int N_kv,
    float scale_log2, int nqb) {
  constexpr int BN = 32;
  constexpr int ST = D + 4;  // LDS row stride (floats)
  constexpr int KH = D / 2;  // K-slots per lane half
  constexpr int DB = D / 32;
  __shared__ __attribute__((aligned(16))) float sK[BN * ST];
  __shared__ __attribute__((aligned(16))) float sV[BN * ST];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int qb = CAUSAL ? (nqb - 1 - (int)blockIdx.x) : (int)blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int hk = h / (H_q / H_kv);
  const float* Qh = Q + ((int64_t)b * H_q + h) * (int64_t)N_q * D;
  const float* Kh = K + ((int64_t)b * H_kv + hk) * (int64_t)N_kv * D;
  const float* Vh = V + ((int64_t)b * H_kv + hk) * (int64_t)N_kv * D;
  const int q0 = qb * kBM + wave * 32, qrow = q0 + lr, off = N_kv - N_q;

  // K index of the score contraction: lane half lh, step s <-> d = lh*D/2 + s
  float qreg[KH];
#pragma unroll
  for (int s = 0; s < KH; s += 4) {
    f32x4_t v = (qrow < N_q) ? *(const f32x4_t*)(Qh + (int64_t)qrow * D + lh * KH + s)
                             : f32x4_t{0, 0, 0, 0};
    qreg[s] = v[0]; qreg[s + 1] = v[1]; qreg[s + 2] = v[2]; qreg[s + 3] = v[3];
  }
  int kv_end = N_kv;
  if (CAUSAL) kv_end = min(N_kv, min(qb * kBM + kBM - 1, N_q - 1) + off + 1);
  const int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;

  f32x16_t oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16_t{0};
  float m = kNegInf, l = 0.f;

  for (int t = 0; t < ntiles; ++t) {
    const int kv0 = t * BN;
    constexpr int CPR = D / 4;
    for (int c = tid; c < BN * CPR; c += kThreads) {
      const int r = c / CPR, cc = c % CPR;
      f32x4_t kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (kv0 + r < N_kv) {
        kv = *(const f32x4_t*)(Kh + (int64_t)(kv0 + r) * D + cc * 4);
        vv = *(const f32x4_t*)(Vh + (int64_t)(kv0 + r) * D + cc * 4);
      }
      *(f32x4_t*)(sK + r * ST + cc * 4) = kv;
      *(f32x4_t*)(sV + r * ST + cc * 4) = vv;
    }
    __syncthreads();
    const bool live = !CAUSAL || kv0 <= q0 + 31 + off;
    if (live) {
      f32x16_t s = f32x16_t{0};
#pragma unroll
      for (int st = 0; st < KH; ++st) {
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(sK[lr * ST + lh * KH + st], qreg[st], s, 0, 0, 0);
      }
      const bool need_mask = (kv0 + BN > N_kv) || (CAUSAL && kv0 + BN - 1 > q0 + off);
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[r] * scale_log2;
        if (need_mask) {
          const int kv = kv0 + 8 * (r >> 2) + 4 * lh + (r & 3);
          if (kv >= N_kv || (CAUSAL && kv > qrow + off)) x = kNegInf;
        }
        s[r] = x;
        mx = fmaxf(mx, x);
      }
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m, mx);
      const float m_ref = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_ref);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(s[r] - m_ref);
        l += p;
        // K-slot of this step: half lh carries key 8*(r/4) + 4*lh + r%4
        const int kr = 8 * (r >> 2) + 4 * lh + (r & 3);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(sV[kr * ST + db * 32 + lr], p, oacc[db], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  l += xor32(l);
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  if (qrow < N_q) {
    float* Orow = O + ((int64_t)b * H_q + h) * (int64_t)N_q * D + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d = db * 32 + 8 * rg + 4 * lh;
        f32x4_t w = {oacc[db][4 * rg] * inv, oacc[db][4 * rg + 1] * inv, oacc[db][4 * rg + 2] * inv,
                     oacc[db][4 * rg + 3] * inv};
        *(f32x4_t*)(Orow + d) = w;
      }
    }
    if (LSE != nullptr && lh == 0) {
      LSE[((int64_t)b * H_q + h) * N_q + qrow] = (l > 0.f) ? (m + log2f(l)) * kLn2 : kNegInf;
    }
  }
}

// 1-D grid covering `items` work items, rounded up to a multiple of the 8 XCDs.
inline int xcd_grid(int64_t items) { return (int)(((items + 7) / 8) * 8); }

template <class TT, int D, int QB>
hipError_t launch16q(const PrefillArgs& a, hipStream_t st) {
  constexpr int BM = 4 * 32 * QB;
  const int nqb = (a.N_q + BM - 1) / BM;
  dim3 grid(xcd_grid((int64_t)nqb * a.H_q * a.B));
  const float sl2 = a.scale * kLog2e;
  auto q = (const uint16_t*)a.q;
  auto k = (const uint16_t*)a.k;
  auto v = (const uint16_t*)a.v;
  auto o = (uint16_t*)a.o;
  if (a.causal)
    hipLaunchKernelGGL((prefill16_kernel<TT, D, true, QB>), grid, dim3(kThreads), 0, st, q, k, v,
                       o, a.lse, a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, nqb, a.B);
  else
    hipLaunchKernelGGL((prefill16_kernel<TT, D, false, QB>), grid, dim3(kThreads), 0, st, q, k, v,
                       o, a.lse, a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, nqb, a.B);
  return hipGetLastError();
}

template <class TT, int D>
hipError_t launch16p(const PrefillArgs& a, hipStream_t st) {
  const int nqb = (a.N_q + kBM - 1) / kBM;
  dim3 grid(xcd_grid((int64_t)nqb * a.H_q * a.B));
  const float sl2 = a.scale * kLog2e;
  auto q = (const uint16_t*)a.q;
  auto k = (const uint16_t*)a.k;
  auto v = (const uint16_t*)a.v;
  auto o = (uint16_t*)a.o;
  if (a.causal)
    hipLaunchKernelGGL((prefill16_pipe_kernel<TT, D, true>), grid, dim3(kThreads), 0, st, q, k, v, o,
                       a.lse, a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, nqb, a.B);
  else
    hipLaunchKernelGGL((prefill16_pipe_kernel<TT, D, false>), grid, dim3(kThreads), 0, st, q, k, v, o,
                       a.lse, a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, nqb, a.B);
  return hipGetLastError();
}

// Kernel form for 16-bit inputs: the loop with one query block per wavefront
// by default; ATTN_PREFILL_VARIANT=2 selects two query blocks per wavefront and
// 3 the software-pipelined loop (tuning overrides).
template <class TT, int D>
hipError_t launch16(const PrefillArgs& a, hipStream_t st) {
  static const int variant = [] {
    const char* e = getenv("ATTN_PREFILL_VARIANT");
    return e ? atoi(e) : 0;
  }();
  if (variant == 2) return launch16q<TT, D, 2>(a, st);
  if (variant == 3) return launch16p<TT, D>(a, st);
  return launch16q<TT, D, 1>(a, st);
}

template <int D>
hipError_t launch32(const PrefillArgs& a, hipStream_t st) {
  const int nqb = (a.N_q + kBM - 1) / kBM;
  dim3 grid(nqb, a.H_q, a.B);
  const float sl2 = a.scale * kLog2e;
  auto q = (const float*)a.q;
  auto k = (const float*)a.k;
  auto v = (const float*)a.v;
  auto o = (float*)a.o;
  if (a.causal)
    hipLaunchKernelGGL((prefill32_kernel<D, true>), grid, dim3(kThreads), 0, st, q, k, v, o, a.lse,
                       a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, nqb);
  else
    hipLaunchKernelGGL((prefill32_kernel<D, false>), grid, dim3(kThreads), 0, st, q, k, v, o, a.lse,
                       a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, nqb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  switch (a.dtype) {
    case kDtypeBF16:
      return a.d == 64 ? launch16<BF16, 64>(a, st) : launch16<BF16, 128>(a, st);
    case kDtypeF16:
      return a.d == 64 ? launch16<F16, 64>(a, st) : launch16<F16, 128>(a, st);
    default:
      return a.d == 64 ? launch32<64>(a, st) : launch32<128>(a, st);
  }
}

}  // namespace attn
