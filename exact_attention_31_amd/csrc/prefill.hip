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
// gfx950 mapping (one workgroup = NW wavefronts of 32 query rows: 8 for
// d = 128, 4 for d = 64; a persistent grid when work items are plentiful):
//   * Q rows stay in VGPRs for the whole loop, laid out as the B operand of
//     S^T = K Q^T (v_mfma_f32_32x32x16): each lane owns one query row, and the
//     accumulator layout then gives each lane 16 of the 32 scores of its row,
//     so the row max/sum needs one exchange with the opposite half-wave only.
//   * K and V tiles (64 keys) go through LDS, shared by all the workgroup's
//     wavefronts: staged through registers with 16-byte coalesced loads
//     (prefill16_kernel), or streamed by direct-to-LDS loads into a ring
//     (prefill16_ring_kernel).
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

// Row stride (elements) of the K and V tiles in LDS (64 banks of 4 bytes).
// K: rows 68 dwords apart, so the 16-byte reads of 16 consecutive rows cover
// all banks once. V: a transposing read has two 16-lane groups each take 4
// rows x 8 dwords, the second group 8 dwords further right; rows 16 (mod 64)
// dwords apart put the 8 row segments of both groups on disjoint banks.
template <int D> struct Lds16 {
  static constexpr int kK = D + 8;
  static constexpr int kV = (D == 128) ? 160 : 96;
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
  int valid;  // an int, not a bool: no padding bytes for a struct copy to move
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
  // wavefronts per SIMD the register budget must allow (d = 64 fits three)
  static constexpr int kWaves = (QB == 2 && D == 128) ? 1 : (QB == 1 && D == 64) ? 3 : 2;
};

// Rows mode (row_period P > 0, used by multi-token decode): the N_q rows of a
// "head" are P consecutive tokens of each of N_q / P query heads that share
// one KV head, row r being token r % P; causal alignment is per token, and
// kv_lens (if given) bounds each request's keys.
template <class TT, int D, bool CAUSAL, int QB, int NW = 4, bool PERSIST = false>
__global__ __launch_bounds__(64 * NW, (NW == 8 ? 1 : Occ<QB, D>::kWaves)) void prefill16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int H_q, int H_kv, int N_q, int N_kv,
    float scale_log2, int nqb, int nbatch, const int* __restrict__ kv_lens = nullptr,
    int row_period = 0) {
  constexpr int KST = Lds16<D>::kK;
  constexpr int VST = Lds16<D>::kV;
  constexpr int KS = D / 16;   // k-steps of the score MFMA
  constexpr int DB = D / 32;   // 32-wide blocks of the output
  constexpr int CPR = D / 8;   // 16-byte chunks per K/V row
  constexpr int NT = 64 * NW;                // threads per workgroup
  constexpr int LPT = kBN * CPR / NT;        // 16-byte loads per thread per tile, per tensor
  constexpr int BM = NW * 32 * QB;           // query rows per workgroup
  static_assert(LPT * NT == kBN * CPR, "tile load must split evenly");
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kBN * KST];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][kBN * VST];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // scalar, so that every per-wavefront decision below is a uniform branch
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const uint32_t head_q_bytes = (uint32_t)N_q * D * 2;

  // ---- work items. One per workgroup (map_work), or, persistent: the grid
  // holds as many workgroups as can be resident, and each walks items of its
  // XCD's contiguous range (the same ranges as map_work). Slot s of an XCD
  // takes items s, then 2*nslots - 1 - s, then 2*nslots + s, ...: a zig-zag, so
  // that with causal masking (items of a head ordered longest first) every
  // slot gets a mix of long and short query blocks.
  int round = 0;
  auto next_item = [&](WorkItem& w) -> bool {
    if constexpr (!PERSIST) {
      if (round++ > 0) return false;
      w = map_work(nqb, H_q, nbatch, CAUSAL);
      return w.valid;
    } else {
      const int total = nqb * H_q * nbatch;
      const int per_xcd = (total + 7) >> 3;
      const int nslots = (int)gridDim.x >> 3, slot = (int)blockIdx.x >> 3;
      const int r = round++;
      const int it = r * nslots + ((r & 1) ? (nslots - 1 - slot) : slot);
      const int item = (int)(blockIdx.x & 7) * per_xcd + it;
      if (it >= per_xcd || item >= total) return false;
      const int unit = item / nqb;
      const int qi = item - unit * nqb;
      w.valid = true;
      w.qblk = CAUSAL ? (nqb - 1 - qi) : qi;
      w.b = unit / H_q;
      w.h = unit - w.b * H_q;
      return true;
    }
  };
  // per-item addressing and bounds
  struct Ctx {
    __amdgpu_buffer_rsrc_t rQ, rK, rV;
    int b, h, qblk, q0, ntiles;
    int lo_lim, hi_lim;  // least and greatest key limit over the wavefront's rows
    int qrow[QB], lim[QB];
  };
  auto ctx_of = [&](const WorkItem& wi) {
    Ctx c;
    c.b = wi.b;
    c.h = wi.h;
    c.qblk = wi.qblk;
    const int hk = wi.h / (H_q / H_kv);
    const int len = kv_lens ? min(max(kv_lens[wi.b], 0), N_kv) : N_kv;  // this request's keys
    const int ntok = row_period > 0 ? row_period : N_q;  // query tokens per head
    const int off = len - ntok;                          // bottom-right causal alignment
    c.rQ = buffer_rsrc(Q + ((int64_t)wi.b * H_q + wi.h) * (int64_t)N_q * D, head_q_bytes);
    c.rK = buffer_rsrc(K + ((int64_t)wi.b * H_kv + hk) * (int64_t)N_kv * D, (uint32_t)len * D * 2);
    c.rV = buffer_rsrc(V + ((int64_t)wi.b * H_kv + hk) * (int64_t)N_kv * D, (uint32_t)len * D * 2);
    c.q0 = wi.qblk * BM + wave * 32 * QB;  // first row of this wavefront
    int lo = len, hi = 0;
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      c.qrow[j] = c.q0 + 32 * j + lr;  // this lane's row in query block j
      const int tok = row_period > 0 ? c.qrow[j] % row_period : c.qrow[j];
      // keys below lim[j] are visible to that row
      c.lim[j] = CAUSAL ? min(len, max(tok + off + 1, 0)) : len;
      lo = min(lo, c.lim[j]);
      hi = max(hi, c.lim[j]);
    }
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) {
      lo = min(lo, __shfl_xor(lo, o));
      hi = max(hi, __shfl_xor(hi, o));
    }
    c.lo_lim = __builtin_amdgcn_readfirstlane(lo);
    c.hi_lim = __builtin_amdgcn_readfirstlane(hi);
    int kv_end = len;
    if (CAUSAL && row_period == 0) {
      const int qlast = min(wi.qblk * BM + BM - 1, N_q - 1);
      kv_end = min(len, qlast + off + 1);
    }
    c.ntiles = kv_end > 0 ? (kv_end + kBN - 1) / kBN : 0;
    return c;
  };

  // Q^T operand: lane holds row qrow[j], d = 16*s + 8*lh + 0..7 (rows past N_q read as 0)
  u32x4_t qreg[QB][KS];
  auto load_q = [&](const Ctx& c) {
#pragma unroll
    for (int j = 0; j < QB; ++j)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        qreg[j][s] = buffer_load16(c.rQ, (uint32_t)(c.qrow[j] * D + 16 * s + 8 * lh) * 2);
  };

  // this thread's share of each tile: chunk c = tid + NT*i -> row c / CPR, column c % CPR
  uint32_t ld_off[LPT];
  int st_k[LPT], st_v[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int c = tid + NT * i;
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
  auto load_tile = [&](const Ctx& c, int t) {
    const uint32_t base = (uint32_t)(t * kBN) * D * 2;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      kbuf[i] = buffer_load16(c.rK, base + ld_off[i]);
      vbuf[i] = buffer_load16(c.rV, base + ld_off[i]);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      *(u32x4_t*)(&sK[buf][st_k[i]]) = kbuf[i];
      *(u32x4_t*)(&sV[buf][st_v[i]]) = vbuf[i];
    }
  };

  WorkItem cur;
  if (!next_item(cur)) return;
  Ctx c = ctx_of(cur);
  // Tile 0 is staged unconditionally (loads past the end read zeros): with no
  // branch here every load issued so far has completed when the loop starts,
  // so the loop only ever waits for its own prefetch, at the LDS store.
  load_q(c);
  load_tile(c, 0);
  store_tile(0);
  vmem_wait_all();
  __syncthreads();
  int par = 0;  // LDS buffer holding the current item's tile 0

  for (;;) {
    // The next item's tile 0 is loaded during this item's last tile, and its
    // Q rows at the end of that tile, so that the next item starts with its
    // operands in place.
    // (with no next item, nwi stays the current one and cn is not used)
    WorkItem nwi = cur;
    const bool has_next = next_item(nwi);
    const Ctx cn = ctx_of(nwi);

    f32x16_t oacc[QB][DB];
    float m[QB], l[QB];
#pragma unroll
    for (int j = 0; j < QB; ++j) {
#pragma unroll
      for (int i = 0; i < DB; ++i) oacc[j][i] = f32x16_t{0};
      m[j] = kNegInf;  // reference maximum, in units of log2 (scores * scale * log2 e)
      l[j] = 0.f;      // this half-wave's part of the denominator
    }
    const int ntiles = c.ntiles;

    for (int t = 0; t < ntiles; ++t) {
      const int buf = (t + par) & 1;
      const bool last = t + 1 == ntiles;
      if (!last) load_tile(c, t + 1);  // in flight during this tile's math
      else if (has_next) load_tile(cn, 0);
      const int kv0 = t * kBN;
      // wavefront-uniform: does this tile hold any key visible to this wavefront?
      const bool live = kv0 < c.hi_lim;
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
        // keep the K operand reads two k-steps ahead of the MFMAs that use them
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int st = 0; st < KS - 2; ++st) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * QB, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * QB, 0);
        // V^T operands of this tile, requested now so that the score MFMAs, the
        // row max and the exponentials cover their LDS latency
        u32x4_t vop[4][DB];
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const u32x2_t lo = lds_read_tr16(tV + 16 * t4 * VST + db * 32);
            const u32x2_t hi = lds_read_tr16(tV + (16 * t4 + 8) * VST + db * 32);
            vop[t4][db] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
          }
        // ---- mask (tail and causal diagonal tiles only), branch-free per element
        const bool need_mask = kv0 + kBN > c.lo_lim;
        if (need_mask) {
#pragma unroll
          for (int j = 0; j < QB; ++j) {
            // key kv0 + 4*lh + e (e a per-register constant) is visible iff e < rel
            const int rel = c.lim[j] - (kv0 + 4 * lh);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int e = 8 * (r >> 2) + (r & 3);
              s[j][0][r] = (e < rel) ? s[j][0][r] : kNegInf;
              s[j][1][r] = (e + 32 < rel) ? s[j][1][r] : kNegInf;
            }
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
            const u32x4_t aop = vop[t4][db];
#pragma unroll
            for (int j = 0; j < QB; ++j) {
              const u32x4_t bop = {pk[j][4 * t4 + 0], pk[j][4 * t4 + 1], pk[j][4 * t4 + 2],
                                   pk[j][4 * t4 + 3]};
              oacc[j][db] = TT::mfma32(aop, bop, oacc[j][db]);
            }
          }
        }
      }
      if (!last || has_next) store_tile(buf ^ 1);
      if (last && has_next) load_q(cn);  // this item's Q is no longer read
      __syncthreads();
    }
    if (ntiles == 0 && has_next) {  // no keys: stage the next item here
      load_q(cn);
      load_tile(cn, 0);
      store_tile(par ^ 1);
    }

    // ---- epilogue: combine half-wave denominators, normalise, store (rows past N_q dropped)
    const auto rO = buffer_rsrc(O + ((int64_t)c.b * H_q + c.h) * (int64_t)N_q * D, head_q_bytes);
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
          buffer_store8(rO, (uint32_t)(c.qrow[j] * D + d) * 2, w);
        }
      }
      if (LSE != nullptr && lh == 0 && c.qrow[j] < N_q) {
        LSE[((int64_t)c.b * H_q + c.h) * N_q + c.qrow[j]] =
            (lt > 0.f) ? (m[j] + log2f(lt)) * kLn2 : kNegInf;
      }
    }
    if (!has_next) break;
    vmem_wait_all();
    __syncthreads();
    par = (par + (ntiles > 0 ? ntiles : 1)) & 1;
    cur = nwi;
    c = ctx_of(cur);
  }
}

// Phase-skewed form: 8 wavefronts, two per SIMD (wavefronts w and w + 4 share
// a SIMD). Group A (wavefronts 0-3) works tile t as S(t) -> softmax(t) ->
// PV(t); group B (4-7) runs half a tile behind: softmax(t-1) -> PV(t-1) ->
// S(t), carrying its scores across the barrier. So while one wavefront of a
// SIMD turns scores into probabilities on the vector ALUs, the other keeps the
// matrix cores busy, instead of both doing the same phase at once. V tiles are
// read one iteration longer (by group B), so V has three LDS buffers and K two;
// one extra iteration at the end lets group B finish the last tile.
template <class TT, int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void prefill16_skew_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int H_q, int H_kv, int N_q, int N_kv,
    float scale_log2, int nqb, int nbatch) {
  constexpr int KST = Lds16<D>::kK;
  constexpr int VST = Lds16<D>::kV;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int CPR = D / 8;
  constexpr int NT = 512;
  constexpr int LPT = kBN * CPR / NT;
  constexpr int BM = 256;
  static_assert(LPT >= 1 && LPT * NT == kBN * CPR, "tile load must split evenly");
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kBN * KST];
  __shared__ __attribute__((aligned(16))) uint16_t sV[3][kBN * VST];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool grpB = wave >= 4;
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
  const int q0 = qblk * BM + wave * 32;
  const int off = N_kv - N_q;
  const int qrow = q0 + lr;
  const int lim = CAUSAL ? min(N_kv, max(qrow + off + 1, 0)) : N_kv;

  u32x4_t qreg[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) qreg[st] = buffer_load16(rQ, (uint32_t)(qrow * D + 16 * st + 8 * lh) * 2);

  int kv_end = N_kv;
  if (CAUSAL) {
    const int qlast = min(qblk * BM + BM - 1, N_q - 1);
    kv_end = min(N_kv, qlast + off + 1);
  }
  const int ntiles = kv_end > 0 ? (kv_end + kBN - 1) / kBN : 0;

  uint32_t ld_off[LPT];
  int st_k[LPT], st_v[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int c = tid + NT * i;
    const int r = c / CPR, cc = c % CPR;
    ld_off[i] = (uint32_t)(r * D + cc * 8) * 2;
    st_k[i] = r * KST + cc * 8;
    st_v[i] = r * VST + cc * 8;
  }
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
  auto store_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      *(u32x4_t*)(&sK[t & 1][st_k[i]]) = kbuf[i];
      *(u32x4_t*)(&sV[t % 3][st_v[i]]) = vbuf[i];
    }
  };

  f32x16_t oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16_t{0};
  float m = kNegInf, l = 0.f;

  // does tile t hold any key visible to this wavefront?
  auto live = [&](int t) { return !CAUSAL || t * kBN <= q0 + 31 + off; };
  auto scores = [&](int t, f32x16_t& s0, f32x16_t& s1) {
    const uint16_t* tK = &sK[t & 1][0] + k_lane;
    s0 = f32x16_t{0};
    s1 = f32x16_t{0};
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const u32x4_t a0 = *(const u32x4_t*)(tK + 16 * st);
      const u32x4_t a1 = *(const u32x4_t*)(tK + 32 * KST + 16 * st);
      s0 = TT::mfma32(a0, qreg[st], s0);
      s1 = TT::mfma32(a1, qreg[st], s1);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int st = 0; st < KS - 2; ++st) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };
  // softmax of the scores in s0/s1 (tile t) and O^T += V(t)^T P^T
  auto softmax_pv = [&](int t, f32x16_t& s0, f32x16_t& s1) {
    const uint16_t* tV = &sV[t % 3][0] + v_lane;
    const int kv0 = t * kBN;
    const bool need_mask = (kv0 + kBN > N_kv) || (CAUSAL && kv0 + kBN - 1 > q0 + off);
    if (need_mask) {
      const int rel = lim - (kv0 + 4 * lh);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = 8 * (r >> 2) + (r & 3);
        s0[r] = (e < rel) ? s0[r] : kNegInf;
        s1[r] = (e + 32 < rel) ? s1[r] : kNegInf;
      }
    }
    float mx = max3(s0[0], s0[1], s1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = max3(mx, s0[r], s1[r]);
    mx = fmaxf(mx, s1[0]);
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
    uint32_t pk[16];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = fast_exp2(__builtin_fmaf(s0[r], scale_log2, nm));
      const float p1 = fast_exp2(__builtin_fmaf(s0[r + 1], scale_log2, nm));
      const float p2 = fast_exp2(__builtin_fmaf(s1[r], scale_log2, nm));
      const float p3 = fast_exp2(__builtin_fmaf(s1[r + 1], scale_log2, nm));
      l += (p0 + p1) + (p2 + p3);
      pk[r >> 1] = TT::pack2(p0, p1);
      pk[8 + (r >> 1)] = TT::pack2(p2, p3);
    }
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const u32x4_t bop = {pk[4 * t4 + 0], pk[4 * t4 + 1], pk[4 * t4 + 2], pk[4 * t4 + 3]};
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2_t lo = lds_read_tr16(tV + 16 * t4 * VST + db * 32);
        const u32x2_t hi = lds_read_tr16(tV + (16 * t4 + 8) * VST + db * 32);
        oacc[db] = TT::mfma32(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, bop, oacc[db]);
      }
    }
    // V operand reads two MFMAs ahead of their use
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 4 * DB - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  };

  load_tile(0);
  store_tile(0);
  vmem_wait_all();
  __syncthreads();

  // The two groups run separate loops (so that group B's carried scores do not
  // occupy registers in group A's code); both pass the same barriers.
  const int niter = ntiles > 0 ? ntiles + 1 : 0;
  if (grpB) {
    f32x16_t c0 = f32x16_t{0}, c1 = f32x16_t{0};  // scores carried to the next iteration
    for (int t = 0; t < niter; ++t) {
      if (t + 1 < ntiles) load_tile(t + 1);
      if (t >= 1 && live(t - 1)) softmax_pv(t - 1, c0, c1);
      if (t < ntiles && live(t)) scores(t, c0, c1);
      if (t + 1 < ntiles) store_tile(t + 1);
      __syncthreads();
    }
  } else {
    for (int t = 0; t < niter; ++t) {
      if (t + 1 < ntiles) load_tile(t + 1);
      if (t < ntiles && live(t)) {
        f32x16_t a0, a1;
        scores(t, a0, a1);
        softmax_pv(t, a0, a1);
      }
      if (t + 1 < ntiles) store_tile(t + 1);
      __syncthreads();
    }
  }

  const auto rO = buffer_rsrc(O + ((int64_t)b * H_q + h) * (int64_t)N_q * D, head_q_bytes);
  const float lt = half_sum(l);
  const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
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
    LSE[((int64_t)b * H_q + h) * N_q + qrow] = (lt > 0.f) ? (m + log2f(lt)) * kLn2 : kNegInf;
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

// Two-group form: 8 wavefronts (two per SIMD) share each K/V tile; 256 query
// rows per workgroup, 32 per wavefront. Every tile t is worked in two phases:
//   X(t): scores of tile t+1 on the matrix cores, interleaved with the
//         softmax of tile t on the vector ALUs;
//   Y(t): O += V(t) P(t) on the matrix cores.
// Group 0 (wavefronts 0-3) runs X(t) while group 1 (wavefronts 4-7) runs
// Y(t-1), and then Y(t) while group 1 runs X(t), so on each SIMD one
// wavefront's vector work overlaps the other's matrix work. Phases are
// separated by workgroup barriers ("half-steps" h = 0 .. 2*ntiles).
// LDS holds two K and two V tiles, rotated as described at the prologue.
constexpr int kPPThreads = 512;
constexpr int kPPBM = 256;

template <class TT, int D, bool CAUSAL, bool PIPE>
__global__ __launch_bounds__(kPPThreads, 1) void prefill16_pp_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int H_q, int H_kv, int N_q, int N_kv,
    float scale_log2, int nqb, int nbatch) {
  constexpr int KST = Lds16<D>::kK;
  constexpr int VST = Lds16<D>::kV;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int CPR = D / 8;
  constexpr int LPT = kBN * CPR / kPPThreads;
  static_assert(LPT >= 1 && LPT * kPPThreads == kBN * CPR, "tile load must split evenly");
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kBN * KST];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][kBN * VST];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
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

  const int q0 = qblk * kPPBM + wave * 32;
  const int qrow = q0 + lr;
  const int off = N_kv - N_q;
  const int lim = CAUSAL ? min(N_kv, max(qrow + off + 1, 0)) : N_kv;

  u32x4_t qreg[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) qreg[st] = buffer_load16(rQ, (uint32_t)(qrow * D + 16 * st + 8 * lh) * 2);

  int kv_end = N_kv;
  if (CAUSAL) kv_end = min(N_kv, min(qblk * kPPBM + kPPBM - 1, N_q - 1) + off + 1);
  const int ntiles = kv_end > 0 ? (kv_end + kBN - 1) / kBN : 0;
  int wtiles = ntiles;  // tiles holding a key visible to some row of this wavefront
  if (CAUSAL) wtiles = min(ntiles, max(0, (q0 + 31 + off + kBN) / kBN));

  uint32_t ld_off[LPT];
  int st_k[LPT], st_v[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int c = tid + kPPThreads * i;
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

  // K look-ahead: with PIPE, X(t) reads K(t+1), else K(t). Buffer schedule:
  //   end of even half-step 2t: store K(t+KA) into K buffer (t+KA)%2, whose
  //     previous tile K(t+KA-2) was last read in half-step 2t-1;
  //   end of odd half-step 2t+1: store V(t+1) into V buffer (t+1)%2, whose
  //     previous tile V(t-1) was last read (group 1, Y(t-1)) in half-step 2t.
  // K(t+KA+1) is loaded at the start of half-step 2t+1, V(t+1) at the start of 2t.
  constexpr int KA = PIPE ? 2 : 1;
  // prologue: K(0..KA-1), V(0) in LDS, K(KA) in flight
  load_k(0);
  load_v(0);
  store_k(0);
  store_v(0);
  if constexpr (PIPE) {
    load_k(1);
    store_k(1);
  }
  load_k(KA);
  vmem_wait_all();
  __syncthreads();

  f32x16_t oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16_t{0};
  float m = kNegInf, l = 0.f;
  f32x16_t sc0, sc1;  // scores of the tile being turned into probabilities
  uint32_t pk[16];    // its probabilities, 16-bit pairs, B operand of P V
  if constexpr (PIPE) {
    const uint16_t* tK = &sK[0][0] + k_lane;
    sc0 = f32x16_t{0};
    sc1 = f32x16_t{0};
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      sc0 = TT::mfma32(*(const u32x4_t*)(tK + 16 * st), qreg[st], sc0);
      sc1 = TT::mfma32(*(const u32x4_t*)(tK + 32 * KST + 16 * st), qreg[st], sc1);
    }
  }

  // X(t): softmax of S(t) -> pk. With PIPE, S(t+1) = K(t+1) Q^T is computed on
  // the matrix cores in the same phase (interleaved with the softmax); without
  // it, S(t) is computed at the start of X(t).
  auto phase_x = [&](int t) {
    const int kv0 = t * kBN;
    if constexpr (!PIPE) {
      const uint16_t* tK = &sK[0][0] + (t & 1) * (kBN * KST) + k_lane;
      sc0 = f32x16_t{0};
      sc1 = f32x16_t{0};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        sc0 = TT::mfma32(*(const u32x4_t*)(tK + 16 * st), qreg[st], sc0);
        sc1 = TT::mfma32(*(const u32x4_t*)(tK + 32 * KST + 16 * st), qreg[st], sc1);
      }
    }
    const bool need_mask = (kv0 + kBN > N_kv) || (CAUSAL && kv0 + kBN - 1 > q0 + off);
    if (need_mask) {
      const int kvb = kv0 + 4 * lh;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kv = kvb + 8 * (r >> 2) + (r & 3);
        sc0[r] = (kv < lim) ? sc0[r] : kNegInf;
        sc1[r] = (kv + 32 < lim) ? sc1[r] : kNegInf;
      }
    }
    float mx = max3(sc0[0], sc0[1], sc1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = max3(mx, sc0[r], sc1[r]);
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
    f32x16_t n0 = f32x16_t{0}, n1 = f32x16_t{0};
    if constexpr (PIPE) {
      const uint16_t* tK = &sK[0][0] + ((t + 1) & 1) * (kBN * KST) + k_lane;
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        n0 = TT::mfma32(*(const u32x4_t*)(tK + 16 * st), qreg[st], n0);
        n1 = TT::mfma32(*(const u32x4_t*)(tK + 32 * KST + 16 * st), qreg[st], n1);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = fast_exp2(__builtin_fmaf(sc0[r], scale_log2, nm));
      const float p1 = fast_exp2(__builtin_fmaf(sc0[r + 1], scale_log2, nm));
      const float p2 = fast_exp2(__builtin_fmaf(sc1[r], scale_log2, nm));
      const float p3 = fast_exp2(__builtin_fmaf(sc1[r + 1], scale_log2, nm));
      l += (p0 + p1) + (p2 + p3);
      pk[r >> 1] = TT::pack2(p0, p1);
      pk[8 + (r >> 1)] = TT::pack2(p2, p3);
    }
    if constexpr (PIPE) {
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads of K
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two score MFMAs
        __builtin_amdgcn_sched_group_barrier(0x002, 112 / KS, 0);  // softmax VALU
      }
      sc0 = n0;
      sc1 = n1;
    }
  };
  // Y(t): O^T += V(t)^T P(t)^T
  auto phase_y = [&](int t) {
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
  };

  const int nhalf = 2 * ntiles + 1;
  for (int hs = 0; hs < nhalf; ++hs) {
    const int t = hs >> 1;
    const bool even = (hs & 1) == 0;
    // HBM -> registers: V(t+1) at even half-steps, K(t+KA+1) at odd ones
    if (even) {
      if (t + 1 < ntiles) load_v(t + 1);
    } else {
      if (t + KA + 1 < ntiles) load_k(t + KA + 1);
    }
    // group 0: X(t) at even half-steps, Y(t) at odd; group 1: Y(t-1), then X(t)
    const bool do_x = (grp == 0) == even;
    const int tt = (grp == 1 && even) ? t - 1 : t;
    if (tt >= 0 && tt < wtiles) {
      if (do_x)
        phase_x(tt);
      else
        phase_y(tt);
    }
    // registers -> LDS: K(t+KA) after even half-steps, V(t+1) after odd ones
    if (even) {
      if (t + KA < ntiles) store_k((t + KA) & 1);
    } else {
      if (t + 1 < ntiles) store_v((t + 1) & 1);
    }
    __syncthreads();
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

// Direct-load form: 32-key tiles streamed HBM -> LDS by buffer loads that
// write LDS themselves (no staging registers), three tiles in a ring, so a tile
// is requested two tiles before its use. LDS rows are unpadded and their
// 16-byte chunks XOR-swizzled:
//   K: chunk c of row r sits at c ^ ((r / RPB) % CPR): the 16 rows read by one
//      16-lane slice of a score-MFMA operand fetch land on 16 distinct banks;
//   V: chunk c of row r sits at c ^ 4*((r / RPB) % (4 / RPB)): the 4 rows of a
//      transposing read land on distinct banks;
// (RPB rows per 256-byte bank sweep, CPR chunks per row). One load instruction
// fills 1 KB of LDS, lane j writing chunk j, so each lane fetches the logical
// chunk that its physical slot holds.
constexpr int kDLBN = 32;
constexpr int kDLStages = 3;

template <int D, int BN = kDLBN> struct DL {
  static constexpr int RB = D * 2;
  static constexpr int CPR = D / 8;
  static constexpr int RPB = 256 / RB;
  static constexpr int TILE = BN * RB;          // bytes per tensor tile
  static constexpr int STAGE = 2 * TILE;        // K then V
  static constexpr int BLK = TILE / 1024;       // 1 KB load blocks per tensor tile
  static constexpr int BPW = BLK / 4;           // per wavefront
  static __device__ __forceinline__ int kswz(int r) { return (r / RPB) & (CPR - 1); }
  static __device__ __forceinline__ int vswz(int r) { return 4 * ((r / RPB) & (RPB == 1 ? 3 : 1)); }
};

template <class TT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, (D == 128 ? 2 : 4)) void prefill16_dl_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int H_q, int H_kv, int N_q, int N_kv,
    float scale_log2, int nqb, int nbatch) {
  using L = DL<D>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  static_assert(L::BPW >= 1 && L::BPW * 4 == L::BLK, "tile must split over 4 wavefronts");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kDLStages * L::STAGE];

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
  const int ntiles = kv_end > 0 ? (kv_end + kDLBN - 1) / kDLBN : 0;
  int wtiles = ntiles;
  if (CAUSAL) wtiles = min(ntiles, max(0, (q0 + 31 + off + kDLBN) / kDLBN));

  // direct loads: block i of this wavefront -> LDS bytes [blk*1024, +1024) of the
  // tile; lane j writes physical chunk p = blk*64 + j = (row p / CPR, slot p % CPR)
  uint32_t kg_off[L::BPW], vg_off[L::BPW];
#pragma unroll
  for (int i = 0; i < L::BPW; ++i) {
    const int p = (wave * L::BPW + i) * 64 + lane;
    const int r = p / L::CPR, slot = p % L::CPR;
    kg_off[i] = (uint32_t)(r * L::RB + ((slot ^ L::kswz(r)) * 16));
    vg_off[i] = (uint32_t)(r * L::RB + ((slot ^ L::vswz(r)) * 16));
  }
  const auto dK = buffer_rsrc(K + ((int64_t)b * H_kv + hk) * (int64_t)N_kv * D, head_kv_bytes);
  const auto dV = buffer_rsrc(V + ((int64_t)b * H_kv + hk) * (int64_t)N_kv * D, head_kv_bytes);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  auto issue_tile = [&](int t) {
    const int stage = t % kDLStages;
    const uint32_t g0 = (uint32_t)(t * kDLBN) * L::RB;
#pragma unroll
    for (int i = 0; i < L::BPW; ++i) {
      const uint32_t kd = lds0 + stage * L::STAGE + (wave * L::BPW + i) * 1024;
      dma_load16(dK, g0 + kg_off[i], kd);
      dma_load16(dV, g0 + vg_off[i], kd + L::TILE);
    }
  };
  // operand addresses within a stage (bytes)
  //   K (score A operand): row lr, logical chunk 2*st + lh
  //   V (transposing read): row 16*t4 + 4*lh + gi/4 (+8), logical chunk
  //     4*db + 2*(g&1) + (gi&3)/2, 8-byte half gi&1
  int ka[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) ka[st] = lr * L::RB + (((2 * st + lh) ^ L::kswz(lr)) * 16);
  const int g = lane >> 4, gi = lane & 15;
  const int vrow = 4 * (g >> 1) + (gi >> 2);  // plus 16*t4 (+8); the swizzle only sees vrow % 4 (or % 8)
  int va[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    va[db] = L::TILE + vrow * L::RB + (((4 * db + 2 * (g & 1) + ((gi & 3) >> 1)) ^ L::vswz(vrow)) * 16) +
             8 * (gi & 1);

  issue_tile(0);
  if (ntiles > 1) issue_tile(1);
  vmem_wait_all();
  __syncthreads();

  f32x16_t oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16_t{0};
  float m = kNegInf, l = 0.f;

  for (int t = 0; t < ntiles; ++t) {
    const bool ahead = t + 2 < ntiles;
    if (ahead) issue_tile(t + 2);
    if (t < wtiles) {
      const uint8_t* st_base = smem + (t % kDLStages) * L::STAGE;
      const int kv0 = t * kDLBN;
      f32x16_t s0 = f32x16_t{0};
#pragma unroll
      for (int st = 0; st < KS; ++st) s0 = TT::mfma32(*(const u32x4_t*)(st_base + ka[st]), qreg[st], s0);
      const bool need_mask = (kv0 + kDLBN > N_kv) || (CAUSAL && kv0 + kDLBN - 1 > q0 + off);
      if (need_mask) {
        const int kvb = kv0 + 4 * lh;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kv = kvb + 8 * (r >> 2) + (r & 3);
          s0[r] = (kv < lim) ? s0[r] : kNegInf;
        }
      }
      float mx = max3(s0[0], s0[1], s0[2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) mx = max3(mx, s0[r], s0[r + 1]);
      mx = fmaxf(mx, s0[15]);
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
      uint32_t pk[8];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s0[r], scale_log2, nm));
        const float p1 = fast_exp2(__builtin_fmaf(s0[r + 1], scale_log2, nm));
        l += p0 + p1;
        pk[r >> 1] = TT::pack2(p0, p1);
      }
#pragma unroll
      for (int t4 = 0; t4 < 2; ++t4) {
        const u32x4_t bop = {pk[4 * t4 + 0], pk[4 * t4 + 1], pk[4 * t4 + 2], pk[4 * t4 + 3]};
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x2_t lo = lds_read_tr16((const uint16_t*)(st_base + va[db] + 16 * t4 * L::RB));
          const u32x2_t hi = lds_read_tr16((const uint16_t*)(st_base + va[db] + (16 * t4 + 8) * L::RB));
          const u32x4_t aop = {lo[0], lo[1], hi[0], hi[1]};
          oacc[db] = TT::mfma32(aop, bop, oacc[db]);
        }
      }
    }
    // tile t+1 must have landed (in-order count: only tile t+2's loads may be pending)
    if (ahead)
      __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * L::BPW));
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
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

// Two-block form: each wavefront owns 64 query rows (two 32-row blocks), so
// every K or V operand read from LDS feeds two MFMAs, halving LDS traffic per
// FLOP; one wavefront per SIMD with the full register file. 32-key tiles are
// streamed by direct loads into a 4-stage LDS ring, issued three tiles ahead.
// The scores of tile t+1 are computed while tile t's exponentials run, so the
// matrix cores and the vector ALUs work in the same stretch of code:
//   iteration t: issue tile t+3; softmax statistics of S(t); S(t+1) = K(t+1) Q^T
//   interleaved with P(t) = exp2(...); O += V(t) P(t); wait for tile t+2; barrier.
constexpr int kW2Stages = 4;
constexpr int kW2BM = 256;

template <class TT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void prefill16_w2_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int H_q, int H_kv, int N_q, int N_kv,
    float scale_log2, int nqb, int nbatch) {
  using L = DL<D>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  static_assert(L::BPW >= 1 && L::BPW * 4 == L::BLK, "tile must split over 4 wavefronts");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kW2Stages * L::STAGE];

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

  const int q0 = qblk * kW2BM + wave * 64;  // first row of this wavefront
  const int off = N_kv - N_q;
  int qrow[2], lim[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    qrow[j] = q0 + 32 * j + lr;
    lim[j] = CAUSAL ? min(N_kv, max(qrow[j] + off + 1, 0)) : N_kv;
  }
  u32x4_t qreg[2][KS];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int st = 0; st < KS; ++st)
      qreg[j][st] = buffer_load16(rQ, (uint32_t)(qrow[j] * D + 16 * st + 8 * lh) * 2);

  int kv_end = N_kv;
  if (CAUSAL) kv_end = min(N_kv, min(qblk * kW2BM + kW2BM - 1, N_q - 1) + off + 1);
  const int ntiles = kv_end > 0 ? (kv_end + kDLBN - 1) / kDLBN : 0;
  int wtiles = ntiles;
  if (CAUSAL) wtiles = min(ntiles, max(0, (q0 + 63 + off + kDLBN) / kDLBN));

  uint32_t kg_off[L::BPW], vg_off[L::BPW];
#pragma unroll
  for (int i = 0; i < L::BPW; ++i) {
    const int p = (wave * L::BPW + i) * 64 + lane;
    const int r = p / L::CPR, slot = p % L::CPR;
    kg_off[i] = (uint32_t)(r * L::RB + ((slot ^ L::kswz(r)) * 16));
    vg_off[i] = (uint32_t)(r * L::RB + ((slot ^ L::vswz(r)) * 16));
  }
  const auto dK = buffer_rsrc(K + ((int64_t)b * H_kv + hk) * (int64_t)N_kv * D, head_kv_bytes);
  const auto dV = buffer_rsrc(V + ((int64_t)b * H_kv + hk) * (int64_t)N_kv * D, head_kv_bytes);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  auto issue_tile = [&](int t) {
    const int stage = t & (kW2Stages - 1);
    const uint32_t g0 = (uint32_t)(t * kDLBN) * L::RB;
#pragma unroll
    for (int i = 0; i < L::BPW; ++i) {
      const uint32_t kd = lds0 + stage * L::STAGE + (wave * L::BPW + i) * 1024;
      dma_load16(dK, g0 + kg_off[i], kd);
      dma_load16(dV, g0 + vg_off[i], kd + L::TILE);
    }
  };
  int ka[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) ka[st] = lr * L::RB + (((2 * st + lh) ^ L::kswz(lr)) * 16);
  const int g = lane >> 4, gi = lane & 15;
  const int vrow = 4 * (g >> 1) + (gi >> 2);
  int va[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    va[db] = L::TILE + vrow * L::RB + (((4 * db + 2 * (g & 1) + ((gi & 3) >> 1)) ^ L::vswz(vrow)) * 16) +
             8 * (gi & 1);
  auto gemm_s = [&](int t, f32x16_t (&sn)[2]) {
    const uint8_t* base = smem + (t & (kW2Stages - 1)) * L::STAGE;
    sn[0] = f32x16_t{0};
    sn[1] = f32x16_t{0};
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const u32x4_t a = *(const u32x4_t*)(base + ka[st]);
      sn[0] = TT::mfma32(a, qreg[0][st], sn[0]);
      sn[1] = TT::mfma32(a, qreg[1][st], sn[1]);
    }
  };

  // prologue: tiles 0, 1, 2 requested; 0 and 1 landed
  issue_tile(0);
  issue_tile(1);
  issue_tile(2);
  if (ntiles > 2)
    __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * L::BPW));
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);
  vmem_wait_all();  // (the Q loads)
  __syncthreads();

  f32x16_t oacc[2][DB];
  float m[2], l[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[j][i] = f32x16_t{0};
    m[j] = kNegInf;
    l[j] = 0.f;
  }
  f32x16_t sa[2], sb[2];
  gemm_s(0, sa);

  auto step = [&](int t, f32x16_t (&sc)[2], f32x16_t (&sn)[2]) {
    const bool ahead = t + 3 < ntiles;
    if (ahead) issue_tile(t + 3);
    if (t < wtiles) {
      const int kv0 = t * kDLBN;
      const bool need_mask = (kv0 + kDLBN > N_kv) || (CAUSAL && kv0 + kDLBN - 1 > q0 + off);
      if (need_mask) {
        const int kvb = kv0 + 4 * lh;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kv = kvb + 8 * (r >> 2) + (r & 3);
            sc[j][r] = (kv < lim[j]) ? sc[j][r] : kNegInf;
          }
      }
      float nm[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float mx = max3(sc[j][0], sc[j][1], sc[j][2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) mx = max3(mx, sc[j][r], sc[j][r + 1]);
        mx = fmaxf(mx, sc[j][15]);
        const float mxs = half_max(mx) * scale_log2;
        const bool need = mxs > m[j] + kLazyRescale;
        if (wave_any(need)) {
          const float alpha = need ? ((m[j] == kNegInf) ? 0.f : fast_exp2(m[j] - mxs)) : 1.f;
          m[j] = need ? mxs : m[j];
          l[j] *= alpha;
#pragma unroll
          for (int i = 0; i < DB; ++i) oacc[j][i] *= alpha;
        }
        nm[j] = (m[j] == kNegInf) ? 0.f : -m[j];
      }
      // S(t+1) on the matrix cores while P(t) is formed
      gemm_s(t + 1, sn);
      uint32_t pk[2][8];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(__builtin_fmaf(sc[j][r], scale_log2, nm[j]));
          const float p1 = fast_exp2(__builtin_fmaf(sc[j][r + 1], scale_log2, nm[j]));
          l[j] += p0 + p1;
          pk[j][r >> 1] = TT::pack2(p0, p1);
        }
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // K operand read
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two score MFMAs
        __builtin_amdgcn_sched_group_barrier(0x002, 80 / KS, 0);  // exp / convert / sum
      }
      // O += V(t) P(t): each transposed V operand feeds both query blocks
      const uint8_t* base = smem + (t & (kW2Stages - 1)) * L::STAGE;
#pragma unroll
      for (int t4 = 0; t4 < 2; ++t4) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x2_t lo = lds_read_tr16((const uint16_t*)(base + va[db] + 16 * t4 * L::RB));
          const u32x2_t hi = lds_read_tr16((const uint16_t*)(base + va[db] + (16 * t4 + 8) * L::RB));
          const u32x4_t aop = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const u32x4_t bop = {pk[j][4 * t4 + 0], pk[j][4 * t4 + 1], pk[j][4 * t4 + 2], pk[j][4 * t4 + 3]};
            oacc[j][db] = TT::mfma32(aop, bop, oacc[j][db]);
          }
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 2 * DB - 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    // tile t+2 must have landed (only tile t+3's loads may still be pending)
    if (ahead)
      __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * L::BPW));
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, sa, sb);
    if (t + 1 < ntiles) step(t + 1, sb, sa);
  }

  const auto rO = buffer_rsrc(O + ((int64_t)b * H_q + h) * (int64_t)N_q * D, head_q_bytes);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
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

constexpr int kRingStages = 3;

// Workgroup barrier for LDS hand-offs: this wavefront's LDS operations have
// completed, and the compiler moves no memory access across it. Unlike
// __syncthreads() it does not wait for outstanding global loads (a workgroup
// release would, since direct-to-LDS loads count as LDS stores): each step
// waits for exactly the loads it needs before calling it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Ring form of the default kernel. K and V tiles travel HBM -> LDS through
// buffer loads that write LDS themselves (no staging registers and no LDS store
// instructions) into a ring of three stages. The tiles of all the workgroup's
// work items form one stream: while stream tile g is worked, the loads of tile
// g+2 are issued, into the stage that tile g-1 used, so each tile has a whole
// tile's time to arrive. They are issued after tile g's V operands have been
// read: the compiler makes a transposing LDS read wait for every direct load in
// flight, and at that point only tile g+1's loads are, which are due anyway.
// LDS rows are unpadded, their 16-byte chunks XOR-swizzled as in the
// direct-load form. One 32-row query block per wavefront; otherwise (work
// items, masking, causal skipping, the online softmax) as the default kernel.
template <class TT, int D, bool CAUSAL, int NW, bool PERSIST>
__global__ __launch_bounds__(64 * NW, (NW == 8 ? 1 : Occ<1, D>::kWaves)) void prefill16_ring_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int H_q, int H_kv, int N_q, int N_kv,
    float scale_log2, int nqb, int nbatch, const int* __restrict__ kv_lens = nullptr,
    int row_period = 0) {
  using L = DL<D, kBN>;
  constexpr int KS = D / 16;   // k-steps of the score MFMA
  constexpr int DB = D / 32;   // 32-wide blocks of the output
  constexpr int BM = NW * 32;  // query rows per workgroup
  constexpr int BPW = L::BLK / NW;  // 1 KB load blocks per wavefront, per tensor tile
  static_assert(BPW >= 1 && BPW * NW == L::BLK, "tile loads must split over the wavefronts");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kRingStages * L::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const uint32_t head_q_bytes = (uint32_t)N_q * D * 2;

  // work item r of this workgroup: as in the default kernel (a single item, or
  // the zig-zag walk of a persistent slot over its XCD's range)
  auto item_at = [&](int r, WorkItem& w) -> bool {
    if constexpr (!PERSIST) {
      if (r > 0) return false;
      w = map_work(nqb, H_q, nbatch, CAUSAL);
      return w.valid;
    } else {
      const int total = nqb * H_q * nbatch;
      const int per_xcd = (total + 7) >> 3;
      const int nslots = (int)gridDim.x >> 3, slot = (int)blockIdx.x >> 3;
      const int it = r * nslots + ((r & 1) ? (nslots - 1 - slot) : slot);
      const int item = (int)(blockIdx.x & 7) * per_xcd + it;
      if (it >= per_xcd || item >= total) return false;
      const int unit = item / nqb;
      const int qi = item - unit * nqb;
      w.valid = 1;
      w.qblk = CAUSAL ? (nqb - 1 - qi) : qi;
      w.b = unit / H_q;
      w.h = unit - w.b * H_q;
      return true;
    }
  };
  // keys of the item's request, and the K/V tiles the item works
  auto item_len = [&](const WorkItem& wi) {
    return kv_lens ? min(max(kv_lens[wi.b], 0), N_kv) : N_kv;
  };
  auto item_tiles = [&](const WorkItem& wi, int len) {
    int kv_end = len;
    if (CAUSAL && row_period == 0) {
      const int qlast = min(wi.qblk * BM + BM - 1, N_q - 1);
      kv_end = min(len, qlast + (len - N_q) + 1);
    }
    return kv_end > 0 ? (kv_end + kBN - 1) / kBN : 0;
  };
  auto kv_rsrc = [&](const uint16_t* base, const WorkItem& wi, int len) {
    const int hk = wi.h / (H_q / H_kv);
    return buffer_rsrc(base + ((int64_t)wi.b * H_kv + hk) * (int64_t)N_kv * D, (uint32_t)len * D * 2);
  };

  struct Ctx {
    __amdgpu_buffer_rsrc_t rQ;
    int b, h, ntiles;
    int lo_lim, hi_lim;  // least and greatest key limit over the wavefront's rows
    int qrow, lim;       // this lane's query row; keys below lim are visible to it
  };
  auto ctx_of = [&](const WorkItem& wi) {
    Ctx c;
    c.b = wi.b;
    c.h = wi.h;
    const int len = item_len(wi);
    const int ntok = row_period > 0 ? row_period : N_q;  // query tokens per head
    const int off = len - ntok;                          // bottom-right causal alignment
    c.rQ = buffer_rsrc(Q + ((int64_t)wi.b * H_q + wi.h) * (int64_t)N_q * D, head_q_bytes);
    c.qrow = wi.qblk * BM + wave * 32 + lr;
    const int tok = row_period > 0 ? c.qrow % row_period : c.qrow;
    c.lim = CAUSAL ? min(len, max(tok + off + 1, 0)) : len;
    int lo = c.lim, hi = c.lim;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) {
      lo = min(lo, __shfl_xor(lo, o));
      hi = max(hi, __shfl_xor(hi, o));
    }
    c.lo_lim = __builtin_amdgcn_readfirstlane(lo);
    c.hi_lim = __builtin_amdgcn_readfirstlane(hi);
    c.ntiles = item_tiles(wi, len);
    return c;
  };

  // Q^T operand: lane holds row qrow, d = 16*s + 8*lh + 0..7 (rows past N_q read as 0)
  u32x4_t qreg[KS];
  auto load_q = [&](const Ctx& c) {
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qreg[s] = buffer_load16(c.rQ, (uint32_t)(c.qrow * D + 16 * s + 8 * lh) * 2);
  };

  // ---- the producer: direct loads of the stream's tiles, two ahead of the
  // tile being worked. Block i of this wavefront fills LDS bytes
  // [(wave*BPW + i) KB, +1 KB) of the tensor tile, lane j writing physical chunk
  // p = 64*(wave*BPW + i) + j, which holds row p / CPR, logical chunk
  // (p % CPR) ^ swizzle(row).
  uint32_t kg_off[BPW], vg_off[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int p = (wave * BPW + i) * 64 + lane;
    const int r = p / L::CPR, slot = p % L::CPR;
    kg_off[i] = (uint32_t)(r * L::RB + ((slot ^ L::kswz(r)) * 16));
    vg_off[i] = (uint32_t)(r * L::RB + ((slot ^ L::vswz(r)) * 16));
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  WorkItem pw;
  int p_round = 0, p_t = 0, p_n = 0, p_stage = 0;
  bool p_more = item_at(0, pw);
  __amdgpu_buffer_rsrc_t pK, pV;
  auto p_open = [&]() {  // the producer's current item
    const int len = item_len(pw);
    pK = kv_rsrc(K, pw, len);
    pV = kv_rsrc(V, pw, len);
    p_n = item_tiles(pw, len);
    p_t = 0;
  };
  auto p_seek = [&]() {  // skip past exhausted items (and items without keys)
    while (p_more && p_t >= p_n) {
      p_more = item_at(++p_round, pw);
      if (p_more) p_open();
    }
  };
  if (p_more) p_open();
  p_seek();
  auto produce = [&]() -> bool {
    if (!p_more) return false;
    const uint32_t g0 = (uint32_t)(p_t * kBN) * L::RB;
    const uint32_t sb = lds0 + p_stage * L::STAGE;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const uint32_t kd = sb + (wave * BPW + i) * 1024;
      dma_load16(pK, g0 + kg_off[i], kd);
      dma_load16(pV, g0 + vg_off[i], kd + L::TILE);
    }
    p_stage = (p_stage == kRingStages - 1) ? 0 : p_stage + 1;
    ++p_t;
    p_seek();
    return true;
  };

  // operand addresses within a stage (bytes)
  //   K (score A operand): row lr (+32 for the second key block), logical chunk 2*st + lh
  //   V (transposing read): row 4*(g/2) + gi/4 (+16*t4, +8), logical chunk
  //     4*db + 2*(g%2) + (gi%4)/2, 8-byte half gi%2 (g = lane/16, gi = lane%16)
  int ka[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) ka[st] = lr * L::RB + (((2 * st + lh) ^ L::kswz(lr)) * 16);
  const int g = lane >> 4, gi = lane & 15;
  const int vrow = 4 * (g >> 1) + (gi >> 2);  // the swizzle only sees vrow % 4 (or % 8)
  int va[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    va[db] = L::TILE + vrow * L::RB + (((4 * db + 2 * (g & 1) + ((gi & 3) >> 1)) ^ L::vswz(vrow)) * 16) +
             8 * (gi & 1);

  WorkItem cur;
  if (!item_at(0, cur)) return;
  Ctx c = ctx_of(cur);
  int c_round = 0;
  produce();
  produce();
  load_q(c);
  vmem_wait_all();
  __syncthreads();
  int stage = 0;  // stage of the stream tile being worked

  for (;;) {
    WorkItem nwi = cur;  // (with no next item, nwi stays the current one, unused)
    const bool has_next = item_at(c_round + 1, nwi);
    const Ctx cn = ctx_of(nwi);

    f32x16_t oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[i] = f32x16_t{0};
    float m = kNegInf;  // reference maximum, in units of log2 (scores * scale * log2 e)
    float l = 0.f;      // this half-wave's part of the denominator
    const int ntiles = c.ntiles;

    for (int t = 0; t < ntiles; ++t) {
      const bool last = t + 1 == ntiles;
      const uint8_t* sb = smem + stage * L::STAGE;
      const int kv0 = t * kBN;
      // wavefront-uniform: does this tile hold any key visible to this wavefront?
      const bool live = kv0 < c.hi_lim;
      f32x16_t s0, s1;
      u32x4_t vop[4][DB];
      if (live) {
        // ---- S^T = K Q^T: two 32-key blocks
        s0 = s1 = f32x16_t{0};
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          const u32x4_t a0 = *(const u32x4_t*)(sb + ka[st]);
          const u32x4_t a1 = *(const u32x4_t*)(sb + ka[st] + 32 * L::RB);
          s0 = TT::mfma32(a0, qreg[st], s0);
          s1 = TT::mfma32(a1, qreg[st], s1);
        }
        // keep the K operand reads two k-steps ahead of the MFMAs that use them
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int st = 0; st < KS - 2; ++st) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        // V^T operands of this tile, requested now so that the score MFMAs, the
        // row max and the exponentials cover their LDS latency
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const u32x2_t lo = lds_read_tr16((const uint16_t*)(sb + va[db] + 16 * t4 * L::RB));
            const u32x2_t hi = lds_read_tr16((const uint16_t*)(sb + va[db] + (16 * t4 + 8) * L::RB));
            vop[t4][db] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
          }
      }
      const bool issued = produce();
      if (live) {
        // ---- mask (tail and causal diagonal tiles only), branch-free per element
        if (kv0 + kBN > c.lo_lim) {
          // key kv0 + 4*lh + e (e a per-register constant) is visible iff e < rel
          const int rel = c.lim - (kv0 + 4 * lh);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int e = 8 * (r >> 2) + (r & 3);
            s0[r] = (e < rel) ? s0[r] : kNegInf;
            s1[r] = (e + 32 < rel) ? s1[r] : kNegInf;
          }
        }
        // ---- row max of the raw scores (scale > 0 commutes with max)
        float mx = max3(s0[0], s0[1], s1[0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = max3(mx, s0[r], s1[r]);
        mx = fmaxf(mx, s1[0]);
        const float mxs = half_max(mx) * scale_log2;
        // wavefront-uniform branch; each lane moves only its own reference
        const bool need = mxs > m + kLazyRescale;
        if (wave_any(need)) {
          const float alpha = need ? ((m == kNegInf) ? 0.f : fast_exp2(m - mxs)) : 1.f;
          m = need ? mxs : m;
          l *= alpha;
#pragma unroll
          for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
        }
        const float nm = (m == kNegInf) ? 0.f : -m;
        // ---- P = exp2(S * scale*log2e - m), packed to 16-bit as the B operand
        uint32_t pk[16];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(__builtin_fmaf(s0[r], scale_log2, nm));
          const float p1 = fast_exp2(__builtin_fmaf(s0[r + 1], scale_log2, nm));
          const float p2 = fast_exp2(__builtin_fmaf(s1[r], scale_log2, nm));
          const float p3 = fast_exp2(__builtin_fmaf(s1[r + 1], scale_log2, nm));
          l += (p0 + p1) + (p2 + p3);
          pk[r >> 1] = TT::pack2(p0, p1);
          pk[8 + (r >> 1)] = TT::pack2(p2, p3);
        }
        // ---- O^T += V^T P^T, four 16-key steps
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          const u32x4_t bop = {pk[4 * t4 + 0], pk[4 * t4 + 1], pk[4 * t4 + 2], pk[4 * t4 + 3]};
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db] = TT::mfma32(vop[t4][db], bop, oacc[db]);
        }
      }
      const bool q_next = last && has_next;
      if (q_next) load_q(cn);  // this item's Q is no longer read
      // stream tile g+1 must have landed before the barrier; the loads issued
      // after it (tile g+2's, the next item's Q) may stay in flight
      if (issued) {
        if (q_next)
          __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * BPW + KS));
        else
          __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * BPW));
      } else {
        if (q_next)
          __builtin_amdgcn_s_waitcnt(0x0F70 | KS);
        else
          vmem_wait_all();
      }
      lds_barrier();
      stage = (stage == kRingStages - 1) ? 0 : stage + 1;
    }

    // ---- epilogue: combine half-wave denominators, normalise, store (rows past N_q dropped)
    const auto rO = buffer_rsrc(O + ((int64_t)c.b * H_q + c.h) * (int64_t)N_q * D, head_q_bytes);
    const float lt = half_sum(l);
    const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d = db * 32 + 8 * rg + 4 * lh;
        const u32x2_t w = {TT::pack2(oacc[db][4 * rg + 0] * inv, oacc[db][4 * rg + 1] * inv),
                           TT::pack2(oacc[db][4 * rg + 2] * inv, oacc[db][4 * rg + 3] * inv)};
        buffer_store8(rO, (uint32_t)(c.qrow * D + d) * 2, w);
      }
    }
    if (LSE != nullptr && lh == 0 && c.qrow < N_q) {
      LSE[((int64_t)c.b * H_q + c.h) * N_q + c.qrow] = (lt > 0.f) ? (m + log2f(lt)) * kLn2 : kNegInf;
    }
    if (!has_next) break;
    if (ntiles == 0) load_q(cn);  // (no tile step loaded it)
    ++c_round;
    cur = nwi;
    c = ctx_of(cur);
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

// Persistent launch of the default kernel: one workgroup per resident slot
// (occupancy from the runtime, times the compute units), at most one per item.
// With fewer than four items per slot the static zig-zag cannot balance
// causal items of very different lengths, and the hardware's dynamic dispatch
// of one item per workgroup does better; the persistent grid is used above that.
// Which form of the default kernel runs: the ring form for d = 64, the
// register-staged form for d = 128 (measured on the two shapes' workloads; at
// d = 128 the two are within noise of each other).
template <int D> constexpr bool kRingDefault = (D == 64);

template <class TT, int D, bool CAUSAL, int NW, bool PERSIST, bool RING>
constexpr auto prefill16_form() {
  if constexpr (RING)
    return prefill16_ring_kernel<TT, D, CAUSAL, NW, PERSIST>;
  else
    return prefill16_kernel<TT, D, CAUSAL, 1, NW, PERSIST>;
}

template <class TT, int D, int NW, bool CAUSAL, bool RING>
hipError_t launch16pers_t(const PrefillArgs& a, hipStream_t st, int nqb, const int* kv_lens = nullptr,
                          int row_period = 0) {
  static int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill16_form<TT, D, CAUSAL, NW, true, RING>(),
                                                     64 * NW, 0) != hipSuccess || n < 1)
      n = 1;
    per_cu = n;
  }
  const int64_t items = (int64_t)nqb * a.H_q * a.B;
  int64_t slots = (int64_t)per_cu * (a.num_cus > 0 ? a.num_cus : 256);
  // tuning and testing: ATTN_PREFILL_SLOTS = n forces the persistent grid with n slots
  const char* env = getenv("ATTN_PREFILL_SLOTS");
  const int64_t forced = env ? atol(env) : 0;
  if (forced > 0) slots = forced < slots ? forced : slots;
  const float sl2 = a.scale * kLog2e;
  if (forced <= 0 && items < 4 * slots) {
    hipLaunchKernelGGL((prefill16_form<TT, D, CAUSAL, NW, false, RING>()), dim3(xcd_grid(items)),
                       dim3(64 * NW), 0, st, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, a.H_q, a.H_kv, a.N_q, a.N_kv, sl2,
                       nqb, a.B, kv_lens, row_period);
  } else {
    hipLaunchKernelGGL((prefill16_form<TT, D, CAUSAL, NW, true, RING>()), dim3(xcd_grid(slots)),
                       dim3(64 * NW), 0, st, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, a.H_q, a.H_kv, a.N_q, a.N_kv, sl2,
                       nqb, a.B, kv_lens, row_period);
  }
  return hipGetLastError();
}

template <class TT, int D, int NW, bool RING = false>
hipError_t launch16pers(const PrefillArgs& a, hipStream_t st, const int* kv_lens = nullptr,
                        int row_period = 0) {
  const int nqb = (a.N_q + NW * 32 - 1) / (NW * 32);
  return a.causal ? launch16pers_t<TT, D, NW, true, RING>(a, st, nqb, kv_lens, row_period)
                  : launch16pers_t<TT, D, NW, false, RING>(a, st, nqb, kv_lens, row_period);
}

template <class TT, int D, int QB, int NW = 4>
hipError_t launch16q(const PrefillArgs& a, hipStream_t st) {
  constexpr int BM = NW * 32 * QB;
  const int nqb = (a.N_q + BM - 1) / BM;
  dim3 grid(xcd_grid((int64_t)nqb * a.H_q * a.B));
  const float sl2 = a.scale * kLog2e;
  auto q = (const uint16_t*)a.q;
  auto k = (const uint16_t*)a.k;
  auto v = (const uint16_t*)a.v;
  auto o = (uint16_t*)a.o;
  if (a.causal)
    hipLaunchKernelGGL((prefill16_kernel<TT, D, true, QB, NW>), grid, dim3(64 * NW), 0, st, q, k, v,
                       o, a.lse, a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, nqb, a.B);
  else
    hipLaunchKernelGGL((prefill16_kernel<TT, D, false, QB, NW>), grid, dim3(64 * NW), 0, st, q, k, v,
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

template <class TT, int D>
hipError_t launch16pp(const PrefillArgs& a, hipStream_t st) {
  const int nqb = (a.N_q + kPPBM - 1) / kPPBM;
  dim3 grid(xcd_grid((int64_t)nqb * a.H_q * a.B));
  const float sl2 = a.scale * kLog2e;
  auto q = (const uint16_t*)a.q;
  auto k = (const uint16_t*)a.k;
  auto v = (const uint16_t*)a.v;
  auto o = (uint16_t*)a.o;
  if (a.causal)
    hipLaunchKernelGGL((prefill16_pp_kernel<TT, D, true, (D == 64)>), grid, dim3(kPPThreads), 0, st, q, k, v,
                       o, a.lse, a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, nqb, a.B);
  else
    hipLaunchKernelGGL((prefill16_pp_kernel<TT, D, false, (D == 64)>), grid, dim3(kPPThreads), 0, st, q, k, v,
                       o, a.lse, a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, nqb, a.B);
  return hipGetLastError();
}

template <class TT, int D>
hipError_t launch16dl(const PrefillArgs& a, hipStream_t st) {
  const int nqb = (a.N_q + kBM - 1) / kBM;
  dim3 grid(xcd_grid((int64_t)nqb * a.H_q * a.B));
  const float sl2 = a.scale * kLog2e;
  auto q = (const uint16_t*)a.q;
  auto k = (const uint16_t*)a.k;
  auto v = (const uint16_t*)a.v;
  auto o = (uint16_t*)a.o;
  if (a.causal)
    hipLaunchKernelGGL((prefill16_dl_kernel<TT, D, true>), grid, dim3(kThreads), 0, st, q, k, v, o,
                       a.lse, a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, nqb, a.B);
  else
    hipLaunchKernelGGL((prefill16_dl_kernel<TT, D, false>), grid, dim3(kThreads), 0, st, q, k, v, o,
                       a.lse, a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, nqb, a.B);
  return hipGetLastError();
}

template <class TT, int D>
hipError_t launch16w2(const PrefillArgs& a, hipStream_t st) {
  const int nqb = (a.N_q + kW2BM - 1) / kW2BM;
  dim3 grid(xcd_grid((int64_t)nqb * a.H_q * a.B));
  const float sl2 = a.scale * kLog2e;
  auto q = (const uint16_t*)a.q;
  auto k = (const uint16_t*)a.k;
  auto v = (const uint16_t*)a.v;
  auto o = (uint16_t*)a.o;
  if (a.causal)
    hipLaunchKernelGGL((prefill16_w2_kernel<TT, D, true>), grid, dim3(kThreads), 0, st, q, k, v, o,
                       a.lse, a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, nqb, a.B);
  else
    hipLaunchKernelGGL((prefill16_w2_kernel<TT, D, false>), grid, dim3(kThreads), 0, st, q, k, v, o,
                       a.lse, a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, nqb, a.B);
  return hipGetLastError();
}

// Kernel form for 16-bit inputs: one 32-row query block per wavefront, 8
// wavefronts (256 rows) per workgroup for d = 128 and 4 (128 rows) for d = 64,
// where the smaller register footprint buys a third resident wavefront per
// SIMD instead. ATTN_PREFILL_VARIANT selects alternative forms (tuning only):
// 1 = 4 wavefronts, 2 = two query blocks per wavefront, 3 = software-pipelined
// scores, 4 = two ping-ponging wavefront groups, 5 = direct-load 3-stage ring,
// 6 = two query blocks with a direct-load ring, 7 = 8 wavefronts, 8 = the
// default kernel with one work item per workgroup instead of a persistent grid,
// 9 = two wavefront groups skewed by half a tile, 10 = the default kernel's ring
// form (direct loads), 11 = its register-staged form.
template <class TT, int D>
hipError_t launch16skew(const PrefillArgs& a, hipStream_t st) {
  const int nqb = (a.N_q + 255) / 256;
  dim3 grid(xcd_grid((int64_t)nqb * a.H_q * a.B));
  const float sl2 = a.scale * kLog2e;
  auto q = (const uint16_t*)a.q;
  auto k = (const uint16_t*)a.k;
  auto v = (const uint16_t*)a.v;
  auto o = (uint16_t*)a.o;
  if (a.causal)
    hipLaunchKernelGGL((prefill16_skew_kernel<TT, D, true>), grid, dim3(512), 0, st, q, k, v, o, a.lse,
                       a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, nqb, a.B);
  else
    hipLaunchKernelGGL((prefill16_skew_kernel<TT, D, false>), grid, dim3(512), 0, st, q, k, v, o, a.lse,
                       a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, nqb, a.B);
  return hipGetLastError();
}

template <class TT, int D>
hipError_t launch16(const PrefillArgs& a, hipStream_t st) {
  const char* env = getenv("ATTN_PREFILL_VARIANT");
  const int variant = env ? atoi(env) : 0;
  if (variant == 2) return launch16q<TT, D, 2>(a, st);
  if (variant == 3) return launch16p<TT, D>(a, st);
  if (variant == 4) return launch16pp<TT, D>(a, st);
  if (variant == 5) return launch16dl<TT, D>(a, st);
  if (variant == 1) return launch16q<TT, D, 1, 4>(a, st);
  if (variant == 6) return launch16w2<TT, D>(a, st);
  if (variant == 7) return launch16q<TT, D, 1, 8>(a, st);
  if (variant == 8) return launch16q<TT, D, 1, (D == 128 ? 8 : 4)>(a, st);
  if (variant == 9) return launch16skew<TT, D>(a, st);
  if (variant == 10) return launch16pers<TT, D, (D == 128 ? 8 : 4), true>(a, st);
  if (variant == 11) return launch16pers<TT, D, (D == 128 ? 8 : 4), false>(a, st);
  return launch16pers<TT, D, (D == 128 ? 8 : 4), kRingDefault<D>>(a, st);
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

// The default kernel in rows mode (multi-token decode against per-request
// lengths; see prefill16_kernel).
hipError_t launch_prefill_rows(const PrefillArgs& a, const int* kv_lens, int row_period,
                               hipStream_t st) {
  const char* env = getenv("ATTN_PREFILL_VARIANT");
  const int variant = env ? atoi(env) : 0;
  if (variant == 10 || variant == 11) {  // tuning and testing: force the ring or the staged form
    const bool ring = variant == 10;
    if (a.dtype == kDtypeBF16)
      return a.d == 64 ? (ring ? launch16pers<BF16, 64, 4, true>(a, st, kv_lens, row_period)
                               : launch16pers<BF16, 64, 4, false>(a, st, kv_lens, row_period))
                       : (ring ? launch16pers<BF16, 128, 8, true>(a, st, kv_lens, row_period)
                               : launch16pers<BF16, 128, 8, false>(a, st, kv_lens, row_period));
    return a.d == 64 ? (ring ? launch16pers<F16, 64, 4, true>(a, st, kv_lens, row_period)
                             : launch16pers<F16, 64, 4, false>(a, st, kv_lens, row_period))
                     : (ring ? launch16pers<F16, 128, 8, true>(a, st, kv_lens, row_period)
                             : launch16pers<F16, 128, 8, false>(a, st, kv_lens, row_period));
  }
  if (a.dtype == kDtypeBF16)
    return a.d == 64 ? launch16pers<BF16, 64, 4, kRingDefault<64>>(a, st, kv_lens, row_period)
                     : launch16pers<BF16, 128, 8, kRingDefault<128>>(a, st, kv_lens, row_period);
  return a.d == 64 ? launch16pers<F16, 64, 4, kRingDefault<64>>(a, st, kv_lens, row_period)
                   : launch16pers<F16, 128, 8, kRingDefault<128>>(a, st, kv_lens, row_period);
}

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
