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
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr int kBN = 64;        // keys per tile
constexpr int kBM = 128;       // fp32 kernel: query rows per workgroup (4 wavefronts x 32)
constexpr int kThreads = 256;  // fp32 kernel: threads per workgroup

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
// a block's probabilities against it could exceed 2^kLazyRescale (see
// softmax_tile), so most blocks skip the rescale of l and u. Probabilities then
// stay below 2^8, and l and u keep one common reference point, so u / l is
// unchanged.
constexpr float kLazyRescale = 8.f;
constexpr float kLazySum = 256.f;  // 2^kLazyRescale

// One 64-key tile of the online softmax for one lane's row (32 of its 64
// scores in s0, s1; lane i + 32 holds the other 32): P = exp2(S * scale*log2e
// - m), rounded to 16 bits as the PV operand, and l and the output
// accumulators rescaled when the reference moves. The exponentials are first
// taken against the current reference m, without the tile's row maximum: if
// both halves of the row sum to at most 2^kLazyRescale, each is at most that,
// which is all the lazy rescale rule asks, and they stand. Otherwise (and
// while m is still -inf) the row raises m to the tile's maximum if that is
// higher, rescales, and takes them again. The second pass is a
// wavefront-uniform branch, but a row whose first pass stood keeps its
// reference and recomputes the same values in the same order, so a row's
// result never depends on the other rows of the wavefront.
template <class TT, int DB>
__device__ __forceinline__ void softmax_tile(const f32x16_t& s0, const f32x16_t& s1, float scale_log2,
                                             float& m, float& nm, float& l, f32x16_t (&oacc)[DB],
                                             uint32_t (&pk)[16]) {
  auto exps = [&]() {
    float ts = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = fast_exp2(__builtin_fmaf(s0[r], scale_log2, nm));
      const float p1 = fast_exp2(__builtin_fmaf(s0[r + 1], scale_log2, nm));
      const float p2 = fast_exp2(__builtin_fmaf(s1[r], scale_log2, nm));
      const float p3 = fast_exp2(__builtin_fmaf(s1[r + 1], scale_log2, nm));
      ts += (p0 + p1) + (p2 + p3);
      pk[r >> 1] = TT::pack2(p0, p1);
      pk[8 + (r >> 1)] = TT::pack2(p2, p3);
    }
    return ts;
  };
  float ts = exps();
  // A lane fails when its 32 sum to more than 2^kLazyRescale (inf and NaN
  // included) or m is still -inf. Lanes i and i + 32 hold the same row and
  // reference and must take the same decision: a row fails if either fails
  // (the exchange is on the scalar ballot mask).
  const bool lane_fail = !(ts <= kLazySum) || m == kNegInf;
  if (wave_any(lane_fail)) {
    const uint64_t fail = __ballot(lane_fail);
    const uint64_t row_fail = fail | (fail >> 32) | (fail << 32);
    const bool ok = ((row_fail >> __lane_id()) & 1) == 0;
    // ---- row max of the raw scores (scale > 0 commutes with max)
    float mx = vmax(s0[0], s1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = max3(mx, s0[r], s1[r]);
    const float mxs = half_max(mx) * scale_log2;
    const bool need = !ok && mxs > m;
    if (wave_any(need)) {
      const float alpha = need ? ((m == kNegInf) ? 0.f : fast_exp2(m - mxs)) : 1.f;
      m = need ? mxs : m;
      nm = (m == kNegInf) ? 0.f : -m;
      l *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
    }
    ts = exps();
  }
  l += ts;
}

// QB query blocks of 32 rows per wavefront (NW * 32 * QB rows per
// workgroup). Each K or V operand read from LDS feeds QB MFMAs, so QB = 2
// halves the LDS bytes per FLOP at the price of twice the registers (a tuning
// alternative only: at d = 128 it spills).
// Workgroup -> (batch, head, query block), in the work order of grid_item
// (query block 0 in that order is the one with the most keys under a causal
// mask). The persistent grids below use their own order.
struct WorkItem {
  int b, h, qblk;
  int valid;  // an int, not a bool: no padding bytes for a struct copy to move
};
__device__ __forceinline__ WorkItem map_work(int nqb, int H_q, int B, bool longest_first) {
  const GridItem g = grid_item(nqb, H_q * B);
  WorkItem w;
  w.valid = g.valid;
  w.qblk = longest_first ? (nqb - 1 - g.blk) : g.blk;
  w.b = g.unit / H_q;
  w.h = g.unit - w.b * H_q;
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
  // holds as many workgroups as can be resident. Items, numbered head-major
  // with the longest query block of a head first, are cut into 8 contiguous
  // ranges, and the slots of XCD x (workgroup ids x, x+8, ...) walk range x, so
  // a head's query blocks, and heads sharing a KV head, run on one XCD and
  // reuse its L2. Slot s of an XCD takes items s, then 2*nslots - 1 - s, then
  // 2*nslots + s, ...: a zig-zag, so that with causal masking every slot gets a
  // mix of long and short query blocks.
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
    float m[QB], l[QB], nm[QB];
#pragma unroll
    for (int j = 0; j < QB; ++j) {
#pragma unroll
      for (int i = 0; i < DB; ++i) oacc[j][i] = f32x16_t{0};
      m[j] = kNegInf;  // reference maximum, in units of log2 (scores * scale * log2 e)
      l[j] = 0.f;      // this half-wave's part of the denominator
      nm[j] = 0.f;     // the exponent offset: -m, or 0 while m is -inf
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
        // V^T operands of the first VE 16-key steps, requested now so that the
        // score MFMAs and the exponentials cover their LDS latency; the rest after
        // the exponentials (fewer registers live across them), covered by the
        // products of the first steps.
        constexpr int VE = (QB == 2) ? 4 : (NW == 8 && D == 128) ? 3 : 2;
        u32x4_t vop[4][DB];
        auto read_v = [&](int t4) {
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const u32x2_t lo = lds_read_tr16(tV + 16 * t4 * VST + db * 32);
            const u32x2_t hi = lds_read_tr16(tV + (16 * t4 + 8) * VST + db * 32);
            vop[t4][db] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
          }
        };
#pragma unroll
        for (int t4 = 0; t4 < VE; ++t4) read_v(t4);
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
        // ---- P = exp2(S * scale*log2e - m), packed to 16-bit as the B operand
        uint32_t pk[QB][16];
#pragma unroll
        for (int j = 0; j < QB; ++j)
          softmax_tile<TT, DB>(s[j][0], s[j][1], scale_log2, m[j], nm[j], l[j], oacc[j], pk[j]);
        if constexpr (VE < 4) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int t4 = VE; t4 < 4; ++t4) read_v(t4);
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

// LDS layout of the ring form: K and V tiles of 64 keys, rows unpadded, their
// 16-byte chunks XOR-swizzled so that both operand reads are conflict-free:
//   K: chunk c of row r sits at c ^ ((r / RPB) % CPR): the 16 rows read by one
//      16-lane slice of a score-MFMA operand fetch land on 16 distinct banks;
//   V: chunk c of row r sits at c ^ 4*((r / RPB) % (4 / RPB)): the 4 rows of a
//      transposing read land on distinct banks;
// (RPB rows per 256-byte bank sweep, CPR chunks per row). One direct load
// instruction fills 1 KB of LDS, lane j writing chunk j, so each lane fetches
// the logical chunk that its physical slot holds.
template <int D> struct RingLds {
  static constexpr int RB = D * 2;              // bytes per row
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int RPB = 256 / RB;          // rows per 256-byte bank sweep
  static constexpr int TILE = kBN * RB;         // bytes per tensor tile
  static constexpr int STAGE = 2 * TILE;        // K then V
  static constexpr int BLK = TILE / 1024;       // 1 KB load blocks per tensor tile
  static __device__ __forceinline__ int kswz(int r) { return (r / RPB) & (CPR - 1); }
  static __device__ __forceinline__ int vswz(int r) { return 4 * ((r / RPB) & (RPB == 1 ? 3 : 1)); }
};

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
// LDS rows are unpadded, their 16-byte chunks XOR-swizzled (RingLds). One
// 32-row query block per wavefront; otherwise (work
// items, masking, causal skipping, the online softmax) as the default kernel.
template <class TT, int D, bool CAUSAL, int NW, bool PERSIST>
__global__ __launch_bounds__(64 * NW, (NW == 8 ? 1 : Occ<1, D>::kWaves)) void prefill16_ring_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int H_q, int H_kv, int N_q, int N_kv,
    float scale_log2, int nqb, int nbatch, const int* __restrict__ kv_lens = nullptr,
    int row_period = 0) {
  using L = RingLds<D>;
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
    float nm = 0.f;     // the exponent offset: -m, or 0 while m is -inf
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
        // V^T operands of this tile, requested now so that the score MFMAs and
        // the exponentials cover their LDS latency
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
        // ---- P = exp2(S * scale*log2e - m), packed to 16-bit as the B operand
        uint32_t pk[16];
        softmax_tile<TT, DB>(s0, s1, scale_log2, m, nm, l, oacc, pk);
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

// Persistent launch of the default kernel: one workgroup per resident slot
// (occupancy from the runtime, times the compute units), at most one per item.
// With fewer than four items per slot the static zig-zag cannot balance
// causal items of very different lengths, and the hardware's dynamic dispatch
// of one item per workgroup does better; the persistent grid is used above that.
template <class TT, int D, int NW, bool CAUSAL, bool RING>
hipError_t launch16pers_t(const PrefillArgs& a, hipStream_t st, int nqb, const int* kv_lens,
                          int row_period) {
  constexpr auto kpers = prefill16_form<TT, D, CAUSAL, NW, true, RING>();
  constexpr auto kone = prefill16_form<TT, D, CAUSAL, NW, false, RING>();
  const int per_cu = occupancy_per_cu((const void*)kpers, 64 * NW, a.device);
  const int64_t items = (int64_t)nqb * a.H_q * a.B;
  int64_t slots = (int64_t)per_cu * (a.num_cus > 0 ? a.num_cus : 256);
  // tuning and testing: the prefill_slots knob forces the persistent grid with n slots
  const int64_t forced = tuning(kTunePrefillSlots);
  if (forced > 0) slots = forced < slots ? forced : slots;
  const float sl2 = a.scale * kLog2e;
  const bool pers = forced > 0 || items >= 4 * slots;
  return launch_kernel(pers ? kpers : kone, dim3(xcd_grid(pers ? slots : items)), dim3(64 * NW), st,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o,
                       a.lse, a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, nqb, a.B, kv_lens, row_period);
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
  const dim3 grid(xcd_grid((int64_t)nqb * a.H_q * a.B));
  const float sl2 = a.scale * kLog2e;
  const auto kern = a.causal ? prefill16_kernel<TT, D, true, QB, NW> : prefill16_kernel<TT, D, false, QB, NW>;
  return launch_kernel(kern, grid, dim3(64 * NW), st, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, nqb,
                       a.B, (const int*)nullptr, 0);
}

// Kernel form for 16-bit inputs: one 32-row query block per wavefront, 8
// wavefronts (256 rows) per workgroup for d = 128 and 4 (128 rows) for d = 64,
// where the smaller register footprint buys a third resident wavefront per
// SIMD instead. The prefill_variant knob selects alternative forms (tuning and
// testing only): 1 = 4 wavefronts per workgroup, one work item each; 2 = two
// query blocks per wavefront; 3 = the default wavefront count with one work
// item per workgroup instead of a persistent grid; 4 = the ring form (direct
// loads) at either d; 5 = the register-staged form at either d.
template <class TT, int D>
hipError_t launch16(const PrefillArgs& a, hipStream_t st) {
  constexpr int NW = (D == 128) ? 8 : 4;
  const int variant = tuning(kTunePrefillVariant);
  if (variant == 1) return launch16q<TT, D, 1, 4>(a, st);
  if (variant == 2) return launch16q<TT, D, 2>(a, st);
  if (variant == 3) return launch16q<TT, D, 1, NW>(a, st);
  if (variant == 4) return launch16pers<TT, D, NW, true>(a, st);
  if (variant == 5) return launch16pers<TT, D, NW, false>(a, st);
  return launch16pers<TT, D, NW, kRingDefault<D>>(a, st);
}

template <int D>
hipError_t launch32(const PrefillArgs& a, hipStream_t st) {
  const int nqb = (a.N_q + kBM - 1) / kBM;
  const dim3 grid(nqb, a.H_q, a.B);
  const float sl2 = a.scale * kLog2e;
  const auto kern = a.causal ? prefill32_kernel<D, true> : prefill32_kernel<D, false>;
  return launch_kernel(kern, grid, dim3(kThreads), st, (const float*)a.q, (const float*)a.k,
                       (const float*)a.v, (float*)a.o, a.lse, a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, nqb);
}

// Rows mode at either head dim: the ring or the staged form (the default form
// unless the prefill_variant knob is 4 or 5).
template <class TT, int D>
hipError_t launch_rows16(const PrefillArgs& a, const int* kv_lens, int row_period, hipStream_t st) {
  constexpr int NW = (D == 128) ? 8 : 4;
  const int variant = tuning(kTunePrefillVariant);
  const bool ring = variant == 4 ? true : variant == 5 ? false : kRingDefault<D>;
  return ring ? launch16pers<TT, D, NW, true>(a, st, kv_lens, row_period)
              : launch16pers<TT, D, NW, false>(a, st, kv_lens, row_period);
}

}  // namespace

// The default kernel in rows mode (multi-token decode against per-request
// lengths; see prefill16_kernel).
hipError_t launch_prefill_rows(const PrefillArgs& a, const int* kv_lens, int row_period,
                               hipStream_t st) {
  if (a.dtype == kDtypeBF16)
    return a.d == 64 ? launch_rows16<BF16, 64>(a, kv_lens, row_period, st)
                     : launch_rows16<BF16, 128>(a, kv_lens, row_period, st);
  return a.d == 64 ? launch_rows16<F16, 64>(a, kv_lens, row_period, st)
                   : launch_rows16<F16, 128>(a, kv_lens, row_period, st);
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
