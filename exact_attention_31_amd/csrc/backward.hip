// Backward pass of exact attention on gfx950, by recomputation.
//
// The forward pass keeps only O and the per-row log-sum-exp; the backward pass
// rebuilds each tile of the probabilities from Q, K and the stored statistics
// instead of reading a stored score matrix (marketmaker.cc, "Rückwärtsdurchlauf:
// Neu berechnen statt speichern"). With S = scale * Q K^T, P = exp(S - lse),
// and Delta_i = sum_d dO_id O_id (which equals sum_j P_ij dP_ij):
//   dV = P^T dO,   dP = dO V^T,   dS = P o (dP - Delta),
//   dQ = scale * dS K,   dK = scale * dS^T Q,
// dK and dV summed over the G query heads that share a KV head.
//
// Two kernels, no atomics (deterministic), the dQ kernel first:
//   bwd_dq_kernel     one workgroup per 256 query rows; each wavefront keeps
//                     its Q and dO rows in registers, forms Delta (from its O
//                     rows) and the log-sum-exp in log2 units for them, writes
//                     both for the dK/dV kernel, and accumulates dQ^T while
//                     K and V tiles stream through LDS;
//   bwd_dkdv_kernel   one workgroup per 256 keys of a KV head; each wavefront
//                     keeps 32 keys of K in registers (their V rows in LDS)
//                     and accumulates dK^T, dV^T while Q and dO tiles stream
//                     through LDS.
// Matrix-core layouts are those of the forward kernels (32x32x16 MFMA); the
// accumulators of S (dK/dV kernel) and S^T (dQ kernel) are fed back as B
// operands with the K-index permutation their layout implies, and the A
// operands that need a transposed tile come from ds_read_b64_tr_b16.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr int kBwdBM = 64;   // query rows per LDS tile (dK/dV kernel)
constexpr int kBwdBN = 64;   // keys per LDS tile (dQ kernel)
constexpr int kBwdNWK = 8;   // wavefronts per dK/dV workgroup (two per SIMD)
constexpr int kBwdKW = 32 * kBwdNWK;  // keys per dK/dV workgroup

template <int D> struct BwdLds {
  // row stride (elements) of LDS tiles read only row-wise (16-byte reads): rows
  // 4 (mod 64) dwords apart, so 16 consecutive rows cover the 64 banks once
  static constexpr int STR = D + 8;
};

// Placement of LDS tiles read both row-wise (16-byte reads, 16 lanes per LDS
// cycle) and by transposing 8-byte reads (32 lanes: 4 consecutive rows x 16
// dwords). Rows go in groups of four: IN elements apart within a group (an odd
// multiple of 16 dwords mod 64, so the 4 rows of a transposing read use
// disjoint banks) and GRP elements apart between groups (an odd multiple of 4
// dwords mod 64, which with the in-group step puts 16 consecutive rows on 16
// distinct 4-bank sets). A plain stride cannot do both: the two reads need it
// 16 * odd and 4 * odd (mod 64) dwords.
template <int D> struct BwdGrp {
  static constexpr int IN = (D == 128) ? 160 : 96;
  static constexpr int GRP = (D == 128) ? 616 : 360;
  static_assert(GRP >= 3 * IN + D, "rows of a group must not overlap");
  static constexpr int size(int rows) { return GRP * (rows / 4); }
  static __device__ __forceinline__ int row(int r) { return GRP * (r >> 2) + IN * (r & 3); }
};

// Workgroup -> (batch, head, block) in the work order of grid_item (block 0
// is the longest under a causal mask in both gradient kernels).
struct BwdItem {
  int b, h, blk;
  bool valid;
};
__device__ __forceinline__ BwdItem bwd_map(int nblk, int H, int B) {
  const GridItem g = grid_item(nblk, H * B);
  BwdItem w;
  w.valid = g.valid;
  w.blk = g.blk;
  w.b = g.unit / H;
  w.h = g.unit - w.b * H;
  return w;
}

// ---------------------------------------------------------------------------
// dK, dV. Workgroup: 256 keys [k0, k0+256) of KV head hk of batch b, eight
// wavefronts (two per SIMD); wavefront w owns keys kw = k0 + 32w .. kw + 31
// (lane: key kw + lane % 32 as the B operand column of S = Q K^T and
// dP = dO V^T). The K operands stay in registers; the V operands are read from
// an LDS copy of the workgroup's V rows, which keeps the register count at two
// wavefronts per SIMD. Query tiles of 64 rows of each of the G query heads
// stream through LDS (double-buffered, register-staged). Per 32-row subtile:
//   S  = Q K^T, dP = dO V^T           (A: Q, dO rows from LDS; B: K in registers, V from LDS)
//   P  = exp2(S * scale*log2e - lse2), dS = P o (dP - Delta)   (per element;
//                                      dP's accumulator starts from -Delta)
//   dV^T += dO^T P,  dK^T += Q^T dS   (A: dO^T, Q^T by transposing LDS reads;
//                                      B: P, dS straight from the accumulators)
template <class TT, int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kBwdNWK, 2) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ delta,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int H_q, int H_kv, int N_q, int N_kv,
    float scale_log2, float scale, int nkb, int nbatch) {
  constexpr int STR = BwdLds<D>::STR;
  constexpr int KS = D / 16;   // k-steps over the head dimension
  constexpr int DB = D / 32;   // 32-wide blocks of the head dimension
  constexpr int CPR = D / 8;   // 16-byte chunks per row
  constexpr int NT = 64 * kBwdNWK;
  constexpr int LPT = kBwdBM * CPR / NT;  // 16-byte loads per thread per tile, per tensor
  static_assert(LPT * NT == kBwdBM * CPR, "tile load must split evenly");
  using Gp = BwdGrp<D>;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2][Gp::size(kBwdBM)];
  __shared__ __attribute__((aligned(16))) uint16_t sG[2][Gp::size(kBwdBM)];
  __shared__ __attribute__((aligned(16))) float sL[2][kBwdBM];
  __shared__ __attribute__((aligned(16))) float sD[2][kBwdBM];
  __shared__ __attribute__((aligned(16))) uint16_t sVk[kBwdKW * STR];  // this workgroup's V rows

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const BwdItem wi = bwd_map(nkb, H_kv, nbatch);
  if (!wi.valid) return;
  const int b = wi.b, hk = wi.h;
  const int G = H_q / H_kv;
  const int k0 = wi.blk * kBwdKW;
  const int kw = k0 + 32 * wave;       // this wavefront's first key
  const int off = N_kv - N_q;          // bottom-right causal alignment

  const uint32_t head_q_bytes = (uint32_t)N_q * D * 2;
  const uint32_t head_kv_bytes = (uint32_t)N_kv * D * 2;
  const int64_t kv_head = ((int64_t)b * H_kv + hk) * (int64_t)N_kv * D;
  const auto rK = buffer_rsrc(K + kv_head, head_kv_bytes);
  const auto rV = buffer_rsrc(V + kv_head, head_kv_bytes);

  // K as B operands: lane holds key kw + lr, d = 16*st + 8*lh + 0..7
  u32x4_t kB[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st)
    kB[st] = buffer_load16(rK, (uint32_t)((kw + lr) * D + 16 * st + 8 * lh) * 2);
  // the workgroup's V rows into LDS (visible after the first barrier below);
  // the V operand of lane (key kw + lr, k-step st) is at vrow + 16*st
  {
    constexpr int VC = kBwdKW * CPR / NT;
    static_assert(VC * NT == kBwdKW * CPR, "V rows must split evenly");
#pragma unroll
    for (int i = 0; i < VC; ++i) {
      const int c = tid + NT * i;
      const u32x4_t x = buffer_load16(rV, (uint32_t)((k0 + c / CPR) * D + (c % CPR) * 8) * 2);
      *(u32x4_t*)(&sVk[(c / CPR) * STR + (c % CPR) * 8]) = x;
    }
  }
  const uint16_t* vrow = &sVk[(32 * wave + lr) * STR + 8 * lh];

  // query tiles: the G heads in turn, each from the first tile that sees key k0
  const int nqt = (N_q + kBwdBM - 1) / kBwdBM;
  const int qt0 = CAUSAL ? min(nqt, max(0, k0 - off) / kBwdBM) : 0;
  const int per_head = nqt - qt0;
  const int ntiles = G * per_head;

  uint32_t ld_off[LPT];
  int st_off[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int c = tid + NT * i;
    ld_off[i] = (uint32_t)((c / CPR) * D + (c % CPR) * 8) * 2;
    st_off[i] = Gp::row(c / CPR) + (c % CPR) * 8;
  }
  u32x4_t qbuf[LPT], gbuf[LPT];
  float lbuf = 0.f;
  auto load_tile = [&](int t) {
    const int hq = hk * G + t / per_head;
    const int q0 = (qt0 + t % per_head) * kBwdBM;
    const int64_t qh = ((int64_t)b * H_q + hq) * (int64_t)N_q;
    const auto rQ = buffer_rsrc(Q + qh * D, head_q_bytes);
    const auto rG = buffer_rsrc(dO + qh * D, head_q_bytes);
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      qbuf[i] = buffer_load16(rQ, (uint32_t)q0 * D * 2 + ld_off[i]);
      gbuf[i] = buffer_load16(rG, (uint32_t)q0 * D * 2 + ld_off[i]);
    }
    // threads 0..63: lse2 of row q0 + tid; 64..127: Delta (rows past N_q: P = 0)
    if (tid < 2 * kBwdBM) {
      const int r = q0 + (tid & (kBwdBM - 1));
      const bool in = r < N_q;
      if (tid < kBwdBM) lbuf = in ? lse2[qh + r] : __builtin_inff();
      else lbuf = in ? -delta[qh + r] : 0.f;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      *(u32x4_t*)(&sQ[buf][st_off[i]]) = qbuf[i];
      *(u32x4_t*)(&sG[buf][st_off[i]]) = gbuf[i];
    }
    if (tid < kBwdBM) sL[buf][tid] = lbuf;
    else if (tid < 2 * kBwdBM) sD[buf][tid - kBwdBM] = lbuf;
  };

  f32x16_t dvT[DB], dkT[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dvT[i] = dkT[i] = f32x16_t{0};

  // per-lane LDS offsets: A rows (lane's row lr, columns 16*st + 8*lh) and the
  // transposing read (lane i of 16-lane group g: row 4*(g/2) + i/4, columns
  // 16*(g%2) + 4*(i%4) of a 4 x 32 block)
  const int a_lane = Gp::row(lr) + 8 * lh;
  const int t_lane = Gp::row(4 * ((lane >> 4) >> 1) + ((lane & 15) >> 2)) + 16 * ((lane >> 4) & 1) +
                     4 * (lane & 3);

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  vmem_wait_all();
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const int q0 = (qt0 + t % per_head) * kBwdBM;
    // one subtile at a time, as a rolled loop: interleaving the two would
    // spill, and unrolled, the subtile skip and the two forms of P keep more
    // registers live (measured slower)
#pragma unroll 1
    for (int sub = 0; sub < kBwdBM / 32; ++sub) {
      if constexpr (!CAUSAL) __builtin_amdgcn_sched_barrier(0);
      const int qs = q0 + 32 * sub;
      // wavefront-uniform: does any query of this subtile see any of our keys?
      if (CAUSAL && qs + 31 + off < kw) continue;
      const uint16_t* tq = &sQ[buf][0] + 8 * Gp::GRP * sub;  // row 32*sub
      const uint16_t* tg = &sG[buf][0] + 8 * Gp::GRP * sub;
      // dP - Delta in one go: the accumulator of dP starts from -Delta of each
      // element's query (LDS holds -Delta in the accumulator's row order)
      f32x16_t s = f32x16_t{0}, dp;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const f32x4_t D4 = *(const f32x4_t*)(&sD[buf][32 * sub + 8 * rg + 4 * lh]);
#pragma unroll
        for (int i = 0; i < 4; ++i) dp[4 * rg + i] = D4[i];
      }
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const u32x4_t aq = *(const u32x4_t*)(tq + a_lane + 16 * st);
        const u32x4_t ag = *(const u32x4_t*)(tg + a_lane + 16 * st);
        s = TT::mfma32(aq, kB[st], s);
        dp = TT::mfma32(ag, *(const u32x4_t*)(vrow + 16 * st), dp);
      }
      // keep the Q, dO and V operand reads one k-step ahead of their MFMAs
      // (the -Delta reads first)
      __builtin_amdgcn_sched_group_barrier(0x100, 7, 0);
#pragma unroll
      for (int st = 0; st < KS - 1; ++st) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      // rows of accumulator r: query qs + 8*(r/4) + 4*lh + r%4; column: key kw + lr
      const bool need_mask = CAUSAL && (kw + 31 > qs + off);
      // element (rg, i) is query qs + 8*rg + 4*lh + i; key kw + lr is visible
      // to it iff 8*rg + i >= thr
      const int thr = kw + lr - qs - off - 4 * lh;
      uint32_t pp[8], pd[8];
      // (one branch for the subtile: the masked and unmasked forms are
      // separate straight-line code)
      auto form_p = [&](bool masked) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const f32x4_t L4 = *(const f32x4_t*)(&sL[buf][32 * sub + 8 * rg + 4 * lh]);
          float p[4], ds[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * rg + i;
            float pv = fast_exp2(__builtin_fmaf(s[r], scale_log2, -L4[i]));
            if (masked) pv = (8 * rg + i >= thr) ? pv : 0.f;
            p[i] = pv;
            ds[i] = pv * dp[r];
          }
          pp[2 * rg] = TT::pack2(p[0], p[1]);
          pp[2 * rg + 1] = TT::pack2(p[2], p[3]);
          pd[2 * rg] = TT::pack2(ds[0], ds[1]);
          pd[2 * rg + 1] = TT::pack2(ds[2], ds[3]);
        }
      };
      if (need_mask)
        form_p(true);
      else
        form_p(false);
      // dV^T += dO^T P and dK^T += Q^T dS over this subtile's 32 queries (two k-steps
      // of 16: accumulator rows 0..7 then 8..15, i.e. queries 4*lh + {0..3, 8..11}
      // and 16 + the same)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4_t bp = {pp[4 * j], pp[4 * j + 1], pp[4 * j + 2], pp[4 * j + 3]};
        const u32x4_t bd = {pd[4 * j], pd[4 * j + 1], pd[4 * j + 2], pd[4 * j + 3]};
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          // rows 16*j + (0..7), then + 8
          const uint16_t* pg = tg + 4 * Gp::GRP * j + t_lane + 32 * db;
          const uint16_t* pq = tq + 4 * Gp::GRP * j + t_lane + 32 * db;
          const u32x2_t g_lo = lds_read_tr16(pg), g_hi = lds_read_tr16(pg + 2 * Gp::GRP);
          const u32x2_t q_lo = lds_read_tr16(pq), q_hi = lds_read_tr16(pq + 2 * Gp::GRP);
          dvT[db] = TT::mfma32(u32x4_t{g_lo[0], g_lo[1], g_hi[0], g_hi[1]}, bp, dvT[db]);
          dkT[db] = TT::mfma32(u32x4_t{q_lo[0], q_lo[1], q_hi[0], q_hi[1]}, bd, dkT[db]);
        }
      }
    }
    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: accumulator rows are d = 32*db + 8*(r/4) + 4*lh + r%4, column
  // key kw + lr; four consecutive d per 8-byte store (keys past N_kv dropped)
  const auto rdK = buffer_rsrc(dK + kv_head, head_kv_bytes);
  const auto rdV = buffer_rsrc(dV + kv_head, head_kv_bytes);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d = db * 32 + 8 * rg + 4 * lh;
      const uint32_t o = (uint32_t)((kw + lr) * D + d) * 2;
      const u32x2_t wv = {TT::pack2(dvT[db][4 * rg + 0], dvT[db][4 * rg + 1]),
                          TT::pack2(dvT[db][4 * rg + 2], dvT[db][4 * rg + 3])};
      const u32x2_t wk = {TT::pack2(dkT[db][4 * rg + 0] * scale, dkT[db][4 * rg + 1] * scale),
                          TT::pack2(dkT[db][4 * rg + 2] * scale, dkT[db][4 * rg + 3] * scale)};
      buffer_store8(rdV, o, wv);
      buffer_store8(rdK, o, wk);
    }
  }
}

// ---------------------------------------------------------------------------
// dQ. Two wavefronts per SIMD (registers capped accordingly). Workgroup:
// 32*NW query rows of head h of batch b; lane: query row
// q0 + lane % 32 as the B operand column of S^T = K Q^T and dP^T = V dO^T.
// Key tiles of 64 rows stream through LDS (double-buffered, register-staged).
// Before the tiles, each lane forms Delta = sum_d dO O over its half of the
// row's d (O read in the same layout as dO) and the other half from the lane
// 32 away, and lse2 = lse * log2(e) (+inf for a row with no visible key, so
// that its recomputed probabilities are 0); lanes of the first half write
// both for the dK/dV kernel, which runs after this one.
// Per 32-key half:
//   S^T = K Q^T, dP^T = V dO^T          (A: K, V rows from LDS; B: Q, dO in registers)
//   P^T, dS^T per element (one lse2 and Delta per lane; dP^T's accumulator
//                                        starts from -Delta)
//   dQ^T += K^T dS^T                     (A: K^T by transposing LDS reads; B: dS^T)
template <class TT, int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
    float* __restrict__ lse2, float* __restrict__ delta, uint16_t* __restrict__ dQ, int H_q, int H_kv,
    int N_q, int N_kv, float scale_log2, float scale, int nqb, int nbatch) {
  constexpr int STR = BwdLds<D>::STR;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int CPR = D / 8;
  constexpr int NT = 64 * NW;
  constexpr int LPT = kBwdBN * CPR / NT;
  constexpr int BM = 32 * NW;
  static_assert(LPT * NT == kBwdBN * CPR, "tile load must split evenly");
  using Gp = BwdGrp<D>;
  // K is read row-wise and transposed (grouped rows), V only row-wise
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][Gp::size(kBwdBN)];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][kBwdBN * STR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const BwdItem wi = bwd_map(nqb, H_q, nbatch);
  if (!wi.valid) return;
  const int b = wi.b, h = wi.h;
  const int hk = h / (H_q / H_kv);
  const int off = N_kv - N_q;

  const uint32_t head_q_bytes = (uint32_t)N_q * D * 2;
  const uint32_t head_kv_bytes = (uint32_t)N_kv * D * 2;
  const int64_t qh = ((int64_t)b * H_q + h) * (int64_t)N_q;
  const auto rQ = buffer_rsrc(Q + qh * D, head_q_bytes);
  const auto rG = buffer_rsrc(dO + qh * D, head_q_bytes);
  const int64_t kv_head = ((int64_t)b * H_kv + hk) * (int64_t)N_kv * D;
  const auto rK = buffer_rsrc(K + kv_head, head_kv_bytes);
  const auto rV = buffer_rsrc(V + kv_head, head_kv_bytes);

  // causal: block 0 (in the work order) is the one with the most keys
  const int qblk = CAUSAL ? nqb - 1 - wi.blk : wi.blk;
  const int q0 = qblk * BM + 32 * wave;
  const int qrow = q0 + lr;
  const int lim = CAUSAL ? min(N_kv, max(qrow + off + 1, 0)) : N_kv;  // keys below lim visible
  u32x4_t qB[KS], gB[KS], oB[KS];
  const auto rO = buffer_rsrc(O + qh * D, head_q_bytes);
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    qB[st] = buffer_load16(rQ, (uint32_t)(qrow * D + 16 * st + 8 * lh) * 2);
    gB[st] = buffer_load16(rG, (uint32_t)(qrow * D + 16 * st + 8 * lh) * 2);
    oB[st] = buffer_load16(rO, (uint32_t)(qrow * D + 16 * st + 8 * lh) * 2);
  }
  const bool in = qrow < N_q;
  const float lse_n = in ? LSE[qh + qrow] : kNegInf;

  int kv_end = N_kv;
  if (CAUSAL) {
    const int qlast = min(qblk * BM + BM - 1, N_q - 1);
    kv_end = min(N_kv, max(qlast + off + 1, 0));
  }
  const int ntiles = (kv_end + kBwdBN - 1) / kBwdBN;

  uint32_t ld_off[LPT];
  int st_k[LPT], st_v[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int c = tid + NT * i;
    ld_off[i] = (uint32_t)((c / CPR) * D + (c % CPR) * 8) * 2;
    st_k[i] = Gp::row(c / CPR) + (c % CPR) * 8;
    st_v[i] = (c / CPR) * STR + (c % CPR) * 8;
  }
  u32x4_t kbuf[LPT], vbuf[LPT];
  auto load_tile = [&](int t) {
    const uint32_t base = (uint32_t)(t * kBwdBN) * D * 2;
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

  f32x16_t dqT[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dqT[i] = f32x16_t{0};
  const int ak_lane = Gp::row(lr) + 8 * lh;
  const int av_lane = lr * STR + 8 * lh;
  const int t_lane = Gp::row(4 * ((lane >> 4) >> 1) + ((lane & 15) >> 2)) + 16 * ((lane >> 4) & 1) +
                     4 * (lane & 3);

  if (ntiles > 0) load_tile(0);
  // ---- this row's Delta and lse2 (O and dO arrive while tile 0 is loading)
  float Dl = 0.f;
#pragma unroll
  for (int st = 0; st < KS; ++st)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      Dl = __builtin_fmaf(TT::lo(gB[st][w]), TT::lo(oB[st][w]), Dl);
      Dl = __builtin_fmaf(TT::hi(gB[st][w]), TT::hi(oB[st][w]), Dl);
    }
  Dl += __shfl_xor(Dl, 32);
  const float L2 = (lse_n == kNegInf) ? __builtin_inff() : lse_n * kLog2e;
  if (in && lh == 0) {
    lse2[qh + qrow] = L2;
    delta[qh + qrow] = Dl;
  }
  if (ntiles > 0) store_tile(0);
  vmem_wait_all();
  __syncthreads();
  const f32x16_t negD = f32x16_t(-Dl);

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const int kv0 = t * kBwdBN;
#pragma unroll 1
    for (int kb = 0; kb < kBwdBN / 32; ++kb) {
      const int ks = kv0 + 32 * kb;
      // wavefront-uniform: does any of our rows see any key of this half?
      if (CAUSAL && ks > q0 + 31 + off) continue;
      const uint16_t* tk = &sK[buf][0] + 8 * Gp::GRP * kb;  // row 32*kb
      const uint16_t* tv = &sV[buf][0] + 32 * kb * STR;
      // dP - Delta in one go: the accumulator of dP^T starts from -Delta (every
      // element of a lane belongs to the lane's query row)
      f32x16_t s = f32x16_t{0}, dp = negD;
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const u32x4_t ak = *(const u32x4_t*)(tk + ak_lane + 16 * st);
        const u32x4_t av = *(const u32x4_t*)(tv + av_lane + 16 * st);
        s = TT::mfma32(ak, qB[st], s);
        dp = TT::mfma32(av, gB[st], dp);
      }
      // keep the K and V operand reads two k-steps ahead of their MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int st = 0; st < KS - 2; ++st) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      // rows of accumulator r: key ks + 8*(r/4) + 4*lh + r%4; column: this lane's row
      const bool need_mask = ks + 32 > N_kv || (CAUSAL && ks + 31 > q0 + off);
      uint32_t pd[8];
      // (one branch for the half: the masked and unmasked forms are separate
      // straight-line code)
      // register r holds key ks + 4*lh + e, e = 8*(r/4) + r%4: visible iff e < thr
      const int thr = lim - ks - 4 * lh;
      auto form_ds = [&](bool masked) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float p0 = fast_exp2(__builtin_fmaf(s[r], scale_log2, -L2));
          float p1 = fast_exp2(__builtin_fmaf(s[r + 1], scale_log2, -L2));
          if (masked) {
            const int e = 8 * (r >> 2) + (r & 3);
            p0 = e < thr ? p0 : 0.f;
            p1 = e + 1 < thr ? p1 : 0.f;
          }
          pd[r >> 1] = TT::pack2(p0 * dp[r], p1 * dp[r + 1]);
        }
      };
      if (need_mask)
        form_ds(true);
      else
        form_ds(false);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4_t bd = {pd[4 * j], pd[4 * j + 1], pd[4 * j + 2], pd[4 * j + 3]};
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint16_t* pk = tk + 4 * Gp::GRP * j + t_lane + 32 * db;  // rows 16*j + ...
          const u32x2_t lo = lds_read_tr16(pk), hi = lds_read_tr16(pk + 2 * Gp::GRP);
          dqT[db] = TT::mfma32(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, bd, dqT[db]);
        }
      }
    }
    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  const auto rdQ = buffer_rsrc(dQ + qh * D, head_q_bytes);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d = db * 32 + 8 * rg + 4 * lh;
      const u32x2_t w = {TT::pack2(dqT[db][4 * rg + 0] * scale, dqT[db][4 * rg + 1] * scale),
                         TT::pack2(dqT[db][4 * rg + 2] * scale, dqT[db][4 * rg + 3] * scale)};
      buffer_store8(rdQ, (uint32_t)(qrow * D + d) * 2, w);
    }
  }
}

unsigned xcd_grid(int64_t items) { return (unsigned)(((items + 7) / 8) * 8); }

template <class TT, int D>
hipError_t launch_bwd_t(const BackwardArgs& a, hipStream_t st) {
  const float sl2 = a.scale * kLog2e;
  const auto q = (const uint16_t*)a.q;
  const auto k = (const uint16_t*)a.k;
  const auto v = (const uint16_t*)a.v;
  const auto d_o = (const uint16_t*)a.d_o;
  // dQ first: it also writes lse2 and Delta for every query row
  if (a.N_q > 0) {
    constexpr int NW = 8;  // 256 rows per workgroup, two wavefronts per SIMD
    const int nqb = (a.N_q + 32 * NW - 1) / (32 * NW);
    const dim3 g(xcd_grid((int64_t)nqb * a.H_q * a.B));
    const auto o = (const uint16_t*)a.o;
    const hipError_t e =
        a.causal ? launch_kernel(bwd_dq_kernel<TT, D, true, NW>, g, dim3(64 * NW), st, q, k, v, o, d_o, a.lse,
                                 a.lse2, a.delta, (uint16_t*)a.dq, a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, a.scale,
                                 nqb, a.B)
                 : launch_kernel(bwd_dq_kernel<TT, D, false, NW>, g, dim3(64 * NW), st, q, k, v, o, d_o, a.lse,
                                 a.lse2, a.delta, (uint16_t*)a.dq, a.H_q, a.H_kv, a.N_q, a.N_kv, sl2, a.scale,
                                 nqb, a.B);
    if (e != hipSuccess) return e;
  }
  if (a.N_kv > 0) {
    const int nkb = (a.N_kv + kBwdKW - 1) / kBwdKW;
    const dim3 g(xcd_grid((int64_t)nkb * a.H_kv * a.B));
    const hipError_t e =
        a.causal ? launch_kernel(bwd_dkdv_kernel<TT, D, true>, g, dim3(64 * kBwdNWK), st, q, k, v, d_o,
                                 a.lse2, a.delta, (uint16_t*)a.dk, (uint16_t*)a.dv, a.H_q, a.H_kv, a.N_q,
                                 a.N_kv, sl2, a.scale, nkb, a.B)
                 : launch_kernel(bwd_dkdv_kernel<TT, D, false>, g, dim3(64 * kBwdNWK), st, q, k, v, d_o,
                                 a.lse2, a.delta, (uint16_t*)a.dk, (uint16_t*)a.dv, a.H_q, a.H_kv, a.N_q,
                                 a.N_kv, sl2, a.scale, nkb, a.B);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, hipStream_t st) {
  if (a.dtype == kDtypeBF16) return a.d == 64 ? launch_bwd_t<BF16, 64>(a, st) : launch_bwd_t<BF16, 128>(a, st);
  return a.d == 64 ? launch_bwd_t<F16, 64>(a, st) : launch_bwd_t<F16, 128>(a, st);
}

}  // namespace attn
