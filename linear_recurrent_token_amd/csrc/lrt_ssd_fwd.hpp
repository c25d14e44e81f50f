// lrt_ssd_fwd.hpp -- the chunkwise forward of the Mamba2 (SSD) mixer in one
// kernel: the scalar-decay recurrence without the delta term (mixer list
// under Table 2 of the AMD ROCm blog "Pretraining hybrid LLMs with Primus",
// section "How hybrid models are defined in Primus").
//
// Per chunk of C tokens with start state Hn (H = S^T, rows d, columns v):
//   g = inclusive cumsum of log a,  gamma = e^g,  Gamma_ij = e^(g_i - g_j)
//   P = (Q K^T) o Gamma  (j <= i)
//   O = diag(gamma) Q Hn + P V
//   Hn <- gamma_C Hn + K^T diag(e^(g_C - g)) V
//
// One workgroup of NW waves per (b, h, block of BV value columns) walks the
// chunks in order, its state block in MFMA accumulators.  Without the delta
// term nothing in a chunk but the state product waits on the previous chunk,
// and the chunk step is short:
//  * every wave computes the chunk's gates itself from one log a per lane
//    (wave scan, values exchanged by lane shuffles): no LDS gate arrays and
//    no barrier to publish them;
//  * V and e^(g_C - g) V stay row-major in LDS and P is stored transposed,
//    so both products that contract over tokens read their operands with the
//    LDS transpose read -- no U staging phase;
//  * the next PF chunks' q, k, v and log a load into registers while this
//    chunk computes; loads and the o-row stores are unconditional (clamped
//    rows and chunk index), so the compiler's wait for a chunk's operands
//    counts exactly and leaves later loads and the stores in flight;
//  * a wave's output and state tiles share one operand fragment per k step;
//  * two barriers per chunk where second copies of q, v and Hn^T fit in LDS
//    (odd chunks use them): the state update runs before the P^T barrier,
//    and a chunk's o rows leave after the next chunk's first barrier, so no
//    barrier separates the output products from the next chunk's staging;
//    otherwise three.
// SAVE (the training forward) also writes each chunk's start state S_n
// ([d_v][d_k] per chunk, as the backward reads it), the gate cumsums g and
// P^T ([j][i] per chunk; the column blocks of one (b, h) write identical
// values).
// Measured on MI355X at B=16, T=2048, H=8, d=128: 64 value columns per
// workgroup beat 32 (two workgroups per CU, but each recomputes Q K^T for
// half the columns) and 16, and PF = 2 gains nothing over PF = 1.
#pragma once
#include "lrt_common.hpp"
#include "lrt_internal.hpp"

namespace lrt {

template <typename E, int C, int DK, int BV>
struct SsdFwdLds {
  static constexpr int P = lds_pad<E>();
  static constexpr int LK = DK + P, LB = BV + P, LC = C + P;
  static constexpr size_t es = sizeof(E);
  static constexpr size_t K = 0;                          // k rows [t][d]
  static constexpr size_t Q = K + (size_t)C * LK * es;    // q rows [t][d]
  static constexpr size_t V = Q + (size_t)C * LK * es;    // v rows [t][v]
  static constexpr size_t VK = V + (size_t)C * LB * es;   // e^(g_C - g_t) v rows [t][v]
  static constexpr size_t S = VK + (size_t)C * LB * es;   // Hn^T [v][d]
  static constexpr size_t PT = S + (size_t)BV * LK * es;  // P^T [j][i]
  static constexpr size_t O = PT + (size_t)C * LC * es;   // o rows [t][v]
  static constexpr size_t TOTAL = O + (size_t)C * LB * es;
  // second copies of q, v and Hn^T for odd chunks where they fit: the chunk
  // step then needs no barrier between its output products and the next
  // chunk's staging
  static constexpr size_t Q2 = TOTAL;
  static constexpr size_t V2 = Q2 + (size_t)C * LK * es;
  static constexpr size_t S2 = V2 + (size_t)C * LB * es;
  static constexpr size_t TOTAL_DB = S2 + (size_t)BV * LK * es;
  static constexpr bool DB = TOTAL_DB <= 160 * 1024;
  static constexpr size_t ALLOC = DB ? TOTAL_DB : TOTAL;
};

template <typename E, int C, int DK, int BV, int NW = 8, int PF = 1, int OCC = 2, bool SAVE = false>
__global__ __launch_bounds__(64 * NW, OCC) void k_ssd_fwd(const E* __restrict__ q, const E* __restrict__ k,
                                                        const E* __restrict__ v, const float* __restrict__ log_a,
                                                        const float* h0, float* ht, E* __restrict__ o, int T,
                                                        int H, int N, int DV, E* __restrict__ wS = nullptr,
                                                        float* __restrict__ wG = nullptr, E* __restrict__ wPt = nullptr) {
  typedef SsdFwdLds<E, C, DK, BV> Lay;
  constexpr int NT = 64 * NW;
  constexpr int LK = Lay::LK, LB = Lay::LB, LC = Lay::LC;
  constexpr int NB = C / 16, NTV = BV / 16;
  constexpr int NH = (DK / 16) * NTV, HPW = (NH + NW - 1) / NW;  // state tiles (rows d, cols v)
  constexpr int NO = NTV * NB;                                   // O^T tiles (rows v, cols t)
  static_assert(C <= 64, "one token per lane in the gate scan");
  constexpr bool DB = Lay::DB;
  __shared__ __attribute__((aligned(16))) char smem[Lay::ALLOC];
  E* sK = (E*)(smem + Lay::K);
  E* sQ0 = (E*)(smem + Lay::Q);
  E* sV0 = (E*)(smem + Lay::V);
  E* sVk = (E*)(smem + Lay::VK);
  E* sS0 = (E*)(smem + Lay::S);
  E* sPt = (E*)(smem + Lay::PT);
  E* sO = (E*)(smem + Lay::O);

  const int nvb = DV / BV;
  const int wg = xcd_group(blockIdx.x, gridDim.x);  // the column blocks of one (b, h) share an L2
  const int vb = wg % nvb, bh = wg / nvb;
  const int b = bh / H, h = bh % H, v0 = vb * BV;
  const int w = wave_id(), l = lane_id();

  f32x4 hacc[HPW];
#pragma unroll
  for (int s = 0; s < HPW; ++s) {
    const int tt = w + NW * s;
    hacc[s] = zero4();
    if (tt < NH && h0 != nullptr) {
      const int td = tt / NTV, tv = tt % NTV;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        hacc[s][r] = h0[((size_t)bh * DK + td * 16 + (l >> 4) * 4 + r) * DV + v0 + tv * 16 + (l & 15)];
    }
  }

  // one chunk's operands in registers; PF sets alternate, so the loads of
  // chunk n + PF are in flight while chunk n computes
  struct Ops {
    Tile<E, C, DK, NT> tk, tq;
    Tile<E, C, BV, NT> tv;
    float la;  // log a of token l of the chunk (every wave holds the chunk's 64)
  };
  auto fetch = [&](Ops& x, int n_) {
    const int fnv = min(C, T - n_ * C);
    const size_t ftok = (size_t)b * T + (size_t)n_ * C;
    x.tk.load_rows_clamped(k + (ftok * H + h) * DK, (size_t)H * DK, fnv);
    x.tq.load_rows_clamped(q + (ftok * H + h) * DK, (size_t)H * DK, fnv);
    x.tv.load_rows_clamped(v + (ftok * H + h) * DV + v0, (size_t)H * DV, fnv);
    x.la = log_a[(ftok + min(l, fnv - 1)) * H + h];
  };

  auto step = [&](Ops& x, int n) {
    const int nv = min(C, T - n * C);
    const size_t tok0 = (size_t)b * T + (size_t)n * C;
    // this chunk's copies of q, v and Hn^T (odd chunks: the second set)
    E* const sQ = DB && (n & 1) ? (E*)(smem + Lay::Q2) : sQ0;
    E* const sV = DB && (n & 1) ? (E*)(smem + Lay::V2) : sV0;
    E* const sS = DB && (n & 1) ? (E*)(smem + Lay::S2) : sS0;
    // ---- gates, in every wave: lane t holds token t's g, gamma, e^(g_C - g)
    asm volatile("" ::"v"(x.la));
    const float g = wave_incl_scan(l < nv ? x.la : 0.f);
    const float gC = __shfl(g, C - 1, 64);
    const float gam = __expf(g), kt = __expf(gC - g);
    // ---- this chunk's operands and the chunk-start state into LDS
    x.tk.store_masked(sK, LK, nv);
    x.tq.store_masked(sQ, LK, nv);
    x.tv.store_masked(sV, LB, nv);
    {
      // e^(g_C - g_t) v_t: each 16-byte piece of the v tile lies in one row t
      constexpr int PR = Tile<E, C, BV, NT>::PR, NP = Tile<E, C, BV, NT>::NP;
#pragma unroll
      for (int s2 = 0; s2 < Tile<E, C, BV, NT>::PT; ++s2) {
        const int idx = threadIdx.x + NT * s2;
        const int r = (idx / PR) & 63;
        const float sc = __shfl(kt, r, 64);
        if (NP % NT == 0 || idx < NP)
          *(u32x4*)(sVk + (idx / PR) * LB + (idx % PR) * (16 / (int)sizeof(E))) =
              (idx / PR) < nv ? vec_scale<E>(x.tv.x[s2], sc) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + NW * s;
      if (tt < NH) {
        const int td = tt / NTV, tv2 = tt % NTV;
        store4<E>(sS + (tv2 * 16 + (l & 15)) * LK + td * 16 + (l >> 4) * 4, hacc[s]);
      }
    }
    lds_barrier();
    // chunk n + PF (the last chunk again near the end: unconditional loads
    // keep the wait for this set exact)
    fetch(x, min(n + PF, N - 1));
    if constexpr (SAVE) {
      // S_n, and g from every lane of every wave (lanes past C hold g of
      // token C - 1, so the duplicate writes agree): a fixed store count
      const size_t tile = (size_t)bh * N + n;
      lds_to_block<E, BV, DK, NT>(wS + (tile * DV + v0) * DK, sS, LK);
      wG[tile * C + min(l, C - 1)] = g;
    }
    // (second copies) the previous chunk's o rows, complete since the
    // barrier; issued after the prefetch, so the next wait for operands
    // leaves these stores in flight
    if (DB && n > 0)
      lds_to_rows_clamped<E, C, BV, NT>(o + (((size_t)b * T + (size_t)(n - 1) * C) * H + h) * DV + v0,
                                        (size_t)H * DV, sO, LB, C);
    // ---- P^T (rows j, cols i): P_ij = (q_i . k_j) e^(g_i - g_j), j <= i
#pragma unroll
    for (int s2 = 0; s2 < (NB * NB + NW - 1) / NW; ++s2) {
      const int tt = w + NW * s2;
      if (tt < NB * NB) {
        const int ti = tt / NB, tj = tt % NB;
        const int j = tj * 16 + (l & 15), i0 = ti * 16 + (l >> 4) * 4;
        f32x4 p = zero4();
        const float gj = __shfl(g, j, 64);
        f32x4 gi;
#pragma unroll
        for (int r = 0; r < 4; ++r) gi[r] = __shfl(g, i0 + r, 64);
        if (tj <= ti) {
          mma<DK>(p, sQ + ti * 16 * LK, LK, sK + tj * 16 * LK, LK);
#pragma unroll
          for (int r = 0; r < 4; ++r) p[r] = (j <= i0 + r) ? p[r] * __expf(gi[r] - gj) : 0.f;
        }
        store4<E>(sPt + j * LC + i0, p);
      }
    }
    // ---- Hn <- gamma_C Hn + K^T (e^(g_C - g) V) (reads only K and e^(g_C - g) V; the
    // output products below read the LDS copy of the chunk-start Hn)
    const float dec = __shfl(gam, C - 1, 64);
#pragma unroll
    for (int s = 0; s < HPW; ++s) hacc[s] *= dec;
    if constexpr (NH % NW == 0 && NW % NTV == 0) {
      // a wave's tiles share their column block v: one e^(g_C - g) V
      // fragment per k step for all of them (tile s is rows td = w / NTV +
      // (NW / NTV) s, as everywhere hacc is indexed)
      mma_nA<C, HPW, true, true>(hacc, sK + (w / NTV) * 16, (NW / NTV) * 16, LK, sVk + (w % NTV) * 16, LB);
    } else {
#pragma unroll
      for (int s = 0; s < HPW; ++s) {
        const int tt = w + NW * s;
        if (tt < NH) {
          const int td = tt / NTV, tv2 = tt % NTV;
          mma<C, true, true>(hacc[s], sK + td * 16, LK, sVk + tv2 * 16, LB);
        }
      }
    }
    lds_barrier();
    if constexpr (SAVE) lds_to_block<E, C, C, NT>(wPt + ((size_t)bh * N + n) * C * C, sPt, LC);
    // ---- O^T = Hn^T (Q diag(gamma))^T + V^T P^T  (rows v, cols i) -> o rows
    if constexpr (NO % NW == 0 && NW % NB == 0) {
      // a wave's tiles share their column block i: one Q and one P^T
      // fragment per k step for all of them
      constexpr int OPW = NO / NW, TVS = NW / NB;
      const int ti = w % NB, tv0 = w / NB;
      const float gi = __shfl(gam, ti * 16 + (l & 15), 64);
      f32x4 acc[OPW];
#pragma unroll
      for (int s2 = 0; s2 < OPW; ++s2) acc[s2] = zero4();
      mma_nA<DK, OPW>(acc, sS + tv0 * 16 * LK, TVS * 16 * LK, LK, sQ + ti * 16 * LK, LK);
#pragma unroll
      for (int s2 = 0; s2 < OPW; ++s2) acc[s2] *= gi;
      mma_nA<C, OPW, true, true>(acc, sV + tv0 * 16, TVS * 16, LB, sPt + ti * 16, LC);
#pragma unroll
      for (int s2 = 0; s2 < OPW; ++s2)
        store4<E>(sO + (ti * 16 + (l & 15)) * LB + (tv0 + TVS * s2) * 16 + (l >> 4) * 4, acc[s2]);
    } else {
#pragma unroll
      for (int s2 = 0; s2 < (NO + NW - 1) / NW; ++s2) {
        const int tt = w + NW * s2;
        const int ti = (tt % NO) % NB;
        const float gi = __shfl(gam, ti * 16 + (l & 15), 64);
        if (tt < NO) {
          const int tv2 = tt / NB;
          f32x4 acc = zero4();
          mma<DK>(acc, sS + tv2 * 16 * LK, LK, sQ + ti * 16 * LK, LK);
          acc *= gi;
          mma<C, true, true>(acc, sV + tv2 * 16, LB, sPt + ti * 16, LC);
          store4<E>(sO + (ti * 16 + (l & 15)) * LB + tv2 * 16 + (l >> 4) * 4, acc);
        }
      }
    }
    if constexpr (!DB) {
      lds_barrier();
      // o rows out; issued after the prefetch, so the next chunk's wait for
      // its operands leaves these stores in flight
      lds_to_rows_clamped<E, C, BV, NT>(o + (tok0 * H + h) * DV + v0, (size_t)H * DV, sO, LB, nv);
    }
  };

  Ops x0, x1;
  fetch(x0, 0);
  if constexpr (PF > 1) fetch(x1, min(1, N - 1));
  for (int n = 0; n < N; n += PF) {
    step(x0, n);
    if (PF > 1 && n + 1 < N) step(x1, n + 1);
  }
  if (DB && N > 0) {  // the last chunk's o rows
    lds_barrier();
    lds_to_rows_clamped<E, C, BV, NT>(o + (((size_t)b * T + (size_t)(N - 1) * C) * H + h) * DV + v0, (size_t)H * DV,
                                      sO, LB, T - (N - 1) * C);
  }
  if (ht != nullptr) {
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + NW * s;
      if (tt < NH) {
        const int td = tt / NTV, tv2 = tt % NTV;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          ht[((size_t)bh * DK + td * 16 + (l >> 4) * 4 + r) * DV + v0 + tv2 * 16 + (l & 15)] = hacc[s][r];
      }
    }
  }
}

// --------------------------------------------------------------- launcher
constexpr int kSsdBV = 64;   // value columns per workgroup
constexpr int kSsdPF = 1;    // chunks of operands in flight
constexpr int kSsdOcc = 1;   // workgroups per CU the registers are sized for
// the widest column block up to kSsdBV whose tiles fit in LDS
template <typename E, int C, int DK, int BV>
constexpr int ssd_bv() {
  if constexpr (BV > 16 && SsdFwdLds<E, C, DK, BV>::TOTAL > 160 * 1024)
    return ssd_bv<E, C, DK, BV / 2>();
  else
    return BV;
}
// One workgroup per (b, h, block of value columns); SAVE also writes S_n, g and P^T.
template <typename E, int C, int DK, int DV, bool SAVE = false>
int launch_ssd_fwd(const FwdArgs& a, E* wS = nullptr, float* wG = nullptr, E* wPt = nullptr) {
  constexpr int BV = ssd_bv<E, C, DK, (DV < kSsdBV ? DV : kSsdBV)>();
  static_assert(SsdFwdLds<E, C, DK, BV>::TOTAL <= 160 * 1024, "k_ssd_fwd LDS");
  const int N = (a.T + C - 1) / C;
  const int grid = a.B * a.H * (DV / BV);
  LRT_LAUNCH(kKSsdFwd, (k_ssd_fwd<E, C, DK, BV, kStateWaves, kSsdPF, kSsdOcc, SAVE>), dim3(grid),
             dim3(64 * kStateWaves), a.stream, (const E*)a.q, (const E*)a.k, (const E*)a.v, a.log_a, a.h0, a.ht,
             (E*)a.o, a.T, a.H, N, DV, wS, wG, wPt);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace lrt
