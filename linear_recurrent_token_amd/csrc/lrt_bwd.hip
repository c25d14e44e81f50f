// lrt_bwd.hip -- chunkwise backward of Gated DeltaNet on gfx950.
//
// Gradients of L = <dO, O> + <dht, ht> for the recurrence of the Gated
// DeltaNet mixer (AMD ROCm blog "Pretraining hybrid LLMs with Primus",
// section "How hybrid models are defined in Primus", mixer list under
// Table 2), differentiated through the chunkwise form used by the forward.
// Per chunk (Hn = start state, dH' = gradient of the end state):
//   dU   = P^T dO + Ktil dH'                       P = (Q K^T) o Gamma_incl
//   dHn  = gamma_C dH' + Q^T diag(gamma) dO - W^T dU           (reverse scan)
//   dS   = (dO U^T) o Gamma_incl
//   dQ   = diag(gamma) dO Hn^T + dS K
//   dK   = dS^T Q + diag(e^(g_C - g)) U dH'^T + diag(b gamma) dX + M K + M^T K
//   dW   = -dU Hn^T,  dX = Tinv^T dW,  dY = Tinv^T dU,  dV = diag(b) dY
//   dT   = dW X^T + dU Y^T,  dA = -strict_lower(Tinv^T dT Tinv^T),
//   M    = dA o diag(b) Gamma,  X = diag(b gamma) K,  Y = diag(b) V
//   dg   = gamma o rowsum(dO o Q Hn) + rowsum(E) - colsum(E) over E = dS o QK^T
//          and E = dA o A, + b gamma o rowsum(dX o K) - s, with
//          s_j = e^(g_C - g_j) k_j . (U dH'^T)_j and dg_C += sum(s) + gamma_C <dH', Hn>
//   dlog_a = reverse cumsum of dg within the chunk;  dh0 = dH at chunk 0.
//
// Kernels, in stream order:
//   k_wy (writes T and P) / k_scan (backward mode)   recompute W, U', g, T, P,
//                S_n and U -- skipped after gdn_fwd_train, which leaves them
//   k_dstate     per (b, h, d_v block), chunks in reverse: dU (with
//                dU_local = P^T dO from the stored P) and dH'
//   k_grad       per chunk: dQ, dK, dV, dbeta, dg -> dlog_a (dW and the
//                state part of dK stay on chip)
// The Mamba2 backward (ssd_bwd) runs k_ssd_prep, k_scan, k_bwd_local
// (dU_local = P^T dO from q and k), k_dstate and k_grad in their no-delta
// modes; after ssd_fwd_train only the last two.
#include <type_traits>

#include "lrt_dstate.hpp"
#include "lrt_fwd_kernels.hpp"
#include "lrt_internal.hpp"
#include "lrt_scan.hpp"
#include "lrt_ssd_fwd.hpp"

namespace lrt {

// ------------------------------------------------------------- k_bwd_local
// dU_local = P^T dO with P = (Q K^T) o Gamma (inclusive), stored as [v][t].
// Workgroups walk the chunks persistently, prefetching the next one.
template <typename E, int C, int DK, int DV>
struct LocalLds {
  static constexpr int P = lds_pad<E>();
  static constexpr int LK = DK + P, LV = DV + P, LC = C + P;
  static constexpr size_t es = sizeof(E);
  static constexpr size_t QK = 0;  // q rows, k rows; later dU_local^T for the copy-out
  static constexpr size_t QKS = (2 * (size_t)C * LK > (size_t)DV * LC ? 2 * (size_t)C * LK : (size_t)DV * LC) * es;
  static constexpr size_t DO = QK + QKS;
  static constexpr size_t PT = DO + (size_t)C * LV * es;
  static constexpr size_t G = PT + (size_t)C * LC * es;
  static constexpr size_t TOTAL = G + C * 4;
};

template <typename E, int C, int DK, int DV>
__global__ __launch_bounds__(kThreads) void k_bwd_local(const E* __restrict__ q, const E* __restrict__ k,
                                                        const E* __restrict__ d_o, const float* __restrict__ wG,
                                                        E* __restrict__ wdUl, int T, int H, int N, int ntiles) {
  typedef LocalLds<E, C, DK, DV> Lay;
  constexpr int LK = Lay::LK, LV = Lay::LV, LC = Lay::LC, NB = C / 16;
  __shared__ __attribute__((aligned(16))) char smem[Lay::TOTAL];
  E* sQ = (E*)(smem + Lay::QK);
  E* sK = sQ + C * LK;
  E* sUl = (E*)(smem + Lay::QK);
  E* sdO = (E*)(smem + Lay::DO);
  E* sPt = (E*)(smem + Lay::PT);
  float* sg = (float*)(smem + Lay::G);
  const int w = wave_id(), l = lane_id();

  Tile<E, C, DK> tq, tk;
  Tile<E, C, DV> to;
  float rg = 0.f;
#define LRT_LOCAL_LOAD(tile_)                                                             \
  {                                                                                       \
    const int ln = (tile_) % N, lbh = (tile_) / N;                                        \
    const int lnv = min(C, T - ln * C);                                                   \
    const size_t ltok = (size_t)(lbh / H) * T + (size_t)ln * C;                           \
    const int lh = lbh % H;                                                               \
    tq.load_rows_clamped(q + (ltok * H + lh) * DK, (size_t)H * DK, lnv);                  \
    tk.load_rows_clamped(k + (ltok * H + lh) * DK, (size_t)H * DK, lnv);                  \
    rg = wG[(size_t)(tile_) * C + min((int)threadIdx.x, C - 1)];                          \
    to.load_rows_clamped(d_o + (ltok * H + lh) * DV, (size_t)H * DV, lnv);                \
  }

  int tile = blockIdx.x;
  if (tile < ntiles) LRT_LOCAL_LOAD(tile)
  for (; tile < ntiles; tile += gridDim.x) {
    const int nv = min(C, T - (tile % N) * C);
    tq.store_masked(sQ, LK, nv);
    tk.store_masked(sK, LK, nv);
    asm volatile("" ::"v"(rg));  // consumed by every lane (no load into it left pending)
    if (threadIdx.x < C) sg[threadIdx.x] = rg;
    to.store_masked(sdO, LV, nv);
    lds_barrier();
    // the next tile (the last one again on the final pass: unconditional
    // loads keep the waits on older ones exact)
    LRT_LOCAL_LOAD(min(tile + (int)gridDim.x, ntiles - 1))
    for (int tt = w; tt < NB * NB; tt += kWaves) {
      const int ti = tt / NB, tj = tt % NB;
      f32x4 acc = zero4();
      if (tj <= ti) mma<DK>(acc, sQ + ti * 16 * LK, LK, sK + tj * 16 * LK, LK);
      const int j = tj * 16 + (l & 15), i0 = ti * 16 + (l >> 4) * 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = (j <= i0 + r) ? acc[r] * __expf(sg[i0 + r] - sg[j]) : 0.f;
      store4<E>(sPt + j * LC + i0, acc);
    }
    lds_barrier();
    // dU_local = P^T dO (rows j, cols v) -> [v][t] over the dead q, k rows
    for (int tt = w; tt < NB * (DV / 16); tt += kWaves) {
      const int tj = tt / (DV / 16), tv = tt % (DV / 16);
      f32x4 acc = zero4();
      mma<C, false, true>(acc, sPt + tj * 16 * LC, LC, sdO + tv * 16, LV);
      store4<E>(sUl + (tv * 16 + (l & 15)) * LC + tj * 16 + (l >> 4) * 4, acc);
    }
    lds_barrier();
    lds_to_block<E, DV, C>(wdUl + (size_t)tile * DV * C, sUl, LC);
    lds_barrier();
  }
#undef LRT_LOCAL_LOAD
}

// ------------------------------------------------------------------ k_grad
// Per chunk, the whole chunk-parallel part of the backward, once the reverse
// state scan has produced dH' (the gradient of the chunk's end state) and dU:
//   phase 1 (the state and intra-chunk attention part)
//     dS  = (dO U^T) o Gamma_incl
//     dQ  = diag(gamma) dO Hn^T + dS K                         (final)
//     dW  = -dU Hn^T                                           (kept on chip)
//     dK1 = diag(e^(g_C - g)) U dH'^T + dS^T Q                 (kept in registers)
//   phase 2 (Gated DeltaNet: the WY part, W = Tinv X, U' = Tinv Y, X = diag(b gamma) K, Y = diag(b) V)
//     dX = Tinv^T dW,  dY = Tinv^T dU,  dV = diag(b) dY
//     dT = dW X^T + dU Y^T,  dA = -strict_lower(Tinv^T dT Tinv^T),  M = dA o diag(b) Gamma
//     dK = dK1 + diag(b gamma) dX + M K + M^T K
//   dg (the Gamma, gamma, Ktil, gamma_C, A and X terms) and dbeta are summed
//   in a fixed order (per-wave partials); dlog_a = reverse cumsum of dg.
// Phase 2's buffers lie over phase 1's, which are dead by then; dW, dK1 and
// the dg partials never leave the chip.  Operands stay in their natural
// layouts; products contracting over their rows use the LDS transpose read.
// DELTA = false is the Mamba2 recurrence (U = V, no W, T = I): phase 1 alone,
// dK = dK1, dV = dU; wU is then the value rows v [B, T, H, d_v] themselves.
template <typename E, int C, int DK, int DV, bool DELTA, int NW = kGradWaves>
struct GradLds {
  static constexpr int P = lds_pad<E>();
  static constexpr int LK = DK + P, LV = DV + P, LC = C + P;
  static constexpr size_t es = sizeof(E);
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  // live through the whole chunk
  static constexpr size_t K = 0;                                          // k rows [t][d]
  static constexpr size_t DUT = K + (size_t)C * LK * es;                  // dU^T [v][t]
  static constexpr size_t G = DUT + (size_t)DV * LC * es;                 // g [C]
  static constexpr size_t BB = G + C * 4;                                 // beta [C]
  static constexpr size_t PDG = BB + C * 4;                               // [NW][C] dg partials
  static constexpr size_t PDB = PDG + (size_t)NW * C * 4;                 // [NW][C] dbeta partials
  static constexpr size_t PCX = PDB + (DELTA ? (size_t)NW * C * 4 : 0);   // [NW][C] cx partials
  static constexpr size_t DOT = PCX + (DELTA ? (size_t)NW * C * 4 : 0);   // [NW] <dH', Hn>, [NW] dg_C terms
  static constexpr size_t U0 = (DOT + 2 * NW * 4 + 15) & ~(size_t)15;
  // phase 1
  static constexpr size_t Q = U0;                                         // q rows [t][d]
  static constexpr size_t DO = Q + (size_t)C * LK * es;                   // do rows [t][v]; later dq rows
  static constexpr size_t UT = DO + mx((size_t)C * LV, (size_t)C * LK) * es;  // U^T [v][t] (Mamba2: v rows [t][v])
  static constexpr size_t ST = UT + mx((size_t)DV * LC, (size_t)C * LV) * es;  // S_n = Hn^T [v][d]; later dH'^T
  static constexpr size_t DSJ = ST + (size_t)DV * LK * es;                // dS^T [j][i]
  static constexpr size_t END1 = DSJ + (size_t)C * LC * es;
  // phase 2, over phase 1's buffers
  static constexpr size_t VV = U0;                                        // v rows [t][v]
  static constexpr size_t TT = VV + (size_t)C * LV * es;                  // Tinv [i][j]
  static constexpr size_t DW = TT + (size_t)C * LC * es;                  // dW rows [i][d]
  static constexpr size_t F = DW + (size_t)C * LK * es;                   // dv rows
  static constexpr size_t TOTAL = DELTA ? mx(END1, F + mx((size_t)C * LV, 3 * (size_t)C * LC) * es) : END1;
  // dT^T, R^T, M^T: past the dv rows where that needs no more LDS (then the dT
  // products need not wait for the dv rows' copy-out), else over them
  static constexpr bool SEPT = F + ((size_t)C * LV + 3 * (size_t)C * LC) * es <= TOTAL;
  static constexpr size_t TR = SEPT ? F + (size_t)C * LV * es : F;
  static constexpr size_t MT = TR + 2 * (size_t)C * LC * es;
  // dk rows: over S^T where they miss M^T (the next chunk stores its S^T only
  // after its first barrier, so no barrier is needed after their copy into
  // registers), else over dW
  static constexpr bool LATE_S = DELTA && (ST + (size_t)C * LK * es <= MT || ST >= MT + (size_t)C * LC * es) &&
                                 ST + (size_t)C * LK * es <= TOTAL;
  static constexpr size_t DKR = LATE_S ? ST : DW;
};

template <typename E, int C, int DK, int DV, int NW = 8, bool DELTA = true>
__global__ __launch_bounds__(64 * NW) void k_grad(const E* __restrict__ q, const E* __restrict__ k,
                                                   const E* __restrict__ v, const E* __restrict__ d_o,
                                                   const float* __restrict__ beta, const float* __restrict__ wG,
                                                   const E* __restrict__ wS, const E* __restrict__ wdS,
                                                   const E* __restrict__ wU, const E* __restrict__ wdU,
                                                   const E* __restrict__ wT, E* __restrict__ dq,
                                                   E* __restrict__ dk_out, E* __restrict__ dv_out,
                                                   float* __restrict__ dlog_a, float* __restrict__ dbeta,
                                                   SeqMap m) {
  typedef GradLds<E, C, DK, DV, DELTA, NW> Lay;
  const int H = m.H, ntiles = tile_count(m);
  constexpr int NT = 64 * NW;
  constexpr int LK = Lay::LK, LV = Lay::LV, LC = Lay::LC, NB = C / 16;
  constexpr int V = 16 / (int)sizeof(E);
  constexpr int NKT = (DK / 16) * NB, KPW = (NKT + NW - 1) / NW;
  static_assert(NW % NB == 0, "waves must cover whole column blocks");
  // Every wave holds KPW tiles d = w / NB + (NW / NB) s of one column block
  // w % NB: the products then read the fragments the tiles share (dO, dS,
  // dU, U, T, M) once per k step for all of them (mma_nA; bf16 operands).
  constexpr int NWB = NW / NB;
  constexpr bool kShared = sizeof(E) == 2 && (DK / 16) % NWB == 0 && (DV / 16) % NWB == 0;
  constexpr bool kSharedT = sizeof(E) == 2 && (NB * NB) % NW == 0;  // the (i, j) tile products: NB * NB / NW per wave
  __shared__ __attribute__((aligned(16))) char smem[Lay::TOTAL];

  Tile<E, C, DK, NT> tq, tk;
  Tile<E, C, DV, NT> to;
  // U^T tiles, or (Mamba2) the v rows of the chunk
  typename std::conditional<DELTA, Tile<E, DV, C, NT>, Tile<E, C, DV, NT>>::type tu;
  Tile<E, DV, C, NT> tdu;
  Tile<E, DV, DK, NT> tS, tdS;
  Tile<E, C, DV, NT> tv;  // phase 2 (GDN): this chunk's v rows
  Tile<E, C, C, NT> tt;   // phase 2 (GDN): this chunk's Tinv
  float rg = 0.f, rb = 0.f;
  // The previous chunk's dk rows, d log a and dbeta (GDN), written out while
  // this chunk runs: stores left at the end of an iteration would be waited
  // for by the next iteration's first wait on its prefetched loads.
  Tile<E, C, DK, NT> pdk;
  float pdla = 0.f, pdb = 0.f;
  size_t ptok = 0;
  int ph = 0, pnv = 0;
  // The next chunk's operands are fetched in parts (bit mask PART_) spread
  // over this chunk's phases, so no wave stalls on a full memory queue.
#define LRT_G_LOAD(tile_, P_, N_, PART_)                                                  \
  {                                                                                       \
    const int lnv = min(C, (P_).len - (N_) * C);                                          \
    const size_t ltok = (P_).tok0 + (size_t)(N_) * C;                                     \
    const int lh = (P_).h;                                                                \
    if ((PART_) & 1) {                                                                    \
      tq.load_rows_clamped(q + (ltok * H + lh) * DK, (size_t)H * DK, lnv);                \
      tk.load_rows_clamped(k + (ltok * H + lh) * DK, (size_t)H * DK, lnv);                \
      rg = wG[(size_t)(tile_) * C + min((int)threadIdx.x, C - 1)];                        \
    }                                                                                     \
    if ((PART_) & 2) {                                                                    \
      to.load_rows_clamped(d_o + (ltok * H + lh) * DV, (size_t)H * DV, lnv);              \
      if constexpr (DELTA)                                                                \
        tu.load_block(wU + (size_t)(tile_) * DV * C);                                     \
      else                                                                                \
        tu.load_rows_clamped(wU + (ltok * H + lh) * DV, (size_t)H * DV, lnv);             \
    }                                                                                     \
    if ((PART_) & 4) tdu.load_block(wdU + (size_t)(tile_) * DV * C);                      \
    if ((PART_) & 8) tS.load_block(wS + (size_t)(tile_) * DV * DK);                       \
  }

  int tile = blockIdx.x;
  if (tile < ntiles) {
    int n0;
    const SeqPos p0 = tile_pos(m, tile, n0);
    LRT_G_LOAD(tile, p0, n0, 15)
  }
  for (; tile < ntiles; tile += gridDim.x) {
    // fp32 (twice the operand registers): per-chunk opaque copies of the
    // buffer and global base addresses and of the lane index, so the compiler
    // recomputes addresses inside the loop instead of hoisting lane-dependent
    // ones out of it and spilling them (bf16 has the registers to keep them).
    int z0 = 0;
    if constexpr (sizeof(E) == 4) {
      asm volatile("" : "+s"(z0));
      asm volatile("" : "+s"(q), "+s"(k), "+s"(v), "+s"(d_o), "+s"(beta), "+s"(wG), "+s"(wS), "+s"(wdS));
      asm volatile("" : "+s"(wU), "+s"(wdU), "+s"(wT), "+s"(dq), "+s"(dk_out), "+s"(dv_out), "+s"(dlog_a), "+s"(dbeta));
    }
    char* smz = smem + z0;
    E* sK = (E*)(smz + Lay::K);
    E* sdUt = (E*)(smz + Lay::DUT);
    float* sg = (float*)(smz + Lay::G);
    float* sb = (float*)(smz + Lay::BB);
    float* pdgs = (float*)(smz + Lay::PDG);
    float* pdbs = (float*)(smz + Lay::PDB);
    float* pcxs = (float*)(smz + Lay::PCX);
    float* sdot = (float*)(smz + Lay::DOT);  // [NW] <dH', Hn>
    float* slast = sdot + NW;                 // [NW] terms of dg_C
    E* sQ = (E*)(smz + Lay::Q);
    E* sdO = (E*)(smz + Lay::DO);
    E* sdQ = (E*)(smz + Lay::DO);
    E* sUt = (E*)(smz + Lay::UT);
    E* sS = (E*)(smz + Lay::ST);
    E* sdSj = (E*)(smz + Lay::DSJ);
    E* sV = (E*)(smz + Lay::VV);
    E* sT = (E*)(smz + Lay::TT);
    E* sdW = (E*)(smz + Lay::DW);
    E* sdK = (E*)(smz + Lay::DKR);
    E* sdV = (E*)(smz + Lay::F);
    E* sdTt = (E*)(smz + Lay::TR);
    E* sRt = sdTt + C * LC;
    E* sMt = sRt + C * LC;
    int tidv = threadIdx.x;
    if constexpr (sizeof(E) == 4) asm volatile("" : "+v"(tidv));
    const int w = tidv >> 6, l = tidv & 63;
    float* mydg = pdgs + w * C;
    float* mydb = pdbs + w * C;
    float* mycx = pcxs + w * C;
    int n;
    const SeqPos cp = tile_pos(m, tile, n);
    const int h = cp.h;
    const int nv = min(C, cp.len - n * C);
    const size_t tok0 = cp.tok0 + (size_t)n * C;
    // the next chunk (the last one again on the final pass: its loads go
    // unused, but unconditional loads keep the waits on older ones exact)
    const int next = min(tile + (int)gridDim.x, ntiles - 1);
    int nn;
    const SeqPos np = tile_pos(m, next, nn);
    tq.store_masked(sQ, LK, nv);
    tk.store_masked(sK, LK, nv);
    to.store_masked(sdO, LV, nv);
    if constexpr (DELTA)
      tu.store(sUt, LC);
    else
      tu.store_masked(sUt, LV, nv);
    tdu.store(sdUt, LC);
    if constexpr (!Lay::LATE_S) tS.store(sS, LK);
    asm volatile("" ::"v"(rg));  // consumed by every lane (no load into it left pending)
    if (threadIdx.x < C) sg[threadIdx.x] = rg;
    slot_zero<NW, C>(pdgs);
    if constexpr (DELTA) {
      slot_zero<NW, C>(pdbs);
      slot_zero<NW, C>(pcxs);
      if (pnv > 0) {
        pdk.store_rows(dk_out + (ptok * H + ph) * DK, (size_t)H * DK, pnv);
        if ((int)threadIdx.x < pnv) {
          dlog_a[(ptok + threadIdx.x) * H + ph] = pdla;
          dbeta[(ptok + threadIdx.x) * H + ph] = pdb;
        }
      }
    }
    tdS.load_block(wdS + (size_t)tile * DV * DK);  // dH' of this chunk, needed after dS
    lds_barrier();
    if constexpr (Lay::LATE_S) tS.store(sS, LK);  // over the previous chunk's dk rows
    LRT_G_LOAD(next, np, nn, 1)

    // dS = (dO U^T) o Gamma (inclusive); E = dS o (Q K^T) -> dg rows +, cols -
    // (a wave's tiles share column block w % NB: one column sum per wave)
    float ecol = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < (NB * NB + NW - 1) / NW; ++s2) {
      const int tt2 = w + NW * s2;
      if (tt2 >= NB * NB) break;
      const int ti = tt2 / NB, tj = tt2 % NB;
      const int j = tj * 16 + (l & 15), i0 = ti * 16 + (l >> 4) * 4;
      f32x4 ds = zero4();
      if (tj <= ti) {
        f32x4 qk = zero4(), dp = zero4(), ev;
        mma<DK>(qk, sQ + ti * 16 * LK, LK, sK + tj * 16 * LK, LK);
        if constexpr (DELTA)
          mma<DV, false, true>(dp, sdO + ti * 16 * LV, LV, sUt + tj * 16, LC);
        else
          mma<DV>(dp, sdO + ti * 16 * LV, LV, sUt + tj * 16 * LV, LV);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = i0 + r;
          ds[r] = (j <= i) ? dp[r] * __expf(sg[i] - sg[j]) : 0.f;
          ev[r] = ds[r] * qk[r];
          ecol += ev[r];
        }
        const float er = rowsum4(ev);
        // a wave's tiles have distinct row blocks: one lane per row
        if ((l & 3) == 0) mydg[i0 + ((l >> 2) & 3)] += er;
      }
      store4<E>(sdSj + j * LC + i0, ds);
      tile_fence();
    }
    ecol = sum4(ecol);
    wave_order();
    if (l < 16) mydg[(w % NB) * 16 + (l & 15)] -= ecol;
    lds_barrier();
    // <dH', Hn> from the registers of this chunk's S and dH' (before any
    // store of this chunk, so the wait for dH' leaves the prefetch in flight);
    // then the next S and more of the next chunk
    {
      float part = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < tS.PT; ++s2) {
        if (threadIdx.x + NT * s2 < tS.NP) {
          E a[V], d[V];
          __builtin_memcpy(a, &tS.x[s2], 16);
          __builtin_memcpy(d, &tdS.x[s2], 16);
#pragma unroll
          for (int e = 0; e < V; ++e) part += to_f(a[e]) * to_f(d[e]);
        }
      }
      part = sum16(part);
      part = sum4(part);
      if (l == 0) sdot[w] = part;
    }
    // (GDN: the next do, U and S wait until after the dQ products, where
    // register use peaks)
    if constexpr (!DELTA) LRT_G_LOAD(next, np, nn, 10)
    // dQ^T = gamma (Hn dO^T) + K^T dS^T (rows d, cols i), kept in registers;
    // dW^T = -Hn dU^T (GDN), kept in registers.  A wave's tiles share their
    // column block, so its dO, dS and dU fragments are the same for every
    // tile and its dg term is one sum.
    f32x4 dqa[KPW], dwa[KPW];
    {
      const int ti = w % NB, i = ti * 16 + (l & 15);
      const float gam = __expf(sg[i]);
      float esum = 0.f;
      if constexpr (kShared) {
        const int td0 = w / NB;
#pragma unroll
        for (int s = 0; s < KPW; ++s) {
          dqa[s] = zero4();
          dwa[s] = zero4();
        }
        if constexpr (DELTA)
          mma_nA2<DV, KPW, true, false, true>(dqa, dwa, sS + td0 * 16, NWB * 16, LK, sdO + ti * 16 * LV, LV,
                                              sdUt + ti * 16, LC);
        else
          mma_nA<DV, KPW, true, false>(dqa, sS + td0 * 16, NWB * 16, LK, sdO + ti * 16 * LV, LV);
#pragma unroll
        for (int s = 0; s < KPW; ++s) {
          const int d0 = (td0 + NWB * s) * 16 + (l >> 4) * 4;
#pragma unroll
          for (int r = 0; r < 4; ++r) esum += to_f(sQ[i * LK + d0 + r]) * dqa[s][r];
          dqa[s] *= gam;
          dwa[s] = -dwa[s];
        }
        mma_nA<C, KPW, true, true>(dqa, sK + td0 * 16, NWB * 16, LK, sdSj + ti * 16, LC);
      } else {
#pragma unroll
        for (int s = 0; s < KPW; ++s) {
          const int td = w / NB + (NW / NB) * s;
          dqa[s] = zero4();
          dwa[s] = zero4();
          if (td < DK / 16) {
            const int d0 = td * 16 + (l >> 4) * 4;
            f32x4 acc = zero4();
            mma<DV, true, false>(acc, sS + td * 16, LK, sdO + ti * 16 * LV, LV);
#pragma unroll
            for (int r = 0; r < 4; ++r) esum += to_f(sQ[i * LK + d0 + r]) * acc[r];
            acc *= gam;
            mma<C, true, true>(acc, sK + td * 16, LK, sdSj + ti * 16, LC);
            dqa[s] = acc;
            if constexpr (DELTA) {
              f32x4 dw = zero4();
              mma<DV, true, true>(dw, sS + td * 16, LK, sdUt + ti * 16, LC);
              dwa[s] = -dw;
            }
          }
          tile_fence();
        }
      }
      esum = sum4(esum * gam);
      wave_order();
      if (l < 16) mydg[i] += esum;
    }
    lds_barrier();
    // dq rows over the dead dO; dH'^T over the dead S
#pragma unroll
    for (int s = 0; s < KPW; ++s) {
      const int td = w / NB + (NW / NB) * s, ti = w % NB;
      if (td < DK / 16) store4<E>(sdQ + (ti * 16 + (l & 15)) * LK + td * 16 + (l >> 4) * 4, dqa[s]);
    }
    tdS.store(sS, LK);
    lds_barrier();
    LRT_G_LOAD(next, np, nn, DELTA ? 6 : 4)
    if constexpr (DELTA) {
      // phase 2's operands of this chunk (clamped rows: unconditional loads),
      // issued here so their registers are not held through the dQ products
      tv.load_rows_clamped(v + (tok0 * H + h) * DV, (size_t)H * DV, nv);
      tt.load_block(wT + (size_t)tile * C * C);
      rb = beta[(tok0 + min((int)threadIdx.x, nv - 1)) * H + h];
    }
    lds_to_rows<E, C, DK, NT>(dq + (tok0 * H + h) * DK, (size_t)H * DK, sdQ, LK, nv);
    // dK1^T = e^(g_C - g_j) (dH' U^T) + Q^T dS   (rows d, cols j); a wave's
    // tiles share their column block j
    const float gC = sg[C - 1];
    f32x4 dka[KPW];
    {
      const int tj = w % NB, j = tj * 16 + (l & 15);
      const float kt = __expf(gC - sg[j]);
      float ssum = 0.f;
      if constexpr (kShared) {
        const int td0 = w / NB;
#pragma unroll
        for (int s = 0; s < KPW; ++s) dka[s] = zero4();
        if constexpr (DELTA)
          mma_nA<DV, KPW, true, true>(dka, sS + td0 * 16, NWB * 16, LK, sUt + tj * 16, LC);
        else
          mma_nA<DV, KPW, true, false>(dka, sS + td0 * 16, NWB * 16, LK, sUt + tj * 16 * LV, LV);
#pragma unroll
        for (int s = 0; s < KPW; ++s) {
          const int d0 = (td0 + NWB * s) * 16 + (l >> 4) * 4;
#pragma unroll
          for (int r = 0; r < 4; ++r) ssum += dka[s][r] * to_f(sK[j * LK + d0 + r]);
          dka[s] *= kt;
        }
        mma_nA<C, KPW, true, false>(dka, sQ + td0 * 16, NWB * 16, LK, sdSj + tj * 16 * LC, LC);
      } else {
#pragma unroll
        for (int s = 0; s < KPW; ++s) {
          const int td = w / NB + (NW / NB) * s;
          dka[s] = zero4();
          if (td < DK / 16) {
            const int d0 = td * 16 + (l >> 4) * 4;
            f32x4 acc = zero4();
            if constexpr (DELTA)
              mma<DV, true, true>(acc, sS + td * 16, LK, sUt + tj * 16, LC);
            else
              mma<DV, true, false>(acc, sS + td * 16, LK, sUt + tj * 16 * LV, LV);
#pragma unroll
            for (int r = 0; r < 4; ++r) ssum += acc[r] * to_f(sK[j * LK + d0 + r]);
            acc *= kt;
            mma<C, true, false>(acc, sQ + td * 16, LK, sdSj + tj * 16 * LC, LC);
            dka[s] = acc;
          }
          tile_fence();
        }
      }
      ssum = sum4(ssum * kt);
      const float stot = sum16(ssum);  // over the wave's 16 columns j (lanes 0..15)
      wave_order();
      if (l < 16) mydg[j] -= ssum;
      if (l == 0) slast[w] = stot;
    }
    lds_barrier();
    if constexpr (DELTA) {
      // ---- phase 2 operands over phase 1's dead buffers: v rows, Tinv, dW rows
      tv.store_masked(sV, LV, nv);
      tt.store(sT, LC);
#pragma unroll
      for (int s = 0; s < KPW; ++s) {
        const int td = w / NB + (NW / NB) * s, ti = w % NB;
        if (td < DK / 16) store4<E>(sdW + (ti * 16 + (l & 15)) * LK + td * 16 + (l >> 4) * 4, dwa[s]);
      }
      asm volatile("" ::"v"(rb));
      if (threadIdx.x < C) sb[threadIdx.x] = (int)threadIdx.x < nv ? rb : 0.f;
      lds_barrier();
      // dX^T = dW^T Tinv (rows d, cols j): dK += b gamma dX, cx_j = dX_j . k_j
      // (a wave's tiles all lie in column block w % NB: one column sum per wave)
      const int jw = (w % NB) * 16 + (l & 15);
      {
        const float bgj = sb[jw] * __expf(sg[jw]);
        float e = 0.f;
        if constexpr (kShared) {
          f32x4 xa[KPW];
#pragma unroll
          for (int s = 0; s < KPW; ++s) xa[s] = zero4();
          mma_nA<C, KPW, true, true>(xa, sdW + (w / NB) * 16, NWB * 16, LK, sT + (w % NB) * 16, LC);
#pragma unroll
          for (int s = 0; s < KPW; ++s) {
            const int d0 = (w / NB + NWB * s) * 16 + (l >> 4) * 4;
            dka[s] += bgj * xa[s];
#pragma unroll
            for (int r = 0; r < 4; ++r) e += xa[s][r] * to_f(sK[jw * LK + d0 + r]);
          }
        } else {
#pragma unroll
          for (int s = 0; s < KPW; ++s) {
            const int kt = w + NW * s;
            if (kt < NKT) {
              const int td = kt / NB, tj = kt % NB;
              const int d0 = td * 16 + (l >> 4) * 4;
              f32x4 acc = zero4();
              mma<C, true, true>(acc, sdW + td * 16, LK, sT + tj * 16, LC);
              dka[s] += bgj * acc;
#pragma unroll
              for (int r = 0; r < 4; ++r) e += acc[r] * to_f(sK[jw * LK + d0 + r]);
            }
            tile_fence();
          }
        }
        e = sum4(e);
        if (l < 16) mycx[jw] += e;
      }
      // dY^T = dU^T Tinv (rows v, cols j): dV = b dY (rows staged), dbeta += dY_j . v_j
      {
        const float bj = sb[jw];
        float e = 0.f;
        if constexpr (kShared) {
          constexpr int VPW = (DV / 16) / NWB;
          f32x4 ya[VPW];
#pragma unroll
          for (int s = 0; s < VPW; ++s) ya[s] = zero4();
          mma_nA<C, VPW, false, true>(ya, sdUt + (w / NB) * 16 * LC, NWB * 16 * LC, LC, sT + (w % NB) * 16, LC);
#pragma unroll
          for (int s = 0; s < VPW; ++s) {
            const int v0 = (w / NB + NWB * s) * 16 + (l >> 4) * 4;
            store4<E>(sdV + jw * LV + v0, bj * ya[s]);
#pragma unroll
            for (int r = 0; r < 4; ++r) e += ya[s][r] * to_f(sV[jw * LV + v0 + r]);
          }
        } else {
#pragma unroll
          for (int s2 = 0; s2 < ((DV / 16) * NB + NW - 1) / NW; ++s2) {
            const int tt2 = w + NW * s2;
            if (tt2 >= (DV / 16) * NB) break;
            const int tvv = tt2 / NB, tj = tt2 % NB;
            const int v0 = tvv * 16 + (l >> 4) * 4;
            f32x4 acc = zero4();
            mma<C, false, true>(acc, sdUt + tvv * 16 * LC, LC, sT + tj * 16, LC);
            store4<E>(sdV + jw * LV + v0, bj * acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) e += acc[r] * to_f(sV[jw * LV + v0 + r]);
            tile_fence();
          }
        }
        e = sum4(e);
        if (l < 16) mydb[jw] += e;
      }
      // dT = (dW K^T) diag(b gamma) + (dU V^T) diag(b)   (rows i, cols j) -> dT^T [j][i]
      // (in the dY phase when dT^T is not over the dv rows, else after their copy-out)
      auto dt_products = [&]() {
        if constexpr (kSharedT) {
          constexpr int TPW = NB * NB / NW;
          f32x4 z1[TPW], z2[TPW];
#pragma unroll
          for (int s = 0; s < TPW; ++s) {
            z1[s] = zero4();
            z2[s] = zero4();
          }
          mma_nA<DK, TPW>(z1, sdW + (w / NB) * 16 * LK, NWB * 16 * LK, LK, sK + (w % NB) * 16 * LK, LK);
          mma_nA<DV, TPW, true, false>(z2, sdUt + (w / NB) * 16, NWB * 16, LC, sV + (w % NB) * 16 * LV, LV);
          const int j = (w % NB) * 16 + (l & 15);
          const float bj = sb[j], bgj = bj * __expf(sg[j]);
#pragma unroll
          for (int s = 0; s < TPW; ++s)
            store4<E>(sdTt + j * LC + (w / NB + NWB * s) * 16 + (l >> 4) * 4, bgj * z1[s] + bj * z2[s]);
        }
#pragma unroll
        for (int s2 = 0; s2 < (kSharedT ? 0 : (NB * NB + NW - 1) / NW); ++s2) {
          const int t2 = w + NW * s2;
          if (t2 >= NB * NB) break;
          const int ti = t2 / NB, tj = t2 % NB;
          const int j = tj * 16 + (l & 15), i0 = ti * 16 + (l >> 4) * 4;
          f32x4 z1 = zero4(), z2 = zero4();
          mma<DK>(z1, sdW + ti * 16 * LK, LK, sK + tj * 16 * LK, LK);
          mma<DV, true, false>(z2, sdUt + ti * 16, LC, sV + tj * 16 * LV, LV);
          store4<E>(sdTt + j * LC + i0, sb[j] * (__expf(sg[j]) * z1 + z2));
          tile_fence();
        }
      };
      if constexpr (Lay::SEPT) dt_products();
      lds_barrier();
      lds_to_rows<E, C, DV, NT>(dv_out + (tok0 * H + h) * DV, (size_t)H * DV, sdV, LV, nv);
      if constexpr (!Lay::SEPT) lds_barrier();
      LRT_G_LOAD(next, np, nn, 8)
      if constexpr (!Lay::SEPT) {
        dt_products();
        lds_barrier();
      }
      // R = dT Tinv^T (rows i, cols k) -> R^T [k][i]
      if constexpr (kSharedT) {
        constexpr int TPW = NB * NB / NW;
        f32x4 ra[TPW];
#pragma unroll
        for (int s = 0; s < TPW; ++s) ra[s] = zero4();
        mma_nA<C, TPW, true, false>(ra, sdTt + (w / NB) * 16, NWB * 16, LC, sT + (w % NB) * 16 * LC, LC);
#pragma unroll
        for (int s = 0; s < TPW; ++s)
          store4<E>(sRt + ((w % NB) * 16 + (l & 15)) * LC + (w / NB + NWB * s) * 16 + (l >> 4) * 4, ra[s]);
      }
#pragma unroll
      for (int s2 = 0; s2 < (kSharedT ? 0 : (NB * NB + NW - 1) / NW); ++s2) {
        const int t2 = w + NW * s2;
        if (t2 >= NB * NB) break;
        const int ti = t2 / NB, tk2 = t2 % NB;
        f32x4 acc = zero4();
        mma<C, true, false>(acc, sdTt + ti * 16, LC, sT + tk2 * 16 * LC, LC);
        store4<E>(sRt + (tk2 * 16 + (l & 15)) * LC + ti * 16 + (l >> 4) * 4, acc);
        tile_fence();
      }
      lds_barrier();
      // dA = -strict_lower(Tinv^T R); with A = b_i (K K^T) o Gamma:
      //   M = dA o b_i Gamma -> M^T [k][i], dbeta_i += sum_k dA o Gamma o KK^T, E = dA o A -> dg
      float ecol2 = 0.f;  // column kk = jw for every tile of this wave
#pragma unroll
      for (int s2 = 0; s2 < (NB * NB + NW - 1) / NW; ++s2) {
        const int t2 = w + NW * s2;
        if (t2 >= NB * NB) break;
        const int ti = t2 / NB, tk2 = t2 % NB;
        const int kk = tk2 * 16 + (l & 15), i0 = ti * 16 + (l >> 4) * 4;
        f32x4 m = zero4();
        if (tk2 <= ti) {
          f32x4 acc = zero4(), kkt = zero4();
          mma<C, true, false>(acc, sT + ti * 16, LC, sRt + tk2 * 16 * LC, LC);
          mma<DK>(kkt, sK + ti * 16 * LK, LK, sK + tk2 * 16 * LK, LK);
          f32x4 ev, bv;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = i0 + r;
            const float gam = (kk < i) ? __expf(sg[i] - sg[kk]) : 0.f;
            const float da = -acc[r];
            const float a = sb[i] * kkt[r] * gam;
            m[r] = da * sb[i] * gam;
            ev[r] = da * a;
            bv[r] = da * gam * kkt[r];
            ecol2 += ev[r];
          }
          const float er = rowsum4(ev), br = rowsum4(bv);
          // a wave's tiles have distinct row blocks: one lane per row
          if ((l & 3) == 0) {
            const int ir = i0 + ((l >> 2) & 3);
            mydg[ir] += er;
            mydb[ir] += br;
          }
        }
        store4<E>(sMt + kk * LC + i0, m);
        tile_fence();
      }
      ecol2 = sum4(ecol2);
      wave_order();
      if (l < 16) mydg[jw] -= ecol2;
      lds_barrier();
      // dK^T += K^T M (cols j: sum_i k_i M_ij) + K^T M^T (cols i: sum_j k_j M_ij) -> dk rows over dW
      if constexpr (kShared) {
        mma_nA2<C, KPW, true, false, true>(dka, dka, sK + (w / NB) * 16, NWB * 16, LK, sMt + (w % NB) * 16 * LC, LC,
                                           sMt + (w % NB) * 16, LC);
#pragma unroll
        for (int s = 0; s < KPW; ++s)
          store4<E>(sdK + ((w % NB) * 16 + (l & 15)) * LK + (w / NB + NWB * s) * 16 + (l >> 4) * 4, dka[s]);
      } else {
#pragma unroll
        for (int s = 0; s < KPW; ++s) {
          const int kt = w + NW * s;
          if (kt < NKT) {
            const int td = kt / NB, tj = kt % NB;
            mma<C, true, false>(dka[s], sK + td * 16, LK, sMt + tj * 16 * LC, LC);
            mma<C, true, true>(dka[s], sK + td * 16, LK, sMt + tj * 16, LC);
            store4<E>(sdK + (tj * 16 + (l & 15)) * LK + td * 16 + (l >> 4) * 4, dka[s]);
          }
          tile_fence();
        }
      }
      // dg (+ the X = diag(b gamma) K term), reverse cumsum -> dlog_a; dbeta
      if (threadIdx.x < 64) {
        const int t = threadIdx.x;
        float dg = 0.f, db = 0.f;
        if (t < C) {
          const float gam = __expf(sg[t]);
          const float cx = slot_sum<NW, C>(pcxs, t);
          dg = slot_sum<NW, C>(pdgs, t) + sb[t] * gam * cx;
          if (t == C - 1) {
            float last = 0.f, dot = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) {
              last += slast[w2];
              dot += sdot[w2];
            }
            dg += last + __expf(gC) * dot;
          }
          db = slot_sum<NW, C>(pdbs, t) + gam * cx;
        }
        pdla = wave_incl_suffix(dg);
        pdb = db;
      }
      lds_barrier();
      pdk.load_lds(sdK, LK);
      ptok = tok0;
      ph = h;
      pnv = nv;
      if constexpr (!Lay::LATE_S) lds_barrier();
    } else {
      // dg, reverse cumsum -> dlog_a (wave 0, one token per lane)
      if (threadIdx.x < 64) {
        const int t = threadIdx.x;
        float dg = 0.f;
        if (t < C) {
          dg = slot_sum<NW, C>(pdgs, t);
          if (t == C - 1) {
            float last = 0.f, dot = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) {
              last += slast[w2];
              dot += sdot[w2];
            }
            dg += last + __expf(gC) * dot;
          }
        }
        const float sfx = wave_incl_suffix(dg);
        if (t < nv) dlog_a[(tok0 + t) * H + h] = sfx;
      }
      // dk rows over the dead dq rows (copied out before the last barrier)
#pragma unroll
      for (int s = 0; s < KPW; ++s) {
        const int td = w / NB + (NW / NB) * s, tj = w % NB;
        if (td < DK / 16) store4<E>(sdQ + (tj * 16 + (l & 15)) * LK + td * 16 + (l >> 4) * 4, dka[s]);
      }
      // dv rows = dU^T read back column-wise from LDS
      for (int idx = threadIdx.x; idx < C * (DV / V); idx += NT) {
        const int t = idx / (DV / V), c0 = (idx % (DV / V)) * V;
        if (t < nv) {
          E x[V];
#pragma unroll
          for (int e = 0; e < V; ++e) x[e] = sdUt[(c0 + e) * LC + t];
          u32x4 pk;
          __builtin_memcpy(&pk, x, 16);
          *(u32x4*)(dv_out + ((tok0 + t) * H + h) * DV + c0) = pk;
        }
      }
      lds_barrier();
      lds_to_rows<E, C, DK, NT>(dk_out + (tok0 * H + h) * DK, (size_t)H * DK, sdQ, LK, nv);
      lds_barrier();
    }
  }
  if constexpr (DELTA) {
    if (pnv > 0) {
      pdk.store_rows(dk_out + (ptok * H + ph) * DK, (size_t)H * DK, pnv);
      if ((int)threadIdx.x < pnv) {
        dlog_a[(ptok + threadIdx.x) * H + ph] = pdla;
        dbeta[(ptok + threadIdx.x) * H + ph] = pdb;
      }
    }
  }
#undef LRT_G_LOAD
}

// ------------------------------------------------------------- k_ssd_prep
// Mamba2 backward, per chunk: g = inclusive cumsum of log a (tokens past the
// end of a ragged last chunk add 0) and U'^T = V^T [d_v][C] (columns past the
// end zero): what the state recompute and the gradient kernels read where the
// Gated DeltaNet path reads the WY pass's g and U (with no delta term U = V).
template <typename E, int C, int DV>
__global__ __launch_bounds__(kThreads) void k_ssd_prep(const E* __restrict__ v, const float* __restrict__ log_a,
                                                       float* __restrict__ wG, E* __restrict__ wUt, int T, int H,
                                                       int N, int ntiles) {
  constexpr int LC = C + lds_pad<E>();
  __shared__ __attribute__((aligned(16))) E sVt[DV * LC];
  Tile<E, C, DV> tv;
  float rla = 0.f;
  // the next tile loads while this one is transposed (clamped rows and tile
  // index: unconditional loads, so no wait lands at their issue)
  auto load = [&](int tile_) {
    const int ln = tile_ % N, lbh = tile_ / N;
    const int lnv = min(C, T - ln * C);
    const size_t ltok = (size_t)(lbh / H) * T + (size_t)ln * C;
    tv.load_rows_clamped(v + (ltok * H + lbh % H) * DV, (size_t)H * DV, lnv);
    rla = log_a[(ltok + min(lane_id(), lnv - 1)) * H + lbh % H];
  };
  int tile = blockIdx.x;
  if (tile < ntiles) load(tile);
  for (; tile < ntiles; tile += gridDim.x) {
    const int nv = min(C, T - (tile % N) * C);
    asm volatile("" ::"v"(rla));
    if (threadIdx.x < 64) {
      const int t = threadIdx.x;
      const float g = wave_incl_scan(t < nv ? rla : 0.f);
      if (t < C) wG[(size_t)tile * C + t] = g;
    }
    // rows past the end of a ragged last chunk become zero columns
#pragma unroll
    for (int s2 = 0; s2 < tv.PT; ++s2)
      if ((int)(threadIdx.x + kThreads * s2) / tv.PR >= nv) tv.x[s2] = u32x4{0u, 0u, 0u, 0u};
    tv.store_T(sVt, LC);
    lds_barrier();
    load(min(tile + (int)gridDim.x, ntiles - 1));
    lds_to_block<E, DV, C>(wUt + (size_t)tile * DV * C, sVt, LC);
    lds_barrier();
  }
}

// --------------------------------------------------------------- launcher
// Whether every kernel of the Gated DeltaNet / Mamba2 training step (the
// training forward, the recompute, the reverse scan and the gradient kernel)
// fits in LDS at this chunk size.
template <typename E, int C, int DK, int DV>
constexpr bool gdn_bwd_fits() {
  return WyLds<E, C, DK, DV>::TOTAL <= kLdsMax && scan_bv<E, C, DK, DV, kScanFwd, false>() > 0 &&
         scan_bv<E, C, DK, DV, kScanBwd, false>() > 0 && dstate_bv<E, C, DK, DV, true>() > 0 &&
         GradLds<E, C, DK, DV, true>::TOTAL <= kLdsMax;
}
template <typename E, int C, int DK, int DV>
constexpr bool ssd_bwd_fits() {
  return scan_bv<E, C, DK, DV, kScanBwd, false>() > 0 && LocalLds<E, C, DK, DV>::TOTAL <= kLdsMax &&
         dstate_bv<E, C, DK, DV, true>() > 0 && dstate_bv<E, C, DK, DV, false>() > 0 &&
         GradLds<E, C, DK, DV, false>::TOTAL <= kLdsMax &&
         (size_t)DV * (C + lds_pad<E>()) * sizeof(E) <= kLdsMax;
}

// The forward quantities the gradient kernels read, recomputed: WY factors
// with T and P (k_wy), then the chunk-start states S_n and U (k_scan,
// backward mode).
template <typename E, int C, int DK, int DV>
void bwd_recompute(const BwdWs& ws, const void* q, const void* k, const void* v, const float* log_a,
                   const float* beta, const float* h0, const SeqMap& sm, int tiles, void* stream) {
  const int B = sm.B, H = sm.H;
  hipStream_t st = (hipStream_t)stream;
  constexpr int BV = scan_bv<E, C, DK, DV, kScanBwd, false>();  // state columns per workgroup
  LRT_LAUNCH(kKWyBwd, (k_wy<E, C, DK, DV, true, true, kWyWaves>),
             dim3(persistent_grid(tiles, WyLds<E, C, DK, DV>::TOTAL)), dim3(64 * kWyWaves), st, (const E*)q,
             (const E*)k, (const E*)v, log_a, beta, sm, (E*)ws.f.W, (E*)ws.f.Up, ws.f.G, (E*)ws.f.P, (E*)ws.T);
  ScanArgs<E> sa{};
  sa.k = (const E*)k;
  sa.W = (const E*)ws.f.W;
  sa.Up = (const E*)ws.f.Up;
  sa.G = ws.f.G;
  sa.hin = h0;
  sa.hs_ld = DV;
  sa.U = (E*)ws.f.U;
  sa.S = (E*)ws.f.S;
  sa.m = sm;
  sa.L = 1 << 30;
  sa.nseg = 1;
  sa.DV = DV;
  LRT_LAUNCH(kKScanBwd, (k_scan<E, C, DK, BV, kScanBwd, false, kStateWaves>), dim3(B * H * (DV / BV)),
             dim3(64 * kStateWaves), st, sa);
}

// saved: the workspace already holds W, g, T, P, S_n and U from
// gdn_fwd_train of the same arguments, so the recompute is skipped.  The
// reverse state scan forms dU_local = P^T dO from the stored P.
template <typename E, int C, int DK, int DV>
int bwd_impl(const BwdArgs& a, bool saved) {
  if constexpr (!gdn_bwd_fits<E, C, DK, DV>()) {
    return -3;  // not reached: the entry point runs a chunk that fits (bwd_max_chunk)
  } else {
    const bool packed = a.cu != nullptr;
    const int tiles = (int)ws_tiles(a.B, a.T, a.H, C, packed);
    const BwdWs ws = bwd_ws_layout(LRT_OP_GDN_BWD, a.B, a.T, a.H, DK, DV, C, sizeof(E), a.workspace, packed);
    const SeqMap sm = seq_map(a.B, a.T, a.H, C, a.cu, ws.f);
    hipStream_t st = (hipStream_t)a.stream;
    constexpr int BV = dstate_bv<E, C, DK, DV, true>();  // state columns per workgroup
    const int sgrid = a.B * a.H * (DV / BV);
    if (packed && launch_varlen_plan(a.cu, a.B, a.T, C, ws.f, a.stream) != 0) return -7;
    if (!saved) bwd_recompute<E, C, DK, DV>(ws, a.q, a.k, a.v, a.log_a, a.beta, a.h0, sm, tiles, a.stream);
    LRT_LAUNCH(kKDState, (k_dstate<E, C, DK, BV, kStateWaves, true, true>), dim3(sgrid), dim3(64 * kStateWaves), st,
               (const E*)a.q, (const E*)a.k, (const E*)a.d_o, ws.f.G, (const E*)ws.f.W, (const E*)ws.f.P, a.dht,
               a.dh0, (E*)ws.dS, (E*)ws.dU, sm, DV);
    LRT_LAUNCH(kKGrad, (k_grad<E, C, DK, DV, kGradWaves, true>),
               dim3(persistent_grid(tiles, GradLds<E, C, DK, DV, true>::TOTAL)), dim3(64 * kGradWaves), st,
               (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.d_o, a.beta, ws.f.G, (const E*)ws.f.S,
               (const E*)ws.dS, (const E*)ws.f.U, (const E*)ws.dU, (const E*)ws.T, (E*)a.dq, (E*)a.dk_out,
               (E*)a.dv_out, a.dlog_a, a.dbeta, sm);
    return hipGetLastError() == hipSuccess ? 0 : -7;
  }
}

// Mamba2 backward: the Gated DeltaNet pipeline without the WY transform
// (T = I, W = 0, U = V, no beta): prep (g, V^T), the state recompute
// (chunk-start states only), dU_local, the reverse state scan (dU = dV) and
// the gradient kernel writing dq, dk, dv and dlog_a.
// saved: the workspace holds S_n, g and P^T from ssd_fwd_train of the same
// arguments, so the prep, the state recompute and dU_local are skipped (the
// reverse scan forms dU_local from the stored P^T).
template <typename E, int C, int DK, int DV>
int ssd_bwd_impl(const BwdArgs& a, bool saved) {
  if constexpr (!ssd_bwd_fits<E, C, DK, DV>()) {
    return -3;  // not reached: the entry point runs a chunk that fits (bwd_max_chunk)
  } else {
    const int N = (a.T + C - 1) / C;
    const int tiles = a.B * a.H * N;
    const BwdWs ws = bwd_ws_layout(LRT_OP_SSD_BWD, a.B, a.T, a.H, DK, DV, C, sizeof(E), a.workspace);
    const SeqMap sm = seq_map(a.B, a.T, a.H, C, nullptr, ws.f);
    hipStream_t st = (hipStream_t)a.stream;
    if (!saved) {
      constexpr int BVS = scan_bv<E, C, DK, DV, kScanBwd, false>();
      E* Ut = (E*)ws.f.U;  // V^T, the scan's U'^T
      LRT_LAUNCH(kKSsdPrep, (k_ssd_prep<E, C, DV>),
                 dim3(persistent_grid(tiles, (size_t)DV * (C + lds_pad<E>()) * sizeof(E))), dim3(kThreads), st,
                 (const E*)a.v, a.log_a, ws.f.G, Ut, a.T, a.H, N, tiles);
      ScanArgs<E> sa{};
      sa.k = (const E*)a.k;
      sa.Up = Ut;
      sa.G = ws.f.G;
      sa.hin = a.h0;
      sa.hs_ld = DV;
      sa.S = (E*)ws.f.S;
      sa.m = sm;
      sa.L = 1 << 30;
      sa.nseg = 1;
      sa.DV = DV;
      LRT_LAUNCH(kKScanBwd, (k_scan<E, C, DK, BVS, kScanBwd, false, kStateWaves, false>), dim3(a.B * a.H * (DV / BVS)),
                 dim3(64 * kStateWaves), st, sa);
    }
    if (saved) {  // dU_local from the P^T the training forward stored
      constexpr int BV = dstate_bv<E, C, DK, DV, true>();
      LRT_LAUNCH(kKDState, (k_dstate<E, C, DK, BV, kStateWaves, false, true, true>), dim3(a.B * a.H * (DV / BV)),
                 dim3(64 * kStateWaves), st, (const E*)a.q, (const E*)a.k, (const E*)a.d_o, ws.f.G, (const E*)nullptr,
                 (const E*)ws.f.P, a.dht, a.dh0, (E*)ws.dS, (E*)ws.dU, sm, DV);
    } else {
      constexpr int BV = dstate_bv<E, C, DK, DV, false>();
      E* dUl = (E*)ws.f.Up;
      LRT_LAUNCH(kKBwdLocal, (k_bwd_local<E, C, DK, DV>), dim3(persistent_grid(tiles, LocalLds<E, C, DK, DV>::TOTAL)),
                 dim3(kThreads), st, (const E*)a.q, (const E*)a.k, (const E*)a.d_o, ws.f.G, dUl, a.T, a.H, N, tiles);
      LRT_LAUNCH(kKDState, (k_dstate<E, C, DK, BV, kStateWaves, false>), dim3(a.B * a.H * (DV / BV)),
                 dim3(64 * kStateWaves), st, (const E*)a.q, (const E*)a.k, (const E*)a.d_o, ws.f.G, (const E*)nullptr,
                 (const E*)dUl, a.dht, a.dh0, (E*)ws.dS, (E*)ws.dU, sm, DV);
    }
    LRT_LAUNCH(kKGrad, (k_grad<E, C, DK, DV, kGradWaves, false>),
               dim3(persistent_grid(tiles, GradLds<E, C, DK, DV, false>::TOTAL)), dim3(64 * kGradWaves), st,
               (const E*)a.q, (const E*)a.k, (const E*)nullptr, (const E*)a.d_o, (const float*)nullptr, ws.f.G,
               (const E*)ws.f.S, (const E*)ws.dS, (const E*)a.v, (const E*)ws.dU, (const E*)nullptr, (E*)a.dq,
               (E*)a.dk_out, (E*)a.dv_out, a.dlog_a, (float*)nullptr, sm);
    return hipGetLastError() == hipSuccess ? 0 : -7;
  }
}

// Gated DeltaNet forward for training: the forward (o, ht) written into the
// backward's workspace together with what the backward reads -- W, g, T and
// P from the WY pass, S_n and U from the scan -- so that gdn_bwd_saved skips
// the recompute and forms dU_local from the stored P.
template <typename E, int C, int DK, int DV>
int fwd_train_impl(const FwdArgs& a) {
  if constexpr (!gdn_bwd_fits<E, C, DK, DV>()) {
    return -3;  // not reached: the entry point runs a chunk that fits (bwd_max_chunk)
  } else {
    const BwdWs ws = bwd_ws_layout(LRT_OP_GDN_BWD, a.B, a.T, a.H, DK, DV, C, sizeof(E), a.workspace);
    const int N = (a.T + C - 1) / C;
    const int tiles = a.B * a.H * N;
    LRT_LAUNCH(kKWy, (k_wy<E, C, DK, DV, true, true, kWyWaves>),
               dim3(persistent_grid(tiles, WyLds<E, C, DK, DV>::TOTAL)), dim3(64 * kWyWaves), a.stream,
               (const E*)a.q, (const E*)a.k, (const E*)a.v, a.log_a, a.beta, seq_map(a, ws.f, C), (E*)ws.f.W,
               (E*)ws.f.Up, ws.f.G, (E*)ws.f.P, (E*)ws.T);
    if (hipGetLastError() != hipSuccess) return -7;
    return launch_scan_fwd<E, C, DK, DV, false, true>(a, ws.f, N);
  }
}

// Mamba2 forward for training: ssd_fwd's kernel also writing S_n, g and P^T
// into the backward's workspace for ssd_bwd_saved.
template <typename E, int C, int DK, int DV>
int fwd_ssd_train_impl(const FwdArgs& a) {
  if constexpr (!ssd_bwd_fits<E, C, DK, DV>()) {
    return -3;  // not reached: the entry point runs a chunk that fits (bwd_max_chunk)
  } else {
    const BwdWs ws = bwd_ws_layout(LRT_OP_SSD_BWD, a.B, a.T, a.H, DK, DV, C, sizeof(E), a.workspace);
    return launch_ssd_fwd<E, C, DK, DV, true>(a, (E*)ws.f.S, ws.f.G, (E*)ws.f.P);
  }
}

template <typename E, int DK, int DV>
constexpr int gdn_bwd_max_chunk_t() {
  return gdn_bwd_fits<E, 64, DK, DV>() ? 64 : gdn_bwd_fits<E, 32, DK, DV>() ? 32 : 16;
}
template <typename E, int DK, int DV>
constexpr int ssd_bwd_max_chunk_t() {
  return ssd_bwd_fits<E, 64, DK, DV>() ? 64 : ssd_bwd_fits<E, 32, DK, DV>() ? 32 : 16;
}

#define LRT_DV(DK_) LRT_CASE(DK_, 16) LRT_CASE(DK_, 32) LRT_CASE(DK_, 64) LRT_CASE(DK_, 128)
#define LRT_DK LRT_DV(16) LRT_DV(32) LRT_DV(64) LRT_DV(128)

int bwd_max_chunk(int op, int dtype, int dk, int dv) {
  const bool ssd = op == LRT_OP_SSD_BWD;
#define LRT_CASE(DK_, DV_)                                                                                     \
  if (dk == DK_ && dv == DV_) {                                                                                \
    if (dtype == LRT_BF16) return ssd ? ssd_bwd_max_chunk_t<bf16, DK_, DV_>() : gdn_bwd_max_chunk_t<bf16, DK_, DV_>(); \
    return ssd ? ssd_bwd_max_chunk_t<float, DK_, DV_>() : gdn_bwd_max_chunk_t<float, DK_, DV_>();              \
  }
  LRT_DK
#undef LRT_CASE
  return 16;
}

template <typename E>
static int fwd_train_dtype(const FwdArgs& a) {
#define LRT_CASE(DK_, DV_)                                                                           \
  if (a.dk == DK_ && a.dv == DV_) {                                                                  \
    if (a.chunk == 16)                                                                               \
      return a.variant == kVarSSD ? fwd_ssd_train_impl<E, 16, DK_, DV_>(a) : fwd_train_impl<E, 16, DK_, DV_>(a); \
    if (a.chunk == 32)                                                                               \
      return a.variant == kVarSSD ? fwd_ssd_train_impl<E, 32, DK_, DV_>(a) : fwd_train_impl<E, 32, DK_, DV_>(a); \
    if (a.chunk == 64)                                                                               \
      return a.variant == kVarSSD ? fwd_ssd_train_impl<E, 64, DK_, DV_>(a) : fwd_train_impl<E, 64, DK_, DV_>(a); \
  }
  LRT_DK
#undef LRT_CASE
  return -2;
}

int fwd_train(const FwdArgs& a) { return a.dtype == LRT_BF16 ? fwd_train_dtype<bf16>(a) : fwd_train_dtype<float>(a); }

template <typename E, bool SSD>
static int bwd_dtype(const BwdArgs& a, bool saved) {
#define LRT_CASE(DK_, DV_)                                                                                   \
  if (a.dk == DK_ && a.dv == DV_) {                                                                          \
    if (a.chunk == 16) return SSD ? ssd_bwd_impl<E, 16, DK_, DV_>(a, saved) : bwd_impl<E, 16, DK_, DV_>(a, saved); \
    if (a.chunk == 32) return SSD ? ssd_bwd_impl<E, 32, DK_, DV_>(a, saved) : bwd_impl<E, 32, DK_, DV_>(a, saved); \
    if (a.chunk == 64) return SSD ? ssd_bwd_impl<E, 64, DK_, DV_>(a, saved) : bwd_impl<E, 64, DK_, DV_>(a, saved); \
  }
  LRT_DK
#undef LRT_CASE
  return -2;
}
#undef LRT_DK
#undef LRT_DV

int bwd_gdn(const BwdArgs& a, bool saved) {
  return a.dtype == LRT_BF16 ? bwd_dtype<bf16, false>(a, saved) : bwd_dtype<float, false>(a, saved);
}
int bwd_ssd(const BwdArgs& a, bool saved) {
  return a.dtype == LRT_BF16 ? bwd_dtype<bf16, true>(a, saved) : bwd_dtype<float, true>(a, saved);
}

}  // namespace lrt
