// lrt_dstate.hpp -- the reverse state scan of the chunkwise backward
// (Gated DeltaNet, Mamba2 and KDA) on gfx950.
//
// Per chunk, walking the chunks of one (b, h, block of value columns) in
// reverse with the gradient of the chunk's end state dH' held in MFMA
// accumulators (AMD ROCm blog "Pretraining hybrid LLMs with Primus",
// section "How hybrid models are defined in Primus", mixer list under
// Table 2, differentiated through the chunkwise form):
//   dU = P^T dO + Ktil dH'
//   dH <- Decay dH' + Qd^T dO - W^T dU
// with Ktil, Qd and Decay the variant's decayed keys, queries and chunk
// decay (scalar for Gated DeltaNet and Mamba2, per key dimension for KDA).
#pragma once
#include "lrt_internal.hpp"

namespace lrt {


// LDS of k_dstate (its __shared__ arrays below), and the widest column
// block (at most 64 columns) whose arrays fit.
// KDA: Ktil^T [d][t] in place of the Ktil rows, no decayed dO copy, d_k gate floats.
template <int C, int DK, int LK, int LC, bool KDA>
constexpr int dstate_kt_elems() {
  return KDA ? (DK * LC > C * LK ? DK * LC : C * LK) : C * LK;
}
template <typename E, int C, int DK, int BV, bool READ_P, bool KDA = false>
constexpr size_t dstate_lds() {
  constexpr size_t P = lds_pad<E>(), LK = DK + P, LC = C + P, LB = BV + P;
  constexpr size_t KT = dstate_kt_elems<C, DK, (int)LK, (int)LC, KDA>(), OG = KDA ? 8 : C * LB;
  constexpr size_t NG = KDA && DK > C ? DK : C;
  return (2 * C * LK + KT + OG + BV * LC + BV * LK + (READ_P ? C * LC + C * LB : 16)) * sizeof(E) +
         (NG + 2 * C) * 4 + 160;
}
template <typename E, int C, int DK, int DV, bool READ_P, int cap = 64, bool KDA = false>
constexpr int dstate_bv() {
  constexpr int b0 = DV < cap ? DV : cap;
  if constexpr (dstate_lds<E, C, DK, b0, READ_P, KDA>() <= kLdsMax)
    return b0;
  else if constexpr (b0 > 16)
    return dstate_bv<E, C, DK, DV, READ_P, b0 / 2, KDA>();
  else
    return 0;
}

// ---------------------------------------------------------------- k_dstate
// Reverse scan over chunks for one (b, h, block of BV value columns), NW
// waves.  q, W and Ktil stay row-major in LDS; the products contracting over
// tokens read them with the LDS transpose read, so nothing is transposed by
// hand.  dH' and dU leave through LDS as coalesced 16-byte rows.
// DELTA = false is the Mamba2 recurrence (W = 0): dH <- gamma_C dH' +
// Q^T diag(gamma) dO, and dU is dV.
// READ_P: wdUl is the stored P = (Q K^T) o Gamma (rows [i][j] per chunk, zero
// above the diagonal; PT: stored transposed, rows [j][i]) and the kernel
// forms dU_local = P^T dO itself, in the phase that adds Ktil dH' (no
// separate dU_local pass).
// KDA (with READ_P): the decays are per key dimension and the operands come
// from the forward pass's workspace: q is Q o e^G rows [C][d_k], k is
// Ktil^T [d_k][C] (Ktil_j = k_j o e^(G_C - G_j)), wG the per-dimension chunk
// log-decay G_C [d_k]; dH <- Diag(e^(G_C)) dH' + (Q o e^G)^T dO - W^T dU.
template <typename E, int C, int DK, int BV, int NW = 8, bool DELTA = true, bool READ_P = false, bool PT = false,
          bool KDA = false>
__global__ __launch_bounds__(64 * NW) void k_dstate(const E* __restrict__ q, const E* __restrict__ k,
                                                    const E* __restrict__ d_o, const float* __restrict__ wG,
                                                    const E* __restrict__ wW, const E* __restrict__ wdUl,
                                                    const float* dht, float* dh0, E* __restrict__ wdS,
                                                    E* __restrict__ wdU, SeqMap m, int DV) {
  constexpr int NT = 64 * NW;
  constexpr int P = lds_pad<E>();
  constexpr int LK = DK + P, LC = C + P, LB = BV + P;
  constexpr int NTV = BV / 16;
  constexpr int NH = (DK / 16) * NTV, HPW = (NH + NW - 1) / NW;
  constexpr int NU = (C / 16) * NTV, UPW = (NU + NW - 1) / NW;
  static_assert(!KDA || (READ_P && DELTA && !PT), "the KDA reverse scan reads the stored P");
  // When every wave holds the same number of tiles of one column block, a
  // wave's bf16 products read the fragment its tiles share once per k step
  // (fp32 operands are read per 16-long k step either way).
  constexpr bool kShU = sizeof(E) == 2 && NU % NW == 0 && NW % NTV == 0;
  constexpr bool kShH = sizeof(E) == 2 && NH % NW == 0 && NW % NTV == 0;
  __shared__ __attribute__((aligned(16))) E sQ[C * LK];    // q rows (KDA: Q o e^G rows)
  __shared__ __attribute__((aligned(16))) E sW[C * LK];    // W rows
  __shared__ __attribute__((aligned(16))) E sKt[dstate_kt_elems<C, DK, LK, LC, KDA>()];  // Ktil rows (KDA: Ktil^T)
  __shared__ __attribute__((aligned(16))) E sOg[KDA ? 8 : C * LB];  // gamma_t dO rows (this block's columns)
  __shared__ __attribute__((aligned(16))) E sdU[BV * LC];  // dU^T
  __shared__ __attribute__((aligned(16))) E sdS[BV * LK];  // dH'^T
  __shared__ __attribute__((aligned(16))) E sP[READ_P ? C * LC : 8];  // P rows [i][j]
  __shared__ __attribute__((aligned(16))) E sO[READ_P ? C * LB : 8];  // dO rows (this block's columns)
  __shared__ __attribute__((aligned(16))) float sg[KDA && DK > C ? DK : C];  // g (KDA: e^(G_C) per key dimension)
  __shared__ float sgs[2 * C];

  const int nvb = DV / BV;
  const int wg = xcd_group(blockIdx.x, gridDim.x);  // the d_v blocks of one (b, h) share an L2
  const int vb = wg % nvb, bh = wg / nvb;
  const SeqPos sp = seq_pos(m, bh);
  const int H = m.H, h = sp.h, v0 = vb * BV;
  const int w = wave_id(), l = lane_id();

  f32x4 hacc[HPW];
#pragma unroll
  for (int s = 0; s < HPW; ++s) {
    const int tt = w + NW * s;
    hacc[s] = zero4();
    if (tt < NH && dht != nullptr) {
      const int td = tt / NTV, tv = tt % NTV;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        hacc[s][r] = dht[((size_t)bh * DK + td * 16 + (l >> 4) * 4 + r) * DV + v0 + tv * 16 + (l & 15)];
    }
  }

  Tile<E, C, DK, NT> tQ, tW;
  Tile<E, KDA ? DK : C, KDA ? C : DK, NT> tK;
  Tile<E, C, BV, NT> tO;
  Tile<E, C, C, NT> tP;
  typename Vec4<E>::T rU[UPW];  // packed: unpacked where used, so the fetch does not wait
  float rg = 0.f;
  // The previous chunk's operands, fetched in two parts while this chunk
  // runs (the registers of each part are free once stored or scaled), with
  // clamped rows and chunk index so no load sits behind a branch.
#define LRT_DSTATE_FETCH(n_, PART_)                                                                 \
  {                                                                                                 \
    const size_t ft = sp.tile0 + (n_);                                                              \
    const int fnv = min(C, sp.len - (n_) * C);                                                      \
    const size_t ftok = sp.tok0 + (size_t)(n_) * C;                                                 \
    if ((PART_) & 1) {                                                                              \
      if constexpr (KDA)                                                                            \
        tQ.load_block(q + ft * C * DK);                                                             \
      else                                                                                          \
        tQ.load_rows_clamped(q + (ftok * H + h) * DK, (size_t)H * DK, fnv);                         \
      if constexpr (DELTA) tW.load_block(wW + ft * C * DK);                                         \
      if constexpr (READ_P) {                                                                       \
        tP.load_block(wdUl + ft * C * C);                                                           \
      } else {                                                                                      \
        _Pragma("unroll") for (int s = 0; s < UPW; ++s) {                                           \
          const int tt = min(w + NW * s, NU - 1);                                                   \
          rU[s] = load4_raw<E>(wdUl + ft * DV * C + (size_t)(v0 + (tt % NTV) * 16 + (l & 15)) * C + \
                               (tt / NTV) * 16 + (l >> 4) * 4);                                     \
        }                                                                                           \
      }                                                                                             \
      if constexpr (KDA)                                                                            \
        rg = wG[ft * DK + min((int)threadIdx.x, DK - 1)];                                           \
      else                                                                                          \
        rg = wG[ft * C + min((int)threadIdx.x, C - 1)];                                             \
    }                                                                                               \
    if ((PART_) & 2) {                                                                              \
      if constexpr (KDA)                                                                            \
        tK.load_block(k + ft * DK * C);                                                             \
      else                                                                                          \
        tK.load_rows_clamped(k + (ftok * H + h) * DK, (size_t)H * DK, fnv);                         \
      tO.load_rows_clamped(d_o + (ftok * H + h) * DV + v0, (size_t)H * DV, fnv);                    \
    }                                                                                               \
  }

  if (sp.nch > 0) LRT_DSTATE_FETCH(sp.nch - 1, 3)
  for (int n = sp.nch - 1; n >= 0; --n) {
    const size_t tile = sp.tile0 + n;
    const int nv = min(C, sp.len - n * C);
    const int nprev = n > 0 ? n - 1 : 0;
    // gates: g, e^(g_C - g_t), gamma_t (wave 0 holds g of this chunk, one token per lane)
    asm volatile("" ::"v"(rg));
    if constexpr (KDA) {
      if (threadIdx.x < DK) sg[threadIdx.x] = __expf(rg);
    } else if (threadIdx.x < 64) {
      const float gC = __shfl(rg, C - 1, 64);
      if (threadIdx.x < C) {
        sg[threadIdx.x] = rg;
        sgs[threadIdx.x] = __expf(gC - rg);
        sgs[C + threadIdx.x] = __expf(rg);
      }
    }
    // dH' (gradient of this chunk's end state) -> LDS as [v][d]
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + NW * s;
      if (tt < NH) {
        const int td = tt / NTV, tv = tt % NTV;
        store4<E>(sdS + (tv * 16 + (l & 15)) * LK + td * 16 + (l >> 4) * 4, hacc[s]);
      }
    }
    tQ.store_masked(sQ, LK, nv);
    if constexpr (DELTA) tW.store(sW, LK);
    f32x4 du[UPW];
    if constexpr (READ_P) {
      tP.store(sP, LC);
    } else {
#pragma unroll
      for (int s = 0; s < UPW; ++s) du[s] = Vec4<E>::unpack(rU[s]);
    }
    lds_barrier();
    LRT_DSTATE_FETCH(nprev, 1)
    lds_to_block<E, BV, DK, NT>(wdS + (tile * DV + v0) * DK, sdS, LK);
    if constexpr (KDA) {
      tK.store(sKt, LC);
      tO.store_masked(sO, LB, nv);
    } else {
      tK.scale_rows(sgs);
      tK.store_masked(sKt, LK, nv);
      if constexpr (READ_P) tO.store_masked(sO, LB, nv);
      tO.scale_rows(sgs + C);
      tO.store_masked(sOg, LB, nv);
    }
    const float dec = KDA ? 0.f : __expf(sg[C - 1]);
    const E* og = KDA ? sO : sOg;  // the dO rows the state gradient contracts with
    lds_barrier();
    LRT_DSTATE_FETCH(nprev, 2)
    // dU = dU_local + Ktil dH'  (rows t, cols v) -> dU^T
    if constexpr (kShU) {
      const int ti0 = w / NTV, tv = w % NTV;
      constexpr int AS = (NW / NTV) * 16;
      f32x4 acc[UPW];
#pragma unroll
      for (int s = 0; s < UPW; ++s) acc[s] = READ_P ? zero4() : du[s];
      if constexpr (READ_P && PT)
        mma_nA<C, UPW, false, true>(acc, sP + ti0 * 16 * LC, AS * LC, LC, sO + tv * 16, LB);
      else if constexpr (READ_P)
        mma_nA<C, UPW, true, true>(acc, sP + ti0 * 16, AS, LC, sO + tv * 16, LB);
      if constexpr (KDA)
        mma_nA<DK, UPW, true, false>(acc, sKt + ti0 * 16, AS, LC, sdS + tv * 16 * LK, LK);
      else
        mma_nA<DK, UPW>(acc, sKt + ti0 * 16 * LK, AS * LK, LK, sdS + tv * 16 * LK, LK);
#pragma unroll
      for (int s = 0; s < UPW; ++s)
        store4<E>(sdU + (tv * 16 + (l & 15)) * LC + (ti0 + (NW / NTV) * s) * 16 + (l >> 4) * 4, acc[s]);
    }
#pragma unroll
    for (int s = 0; s < (kShU ? 0 : UPW); ++s) {
      const int tt = w + NW * s;
      if (tt < NU) {
        const int ti = tt / NTV, tv = tt % NTV;
        f32x4 acc;
        if constexpr (READ_P) {
          acc = zero4();
          if constexpr (PT)
            mma<C, false, true>(acc, sP + ti * 16 * LC, LC, sO + tv * 16, LB);  // dU_local = P^T dO
          else
            mma<C, true, true>(acc, sP + ti * 16, LC, sO + tv * 16, LB);
        } else {
          acc = du[s];
        }
        if constexpr (KDA)
          mma<DK, true, false>(acc, sKt + ti * 16, LC, sdS + tv * 16 * LK, LK);
        else
          mma<DK>(acc, sKt + ti * 16 * LK, LK, sdS + tv * 16 * LK, LK);
        store4<E>(sdU + (tv * 16 + (l & 15)) * LC + ti * 16 + (l >> 4) * 4, acc);
      }
    }
    lds_barrier();
    lds_to_block<E, BV, C, NT>(wdU + (tile * DV + v0) * C, sdU, LC);
    // dH <- gamma_C dH' + Q^T diag(gamma) dO - W^T dU
    if constexpr (kShH) {
      const int td0 = w / NTV, tv = w % NTV;
      constexpr int AS = (NW / NTV) * 16;
#pragma unroll
      for (int s = 0; s < HPW; ++s) {
        if constexpr (KDA)
          hacc[s] *= *(const f32x4*)(sg + (td0 + (NW / NTV) * s) * 16 + (l >> 4) * 4);
        else
          hacc[s] *= dec;
      }
      mma_nA<C, HPW, true, true>(hacc, sQ + td0 * 16, AS, LK, og + tv * 16, LB);
      if constexpr (DELTA) {
        f32x4 wdu[HPW];
#pragma unroll
        for (int s = 0; s < HPW; ++s) wdu[s] = zero4();
        mma_nA<C, HPW, true, false>(wdu, sW + td0 * 16, AS, LK, sdU + tv * 16 * LC, LC);
#pragma unroll
        for (int s = 0; s < HPW; ++s) hacc[s] -= wdu[s];
      }
    }
#pragma unroll
    for (int s = 0; s < (kShH ? 0 : HPW); ++s) {
      const int tt = w + NW * s;
      if (tt < NH) {
        const int td = tt / NTV, tv = tt % NTV;
        if constexpr (KDA)
          hacc[s] *= *(const f32x4*)(sg + td * 16 + (l >> 4) * 4);
        else
          hacc[s] *= dec;
        mma<C, true, true>(hacc[s], sQ + td * 16, LK, og + tv * 16, LB);
        if constexpr (DELTA) {
          f32x4 wdu = zero4();
          mma<C, true, false>(wdu, sW + td * 16, LK, sdU + tv * 16 * LC, LC);
          hacc[s] -= wdu;
        }
      }
    }
    lds_barrier();
  }
#undef LRT_DSTATE_FETCH
  if (dh0 != nullptr) {
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + NW * s;
      if (tt < NH) {
        const int td = tt / NTV, tv = tt % NTV;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          dh0[((size_t)bh * DK + td * 16 + (l >> 4) * 4 + r) * DV + v0 + tv * 16 + (l & 15)] = hacc[s][r];
      }
    }
  }
}

}  // namespace lrt
