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
// Kernels (256 threads each), in stream order:
//   k_prep (WRITE_T) / k_state   recompute W, U', Ktil, Tinv, S_n and U
//   k_bwd_local  per chunk: dU_local = P^T dO
//   k_dstate     per (b, h, d_v block), chunks in reverse: dU and dH'
//   k_grad1      per chunk: dQ, the dS/state part of dK, dW, part of dg
//   k_grad2      per chunk: the WY part of dK, dV, dbeta, dg -> dlog_a
#include "lrt_fwd_kernels.hpp"
#include "lrt_internal.hpp"

namespace lrt {

// Backward-only workspace tiles, after the forward's (chunk-major per (b, h)):
//   T   [C][C]   E    Tinv
//   dS  [dv][dk] E    dH'^T, gradient of each chunk's end state
//   dU  [dv][C]  E    dU^T
//   dW  [C][dk]  E    dW
//   dK1 [C][dk]  f32  the dS / state part of dK
//   dg1 [C]      f32  part of dg
// dU_local reuses the forward's U' tiles (dead once the state pass has run).
struct BwdWs {
  FwdWs f;
  void *T, *dS, *dU, *dW;
  float *dK1, *dg1;
  size_t bytes;
};

static BwdWs bwd_ws_layout(int B, int T, int H, int dk, int dv, int C, size_t esz, void* base) {
  BwdWs w;
  w.f = fwd_ws_layout(B, T, H, dk, dv, C, esz, base);
  const size_t tiles = (size_t)B * H * ((size_t)(T + C - 1) / C);
  size_t off = w.f.bytes;
  char* p = (char*)base;
  auto take = [&](size_t bytes) {
    void* r = p ? (void*)(p + off) : nullptr;
    off += align256(bytes);
    return r;
  };
  w.T = take(tiles * C * C * esz);
  w.dS = take(tiles * dv * dk * esz);
  w.dU = take(tiles * dv * C * esz);
  w.dW = take(tiles * C * dk * esz);
  w.dK1 = (float*)take(tiles * C * dk * sizeof(float));
  w.dg1 = (float*)take(tiles * C * sizeof(float));
  w.bytes = off;
  return w;
}

size_t bwd_ws_extra(int B, int T, int H, int dk, int dv, int C, size_t esz) {
  const BwdWs w = bwd_ws_layout(B, T, H, dk, dv, C, esz, nullptr);
  return w.bytes - w.f.bytes;
}

// ------------------------------------------------------------- k_bwd_local
// dU_local = P^T dO with P = (Q K^T) o Gamma (inclusive), stored as [v][t].
template <typename E, int C, int DK, int DV>
__global__ __launch_bounds__(kThreads) void k_bwd_local(const E* __restrict__ q, const E* __restrict__ k,
                                                        const E* __restrict__ d_o, const float* __restrict__ wG,
                                                        E* __restrict__ wdUl, int T, int H, int N) {
  constexpr int P = lds_pad<E>();
  constexpr int LK = DK + P, LC = C + P, NB = C / 16;
  constexpr int V = 16 / (int)sizeof(E);
  __shared__ float sg[C];
  __shared__ __attribute__((aligned(16))) E sQ[C * LK];
  __shared__ __attribute__((aligned(16))) E sK[C * LK];
  __shared__ __attribute__((aligned(16))) E sdOt[DV * LC];
  __shared__ __attribute__((aligned(16))) E sPt[C * LC];

  const int tile = blockIdx.x;
  const int n = tile % N, bh = tile / N, h = bh % H, b = bh / H;
  const int t0 = n * C, nv = min(C, T - t0);
  const size_t tok0 = (size_t)b * T + t0;
  const int w = wave_id(), l = lane_id();

  {
    Tile<E, C, DK> tq, tk;
    Tile<E, C, DV> to;
    tq.load_rows(q + (tok0 * H + h) * DK, (size_t)H * DK, nv);
    tk.load_rows(k + (tok0 * H + h) * DK, (size_t)H * DK, nv);
    to.load_rows(d_o + (tok0 * H + h) * DV, (size_t)H * DV, nv);
    if (threadIdx.x < C) sg[threadIdx.x] = wG[(size_t)tile * C + threadIdx.x];
    tq.store(sQ, LK);
    tk.store(sK, LK);
    to.store_T(sdOt, LC);
  }
  __syncthreads();
  for (int tt = w; tt < NB * NB; tt += kWaves) {
    const int ti = tt / NB, tj = tt % NB;
    f32x4 acc = zero4();
    if (tj <= ti) mma<DK>(acc, sQ + ti * 16 * LK, LK, sK + tj * 16 * LK, LK);
    const int j = tj * 16 + (l & 15), i0 = ti * 16 + (l >> 4) * 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = (j <= i0 + r) ? acc[r] * __expf(sg[i0 + r] - sg[j]) : 0.f;
    store4<E>(sPt + j * LC + i0, acc);
  }
  __syncthreads();
  for (int tt = w; tt < NB * (DV / 16); tt += kWaves) {
    const int tj = tt / (DV / 16), tv = tt % (DV / 16);
    f32x4 acc = zero4();
    mma<C>(acc, sPt + tj * 16 * LC, LC, sdOt + tv * 16 * LC, LC);
    store4<E>(wdUl + (size_t)tile * DV * C + (size_t)(tv * 16 + (l & 15)) * C + tj * 16 + (l >> 4) * 4, acc);
  }
}

// ---------------------------------------------------------------- k_dstate
// Reverse scan over chunks for one (b, h, block of BV value columns).
template <typename E, int C, int DK, int BV>
__global__ __launch_bounds__(kThreads) void k_dstate(const E* __restrict__ q, const E* __restrict__ k,
                                                     const E* __restrict__ d_o, const float* __restrict__ wG,
                                                     const E* __restrict__ wW, const E* __restrict__ wdUl,
                                                     const float* dht, float* dh0, E* __restrict__ wdS,
                                                     E* __restrict__ wdU, int T, int H, int N, int DV) {
  constexpr int P = lds_pad<E>();
  constexpr int LK = DK + P, L2 = 2 * C + P;
  constexpr int V = 16 / (int)sizeof(E);
  constexpr int NTV = BV / 16;
  constexpr int NH = (DK / 16) * NTV, HPW = (NH + kWaves - 1) / kWaves;
  constexpr int NU = (C / 16) * NTV, UPW = (NU + kWaves - 1) / kWaves;
  constexpr int PR = DK / V;                      // 16-byte pieces per row of q, k, W
  constexpr int NQ = C * PR, PQ = (NQ + kThreads - 1) / kThreads;
  constexpr int PRO = BV / V, NO = C * PRO, PO = (NO + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) E sA2[DK * L2];  // [d][t] = Q^T | [d][C+t] = W^T
  __shared__ __attribute__((aligned(16))) E sB2[BV * L2];  // [v][t] = (gamma dO)^T | [v][C+t] = -dU^T
  __shared__ __attribute__((aligned(16))) E sKt[C * LK];   // Ktil, row-major
  __shared__ __attribute__((aligned(16))) E sdS[BV * LK];  // dH'^T
  __shared__ float sg[C];
  __shared__ float sgs[2 * C];

  const int nvb = DV / BV;
  const int vb = blockIdx.x % nvb, bh = blockIdx.x / nvb;
  const int b = bh / H, h = bh % H, v0 = vb * BV;
  const int w = wave_id(), l = lane_id();

  f32x4 hacc[HPW];
#pragma unroll
  for (int s = 0; s < HPW; ++s) {
    const int tt = w + kWaves * s;
    hacc[s] = zero4();
    if (tt < NH && dht != nullptr) {
      const int td = tt / NTV, tv = tt % NTV;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        hacc[s][r] = dht[((size_t)bh * DK + td * 16 + (l >> 4) * 4 + r) * DV + v0 + tv * 16 + (l & 15)];
    }
  }

  Tile<E, C, DK> tQ, tK, tW;
  Tile<E, C, BV> tO;
  f32x4 rU[UPW];
  float rg = 0.f;
#define LRT_DSTATE_FETCH(n_)                                                                        \
  {                                                                                                 \
    const size_t ft = (size_t)bh * N + (n_);                                                        \
    const int fnv = min(C, T - (n_) * C);                                                           \
    const size_t ftok = (size_t)b * T + (size_t)(n_) * C;                                           \
    tQ.load_rows(q + (ftok * H + h) * DK, (size_t)H * DK, fnv);                                     \
    tK.load_rows(k + (ftok * H + h) * DK, (size_t)H * DK, fnv);                                     \
    tW.load_block(wW + ft * C * DK);                                                                \
    tO.load_rows(d_o + (ftok * H + h) * DV + v0, (size_t)H * DV, fnv);                              \
    _Pragma("unroll") for (int s = 0; s < UPW; ++s) {                                               \
      const int tt = w + kWaves * s;                                                                \
      if (tt < NU)                                                                                  \
        rU[s] = load4<E>(wdUl + ft * DV * C + (size_t)(v0 + (tt % NTV) * 16 + (l & 15)) * C +      \
                         (tt / NTV) * 16 + (l >> 4) * 4);                                           \
    }                                                                                               \
    rg = threadIdx.x < C ? wG[ft * C + threadIdx.x] : 0.f;                                          \
  }

  LRT_DSTATE_FETCH(N - 1)
  for (int n = N - 1; n >= 0; --n) {
    const size_t tile = (size_t)bh * N + n;
    if (threadIdx.x < C) sg[threadIdx.x] = rg;
    // dH' (gradient of this chunk's end state) -> LDS and workspace, as [v][d]
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + kWaves * s;
      if (tt < NH) {
        const int td = tt / NTV, tv = tt % NTV;
        const int vv = tv * 16 + (l & 15), d = td * 16 + (l >> 4) * 4;
        store4<E>(sdS + vv * LK + d, hacc[s]);
        store4<E>(wdS + tile * DV * DK + (size_t)(v0 + vv) * DK + d, hacc[s]);
      }
    }
    __syncthreads();
    const float gC = sg[C - 1];
    tQ.store_T(sA2, L2);
    tW.store_T(sA2 + C, L2);
    {
      float* sc = sgs;  // e^(g_C - g_t) and gamma_t, per token
      if (threadIdx.x < C) {
        sc[threadIdx.x] = __expf(gC - sg[threadIdx.x]);
        sc[C + threadIdx.x] = __expf(sg[threadIdx.x]);
      }
    }
    f32x4 du[UPW];
#pragma unroll
    for (int s = 0; s < UPW; ++s) du[s] = rU[s];
    __syncthreads();
    tK.scale_rows(sgs);
    tK.store(sKt, LK);
    tO.scale_rows(sgs + C);
    tO.store_T(sB2, L2);
    if (n > 0) LRT_DSTATE_FETCH(n - 1)
    __syncthreads();
    // dU = dU_local + Ktil dH'  (rows t, cols v)
#pragma unroll
    for (int s = 0; s < UPW; ++s) {
      const int tt = w + kWaves * s;
      if (tt < NU) {
        const int ti = tt / NTV, tv = tt % NTV;
        const int vv = tv * 16 + (l & 15), t = ti * 16 + (l >> 4) * 4;
        f32x4 acc = du[s];
        mma<DK>(acc, sKt + ti * 16 * LK, LK, sdS + tv * 16 * LK, LK);
        store4<E>(wdU + tile * DV * C + (size_t)(v0 + vv) * C + t, acc);
        store4<E>(sB2 + vv * L2 + C + t, -acc);
      }
    }
    __syncthreads();
    // dH <- gamma_C dH' + Q^T diag(gamma) dO - W^T dU
    const float dec = __expf(gC);
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + kWaves * s;
      if (tt < NH) {
        const int td = tt / NTV, tv = tt % NTV;
        hacc[s] *= dec;
        mma<2 * C>(hacc[s], sA2 + td * 16 * L2, L2, sB2 + tv * 16 * L2, L2);
      }
    }
    __syncthreads();
  }
#undef LRT_DSTATE_FETCH
  if (dh0 != nullptr) {
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + kWaves * s;
      if (tt < NH) {
        const int td = tt / NTV, tv = tt % NTV;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          dh0[((size_t)bh * DK + td * 16 + (l >> 4) * 4 + r) * DV + v0 + tv * 16 + (l & 15)] = hacc[s][r];
      }
    }
  }
}

// ----------------------------------------------------------------- k_grad1
// Per chunk: dS, dQ (final), dW, the dS^T Q + Ktil-path part of dK (fp32),
// and the Gamma / output / Ktil / gamma_C parts of dg.
template <typename E, int C, int DK, int DV>
struct Grad1Lds {
  static constexpr int P = lds_pad<E>();
  static constexpr int LK = DK + P, LV = DV + P, LC = C + P;
  static constexpr size_t sTK = (size_t)C * LK * sizeof(E), sTV = (size_t)C * LV * sizeof(E);
  static constexpr size_t sDC = (size_t)DK * LC * sizeof(E), sCC = (size_t)C * LC * sizeof(E);
  static constexpr size_t sDV = (size_t)DK * LV * sizeof(E);
  static constexpr size_t R1 = 0;                                    // Q, later dU (rows t)
  static constexpr size_t R23 = R1 + (sTK > sTV ? sTK : sTV);        // K, later Hn / dH' [d][v]
  static constexpr size_t DO = R23 + (sTK > sDV ? sTK : sDV);
  static constexpr size_t U = DO + sTV;
  static constexpr size_t QT = U + sTV;
  static constexpr size_t KT = QT + sDC;
  static constexpr size_t DSIJ = KT + sDC;
  static constexpr size_t DSJI = DSIJ + sCC;
  static constexpr size_t G = DSJI + sCC;
  static constexpr size_t DG = G + C * sizeof(float);
  static constexpr size_t DOT = DG + C * sizeof(float);
  static constexpr size_t TOTAL = DOT + 16;
};

template <typename E, int C, int DK, int DV>
__global__ __launch_bounds__(kThreads) void k_grad1(const E* __restrict__ q, const E* __restrict__ k,
                                                    const E* __restrict__ d_o, const float* __restrict__ wG,
                                                    const E* __restrict__ wS, const E* __restrict__ wdS,
                                                    const E* __restrict__ wU, const E* __restrict__ wdU,
                                                    E* __restrict__ dq, E* __restrict__ wdW,
                                                    float* __restrict__ wdK1, float* __restrict__ wdg1, int T,
                                                    int H, int N) {
  typedef Grad1Lds<E, C, DK, DV> Lay;
  constexpr int LK = Lay::LK, LV = Lay::LV, LC = Lay::LC, NB = C / 16;
  constexpr int V = 16 / (int)sizeof(E);
  __shared__ __attribute__((aligned(16))) char smem[Lay::TOTAL];
  E* sQ = (E*)(smem + Lay::R1);
  E* sK = (E*)(smem + Lay::R23);
  E* sdO = (E*)(smem + Lay::DO);
  E* sU = (E*)(smem + Lay::U);
  E* sQt = (E*)(smem + Lay::QT);
  E* sKt = (E*)(smem + Lay::KT);
  E* sdSij = (E*)(smem + Lay::DSIJ);
  E* sdSji = (E*)(smem + Lay::DSJI);
  float* sg = (float*)(smem + Lay::G);
  float* sdg = (float*)(smem + Lay::DG);
  float* sdot = (float*)(smem + Lay::DOT);

  const int tile = blockIdx.x;
  const int n = tile % N, bh = tile / N, h = bh % H, b = bh / H;
  const int t0 = n * C, nv = min(C, T - t0);
  const size_t tok0 = (size_t)b * T + t0;
  const int w = wave_id(), l = lane_id();

  Tile<E, C, DK> tq, tk;
  {
    Tile<E, C, DV> to;
    Tile<E, DV, C> tu;
    tq.load_rows(q + (tok0 * H + h) * DK, (size_t)H * DK, nv);
    tk.load_rows(k + (tok0 * H + h) * DK, (size_t)H * DK, nv);
    to.load_rows(d_o + (tok0 * H + h) * DV, (size_t)H * DV, nv);
    tu.load_block(wU + (size_t)tile * DV * C);
    if (threadIdx.x < C) {
      sg[threadIdx.x] = wG[(size_t)tile * C + threadIdx.x];
      sdg[threadIdx.x] = 0.f;
    }
    if (threadIdx.x == 0) sdot[0] = 0.f;
    tq.store(sQ, LK);
    tk.store(sK, LK);
    to.store(sdO, LV);
    tu.store_T(sU, LV);
  }
  __syncthreads();
  // states, state gradients and dU of this chunk: in flight during dS
  Tile<E, DV, DK> tS, tdS;
  Tile<E, DV, C> tdU;
  tS.load_block(wS + (size_t)tile * DV * DK);
  tdS.load_block(wdS + (size_t)tile * DV * DK);
  tdU.load_block(wdU + (size_t)tile * DV * C);

  // dS = (dO U^T) o Gamma (inclusive); E = dS o (Q K^T) -> dg rows +, cols -
  for (int tt = w; tt < NB * NB; tt += kWaves) {
    const int ti = tt / NB, tj = tt % NB;
    const int j = tj * 16 + (l & 15), i0 = ti * 16 + (l >> 4) * 4;
    f32x4 ds = zero4();
    if (tj <= ti) {
      f32x4 qk = zero4(), dp = zero4();
      mma<DK>(qk, sQ + ti * 16 * LK, LK, sK + tj * 16 * LK, LK);
      mma<DV>(dp, sdO + ti * 16 * LV, LV, sU + tj * 16 * LV, LV);
      float ecol = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + r;
        ds[r] = (j <= i) ? dp[r] * __expf(sg[i] - sg[j]) : 0.f;
        const float e = ds[r] * qk[r];
        ecol += e;
        const float er = sum16(e);
        if ((l & 15) == 0) atomicAdd(&sdg[i], er);
      }
      ecol = sum4(ecol);
      if (l < 16) atomicAdd(&sdg[j], -ecol);
    }
    store4<E>(sdSji + j * LC + i0, ds);
#pragma unroll
    for (int r = 0; r < 4; ++r) sdSij[(i0 + r) * LC + j] = from_f<E>(ds[r]);
  }
  // Q^T, K^T from the registers still holding q and k
  tq.store_T(sQt, LC);
  tk.store_T(sKt, LC);
  __syncthreads();
  // Hn [d][v] into R23, dU [t][v] into R1; <dH', Hn> from the same registers
  E* sH = (E*)(smem + Lay::R23);
  E* sdU = (E*)(smem + Lay::R1);
  tS.store_T(sH, LV);
  tdU.store_T(sdU, LV);
  {
    float part = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < tS.PT; ++s2) {
      if (threadIdx.x + kThreads * s2 < tS.NP) {
        E a[V], d[V];
        __builtin_memcpy(a, &tS.x[s2], 16);
        __builtin_memcpy(d, &tdS.x[s2], 16);
#pragma unroll
        for (int e = 0; e < V; ++e) part += to_f(a[e]) * to_f(d[e]);
      }
    }
    part = sum16(part);
    part = sum4(part);
    if (l == 0) atomicAdd(sdot, part);
  }
  __syncthreads();
  // dQ^T = gamma (Hn dO^T) + K^T dS^T  (rows d, cols i);  dW^T = -Hn dU^T
  for (int tt = w; tt < (DK / 16) * NB; tt += kWaves) {
    const int td = tt / NB, ti = tt % NB;
    const int i = ti * 16 + (l & 15), d0 = td * 16 + (l >> 4) * 4;
    f32x4 acc = zero4();
    mma<DV>(acc, sH + td * 16 * LV, LV, sdO + ti * 16 * LV, LV);
    const float gam = __expf(sg[i]);
    float e = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) e += to_f(sQt[(d0 + r) * LC + i]) * acc[r];
    e = sum4(e * gam);
    if (l < 16) atomicAdd(&sdg[i], e);
    acc *= gam;
    mma<C>(acc, sKt + td * 16 * LC, LC, sdSij + ti * 16 * LC, LC);
    if (i < nv) store4<E>(dq + ((tok0 + i) * H + h) * DK + d0, acc);
    f32x4 dw = zero4();
    mma<DV>(dw, sH + td * 16 * LV, LV, sdU + ti * 16 * LV, LV);
    store4<E>(wdW + (size_t)tile * C * DK + (size_t)i * DK + d0, -dw);
  }
  __syncthreads();
  // dH' [d][v] into R23
  E* sdH = (E*)(smem + Lay::R23);
  tdS.store_T(sdH, LV);
  __syncthreads();
  // dK1^T = e^(g_C - g_j) (dH' U^T) + Q^T dS   (rows d, cols j)
  const float gC = sg[C - 1];
  for (int tt = w; tt < (DK / 16) * NB; tt += kWaves) {
    const int td = tt / NB, tj = tt % NB;
    const int j = tj * 16 + (l & 15), d0 = td * 16 + (l >> 4) * 4;
    f32x4 acc = zero4();
    mma<DV>(acc, sdH + td * 16 * LV, LV, sU + tj * 16 * LV, LV);
    const float kt = __expf(gC - sg[j]);
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) s += acc[r] * to_f(sKt[(d0 + r) * LC + j]);
    s = sum4(s * kt);
    if (l < 16) {
      atomicAdd(&sdg[j], -s);
      atomicAdd(&sdg[C - 1], s);
    }
    acc *= kt;
    mma<C>(acc, sQt + td * 16 * LC, LC, sdSji + tj * 16 * LC, LC);
    *(float4*)(wdK1 + (size_t)tile * C * DK + (size_t)j * DK + d0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  }
  __syncthreads();
  if (threadIdx.x < C) {
    float x = sdg[threadIdx.x];
    if (threadIdx.x == C - 1) x += __expf(gC) * sdot[0];
    wdg1[(size_t)tile * C + threadIdx.x] = x;
  }
}

// ----------------------------------------------------------------- k_grad2
// Per chunk: the WY part of the gradient (through Tinv, W = Tinv X, U' = Tinv Y
// and A), dV, dbeta and dlog_a.
template <typename E, int C, int DK, int DV>
struct Grad2Lds {
  static constexpr int P = lds_pad<E>();
  static constexpr int LK = DK + P, LV = DV + P, LC = C + P;
  static constexpr size_t sTK = (size_t)C * LK * sizeof(E), sTV = (size_t)C * LV * sizeof(E);
  static constexpr size_t sDC = (size_t)DK * LC * sizeof(E), sVC = (size_t)DV * LC * sizeof(E);
  static constexpr size_t sCC = (size_t)C * LC * sizeof(E);
  static constexpr size_t K = 0, KT = K + sTK, VV = KT + sDC, TT = VV + sTV, TTT = TT + sCC, DW = TTT + sCC;
  static constexpr size_t DU = DW + sTK;
  static constexpr size_t F = DU + sTV;  // dW^T, dU^T; later dT, R^T, M, M^T
  static constexpr size_t FS = (sDC + sVC) > 4 * sCC ? (sDC + sVC) : 4 * sCC;
  static constexpr size_t G = F + FS;
  static constexpr size_t BB = G + C * 4, DG = BB + C * 4, DB = DG + C * 4, CX = DB + C * 4;
  static constexpr size_t TOTAL = CX + C * 4;
};

template <typename E, int C, int DK, int DV>
__global__ __launch_bounds__(kThreads) void k_grad2(const E* __restrict__ k, const E* __restrict__ v,
                                                    const float* __restrict__ beta, const float* __restrict__ wG,
                                                    const E* __restrict__ wT, const E* __restrict__ wdW,
                                                    const E* __restrict__ wdU, const float* __restrict__ wdK1,
                                                    const float* __restrict__ wdg1, E* __restrict__ dk,
                                                    E* __restrict__ dv, float* __restrict__ dlog_a,
                                                    float* __restrict__ dbeta, int T, int H, int N) {
  typedef Grad2Lds<E, C, DK, DV> Lay;
  constexpr int LK = Lay::LK, LV = Lay::LV, LC = Lay::LC, NB = C / 16;
  constexpr int V = 16 / (int)sizeof(E);
  constexpr int NKT = (DK / 16) * NB, KPW = (NKT + kWaves - 1) / kWaves;
  __shared__ __attribute__((aligned(16))) char smem[Lay::TOTAL];
  E* sK = (E*)(smem + Lay::K);
  E* sKt = (E*)(smem + Lay::KT);
  E* sV = (E*)(smem + Lay::VV);
  E* sT = (E*)(smem + Lay::TT);
  E* sTt = (E*)(smem + Lay::TTT);
  E* sdW = (E*)(smem + Lay::DW);
  E* sdU = (E*)(smem + Lay::DU);
  E* sdWt = (E*)(smem + Lay::F);
  E* sdUt = (E*)(smem + Lay::F + Lay::sDC);
  float* sg = (float*)(smem + Lay::G);
  float* sb = (float*)(smem + Lay::BB);
  float* sdg = (float*)(smem + Lay::DG);
  float* sdb = (float*)(smem + Lay::DB);
  float* scx = (float*)(smem + Lay::CX);

  const int tile = blockIdx.x;
  const int n = tile % N, bh = tile / N, h = bh % H, b = bh / H;
  const int t0 = n * C, nv = min(C, T - t0);
  const size_t tok0 = (size_t)b * T + t0;
  const int w = wave_id(), l = lane_id();

  {
    Tile<E, C, DK> tk, tdw;
    Tile<E, C, DV> tv;
    Tile<E, C, C> tt;
    Tile<E, DV, C> tdu;
    tk.load_rows(k + (tok0 * H + h) * DK, (size_t)H * DK, nv);
    tdw.load_block(wdW + (size_t)tile * C * DK);
    tv.load_rows(v + (tok0 * H + h) * DV, (size_t)H * DV, nv);
    tt.load_block(wT + (size_t)tile * C * C);
    tdu.load_block(wdU + (size_t)tile * DV * C);
    tk.store(sK, LK);
    tk.store_T(sKt, LC);
    tdw.store(sdW, LK);
    tdw.store_T(sdWt, LC);
    tv.store(sV, LV);
    tt.store(sT, LC);
    tt.store_T(sTt, LC);
    tdu.store(sdUt, LC);
    tdu.store_T(sdU, LV);
  }
  if (threadIdx.x < C) {
    const int t = threadIdx.x;
    sg[t] = wG[(size_t)tile * C + t];
    sb[t] = t < nv ? beta[(tok0 + t) * H + h] : 0.f;
    sdg[t] = wdg1[(size_t)tile * C + t];
    sdb[t] = 0.f;
    scx[t] = 0.f;
  }
  // dK^T accumulators (rows d, cols j), seeded with the first part of dK
  f32x4 dka[KPW];
#pragma unroll
  for (int s = 0; s < KPW; ++s) {
    const int tt = w + kWaves * s;
    dka[s] = zero4();
    if (tt < NKT) {
      const int td = tt / NB, tj = tt % NB;
      const float4 x = *(const float4*)(wdK1 + (size_t)tile * C * DK + (size_t)(tj * 16 + (l & 15)) * DK +
                                        td * 16 + (l >> 4) * 4);
      dka[s] = f32x4{x.x, x.y, x.z, x.w};
    }
  }
  __syncthreads();
  // dX^T = dW^T Tinv (rows d, cols j): dK += b gamma dX, cx_j = dX_j . k_j
#pragma unroll
  for (int s = 0; s < KPW; ++s) {
    const int tt = w + kWaves * s;
    if (tt < NKT) {
      const int td = tt / NB, tj = tt % NB;
      const int j = tj * 16 + (l & 15), d0 = td * 16 + (l >> 4) * 4;
      f32x4 acc = zero4();
      mma<C>(acc, sdWt + td * 16 * LC, LC, sTt + tj * 16 * LC, LC);
      dka[s] += (sb[j] * __expf(sg[j])) * acc;
      float e = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) e += acc[r] * to_f(sK[j * LK + d0 + r]);
      e = sum4(e);
      if (l < 16) atomicAdd(&scx[j], e);
    }
  }
  // dY^T = dU^T Tinv (rows v, cols j): dV = b dY, dbeta += dY_j . v_j
  for (int tt = w; tt < (DV / 16) * NB; tt += kWaves) {
    const int tv = tt / NB, tj = tt % NB;
    const int j = tj * 16 + (l & 15), v0 = tv * 16 + (l >> 4) * 4;
    f32x4 acc = zero4();
    mma<C>(acc, sdUt + tv * 16 * LC, LC, sTt + tj * 16 * LC, LC);
    if (j < nv) store4<E>(dv + ((tok0 + j) * H + h) * DV + v0, sb[j] * acc);
    float e = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) e += acc[r] * to_f(sV[j * LV + v0 + r]);
    e = sum4(e);
    if (l < 16) atomicAdd(&sdb[j], e);
  }
  __syncthreads();
  E* sdT = (E*)(smem + Lay::F);
  E* sRt = sdT + C * LC;
  E* sM = sRt + C * LC;
  E* sMt = sM + C * LC;
  // dT = dW X^T + dU Y^T = (dW K^T) diag(b gamma) + (dU V^T) diag(b)   (rows i, cols j)
  for (int tt = w; tt < NB * NB; tt += kWaves) {
    const int ti = tt / NB, tj = tt % NB;
    const int j = tj * 16 + (l & 15), i0 = ti * 16 + (l >> 4) * 4;
    f32x4 z1 = zero4(), z2 = zero4();
    mma<DK>(z1, sdW + ti * 16 * LK, LK, sK + tj * 16 * LK, LK);
    mma<DV>(z2, sdU + ti * 16 * LV, LV, sV + tj * 16 * LV, LV);
    const f32x4 d = sb[j] * (__expf(sg[j]) * z1 + z2);
#pragma unroll
    for (int r = 0; r < 4; ++r) sdT[(i0 + r) * LC + j] = from_f<E>(d[r]);
  }
  __syncthreads();
  // R = dT Tinv^T (rows i, cols k) -> R^T [k][i]
  for (int tt = w; tt < NB * NB; tt += kWaves) {
    const int ti = tt / NB, tk = tt % NB;
    f32x4 acc = zero4();
    mma<C>(acc, sdT + ti * 16 * LC, LC, sT + tk * 16 * LC, LC);
    store4<E>(sRt + (tk * 16 + (l & 15)) * LC + ti * 16 + (l >> 4) * 4, acc);
  }
  __syncthreads();
  // dA = -strict_lower(Tinv^T R); with A = b_i (K K^T) o Gamma:
  //   M = dA o b_i Gamma, dbeta_i += sum_k dA o Gamma o KK^T, E = dA o A -> dg
  for (int tt = w; tt < NB * NB; tt += kWaves) {
    const int ti = tt / NB, tk = tt % NB;
    const int kk = tk * 16 + (l & 15), i0 = ti * 16 + (l >> 4) * 4;
    f32x4 m = zero4();
    if (tk <= ti) {
      f32x4 acc = zero4(), kkt = zero4();
      mma<C>(acc, sTt + ti * 16 * LC, LC, sRt + tk * 16 * LC, LC);
      mma<DK>(kkt, sK + ti * 16 * LK, LK, sK + tk * 16 * LK, LK);
      float ecol = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + r;
        const float gam = (kk < i) ? __expf(sg[i] - sg[kk]) : 0.f;
        const float da = -acc[r];
        const float a = sb[i] * kkt[r] * gam;
        m[r] = da * sb[i] * gam;
        const float e = da * a;
        ecol += e;
        const float er = sum16(e);
        const float br = sum16(da * gam * kkt[r]);
        if ((l & 15) == 0) {
          atomicAdd(&sdg[i], er);
          atomicAdd(&sdb[i], br);
        }
      }
      ecol = sum4(ecol);
      if (l < 16) atomicAdd(&sdg[kk], -ecol);
    }
    store4<E>(sMt + kk * LC + i0, m);
#pragma unroll
    for (int r = 0; r < 4; ++r) sM[(i0 + r) * LC + kk] = from_f<E>(m[r]);
  }
  __syncthreads();
  // dK^T += K^T M (cols j: sum_i k_i M_ij) + K^T M^T (cols i: sum_j k_j M_ij)
#pragma unroll
  for (int s = 0; s < KPW; ++s) {
    const int tt = w + kWaves * s;
    if (tt < NKT) {
      const int td = tt / NB, tj = tt % NB;
      const int j = tj * 16 + (l & 15), d0 = td * 16 + (l >> 4) * 4;
      mma<C>(dka[s], sKt + td * 16 * LC, LC, sMt + tj * 16 * LC, LC);
      mma<C>(dka[s], sKt + td * 16 * LC, LC, sM + tj * 16 * LC, LC);
      if (j < nv) store4<E>(dk + ((tok0 + j) * H + h) * DK + d0, dka[s]);
    }
  }
  // dg (+ the X = diag(b gamma) K term), reverse cumsum -> dlog_a; dbeta
  if (threadIdx.x < 64) {
    const int t = threadIdx.x;
    float dg = 0.f, db = 0.f;
    if (t < C) {
      const float gam = __expf(sg[t]);
      dg = sdg[t] + sb[t] * gam * scx[t];
      db = sdb[t] + gam * scx[t];
    }
    const float dla = wave_incl_suffix(dg);
    if (t < nv) {
      dlog_a[(tok0 + t) * H + h] = dla;
      dbeta[(tok0 + t) * H + h] = db;
    }
  }
}

// --------------------------------------------------------------- launcher
template <typename E, int C, int DK, int DV>
int bwd_impl(const BwdArgs& a) {
  // fp32 gradient tiles need twice the LDS of bf16 ones: the fp32 backward
  // is limited to d_k, d_v <= 64 and chunk <= 32
  if constexpr (sizeof(E) == 4 && (DK > 64 || DV > 64)) {
    return -2;
  } else if constexpr (sizeof(E) == 4 && C > 32) {
    return -3;
  } else {
    const int N = (a.T + C - 1) / C;
    const int tiles = a.B * a.H * N;
    const BwdWs ws = bwd_ws_layout(a.B, a.T, a.H, DK, DV, C, sizeof(E), a.workspace);
    hipStream_t st = (hipStream_t)a.stream;
    constexpr int BV = DV < 32 ? DV : 32;
    const int sgrid = a.B * a.H * (DV / BV);
    LRT_LAUNCH(kKPrep, (k_prep<E, C, DK, DV, true, true>), dim3(tiles), dim3(kThreads), st, (const E*)a.k,
                       (const E*)a.v, a.log_a, a.beta, a.T, a.H, N, (E*)ws.f.W, (E*)ws.f.Up, (E*)ws.f.Kt,
                       ws.f.G, (E*)ws.T);
    LRT_LAUNCH(kKState, (k_state<E, C, DK, BV, true>), dim3(sgrid), dim3(kThreads), st, (const E*)ws.f.W,
                       (const E*)ws.f.Up, (const E*)ws.f.Kt, ws.f.G, (const float*)nullptr, a.h0, (float*)nullptr, (E*)ws.f.U,
                       (E*)ws.f.S, N, DV);
    E* dUl = (E*)ws.f.Up;
    LRT_LAUNCH(kKBwdLocal, (k_bwd_local<E, C, DK, DV>), dim3(tiles), dim3(kThreads), st, (const E*)a.q,
                       (const E*)a.k, (const E*)a.d_o, ws.f.G, dUl, a.T, a.H, N);
    LRT_LAUNCH(kKDState, (k_dstate<E, C, DK, BV>), dim3(sgrid), dim3(kThreads), st, (const E*)a.q,
                       (const E*)a.k, (const E*)a.d_o, ws.f.G, (const E*)ws.f.W, (const E*)dUl, a.dht, a.dh0,
                       (E*)ws.dS, (E*)ws.dU, a.T, a.H, N, DV);
    LRT_LAUNCH(kKGrad1, (k_grad1<E, C, DK, DV>), dim3(tiles), dim3(kThreads), st, (const E*)a.q,
                       (const E*)a.k, (const E*)a.d_o, ws.f.G, (const E*)ws.f.S, (const E*)ws.dS,
                       (const E*)ws.f.U, (const E*)ws.dU, (E*)a.dq, (E*)ws.dW, ws.dK1, ws.dg1, a.T, a.H, N);
    LRT_LAUNCH(kKGrad2, (k_grad2<E, C, DK, DV>), dim3(tiles), dim3(kThreads), st, (const E*)a.k,
                       (const E*)a.v, a.beta, ws.f.G, (const E*)ws.T, (const E*)ws.dW, (const E*)ws.dU, ws.dK1,
                       ws.dg1, (E*)a.dk_out, (E*)a.dv_out, a.dlog_a, a.dbeta, a.T, a.H, N);
    return hipGetLastError() == hipSuccess ? 0 : -7;
  }
}

template <typename E>
static int bwd_dtype(const BwdArgs& a) {
#define LRT_CASE(C_, DK_, DV_) \
  if (a.chunk == C_ && a.dk == DK_ && a.dv == DV_) return bwd_impl<E, C_, DK_, DV_>(a);
#define LRT_DV(C_, DK_) LRT_CASE(C_, DK_, 16) LRT_CASE(C_, DK_, 32) LRT_CASE(C_, DK_, 64) LRT_CASE(C_, DK_, 128)
#define LRT_DK(C_) LRT_DV(C_, 16) LRT_DV(C_, 32) LRT_DV(C_, 64) LRT_DV(C_, 128)
  LRT_DK(16) LRT_DK(32) LRT_DK(64)
#undef LRT_DK
#undef LRT_DV
#undef LRT_CASE
  return -2;
}

int bwd_gdn(const BwdArgs& a) { return a.dtype == 1 ? bwd_dtype<bf16>(a) : bwd_dtype<float>(a); }

}  // namespace lrt
