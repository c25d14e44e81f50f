// lrt_fwd_kernels.hpp -- chunkwise forward of the gated delta-rule mixers on gfx950.
//
// The recurrences (state H = S^T, [d_k, d_v]) are those of the mixers on the
// AMD ROCm blog "Pretraining hybrid LLMs with Primus", section "How hybrid
// models are defined in Primus" (mixer list under Table 2).  Inside a chunk of
// C tokens with start state Hn, g = inclusive cumsum of log a, gamma = e^g:
//   A     = strict_lower(diag(b) (K K^T) o Gamma),   Gamma_ij = e^(g_i - g_j)
//   Tinv  = (I + A)^-1
//   W     = Tinv diag(b gamma) K,   U' = Tinv diag(b) V           (chunk prep)
//   U     = U' - W Hn,   H_next = gamma_C Hn + Ktil^T U,  Ktil_j = e^(g_C - g_j) k_j
//                                                              (state pass)
//   O     = diag(gamma) Q Hn + ((Q K^T) o Gamma_incl) U           (output)
// SSD has no beta and no delta term (U = V).  Every exponent is a difference
// g_later - g_earlier <= 0, so nothing overflows however strong the decay.
//
// Three kernels, all 256 threads:
//   k_prep  one workgroup per (b, h, chunk): gates, K K^T, (I + A)^-1, W, U', Ktil
//   k_state one workgroup per (b, h, d_v block): serial over chunks, state in
//           MFMA accumulators, writes each chunk's start state S_n and U
//   k_out   one workgroup per (b, h, chunk): O = gamma Q Hn + P U
// Workspace tiles are chunk-major per (b, h): tile = (b*H + h)*N + n.
#pragma once
#include "lrt_common.hpp"

namespace lrt {

// (I + A)^-1 for a strictly lower-triangular C x C matrix A in LDS (fp32,
// row stride C + 1), written to Tf (same layout; only the lower triangle,
// diagonal included, is defined).  Stage 1 inverts the 16 x 16 diagonal
// blocks by forward substitution, one lane per column; stage 2 fills block
// row bi from  T[bi][bj] = -T[bi][bi] sum_{m=bj}^{bi-1} A[bi][m] T[m][bj].
// R is a 3 * 256-float scratch.  All 256 threads must call it after A is
// visible to them; Tf is visible to all threads on return.
template <int C>
__device__ __forceinline__ void unit_lower_inverse(const float* sA, float* sTf, float* sR) {
  constexpr int NB = C / 16;
  constexpr int LA = C + 1;
  // (I + A)^-1, stage 1: the 16x16 diagonal blocks by forward substitution,
  // one lane per column (lanes 16*bb .. 16*bb+15 own block bb).
  if (threadIdx.x < 16 * NB) {
    const int bb = threadIdx.x >> 4, j = threadIdx.x & 15;
    const float* Ab = sA + (bb * 16) * LA + bb * 16;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = (r == j) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) s -= Ab[r * LA + m] * x[m];
      x[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sTf[(bb * 16 + r) * LA + bb * 16 + j] = x[r];
  }
  __syncthreads();
  // stage 2: block row bi, T[bi][bj] = -T[bi][bi] sum_{m=bj}^{bi-1} A[bi][m] T[m][bj]
  {
    const int r = threadIdx.x >> 4, c = threadIdx.x & 15;
    for (int bi = 1; bi < NB; ++bi) {
      for (int bj = 0; bj < bi; ++bj) {
        float s = 0.f;
        for (int m = bj * 16; m < bi * 16; ++m) s += sA[(bi * 16 + r) * LA + m] * sTf[m * LA + bj * 16 + c];
        sR[bj * 256 + r * 16 + c] = s;
      }
      __syncthreads();
      for (int bj = 0; bj < bi; ++bj) {
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m) s += sTf[(bi * 16 + r) * LA + bi * 16 + m] * sR[bj * 256 + m * 16 + c];
        sTf[(bi * 16 + r) * LA + bj * 16 + c] = -s;
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ k_prep
// WRITE_T (backward only) also stores Tinv [C][C] per chunk.
template <typename E, int C, int DK, int DV, bool DELTA, bool WRITE_T = false>
__global__ __launch_bounds__(kThreads) void k_prep(const E* __restrict__ k, const E* __restrict__ v,
                                                   const float* __restrict__ log_a,
                                                   const float* __restrict__ beta, int T, int H, int N,
                                                   E* __restrict__ wW, E* __restrict__ wUp,
                                                   E* __restrict__ wKt, float* __restrict__ wG,
                                                   E* __restrict__ wT) {
  constexpr int P = lds_pad<E>();
  constexpr int LK = DK + P;  // rows indexed by token, contiguous over d
  constexpr int LC = C + P;   // rows indexed by d or v, contiguous over tokens
  constexpr int NB = C / 16;
  constexpr int LA = C + 1;
  __shared__ float sg[C], sgam[C], sb[C], sbg[C];
  __shared__ __attribute__((aligned(16))) E sK[C * LK];
  __shared__ __attribute__((aligned(16))) E sYt[DV * LC];
  __shared__ __attribute__((aligned(16))) E sXt[DELTA ? DK * LC : 8];
  __shared__ __attribute__((aligned(16))) E sT[DELTA ? C * LC : 8];
  __shared__ float sA[DELTA ? C * LA : 1];
  __shared__ float sTf[DELTA ? C * LA : 1];
  __shared__ float sR[DELTA ? 3 * 256 : 1];

  const int tile = blockIdx.x;
  const int n = tile % N, bh = tile / N, h = bh % H, b = bh / H;
  const int t0 = n * C, nv = min(C, T - t0);
  const size_t tok0 = (size_t)b * T + t0;
  const int w = wave_id(), l = lane_id();

  Tile<E, C, DK> tk;
  Tile<E, C, DV> tv;
  tk.load_rows(k + (tok0 * H + h) * DK, (size_t)H * DK, nv);
  tv.load_rows(v + (tok0 * H + h) * DV, (size_t)H * DV, nv);
  if (threadIdx.x < 64) {
    const int t = threadIdx.x;
    float la = 0.f, bt = 0.f;
    if (t < nv) {
      la = log_a[(tok0 + t) * H + h];
      if (DELTA) bt = beta[(tok0 + t) * H + h];
    }
    const float g = wave_incl_scan(la);
    if (t < C) {
      sg[t] = g;
      sgam[t] = __expf(g);
      sb[t] = bt;
      sbg[t] = bt * __expf(g);
      wG[(size_t)tile * C + t] = g;
    }
  }
  tk.store(sK, LK);
  __syncthreads();

  // Y^T = (diag(b) V)^T (SSD: V^T) -> sYt[v][t]
  if (DELTA) tv.scale_rows(sb);
  tv.store_T(sYt, LC);
  // Ktil^T[d][t] = e^(g_C - g_t) k_t[d] -> workspace, 16 bytes per store
  {
    constexpr int V = 16 / (int)sizeof(E);
    const float gC = sg[C - 1];
    E* out = wKt + (size_t)tile * DK * C;
    for (int idx = threadIdx.x; idx < DK * (C / V); idx += kThreads) {
      const int d = idx / (C / V), t = (idx % (C / V)) * V;
      E e[V];
#pragma unroll
      for (int i = 0; i < V; ++i) e[i] = from_f<E>(__expf(gC - sg[t + i]) * to_f(sK[(t + i) * LK + d]));
      u32x4 x;
      __builtin_memcpy(&x, e, 16);
      *(u32x4*)(out + (size_t)d * C + t) = x;
    }
  }
  if constexpr (!DELTA) {
    __syncthreads();
    constexpr int V = 16 / (int)sizeof(E);
    E* out = wUp + (size_t)tile * DV * C;
    for (int idx = threadIdx.x; idx < DV * (C / V); idx += kThreads) {
      const int c = idx / (C / V), t = (idx % (C / V)) * V;
      *(u32x4*)(out + (size_t)c * C + t) = *(const u32x4*)(sYt + c * LC + t);
    }
    return;
  } else {
    // X^T = (diag(b gamma) K)^T -> sXt[d][t], from the registers of K
    tk.scale_rows(sbg);
    tk.store_T(sXt, LC);
    // A = strict_lower(b_i (k_i . k_j) e^(g_i - g_j))
    for (int tt = w; tt < NB * NB; tt += kWaves) {
      const int ti = tt / NB, tj = tt % NB;
      f32x4 acc = zero4();
      if (tj <= ti) mma<DK>(acc, sK + ti * 16 * LK, LK, sK + tj * 16 * LK, LK);
      const int j = tj * 16 + (l & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = ti * 16 + (l >> 4) * 4 + r;
        sA[i * LA + j] = (j < i) ? sb[i] * acc[r] * __expf(sg[i] - sg[j]) : 0.f;
      }
    }
    __syncthreads();
    unit_lower_inverse<C>(sA, sTf, sR);
    for (int idx = threadIdx.x; idx < C * C; idx += kThreads) {
      const int i = idx / C, j = idx % C;
      const E x = from_f<E>(j <= i ? sTf[i * LA + j] : 0.f);
      sT[i * LC + j] = x;
      if (WRITE_T) wT[(size_t)tile * C * C + idx] = x;
    }
    __syncthreads();
    // W^T = X^T Tinv^T (rows d, cols t) -> W[t][d]
    E* wout = wW + (size_t)tile * C * DK;
    for (int tt = w; tt < (DK / 16) * NB; tt += kWaves) {
      const int td = tt / NB, tc = tt % NB;
      f32x4 acc = zero4();
      mma<C>(acc, sXt + td * 16 * LC, LC, sT + tc * 16 * LC, LC);
      store4<E>(wout + (size_t)(tc * 16 + (l & 15)) * DK + td * 16 + (l >> 4) * 4, acc);
    }
    // U' = Tinv Y (rows t, cols v) -> U'^T[v][t]
    E* uout = wUp + (size_t)tile * DV * C;
    for (int tt = w; tt < NB * (DV / 16); tt += kWaves) {
      const int ti = tt / (DV / 16), tv = tt % (DV / 16);
      f32x4 acc = zero4();
      mma<C>(acc, sT + ti * 16 * LC, LC, sYt + tv * 16 * LC, LC);
      store4<E>(uout + (size_t)(tv * 16 + (l & 15)) * C + ti * 16 + (l >> 4) * 4, acc);
    }
  }
}

// ----------------------------------------------------------------- k_state
// One workgroup per (b, h, d_v block of BV columns); walks the N chunks.
// PERDIM (KDA): the chunk decay is per key dimension, e^(GC[d]) from wGC.
template <typename E, int C, int DK, int BV, bool DELTA, bool PERDIM = false>
__global__ __launch_bounds__(kThreads) void k_state(const E* __restrict__ wW, const E* __restrict__ wUp,
                                                    const E* __restrict__ wKt, const float* __restrict__ wG,
                                                    const float* __restrict__ wGC, const float* h0, float* ht,
                                                    E* __restrict__ wU, E* __restrict__ wS, int N, int DV) {
  constexpr int P = lds_pad<E>();
  constexpr int LK = DK + P, LC = C + P;
  constexpr int NTV = BV / 16;
  constexpr int NH = (DK / 16) * NTV;  // state tiles
  constexpr int HPW = (NH + kWaves - 1) / kWaves;
  constexpr int NU = (C / 16) * NTV;  // U tiles
  constexpr int UPW = (NU + kWaves - 1) / kWaves;
  constexpr int V16 = 16 / (int)sizeof(E);
  constexpr int NW16 = DELTA ? C * DK / V16 : 0;
  constexpr int NK16 = DK * C / V16;
  constexpr int PW = (NW16 + kThreads - 1) / kThreads;
  constexpr int PK = (NK16 + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) E sW[DELTA ? C * LK : 8];
  __shared__ __attribute__((aligned(16))) E sKt[DK * LC];
  __shared__ __attribute__((aligned(16))) E sS[DELTA ? BV * LK : 8];
  __shared__ __attribute__((aligned(16))) E sU[BV * LC];

  const int nvb = DV / BV;
  const int vb = blockIdx.x % nvb, bh = blockIdx.x / nvb;
  const int v0 = vb * BV;
  const int w = wave_id(), l = lane_id();

  f32x4 hacc[HPW];
#pragma unroll
  for (int s = 0; s < HPW; ++s) {
    const int tt = w + kWaves * s;
    hacc[s] = zero4();
    if (tt < NH && h0 != nullptr) {
      const int td = tt / NTV, tv = tt % NTV;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        hacc[s][r] = h0[((size_t)bh * DK + td * 16 + (l >> 4) * 4 + r) * DV + v0 + tv * 16 + (l & 15)];
    }
  }

  Tile<E, C, DK> tW;   // W of the next chunk (delta variants)
  Tile<E, DK, C> tK;   // Ktil^T of the next chunk
  f32x4 rUp[UPW];
  f32x4 rgd[PERDIM ? HPW : 1];
  float rgc = 0.f;
#define LRT_STATE_FETCH(n_)                                                                         \
  {                                                                                                 \
    const size_t ft = (size_t)bh * N + (n_);                                                        \
    if (DELTA) tW.load_block(wW + ft * C * DK);                                                     \
    tK.load_block(wKt + ft * DK * C);                                                               \
    _Pragma("unroll") for (int s = 0; s < UPW; ++s) {                                               \
      const int tt = w + kWaves * s;                                                                \
      if (tt < NU)                                                                                  \
        rUp[s] = load4<E>(wUp + ft * DV * C + (size_t)(v0 + (tt % NTV) * 16 + (l & 15)) * C +      \
                          (tt / NTV) * 16 + (l >> 4) * 4);                                          \
    }                                                                                               \
    if constexpr (PERDIM) {                                                                         \
      _Pragma("unroll") for (int s = 0; s < HPW; ++s) {                                             \
        const int tt = w + kWaves * s;                                                              \
        if (tt < NH) rgd[s] = *(const f32x4*)(wGC + ft * DK + (tt / NTV) * 16 + (l >> 4) * 4);     \
      }                                                                                             \
    } else {                                                                                        \
      rgc = wG[ft * C + C - 1];                                                                     \
    }                                                                                               \
  }

  LRT_STATE_FETCH(0)
  for (int n = 0; n < N; ++n) {
    const size_t tile = (size_t)bh * N + n;
    if (DELTA) tW.store(sW, LK);
    tK.store(sKt, LC);
    f32x4 up[UPW];
#pragma unroll
    for (int s = 0; s < UPW; ++s) up[s] = rUp[s];
    const float dec = __expf(rgc);
    f32x4 decd[PERDIM ? HPW : 1];
    if constexpr (PERDIM) {
#pragma unroll
      for (int s = 0; s < HPW; ++s)
        decd[s] = f32x4{__expf(rgd[s][0]), __expf(rgd[s][1]), __expf(rgd[s][2]), __expf(rgd[s][3])};
    }
    if (n + 1 < N) LRT_STATE_FETCH(n + 1)
#undef LRT_STATE_FETCH

    // chunk start state: S = H^T -> LDS (operand of W Hn) and workspace
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + kWaves * s;
      if (tt < NH) {
        const int td = tt / NTV, tv = tt % NTV;
        const int vv = tv * 16 + (l & 15), d = td * 16 + (l >> 4) * 4;
        if (DELTA) store4<E>(sS + vv * LK + d, hacc[s]);
        store4<E>(wS + tile * DV * DK + (size_t)(v0 + vv) * DK + d, hacc[s]);
      }
    }
    __syncthreads();
    // U = U' - W Hn  (rows t, cols v)
#pragma unroll
    for (int s = 0; s < UPW; ++s) {
      const int tt = w + kWaves * s;
      if (tt < NU) {
        const int ti = tt / NTV, tv = tt % NTV;
        const int vv = tv * 16 + (l & 15), t = ti * 16 + (l >> 4) * 4;
        f32x4 u = up[s];
        if constexpr (DELTA) {
          f32x4 acc = zero4();
          mma<DK>(acc, sW + ti * 16 * LK, LK, sS + tv * 16 * LK, LK);
          u -= acc;
        }
        store4<E>(sU + vv * LC + t, u);
        store4<E>(wU + tile * DV * C + (size_t)(v0 + vv) * C + t, u);
      }
    }
    __syncthreads();
    // H <- e^(g_C) H + Ktil^T U
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + kWaves * s;
      if (tt < NH) {
        const int td = tt / NTV, tv = tt % NTV;
        if constexpr (PERDIM)
          hacc[s] *= decd[s];
        else
          hacc[s] *= dec;
        mma<C>(hacc[s], sKt + td * 16 * LC, LC, sU + tv * 16 * LC, LC);
      }
    }
    __syncthreads();
  }
  if (ht != nullptr) {
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + kWaves * s;
      if (tt < NH) {
        const int td = tt / NTV, tv = tt % NTV;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          ht[((size_t)bh * DK + td * 16 + (l >> 4) * 4 + r) * DV + v0 + tv * 16 + (l & 15)] = hacc[s][r];
      }
    }
  }
}

// ------------------------------------------------------------------- k_out
// O^T = S Q^T (scaled by gamma per token) + U^T P^T, one workgroup per
// (chunk, block of BVO value columns).
// FROM_WS (KDA): Q o e^G and P are read from the workspace instead of being
// formed from q, k and the scalar gates.
template <typename E, int C, int DK, int BVO, bool FROM_WS = false>
__global__ __launch_bounds__(kThreads) void k_out(const E* __restrict__ q, const E* __restrict__ k,
                                                  const float* __restrict__ wG, const E* __restrict__ wS,
                                                  const E* __restrict__ wU, const E* __restrict__ wQg,
                                                  const E* __restrict__ wP, E* __restrict__ o, int T, int H,
                                                  int N, int DV) {
  constexpr int P = lds_pad<E>();
  constexpr int LK = DK + P, LC = C + P;
  constexpr int NB = C / 16;
  __shared__ float sg[C];
  __shared__ __attribute__((aligned(16))) E sQ[C * LK];
  __shared__ __attribute__((aligned(16))) E sK[FROM_WS ? 8 : C * LK];
  __shared__ __attribute__((aligned(16))) E sS[BVO * LK];
  __shared__ __attribute__((aligned(16))) E sU[BVO * LC];
  __shared__ __attribute__((aligned(16))) E sP[C * LC];

  const int nvb = DV / BVO;
  const int tile = blockIdx.x / nvb, v0 = (blockIdx.x % nvb) * BVO;
  const int n = tile % N, bh = tile / N, h = bh % H, b = bh / H;
  const int t0 = n * C, nv = min(C, T - t0);
  const size_t tok0 = (size_t)b * T + t0;
  const int w = wave_id(), l = lane_id();

  {
    Tile<E, C, DK> tq;
    Tile<E, FROM_WS ? C : C, FROM_WS ? C : DK> tk;  // K rows, or P (FROM_WS)
    Tile<E, BVO, DK> ts;
    Tile<E, BVO, C> tu;
    if constexpr (FROM_WS) {
      tq.load_block(wQg + (size_t)tile * C * DK);
      tk.load_block(wP + (size_t)tile * C * C);
    } else {
      tq.load_rows(q + (tok0 * H + h) * DK, (size_t)H * DK, nv);
      tk.load_rows(k + (tok0 * H + h) * DK, (size_t)H * DK, nv);
      if (threadIdx.x < C) sg[threadIdx.x] = wG[(size_t)tile * C + threadIdx.x];
    }
    ts.load_block(wS + ((size_t)tile * DV + v0) * DK);
    tu.load_block(wU + ((size_t)tile * DV + v0) * C);
    tq.store(sQ, LK);
    if constexpr (FROM_WS)
      tk.store(sP, LC);
    else
      tk.store(sK, LK);
    ts.store(sS, LK);
    tu.store(sU, LC);
  }
  __syncthreads();
  // P = (Q K^T) o Gamma, inclusive lower triangle
  if constexpr (!FROM_WS) {
  for (int tt = w; tt < NB * NB; tt += kWaves) {
    const int ti = tt / NB, tj = tt % NB;
    f32x4 acc = zero4();
    if (tj <= ti) mma<DK>(acc, sQ + ti * 16 * LK, LK, sK + tj * 16 * LK, LK);
    const int j = tj * 16 + (l & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = ti * 16 + (l >> 4) * 4 + r;
      sP[i * LC + j] = from_f<E>(j <= i ? acc[r] * __expf(sg[i] - sg[j]) : 0.f);
    }
  }
  __syncthreads();
  }
  for (int tt = w; tt < (BVO / 16) * NB; tt += kWaves) {
    const int tv = tt / NB, ti = tt % NB;
    f32x4 acc = zero4();
    mma<DK>(acc, sS + tv * 16 * LK, LK, sQ + ti * 16 * LK, LK);
    const int i = ti * 16 + (l & 15);
    if constexpr (!FROM_WS) acc *= __expf(sg[i]);
    mma<C>(acc, sU + tv * 16 * LC, LC, sP + ti * 16 * LC, LC);
    if (i < nv) store4<E>(o + ((tok0 + i) * H + h) * DV + v0 + tv * 16 + (l >> 4) * 4, acc);
  }
}

}  // namespace lrt
