// lrt_scan.hpp -- the chunkwise Gated DeltaNet forward split in two passes:
// a chunk-parallel WY pass and a serial chunk scan.
//
// Chunk algebra (state H = S^T, [d_k, d_v]; one chunk of C tokens with start
// state Hn; the recurrence of the mixer list on the AMD ROCm blog
// "Pretraining hybrid LLMs with Primus", section "How hybrid models are
// defined in Primus", under Table 2):
//   g = inclusive cumsum of log a,  gamma = e^g,  Gamma_ij = e^(g_i - g_j)
//   A  = strict_lower(diag(b) (K K^T) o Gamma),  T = (I + A)^-1
//   W  = T diag(b gamma) K,   U' = T diag(b) V,   P = (Q K^T) o Gamma (j <= i)
//   U  = U' - W Hn
//   O  = diag(gamma) Q Hn + P U
//   Hn <- gamma_C Hn + K^T diag(e^(g_C - g)) U
//
// k_wy   (one chunk per step, persistent over all (b, h, chunk) tiles) forms
//        g, A, T, W, U' and P, or T instead of P for the backward.  Every
//        chunk is independent, so two workgroups per CU hide each other's
//        latency in the triangular solve.
// k_scan (one workgroup per (b, h, block of BV value columns), serial over
//        chunks) carries the state in MFMA accumulators and does only what
//        depends on it: U, then O (forward) or the chunk-start states S_n and
//        U (backward recompute).  The next chunk's operands load into
//        registers while this one computes.
#pragma once
#include "lrt_fwd_kernels.hpp"

namespace lrt {

// ------------------------------------------------------------------- k_wy
template <typename E, int C, int DK, int DV>
struct WyLds {
  static constexpr int P = lds_pad<E>();
  static constexpr int LK = DK + P, LV = DV + P, LC = C + P, LA = C + 1;
  static constexpr size_t es = sizeof(E);
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t K = 0;                                                      // k rows [t][d]
  static constexpr size_t V = K + (size_t)C * LK * es;                                // b v rows [t][v]
  static constexpr size_t QT = V + (size_t)C * LV * es;                               // q rows; then T, T diag(b gamma)
  static constexpr size_t A = QT + mx((size_t)C * LK * es, 2 * (size_t)C * LC * es);  // A (fp32), inverted in place
  static constexpr size_t G = A + (size_t)C * LA * 4;                                 // g, gamma, b, b gamma
  static constexpr size_t TOTAL = G + 4 * C * 4;
};

// Outputs per tile (chunk-major per (b, h)): W [C][d_k] rows, U'^T [d_v][C],
// g [C]; WRITE_P: P [C][C] rows (zero above the diagonal); WRITE_T: T [C][C].
template <typename E, int C, int DK, int DV, bool WRITE_P, bool WRITE_T, int NW = 8>
__global__ __launch_bounds__(64 * NW, 4) void k_wy(const E* __restrict__ q, const E* __restrict__ k,
                                                const E* __restrict__ v, const float* __restrict__ log_a,
                                                const float* __restrict__ beta, int T, int H, int N, int ntiles,
                                                E* __restrict__ wW, E* __restrict__ wUp, float* __restrict__ wG,
                                                E* __restrict__ wP, E* __restrict__ wT) {
  typedef WyLds<E, C, DK, DV> Lay;
  constexpr int NT = 64 * NW;
  constexpr int LK = Lay::LK, LV = Lay::LV, LC = Lay::LC, LA = Lay::LA;
  constexpr int NB = C / 16;
  constexpr int NWT = (DK / 16) * NB, NUT = NB * (DV / 16);  // W^T and U' output tiles
  __shared__ __attribute__((aligned(16))) char smem[Lay::TOTAL];
  E* sK = (E*)(smem + Lay::K);
  E* sV = (E*)(smem + Lay::V);
  E* sQ = (E*)(smem + Lay::QT);
  E* sT = (E*)(smem + Lay::QT);
  E* sTw = sT + C * LC;
  float* sA = (float*)(smem + Lay::A);
  float* sg = (float*)(smem + Lay::G);
  float* sgam = sg + C;
  float* sb = sg + 2 * C;
  float* sbg = sg + 3 * C;
  const int w = wave_id(), l = lane_id();

  Tile<E, C, DK, NT> tk, tq;
  Tile<E, C, DV, NT> tv;
  float la = 0.f, bt = 0.f;
#define LRT_WY_LOAD(tile_)                                                                \
  {                                                                                       \
    const int ln = (tile_) % N, lbh = (tile_) / N;                                        \
    const int lnv = min(C, T - ln * C);                                                   \
    const size_t ltok = (size_t)(lbh / H) * T + (size_t)ln * C;                           \
    const int lh = lbh % H;                                                               \
    tk.load_rows(k + (ltok * H + lh) * DK, (size_t)H * DK, lnv);                          \
    if (WRITE_P) tq.load_rows(q + (ltok * H + lh) * DK, (size_t)H * DK, lnv);             \
    tv.load_rows(v + (ltok * H + lh) * DV, (size_t)H * DV, lnv);                          \
    {                                                                                     \
      const int tc = min((int)threadIdx.x, lnv - 1); /* masked where used */              \
      la = log_a[(ltok + tc) * H + lh];                                                   \
      bt = beta[(ltok + tc) * H + lh];                                                    \
    }                                                                                     \
  }

  int tile = blockIdx.x;
  if (tile < ntiles) LRT_WY_LOAD(tile)
  for (; tile < ntiles; tile += gridDim.x) {
    const int nv = min(C, T - (tile % N) * C);
    if (threadIdx.x < 64) {
      const bool valid = (int)threadIdx.x < nv;
      const float g = wave_incl_scan(valid ? la : 0.f);
      if (threadIdx.x < C) {
        const int t = threadIdx.x;
        const float gam = __expf(g);
        const float b_ = valid ? bt : 0.f;
        sg[t] = g;
        sgam[t] = gam;
        sb[t] = b_;
        sbg[t] = b_ * gam;
        wG[(size_t)tile * C + t] = g;
      }
    }
    tk.store(sK, LK);
    if constexpr (WRITE_P) tq.store(sQ, LK);
    lds_barrier();
    tv.scale_rows(sb);
    tv.store(sV, LV);
    if (tile + (int)gridDim.x < ntiles) LRT_WY_LOAD(tile + (int)gridDim.x)
    // A (lower tiles; the solve reads nothing above the diagonal) and P^T
    // tiles, P^T[j][i] = (k_j . q_i) e^(g_i - g_j) for j <= i, stored as rows of P
    constexpr int NA = NB * (NB + 1) / 2;
    for (int tt = w; tt < NA + (WRITE_P ? NB * NB : 0); tt += NW) {
      if (tt < NA) {
        int ti = 0, r0 = tt;
        while (r0 > ti) {
          r0 -= ti + 1;
          ++ti;
        }
        const int tj = r0;
        f32x4 acc = zero4();
        mma<DK>(acc, sK + ti * 16 * LK, LK, sK + tj * 16 * LK, LK);
        const int j = tj * 16 + (l & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = ti * 16 + (l >> 4) * 4 + r;
          sA[i * LA + j] = (j < i) ? sb[i] * acc[r] * __expf(sg[i] - sg[j]) : 0.f;
        }
      } else {
        const int t2 = tt - NA, rj = t2 / NB, ci = t2 % NB;
        f32x4 acc = zero4();
        if (rj <= ci) mma<DK>(acc, sK + rj * 16 * LK, LK, sQ + ci * 16 * LK, LK);
        const int i = ci * 16 + (l & 15), j0 = rj * 16 + (l >> 4) * 4;
        f32x4 p;
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = (j0 + r <= i) ? acc[r] * __expf(sg[i] - sg[j0 + r]) : 0.f;
        store4<E>(wP + (size_t)tile * C * C + (size_t)i * C + j0, p);
      }
    }
    lds_barrier();
    unit_lower_inverse<C, NT>(sA, sA);
    for (int idx = threadIdx.x; idx < C * C; idx += NT) {
      const int i = idx / C, j = idx % C;
      const float x = j <= i ? sA[i * LA + j] : 0.f;
      sT[i * LC + j] = from_f<E>(x);
      sTw[i * LC + j] = from_f<E>(x * sbg[j]);
    }
    lds_barrier();
    if constexpr (WRITE_T) lds_to_block<E, C, C, NT>(wT + (size_t)tile * C * C, sT, LC);
    // W^T = K^T (T diag(b gamma))^T (rows d, cols t): a lane's 4 values are
    // 4 consecutive d of one row of W; U' = T (b V) (rows t, cols v): 4
    // consecutive t of one row of U'^T
    for (int tt = w; tt < NWT + NUT; tt += NW) {
      f32x4 acc = zero4();
      if (tt < NWT) {
        const int td = tt / NB, ti = tt % NB;
        mma<C, true, false>(acc, sK + td * 16, LK, sTw + ti * 16 * LC, LC);
        const int t = ti * 16 + (l & 15), d0 = td * 16 + (l >> 4) * 4;
        store4<E>(wW + ((size_t)tile * C + t) * DK + d0, acc);
      } else {
        const int u = tt - NWT, ti = u / (DV / 16), tvb = u % (DV / 16);
        mma<C, false, true>(acc, sT + ti * 16 * LC, LC, sV + tvb * 16, LV);
        const int vv = tvb * 16 + (l & 15), t0 = ti * 16 + (l >> 4) * 4;
        store4<E>(wUp + ((size_t)tile * DV + vv) * C + t0, acc);
      }
    }
    lds_barrier();
  }
#undef LRT_WY_LOAD
}

// ----------------------------------------------------------------- k_scan
template <typename E, int C, int DK, int BV, bool FWD>
struct ScanLds {
  static constexpr int P = lds_pad<E>();
  static constexpr int LK = DK + P, LB = BV + P, LC = C + P;
  static constexpr size_t es = sizeof(E);
  static constexpr size_t W = 0;                                     // W rows [t][d]
  static constexpr size_t K = W + (size_t)C * LK * es;               // k rows [t][d]
  static constexpr size_t S = K + (size_t)C * LK * es;               // Hn^T [v][d]
  static constexpr size_t U = S + (size_t)BV * LK * es;              // U^T, (e^(g_C - g) U)^T [v][t]
  static constexpr size_t Q = U + 2 * (size_t)BV * LC * es;          // q rows [t][d]
  static constexpr size_t P_ = Q + (FWD ? (size_t)C * LK * es : 0);  // P [i][j]
  static constexpr size_t O = P_ + (FWD ? (size_t)C * LC * es : 0);  // o rows [t][v]
  static constexpr size_t G = O + (FWD ? (size_t)C * LB * es : 0);   // g, gamma, e^(g_C - g)
  static constexpr size_t TOTAL = G + 3 * C * 4;
};

// FWD: writes o and ht.  Backward recompute (!FWD): writes S_n [d_v][d_k]
// and U^T [d_v][C] per tile (chunk-major per (b, h)).
template <typename E, int C, int DK, int BV, bool FWD, int NW = 8>
__global__ __launch_bounds__(64 * NW) void k_scan(const E* __restrict__ q, const E* __restrict__ k,
                                                  const E* __restrict__ wW, const E* __restrict__ wUp,
                                                  const float* __restrict__ wG, const E* __restrict__ wP,
                                                  const float* h0, float* ht, E* __restrict__ o,
                                                  E* __restrict__ wU, E* __restrict__ wS, int T, int H, int N,
                                                  int DV) {
  typedef ScanLds<E, C, DK, BV, FWD> Lay;
  constexpr int NT = 64 * NW;
  constexpr int LK = Lay::LK, LB = Lay::LB, LC = Lay::LC;
  constexpr int NB = C / 16, NTV = BV / 16;
  constexpr int NH = (DK / 16) * NTV, HPW = (NH + NW - 1) / NW;  // state tiles (rows d, cols v)
  constexpr int NU = NB * NTV, UPW = (NU + NW - 1) / NW;         // U tiles (rows t, cols v)
  constexpr int NO = NTV * NB;                                   // O^T tiles (rows v, cols t)
  __shared__ __attribute__((aligned(16))) char smem[Lay::TOTAL];
  E* sW = (E*)(smem + Lay::W);
  E* sK = (E*)(smem + Lay::K);
  E* sS = (E*)(smem + Lay::S);
  E* sU = (E*)(smem + Lay::U);
  E* sUk = sU + BV * LC;
  E* sQ = (E*)(smem + Lay::Q);
  E* sP = (E*)(smem + Lay::P_);
  E* sO = (E*)(smem + Lay::O);
  float* sg = (float*)(smem + Lay::G);
  float* sgam = sg + C;
  float* skt = sg + 2 * C;

  const int nvb = DV / BV;
  const int wg = xcd_group(blockIdx.x, gridDim.x);  // the column blocks of one (b, h) share an L2
  const int vb = wg % nvb, bh = wg / nvb;
  const int h = bh % H, b = bh / H;
  const int v0 = vb * BV;
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

  // One chunk's operands in registers.  Two sets alternate, so the loads of
  // chunk n + 2 are in flight while chunk n computes.
  struct Ops {
    Tile<E, C, DK, NT> W, K, Q;
    Tile<E, C, C, NT> P;
    typename Vec4<E>::T up[UPW];
    float g;
  };
  auto fetch = [&](Ops& x, int n_) {
    const size_t ft = (size_t)bh * N + n_;
    const int fnv = min(C, T - n_ * C);
    const size_t ftok = (size_t)b * T + (size_t)n_ * C;
    x.W.load_block(wW + ft * C * DK);
    x.K.load_rows(k + (ftok * H + h) * DK, (size_t)H * DK, fnv);
    if constexpr (FWD) {
      x.Q.load_rows(q + (ftok * H + h) * DK, (size_t)H * DK, fnv);
      x.P.load_block(wP + ft * C * C);
    }
    // unconditional loads (clamped indices), so nothing waits for them here
#pragma unroll
    for (int s = 0; s < UPW; ++s) {
      const int tt = min(w + NW * s, NU - 1);
      x.up[s] = load4_raw<E>(wUp + (ft * DV + v0 + (tt % NTV) * 16 + (l & 15)) * C + (tt / NTV) * 16 + (l >> 4) * 4);
    }
    x.g = wG[ft * C + min((int)threadIdx.x, C - 1)];
  };

  size_t otok = 0;  // first token of the chunk whose o rows wait in sO
  int onv = 0;
  auto step = [&](Ops& x, int n) {
    const size_t tile = (size_t)bh * N + n;
    const int nv = min(C, T - n * C);
    const size_t tok0 = (size_t)b * T + (size_t)n * C;
    // ---- this chunk's operands and start state into LDS
    if (threadIdx.x < 64) {
      const float gC = __shfl(x.g, C - 1, 64);
      if (threadIdx.x < C) {
        sg[threadIdx.x] = x.g;
        sgam[threadIdx.x] = __expf(x.g);
        skt[threadIdx.x] = __expf(gC - x.g);
      }
    }
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + NW * s;
      if (tt < NH) {
        const int td = tt / NTV, tv = tt % NTV;
        store4<E>(sS + (tv * 16 + (l & 15)) * LK + td * 16 + (l >> 4) * 4, hacc[s]);
      }
    }
    x.W.store(sW, LK);
    x.K.store(sK, LK);
    if constexpr (FWD) {
      x.Q.store(sQ, LK);
      x.P.store(sP, LC);
    }
    f32x4 up[UPW];
#pragma unroll
    for (int s = 0; s < UPW; ++s) up[s] = Vec4<E>::unpack(x.up[s]);
    if (n + 2 < N) fetch(x, n + 2);
    lds_barrier();
    if constexpr (FWD) {
      // o rows of the previous chunk (staged in sO by its last step)
      if (n > 0) lds_to_rows<E, C, BV, NT>(o + (otok * H + h) * DV + v0, (size_t)H * DV, sO, LB, onv);
    } else {
      lds_to_block<E, BV, DK, NT>(wS + (tile * DV + v0) * DK, sS, LK);
    }
    // ---- U = U' - W Hn -> U^T and (e^(g_C - g) U)^T
#pragma unroll
    for (int s = 0; s < UPW; ++s) {
      const int tt = w + NW * s;
      if (tt < NU) {
        const int ti = tt / NTV, tv = tt % NTV;
        f32x4 acc = zero4();
        mma<DK>(acc, sW + ti * 16 * LK, LK, sS + tv * 16 * LK, LK);
        const f32x4 u = up[s] - acc;
        const int vv = tv * 16 + (l & 15), t = ti * 16 + (l >> 4) * 4;
        store4<E>(sU + vv * LC + t, u);
        store4<E>(sUk + vv * LC + t, f32x4{u[0] * skt[t], u[1] * skt[t + 1], u[2] * skt[t + 2], u[3] * skt[t + 3]});
        if constexpr (!FWD) store4<E>(wU + (tile * DV + v0 + vv) * C + t, u);
      }
    }
    lds_barrier();
    // ---- O^T = (Hn^T Q^T) diag(gamma) + U^T P^T -> o rows; state update
    if constexpr (FWD) {
      for (int tt = w; tt < NO; tt += NW) {
        const int tv = tt / NB, ti = tt % NB;
        f32x4 acc = zero4();
        mma<DK>(acc, sS + tv * 16 * LK, LK, sQ + ti * 16 * LK, LK);
        const int i = ti * 16 + (l & 15);
        acc *= sgam[i];
        mma<C>(acc, sU + tv * 16 * LC, LC, sP + ti * 16 * LC, LC);
        store4<E>(sO + i * LB + tv * 16 + (l >> 4) * 4, acc);
      }
      otok = tok0;
      onv = nv;
    }
    const float dec = __expf(sg[C - 1]);
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + NW * s;
      if (tt < NH) {
        const int td = tt / NTV, tv = tt % NTV;
        hacc[s] *= dec;
        mma<C, true, false>(hacc[s], sK + td * 16, LK, sUk + tv * 16 * LC, LC);
      }
    }
    lds_barrier();
  };

  Ops x0, x1;
  fetch(x0, 0);
  if (N > 1) fetch(x1, 1);
  for (int n = 0; n < N; n += 2) {
    step(x0, n);
    if (n + 1 < N) step(x1, n + 1);
  }
  if constexpr (FWD) {
    if (N > 0) lds_to_rows<E, C, BV, NT>(o + (otok * H + h) * DV + v0, (size_t)H * DV, sO, LB, onv);
  }
  if (ht != nullptr) {
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + NW * s;
      if (tt < NH) {
        const int td = tt / NTV, tv = tt % NTV;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          ht[((size_t)bh * DK + td * 16 + (l >> 4) * 4 + r) * DV + v0 + tv * 16 + (l & 15)] = hacc[s][r];
      }
    }
  }
}

}  // namespace lrt
