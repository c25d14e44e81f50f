// lrt_fused_fwd.hpp -- the whole chunkwise forward of Gated DeltaNet in one
// kernel (used where the WY pass + scan split does not fit in LDS).
//
// One workgroup of NW waves per (b, h, block of BV value columns) walks the
// chunks in order.  Per chunk of C tokens (state Hn = S^T kept in MFMA
// accumulators, rows d, columns v):
//   g = cumsum log a,  gamma = e^g,  Gamma_ij = e^(g_i - g_j)   (j <= i)
//   A  = strict_lower(diag(b) (K K^T) o Gamma),  T = (I + A)^-1
//   W  = T diag(b gamma) K,   U' = T diag(b) V
//   U  = U' - W Hn
//   O  = diag(gamma) Q Hn + ((Q K^T) o Gamma) U
//   Hn <- gamma_C Hn + K^T diag(e^(g_C - g)) U
// The state never leaves the chip; q, k, v and the
// gates are read once per chunk (the value-column blocks of one (b, h) share
// an XCD's L2) and o is written once, so HBM traffic is the method's minimum
// plus the duplicated q/k reads of the column blocks.  The next chunk's
// inputs load into registers while this one computes.  Operands are kept in
// their natural row-major layouts; products contracting over tokens read them
// with the LDS transpose read.
#pragma once
#include "lrt_fwd_kernels.hpp"

namespace lrt {

template <typename E, int C, int DK, int BV>
struct FusedLds {
  static constexpr int P = lds_pad<E>();
  static constexpr int LK = DK + P, LB = BV + P, LC = C + P, LA = tri_ld<C>();
  static constexpr size_t es = sizeof(E);
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t K = 0;                                        // k rows [t][d]
  static constexpr size_t Q = K + (size_t)C * LK * es;                  // q rows [t][d]
  static constexpr size_t V = Q + (size_t)C * LK * es;                  // b v rows [t][v]
  static constexpr size_t S = V + (size_t)C * LB * es;                  // Hn^T [v][d]
  static constexpr size_t P_ = S + (size_t)BV * LK * es;                // (Q K^T) o Gamma [i][j]
  static constexpr size_t U = P_ + (size_t)C * LC * es;                 // A, T (fp32, column-major); then U^T, (kt U)^T
  static constexpr size_t USZ = mx((size_t)C * LA * 4, 2 * (size_t)BV * LC * es);
  static constexpr size_t TW = U + USZ;                                 // W rows [t][d]
  static constexpr size_t TWSZ = (size_t)C * LK * es;
  static constexpr size_t T = TW + TWSZ;                                // Tinv, Tinv diag(b gamma) (E)
  static constexpr size_t TSZ = 2 * (size_t)C * LC * es;
  static constexpr size_t O = T + TSZ;                                  // o rows [t][v]
  static constexpr size_t OSZ = (size_t)C * LB * es;
  static constexpr size_t G = O + OSZ;                                  // g, gamma, b, b gamma, e^(g_C - g)
  static constexpr size_t TOTAL = G + 5 * C * 4;
};

template <typename E, int C, int DK, int BV, int NW = 8>
__global__ __launch_bounds__(64 * NW) void k_fwd(const E* __restrict__ q, const E* __restrict__ k,
                                                 const E* __restrict__ v, const float* __restrict__ log_a,
                                                 const float* __restrict__ beta, const float* h0, float* ht,
                                                 E* __restrict__ o, int T, int H, int N, int DV) {
  typedef FusedLds<E, C, DK, BV> Lay;
  constexpr int NT = 64 * NW;
  constexpr int LK = Lay::LK, LB = Lay::LB, LC = Lay::LC, LA = Lay::LA;
  constexpr int NB = C / 16, NTV = BV / 16;
  constexpr int NH = (DK / 16) * NTV, HPW = (NH + NW - 1) / NW;   // state tiles (rows d, cols v)
  constexpr int NU = NB * NTV, UPW = (NU + NW - 1) / NW;          // U tiles (rows t, cols v)
  constexpr int NO = NTV * NB;                                    // O^T tiles (rows v, cols t)
  __shared__ __attribute__((aligned(16))) char smem[Lay::TOTAL];
  E* sK = (E*)(smem + Lay::K);
  E* sQ = (E*)(smem + Lay::Q);
  E* sV = (E*)(smem + Lay::V);
  E* sS = (E*)(smem + Lay::S);
  E* sP = (E*)(smem + Lay::P_);
  float* sA = (float*)(smem + Lay::U);
  E* sU = (E*)(smem + Lay::U);
  E* sUk = sU + BV * LC;
  E* sW = (E*)(smem + Lay::TW);
  E* sT = (E*)(smem + Lay::T);
  E* sTw = sT + C * LC;
  E* sO = (E*)(smem + Lay::O);
  float* sg = (float*)(smem + Lay::G);
  float* sgam = sg + C;
  float* sb = sg + 2 * C;
  float* sbg = sg + 3 * C;
  float* skt = sg + 4 * C;

  const int nvb = DV / BV;
  const int wg = xcd_group(blockIdx.x, gridDim.x);
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

  Tile<E, C, DK, NT> tk, tq;
  Tile<E, C, BV, NT> tv;
  float rla = 0.f, rb = 0.f;
#define LRT_FWD_FETCH(n_)                                                                   \
  {                                                                                         \
    const int fnv = min(C, T - (n_) * C);                                                   \
    const size_t ftok = (size_t)b * T + (size_t)(n_) * C;                                   \
    tk.load_rows(k + (ftok * H + h) * DK, (size_t)H * DK, fnv);                             \
    tq.load_rows(q + (ftok * H + h) * DK, (size_t)H * DK, fnv);                             \
    tv.load_rows(v + (ftok * H + h) * DV + v0, (size_t)H * DV, fnv);                        \
    rla = 0.f;                                                                              \
    rb = 0.f;                                                                               \
    if ((int)threadIdx.x < fnv) {                                                           \
      rla = log_a[(ftok + threadIdx.x) * H + h];                                            \
      rb = beta[(ftok + threadIdx.x) * H + h];                                              \
    }                                                                                       \
  }

  LRT_FWD_FETCH(0)
  for (int n = 0; n < N; ++n) {
    const int t0 = n * C, nv = min(C, T - t0);
    const size_t tok0 = (size_t)b * T + t0;
    // ---- S1: this chunk's inputs and the chunk-start state into LDS
    if (threadIdx.x < 64) {
      const float g = wave_incl_scan(rla);
      const float gC = __shfl(g, C - 1, 64);
      if (threadIdx.x < C) {
        const float gam = __expf(g);
        sg[threadIdx.x] = g;
        sgam[threadIdx.x] = gam;
        sb[threadIdx.x] = rb;
        sbg[threadIdx.x] = rb * gam;
        skt[threadIdx.x] = __expf(gC - g);
      }
    }
    tk.store(sK, LK);
    tq.store(sQ, LK);
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + NW * s;
      if (tt < NH) {
        const int td = tt / NTV, tv2 = tt % NTV;
        store4<E>(sS + (tv2 * 16 + (l & 15)) * LK + td * 16 + (l >> 4) * 4, hacc[s]);
      }
    }
    lds_barrier();
    tv.scale_rows(sb);
    tv.store(sV, LB);
    if (n + 1 < N) LRT_FWD_FETCH(n + 1)
    // ---- S2: A and P
    for (int tt = w; tt < NB * NB; tt += NW) {
      const int ti = tt / NB, tj = tt % NB;
      if (tj > ti) {
        store4<E>(sP + (ti * 16 + (l & 15)) * LC + tj * 16 + (l >> 4) * 4, zero4());
        continue;
      }
      const int j = tj * 16 + (l & 15), i0 = ti * 16 + (l >> 4) * 4;
      f32x4 qk = zero4();
      mma<DK>(qk, sQ + ti * 16 * LK, LK, sK + tj * 16 * LK, LK);
      // P[i][j] = (q_i . k_j) e^(g_i - g_j), j <= i; this lane holds rows i0.. of column j
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + r;
        sP[i * LC + j] = from_f<E>((j <= i) ? qk[r] * __expf(sg[i] - sg[j]) : 0.f);
      }
      f32x4 kk = zero4();
      mma<DK>(kk, sK + ti * 16 * LK, LK, sK + tj * 16 * LK, LK);
      f32x4 av;
#pragma unroll
      for (int r = 0; r < 4; ++r) av[r] = (j < i0 + r) ? sb[i0 + r] * kk[r] * __expf(sg[i0 + r] - sg[j]) : 0.f;
      *(f32x4*)(sA + j * LA + i0) = av;  // column-major
    }
    lds_barrier();
    // ---- S3: T = (I + A)^-1, in E twice: T and T diag(b gamma)
    unit_lower_inverse<C, NT>(sA);
    for (int idx = threadIdx.x; idx < C * C; idx += NT) {
      const int j = idx / C, i = idx % C;
      const float x = j <= i ? sA[j * LA + i] : 0.f;
      sT[i * LC + j] = from_f<E>(x);
      sTw[i * LC + j] = from_f<E>(x * sbg[j]);
    }
    lds_barrier();
    // ---- S4: W^T = K^T (T diag(b gamma))^T -> W rows [t][d] (over the dead inverse)
    for (int tt = w; tt < (DK / 16) * NB; tt += NW) {
      const int td = tt / NB, ti = tt % NB;
      f32x4 acc = zero4();
      mma<C, true, false>(acc, sK + td * 16, LK, sTw + ti * 16 * LC, LC);
      store4<E>(sW + (ti * 16 + (l & 15)) * LK + td * 16 + (l >> 4) * 4, acc);
    }
    // U' = T (b V) (rows t, cols v), in registers
    f32x4 up[UPW];
#pragma unroll
    for (int s = 0; s < UPW; ++s) {
      const int tt = w + NW * s;
      up[s] = zero4();
      if (tt < NU) {
        const int ti = tt / NTV, tv2 = tt % NTV;
        mma<C, false, true>(up[s], sT + ti * 16 * LC, LC, sV + tv2 * 16, LB);
      }
    }
    lds_barrier();
    // ---- S5: U = U' - W Hn  -> U^T and (e^(g_C - g) U)^T, rows v
#pragma unroll
    for (int s = 0; s < UPW; ++s) {
      const int tt = w + NW * s;
      if (tt < NU) {
        const int ti = tt / NTV, tv2 = tt % NTV;
        f32x4 u = up[s];
        f32x4 acc = zero4();
        mma<DK>(acc, sW + ti * 16 * LK, LK, sS + tv2 * 16 * LK, LK);
        u -= acc;
        const int vv = tv2 * 16 + (l & 15), t = ti * 16 + (l >> 4) * 4;
        store4<E>(sU + vv * LC + t, u);
        store4<E>(sUk + vv * LC + t, f32x4{u[0] * skt[t], u[1] * skt[t + 1], u[2] * skt[t + 2], u[3] * skt[t + 3]});
      }
    }
    lds_barrier();
    // ---- S6: O^T = (S Q^T) diag(gamma) + U^T P^T -> o rows; H update
    for (int tt = w; tt < NO; tt += NW) {
      const int tv2 = tt / NB, ti = tt % NB;
      f32x4 acc = zero4();
      mma<DK>(acc, sS + tv2 * 16 * LK, LK, sQ + ti * 16 * LK, LK);
      const int i = ti * 16 + (l & 15);
      acc *= sgam[i];
      mma<C>(acc, sU + tv2 * 16 * LC, LC, sP + ti * 16 * LC, LC);
      store4<E>(sO + i * LB + tv2 * 16 + (l >> 4) * 4, acc);
    }
    const float dec = __expf(sg[C - 1]);
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + NW * s;
      if (tt < NH) {
        const int td = tt / NTV, tv2 = tt % NTV;
        hacc[s] *= dec;
        mma<C, true, false>(hacc[s], sK + td * 16, LK, sUk + tv2 * 16 * LC, LC);
      }
    }
    lds_barrier();
    // ---- S7: o rows out
    lds_to_rows<E, C, BV, NT>(o + (tok0 * H + h) * DV + v0, (size_t)H * DV, sO, LB, nv);
  }
#undef LRT_FWD_FETCH
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

}  // namespace lrt
