// lrt_kda.hip -- chunkwise forward of Kimi Delta Attention on gfx950.
//
// KDA is Gated DeltaNet with one gate per key dimension (AMD ROCm blog
// "Pretraining hybrid LLMs with Primus", section "How hybrid models are
// defined in Primus", mixer list under Table 2).  With the state H = S^T:
//   H_t = (I - b_t k_t k_t^T) Diag(a_t) H_{t-1} + b_t k_t v_t^T,  o_t = H_t^T q_t.
// Inside a chunk, G = per-dimension inclusive cumsum of log a (C x d_k):
//   A_ij   = b_i sum_d k_id k_jd e^(G_id - G_jd)   (j < i)
//   P_ij   =     sum_d q_id k_jd e^(G_id - G_jd)   (j <= i)
//   W = Tinv diag(b) (K o e^G),  U' = Tinv diag(b) V,  Tinv = (I + A)^-1
//   U = U' - W Hn,  O = (Q o e^G) Hn + P U,
//   H_next = Diag(e^(G_C)) Hn + (K o e^(G_C - G))^T U.
// The decays inside A and P sit inside the d_k contraction, so they cannot be
// applied as a row/column scaling of one GEMM.  For a pair i >= r >= j the
// factor splits as e^(G_i - G_r) e^(G_r - G_j) with both exponents <= 0:
// blocks of 16 rows take r = the block's first row and run on MFMA for all
// columns of earlier blocks; pairs inside a 16 x 16 diagonal block are summed
// element by element with the exact exponent difference.  Nothing overflows
// for any finite log a <= 0.
//
// k_kda_prep (one workgroup per chunk) writes W, U'^T, Ktil^T, Q o e^G, P and
// the per-dimension chunk decay; the generic state pass (per-dimension decay)
// and output kernel (operands from the workspace) then finish the chunk.
#include "lrt_fwd_kernels.hpp"
#include "lrt_internal.hpp"

namespace lrt {

template <typename E, int C, int DK, int DV>
struct KdaLds {
  static constexpr int P = lds_pad<E>();
  static constexpr int LK = DK + P, LC = C + P, LG = DK + 4, LA = C + 1, NB = C / 16;
  static constexpr size_t es = sizeof(E);
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t K = 0;                                         // K rows
  static constexpr size_t QY = K + C * LK * es;                          // Q rows, later (b V)^T
  static constexpr size_t G = QY + mx(C * LK * es, DV * LC * es);        // G (fp32)
  static constexpr size_t S = G + (size_t)C * LG * 4;                    // scaled operands, later (b K e^G)^T
  static constexpr size_t A = S + mx((size_t)16 * (NB + 1) * LK * es, (size_t)DK * LC * es);
  static constexpr size_t TF = A + (size_t)C * LA * 4;
  static constexpr size_t T = TF + (size_t)C * LA * 4;
  static constexpr size_t BB = T + (size_t)C * LC * es;
  static constexpr size_t TOTAL = BB + C * 4;
};

template <typename E, int C, int DK, int DV>
__global__ __launch_bounds__(kThreads) void k_kda_prep(const E* __restrict__ q, const E* __restrict__ k,
                                                       const E* __restrict__ v, const float* __restrict__ log_a,
                                                       const float* __restrict__ beta, int T, int H, int N,
                                                       E* __restrict__ wW, E* __restrict__ wUp,
                                                       E* __restrict__ wKt, float* __restrict__ wGC,
                                                       E* __restrict__ wQg, E* __restrict__ wP) {
  typedef KdaLds<E, C, DK, DV> Lay;
  constexpr int LK = Lay::LK, LC = Lay::LC, LG = Lay::LG, LA = Lay::LA, NB = Lay::NB;
  constexpr int V = 16 / (int)sizeof(E);
  __shared__ __attribute__((aligned(16))) char smem[Lay::TOTAL];
  E* sK = (E*)(smem + Lay::K);
  E* sQ = (E*)(smem + Lay::QY);
  float* sG = (float*)(smem + Lay::G);
  E* sS = (E*)(smem + Lay::S);
  float* sA = (float*)(smem + Lay::A);
  float* sTf = (float*)(smem + Lay::TF);
  E* sT = (E*)(smem + Lay::T);
  float* sb = (float*)(smem + Lay::BB);

  const int tile = blockIdx.x;
  const int n = tile % N, bh = tile / N, h = bh % H, b = bh / H;
  const int t0 = n * C, nv = min(C, T - t0);
  const size_t tok0 = (size_t)b * T + t0;
  const int w = wave_id(), l = lane_id();

  Tile<E, C, DV> tv;  // v, stored after the solve
  {
    Tile<E, C, DK> tk, tq;
    Tile<float, C, DK> tg;
    tk.load_rows(k + (tok0 * H + h) * DK, (size_t)H * DK, nv);
    tq.load_rows(q + (tok0 * H + h) * DK, (size_t)H * DK, nv);
    tg.load_rows(log_a + (tok0 * H + h) * DK, (size_t)H * DK, nv);
    tv.load_rows(v + (tok0 * H + h) * DV, (size_t)H * DV, nv);
    tk.store(sK, LK);
    tq.store(sQ, LK);
    tg.store(sG, LG);
  }
  if (threadIdx.x < C) sb[threadIdx.x] = threadIdx.x < nv ? beta[(tok0 + threadIdx.x) * H + h] : 0.f;
  for (int idx = threadIdx.x; idx < C * LA; idx += kThreads) sA[idx] = 0.f;
  lds_barrier();
  // G: inclusive cumsum over the chunk's tokens, per key dimension
  for (int d = threadIdx.x; d < DK; d += kThreads) {
    float s = 0.f;
    for (int t = 0; t < C; ++t) {
      s += sG[t * LG + d];
      sG[t * LG + d] = s;
    }
  }
  lds_barrier();
  // Q o e^G [t][d], Ktil^T [d][t] = (k_t o e^(G_C - G_t))^T, chunk decay G_C
  {
    E* qg = wQg + (size_t)tile * C * DK;
    for (int idx = threadIdx.x; idx < C * DK; idx += kThreads) {
      const int t = idx / DK, d = idx % DK;
      qg[idx] = from_f<E>(to_f(sQ[t * LK + d]) * __expf(sG[t * LG + d]));
    }
    E* kt = wKt + (size_t)tile * DK * C;
    for (int idx = threadIdx.x; idx < DK * C; idx += kThreads) {
      const int d = idx / C, t = idx % C;
      kt[idx] = from_f<E>(to_f(sK[t * LK + d]) * __expf(sG[(C - 1) * LG + d] - sG[t * LG + d]));
    }
    for (int d = threadIdx.x; d < DK; d += kThreads) wGC[(size_t)tile * DK + d] = sG[(C - 1) * LG + d];
  }
  E* pout = wP + (size_t)tile * C * C;
  // off-diagonal 16-row blocks: reference r = 16 s, operands scaled in LDS
  //   rows [0, 16):       k_i o e^(G_i - G_r)   (i in block s)
  //   rows [16, 32):      q_i o e^(G_i - G_r)
  //   rows [32, 32 + r):  k_j o e^(G_r - G_j)   (j < r)
  for (int s = 1; s < NB; ++s) {
    const int r0 = 16 * s;
    const int nrow = 32 + r0;
    for (int idx = threadIdx.x; idx < nrow * DK; idx += kThreads) {
      const int row = idx / DK, d = idx % DK;
      const float gr = sG[r0 * LG + d];
      float x;
      if (row < 16) {
        x = to_f(sK[(r0 + row) * LK + d]) * __expf(sG[(r0 + row) * LG + d] - gr);
      } else if (row < 32) {
        x = to_f(sQ[(r0 + row - 16) * LK + d]) * __expf(sG[(r0 + row - 16) * LG + d] - gr);
      } else {
        const int j = row - 32;
        x = to_f(sK[j * LK + d]) * __expf(gr - sG[j * LG + d]);
      }
      sS[row * LK + d] = from_f<E>(x);
    }
    lds_barrier();
    // tiles: (kind, column block sj) for kind 0 = A (kk), 1 = P (qk)
    for (int tt = w; tt < 2 * s; tt += kWaves) {
      const int kind = tt / s, sj = tt % s;
      f32x4 acc = zero4();
      mma<DK>(acc, sS + kind * 16 * LK, LK, sS + (32 + sj * 16) * LK, LK);
      const int j = sj * 16 + (l & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = r0 + (l >> 4) * 4 + r;
        if (kind == 0)
          sA[i * LA + j] = sb[i] * acc[r];
        else
          pout[(size_t)i * C + j] = from_f<E>(acc[r]);
      }
    }
    lds_barrier();
  }
  // diagonal 16 x 16 blocks, element by element: pairs j <= i of one block
  for (int p = threadIdx.x; p < NB * 136; p += kThreads) {
    const int s = p / 136;
    int qi = p % 136, ii = 0;
    while (qi >= ii + 1) {
      qi -= ii + 1;
      ++ii;
    }
    const int i = 16 * s + ii, j = 16 * s + qi;
    float akk = 0.f, aqk = 0.f;
    for (int d = 0; d < DK; ++d) {
      const float e = __expf(sG[i * LG + d] - sG[j * LG + d]);
      const float kj = to_f(sK[j * LK + d]) * e;
      akk += to_f(sK[i * LK + d]) * kj;
      aqk += to_f(sQ[i * LK + d]) * kj;
    }
    if (j < i) sA[i * LA + j] = sb[i] * akk;
    pout[(size_t)i * C + j] = from_f<E>(aqk);
  }
  // P above the diagonal blocks is zero
  for (int idx = threadIdx.x; idx < C * C; idx += kThreads) {
    const int i = idx / C, j = idx % C;
    if ((j >> 4) > (i >> 4) || ((j >> 4) == (i >> 4) && j > i)) pout[idx] = from_f<E>(0.f);
  }
  lds_barrier();
  // (b K o e^G)^T -> sXt (over the staging area), (b V)^T -> sYt (over Q)
  E* sXt = sS;
  E* sYt = sQ;
  for (int idx = threadIdx.x; idx < C * DK; idx += kThreads) {
    const int t = idx / DK, d = idx % DK;
    sXt[d * LC + t] = from_f<E>(sb[t] * to_f(sK[t * LK + d]) * __expf(sG[t * LG + d]));
  }
  tv.scale_rows(sb);
  tv.store_T(sYt, LC);
  unit_lower_inverse<C>(sA, sTf);
  for (int idx = threadIdx.x; idx < C * C; idx += kThreads) {
    const int i = idx / C, j = idx % C;
    sT[i * LC + j] = from_f<E>(j <= i ? sTf[i * LA + j] : 0.f);
  }
  lds_barrier();
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

template <typename E, int C, int DK, int DV>
int kda_impl(const FwdArgs& a) {
  if constexpr (KdaLds<E, C, DK, DV>::TOTAL > 160 * 1024) {
    return -2;  // fp32 operands at d_k = 128 do not fit in LDS
  } else {
    const int N = (a.T + C - 1) / C;
    const int tiles = a.B * a.H * N;
    const FwdWs ws = fwd_ws_layout(a.B, a.T, a.H, DK, DV, C, sizeof(E), a.workspace, true);
    hipStream_t st = (hipStream_t)a.stream;
    LRT_LAUNCH(kKKdaPrep, (k_kda_prep<E, C, DK, DV>), dim3(tiles), dim3(kThreads), st, (const E*)a.q,
               (const E*)a.k, (const E*)a.v, a.log_a, a.beta, a.T, a.H, N, (E*)ws.W, (E*)ws.Up, (E*)ws.Kt,
               ws.GC, (E*)ws.Qg, (E*)ws.P);
    constexpr int BV = DV < 64 ? DV : 64;  // state columns per workgroup
    LRT_LAUNCH(kKState, (k_state<E, C, DK, BV, true, true, kStateWaves>), dim3(a.B * a.H * (DV / BV)), dim3(64 * kStateWaves), st,
               (const E*)ws.W, (const E*)ws.Up, (const E*)ws.Kt, ws.G, (const float*)ws.GC, a.h0, a.ht,
               (E*)ws.U, (E*)ws.S, N, DV);
    constexpr int BVO = (sizeof(E) == 4 && DV > 64) ? 64 : DV;
    LRT_LAUNCH(kKOut, (k_out<E, C, DK, BVO, true>), dim3(persistent_grid(tiles * (DV / BVO), out_lds_bytes<E, C, DK, BVO, true>())), dim3(kThreads), st,
               (const E*)a.q, (const E*)a.k, ws.G, (const E*)ws.S, (const E*)ws.U, (const E*)ws.Qg,
               (const E*)ws.P, (E*)a.o, a.T, a.H, N, DV, tiles * (DV / BVO));
    return hipGetLastError() == hipSuccess ? 0 : -7;
  }
}

template <typename E>
static int kda_dtype(const FwdArgs& a) {
#define LRT_CASE(C_, DK_, DV_) \
  if (a.chunk == C_ && a.dk == DK_ && a.dv == DV_) return kda_impl<E, C_, DK_, DV_>(a);
#define LRT_DV(C_, DK_) LRT_CASE(C_, DK_, 16) LRT_CASE(C_, DK_, 32) LRT_CASE(C_, DK_, 64) LRT_CASE(C_, DK_, 128)
#define LRT_DK(C_) LRT_DV(C_, 16) LRT_DV(C_, 32) LRT_DV(C_, 64) LRT_DV(C_, 128)
  LRT_DK(16) LRT_DK(32) LRT_DK(64)
#undef LRT_DK
#undef LRT_DV
#undef LRT_CASE
  return -2;
}

int fwd_kda(const FwdArgs& a) { return a.dtype == 1 ? kda_dtype<bf16>(a) : kda_dtype<float>(a); }

}  // namespace lrt
