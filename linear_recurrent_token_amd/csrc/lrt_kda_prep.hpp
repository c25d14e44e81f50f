// lrt_kda_prep.hpp -- the chunk-parallel pass of Kimi Delta Attention on gfx950.
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
// k_kda_prep (persistent over the chunks) writes W, U'^T, Ktil^T, Q o e^G, P and
// the per-dimension chunk decay (and, for the backward, Tinv); the serial
// scan in KDA mode (per-dimension decay, operands from the workspace) then
// carries the state and forms o.
#pragma once
#include <type_traits>

#include "lrt_fwd_kernels.hpp"
#include "lrt_internal.hpp"

namespace lrt {

template <typename E, int C, int DK, int DV, int NT>
struct KdaLds {
  static constexpr int P = lds_pad<E>();
  static constexpr int LK = DK + P, LV = DV + P, LC = C + P, LG = DK + 4, LA = tri_ld<C>(), NB = C / 16;
  static constexpr int NQ = (NT / DK < C) ? NT / DK : C;  // row segments of the cumsum
  static constexpr size_t es = sizeof(E);
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t K = 0;                                 // k rows [t][d]
  static constexpr size_t Q = K + (size_t)C * LK * es;           // q rows
  static constexpr size_t V = Q + (size_t)C * LK * es;           // b v rows
  static constexpr size_t G = V + (size_t)C * LV * es;           // G = cumsum log a [t][d] (fp32)
  static constexpr size_t S = G + (size_t)C * LG * 4;            // cumsum totals; scaled operands; X rows
  static constexpr size_t SSZ = mx(mx((size_t)16 * (NB + 1) * LK * es, (size_t)C * LK * es), (size_t)NQ * DK * 4);
  static constexpr size_t A = S + SSZ;                           // A (fp32), inverted in place
  static constexpr size_t T = A + (size_t)C * LA * 4;            // T, T diag(b) (E)
  static constexpr size_t BB = T + 2 * (size_t)C * LC * es;      // b
  static constexpr size_t FL = BB + C * 4;                       // max |G| over the chunk (float bits)
  static constexpr size_t TOTAL = FL + 16;
};

// Eight values of E from 16 bytes of LDS (or four for fp32), and back.
template <typename E>
__device__ __forceinline__ void lds_vec_load(const E* p, float* x) {
  constexpr int V = 16 / (int)sizeof(E);
  E e[V];
  const u32x4 r = *(const u32x4*)p;
  __builtin_memcpy(e, &r, 16);
#pragma unroll
  for (int i = 0; i < V; ++i) x[i] = to_f(e[i]);
}
template <typename E>
__device__ __forceinline__ u32x4 vec_pack(const float* x) {
  constexpr int V = 16 / (int)sizeof(E);
  E e[V];
#pragma unroll
  for (int i = 0; i < V; ++i) e[i] = from_f<E>(x[i]);
  u32x4 r;
  __builtin_memcpy(&r, e, 16);
  return r;
}
template <int V>
__device__ __forceinline__ void lds_f32_load(const float* p, float* x) {
#pragma unroll
  for (int i = 0; i < V; i += 4) {
    const f32x4 r = *(const f32x4*)(p + i);
    x[i] = r[0];
    x[i + 1] = r[1];
    x[i + 2] = r[2];
    x[i + 3] = r[3];
  }
}

// Persistent over the chunk tiles; the next tile's inputs load into
// registers while this one computes.  wT (nullable): Tinv rows [C][C] per
// chunk (zero above the diagonal), for the backward.  list (nullable): walk
// only the tiles listed there (count in list[0], tiles from list[1]) -- the
// exact-path chunks k_kda_prep_fast left.  LOWRANK (with FUSE):
// the gate comes as its rank-kGateRank bottleneck, log_a_ = z [tokens][R]
// (the activations W_down x of each token, shared by the heads) and wup =
// W_up [H * d_k][R]; the kernel forms W_up z per chunk on MFMA and applies
// -softplus.  FUSE: q, k, log_a and beta are the raw
// projections -- the gate pre-activation in E ([B, T, H, d_k]) -- and the
// fused prologue (L2-normalised q, k rows; log a = -softplus; sigmoid) is
// applied as they are staged.
template <typename E, int C, int DK, int DV, int NW = 8, bool FUSE = false, bool LOWRANK = false>
__global__ __launch_bounds__(64 * NW) void k_kda_prep(const E* __restrict__ q, const E* __restrict__ k,
                                                      const E* __restrict__ v, const void* __restrict__ log_a_,
                                                      const float* __restrict__ beta, SeqMap m,
                                                      E* __restrict__ wW, E* __restrict__ wUp,
                                                      E* __restrict__ wKt, float* __restrict__ wGC,
                                                      E* __restrict__ wQg, E* __restrict__ wP,
                                                      E* __restrict__ wT, const E* __restrict__ wup,
                                                      const int* __restrict__ list) {
  static_assert(!LOWRANK || FUSE, "the low-rank gate is a fused-prologue input");
  constexpr int NT = 64 * NW;
  typedef KdaLds<E, C, DK, DV, NT> Lay;
  constexpr int LK = Lay::LK, LV = Lay::LV, LC = Lay::LC, LG = Lay::LG, LA = Lay::LA, NB = Lay::NB;
  constexpr int V = 16 / (int)sizeof(E);
  __shared__ __attribute__((aligned(16))) char smem[Lay::TOTAL];
  int tid = threadIdx.x;  // (re-derived per chunk below, opaque to the compiler)
  const int H = m.H, ntiles = tile_count(m);

  typedef typename std::conditional<FUSE, E, float>::type GE;  // element type of the gate input
  const GE* log_a = (const GE*)log_a_;  // LOWRANK: the bottleneck activations z [tokens][kGateRank]
  constexpr int R = kGateRank, LZ = R + lds_pad<E>();
  Tile<E, C, DK, NT> tk, tq;
  Tile<E, C, DV, NT> tv;
  Tile<GE, C, LOWRANK ? R : DK, NT> tg;
  Tile<E, LOWRANK ? DK : 16, LOWRANK ? R : 16, NT> tw;  // LOWRANK: this head's W_up rows [d_k][R]
  static_assert(!LOWRANK || (size_t)(C + DK) * LZ * sizeof(E) <= Lay::SSZ, "z and W_up are staged in S");
  float rb = 0.f;
#define LRT_KDA_LOAD(tile_)                                                               \
  {                                                                                       \
    int ln;                                                                               \
    const SeqPos lp = tile_pos(m, (tile_), ln);                                           \
    const int lnv = min(C, lp.len - ln * C);                                              \
    const size_t ltok = lp.tok0 + (size_t)ln * C;                                         \
    const int lh = lp.h;                                                                  \
    tk.load_rows_clamped(k + (ltok * H + lh) * DK, (size_t)H * DK, lnv);                  \
    tq.load_rows_clamped(q + (ltok * H + lh) * DK, (size_t)H * DK, lnv);                  \
    tv.load_rows_clamped(v + (ltok * H + lh) * DV, (size_t)H * DV, lnv);                  \
    if constexpr (LOWRANK) {                                                              \
      tg.load_rows_clamped(log_a + ltok * R, (size_t)R, lnv);                             \
      tw.load_block(wup + (size_t)lh * DK * R);                                           \
    } else {                                                                              \
      tg.load_rows_clamped(log_a + (ltok * H + lh) * DK, (size_t)H * DK, lnv);            \
    }                                                                                     \
    rb = beta[(ltok + min(tid, lnv - 1)) * H + lh]; /* masked where used */               \
  }

  const int nitems = list != nullptr ? list[0] : ntiles;
  auto tile_of = [&](int i) { return list != nullptr ? list[1 + i] : i; };
  int it = blockIdx.x;
  if (it < nitems) LRT_KDA_LOAD(tile_of(it))
  for (; it < nitems; it += gridDim.x) {
    const int tile = tile_of(it);
    // fp32 (twice the operand registers): per-chunk opaque copies of the
    // buffer and global base addresses and of the thread index, so addresses
    // are recomputed inside the loop instead of hoisted out of it and spilled
    // (bf16 has the registers to keep them).
    int z0 = 0;
    tid = threadIdx.x;
    if constexpr (sizeof(E) == 4) {
      asm volatile("" : "+s"(z0));
      asm volatile("" : "+s"(q), "+s"(k), "+s"(v), "+s"(log_a), "+s"(beta), "+s"(wW), "+s"(wUp), "+s"(wKt));
      asm volatile("" : "+s"(wGC), "+s"(wQg), "+s"(wP), "+s"(wT), "+s"(wup));
      asm volatile("" : "+v"(tid));
    }
    const int w = tid >> 6, l = tid & 63;
    char* smz = smem + z0;
    E* sK = (E*)(smz + Lay::K);
    E* sQ = (E*)(smz + Lay::Q);
    E* sV = (E*)(smz + Lay::V);
    float* sG = (float*)(smz + Lay::G);
    E* sS = (E*)(smz + Lay::S);
    float* sA = (float*)(smz + Lay::A);
    E* sT = (E*)(smz + Lay::T);
    E* sTw = sT + C * LC;
    float* sb = (float*)(smz + Lay::BB);
    int* sgmax = (int*)(smz + Lay::FL);
    int cn;
    const int nv = min(C, tile_pos(m, tile, cn).len - cn * C);
    if constexpr (FUSE) {
      tk.normalize_rows(kL2Eps);
      tq.normalize_rows(kL2Eps);
    }
    tk.store_masked(sK, LK, nv);
    tq.store_masked(sQ, LK, nv);
    if constexpr (LOWRANK) {
      // z rows and W_up rows into S (the gate is formed after the barrier)
      tg.store_masked(sS, LZ, nv);
      tw.store(sS + C * LZ, LZ);
    } else if constexpr (FUSE) {
      // log a = -softplus(z) in fp32, rows past the end zero (as store_masked)
      constexpr int GV = 16 / (int)sizeof(GE), GPR = DK / GV;
#pragma unroll
      for (int s2 = 0; s2 < tg.PT; ++s2) {
        const int idx = tid + NT * s2;
        if (tg.NP % NT == 0 || idx < tg.NP) {
          const int r = idx / GPR, c0 = (idx % GPR) * GV;
          GE e[GV];
          __builtin_memcpy(e, &tg.x[s2], 16);
#pragma unroll
          for (int i = 0; i < GV; i += 4) {
            f32x4 y;
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = r < nv ? neg_softplus_f(to_f(e[i + j])) : 0.f;
            *(f32x4*)(sG + r * LG + c0 + i) = y;
          }
        }
      }
    } else {
      tg.store_masked(sG, LG, nv);
    }
    asm volatile("" ::"v"(rb));  // consumed by every lane (no load into it left pending)
    if (tid < C) sb[tid] = tid < nv ? (FUSE ? sigmoid_f(rb) : rb) : 0.f;
    if (tid == 0) *sgmax = 0;
    lds_barrier();
    tv.scale_rows(sb);  // rows past the end scale by 0
    tv.store(sV, LV);
    // the next tile (the last one again on the final pass: unconditional
    // loads keep the waits on older ones exact)
    LRT_KDA_LOAD(tile_of(min(it + (int)gridDim.x, nitems - 1)))
    if constexpr (LOWRANK) {
      // the gate pre-activation W_up z (rows d, cols t; one 16-long MFMA
      // product per tile), then log a = -softplus, rows past the end zero
      for (int tt = w; tt < (DK / 16) * NB; tt += NW) {
        const int td = tt / NB, ti = tt % NB;
        f32x4 acc = zero4();
        mma<R>(acc, sS + C * LZ + td * 16 * LZ, LZ, sS + ti * 16 * LZ, LZ);
        const int t = ti * 16 + (l & 15);
        f32x4 y;
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = t < nv ? neg_softplus_f(acc[r]) : 0.f;
        *(f32x4*)(sG + t * LG + td * 16 + (l >> 4) * 4) = y;
      }
      lds_barrier();
    }
    // ---- G: inclusive cumsum over the chunk's tokens, per key dimension;
    // thread (d, segment) scans RS rows in registers, then adds the totals of
    // the earlier segments
    {
      constexpr int NQ = Lay::NQ, RS = C / NQ;
      float* stot = (float*)sS;
      const int d = tid % DK, seg = tid / DK;
      float x[RS];
      if (seg < NQ) {
#pragma unroll
        for (int r = 0; r < RS; ++r) x[r] = sG[(seg * RS + r) * LG + d];
#pragma unroll
        for (int r = 1; r < RS; ++r) x[r] += x[r - 1];
        stot[seg * DK + d] = x[RS - 1];
      }
      lds_barrier();
      if (seg < NQ) {
        float off = 0.f, m = 0.f;
        for (int s2 = 0; s2 < seg; ++s2) off += stot[s2 * DK + d];
#pragma unroll
        for (int r = 0; r < RS; ++r) {
          sG[(seg * RS + r) * LG + d] = x[r] + off;
          m = fmaxf(m, fabsf(x[r] + off));
        }
        atomicMax(sgmax, __float_as_int(m));  // non-negative floats order as ints
      }
      lds_barrier();
    }
    // Whole-chunk factorization e^(G_i - G_j) = e^(G_i) e^(-G_j) when every
    // |G| <= 60 (both factors stay normal in fp32 / bf16): A and P become one
    // MFMA product each.  Otherwise the exact blocked path below.
    const bool fast = __int_as_float(*sgmax) <= 60.f;
    E* pout = wP + (size_t)tile * C * C;
    if (fast) {
      // KE = K o e^G (over the scaled-operand area), KF = K o e^(-G) (in place of
      // K), QE = Q o e^G (in place of Q; also the Q o e^G output)
      E* sKE = sS;
      E* qg = wQg + (size_t)tile * C * DK;
      for (int p = tid; p < C * (DK / V); p += NT) {
        const int t = p / (DK / V), d0 = (p % (DK / V)) * V;
        float kx[V], qx[V], g[V], ke[V];
        lds_vec_load<E>(sK + t * LK + d0, kx);
        lds_vec_load<E>(sQ + t * LK + d0, qx);
        lds_f32_load<V>(sG + t * LG + d0, g);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float ep = __expf(g[e]), em = __expf(-g[e]);
          ke[e] = kx[e] * ep;
          qx[e] *= ep;
          kx[e] *= em;
        }
        const u32x4 qv = vec_pack<E>(qx);
        *(u32x4*)(sKE + t * LK + d0) = vec_pack<E>(ke);
        *(u32x4*)(sK + t * LK + d0) = vec_pack<E>(kx);
        *(u32x4*)(sQ + t * LK + d0) = qv;
        *(u32x4*)(qg + (size_t)t * DK + d0) = qv;
      }
      lds_barrier();
      // A (lower tiles) = b_i (KE KF^T); P^T tiles = KF QE^T, stored as rows of P
      constexpr int NA = NB * (NB + 1) / 2;
      for (int tt = w; tt < NA + NB * NB; tt += NW) {
        if (tt < NA) {
          int ti = 0, r0 = tt;
          while (r0 > ti) {
            r0 -= ti + 1;
            ++ti;
          }
          const int tj = r0;
          f32x4 acc = zero4();
          mma<DK>(acc, sKE + ti * 16 * LK, LK, sK + tj * 16 * LK, LK);
          const int j = tj * 16 + (l & 15), i0 = ti * 16 + (l >> 4) * 4;
          f32x4 av;
#pragma unroll
          for (int r = 0; r < 4; ++r) av[r] = (j < i0 + r) ? sb[i0 + r] * acc[r] : 0.f;
          *(f32x4*)(sA + j * LA + i0) = av;  // column-major
        } else {
          const int t2 = tt - NA, rj = t2 / NB, ci = t2 % NB;
          f32x4 acc = zero4();
          if (rj <= ci) mma<DK>(acc, sK + rj * 16 * LK, LK, sQ + ci * 16 * LK, LK);
          const int i = ci * 16 + (l & 15), j0 = rj * 16 + (l >> 4) * 4;
          f32x4 p4;
#pragma unroll
          for (int r = 0; r < 4; ++r) p4[r] = (j0 + r <= i) ? acc[r] : 0.f;
          store4<E>(pout + (size_t)i * C + j0, p4);
        }
      }
      // Ktil^T [d][t] = KF[t][d] e^(G_C[d]), and G_C
      E* kt = wKt + (size_t)tile * DK * C;
      if constexpr (std::is_same<E, bf16>::value && C >= 32) {
        // the LDS transpose read hands each lane 8 consecutive tokens of one
        // dimension (16 dimensions x 32 tokens per wave and step): one
        // 16-byte piece of a Ktil^T row, without bank conflicts
        for (int blk = w; blk < (DK / 16) * (C / 32); blk += NW) {
          const int n0 = (blk / (C / 32)) * 16, k0 = (blk % (C / 32)) * 32;
          const bf16x8 f = frag_k8_outer(sK, LK, k0, n0);
          const int d = n0 + (l & 15), t0 = k0 + 8 * (l >> 4);
          const float eC = __expf(sG[(C - 1) * LG + d]);
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = (float)f[e] * eC;
          *(u32x4*)(kt + (size_t)d * C + t0) = vec_pack<E>(x);
        }
      } else {
        for (int p = tid; p < DK * (C / V); p += NT) {
          const int d = p % DK, t0 = (p / DK) * V;  // consecutive lanes, consecutive dimensions
          const float eC = __expf(sG[(C - 1) * LG + d]);
          float x[V];
#pragma unroll
          for (int e = 0; e < V; ++e) x[e] = to_f(sK[(t0 + e) * LK + d]) * eC;
          *(u32x4*)(kt + (size_t)d * C + t0) = vec_pack<E>(x);
        }
      }
      for (int d = tid; d < DK; d += NT) wGC[(size_t)tile * DK + d] = sG[(C - 1) * LG + d];
    } else {
      // ---- elementwise outputs: Q o e^G [t][d], Ktil^T [d][t] = (k_t o e^(G_C - G_t))^T, G_C
      {
        E* qg = wQg + (size_t)tile * C * DK;
        for (int p = tid; p < C * (DK / V); p += NT) {
          const int t = p / (DK / V), d0 = (p % (DK / V)) * V;
          float x[V], g[V];
          lds_vec_load<E>(sQ + t * LK + d0, x);
          lds_f32_load<V>(sG + t * LG + d0, g);
#pragma unroll
          for (int e = 0; e < V; ++e) x[e] *= __expf(g[e]);
          *(u32x4*)(qg + (size_t)t * DK + d0) = vec_pack<E>(x);
        }
        E* kt = wKt + (size_t)tile * DK * C;
        for (int p = tid; p < DK * (C / V); p += NT) {
          const int d = p / (C / V), t0 = (p % (C / V)) * V;
          const float gC = sG[(C - 1) * LG + d];
          float x[V];
#pragma unroll
          for (int e = 0; e < V; ++e) x[e] = to_f(sK[(t0 + e) * LK + d]) * __expf(gC - sG[(t0 + e) * LG + d]);
          *(u32x4*)(kt + (size_t)d * C + t0) = vec_pack<E>(x);
        }
        for (int d = tid; d < DK; d += NT) wGC[(size_t)tile * DK + d] = sG[(C - 1) * LG + d];
      }
      // ---- off-diagonal 16-row blocks: reference r = 16 s, operands scaled in LDS
      //   rows [0, 16):       k_i o e^(G_i - G_r)   (i in block s)
      //   rows [16, 32):      q_i o e^(G_i - G_r)
      //   rows [32, 32 + r):  k_j o e^(G_r - G_j)   (j < r)
      // both exponents are <= 0 (G is non-increasing in t for log a <= 0)
      for (int s = 1; s < NB; ++s) {
        const int r0 = 16 * s, nrow = 32 + r0;
        for (int p = tid; p < nrow * (DK / V); p += NT) {
          const int row = p / (DK / V), d0 = (p % (DK / V)) * V;
          const E* src;
          int t;
          float sgn;
          if (row < 16) {
            src = sK, t = r0 + row, sgn = 1.f;
          } else if (row < 32) {
            src = sQ, t = r0 + row - 16, sgn = 1.f;
          } else {
            src = sK, t = row - 32, sgn = -1.f;
          }
          float x[V], g[V], gr[V];
          lds_vec_load<E>(src + t * LK + d0, x);
          lds_f32_load<V>(sG + t * LG + d0, g);
          lds_f32_load<V>(sG + r0 * LG + d0, gr);
#pragma unroll
          for (int e = 0; e < V; ++e) x[e] *= __expf(sgn * (g[e] - gr[e]));
          *(u32x4*)(sS + row * LK + d0) = vec_pack<E>(x);
        }
        lds_barrier();
        // D[j][i] = sum_d (k_j e^(G_r - G_j)) (k_i or q_i) e^(G_i - G_r): a lane
        // holds 4 consecutive j of one row i
        for (int tt = w; tt < 2 * s; tt += NW) {
          const int kind = tt / s, sj = tt % s;
          f32x4 acc = zero4();
          mma<DK>(acc, sS + (32 + sj * 16) * LK, LK, sS + kind * 16 * LK, LK);
          const int i = r0 + (l & 15), j0 = sj * 16 + (l >> 4) * 4;
          if (kind == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) sA[(j0 + r) * LA + i] = sb[i] * acc[r];  // column-major
          } else {
            store4<E>(pout + (size_t)i * C + j0, acc);
          }
        }
        lds_barrier();
      }
      // ---- diagonal 16 x 16 blocks, element by element with the exact exponent
      // difference: one thread per pair j <= i, 16 bytes of k / q per step
      for (int p = tid; p < NB * 136; p += NT) {
        const int s = p / 136;
        int jj = p % 136, ii = 0;
        while (jj > ii) {
          jj -= ii + 1;
          ++ii;
        }
        const int i = 16 * s + ii, j = 16 * s + jj;
        float akk = 0.f, aqk = 0.f;
        for (int d0 = 0; d0 < DK; d0 += V) {
          float kj[V], ki[V], qi[V], gi[V], gj[V];
          lds_vec_load<E>(sK + j * LK + d0, kj);
          lds_vec_load<E>(sK + i * LK + d0, ki);
          lds_vec_load<E>(sQ + i * LK + d0, qi);
          lds_f32_load<V>(sG + i * LG + d0, gi);
          lds_f32_load<V>(sG + j * LG + d0, gj);
#pragma unroll
          for (int e = 0; e < V; ++e) {
            const float x = kj[e] * __expf(gi[e] - gj[e]);
            akk += ki[e] * x;
            aqk += qi[e] * x;
          }
        }
        if (j < i) sA[j * LA + i] = sb[i] * akk;  // column-major
        pout[(size_t)i * C + j] = from_f<E>(aqk);
      }
      // P above the diagonal is zero: whole blocks (16-byte stores) and the
      // upper triangles of the diagonal blocks
      for (int p = tid; p < C * (C / V); p += NT) {
        const int i = p / (C / V), j0 = (p % (C / V)) * V;
        if ((j0 >> 4) > (i >> 4)) *(u32x4*)(pout + (size_t)i * C + j0) = u32x4{0u, 0u, 0u, 0u};
      }
      for (int p = tid; p < NB * 256; p += NT) {
        const int s = p >> 8, ii = (p >> 4) & 15, jj = p & 15;
        if (jj > ii) pout[(size_t)(16 * s + ii) * C + 16 * s + jj] = from_f<E>(0.f);
      }
    }
    lds_barrier();
    unit_lower_inverse<C, NT>(sA);
    // T and T diag(b) in E; X = K o e^G rows (the fast path staged them already)
    E* sX = sS;
    // (a thread fills V consecutive columns of one row: consecutive lanes read
    // consecutive rows of the column-major inverse and write 16-byte pieces)
    for (int p = tid; p < C * (C / V); p += NT) {
      const int i = p % C, j0 = (p / C) * V;
      float x[V], xw[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        x[e] = j0 + e <= i ? sA[(j0 + e) * LA + i] : 0.f;
        xw[e] = x[e] * sb[j0 + e];
      }
      *(u32x4*)(sT + i * LC + j0) = vec_pack<E>(x);
      *(u32x4*)(sTw + i * LC + j0) = vec_pack<E>(xw);
    }
    if (!fast) {
      for (int p = tid; p < C * (DK / V); p += NT) {
        const int t = p / (DK / V), d0 = (p % (DK / V)) * V;
        float x[V], g[V];
        lds_vec_load<E>(sK + t * LK + d0, x);
        lds_f32_load<V>(sG + t * LG + d0, g);
#pragma unroll
        for (int e = 0; e < V; ++e) x[e] *= __expf(g[e]);
        *(u32x4*)(sX + t * LK + d0) = vec_pack<E>(x);
      }
    }
    lds_barrier();
    if (wT != nullptr) lds_to_block<E, C, C, NT>(wT + (size_t)tile * C * C, sT, LC);
    // W^T = X^T (T diag(b))^T (rows d, cols t): 4 consecutive d of one row of W
    // per lane; U' = T (b V) (rows t, cols v) in accumulator-tile order (a
    // wave's 64 lanes write 512 contiguous bytes; the scan reads it per lane)
    constexpr int NWT = (DK / 16) * NB, NUT = NB * (DV / 16);
    for (int tt = w; tt < NWT + NUT; tt += NW) {
      f32x4 acc = zero4();
      if (tt < NWT) {
        const int td = tt / NB, ti = tt % NB;
        mma<C, true, false>(acc, sX + td * 16, LK, sTw + ti * 16 * LC, LC);
        store4<E>(wW + ((size_t)tile * C + ti * 16 + (l & 15)) * DK + td * 16 + (l >> 4) * 4, acc);
      } else {
        const int u = tt - NWT, ti = u / (DV / 16), tvb = u % (DV / 16);
        mma<C, false, true>(acc, sT + ti * 16 * LC, LC, sV + tvb * 16, LV);
        acc_tile_store<E>(wUp + (size_t)tile * DV * C, ti * (DV / 16) + tvb, acc);
      }
    }
    lds_barrier();
  }
#undef LRT_KDA_LOAD
}

}  // namespace lrt

namespace lrt {

// ------------------------------------------------------------ k_kda_prep_fast
// k_kda_prep's fast path (every |G| <= 60 in the chunk, so A and P are one
// MFMA product each) in 4-wave workgroups that need at most half of a CU's
// LDS: two workgroups share a CU and one's barriers overlap the other's work.
// G is formed and consumed one half of d_k at a time (cumsum, then the scaled
// rows K o e^G, K o e^-G, Q o e^G of that half); A, then the b v rows, reuse
// the half-G area, T and T diag(b) the dead K o e^-G and Q o e^G areas.  A
// chunk whose |G| exceeds 60 is appended to `slow` (count in slow[0], tiles
// from slow[1]) and left to k_kda_prep's exact path.  Outputs as k_kda_prep.
// LOWRANK (with FUSE): the gate as its rank-kGateRank factors, log_a_ = z
// [tokens][R] and wup = W_up [H * d_k][R]; z and one half's W_up rows sit in
// the columns [d_k/2, d_k/2 + 2R) of the K o e^G rows, free until that half
// is staged, and the half's pre-activation W_up z is one MFMA product.
template <typename E, int C, int DK, int DV>
struct KdaFastLds {
  static constexpr int NT = 256;
  static constexpr int P = lds_pad<E>();
  static constexpr int LK = DK + P, LV = DV + P, LC = C + P, DH = DK / 2, LGH = DH + 4, LA = tri_ld<C>();
  static constexpr int NQ = NT / DH < C ? NT / DH : C;  // row segments of the cumsum
  static constexpr size_t es = sizeof(E);
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t al(size_t x) { return (x + 15) & ~(size_t)15; }
  static constexpr size_t RKQ = al(mx((size_t)C * LK * es, (size_t)C * LC * es));
  static constexpr size_t K = 0;          // k rows -> K o e^-G -> T
  static constexpr size_t Q = K + RKQ;    // q rows -> Q o e^G -> T diag(b)
  static constexpr size_t S = Q + RKQ;    // K o e^G (X)
  static constexpr size_t GA = S + al((size_t)C * LK * es);  // G (half of d_k) -> A (fp32) -> b v rows
  static constexpr size_t GASZ = mx(mx((size_t)C * LGH * 4, (size_t)C * LA * 4), (size_t)C * LV * es);
  static constexpr size_t BB = GA + al(GASZ);           // b [C]
  static constexpr size_t GCA = BB + C * 4;             // G_C [d_k]
  static constexpr size_t STOT = GCA + DK * 4;          // [NQ][DH] segment totals
  static constexpr size_t FL = STOT + (size_t)NQ * DH * 4;  // max |G| over the chunk (float bits)
  static constexpr size_t TOTAL = FL + 16;
};

// slow[0] = 0 before k_kda_prep_fast appends to the list.
template <int = 0>
__global__ void k_list_reset(int* slow) {
  if (threadIdx.x == 0) slow[0] = 0;
}

// Whether the low-rank gate's staging fits the fast kernel's layout.
template <typename E, int C, int DK, int DV>
constexpr bool kda_fast_lowrank_fits() {
  return DK / 2 + 2 * kGateRank <= KdaFastLds<E, C, DK, DV>::LK && DK / 2 <= C;
}

template <typename E, int C, int DK, int DV, bool FUSE = false, bool LOWRANK = false>
__global__ __launch_bounds__(256, 2) void k_kda_prep_fast(const E* __restrict__ q, const E* __restrict__ k,
                                                          const E* __restrict__ v, const void* __restrict__ log_a_,
                                                          const float* __restrict__ beta, SeqMap m,
                                                          E* __restrict__ wW, E* __restrict__ wUp,
                                                          E* __restrict__ wKt, float* __restrict__ wGC,
                                                          E* __restrict__ wQg, E* __restrict__ wP,
                                                          E* __restrict__ wT, int* __restrict__ slow,
                                                          const E* __restrict__ wup) {
  typedef KdaFastLds<E, C, DK, DV> Lay;
  static_assert(!LOWRANK || (FUSE && kda_fast_lowrank_fits<E, C, DK, DV>()), "low-rank gate staging");
  constexpr int NT = 256, NW = 4;
  constexpr int LK = Lay::LK, LV = Lay::LV, LC = Lay::LC, DH = Lay::DH, LGH = Lay::LGH, LA = Lay::LA;
  constexpr int NQ = Lay::NQ, NB = C / 16;
  constexpr int V = 16 / (int)sizeof(E);
  static_assert(DH % V == 0, "a half of d_k holds whole 16-byte pieces");
  static_assert(C % NQ == 0 && NQ * DH <= NT, "cumsum segments");
  __shared__ __attribute__((aligned(16))) char smem[Lay::TOTAL];
  E* sK = (E*)(smem + Lay::K);
  E* sT = sK;
  E* sQ = (E*)(smem + Lay::Q);
  E* sTw = sQ;
  E* sS = (E*)(smem + Lay::S);
  float* sG = (float*)(smem + Lay::GA);
  float* sA = sG;
  E* sV = (E*)(smem + Lay::GA);
  float* sb = (float*)(smem + Lay::BB);
  float* sGC = (float*)(smem + Lay::GCA);
  float* stot = (float*)(smem + Lay::STOT);
  int* sgmax = (int*)(smem + Lay::FL);
  const int w = wave_id(), l = lane_id(), tid = threadIdx.x;
  const int H = m.H, ntiles = tile_count(m);

  typedef typename std::conditional<FUSE, E, float>::type GE;  // element type of the gate input
  const GE* log_a = (const GE*)log_a_;  // LOWRANK: z [tokens][R]
  constexpr int GV = 16 / (int)sizeof(GE), GPR = DK / GV;  // gate elements per piece, pieces per row
  static_assert(DH % GV == 0, "a gate piece lies in one half of d_k");
  constexpr int R = kGateRank;
  Tile<E, C, DK, NT> tk, tq;
  Tile<E, C, DV, NT> tv;
  Tile<GE, C, LOWRANK ? R : DK, NT> tg;
  Tile<E, LOWRANK ? DH : 16, LOWRANK ? R : 16, NT> tw0, tw1;  // LOWRANK: this head's W_up rows, by half
  float rb = 0.f;
  // the next tile's inputs in three parts, each issued once the current
  // tile's copy of it has reached LDS: 1 k, q, beta; 2 the gate; 4 v
#define LRT_KF_LOAD(tile_, PART_)                                                       \
  {                                                                                     \
    int ln;                                                                             \
    const SeqPos lp = tile_pos(m, (tile_), ln);                                         \
    const int lnv = min(C, lp.len - ln * C);                                            \
    const size_t ltok = lp.tok0 + (size_t)ln * C;                                       \
    const int lh = lp.h;                                                                \
    if ((PART_) & 1) {                                                                  \
      tk.load_rows_clamped(k + (ltok * H + lh) * DK, (size_t)H * DK, lnv);              \
      tq.load_rows_clamped(q + (ltok * H + lh) * DK, (size_t)H * DK, lnv);              \
      rb = beta[(ltok + min(tid, lnv - 1)) * H + lh]; /* masked where used */           \
    }                                                                                   \
    if ((PART_) & 2) {                                                                  \
      if constexpr (LOWRANK) {                                                          \
        tg.load_rows_clamped(log_a + ltok * R, (size_t)R, lnv);                         \
        tw0.load_block(wup + (size_t)lh * DK * R);                                      \
        tw1.load_block(wup + ((size_t)lh * DK + DH) * R);                               \
      } else {                                                                          \
        tg.load_rows_clamped(log_a + (ltok * H + lh) * DK, (size_t)H * DK, lnv);        \
      }                                                                                 \
    }                                                                                   \
    if ((PART_) & 4) tv.load_rows_clamped(v + (ltok * H + lh) * DV, (size_t)H * DV, lnv); \
  }

  int tile = blockIdx.x;
  if (tile < ntiles) LRT_KF_LOAD(tile, 7)
  for (; tile < ntiles; tile += gridDim.x) {
    int cn;
    const int nv = min(C, tile_pos(m, tile, cn).len - cn * C);
    const int next = min(tile + (int)gridDim.x, ntiles - 1);
    if constexpr (FUSE) {
      tk.normalize_rows(kL2Eps);
      tq.normalize_rows(kL2Eps);
    }
    tk.store_masked(sK, LK, nv);
    tq.store_masked(sQ, LK, nv);
    if constexpr (LOWRANK) {
      tg.store_masked(sS + DH, LK, nv);  // z rows
      tw0.store(sS + DH + R, LK);        // W_up rows of the first half
    }
    asm volatile("" ::"v"(rb));  // consumed by every lane (no load into it left pending)
    if (tid < C) sb[tid] = tid < nv ? (FUSE ? sigmoid_f(rb) : rb) : 0.f;
    if (tid == 0) *sgmax = 0;
    LRT_KF_LOAD(next, 1)
    // ---- per half of d_k: G (cumsum of log a, rows past the end add 0), then
    // the scaled rows of that half
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      if constexpr (LOWRANK) {
        // this half's pre-activation W_up z (rows d, cols t) on MFMA, then
        // log a = -softplus, rows past the end zero
        if (hf == 1) tw1.store(sS + DH + R, LK);  // (the first half's rows are dead)
        lds_barrier();
        for (int tt = w; tt < (DH / 16) * NB; tt += NW) {
          const int td = tt / NB, ti = tt % NB;
          f32x4 acc = zero4();
          mma<R>(acc, sS + DH + R + td * 16 * LK, LK, sS + DH + ti * 16 * LK, LK);
          const int t = ti * 16 + (l & 15);
          f32x4 y;
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = t < nv ? neg_softplus_f(acc[r]) : 0.f;
          *(f32x4*)(sG + t * LGH + td * 16 + (l >> 4) * 4) = y;
        }
      }
#pragma unroll
      for (int s2 = 0; s2 < (LOWRANK ? 0 : tg.PT); ++s2) {
        const int idx = tid + NT * s2;
        if (tg.NP % NT == 0 || idx < tg.NP) {
          const int r = idx / GPR, c0 = (idx % GPR) * GV;
          if (c0 / DH == hf) {
            GE e[GV];
            __builtin_memcpy(e, &tg.x[s2], 16);
#pragma unroll
            for (int i = 0; i < GV; i += 4) {
              f32x4 y;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float z = to_f(e[i + j]);
                y[j] = r < nv ? (FUSE ? neg_softplus_f(z) : z) : 0.f;
              }
              *(f32x4*)(sG + r * LGH + c0 - hf * DH + i) = y;
            }
          }
        }
      }
      if (hf == 1) LRT_KF_LOAD(next, 2)
      lds_barrier();
      {
        constexpr int RS = C / NQ;
        const int d = tid % DH, seg = tid / DH;
        float x[RS];
        if (seg < NQ) {
#pragma unroll
          for (int r = 0; r < RS; ++r) x[r] = sG[(seg * RS + r) * LGH + d];
#pragma unroll
          for (int r = 1; r < RS; ++r) x[r] += x[r - 1];
          stot[seg * DH + d] = x[RS - 1];
        }
        lds_barrier();
        if (seg < NQ) {
          float off = 0.f, mm = 0.f;
          for (int s2 = 0; s2 < seg; ++s2) off += stot[s2 * DH + d];
#pragma unroll
          for (int r = 0; r < RS; ++r) {
            sG[(seg * RS + r) * LGH + d] = x[r] + off;
            mm = fmaxf(mm, fabsf(x[r] + off));
          }
          if (seg == NQ - 1) sGC[hf * DH + d] = x[RS - 1] + off;
          atomicMax(sgmax, __float_as_int(mm));  // non-negative floats order as ints
        }
        lds_barrier();
      }
      // KE = K o e^G (into S), KF = K o e^-G (in place of K), QE = Q o e^G
      // (in place of Q), for this half's columns
      for (int p = tid; p < C * (DH / V); p += NT) {
        const int t = p / (DH / V), dh = (p % (DH / V)) * V, d0 = hf * DH + dh;
        float kx[V], qx[V], g[V], ke[V];
        lds_vec_load<E>(sK + t * LK + d0, kx);
        lds_vec_load<E>(sQ + t * LK + d0, qx);
        lds_f32_load<V>(sG + t * LGH + dh, g);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float ep = __expf(g[e]), em = __expf(-g[e]);
          ke[e] = kx[e] * ep;
          qx[e] *= ep;
          kx[e] *= em;
        }
        *(u32x4*)(sS + t * LK + d0) = vec_pack<E>(ke);
        *(u32x4*)(sK + t * LK + d0) = vec_pack<E>(kx);
        *(u32x4*)(sQ + t * LK + d0) = vec_pack<E>(qx);
      }
      lds_barrier();  // (the next half overwrites G)
    }
    if (__int_as_float(*sgmax) > 60.f) {
      // the exact path's chunk: k_kda_prep takes it from the list
      if (tid == 0) slow[1 + atomicAdd(slow, 1)] = tile;
      lds_barrier();  // every wave has read the flag before the next chunk resets it
      LRT_KF_LOAD(next, 4)
      continue;
    }
    // ---- A (lower tiles) = b_i (KE KF^T); P rows from P^T tiles = KF QE^T;
    // Q o e^G rows out; Ktil^T [d][t] = KF[t][d] e^(G_C[d]); G_C
    E* pout = wP + (size_t)tile * C * C;
    lds_to_block<E, C, DK, NT>(wQg + (size_t)tile * C * DK, sQ, LK);
    constexpr int NA = NB * (NB + 1) / 2;
    for (int tt = w; tt < NA + NB * NB; tt += NW) {
      if (tt < NA) {
        int ti = 0, r0 = tt;
        while (r0 > ti) {
          r0 -= ti + 1;
          ++ti;
        }
        const int tj = r0;
        f32x4 acc = zero4();
        mma<DK>(acc, sS + ti * 16 * LK, LK, sK + tj * 16 * LK, LK);
        const int j = tj * 16 + (l & 15), i0 = ti * 16 + (l >> 4) * 4;
        f32x4 av;
#pragma unroll
        for (int r = 0; r < 4; ++r) av[r] = (j < i0 + r) ? sb[i0 + r] * acc[r] : 0.f;
        *(f32x4*)(sA + j * LA + i0) = av;  // column-major
      } else {
        const int t2 = tt - NA, rj = t2 / NB, ci = t2 % NB;
        f32x4 acc = zero4();
        if (rj <= ci) mma<DK>(acc, sK + rj * 16 * LK, LK, sQ + ci * 16 * LK, LK);
        const int i = ci * 16 + (l & 15), j0 = rj * 16 + (l >> 4) * 4;
        f32x4 p4;
#pragma unroll
        for (int r = 0; r < 4; ++r) p4[r] = (j0 + r <= i) ? acc[r] : 0.f;
        store4<E>(pout + (size_t)i * C + j0, p4);
      }
    }
    E* kt = wKt + (size_t)tile * DK * C;
    if constexpr (std::is_same<E, bf16>::value && C >= 32) {
      for (int blk = w; blk < (DK / 16) * (C / 32); blk += NW) {
        const int n0 = (blk / (C / 32)) * 16, k0 = (blk % (C / 32)) * 32;
        const bf16x8 f = frag_k8_outer(sK, LK, k0, n0);
        const int d = n0 + (l & 15), t0 = k0 + 8 * (l >> 4);
        const float eC = __expf(sGC[d]);
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (float)f[e] * eC;
        *(u32x4*)(kt + (size_t)d * C + t0) = vec_pack<E>(x);
      }
    } else {
      for (int p = tid; p < DK * (C / V); p += NT) {
        const int d = p % DK, t0 = (p / DK) * V;
        const float eC = __expf(sGC[d]);
        float x[V];
#pragma unroll
        for (int e = 0; e < V; ++e) x[e] = to_f(sK[(t0 + e) * LK + d]) * eC;
        *(u32x4*)(kt + (size_t)d * C + t0) = vec_pack<E>(x);
      }
    }
    for (int d = tid; d < DK; d += NT) wGC[(size_t)tile * DK + d] = sGC[d];
    lds_barrier();
    unit_lower_inverse<C, NT>(sA);
    // T and T diag(b) over the dead KF and QE rows
    for (int p = tid; p < C * (C / V); p += NT) {
      const int i = p % C, j0 = (p / C) * V;
      float x[V], xw[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        x[e] = j0 + e <= i ? sA[(j0 + e) * LA + i] : 0.f;
        xw[e] = x[e] * sb[j0 + e];
      }
      *(u32x4*)(sT + i * LC + j0) = vec_pack<E>(x);
      *(u32x4*)(sTw + i * LC + j0) = vec_pack<E>(xw);
    }
    lds_barrier();
    if (wT != nullptr) lds_to_block<E, C, C, NT>(wT + (size_t)tile * C * C, sT, LC);
    tv.scale_rows(sb);  // rows past the end scale by 0
    tv.store(sV, LV);   // b v rows over the dead A
    LRT_KF_LOAD(next, 4)
    lds_barrier();
    // W^T = X^T (T diag(b))^T; U' = T (b V) in accumulator-tile order
    constexpr int NWT = (DK / 16) * NB, NUT = NB * (DV / 16);
    for (int tt = w; tt < NWT + NUT; tt += NW) {
      f32x4 acc = zero4();
      if (tt < NWT) {
        const int td = tt / NB, ti = tt % NB;
        mma<C, true, false>(acc, sS + td * 16, LK, sTw + ti * 16 * LC, LC);
        store4<E>(wW + ((size_t)tile * C + ti * 16 + (l & 15)) * DK + td * 16 + (l >> 4) * 4, acc);
      } else {
        const int u = tt - NWT, ti = u / (DV / 16), tvb = u % (DV / 16);
        mma<C, false, true>(acc, sT + ti * 16 * LC, LC, sV + tvb * 16, LV);
        acc_tile_store<E>(wUp + (size_t)tile * DV * C, ti * (DV / 16) + tvb, acc);
      }
    }
    lds_barrier();
  }
#undef LRT_KF_LOAD
}

// The chunk-parallel pass of the KDA forward: k_kda_prep_fast (two
// workgroups per CU) where it fits in half of a CU's LDS (and, for the
// low-rank gate, where its staging fits), with k_kda_prep taking the chunks
// it leaves to the exact path; k_kda_prep alone otherwise.  wT (nullable): also write Tinv.  fast_kind /
// kind: the timing hook's ids of the two kernels.
template <typename E, int C, int DK, int DV, bool FUSE, bool LOWRANK = false>
int launch_kda_prep(const void* q, const void* k, const void* v, const void* log_a, const float* beta,
                    const SeqMap& sm, const FwdWs& ws, E* wT, const void* wup, int tiles, int fast_kind, int kind,
                    hipStream_t st) {
  typedef KdaLds<E, C, DK, DV, 64 * kWyWaves> Lay;
  if constexpr (KdaFastLds<E, C, DK, DV>::TOTAL <= kLdsMax / 2 &&
                (!LOWRANK || kda_fast_lowrank_fits<E, C, DK, DV>())) {
    LRT_LAUNCH(kKListReset, k_list_reset<>, dim3(1), dim3(64), st, ws.slow);
    LRT_LAUNCH(fast_kind, (k_kda_prep_fast<E, C, DK, DV, FUSE, LOWRANK>),
               dim3(persistent_grid(tiles, KdaFastLds<E, C, DK, DV>::TOTAL)), dim3(256), st, (const E*)q, (const E*)k,
               (const E*)v, log_a, beta, sm, (E*)ws.W, (E*)ws.Up, (E*)ws.Kt, ws.GC, (E*)ws.Qg, (E*)ws.P, wT,
               ws.slow, (const E*)wup);
    LRT_LAUNCH(kind, (k_kda_prep<E, C, DK, DV, kWyWaves, FUSE, LOWRANK>), dim3(persistent_grid(tiles, Lay::TOTAL)),
               dim3(64 * kWyWaves), st, (const E*)q, (const E*)k, (const E*)v, log_a, beta, sm, (E*)ws.W,
               (E*)ws.Up, (E*)ws.Kt, ws.GC, (E*)ws.Qg, (E*)ws.P, wT, (const E*)wup, (const int*)ws.slow);
  } else {
    LRT_LAUNCH(kind, (k_kda_prep<E, C, DK, DV, kWyWaves, FUSE, LOWRANK>), dim3(persistent_grid(tiles, Lay::TOTAL)),
               dim3(64 * kWyWaves), st, (const E*)q, (const E*)k, (const E*)v, log_a, beta, sm, (E*)ws.W,
               (E*)ws.Up, (E*)ws.Kt, ws.GC, (E*)ws.Qg, (E*)ws.P, wT, (const E*)wup, (const int*)nullptr);
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace lrt
