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

// LDS writes of one wave made visible to the rest of that wave: the wave's
// LDS operations complete in order, the clobber keeps the compiler from
// moving reads above the writes.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Triangular matrices of a chunk (A, then its inverse in place) live in LDS
// column-major, element (r, c) at p[c * tri_ld<C>() + r]: a column of four
// consecutive rows is one 16-byte access.
template <int C>
constexpr int tri_ld() {
  return C + 4;
}

// One 16 x 16 x 16 fp32 product on the 16x16x4 MFMA from column-major LDS
// blocks: acc += X Y with X(m, k) at x[k * ld + m], Y(k, n) at y[n * ld + k].
// Lane group g feeds k = 4g + s at step s.
__device__ __forceinline__ void mma16_cm(f32x4& acc, const float* x, const float* y, int ld) {
  const int l = lane_id(), g = l >> 4, j = l & 15;
  const f32x4 yv = *(const f32x4*)(y + j * ld + 4 * g);
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[(4 * g + s) * ld + j], yv[s], acc, 0, 0, 0);
}

// Store a 16 x 16 accumulator tile (times sc) column-major: D(m, n) at d[n * ld + m].
__device__ __forceinline__ void acc16_store_cm(float* d, int ld, f32x4 acc, float sc) {
  const int l = lane_id();
  *(f32x4*)(d + (l & 15) * ld + (l >> 4) * 4) = sc * acc;
}

// Broadcast lane q of every group of four lanes to the whole group (DPP).
template <int Q>
__device__ __forceinline__ float quad_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), Q * 0x55, 0xf, 0xf, false));
}

// (I + A)^-1 for a strictly lower-triangular C x C matrix A (fp32, C in
// {16, 32, 64}), column-major in LDS with leading dimension tri_ld<C>(),
// computed in place.  Only the lower triangle, diagonal included, is defined
// on return: the strictly upper off-diagonal 16-blocks serve as scratch.
//   stage 1  the 16 x 16 diagonal blocks by forward substitution, one wave per
//            block, four lanes per column (each holding four rows): after
//            x_m is known (a DPP broadcast inside the group of four) every
//            later row takes its term, and the column of A that step m needs
//            is one 16-byte read per lane, independent of x;
//   stage 2  doubling to 32 x 32: [[X, 0], [Y, Z]]^-1 has lower-left block
//            -Z^-1 Y X^-1, two fp32 MFMA products in the wave that owns the
//            upper diagonal block (so no workgroup barrier in between);
//   stage 3  (C = 64) the same doubling to 64 x 64 with 32 x 32 blocks, the
//            four 16-block outputs of each product on four waves.
// All NT threads must call it after A is visible to them; the result is
// visible to all threads on return.
template <int C, int NT = kThreads>
__device__ __forceinline__ void unit_lower_inverse(float* p) {
  static_assert(C == 16 || C == 32 || C == 64, "chunk must be 16, 32 or 64");
  static_assert(NT >= 256, "the 64 x 64 doubling uses four waves");
  constexpr int NB = C / 16;
  constexpr int LD = tri_ld<C>();
  const int w = wave_id(), l = lane_id();
  if (w < NB) {
    // stage 1: block bb = w; lane (column j, row quarter rq) holds rows 4rq..4rq+3
    const int bb = w, j = l >> 2, rq = l & 3;
    float* blk = p + bb * 16 * LD + bb * 16;  // block (bb, bb)
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (4 * rq + i == j) ? 1.f : 0.f;
    // columns of A four steps at a time, the next four loading meanwhile
    f32x4 cur[4], nxt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cur[i] = *(const f32x4*)(blk + i * LD + 4 * rq);  // A(4rq.., m)
#define LRT_INV_STEP(m_, a_)                                                                      \
  {                                                                                               \
    const float xm = quad_bcast<((m_) >> 2)>(x[(m_) & 3]);                                        \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) if (4 * rq + i > (m_)) x[i] -= (a_)[i] * xm;    \
  }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (g < 3) {
#pragma unroll
        for (int i = 0; i < 4; ++i) nxt[i] = *(const f32x4*)(blk + min(4 * g + 4 + i, 14) * LD + 4 * rq);
      }
      if (g == 0) { LRT_INV_STEP(0, cur[0]) LRT_INV_STEP(1, cur[1]) LRT_INV_STEP(2, cur[2]) LRT_INV_STEP(3, cur[3]) }
      if (g == 1) { LRT_INV_STEP(4, cur[0]) LRT_INV_STEP(5, cur[1]) LRT_INV_STEP(6, cur[2]) LRT_INV_STEP(7, cur[3]) }
      if (g == 2) { LRT_INV_STEP(8, cur[0]) LRT_INV_STEP(9, cur[1]) LRT_INV_STEP(10, cur[2]) LRT_INV_STEP(11, cur[3]) }
      if (g == 3) { LRT_INV_STEP(12, cur[0]) LRT_INV_STEP(13, cur[1]) LRT_INV_STEP(14, cur[2]) }
#pragma unroll
      for (int i = 0; i < 4; ++i) cur[i] = nxt[i];
    }
#undef LRT_INV_STEP
    *(f32x4*)(blk + j * LD + 4 * rq) = f32x4{x[0], x[1], x[2], x[3]};
  }
  if constexpr (NB > 1) {
    lds_barrier();
    // stage 2: wave w < NB/2 fills T[2w+1][2w] = -T[2w+1][2w+1] (A[2w+1][2w] T[2w][2w]),
    // the intermediate in the upper block [2w][2w+1]
    if (w < NB / 2) {
      const int b0 = 2 * w * 16, b1 = b0 + 16;
      f32x4 y = zero4();
      mma16_cm(y, p + b0 * LD + b1, p + b0 * LD + b0, LD);
      acc16_store_cm(p + b1 * LD + b0, LD, y, 1.f);
      wave_lds_sync();
      f32x4 z = zero4();
      mma16_cm(z, p + b1 * LD + b1, p + b1 * LD + b0, LD);
      acc16_store_cm(p + b0 * LD + b1, LD, z, -1.f);
    }
  }
  if constexpr (NB == 4) {
    lds_barrier();
    // stage 3a: X = A[hi][lo] T[lo] (32 x 32) into the upper rows 0..31,
    // columns 32..63; wave w makes 16-block (a, b) = (2 + w/2, w%2)
    if (w < 4) {
      const int a = 2 + (w >> 1), b = w & 1;
      f32x4 x = zero4();
      for (int c = b; c < 2; ++c) mma16_cm(x, p + c * 16 * LD + a * 16, p + b * 16 * LD + c * 16, LD);
      acc16_store_cm(p + (2 + b) * 16 * LD + (a - 2) * 16, LD, x, 1.f);
    }
    lds_barrier();
    // stage 3b: T[a][b] = -sum_{c=2..a} T[a][c] X[c][b]
    if (w < 4) {
      const int a = 2 + (w >> 1), b = w & 1;
      f32x4 t = zero4();
      for (int c = 2; c <= a; ++c)
        mma16_cm(t, p + c * 16 * LD + a * 16, p + (2 + b) * 16 * LD + (c - 2) * 16, LD);
      acc16_store_cm(p + b * 16 * LD + a * 16, LD, t, -1.f);
    }
  }
  lds_barrier();
}

// LDS of k_prep, with the live ranges overlaid: K rows until K K^T is formed,
// then the fp32 inverse; A until it is inverted, then Tinv in E.
template <typename E, int C, int DK, int DV, bool DELTA>
struct PrepLds {
  static constexpr int P = lds_pad<E>();
  static constexpr int LK = DK + P, LC = C + P, LA = tri_ld<C>();
  static constexpr size_t es = sizeof(E);
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t K = 0;
  static constexpr size_t A = K + mx((size_t)C * LK * es, DELTA ? (size_t)C * LA * 4 : 0);
  static constexpr size_t XT = A + (DELTA ? mx((size_t)C * LA * 4, (size_t)C * LK * es) : 0);
  static constexpr size_t YT = XT + (DELTA ? (size_t)(DK > DV ? DK : DV) * LC * es : 0);
  static constexpr size_t G = YT + (size_t)DV * LC * es;
  static constexpr size_t TOTAL = G + 4 * C * 4;
};

// Chunk-parallel: each workgroup walks tiles blockIdx.x, + gridDim.x, ...,
// with the next tile's inputs loading into registers while this one computes.
// WRITE_T (backward only) also stores Tinv [C][C] per chunk.
template <typename E, int C, int DK, int DV, bool DELTA, bool WRITE_T = false>
__global__ __launch_bounds__(kThreads) void k_prep(const E* __restrict__ k, const E* __restrict__ v,
                                                   const float* __restrict__ log_a,
                                                   const float* __restrict__ beta, int T, int H, int N,
                                                   int ntiles, E* __restrict__ wW, E* __restrict__ wUp,
                                                   E* __restrict__ wKt, float* __restrict__ wG,
                                                   E* __restrict__ wT) {
  typedef PrepLds<E, C, DK, DV, DELTA> Lay;
  constexpr int LK = Lay::LK, LC = Lay::LC, LA = Lay::LA;
  constexpr int NB = C / 16;
  constexpr int V = 16 / (int)sizeof(E);
  __shared__ __attribute__((aligned(16))) char smem[Lay::TOTAL];
  E* sK = (E*)(smem + Lay::K);
  float* sA = (float*)(smem + Lay::A);
  E* sT = (E*)(smem + Lay::K);
  E* sXt = (E*)(smem + Lay::XT);
  E* sYt = (E*)(smem + Lay::YT);
  float* sg = (float*)(smem + Lay::G);
  float* sgam = sg + C;
  float* sb = sg + 2 * C;
  float* sbg = sg + 3 * C;
  const int w = wave_id(), l = lane_id();

  Tile<E, C, DK> tk;
  Tile<E, C, DV> tv;
  float la = 0.f, bt = 0.f;
#define LRT_PREP_LOAD(tile_)                                                              \
  {                                                                                       \
    const int ln = (tile_) % N, lbh = (tile_) / N;                                        \
    const int lnv = min(C, T - ln * C);                                                   \
    const size_t ltok = (size_t)(lbh / H) * T + (size_t)ln * C;                           \
    const int lh = lbh % H;                                                               \
    tk.load_rows(k + (ltok * H + lh) * DK, (size_t)H * DK, lnv);                          \
    tv.load_rows(v + (ltok * H + lh) * DV, (size_t)H * DV, lnv);                          \
    la = 0.f;                                                                             \
    bt = 0.f;                                                                             \
    if (threadIdx.x < lnv) {                                                              \
      la = log_a[(ltok + threadIdx.x) * H + lh];                                          \
      if (DELTA) bt = beta[(ltok + threadIdx.x) * H + lh];                                \
    }                                                                                     \
  }

  int tile = blockIdx.x;
  if (tile < ntiles) LRT_PREP_LOAD(tile)
  for (; tile < ntiles; tile += gridDim.x) {
    if (threadIdx.x < 64) {
      const int t = threadIdx.x;
      const float g = wave_incl_scan(la);
      if (t < C) {
        const float gam = __expf(g);
        sg[t] = g;
        sgam[t] = gam;
        sb[t] = bt;
        sbg[t] = bt * gam;
        wG[(size_t)tile * C + t] = g;
      }
    }
    tk.store(sK, LK);
    lds_barrier();
    // Y^T = (diag(b) V)^T (SSD: V^T) -> sYt[v][t]
    if (DELTA) tv.scale_rows(sb);
    tv.store_T(sYt, LC);
    if constexpr (DELTA) {
      // X^T = (diag(b gamma) K)^T -> sXt[d][t], from the registers of K
      tk.scale_rows(sbg);
      tk.store_T(sXt, LC);
    }
    // Ktil^T[d][t] = e^(g_C - g_t) k_t[d] -> workspace, 16 bytes per store
    {
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
    // every register tile is consumed: start loading the next one
    if (tile + (int)gridDim.x < ntiles) LRT_PREP_LOAD(tile + (int)gridDim.x)
    if constexpr (!DELTA) {
      lds_barrier();
      E* out = wUp + (size_t)tile * DV * C;
      for (int idx = threadIdx.x; idx < DV * (C / V); idx += kThreads) {
        const int c = idx / (C / V), t = (idx % (C / V)) * V;
        *(u32x4*)(out + (size_t)c * C + t) = *(const u32x4*)(sYt + c * LC + t);
      }
      lds_barrier();
    } else {
      // A = strict_lower(b_i (k_i . k_j) e^(g_i - g_j))
      for (int tt = w; tt < NB * NB; tt += kWaves) {
        const int ti = tt / NB, tj = tt % NB;
        f32x4 acc = zero4();
        if (tj <= ti) mma<DK>(acc, sK + ti * 16 * LK, LK, sK + tj * 16 * LK, LK);
        const int j = tj * 16 + (l & 15);
        const int i0 = ti * 16 + (l >> 4) * 4;
        f32x4 av;
#pragma unroll
        for (int r = 0; r < 4; ++r) av[r] = (j < i0 + r) ? sb[i0 + r] * acc[r] * __expf(sg[i0 + r] - sg[j]) : 0.f;
        *(f32x4*)(sA + j * LA + i0) = av;  // column-major
      }
      lds_barrier();
      unit_lower_inverse<C>(sA);
      for (int idx = threadIdx.x; idx < C * C; idx += kThreads) {
        const int j = idx / C, i = idx % C;
        const E x = from_f<E>(j <= i ? sA[j * LA + i] : 0.f);
        sT[i * LC + j] = x;  // over the dead K rows
        if (WRITE_T) wT[(size_t)tile * C * C + i * C + j] = x;
      }
      lds_barrier();
      // W^T = X^T Tinv^T (rows d, cols t), staged as W[t][d] over the dead inverse
      E* sWo = (E*)(smem + Lay::A);
      for (int tt = w; tt < (DK / 16) * NB; tt += kWaves) {
        const int td = tt / NB, tc = tt % NB;
        f32x4 acc = zero4();
        mma<C>(acc, sXt + td * 16 * LC, LC, sT + tc * 16 * LC, LC);
        store4<E>(sWo + (tc * 16 + (l & 15)) * LK + td * 16 + (l >> 4) * 4, acc);
      }
      lds_barrier();
      lds_to_block<E, C, DK>(wW + (size_t)tile * C * DK, sWo, LK);
      // U' = Tinv Y (rows t, cols v), staged as U'^T[v][t] over the dead X^T
      E* sUo = sXt;
      for (int tt = w; tt < NB * (DV / 16); tt += kWaves) {
        const int ti = tt / (DV / 16), tv = tt % (DV / 16);
        f32x4 acc = zero4();
        mma<C>(acc, sT + ti * 16 * LC, LC, sYt + tv * 16 * LC, LC);
        store4<E>(sUo + (tv * 16 + (l & 15)) * LC + ti * 16 + (l >> 4) * 4, acc);
      }
      lds_barrier();
      lds_to_block<E, DV, C>(wUp + (size_t)tile * DV * C, sUo, LC);
      lds_barrier();
    }
  }
#undef LRT_PREP_LOAD
}

// ----------------------------------------------------------------- k_state
// One workgroup of NW waves per (b, h, d_v block of BV columns); walks the N
// chunks.  The state block (d_k x BV, fp32) lives in MFMA accumulators; the
// next chunk's W, Ktil^T and U' load into registers while this one computes;
// chunk-start states and U leave through LDS as coalesced 16-byte rows.
// PERDIM (KDA): the chunk decay is per key dimension, e^(GC[d]) from wGC.
template <typename E, int C, int DK, int BV, bool DELTA, bool PERDIM = false, int NW = 8>
__global__ __launch_bounds__(64 * NW) void k_state(const E* __restrict__ wW, const E* __restrict__ wUp,
                                                   const E* __restrict__ wKt, const float* __restrict__ wG,
                                                   const float* __restrict__ wGC, const float* h0, float* ht,
                                                   E* __restrict__ wU, E* __restrict__ wS, int N, int DV) {
  constexpr int NT = 64 * NW;
  constexpr int P = lds_pad<E>();
  constexpr int LK = DK + P, LC = C + P;
  constexpr int NTV = BV / 16;
  constexpr int NH = (DK / 16) * NTV;  // state tiles
  constexpr int HPW = (NH + NW - 1) / NW;
  constexpr int NU = (C / 16) * NTV;  // U tiles
  constexpr int UPW = (NU + NW - 1) / NW;
  __shared__ __attribute__((aligned(16))) E sW[DELTA ? C * LK : 8];
  __shared__ __attribute__((aligned(16))) E sKt[DK * LC];
  __shared__ __attribute__((aligned(16))) E sS[BV * LK];
  __shared__ __attribute__((aligned(16))) E sU[BV * LC];

  const int nvb = DV / BV;
  const int wg = xcd_group(blockIdx.x, gridDim.x);  // the d_v blocks of one (b, h) share an L2
  const int vb = wg % nvb, bh = wg / nvb;
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

  Tile<E, C, DK, NT> tW;   // W of the next chunk (delta variants)
  Tile<E, DK, C, NT> tK;   // Ktil^T of the next chunk
  f32x4 rUp[UPW];
  f32x4 rgd[PERDIM ? HPW : 1];
  float rgc = 0.f;
#define LRT_STATE_FETCH(n_)                                                                         \
  {                                                                                                 \
    const size_t ft = (size_t)bh * N + (n_);                                                        \
    if (DELTA) tW.load_block(wW + ft * C * DK);                                                     \
    tK.load_block(wKt + ft * DK * C);                                                               \
    _Pragma("unroll") for (int s = 0; s < UPW; ++s) {                                               \
      const int tt = w + NW * s;                                                                    \
      if (tt < NU)                                                                                  \
        rUp[s] = load4<E>(wUp + ft * DV * C + (size_t)(v0 + (tt % NTV) * 16 + (l & 15)) * C +      \
                          (tt / NTV) * 16 + (l >> 4) * 4);                                          \
    }                                                                                               \
    if constexpr (PERDIM) {                                                                         \
      _Pragma("unroll") for (int s = 0; s < HPW; ++s) {                                             \
        const int tt = w + NW * s;                                                                  \
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
    // chunk start state S = H^T -> LDS (operand of W Hn, then copied out)
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + NW * s;
      if (tt < NH) {
        const int td = tt / NTV, tv = tt % NTV;
        store4<E>(sS + (tv * 16 + (l & 15)) * LK + td * 16 + (l >> 4) * 4, hacc[s]);
      }
    }
    if (n + 1 < N) LRT_STATE_FETCH(n + 1)
    lds_barrier();
    lds_to_block<E, BV, DK, NT>(wS + (tile * DV + v0) * DK, sS, LK);
    // U = U' - W Hn  (rows t, cols v)
#pragma unroll
    for (int s = 0; s < UPW; ++s) {
      const int tt = w + NW * s;
      if (tt < NU) {
        const int ti = tt / NTV, tv = tt % NTV;
        f32x4 u = up[s];
        if constexpr (DELTA) {
          f32x4 acc = zero4();
          mma<DK>(acc, sW + ti * 16 * LK, LK, sS + tv * 16 * LK, LK);
          u -= acc;
        }
        store4<E>(sU + (tv * 16 + (l & 15)) * LC + ti * 16 + (l >> 4) * 4, u);
      }
    }
    lds_barrier();
    lds_to_block<E, BV, C, NT>(wU + (tile * DV + v0) * C, sU, LC);
    // H <- e^(g_C) H + Ktil^T U
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + NW * s;
      if (tt < NH) {
        const int td = tt / NTV, tv = tt % NTV;
        if constexpr (PERDIM)
          hacc[s] *= decd[s];
        else
          hacc[s] *= dec;
        mma<C>(hacc[s], sKt + td * 16 * LC, LC, sU + tv * 16 * LC, LC);
      }
    }
    lds_barrier();
  }
#undef LRT_STATE_FETCH
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

// ------------------------------------------------------------------- k_out
// O^T = S Q^T (scaled by gamma per token) + U^T P^T per (chunk, block of BVO
// value columns); workgroups walk these work items persistently, prefetching.
// FROM_WS (KDA): Q o e^G and P are read from the workspace instead of being
// formed from q, k and the scalar gates.
template <typename E, int C, int DK, int BVO, bool FROM_WS>
constexpr size_t out_lds_bytes() {
  constexpr size_t P = lds_pad<E>(), es = sizeof(E);
  constexpr size_t ko = C * ((DK > BVO ? DK : BVO) + P);
  return C * 4 + (C * (DK + P) + ko + BVO * (DK + P) + BVO * (C + P) + C * (C + P)) * es;
}

template <typename E, int C, int DK, int BVO, bool FROM_WS = false>
__global__ __launch_bounds__(kThreads) void k_out(const E* __restrict__ q, const E* __restrict__ k,
                                                  const float* __restrict__ wG, const E* __restrict__ wS,
                                                  const E* __restrict__ wU, const E* __restrict__ wQg,
                                                  const E* __restrict__ wP, E* __restrict__ o, int T, int H,
                                                  int N, int DV, int nitems) {
  constexpr int P = lds_pad<E>();
  constexpr int LK = DK + P, LC = C + P;
  constexpr int NB = C / 16;
  constexpr int LO = BVO + P;
  __shared__ float sg[C];
  __shared__ __attribute__((aligned(16))) E sQ[C * LK];
  // K rows (dead once P is formed), then the output rows of this item
  __shared__ __attribute__((aligned(16))) E sK[C * (DK > BVO ? LK : LO)];
  __shared__ __attribute__((aligned(16))) E sS[BVO * LK];
  __shared__ __attribute__((aligned(16))) E sU[BVO * LC];
  __shared__ __attribute__((aligned(16))) E sP[C * LC];
  E* sO = sK;

  const int nvb = DV / BVO;
  const int w = wave_id(), l = lane_id();
  Tile<E, C, DK> tq;
  Tile<E, C, FROM_WS ? C : DK> tk;  // K rows, or P (FROM_WS)
  Tile<E, BVO, DK> ts;
  Tile<E, BVO, C> tu;
  float rg = 0.f;
#define LRT_OUT_LOAD(item_)                                                               \
  {                                                                                       \
    const int ltile = (item_) / nvb, lv0 = ((item_) % nvb) * BVO;                         \
    const int ln = ltile % N, lbh = ltile / N;                                            \
    const int lnv = min(C, T - ln * C);                                                   \
    const size_t ltok = (size_t)(lbh / H) * T + (size_t)ln * C;                           \
    const int lh = lbh % H;                                                               \
    if constexpr (FROM_WS) {                                                              \
      tq.load_block(wQg + (size_t)ltile * C * DK);                                        \
      tk.load_block(wP + (size_t)ltile * C * C);                                          \
    } else {                                                                              \
      tq.load_rows(q + (ltok * H + lh) * DK, (size_t)H * DK, lnv);                        \
      tk.load_rows(k + (ltok * H + lh) * DK, (size_t)H * DK, lnv);                        \
      if (threadIdx.x < C) rg = wG[(size_t)ltile * C + threadIdx.x];                      \
    }                                                                                     \
    ts.load_block(wS + ((size_t)ltile * DV + lv0) * DK);                                  \
    tu.load_block(wU + ((size_t)ltile * DV + lv0) * C);                                   \
  }

  int item = blockIdx.x;
  if (item < nitems) LRT_OUT_LOAD(item)
  for (; item < nitems; item += gridDim.x) {
    const int tile = item / nvb, v0 = (item % nvb) * BVO;
    const int n = tile % N, bh = tile / N, h = bh % H, b = bh / H;
    const int t0 = n * C, nv = min(C, T - t0);
    const size_t tok0 = (size_t)b * T + t0;
    tq.store(sQ, LK);
    if constexpr (FROM_WS)
      tk.store(sP, LC);
    else
      tk.store(sK, LK);
    ts.store(sS, LK);
    tu.store(sU, LC);
    if (!FROM_WS && threadIdx.x < C) sg[threadIdx.x] = rg;
    lds_barrier();
    if (item + (int)gridDim.x < nitems) LRT_OUT_LOAD(item + (int)gridDim.x)
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
      lds_barrier();
    }
    for (int tt = w; tt < (BVO / 16) * NB; tt += kWaves) {
      const int tv = tt / NB, ti = tt % NB;
      f32x4 acc = zero4();
      mma<DK>(acc, sS + tv * 16 * LK, LK, sQ + ti * 16 * LK, LK);
      const int i = ti * 16 + (l & 15);
      if constexpr (!FROM_WS) acc *= __expf(sg[i]);
      mma<C>(acc, sU + tv * 16 * LC, LC, sP + ti * 16 * LC, LC);
      store4<E>(sO + i * LO + tv * 16 + (l >> 4) * 4, acc);
    }
    lds_barrier();
    lds_to_rows<E, C, BVO>(o + (tok0 * H + h) * DV + v0, (size_t)H * DV, sO, LO, nv);
    lds_barrier();
  }
#undef LRT_OUT_LOAD
}

}  // namespace lrt
