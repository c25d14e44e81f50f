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
#include "lrt_internal.hpp"

namespace lrt {

// ------------------------------------------------------------------- k_wy
template <typename E, int C, int DK, int DV>
struct WyLds {
  static constexpr int P = lds_pad<E>();
  static constexpr int LK = DK + P, LV = DV + P, LC = C + P, LA = tri_ld<C>();
  static constexpr size_t es = sizeof(E);
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t K = 0;                                                      // k rows [t][d]
  static constexpr size_t V = K + (size_t)C * LK * es;                                // b v rows [t][v]
  static constexpr size_t QT = V + (size_t)C * LV * es;                               // q rows; then T, T diag(b gamma)
  static constexpr size_t A = QT + mx((size_t)C * LK * es, 2 * (size_t)C * LC * es);  // A (fp32, column-major), inverted in place
  static constexpr size_t G = A + (size_t)C * LA * 4;                                 // g, gamma, b, b gamma
  static constexpr size_t TOTAL = G + 4 * C * 4;
};

// Outputs per tile (chunk-major per (b, h)): W [C][d_k] rows, U' [C][d_v] in
// accumulator-tile order (acc_tile_store), g [C]; WRITE_P: P [C][C] rows
// (zero above the diagonal); WRITE_T: T [C][C].  FUSE: q, k, log_a and beta
// are the raw projections (the fused prologue: L2-normalised rows, -softplus,
// sigmoid, applied as they are staged).
template <typename E, int C, int DK, int DV, bool WRITE_P, bool WRITE_T, int NW = 8, bool FUSE = false>
__global__ __launch_bounds__(64 * NW, 4) void k_wy(const E* __restrict__ q, const E* __restrict__ k,
                                                const E* __restrict__ v, const float* __restrict__ log_a,
                                                const float* __restrict__ beta, SeqMap m,
                                                E* __restrict__ wW, E* __restrict__ wUp, float* __restrict__ wG,
                                                E* __restrict__ wP, E* __restrict__ wT) {
  typedef WyLds<E, C, DK, DV> Lay;
  const int H = m.H, ntiles = tile_count(m);
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
  // The next chunk's operands, in parts (bit mask PART_) spread over this
  // chunk's phases; rows and chunk index clamped so no load sits behind a
  // branch (rows past the end are masked where staged).
#define LRT_WY_LOAD(P_, N_, PART_)                                                        \
  {                                                                                       \
    const int lnv = min(C, (P_).len - (N_) * C);                                          \
    const size_t ltok = (P_).tok0 + (size_t)(N_) * C;                                     \
    const int lh = (P_).h;                                                                \
    if ((PART_) & 1) {                                                                    \
      tk.load_rows_clamped(k + (ltok * H + lh) * DK, (size_t)H * DK, lnv);                \
      const int tc = min((int)threadIdx.x, lnv - 1); /* masked where used */              \
      la = log_a[(ltok + tc) * H + lh];                                                   \
      bt = beta[(ltok + tc) * H + lh];                                                    \
    }                                                                                     \
    if (WRITE_P && ((PART_) & 2)) tq.load_rows_clamped(q + (ltok * H + lh) * DK, (size_t)H * DK, lnv); \
    if ((PART_) & 4) tv.load_rows_clamped(v + (ltok * H + lh) * DV, (size_t)H * DV, lnv); \
  }

  int tile = blockIdx.x;
  if (tile < ntiles) {
    int n0;
    const SeqPos p0 = tile_pos(m, tile, n0);
    LRT_WY_LOAD(p0, n0, 7)
  }
  for (; tile < ntiles; tile += gridDim.x) {
    int cn;
    const int nv = min(C, tile_pos(m, tile, cn).len - cn * C);
    const int next = min(tile + (int)gridDim.x, ntiles - 1);
    int nn;
    const SeqPos np = tile_pos(m, next, nn);
    asm volatile("" ::"v"(la), "v"(bt));
    if (threadIdx.x < 64) {
      const bool valid = (int)threadIdx.x < nv;
      const float g = wave_incl_scan(valid ? (FUSE ? neg_softplus_f(la) : la) : 0.f);
      if (threadIdx.x < C) {
        const int t = threadIdx.x;
        const float gam = __expf(g);
        const float b_ = valid ? (FUSE ? sigmoid_f(bt) : bt) : 0.f;
        sg[t] = g;
        sgam[t] = gam;
        sb[t] = b_;
        sbg[t] = b_ * gam;
        wG[(size_t)tile * C + t] = g;
      }
    }
    if constexpr (FUSE) tk.normalize_rows(kL2Eps);
    tk.store_masked(sK, LK, nv);
    if constexpr (WRITE_P) {
      if constexpr (FUSE) tq.normalize_rows(kL2Eps);
      tq.store_masked(sQ, LK, nv);
    }
    lds_barrier();
    LRT_WY_LOAD(np, nn, 1)
    tv.scale_rows(sb);
    tv.store_masked(sV, LV, nv);
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
        const int j = tj * 16 + (l & 15), i0 = ti * 16 + (l >> 4) * 4;
        f32x4 av;
#pragma unroll
        for (int r = 0; r < 4; ++r) av[r] = (j < i0 + r) ? sb[i0 + r] * acc[r] * __expf(sg[i0 + r] - sg[j]) : 0.f;
        *(f32x4*)(sA + j * LA + i0) = av;  // column-major
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
    LRT_WY_LOAD(np, nn, 4)
    unit_lower_inverse<C, NT>(sA);
    LRT_WY_LOAD(np, nn, 2)
    for (int idx = threadIdx.x; idx < C * C; idx += NT) {
      const int j = idx / C, i = idx % C;
      const float x = j <= i ? sA[j * LA + i] : 0.f;
      sT[i * LC + j] = from_f<E>(x);
      sTw[i * LC + j] = from_f<E>(x * sbg[j]);
    }
    lds_barrier();
    if constexpr (WRITE_T) lds_to_block<E, C, C, NT>(wT + (size_t)tile * C * C, sT, LC);
    // W^T = K^T (T diag(b gamma))^T (rows d, cols t): a lane's 4 values are
    // 4 consecutive d of one row of W; U' = T (b V) (rows t, cols v) in
    // accumulator-tile order (a wave's 64 lanes write 512 contiguous bytes;
    // the scan reads it per lane).  W stays row-major: its readers stage it in
    // LDS, where rebuilding rows from tile order costs more than it saves.
    // unrolled (a known store count keeps the next chunk's wait exact) where
    // the registers allow
    constexpr int UWU = WRITE_P ? 1 : (NWT + NUT + NW - 1) / NW;
#pragma unroll UWU
    for (int s2 = 0; s2 < (NWT + NUT + NW - 1) / NW; ++s2) {
      const int tt = w + NW * s2;
      if (tt >= NWT + NUT) break;
      f32x4 acc = zero4();
      if (tt < NWT) {
        const int td = tt / NB, ti = tt % NB;
        mma<C, true, false>(acc, sK + td * 16, LK, sTw + ti * 16 * LC, LC);
        store4<E>(wW + ((size_t)tile * C + ti * 16 + (l & 15)) * DK + td * 16 + (l >> 4) * 4, acc);
      } else {
        const int u = tt - NWT, ti = u / (DV / 16), tvb = u % (DV / 16);
        mma<C, false, true>(acc, sT + ti * 16 * LC, LC, sV + tvb * 16, LV);
        acc_tile_store<E>(wUp + (size_t)tile * DV * C, ti * (DV / 16) + tvb, acc);
      }
    }
    lds_barrier();
  }
#undef LRT_WY_LOAD
}

// ----------------------------------------------------------------- k_scan
// Modes: forward (writes o), backward recompute (writes the chunk-start
// states S_n and U), or local (writes only the end state of its segment).
enum ScanMode { kScanFwd = 0, kScanBwd = 1, kScanLocal = 2 };

// Operands of k_scan.  Per-tile workspace arrays are chunk-major per (b, h).
// States (hin / hout) are fp32 [b*h][segment][d_k][hs_ld].
template <typename E>
struct ScanArgs {
  const E* q;       // q rows (GDN forward)
  const E* k;       // k rows (GDN)
  const E* W;       // W rows [C][d_k]
  const E* Up;      // U' [C][d_v], accumulator-tile order (Mamba2: V^T rows [d_v][C])
  const E* P;       // P rows [C][C] (forward)
  const E* Qg;      // (Q o e^G) rows [C][d_k] (KDA forward)
  const E* Kt;      // Ktil^T [d_k][C] (KDA)
  const float* G;   // g [C] (GDN)
  const float* GC;  // per-dim chunk log-decay [d_k] (KDA)
  const float* hin; // start state of each segment, or nullptr = zero
  float* hout;      // end state of each segment, or nullptr
  E* o;             // forward output
  E* U;             // U^T [d_v][C] (backward recompute)
  E* S;             // chunk-start states [d_v][d_k] (backward recompute)
  int hs_ld;        // columns of a state row in hin / hout
  SeqMap m;         // where each (sequence, head)'s chunks lie
  int L, nseg;      // chunks per segment, segments per sequence
  int DV;           // value columns (local mode appends d_k identity columns)
};

template <typename E, int C, int DK, int BV, int MODE, bool KDA>
struct ScanLds {
  static constexpr int P = lds_pad<E>();
  static constexpr int LK = DK + P, LB = BV + P, LC = C + P;
  static constexpr size_t es = sizeof(E);
  static constexpr bool FWD = MODE == kScanFwd;
  static constexpr size_t W = 0;                                                  // W rows [t][d]
  static constexpr size_t K = W + (size_t)C * LK * es;                            // k rows [t][d] / Ktil^T [d][t]
  static constexpr size_t S = K + (KDA ? (size_t)DK * LC : (size_t)C * LK) * es;  // Hn^T [v][d]
  static constexpr size_t U = S + (size_t)BV * LK * es;                           // U^T (, (e^(g_C - g) U)^T) [v][t]
  static constexpr size_t Q = U + (KDA ? 1 : 2) * (size_t)BV * LC * es;           // q / Q o e^G rows [t][d]
  static constexpr size_t P_ = Q + (FWD ? (size_t)C * LK * es : 0);               // P [i][j]
  static constexpr size_t O = P_ + (FWD ? (size_t)C * LC * es : 0);               // o rows [t][v]
  static constexpr size_t G = O + (FWD ? (size_t)C * LB * es : 0);                // g, gamma, e^(g_C - g) / KDA: G_C
  static constexpr size_t TOTAL = G + (KDA ? DK : 3 * C) * 4;
};

// One workgroup per (b, h, block of BV columns, segment) walks its chunks in
// order, the state block in MFMA accumulators.  Local mode runs each segment
// from a zero state and also carries d_k identity columns with U' = 0, so
// its end state holds both the segment's own contribution E and its
// transition M (the state map is affine: H_end = M H_start + E).
// DELTA = false is the Mamba2 recurrence (no delta term: W = 0, U = U' = V,
// with U'^T supplied in a.Up); the backward recompute then writes only S_n.
// SAVE (forward mode) also writes S_n and U, as the backward recompute does,
// for a backward that reuses them.
// FUSE (forward of the fused prologue): the q and k rows read here are the
// raw projections, L2-normalised as they are staged.
template <typename E, int C, int DK, int BV, int MODE, bool KDA, int NW = 8, bool DELTA = true, bool SAVE = false,
          bool FUSE = false>
__global__ __launch_bounds__(64 * NW) void k_scan(ScanArgs<E> a) {
  typedef ScanLds<E, C, DK, BV, MODE, KDA> Lay;
  constexpr bool FWD = MODE == kScanFwd;
  constexpr int NT = 64 * NW;
  constexpr int LK = Lay::LK, LB = Lay::LB, LC = Lay::LC;
  constexpr int NB = C / 16, NTV = BV / 16;
  constexpr int NH = (DK / 16) * NTV, HPW = (NH + NW - 1) / NW;  // state tiles (rows d, cols v)
  constexpr int NU = NB * NTV, UPW = (NU + NW - 1) / NW;         // U tiles (rows t, cols v)
  constexpr int NO = NTV * NB;                                   // O^T tiles (rows v, cols t)
  // When every wave holds the same number of tiles of one column block, a
  // wave's bf16 products read the fragment its tiles share once per k step
  // (fp32 operands are read per 16-long k step either way).
  constexpr bool kShU = sizeof(E) == 2 && NU % NW == 0 && NW % NTV == 0;
  constexpr bool kShH = sizeof(E) == 2 && NH % NW == 0 && NW % NTV == 0;
  constexpr bool kShO = sizeof(E) == 2 && NO % NW == 0 && NW % NB == 0;
  __shared__ __attribute__((aligned(16))) char smem[Lay::TOTAL];
  E* sW = (E*)(smem + Lay::W);
  E* sK = (E*)(smem + Lay::K);  // GDN: k rows; KDA: Ktil^T
  E* sS = (E*)(smem + Lay::S);
  E* sU = (E*)(smem + Lay::U);
  E* sUk = sU + BV * LC;
  E* sQ = (E*)(smem + Lay::Q);
  E* sP = (E*)(smem + Lay::P_);
  E* sO = (E*)(smem + Lay::O);
  float* sg = (float*)(smem + Lay::G);
  float* sgam = sg + C;
  float* skt = sg + 2 * C;

  const int DVX = MODE == kScanLocal ? a.DV + DK : a.DV;
  const int nvb = DVX / BV;
  // the column blocks of one (b, h, segment) are consecutive, so they share an
  // XCD and its L2 (they read the same W, K, Q and P tiles)
  const int wg = xcd_group(blockIdx.x, gridDim.x);
  const int vb = wg % nvb, seg = (wg / nvb) % a.nseg, bh = wg / nvb / a.nseg;
  const SeqPos sp = seq_pos(a.m, bh);
  const int H = a.m.H, DV = a.DV;
  const int h = sp.h;
  const int v0 = vb * BV;
  const bool ident = MODE == kScanLocal && v0 >= DV;  // identity columns (U' = 0)
  const int n0 = seg * a.L, n1 = min(sp.nch, n0 + a.L);
  const int w = wave_id(), l = lane_id();
  const size_t st0 = ((size_t)bh * a.nseg + seg) * DK;  // first state row of this segment

  f32x4 hacc[HPW];
#pragma unroll
  for (int s = 0; s < HPW; ++s) {
    const int tt = w + NW * s;
    hacc[s] = zero4();
    if (tt < NH) {
      const int td = tt / NTV, tv = tt % NTV;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = td * 16 + (l >> 4) * 4 + r, c = v0 + tv * 16 + (l & 15);
        if (ident)
          hacc[s][r] = (d == c - DV) ? 1.f : 0.f;
        else if (a.hin != nullptr && MODE != kScanLocal)
          hacc[s][r] = a.hin[(st0 + d) * a.hs_ld + c];
      }
    }
  }

  // One chunk's operands in registers; two sets alternate, so the loads of
  // chunk n + 2 are in flight while chunk n computes.
  struct Ops {
    Tile<E, C, DK, NT> W, Q;
    Tile<E, KDA ? DK : C, KDA ? C : DK, NT> K;
    Tile<E, C, C, NT> P;
    typename Vec4<E>::T up[UPW];
    float g;  // GDN: g of token tid; KDA: G_C of key dimension tid
  };
  auto fetch = [&](Ops& x, int n_) {
    const size_t ft = sp.tile0 + n_;
    const int fnv = min(C, sp.len - n_ * C);
    const size_t ftok = sp.tok0 + (size_t)n_ * C;
    if constexpr (DELTA) x.W.load_block(a.W + ft * C * DK);
    if constexpr (KDA) {
      x.K.load_block(a.Kt + ft * DK * C);
      x.g = a.GC[ft * DK + min((int)threadIdx.x, DK - 1)];
    } else {
      x.K.load_rows(a.k + (ftok * H + h) * DK, (size_t)H * DK, fnv);
      x.g = a.G[ft * C + min((int)threadIdx.x, C - 1)];
    }
    if constexpr (FWD) {
      if constexpr (KDA)
        x.Q.load_block(a.Qg + ft * C * DK);
      else
        x.Q.load_rows(a.q + (ftok * H + h) * DK, (size_t)H * DK, fnv);
      x.P.load_block(a.P + ft * C * C);
    }
    // unconditional loads (clamped indices), so nothing waits for them here
    if (!ident) {
#pragma unroll
      for (int s = 0; s < UPW; ++s) {
        const int tt = min(w + NW * s, NU - 1);
        if constexpr (DELTA)  // U'^T in accumulator-tile order: one tile's 64 lanes are contiguous
          x.up[s] = load4_raw<E>(a.Up + ft * DV * C +
                                 ((size_t)((tt / NTV) * (DV / 16) + v0 / 16 + tt % NTV) * 64 + l) * 4);
        else  // the Mamba2 recompute's V^T rows
          x.up[s] = load4_raw<E>(a.Up + (ft * DV + v0 + (tt % NTV) * 16 + (l & 15)) * C + (tt / NTV) * 16 + (l >> 4) * 4);
      }
    }
  };

  auto step = [&](Ops& x, int n) {
    const size_t tile = sp.tile0 + n;
    const int nv = min(C, sp.len - n * C);
    const size_t tok0 = sp.tok0 + (size_t)n * C;
    // ---- this chunk's operands and start state into LDS
    if constexpr (KDA) {
      if (threadIdx.x < DK) sg[threadIdx.x] = __expf(x.g);  // per-dim chunk decay
    } else {
      if (threadIdx.x < 64) {
        const float gC = __shfl(x.g, C - 1, 64);
        if (threadIdx.x < C) {
          sg[threadIdx.x] = x.g;
          sgam[threadIdx.x] = __expf(x.g);
          skt[threadIdx.x] = __expf(gC - x.g);
        }
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
    if constexpr (DELTA) x.W.store(sW, LK);
    if constexpr (FUSE && !KDA) x.K.normalize_rows(kL2Eps);
    x.K.store(sK, KDA ? LC : LK);
    if constexpr (FWD) {
      if constexpr (FUSE && !KDA) x.Q.normalize_rows(kL2Eps);
      x.Q.store(sQ, LK);
      x.P.store(sP, LC);
    }
    f32x4 up[UPW];
#pragma unroll
    for (int s = 0; s < UPW; ++s) up[s] = ident ? zero4() : Vec4<E>::unpack(x.up[s]);
    // chunk n + 2 (the segment's last chunk again near its end: unconditional
    // loads keep the compiler's wait for the next set exact)
    fetch(x, min(n + 2, n1 - 1));
    lds_barrier();
    if constexpr (MODE == kScanBwd || SAVE) lds_to_block<E, BV, DK, NT>(a.S + (tile * DV + v0) * DK, sS, LK);
    // ---- U = U' - W Hn -> U^T (GDN: and (e^(g_C - g) U)^T)
    f32x4 wh[UPW];
#pragma unroll
    for (int s = 0; s < UPW; ++s) wh[s] = zero4();
    if constexpr (DELTA && kShU)
      mma_nA<DK, UPW>(wh, sW + (w / NTV) * 16 * LK, (NW / NTV) * 16 * LK, LK, sS + (w % NTV) * 16 * LK, LK);
#pragma unroll
    for (int s = 0; s < UPW; ++s) {
      const int tt = w + NW * s;
      if (tt < NU) {
        const int ti = tt / NTV, tv = tt % NTV;
        f32x4 acc = wh[s];
        if constexpr (DELTA && !kShU) mma<DK>(acc, sW + ti * 16 * LK, LK, sS + tv * 16 * LK, LK);
        const f32x4 u = up[s] - acc;
        const int vv = tv * 16 + (l & 15), t = ti * 16 + (l >> 4) * 4;
        store4<E>(sU + vv * LC + t, u);
        if constexpr (!KDA)
          store4<E>(sUk + vv * LC + t, f32x4{u[0] * skt[t], u[1] * skt[t + 1], u[2] * skt[t + 2], u[3] * skt[t + 3]});
      }
    }
    lds_barrier();
    // U^T rows out from their LDS copy (16 bytes per access)
    if constexpr ((MODE == kScanBwd || SAVE) && DELTA) lds_to_block<E, BV, C, NT>(a.U + (tile * DV + v0) * C, sU, LC);
    // ---- O^T = Hn^T (Q diag(gamma))^T + U^T P^T -> o rows; state update
    if constexpr (FWD && kShO) {
      constexpr int OPW = NO / NW;
      const int ti = w % NB, i = ti * 16 + (l & 15);
      f32x4 oa[OPW];
#pragma unroll
      for (int s = 0; s < OPW; ++s) oa[s] = zero4();
      mma_nA<DK, OPW>(oa, sS + (w / NB) * 16 * LK, (NW / NB) * 16 * LK, LK, sQ + ti * 16 * LK, LK);
      if constexpr (!KDA) {
        const float gm = sgam[i];
#pragma unroll
        for (int s = 0; s < OPW; ++s) oa[s] *= gm;
      }
      mma_nA<C, OPW>(oa, sU + (w / NB) * 16 * LC, (NW / NB) * 16 * LC, LC, sP + ti * 16 * LC, LC);
#pragma unroll
      for (int s = 0; s < OPW; ++s) store4<E>(sO + i * LB + (w / NB + (NW / NB) * s) * 16 + (l >> 4) * 4, oa[s]);
    } else if constexpr (FWD) {
      for (int tt = w; tt < NO; tt += NW) {
        const int tv = tt / NB, ti = tt % NB;
        f32x4 acc = zero4();
        mma<DK>(acc, sS + tv * 16 * LK, LK, sQ + ti * 16 * LK, LK);
        const int i = ti * 16 + (l & 15);
        if constexpr (!KDA) acc *= sgam[i];
        mma<C>(acc, sU + tv * 16 * LC, LC, sP + ti * 16 * LC, LC);
        store4<E>(sO + i * LB + tv * 16 + (l >> 4) * 4, acc);
      }
    }
    const float gdec = KDA ? 0.f : __expf(sg[C - 1]);
    if constexpr (kShH) {
#pragma unroll
      for (int s = 0; s < HPW; ++s) {
        if constexpr (KDA)
          hacc[s] *= *(const f32x4*)(sg + (w / NTV + (NW / NTV) * s) * 16 + (l >> 4) * 4);
        else
          hacc[s] *= gdec;
      }
      if constexpr (KDA)
        mma_nA<C, HPW>(hacc, sK + (w / NTV) * 16 * LC, (NW / NTV) * 16 * LC, LC, sU + (w % NTV) * 16 * LC, LC);
      else
        mma_nA<C, HPW, true, false>(hacc, sK + (w / NTV) * 16, (NW / NTV) * 16, LK, sUk + (w % NTV) * 16 * LC, LC);
    }
#pragma unroll
    for (int s = 0; s < (kShH ? 0 : HPW); ++s) {
      const int tt = w + NW * s;
      if (tt < NH) {
        const int td = tt / NTV, tv = tt % NTV;
        if constexpr (KDA) {
          hacc[s] *= *(const f32x4*)(sg + td * 16 + (l >> 4) * 4);
          mma<C>(hacc[s], sK + td * 16 * LC, LC, sU + tv * 16 * LC, LC);
        } else {
          hacc[s] *= gdec;
          mma<C, true, false>(hacc[s], sK + td * 16, LK, sUk + tv * 16 * LC, LC);
        }
      }
    }
    lds_barrier();
    // o rows out, after this chunk's prefetch (clamped rows: a fixed number of
    // stores, so the next wait for operands leaves them in flight)
    if constexpr (FWD)
      lds_to_rows_clamped<E, C, BV, NT>(a.o + (tok0 * H + h) * DV + v0, (size_t)H * DV, sO, LB, nv);
  };

  Ops x0, x1;
  if (n0 < n1) fetch(x0, n0);
  if (n0 + 1 < n1) fetch(x1, n0 + 1);
  for (int n = n0; n < n1; n += 2) {
    step(x0, n);
    if (n + 1 < n1) step(x1, n + 1);
  }
  if (a.hout != nullptr) {
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + NW * s;
      if (tt < NH) {
        const int td = tt / NTV, tv = tt % NTV;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          a.hout[(st0 + td * 16 + (l >> 4) * 4 + r) * a.hs_ld + v0 + tv * 16 + (l & 15)] = hacc[s][r];
      }
    }
  }
}

// --------------------------------------------------------------- k_carry
// The serial pass over segments, one workgroup per (b, h, block of BV
// columns): from the local pass's end states [E | M] of each segment,
//   Hstart(s) = H,  H <- M(s) H + E(s)
// starting from h0 (or zero); writes every segment's start state and the
// final state.  M and H enter the MFMA in the call's element type E (bf16, or
// fp32 on the fp32 MFMA), with fp32 accumulation, as the state does in the
// chunk scan.
template <typename E, int DK, int BV>
struct CarryLds {
  static constexpr int LK = DK + lds_pad<E>();
  static constexpr size_t M = 0;                                          // M rows [d][e]
  static constexpr size_t HT = M + (size_t)DK * LK * sizeof(E);           // H^T [c][e]
  static constexpr size_t TOTAL = HT + (size_t)BV * LK * sizeof(E);
};

template <typename E, int DK, int BV, int NW = 8>
__global__ __launch_bounds__(64 * NW) void k_carry(const float* __restrict__ hloc, const float* h0,
                                                   float* __restrict__ hstart, float* ht, int nseg, int DV) {
  typedef CarryLds<E, DK, BV> Lay;
  constexpr int NT = 64 * NW, LK = Lay::LK, NTV = BV / 16;
  constexpr int NH = (DK / 16) * NTV, HPW = (NH + NW - 1) / NW;
  __shared__ __attribute__((aligned(16))) char smem[Lay::TOTAL];
  E* sM = (E*)(smem + Lay::M);
  E* sH = (E*)(smem + Lay::HT);
  const int nvb = DV / BV;
  const int vb = blockIdx.x % nvb, bh = blockIdx.x / nvb, v0 = vb * BV;
  const int w = wave_id(), l = lane_id();
  const int LDX = DV + DK;  // columns of a local end state: E then M

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
  for (int sg = 0; sg < nseg; ++sg) {
    const float* base = hloc + ((size_t)bh * nseg + sg) * DK * LDX;
    // this segment's start state; H^T -> LDS
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + NW * s;
      if (tt < NH) {
        const int td = tt / NTV, tv = tt % NTV;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          hstart[(((size_t)bh * nseg + sg) * DK + td * 16 + (l >> 4) * 4 + r) * DV + v0 + tv * 16 + (l & 15)] =
              hacc[s][r];
        store4<E>(sH + (tv * 16 + (l & 15)) * LK + td * 16 + (l >> 4) * 4, hacc[s]);
      }
    }
    // M rows -> LDS
    for (int p = threadIdx.x; p < DK * (DK / 4); p += NT) {
      const int d = p / (DK / 4), e0 = (p % (DK / 4)) * 4;
      store4<E>(sM + d * LK + e0, *(const f32x4*)(base + (size_t)d * LDX + DV + e0));
    }
    lds_barrier();
    // H <- M H + E
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
      const int tt = w + NW * s;
      if (tt < NH) {
        const int td = tt / NTV, tv = tt % NTV;
        f32x4 acc = zero4();
        mma<DK>(acc, sM + td * 16 * LK, LK, sH + tv * 16 * LK, LK);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[r] += base[(size_t)(td * 16 + (l >> 4) * 4 + r) * LDX + v0 + tv * 16 + (l & 15)];
        hacc[s] = acc;
      }
    }
    lds_barrier();
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

// ------------------------------------------------------------- launchers
// The forward scan over (b, h, column block) workgroups; when those are too
// few to occupy the device the sequence is cut into segments: a local pass
// per segment, the carry over segments, and the scan from the true segment
// start states.
template <typename E, int C, int DK, int DV, int BV, bool KDA, bool SAVE = false, bool FUSE = false>
int launch_scan_fwd_bv(const FwdArgs& a, const FwdWs& ws, int N, int nseg) {
  hipStream_t st = (hipStream_t)a.stream;
  ScanArgs<E> s{};
  s.q = (const E*)a.q;
  s.k = (const E*)a.k;
  s.W = (const E*)ws.W;
  s.Up = (const E*)ws.Up;
  s.P = (const E*)ws.P;
  s.Qg = (const E*)ws.Qg;
  s.Kt = (const E*)ws.Kt;
  s.G = ws.G;
  s.GC = ws.GC;
  s.o = (E*)a.o;
  s.S = (E*)ws.S;  // written only by SAVE
  s.U = (E*)ws.U;
  s.m = seq_map(a, ws, C);
  s.DV = DV;
  const int bhv = a.B * a.H * (DV / BV);
  if (nseg == 1) {
    s.hin = a.h0;
    s.hout = a.ht;
    s.hs_ld = DV;
    s.L = 1 << 30;  // one segment: every chunk of the sequence
    s.nseg = 1;
    LRT_LAUNCH(kKScan, (k_scan<E, C, DK, BV, kScanFwd, KDA, kStateWaves, true, SAVE, FUSE>), dim3(bhv),
               dim3(64 * kStateWaves), st, s);
  } else {
    s.L = (N + nseg - 1) / nseg;
    s.nseg = nseg;
    s.hin = nullptr;
    s.hout = ws.SegLoc;
    s.hs_ld = DV + DK;
    LRT_LAUNCH(kKScanLocal, (k_scan<E, C, DK, BV, kScanLocal, KDA, kStateWaves, true, false, FUSE>),
               dim3(a.B * a.H * ((DV + DK) / BV) * nseg), dim3(64 * kStateWaves), st, s);
    static_assert(CarryLds<E, DK, BV>::TOTAL <= 160 * 1024, "k_carry LDS");
    LRT_LAUNCH(kKCarry, (k_carry<E, DK, BV, kStateWaves>), dim3(bhv), dim3(64 * kStateWaves), st,
               (const float*)ws.SegLoc, a.h0, ws.SegStart, a.ht, nseg, DV);
    s.hin = ws.SegStart;
    s.hout = nullptr;
    s.hs_ld = DV;
    LRT_LAUNCH(kKScan, (k_scan<E, C, DK, BV, kScanFwd, KDA, kStateWaves, true, SAVE, FUSE>), dim3(bhv * nseg),
               dim3(64 * kStateWaves), st, s);
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

// The widest column block (at most `cap` columns, at least 16) whose
// operands of scan mode MODE fit in LDS; 0 if none does.
template <typename E, int C, int DK, int DV, int MODE, bool KDA, int cap = 64>
constexpr int scan_bv() {
  constexpr int b0 = DV < cap ? DV : cap;
  if constexpr (ScanLds<E, C, DK, b0, MODE, KDA>::TOTAL <= kLdsMax && CarryLds<E, DK, b0>::TOTAL <= kLdsMax)
    return b0;
  else if constexpr (b0 > 16)
    return scan_bv<E, C, DK, DV, MODE, KDA, b0 / 2>();
  else
    return 0;
}

template <typename E, int C, int DK, int DV, bool KDA, bool SAVE = false, bool FUSE = false>
int launch_scan_fwd(const FwdArgs& a, const FwdWs& ws, int N) {
  constexpr int BV64 = scan_bv<E, C, DK, DV, kScanFwd, KDA, 64>();
  constexpr int BV128 = scan_bv<E, C, DK, DV, kScanFwd, KDA, 128>();
  static_assert(BV64 > 0, "no column block of the forward scan fits in LDS");
  // packed sequences: one segment per (sequence, head) (their count is the parallelism)
  const ScanPlan pl = a.cu != nullptr ? ScanPlan{64, 1} : scan_plan(a.B, a.H, DK, DV, N);
  if constexpr (BV128 > BV64) {
    if (pl.bv > 64) return launch_scan_fwd_bv<E, C, DK, DV, BV128, KDA, SAVE, FUSE>(a, ws, N, pl.nseg);
  }
  return launch_scan_fwd_bv<E, C, DK, DV, BV64, KDA, SAVE, FUSE>(a, ws, N, pl.nseg);
}

}  // namespace lrt
