// lrt_kda_bwd.hip -- chunkwise backward of Kimi Delta Attention on gfx950.
//
// Gradients of L = <dO, O> + <dht, ht> for the KDA mixer (AMD ROCm blog
// "Pretraining hybrid LLMs with Primus", section "How hybrid models are
// defined in Primus", mixer list under Table 2; a pure-KDA model is among
// the models trained there, Table 1), differentiated through the chunkwise
// form of the forward (lrt_kda_prep.hpp).  Per chunk, with G the
// per-dimension inclusive cumsum of log a, E = e^G and E_C its last row, the
// forward in effective operands Qh = Q o E, Kh = K o E, Kb = K o E^-1,
// Kt = K o (E_C / E) is the Gated DeltaNet chunk with no scalar decay:
//   A = strict_lower(diag(b) Kh Kb^T),  T = (I + A)^-1,  W = T diag(b) Kh,
//   U = T diag(b) V - W Hn,  O = Qh Hn + lower(Qh Kb^T) U,
//   H_next = Diag(E_C) Hn + Kt^T U.
// The reverse state scan (lrt_dstate.hpp, KDA mode) gives dU and dH' (the
// gradient of each chunk's end state).  Then, per chunk (k_grad_kda):
//   dP = lower(dO U^T),  dW = -dU Hn^T,  dX = T^T dW,  dY = T^T dU,
//   dA = -strict_lower((dX X^T + dY Y^T) T^T),  X = diag(b) Kh,  Y = diag(b) V,
//   dq = E o (dO Hn^T) + R(dP),
//   dk = [b o R(dA) + b o E o dX] + [C(dP, q) + C(diag(b) dA, k) + (E_C / E) o (U dH'^T)],
//   dv = b o dY,  dbeta = rowsum(k o R(dA)) + rowsum(dX o Kh) + rowsum(dY o V),
//   dG = q o dq + k o ([first bracket] - [second bracket]),
//   dG_C += sum over the chunk of k o (E_C / E) o (U dH'^T) + E_C o rowsum(dH' o Hn),
//   dlog_a = the within-chunk reverse cumsum of dG, per key dimension,
// where the token sums carry the decay inside them:
//   R(M)_i = sum_{j <= i} M_ij k_j o e^(G_i - G_j),
//   C(M, x)_j = sum_{i >= j} M_ij x_i o e^(G_i - G_j).
// They run in blocks of 16 tokens.  For i in block si and j in an earlier
// block sj, with r the last row of block si - 1 and s the last row of sj,
//   e^(G_i - G_j) = e^(G_i - G_r) e^(G_r - G_s) e^(G_s - G_j):
// the outer factors scale operand rows (Kend_j = k_j e^(G_s - G_j),
// Qst_i = q_i e^(G_i - G_r)) or the product's output, the middle one is a
// per-dimension scale of one 16-token block product on MFMA, and every
// exponent is <= 0 -- nothing overflows for any finite log a <= 0.  While no
// block decays by more than e^60 in any dimension, r moves to the last row
// of block si itself (the first factor then in [1, e^60]) and the diagonal
// blocks (i, j in one block) are block products too; past that their pairs
// are summed element by element with the exact exponent difference.
//
// Kernels, in stream order: k_kda_prep (the forward's chunk-parallel pass,
// also writing T), k_scan (KDA, backward mode: chunk-start states S_n and U),
// k_dstate (KDA mode: dU and dH'), k_grad_kda.
#include <type_traits>

#include "lrt_dstate.hpp"
#include "lrt_internal.hpp"
#include "lrt_kda_prep.hpp"
#include "lrt_scan.hpp"

namespace lrt {

// LDS of k_grad_kda.  Three phases reuse one area: A (the state part), B
// (the WY part), C (the decayed token sums).
template <typename E, int C, int DK, int DV, int NW>
struct KdaGradLds {
  static constexpr int P = lds_pad<E>();
  static constexpr int LK = DK + P, LV = DV + P, LC = C + P, LG = DK + 4, NB = C / 16;
  static constexpr int NQ = (64 * NW) / DK < C ? (64 * NW) / DK : C;  // row segments of the cumsums
  static constexpr size_t es = sizeof(E);
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t al(size_t x) { return (x + 15) & ~(size_t)15; }
  static constexpr size_t CK = al((size_t)C * LK * es), CV = al((size_t)C * LV * es), CC = al((size_t)C * LC * es);
  static constexpr size_t VC = al((size_t)DV * LC * es), VK = al((size_t)DV * LK * es);
  // live through the chunk
  static constexpr size_t DPT = 0;                           // dP^T [j][i]
  static constexpr size_t DUT = DPT + CC;                    // dU^T [v][t]; phase C: q rows
  static constexpr size_t BB = DUT + mx(VC, CK);             // beta [C]
  static constexpr size_t GCE = BB + C * 4;                  // e^(G_C) [d_k]
  static constexpr size_t PDB = GCE + DK * 4;                // [NW][C] dbeta partials
  static constexpr size_t PCOL = PDB + (size_t)NW * C * 4;   // [NB][d_k] per-block sums of k o Kt-part
  static constexpr size_t PDEC = PCOL + (size_t)NB * DK * 4; // [NW][d_k] partials of rowsum(dH' o Hn)
  static constexpr size_t STOT = PDEC + (size_t)NW * DK * 4; // [NQ][d_k] segment totals of the cumsums
  static constexpr size_t FL = STOT + (size_t)NQ * DK * 4;    // largest decay of a 16-token block, largest |G| (float bits)
  static constexpr size_t U0 = al(FL + 16);
  // phase A
  static constexpr size_t SA = U0;    // Hn^T [v][d]; then dH'^T
  static constexpr size_t DOA = SA + VK;  // dO rows [t][v]
  static constexpr size_t UTA = DOA + CV;  // U^T [v][t]
  static constexpr size_t ENDA = UTA + VC;
  // phase B, over A (G, the k rows and dA^T stay through phase C).  X and H
  // lie past phase A's buffers: phase A already writes dW rows into X and
  // dKt rows into H.
  static constexpr size_t GL = U0;                            // G rows [t][d] (fp32); at the end dG
  static constexpr size_t KR = GL + al((size_t)C * LG * 4);   // k rows
  static constexpr size_t DAT = KR + CK;                      // dA^T [j][i]
  static constexpr size_t TB = DAT + CC;                      // Tinv rows [i][j]
  static constexpr size_t ZB = TB + CC;                       // Z^T [k][i]
  static constexpr size_t XB = mx(ZB + CC, ENDA);             // dW rows, then dX rows, then dY rows
  static constexpr size_t HB = XB + mx(CK, CV);               // dKt rows, then (K o E) rows, then v rows
  static constexpr size_t ENDB = HB + mx(CK, CV);
  // phase C, over B's T, Z, X and H; at the end the dq and dk rows
  static constexpr size_t KE = TB;        // Kend rows
  static constexpr size_t QS = KE + CK;   // Qst rows
  static constexpr size_t KS = QS + CK;   // b o Kst rows
  static constexpr size_t ENDC = KS + CK;
  static constexpr size_t TOTAL = mx(mx(ENDA, ENDB), ENDC);
};

// Persistent over the chunk tiles.  Output tiles are 16 x 16 (rows: key
// dimensions, columns: tokens); wave w owns the tiles of token block w % NB,
// so a lane's token is fixed and its four dimensions vary by tile.  Inputs
// are fetched half a chunk ahead: phase A's (S, dO, U, dU, dH') of the next
// chunk during phase C, phases B and C's (log a, k, Tinv, beta, v, q) during
// phase A.  dq, dk and dG are the only register arrays carried into phase C.
template <typename E, int C, int DK, int DV, int NW = kGradWaves>
__global__ __launch_bounds__(64 * NW) void k_grad_kda(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v, const E* __restrict__ d_o,
    const float* __restrict__ log_a, const float* __restrict__ beta, const E* __restrict__ wS,
    const E* __restrict__ wdS, const E* __restrict__ wU, const E* __restrict__ wdU, const E* __restrict__ wT,
    E* __restrict__ dq, E* __restrict__ dk_out, E* __restrict__ dv_out, float* __restrict__ dlog_a,
    float* __restrict__ dbeta, SeqMap m) {
  typedef KdaGradLds<E, C, DK, DV, NW> Lay;
  constexpr int NT = 64 * NW;
  constexpr int LK = Lay::LK, LV = Lay::LV, LC = Lay::LC, LG = Lay::LG, NB = Lay::NB, NQ = Lay::NQ;
  constexpr int V = 16 / (int)sizeof(E);
  constexpr int NDT = DK / 16, NVT = DV / 16;
  constexpr int WPB = NW / NB;                // waves per token block
  constexpr int KPW = (NDT + WPB - 1) / WPB;  // (dimension, token) tiles per wave
  constexpr int YPW = (NVT + WPB - 1) / WPB;  // dY^T tiles per wave
  constexpr int NZ = NB * NB, ZPW = (NZ + NW - 1) / NW;
  static_assert(NW % NB == 0, "waves must cover whole token blocks");
  // When every wave holds KPW (YPW) tiles of its token block, a wave's
  // bf16 products read the fragments its tiles share once per k step (mma_nA).
  constexpr bool kSh = sizeof(E) == 2 && NDT % WPB == 0 && NVT % WPB == 0;
  __shared__ __attribute__((aligned(16))) char smem[Lay::TOTAL];
  const int H = m.H, ntiles = tile_count(m);
  int tid = threadIdx.x;  // (re-derived per chunk below, opaque to the compiler)

  Tile<E, DV, DK, NT> tS, tdS;
  Tile<E, C, DV, NT> to, tv;
  Tile<E, DV, C, NT> tu, tdu;
  Tile<E, C, DK, NT> tq, tk;
  Tile<E, C, C, NT> tt;
  Tile<float, C, DK, NT> tg;
  float rb = 0.f;
  // parts: 1 S, dO, U, dU (phase A); 2 dH'; 4 log a, k, T, beta (phase B);
  // 8 v; 16 q (phase C).  Rows are clamped, so no load sits behind a branch.
#define LRT_KG_LOAD(tile_, P_, N_, PART_)                                          \
  {                                                                                \
    const int lnv = min(C, (P_).len - (N_) * C);                                   \
    const size_t ltok = (P_).tok0 + (size_t)(N_) * C;                              \
    const int lh = (P_).h;                                                         \
    const size_t lt = (size_t)(tile_);                                             \
    if ((PART_) & 1) {                                                             \
      tS.load_block(wS_ + lt * DV * DK);                                            \
      to.load_rows_clamped(do_ + (ltok * H + lh) * DV, (size_t)H * DV, lnv);       \
      tu.load_block(wU_ + lt * DV * C);                                             \
      tdu.load_block(wdU_ + lt * DV * C);                                           \
    }                                                                              \
    if ((PART_) & 2) tdS.load_block(wdS_ + lt * DV * DK);                           \
    if ((PART_) & 4) {                                                             \
      tg.load_rows_clamped(la_ + (ltok * H + lh) * DK, (size_t)H * DK, lnv);     \
      tk.load_rows_clamped(k_ + (ltok * H + lh) * DK, (size_t)H * DK, lnv);         \
      tt.load_block(wT_ + lt * C * C);                                              \
      rb = beta_[(ltok + min(tid, lnv - 1)) * H + lh];                              \
    }                                                                              \
    if ((PART_) & 8) tv.load_rows_clamped(v_ + (ltok * H + lh) * DV, (size_t)H * DV, lnv); \
    if ((PART_) & 16) tq.load_rows_clamped(q_ + (ltok * H + lh) * DK, (size_t)H * DK, lnv); \
  }

  int tile = blockIdx.x;
  if (tile < ntiles) {
    const E *q_ = q, *k_ = k, *v_ = v, *do_ = d_o, *wS_ = wS, *wdS_ = wdS, *wU_ = wU, *wdU_ = wdU, *wT_ = wT;
    const float *la_ = log_a, *beta_ = beta;
    int n0;
    const SeqPos p0 = tile_pos(m, tile, n0);
    LRT_KG_LOAD(tile, p0, n0, 3)
  }
  for (; tile < ntiles; tile += gridDim.x) {
    const E *q_ = q, *k_ = k, *v_ = v, *do_ = d_o, *wS_ = wS, *wdS_ = wdS, *wU_ = wU, *wdU_ = wdU, *wT_ = wT;
    const float *la_ = log_a, *beta_ = beta;
    E *dq_ = dq, *dk_ = dk_out, *dv_ = dv_out;
    float *dla_ = dlog_a, *db_ = dbeta;
    asm volatile("" : "+s"(q_), "+s"(k_), "+s"(v_), "+s"(do_), "+s"(wS_), "+s"(wdS_), "+s"(wU_), "+s"(wdU_));
    asm volatile("" : "+s"(wT_), "+s"(la_), "+s"(beta_), "+s"(dq_), "+s"(dk_), "+s"(dv_), "+s"(dla_), "+s"(db_));
    // Per-chunk opaque copies of the buffer and global base addresses: the
    // compiler recomputes addresses inside the loop instead of hoisting
    // hundreds of lane-dependent ones out of it (and spilling them).
    int z0 = 0;
    asm volatile("" : "+s"(z0));
    tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int w = tid >> 6, l = tid & 63;
    const int tb = w % NB;                // token block of this wave's tiles
    const int tl = tb * 16 + (l & 15);    // this lane's token
    const int dsub = (l >> 4) * 4;        // first of this lane's four rows inside a tile
    char* smz = smem + z0;
    E* sdPT = (E*)(smz + Lay::DPT);
    E* sdUt = (E*)(smz + Lay::DUT);
    E* sQ = (E*)(smz + Lay::DUT);
    float* sb = (float*)(smz + Lay::BB);
    float* sgce = (float*)(smz + Lay::GCE);
    float* pdb = (float*)(smz + Lay::PDB);
    float* pcol = (float*)(smz + Lay::PCOL);
    float* pdec = (float*)(smz + Lay::PDEC);
    float* stot = (float*)(smz + Lay::STOT);
    int* sbmax = (int*)(smz + Lay::FL);
    int* scmax = sbmax + 1;
    E* sS = (E*)(smz + Lay::SA);
    E* sdO = (E*)(smz + Lay::DOA);
    E* sUt = (E*)(smz + Lay::UTA);
    float* sG = (float*)(smz + Lay::GL);
    E* sK = (E*)(smz + Lay::KR);
    E* sdAT = (E*)(smz + Lay::DAT);
    E* sT = (E*)(smz + Lay::TB);
    E* sX = (E*)(smz + Lay::XB);
    E* sH = (E*)(smz + Lay::HB);
    E* sZT = (E*)(smz + Lay::ZB);
    E* sKe = (E*)(smz + Lay::KE);
    E* sQs = (E*)(smz + Lay::QS);
    E* sKs = (E*)(smz + Lay::KS);
    E* sDq = (E*)(smz + Lay::KE);
    E* sDk = (E*)(smz + Lay::QS);
    int n;
    const SeqPos cp = tile_pos(m, tile, n);
    const int h = cp.h;
    const int nv = min(C, cp.len - n * C);
    const size_t tok0 = cp.tok0 + (size_t)n * C;
    // the next chunk (the last one again on the final pass: unconditional
    // loads keep the waits on older ones exact)
    const int next = min(tile + (int)gridDim.x, ntiles - 1);
    int nn;
    const SeqPos np = tile_pos(m, next, nn);

    // ================================================ phase A: the state part
    tS.store(sS, LK);
    to.store_masked(sdO, LV, nv);
    tu.store(sUt, LC);
    tdu.store(sdUt, LC);
    lds_barrier();
    LRT_KG_LOAD(tile, cp, n, 4)
    // dP^T = lower(dO U^T)^T: products for the tiles (ti, tj) with tj <= ti,
    // zeros written for the others (phase C's whole-chunk sums read them)
#pragma unroll
    for (int s2 = 0; s2 < ZPW; ++s2) {
      const int t2 = w + NW * s2;
      if (t2 < NZ) {
        const int ti = t2 / NB, tj = t2 % NB;
        f32x4 acc = zero4();
        if (tj <= ti) mma<DV, false, true>(acc, sdO + ti * 16 * LV, LV, sUt + tj * 16, LC);
        const int j = tj * 16 + (l & 15), i0 = ti * 16 + dsub;
        f32x4 dp;
#pragma unroll
        for (int r = 0; r < 4; ++r) dp[r] = (j <= i0 + r) ? acc[r] : 0.f;
        store4<E>(sdPT + j * LC + i0, dp);
      }
      tile_fence();
    }
    // (dO Hn^T)^T (rows d, cols t) kept in registers; dW = -dU Hn^T rows into X
    f32x4 dqa[KPW];
    if constexpr (kSh) {
      f32x4 xw[KPW];
#pragma unroll
      for (int s = 0; s < KPW; ++s) {
        dqa[s] = zero4();
        xw[s] = zero4();
      }
      mma_nA2<DV, KPW, true, false, true>(dqa, xw, sS + (w / NB) * 16, WPB * 16, LK, sdO + tb * 16 * LV, LV,
                                          sdUt + tb * 16, LC);
#pragma unroll
      for (int s = 0; s < KPW; ++s) store4<E>(sX + tl * LK + (w / NB + WPB * s) * 16 + dsub, -xw[s]);
    }
#pragma unroll
    for (int s = 0; s < (kSh ? 0 : KPW); ++s) {
      const int td = w / NB + WPB * s;
      dqa[s] = zero4();
      if (td < NDT) {
        mma<DV, true, false>(dqa[s], sS + td * 16, LK, sdO + tb * 16 * LV, LV);
        f32x4 x = zero4();
        mma<DV, true, true>(x, sS + td * 16, LK, sdUt + tb * 16, LC);
        store4<E>(sX + tl * LK + td * 16 + dsub, -x);
      }
      tile_fence();
    }
    // rowsum(dH' o Hn) per key dimension: dH' from this chunk's registers, Hn
    // from LDS; the lanes holding the same dimensions are summed in the wave,
    // the waves later in wave order
    {
      constexpr int PRs = DK / V;  // 16-byte pieces per state row
      float part[V];
#pragma unroll
      for (int e = 0; e < V; ++e) part[e] = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < tdS.PT; ++s2) {
        const int idx = tid + NT * s2;
        if (tdS.NP % NT == 0 || idx < tdS.NP) {
          const int r = idx / PRs, c = (idx % PRs) * V;
          E a[V];
          __builtin_memcpy(a, &tdS.x[s2], 16);
          float hv[V];
          lds_vec_load<E>(sS + r * LK + c, hv);
#pragma unroll
          for (int e = 0; e < V; ++e) part[e] += to_f(a[e]) * hv[e];
        }
      }
#pragma unroll
      for (int msk = PRs; msk < 64; msk <<= 1) {
#pragma unroll
        for (int e = 0; e < V; ++e) part[e] += __shfl_xor(part[e], msk, 64);
      }
      if (l < PRs) {
#pragma unroll
        for (int e = 0; e < V; ++e) pdec[w * DK + l * V + e] = part[e];
      }
    }
    lds_barrier();
    tdS.store(sS, LK);  // dH'^T over Hn^T
    LRT_KG_LOAD(tile, cp, n, 24)
    lds_barrier();
    // dKt = U dH'^T rows into H
    if constexpr (kSh) {
      f32x4 xk[KPW];
#pragma unroll
      for (int s = 0; s < KPW; ++s) xk[s] = zero4();
      mma_nA<DV, KPW, true, true>(xk, sS + (w / NB) * 16, WPB * 16, LK, sUt + tb * 16, LC);
#pragma unroll
      for (int s = 0; s < KPW; ++s) store4<E>(sH + tl * LK + (w / NB + WPB * s) * 16 + dsub, xk[s]);
    }
#pragma unroll
    for (int s = 0; s < (kSh ? 0 : KPW); ++s) {
      const int td = w / NB + WPB * s;
      if (td < NDT) {
        f32x4 x = zero4();
        mma<DV, true, true>(x, sS + td * 16, LK, sUt + tb * 16, LC);
        store4<E>(sH + tl * LK + td * 16 + dsub, x);
      }
      tile_fence();
    }
    lds_barrier();

    // ================================================ phase B: the WY part
    tg.store_masked(sG, LG, nv);  // log a (rows past the end add 0)
    tk.store_masked(sK, LK, nv);
    tt.store(sT, LC);
    asm volatile("" ::"v"(rb));  // consumed by every lane (no load into it left pending)
    if (tid < C) sb[tid] = tid < nv ? rb : 0.f;
    if (tid == 0) {
      *sbmax = 0;
      *scmax = 0;
    }
    lds_barrier();
    // G = inclusive cumsum of log a over the chunk, per key dimension: thread
    // (d, segment) scans RS rows in registers, then adds the earlier segments' totals
    {
      constexpr int RS = C / NQ;
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
        float off = 0.f;
        for (int s2 = 0; s2 < seg; ++s2) off += stot[s2 * DK + d];
#pragma unroll
        for (int r = 0; r < RS; ++r) sG[(seg * RS + r) * LG + d] = x[r] + off;
      }
      lds_barrier();
    }
    // Running sums from here on, per (dimension, token) of this lane's tiles:
    //   dq = E o (dO Hn^T) (+ R(dP) in phase C),
    //   dk = e^(G_C - G) dKt + b E dX (+ b R(dA) + C in phase C),
    //   dg = k o (the dk terms, those of C and dKt with a minus sign) (+ q o dq at the end).
    // dX^T = (T^T dW)^T, rows d, cols j; dbeta += rowsum(dX o K o E); the
    // row C - 1 term sum_j k_j o e^(G_C - G_j) dKt_j, per token block
    const float btl = sb[tl];
    float dbp = 0.f;  // this lane's dbeta terms (token tl)
    f32x4 dka[KPW], dga[KPW], dxa[KPW];
#pragma unroll
    for (int s = 0; s < KPW; ++s) dxa[s] = zero4();
    if constexpr (kSh) mma_nA<C, KPW, true, true>(dxa, sX + (w / NB) * 16, WPB * 16, LK, sT + tb * 16, LC);
#pragma unroll
    for (int s = 0; s < KPW; ++s) {
      const int td = w / NB + WPB * s;
      dka[s] = zero4();
      dga[s] = zero4();
      if (td < NDT) {
        const int d0 = td * 16 + dsub;
        if constexpr (!kSh) mma<C, true, true>(dxa[s], sX + td * 16, LK, sT + tb * 16, LC);
        const f32x4 g = *(const f32x4*)(sG + tl * LG + d0);
        const f32x4 gc = *(const f32x4*)(sG + (C - 1) * LG + d0);
        const f32x4 kk = load4<E>(sK + tl * LK + d0);
        const f32x4 dkt = load4<E>(sH + tl * LK + d0);
        f32x4 colp;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __expf(g[r]);
          const float kt = __expf(gc[r] - g[r]) * dkt[r];
          const float xp = btl * e * dxa[s][r];
          dqa[s][r] *= e;
          dka[s][r] = xp + kt;
          dga[s][r] = kk[r] * (xp - kt);
          dbp += dxa[s][r] * kk[r] * e;
          colp[r] = sum16(kk[r] * kt);  // over the 16 tokens of the tile
        }
        if ((l & 15) == 0) *(f32x4*)(pcol + tb * DK + d0) = colp;
      }
      tile_fence();
    }
    lds_barrier();
    // dX rows over dW; K o E rows; e^(G_C)
#pragma unroll
    for (int s = 0; s < KPW; ++s) {
      const int td = w / NB + WPB * s;
      if (td < NDT) store4<E>(sX + tl * LK + td * 16 + dsub, dxa[s]);
    }
    for (int p = tid; p < C * (DK / V); p += NT) {
      const int t = p / (DK / V), d0 = (p % (DK / V)) * V;
      float x[V], g[V];
      lds_vec_load<E>(sK + t * LK + d0, x);
      lds_f32_load<V>(sG + t * LG + d0, g);
#pragma unroll
      for (int e = 0; e < V; ++e) x[e] *= __expf(g[e]);
      *(u32x4*)(sH + t * LK + d0) = vec_pack<E>(x);
    }
    if (tid < DK) sgce[tid] = __expf(sG[(C - 1) * LG + tid]);
    {
      // the largest decay of one 16-token block, max over (block, d) of
      // G(row before the block) - G(the block's last row)
      // and the largest |G| of the chunk (every one within e^60: the whole
      // chunk factorises, phase C)
      float bm = 0.f, cm = 0.f;
      if (tid < DK) {
        for (int b2 = 0; b2 < NB; ++b2)
          bm = fmaxf(bm, (b2 > 0 ? sG[(b2 * 16 - 1) * LG + tid] : 0.f) - sG[(b2 * 16 + 15) * LG + tid]);
#pragma unroll 8
        for (int t = 0; t < C; ++t) cm = fmaxf(cm, fabsf(sG[t * LG + tid]));
      }
#pragma unroll
      for (int msk = 1; msk < 64; msk <<= 1) {
        bm = fmaxf(bm, __shfl_xor(bm, msk, 64));
        cm = fmaxf(cm, __shfl_xor(cm, msk, 64));
      }
      if (l == 0 && w * 64 < DK) {  // non-negative floats order as ints
        atomicMax(sbmax, __float_as_int(bm));
        atomicMax(scmax, __float_as_int(cm));
      }
    }
    lds_barrier();
    // Z = dX (K o E)^T + dY V^T, then Z diag(b) = dX X^T + dY Y^T; tiles (ti, tk), tk <= ti
    f32x4 za[ZPW];
#pragma unroll
    for (int s2 = 0; s2 < ZPW; ++s2) {
      const int t2 = w + NW * s2;
      za[s2] = zero4();
      if (t2 < NZ && t2 % NB <= t2 / NB)
        mma<DK>(za[s2], sX + (t2 / NB) * 16 * LK, LK, sH + (t2 % NB) * 16 * LK, LK);
      tile_fence();
    }
    lds_barrier();
    tv.store_masked(sH, LV, nv);  // v rows over K o E
    // dY^T = (T^T dU)^T, rows v, cols j -> dY rows over dX
    f32x4 ya[YPW];
#pragma unroll
    for (int s = 0; s < YPW; ++s) ya[s] = zero4();
    if constexpr (kSh) {
      mma_nA<C, YPW, false, true>(ya, sdUt + (w / NB) * 16 * LC, WPB * 16 * LC, LC, sT + tb * 16, LC);
    } else {
#pragma unroll
      for (int s = 0; s < YPW; ++s) {
        const int tvb = w / NB + WPB * s;
        if (tvb < NVT) mma<C, false, true>(ya[s], sdUt + tvb * 16 * LC, LC, sT + tb * 16, LC);
        tile_fence();
      }
    }
#pragma unroll
    for (int s = 0; s < YPW; ++s) {
      const int tvb = w / NB + WPB * s;
      if (tvb < NVT) store4<E>(sX + tl * LV + tvb * 16 + dsub, ya[s]);
    }
    lds_barrier();
    // dbeta += rowsum(dY o V)
#pragma unroll
    for (int s = 0; s < YPW; ++s) {
      const int tvb = w / NB + WPB * s;
      if (tvb < NVT) {
        const f32x4 vv = load4<E>(sH + tl * LV + tvb * 16 + dsub);
#pragma unroll
        for (int r = 0; r < 4; ++r) dbp += ya[s][r] * vv[r];
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < ZPW; ++s2) {
      const int t2 = w + NW * s2;
      if (t2 < NZ) {
        const int ti = t2 / NB, tk2 = t2 % NB;
        if (tk2 <= ti) mma<DV>(za[s2], sX + ti * 16 * LV, LV, sH + tk2 * 16 * LV, LV);
        const int kc = tk2 * 16 + (l & 15);
        store4<E>(sZT + kc * LC + ti * 16 + dsub, za[s2] * sb[kc]);
      }
      tile_fence();
    }
    lds_barrier();
    // dA^T = -strict_lower(Z diag(b) T^T)^T: products for the tiles (ti, tj)
    // with tj <= ti, zeros written for the others
#pragma unroll
    for (int s2 = 0; s2 < ZPW; ++s2) {
      const int t2 = w + NW * s2;
      if (t2 < NZ) {
        const int ti = t2 / NB, tj = t2 % NB;
        f32x4 acc = zero4();
        if (tj <= ti) mma<C, true, false>(acc, sZT + ti * 16, LC, sT + tj * 16 * LC, LC);
        const int j = tj * 16 + (l & 15), i0 = ti * 16 + dsub;
        f32x4 da;
#pragma unroll
        for (int r = 0; r < 4; ++r) da[r] = (j < i0 + r) ? -acc[r] : 0.f;
        store4<E>(sdAT + j * LC + i0, da);
      }
      tile_fence();
    }
    // dv = b dY rows out
    for (int p = tid; p < C * (DV / V); p += NT) {
      const int t = p / (DV / V), c0 = (p % (DV / V)) * V;
      if (t < nv)
        *(u32x4*)(dv_ + ((tok0 + t) * H + h) * DV + c0) = vec_scale<E>(*(const u32x4*)(sX + t * LV + c0), sb[t]);
    }
    lds_barrier();

    // ================================================ phase C: the decayed token sums
    // Regime: "fast" while no 16-token block decays by more than e^60 in any
    // dimension.  Every pair i >= j splits its decay as
    //   e^(G_i - G_j) = e^(G_i - G_ref(i)) e^(G_ref(i) - G_s(j)) e^(G_s(j) - G_j),
    // s(j) = the last row of j's block; ref(i) = the last row of i's block
    // (fast: the first factor in [1, e^60]) or the row before i's block
    // (exact: every factor <= 1, diagonal blocks pair by pair).  Staged rows:
    //   Kend_j = k_j e^(G_s(j) - G_j),  Qx_i = q_i e^(G_i - G_ref(i)),  bKx_i = b_i k_i e^(G_i - G_ref(i)).
    // In the fast regime both halves of a pair's dG term (row side +, column
    // side -) are formed from the same rounded staged rows, so they cancel
    // in the reverse cumsum as they do in exact arithmetic.  While every |G|
    // of the chunk is within e^60 (fastc) the whole chunk is one block with
    // its reference at the chunk start (G = 0): Kend_j = k_j e^(-G_j),
    // Qx_i = q_i e^(G_i), and each sum is one product over all C tokens.
    const bool fastd = __int_as_float(*sbmax) <= 60.f;
    const bool fastc = fastd && __int_as_float(*scmax) <= 60.f;
    // q rows over dU^T; Qx from this thread's own q pieces, before the
    // registers take the next chunk's q
    tq.store_masked(sQ, LK, nv);
#pragma unroll
    for (int s2 = 0; s2 < tq.PT; ++s2) {
      const int idx = tid + NT * s2;
      if (tq.NP % NT == 0 || idx < tq.NP) {
        const int t = idx / (DK / V), d0 = (idx % (DK / V)) * V, blk = t >> 4;
        const int ref = fastc ? -1 : fastd ? blk * 16 + 15 : blk * 16 - 1;
        E e[V];
        __builtin_memcpy(e, &tq.x[s2], 16);
        float g[V], gr[V], x[V];
        lds_f32_load<V>(sG + t * LG + d0, g);
        if (ref >= 0)
          lds_f32_load<V>(sG + ref * LG + d0, gr);
        else
#pragma unroll
          for (int i = 0; i < V; ++i) gr[i] = 0.f;
#pragma unroll
        for (int i = 0; i < V; ++i) x[i] = t < nv ? to_f(e[i]) * __expf(g[i] - gr[i]) : 0.f;
        *(u32x4*)(sQs + t * LK + d0) = vec_pack<E>(x);
      }
    }
    LRT_KG_LOAD(next, np, nn, 1)
    for (int p = tid; p < C * (DK / V); p += NT) {
      const int t = p / (DK / V), d0 = (p % (DK / V)) * V, blk = t >> 4;
      const int ref = fastc ? -1 : fastd ? blk * 16 + 15 : blk * 16 - 1;
      float kx[V], g[V], gs[V], gr[V], a[V], b2[V];
      lds_vec_load<E>(sK + t * LK + d0, kx);
      lds_f32_load<V>(sG + t * LG + d0, g);
      if (fastc)
#pragma unroll
        for (int i = 0; i < V; ++i) gs[i] = 0.f;
      else
        lds_f32_load<V>(sG + (blk * 16 + 15) * LG + d0, gs);
      if (ref >= 0)
        lds_f32_load<V>(sG + ref * LG + d0, gr);
      else
#pragma unroll
        for (int i = 0; i < V; ++i) gr[i] = 0.f;
      const float bt = sb[t];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        a[i] = kx[i] * __expf(gs[i] - g[i]);
        b2[i] = bt * kx[i] * __expf(g[i] - gr[i]);
      }
      *(u32x4*)(sKe + t * LK + d0) = vec_pack<E>(a);
      *(u32x4*)(sKs + t * LK + d0) = vec_pack<E>(b2);
    }
    lds_barrier();
    // R over the tokens j <= i of this lane's token i (rows d, cols i):
    //   R = e^(G_i - G_ref) sum_{sj} e^(G_ref - G_s(sj)) (M_{si,sj} Kend_{sj})  [+ exact diagonal]
    // dq += R(dP); dk += b R(dA); dbeta += rowsum(k o R(dA)); dG += q o dq + b k o R(dA)
#pragma unroll
    for (int s = 0; s < KPW; ++s) {
      const int td = w / NB + WPB * s;
      if (td < NDT) {
        const int d0 = td * 16 + dsub;
        const f32x4 gi = *(const f32x4*)(sG + tl * LG + d0);
        const int ref = fastc ? -1 : fastd ? tb * 16 + 15 : tb * 16 - 1;
        const f32x4 gref = ref >= 0 ? *(const f32x4*)(sG + ref * LG + d0) : zero4();
        const f32x4 kk = load4<E>(sK + tl * LK + d0), qq = load4<E>(sQ + tl * LK + d0);
        f32x4 rp = zero4(), ra = zero4();
        if (fastc) {
          mma<C, true, true>(rp, sKe + td * 16, LK, sdPT + tb * 16, LC);
          mma<C, true, true>(ra, sKe + td * 16, LK, sdAT + tb * 16, LC);
        }
        const int nsj = fastc ? 0 : fastd ? tb + 1 : tb;
        for (int sj = 0; sj < nsj; ++sj) {
          f32x4 xp = zero4(), xa = zero4();
          mma<16, true, true>(xp, sKe + sj * 16 * LK + td * 16, LK, sdPT + sj * 16 * LC + tb * 16, LC);
          mma<16, true, true>(xa, sKe + sj * 16 * LK + td * 16, LK, sdAT + sj * 16 * LC + tb * 16, LC);
          const f32x4 gs = *(const f32x4*)(sG + (sj * 16 + 15) * LG + d0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float f = __expf(gref[r] - gs[r]);
            rp[r] += f * xp[r];
            ra[r] += f * xa[r];
          }
        }
        f32x4 dg = qq * dqa[s];  // dG's q o (E o dO Hn^T) term
        if (fastd) {
          const f32x4 qx = load4<E>(sQs + tl * LK + d0), kx = load4<E>(sKs + tl * LK + d0);
          dg += qx * rp + kx * ra;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __expf(gi[r] - gref[r]);
          rp[r] *= e;
          ra[r] *= e;
        }
        if (!fastd) {
#pragma unroll 1
          for (int jj = 0; jj < 16; ++jj) {
            const int j = tb * 16 + jj;
            const f32x4 gj = *(const f32x4*)(sG + j * LG + d0);
            const f32x4 kj = load4<E>(sK + j * LK + d0);
            const float dp = to_f(sdPT[j * LC + tl]);  // zero for j > i
            const float da = to_f(sdAT[j * LC + tl]);  // zero for j >= i
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float D = j <= tl ? __expf(gi[r] - gj[r]) : 0.f;  // never e^(positive)
              rp[r] += dp * kj[r] * D;
              ra[r] += da * kj[r] * D;
            }
          }
          dg += qq * rp + btl * kk * ra;
        }
        dga[s] += dg;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          dqa[s][r] += rp[r];
          dka[s][r] += btl * ra[r];
          dbp += kk[r] * ra[r];
        }
      }
      tile_fence();
    }
    // C over the tokens i >= j of this lane's token j (rows d, cols j):
    //   C = e^(G_s(sj) - G_j) sum_{si} e^(G_ref(si) - G_s(sj)) (Qx_si^T dP_{si,sj} + bKx_si^T dA_{si,sj})
    //   [+ exact diagonal];  dk += C; dG -= k o C
#pragma unroll
    for (int s = 0; s < KPW; ++s) {
      const int td = w / NB + WPB * s;
      if (td < NDT) {
        const int d0 = td * 16 + dsub;
        const f32x4 gj = *(const f32x4*)(sG + tl * LG + d0);
        const f32x4 gs = fastc ? zero4() : *(const f32x4*)(sG + (tb * 16 + 15) * LG + d0);
        f32x4 cc = zero4();
        if (fastc) {
          mma<C, true, false>(cc, sQs + td * 16, LK, sdPT + tb * 16 * LC, LC);
          mma<C, true, false>(cc, sKs + td * 16, LK, sdAT + tb * 16 * LC, LC);
        }
        for (int si = fastc ? NB : fastd ? tb : tb + 1; si < NB; ++si) {
          f32x4 x = zero4();
          mma<16, true, false>(x, sQs + si * 16 * LK + td * 16, LK, sdPT + tb * 16 * LC + si * 16, LC);
          mma<16, true, false>(x, sKs + si * 16 * LK + td * 16, LK, sdAT + tb * 16 * LC + si * 16, LC);
          const int ref = fastd ? si * 16 + 15 : si * 16 - 1;
          const f32x4 gr = *(const f32x4*)(sG + ref * LG + d0);
#pragma unroll
          for (int r = 0; r < 4; ++r) cc[r] += __expf(gr[r] - gs[r]) * x[r];
        }
        f32x4 dg = zero4();
        if (fastd) dg = load4<E>(sKe + tl * LK + d0) * cc;
#pragma unroll
        for (int r = 0; r < 4; ++r) cc[r] *= __expf(gs[r] - gj[r]);
        if (!fastd) {
#pragma unroll 1
          for (int ii = 0; ii < 16; ++ii) {
            const int i = tb * 16 + ii;
            const f32x4 gi = *(const f32x4*)(sG + i * LG + d0);
            const f32x4 qi = load4<E>(sQ + i * LK + d0);
            const f32x4 ki = load4<E>(sK + i * LK + d0);
            const float dp = to_f(sdPT[tl * LC + i]);            // zero for i < j
            const float bda = sb[i] * to_f(sdAT[tl * LC + i]);  // zero for i <= j
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float D = i >= tl ? __expf(gi[r] - gj[r]) : 0.f;
              cc[r] += (dp * qi[r] + bda * ki[r]) * D;
            }
          }
          dg = load4<E>(sK + tl * LK + d0) * cc;
        }
        dka[s] += cc;
        dga[s] -= dg;
      }
      tile_fence();
    }
    dbp = sum4(dbp);  // over the lanes of this token (its four row groups)
    if (l < 16) pdb[w * C + tl] = dbp;
    lds_barrier();
    // dG over G, dq and dk rows over the staged operands
#pragma unroll
    for (int s = 0; s < KPW; ++s) {
      const int td = w / NB + WPB * s;
      if (td < NDT) {
        const int d0 = td * 16 + dsub;
        *(f32x4*)(sG + tl * LG + d0) = dga[s];
        store4<E>(sDq + tl * LK + d0, dqa[s]);
        store4<E>(sDk + tl * LK + d0, dka[s]);
      }
    }
    lds_barrier();
    // row C - 1 also carries the chunk-decay terms: sum_j k_j o e^(G_C - G_j) dKt_j
    // (per token block, in block order) and e^(G_C) o rowsum(dH' o Hn) (in wave order)
    if (tid < DK) {
      float add = 0.f, dec = 0.f;
      for (int b2 = 0; b2 < NB; ++b2) add += pcol[b2 * DK + tid];
      for (int w2 = 0; w2 < NW; ++w2) dec += pdec[w2 * DK + tid];
      sG[(C - 1) * LG + tid] += add + sgce[tid] * dec;
    }
    lds_barrier();
    // dlog_a = reverse cumsum of dG over the chunk, per key dimension
    {
      constexpr int RS = C / NQ;
      const int d = tid % DK, seg = tid / DK;
      float x[RS];
      if (seg < NQ) {
#pragma unroll
        for (int r = 0; r < RS; ++r) x[r] = sG[(seg * RS + r) * LG + d];
#pragma unroll
        for (int r = RS - 2; r >= 0; --r) x[r] += x[r + 1];
        stot[seg * DK + d] = x[0];
      }
      lds_barrier();
      if (seg < NQ) {
        float off = 0.f;
        for (int s2 = NQ - 1; s2 > seg; --s2) off += stot[s2 * DK + d];
#pragma unroll
        for (int r = 0; r < RS; ++r) sG[(seg * RS + r) * LG + d] = x[r] + off;
      }
      lds_barrier();
    }
    LRT_KG_LOAD(next, np, nn, 2)
    lds_to_rows<float, C, DK, NT>(dla_ + (tok0 * H + h) * DK, (size_t)H * DK, sG, LG, nv);
    lds_to_rows<E, C, DK, NT>(dq_ + (tok0 * H + h) * DK, (size_t)H * DK, sDq, LK, nv);
    lds_to_rows<E, C, DK, NT>(dk_ + (tok0 * H + h) * DK, (size_t)H * DK, sDk, LK, nv);
    if (tid < nv) {
      const int bt = tid >> 4;
      float sum = 0.f;
      for (int i2 = 0; i2 < WPB; ++i2) sum += pdb[(bt + NB * i2) * C + tid];
      db_[(tok0 + tid) * H + h] = sum;
    }
    lds_barrier();
  }
#undef LRT_KG_LOAD
}

template <typename E, int C, int DK, int DV>
constexpr bool kda_bwd_fits() {
  return KdaLds<E, C, DK, DV, 64 * kWyWaves>::TOTAL <= kLdsMax && scan_bv<E, C, DK, DV, kScanBwd, true>() > 0 &&
         scan_bv<E, C, DK, DV, kScanFwd, true>() > 0 &&
         dstate_bv<E, C, DK, DV, true, 64, true>() > 0 && KdaGradLds<E, C, DK, DV, kGradWaves>::TOTAL <= kLdsMax;
}

// saved: the workspace already holds W, U', Ktil, G_C, Q o e^G, P, Tinv, S_n
// and U from kda_fwd_train of the same arguments, so the recompute is
// skipped.
template <typename E, int C, int DK, int DV>
int kda_bwd_impl(const BwdArgs& a, bool saved) {
  if constexpr (!kda_bwd_fits<E, C, DK, DV>()) {
    return -3;  // not reached: the entry point runs a chunk that fits (kda_bwd_max_chunk)
  } else {
    const bool packed = a.cu != nullptr;
    const int tiles = (int)ws_tiles(a.B, a.T, a.H, C, packed);
    const BwdWs ws = bwd_ws_layout(LRT_OP_KDA_BWD, a.B, a.T, a.H, DK, DV, C, sizeof(E), a.workspace, packed);
    const SeqMap sm = seq_map(a.B, a.T, a.H, C, a.cu, ws.f);
    hipStream_t st = (hipStream_t)a.stream;
    if (packed && launch_varlen_plan(a.cu, a.B, a.T, C, ws.f, a.stream) != 0) return -7;
    if (!saved) {
      // the forward recomputed: the chunk-parallel pass (with Tinv), then the
      // state scan writing the chunk-start states and U
      if (launch_kda_prep<E, C, DK, DV, false>(a.q, a.k, a.v, a.log_a, a.beta, sm, ws.f, (E*)ws.T, nullptr, tiles,
                                               kKKdaPrepFastBwd, kKKdaPrepBwd, st) != 0)
        return -7;
      constexpr int BVS = scan_bv<E, C, DK, DV, kScanBwd, true>();
      ScanArgs<E> sa{};
      sa.W = (const E*)ws.f.W;
      sa.Up = (const E*)ws.f.Up;
      sa.Kt = (const E*)ws.f.Kt;
      sa.GC = ws.f.GC;
      sa.hin = a.h0;
      sa.hs_ld = DV;
      sa.U = (E*)ws.f.U;
      sa.S = (E*)ws.f.S;
      sa.m = sm;
      sa.L = 1 << 30;
      sa.nseg = 1;
      sa.DV = DV;
      LRT_LAUNCH(kKScanBwd, (k_scan<E, C, DK, BVS, kScanBwd, true, kStateWaves>), dim3(a.B * a.H * (DV / BVS)),
                 dim3(64 * kStateWaves), st, sa);
    }
    constexpr int BV = dstate_bv<E, C, DK, DV, true, 64, true>();
    LRT_LAUNCH(kKDState, (k_dstate<E, C, DK, BV, kStateWaves, true, true, false, true>), dim3(a.B * a.H * (DV / BV)),
               dim3(64 * kStateWaves), st, (const E*)ws.f.Qg, (const E*)ws.f.Kt, (const E*)a.d_o, ws.f.GC,
               (const E*)ws.f.W, (const E*)ws.f.P, a.dht, a.dh0, (E*)ws.dS, (E*)ws.dU, sm, DV);
    LRT_LAUNCH(kKGradKda, (k_grad_kda<E, C, DK, DV, kGradWaves>),
               dim3(persistent_grid(tiles, KdaGradLds<E, C, DK, DV, kGradWaves>::TOTAL)), dim3(64 * kGradWaves), st,
               (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.d_o, a.log_a, a.beta, (const E*)ws.f.S,
               (const E*)ws.dS, (const E*)ws.f.U, (const E*)ws.dU, (const E*)ws.T, (E*)a.dq, (E*)a.dk_out,
               (E*)a.dv_out, a.dlog_a, a.dbeta, sm);
    return hipGetLastError() == hipSuccess ? 0 : -7;
  }
}

// KDA forward for training: kda_fwd's kernels writing into the backward's
// workspace what kda_bwd_saved reads -- the chunk-parallel pass with Tinv,
// the forward scan also saving the chunk-start states and U.
template <typename E, int C, int DK, int DV>
int kda_fwd_train_impl(const FwdArgs& a) {
  if constexpr (!kda_bwd_fits<E, C, DK, DV>()) {
    return -3;  // not reached: the entry point runs a chunk that fits (kda_bwd_max_chunk)
  } else {
    const BwdWs ws = bwd_ws_layout(LRT_OP_KDA_BWD, a.B, a.T, a.H, DK, DV, C, sizeof(E), a.workspace);
    const int N = (a.T + C - 1) / C;
    const int tiles = a.B * a.H * N;
    if (launch_kda_prep<E, C, DK, DV, false>(a.q, a.k, a.v, a.log_a, a.beta, seq_map(a, ws.f, C), ws.f, (E*)ws.T,
                                             nullptr, tiles, kKKdaPrepFast, kKKdaPrep, (hipStream_t)a.stream) != 0)
      return -7;
    return launch_scan_fwd<E, C, DK, DV, true, true>(a, ws.f, N);
  }
}

template <typename E, int DK, int DV>
constexpr int kda_bwd_max_chunk_t() {
  return kda_bwd_fits<E, 64, DK, DV>() ? 64 : kda_bwd_fits<E, 32, DK, DV>() ? 32 : 16;
}

#define LRT_DV(DK_) LRT_CASE(DK_, 16) LRT_CASE(DK_, 32) LRT_CASE(DK_, 64) LRT_CASE(DK_, 128)
#define LRT_DK LRT_DV(16) LRT_DV(32) LRT_DV(64) LRT_DV(128)

int kda_bwd_max_chunk(int dtype, int dk, int dv) {
#define LRT_CASE(DK_, DV_) \
  if (dk == DK_ && dv == DV_) return dtype == LRT_BF16 ? kda_bwd_max_chunk_t<bf16, DK_, DV_>() : kda_bwd_max_chunk_t<float, DK_, DV_>();
  LRT_DK
#undef LRT_CASE
  return 16;
}

template <typename E>
static int kda_bwd_dtype(const BwdArgs& a, bool saved) {
#define LRT_CASE(DK_, DV_)                                             \
  if (a.dk == DK_ && a.dv == DV_) {                                    \
    if (a.chunk == 16) return kda_bwd_impl<E, 16, DK_, DV_>(a, saved); \
    if (a.chunk == 32) return kda_bwd_impl<E, 32, DK_, DV_>(a, saved); \
    if (a.chunk == 64) return kda_bwd_impl<E, 64, DK_, DV_>(a, saved); \
  }
  LRT_DK
#undef LRT_CASE
  return -2;
}
template <typename E>
static int kda_fwd_train_dtype(const FwdArgs& a) {
#define LRT_CASE(DK_, DV_)                                         \
  if (a.dk == DK_ && a.dv == DV_) {                                \
    if (a.chunk == 16) return kda_fwd_train_impl<E, 16, DK_, DV_>(a); \
    if (a.chunk == 32) return kda_fwd_train_impl<E, 32, DK_, DV_>(a); \
    if (a.chunk == 64) return kda_fwd_train_impl<E, 64, DK_, DV_>(a); \
  }
  LRT_DK
#undef LRT_CASE
  return -2;
}
#undef LRT_DK
#undef LRT_DV

int bwd_kda(const BwdArgs& a, bool saved) {
  return a.dtype == LRT_BF16 ? kda_bwd_dtype<bf16>(a, saved) : kda_bwd_dtype<float>(a, saved);
}
int fwd_train_kda(const FwdArgs& a) {
  return a.dtype == LRT_BF16 ? kda_fwd_train_dtype<bf16>(a) : kda_fwd_train_dtype<float>(a);
}

}  // namespace lrt
