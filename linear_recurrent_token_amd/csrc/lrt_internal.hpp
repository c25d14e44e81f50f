// lrt_internal.hpp -- host-side argument bundles and workspace layout of liblrt.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/lrt.h"
#include "lrt_common.hpp"

namespace lrt {

// LDS of one workgroup on gfx950.
constexpr size_t kLdsMax = 160 * 1024;
// Rank of KDA's low-rank gate projection (the bottleneck of the fused
// prologue's gate input).
constexpr int kGateRank = 16;

enum { kVarGDN = 0, kVarSSD = 1, kVarKDA = 2 };

struct FwdArgs {
  int variant;
  const void *q, *k, *v;
  const float *log_a, *beta, *h0;
  void* o;
  float* ht;
  int B, T, H, dk, dv, chunk, dtype;
  void* workspace;
  void* stream;
  const int* cu = nullptr;  // packed sequences: cu_seqlens [B + 1] (B sequences in [1, T, H, d]); nullptr: dense
  bool fuse = false;        // q, k, log_a, beta are raw projections (the fused prologue)
  const void* gate_up = nullptr;  // KDA fused prologue with the low-rank gate: W_up [H*d_k][kGateRank]; log_a = z
};

struct BwdArgs {
  const void *q, *k, *v;
  const float *log_a, *beta, *h0;
  const void* d_o;
  const float* dht;
  void *dq, *dk_out, *dv_out;
  float *dlog_a, *dbeta, *dh0;
  int B, T, H, dk, dv, chunk, dtype;
  void* workspace;
  void* stream;
  const int* cu = nullptr;  // as FwdArgs::cu
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Per-chunk workspace tiles, chunk-major per (b, h); each op reserves only
// the tiles its kernels use (lrt_workspace_bytes op codes):
//   W   [C][dk]   E   W = Tinv diag(b gamma) K           GDN_FWD, KDA_FWD, GDN_BWD, KDA_BWD
//   Up  [dv][C]   E   U' = Tinv diag(b) V (tile order)   GDN_FWD, KDA_FWD, GDN_BWD, KDA_BWD; SSD_BWD: dU_local^T
//   Kt  [dk][C]   E   Ktil^T, Ktil_j = e^(G_C - G_j) k_j KDA_FWD, KDA_BWD
//   U   [dv][C]   E   U^T = (U' - W Hn)^T                GDN_BWD, KDA_BWD; SSD_BWD: V^T
//   S   [dv][dk]  E   S_n = Hn^T, the chunk-start state  GDN_BWD, SSD_BWD, KDA_BWD
//   G   [C]       f32 within-chunk inclusive cumsum of log a   GDN_FWD, GDN_BWD, SSD_BWD
//   GC  [dk]      f32 per-key-dim chunk log-decay        KDA_FWD, KDA_BWD
//   Qg  [C][dk]   E   Q o e^G                            KDA_FWD, KDA_BWD
//   P   [C][C]    E   (Q K^T) o Gamma (SSD_BWD: P^T)     GDN_FWD, KDA_FWD, GDN_BWD, SSD_BWD, KDA_BWD
//   SegLoc   [b*h][seg][dk][dv+dk] f32  end state of each segment from zero, and its map
//   SegStart [b*h][seg][dk][dv]    f32  true start state of each segment
//                                       (segmented scans: GDN_FWD, KDA_FWD, GDN_BWD)
// The backward's own tiles (T, dS, dU) follow (bwd_ws_layout).
//   cs, cl [B], co [B + 1]  int  packed sequences: starts, lengths, chunk offsets
struct FwdWs {
  void *W, *Up, *Kt, *U, *S, *Qg, *P;
  float *G, *GC, *SegLoc, *SegStart;
  int *cs, *cl, *co;
  int* slow;  // KDA: the exact-path chunk list k_kda_prep_fast leaves (count, then tiles)
  size_t bytes;
};

// Column block and segments of the forward scan.  One segment of up to 64
// columns per workgroup unless those (b, h, column block) workgroups alone
// would leave the device mostly idle; then 128-column blocks (when d_k is a
// multiple, for the identity columns of the local pass) and enough segments
// for about 512 workgroups, each at least 16 chunks long.  Depends on the
// shape only, so the workspace size does not depend on the device.  (The
// scan may run narrower column blocks where its operands need more LDS; the
// segments stay as planned.)
struct ScanPlan {
  int bv, nseg;
};
inline ScanPlan scan_plan(int B, int H, int DK, int DV, int N) {
  const int bv64 = DV < 64 ? DV : 64;
  if ((long)B * H * (DV / bv64) >= 256 || N < 32) return {bv64, 1};
  int bv = DV < 128 ? DV : 128;
  if (DK % bv != 0) bv = bv64;
  if (DK % bv != 0) return {bv64, 1};
  const long wgs = (long)B * H * (DV / bv);
  long ns = (512 + wgs - 1) / wgs;
  if (ns > N / 16) ns = N / 16;
  return {bv, ns < 1 ? 1 : (int)ns};
}

// Chunk tiles of a workspace: B H ceil(T / C) (dense), or, for B packed
// sequences of T tokens in all, at most H (ceil(T / C) + B) (each sequence
// adds at most one partial chunk).
inline size_t ws_tiles(int B, int T, int H, int C, bool packed) {
  const size_t N = (size_t)(T + C - 1) / C;
  return packed ? (size_t)H * (N + B) : (size_t)B * H * N;
}

inline FwdWs fwd_ws_layout(int op, int B, int T, int H, int dk, int dv, int C, size_t esz, void* base,
                           bool packed = false) {
  const size_t N = (size_t)(T + C - 1) / C;
  const size_t tiles = ws_tiles(B, T, H, C, packed);
  const bool gf = op == LRT_OP_GDN_FWD, kf = op == LRT_OP_KDA_FWD, gb = op == LRT_OP_GDN_BWD,
             sb = op == LRT_OP_SSD_BWD, kb = op == LRT_OP_KDA_BWD;
  size_t off = 0;
  FwdWs w;
  char* p = (char*)base;
  auto take = [&](bool need, size_t bytes) {
    if (!need) return (void*)nullptr;
    void* r = p ? (void*)(p + off) : nullptr;
    off += align256(bytes);
    return r;
  };
  w.W = take(gf || kf || gb || kb, tiles * C * dk * esz);
  w.Up = take(gf || kf || gb || sb || kb, tiles * dv * C * esz);
  w.Kt = take(kf || kb, tiles * dk * C * esz);
  w.U = take(gb || sb || kb, tiles * dv * C * esz);
  w.S = take(gb || sb || kb, tiles * dv * dk * esz);
  w.G = (float*)take(gf || gb || sb, tiles * C * sizeof(float));
  w.GC = (float*)take(kf || kb, tiles * dk * sizeof(float));
  w.Qg = take(kf || kb, tiles * C * dk * esz);
  w.P = take(gf || kf || gb || sb || kb, tiles * C * C * esz);
  const int nseg = (gf || kf || gb || kb) && !packed ? scan_plan(B, H, dk, dv, (int)N).nseg : 1;
  w.SegLoc = (float*)take(nseg > 1, (size_t)B * H * nseg * dk * (dv + dk) * sizeof(float));
  w.SegStart = (float*)take(nseg > 1, (size_t)B * H * nseg * dk * dv * sizeof(float));
  w.cs = (int*)take(packed, (size_t)B * sizeof(int));
  w.cl = (int*)take(packed, (size_t)B * sizeof(int));
  w.co = (int*)take(packed, (size_t)(B + 1) * sizeof(int));
  w.slow = (int*)take(kf || kb, (tiles + 1) * sizeof(int));
  w.bytes = off;
  return w;
}

// Backward-only workspace tiles, after the forward's (chunk-major per (b, h)):
//   T   [C][C]   E    Tinv
//   dS  [dv][dk] E    dH'^T, gradient of each chunk's end state
//   dU  [dv][C]  E    dU^T
// dU_local reuses the forward's U' tiles (dead once the state pass has run).
struct BwdWs {
  FwdWs f;
  void *T, *dS, *dU;
  size_t bytes;
};

// op: LRT_OP_GDN_BWD (also the Gated DeltaNet training forward),
// LRT_OP_KDA_BWD, or LRT_OP_SSD_BWD (also the Mamba2 training forward; no Tinv)
inline BwdWs bwd_ws_layout(int op, int B, int T, int H, int dk, int dv, int C, size_t esz, void* base,
                           bool packed = false) {
  BwdWs w;
  w.f = fwd_ws_layout(op, B, T, H, dk, dv, C, esz, base, packed);
  const size_t tiles = ws_tiles(B, T, H, C, packed);
  size_t off = w.f.bytes;
  char* p = (char*)base;
  auto take = [&](size_t bytes) {
    void* r = p ? (void*)(p + off) : nullptr;
    off += align256(bytes);
    return r;
  };
  w.T = op == LRT_OP_GDN_BWD || op == LRT_OP_KDA_BWD ? take(tiles * C * C * esz) : nullptr;
  w.dS = take(tiles * dv * dk * esz);
  w.dU = take(tiles * dv * C * esz);
  w.bytes = off;
  return w;
}

inline size_t bwd_ws_extra(int op, int B, int T, int H, int dk, int dv, int C, size_t esz, bool packed = false) {
  const BwdWs w = bwd_ws_layout(op, B, T, H, dk, dv, C, esz, nullptr, packed);
  return w.bytes - w.f.bytes;
}

// The kernels' view of the sequences (the packed layout's tables live in
// the workspace, filled by k_varlen_plan).
inline SeqMap seq_map(int B, int T, int H, int C, const int* cu, const FwdWs& ws) {
  if (cu == nullptr) return SeqMap{nullptr, nullptr, nullptr, T, H, C, (T + C - 1) / C, B};
  return SeqMap{ws.cs, ws.cl, ws.co, T, H, C, 0, B};
}
inline SeqMap seq_map(const FwdArgs& a, const FwdWs& ws, int C) { return seq_map(a.B, a.T, a.H, C, a.cu, ws); }

// Kernel ids reported by the benchmark timing hook (lrt_profile_attach).
enum KernelKind {
  kKBwdLocal = 0,
  kKDState,
  kKGrad,
  kKKdaPrep,
  kKStateCopy,
  kKWy,
  kKScan,
  kKWyBwd,
  kKScanBwd,
  kKScanLocal,
  kKCarry,
  kKSsdPrep,
  kKSsdFwd,
  kKVarlenPlan,
  kKKdaPrepBwd,
  kKGradKda,
  kKKdaPrepFast,
  kKKdaPrepFastBwd,
  kKListReset,
  kKConvFwd,
  kKConvBwd,
  kKConvDw,
  kKNormFwd,
  kKNormBwd,
  kKNormDw,
  kKNumKinds
};
// Bracket one launch with the timing hook's events (no-ops unless attached).
void prof_before(int kind, void* stream);
void prof_after(void* stream);

#define LRT_LAUNCH(kind, kernel, grid, block, stream, ...)                        \
  do {                                                                         \
    ::lrt::prof_before((kind), (void*)(stream));                               \
    hipLaunchKernelGGL(kernel, grid, block, 0, (hipStream_t)(stream), __VA_ARGS__); \
    ::lrt::prof_after((void*)(stream));                                        \
  } while (0)

// Waves per workgroup of the serial state passes.
constexpr int kStateWaves = 8;
// Waves per workgroup of the chunk-parallel gradient kernel.
constexpr int kGradWaves = 8;
// Waves per workgroup of the chunk-parallel WY pass.
constexpr int kWyWaves = 8;

// Compute units of the current device (cached per device id).
int device_cu_count();
// Packed sequences: fills the workspace's sequence tables from cu_seqlens
// (on the caller's stream, before any kernel that reads them).
int launch_varlen_plan(const int* cu, int B, int T, int C, const FwdWs& ws, void* stream);

// Grid of a chunk-parallel kernel that walks its tiles persistently: enough
// workgroups to fill every CU at the occupancy its LDS allows, never more
// than there are tiles.
inline int persistent_grid(int tiles, size_t lds_bytes) {
  int per_cu = lds_bytes ? (int)(160 * 1024 / lds_bytes) : 8;
  per_cu = per_cu < 1 ? 1 : (per_cu > 8 ? 8 : per_cu);
  const long g = (long)device_cu_count() * per_cu;
  return (int)(tiles < g ? tiles : g);
}

int fwd_scalar_gate(const FwdArgs& a);
int fwd_kda(const FwdArgs& a);
int bwd_gdn(const BwdArgs& a, bool saved);
int fwd_train(const FwdArgs& a);  // GDN or SSD by a.variant
int bwd_ssd(const BwdArgs& a, bool saved);
int bwd_kda(const BwdArgs& a, bool saved);
int fwd_train_kda(const FwdArgs& a);  // kda_fwd_train

// The largest chunk in {16, 32, 64} at which every kernel of `op` (an
// LRT_OP_* code; the training forwards count as the backward's op) fits in
// LDS for this dtype and d_k, d_v.  The kernels run min(requested chunk,
// this); the chunkwise form is exact for every chunk size, so only the
// rounding of the result depends on it.
int fwd_max_chunk(int dtype, int dk, int dv);  // GDN_FWD, SSD_FWD
int kda_max_chunk(int dtype, int dk, int dv);
int bwd_max_chunk(int op, int dtype, int dk, int dv);  // GDN_BWD, SSD_BWD
int kda_bwd_max_chunk(int dtype, int dk, int dv);

}  // namespace lrt
