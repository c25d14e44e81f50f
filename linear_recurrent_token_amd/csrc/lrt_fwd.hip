// lrt_fwd.hip -- launchers of the chunkwise forward (gdn_fwd, ssd_fwd).
#include "lrt_internal.hpp"
#include "lrt_scan.hpp"
#include "lrt_ssd_fwd.hpp"

namespace lrt {

// ------------------------------------------------------------ k_varlen_plan
// Packed sequences: sequence s spans tokens [cu[s], cu[s + 1]) of the
// [1, T, H, d] tensors.  One workgroup writes the tables every kernel reads:
//   cs[s] = m_s, cl[s] = m_{s+1} - m_s, co[s] = chunks of the sequences before s,
// with m_i = max(cu[0..i]) clamped into [0, T].  For a valid cu_seqlens
// (non-decreasing, cu[0] = 0, cu[B] = T) this is cu itself; any other input
// still yields disjoint sequences inside [0, T], so no kernel reads or
// writes outside the tensors or beyond the workspace's chunk tiles.
// Each thread takes a contiguous range of entries; block scans (max, then
// sum) over the per-thread partials in LDS.
__device__ __forceinline__ int block_scan_incl(int* part, int x, bool is_max) {
  const int t = threadIdx.x;
  part[t] = x;
  __syncthreads();
  for (int d = 1; d < (int)blockDim.x; d <<= 1) {
    const int y = t >= d ? part[t - d] : (is_max ? -1 : 0);
    __syncthreads();
    part[t] = is_max ? max(part[t], y) : part[t] + y;
    __syncthreads();
  }
  return part[t];
}

__global__ __launch_bounds__(1024) void k_varlen_plan(const int* __restrict__ cu, int B, int T, int C, int* cs,
                                                      int* cl, int* co) {
  __shared__ int part[1024];
  const int t = threadIdx.x, nt = blockDim.x;
  // entries 0..B of cu: running maximum m_i, stored as the starts cs[i] (i < B)
  const int per = (B + 1 + nt - 1) / nt;
  const int i0 = min(B + 1, t * per), i1 = min(B + 1, i0 + per);
  int mx = -1;
  for (int i = i0; i < i1; ++i) mx = max(mx, min(max(cu[i], 0), T));
  const int incl = block_scan_incl(part, mx, true);
  int run = t > 0 ? part[t - 1] : -1;  // the maximum over the entries before this range
  (void)incl;
  __syncthreads();
  for (int i = i0; i < i1; ++i) {
    run = max(run, min(max(cu[i], 0), T));
    if (i < B) cs[i] = run;
    else part[0] = run;  // m_B (read after the next barrier)
  }
  __syncthreads();
  const int mB = part[0];
  __syncthreads();
  // lengths and chunk counts of this thread's sequences
  const int ps = (B + nt - 1) / nt;
  const int s0 = min(B, t * ps), s1 = min(B, s0 + ps);
  int nch = 0;
  for (int s = s0; s < s1; ++s) {
    const int len = (s + 1 < B ? cs[s + 1] : mB) - cs[s];
    cl[s] = len;
    nch += (len + C - 1) / C;
  }
  const int csum = block_scan_incl(part, nch, false);
  int off = csum - nch;
  for (int s = s0; s < s1; ++s) {
    co[s] = off;
    off += (cl[s] + C - 1) / C;
  }
  if (t == nt - 1) co[B] = csum;
}

int launch_varlen_plan(const int* cu, int B, int T, int C, const FwdWs& ws, void* stream) {
  LRT_LAUNCH(kKVarlenPlan, k_varlen_plan, dim3(1), dim3(1024), stream, cu, B, T, C, ws.cs, ws.cl, ws.co);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

// Gated DeltaNet: the chunk-parallel WY pass, then the serial scan (which
// also forms the output).  Mamba2: one fused kernel (no WY transform).
template <typename E, int C, int DK, int DV>
constexpr bool gdn_fwd_fits() {
  return WyLds<E, C, DK, DV>::TOTAL <= kLdsMax && scan_bv<E, C, DK, DV, kScanFwd, false>() > 0;
}

template <typename E, int C, int DK, int DV, bool FUSE>
int gdn_fwd_impl(const FwdArgs& a) {
  if constexpr (!gdn_fwd_fits<E, C, DK, DV>()) {
    return -3;  // not reached: the entry point runs a chunk that fits (fwd_max_chunk)
  } else {
    const bool packed = a.cu != nullptr;
    const int N = (a.T + C - 1) / C;
    const int tiles = (int)ws_tiles(a.B, a.T, a.H, C, packed);
    const FwdWs ws = fwd_ws_layout(LRT_OP_GDN_FWD, a.B, a.T, a.H, DK, DV, C, sizeof(E), a.workspace, packed);
    if (packed && launch_varlen_plan(a.cu, a.B, a.T, C, ws, a.stream) != 0) return -7;
    LRT_LAUNCH(kKWy, (k_wy<E, C, DK, DV, true, false, kWyWaves, FUSE>),
               dim3(persistent_grid(tiles, WyLds<E, C, DK, DV>::TOTAL)), dim3(64 * kWyWaves), a.stream,
               (const E*)a.q, (const E*)a.k, (const E*)a.v, a.log_a, a.beta, seq_map(a, ws, C), (E*)ws.W,
               (E*)ws.Up, ws.G, (E*)ws.P, (E*)nullptr);
    if (hipGetLastError() != hipSuccess) return -7;
    return launch_scan_fwd<E, C, DK, DV, false, false, FUSE>(a, ws, N);
  }
}

template <typename E, int C, int DK, int DV>
int fwd_impl(const FwdArgs& a) {
  if (a.variant == kVarSSD) return launch_ssd_fwd<E, C, DK, DV>(a);
  return a.fuse ? gdn_fwd_impl<E, C, DK, DV, true>(a) : gdn_fwd_impl<E, C, DK, DV, false>(a);
}

template <typename E, int DK, int DV>
constexpr int fwd_max_chunk_t() {
  return gdn_fwd_fits<E, 64, DK, DV>() ? 64 : gdn_fwd_fits<E, 32, DK, DV>() ? 32 : 16;
}

#define LRT_DV(DK_) LRT_CASE(DK_, 16) LRT_CASE(DK_, 32) LRT_CASE(DK_, 64) LRT_CASE(DK_, 128)
#define LRT_DK LRT_DV(16) LRT_DV(32) LRT_DV(64) LRT_DV(128)

int fwd_max_chunk(int dtype, int dk, int dv) {
#define LRT_CASE(DK_, DV_) \
  if (dk == DK_ && dv == DV_) return dtype == LRT_BF16 ? fwd_max_chunk_t<bf16, DK_, DV_>() : fwd_max_chunk_t<float, DK_, DV_>();
  LRT_DK
#undef LRT_CASE
  return 16;
}

template <typename E>
static int fwd_dtype(const FwdArgs& a) {
#define LRT_CASE(DK_, DV_)                                                   \
  if (a.dk == DK_ && a.dv == DV_) {                                          \
    if (a.chunk == 16) return fwd_impl<E, 16, DK_, DV_>(a);                  \
    if (a.chunk == 32) return fwd_impl<E, 32, DK_, DV_>(a);                  \
    if (a.chunk == 64) return fwd_impl<E, 64, DK_, DV_>(a);                  \
  }
  LRT_DK
#undef LRT_CASE
  return -2;
}
#undef LRT_DK
#undef LRT_DV

int fwd_scalar_gate(const FwdArgs& a) { return a.dtype == LRT_BF16 ? fwd_dtype<bf16>(a) : fwd_dtype<float>(a); }

}  // namespace lrt
