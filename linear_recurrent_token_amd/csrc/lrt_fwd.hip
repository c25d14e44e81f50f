// lrt_fwd.hip -- launchers of the chunkwise forward (gdn_fwd, ssd_fwd).
#include "lrt_fused_fwd.hpp"
#include "lrt_scan.hpp"
#include "lrt_ssd_fwd.hpp"
#include "lrt_fwd_kernels.hpp"
#include "lrt_internal.hpp"

namespace lrt {

// The GDN forward as the WY pass + serial scan (the backward's recompute
// path) instead of the single fused kernel.
constexpr bool kFwdSplit = true;

// --------------------------------------------------------------- launchers
template <typename E, int C, int DK, int DV>
int fwd_impl(const FwdArgs& a) {
  if (a.variant == kVarSSD) return launch_ssd_fwd<E, C, DK, DV>(a);
  constexpr int BVF = DV < 64 ? DV : 64;
  if constexpr (WyLds<E, C, DK, DV>::TOTAL <= 160 * 1024 && ScanLds<E, C, DK, BVF, kScanFwd, false>::TOTAL <= 160 * 1024) {
    if (kFwdSplit) {
      // chunk-parallel WY pass, then the serial scan
      const int N = (a.T + C - 1) / C;
      const int tiles = a.B * a.H * N;
      const FwdWs ws = fwd_ws_layout(a.B, a.T, a.H, DK, DV, C, sizeof(E), a.workspace);
      hipStream_t st = (hipStream_t)a.stream;
      LRT_LAUNCH(kKWy, (k_wy<E, C, DK, DV, true, false, kWyWaves>),
                 dim3(persistent_grid(tiles, WyLds<E, C, DK, DV>::TOTAL)), dim3(64 * kWyWaves), st,
                 (const E*)a.q, (const E*)a.k, (const E*)a.v, a.log_a, a.beta, a.T, a.H, N, tiles, (E*)ws.W,
                 (E*)ws.Up, ws.G, (E*)ws.P, (E*)nullptr);
      if (hipGetLastError() != hipSuccess) return -7;
      return launch_scan_fwd<E, C, DK, DV, false>(a, ws, N);
    }
  }
  if constexpr (FusedLds<E, C, DK, BVF>::TOTAL <= 160 * 1024) {
    // the whole forward in one kernel: state on chip, inputs read once
    const int N = (a.T + C - 1) / C;
    hipStream_t st = (hipStream_t)a.stream;
    const int grid = a.B * a.H * (DV / BVF);
    LRT_LAUNCH(kKFwd, (k_fwd<E, C, DK, BVF, kStateWaves>), dim3(grid), dim3(64 * kStateWaves), st,
               (const E*)a.q, (const E*)a.k, (const E*)a.v, a.log_a, a.beta, a.h0, a.ht, (E*)a.o, a.T, a.H, N, DV);
    return hipGetLastError() == hipSuccess ? 0 : -7;
  }
  const int N = (a.T + C - 1) / C;
  const int tiles = a.B * a.H * N;
  const FwdWs ws = fwd_ws_layout(a.B, a.T, a.H, DK, DV, C, sizeof(E), a.workspace);
  hipStream_t st = (hipStream_t)a.stream;
  LRT_LAUNCH(kKPrep, (k_prep<E, C, DK, DV, true>), dim3(persistent_grid(tiles, PrepLds<E, C, DK, DV, true>::TOTAL)), dim3(kThreads), st, (const E*)a.k,
                     (const E*)a.v, a.log_a, a.beta, a.T, a.H, N, tiles, (E*)ws.W, (E*)ws.Up, (E*)ws.Kt, ws.G, (E*)nullptr);
  constexpr int BV = DV < 64 ? DV : 64;  // state columns per workgroup
  const int sgrid = a.B * a.H * (DV / BV);
  LRT_LAUNCH(kKState, (k_state<E, C, DK, BV, true, false, kStateWaves>), dim3(sgrid), dim3(64 * kStateWaves), st, (const E*)ws.W,
                     (const E*)ws.Up, (const E*)ws.Kt, ws.G, (const float*)nullptr, a.h0, a.ht, (E*)ws.U, (E*)ws.S, N, DV);
  // fp32 operands need twice the LDS: split the value columns in blocks of 64
  constexpr int BVO = (sizeof(E) == 4 && DV > 64) ? 64 : DV;
  LRT_LAUNCH(kKOut, (k_out<E, C, DK, BVO>), dim3(persistent_grid(tiles * (DV / BVO), out_lds_bytes<E, C, DK, BVO, false>())), dim3(kThreads), st, (const E*)a.q,
                     (const E*)a.k, ws.G, (const E*)ws.S, (const E*)ws.U, (const E*)nullptr, (const E*)nullptr, (E*)a.o, a.T, a.H, N, DV, tiles * (DV / BVO));
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

template <typename E>
static int fwd_dtype(const FwdArgs& a) {
#define LRT_CASE(C_, DK_, DV_) \
  if (a.chunk == C_ && a.dk == DK_ && a.dv == DV_) return fwd_impl<E, C_, DK_, DV_>(a);
#define LRT_DV(C_, DK_) LRT_CASE(C_, DK_, 16) LRT_CASE(C_, DK_, 32) LRT_CASE(C_, DK_, 64) LRT_CASE(C_, DK_, 128)
#define LRT_DK(C_) LRT_DV(C_, 16) LRT_DV(C_, 32) LRT_DV(C_, 64) LRT_DV(C_, 128)
  LRT_DK(16) LRT_DK(32) LRT_DK(64)
#undef LRT_DK
#undef LRT_DV
#undef LRT_CASE
  return -2;
}

int fwd_scalar_gate(const FwdArgs& a) {
  return a.dtype == 1 ? fwd_dtype<bf16>(a) : fwd_dtype<float>(a);
}

}  // namespace lrt
