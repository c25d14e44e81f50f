// lrt_fwd.hip -- launchers of the chunkwise forward (gdn_fwd, ssd_fwd).
#include "lrt_internal.hpp"
#include "lrt_scan.hpp"
#include "lrt_ssd_fwd.hpp"

namespace lrt {

// Gated DeltaNet: the chunk-parallel WY pass, then the serial scan (which
// also forms the output).  Mamba2: one fused kernel (no WY transform).
template <typename E, int C, int DK, int DV>
constexpr bool gdn_fwd_fits() {
  return WyLds<E, C, DK, DV>::TOTAL <= kLdsMax && scan_bv<E, C, DK, DV, kScanFwd, false>() > 0;
}

template <typename E, int C, int DK, int DV>
int fwd_impl(const FwdArgs& a) {
  if (a.variant == kVarSSD) return launch_ssd_fwd<E, C, DK, DV>(a);
  if constexpr (!gdn_fwd_fits<E, C, DK, DV>()) {
    return -3;  // not reached: the entry point runs a chunk that fits (fwd_max_chunk)
  } else {
    const int N = (a.T + C - 1) / C;
    const int tiles = a.B * a.H * N;
    const FwdWs ws = fwd_ws_layout(LRT_OP_GDN_FWD, a.B, a.T, a.H, DK, DV, C, sizeof(E), a.workspace);
    LRT_LAUNCH(kKWy, (k_wy<E, C, DK, DV, true, false, kWyWaves>),
               dim3(persistent_grid(tiles, WyLds<E, C, DK, DV>::TOTAL)), dim3(64 * kWyWaves), a.stream,
               (const E*)a.q, (const E*)a.k, (const E*)a.v, a.log_a, a.beta, a.T, a.H, N, tiles, (E*)ws.W,
               (E*)ws.Up, ws.G, (E*)ws.P, (E*)nullptr);
    if (hipGetLastError() != hipSuccess) return -7;
    return launch_scan_fwd<E, C, DK, DV, false>(a, ws, N);
  }
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
