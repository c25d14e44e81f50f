// lrt_kda.hip -- chunkwise forward of Kimi Delta Attention on gfx950.
//
// KDA is Gated DeltaNet with one gate per key dimension (AMD ROCm blog
// "Pretraining hybrid LLMs with Primus", section "How hybrid models are
// defined in Primus", mixer list under Table 2).  With the state H = S^T:
//   H_t = (I - b_t k_t k_t^T) Diag(a_t) H_{t-1} + b_t k_t v_t^T,  o_t = H_t^T q_t.
// The chunk-parallel pass (k_kda_prep_fast and k_kda_prep, lrt_kda_prep.hpp) writes the WY
// factors and decayed operands per chunk; the serial scan in KDA mode
// (per-dimension decay, operands from the workspace) then carries the state
// and forms o.
#include <type_traits>

#include "lrt_internal.hpp"
#include "lrt_kda_prep.hpp"
#include "lrt_scan.hpp"

namespace lrt {

template <typename E, int C, int DK, int DV>
constexpr bool kda_fits() {
  return KdaLds<E, C, DK, DV, 64 * kWyWaves>::TOTAL <= kLdsMax && scan_bv<E, C, DK, DV, kScanFwd, true>() > 0;
}

template <typename E, int C, int DK, int DV, bool FUSE, bool LOWRANK = false>
int kda_impl_t(const FwdArgs& a) {
  if constexpr (!kda_fits<E, C, DK, DV>()) {
    return -3;  // not reached: the entry point runs a chunk that fits (kda_max_chunk)
  } else {
    const bool packed = a.cu != nullptr;
    const int N = (a.T + C - 1) / C;
    const int tiles = (int)ws_tiles(a.B, a.T, a.H, C, packed);
    const FwdWs ws = fwd_ws_layout(LRT_OP_KDA_FWD, a.B, a.T, a.H, DK, DV, C, sizeof(E), a.workspace, packed);
    hipStream_t st = (hipStream_t)a.stream;
    if (packed && launch_varlen_plan(a.cu, a.B, a.T, C, ws, a.stream) != 0) return -7;
    if (launch_kda_prep<E, C, DK, DV, FUSE, LOWRANK>(a.q, a.k, a.v, a.log_a, a.beta, seq_map(a, ws, C), ws,
                                                     (E*)nullptr, a.gate_up, tiles, kKKdaPrepFast, kKKdaPrep, st) != 0)
      return -7;
    return launch_scan_fwd<E, C, DK, DV, true>(a, ws, N);
  }
}
template <typename E, int C, int DK, int DV>
int kda_impl(const FwdArgs& a) {
  if (!a.fuse) return kda_impl_t<E, C, DK, DV, false>(a);
  return a.gate_up ? kda_impl_t<E, C, DK, DV, true, true>(a) : kda_impl_t<E, C, DK, DV, true>(a);
}

template <typename E, int DK, int DV>
constexpr int kda_max_chunk_t() {
  return kda_fits<E, 64, DK, DV>() ? 64 : kda_fits<E, 32, DK, DV>() ? 32 : 16;
}

#define LRT_DV(DK_) LRT_CASE(DK_, 16) LRT_CASE(DK_, 32) LRT_CASE(DK_, 64) LRT_CASE(DK_, 128)
#define LRT_DK LRT_DV(16) LRT_DV(32) LRT_DV(64) LRT_DV(128)

int kda_max_chunk(int dtype, int dk, int dv) {
#define LRT_CASE(DK_, DV_) \
  if (dk == DK_ && dv == DV_) return dtype == LRT_BF16 ? kda_max_chunk_t<bf16, DK_, DV_>() : kda_max_chunk_t<float, DK_, DV_>();
  LRT_DK
#undef LRT_CASE
  return 16;
}

template <typename E>
static int kda_dtype(const FwdArgs& a) {
#define LRT_CASE(DK_, DV_)                                   \
  if (a.dk == DK_ && a.dv == DV_) {                          \
    if (a.chunk == 16) return kda_impl<E, 16, DK_, DV_>(a);  \
    if (a.chunk == 32) return kda_impl<E, 32, DK_, DV_>(a);  \
    if (a.chunk == 64) return kda_impl<E, 64, DK_, DV_>(a);  \
  }
  LRT_DK
#undef LRT_CASE
  return -2;
}
#undef LRT_DK
#undef LRT_DV

int fwd_kda(const FwdArgs& a) { return a.dtype == LRT_BF16 ? kda_dtype<bf16>(a) : kda_dtype<float>(a); }

}  // namespace lrt
