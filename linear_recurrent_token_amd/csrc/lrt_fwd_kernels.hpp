// lrt_fwd_kernels.hpp -- the triangular solve of the chunkwise gated
// delta-rule mixers on gfx950.
//
// Inside a chunk of C tokens (state H = S^T, [d_k, d_v]; the recurrences of
// the mixers on the AMD ROCm blog "Pretraining hybrid LLMs with Primus",
// section "How hybrid models are defined in Primus", mixer list under
// Table 2), the WY/UT form needs Tinv = (I + A)^-1 for the strictly lower
// triangular A = strict_lower(diag(b) (K K^T) o Gamma) (KDA: the
// per-dimension gated K K^T).  unit_lower_inverse computes it in LDS.
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

}  // namespace lrt
