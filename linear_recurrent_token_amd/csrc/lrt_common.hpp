// lrt_common.hpp -- device toolkit shared by the gfx950 kernels of liblrt.
//
// 16x16 output tiles on the matrix cores (MFMA), 64-wide wavefronts, 256-thread
// workgroups.  Every GEMM operand is staged in LDS with its contraction index
// contiguous, so each lane fetches its fragment with one 16-byte LDS read:
//   A element (m, k) at a[m * lda + k]      (row-major A)
//   B element (k, n) at bt[n * ldb + k]     (B stored transposed)
// Accumulator layout of a 16x16 fp32 tile (both MFMA shapes used here):
//   lane l holds rows 4*(l/16) + i, i = 0..3, of column l % 16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrt {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16 raw bytes in four VGPRs (a native vector, so register arrays of it stay in
// registers; HIP's uint4 is a class type)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;

// LDS row padding (elements): 16 bytes keeps vector alignment and shifts
// consecutive rows by four banks.
template <typename E>
constexpr int lds_pad() {
  return 16 / (int)sizeof(E);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }

template <typename E>
__device__ __forceinline__ E from_f(float x);
template <>
__device__ __forceinline__ float from_f<float>(float x) {
  return x;
}
// round to nearest even (hardware conversion on gfx950)
template <>
__device__ __forceinline__ bf16 from_f<bf16>(float x) {
  return (bf16)x;
}

// ---------------------------------------------------------------- MFMA tiles
// acc(16x16) += A(16 x K) * B(K x 16), operands in LDS as described above.
template <int K>
__device__ __forceinline__ void mma(f32x4& acc, const bf16* a, int lda, const bf16* bt, int ldb) {
  const int l = lane_id();
  const bf16* pa = a + (l & 15) * lda + (l >> 4) * 8;
  const bf16* pb = bt + (l & 15) * ldb + (l >> 4) * 8;
#pragma unroll
  for (int k = 0; k + 32 <= K; k += 32)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(pa + k), *(const bf16x8*)(pb + k),
                                                  acc, 0, 0, 0);
  if constexpr (K % 32 == 16) {
    const bf16* qa = a + (l & 15) * lda + (K - 16) + (l >> 4) * 4;
    const bf16* qb = bt + (l & 15) * ldb + (K - 16) + (l >> 4) * 4;
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(*(const i16x4*)qa, *(const i16x4*)qb, acc, 0, 0, 0);
  }
}

// fp32 operands: 16x16x4 MFMA.  Lane group g = l/16 feeds k = 4g + s at step
// s, so each lane reads 4 consecutive k with one 16-byte load per 16 k.
template <int K>
__device__ __forceinline__ void mma(f32x4& acc, const float* a, int lda, const float* bt, int ldb) {
  static_assert(K % 16 == 0, "fp32 contraction length must be a multiple of 16");
  const int l = lane_id();
  const float* pa = a + (l & 15) * lda + (l >> 4) * 4;
  const float* pb = bt + (l & 15) * ldb + (l >> 4) * 4;
#pragma unroll
  for (int k = 0; k < K; k += 16) {
    const f32x4 va = *(const f32x4*)(pa + k);
    const f32x4 vb = *(const f32x4*)(pb + k);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(va[0], vb[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(va[1], vb[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(va[2], vb[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(va[3], vb[3], acc, 0, 0, 0);
  }
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ------------------------------------------------------------- vector moves
// Four consecutive elements of E packed for one store / load.
template <typename E>
struct Vec4;
template <>
struct Vec4<float> {
  typedef float4 T;
  static __device__ __forceinline__ T pack(f32x4 x) { return make_float4(x[0], x[1], x[2], x[3]); }
  static __device__ __forceinline__ f32x4 unpack(T x) { return f32x4{x.x, x.y, x.z, x.w}; }
};
template <>
struct Vec4<bf16> {
  typedef uint2 T;
  static __device__ __forceinline__ T pack(f32x4 x) {
    bf16 b0 = (bf16)x[0], b1 = (bf16)x[1], b2 = (bf16)x[2], b3 = (bf16)x[3];
    uint2 r;
    r.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
    r.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
    return r;
  }
  static __device__ __forceinline__ f32x4 unpack(T x) {
    return f32x4{__builtin_bit_cast(float, x.x << 16), __builtin_bit_cast(float, x.x & 0xffff0000u),
                 __builtin_bit_cast(float, x.y << 16), __builtin_bit_cast(float, x.y & 0xffff0000u)};
  }
};

template <typename E>
__device__ __forceinline__ void store4(E* p, f32x4 x) {
  *(typename Vec4<E>::T*)p = Vec4<E>::pack(x);
}
template <typename E>
__device__ __forceinline__ f32x4 load4(const E* p) {
  return Vec4<E>::unpack(*(const typename Vec4<E>::T*)p);
}

// Scatter the 16 bytes x (elements c0.. of row r of a row-major source) into
// an LDS array stored transposed: lds[(c0 + e) * ld + r].
template <typename E>
__device__ __forceinline__ void vec_to_lds_T(E* lds, int ld, int r, int c0, u32x4 x) {
  constexpr int V = 16 / (int)sizeof(E);
  E e[V];
  __builtin_memcpy(e, &x, 16);
#pragma unroll
  for (int i = 0; i < V; ++i) lds[(c0 + i) * ld + r] = e[i];
}

// Elementwise scale of the 16 bytes x by s (in fp32, rounded back to E).
template <typename E>
__device__ __forceinline__ u32x4 vec_scale(u32x4 x, float s) {
  constexpr int V = 16 / (int)sizeof(E);
  E e[V];
  __builtin_memcpy(e, &x, 16);
#pragma unroll
  for (int i = 0; i < V; ++i) e[i] = from_f<E>(to_f(e[i]) * s);
  __builtin_memcpy(&x, e, 16);
  return x;
}

// An R x W tile of E moved global -> registers -> LDS in 16-byte pieces.
// Every load of a tile is issued before the first LDS store, so a thread
// keeps all its loads in flight at once (the loops unroll completely).
template <typename E, int R, int W>
struct Tile {
  static constexpr int V = 16 / (int)sizeof(E);
  static constexpr int PR = W / V;  // pieces per row
  static constexpr int NP = R * PR;
  static constexpr int PT = (NP + kThreads - 1) / kThreads;
  u32x4 x[PT];

  // rows of a strided global array; rows >= nvalid read as zero
  __device__ __forceinline__ void load_rows(const E* g, size_t gs, int nvalid) {
#pragma unroll
    for (int s = 0; s < PT; ++s) {
      const int idx = threadIdx.x + kThreads * s;
      x[s] = u32x4{0u, 0u, 0u, 0u};
      if (idx < NP) {
        const int r = idx / PR, c = (idx % PR) * V;
        if (r < nvalid) x[s] = *(const u32x4*)(g + (size_t)r * gs + c);
      }
    }
  }
  // a dense, contiguous R x W block
  __device__ __forceinline__ void load_block(const E* g) {
#pragma unroll
    for (int s = 0; s < PT; ++s) {
      const int idx = threadIdx.x + kThreads * s;
      if (idx < NP) x[s] = *(const u32x4*)(g + (size_t)idx * V);
    }
  }
  __device__ __forceinline__ void scale_rows(const float* rs) {
#pragma unroll
    for (int s = 0; s < PT; ++s) {
      const int idx = threadIdx.x + kThreads * s;
      if (idx < NP) x[s] = vec_scale<E>(x[s], rs[idx / PR]);
    }
  }
  // lds[r * ls + c]
  __device__ __forceinline__ void store(E* lds, int ls) const {
#pragma unroll
    for (int s = 0; s < PT; ++s) {
      const int idx = threadIdx.x + kThreads * s;
      if (idx < NP) {
        const int r = idx / PR, c = (idx % PR) * V;
        *(u32x4*)(lds + r * ls + c) = x[s];
      }
    }
  }
  // transposed: lds[c * ld + r]
  __device__ __forceinline__ void store_T(E* lds, int ld) const {
#pragma unroll
    for (int s = 0; s < PT; ++s) {
      const int idx = threadIdx.x + kThreads * s;
      if (idx < NP) {
        const int r = idx / PR, c = (idx % PR) * V;
        vec_to_lds_T<E>(lds, ld, r, c, x[s]);
      }
    }
  }
};

// Copy R rows of W elements from global (row stride gs elements) into LDS
// (row stride ls); rows >= nvalid become zero.
template <typename E, int R, int W>
__device__ __forceinline__ void rows_to_lds(E* lds, int ls, const E* g, size_t gs, int nvalid) {
  Tile<E, R, W> t;
  t.load_rows(g, gs, nvalid);
  t.store(lds, ls);
}

// Copy a dense block of R x W elements (contiguous in global) into LDS.
template <typename E, int R, int W>
__device__ __forceinline__ void block_to_lds(E* lds, int ls, const E* g) {
  Tile<E, R, W> t;
  t.load_block(g);
  t.store(lds, ls);
}

// Sum over the 16 lanes of a row group (lanes with equal l / 16).
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 4, 64);
  x += __shfl_xor(x, 8, 64);
  return x;
}
// Sum over the 4 lanes sharing a column (lanes with equal l % 16).
__device__ __forceinline__ float sum4(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ float wave_incl_scan(float x) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float y = __shfl_up(x, d, 64);
    if (l >= d) x += y;
  }
  return x;
}

// Inclusive suffix sum across the 64 lanes of a wave.
__device__ __forceinline__ float wave_incl_suffix(float x) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float y = __shfl_down(x, d, 64);
    if (l + d < 64) x += y;
  }
  return x;
}

}  // namespace lrt
