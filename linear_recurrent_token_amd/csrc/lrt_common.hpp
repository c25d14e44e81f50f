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
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;

// LDS row padding (elements): 32 bytes keeps vector alignment and shifts
// consecutive rows by eight banks, so the four rows one transpose read
// touches fall in different banks (measured slightly faster than 16 bytes).
template <typename E>
constexpr int lds_pad() {
  return 32 / (int)sizeof(E);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, then s_barrier.  Unlike __syncthreads() it does not drain the
// wave's outstanding global loads and stores, so prefetched tiles stay in
// flight across it.  Every kernel here exchanges data between waves through
// LDS only.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Compiler-only ordering of one wave's LDS accesses: the LDS unit executes a
// wave's instructions in order, so a later access of the same wave (any lane)
// sees an earlier write once the compiler keeps the two in program order.
__device__ __forceinline__ void wave_order() { asm volatile("" ::: "memory"); }

// Instruction-scheduling fence: nothing moves across it, so the operand
// fragments of the products after it are not loaded early into registers
// (bounds register use where one wave computes several output tiles).
__device__ __forceinline__ void tile_fence() { __builtin_amdgcn_sched_barrier(0); }

// Reductions over the tokens of a chunk without atomics, so that repeated
// runs give bitwise-identical sums: every wave adds its terms into its own
// slot of NW x C partials (one lane per address per instruction, in program
// order), and after a workgroup barrier the slots of token t are added in
// wave order.
template <int NW, int C>
__device__ __forceinline__ void slot_zero(float* slots) {
  float* s = slots + wave_id() * C;
  for (int t = lane_id(); t < C; t += 64) s[t] = 0.f;
  wave_order();
}
template <int NW, int C>
__device__ __forceinline__ float slot_sum(const float* slots, int t) {
  float x = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) x += slots[w * C + t];
  return x;
}

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2.  Renumber them so that consecutive logical ids run on one XCD (when
// the grid divides evenly): work items that read the same data share a cache.
__device__ __forceinline__ int xcd_group(int bid, int nblocks) {
  if (nblocks % 8 != 0) return bid;
  return (bid % 8) * (nblocks / 8) + bid / 8;
}

// ------------------------------------------------------------ fused prologue
// The mixers' input activations, applied in the kernels' load stage by the
// *_fused entry points to the raw projections:
//   q, k  <- x / sqrt(sum x^2 + kL2Eps) per (token, head) row over d_k;
//   beta  <- sigmoid(z);   log a <- -softplus(z) = -(max(z, 0) + log(1 + e^-|z|))
// (the stable form).  They run on the hardware's base-2 exponential and
// logarithm, reciprocal and reciprocal square root (about 1 ulp each), whose
// arguments stay in range here: 1 + e^-|z| lies in [1, 2], a reciprocal of
// 1 + e^-z is 0 for an infinite argument, and a row's sum of squares plus
// kL2Eps is positive.
constexpr float kL2Eps = 1e-6f;
constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float hw_rsq(float x) { return __builtin_amdgcn_rsqf(x); }
__device__ __forceinline__ float sigmoid_f(float z) { return hw_rcp(1.f + hw_exp2(-z * kLog2e)); }
__device__ __forceinline__ float neg_softplus_f(float z) {
  return -(fmaxf(z, 0.f) + kLn2 * hw_log2(1.f + hw_exp2(-fabsf(z) * kLog2e)));
}

// x from another lane of the same 16-lane row, by a DPP control (VALU only).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
// Sum of x over aligned groups of G consecutive lanes (G a power of two up to
// 64), every lane of a group receiving its group's sum.  Inside a 16-lane row
// the partner values move by DPP: pairs (quad_perm 1,0,3,2), quads (2,3,0,1),
// the other quad of eight (mirror inside 8 lanes), the other half of the row
// (mirror inside 16 lanes), with no LDS traffic; wider groups add
// ds_bpermute steps.
template <int G>
__device__ __forceinline__ float lane_group_sum(float x) {
  static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "lane groups are powers of two");
  if constexpr (G >= 2) x += dpp_mov<0xB1>(x);
  if constexpr (G >= 4) x += dpp_mov<0x4E>(x);
  if constexpr (G >= 8) x += dpp_mov<0x141>(x);
  if constexpr (G >= 16) x += dpp_mov<0x140>(x);
  if constexpr (G >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (G >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

// ------------------------------------------------------------ sequence map
// Where the chunk tiles of the kernels lie.  Dense (cs == nullptr): B
// sequences of T tokens each, N = ceil(T / C) chunks, the tiles of (b, h) from
// (b H + h) N on.  Packed variable-length sequences (cs != nullptr): one
// [1, T, H, d] tensor holds B sequences, sequence s at tokens
// [cs[s], cs[s] + cl[s]) with co[s] chunks before it; its chunks never straddle
// a sequence boundary, and the tiles of (s, h) start at
// co[s] H + h ceil(cl[s] / C).  Workspace tiles stay chunk-major per (b, h),
// and states are indexed b H + h in both layouts.
struct SeqMap {
  const int* cs;  // packed: sequence starts [B] (clamped into [0, T]); nullptr when dense
  const int* cl;  // packed: sequence lengths [B]
  const int* co;  // packed: chunks before each sequence [B + 1]
  int T, H, C, N, B;
};
struct SeqPos {
  size_t tok0;   // the sequence's first token (its rows of a [.., H, d] tensor start at tok0 H + h)
  size_t tile0;  // workspace tile of its chunk 0
  int len, nch;  // tokens, chunks
  int h, bh;     // head; state index b H + h
};
__device__ __forceinline__ SeqPos seq_pos(const SeqMap& m, int bh) {
  SeqPos p;
  p.bh = bh;
  p.h = bh % m.H;
  const int b = bh / m.H;
  if (m.cs == nullptr) {
    p.tok0 = (size_t)b * m.T;
    p.len = m.T;
    p.nch = m.N;
    p.tile0 = (size_t)bh * m.N;
  } else {
    p.tok0 = (size_t)m.cs[b];
    p.len = m.cl[b];
    p.nch = (p.len + m.C - 1) / m.C;
    p.tile0 = (size_t)m.co[b] * m.H + (size_t)p.h * p.nch;
  }
  return p;
}
// The (sequence, head) and the chunk n of workspace tile `tile` (which must
// be below tile_count).
__device__ __forceinline__ SeqPos tile_pos(const SeqMap& m, int tile, int& n) {
  if (m.cs == nullptr) {
    n = tile % m.N;
    return seq_pos(m, tile / m.N);
  }
  // the last sequence whose first tile is <= tile (empty sequences own none)
  int lo = 0, hi = m.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (m.co[mid] * m.H <= tile) lo = mid;
    else hi = mid - 1;
  }
  const int nch = m.co[lo + 1] - m.co[lo];
  const int local = tile - m.co[lo] * m.H;
  n = local % nch;
  return seq_pos(m, lo * m.H + local / nch);
}
// Tiles in use: B H N (dense), or H times the chunks of all sequences (packed).
__device__ __forceinline__ int tile_count(const SeqMap& m) { return m.cs == nullptr ? m.B * m.H * m.N : m.co[m.B] * m.H; }

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
// acc(16x16) += A(16 x K) * B(K x 16) from LDS.  Each operand is stored either
//   "k-inner":  A(m, k) at a[m * lda + k],   B(k, n) at b[n * ldb + k]
//   "k-outer":  A(m, k) at a[k * lda + m],   B(k, n) at b[k * ldb + n]
// (template flags AK / BK select k-outer).  A k-inner fragment is one 16-byte
// LDS read per lane.  A k-outer bf16 fragment uses the gfx950 LDS transpose
// read (ds_read_b64_tr_b16): within each group of 16 lanes, lane j supplies
// the address of 4 consecutive elements of row j/4, columns 4*(j%4).., and
// lane r receives element r%4 of the rows supplied by lanes 4e + r/4
// (e = 0..3), i.e. 4 consecutive k of column r -- so operands laid out
// row-major by k feed the matrix cores without a transposed copy.
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ i16x4 lds_read_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const void*)p);
}

// 8 consecutive k (k0 + 8g .. k0 + 8g + 7, g = lane/16) of column n0 + lane%16
// of a k-outer bf16 operand.
__device__ __forceinline__ bf16x8 frag_k8_outer(const bf16* p, int ld, int k0, int n0) {
  const int l = lane_id(), g = l >> 4, j = l & 15;
  const bf16* src = p + (k0 + 8 * g + (j >> 2)) * ld + n0 + 4 * (j & 3);
  const i16x4 lo = lds_read_tr(src);
  const i16x4 hi = lds_read_tr(src + 4 * ld);
  const short __attribute__((ext_vector_type(8))) v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}
// A 16-long k range as the 16x16x32 operand: lane groups 0 and 1 carry
// k0 .. k0 + 15, groups 2 and 3 read the same rows and are zeroed.
__device__ __forceinline__ bf16x8 frag_k16_outer(const bf16* p, int ld, int k0) {
  const int l = lane_id(), g = l >> 4, j = l & 15;
  const bf16* src = p + (k0 + 8 * (g & 1) + (j >> 2)) * ld + 4 * (j & 3);
  const i16x4 lo = lds_read_tr(src);
  const i16x4 hi = lds_read_tr(src + 4 * ld);
  const short z = g < 2 ? (short)-1 : (short)0;
  const short __attribute__((ext_vector_type(8))) v = {(short)(lo[0] & z), (short)(lo[1] & z), (short)(lo[2] & z),
                                                       (short)(lo[3] & z), (short)(hi[0] & z), (short)(hi[1] & z),
                                                       (short)(hi[2] & z), (short)(hi[3] & z)};
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ bf16x8 frag_k16_inner(const bf16* p, int ld, int k0) {
  const int l = lane_id(), g = l >> 4;
  u32x4 x = *(const u32x4*)(p + (l & 15) * ld + k0 + 8 * (g & 1));
  const unsigned z = g < 2 ? ~0u : 0u;
  x &= u32x4{z, z, z, z};
  return __builtin_bit_cast(bf16x8, x);
}

template <int K, bool AK = false, bool BK = false>
__device__ __forceinline__ void mma(f32x4& acc, const bf16* a, int lda, const bf16* b, int ldb) {
  const int l = lane_id();
#pragma unroll
  for (int k = 0; k + 32 <= K; k += 32) {
    bf16x8 fa, fb;
    if constexpr (AK)
      fa = frag_k8_outer(a, lda, k, 0);
    else
      fa = *(const bf16x8*)(a + (l & 15) * lda + k + (l >> 4) * 8);
    if constexpr (BK)
      fb = frag_k8_outer(b, ldb, k, 0);
    else
      fb = *(const bf16x8*)(b + (l & 15) * ldb + k + (l >> 4) * 8);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc, 0, 0, 0);
  }
  if constexpr (K % 32 == 16) {
    // The 16-long tail also runs on the 16x16x32 instruction (half its lanes
    // zero): a 16x16x16 MFMA accumulating directly onto a 16x16x32 result
    // gave intermittently wrong sums on gfx950.
    constexpr int k = K - 16;
    const bf16x8 fa = AK ? frag_k16_outer(a, lda, k) : frag_k16_inner(a, lda, k);
    const bf16x8 fb = BK ? frag_k16_outer(b, ldb, k) : frag_k16_inner(b, ldb, k);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc, 0, 0, 0);
  }
}

// fp32 operands: 16x16x4 MFMA.  Lane group g = l/16 feeds k = 4g + s at step
// s, so a k-inner lane reads 4 consecutive k with one 16-byte load per 16 k;
// a k-outer lane reads them one by one (consecutive lanes, consecutive m/n).
template <int K, bool AK = false, bool BK = false>
__device__ __forceinline__ void mma(f32x4& acc, const float* a, int lda, const float* b, int ldb) {
  static_assert(K % 16 == 0, "fp32 contraction length must be a multiple of 16");
  const int l = lane_id(), g = l >> 4, j = l & 15;
#pragma unroll
  for (int k = 0; k < K; k += 16) {
    f32x4 va, vb;
    if constexpr (AK) {
#pragma unroll
      for (int s = 0; s < 4; ++s) va[s] = a[(k + 4 * g + s) * lda + j];
    } else {
      va = *(const f32x4*)(a + j * lda + k + 4 * g);
    }
    if constexpr (BK) {
#pragma unroll
      for (int s = 0; s < 4; ++s) vb[s] = b[(k + 4 * g + s) * ldb + j];
    } else {
      vb = *(const f32x4*)(b + j * ldb + k + 4 * g);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(va[0], vb[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(va[1], vb[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(va[2], vb[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(va[3], vb[3], acc, 0, 0, 0);
  }
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// NA tiles sharing their B operand: acc[s] += A_s (16 x K) B (K x 16) with
// A_s = a + s * astep.  B's fragment is read from LDS once per k step for all
// NA products (mma() per tile would read it NA times).
template <int K, int NA, bool AK = false, bool BK = false>
__device__ __forceinline__ void mma_nA(f32x4 (&acc)[NA], const bf16* a, int astep, int lda, const bf16* b,
                                       int ldb) {
  const int l = lane_id();
#pragma unroll
  for (int k = 0; k + 32 <= K; k += 32) {
    bf16x8 fb;
    if constexpr (BK)
      fb = frag_k8_outer(b, ldb, k, 0);
    else
      fb = *(const bf16x8*)(b + (l & 15) * ldb + k + (l >> 4) * 8);
#pragma unroll
    for (int s = 0; s < NA; ++s) {
      const bf16* as = a + s * astep;
      bf16x8 fa;
      if constexpr (AK)
        fa = frag_k8_outer(as, lda, k, 0);
      else
        fa = *(const bf16x8*)(as + (l & 15) * lda + k + (l >> 4) * 8);
      acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc[s], 0, 0, 0);
    }
  }
  if constexpr (K % 32 == 16) {
    constexpr int k = K - 16;
    const bf16x8 fb = BK ? frag_k16_outer(b, ldb, k) : frag_k16_inner(b, ldb, k);
#pragma unroll
    for (int s = 0; s < NA; ++s) {
      const bf16x8 fa = AK ? frag_k16_outer(a + s * astep, lda, k) : frag_k16_inner(a + s * astep, lda, k);
      acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc[s], 0, 0, 0);
    }
  }
}
template <int K, int NA, bool AK = false, bool BK = false>
__device__ __forceinline__ void mma_nA(f32x4 (&acc)[NA], const float* a, int astep, int lda, const float* b,
                                       int ldb) {
#pragma unroll
  for (int s = 0; s < NA; ++s) mma<K, AK, BK>(acc[s], a + s * astep, lda, b, ldb);
}
// NA tiles, each A_s times two B operands: acc1[s] += A_s B1 and
// acc2[s] += A_s B2, every fragment read once per k step (acc1 and acc2 may
// be the same array: the two products then interleave by k step).
template <int K, int NA, bool AK, bool B1K, bool B2K>
__device__ __forceinline__ void mma_nA2(f32x4 (&acc1)[NA], f32x4 (&acc2)[NA], const bf16* a, int astep, int lda,
                                        const bf16* b1, int ldb1, const bf16* b2, int ldb2) {
  const int l = lane_id();
#pragma unroll
  for (int k = 0; k + 32 <= K; k += 32) {
    const bf16x8 f1 = B1K ? frag_k8_outer(b1, ldb1, k, 0) : *(const bf16x8*)(b1 + (l & 15) * ldb1 + k + (l >> 4) * 8);
    const bf16x8 f2 = B2K ? frag_k8_outer(b2, ldb2, k, 0) : *(const bf16x8*)(b2 + (l & 15) * ldb2 + k + (l >> 4) * 8);
#pragma unroll
    for (int s = 0; s < NA; ++s) {
      const bf16* as = a + s * astep;
      const bf16x8 fa = AK ? frag_k8_outer(as, lda, k, 0) : *(const bf16x8*)(as + (l & 15) * lda + k + (l >> 4) * 8);
      acc1[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, f1, acc1[s], 0, 0, 0);
      acc2[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, f2, acc2[s], 0, 0, 0);
    }
  }
  if constexpr (K % 32 == 16) {
    constexpr int k = K - 16;
    const bf16x8 f1 = B1K ? frag_k16_outer(b1, ldb1, k) : frag_k16_inner(b1, ldb1, k);
    const bf16x8 f2 = B2K ? frag_k16_outer(b2, ldb2, k) : frag_k16_inner(b2, ldb2, k);
#pragma unroll
    for (int s = 0; s < NA; ++s) {
      const bf16x8 fa = AK ? frag_k16_outer(a + s * astep, lda, k) : frag_k16_inner(a + s * astep, lda, k);
      acc1[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, f1, acc1[s], 0, 0, 0);
      acc2[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, f2, acc2[s], 0, 0, 0);
    }
  }
}
template <int K, int NA, bool AK, bool B1K, bool B2K>
__device__ __forceinline__ void mma_nA2(f32x4 (&acc1)[NA], f32x4 (&acc2)[NA], const float* a, int astep, int lda,
                                        const float* b1, int ldb1, const float* b2, int ldb2) {
#pragma unroll
  for (int s = 0; s < NA; ++s) {
    mma<K, AK, B1K>(acc1[s], a + s * astep, lda, b1, ldb1);
    mma<K, AK, B2K>(acc2[s], a + s * astep, lda, b2, ldb2);
  }
}

// ------------------------------------------------------------- vector moves
// Four consecutive elements of E packed for one store / load.
template <typename E>
struct Vec4;
template <>
struct Vec4<float> {
  typedef f32x4 T;
  static __device__ __forceinline__ T pack(f32x4 x) { return x; }
  static __device__ __forceinline__ f32x4 unpack(T x) { return x; }
};
template <>
struct Vec4<bf16> {
  typedef u32x2 T;
  static __device__ __forceinline__ T pack(f32x4 x) {
    bf16 b0 = (bf16)x[0], b1 = (bf16)x[1], b2 = (bf16)x[2], b3 = (bf16)x[3];
    u32x2 r;
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
// The packed bits only: a prefetch that is unpacked where it is used does not
// make the load wait at the point of issue.
template <typename E>
__device__ __forceinline__ typename Vec4<E>::T load4_raw(const E* p) {
  return *(const typename Vec4<E>::T*)p;
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

// 16 bytes at element offset `off` of a global array, the byte offset formed
// in 32 bits (so a shared base pointer plus a 32-bit per-lane offset can be
// addressed without 64-bit vector arithmetic).
template <typename E>
__device__ __forceinline__ const u32x4* g16(const E* base, unsigned off) {
  return (const u32x4*)((const char*)base + off * (unsigned)sizeof(E));
}
template <typename E>
__device__ __forceinline__ u32x4* g16(E* base, unsigned off) {
  return (u32x4*)((char*)base + off * (unsigned)sizeof(E));
}

// An R x W tile of E moved global -> registers -> LDS in 16-byte pieces.
// Every load of a tile is issued before the first LDS store, so a thread
// keeps all its loads in flight at once (the loops unroll completely).
// Element offsets within a tile are 32-bit unsigned (the entry points
// require H * d < 2^24, so r * gs + c < 2^30): added to a base pointer the
// workgroup shares, they let the compiler address with a scalar base and a
// 32-bit vector offset instead of per-lane 64-bit arithmetic.
template <typename E, int R, int W, int NT = kThreads>
struct Tile {
  static constexpr int V = 16 / (int)sizeof(E);
  static constexpr int PR = W / V;  // pieces per row
  static constexpr int NP = R * PR;
  static constexpr int PT = (NP + NT - 1) / NT;
  u32x4 x[PT];

  // rows of a strided global array; rows >= nvalid read as zero
  __device__ __forceinline__ void load_rows(const E* g, size_t gs, int nvalid) {
#pragma unroll
    for (int s = 0; s < PT; ++s) {
      const int idx = threadIdx.x + NT * s;
      x[s] = u32x4{0u, 0u, 0u, 0u};
      if (NP % NT == 0 || idx < NP) {
        const int r = idx / PR, c = (idx % PR) * V;
        if (r < nvalid) x[s] = *g16(g, (unsigned)r * (unsigned)gs + (unsigned)c);
      }
    }
  }
  // as load_rows, but every lane loads (rows >= nvalid repeat row
  // nvalid - 1, nvalid >= 1): no branch around the loads, so a later wait
  // on an older load can count them; store_masked zeroes those rows
  __device__ __forceinline__ void load_rows_clamped(const E* g, size_t gs, int nvalid) {
#pragma unroll
    for (int s = 0; s < PT; ++s) {
      const int idx = threadIdx.x + NT * s;
      if (NP % NT == 0 || idx < NP) {
        const int r = idx / PR, c = (idx % PR) * V;
        x[s] = *g16(g, (unsigned)min(r, nvalid - 1) * (unsigned)gs + (unsigned)c);
      }
    }
  }
  // lds[r * ls + c], rows >= nvalid as zero
  __device__ __forceinline__ void store_masked(E* lds, int ls, int nvalid) const {
#pragma unroll
    for (int s = 0; s < PT; ++s) {
      const int idx = threadIdx.x + NT * s;
      if (NP % NT == 0 || idx < NP) {
        const int r = idx / PR, c = (idx % PR) * V;
        *(u32x4*)(lds + r * ls + c) = r < nvalid ? x[s] : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  // a dense, contiguous R x W block
  __device__ __forceinline__ void load_block(const E* g) {
#pragma unroll
    for (int s = 0; s < PT; ++s) {
      const int idx = threadIdx.x + NT * s;
      if (NP % NT == 0 || idx < NP) x[s] = *g16(g, (unsigned)idx * (unsigned)V);
    }
  }
  // Every row scaled to unit L2 norm, x / sqrt(sum_row x^2 + eps): the sum
  // in fp32 over the row's PR pieces, which sit on PR consecutive lanes
  // (butterfly over them), the result rounded back to E.  Rows of zeros
  // stay zero.
  __device__ __forceinline__ void normalize_rows(float eps) {
    static_assert(PR <= 64 && (PR & (PR - 1)) == 0, "a row's pieces must be a power-of-two lane group");
#pragma unroll
    for (int s = 0; s < PT; ++s) {
      E e[V];
      __builtin_memcpy(e, &x[s], 16);
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < V; ++i) ss += to_f(e[i]) * to_f(e[i]);
      ss = lane_group_sum<PR>(ss);
      const float sc = hw_rsq(ss + eps);
#pragma unroll
      for (int i = 0; i < V; ++i) e[i] = from_f<E>(to_f(e[i]) * sc);
      __builtin_memcpy(&x[s], e, 16);
    }
  }
  __device__ __forceinline__ void scale_rows(const float* rs) {
#pragma unroll
    for (int s = 0; s < PT; ++s) {
      const int idx = threadIdx.x + NT * s;
      if (NP % NT == 0 || idx < NP) x[s] = vec_scale<E>(x[s], rs[idx / PR]);
    }
  }
  // lds[r * ls + c]
  __device__ __forceinline__ void store(E* lds, int ls) const {
#pragma unroll
    for (int s = 0; s < PT; ++s) {
      const int idx = threadIdx.x + NT * s;
      if (NP % NT == 0 || idx < NP) {
        const int r = idx / PR, c = (idx % PR) * V;
        *(u32x4*)(lds + r * ls + c) = x[s];
      }
    }
  }
  // the R x W block back from lds[r * ls + c]
  __device__ __forceinline__ void load_lds(const E* lds, int ls) {
#pragma unroll
    for (int s = 0; s < PT; ++s) {
      const int idx = threadIdx.x + NT * s;
      if (NP % NT == 0 || idx < NP) {
        const int r = idx / PR, c = (idx % PR) * V;
        x[s] = *(const u32x4*)(lds + r * ls + c);
      }
    }
  }
  // rows [0, nvalid) to a strided global array
  __device__ __forceinline__ void store_rows(E* g, size_t gs, int nvalid) const {
#pragma unroll
    for (int s = 0; s < PT; ++s) {
      const int idx = threadIdx.x + NT * s;
      if (NP % NT == 0 || idx < NP) {
        const int r = idx / PR, c = (idx % PR) * V;
        if (r < nvalid) *g16(g, (unsigned)r * (unsigned)gs + (unsigned)c) = x[s];
      }
    }
  }
  // transposed: lds[c * ld + r]
  __device__ __forceinline__ void store_T(E* lds, int ld) const {
#pragma unroll
    for (int s = 0; s < PT; ++s) {
      const int idx = threadIdx.x + NT * s;
      if (NP % NT == 0 || idx < NP) {
        const int r = idx / PR, c = (idx % PR) * V;
        vec_to_lds_T<E>(lds, ld, r, c, x[s]);
      }
    }
  }
};

// Copy an R x W block from LDS (row stride ls) to a dense global block,
// 16 bytes per access, threads [0, NT).
template <typename E, int R, int W, int NT = kThreads>
__device__ __forceinline__ void lds_to_block(E* g, const E* lds, int ls) {
  constexpr int V = 16 / (int)sizeof(E), PR = W / V;
#pragma unroll
  for (int s = 0; s < (R * PR + NT - 1) / NT; ++s) {
    const int idx = threadIdx.x + NT * s;
    if ((R * PR) % NT == 0 || idx < R * PR) {
      const int r = idx / PR, c = (idx % PR) * V;
      *g16(g, (unsigned)r * (unsigned)W + (unsigned)c) = *(const u32x4*)(lds + r * ls + c);
    }
  }
}

// Accumulator-tile order: a matrix produced as 16x16 accumulator tiles of its
// transpose (tile (ta, tb) holds X^T rows 16ta.., cols 16tb..) is written
// lane-major -- each lane's 4 values at ((tile * 64 + lane) * 4) -- so one
// wave writes 64 contiguous 4-element pieces.  AccTiles rebuilds X
// row-major in LDS, X[16tb + l%16][16ta + 4(l/16) + r] = value r of lane l.
template <typename E>
__device__ __forceinline__ void acc_tile_store(E* base, int tile_id, f32x4 acc) {
  store4<E>((E*)((char*)base + ((unsigned)tile_id * 64u + (unsigned)lane_id()) * 4u * (unsigned)sizeof(E)), acc);
}
// load() issues the global loads into registers (packed, so nothing waits
// for them), store() writes X into LDS.
template <typename E, int NTA, int NTB, int NT = kThreads>
struct AccTiles {
  static constexpr int NS = NTA * NTB * 64;
  static constexpr int PT = (NS + NT - 1) / NT;
  typename Vec4<E>::T x[PT];
  __device__ __forceinline__ void load(const E* g) {
#pragma unroll
    for (int s = 0; s < PT; ++s) {
      const int p = min((int)threadIdx.x + NT * s, NS - 1);
      x[s] = load4_raw<E>((const E*)((const char*)g + (unsigned)p * 4u * (unsigned)sizeof(E)));
    }
  }
  __device__ __forceinline__ void store(E* lds, int ld) const {
#pragma unroll
    for (int s = 0; s < PT; ++s) {
      const int p = threadIdx.x + NT * s;
      if (NS % NT == 0 || p < NS) {
        const int tile = p >> 6, ln = p & 63;
        const int ta = tile / NTB, tb = tile % NTB;
        *(typename Vec4<E>::T*)(lds + (tb * 16 + (ln & 15)) * ld + ta * 16 + (ln >> 4) * 4) = x[s];
      }
    }
  }
};

// Copy R rows of W elements from LDS (row stride ls) to global rows (row
// stride gs), 16 bytes per access; rows >= nvalid are not written.
template <typename E, int R, int W, int NT = kThreads>
__device__ __forceinline__ void lds_to_rows(E* g, size_t gs, const E* lds, int ls, int nvalid) {
  constexpr int V = 16 / (int)sizeof(E), PR = W / V;
#pragma unroll
  for (int s = 0; s < (R * PR + NT - 1) / NT; ++s) {
    const int idx = threadIdx.x + NT * s;
    if ((R * PR) % NT == 0 || idx < R * PR) {
      const int r = idx / PR, c = (idx % PR) * V;
      if (r < nvalid) *g16(g, (unsigned)r * (unsigned)gs + (unsigned)c) = *(const u32x4*)(lds + r * ls + c);
    }
  }
}

// As lds_to_rows, but every thread stores (rows >= nvalid write row
// nvalid - 1 again, with its own value; nvalid >= 1): no branch around the
// stores, so the compiler's waits on older loads can count them exactly.
template <typename E, int R, int W, int NT = kThreads>
__device__ __forceinline__ void lds_to_rows_clamped(E* g, size_t gs, const E* lds, int ls, int nvalid) {
  constexpr int V = 16 / (int)sizeof(E), PR = W / V;
#pragma unroll
  for (int s = 0; s < (R * PR + NT - 1) / NT; ++s) {
    const int idx = threadIdx.x + NT * s;
    if ((R * PR) % NT == 0 || idx < R * PR) {
      const int r = min(idx / PR, nvalid - 1), c = (idx % PR) * V;
      *g16(g, (unsigned)r * (unsigned)gs + (unsigned)c) = *(const u32x4*)(lds + r * ls + c);
    }
  }
}

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
__device__ __forceinline__ float sum16(float x) { return lane_group_sum<16>(x); }
// Row sums of an accumulator tile: v[r] holds row 4 * (l / 16) + r of column
// l % 16.  Returns, in every lane, the sum over the 16 columns of row
// 4 * (l / 16) + ((l >> 2) & 3): halves of the row group trade rows (lane
// l ^ 8), then quarters (lane 7 - l within eight), then the quad sums.
__device__ __forceinline__ float rowsum4(f32x4 v) {
  const int l = lane_id();
  const bool hi = (l & 8) != 0, b2 = (l & 4) != 0;
  const float p0 = (hi ? v[2] : v[0]) + dpp_mov<0x128>(hi ? v[0] : v[2]);
  const float p1 = (hi ? v[3] : v[1]) + dpp_mov<0x128>(hi ? v[1] : v[3]);
  float q = (b2 ? p1 : p0) + dpp_mov<0x141>(b2 ? p0 : p1);
  q += dpp_mov<0xB1>(q);
  q += dpp_mov<0x4E>(q);
  return q;
}
// Sum over the 4 lanes sharing a column (lanes with equal l % 16).
__device__ __forceinline__ float sum4(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

// x moved across lanes by the DPP control CTRL (rows of 16 lanes outside
// ROW_MASK, and lanes whose source lies outside their row, read 0).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_or_zero(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}

// Inclusive prefix sum across the 64 lanes of a wave, in DPP moves (no LDS
// round trip): a Hillis-Steele scan inside each row of 16 lanes (row_shr 1,
// 2, 4, 8), then lane 15 of rows 0 and 2 added into rows 1 and 3
// (row_bcast:15) and lane 31 into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ float wave_incl_scan(float x) {
  x += dpp_or_zero<0x111>(x);
  x += dpp_or_zero<0x112>(x);
  x += dpp_or_zero<0x114>(x);
  x += dpp_or_zero<0x118>(x);
  x += dpp_or_zero<0x142, 0xa>(x);
  x += dpp_or_zero<0x143, 0xc>(x);
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
