// lrt_conv_norm.hip -- the two steps either side of the mixer as single-pass
// kernels on gfx950: the short causal convolution (+ SiLU) on its q/k/v
// inputs and the gated RMSNorm on its output, forward and backward.
//
// The pretraining recipe of the AMD ROCm blog "Pretraining hybrid LLMs with
// Primus" ("Recipe", Table 4, FLA fusion row) replaces the element-wise short
// conv and gated-norm paths by fused kernels, and fixes the norm epsilon at
// 1e-6 (epsilon row).  Definitions (the pages name the steps only):
//   short conv   pre[t, c] = sum_j w[c, j] x[t - (W - 1) + j, c] over the
//                tokens of t's sequence (earlier tokens count as zero),
//                y = pre * sigmoid(pre);
//   gated norm   y = o / sqrt(mean(o^2) + eps) * w * silu(z) per row of d.
// Both are HBM-bound streams: every input element is read once and every
// output element written once (the convolution re-reads the W - 1 rows before
// each 16-token block, from cache); consecutive lanes take consecutive pieces
// of a row.  The weight gradients are summed per
// workgroup in a fixed order, then over workgroups in a second small pass, so
// repeated calls give bitwise-identical results.
#include <type_traits>

#include "lrt_internal.hpp"

namespace lrt {

namespace {

constexpr int kConvGroups = 64; // range groups (workgroups per piece group; the backward's dw partials)
constexpr int kNormBlocks = 1024;  // workgroups of the norm backward (its dw partials)

__device__ __forceinline__ float silu_f(float p) { return p * sigmoid_f(p); }
// d silu / dp = s (1 + p (1 - s)), s = sigmoid(p)
__device__ __forceinline__ float dsilu_f(float p) {
  const float s = sigmoid_f(p);
  return s * (1.f + p * (1.f - s));
}

template <typename E>
__device__ __forceinline__ void piece_load(const E* p, float* x) {
  constexpr int V = 16 / (int)sizeof(E);
  const u32x4 r = *(const u32x4*)p;
  E e[V];
  __builtin_memcpy(e, &r, 16);
#pragma unroll
  for (int i = 0; i < V; ++i) x[i] = to_f(e[i]);
}
template <typename E>
__device__ __forceinline__ void piece_store(E* p, const float* x) {
  constexpr int V = 16 / (int)sizeof(E);
  E e[V];
#pragma unroll
  for (int i = 0; i < V; ++i) e[i] = from_f<E>(x[i]);
  u32x4 r;
  __builtin_memcpy(&r, e, 16);
  *(u32x4*)p = r;
}

// Sequence bounds of token t: [s0, s1) with s0 <= t < s1 <= ntok.  Dense
// (cu == nullptr): sequences of T tokens.  Packed: the last boundary cu[s] <= t
// among cu[0..n-1] (binary search) and the next one, clamped into range so
// that malformed tables cannot move an access outside the tensor.
__device__ __forceinline__ void seq_bounds(const int* cu, int n, int T, int ntok, int t, int& s0, int& s1) {
  if (cu == nullptr) {
    s0 = (t / T) * T;
    s1 = s0 + T;
    return;
  }
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t)
      lo = mid;
    else
      hi = mid - 1;
  }
  s0 = min(max(cu[lo], 0), t);
  s1 = max(min(cu[lo + 1], ntok), t + 1);
}

// Both convolution kernels: four channels per lane (8-byte bf16 / 16-byte
// fp32 pieces: a wave covers 256 consecutive channels of a row); grid (piece
// groups of 64, range groups); wave w of workgroup (gx, gy) walks the tokens
// [r0, r1) of range q = gy * 4 + w in order, kConvCB rows at a time (issued
// together, clamped addresses, zero selected outside the range), carrying
// the last W - 1 rows of x (and, backward, the last W values of g) from one
// chunk to the next, so only a range's first W - 1 rows (and, backward, the
// W - 1 after it) are read twice.  A chunk whose window holds a sequence
// boundary takes each token's own sequence bounds and masks (edge path).
constexpr int kConvCB = 8;  // rows per chunk

// tokens per range: the ranges of one piece group cover ntok
__device__ __forceinline__ int conv_range(int ntok, int nranges) {
  const int r = (ntok + nranges - 1) / nranges;
  return (r + kConvCB - 1) / kConvCB * kConvCB;
}

// ------------------------------------------------------------ k_conv_fwd
template <typename E, int W>
__global__ __launch_bounds__(256) void k_conv_fwd(const E* __restrict__ x, const float* __restrict__ w,
                                                  E* __restrict__ y, const int* __restrict__ cu, int n, int T,
                                                  int ntok, int D) {
  typedef typename Vec4<E>::T Raw;
  const int P = D / 4, p = blockIdx.x * 64 + lane_id();
  const int RL = conv_range(ntok, 4 * gridDim.y);
  const int r0 = (blockIdx.y * 4 + wave_id()) * RL, r1 = min(r0 + RL, ntok);
  if (p >= P || r0 >= ntok) return;
  f32x4 wv[W], xw[W];
#pragma unroll
  for (int j = 0; j < W; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) wv[j][e] = w[(size_t)(p * 4 + e) * W + j];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) {
    const int t = r0 - (W - 1) + j;
    const f32x4 r = load4<E>(x + (size_t)max(t, 0) * D + p * 4);
    xw[j] = t >= 0 ? r : zero4();
  }
  auto load_chunk = [&](Raw(&raw)[kConvCB], int c0) {
#pragma unroll
    for (int i = 0; i < kConvCB; ++i) {
      const int t = c0 + i;
      const Raw r = load4_raw<E>(x + (size_t)min(t, ntok - 1) * D + p * 4);
      raw[i] = t < r1 ? r : Vec4<E>::pack(zero4());
    }
  };
  auto do_chunk = [&](const Raw(&raw)[kConvCB], int c0) {
    int s0, s1;
    seq_bounds(cu, n, T, ntok, c0, s0, s1);
    const bool edge = s0 > c0 - (W - 1) || s1 < min(c0 + kConvCB, ntok);  // wave-uniform
#pragma unroll
    for (int i = 0; i < kConvCB; ++i) {
      const int t = c0 + i;
      xw[W - 1] = Vec4<E>::unpack(raw[i]);
      if (t < r1) {
        int a = s0;  // first token of t's sequence
        if (edge) {
          int b_;
          seq_bounds(cu, n, T, ntok, t, a, b_);
        }
        f32x4 pre = zero4();
#pragma unroll
        for (int j = 0; j < W; ++j)
          if (!edge || t - (W - 1) + j >= a) pre += wv[j] * xw[j];
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = silu_f(pre[e]);
        store4<E>(y + (size_t)t * D + p * 4, o);
      }
#pragma unroll
      for (int j = 0; j < W - 1; ++j) xw[j] = xw[j + 1];
    }
  };
  for (int c0 = r0; c0 < r1; c0 += kConvCB) {
    Raw raw[kConvCB];
    load_chunk(raw, c0);
    do_chunk(raw, c0);
  }
}

// ------------------------------------------------------------ k_conv_bwd
// Rolling over t' = r0 .. r1 + W - 2 (the W - 1 rows after the range are the
// look-ahead its last dx rows need):
//   g[t'] = dy[t'] silu'(pre[t']),
//   dx[t] = sum_m w[W - 1 - m] g[t + m]  for t = t' - (W - 1) in [r0, r1),
//           t + m inside t's sequence,
//   dw[j] += g[t'] x[t' - (W - 1) + j]   for t' in [r0, r1), taps inside t''s
//           sequence,
// dw summed in registers over the range, then over the four waves in LDS,
// into partial[gridDim.y][D][W] for k_rows_reduce.
template <typename E, int W>
__global__ __launch_bounds__(256) void k_conv_bwd(const E* __restrict__ x, const float* __restrict__ w,
                                                  const E* __restrict__ dy, E* __restrict__ dx,
                                                  float* __restrict__ partial, const int* __restrict__ cu, int n,
                                                  int T, int ntok, int D) {
  typedef typename Vec4<E>::T Raw;
  __shared__ float sdw[4][64][4 * W];
  const int P = D / 4, p = blockIdx.x * 64 + lane_id(), wv_ = wave_id();
  const bool active = p < P;
  const int pc = active ? p : 0;  // inactive lanes read piece 0 and write nothing
  const int RL = conv_range(ntok, 4 * gridDim.y);
  const int r0 = (blockIdx.y * 4 + wv_) * RL, r1 = min(r0 + RL, ntok), lim = min(r1 + W - 1, ntok);
  f32x4 wv[W], dwa[W], xw[W], gh[W];
#pragma unroll
  for (int j = 0; j < W; ++j) {
#pragma unroll
    for (int e = 0; e < 4; ++e) wv[j][e] = w[(size_t)(pc * 4 + e) * W + j];
    dwa[j] = zero4();
    gh[j] = zero4();
  }
  if (r0 < ntok) {
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
      const int t = r0 - (W - 1) + j;
      const f32x4 r = load4<E>(x + (size_t)max(t, 0) * D + pc * 4);
      xw[j] = t >= 0 ? r : zero4();
    }
  }
  const int end = r1 + W - 1;  // the last chunk covers the look-ahead rows
  auto load_chunk = [&](Raw(&xr)[kConvCB], Raw(&dr)[kConvCB], int c0) {
#pragma unroll
    for (int i = 0; i < kConvCB; ++i) {
      const int t = c0 + i;
      const size_t off = (size_t)min(t, ntok - 1) * D + pc * 4;
      const Raw a = load4_raw<E>(x + off), b = load4_raw<E>(dy + off);
      xr[i] = t < lim ? a : Vec4<E>::pack(zero4());
      dr[i] = t < lim ? b : Vec4<E>::pack(zero4());
    }
  };
  auto do_chunk = [&](const Raw(&xr)[kConvCB], const Raw(&dr)[kConvCB], int c0) {
    int s0, s1;
    seq_bounds(cu, n, T, ntok, min(c0, ntok - 1), s0, s1);
    // wave-uniform: a boundary inside the chunk's window [c0 - (W - 1), c0 + kConvCB)
    const bool edge = s0 > c0 - (W - 1) || s1 < min(c0 + kConvCB, ntok);
#pragma unroll
    for (int i = 0; i < kConvCB; ++i) {
      const int tp = c0 + i;
      xw[W - 1] = Vec4<E>::unpack(xr[i]);
      const f32x4 dv = Vec4<E>::unpack(dr[i]);
      int a = s0;
      if (edge && tp < ntok) {
        int b_;
        seq_bounds(cu, n, T, ntok, tp, a, b_);
      }
      f32x4 pre = zero4();
#pragma unroll
      for (int j = 0; j < W; ++j)
        if (!edge || tp - (W - 1) + j >= a) pre += wv[j] * xw[j];
      f32x4 g;
#pragma unroll
      for (int e = 0; e < 4; ++e) g[e] = dv[e] * dsilu_f(pre[e]);
      if (tp < r1) {
#pragma unroll
        for (int j = 0; j < W; ++j)
          if (!edge || tp - (W - 1) + j >= a) dwa[j] += g * xw[j];
      }
#pragma unroll
      for (int m = 0; m < W - 1; ++m) gh[m] = gh[m + 1];
      gh[W - 1] = g;  // gh[m] = g[tp - (W - 1) + m]
      const int t = tp - (W - 1);
      if (t >= r0 && t < r1 && active) {
        int b = s1;  // end of t's sequence
        if (edge) {
          int a_;
          seq_bounds(cu, n, T, ntok, t, a_, b);
        }
        f32x4 o = zero4();
#pragma unroll
        for (int m = 0; m < W; ++m)
          if (!edge || t + m < b) o += wv[W - 1 - m] * gh[m];
        store4<E>(dx + (size_t)t * D + p * 4, o);
      }
#pragma unroll
      for (int j = 0; j < W - 1; ++j) xw[j] = xw[j + 1];
    }
  };
  for (int c0 = r0; r0 < ntok && c0 < end; c0 += kConvCB) {
    Raw xr[kConvCB], dr[kConvCB];
    load_chunk(xr, dr, c0);
    do_chunk(xr, dr, c0);
  }
  // the four waves' dw sums of this workgroup's pieces, added in wave order
#pragma unroll
  for (int j = 0; j < W; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) sdw[wv_][lane_id()][e * W + j] = dwa[j][e];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 64 * 4 * W; idx += 256) {
    const int l = idx / (4 * W), k = idx % (4 * W);
    const int pp = blockIdx.x * 64 + l;
    if (pp < P) {
      const float s = ((sdw[0][l][k] + sdw[1][l][k]) + sdw[2][l][k]) + sdw[3][l][k];
      partial[((size_t)blockIdx.y * D + pp * 4) * W + k] = s;  // [gy][channel pp * 4 + e][tap j], k = e * W + j
    }
  }
}

// out[i] = sum over n partial rows of partial[row][i], i < n_cols: lane l of
// workgroup bx takes column bx * 64 + l (coalesced rows), wave w the rows
// [w n / NWR, (w + 1) n / NWR) in order, 16 loads in flight per step; the NWR
// wave sums are then added in wave order.  Fixed order throughout: repeated
// calls are bitwise equal.
template <int NWR>
__global__ __launch_bounds__(64 * NWR) void k_rows_reduce(const float* __restrict__ partial, float* __restrict__ out,
                                                          int n, int n_cols) {
  __shared__ float ssum[NWR][64];
  const int c = blockIdx.x * 64 + lane_id(), w = wave_id();
  const int r0 = (int)((long long)w * n / NWR), r1 = (int)((long long)(w + 1) * n / NWR);
  float s = 0.f;
  if (c < n_cols) {
    int r = r0;
    for (; r + 16 <= r1; r += 16) {
      float v[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = partial[(size_t)(r + k) * n_cols + c];
#pragma unroll
      for (int k = 0; k < 16; ++k) s += v[k];
    }
    for (; r < r1; ++r) s += partial[(size_t)r * n_cols + c];
  }
  ssum[w][lane_id()] = s;
  __syncthreads();
  if (w == 0 && c < n_cols) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < NWR; ++k) t += ssum[k][lane_id()];
    out[c] = t;
  }
}
constexpr int kReduceWaves = 16;

// ------------------------------------------------------------ gated norm
// G = d / V lanes per row (a power of two dividing 64): a row's sums run over
// its G lanes (lane_group_sum).  A thread keeps one piece index
// (threadIdx.x % G) for every row it visits, so its w piece loads once.
template <typename E, int G>
__global__ __launch_bounds__(256) void k_gnorm_fwd(const E* __restrict__ o, const E* __restrict__ z,
                                                   const float* __restrict__ w, E* __restrict__ y, int rows, int d,
                                                   float eps) {
  constexpr int V = 16 / (int)sizeof(E), per = 256 / G;
  const int pc = threadIdx.x % G;
  const float inv_d = 1.f / (float)d;
  float wv[V];
#pragma unroll
  for (int e = 0; e < V; ++e) wv[e] = w[pc * V + e];
  for (int r = blockIdx.x * per + threadIdx.x / G; r < rows; r += gridDim.x * per) {
    const size_t off = (size_t)r * d + pc * V;
    float ov[V], zv[V], out[V];
    piece_load<E>(o + off, ov);
    piece_load<E>(z + off, zv);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < V; ++e) ss += ov[e] * ov[e];
    const float rstd = hw_rsq(lane_group_sum<G>(ss) * inv_d + eps);
#pragma unroll
    for (int e = 0; e < V; ++e) out[e] = ov[e] * rstd * wv[e] * silu_f(zv[e]);
    piece_store<E>(y + off, out);
  }
}

// do = r (dn - n mean(dn n)), dn = dy w silu(z); dz = dy n w silu'(z);
// dw partial per workgroup: sum over its rows of dy n silu(z), the row slots
// added in slot order.
template <typename E, int G>
__global__ __launch_bounds__(256) void k_gnorm_bwd(const E* __restrict__ o, const E* __restrict__ z,
                                                   const float* __restrict__ w, const E* __restrict__ dy,
                                                   E* __restrict__ dout, E* __restrict__ dz,
                                                   float* __restrict__ partial, int rows, int d, float eps) {
  constexpr int V = 16 / (int)sizeof(E), per = 256 / G;
  __shared__ float sdw[256][V];
  const int pc = threadIdx.x % G;
  const float inv_d = 1.f / (float)d;
  float wv[V], dwa[V];
#pragma unroll
  for (int e = 0; e < V; ++e) {
    wv[e] = w[pc * V + e];
    dwa[e] = 0.f;
  }
  for (int r = blockIdx.x * per + threadIdx.x / G; r < rows; r += gridDim.x * per) {
    const size_t off = (size_t)r * d + pc * V;
    float ov[V], zv[V], gv[V];
    piece_load<E>(o + off, ov);
    piece_load<E>(z + off, zv);
    piece_load<E>(dy + off, gv);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < V; ++e) ss += ov[e] * ov[e];
    const float rstd = hw_rsq(lane_group_sum<G>(ss) * inv_d + eps);
    float n[V], dn[V], dzv[V], dot = 0.f;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      n[e] = ov[e] * rstd;
      const float s = sigmoid_f(zv[e]), sz = zv[e] * s;
      dn[e] = gv[e] * wv[e] * sz;
      dzv[e] = gv[e] * n[e] * wv[e] * (s * (1.f + zv[e] * (1.f - s)));
      dwa[e] += gv[e] * n[e] * sz;
      dot += dn[e] * n[e];
    }
    const float mdot = lane_group_sum<G>(dot) * inv_d;
    float dov[V];
#pragma unroll
    for (int e = 0; e < V; ++e) dov[e] = rstd * (dn[e] - n[e] * mdot);
    piece_store<E>(dout + off, dov);
    piece_store<E>(dz + off, dzv);
  }
#pragma unroll
  for (int e = 0; e < V; ++e) sdw[threadIdx.x][e] = dwa[e];
  __syncthreads();
  for (int c = threadIdx.x; c < d; c += 256) {
    const int pp = c / V, e = c % V;
    float s = 0.f;
    for (int slot = 0; slot < per; ++slot) s += sdw[slot * G + pp][e];
    partial[(size_t)blockIdx.x * d + c] = s;
  }
}


// launch shapes (range groups of four waves): the forward takes ranges down
// to 32 rows, up to 256 groups; the backward at most kConvGroups (its dw
// partials), ranges of at least 16 rows
int conv_groups_fwd(int ntok) { return max(1, min((ntok + 127) / 128, 256)); }
int conv_groups(int ntok) { return max(1, min((ntok + 63) / 64, kConvGroups)); }
int gnorm_blocks(long long rows, int d, int esz) {
  const int per = 256 / (d / (16 / esz));
  const long long nb = (rows + per - 1) / per;
  return (int)(nb < 1 ? 1 : nb > kNormBlocks ? kNormBlocks : nb);
}

// the norm kernels at G = d / V lanes per row
template <typename E>
void gnorm_fwd_t(const void* o, const void* z, const float* w, void* y, int rows, int d, float eps, int nb,
                 hipStream_t st) {
  constexpr int V = 16 / (int)sizeof(E);
#define LRT_GN(G_)                                                                                         \
  if (d / V == G_)                                                                                         \
    LRT_LAUNCH(kKNormFwd, (k_gnorm_fwd<E, G_>), dim3(nb), dim3(256), st, (const E*)o, (const E*)z, w, (E*)y, \
               rows, d, eps);
  LRT_GN(2) LRT_GN(4) LRT_GN(8) LRT_GN(16) LRT_GN(32) LRT_GN(64)
#undef LRT_GN
}
template <typename E>
void gnorm_bwd_t(const void* o, const void* z, const float* w, const void* dy, void* d_o, void* dz, float* partial,
                 int rows, int d, float eps, int nb, hipStream_t st) {
  constexpr int V = 16 / (int)sizeof(E);
#define LRT_GN(G_)                                                                                             \
  if (d / V == G_)                                                                                             \
    LRT_LAUNCH(kKNormBwd, (k_gnorm_bwd<E, G_>), dim3(nb), dim3(256), st, (const E*)o, (const E*)z, w,           \
               (const E*)dy, (E*)d_o, (E*)dz, partial, rows, d, eps);
  LRT_GN(2) LRT_GN(4) LRT_GN(8) LRT_GN(16) LRT_GN(32) LRT_GN(64)
#undef LRT_GN
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4b(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// Shapes, dtype, x and w; a and b are further token tensors (alignment only).
int conv_check(const void* x, const float* w, const void* a, const void* b, const int* cu, int n_seq, int T, int D,
               int W, int dtype, long long& ntok) {
  if (dtype != LRT_F32 && dtype != LRT_BF16) return LRT_ERR_DTYPE;
  if (n_seq < 1 || T < 0 || D < 8 || D % 8 != 0 || D >= (1 << 24) || W < 2 || W > 4) return LRT_ERR_SHAPE;
  ntok = cu != nullptr ? (long long)T : (long long)n_seq * T;
  if (ntok > 0x7fffffffLL) return LRT_ERR_SHAPE;
  if (!w || (ntok > 0 && !x)) return LRT_ERR_NULL;
  const void* vec[] = {x, a, b};
  for (const void* q : vec)
    if (q && !aligned16(q)) return LRT_ERR_ALIGN;
  if (!aligned4b(w) || (cu && !aligned4b(cu))) return LRT_ERR_ALIGN;
  return LRT_OK;
}

template <typename E, int W>
void conv_fwd_t(const void* x, const float* w, void* y, const int* cu, int n, int T, int ntok, int D,
                hipStream_t st) {
  const int P = D / 4;
  LRT_LAUNCH(kKConvFwd, (k_conv_fwd<E, W>), dim3((P + 63) / 64, conv_groups_fwd(ntok)), dim3(256), st,
             (const E*)x, w, (E*)y, cu, n, T, ntok, D);
}
template <typename E, int W>
void conv_bwd_t(const void* x, const float* w, const void* dy, void* dx, float* dw, float* partial, const int* cu,
                int n, int T, int ntok, int D, hipStream_t st) {
  const int P = D / 4, ng = conv_groups(ntok);
  LRT_LAUNCH(kKConvBwd, (k_conv_bwd<E, W>), dim3((P + 63) / 64, ng), dim3(256), st, (const E*)x, w,
             (const E*)dy, (E*)dx, partial, cu, n, T, ntok, D);
  LRT_LAUNCH(kKConvDw, k_rows_reduce<kReduceWaves>, dim3((D * W + 63) / 64), dim3(64 * kReduceWaves), st,
             (const float*)partial, dw, ng, D * W);
}

}  // namespace

}  // namespace lrt

using namespace lrt;

extern "C" {

size_t short_conv_bwd_workspace_bytes(long long n_tokens, int D, int W) {
  if (n_tokens < 0 || n_tokens > 0x7fffffffLL || D < 8 || D % 8 != 0 || D >= (1 << 24) || W < 2 || W > 4)
    return (size_t)-1;
  // the partial sums of at most kConvGroups range groups
  return (size_t)kConvGroups * D * W * sizeof(float);
}

int short_conv_fwd(const void* x, const float* w, void* y, const int* cu_seqlens, int n_seq, int T, int D, int W,
                   int dtype, void* stream) {
  long long ntok = 0;
  int rc = conv_check(x, w, y, nullptr, cu_seqlens, n_seq, T, D, W, dtype, ntok);
  if (rc) return rc;
  if (ntok > 0 && !y) return LRT_ERR_NULL;
  if (ntok > 0 && y == x) return LRT_ERR_SHAPE;  // not in place: the look-back rows would be overwritten
  if (ntok == 0) return LRT_OK;
  hipStream_t st = (hipStream_t)stream;
  const int n = n_seq;
#define LRT_CONV_FWD(E_)                                                                                  \
  {                                                                                                       \
    if (W == 2) conv_fwd_t<E_, 2>(x, w, y, cu_seqlens, n, T, (int)ntok, D, st);                           \
    if (W == 3) conv_fwd_t<E_, 3>(x, w, y, cu_seqlens, n, T, (int)ntok, D, st);                           \
    if (W == 4) conv_fwd_t<E_, 4>(x, w, y, cu_seqlens, n, T, (int)ntok, D, st);                           \
  }
  if (dtype == LRT_BF16)
    LRT_CONV_FWD(bf16)
  else
    LRT_CONV_FWD(float)
#undef LRT_CONV_FWD
  return hipGetLastError() == hipSuccess ? LRT_OK : LRT_ERR_LAUNCH;
}

int short_conv_bwd(const void* x, const float* w, const void* dy, void* dx, float* dw, const int* cu_seqlens,
                   int n_seq, int T, int D, int W, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  long long ntok = 0;
  int rc = conv_check(x, w, dy, dx, cu_seqlens, n_seq, T, D, W, dtype, ntok);
  if (rc) return rc;
  if (!dw || (ntok > 0 && (!dy || !dx))) return LRT_ERR_NULL;
  if (!aligned4b(dw)) return LRT_ERR_ALIGN;
  if (ntok > 0 && (dx == x || dx == dy)) return LRT_ERR_SHAPE;
  if (!workspace || !aligned16(workspace) || workspace_bytes < short_conv_bwd_workspace_bytes(ntok, D, W))
    return LRT_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  float* partial = (float*)workspace;
  if (ntok == 0) {
    // no tokens: dw = 0 (a fill kernel, so the call stays capturable)
    LRT_LAUNCH(kKConvDw, k_rows_reduce<kReduceWaves>, dim3((D * W + 63) / 64), dim3(64 * kReduceWaves), st,
               (const float*)partial, dw, 0, D * W);
    return hipGetLastError() == hipSuccess ? LRT_OK : LRT_ERR_LAUNCH;
  }
#define LRT_CONV_BWD(E_)                                                                                  \
  {                                                                                                       \
    if (W == 2) conv_bwd_t<E_, 2>(x, w, dy, dx, dw, partial, cu_seqlens, n_seq, T, (int)ntok, D, st);     \
    if (W == 3) conv_bwd_t<E_, 3>(x, w, dy, dx, dw, partial, cu_seqlens, n_seq, T, (int)ntok, D, st);     \
    if (W == 4) conv_bwd_t<E_, 4>(x, w, dy, dx, dw, partial, cu_seqlens, n_seq, T, (int)ntok, D, st);     \
  }
  if (dtype == LRT_BF16)
    LRT_CONV_BWD(bf16)
  else
    LRT_CONV_BWD(float)
#undef LRT_CONV_BWD
  return hipGetLastError() == hipSuccess ? LRT_OK : LRT_ERR_LAUNCH;
}

static int gnorm_check(const void* o, const void* z, const float* w, long long rows, int d, float eps, int dtype) {
  if (dtype != LRT_F32 && dtype != LRT_BF16) return LRT_ERR_DTYPE;
  if (rows < 0 || rows > 0x7fffffffLL || !(d == 16 || d == 32 || d == 64 || d == 128 || d == 256)) return LRT_ERR_SHAPE;
  if (!(eps >= 0.f) || eps > 1.f) return LRT_ERR_SHAPE;
  if (!w || (rows > 0 && (!o || !z))) return LRT_ERR_NULL;
  if ((o && !aligned16(o)) || (z && !aligned16(z)) || !aligned4b(w)) return LRT_ERR_ALIGN;
  return LRT_OK;
}

size_t gated_rmsnorm_bwd_workspace_bytes(long long rows, int d) {
  if (rows < 0 || rows > 0x7fffffffLL || !(d == 16 || d == 32 || d == 64 || d == 128 || d == 256)) return (size_t)-1;
  // the block count is at most kNormBlocks for either dtype
  const size_t b = (size_t)kNormBlocks * d * sizeof(float);
  return b;
}

int gated_rmsnorm_fwd(const void* o, const void* z, const float* w, void* y, long long rows, int d, float eps,
                      int dtype, void* stream) {
  int rc = gnorm_check(o, z, w, rows, d, eps, dtype);
  if (rc) return rc;
  if (rows > 0 && !y) return LRT_ERR_NULL;
  if (y && !aligned16(y)) return LRT_ERR_ALIGN;
  if (rows > 0 && (y == o || y == z)) return LRT_ERR_SHAPE;
  if (rows == 0) return LRT_OK;
  const int esz = dtype == LRT_BF16 ? 2 : 4;
  const int nb = gnorm_blocks(rows, d, esz);
  hipStream_t st = (hipStream_t)stream;
  if (dtype == LRT_BF16)
    gnorm_fwd_t<bf16>(o, z, w, y, (int)rows, d, eps, nb, st);
  else
    gnorm_fwd_t<float>(o, z, w, y, (int)rows, d, eps, nb, st);
  return hipGetLastError() == hipSuccess ? LRT_OK : LRT_ERR_LAUNCH;
}

int gated_rmsnorm_bwd(const void* o, const void* z, const float* w, const void* dy, void* d_o, void* dz, float* dw,
                      long long rows, int d, float eps, int dtype, void* workspace, size_t workspace_bytes,
                      void* stream) {
  int rc = gnorm_check(o, z, w, rows, d, eps, dtype);
  if (rc) return rc;
  if (!dw || (rows > 0 && (!dy || !d_o || !dz))) return LRT_ERR_NULL;
  const void* vec[] = {dy, d_o, dz};
  for (const void* p : vec)
    if (p && !aligned16(p)) return LRT_ERR_ALIGN;
  if (!aligned4b(dw)) return LRT_ERR_ALIGN;
  if (rows > 0 && (d_o == o || d_o == z || d_o == dy || dz == o || dz == z || dz == dy || dz == d_o))
    return LRT_ERR_SHAPE;
  if (!workspace || !aligned16(workspace) || workspace_bytes < gated_rmsnorm_bwd_workspace_bytes(rows, d))
    return LRT_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  float* partial = (float*)workspace;
  const int esz = dtype == LRT_BF16 ? 2 : 4;
  const int nb = rows > 0 ? gnorm_blocks(rows, d, esz) : 0;
  if (rows > 0) {
    if (dtype == LRT_BF16)
      gnorm_bwd_t<bf16>(o, z, w, dy, d_o, dz, partial, (int)rows, d, eps, nb, st);
    else
      gnorm_bwd_t<float>(o, z, w, dy, d_o, dz, partial, (int)rows, d, eps, nb, st);
  }
  LRT_LAUNCH(kKNormDw, k_rows_reduce<kReduceWaves>, dim3((d + 63) / 64), dim3(64 * kReduceWaves), st,
             (const float*)partial, dw, nb, d);
  return hipGetLastError() == hipSuccess ? LRT_OK : LRT_ERR_LAUNCH;
}

}  // extern "C"
