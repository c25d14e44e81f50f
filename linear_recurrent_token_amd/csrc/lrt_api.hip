// lrt_api.hip -- the C ABI of liblrt.so: argument validation, workspace
// sizing and dispatch onto the caller's stream.  Nothing here allocates,
// frees or synchronises.
#include <stdint.h>

#include <mutex>

#include "lrt_common.hpp"
#include "lrt_internal.hpp"

namespace lrt {

// --------------------------------------------------- static scratch (noalloc)
// The workspace of gdn_fwd_noalloc: a device array of LRT_NOALLOC_MAX_BYTES,
// one copy per GPU the library runs on, held until the process ends.  Host
// code never uses the array's name as an address: the device address of
// each GPU's copy is looked up once per device (hipGetSymbolAddress, with
// that device current) and kept in g_scratch_addr.
static __device__ __align__(256) unsigned char scratch[LRT_NOALLOC_MAX_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_addr[kMaxDevices];  // per device id; nullptr until looked up

// The current device's copy of `scratch`, or nullptr if it cannot be found.
static void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_addr[dev] = ptr;
  }
  return g_scratch_addr[dev];
}

// ---------------------------------------------------------------- timing hook
// Per calling thread (only the benchmark attaches it): entry points called
// from other threads are never bracketed, and no state is shared between
// threads.
struct ProfHook {
  hipEvent_t* ev = nullptr;
  int* kinds = nullptr;
  int n = 0;     // kernels that fit
  int next = 0;  // kernels recorded
};
static thread_local ProfHook g_prof;

void prof_before(int kind, void* stream) {
  if (g_prof.ev == nullptr || g_prof.next >= g_prof.n) return;
  g_prof.kinds[g_prof.next] = kind;
  hipEventRecord(g_prof.ev[2 * g_prof.next], (hipStream_t)stream);
}

void prof_after(void* stream) {
  if (g_prof.ev == nullptr || g_prof.next >= g_prof.n) return;
  hipEventRecord(g_prof.ev[2 * g_prof.next + 1], (hipStream_t)stream);
  ++g_prof.next;
}

static const char* const kKernelNames[kKNumKinds] = {
    "k_bwd_local", "k_dstate",   "k_grad",       "k_kda_prep", "k_state_copy", "k_wy",     "k_scan",
    "k_wy_bwd",    "k_scan_bwd", "k_scan_local", "k_carry",    "k_ssd_prep",   "k_ssd_fwd",
    "k_varlen_plan", "k_kda_prep_bwd", "k_grad_kda", "k_kda_prep_fast", "k_kda_prep_fast_bwd", "k_list_reset",
    "k_conv_fwd", "k_conv_bwd", "k_rows_reduce(conv dw)", "k_gnorm_fwd", "k_gnorm_bwd", "k_rows_reduce(norm dw)"};

// Queried on every call (a device attribute read; nothing is cached between
// calls).
int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  return n;
}

// ht = h0 (or zeros) for an empty sequence.
__global__ void k_state_copy(const float* __restrict__ h0, float* ht, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) ht[i] = h0 ? h0[i] : 0.f;
}

static bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
static bool aligned(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// packed: B sequences of T tokens in all (cu_seqlens), else B sequences of T tokens each
static int check_common(int B, int T, int H, int dk, int dv, int chunk, int dtype, bool packed = false) {
  if (dtype != LRT_F32 && dtype != LRT_BF16) return LRT_ERR_DTYPE;
  if (B < 1 || H < 1 || T < 0 || !dim_ok(dk) || !dim_ok(dv)) return LRT_ERR_SHAPE;
  // 64-bit offsets everywhere; keep token counts within int for the grid math
  if (!packed && (long long)B * T > 0x7fffffffLL) return LRT_ERR_SHAPE;
  if (chunk != 16 && chunk != 32 && chunk != 64) return LRT_ERR_CHUNK;
  // a chunk tile's element offsets are 32-bit in the kernels
  if ((long long)H * (dk > dv ? dk : dv) >= (1LL << 24)) return LRT_ERR_SHAPE;
  // chunk tiles times value blocks index the grids as int
  const long long tiles = packed ? (long long)H * ((T + chunk - 1) / chunk + B) : (long long)B * H * ((T + chunk - 1) / chunk);
  if (tiles * (dv / 16) > 0x7fffffffLL || (long long)B * H * (dv / 16) > 0x7fffffffLL) return LRT_ERR_SHAPE;
  return LRT_OK;
}

// the base op of a workspace op code, and whether it is the packed form
static int base_op(int op, bool* packed) {
  *packed = true;
  switch (op) {
    case LRT_OP_GDN_FWD_VARLEN: return LRT_OP_GDN_FWD;
    case LRT_OP_GDN_BWD_VARLEN: return LRT_OP_GDN_BWD;
    case LRT_OP_KDA_FWD_VARLEN: return LRT_OP_KDA_FWD;
    case LRT_OP_KDA_BWD_VARLEN: return LRT_OP_KDA_BWD;
    default: *packed = false; return op;
  }
}

// The chunk the kernels of `op` run: the requested one, or the largest
// smaller one at which all of them fit in LDS (fp32 at d_k or d_v = 128).
// The chunkwise form is exact for every chunk size; only rounding depends
// on it.  The training forwards run the backward's chunk, so that the saved
// tensors match the backward's tiles.
static int run_chunk(int op, int dtype, int dk, int dv, int chunk) {
  int m = 64;
  if (op == LRT_OP_GDN_FWD) m = fwd_max_chunk(dtype, dk, dv);
  if (op == LRT_OP_KDA_FWD) m = kda_max_chunk(dtype, dk, dv);
  if (op == LRT_OP_GDN_BWD || op == LRT_OP_SSD_BWD) m = bwd_max_chunk(op, dtype, dk, dv);
  if (op == LRT_OP_KDA_BWD) m = kda_bwd_max_chunk(dtype, dk, dv);
  return chunk < m ? chunk : m;
}

static size_t ws_bytes(int op_code, int B, int T, int H, int dk, int dv, int chunk, int dtype) {
  bool packed = false;
  const int op = base_op(op_code, &packed);
  const size_t esz = dtype == LRT_BF16 ? 2 : 4;
  const int c = run_chunk(op, dtype, dk, dv, chunk);
  size_t b = fwd_ws_layout(op, B, T, H, dk, dv, c, esz, nullptr, packed).bytes;
  if (op == LRT_OP_GDN_BWD || op == LRT_OP_SSD_BWD || op == LRT_OP_KDA_BWD)
    b += bwd_ws_extra(op, B, T, H, dk, dv, c, esz, packed);
  return b < 256 ? 256 : b;
}

static int launch_empty(const float* h0, float* ht, int B, int H, int dk, int dv, void* stream) {
  if (ht == nullptr || ht == h0) return LRT_OK;
  const size_t n = (size_t)B * H * dk * dv;
  LRT_LAUNCH(kKStateCopy, k_state_copy, dim3((unsigned)((n + 255) / 256)), dim3(256), stream, h0, ht, n);
  return hipGetLastError() == hipSuccess ? LRT_OK : LRT_ERR_LAUNCH;
}

static int fwd_entry(int variant, const void* q, const void* k, const void* v, const float* log_a,
                     const float* beta, const float* h0, void* o, float* ht, int B, int T, int H, int dk,
                     int dv, int chunk, int dtype, void* workspace, size_t workspace_bytes, void* stream,
                     bool train = false, const int* cu = nullptr, bool packed = false, bool fuse = false,
                     const void* gate_up = nullptr) {
  int rc = check_common(B, T, H, dk, dv, chunk, dtype, packed);
  if (rc) return rc;
  if (packed && !cu) return LRT_ERR_NULL;
  if (packed && !aligned4(cu)) return LRT_ERR_ALIGN;
  // with T == 0 the token tensors are empty and may carry NULL pointers
  if (T > 0 && (!q || !k || !v || !log_a || !o || (variant != kVarSSD && !beta))) return LRT_ERR_NULL;
  // token tensors and the workspace are read with 16-byte vectors; gates and
  // states with 4-byte scalars
  const void* vec[] = {q, k, v, o, workspace};
  for (const void* p : vec)
    if (p && !aligned(p)) return LRT_ERR_ALIGN;
  const void* sca[] = {log_a, beta, h0, ht};
  for (const void* p : sca)
    if (p && !aligned4(p)) return LRT_ERR_ALIGN;
  // the fused KDA gate pre-activation (or its low-rank factors) is read in 16-byte pieces
  if (fuse && variant == kVarKDA && log_a && !aligned(log_a)) return LRT_ERR_ALIGN;
  if (gate_up && !aligned(gate_up)) return LRT_ERR_ALIGN;
  const int op = train ? (variant == kVarSSD ? LRT_OP_SSD_BWD : variant == kVarKDA ? LRT_OP_KDA_BWD : LRT_OP_GDN_BWD)
                       : variant == kVarGDN ? LRT_OP_GDN_FWD : variant == kVarSSD ? LRT_OP_SSD_FWD : LRT_OP_KDA_FWD;
  const int ws_op = !packed ? op : op == LRT_OP_GDN_FWD ? LRT_OP_GDN_FWD_VARLEN : LRT_OP_KDA_FWD_VARLEN;
  if (!workspace || workspace_bytes < ws_bytes(ws_op, B, T, H, dk, dv, chunk, dtype)) return LRT_ERR_WORKSPACE;
  if (T == 0) return launch_empty(h0, ht, B, H, dk, dv, stream);
  FwdArgs a{variant, q, k, v, log_a, beta, h0, o, ht, B, T, H, dk, dv, run_chunk(op, dtype, dk, dv, chunk), dtype,
            workspace, stream, packed ? cu : nullptr, fuse, gate_up};
  rc = train ? (variant == kVarKDA ? fwd_train_kda(a) : fwd_train(a)) : variant == kVarKDA ? fwd_kda(a)
                                                                      : fwd_scalar_gate(a);
  return rc == 0 ? LRT_OK : (rc == -7 ? LRT_ERR_LAUNCH : rc == -3 ? LRT_ERR_CHUNK : LRT_ERR_SHAPE);
}

static int bwd_entry(int variant, const void* q, const void* k, const void* v, const float* log_a,
                     const float* beta, const float* h0, const void* d_o, const float* dht, void* dq, void* dk,
                     void* dv, float* dlog_a, float* dbeta, float* dh0, int B, int T, int H, int d_k, int d_v,
                     int chunk, int dtype, void* workspace, size_t workspace_bytes, void* stream,
                     bool saved = false, const int* cu = nullptr, bool packed = false) {
  int rc = check_common(B, T, H, d_k, d_v, chunk, dtype, packed);
  if (rc) return rc;
  if (packed && !cu) return LRT_ERR_NULL;
  if (packed && !aligned4(cu)) return LRT_ERR_ALIGN;
  const bool delta = variant != kVarSSD;
  if (T > 0 && (!q || !k || !v || !log_a || !d_o || !dq || !dk || !dv || !dlog_a || (delta && (!beta || !dbeta))))
    return LRT_ERR_NULL;
  const void* vec[] = {q, k, v, d_o, dq, dk, dv, workspace};
  for (const void* p : vec)
    if (p && !aligned(p)) return LRT_ERR_ALIGN;
  const void* sca[] = {log_a, beta, h0, dht, dlog_a, dbeta, dh0};
  for (const void* p : sca)
    if (p && !aligned4(p)) return LRT_ERR_ALIGN;
  const int op = variant == kVarGDN ? LRT_OP_GDN_BWD : variant == kVarKDA ? LRT_OP_KDA_BWD : LRT_OP_SSD_BWD;
  const int ws_op = !packed ? op : op == LRT_OP_GDN_BWD ? LRT_OP_GDN_BWD_VARLEN : LRT_OP_KDA_BWD_VARLEN;
  if (!workspace || workspace_bytes < ws_bytes(ws_op, B, T, H, d_k, d_v, chunk, dtype)) return LRT_ERR_WORKSPACE;
  if (T == 0) return launch_empty(dht, dh0, B, H, d_k, d_v, stream);
  BwdArgs a{q, k, v, log_a, beta, h0, d_o, dht, dq, dk, dv, dlog_a, dbeta, dh0,
            B, T, H, d_k, d_v, run_chunk(op, dtype, d_k, d_v, chunk), dtype, workspace, stream, packed ? cu : nullptr};
  rc = variant == kVarGDN ? bwd_gdn(a, saved) : variant == kVarKDA ? bwd_kda(a, saved) : bwd_ssd(a, saved);
  return rc == 0 ? LRT_OK : (rc == -7 ? LRT_ERR_LAUNCH : rc == -3 ? LRT_ERR_CHUNK : LRT_ERR_SHAPE);
}

}  // namespace lrt

using namespace lrt;

extern "C" {

int gdn_fwd(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
            const float* h0, void* o, float* ht, int B, int T, int H, int d_k, int d_v, int chunk,
            int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_entry(kVarGDN, q, k, v, log_a, beta, h0, o, ht, B, T, H, d_k, d_v, chunk, dtype, workspace,
                   workspace_bytes, stream);
}

int gdn_fwd_noalloc(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
                    const float* h0, void* o, float* ht, int B, int T, int H, int d_k, int d_v, int chunk,
                    int dtype, void* stream) {
  const size_t need = lrt_workspace_bytes(LRT_OP_GDN_FWD, B, T, H, d_k, d_v, chunk, dtype);
  if (need != (size_t)-1 && need > (size_t)LRT_NOALLOC_MAX_BYTES) return LRT_ERR_TOO_LARGE;
  void* ws = scratch_address();
  if (ws == nullptr) return LRT_ERR_LAUNCH;
  // gdn_fwd validates every other argument; its kernels write every
  // workspace tile they read, so the array's earlier contents do not matter
  return fwd_entry(kVarGDN, q, k, v, log_a, beta, h0, o, ht, B, T, H, d_k, d_v, chunk, dtype, ws,
                   (size_t)LRT_NOALLOC_MAX_BYTES, stream);
}

int kda_fwd(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
            const float* h0, void* o, float* ht, int B, int T, int H, int d_k, int d_v, int chunk,
            int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_entry(kVarKDA, q, k, v, log_a, beta, h0, o, ht, B, T, H, d_k, d_v, chunk, dtype, workspace,
                   workspace_bytes, stream);
}

int ssd_fwd(const void* q, const void* k, const void* v, const float* log_a, const float* h0, void* o,
            float* ht, int B, int T, int H, int d_k, int d_v, int chunk, int dtype, void* workspace,
            size_t workspace_bytes, void* stream) {
  return fwd_entry(kVarSSD, q, k, v, log_a, nullptr, h0, o, ht, B, T, H, d_k, d_v, chunk, dtype, workspace,
                   workspace_bytes, stream);
}

int gdn_bwd(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
            const float* h0, const void* d_o, const float* dht, void* dq, void* dk, void* dv,
            float* dlog_a, float* dbeta, float* dh0, int B, int T, int H, int d_k, int d_v, int chunk,
            int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_entry(kVarGDN, q, k, v, log_a, beta, h0, d_o, dht, dq, dk, dv, dlog_a, dbeta, dh0, B, T, H, d_k, d_v,
                   chunk, dtype, workspace, workspace_bytes, stream);
}

int kda_bwd(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
            const float* h0, const void* d_o, const float* dht, void* dq, void* dk, void* dv,
            float* dlog_a, float* dbeta, float* dh0, int B, int T, int H, int d_k, int d_v, int chunk,
            int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_entry(kVarKDA, q, k, v, log_a, beta, h0, d_o, dht, dq, dk, dv, dlog_a, dbeta, dh0, B, T, H, d_k, d_v,
                   chunk, dtype, workspace, workspace_bytes, stream);
}

int kda_fwd_train(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
                  const float* h0, void* o, float* ht, int B, int T, int H, int d_k, int d_v, int chunk,
                  int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_entry(kVarKDA, q, k, v, log_a, beta, h0, o, ht, B, T, H, d_k, d_v, chunk, dtype, workspace,
                   workspace_bytes, stream, true);
}

int kda_bwd_saved(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
                  const float* h0, const void* d_o, const float* dht, void* dq, void* dk, void* dv,
                  float* dlog_a, float* dbeta, float* dh0, int B, int T, int H, int d_k, int d_v, int chunk,
                  int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_entry(kVarKDA, q, k, v, log_a, beta, h0, d_o, dht, dq, dk, dv, dlog_a, dbeta, dh0, B, T, H, d_k, d_v,
                   chunk, dtype, workspace, workspace_bytes, stream, true);
}

int gdn_fwd_train(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
                  const float* h0, void* o, float* ht, int B, int T, int H, int d_k, int d_v, int chunk,
                  int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_entry(kVarGDN, q, k, v, log_a, beta, h0, o, ht, B, T, H, d_k, d_v, chunk, dtype, workspace,
                   workspace_bytes, stream, true);
}

int gdn_bwd_saved(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
                  const float* h0, const void* d_o, const float* dht, void* dq, void* dk, void* dv,
                  float* dlog_a, float* dbeta, float* dh0, int B, int T, int H, int d_k, int d_v, int chunk,
                  int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_entry(kVarGDN, q, k, v, log_a, beta, h0, d_o, dht, dq, dk, dv, dlog_a, dbeta, dh0, B, T, H, d_k, d_v,
                   chunk, dtype, workspace, workspace_bytes, stream, true);
}

int ssd_fwd_train(const void* q, const void* k, const void* v, const float* log_a, const float* h0, void* o,
                  float* ht, int B, int T, int H, int d_k, int d_v, int chunk, int dtype, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return fwd_entry(kVarSSD, q, k, v, log_a, nullptr, h0, o, ht, B, T, H, d_k, d_v, chunk, dtype, workspace,
                   workspace_bytes, stream, true);
}

int ssd_bwd_saved(const void* q, const void* k, const void* v, const float* log_a, const float* h0,
                  const void* d_o, const float* dht, void* dq, void* dk, void* dv, float* dlog_a, float* dh0,
                  int B, int T, int H, int d_k, int d_v, int chunk, int dtype, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return bwd_entry(kVarSSD, q, k, v, log_a, nullptr, h0, d_o, dht, dq, dk, dv, dlog_a, nullptr, dh0, B, T, H, d_k,
                   d_v, chunk, dtype, workspace, workspace_bytes, stream, true);
}

int ssd_bwd(const void* q, const void* k, const void* v, const float* log_a, const float* h0, const void* d_o,
            const float* dht, void* dq, void* dk, void* dv, float* dlog_a, float* dh0, int B, int T, int H,
            int d_k, int d_v, int chunk, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_entry(kVarSSD, q, k, v, log_a, nullptr, h0, d_o, dht, dq, dk, dv, dlog_a, nullptr, dh0, B, T, H, d_k,
                   d_v, chunk, dtype, workspace, workspace_bytes, stream);
}

size_t lrt_workspace_bytes(int op, int B, int T, int H, int d_k, int d_v, int chunk, int dtype) {
  if (op < LRT_OP_GDN_FWD || op > LRT_OP_KDA_BWD_VARLEN) return (size_t)-1;
  bool packed = false;
  base_op(op, &packed);
  if (check_common(B, T, H, d_k, d_v, chunk, dtype, packed) != LRT_OK) return (size_t)-1;
  return ws_bytes(op, B, T, H, d_k, d_v, chunk, dtype);
}

int gdn_fwd_fused(const void* q_raw, const void* k_raw, const void* v, const float* gate_raw,
                  const float* beta_raw, const float* h0, void* o, float* ht, int B, int T, int H, int d_k, int d_v,
                  int chunk, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_entry(kVarGDN, q_raw, k_raw, v, gate_raw, beta_raw, h0, o, ht, B, T, H, d_k, d_v, chunk, dtype,
                   workspace, workspace_bytes, stream, false, nullptr, false, true);
}

int kda_fwd_fused(const void* q_raw, const void* k_raw, const void* v, const void* gate_raw, const float* beta_raw,
                  const float* h0, void* o, float* ht, int B, int T, int H, int d_k, int d_v, int chunk, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_entry(kVarKDA, q_raw, k_raw, v, (const float*)gate_raw, beta_raw, h0, o, ht, B, T, H, d_k, d_v, chunk,
                   dtype, workspace, workspace_bytes, stream, false, nullptr, false, true);
}

int kda_fwd_fused_lowrank(const void* q_raw, const void* k_raw, const void* v, const void* z, const void* w_up,
                          int rank, const float* beta_raw, const float* h0, void* o, float* ht, int B, int T, int H,
                          int d_k, int d_v, int chunk, int dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (rank != kGateRank) return LRT_ERR_SHAPE;
  if (T > 0 && !w_up) return LRT_ERR_NULL;
  return fwd_entry(kVarKDA, q_raw, k_raw, v, (const float*)z, beta_raw, h0, o, ht, B, T, H, d_k, d_v, chunk, dtype,
                   workspace, workspace_bytes, stream, false, nullptr, false, true, T > 0 ? w_up : nullptr);
}

int gdn_fwd_varlen(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
                   const float* h0, void* o, float* ht, const int* cu_seqlens, int n_seq, int T, int H, int d_k,
                   int d_v, int chunk, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_entry(kVarGDN, q, k, v, log_a, beta, h0, o, ht, n_seq, T, H, d_k, d_v, chunk, dtype, workspace,
                   workspace_bytes, stream, false, cu_seqlens, true);
}

int kda_fwd_varlen(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
                   const float* h0, void* o, float* ht, const int* cu_seqlens, int n_seq, int T, int H, int d_k,
                   int d_v, int chunk, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_entry(kVarKDA, q, k, v, log_a, beta, h0, o, ht, n_seq, T, H, d_k, d_v, chunk, dtype, workspace,
                   workspace_bytes, stream, false, cu_seqlens, true);
}

int gdn_bwd_varlen(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
                   const float* h0, const void* d_o, const float* dht, void* dq, void* dk, void* dv, float* dlog_a,
                   float* dbeta, float* dh0, const int* cu_seqlens, int n_seq, int T, int H, int d_k, int d_v,
                   int chunk, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_entry(kVarGDN, q, k, v, log_a, beta, h0, d_o, dht, dq, dk, dv, dlog_a, dbeta, dh0, n_seq, T, H, d_k,
                   d_v, chunk, dtype, workspace, workspace_bytes, stream, false, cu_seqlens, true);
}
int kda_bwd_varlen(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
                   const float* h0, const void* d_o, const float* dht, void* dq, void* dk, void* dv, float* dlog_a,
                   float* dbeta, float* dh0, const int* cu_seqlens, int n_seq, int T, int H, int d_k, int d_v,
                   int chunk, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_entry(kVarKDA, q, k, v, log_a, beta, h0, d_o, dht, dq, dk, dv, dlog_a, dbeta, dh0, n_seq, T, H, d_k,
                   d_v, chunk, dtype, workspace, workspace_bytes, stream, false, cu_seqlens, true);
}
int lrt_profile_attach(void** events, int* kinds, int n_kernels) {
  if (events == nullptr || kinds == nullptr || n_kernels <= 0) {
    g_prof.ev = nullptr;
    g_prof.kinds = nullptr;
    g_prof.n = g_prof.next = 0;
    return LRT_OK;
  }
  g_prof.ev = (hipEvent_t*)events;
  g_prof.kinds = kinds;
  g_prof.n = n_kernels;
  g_prof.next = 0;
  return LRT_OK;
}

int lrt_profile_count(void) { return g_prof.next; }

const char* lrt_kernel_name(int kind) {
  return (kind >= 0 && kind < kKNumKinds) ? kKernelNames[kind] : "unknown";
}

const char* lrt_status_string(int status) {
  switch (status) {
    case LRT_OK: return "ok";
    case LRT_ERR_NULL: return "a required pointer is NULL";
    case LRT_ERR_SHAPE: return "unsupported shape (B, H >= 1, T >= 0, d_k and d_v in {16, 32, 64, 128})";
    case LRT_ERR_CHUNK: return "unsupported chunk size (16, 32 or 64)";
    case LRT_ERR_DTYPE: return "unsupported dtype (LRT_F32 or LRT_BF16)";
    case LRT_ERR_WORKSPACE: return "workspace missing or smaller than lrt_workspace_bytes";
    case LRT_ERR_ALIGN: return "a pointer is under-aligned (token tensors and workspace: 16 bytes; gates and states: 4)";
    case LRT_ERR_LAUNCH: return "kernel launch failed";
    case LRT_ERR_OP: return "unknown op";
    case LRT_ERR_TOO_LARGE: return "the workspace these sizes need exceeds LRT_NOALLOC_MAX_BYTES (use gdn_fwd with a workspace)";
    default: return "unknown status";
  }
}

}  // extern "C"
