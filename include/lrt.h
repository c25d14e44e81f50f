/*
 * lrt.h -- C ABI of liblrt.so: gated delta-rule token mixers on AMD MI355X (gfx950).
 *
 * The mixers are the linear-recurrent "M" layers of the hybrid stacks in the
 * AMD ROCm blog "Pretraining hybrid LLMs with Primus" (section "How hybrid
 * models are defined in Primus", mixer list under Table 2):
 *   - Mamba2 (ssd_fwd, ssd_bwd; ssd_fwd_train + ssd_bwd_saved): the state
 *     is decayed by one scalar gate per head and a rank-one k v^T write is
 *     added each token;
 *   - Gated DeltaNet (gdn_fwd, gdn_bwd; gdn_fwd_train + gdn_bwd_saved for a
 *     training step that keeps the forward's intermediates): Mamba2 plus the
 *     delta rule, which replaces the value stored under the current key
 *     instead of only adding; one scalar forget gate per head;
 *   - Kimi Delta Attention (kda_fwd): GDN with one gate value per key
 *     dimension (the low-rank projection producing it is the caller's).
 *
 * With the state kept as H = S^T ([d_k, d_v], fp32), per batch b and head h:
 *   GDN: H_t = a_t (I - b_t k_t k_t^T) H_{t-1} + b_t k_t v_t^T
 *   SSD: H_t = a_t H_{t-1} + k_t v_t^T
 *   KDA: H_t = (I - b_t k_t k_t^T) Diag(a_t) H_{t-1} + b_t k_t v_t^T
 *   o_t = H_t^T q_t  (after token t's write),  a_t = exp(log_a_t),
 *   H_0 = h0 (NULL = zeros),  ht = H_T.
 * No query scaling is applied (pre-scale q if wanted).  The library evaluates
 * the chunkwise form of these recurrences, an exact rewrite of them.
 *
 * Layouts (all dense, row-major, contiguous; element offsets are 64-bit):
 *   q, k, do, dq, dk      [B, T, H, d_k]   dtype
 *   v, o, dv              [B, T, H, d_v]   dtype
 *   log_a, beta, dlog_a, dbeta   [B, T, H]  fp32   (KDA log_a: [B, T, H, d_k])
 *   h0, ht, dht, dh0      [B, H, d_k, d_v] fp32
 * dtype: LRT_F32 or LRT_BF16 (q, k, v, o and their gradients).  bf16 outputs
 * are rounded to nearest even.  log_a must be finite (normally <= 0).
 *
 * Supported: B, H >= 1; T >= 0; d_k, d_v in {16, 32, 64, 128};
 * chunk in {16, 32, 64}; B * T and B * H * ceil(T / chunk) * d_v / 16 at
 * most 2^31 - 1; H * max(d_k, d_v) below 2^24.  T need not be a multiple of
 * chunk.  Every entry point accepts every such size in both dtypes.
 *
 * chunk is the tile length of the chunkwise form, an exact rewrite of the
 * recurrence for every chunk size (only the rounding of the results depends
 * on it).  The kernels run the requested chunk or, where their fp32
 * operands would not fit in the 160 KB of LDS of a workgroup, the largest
 * smaller one that fits: with LRT_F32, kda_fwd at d_k = 128 or d_v = 128
 * (and at d_k = d_v = 64) runs 32-token chunks, and the backward and
 * training entry points run 16-token chunks at d_k or d_v = 128 (32 at
 * d_k = 128, d_v = 64 and the like).  lrt_workspace_bytes accounts for it.
 *
 * Ownership and execution: the caller allocates and frees every buffer,
 * including the workspace (size from lrt_workspace_bytes).  The library never
 * allocates, frees or synchronises; it enqueues kernels on `stream`
 * (a hipStream_t; NULL = the default stream) and returns.  Device faults
 * surface at the caller's next synchronisation.  Calls on different streams
 * with different workspaces may run concurrently.  All pointers are device
 * pointers.  q, k, v, o, do, dq, dk, dv and the workspace must be 16-byte
 * aligned; gates, beta, states and their gradients 4-byte aligned.
 *
 * Aliasing: ht may alias h0.  No other output may alias any input or output.
 *
 * Errors: every entry point validates all arguments before enqueuing
 * anything; on a non-zero return nothing has been written.
 */
#ifndef LRT_H
#define LRT_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define LRT_OK 0
#define LRT_ERR_NULL (-1)      /* a required pointer is NULL */
#define LRT_ERR_SHAPE (-2)     /* B, T, H, d_k or d_v out of the supported set */
#define LRT_ERR_CHUNK (-3)     /* chunk not in {16, 32, 64} */
#define LRT_ERR_DTYPE (-4)     /* dtype not LRT_F32 / LRT_BF16 */
#define LRT_ERR_WORKSPACE (-5) /* workspace NULL or smaller than lrt_workspace_bytes */
#define LRT_ERR_ALIGN (-6)     /* a pointer is under-aligned (see Ownership) */
#define LRT_ERR_LAUNCH (-7)    /* the HIP runtime rejected a launch */
#define LRT_ERR_OP (-8)        /* unknown op code */
#define LRT_ERR_TOO_LARGE (-9) /* gdn_fwd_noalloc: the sizes need more than LRT_NOALLOC_MAX_BYTES */

/* dtypes of q, k, v, o, do and the q/k/v gradients */
#define LRT_F32 0
#define LRT_BF16 1

/* op codes for lrt_workspace_bytes */
#define LRT_OP_GDN_FWD 0
#define LRT_OP_GDN_BWD 1
#define LRT_OP_KDA_FWD 2
#define LRT_OP_SSD_FWD 3
#define LRT_OP_SSD_BWD 4
/* packed variable-length sequences: B = number of sequences, T = total tokens */
#define LRT_OP_GDN_FWD_VARLEN 5
#define LRT_OP_GDN_BWD_VARLEN 6
#define LRT_OP_KDA_FWD_VARLEN 7
#define LRT_OP_KDA_BWD 8
#define LRT_OP_KDA_BWD_VARLEN 9

/*
 * Gated DeltaNet forward.  Writes o and (if not NULL) ht.
 * h0 may be NULL (zero initial state); ht may be NULL or equal to h0.
 */
int gdn_fwd(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
            const float* h0, void* o, float* ht, int B, int T, int H, int d_k, int d_v, int chunk,
            int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Gated DeltaNet backward: gradients of L = <do, o> + <dht, ht> with respect
 * to q, k, v, log_a, beta and h0, for the forward of the same arguments.
 * The forward is recomputed internally (no state is kept between calls).
 * dht may be NULL (zero).  dh0 may be NULL (not written).  dq, dk, dv,
 * dlog_a and dbeta are required.
 */
int gdn_bwd(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
            const float* h0, const void* d_o, const float* dht, void* dq, void* dk, void* dv,
            float* dlog_a, float* dbeta, float* dh0, int B, int T, int H, int d_k, int d_v,
            int chunk, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Kimi Delta Attention backward: gradients of L = <do, o> + <dht, ht> for
 * the forward of kda_fwd with the same arguments (the KDA mixer of the AMD
 * ROCm blog "Pretraining hybrid LLMs with Primus", section "How hybrid
 * models are defined in Primus", mixer list under Table 2; a pure-KDA
 * model is among the models trained there, Table 1).  As gdn_bwd, except
 * that the gate is per key dimension: log_a and dlog_a are [B, T, H, d_k]
 * fp32.  The forward is recomputed internally.  dht may be NULL (zero);
 * dh0 may be NULL (not written); dq, dk, dv, dlog_a and dbeta are
 * required.  Workspace: lrt_workspace_bytes(LRT_OP_KDA_BWD, ...).  Exact
 * for any finite log_a <= 0 (no factor of the decay that could overflow is
 * ever formed).
 */
int kda_bwd(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
            const float* h0, const void* d_o, const float* dht, void* dq, void* dk, void* dv,
            float* dlog_a, float* dbeta, float* dh0, int B, int T, int H, int d_k, int d_v,
            int chunk, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Kimi Delta Attention forward for training and the backward that reuses
 * it: kda_fwd_train is kda_fwd (same arguments, same o and ht) that also
 * leaves in the workspace what kda_bwd would recompute -- the chunk-parallel
 * pass's W, U', Ktil, G_C, Q o e^G, P and T = (I + A)^-1, the chunk-start
 * states and U; kda_bwd_saved, given that workspace unchanged and the same
 * q, k, v, log_a, beta, h0, skips the recompute and returns kda_bwd's
 * gradients.  Workspace: lrt_workspace_bytes(LRT_OP_KDA_BWD, ...); it may be
 * passed to kda_bwd_saved any number of times (other do / dht).
 */
int kda_fwd_train(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
                  const float* h0, void* o, float* ht, int B, int T, int H, int d_k, int d_v, int chunk,
                  int dtype, void* workspace, size_t workspace_bytes, void* stream);
int kda_bwd_saved(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
                  const float* h0, const void* d_o, const float* dht, void* dq, void* dk, void* dv,
                  float* dlog_a, float* dbeta, float* dh0, int B, int T, int H, int d_k, int d_v, int chunk,
                  int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Gated DeltaNet forward for training: gdn_fwd (same arguments, same o and
 * ht) that also leaves in the workspace what gdn_bwd would recompute -- the
 * WY factors W and T = (I + A)^-1, the in-chunk gate cumsums, the
 * chunk-start states and the new values U of the chunkwise form (the Gated
 * DeltaNet recurrence of the mixer list under Table 2 of the AMD ROCm blog
 * "Pretraining hybrid LLMs with Primus") -- for gdn_bwd_saved.  The
 * workspace must hold lrt_workspace_bytes(LRT_OP_GDN_BWD, ...) bytes.
 */
int gdn_fwd_train(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
                  const float* h0, void* o, float* ht, int B, int T, int H, int d_k, int d_v, int chunk,
                  int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_bwd without the recompute: the workspace must be the one a preceding
 * gdn_fwd_train of the same q, k, v, log_a, beta, h0 and sizes filled (stream
 * ordered after it), unmodified since.  Arguments, outputs and errors as
 * gdn_bwd.  The saved tensors stay in place (the backward's own scratch
 * lies elsewhere in the workspace), so further gdn_bwd_saved calls, e.g. for
 * another d_o, may follow.
 */
int gdn_bwd_saved(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
                  const float* h0, const void* d_o, const float* dht, void* dq, void* dk, void* dv,
                  float* dlog_a, float* dbeta, float* dh0, int B, int T, int H, int d_k, int d_v,
                  int chunk, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_fwd for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same arguments,
 * outputs and kernels, without the workspace arguments.  The workspace is a
 * static device array of LRT_NOALLOC_MAX_BYTES (64 MiB) inside the library,
 * one per GPU, held until the process ends; its device address is looked up
 * on the first call on each device.  Sizes whose workspace
 * (lrt_workspace_bytes(LRT_OP_GDN_FWD, ...)) exceeds it are rejected with
 * LRT_ERR_TOO_LARGE before anything is enqueued; other errors as gdn_fwd.
 * Every call on a GPU uses that GPU's one array: calls that overlap on one
 * GPU (other streams, other threads) race and give undefined results.
 * Nothing is allocated, freed or synchronised.
 */
#define LRT_NOALLOC_MAX_BYTES (64u << 20)
int gdn_fwd_noalloc(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
                    const float* h0, void* o, float* ht, int B, int T, int H, int d_k, int d_v, int chunk,
                    int dtype, void* stream);

/*
 * Kimi Delta Attention forward: as gdn_fwd, with log_a of shape [B, T, H, d_k]
 * (one log-gate per key dimension).
 */
int kda_fwd(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
            const float* h0, void* o, float* ht, int B, int T, int H, int d_k, int d_v, int chunk,
            int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Mamba2 / SSD forward (scalar decay, no delta term): as gdn_fwd without beta.
 */
int ssd_fwd(const void* q, const void* k, const void* v, const float* log_a, const float* h0,
            void* o, float* ht, int B, int T, int H, int d_k, int d_v, int chunk, int dtype,
            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Mamba2 / SSD backward: gradients of L = <do, o> + <dht, ht> with respect to
 * q, k, v, log_a and h0 for ssd_fwd of the same arguments (the scalar-decay
 * recurrence of the Mamba2 mixer on the AMD ROCm blog "Pretraining hybrid
 * LLMs with Primus", section "How hybrid models are defined in Primus",
 * mixer list under Table 2).  As gdn_bwd without beta and dbeta: the forward
 * is recomputed internally; dht may be NULL (zero); dh0 may be NULL (not
 * written); dq, dk, dv and dlog_a are required.  Workspace: LRT_OP_SSD_BWD.
 */
int ssd_bwd(const void* q, const void* k, const void* v, const float* log_a, const float* h0,
            const void* d_o, const float* dht, void* dq, void* dk, void* dv, float* dlog_a, float* dh0,
            int B, int T, int H, int d_k, int d_v, int chunk, int dtype, void* workspace,
            size_t workspace_bytes, void* stream);

/*
 * Mamba2 / SSD forward for training: ssd_fwd (same arguments, same o and ht)
 * that also leaves each chunk's start state and in-chunk gate cumsums in a
 * workspace of lrt_workspace_bytes(LRT_OP_SSD_BWD, ...) bytes for
 * ssd_bwd_saved.
 */
int ssd_fwd_train(const void* q, const void* k, const void* v, const float* log_a, const float* h0,
                  void* o, float* ht, int B, int T, int H, int d_k, int d_v, int chunk, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * ssd_bwd without the recompute, from the workspace a preceding
 * ssd_fwd_train of the same inputs and sizes filled (stream ordered after it,
 * unmodified since).  Arguments, outputs and errors as ssd_bwd; the saved
 * tensors stay in place, so several backward passes may follow.
 */
int ssd_bwd_saved(const void* q, const void* k, const void* v, const float* log_a, const float* h0,
                  const void* d_o, const float* dht, void* dq, void* dk, void* dv, float* dlog_a,
                  float* dh0, int B, int T, int H, int d_k, int d_v, int chunk, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * The mixer with its input activations fused into the kernels' load stage
 * (the fused-kernel recipe of the AMD ROCm blog "Pretraining hybrid LLMs with
 * Primus", section "Recipe", Table 4 and the paragraph on the use_fla_*
 * flags: unfused elementwise passes cost throughput).  Same outputs and
 * arguments as gdn_fwd / kda_fwd, for the raw projections:
 *   q = q_raw / sqrt(sum_d q_raw^2 + 1e-6)   per (b, t, h) row over d_k, in
 *   k = k_raw / sqrt(sum_d k_raw^2 + 1e-6)   fp32, rounded to dtype
 *   beta = sigmoid(beta_raw)                  beta_raw fp32 [B, T, H]
 *   log a = -softplus(gate_raw) = -(max(z, 0) + log(1 + exp(-|z|)))
 * gdn_fwd_fused: gate_raw fp32 [B, T, H].  kda_fwd_fused: gate_raw is the
 * per-key-dimension pre-activation (the low-rank projection's output) in
 * dtype, [B, T, H, d_k], 16-byte aligned -- half the bytes of an fp32 log-gate
 * for bf16.  The normalised q, k, the gates and beta are never written: one
 * read of the raw projections replaces the separate activation passes.
 */
int gdn_fwd_fused(const void* q_raw, const void* k_raw, const void* v, const float* gate_raw,
                  const float* beta_raw, const float* h0, void* o, float* ht, int B, int T, int H, int d_k, int d_v,
                  int chunk, int dtype, void* workspace, size_t workspace_bytes, void* stream);
int kda_fwd_fused(const void* q_raw, const void* k_raw, const void* v, const void* gate_raw, const float* beta_raw,
                  const float* h0, void* o, float* ht, int B, int T, int H, int d_k, int d_v, int chunk, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_fwd_fused with the gate given as its low-rank factors (KDA's gate is
 * a projection through a bottleneck, the KDA mixer of the AMD ROCm blog
 * "Pretraining hybrid LLMs with Primus", mixer list under Table 2): z
 * [B, T, rank] in dtype holds each token's bottleneck activations (W_down x,
 * shared by the heads) and w_up [H * d_k, rank] in dtype the up-projection;
 * the kernels form the pre-activation w_up z per (token, head) in fp32 and
 * apply -softplus, so only rank values per token are read for the gate
 * instead of H * d_k.  rank must be 16 (else LRT_ERR_SHAPE); z and w_up
 * 16-byte aligned.  Other arguments, outputs and workspace as kda_fwd_fused.
 */
int kda_fwd_fused_lowrank(const void* q_raw, const void* k_raw, const void* v, const void* z, const void* w_up,
                          int rank, const float* beta_raw, const float* h0, void* o, float* ht, int B, int T, int H,
                          int d_k, int d_v, int chunk, int dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * Packed variable-length sequences (the packed batches of long-context
 * training, where many sequences of different lengths share one
 * [1, T, H, d] tensor; the 1M-context 7-MLA / 21-GDN hybrid guide packs
 * 20-160 sequences per 1M tokens).  gdn_fwd, kda_fwd, gdn_bwd and kda_bwd for
 * n_seq >= 1 sequences: sequence s spans tokens [cu_seqlens[s],
 * cu_seqlens[s + 1]) of q, k, v, log_a, beta, o (and do, dq, dk, dv,
 * dlog_a, dbeta), each laid out as [1, T, H, d] ([1, T, H] for gates;
 * KDA log_a [1, T, H, d_k]).  cu_seqlens is a device array of n_seq + 1
 * int32 (cu[0] = 0, non-decreasing, cu[n_seq] = T).  Every sequence starts
 * from its own initial state: h0, ht, dht, dh0 are [n_seq, H, d_k, d_v]
 * fp32 (h0 / dht NULL = zeros).  The result for each sequence is that of
 * the dense entry point on that sequence alone; chunks never straddle a
 * sequence boundary (a sequence shorter than `chunk` is one short chunk).
 * Entries outside [0, T] or decreasing are clamped (running maximum) so
 * that no kernel touches memory outside the tensors; the results are then
 * undefined.  Workspace: lrt_workspace_bytes(LRT_OP_*_VARLEN, n_seq, T, ...).
 * Arguments, outputs and other errors as the dense entry points.
 */
int gdn_fwd_varlen(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
                   const float* h0, void* o, float* ht, const int* cu_seqlens, int n_seq, int T, int H, int d_k,
                   int d_v, int chunk, int dtype, void* workspace, size_t workspace_bytes, void* stream);
int kda_fwd_varlen(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
                   const float* h0, void* o, float* ht, const int* cu_seqlens, int n_seq, int T, int H, int d_k,
                   int d_v, int chunk, int dtype, void* workspace, size_t workspace_bytes, void* stream);
int gdn_bwd_varlen(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
                   const float* h0, const void* d_o, const float* dht, void* dq, void* dk, void* dv, float* dlog_a,
                   float* dbeta, float* dh0, const int* cu_seqlens, int n_seq, int T, int H, int d_k, int d_v,
                   int chunk, int dtype, void* workspace, size_t workspace_bytes, void* stream);
int kda_bwd_varlen(const void* q, const void* k, const void* v, const float* log_a, const float* beta,
                   const float* h0, const void* d_o, const float* dht, void* dq, void* dk, void* dv, float* dlog_a,
                   float* dbeta, float* dh0, const int* cu_seqlens, int n_seq, int T, int H, int d_k, int d_v,
                   int chunk, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two steps either side of the mixer, as the single-pass fused kernels
 * of the pretraining recipe (AMD ROCm blog "Pretraining hybrid LLMs with
 * Primus", "Recipe", Table 4: the FLA fusion row names fused gated norm and
 * short conv kernels; the epsilon row gives 1e-6).  The pages name the steps
 * without defining them; the library computes:
 *
 * short_conv_fwd: the short convolution on the mixer's q, k or v projection,
 *   a causal depthwise convolution of width W over the tokens of each
 *   sequence followed by SiLU:
 *     pre[t, c] = sum_{j<W} w[c, j] x[t - (W - 1) + j, c],  y = pre * sigmoid(pre),
 *   tokens before the sequence start counting as zero.  x, y: [n_seq, T, D]
 *   (dense, cu_seqlens NULL) or one packed row [1, T, D] holding n_seq
 *   sequences at [cu_seqlens[s], cu_seqlens[s + 1]) (the mixers' varlen
 *   convention: n_seq + 1 int32, cu[0] = 0, non-decreasing, cu[n_seq] = T;
 *   malformed tables are clamped, results then undefined); dtype LRT_F32 or
 *   LRT_BF16.  w: [D, W] fp32 (tap W - 1 multiplies the current token).
 *   D a multiple of 8 below 2^24; W in {2, 3, 4}; at most 2^31 - 1 tokens.
 *   q, k and v may go through one call as the columns of one [.., 3 D]
 *   tensor.  y must not alias x (LRT_ERR_SHAPE).
 * short_conv_bwd: dx [like x] and dw [D, W] fp32 (overwritten) of
 *   L = sum(dy * y), from x, w and dy; dx aliases neither x nor dy.
 *   Workspace: short_conv_bwd_workspace_bytes(tokens, D, W) bytes, 16-byte
 *   aligned (tokens = n_seq * T dense, T packed); (size_t)-1 for invalid
 *   sizes.  dw is summed in a fixed order: repeated calls are bitwise equal.
 *
 * gated_rmsnorm_fwd: the mixer's output gate and norm over rows of d values
 *   (one token and head each):  y = o / sqrt(mean(o^2) + eps) * w * silu(z).
 *   o, z, y: [rows, d] dtype (y aliases neither, LRT_ERR_SHAPE); w: [d] fp32; d in
 *   {16, 32, 64, 128, 256}; rows <= 2^31 - 1; eps in [0, 1].
 * gated_rmsnorm_bwd: do, dz [rows, d] dtype and dw [d] fp32 (overwritten) of
 *   L = sum(dy * y); do and dz alias no input.  Workspace:
 *   gated_rmsnorm_bwd_workspace_bytes(rows, d) bytes, 16-byte aligned.
 *   Deterministic as above.
 *
 * All: device pointers; token tensors and workspaces 16-byte aligned, w, dw
 * and cu_seqlens 4-byte aligned; nothing allocated or synchronised; errors
 * (LRT_ERR_*) returned before anything is enqueued.  With no tokens or rows
 * the forwards do nothing and the backwards write dw = 0.
 */
int short_conv_fwd(const void* x, const float* w, void* y, const int* cu_seqlens, int n_seq, int T, int D, int W,
                   int dtype, void* stream);
int short_conv_bwd(const void* x, const float* w, const void* dy, void* dx, float* dw, const int* cu_seqlens,
                   int n_seq, int T, int D, int W, int dtype, void* workspace, size_t workspace_bytes, void* stream);
size_t short_conv_bwd_workspace_bytes(long long n_tokens, int D, int W);
int gated_rmsnorm_fwd(const void* o, const void* z, const float* w, void* y, long long rows, int d, float eps,
                      int dtype, void* stream);
int gated_rmsnorm_bwd(const void* o, const void* z, const float* w, const void* dy, void* d_o, void* dz, float* dw,
                      long long rows, int d, float eps, int dtype, void* workspace, size_t workspace_bytes,
                      void* stream);
size_t gated_rmsnorm_bwd_workspace_bytes(long long rows, int d);

/*
 * Workspace bytes needed by `op` (LRT_OP_*) at these sizes.  Returns
 * (size_t)-1 for invalid arguments.  0 is never returned for valid ones.
 */
size_t lrt_workspace_bytes(int op, int B, int T, int H, int d_k, int d_v, int chunk, int dtype);

/* Static, human-readable text for a status code. */
const char* lrt_status_string(int status);

/*
 * Per-kernel timing hook for benchmarks.  It is per calling thread (kept in
 * thread-local storage): it brackets only kernels enqueued by the thread
 * that attached it, and calls from other threads neither see nor change it.
 * After lrt_profile_attach(events, kinds, n) on a thread, the next n kernels
 * the library enqueues from that thread are each bracketed by
 * hipEventRecord(events[2i]) and hipEventRecord(events[2i + 1]) on the
 * kernel's own stream, and kinds[i] receives the kernel's id.  `events`
 * holds 2n hipEvent_t created by the caller; `kinds` holds n ints.  Passing
 * NULL detaches.  lrt_profile_count() returns the kernels recorded since the
 * last attach; lrt_kernel_name(id) a static name for an id.
 */
int lrt_profile_attach(void** events, int* kinds, int n_kernels);
int lrt_profile_count(void);
const char* lrt_kernel_name(int kind);

#ifdef __cplusplus
}
#endif

#endif /* LRT_H */
