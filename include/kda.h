/*
 * kda.h -- C ABI of the MI355X (gfx950) KDA chunk library.
 *
 * KDA (Kimi Delta Attention) is the gated delta rule with a per-channel log-decay g_t and a
 * write strength beta_t:
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = scale * S_t^T q_t,
 * with S a K x V state per (sequence, value head). The chunkwise form processes C tokens
 * at a time through the chunk-local cumsum G of g, the WY/UT inverse
 * INV = (I + strict_tril(diag(beta) (k e^G)(k e^-G)^T))^-1 and the chunk states S_in
 * (FlashKDA backward page: the forward workspace kd, qd, kr, ki, INV, Mqk and S_in per
 * chunk; FLA chunk_kda_bwd page: chunk_gated_delta_rule_fwd_h / recompute_w_u_fwd and the
 * driver chunk_kda_bwd with its returns dq, dk, dv, db, dg, dh0).
 *
 * Two entry points do the work:
 *   kda_fwd_states -- forward chunk-state materialisation: INV and S_in per chunk, the
 *                     final state, optionally the output o;
 *   kda_chunk_bwd  -- the chunkwise backward: given dO and optionally dS_final (the
 *                     gradient w.r.t. the final state) returns dq, dk, dv, dg, dbeta, dh0,
 *                     the vector-Jacobian product of sum<dO,o> + <dS_final,S_T>.
 * kda_fwd_states_save / kda_chunk_bwd_saved are the same pair with the backward's chunk
 * operands kept from the forward (saved-operand mode, below).
 *
 * Conventions shared by every call:
 *  - All tensor arguments are DEVICE pointers (the GPU of the current HIP device),
 *    row-major and contiguous, owned by the caller. The library never allocates, frees or
 *    synchronises; it enqueues its kernels on `stream` (a hipStream_t; NULL = the null
 *    stream) and returns. Scratch memory is the caller's `workspace`.
 *  - Token axis: dense batches use [B, T, ...]; packed variable-length batches use B = 1
 *    and [1, T_total, ...] with cu_seqlens. Sequences never share a chunk; the state
 *    resets to h0[n] at each sequence start.
 *  - Grouped value heads: HV value heads, H query/key heads, HV % H == 0; value head h
 *    reads q/k head h / (HV / H). g and beta are per value head.
 *  - Element types: q, k, v, dO, h0, dS_final, states, inv, o, dq, dk, dv use `dtype`
 *    (fp32 or bf16, converted with round-to-nearest-even). g, beta, dg, dbeta, dh0 and
 *    final_state are fp32.
 *  - Errors: no exception crosses the ABI. Arguments are validated before any HIP call;
 *    a failed check returns KDA_EINVAL or KDA_EUNSUPPORTED with a message available from
 *    kda_last_error() (thread-local). A failed kernel launch returns KDA_EHIP. Kernel
 *    faults surface asynchronously on the stream, as for any HIP work.
 *  - Supported (dtype, K, V, C): (F32, 16, 16, 16), (BF16, 128, 128, 64), (BF16, 128, 128, 16).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KDA_OK = 0, KDA_EINVAL = -1, KDA_EUNSUPPORTED = -2, KDA_EHIP = -3 } kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

typedef struct {
    int32_t B;        /* dense batch size; 1 when cu_seqlens is given                       */
    int32_t T;        /* tokens per sequence (dense) or total tokens (packed); >= 0          */
    int32_t H;        /* query/key heads                                                      */
    int32_t HV;       /* value heads (multiple of H)                                          */
    int32_t K;        /* key dimension (rows of the state)                                    */
    int32_t V;        /* value dimension (columns of the state)                               */
    int32_t C;        /* chunk size. The chunk kernels take each gate factor e^(G_i - G_j)
                         (G: chunk-local cumsum of g) relative to the first row of the
                         16-row block holding i or j, in fp32 and bf16: the gates of the 15
                         tokens after any block's first row must sum to more than about -85
                         (per-token gates >= -5.6 always are; no guard, beyond it results are
                         not finite). The sum over a whole chunk is not limited.             */
    int32_t N;        /* number of sequences: B when dense, len(cu_seqlens) - 1 when packed   */
    const int32_t* cu_seqlens_dev;   /* [N+1] device copy, or NULL when dense                 */
    const int32_t* cu_seqlens_host;  /* [N+1] host copy with the same values (sizes the grids
                                        with no device synchronisation), or NULL when dense.
                                        Non-decreasing, cu[0] = 0, cu[N] = T; empty sequences
                                        are allowed.                                          */
    float scale;      /* output scale (1/sqrt(K) in the usual parameterisation)               */
    int32_t dtype;    /* kda_dtype                                                            */
    int32_t beta_logits; /* 0: beta holds the write strengths in (0, 1). 1: beta holds their
                            logits; every kernel takes beta = sigmoid(logit) (the FlashKDA
                            backward page loads raw beta and applies a sigmoid), and
                            kda_chunk_bwd's dbeta is the gradient w.r.t. the logits,
                            dbeta * beta (1 - beta). Other values: KDA_EINVAL.              */
} kda_dims;

/* Total number of chunks NT = sum_n ceil(len_n / C); -1 if dims are invalid. Valid dims have
 * NT <= 2^30 and NT * HV + 8 HV / H <= 2^31 - 1 (the kernels launch one workgroup per chunk and
 * head, rounded up to whole runs of 8 q/k groups). */
int64_t kda_num_chunks(const kda_dims* dims);

/* Workspace bytes needed by kda_fwd_states / kda_chunk_bwd; 0 if dims are invalid. The
 * workspace must be 256-byte aligned device memory of at least this size. Its contents
 * need no initialisation and are meaningless after the call. */
size_t kda_fwd_workspace_bytes(const kda_dims* dims);
size_t kda_bwd_workspace_bytes(const kda_dims* dims);

/*
 * Forward chunk states (the forward of the chunkwise KDA; FLA page:
 * recompute_w_u_fwd + chunk_gated_delta_rule_fwd_h; FlashKDA page: the workspace the
 * backward consumes, INV and S_in per chunk).
 *   q        [B,T,H,K]  dtype   needed only when o != NULL (may be NULL otherwise)
 *   k        [B,T,H,K]  dtype
 *   v        [B,T,HV,V] dtype
 *   g        [B,T,HV,K] fp32    per-token natural-log decay (g <= 0 in practice)
 *   beta     [B,T,HV]   fp32    write strength, or its logit when dims->beta_logits = 1
 *   h0       [N,HV,K,V] dtype   initial state, NULL = zero
 * outputs:
 *   states   [NT,HV,K,V] dtype  S_in of every chunk (the state entering the chunk), chunks
 *                               numbered sequence by sequence
 *   inv      [NT,HV,C,C] dtype  INV of every chunk; rows/columns past a partial chunk's
 *                               end hold the identity
 *   final_state [N,HV,K,V] fp32 S_T, NULL = not written
 *   o        [B,T,HV,V] dtype   o_t = scale S_t^T q_t, NULL = not computed
 */
kda_status kda_fwd_states(const kda_dims* dims, const void* q, const void* k, const void* v,
                          const float* g, const float* beta, const void* h0,
                          void* states, void* inv, float* final_state, void* o,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * Chunkwise backward (FLA page: chunk_kda_bwd -- dAv, bwd_dhu, wy_dqkg_fused, intra, the
 * GVA reduction and the reverse chunk-local cumsum of dg; FlashKDA page: the per-chunk
 * reverse walk that recomputes U, forms dU, dvcorr, dL, dMqk, dv, dbeta and the key/query
 * gradients, and stores the initial-state gradient).
 *   q, k     [B,T,H,K]  dtype
 *   v        [B,T,HV,V] dtype
 *   g        [B,T,HV,K] fp32
 *   beta     [B,T,HV]   fp32
 *   states   [NT,HV,K,V] dtype  S_in per chunk, as written by kda_fwd_states
 *   inv      [NT,HV,C,C] dtype  INV per chunk, as written by kda_fwd_states
 *   dO       [B,T,HV,V] dtype   gradient w.r.t. o
 *   dS_final [N,HV,K,V] dtype   gradient w.r.t. the final state, NULL = zero
 * outputs (each fully overwritten):
 *   dq, dk   [B,T,H,K]  dtype   summed over the value heads of each group
 *   dv       [B,T,HV,V] dtype
 *   dg       [B,T,HV,K] fp32    gradient w.r.t. the per-token g
 *   dbeta    [B,T,HV]   fp32    gradient w.r.t. beta as given: the strength itself, or its
 *                               logit when dims->beta_logits = 1
 *   dh0      [N,HV,K,V] fp32    gradient w.r.t. h0, NULL = not written
 */
kda_status kda_chunk_bwd(const kda_dims* dims, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const void* states, const void* inv,
                         const void* dO, const void* dS_final,
                         void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dh0,
                         void* workspace, size_t ws_bytes, void* stream);

/*
 * Saved-operand mode (FLA chunk_kda_bwd page: its disable_recompute switch, under which the
 * backward takes the w, u and state tensors the forward kept instead of recomputing them):
 * the forward also writes, per chunk, what kda_chunk_bwd's first kernel would otherwise
 * recompute from q, k, g, beta and INV -- kr = k e^(gam - G), -w^T with
 * w = INV diag(beta) (k e^G), Q'^T with Q' = qd - Mqk w, and e^gam -- and the backward
 * reads them. Same results as kda_fwd_states + kda_chunk_bwd (up to fp32 rounding order in
 * Q'); the backward no longer runs its prep kernel (where its reverse scan takes W = Q'^T dO
 * precomputed, a smaller kernel forms W from the saved Q'^T), the forward writes the extra
 * tensors (48.5 KB per chunk and value head at K = V = 128, C = 64).
 *
 * kda_saved_bytes: size of the `saved` buffer (a caller-owned device buffer, 256-byte
 * aligned; contents opaque, valid for the dims, inputs and states it was written with);
 * 0 if dims are invalid.
 */
size_t kda_saved_bytes(const kda_dims* dims);

/*
 * kda_fwd_states that also fills `saved`. Arguments as kda_fwd_states, except that q and o
 * are required (the save's Q' is formed beside o). Errors: KDA_EINVAL for a NULL, short or
 * misaligned `saved`, or a NULL q or o (when the dims have at least one chunk).
 */
kda_status kda_fwd_states_save(const kda_dims* dims, const void* q, const void* k, const void* v,
                               const float* g, const float* beta, const void* h0,
                               void* states, void* inv, float* final_state, void* o,
                               void* saved, size_t saved_bytes,
                               void* workspace, size_t ws_bytes, void* stream);

/*
 * kda_chunk_bwd reading `saved` as written by kda_fwd_states_save for the same dims and
 * inputs. Arguments and outputs as kda_chunk_bwd (same workspace size); q, k, g, beta and
 * inv are still read by its gradient kernel. Errors as kda_chunk_bwd, plus KDA_EINVAL for a
 * NULL, short or misaligned `saved`.
 */
kda_status kda_chunk_bwd_saved(const kda_dims* dims, const void* q, const void* k, const void* v,
                               const float* g, const float* beta, const void* states, const void* inv,
                               const void* saved, size_t saved_bytes,
                               const void* dO, const void* dS_final,
                               void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dh0,
                               void* workspace, size_t ws_bytes, void* stream);

/* Message describing the last non-OK status returned on this thread ("" if none). */
const char* kda_last_error(void);

/*
 * kda_chunk_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same computation and
 * arguments without `workspace` / `ws_bytes`. The workspace is a device array inside the
 * library, KDA_NOALLOC_MAX_WORKSPACE bytes per GPU, held from the library's load until the
 * process ends; the call itself allocates nothing. A call whose kda_bwd_workspace_bytes
 * exceeds that size returns KDA_EINVAL (before any HIP work). All calls on one GPU share
 * its array, so calls that overlap on one GPU (different streams or threads) race: order
 * them on one stream. Its first call on a device looks the array's address up on that
 * device (which must be current, as for every call).
 */
#define KDA_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
kda_status kda_chunk_bwd_noalloc(const kda_dims* dims, const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const void* states, const void* inv,
                                 const void* dO, const void* dS_final,
                                 void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dh0,
                                 void* stream);


#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
