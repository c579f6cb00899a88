/*
 * kda_measure.h -- measurement and inspection extension of the KDA chunk library (not
 * part of the operation's interface in kda.h; nothing in the computation depends on it).
 *
 * Per-kernel timing. While `events` is non-NULL, every kda_fwd_states / kda_chunk_bwd call made on the calling
 * thread records, on its stream, events[2*i] right before and events[2*i+1] right after its
 * i-th kernel launch, for i < count / 2, so that a caller can time each kernel with
 * hipEventElapsedTime. The handles are hipEvent_t values created by the caller; the array
 * must stay valid while it is set (the library keeps the pointer in thread-local storage).
 * Launch order of kda_chunk_bwd: [chunk table, packed sequences only], backward preparation,
 * reverse state-gradient scan, chunk gradients. Of kda_fwd_states: [chunk table], forward
 * preparation, forward state scan, [output o]. Pass NULL (or count 0) to stop recording.
 */
#ifndef KDA_MEASURE_H
#define KDA_MEASURE_H

#include "kda.h"

#ifdef __cplusplus
extern "C" {
#endif

void kda_set_kernel_events(void* const* events, int count);

/*
 * Inspection of a backward stage (FlashKDA backward page, step 2: the state gradient each
 * chunk's products consume). After a kda_chunk_bwd call made with `workspace` (and before
 * that workspace is reused), writes the gradient w.r.t. every chunk's outgoing state --
 * dS_out of chunk c, which the reverse scan carried into it -- as plain fp32
 * dstates[NT, HV, K, V] (row-major, chunks numbered as in kda.h), enqueued on `stream`.
 * `dims`, `workspace` and `ws_bytes` are those of that call; dstates is caller-owned device
 * memory. Validation as for kda_chunk_bwd (KDA_EINVAL / KDA_EUNSUPPORTED before any HIP
 * call, KDA_EHIP for a failed launch).
 */
kda_status kda_bwd_state_grads(const kda_dims* dims, const void* workspace, size_t ws_bytes, float* dstates,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_MEASURE_H */
