/*
 * specverify profiling entry points -- for benchmarks, not for serving.
 *
 * Each *_profiled call below is the call of the same name in specverify.h
 * with one more leading argument, `events`.  When `events` is non-NULL, the call records
 * events->start on its stream right before the launch of its streaming pass
 * (the kernel that reads every logit row once) and events->stop right after
 * it, so that hipEventElapsedTime(start, stop) is that kernel's duration.
 * With events == NULL a call is exactly its plain counterpart.
 *
 * The events are created by the caller (hipEventCreate) and only recorded
 * here.  Nothing is kept between calls: every call reads the events it is
 * given, so concurrent calls on different streams with their own events
 * and workspaces are safe, as for the plain calls.
 *
 * Arguments, results and errors are those of the plain calls; a call that
 * launches no streaming pass (workspace query, empty draft) records nothing.
 */
#ifndef SPECVERIFY_PROFILE_H
#define SPECVERIFY_PROFILE_H

#include "specverify.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    hipEvent_t start; /* recorded right before the streaming pass */
    hipEvent_t stop;  /* recorded right after it                  */
} sv_profile_events_t;

SV_API sv_status_t spec_verify_sample_profiled(const sv_profile_events_t* events, const sv_shape_t* shape,
                                               const void* target_logits, const void* draft_logits,
                                               const int32_t* draft_ids, float temperature, int32_t top_k,
                                               float top_p, uint64_t seed, uint32_t offset, int32_t* out_tokens,
                                               int32_t* out_num_accepted, float* out_probs,
                                               float* out_residual_mass, void* workspace, size_t* workspace_bytes,
                                               hipStream_t stream);

SV_API sv_status_t spec_verify_argmax_profiled(const sv_profile_events_t* events, const sv_shape_t* shape,
                                               const void* target_logits, const void* draft_logits,
                                               const int32_t* draft_ids, float temperature, int32_t top_k,
                                               float top_p, uint64_t seed, uint32_t offset, int32_t* out_tokens,
                                               int32_t* out_num_accepted, float* out_probs,
                                               float* out_residual_mass, void* workspace, size_t* workspace_bytes,
                                               hipStream_t stream);

SV_API sv_status_t spec_verify_greedy_profiled(const sv_profile_events_t* events, const sv_shape_t* shape,
                                               const void* target_logits, const int32_t* draft_ids,
                                               int32_t* out_tokens, int32_t* out_num_accepted, void* workspace,
                                               size_t* workspace_bytes, hipStream_t stream);

SV_API sv_status_t spec_draft_sample_profiled(const sv_profile_events_t* events, const sv_shape_t* shape,
                                              const void* draft_logits, float temperature, int32_t top_k,
                                              float top_p, uint64_t seed, uint32_t offset, int32_t* out_ids,
                                              void* workspace, size_t* workspace_bytes, hipStream_t stream);

SV_API sv_status_t spec_token_likelihood_profiled(const sv_profile_events_t* events, const sv_shape_t* shape,
                                                  const void* target_logits, const void* draft_logits,
                                                  const int32_t* tokens, float temperature, int32_t top_k,
                                                  float top_p, float* out_terms, float* out_beta, double* out_nll,
                                                  void* workspace, size_t* workspace_bytes, hipStream_t stream);

/*
 * A plain streaming read, the practical roof the streaming passes are
 * measured against: every 16-byte block of [data, data + bytes) is loaded
 * once, with the nontemporal 16-byte loads and the tile shape of the top-k
 * candidate pass (256 threads per workgroup, 6 loads per thread, one tile per
 * workgroup), and nothing is computed from it.  data: device memory, 16-byte
 * aligned; bytes: a positive multiple of 16.  sink: device memory of 4 bytes,
 * written only when the xor of a thread's words equals 0x9E3779B9 (this keeps
 * the loads; its content has no meaning).  events as above, recorded around
 * the read.  SV_ERR_INVALID_ARGUMENT for a null or misaligned pointer or a
 * bad size.
 */
SV_API sv_status_t spec_profile_stream_read(const sv_profile_events_t* events, const void* data, size_t bytes,
                                            uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_PROFILE_H */
