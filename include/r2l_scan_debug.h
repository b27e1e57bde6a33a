/*
 * r2l_scan_debug.h -- a host-only test aid of libr2l_scan.so (declared apart
 * from the main ABI in r2l_scan.h because no production caller needs it).
 */
#ifndef R2L_SCAN_DEBUG_H_
#define R2L_SCAN_DEBUG_H_

#include "r2l_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct r2l_access_report {
    int64_t launches;   /* kernel launches replayed */
    int64_t accesses;   /* memory accesses checked */
    int64_t vector_staging; /* segment launches that stage Bm/Cm with vector loads
                               (every row start aligned for them) */
    char message[512];  /* the first out-of-bounds access, or "" */
} r2l_access_report;

/*
 * r2l_check_access -- replays on the host every memory access that the call
 * `op` (R2L_OP_*) with these arguments would make on the GPU: the same
 * argument checks, the same plan and launches, the kernels' own index math.
 * Nothing is launched and no pointer is dereferenced: device pointers are
 * compared as numbers against the buffers the arguments describe (a buffer of
 * zero bytes admits no access). For the ragged layout `cu_seqlens_host` is a
 * host copy of the [batch+1] offsets (ignored for the dense layout).
 * Returns the entry point's status when an argument check fails, R2L_OK when
 * every access is in bounds, and R2L_ERR_INVALID_ARG with report->message
 * naming the first access that is not. Callers: the test suite, before a
 * kernel change reaches a GPU.
 */
R2L_API r2l_status r2l_check_access(int32_t op, const r2l_scan_args *a, const int32_t *cu_seqlens_host,
                            r2l_access_report *report);

/*
 * r2l_check_access_backward -- the same replay for r2l_scan_backward
 * (reverse = 1) or prefix_scan_backward (reverse = 0) with these arguments
 * (their checks, their launches, every access), which also requires that
 * each workspace word a launch reads (checkpoints, partial sums) was written
 * by an earlier launch of the call.
 */
R2L_API r2l_status r2l_check_access_backward(int32_t reverse, const r2l_scan_args *fwd,
                                             const r2l_grad_args *grad,
                                             const int32_t *cu_seqlens_host,
                                             r2l_access_report *report);

/*
 * The same replays for r2l_scan_save / prefix_scan_save (reverse 1 / 0; the
 * checkpoints are one more output buffer, and every row the backward reads
 * must be written) and r2l_scan_backward_saved / prefix_scan_backward_saved
 * (the checkpoints an input the replay treats as written).
 */
R2L_API r2l_status r2l_check_access_save(int32_t reverse, const r2l_scan_args *a,
                                         const float *ckpt, size_t ckpt_bytes,
                                         const int32_t *cu_seqlens_host,
                                         r2l_access_report *report);
R2L_API r2l_status r2l_check_access_backward_saved(int32_t reverse, const r2l_scan_args *fwd,
                                                   const r2l_grad_args *grad, const float *ckpt,
                                                   size_t ckpt_bytes,
                                                   const int32_t *cu_seqlens_host,
                                                   r2l_access_report *report);

/*
 * r2l_check_access_bidir -- the same replay for bidir_scan with these
 * arguments (the workspace's fp32 rows that the forward pass adds must have
 * been written by the reverse pass).
 */
R2L_API r2l_status r2l_check_access_bidir(const r2l_scan_args *a, const r2l_dir_args *rev,
                                          const int32_t *cu_seqlens_host,
                                          r2l_access_report *report);

/*
 * r2l_check_access_sidecar -- the same replay for r2l_sidecar_forward: every
 * access of its own kernels (conv, scan, residual copy) and, for each library
 * GEMM, that every matrix it is given lies inside its buffer.
 */
R2L_API r2l_status r2l_check_access_sidecar(const r2l_sidecar_args *a,
                                            const int32_t *cu_seqlens_host,
                                            r2l_access_report *report);

typedef struct r2l_plan_info {
    int32_t lanes_per_channel; /* 1, 2 or 4 */
    int32_t chunked;           /* 1: chunk pass + carry (+ readout pass) */
    int64_t chunk_tokens;      /* tokens per chunk (the longest sequence when not chunked) */
    int64_t chunks;            /* chunks per sequence in the grid */
    int64_t workspace_bytes;
    int32_t launches;          /* kernel launches the call makes */
} r2l_plan_info;

/*
 * r2l_describe_plan -- the plan the library picks for call `op` with these
 * arguments (only the shape fields and planning hints are read). For
 * benchmark reports and tests. Returns R2L_OK or a shape-check status.
 */
R2L_API r2l_status r2l_describe_plan(int32_t op, const r2l_scan_args *a, r2l_plan_info *info);

#ifdef __cplusplus
}
#endif

#endif /* R2L_SCAN_DEBUG_H_ */
