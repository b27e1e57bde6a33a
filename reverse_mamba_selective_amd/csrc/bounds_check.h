// bounds_check.h -- host replay of the kernels' memory accesses (internal).
#pragma once

#include "r2l_scan_debug.h"
#include "scan_plan.h"

namespace r2l {

// Checks every access of the launches of (op, a, pl); the arguments must have
// passed the entry point's checks. cu_host: host copy of cu_seqlens (ragged).
// ckpt: a saving forward (r2l_scan_save; pl made with ckpt = true), whose
// checkpoints must cover every row the backward reads.
r2l_status check_accesses(Op op, const r2l_scan_args *a, const Plan &pl, const int32_t *cu_host,
                          r2l_access_report *rep, float *ckpt = nullptr, size_t ckpt_bytes = 0);

// The same for r2l_scan_backward (after its checks); saved: the checkpoints of
// r2l_scan_backward_saved (pl made with saved = true).
r2l_status check_backward_accesses(bool reverse, const r2l_scan_args *a, const r2l_grad_args *g,
                                   const BwdPlan &pl, const int32_t *cu_host, r2l_access_report *rep,
                                   const float *saved = nullptr, size_t saved_bytes = 0);

// The same for bidir_scan (after its checks).
r2l_status check_bidir_accesses(const r2l_scan_args *a, const r2l_dir_args *rev, const BidirPlan &bp,
                                const int32_t *cu_host, r2l_access_report *rep);

// The same for r2l_sidecar_forward (after its checks).
r2l_status check_sidecar_accesses(const r2l_sidecar_args *a, const SidecarPlan &sp,
                                  const int32_t *cu_host, r2l_access_report *rep);

}  // namespace r2l
