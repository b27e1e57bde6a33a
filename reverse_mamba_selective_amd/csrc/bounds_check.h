// bounds_check.h -- host replay of the kernels' memory accesses (internal).
#pragma once

#include "r2l_scan_debug.h"
#include "scan_plan.h"

namespace r2l {

// Checks every access of the launches of (op, a, pl); the arguments must have
// passed the entry point's checks. cu_host: host copy of cu_seqlens (ragged).
r2l_status check_accesses(Op op, const r2l_scan_args *a, const Plan &pl, const int32_t *cu_host,
                          r2l_access_report *rep);

// The same for r2l_scan_backward (after its checks).
r2l_status check_backward_accesses(bool reverse, const r2l_scan_args *a, const r2l_grad_args *g,
                                   const BwdPlan &pl, const int32_t *cu_host, r2l_access_report *rep);

// The same for bidir_scan (after its checks).
r2l_status check_bidir_accesses(const r2l_scan_args *a, const r2l_dir_args *rev, const BidirPlan &bp,
                                const int32_t *cu_host, r2l_access_report *rep);

// The same for r2l_sidecar_forward (after its checks).
r2l_status check_sidecar_accesses(const r2l_sidecar_args *a, const SidecarPlan &sp,
                                  const int32_t *cu_host, r2l_access_report *rep);

}  // namespace r2l
