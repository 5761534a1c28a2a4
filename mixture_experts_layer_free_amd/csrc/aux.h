// Internal interface of the auxiliary load-balancing loss (aux.hip) used by
// the backward (backward.hip).
#pragma once

#include "moe_common.h"

size_t moe_aux_workspace(int64_t T, int E);
size_t moe_aux_bwd_workspace(int64_t T, int E, int64_t d);

// Dense router gradient with the auxiliary loss on: dl_dense = aux gradient
// + the chosen experts' dl; dw_router = dl_dense^T x; dx = sum_j
// dx_perm[row_of[t,j]] (bf16 rows; slots with row_of < 0 skipped) + dl_dense w_router (+ extra[t], the shared expert's
// input gradient, when not null).  ws: moe_aux_bwd_workspace bytes.
moe_status moe_aux_backward_launch(const float* logits, const int32_t* counts, const int32_t* idx, const float* dl,
                                   const bf16_t* x, const float* w_router, const u32x4* dx_perm,
                                   const f32x4* extra, const int32_t* row_of, int64_t T, int E, int k, int64_t d, int fn, float alpha,
                                   float* dw_router, float* dx, void* ws, hipStream_t s);
