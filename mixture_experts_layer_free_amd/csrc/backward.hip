// Backward of the routed MoE layer (placeholder until the kernels land).
#include "moe_common.h"

size_t moe_backward_workspace(int64_t T, int k, int E, int64_t d, int64_t f) { return 0; }

extern "C" moe_status moe_backward(const moe_bwd_args* a, void* stream) { return MOE_ENOTSUP; }
