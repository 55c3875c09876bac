// Backward of one Pass-KV ring step (placeholder until the kernel lands).
#include <hip/hip_runtime.h>

#include "internal.h"

using namespace cpattn;

extern "C" cp_status cp_attn_bwd_step(const cp_attn_problem* p, const void* q, const void* k, const void* v,
                                      const void* d_o, const float* lse, const float* delta, float* dq_acc,
                                      float* dk_out, float* dv_out, hipStream_t stream) {
    cp_status st = validate_problem(p, true);
    if (st != CP_OK) return st;
    (void)q; (void)k; (void)v; (void)d_o; (void)lse; (void)delta; (void)dq_acc; (void)dk_out; (void)dv_out;
    (void)stream;
    return fail(CP_ERR_UNSUPPORTED, "backward step not built yet");
}
