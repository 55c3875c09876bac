/*
 * cpattn_diag -- diagnostics of libcpattn.so that are not part of the method.
 *
 * The pages describe no such call.  It exists to measure the shader clock the
 * forward step kernel runs at (the chip throttles under load), so that a
 * throughput figure can be read against the clock it was reached at.
 */
#ifndef CPATTN_DIAG_H
#define CPATTN_DIAG_H

#include "cpattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* While dev_buf (device memory of `capacity` uint64 values) is set, every
 * forward step launch (cp_attn_fwd_step, cp_attn_fwd_step_merge) records, for
 * each of its first capacity / 4 workgroups b, four values at
 * dev_buf[4b .. 4b+3]: the shader cycle counter and the constant 100 MHz
 * counter when the workgroup starts, then the same two when it ends; the ratio
 * of the differences gives the shader clock the work ran at.  Each launch
 * overwrites the records of its workgroups.  NULL (the default) turns
 * recording off.
 * PROCESS-WIDE STATE: the setting applies to every thread and stream of the
 * process and is read at each launch; the caller keeps dev_buf alive while it
 * is set.  With it off, the kernels take one extra scalar branch per workgroup
 * and write nothing.
 * Returns CP_ERR_INVALID_ARG for a non-NULL buffer with capacity < 4. */
cp_status cp_debug_clock_probe(uint64_t* dev_buf, int64_t capacity);

#ifdef __cplusplus
}
#endif
#endif /* CPATTN_DIAG_H */
