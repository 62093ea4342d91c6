/*
 * ccv_calib.h -- measurement aids shipped beside libccv (libccv_calib.so).
 *
 * These are not part of the conv method; the pages define no such operation.
 * They give the bench two reference points on the same GPU: a plain streaming
 * copy (what a kernel that reads N bytes once and writes N bytes once can
 * reach, and the factor that turns the FETCH_SIZE / WRITE_SIZE counters into
 * bytes) and an empty kernel (the launch floor).
 *
 * Ownership and errors as in ccv.h: caller-owned device buffers, asynchronous on
 * the given stream, 0 on success, CCV_E_* style negative codes on bad arguments
 * (-1 NULL pointer, -2 bad size or alignment, -8 launch refused).
 */
#ifndef CCV_CALIB_H
#define CCV_CALIB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst[0:nbytes) = src[0:nbytes).  Both pointers 16-byte aligned, nbytes a
 * multiple of 16; the ranges must not overlap. */
int ccv_calib_copy(void* dst, const void* src, int64_t nbytes, void* hip_stream);

/* One workgroup of one wave that does nothing. */
int ccv_calib_empty(void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif
