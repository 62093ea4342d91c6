/*
 * ccv_calib.h -- measurement aids shipped beside libccv (libccv_calib.so).
 *
 * These are not part of the conv method; the pages define no such operation.
 * They give the bench reference points on the same GPU: a streaming copy (what a
 * kernel that reads N bytes once and writes N bytes once can reach, and the
 * factor that turns the FETCH_SIZE / WRITE_SIZE counters into bytes), a
 * read-only sweep (the second half of a cache flush, which leaves the caches
 * holding clean lines), and an empty kernel (the launch floor).
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
 * multiple of 16; the ranges must not overlap.  Each wave instruction moves 1 KB
 * of consecutive bytes.  waves_per_cu > 0: a grid of that many waves per CU
 * (256 CUs) walks the buffer in 4 KB chunks; <= 0: one wave per chunk.
 * nontemporal != 0: streaming (non-temporal) loads and stores. */
int ccv_calib_copy_ex(void* dst, const void* src, int64_t nbytes, int32_t waves_per_cu,
                      int32_t nontemporal, void* hip_stream);

/* ccv_calib_copy_ex with 16 waves per CU and non-temporal accesses. */
int ccv_calib_copy(void* dst, const void* src, int64_t nbytes, void* hip_stream);

/* Reads src[0:nbytes) once with ordinary cached loads (16-byte aligned, nbytes a
 * multiple of 16).  sink: device buffer of 64 uint32, written only in the
 * unlikely case that a wave's xor of its data equals `key`. */
int ccv_calib_read(const void* src, int64_t nbytes, uint32_t key, void* sink, void* hip_stream);

/* One workgroup of one wave that does nothing. */
int ccv_calib_empty(void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif
