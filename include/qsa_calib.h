/*
 * qsa_calib.h - C ABI of libqsa_calib, a measurement aid that is not part of the decode
 * path: a plain device copy whose loads are issued like the indexer scan's (16-byte
 * nontemporal loads, plain stores), and a read of the same kind. Running it next to the scan under a hardware-counter
 * profiler gives the factor between a read or write counter and the bytes actually moved
 * by that kind of load, so the scan's counted traffic can be converted to bytes.
 *
 * Memory, streams and errors follow libqsa's conventions (qsa.h): device pointers, the
 * caller owns both buffers, the call only enqueues work.
 */
#ifndef QSA_CALIB_H_
#define QSA_CALIB_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Copy `bytes` bytes from src to dst on `stream` (a hipStream_t, NULL = null stream).
 * bytes must be a multiple of 16 and both pointers 16-byte aligned; the buffers must not
 * overlap. Returns 0 on success, 1 for a NULL pointer with bytes > 0, 2 for a size or
 * alignment outside the above, 5 if the launch failed.
 */
int qsa_calib_copy(void* dst, const void* src, size_t bytes, void* stream);

/*
 * Read `bytes` bytes of src on `stream` with the same loads and write nothing but one int32
 * to *sink (device), and only if the data happen to fold to a fixed value: the read ceiling
 * of the GPU for that kind of load. Same conditions and return codes as qsa_calib_copy.
 */
int qsa_calib_read(const void* src, size_t bytes, int* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif  // QSA_CALIB_H_
