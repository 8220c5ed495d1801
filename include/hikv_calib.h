/* hikv_calib.h -- measurement aids for the decode step's roofline (not part
 * of the method): a plain streaming read of a KV cache's live rows, laid out
 * as the decode step reads them, and an empty kernel.  The benchmark times
 * them to report the floor a launch reading the same bytes reaches, and the
 * cost of a dependent launch.  Built as libhikv_calib.so beside libhikv.so.
 *
 * Calls are asynchronous on `stream` (a hipStream_t; NULL: the default
 * stream).  Return codes are those of hikv.h (0 ok, -1 invalid argument,
 * -3 device error).
 */
#ifndef HIKV_CALIB_H
#define HIKV_CALIB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read rows [t0, t1) of unit u from both arrays k and v (device, each
 * [units][cap][row_bytes] bytes, row_bytes a multiple of 16, 16-byte
 * aligned) for every tile of `tiles` (device int32 [n_tiles][3]: u, t0, t1;
 * one workgroup per tile), 16 bytes per lane per load with several loads in
 * flight, and write one word per tile to `sink` (device uint32 [n_tiles]) so
 * that no load is dropped.  ev_start / ev_stop: optional hipEvents (both or
 * neither) the dispatch records when it starts and ends executing. */
int hikv_calib_stream(const void *k, const void *v, int64_t cap, int64_t row_bytes, const int32_t *tiles,
                      int32_t n_tiles, uint32_t *sink, void *ev_start, void *ev_stop, void *stream);

/* n back-to-back launches of an empty kernel (one workgroup each). */
int hikv_calib_empty(int32_t n, void *stream);

#ifdef __cplusplus
}
#endif

#endif
