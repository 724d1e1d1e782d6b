/*
 * rgc_timing.h -- per-kernel timing, exported only by the instrumented build
 * of the library (librgc_timed.so, compiled with RGC_KERNEL_TIMING).  The
 * product library (librgc.so) does not export these calls and keeps no
 * global state; the instrumented build exports everything rgc.h declares,
 * with the same kernels, plus the two calls below.  It is meant for
 * measurement only: it keeps a pool of HIP events, a record guarded by a
 * mutex, and rgc_timing_report waits for the recorded events.
 *
 * While timing is on, every kernel the library launches is bracketed by two
 * HIP events recorded on the stream it runs on, so each kernel's own
 * duration is taken on the device clock apart from the other kernels of the
 * same call (each event pair costs a few microseconds of stream time).
 *   rgc_timing_enable   on != 0 starts recording, 0 stops (what was
 *                       recorded stays until the next report).  Returns 0.
 *   rgc_timing_report   waits for the recorded events, writes one line
 *                       "kernel_name launches total_microseconds\n" per
 *                       kernel into buf (NUL-terminated) and clears the
 *                       record.  Returns the bytes written without the NUL,
 *                       or -10 (RGC_ERR_ARG) when buf is NULL or too small or
 *                       an event could not be read (the record is cleared in
 *                       every case).  Host-thread safe.
 */
#ifndef RGC_TIMING_H
#define RGC_TIMING_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

int rgc_timing_enable(int on);
long rgc_timing_report(char* buf, size_t buf_bytes);

#ifdef __cplusplus
}
#endif

#endif /* RGC_TIMING_H */
