/*
 * Phase trace of the verification attention kernel, in the trace build of
 * the library only (libdustin_trace.so: `python -m sparse_kv_verification_amd.build
 * --trace`, sources compiled with DUSTIN_ATTN_TRACE).  The library proper
 * exports none of this and its kernels record nothing.
 *
 * Thread 0 of every work-group of the bf16 attention kernel writes eight
 * 64-bit words per launch: the 100 MHz real-time counter at kernel entry,
 * when the row table is ready, when the first K/V tile has landed, at the
 * end of the token loop, after the split partial is stored, after the split
 * handshake and at exit, then (path | XCD << 8), path 0 = one split, 1 =
 * merged at once, 2 = merged after arriving last, 3 = published only.
 * Launch l (counted from the last restart) fills row l mod 80 of a
 * [80][1024][8] array; work-groups past 1024 are not recorded.
 */
#ifndef DUSTIN_TRACE_H
#define DUSTIN_TRACE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Copy the whole trace array (80 * 1024 * 8 * 8 bytes) to host memory;
 * returns a hipError_t code (0 on success). */
int dustin_trace_attn_read(void *host_dst, size_t bytes);

/* The next attention launch fills row 0 again. */
void dustin_trace_attn_restart(void);

#ifdef __cplusplus
}
#endif

#endif /* DUSTIN_TRACE_H */
