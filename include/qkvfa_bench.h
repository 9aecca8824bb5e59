/*
 * qkvfa_bench.h -- measurement helper library (libqkvfa_bench.so), not part
 * of the attention ABI.
 *
 * The achievable-HBM leg of the decode roofline: a plain streaming read of a
 * device buffer, so that a decode kernel's bandwidth can be set beside what
 * a kernel that only reads reaches on the same GPU.
 */
#ifndef QKVFA_BENCH_H
#define QKVFA_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` bytes of device memory at `src` once, in 16-byte non-temporal
 * loads (each word is read once: the policy that streams fastest), with
 * `grid` workgroups of 256 threads striding over the buffer in blocks of
 * 16 KiB (each thread keeps four loads in flight), and write one 32-bit XOR
 * of everything each workgroup read to out[blockIdx] (so the loads cannot be
 * elided).
 *   src    device pointer, 16-byte aligned; bytes a multiple of 16
 *   out    device uint32 [grid] (written)
 *   grid   1 .. 65536
 *   stream hipStream_t (NULL = default stream)
 * Returns 0, or a nonzero code (1: invalid argument, 4: HIP launch error);
 * nothing is enqueued on an invalid argument.
 */
int qkvb_stream_read(const void* src, size_t bytes, uint32_t* out, int grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif
