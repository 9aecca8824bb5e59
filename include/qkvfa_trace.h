/*
 * qkvfa_trace.h -- measurement build of the library (libqkvfa_trace.so), not
 * part of the attention ABI.
 *
 * libqkvfa_trace.so exports every call of qkvfa.h, built with per-workgroup
 * phase timestamps in the decode kernel, and the one call below.  It is the
 * same code as libqkvfa.so except for the timestamp stores, which cost a few
 * hundredths of a microsecond each; it exists to show where the time of a
 * decode launch goes (the online softmax with the final normalisation by
 * the running maximum and sum, and the cross-split merge -- TurboAttention,
 * arXiv 2412.08585, section 2.2).
 */
#ifndef QKVFA_TRACE_H
#define QKVFA_TRACE_H

#include <stdint.h>

#include "qkvfa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Copy the phase timestamps that workgroups [0, n_wgs) of the most recent
 * decode launch wrote (workgroups 0 .. 4095 record; a launch's workgroup
 * index is split-major: split s, (batch b, KV head g) unit u is workgroup
 * s * B * Hkv + u) into dst, 16 uint64 per workgroup:
 *   [0]  kernel entry            [1] chunk loop start (query converted)
 *   [2 + w] wave w's last chunk done (w < 8)
 *   [10] wave merge done, partial or output written
 *   [11] split ticket drawn (multi-split launches)
 *   [12] workgroup exit          [13] 1 if this workgroup merged the splits
 * Timestamps are s_memrealtime counts (100 MHz, one clock for the device).
 * Slots a launch does not reach keep older values.
 *   dst    host memory of n_wgs * 16 uint64 (written)
 *   n_wgs  0 .. 4096
 * Synchronizes with the device.  Returns QKV_OK, QKV_ERR_INVALID_ARG (null
 * dst, n_wgs out of range) or QKV_ERR_HIP.
 */
qkv_status qkv_trace_read(uint64_t* dst, int64_t n_wgs);

#ifdef __cplusplus
}
#endif

#endif /* QKVFA_TRACE_H */
