/*
 * qsa_probe.h -- C ABI of libqsa_probe.so, a measurement aid kept apart
 * from the method's library (libqsa_amd.so, include/qsa.h): one plain
 * streaming read of device memory, whose rate is the practical HBM read
 * ceiling a benchmark reports beside the 8 TB/s peak.  It computes nothing
 * of the QSA path.
 */
#ifndef QSA_PROBE_H_
#define QSA_PROBE_H_

#include <stddef.h>

#include "qsa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * qsa_read_probe -- read `bytes` bytes at `data` (device memory, 16-byte
 * aligned, a multiple of 16 bytes) once, with coalesced nontemporal loads,
 * each workgroup a contiguous span.  `sink` (device, >= 4 aligned bytes, not
 * overlapping `data`) may receive one word.  Asynchronous on `stream`.
 * Returns QSA_OK, QSA_ERR_NULL (data or sink NULL), QSA_ERR_LAYOUT
 * (alignment or size), QSA_ERR_WORKSPACE (sink too small or misaligned),
 * QSA_ERR_ALIAS (sink inside data) or QSA_ERR_LAUNCH; nothing is launched
 * unless QSA_OK or QSA_ERR_LAUNCH.  bytes == 0 is a no-op.
 */
QSA_API int qsa_read_probe(const void* data, size_t bytes, void* sink, size_t sink_bytes,
                           qsa_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_PROBE_H_ */
