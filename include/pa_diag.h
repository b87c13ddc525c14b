/*
 * pa_diag.h -- diagnostics of libpagedattn.so (not part of the paged-attention method).
 *
 * pa_diag_read_bandwidth measures the HBM read rate this GPU actually sustains for the access
 * pattern of the paged kernels, so that their roofline fraction can also be read against a
 * measured ceiling and not only against the published 8 TB/s.
 */
#ifndef PA_DIAG_H
#define PA_DIAG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `num_tiles` tiles of `tile_bytes` bytes each from device buffer `buf` with 16-byte loads
 * and folds them into `sink` (device, >= 64 * 1024 uint32 words, overwritten) so the loads cannot
 * be elided. Tile i is tile tile_order[i] of the buffer (device int32 [num_tiles], every entry in
 * [0, buffer_tiles)); tile_order == NULL reads the tiles in address order. One wave64 reads one
 * tile at a time, like the attention kernels read one (block, head) tile.
 *   tile_bytes: 1, 2, 4, 8 or 16 KiB (else PA_ERR_UNSUPPORTED); num_tiles > 0; buffer_tiles >=
 *   num_tiles when tile_order is NULL. Returns a pa_status value; enqueues on `stream` only.
 */
int pa_diag_read_bandwidth(const void* buf, size_t buffer_tiles, const int32_t* tile_order,
                           int num_tiles, int tile_bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_DIAG_H */
