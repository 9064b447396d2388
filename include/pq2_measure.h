/*
 * pq2_measure.h -- measurement probes of libpq2: the read ceilings and the
 * launch floor that the matmuls are timed against.
 *
 * Page "Kernel experiments: recorded evidence", section H, Test 24 timed
 * copy-free read patterns of the weight layouts against a linear stream to
 * separate what an access pattern allows from what a kernel's work costs.
 * These probes do the same on gfx950: the decode engines' own weight loads
 * (pq2_read_probe), a linear stream shaped like no engine
 * (pq2_stream_probe, and pq2_stream_probe_cfg with the grid, loads in flight
 * and load instruction as parameters), and an empty kernel
 * (pq2_empty_probe), whose cost per
 * launch in a graph of back-to-back launches is the floor under any kernel.
 * Conventions (device pointers, void* stream, validation before any HIP
 * call, status codes) are those of pq2.h.
 */
#ifndef PQ2_MEASURE_H
#define PQ2_MEASURE_H

#include "pq2.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read-only probe of a prepared weight layout (page "Kernel experiments",
 * section H, Test 24: copy-free read patterns of the layouts, the ceiling
 * the matmuls are measured against).  It issues exactly the weight loads of
 * the decode engine that reads the layout (planes: the packed-dot engine;
 * tiles: the tile-layout engine): same grid, waves, k split, load widths and
 * cache policy, one segment at a time, and no arithmetic but an XOR fold of
 * what each wave read.  Every byte is read once, so the XOR of the output
 * words equals the XOR of the layout's dwords (for the planes: the code
 * plane's dwords and the fp16 scales, each zero-extended).
 *   weights  device planes (layout PQ2_LAYOUT_PLANES) or tile layout
 *            (PQ2_LAYOUT_TILES) of an n x k matrix, 16-byte aligned.
 *   out      device uint32 [pq2_read_probe_words(layout, n, k)], 4-byte
 *            aligned, fully overwritten; must not overlap the weights.
 * Errors: EINVAL (null, layout, overlap), ESHAPE (n < 1, k < 128, k % 128,
 *         k > PQ2_MAX_K), EALIGN, ELAUNCH, EDEVICE. */
int pq2_read_probe(const void* weights, int layout, int64_t n, int64_t k, uint32_t* out, void* stream);

/* Number of uint32 words pq2_read_probe writes for this layout and shape
 * (one per wave of its grid); 0 for an invalid layout or shape.  Host only. */
int64_t pq2_read_probe_words(int layout, int64_t n, int64_t k);

/* Linear streaming read of `bytes` bytes at buf: `workgroups` workgroups of 4
 * waves walk the buffer grid-stride in 1 KB wave chunks (iteration i,
 * workgroup w, wave v reads chunk (i * workgroups + w) * 4 + v), one 16-byte
 * non-temporal load per lane, and fold what they read with XOR.  Reads past
 * the end return zero.
 *   buf        device, bytes >= 16, a multiple of 16 and < 2^31; 16-byte aligned.
 *   workgroups 1..65536 (512-4096 are the fastest measured for 8-200 MB).
 *   store_all  nonzero: every wave writes its fold to out[wave], and the XOR
 *              of all pq2_stream_probe_words(workgroups) words equals the XOR
 *              of the buffer's dwords.  Zero: a lane writes its own fold to
 *              out[wave] only if it equals `sentinel` (practically never: a
 *              timed run is then a pure read; any output store adds the
 *              latency of one store to the launch).
 *   out        device uint32 [pq2_stream_probe_words(workgroups)], 4-byte
 *              aligned; must not overlap buf.
 * Errors: EINVAL (null, overlap), ESHAPE (bytes, workgroups), EALIGN,
 *         ELAUNCH, EDEVICE. */
int pq2_stream_probe(const void* buf, int64_t bytes, int64_t workgroups, int store_all, uint32_t sentinel,
                     uint32_t* out, void* stream);

/* Words pq2_stream_probe writes: 4 per workgroup; 0 for workgroups outside
 * 1..65536.  Host only. */
int64_t pq2_stream_probe_words(int64_t workgroups);

/* Load instruction and cache policy of pq2_stream_probe_cfg. */
enum {
    PQ2_STREAM_BUFFER = 0,    /* buffer_load_dwordx4 into registers, default cache policy */
    PQ2_STREAM_BUFFER_NT = 1, /* the same, non-temporal (what pq2_stream_probe uses) */
    PQ2_STREAM_LDS = 2,       /* global_load_lds_dwordx4 straight into LDS, default policy */
    PQ2_STREAM_LDS_NT = 3     /* the same, non-temporal */
};

/* The linear stream read of pq2_stream_probe with its shape as parameters, to
 * map the read ceiling against waves per SIMD, loads in flight per lane and
 * the load instruction (page "Kernel experiments", section H, Test 24: read
 * patterns timed without the kernel's work).  `workgroups` workgroups of
 * `waves` waves walk the buffer grid-stride in wave chunks of
 * `loads_per_lane` KB: iteration i, workgroup w, wave v reads the
 * loads_per_lane consecutive 1 KB blocks from block ((i * workgroups + w) *
 * waves + v) * loads_per_lane, one 16-byte load per lane per block, all of
 * an iteration's loads issued before any is used.  The LDS policies load
 * into a per-wave LDS slot of loads_per_lane KB (dynamic LDS of waves x
 * loads_per_lane KB per workgroup) and read each 16 bytes back once they
 * have landed.  Each wave folds what it read with XOR; blocks past the end
 * read zero.
 *   buf            device, 16-byte aligned; bytes >= 16, a multiple of 16
 *                  (of 1024 for the LDS policies) and < 2^31.
 *   workgroups     1..65536; waves 1..16; loads_per_lane 1, 2, 4, 8 or 16,
 *                  with waves x loads_per_lane <= 64 and workgroups x waves
 *                  x loads_per_lane x 1024 <= 2^30 (one iteration's span).
 *   policy         PQ2_STREAM_*.
 *   store_all      as for pq2_stream_probe: nonzero, every wave writes its
 *                  fold to out[wave] (workgroup w, wave v: w * waves + v) and
 *                  the XOR of all workgroups x waves words is the XOR of the
 *                  buffer's dwords; zero, a lane writes only if its own fold
 *                  equals `sentinel` (a pure read when timed).
 *   out            device uint32 [workgroups x waves], 4-byte aligned; must
 *                  not overlap buf.
 * Errors: EINVAL (null, policy, overlap), ESHAPE (bytes, workgroups, waves,
 *         loads_per_lane and their limits), EALIGN, ELAUNCH, EDEVICE. */
int pq2_stream_probe_cfg(const void* buf, int64_t bytes, int64_t workgroups, int waves, int loads_per_lane,
                         int policy, int store_all, uint32_t sentinel, uint32_t* out, void* stream);

/* An empty kernel of `workgroups` (1..2^20) workgroups of `waves` (1..16)
 * waves that touches no memory: timed as a graph of back-to-back launches it
 * gives the launch floor.  Errors: ESHAPE, ELAUNCH, EDEVICE. */
int pq2_empty_probe(int64_t workgroups, int waves, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PQ2_MEASURE_H */
