/*
 * pq2_tuning.h -- tuning hooks of libpq2 (benchmarks and tests).
 *
 * Each hook takes the arguments of the pq2.h entry point it is named after
 * plus explicit kernel settings (0 = the library's choice), validates them
 * the same way, and returns the same status codes; an unsupported setting is
 * PQ2_EINVAL.  The settings choose among kernels that compute the same
 * definition; where a setting changes the summation order, the comment says
 * so.  Conventions (device pointers, void* stream, no allocation, no
 * synchronisation, validation before any HIP call) are those of pq2.h.
 */
#ifndef PQ2_TUNING_H
#define PQ2_TUNING_H

#include "pq2.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Tuning hook for the small-m matmul (benchmarks and tests only; same
 * arguments and result as pq2_matmul_small_m).  engine selects one of four
 * kernels that compute the same bits:
 *   1 = packed dot products (v_dot4), `rows` = weight rows per lane (1, 2);
 *   2 = INT8 matrix cores (v_mfma), one 8-row block per workgroup, `rows` = 1;
 *   3 = INT8 matrix cores, one 8-wave workgroup per CU that stages the
 *       activations of its k range once in LDS for `rows` 8-row blocks;
 *       its waves take the (row block, k slice) units in turn;
 *   4 = the kernel of engine 3 with one unit per wave: `rows` 8-row blocks
 *       per workgroup, one wave per (row block, k slice).
 *   Engines 3 and 4 cover at most 4 columns per pass over the weights and
 *   accept only the `rows` whose staging fits LDS and the wave limits.
 * max_waves in 1..8 is the number of waves that split k inside one
 * workgroup.  0 for any setting picks the library's default (with an
 * explicit engine, that engine's default rows).  The summation order of an
 * output depends on max_waves only (through the number of waves k is split
 * over): neither rows nor the engine changes the bits.  Errors as
 * pq2_matmul_small_m, plus EINVAL for an unsupported setting. */
int pq2_matmul_small_m_tuned(const int8_t* q, const float* xs, const void* planes, int64_t m,
                             int64_t n, int64_t k, float* y, int rows, int max_waves,
                             int engine, void* stream);

/* Tuning hook for pq2_matmul_small_m_planes (benchmarks and tests only; same
 * arguments and result): settings as for pq2_matmul_small_m_tuned, and the
 * same bits as pq2_matmul_small_m_tuned with the same settings.  Errors as
 * pq2_matmul_small_m_planes, plus EINVAL for an unsupported setting. */
int pq2_matmul_small_m_planes_tuned(const int8_t* qp, const float* xs, const int32_t* qsum, const void* planes,
                                    int64_t m, int64_t n, int64_t k, float* y, int rows,
                                    int max_waves, int engine, void* stream);

/* Tuning hook for pq2_matmul_small_m_fused (benchmarks and tests only):
 * settings as for pq2_matmul_small_m_tuned, and the same bits as
 * pq2_quantize_act_i8 + pq2_matmul_small_m_tuned with the same settings.
 * Errors as pq2_matmul_small_m_fused, plus EINVAL for an unsupported
 * setting. */
int pq2_matmul_small_m_fused_tuned(const void* x, int dtype, int64_t x_row_stride_elems, const void* planes,
                                   int64_t m, int64_t n, int64_t k, float* y, int rows, int max_waves,
                                   int engine, void* stream);

/* Tuning hook for pq2_matmul_small_m_tiles (benchmarks and tests only):
 * max_waves in 1..16 fixes the k split (segments of 8 groups over at most
 * max_waves waves, as pq2_matmul_small_m_tuned does for 1..8; the default is
 * 16); split in {1, 2, 4} is the number of waves that share one k slice
 * (each takes 8/split of its group classes), with at most 16 waves per
 * workgroup.  0 for either picks the library's default.  For max_waves <= 8
 * the bits equal pq2_matmul_small_m_tuned's at the same max_waves, whatever
 * the split.
 * Errors as pq2_matmul_small_m_tiles, plus EINVAL for an unsupported
 * setting. */
int pq2_matmul_small_m_tiles_tuned(const int8_t* q, const float* xs, const void* tiles, int64_t m, int64_t n,
                                   int64_t k, float* y, int max_waves, int split, void* stream);

/* Tuning hook for pq2_matmul_small_m_tiles_fused (benchmarks and tests
 * only): max_waves and split as for pq2_matmul_small_m_tiles_tuned, with
 * the same bits as pq2_quantize_act_i8 + pq2_matmul_small_m_tiles_tuned at
 * the same settings.  Errors as pq2_matmul_small_m_tiles_fused, plus EINVAL
 * for an unsupported setting. */
int pq2_matmul_small_m_tiles_fused_tuned(const void* x, int dtype, int64_t x_row_stride_elems, const void* tiles,
                                         int64_t m, int64_t n, int64_t k, float* y, int max_waves, int split,
                                         void* stream);

/* Tuning hook for the prefill matmul (benchmarks and tests only; same
 * arguments and result as pq2_matmul_prefill): tile 1 = 128x128, 2 = 64x128,
 * 3 = 64x64, 4 = 128x64 outputs per workgroup of four waves, 5 = 128x128 on
 * eight waves, 0 = the library's choice.
 * The result does not depend on the tile.  Errors as pq2_matmul_prefill,
 * plus EINVAL for an unknown tile. */
int pq2_matmul_prefill_tuned(const int8_t* q, const float* xs, const void* planes, int64_t m, int64_t n,
                             int64_t k, float* y, int tile, void* stream);

/* Tuning hook for pq2_matmul_prefill_planes (tile as for
 * pq2_matmul_prefill_tuned). */
int pq2_matmul_prefill_planes_tuned(const int8_t* qp, const float* xs, const void* planes, int64_t m, int64_t n,
                                    int64_t k, float* y, int tile, void* stream);

/* Tuning hook for pq2_matmul_prefill_tiles: tile as for
 * pq2_matmul_prefill_tuned (0 = the library's choice), same bits.  Errors as
 * pq2_matmul_prefill_tiles, plus EINVAL for tile outside 0..5. */
int pq2_matmul_prefill_tiles_tuned(const int8_t* q, const float* xs, const void* tiles, int64_t m, int64_t n,
                                   int64_t k, float* y, int tile, void* stream);

/* Split-k tile matmul with at most `waves` (1..16, 0 = the library's choice
 * of 6) waves per workgroup; the k slices are the same (one 1024-element
 * segment each) for every setting, so the bits do not depend on it. */
int pq2_matmul_small_m_tiles_splitk_tuned(const int8_t* q, const float* xs, const void* tiles, int64_t m, int64_t n,
                                          int64_t k, float* y, float* partials, uint32_t* counters, int waves,
                                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PQ2_TUNING_H */
