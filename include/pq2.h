/*
 * pq2.h -- C ABI of the MI355X (gfx950) library for the packed-ternary
 * weight ("PQ2") x group-128 INT8 activation matmul.
 *
 * The method (pages "Kernel experiments: recorded evidence" and "Baseline and
 * the integer breakthrough", series "Making a ternary reasoning model fast in
 * vLLM"):
 *   w[n][k]  = (c[n][k] - 1) * ws[n][k/128]   c in 0..3 (2-bit code), ws fp16
 *   xs[m][g] = max_{i in g} |x[m][i]| / 127    (FP32, one correctly rounded division)
 *   q[m][i]  = clamp(round_half_even(x[m][i] / xs[m][g]), -127, 127)   (divide by 1 if xs == 0)
 *   y[m][n]  = sum_g float(sum_{i in g} q[m][i] * (c[n][i] - 1)) * xs[m][g] * ws[n][g]
 * The per-group integer dot product is exact; each output sums one FP32 term
 * per group.
 *
 * Conventions for every entry point
 *  - Data pointers are DEVICE pointers on the current HIP device; the caller
 *    allocates and owns every buffer.  The library keeps no reference to any
 *    argument after the call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is enqueued asynchronously on it; nothing synchronises the host.
 *  - Arguments are validated on the host BEFORE any HIP call.  A bad argument
 *    returns a status and enqueues nothing.  The library never aborts.
 *  - Values: NaN/Inf activations are unsupported (results are unspecified);
 *    FP32 subnormals are kept (gradual underflow), as on the CPU.
 *
 * Layouts
 *  - Raw PQ2 rows: row n starts at raw + n*raw_row_stride_bytes and holds
 *    k/128 blocks of 34 bytes: bytes 0-1 the block's fp16 scale (IEEE
 *    binary16, little-endian), bytes 2..33 the 32 code bytes.  Weight 4b+s of
 *    the block is bits 2s..2s+1 of code byte b (lowest bits first); code c
 *    stands for c-1 (page "Kernel experiments: recorded evidence", section A,
 *    Diagram 1 and Tests 1-2).
 *  - Prepared planes (layout version 1): ONE allocation of n*(k/128)*34
 *    bytes: the code plane [n][k/4] (row*k/4 + block*32 + byte) followed by
 *    the fp16 scale plane [n][k/128] starting at byte n*k/4 (page "Baseline
 *    and the integer breakthrough", section "Separate the codes from their
 *    scales"; "Kernel experiments", Test 4).  Same values, other addresses.
 *  - Activations x: [m][k] with a row stride in elements; bf16, fp16 or fp32.
 *  - q: int8 [m][k] contiguous (row stride k).  xs: float [m][k/128].
 *  - y: float [m][n] contiguous (row stride n).
 */
#ifndef PQ2_H
#define PQ2_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
    PQ2_OK = 0,
    PQ2_EINVAL = 1,   /* null pointer, unknown dtype, overlapping buffers      */
    PQ2_ESHAPE = 2,   /* k % 128 != 0, m/n/k out of range, raw stride too small */
    PQ2_EALIGN = 3,   /* a pointer or stride breaks the alignment stated below */
    PQ2_ELAUNCH = 4,  /* the HIP runtime reported an error for a launch        */
    PQ2_EDEVICE = 5   /* the current device is not a gfx950 GPU                */
};

/* Activation element types for pq2_quantize_act_i8. */
enum { PQ2_BF16 = 0, PQ2_F16 = 1, PQ2_F32 = 2 };
/* Weight layouts, for the read probe. */
enum { PQ2_LAYOUT_PLANES = 0, PQ2_LAYOUT_TILES = 1 };

/* Limits (inclusive). */
#define PQ2_MAX_SMALL_M 16
#define PQ2_MAX_K 65536

/* Version of the prepared-plane layout the matmul entry points read: 1 =
 * code plane [n][k/4] followed by the fp16 scale plane [n][k/128].  A layout
 * switch must change what callers key compiled graphs on (page "Baseline and
 * the integer breakthrough", "Separate the codes from their scales": the
 * cache-key bug). */
int pq2_layout_version(void);

/* Human-readable name of a status code (static storage; never NULL). */
const char* pq2_status_str(int status);

/* Name of the HIP runtime error behind the last PQ2_ELAUNCH returned on the
 * calling thread ("hipSuccess" if the last launch succeeded); static storage. */
const char* pq2_last_hip_error(void);

/* Raw PQ2 rows -> prepared planes.  One-time weight preparation, outside
 * any timed loop (page "Kernel experiments", Tests 1 and 4).
 *   raw     device, n rows of raw_row_stride_bytes >= (k/128)*34; any alignment.
 *   planes  device, n*(k/128)*34 bytes, 16-byte aligned; must not overlap raw.
 * Errors: EINVAL (null, overlap), ESHAPE (k%128, n<1, stride too small),
 *         EALIGN (planes not 16-byte aligned), ELAUNCH, EDEVICE. */
int pq2_prepare_planes(const void* raw, int64_t raw_row_stride_bytes, int64_t n, int64_t k,
                       void* planes, void* stream);

/* Group-128 INT8 activation quantisation, bit-exact with the definition
 * above (page "Baseline and the integer breakthrough", "Calculate with small
 * integers" step 1; page "Kernel experiments", Test 6 quantizer).
 *   x       device, dtype PQ2_BF16 / PQ2_F16 / PQ2_F32, m rows of
 *           x_row_stride_elems >= k elements; element-aligned.
 *   q       device int8 [m][k], 8-byte aligned.   xs  device float [m][k/128], 4-byte aligned.
 * Errors: EINVAL (null, dtype), ESHAPE (m<1, k<128, k%128, k > PQ2_MAX_K,
 *         stride < k), EALIGN, ELAUNCH, EDEVICE. */
int pq2_quantize_act_i8(const void* x, int dtype, int64_t x_row_stride_elems, int64_t m, int64_t k,
                        int8_t* q, float* xs, void* stream);

/* Decode / small-batch verification matmul for 1 <= m <= 16 activation
 * columns: y = the definition above, from prepared planes (page "Baseline
 * and the integer breakthrough", "Calculate with small integers" steps 2-4;
 * page "Kernel experiments", section B, Test 6 DP4A GEMV).  Each output is
 * the FP32 sum of k/128 group terms float(dot)*xs*ws, each group's integer
 * dot product formed exactly before it is scaled; the summation order does
 * not depend on m (batch-invariant).
 *   q       device int8 [m][k], 16-byte aligned.   xs  device float [m][k/128], 4-byte aligned.
 *   planes  device prepared planes (layout version 1), 16-byte aligned.
 *   y       device float [m][n], 4-byte aligned; fully overwritten.
 * Errors: EINVAL (null), ESHAPE (m outside 1..16, n<1, k<128, k%128,
 *         k > PQ2_MAX_K), EALIGN, ELAUNCH, EDEVICE. */
int pq2_matmul_small_m(const int8_t* q, const float* xs, const void* planes, int64_t m, int64_t n,
                       int64_t k, float* y, void* stream);

/* Prefill matmul on the INT8 matrix cores (MFMA) for any m >= 1 (tuned for
 * m >= 128): same definition and output as pq2_matmul_small_m (page
 * "Baseline and the integer breakthrough", "Use matrix hardware for
 * prefill"; page "Kernel experiments", Tests 2 and 7).  Argument rules as
 * for pq2_matmul_small_m, except that 1 <= m <= 65535*64.
 * Errors: EINVAL, ESHAPE, EALIGN, ELAUNCH, EDEVICE. */
int pq2_matmul_prefill(const int8_t* q, const float* xs, const void* planes, int64_t m, int64_t n,
                       int64_t k, float* y, void* stream);

/* Prefill matmul from plane-order activations (the qp output of
 * pq2_quantize_act_i8_planes; its qsum is not needed): the same result as
 * pq2_matmul_prefill on the natural-order q, bit for bit, without the byte
 * transpose while staging (page "Kernel experiments", Test 21: activations
 * prepared in the order the decoded codes need).  Argument rules as for
 * pq2_matmul_prefill, qp 16-byte aligned.
 * Errors: EINVAL, ESHAPE, EALIGN, ELAUNCH, EDEVICE. */
int pq2_matmul_prefill_planes(const int8_t* qp, const float* xs, const void* planes, int64_t m, int64_t n,
                              int64_t k, float* y, void* stream);

/* pq2_matmul_small_m straight from the raw block layout, with no
 * preparation pass (page "Kernel experiments", section A, Tests 4 and 24:
 * the interleaved 34-byte blocks, fp16 scale then 32 code bytes, read in
 * place): the same definition, limits and summation order as
 * pq2_matmul_small_m, hence the same bits, from the packed-dot engine.
 *   q       device int8 [m][k], 16-byte aligned.   xs  device float [m][k/128], 4-byte aligned.
 *   raw     device, n rows of raw_row_stride_bytes >= k/128*34 bytes (even,
 *           at most 2^26); 2-byte aligned.  Row padding is never read.
 *   y       device float [m][n], 4-byte aligned; fully overwritten; must
 *           not overlap any input.
 * Errors: EINVAL (null, overlap), ESHAPE (m outside 1..16, n<1, k<128,
 *         k%128, k > PQ2_MAX_K, stride too small, odd or too large),
 *         EALIGN, ELAUNCH, EDEVICE. */
int pq2_matmul_small_m_raw(const int8_t* q, const float* xs, const void* raw, int64_t raw_row_stride_bytes, int64_t m,
                           int64_t n, int64_t k, float* y, void* stream);

/* Plane-order variant of pq2_quantize_act_i8 for the decode path (page
 * "Kernel experiments: recorded evidence", Test 21 and Diagram 7: activations
 * stored in the order of the code planes, with per-group sums that absorb the
 * -1 code offset).  Same xs and the same q values as pq2_quantize_act_i8,
 * stored differently: inside every 16-byte block (weights 16t..16t+15 of a
 * row) the bytes are 4x4-transposed,
 *     qp[m][16t + 4s + j] = q[m][16t + 4j + s],   s, j in 0..3,
 * so dword s of the block pairs with bit plane s of code dword t.  Also
 *     qsum[m][g] = sum_{i in group g} q[m][i]   (int32, |qsum| <= 16256).
 *   x       as for pq2_quantize_act_i8.
 *   qp      device int8 [m][k] (plane order), 16-byte aligned.
 *   xs      device float [m][k/128], 4-byte aligned.
 *   qsum    device int32 [m][k/128], 4-byte aligned.
 * No output may overlap x or another output.
 * Errors: EINVAL (null, dtype, overlap), ESHAPE (m<1, k<128, k%128,
 *         k > PQ2_MAX_K, stride < k), EALIGN, ELAUNCH, EDEVICE. */
int pq2_quantize_act_i8_planes(const void* x, int dtype, int64_t x_row_stride_elems, int64_t m, int64_t k,
                               int8_t* qp, float* xs, int32_t* qsum, void* stream);

/* Small-m matmul from the outputs of pq2_quantize_act_i8_planes: the same
 * definition, limits and summation order as pq2_matmul_small_m, and the
 * same bits for the same inputs (page "Kernel experiments", Test 21: the
 * masked-plane decode with the -sum(q) correction gives the identical
 * integer dot).
 *   qp      device int8 [m][k] in plane order, 16-byte aligned.
 *   xs      device float [m][k/128], 4-byte aligned.
 *   qsum    device int32 [m][k/128], 4-byte aligned; must equal the group
 *           sums of the q values held in qp (otherwise y is wrong).
 *   planes  device prepared planes (layout version 1), 16-byte aligned.
 *   y       device float [m][n], 4-byte aligned; fully overwritten; must not
 *           overlap any input.
 * Errors: EINVAL (null, overlap), ESHAPE (m outside 1..16, n<1, k<128,
 *         k%128, k > PQ2_MAX_K), EALIGN, ELAUNCH, EDEVICE. */
int pq2_matmul_small_m_planes(const int8_t* qp, const float* xs, const int32_t* qsum, const void* planes,
                              int64_t m, int64_t n, int64_t k, float* y, void* stream);

/* Quantise + small-m matmul in one launch: y = the definition above for the
 * activations pq2_quantize_act_i8 would produce from x, bit for bit the y of
 * pq2_quantize_act_i8 followed by pq2_matmul_small_m (same codes, scales and
 * summation order), without the intermediate q / xs buffers or the second
 * launch.  Every workgroup quantises the k slice of x it reads (page
 * "Kernel experiments", Test 12 fusion screen and Test 18: fused preparation
 * must reproduce the standalone quantiser's codes exactly).
 *   x       device, dtype PQ2_BF16 / PQ2_F16 / PQ2_F32, m rows of
 *           x_row_stride_elems elements (>= k); x and the row stride in
 *           bytes 16-byte aligned; all m rows within 2^31 - 1 bytes.
 *   planes  device prepared planes (layout version 1), 16-byte aligned.
 *   y       device float [m][n], 4-byte aligned; fully overwritten; must not
 *           overlap x or planes.
 * Errors: EINVAL (null, dtype, overlap), ESHAPE (m outside 1..16, n<1,
 *         k<128, k%128, k > PQ2_MAX_K, stride < k, x span >= 2^31 bytes),
 *         EALIGN, ELAUNCH, EDEVICE. */
int pq2_matmul_small_m_fused(const void* x, int dtype, int64_t x_row_stride_elems, const void* planes,
                             int64_t m, int64_t n, int64_t k, float* y, void* stream);

/* ---- Tile-major weights for the decode GEMV (page "Kernel experiments:
 * recorded evidence", section H, Tests 24 and 25: storing the bytes one
 * warp loads next to each other, same values at other addresses).
 *
 * Tile layout: T = ceil(n/16) tiles of 16 rows, G = k/128 groups,
 * S8 = ceil(G/8) segments of 8 groups.  ONE allocation of
 * pq2_tiles_bytes(n, k) = T*S8*4352 bytes made of segment units: unit
 * (t, sb) at (t*S8 + sb)*4352 holds
 *  - four code blocks b = 0..3 of 1024 bytes: bytes 1024*b + 16*l ..
 *    1024*b + 16*l + 15 with l = j + 16*kb (j = 0..15, kb = 0..3) hold four
 *    dwords u = 0..3, dword u = the 16 weights k0..k0+15 of row 16t+j with
 *    k0 = 128*(8sb + 2b + u/2) + 64*(u%2) + 16*kb; bits 2s..2s+1 of its byte
 *    v are the code of weight k0 + 4s + v;
 *  - then 256 bytes of scales: bytes 4096 + 16*j .. 4096 + 16*j + 15 are the
 *    eight fp16 scales of row 16t+j, groups 8*sb .. 8*sb+7;
 *  - padding rows (>= n) and groups (>= G) hold code 1 (weight 0), scale 0. */

/* Bytes of the tile layout for an n x k weight matrix; -1 if n < 1,
 * n > 2^30, k < 128, k % 128 or k > PQ2_MAX_K. */
int64_t pq2_tiles_bytes(int64_t n, int64_t k);

/* Raw PQ2 rows -> tile layout.  One-time weight preparation, outside any
 * timed loop.
 *   raw     device, n rows of raw_row_stride_bytes >= (k/128)*34; any alignment.
 *   tiles   device, pq2_tiles_bytes(n, k) bytes, 16-byte aligned, fully
 *           written (padding included); must not overlap raw.
 * Errors: EINVAL (null, overlap), ESHAPE (k%128, n<1, stride too small),
 *         EALIGN, ELAUNCH, EDEVICE. */
int pq2_prepare_tiles(const void* raw, int64_t raw_row_stride_bytes, int64_t n, int64_t k, void* tiles,
                      void* stream);

/* pq2_matmul_small_m from the tile layout: the same definition and limits
 * (page "Kernel experiments", Test 25: the tile-major projection matched the
 * row-major one bit for bit).  Each group's exact integer dot comes from the
 * INT8 matrix cores.  k is cut into 1024-element segments split over up to
 * 16 waves (pq2_matmul_small_m: up to 8), so for k <= 8192 (one segment per
 * wave in both) the bits equal pq2_matmul_small_m's; for longer k the
 * summation order differs (still one FP32 term per group, batch-invariant:
 * the split depends on k only).
 *   q       device int8 [m][k], 16-byte aligned.   xs  device float [m][k/128], 4-byte aligned.
 *   tiles   device tile layout of the weights, 16-byte aligned.
 *   y       device float [m][n], 4-byte aligned; fully overwritten; must
 *           not overlap any input.
 * Errors: EINVAL (null, overlap), ESHAPE (m outside 1..16, n<1, k<128,
 *         k%128, k > PQ2_MAX_K), EALIGN, ELAUNCH, EDEVICE. */
int pq2_matmul_small_m_tiles(const int8_t* q, const float* xs, const void* tiles, int64_t m, int64_t n,
                             int64_t k, float* y, void* stream);

/* Quantise + tile-layout matmul in one launch: bit for bit the y of
 * pq2_quantize_act_i8 followed by pq2_matmul_small_m_tiles (same codes,
 * scales and summation order).  Every wave quantises the activation groups
 * it stages, with the exact in-kernel quantiser of
 * pq2_matmul_small_m_fused (page "Kernel experiments", Test 12 fusion screen
 * and Test 18: fused preparation must reproduce the standalone quantiser's
 * codes exactly).
 *   x       device, dtype PQ2_BF16 / PQ2_F16 / PQ2_F32, m rows of
 *           x_row_stride_elems elements (>= k); x and the row stride in
 *           bytes 16-byte aligned; all m rows within 2^31 - 1 bytes.
 *   tiles   device tile layout of the weights, 16-byte aligned.
 *   y       device float [m][n], 4-byte aligned; fully overwritten; must not
 *           overlap x or tiles.
 * Errors: EINVAL (null, dtype, overlap), ESHAPE (m outside 1..16, n<1,
 *         k<128, k%128, k > PQ2_MAX_K, stride < k, x span >= 2^31 bytes),
 *         EALIGN, ELAUNCH, EDEVICE. */
int pq2_matmul_small_m_tiles_fused(const void* x, int dtype, int64_t x_row_stride_elems, const void* tiles,
                                   int64_t m, int64_t n, int64_t k, float* y, void* stream);

/* Decode GEMV from activations, y = W x for 1 <= m <= 16 (page "Kernel
 * experiments", Tests 3-5: the integer GEMV is called with the activations
 * and the weights and returns the outputs, quantising inside): the
 * library's faster of pq2_matmul_small_m_tiles_fused (one launch; taken at
 * m <= 2 with k <= 8192, where every wave holds one k segment, and
 * m * ceil(n/16) <= 1600, since every 16-row tile repeats the quantisation)
 * and pq2_quantize_act_i8 into the caller's q_work / xs_work followed by
 * pq2_matmul_small_m_tiles.  Both give the same bits.  Rows the fused
 * kernel cannot read (x or its row stride in bytes not 16-byte aligned)
 * take the two-launch path when scratch is given.
 *   x       as pq2_matmul_small_m_tiles_fused (on the fused path) or
 *           pq2_quantize_act_i8 (otherwise).
 *   q_work  device int8 [m][k], 16-byte aligned; xs_work device float
 *           [m][k/128], 4-byte aligned: scratch owned by the caller, written
 *           on the two-launch path (may be NULL when the fused path is
 *           taken).
 *   tiles, y as pq2_matmul_small_m_tiles; nothing may overlap.
 * Errors: those of the path taken, checked before anything is enqueued. */
int pq2_gemv_tiles(const void* x, int dtype, int64_t x_row_stride_elems, const void* tiles, int64_t m, int64_t n,
                   int64_t k, float* y, int8_t* q_work, float* xs_work, void* stream);

/* pq2_gemv_tiles for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without q_work / xs_work, the same bits, and no allocation of
 * any kind.  Its scratch (quantised activations and their scales) is one
 * library-owned device array of 1 MiB + 32 KiB per GPU, sized for
 * m <= PQ2_MAX_SMALL_M and k <= PQ2_MAX_K and held until the process ends;
 * its address is looked up on the first call on each device (make that
 * first call outside graph capture).  Every call on a GPU shares that GPU's
 * array, so calls that overlap on one GPU (other streams, other threads)
 * race and must be ordered by the caller.
 * Errors: those of pq2_gemv_tiles; ESHAPE for a shape beyond the scratch
 * (m > 16 or k > 65536). */
int pq2_gemv_tiles_static(const void* x, int dtype, int64_t x_row_stride_elems, const void* tiles, int64_t m,
                          int64_t n, int64_t k, float* y, void* stream);

/* ---- Split k over workgroups (page "Kernel experiments: recorded
 * evidence", Test 30: split-K with a fixed-order combine in the last block,
 * which resets its counter; page "KERNEL_REPORT: PTQ1_0 small-batch
 * decoding", "Facts": a column's result must not depend on how many columns
 * share the call).
 *
 * The same definition as pq2_matmul_small_m_tiles with k cut into slices of
 * one 1024-element segment (8 groups); the slices of a 16-row tile run in
 * several workgroups, each slice's sum of its group terms goes to
 * `partials`, and the workgroup that arrives last at the tile's counter adds
 * the slices in index order, writes y and sets the counter back to zero.
 * No workgroup waits for another.  The summation order depends on k only
 * (not on m: batch-invariant); for k <= 8192 it is the order of
 * pq2_matmul_small_m_tiles, so the bits are the same.  On MI355X it is
 * slower than the single-workgroup kernel at every measured shape (the
 * device-scope stores, ticket and reloads add about 1.4 us per call at
 * k = 17408), so no default path takes it.
 *   q, xs, tiles, y, limits: as pq2_matmul_small_m_tiles.
 *   partials  device float [pq2_tiles_splitk_partial_floats(m, n, k)], 4-byte
 *             aligned, scratch (contents on entry do not matter).
 *   counters  device uint32 [pq2_tiles_splitk_counter_words(n)], 4-byte
 *             aligned: ALL ZERO before the first call; every call leaves
 *             them zero.  Calls that share partials or counters must not
 *             run at the same time.
 * Errors: EINVAL (null, overlap), ESHAPE, EALIGN, ELAUNCH, EDEVICE. */
int pq2_matmul_small_m_tiles_splitk(const int8_t* q, const float* xs, const void* tiles, int64_t m, int64_t n,
                                    int64_t k, float* y, float* partials, uint32_t* counters, void* stream);

/* Floats of partial sums pq2_matmul_small_m_tiles_splitk needs:
 * ceil(k/1024) * m * n; -1 for an invalid shape.  Host only. */
int64_t pq2_tiles_splitk_partial_floats(int64_t m, int64_t n, int64_t k);

/* Counter words pq2_matmul_small_m_tiles_splitk needs: 4 * ceil(n/16); -1 for
 * an invalid n.  Host only. */
int64_t pq2_tiles_splitk_counter_words(int64_t n);

/* Smaller activation groups (page "Kernel experiments", section C,
 * Diagram 3, Tests 8 and 9): the weights keep their 128-weight blocks and
 * fp16 scales; activations are quantised in groups of agroup = 128, 64 or 32
 * elements, each with its own scale max|x|/127 (the same steps as
 * pq2_quantize_act_i8 on the smaller group; agroup = 128 is that function).
 *   x, q    as pq2_quantize_act_i8.   xs  device float [m][k/agroup], 4-byte aligned.
 * Errors: EINVAL (null, dtype, agroup not 128/64/32, overlap), otherwise as
 *         pq2_quantize_act_i8. */
int pq2_quantize_act_i8_g(const void* x, int dtype, int64_t x_row_stride_elems, int64_t m, int64_t k,
                          int64_t agroup, int8_t* q, float* xs, void* stream);

/* Tile-layout decode matmul with activation groups of agroup elements:
 *   y[m][n] = sum over weight blocks g of ws[n][g] * sum over the activation
 *             groups a inside block g of float(dot_a) * xs[m][a],
 * dot_a the exact integer dot of group a's q with the block's codes minus 1.
 * Each activation group has its own integer product (no rounding inside it);
 * a weight block's terms float(dot_a) * xs[m][a] are summed in k order and
 * scaled by ws[n][g], and these block terms are added as
 * pq2_matmul_small_m_tiles adds its group terms (so agroup = 128 gives the
 * same bits as pq2_matmul_small_m_tiles).  q and xs come from
 * pq2_quantize_act_i8_g with the same agroup.
 *   q       device int8 [m][k], 16-byte aligned.  xs  device float [m][k/agroup].
 *   tiles, y, limits and errors as pq2_matmul_small_m_tiles, plus EINVAL for
 *   agroup not 128/64/32. */
int pq2_matmul_small_m_tiles_g(const int8_t* q, const float* xs, const void* tiles, int64_t m, int64_t n, int64_t k,
                               int64_t agroup, float* y, void* stream);

/* pq2_quantize_act_i8_g + pq2_matmul_small_m_tiles_g in one launch (page
 * "Kernel experiments", section C, activation groups of 64 or 32, with the
 * fusion of Tests 12 and 18): every workgroup quantises the activation
 * groups it reads while staging them, with the definition of
 * pq2_quantize_act_i8_g, so y has the same bits as the two calls with the
 * same agroup.
 *   x       device bf16 / fp16 / fp32 [m][x_row_stride_elems], read in place;
 *           16-byte aligned rows (x and x_row_stride_elems * element size).
 *   tiles, y, limits and errors as pq2_matmul_small_m_tiles_fused, plus
 *   EINVAL for agroup not 128/64/32. */
int pq2_matmul_small_m_tiles_fused_g(const void* x, int dtype, int64_t x_row_stride_elems, const void* tiles,
                                     int64_t m, int64_t n, int64_t k, int64_t agroup, float* y, void* stream);

/* Prefill matmul from the tile layout: the definition, limits and output of
 * pq2_matmul_prefill, and the same bits, with the weights read from the
 * decode GEMV's tile layout, so one prepared copy serves decode and prefill
 * (page "Kernel experiments", section H: keeping one weight layout for
 * every reader).
 *   q       device int8 [m][k], 16-byte aligned.   xs  device float [m][k/128], 4-byte aligned.
 *   tiles   device tile layout of the weights, 16-byte aligned.
 *   y       device float [m][n], 4-byte aligned; fully overwritten; must
 *           not overlap any input.
 * Errors: EINVAL (null, overlap), ESHAPE (m outside 1..65535*64, n<1,
 *         k<128, k%128, k > PQ2_MAX_K), EALIGN, ELAUNCH, EDEVICE. */
int pq2_matmul_prefill_tiles(const int8_t* q, const float* xs, const void* tiles, int64_t m, int64_t n,
                             int64_t k, float* y, void* stream);

/* Tile-layout prefill matmul with activation groups of agroup elements
 * (page "Kernel experiments", section C, Tests 8 and 9, which timed them at
 * prefill sizes): the y of pq2_matmul_small_m_tiles_g's definition for any m.
 * Each activation group's integer product is exact; a weight block's terms
 * float(dot_a) * xs[m][a] are summed in k order, then scaled by ws[n][g] into
 * the output's fp32 sum, block after block; agroup = 128 gives the bits of
 * pq2_matmul_prefill_tiles.  q and xs come from pq2_quantize_act_i8_g with
 * the same agroup.
 *   q       device int8 [m][k], 16-byte aligned.  xs  device float [m][k/agroup].
 *   tiles, y, limits and errors as pq2_matmul_prefill_tiles, plus EINVAL for
 *   agroup not 128/64/32. */
int pq2_matmul_prefill_tiles_g(const int8_t* q, const float* xs, const void* tiles, int64_t m, int64_t n, int64_t k,
                               int64_t agroup, float* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PQ2_H */
