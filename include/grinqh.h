/*
 * grinqh.h -- C ABI of the GRINQH decode-stage vector-matrix multiply for
 * AMD Instinct MI355X (gfx950).
 *
 * Method: "GRINQH: Graded Input-based Quantization Hierarchy for Efficient
 * LLM Generation" (arXiv 2606.23419).  At batch size 1, y = x W over one
 * linear layer, W stored input-major (row i = input channel i) as b_max-bit
 * codes (b_max = 8, or a smaller maximum width such as the 4 and 6 of
 * section 3.3).  Each row i gets a bit width b_i in {0..b_max} from |x_i| and
 * calibrated thresholds (section 3.1); only the b_i most significant bit
 * planes of that row are read from a nested bit-plane store (section 3.3,
 * Appendix C.1); the truncated code is rebuilt with the midpoint term and
 * dequantised with the row group's scale and zero (section 3.3), and products
 * accumulate in fp32.
 *
 * Conventions shared by every call below
 * - Pointers are DEVICE pointers unless the argument says "host".  The caller
 *   allocates and owns every buffer; the library allocates nothing and keeps
 *   no state between calls (the one exception is the device array of the
 *   allocation-free entry point at the end of this header).
 * - fp16 values travel as their IEEE binary16 bit patterns (uint16_t).
 * - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *   enqueues work on it and returns without waiting for the device.
 * - Arguments are validated on the host before any HIP call; a rejected call
 *   returns GRINQH_EINVAL and enqueues nothing.  A failed launch returns
 *   GRINQH_EDEVICE.  grinqh_last_error() then describes the failure.
 * - Calls that share a workspace buffer must not overlap in time (run them
 *   on one stream, or give each stream its own workspace).
 *
 * Store layout (this library's concrete form of the paper's bit-planar
 * store; grinqh_layout_version() == 4), for b_max-bit codes, 1 <= b_max <= 8:
 * - N_pad = N rounded up to a multiple of 128.  Columns are cut into tiles of
 *   GRINQH_TILE = 1024 columns; tile t has width C_t = min(1024, N_pad - 1024 t).
 * - Let R = b_max / 8.  Tile t occupies bytes [1024 K t R, (1024 K t + K C_t) R).
 *   Inside it, row tile (t, i) starts at (1024 K t + i C_t) R and holds planes
 *   0 .. b_max - 1 back to back, C_t / 8 bytes each; plane p holds bit
 *   (b_max - 1 - p) of the code, so the top b planes of a row are one
 *   contiguous span of b C_t / 8 bytes.  At b_max = 8 this is the full 8-plane
 *   store; a smaller b_max keeps only the planes it has (section 3.3 and
 *   Appendix C.1: the format does not depend on the maximum width).
 * - A plane is a run of little-endian 32-bit words, one per 32 columns.  In
 *   the word for columns 32w .. 32w + 31 of the tile, column 32w + 4m + j
 *   (m = 0..7, j = 0..3) sits at bit 8j + m.
 * - Padding columns N .. N_pad - 1 hold code 0 and are never written to y.
 *
 * Scales and zeros: fp16 [G][N] row-major with G = ceil(K / 128); rows
 * 128g .. 128g + 127 share s[g][j] and z[g][j] (section 4: group size 128).
 */
#ifndef GRINQH_H
#define GRINQH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    GRINQH_OK = 0,
    GRINQH_EINVAL = -1,   /* bad argument; nothing was enqueued */
    GRINQH_EDEVICE = -2,  /* HIP reported an error (no device, launch failure) */
    GRINQH_ENOSYS = -3    /* the library was built without the feature the call needs
                             (only grinqh_timeline_read, outside a timeline build) */
};

#define GRINQH_GROUP 128          /* rows per (scale, zero) group */
#define GRINQH_TILE 1024          /* columns per row tile of the store */
#define GRINQH_MAX_THRESHOLDS 8   /* n <= 8 thresholds, n + 1 <= 9 levels */
#define GRINQH_MAX_BITS 8         /* largest b_max */
#define GRINQH_MAX_GROUP 4        /* members of one grouped launch */

/* Version of the store layout described above (4). */
int grinqh_layout_version(void);

/* Static description of a status code.  Never NULL. */
const char* grinqh_status_string(int status);

/* Message for the most recent failed call on this host thread ("" if none). */
const char* grinqh_last_error(void);

/* Size in bytes of the bit-plane store for K rows and N columns of b_max-bit
 * codes: K * N_pad * b_max / 8.  Returns -1 if K <= 0, N <= 0 or b_max is
 * outside 1..8. */
int64_t grinqh_planes_bytes(int64_t K, int64_t N, int b_max);

/* Workspace bytes grinqh_vmm / grinqh_decode_vmm need for a K x N layer
 * (split-K partial sums, per-tile counters and two 8-byte words per padded
 * column).  Returns -1 for K, N <= 0. */
int64_t grinqh_workspace_bytes(int64_t K, int64_t N);

/* Zero a workspace so it can be used by grinqh_vmm / grinqh_decode_vmm.
 * Needed once after allocation: every successful VMM call leaves the
 * counters and column words at zero again.  Uses a fill kernel, so it may be
 * captured in a HIP graph. */
int grinqh_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * Offline packing (section 3.3 "Storage Layout and Weight Loading";
 * Appendix C.1 "Bit-packing", "Grouping").
 * codes:  u8 [K][N] row-major, b_max-bit codes (row = input channel), each
 *         below 2^b_max; only the low b_max bits of a code are stored.
 * b_max:  1..8, the planes per row of the store.
 * planes: u8 [grinqh_planes_bytes(K, N, b_max)], written completely (padding too).
 * Errors: EINVAL for NULL pointers, K, N <= 0, b_max outside 1..8 or
 * K * N_pad >= 2^40.
 */
int grinqh_pack(const uint8_t* codes, int64_t K, int64_t N, int b_max, uint8_t* planes, void* stream);

/*
 * Offline threshold calibration by percentile mapping (section 3.2;
 * Appendix A.1 eq. (2)).
 * calib:      fp16 [V][K] row-major, V calibration activation vectors.
 * P:          host double [n_levels], the target share p_k of rows at level k.
 * n_levels:   1 .. 9; n = n_levels - 1 thresholds are produced.
 * thresholds: fp32 [n] (device).  theta_k = mean over vectors of the
 *             linear-interpolation c_k-quantile of |v| with c_k = p_0 + ... +
 *             p_{k-1} (position c_k (K - 1) between order statistics),
 *             averaged in fp64 in vector order and rounded to fp32;
 *             c_k <= 0 gives 0 and c_k >= 1 gives +inf.
 * Errors: EINVAL for NULL pointers, V <= 0, K <= 0, n_levels outside 1..9,
 * or a P entry that is negative or not finite.
 */
int grinqh_calibrate(const uint16_t* calib, int64_t V, int64_t K, const double* P, int n_levels,
                     float* thresholds, void* stream);

/*
 * Dynamic precision assignment and active-row selection (section 3.1).
 * x:          fp16 [K].
 * thresholds: host fp32 [n], non-decreasing, >= 0 (+inf allowed), 0 <= n <= 8.
 * levels:     host u8 [n + 1], each 0..8.
 * bits:       u8 [K] out: b_i = levels[#{t : |x_i| >= thresholds[t]}] (fp32
 *             compare; a tie goes to the upper level; NaN gets levels[0]).
 * active_idx: i32 [K] out: the rows with b_i > 0 in ascending order in its
 *             first *n_active entries (the rest is left untouched).
 * n_active:   i32 [1] out.
 * Errors: EINVAL for NULL pointers, K <= 0 or K >= 2^31, n outside 0..8,
 * thresholds negative, NaN or decreasing, or a level above 8.
 */
int grinqh_assign_bits(const uint16_t* x, int64_t K, const float* thresholds, const uint8_t* levels,
                       int n, uint8_t* bits, int32_t* active_idx, int32_t* n_active, void* stream);

/*
 * The decode-stage VMM from an explicit assignment (section 3.3).
 * y[j] = sum over listed rows i of x_i (s[g][j] r_ij + z[g][j]), g = i / 128,
 * r_ij = (q_ij with its low b_max - b_i bits cleared) + phi_i,
 * phi_i = 2^(b_max - 1 - b_i) for b_i < b_max and 0 for b_i = b_max; only
 * the top b_i planes of a row are read.
 * planes:     the store (layout above) for K x N, packed with this b_max.
 * scales, zeros: fp16 [ceil(K/128)][N], the step and offset of the b_max-bit
 *             codes (w = s q + z).
 * x:          fp16 [K].
 * bits:       u8 [K]; entries above b_max are treated as b_max, rows with 0
 *             add nothing.
 * active_idx: i32 [*n_active], strictly ascending, each in [0, K) -- for
 *             example the output of grinqh_assign_bits.
 * n_active:   i32 [1] on the device (read by the kernel; no host sync).
 * y:          fp32 [N] out (written completely).
 * workspace:  grinqh_workspace_bytes(K, N) bytes, zeroed once with
 *             grinqh_workspace_init.
 * The K-splits' partial sums are combined so that y does not depend on
 * scheduling (bit-identical from call to call): up to 64 splits as exact
 * integer sums of the partials in units of 2^-20 (partials of magnitude 2^22
 * or more, or not finite, added as floats in split order), beyond that as
 * floats in split order.
 * Errors: EINVAL for NULL pointers, K, N <= 0, K >= 2^31, b_max outside
 * 1..8, or a workspace smaller than grinqh_workspace_bytes(K, N).
 */
int grinqh_vmm(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
               const uint16_t* x, const uint8_t* bits, const int32_t* active_idx,
               const int32_t* n_active, int64_t K, int64_t N, int b_max, float* y,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * The whole decode step in one launch: assignment (section 3.1) fused into
 * the VMM (section 3.3).  Same result as grinqh_assign_bits followed by
 * grinqh_vmm, without materialising bits or the active list.
 * thresholds/levels/n as in grinqh_assign_bits (host arrays), with every
 * level at most b_max (EINVAL otherwise); the remaining arguments as in
 * grinqh_vmm.
 */
int grinqh_decode_vmm(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                      const uint16_t* x, int64_t K, int64_t N, int b_max,
                      const float* thresholds, const uint8_t* levels, int n, float* y,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Accumulating form of grinqh_decode_vmm: y[j] += (x W)[j] for the same
 * decode-stage VMM (sections 3.1 and 3.3).  Workgroups add their results into
 * y with fp32 device-scope atomic adds, so no split-K workspace and no final
 * reduction pass are needed; the order of the additions is not fixed, so the
 * last bits of y can differ from run to run.
 * y:     fp32 [N], read and updated.  Zero it first for a plain product, or
 *        pass the residual stream of a projection that adds into it.
 * clear: fp32 [N] or NULL.  When given, this call sets it to zero, so a decode
 *        loop can alternate two output buffers without a separate fill launch.
 *        It must not overlap y or x (it is zeroed while x is still read).
 * Other arguments as in grinqh_decode_vmm (no workspace).
 * Errors: as grinqh_decode_vmm, and EINVAL when clear overlaps y or x.
 */
int grinqh_decode_vmm_accumulate(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                                 const uint16_t* x, int64_t K, int64_t N, int b_max,
                                 const float* thresholds, const uint8_t* levels, int n,
                                 float* y, float* clear, void* stream);

/*
 * Several independent accumulating decode steps in one launch (sections 3.1
 * and 3.3, each step as grinqh_decode_vmm_accumulate): member m computes
 *   y[m][j] += (x[m] W[m])[j],  j < N[m],
 * with its own store, scales, zeros, activation, thresholds and levels.
 * Meant for the projections of a layer that read the same position of the
 * model (q, k and v; gate and up), which a decode step can issue together:
 * one launch instead of count, and the members' column tiles fill the CUs
 * together.  Each member's result is the one grinqh_decode_vmm_accumulate
 * gives up to the order of the fp32 additions (the workgroup shape is chosen
 * for the members together).
 * count:      1 .. GRINQH_MAX_GROUP members.
 * planes, scales, zeros, x, y: host arrays of count device pointers, each as
 *             in grinqh_decode_vmm_accumulate for a K x N[m] layer.
 * K, b_max:   shared by all members.
 * N:          host int64 [count].
 * thresholds, levels: host arrays of count host pointers; n: host int
 *             [count]; member m's as in grinqh_decode_vmm.
 * clear:      NULL, or a host array of count pointers each NULL or an fp32
 *             [N[m]] buffer that this call zeroes; a clear buffer must not
 *             overlap any member's y or x.  Members' y may be the same
 *             buffer (their contributions add).
 * Errors: EINVAL for count outside 1..GRINQH_MAX_GROUP, NULL arrays, a
 * clear buffer overlapping a y or an x, and anything grinqh_decode_vmm_accumulate
 * rejects for a member.
 */
int grinqh_decode_vmm_accumulate_group(int count, const uint8_t* const* planes, const uint16_t* const* scales,
                                       const uint16_t* const* zeros, const uint16_t* const* x, int64_t K,
                                       const int64_t* N, int b_max, const float* const* thresholds,
                                       const uint8_t* const* levels, const int* n, float* const* y,
                                       float* const* clear, void* stream);

/*
 * Look-up-table reconstruction of nested non-uniform weights (section 3.3:
 * k-means style nested codes in the same bit-plane store, and with tables
 * the nested levels are already centred, so no midpoint term; Appendix E.2).
 * Column j has one fp16 table per width b = 1..b_max with 2^b entries; row i
 * at width b_i reads entry (q_ij >> (b_max - b_i)) of column j's b_i-bit
 * table.  The flat table buffer holds, for b = 1, 2, ..., b_max in turn, a
 * block of N tables of 2^b entries (column j's at j 2^b), so block b starts
 * at entry N (2^b - 2); grinqh_lut_entries(N, b_max) = N (2^(b_max+1) - 2)
 * entries in all.  Returns -1 for N <= 0 or b_max outside 1..8.
 */
int64_t grinqh_lut_entries(int64_t N, int b_max);

/*
 * Accumulating decode step with table reconstruction (sections 3.1 and 3.3):
 *   y[j] += sum over i with b_i > 0 of x_i T_{b_i}[j][q_ij >> (b_max - b_i)],
 * b_i from |x_i| and the thresholds as in grinqh_assign_bits.  Only the top
 * b_i planes of a row are read; only the tables of the levels in use are
 * read.  Sums are fp32, added into y with fp32 device-scope atomics (the
 * order of the additions is not fixed).
 * planes:  the store (layout above) of the b_max-bit parent codes.
 * lut:     fp16 [grinqh_lut_entries(N, b_max)], layout above, 4-byte aligned.
 * x:       fp16 [K].  thresholds, levels, n: as in grinqh_assign_bits, levels
 *          at most b_max.
 * y:       fp32 [N], read and updated.  clear: fp32 [N] or NULL, set to zero
 *          by this call (it must not overlap y or x).
 * Errors: as grinqh_decode_vmm_accumulate, and EINVAL for a NULL or
 * misaligned table.
 */
int grinqh_decode_vmm_lut(const uint8_t* planes, const uint16_t* lut, const uint16_t* x, int64_t K, int64_t N,
                          int b_max, const float* thresholds, const uint8_t* levels, int n, float* y,
                          float* clear, void* stream);

/*
 * Dense prefill of a batch of M tokens (section 3: the prefill stage loads
 * weights at one fixed precision; section 4 "Prefill vs. Decoding
 * Evaluation": weights are unpacked at full b_max precision and multiplied
 * densely).  Every row is read at its full width b_max (nothing truncated, no
 * midpoint term):
 *   Y[m][n] = sum_k X[m][k] w[k][n],  w[k][n] = s[k/128][n] q[k][n] + z[k/128][n],
 * with w rounded to fp16 once (a fused multiply-add) and products summed in
 * fp32 on the matrix cores.
 * planes:        the store (layout above) for K x N, packed with this b_max.
 * scales, zeros: fp16 [ceil(K/128)][N].
 * X:             fp16 [M][K] row-major (token m's activations in row m).
 * Y:             fp32 [M][N] row-major out (written completely).
 * Errors: EINVAL for NULL pointers, M, K, N <= 0, M or N >= 2^31,
 * K >= 2^21, b_max outside 1..8, or more than 2^31 - 1 workgroups
 * (ceil(M / 128) x 2 ceil(N / 1024)).
 */
int grinqh_prefill(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                   const uint16_t* X, int64_t M, int64_t K, int64_t N, int b_max, float* Y, void* stream);

/*
 * Unpacked prefill, first half: the store at full width as dense fp16
 * weights (section 4 "Prefill vs. Decoding Evaluation": weights unpacked at
 * full b_max precision for a dense product; section 3.3: w = s q + z, nothing
 * truncated at b_max), each rounded once to the nearest fp16.
 * Layout ("B-fragment order"): w[k][n] at fp16 index ((k / 8) N_pad + n) 8 +
 * k % 8, where N_pad = N rounded up to 128: eight consecutive rows of a column
 * are one 16-byte fragment.  Rows past K, up to K_pad = K rounded up to 64,
 * and columns past N are 0.
 * grinqh_dense_bytes(K, N) = K_pad N_pad 2 bytes (-1 for K, N <= 0).
 * dense: device buffer of at least that size, 16-byte aligned, written
 * completely.  Unpacking once lets several token batches share it (the buffer
 * costs 2 bytes per weight while it lives).
 * Errors: as grinqh_pack, and EINVAL for a NULL, misaligned or small buffer.
 */
int64_t grinqh_dense_bytes(int64_t K, int64_t N);
int grinqh_unpack_dense(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros, int64_t K,
                        int64_t N, int b_max, void* dense, size_t dense_bytes, void* stream);

/*
 * Unpacked prefill, second half: Y fp32 [M][N] = X fp16 [M][K] times the
 * weights in `dense` (from grinqh_unpack_dense for the same K, N), products
 * summed in fp32 on the matrix cores.  Together the two calls compute what
 * grinqh_prefill computes (same fp16 weight rounding), trading a 2-byte-per-
 * weight buffer for a plain matrix product.
 * Errors: EINVAL for NULL pointers, M, K, N <= 0, M or N >= 2^31, K >= 2^21,
 * or a misaligned buffer.
 */
int grinqh_dense_gemm(const uint16_t* X, const void* dense, int64_t M, int64_t K, int64_t N, float* Y, void* stream);

/*
 * For callers that cannot allocate memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): grinqh_decode_vmm
 * with no workspace argument.  The split-K partial rows and tile counters
 * live in a device array inside the library, GRINQH_NOALLOC_SCRATCH_BYTES
 * per GPU, held from first use until the process ends; this call allocates
 * nothing.  Every call on one GPU shares that GPU's array, so calls that
 * overlap in time on one GPU (two streams, or two graphs replayed at once)
 * race and must not be issued; calls in stream order are fine.
 * Arguments, result (bit-identical to grinqh_decode_vmm) and errors as in
 * grinqh_decode_vmm, plus EINVAL when the layer needs more than the array
 * holds (more than GRINQH_NOALLOC_SCRATCH_BYTES - 4 MiB - 64 KiB of partial
 * rows, or N above 262144; every layer up to 8192 x 28672 and 28672 x 8192
 * fits) and EDEVICE when the array's device address cannot be obtained.
 */
#define GRINQH_NOALLOC_SCRATCH_BYTES (16u << 20)
int grinqh_decode_vmm_noalloc(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                              const uint16_t* x, int64_t K, int64_t N, int b_max,
                              const float* thresholds, const uint8_t* levels, int n, float* y, void* stream);

/*
 * Measurement aid, not part of the decode path.  A library built with
 * GRINQH_TIMELINE defined (libgrinqh_timeline.so, `python -m
 * decode_stage_gemv_amd.build --timeline`) records, in every plain
 * (not grouped) VMM launch, the GPU's 100 MHz constant clock at fixed points
 * of each workgroup's work into a device array of
 * GRINQH_TIMELINE_WORKGROUPS x GRINQH_TIMELINE_SLOTS 64-bit stamps
 * (workgroup-major; workgroups past the first GRINQH_TIMELINE_WORKGROUPS
 * record nothing).  Slots, taken by the workgroup's first wave unless noted:
 *   0 start; 1 widths known (activations arrived); 2 buckets counted;
 *   3 record tables written; 4 first three records' loads issued;
 *   5 waves reduced (after the workgroup barrier); 6 atomics issued
 *   (accumulate), the column words added and acknowledged (split-K up to
 *   64 splits) or the partial row stored and acknowledged (more splits);
 *   7 atomics acknowledged (accumulate) or the tile's sum written (split-K
 *   past 64 splits, the tile's last workgroup only); 8 + w: wave w's
 *   records done.
 * Each launch overwrites the slots it records; other slots keep older values.
 * grinqh_timeline_read copies the first `count` stamps to host memory
 * `stamps` (synchronous: it waits for the device).
 * Errors: ENOSYS in a library built without the timeline; EINVAL for a NULL
 * buffer or a count outside [0, GRINQH_TIMELINE_WORKGROUPS x
 * GRINQH_TIMELINE_SLOTS]; EDEVICE if the copy fails.
 */
#define GRINQH_TIMELINE_WORKGROUPS 8192
#define GRINQH_TIMELINE_SLOTS 24
int grinqh_timeline_read(uint64_t* stamps, int64_t count);

#ifdef __cplusplus
}
#endif

#endif /* GRINQH_H */
