/*
 * nvfp4_group_gemm.h -- C ABI of the MI355X (gfx950) NVFP4 grouped GEMM.
 *
 * Operation (pages "nvfp4 group gemm", kernelindex.com submissions 474067,
 * 482269 and 496386: the header comment and MMA helper of submission 474067
 * define E2M1 operands with one E4M3FN scale per 16 K-elements, fp32
 * accumulation and an fp16 epilogue rounded to nearest-even; its Python entry
 * point custom_kernel takes per-group (A, B, C) tensors, scale tensors and
 * (M, N, K) sizes):
 *
 *   for each group g and every m < M_g, n < N_g:
 *     C_g[m][n] = fp16( sum_k  e2m1(A_g[m][k]) * e4m3fn(SFA_g[m][k/16])
 *                            * e2m1(B_g[n][k]) * e4m3fn(SFB_g[n][k/16]) )
 *
 * Groups are independent problems, each with its own A, B, scales and C.
 */
#ifndef NVFP4_GROUP_GEMM_H
#define NVFP4_GROUP_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define NVFP4_OK           0
#define NVFP4_EINVAL       1  /* malformed arguments: nothing was launched            */
#define NVFP4_EUNSUPPORTED 2  /* well-formed but outside what the kernels handle      */
#define NVFP4_EHIP         3  /* the HIP runtime reported an error (see last_error)   */

/*
 * One group.  All pointers are DEVICE pointers owned by the caller; the
 * library never frees or retains them.
 *
 *   a    E2M1 codes of A, [m][k/2] bytes, row-major.  Element k of a row sits
 *        in byte k/2: even k in the low nibble, odd k in the high nibble.
 *        16-byte aligned.
 *   b    E2M1 codes of B, [n][k/2] bytes, same packing (C = A * B^T: both
 *        operands are K-contiguous).  16-byte aligned.
 *   sfa  E4M3FN scales of A, [m][k/16] bytes, row-major, one per 16
 *        consecutive k.  4-byte aligned.
 *   sfb  E4M3FN scales of B, [n][k/16] bytes, row-major.  4-byte aligned.
 *        With NVFP4_SFB_SWIZZLED in flags: the same scales in the
 *        window-major layout nvfp4_swizzle_scales writes (16-byte aligned).
 *   c    output, [m][n] IEEE fp16, row-major; written, never read.
 *        4-byte aligned.  Must not overlap another group's c or any input.
 *   m, n, k  problem sizes; m == 0 or n == 0 makes the group a no-op (its
 *        pointers are not read), k == 0 writes +0 to every element of c (a, b,
 *        sfa and sfb may then be NULL).
 *   flags  0, or NVFP4_SFB_SWIZZLED; other bits are invalid.
 */
typedef struct nvfp4_group {
    const void *a;
    const void *b;
    const void *sfa;
    const void *sfb;
    void *c;
    int32_t m;
    int32_t n;
    int32_t k;
    int32_t flags;
} nvfp4_group_t;

/* sfb holds the window-major layout (see nvfp4_swizzle_scales). */
#define NVFP4_SFB_SWIZZLED 1

/*
 * Enqueue the grouped GEMM on `stream` (a hipStream_t; NULL = the null
 * stream) and return without synchronising.  `groups` is host memory, read
 * only during the call.
 *
 * Errors (nothing is launched):
 *   NVFP4_EINVAL        ng < 0; groups == NULL with ng > 0; m, n or k < 0;
 *                       k % 16 != 0; c == NULL in a group with m, n > 0; a,
 *                       b, sfa or sfb == NULL in such a group with k > 0;
 *                       flags with a bit other than NVFP4_SFB_SWIZZLED.
 *   NVFP4_EUNSUPPORTED  k % 64 != 0 (the kernel moves k in stages of 64); a
 *                       pointer that breaks the alignment stated above; m,
 *                       n times k/2 reaching 2 GiB; the stream is being
 *                       captured into a graph and has no workspace yet.
 *   NVFP4_EHIP          a workspace allocation or the launch failed (message
 *                       via nvfp4_last_error).
 * Workspace: the first call on a (device, stream) pair allocates a device
 * workspace for that pair (partial sums of split tiles and their flags, 128
 * KiB per compute unit, at most 256 units) and keeps it until
 * nvfp4_release_workspace(stream) or the end of the process; later calls on
 * that pair allocate nothing.  Calls on one stream
 * are ordered by the stream; calls on different streams use different
 * workspaces and may run concurrently.
 * Split tiles: a workgroup that finishes a tile waits (bounded) for the
 * partial sums of the other workgroups sharing it, and computes a part that
 * does not arrive in time itself.  The environment variable
 * NVFP4_SPIN_LIMIT (read at each call) sets the number of polls of that
 * wait; 0 makes every such part be recomputed (used to test that path).
 * Graphs: the call keeps no per-call host state (the epoch that tells a
 * split tile's partial sums of this launch from older ones lives in the
 * workspace and is advanced by the kernel), so it may be captured in a HIP
 * graph and replayed, once its stream's workspace exists (a first call on
 * that stream outside capture creates it; a call on a capturing stream
 * without one returns NVFP4_EUNSUPPORTED and records nothing).  Replays of one captured call are ordered by the
 * stream like calls.
 * Host cost: each launch of up to 32 groups uses at most min(compute units,
 * 256) workgroups, whose work ranges the host balances with a timing model
 * of the kernel (tens of microseconds); the last result is reused, per host
 * thread, while the groups' sizes stay the same.
 * Tiny launches: a launch (up to 32 groups) whose every k is at most 512
 * and whose work is at most 64 units of 128 or fewer rows x 256 columns x
 * 256 k goes to a direct kernel instead: one wave per 16, 32 or 64 rows x 32
 * columns, operands loaded straight into registers, no split tiles, hence
 * no workspace (such a call may be captured on any stream).  Its sums round
 * exactly as the persistent kernel's for k <= 256.  The environment
 * variable NVFP4_PATH (read at each call) forces a path: "main" (the
 * persistent kernel) or "direct" (wherever every k is at most 512 and at
 * most 256 workgroups of 4 waves suffice).
 */
int nvfp4_group_gemm(const nvfp4_group_t *groups, int ng, void *stream);

/*
 * The same operation for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It calls no hipMalloc, hipFree or other allocating routine.
 * Instead of the per-stream workspace it uses one fixed device array of the
 * library (32 MiB of partial-sum slots for up to 256 workgroups, plus 1.3
 * KiB of flags and control words), which every GPU the library runs on
 * holds from the library's load until the process ends.  Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (on any
 * streams, including nvfp4_group_gemm_noalloc calls on two streams) race
 * and must be ordered by the caller.  Arguments, errors, results and graph
 * capture are as for nvfp4_group_gemm (a capturing stream needs no prior
 * call); a launch that would need more workgroups than the array has slots
 * returns NVFP4_EUNSUPPORTED (not on MI355X, whose 256 compute units all fit).
 */
int nvfp4_group_gemm_noalloc(const nvfp4_group_t *groups, int ng, void *stream);

/*
 * Bytes of the window-major layout of a [rows][k/16] scale matrix:
 * ceil(rows/32)*32 rows of ceil(k/256)*16 bytes.  0 for rows or k <= 0.
 */
int64_t nvfp4_swizzled_scale_bytes(int rows, int k);

/*
 * Enqueues on `stream` a copy of the plain row-major scale matrix `sf`
 * ([rows][k/16] E4M3FN bytes, device memory) into `out` (device memory of
 * nvfp4_swizzled_scale_bytes(rows, k) bytes, 16-byte aligned, not
 * overlapping sf) in the window-major layout: for each block of 32 rows and
 * each 256-k window, the window's 16 scale bytes of the 32 rows, row after
 * row; windows of a row block consecutive, row blocks consecutive.  Rows
 * past `rows` repeat the last row, bytes past k/16 are 0.  Meant for a
 * weight operand's scales, reordered once and reused: with
 * NVFP4_SFB_SWIZZLED a wave's 32 columns read a window's scales as one
 * contiguous 512-byte run instead of 32 runs of 16 bytes at a stride of
 * k/16.  Results are identical to the plain layout's.
 * Errors: NVFP4_EINVAL (rows or k < 0, k % 16 != 0, NULL pointer with rows,
 * k > 0), NVFP4_EUNSUPPORTED (misaligned out, or the layout reaching 2 GiB),
 * NVFP4_EHIP.
 */
int nvfp4_swizzle_scales(const void *sf, void *out, int rows, int k, void *stream);

/*
 * Host-only argument check: the same validation nvfp4_group_gemm performs,
 * without touching the GPU.  Returns one of the codes above.
 */
int nvfp4_validate(const nvfp4_group_t *groups, int ng);

/*
 * Host-only view of the work decomposition the persistent kernel would use
 * for a launch on a device with `num_workgroups` compute units (tiny
 * launches take the direct kernel instead; see nvfp4_group_gemm).  Writes up to `cap` segment
 * records of eight int32 each and returns the total number of segments
 * (which may exceed cap), or a negative NVFP4 code negated on invalid input.
 *
 * A record is (workgroup, group, first row, row count, first column,
 * k_begin, k_end, role): workgroup `workgroup` accumulates k in
 * [k_begin, k_end) of the output tile rows [first row, first row + row
 * count) x columns [first column, first column + nvfp4_tile_cols()) of
 * `group` (clipped to n).  role 0: the segment covers the whole k range and
 * writes C; role 1: a partial sum handed to the tile's finalizer; role 2: the
 * finalizer, holding k_begin == 0, which adds the partial sums of the other
 * segments of its tile and writes C.  k_end may exceed k (the last k block
 * is padded).  Groups are launched in batches of at most 32 non-empty groups;
 * the records of each batch follow those of the previous one.
 */
int nvfp4_plan(const nvfp4_group_t *groups, int ng, int num_workgroups, int32_t *segs, int cap);

/*
 * Frees the workspace of (current device, stream), after waiting for the
 * work queued on `stream`.  A later call on that stream creates a new one.
 * Returns NVFP4_OK (also when there is none) or NVFP4_EHIP.
 */
int nvfp4_release_workspace(void *stream);

/*
 * Waits for the work queued on `stream`, then returns (and clears) the number
 * of internal hand-off waits that ran out since the last call, counted in
 * the workspace of (current device, stream) and in the device's
 * allocation-free workspace.  Inside a workgroup the waves hand decoded A
 * operands to each other through LDS counters with a bounded wait; a wait
 * that runs out (never expected: it would mean a bug, and the affected
 * outputs are then wrong) is counted here instead of hanging the GPU.  The
 * environment variable NVFP4_SYNC_SPIN_LIMIT (read at each call of the GEMM)
 * sets the polls of that wait; a tiny value forces it to run out (a test of
 * this path).  Returns the count (>= 0) or a negated NVFP4 code.
 */
int nvfp4_stream_errors(void *stream);

/* Largest row and column extent of one tile. */
int nvfp4_tile_rows(void);
int nvfp4_tile_cols(void);

/*
 * Message describing the last non-OK return on the calling thread ("" if
 * none).  The pointer stays valid until the next call on that thread.
 */
const char *nvfp4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_GROUP_GEMM_H */
