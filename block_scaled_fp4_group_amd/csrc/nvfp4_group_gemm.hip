// nvfp4_group_gemm.hip -- gfx950 (MI355X) kernels and C ABI of the NVFP4
// grouped GEMM declared in include/nvfp4_group_gemm.h.
//
// Operation (pages "nvfp4 group gemm", kernelindex.com submissions 474067,
// 482269, 496386): per group, C = A * B^T with A [M][K] and B [N][K] given as
// E2M1 codes with one E4M3FN scale per 16 consecutive k, fp32 accumulation,
// fp16 output rounded to nearest-even (submission 474067: header comment, the
// block16 MMA helper and the epilogue of group_gemm_persistent_kernel).
//
// gfx950 design (not the pages' tcgen05/TMA/TMEM design):
//  * CDNA4's block-scaled MFMA takes power-of-two (E8M0) scales per 32 k,
//    while NVFP4 carries E4M3 scales per 16 k.  Every E2M1 x E4M3FN product
//    has at most 6 significant bits and lies in [2^-10, 2688], so it is exact
//    in fp16.  Operands are decoded exactly to fp16 (hardware FP4->f16
//    convert, then one packed f16 multiply by the scale) and fed to
//    v_mfma_f32_16x16x32_f16 with fp32 accumulation.
//  * Workgroup = 8 waves, output tile = up to 128 rows x 256 columns of one
//    group.  Per 128-k stage the waves decode the tile's A rows once into LDS
//    (fragment-major, so every MFMA operand read is one conflict-free
//    ds_read_b128), while each wave decodes its own 32 columns of B into
//    registers.  Raw codes and scales arrive by direct HBM-to-LDS loads,
//    issued two stages ahead into a wave-private ring; the decoded A
//    operands are double-buffered.  The waves hand the shared A operands
//    over through two LDS counters instead of a barrier per stage, so they
//    drift apart and one wave's decode overlaps another's MFMAs.
//  * One workgroup per CU, each with one contiguous range of the launch's
//    (tile, 256-k pair) units ("stream-K"); the host balances the ranges
//    with a clock model of the kernel, and a tile split between workgroups
//    is summed by the one holding its first pair.
//  * Inside a 128-k stage lane (r, q) of a wave holds k = 32q + 8s + [0, 8)
//    at MFMA step s; A and B use the same permutation of k, which leaves the
//    sum unchanged and lets every lane read 16 contiguous bytes per row.
//  * Accuracy: the MFMA accumulators restart from zero every 512 k and are
//    then added into a separate fp32 sum, so rounding happens at the
//    magnitude of 512-k partial sums instead of the full sum.  An output
//    whose exact value is small next to the tile's typical partial sums
//    (heavy cancellation) can still carry more absolute error than the
//    tolerance allows; each finished tile estimates that error from its own
//    sums and recomputes the few outputs at risk exactly (fix_small_outputs).
//  * Launches too small to fill the chip (every K <= 512, at most 64 units)
//    run on nvfp4_direct_kernel instead: one wave per 16-64 rows x 32
//    columns with its operands in registers, the same decode, MFMA chain,
//    epilogue and exact fix-up, and no workspace.
//  * B's scales may also come in a window-major layout (NVFP4_SFB_SWIZZLED,
//    written once by nvfp4_swizzle_scales): a wave's 32 columns then read a
//    256-k window's scales as one contiguous 512-byte run.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <vector>
#include <mutex>
#include <type_traits>
#include <utility>

#include "nvfp4_group_gemm.h"

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;            // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kTileM = 128;          // max rows of one tile (8 blocks of 16)
constexpr int kRowBlocks = kTileM / 16;
constexpr int kTileN = 32 * kWaves;  // columns of one tile (32 per wave)
constexpr int kStageK = 128;         // k per pipeline stage (4 MFMA steps)
constexpr int kFoldStages = 4;       // stages summed by MFMA before a fold (512 k)
constexpr int kMaxGroupsPerLaunch = 32;
constexpr int kMaxWorkgroups = 256;   // workgroups of one launch (one per CU on MI355X)

// Work decomposition.  A group's output is cut into tiles of up to kTileM
// rows (the rows spread evenly over the fewest tiles) by kTileN columns; K
// is cut into stage pairs of 2 * kStageK.  The (tile, stage pair) units of a
// launch are ordered group by group, column strip by column strip, row tile
// by row tile, pair by pair, and every workgroup takes one contiguous range
// of that order ("stream-K").  The host chooses the ranges (plan_cuts) by
// balancing a clock model of each workgroup.  A tile whose pairs fall into
// several ranges is finished by the workgroup holding its first pair; the
// others leave fp32 partial sums in a workspace.
// Positions in the order are cost coordinates: a tile is [head][pair 0]
// [pair 1]..., a pair of a tile with nrb row blocks spans pair_cost(nrb,
// npairs) units and a head kCostHead, and a pair belongs to the range
// (lo, hi] that holds its end.  The host places cuts on pair ends, so these
// weights only fix the coordinates (their values were an earlier cost
// estimate, in units of about 127 clocks).
constexpr int kCostRowBlock = 4;
constexpr int kCostFixed = 29;
constexpr int kCostHead = 60;
constexpr int kCostSpread = 40;

struct GroupArgs {
    const uint8_t *a;
    const uint8_t *b;
    const uint8_t *sfa;
    const uint8_t *sfb;
    _Float16 *c;
    int32_t m, n, k;
    int32_t row_tiles;   // tiles along M
    int32_t tile_rows;   // rows per tile (multiple of 16, <= kTileM)
    int32_t col_tiles;   // tiles along N
    int32_t npairs;      // stage pairs along K (>= 1)
    int32_t cost_full;   // cost of one pair of a tile with tile_rows rows
    int32_t cost_last;   // cost of one pair of the last row tile
    int32_t flags;       // NVFP4_SFB_SWIZZLED: sfb in the window-major layout
    int64_t strip_cost;  // cost of one column strip (all row tiles with heads)
    int64_t cost_begin;  // cost before this group's first tile
};

// The window-major scale layout (NVFP4_SFB_SWIZZLED): for each block of 32
// rows and each 256-k window, the 16 scale bytes of the window of the 32
// rows are contiguous, row after row (512 bytes), windows of one row block
// after each other, row blocks after each other.  Rows are padded to a
// multiple of 32 by repeating the last row and K to a multiple of 256 with
// zero bytes.  Byte (row, b) of the plain [rows][k/16] matrix (b = scale
// block along k) sits at swz_offset(row, b).  A wave's 32 columns then
// fetch a window's scales as one contiguous 512-byte run.
__host__ __device__ inline uint32_t swz_windows(int k)
{
    return (uint32_t)(k + 255) / 256u;
}
__host__ __device__ inline uint32_t swz_offset(uint32_t row, uint32_t b, uint32_t windows)
{
    return ((row >> 5) * windows + (b >> 4)) * 512u + (row & 31u) * 16u + (b & 15u);
}
__host__ __device__ inline uint64_t swz_bytes(int rows, int k)
{
    return (uint64_t)((rows + 31) / 32) * 32u * swz_windows(k) * 16u;
}

// Where one workgroup's range starts: its logical index w (workgroups are
// dealt round-robin to the XCDs, and consecutive logical ranges share A rows
// and B columns, so the host maps block b to w = (b % 8) (num_wg / 8) + b / 8
// when num_wg % 8 == 0), its first tile and pair (pack_start) and the end of
// its pairs in that tile (pe = 0: no work).
struct WgStart {
    uint64_t pos;
    int32_t w;
    int32_t pe;
};

struct LaunchArgs {
    GroupArgs g[kMaxGroupsPerLaunch];
    // g[i].cost_begin again, contiguous (INT64_MAX past the last group), so
    // that finding a cost's group is one batch of independent loads
    int64_t group_begin[kMaxGroupsPerLaunch];
    int32_t ng;
    int32_t num_wg;      // workgroups of the launch
    int64_t total_cost;
    float *partials;     // num_wg slots of kPartialSlot bytes
    uint32_t *flags;     // num_wg flags: slot holds this launch's partial when == its epoch
    // [0]: epoch of the last finished launch on this workspace, [1]:
    // workgroups of this launch that have finished (device-resident, so a
    // launch replayed from a captured graph still gets a fresh epoch), [2]:
    // hand-off waits that ran out (a sticky count, read and cleared by
    // nvfp4_stream_errors)
    uint32_t *control;
    int32_t spin_limit;  // flag polls before a missing part is recomputed instead
    int32_t sync_spin_limit;  // polls of an A hand-off wait before it gives up (and counts an error)
    // Workgroup w's range is the cost interval (cut[w], cut[w + 1]]: the
    // pairs whose end cost lies in it belong to w (cut[0] = 0, cut[num_wg] =
    // total_cost, non-decreasing; chosen on the host)
    int64_t cut[kMaxWorkgroups + 1];
    // indexed by blockIdx.x: the logical workgroup it runs and where its
    // range starts, found by the host so that a workgroup reaches its first
    // loads of operand data after two dependent rounds of argument loads
    WgStart first[kMaxWorkgroups];
};

__host__ __device__ inline int pair_cost(int nrb, int npairs)
{
    return kCostRowBlock * nrb + kCostFixed + (kCostSpread + npairs - 1) / npairs;
}

__host__ __device__ inline int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Position of one tile and of a pair in it.
struct TilePos {
    int g, strip, rt;       // group, column strip, row tile
    int pair;               // first pair of interest
    int64_t cost_begin;     // cost where the tile (its head) starts
    int pcost;              // cost of each of its pairs
    int nrb;                // 16-row blocks of the tile
};

__host__ __device__ inline int tile_nrb(const GroupArgs &G, int rt)
{
    const int rows = G.m - rt * G.tile_rows < G.tile_rows ? G.m - rt * G.tile_rows : G.tile_rows;
    return (rows + 15) >> 4;
}

// First pair of a tile starting at cost `start` (pairs of cost pc) whose
// end cost is > x; npairs when there is none.
__host__ __device__ inline int first_pair_ending_after(int64_t start, int pc, int npairs, int64_t x)
{
    const int64_t off = x - start - kCostHead;     // pair j ends at (j + 1) pc
    if (off < 0)
        return 0;
    const int64_t j = off / pc;
    return (int)(j < npairs ? j : npairs);
}

__host__ __device__ inline void finish_pos(const GroupArgs &G, TilePos &p)
{
    const int64_t full = kCostHead + (int64_t)G.npairs * G.cost_full;
    p.cost_begin = G.cost_begin + p.strip * G.strip_cost + p.rt * full;
    p.pcost = p.rt == G.row_tiles - 1 ? G.cost_last : G.cost_full;
    p.nrb = tile_nrb(G, p.rt);
}

// The tile holding the first pair whose end cost is > x (g == ng: none).
__host__ __device__ inline TilePos locate(const LaunchArgs &args, int64_t x)
{
    const GroupArgs *gs = args.g;
    const int ng = args.ng;
    const int64_t total = args.total_cost;
    TilePos p{ng, 0, 0, 0, total, 1, 1};
    if (x >= total)
        return p;
    int g = 0;
#pragma unroll
    for (int i = 1; i < kMaxGroupsPerLaunch; ++i)
        g += args.group_begin[i] <= x ? 1 : 0;
    const GroupArgs &G = gs[g];
    int64_t off = x - G.cost_begin;
    p.g = g;
    p.strip = (int)(off / G.strip_cost);
    off -= p.strip * G.strip_cost;
    const int64_t full = kCostHead + (int64_t)G.npairs * G.cost_full;
    if (off < (int64_t)(G.row_tiles - 1) * full) {
        p.rt = (int)(off / full);
        p.pair = first_pair_ending_after(p.rt * full, G.cost_full, G.npairs, off);
    } else {
        p.rt = G.row_tiles - 1;
        p.pair = first_pair_ending_after((int64_t)(G.row_tiles - 1) * full, G.cost_last, G.npairs, off);
    }
    if (p.pair >= G.npairs) {        // no pair of this tile ends after x: start at the next tile
        p.pair = 0;
        if (++p.rt == G.row_tiles) {
            p.rt = 0;
            if (++p.strip == G.col_tiles) {
                p.strip = 0;
                if (++p.g == ng) {
                    p.cost_begin = total;
                    return p;
                }
            }
        }
    }
    finish_pos(gs[p.g], p);
    return p;
}

// The tile after p (pair 0); g == ng past the last tile.
__host__ __device__ inline TilePos next_tile(const GroupArgs *gs, int ng, int64_t total, TilePos p)
{
    p.pair = 0;
    if (++p.rt == gs[p.g].row_tiles) {
        p.rt = 0;
        if (++p.strip == gs[p.g].col_tiles) {
            p.strip = 0;
            if (++p.g == ng) {
                p.cost_begin = total;
                return p;
            }
        }
    }
    finish_pos(gs[p.g], p);
    return p;
}

// A tile position packed into 64 bits: pair [0, 20), row tile [20, 38),
// column strip [38, 58), group [58, 64) (63: no tile).
__host__ __device__ inline uint64_t pack_start(const TilePos &p, int ng)
{
    if (p.g >= ng)
        return 63ull << 58;
    return (uint64_t)p.pair | (uint64_t)p.rt << 20 | (uint64_t)p.strip << 38 | (uint64_t)p.g << 58;
}

// The position packed by pack_start (its cost fields are set by finish_pos).
__host__ __device__ inline TilePos unpack_pos(uint64_t v)
{
    return TilePos{(int)(v >> 58), (int)((v >> 38) & 0xFFFFF), (int)((v >> 20) & 0x3FFFF), (int)(v & 0xFFFFF), 0, 1, 1};
}

// Pairs [*pb, *pe) of the tile at p whose end cost lies in (lo, hi].
__host__ __device__ inline void pairs_in(const TilePos &p, int npairs, int64_t lo, int64_t hi, int &pb, int &pe)
{
    pb = first_pair_ending_after(p.cost_begin, p.pcost, npairs, lo);
    pe = first_pair_ending_after(p.cost_begin, p.pcost, npairs, hi);
}

// Bytes of one workgroup's partial-sum slot: [wave][row block][cb][lane] f32x4.
constexpr int kControlWords = 4;
constexpr uint32_t kPartialSlot = kWaves * kRowBlocks * 2u * 64u * 16u;

// ---------------------------------------------------------------- device --

// Eight E2M1 codes (one dword, element i in nibble i) times one scale, as
// eight exact fp16 values.  The convert instruction applies a power-of-two
// scale only, so it runs with 1.0 and the E4M3 scale is applied by a packed
// f16 multiply (exact: <= 6 significant bits, result in the normal range).
__device__ __forceinline__ f16x8 decode8(uint32_t codes, f16x2 s)
{
    f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s;
    f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s;
    f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s;
    f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s;
    f16x8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    return r;
}

// Two E4M3FN scale bytes (low 16 bits) -> fp16 pair.
__device__ __forceinline__ f16x2 scales2(uint32_t bytes)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bytes, 1.0f, false);
}

__device__ __forceinline__ f16x2 bcast(_Float16 x)
{
    f16x2 r = {x, x};
    return r;
}

// ---- LDS layout ----------------------------------------------------------
// [0, 64 KiB): decoded A operand fragments of two stages,
//              [stage][row block][MFMA step][lane] x 16 bytes.
// then kRing raw code stages, each holding what every wave fetched for one
// stage (lane l's 16 bytes at 16 l):
//   A codes  [wave][lane] x 16 B   (the rows of the wave's A-decode role)
//   B codes  [wave][cb][lane] x 16 B   (the wave's own 32 columns)
// then two scale windows, each holding the scale bytes of two consecutive
// stages (16 bytes per row, fetched by lanes 0..15, one row each):
//   A scales [wave][16 rows] x 16 B,  B scales [wave][cb][16 rows] x 16 B
// then two counters of decoded A halves (MFMA steps 0-1 and 2-3) that
// order the waves' shared use of the A operand buffers.
constexpr int kRing = 3;
constexpr uint32_t kLdsAOps = 2u * kRowBlocks * 4u * 64u * 16u;
constexpr uint32_t kRawACodes = 0;
constexpr uint32_t kRawBCodes = kRawACodes + kWaves * 1024u;
constexpr uint32_t kRawStage = kRawBCodes + kWaves * 2u * 1024u;
constexpr uint32_t kWinAScales = 0;
constexpr uint32_t kWinBScales = kWinAScales + kWaves * 256u;
constexpr uint32_t kWindow = kWinBScales + kWaves * 2u * 256u;
constexpr uint32_t kLdsWindows = kLdsAOps + kRing * kRawStage;
constexpr uint32_t kLdsSync = kLdsWindows + 2u * kWindow;
constexpr uint32_t kLdsBytes = kLdsSync + 16u;
// Loads a wave issues: kCodeLoads code loads every stage, kScaleLoads
// scale loads every odd stage (after its code loads, for the pair starting
// three stages on).  With kRing = 3 stages in flight, at the top of every
// stage c exactly kWaitAfterNext loads have been issued after the last load
// that stage c + 1 needs: the codes of c + 1 when c is even, the scale
// window of the pair starting at c + 1 when c is odd.
constexpr int kCodeLoads = 3;
constexpr int kScaleLoads = 2;
constexpr int kWaitAfterNext = 2 * kCodeLoads + kScaleLoads;

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes at `p` (raw buffer, no stride); reads
// past the end return zero.
__device__ __forceinline__ i32x4 rsrc(const void *p, uint32_t bytes)
{
    const uint64_t a = (uint64_t)(uintptr_t)p;
    i32x4 r = {(int32_t)(uint32_t)a, (int32_t)(uint32_t)(a >> 32) & 0xFFFF, (int32_t)bytes, 0x00020000};
    return r;
}

// Direct HBM -> LDS loads: lane l's 16 bytes at voff + soff land at LDS
// byte lds + 16 l.  Issued from inline assembly that sets m0 (the LDS
// address) and restores it, so the compiler neither loses a value it keeps
// in m0 nor orders later LDS reads behind these writes (it cannot tell the
// ring slots apart); callers wait with an explicit vmcnt before reading.
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, i32x4 rs, uint32_t soff)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(lds), "v"(voff), "s"(rs), "s"(soff) : "memory");
}
// The same for lanes 0..15 only (exec narrowed and restored inside the asm,
// so the compiler sees no divergent branch around a load it cannot see).
__device__ __forceinline__ void dma16_lanes16(uint32_t lds, uint32_t voff, i32x4 rs, uint32_t soff)
{
    uint64_t saved;
    uint32_t saved_m0;
    asm volatile("s_mov_b64 %0, exec\n\ts_mov_b64 exec, 0xffff\n\ts_mov_b32 %1, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %3, %4, %5 offen lds\n\ts_mov_b32 m0, %1\n\ts_mov_b64 exec, %0"
                 : "=&s"(saved), "=&s"(saved_m0) : "s"(lds), "v"(voff), "s"(rs), "s"(soff) : "memory");
}
// The same for lanes 0..31.
__device__ __forceinline__ void dma16_lanes32(uint32_t lds, uint32_t voff, i32x4 rs, uint32_t soff)
{
    uint64_t saved;
    uint32_t saved_m0;
    asm volatile("s_mov_b64 %0, exec\n\ts_mov_b64 exec, 0xffffffff\n\ts_mov_b32 %1, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %3, %4, %5 offen lds\n\ts_mov_b32 m0, %1\n\ts_mov_b64 exec, %0"
                 : "=&s"(saved), "=&s"(saved_m0) : "s"(lds), "v"(voff), "s"(rs), "s"(soff) : "memory");
}
// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    __builtin_amdgcn_sched_barrier(0);
}

// Lane index, opaque to the optimiser: addresses derived from it are formed
// where they are used instead of being hoisted out of the persistent loop
// (for every tile shape at once) and kept live in registers.
__device__ __forceinline__ int lane_id()
{
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));
    return l;
}

// The decoded A operands are the only LDS data the waves share inside the
// stage loop (codes and scales are wave-private DMA targets).  Instead of a
// workgroup barrier per stage, counter h (h = 0: MFMA steps 0-1, h = 1:
// steps 2-3) counts the waves that have written their part of those steps
// for the next stage.  Before a wave reads half h of stage c it waits until
// every wave has written it (count >= waves * (c - first stage)); every wave
// writes half h of stage c + 1 only after reading half h of stage c - 1,
// which shares its buffer, so the same wait also keeps the writes of stage
// c + 1 from overtaking a slower wave's reads of stage c - 1.  LDS performs
// a wave's operations in issue order, so a count is added only after the
// wave's writes.  Waves thus drift up to a stage apart, and one wave's
// decode overlaps another's MFMAs.  The wait is bounded: a count that never
// arrives (which would be a bug) gives wrong sums instead of a hang, and is
// recorded in a device error word the host can read (nvfp4_stream_errors).
constexpr int kSyncSpinLimit = 1 << 14;   // default polls (NVFP4_SYNC_SPIN_LIMIT overrides)
// Both are single asm statements so that the hot loop stays one basic
// block for the compiler; the LDS operations they add only make the
// compiler's own (in-order) LDS waits more conservative.
// `pre` is the counter as read some MFMA steps earlier by a plain LDS load:
// the counter only grows, so if that value already meets the target the
// wait ends without a new read (whose lgkmcnt(0) would drain every LDS
// operation in flight), and the compiler's wait for `pre` covers only the
// LDS operations issued before it.
// Polls at most `limit` + 1 times; returns true if the wait ran out.
__device__ __forceinline__ bool half_wait(uint32_t count_addr, int target, int pre, int limit)
{
    int v;
    int seen, left = limit + 1;
    asm volatile("v_readfirstlane_b32 %1, %5\n\t"
                 "s_cmp_ge_i32 %1, %4\n\t"
                 "s_cbranch_scc1 2f\n"
                 "1:\n\t"
                 "ds_read_b32 %0, %3\n\t"
                 "s_waitcnt lgkmcnt(0)\n\t"
                 "v_readfirstlane_b32 %1, %0\n\t"
                 "s_cmp_ge_i32 %1, %4\n\t"
                 "s_cbranch_scc1 2f\n\t"
                 "s_sleep 1\n\t"
                 "s_sub_i32 %2, %2, 1\n\t"
                 "s_cmp_gt_i32 %2, 0\n\t"
                 "s_cbranch_scc1 1b\n"
                 "2:"
                 : "=&v"(v), "=&s"(seen), "+s"(left)
                 : "v"(count_addr), "s"(target), "v"(pre)
                 : "memory", "scc");
    return left <= 0;
}
// Early read of a counter for half_wait (a volatile LDS load, so it stays
// where it is issued relative to the other LDS operations).
typedef __attribute__((address_space(3))) const volatile int lds_cvint;
__device__ __forceinline__ int count_read(uint32_t count_addr)
{
    return *reinterpret_cast<lds_cvint *>((uintptr_t)count_addr);
}
__device__ __forceinline__ void half_done(uint32_t count_addr, uint32_t one)
{
    uint64_t saved;
    asm volatile("s_mov_b64 %0, exec\n\t"
                 "s_mov_b64 exec, 1\n\t"
                 "ds_add_u32 %1, %2\n\t"
                 "s_mov_b64 exec, %0"
                 : "=&s"(saved)
                 : "v"(count_addr), "v"(one)
                 : "memory");
}

// Stage pairs [pb, pe) of one output tile with NRB row blocks (compile
// time, so the hot loop has no branches), added into `outer`.  W waves; the
// tile is rows [m0, m0 + 16 NRB) and columns [n0, n0 + 32 W) of one group.
// Lane (r, q) of wave w holds outer[i][cb][e] = C[m0 + 16i + 4q + e][n0 + 32w + 16cb + r].
template <int NRB, int W>
__device__ __forceinline__ void segment(const GroupArgs &G, uint32_t *err, int sync_limit, int m0, int n0, int wave,
                                        uint8_t *smem,
                                        int pb, int pe, f32x4 (&outer)[NRB][2])
{
    const int M = G.m, N = G.n, K = G.k;
    const int lane = lane_id();
    const int r = lane & 15, q = lane >> 4;
    const uint32_t row_bytes = (uint32_t)K >> 1, row_scales = (uint32_t)K >> 4;
    const int nstages = (K + kStageK - 1) / kStageK;
    const int c_begin = 2 * pb, c_end = min(2 * pe, (nstages + 1) & ~1);

    if (c_begin < c_end) {
    const i32x4 ra_codes = rsrc(G.a, (uint32_t)M * row_bytes);
    const i32x4 ra_scales = rsrc(G.sfa, (uint32_t)M * row_scales);
    const i32x4 rb_codes = rsrc(G.b, (uint32_t)N * row_bytes);
    const bool sfb_swz = (G.flags & NVFP4_SFB_SWIZZLED) != 0;
    const uint32_t swz_w = swz_windows(K);
    const i32x4 rb_scales = rsrc(G.sfb, sfb_swz ? (uint32_t)swz_bytes(N, K) : (uint32_t)N * row_scales);

    // A decode role: wave w decodes row block w % NRB (all four MFMA steps).
    // For NRB < W several waves decode the same block and store identical
    // bytes, which keeps the hot loop free of branches.
    const int a_rb = wave % NRB;
    const uint32_t arow = (uint32_t)min(m0 + 16 * a_rb + r, M - 1);
    // Lane (r, q) covers k0 + 32q + [0, 32): 16 code bytes at k0/2 + 16q and
    // the two scale bytes at k0/16 + 2q of its row.
    const uint32_t a_voff = arow * row_bytes + 16u * q;
    const uint32_t sa_voff = arow * row_scales;
    uint32_t b_voff[2], sb_voff[2];
    // B scale rows for one 32-lane load: lane 16 cb + r fetches column block
    // cb's row r (lanes 32..63 are masked off)
    // (window-major layout: the wave's 32 columns are one 32-row block, so
    // lane l's 16 bytes are at 16 l of the window's 512-byte run)
    const uint32_t sb_voff32 = sfb_swz ? 16u * (uint32_t)(16 * (q & 1) + r)
                                       : (uint32_t)min(n0 + 32 * wave + 16 * (q & 1) + r, N - 1) * row_scales;
    const uint32_t sb_base = sfb_swz ? (uint32_t)((n0 + 32 * wave) >> 5) * swz_w * 512u : 0u;
    const uint32_t sb_stride = sfb_swz ? 512u : 16u;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const uint32_t col = (uint32_t)min(n0 + 32 * wave + 16 * cb + r, N - 1);
        b_voff[cb] = col * row_bytes + 16u * q;
        sb_voff[cb] = col * row_scales;
    }
    const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
    const uint32_t raw_base = smem_base + kLdsAOps;
    int *sync = reinterpret_cast<int *>(smem + kLdsSync);
    const uint32_t sync_addr = smem_base + kLdsSync;
    const uint32_t one = 1u;
    f16x8 *lds_a = reinterpret_cast<f16x8 *>(smem);            // [2][kRowBlocks][4][64]
    auto aop = [&](int buf, int rb, int s) -> f16x8 & {
        return lds_a[((buf * kRowBlocks + rb) * 4 + s) * 64 + lane];
    };

    f32x4 inner[NRB][2];
    bool late = false;  // a hand-off wait ran out
    f16x8 bf[2][4];     // decoded B operands of the current stage, per MFMA step
    f16x8 af[NRB];

    // Codes of stage c (clamped to the last stage, so the number of loads in
    // flight never depends on K) into ring slot c % kRing.
    auto fetch_codes = [&](int c) {
        const uint32_t k0 = (uint32_t)min(c, nstages - 1) * kStageK;
        const uint32_t slot = raw_base + (uint32_t)(c % kRing) * kRawStage;
        dma16(slot + kRawACodes + wave * 1024u, a_voff, ra_codes, k0 >> 1);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
            dma16(slot + kRawBCodes + (wave * 2 + cb) * 1024u, b_voff[cb], rb_codes, k0 >> 1);
    };
    // Scale window w (stages 2w and 2w + 1: 16 bytes of each row) into window
    // buffer w % 2, fetched by lanes 0..15 (row r = lane).
    auto fetch_scales = [&](int w) {
        const uint32_t wc = (uint32_t)min(w, (nstages - 1) >> 1);
        const uint32_t sk = wc * (2u * kStageK / 16u);
        const uint32_t win = smem_base + kLdsWindows + (uint32_t)(w & 1) * kWindow;
        dma16_lanes16(win + kWinAScales + wave * 256u, sa_voff, ra_scales, sk);
        dma16_lanes32(win + kWinBScales + wave * 2 * 256u, sb_voff32, rb_scales, sb_base + wc * sb_stride);
    };
    auto raw_slot = [&](int c) -> const uint8_t * {
        return smem + kLdsAOps + (uint32_t)(c % kRing) * kRawStage;
    };
    // The scale dword holding lane (r, q)'s two scale bytes of stage c: row r,
    // byte 8 (c % 2) + 2q of window c / 2 (returned shifted into the low half).
    auto read_scales = [&](int c, uint32_t &sa, uint32_t (&sb)[2]) {
        const uint8_t *win = smem + kLdsWindows + (uint32_t)((c >> 1) & 1) * kWindow;
        const uint32_t off = 16u * r + 8u * (c & 1) + 4u * (q >> 1);
        const uint32_t sh = 16u * (q & 1);
        sa = *reinterpret_cast<const uint32_t *>(win + kWinAScales + wave * 256u + off) >> sh;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
            sb[cb] = *reinterpret_cast<const uint32_t *>(win + kWinBScales + (wave * 2 + cb) * 256u + off) >> sh;
    };
    auto a_codes = [&](const uint8_t *slot) -> u32x4 {
        return reinterpret_cast<const u32x4 *>(slot + kRawACodes + wave * 1024u)[lane];
    };
    auto b_codes = [&](const uint8_t *slot, int cb) -> u32x4 {
        return reinterpret_cast<const u32x4 *>(slot + kRawBCodes + (wave * 2 + cb) * 1024u)[lane];
    };
    // The two scales of a raw block of stage c as fp16; zero for lanes whose
    // 32 k lie past K (K % 64 == 0: a lane's 32 k are all in or all out).
    auto scales_of = [&](uint32_t two, int c) -> f16x2 {
        const bool valid = c * kStageK + 32 * q < K;
        return scales2(valid ? two : 0u);
    };
    // Operand of MFMA step s (k = 32q + 8s + [0, 8)) from its code dword.
    auto operand = [&](uint32_t codes, f16x2 sc, int s) -> f16x8 {
        return decode8(codes, bcast(sc[s >> 1]));
    };
    auto decode_a_into = [&](const u32x4 &codes, f16x2 sc, int buf, int s) {
        aop(buf, a_rb, s) = operand(codes[s], sc, s);
    };

    // prologue: stages c_begin .. c_begin + 2 in flight; c_begin decoded (A to
    // LDS buffer 0, B to bf)
    // Issue order keeps exactly kWaitAfterNext loads behind the codes of
    // stage c + 1 at the top of every stage c, this first one included.
    fetch_scales(c_begin >> 1);
    fetch_codes(c_begin);
    fetch_codes(c_begin + 1);
    fetch_scales((c_begin >> 1) + 1);
    fetch_codes(c_begin + 2);
    wait_vmcnt<kWaitAfterNext>();
    {
        const uint8_t *slot = raw_slot(c_begin);
        uint32_t sa, sb[2];
        read_scales(c_begin, sa, sb);
        const f16x2 sca = scales_of(sa, c_begin);
        const u32x4 ac = a_codes(slot);
#pragma unroll
        for (int s = 0; s < 4; ++s)
            decode_a_into(ac, sca, 0, s);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const f16x2 sc = scales_of(sb[cb], c_begin);
            const u32x4 bc = b_codes(slot, cb);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                bf[cb][s] = operand(bc[s], sc, s);
        }
    }
    if (threadIdx.x < 2)
        sync[threadIdx.x] = 0;     // no wave counts again before this barrier
    __syncthreads();
    int pre0 = 0;       // early read of counter 0 for the next stage (the first stage needs none)

    // Stage c: fetch the codes of stage c + 3 into the ring slot stage c used
    // (and, on odd stages, the scale window of stages c + 3 and c + 4 into the
    // window buffer the stages before c used); wait for stage c + 1; per MFMA step s: 2 * NRB MFMAs on the A fragments of step s
    // (read from LDS; a row block's fragment for step s + 1 is read right
    // after its last use), then step s of B (stage c + 1) is decoded into the
    // freed bf slot and step s of A (stage c + 1) into the other LDS buffer
    // (step 0 of A right after the top-of-stage reads, which it covers).
    // Each half of stage c's A is read only after every wave has written it
    // (half_wait), and each written half of stage c + 1 is counted
    // (half_done).  The last stage decodes unused data instead of branching.
    auto stage = [&](int c, auto buf_t, auto first_t) {
        constexpr int kBuf = decltype(buf_t)::value;
        constexpr bool kFirst = decltype(first_t)::value;   // first stage after a fold: MFMA sums restart
        constexpr int kNext = 1 - kBuf;
        fetch_codes(c + 3);
        if (kBuf == 1)
            fetch_scales((c + 3) >> 1);
        wait_vmcnt<kWaitAfterNext>();
        const uint8_t *nslot = raw_slot(c + 1);
        uint32_t sa, sb[2];
        read_scales(c + 1, sa, sb);
        const f16x2 sa_next = scales_of(sa, c + 1);
        f16x2 sb_next[2];
        u32x4 bc_next[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            sb_next[cb] = scales_of(sb[cb], c + 1);
            bc_next[cb] = b_codes(nslot, cb);
        }
        const u32x4 ac_next = a_codes(nslot);
        const int ready = __builtin_amdgcn_readfirstlane(kWaves * (c - c_begin));
        late |= half_wait(sync_addr, ready, pre0, sync_limit);
#pragma unroll
        for (int i = 0; i < NRB; ++i)
            af[i] = aop(kBuf, i, 0);
        // step 0 of the next stage's A while this stage's step-0 reads land
        decode_a_into(ac_next, sa_next, kNext, 0);
        int pre1 = 0;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            __builtin_amdgcn_sched_barrier(0);
            if (s == 1)
                late |= half_wait(sync_addr + 4u, ready, pre1, sync_limit);   // step 2's fragments are read during step 1
#pragma unroll
            for (int i = 0; i < NRB; ++i) {
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    inner[i][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        af[i], bf[cb][s], (kFirst && s == 0) ? f32x4{0.f, 0.f, 0.f, 0.f} : inner[i][cb], 0, 0, 0);
                if (s < 3)
                    af[i] = aop(kBuf, i, s + 1);
                // early counter reads, half a step (second half of this
                // stage's A) or one and a half steps (first half of the next
                // stage's A) before they are checked
                if (i == (NRB - 1) / 2) {
                    if (s == 0)
                        pre1 = count_read(sync_addr + 4u);
                    else if (s == 3)
                        pre0 = count_read(sync_addr);
                }
            }
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                bf[cb][s] = operand(bc_next[cb][s], sb_next[cb], s);
                asm volatile("" : "+v"(bf[cb][s]));   // keep the decode inside step s
            }
            if (s > 0)
                decode_a_into(ac_next, sa_next, kNext, s);
            if (s & 1)
                half_done(sync_addr + 4u * (s >> 1), one);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto fold = [&]() {
#pragma unroll
        for (int i = 0; i < NRB; ++i)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                outer[i][cb] += inner[i][cb];
    };

    // Stages alternate the LDS buffer; the MFMA sums are folded into `outer`
    // every kFoldStages stages (and after a last lone pair).  An odd stage
    // count gets one extra stage whose scales are all zero (its k lie past
    // K), so the loop body has no branch.
    static_assert(kFoldStages == 4, "a fold every two stage pairs");
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    int c = c_begin;
    for (; c + 4 <= c_end; c += 4) {
        stage(c, B0{}, std::true_type{});
        stage(c + 1, B1{}, std::false_type{});
        stage(c + 2, B0{}, std::false_type{});
        stage(c + 3, B1{}, std::false_type{});
        fold();
    }
    if (c < c_end) {
        stage(c, B0{}, std::true_type{});
        stage(c + 1, B1{}, std::false_type{});
        fold();
    }
    // drain the clamped prefetches before the LDS is reused
    wait_vmcnt<0>();
    if (late && (threadIdx.x & 63) == 0)
        __hip_atomic_fetch_add(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    }
}

// fp16 (round to nearest even) of the tile's sums into C, rows < m0 + rows.
// Fast path (n % 4 == 0 and c 8-byte aligned, so every group of four
// columns is wholly inside or outside the matrix): the four lanes of a quad
// (r = 4j .. 4j + 3) hold rows 4q .. 4q + 3 of four consecutive columns, so a
// 4 x 4 transpose of fp16 values across the quad (two DPP exchanges) leaves
// each lane with four consecutive columns of one row, written as one 8-byte
// store instead of four 2-byte ones.
__device__ __forceinline__ uint32_t quad_swap1(uint32_t x)   // value of lane r ^ 1
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t quad_swap2(uint32_t x)   // value of lane r ^ 2
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);
}

template <int NRB>
__device__ __forceinline__ void store_tile(const GroupArgs &G, int m0, int rows, int n0, int wave,
                                           const f32x4 (&outer)[NRB][2])
{
    const int lane = lane_id();
    const int r = lane & 15, q = lane >> 4;
    _Float16 *C = G.c;
    const int N = G.n;
    if ((N & 3) == 0 && ((uintptr_t)C & 7) == 0) {
        const bool odd = (r & 1) != 0, hi2 = (r & 2) != 0;
        // this lane's row and first column after the transpose
        const int row_in = 4 * q + 2 * (r & 1) + ((r >> 1) & 1);
        const int col = n0 + 32 * wave + (r & ~3);
#pragma unroll
        for (int i = 0; i < NRB; ++i) {
            const int row = m0 + 16 * i + row_in;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                const f32x4 v = outer[i][cb];
                const uint32_t p01 = __builtin_bit_cast(uint32_t, f16x2{(_Float16)v[0], (_Float16)v[1]});
                const uint32_t p23 = __builtin_bit_cast(uint32_t, f16x2{(_Float16)v[2], (_Float16)v[3]});
                // step 1: even lanes end with rows 4q, 4q+1 and odd lanes with
                // rows 4q+2, 4q+3, each for the column pair (r & ~1, +1)
                const uint32_t mine = odd ? p23 : p01;
                const uint32_t recv = quad_swap1(odd ? p01 : p23);
                const uint32_t lo = odd ? recv : mine, hi = odd ? mine : recv;
                const uint32_t rowA = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                const uint32_t rowB = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
                // step 2: lanes r and r ^ 2 swap halves of their column quad
                const uint32_t keep = hi2 ? rowB : rowA;
                const uint32_t recv2 = quad_swap2(hi2 ? rowA : rowB);
                const uint64_t out = hi2 ? ((uint64_t)keep << 32 | recv2) : ((uint64_t)recv2 << 32 | keep);
                const int c0 = col + 16 * cb;
                if (row < m0 + rows && c0 < N)
                    *reinterpret_cast<uint64_t *>(C + (size_t)row * N + c0) = out;
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int col = n0 + 32 * wave + 16 * cb + r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + 16 * i + 4 * q + e;
                if (row < m0 + rows && col < N)
                    C[(size_t)row * N + col] = (_Float16)outer[i][cb][e];
            }
        }
    }
}

// Partial sums of split tiles.  Slot w (one per workgroup) holds the sums of
// workgroup w's first segment in the register layout of `outer`:
// [wave][row block][cb][lane] x f32x4.  They are written and read with
// agent-coherent (sc1) buffer accesses, and the flag with relaxed agent-scope
// atomics; ordering comes from waiting for the stores (vmcnt) before the flag
// is set.  No release/acquire fence is used: on gfx950 those write back or
// invalidate the whole L2 of the XCD, which the other workgroups streaming B
// through that L2 would pay for.
constexpr int kCoherent = 16;      // buffer cache-policy bits: sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(const LaunchArgs &args)
{
    return __builtin_amdgcn_make_buffer_rsrc(args.partials, 0, args.num_wg * (int)kPartialSlot, 0x00020000);
}

__device__ __forceinline__ int partial_base(int slot, int wave)
{
    return slot * (int)kPartialSlot + wave * kRowBlocks * 2 * 1024;
}

// Producer side: publish the partial sums of this workgroup's first segment.
template <int NRB>
__device__ __forceinline__ void publish_partial(const LaunchArgs &args, uint32_t epoch, int slot, int wave,
                                                const f32x4 (&outer)[NRB][2])
{
    const int lane = lane_id();
    const __amdgpu_buffer_rsrc_t rs = partial_rsrc(args);
    const int base = partial_base(slot, wave);
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
            __builtin_amdgcn_raw_buffer_store_b128(outer[i][cb], rs, lane * 16, base + (i * 2 + cb) * 1024, kCoherent);
    wait_vmcnt<0>();               // every store of this wave has reached the coherence point
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_store(&args.flags[slot], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Finalizer side: wait (bounded) for producer `slot`; true if its sums arrived.
__device__ __forceinline__ bool await_partial(const LaunchArgs &args, uint32_t epoch, int slot)
{
    __shared__ int ready;
    if (threadIdx.x == 0) {
        int ok = 0;
        // bounded (about 0.1 s by default): a producer that never starts (not
        // resident) makes the caller compute that part itself instead of
        // waiting forever
        for (int it = 0; it < args.spin_limit; ++it) {
            if (__hip_atomic_load(&args.flags[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch) {
                ok = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        ready = ok;
    }
    __syncthreads();
    // uniform by construction; readfirstlane tells the compiler so, which
    // keeps everything derived from it (the next segment's bounds) scalar
    const bool ok = __builtin_amdgcn_readfirstlane(ready) != 0;
    __syncthreads();               // `ready` is read by everyone before the next reuse
    return ok;
}

template <int NRB>
__device__ __forceinline__ void add_partial(const LaunchArgs &args, int slot, int wave, f32x4 (&outer)[NRB][2])
{
    const int lane = lane_id();
    const __amdgpu_buffer_rsrc_t rs = partial_rsrc(args);
    const int base = partial_base(slot, wave);
    // all loads first (the accumulators of the hot loop are dead here, so
    // the registers exist), then the adds: one memory latency, not 2 NRB
    f32x4 v[NRB][2];
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
            v[i][cb] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16, base + (i * 2 + cb) * 1024, kCoherent);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
            outer[i][cb] += v[i][cb];
}

// ---- accuracy fix-up ------------------------------------------------------
// Accumulation in the matrix core rounds to fp32 after every group of 8
// products (measured on gfx950: each lane's 8 products of a 32x32x16 or
// 16x16x32 f16 MFMA are summed exactly, then added to the accumulator with
// one round-to-nearest-even).  With the fold every 512 k the error of a sum
// behaves like a random walk whose scale is set by the magnitude of its
// partial sums.  For an output whose exact value is small next to them
// (heavy cancellation) that error can exceed the absolute part of the
// tolerance (|d| <= 2e-3 |ref| + 1e-2), so each finished tile is checked:
//   sigma = 2^-24 * rms(C) * sqrt(min(F, K) / 16 + K / (2 F) + parts)
// is the error scale of an output whose partial sums are of the tile's
// typical size (F = fold period, rms over the wave's in-range outputs; the
// square-root terms count the roundings inside the MFMA chains and at the
// folds and part sums).  Outputs with 2e-3 |c| + 1e-2 < kSigmaMargin *
// sigma are recomputed exactly.  Calibrated on the hardware's rounding
// model over the five benchmark workloads, the largest error of an output
// small next to rms(C) is 3.3 sigma (the rms error is about 0.25 sigma).
constexpr float kSigmaMargin = 5.0f;
constexpr float kTolRel = 2e-3f;
constexpr float kTolAbs = 1e-2f;

// Exact sum of the products of eight E2M1 code pairs (one dword each): the
// codes are converted to fp16 (exact) and multiplied and summed in fp32 by
// packed dot products; every partial sum is a multiple of 1/4 below 2^9, so
// nothing rounds.
__device__ __forceinline__ float code_dot8_f16(uint32_t xa, uint32_t xb, float acc)
{
    acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(xa, 1.0f, 0),
                                 __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(xb, 1.0f, 0), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(xa, 1.0f, 1),
                                 __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(xb, 1.0f, 1), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(xa, 1.0f, 2),
                                 __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(xb, 1.0f, 2), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(xa, 1.0f, 3),
                                 __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(xb, 1.0f, 3), acc, false);
    return acc;
}

// f64 -> fp16 rounded once: the value is first rounded to f32 with round-to-
// odd (truncation, with the last bit set when anything was dropped), which
// keeps enough to let the f32 -> fp16 rounding to nearest-even decide as a
// direct rounding would.
__device__ __forceinline__ _Float16 f64_to_f16(double x)
{
    float f = (float)x;
    if (__builtin_isfinite(f) && (double)f != x) {
        uint32_t u = __builtin_bit_cast(uint32_t, f);
        if (__builtin_fabs((double)f) > __builtin_fabs(x))
            u -= 1u;               // the value truncated toward zero
        f = __builtin_bit_cast(float, u | 1u);
    }
    return (_Float16)f;
}

// f64 value of lane (lane ^ pattern) for a DPP lane pattern.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, (uint64_t)hi << 32 | lo);
}

__device__ __forceinline__ double readlane_f64(double x, int l)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, (uint64_t)hi << 32 | lo);
}

// Exact values of the n outputs listed in lanes 0..n-1 (row lrow, column
// lcol of one group), rounded once to fp16 and stored over what the tile's
// store wrote there (the same wave's later store to the same address wins).
// Per 16-k block the sum of the 16 code products is exact in fp32 (multiples
// of 1/4, |sum| <= 576), and so is its product with both block scales (at
// most 20 significant bits); the blocks are summed in fp64.
// Outputs are taken eight at a time; each of a batch's outputs gets L = 64 /
// (batch size rounded up to a power of two, at least 8) lanes, and lane s
// of an output takes blocks 4 s + 4 L t + [0, 4) for t = 0, 1, ...  The
// loads of four such steps are issued one group ahead of the arithmetic, so
// one memory latency covers most of a batch.  The L lanes' sums are then
// combined (DPP within 16 lanes, lane reads beyond) and lane 0 of each
// output stores it.  kCompact: one step per load group and no loads ahead,
// for the out-of-line copy, which must fit in few registers.
template <bool kCompact>
__device__ __forceinline__ void store_exact(const uint8_t *a, const uint8_t *sfa, const uint8_t *b, const uint8_t *sfb,
                                            _Float16 *c, int M, int N, int K, int lrow, int lcol, int n, bool sfb_swz)
{
    const int lane = lane_id();
    const int nb = K >> 4;
    const uint32_t row_bytes = (uint32_t)K >> 1, row_sc = (uint32_t)K >> 4;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void *)a, 0, M * (int)row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void *)b, 0, N * (int)row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc((void *)sfa, 0, M * (int)row_sc, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
        (void *)sfb, 0, sfb_swz ? (int)swz_bytes(N, K) : N * (int)row_sc, 0x00020000);
    const uint32_t swz_w = swz_windows(K);
    for (int base = 0; base < n; base += 8) {
        const int cnt = n - base < 8 ? n - base : 8;
        const int lg = cnt == 1 ? 6 : (cnt == 2 ? 5 : (cnt <= 4 ? 4 : 3));   // log2 of the lanes per output
        const int L = 1 << lg;
        const int j = lane >> lg, sl = lane & (L - 1);
        const int idx = base + (j < cnt ? j : cnt - 1);     // spare lanes repeat the batch's last output
        const uint32_t row = (uint32_t)__builtin_amdgcn_ds_bpermute(idx << 2, lrow);
        const uint32_t col = (uint32_t)__builtin_amdgcn_ds_bpermute(idx << 2, lcol);
        const int steps = (nb + 4 * L - 1) / (4 * L);       // 4-block steps of one lane
        constexpr int kSteps = kCompact ? 1 : 4;             // steps per load group
        constexpr int kBufs = kCompact ? 1 : 2;
        const int groups = (steps + kSteps - 1) / kSteps;
        u32x4 ca[kBufs][kSteps][2], cb[kBufs][kSteps][2];
        uint32_t sa[kBufs][kSteps], sb[kBufs][kSteps];
        // group g's loads into buffer buf; steps past the lane's blocks load
        // from offset 0 (in bounds) and are not summed
        auto load = [&](auto buf_t, int g) {
            constexpr int buf = decltype(buf_t)::value;
#pragma unroll
            for (int t = 0; t < kSteps; ++t) {
                const int blk = 4 * sl + 4 * L * (kSteps * g + t);
                const uint32_t bo = blk < nb ? (uint32_t)blk : 0u;
                const uint32_t oa = row * row_bytes + 8u * bo, ob = col * row_bytes + 8u * bo;
                ca[buf][t][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, oa, 0, 0));
                ca[buf][t][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, oa + 16u, 0, 0));
                cb[buf][t][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, ob, 0, 0));
                cb[buf][t][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, ob + 16u, 0, 0));
                sa[buf][t] = __builtin_amdgcn_raw_buffer_load_b32(rsa, row * row_sc + bo, 0, 0);
                sb[buf][t] = __builtin_amdgcn_raw_buffer_load_b32(
                    rsb, sfb_swz ? swz_offset(col, bo, swz_w) : col * row_sc + bo, 0, 0);
            }
        };
        auto sum = [&](auto buf_t, int g) -> double {
            constexpr int buf = decltype(buf_t)::value;
            double acc = 0.0;
#pragma unroll
            for (int t = 0; t < kSteps; ++t) {
                const int blk = 4 * sl + 4 * L * (kSteps * g + t);
                float prod[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x4 &xa = ca[buf][t][q >> 1], &xb = cb[buf][t][q >> 1];
                    const int d = 2 * (q & 1);
                    prod[q] = code_dot8_f16(xa[d + 1], xb[d + 1], code_dot8_f16(xa[d], xb[d], 0.0f));
                }
                const float s0 = __builtin_amdgcn_cvt_scalef32_f32_fp8(sa[buf][t], 1.0f, 0) *
                                 __builtin_amdgcn_cvt_scalef32_f32_fp8(sb[buf][t], 1.0f, 0);
                const float s1 = __builtin_amdgcn_cvt_scalef32_f32_fp8(sa[buf][t], 1.0f, 1) *
                                 __builtin_amdgcn_cvt_scalef32_f32_fp8(sb[buf][t], 1.0f, 1);
                const float s2 = __builtin_amdgcn_cvt_scalef32_f32_fp8(sa[buf][t], 1.0f, 2) *
                                 __builtin_amdgcn_cvt_scalef32_f32_fp8(sb[buf][t], 1.0f, 2);
                const float s3 = __builtin_amdgcn_cvt_scalef32_f32_fp8(sa[buf][t], 1.0f, 3) *
                                 __builtin_amdgcn_cvt_scalef32_f32_fp8(sb[buf][t], 1.0f, 3);
                const double part = (double)(prod[0] * s0) + (double)(prod[1] * s1) + (double)(prod[2] * s2) +
                                    (double)(prod[3] * s3);
                acc += blk < nb ? part : 0.0;
            }
            return acc;
        };
        std::integral_constant<int, 0> b0;
        std::integral_constant<int, 1> b1;
        double acc = 0.0;
        if constexpr (kCompact) {
            for (int g = 0; g < groups; ++g) {
                load(b0, g);
                acc += sum(b0, g);
            }
        } else {
            // every load issued is summed: a load left in flight at the end
            // would make later code wait for all memory operations
            load(b0, 0);
            for (int g = 0; g < groups; g += 2) {
                if (g + 1 < groups)
                    load(b1, g + 1);
                acc += sum(b0, g);
                if (g + 1 < groups) {
                    if (g + 2 < groups)
                        load(b0, g + 2);
                    acc += sum(b1, g + 1);
                }
            }
        }
        // sum over each output's L lanes: xor 1, xor 2, then the mirrors
        // within 8 and 16 lanes (each lane already holds its quad's or
        // half's sum), then lane reads across rows of 16
        acc += dpp_f64<0xB1>(acc);        // quad_perm [1, 0, 3, 2]
        acc += dpp_f64<0x4E>(acc);        // quad_perm [2, 3, 0, 1]
        acc += dpp_f64<0x141>(acc);       // row_half_mirror
        if (L >= 16)
            acc += dpp_f64<0x140>(acc);   // row_mirror
        if (L == 32)
            acc = j == 0 ? readlane_f64(acc, 0) + readlane_f64(acc, 16) : readlane_f64(acc, 32) + readlane_f64(acc, 48);
        else if (L == 64)
            acc = (readlane_f64(acc, 0) + readlane_f64(acc, 16)) + (readlane_f64(acc, 32) + readlane_f64(acc, 48));
        if (sl == 0 && j < cnt)
            c[(size_t)row * N + col] = f64_to_f16(acc);
    }
}

// The batches of a list beyond its first 64 entries (rare: more than 64
// outputs of one wave at risk), one copy for every tile height.
__device__ __noinline__ void store_exact_more(const uint8_t *a, const uint8_t *sfa, const uint8_t *b,
                                              const uint8_t *sfb, _Float16 *c, int M, int N, int K, int lrow,
                                              int lcol, int n, bool sfb_swz)
{
    store_exact<true>(a, sfa, b, sfb, c, M, N, K, lrow, lcol, n, sfb_swz);
}

// Outputs one wave must recompute after its tile's store: entry p of the
// list (row, column) in lane p, n entries.
struct FixList {
    int lrow, lcol, n;
};

// The check for one finished tile (see above); `parts` is the number of
// partial sums the finalizer added.  Lane (r, q) holds outer[i][cb][e] =
// C[m0 + 16 i + 4 q + e][n0 + 32 wave + 16 cb + r].  The outputs at risk
// are listed (position p of the list in lane p); the first 64 are returned
// for the caller to recompute (store_exact), any further ones are
// recomputed here.  Called after the tile's store.
template <int NRB>
__device__ __forceinline__ FixList fix_small_outputs(const GroupArgs &G, int m0, int rows, int n0, int wave,
                                                     int parts, f32x4 (&outer)[NRB][2])
{
    FixList first{0, 0, 0};
    const int lane = lane_id();
    const int r = lane & 15, q = lane >> 4;
    const int row_end = m0 + rows;
    const int col_base = n0 + 32 * wave + r;
    // rms over every sum the wave holds: rows and columns past the group
    // repeat its last row or column (the operand loads are clamped), which
    // leaves the estimate unbiased enough for a threshold
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ss = __builtin_fmaf(outer[i][cb][e], outer[i][cb][e], ss);
    // inclusive scan within each row of 16 lanes, then the four row totals
    ss += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, ss), 0x111, 0xF, 0xF, true));
    ss += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, ss), 0x112, 0xF, 0xF, true));
    ss += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, ss), 0x114, 0xF, 0xF, true));
    ss += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, ss), 0x118, 0xF, 0xF, true));
    {
        const int si = __builtin_bit_cast(int, ss);
        ss = __builtin_bit_cast(float, __builtin_amdgcn_readlane(si, 15)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(si, 31)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(si, 47)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(si, 63));
    }
    const float cnt = (float)(NRB * 8 * 64);
    if (!__builtin_isfinite(ss))
        ss = 0x1p100f;             // a non-finite sum: every output of the wave is checked exactly
    const float K = (float)G.k;
    const float F = (float)(kFoldStages * kStageK);
    const float sigma = 0x1p-24f * __builtin_amdgcn_sqrtf(ss * (1.0f / cnt)) *
                        __builtin_amdgcn_sqrtf(fminf(F, K) * (1.0f / 16.0f) + K * (0.5f / F) + (float)parts);
    const float thresh = (kSigmaMargin * sigma - kTolAbs) * (1.0f / kTolRel);   // recompute |c| < thresh
    if (!(thresh > 0.0f))
        return first;
    // Per lane, bit 2 (4 i + e) + cb of a 64-bit mask (lo: i < 4, hi: i >= 4)
    // marks an output at risk: a compare and a shift per output.
    uint32_t risk[2] = {0u, 0u};
#pragma unroll
    for (int h = 0; h < (NRB > 4 ? 2 : 1); ++h)
#pragma unroll
        for (int i = (h + 1) * 4 - 1; i >= h * 4; --i)
#pragma unroll
            for (int e = 3; e >= 0; --e)
#pragma unroll
                for (int cb = 1; cb >= 0; --cb)
                    if (i < NRB)
                        risk[h] = 2u * risk[h] + (__builtin_fabsf(outer[i][cb][e]) < thresh ? 1u : 0u);
    // rows past the tile: (i, e) pairs of lane quarter q with 16 i + 4 q + e
    // >= rows are a suffix of the pair order; columns past the group drop cb
    {
        const int left = rows - 4 * q;                 // valid (i, e) pairs: a prefix of length pv
        const int pv = left <= 0 ? 0 : min(4 * (left >> 4) + min(left & 15, 4), 4 * NRB);
        const uint32_t cols = (col_base < G.n ? 0x55555555u : 0u) | (col_base + 16 < G.n ? 0xAAAAAAAAu : 0u);
        risk[0] &= (pv >= 16 ? ~0u : (1u << (2 * pv)) - 1u) & cols;
        risk[1] &= (pv >= 32 ? ~0u : (pv <= 16 ? 0u : (1u << (2 * (pv - 16))) - 1u)) & cols;
    }
    // list the outputs at risk, lane by lane (few lanes hold any); every 64
    // entries beyond the first 64 are recomputed here (rare)
    int lrow = 0, lcol = 0, n = 0;
    bool full = false;             // the first 64 entries are listed
    uint64_t lanes = __ballot((risk[0] | risk[1]) != 0u);
    while (lanes) {
        const int l = __builtin_ctzll(lanes);
        lanes &= lanes - 1;
        uint64_t bits = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)risk[0], l) |
                        (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)risk[1], l) << 32;
        while (bits) {
            const int bi = __builtin_ctzll(bits);
            bits &= bits - 1;
            const int pair = bi >> 1, cb = bi & 1;     // pair = 4 i + e
            const int orow = m0 + 16 * (pair >> 2) + 4 * (l >> 4) + (pair & 3);
            const int ocol = n0 + 32 * wave + 16 * cb + (l & 15);
            lrow = lane == n ? orow : lrow;
            lcol = lane == n ? ocol : lcol;
            if (++n == 64) {
                if (!full) {
                    first = FixList{lrow, lcol, 64};
                    full = true;
                } else {
                    store_exact_more(G.a, G.sfa, G.b, G.sfb, G.c, G.m, G.n, G.k, lrow, lcol, 64,
                                     (G.flags & NVFP4_SFB_SWIZZLED) != 0);
                }
                n = 0;
            }
        }
    }
    if (!full)
        first = FixList{lrow, lcol, n};
    else if (n > 0)
        store_exact_more(G.a, G.sfa, G.b, G.sfb, G.c, G.m, G.n, G.k, lrow, lcol, n, (G.flags & NVFP4_SFB_SWIZZLED) != 0);
    return first;
}

// One tile's share of this workgroup: pairs [pb, pe).  `w` is the logical
// workgroup index, [lo, hi) its cost range.
template <int NRB, int W>
__device__ __forceinline__ FixList run_tile(const LaunchArgs &args, const GroupArgs &G, uint32_t epoch,
                                            const TilePos &p, int pb, int pe, int w, int wave, uint8_t *smem)
{
    const int m0 = p.rt * G.tile_rows, n0 = p.strip * kTileN;
    const int rows = min(G.tile_rows, G.m - m0);
    f32x4 outer[NRB][2];
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
            outer[i][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // One call site of the pipelined loop: the own segment first, then (on
    // the finalizer) any producer part that did not arrive in time.
    int sb = pb, se = pe, w2 = w;
    int parts = 0;                 // partial sums added by this finalizer
    for (;;) {
        segment<NRB, W>(G, args.control + 2, args.sync_spin_limit, m0, n0, wave, smem, sb, se, outer);
        if (pb > 0) {              // a later part of a split tile
            publish_partial<NRB>(args, epoch, w, wave, outer);
            return FixList{0, 0, 0};
        }
        // finalizer: add the other parts of the tile in k order
        bool recompute = false;
        const int64_t tile_end = p.cost_begin + kCostHead + (int64_t)G.npairs * p.pcost;
        while (pe < G.npairs && ++w2 < args.num_wg) {
            const int64_t lo = args.cut[w2];
            const int64_t hi = args.cut[w2 + 1];
            if (lo >= tile_end)
                break;
            int qb, qe;
            pairs_in(p, G.npairs, lo, hi, qb, qe);
            if (qb >= qe)
                continue;
            if (await_partial(args, epoch, w2)) {
                add_partial<NRB>(args, w2, wave, outer);
                ++parts;
            } else {
                sb = qb;
                se = qe;
                recompute = true;
                break;
            }
        }
        if (!recompute)
            break;
        ++parts;                   // the recomputed part restarts its sums too
    }
    store_tile<NRB>(G, m0, rows, n0, wave, outer);
    return fix_small_outputs<NRB>(G, m0, rows, n0, wave, parts, outer);
}

template <int W>
__global__ __launch_bounds__(64 * W, 1) void nvfp4_group_gemm_kernel(const LaunchArgs args)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];

    const int nwg = args.num_wg;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Two rounds of argument loads before the first operand load: this
    // block's start record, then (all at once) its first group's fields, its
    // cost range and the epoch word.  Pinning the values in one asm keeps the
    // compiler from sinking those loads to their first uses, which would make
    // them dependent rounds of their own.
    const WgStart fs = args.first[blockIdx.x];
    const int w = fs.w;
    TilePos p = unpack_pos(fs.pos);
    GroupArgs G = args.g[p.g];
    int64_t lo = args.cut[w];
    int64_t hi = args.cut[w + 1];
    // this launch's epoch: one past the last finished launch's (0 marks an
    // unwritten flag); no workgroup changes it before all have started
    uint32_t last = __hip_atomic_load(&args.control[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" : "+s"(G.a), "+s"(G.b), "+s"(G.sfa), "+s"(G.sfb), "+s"(G.c), "+s"(G.m), "+s"(G.n), "+s"(G.k),
                 "+s"(G.tile_rows), "+s"(G.npairs), "+s"(G.row_tiles), "+s"(G.cost_full), "+s"(G.cost_last), "+s"(G.flags),
                 "+s"(G.strip_cost), "+s"(G.cost_begin), "+s"(lo), "+s"(hi), "+v"(last));
    last = (uint32_t)__builtin_amdgcn_readfirstlane((int)last);
    const uint32_t epoch = last + 1u == 0u ? 1u : last + 1u;

    int pb = p.pair, pe = fs.pe;
    while (pb < pe) {
        finish_pos(G, p);
        FixList fix;
        switch (p.nrb) {
        case 1: fix = run_tile<1, W>(args, G, epoch, p, pb, pe, w, wave, smem); break;
        case 2: fix = run_tile<2, W>(args, G, epoch, p, pb, pe, w, wave, smem); break;
        case 3: fix = run_tile<3, W>(args, G, epoch, p, pb, pe, w, wave, smem); break;
        case 4: fix = run_tile<4, W>(args, G, epoch, p, pb, pe, w, wave, smem); break;
        case 5: fix = run_tile<5, W>(args, G, epoch, p, pb, pe, w, wave, smem); break;
        case 6: fix = run_tile<6, W>(args, G, epoch, p, pb, pe, w, wave, smem); break;
        case 7: fix = run_tile<7, W>(args, G, epoch, p, pb, pe, w, wave, smem); break;
        default: fix = run_tile<8, W>(args, G, epoch, p, pb, pe, w, wave, smem); break;
        }
        // the tile's outputs at risk of exceeding the tolerance, recomputed
        // exactly over its stored values (one copy for every tile height)
        if (fix.n > 0)
            store_exact<false>(G.a, G.sfa, G.b, G.sfb, G.c, G.m, G.n, G.k, fix.lrow, fix.lcol, fix.n,
                               (G.flags & NVFP4_SFB_SWIZZLED) != 0);
        if (pe < G.npairs)
            break;                 // the range ends inside this tile
        p = next_tile(args.g, args.ng, args.total_cost, p);
        if (p.g >= args.ng)
            break;
        G = args.g[p.g];
        pairs_in(p, G.npairs, lo, hi, pb, pe);
    }
    // The last workgroup to finish resets the count and records the epoch
    // for the next launch on this workspace (ordered after this one by the
    // stream).
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t done = __hip_atomic_fetch_add(&args.control[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == (uint32_t)nwg - 1u) {
            __hip_atomic_store(&args.control[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&args.control[0], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------- direct path --
// Launches too small to fill the chip (config 0: two 256-k tiles) are bound
// by latency: the persistent kernel's fill, hand-offs and epilogue cost
// more than their MFMAs.  Here each wave owns one task of up to 16, 32 or
// 64 rows (the fewest that keep the task table within kDirectMaxTasks
// workgroups, so tiny launches spread over more waves) by 32 columns and
// runs it alone: its operand codes and scales are loaded
// straight into registers (every load of the whole K at once), decoded as
// in the persistent kernel, summed by the same MFMA chain with the same
// 512-k fold, stored by the same epilogue and checked by the same fix-up.
// Four waves share a workgroup (128 columns) but nothing else.
constexpr int kDirectWaves = 4;
constexpr int kDirectRowBlocks = 4;
constexpr int kDirectRows = 16 * kDirectRowBlocks;
constexpr int kDirectCols = 32 * kDirectWaves;
constexpr int kDirectMaxK = 4 * kStageK;       // four 128-k chunks in registers
constexpr int kDirectMaxTasks = 256;
constexpr int64_t kDirectMaxUnits = 64;        // (tile, pair) units of the persistent schedule

struct DirectTask {
    int32_t g, m0, n0, pad;
};

struct DirectArgs {
    GroupArgs g[kMaxGroupsPerLaunch];
    int32_t ntasks;
    int32_t task_rows;   // 16, 32 or 64
    int32_t ngroups;     // records in g (unused ones zeroed)
    int32_t pad_;
    DirectTask task[kDirectMaxTasks];
};

// One task: rows [m0, m0 + rows) (NRB blocks of 16) and columns [n0 + 32
// wave, + 32) of group G, in the persistent kernel's register layout
// (lane (r, q) holds outer[i][cb][e] = C[m0 + 16 i + 4 q + e][n0 + 32 wave
// + 16 cb + r]) and the same k order within each 128-k chunk (lane q takes
// k = 32 q + [0, 32), eight of them per MFMA step).
template <int NRB>
__device__ __forceinline__ FixList direct_task(const GroupArgs &G, int m0, int rows, int n0, int wave)
{
    const int lane = lane_id();
    const int r = lane & 15, q = lane >> 4;
    const int M = G.m, N = G.n, K = G.k;
    const uint32_t row_bytes = (uint32_t)K >> 1, row_sc = (uint32_t)K >> 4;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void *)G.a, 0, M * (int)row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc((void *)G.sfa, 0, M * (int)row_sc, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void *)G.b, 0, N * (int)row_bytes, 0x00020000);
    const bool sfb_swz = (G.flags & NVFP4_SFB_SWIZZLED) != 0;
    const uint32_t swz_w = swz_windows(K);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
        (void *)G.sfb, 0, sfb_swz ? (int)swz_bytes(N, K) : N * (int)row_sc, 0x00020000);
    uint32_t a_off[NRB], sa_off[NRB], b_off[2], sb_col[2];
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
        const uint32_t row = (uint32_t)min(m0 + 16 * i + r, M - 1);
        a_off[i] = row * row_bytes + 16u * q;
        sa_off[i] = row * row_sc + 2u * q;
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const uint32_t col = (uint32_t)min(n0 + 32 * wave + 16 * cb + r, N - 1);
        b_off[cb] = col * row_bytes + 16u * q;
        sb_col[cb] = col;
    }
    // scale bytes (column col, blocks b and b + 1) in either layout
    auto sb_at = [&](uint32_t col, uint32_t b) -> uint32_t {
        return sfb_swz ? swz_offset(col, b, swz_w) : col * row_sc + b;
    };
    const int nch = (K + kStageK - 1) / kStageK;    // <= 4
    // every chunk's loads first; chunks past K are not loaded
    u32x4 ac[4][NRB], bc[4][2];
    uint32_t sa[4][NRB], sb[4][2];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (c < nch) {
            const uint32_t kb = (uint32_t)c * (kStageK / 2), ks = (uint32_t)c * (kStageK / 16);
#pragma unroll
            for (int i = 0; i < NRB; ++i) {
                ac[c][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, a_off[i] + kb, 0, 0));
                sa[c][i] = __builtin_amdgcn_raw_buffer_load_b16(rsa, sa_off[i] + ks, 0, 0);
            }
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                bc[c][cb] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, b_off[cb] + kb, 0, 0));
                sb[c][cb] = __builtin_amdgcn_raw_buffer_load_b16(rsb, sb_at(sb_col[cb], ks + 2u * q), 0, 0);
            }
        }
    }
    f32x4 outer[NRB][2];
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
            outer[i][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // K <= 512: one MFMA chain over all chunks, folded once (the persistent
    // kernel folds every 512 k, so the sums round the same way)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (c < nch) {
            // lanes whose 32 k lie past K get zero scales (K % 64 == 0)
            const bool valid = c * kStageK + 32 * q < K;
            f16x2 sca[NRB], scb[2];
#pragma unroll
            for (int i = 0; i < NRB; ++i)
                sca[i] = scales2(valid ? sa[c][i] : 0u);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                scb[cb] = scales2(valid ? sb[c][cb] : 0u);
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                f16x8 bf[2];
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    bf[cb] = decode8(bc[c][cb][s2], bcast(scb[cb][s2 >> 1]));
#pragma unroll
                for (int i = 0; i < NRB; ++i) {
                    const f16x8 af = decode8(ac[c][i][s2], bcast(sca[i][s2 >> 1]));
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb)
                        outer[i][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[cb], outer[i][cb], 0, 0, 0);
                }
            }
        }
    }
    store_tile<NRB>(G, m0, rows, n0, wave, outer);
    return fix_small_outputs<NRB>(G, m0, rows, n0, wave, 0, outer);
}

__global__ __launch_bounds__(64 * kDirectWaves) void nvfp4_direct_kernel(const DirectArgs args)
{
    // One round of argument loads for launches of at most two groups: the
    // task and both groups' fields at once (pinned, so the compiler cannot
    // sink them to their uses), then a select; a second round, for the
    // task's group, only with more groups.
    DirectTask t = args.task[blockIdx.x];
    int task_rows = args.task_rows, ng = args.ngroups;
    GroupArgs G0 = args.g[0], G1 = args.g[1];
    asm volatile("" : "+s"(t.g), "+s"(t.m0), "+s"(t.n0), "+s"(task_rows), "+s"(ng));
    asm volatile("" : "+s"(G0.a), "+s"(G0.b), "+s"(G0.sfa), "+s"(G0.sfb), "+s"(G0.c), "+s"(G0.m), "+s"(G0.n),
                 "+s"(G0.k), "+s"(G0.flags));
    asm volatile("" : "+s"(G1.a), "+s"(G1.b), "+s"(G1.sfa), "+s"(G1.sfb), "+s"(G1.c), "+s"(G1.m), "+s"(G1.n),
                 "+s"(G1.k), "+s"(G1.flags));
    GroupArgs G = t.g == 0 ? G0 : G1;
    if (ng > 2) {
        G = args.g[t.g];
        asm volatile("" : "+s"(G.a), "+s"(G.b), "+s"(G.sfa), "+s"(G.sfb), "+s"(G.c), "+s"(G.m), "+s"(G.n), "+s"(G.k),
                     "+s"(G.flags));
    }
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t.n0 + 32 * wave >= G.n)
        return;                    // this wave's columns lie past the group (no barrier follows)
    const int rows = min(task_rows, G.m - t.m0);
    FixList fix;
    switch ((rows + 15) >> 4) {
    case 1: fix = direct_task<1>(G, t.m0, rows, t.n0, wave); break;
    case 2: fix = direct_task<2>(G, t.m0, rows, t.n0, wave); break;
    case 3: fix = direct_task<3>(G, t.m0, rows, t.n0, wave); break;
    default: fix = direct_task<4>(G, t.m0, rows, t.n0, wave); break;
    }
    if (fix.n > 0)
        store_exact<false>(G.a, G.sfa, G.b, G.sfb, G.c, G.m, G.n, G.k, fix.lrow, fix.lcol, fix.n,
                           (G.flags & NVFP4_SFB_SWIZZLED) != 0);
}

// Window-major copy of a scale matrix (see swz_offset): thread t writes the
// 16 bytes of one (row, window) entry of the output.
__global__ __launch_bounds__(256) void nvfp4_swizzle_kernel(const uint8_t *sf, uint8_t *out, int rows, int k,
                                                              uint32_t entries)
{
    const uint32_t e = blockIdx.x * 256u + threadIdx.x;
    if (e >= entries)
        return;
    const uint32_t windows = swz_windows(k);
    const uint32_t row = ((e >> 5) / windows) * 32u + (e & 31u);     // entry order = output order
    const uint32_t w = (e >> 5) % windows;
    const uint32_t src_row = row < (uint32_t)rows ? row : (uint32_t)rows - 1u;
    const uint32_t nb = (uint32_t)k >> 4;
    uint8_t v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const uint32_t b = 16u * w + (uint32_t)j;
        v[j] = b < nb ? sf[(size_t)src_row * nb + b] : (uint8_t)0;
    }
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = (uint32_t)v[4 * j] | (uint32_t)v[4 * j + 1] << 8 | (uint32_t)v[4 * j + 2] << 16 |
               (uint32_t)v[4 * j + 3] << 24;
    *reinterpret_cast<u32x4 *>(out + (size_t)e * 16u) = o;
}

// ------------------------------------------------------------------ host --

thread_local char g_err[512];

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int validate(const nvfp4_group_t *groups, int ng)
{
    g_err[0] = '\0';
    if (ng < 0)
        return fail(NVFP4_EINVAL, "ng = %d is negative", ng);
    if (ng > 0 && groups == nullptr)
        return fail(NVFP4_EINVAL, "groups is NULL with ng = %d", ng);
    for (int i = 0; i < ng; ++i) {
        const nvfp4_group_t &G = groups[i];
        if (G.m < 0 || G.n < 0 || G.k < 0)
            return fail(NVFP4_EINVAL, "group %d: negative size (m=%d n=%d k=%d)", i, G.m, G.n, G.k);
        if (G.k % 16 != 0)
            return fail(NVFP4_EINVAL, "group %d: k=%d is not a multiple of 16", i, G.k);
        if ((G.flags & ~NVFP4_SFB_SWIZZLED) != 0)
            return fail(NVFP4_EINVAL, "group %d: unknown flags 0x%x", i, (unsigned)G.flags);
        if (G.m == 0 || G.n == 0)
            continue;
        if (G.c == nullptr)
            return fail(NVFP4_EINVAL, "group %d: c is NULL", i);
        if (G.k > 0 && (G.a == nullptr || G.b == nullptr || G.sfa == nullptr || G.sfb == nullptr))
            return fail(NVFP4_EINVAL, "group %d: NULL operand pointer", i);
    }
    for (int i = 0; i < ng; ++i) {
        const nvfp4_group_t &G = groups[i];
        if (G.m == 0 || G.n == 0)
            continue;
        if (G.k % 64 != 0)
            return fail(NVFP4_EUNSUPPORTED, "group %d: k=%d is not a multiple of 64", i, G.k);
        if ((uint64_t)(G.m > G.n ? G.m : G.n) * (uint64_t)(G.k / 2) >= (1ull << 31))
            return fail(NVFP4_EUNSUPPORTED, "group %d: an operand reaches 2 GiB", i);
        if (((uintptr_t)G.c & 3u) != 0)
            return fail(NVFP4_EUNSUPPORTED, "group %d: c is not 4-byte aligned", i);
        if (G.k > 0 && ((((uintptr_t)G.a | (uintptr_t)G.b) & 15u) != 0 ||
                        (((uintptr_t)G.sfa | (uintptr_t)G.sfb) & 3u) != 0))
            return fail(NVFP4_EUNSUPPORTED, "group %d: operand pointer misaligned", i);
        if ((G.flags & NVFP4_SFB_SWIZZLED) != 0) {
            if (G.k > 0 && ((uintptr_t)G.sfb & 15u) != 0)
                return fail(NVFP4_EUNSUPPORTED, "group %d: window-major sfb is not 16-byte aligned", i);
            if (swz_bytes(G.n, G.k) >= (1ull << 31))
                return fail(NVFP4_EUNSUPPORTED, "group %d: window-major sfb reaches 2 GiB", i);
        }
    }
    return NVFP4_OK;
}

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Row tiling of a group: the fewest tiles of at most kTileM rows, with the
// rows spread evenly (rounded up to 16) so a ragged M wastes little.
inline void row_tiling(int m, int &tiles, int &rows_per_tile)
{
    tiles = ceil_div(m, kTileM);
    rows_per_tile = 16 * ceil_div(ceil_div(m, tiles), 16);
    tiles = ceil_div(m, rows_per_tile);
}

// Fills the schedule fields of the launch's groups (non-empty groups of
// `groups` from index *next, at most kMaxGroupsPerLaunch); returns the
// number packed.
int pack_launch(const nvfp4_group_t *groups, int ng, int &next, LaunchArgs &args)
{
    memset(&args, 0, sizeof args);
    int n = 0;
    int64_t cost = 0;
    for (; next < ng && n < kMaxGroupsPerLaunch; ++next) {
        const nvfp4_group_t &G = groups[next];
        if (G.m == 0 || G.n == 0)
            continue;
        GroupArgs &A = args.g[n++];
        A.a = static_cast<const uint8_t *>(G.a);
        A.b = static_cast<const uint8_t *>(G.b);
        A.sfa = static_cast<const uint8_t *>(G.sfa);
        A.sfb = static_cast<const uint8_t *>(G.sfb);
        A.flags = G.flags;
        A.c = static_cast<_Float16 *>(G.c);
        A.m = G.m;
        A.n = G.n;
        A.k = G.k;
        row_tiling(G.m, A.row_tiles, A.tile_rows);
        A.col_tiles = ceil_div(G.n, kTileN);
        A.npairs = ceil_div(ceil_div(G.k, kStageK), 2);
        if (A.npairs < 1)
            A.npairs = 1;      // k == 0: one empty pair, the tile is still written
        A.cost_full = pair_cost(A.tile_rows / 16, A.npairs);
        A.cost_last = pair_cost(tile_nrb(A, A.row_tiles - 1), A.npairs);
        A.strip_cost = (int64_t)A.row_tiles * kCostHead +
                       (int64_t)A.npairs * ((int64_t)(A.row_tiles - 1) * A.cost_full + A.cost_last);
        A.cost_begin = cost;
        args.group_begin[n - 1] = cost;
        cost += A.strip_cost * A.col_tiles;
    }
    for (int i = n; i < kMaxGroupsPerLaunch; ++i)
        args.group_begin[i] = INT64_MAX;
    args.ng = n;
    args.total_cost = cost;
    return n;
}

int64_t total_pairs(const LaunchArgs &args)
{
    int64_t t = 0;
    for (int i = 0; i < args.ng; ++i)
        t += (int64_t)args.g[i].row_tiles * args.g[i].col_tiles * args.g[i].npairs;
    return t;
}

int grid_for(const LaunchArgs &args, int units)
{
    const int64_t tp = total_pairs(args);
    int64_t g = tp < units ? tp : units;
    if (g > kMaxWorkgroups)
        g = kMaxWorkgroups;
    return (int)g;
}

// Partition of a launch's (tile, pair) sequence among num_wg workgroups.
// A greedy fill against a target makespan, binary-searched: each workgroup
// takes pairs in order while its modelled time stays within the target.
// The model (clocks, fitted to per-workgroup timestamps of this kernel on
// MI355X) charges a workgroup its start-up, a pipeline fill per segment (the
// first one dearer), the pairs (measured per tile height: a pair of a short
// tile is bound by streaming B, not by its MFMAs), and each segment's
// epilogue:
//  * a whole tile: its store;
//  * the later part of a split tile (its workgroup's first segment): the
//    publish of its partial sums;
//  * the first part (the finalizer's): the store plus one sum per other
//    part (one other part if the next workgroup can take the rest of the
//    tile, else two);
//  * a middle part (a workgroup whose whole range lies inside the tile): its
//    publish must leave the finalizer time for two sums and the store;
//  * the last part of a split tile: its publish must leave the finalizer
//    time for one sum and the store (the finalizer ends after the last part
//    arrives, so a last part that ends at the makespan would set the
//    makespan one sum and a store later).
// Start-up, fills, store and publish are a least-squares fit of per-
// workgroup timestamps (segment entry, loop start and end, kernel entry and
// exit) over seven workloads; start-up and the first fill include the
// workgroup's end-of-kernel work.  The pair costs, measured per tile height
// on the balanced schedule, sit 6-14% above the bare loop's cost: they also
// carry what a segment of short tiles pays beyond its loop, and a table
// fitted to the loop alone balanced the ragged workloads worse.  The cost of
// a finalizer's sum of one part (6000) is the value interleaved timing
// preferred over 4000 and 8000: finalizers end 15-19k clk after their
// tile's last part, more than one sum and a store at the fitted costs.
constexpr double kClkStart = 3500;
constexpr double kClkFillFirst = 5850;
constexpr double kClkFillNext = 9400;
constexpr double kClkPair[kRowBlocks + 1] = {0, 4212, 4634, 4648, 4880, 5305, 5622, 6141, 6988};
constexpr double kClkPublish = 7900;
constexpr double kClkStore = 7200;
constexpr double kClkAdd = 6000;

// One tile of the launch for the partition: where it starts in cost order,
// its pair cost there, and its pairs' modelled clocks.
struct PlanTile {
    int64_t cost_begin;
    int32_t pcost, npairs;
    double pair_clk;
};

bool greedy_cuts(const std::vector<PlanTile> &tiles, int nwg, int64_t total, double tmax, int64_t *cut)
{
    int w = 0;
    double cur = kClkStart;
    bool fresh = true;             // workgroup w has no segment yet
    cut[0] = 0;
    for (const PlanTile &t : tiles) {
        const int npairs = t.npairs;
        const double pc = t.pair_clk;
        int j = 0;
        while (j < npairs) {
            const double base = cur + (fresh ? kClkFillFirst : kClkFillNext);
            const int rest = npairs - j;
            const double epi_full = j == 0 ? kClkStore : kClkPublish;
            // a last part of a split tile leaves the finalizer its sum and store
            const double tail = j == 0 ? 0.0 : kClkAdd + kClkStore;
            if (base + rest * pc + epi_full + tail <= tmax) {   // the rest of the tile fits
                cur = base + rest * pc + epi_full;
                fresh = false;
                break;
            }
            // pairs this workgroup can take before its range ends in the tile
            auto take = [&](double epi) {
                const double fit = (tmax - base - epi) / pc;
                return fit < 0 ? 0 : (fit > rest - 1 ? rest - 1 : (int)fit);
            };
            auto next_takes_rest = [&](int r) {
                return kClkStart + kClkFillFirst + r * pc + kClkPublish + kClkAdd + kClkStore <= tmax;
            };
            int k;
            if (j == 0) {
                k = take(kClkStore + kClkAdd);
                if (!(k >= 1 && next_takes_rest(rest - k)))
                    k = take(kClkStore + 2 * kClkAdd);
            } else {
                k = take(kClkPublish + kClkStore + 2 * kClkAdd);
            }
            j += k;
            // workgroup w ends with pair j - 1 of this tile (or before the tile)
            if (++w >= nwg)
                return false;
            cut[w] = j == 0 ? t.cost_begin : t.cost_begin + kCostHead + (int64_t)j * t.pcost;
            cur = kClkStart;
            fresh = true;
        }
    }
    for (int i = w + 1; i <= nwg; ++i)
        cut[i] = total;
    return true;
}

// The last partition computed on this host thread, reused while the
// launch's shapes and workgroup count stay the same.
struct CutCache {
    int nwg = -1, ng = 0;
    int32_t mnk[kMaxGroupsPerLaunch][3];
    int64_t cut[kMaxWorkgroups + 1];
    WgStart first[kMaxWorkgroups];
};
thread_local CutCache g_cut_cache;

// Logical workgroup of block b (see WgStart).
inline int logical_wg(int b, int nwg)
{
    return nwg % 8 == 0 ? (b % 8) * (nwg / 8) + b / 8 : b;
}

// The start records of a launch whose cuts are set.
void fill_starts(LaunchArgs &a, int nwg)
{
    for (int b = 0; b < nwg; ++b) {
        const int w = logical_wg(b, nwg);
        TilePos p = locate(a, a.cut[w]);
        WgStart &f = a.first[b];
        f.w = w;
        f.pe = 0;
        f.pos = 0;                 // no tile: group 0, no pairs
        if (p.g < a.ng) {
            int pb, pe;
            pairs_in(p, a.g[p.g].npairs, a.cut[w], a.cut[w + 1], pb, pe);
            if (pb < pe) {
                p.pair = pb;
                f.pos = pack_start(p, a.ng);
                f.pe = pe;
            }
        }
    }
}

void plan_cuts(LaunchArgs &a, int nwg)
{
    CutCache &cc = g_cut_cache;
    bool same = cc.nwg == nwg && cc.ng == a.ng;
    for (int i = 0; same && i < a.ng; ++i)
        same = cc.mnk[i][0] == a.g[i].m && cc.mnk[i][1] == a.g[i].n && cc.mnk[i][2] == a.g[i].k;
    if (same) {
        memcpy(a.cut, cc.cut, sizeof(int64_t) * (nwg + 1));
        memcpy(a.first, cc.first, sizeof(WgStart) * nwg);
        return;
    }
    std::vector<PlanTile> tiles;
    double work = 0, biggest = 0;
    for (TilePos p = locate(a, 0); p.g < a.ng; p = next_tile(a.g, a.ng, a.total_cost, p)) {
        const PlanTile t{p.cost_begin, p.pcost, a.g[p.g].npairs, kClkPair[p.nrb]};
        const double tile = kClkFillFirst + kClkStore + 2 * kClkAdd + t.npairs * t.pair_clk;
        work += t.npairs * t.pair_clk;
        biggest = tile > biggest ? tile : biggest;
        tiles.push_back(t);
    }
    // the makespan lies between the average work and that plus a whole tile
    double lo = kClkStart + work / nwg;
    double hi = lo + biggest + kClkFillFirst + kClkStore + 2 * kClkAdd;
    while (!greedy_cuts(tiles, nwg, a.total_cost, hi, a.cut))
        hi *= 2;
    for (int it = 0; it < 24 && hi - lo > 64.0; ++it) {
        const double mid = 0.5 * (lo + hi);
        if (greedy_cuts(tiles, nwg, a.total_cost, mid, a.cut))
            hi = mid;
        else
            lo = mid;
    }
    greedy_cuts(tiles, nwg, a.total_cost, hi, a.cut);
    fill_starts(a, nwg);
    cc.nwg = nwg;
    cc.ng = a.ng;
    for (int i = 0; i < a.ng; ++i) {
        cc.mnk[i][0] = a.g[i].m;
        cc.mnk[i][1] = a.g[i].n;
        cc.mnk[i][2] = a.g[i].k;
    }
    memcpy(cc.cut, a.cut, sizeof(int64_t) * (nwg + 1));
    memcpy(cc.first, a.first, sizeof(WgStart) * nwg);
}

// Library-owned workspace for one stream: partial-sum slots, their flags,
// and kControlWords control words after the flags (see LaunchArgs::control).
struct Workspace {
    float *partials = nullptr;
    uint32_t *flags = nullptr;
    int slots = 0;
};

std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

// The workspace of (device, stream), created on first use.  Creation
// allocates and zeroes device memory, which a stream under graph capture
// must not record, so a capturing stream without a workspace is refused.
int workspace_for(hipStream_t st, int device, int slots, Workspace *&out)
{
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    auto it = g_ws.find({device, st});
    if (it != g_ws.end() && it->second.slots >= slots) {
        out = &it->second;
        return NVFP4_OK;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(st, &cs);
    if (e != hipSuccess)
        return fail(NVFP4_EHIP, "cannot query the stream's capture status: %s", hipGetErrorString(e));
    if (cs != hipStreamCaptureStatusNone)
        return fail(NVFP4_EUNSUPPORTED,
                    "the stream is capturing and has no workspace yet: call once outside capture first");
    Workspace &ws = g_ws[{device, st}];
    if (ws.partials) {
        // the previous buffers may still be read by work queued on `st`
        e = hipStreamSynchronize(st);
        if (e != hipSuccess)
            return fail(NVFP4_EHIP, "stream synchronize failed: %s", hipGetErrorString(e));
        (void)hipFree(ws.partials);
        (void)hipFree(ws.flags);
        ws.partials = nullptr;
        ws.flags = nullptr;
        ws.slots = 0;
    }
    e = hipMalloc(reinterpret_cast<void **>(&ws.partials), (size_t)slots * kPartialSlot);
    if (e == hipSuccess)
        e = hipMalloc(reinterpret_cast<void **>(&ws.flags), ((size_t)slots + kControlWords) * sizeof(uint32_t));
    if (e == hipSuccess)
        e = hipMemsetAsync(ws.flags, 0, ((size_t)slots + kControlWords) * sizeof(uint32_t), st);
    if (e != hipSuccess) {
        if (ws.partials)
            (void)hipFree(ws.partials);
        if (ws.flags)
            (void)hipFree(ws.flags);
        g_ws.erase({device, st});
        return fail(NVFP4_EHIP, "workspace allocation failed: %s", hipGetErrorString(e));
    }
    ws.slots = slots;
    out = &ws;
    return NVFP4_OK;
}

// Flag polls before a finalizer recomputes a missing part itself.  The
// environment variable NVFP4_SPIN_LIMIT overrides the default (0 makes every
// split tile take the recomputation path: a test of that path).
int spin_limit()
{
    const char *e = getenv("NVFP4_SPIN_LIMIT");
    return e != nullptr ? atoi(e) : (1 << 20);
}

// Polls of an A hand-off wait (NVFP4_SYNC_SPIN_LIMIT overrides the default;
// a tiny value forces the waits to run out: a test of their error word).
int sync_spin_limit()
{
    const char *e = getenv("NVFP4_SYNC_SPIN_LIMIT");
    const int v = e != nullptr ? atoi(e) : kSyncSpinLimit;
    return v < 0 ? 0 : v;
}

int device_units(int &device, int &units)
{
    static std::mutex m;
    static std::map<int, int> cache;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess)
        return fail(NVFP4_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(m);
    auto it = cache.find(device);
    if (it == cache.end()) {
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
        if (e != hipSuccess || cus <= 0)
            return fail(NVFP4_EHIP, "cannot query the compute-unit count");
        it = cache.emplace(device, cus).first;
    }
    units = it->second;
    return NVFP4_OK;
}

// Allocation-free variant: the same workspace layout (partial-sum slots,
// their flags, two control words) in a file-scope device array instead of a
// per-stream allocation.  Each GPU the library runs on holds its own copy
// until the process ends; it starts zeroed (the loader clears it), which is
// the state the epoch logic needs, so nothing is cleared per call.  Host code
// reaches it only through the address hipGetSymbolAddress returns for the
// current device (the array's name in host code is a stand-in, not a device
// address).
constexpr int kStaticSlots = kMaxWorkgroups;
constexpr size_t kStaticPartialBytes = (size_t)kStaticSlots * kPartialSlot;
constexpr size_t kStaticBytes = kStaticPartialBytes + ((size_t)kStaticSlots + kControlWords) * sizeof(uint32_t);
static __device__ __align__(256) uint8_t scratch[kStaticBytes];

// Device address of `scratch` on the current device, looked up once per
// device and kept.
int static_scratch(int device, uint8_t *&out)
{
    static std::mutex m;
    static std::map<int, uint8_t *> addr;
    std::lock_guard<std::mutex> lock(m);
    auto it = addr.find(device);
    if (it == addr.end()) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return fail(NVFP4_EHIP, "cannot find the static workspace on device %d: %s", device,
                        hipGetErrorString(e));
        it = addr.emplace(device, static_cast<uint8_t *>(ptr)).first;
    }
    out = it->second;
    return NVFP4_OK;
}

// Every launch of one call: the stream's allocated workspace, or (use_static)
// the device's static one.
// Path of a launch: NVFP4_PATH=main or =direct forces one (direct only
// where its argument table fits); by default the direct path takes
// launches whose every K is at most kDirectMaxK and whose persistent
// schedule would have at most kDirectMaxUnits (tile, pair) units.
int path_override()
{
    const char *e = getenv("NVFP4_PATH");
    if (e == nullptr)
        return 0;
    if (strcmp(e, "main") == 0)
        return 1;
    if (strcmp(e, "direct") == 0)
        return 2;
    return 0;
}

// The direct path's task table for a packed launch; false if it does not
// fit (some K above kDirectMaxK, or more than kDirectMaxTasks tasks).
bool direct_tasks(const LaunchArgs &args, DirectArgs &d)
{
    for (int gi = 0; gi < args.ng; ++gi)
        if (args.g[gi].k > kDirectMaxK)
            return false;
    for (int rows = 16; rows <= kDirectRows; rows *= 2) {
        int64_t count = 0;
        for (int gi = 0; gi < args.ng; ++gi)
            count += (int64_t)ceil_div(args.g[gi].m, rows) * ceil_div(args.g[gi].n, kDirectCols);
        if (count > kDirectMaxTasks)
            continue;
        int n = 0;
        for (int gi = 0; gi < args.ng; ++gi)
            for (int m0 = 0; m0 < args.g[gi].m; m0 += rows)
                for (int n0 = 0; n0 < args.g[gi].n; n0 += kDirectCols)
                    d.task[n++] = DirectTask{gi, m0, n0, 0};
        memcpy(d.g, args.g, sizeof d.g);
        d.ntasks = n;
        d.task_rows = rows;
        d.ngroups = args.ng;
        return true;
    }
    return false;
}

int launch_all(const nvfp4_group_t *groups, int ng, hipStream_t st, bool use_static)
{
    const int path = path_override();
    int device = 0, units = 0;
    LaunchArgs args;
    int next = 0;
    bool queried = false;
    while (next < ng) {
        if (pack_launch(groups, ng, next, args) == 0)
            break;
        if (path != 1 && (path == 2 || total_pairs(args) <= kDirectMaxUnits)) {
            DirectArgs d;
            if (direct_tasks(args, d)) {
                hipLaunchKernelGGL(nvfp4_direct_kernel, dim3((unsigned)d.ntasks), dim3(64 * kDirectWaves), 0, st, d);
                const hipError_t e = hipGetLastError();
                if (e != hipSuccess)
                    return fail(NVFP4_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
                continue;
            }
        }
        if (!queried) {
            const int rc2 = device_units(device, units);
            if (rc2 != NVFP4_OK)
                return rc2;
            queried = true;
        }
        const int nwg = grid_for(args, units);
        if (use_static) {
            if (nwg > kStaticSlots)
                return fail(NVFP4_EUNSUPPORTED, "%d workgroups exceed the static workspace's %d slots", nwg,
                            kStaticSlots);
            uint8_t *base = nullptr;
            const int rc3 = static_scratch(device, base);
            if (rc3 != NVFP4_OK)
                return rc3;
            args.partials = reinterpret_cast<float *>(base);
            args.flags = reinterpret_cast<uint32_t *>(base + kStaticPartialBytes);
            args.control = args.flags + kStaticSlots;
        } else {
            Workspace *ws = nullptr;
            const int rc3 = workspace_for(st, device, units < kMaxWorkgroups ? units : kMaxWorkgroups, ws);
            if (rc3 != NVFP4_OK)
                return rc3;
            args.partials = ws->partials;
            args.flags = ws->flags;
            args.control = ws->flags + ws->slots;
        }
        args.num_wg = nwg;
        plan_cuts(args, nwg);
        args.spin_limit = spin_limit();
        args.sync_spin_limit = sync_spin_limit();
        hipLaunchKernelGGL((nvfp4_group_gemm_kernel<kWaves>), dim3((unsigned)nwg), dim3(kThreads), 0, st, args);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return fail(NVFP4_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return NVFP4_OK;
}

}  // namespace

extern "C" int64_t nvfp4_swizzled_scale_bytes(int rows, int k)
{
    if (rows <= 0 || k <= 0)
        return 0;
    return (int64_t)swz_bytes(rows, k);
}

extern "C" int nvfp4_swizzle_scales(const void *sf, void *out, int rows, int k, void *stream)
{
    g_err[0] = '\0';
    if (rows < 0 || k < 0 || k % 16 != 0)
        return fail(NVFP4_EINVAL, "rows = %d, k = %d: negative, or k not a multiple of 16", rows, k);
    if (rows == 0 || k == 0)
        return NVFP4_OK;
    if (sf == nullptr || out == nullptr)
        return fail(NVFP4_EINVAL, "NULL scale pointer");
    if (((uintptr_t)out & 15u) != 0)
        return fail(NVFP4_EUNSUPPORTED, "out is not 16-byte aligned");
    const uint64_t bytes = swz_bytes(rows, k);
    if (bytes >= (1ull << 31))
        return fail(NVFP4_EUNSUPPORTED, "the layout reaches 2 GiB");
    const uint32_t entries = (uint32_t)(bytes / 16u);
    hipLaunchKernelGGL(nvfp4_swizzle_kernel, dim3((entries + 255u) / 256u), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), static_cast<const uint8_t *>(sf),
                       static_cast<uint8_t *>(out), rows, k, entries);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(NVFP4_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return NVFP4_OK;
}

extern "C" int nvfp4_validate(const nvfp4_group_t *groups, int ng)
{
    return validate(groups, ng);
}

extern "C" int nvfp4_tile_rows(void) { return kTileM; }
extern "C" int nvfp4_tile_cols(void) { return kTileN; }

extern "C" int nvfp4_plan(const nvfp4_group_t *groups, int ng, int num_workgroups, int32_t *segs, int cap)
{
    const int rc = validate(groups, ng);
    if (rc != NVFP4_OK)
        return -rc;
    if (num_workgroups <= 0)
        return -fail(NVFP4_EINVAL, "num_workgroups must be positive");
    LaunchArgs args;
    int next = 0, launch_first = 0;
    long long count = 0;
    while (next < ng) {
        // group indices of this launch (pack_launch skips empty groups)
        int map[kMaxGroupsPerLaunch];
        int n = 0;
        for (int i = launch_first; i < ng && n < kMaxGroupsPerLaunch; ++i)
            if (groups[i].m != 0 && groups[i].n != 0)
                map[n++] = i;
        if (pack_launch(groups, ng, next, args) == 0)
            break;
        launch_first = next;
        const int nwg = grid_for(args, num_workgroups);
        plan_cuts(args, nwg);
        // the kernel's walk (its start records, then pairs_in per tile),
        // listed in logical workgroup order
        int block_of[kMaxWorkgroups];
        for (int b = 0; b < nwg; ++b)
            block_of[args.first[b].w] = b;
        for (int w = 0; w < nwg; ++w) {
            const WgStart &fs = args.first[block_of[w]];
            const int64_t lo = args.cut[w];
            const int64_t hi = args.cut[w + 1];
            TilePos p = unpack_pos(fs.pos);
            int pb = p.pair, pe = fs.pe;
            while (pb < pe) {
                const GroupArgs &G = args.g[p.g];
                finish_pos(G, p);
                if (segs != nullptr && count < cap) {
                    int32_t *o = segs + 8 * count;
                    const int m0 = p.rt * G.tile_rows;
                    o[0] = w;
                    o[1] = map[p.g];
                    o[2] = m0;
                    o[3] = G.m - m0 < G.tile_rows ? G.m - m0 : G.tile_rows;
                    o[4] = p.strip * kTileN;
                    o[5] = 2 * kStageK * pb;
                    o[6] = 2 * kStageK * pe;
                    o[7] = (pb == 0 && pe == G.npairs) ? 0 : (pb > 0 ? 1 : 2);
                }
                ++count;
                if (pe < G.npairs)
                    break;
                p = next_tile(args.g, args.ng, args.total_cost, p);
                if (p.g >= args.ng)
                    break;
                pairs_in(p, args.g[p.g].npairs, lo, hi, pb, pe);
            }
        }
    }
    if (count > 0x7fffffffLL)
        return -fail(NVFP4_EUNSUPPORTED, "too many segments");
    return (int)count;
}

extern "C" int nvfp4_group_gemm(const nvfp4_group_t *groups, int ng, void *stream)
{
    const int rc = validate(groups, ng);
    if (rc != NVFP4_OK)
        return rc;
    return launch_all(groups, ng, reinterpret_cast<hipStream_t>(stream), false);
}

extern "C" int nvfp4_group_gemm_noalloc(const nvfp4_group_t *groups, int ng, void *stream)
{
    const int rc = validate(groups, ng);
    if (rc != NVFP4_OK)
        return rc;
    return launch_all(groups, ng, reinterpret_cast<hipStream_t>(stream), true);
}

extern "C" int nvfp4_release_workspace(void *stream)
{
    g_err[0] = '\0';
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess)
        return fail(NVFP4_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    auto it = g_ws.find({device, st});
    if (it == g_ws.end())
        return NVFP4_OK;
    e = hipStreamSynchronize(st);
    if (e != hipSuccess)
        return fail(NVFP4_EHIP, "stream synchronize failed: %s", hipGetErrorString(e));
    (void)hipFree(it->second.partials);
    (void)hipFree(it->second.flags);
    g_ws.erase(it);
    return NVFP4_OK;
}

extern "C" int nvfp4_stream_errors(void *stream)
{
    g_err[0] = '\0';
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess)
        return -fail(NVFP4_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    e = hipStreamSynchronize(st);
    if (e != hipSuccess)
        return -fail(NVFP4_EHIP, "stream synchronize failed: %s", hipGetErrorString(e));
    uint32_t *words[2] = {nullptr, nullptr};
    {
        std::lock_guard<std::mutex> lock(g_ws_mutex);
        auto it = g_ws.find({device, st});
        if (it != g_ws.end())
            words[0] = it->second.flags + it->second.slots + 2;
    }
    uint8_t *base = nullptr;
    if (static_scratch(device, base) == NVFP4_OK)
        words[1] = reinterpret_cast<uint32_t *>(base + kStaticPartialBytes) + kStaticSlots + 2;
    long long total = 0;
    for (uint32_t *w : words) {
        if (w == nullptr)
            continue;
        uint32_t v = 0;
        e = hipMemcpy(&v, w, sizeof v, hipMemcpyDeviceToHost);
        if (e == hipSuccess && v != 0) {
            const uint32_t zero = 0;
            e = hipMemcpy(w, &zero, sizeof zero, hipMemcpyHostToDevice);
        }
        if (e != hipSuccess)
            return -fail(NVFP4_EHIP, "reading the error word failed: %s", hipGetErrorString(e));
        total += v;
    }
    return total > 0x7fffffff ? 0x7fffffff : (int)total;
}

extern "C" const char *nvfp4_last_error(void) { return g_err; }
