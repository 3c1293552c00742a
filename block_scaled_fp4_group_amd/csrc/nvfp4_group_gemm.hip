// nvfp4_group_gemm.hip -- gfx950 (MI355X) kernel and C ABI of the NVFP4
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
//    while NVFP4 carries E4M3 scales per 16 k, and a decoded product a*s
//    needs up to 6 significant bits (more than FP8 holds).  Every E2M1 x
//    E4M3FN product lies in [2^-10, 2688] with at most 6 significant bits, so
//    it is exact in fp16: operands are decoded exactly to fp16 (hardware
//    FP4->f16 convert, then one packed f16 multiply by the scale) and fed to
//    v_mfma_f32_32x32x16_f16 with fp32 accumulation.  The 32x32x16 shape
//    keeps the matrix core at full rate with one wave per SIMD and lets the
//    decode VALU issue while it runs.
//  * Workgroup = 4 waves (one per SIMD), output tile = up to 128 rows x 256
//    columns of one group.  Wave w owns columns [64 w, 64 w + 64) of the tile
//    and every row of it, and decodes both its B columns and the tile's A
//    rows itself, straight into MFMA operand registers, one MFMA step ahead.
//    Raw codes and scales arrive by direct HBM-to-LDS loads into a ring of
//    kRing 64-k stages that belongs to the wave alone, so the waves never
//    wait for each other inside the loop.
//  * One workgroup per CU, each with one contiguous range of the launch's
//    (tile, 256-k unit) sequence ("stream-K"); the host balances the ranges
//    with a clock model of the kernel, and a tile split between workgroups
//    is summed by the one holding its first unit.
//  * Inside a 64-k stage lane (r, h) of a wave (r = lane % 32, h = lane / 32)
//    holds k = 32 h + 8 s + [0, 8) of its row (A) or column (B) at MFMA step
//    s; A and B use the same permutation of k, which leaves the sum unchanged
//    and lets every lane fetch 16 contiguous code bytes per row and stage.
//  * Accuracy: the MFMA accumulators restart from zero every 512 k and are
//    then added into a separate fp32 sum, so rounding happens at the
//    magnitude of 512-k partial sums instead of the running total.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "nvfp4_group_gemm.h"

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;                       // waves per workgroup (one per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kBlockM = 32;                     // rows of one MFMA block
constexpr int kRowBlocks = 4;                   // row blocks of a full tile
constexpr int kTileM = kBlockM * kRowBlocks;    // 128
constexpr int kWaveCols = 64;                   // columns per wave (two 32-column blocks)
constexpr int kTileN = kWaveCols * kWaves;      // 256
constexpr int kStageK = 64;                     // k per pipeline stage (4 MFMA steps of 16)
constexpr int kUnitK = 256;                     // k per scheduling unit
constexpr int kStagesPerUnit = kUnitK / kStageK;
constexpr int kFoldStages = 8;                  // stages summed by MFMA before a fold (512 k)
constexpr int kRing = 5;                        // stages in a wave's raw-code ring
constexpr int kMaxGroupsPerLaunch = 32;
constexpr int kMaxWorkgroups = 256;             // workgroups of one launch (one per CU on MI355X)

// Work decomposition.  A group's output is cut into tiles of up to kTileM
// rows (the rows spread evenly over the fewest tiles, rounded up to 32) by
// kTileN columns; K is cut into units of kUnitK.  The (tile, unit) pairs of a
// launch are ordered group by group, column strip by column strip, row tile
// by row tile, unit by unit, and every workgroup takes one contiguous range
// of that order ("stream-K").  The host chooses the ranges (plan_cuts) by
// balancing a clock model of each workgroup.  A tile whose units fall into
// several ranges is finished by the workgroup holding its first unit; the
// others leave fp32 partial sums in a workspace.
// Positions in the order are cost coordinates: a tile is [head][unit 0]
// [unit 1]..., a unit of a tile with nrb row blocks spans unit_cost(nrb,
// nunits) coordinates and a head kCostHead, and a unit belongs to the range
// (lo, hi] that holds its end.  The host places cuts on unit ends, so these
// weights only fix the coordinates.
constexpr int kCostRowBlock = 8;
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
    int32_t tile_rows;   // rows per tile (multiple of 32, <= kTileM)
    int32_t col_tiles;   // tiles along N
    int32_t nunits;      // units along K (>= 1)
    int32_t cost_full;   // cost of one unit of a tile with tile_rows rows
    int32_t cost_last;   // cost of one unit of the last row tile
    int32_t pad_;
    int64_t strip_cost;  // cost of one column strip (all row tiles with heads)
    int64_t cost_begin;  // cost before this group's first tile
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
    // launch replayed from a captured graph still gets a fresh epoch)
    uint32_t *control;
    int32_t spin_limit;  // flag polls before a missing part is recomputed instead
    // Workgroup w's range is the cost interval (cut[w], cut[w + 1]]: the
    // units whose end cost lies in it belong to w (cut[0] = 0, cut[num_wg] =
    // total_cost, non-decreasing; chosen on the host)
    int64_t cut[kMaxWorkgroups + 1];
    // workgroup w's first tile and unit (pack_start), found by the host
    uint64_t start[kMaxWorkgroups];
};

__host__ __device__ inline int unit_cost(int nrb, int nunits)
{
    return kCostRowBlock * nrb + kCostFixed + (kCostSpread + nunits - 1) / nunits;
}

// Position of one tile and of a unit in it.
struct TilePos {
    int g, strip, rt;       // group, column strip, row tile
    int unit;               // first unit of interest
    int64_t cost_begin;     // cost where the tile (its head) starts
    int ucost;              // cost of each of its units
    int nrb;                // 32-row blocks of the tile
};

__host__ __device__ inline int tile_nrb(const GroupArgs &G, int rt)
{
    const int rows = G.m - rt * G.tile_rows < G.tile_rows ? G.m - rt * G.tile_rows : G.tile_rows;
    return (rows + kBlockM - 1) / kBlockM;
}

// First unit of a tile starting at cost `start` (units of cost uc) whose
// end cost is > x; nunits when there is none.
__host__ __device__ inline int first_unit_ending_after(int64_t start, int uc, int nunits, int64_t x)
{
    const int64_t off = x - start - kCostHead;     // unit j ends at (j + 1) uc
    if (off < 0)
        return 0;
    const int64_t j = off / uc;
    return (int)(j < nunits ? j : nunits);
}

__host__ __device__ inline void finish_pos(const GroupArgs &G, TilePos &p)
{
    const int64_t full = kCostHead + (int64_t)G.nunits * G.cost_full;
    p.cost_begin = G.cost_begin + p.strip * G.strip_cost + p.rt * full;
    p.ucost = p.rt == G.row_tiles - 1 ? G.cost_last : G.cost_full;
    p.nrb = tile_nrb(G, p.rt);
}

// The tile holding the first unit whose end cost is > x (g == ng: none).
inline TilePos locate(const LaunchArgs &args, int64_t x)
{
    const GroupArgs *gs = args.g;
    const int ng = args.ng;
    const int64_t total = args.total_cost;
    TilePos p{ng, 0, 0, 0, total, 1, 1};
    if (x >= total)
        return p;
    int g = 0;
    for (int i = 1; i < kMaxGroupsPerLaunch; ++i)
        g += args.group_begin[i] <= x ? 1 : 0;
    const GroupArgs &G = gs[g];
    int64_t off = x - G.cost_begin;
    p.g = g;
    p.strip = (int)(off / G.strip_cost);
    off -= p.strip * G.strip_cost;
    const int64_t full = kCostHead + (int64_t)G.nunits * G.cost_full;
    if (off < (int64_t)(G.row_tiles - 1) * full) {
        p.rt = (int)(off / full);
        p.unit = first_unit_ending_after(p.rt * full, G.cost_full, G.nunits, off);
    } else {
        p.rt = G.row_tiles - 1;
        p.unit = first_unit_ending_after((int64_t)(G.row_tiles - 1) * full, G.cost_last, G.nunits, off);
    }
    if (p.unit >= G.nunits) {        // no unit of this tile ends after x: start at the next tile
        p.unit = 0;
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

// The tile after p (unit 0); g == ng past the last tile.
__host__ __device__ inline TilePos next_tile(const GroupArgs *gs, int ng, int64_t total, TilePos p)
{
    p.unit = 0;
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

// A tile position packed into 64 bits: unit [0, 20), row tile [20, 38),
// column strip [38, 58), group [58, 64) (63: no tile).
__host__ __device__ inline uint64_t pack_start(const TilePos &p, int ng)
{
    if (p.g >= ng)
        return 63ull << 58;
    return (uint64_t)p.unit | (uint64_t)p.rt << 20 | (uint64_t)p.strip << 38 | (uint64_t)p.g << 58;
}

__host__ __device__ inline TilePos unpack_start(const LaunchArgs &args, uint64_t v)
{
    TilePos p{(int)(v >> 58), (int)((v >> 38) & 0xFFFFF), (int)((v >> 20) & 0x3FFFF), (int)(v & 0xFFFFF),
              args.total_cost, 1, 1};
    if (p.g < args.ng)
        finish_pos(args.g[p.g], p);
    else
        p.g = args.ng;
    return p;
}

// Units [*ub, *ue) of the tile at p whose end cost lies in (lo, hi].
__host__ __device__ inline void units_in(const TilePos &p, int nunits, int64_t lo, int64_t hi, int &ub, int &ue)
{
    ub = first_unit_ending_after(p.cost_begin, p.ucost, nunits, lo);
    ue = first_unit_ending_after(p.cost_begin, p.ucost, nunits, hi);
}

// Bytes of one workgroup's partial-sum slot: [wave][row block][cb][lane] f32x16.
constexpr uint32_t kPartialSlot = kWaves * kRowBlocks * 2u * 64u * 64u;

// ---------------------------------------------------------------- device --

// Eight E2M1 codes (one dword, element i in nibble i) times one scale, as
// eight exact fp16 values.  The convert instruction applies a power-of-two
// scale only, so it runs with 1.0 and the E4M3 scale is applied by a packed
// f16 multiply (exact: <= 6 significant bits, result in the normal range).
__device__ __forceinline__ f16x8 decode8(uint32_t codes, _Float16 s)
{
    const f16x2 ss = {s, s};
    const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * ss;
    const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * ss;
    const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * ss;
    const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * ss;
    const f16x8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    return r;
}

// The two E4M3FN scale bytes in the low half of a dword -> an fp16 pair.
__device__ __forceinline__ f16x2 scales2(uint32_t bytes)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bytes, 1.0f, false);
}

// ---- LDS layout ----------------------------------------------------------
// Each wave owns kRing stage slots of kSlotBytes.  A slot holds what the
// wave fetched for one 64-k stage (lane l's bytes at size * l):
//   A codes  [row block][lane] x 16 B  (row 32 rb + lane % 32, k 32 (lane / 32) + [0, 32))
//   B codes  [cb][lane] x 16 B        (column 64 w + 32 cb + lane % 32)
//   A scales [r][rb] x 4 B             (the stage's four scale bytes of row 32 rb + r)
//   B scales [r][cb] x 4 B             (likewise for column 64 w + 32 cb + r)
// After a segment the ring is free and its first 4 KiB serve as the wave's
// staging area for the transposed fp16 output.
constexpr uint32_t kSlotACodes = 0;
constexpr uint32_t kSlotBCodes = kSlotACodes + kRowBlocks * 1024u;
constexpr uint32_t kSlotAScales = kSlotBCodes + 2u * 1024u;
constexpr uint32_t kSlotBScales = kSlotAScales + kTileM * 4u;
constexpr uint32_t kSlotBytes = kSlotBScales + kWaveCols * 4u;
constexpr uint32_t kWaveRing = kRing * kSlotBytes;
constexpr uint32_t kLdsBytes = kWaves * kWaveRing;
static_assert(kLdsBytes <= 160u * 1024u, "LDS budget of one CU");

// Buffer resource over `bytes` bytes at `p` (raw buffer, no stride); reads
// past the end return zero.
__device__ __forceinline__ i32x4 rsrc(const void *p, uint32_t bytes)
{
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const i32x4 r = {(int32_t)(uint32_t)a, (int32_t)(uint32_t)(a >> 32) & 0xFFFF, (int32_t)bytes, 0x00020000};
    return r;
}

// Direct HBM -> LDS load: lane l's 16 (or 4) bytes at voff + soff land at
// LDS byte lds + 16 l (4 l); a buffer resource reads 0 past its end.  The
// load is issued from inline assembly that sets m0 (the LDS address) and
// restores it, so the compiler neither loses a value it keeps in m0 nor
// sees an LDS write it would have to wait for before every later LDS read
// (it cannot tell the ring slots apart).  Callers wait for these loads
// with an explicit vmcnt before reading what they wrote.
__device__ __forceinline__ void dma16(i32x4 rs, uint32_t lds, uint32_t voff, uint32_t soff)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(lds), "v"(voff), "s"(rs), "s"(soff) : "memory");
}
__device__ __forceinline__ void dma4(i32x4 rs, uint32_t lds, uint32_t voff, uint32_t soff)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "buffer_load_dword %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(lds), "v"(voff), "s"(rs), "s"(soff) : "memory");
}

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding), not
// moved across by the scheduler.
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

// Raw codes and scale bytes of one stage, as one lane holds them.
template <int NRB>
struct StageRaw {
    u32x4 a[NRB];   // dword s: the eight codes of MFMA step s, per row block
    u32x4 b[2];     // likewise per column block
    u32x4 sa;       // dword rb: scale bytes of row 32 rb + r (bytes 2h, 2h + 1 are this lane's)
    u32x2 sb;       // dword cb: scale bytes of column 32 cb + r
};

// Stage units [ub, ue) of one output tile with NRB row blocks (compile time,
// so the hot loop has no branches), added into `outer`.  The tile is rows
// [m0, m0 + 32 NRB) and columns [n0, n0 + 256) of one group; wave `wave`
// owns columns n0 + 64 wave + [0, 64).  Lane (r, h) of the wave holds
// outer[i][cb][v] = C[m0 + 32 i + 8 (v / 4) + 4 h + v % 4][n0 + 64 wave + 32 cb + r].
template <int NRB>
__device__ __forceinline__ void segment(const GroupArgs &G, int m0, int n0, int wave, uint8_t *smem,
                                        int ub, int ue, f32x16 (&outer)[NRB][2])
{
    const int M = G.m, N = G.n, K = G.k;
    const int lane = lane_id();
    const int r = lane & 31, h = lane >> 5;
    const uint32_t row_bytes = (uint32_t)K >> 1, row_scales = (uint32_t)K >> 4;
    const int nstages = K / kStageK;
    const int c_begin = ub * kStagesPerUnit;
    const int c_end = min(ue * kStagesPerUnit, nstages);
    if (c_begin >= c_end)
        return;

    const i32x4 ra_codes = rsrc(G.a, (uint32_t)M * row_bytes);
    const i32x4 ra_scales = rsrc(G.sfa, (uint32_t)M * row_scales);
    const i32x4 rb_codes = rsrc(G.b, (uint32_t)N * row_bytes);
    const i32x4 rb_scales = rsrc(G.sfb, (uint32_t)N * row_scales);
    uint8_t *ring = smem + wave * kWaveRing;
    const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;

    // Per-lane byte offsets of what the lane fetches each stage (the stage
    // adds its k offset as the scalar offset).  Rows past M and columns past
    // N lie past the resource's end and read as 0.
    uint32_t voff_a[NRB], voff_b[2], voff_sa[2], voff_sb;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
        voff_a[rb] = ((uint32_t)(m0 + kBlockM * rb + r)) * row_bytes + 16u * (uint32_t)h;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
        voff_b[cb] = ((uint32_t)(n0 + kWaveCols * wave + 32 * cb + r)) * row_bytes + 16u * (uint32_t)h;
    // A scales: load i, lane l fetches row 32 (l % 4) + 16 i + l / 4, landing at [r][rb]
#pragma unroll
    for (int i = 0; i < 2; ++i)
        voff_sa[i] = ((uint32_t)(m0 + 32 * (lane & 3) + 16 * i + (lane >> 2))) * row_scales;
    // B scales: lane l fetches column 32 (l % 2) + l / 2, landing at [r][cb]
    voff_sb = ((uint32_t)(n0 + kWaveCols * wave + 32 * (lane & 1) + (lane >> 1))) * row_scales;

    // Fetch stage c (clamped to the group's last stage, so the number of
    // loads in flight never depends on K) into ring slot `slot`: NRB + 2
    // code loads and 3 scale loads.
    auto fetch = [&](int c, int slot) {
        const uint32_t k0 = (uint32_t)min(c, nstages - 1) * kStageK;
        const uint32_t s = ring_lds + (uint32_t)slot * kSlotBytes;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
            dma16(ra_codes, s + kSlotACodes + rb * 1024u, voff_a[rb], k0 >> 1);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
            dma16(rb_codes, s + kSlotBCodes + cb * 1024u, voff_b[cb], k0 >> 1);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            dma4(ra_scales, s + kSlotAScales + 256u * i, voff_sa[i], k0 >> 4);
        dma4(rb_scales, s + kSlotBScales, voff_sb, k0 >> 4);
    };
    constexpr int kLoadsPerStage = NRB + 5;
    // at the top of stage c the loads of stages c + 2 .. c + kRing - 1 may
    // still be in flight; those of stage c + 1 must have landed
    constexpr int kWaitNext = (kRing - 2) * kLoadsPerStage;

    auto read_raw = [&](int slot) -> StageRaw<NRB> {
        const uint8_t *s = ring + slot * kSlotBytes;
        const int l = lane_id();
        StageRaw<NRB> v;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
            v.a[rb] = reinterpret_cast<const u32x4 *>(s + kSlotACodes + rb * 1024)[l];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
            v.b[cb] = reinterpret_cast<const u32x4 *>(s + kSlotBCodes + cb * 1024)[l];
        v.sa = reinterpret_cast<const u32x4 *>(s + kSlotAScales)[l & 31];
        v.sb = reinterpret_cast<const u32x2 *>(s + kSlotBScales)[l & 31];
        return v;
    };

    // Per-stage fp16 scales of this lane: [0] for steps 0-1, [1] for steps 2-3.
    struct Scales {
        f16x2 a[NRB];
        f16x2 b[2];
    };
    auto scales_of = [&](const StageRaw<NRB> &v) -> Scales {
        Scales sc;
        const uint32_t sh = 16u * (uint32_t)h;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
            sc.a[rb] = scales2(v.sa[rb] >> sh);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
            sc.b[cb] = scales2(v.sb[cb] >> sh);
        return sc;
    };

    f32x16 inner[NRB][2];
    f16x8 da[2][NRB], db[2][2];     // decoded operands of two MFMA steps

    auto decode_step = [&](const StageRaw<NRB> &v, const Scales &sc, int s, f16x8 (&oa)[NRB], f16x8 (&ob)[2]) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
            oa[rb] = decode8(v.a[rb][s], sc.a[rb][s >> 1]);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
            ob[cb] = decode8(v.b[cb][s], sc.b[cb][s >> 1]);
    };

    // prologue: stages c_begin .. c_begin + kRing - 2 in flight, stage
    // c_begin read and its step 0 decoded
#pragma unroll
    for (int i = 0; i < kRing - 1; ++i)
        fetch(c_begin + i, i);
    wait_vmcnt<kWaitNext>();
    StageRaw<NRB> cur = read_raw(0);
    Scales sc = scales_of(cur);
    decode_step(cur, sc, 0, da[0], db[0]);
    int slot = 0;                   // ring slot of the current stage

    // Stage c: fetch stage c + kRing - 1 into the slot stage c - 1 used (read
    // one stage ago); per MFMA step s: 2 NRB MFMAs on the operands of step s,
    // then decode step s + 1 (at s = 3: step 0 of stage c + 1, whose raw
    // codes are read from the ring at the start of step 3, once stage c's
    // codes are all decoded and their registers are free).
    auto stage = [&](int c, auto first_t) {
        constexpr bool kFirst = decltype(first_t)::value;   // first stage after a fold: MFMA sums restart
        const int fslot = slot == 0 ? kRing - 1 : slot - 1;
        const int nslot = slot == kRing - 1 ? 0 : slot + 1;
        fetch(c + kRing - 1, fslot);
        StageRaw<NRB> nxt;
        Scales nsc;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s == 3) {
                wait_vmcnt<kWaitNext>();
                nxt = read_raw(nslot);
            }
#pragma unroll
            for (int i = 0; i < NRB; ++i)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    inner[i][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        da[s & 1][i], db[s & 1][cb], (kFirst && s == 0) ? f32x16{} : inner[i][cb], 0, 0, 0);
            if (s < 3) {
                decode_step(cur, sc, s + 1, da[(s + 1) & 1], db[(s + 1) & 1]);
            } else {
                nsc = scales_of(nxt);
                decode_step(nxt, nsc, 0, da[0], db[0]);
            }
        }
        cur = nxt;
        sc = nsc;
        slot = nslot;
    };
    auto fold = [&]() {
#pragma unroll
        for (int i = 0; i < NRB; ++i)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                outer[i][cb] += inner[i][cb];
    };

    int c = c_begin;
    while (c < c_end) {
        stage(c, std::true_type{});
        ++c;
        const int n = min(kFoldStages - 1, c_end - c);
        for (int i = 0; i < n; ++i, ++c)
            stage(c, std::false_type{});
        fold();
    }
    // drain the clamped prefetches before the ring is reused
    wait_vmcnt<0>();
}

// fp16 (round to nearest even) of the tile's sums into C, rows < m0 + rows.
// Fast path (n % 4 == 0 and c 8-byte aligned, so every group of four
// columns is wholly inside or outside the matrix): the four lanes of a quad
// (r = 4t .. 4t + 3) hold rows 8 g + 4 h .. + 3 of four consecutive columns
// in accumulator elements 4 g .. 4 g + 3, so a 4 x 4 transpose of fp16
// values across the quad (two DPP exchanges) leaves each lane with four
// consecutive columns of one row, written as one 8-byte store.
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
                                           const f32x16 (&outer)[NRB][2])
{
    const int lane = lane_id();
    const int r = lane & 31, h = lane >> 5;
    _Float16 *C = G.c;
    const int N = G.n;
    if ((N & 3) == 0 && ((uintptr_t)C & 7) == 0) {
        const int u = r & 3;
        const bool odd = (u & 1) != 0, hi2 = (u & 2) != 0;
        // this lane's row within a group of four after the transpose
        const int row_in = 4 * h + 2 * (u & 1) + (u >> 1);
        const int col = n0 + kWaveCols * wave + (r & ~3);
#pragma unroll
        for (int i = 0; i < NRB; ++i) {
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int row = m0 + kBlockM * i + 8 * g + row_in;
                    const f32x16 &v = outer[i][cb];
                    const uint32_t p01 =
                        __builtin_bit_cast(uint32_t, f16x2{(_Float16)v[4 * g], (_Float16)v[4 * g + 1]});
                    const uint32_t p23 =
                        __builtin_bit_cast(uint32_t, f16x2{(_Float16)v[4 * g + 2], (_Float16)v[4 * g + 3]});
                    // step 1: even lanes end with rows +0, +1 and odd lanes with
                    // rows +2, +3, each for the column pair (r & ~1, +1)
                    const uint32_t mine = odd ? p23 : p01;
                    const uint32_t recv = quad_swap1(odd ? p01 : p23);
                    const uint32_t lo = odd ? recv : mine, hi = odd ? mine : recv;
                    const uint32_t rowA = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                    const uint32_t rowB = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
                    // step 2: lanes r and r ^ 2 swap halves of their column quad
                    const uint32_t keep = hi2 ? rowB : rowA;
                    const uint32_t recv2 = quad_swap2(hi2 ? rowA : rowB);
                    const uint64_t out = hi2 ? ((uint64_t)keep << 32 | recv2) : ((uint64_t)recv2 << 32 | keep);
                    const int c0 = col + 32 * cb;
                    if (row < m0 + rows && c0 < N)
                        *reinterpret_cast<uint64_t *>(C + (size_t)row * N + c0) = out;
                }
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int col = n0 + kWaveCols * wave + 32 * cb + r;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + kBlockM * i + 8 * (v >> 2) + 4 * h + (v & 3);
                if (row < m0 + rows && col < N)
                    C[(size_t)row * N + col] = (_Float16)outer[i][cb][v];
            }
        }
    }
}

// Partial sums of split tiles.  Slot w (one per workgroup) holds the sums of
// workgroup w's first segment in the register layout of `outer`:
// [wave][row block][cb][lane] x f32x16.  They are written and read with
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
    return slot * (int)kPartialSlot + wave * kRowBlocks * 2 * 4096;
}

// Producer side: publish the partial sums of this workgroup's first segment.
template <int NRB>
__device__ __forceinline__ void publish_partial(const LaunchArgs &args, uint32_t epoch, int slot, int wave,
                                                const f32x16 (&outer)[NRB][2])
{
    const int lane = lane_id();
    const __amdgpu_buffer_rsrc_t rs = partial_rsrc(args);
    const int base = partial_base(slot, wave);
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v = {outer[i][cb][4 * q], outer[i][cb][4 * q + 1], outer[i][cb][4 * q + 2],
                                 outer[i][cb][4 * q + 3]};
                __builtin_amdgcn_raw_buffer_store_b128(v, rs, lane * 16, base + ((i * 2 + cb) * 4 + q) * 1024,
                                                       kCoherent);
            }
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
    const bool ok = ready != 0;
    __syncthreads();               // `ready` is read by everyone before the next reuse
    return ok;
}

template <int NRB>
__device__ __forceinline__ void add_partial(const LaunchArgs &args, int slot, int wave, f32x16 (&outer)[NRB][2])
{
    const int lane = lane_id();
    const __amdgpu_buffer_rsrc_t rs = partial_rsrc(args);
    const int base = partial_base(slot, wave);
    // all loads of a row block first, then the adds: one memory latency per
    // row block instead of one per load
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
        f32x4 v[2][4];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                v[cb][q] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16, base + ((i * 2 + cb) * 4 + q) * 1024,
                                                                 kCoherent);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    outer[i][cb][4 * q + e] += v[cb][q][e];
    }
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
// small next to rms(C) is 3.3 sigma.
constexpr float kSigmaMargin = 6.0f;
constexpr float kTolRel = 2e-3f;
constexpr float kTolAbs = 1e-2f;

// Sum of the products of eight E2M1 code pairs (one dword each), exact in
// fp32 (multiples of 1/4 below 2^9).
__device__ __forceinline__ float code_dot8(uint32_t xa, uint32_t xb)
{
    float s = 0.0f;
    const auto a0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(xa, 1.0f, 0);
    const auto b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(xb, 1.0f, 0);
    const auto a1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(xa, 1.0f, 1);
    const auto b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(xb, 1.0f, 1);
    const auto a2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(xa, 1.0f, 2);
    const auto b2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(xb, 1.0f, 2);
    const auto a3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(xa, 1.0f, 3);
    const auto b3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(xb, 1.0f, 3);
    s += a0[0] * b0[0];
    s += a0[1] * b0[1];
    s += a1[0] * b1[0];
    s += a1[1] * b1[1];
    s += a2[0] * b2[0];
    s += a2[1] * b2[1];
    s += a3[0] * b3[0];
    s += a3[1] * b3[1];
    return s;
}

// Exact value of one output: per 16-k block, the sum of the 16 code
// products is exact in fp32 (multiples of 1/4, |sum| <= 576), times both
// block scales exact in fp64, summed over blocks in fp64.  Every lane takes
// blocks lane, lane + 64, ...; the wave's partial sums are combined at the
// end, and every lane returns the total.
__device__ __noinline__ double exact_entry(const uint8_t *a, const uint8_t *sfa, const uint8_t *b, const uint8_t *sfb,
                                           int m, int n, int K)
{
    const int lane = threadIdx.x & 63;
    const int nb = K >> 4;
    const uint8_t *ar = a + (size_t)m * (size_t)(K >> 1);
    const uint8_t *br = b + (size_t)n * (size_t)(K >> 1);
    const uint8_t *sar = sfa + (size_t)m * (size_t)nb;
    const uint8_t *sbr = sfb + (size_t)n * (size_t)nb;
    double acc = 0.0;
    for (int blk0 = 0; blk0 < nb; blk0 += 64 * 8) {
        uint2 ca[8], cb[8];
        uint32_t sa[8], sb[8];
        // all loads of up to eight blocks first: one memory latency
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int blk = blk0 + 64 * j + lane;
            const bool in = blk < nb;
            ca[j] = in ? *reinterpret_cast<const uint2 *>(ar + 8 * blk) : make_uint2(0, 0);
            cb[j] = in ? *reinterpret_cast<const uint2 *>(br + 8 * blk) : make_uint2(0, 0);
            sa[j] = in ? sar[blk] : 0u;
            sb[j] = in ? sbr[blk] : 0u;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                const uint32_t xa = w ? ca[j].y : ca[j].x, xb = w ? cb[j].y : cb[j].x;
                s += code_dot8(xa, xb);
            }
            const double scale = (double)__builtin_amdgcn_cvt_scalef32_f32_fp8(sa[j], 1.0f, 0) *
                                 (double)__builtin_amdgcn_cvt_scalef32_f32_fp8(sb[j], 1.0f, 0);
            acc += (double)s * scale;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        acc += __shfl_xor(acc, off);
    return acc;
}

// The check and the exact recomputation for one finished tile (see above);
// `parts` is the number of partial sums the finalizer added.
template <int NRB>
__device__ __forceinline__ void fix_small_outputs(const GroupArgs &G, int m0, int rows, int n0, int wave, int parts,
                                                  f32x16 (&outer)[NRB][2])
{
    const int lane = lane_id();
    const int r = lane & 31, h = lane >> 5;
    const int row_end = m0 + rows;
    const int col_base = n0 + kWaveCols * wave + r;
    float ss = 0.0f;
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + kBlockM * i + 8 * (v >> 2) + 4 * h + (v & 3);
                const float x = outer[i][cb][v];
                const bool use = row < row_end && col_base + 32 * cb < G.n && __builtin_isfinite(x);
                ss += use ? x * x : 0.0f;
                cnt += use ? 1 : 0;
            }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        ss += __shfl_xor(ss, off);
        cnt += __shfl_xor(cnt, off);
    }
    if (cnt == 0)
        return;
    const float K = (float)G.k;
    const float F = (float)(kFoldStages * kStageK);
    const float sigma = 0x1p-24f * __builtin_sqrtf(ss / (float)cnt) *
                        __builtin_sqrtf(fminf(F, K) / 16.0f + K / (2.0f * F) + (float)parts);
    const float thresh = (kSigmaMargin * sigma - kTolAbs) / kTolRel;   // recompute |c| < thresh
    if (!(thresh > 0.0f))
        return;
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + kBlockM * i + 8 * (v >> 2) + 4 * h + (v & 3);
                const int col = col_base + 32 * cb;
                const bool flag = row < row_end && col < G.n && __builtin_fabsf(outer[i][cb][v]) < thresh;
                uint64_t todo = __ballot(flag);
                while (todo) {
                    const int owner = __builtin_ctzll(todo);
                    todo &= todo - 1;
                    const int orow = __shfl(row, owner), ocol = __shfl(col, owner);
                    const double e = exact_entry(G.a, G.sfa, G.b, G.sfb, orow, ocol, G.k);
                    if (lane == owner)
                        outer[i][cb][v] = (float)e;
                }
            }
}

// One tile's share of this workgroup: units [ub, ue).  `w` is the logical
// workgroup index.
template <int NRB>
__device__ __forceinline__ void run_tile(const LaunchArgs &args, uint32_t epoch, const TilePos &p, int ub, int ue,
                                         int w, int wave, uint8_t *smem)
{
    const GroupArgs &G = args.g[p.g];
    const int m0 = p.rt * G.tile_rows, n0 = p.strip * kTileN;
    const int rows = min(G.tile_rows, G.m - m0);
    f32x16 outer[NRB][2];
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
            outer[i][cb] = f32x16{};
    // One call site of the pipelined loop: the own segment first, then (on
    // the finalizer) any producer part that did not arrive in time.
    int sb = ub, se = ue, w2 = w;
    int parts = 0;                 // partial sums added by this finalizer
    for (;;) {
        segment<NRB>(G, m0, n0, wave, smem, sb, se, outer);
        if (ub > 0) {              // a later part of a split tile
            publish_partial<NRB>(args, epoch, w, wave, outer);
            return;
        }
        // finalizer: add the other parts of the tile in k order
        bool recompute = false;
        const int64_t tile_end = p.cost_begin + kCostHead + (int64_t)G.nunits * p.ucost;
        while (ue < G.nunits && ++w2 < args.num_wg) {
            const int64_t lo = args.cut[w2];
            const int64_t hi = args.cut[w2 + 1];
            if (lo >= tile_end)
                break;
            int qb, qe;
            units_in(p, G.nunits, lo, hi, qb, qe);
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
    fix_small_outputs<NRB>(G, m0, rows, n0, wave, parts, outer);
    store_tile<NRB>(G, m0, rows, n0, wave, outer);
}

__global__ __launch_bounds__(kThreads, 1) void nvfp4_group_gemm_kernel(const LaunchArgs args)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];

    // Logical workgroup index: consecutive ranges (which share A rows and B
    // columns) on the same XCD when workgroups are dealt round-robin to 8 XCDs.
    const int b = blockIdx.x, nwg = args.num_wg;
    const int w = (nwg % 8 == 0) ? (b % 8) * (nwg / 8) + b / 8 : b;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // this launch's epoch: one past the last finished launch's (0 marks an
    // unwritten flag); no workgroup changes it before all have started
    const uint32_t last = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)__hip_atomic_load(&args.control[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    const uint32_t epoch = last + 1u == 0u ? 1u : last + 1u;
    const int64_t lo = args.cut[w];
    const int64_t hi = args.cut[w + 1];

    TilePos p = unpack_start(args, args.start[w]);
    while (p.g < args.ng) {
        const int nunits = args.g[p.g].nunits;
        int ub, ue;
        units_in(p, nunits, lo, hi, ub, ue);
        if (ub >= ue)
            break;
        switch (p.nrb) {
        case 1: run_tile<1>(args, epoch, p, ub, ue, w, wave, smem); break;
        case 2: run_tile<2>(args, epoch, p, ub, ue, w, wave, smem); break;
        case 3: run_tile<3>(args, epoch, p, ub, ue, w, wave, smem); break;
        default: run_tile<4>(args, epoch, p, ub, ue, w, wave, smem); break;
        }
        if (ue < nunits)
            break;                 // the range ends inside this tile
        p = next_tile(args.g, args.ng, args.total_cost, p);
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
        if (G.reserved != 0)
            return fail(NVFP4_EINVAL, "group %d: reserved field must be 0", i);
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
        if (G.k % kStageK != 0)
            return fail(NVFP4_EUNSUPPORTED, "group %d: k=%d is not a multiple of %d", i, G.k, kStageK);
        if ((uint64_t)(G.m > G.n ? G.m : G.n) * (uint64_t)(G.k / 2) >= (1ull << 31))
            return fail(NVFP4_EUNSUPPORTED, "group %d: an operand reaches 2 GiB", i);
        if (((uintptr_t)G.c & 3u) != 0)
            return fail(NVFP4_EUNSUPPORTED, "group %d: c is not 4-byte aligned", i);
        if (G.k > 0 && ((((uintptr_t)G.a | (uintptr_t)G.b) & 15u) != 0 ||
                        (((uintptr_t)G.sfa | (uintptr_t)G.sfb) & 3u) != 0))
            return fail(NVFP4_EUNSUPPORTED, "group %d: operand pointer misaligned", i);
    }
    return NVFP4_OK;
}

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Row tiling of a group: the fewest tiles of at most kTileM rows, with the
// rows spread evenly (rounded up to 32) so a ragged M wastes little.
inline void row_tiling(int m, int &tiles, int &rows_per_tile)
{
    tiles = ceil_div(m, kTileM);
    rows_per_tile = kBlockM * ceil_div(ceil_div(m, tiles), kBlockM);
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
        A.c = static_cast<_Float16 *>(G.c);
        A.m = G.m;
        A.n = G.n;
        A.k = G.k;
        row_tiling(G.m, A.row_tiles, A.tile_rows);
        A.col_tiles = ceil_div(G.n, kTileN);
        A.nunits = ceil_div(G.k, kUnitK);
        if (A.nunits < 1)
            A.nunits = 1;      // k == 0: one empty unit, the tile is still written
        A.cost_full = unit_cost(A.tile_rows / kBlockM, A.nunits);
        A.cost_last = unit_cost(tile_nrb(A, A.row_tiles - 1), A.nunits);
        A.strip_cost = (int64_t)A.row_tiles * kCostHead +
                       (int64_t)A.nunits * ((int64_t)(A.row_tiles - 1) * A.cost_full + A.cost_last);
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

int64_t total_units(const LaunchArgs &args)
{
    int64_t t = 0;
    for (int i = 0; i < args.ng; ++i)
        t += (int64_t)args.g[i].row_tiles * args.g[i].col_tiles * args.g[i].nunits;
    return t;
}

int grid_for(const LaunchArgs &args, int units)
{
    const int64_t tu = total_units(args);
    int64_t g = tu < units ? tu : units;
    if (g > kMaxWorkgroups)
        g = kMaxWorkgroups;
    return (int)g;
}

// Partition of a launch's (tile, unit) sequence among num_wg workgroups.
// A greedy fill against a target makespan, binary-searched: each workgroup
// takes units in order while its modelled time stays within the target.
// The model (clocks) charges a workgroup its start-up, a pipeline fill per
// segment (the first one dearer), the units (per tile height: a unit of a
// short tile is bound by streaming B, not by its MFMAs), and each
// segment's epilogue:
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
constexpr double kClkStart = 3000;
constexpr double kClkFillFirst = 6000;
constexpr double kClkFillNext = 4000;
constexpr double kClkUnit[kRowBlocks + 1] = {0, 2800, 3300, 4200, 5200};
constexpr double kClkPublish = 4000;
constexpr double kClkStore = 3000;
constexpr double kClkAdd = 3500;

// One tile of the launch for the partition: where it starts in cost order,
// its unit cost there, and its units' modelled clocks.
struct PlanTile {
    int64_t cost_begin;
    int32_t ucost, nunits;
    double unit_clk;
};

bool greedy_cuts(const std::vector<PlanTile> &tiles, int nwg, int64_t total, double tmax, int64_t *cut)
{
    int w = 0;
    double cur = kClkStart;
    bool fresh = true;             // workgroup w has no segment yet
    cut[0] = 0;
    for (const PlanTile &t : tiles) {
        const int nunits = t.nunits;
        const double uc = t.unit_clk;
        int j = 0;
        while (j < nunits) {
            const double base = cur + (fresh ? kClkFillFirst : kClkFillNext);
            const int rest = nunits - j;
            const double epi_full = j == 0 ? kClkStore : kClkPublish;
            // a last part of a split tile leaves the finalizer its sum and store
            const double tail = j == 0 ? 0.0 : kClkAdd + kClkStore;
            if (base + rest * uc + epi_full + tail <= tmax) {   // the rest of the tile fits
                cur = base + rest * uc + epi_full;
                fresh = false;
                break;
            }
            // units this workgroup can take before its range ends in the tile
            auto take = [&](double epi) {
                const double fit = (tmax - base - epi) / uc;
                return fit < 0 ? 0 : (fit > rest - 1 ? rest - 1 : (int)fit);
            };
            auto next_takes_rest = [&](int rr) {
                return kClkStart + kClkFillFirst + rr * uc + kClkPublish + kClkAdd + kClkStore <= tmax;
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
            // workgroup w ends with unit j - 1 of this tile (or before the tile)
            if (++w >= nwg)
                return false;
            cut[w] = j == 0 ? t.cost_begin : t.cost_begin + kCostHead + (int64_t)j * t.ucost;
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
    uint64_t start[kMaxWorkgroups];
};
thread_local CutCache g_cut_cache;

void plan_cuts(LaunchArgs &a, int nwg)
{
    CutCache &cc = g_cut_cache;
    bool same = cc.nwg == nwg && cc.ng == a.ng;
    for (int i = 0; same && i < a.ng; ++i)
        same = cc.mnk[i][0] == a.g[i].m && cc.mnk[i][1] == a.g[i].n && cc.mnk[i][2] == a.g[i].k;
    if (same) {
        memcpy(a.cut, cc.cut, sizeof(int64_t) * (nwg + 1));
        memcpy(a.start, cc.start, sizeof(uint64_t) * nwg);
        return;
    }
    std::vector<PlanTile> tiles;
    double work = 0, biggest = 0;
    for (TilePos p = locate(a, 0); p.g < a.ng; p = next_tile(a.g, a.ng, a.total_cost, p)) {
        const PlanTile t{p.cost_begin, p.ucost, a.g[p.g].nunits, kClkUnit[p.nrb]};
        const double tile = kClkFillFirst + kClkStore + 2 * kClkAdd + t.nunits * t.unit_clk;
        work += t.nunits * t.unit_clk;
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
    for (int w = 0; w < nwg; ++w)
        a.start[w] = pack_start(locate(a, a.cut[w]), a.ng);
    cc.nwg = nwg;
    cc.ng = a.ng;
    for (int i = 0; i < a.ng; ++i) {
        cc.mnk[i][0] = a.g[i].m;
        cc.mnk[i][1] = a.g[i].n;
        cc.mnk[i][2] = a.g[i].k;
    }
    memcpy(cc.cut, a.cut, sizeof(int64_t) * (nwg + 1));
    memcpy(cc.start, a.start, sizeof(uint64_t) * nwg);
}

// Library-owned workspace for one stream: partial-sum slots, their flags,
// and two control words after the flags (the epoch of the last finished
// launch and a count of finished workgroups).
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
        e = hipMalloc(reinterpret_cast<void **>(&ws.flags), ((size_t)slots + 2) * sizeof(uint32_t));
    if (e == hipSuccess)
        e = hipMemsetAsync(ws.flags, 0, ((size_t)slots + 2) * sizeof(uint32_t), st);
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

}  // namespace

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
        for (int w = 0; w < nwg; ++w) {
            const int64_t lo = args.cut[w];
            const int64_t hi = args.cut[w + 1];
            TilePos p = unpack_start(args, args.start[w]);
            while (p.g < args.ng) {
                const GroupArgs &G = args.g[p.g];
                int ub, ue;
                units_in(p, G.nunits, lo, hi, ub, ue);
                if (ub >= ue)
                    break;
                if (segs != nullptr && count < cap) {
                    int32_t *o = segs + 8 * count;
                    const int m0 = p.rt * G.tile_rows;
                    o[0] = w;
                    o[1] = map[p.g];
                    o[2] = m0;
                    o[3] = G.m - m0 < G.tile_rows ? G.m - m0 : G.tile_rows;
                    o[4] = p.strip * kTileN;
                    o[5] = kUnitK * ub;
                    o[6] = kUnitK * ue;
                    o[7] = (ub == 0 && ue == G.nunits) ? 0 : (ub > 0 ? 1 : 2);
                }
                ++count;
                if (ue < G.nunits)
                    break;
                p = next_tile(args.g, args.ng, args.total_cost, p);
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
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    int device = 0, units = 0;
    LaunchArgs args;
    int next = 0;
    bool queried = false;
    while (next < ng) {
        if (pack_launch(groups, ng, next, args) == 0)
            break;
        if (!queried) {
            const int rc2 = device_units(device, units);
            if (rc2 != NVFP4_OK)
                return rc2;
            queried = true;
        }
        const int nwg = grid_for(args, units);
        Workspace *ws = nullptr;
        const int rc3 = workspace_for(st, device, units < kMaxWorkgroups ? units : kMaxWorkgroups, ws);
        if (rc3 != NVFP4_OK)
            return rc3;
        args.num_wg = nwg;
        plan_cuts(args, nwg);
        args.partials = ws->partials;
        args.flags = ws->flags;
        args.control = ws->flags + ws->slots;
        args.spin_limit = spin_limit();
        hipLaunchKernelGGL(nvfp4_group_gemm_kernel, dim3((unsigned)nwg), dim3(kThreads), 0, st, args);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return fail(NVFP4_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return NVFP4_OK;
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

extern "C" const char *nvfp4_last_error(void) { return g_err; }
