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
//    ds_read_b128), while each wave streams and decodes its own 32 columns of
//    B straight from HBM into registers.  LDS stages are double-buffered and
//    raw HBM loads are issued two stages ahead.
//  * Inside a 128-k stage lane (r, q) of a wave holds k = 32q + 8s + [0, 8)
//    at MFMA step s; A and B use the same permutation of k, which leaves the
//    sum unchanged and lets every lane read 16 contiguous bytes per row.
//  * Accuracy: the MFMA accumulators restart from zero every 512 k and are
//    then added into a separate fp32 sum.  Rounding therefore happens at the
//    magnitude of 512-k partial sums instead of the full sum, which keeps the
//    error far below the fp16 output tolerance for long K and large scales.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <type_traits>

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
constexpr int kFoldStages = 2;       // stages summed by MFMA before a fold (256 k)
constexpr int kMaxGroupsPerLaunch = 32;

struct GroupArgs {
    const uint8_t *a;
    const uint8_t *b;
    const uint8_t *sfa;
    const uint8_t *sfb;
    _Float16 *c;
    int32_t m, n, k;
    int32_t row_tiles;   // tiles along M
    int32_t tile_rows;   // rows per tile (multiple of 16, <= kTileM)
    int32_t tile_begin;  // index of this group's first tile in the launch
};

struct LaunchArgs {
    GroupArgs g[kMaxGroupsPerLaunch];
    int32_t ng;
    int32_t total_tiles;
};

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
constexpr int kRing = 3;
constexpr uint32_t kLdsAOps = 2u * kRowBlocks * 4u * 64u * 16u;
constexpr uint32_t kRawACodes = 0;
constexpr uint32_t kRawBCodes = kRawACodes + kWaves * 1024u;
constexpr uint32_t kRawStage = kRawBCodes + kWaves * 2u * 1024u;
constexpr uint32_t kWinAScales = 0;
constexpr uint32_t kWinBScales = kWinAScales + kWaves * 256u;
constexpr uint32_t kWindow = kWinBScales + kWaves * 2u * 256u;
constexpr uint32_t kLdsWindows = kLdsAOps + kRing * kRawStage;
constexpr uint32_t kLdsBytes = kLdsWindows + 2u * kWindow;
// Loads a wave issues: 3 code loads every stage, 3 scale loads every odd
// stage; with kRing = 3 stages in flight the count of loads issued after the
// code loads of stage c + 1 is 9 at the start of every stage c.
constexpr int kCodeLoads = 3;
constexpr int kWaitAfterNext = 9;

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
// byte lds + 16 l.  Issued through asm so the compiler does not
// order later LDS reads behind them; callers wait with vmcnt explicitly.
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, i32x4 rs, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
}
// The same for lanes 0..15 only (exec narrowed inside the asm, so the
// compiler sees no divergent branch).
__device__ __forceinline__ void dma16_lanes16(uint32_t lds, uint32_t voff, i32x4 rs, uint32_t soff)
{
    uint64_t saved;
    asm volatile("s_mov_b64 %0, exec\n\ts_mov_b64 exec, 0xffff\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b64 exec, %0"
                 : "=&s"(saved) : "s"(lds), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
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

// Work of one output tile with NRB row blocks (compile-time, so the hot
// loop has no branches).  W waves; the tile is rows [m0, m0 + rows) and
// columns [n0, n0 + 32 W) of one group.
template <int NRB, int W>
__device__ __forceinline__ void tile_body(const GroupArgs &G, int m0, int rows, int n0, int wave,
                                          uint8_t *smem)
{
    const int M = G.m, N = G.n, K = G.k;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, q = lane >> 4;
    const uint32_t row_bytes = (uint32_t)K >> 1, row_scales = (uint32_t)K >> 4;
    const int nstages = (K + kStageK - 1) / kStageK;

    f32x4 outer[NRB][2];
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
            outer[i][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (nstages > 0) {
    const i32x4 ra_codes = rsrc(G.a, (uint32_t)M * row_bytes);
    const i32x4 ra_scales = rsrc(G.sfa, (uint32_t)M * row_scales);
    const i32x4 rb_codes = rsrc(G.b, (uint32_t)N * row_bytes);
    const i32x4 rb_scales = rsrc(G.sfb, (uint32_t)N * row_scales);

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
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const uint32_t col = (uint32_t)min(n0 + 32 * wave + 16 * cb + r, N - 1);
        b_voff[cb] = col * row_bytes + 16u * q;
        sb_voff[cb] = col * row_scales;
    }
    const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
    const uint32_t raw_base = smem_base + kLdsAOps;
    f16x8 *lds_a = reinterpret_cast<f16x8 *>(smem);            // [2][kRowBlocks][4][64]
    auto aop = [&](int buf, int rb, int s) -> f16x8 & {
        return lds_a[((buf * kRowBlocks + rb) * 4 + s) * 64 + lane];
    };

    f32x4 inner[NRB][2];
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
        const uint32_t sk = (uint32_t)min(w, (nstages - 1) >> 1) * (2u * kStageK / 16u);
        const uint32_t win = smem_base + kLdsWindows + (uint32_t)(w & 1) * kWindow;
        dma16_lanes16(win + kWinAScales + wave * 256u, sa_voff, ra_scales, sk);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
            dma16_lanes16(win + kWinBScales + (wave * 2 + cb) * 256u, sb_voff[cb], rb_scales, sk);
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

    // prologue: stages 0, 1, 2 in flight; stage 0 decoded (A to LDS, B to bf)
    fetch_scales(0);
    fetch_scales(1);
    fetch_codes(0);
    fetch_codes(1);
    fetch_codes(2);
    wait_vmcnt<2 * kCodeLoads>();
    {
        const uint8_t *slot = raw_slot(0);
        uint32_t sa, sb[2];
        read_scales(0, sa, sb);
        const f16x2 sca = scales_of(sa, 0);
        const u32x4 ac = a_codes(slot);
#pragma unroll
        for (int s = 0; s < 4; ++s)
            decode_a_into(ac, sca, 0, s);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const f16x2 sc = scales_of(sb[cb], 0);
            const u32x4 bc = b_codes(slot, cb);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                bf[cb][s] = operand(bc[s], sc, s);
        }
    }
    __syncthreads();

    // Stage c: fetch the codes of stage c + 3 into the ring slot stage c used
    // (and, on odd stages, the scale window of stages c + 3 and c + 4 into the
    // window buffer the stages before c used); wait for stage c + 1; per MFMA step s: 2 * NRB MFMAs on the A fragments of step s
    // (read from LDS; a row block's fragment for step s + 1 is read right
    // after its last use), then step s of B (stage c + 1) is decoded into the
    // freed bf slot and step s of A (stage c + 1) into the other LDS buffer.
    // The last stage decodes unused data instead of branching.
    auto stage = [&](int c, auto buf_t) {
        constexpr int kBuf = decltype(buf_t)::value;
        constexpr bool kFirst = kBuf == 0;   // first stage after a fold: MFMA sums restart
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
#pragma unroll
        for (int i = 0; i < NRB; ++i)
            af[i] = aop(kBuf, i, 0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NRB; ++i) {
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    inner[i][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        af[i], bf[cb][s], (kFirst && s == 0) ? f32x4{0.f, 0.f, 0.f, 0.f} : inner[i][cb], 0, 0, 0);
                if (s < 3)
                    af[i] = aop(kBuf, i, s + 1);
            }
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                bf[cb][s] = operand(bc_next[cb][s], sb_next[cb], s);
                asm volatile("" : "+v"(bf[cb][s]));   // keep the decode inside step s
            }
            decode_a_into(ac_next, sa_next, kNext, s);
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    };
    auto fold = [&]() {
#pragma unroll
        for (int i = 0; i < NRB; ++i)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                outer[i][cb] += inner[i][cb];
    };

    // Stages run in pairs (LDS buffer parity) and every pair is folded into
    // `outer`.  An odd stage count gets one extra stage whose scales are all
    // zero (its k lie past K), so the loop body has no branch.
    static_assert(kFoldStages == 2, "one fold per stage pair");
    for (int c = 0; c < nstages; c += 2) {
        stage(c, std::integral_constant<int, 0>{});
        stage(c + 1, std::integral_constant<int, 1>{});
        fold();
    }
    // drain the clamped prefetches before the LDS can be reused
    wait_vmcnt<0>();
    }

    // epilogue: element (16i + 4q + e, 16cb + r) of this wave's 16x16 blocks
    _Float16 *C = G.c;
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

template <int W>
__global__ __launch_bounds__(64 * W, 1) void nvfp4_group_gemm_kernel(const LaunchArgs args)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];

    const int tile = blockIdx.x;
    int g = 0;
    for (int i = 1; i < args.ng; ++i)
        if (args.g[i].tile_begin <= tile)
            g = i;
    const GroupArgs &G = args.g[g];
    const int local = tile - G.tile_begin;
    const int m0 = (local % G.row_tiles) * G.tile_rows;
    const int n0 = (local / G.row_tiles) * (32 * W);
    const int rows = min(G.tile_rows, G.m - m0);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    switch ((rows + 15) >> 4) {
    case 1: tile_body<1, W>(G, m0, rows, n0, wave, smem); break;
    case 2: tile_body<2, W>(G, m0, rows, n0, wave, smem); break;
    case 3: tile_body<3, W>(G, m0, rows, n0, wave, smem); break;
    case 4: tile_body<4, W>(G, m0, rows, n0, wave, smem); break;
    case 5: tile_body<5, W>(G, m0, rows, n0, wave, smem); break;
    case 6: tile_body<6, W>(G, m0, rows, n0, wave, smem); break;
    case 7: tile_body<7, W>(G, m0, rows, n0, wave, smem); break;
    default: tile_body<8, W>(G, m0, rows, n0, wave, smem); break;
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
        if (G.k % 64 != 0)
            return fail(NVFP4_EUNSUPPORTED, "group %d: k=%d is not a multiple of 64", i, G.k);
        if ((uint64_t)(G.m > G.n ? G.m : G.n) * (uint64_t)(G.k / 2) >= (1ull << 32))
            return fail(NVFP4_EUNSUPPORTED, "group %d: an operand exceeds 4 GiB", i);
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
// rows spread evenly (rounded up to 16) so a ragged M wastes little.
inline void row_tiling(int m, int &tiles, int &rows_per_tile)
{
    tiles = ceil_div(m, kTileM);
    rows_per_tile = 16 * ceil_div(ceil_div(m, tiles), 16);
    tiles = ceil_div(m, rows_per_tile);
}

// Visits the tiles of all non-empty groups in dispatch order: group by group,
// column strip by column strip, row tiles of a strip adjacent (they read the
// same B columns).  fn(group, m0, rows, n0) is called once per tile.
template <typename Fn>
long long for_each_tile(const nvfp4_group_t *groups, int ng, Fn fn)
{
    long long t = 0;
    for (int i = 0; i < ng; ++i) {
        const nvfp4_group_t &G = groups[i];
        if (G.m == 0 || G.n == 0)
            continue;
        int rt, tr;
        row_tiling(G.m, rt, tr);
        const int ct = ceil_div(G.n, kTileN);
        for (int nb = 0; nb < ct; ++nb)
            for (int mb = 0; mb < rt; ++mb, ++t)
                fn(i, mb * tr, (G.m - mb * tr < tr) ? G.m - mb * tr : tr, nb * kTileN);
    }
    return t;
}

}  // namespace

extern "C" int nvfp4_validate(const nvfp4_group_t *groups, int ng)
{
    return validate(groups, ng);
}

extern "C" int nvfp4_tile_rows(void) { return kTileM; }
extern "C" int nvfp4_tile_cols(void) { return kTileN; }

extern "C" int nvfp4_plan(const nvfp4_group_t *groups, int ng, int32_t *tiles, int cap)
{
    const int rc = validate(groups, ng);
    if (rc != NVFP4_OK)
        return -rc;
    long long t = 0;
    const long long n = for_each_tile(groups, ng, [&](int g, int m0, int rows, int n0) {
        if (tiles != nullptr && t < cap) {
            tiles[4 * t + 0] = g;
            tiles[4 * t + 1] = m0;
            tiles[4 * t + 2] = rows;
            tiles[4 * t + 3] = n0;
        }
        ++t;
    });
    if (n > 0x7fffffffLL)
        return -fail(NVFP4_EUNSUPPORTED, "too many tiles");
    return (int)n;
}

extern "C" int nvfp4_group_gemm(const nvfp4_group_t *groups, int ng, void *stream)
{
    const int rc = validate(groups, ng);
    if (rc != NVFP4_OK)
        return rc;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    LaunchArgs args;
    int i = 0;
    while (i < ng) {
        memset(&args, 0, sizeof args);
        long long tiles = 0;
        int n = 0;
        for (; i < ng && n < kMaxGroupsPerLaunch; ++i) {
            const nvfp4_group_t &G = groups[i];
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
            A.tile_begin = (int32_t)tiles;
            tiles += (long long)A.row_tiles * ceil_div(G.n, kTileN);
            if (tiles > 0x7fffffffLL)
                return fail(NVFP4_EUNSUPPORTED, "too many tiles in one launch");
        }
        if (n == 0)
            break;
        args.ng = n;
        args.total_tiles = (int32_t)tiles;
        hipLaunchKernelGGL((nvfp4_group_gemm_kernel<kWaves>), dim3((unsigned)tiles),
                           dim3(kThreads), 0, st, args);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return fail(NVFP4_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return NVFP4_OK;
}

extern "C" const char *nvfp4_last_error(void) { return g_err; }
