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
//    in fp16.  Operands are therefore decoded exactly to fp16 in registers
//    (hardware FP4->f16 convert, then one packed f16 multiply by the scale)
//    and fed to v_mfma_f32_16x16x32_f16 with fp32 accumulation.
//  * Loads go straight from HBM into registers in the MFMA operand layout:
//    lane (r, q) of a wave reads 32 contiguous bytes (64 k) of one row.  The
//    contraction order inside a 256-k chunk is permuted identically for A and
//    B, which leaves the sum unchanged.
//  * A workgroup of W waves owns one output tile and splits K between its
//    waves (chunk c goes to wave c mod W); every wave folds each 256-k chunk's
//    MFMA sum into an outer fp32 accumulator, and the W partial sums are added
//    in a fixed order through LDS.  Both steps keep fp32 rounding error far
//    below the fp16 output tolerance for long K.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "nvfp4_group_gemm.h"

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileM = 64;           // rows of one output tile
constexpr int kTileN = 64;           // columns of one output tile
constexpr int kWaves = 4;            // waves per workgroup (split-K)
constexpr int kChunkK = 256;         // k per chunk (8 MFMA steps of 32)
constexpr int kMaxGroupsPerLaunch = 32;

struct GroupArgs {
    const uint8_t *a;
    const uint8_t *b;
    const uint8_t *sfa;
    const uint8_t *sfb;
    _Float16 *c;
    int32_t m, n, k;
    int32_t tiles_m;     // row tiles of this group
    int32_t tile_begin;  // index of this group's first tile in the launch
    int32_t pad;
};

struct LaunchArgs {
    GroupArgs g[kMaxGroupsPerLaunch];
    int32_t ng;
    int32_t total_tiles;
};

// ---------------------------------------------------------------- device --

// Eight E2M1 codes (one dword, element i in nibble i) times one scale, as
// eight exact fp16 values.  The convert instruction takes a power-of-two
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

// Four E4M3FN scale bytes -> fp16 pairs (lo pair: bytes 0,1; hi pair: bytes 2,3).
__device__ __forceinline__ void scales4(uint32_t bytes, f16x2 &lo, f16x2 &hi)
{
    lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bytes, 1.0f, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bytes, 1.0f, true);
}

__device__ __forceinline__ f16x2 bcast(_Float16 x)
{
    f16x2 r = {x, x};
    return r;
}

template <int TM, int TN, int W>
__global__ __launch_bounds__(64 * W, 1) void nvfp4_group_gemm_kernel(const LaunchArgs args)
{
    constexpr int RB = TM / 16;   // 16-row blocks per tile
    constexpr int CB = TN / 16;   // 16-column blocks per tile
    __shared__ float red[W][TM][TN + 4];

    const int tile = blockIdx.x;
    int g = 0;
    for (int i = 1; i < args.ng; ++i)
        if (args.g[i].tile_begin <= tile)
            g = i;
    const GroupArgs &G = args.g[g];
    const int M = G.m, N = G.n, K = G.k;
    const int local = tile - G.tile_begin;
    const int m0 = (local % G.tiles_m) * TM;
    const int n0 = (local / G.tiles_m) * TN;
    const int rows = min(TM, M - m0);
    const int nrb = (rows + 15) >> 4;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, q = lane >> 4;
    const size_t row_bytes = (size_t)K >> 1, row_scales = (size_t)K >> 4;

    // Row pointers of this lane (rows past the edge are clamped: their
    // results are computed but never stored).
    const uint8_t *pa[RB], *psa[RB], *pb[CB], *psb[CB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
        const size_t row = (size_t)min(m0 + 16 * i + r, M - 1);
        pa[i] = G.a + row * row_bytes + 32 * q;
        psa[i] = G.sfa + row * row_scales + 4 * q;
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
        const size_t col = (size_t)min(n0 + 16 * j + r, N - 1);
        pb[j] = G.b + col * row_bytes + 32 * q;
        psb[j] = G.sfb + col * row_scales + 4 * q;
    }

    f32x4 acc[RB][CB];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nchunks = (K + kChunkK - 1) / kChunkK;
    for (int c = wave; c < nchunks; c += W) {
        const int k0 = c * kChunkK;
        // this lane's 64-k segment [k0 + 64q, k0 + 64q + 64) exists (K % 64 == 0)
        const bool seg = (k0 + 64 * q) < K;
        const size_t boff = (size_t)(k0 >> 1), soff = (size_t)(k0 >> 4);
        u32x4 ra[RB][2], rb[CB][2];
        uint32_t sa[RB], sb[CB];
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            if (i < nrb) {
                if (seg) {
                    ra[i][0] = *reinterpret_cast<const u32x4 *>(pa[i] + boff);
                    ra[i][1] = *reinterpret_cast<const u32x4 *>(pa[i] + boff + 16);
                    sa[i] = *reinterpret_cast<const uint32_t *>(psa[i] + soff);
                } else {
                    ra[i][0] = ra[i][1] = u32x4{0u, 0u, 0u, 0u};
                    sa[i] = 0u;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            if (seg) {
                rb[j][0] = *reinterpret_cast<const u32x4 *>(pb[j] + boff);
                rb[j][1] = *reinterpret_cast<const u32x4 *>(pb[j] + boff + 16);
                sb[j] = *reinterpret_cast<const uint32_t *>(psb[j] + soff);
            } else {
                rb[j][0] = rb[j][1] = u32x4{0u, 0u, 0u, 0u};
                sb[j] = 0u;
            }
        }
        f16x2 sal[RB], sah[RB], sbl[CB], sbh[CB];
#pragma unroll
        for (int i = 0; i < RB; ++i)
            if (i < nrb)
                scales4(sa[i], sal[i], sah[i]);
#pragma unroll
        for (int j = 0; j < CB; ++j)
            scales4(sb[j], sbl[j], sbh[j]);

        f32x4 part[RB][CB];
#pragma unroll
        for (int s = 0; s < 8; ++s) {          // MFMA step: k0 + 64q + 8s + [0, 8)
            f16x8 af[RB], bf[CB];
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                if (i < nrb) {
                    const f16x2 sc = (s < 4) ? sal[i] : sah[i];
                    af[i] = decode8(ra[i][s >> 2][s & 3], bcast(sc[(s >> 1) & 1]));
                }
            }
#pragma unroll
            for (int j = 0; j < CB; ++j) {
                const f16x2 sc = (s < 4) ? sbl[j] : sbh[j];
                bf[j] = decode8(rb[j][s >> 2][s & 3], bcast(sc[(s >> 1) & 1]));
            }
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                if (i < nrb) {
#pragma unroll
                    for (int j = 0; j < CB; ++j)
                        part[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            af[i], bf[j], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : part[i][j], 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < RB; ++i)
            if (i < nrb)
#pragma unroll
                for (int j = 0; j < CB; ++j)
                    acc[i][j] += part[i][j];
    }

    // Output element (16i + 4q + e, 16j + r) of this wave's partial sum.
#pragma unroll
    for (int i = 0; i < RB; ++i)
        if (i < nrb)
#pragma unroll
            for (int j = 0; j < CB; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    red[wave][16 * i + 4 * q + e][16 * j + r] = acc[i][j][e];
    __syncthreads();

    const int cols = min(TN, N - n0);
    _Float16 *C = G.c;
    for (int idx = threadIdx.x; idx < TM * TN; idx += 64 * W) {
        const int row = idx / TN, col = idx % TN;
        if (row < rows && col < cols) {
            float s = red[0][row][col];
#pragma unroll
            for (int w = 1; w < W; ++w)
                s += red[w][row][col];
            C[(size_t)(m0 + row) * N + n0 + col] = (_Float16)s;
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
        if (G.k % 64 != 0)
            return fail(NVFP4_EUNSUPPORTED, "group %d: k=%d is not a multiple of 64", i, G.k);
        if (((uintptr_t)G.c & 3u) != 0)
            return fail(NVFP4_EUNSUPPORTED, "group %d: c is not 4-byte aligned", i);
        if (G.k > 0 && ((((uintptr_t)G.a | (uintptr_t)G.b) & 15u) != 0 ||
                        (((uintptr_t)G.sfa | (uintptr_t)G.sfb) & 3u) != 0))
            return fail(NVFP4_EUNSUPPORTED, "group %d: operand pointer misaligned", i);
    }
    return NVFP4_OK;
}

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Visits the tiles of all non-empty groups in dispatch order: group by group,
// row tiles fastest.  fn(group, m0, rows, n0) is called once per tile.
template <typename Fn>
long long for_each_tile(const nvfp4_group_t *groups, int ng, Fn fn)
{
    long long t = 0;
    for (int i = 0; i < ng; ++i) {
        const nvfp4_group_t &G = groups[i];
        if (G.m == 0 || G.n == 0)
            continue;
        const int tm = ceil_div(G.m, kTileM), tn = ceil_div(G.n, kTileN);
        for (int nb = 0; nb < tn; ++nb)
            for (int mb = 0; mb < tm; ++mb, ++t)
                fn(i, mb * kTileM, (G.m - mb * kTileM < kTileM) ? G.m - mb * kTileM : kTileM, nb * kTileN);
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
    long long n = for_each_tile(groups, ng, [&](int g, int m0, int rows, int n0) {});
    long long t = 0;
    for_each_tile(groups, ng, [&](int g, int m0, int rows, int n0) {
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
            A.tiles_m = ceil_div(G.m, kTileM);
            A.tile_begin = (int32_t)tiles;
            tiles += (long long)A.tiles_m * ceil_div(G.n, kTileN);
            if (tiles > 0x7fffffffLL)
                return fail(NVFP4_EUNSUPPORTED, "too many tiles in one launch");
        }
        if (n == 0)
            break;
        args.ng = n;
        args.total_tiles = (int32_t)tiles;
        hipLaunchKernelGGL((nvfp4_group_gemm_kernel<kTileM, kTileN, kWaves>), dim3((unsigned)tiles),
                           dim3(64 * kWaves), 0, st, args);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return fail(NVFP4_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return NVFP4_OK;
}

extern "C" const char *nvfp4_last_error(void) { return g_err; }
