// Weight-streaming kernels of the DFlash drafter on gfx950:
//  - re-tiling of weight matrices into the wavefront-contiguous layout,
//  - weight-only FP8 E4M3 row quantisation,
//  - the split-K "GEMV" for the 16*B block rows (MFMA, fused epilogues),
//  - the large-M GEMM used by encode and inject.
//
// Arithmetic is fp32 whatever the storage dtype (dflash-ops card, Method):
// bf16 and fp8 weights meet activations split exactly into three bf16 terms,
// so every bf16 x bf16 MFMA product is exact and accumulation is fp32; f32
// weights use the f32 MFMA.
#include "gemv_device.h"

// ---------------------------------------------------------------------------
// Re-tiling
// ---------------------------------------------------------------------------
// row_map 0: source row r goes to tiled row dst_row0 + r.
// row_map 1: gate/up pairing. Row r of a [F, K] matrix goes to tiled row
//            64 * (r / 32) + 32 * pair_half + r % 32, so column group g holds
//            gate rows 32g..32g+31 in its first two tiles and the matching up
//            rows in its last two.
__host__ __device__ inline int tiled_row(int r, int row_map, int dst_row0, int pair_half) {
    if (row_map == 0) return dst_row0 + r;
    return 64 * (r / 32) + 32 * pair_half + (r % 32);
}

__global__ void tile_weights_kernel(const uint8_t *__restrict__ src, int rows, int K, int esize,
                                    uint8_t *__restrict__ dst, int KB, int row_map, int dst_row0, int pair_half,
                                    int tpg) {
    const size_t chunks = (size_t)K / LANE_ELEMS;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)rows * chunks) return;
    const int r = (int)(idx / chunks);
    const int k = (int)(idx % chunks) * LANE_ELEMS;
    const int v = tiled_row(r, row_map, dst_row0, pair_half);
    const u32x4 *s = (const u32x4 *)(src + ((size_t)r * K + k) * esize);
    const int epw = 16 / esize;  // 16 elements = esize 16-byte words, each stored with its wavefront neighbours
    for (int w = 0; w < esize; ++w) *(u32x4 *)(dst + tiled_offset(v, k + w * epw, KB, esize, tpg) * esize) = s[w];
}

hipError_t launch_tile_weights(const void *src, int src_rows, int K, int esize, void *dst, int KB, int row_map,
                               int dst_row0, int pair_half, int tpg, hipStream_t s) {
    size_t n = (size_t)src_rows * (K / LANE_ELEMS);
    dim3 grid((unsigned)((n + 255) / 256));
    hipLaunchKernelGGL(tile_weights_kernel, grid, dim3(256), 0, s, (const uint8_t *)src, src_rows, K, esize,
                       (uint8_t *)dst, KB, row_map, dst_row0, pair_half, tpg);
    return hipGetLastError();
}

__global__ void tile_scales_kernel(const float *src, int rows, float *dst, int row_map, int dst_row0, int pair_half) {
    int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r < rows) dst[tiled_row(r, row_map, dst_row0, pair_half)] = src[r];
}

hipError_t launch_tile_scales(const float *src, int src_rows, float *dst, int row_map, int dst_row0, int pair_half,
                              hipStream_t s) {
    hipLaunchKernelGGL(tile_scales_kernel, dim3((src_rows + 255) / 256), dim3(256), 0, s, src, src_rows, dst, row_map,
                       dst_row0, pair_half);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// FP8 row quantisation (metrale dflash_head.rs page, DflashQuantization)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const float *__restrict__ w, int cols,
                                                           uint8_t *__restrict__ codes, float *__restrict__ scales) {
    const int row = blockIdx.x;
    const float *wr = w + (size_t)row * cols;
    float m = 0.0f;
    for (int c = threadIdx.x; c < cols; c += 256) m = fmaxf(m, fabsf(wr[c]));
    m = wave_max(m);
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float scale = amax == 0.0f ? 1.0f : amax / 448.0f;
    uint8_t *cr = codes + (size_t)row * cols;
    for (int c = threadIdx.x; c < cols; c += 256) cr[c] = f32_to_e4m3(wr[c] / scale);
    if (threadIdx.x == 0) scales[row] = scale;
}

hipError_t launch_quantize_fp8(const float *w, int rows, int cols, uint8_t *codes, float *scales, hipStream_t s) {
    hipLaunchKernelGGL(quantize_fp8_kernel, dim3(rows), dim3(256), 0, s, w, cols, codes, scales);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-K weight-streaming kernel for the block rows
// ---------------------------------------------------------------------------
// Grid (G column groups of 64*WN columns, S k-splits), 256 threads = 4
// wavefronts: WN along the columns (4 tiles each) and 4/WN along the
// reduction. Workgroup (g, s) owns group g and k-blocks [s*kbps, (s+1)*kbps);
// its waves along the reduction take every (4/WN)-th k-block. Each wave keeps
// MT*4 16x16 accumulators (MT 16-row tiles x 4 column tiles), the waves are
// summed in a fixed order through LDS, and when S > 1 the partial tile goes to
// global memory; the last workgroup of the group to arrive sums the S partials
// in split order and runs the epilogue, so results do not depend on scheduling.
template <int WT, int AF, int MT, int EPI, int WN>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
    constexpr int NV = WTraits<WT>::NV;
    constexpr int NW = AFTraits<AF>::NW;
    constexpr int MP = MT * 16;
    constexpr int GN = GROUP_N * WN;  // columns per group
    constexpr int WK = 4 / WN;        // waves along the reduction
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave % WN, wk = wave / WN;
    const int g = blockIdx.x, s = blockIdx.y;
    const int G = a.N / GN, KB = a.K / KBLK;
    const int kb0 = s * a.kb_per_split;
    const int kb1 = min(KB, kb0 + a.kb_per_split);
    const int M = a.epi.M;

    f32x4 acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kb = kb0 + wk; kb < kb1; kb += WK) {
        u32x4 w[4][NV];
#pragma unroll
        for (int t = 0; t < 4; ++t) load_wtile<WT>(a.W, ((size_t)g * KB + kb) * 4 * WN + 4 * wn + t, lane, w[t]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            u32x4 av[NW];
            load_act_lanes<AF>(a.act, a.act_rows, a.K, mt, mt * 16 < M, kb, lane, av);
#pragma unroll
            for (int t = 0; t < 4; ++t) tile_mfma<WT, AF>(w[t], av, acc[mt][t]);
        }
    }

    __shared__ float tile[MP * GN];
    __shared__ float rs_s[MP];
    __shared__ int best_s[MP];
    __shared__ int flag_s;
    reduce_waves<MT, WN>(acc, tile, wn, wk, lane);
    if (a.S > 1) {
        constexpr int TE = MP * GN;
        if (!splitk_last<TE / 256>(tile, a.partial + ((size_t)s * G + g) * TE, a.partial + (size_t)g * TE,
                                   (size_t)G * TE, a.S, &a.counters[g], &flag_s))
            return;
    }
    gemv_epilogue<EPI, MT, WN>(a.epi, g, G, tile, rs_s, &flag_s, best_s);
}

template <int WT, int AF, int EPI, int WN>
static hipError_t launch_gemv_mt(int MT, dim3 grid, const GemvArgs &a, hipStream_t s) {
    switch (MT) {
        case 1: hipLaunchKernelGGL((gemv_kernel<WT, AF, 1, EPI, WN>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((gemv_kernel<WT, AF, 2, EPI, WN>), grid, dim3(256), 0, s, a); break;
        case 4: hipLaunchKernelGGL((gemv_kernel<WT, AF, 4, EPI, WN>), grid, dim3(256), 0, s, a); break;
        case 8: hipLaunchKernelGGL((gemv_kernel<WT, AF, 8, EPI, WN>), grid, dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Every projection streams 64-column groups (WN = 1).
template <int WT, int AF>
static hipError_t launch_gemv_epi(int MT, int WN, dim3 grid, const GemvArgs &a, hipStream_t s) {
    if (WN != 1) return hipErrorInvalidValue;
    switch (a.epi.kind) {
        case EPI_SCALED: return launch_gemv_mt<WT, AF, EPI_SCALED, 1>(MT, grid, a, s);
        case EPI_RESID: return launch_gemv_mt<WT, AF, EPI_RESID, 1>(MT, grid, a, s);
        case EPI_SWIGLU: return launch_gemv_mt<WT, AF, EPI_SWIGLU, 1>(MT, grid, a, s);
        case EPI_LOGITS: return launch_gemv_mt<WT, AF, EPI_LOGITS, 1>(MT, grid, a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv(int wdtype, int act_fmt, int MT, int WN, dim3 grid, const GemvArgs &a, hipStream_t s) {
    if (wdtype == DFLASH_F32 && act_fmt == ACT_F32) return launch_gemv_epi<DFLASH_F32, ACT_F32>(MT, WN, grid, a, s);
    if (wdtype == DFLASH_BF16 && act_fmt == ACT_SPLIT3)
        return launch_gemv_epi<DFLASH_BF16, ACT_SPLIT3>(MT, WN, grid, a, s);
    if (wdtype == DFLASH_FP8_E4M3 && act_fmt == ACT_SPLIT3)
        return launch_gemv_epi<DFLASH_FP8_E4M3, ACT_SPLIT3>(MT, WN, grid, a, s);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Large-M GEMM (encode's fc, inject's fused K/V projection)
// ---------------------------------------------------------------------------
// Grid (N/64 column groups, ceil(M/64) row blocks), 256 threads. Wave w of
// block (g, mb) computes rows mb*64 + 16w .. +16 against the 64 columns of
// group g over the whole reduction; the four waves read the same weight
// tiles, so three of the four reads hit the caches.
template <int WT, int AF>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
    constexpr int NV = WTraits<WT>::NV;
    constexpr int NW = AFTraits<AF>::NW;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = blockIdx.x;
    const int m0 = blockIdx.y * 64 + wave * 16;
    const int KB = a.K / KBLK;
    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (m0 < a.M) {
        for (int kb = 0; kb < KB; ++kb) {
            u32x4 w[4][NV];
#pragma unroll
            for (int t = 0; t < 4; ++t) load_wtile<WT>(a.W, ((size_t)g * KB + kb) * 4 + t, lane, w[t]);
            u32x4 av[NW];
            load_act<AF>(a.act, a.act_rows, a.K, m0 + (lane & 15), a.M, kb, lane, av);
#pragma unroll
            for (int t = 0; t < 4; ++t) tile_mfma<WT, AF>(w[t], av, acc[t]);
        }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + 4 * (lane >> 4) + i;
            const int n = g * GROUP_N + 16 * t + (lane & 15);
            if (m < a.M) {
                float v = acc[t][i];
                if (a.wscale) v *= a.wscale[n];
                a.out[(size_t)m * a.N + n] = v;
            }
        }
}

hipError_t launch_gemm(int wdtype, int act_fmt, const GemmArgs &a, hipStream_t s) {
    dim3 grid(a.N / GROUP_N, (a.M + 63) / 64);
    if (wdtype == DFLASH_F32 && act_fmt == ACT_F32)
        hipLaunchKernelGGL((gemm_kernel<DFLASH_F32, ACT_F32>), grid, dim3(256), 0, s, a);
    else if (wdtype == DFLASH_BF16 && act_fmt == ACT_BF16)
        hipLaunchKernelGGL((gemm_kernel<DFLASH_BF16, ACT_BF16>), grid, dim3(256), 0, s, a);
    else if (wdtype == DFLASH_BF16 && act_fmt == ACT_SPLIT3)
        hipLaunchKernelGGL((gemm_kernel<DFLASH_BF16, ACT_SPLIT3>), grid, dim3(256), 0, s, a);
    else if (wdtype == DFLASH_FP8_E4M3 && act_fmt == ACT_SPLIT3)
        hipLaunchKernelGGL((gemm_kernel<DFLASH_FP8_E4M3, ACT_SPLIT3>), grid, dim3(256), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}
