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
//
// NWV = 16 (one 16-row tile, WN = 1) widens the workgroup to 16 wavefronts
// along the reduction, so that a group needs fewer k-splits (often none): the
// waves are summed through LDS in a fixed order, then the first four waves
// carry on as above. With it, CW = 32 narrows a workgroup to half a column
// group (two of its four tiles), which doubles the workgroups without a k-split.
// Occupancy: a four-wave one-tile workgroup with bf16 or fp8 weights must fit
// five per compute unit (five waves per SIMD), so that the gate/up grid of
// about five workgroups per compute unit is resident at once (real-dims bf16
// gate/up: 93.8 us at four per SIMD, 88.8 us at five); f32 weight tiles need
// the registers (five per SIMD spills). A 16-wave workgroup needs four per SIMD.
template <int WT, int AF, int MT, int EPI, int WN, int NWV = 4, int CW = GROUP_N>
__global__ __launch_bounds__(64 * NWV, NWV == 16 ? 4 : (MT == 1 && WT != DFLASH_F32 ? 5 : 1)) void gemv_kernel(GemvArgs a) {
    static_assert(NWV == 4 || (NWV == 16 && MT == 1 && WN == 1), "wide workgroups take one tile group");
    static_assert(CW == GROUP_N || (CW == 32 && NWV == 16 && EPI != EPI_SWIGLU), "half groups: 16 waves, no SwiGLU");
    constexpr int NV = WTraits<WT>::NV;
    constexpr int AFO = ActOp<WT, AF>::AFO;  // MFMA operand format
    constexpr int NW = AFTraits<AFO>::NW;
    constexpr int MP = MT * 16;
    constexpr int TPW = CW / 16;     // 16-column tiles per workgroup and wave column
    constexpr int GN = CW * WN;      // columns per group
    constexpr int WK = NWV / WN;     // waves along the reduction
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave % WN, wk = wave / WN;
    const int g = blockIdx.x, s = blockIdx.y;
    const int G = a.N / GN, KB = a.K / KBLK;
    // stored 64-column group and first tile of this workgroup's columns
    const int gs = g * CW / GROUP_N, t0 = (g * CW % GROUP_N) / 16;
    const int kb0 = s * a.kb_per_split;
    const int kb1 = min(KB, kb0 + a.kb_per_split);
    const int M = a.epi.M;

    // A 16-wave workgroup runs one per compute unit, so registers are not what
    // limits its occupancy: the four waves that may run the epilogue load its
    // operands (norm sums, residual row, column scales) before the weight
    // stream, taking their latency off the kernel's tail.
    constexpr bool PF = NWV == 16 && CW == GROUP_N;
    EpiPre pre{};
    if constexpr (PF)
        if (tid < 256) epi_prefetch<EPI, 1>(a.epi, g, pre);

    f32x4 acc[MT][TPW];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < TPW; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kb = kb0 + wk; kb < kb1; kb += WK) {
        u32x4 w[TPW][NV];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
            load_wtile<WT>(a.W, ((size_t)gs * KB + kb) * 4 * WN + 4 * wn + t0 + t, lane, w[t]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            u32x4 av[NW];
            load_act_operands<WT, AF>(a.act, a.act_rows, a.K, mt, mt * 16 < M, kb, lane, av);
#pragma unroll
            for (int t = 0; t < TPW; ++t) tile_mfma<WT, AFO>(w[t], av, acc[mt][t]);
        }
    }

    __shared__ float tile[MP * GN];
    __shared__ float rs_s[MP];
    __shared__ int best_s[MP];
    __shared__ int flag_s;
    if constexpr (NWV == 16) {
        // waves 0-7 store, waves 8-15 add into wave w-8's slot, then thread t
        // sums element t over the eight slots in slot order
        __shared__ float red[8][16 * CW];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if ((wk >> 3) == half) {
#pragma unroll
                for (int t = 0; t < TPW; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = 4 * (lane >> 4) + i, col = 16 * t + (lane & 15);
                        float *r = &red[wk & 7][m * CW + col];
                        if (half == 0)
                            *r = acc[0][t][i];
                        else
                            *r += acc[0][t][i];
                    }
            }
            __syncthreads();
        }
        if (tid < 16 * CW) {
            float v = red[0][tid];
#pragma unroll
            for (int i = 1; i < 8; ++i) v += red[i][tid];
            tile[tid] = v;
        }
        __syncthreads();
        if (tid >= 256) return;  // the split-K handshake and the epilogue run on four waves
    } else {
        reduce_waves<MT, WN>(acc, tile, wn, wk, lane);
    }
    if (a.S > 1) {
        constexpr int TE = MP * GN;
        if constexpr (NWV == 16 && EPI == EPI_SCALED && CW == GROUP_N) {
            if (a.S == 2 && a.xslot) {  // per-element epilogue: the splits meet through exchange slots
                scaled_exchange<PF>(a.epi, g, tile, rs_s, a.xslot + (size_t)g * TE, pre);
                return;
            }
        }
        if constexpr (NWV == 16 && EPI == EPI_LOGITS && CW == GROUP_N) {
            if (a.S == 2 && a.xslot) {
                logits_exchange<PF>(a.epi, g, G, s, tile, rs_s, a.xslot + (size_t)g * TE, pre, &flag_s, best_s);
                return;
            }
        }
        // Many four-wave workgroups: only the earlier arrivals store their partial
        // (gate/up at the real dimensions: 96.5 -> 94.9 us). One workgroup per
        // compute unit: the splits of a group finish together, so the last one
        // would wait on the other's stores; every split stores its partial first.
        if constexpr (NWV == 4) {
            if (!splitk_hand_off<TE / 256>(tile, a.partial + ((size_t)s * G + g) * TE, a.partial + (size_t)g * TE,
                                           (size_t)G * TE, a.S, s, &a.counters[g], &a.written[g], a.err, &flag_s))
                return;
        } else {
            if (!splitk_last<TE / 256>(tile, a.partial + ((size_t)s * G + g) * TE, a.partial + (size_t)g * TE,
                                       (size_t)G * TE, a.S, &a.counters[g], &flag_s))
                return;
        }
    }
    gemv_epilogue<EPI, MT, WN, PF, CW>(a.epi, g, G, tile, rs_s, &flag_s, best_s, pre);
}

template <int WT, int AF, int EPI, int WN>
static hipError_t launch_gemv_mt(int MT, int NWV, int CW, dim3 grid, const GemvArgs &a, hipStream_t s) {
    if (NWV == 16) {
        if (MT != 1 || WN != 1) return hipErrorInvalidValue;
        if (CW == 32) {
            if constexpr (EPI == EPI_SWIGLU) return hipErrorInvalidValue;
            else hipLaunchKernelGGL((gemv_kernel<WT, AF, 1, EPI, 1, 16, 32>), grid, dim3(1024), 0, s, a);
        } else {
            hipLaunchKernelGGL((gemv_kernel<WT, AF, 1, EPI, 1, 16>), grid, dim3(1024), 0, s, a);
        }
        return hipGetLastError();
    }
    if (CW != GROUP_N) return hipErrorInvalidValue;
    if (NWV != 4) return hipErrorInvalidValue;
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
static hipError_t launch_gemv_epi(int MT, int WN, int NWV, int CW, dim3 grid, const GemvArgs &a, hipStream_t s) {
    if (WN != 1) return hipErrorInvalidValue;
    switch (a.epi.kind) {
        case EPI_SCALED: return launch_gemv_mt<WT, AF, EPI_SCALED, 1>(MT, NWV, CW, grid, a, s);
        case EPI_RESID: return launch_gemv_mt<WT, AF, EPI_RESID, 1>(MT, NWV, CW, grid, a, s);
        case EPI_SWIGLU: return launch_gemv_mt<WT, AF, EPI_SWIGLU, 1>(MT, NWV, CW, grid, a, s);
        case EPI_LOGITS: return launch_gemv_mt<WT, AF, EPI_LOGITS, 1>(MT, NWV, CW, grid, a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv(int wdtype, int act_fmt, int MT, int WN, int NWV, int CW, dim3 grid, const GemvArgs &a,
                       hipStream_t s) {
    if (wdtype == DFLASH_F32 && act_fmt == ACT_F32)
        return launch_gemv_epi<DFLASH_F32, ACT_F32>(MT, WN, NWV, CW, grid, a, s);
    if (wdtype == DFLASH_BF16 && act_fmt == ACT_SPLIT3)
        return launch_gemv_epi<DFLASH_BF16, ACT_SPLIT3>(MT, WN, NWV, CW, grid, a, s);
    if (wdtype == DFLASH_FP8_E4M3 && act_fmt == ACT_SPLIT3)
        return launch_gemv_epi<DFLASH_FP8_E4M3, ACT_SPLIT3>(MT, WN, NWV, CW, grid, a, s);
    if (wdtype == DFLASH_BF16 && act_fmt == ACT_F32)  // split at load
        return launch_gemv_epi<DFLASH_BF16, ACT_F32>(MT, WN, NWV, CW, grid, a, s);
    if (wdtype == DFLASH_FP8_E4M3 && act_fmt == ACT_F32)
        return launch_gemv_epi<DFLASH_FP8_E4M3, ACT_F32>(MT, WN, NWV, CW, grid, a, s);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Large-M GEMM (encode's fc, inject's fused K/V projection, the batched block
// rows): out[M][N] = act[M][K] . W[N][K]^T (* per-column scale), f32 out,
// activations row-major or in the block rows' lane order (one bf16 plane,
// three bf16 planes of an exact split, or f32).
// ---------------------------------------------------------------------------
// Workgroup tile 128 rows x 256 columns (four column groups) x one k-split,
// 8 wavefronts of 64 rows x 64 columns each; split s writes its partial
// product to out + s*M*N and the consumer sums the splits in order. Per
// k-block the workgroup stages the activation rows and the four groups'
// weight tiles in LDS once (activation rows padded against bank conflicts;
// weight tiles copied in their lane order) and every wave reads its operands
// from there. Where two stages fit the 160 KB of LDS, k-block kb + 1 moves
// from registers to the free stage and the loads of kb + 2 are issued while kb
// is multiplied (one barrier per k-block); otherwise the next k-block waits in
// registers. Column groups past N are masked. With rs_out set, one extra
// workgroup (the first) computes the row scales of the epilogue that follows.
template <int AF>
struct GemmA;
template <>
struct GemmA<ACT_BF16> {
    static constexpr int TERMS = 1, ES = 2, ROWB = 144;  // 64 bf16 + 8 pad per row
};
template <>
struct GemmA<ACT_SPLIT3> {
    static constexpr int TERMS = 3, ES = 2, ROWB = 144;
};
template <>
struct GemmA<ACT_F32> {
    static constexpr int TERMS = 1, ES = 4, ROWB = 272;  // 64 f32 + 4 pad per row
};

constexpr int GEMM_BM = 128, GEMM_GROUPS = 4, GEMM_THREADS = 512;

// ALANES: the activations are in the block rows' lane-ordered layout (act_offset;
// planes of act_rows rows) instead of row-major; a 16-row k-block tile of a plane
// is then one contiguous run of 64-lane words, staged to LDS in the same order.
template <int WT, int AF, bool ALANES>
struct GemmShape {
    static constexpr int NV = WTraits<WT>::NV;
    static constexpr int TERMS = GemmA<AF>::TERMS, ES = GemmA<AF>::ES, ROWB = GemmA<AF>::ROWB;
    static constexpr int WPR = 64 * ES / 16;                     // 16-byte words per row of a k-block
    static constexpr int A_WORDS = TERMS * GEMM_BM * WPR;        // per k-block
    static constexpr int A_PT = A_WORDS / GEMM_THREADS;          // per thread
    static constexpr int B_GROUP = 4 * NV * 64;                  // words of one group's k-block
    static constexpr int B_WORDS = GEMM_GROUPS * B_GROUP;
    static constexpr int B_PT = B_WORDS / GEMM_THREADS;
    static constexpr int A_LDS = ALANES ? A_WORDS * 16 : TERMS * GEMM_BM * ROWB;
    static constexpr int STAGE = A_LDS + B_WORDS * 16;
    // two LDS stages where they fit the compute unit's 160 KB
    static constexpr bool DB = 2 * STAGE <= 160 * 1024;
    static constexpr int LDS = DB ? 2 * STAGE : STAGE;
    static constexpr int LW = ES == 2 ? 2 : 4;                   // lane-ordered words per lane per tile
};

template <int WT, int AF, bool ALANES>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_kernel(GemmArgs a) {
    using Sh = GemmShape<WT, AF, ALANES>;
    constexpr int NV = Sh::NV, NW = AFTraits<AF>::NW, TERMS = Sh::TERMS, ES = Sh::ES, ROWB = Sh::ROWB;
    constexpr int BM = GEMM_BM, WPR = Sh::WPR, A_PT = Sh::A_PT, B_GROUP = Sh::B_GROUP, B_PT = Sh::B_PT;
    constexpr int LW = Sh::LW;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    char *A_s = lds;
    u32x4 *B_s = (u32x4 *)(lds + Sh::A_LDS);
    auto use_stage = [&](int buf) {
        A_s = lds + buf * Sh::STAGE;
        B_s = (u32x4 *)(lds + buf * Sh::STAGE + Sh::A_LDS);
    };

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (a.rs_out != nullptr && blockIdx.x == 0) {
        // the first workgroup: row scales for the epilogue that follows (16
        // threads per row, groups summed in the order the epilogue would), the
        // loads of up to 128 rows (four rows per thread) issued together
        constexpr int RPT = 4, GPT = 16;  // rows per thread, groups per thread and row (rs_groups <= 256)
        const int sub = tid & 15;
        float v[RPT][GPT];
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int m = r * (GEMM_THREADS / 16) + (tid >> 4);
#pragma unroll
            for (int j = 0; j < GPT; ++j) {
                const int gg = sub + 16 * j;
                v[r][j] = (m < a.M && gg < a.rs_groups) ? a.rs_ss[(size_t)m * a.rs_gs + gg] : 0.0f;
            }
        }
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int m = r * (GEMM_THREADS / 16) + (tid >> 4);
            float part = 0.0f;
#pragma unroll
            for (int j = 0; j < GPT; ++j)
                if (sub + 16 * j < a.rs_groups) part += v[r][j];
            for (int o = 8; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
            if (sub == 0 && m < a.M) a.rs_out[m] = 1.0f / sqrtf(part * a.rs_inv_E + a.rs_eps);
        }
        return;
    }
    const int bid = blockIdx.x - (a.rs_out != nullptr);  // the main workgroups' index
    const int wr = wave >> 2, wc = wave & 3;  // rows 64wr.., column group g0 + wc
    const int G = a.N / GROUP_N;
    // One-dimensional grid in an L2-friendly order: the row tiles that share a (column tile, k-split) are
    // consecutive in launch order and eight apart in it, so that the round-robin placement of workgroups
    // on the eight XCDs puts them on one XCD at about the same time, and its L2 serves their common weight
    // tiles once: L = (q * Y + y) * 8 + c with column-tile-and-split index xz = 8 q + c.
    const int X = (G + GEMM_GROUPS - 1) / GEMM_GROUPS, Y = (a.M + BM - 1) / BM;
    const int Lc = bid % 8, Lr = bid / 8;
    const int xz = (Lr / Y) * 8 + Lc;
    if (xz >= X * a.S) return;
    const int g0 = (xz % X) * GEMM_GROUPS, r0 = (Lr % Y) * BM, sp = xz / X;
    const int KB = a.K / KBLK;
    const int kb0 = sp * a.kbps, kb1 = min(KB, kb0 + a.kbps);
    float *out = a.out + (size_t)sp * a.M * a.N;
    const bool wave_live = g0 + wc < G;

    u32x4 sa[A_PT], sb[B_PT];
    auto load_stage = [&](int kb) {
#pragma unroll
        for (int i = 0; i < A_PT; ++i) {
            const int w = tid + GEMM_THREADS * i;
            if constexpr (ALANES) {
                // w = ((t * 8 + mt) * LW + v) * 64 + lane_word
                const int t = w / (8 * LW * 64), mt = (w / (LW * 64)) % 8, rest = w % (LW * 64);
                const int mtg = r0 / 16 + mt;
                if (mtg * 16 < a.M)
                    sa[i] = *((const u32x4 *)a.act + (size_t)t * a.act_rows * a.K / (16 / ES) +
                              ((size_t)mtg * KB + kb) * LW * 64 + rest);
                else
                    sa[i] = u32x4{0u, 0u, 0u, 0u};
            } else {
                const int t = w / (BM * WPR), rem = w % (BM * WPR), row = rem / WPR, cw = rem % WPR;
                const int m = r0 + row;
                if (m < a.M)
                    sa[i] = *(const u32x4 *)((const char *)a.act +
                                             (((size_t)t * a.act_rows + m) * a.K + (size_t)kb * KBLK) * ES +
                                             (size_t)cw * 16);
                else
                    sa[i] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int i = 0; i < B_PT; ++i) {
            const int w = tid + GEMM_THREADS * i;
            const int gi = w / B_GROUP, rest = w % B_GROUP;
            if (g0 + gi < G)
                sb[i] = ((const u32x4 *)a.W)[((size_t)(g0 + gi) * KB + kb) * B_GROUP + rest];
            else
                sb[i] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_stage = [&]() {
#pragma unroll
        for (int i = 0; i < A_PT; ++i) {
            const int w = tid + GEMM_THREADS * i;
            if constexpr (ALANES) {
                ((u32x4 *)A_s)[w] = sa[i];
            } else {
                const int t = w / (BM * WPR), rem = w % (BM * WPR), row = rem / WPR, cw = rem % WPR;
                *(u32x4 *)(A_s + (t * BM + row) * ROWB + cw * 16) = sa[i];
            }
        }
#pragma unroll
        for (int i = 0; i < B_PT; ++i) B_s[tid + GEMM_THREADS * i] = sb[i];
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto mult_stage = [&]() {
        if (wave_live) {
            u32x4 w[4][NV];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int v = 0; v < NV; ++v) w[t][v] = B_s[wc * B_GROUP + (t * NV + v) * 64 + lane];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int mt = wr * 4 + rt;
                u32x4 av[NW];
                if constexpr (ALANES) {
#pragma unroll
                    for (int t = 0; t < TERMS; ++t)
#pragma unroll
                        for (int v = 0; v < LW; ++v)
                            av[t * LW + v] = ((const u32x4 *)A_s)[((t * 8 + mt) * LW + v) * 64 + lane];
                } else if constexpr (AF == ACT_F32) {
                    const int row = mt * 16 + (lane & 15);
#pragma unroll
                    for (int v = 0; v < 4; ++v) av[v] = *(const u32x4 *)(A_s + row * ROWB + (lane >> 4) * 64 + v * 16);
                } else {
                    const int row = mt * 16 + (lane & 15);
#pragma unroll
                    for (int t = 0; t < TERMS; ++t)
#pragma unroll
                        for (int h = 0; h < 2; ++h)
                            av[2 * t + h] = *(const u32x4 *)(A_s + (t * BM + row) * ROWB + (lane >> 4) * 32 + h * 16);
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) tile_mfma<WT, AF>(w[t], av, acc[rt][t]);
            }
        }
    };
    if constexpr (Sh::DB) {
        // LDS stage (kb - kb0) % 2 holds kb while k-block kb + 1 goes from the
        // registers to the other stage and the loads of kb + 2 are in flight:
        // the HBM latency of a k-block is hidden behind a whole k-block of MFMAs
        load_stage(kb0);
        use_stage(0);
        store_stage();
        if (kb0 + 1 < kb1) load_stage(kb0 + 1);
        __syncthreads();
        for (int kb = kb0; kb < kb1; ++kb) {
            const int c = (kb - kb0) & 1;
            if (kb + 1 < kb1) {
                use_stage(c ^ 1);
                store_stage();  // the other stage was last read before the previous barrier
            }
            if (kb + 2 < kb1) load_stage(kb + 2);
            use_stage(c);
            mult_stage();
            __syncthreads();
        }
    } else {
        load_stage(kb0);
        store_stage();
        __syncthreads();
        for (int kb = kb0; kb < kb1; ++kb) {
            if (kb + 1 < kb1) load_stage(kb + 1);
            mult_stage();
            __syncthreads();
            if (kb + 1 < kb1) {
                store_stage();
                __syncthreads();
            }
        }
    }
    if (!wave_live) return;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = r0 + wr * 64 + rt * 16 + 4 * (lane >> 4) + i;
                const int n = (g0 + wc) * GROUP_N + 16 * t + (lane & 15);
                if (m < a.M) {
                    float v = acc[rt][t][i];
                    if (a.wscale) v *= a.wscale[n];
                    out[(size_t)m * a.N + n] = v;
                }
            }
}

int gemm_workgroups(const GemmArgs &a) {
    const int X = (a.N / GROUP_N + GEMM_GROUPS - 1) / GEMM_GROUPS, Y = (a.M + GEMM_BM - 1) / GEMM_BM;
    return (X * a.S + 7) / 8 * 8 * Y;  // see the kernel's decoding of blockIdx.x
}

template <int WT, int AF, bool ALANES>
static hipError_t gemm_go(const GemmArgs &a, hipStream_t s) {
    using Sh = GemmShape<WT, AF, ALANES>;
    if (a.rs_out != nullptr && (a.M > 128 || a.rs_groups > 256)) return hipErrorInvalidValue;
    const int n = gemm_workgroups(a) + (a.rs_out != nullptr);
    hipLaunchKernelGGL((gemm_kernel<WT, AF, ALANES>), dim3(n), dim3(GEMM_THREADS), Sh::LDS, s, a);
    return hipGetLastError();
}

template <int WT, int AF, bool ALANES>
static hipError_t gemm_attr() {
    return hipFuncSetAttribute((const void *)gemm_kernel<WT, AF, ALANES>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               GemmShape<WT, AF, ALANES>::LDS);
}

hipError_t gemm_set_smem_limit() {
    hipError_t e;
    if ((e = gemm_attr<DFLASH_F32, ACT_F32, false>()) != hipSuccess) return e;
    if ((e = gemm_attr<DFLASH_F32, ACT_F32, true>()) != hipSuccess) return e;
    if ((e = gemm_attr<DFLASH_BF16, ACT_BF16, false>()) != hipSuccess) return e;
    if ((e = gemm_attr<DFLASH_BF16, ACT_SPLIT3, false>()) != hipSuccess) return e;
    if ((e = gemm_attr<DFLASH_BF16, ACT_SPLIT3, true>()) != hipSuccess) return e;
    if ((e = gemm_attr<DFLASH_FP8_E4M3, ACT_SPLIT3, false>()) != hipSuccess) return e;
    return gemm_attr<DFLASH_FP8_E4M3, ACT_SPLIT3, true>();
}

hipError_t launch_gemm(int wdtype, int act_fmt, const GemmArgs &a, hipStream_t s, bool lanes) {
    if (a.S < 1 || a.kbps < 1 || (a.S - 1) * a.kbps >= a.K / KBLK) return hipErrorInvalidValue;
    if (wdtype == DFLASH_F32 && act_fmt == ACT_F32)
        return lanes ? gemm_go<DFLASH_F32, ACT_F32, true>(a, s) : gemm_go<DFLASH_F32, ACT_F32, false>(a, s);
    if (wdtype == DFLASH_BF16 && act_fmt == ACT_BF16 && !lanes) return gemm_go<DFLASH_BF16, ACT_BF16, false>(a, s);
    if (wdtype == DFLASH_BF16 && act_fmt == ACT_SPLIT3)
        return lanes ? gemm_go<DFLASH_BF16, ACT_SPLIT3, true>(a, s) : gemm_go<DFLASH_BF16, ACT_SPLIT3, false>(a, s);
    if (wdtype == DFLASH_FP8_E4M3 && act_fmt == ACT_SPLIT3)
        return lanes ? gemm_go<DFLASH_FP8_E4M3, ACT_SPLIT3, true>(a, s)
                     : gemm_go<DFLASH_FP8_E4M3, ACT_SPLIT3, false>(a, s);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Epilogue of a batched projection computed by gemm_kernel. Workgroup
// (g, y) owns column group g and rows [16*MT*y, 16*MT*(y+1)): it sums the S
// k-split partials [S][M][N] of that tile in split order (loads of eight
// splits in flight at a time) into LDS and runs the fused epilogue of the
// block-row kernels on it, with the row-indexed pointers moved to its first
// row. The logits epilogue also runs per 16-row tile, which is one sequence
// (block width 16): its argmax keys go to the rows of the whole step, and the
// last of the G workgroups of a tile reduces that tile's rows, writes its
// drafts and runs its acceptance scan, each tile on its own arrival counter
// (M <= 128, the counters held for eight sequences). One workgroup per group
// over all 128 rows measured 62 us per step at batch 8; one last stage over
// all rows, after every tile had arrived, 34 us against 25 us per tile.
// ---------------------------------------------------------------------------
template <int EPI, int MT>
__global__ __launch_bounds__(256) void batch_epi_kernel(const float *part, int S, int M, int N, EpiArgs e,
                                                        const float *rs) {
    constexpr int MP = 16 * MT, PT = MP * GROUP_N / 4 / 256;  // float4 per thread per split
    constexpr int UNR = MT >= 8 ? 2 : 8;                               // splits in flight
    __shared__ __attribute__((aligned(16))) float tile[MP * GROUP_N];
    __shared__ float rs_s[MP];
    __shared__ int best_s[MP];
    __shared__ int flag_s;
    const int g = blockIdx.x, G = N / GROUP_N, row0 = blockIdx.y * MP, tid = threadIdx.x;
    const int rows = min(MP, M - row0);
    EpiArgs el = e;
    el.M = rows;
    if constexpr (EPI == EPI_LOGITS) {
        // argmax keys, noise and drafts index the step's rows; a 16-row tile is one sequence, and the last
        // of its G workgroups finishes its argmax and acceptance (one arrival counter per tile)
        el.row0 = row0;
        el.rows_all = 0;
        el.arrivals = G;
        el.am_counter = e.am_counter + blockIdx.y;
    }
    if (row0 > 0) {
        const size_t es = e.act_fmt == ACT_F32 ? 4 : 2;
        if (el.ss) el.ss += (size_t)row0 * e.ss_gs;
        if (el.out) el.out += (size_t)row0 * e.ld_out;
        if (el.x) el.x += (size_t)row0 * e.ld_x;
        if (el.x_out) el.x_out += (size_t)row0 * e.ld_x;
        if (el.ss_out) el.ss_out += (size_t)row0 * e.ss_gs;
        if (el.act_out) el.act_out = (char *)el.act_out + (size_t)row0 * e.act_K * es;
    }
    // row scales computed once for the launch (by the GEMM before it; scaled and
    // SwiGLU epilogues): no sums of squares to load
    constexpr bool RS_KIND = EPI == EPI_SCALED || EPI == EPI_SWIGLU;
    const bool rs_given = RS_KIND && rs != nullptr;
    EpiPre pre;
    if (rs_given) {
        EpiArgs ep = el;
        ep.ss = nullptr;
        epi_prefetch<EPI, MT>(ep, g, pre);
        if (tid < MP) rs_s[tid] = tid < rows ? rs[row0 + tid] : 1.0f;
    } else {
        epi_prefetch<EPI, MT>(el, g, pre);
    }
    f32x4 acc[PT];
#pragma unroll
    for (int j = 0; j < PT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float *base = part + (size_t)row0 * N + (size_t)g * GROUP_N;
    for (int s0 = 0; s0 < S; s0 += UNR) {
        f32x4 v[UNR][PT];
#pragma unroll
        for (int u = 0; u < UNR; ++u)
#pragma unroll
            for (int j = 0; j < PT; ++j) {
                const int idx = tid + 256 * j, m = idx / (GROUP_N / 4), c4 = idx % (GROUP_N / 4);
                v[u][j] = (s0 + u < S && m < rows)
                              ? *(const f32x4 *)(base + ((size_t)(s0 + u) * M + m) * N + c4 * 4)
                              : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int u = 0; u < UNR; ++u)
#pragma unroll
            for (int j = 0; j < PT; ++j)
                if (s0 + u < S) acc[j] += v[u][j];
    }
#pragma unroll
    for (int j = 0; j < PT; ++j) *(f32x4 *)(tile + 4 * (tid + 256 * j)) = acc[j];
    __syncthreads();
    if constexpr (RS_KIND) {
        if (rs_given) {  // rs_s was filled before the barrier above
            gemv_epilogue<EPI, MT, 1, MT == 1, GROUP_N, true>(el, g, G, tile, rs_s, &flag_s, best_s, pre);
            return;
        }
    }
    gemv_epilogue<EPI, MT, 1, MT == 1, GROUP_N, false, EPI == EPI_LOGITS>(el, g, G, tile, rs_s, &flag_s, best_s, pre);
}

hipError_t launch_batch_epi(const float *part, int S, int M, int N, const EpiArgs &e, const float *rs, hipStream_t s) {
    if (M < 1 || M % 16 != 0 || S < 1) return hipErrorInvalidValue;
    const dim3 rows_grid(N / GROUP_N, M / 16);
    switch (e.kind) {
        case EPI_SCALED:
            hipLaunchKernelGGL((batch_epi_kernel<EPI_SCALED, 1>), rows_grid, dim3(256), 0, s, part, S, M, N, e, rs);
            break;
        case EPI_RESID:
            hipLaunchKernelGGL((batch_epi_kernel<EPI_RESID, 1>), rows_grid, dim3(256), 0, s, part, S, M, N, e, rs);
            break;
        case EPI_SWIGLU:
            hipLaunchKernelGGL((batch_epi_kernel<EPI_SWIGLU, 1>), rows_grid, dim3(256), 0, s, part, S, M, N, e, rs);
            break;
        case EPI_LOGITS:  // one 16-row tile (one sequence) per workgroup row; one arrival counter per tile
            if (M > 128 || e.block != 16) return hipErrorInvalidValue;
            hipLaunchKernelGGL((batch_epi_kernel<EPI_LOGITS, 1>), rows_grid, dim3(256), 0, s, part, S, M, N, e, rs);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
