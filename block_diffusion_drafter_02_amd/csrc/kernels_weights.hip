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
#include "dflash_internal.h"

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

template <int WT>
struct WTraits;
template <>
struct WTraits<DFLASH_F32> {
    static constexpr int ES = 4;  // bytes per element
    static constexpr int NV = 4;  // 16-byte words per lane per tile
};
template <>
struct WTraits<DFLASH_BF16> {
    static constexpr int ES = 2;
    static constexpr int NV = 2;
};
template <>
struct WTraits<DFLASH_FP8_E4M3> {
    static constexpr int ES = 1;
    static constexpr int NV = 1;
};

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
// Operand loading and the per-tile MFMA step
// ---------------------------------------------------------------------------
template <int WT>
__device__ __forceinline__ void load_wtile(const void *W, size_t tile_index, int lane, u32x4 (&w)[WTraits<WT>::NV]) {
    constexpr int NV = WTraits<WT>::NV;
    const u32x4 *p = (const u32x4 *)W + tile_index * NV * 64 + lane;
#pragma unroll
    for (int v = 0; v < NV; ++v) w[v] = p[v * 64];
}

// 16 bf16 values of one lane as two MFMA operands
__device__ __forceinline__ void as_bf16x8x2(const u32x4 (&w)[2], bf16x8 &lo, bf16x8 &hi) {
    lo = __builtin_bit_cast(bf16x8, w[0]);
    hi = __builtin_bit_cast(bf16x8, w[1]);
}

__device__ __forceinline__ void fp8x16_to_bf16x8x2(const u32x4 &w, bf16x8 &lo, bf16x8 &hi) {
    u32x4 a, b;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        uint32_t x = w[i];
        a[2 * i] = (uint32_t)e4m3_to_bf16(x & 0xff) | ((uint32_t)e4m3_to_bf16((x >> 8) & 0xff) << 16);
        a[2 * i + 1] = (uint32_t)e4m3_to_bf16((x >> 16) & 0xff) | ((uint32_t)e4m3_to_bf16(x >> 24) << 16);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        uint32_t x = w[2 + i];
        b[2 * i] = (uint32_t)e4m3_to_bf16(x & 0xff) | ((uint32_t)e4m3_to_bf16((x >> 8) & 0xff) << 16);
        b[2 * i + 1] = (uint32_t)e4m3_to_bf16((x >> 16) & 0xff) | ((uint32_t)e4m3_to_bf16(x >> 24) << 16);
    }
    lo = __builtin_bit_cast(bf16x8, a);
    hi = __builtin_bit_cast(bf16x8, b);
}

// Activation operand of one lane: row `row`, columns kb*64 + 16*(lane/16) .. +16.
// NT = number of 16-byte words per lane: SPLIT3 -> 3 terms x 2, F32 -> 4, BF16 -> 2.
template <int AF>
struct AFTraits;
template <>
struct AFTraits<ACT_SPLIT3> {
    static constexpr int NW = 6;
};
template <>
struct AFTraits<ACT_F32> {
    static constexpr int NW = 4;
};
template <>
struct AFTraits<ACT_BF16> {
    static constexpr int NW = 2;
};

// Row-major activation planes (the large-M GEMM reads caller inputs and its
// own row-major staging).
template <int AF>
__device__ __forceinline__ void load_act(const void *act, int act_rows, int K, int row, int M, int kb, int lane,
                                         u32x4 (&a)[AFTraits<AF>::NW]) {
    constexpr int NW = AFTraits<AF>::NW;
    if (row >= M) {
#pragma unroll
        for (int i = 0; i < NW; ++i) a[i] = u32x4{0, 0, 0, 0};
        return;
    }
    const int col = kb * KBLK + LANE_ELEMS * (lane >> 4);
    if constexpr (AF == ACT_SPLIT3) {
        const uint16_t *base = (const uint16_t *)act;
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const u32x4 *p = (const u32x4 *)(base + ((size_t)t * act_rows + row) * K + col);
            a[2 * t] = p[0];
            a[2 * t + 1] = p[1];
        }
    } else if constexpr (AF == ACT_F32) {
        const u32x4 *p = (const u32x4 *)((const float *)act + (size_t)row * K + col);
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = p[i];
    } else {
        const u32x4 *p = (const u32x4 *)((const uint16_t *)act + (size_t)row * K + col);
        a[0] = p[0];
        a[1] = p[1];
    }
}

// Lane-ordered activation planes (act_offset): one k-block of one 16-row tile
// is 1 KB per plane word, read by one contiguous wavefront load.
template <int AF>
__device__ __forceinline__ void load_act_lanes(const void *act, int act_rows, int K, int mt, bool live, int kb,
                                               int lane, u32x4 (&a)[AFTraits<AF>::NW]) {
    constexpr int NW = AFTraits<AF>::NW;
    if (!live) {
#pragma unroll
        for (int i = 0; i < NW; ++i) a[i] = u32x4{0, 0, 0, 0};
        return;
    }
    const int KB = K / KBLK;
    if constexpr (AF == ACT_SPLIT3) {
        const u32x4 *base = (const u32x4 *)act + ((size_t)mt * KB + kb) * 128 + lane;
        const size_t plane = (size_t)act_rows * K / 8;  // 16-byte words per plane
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            a[2 * t] = base[t * plane];
            a[2 * t + 1] = base[t * plane + 64];
        }
    } else {
        static_assert(AF == ACT_F32, "lane-ordered activations are split bf16 or f32");
        const u32x4 *base = (const u32x4 *)act + ((size_t)mt * KB + kb) * 256 + lane;
#pragma unroll
        for (int v = 0; v < 4; ++v) a[v] = base[v * 64];
    }
}

// acc += A(16 rows x 64 k) * W(16 cols x 64 k)^T for one tile
template <int WT, int AF>
__device__ __forceinline__ void tile_mfma(const u32x4 (&w)[WTraits<WT>::NV], const u32x4 (&a)[AFTraits<AF>::NW],
                                          f32x4 &acc) {
    if constexpr (WT == DFLASH_F32) {
        static_assert(AF == ACT_F32, "f32 weights take f32 activations");
#pragma unroll
        for (int v = 0; v < 4; ++v) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float av = __uint_as_float(a[v][j]);
                float wv = __uint_as_float(w[v][j]);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, wv, acc, 0, 0, 0);
            }
        }
    } else {
        bf16x8 wlo, whi;
        if constexpr (WT == DFLASH_BF16)
            as_bf16x8x2(w, wlo, whi);
        else
            fp8x16_to_bf16x8x2(w[0], wlo, whi);
        if constexpr (AF == ACT_SPLIT3) {
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[2 * t]), wlo, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[2 * t + 1]), whi, acc, 0, 0,
                                                              0);
            }
        } else {
            static_assert(AF == ACT_BF16, "bf16 weights take split or bf16 activations");
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[0]), wlo, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[1]), whi, acc, 0, 0, 0);
        }
    }
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

    __shared__ float tile[MP][GN];
    __shared__ float rs_s[MP];
    __shared__ int is_last;
    for (int wv = 0; wv < WK; ++wv) {
        if (wk == wv) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = mt * 16 + 4 * (lane >> 4) + i;
                        const int col = 64 * wn + 16 * t + (lane & 15);
                        if (wv == 0)
                            tile[m][col] = acc[mt][t][i];
                        else
                            tile[m][col] += acc[mt][t][i];
                    }
        }
        __syncthreads();
    }

    float *tflat = &tile[0][0];
    if (a.S > 1) {
        // Split-K handshake without cache-wide maintenance: partials are written
        // and read with device-coherent (agent-scope) atomic accesses, each wave
        // waits for its stores to complete before the workgroup signals, and the
        // last workgroup of the group to arrive sums the partials in split order.
        float *part = a.partial + ((size_t)s * G + g) * (MP * GN);
        for (int e = tid; e < MP * GN; e += 256)
            __hip_atomic_store((uint32_t *)(part + e), __float_as_uint(tflat[e]), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __syncthreads();
        if (tid == 0)
            is_last = __hip_atomic_fetch_add(&a.counters[g], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.S - 1;
        __syncthreads();
        if (!is_last) return;
        constexpr int EPT = MP * GN / 256;  // tile elements per thread
        float sum[EPT];
#pragma unroll
        for (int k = 0; k < EPT; ++k) sum[k] = 0.0f;
        for (int s0 = 0; s0 < a.S; s0 += 4) {  // four splits' loads in flight, summed in split order
            float v[4][EPT];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int k = 0; k < EPT; ++k)
                    v[u][k] = s0 + u < a.S ? __uint_as_float(__hip_atomic_load(
                                                 (const uint32_t *)(a.partial + ((size_t)(s0 + u) * G + g) * (MP * GN) +
                                                                    tid + 256 * k),
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                                           : 0.0f;
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int k = 0; k < EPT; ++k)
                    if (s0 + u < a.S) sum[k] += v[u][k];
        }
#pragma unroll
        for (int k = 0; k < EPT; ++k) tflat[tid + 256 * k] = sum[k];
        if (tid == 0) __hip_atomic_store(&a.counters[g], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
    }

    // ---- epilogue on the 16*MT x GN tile ----
    const EpiArgs &e = a.epi;
    // rs[m] = 1/sqrt(sum_g ss[g][m] / E + eps): 16 threads per row, fixed-order tree
    for (int m0 = 0; m0 < MP; m0 += 16) {
        const int m = m0 + (tid >> 4), sub = tid & 15;
        float part = 0.0f;
        if (e.ss != nullptr && m < M)
            for (int gg = sub; gg < e.ss_groups; gg += 16) part += e.ss[(size_t)gg * e.ss_stride + m];
        for (int o = 8; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
        if (sub == 0) rs_s[m] = (e.ss != nullptr && m < M) ? 1.0f / sqrtf(part * e.inv_E + e.eps) : 1.0f;
    }
    __syncthreads();

    if constexpr (EPI == EPI_QKV) {
        // columns of this group: whole heads of q (RMSNorm q_norm, rope, * 1/sqrt(D)), of k (RMSNorm
        // k_norm, rope) or of v (as is), one wave per (row, head) vector
        const int D = e.D, hpg = GN / D;  // heads per group
        // the lane's norm weights and the (cos, sin) of its rope pair for all 16 block rows, loaded once
        float qn[2], kn[2], cosr[16], sinr[16];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int d = min(lane + 64 * u, D - 1);
            qn[u] = e.q_norm[d];
            kn[u] = e.k_norm[d];
        }
        const int pair = D == 128 ? lane : (lane & 31);
        const int b0 = (wave < M * hpg) ? (wave / hpg) / e.block : 0;  // rows of one wave share a sequence
        for (int i = 0; i < 16; ++i) {
            const float2 cs = *(const float2 *)(e.rope_cs + ((size_t)b0 * e.block + i) * D + 2 * pair);
            cosr[i] = cs.x;
            sinr[i] = cs.y;
        }
        for (int vec = wave; vec < M * hpg; vec += 4) {
            const int m = vec / hpg, hg = vec % hpg;
            const int c0 = hg * D;            // first column of the head inside the tile
            const int n0 = g * GN + c0;       // first column of the head in the output
            const bool is_q = n0 < e.qdim, is_k = !is_q && n0 < e.qdim + e.kvdim;
            const int b = m / e.block, i = m % e.block;
            float x[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int d = lane + 64 * u;
                float v = 0.0f;
                if (d < D) {
                    v = tile[m][c0 + d] * rs_s[m];
                    if (e.wscale) v *= e.wscale[n0 + d];
                }
                x[u] = v;
            }
            if (is_q || is_k) {
                float ss = x[0] * x[0] + x[1] * x[1];
                ss = wave_sum(ss);
                const float r = 1.0f / sqrtf(ss / (float)D + e.eps);
                float cn = 0.0f, sn = 0.0f;
                if (b == b0) {
#pragma unroll
                    for (int k = 0; k < 16; ++k)
                        if (k == i) {
                            cn = cosr[k];
                            sn = sinr[k];
                        }
                } else {
                    const float2 cs = *(const float2 *)(e.rope_cs + ((size_t)b * e.block + i) * D + 2 * pair);
                    cn = cs.x;
                    sn = cs.y;
                }
                const float w0 = is_q ? qn[0] : kn[0], w1 = is_q ? qn[1] : kn[1];
                if (D == 128) {
                    const float x1 = x[0] * r * w0, x2 = x[1] * r * w1;
                    x[0] = x1 * cn - x2 * sn;
                    x[1] = x1 * sn + x2 * cn;
                } else {  // D == 64: the pair partner of lane l is lane l ^ 32
                    const float x1 = x[0] * r * w0;
                    const float partner = __shfl_xor(x1, 32, 64);
                    x[0] = lane < 32 ? x1 * cn - partner * sn : partner * sn + x1 * cn;
                }
                if (is_q) {
                    x[0] *= e.qscale;
                    x[1] *= e.qscale;
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int d = lane + 64 * u;
                if (d < D) e.out[(size_t)m * e.ld_out + n0 + d] = x[u];
            }
        }
    } else if constexpr (EPI == EPI_SCALED) {
        for (int m = wave; m < M; m += 4) {
            const int n = g * GROUP_N + lane;
            float v = tile[m][lane] * rs_s[m];
            if (e.wscale) v *= e.wscale[n];
            e.out[(size_t)m * e.ld_out + n] = v;
        }
    } else if constexpr (EPI == EPI_RESID) {
        constexpr int RPW = MP / 4;  // rows per wave; all residual loads issued first
        const int n = g * GROUP_N + lane;
        const float sc = e.wscale ? e.wscale[n] : 1.0f;
        float xv[RPW];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const int m = wave + 4 * r;
            xv[r] = m < M ? e.x[(size_t)m * e.ld_x + n] : 0.0f;
        }
        const float wn = e.wnext[n];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const int m = wave + 4 * r;
            if (m < M) {
                const float xn = xv[r] + tile[m][lane] * sc;
                e.x[(size_t)m * e.ld_x + n] = xn;
                write_act(e.act_out, e.act_fmt, e.act_rows, e.act_K, m, n, xn * wn);
                const float sq = wave_sum(xn * xn);
                if (lane == 0) e.ss_out[(size_t)g * e.ss_stride + m] = sq;
            }
        }
    } else if constexpr (EPI == EPI_SWIGLU) {
        for (int m = wave; m < M; m += 4) {
            if (lane < 32) {
                float gv = tile[m][lane] * rs_s[m];
                float uv = tile[m][lane + 32] * rs_s[m];
                if (e.wscale) {
                    gv *= e.wscale[g * GROUP_N + lane];
                    uv *= e.wscale[g * GROUP_N + 32 + lane];
                }
                const float act = gv / (1.0f + expf(-gv)) * uv;
                write_act(e.act_out, e.act_fmt, e.act_rows, e.act_K, m, g * 32 + lane, act);
            }
        }
    } else {  // EPI_LOGITS
        for (int m = wave; m < M; m += 4) {
            const int n = g * GROUP_N + lane;
            float v = tile[m][lane] * rs_s[m];
            if (e.wscale) v *= e.wscale[n];
            e.out[(size_t)m * e.ld_out + n] = v;
            float bv = v;
            int bi = n;
            for (int o = 32; o > 0; o >>= 1) {
                const float ov = __shfl_xor(bv, o, 64);
                const int oi = __shfl_xor(bi, o, 64);
                if (ov > bv || (ov == bv && oi < bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            if (lane == 0) {
                __hip_atomic_store((uint32_t *)(e.am_val + (size_t)g * e.ss_stride + m), __float_as_uint(bv),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(e.am_idx + (size_t)g * e.ss_stride + m, bi, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __syncthreads();
        if (tid == 0)
            is_last = __hip_atomic_fetch_add(e.am_counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == G - 1;
        __syncthreads();
        if (!is_last) return;
        __shared__ int best_s[MP];
        for (int m0 = 0; m0 < M; m0 += 16) {
            const int m = m0 + (tid >> 4), sub = tid & 15;
            float bv = -INFINITY;
            int bi = 0x7fffffff;
            if (m < M)
                for (int gg = sub; gg < G; gg += 16) {
                    const float v = __uint_as_float(__hip_atomic_load(
                        (const uint32_t *)(e.am_val + (size_t)gg * e.ss_stride + m), __ATOMIC_RELAXED,
                        __HIP_MEMORY_SCOPE_AGENT));
                    const int i = __hip_atomic_load(e.am_idx + (size_t)gg * e.ss_stride + m, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
                    if (v > bv || (v == bv && i < bi)) {
                        bv = v;
                        bi = i;
                    }
                }
            for (int o = 8; o > 0; o >>= 1) {
                const float ov = __shfl_xor(bv, o, 64);
                const int oi = __shfl_xor(bi, o, 64);
                if (ov > bv || (ov == bv && oi < bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            if (sub == 0 && m < M) {
                best_s[m] = bi;
                const int b = m / e.block, i = m % e.block;
                if (i > 0) e.drafts[(size_t)b * (e.block - 1) + i - 1] = bi;
            }
        }
        __syncthreads();
        if (e.target != nullptr && tid < M / e.block) {
            const int b = tid;
            int n = 0;
            while (n < e.block - 1 && best_s[b * e.block + 1 + n] == e.target[(size_t)b * (e.block - 1) + n]) ++n;
            e.n_ok[b] = n;
        }
        if (tid == 0) __hip_atomic_store(e.am_counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
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

// The q/k/v projection runs with 128-column groups (WN = 2, whole heads for its
// epilogue); every other projection with 64-column groups.
template <int WT, int AF>
static hipError_t launch_gemv_epi(int MT, int WN, dim3 grid, const GemvArgs &a, hipStream_t s) {
    if (a.epi.kind == EPI_QKV) return WN == 2 ? launch_gemv_mt<WT, AF, EPI_QKV, 2>(MT, grid, a, s) : hipErrorInvalidValue;
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
