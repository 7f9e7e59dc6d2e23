// Device code shared by the weight-streaming kernels: operand loading of the
// tiled weights and lane-ordered activations, the per-tile MFMA step, the
// fixed-order reduction of a workgroup's waves, the split-K handshake and the
// fused epilogues. Included by the per-launch kernels and by the dataflow
// chain.
#pragma once

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
// Operand loading and the per-tile MFMA step
// ---------------------------------------------------------------------------
// Weights are read exactly once per step, so their loads are non-temporal: they do not displace the
// activations, partial sums and ring entries that the caches hold for the rest of the step (measured on
// the real-dimension bf16 step: gate/up 104.7 -> 97.0 us, step 1176 -> 1108 us).
template <int WT>
__device__ __forceinline__ void load_wtile(const void *W, size_t tile_index, int lane, u32x4 (&w)[WTraits<WT>::NV]) {
    constexpr int NV = WTraits<WT>::NV;
    const u32x4 *p = (const u32x4 *)W + tile_index * NV * 64 + lane;
#pragma unroll
    for (int v = 0; v < NV; ++v) w[v] = __builtin_nontemporal_load(p + v * 64);
}

// 16 bf16 values of one lane as two MFMA operands
__device__ __forceinline__ void as_bf16x8x2(const u32x4 (&w)[2], bf16x8 &lo, bf16x8 &hi) {
    lo = __builtin_bit_cast(bf16x8, w[0]);
    hi = __builtin_bit_cast(bf16x8, w[1]);
}

// 16 E4M3FN codes of one lane (byte j of word i = element 4i + j) as two bf16x8
// operands. The hardware conversion is exact (every E4M3 value is a bf16
// value); it decodes two codes per instruction.
__device__ __forceinline__ void fp8x16_to_bf16x8x2(const u32x4 &w, bf16x8 &lo, bf16x8 &hi) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    u32x4 a, b;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        a[2 * i] = __builtin_bit_cast(uint32_t, (bf16x2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false));
        a[2 * i + 1] = __builtin_bit_cast(uint32_t, (bf16x2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true));
        b[2 * i] = __builtin_bit_cast(uint32_t, (bf16x2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 + i], 1.0f, false));
        b[2 * i + 1] =
            __builtin_bit_cast(uint32_t, (bf16x2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 + i], 1.0f, true));
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

// MFMA operand format of an activation format: f32 lane words feeding bf16 or
// fp8 weights are split at load into the three bf16 terms of the exact split
// (the terms a three-plane activation would hold), so a producer writes 4
// bytes per value instead of 6 and a consumer reads a third less.
template <int WT, int AF>
struct ActOp {
    static constexpr int AFO = (WT != DFLASH_F32 && AF == ACT_F32) ? ACT_SPLIT3 : AF;
};

template <int WT, int AF>
__device__ __forceinline__ void load_act_operands(const void *act, int act_rows, int K, int mt, bool live, int kb,
                                                  int lane, u32x4 (&a)[AFTraits<ActOp<WT, AF>::AFO>::NW]) {
    if constexpr (WT != DFLASH_F32 && AF == ACT_F32) {
        u32x4 f[4];
        load_act_lanes<ACT_F32>(act, act_rows, K, mt, live, kb, lane, f);
        // f32 words 0-1 hold elements 0-7 (the first MFMA of the k-block), words 2-3 elements 8-15;
        // term t of half h goes where the three-plane layout keeps it, a[2t + h]
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float v[8] = {__uint_as_float(f[2 * h].x),     __uint_as_float(f[2 * h].y),
                                __uint_as_float(f[2 * h].z),     __uint_as_float(f[2 * h].w),
                                __uint_as_float(f[2 * h + 1].x), __uint_as_float(f[2 * h + 1].y),
                                __uint_as_float(f[2 * h + 1].z), __uint_as_float(f[2 * h + 1].w)};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t w0, w1, w2;
                split3_pair(v[2 * i], v[2 * i + 1], w0, w1, w2);
                a[h][i] = w0;
                a[2 + h][i] = w1;
                a[4 + h][i] = w2;
            }
        }
    } else {
        load_act_lanes<AF>(act, act_rows, K, mt, live, kb, lane, a);
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
// Workgroup reduction and split-K handshake
// ---------------------------------------------------------------------------
// The WK waves along the reduction add their accumulators into the LDS tile
// [16*MT][64*WN] in wave order (the same order on every launch).
template <int MT, int WN>
__device__ __forceinline__ void reduce_waves(const f32x4 (&acc)[MT][4], float *tile, int wn, int wk, int lane) {
    constexpr int WK = 4 / WN, GN = GROUP_N * WN;
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
                            tile[m * GN + col] = acc[mt][t][i];
                        else
                            tile[m * GN + col] += acc[mt][t][i];
                    }
        }
        __syncthreads();
    }
}

// Split-K handshake without cache-wide maintenance. The workgroup's partial
// tile (n_el floats) goes to `mine` with device-coherent (agent-scope) stores;
// every thread waits for its stores before the workgroup bumps `counter`. The
// workgroup that brings the count to nparts reads the nparts partials
// parts + i * stride (i = 0 .. nparts-1) with device-coherent loads, sums
// them in that order into `tile`, re-arms the counter and returns true; the
// others return false. The result does not depend on arrival order.
template <int EPT>
__device__ __forceinline__ bool splitk_last(float *tile, float *mine, const float *parts, size_t stride, int nparts,
                                            int *counter, int *flag_s) {
    const int tid = threadIdx.x;
    for (int k = 0; k < EPT; ++k)
        __hip_atomic_store((uint32_t *)(mine + tid + 256 * k), __float_as_uint(tile[tid + 256 * k]), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (tid == 0)
        *flag_s = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nparts - 1;
    __syncthreads();
    if (!*flag_s) return false;
    constexpr int UB = EPT <= 4 ? 16 : (EPT <= 8 ? 8 : (EPT <= 16 ? 4 : 2));  // partials in flight together
    float sum[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) sum[k] = 0.0f;
    for (int s0 = 0; s0 < nparts; s0 += UB) {  // summed in partial order
        float v[UB][EPT];
#pragma unroll
        for (int u = 0; u < UB; ++u)
#pragma unroll
            for (int k = 0; k < EPT; ++k)
                v[u][k] = s0 + u < nparts
                              ? __uint_as_float(__hip_atomic_load(
                                    (const uint32_t *)(parts + (size_t)(s0 + u) * stride + tid + 256 * k),
                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                              : 0.0f;
#pragma unroll
        for (int u = 0; u < UB; ++u)
#pragma unroll
            for (int k = 0; k < EPT; ++k)
                if (s0 + u < nparts) sum[k] += v[u][k];
    }
#pragma unroll
    for (int k = 0; k < EPT; ++k) tile[tid + 256 * k] = sum[k];
    if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    return true;
}

// Split-K hand-off in which only the earlier arrivals store their partial tile.
// Writes issued while the weight stream saturates HBM cost far more than their
// size (measured: a 4 KB store per workgroup of a 1248-workgroup, 532 MB read
// stream adds 4.7 us), so the last arrival keeps its own partial in LDS. Each
// workgroup first bumps `arrive`; one that is not last stores its tile to
// `mine` with device-coherent stores, waits for them and bumps `written`. The
// last one polls `written` (tid 0, bounded: on giving up it sets *err, which
// dflash_check_device reports) until the other nparts - 1 partials are out,
// then sums the nparts partials in split order, its own (split s) from LDS, so
// the result is the same as when every split stores its partial. It re-arms
// both counters and returns true; the others return false.
constexpr int SPLITK_POLL_LIMIT = 1 << 22;

template <int EPT>
__device__ __forceinline__ bool splitk_hand_off(float *tile, float *mine, const float *parts, size_t stride,
                                                int nparts, int s, int *arrive, int *written, int *err, int *flag_s) {
    const int tid = threadIdx.x;
    if (tid == 0)
        *flag_s = __hip_atomic_fetch_add(arrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nparts - 1;
    __syncthreads();
    if (!*flag_s) {
        for (int k = 0; k < EPT; ++k)
            __hip_atomic_store((uint32_t *)(mine + tid + 256 * k), __float_as_uint(tile[tid + 256 * k]),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __syncthreads();
        if (tid == 0) __hip_atomic_fetch_add(written, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
    }
    if (tid == 0) {
        int polls = 0;
        while (__hip_atomic_load(written, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nparts - 1) {
            if (++polls > SPLITK_POLL_LIMIT) {
                __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    __syncthreads();
    constexpr int UB = EPT <= 4 ? 16 : (EPT <= 8 ? 8 : (EPT <= 16 ? 4 : 2));  // partials in flight together
    float sum[EPT], own[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        sum[k] = 0.0f;
        own[k] = tile[tid + 256 * k];
    }
    for (int s0 = 0; s0 < nparts; s0 += UB) {  // summed in partial order
        float v[UB][EPT];
#pragma unroll
        for (int u = 0; u < UB; ++u)
#pragma unroll
            for (int k = 0; k < EPT; ++k)
                v[u][k] = s0 + u < nparts && s0 + u != s
                              ? __uint_as_float(__hip_atomic_load(
                                    (const uint32_t *)(parts + (size_t)(s0 + u) * stride + tid + 256 * k),
                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                              : own[k];
#pragma unroll
        for (int u = 0; u < UB; ++u)
#pragma unroll
            for (int k = 0; k < EPT; ++k)
                if (s0 + u < nparts) sum[k] += v[u][k];
    }
#pragma unroll
    for (int k = 0; k < EPT; ++k) tile[tid + 256 * k] = sum[k];  // each thread rewrites only its own elements
    if (tid == 0) {
        __hip_atomic_store(arrive, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(written, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    return true;
}

// ---------------------------------------------------------------------------
// Sampling noise: Philox-4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw,
// SC 2011) -- its first output word at counter (c0, c1, c2, c3) under key
// (k0, k1) -- and the Gumbel(0, 1) value of that word: u = ((x >> 8) + 1/2)
// 2^-24, exact in fp32, and -log(-log(u)).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t philox4x32_10_x0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                     uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
        const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    return c0;
}

__device__ __forceinline__ float gumbel_noise(uint32_t seed_lo, uint32_t seed_hi, int b, int pos, int n) {
    const uint32_t x = philox4x32_10_x0((uint32_t)pos, (uint32_t)n, (uint32_t)b, 0u, seed_lo, seed_hi);
    const float u = ((float)(x >> 8) + 0.5f) * 0x1p-24f;
    return -logf(-logf(u));
}

// ---------------------------------------------------------------------------
// Fused epilogues on the finished [16*MT][64*WN] tile of column group g
// ---------------------------------------------------------------------------
// All outputs are written with device-coherent stores, so a consumer in the
// same launch (the persistent kernel) reads them after a grid barrier.
// LDS: tile (MP*GN floats), rs_s (MP floats), flag_s (1 int), best_s (MP ints).
// Operands of the epilogue of a one-tile (MT = 1) group that do not depend on
// the product: the partial sums of squares of this thread's row, the residual
// rows, the next norm weight and the fp8 column scales. A kernel loads them
// before its weight stream so that their latency is hidden; for MT > 1 the
// epilogue loads them itself.
struct EpiPre {
    static constexpr int SSN = 8;  // ss partials per thread (ss_groups <= 16 * SSN)
    float ss[SSN];
    float x[4];
    float sc, sc2, wn;
    bool ss_ok;
};

template <int EPI, int MT>
__device__ __forceinline__ void epi_prefetch(const EpiArgs &e, int g, EpiPre &p) {
    if constexpr (MT != 1) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int M = e.M;
    if constexpr (EPI != EPI_RESID) {
        const int m = tid >> 4, sub = tid & 15;
        p.ss_ok = e.ss_groups <= 16 * EpiPre::SSN;
#pragma unroll
        for (int j = 0; j < EpiPre::SSN; ++j) {
            const int gg = sub + 16 * j;
            p.ss[j] = (e.ss != nullptr && m < M && gg < e.ss_groups) ? e.ss[(size_t)m * e.ss_gs + gg] : 0.0f;
        }
    }
    if constexpr (EPI == EPI_SWIGLU) {
        p.sc = e.wscale && lane < 32 ? e.wscale[g * GROUP_N + lane] : 1.0f;
        p.sc2 = e.wscale && lane < 32 ? e.wscale[g * GROUP_N + 32 + lane] : 1.0f;
    } else {
        p.sc = e.wscale ? e.wscale[g * GROUP_N + lane] : 1.0f;
    }
    if constexpr (EPI == EPI_RESID) {
        const int n = g * GROUP_N + lane;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = wave + 4 * r;
            p.x[r] = m < M ? e.x[(size_t)m * e.ld_x + n] : 0.0f;
        }
        p.wn = e.wnext[n];
    }
}

// Two k-splits meeting through per-element exchange slots (a q/k/v group: 16
// rows x 64 columns, whose epilogue is per element). Each split swaps its
// partial value into the element's slot, which holds XSLOT_EMPTY between
// launches: the split that receives XSLOT_EMPTY is first and leaves its value
// there; the other receives it, adds (IEEE addition is commutative, so the sum
// does not depend on which split came first), re-arms the slot and writes the
// output element. One device round trip instead of the counter hand-off's
// store, wait, counter and load.
// rs[m] = 1/sqrt(sum_g ss[m][g] / E + eps) of one 16-row tile into LDS (256 threads, as in gemv_epilogue)
template <bool PF>
__device__ __forceinline__ void tile_row_scales(const EpiArgs &e, float *rs_s, const EpiPre &pre) {
    const int tid = threadIdx.x;
    const int m = tid >> 4, sub = tid & 15;
    float part = 0.0f;
    if (PF && pre.ss_ok) {
#pragma unroll
        for (int j = 0; j < EpiPre::SSN; ++j) part += pre.ss[j];
    } else if (e.ss != nullptr && m < e.M) {
        for (int gg = sub; gg < e.ss_groups; gg += 16) part += e.ss[(size_t)m * e.ss_gs + gg];
    }
    for (int o = 8; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
    if (sub == 0) rs_s[m] = (e.ss != nullptr && m < e.M) ? 1.0f / sqrtf(part * e.inv_E + e.eps) : 1.0f;
    __syncthreads();
}

// Both splits swap their four elements into the slots at once; returns, per element, whether this split
// received the other's value (and so owns the element) and the sum in v[k]. Owners re-arm their slots.
__device__ __forceinline__ void exchange_tile(const float *tile, uint32_t *slot, float (&v)[4], bool (&own)[4]) {
    const int tid = threadIdx.x;
    uint32_t old[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)  // all four exchanges in flight together
        old[k] = __hip_atomic_exchange(slot + tid + 256 * k, __float_as_uint(tile[tid + 256 * k]), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        own[k] = old[k] != XSLOT_EMPTY;
        v[k] = own[k] ? __uint_as_float(old[k]) + tile[tid + 256 * k] : 0.0f;
        if (own[k]) __hip_atomic_store(slot + tid + 256 * k, XSLOT_EMPTY, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <bool PF>
__device__ __forceinline__ void scaled_exchange(const EpiArgs &e, int g, const float *tile, float *rs_s, uint32_t *slot,
                                                const EpiPre &pre) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int M = e.M;
    tile_row_scales<PF>(e, rs_s, pre);
    const int n = g * GROUP_N + lane;
    const float sc = PF ? pre.sc : (e.wscale ? e.wscale[n] : 1.0f);
    float v[4];
    bool own[4];
    exchange_tile(tile, slot, v, own);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int m = wave + 4 * k;  // element tid + 256 k of the [16][64] tile
        if (own[k] && m < M) {
            float r = v[k] * rs_s[m];
            if (e.wscale) r *= sc;
            st_f32(e.out + (size_t)m * e.ld_out + n, r);
        }
    }
}

// Argmax across the groups of one launch: every group stores its (value,
// column) maximum of row m as one 64-bit key that orders by value, then by
// lower column (values that compare equal, +0 and -0 among them, give the same
// upper word), so the largest key of a row names the first column of the row
// maximum whatever the order the keys are compared in. (One shared key per row
// updated with 64-bit atomic max was measured slower: 128 groups contend on
// the same two cache lines.)
__device__ __forceinline__ unsigned long long argmax_key(float v, int col) {
    uint32_t b = __float_as_uint(v);
    if (b == 0x80000000u) b = 0u;  // -0 ranks as +0
    const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((unsigned long long)ord << 32) | (uint32_t)~(uint32_t)col;
}
__device__ __forceinline__ int argmax_key_index(unsigned long long k) { return (int)~(uint32_t)(k & 0xffffffffull); }

// The argmax's last stage: once a workgroup's keys for its rows are stored in key slots 0..NK-1
// (am_key[slot][row]), it counts itself in; the last of the arrivals (NK unless e.arrivals is set) takes
// the largest key of every row of the step (e.rows_all, else M), writes the drafts, runs the acceptance
// scan and re-arms the counter. best_s holds one int per row of the step.
// TILE: the arrivals are those of one 16-row tile, rows e.row0 .. e.row0 + e.M
// (one sequence of a batch), which the last of them finishes on its own.
template <bool TILE = false>
__device__ __forceinline__ void argmax_finish(const EpiArgs &e, int NK, int *flag_s, int *best_s) {
    const int tid = threadIdx.x;
    const int M = TILE ? e.M : (e.rows_all ? e.rows_all : e.M);
    const int r0 = TILE ? e.row0 : 0;  // first row of the step handled here
    const int arrivals = e.arrivals ? e.arrivals : NK;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (tid == 0)
        *flag_s = __hip_atomic_fetch_add(e.am_counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == arrivals - 1;
    __syncthreads();
    if (!*flag_s) return;
    // every group's key is in: 16 threads per row take the largest key of the
    // groups sub, sub + 16, ... with the loads of a batch issued together,
    // then a 16-lane reduction (the order does not change a maximum)
    constexpr int KU = 8;
    for (int m0 = 0; m0 < M; m0 += 16) {
        const int m = m0 + (tid >> 4), sub = tid & 15;
        unsigned long long best = 0ull;
        if (m < M)
            for (int g0 = sub; g0 < NK; g0 += 16 * KU) {
                unsigned long long k[KU];
#pragma unroll
                for (int u = 0; u < KU; ++u)
                    k[u] = g0 + 16 * u < NK ? __hip_atomic_load(e.am_key + (size_t)(g0 + 16 * u) * e.ss_stride + r0 + m,
                                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                           : 0ull;
#pragma unroll
                for (int u = 0; u < KU; ++u) best = k[u] > best ? k[u] : best;
            }
        for (int o = 8; o > 0; o >>= 1) {
            const unsigned long long ok = __shfl_xor(best, o, 64);
            best = ok > best ? ok : best;
        }
        if (sub == 0 && m < M) {
            const int bi = argmax_key_index(best);
            best_s[m] = bi;
            const int b = (r0 + m) / e.block, i = (r0 + m) % e.block;
            if (i > 0 && i < e.gamma) st_i32(e.drafts + (size_t)b * (e.gamma - 1) + i - 1, bi);
        }
    }
    __syncthreads();
    if (e.target != nullptr && tid < M / e.block) {
        const int b = r0 / e.block + tid;  // sequence; its rows are best_s[tid * block ..]
        int n = 0;
        while (n < e.gamma - 1 && best_s[tid * e.block + 1 + n] == e.target[(size_t)b * (e.gamma - 1) + n]) ++n;
        st_i32(e.n_ok + b, n);
    }
    if (tid == 0) __hip_atomic_store(e.am_counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The lm_head's two k-splits meet through exchange slots (as q/k/v): each split
// finishes the logits it owns, and stores per row the argmax key of those
// columns in key slot 2g + s (0 for a row where it owns none), so the argmax's
// last stage reduces 2G key slots. The logits and the maximum do not depend on
// which split owns which element.
template <bool PF>
__device__ __forceinline__ void logits_exchange(const EpiArgs &e, int g, int G, int s, const float *tile, float *rs_s,
                                                uint32_t *slot, const EpiPre &pre, int *flag_s, int *best_s) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int M = e.M;
    tile_row_scales<PF>(e, rs_s, pre);
    const int n = g * GROUP_N + lane;
    const float sc = PF ? pre.sc : (e.wscale ? e.wscale[n] : 1.0f);
    float v[4];
    bool own[4];
    exchange_tile(tile, slot, v, own);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int m = wave + 4 * k;
        if (m >= M) continue;  // uniform over the wave
        unsigned long long key = 0ull;
        if (own[k]) {
            float r = v[k] * rs_s[m];
            if (e.wscale) r *= sc;
            st_f32(e.out + (size_t)m * e.ld_out + n, r);
            if (e.temp > 0.0f) {  // the draft is a sample: the argmax runs on logit / T + Gumbel noise
                const int b = m / e.block;
                r = r / e.temp + gumbel_noise(e.seed_lo, e.seed_hi, b, e.n_past[b] + m % e.block, n);
            }
            key = argmax_key(r, n);
        }
        for (int o = 32; o > 0; o >>= 1) {
            const unsigned long long ok = __shfl_xor(key, o, 64);
            key = ok > key ? ok : key;
        }
        if (lane == 0)
            __hip_atomic_store(e.am_key + (size_t)(2 * g + s) * e.ss_stride + m, key, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    argmax_finish(e, 2 * G, flag_s, best_s);
}

// CW: columns of group g (64, or 32 for half groups; lanes >= CW idle). The
// G groups of one launch write ss_out rows 0..G-1.
// RSR: rs_s already holds the row scales (the batched epilogue's precomputed ones).
// ATILE: the logits' argmax finishes per 16-row tile (argmax_finish<true>).
template <int EPI, int MT, int WN, bool PF = false, int CW = GROUP_N, bool RSR = false, bool ATILE = false>  // PF: operands from epi_prefetch (MT = 1)
__device__ __forceinline__ void gemv_epilogue(const EpiArgs &e, int g, int G, float *tile, float *rs_s, int *flag_s,
                                              int *best_s, const EpiPre &pre = EpiPre{}) {
    static_assert(!PF || MT == 1, "prefetched epilogue operands cover one row tile");
    static_assert(!PF || CW == GROUP_N, "prefetched epilogue operands cover a full group");
    static_assert(CW == GROUP_N || (WN == 1 && EPI != EPI_SWIGLU), "half groups: one wave column, no SwiGLU");
    constexpr int MP = MT * 16;
    constexpr int GN = CW * WN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int M = e.M;
    // rs[m] = 1/sqrt(sum_g ss[m][g] / E + eps): 16 threads per row, each summing
    // groups sub, sub + 16, ... in order, then a fixed-order tree
    if ((EPI != EPI_RESID || !PF) && !RSR) {
        for (int m0 = 0; m0 < MP; m0 += 16) {
            const int m = m0 + (tid >> 4), sub = tid & 15;
            float part = 0.0f;
            if (PF && pre.ss_ok) {
#pragma unroll
                for (int j = 0; j < EpiPre::SSN; ++j) part += pre.ss[j];
            } else if (e.ss != nullptr && m < M) {
                for (int gg = sub; gg < e.ss_groups; gg += 16) part += e.ss[(size_t)m * e.ss_gs + gg];
            }
            for (int o = 8; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
            if (sub == 0) rs_s[m] = (e.ss != nullptr && m < M) ? 1.0f / sqrtf(part * e.inv_E + e.eps) : 1.0f;
        }
        __syncthreads();
    }

    const bool col_ok = CW == GROUP_N || lane < CW;
    if constexpr (EPI == EPI_SCALED) {
        const int n = g * CW + lane;
        const float sc = PF ? pre.sc : (e.wscale && col_ok ? e.wscale[n] : 1.0f);
        if (col_ok)
            for (int m = wave; m < M; m += 4) {
                float v = tile[m * GN + lane] * rs_s[m];
                if (e.wscale) v *= sc;
                st_f32(e.out + (size_t)m * e.ld_out + n, v);
            }
    } else if constexpr (EPI == EPI_RESID) {
        constexpr int RPW = MP / 4;  // rows per wave; all residual loads issued first
        const int n = g * CW + lane;
        float sc, wn;
        float xv[RPW];
        if constexpr (PF) {
            sc = pre.sc;
            wn = pre.wn;
#pragma unroll
            for (int r = 0; r < RPW; ++r) xv[r] = pre.x[r];
        } else {
            sc = e.wscale && col_ok ? e.wscale[n] : 1.0f;
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                const int m = wave + 4 * r;
                xv[r] = m < M && col_ok ? e.x[(size_t)m * e.ld_x + n] : 0.0f;
            }
            wn = col_ok ? e.wnext[n] : 0.0f;
        }
        float *xo = e.x_out ? e.x_out : e.x;
        // a whole 64-column group of 16 rows: the next projection's activations for k-block g are one
        // contiguous block (4 KB of f32 words, or 2 KB in each bf16 plane), staged in LDS and stored as
        // contiguous dwords
        constexpr bool STAGE_OK = MT == 1 && CW == GROUP_N;
        __shared__ uint32_t stage[STAGE_OK ? 6 * 256 : 1];
        const bool staged = STAGE_OK && M == 16 && (e.act_fmt == ACT_SPLIT3 || e.act_fmt == ACT_F32);
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const int m = wave + 4 * r;
            if (m < M) {
                const float xn = col_ok ? xv[r] + tile[m * GN + lane] * sc : 0.0f;
                if (col_ok) {
                    st_f32(xo + (size_t)m * e.ld_x + n, xn);
                    if (staged) {
                        const int ll = m + 16 * (lane / 16);
                        if (e.act_fmt == ACT_F32) {
                            stage[(((lane % 16) / 4) * 64 + ll) * 4 + lane % 4] = __float_as_uint(xn * wn);
                        } else {
                            uint16_t t[3];
                            split3(xn * wn, t[0], t[1], t[2]);
                            const int v = (lane % 16) / 8, i = lane % 8;
#pragma unroll
                            for (int p = 0; p < 3; ++p) ((uint16_t *)stage)[((p * 2 + v) * 64 + ll) * 8 + i] = t[p];
                        }
                    } else {
                        write_act(e.act_out, e.act_fmt, e.act_rows, e.act_K, m, n, xn * wn);
                    }
                }
                const float sq = wave_sum(xn * xn);
                if (lane == 0) st_f32(e.ss_out + (size_t)m * e.ss_gs + g, sq);
            }
        }
        if (staged) {
            __syncthreads();
            if (e.act_fmt == ACT_F32) {
                int32_t *dst = (int32_t *)e.act_out + (size_t)g * 1024;  // k-block g: 4 words x 64 lanes x 4
                for (int d = tid; d < 1024; d += 256) st_i32(dst + d, (int32_t)stage[d]);
            } else {
                const size_t plane = (size_t)e.act_rows * e.act_K;
                for (int d = tid; d < 3 * 512; d += 256) {  // plane p: 2 words x 64 lanes x 8 bf16
                    const int p = d / 512;
                    st_i32((int32_t *)((uint16_t *)e.act_out + (size_t)p * plane + (size_t)g * 1024) + d % 512,
                           (int32_t)stage[d]);
                }
            }
        }
    } else if constexpr (EPI == EPI_SWIGLU) {
        const float sg = PF ? pre.sc : (e.wscale && lane < 32 ? e.wscale[g * GROUP_N + lane] : 1.0f);
        const float su = PF ? pre.sc2 : (e.wscale && lane < 32 ? e.wscale[g * GROUP_N + 32 + lane] : 1.0f);
        if constexpr (MT == 1 && CW == GROUP_N) {
            if (M == 16 && (e.act_fmt == ACT_SPLIT3 || e.act_fmt == ACT_F32)) {
                // The group's 16 x 32 outputs in the lane-ordered layout are runs of 32 16-byte words
                // (word v of k-block g / 2, lanes 32 (g % 2) ..): f32, 4 words per lane; three bf16
                // planes, 2 words per lane each. They are staged in LDS in that order, then stored as
                // contiguous dwords instead of one store per value (and term).
                __shared__ uint32_t stage[6 * 128];
                const bool f32 = e.act_fmt == ACT_F32;
                for (int m = wave; m < 16; m += 4) {
                    if (lane < 32) {
                        float gv = tile[m * GN + lane] * rs_s[m];
                        float uv = tile[m * GN + lane + 32] * rs_s[m];
                        if (e.wscale) {
                            gv *= sg;
                            uv *= su;
                        }
                        const float act = gv / (1.0f + expf(-gv)) * uv;
                        const int ll = m + 16 * (lane / 16);
                        if (f32) {
                            stage[(((lane % 16) / 4) * 32 + ll) * 4 + lane % 4] = __float_as_uint(act);
                        } else {
                            uint16_t t[3];
                            split3(act, t[0], t[1], t[2]);
                            const int v = (lane % 16) / 8, i = lane % 8;
#pragma unroll
                            for (int p = 0; p < 3; ++p) ((uint16_t *)stage)[((p * 2 + v) * 32 + ll) * 8 + i] = t[p];
                        }
                    }
                }
                __syncthreads();
                const int kb = g / 2, h = g % 2;
                if (f32) {
                    for (int d = tid; d < 4 * 128; d += 256) {  // run v: 128 floats
                        const int v = d / 128;
                        const size_t el = (((size_t)kb * 4 + v) * 64 + 32 * h) * 4 + d % 128;
                        st_i32((int32_t *)e.act_out + el, (int32_t)stage[d]);
                    }
                } else {
                    const size_t plane = (size_t)e.act_rows * e.act_K;
                    for (int d = tid; d < 6 * 128; d += 256) {  // run (p, v): 128 dwords
                        const int run = d / 128, p = run / 2, v = run % 2;
                        const size_t el = (size_t)p * plane + (((size_t)kb * 2 + v) * 64 + 32 * h) * 8;
                        st_i32((int32_t *)((uint16_t *)e.act_out + el) + d % 128, (int32_t)stage[d]);
                    }
                }
                return;
            }
        }
        for (int m = wave; m < M; m += 4) {
            if (lane < 32) {
                float gv = tile[m * GN + lane] * rs_s[m];
                float uv = tile[m * GN + lane + 32] * rs_s[m];
                if (e.wscale) {
                    gv *= sg;
                    uv *= su;
                }
                const float act = gv / (1.0f + expf(-gv)) * uv;
                write_act(e.act_out, e.act_fmt, e.act_rows, e.act_K, m, g * 32 + lane, act);
            }
        }
    } else {  // EPI_LOGITS
        const int n = g * CW + lane;
        const float sc = PF ? pre.sc : (e.wscale && col_ok ? e.wscale[n] : 1.0f);
        for (int m = wave; m < M; m += 4) {
            const int mg = e.row0 + m;  // row within the step
            float v = -INFINITY;
            if (col_ok) {
                v = tile[m * GN + lane] * rs_s[m];
                if (e.wscale) v *= sc;
                st_f32(e.out + (size_t)m * e.ld_out + n, v);
                if (e.temp > 0.0f) {  // the draft is a sample: the argmax runs on logit / T + Gumbel noise
                    const int b = mg / e.block;
                    v = v / e.temp + gumbel_noise(e.seed_lo, e.seed_hi, b, e.n_past[b] + mg % e.block, n);
                }
            }
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
            if (lane == 0)
                __hip_atomic_store(e.am_key + (size_t)g * e.ss_stride + mg, argmax_key(bv, bi), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        argmax_finish<ATILE>(e, G, flag_s, best_s);
    }
}
