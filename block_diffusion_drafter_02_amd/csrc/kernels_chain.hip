// Dataflow chain of the DFlash drafter block step (one sequence).
//
// Run as one kernel each, the weight-streaming projections of a layer pay at
// every boundary for the drain of the previous kernel (its last split-K
// handshakes and epilogues), for the launch itself and for the ramp of the
// next kernel's first loads, while HBM sits partly idle. Here the projections
// between two attention launches (Wo, gate/up, down and the next layer's
// q/k/v, or the lm_head) run as one launch of exactly as many workgroups as
// the GPU holds at once. Workgroup w takes item w of every phase in turn: one
// 64-column group and one k-split of that projection, the same decomposition
// as the per-launch kernels. An item
//   1. issues the weight loads of its first k-block (weights never depend on
//      earlier phases),
//   2. waits until the column groups that produce its k-slice of the input
//      activation have published their done flags (64-column producers map
//      one group to one k-block; the SwiGLU producer writes 32 columns per
//      group, so two groups per k-block),
//   3. streams its k-blocks through the MFMA loop of the per-launch kernel,
//   4. meets the other k-splits of its group in the last-arriver handshake;
//      the last arriver waits for every producer group when its epilogue needs
//      their norm statistics, runs the fused epilogue, and publishes the
//      group's done flag.
// Because every workgroup is resident and takes its items in phase order, a
// wait only ever depends on items of earlier phases held by running
// workgroups, so it always ends; it is still bounded in wall-clock time and
// raises a sticky error word if it gives up (then the step's outputs are
// invalid and dflash_check_device reports it).
//
// A flag holds the epoch of the step that set it; the workgroup that finishes
// the lm_head's argmax advances the epoch, so flags never need clearing.
// Every buffer a launch writes is written once in that launch (the residual
// stream alternates between x and x2) and read only after its producer's
// flag, with device-coherent stores on the producer side, so no reader meets
// a stale cached copy.
//
// The arithmetic and the epilogues are those of the per-launch kernels; with
// the same k-split counts the results are bitwise the same.
#include "gemv_device.h"

namespace {

// The calling thread's earlier stores are complete (written through to
// memory) once this returns.
__device__ __forceinline__ void stores_done() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait (wave 0 polls, the workgroup then agrees) until flags[first .. first +
// count) all hold `ep`. Gives up after a.spin_ticks of wall clock, or at once
// when another workgroup has already given up; then raises the sticky error
// and returns false, the same value in every thread.
__device__ __forceinline__ bool wait_flags(const ChainArgs &a, const int *flags, int first, int count, unsigned ep,
                                           int *ok_s) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int ok = 1;
        const long long t0 = wall_clock64();
        for (int base = 0; base < count && ok; base += 64) {
            const int i = base + lane;
            while (true) {
                const bool mine = i >= count || (unsigned)__hip_atomic_load(flags + first + i, __ATOMIC_RELAXED,
                                                                             __HIP_MEMORY_SCOPE_AGENT) == ep;
                if (__all(mine)) break;
                if (__hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0 ||
                    wall_clock64() - t0 > a.spin_ticks) {
                    if (lane == 0) __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    ok = 0;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        if (lane == 0) *ok_s = ok;
    }
    __syncthreads();
    return *ok_s != 0;
}

// Publish column group g of a phase: every thread's output stores are complete
// before one thread stores the epoch into the group's flag.
__device__ __forceinline__ void publish(int *flags, int g, unsigned ep) {
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(flags + g, (int)ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct ChainLds {
    float tile[16 * GROUP_N];
    float rs[16];
    int best[16];
    int flag;
    int ok;
};

// One item of a weight-streaming phase: column group g = w / S, k-split s = w % S of y = act . W^T for the
// 16 block rows, with the EPI epilogue. dep: flags of the producers of the input activation, dep_mul of
// them per k-block (null: produced by an earlier launch). epi_dep: epi_dep_n flags that must all be set
// before the epilogue (null: none). done: this phase's flags (null: nobody in this launch waits for them).
// Returns false when a wait gave up.
template <int WT, int AF, int EPI>
__device__ __forceinline__ bool chain_item(const ChainArgs &a, unsigned ep, int w, const void *W, int N, int K,
                                           const void *act, int S, float *partial, int *counters, const int *dep,
                                           int dep_mul, const int *epi_dep, int epi_dep_n, int *done,
                                           const EpiArgs &e, ChainLds &sh) {
    constexpr int NV = WTraits<WT>::NV;
    constexpr int AFO = ActOp<WT, AF>::AFO;  // MFMA operand format (f32 words split at load)
    constexpr int NW = AFTraits<AFO>::NW;
    constexpr int TE = 16 * GROUP_N;
    const int G = N / GROUP_N, KB = K / KBLK;
    if (w >= G * S) return true;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = w / S, s = w % S;
    const int kbps = (KB + S - 1) / S;
    const int kb0 = s * kbps, kb1 = min(KB, kb0 + kbps);
    int kb = kb0 + wave;
    u32x4 wt[4][NV];
    if (kb < kb1) {
#pragma unroll
        for (int t = 0; t < 4; ++t) load_wtile<WT>(W, ((size_t)g * KB + kb) * 4 + t, lane, wt[t]);
    }
    if (dep != nullptr && !wait_flags(a, dep, kb0 * dep_mul, (kb1 - kb0) * dep_mul, ep, &sh.ok)) return false;
    f32x4 acc[1][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[0][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (kb < kb1) {
        u32x4 av[NW];
        load_act_operands<WT, AF>(act, a.act_rows, K, 0, true, kb, lane, av);
#pragma unroll
        for (int t = 0; t < 4; ++t) tile_mfma<WT, AFO>(wt[t], av, acc[0][t]);
        for (kb += 4; kb < kb1; kb += 4) {
#pragma unroll
            for (int t = 0; t < 4; ++t) load_wtile<WT>(W, ((size_t)g * KB + kb) * 4 + t, lane, wt[t]);
            load_act_operands<WT, AF>(act, a.act_rows, K, 0, true, kb, lane, av);
#pragma unroll
            for (int t = 0; t < 4; ++t) tile_mfma<WT, AFO>(wt[t], av, acc[0][t]);
        }
    }
    reduce_waves<1, 1>(acc, sh.tile, 0, wave, lane);
    if (S > 1 && !splitk_last<TE / 256>(sh.tile, partial + ((size_t)s * G + g) * TE, partial + (size_t)g * TE,
                                        (size_t)G * TE, S, counters + g, &sh.flag))
        return true;
    if (epi_dep != nullptr && !wait_flags(a, epi_dep, 0, epi_dep_n, ep, &sh.ok)) return false;
    gemv_epilogue<EPI, 1, 1>(e, g, G, sh.tile, sh.rs, &sh.flag, sh.best);
    if constexpr (EPI == EPI_LOGITS) {
        // the workgroup that completed the argmax of every row ends the step: advance the epoch (never 0,
        // the value of flags that were never set)
        if (sh.flag && threadIdx.x == 0) {
            const unsigned nx = ep + 1u == 0u ? 1u : ep + 1u;
            __hip_atomic_store(a.epoch, nx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (done != nullptr) publish(done, g, ep);
    __syncthreads();  // the tile and flag words are reused by the next item
    return true;
}

__device__ __forceinline__ EpiArgs epi_base(const ChainArgs &a, const ChainIO &io, int kind) {
    EpiArgs e = {};
    e.kind = kind;
    e.M = 16;
    e.ss_stride = a.ss_stride;
    e.ss_gs = a.ss_gs;
    e.inv_E = a.inv_E;
    e.eps = a.eps;
    e.block = a.block;
    e.gamma = io.gamma;
    e.act_rows = a.act_rows;
    e.act_fmt = a.act_fmt;
    return e;
}

// q/k/v of layer l with the attention norm folded in (the attention kernel norms and ropes q and k); its
// input act_a and norm statistics ss_a come from the column groups whose flags are `dep` (the embedding,
// or the previous layer's down projection).
template <int WT, int AF>
__device__ __forceinline__ bool phase_qkv(const ChainArgs &a, const ChainIO &io, unsigned ep, int w, int l,
                                          const int *dep, ChainLds &sh) {
    EpiArgs e = epi_base(a, io, EPI_SCALED);
    e.wscale = a.layer[l].s_qkv;
    e.ss = a.ss_a;
    e.ss_groups = a.G_E;
    e.out = a.qkv_out;
    e.ld_out = a.nqkv;
    return chain_item<WT, AF, EPI_SCALED>(a, ep, w, a.layer[l].qkv, a.nqkv, a.E, a.act_a, a.S[CS_QKV],
                                          a.partial[CS_QKV], a.counters[CS_QKV], dep, 1, dep, a.G_E, nullptr, e, sh);
}

// Embedding of the noise block [id_last, mask x (block-1)] (dflash-ops card, Usage) for column group g: x,
// the first layer's norm input and the group's sums of squares.
__device__ __forceinline__ void embed_group(const ChainArgs &a, const ChainIO &io, int g) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = g * GROUP_N + lane;
    for (int i = wave; i < a.block; i += 4) {
        const int id = io.block_ids ? io.block_ids[i] : (i == 0 ? io.id_last[0] : a.mask_id);
        float v = 0.0f;
        if (id >= 0 && id < a.V) {
            const size_t off = (size_t)id * a.E + n;
            v = a.aux_dtype == DFLASH_BF16 ? bf16_to_f32(((const uint16_t *)a.tok_embd)[off])
                                           : ((const float *)a.tok_embd)[off];
        }
        st_f32(a.x + (size_t)i * a.E + n, v);
        write_act(a.act_a, a.act_fmt, a.act_rows, a.E, i, n, v * a.attn_norm[n]);
        const float sq = wave_sum(v * v);
        if (lane == 0) st_f32(a.ss_a + (size_t)i * a.ss_gs + g, sq);
    }
}

}  // namespace

// Head launch: embedding (one item per 64-column group), the block's rope table (fp64 angles and sincos,
// rounded to f32, spread one entry per thread), then the q/k/v projection of layer 0.
template <int WT, int AF>
__device__ __forceinline__ void chain_head(const ChainArgs *__restrict__ ap, const ChainIO &io) {
    __shared__ ChainLds sh;
    const ChainArgs &a = *ap;
    const int w = blockIdx.x;
    const unsigned ep = __hip_atomic_load(a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int half = a.D / 2;
    for (int idx = w * CHAIN_THREADS + threadIdx.x; idx < a.block * half; idx += gridDim.x * CHAIN_THREADS) {
        const int i = idx / half, f = idx % half;
        const double theta = (double)(io.n_past[0] + i) * a.inv_freq[f];
        double sn, cn;
        sincos(theta, &sn, &cn);
        a.rope_cs[((size_t)i * half + f) * 2] = (float)cn;
        a.rope_cs[((size_t)i * half + f) * 2 + 1] = (float)sn;
    }
    if (w < a.G_E) {
        embed_group(a, io, w);
        publish(a.done_embed, w, ep);
    }
    phase_qkv<WT, AF>(a, io, ep, w, 0, a.done_embed, sh);
}

// Layer l after its attention: Wo (+ residual into x2), gate/up (+ SwiGLU), down (+ residual back into x),
// then the q/k/v projection of layer l + 1, or (LAST) the lm_head with argmax and acceptance.
template <int WT, int AF, bool LAST>
__device__ __forceinline__ void chain_layer(const ChainArgs *__restrict__ ap, const ChainIO &io, int l) {
    __shared__ ChainLds sh;
    const ChainArgs &a = *ap;
    const int w = blockIdx.x;
    const unsigned ep = __hip_atomic_load(a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const ChainLayer &P = a.layer[l];
    const int G_GU = 2 * a.F / GROUP_N;
    int *done_o = a.done_o + (size_t)l * a.G_E;
    int *done_gu = a.done_gu + (size_t)l * G_GU;
    int *done_down = a.done_down + (size_t)l * a.G_E;
    {  // Wo + residual into x2; the ffn norm's input and statistics (its input comes from the attention launch)
        EpiArgs e = epi_base(a, io, EPI_RESID);
        e.wscale = P.s_o;
        e.x = a.x;
        e.x_out = a.x2;
        e.ld_x = a.E;
        e.wnext = a.ffn_norm + (size_t)l * a.E;
        e.act_out = a.act_f;
        e.act_K = a.E;
        e.ss_out = a.ss_f;
        if (!chain_item<WT, AF, EPI_RESID>(a, ep, w, P.o, a.E, a.qdim, a.act_o, a.S[CS_O], a.partial[CS_O],
                                           a.counters[CS_O], nullptr, 1, nullptr, 0, done_o, e, sh))
            return;
    }
    {  // gate/up with the ffn norm folded in; SwiGLU
        EpiArgs e = epi_base(a, io, EPI_SWIGLU);
        e.wscale = P.s_gu;
        e.ss = a.ss_f;
        e.ss_groups = a.G_E;
        e.act_out = a.act_d;
        e.act_K = a.F;
        if (!chain_item<WT, AF, EPI_SWIGLU>(a, ep, w, P.gu, 2 * a.F, a.E, a.act_f, a.S[CS_GU], a.partial[CS_GU],
                                            a.counters[CS_GU], done_o, 1, done_o, a.G_E, done_gu, e, sh))
            return;
    }
    {  // down + residual back into x; the next attention-norm (or output-norm) input and statistics
        EpiArgs e = epi_base(a, io, EPI_RESID);
        e.wscale = P.s_down;
        e.x = a.x2;
        e.x_out = a.x;
        e.ld_x = a.E;
        e.wnext = LAST ? a.output_norm : a.attn_norm + (size_t)(l + 1) * a.E;
        e.act_out = a.act_a;
        e.act_K = a.E;
        e.ss_out = a.ss_a;
        if (!chain_item<WT, AF, EPI_RESID>(a, ep, w, P.down, a.E, a.F, a.act_d, a.S[CS_DOWN], a.partial[CS_DOWN],
                                           a.counters[CS_DOWN], done_gu, 2, nullptr, 0, done_down, e, sh))
            return;
    }
    if constexpr (LAST) {  // output norm folded in; lm_head, argmax of rows 1..g-1, acceptance scan
        EpiArgs e = epi_base(a, io, EPI_LOGITS);
        e.wscale = a.s_lm;
        e.ss = a.ss_a;
        e.ss_groups = a.G_E;
        e.out = io.logits;
        e.ld_out = a.V;
        e.am_key = a.am_key;
        e.am_counter = a.am_counter;
        e.drafts = io.drafts;
        e.target = io.target;
        e.n_ok = io.n_ok;
        e.temp = io.temp;
        e.seed_lo = io.seed_lo;
        e.seed_hi = io.seed_hi;
        e.n_past = io.n_past;
        chain_item<WT, AF, EPI_LOGITS>(a, ep, w, a.lm, a.V, a.E, a.act_a, a.S[CS_LM], a.partial[CS_LM],
                                       a.counters[CS_LM], done_down, 1, done_down, a.G_E, nullptr, e, sh);
    } else {
        phase_qkv<WT, AF>(a, io, ep, w, l + 1, done_down, sh);
    }
}

template <int WT, int AF>
__global__ __launch_bounds__(CHAIN_THREADS) __attribute__((amdgpu_waves_per_eu(5))) void chain_head_kernel(const ChainArgs *__restrict__ ap, ChainIO io) {
    chain_head<WT, AF>(ap, io);
}
template <int WT, int AF, bool LAST>
__global__ __launch_bounds__(CHAIN_THREADS) __attribute__((amdgpu_waves_per_eu(5))) void chain_layer_kernel(const ChainArgs *__restrict__ ap, ChainIO io,
                                                                     int l) {
    chain_layer<WT, AF, LAST>(ap, io, l);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

typedef void (*head_fn)(const ChainArgs *, ChainIO);
typedef void (*layer_fn)(const ChainArgs *, ChainIO, int);

struct ChainFns {
    head_fn head;
    layer_fn mid, last;
};

ChainFns pick(const dflash_ctx *c) {
    switch (c->cfg.weight_dtype) {
        case DFLASH_F32:
            return {chain_head_kernel<DFLASH_F32, ACT_F32>, chain_layer_kernel<DFLASH_F32, ACT_F32, false>,
                    chain_layer_kernel<DFLASH_F32, ACT_F32, true>};
        case DFLASH_BF16:  // f32 activation words, split into the three bf16 terms at load
            return {chain_head_kernel<DFLASH_BF16, ACT_F32>, chain_layer_kernel<DFLASH_BF16, ACT_F32, false>,
                    chain_layer_kernel<DFLASH_BF16, ACT_F32, true>};
        case DFLASH_FP8_E4M3:
            return {chain_head_kernel<DFLASH_FP8_E4M3, ACT_F32>, chain_layer_kernel<DFLASH_FP8_E4M3, ACT_F32, false>,
                    chain_layer_kernel<DFLASH_FP8_E4M3, ACT_F32, true>};
        default: return {nullptr, nullptr, nullptr};
    }
}

}  // namespace

int chain_grid(const dflash_ctx *c) {
    const ChainFns f = pick(c);
    if (!f.head || c->L > CHAIN_MAX_LAYERS) return 0;
    int cus = 0, per_cu = 1 << 20;
    for (const void *k : {(const void *)f.head, (const void *)f.mid, (const void *)f.last}) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, CHAIN_THREADS, 0) != hipSuccess) return 0;
        per_cu = per_cu < n ? per_cu : n;
    }
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, c->device) != hipSuccess) return 0;
    if (per_cu < 1 || cus < 1) return 0;
    return per_cu * cus;
}

hipError_t launch_chain_head(const dflash_ctx *c, const ChainIO &io, hipStream_t s) {
    const ChainFns f = pick(c);
    if (!f.head || c->chain_wg < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(f.head, dim3(c->chain_wg), dim3(CHAIN_THREADS), 0, s, (const ChainArgs *)c->cargs, io);
    return hipGetLastError();
}

hipError_t launch_chain_layer(const dflash_ctx *c, const ChainIO &io, int l, hipStream_t s) {
    const ChainFns f = pick(c);
    if (!f.head || c->chain_wg < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(l + 1 == c->L ? f.last : f.mid, dim3(c->chain_wg), dim3(CHAIN_THREADS), 0, s,
                       (const ChainArgs *)c->cargs, io, l);
    return hipGetLastError();
}
