// Persistent weight-streaming chain of the DFlash drafter block step (one
// sequence).
//
// Run as one kernel each, the weight-streaming projections of a layer pay at
// every boundary for a launch, for the ramp of the next kernel's first loads
// and for the tail of the previous kernel's split-K epilogues, while HBM sits
// partly idle. Here one launch of exactly as many workgroups as the GPU holds
// at once runs a chain of consecutive phases (Wo, gate/up, down and the next
// layer's q/k/v, or the lm_head) separated by grid-wide barriers; before a
// workgroup waits at a barrier it already issues the weight loads of its first
// piece of work in the next phase, so HBM keeps streaming while the last
// epilogues and the barrier complete.
//
// A phase is split "stream-K" style: its G column groups x KB k-blocks form
// one list of units, and workgroup w takes the contiguous units
// [w*U/n, (w+1)*U/n), so every workgroup streams the same number of weight
// bytes. A column group spread over several workgroups is finished by the last
// of them to arrive, which sums the partials in workgroup order.
//
// The arithmetic and the epilogues are those of the per-launch kernels; only
// the split points of the reductions differ.
#include "gemv_device.h"

namespace {

// ---------------------------------------------------------------------------
// Grid barrier
// ---------------------------------------------------------------------------
// The calling thread's earlier stores are complete (written through to
// memory) once this returns.
__device__ __forceinline__ void stores_done() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Arrive and wait until `target` arrivals have been counted. Every wait ends:
// after a.spin_ticks of wall clock the workgroup raises a.err and gives up,
// and a workgroup that sees a.err raised gives up too. Returns false then.
__device__ __forceinline__ bool grid_wait(const PStepArgs &a, unsigned target, int *flag_s) {
    __syncthreads();
    if (threadIdx.x == 0) {
        int ok = 1;
        __hip_atomic_fetch_add(a.bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const long long t0 = wall_clock64();
        while (__hip_atomic_load(a.bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (__hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0 ||
                wall_clock64() - t0 > a.spin_ticks) {
                __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        *flag_s = ok;
    }
    __syncthreads();
    return *flag_s != 0;
}

// ---------------------------------------------------------------------------
// Stream-K partition of a weight-streaming phase
// ---------------------------------------------------------------------------
// A phase of U units uses n = min(nWG, U) workgroups, so every one of them owns at least one unit;
// workgroups w >= n skip the phase (they still take part in the grid barriers).
__device__ __forceinline__ int sk_workers(int nWG, long U) { return U < nWG ? (int)U : nWG; }
__device__ __forceinline__ long sk_begin(int w, int n, long U) { return (long)w * U / n; }
// the workgroup whose units contain unit u
__device__ __forceinline__ int sk_owner(long u, int n, long U) { return (int)(((u + 1) * n - 1) / U); }

// Issue the weight loads of this wave's first k-block of the workgroup's first
// piece of a phase over W [N, K] with 64*WN-column groups; ok says whether
// there is one.
template <int WT, int WN>
__device__ __forceinline__ void sk_prefetch(const void *W, int N, int K, int wg, int nWG,
                                            u32x4 (&pf)[4][WTraits<WT>::NV], bool &ok) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wn = wave % WN, wk = wave / WN;
    const int G = N / (GROUP_N * WN), KB = K / KBLK;
    const long U = (long)G * KB;
    const int n = sk_workers(nWG, U);
    ok = false;
    if (wg >= n) return;
    const long u0 = sk_begin(wg, n, U), u1 = sk_begin(wg + 1, n, U);
    const int g = (int)(u0 / KB), ka = (int)(u0 - (long)g * KB);
    const int kbb = (int)(min(u1, (long)(g + 1) * KB) - (long)g * KB);
    const int kb = ka + wk;
    if (kb >= kbb) return;
#pragma unroll
    for (int t = 0; t < 4; ++t) load_wtile<WT>(W, ((size_t)g * KB + kb) * 4 * WN + 4 * wn + t, lane, pf[t]);
    ok = true;
}

// One weight-streaming phase: y = act . W^T for the 16 block rows with the EPI
// epilogue. LDS: tile [16][64*WN] f32, rs [16], best [16], flag.
template <int WT, int AF, int EPI, int WN>
__device__ __forceinline__ void sk_gemv(const void *W, int N, int K, const void *act, int act_rows, const EpiArgs &e,
                                        float *partial, int pmax, int *counters, int wg, int nWG, char *lds,
                                        const u32x4 (&pf)[4][WTraits<WT>::NV], bool pf_ok) {
    constexpr int NV = WTraits<WT>::NV;
    constexpr int NW = AFTraits<AF>::NW;
    constexpr int GN = GROUP_N * WN, WK = 4 / WN, TE = 16 * GN;
    float *tile = (float *)lds;
    float *rs_s = tile + TE;
    int *best_s = (int *)(rs_s + 16);
    int *flag_s = best_s + 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wn = wave % WN, wk = wave / WN;
    const int G = N / GN, KB = K / KBLK;
    const long U = (long)G * KB;
    const int n = sk_workers(nWG, U);
    if (wg >= n) return;
    const long u0 = sk_begin(wg, n, U), u1 = sk_begin(wg + 1, n, U);
    bool first = true;
    for (long u = u0; u < u1;) {
        const int g = (int)(u / KB), ka = (int)(u - (long)g * KB);
        const int kbb = (int)(min(u1, (long)(g + 1) * KB) - (long)g * KB);
        f32x4 acc[1][4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[0][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        int kb = ka + wk;
        if (first && pf_ok && kb < kbb) {
            u32x4 av[NW];
            load_act_lanes<AF>(act, act_rows, K, 0, true, kb, lane, av);
#pragma unroll
            for (int t = 0; t < 4; ++t) tile_mfma<WT, AF>(pf[t], av, acc[0][t]);
            kb += WK;
        }
        first = false;
        for (; kb < kbb; kb += WK) {
            u32x4 w[4][NV];
#pragma unroll
            for (int t = 0; t < 4; ++t) load_wtile<WT>(W, ((size_t)g * KB + kb) * 4 * WN + 4 * wn + t, lane, w[t]);
            u32x4 av[NW];
            load_act_lanes<AF>(act, act_rows, K, 0, true, kb, lane, av);
#pragma unroll
            for (int t = 0; t < 4; ++t) tile_mfma<WT, AF>(w[t], av, acc[0][t]);
        }
        reduce_waves<1, WN>(acc, tile, wn, wk, lane);
        const int first_wg = sk_owner((long)g * KB, n, U);
        const int np = sk_owner((long)(g + 1) * KB - 1, n, U) - first_wg + 1;
        bool done = true;
        if (np > 1)
            done = splitk_last<TE / 256>(tile, partial + ((size_t)g * pmax + (wg - first_wg)) * TE,
                                         partial + (size_t)g * pmax * TE, TE, np, counters + g, flag_s);
        if (done) gemv_epilogue<EPI, 1, WN>(e, g, G, tile, rs_s, flag_s, best_s);
        __syncthreads();
        u = (long)(g + 1) * KB;
    }
}

// ---------------------------------------------------------------------------
// Embedding of the noise block [id_last, mask x (block-1)] (dflash-ops card,
// Usage), the first layer's norm input and statistics, and the block's rope
// table (fp64 angles and sincos, rounded to f32)
// ---------------------------------------------------------------------------
__device__ __forceinline__ void embed_group(const PStepArgs &a, const PStepIO &io, int g) {
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
        if (lane == 0) st_f32(a.ss_a + (size_t)g * a.ss_stride + i, sq);
    }
}

__device__ __forceinline__ void rope_table(const PStepArgs &a, const PStepIO &io) {
    const int half = a.D / 2;
    for (int idx = threadIdx.x; idx < a.block * half; idx += 256) {
        const int i = idx / half, f = idx % half;
        const double theta = (double)(io.n_past[0] + i) * a.inv_freq[f];
        double sn, cn;
        sincos(theta, &sn, &cn);
        st_f32(a.rope_cs + ((size_t)i * half + f) * 2, (float)cn);
        st_f32(a.rope_cs + ((size_t)i * half + f) * 2 + 1, (float)sn);
    }
}

// ---------------------------------------------------------------------------
// Phases
// ---------------------------------------------------------------------------
__device__ __forceinline__ EpiArgs epi_base(const PStepArgs &a, int kind) {
    EpiArgs e = {};
    e.kind = kind;
    e.M = 16;
    e.ss_stride = a.ss_stride;
    e.inv_E = a.inv_E;
    e.eps = a.eps;
    e.block = a.block;
    e.gamma = a.block;  // the persistent chain runs full-width blocks only
    e.act_rows = a.act_rows;
    e.act_fmt = a.act_fmt;
    return e;
}

// q/k/v of layer l with the attention norm folded in (the attention kernel norms and ropes q and k)
template <int WT, int AF>
__device__ __forceinline__ void phase_qkv(const PStepArgs &a, int l, int wg, int nWG, char *lds,
                                          const u32x4 (&pf)[4][WTraits<WT>::NV], bool pok) {
    EpiArgs e = epi_base(a, EPI_SCALED);
    e.wscale = a.layer[l].s_qkv;
    e.ss = a.ss_a;
    e.ss_groups = a.G_E;
    e.out = a.qkv_out;
    e.ld_out = a.nqkv;
    sk_gemv<WT, AF, EPI_SCALED, 1>(a.layer[l].qkv, a.nqkv, a.E, a.act_a, a.act_rows, e, a.partial, a.pmax[0],
                                   a.counters, wg, nWG, lds, pf, pok);
}

}  // namespace

// Embedding and rope table, then the q/k/v projection of layer 0.
template <int WT, int AF>
__device__ __forceinline__ void chain_head(const PStepArgs *__restrict__ ap, const PStepIO &io) {
    __shared__ __attribute__((aligned(16))) char lds[4 * (16 * 64 + 16 + 16 + 4)];
    __shared__ int bar_flag;
    constexpr int NV = WTraits<WT>::NV;
    const PStepArgs &a = *ap;
    const int wg = blockIdx.x, nWG = gridDim.x;
    u32x4 pf[4][NV];
    bool pok = false;
    for (int g = wg; g < a.G_E; g += nWG) embed_group(a, io, g);
    if (wg == nWG - 1) rope_table(a, io);
    stores_done();
    sk_prefetch<WT, 1>(a.layer[0].qkv, a.nqkv, a.E, wg, nWG, pf, pok);
    if (!grid_wait(a, (unsigned)nWG, &bar_flag)) return;
    phase_qkv<WT, AF>(a, 0, wg, nWG, lds, pf, pok);
}

// Layer l after its attention: Wo (+ residual), gate/up (+ SwiGLU), down (+ residual), then the q/k/v
// projection of layer l + 1, or (LAST) the lm_head with argmax and acceptance. bar_base = grid barriers
// passed earlier in the step. Every buffer a phase writes is written once per launch and read only by
// later phases or later launches, so no workgroup reads a stale cached copy.
template <int WT, int AF, bool LAST>
__device__ __forceinline__ void chain_layer(const PStepArgs *__restrict__ ap, const PStepIO &io, int l,
                                            unsigned bar_base) {
    __shared__ __attribute__((aligned(16))) char lds[4 * (16 * 64 + 16 + 16 + 4)];
    __shared__ int bar_flag;
    constexpr int NV = WTraits<WT>::NV;
    const PStepArgs &a = *ap;
    const int wg = blockIdx.x, nWG = gridDim.x;
    const PLayer &P = a.layer[l];
    u32x4 pf[4][NV];
    bool pok = false;
    unsigned nb = bar_base;
    {  // Wo + residual into x2; the ffn norm's input and statistics
        EpiArgs e = epi_base(a, EPI_RESID);
        e.wscale = P.s_o;
        e.x = a.x;
        e.x_out = a.x2;
        e.ld_x = a.E;
        e.wnext = a.ffn_norm + (size_t)l * a.E;
        e.act_out = a.act_f;
        e.act_K = a.E;
        e.ss_out = a.ss_f;
        sk_gemv<WT, AF, EPI_RESID, 1>(P.o, a.E, a.qdim, a.act_o, a.act_rows, e, a.partial, a.pmax[1], a.counters, wg,
                                      nWG, lds, pf, pok);
    }
    stores_done();
    sk_prefetch<WT, 1>(P.gu, 2 * a.F, a.E, wg, nWG, pf, pok);
    if (!grid_wait(a, ++nb * (unsigned)nWG, &bar_flag)) return;
    {  // gate/up with the ffn norm folded in; SwiGLU
        EpiArgs e = epi_base(a, EPI_SWIGLU);
        e.wscale = P.s_gu;
        e.ss = a.ss_f;
        e.ss_groups = a.G_E;
        e.act_out = a.act_d;
        e.act_K = a.F;
        sk_gemv<WT, AF, EPI_SWIGLU, 1>(P.gu, 2 * a.F, a.E, a.act_f, a.act_rows, e, a.partial, a.pmax[2], a.counters,
                                       wg, nWG, lds, pf, pok);
    }
    stores_done();
    sk_prefetch<WT, 1>(P.down, a.E, a.F, wg, nWG, pf, pok);
    if (!grid_wait(a, ++nb * (unsigned)nWG, &bar_flag)) return;
    {  // down + residual back into x; the next attention-norm (or output-norm) input
        EpiArgs e = epi_base(a, EPI_RESID);
        e.wscale = P.s_down;
        e.x = a.x2;
        e.x_out = a.x;
        e.ld_x = a.E;
        e.wnext = LAST ? a.output_norm : a.attn_norm + (size_t)(l + 1) * a.E;
        e.act_out = a.act_a;
        e.act_K = a.E;
        e.ss_out = a.ss_a;
        sk_gemv<WT, AF, EPI_RESID, 1>(P.down, a.E, a.F, a.act_d, a.act_rows, e, a.partial, a.pmax[3], a.counters, wg,
                                      nWG, lds, pf, pok);
    }
    stores_done();
    if (LAST)
        sk_prefetch<WT, 1>(a.lm, a.V, a.E, wg, nWG, pf, pok);
    else
        sk_prefetch<WT, 1>(a.layer[l + 1].qkv, a.nqkv, a.E, wg, nWG, pf, pok);
    if (!grid_wait(a, ++nb * (unsigned)nWG, &bar_flag)) return;
    if (LAST) {  // output norm folded in; lm_head, argmax of rows 1..15, acceptance scan
        EpiArgs e = epi_base(a, EPI_LOGITS);
        e.wscale = a.s_lm;
        e.ss = a.ss_a;
        e.ss_groups = a.G_E;
        e.out = io.logits;
        e.ld_out = a.V;
        e.am_val = a.am_val;
        e.am_idx = a.am_idx;
        e.am_counter = a.am_counter;
        e.drafts = io.drafts;
        e.target = io.target;
        e.n_ok = io.n_ok;
        sk_gemv<WT, AF, EPI_LOGITS, 1>(a.lm, a.V, a.E, a.act_a, a.act_rows, e, a.partial, a.pmax[4], a.counters, wg,
                                       nWG, lds, pf, pok);
    } else {
        phase_qkv<WT, AF>(a, l + 1, wg, nWG, lds, pf, pok);
    }
}

template <int WT, int AF>
__global__ __launch_bounds__(256) void pchain_head_kernel(const PStepArgs *__restrict__ ap, PStepIO io) {
    chain_head<WT, AF>(ap, io);
}
template <int WT, int AF, bool LAST>
__global__ __launch_bounds__(256) void pchain_layer_kernel(const PStepArgs *__restrict__ ap, PStepIO io, int l,
                                                           unsigned bar_base) {
    chain_layer<WT, AF, LAST>(ap, io, l, bar_base);
}
// bf16 weights fit three workgroups per CU without spills (fp8 with its software decode, and f32, take two)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void
pchain_head_bf16_kernel(const PStepArgs *__restrict__ ap, PStepIO io) {
    chain_head<DFLASH_BF16, ACT_SPLIT3>(ap, io);
}
template <bool LAST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void
pchain_layer_bf16_kernel(const PStepArgs *__restrict__ ap, PStepIO io, int l, unsigned bar_base) {
    chain_layer<DFLASH_BF16, ACT_SPLIT3, LAST>(ap, io, l, bar_base);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

typedef void (*head_fn)(const PStepArgs *, PStepIO);
typedef void (*layer_fn)(const PStepArgs *, PStepIO, int, unsigned);

struct ChainFns {
    head_fn head;
    layer_fn mid, last;
};

ChainFns pick(const dflash_ctx *c) {
    switch (c->cfg.weight_dtype) {
        case DFLASH_F32:
            return {pchain_head_kernel<DFLASH_F32, ACT_F32>, pchain_layer_kernel<DFLASH_F32, ACT_F32, false>,
                    pchain_layer_kernel<DFLASH_F32, ACT_F32, true>};
        case DFLASH_BF16:
            return {pchain_head_bf16_kernel, pchain_layer_bf16_kernel<false>, pchain_layer_bf16_kernel<true>};
        case DFLASH_FP8_E4M3:
            return {pchain_head_kernel<DFLASH_FP8_E4M3, ACT_SPLIT3>,
                    pchain_layer_kernel<DFLASH_FP8_E4M3, ACT_SPLIT3, false>,
                    pchain_layer_kernel<DFLASH_FP8_E4M3, ACT_SPLIT3, true>};
        default: return {nullptr, nullptr, nullptr};
    }
}

}  // namespace

int pchain_grid(const dflash_ctx *c) {
    const ChainFns f = pick(c);
    if (!f.head || c->L > PSTEP_MAX_LAYERS) return 0;
    int cus = 0, per_cu = 1 << 20;
    for (const void *k : {(const void *)f.head, (const void *)f.mid, (const void *)f.last}) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, 256, 0) != hipSuccess) return 0;
        per_cu = per_cu < n ? per_cu : n;
    }
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, c->device) != hipSuccess) return 0;
    if (per_cu < 1 || cus < 1) return 0;
    const int n = per_cu * cus;
    return n > PSTEP_MAX_WG ? PSTEP_MAX_WG : n;
}

hipError_t launch_pchain_head(const dflash_ctx *c, const PStepArgs *dev_args, const PStepIO &io, int nWG,
                              hipStream_t s) {
    const ChainFns f = pick(c);
    if (!f.head) return hipErrorInvalidValue;
    hipLaunchKernelGGL(f.head, dim3(nWG), dim3(256), 0, s, dev_args, io);
    return hipGetLastError();
}

hipError_t launch_pchain_layer(const dflash_ctx *c, const PStepArgs *dev_args, const PStepIO &io, int l,
                               unsigned bar_base, int nWG, hipStream_t s) {
    const ChainFns f = pick(c);
    if (!f.head) return hipErrorInvalidValue;
    hipLaunchKernelGGL(l + 1 == c->L ? f.last : f.mid, dim3(nWG), dim3(256), 0, s, dev_args, io, l, bar_base);
    return hipGetLastError();
}
