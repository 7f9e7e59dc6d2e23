// Internal declarations of the DFlash HIP library: device helpers, the weight
// tiling, the context layout and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "dflash.h"

// ---------------------------------------------------------------------------
// Tiling of streamed weights
// ---------------------------------------------------------------------------
// Every matrix the step streams is re-tiled once at create time so that every
// wavefront load instruction reads one contiguous kilobyte.
//
// A tile covers 16 output rows x 64 reduction columns (one "k-block"). Lane
// l (0..63) of a wavefront owns row (l % 16) and the 16 consecutive columns
// starting at 16 * (l / 16). A lane's 16 elements are cut into 16-byte words
// (es words of 16/es elements for an element size of es bytes); the tile
// stores word 0 of lanes 0..63, then word 1 of lanes 0..63, and so on. Four
// tiles side by side (64 output rows) form a column group; memory order is
// [group][k-block][tile 0..3][word][lane][16 bytes].
//
// The MFMA 16x16x32 bf16 operands take 8 reduction elements per lane, so a
// lane's two bf16 words feed two MFMAs; for f32 weights the four words feed
// sixteen 16x16x4 f32 MFMAs. The activation operand is laid out with the same
// lane -> (row, columns) map and the same word split, so any permutation of
// the reduction index inside a k-block cancels out.
constexpr int TILE_N = 16;
constexpr int KBLK = 64;
constexpr int TILES_PER_GROUP = 4;
constexpr int GROUP_N = TILE_N * TILES_PER_GROUP;  // 64 output columns per group
constexpr int LANE_ELEMS = 16;

// element offset of weight (n, k) in a tiled matrix with KB = K / 64 k-blocks, es-byte elements and tpg
// tiles per column group (4, or 8 for the q/k/v projection whose groups are 128 columns = one head)
__host__ __device__ inline size_t tiled_offset(int n, int k, int KB, int es, int tpg = TILES_PER_GROUP) {
    const int epw = 16 / es;  // elements per 16-byte word
    int g = n / (TILE_N * tpg), t = (n / TILE_N) % tpg, r = n % TILE_N;
    int kb = k / KBLK, c = (k % KBLK) / LANE_ELEMS, j = k % LANE_ELEMS;
    int lane = r + 16 * c, v = j / epw, i = j % epw;
    return (((((size_t)g * KB + kb) * tpg + t) * es + v) * 64 + lane) * epw + i;
}

// Activation operands of the block-row kernels use the same lane order: for
// row m, column k of a [rows][K] activation (rows a multiple of 16), element
// offset inside one plane. es = 2 (bf16 planes of the three-term split) or 4
// (f32). Plane p of a split activation starts at p * rows * K.
__host__ __device__ inline size_t act_offset(int m, int k, int K, int es) {
    const int epw = 16 / es;
    const int KB = K / KBLK;
    int mt = m / 16, r = m % 16, kb = k / KBLK, c = (k % KBLK) / LANE_ELEMS, j = k % LANE_ELEMS;
    int lane = r + 16 * c, v = j / epw, i = j % epw;
    return ((((size_t)mt * KB + kb) * es + v) * 64 + lane) * epw + i;
}

// ---------------------------------------------------------------------------
// Scalar conversions (device)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bfloat16, round to nearest even (finite inputs; NaN stays NaN)
// Round to nearest even (the hardware conversion; NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Exact three-term split v = t0 + t1 + t2 with each term a bfloat16. Each
// subtraction is exact (Sterbenz: the operands agree to within a factor of
// two), and the last remainder has at most 8 significant bits, so the three
// bf16 products with a bf16 weight reproduce the fp32 product exactly.
__device__ __forceinline__ void split3(float v, uint16_t &t0, uint16_t &t1, uint16_t &t2) {
    t0 = f32_to_bf16(v);
    float r = v - bf16_to_f32(t0);
    t1 = f32_to_bf16(r);
    r = r - bf16_to_f32(t1);
    t2 = f32_to_bf16(r);
}

// The same split of two values at once, each term packed as (a | b << 16):
// one packed conversion per term.
__device__ __forceinline__ void split3_pair(float a, float b, uint32_t &w0, uint32_t &w1, uint32_t &w2) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    const bf16x2_t h0 = bf16x2_t{(__bf16)a, (__bf16)b};
    const float ra = a - (float)h0[0], rb = b - (float)h0[1];
    const bf16x2_t h1 = bf16x2_t{(__bf16)ra, (__bf16)rb};
    const float sa = ra - (float)h1[0], sb = rb - (float)h1[1];
    const bf16x2_t h2 = bf16x2_t{(__bf16)sa, (__bf16)sb};
    w0 = __builtin_bit_cast(uint32_t, h0);
    w1 = __builtin_bit_cast(uint32_t, h1);
    w2 = __builtin_bit_cast(uint32_t, h2);
}

// E4M3FN code -> bfloat16 bits (exact: 3 mantissa bits and exponents
// 2^-9 .. 2^8 all fit bf16). The NaN code is not supported.
__device__ __forceinline__ uint16_t e4m3_to_bf16(uint32_t c) {
    uint32_t s = (c & 0x80u) << 8;
    uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
    if (e == 0) {
        if (m == 0) return (uint16_t)s;
        int p = 31 - __clz(m);  // m = 2^p * (1 + f), value m * 2^-9
        return (uint16_t)(s | ((uint32_t)(p - 9 + 127) << 7) | ((m << (7 - p)) & 0x7Fu));
    }
    return (uint16_t)(s | ((e + 120u) << 7) | (m << 4));
}

// fp32 -> E4M3FN code, round to nearest even, saturating at +-448.
__device__ __forceinline__ uint8_t f32_to_e4m3(float v) {
    uint32_t u = __float_as_uint(v);
    uint32_t s = (u >> 24) & 0x80u;
    float a = fabsf(v);
    if (!(a < 448.0f)) return (uint8_t)(s | 0x7Eu);  // >= 448 (and NaN) saturate
    if (a >= 0.015625f) {                             // normal: keep 3 mantissa bits
        uint32_t au = u & 0x7fffffffu;
        au += 0x7ffffu + ((au >> 20) & 1u);
        au &= 0xfff00000u;
        if (__uint_as_float(au) > 448.0f) return (uint8_t)(s | 0x7Eu);
        int e = (int)(au >> 23) - 127;
        return (uint8_t)(s | ((uint32_t)(e + 7) << 3) | ((au >> 20) & 7u));
    }
    float q = rintf(a * 512.0f);  // subnormal quantum 2^-9; q == 8 is the smallest normal
    return (uint8_t)(s | (uint32_t)q);
}

template <typename T>
__device__ __forceinline__ float load_f32(const T *p, size_t i);
template <>
__device__ __forceinline__ float load_f32<float>(const float *p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_f32<uint16_t>(const uint16_t *p, size_t i) { return bf16_to_f32(p[i]); }

__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// ---------------------------------------------------------------------------
// Activation formats for the weight-streaming kernels
// ---------------------------------------------------------------------------
// ACT_SPLIT3: three bf16 planes of [Mrows][K] (exact three-term split of fp32
//             values), used with bf16 and fp8 weights.
// ACT_F32:    f32 [Mrows][K], used with f32 weights (f32 MFMA).
// ACT_BF16:   bf16 [Mrows][K] holding exact values (features already bf16).
// The block-row kernels read lane-ordered planes (act_offset); the large-M
// GEMM of encode / inject reads row-major planes.
enum ActFmt { ACT_SPLIT3 = 0, ACT_F32 = 1, ACT_BF16 = 2 };

// Device-coherent (agent-scope) stores: written through to memory, so that a
// workgroup on another XCD reads the value in the same launch after a
// grid-wide handshake. Used for every activation a block-step kernel produces.
__device__ __forceinline__ void st_f32(float *p, float v) {
    __hip_atomic_store((uint32_t *)p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_i32(int32_t *p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u16(uint16_t *p, uint16_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_f32(const float *p) {
    return __uint_as_float(__hip_atomic_load((const uint32_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Write one activation value in the lane-ordered layout: f32, or the exact
// three-term bf16 split over three planes of act_rows * K elements.
__device__ __forceinline__ void write_act(void *act, int fmt, int act_rows, int K, int row, int col, float v) {
    if (fmt == ACT_F32) {
        st_f32((float *)act + act_offset(row, col, K, 4), v);
    } else {
        uint16_t t0, t1, t2;
        split3(v, t0, t1, t2);
        uint16_t *p = (uint16_t *)act;
        const size_t plane = (size_t)act_rows * K;
        const size_t o = act_offset(row, col, K, 2);
        st_u16(p + o, t0);
        st_u16(p + plane + o, t1);
        st_u16(p + 2 * plane + o, t2);
    }
}

// ---------------------------------------------------------------------------
// Epilogues of the split-K weight-streaming kernel
// ---------------------------------------------------------------------------
enum EpiKind { EPI_SCALED = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };

struct EpiArgs {
    int kind;
    int M;                // live rows (16 * B)
    const float *wscale;  // fp8 per-column scales in tiled column order, or null
    // row normalisation folded into the consumer: rs[m] = 1/sqrt(sum_g ss[m][g] / E + eps)
    const float *ss;      // [rows][ss_gs] partial sums of squares, a row's groups contiguous, or null
    int ss_groups;
    int ss_gs;            // row stride of ss and ss_out (groups)
    int ss_stride;        // row stride of the per-group argmax keys (am_key: [G][ss_stride])
    float inv_E, eps;
    // EPI_SCALED / EPI_LOGITS output [M][ld_out]
    float *out;
    int ld_out;
    // EPI_RESID: residual stream x [M][ld_x], updated in place or written to x_out when that is
    // set; next activation
    float *x;
    float *x_out;
    int ld_x;
    const float *wnext;   // next norm weight [E]
    void *act_out;        // next activation (format act_fmt, K = ld_x or F)
    int act_fmt;
    int act_rows;         // row stride of act_out (Mmax)
    int act_K;
    float *ss_out;        // [rows][ss_gs] sums of squares of the updated x, one per group
    int block;  // rows per sequence
    int gamma;  // block width in use: drafts and acceptance cover rows 1..gamma-1
    // EPI_LOGITS: argmax across groups
    unsigned long long *am_key;  // [G][ss_stride] per-group argmax keys (argmax_key)
    int row0;      // first row of this tile within the step's rows (argmax keys, noise, drafts); 0 if whole
    int rows_all;  // rows of the whole step for the argmax's last stage (0: M)
    int arrivals;  // workgroups that count in for the argmax's last stage (0: the key slots)
    int *am_counter;
    int32_t *drafts;      // [B][gamma-1]
    const int32_t *target;  // [B][gamma-1] or null
    int32_t *n_ok;        // [B] or null
    // temperature sampling of the drafts (temp > 0): argmax of logit / temp +
    // Gumbel noise of (position n_past[b] + i, vocab id, b) under the seed
    float temp;
    uint32_t seed_lo, seed_hi;
    const int32_t *n_past;
};

// Bytes that a later launch reads, to be read now by otherwise idle compute
// units so that they sit in the memory-side cache. (Measured: worth it only
// inside the attention launch; compute units left idle by a weight-streaming
// launch are not free, extra reads there slow its own stream.)
struct Prefetch {
    const char *base;
    size_t bytes;
    unsigned *sink;  // written only if the loaded words hash to a fixed value (keeps the loads)
};

// Workgroup p of P reads its share of the prefetch bytes and drops them.
// (Taken by value: a reference into a kernel argument would put the argument
// in scratch memory.)
__device__ __forceinline__ void prefetch_slice(Prefetch f, int p, int P) {
    const size_t n16 = f.bytes / 16, per = (n16 + P - 1) / P;
    const size_t i0 = (size_t)p * per, i1 = n16 < i0 + per ? n16 : i0 + per;
    const uint4 *src = (const uint4 *)f.base;
    uint32_t acc = 0;
    constexpr int U = 8;
    const size_t nt = blockDim.x;
    for (size_t i = i0 + threadIdx.x; i < i1; i += U * nt) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t k = i + u * nt;
            v[u] = k < i1 ? src[k] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9e3779b9u && f.sink != nullptr) *f.sink = acc;
}

// Contents of an idle q/k/v exchange slot (scaled_exchange): a NaN payload that a finite partial sum never takes.
constexpr uint32_t XSLOT_EMPTY = 0x7fbadbadu;

struct GemvArgs {
    const void *W;  // tiled weights
    int N, K;       // output columns (multiple of 64), reduction length (multiple of 64)
    const void *act;
    int act_rows;   // row stride of the activation terms (>= M)
    int S;          // k-splits
    int kb_per_split;
    float *partial; // [S][G][Mp][64]
    int *counters;  // [G] arrivals, zero between launches
    int *written;   // [G] partials stored, zero between launches
    int *err;       // sticky device error word (a bounded wait gave up)
    uint32_t *xslot;  // [G][16*64] exchange slots of two-split q/k/v launches (XSLOT_EMPTY between launches)
    EpiArgs epi;
};

struct GemmArgs {
    const void *W;  // tiled weights [N, K]
    const float *wscale;
    int N, K, M;
    const void *act;
    int act_rows;   // row stride between terms (for ACT_SPLIT3)
    float *out;     // [S][M][N] f32: split s sums k-blocks [s * kbps, (s + 1) * kbps)
    int S, kbps;
    // rs_out set: one extra workgroup writes the row scales of the epilogue that
    // follows, rs_out[m] = 1/sqrt(sum_g rs_ss[m][g] * rs_inv_E + rs_eps), m < M
    const float *rs_ss;
    int rs_groups, rs_gs;
    float rs_inv_E, rs_eps;
    float *rs_out;
};

// ---------------------------------------------------------------------------
// Context
// ---------------------------------------------------------------------------
struct LayerBufs {
    void *qkv, *o, *gu, *down;           // tiled weights
    float *s_qkv, *s_o, *s_gu, *s_down;  // fp8 scales in tiled column order (or null)
};

struct ChainArgs;  // dataflow chain arguments (below)

// Paged drafter KV: a page holds PAGE_SLOTS ring slots of every layer in the
// ring layout (K, V, slot_pos); a sequence's ring is then a block table of
// W / PAGE_SLOTS int32 page ids into one pool, shared by all layers. Attention
// chunks (at most 128 slots, dividing 128) never straddle a page.
constexpr int PAGE_SLOTS = 128;
struct PagedPool {
    char *pool;  // null: rings are contiguous
    int n_pages;
    size_t page_bytes;
};

struct dflash_ctx {
    dflash_config cfg;
    int device;
    int E, H, Hkv, D, F, W, L, V, C, qdim, kvdim, nqkv, Mmax, G_E;
    int act_fmt;       // activation format of the batched projections, the dataflow chain, encode and inject
    int blk_fmt;       // activation format of the block rows in the step being issued: f32 lane words (split
                       // at load) for one sequence on the per-launch kernels, else act_fmt
    int last_B;        // batch of the last block step (0 before the first)
    int gamma;         // block width of the steps (2..block; rows gamma.. of each sequence are padding)
    PagedPool paged;   // paged drafter KV (pool null: contiguous rings)
    float temp;        // draft sampling temperature (0: greedy)
    uint64_t seed;     // key of the sampling noise
    int cus;           // compute units of the device
    unsigned *pf_sink; // target of the prefetch workgroups' never-taken store
    size_t wbytes_el;  // bytes per streamed weight element (4, 2, 1)
    char *ws;
    size_t ws_bytes;
    // fixed tables and weights
    double *inv_freq;
    float *hidden_norm, *output_norm;
    void *fc;      // tiled [E, C]
    void *kv;      // tiled [L*2*kvdim, E], rows [K0; V0; K1; V1; ...]
    float *s_kv;
    void *lm;
    float *s_lm;
    LayerBufs layer[16];
    // fp32 copies of the norm vectors, one contiguous array per family
    float *attn_norm;   // [L][E]
    float *ffn_norm;    // [L][E]
    float *q_norm;      // [L][D]
    float *k_norm;      // [L][D]
    const void *tok_embd;
    // step buffers
    float *x;           // [Mmax][E]
    void *act_a;        // attention-norm input (x * attn_norm), format act_fmt, [.][Mmax][E]
    void *act_f;        // ffn-norm input
    void *act_d;        // SwiGLU output [.][Mmax][F]
    void *act_o;        // attention output [.][Mmax][qdim]
    float *ss_a, *ss_f; // [G_E][Mmax]
    float *qkv_out;     // [Mmax][nqkv]
    float *rope_cs;     // [max_batch][block][D/2][2]
    float *att_ml;      // [max_batch][Hkv][NCH+1][G*16][2], NCH = window / attn_chunk
    float *att_o;       // [max_batch][Hkv][NCH+1][G*16][D]
    float *partial;
    size_t partial_floats;
    int *counters;
    int *written;  // split-K partials stored per group (the hand-off of the per-launch kernels)
    uint32_t *xslot;  // exchange slots of the two-split q/k/v projection, nqkv / 64 groups x 1024
    int n_xslot;
    int n_counters;
    unsigned long long *am_key;  // [G][ss_stride] per-group argmax keys (argmax_key)
    int *am_counter;  // [max_batch] argmax arrivals (one per 16-row tile of a batched step)
    int32_t *ids;       // [Mmax] block ids
    // encode / inject buffers
    float *enc_y;       // [max_inject][E]
    void *enc_act;      // features converted for the fc GEMM (if needed)
    void *inj_act;      // h converted for the kv GEMM (if needed)
    float *inj_kv;      // [max_inject][L*2*kvdim]
    // dataflow chain (one sequence per step)
    float *x2;          // second residual buffer [Mmax][E]
    ChainArgs *cargs;   // device copy of the chain arguments
    float *cpartial;    // split-K partial tiles, one region per phase slot
    int *csync;         // [epoch, sticky error, argmax counter, pad, split-K counters..., done flags...]
    int n_csync;        // ints of csync cleared at create and after a reported failure
    int chain_wg;       // workgroups per chain launch (0: chain unavailable)
    int chain_S[5];     // k-splits of the chain's q/k/v, Wo, gate/up, down and lm_head phases
    float *bpartial;    // split partials of the batched projections (null when max_batch == 1)
    float *brs;         // [Mmax] row scales of a batched epilogue (null when max_batch == 1)
    int path;           // DFLASH_PATH_*
    void *static_scratch;  // this device's address of the allocation-free encode's static scratch
};

// ---------------------------------------------------------------------------
// Dataflow chain of the block step (kernels_chain.hip)
// ---------------------------------------------------------------------------
// The block step of one sequence as 2L + 1 launches: a head launch (embedding
// and the q/k/v projection of layer 0), then per layer the attention launch and
// one chain launch of Wo, gate/up, down and the next layer's q/k/v (or the
// lm_head). A chain launch runs exactly as many 256-thread workgroups as the
// GPU holds at once; workgroup w takes item w of every phase (a column group
// and k-split of that projection). Instead of waiting for a whole phase, an
// item first issues the weight loads of its first k-block, then waits only for
// the producer column groups of its own k-slice; the epilogue waits for all
// producer groups when it needs their norm statistics. Every column group
// publishes a done flag that holds the step's epoch; the lm_head's last
// workgroup advances the epoch at the end of the step, so flags never need
// clearing. All waits are bounded in wall-clock time and raise a sticky error
// word that only dflash_check_device clears.
constexpr int CHAIN_MAX_LAYERS = 16;
constexpr int CHAIN_THREADS = 256;

struct ChainLayer {
    const void *qkv, *o, *gu, *down;          // tiled weights
    const float *s_qkv, *s_o, *s_gu, *s_down;  // fp8 column scales (tiled order) or null
};

// Phase slots of the chain (each with its own split-K partials and counters).
enum ChainSlot { CS_QKV = 0, CS_O = 1, CS_GU = 2, CS_DOWN = 3, CS_LM = 4, CS_N = 5 };

// Lives in device memory for the life of the context.
struct ChainArgs {
    int L, E, F, V, D, nqkv, qdim, G_E, block;
    int mask_id, aux_dtype, act_fmt, act_rows;
    float eps, inv_E;
    const void *tok_embd;
    const double *inv_freq;
    const float *attn_norm, *ffn_norm, *output_norm;
    ChainLayer layer[CHAIN_MAX_LAYERS];
    const void *lm;
    const float *s_lm;
    float *x, *x2;
    void *act_a, *act_f, *act_d, *act_o;
    float *ss_a, *ss_f, *qkv_out, *rope_cs;
    int ss_stride, ss_gs;
    int S[CS_N];              // k-splits per phase slot
    float *partial[CS_N];     // [S][G][16*64] per phase slot
    int *counters[CS_N];      // [G] split-K arrival counters per phase slot (zero between uses)
    // done flags: the embedding's column groups, then per layer those of Wo, gate/up and down (the q/k/v
    // and lm_head outputs are read only by later launches)
    int *done_embed;          // [G_E]
    int *done_o, *done_gu, *done_down;  // [L][groups of that projection]
    unsigned long long *am_key;  // [G][ss_stride] per-group argmax keys (argmax_key)
    int *am_counter;
    unsigned *epoch;          // the step's flag value; advanced by the step's last workgroup
    int *err;                 // sticky: a bounded wait gave up
    long long spin_ticks;
};

// Per-call inputs and outputs and per-ctx step settings, passed by value.
struct ChainIO {
    const int32_t *id_last, *block_ids, *n_past;
    float *logits;
    int32_t *drafts;
    const int32_t *target;
    int32_t *n_ok;
    int gamma;
    float temp;
    uint32_t seed_lo, seed_hi;
};

// Workgroups per chain launch for this configuration (0: not available).
int chain_grid(const dflash_ctx *c);
// Embedding, the block's rope table and the q/k/v projection of layer 0.
hipError_t launch_chain_head(const dflash_ctx *c, const ChainIO &io, hipStream_t s);
// Wo, gate/up and down of layer l, then the q/k/v projection of layer l + 1 or the lm_head.
hipError_t launch_chain_layer(const dflash_ctx *c, const ChainIO &io, int l, hipStream_t s);

struct dflash_graph {
    dflash_ctx *ctx;
    hipGraph_t graph;
    hipGraphExec_t exec;
};

// ---------------------------------------------------------------------------
// Launchers (kernels_*.hip)
// ---------------------------------------------------------------------------
hipError_t launch_tile_weights(const void *src, int src_rows, int K, int esize, void *dst, int KB, int row_map,
                               int dst_row0, int pair_half, int tpg, hipStream_t s);
hipError_t launch_tile_scales(const float *src, int src_rows, float *dst, int row_map, int dst_row0, int pair_half,
                              hipStream_t s);
hipError_t launch_vec_to_f32(const void *src, int dtype, int n, float *dst, hipStream_t s);
hipError_t launch_fill_i32(int32_t *p, int32_t v, size_t n, hipStream_t s);
hipError_t launch_quantize_fp8(const float *w, int rows, int cols, uint8_t *codes, float *scales, hipStream_t s);
int gemm_workgroups(const GemmArgs &a);  // main workgroups of a launch_gemm grid
hipError_t launch_gemv(int wdtype, int act_fmt, int MT, int WN, int NWV, int CW, dim3 grid, const GemvArgs &a,
                       hipStream_t s);
hipError_t launch_gemm(int wdtype, int act_fmt, const GemmArgs &a, hipStream_t s, bool lanes = false);
// rs: the row scales already computed from e.ss (one per row, rows 0..M-1; scaled and SwiGLU epilogues), or null
hipError_t launch_batch_epi(const float *part, int S, int M, int N, const EpiArgs &e, const float *rs, hipStream_t s);
hipError_t gemm_set_smem_limit();
hipError_t launch_split(const float *src, int rows, int K, int ld_src, void *dst, int act_fmt, int act_rows,
                        hipStream_t s);
hipError_t launch_bf16_to_f32(const uint16_t *src, size_t n, float *dst, hipStream_t s);
hipError_t launch_rmsnorm_rows(const float *y, int S, int T, int E, const float *w, float eps, float *h, hipStream_t s);
hipError_t launch_inject(const dflash_ctx *c, void *ring, void *const *rings, const int32_t *seq, int n_seq,
                         const int32_t *pos, int T, int S, hipStream_t s);
hipError_t launch_embed(const dflash_ctx *c, const int32_t *id_last, const int32_t *block_ids, const int32_t *n_past,
                        int B, hipStream_t s);
hipError_t launch_attention(const dflash_ctx *c, int l, void *const *rings, const int32_t *n_past, int B,
                            hipStream_t s);
hipError_t attention_set_smem_limit();
// Attention partial workgroups: 512 threads (two wavefronts per q head) for one
// sequence, whose chunks alone leave most compute units idle; 256 threads for
// several sequences, so that two workgroups share a compute unit.
inline int attn_threads(int B) { return B == 1 ? 512 : 256; }
// ring slots per attention chunk (one workgroup per chunk and kv head): with 512
// threads 128 (64, then 32, when the window is not a multiple of 128); with 256
// threads 64 for a bf16 ring and 32 for an f32 ring (whose values take three
// planes of LDS). For an f32 ring 128 slots measured fastest at the real
// dimensions (step 1950 us at 32 slots, 1909 at 64, 1872 at 128): fewer chunk
// partials for the combine launch to merge.
inline int attn_chunk(int ring_dtype, int W, int B) {
    if (attn_threads(B) == 512) return W % 128 == 0 ? 128 : (W % 64 == 0 ? 64 : 32);
    return ring_dtype == DFLASH_BF16 ? 64 : 32;
}
hipError_t launch_accept(const int32_t *drafts, const int32_t *target, int B, int n, int32_t *n_ok, hipStream_t s,
                         int32_t *bonus = nullptr);

// ring layout helpers (host and device)
__host__ __device__ inline size_t ring_kv_elems(int L, int Hkv, int W, int D) { return (size_t)L * Hkv * W * D; }
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
__host__ __device__ inline size_t ring_v_offset(int L, int Hkv, int W, int D, int es) {
    return align256(ring_kv_elems(L, Hkv, W, D) * es);
}
__host__ __device__ inline size_t ring_pos_offset(int L, int Hkv, int W, int D, int es) {
    return ring_v_offset(L, Hkv, W, D, es) + align256(ring_kv_elems(L, Hkv, W, D) * es);
}

struct RingLoc {
    char *base;  // ring or page holding the slot
    int slot;    // slot within it
    int W;       // its window
    bool ok;     // false for a page id outside 0..n_pages-1 (the slot then reads as empty, writes are dropped)
};
__device__ __forceinline__ RingLoc ring_locate(const void *ring_or_table, PagedPool pp, int W, int slot) {
    if (pp.pool == nullptr) return RingLoc{(char *)ring_or_table, slot, W, true};
    const int pg = ((const int32_t *)ring_or_table)[slot / PAGE_SLOTS];
    const bool ok = pg >= 0 && pg < pp.n_pages;
    return RingLoc{pp.pool + (size_t)(ok ? pg : 0) * pp.page_bytes, slot % PAGE_SLOTS, PAGE_SLOTS, ok};
}

// Memory-side cache prefetch of the attention launch
inline size_t gu_bytes(const dflash_ctx &c) { return (size_t)2 * c.F * c.E * c.wbytes_el; }
// prefetch workgroups of an attention launch (one per compute unit its grid leaves idle, per kv head and sequence)
inline int attn_pf_x(const dflash_ctx &c, int B) {
    const int attn_wgs = (c.W / attn_chunk(c.cfg.ring_dtype, c.W, B) + 1) * c.Hkv * B;
    return (c.cus > attn_wgs ? c.cus - attn_wgs : 0) / (c.Hkv * B);
}
// gate/up bytes the attention launch of one layer reads ahead: 0.5 MB per prefetch workgroup
inline size_t attn_gu_prefetch(const dflash_ctx &c, int B) {
    const size_t want = (size_t)attn_pf_x(c, B) * c.Hkv * B << 19;
    return want < gu_bytes(c) ? want : gu_bytes(c);
}
