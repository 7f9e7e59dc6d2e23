// C ABI of the DFlash drafter library: validation, workspace carving, weight
// re-tiling at create time, and the orchestration of encode, inject, the block
// step (optionally captured into a HIP graph) and the acceptance scan.
#include <math.h>
#include <stddef.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "dflash_internal.h"

// Scratch of the allocation-free encode (dflash_encode_static): one array per GPU the library runs on,
// allocated with the code object and held until the process ends. Host code never passes this name to a
// kernel: it holds a host-side stand-in; the array's device address comes from hipGetSymbolAddress.
constexpr size_t ENCODE_STATIC_SCRATCH_BYTES = 64ull << 20;
static __device__ __align__(256) unsigned char scratch[ENCODE_STATIC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(DFLASH_EHIP, "%s failed: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                          \
    do {                                             \
        hipError_t _e = (expr);                      \
        if (_e != hipSuccess) return hip_fail(_e, what); \
    } while (0)

size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// Device address of `scratch` on each device, looked up once per device with that device current.
std::mutex g_scratch_mu;
constexpr int MAX_DEVICES = 64;
void *g_scratch_dev[MAX_DEVICES];

int bind_static_scratch(int device, void **out) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (device < 0 || device >= MAX_DEVICES) return fail(DFLASH_EUNSUPPORTED, "device %d outside 0..%d", device, MAX_DEVICES - 1);
    if (g_scratch_dev[device] == nullptr) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return fail(DFLASH_EHIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        g_scratch_dev[device] = p;
    }
    *out = g_scratch_dev[device];
    return DFLASH_OK;
}

// the q/k/v projection streams 64-column groups like every other projection
// (its per-head RMSNorm and rope run in the attention kernel)
constexpr int QKV_TPG = TILES_PER_GROUP;
constexpr int QKV_WN = 1;

int dtype_bytes(int dt) { return dt == DFLASH_F32 ? 4 : dt == DFLASH_BF16 ? 2 : 1; }

int check_config(const dflash_config *c) {
    if (!c) return fail(DFLASH_EINVAL, "config is NULL");
    if (c->n_layer < 1 || c->n_layer > 16) return fail(DFLASH_EUNSUPPORTED, "n_layer must be in 1..16");
    if (c->head_dim != 64 && c->head_dim != 128) return fail(DFLASH_EUNSUPPORTED, "head_dim must be 64 or 128");
    if (c->n_head_kv < 1 || c->n_head < c->n_head_kv || c->n_head % c->n_head_kv)
        return fail(DFLASH_EUNSUPPORTED, "n_head must be a positive multiple of n_head_kv");
    if (c->n_head / c->n_head_kv > 4)
        return fail(DFLASH_EUNSUPPORTED, "at most 4 query heads per kv head are supported");
    if (c->block != 16) return fail(DFLASH_EUNSUPPORTED, "block must be 16");
    const int64_t m64[] = {c->n_embd, c->n_ff, c->n_vocab, (int64_t)c->n_capture * c->target_hidden,
                           (int64_t)c->n_head * c->head_dim, (int64_t)c->n_head_kv * c->head_dim, c->window};
    for (int64_t v : m64)
        if (v <= 0 || v % 64) return fail(DFLASH_EUNSUPPORTED, "dimensions must be positive multiples of 64");
    if (c->window > 65536) return fail(DFLASH_EUNSUPPORTED, "window must be <= 65536");
    if (c->max_batch < 1 || c->max_batch > 8) return fail(DFLASH_EUNSUPPORTED, "max_batch must be in 1..8");
    if (c->max_inject < 1) return fail(DFLASH_EINVAL, "max_inject must be >= 1");
    if (c->mask_id < 0 || c->mask_id >= c->n_vocab) return fail(DFLASH_EINVAL, "mask_id out of range");
    if (!(c->rms_eps >= 0.0f) || !(c->rope_base > 0.0)) return fail(DFLASH_EINVAL, "bad rms_eps or rope_base");
    if (c->weight_dtype < DFLASH_F32 || c->weight_dtype > DFLASH_FP8_E4M3)
        return fail(DFLASH_EINVAL, "weight_dtype must be F32, BF16 or FP8_E4M3");
    if (c->aux_dtype != DFLASH_F32 && c->aux_dtype != DFLASH_BF16) return fail(DFLASH_EINVAL, "aux_dtype must be F32 or BF16");
    if (c->ring_dtype != DFLASH_F32 && c->ring_dtype != DFLASH_BF16) return fail(DFLASH_EINVAL, "ring_dtype must be F32 or BF16");
    if (c->feature_dtype != DFLASH_F32 && c->feature_dtype != DFLASH_BF16)
        return fail(DFLASH_EINVAL, "feature_dtype must be F32 or BF16");
    return DFLASH_OK;
}

// k-split of a weight-streaming launch: aim for ~1536 workgroups (six per CU,
// rounded to the nearest split count) with at least 8 k-blocks (two per wave)
// in each; capped at 16 splits.
void choose_split(int G, int KB, int &S, int &kbps) {
    S = std::max(1, std::min(16, std::min((KB + 7) / 8, (1536 + G / 2) / G)));
    kbps = (KB + S - 1) / S;
    S = (KB + kbps - 1) / kbps;
}

int mt_for(int M) { return M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8; }

// k-splits of a batched block-row projection (gemm_kernel over all 16*B rows,
// 256 columns per workgroup, one workgroup resident per compute unit). The
// MFMA work comes in rounds of 256 workgroups (an MI355X's compute units), so
// the split count is the one that minimises rounds x k-blocks per workgroup x
// the time of a k-block (about 3 us for a 128 x 256 tile with three-term
// products) plus the split partials' traffic (S x 128 rows x N f32, written
// and read back, at about 5 TB/s); at least 8 k-blocks per split. Depends
// only on N and K, so the workspace can be sized from the config.
void batch_split(int N, int K, int &S, int &kbps) {
    constexpr int SLOTS = 256;
    constexpr double KBLOCK_US = 3.0, ROWS = 128.0, BYTES_PER_US = 5.0e6;
    const int KB = K / KBLK, tiles = (N / GROUP_N + 3) / 4;  // 256-column workgroup tiles
    const int smax = std::max(1, KB / 8);
    double best = 0.0;
    S = 1;
    for (int s = 1; s <= smax; ++s) {
        const int kb = (KB + s - 1) / s, se = (KB + kb - 1) / kb;
        const double rounds = (double)((tiles * se + SLOTS - 1) / SLOTS);
        const double us = rounds * kb * KBLOCK_US + se * ROWS * N * 8.0 / BYTES_PER_US;
        if (s == 1 || us < best) {
            best = us;
            S = se;
        }
    }
    kbps = (KB + S - 1) / S;
    S = (KB + kbps - 1) / kbps;
}

// k-splits of an encode / inject GEMM (128 x 256 tiles, one workgroup
// resident per compute unit): the count that minimises rounds of 256
// workgroups x k-blocks per workgroup x about 3 us plus the partials' traffic
// (S x M x N f32, written and read back, at about 5 TB/s), with at least 16
// k-blocks per split and the S partial [M][N] products fitting the
// [rows_cap][N] output buffer.
void gemm_split(GemmArgs &g, int rows_cap) {
    constexpr int SLOTS = 256;
    constexpr double KBLOCK_US = 3.0, BYTES_PER_US = 5.0e6;
    const int KB = g.K / KBLK, tiles = ((g.N / GROUP_N + 3) / 4) * ((g.M + 127) / 128);  // 128 x 256 tiles
    const int smax = std::max(1, std::min(KB / 16, rows_cap / g.M));
    double best = 0.0;
    int S = 1;
    for (int s = 1; s <= smax; ++s) {
        const int kb = (KB + s - 1) / s, se = (KB + kb - 1) / kb;
        const double rounds = (double)((tiles * se + SLOTS - 1) / SLOTS);
        const double us = rounds * kb * KBLOCK_US + (double)se * g.M * g.N * 8.0 / BYTES_PER_US;
        if (s == 1 || us < best) {
            best = us;
            S = se;
        }
    }
    g.kbps = (KB + S - 1) / S;
    g.S = (KB + g.kbps - 1) / g.kbps;
}

// k-splits of a chain phase with G column groups of KB k-blocks when nwg workgroups each take one item
// (a group and a k-split) of every phase: as many as keep G * S <= nwg.
int chain_split(int G, int KB, int nwg) {
    const int s = std::max(1, std::min(KB, nwg / G));
    const int kbps = (KB + s - 1) / s;
    return (KB + kbps - 1) / kbps;
}

// Most workgroups a chain launch uses (sizes the chain's partial buffers).
constexpr int CHAIN_MAX_WG = 2048;

struct Carver {
    char *base;
    size_t off = 0;
    explicit Carver(char *b) : base(b) {}
    template <typename T>
    T *take(size_t bytes) {
        size_t o = off;
        off = a256(off + bytes);
        return base ? (T *)(base + o) : nullptr;
    }
};

// Carve (or, with base == nullptr, just size) the workspace.
size_t carve(dflash_ctx &x, char *base) {
    const dflash_config &c = x.cfg;
    Carver cv(base);
    const int E = c.n_embd, L = c.n_layer, D = c.head_dim, F = c.n_ff, V = c.n_vocab;
    const int qdim = c.n_head * D, kvdim = c.n_head_kv * D, nqkv = qdim + 2 * kvdim;
    const int Cin = c.n_capture * c.target_hidden;
    const int Mmax = 16 * c.max_batch;
    const size_t esw = dtype_bytes(c.weight_dtype), esa = dtype_bytes(c.aux_dtype);
    const bool fp8 = c.weight_dtype == DFLASH_FP8_E4M3;
    const int act_fmt = c.weight_dtype == DFLASH_F32 ? ACT_F32 : ACT_SPLIT3;
    const size_t act_es = act_fmt == ACT_F32 ? 4 : 6;  // bytes per activation element (3 bf16 planes)

    x.inv_freq = cv.take<double>(sizeof(double) * D / 2);
    x.hidden_norm = cv.take<float>(4ull * E);
    x.output_norm = cv.take<float>(4ull * E);
    x.attn_norm = cv.take<float>(4ull * L * E);
    x.ffn_norm = cv.take<float>(4ull * L * E);
    x.q_norm = cv.take<float>(4ull * L * D);
    x.k_norm = cv.take<float>(4ull * L * D);
    x.fc = cv.take<void>(esa * E * Cin);
    x.kv = cv.take<void>(esw * (size_t)L * 2 * kvdim * E);
    x.s_kv = fp8 ? cv.take<float>(4ull * L * 2 * kvdim) : nullptr;
    for (int l = 0; l < L; ++l) {
        LayerBufs &b = x.layer[l];
        b.qkv = cv.take<void>(esw * nqkv * E);
        b.o = cv.take<void>(esw * E * qdim);
        b.gu = cv.take<void>(esw * 2ull * F * E);
        b.down = cv.take<void>(esw * (size_t)E * F);
        b.s_qkv = fp8 ? cv.take<float>(4ull * nqkv) : nullptr;
        b.s_o = fp8 ? cv.take<float>(4ull * E) : nullptr;
        b.s_gu = fp8 ? cv.take<float>(8ull * F) : nullptr;
        b.s_down = fp8 ? cv.take<float>(4ull * E) : nullptr;
    }
    x.lm = cv.take<void>(esw * (size_t)V * E);
    x.s_lm = fp8 ? cv.take<float>(4ull * V) : nullptr;

    // attention partials: the most chunks any batch size uses (the smallest chunk)
    const int G_E = E / GROUP_N, G = c.n_head / c.n_head_kv,
              NCH = c.window / std::min(attn_chunk(c.ring_dtype, c.window, 1), attn_chunk(c.ring_dtype, c.window, 2));
    x.x = cv.take<float>(4ull * Mmax * E);
    x.act_a = cv.take<void>(act_es * Mmax * E);
    x.act_f = cv.take<void>(act_es * Mmax * E);
    x.act_d = cv.take<void>(act_es * Mmax * F);
    x.act_o = cv.take<void>(act_es * Mmax * qdim);
    // sums of squares per column group; half-group launches write twice as many
    x.ss_a = cv.take<float>(4ull * 2 * G_E * Mmax);
    x.ss_f = cv.take<float>(4ull * 2 * G_E * Mmax);
    x.qkv_out = cv.take<float>(4ull * Mmax * nqkv);
    x.rope_cs = cv.take<float>(4ull * c.max_batch * c.block * D);
    x.att_ml = cv.take<float>(4ull * c.max_batch * c.n_head_kv * (NCH + 1) * G * 16 * 2);
    x.att_o = cv.take<float>(4ull * c.max_batch * c.n_head_kv * (NCH + 1) * G * 16 * D);
    // split-K partials: the largest S * G * Mp * 64 over the step's launches
    const int Mp = 16 * mt_for(Mmax);
    const int shapes[5][3] = {{nqkv, E, QKV_WN}, {E, qdim, 1}, {2 * F, E, 1}, {E, F, 1}, {V, E, 1}};
    size_t pmax = 0;
    int gmax = 0;
    for (auto &sh : shapes) {
        int Gn = sh[0] / (GROUP_N * sh[2]), KB = sh[1] / KBLK, S, kbps;
        choose_split(Gn, KB, S, kbps);
        pmax = std::max(pmax, (size_t)S * Gn * Mp * GROUP_N * sh[2]);
        gmax = std::max(gmax, Gn);
    }
    x.partial = cv.take<float>(4 * pmax);
    x.partial_floats = pmax;
    x.counters = cv.take<int>(4ull * 2 * gmax);  // half-group launches count per 32 columns
    x.written = cv.take<int>(4ull * 2 * gmax);
    x.n_xslot = (std::max(nqkv, V) / GROUP_N) * 16 * GROUP_N;  // q/k/v and lm_head groups
    x.xslot = cv.take<uint32_t>(4ull * x.n_xslot);
    x.pf_sink = cv.take<unsigned>(64);
    x.n_counters = 2 * gmax;
    x.am_key = cv.take<unsigned long long>(8ull * (V / 32) * Mmax);
    x.am_counter = cv.take<int>(4ull * c.max_batch);  // one per sequence (a batched step's 16-row tiles)
    x.ids = cv.take<int32_t>(4ull * Mmax);

    const int T = c.max_inject;
    x.enc_y = cv.take<float>(4ull * T * E);
    x.enc_act = nullptr;
    if (c.aux_dtype == DFLASH_F32 && c.feature_dtype == DFLASH_BF16) x.enc_act = cv.take<void>(4ull * T * Cin);
    if (c.aux_dtype == DFLASH_BF16 && c.feature_dtype == DFLASH_F32) x.enc_act = cv.take<void>(6ull * T * Cin);
    x.inj_act = act_fmt == ACT_SPLIT3 ? cv.take<void>(6ull * T * E) : nullptr;
    x.inj_kv = cv.take<float>(4ull * T * L * 2 * kvdim);

    // dataflow chain: split-K partials and counters per phase slot for the most workgroups a launch may
    // have; then the epoch, the sticky error word, the argmax counter and the done flags
    x.x2 = cv.take<float>(4ull * Mmax * E);
    x.cargs = cv.take<ChainArgs>(sizeof(ChainArgs));
    {
        const int slot_shape[CS_N][2] = {{nqkv, E}, {E, qdim}, {2 * F, E}, {E, F}, {V, E}};
        size_t pf = 0;
        int cnt = 0;
        for (auto &sh : slot_shape) {
            const int Gn = sh[0] / GROUP_N, KBn = sh[1] / KBLK;
            pf += a256(4ull * chain_split(Gn, KBn, CHAIN_MAX_WG) * Gn * 16 * GROUP_N) / 4;
            cnt += Gn;
        }
        x.cpartial = cv.take<float>(4 * pf);
        x.n_csync = 4 + cnt + G_E + L * (G_E + 2 * F / GROUP_N + G_E);
        x.csync = cv.take<int>(4ull * x.n_csync);
    }
    // split partials of the batched projections (16*B rows, B > 1)
    x.bpartial = nullptr;
    x.brs = nullptr;
    if (c.max_batch > 1) {
        size_t bmax = 0;
        for (auto &sh : shapes) {
            int S, kbps;
            batch_split(sh[0], sh[1], S, kbps);
            bmax = std::max(bmax, (size_t)S * Mmax * sh[0]);
        }
        x.bpartial = cv.take<float>(4 * bmax);
        x.brs = cv.take<float>(4ull * Mmax);
    }
    return cv.off;
}

void derive(dflash_ctx &x) {
    const dflash_config &c = x.cfg;
    x.E = c.n_embd;
    x.H = c.n_head;
    x.Hkv = c.n_head_kv;
    x.D = c.head_dim;
    x.F = c.n_ff;
    x.W = c.window;
    x.L = c.n_layer;
    x.V = c.n_vocab;
    x.C = c.n_capture * c.target_hidden;
    x.qdim = x.H * x.D;
    x.kvdim = x.Hkv * x.D;
    x.nqkv = x.qdim + 2 * x.kvdim;
    x.Mmax = 16 * c.max_batch;
    x.G_E = x.E / GROUP_N;
    x.act_fmt = c.weight_dtype == DFLASH_F32 ? ACT_F32 : ACT_SPLIT3;
    x.blk_fmt = x.act_fmt;
    x.wbytes_el = dtype_bytes(c.weight_dtype);
}

// bytes of a ring of `window` slots (a page is one with PAGE_SLOTS)
size_t ring_bytes_w(const dflash_config &c, int window) {
    const int es = dtype_bytes(c.ring_dtype);
    const size_t kv = a256((size_t)c.n_layer * c.n_head_kv * window * c.head_dim * es);
    return 2 * kv + a256(4ull * window);
}
size_t ring_bytes_of(const dflash_config &c) { return ring_bytes_w(c, c.window); }

int tile_matrix(const void *src, int rows, int K, int es, void *dst, int row_map, int row0, int half, hipStream_t s,
                int tpg = TILES_PER_GROUP) {
    HIP_TRY(launch_tile_weights(src, rows, K, es, dst, K / KBLK, row_map, row0, half, tpg, s), "weight tiling launch");
    return DFLASH_OK;
}

int tile_scales(const float *src, int rows, float *dst, int row_map, int row0, int half, hipStream_t s) {
    if (!dst) return DFLASH_OK;
    HIP_TRY(launch_tile_scales(src, rows, dst, row_map, row0, half, s), "scale tiling launch");
    return DFLASH_OK;
}

#define TRY(expr)                      \
    do {                               \
        int _r = (expr);               \
        if (_r != DFLASH_OK) return _r; \
    } while (0)

int check_weights(const dflash_config &c, const dflash_weights *w) {
    if (!w) return fail(DFLASH_EINVAL, "weights is NULL");
    if (!w->tok_embd || !w->lm_head || !w->fc || !w->hidden_norm || !w->output_norm || !w->layers)
        return fail(DFLASH_EINVAL, "a global weight pointer is NULL");
    const bool fp8 = c.weight_dtype == DFLASH_FP8_E4M3;
    if (fp8 && !w->s_lm_head) return fail(DFLASH_EINVAL, "s_lm_head is NULL for FP8 weights");
    for (int l = 0; l < c.n_layer; ++l) {
        const dflash_layer_weights &lw = w->layers[l];
        if (!lw.attn_norm || !lw.wq || !lw.wk || !lw.wv || !lw.wo || !lw.q_norm || !lw.k_norm || !lw.ffn_norm ||
            !lw.w_gate || !lw.w_up || !lw.w_down)
            return fail(DFLASH_EINVAL, "a weight pointer of layer %d is NULL", l);
        if (fp8 && (!lw.s_q || !lw.s_k || !lw.s_v || !lw.s_o || !lw.s_gate || !lw.s_up || !lw.s_down))
            return fail(DFLASH_EINVAL, "an FP8 scale pointer of layer %d is NULL", l);
    }
    return DFLASH_OK;
}

int prepare_chain(dflash_ctx &x, hipStream_t s);

int prepare(dflash_ctx &x, const dflash_weights *w, hipStream_t s) {
    const dflash_config &c = x.cfg;
    const int E = x.E, L = x.L, D = x.D, F = x.F, V = x.V;
    const int esw = (int)x.wbytes_el, esa = dtype_bytes(c.aux_dtype);
    std::vector<double> f(D / 2);
    for (int i = 0; i < D / 2; ++i) f[i] = pow(c.rope_base, -2.0 * i / D);
    HIP_TRY(hipMemcpyAsync(x.inv_freq, f.data(), sizeof(double) * f.size(), hipMemcpyHostToDevice, s),
            "inverse-frequency upload");
    HIP_TRY(hipStreamSynchronize(s), "inverse-frequency upload");
    HIP_TRY(launch_vec_to_f32(w->hidden_norm, c.aux_dtype, E, x.hidden_norm, s), "norm copy");
    HIP_TRY(launch_vec_to_f32(w->output_norm, c.aux_dtype, E, x.output_norm, s), "norm copy");
    for (int l = 0; l < L; ++l) {
        const dflash_layer_weights &lw = w->layers[l];
        HIP_TRY(launch_vec_to_f32(lw.attn_norm, c.aux_dtype, E, x.attn_norm + (size_t)l * E, s), "norm copy");
        HIP_TRY(launch_vec_to_f32(lw.ffn_norm, c.aux_dtype, E, x.ffn_norm + (size_t)l * E, s), "norm copy");
        HIP_TRY(launch_vec_to_f32(lw.q_norm, c.aux_dtype, D, x.q_norm + (size_t)l * D, s), "norm copy");
        HIP_TRY(launch_vec_to_f32(lw.k_norm, c.aux_dtype, D, x.k_norm + (size_t)l * D, s), "norm copy");
    }
    TRY(tile_matrix(w->fc, E, x.C, esa, x.fc, 0, 0, 0, s));
    for (int l = 0; l < L; ++l) {
        const dflash_layer_weights &lw = w->layers[l];
        const int r0 = l * 2 * x.kvdim;
        TRY(tile_matrix(lw.wk, x.kvdim, E, esw, x.kv, 0, r0, 0, s));
        TRY(tile_matrix(lw.wv, x.kvdim, E, esw, x.kv, 0, r0 + x.kvdim, 0, s));
        TRY(tile_scales(lw.s_k, x.kvdim, x.s_kv, 0, r0, 0, s));
        TRY(tile_scales(lw.s_v, x.kvdim, x.s_kv, 0, r0 + x.kvdim, 0, s));
        LayerBufs &b = x.layer[l];
        TRY(tile_matrix(lw.wq, x.qdim, E, esw, b.qkv, 0, 0, 0, s, QKV_TPG));
        TRY(tile_matrix(lw.wk, x.kvdim, E, esw, b.qkv, 0, x.qdim, 0, s, QKV_TPG));
        TRY(tile_matrix(lw.wv, x.kvdim, E, esw, b.qkv, 0, x.qdim + x.kvdim, 0, s, QKV_TPG));
        TRY(tile_scales(lw.s_q, x.qdim, b.s_qkv, 0, 0, 0, s));
        TRY(tile_scales(lw.s_k, x.kvdim, b.s_qkv, 0, x.qdim, 0, s));
        TRY(tile_scales(lw.s_v, x.kvdim, b.s_qkv, 0, x.qdim + x.kvdim, 0, s));
        TRY(tile_matrix(lw.wo, E, x.qdim, esw, b.o, 0, 0, 0, s));
        TRY(tile_scales(lw.s_o, E, b.s_o, 0, 0, 0, s));
        TRY(tile_matrix(lw.w_gate, F, E, esw, b.gu, 1, 0, 0, s));
        TRY(tile_matrix(lw.w_up, F, E, esw, b.gu, 1, 0, 1, s));
        TRY(tile_scales(lw.s_gate, F, b.s_gu, 1, 0, 0, s));
        TRY(tile_scales(lw.s_up, F, b.s_gu, 1, 0, 1, s));
        TRY(tile_matrix(lw.w_down, E, F, esw, b.down, 0, 0, 0, s));
        TRY(tile_scales(lw.s_down, E, b.s_down, 0, 0, 0, s));
    }
    TRY(tile_matrix(w->lm_head, V, E, esw, x.lm, 0, 0, 0, s));
    TRY(tile_scales(w->s_lm_head, V, x.s_lm, 0, 0, 0, s));
    HIP_TRY(launch_fill_i32(x.counters, 0, x.n_counters, s), "counter reset");
    HIP_TRY(launch_fill_i32(x.written, 0, x.n_counters, s), "counter reset");
    HIP_TRY(launch_fill_i32((int *)x.xslot, (int)XSLOT_EMPTY, x.n_xslot, s), "exchange slot reset");
    HIP_TRY(launch_fill_i32(x.am_counter, 0, x.cfg.max_batch, s), "counter reset");
    HIP_TRY(launch_fill_i32(x.csync, 0, x.n_csync, s), "counter reset");
    HIP_TRY(launch_fill_i32(x.csync, 1, 1, s), "epoch reset");  // epoch 1: flags hold 0 until first set
    return prepare_chain(x, s);
}

// Arguments of the dataflow chain, kept in the workspace for the life of the context.
int prepare_chain(dflash_ctx &x, hipStream_t s) {
    x.chain_wg = 0;
    x.path = DFLASH_PATH_AUTO;
    // At most three workgroups per compute unit (fewer weight bytes in flight keep the phases' hand-off round
    // trips short: real-dims bf16 step 1248 us at five per compute unit, 1219 at four, 1169 at three), but at
    // least one per column group of the widest phase, so every phase fits in one pass.
    const int cap = std::max(3 * x.cus, std::max(std::max(x.nqkv, x.E), std::max(2 * x.F, x.V)) / GROUP_N);
    const int nwg = std::min(std::min(chain_grid(&x), CHAIN_MAX_WG), cap);
    if (nwg < 1) return DFLASH_OK;  // the per-launch kernels serve every step
    int rate_khz = 0;
    HIP_TRY(hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, x.device), "wall clock rate query");
    ChainArgs a = {};
    a.L = x.L;
    a.E = x.E;
    a.F = x.F;
    a.V = x.V;
    a.D = x.D;
    a.nqkv = x.nqkv;
    a.qdim = x.qdim;
    a.G_E = x.G_E;
    a.block = x.cfg.block;
    a.mask_id = x.cfg.mask_id;
    a.aux_dtype = x.cfg.aux_dtype;
    a.act_fmt = ACT_F32;  // one sequence: f32 lane words, split into the bf16 terms at load for bf16 / fp8 weights
    a.act_rows = x.Mmax;
    a.eps = x.cfg.rms_eps;
    a.inv_E = 1.0f / (float)x.E;
    a.tok_embd = x.tok_embd;
    a.inv_freq = x.inv_freq;
    a.attn_norm = x.attn_norm;
    a.ffn_norm = x.ffn_norm;
    a.output_norm = x.output_norm;
    for (int l = 0; l < x.L; ++l) {
        const LayerBufs &b = x.layer[l];
        a.layer[l] = ChainLayer{b.qkv, b.o, b.gu, b.down, b.s_qkv, b.s_o, b.s_gu, b.s_down};
    }
    a.lm = x.lm;
    a.s_lm = x.s_lm;
    a.x = x.x;
    a.x2 = x.x2;
    a.act_a = x.act_a;
    a.act_f = x.act_f;
    a.act_d = x.act_d;
    a.act_o = x.act_o;
    a.ss_a = x.ss_a;
    a.ss_f = x.ss_f;
    a.qkv_out = x.qkv_out;
    a.rope_cs = x.rope_cs;
    a.ss_stride = x.Mmax;
    a.ss_gs = 2 * x.G_E;
    const int slot_shape[CS_N][2] = {{x.nqkv, x.E}, {x.E, x.qdim}, {2 * x.F, x.E}, {x.E, x.F}, {x.V, x.E}};
    float *pp = x.cpartial;
    int *sync = x.csync;
    a.epoch = (unsigned *)sync;
    a.err = sync + 1;
    a.am_counter = sync + 2;
    int *cnt = sync + 4;
    for (int i = 0; i < CS_N; ++i) {
        const int Gn = slot_shape[i][0] / GROUP_N, KBn = slot_shape[i][1] / KBLK;
        a.S[i] = x.chain_S[i] = chain_split(Gn, KBn, nwg);
        a.partial[i] = pp;
        pp += a256(4ull * chain_split(Gn, KBn, CHAIN_MAX_WG) * Gn * 16 * GROUP_N) / 4;
        a.counters[i] = cnt;
        cnt += Gn;
        if (a.S[i] > chain_split(Gn, KBn, CHAIN_MAX_WG) || (size_t)Gn * a.S[i] > (size_t)nwg)
            return fail(DFLASH_EHIP, "internal: chain split of phase slot %d does not fit", i);
    }
    a.done_embed = cnt;
    a.done_o = a.done_embed + x.G_E;
    a.done_gu = a.done_o + (size_t)x.L * x.G_E;
    a.done_down = a.done_gu + (size_t)x.L * (2 * x.F / GROUP_N);
    if (a.done_down + (size_t)x.L * x.G_E != x.csync + x.n_csync)
        return fail(DFLASH_EHIP, "internal: chain flag layout");
    a.am_key = x.am_key;
    a.spin_ticks = (long long)rate_khz * 1000;  // one second
    HIP_TRY(hipMemcpyAsync(x.cargs, &a, sizeof a, hipMemcpyHostToDevice, s), "chain argument upload");
    HIP_TRY(hipStreamSynchronize(s), "chain argument upload");
    x.chain_wg = nwg;
    return DFLASH_OK;
}

// DFLASH_PATH_AUTO takes the per-launch kernels: measured on MI355X at the real drafter dimensions, the
// dataflow chain overlaps each projection's tail with the next one's weight stream, but the handshakes,
// epilogues and flags on its critical path then queue behind that stream, and the chain launch ends up
// slower than the kernels it replaces; it stays an explicit choice.
bool use_chain(const dflash_ctx &x, int B) {
    return B == 1 && x.chain_wg >= 1 && x.path == DFLASH_PATH_PERSISTENT;
}

EpiArgs epi_base(const dflash_ctx &x, int kind, int M) {
    EpiArgs e = {};
    e.kind = kind;
    e.M = M;
    e.ss_stride = x.Mmax;
    e.ss_gs = 2 * x.G_E;  // half-group launches write two sums per 64 columns
    e.inv_E = 1.0f / (float)x.E;
    e.eps = x.cfg.rms_eps;
    e.block = x.cfg.block;
    e.gamma = x.gamma;
    e.temp = x.temp;
    e.seed_lo = (uint32_t)x.seed;
    e.seed_hi = (uint32_t)(x.seed >> 32);
    e.act_rows = x.Mmax;
    e.act_fmt = x.blk_fmt;
    return e;
}

// Columns per workgroup of a block-step projection: 32 (half a column group,
// 16 waves, no k-split) for f32 weights when one sequence's projection has at
// most as many half groups as the GPU has compute units and its epilogue is
// not SwiGLU (which pairs the two halves of a group); 64 otherwise. Half groups
// drop the split-K handshake but make every workgroup read the whole
// activation row, which only pays where the weights dominate the reads (f32:
// measured 2128 -> 2087 us per real-dims step; bf16 1184 -> 1250, so not used).
// The consumers of the sums of squares that a residual epilogue writes count
// N / width groups.
int gemv_col_width(const dflash_ctx &x, int N, int M, int WN, int kind) {
    if (M > 16 && x.bpartial) return GROUP_N;  // batched path: 64-column tiles
    if (x.cfg.weight_dtype != DFLASH_F32 || mt_for(M) != 1 || WN != 1 || kind == EPI_SWIGLU) return GROUP_N;
    return N / 32 <= x.cus ? 32 : GROUP_N;
}

int gemv(const dflash_ctx &x, const void *W, int N, int K, const void *act, const EpiArgs &epi, hipStream_t s,
         int WN = 1) {
    if (epi.M > 16 && x.bpartial) {
        // several sequences: an MFMA GEMM over all rows writes split partials, then the epilogue kernel
        GemmArgs g = {};
        g.W = W;
        g.N = N;
        g.K = K;
        g.M = epi.M;
        g.act = act;
        g.act_rows = x.Mmax;
        g.out = x.bpartial;
        batch_split(N, K, g.S, g.kbps);
        const float *rs = nullptr;
        if (epi.ss != nullptr && (epi.kind == EPI_SCALED || epi.kind == EPI_SWIGLU) && epi.M <= 128 && epi.ss_groups <= 256 &&
            gemm_workgroups(g) % x.cus != 0) {
            // the row scales once per launch, by an extra GEMM workgroup on a compute unit the GEMM's last
            // round leaves free, instead of in every epilogue workgroup
            g.rs_ss = epi.ss;
            g.rs_groups = epi.ss_groups;
            g.rs_gs = epi.ss_gs;
            g.rs_inv_E = epi.inv_E;
            g.rs_eps = epi.eps;
            g.rs_out = x.brs;
            rs = x.brs;
        }
        HIP_TRY(launch_gemm(x.cfg.weight_dtype, x.blk_fmt, g, s, true), "batched projection launch");
        HIP_TRY(launch_batch_epi(x.bpartial, g.S, g.M, N, epi, rs, s), "batched epilogue launch");
        return DFLASH_OK;
    }
    GemvArgs a = {};
    a.W = W;
    a.N = N;
    a.K = K;
    a.act = act;
    a.act_rows = x.Mmax;
    const int KB = K / KBLK;
    const int cw = gemv_col_width(x, N, epi.M, WN, epi.kind);
    const int G = N / (cw * WN);
    int nwv = 4;
    choose_split(G, KB, a.S, a.kb_per_split);
    if (cw < GROUP_N || (mt_for(epi.M) == 1 && WN == 1 && 2 * G <= x.cus)) {
        // few column groups: one 16-wave workgroup per compute unit (half
        // groups where that is enough to fill the GPU), as many k-splits as fit
        nwv = 16;
        const int cap = (int)std::min<size_t>(x.partial_floats / ((size_t)G * 16 * cw), 64);
        const int S = std::max(1, std::min(std::min(x.cus / G, KB / 8), cap));
        a.kb_per_split = (KB + S - 1) / S;
        a.S = (KB + a.kb_per_split - 1) / a.kb_per_split;
    }
    a.partial = x.partial;
    a.counters = x.counters;
    a.written = x.written;
    a.err = x.csync + 1;
    // exchange slots for the per-element epilogues (q/k/v; lm_head, whose argmax keys take 2G slots)
    a.xslot = ((epi.kind == EPI_SCALED || (epi.kind == EPI_LOGITS && 2 * G <= x.V / 32)) &&
               (size_t)G * 16 * GROUP_N <= (size_t)x.n_xslot)
                  ? x.xslot
                  : nullptr;
    a.epi = epi;
    if (G > x.n_counters) return fail(DFLASH_EINVAL, "GEMV with %d column groups exceeds the counter table", G);
    HIP_TRY(launch_gemv(x.cfg.weight_dtype, x.blk_fmt, mt_for(epi.M), WN, nwv, cw, dim3(G, a.S), a, s),
            "block-step GEMV launch");
    return DFLASH_OK;
}

// q/k/v projection with the attention norm folded in (the attention kernel
// RMS-norms and ropes the q and k heads)
int stage_qkv(const dflash_ctx &x, int l, int M, hipStream_t s) {
    const LayerBufs &b = x.layer[l];
    EpiArgs e = epi_base(x, EPI_SCALED, M);
    e.wscale = b.s_qkv;
    e.ss = x.ss_a;
    // layer 0 reads the embed kernel's 64-column sums, later layers the down projection's
    e.ss_groups = l == 0 ? x.G_E : x.E / gemv_col_width(x, x.E, M, 1, EPI_RESID);
    e.out = x.qkv_out;
    e.ld_out = x.nqkv;
    return gemv(x, b.qkv, x.nqkv, x.E, x.act_a, e, s, QKV_WN);
}

int stage_o(const dflash_ctx &x, int l, int M, hipStream_t s) {
    const LayerBufs &b = x.layer[l];
    EpiArgs e = epi_base(x, EPI_RESID, M);
    e.wscale = b.s_o;
    e.x = x.x;
    e.ld_x = x.E;
    e.wnext = x.ffn_norm + (size_t)l * x.E;
    e.act_out = x.act_f;
    e.act_K = x.E;
    e.ss_out = x.ss_f;
    return gemv(x, b.o, x.E, x.qdim, x.act_o, e, s);
}

int stage_gu(const dflash_ctx &x, int l, int M, hipStream_t s) {
    const LayerBufs &b = x.layer[l];
    EpiArgs e = epi_base(x, EPI_SWIGLU, M);
    e.wscale = b.s_gu;
    e.ss = x.ss_f;
    e.ss_groups = x.E / gemv_col_width(x, x.E, M, 1, EPI_RESID);  // written by Wo
    e.act_out = x.act_d;
    e.act_K = x.F;
    return gemv(x, b.gu, 2 * x.F, x.E, x.act_f, e, s);
}

int stage_down(const dflash_ctx &x, int l, int M, hipStream_t s) {
    const LayerBufs &b = x.layer[l];
    EpiArgs e = epi_base(x, EPI_RESID, M);
    e.wscale = b.s_down;
    e.x = x.x;
    e.ld_x = x.E;
    e.wnext = l + 1 < x.L ? x.attn_norm + (size_t)(l + 1) * x.E : x.output_norm;
    e.act_out = x.act_a;
    e.act_K = x.E;
    e.ss_out = x.ss_a;
    return gemv(x, b.down, x.E, x.F, x.act_d, e, s);
}

int stage_lm(const dflash_ctx &x, int M, float *logits, int32_t *drafts, const int32_t *target, int32_t *n_ok,
             const int32_t *n_past, hipStream_t s) {
    EpiArgs e = epi_base(x, EPI_LOGITS, M);
    e.wscale = x.s_lm;
    e.ss = x.ss_a;
    e.ss_groups = x.E / gemv_col_width(x, x.E, M, 1, EPI_RESID);  // written by the last down
    e.out = logits;
    e.ld_out = x.V;
    e.am_key = x.am_key;
    e.am_counter = x.am_counter;
    e.drafts = drafts;
    e.target = target;
    e.n_ok = n_ok;
    e.n_past = n_past;  // positions of the sampling noise
    return gemv(x, x.lm, x.V, x.E, x.act_a, e, s);
}

// The block step: embed; per layer QKV, attention, Wo (+residual), gate/up
// (+SwiGLU), down (+residual); lm_head with argmax (and acceptance).
int run_step(dflash_ctx &x, void *const *rings, const int32_t *id_last, const int32_t *block_ids,
             const int32_t *n_past, int B, float *logits, int32_t *drafts, const int32_t *target, int32_t *n_ok,
             hipStream_t s) {
    // one sequence on the per-launch kernels: f32 activations split at load (4 bytes per value written and
    // read instead of 6); the batched projections and the chain read three bf16 planes
    x.blk_fmt = B == 1 ? ACT_F32 : x.act_fmt;
    if (use_chain(x, B)) {
        // dataflow chain: head (embed + q/k/v of layer 0); per layer attention, then Wo .. q/k/v(l+1) or lm_head
        ChainIO io{id_last, block_ids, n_past, logits, drafts, target, n_ok, x.gamma, x.temp, (uint32_t)x.seed,
                   (uint32_t)(x.seed >> 32)};
        HIP_TRY(launch_chain_head(&x, io, s), "chain head launch");
        for (int l = 0; l < x.L; ++l) {
            HIP_TRY(launch_attention(&x, l, rings, n_past, B, s), "attention launch");
            HIP_TRY(launch_chain_layer(&x, io, l, s), "chain launch");
        }
        x.last_B = B;
        return DFLASH_OK;
    }
    const int M = 16 * B;
    HIP_TRY(launch_embed(&x, id_last, block_ids, n_past, B, s), "embed launch");
    for (int l = 0; l < x.L; ++l) {
        TRY(stage_qkv(x, l, M, s));
        HIP_TRY(launch_attention(&x, l, rings, n_past, B, s), "attention launch");
        TRY(stage_o(x, l, M, s));
        TRY(stage_gu(x, l, M, s));
        TRY(stage_down(x, l, M, s));
    }
    TRY(stage_lm(x, M, logits, drafts, target, n_ok, n_past, s));
    x.last_B = B;
    return DFLASH_OK;
}

int check_step_args(dflash_ctx *x, void *const *rings, const void *ids, const int32_t *n_past, int B, float *logits,
                     int32_t *drafts) {
    if (!x) return fail(DFLASH_EINVAL, "ctx is NULL");
    if (!rings || !ids || !n_past || !logits || !drafts) return fail(DFLASH_EINVAL, "a step pointer is NULL");
    if (B < 1 || B > x->cfg.max_batch) return fail(DFLASH_ERANGE, "B=%d outside 1..max_batch=%d", B, x->cfg.max_batch);
    return DFLASH_OK;
}

}  // namespace

extern "C" {

const char *dflash_last_error(void) { return g_err.c_str(); }

size_t dflash_workspace_bytes(const dflash_config *cfg) {
    if (check_config(cfg) != DFLASH_OK) return 0;
    dflash_ctx x = {};
    x.cfg = *cfg;
    derive(x);
    return carve(x, nullptr);
}

size_t dflash_ring_bytes(const dflash_config *cfg) {
    if (check_config(cfg) != DFLASH_OK) return 0;
    return ring_bytes_of(*cfg);
}

int dflash_create(const dflash_config *cfg, const dflash_weights *w, void *workspace, size_t workspace_bytes,
                  void *stream, dflash_ctx **out) {
    if (!out) return fail(DFLASH_EINVAL, "out is NULL");
    *out = nullptr;
    TRY(check_config(cfg));
    TRY(check_weights(*cfg, w));
    if (!workspace) return fail(DFLASH_EINVAL, "workspace is NULL");
    if ((uintptr_t)workspace % 256) return fail(DFLASH_EINVAL, "workspace must be 256-byte aligned");
    dflash_ctx *x = new dflash_ctx();
    x->cfg = *cfg;
    derive(*x);
    const size_t need = carve(*x, nullptr);
    if (workspace_bytes < need) {
        delete x;
        return fail(DFLASH_ERANGE, "workspace holds %zu bytes, %zu needed", workspace_bytes, need);
    }
    carve(*x, (char *)workspace);
    x->ws = (char *)workspace;
    x->ws_bytes = workspace_bytes;
    x->tok_embd = w->tok_embd;
    x->gamma = x->cfg.block;
    x->paged = PagedPool{nullptr, 0, 0};
    x->temp = 0.0f;
    x->seed = 0;
    hipError_t e = hipGetDevice(&x->device);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&x->cus, hipDeviceAttributeMultiprocessorCount, x->device);
    if (e != hipSuccess) {
        delete x;
        return hip_fail(e, "hipGetDevice / compute unit count");
    }
    if (bind_static_scratch(x->device, &x->static_scratch) != DFLASH_OK) {
        delete x;
        return DFLASH_EHIP;
    }
    e = attention_set_smem_limit();
    if (e == hipSuccess) e = gemm_set_smem_limit();
    if (e != hipSuccess) {
        delete x;
        return hip_fail(e, "hipFuncSetAttribute (attention / GEMM LDS)");
    }
    int r = prepare(*x, w, (hipStream_t)stream);
    if (r != DFLASH_OK) {
        delete x;
        return r;
    }
    *out = x;
    return DFLASH_OK;
}

void dflash_destroy(dflash_ctx *ctx) { delete ctx; }

// Empty a ring of `window` slots: K and V are zeroed too, since attention
// weights a masked slot's value by an exact 0, which only stays 0 when the
// value is finite.
int reset_ring_w(const dflash_ctx &x, char *ring, int window, hipStream_t s) {
    const int es = dtype_bytes(x.cfg.ring_dtype);
    const size_t kv = a256((size_t)x.L * x.Hkv * window * x.D * es);
    HIP_TRY(launch_fill_i32((int32_t *)ring, 0, 2 * kv / 4, s), "ring reset launch");
    HIP_TRY(launch_fill_i32((int32_t *)(ring + 2 * kv), -1, window, s), "ring reset launch");
    return DFLASH_OK;
}

int dflash_ring_reset(dflash_ctx *x, void *ring, void *stream) {
    if (!x || !ring) return fail(DFLASH_EINVAL, "ctx or ring is NULL");
    if (x->paged.pool) return fail(DFLASH_ESTATE, "paged mode: reset pages with dflash_pages_reset");
    if ((uintptr_t)ring % 256) return fail(DFLASH_EINVAL, "ring must be 256-byte aligned");
    return reset_ring_w(*x, (char *)ring, x->W, (hipStream_t)stream);
}

size_t dflash_page_bytes(const dflash_config *cfg) {
    if (check_config(cfg) != DFLASH_OK || cfg->window % PAGE_SLOTS) return 0;
    return ring_bytes_w(*cfg, PAGE_SLOTS);
}

int dflash_set_paged_pool(dflash_ctx *x, void *pool, int32_t n_pages) {
    if (!x) return fail(DFLASH_EINVAL, "ctx is NULL");
    if (pool == nullptr) {
        x->paged = PagedPool{nullptr, 0, 0};
        return DFLASH_OK;
    }
    if (x->W % PAGE_SLOTS) return fail(DFLASH_EUNSUPPORTED, "paged KV needs a window that is a multiple of %d", PAGE_SLOTS);
    if ((uintptr_t)pool % 256) return fail(DFLASH_EINVAL, "pool must be 256-byte aligned");
    if (n_pages < 1) return fail(DFLASH_ERANGE, "n_pages=%d must be >= 1", n_pages);
    x->paged = PagedPool{(char *)pool, n_pages, ring_bytes_w(x->cfg, PAGE_SLOTS)};
    return DFLASH_OK;
}

int dflash_pages_reset(dflash_ctx *x, int32_t first, int32_t count, void *stream) {
    if (!x) return fail(DFLASH_EINVAL, "ctx is NULL");
    if (!x->paged.pool) return fail(DFLASH_ESTATE, "no page pool is set");
    if (first < 0 || count < 0 || first + count > x->paged.n_pages)
        return fail(DFLASH_ERANGE, "pages [%d, %d) outside 0..%d", first, first + count, x->paged.n_pages);
    for (int p = first; p < first + count; ++p)
        TRY(reset_ring_w(*x, x->paged.pool + (size_t)p * x->paged.page_bytes, PAGE_SLOTS, (hipStream_t)stream));
    return DFLASH_OK;
}

// Encode with caller-chosen scratch: `stage` holds the converted features (term planes of stage_rows
// rows) when the feature and fc dtypes need a conversion, `parts` the split-K partials [S][T][E] of the fc
// GEMM in at most parts_rows rows of E floats.
int encode_with(dflash_ctx &x, const void *feats, int T, float *h, hipStream_t s, void *stage, int stage_rows,
                float *parts, int parts_rows) {
    const dflash_config &c = x.cfg;
    const void *act = feats;
    int fmt;
    int act_rows = T;
    if (c.aux_dtype == DFLASH_F32) {
        fmt = ACT_F32;
        if (c.feature_dtype == DFLASH_BF16) {
            HIP_TRY(launch_bf16_to_f32((const uint16_t *)feats, (size_t)T * x.C, (float *)stage, s),
                    "feature conversion launch");
            act = stage;
        }
    } else if (c.feature_dtype == DFLASH_BF16) {
        fmt = ACT_BF16;
    } else {
        fmt = ACT_SPLIT3;
        act_rows = stage_rows;
        HIP_TRY(launch_split((const float *)feats, T, x.C, x.C, stage, ACT_SPLIT3, act_rows, s), "feature split launch");
        act = stage;
    }
    GemmArgs g = {};
    g.W = x.fc;
    g.N = x.E;
    g.K = x.C;
    g.M = T;
    g.act = act;
    g.act_rows = act_rows;
    g.out = parts;
    gemm_split(g, parts_rows);
    HIP_TRY(launch_gemm(c.aux_dtype, fmt, g, s), "encode GEMM launch");
    HIP_TRY(launch_rmsnorm_rows(parts, g.S, T, x.E, x.hidden_norm, c.rms_eps, h, s), "encode norm launch");
    return DFLASH_OK;
}

int check_encode_args(const dflash_ctx *x, const void *feats, int32_t T, const float *h) {
    if (!x || !feats || !h) return fail(DFLASH_EINVAL, "ctx, feats or h is NULL");
    if ((uintptr_t)feats % 16 || (uintptr_t)h % 16) return fail(DFLASH_EINVAL, "feats and h must be 16-byte aligned");
    if (T < 1 || T > x->cfg.max_inject) return fail(DFLASH_ERANGE, "T=%d outside 1..max_inject=%d", T, x->cfg.max_inject);
    return DFLASH_OK;
}

// Bytes of converted-feature staging an encode of T positions needs (0 when the features are used as
// they are): f32 copies of bf16 features, or the three-term bf16 split of f32 features.
size_t encode_stage_bytes(const dflash_ctx &x, int T) {
    const dflash_config &c = x.cfg;
    if (c.aux_dtype == DFLASH_F32) return c.feature_dtype == DFLASH_BF16 ? 4ull * T * x.C : 0;
    return c.feature_dtype == DFLASH_BF16 ? 0 : 6ull * T * x.C;
}

int dflash_encode(dflash_ctx *x, const void *feats, int32_t T, float *h, void *stream) {
    TRY(check_encode_args(x, feats, T, h));
    return encode_with(*x, feats, T, h, (hipStream_t)stream, x->enc_act, x->cfg.max_inject, x->enc_y,
                       x->cfg.max_inject);
}

int dflash_encode_static(dflash_ctx *x, const void *feats, int32_t T, float *h, void *stream) {
    TRY(check_encode_args(x, feats, T, h));
    const size_t stage = a256(encode_stage_bytes(*x, T));
    const size_t row = 4ull * x->E;  // one row of split-K partials
    if (stage + row * T > ENCODE_STATIC_SCRATCH_BYTES)
        return fail(DFLASH_ERANGE, "T=%d needs %zu bytes of static scratch, more than the %zu it holds", T,
                    stage + row * T, ENCODE_STATIC_SCRATCH_BYTES);
    char *base = (char *)x->static_scratch;  // this device's copy of `scratch`
    const int parts_rows = (int)std::min<size_t>((ENCODE_STATIC_SCRATCH_BYTES - stage) / row, 1u << 30);
    return encode_with(*x, feats, T, h, (hipStream_t)stream, base, T, (float *)(base + stage), parts_rows);
}

// The fused K/V projection of T encoded rows (one GEMM over every layer's wk/wv) and the ring writes: to
// `ring`, or (rings set) row t to rings[seq[t]].
int inject_rows(dflash_ctx &x, void *ring, void *const *rings, const int32_t *seq, int n_seq, const float *h,
                const int32_t *pos, int T, hipStream_t s) {
    const void *act = h;
    int act_rows = T;
    if (x.act_fmt == ACT_SPLIT3) {
        act_rows = x.cfg.max_inject;
        HIP_TRY(launch_split(h, T, x.E, x.E, x.inj_act, ACT_SPLIT3, act_rows, s), "inject split launch");
        act = x.inj_act;
    }
    GemmArgs g = {};
    g.W = x.kv;
    g.wscale = x.s_kv;
    g.N = x.L * 2 * x.kvdim;
    g.K = x.E;
    g.M = T;
    g.act = act;
    g.act_rows = act_rows;
    g.out = x.inj_kv;
    gemm_split(g, x.cfg.max_inject);
    HIP_TRY(launch_gemm(x.cfg.weight_dtype, x.act_fmt, g, s), "inject GEMM launch");
    HIP_TRY(launch_inject(&x, ring, rings, seq, n_seq, pos, T, g.S, s), "inject launch");
    return DFLASH_OK;
}

int dflash_inject(dflash_ctx *x, void *ring, const float *h, const int32_t *pos, int32_t T, void *stream) {
    if (!x || !ring || !h || !pos) return fail(DFLASH_EINVAL, "ctx, ring, h or pos is NULL");
    if ((uintptr_t)ring % (x->paged.pool ? 4 : 256))
        return fail(DFLASH_EINVAL, x->paged.pool ? "block table must be 4-byte aligned" : "ring must be 256-byte aligned");
    if (T < 1 || T > x->W || T > x->cfg.max_inject)
        return fail(DFLASH_ERANGE, "T=%d outside 1..min(window=%d, max_inject=%d)", T, x->W, x->cfg.max_inject);
    return inject_rows(*x, ring, nullptr, nullptr, 0, h, pos, T, (hipStream_t)stream);
}

int dflash_inject_batch(dflash_ctx *x, void *const *rings, int32_t n_seq, const int32_t *seq, const float *h,
                        const int32_t *pos, int32_t T, void *stream) {
    if (!x || !rings || !seq || !h || !pos) return fail(DFLASH_EINVAL, "ctx, rings, seq, h or pos is NULL");
    if (n_seq < 1) return fail(DFLASH_ERANGE, "n_seq=%d must be >= 1", n_seq);
    if (T < 1 || T > x->cfg.max_inject) return fail(DFLASH_ERANGE, "T=%d outside 1..max_inject=%d", T, x->cfg.max_inject);
    return inject_rows(*x, nullptr, rings, seq, n_seq, h, pos, T, (hipStream_t)stream);
}

int dflash_block_step(dflash_ctx *x, void *const *rings, const int32_t *id_last, const int32_t *n_past, int32_t B,
                      float *logits, int32_t *drafts, void *stream) {
    TRY(check_step_args(x, rings, id_last, n_past, B, logits, drafts));
    return run_step(*x, rings, id_last, nullptr, n_past, B, logits, drafts, nullptr, nullptr, (hipStream_t)stream);
}

int dflash_block_step_accept(dflash_ctx *x, void *const *rings, const int32_t *id_last, const int32_t *n_past,
                             int32_t B, float *logits, int32_t *drafts, const int32_t *target, int32_t *n_ok,
                             void *stream) {
    TRY(check_step_args(x, rings, id_last, n_past, B, logits, drafts));
    if (!target || !n_ok) return fail(DFLASH_EINVAL, "target or n_ok is NULL");
    return run_step(*x, rings, id_last, nullptr, n_past, B, logits, drafts, target, n_ok, (hipStream_t)stream);
}

int dflash_block_forward(dflash_ctx *x, void *const *rings, const int32_t *block_ids, const int32_t *n_past, int32_t B,
                         float *logits, int32_t *drafts, void *stream) {
    TRY(check_step_args(x, rings, block_ids, n_past, B, logits, drafts));
    return run_step(*x, rings, nullptr, block_ids, n_past, B, logits, drafts, nullptr, nullptr, (hipStream_t)stream);
}

int dflash_accept(dflash_ctx *x, const int32_t *drafts, const int32_t *target, int32_t B, int32_t *n_ok,
                  void *stream) {
    if (!x || !drafts || !target || !n_ok) return fail(DFLASH_EINVAL, "a pointer is NULL");
    if (B < 1 || B > x->cfg.max_batch) return fail(DFLASH_ERANGE, "B=%d outside 1..max_batch=%d", B, x->cfg.max_batch);
    HIP_TRY(launch_accept(drafts, target, B, x->gamma - 1, n_ok, (hipStream_t)stream), "accept launch");
    return DFLASH_OK;
}

int dflash_accept_bonus(dflash_ctx *x, const int32_t *drafts, const int32_t *target, int32_t B, int32_t *n_ok,
                        int32_t *bonus, void *stream) {
    if (!x || !drafts || !target || !n_ok || !bonus) return fail(DFLASH_EINVAL, "a pointer is NULL");
    if (B < 1 || B > x->cfg.max_batch) return fail(DFLASH_ERANGE, "B=%d outside 1..max_batch=%d", B, x->cfg.max_batch);
    HIP_TRY(launch_accept(drafts, target, B, x->gamma - 1, n_ok, (hipStream_t)stream, bonus), "accept launch");
    return DFLASH_OK;
}

int dflash_step_graph_create(dflash_ctx *x, void *const *rings, const int32_t *id_last, const int32_t *n_past,
                             int32_t B, float *logits, int32_t *drafts, const int32_t *target, int32_t *n_ok,
                             void *stream, dflash_graph **out) {
    if (!out) return fail(DFLASH_EINVAL, "out is NULL");
    *out = nullptr;
    TRY(check_step_args(x, rings, id_last, n_past, B, logits, drafts));
    if ((target == nullptr) != (n_ok == nullptr)) return fail(DFLASH_EINVAL, "target and n_ok go together");
    hipStream_t s = (hipStream_t)stream;
    if (s == nullptr) return fail(DFLASH_EINVAL, "graph capture needs a non-default stream");
    hipStreamCaptureStatus st;
    HIP_TRY(hipStreamIsCapturing(s, &st), "hipStreamIsCapturing");
    if (st != hipStreamCaptureStatusNone) return fail(DFLASH_ESTATE, "stream is already capturing");
    HIP_TRY(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal), "hipStreamBeginCapture");
    int r = run_step(*x, rings, id_last, nullptr, n_past, B, logits, drafts, target, n_ok, s);
    hipGraph_t graph = nullptr;
    hipError_t e = hipStreamEndCapture(s, &graph);
    if (r != DFLASH_OK) {
        if (graph) hipGraphDestroy(graph);
        return r;
    }
    if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        hipGraphDestroy(graph);
        return hip_fail(e, "hipGraphInstantiate");
    }
    dflash_graph *g = new dflash_graph();
    g->ctx = x;
    g->graph = graph;
    g->exec = exec;
    *out = g;
    return DFLASH_OK;
}

int dflash_step_graph_launch(dflash_graph *g, void *stream) {
    if (!g || !g->exec) return fail(DFLASH_EINVAL, "graph is NULL");
    HIP_TRY(hipGraphLaunch(g->exec, (hipStream_t)stream), "hipGraphLaunch");
    return DFLASH_OK;
}

void dflash_graph_destroy(dflash_graph *g) {
    if (!g) return;
    if (g->exec) hipGraphExecDestroy(g->exec);
    if (g->graph) hipGraphDestroy(g->graph);
    delete g;
}

int dflash_replay_stage(dflash_ctx *x, int32_t stage, int32_t layer, void *stream) {
    if (!x) return fail(DFLASH_EINVAL, "ctx is NULL");
    if (x->last_B < 1) return fail(DFLASH_ESTATE, "no block step has run on this ctx yet");
    if (layer < 0 || layer >= x->L) return fail(DFLASH_ERANGE, "layer %d outside 0..%d", layer, x->L - 1);
    const int M = 16 * x->last_B;
    hipStream_t s = (hipStream_t)stream;
    switch (stage) {
        case DFLASH_STAGE_QKV: return stage_qkv(*x, layer, M, s);
        case DFLASH_STAGE_O: return stage_o(*x, layer, M, s);
        case DFLASH_STAGE_GATE_UP: return stage_gu(*x, layer, M, s);
        case DFLASH_STAGE_DOWN: return stage_down(*x, layer, M, s);
        default: return fail(DFLASH_EINVAL, "unknown stage %d", stage);
    }
}

int dflash_set_block_width(dflash_ctx *x, int32_t gamma) {
    if (!x) return fail(DFLASH_EINVAL, "ctx is NULL");
    x->gamma = std::max(2, std::min((int)gamma, x->cfg.block));  // clamped into 2..block
    return DFLASH_OK;
}

int32_t dflash_block_width(const dflash_ctx *x) { return x ? x->gamma : 0; }

int dflash_set_sampling(dflash_ctx *x, float temperature, uint64_t seed) {
    if (!x) return fail(DFLASH_EINVAL, "ctx is NULL");
    if (!(temperature >= 0.0f) || !isfinite(temperature))
        return fail(DFLASH_EINVAL, "temperature must be finite and >= 0");
    x->temp = temperature;
    x->seed = seed;
    return DFLASH_OK;
}

int dflash_set_path(dflash_ctx *x, int32_t path) {
    if (!x) return fail(DFLASH_EINVAL, "ctx is NULL");
    if (path != DFLASH_PATH_AUTO && path != DFLASH_PATH_KERNELS && path != DFLASH_PATH_PERSISTENT)
        return fail(DFLASH_EINVAL, "unknown path %d", path);
    if (path == DFLASH_PATH_PERSISTENT && x->chain_wg < 1)
        return fail(DFLASH_EUNSUPPORTED, "the dataflow chain is not available for this configuration");
    x->path = path;
    return DFLASH_OK;
}

int32_t dflash_step_path(const dflash_ctx *x, int32_t B) {
    if (!x) return -1;
    return use_chain(*x, B) ? DFLASH_PATH_PERSISTENT : DFLASH_PATH_KERNELS;
}

int dflash_check_device(dflash_ctx *x, void *stream) {
    if (!x) return fail(DFLASH_EINVAL, "ctx is NULL");
    hipStream_t s = (hipStream_t)stream;
    HIP_TRY(hipStreamSynchronize(s), "hipStreamSynchronize");
    int err = 0;
    HIP_TRY(hipMemcpy(&err, x->csync + 1, sizeof err, hipMemcpyDeviceToHost), "device status read");
    if (err) {
        // a step gave up a wait: its flags and split-K counters may be left mid-way, so clear them all
        // (epoch back to 1) before the next step
        HIP_TRY(launch_fill_i32(x->csync, 0, x->n_csync, s), "chain state reset");
        HIP_TRY(launch_fill_i32(x->csync, 1, 1, s), "chain state reset");
        HIP_TRY(launch_fill_i32(x->counters, 0, x->n_counters, s), "counter reset");
        HIP_TRY(launch_fill_i32(x->written, 0, x->n_counters, s), "counter reset");
        HIP_TRY(launch_fill_i32((int *)x->xslot, (int)XSLOT_EMPTY, x->n_xslot, s), "exchange slot reset");
        HIP_TRY(hipStreamSynchronize(s), "chain state reset");
        return fail(DFLASH_ESTATE, "a bounded wait on the device (the dataflow chain, or a split-K hand-off) gave "
                                   "up; the outputs of the steps since the last check are invalid");
    }
    return DFLASH_OK;
}

int dflash_set_wait_limit(dflash_ctx *x, int64_t microseconds, void *stream) {
    if (!x) return fail(DFLASH_EINVAL, "ctx is NULL");
    if (microseconds < 0) return fail(DFLASH_EINVAL, "wait limit must be >= 0");
    if (x->chain_wg < 1) return fail(DFLASH_EUNSUPPORTED, "the dataflow chain is not available for this configuration");
    int rate_khz = 0;
    HIP_TRY(hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, x->device), "wall clock rate query");
    const long long ticks = (long long)((double)microseconds * rate_khz / 1000.0);
    hipStream_t s = (hipStream_t)stream;
    HIP_TRY(hipMemcpyAsync((char *)x->cargs + offsetof(ChainArgs, spin_ticks), &ticks, sizeof ticks,
                           hipMemcpyHostToDevice, s),
            "wait limit upload");
    HIP_TRY(hipStreamSynchronize(s), "wait limit upload");
    return DFLASH_OK;
}

int dflash_quantize_fp8_rows(const float *w, int32_t rows, int32_t cols, uint8_t *codes, float *scales, void *stream) {
    if (!w || !codes || !scales) return fail(DFLASH_EINVAL, "a pointer is NULL");
    if (rows < 1 || cols < 1) return fail(DFLASH_EINVAL, "rows and cols must be positive");
    HIP_TRY(launch_quantize_fp8(w, rows, cols, codes, scales, (hipStream_t)stream), "quantize launch");
    return DFLASH_OK;
}

}  // extern "C"
