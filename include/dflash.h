/*
 * dflash.h -- C ABI of the DFlash block-diffusion drafter block step for AMD
 * Instinct MI355X (gfx950).
 *
 * The operations follow the dflash-ops card (Hugging Face kernels hub):
 *   - "Usage": encode fused target features, inject them into the ring,
 *     run the graphed block step on [id_last, mask x 15], take greedy
 *     drafts at block positions 1..15, and count accepted drafts on the device;
 *   - "Method": injection through wk/wv with no attention norm, K per-head
 *     RMS-normed and NEOX-roped, V raw; non-causal block attention; the window
 *     masks only the deep past (0 <= qpos - kpos < window); rope angles from a
 *     host fp64 inverse-frequency table; fp32 arithmetic whatever the storage
 *     dtype; the captured step allocates nothing;
 *   - "Requirements and limits": slot = pos % window, at most window tokens
 *     per inject call, later calls overwrite.
 * The cross-sequence batch (sequence-major rows, weight GEMMs once over all
 * rows, attention / slot writes / acceptance per sequence) follows the metrale
 * dflash_head.rs page, DflashBatch; weight-only FP8 E4M3 with per-row f32
 * scales follows its DflashQuantization.
 *
 * Conventions for every entry point:
 *   - All pointers are DEVICE pointers unless the comment says "host".
 *   - `stream` is a hipStream_t (passed as void* so this header needs no HIP
 *     include). Every call is asynchronous on that stream; nothing is
 *     allocated; no host synchronisation happens except where stated.
 *   - The caller owns all memory: weights, workspace, rings, inputs, outputs.
 *   - Host-checkable errors return a negative dflash_status before any launch
 *     and leave a message for dflash_last_error() (thread-local).
 *   - Matrices are row-major [out, in] (the PyTorch / GGUF order); vectors are
 *     dense.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DFLASH_OK = 0,
    DFLASH_EINVAL = -1,       /* NULL pointer, bad dtype, inconsistent shape */
    DFLASH_ERANGE = -2,       /* T > window or T > max_inject, B > max_batch, buffer too small */
    DFLASH_EUNSUPPORTED = -3, /* a shape the kernels do not support (see dflash_config) */
    DFLASH_EHIP = -4,         /* a HIP runtime call failed; the message names it */
    DFLASH_ESTATE = -5        /* object used in the wrong state (e.g. capture already active) */
} dflash_status;

typedef enum {
    DFLASH_F32 = 0,
    DFLASH_BF16 = 1,
    DFLASH_FP8_E4M3 = 2 /* OCP E4M3FN (max 448, no infinities); NaN codes are not supported */
} dflash_dtype;

/*
 * Drafter geometry and storage dtypes.
 *
 * Supported shapes: head_dim 64 or 128; n_head a multiple of n_head_kv with
 * n_head / n_head_kv <= 4; block == 16; n_embd, n_ff, n_vocab,
 * n_capture * target_hidden, n_head * head_dim and n_head_kv * head_dim
 * multiples of 64; window a multiple of 64 and <= 65536; 1 <= max_batch <= 8.
 */
typedef struct dflash_config {
    int32_t n_layer;       /* drafter layers (5 for the released drafter) */
    int32_t n_embd;        /* drafter hidden size E */
    int32_t n_head;        /* query heads */
    int32_t n_head_kv;     /* key/value heads (GQA: q head h uses kv head h / (n_head / n_head_kv)) */
    int32_t head_dim;      /* D; rope covers the whole head */
    int32_t n_ff;          /* SwiGLU width F */
    int32_t window;        /* ring slots W per layer */
    int32_t block;         /* noise block length (16) */
    int32_t n_vocab;       /* rows of tok_embd and lm_head */
    int32_t n_capture;     /* captured target layers (5) */
    int32_t target_hidden; /* target hidden size; fused features are [T, n_capture * target_hidden] */
    int32_t mask_id;       /* token id of the 15 mask positions */
    int32_t max_batch;     /* largest B passed to the block step */
    int32_t max_inject;    /* largest T passed to encode / inject (<= window for inject) */
    float rms_eps;         /* RMSNorm epsilon (1e-6) */
    double rope_base;      /* rope theta; inverse frequencies base^(-2i/D) are built in fp64 on the host */
    int32_t weight_dtype;  /* wq wk wv wo w_gate w_up w_down lm_head: F32, BF16 or FP8_E4M3 */
    int32_t aux_dtype;     /* tok_embd, fc and every norm vector: F32 or BF16 */
    int32_t ring_dtype;    /* ring K/V storage: F32 or BF16 */
    int32_t feature_dtype; /* fused target features: F32 or BF16 */
} dflash_config;

/* One layer's weights (metrale dflash_head.rs page, DflashLayer; no biases).
 * Matrices: wq [H*D, E], wk/wv [Hkv*D, E], wo [E, H*D], w_gate/w_up [F, E],
 * w_down [E, F], in weight_dtype. Norm vectors (aux_dtype): attn_norm [E],
 * q_norm/k_norm [D], ffn_norm [E]. s_*: FP8 per-row scales [rows] (f32),
 * required when weight_dtype is FP8_E4M3 and ignored otherwise. */
typedef struct dflash_layer_weights {
    const void *attn_norm, *wq, *wk, *wv, *wo, *q_norm, *k_norm, *ffn_norm, *w_gate, *w_up, *w_down;
    const float *s_q, *s_k, *s_v, *s_o, *s_gate, *s_up, *s_down;
} dflash_layer_weights;

/* Global weights. tok_embd [V, E] (aux_dtype) and lm_head [V, E]
 * (weight_dtype, scales s_lm_head for FP8) are the target model's; fc
 * [E, n_capture*target_hidden], hidden_norm [E] and output_norm [E] are the
 * drafter's (aux_dtype). `layers` is a HOST array of n_layer entries. */
typedef struct dflash_weights {
    const void *tok_embd, *lm_head, *fc, *hidden_norm, *output_norm;
    const float *s_lm_head;
    const dflash_layer_weights *layers;
} dflash_weights;

typedef struct dflash_ctx dflash_ctx;
typedef struct dflash_graph dflash_graph;

/* Bytes of device workspace dflash_create needs for `cfg`, or 0 if cfg is
 * invalid (dflash_last_error says why). The workspace holds the re-tiled
 * copies of every weight matrix the kernels stream, fp32 copies of the norm
 * vectors, the fp64 inverse-frequency table and every intermediate of
 * encode / inject / block step. It must be 256-byte aligned. */
size_t dflash_workspace_bytes(const dflash_config *cfg);

/* Bytes of one sequence's ring: K and V [n_layer][n_kv][window][head_dim] in
 * ring_dtype, then int32 slot_pos[window] (the position each slot holds, -1
 * when empty). 256-byte alignment required. Slot s holds -1 or a position p
 * >= 0 with p % window == s, as dflash_inject and dflash_ring_reset leave it;
 * the block step relies on this to skip slots at or past n_past + 16, which
 * no block row can see (a ring written by other means must keep it). */
size_t dflash_ring_bytes(const dflash_config *cfg);

/* Validate cfg, carve the caller's workspace and, on `stream`, re-tile every
 * weight matrix into it (the streaming layout of the step kernels) and copy
 * the norm vectors as fp32. The inverse-frequency table is computed on the
 * host in fp64 and uploaded with a synchronous copy. After the stream has
 * drained, the library reads only tok_embd from `w`; every other weight
 * buffer may be freed. *out receives a host handle; free it with
 * dflash_destroy. The handle may be used from one host thread at a time. */
int dflash_create(const dflash_config *cfg, const dflash_weights *w, void *workspace, size_t workspace_bytes,
                  void *stream, dflash_ctx **out);
void dflash_destroy(dflash_ctx *ctx);

/* Mark every slot of `ring` empty (slot_pos[] = -1) and zero its K/V
 * storage. Empty slots get attention weight exactly 0; zeroed storage keeps
 * their contribution 0 (an arbitrary bit pattern could be NaN). A ring must be
 * reset once before its first inject. ESTATE in paged mode (reset pages with
 * dflash_pages_reset). */
int dflash_ring_reset(dflash_ctx *ctx, void *ring, void *stream);

/* Cross-layer feature fusion (dflash_engine.py page, TargetContextFeatureFuser):
 * h = RMSNorm(feats . fc^T) * hidden_norm. feats [T, n_capture*target_hidden]
 * in feature_dtype, h [T, n_embd] f32, both device buffers 16-byte aligned
 * (EINVAL otherwise). 1 <= T <= max_inject (ERANGE otherwise). */
int dflash_encode(dflash_ctx *ctx, const void *feats, int32_t T, float *h, void *stream);

/* dflash_encode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same operation and arguments, but its scratch -- the converted
 * features and the fc GEMM's split-K partials -- lives in a static device
 * array of 64 MiB that the library holds on every GPU it runs on until the
 * process ends, instead of in the ctx's workspace. No call allocates (no
 * hipMalloc, no allocating library routine). ERANGE when T positions need
 * more than the 64 MiB (one f32 row of n_embd per position, plus n_capture *
 * target_hidden * 4 bytes per position for bf16 features with f32 fc, or * 6
 * for f32 features with bf16 fc). All calls on one GPU share the one array:
 * calls that overlap on one GPU (other streams, other ctxs, other threads)
 * race and must be serialised by the caller; nothing in the array needs to
 * start at zero. */
int dflash_encode_static(dflash_ctx *ctx, const void *feats, int32_t T, float *h, void *stream);

/* KV injection (dflash-ops card, Method; Requirements and limits): for every
 * layer l, position t and kv head j, k = rope(RMSNorm(h_t . wk_l^T)[j] *
 * k_norm_l, pos_t) and v = (h_t . wv_l^T)[j], rounded to ring_dtype and stored
 * at slot pos_t % window; slot_pos[slot] = pos_t. h [T, n_embd] f32, pos [T]
 * int32. 1 <= T <= min(window, max_inject). Device preconditions (not
 * checked): positions of one call map to distinct slots; a negative position
 * is skipped. */
int dflash_inject(dflash_ctx *ctx, void *ring, const float *h, const int32_t *pos, int32_t T, void *stream);

/* Batched context precompute (metrale dflash_head.rs page, PRECOMPUTE_BATCH_ROWS
 * and batched_precompute_enabled: one fc + fused-KV pass over every
 * sequence's uncommitted context rows): the injection of dflash_inject for T
 * rows that belong to several sequences, with one fused K/V projection over
 * all of them. Row t (h[t], pos[t]) goes to the ring (in paged mode: the block
 * table) rings[seq[t]]; rings is a device array [n_seq] of ring pointers (or
 * of int32 block-table pointers), seq [T] int32 device. Encode the rows
 * beforehand with one dflash_encode call over their concatenated features.
 * 1 <= T <= max_inject (ERANGE otherwise); n_seq >= 1. Device preconditions
 * (not checked): the rows of one sequence map to distinct slots; a row with a
 * negative position or a sequence index outside 0..n_seq-1 is skipped. Each
 * ring's result equals injecting its own rows with dflash_inject (up to fp32
 * summation order of the projection). */
int dflash_inject_batch(dflash_ctx *ctx, void *const *rings, int32_t n_seq, const int32_t *seq, const float *h,
                        const int32_t *pos, int32_t T, void *stream);

/* The drafter block step (dflash-ops card, Usage: the step on the noise block
 * [id_last, mask x 15] returns logits [16, n_vocab] and greedy drafts at block
 * positions 1..15; Method: the block attends non-causally to itself and to the
 * ring, whose window masks only the deep past) for B sequences (rows
 * sequence-major, 16 per sequence; metrale dflash_head.rs page, DflashBatch). rings: device array [B] of ring pointers; id_last [B] and
 * n_past [B] int32 (device, so a graph replays with fresh values). With the
 * block width g of dflash_set_block_width (16 unless set), block row i < g of
 * sequence b holds [id_last, mask...][i] at position n_past[b] + i and
 * attends non-causally to block rows 0..g-1 and to the ring slots with
 * 0 <= n_past[b] + i - slot_pos < window; rows g..15 are padding that no row
 * attends to. Outputs logits [16*B, n_vocab] f32 (rows g..15 of a sequence
 * hold padding values) and drafts [B, g-1] int32 = argmax of rows 1..g-1
 * (ties to the lowest index). Ids outside [0, n_vocab) embed as zero vectors.
 * 1 <= B <= max_batch. */
int dflash_block_step(dflash_ctx *ctx, void *const *rings, const int32_t *id_last, const int32_t *n_past, int32_t B,
                      float *logits, int32_t *drafts, void *stream);

/* dflash_block_step followed by the first-mismatch acceptance of
 * dflash_accept (dflash-ops card, Usage; dflash_engine.py page,
 * DFlashSpeculativeVerifier.verify_block), launched directly on `stream`:
 * the scan runs inside the logits launch (in the last workgroup to finish a
 * sequence's logits), as in a graph captured with target and n_ok. target [B, g-1] int32 (device) holds the
 * target's tokens at the draft positions; n_ok [B] int32 (device) receives
 * the number of leading draft positions that match. The other arguments,
 * outputs and errors are those of dflash_block_step; target and n_ok must be
 * non-NULL. */
int dflash_block_step_accept(dflash_ctx *ctx, void *const *rings, const int32_t *id_last, const int32_t *n_past,
                             int32_t B, float *logits, int32_t *drafts, const int32_t *target, int32_t *n_ok,
                             void *stream);

/* As dflash_block_step but with explicit block ids [B, 16] (device) instead
 * of id_last: a hook for testing joint (non-causal) denoising (dflash-ops
 * card, Correctness: a change at a later block position must move the logits
 * of earlier positions). */
int dflash_block_forward(dflash_ctx *ctx, void *const *rings, const int32_t *block_ids, const int32_t *n_past,
                         int32_t B, float *logits, int32_t *drafts, void *stream);

/* First-mismatch acceptance (dflash-ops card, Usage; dflash_engine.py page,
 * DFlashSpeculativeVerifier.verify_block): n_ok[b] = number of leading i with
 * drafts[b][i] == target[b][i], in 0..g-1 for the block width g in use.
 * drafts, target [B, g-1] int32. */
int dflash_accept(dflash_ctx *ctx, const int32_t *drafts, const int32_t *target, int32_t B, int32_t *n_ok,
                  void *stream);

/* Acceptance with the bonus token (dflash_engine.py page,
 * DFlashSpeculativeVerifier.verify_block): target [B, g] int32 holds the
 * target's tokens at the g-1 draft positions and at the position after them.
 * n_ok[b] as dflash_accept; bonus[b] = target[b][n_ok[b]], the target's token
 * at the first mismatch (or after the last draft when all match), so the
 * accepted run is drafts[b][0..n_ok[b]) followed by bonus[b], tau = n_ok + 1
 * tokens. drafts [B, g-1], n_ok and bonus [B] int32, all device. */
int dflash_accept_bonus(dflash_ctx *ctx, const int32_t *drafts, const int32_t *target, int32_t B, int32_t *n_ok,
                        int32_t *bonus, void *stream);

/* Capture the block step (and, when target and n_ok are non-NULL, the
 * acceptance scan) for fixed pointers into a HIP graph by stream capture on
 * `stream` (dflash-ops card, Usage: capture_step; Method: the captured step
 * allocates nothing and a replay reads fresh inputs from fixed buffers). Nothing is allocated inside the capture; every intermediate
 * lives in the workspace. Replay with dflash_step_graph_launch after writing
 * fresh values into id_last / n_past / target. The graph reads the ctx's
 * workspace, so the ctx must outlive it and no other call on the same ctx may
 * overlap a replay. */
int dflash_step_graph_create(dflash_ctx *ctx, void *const *rings, const int32_t *id_last, const int32_t *n_past,
                             int32_t B, float *logits, int32_t *drafts, const int32_t *target, int32_t *n_ok,
                             void *stream, dflash_graph **out);
int dflash_step_graph_launch(dflash_graph *g, void *stream);
void dflash_graph_destroy(dflash_graph *g);

/* Weight-only FP8 (metrale dflash_head.rs page, DflashQuantization): for
 * each row r of w [rows, cols] f32, scales[r] = amax_r / 448 (1 for an
 * all-zero row) and codes[r][c] = E4M3FN(w[r][c] / scales[r]), rounded to
 * nearest even and saturated at +-448; both divisions in IEEE fp32. */
int dflash_quantize_fp8_rows(const float *w, int32_t rows, int32_t cols, uint8_t *codes, float *scales,
                             void *stream);

/* How a block step runs. DFLASH_PATH_KERNELS: one kernel per projection,
 * attention and combine (about six per layer). DFLASH_PATH_PERSISTENT, for a
 * single sequence (B == 1): the dataflow chain, 2 * n_layer + 1 launches (the
 * embedding with layer 0's q/k/v; per layer the attention, then one launch of
 * Wo, gate/up, down and the next q/k/v or the lm_head). A chain launch holds
 * as many workgroups as the GPU runs at once; each takes one column group and
 * k-split of every projection in turn, issues its first weight loads, and
 * waits only for the column groups that produce its slice of the input
 * (per-group done flags), so one projection's tail overlaps the next one's
 * weight stream. These waits are bounded in time (one second unless
 * dflash_set_wait_limit says otherwise); a wait that gives up raises a sticky
 * error that dflash_check_device reports. The dflash-ops card (Requirements
 * and limits) names a fused whole-block persistent kernel as not implemented
 * there; this is this library's form of it. Both paths compute the same
 * operations with the same operand splits; their reductions may split at
 * different points, so results agree to fp32 rounding. DFLASH_PATH_AUTO (the
 * default) takes the faster path measured for this library, currently the
 * per-launch kernels. */
typedef enum { DFLASH_PATH_AUTO = 0, DFLASH_PATH_KERNELS = 1, DFLASH_PATH_PERSISTENT = 2 } dflash_path;

/* Choose the path of later block steps (and of graphs captured later).
 * EUNSUPPORTED for DFLASH_PATH_PERSISTENT when the dataflow chain does not
 * fit this configuration or device. */
int dflash_set_path(dflash_ctx *ctx, int32_t path);

/* Block width g (metrale dflash_head.rs page, BlockDiffusionDraftHead,
 * block_g / set_block_g and its per-width propose graphs): later block steps,
 * acceptance scans and graph captures use g tokens [id_last, mask x (g-1)]
 * and g-1 drafts. g is clamped into 2..block (16). A graph keeps the width it
 * was captured with. dflash_block_width returns the width in use (0 for a
 * NULL ctx). */
int dflash_set_block_width(dflash_ctx *ctx, int32_t g);
int32_t dflash_block_width(const dflash_ctx *ctx);

/* Draft sampling (dflash_engine.py page, DFlashDraftModel.forward: greedy at
 * temperature 0, otherwise a draw from softmax(logits / T)): later block steps
 * and graph captures take draft i of sequence b as the argmax over the
 * vocabulary of logits[i] / T + G, with G = -log(-log(u)) Gumbel noise and
 * u = ((x >> 8) + 1/2) * 2^-24, x the first output word of Philox-4x32-10
 * (Salmon et al., SC 2011) at counter (n_past[b] + i, vocab id, b, 0) under key
 * (seed & 0xffffffff, seed >> 32); ties to the lowest index. The logits output
 * stays the unperturbed logits. temperature must be finite and >= 0 (0:
 * greedy), else DFLASH_EINVAL. */
int dflash_set_sampling(dflash_ctx *ctx, float temperature, uint64_t seed);

/* Paged drafter KV (metrale dflash_head.rs page, DflashBatch: a drafter block
 * table per sequence, one table for all layers). A page holds 128 ring slots
 * of every layer in the ring layout above (K [L][Hkv][128][D], V, slot_pos
 * [128], each region 256-byte aligned): dflash_page_bytes of the config bytes
 * (0 if window is not a multiple of 128). After dflash_set_paged_pool(ctx,
 * pool, n_pages) with a non-NULL, 256-byte aligned device pool of n_pages
 * pages, the `ring` of dflash_inject and the entries of `rings` of the step
 * calls are device block tables instead: int32 [window / 128] page ids, slot s
 * of the sequence living in page table[s / 128] at slot s % 128. A table
 * entry outside 0..n_pages-1 makes its 128 slots empty (injection there is
 * dropped); pages must not be shared by two live tables. Reset pages before
 * their first use with dflash_pages_reset (zeroes K/V, slot_pos = -1; an
 * invalid entry reads page 0's memory under an all-masked chunk, so page 0
 * must hold finite values). pool NULL returns to contiguous rings; the mode
 * applies to later calls and captures. EUNSUPPORTED if window % 128 != 0. */
size_t dflash_page_bytes(const dflash_config *cfg);
int dflash_set_paged_pool(dflash_ctx *ctx, void *pool, int32_t n_pages);
int dflash_pages_reset(dflash_ctx *ctx, int32_t first, int32_t count, void *stream);

/* The path (DFLASH_PATH_KERNELS or DFLASH_PATH_PERSISTENT) a block step of B
 * sequences takes now; -1 for a NULL ctx. */
int32_t dflash_step_path(const dflash_ctx *ctx, int32_t B);

/* Synchronise `stream` and report whether a bounded device wait gave up since
 * the last check: a dataflow-chain wait (e.g. when other work holds compute
 * units so that not every chain workgroup is resident), or the wait of a
 * per-launch gate/up projection's last k-split for the other splits' partial
 * tiles (which those splits store right after taking their place, so it ends
 * unless the device is faulty): ESTATE if so. The error word is sticky: every
 * chain step after the failing one also gives up its waits at once and leaves
 * invalid outputs, until this call reports the error, clears it and resets the
 * flags and split-K counters, after which steps are valid again. OK
 * otherwise. */
int dflash_check_device(dflash_ctx *ctx, void *stream);

/* Wall-clock limit of each bounded wait of the dataflow chain, in
 * microseconds (default 1000000). A test and tuning hook: a limit of 0 makes
 * every wait that is not satisfied at once give up, so failure handling can be
 * exercised with every kernel ending normally. Synchronises `stream`.
 * EUNSUPPORTED when the chain is not available. */
int dflash_set_wait_limit(dflash_ctx *ctx, int64_t microseconds, void *stream);

/* Stages of the block step that dflash_replay_stage can re-run. */
typedef enum {
    DFLASH_STAGE_QKV = 0,     /* fused q/k/v projection of one layer (attention-norm folded in) */
    DFLASH_STAGE_O = 1,       /* output projection + residual (+ ffn-norm input of the next stage) */
    DFLASH_STAGE_GATE_UP = 2, /* gate/up projection + SwiGLU */
    DFLASH_STAGE_DOWN = 3     /* down projection + residual (+ next layer's norm input) */
} dflash_stage;

/* Re-run one weight-streaming stage of layer `layer` of the last block step
 * on the activations the workspace holds now, with that step's batch; a
 * timing hook for a single kernel (the per-launch kernel of that stage, as
 * DFLASH_PATH_KERNELS runs it). DFLASH_STAGE_GATE_UP and DFLASH_STAGE_QKV leave the step's state
 * consistent; DFLASH_STAGE_O and DFLASH_STAGE_DOWN add into the residual
 * stream again, so run a full step before reading results. ESTATE before the
 * first block step. */
int dflash_replay_stage(dflash_ctx *ctx, int32_t stage, int32_t layer, void *stream);

/* Message of the last failed call on this thread ("" if none). */
const char *dflash_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
