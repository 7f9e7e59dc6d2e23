// Non-GEMM kernels of the DFlash drafter on gfx950: embedding of the noise
// block, non-causal sliding-window GQA attention of the block against ring
// plus block, ring injection (per-head RMSNorm, NEOX rope, slot scatter),
// encode's row RMSNorm, activation conversion, and the acceptance scan.
#include <algorithm>

#include "dflash_internal.h"

// ---------------------------------------------------------------------------
// Ring layout: K [L][Hkv][W][D], V [L][Hkv][W][D] (ring dtype), slot_pos [W]
// ---------------------------------------------------------------------------
// (helpers ring_v_offset / ring_pos_offset in dflash_internal.h)

__device__ __forceinline__ float ring_load(const void *base, int ring_dtype, size_t i) {
    return ring_dtype == DFLASH_BF16 ? bf16_to_f32(((const uint16_t *)base)[i]) : ((const float *)base)[i];
}
__device__ __forceinline__ void ring_store(void *base, int ring_dtype, size_t i, float v) {
    if (ring_dtype == DFLASH_BF16)
        ((uint16_t *)base)[i] = f32_to_bf16(v);
    else
        ((float *)base)[i] = v;
}

// ---------------------------------------------------------------------------
// Small utilities
// ---------------------------------------------------------------------------
__global__ void fill_i32_kernel(int32_t *p, int32_t v, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

hipError_t launch_fill_i32(int32_t *p, int32_t v, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    unsigned blocks = (unsigned)min((n + 255) / 256, (size_t)4096);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(blocks), dim3(256), 0, s, p, v, n);
    return hipGetLastError();
}

__global__ void vec_to_f32_kernel(const void *src, int dtype, int n, float *dst) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = dtype == DFLASH_BF16 ? bf16_to_f32(((const uint16_t *)src)[i]) : ((const float *)src)[i];
}

hipError_t launch_vec_to_f32(const void *src, int dtype, int n, float *dst, hipStream_t s) {
    hipLaunchKernelGGL(vec_to_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, src, dtype, n, dst);
    return hipGetLastError();
}

__global__ void bf16_to_f32_kernel(const uint16_t *src, size_t n, float *dst) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        dst[i] = bf16_to_f32(src[i]);
}

hipError_t launch_bf16_to_f32(const uint16_t *src, size_t n, float *dst, hipStream_t s) {
    unsigned blocks = (unsigned)min((n + 255) / 256, (size_t)8192);
    hipLaunchKernelGGL(bf16_to_f32_kernel, dim3(blocks), dim3(256), 0, s, src, n, dst);
    return hipGetLastError();
}

// f32 [rows][ld_src] -> activation format (split into three bf16 planes, or f32 copy)
__global__ void split_kernel(const float *src, int rows, int K, int ld_src, void *dst, int fmt, int act_rows) {
    const size_t n = (size_t)rows * K;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        const int r = (int)(i / K), c = (int)(i % K);
        const float v = src[(size_t)r * ld_src + c];
        if (fmt == ACT_F32) {
            ((float *)dst)[(size_t)r * K + c] = v;
        } else {
            uint16_t t0, t1, t2;
            split3(v, t0, t1, t2);
            uint16_t *p = (uint16_t *)dst;
            const size_t plane = (size_t)act_rows * K;
            p[(size_t)r * K + c] = t0;
            p[plane + (size_t)r * K + c] = t1;
            p[2 * plane + (size_t)r * K + c] = t2;
        }
    }
}

hipError_t launch_split(const float *src, int rows, int K, int ld_src, void *dst, int act_fmt, int act_rows,
                        hipStream_t s) {
    size_t n = (size_t)rows * K;
    unsigned blocks = (unsigned)min((n + 255) / 256, (size_t)8192);
    hipLaunchKernelGGL(split_kernel, dim3(blocks), dim3(256), 0, s, src, rows, K, ld_src, dst, act_fmt, act_rows);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Encode: h = y * rsqrt(mean(y^2) + eps) * w   (one workgroup per row)
// ---------------------------------------------------------------------------
// y holds S k-split partials [S][T][E], summed here in split order first.
// Each thread takes float4 columns c and c + 256 of the row at once and issues
// the loads of up to eight splits of both together before adding them in
// split order (E is a multiple of 64, so a row is whole float4 words).
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const float *y, int S, int T, int E, const float *w,
                                                           float eps, float *h) {
    constexpr int U = 2, SB = 8;
    const int t = blockIdx.x, E4 = E / 4;
    const float4 *y4 = (const float4 *)y;
    float4 *h4 = (float4 *)(h + (size_t)t * E);
    float ss = 0.0f;
    for (int c0 = threadIdx.x; c0 < E4; c0 += 256 * U) {
        float4 v[U];
        for (int s0 = 0; s0 < S; s0 += SB) {
            float4 p[SB][U];
#pragma unroll
            for (int j = 0; j < SB; ++j)
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = c0 + 256 * u;
                    p[j][u] = (s0 + j < S && c < E4) ? y4[((size_t)(s0 + j) * T + t) * E4 + c]
                                                     : make_float4(0.f, 0.f, 0.f, 0.f);
                }
#pragma unroll
            for (int j = 0; j < SB; ++j)
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (s0 + j == 0) {
                        v[u] = p[j][u];
                    } else if (s0 + j < S) {
                        v[u].x += p[j][u].x;
                        v[u].y += p[j][u].y;
                        v[u].z += p[j][u].z;
                        v[u].w += p[j][u].w;
                    }
                }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + 256 * u;
            if (c < E4) {
                h4[c] = v[u];
                ss += v[u].x * v[u].x + v[u].y * v[u].y + v[u].z * v[u].z + v[u].w * v[u].w;
            }
        }
    }
    ss = wave_sum(ss);
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float r = 1.0f / sqrtf(tot / (float)E + eps);
    const float4 *w4 = (const float4 *)w;
    for (int c = threadIdx.x; c < E4; c += 256) {  // the words this thread wrote above
        const float4 x = h4[c], g = w4[c];
        h4[c] = make_float4(x.x * r * g.x, x.y * r * g.y, x.z * r * g.z, x.w * r * g.w);
    }
}

hipError_t launch_rmsnorm_rows(const float *y, int S, int T, int E, const float *w, float eps, float *h,
                               hipStream_t s) {
    hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3(T), dim3(256), 0, s, y, S, T, E, w, eps, h);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-head RMSNorm + NEOX rope of one D-vector held by one wavefront.
// D = 128: lane holds elements lane and lane + 64 (a rope pair).
// D = 64:  lane holds element lane; its pair partner lives in lane ^ 32.
// cs: [D/2][2] (cos, sin) of this vector's position.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void head_norm_rope(float (&x)[D / 64], const float *nw, const float *cs, float eps,
                                               int lane) {
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) ss += x[e] * x[e];
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
    for (int e = 0; e < D / 64; ++e) x[e] = x[e] * r * nw[lane + 64 * e];
    if constexpr (D == 128) {
        const float c = cs[2 * lane], s = cs[2 * lane + 1];
        const float x1 = x[0], x2 = x[1];
        x[0] = x1 * c - x2 * s;
        x[1] = x1 * s + x2 * c;
    } else {
        const float partner = __shfl_xor(x[0], 32, 64);
        const int i = lane & 31;
        const float c = cs[2 * i], s = cs[2 * i + 1];
        x[0] = lane < 32 ? x[0] * c - partner * s : partner * s + x[0] * c;
    }
}

// ---------------------------------------------------------------------------
// Inject (dflash-ops card, Method; Requirements and limits)
// ---------------------------------------------------------------------------
// Grid (T, L), 256 threads. kv row t holds [K_0 | V_0 | K_1 | V_1 | ...],
// each kvdim wide. Wave w handles kv heads w, w+4, ... The rope angle is
// pos * inv_freq[f] in fp64 and its sine and cosine are taken in fp64.
template <int D>
// kv holds S k-split partials [S][T][L*2*Hkv*D] of the projection, summed here in split order. With `rings`
// set (a batched injection), row t goes to sequence seq[t]'s ring (or block table) rings[seq[t]] and a row
// whose sequence index lies outside 0..n_seq-1 is skipped; otherwise every row goes to `ring`.
__global__ __launch_bounds__(256) void inject_kernel(const float *__restrict__ kv, int S, int T, int L, int Hkv, int W,
                                                     const int32_t *__restrict__ pos,
                                                     const double *__restrict__ inv_freq,
                                                     const float *__restrict__ k_norm_all, float eps, void *ring,
                                                     void *const *rings, const int32_t *__restrict__ seq, int n_seq,
                                                     int ring_dtype, PagedPool pp) {
    const int t = blockIdx.x, l = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = pos[t];
    if (p < 0) return;
    if (rings != nullptr) {
        const int q = seq[t];
        if (q < 0 || q >= n_seq) return;
        ring = rings[q];
    }
    const RingLoc loc = ring_locate(ring, pp, W, p % W);
    if (!loc.ok) return;  // a page id outside the pool: the write is dropped
    const int slot = loc.slot;
    __shared__ float cs[D];
    for (int f = tid; f < D / 2; f += 256) {
        double sn, cn;
        sincos((double)p * inv_freq[f], &sn, &cn);
        cs[2 * f] = (float)cn;
        cs[2 * f + 1] = (float)sn;
    }
    __syncthreads();
    const int es = ring_dtype == DFLASH_BF16 ? 2 : 4;
    const size_t kvdim = (size_t)Hkv * D;
    const float *row = kv + (size_t)t * L * 2 * kvdim + (size_t)l * 2 * kvdim;
    const size_t split = (size_t)T * L * 2 * kvdim;  // floats between partials
    char *rb = loc.base;
    void *Kb = rb;
    void *Vb = rb + ring_v_offset(L, Hkv, loc.W, D, es);
    const float *kn = k_norm_all + (size_t)l * D;
    for (int j = wave; j < Hkv; j += 4) {
        float x[D / 64], v[D / 64];
#pragma unroll
        for (int e = 0; e < D / 64; ++e) {
            x[e] = row[(size_t)j * D + lane + 64 * e];
            v[e] = row[kvdim + (size_t)j * D + lane + 64 * e];
            for (int sp = 1; sp < S; ++sp) {
                x[e] += row[sp * split + (size_t)j * D + lane + 64 * e];
                v[e] += row[sp * split + kvdim + (size_t)j * D + lane + 64 * e];
            }
        }
        head_norm_rope<D>(x, kn, cs, eps, lane);
        const size_t base = (((size_t)l * Hkv + j) * loc.W + slot) * D;
#pragma unroll
        for (int e = 0; e < D / 64; ++e) {
            ring_store(Kb, ring_dtype, base + lane + 64 * e, x[e]);
            ring_store(Vb, ring_dtype, base + lane + 64 * e, v[e]);
        }
    }
    if (l == 0 && tid == 0) {
        int32_t *sp = (int32_t *)(rb + ring_pos_offset(L, Hkv, loc.W, D, es));
        sp[slot] = p;
    }
}

hipError_t launch_inject(const dflash_ctx *c, void *ring, void *const *rings, const int32_t *seq, int n_seq,
                         const int32_t *pos, int T, int S, hipStream_t s) {
    dim3 grid(T, c->L);
    const float eps = c->cfg.rms_eps;
    if (c->D == 128)
        hipLaunchKernelGGL(inject_kernel<128>, grid, dim3(256), 0, s, c->inj_kv, S, T, c->L, c->Hkv, c->W, pos, c->inv_freq,
                           c->k_norm, eps, ring, rings, seq, n_seq, c->cfg.ring_dtype, c->paged);
    else if (c->D == 64)
        hipLaunchKernelGGL(inject_kernel<64>, grid, dim3(256), 0, s, c->inj_kv, S, T, c->L, c->Hkv, c->W, pos, c->inv_freq,
                           c->k_norm, eps, ring, rings, seq, n_seq, c->cfg.ring_dtype, c->paged);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Embedding of the noise block [id_last, mask x (block-1)] (dflash-ops card,
// Usage), first layer's norm input, and the block's rope table.
// ---------------------------------------------------------------------------
// Grid (E/64, B), 256 threads. Writes x [M][E], act_a = x * attn_norm_0 in the
// activation format, ss_a[m][g] = sum of x^2 over the group's 64 columns.
// The workgroups of sequence b also write rope_cs[b][i][f] = (cos, sin)((n_past
// + i) * inv_freq[f]), computed in fp64, one entry per thread.
struct EmbedArgs {
    const void *tok_embd;
    int aux_dtype, E, V, mask_id, block, D;
    const int32_t *id_last, *block_ids, *n_past;
    float *x;
    void *act_a;
    int act_fmt, act_rows;
    const float *attn_norm0;
    float *ss_a;
    int ss_gs;  // row stride of ss_a (groups)
    float *rope_cs;
    const double *inv_freq;
};

__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) {
    const int g = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = g * GROUP_N + lane;
    // four rows per wave at a time: their ids, then their embedding values, then the stores, so the
    // dependent loads of the rows overlap instead of running one row after another
    const float wn = a.attn_norm0[n];
    for (int i0 = wave; i0 < a.block; i0 += 16) {
        int id[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 4 * r;
            id[r] = i >= a.block ? -1 : a.block_ids ? a.block_ids[b * a.block + i] : (i == 0 ? a.id_last[b] : a.mask_id);
        }
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            v[r] = 0.0f;
            if (id[r] >= 0 && id[r] < a.V) {
                const size_t off = (size_t)id[r] * a.E + n;
                v[r] = a.aux_dtype == DFLASH_BF16 ? bf16_to_f32(((const uint16_t *)a.tok_embd)[off])
                                                  : ((const float *)a.tok_embd)[off];
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 4 * r;
            if (i >= a.block) break;
            const int m = b * a.block + i;
            a.x[(size_t)m * a.E + n] = v[r];
            write_act(a.act_a, a.act_fmt, a.act_rows, a.E, m, n, v[r] * wn);
            const float sq = wave_sum(v[r] * v[r]);
            if (lane == 0) a.ss_a[(size_t)m * a.ss_gs + g] = sq;
        }
    }
    {  // the rope table's block * D/2 entries, spread over the sequence's workgroups
        const int half = a.D / 2;
        for (int idx = g * 256 + tid; idx < a.block * half; idx += gridDim.x * 256) {
            const int i = idx / half, f = idx % half;
            const double theta = (double)(a.n_past[b] + i) * a.inv_freq[f];
            double sn, cn;
            sincos(theta, &sn, &cn);
            float *cs = a.rope_cs + (((size_t)b * a.block + i) * half + f) * 2;
            cs[0] = (float)cn;
            cs[1] = (float)sn;
        }
    }
}

hipError_t launch_embed(const dflash_ctx *c, const int32_t *id_last, const int32_t *block_ids, const int32_t *n_past,
                        int B, hipStream_t s) {
    EmbedArgs a;
    a.tok_embd = c->tok_embd;
    a.aux_dtype = c->cfg.aux_dtype;
    a.E = c->E;
    a.V = c->V;
    a.mask_id = c->cfg.mask_id;
    a.block = c->cfg.block;
    a.D = c->D;
    a.id_last = id_last;
    a.block_ids = block_ids;
    a.n_past = n_past;
    a.x = c->x;
    a.act_a = c->act_a;
    a.act_fmt = c->blk_fmt;
    a.act_rows = c->Mmax;
    a.attn_norm0 = c->attn_norm;
    a.ss_a = c->ss_a;
    a.ss_gs = 2 * c->G_E;
    a.rope_cs = c->rope_cs;
    a.inv_freq = c->inv_freq;
    hipLaunchKernelGGL(embed_kernel, dim3(c->G_E, B), dim3(256), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Non-causal sliding-window GQA attention (dflash-ops card, Method)
// ---------------------------------------------------------------------------
// Partial kernel: grid (NCH + 1, Hkv, B), NT threads (512 for one sequence,
// 256 for several). Chunk c < NCH covers ring slots [c*CH, c*CH + CH) with
// CH = 16 * HKT * NT / 256; chunk NCH is the block's own 16 keys. Every wave
// RMS-norms (q_norm) and ropes its q head at positions n_past + i and scales it
// by 1/sqrt(D); the block chunk does the same for the block's k (k_norm, no
// scale). Wave w serves q head jG + (w % 4) for HKT key tiles: with 512 threads
// the first (w < 4) or second half of the chunk, the two halves merging through
// LDS; with 256 threads the whole chunk, so that two workgroups share a
// compute unit when a batch brings many more chunks than compute units.
//
// Scores are computed transposed, S^T = K Q^T (keys as MFMA rows, queries as
// columns), so that each lane holds the scores of one query for 4 keys of every
// 16-key tile. Those registers are exactly the B operand of O^T = V^T P^T when
// lane group c supplies keys {4c..4c+3} of two consecutive key tiles: the
// reduction index of an MFMA may be permuted freely as long as both operands
// use the same permutation, and V^T is read from LDS in that order.
// Operands are exact: fp32 values enter as three bf16 terms (a + b <= 2 cross
// products, error ~2^-27 relative), bf16 ring keys and values as one term.
// A ring key at slot s is visible to block row i when slot_pos[s] >= 0 and
// 0 <= n_past + i - slot_pos[s] < W; block keys 0..gamma-1 are always visible
// (with a block width gamma < 16 the rows gamma..15 are padding).
struct AttnArgs {
    const float *qkv;  // [M][nqkv]: the raw q/k/v projection of the block rows
    int nqkv, qdim, kvdim;
    void *const *rings;  // rings, or block tables when paged.pool is set
    PagedPool paged;
    int layer, L, Hkv, W, ring_dtype, G, NCH, CH, block;
    int gamma;     // block keys gamma..block-1 are padding, visible to no row
    int vt_elems;  // bf16 elements of the V^T region in LDS
    const int32_t *n_past;
    float *ml, *o;
    // per-head RMSNorm (q_norm / k_norm of this layer) and NEOX rope of q and of the block's k
    const float *q_norm, *k_norm;  // [D]
    const float *rope_cs;          // [B][block][D/2][2] (cos, sin) at position n_past + i
    float eps, qscale;             // qscale = 1/sqrt(D), folded into q
    // workgroups c > NCH read `pf` (into the memory-side cache) while the
    // attention workgroups run
    Prefetch pf;
    int pf_x;                      // such workgroups per (kv head, sequence)
};


// One head vector of query or key row `row` of sequence b, held as
// v[ks][e] = element 32ks + 8grp + e by the four lanes grp = 0..3 that share a
// row (lane bits 4 and 5). The rope partner d + D/2 of element d sits in the
// same lane at ks + KS/2.
template <int D>
__device__ __forceinline__ void head_load(float (&v)[D / 32][8], const float *src, int grp) {
    constexpr int KS = D / 32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const float4 a0 = *(const float4 *)(src + 32 * ks + 8 * grp), a1 = *(const float4 *)(src + 32 * ks + 8 * grp + 4);
        v[ks][0] = a0.x; v[ks][1] = a0.y; v[ks][2] = a0.z; v[ks][3] = a0.w;
        v[ks][4] = a1.x; v[ks][5] = a1.y; v[ks][6] = a1.z; v[ks][7] = a1.w;
    }
}

// Per-head RMSNorm (sum of squares reduced over the four lanes of the row),
// norm weight w[D], NEOX rope with the row's (cos, sin) pairs cs[D/2][2] and a
// scale, in place; w and cs are read from LDS (16-byte aligned).
template <int D>
__device__ __forceinline__ void head_norm_rope_row(float (&v)[D / 32][8], const float *w, const float *cs, int grp,
                                                   float eps, float scale) {
    constexpr int KS = D / 32;
    float ss = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += v[ks][e] * v[ks][e];
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float r = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const float4 w0 = *(const float4 *)(w + 32 * ks + 8 * grp), w1 = *(const float4 *)(w + 32 * ks + 8 * grp + 4);
        const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[ks][e] = v[ks][e] * r * wv[e];
    }
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            const float4 c = *(const float4 *)(cs + 2 * (32 * ks + 8 * grp) + 4 * e2);  // pairs 2 e2, 2 e2 + 1
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int e = 2 * e2 + h;
                const float cx = h ? c.z : c.x, sy = h ? c.w : c.y;
                const float x1 = v[ks][e], x2 = v[ks + KS / 2][e];
                v[ks][e] = (x1 * cx - x2 * sy) * scale;
                v[ks + KS / 2][e] = (x1 * sy + x2 * cx) * scale;
            }
        }
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// 8 fp32 values -> three bf16x8 operands (exact split)
__device__ __forceinline__ void split8(const float (&v)[8], bf16x8_t (&t)[3]) {
    u32x4_t w0, w1, w2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t x0, x1, x2;
        split3_pair(v[2 * i], v[2 * i + 1], x0, x1, x2);
        w0[i] = x0;
        w1[i] = x1;
        w2[i] = x2;
    }
    t[0] = __builtin_bit_cast(bf16x8_t, w0);
    t[1] = __builtin_bit_cast(bf16x8_t, w1);
    t[2] = __builtin_bit_cast(bf16x8_t, w2);
}

__device__ __forceinline__ void load8(const float *p, float (&v)[8]) {
    const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

#define MFMA_BF16(A, B, C) __builtin_amdgcn_mfma_f32_16x16x32_bf16((A), (B), (C), 0, 0, 0)

template <int D, int HKT, int NT>
__global__ __launch_bounds__(NT) void attn_partial_kernel(AttnArgs a) {
    static_assert(NT == 256 || NT == 512, "one or two wavefronts per q head");
    constexpr int NHALF = NT / 256;  // wavefronts per q head
    constexpr int KS = D / 32;   // MFMA k-steps over the head dimension
    constexpr int DT = D / 16;   // 16-wide tiles of the head dimension
    constexpr int KROW = D + 8;  // bf16 elements per staged K row (+8 spreads LDS banks)
                                 // HKT: 16-key tiles per wavefront (CH = 16 * HKT * NHALF)
    extern __shared__ float smem[];
    const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    if (c > a.NCH) {  // a prefetch workgroup: no LDS, no barriers
        prefetch_slice(a.pf, (b * a.Hkv + j) * a.pf_x + (c - a.NCH - 1), a.pf_x * a.Hkv * gridDim.z);
        return;
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int NQ = a.G * 16;
    const bool is_block = (c == a.NCH);
    const bool bf16_ring = a.ring_dtype == DFLASH_BF16;
    const bool split_kv = is_block || !bf16_ring;  // fp32 keys/values need three terms
    // A ring chunk whose slots all lie at or past n_past + block holds no key that a block row sees: slot s
    // holds a position p = s (mod W) with p >= s > n_past + i for every row i. It loads nothing and its
    // partial comes out empty (m = -inf, l = 0, o = 0), exactly as for a chunk of masked keys.
    const int np = a.n_past[b];
    const bool past = !is_block && c * a.CH >= np + a.block;
    const int nkeys = is_block ? 16 : (past ? 0 : a.CH);
    const int nks2 = (nkeys + 31) / 32;    // k-steps over keys for P V (the block pads 16 keys to 32)
    const int CHP = nks2 * 32 + 4;         // V^T row length: keys padded to 32, +4 to spread LDS banks
    const int nplanes = split_kv ? 3 : 1;
    uint16_t *ksh = (uint16_t *)smem;                              // [CH][KROW] bf16 ring keys
    uint16_t *vt = ksh + (bf16_ring ? a.CH * KROW : 0);            // [planes][D][CHP] V^T in bf16 terms
    int *kpos = (int *)(vt + a.vt_elems);                          // [CH] positions of the chunk's slots
    float4 *xch = (float4 *)(kpos + a.CH);                         // [4][DT + 1][64] second-half results (NHALF 2)
    float *wsh = (float *)(xch + (NHALF > 1 ? 4 * (DT + 1) * 64 : 0)); // [2][D] q_norm, k_norm
    float *csh = wsh + 2 * D;                                       // [block][D + 4] rope (cos, sin) pairs

    const int es = bf16_ring ? 2 : 4;
    // the ring (or the page) holding the chunk's slots; the block chunk reads none
    const RingLoc loc = ring_locate(a.rings[b], a.paged, a.W, is_block ? 0 : c * a.CH);
    const char *rb = loc.base;
    const void *Kb = rb;
    const void *Vb = rb + ring_v_offset(a.L, a.Hkv, loc.W, D, es);
    const int32_t *sp = (const int32_t *)(rb + ring_pos_offset(a.L, a.Hkv, loc.W, D, es));
    const size_t head_base = ((size_t)a.layer * a.Hkv + j) * loc.W;  // slot-row index of slot 0
    const int s0 = loc.slot;  // the chunk's first slot within it
    const float *qkvb = a.qkv + (size_t)b * a.block * a.nqkv;     // this sequence's 16 rows
    const int hh = wave & 3, half = wave >> 2;
    const bool active = hh < a.G;
    const int q = lane & 15, grp = lane >> 4;

    // ---- loads that do not depend on the chunk, issued ahead of it: the query
    // position, this wave's query row (and the block's key row), the chunk's slot
    // positions, and (staged to LDS with the chunk) the two norm weight vectors
    // and the block rows' rope pairs ----
    const int qpos = np + q;
    float qv[KS][8], kbv[KS][8];
    if (active) {
        head_load<D>(qv, qkvb + (size_t)q * a.nqkv + (size_t)(j * a.G + hh) * D, grp);
        if (is_block) head_load<D>(kbv, qkvb + (size_t)q * a.nqkv + a.qdim + (size_t)j * D, grp);
    }
    const int kp_reg = (!is_block && !past && tid < a.CH) ? (loc.ok ? sp[s0 + tid] : -1) : 0;  // bad page: empty
    const int ncs4 = a.block * D / 4;  // float4 words of the rope table rows (at most 512)
    constexpr int NCS = 512 / NT;
    float4 cs_reg[NCS], w_reg = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < NCS; ++u)
        cs_reg[u] = tid + NT * u < ncs4 ? *(const float4 *)(a.rope_cs + (size_t)b * a.block * D + 4 * (tid + NT * u))
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid < D / 2) w_reg = *(const float4 *)((tid < D / 4 ? a.q_norm : a.k_norm) + 4 * (tid % (D / 4)));

    // ---- chunk keys and values into LDS ----
    if (is_block) {
        for (int idx = tid; idx < 3 * D * CHP; idx += NT) vt[idx] = 0;  // keys 16..31 pad the k-step
        __syncthreads();
        for (int idx = tid; idx < 16 * D; idx += NT) {
            const int key = idx / D, d = idx % D;
            uint16_t t0, t1, t2;
            split3(qkvb[(size_t)key * a.nqkv + a.qdim + a.kvdim + (size_t)j * D + d], t0, t1, t2);
            vt[(0 * D + d) * CHP + key] = t0;
            vt[(1 * D + d) * CHP + key] = t1;
            vt[(2 * D + d) * CHP + key] = t2;
        }
    } else if (past) {
        // nothing to stage
    } else if (bf16_ring) {
        // K rows and V rows: CH*D/8 16-byte words each, in batches with all loads in flight
        constexpr int NWORD = (16 * NHALF * HKT * D / 8 + NT - 1) / NT;
        constexpr int BATCH = NWORD < 4 ? NWORD : 4;
        const int nword = a.CH * D / 8;
        const uint16_t *kg = (const uint16_t *)Kb + (head_base + s0) * D;
        const uint16_t *vg = (const uint16_t *)Vb + (head_base + s0) * D;
#pragma unroll
        for (int u0 = 0; u0 < NWORD; u0 += BATCH) {
            // native vectors, not uint4: a struct copy into LDS can leave the buffer in scratch memory
            u32x4_t kbuf[BATCH], vbuf[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int w = min(tid + NT * (u0 + u), nword - 1);  // clamped: every lane loads
                kbuf[u] = *(const u32x4_t *)(kg + 8 * (size_t)w);
                vbuf[u] = *(const u32x4_t *)(vg + 8 * (size_t)w);
            }
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int w = tid + NT * (u0 + u);
                if (w < nword) {
                    const int key = (8 * w) / D, d = (8 * w) % D;
                    *(u32x4_t *)(ksh + key * KROW + d) = kbuf[u];
                    const uint32_t pk[4] = {vbuf[u].x, vbuf[u].y, vbuf[u].z, vbuf[u].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        vt[(size_t)(d + 2 * e) * CHP + key] = (uint16_t)(pk[e] & 0xffffu);
                        vt[(size_t)(d + 2 * e + 1) * CHP + key] = (uint16_t)(pk[e] >> 16);
                    }
                }
            }
        }
    } else {
        // f32 ring: values split into three planes (keys are read from memory and split at use)
        constexpr int NW4 = (16 * NHALF * HKT * D / 4 + NT - 1) / NT;
        constexpr int BATCH = NW4 < 8 ? NW4 : 8;
        const int nw4 = a.CH * D / 4;
        const float *vg = (const float *)Vb + (head_base + s0) * D;
#pragma unroll
        for (int u0 = 0; u0 < NW4; u0 += BATCH) {
            float4 buf[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) buf[u] = *(const float4 *)(vg + 4 * (size_t)min(tid + NT * (u0 + u), nw4 - 1));
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int w = tid + NT * (u0 + u);
                if (w < nw4) {
                    const int key = (4 * w) / D, d = (4 * w) % D;
                    const float f[4] = {buf[u].x, buf[u].y, buf[u].z, buf[u].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        uint16_t t0, t1, t2;
                        split3(f[e], t0, t1, t2);
                        vt[(size_t)(0 * D + d + e) * CHP + key] = t0;
                        vt[(size_t)(1 * D + d + e) * CHP + key] = t1;
                        vt[(size_t)(2 * D + d + e) * CHP + key] = t2;
                    }
                }
            }
        }
    }
    if (!is_block && tid < a.CH) kpos[tid] = kp_reg;
#pragma unroll
    for (int u = 0; u < NCS; ++u) {  // rope rows padded against bank conflicts
        const int i4 = 4 * (tid + NT * u);
        if (tid + NT * u < ncs4) *(float4 *)(csh + (i4 / D) * (D + 4) + i4 % D) = cs_reg[u];
    }
    if (tid < D / 2) *(float4 *)(wsh + 4 * tid) = w_reg;
    __syncthreads();

    // key tiles of this wave: [half * HKT, half * HKT + HKT) intersected with the chunk
    const int kt0 = half * HKT;
    const int nkt = max(0, min(HKT, nkeys / 16 - kt0));
    float mx = -INFINITY, lsum = 0.0f;
    f32x4_t ot[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) ot[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (active && nkt > 0) {
        // ---- Q^T operand: query q, head elements 32ks + 8grp .. +8 (normed, roped, scaled), three terms ----
        bf16x8_t qb[KS][3];
        head_norm_rope_row<D>(qv, wsh, csh + q * (D + 4), grp, a.eps, a.qscale);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) split8(qv[ks], qb[ks]);
        // the block's key q of this kv head (normed, roped), for the block chunk
        if (is_block) head_norm_rope_row<D>(kbv, wsh + D, csh + q * (D + 4), grp, a.eps, 1.0f);
        // ---- S^T = K Q^T, key tile kt: lane holds keys 16(kt0+kt) + 4grp + i (i < 4) of query q ----
        f32x4_t st[HKT];
#pragma unroll
        for (int kt = 0; kt < HKT; ++kt) st[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // A full chunk of bf16 ring keys (every ring chunk of a bf16 ring) runs
        // as straight-line code: per k-step the wave's key tiles are read from
        // LDS together and their MFMA chains interleave. Each accumulator sums
        // in the same order as the general loop below.
        const bool fast = !split_kv && nkt == HKT;
        if (fast) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8_t ka[HKT];
#pragma unroll
                for (int kt = 0; kt < HKT; ++kt)
                    ka[kt] = __builtin_bit_cast(
                        bf16x8_t, *(const u32x4_t *)(ksh + (16 * (kt0 + kt) + q) * KROW + 32 * ks + 8 * grp));
#pragma unroll
                for (int t = 0; t < 3; ++t)
#pragma unroll
                    for (int kt = 0; kt < HKT; ++kt) st[kt] = MFMA_BF16(ka[kt], qb[ks][t], st[kt]);
            }
        }
#pragma clang loop unroll(full)
        for (int kt = 0; kt < HKT; ++kt) {
            if (fast || kt >= nkt) continue;
            const int key = 16 * (kt0 + kt) + q;  // A-operand row of this lane
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int d0 = 32 * ks + 8 * grp;
                if (!split_kv) {
                    const bf16x8_t ka = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(ksh + key * KROW + d0));
#pragma unroll
                    for (int t = 0; t < 3; ++t) st[kt] = MFMA_BF16(ka, qb[ks][t], st[kt]);
                } else {
                    float kv[8];
                    if (is_block) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) kv[e] = kbv[ks][e];  // key == q: the block has one key tile
                    } else {
                        load8((const float *)Kb + (head_base + s0 + key) * D + d0, kv);
                    }
                    bf16x8_t ka[3];
                    split8(kv, ka);
                    // the six products with term-order sum <= 2
                    st[kt] = MFMA_BF16(ka[0], qb[ks][0], st[kt]);
                    st[kt] = MFMA_BF16(ka[0], qb[ks][1], st[kt]);
                    st[kt] = MFMA_BF16(ka[1], qb[ks][0], st[kt]);
                    st[kt] = MFMA_BF16(ka[0], qb[ks][2], st[kt]);
                    st[kt] = MFMA_BF16(ka[1], qb[ks][1], st[kt]);
                    st[kt] = MFMA_BF16(ka[2], qb[ks][0], st[kt]);
                }
            }
        }
        // ---- mask and softmax statistics of this wave's keys for query q ----
#pragma clang loop unroll(full)
        for (int kt = 0; kt < HKT; ++kt) {
            const int key0 = 16 * (kt0 + kt) + 4 * grp;  // this lane's four keys: key0 .. key0 + 3
            int4 kp = make_int4(-1, -1, -1, -1);
            if (!is_block && kt < nkt) kp = *(const int4 *)(kpos + key0);
            const int kpv[4] = {kp.x, kp.y, kp.z, kp.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // ring key: a written slot whose position lies in [qpos - W + 1, qpos]; block key: < gamma
                // (evaluated without short-circuits, so the mask is selects rather than branches)
                const bool ring_vis = (kpv[i] >= 0) & ((unsigned)(qpos - kpv[i]) < (unsigned)a.W);
                const bool vis = (kt < nkt) & (is_block ? key0 + i < a.gamma : ring_vis);
                st[kt][i] = vis ? st[kt][i] : -INFINITY;
                mx = fmaxf(mx, st[kt][i]);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // exp(-inf) is 0, so a masked key needs no test; with no visible key (mx
        // = -inf) every score is -inf and 0 stands in for the maximum
        const float mxs = mx == -INFINITY ? 0.0f : mx;
#pragma clang loop unroll(full)
        for (int kt = 0; kt < HKT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = expf(st[kt][i] - mxs);
                st[kt][i] = p;
                lsum += p;
            }
        lsum += __shfl_xor(lsum, 16, 64);
        lsum += __shfl_xor(lsum, 32, 64);
        // ---- O^T = V^T P^T over key pairs of tiles (2ks2, 2ks2 + 1) of this half ----
        if constexpr (HKT % 2 == 0) {
            if (fast) {  // one bf16 plane; per key pair all V^T reads first, then the interleaved chains
#pragma unroll
                for (int ks2 = 0; ks2 < HKT / 2; ++ks2) {
                    float pv[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        pv[i] = st[2 * ks2][i];
                        pv[4 + i] = st[2 * ks2 + 1][i];
                    }
                    bf16x8_t pb[3];
                    split8(pv, pb);
                    const int kbase = 16 * kt0 + 32 * ks2;
                    const int k0 = kbase + 4 * grp, k1 = kbase + 16 + 4 * grp;
                    bf16x8_t va[DT];
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const uint16_t *row = vt + (size_t)(16 * dt + q) * CHP;
                        const uint2 lo = *(const uint2 *)(row + k0), hi = *(const uint2 *)(row + k1);
                        va[dt] = __builtin_bit_cast(bf16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
                    }
#pragma unroll
                    for (int t = 0; t < 3; ++t)
#pragma unroll
                        for (int dt = 0; dt < DT; ++dt) ot[dt] = MFMA_BF16(va[dt], pb[t], ot[dt]);
                }
            }
        }
#pragma clang loop unroll(full)
        for (int ks2 = 0; ks2 < (HKT + 1) / 2; ++ks2) {
            if ((HKT % 2 == 0 && fast) || 2 * ks2 >= nkt) continue;
            float pv[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pv[i] = st[2 * ks2][i];
                pv[4 + i] = 2 * ks2 + 1 < HKT ? st[(2 * ks2 + 1) % HKT][i] : 0.0f;
            }
            bf16x8_t pb[3];
            split8(pv, pb);
            const int kbase = 16 * kt0 + 32 * ks2;
            const int k0 = kbase + 4 * grp, k1 = kbase + 16 + 4 * grp;  // the lane group's keys in V^T
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int d = 16 * dt + q;
                bf16x8_t va[3];
#pragma unroll
                for (int t = 0; t < 3; ++t) {
                    if (t >= nplanes) break;
                    const uint16_t *row = vt + ((size_t)t * D + d) * CHP;
                    const uint2 lo = *(const uint2 *)(row + k0);
                    // a half with one key tile has no second tile in the pair: its keys (and P) are zero
                    const uint2 hi = 2 * ks2 + 1 < HKT ? *(const uint2 *)(row + k1) : make_uint2(0u, 0u);
                    va[t] = __builtin_bit_cast(bf16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
                }
                if (!split_kv) {
#pragma unroll
                    for (int t = 0; t < 3; ++t) ot[dt] = MFMA_BF16(va[0], pb[t], ot[dt]);
                } else {
                    ot[dt] = MFMA_BF16(va[0], pb[0], ot[dt]);
                    ot[dt] = MFMA_BF16(va[0], pb[1], ot[dt]);
                    ot[dt] = MFMA_BF16(va[1], pb[0], ot[dt]);
                    ot[dt] = MFMA_BF16(va[0], pb[2], ot[dt]);
                    ot[dt] = MFMA_BF16(va[1], pb[1], ot[dt]);
                    ot[dt] = MFMA_BF16(va[2], pb[0], ot[dt]);
                }
            }
        }
    }
    // ---- merge the second half into the first through LDS ----
    if constexpr (NHALF == 1) {
        if (!active) return;
    } else {
    // slot c of lane l of q head hh at xch[(hh * (DT + 1) + c) * 64 + l]: the
    // output tile dt in slot dt, (max, sum) in slot DT; each slot of a wave is
    // one contiguous 1 KB run of 16-byte words
    float4 *xw = xch + (size_t)hh * (DT + 1) * 64 + lane;
    if (half == 1 && active) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) xw[dt * 64] = make_float4(ot[dt][0], ot[dt][1], ot[dt][2], ot[dt][3]);
        xw[DT * 64] = make_float4(mx, lsum, 0.0f, 0.0f);
    }
    __syncthreads();
    if (half == 1 || !active) return;
    {
        const float4 ml2 = xw[DT * 64];
        const float m2 = ml2.x, l2 = ml2.y;
        const float mn = fmaxf(mx, m2), mns = mn == -INFINITY ? 0.0f : mn;  // exp(-inf) = 0, as above
        const float a1 = expf(mx - mns);
        const float a2 = expf(m2 - mns);
        lsum = lsum * a1 + l2 * a2;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const float4 o2 = xw[dt * 64];
            ot[dt][0] = ot[dt][0] * a1 + o2.x * a2;
            ot[dt][1] = ot[dt][1] * a1 + o2.y * a2;
            ot[dt][2] = ot[dt][2] * a1 + o2.z * a2;
            ot[dt][3] = ot[dt][3] * a1 + o2.w * a2;
        }
        mx = mn;
    }
    }
    // ---- partial (max, sum, unnormalised output) of query (hh, q) ----
    const size_t slot = (((size_t)b * a.Hkv + j) * (a.NCH + 1) + c) * NQ + hh * 16 + q;
    if (grp == 0) {
        a.ml[slot * 2] = mx;
        a.ml[slot * 2 + 1] = lsum;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        *(float4 *)(a.o + slot * D + 16 * dt + 4 * grp) = make_float4(ot[dt][0], ot[dt][1], ot[dt][2], ot[dt][3]);
}

// LDS of the partial kernel: for a bf16 ring the chunk's keys [CH][D+8] bf16;
// the V^T planes (one bf16 plane of CH keys for a bf16 ring, three planes for
// f32 values, the block padded to 32 keys; every row +4 elements); the chunk's
// slot positions; the second-half exchange [4][D/16 + 1][64] float4 (512
// threads only); the q and k norm weights [2][D] and the block rows' rope
// pairs [block][D + 4] f32.
int attn_vt_elems(int D, int CH, int ring_dtype) {
    const int ring = (CH + 4) * (ring_dtype == DFLASH_BF16 ? 1 : 3);
    return (ring > 3 * 36 ? ring : 3 * 36) * D;
}
size_t attn_smem_bytes(int D, int CH, int ring_dtype, int block, int NT) {
    const size_t kbytes = ring_dtype == DFLASH_BF16 ? (size_t)CH * (D + 8) * 2 : 0;
    return kbytes + (size_t)attn_vt_elems(D, CH, ring_dtype) * 2 + (size_t)CH * 4 +
           (NT > 256 ? (size_t)4 * (D / 16 + 1) * 64 * 16 : 0) + (size_t)(2 * D + block * (D + 4)) * 4;
}

template <int D, int KT, int NT>
static hipError_t set_attn_limit(int bytes) {
    return hipFuncSetAttribute((const void *)attn_partial_kernel<D, KT, NT>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

hipError_t attention_set_smem_limit() {
    const int bytes = 160 * 1024;
    hipError_t e;
    if ((e = set_attn_limit<128, 4, 512>(bytes)) != hipSuccess) return e;
    if ((e = set_attn_limit<128, 2, 512>(bytes)) != hipSuccess) return e;
    if ((e = set_attn_limit<128, 1, 512>(bytes)) != hipSuccess) return e;
    if ((e = set_attn_limit<64, 4, 512>(bytes)) != hipSuccess) return e;
    if ((e = set_attn_limit<64, 2, 512>(bytes)) != hipSuccess) return e;
    if ((e = set_attn_limit<64, 1, 512>(bytes)) != hipSuccess) return e;
    if ((e = set_attn_limit<128, 4, 256>(bytes)) != hipSuccess) return e;
    if ((e = set_attn_limit<128, 2, 256>(bytes)) != hipSuccess) return e;
    if ((e = set_attn_limit<64, 4, 256>(bytes)) != hipSuccess) return e;
    return set_attn_limit<64, 2, 256>(bytes);
}

// Combine kernel: grid (H, B, D / 32), 256 threads. Thread t serves block row
// t / 16 of q head h and head elements 32 * blockIdx.z + 2 * (t % 16) + {0, 1};
// it merges the NCH + 1 chunk partials in chunk order and writes the attention
// output in the activation format of the Wo projection.
struct CombArgs {
    const float *ml, *o;
    int NCH, G, Hkv, D, block;
    void *act_o;
    int act_fmt, act_rows, qdim;
};

__global__ __launch_bounds__(256) void attn_combine_kernel(CombArgs a) {
    const int h = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x;
    const int i = tid >> 4;
    const int d = blockIdx.z * 32 + 2 * (tid & 15);
    const int j = h / a.G, hh = h % a.G;
    const int NQ = a.G * 16, qi = hh * 16 + i;
    const size_t base = ((size_t)b * a.Hkv + j) * (a.NCH + 1);
    const int nc = a.NCH + 1;
    // batches of 17 chunks whose loads are all in flight together (one batch for
    // one sequence's 128-slot chunks of a 2048-slot window: 4.6 against 5.3 us
    // with batches of 24; two for the 64-slot chunks of a batch: 17.2 against
    // 19.6 us at batch 8); per batch
    // the running state is rescaled once to the batch's maximum and every
    // chunk weight exp(m_c - max) is independent of the others
    constexpr int UNR = 17;
    float mstar = -INFINITY, lsum = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int c0 = 0; c0 < nc; c0 += UNR) {
        float2 mlb[UNR], ovb[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int cc = min(c0 + u, nc - 1);
            mlb[u] = *(const float2 *)(a.ml + ((base + cc) * NQ + qi) * 2);
            ovb[u] = *(const float2 *)(a.o + ((base + cc) * NQ + qi) * a.D + d);
        }
        float bm = -INFINITY;
#pragma unroll
        for (int u = 0; u < UNR; ++u)
            if (c0 + u < nc) bm = fmaxf(bm, mlb[u].x);
        if (bm == -INFINITY) continue;  // no visible key in this batch
        const float mn = fmaxf(mstar, bm);
        const float alpha = expf(mstar - mn);  // 0 while mstar is -inf
        lsum *= alpha;
        o0 *= alpha;
        o1 *= alpha;
        // a chunk without visible keys (m = -inf, sum and output 0) gets weight
        // exp(-inf) = 0 and adds exactly nothing, so it needs no test
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            if (c0 + u < nc) {
                const float w = expf(mlb[u].x - mn);
                lsum += w * mlb[u].y;
                o0 += w * ovb[u].x;
                o1 += w * ovb[u].y;
            }
        }
        mstar = mn;
    }
    const float inv = 1.0f / lsum;
    const int row = b * a.block + i;
    write_act(a.act_o, a.act_fmt, a.act_rows, a.qdim, row, h * a.D + d, o0 * inv);
    write_act(a.act_o, a.act_fmt, a.act_rows, a.qdim, row, h * a.D + d + 1, o1 * inv);
}

hipError_t launch_attention(const dflash_ctx *c, int l, void *const *rings, const int32_t *n_past, int B,
                            hipStream_t s) {
    AttnArgs a;
    a.qkv = c->qkv_out;
    a.q_norm = c->q_norm + (size_t)l * c->D;
    a.k_norm = c->k_norm + (size_t)l * c->D;
    a.rope_cs = c->rope_cs;
    a.eps = c->cfg.rms_eps;
    a.qscale = 1.0f / sqrtf((float)c->D);
    a.nqkv = c->nqkv;
    a.qdim = c->qdim;
    a.kvdim = c->kvdim;
    a.rings = rings;
    a.paged = c->paged;
    a.layer = l;
    a.L = c->L;
    a.Hkv = c->Hkv;
    a.W = c->W;
    a.ring_dtype = c->cfg.ring_dtype;
    a.G = c->H / c->Hkv;
    const int NT = attn_threads(B);
    a.CH = attn_chunk(c->cfg.ring_dtype, c->W, B);
    a.NCH = c->W / a.CH;
    a.vt_elems = attn_vt_elems(c->D, a.CH, c->cfg.ring_dtype);
    a.block = c->cfg.block;
    a.gamma = c->gamma;
    a.n_past = n_past;
    a.ml = c->att_ml;
    a.o = c->att_o;
    // Idle compute units read the head of this layer's gate/up weights into the
    // memory-side cache meanwhile (the gate/up GEMV is bandwidth-bound; the Wo
    // GEMV in between is latency-bound): 0.5 MB per such workgroup, an amount
    // one compute unit reads within the attention kernel's run time.
    a.pf_x = attn_pf_x(*c, B);
    a.pf = Prefetch{};
    a.pf.base = (const char *)c->layer[l].gu;
    a.pf.bytes = attn_gu_prefetch(*c, B);
    a.pf.sink = c->pf_sink;
    dim3 grid(a.NCH + 1 + a.pf_x, c->Hkv, B);
    if (c->cfg.block * c->D / 4 > 512) return hipErrorInvalidValue;  // rope rows: at most 512 float4 words
    const size_t smem = attn_smem_bytes(c->D, a.CH, c->cfg.ring_dtype, c->cfg.block, NT);
    const int hkt = a.CH * 256 / (16 * NT);
#define DFLASH_ATTN_LAUNCH(DD, KK, TT) \
    hipLaunchKernelGGL((attn_partial_kernel<DD, KK, TT>), grid, dim3(TT), smem, s, a)
    if (NT == 512 && c->D == 128 && hkt == 4) DFLASH_ATTN_LAUNCH(128, 4, 512);
    else if (NT == 512 && c->D == 128 && hkt == 2) DFLASH_ATTN_LAUNCH(128, 2, 512);
    else if (NT == 512 && c->D == 128 && hkt == 1) DFLASH_ATTN_LAUNCH(128, 1, 512);
    else if (NT == 512 && c->D == 64 && hkt == 4) DFLASH_ATTN_LAUNCH(64, 4, 512);
    else if (NT == 512 && c->D == 64 && hkt == 2) DFLASH_ATTN_LAUNCH(64, 2, 512);
    else if (NT == 512 && c->D == 64 && hkt == 1) DFLASH_ATTN_LAUNCH(64, 1, 512);
    else if (NT == 256 && c->D == 128 && hkt == 4) DFLASH_ATTN_LAUNCH(128, 4, 256);
    else if (NT == 256 && c->D == 128 && hkt == 2) DFLASH_ATTN_LAUNCH(128, 2, 256);
    else if (NT == 256 && c->D == 64 && hkt == 4) DFLASH_ATTN_LAUNCH(64, 4, 256);
    else if (NT == 256 && c->D == 64 && hkt == 2) DFLASH_ATTN_LAUNCH(64, 2, 256);
    else return hipErrorInvalidValue;
#undef DFLASH_ATTN_LAUNCH
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    CombArgs cb;
    cb.ml = c->att_ml;
    cb.o = c->att_o;
    cb.NCH = a.NCH;
    cb.G = a.G;
    cb.Hkv = c->Hkv;
    cb.D = c->D;
    cb.block = c->cfg.block;
    cb.act_o = c->act_o;
    cb.act_fmt = c->blk_fmt;
    cb.act_rows = c->Mmax;
    cb.qdim = c->qdim;
    hipLaunchKernelGGL(attn_combine_kernel, dim3(c->H, B, c->D / 32), dim3(256), 0, s, cb);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Acceptance scan: one wavefront per sequence; lane i compares draft i with the
// target token; the first set bit of the mismatch ballot is n_ok.
// ---------------------------------------------------------------------------
// target rows are ld_t long; with bonus, bonus[b] = target[b][n_ok[b]] (the
// target's token at the first mismatch, or at position n after n matches).
__global__ void accept_kernel(const int32_t *drafts, const int32_t *target, int n, int ld_t, int32_t *n_ok,
                              int32_t *bonus) {
    const int b = blockIdx.x, lane = threadIdx.x;
    const bool mis = lane < n && drafts[(size_t)b * n + lane] != target[(size_t)b * ld_t + lane];
    const unsigned long long mask = __ballot(mis);
    const int k = mask ? (__ffsll((long long)mask) - 1) : n;
    if (lane == 0) {
        n_ok[b] = k;
        if (bonus != nullptr) bonus[b] = target[(size_t)b * ld_t + k];
    }
}

hipError_t launch_accept(const int32_t *drafts, const int32_t *target, int B, int n, int32_t *n_ok, hipStream_t s,
                         int32_t *bonus) {
    if (n < 0 || n > 63) return hipErrorInvalidValue;  // one wavefront compares the drafts
    hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(64), 0, s, drafts, target, n, bonus ? n + 1 : n, n_ok, bonus);
    return hipGetLastError();
}
