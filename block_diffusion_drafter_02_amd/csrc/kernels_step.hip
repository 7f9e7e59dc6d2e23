// Non-GEMM kernels of the DFlash drafter on gfx950: embedding of the noise
// block, non-causal sliding-window GQA attention of the block against ring
// plus block, ring injection (per-head RMSNorm, NEOX rope, slot scatter),
// encode's row RMSNorm, activation conversion, and the acceptance scan.
#include "dflash_internal.h"

// ---------------------------------------------------------------------------
// Ring layout: K [L][Hkv][W][D], V [L][Hkv][W][D] (ring dtype), slot_pos [W]
// ---------------------------------------------------------------------------
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
__host__ __device__ inline size_t ring_v_offset(int L, int Hkv, int W, int D, int es) {
    return align256(ring_kv_elems(L, Hkv, W, D) * es);
}
__host__ __device__ inline size_t ring_pos_offset(int L, int Hkv, int W, int D, int es) {
    return ring_v_offset(L, Hkv, W, D, es) + align256(ring_kv_elems(L, Hkv, W, D) * es);
}

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
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const float *y, int E, const float *w, float eps, float *h) {
    const int t = blockIdx.x;
    const float *yr = y + (size_t)t * E;
    float ss = 0.0f;
    for (int c = threadIdx.x; c < E; c += 256) ss += yr[c] * yr[c];
    ss = wave_sum(ss);
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float r = 1.0f / sqrtf(tot / (float)E + eps);
    for (int c = threadIdx.x; c < E; c += 256) h[(size_t)t * E + c] = yr[c] * r * w[c];
}

hipError_t launch_rmsnorm_rows(const float *y, int T, int E, const float *w, float eps, float *h, hipStream_t s) {
    hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3(T), dim3(256), 0, s, y, E, w, eps, h);
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
__global__ __launch_bounds__(256) void inject_kernel(const float *__restrict__ kv, int L, int Hkv, int W,
                                                     const int32_t *__restrict__ pos,
                                                     const double *__restrict__ inv_freq,
                                                     const float *__restrict__ k_norm_all, float eps, void *ring,
                                                     int ring_dtype) {
    const int t = blockIdx.x, l = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = pos[t];
    if (p < 0) return;
    const int slot = p % W;
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
    char *rb = (char *)ring;
    void *Kb = rb;
    void *Vb = rb + ring_v_offset(L, Hkv, W, D, es);
    const float *kn = k_norm_all + (size_t)l * D;
    for (int j = wave; j < Hkv; j += 4) {
        float x[D / 64], v[D / 64];
#pragma unroll
        for (int e = 0; e < D / 64; ++e) {
            x[e] = row[(size_t)j * D + lane + 64 * e];
            v[e] = row[kvdim + (size_t)j * D + lane + 64 * e];
        }
        head_norm_rope<D>(x, kn, cs, eps, lane);
        const size_t base = (((size_t)l * Hkv + j) * W + slot) * D;
#pragma unroll
        for (int e = 0; e < D / 64; ++e) {
            ring_store(Kb, ring_dtype, base + lane + 64 * e, x[e]);
            ring_store(Vb, ring_dtype, base + lane + 64 * e, v[e]);
        }
    }
    if (l == 0 && tid == 0) {
        int32_t *sp = (int32_t *)(rb + ring_pos_offset(L, Hkv, W, D, es));
        sp[slot] = p;
    }
}

hipError_t launch_inject(const dflash_ctx *c, void *ring, const int32_t *pos, int T, hipStream_t s) {
    dim3 grid(T, c->L);
    const float eps = c->cfg.rms_eps;
    if (c->D == 128)
        hipLaunchKernelGGL(inject_kernel<128>, grid, dim3(256), 0, s, c->inj_kv, c->L, c->Hkv, c->W, pos, c->inv_freq,
                           c->k_norm, eps, ring, c->cfg.ring_dtype);
    else if (c->D == 64)
        hipLaunchKernelGGL(inject_kernel<64>, grid, dim3(256), 0, s, c->inj_kv, c->L, c->Hkv, c->W, pos, c->inv_freq,
                           c->k_norm, eps, ring, c->cfg.ring_dtype);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Embedding of the noise block [id_last, mask x (block-1)] (dflash-ops card,
// Usage), first layer's norm input, and the block's rope table.
// ---------------------------------------------------------------------------
// Grid (E/64, B), 256 threads. Writes x [M][E], act_a = x * attn_norm_0 in the
// activation format, ss_a[g][m] = sum of x^2 over the group's 64 columns.
// Workgroup (0, b) also writes rope_cs[b][i][f] = (cos, sin)((n_past + i) *
// inv_freq[f]), computed in fp64.
struct EmbedArgs {
    const void *tok_embd;
    int aux_dtype, E, V, mask_id, block, D;
    const int32_t *id_last, *block_ids, *n_past;
    float *x;
    void *act_a;
    int act_fmt, act_rows;
    const float *attn_norm0;
    float *ss_a;
    int ss_stride;
    float *rope_cs;
    const double *inv_freq;
};

__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) {
    const int g = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = g * GROUP_N + lane;
    for (int i = wave; i < a.block; i += 4) {
        const int m = b * a.block + i;
        const int id = a.block_ids ? a.block_ids[m] : (i == 0 ? a.id_last[b] : a.mask_id);
        float v = 0.0f;
        if (id >= 0 && id < a.V) {
            const size_t off = (size_t)id * a.E + n;
            v = a.aux_dtype == DFLASH_BF16 ? bf16_to_f32(((const uint16_t *)a.tok_embd)[off])
                                           : ((const float *)a.tok_embd)[off];
        }
        a.x[(size_t)m * a.E + n] = v;
        if (a.act_fmt == ACT_F32) {
            ((float *)a.act_a)[(size_t)m * a.E + n] = v * a.attn_norm0[n];
        } else {
            uint16_t t0, t1, t2;
            split3(v * a.attn_norm0[n], t0, t1, t2);
            uint16_t *p = (uint16_t *)a.act_a;
            const size_t plane = (size_t)a.act_rows * a.E;
            p[(size_t)m * a.E + n] = t0;
            p[plane + (size_t)m * a.E + n] = t1;
            p[2 * plane + (size_t)m * a.E + n] = t2;
        }
        const float sq = wave_sum(v * v);
        if (lane == 0) a.ss_a[(size_t)g * a.ss_stride + m] = sq;
    }
    if (g == 0) {
        const int half = a.D / 2;
        for (int idx = tid; idx < a.block * half; idx += 256) {
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
    a.act_fmt = c->act_fmt;
    a.act_rows = c->Mmax;
    a.attn_norm0 = c->attn_norm;
    a.ss_a = c->ss_a;
    a.ss_stride = c->Mmax;
    a.rope_cs = c->rope_cs;
    a.inv_freq = c->inv_freq;
    hipLaunchKernelGGL(embed_kernel, dim3(c->G_E, B), dim3(256), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Non-causal sliding-window GQA attention (dflash-ops card, Method)
// ---------------------------------------------------------------------------
// Partial kernel: grid (NCH + 1, Hkv, B), 256 threads. Chunk c < NCH covers
// ring slots [64c, 64c + 64); chunk NCH is the block's own 16 keys. The G*16
// query vectors of kv head j (q heads jG .. jG+G-1, 16 block rows each) are
// RMS-normed with q_norm and roped at n_past + i, then scaled by 1/sqrt(D).
// Thread t serves query t/4 and head elements (t%4) + 4e. Keys are taken 16 at a
// time with a running max and sum; the chunk's (max, sum, unnormalised output)
// goes to the partial buffers. A ring key at slot s is visible to row i when
// slot_pos[s] >= 0 and 0 <= n_past + i - slot_pos[s] < W; block keys are always
// visible.
struct AttnArgs {
    const float *qkv;
    int nqkv, qdim, kvdim;
    const float *rope_cs;
    const float *q_norm, *k_norm;  // this layer's [D]
    void *const *rings;
    int layer, L, Hkv, W, ring_dtype, G, NCH, block;
    const int32_t *n_past;
    float eps, scale;
    float *ml, *o;
};

template <int D>
__global__ __launch_bounds__(256) void attn_partial_kernel(AttnArgs a) {
    constexpr int DE = D / 4;  // elements per thread
    const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int NQ = a.G * 16;
    const bool is_block = (c == a.NCH);
    const int nvec = NQ + (is_block ? 16 : 0);
    __shared__ float stage[64 + 16][D];
    __shared__ float ksh[16][D];
    __shared__ float vsh[16][D];
    __shared__ int kpos[16];

    // raw q (and block k, v) of this kv head
    for (int idx = tid; idx < nvec * D; idx += 256) {
        const int vec = idx / D, d = idx % D;
        const int i = vec % 16;
        const size_t m = (size_t)b * a.block + i;
        float v;
        if (vec < NQ)
            v = a.qkv[m * a.nqkv + (size_t)(j * a.G + vec / 16) * D + d];
        else
            v = a.qkv[m * a.nqkv + a.qdim + (size_t)j * D + d];
        stage[vec][d] = v;
    }
    if (is_block) {
        for (int idx = tid; idx < 16 * D; idx += 256) {
            const int i = idx / D, d = idx % D;
            vsh[i][d] = a.qkv[((size_t)b * a.block + i) * a.nqkv + a.qdim + a.kvdim + (size_t)j * D + d];
        }
    }
    __syncthreads();
    for (int vec = wave; vec < nvec; vec += 4) {
        float x[D / 64];
#pragma unroll
        for (int e = 0; e < D / 64; ++e) x[e] = stage[vec][lane + 64 * e];
        const int i = vec % 16;
        const float *cs = a.rope_cs + ((size_t)b * a.block + i) * D;  // (D/2) pairs of (cos, sin)
        head_norm_rope<D>(x, vec < NQ ? a.q_norm : a.k_norm, cs, a.eps, lane);
#pragma unroll
        for (int e = 0; e < D / 64; ++e) stage[vec][lane + 64 * e] = x[e];
    }
    __syncthreads();

    const int qi = tid >> 2, dq = tid & 3;
    const bool live = qi < NQ;
    float q[DE], o[DE];
#pragma unroll
    for (int e = 0; e < DE; ++e) {
        q[e] = live ? stage[qi][dq + 4 * e] * a.scale : 0.0f;
        o[e] = 0.0f;
    }
    const int qpos = a.n_past[b] + (qi & 15);
    float m_run = -INFINITY, l_run = 0.0f;

    const int es = a.ring_dtype == DFLASH_BF16 ? 2 : 4;
    const char *rb = (const char *)a.rings[b];
    const void *Kb = rb;
    const void *Vb = rb + ring_v_offset(a.L, a.Hkv, a.W, D, es);
    const int32_t *sp = (const int32_t *)(rb + ring_pos_offset(a.L, a.Hkv, a.W, D, es));
    const int nsub = is_block ? 1 : 4;
    for (int st = 0; st < nsub; ++st) {
        const float(*Kt)[D];
        const float(*Vt)[D];
        if (is_block) {
            Kt = (const float(*)[D]) & stage[NQ][0];
            Vt = (const float(*)[D]) & vsh[0][0];
        } else {
            __syncthreads();
            const int s0 = c * 64 + st * 16;
            const size_t base = (((size_t)a.layer * a.Hkv + j) * a.W + s0) * D;
            for (int idx = tid; idx < 16 * D; idx += 256) {
                ksh[idx / D][idx % D] = ring_load(Kb, a.ring_dtype, base + idx);
                vsh[idx / D][idx % D] = ring_load(Vb, a.ring_dtype, base + idx);
            }
            if (tid < 16) kpos[tid] = sp[s0 + tid];
            __syncthreads();
            Kt = (const float(*)[D]) & ksh[0][0];
            Vt = (const float(*)[D]) & vsh[0][0];
        }
        float sc[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            float acc = 0.0f;
#pragma unroll
            for (int e = 0; e < DE; ++e) acc += q[e] * Kt[k][dq + 4 * e];
            sc[k] = acc;
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            sc[k] += __shfl_xor(sc[k], 1, 64);
            sc[k] += __shfl_xor(sc[k], 2, 64);
        }
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            bool vis = true;
            if (!is_block) {
                const int kp = kpos[k];
                const int dlt = qpos - kp;
                vis = kp >= 0 && dlt >= 0 && dlt < a.W;
            }
            if (!vis) sc[k] = -INFINITY;
            mx = fmaxf(mx, sc[k]);
        }
        const float m_new = fmaxf(m_run, mx);
        if (m_new == -INFINITY) continue;  // nothing visible yet
        const float alpha = expf(m_run - m_new);
        float psum = 0.0f;
#pragma unroll
        for (int e = 0; e < DE; ++e) o[e] *= alpha;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const float p = expf(sc[k] - m_new);
            psum += p;
#pragma unroll
            for (int e = 0; e < DE; ++e) o[e] += p * Vt[k][dq + 4 * e];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
    }
    if (live) {
        const size_t slot = (((size_t)b * a.Hkv + j) * (a.NCH + 1) + c) * NQ + qi;
        if (dq == 0) {
            a.ml[slot * 2] = m_run;
            a.ml[slot * 2 + 1] = l_run;
        }
#pragma unroll
        for (int e = 0; e < DE; ++e) a.o[slot * D + dq + 4 * e] = o[e];
    }
}

// Combine kernel: grid (H, B), 256 threads; row i = t/16 of q head h merges the
// NCH + 1 chunk partials in chunk order and writes the attention output in the
// activation format of the Wo projection.
struct CombArgs {
    const float *ml, *o;
    int NCH, G, Hkv, D, block;
    void *act_o;
    int act_fmt, act_rows, qdim;
};

__global__ __launch_bounds__(256) void attn_combine_kernel(CombArgs a) {
    const int h = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x;
    const int i = tid >> 4, dl = tid & 15;
    const int j = h / a.G, hh = h % a.G;
    const int NQ = a.G * 16, qi = hh * 16 + i;
    const size_t base = ((size_t)b * a.Hkv + j) * (a.NCH + 1);
    float mstar = -INFINITY;
    for (int c = 0; c <= a.NCH; ++c) mstar = fmaxf(mstar, a.ml[((base + c) * NQ + qi) * 2]);
    float lsum = 0.0f;
    for (int c = 0; c <= a.NCH; ++c) {
        const float mc = a.ml[((base + c) * NQ + qi) * 2];
        if (mc != -INFINITY) lsum += expf(mc - mstar) * a.ml[((base + c) * NQ + qi) * 2 + 1];
    }
    const float inv = 1.0f / lsum;
    const int row = b * a.block + i;
    for (int d = dl; d < a.D; d += 16) {
        float acc = 0.0f;
        for (int c = 0; c <= a.NCH; ++c) {
            const float mc = a.ml[((base + c) * NQ + qi) * 2];
            if (mc != -INFINITY) acc += expf(mc - mstar) * a.o[((base + c) * NQ + qi) * a.D + d];
        }
        const float v = acc * inv;
        const int col = h * a.D + d;
        if (a.act_fmt == ACT_F32) {
            ((float *)a.act_o)[(size_t)row * a.qdim + col] = v;
        } else {
            uint16_t t0, t1, t2;
            split3(v, t0, t1, t2);
            uint16_t *p = (uint16_t *)a.act_o;
            const size_t plane = (size_t)a.act_rows * a.qdim;
            p[(size_t)row * a.qdim + col] = t0;
            p[plane + (size_t)row * a.qdim + col] = t1;
            p[2 * plane + (size_t)row * a.qdim + col] = t2;
        }
    }
}

hipError_t launch_attention(const dflash_ctx *c, int l, void *const *rings, const int32_t *n_past, int B,
                            hipStream_t s) {
    AttnArgs a;
    a.qkv = c->qkv_out;
    a.nqkv = c->nqkv;
    a.qdim = c->qdim;
    a.kvdim = c->kvdim;
    a.rope_cs = c->rope_cs;
    a.q_norm = c->q_norm + (size_t)l * c->D;
    a.k_norm = c->k_norm + (size_t)l * c->D;
    a.rings = rings;
    a.layer = l;
    a.L = c->L;
    a.Hkv = c->Hkv;
    a.W = c->W;
    a.ring_dtype = c->cfg.ring_dtype;
    a.G = c->H / c->Hkv;
    a.NCH = c->NCH;
    a.block = c->cfg.block;
    a.n_past = n_past;
    a.eps = c->cfg.rms_eps;
    a.scale = 1.0f / sqrtf((float)c->D);
    a.ml = c->att_ml;
    a.o = c->att_o;
    dim3 grid(c->NCH + 1, c->Hkv, B);
    if (c->D == 128)
        hipLaunchKernelGGL(attn_partial_kernel<128>, grid, dim3(256), 0, s, a);
    else if (c->D == 64)
        hipLaunchKernelGGL(attn_partial_kernel<64>, grid, dim3(256), 0, s, a);
    else
        return hipErrorInvalidValue;
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    CombArgs cb;
    cb.ml = c->att_ml;
    cb.o = c->att_o;
    cb.NCH = c->NCH;
    cb.G = a.G;
    cb.Hkv = c->Hkv;
    cb.D = c->D;
    cb.block = c->cfg.block;
    cb.act_o = c->act_o;
    cb.act_fmt = c->act_fmt;
    cb.act_rows = c->Mmax;
    cb.qdim = c->qdim;
    hipLaunchKernelGGL(attn_combine_kernel, dim3(c->H, B), dim3(256), 0, s, cb);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Acceptance scan: one wavefront per sequence; lane i compares draft i with the
// target token; the first set bit of the mismatch ballot is n_ok.
// ---------------------------------------------------------------------------
__global__ void accept_kernel(const int32_t *drafts, const int32_t *target, int n, int32_t *n_ok) {
    const int b = blockIdx.x, lane = threadIdx.x;
    const bool mis = lane < n && drafts[(size_t)b * n + lane] != target[(size_t)b * n + lane];
    const unsigned long long mask = __ballot(mis);
    if (lane == 0) n_ok[b] = mask ? (__ffsll((long long)mask) - 1) : n;
}

hipError_t launch_accept(const int32_t *drafts, const int32_t *target, int B, int n, int32_t *n_ok, hipStream_t s) {
    hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(64), 0, s, drafts, target, n, n_ok);
    return hipGetLastError();
}
