// KIVI-style 2-bit asymmetric KV cache: append (prefill / decode) and decode
// attention over the quantized and fp16 segments with one softmax.
//
// KIVI page ("KIVI 完全拆解：非对称 2-bit KV Cache 量化"): "definitions"
// (q = clamp(round(x/s + z), 0, 2^b - 1), x_hat = s (q - z), [min, max]
// split evenly by s), "core design" (keys per channel over G-token groups,
// values per token, fp16 residual of at most R rows, the prefill/decode
// pseudo-code, segment logits concatenated under one softmax, fp16 scale and
// zero-point), "engineering" (the shared-normaliser pitfall).
#include "common.h"

#include <algorithm>

namespace lvq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct KArgs {
    int D, H, G, R, cap, ring;
    kivi_cache c;
};

__device__ __forceinline__ uint16_t* U16(void* p) { return static_cast<uint16_t*>(p); }

// The quantizer in IEEE binary32 steps (round to nearest even, no contraction).
struct GroupParams {
    uint16_t s16, z16;
    float s, z;
};

__device__ __forceinline__ GroupParams group_params(float mn, float mx) {
    GroupParams p;
    p.s16 = f32_to_f16_rne(__fdiv_rn(__fsub_rn(mx, mn), 3.0f));
    if ((p.s16 & 0x7fff) == 0) p.s16 = 0x3c00;       // s == 0 (constant group) -> 1
    p.s = f16_to_f32(p.s16);
    p.z16 = f32_to_f16_rne(__fdiv_rn(-mn, p.s));
    p.z = f16_to_f32(p.z16);
    return p;
}

__device__ __forceinline__ uint32_t code_of(float x, float s, float z) {
    float u = __fadd_rn(__fdiv_rn(x, s), z);
    u = rintf(u);
    u = fminf(fmaxf(u, 0.f), 3.f);
    return uint32_t(u);
}

__device__ __forceinline__ long bh(const KArgs& a, int b, int h) { return long(b) * a.H + h; }

// Key groups: one thread per (group of 32 tokens, 4 channels).  Tokens come
// from `src(token)` rows of D fp16 values.
template <typename Src>
__device__ void quantize_key_group(const KArgs& a, int b, int h, int gi, int quad, Src src) {
    const int D = a.D;
    float mn[4], mx[4];
    for (int u = 0; u < 4; ++u) { mn[u] = INFINITY; mx[u] = -INFINITY; }
    for (int j = 0; j < a.G; ++j) {
        const uint16_t* row = src(gi * a.G + j);
        for (int u = 0; u < 4; ++u) {
            const float x = f16_to_f32(row[quad * 4 + u]);
            mn[u] = fminf(mn[u], x);
            mx[u] = fmaxf(mx[u], x);
        }
    }
    GroupParams gp[4];
    for (int u = 0; u < 4; ++u) {
        gp[u] = group_params(mn[u], mx[u]);
        U16(a.c.k_scale)[(bh(a, b, h) * (a.cap / a.G) + gi) * D + quad * 4 + u] = gp[u].s16;
        U16(a.c.k_zero)[(bh(a, b, h) * (a.cap / a.G) + gi) * D + quad * 4 + u] = gp[u].z16;
    }
    for (int j = 0; j < a.G; ++j) {
        const int tok = gi * a.G + j;
        const uint16_t* row = src(tok);
        uint32_t byte = 0;
        for (int u = 0; u < 4; ++u) byte |= code_of(f16_to_f32(row[quad * 4 + u]), gp[u].s, gp[u].z) << (2 * u);
        a.c.k_codes[(bh(a, b, h) * a.cap + tok) * (D / 4) + quad] = uint8_t(byte);
    }
}

// Value groups: one thread per (token, group of 32 channels).
__device__ void quantize_value_group(const KArgs& a, int b, int h, int tok, int gi, const uint16_t* row) {
    const int D = a.D;
    float mn = INFINITY, mx = -INFINITY;
    for (int e = 0; e < a.G; ++e) {
        const float x = f16_to_f32(row[gi * a.G + e]);
        mn = fminf(mn, x);
        mx = fmaxf(mx, x);
    }
    const GroupParams gp = group_params(mn, mx);
    U16(a.c.v_scale)[(bh(a, b, h) * a.cap + tok) * (D / a.G) + gi] = gp.s16;
    U16(a.c.v_zero)[(bh(a, b, h) * a.cap + tok) * (D / a.G) + gi] = gp.z16;
    uint8_t* out = a.c.v_codes + (bh(a, b, h) * a.cap + tok) * (D / 4) + gi * a.G / 4;
    for (int e = 0; e < a.G; e += 4) {
        uint32_t byte = 0;
        for (int u = 0; u < 4; ++u)
            byte |= code_of(f16_to_f32(row[gi * a.G + e + u]), gp.s, gp.z) << (2 * u);
        out[e / 4] = uint8_t(byte);
    }
}

// ---------------------------------------------------------------------------
// Prefill
// ---------------------------------------------------------------------------
struct NewSrc {
    const uint16_t* base;
    long s0, s1, s2;
    __device__ const uint16_t* row(int b, int h, int j) const { return base + b * s0 + h * s1 + j * s2; }
};

__global__ void prefill_keys_kernel(KArgs a, NewSrc k, int n_kq) {
    // grid (groups, H, B), block D/4 threads
    const int gi = blockIdx.x, h = blockIdx.y, b = blockIdx.z, quad = threadIdx.x;
    (void)n_kq;
    quantize_key_group(a, b, h, gi, quad, [&](int tok) { return k.row(b, h, tok); });
}

__global__ void prefill_values_kernel(KArgs a, NewSrc v, int n_vq) {
    // grid (ceil(n_vq*ngroups/256), H, B), block 256: thread = (token, channel group)
    const int ng = a.D / a.G;
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    const int h = blockIdx.y, b = blockIdx.z;
    if (e >= n_vq * ng) return;
    const int tok = e / ng, gi = e % ng;
    quantize_value_group(a, b, h, tok, gi, v.row(b, h, tok));
}

__global__ void prefill_residual_kernel(KArgs a, NewSrc k, NewSrc v, int L, int n_kq, int n_vq) {
    // grid (L - min(n_kq, n_vq), H, B), block D: copies rows into the rings.
    const int first = min(n_kq, n_vq);
    const int tok = first + blockIdx.x, h = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
    if (tok >= L) return;
    const long slot = bh(a, b, h) * a.ring + tok % a.ring;
    if (tok >= n_kq) U16(a.c.k_res)[slot * a.D + d] = k.row(b, h, tok)[d];
    if (tok >= n_vq) U16(a.c.v_res)[slot * a.D + d] = v.row(b, h, tok)[d];
}

__global__ void prefill_counters_kernel(KArgs a, int B, int L, int n_kq, int n_vq) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    a.c.len[b] = L;
    a.c.n_kq[b] = n_kq;
    a.c.n_vq[b] = n_vq;
}

// ---------------------------------------------------------------------------
// Decode append: grid (H, B), block 128.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(128) decode_append_kernel(KArgs a, NewSrc k, NewSrc v) {
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int L0 = a.c.len[b], nk = a.c.n_kq[b], nv = a.c.n_vq[b];
    if (L0 < 0 || L0 >= a.cap) return;          // full cache: the token is dropped
    const long base = bh(a, b, h) * a.ring;
    const int p = L0;
    for (int d = tid; d < a.D; d += blockDim.x) {
        U16(a.c.k_res)[(base + p % a.ring) * a.D + d] = k.row(b, h, 0)[d];
        U16(a.c.v_res)[(base + p % a.ring) * a.D + d] = v.row(b, h, 0)[d];
    }
    __syncthreads();
    const int rk = L0 + 1 - nk;
    if (rk >= a.R) {
        // quantize key rows [nk, nk + R): R/G groups x D/4 channel quads
        const int nquads = a.D / 4, ngroups = a.R / a.G;
        for (int e = tid; e < ngroups * nquads; e += blockDim.x) {
            const int gl = e / nquads, quad = e % nquads;
            const int gi = nk / a.G + gl;
            quantize_key_group(a, b, h, gi, quad, [&](int tok) {
                return U16(a.c.k_res) + (base + tok % a.ring) * a.D;
            });
        }
    }
    const int rv = L0 + 1 - nv;
    if (rv > a.R) {
        const int n_over = rv - a.R, ng = a.D / a.G;
        for (int e = tid; e < n_over * ng; e += blockDim.x) {
            const int tok = nv + e / ng, gi = e % ng;
            quantize_value_group(a, b, h, tok, gi, U16(a.c.v_res) + (base + tok % a.ring) * a.D);
        }
    }
}

__global__ void decode_counters_kernel(KArgs a, int B) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    if (a.c.len[b] < 0 || a.c.len[b] >= a.cap) return;
    const int L1 = a.c.len[b] + 1;
    if (L1 - a.c.n_kq[b] >= a.R) a.c.n_kq[b] += a.R;
    if (L1 - a.c.n_vq[b] > a.R) a.c.n_vq[b] = L1 - a.R;
    a.c.len[b] = L1;
}

// ---------------------------------------------------------------------------
// Decode attention partial: grid (split, H, B), 256 threads (4 waves).  Each
// wave takes every fourth token of the split; lane l owns channels 2l, 2l+1.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) kivi_attn_partial_kernel(KArgs a, const uint16_t* __restrict__ q,
                                                                float scale_log2, int tps, int S_tot, int max_len,
                                                                float* __restrict__ po, float* __restrict__ pl) {
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int D = a.D;
    const int L = min(max(a.c.len[b], 0), max_len);
    const int nk = min(a.c.n_kq[b], L), nv = min(a.c.n_vq[b], L);
    const int t_lo = min(L, split * tps), t_hi = min(L, (split + 1) * tps);
    const long orow = bh(a, b, h) * S_tot + split;
    const int d0 = 2 * lane;
    const uint16_t* qp = q + bh(a, b, h) * D;
    const float q0 = f16_to_f32(qp[d0]), q1 = f16_to_f32(qp[d0 + 1]);
    const long cb = bh(a, b, h) * a.cap;
    float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
    for (int tok = t_lo + wave; tok < t_hi; tok += 4) {
        float k0, k1, v0, v1;
        if (tok < nk) {
            const uint32_t byte = a.c.k_codes[(cb + tok) * (D / 4) + d0 / 4];
            const int sh = 2 * (d0 & 3);
            const long pidx = (bh(a, b, h) * (a.cap / a.G) + tok / a.G) * D + d0;
            const float s0 = f16_to_f32(U16(a.c.k_scale)[pidx]), s1 = f16_to_f32(U16(a.c.k_scale)[pidx + 1]);
            const float z0 = f16_to_f32(U16(a.c.k_zero)[pidx]), z1 = f16_to_f32(U16(a.c.k_zero)[pidx + 1]);
            k0 = s0 * (float((byte >> sh) & 3) - z0);
            k1 = s1 * (float((byte >> (sh + 2)) & 3) - z1);
        } else {
            const uint16_t* r = U16(a.c.k_res) + (bh(a, b, h) * a.ring + tok % a.ring) * D;
            k0 = f16_to_f32(r[d0]);
            k1 = f16_to_f32(r[d0 + 1]);
        }
        const float s = wave_sum(q0 * k0 + q1 * k1) * scale_log2;
        if (tok < nv) {
            const uint32_t byte = a.c.v_codes[(cb + tok) * (D / 4) + d0 / 4];
            const int sh = 2 * (d0 & 3);
            const long pidx = (cb + tok) * (D / a.G) + d0 / a.G;
            const float sv = f16_to_f32(U16(a.c.v_scale)[pidx]), zv = f16_to_f32(U16(a.c.v_zero)[pidx]);
            v0 = sv * (float((byte >> sh) & 3) - zv);
            v1 = sv * (float((byte >> (sh + 2)) & 3) - zv);
        } else {
            const uint16_t* r = U16(a.c.v_res) + (bh(a, b, h) * a.ring + tok % a.ring) * D;
            v0 = f16_to_f32(r[d0]);
            v1 = f16_to_f32(r[d0 + 1]);
        }
        const float m_new = fmaxf(m, s);
        const float alpha = exp2f(m - m_new), w = exp2f(s - m_new);
        l = l * alpha + w;
        o0 = o0 * alpha + w * v0;
        o1 = o1 * alpha + w * v1;
        m = m_new;
    }
    __shared__ float red[4][130];
    red[wave][d0] = o0;
    red[wave][d0 + 1] = o1;
    if (lane == 0) {
        red[wave][128] = m;
        red[wave][129] = l;
    }
    __syncthreads();
    if (tid < D) {
        float M = -INFINITY;
        for (int w2 = 0; w2 < 4; ++w2) M = fmaxf(M, red[w2][128]);
        if (M == -INFINITY) {
            po[orow * D + tid] = 0.f;
            if (tid == 0) pl[orow] = -INFINITY;
            return;
        }
        float Ls = 0.f, o = 0.f;
        for (int w2 = 0; w2 < 4; ++w2) {
            const float fw = red[w2][128] == -INFINITY ? 0.f : exp2f(red[w2][128] - M);
            Ls += red[w2][129] * fw;
            o += red[w2][tid] * fw;
        }
        po[orow * D + tid] = o / Ls;
        if (tid == 0) pl[orow] = (M + log2f(Ls)) * kLn2;
    }
}

__global__ void kivi_merge_kernel(const float* __restrict__ po, const float* __restrict__ pl, int S, int D,
                                  float* __restrict__ out, float* __restrict__ lse_out) {
    const long n = blockIdx.x;
    const float* lr = pl + n * S;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, lr[s]);
    float L = 0.f;
    if (M != -INFINITY)
        for (int s = 0; s < S; ++s) L += (lr[s] == -INFINITY) ? 0.f : __expf(lr[s] - M);
    const float lse = (M == -INFINITY) ? -INFINITY : M + __logf(L);
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float o = 0.f;
        if (M != -INFINITY)
            for (int s = 0; s < S; ++s)
                if (lr[s] != -INFINITY) o += __expf(lr[s] - lse) * po[(n * S + s) * D + d];
        out[n * D + d] = o;
    }
    if (lse_out && threadIdx.x == 0) lse_out[n] = lse;
}

lvq_status validate_kivi(const kivi_geom* g, const kivi_cache* c) {
    LVQ_REQUIRE(g && c, LVQ_ERR_INVALID_ARG, "kivi: NULL geometry or cache");
    LVQ_REQUIRE(g->D == 128, LVQ_ERR_UNSUPPORTED, "kivi: head dimension %d unsupported (128)", g->D);
    LVQ_REQUIRE(g->bits == 2, LVQ_ERR_UNSUPPORTED, "kivi: %d-bit codes unsupported (2)", g->bits);
    LVQ_REQUIRE(g->group == 32, LVQ_ERR_UNSUPPORTED, "kivi: group %d unsupported (32)", g->group);
    LVQ_REQUIRE(g->H > 0 && g->R > 0 && g->R % g->group == 0, LVQ_ERR_INVALID_ARG,
                "kivi: R=%d must be a positive multiple of the group", g->R);
    LVQ_REQUIRE(g->cap > 0 && g->cap % g->group == 0, LVQ_ERR_INVALID_ARG,
                "kivi: capacity %d must be a positive multiple of the group", g->cap);
    LVQ_REQUIRE(c->k_codes && c->k_scale && c->k_zero && c->v_codes && c->v_scale && c->v_zero && c->k_res &&
                    c->v_res && c->len && c->n_kq && c->n_vq,
                LVQ_ERR_INVALID_ARG, "kivi: NULL cache pointer");
    return LVQ_OK;
}

KArgs make_args(const kivi_geom* g, const kivi_cache* c) {
    KArgs a;
    a.D = g->D; a.H = g->H; a.G = g->group; a.R = g->R; a.cap = g->cap; a.ring = g->R + g->group;
    a.c = *c;
    return a;
}

int choose_kivi_splits(const kivi_geom* g, int B, int max_len) {
    const int wgs = B * g->H;
    int s = ceil_div(1024, std::max(1, wgs));
    s = std::max(s, ceil_div(max_len, 2048));
    s = std::min(s, std::max(1, ceil_div(max_len, 64)));
    return std::max(1, std::min(s, 1024));
}

}  // namespace
}  // namespace lvq

using namespace lvq;

extern "C" lvq_status kivi_append(const kivi_geom* g, const void* k_new, const void* v_new,
                                  const int64_t new_strides[3], int32_t n_new, int32_t prefill,
                                  const kivi_cache* c, int32_t B, hipStream_t stream) {
    lvq_status st = validate_kivi(g, c);
    if (st != LVQ_OK) return st;
    LVQ_REQUIRE(k_new && v_new && new_strides, LVQ_ERR_INVALID_ARG, "kivi_append: NULL input");
    LVQ_REQUIRE(B >= 0 && B <= 65535, LVQ_ERR_INVALID_ARG, "kivi_append: batch %d", B);
    LVQ_REQUIRE(n_new >= 1, LVQ_ERR_INVALID_ARG, "kivi_append: n_new %d < 1", n_new);
    LVQ_REQUIRE(prefill || n_new == 1, LVQ_ERR_UNSUPPORTED, "kivi_append: decode appends one token per call");
    LVQ_REQUIRE(n_new <= g->cap, LVQ_ERR_INVALID_ARG, "kivi_append: %d tokens exceed capacity %d", n_new, g->cap);
    if (B == 0) return LVQ_OK;
    KArgs a = make_args(g, c);
    NewSrc ks{static_cast<const uint16_t*>(k_new), long(new_strides[0]), long(new_strides[1]), long(new_strides[2])};
    NewSrc vs{static_cast<const uint16_t*>(v_new), long(new_strides[0]), long(new_strides[1]), long(new_strides[2])};
    if (prefill) {
        const int n_kq = g->group * std::max(0, (n_new - g->R) / g->group);
        const int n_vq = std::max(0, n_new - g->R);
        if (n_kq > 0) {
            hipLaunchKernelGGL(prefill_keys_kernel, dim3(n_kq / g->group, g->H, B), dim3(g->D / 4), 0, stream, a, ks,
                               n_kq);
            if ((st = check_launch("kivi_append: keys")) != LVQ_OK) return st;
        }
        if (n_vq > 0) {
            const int ng = g->D / g->group;
            hipLaunchKernelGGL(prefill_values_kernel, dim3(ceil_div(long(n_vq) * ng, 256), g->H, B), dim3(256), 0,
                               stream, a, vs, n_vq);
            if ((st = check_launch("kivi_append: values")) != LVQ_OK) return st;
        }
        const int first = std::min(n_kq, n_vq);
        hipLaunchKernelGGL(prefill_residual_kernel, dim3(n_new - first, g->H, B), dim3(g->D), 0, stream, a, ks, vs,
                           n_new, n_kq, n_vq);
        if ((st = check_launch("kivi_append: residual")) != LVQ_OK) return st;
        hipLaunchKernelGGL(prefill_counters_kernel, dim3(ceil_div(B, 256)), dim3(256), 0, stream, a, B, n_new, n_kq,
                           n_vq);
        return check_launch("kivi_append: counters");
    }
    hipLaunchKernelGGL(decode_append_kernel, dim3(g->H, B), dim3(128), 0, stream, a, ks, vs);
    if ((st = check_launch("kivi_append: decode")) != LVQ_OK) return st;
    hipLaunchKernelGGL(decode_counters_kernel, dim3(ceil_div(B, 256)), dim3(256), 0, stream, a, B);
    return check_launch("kivi_append: counters");
}

extern "C" size_t kivi_decode_attn_workspace(const kivi_geom* g, int32_t B, int32_t max_len, int32_t num_splits) {
    if (!g || B < 0 || max_len < 0 || num_splits < 0 || g->H <= 0 || g->D <= 0) return 0;
    const int S = num_splits > 0 ? num_splits : choose_kivi_splits(g, B, max_len);
    const size_t rows = size_t(B) * g->H * S;
    return rows * g->D * sizeof(float) + rows * sizeof(float);
}

extern "C" lvq_status kivi_decode_attn(const kivi_geom* g, const void* q, const kivi_cache* c, int32_t max_len,
                                       float sm_scale, float* out, float* lse_out, void* ws, size_t ws_bytes,
                                       int32_t num_splits, int32_t B, hipStream_t stream) {
    lvq_status st = validate_kivi(g, c);
    if (st != LVQ_OK) return st;
    LVQ_REQUIRE(B >= 0 && B <= 65535 && max_len >= 1 && max_len <= g->cap, LVQ_ERR_INVALID_ARG,
                "kivi_decode_attn: bad sizes B=%d max_len=%d", B, max_len);
    LVQ_REQUIRE(num_splits >= 0 && num_splits <= 1024, LVQ_ERR_INVALID_ARG, "kivi_decode_attn: num_splits %d",
                num_splits);
    LVQ_REQUIRE(std::isfinite(sm_scale), LVQ_ERR_INVALID_ARG, "kivi_decode_attn: sm_scale not finite");
    if (B == 0) return LVQ_OK;
    LVQ_REQUIRE(q && out && ws, LVQ_ERR_INVALID_ARG, "kivi_decode_attn: NULL pointer");
    const int S = num_splits > 0 ? num_splits : choose_kivi_splits(g, B, max_len);
    const size_t need = kivi_decode_attn_workspace(g, B, max_len, S);
    LVQ_REQUIRE(ws_bytes >= need, LVQ_ERR_WORKSPACE, "kivi_decode_attn: workspace %zu < %zu bytes", ws_bytes, need);
    KArgs a = make_args(g, c);
    const size_t rows = size_t(B) * g->H * S;
    float* po = static_cast<float*>(ws);
    float* pl = po + rows * g->D;
    const int tps = ceil_div(max_len, S);
    hipLaunchKernelGGL(kivi_attn_partial_kernel, dim3(S, g->H, B), dim3(256), 0, stream, a,
                       static_cast<const uint16_t*>(q), sm_scale * kLog2e, tps, S, max_len, po, pl);
    if ((st = check_launch("kivi_decode_attn: partial")) != LVQ_OK) return st;
    hipLaunchKernelGGL(kivi_merge_kernel, dim3(B * g->H), dim3(128), 0, stream, po, pl, S, g->D, out, lse_out);
    return check_launch("kivi_decode_attn: merge");
}
