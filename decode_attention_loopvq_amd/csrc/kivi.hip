// KIVI-style asymmetric KV cache with 2- or 4-bit codes (key and value widths
// chosen apart): append (prefill / decode) and decode attention over the
// quantized and fp16 segments with one softmax, for Hq query heads sharing
// each of the H KV heads (grouped-query attention).
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
    int kb, vb;           // key and value code widths (2 or 4 bits)
    int nrep;             // query heads per KV head
    kivi_cache c;
};

__device__ __forceinline__ uint16_t* U16(void* p) { return static_cast<uint16_t*>(p); }

// The quantizer in IEEE binary32 steps (round to nearest even, no contraction).
struct GroupParams {
    uint16_t s16, z16;
    float s, z;
};

// levels = 2^b - 1
__device__ __forceinline__ GroupParams group_params(float mn, float mx, float levels) {
    GroupParams p;
    p.s16 = f32_to_f16_rne(__fdiv_rn(__fsub_rn(mx, mn), levels));
    if ((p.s16 & 0x7fff) == 0) p.s16 = 0x3c00;       // s == 0 (constant group) -> 1
    p.s = f16_to_f32(p.s16);
    p.z16 = f32_to_f16_rne(__fdiv_rn(-mn, p.s));
    p.z = f16_to_f32(p.z16);
    return p;
}

__device__ __forceinline__ uint32_t code_of(float x, float s, float z, float levels) {
    float u = __fadd_rn(__fdiv_rn(x, s), z);
    u = rintf(u);
    u = fminf(fmaxf(u, 0.f), levels);
    return uint32_t(u);
}

// The same code with the quotient fl32(x / s) from r = v_rcp_f32(s) and one Newton step on the quotient
// (Markstein): q0 = x r, e = x - q0 s (exact in one FMA), q = q0 + e r rounded once.  For fp16 x and s
// this is the correctly rounded quotient: x / s = M / N 2^k with N < 2^11, so unless it is exact it lies
// at least 2^-12 ulp from every rounding midpoint, while q0 + e r is within 2^-20 ulp of x / s
// (|e| <= 2 ulp(q0) s and |r - 1/s| <= 1 ulp(1/s)).
__device__ __forceinline__ uint32_t code_of_r(float x, float s, float r, float z, float levels) {
    const float q0 = x * r;
    const float e = fmaf(-q0, s, x);
    float u = __fadd_rn(fmaf(e, r, q0), z);
    u = rintf(u);
    u = fminf(fmaxf(u, 0.f), levels);
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
    const int kb = a.kb;
    const float levels = float((1 << kb) - 1);
    GroupParams gp[4];
    for (int u = 0; u < 4; ++u) {
        gp[u] = group_params(mn[u], mx[u], levels);
        U16(a.c.k_scale)[(bh(a, b, h) * (a.cap / a.G) + gi) * D + quad * 4 + u] = gp[u].s16;
        U16(a.c.k_zero)[(bh(a, b, h) * (a.cap / a.G) + gi) * D + quad * 4 + u] = gp[u].z16;
    }
    for (int j = 0; j < a.G; ++j) {
        const int tok = gi * a.G + j;
        const uint16_t* row = src(tok);
        uint32_t word = 0;             // 4 channels: kb / 2 bytes
        for (int u = 0; u < 4; ++u)
            word |= code_of(f16_to_f32(row[quad * 4 + u]), gp[u].s, gp[u].z, levels) << (kb * u);
        uint8_t* dst = a.c.k_codes + (bh(a, b, h) * a.cap + tok) * (D * kb / 8) + quad * (kb / 2);
        for (int i = 0; i < kb / 2; ++i) dst[i] = uint8_t(word >> (8 * i));
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
    const int vb = a.vb;
    const float levels = float((1 << vb) - 1);
    const GroupParams gp = group_params(mn, mx, levels);
    U16(a.c.v_scale)[(bh(a, b, h) * a.cap + tok) * (D / a.G) + gi] = gp.s16;
    U16(a.c.v_zero)[(bh(a, b, h) * a.cap + tok) * (D / a.G) + gi] = gp.z16;
    uint8_t* out = a.c.v_codes + (bh(a, b, h) * a.cap + tok) * (D * vb / 8) + gi * a.G * vb / 8;
    for (int e = 0; e < a.G; e += 4) {
        uint32_t word = 0;             // 4 channels: vb / 2 bytes
        for (int u = 0; u < 4; ++u)
            word |= code_of(f16_to_f32(row[gi * a.G + e + u]), gp.s, gp.z, levels) << (vb * u);
        for (int i = 0; i < vb / 2; ++i) out[(e / 4) * (vb / 2) + i] = uint8_t(word >> (8 * i));
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
// Prefill in one pass (D = 128, group 32, 16-byte aligned rows): grid
// (ceil(L / 128), H, B), 256 threads.  Wave w takes tokens t0 .. t0+31,
// t0 = 128 bx + 32 w (one key group); lane l holds channels 8(l & 15) .. +7
// of tokens t0 + 8(l >> 4) .. +7, K and V each loaded once (16 bytes per lane
// and token, V after K is done).  Keys of a whole quantized group: per-channel minimum and
// maximum over the lane's 8 tokens, then over the 4 lanes l ^ 16k (permlane
// swaps).  Values of quantized tokens: per-token minimum and maximum over the
// lane's 8 channels, then over the 4 lanes of the 32-channel group (DPP).
// Codes go out 8 * bits / 8 bytes per lane and token; the rows past the quantized
// ranges go to the fp16 rings; block (0, 0, b) sets request b's counters.
// ---------------------------------------------------------------------------
template <typename F>
__device__ __forceinline__ float rows4_reduce(float x, F op) {   // over lanes l, l ^ 16, l ^ 32, l ^ 48
    const uint32_t xi = __float_as_uint(x);
    const auto t = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
    const uint32_t t0 = t[0], t1 = t[1];
    const float y = op(__uint_as_float(t0), __uint_as_float(t1));
    const uint32_t yi = __float_as_uint(y);
    const auto u = __builtin_amdgcn_permlane16_swap(yi, yi, false, false);
    const uint32_t u0 = u[0], u1 = u[1];
    return op(__uint_as_float(u0), __uint_as_float(u1));
}
template <int CTRL>
__device__ __forceinline__ float kdpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// the 8 fp16 of a 16-byte word as floats
__device__ __forceinline__ void half8_f(const uint4& w, float (&f)[8]) {
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        f[2 * u] = f16_to_f32(uint16_t(d[u] & 0xffffu));
        f[2 * u + 1] = f16_to_f32(uint16_t(d[u] >> 16));
    }
}

// the codes of a lane's 8 channels (8 * BITS bits) into their place in a token's code row
template <int BITS>
__device__ __forceinline__ void store_codes8(uint8_t* row, int co, uint32_t word) {
    if constexpr (BITS == 2) *reinterpret_cast<uint16_t*>(row + 2 * co) = uint16_t(word);
    else *reinterpret_cast<uint32_t*>(row + 4 * co) = word;
}

template <int KB, int VB>
__global__ void __launch_bounds__(256, 4) prefill_kv_kernel(KArgs a, NewSrc k, NewSrc v, int L, int n_kq, int n_vq) {
    constexpr int D = 128, G = 32;
    constexpr float kLevels = float((1 << KB) - 1), vLevels = float((1 << VB) - 1);
    const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x, lane = tid & 63;
    const int t0 = blockIdx.x * 128 + (tid >> 6) * 32;
    const int co = lane & 15, tq = lane >> 4;
    const long bhi = bh(a, b, h);
    if (blockIdx.x == 0 && h == 0 && tid == 0) {
        a.c.len[b] = L;
        a.c.n_kq[b] = n_kq;
        a.c.n_vq[b] = n_vq;
    }
    if (t0 >= L) return;                            // (whole wave)
    uint4 kx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int t = min(t0 + 8 * tq + i, L - 1);  // rows past L load a valid row and are not stored
        kx[i] = *reinterpret_cast<const uint4*>(k.row(b, h, t) + 8 * co);
    }
    // ---- keys: one group of 32 tokens per wave ----
    if (t0 + G <= n_kq) {
        float mn[8], mx[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) { mn[u] = INFINITY; mx[u] = -INFINITY; }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float f[8];
            half8_f(kx[i], f);
#pragma unroll
            for (int u = 0; u < 8; ++u) { mn[u] = fminf(mn[u], f[u]); mx[u] = fmaxf(mx[u], f[u]); }
        }
        GroupParams gp[8];
        float rs[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            mn[u] = rows4_reduce(mn[u], [](float p, float q) { return fminf(p, q); });
            mx[u] = rows4_reduce(mx[u], [](float p, float q) { return fmaxf(p, q); });
            gp[u] = group_params(mn[u], mx[u], kLevels);
            rs[u] = __builtin_amdgcn_rcpf(gp[u].s);
        }
        if (tq == 0) {
            const long pofs = (bhi * (a.cap / G) + t0 / G) * D + 8 * co;
            uint32_t sw[4], zw[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                sw[u] = uint32_t(gp[2 * u].s16) | uint32_t(gp[2 * u + 1].s16) << 16;
                zw[u] = uint32_t(gp[2 * u].z16) | uint32_t(gp[2 * u + 1].z16) << 16;
            }
            *reinterpret_cast<uint4*>(U16(a.c.k_scale) + pofs) = make_uint4(sw[0], sw[1], sw[2], sw[3]);
            *reinterpret_cast<uint4*>(U16(a.c.k_zero) + pofs) = make_uint4(zw[0], zw[1], zw[2], zw[3]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float f[8];
            half8_f(kx[i], f);
            uint32_t c2 = 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) c2 |= code_of_r(f[u], gp[u].s, rs[u], gp[u].z, kLevels) << (KB * u);
            const int t = t0 + 8 * tq + i;
            store_codes8<KB>(a.c.k_codes + (bhi * a.cap + t) * (D * KB / 8), co, c2);
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {                   // key rows past the quantized groups: fp16 ring
        const int t = t0 + 8 * tq + i;
        if (t < L && t >= n_kq) *reinterpret_cast<uint4*>(U16(a.c.k_res) + (bhi * a.ring + t % a.ring) * D + 8 * co) = kx[i];
    }
    // ---- values: per token, groups of 32 channels (lanes 4g .. 4g+3 of a row) ----
    uint4 vx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) vx[i] = *reinterpret_cast<const uint4*>(v.row(b, h, min(t0 + 8 * tq + i, L - 1)) + 8 * co);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int t = t0 + 8 * tq + i;
        float f[8];
        half8_f(vx[i], f);
        float mn = f[0], mx = f[0];
#pragma unroll
        for (int u = 1; u < 8; ++u) { mn = fminf(mn, f[u]); mx = fmaxf(mx, f[u]); }
        mn = fminf(mn, kdpp_f<0xb1>(mn));           // quad_perm [1,0,3,2]
        mx = fmaxf(mx, kdpp_f<0xb1>(mx));
        mn = fminf(mn, kdpp_f<0x4e>(mn));           // quad_perm [2,3,0,1]
        mx = fmaxf(mx, kdpp_f<0x4e>(mx));
        if (t < n_vq) {
            const GroupParams gp = group_params(mn, mx, vLevels);
            const float r = __builtin_amdgcn_rcpf(gp.s);
            uint32_t c2 = 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) c2 |= code_of_r(f[u], gp.s, r, gp.z, vLevels) << (VB * u);
            store_codes8<VB>(a.c.v_codes + (bhi * a.cap + t) * (D * VB / 8), co, c2);
            if ((co & 3) == 0) {
                U16(a.c.v_scale)[(bhi * a.cap + t) * (D / G) + (co >> 2)] = gp.s16;
                U16(a.c.v_zero)[(bhi * a.cap + t) * (D / G) + (co >> 2)] = gp.z16;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {                   // value rows past the quantized tokens: fp16 ring
        const int t = t0 + 8 * tq + i;
        if (t < L && t >= n_vq) *reinterpret_cast<uint4*>(U16(a.c.v_res) + (bhi * a.ring + t % a.ring) * D + 8 * co) = vx[i];
    }
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
// Decode attention partial on the VALU, per token (the kernel for 32 query heads per KV head, and the body
// of the residual slot of the matrix-core kernel further below): grid (split, KV head h, B), 256 threads in 32 lane
// groups of 8; lane c of a group owns channels 16c .. 16c+15 (16 * bits bits
// of codes per token: one dword at 2 bits, two at 4).  The nrep query heads of
// KV head h share the workgroup in sets of HPL (2 when nrep is even, else 1): lane group lg
// serves set lg % (nrep / HPL) and takes every (32 / (nrep / HPL))-th token
// range; it dequantises each token once and scores it for the HPL heads of
// its set, and the lane groups of different sets in one wave read the same
// code words in the same instruction.  A split is a multiple of 32 tokens.  Fast path: a lane
// group takes whole 32-token key groups inside the fully quantized range
// [0, min(n_kq, n_vq)); it loads the group's key scale/zero once and the
// codes and value parameters of TB tokens at once (all 32 at 2 bits, 16 at a
// time when a side has 4-bit codes), scores them (q_d s_d folded into one
// weight per channel, the zero point into one bias), then adds their values
// (rescaling its running softmax per batch):
//   o_d += p_t s_t (c_td - z_t)  =  sum_t (p_t s_t) c_td - sum_t p_t s_t z_t,
// the second sum kept once per lane.  Tokens past the quantized range (the
// fp16 residual, a partial group) take a generic path, one or two tokens per lane
// group at a time.  Each lane group keeps its own softmax state; those of one
// query head are combined through LDS.
// ---------------------------------------------------------------------------
constexpr int kKiviLaneGroups = 32;
constexpr int kKiviD = 128;          // head dimension of the attention kernels

template <int CTRL>
__device__ __forceinline__ float kdpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// sum over the 8 lanes of a lane group (every lane gets it)
__device__ __forceinline__ float sum8(float x) {
    x += kdpp<0xb1>(x);      // quad_perm [1,0,3,2]
    x += kdpp<0x4e>(x);      // quad_perm [2,3,0,1]
    x += kdpp<0x141>(x);     // row_half_mirror
    return x;
}

// The code words of one lane's 16 channels: channel j at bits BITS * j.
template <int BITS>
struct Codes16 {
    uint32_t w[BITS / 2];
};
template <int BITS>
__device__ __forceinline__ Codes16<BITS> load_codes16(const uint8_t* row, int c8) {
    Codes16<BITS> c;
    if constexpr (BITS == 2) {
        c.w[0] = reinterpret_cast<const uint32_t*>(row)[c8];
    } else {
        const uint2 v = reinterpret_cast<const uint2*>(row)[c8];
        c.w[0] = v.x;
        c.w[1] = v.y;
    }
    return c;
}
// the 16 codes as floats
template <int BITS>
__device__ __forceinline__ void codes16(const Codes16<BITS>& cw, float (&c)[16]) {
    if constexpr (BITS == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t x = (cw.w[0] >> (2 * k)) & 0x03030303u;    // bytes: channels k, 4+k, 8+k, 12+k
            c[k] = float(x & 0xffu);                                 // v_cvt_f32_ubyte0 .. 3
            c[4 + k] = float((x >> 8) & 0xffu);
            c[8 + k] = float((x >> 16) & 0xffu);
            c[12 + k] = float(x >> 24);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const uint32_t x = (cw.w[i] >> (4 * k)) & 0x0f0f0f0fu;   // bytes: channels 8i + k, +2, +4, +6
                c[8 * i + k] = float(x & 0xffu);
                c[8 * i + 2 + k] = float((x >> 8) & 0xffu);
                c[8 * i + 4 + k] = float((x >> 16) & 0xffu);
                c[8 * i + 6 + k] = float(x >> 24);
            }
    }
}
__device__ __forceinline__ void half8(uint4 w, float* out) {
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        out[2 * u] = f16_to_f32(uint16_t(ww[u]));
        out[2 * u + 1] = f16_to_f32(uint16_t(ww[u] >> 16));
    }
}

// The body of the kernel for one (split, KV head, request); red is the workgroup's combine buffer.  FAST =
// false leaves out the whole-key-group path (a split holding only the rows past them).
template <int KB, int VB, int HPL, bool FAST = true>
__device__ __forceinline__ void kivi_attn_rows(const KArgs& a, const uint16_t* __restrict__ q, float scale_log2,
                                               int S_tot, int max_len, float* __restrict__ po,
                                               float* __restrict__ pl, int split, int h, int b,
                                               float (*red)[kKiviD + 2]) {
    constexpr int D = kKiviD, NLG = kKiviLaneGroups;
    // tokens whose codes are held at once: fewer with 4-bit codes or several heads per lane group
    static_assert(HPL == 1 || HPL == 2, "one or two heads per lane group (four spill registers)");
    constexpr int TB = HPL == 2 ? 8 : (KB == 4 || VB == 4) ? 16 : 32;
    constexpr int KROW = D * KB / 8, VROW = D * VB / 8;  // code bytes per token
    const int tid = threadIdx.x, c8 = tid & 7, lg = tid >> 3;
    // The nrep query heads of KV head h form nset = nrep / HPL sets of HPL heads; lane group lg serves
    // set lg % nset (heads h*nrep + set*HPL + u) and takes every (32 / nset)-th token range.
    const int nset = a.nrep / HPL, hset = lg % nset, tl = lg / nset, NT = NLG / nset;
    const int L = min(max(a.c.len[b], 0), max_len);
    const int nk = min(a.c.n_kq[b], L), nv = min(a.c.n_vq[b], L);
    // Splits 0 .. S_tot-2 share the whole key groups of [0, q_end) (both sides quantized) evenly and the last
    // slot takes the rest (fp16 residual rows, a partial group), so that it runs beside the quantized splits
    // instead of after one of them (a lane group walks those rows one at a time for all its heads).
    const int q_end = min(nk, nv) & ~31;
    const int nq = S_tot - 1;
    int t_lo, t_hi;
    if (split < nq) {
        const int tq = ((q_end + nq - 1) / nq + 31) & ~31;   // whole key groups per split
        t_lo = min(q_end, split * tq);
        t_hi = min(q_end, (split + 1) * tq);
    } else {
        t_lo = q_end;
        t_hi = L;
    }
    const long row = bh(a, b, h);                    // KV row
    const long qrow0 = row * a.nrep + hset * HPL;    // first query row: b * Hq + h * nrep + set * HPL
    const int ch0 = 16 * c8, vg = c8 >> 1;          // channels and their value group
    // the lane's 16 query channels of head u of its set, times sm_scale * log2 e (read again where
    // needed rather than held: with several heads per lane group the registers go to the accumulators)
    auto load_q = [&](int u, float (&qv)[16]) {
        const uint4* qp = reinterpret_cast<const uint4*>(q + (qrow0 + u) * D + ch0);
        half8(qp[0], qv);
        half8(qp[1], qv + 8);
#pragma unroll
        for (int j = 0; j < 16; ++j) qv[j] *= scale_log2;
    };
    float m[HPL], l[HPL], o[HPL][16], ob[HPL];
#pragma unroll
    for (int u = 0; u < HPL; ++u) {
        m[u] = -INFINITY;
        l[u] = 0.f;
        ob[u] = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) o[u][j] = 0.f;
    }
    const long cb = row * a.cap;

    // ---- fast path: whole key groups inside [0, min(nk, nv)) ----
    const int f_hi = FAST ? min(t_hi, q_end) : t_lo;
    for (int t0 = t_lo + 32 * tl; FAST && t0 + 32 <= f_hi; t0 += 32 * NT) {
        float w[HPL][16], bk[HPL];
        {
            const long pidx = (row * (a.cap / 32) + t0 / 32) * D + ch0;
            const uint4* sp = reinterpret_cast<const uint4*>(U16(a.c.k_scale) + pidx);
            const uint4* zp = reinterpret_cast<const uint4*>(U16(a.c.k_zero) + pidx);
            float s16[16], z16[16];
            half8(sp[0], s16); half8(sp[1], s16 + 8);
            half8(zp[0], z16); half8(zp[1], z16 + 8);
#pragma unroll
            for (int u = 0; u < HPL; ++u) {
                float qv[16];
                load_q(u, qv);
                bk[u] = 0.f;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    w[u][j] = qv[j] * s16[j];
                    bk[u] = fmaf(w[u][j], z16[j], bk[u]);
                }
            }
        }
#pragma unroll 1
        for (int tb = 0; tb < 32; tb += TB) {           // rolled: each batch's loads stay in its iteration
            Codes16<KB> kc[TB];
            Codes16<VB> vc[TB];
            uint32_t vs[TB], vz[TB];
#pragma unroll
            for (int k = 0; k < TB; ++k) {
                const long tok = cb + t0 + tb + k;
                kc[k] = load_codes16<KB>(a.c.k_codes + tok * KROW, c8);
                vc[k] = load_codes16<VB>(a.c.v_codes + tok * VROW, c8);
                vs[k] = reinterpret_cast<const uint32_t*>(U16(a.c.v_scale) + tok * (D / 32))[vg >> 1];
                vz[k] = reinterpret_cast<const uint32_t*>(U16(a.c.v_zero) + tok * (D / 32))[vg >> 1];
            }
            float sc[TB][HPL];
            float mb[HPL];
#pragma unroll
            for (int u = 0; u < HPL; ++u) mb[u] = m[u];
#pragma unroll
            for (int k = 0; k < TB; ++k) {
                float c[16];
                codes16<KB>(kc[k], c);                // dequantised once for every head of the set
#pragma unroll
                for (int u = 0; u < HPL; ++u) {
                    float part = -bk[u];
#pragma unroll
                    for (int j = 0; j < 16; ++j) part = fmaf(w[u][j], c[j], part);
                    sc[k][u] = sum8(part);
                    mb[u] = fmaxf(mb[u], sc[k][u]);
                }
            }
            // the batch joins each head's running softmax
#pragma unroll
            for (int u = 0; u < HPL; ++u) {
                const float alpha = __builtin_amdgcn_exp2f(m[u] - mb[u]);
                l[u] *= alpha;
                ob[u] *= alpha;
#pragma unroll
                for (int j = 0; j < 16; ++j) o[u][j] *= alpha;
                m[u] = mb[u];
            }
            const int hsel = 16 * (vg & 1);          // which half of the dword holds this lane's group
#pragma unroll
            for (int k = 0; k < TB; ++k) {
                float c[16];
                codes16<VB>(vc[k], c);
                const float vsf = f16_to_f32(uint16_t(vs[k] >> hsel)), vzf = f16_to_f32(uint16_t(vz[k] >> hsel));
#pragma unroll
                for (int u = 0; u < HPL; ++u) {
                    const float p = __builtin_amdgcn_exp2f(sc[k][u] - m[u]);
                    l[u] += p;
                    const float av = p * vsf;
                    ob[u] = fmaf(av, vzf, ob[u]);
#pragma unroll
                    for (int j = 0; j < 16; ++j) o[u][j] = fmaf(av, c[j], o[u][j]);
                }
            }
        }
    }

    // ---- generic path: the rest of the split, GB tokens per lane group at a time (the loads of all are
    // issued before any is worked, raw; a token past the range repeats the first).  Two in the kernel's
    // own tail; one where the body is the residual slot of the matrix-core kernel, whose registers it
    // would otherwise raise. ----
    const int g_lo = max(t_lo, f_hi);
    constexpr int GB = FAST ? 2 : 1;
    for (int tok0 = g_lo + tl; tok0 < t_hi; tok0 += GB * NT) {
        uint4 kw[GB][4], vw[GB][2];               // key scale and zero (quantized) or key row; value row
        Codes16<KB> kc[GB];
        Codes16<VB> vc[GB];
        uint16_t vs[GB], vz[GB];
#pragma unroll
        for (int j = 0; j < GB; ++j) {
            const int tok = tok0 + j * NT < t_hi ? tok0 + j * NT : tok0;
            if (tok < nk) {
                kc[j] = load_codes16<KB>(a.c.k_codes + (cb + tok) * KROW, c8);
                const long pidx = (row * (a.cap / 32) + tok / 32) * D + ch0;
                const uint4* sp = reinterpret_cast<const uint4*>(U16(a.c.k_scale) + pidx);
                const uint4* zp = reinterpret_cast<const uint4*>(U16(a.c.k_zero) + pidx);
                kw[j][0] = sp[0]; kw[j][1] = sp[1]; kw[j][2] = zp[0]; kw[j][3] = zp[1];
            } else {
                const uint4* r = reinterpret_cast<const uint4*>(U16(a.c.k_res) + (row * a.ring + tok % a.ring) * D + ch0);
                kw[j][0] = r[0]; kw[j][1] = r[1];
            }
            if (tok < nv) {
                vc[j] = load_codes16<VB>(a.c.v_codes + (cb + tok) * VROW, c8);
                vs[j] = U16(a.c.v_scale)[(cb + tok) * (D / 32) + vg];
                vz[j] = U16(a.c.v_zero)[(cb + tok) * (D / 32) + vg];
            } else {
                const uint4* r = reinterpret_cast<const uint4*>(U16(a.c.v_res) + (row * a.ring + tok % a.ring) * D + ch0);
                vw[j][0] = r[0]; vw[j][1] = r[1];
            }
        }
#pragma unroll
        for (int j = 0; j < GB; ++j) {
            const int tok = tok0 + j * NT;
            if (tok >= t_hi) break;
            float kf[16], vf[16];
            if (tok < nk) {
                float c[16], s16[16], z16[16];
                codes16<KB>(kc[j], c);
                half8(kw[j][0], s16); half8(kw[j][1], s16 + 8);
                half8(kw[j][2], z16); half8(kw[j][3], z16 + 8);
#pragma unroll
                for (int i = 0; i < 16; ++i) kf[i] = s16[i] * (c[i] - z16[i]);
            } else {
                half8(kw[j][0], kf); half8(kw[j][1], kf + 8);
            }
            if (tok < nv) {
                float c[16];
                codes16<VB>(vc[j], c);
                const float s1 = f16_to_f32(vs[j]), z1 = f16_to_f32(vz[j]);
#pragma unroll
                for (int i = 0; i < 16; ++i) vf[i] = s1 * (c[i] - z1);
            } else {
                half8(vw[j][0], vf); half8(vw[j][1], vf + 8);
            }
#pragma unroll
            for (int u = 0; u < HPL; ++u) {
                float qv[16];
                load_q(u, qv);
                float part = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) part = fmaf(qv[i], kf[i], part);
                const float sc = sum8(part);
                const float m_new = fmaxf(m[u], sc);
                const float alpha = __builtin_amdgcn_exp2f(m[u] - m_new), p = __builtin_amdgcn_exp2f(sc - m_new);
                l[u] = l[u] * alpha + p;
                ob[u] *= alpha;
#pragma unroll
                for (int i = 0; i < 16; ++i) o[u][i] = fmaf(p, vf[i], o[u][i] * alpha);
                m[u] = m_new;
            }
        }
    }

    // ---- combine the lane groups of each query head, one head of every set per round ----
#pragma unroll
    for (int u = 0; u < HPL; ++u) {
        if (u > 0) __syncthreads();                  // the previous round has read red
#pragma unroll
        for (int j = 0; j < 16; ++j) red[lg][ch0 + j] = o[u][j] - ob[u];
        if (c8 == 0) {
            red[lg][D] = m[u];
            red[lg][D + 1] = l[u];
        }
        __syncthreads();
        for (int e = tid; e < nset * D; e += 256) {
            const int hs = e / D, d = e % D;
            const long orow = (row * a.nrep + hs * HPL + u) * S_tot + split;
            float M = -INFINITY;
            for (int g2 = hs; g2 < NLG; g2 += nset) M = fmaxf(M, red[g2][D]);
            if (M == -INFINITY) {
                po[orow * D + d] = 0.f;
                if (d == 0) pl[orow] = -INFINITY;
                continue;
            }
            float Ls = 0.f, ov = 0.f;
            for (int g2 = hs; g2 < NLG; g2 += nset) {
                const float fw = red[g2][D] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(red[g2][D] - M);
                Ls += red[g2][D + 1] * fw;
                ov += red[g2][d] * fw;
            }
            po[orow * D + d] = ov / Ls;
            if (d == 0) pl[orow] = (M + log2f(Ls)) * kLn2;
        }
    }
}

template <int KB, int VB, int HPL>
__global__ void __launch_bounds__(256, 2) kivi_attn_partial_kernel(KArgs a, const uint16_t* __restrict__ q,
                                                                   float scale_log2, int S_tot,
                                                                   int max_len, float* __restrict__ po,
                                                                   float* __restrict__ pl) {
    __shared__ float red[kKiviLaneGroups][kKiviD + 2];
    kivi_attn_rows<KB, VB, HPL>(a, q, scale_log2, S_tot, max_len, po, pl, blockIdx.x, blockIdx.y, blockIdx.z, red);
}

// ---------------------------------------------------------------------------
// KIVI decode attention on the matrix cores, for 1 to 16 query heads per KV head (nrep; the residual slot
// runs the per-token body with HPL = 2 when nrep is even, else 1).  One workgroup per (split, KV head,
// request), 4 waves; wave w takes the key groups (32 tokens, both sides quantized) w, w + 4, ... of the
// split, and the residual slot (the last split slot, run by the first B * H workgroups so that they all
// start in the first round) runs the per-token body above over the rows past them.  With W[n][c] = q_n[c] s_k[c] (exact: the product of two fp16
// values is the sum of its fp16 rounding and the fma remainder, two chains) and the codes as exact fp16
// integers,
//   logit(t, n) = sm_scale (sum_c code[t][c] W[n][c] - sum_c z_k[c] W[n][c])          (KIVI page, keys)
// is one v_mfma_f32_16x16x32_f16 chain per 16 tokens (rows = tokens, columns = the nrep heads, K = channels)
// plus one chain with z_k as every row (the bias), and with P'_g[t][n] = p(t, n) s_v[t][g] (fp16),
//   o[n][c] = sum_t code_v[t][c] P'_g[t][n] - sum_t z_v[t][g] P'_g[t][n],    g = c / 32   (values)
// is one chain per 16 channels (rows = channels, columns = heads, K = the group's 32 tokens); the second
// sum is kept per lane with dot2.  MFMA lane l = (n, kb) = (l & 15, l >> 4) holds row / column n and
// k-slots 8 kb .. 8 kb + 7.
//  - Keys: lane (m, kb) of a token tile holds token m's channels 32 kb .. 32 kb + 31 (one 8- or 16-byte
//    load); a k-block takes their codes in the order the conversion gives them.  2-bit codes: x &
//    0x33333333 (and the same of x >> 2) leaves one code per nibble and v_cvt_scalef32_pk_f16_fp4 turns
//    the two nibbles of a byte into two exact fp16 values (an fp4 E2M1 nibble k < 4 is k / 2, scaled by
//    2); 4-bit codes: one code per byte and v_cvt_scalef32_pk_f16_fp8 (an fp8 E4M3 byte k < 16 is
//    k * 2^-9, scaled by 512).  So k-slot pair d of k-block kk holds channels 32 kb + gq_kchan(kk, d,
//    0 / 1); W and z_k follow the same order (staged in LDS as pairs).
//  - Values: the value contraction's k-slot s holds token gq_tok(s), chosen so that lane (n, kb) of the
//    key tiles already holds the weights of slots 8 kb .. 8 kb + 7 (tile 0 rows 4 kb + i, tile 1 rows
//    16 + 4 kb + i).  The key group's value codes are byte-transposed into LDS ([code byte][slot]: a lane
//    loads one dword of four consecutive tokens and transposes the 4 x 4 bytes with v_perm), so a lane
//    reads the 8 slots of one code byte with one 8-byte load; 16-channel tile (g, p) puts lane m on
//    channel gq_vchan(g, p, m), all in value group g.  Value codes go through the fp8 conversion: 2-bit
//    codes at bits 2 u of a byte are masked in place for odd u (byte values 0, 4, 8, 12, a quarter of
//    the scale) and shifted by 4 first for u >= 2.
// Online softmax per head in log2 units; a wave rescales only when some lane's maximum grew.  The waves'
// states are combined through LDS.
// ---------------------------------------------------------------------------
typedef _Float16 kh8_t __attribute__((ext_vector_type(8)));
typedef _Float16 kh2_t __attribute__((ext_vector_type(2)));
typedef float kf4_t __attribute__((ext_vector_type(4)));

constexpr int kGqWaves = 4;
constexpr int kVtStride = 40;         // bytes per row of the transposed value codes (32 slots, padded)

// channel (relative to 32 kb) of half e of k-slot pair d of k-block kk, key codes of BITS bits
template <int BITS>
__host__ __device__ constexpr int gq_kchan(int kk, int d, int e) {
    return BITS == 2 ? 16 * (kk >> 1) + 4 * d + (kk & 1) + 2 * e : 8 * kk + 4 * (d & 1) + 2 * e + (d >> 1);
}
// the inverse: (kk * 4 + d) * 2 + e of channel r (relative to 32 kb)
template <int BITS>
__host__ __device__ constexpr int gq_kslot(int r) {
    return BITS == 2 ? ((2 * (r >> 4) + (r & 1)) * 4 + ((r >> 2) & 3)) * 2 + ((r >> 1) & 1)
                     : ((r >> 3) * 4 + 2 * (r & 1) + ((r >> 2) & 1)) * 2 + ((r >> 1) & 1);
}
template <int BITS>
constexpr bool gq_kslots_inverse() {
    for (int kk = 0; kk < 4; ++kk)
        for (int d = 0; d < 4; ++d)
            for (int e = 0; e < 2; ++e)
                if (gq_kslot<BITS>(gq_kchan<BITS>(kk, d, e)) != (kk * 4 + d) * 2 + e) return false;
    return true;
}
static_assert(gq_kslots_inverse<2>() && gq_kslots_inverse<4>(), "gq_kslot inverts gq_kchan");
// channel of row m of value tile (g, p)
template <int BITS>
__host__ __device__ constexpr int gq_vchan(int g, int p, int m) {
    return BITS == 2 ? 32 * g + 4 * (m & 7) + 2 * p + (m >> 3) : 32 * g + 16 * p + 2 * (m & 7) + (m >> 3);
}
// value k-slot of token tau of a key group, and back
__host__ __device__ constexpr int gq_slot(int tau) { return 8 * ((tau & 15) >> 2) + 4 * (tau >> 4) + (tau & 3); }
__host__ __device__ constexpr int gq_tok(int s) { return ((s & 4) << 2) + 4 * (s >> 3) + (s & 3); }
constexpr bool gq_slots_inverse() {
    for (int t = 0; t < 32; ++t)
        if (gq_tok(gq_slot(t)) != t) return false;
    return true;
}
static_assert(gq_slots_inverse(), "gq_slot and gq_tok are inverse permutations of the 32 tokens");

// bytes 2W, 2W + 1 of x (values < 16: an fp8 E4M3 byte k < 16 is k * 2^-9) as fp16, times 2^-9 * scale
template <int W>
__device__ __forceinline__ uint32_t code_pair(uint32_t x, float scale = 512.f) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, scale, W != 0));
}
// the two nibbles of byte B of x (values < 4: an fp4 E2M1 nibble k < 4 is k / 2) as exact fp16
template <int B>
__device__ __forceinline__ uint32_t nib_pair(uint32_t x) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.f, B));
}
__device__ __forceinline__ float fmax2(float x, float y) { return __builtin_amdgcn_fmed3f(x, y, INFINITY); }
// halves r0 and r1 of w (16 dwords, half i of dword i / 2 in natural order) as one dword, r0 in the low half
__device__ __forceinline__ uint32_t half_pair(const uint32_t* w, int r0, int r1) {
    const uint32_t lo = (w[r0 >> 1] >> (16 * (r0 & 1))) & 0xffffu, hi = (w[r1 >> 1] >> (16 * (r1 & 1))) & 0xffffu;
    return lo | (hi << 16);
}

struct GqStage {
    unsigned char vt[64 * kVtStride];   // value codes [code byte][slot]
    uint32_t skp[64], zkp[64];          // key scale / zero point pairs [kb][kk][d]
    uint16_t sv[4][32], zv[4][32];      // value scale / zero point [group][slot]
};
union GqLds {
    GqStage st[kGqWaves];
    float cmb[kGqWaves][16][kKiviD + 2];
    float red[kKiviLaneGroups][kKiviD + 2];
};

template <int KB, int VB>
__global__ void __launch_bounds__(256, 2) kivi_attn_mfma_kernel(KArgs a, const uint16_t* __restrict__ q,
                                                                float scale_log2, int S_tot, int max_len,
                                                                float* __restrict__ po, float* __restrict__ pl) {
    constexpr int D = kKiviD;
    constexpr int KROW = D * KB / 8, VROW = D * VB / 8;
    constexpr int KW = KB == 2 ? 2 : 4, VW = VB == 2 ? 4 : 8;    // key dwords per lane and tile, value dwords per lane
    __shared__ __align__(16) GqLds lds;
    // The residual slots take the first B * H workgroups, so that they all start in the first round beside
    // the others (their per-token path is latency-bound); then (split, KV head, request), split fastest.
    const int nq = S_tot - 1;
    const int lin = blockIdx.x + S_tot * (blockIdx.y + gridDim.y * blockIdx.z), nres = gridDim.y * gridDim.z;
    if (lin < nres) {
        if (a.nrep % 2)
            kivi_attn_rows<KB, VB, 1, false>(a, q, scale_log2, S_tot, max_len, po, pl, nq, lin % gridDim.y,
                                             lin / gridDim.y, lds.red);
        else
            kivi_attn_rows<KB, VB, 2, false>(a, q, scale_log2, S_tot, max_len, po, pl, nq, lin % gridDim.y,
                                             lin / gridDim.y, lds.red);
        return;
    }
    const int split = (lin - nres) % nq, h = ((lin - nres) / nq) % gridDim.y, b = (lin - nres) / (nq * gridDim.y);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, kb = lane >> 4;
    const int L = min(max(a.c.len[b], 0), max_len);
    const int nk = min(a.c.n_kq[b], L), nv = min(a.c.n_vq[b], L);
    const int q_end = min(nk, nv) & ~31;
    const int tq = ((q_end + nq - 1) / nq + 31) & ~31;
    const int t_lo = min(q_end, split * tq), t_hi = min(q_end, (split + 1) * tq);
    const long row = long(b) * a.H + h;
    const long cb = row * a.cap;
    const int nch = (t_hi - t_lo) >> 5;
    const int nmine = wave < nch ? (nch - wave + kGqWaves - 1) / kGqWaves : 0;
    GqStage& st = lds.st[wave];

    // the lane's query pairs (head n, channels 32 kb + gq_kchan), zero for n >= nrep
    uint32_t qp[4][4];
    {
        uint32_t w[16];
        const uint4* src = reinterpret_cast<const uint4*>(
            q + ((long(b) * a.H + h) * a.nrep + min(n, a.nrep - 1)) * D + 32 * kb);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 v = src[i];
            w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int d = 0; d < 4; ++d)
                qp[kk][d] = n < a.nrep ? half_pair(w, gq_kchan<KB>(kk, d, 0), gq_kchan<KB>(kk, d, 1)) : 0u;
    }
    // staging positions of the lane's halves: key scale / zero channels 2 lane + e, value scale / zero of
    // token lane >> 1, groups 2 (lane & 1) + e
    int kpos[2], vpos[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int c = 2 * lane + e;
        kpos[e] = 32 * (c >> 5) + gq_kslot<KB>(c & 31);     // [kb][kk][d] pairs, half e
        vpos[e] = (2 * (lane & 1) + e) * 32 + gq_slot(lane >> 1);
    }

    struct Loads {
        uint32_t kc[2][KW];
        uint32_t sk, zk, sv, zv;
        uint32_t vc[VW];
    };
    // per-lane byte offsets from the key group's first token (the bases are wave-uniform)
    const int koff = n * KROW + 4 * KW * kb, voff = 4 * (lane >> 3) * VROW + 4 * (lane & 7);
    auto issue = [&](int k, Loads& ld) {
        const int t0 = __builtin_amdgcn_readfirstlane(t_lo + 32 * (wave + kGqWaves * min(k, nmine - 1)));
        const uint8_t* kg = a.c.k_codes + (cb + t0) * KROW;
        const uint8_t* vg = a.c.v_codes + (cb + t0) * VROW;
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            const uint8_t* kr = kg + 16 * T * KROW + koff;
            if constexpr (KB == 2) {
                const uint2 v = *reinterpret_cast<const uint2*>(kr);
                ld.kc[T][0] = v.x; ld.kc[T][1] = v.y;
            } else {
                const uint4 v = *reinterpret_cast<const uint4*>(kr);
                ld.kc[T][0] = v.x; ld.kc[T][1] = v.y; ld.kc[T][2] = v.z; ld.kc[T][3] = v.w;
            }
        }
        const long gidx = (row * (a.cap / 32) + t0 / 32) * D;
        ld.sk = reinterpret_cast<const uint32_t*>(U16(a.c.k_scale) + gidx)[lane];
        ld.zk = reinterpret_cast<const uint32_t*>(U16(a.c.k_zero) + gidx)[lane];
        ld.sv = reinterpret_cast<const uint32_t*>(U16(a.c.v_scale) + (cb + t0) * 4)[lane];
        ld.zv = reinterpret_cast<const uint32_t*>(U16(a.c.v_zero) + (cb + t0) * 4)[lane];
#pragma unroll
        for (int i = 0; i < VW; ++i)     // token 4 (lane >> 3) + (i & 3), dword (lane & 7) + 8 (i >> 2)
            ld.vc[i] = *reinterpret_cast<const uint32_t*>(vg + voff + (i & 3) * VROW + 32 * (i >> 2));
    };
    auto stage = [&](const Loads& ld) {
        uint16_t* skh = reinterpret_cast<uint16_t*>(st.skp);
        uint16_t* zkh = reinterpret_cast<uint16_t*>(st.zkp);
        uint16_t* svh = &st.sv[0][0];
        uint16_t* zvh = &st.zv[0][0];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            skh[kpos[e]] = uint16_t(ld.sk >> (16 * e));
            zkh[kpos[e]] = uint16_t(ld.zk >> (16 * e));
            svh[vpos[e]] = uint16_t(ld.sv >> (16 * e));
            zvh[vpos[e]] = uint16_t(ld.zv >> (16 * e));
        }
        const int q4 = lane >> 3, sb = 8 * (q4 & 3) + 4 * (q4 >> 2);
#pragma unroll
        for (int hh = 0; hh < VW / 4; ++hh) {
            const uint32_t x0 = ld.vc[4 * hh], x1 = ld.vc[4 * hh + 1], x2 = ld.vc[4 * hh + 2], x3 = ld.vc[4 * hh + 3];
            const uint32_t p01l = __builtin_amdgcn_perm(x1, x0, 0x05010400u), p01h = __builtin_amdgcn_perm(x1, x0, 0x07030602u);
            const uint32_t p23l = __builtin_amdgcn_perm(x3, x2, 0x05010400u), p23h = __builtin_amdgcn_perm(x3, x2, 0x07030602u);
            const uint32_t y[4] = {__builtin_amdgcn_perm(p23l, p01l, 0x05040100u), __builtin_amdgcn_perm(p23l, p01l, 0x07060302u),
                                   __builtin_amdgcn_perm(p23h, p01h, 0x05040100u), __builtin_amdgcn_perm(p23h, p01h, 0x07060302u)};
            const int d = (lane & 7) + 8 * hh;
#pragma unroll
            for (int e = 0; e < 4; ++e) *reinterpret_cast<uint32_t*>(&st.vt[(4 * d + e) * kVtStride + sb]) = y[e];
        }
        asm volatile("" ::: "memory");
    };

    const uint32_t vmask = n < 8 ? 0x03030303u : 0x0c0c0c0cu;     // 2-bit value codes: see the value tiles
    const float vscale = n < 8 ? 512.f : 128.f;
    float m = -INFINITY, l = 0.f, vbias[4] = {0.f, 0.f, 0.f, 0.f};
    kf4_t acc[4][2];
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[g][0] = acc[g][1] = kf4_t{0.f, 0.f, 0.f, 0.f};
    const kf4_t zero4 = kf4_t{0.f, 0.f, 0.f, 0.f};

    Loads cur, nxt;
    if (nmine > 0) issue(0, cur);
    for (int k = 0; k < nmine; ++k) {
        stage(cur);
        issue(k + 1, nxt);
        // scores: bias chain and the two token tiles
        kf4_t dz = zero4, dt[2] = {zero4, zero4};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const uint4 sp = *reinterpret_cast<const uint4*>(&st.skp[(kb * 4 + kk) * 4]);
            const uint4 zp = *reinterpret_cast<const uint4*>(&st.zkp[(kb * 4 + kk) * 4]);
            const uint32_t spw[4] = {sp.x, sp.y, sp.z, sp.w};
            uint32_t wh[4], wl[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const kh2_t qh = __builtin_bit_cast(kh2_t, qp[kk][d]), sh = __builtin_bit_cast(kh2_t, spw[d]);
                const kh2_t hi = qh * sh;
                wh[d] = __builtin_bit_cast(uint32_t, hi);
                wl[d] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(qh, sh, -hi));
            }
            const kh8_t W = __builtin_bit_cast(kh8_t, make_uint4(wh[0], wh[1], wh[2], wh[3]));
            const kh8_t Wl = __builtin_bit_cast(kh8_t, make_uint4(wl[0], wl[1], wl[2], wl[3]));
            dz = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(kh8_t, zp), Wl, dz, 0, 0, 0);
            dz = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(kh8_t, zp), W, dz, 0, 0, 0);
#pragma unroll
            for (int T = 0; T < 2; ++T) {
                uint32_t c[4];
                if constexpr (KB == 2) {
                    // byte d of y: channels 4 d + u' (low nibble) and 4 d + u' + 2 (high), u' = kk & 1
                    const uint32_t X = cur.kc[T][kk >> 1];
                    const uint32_t y = (kk & 1 ? X >> 2 : X) & 0x33333333u;
                    c[0] = nib_pair<0>(y); c[1] = nib_pair<1>(y); c[2] = nib_pair<2>(y); c[3] = nib_pair<3>(y);
                } else {
                    const uint32_t X = cur.kc[T][kk];
                    const uint32_t y0 = X & 0x0f0f0f0fu, y1 = (X >> 4) & 0x0f0f0f0fu;
                    c[0] = code_pair<0>(y0); c[1] = code_pair<1>(y0); c[2] = code_pair<0>(y1); c[3] = code_pair<1>(y1);
                }
                const kh8_t Ac = __builtin_bit_cast(kh8_t, make_uint4(c[0], c[1], c[2], c[3]));
                dt[T] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ac, Wl, dt[T], 0, 0, 0);
                dt[T] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ac, W, dt[T], 0, 0, 0);
            }
        }
        // online softmax (log2 units): lane (n, kb) holds tokens 4 kb + i (tile 0) and 16 + 4 kb + i (tile 1)
        float mx = fmax2(fmax2(fmax2(dt[0][0], dt[0][1]), dt[0][2]), fmax2(fmax2(dt[0][3], dt[1][0]), dt[1][1]));
        mx = fmax2(fmax2(mx, dt[1][2]), dt[1][3]);
        mx = rows4_reduce(mx, [](float x, float y) { return fmax2(x, y); });
        const float m_new = fmax2(m, scale_log2 * (mx - dz[0]));
        if (__builtin_amdgcn_ballot_w64(m_new > m)) {
            const float alpha = __builtin_amdgcn_exp2f(m - m_new);
            l *= alpha;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                vbias[g] *= alpha;
                acc[g][0] *= alpha;
                acc[g][1] *= alpha;
            }
            m = m_new;
        }
        const float cz = fmaf(scale_log2, dz[0], m);
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = __builtin_amdgcn_exp2f(fmaf(scale_log2, dt[i >> 2][i & 3], -cz));
            l += p[i];
        }
        uint32_t P[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const kh2_t v = {(_Float16)p[2 * d], (_Float16)p[2 * d + 1]};
            P[d] = __builtin_bit_cast(uint32_t, v);
        }
        // values
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint4 sv = *reinterpret_cast<const uint4*>(&st.sv[g][8 * kb]);
            const uint4 zv = *reinterpret_cast<const uint4*>(&st.zv[g][8 * kb]);
            const uint32_t svw[4] = {sv.x, sv.y, sv.z, sv.w}, zvw[4] = {zv.x, zv.y, zv.z, zv.w};
            uint32_t pg[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const kh2_t w = __builtin_bit_cast(kh2_t, P[d]) * __builtin_bit_cast(kh2_t, svw[d]);
                pg[d] = __builtin_bit_cast(uint32_t, w);
                vbias[g] = __builtin_amdgcn_fdot2(w, __builtin_bit_cast(kh2_t, zvw[d]), vbias[g], false);
            }
            const kh8_t Bg = __builtin_bit_cast(kh8_t, make_uint4(pg[0], pg[1], pg[2], pg[3]));
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                uint32_t y0, y1;
                float vsc = 512.f;
                if constexpr (VB == 2) {
                    // channel u = 2 pp + (n >> 3) of the byte: bits 2 u; u odd is masked in place (byte values
                    // 0, 4, 8, 12, converted with a quarter of the scale)
                    const uint2 Y = *reinterpret_cast<const uint2*>(&st.vt[(8 * g + (n & 7)) * kVtStride + 8 * kb]);
                    const uint32_t x0 = pp ? Y.x >> 4 : Y.x, x1 = pp ? Y.y >> 4 : Y.y;
                    y0 = x0 & vmask; y1 = x1 & vmask;
                    vsc = vscale;
                } else {
                    const uint2 Y = *reinterpret_cast<const uint2*>(&st.vt[(16 * g + 8 * pp + (n & 7)) * kVtStride + 8 * kb]);
                    const int sh = 4 * (n >> 3);
                    y0 = (Y.x >> sh) & 0x0f0f0f0fu; y1 = (Y.y >> sh) & 0x0f0f0f0fu;
                }
                const uint4 A = make_uint4(code_pair<0>(y0, vsc), code_pair<1>(y0, vsc), code_pair<0>(y1, vsc),
                                           code_pair<1>(y1, vsc));
                acc[g][pp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(kh8_t, A), Bg, acc[g][pp], 0, 0, 0);
            }
        }
        cur = nxt;
    }

    // ---- combine the waves: lane (n, kb) holds channels gq_vchan(g, p, 4 kb + i) of head n ----
    l = rows4_reduce(l, [](float x, float y) { return x + y; });
#pragma unroll
    for (int g = 0; g < 4; ++g) vbias[g] = rows4_reduce(vbias[g], [](float x, float y) { return x + y; });
    __syncthreads();                                  // every wave is done with its staging area
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
            for (int i = 0; i < 4; ++i) lds.cmb[wave][n][gq_vchan<VB>(g, pp, 4 * kb + i)] = acc[g][pp][i] - vbias[g];
    if (kb == 0) {
        lds.cmb[wave][n][D] = m;
        lds.cmb[wave][n][D + 1] = l;
    }
    __syncthreads();
    for (int e = tid; e < a.nrep * D; e += 256) {
        const int hn = e / D, d = e % D;
        const long orow = (row * a.nrep + hn) * S_tot + split;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kGqWaves; ++w) M = fmaxf(M, lds.cmb[w][hn][D]);
        if (M == -INFINITY) {
            po[orow * D + d] = 0.f;
            if (d == 0) pl[orow] = -INFINITY;
            continue;
        }
        float Ls = 0.f, ov = 0.f;
#pragma unroll
        for (int w = 0; w < kGqWaves; ++w) {
            const float mw = lds.cmb[w][hn][D];
            const float fw = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
            Ls += lds.cmb[w][hn][D + 1] * fw;
            ov += lds.cmb[w][hn][d] * fw;
        }
        po[orow * D + d] = ov / Ls;
        if (d == 0) pl[orow] = (M + log2f(Ls)) * kLn2;
    }
}

// One wave per output row (request, query head), the row's 128 channels two per lane.  Up to 16 splits
// every load of the row is issued at once (the splits' lse are the same for all lanes: scalar loads, the
// maximum and the sum taken in every lane); more splits, the lse spread over the lanes for the maximum and
// the sum, then the partial rows.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}
constexpr int kMergeRegs = 16;
__global__ void __launch_bounds__(256) kivi_merge_kernel(const float* __restrict__ po, const float* __restrict__ pl,
                                                         int n_rows, int S, float* __restrict__ out,
                                                         float* __restrict__ lse_out) {
    constexpr int D = kKiviD;
    const int lane = threadIdx.x & 63;
    const long n = long(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (n >= n_rows) return;
    const float* lr = pl + n * S;
    const float2* pp = reinterpret_cast<const float2*>(po + n * S * D) + lane;
    float2 o = make_float2(0.f, 0.f);
    float lse;
    if (S <= kMergeRegs) {
        float ls[kMergeRegs];
        float2 v[kMergeRegs];
#pragma unroll
        for (int s = 0; s < kMergeRegs; ++s) {
            ls[s] = s < S ? lr[s] : -INFINITY;
            v[s] = s < S ? pp[long(s) * (D / 2)] : make_float2(0.f, 0.f);
        }
        float M = -INFINITY;
#pragma unroll
        for (int s = 0; s < kMergeRegs; ++s) M = fmaxf(M, ls[s]);
        float L = 0.f;
#pragma unroll
        for (int s = 0; s < kMergeRegs; ++s) L += (ls[s] == -INFINITY) ? 0.f : __expf(ls[s] - M);
        lse = (M == -INFINITY) ? -INFINITY : M + __logf(L);
        if (M != -INFINITY) {
#pragma unroll
            for (int s = 0; s < kMergeRegs; ++s) {
                const float w = ls[s] == -INFINITY ? 0.f : __expf(ls[s] - lse);
                o.x += w * v[s].x;
                o.y += w * v[s].y;
            }
        }
    } else {
        float M = -INFINITY;
        for (int s = lane; s < S; s += 64) M = fmaxf(M, lr[s]);
        M = wave_max(M);
        float L = 0.f;
        if (M != -INFINITY)
            for (int s = lane; s < S; s += 64) L += (lr[s] == -INFINITY) ? 0.f : __expf(lr[s] - M);
        L = wave_sum(L);
        lse = (M == -INFINITY) ? -INFINITY : M + __logf(L);
        if (M != -INFINITY) {
#pragma unroll 4
            for (int s = 0; s < S; ++s) {
                const float ls = lr[s];
                const float2 v = pp[long(s) * (D / 2)];
                const float w = ls == -INFINITY ? 0.f : __expf(ls - lse);
                o.x += w * v.x;
                o.y += w * v.y;
            }
        }
    }
    reinterpret_cast<float2*>(out + n * D)[lane] = o;
    if (lse_out && lane == 0) lse_out[n] = lse;
}

lvq_status validate_kivi(const kivi_geom* g, const kivi_cache* c) {
    LVQ_REQUIRE(g && c, LVQ_ERR_INVALID_ARG, "kivi: NULL geometry or cache");
    LVQ_REQUIRE(g->D == 128, LVQ_ERR_UNSUPPORTED, "kivi: head dimension %d unsupported (128)", g->D);
    LVQ_REQUIRE(g->bits == 2 || g->bits == 4, LVQ_ERR_UNSUPPORTED, "kivi: %d-bit key codes unsupported (2, 4)",
                g->bits);
    LVQ_REQUIRE(g->v_bits == 0 || g->v_bits == 2 || g->v_bits == 4, LVQ_ERR_UNSUPPORTED,
                "kivi: %d-bit value codes unsupported (0 = as keys, 2, 4)", g->v_bits);
    LVQ_REQUIRE(g->group == 32, LVQ_ERR_UNSUPPORTED, "kivi: group %d unsupported (32)", g->group);
    LVQ_REQUIRE(g->H > 0 && g->R > 0 && g->R % g->group == 0, LVQ_ERR_INVALID_ARG,
                "kivi: R=%d must be a positive multiple of the group", g->R);
    LVQ_REQUIRE(g->Hq >= 0 && (g->Hq == 0 || (g->Hq % g->H == 0 && kKiviLaneGroups % (g->Hq / g->H) == 0)),
                LVQ_ERR_UNSUPPORTED, "kivi: %d query heads over %d KV heads (a multiple, at most 32 per KV head, "
                "dividing 32)", g->Hq, g->H);
    LVQ_REQUIRE(g->cap > 0 && g->cap % g->group == 0, LVQ_ERR_INVALID_ARG,
                "kivi: capacity %d must be a positive multiple of the group", g->cap);
    LVQ_REQUIRE(c->k_codes && c->k_scale && c->k_zero && c->v_codes && c->v_scale && c->v_zero && c->k_res &&
                    c->v_res && c->len && c->n_kq && c->n_vq,
                LVQ_ERR_INVALID_ARG, "kivi: NULL cache pointer");
    return LVQ_OK;
}

// query heads per KV head
int kivi_nrep(const kivi_geom* g) { return g->Hq ? g->Hq / g->H : 1; }

KArgs make_args(const kivi_geom* g, const kivi_cache* c) {
    KArgs a;
    a.D = g->D; a.H = g->H; a.G = g->group; a.R = g->R; a.cap = g->cap; a.ring = g->R + g->group;
    a.kb = g->bits;
    a.vb = g->v_bits ? g->v_bits : g->bits;
    a.nrep = kivi_nrep(g);
    a.c = *c;
    return a;
}

// up to 16 query heads per KV head take the matrix-core kernel (one MFMA column tile of heads), 32 the
// per-token kernel
bool kivi_use_mfma(const KArgs& a) { return a.nrep <= 16; }

template <int KB, int VB>
void launch_kivi_attn(dim3 grid, hipStream_t stream, const KArgs& a, const uint16_t* q, float sl2, int S_tot,
                      int max_len, float* po, float* pl) {
    if (kivi_use_mfma(a))
        hipLaunchKernelGGL((kivi_attn_mfma_kernel<KB, VB>), grid, dim3(256), 0, stream, a, q, sl2, S_tot, max_len, po, pl);
    else   // 32 query heads per KV head: two per lane group
        hipLaunchKernelGGL((kivi_attn_partial_kernel<KB, VB, 2>), grid, dim3(256), 0, stream, a, q, sl2, S_tot, max_len, po, pl);
}

int choose_kivi_splits(const kivi_geom* g, int B, int max_len) {
    const int wgs = B * g->H;
    int s = ceil_div(1024, std::max(1, wgs));
    // About 1024 workgroups, splits of at most 2048 tokens (measured with the matrix-core kernel on the 4K
    // batch-16 workloads: 2-bit, 32 KV heads: 1 split 75.4 us, 2 59.5, 4 59.9; 32 query heads over 8 KV
    // heads: 4 splits 24.3, 8 24.5).
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
        // One pass when every row starts on a 16-byte boundary (the usual contiguous layouts).
        const bool aligned = reinterpret_cast<uintptr_t>(k_new) % 16 == 0 &&
                             reinterpret_cast<uintptr_t>(v_new) % 16 == 0 && new_strides[0] % 8 == 0 &&
                             new_strides[1] % 8 == 0 && new_strides[2] % 8 == 0;
        if (aligned) {
            const dim3 grid(ceil_div(n_new, 128), g->H, B);
            if (a.kb == 2 && a.vb == 2)
                hipLaunchKernelGGL((prefill_kv_kernel<2, 2>), grid, dim3(256), 0, stream, a, ks, vs, n_new, n_kq, n_vq);
            else if (a.kb == 2)
                hipLaunchKernelGGL((prefill_kv_kernel<2, 4>), grid, dim3(256), 0, stream, a, ks, vs, n_new, n_kq, n_vq);
            else if (a.vb == 2)
                hipLaunchKernelGGL((prefill_kv_kernel<4, 2>), grid, dim3(256), 0, stream, a, ks, vs, n_new, n_kq, n_vq);
            else
                hipLaunchKernelGGL((prefill_kv_kernel<4, 4>), grid, dim3(256), 0, stream, a, ks, vs, n_new, n_kq, n_vq);
            return check_launch("kivi_append: prefill");
        }
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
    if (g->Hq < 0 || (g->Hq && g->Hq % g->H)) return 0;
    // the splits and one slot of its own for the rows past the whole key groups
    const int S = (num_splits > 0 ? num_splits : choose_kivi_splits(g, B, max_len)) + 1;
    const size_t rows = size_t(B) * (g->Hq ? g->Hq : g->H) * S;     // (request, query head, split)
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
    const int Hq = g->H * a.nrep;
    const int S_tot = S + 1;                                      // + the residual slot
    const size_t rows = size_t(B) * Hq * S_tot;
    float* po = static_cast<float*>(ws);
    float* pl = po + rows * g->D;
    const dim3 grid(S_tot, g->H, B);
    const auto* qp = static_cast<const uint16_t*>(q);
    const float sl2 = sm_scale * kLog2e;
    if (a.kb == 2 && a.vb == 2) launch_kivi_attn<2, 2>(grid, stream, a, qp, sl2, S_tot, max_len, po, pl);
    else if (a.kb == 2) launch_kivi_attn<2, 4>(grid, stream, a, qp, sl2, S_tot, max_len, po, pl);
    else if (a.vb == 2) launch_kivi_attn<4, 2>(grid, stream, a, qp, sl2, S_tot, max_len, po, pl);
    else launch_kivi_attn<4, 4>(grid, stream, a, qp, sl2, S_tot, max_len, po, pl);
    if ((st = check_launch("kivi_decode_attn: partial")) != LVQ_OK) return st;
    hipLaunchKernelGGL(kivi_merge_kernel, dim3(ceil_div(B * Hq, 4)), dim3(256), 0, stream, po, pl, B * Hq, S_tot, out,
                       lse_out);
    return check_launch("kivi_decode_attn: merge");
}
