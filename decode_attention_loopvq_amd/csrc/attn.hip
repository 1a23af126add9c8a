// LoopVQ decode attention: quantized-page partials, bf16-window partial and
// the exact logsumexp merge.
//
// LoopVQ page ("LoopVQ: Sub 1-bit KV Cache Quantization for Looped
// Transformers"): "method steps" step 5 and Figure 5 (load the step's slice
// B_t once, rebuild K/V from indices, RoPE, score; index pages and bf16 pages
// attended by two kernels, partials merged through logsumexp; two requests
// share one workgroup and with it the B_t and RoPE-table loads); background
// "SGLang and Flash-Decoding" (split-K partial softmax, exact merge).
#include "common.h"

#include <algorithm>

namespace lvq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
    Geo geo;
    int step, beta;
    const uint16_t* q;          // [B][H][D] bf16
    const uint8_t* pool;
    const int32_t* pt;
    int pt_stride;
    const int32_t* seq_len;
    const uint16_t* wk;         // [B][T][H][Wcap][D] bf16
    const uint16_t* wv;
    const void* slice_k;        // this step's K slice [NG][K][c]
    const void* slice_v;        // this step's V slice; the slices of (step, head h) are at +h*hstride
    long slice_hstride;         // elements between heads
    const float* rc;            // [rope_len][D/2]
    const float* rs;
    float scale_log2;           // sm_scale * log2(e)
    float* part_o;              // [B*H][S_tot][D]
    float* part_lse;            // [B*H][S_tot]
    int S_tot;                  // num_splits + 1 (the last slot is the window partial)
    int num_splits;
    int pps;                    // index pages per split
    int B;
    int max_len;                // device lengths are clamped to this
    int rope_len;
    const uint32_t* qpack;      // [B*H][128]: (q_i, q_{i+64}) then (q_{i+64}, -q_i) as bf16 pairs
    int fix_bits;               // fixed-point bits of the softmax weights in the V bins
};

__device__ __forceinline__ int clamp_len(const AttnArgs& a, int rb) {
    const int L = a.seq_len[rb];
    return L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
}

__device__ __forceinline__ int n_index_pages(int L, const Geo& g) {
    const int r = L - g.sink - g.W;
    return r > 0 ? r / g.page : 0;
}

// Load C codeword coordinates as floats.
template <int C>
__device__ __forceinline__ void load_cw(const uint16_t* p, float* out) {   // bf16
    if constexpr (C == 8) {
        const uint4 w = *reinterpret_cast<const uint4*>(p);
        out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x); out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
        out[4] = bf16_lo(w.z); out[5] = bf16_hi(w.z); out[6] = bf16_lo(w.w); out[7] = bf16_hi(w.w);
    } else {
        const uint2 w = *reinterpret_cast<const uint2*>(p);
        out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x); out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
    }
}
template <int C>
__device__ __forceinline__ void load_cw(const float* p, float* out) {      // fp32
    if constexpr (C == 8) {
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    } else {
        const float4 a = *reinterpret_cast<const float4*>(p);
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    }
}

// The index bytes of GPC consecutive groups starting at byte offset `off`.
template <int GPC>
__device__ __forceinline__ uint64_t load_idx(const uint8_t* row, int off) {
    if constexpr (GPC == 4) return *reinterpret_cast<const uint32_t*>(row + off);
    else return *reinterpret_cast<const uint64_t*>(row + off);
}

// ---------------------------------------------------------------------------
// Quantized-page partial.
//
// Grid (split, head, request pair); 256 threads.  The step's K and V slices
// of head h are staged in LDS once (bf16) and serve both requests.  Two
// lanes of one wave share a token: lane half 0 owns RoPE pairs [0,32)
// (channels 0..31 and 64..95), half 1 pairs [32,64); the two partial scores
// are added across the halves.  Each lane pair keeps an online softmax over
// its tokens; the 128 pairs are folded at the end (shuffles within the wave,
// LDS across the four waves).
// ---------------------------------------------------------------------------
template <int C, typename E, bool kLdsCb>
__global__ void __launch_bounds__(256) quant_partial_kernel(AttnArgs a) {
    constexpr int D = 128;
    constexpr int GPC = 32 / C;          // groups per 32-channel chunk
    const Geo& g = a.geo;
    const int NG = D / C;
    const int K = 256;
    const int split = blockIdx.x, h = blockIdx.y;
    const int r0 = 2 * blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5;
    const int slot = wave * 32 + (lane & 31);

    // Page ranges of the two requests; leave early when both are empty.
    int plo[2], phi[2];
    bool any = false;
    for (int j = 0; j < 2; ++j) {
        const int rb = r0 + j;
        plo[j] = phi[j] = 0;
        if (rb < a.B) {
            const int np = n_index_pages(clamp_len(a, rb), g);
            plo[j] = min(np, split * a.pps);
            phi[j] = min(np, (split + 1) * a.pps);
            any |= phi[j] > plo[j];
        }
    }
    if (!any) {
        for (int j = 0; j < 2; ++j) {
            const int rb = r0 + j;
            if (rb >= a.B) continue;
            const long row = (long(rb) * g.H + h) * a.S_tot + split;
            if (tid < D) a.part_o[row * D + tid] = 0.f;
            if (tid == 0) a.part_lse[row] = -INFINITY;
        }
        return;
    }

    extern __shared__ __align__(16) unsigned char smem[];
    const E* gk = static_cast<const E*>(a.slice_k) + h * a.slice_hstride;
    const E* gv = static_cast<const E*>(a.slice_v) + h * a.slice_hstride;
    const E* cbk;
    const E* cbv;
    float* red = nullptr;
    if constexpr (kLdsCb) {
        E* sk = reinterpret_cast<E*>(smem);
        E* sv = sk + K * D;
        const int n16 = K * D * int(sizeof(E)) / 16;
        const uint4* srck = reinterpret_cast<const uint4*>(gk);
        const uint4* srcv = reinterpret_cast<const uint4*>(gv);
        uint4* dk = reinterpret_cast<uint4*>(sk);
        uint4* dv = reinterpret_cast<uint4*>(sv);
        for (int e = tid; e < n16; e += 256) {
            dk[e] = srck[e];
            dv[e] = srcv[e];
        }
        cbk = sk;
        cbv = sv;
        red = reinterpret_cast<float*>(smem + 2 * K * D * sizeof(E));
        __syncthreads();
    } else {
        cbk = gk;
        cbv = gv;
        red = reinterpret_cast<float*>(smem);
    }

    const int chA = 32 * half, chB = 64 + 32 * half;     // first channel of each chunk
    const int gA = chA / C, gB = chB / C;                // first group of each chunk

    for (int j = 0; j < 2; ++j) {
        const int rb = r0 + j;
        if (rb >= a.B) break;
        const long orow = (long(rb) * g.H + h) * a.S_tot + split;
        if (phi[j] <= plo[j]) {
            if (tid < D) a.part_o[orow * D + tid] = 0.f;
            if (tid == 0) a.part_lse[orow] = -INFINITY;
            continue;
        }
        float qA[32], qB[32];
        const uint16_t* qp = a.q + (long(rb) * g.H + h) * D;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            qA[i] = bf16_to_f32(qp[chA + i]);
            qB[i] = bf16_to_f32(qp[chB + i]);
        }
        float m = -INFINITY, l = 0.f;
        float oA[32], oB[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) { oA[i] = 0.f; oB[i] = 0.f; }

        const int tok_lo = plo[j] * g.page, tok_hi = phi[j] * g.page;
        const int32_t* ptr = a.pt + long(rb) * a.pt_stride;
        for (int tok = tok_lo + slot; tok < tok_hi; tok += 128) {
            const int p = g.sink + tok;
            const long phys = ptr[tok >> 3];
            const uint8_t* krow = a.pool + phys * g.page_bytes + (long(a.beta) * g.H + h) * 2 * 8 * NG + (tok & 7) * NG;
            const uint8_t* vrow = krow + 8 * NG;
            const uint64_t ikA = load_idx<GPC>(krow, gA), ikB = load_idx<GPC>(krow, gB);
            const uint64_t ivA = load_idx<GPC>(vrow, gA), ivB = load_idx<GPC>(vrow, gB);
            float kA[32], kB[32];
#pragma unroll
            for (int q = 0; q < GPC; ++q) {
                const int ia = int((ikA >> (8 * q)) & 0xff), ib = int((ikB >> (8 * q)) & 0xff);
                load_cw<C>(cbk + ((gA + q) * K + ia) * C, kA + q * C);
                load_cw<C>(cbk + ((gB + q) * K + ib) * C, kB + q * C);
            }
            const float* cp = a.rc + long(p) * (D / 2) + chA;
            const float* sp = a.rs + long(p) * (D / 2) + chA;
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < 32; i += 4) {
                const float4 c4 = *reinterpret_cast<const float4*>(cp + i);
                const float4 s4 = *reinterpret_cast<const float4*>(sp + i);
                const float cs[4] = {c4.x, c4.y, c4.z, c4.w};
                const float sn[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float x1 = kA[i + u], x2 = kB[i + u];
                    const float r1 = x1 * cs[u] - x2 * sn[u];
                    const float r2 = x2 * cs[u] + x1 * sn[u];
                    part += qA[i + u] * r1 + qB[i + u] * r2;
                }
            }
            const float s = (part + __shfl_xor(part, 32, 64)) * a.scale_log2;
            float vA[32], vB[32];
#pragma unroll
            for (int q = 0; q < GPC; ++q) {
                const int ia = int((ivA >> (8 * q)) & 0xff), ib = int((ivB >> (8 * q)) & 0xff);
                load_cw<C>(cbv + ((gA + q) * K + ia) * C, vA + q * C);
                load_cw<C>(cbv + ((gB + q) * K + ib) * C, vB + q * C);
            }
            const float m_new = fmaxf(m, s);
            const float alpha = exp2f(m - m_new);
            const float w = exp2f(s - m_new);
            l = l * alpha + w;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                oA[i] = oA[i] * alpha + w * vA[i];
                oB[i] = oB[i] * alpha + w * vB[i];
            }
            m = m_new;
        }

        // Fold the 32 lane pairs of this wave (xor offsets below 32 stay in a half).
        float mw = m;
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) mw = fmaxf(mw, __shfl_xor(mw, off, 64));
        const float f = (m == -INFINITY) ? 0.f : exp2f(m - mw);
        float lw = l * f;
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) lw += __shfl_xor(lw, off, 64);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            float x = oA[i] * f, y = oB[i] * f;
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) {
                x += __shfl_xor(x, off, 64);
                y += __shfl_xor(y, off, 64);
            }
            oA[i] = x;
            oB[i] = y;
        }
        // red layout: [4 waves][D + 2]
        float* rw = red + wave * (D + 2);
        if ((lane & 31) == 0) {
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                rw[chA + i] = oA[i];
                rw[chB + i] = oB[i];
            }
            if (half == 0) {
                rw[D] = mw;
                rw[D + 1] = lw;
            }
        }
        __syncthreads();
        if (tid < D) {
            float M = -INFINITY;
            for (int w2 = 0; w2 < 4; ++w2) M = fmaxf(M, red[w2 * (D + 2) + D]);
            float L = 0.f, o = 0.f;
            for (int w2 = 0; w2 < 4; ++w2) {
                const float mw2 = red[w2 * (D + 2) + D];
                const float fw = (mw2 == -INFINITY) ? 0.f : exp2f(mw2 - M);
                L += red[w2 * (D + 2) + D + 1] * fw;
                o += red[w2 * (D + 2) + tid] * fw;
            }
            a.part_o[orow * D + tid] = o / L;
            if (tid == 0) a.part_lse[orow] = (M + log2f(L)) * kLn2;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Query pairs for the packed dot products: row r of qpack holds, for RoPE
// pair i (channel i with channel i + 64), the bf16 pair (q_i, q_{i+64}) at
// [i] and (q_{i+64}, -q_i) at [64 + i].  With k-pair (k_i, k_{i+64}):
//   dot2(k, qpack[i])      = q_i k_i + q_{i+64} k_{i+64}        (= A_i)
//   dot2(k, qpack[64 + i]) = q_{i+64} k_i - q_i k_{i+64}        (= B_i)
// and q . RoPE_p(k) = sum_i cos(p th_i) A_i + sin(p th_i) B_i.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void pack_q_row(const uint16_t* q, uint32_t* out, int i) {
    const uint32_t lo = q[i], hi = q[i + 64];
    out[i] = lo | (hi << 16);
    out[64 + i] = hi | ((lo ^ 0x8000u) << 16);
}

__global__ void pack_q_kernel(const uint16_t* __restrict__ q, uint32_t* __restrict__ qpack) {
    const long row = blockIdx.x;
    pack_q_row(q + row * 128, qpack + row * 128, threadIdx.x);
}

typedef short bf16x2_t __attribute__((ext_vector_type(2)));

// Read-only data that the kernel reads at wave-uniform addresses: through the
// constant address space the compiler turns such reads into scalar loads.
template <typename T>
using const_ptr = const __attribute__((address_space(4))) T*;
template <typename T>
__device__ __forceinline__ const_ptr<T> as_const(const T* p) {
    return reinterpret_cast<const_ptr<T>>(reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

// Two RoPE pairs of one token: acc += cos0 A0 + sin0 B0 + cos1 A1 + sin1 B1, with
// (k_i, k_{i+64}) taken from the low (pair 0) and high (pair 1) bf16 halves of
// kl / kh.  One block so that the packed dot products use the three-operand
// form with a zero accumulator (no register to clear) and every dot result is
// read at least three instructions after it is written, as gfx950 requires
// after a DOT instruction.
__device__ __forceinline__ float two_pairs(float acc, uint32_t kl, uint32_t kh, uint32_t q0a, uint32_t q0b,
                                           uint32_t q1a, uint32_t q1b, float c0, float s0, float c1, float s1) {
    uint32_t kp0, kp1;
    float a0, b0, a1, b1;
    asm("v_perm_b32 %[kp0], %[kh], %[kl], %[sl]\n\t"
        "v_perm_b32 %[kp1], %[kh], %[kl], %[sh]\n\t"
        "v_dot2_f32_bf16 %[a0], %[kp0], %[q0a], 0\n\t"
        "v_dot2_f32_bf16 %[b0], %[kp0], %[q0b], 0\n\t"
        "v_dot2_f32_bf16 %[a1], %[kp1], %[q1a], 0\n\t"
        "v_dot2_f32_bf16 %[b1], %[kp1], %[q1b], 0\n\t"
        "v_fmac_f32 %[acc], %[c0], %[a0]\n\t"
        "v_fmac_f32 %[acc], %[s0], %[b0]\n\t"
        "v_fmac_f32 %[acc], %[c1], %[a1]\n\t"
        "v_fmac_f32 %[acc], %[s1], %[b1]"
        : [acc] "+v"(acc), [kp0] "=&v"(kp0), [kp1] "=&v"(kp1), [a0] "=&v"(a0), [b0] "=&v"(b0), [a1] "=&v"(a1),
          [b1] "=&v"(b1)
        : [kl] "v"(kl), [kh] "v"(kh), [q0a] "s"(q0a), [q0b] "s"(q0b), [q1a] "s"(q1a), [q1b] "s"(q1b),
          [c0] "v"(c0), [s0] "v"(s0), [c1] "v"(c1), [s1] "v"(s1), [sl] "s"(0x05040100u), [sh] "s"(0x07060302u));
    return acc;
}

// (k_i, k_{i+64}) from the dwords holding k_i (group g) and k_{i+64} (group g + NG/2).
__device__ __forceinline__ uint32_t kpair(uint32_t lo_dw, uint32_t hi_dw, int half) {
    return __builtin_amdgcn_perm(hi_dw, lo_dw, half ? 0x07060302u : 0x05040100u);
}

constexpr int kSeg = 2048;       // tokens per request per scoring segment
constexpr int kThreadsV2 = 512;  // 8 waves: two per SIMD
constexpr int kBinPad = 264;     // padded bin row (256 codewords) to spread LDS banks

// Score contribution of pair chunk `ch` (pairs 8ch .. 8ch+7) for one request.
template <int C>
__device__ __forceinline__ float chunk_score(int ch, const uint32_t* ik, const uint16_t* cb,
                                             const_ptr<uint32_t> qp, const float* cs, const float* sn,
                                             float acc) {
    constexpr int K = 256, NG = 128 / C, HALF = NG / 2;
    uint32_t kl[4], kh[4];   // 8 bf16 of channels 8ch.. (kl) and 64+8ch.. (kh)
    if constexpr (C == 8) {
        const int al = (ik[ch >> 2] >> (8 * (ch & 3))) & 0xff;
        const int ah = (ik[2 + (ch >> 2)] >> (8 * (ch & 3))) & 0xff;
        const uint4 vl = *reinterpret_cast<const uint4*>(cb + (ch * K + al) * 8);
        const uint4 vh = *reinterpret_cast<const uint4*>(cb + ((ch + HALF) * K + ah) * 8);
        kl[0] = vl.x; kl[1] = vl.y; kl[2] = vl.z; kl[3] = vl.w;
        kh[0] = vh.x; kh[1] = vh.y; kh[2] = vh.z; kh[3] = vh.w;
    } else {
        const uint32_t wl = ik[ch >> 1] >> (16 * (ch & 1));
        const uint32_t wh = ik[4 + (ch >> 1)] >> (16 * (ch & 1));
        const int g0 = 2 * ch;
        const uint2 l0 = *reinterpret_cast<const uint2*>(cb + (g0 * K + (wl & 0xff)) * 4);
        const uint2 l1 = *reinterpret_cast<const uint2*>(cb + ((g0 + 1) * K + ((wl >> 8) & 0xff)) * 4);
        const uint2 h0 = *reinterpret_cast<const uint2*>(cb + ((g0 + HALF) * K + (wh & 0xff)) * 4);
        const uint2 h1 = *reinterpret_cast<const uint2*>(cb + ((g0 + 1 + HALF) * K + ((wh >> 8) & 0xff)) * 4);
        kl[0] = l0.x; kl[1] = l0.y; kl[2] = l1.x; kl[3] = l1.y;
        kh[0] = h0.x; kh[1] = h0.y; kh[2] = h1.x; kh[3] = h1.y;
    }
#pragma unroll
    for (int u = 0; u < 8; u += 2)
        acc = two_pairs(acc, kl[u >> 1], kh[u >> 1], qp[8 * ch + u], qp[64 + 8 * ch + u], qp[8 * ch + u + 1],
                        qp[64 + 8 * ch + u + 1], cs[u], sn[u], cs[u + 1], sn[u + 1]);
    return acc;
}

// ---------------------------------------------------------------------------
// Index-page partial, bf16 codebooks.
//
// Grid (split, head, request pair); 256 threads; one workgroup per CU
// (~150 KB of LDS).  B_t^K of head h is staged in LDS and serves both
// requests.  Each split is scored in segments of up to 2048 tokens per
// request:
//   1. lane = position: a lane rebuilds the key of its position for both
//      requests (16 codeword gathers each), forms the exact RoPE score
//      sum_i cos A_i + sin B_i with packed bf16 dot products, and keeps it in
//      LDS.  cos/sin(p th_i) is formed once per position for both requests as
//      cos(P th)cos(l th) - sin(P th)sin(l th) from the table rows of the
//      wave's base position P (uniform, scalar loads) and of the lane offset
//      l (held in registers).
//   2. block max per request; bins are rescaled if the max grew.
//   3. each token adds its weight exp(s - max) in fixed point to one bin per
//      (group, codeword) of its V indices (integer LDS atomics).
// At the end B_t^V replaces B_t^K in LDS and o = sum_r bin[g][r] B_t^V[g][r]
// gives the partial output; l is the bin total of any one group.
// ---------------------------------------------------------------------------
template <int C>
__global__ void __launch_bounds__(kThreadsV2, 1) quant_v2_kernel(AttnArgs a) {
    constexpr int D = 128, K = 256, NG = D / C, IW = NG / 4;
    const Geo& g = a.geo;
    const int split = blockIdx.x, h = blockIdx.y;
    const int r0 = 2 * blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    int lo[2], hi[2];
    bool any = false;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        lo[j] = hi[j] = 0;
        const int rb = r0 + j;
        if (rb < a.B) {
            const int np = n_index_pages(clamp_len(a, rb), g);
            lo[j] = min(np, split * a.pps) * g.page;
            hi[j] = min(np, (split + 1) * a.pps) * g.page;
            any |= hi[j] > lo[j];
        }
    }
    if (!any) {
        for (int j = 0; j < 2; ++j) {
            const int rb = r0 + j;
            if (rb >= a.B) continue;
            const long row = (long(rb) * g.H + h) * a.S_tot + split;
            if (tid < D) a.part_o[row * D + tid] = 0.f;
            if (tid == 0) a.part_lse[row] = -INFINITY;
        }
        return;
    }

    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* cb = reinterpret_cast<uint16_t*>(smem);                           // 66 KB: B_t^K, later B_t^V
    constexpr int kCbBytes = NG * (K * C + 8) * 2;                               // padded rows for the final pass
    uint32_t* bins = reinterpret_cast<uint32_t*>(smem + kCbBytes);               // [2][NG][kBinPad]
    float* sc = reinterpret_cast<float*>(bins + 2 * NG * kBinPad);              // [2][kSeg]
    float* red = sc + 2 * kSeg;                                                  // [2][8] max + [2][8] sums
    int32_t* spt = reinterpret_cast<int32_t*>(red + 32);                         // [2][kSeg/8] page ids

    {   // stage B_t^K (unpadded rows), clear the bins
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.slice_k) +
                                                          h * a.slice_hstride);
        uint4* dst = reinterpret_cast<uint4*>(cb);
        for (int e = tid; e < K * D * 2 / 16; e += kThreadsV2) dst[e] = src[e];
        for (int e = tid; e < 2 * NG * kBinPad; e += kThreadsV2) bins[e] = 0u;
    }

    // cos/sin of the lane offset, all 64 pairs
    float cl[64], sl[64];
    {
        const int row = min(lane, a.rope_len - 1);
        const float4* c4 = reinterpret_cast<const float4*>(a.rc + long(row) * 64);
        const float4* s4 = reinterpret_cast<const float4*>(a.rs + long(row) * 64);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float4 c = c4[i], s_ = s4[i];
            cl[4 * i] = c.x; cl[4 * i + 1] = c.y; cl[4 * i + 2] = c.z; cl[4 * i + 3] = c.w;
            sl[4 * i] = s_.x; sl[4 * i + 1] = s_.y; sl[4 * i + 2] = s_.z; sl[4 * i + 3] = s_.w;
        }
    }
    const_ptr<uint32_t> qp[2];
    const int32_t* ptr[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int rb = min(r0 + j, a.B - 1);
        qp[j] = as_const(a.qpack + (long(rb) * g.H + h) * 128);
        ptr[j] = a.pt + long(rb) * a.pt_stride;
    }
    const long kv_off = (long(a.beta) * g.H + h) * 2 * 8 * NG;   // (block, head) slab inside a page
    const float fix_scale = float(1u << a.fix_bits);
    __syncthreads();

    float M[2] = {-INFINITY, -INFINITY};
    uint32_t lsum[2] = {0u, 0u};
    const int t_lo = min(hi[0] > lo[0] ? lo[0] : 0x7fffffff, hi[1] > lo[1] ? lo[1] : 0x7fffffff);
    const int t_hi = max(hi[0] > lo[0] ? hi[0] : 0, hi[1] > lo[1] ? hi[1] : 0);

    for (int s0 = t_lo; s0 < t_hi; s0 += kSeg) {
        const int s1 = min(t_hi, s0 + kSeg);
        float mloc[2] = {-INFINITY, -INFINITY};
        // page ids of this segment's pages, both requests
        for (int e = tid; e < 2 * (kSeg / 8); e += kThreadsV2) {
            const int jj = e / (kSeg / 8), lp = (s0 >> 3) + e % (kSeg / 8);
            spt[e] = (lp >= (lo[jj] >> 3) && lp < (hi[jj] >> 3)) ? ptr[jj][lp] : 0;
        }
        __syncthreads();
        // ---- phase 1: scores ----
        // Index rows of the next iteration are fetched while this one is scored.
        uint32_t ik[2][IW], nk[2][IW];
        auto fetch_k = [&](int base_, uint32_t (*dst)[IW]) {
            // Branch-free: lanes outside a request's range read page 0 (always present); their
            // scores are discarded.
            const int tk = base_ + lane;
            const int pi = min(max((tk - s0) >> 3, 0), kSeg / 8 - 1);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const long phys = spt[j * (kSeg / 8) + pi];
                const uint4* row = reinterpret_cast<const uint4*>(a.pool + phys * g.page_bytes + kv_off +
                                                                  (tk & 7) * NG);
#pragma unroll
                for (int w = 0; w < IW / 4; ++w) {
                    const uint4 v = row[w];
                    dst[j][4 * w] = v.x; dst[j][4 * w + 1] = v.y; dst[j][4 * w + 2] = v.z; dst[j][4 * w + 3] = v.w;
                }
            }
        };
        int base = s0 + wave * 64;
        if (base < s1) fetch_k(base, ik);
        for (; base < s1; base += kThreadsV2) {
            const int tok = base + lane;
            const int P = __builtin_amdgcn_readfirstlane(g.sink + base);   // position of lane 0 (wave-uniform)
            if (base + kThreadsV2 < s1) fetch_k(base + kThreadsV2, nk);
            bool in[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) in[j] = tok >= lo[j] && tok < hi[j] && tok < s1;
            const_ptr<float> rcP = as_const(a.rc + long(P) * 64);
            const_ptr<float> rsP = as_const(a.rs + long(P) * 64);
            float acc[2] = {0.f, 0.f};
#pragma unroll
            for (int ch = 0; ch < 8; ++ch) {
                float cs[8], sn[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float cp = rcP[8 * ch + u], sp = rsP[8 * ch + u];
                    cs[u] = fmaf(cp, cl[8 * ch + u], -sp * sl[8 * ch + u]);
                    sn[u] = fmaf(sp, cl[8 * ch + u], cp * sl[8 * ch + u]);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    if (in[j]) acc[j] = chunk_score<C>(ch, ik[j], cb, qp[j], cs, sn, acc[j]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (in[j]) {
                    const float sv = acc[j] * a.scale_log2;
                    sc[j * kSeg + (tok - s0)] = sv;
                    mloc[j] = fmaxf(mloc[j], sv);
                }
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int w = 0; w < IW; ++w) ik[j][w] = nk[j][w];
        }
        // ---- block max, rescale ----
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float mw = wave_max(mloc[j]);
            if (lane == 0) red[j * 8 + wave] = mw;
        }
        __syncthreads();
        float Mn[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            Mn[j] = red[j * 8];
            for (int w = 1; w < kThreadsV2 / 64; ++w) Mn[j] = fmaxf(Mn[j], red[j * 8 + w]);
            if (Mn[j] > M[j]) {
                if (M[j] != -INFINITY) {
                    const float f = exp2f(M[j] - Mn[j]);
                    for (int e = tid; e < NG * kBinPad; e += kThreadsV2) {
                        uint32_t* bp = bins + j * NG * kBinPad + e;
                        *bp = uint32_t(float(*bp) * f + 0.5f);
                    }
                    lsum[j] = uint32_t(float(lsum[j]) * f + 0.5f);
                }
                M[j] = Mn[j];
            }
        }
        __syncthreads();
        // ---- phase 2: V bins ----
        uint32_t iv[2][IW], nv[2][IW];
        auto fetch_v = [&](int tk, uint32_t (*dst)[IW]) {
            const int pi = min(max((tk - s0) >> 3, 0), kSeg / 8 - 1);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const long phys = spt[j * (kSeg / 8) + pi];
                const uint4* row = reinterpret_cast<const uint4*>(a.pool + phys * g.page_bytes + kv_off + 8 * NG +
                                                                  (tk & 7) * NG);
#pragma unroll
                for (int w = 0; w < IW / 4; ++w) {
                    const uint4 v = row[w];
                    dst[j][4 * w] = v.x; dst[j][4 * w + 1] = v.y; dst[j][4 * w + 2] = v.z; dst[j][4 * w + 3] = v.w;
                }
            }
        };
        int tok = s0 + tid;
        if (tok < s1) fetch_v(tok, iv);
        for (; tok < s1; tok += kThreadsV2) {
            if (tok + kThreadsV2 < s1) fetch_v(tok + kThreadsV2, nv);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (tok >= lo[j] && tok < hi[j]) {
                    const float w = exp2f(sc[j * kSeg + (tok - s0)] - M[j]);
                    const uint32_t u = uint32_t(fmaf(w, fix_scale, 0.5f));
                    lsum[j] += u;
                    uint32_t* bj = bins + j * NG * kBinPad;
#pragma unroll
                    for (int grp = 0; grp < NG; ++grp)
                        atomicAdd(bj + grp * kBinPad + ((iv[j][grp >> 2] >> (8 * (grp & 3))) & 0xff), u);
                }
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int w = 0; w < IW; ++w) iv[j][w] = nv[j][w];
        }
    }
    // ---- totals ----
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        uint32_t t = lsum[j];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off, 64);
        if (lane == 0) reinterpret_cast<uint32_t*>(red)[16 + j * 8 + wave] = t;
    }
    __syncthreads();
    {   // stage B_t^V over B_t^K with a 16-B pad per group row
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.slice_v) +
                                                          h * a.slice_hstride);
        uint4* dst = reinterpret_cast<uint4*>(cb);
        constexpr int row16 = K * C * 2 / 16;          // 16-B units per group row
        for (int e = tid; e < NG * row16; e += kThreadsV2) dst[(e / row16) * (row16 + 1) + e % row16] = src[e];
    }
    __syncthreads();
    // ---- o = sum_r bin[g][r] B_t^V[g][r] ----
    constexpr int RCH = kThreadsV2 / (2 * NG);       // codeword chunks per (request, group): 16 (C=8), 8 (C=4)
    constexpr int RPC = K / RCH;                     // codewords per chunk
    const int j = tid / (kThreadsV2 / 2);
    const int grp = (tid / RCH) & (NG - 1);
    const int rc = tid & (RCH - 1);
    float o[C];
#pragma unroll
    for (int i = 0; i < C; ++i) o[i] = 0.f;
    const uint32_t* bj = bins + (j * NG + grp) * kBinPad;
    const uint16_t* vrow = cb + grp * (K * C + 8);
    for (int k = 0; k < RPC; ++k) {
        const int r = rc + RCH * k;
        const float bw = float(bj[r]);
        float v[C];
        if constexpr (C == 8) {
            const uint4 w = *reinterpret_cast<const uint4*>(vrow + r * 8);
            v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
            v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
        } else {
            const uint2 w = *reinterpret_cast<const uint2*>(vrow + r * 4);
            v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
        }
#pragma unroll
        for (int i = 0; i < C; ++i) o[i] = fmaf(bw, v[i], o[i]);
    }
    // reduce over the RCH chunks (adjacent lanes)
#pragma unroll
    for (int i = 0; i < C; ++i)
#pragma unroll
        for (int off = 1; off < RCH; off <<= 1) o[i] += __shfl_xor(o[i], off, 64);
    float* ored = reinterpret_cast<float*>(bins);    // bins are consumed above: reuse [2][128]
    __syncthreads();
    if (rc == 0)
#pragma unroll
        for (int i = 0; i < C; ++i) ored[j * D + grp * C + i] = o[i];
    __syncthreads();
    if (tid < 256) {
        const int jj = tid >> 7, d = tid & 127;
        const int rb = r0 + jj;
        if (rb < a.B) {
            const long orow = (long(rb) * g.H + h) * a.S_tot + split;
            if (hi[jj] > lo[jj]) {
                const uint32_t* tr = reinterpret_cast<const uint32_t*>(red) + 16 + jj * 8;
                float L = 0.f;                                                              // fixed point
                for (int w = 0; w < kThreadsV2 / 64; ++w) L += float(tr[w]);
                a.part_o[orow * D + d] = ored[jj * D + d] / L;
                if (d == 0) a.part_lse[orow] = (M[jj] + log2f(L / fix_scale)) * kLn2;
            } else {
                a.part_o[orow * D + d] = 0.f;
                if (d == 0) a.part_lse[orow] = -INFINITY;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bf16-window partial: sinks [0, min(L, sink)) and recent tokens
// [sink + 8*n_pages, L) of loop step t.  Grid (head, request); 256 threads;
// each wave takes every fourth window token, lane l owns RoPE pair
// (l, l + 64).  Writes partial slot num_splits.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) window_partial_kernel(AttnArgs a) {
    constexpr int D = 128;
    const Geo& g = a.geo;
    const int h = blockIdx.x, rb = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = clamp_len(a, rb);
    const int np = n_index_pages(L, g);
    const int q_hi = g.sink + g.page * np;
    const int n_sink = min(L, g.sink);
    const int n_recent = max(0, L - q_hi);
    const int n_w = n_sink + n_recent;
    const int ring = g.W + g.page;

    const uint16_t* qp = a.q + (long(rb) * g.H + h) * D;
    const float q1 = bf16_to_f32(qp[lane]), q2 = bf16_to_f32(qp[lane + 64]);
    const long wbase = ((long(rb) * g.T + a.step) * g.H + h) * long(g.Wcap) * D;
    float m = -INFINITY, l = 0.f, o1 = 0.f, o2 = 0.f;
    for (int w = wave; w < n_w; w += 4) {
        const int p = w < n_sink ? w : q_hi + (w - n_sink);
        const int slot = p < g.sink ? p : g.sink + (p - g.sink) % ring;
        const uint16_t* kr = a.wk + wbase + long(slot) * D;
        const uint16_t* vr = a.wv + wbase + long(slot) * D;
        const float k1 = bf16_to_f32(kr[lane]), k2 = bf16_to_f32(kr[lane + 64]);
        const float cs = a.rc[long(p) * (D / 2) + lane], sn = a.rs[long(p) * (D / 2) + lane];
        const float r1 = k1 * cs - k2 * sn, r2 = k2 * cs + k1 * sn;
        const float s = wave_sum(q1 * r1 + q2 * r2) * a.scale_log2;
        const float m_new = fmaxf(m, s);
        const float alpha = exp2f(m - m_new), wgt = exp2f(s - m_new);
        l = l * alpha + wgt;
        o1 = o1 * alpha + wgt * bf16_to_f32(vr[lane]);
        o2 = o2 * alpha + wgt * bf16_to_f32(vr[lane + 64]);
        m = m_new;
    }
    __shared__ float red[4][D + 2];
    red[wave][lane] = o1;
    red[wave][lane + 64] = o2;
    if (lane == 0) {
        red[wave][D] = m;
        red[wave][D + 1] = l;
    }
    __syncthreads();
    if (tid < D) {
        float M = -INFINITY;
        for (int w2 = 0; w2 < 4; ++w2) M = fmaxf(M, red[w2][D]);
        float Ls = 0.f, o = 0.f;
        for (int w2 = 0; w2 < 4; ++w2) {
            const float fw = red[w2][D] == -INFINITY ? 0.f : exp2f(red[w2][D] - M);
            Ls += red[w2][D + 1] * fw;
            o += red[w2][tid] * fw;
        }
        const long orow = (long(rb) * g.H + h) * a.S_tot + a.num_splits;
        a.part_o[orow * D + tid] = o / Ls;
        if (tid == 0) a.part_lse[orow] = (M + log2f(Ls)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// Exact merge of S partials per row.
// ---------------------------------------------------------------------------
__global__ void merge_kernel(const float* __restrict__ po, const float* __restrict__ pl, int S, int D,
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

int choose_splits(const Geo& g, int B, int max_len) {
    const int max_pages = std::max(0, (max_len - g.sink - g.W) / g.page);
    if (max_pages == 0) return 1;
    const int wgs = ((B + 1) / 2) * g.H;
    int s = ceil_div(512, std::max(1, wgs));
    s = std::max(s, ceil_div(max_pages, 256));          // at most 256 pages (2048 tokens) per split
    s = std::min(s, std::max(1, ceil_div(max_pages, 16)));
    return std::max(1, std::min(s, 1024));
}

}  // namespace
}  // namespace lvq

using namespace lvq;

extern "C" size_t lvq_decode_attn_workspace(const lvq_geom* gp, int32_t B, int32_t max_len, int32_t num_splits) {
    Geo g;
    if (validate_geom(gp, &g) != LVQ_OK || B < 0 || max_len < 0 || num_splits < 0) return 0;
    const int S = num_splits > 0 ? num_splits : choose_splits(g, B, max_len);
    const size_t rows = size_t(B) * g.H * (S + 1);
    return rows * g.D * sizeof(float) + rows * sizeof(float) + size_t(B) * g.H * 128 * sizeof(uint32_t);
}

extern "C" size_t lvq_quant_partial_workspace(const lvq_geom* gp, int32_t B) {
    Geo g;
    if (validate_geom(gp, &g) != LVQ_OK || B < 0) return 0;
    return size_t(B) * g.H * 128 * sizeof(uint32_t);
}

namespace lvq {
namespace {

// Checks shared by the attention entry points; fills the kernel arguments
// except the partial buffers.
lvq_status prepare(const char* fn, const lvq_geom* gp, int32_t step, const void* q, const int32_t* seq_len,
                   int32_t max_len, const float* rope_cos, const float* rope_sin, int32_t rope_len, float sm_scale,
                   int32_t B, AttnArgs* a) {
    Geo& g = a->geo;
    lvq_status st = validate_geom(gp, &g);
    if (st != LVQ_OK) return st;
    LVQ_REQUIRE(step >= 0 && step < g.T, LVQ_ERR_INVALID_ARG, "%s: step %d out of [0,%d)", fn, step, g.T);
    LVQ_REQUIRE(B >= 0 && max_len >= 1, LVQ_ERR_INVALID_ARG, "%s: bad sizes B=%d max_len=%d", fn, B, max_len);
    LVQ_REQUIRE(max_len <= rope_len, LVQ_ERR_INVALID_ARG, "%s: max_len %d exceeds rope_len %d", fn, max_len,
                rope_len);
    LVQ_REQUIRE(std::isfinite(sm_scale), LVQ_ERR_INVALID_ARG, "%s: sm_scale not finite", fn);
    LVQ_REQUIRE(B <= 65535 * 2, LVQ_ERR_UNSUPPORTED, "%s: batch too large", fn);
    LVQ_REQUIRE(B == 0 || (q && seq_len && rope_cos && rope_sin), LVQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    a->step = step;
    a->beta = step / g.Tc;
    a->q = static_cast<const uint16_t*>(q);
    a->seq_len = seq_len;
    a->rc = rope_cos;
    a->rs = rope_sin;
    a->scale_log2 = sm_scale * kLog2e;
    a->B = B;
    a->max_len = max_len;
    a->rope_len = rope_len;
    return LVQ_OK;
}

int max_index_pages(const Geo& g, int max_len) { return std::max(0, (max_len - g.sink - g.W) / g.page); }

int ceil_log2(long x) {
    int r = 0;
    while ((1L << r) < x) ++r;
    return r;
}

// Packs q into a.qpack (bf16 codebooks only) and launches the index-page partial.
lvq_status launch_quant(AttnArgs& a, uint32_t* qpack, hipStream_t stream) {
    const Geo& g = a.geo;
    const dim3 grid(a.num_splits, g.H, (a.B + 1) / 2);
    if (g.cb == LVQ_BF16) {
        hipLaunchKernelGGL(pack_q_kernel, dim3(a.B * g.H), dim3(64), 0, stream, a.q, qpack);
        lvq_status st = check_launch("query packing");
        if (st != LVQ_OK) return st;
        a.qpack = qpack;
        a.fix_bits = std::max(8, std::min(20, 31 - ceil_log2(long(a.pps) * g.page)));
        const size_t lds = size_t(g.NG) * (g.K * g.c + 8) * 2 + size_t(2) * g.NG * kBinPad * 4 +
                           size_t(2) * kSeg * 4 + 32 * 4 + size_t(2) * (kSeg / 8) * 4;
        auto kern = g.c == 8 ? quant_v2_kernel<8> : quant_v2_kernel<4>;
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                int(lds)) != hipSuccess) {
            (void)hipGetLastError();
            set_error("quantized partial: cannot reserve %zu bytes of LDS", lds);
            return LVQ_ERR_HIP;
        }
        hipLaunchKernelGGL(kern, grid, dim3(kThreadsV2), lds, stream, a);
    } else {
        const size_t red_bytes = 4 * (g.D + 2) * sizeof(float);
        if (g.c == 8)
            hipLaunchKernelGGL((quant_partial_kernel<8, float, false>), grid, dim3(256), red_bytes, stream, a);
        else
            hipLaunchKernelGGL((quant_partial_kernel<4, float, false>), grid, dim3(256), red_bytes, stream, a);
    }
    return check_launch("quantized partial");
}

lvq_status launch_window(AttnArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(window_partial_kernel, dim3(a.geo.H, a.B), dim3(256), 0, stream, a);
    return check_launch("window partial");
}

void set_slices(AttnArgs* a, const void* slices) {
    const Geo& g = a->geo;
    const long hstride = 2L * g.K * g.D;              // elements per (step, head): K and V slices
    const long kvstride = long(g.K) * g.D;
    const char* base = static_cast<const char*>(slices) + long(a->step) * g.H * hstride * g.cb_bytes;
    a->slice_k = base;
    a->slice_v = base + kvstride * g.cb_bytes;
    a->slice_hstride = hstride;
}

}  // namespace
}  // namespace lvq

extern "C" lvq_status lvq_quant_partial(const lvq_geom* gp, int32_t step, const void* q, const uint8_t* pool,
                                        const int32_t* page_table, int32_t pt_stride, const int32_t* seq_len,
                                        int32_t max_len, const void* slices, const float* rope_cos,
                                        const float* rope_sin, int32_t rope_len, float sm_scale, float* part_o,
                                        float* part_lse, int32_t num_splits, int32_t S_tot, void* ws,
                                        size_t ws_bytes, int32_t B, hipStream_t stream) {
    AttnArgs a{};
    lvq_status st = prepare("lvq_quant_partial", gp, step, q, seq_len, max_len, rope_cos, rope_sin, rope_len,
                            sm_scale, B, &a);
    if (st != LVQ_OK) return st;
    const Geo& g = a.geo;
    LVQ_REQUIRE(num_splits >= 1 && num_splits <= 1024 && S_tot >= num_splits, LVQ_ERR_INVALID_ARG,
                "lvq_quant_partial: num_splits %d, S_tot %d", num_splits, S_tot);
    if (B == 0) return LVQ_OK;
    const int max_pages = max_index_pages(g, max_len);
    LVQ_REQUIRE(slices && part_o && part_lse && ws, LVQ_ERR_INVALID_ARG, "lvq_quant_partial: NULL pointer");
    LVQ_REQUIRE(ws_bytes >= lvq_quant_partial_workspace(gp, B), LVQ_ERR_WORKSPACE,
                "lvq_quant_partial: workspace %zu < %zu bytes", ws_bytes, lvq_quant_partial_workspace(gp, B));
    LVQ_REQUIRE(max_pages == 0 || (pool && page_table), LVQ_ERR_INVALID_ARG,
                "lvq_quant_partial: NULL pool or page table");
    LVQ_REQUIRE(pt_stride >= max_pages, LVQ_ERR_INVALID_ARG, "lvq_quant_partial: pt_stride %d < %d pages",
                pt_stride, max_pages);
    a.pool = pool;
    a.pt = page_table;
    a.pt_stride = pt_stride;
    set_slices(&a, slices);
    a.part_o = part_o;
    a.part_lse = part_lse;
    a.S_tot = S_tot;
    a.num_splits = num_splits;
    a.pps = max_pages > 0 ? ceil_div(max_pages, num_splits) : 1;
    return launch_quant(a, static_cast<uint32_t*>(ws), stream);
}

extern "C" lvq_status lvq_window_partial(const lvq_geom* gp, int32_t step, const void* q, const int32_t* seq_len,
                                         int32_t max_len, const void* win_k, const void* win_v,
                                         const float* rope_cos, const float* rope_sin, int32_t rope_len,
                                         float sm_scale, float* part_o, float* part_lse, int32_t slot,
                                         int32_t S_tot, int32_t B, hipStream_t stream) {
    AttnArgs a{};
    lvq_status st = prepare("lvq_window_partial", gp, step, q, seq_len, max_len, rope_cos, rope_sin, rope_len,
                            sm_scale, B, &a);
    if (st != LVQ_OK) return st;
    LVQ_REQUIRE(slot >= 0 && slot < S_tot, LVQ_ERR_INVALID_ARG, "lvq_window_partial: slot %d of %d", slot, S_tot);
    if (B == 0) return LVQ_OK;
    LVQ_REQUIRE(win_k && win_v && part_o && part_lse, LVQ_ERR_INVALID_ARG, "lvq_window_partial: NULL pointer");
    a.wk = static_cast<const uint16_t*>(win_k);
    a.wv = static_cast<const uint16_t*>(win_v);
    a.part_o = part_o;
    a.part_lse = part_lse;
    a.S_tot = S_tot;
    a.num_splits = slot;
    return launch_window(a, stream);
}

extern "C" lvq_status lvq_decode_attn(const lvq_geom* gp, int32_t step, const void* q, const uint8_t* pool,
                                      const int32_t* page_table, int32_t pt_stride, const int32_t* seq_len,
                                      int32_t max_len, const void* win_k, const void* win_v, const void* slices,
                                      const float* rope_cos, const float* rope_sin, int32_t rope_len,
                                      float sm_scale, float* out, float* lse_out, void* ws, size_t ws_bytes,
                                      int32_t num_splits, int32_t B, hipStream_t stream) {
    AttnArgs a{};
    lvq_status st = prepare("lvq_decode_attn", gp, step, q, seq_len, max_len, rope_cos, rope_sin, rope_len,
                            sm_scale, B, &a);
    if (st != LVQ_OK) return st;
    const Geo& g = a.geo;
    LVQ_REQUIRE(num_splits >= 0 && num_splits <= 1024, LVQ_ERR_INVALID_ARG, "lvq_decode_attn: num_splits %d",
                num_splits);
    LVQ_REQUIRE(pt_stride >= 0, LVQ_ERR_INVALID_ARG, "lvq_decode_attn: negative pt_stride");
    if (B == 0) return LVQ_OK;
    LVQ_REQUIRE(win_k && win_v && slices && out && ws, LVQ_ERR_INVALID_ARG, "lvq_decode_attn: NULL pointer");
    const int max_pages = max_index_pages(g, max_len);
    LVQ_REQUIRE(max_pages == 0 || (pool && page_table), LVQ_ERR_INVALID_ARG,
                "lvq_decode_attn: NULL pool or page table");
    LVQ_REQUIRE(pt_stride >= max_pages, LVQ_ERR_INVALID_ARG, "lvq_decode_attn: pt_stride %d < %d pages",
                pt_stride, max_pages);
    const int S = num_splits > 0 ? num_splits : choose_splits(g, B, max_len);
    const size_t need = lvq_decode_attn_workspace(gp, B, max_len, S);
    LVQ_REQUIRE(ws_bytes >= need, LVQ_ERR_WORKSPACE, "lvq_decode_attn: workspace %zu < %zu bytes", ws_bytes, need);

    a.pool = pool;
    a.pt = page_table;
    a.pt_stride = pt_stride;
    a.wk = static_cast<const uint16_t*>(win_k);
    a.wv = static_cast<const uint16_t*>(win_v);
    set_slices(&a, slices);
    const size_t rows = size_t(B) * g.H * (S + 1);
    a.part_o = static_cast<float*>(ws);
    a.part_lse = a.part_o + rows * g.D;
    a.S_tot = S + 1;
    a.num_splits = S;
    a.pps = max_pages > 0 ? ceil_div(max_pages, S) : 1;
    uint32_t* qpack = reinterpret_cast<uint32_t*>(a.part_lse + rows);
    if ((st = launch_quant(a, qpack, stream)) != LVQ_OK) return st;
    if ((st = launch_window(a, stream)) != LVQ_OK) return st;
    hipLaunchKernelGGL(merge_kernel, dim3(B * g.H), dim3(128), 0, stream, a.part_o, a.part_lse, S + 1, g.D, out,
                       lse_out);
    return check_launch("lvq_decode_attn: merge");
}

extern "C" int32_t lvq_decode_attn_splits(const lvq_geom* gp, int32_t B, int32_t max_len) {
    Geo g;
    if (validate_geom(gp, &g) != LVQ_OK || B < 0 || max_len < 1) return 0;
    return choose_splits(g, B, max_len);
}

extern "C" lvq_status splitk_lse_merge(const float* part_o, const float* part_lse, int32_t n, int32_t S, int32_t D,
                                       float* out, float* lse_out, hipStream_t stream) {
    LVQ_REQUIRE(n >= 0 && S >= 1 && D >= 1, LVQ_ERR_INVALID_ARG, "splitk_lse_merge: bad sizes n=%d S=%d D=%d", n,
                S, D);
    if (n == 0) return LVQ_OK;
    LVQ_REQUIRE(part_o && part_lse && out, LVQ_ERR_INVALID_ARG, "splitk_lse_merge: NULL pointer");
    LVQ_REQUIRE(n <= 0x7fffffff, LVQ_ERR_UNSUPPORTED, "splitk_lse_merge: too many rows");
    hipLaunchKernelGGL(merge_kernel, dim3(n), dim3(D < 256 ? ((D + 63) / 64) * 64 : 256), 0, stream, part_o,
                       part_lse, S, D, out, lse_out);
    return check_launch("splitk_lse_merge");
}
