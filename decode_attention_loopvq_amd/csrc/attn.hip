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
    return rows * g.D * sizeof(float) + rows * sizeof(float);
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
    return LVQ_OK;
}

int max_index_pages(const Geo& g, int max_len) { return std::max(0, (max_len - g.sink - g.W) / g.page); }

lvq_status launch_quant(AttnArgs& a, hipStream_t stream) {
    const Geo& g = a.geo;
    const dim3 grid(a.num_splits, g.H, (a.B + 1) / 2);
    const size_t red_bytes = 4 * (g.D + 2) * sizeof(float);
    if (g.cb == LVQ_BF16) {
        const size_t lds = 2 * size_t(g.K) * g.D * sizeof(uint16_t) + red_bytes;
        auto kern = g.c == 8 ? quant_partial_kernel<8, uint16_t, true> : quant_partial_kernel<4, uint16_t, true>;
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                int(lds)) != hipSuccess) {
            (void)hipGetLastError();
            set_error("quantized partial: cannot reserve %zu bytes of LDS", lds);
            return LVQ_ERR_HIP;
        }
        hipLaunchKernelGGL(kern, grid, dim3(256), lds, stream, a);
    } else {
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
                                        float* part_lse, int32_t num_splits, int32_t S_tot, int32_t B,
                                        hipStream_t stream) {
    AttnArgs a{};
    lvq_status st = prepare("lvq_quant_partial", gp, step, q, seq_len, max_len, rope_cos, rope_sin, rope_len,
                            sm_scale, B, &a);
    if (st != LVQ_OK) return st;
    const Geo& g = a.geo;
    LVQ_REQUIRE(num_splits >= 1 && num_splits <= 1024 && S_tot >= num_splits, LVQ_ERR_INVALID_ARG,
                "lvq_quant_partial: num_splits %d, S_tot %d", num_splits, S_tot);
    if (B == 0) return LVQ_OK;
    const int max_pages = max_index_pages(g, max_len);
    LVQ_REQUIRE(slices && part_o && part_lse, LVQ_ERR_INVALID_ARG, "lvq_quant_partial: NULL pointer");
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
    return launch_quant(a, stream);
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
    if ((st = launch_quant(a, stream)) != LVQ_OK) return st;
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
