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
#include <cmath>
#include <type_traits>

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
    const int32_t* order;       // [B] request of each workgroup slot (NULL: request i in slot i)
    const uint16_t* kscale;     // key scale stream fp16 [physical page][T][8] (NULL: none)
    int rope_len;
    const uint32_t* qpack;      // [B*H][64] packed fp16 query rows (written and read by index_attn_kernel)
    const uint4* rope16;        // [16][rope_len] packed fp16 cos/sin chunks (lvq_rope_table_f16)
    int fix_bits;               // fixed-point fraction bits of the softmax weights in the V bins
};

__device__ __forceinline__ int clamp_len(const AttnArgs& a, int rb) {
    const int L = a.seq_len[rb];
    return L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
}

// The request in slot i of the batch's grouping (workgroups take consecutive slots): order[i] when an
// order is given, else i; B (no request) for slots past the batch and for entries outside [0, B).
__device__ __forceinline__ int group_request(const AttnArgs& a, int i) {
    if (i >= a.B) return a.B;
    if (!a.order) return i;
    const int r = a.order[i];
    return r >= 0 && r < a.B ? r : a.B;
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
    int rq[2];
    for (int j = 0; j < 2; ++j) {
        const int rb = rq[j] = group_request(a, r0 + j);
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
            const int rb = rq[j];
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
        const int rb = rq[j];
        if (rb >= a.B) continue;
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
            float s = (part + __shfl_xor(part, 32, 64)) * a.scale_log2;
            if (a.kscale) s *= f16_to_f32(a.kscale[(phys * g.T + a.step) * 8 + (tok & 7)]);
            float vA[32], vB[32];
#pragma unroll
            for (int q = 0; q < GPC; ++q) {
                const int ia = vrow[(gA + q) ^ (tok & 15)], ib = vrow[(gB + q) ^ (tok & 15)];
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
// Index-page partial for bf16 codebooks.
//
// RoPE score without rotating keys: with the rotate-half pairing (channel i
// with i + 64, angle p*th_i), q . R(p) k = k . psi(p) where
//   psi_i      = cos(p th_i) q_i + sin(p th_i) q_{i+64}
//   psi_{i+64} = cos(p th_i) q_{i+64} - sin(p th_i) q_i      (i < 64),
// i.e. the query turned back by the key's angle.  psi is formed per
// (request, position) in packed fp16 and dotted with the key rebuilt from
// the step's K slice (fp16 in LDS) with fp32 accumulation.  The query is
// pre-scaled by sm_scale * log2(e) so scores come out in log2 units.
//
// V is never rebuilt per token: the softmax weight of each token is added,
// in fixed point, to one bin per (group, codeword) of its V indices, and the
// partial output is sum_r bin[g][r] * B_t^V[g][r] at the end (exact up to
// the weights' rounding).  Weights need the split's running maximum, so each
// segment of tokens is scored first, the maximum taken, the bins rescaled if
// it grew, and the weights then binned.
//
// Workgroup: R requests x one head x one split, 512 threads, one lane per
// token position.  A position's cos/sin (packed fp16, 256 B) is loaded once
// and serves all R requests; the K slice staged once serves all of them.
//
// LDS (bytes):  [0, 64K)    K slice as fp16 [NG][256][C]  (later: V slice)
//               [64K, 128K) bins u32 [256 codewords][R*NG slots]
//               then page ids of the segment and reduction scratch.
// Bin slot of (request j, group g) is j*NG + g; row r holds slot s at
// byte r*256 + 4*s.  The V index bytes of a token sit XOR-rotated by
// (token & 15) in the pool (byte m holds group m ^ (token & 15)), so at
// step m the 16 lanes of each LDS phase hit 16 distinct groups and thus 16
// distinct banks.
// ---------------------------------------------------------------------------
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

template <typename T>
using const_ptr = const __attribute__((address_space(4))) T*;
template <typename T>
__device__ __forceinline__ const_ptr<T> as_const(const T* p) {
    return reinterpret_cast<const_ptr<T>>(reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ h2_t as_h2(uint32_t x) { return __builtin_bit_cast(h2_t, x); }

__device__ __forceinline__ float dot2h(uint32_t a, h2_t b, float c) {
    return __builtin_amdgcn_fdot2(as_h2(a), b, c, false);
}

// Two bf16 (one dword) to two fp16 (one dword), round to nearest even.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
    const h2_t h = {(_Float16)bf16_lo(w), (_Float16)bf16_hi(w)};
    return __builtin_bit_cast(uint32_t, h);
}

// Byte offset (r << SH) of the codeword r held in byte B of w (one SDWA shift).
template <int SH, int B>
__device__ __forceinline__ uint32_t byte_shl(uint32_t w) {
    uint32_t d;
    if constexpr (B == 0)
        asm("v_lshlrev_b32_sdwa %0, %2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
            : "=v"(d) : "v"(w), "i"(SH));
    else if constexpr (B == 1)
        asm("v_lshlrev_b32_sdwa %0, %2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
            : "=v"(d) : "v"(w), "i"(SH));
    else if constexpr (B == 2)
        asm("v_lshlrev_b32_sdwa %0, %2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
            : "=v"(d) : "v"(w), "i"(SH));
    else
        asm("v_lshlrev_b32_sdwa %0, %2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
            : "=v"(d) : "v"(w), "i"(SH));
    return d;
}

template <int M, int N>
struct StaticFor {
    template <typename F>
    __device__ __forceinline__ static void run(F&& f) {
        if constexpr (M < N) {
            f(std::integral_constant<int, M>{});
            StaticFor<M + 1, N>::run(f);
        }
    }
};

constexpr int kIThreads = 256;                    // index-page partial: 4 waves, two workgroups per CU
constexpr int kChunk = 64;                        // tokens per wave iteration (one per lane)
constexpr int kMaxSplitTok = 1536;                // index tokens per split at most (192 pages)
constexpr int kChunksPerWave = kMaxSplitTok / kChunk / (kIThreads / 64);

// Index-token range [lo, hi) of request slot j (request rq[j], none when >= B) of a workgroup in split
// `split` (hi <= lo: empty).
template <int R>
__device__ __forceinline__ bool split_ranges(const AttnArgs& a, int split, const int (&rq)[R], int (&lo)[R],
                                             int (&hi)[R]) {
    const Geo& g = a.geo;
    const int split_tok = a.pps * g.page;
    bool any = false;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int rb = rq[j];
        const int np8 = rb < a.B ? n_index_pages(clamp_len(a, rb), g) * g.page : 0;
        lo[j] = min(np8, split * split_tok);
        hi[j] = min(np8, (split + 1) * split_tok);
        any |= hi[j] > lo[j];
    }
    return any;
}

// ---------------------------------------------------------------------------
// Index-page partial for bf16 codebooks: one workgroup per (split, head,
// group of R requests), 256 threads (4 waves), two workgroups per CU.  A
// split holds at most kMaxSplitTok index tokens, so a wave meets at most
// kChunksPerWave chunks of 64 tokens and keeps their scores in registers.
//
// Setup.  The workgroup packs the query rows of its R requests as fp16
// (pre-scaled by sm_scale * log2 e) into the workspace, from where the score
// phase reads them with scalar loads, and stages the step's K slice of head
// h in LDS as fp16 (64 KB).
//
// Scores.  The RoPE score needs no rotated key: with the rotate-half pairing
// (channel i with i + 64, angle p * th_i), q . R(p) k = k . psi(p) with
//   psi_i      = cos(p th_i) q_i + sin(p th_i) q_{i+64}
//   psi_{i+64} = cos(p th_i) q_{i+64} - sin(p th_i) q_i      (i < 64),
// the query turned back by the key's angle.  A lane scores its token for all
// R requests: the position's cos/sin (packed fp16 table, 256 B) are loaded
// once and serve all of them; psi is formed in packed fp16 and dotted with
// the fp16 codewords gathered from LDS (fp32 accumulation).  A chunk is
// worked in steps (frequency quarter qq, request j), quarters outermost:
// step (qq, j) uses the codewords of the groups holding frequencies
// 16qq .. 16qq+15, the 16 query dwords of that quarter (scalar registers)
// and the quarter's cos/sin.  Each step first waits for its own LDS gathers
// and query load, then issues the next step's, so the gathers of one step
// are in flight while the previous one computes and the scalar loads never
// hold up the LDS pipeline.  The cos/sin of a quarter are loaded one
// quarter ahead.
//
// Weights.  The workgroup's maximum per request is taken; the K slice's LDS
// becomes bins [256 codewords][64 slots] (slot g*R + j for group g of
// request j), and every token adds exp2(s - max), in fixed point with
// fix_bits fraction bits, to the bin of each (group, codeword) of its V
// indices (integer LDS atomics).  V index bytes sit XOR-rotated by
// (token & 15) in the pool (byte m holds group m ^ (token & 15)), so at step
// m the 16 lanes of an LDS phase hit 16 distinct groups, hence 16 distinct
// banks.
//
// Contraction.  o = sum_r bin[g][r] * B_t^V[g][r] / sum of weights: lane
// (rb, g16) = (tid >> 4, tid & 15) owns codewords 16rb .. 16rb+15 of group g16
// (and g16 + 16 when c = 4); its V rows are loaded when the weight phase
// starts.  A 16-lane phase reads one bin row at 16 distinct slots.  Each
// wave then overwrites its own bin rows with its lanes' partial sums, and
// after a barrier every output sums 16 partials.  The weight total is exact:
// every group's bins add up to the same integer.
// ---------------------------------------------------------------------------
template <int C, int R, bool KS>
__global__ void __launch_bounds__(kIThreads, 2) index_attn_kernel(AttnArgs a) {
    constexpr int D = 128, K = 256, NG = D / C, NT = kIThreads, NW = NT / 64;
    constexpr int CPW = kChunksPerWave;
    constexpr int SH = (C == 8) ? 4 : 3;           // byte offset of codeword r in its group row: r << SH
    constexpr int IW = NG / 4;                     // index dwords per token row
    constexpr int GQ = (C == 8) ? 4 : 8;           // codewords gathered per score step
    constexpr int GW = C / 2;                      // dwords per fp16 codeword
    constexpr int NSTEP = 4 * R;                   // score steps per chunk (even: buffers alternate)
    constexpr int CB16 = NG * K * C * 2 / 16;      // 16-byte words of the staged slice
    constexpr int NSTAGE = CB16 / NT;
    constexpr int GPL = NG / 16;                   // groups per contraction lane
    constexpr int PL = R * C * GPL;                // partial sums per contraction lane
    static_assert(NSTEP % 2 == 0, "step buffers alternate within a chunk");
    static_assert(R * NG == 64, "one bin row holds R*NG = 64 slots");
    static_assert(NT == 256 && CB16 % NT == 0, "contraction lanes: 16 codeword blocks x 16 groups");
    static_assert(CPW * NW * kChunk == kMaxSplitTok, "a split fills the waves' score registers");
    // Static LDS: the K slice (fp16), later the V bins [256][64] u32; both start at address 0, which
    // folds into instruction offsets.
    __shared__ __align__(16) unsigned char lds[NG * K * C * 2];
    __shared__ float wmax[NW][R];
    uint32_t* bins = reinterpret_cast<uint32_t*>(lds);
    const Geo& g = a.geo;
    // Head fastest in the grid: workgroup ids of one head are congruent modulo 8, so the head's slices
    // stay in one XCD's L2.
    const int h = blockIdx.x, split = blockIdx.y, r0 = blockIdx.z * R;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int rq[R];                                      // the requests of the workgroup's slots (>= B: none)
#pragma unroll
    for (int j = 0; j < R; ++j) rq[j] = group_request(a, r0 + j);
    // Loads that need no request length go first: the K slice of head h and the query elements this
    // thread packs.
    uint4 stage[NSTAGE];
    {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.slice_k) +
                                                          h * a.slice_hstride);
#pragma unroll
        for (int i = 0; i < NSTAGE; ++i) stage[i] = src[tid + i * NT];
    }
    uint32_t qraw = 0;                              // two bf16 query elements (packed-query dword tid & 63)
    const int qj = tid >> 6, qt = tid & 63;
    const long qprow = long(min(rq[min(qj, R - 1)], a.B - 1)) * g.H + h;
    if (tid < R * 64) {
        const int m = qt >> 2, k = qt & 3;
        const int ch = (k < 2 ? 0 : 64) + 4 * m + 2 * (k & 1);
        qraw = *reinterpret_cast<const uint32_t*>(a.q + qprow * D + ch);
    }
    int lo[R], hi[R];
    if (!split_ranges<R>(a, split, rq, lo, hi)) {
        for (int e = tid; e < R * D; e += NT) {
            const int j = e / D, d = e % D, rb = rq[j];
            if (rb >= a.B) continue;
            const long row = (long(rb) * g.H + h) * a.S_tot + split;
            a.part_o[row * D + d] = 0.f;
            if (d == 0) a.part_lse[row] = -INFINITY;
        }
        return;
    }
    long srow[R];
    const int32_t* ptr[R];
    int t_lo = 0x7fffffff, t_hi = 0;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int rb = min(rq[j], a.B - 1);
        ptr[j] = a.pt + long(rb) * a.pt_stride;
        srow[j] = long(rb) * g.H + h;
        if (hi[j] > lo[j]) {
            t_lo = min(t_lo, lo[j]);
            t_hi = max(t_hi, hi[j]);
        }
    }

    // ---- setup: packed query rows (dword t of row j: the fp16 pair of chunk t >> 2, see the score steps) ----
    if (tid < R * 64) {
        const h2_t v = {(_Float16)(bf16_lo(qraw) * a.scale_log2), (_Float16)(bf16_hi(qraw) * a.scale_log2)};
        const_cast<uint32_t*>(a.qpack)[qprow * 64 + qt] = __builtin_bit_cast(uint32_t, v);
    }
    {   // K slice of head h, bf16 -> fp16
        uint4* dst = reinterpret_cast<uint4*>(lds);
#pragma unroll
        for (int i = 0; i < NSTAGE; ++i)
            dst[tid + i * NT] = make_uint4(bf16x2_to_f16x2(stage[i].x), bf16x2_to_f16x2(stage[i].y),
                                           bf16x2_to_f16x2(stage[i].z), bf16x2_to_f16x2(stage[i].w));
    }
    // Other waves read the packed rows through the scalar cache after the barrier below, which orders
    // LDS only: the vector stores must have reached L2 first.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint32_t page_bytes = uint32_t(g.page_bytes);
    const unsigned char* slab = a.pool + (long(a.beta) * g.H + h) * 2 * 8 * NG;   // (block, head) slab of page 0

    // Page ids two chunks ahead, index rows one chunk ahead (two alternating buffers).  Every lane
    // issues the same loads: lanes out of range read a valid page of the request through the clamped
    // page id (a request with no index page reads physical page 0), so the loads in flight can be
    // counted exactly across iterations.
    auto in_req = [&](int j, int tau) { return tau >= lo[j] && tau < hi[j]; };
    auto load_pid = [&](int c, uint32_t (&pid)[R]) {
        const int tau = c * kChunk + lane;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const uint32_t e = uint32_t(ptr[j][max(0, min(tau, hi[j] - 1)) >> 3]);
            pid[j] = hi[j] > 0 ? e : 0u;
        }
    };
    // index row words of chunk c: kv = 0 for the key row, 1 for the value row
    auto load_idx = [&](int c, int kv, const uint32_t (&pid)[R], uint32_t (&ix)[R][IW]) {
        const int tau = c * kChunk + lane;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const uint4* row = reinterpret_cast<const uint4*>(slab + uint64_t(pid[j]) * page_bytes +
                                                              (kv * 8 + (tau & 7)) * NG);
#pragma unroll
            for (int w = 0; w < IW / 4; ++w) {
                const uint4 kv4 = row[w];
                ix[j][4 * w] = kv4.x; ix[j][4 * w + 1] = kv4.y; ix[j][4 * w + 2] = kv4.z; ix[j][4 * w + 3] = kv4.w;
            }
        }
    };

    // key scales of chunk c (KS): token tau of request j at (page, step, tau & 7) of the scale stream
    auto load_ks = [&](int c, const uint32_t (&pid)[R], float (&ks)[R]) {
        if constexpr (KS) {
            const int tau = c * kChunk + lane;
#pragma unroll
            for (int j = 0; j < R; ++j)
                ks[j] = f16_to_f32(a.kscale[(uint64_t(pid[j]) * g.T + a.step) * 8 + (tau & 7)]);
        }
    };

    // ---- scores ----
    uint4 tr[16];                                   // cos/sin of the lane's position, 4 frequencies each
    auto load_tr = [&](int c, auto qc) {
        constexpr int qq = decltype(qc)::value;
        const int p = min(g.sink + c * kChunk + lane, a.rope_len - 1);
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) tr[4 * qq + mm] = a.rope16[long(4 * qq + mm) * a.rope_len + p];
    };
    // Group of the i-th codeword gathered in quarter qq: lo groups first, then the hi groups holding
    // channels 64 + (the same frequencies).
    auto group_of = [](int qq, int i) constexpr {
        return C == 8 ? (i < 2 ? 2 * qq + i : 8 + 2 * qq + (i - 2)) : (i < 4 ? 4 * qq + i : 16 + 4 * qq + (i - 4));
    };
    auto gather = [&](const uint32_t (&ik)[R][IW], auto qc, auto jc, uint32_t (&G)[GQ][GW]) {
        constexpr int qq = decltype(qc)::value, j = decltype(jc)::value;
        StaticFor<0, GQ>::run([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            constexpr int gi = group_of(qq, i);
            const uint32_t off = byte_shl<SH, gi & 3>(ik[j][gi >> 2]);
            const unsigned char* pcw = lds + gi * (K * C * 2) + off;
            if constexpr (C == 8) {
                const uint4 v = *reinterpret_cast<const uint4*>(pcw);
                G[i][0] = v.x; G[i][1] = v.y; G[i][2] = v.z; G[i][3] = v.w;
            } else {
                const uint2 v = *reinterpret_cast<const uint2*>(pcw);
                G[i][0] = v.x; G[i][1] = v.y;
            }
        });
    };
    const_ptr<uint32_t> qrow[R];
#pragma unroll
    for (int j = 0; j < R; ++j) qrow[j] = as_const(a.qpack + srow[j] * 64);
    auto load_q = [&](auto qc, auto jc, uint32_t (&qs)[16]) {
        constexpr int qq = decltype(qc)::value, j = decltype(jc)::value;
#pragma unroll
        for (int u = 0; u < 16; ++u) qs[u] = qrow[j][16 * qq + u];
    };
    float acc[R][2];
    float rmax[R];                                  // the lane's running maximum per request
    float sreg[CPW][R];                             // scores of the wave's chunks, the latest in the last row
    auto compute = [&](auto qc, auto jc, const uint32_t (&G)[GQ][GW], const uint32_t (&qs)[16]) {
        constexpr int qq = decltype(qc)::value, j = decltype(jc)::value;
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {           // RoPE frequencies 4m .. 4m+3
            const int m = 4 * qq + mm;
            const h2_t c01 = as_h2(tr[m].x), c23 = as_h2(tr[m].y);
            const h2_t s01 = as_h2(tr[m].z), s23 = as_h2(tr[m].w);
            const h2_t l01 = as_h2(qs[4 * mm]), l23 = as_h2(qs[4 * mm + 1]);
            const h2_t u01 = as_h2(qs[4 * mm + 2]), u23 = as_h2(qs[4 * mm + 3]);
            const h2_t pl01 = __builtin_elementwise_fma(c01, l01, s01 * u01);
            const h2_t pl23 = __builtin_elementwise_fma(c23, l23, s23 * u23);
            const h2_t ph01 = __builtin_elementwise_fma(c01, u01, -(s01 * l01));
            const h2_t ph23 = __builtin_elementwise_fma(c23, u23, -(s23 * l23));
            uint32_t kl01, kl23, kh01, kh23;
            if constexpr (C == 8) {
                const int il = mm >> 1, d = (mm & 1) * 2;
                kl01 = G[il][d]; kl23 = G[il][d + 1];
                kh01 = G[2 + il][d]; kh23 = G[2 + il][d + 1];
            } else {
                kl01 = G[mm][0]; kl23 = G[mm][1];
                kh01 = G[4 + mm][0]; kh23 = G[4 + mm][1];
            }
            acc[j][0] = dot2h(kl01, pl01, acc[j][0]);
            acc[j][1] = dot2h(kl23, pl23, acc[j][1]);
            acc[j][0] = dot2h(kh01, ph01, acc[j][0]);
            acc[j][1] = dot2h(kh23, ph23, acc[j][1]);
        }
    };
    auto finish = [&](int c, auto jc, const float (&ks)[R]) {
        constexpr int j = decltype(jc)::value;
        const bool in = in_req(j, c * kChunk + lane);
        float s_all = acc[j][0] + acc[j][1];
        if constexpr (KS) s_all *= ks[j];
        acc[j][0] = 0.f;
        acc[j][1] = 0.f;
        sreg[CPW - 1][j] = s_all;
        rmax[j] = fmaxf(rmax[j], in ? s_all : -INFINITY);
    };
    auto shift_scores = [&]() {
#pragma unroll
        for (int k = 0; k + 1 < CPW; ++k)
#pragma unroll
            for (int j = 0; j < R; ++j) sreg[k][j] = sreg[k + 1][j];
    };
    uint32_t G[2][GQ][GW];
    uint32_t qs[2][16];
    // One chunk: steps k = (qq, j); the last step issues the first gathers of the next chunk (ikn).
    auto run_chunk = [&](int c, const uint32_t (&ikc)[R][IW], const uint32_t (&ikn)[R][IW], const float (&ks)[R]) {
        shift_scores();
        StaticFor<0, NSTEP>::run([&](auto kc) {
            constexpr int k = decltype(kc)::value, qq = k / R, j = k % R, b = k & 1;
            constexpr int k1 = (k + 1) % NSTEP;
            using QN = std::integral_constant<int, k1 / R>;
            using JN = std::integral_constant<int, k1 % R>;
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0): this step's gathers and query quarter
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (k + 1 < NSTEP) gather(ikc, QN{}, JN{}, G[b ^ 1]);
            else gather(ikn, QN{}, JN{}, G[b ^ 1]);
            load_q(QN{}, JN{}, qs[b ^ 1]);
            __builtin_amdgcn_sched_barrier(0);
            // at the start of a quarter, the cos/sin of the next quarter (of the wave's next chunk after the last)
            if constexpr (j == 0) load_tr(qq < 3 ? c : c + NW, std::integral_constant<int, (qq + 1) % 4>{});
            compute(std::integral_constant<int, qq>{}, std::integral_constant<int, j>{}, G[b], qs[b]);
            if constexpr (qq == 3) finish(c, std::integral_constant<int, j>{}, ks);
        });
    };
#pragma unroll
    for (int j = 0; j < R; ++j) {
        acc[j][0] = acc[j][1] = 0.f;
        rmax[j] = -INFINITY;
#pragma unroll
        for (int k = 0; k < CPW; ++k) sreg[k][j] = 0.f;
    }
    const int c0 = t_lo / kChunk + wave;
    // page ids of the weight phase's first two chunks, loaded now so that they wait in registers
    uint32_t pidA[R], pidB[R];
    load_pid(c0, pidA);
    load_pid(c0 + NW, pidB);
    int nch = 0;                                    // chunks of this wave
    {
        int c = c0;
        uint32_t pidA[R], pidB[R];
        uint32_t ikA[R][IW], ikB[R][IW];
        float ksA[R], ksB[R];
        load_pid(c, pidA);
        load_pid(c + NW, pidB);
        load_idx(c, 0, pidA, ikA);
        load_ks(c, pidA, ksA);
        load_pid(c + 2 * NW, pidA);
        load_tr(c, std::integral_constant<int, 0>{});
        __syncthreads();                            // K slice staged, query rows packed
        gather(ikA, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, G[0]);
        load_q(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, qs[0]);
        while (c * kChunk < t_hi) {
            load_idx(c + NW, 0, pidB, ikB);
            load_ks(c + NW, pidB, ksB);
            load_pid(c + 3 * NW, pidB);
            run_chunk(c, ikA, ikB, ksA);
            c += NW;
            ++nch;
            if (c * kChunk >= t_hi) break;
            load_idx(c + NW, 0, pidA, ikA);
            load_ks(c + NW, pidA, ksA);
            load_pid(c + 3 * NW, pidA);
            run_chunk(c, ikB, ikA, ksB);
            c += NW;
            ++nch;
        }
    }
    // value index rows of the weight phase's first chunk
    uint32_t ivA[R][IW], ivB[R][IW];
    load_idx(c0, 1, pidA, ivA);
    load_pid(c0 + 2 * NW, pidA);
    // scores of this wave's chunk i now in sreg[CPW - nch + i]: move chunk 0 to the first row
    for (int s = nch; s < CPW; ++s) shift_scores();

    // ---- weights ----
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const float mw = wave_max_dpp(rmax[j]);
        if (lane == 0) wmax[wave][j] = mw;
    }
    __syncthreads();                                // every wave is done with the K slice
#pragma unroll
    for (int i = 0; i < K * 64 / 4 / NT; ++i) reinterpret_cast<uint4*>(bins)[tid + i * NT] = make_uint4(0u, 0u, 0u, 0u);
    // V rows of this lane's contraction block, needed once the bins are complete
    const int cb_blk = tid >> 4, g16 = tid & 15;
    uint4 vrow[16];
    {
        const uint16_t* vsl = static_cast<const uint16_t*>(a.slice_v) + h * a.slice_hstride;
#pragma unroll
        for (int k = 0; k < GPL; ++k) {
            const uint4* src = reinterpret_cast<const uint4*>(vsl + (long(g16 + 16 * k) * K + 16 * cb_blk) * C);
#pragma unroll
            for (int i = 0; i < 16 / GPL; ++i) vrow[k * (16 / GPL) + i] = src[i];
        }
    }
    __syncthreads();                                // bins cleared, wave maxima visible
    float M[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        M[j] = wmax[0][j];
#pragma unroll
        for (int w = 1; w < NW; ++w) M[j] = fmaxf(M[j], wmax[w][j]);
    }
    const float fix_scale = float(1u << a.fix_bits);
    auto bin_chunk = [&](int c, const uint32_t (&iv)[R][IW]) {
        const int tau = c * kChunk + lane;
        // byte k of base[w]: slot byte offset 4R * ((4w + k) ^ (tau & 15)) of the group held in V index byte 4w + k
        const uint32_t rot = (uint32_t(tau) & 15u) * (4u * R) * 0x01010101u;
        uint32_t base[IW];
#pragma unroll
        for (int w = 0; w < IW; ++w) base[w] = ((4u * R) * (0x03020100u + uint32_t(w) * 0x04040404u)) ^ rot;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            // lanes out of range add 0 (their index rows are valid memory, their bins any)
            const uint32_t u = in_req(j, tau)
                                   ? uint32_t(fmaf(__builtin_amdgcn_exp2f(sreg[0][j] - M[j]), fix_scale, 0.5f))
                                   : 0u;
            StaticFor<0, NG>::run([&](auto mc) {
                constexpr int m = decltype(mc)::value;
                // bin byte address [slot offset, codeword, 0, 0] (one v_perm): row = codeword, 256 B per row
                constexpr uint32_t sel = 0x0c0c0000u | (uint32_t(4 + (m & 3)) << 8) | uint32_t(m & 3);
                const uint32_t addr = __builtin_amdgcn_perm(iv[j][m >> 2], base[m >> 2], sel);
                uint32_t* bin = static_cast<uint32_t*>(__builtin_assume_aligned(lds + addr + 4 * j, 4));
                __hip_atomic_fetch_add(bin, u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            });
        }
        shift_scores();
    };
    {
        int c = c0;
        while (c * kChunk < t_hi) {
            load_idx(c + NW, 1, pidB, ivB);
            load_pid(c + 3 * NW, pidB);
            bin_chunk(c, ivA);
            c += NW;
            if (c * kChunk >= t_hi) break;
            load_idx(c + NW, 1, pidA, ivA);
            load_pid(c + 3 * NW, pidA);
            bin_chunk(c, ivB);
            c += NW;
        }
    }
    __syncthreads();

    // ---- contraction: lane (cb_blk, g16) over its 16 codewords ----
    float o[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) o[i] = 0.f;
    uint32_t lsum[R];
#pragma unroll
    for (int j = 0; j < R; ++j) lsum[j] = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = 16 * cb_blk + i;
#pragma unroll
        for (int k = 0; k < GPL; ++k) {
            uint32_t bv[R];
            if constexpr (R == 4) {
                const uint4 b4 = *reinterpret_cast<const uint4*>(bins + r * 64 + (g16 + 16 * k) * R);
                bv[0] = b4.x; bv[1] = b4.y; bv[2] = b4.z; bv[3] = b4.w;
            } else {
                const uint2 b2 = *reinterpret_cast<const uint2*>(bins + r * 64 + (g16 + 16 * k) * R);
                bv[0] = b2.x; bv[1] = b2.y;
            }
            uint32_t vw[C / 2];                     // V row: C bf16 of codeword r, group g16 + 16k
            if constexpr (C == 8) {
                vw[0] = vrow[i].x; vw[1] = vrow[i].y; vw[2] = vrow[i].z; vw[3] = vrow[i].w;
            } else {
                const uint4 q = vrow[k * 8 + (i >> 1)];
                vw[0] = (i & 1) ? q.z : q.x;
                vw[1] = (i & 1) ? q.w : q.y;
            }
#pragma unroll
            for (int j = 0; j < R; ++j) {
                if (k == 0) lsum[j] += bv[j];
                const float bw = float(bv[j]);
#pragma unroll
                for (int u = 0; u < C / 2; ++u) {
                    o[j * C * GPL + k * C + 2 * u] = fmaf(bw, bf16_lo(vw[u]), o[j * C * GPL + k * C + 2 * u]);
                    o[j * C * GPL + k * C + 2 * u + 1] = fmaf(bw, bf16_hi(vw[u]), o[j * C * GPL + k * C + 2 * u + 1]);
                }
            }
        }
    }
    // Partials over this wave's own bin rows (64 rows of 256 B, read by no other wave): lane slot
    // (cb_blk & 3) * 16 + g16 holds PL floats, then the weight totals of the g16 = 0 lanes.
    float* part = reinterpret_cast<float*>(lds) + wave * 4096;
    {
        float4* dst = reinterpret_cast<float4*>(part + ((cb_blk & 3) * 16 + g16) * PL);
#pragma unroll
        for (int i = 0; i < PL / 4; ++i) dst[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
        if (g16 == 0) {
            uint32_t* ld = reinterpret_cast<uint32_t*>(part + 64 * PL) + (cb_blk & 3) * R;
#pragma unroll
            for (int j = 0; j < R; ++j) ld[j] = lsum[j];
        }
    }
    __syncthreads();
    for (int e = tid; e < R * D; e += NT) {
        const int j = e / D, d = e % D, rb = rq[j];
        if (rb >= a.B) continue;
        const long orow = (long(rb) * g.H + h) * a.S_tot + split;
        if (hi[j] <= lo[j]) {
            a.part_o[orow * D + d] = 0.f;
            if (d == 0) a.part_lse[orow] = -INFINITY;
            continue;
        }
        const int gr = d / C, u = d % C;
        const int p = j * C * GPL + (gr >> 4) * C + u;
        const float* pbase = reinterpret_cast<const float*>(lds);
        float accv = 0.f;
        uint64_t L = 0;
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            const float* pw = pbase + (b >> 2) * 4096;
            accv += pw[((b & 3) * 16 + (gr & 15)) * PL + p];
            L += reinterpret_cast<const uint32_t*>(pw + 64 * PL)[(b & 3) * R + j];
        }
        const float Lf = float(L);
        a.part_o[orow * D + d] = accv / Lf;
        if (d == 0) a.part_lse[orow] = (M[j] + (log2f(Lf) - float(a.fix_bits))) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// bf16 window: sinks [0, min(L, sink)) and recent tokens [sink + 8*n_pages, L)
// of loop step t.  Grid (head, request); 256 threads in 16 rows of 16 lanes;
// row r takes window tokens r, r + 16, ...  Lane c of a row owns channels
// 8c .. 8c+7 of its token (one 16-byte load of K and of V); lanes c and c ^ 8
// hold the two halves of each RoPE pair (i, i + 64) and trade them, and the
// cos (loaded by c < 8) and sin (by c >= 8) of their frequencies, through
// DPP; a score is a 16-lane DPP sum.  Each row keeps its own online softmax
// over kWinBatch tokens at a time (every load of the batch issued first);
// the 16 rows are combined through LDS.  kMerge: the window partial is
// merged at once with the row's index-page partials (slots
// 0 .. num_splits-1) into the attention output (the exact logsumexp merge);
// otherwise it is written to slot num_splits.
// ---------------------------------------------------------------------------
constexpr int kWinBatch = 5;
constexpr int kWinPrefetch = 8;                   // index-page partials loaded at the start of the merge

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// Sum over the 16 lanes of a DPP row (every lane gets it).
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp<0x128>(x);     // row_ror:8
    x += dpp<0x124>(x);     // row_ror:4
    x += dpp<0x122>(x);     // row_ror:2
    x += dpp<0x121>(x);     // row_ror:1
    return x;
}

// Window tokens of one request as seen by one row of 16 lanes: lane c16 holds the RoPE pairs of frequencies
// 4*c16 .. 4*c16+3, i.e. channels 4*c16 .. 4*c16+3 and 64 + the same (window_channel); the sinks
// [0, min(L, sink)), then the recent tokens [sink + 8*n_pages, L); n_w of them (none when !live).
__device__ __forceinline__ int window_channel(int c16, int u) { return (u < 4 ? 0 : 64) + 4 * c16 + (u & 3); }

struct WinRow {
    int n_sink, q_hi, n_w, ring;
    long wbase;                                    // element offset of the row's (request, step, head) buffer
    const float* rc;                               // cos and sin of the lane's frequencies at position 0
    const float* rs;
    float ql[4], qh[4];                            // the lane's query channels (i, then i + 64), times sm_scale * log2 e
};

__device__ __forceinline__ WinRow window_setup(const AttnArgs& a, int rb, int h, bool live, int c16) {
    constexpr int D = 128;
    const Geo& g = a.geo;
    WinRow w;
    const int L = clamp_len(a, rb);
    w.q_hi = g.sink + g.page * n_index_pages(L, g);
    w.n_sink = min(L, g.sink);
    w.n_w = live ? w.n_sink + max(0, L - w.q_hi) : 0;
    w.ring = g.W + g.page;
    w.wbase = ((long(rb) * g.T + a.step) * g.H + h) * long(g.Wcap) * D + 4 * c16;
    w.rc = a.rc + 4 * c16;
    w.rs = a.rs + 4 * c16;
    const uint16_t* qp = a.q + (long(rb) * g.H + h) * D + 4 * c16;
    const uint2 lo = *reinterpret_cast<const uint2*>(qp), hi = *reinterpret_cast<const uint2*>(qp + 64);
    w.ql[0] = bf16_lo(lo.x) * a.scale_log2; w.ql[1] = bf16_hi(lo.x) * a.scale_log2;
    w.ql[2] = bf16_lo(lo.y) * a.scale_log2; w.ql[3] = bf16_hi(lo.y) * a.scale_log2;
    w.qh[0] = bf16_lo(hi.x) * a.scale_log2; w.qh[1] = bf16_hi(hi.x) * a.scale_log2;
    w.qh[2] = bf16_lo(hi.y) * a.scale_log2; w.qh[3] = bf16_hi(hi.y) * a.scale_log2;
    return w;
}

// Online softmax step over the window tokens w0, w0 + stride, ... (NB of them, those >= n_w masked; needs
// n_w >= 1), in log2 units: o[] is the lane's part (channels window_channel(c16, u)) of the unnormalised
// sum_w 2^(s_w - m) v_w, with m the row's running maximum (-inf before the first token) and
// l = sum_w 2^(s_w - m), the same in every lane.  The score needs no rotated key: per pair (i, i + 64),
// q . R(p) k = k_i (q_i cos + q_{i+64} sin) + k_{i+64} (q_{i+64} cos - q_i sin).
template <int NB = kWinBatch>
__device__ __forceinline__ void window_batch(const AttnArgs& a, const WinRow& w, int w0, int stride, int c16,
                                             float& m, float& l, float (&o)[8]) {
    constexpr int D = 128;
    const Geo& g = a.geo;
    uint2 kl[NB], kh[NB], vl[NB], vh[NB];
    float4 cs[NB], sn[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int t = min(w0 + stride * i, w.n_w - 1);    // a valid window token; extra ones are masked below
        const int p = t < w.n_sink ? t : w.q_hi + (t - w.n_sink);
        const int slot = p < g.sink ? p : g.sink + (p - g.sink) % w.ring;
        const uint16_t* kr = a.wk + w.wbase + long(slot) * D;
        const uint16_t* vr = a.wv + w.wbase + long(slot) * D;
        kl[i] = *reinterpret_cast<const uint2*>(kr);
        kh[i] = *reinterpret_cast<const uint2*>(kr + 64);
        vl[i] = *reinterpret_cast<const uint2*>(vr);
        vh[i] = *reinterpret_cast<const uint2*>(vr + 64);
        cs[i] = *reinterpret_cast<const float4*>(w.rc + long(p) * (D / 2));
        sn[i] = *reinterpret_cast<const float4*>(w.rs + long(p) * (D / 2));
    }
    float s[NB];
    float mb = m;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const float c4[4] = {cs[i].x, cs[i].y, cs[i].z, cs[i].w};
        const float s4[4] = {sn[i].x, sn[i].y, sn[i].z, sn[i].w};
        const float k_lo[4] = {bf16_lo(kl[i].x), bf16_hi(kl[i].x), bf16_lo(kl[i].y), bf16_hi(kl[i].y)};
        const float k_hi[4] = {bf16_lo(kh[i].x), bf16_hi(kh[i].x), bf16_lo(kh[i].y), bf16_hi(kh[i].y)};
        float part = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float psl = fmaf(w.ql[u], c4[u], w.qh[u] * s4[u]);
            const float psh = fmaf(w.qh[u], c4[u], -(w.ql[u] * s4[u]));
            part = fmaf(k_lo[u], psl, part);
            part = fmaf(k_hi[u], psh, part);
        }
        const float si = row_sum16(part);
        s[i] = w0 + stride * i < w.n_w ? si : -INFINITY;
        mb = fmaxf(mb, s[i]);
    }
    const float mref = mb == -INFINITY ? 0.f : mb;  // a row with no token yet and none in this batch adds 0
    const float alpha = __builtin_amdgcn_exp2f(m - mref);
    l *= alpha;
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] *= alpha;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const float wgt = __builtin_amdgcn_exp2f(s[i] - mref);
        l += wgt;
        const uint32_t v4[4] = {vl[i].x, vl[i].y, vh[i].x, vh[i].y};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            o[2 * u] = fmaf(wgt, bf16_lo(v4[u]), o[2 * u]);
            o[2 * u + 1] = fmaf(wgt, bf16_hi(v4[u]), o[2 * u + 1]);
        }
    }
    m = mb;
}

// One row of 16 lanes attends all window tokens first, first + stride, ... of request rb; on return (m, l,
// o[]) as left by window_batch (m = -inf, l = 0, o = 0 when the row has no token).
__device__ __forceinline__ void window_row(const AttnArgs& a, int rb, int h, bool live, int first, int stride,
                                           int c16, float& m_out, float& l_out, float (&o)[8]) {
    const WinRow w = window_setup(a, rb, h, live, c16);
    float m = -INFINITY, l = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] = 0.f;
    for (int w0 = first; w0 < w.n_w; w0 += stride * kWinBatch) window_batch(a, w, w0, stride, c16, m, l, o);
    m_out = m;
    l_out = l;
}

template <bool kMerge>
__global__ void __launch_bounds__(256, 4) window_kernel(AttnArgs a, float* __restrict__ out, float* __restrict__ lse_out) {
    constexpr int D = 128, NR = 16;
    const int h = blockIdx.x, rb = blockIdx.y;
    const int tid = threadIdx.x, c16 = tid & 15, trow = tid >> 4;
    const long row = long(rb) * a.geo.H + h;
    // merge inputs (the first kWinPrefetch index-page partials of the row), loaded with the window
    float pre_l[kWinPrefetch], pre_o[kWinPrefetch];
    if constexpr (kMerge) {
#pragma unroll
        for (int s2 = 0; s2 < kWinPrefetch; ++s2) {
            const int sc = min(s2, max(a.num_splits - 1, 0));
            pre_l[s2] = a.part_lse[row * a.S_tot + sc];
            pre_o[s2] = a.part_o[(row * a.S_tot + sc) * D + (tid & (D - 1))];
        }
    }
    float m, l, o[8];
    window_row(a, rb, h, true, trow, NR, c16, m, l, o);
    __shared__ float red[NR][D + 2];
#pragma unroll
    for (int u = 0; u < 8; ++u) red[trow][window_channel(c16, u)] = o[u];
    if (c16 == 0) {
        red[trow][D] = m;
        red[trow][D + 1] = l;
    }
    __syncthreads();
    if (tid >= D) return;
    float M = -INFINITY;
    for (int r = 0; r < NR; ++r) M = fmaxf(M, red[r][D]);
    float Ls = 0.f, ov = 0.f;
    for (int r = 0; r < NR; ++r) {
        const float fw = red[r][D] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(red[r][D] - M);
        Ls += red[r][D + 1] * fw;
        ov += red[r][tid] * fw;
    }
    // an empty window (no sink, no recent token) contributes nothing
    const float o_win = Ls > 0.f ? ov / Ls : 0.f;
    const float lse_win = Ls > 0.f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
    if constexpr (!kMerge) {
        const long orow = row * a.S_tot + a.num_splits;
        a.part_o[orow * D + tid] = o_win;
        if (tid == 0) a.part_lse[orow] = lse_win;
    } else {
        const int S = a.num_splits;
        const float* pl = a.part_lse + row * a.S_tot;
        float Mx = lse_win;
#pragma unroll
        for (int s2 = 0; s2 < kWinPrefetch; ++s2)
            if (s2 < S) Mx = fmaxf(Mx, pre_l[s2]);
        for (int s2 = kWinPrefetch; s2 < S; ++s2) Mx = fmaxf(Mx, pl[s2]);
        float Lx = lse_win == -INFINITY ? 0.f : __expf(lse_win - Mx);
#pragma unroll
        for (int s2 = 0; s2 < kWinPrefetch; ++s2)
            if (s2 < S && pre_l[s2] != -INFINITY) Lx += __expf(pre_l[s2] - Mx);
        for (int s2 = kWinPrefetch; s2 < S; ++s2) Lx += pl[s2] == -INFINITY ? 0.f : __expf(pl[s2] - Mx);
        const float lse = Mx + __logf(Lx);              // finite: a row holds at least one token
        float acc = lse_win == -INFINITY ? 0.f : __expf(lse_win - lse) * o_win;
#pragma unroll
        for (int s2 = 0; s2 < kWinPrefetch; ++s2)
            if (s2 < S && pre_l[s2] != -INFINITY) acc += __expf(pre_l[s2] - lse) * pre_o[s2];
        for (int s2 = kWinPrefetch; s2 < S; ++s2)
            if (pl[s2] != -INFINITY) acc += __expf(pl[s2] - lse) * a.part_o[(row * a.S_tot + s2) * D + tid];
        out[row * D + tid] = acc;
        if (lse_out && tid == 0) lse_out[row] = lse;
    }
}

// ---------------------------------------------------------------------------
// Single-pass decode attention for bf16 codebooks: one workgroup of 512
// threads (8 waves, alone on its CU) per (head, group of R requests) does the
// whole call, window and merge included, and writes the output rows.  The K
// slice is staged in LDS once; the index tokens are taken in items of
// kItemTok (the fixed-point weights of an item share one maximum), each
// scored, binned and contracted as in index_attn_kernel, and the items and
// the window are merged per output element with a running logsumexp.  Wave w
// takes chunks w, w + 8, w + 16, ... of 64 tokens, three per item, so its
// load stream runs on across items: the page ids of the next item and the
// key index rows of its first chunk are in flight while the current item
// finishes.
//
// LDS (bytes): [0, 64K) K slice (fp16); [64K, 128K) bins u32 [256][R*NG];
// [128K, 144K) partials (window rows, then per-wave contraction partials);
// then wave maxima, wave weight totals and the window rows' (m, l).  The bin
// address of an atomic is one v_perm: [slot offset, codeword, 0x01, 0] with
// the 0x01 (the 64K page of the bins) taken from the base word.  Each wave
// contracts, and zeroes behind itself, the 32 bin rows no other wave reads,
// so the bins are clear for the next item without a pass of their own.
// ---------------------------------------------------------------------------
constexpr int kFThreads = 512;
constexpr int kItemTok = 1536;                    // index tokens per item (fixed-point weights of one maximum)

// Sum of x over the four 16-lane rows of the wave (every lane gets the sum at its position in the row).
// (The swap results are copied out of their vector before the bit casts: a bit cast of a vector element
// reads element 0.)
template <typename T>
__device__ __forceinline__ T sum_rows4(T x) {
    const uint32_t xi = __builtin_bit_cast(uint32_t, x);
    const auto t = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);   // lanes l and l ^ 32
    const uint32_t t0 = t[0], t1 = t[1];
    const T y = __builtin_bit_cast(T, t0) + __builtin_bit_cast(T, t1);
    const uint32_t yi = __builtin_bit_cast(uint32_t, y);
    const auto u = __builtin_amdgcn_permlane16_swap(yi, yi, false, false);   // rows r and r ^ 1
    const uint32_t u0 = u[0], u1 = u[1];
    return __builtin_bit_cast(T, u0) + __builtin_bit_cast(T, u1);
}

template <int C, int R>
__global__ void __launch_bounds__(kFThreads, 1) index_full_kernel(AttnArgs a, float* __restrict__ out,
                                                                   float* __restrict__ lse_out) {
    constexpr int D = 128, K = 256, NG = D / C, NT = kFThreads, NW = NT / 64;
    constexpr int CPI = kItemTok / kChunk;         // chunks per item
    constexpr int NFAST = NW / 2;                  // the first waves of the workgroup
    constexpr int FCH = 3, SCH = 3;                // chunks per item of the first waves, of the others
    constexpr int SH = (C == 8) ? 4 : 3;           // byte offset of codeword r in its group row: r << SH
    constexpr int IW = NG / 4;                     // index dwords per token row
    constexpr int GQ = (C == 8) ? 4 : 8;           // codewords gathered per score step
    constexpr int GW = C / 2;                      // dwords per fp16 codeword
    constexpr int NSTEP = 4 * R;                   // score steps per chunk (even: buffers alternate)
    constexpr int KS = NG * K * C * 2;             // bytes of the fp16 K slice
    constexpr int NSTAGE = KS / 16 / NT;
    constexpr int GPL = NG / 16;                   // groups per contraction lane
    constexpr int PL = R * C * GPL;                // partial sums per contraction lane
    constexpr int CPB = K / (NT / 16);             // codewords per contraction lane
    constexpr int VPG = CPB * C * 2 / 16;          // 16-byte V words per contraction lane and group
    constexpr int NWW = NFAST;                     // waves that attend the window: the first ones
    constexpr int RPJ = NWW * 4 / R;               // window rows (of 16 lanes) per request
    constexpr int PART = 4096;                     // floats of the partials region
    static_assert(NFAST * FCH + (NW - NFAST) * SCH == CPI && NSTEP % 2 == 0 && R * NG == 64 && CPB == 8,
                  "item and contraction shapes");
    static_assert(16 * PL * NW <= PART && NWW * 4 * D <= PART, "partials region");
    static_assert(RPJ % 4 == 0, "a wave's window rows belong to one request");
    __shared__ __align__(16) unsigned char lds[2 * KS + PART * 4 + 2 * NW * R * 4 + 32 * 2 * 4];
    uint32_t* const bins = reinterpret_cast<uint32_t*>(lds + KS);
    float* const part = reinterpret_cast<float*>(lds + 2 * KS);
    float (*const wmax)[R] = reinterpret_cast<float (*)[R]>(lds + 2 * KS + PART * 4);
    uint32_t (*const lw)[R] = reinterpret_cast<uint32_t (*)[R]>(lds + 2 * KS + PART * 4 + NW * R * 4);
    float (*const wml)[2] = reinterpret_cast<float (*)[2]>(lds + 2 * KS + PART * 4 + 2 * NW * R * 4);   // [16]
    const Geo& g = a.geo;
    const int h = blockIdx.x, r0 = blockIdx.y * R;
    int rq[R];                                      // the requests of the workgroup's slots (>= B: none)
#pragma unroll
    for (int j = 0; j < R; ++j) rq[j] = group_request(a, r0 + j);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // ---- setup ----
    uint32_t qraw = 0;                              // two bf16 query elements (packed-query dword tid & 63)
    const int qj = tid >> 6, qt = tid & 63;
    const long qprow = long(min(rq[min(qj, R - 1)], a.B - 1)) * g.H + h;
    if (tid < R * 64) {
        const int m = qt >> 2, k = qt & 3;
        const int ch = (k < 2 ? 0 : 64) + 4 * m + 2 * (k & 1);
        qraw = *reinterpret_cast<const uint32_t*>(a.q + qprow * D + ch);
    }
    uint4 stage[NSTAGE];
    {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.slice_k) +
                                                          h * a.slice_hstride);
#pragma unroll
        for (int i = 0; i < NSTAGE; ++i) stage[i] = src[tid + i * NT];
    }
    if (tid < R * 64) {   // packed query rows: dword t of row j is the fp16 pair of score chunk t >> 2
        const h2_t v = {(_Float16)(bf16_lo(qraw) * a.scale_log2), (_Float16)(bf16_hi(qraw) * a.scale_log2)};
        const_cast<uint32_t*>(a.qpack)[qprow * 64 + qt] = __builtin_bit_cast(uint32_t, v);
    }
    int hi[R];
    long srow[R];
    const int32_t* ptr[R];
    int t_hi = 0;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int rb = min(rq[j], a.B - 1);
        hi[j] = rq[j] < a.B ? n_index_pages(clamp_len(a, rb), g) * g.page : 0;
        ptr[j] = a.pt + long(rb) * a.pt_stride;
        srow[j] = long(rb) * g.H + h;
        t_hi = max(t_hi, hi[j]);
    }
    const uint32_t page_bytes = uint32_t(g.page_bytes);
    const unsigned char* slab = a.pool + (long(a.beta) * g.H + h) * 2 * 8 * NG;   // (block, head) slab of page 0

    // Every lane issues the same loads: lanes past a request's last token read a valid page of the request
    // through the clamped page id (a request with no index page reads physical page 0).
    auto in_req = [&](int j, int tau) { return tau < hi[j]; };
    auto load_pid = [&](int c, uint32_t (&pid)[R]) {
        const int tau = c * kChunk + lane;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const uint32_t e = uint32_t(ptr[j][max(0, min(tau, hi[j] - 1)) >> 3]);
            pid[j] = hi[j] > 0 ? e : 0u;
        }
    };
    // index row words of chunk c: kv = 0 for the key row, 1 for the value row
    auto load_idx = [&](int c, int kv, const uint32_t (&pid)[R], uint32_t (&ix)[R][IW]) {
        const int tau = c * kChunk + lane;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const uint4* row = reinterpret_cast<const uint4*>(slab + uint64_t(pid[j]) * page_bytes +
                                                              (kv * 8 + (tau & 7)) * NG);
#pragma unroll
            for (int w = 0; w < IW / 4; ++w) {
                const uint4 kv4 = row[w];
                ix[j][4 * w] = kv4.x; ix[j][4 * w + 1] = kv4.y; ix[j][4 * w + 2] = kv4.z; ix[j][4 * w + 3] = kv4.w;
            }
        }
    };
    // Chunks of an item (CPI of them): waves w < NFAST take w + 4i (i < FCH), the others
    // 4 FCH + (w - NFAST) + 4i (i < SCH); a SIMD holds wave w and wave w + NFAST.
    const bool fast = wave < NFAST;
    const int cbase = fast ? wave : 4 * FCH + wave - NFAST;   // chunk of slot 0 in item 0
    constexpr int MCH = FCH > SCH ? FCH : SCH;
    uint32_t pidc[MCH][R];                          // page ids of the current item's chunks (slots)
    if (t_hi > 0) {                                 // (no page table to read otherwise)
#pragma unroll
        for (int i = 0; i < MCH; ++i)
            if (i < (fast ? FCH : SCH)) load_pid(cbase + 4 * i, pidc[i]);
    }
    {   // bins start clear; each item's contraction clears them again behind itself
#pragma unroll
        for (int i = 0; i < 64 * K / 4 / NT; ++i) reinterpret_cast<uint4*>(bins)[tid + i * NT] = make_uint4(0u, 0u, 0u, 0u);
    }

    {   // K slice of head h, bf16 -> fp16
        uint4* dst = reinterpret_cast<uint4*>(lds);
#pragma unroll
        for (int i = 0; i < NSTAGE; ++i)
            dst[tid + i * NT] = make_uint4(bf16x2_to_f16x2(stage[i].x), bf16x2_to_f16x2(stage[i].y),
                                           bf16x2_to_f16x2(stage[i].z), bf16x2_to_f16x2(stage[i].w));
    }
    // Other waves read the packed query rows through the scalar cache after the barrier below, which
    // orders LDS only: the vector stores must have reached L2 first.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- score machinery (as in index_attn_kernel) ----
    uint4 tr[16];                                   // cos/sin of the lane's position, 4 frequencies each
    auto load_tr = [&](int c, auto qc) {
        constexpr int qq = decltype(qc)::value;
        const int p = min(g.sink + c * kChunk + lane, a.rope_len - 1);
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) tr[4 * qq + mm] = a.rope16[long(4 * qq + mm) * a.rope_len + p];
    };
    auto group_of = [](int qq, int i) constexpr {
        return C == 8 ? (i < 2 ? 2 * qq + i : 8 + 2 * qq + (i - 2)) : (i < 4 ? 4 * qq + i : 16 + 4 * qq + (i - 4));
    };
    auto gather = [&](const uint32_t (&ik)[R][IW], auto qc, auto jc, uint32_t (&G)[GQ][GW]) {
        constexpr int qq = decltype(qc)::value, j = decltype(jc)::value;
        StaticFor<0, GQ>::run([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            constexpr int gi = group_of(qq, i);
            const uint32_t off = byte_shl<SH, gi & 3>(ik[j][gi >> 2]);
            const unsigned char* pcw = lds + gi * (K * C * 2) + off;
            if constexpr (C == 8) {
                const uint4 v = *reinterpret_cast<const uint4*>(pcw);
                G[i][0] = v.x; G[i][1] = v.y; G[i][2] = v.z; G[i][3] = v.w;
            } else {
                const uint2 v = *reinterpret_cast<const uint2*>(pcw);
                G[i][0] = v.x; G[i][1] = v.y;
            }
        });
    };
    const_ptr<uint32_t> qrow[R];
    // The packed query rows and the V rows are the same in every item: their base pointers pass through an
    // empty asm at the top of each item, so that their loads stay where they are written instead of being
    // hoisted out of the item loop (which would hold all of them in registers across it).
    auto set_qrow = [&]() {
        const uint32_t* qp = a.qpack;
        asm volatile("" : "+s"(qp));
#pragma unroll
        for (int j = 0; j < R; ++j) qrow[j] = as_const(qp + srow[j] * 64);
    };
    set_qrow();
    auto load_q = [&](auto qc, auto jc, uint32_t (&qs)[16]) {
        constexpr int qq = decltype(qc)::value, j = decltype(jc)::value;
#pragma unroll
        for (int u = 0; u < 16; ++u) qs[u] = qrow[j][16 * qq + u];
    };
    float acc[R][2];
    float rmax[R];
    float sreg[MCH][R];                             // scores of the wave's chunks of the item
    auto compute = [&](auto qc, auto jc, const uint32_t (&G)[GQ][GW], const uint32_t (&qs)[16]) {
        constexpr int qq = decltype(qc)::value, j = decltype(jc)::value;
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {           // RoPE frequencies 4m .. 4m+3
            const int m = 4 * qq + mm;
            const h2_t c01 = as_h2(tr[m].x), c23 = as_h2(tr[m].y);
            const h2_t s01 = as_h2(tr[m].z), s23 = as_h2(tr[m].w);
            const h2_t l01 = as_h2(qs[4 * mm]), l23 = as_h2(qs[4 * mm + 1]);
            const h2_t u01 = as_h2(qs[4 * mm + 2]), u23 = as_h2(qs[4 * mm + 3]);
            const h2_t pl01 = __builtin_elementwise_fma(c01, l01, s01 * u01);
            const h2_t pl23 = __builtin_elementwise_fma(c23, l23, s23 * u23);
            const h2_t ph01 = __builtin_elementwise_fma(c01, u01, -(s01 * l01));
            const h2_t ph23 = __builtin_elementwise_fma(c23, u23, -(s23 * l23));
            uint32_t kl01, kl23, kh01, kh23;
            if constexpr (C == 8) {
                const int il = mm >> 1, d = (mm & 1) * 2;
                kl01 = G[il][d]; kl23 = G[il][d + 1];
                kh01 = G[2 + il][d]; kh23 = G[2 + il][d + 1];
            } else {
                kl01 = G[mm][0]; kl23 = G[mm][1];
                kh01 = G[4 + mm][0]; kh23 = G[4 + mm][1];
            }
            acc[j][0] = dot2h(kl01, pl01, acc[j][0]);
            acc[j][1] = dot2h(kl23, pl23, acc[j][1]);
            acc[j][0] = dot2h(kh01, ph01, acc[j][0]);
            acc[j][1] = dot2h(kh23, ph23, acc[j][1]);
        }
    };
    uint32_t G[2][GQ][GW];
    uint32_t qs[2][16];
    // Chunk slot I of N in the item (chunk c): steps k = (qq, j); the last step issues the cos/sin of the
    // first quarter of the wave's next chunk cn and, but in the item's last slot, its first gathers (from
    // ikn) and query quarter.  (The item's end starts the next item's gathers afresh, so that they are not
    // held in registers through the weights and the contraction.)
    auto run_chunk = [&](auto Ic, auto Nc, int c, int cn, const uint32_t (&ikc)[R][IW],
                         const uint32_t (&ikn)[R][IW]) {
        constexpr int I = decltype(Ic)::value, N = decltype(Nc)::value;
        StaticFor<0, NSTEP>::run([&](auto kc) {
            constexpr int k = decltype(kc)::value, qq = k / R, j = k % R, b = k & 1;
            constexpr int k1 = (k + 1) % NSTEP;
            using QN = std::integral_constant<int, k1 / R>;
            using JN = std::integral_constant<int, k1 % R>;
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0): this step's gathers and query quarter
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (k + 1 < NSTEP) gather(ikc, QN{}, JN{}, G[b ^ 1]);
            else if constexpr (I + 1 < N) gather(ikn, QN{}, JN{}, G[b ^ 1]);
            if constexpr (k + 1 < NSTEP || I + 1 < N) load_q(QN{}, JN{}, qs[b ^ 1]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (j == 0) load_tr(qq < 3 ? c : cn, std::integral_constant<int, (qq + 1) % 4>{});
            compute(std::integral_constant<int, qq>{}, std::integral_constant<int, j>{}, G[b], qs[b]);
            if constexpr (qq == 3) {
                const bool in = in_req(j, c * kChunk + lane);
                const float s_all = acc[j][0] + acc[j][1];
                acc[j][0] = 0.f;
                acc[j][1] = 0.f;
                sreg[I][j] = s_all;
                rmax[j] = fmaxf(rmax[j], in ? s_all : -INFINITY);
            }
        });
    };

    uint32_t ik[3][R][IW];                          // key index rows of slot I in ik[I % (N even ? 2 : 3)]
    if (t_hi > 0) {
        load_idx(cbase, 0, pidc[0], ik[0]);
        load_tr(cbase, std::integral_constant<int, 0>{});
    }
    __syncthreads();                                // K slice staged, query rows packed

    // ---- window: the first NWW waves attend it while the others start on the first item (the first waves
    // of a workgroup get the issue slots first when both of a SIMD's waves are ready, and run their score
    // loop about twice as fast).  Window row wr = tid >> 4 of 16 lanes takes tokens of request wj spaced
    // RPJ apart; every row of a wave serves the same request.  The rows' results wait in registers until
    // after the last item.
    const int c16 = tid & 15, wr = tid >> 4;
    float wm = -INFINITY, wl = 0.f, wo[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) wo[u] = 0.f;
    if (wave < NWW) {
        const int wj = wave * 4 / RPJ;
        const int wrb = group_request(a, r0 + wj);
        window_row(a, min(wrb, a.B - 1), h, wrb < a.B, wr % RPJ, RPJ, c16, wm, wl, wo);
    }

    // Running merge of this thread's output element (request j, channel d), in log2 units: each item, then
    // the window.  m = -inf: nothing yet.
    const int oj = tid / D, od = tid % D;
    float run_m = -INFINITY, run_l = 0.f, run_o = 0.f;
#pragma unroll
    for (int j = 0; j < R; ++j) acc[j][0] = acc[j][1] = 0.f;

    const float fix_scale = float(1u << a.fix_bits);
    const uint16_t* vsl = static_cast<const uint16_t*>(a.slice_v) + h * a.slice_hstride;
    const int n_items = (t_hi + kItemTok - 1) / kItemTok;
    auto item_loop = [&](auto Nc) {
      constexpr int N = decltype(Nc)::value;        // chunk slots of this wave
      int c = cbase;                                // the wave's chunk in slot 0 of the item
      for (int it = 0; it < n_items; ++it, c += CPI) {
        // Values that are the same in every item pass through empty asm here, so that the addresses
        // derived from them are formed where they are used instead of being hoisted out of the loop
        // and held in registers through the score phase.
        set_qrow();
        long vofs = 0;                              // (an integer, so that the loads stay global ones)
        asm volatile("" : "+s"(vofs));
        const uint16_t* vsl_it = vsl + vofs;
        int tid_it = tid;
        asm volatile("" : "+v"(tid_it));
        const int cb_blk = tid_it >> 4, g16 = tid_it & 15;
        // ---- scores ----
        gather(ik[0], std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, G[0]);
        load_q(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, qs[0]);
        uint32_t pidn[N][R];                        // page ids of the next item's chunks
#pragma unroll
        for (int i = 0; i < N; ++i) load_pid(c + CPI + 4 * i, pidn[i]);
#pragma unroll
        for (int j = 0; j < R; ++j) rmax[j] = -INFINITY;
        StaticFor<0, N>::run([&](auto Ic) {
            constexpr int I = decltype(Ic)::value, NB = N % 2 == 0 ? 2 : 3;
            auto& cur = ik[I % NB];
            auto& nxt = ik[(I + 1) % NB];           // (after the last slot: ik[0], the next item's first)
            if constexpr (I + 1 < N) load_idx(c + 4 * (I + 1), 0, pidc[I + 1], nxt);
            else load_idx(c + CPI, 0, pidn[0], nxt);
            run_chunk(Ic, Nc, c + 4 * I, I + 1 < N ? c + 4 * (I + 1) : c + CPI, cur, nxt);
        });
        uint32_t iv[N][R][IW];                      // value index rows of the item's chunks
#pragma unroll
        for (int i = 0; i < N; ++i) load_idx(c + 4 * i, 1, pidc[i], iv[i]);
        // (Stores in this loop come from all lanes of a wave, with the same value where they meet: a
        // lane-divergent branch here costs the score phase its registers.)
#pragma unroll
        for (int j = 0; j < R; ++j) wmax[wave][j] = wave_max_dpp(rmax[j]);
        __syncthreads();                            // wave maxima visible
        float M[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            M[j] = wmax[0][j];
#pragma unroll
            for (int w = 1; w < NW; ++w) M[j] = fmaxf(M[j], wmax[w][j]);
        }

        // ---- weights: one atomic per (token, request, value group) ----
        uint4 vrow[GPL * VPG];                      // V rows of this lane's contraction block (L2 hits)
        StaticFor<0, N>::run([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (i == N - 1) {             // issued once the first chunks' index rows are dead
#pragma unroll
                for (int k = 0; k < GPL; ++k) {
                    const uint4* src =
                        reinterpret_cast<const uint4*>(vsl_it + (long(g16 + 16 * k) * K + CPB * cb_blk) * C);
#pragma unroll
                    for (int v = 0; v < VPG; ++v) vrow[k * VPG + v] = src[v];
                }
            }
            const int tau = (c + 4 * i) * kChunk + lane;
            // byte k of base2[v]: slot byte offset 4R * ((2v + k) ^ (tau & 15)) of the group held in V index
            // byte 2v + k; byte 2: the bins' 64K page
            const uint32_t rot = (uint32_t(tau) & 15u) * (4u * R) * 0x0101u;
            uint32_t base2[NG / 2];
#pragma unroll
            for (int v = 0; v < NG / 2; ++v) base2[v] = (((4u * R) * (0x0100u + uint32_t(v) * 0x0202u)) ^ rot) | 0x10000u;
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const uint32_t u = in_req(j, tau)
                                       ? uint32_t(fmaf(__builtin_amdgcn_exp2f(sreg[i][j] - M[j]), fix_scale, 0.5f))
                                       : 0u;
                StaticFor<0, NG>::run([&](auto mc) {
                    constexpr int m = decltype(mc)::value;
                    // bin byte address [slot offset, codeword, 0x01, 0]: row = codeword, 256 B per row
                    constexpr uint32_t sel = 0x0c020000u | (uint32_t(4 + (m & 3)) << 8) | uint32_t(m & 1);
                    const uint32_t addr = __builtin_amdgcn_perm(iv[i][j][m >> 2], base2[m >> 1], sel);
                    uint32_t* bin = static_cast<uint32_t*>(__builtin_assume_aligned(lds + addr + 4 * j, 4));
                    __hip_atomic_fetch_add(bin, u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                });
            }
        });
        __syncthreads();                            // bins complete

        // ---- contraction: lane (cb_blk, g16) over codewords CPB*cb_blk .. +CPB-1 of its groups ----
        float o[PL];
#pragma unroll
        for (int i = 0; i < PL; ++i) o[i] = 0.f;
        uint32_t lsum[R];
#pragma unroll
        for (int j = 0; j < R; ++j) lsum[j] = 0u;
#pragma unroll
        for (int i = 0; i < CPB; ++i) {
            const int r = CPB * cb_blk + i;
#pragma unroll
            for (int k = 0; k < GPL; ++k) {
                uint32_t bv[R];
                uint32_t* bp = bins + r * 64 + (g16 + 16 * k) * R;
                if constexpr (R == 4) {
                    const uint4 b4 = *reinterpret_cast<const uint4*>(bp);
                    bv[0] = b4.x; bv[1] = b4.y; bv[2] = b4.z; bv[3] = b4.w;
                    *reinterpret_cast<uint4*>(bp) = make_uint4(0u, 0u, 0u, 0u);
                } else {
                    const uint2 b2 = *reinterpret_cast<const uint2*>(bp);
                    bv[0] = b2.x; bv[1] = b2.y;
                    *reinterpret_cast<uint2*>(bp) = make_uint2(0u, 0u);
                }
                uint32_t vw[C / 2];                 // V row: C bf16 of codeword r, group g16 + 16k
                if constexpr (C == 8) {
                    vw[0] = vrow[i].x; vw[1] = vrow[i].y; vw[2] = vrow[i].z; vw[3] = vrow[i].w;
                } else {
                    const uint4 q = vrow[k * VPG + (i >> 1)];
                    vw[0] = (i & 1) ? q.z : q.x;
                    vw[1] = (i & 1) ? q.w : q.y;
                }
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    if (k == 0) lsum[j] += bv[j];
                    const float bw = float(bv[j]);
#pragma unroll
                    for (int u = 0; u < C / 2; ++u) {
                        o[j * C * GPL + k * C + 2 * u] = fmaf(bw, bf16_lo(vw[u]), o[j * C * GPL + k * C + 2 * u]);
                        o[j * C * GPL + k * C + 2 * u + 1] =
                            fmaf(bw, bf16_hi(vw[u]), o[j * C * GPL + k * C + 2 * u + 1]);
                    }
                }
            }
        }
        // sum over the wave's four codeword blocks; row 0 of the wave writes the wave's partials
#pragma unroll
        for (int i = 0; i < PL; ++i) o[i] = sum_rows4(o[i]);
#pragma unroll
        for (int j = 0; j < R; ++j) lsum[j] = sum_rows4(lsum[j]);
        {   // the four rows of the wave hold the same sums: they write them to the same place
            float4* dst = reinterpret_cast<float4*>(part + (wave * 16 + g16) * PL);
#pragma unroll
            for (int i = 0; i < PL / 4; ++i) dst[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
#pragma unroll
            for (int j = 0; j < R; ++j) lw[wave][j] = __builtin_amdgcn_readlane(lsum[j], 0);   // group 0's total
        }
        __syncthreads();                            // partials complete

        // ---- merge the item into the running output element ----
        if (wave < R * D / 64) {
            const int gr = od / C, u = od % C;
            const int p = oj * C * GPL + (gr >> 4) * C + u;
            float U = 0.f;
            uint64_t Ls = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                U += part[(w * 16 + (gr & 15)) * PL + p];
                Ls += lw[w][oj];
            }
            float Mo = M[0];
#pragma unroll
            for (int j = 1; j < R; ++j) Mo = oj == j ? M[j] : Mo;
            if (Ls > 0) {
                const float e = Mo - float(a.fix_bits);     // the item's weights are 2^(s - e) in fixed point
                const float mn = fmaxf(run_m, e);
                const float sa = exp2f(run_m - mn), sb = exp2f(e - mn);
                run_o = fmaf(run_o, sa, U * sb);
                run_l = fmaf(run_l, sa, float(Ls) * sb);
                run_m = mn;
            }
        }
#pragma unroll
        for (int i = 0; i < N; ++i)
#pragma unroll
            for (int j = 0; j < R; ++j) pidc[i][j] = pidn[i][j];
      }
    };
    if constexpr (FCH == SCH) item_loop(std::integral_constant<int, FCH>{});
    else if (fast) item_loop(std::integral_constant<int, FCH>{});
    else item_loop(std::integral_constant<int, SCH>{});

    // ---- the window rows, merged like an item ----
    __syncthreads();                                // the last item's partials are read
    if (wave < NWW) {
        *reinterpret_cast<float4*>(part + wr * D + window_channel(c16, 0)) = make_float4(wo[0], wo[1], wo[2], wo[3]);
        *reinterpret_cast<float4*>(part + wr * D + window_channel(c16, 4)) = make_float4(wo[4], wo[5], wo[6], wo[7]);
        wml[wr][0] = wm;                            // (the row's 16 lanes hold the same m and l)
        wml[wr][1] = wl;
    }
    __syncthreads();
    if (wave < R * D / 64) {
        float mw = -INFINITY;
#pragma unroll
        for (int r = 0; r < RPJ; ++r) mw = fmaxf(mw, wml[oj * RPJ + r][0]);
        if (mw != -INFINITY) {
            float lw_ = 0.f, ow = 0.f;
#pragma unroll
            for (int r = 0; r < RPJ; ++r) {
                const float f = exp2f(wml[oj * RPJ + r][0] - mw);   // 0 for a row without tokens
                lw_ = fmaf(wml[oj * RPJ + r][1], f, lw_);
                ow = fmaf(part[(oj * RPJ + r) * D + od], f, ow);
            }
            const float mn = fmaxf(run_m, mw);
            const float sa = exp2f(run_m - mn), sb = exp2f(mw - mn);
            run_o = fmaf(run_o, sa, ow * sb);
            run_l = fmaf(run_l, sa, lw_ * sb);
            run_m = mn;
        }
    }

    // ---- output: a request holds at least one token, so run_l > 0 ----
    const int orb = group_request(a, r0 + min(oj, R - 1));
    if (tid < R * D && orb < a.B) {
        const long row = long(orb) * g.H + h;
        out[row * D + od] = run_o / run_l;
        if (lse_out && od == 0) lse_out[row] = (run_m + log2f(run_l)) * kLn2;
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


int max_index_pages(const Geo& g, int max_len) { return std::max(0, (max_len - g.sink - g.W) / g.page); }

// Requests per workgroup of the bf16 index-page kernel (R * NG = 64 bin slots).
int reqs_per_wg(const Geo& g) { return g.c == 8 ? 4 : 2; }

int choose_splits(const Geo& g, int B, int max_len) {
    const int max_pages = max_index_pages(g, max_len);
    if (max_pages == 0) return 1;
    // Splits of at most 192 pages (1536 tokens): a wave's scores fit its registers and the fixed-point
    // softmax weights keep 21 fraction bits.
    int s = ceil_div(max_pages, kMaxSplitTok / g.page);
    // Enough (split, head, request group) workgroups for 256 CUs x 2, splits of >= 16 pages.
    const int pairs = ceil_div(B, reqs_per_wg(g)) * g.H;
    s = std::max(s, std::min(ceil_div(512, std::max(1, pairs)), ceil_div(max_pages, 16)));
    return std::max(1, std::min(s, 1024));
}

// Pages per split: a multiple of 8 (64 tokens), so that score chunks never straddle splits.
int pages_per_split(int max_pages, int S) { return max_pages > 0 ? ceil_div(ceil_div(max_pages, S), 8) * 8 : 8; }

// Scratch of the index-page partial (bf16 codebooks): the packed query rows, 256 B per (request, head).
size_t quant_scratch_bytes(const Geo& g, int B) { return size_t(B) * g.H * 64 * sizeof(uint32_t); }

// Bytes of the partials (part_o, part_lse) of S_tot slots per row, rounded up to 256 so that the
// scratch after them starts on a whole cache line.
size_t partials_bytes(const Geo& g, int B, int S_tot) {
    const size_t rows = size_t(B) * g.H * S_tot;
    return (rows * (g.D + 1) * sizeof(float) + 255) / 256 * 256;
}

// A split count the bf16 index-page partial can run: splits of at most kMaxSplitTok tokens.
bool splits_fit(const Geo& g, int max_pages, int S) {
    return g.cb != LVQ_BF16 || max_pages == 0 || pages_per_split(max_pages, S) * g.page <= kMaxSplitTok;
}

int ceil_log2(long x) {
    int r = 0;
    while ((1L << r) < x) ++r;
    return r;
}

}  // namespace
}  // namespace lvq

using namespace lvq;

extern "C" size_t lvq_decode_attn_workspace(const lvq_geom* gp, int32_t B, int32_t max_len, int32_t num_splits) {
    Geo g;
    if (validate_geom(gp, &g) != LVQ_OK || B < 0 || max_len < 0 || num_splits < -1) return 0;
    if (num_splits == -1) return quant_scratch_bytes(g, B);   // the single-pass kernel
    const int S = num_splits > 0 ? num_splits : choose_splits(g, B, max_len);
    return partials_bytes(g, B, S + 1) + quant_scratch_bytes(g, B);
}

extern "C" size_t lvq_quant_partial_workspace(const lvq_geom* gp, int32_t B, int32_t max_len) {
    Geo g;
    if (validate_geom(gp, &g) != LVQ_OK || B < 0 || max_len < 0) return 0;
    return quant_scratch_bytes(g, B);
}

namespace lvq {
namespace {

// Checks shared by the attention entry points; fills the kernel arguments
// except the partial buffers.
lvq_status prepare(const char* fn, const lvq_geom* gp, int32_t step, const void* q, const int32_t* seq_len,
                   int32_t max_len, const float* rope_cos, const float* rope_sin, const void* rope_f16,
                   int32_t rope_len, float sm_scale, int32_t B, AttnArgs* a, bool need_f16 = true) {
    Geo& g = a->geo;
    lvq_status st = validate_geom(gp, &g);
    if (st != LVQ_OK) return st;
    LVQ_REQUIRE(step >= 0 && step < g.T, LVQ_ERR_INVALID_ARG, "%s: step %d out of [0,%d)", fn, step, g.T);
    LVQ_REQUIRE(B >= 0 && max_len >= 1, LVQ_ERR_INVALID_ARG, "%s: bad sizes B=%d max_len=%d", fn, B, max_len);
    LVQ_REQUIRE(max_len <= rope_len, LVQ_ERR_INVALID_ARG, "%s: max_len %d exceeds rope_len %d", fn, max_len,
                rope_len);
    LVQ_REQUIRE(std::isfinite(sm_scale), LVQ_ERR_INVALID_ARG, "%s: sm_scale not finite", fn);
    LVQ_REQUIRE(B <= 65535, LVQ_ERR_UNSUPPORTED, "%s: batch too large", fn);
    LVQ_REQUIRE(B == 0 || (q && seq_len && rope_cos && rope_sin), LVQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    LVQ_REQUIRE(B == 0 || !need_f16 || g.cb != LVQ_BF16 || rope_f16, LVQ_ERR_INVALID_ARG,
                "%s: bf16 codebooks need the packed fp16 RoPE table", fn);
    a->step = step;
    a->beta = step / g.Tc;
    a->q = static_cast<const uint16_t*>(q);
    a->seq_len = seq_len;
    a->rc = rope_cos;
    a->rs = rope_sin;
    a->rope16 = static_cast<const uint4*>(rope_f16);
    a->scale_log2 = sm_scale * kLog2e;
    a->B = B;
    a->max_len = max_len;
    a->rope_len = rope_len;
    return LVQ_OK;
}

// Launches the index-page partial; `scratch` (256-byte aligned) holds the packed query rows.
lvq_status launch_quant(AttnArgs& a, void* scratch, hipStream_t stream) {
    const Geo& g = a.geo;
    if (g.cb == LVQ_BF16) {
        a.qpack = static_cast<const uint32_t*>(scratch);
        a.fix_bits = 32 - ceil_log2(long(a.pps) * g.page + 1);
        const int R = reqs_per_wg(g);
        const dim3 grid(g.H, a.num_splits, ceil_div(a.B, R));
        if (g.c == 8) {
            if (a.kscale) hipLaunchKernelGGL((index_attn_kernel<8, 4, true>), grid, dim3(kIThreads), 0, stream, a);
            else hipLaunchKernelGGL((index_attn_kernel<8, 4, false>), grid, dim3(kIThreads), 0, stream, a);
        } else {
            if (a.kscale) hipLaunchKernelGGL((index_attn_kernel<4, 2, true>), grid, dim3(kIThreads), 0, stream, a);
            else hipLaunchKernelGGL((index_attn_kernel<4, 2, false>), grid, dim3(kIThreads), 0, stream, a);
        }
    } else {
        const dim3 grid(a.num_splits, g.H, (a.B + 1) / 2);
        const size_t red_bytes = 4 * (g.D + 2) * sizeof(float);
        if (g.c == 8)
            hipLaunchKernelGGL((quant_partial_kernel<8, float, false>), grid, dim3(256), red_bytes, stream, a);
        else
            hipLaunchKernelGGL((quant_partial_kernel<4, float, false>), grid, dim3(256), red_bytes, stream, a);
    }
    return check_launch("quantized partial");
}

// Whether the library's choice for lvq_decode_attn is the single-pass kernel.  (Not yet: it runs no faster
// than the split path on the shapes measured so far, so num_splits = 0 keeps the split path.)
bool use_full(const Geo& g, int B, int max_pages) {
    (void)g, (void)B, (void)max_pages;
    return false;
}

// The single-pass kernel; `scratch` (256-byte aligned) holds the packed query rows.
lvq_status launch_full(AttnArgs& a, void* scratch, float* out, float* lse_out, hipStream_t stream) {
    const Geo& g = a.geo;
    a.qpack = static_cast<const uint32_t*>(scratch);
    a.fix_bits = 32 - ceil_log2(long(kItemTok) + 1);
    const dim3 grid(g.H, ceil_div(a.B, reqs_per_wg(g)));
    if (g.c == 8)
        hipLaunchKernelGGL((index_full_kernel<8, 4>), grid, dim3(kFThreads), 0, stream, a, out, lse_out);
    else
        hipLaunchKernelGGL((index_full_kernel<4, 2>), grid, dim3(kFThreads), 0, stream, a, out, lse_out);
    return check_launch("single-pass attention");
}

// The window partial into slot a.num_splits, or (out != NULL) merged with slots 0 .. a.num_splits-1 into
// the attention output.
lvq_status launch_window(AttnArgs& a, float* out, float* lse_out, hipStream_t stream) {
    if (out)
        hipLaunchKernelGGL(window_kernel<true>, dim3(a.geo.H, a.B), dim3(256), 0, stream, a, out, lse_out);
    else
        hipLaunchKernelGGL(window_kernel<false>, dim3(a.geo.H, a.B), dim3(256), 0, stream, a, nullptr, nullptr);
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
                                        int32_t max_len, const int32_t* order, const void* k_scales,
                                        const void* slices, const float* rope_cos,
                                        const float* rope_sin, const void* rope_f16, int32_t rope_len,
                                        float sm_scale, float* part_o,
                                        float* part_lse, int32_t num_splits, int32_t S_tot, void* ws,
                                        size_t ws_bytes, int32_t B, hipStream_t stream) {
    AttnArgs a{};
    lvq_status st = prepare("lvq_quant_partial", gp, step, q, seq_len, max_len, rope_cos, rope_sin, rope_f16,
                            rope_len, sm_scale, B, &a);
    if (st != LVQ_OK) return st;
    a.order = order;
    a.kscale = static_cast<const uint16_t*>(k_scales);
    const Geo& g = a.geo;
    LVQ_REQUIRE(num_splits >= 1 && num_splits <= 1024 && S_tot >= num_splits, LVQ_ERR_INVALID_ARG,
                "lvq_quant_partial: num_splits %d, S_tot %d", num_splits, S_tot);
    if (B == 0) return LVQ_OK;
    const int max_pages = max_index_pages(g, max_len);
    LVQ_REQUIRE(slices && part_o && part_lse && ws, LVQ_ERR_INVALID_ARG, "lvq_quant_partial: NULL pointer");
    LVQ_REQUIRE(ws_bytes >= lvq_quant_partial_workspace(gp, B, max_len), LVQ_ERR_WORKSPACE,
                "lvq_quant_partial: workspace %zu < %zu bytes", ws_bytes,
                lvq_quant_partial_workspace(gp, B, max_len));
    LVQ_REQUIRE(max_pages == 0 || (pool && page_table), LVQ_ERR_INVALID_ARG,
                "lvq_quant_partial: NULL pool or page table");
    LVQ_REQUIRE(pt_stride >= max_pages, LVQ_ERR_INVALID_ARG, "lvq_quant_partial: pt_stride %d < %d pages",
                pt_stride, max_pages);
    LVQ_REQUIRE(splits_fit(g, max_pages, num_splits), LVQ_ERR_INVALID_ARG,
                "lvq_quant_partial: %d splits of %d index pages exceed %d tokens per split", num_splits, max_pages,
                kMaxSplitTok);
    LVQ_REQUIRE(reinterpret_cast<uintptr_t>(ws) % 256 == 0, LVQ_ERR_INVALID_ARG,
                "lvq_quant_partial: workspace not 256-byte aligned");
    a.pool = pool;
    a.pt = page_table;
    a.pt_stride = pt_stride;
    set_slices(&a, slices);
    a.part_o = part_o;
    a.part_lse = part_lse;
    a.S_tot = S_tot;
    a.num_splits = num_splits;
    a.pps = pages_per_split(max_pages, num_splits);
    return launch_quant(a, ws, stream);
}

extern "C" lvq_status lvq_window_partial(const lvq_geom* gp, int32_t step, const void* q, const int32_t* seq_len,
                                         int32_t max_len, const void* win_k, const void* win_v,
                                         const float* rope_cos, const float* rope_sin, int32_t rope_len,
                                         float sm_scale, float* part_o, float* part_lse, int32_t slot,
                                         int32_t S_tot, int32_t B, hipStream_t stream) {
    AttnArgs a{};
    lvq_status st = prepare("lvq_window_partial", gp, step, q, seq_len, max_len, rope_cos, rope_sin, nullptr,
                            rope_len, sm_scale, B, &a, false);
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
    return launch_window(a, nullptr, nullptr, stream);
}

namespace lvq {

lvq_status decode_attn_impl(const char* fn, const lvq_geom* gp, int32_t step, const void* q, const uint8_t* pool,
                            const int32_t* page_table, int32_t pt_stride, const int32_t* seq_len, int32_t max_len,
                            const int32_t* order, const void* k_scales, const void* win_k, const void* win_v,
                            const void* slices, const float* rope_cos, const float* rope_sin, const void* rope_f16,
                            int32_t rope_len, float sm_scale, float* out, float* lse_out, void* ws, size_t ws_bytes,
                            WorkspaceProvider provider, int32_t num_splits, int32_t B, hipStream_t stream) {
    AttnArgs a{};
    lvq_status st = prepare(fn, gp, step, q, seq_len, max_len, rope_cos, rope_sin, rope_f16, rope_len, sm_scale, B, &a);
    if (st != LVQ_OK) return st;
    a.order = order;
    a.kscale = static_cast<const uint16_t*>(k_scales);
    const Geo& g = a.geo;
    LVQ_REQUIRE(num_splits >= -1 && num_splits <= 1024, LVQ_ERR_INVALID_ARG, "%s: num_splits %d", fn, num_splits);
    LVQ_REQUIRE(num_splits != -1 || !k_scales, LVQ_ERR_UNSUPPORTED,
                "%s: the single-pass kernel (num_splits -1) takes no key scale stream", fn);
    LVQ_REQUIRE(num_splits != -1 || g.cb == LVQ_BF16, LVQ_ERR_UNSUPPORTED,
                "%s: the single-pass kernel (num_splits -1) needs bf16 codebooks", fn);
    LVQ_REQUIRE(pt_stride >= 0, LVQ_ERR_INVALID_ARG, "%s: negative pt_stride", fn);
    if (B == 0) return LVQ_OK;
    LVQ_REQUIRE(win_k && win_v && slices && out, LVQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    const int max_pages = max_index_pages(g, max_len);
    LVQ_REQUIRE(max_pages == 0 || (pool && page_table), LVQ_ERR_INVALID_ARG, "%s: NULL pool or page table", fn);
    LVQ_REQUIRE(pt_stride >= max_pages, LVQ_ERR_INVALID_ARG, "%s: pt_stride %d < %d pages", fn, pt_stride, max_pages);
    const bool single = num_splits == -1 || (num_splits == 0 && !k_scales && use_full(g, B, max_pages));
    const int S = num_splits > 0 ? num_splits : choose_splits(g, B, max_len);
    LVQ_REQUIRE(single || splits_fit(g, max_pages, S), LVQ_ERR_INVALID_ARG,
                "%s: %d splits of %d index pages exceed %d tokens per split", fn, S, max_pages, kMaxSplitTok);
    const size_t need = lvq_decode_attn_workspace(gp, B, max_len, num_splits);
    if (provider && (st = provider(need, &ws, &ws_bytes)) != LVQ_OK) return st;
    LVQ_REQUIRE(ws, LVQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    LVQ_REQUIRE(ws_bytes >= need, LVQ_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
    LVQ_REQUIRE(reinterpret_cast<uintptr_t>(ws) % 256 == 0, LVQ_ERR_INVALID_ARG, "%s: workspace not 256-byte aligned",
                fn);

    a.pool = pool;
    a.pt = page_table;
    a.pt_stride = pt_stride;
    a.wk = static_cast<const uint16_t*>(win_k);
    a.wv = static_cast<const uint16_t*>(win_v);
    set_slices(&a, slices);
    if (single) return launch_full(a, ws, out, lse_out, stream);
    const size_t rows = size_t(B) * g.H * (S + 1);
    a.part_o = static_cast<float*>(ws);
    a.part_lse = a.part_o + rows * g.D;
    a.S_tot = S + 1;
    a.num_splits = S;
    a.pps = pages_per_split(max_pages, S);
    if ((st = launch_quant(a, static_cast<unsigned char*>(ws) + partials_bytes(g, B, S + 1), stream)) != LVQ_OK)
        return st;
    return launch_window(a, out, lse_out, stream);
}

}  // namespace lvq

extern "C" lvq_status lvq_decode_attn(const lvq_geom* gp, int32_t step, const void* q, const uint8_t* pool,
                                      const int32_t* page_table, int32_t pt_stride, const int32_t* seq_len,
                                      int32_t max_len, const int32_t* order, const void* k_scales,
                                      const void* win_k, const void* win_v, const void* slices,
                                      const float* rope_cos, const float* rope_sin, const void* rope_f16,
                                      int32_t rope_len, float sm_scale, float* out, float* lse_out, void* ws,
                                      size_t ws_bytes,
                                      int32_t num_splits, int32_t B, hipStream_t stream) {
    return decode_attn_impl("lvq_decode_attn", gp, step, q, pool, page_table, pt_stride, seq_len, max_len, order,
                            k_scales, win_k, win_v, slices, rope_cos, rope_sin, rope_f16, rope_len, sm_scale, out,
                            lse_out, ws, ws_bytes, nullptr, num_splits, B, stream);
}

extern "C" int32_t lvq_decode_attn_splits(const lvq_geom* gp, int32_t B, int32_t max_len) {
    Geo g;
    if (validate_geom(gp, &g) != LVQ_OK || B < 0 || max_len < 1) return 0;
    if (use_full(g, B, max_index_pages(g, max_len))) return -1;
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

// ---------------------------------------------------------------------------
// Request order for ragged batches: the batch ranked by length, longest first (ties by index), so that
// the requests a workgroup takes together have similar lengths.  Request i's key
// (clamped length << 12) | (4095 - i) is distinct and orders by length, then by index; its rank is the
// number of larger keys.  One workgroup; batches over kOrderMaxB or lengths from 2^20 get the identity.
// ---------------------------------------------------------------------------
namespace lvq {
namespace {
constexpr int kOrderThreads = 1024;
constexpr int kOrderMaxB = 4096;

__global__ void __launch_bounds__(kOrderThreads) request_order_kernel(const int32_t* __restrict__ seq_len, int B,
                                                                       int max_len, int32_t* __restrict__ order) {
    __shared__ __align__(16) uint32_t key[kOrderMaxB];
    const int B4 = (B + 3) & ~3;
    for (int i = threadIdx.x; i < B4; i += kOrderThreads) {
        const int L = i < B ? min(max(seq_len[i], 0), max_len) : 0;
        key[i] = i < B ? (uint32_t(L) << 12) | uint32_t(4095 - i) : 0u;   // padding ranks no request
    }
    __syncthreads();
    for (int i = threadIdx.x; i < B; i += kOrderThreads) {
        const uint32_t ki = key[i];
        int rank = 0;
        for (int k = 0; k < B4; k += 4) {
            const uint4 v = *reinterpret_cast<const uint4*>(key + k);
            rank += int(v.x > ki) + int(v.y > ki) + int(v.z > ki) + int(v.w > ki);
        }
        order[rank] = i;
    }
}

__global__ void identity_order_kernel(int B, int32_t* __restrict__ order) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < B) order[i] = i;
}
}  // namespace
}  // namespace lvq

extern "C" lvq_status lvq_request_order(const int32_t* seq_len, int32_t B, int32_t max_len, int32_t* order,
                                        hipStream_t stream) {
    LVQ_REQUIRE(B >= 0 && max_len >= 1, LVQ_ERR_INVALID_ARG, "lvq_request_order: B=%d max_len=%d", B, max_len);
    if (B == 0) return LVQ_OK;
    LVQ_REQUIRE(seq_len && order, LVQ_ERR_INVALID_ARG, "lvq_request_order: NULL pointer");
    if (B <= kOrderMaxB && max_len < (1 << 20))
        hipLaunchKernelGGL(request_order_kernel, dim3(1), dim3(kOrderThreads), 0, stream, seq_len, B, max_len, order);
    else
        hipLaunchKernelGGL(identity_order_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, B, order);
    return check_launch("lvq_request_order");
}

// ---------------------------------------------------------------------------
// Window append (LoopVQ page, Figure 5: each generated token's bf16 K and V of a loop step go into the
// recent window; the oldest page leaves it for the index pool every 8 tokens).  Position
// p = seq_len[b] - 1 (the caller has counted the new token) goes to window slot p for p < sink, else
// sink + (p - sink) mod (W + page); one 16-byte chunk per thread.
// ---------------------------------------------------------------------------
namespace lvq {
namespace {
__global__ void window_append_kernel(Geo g, int step, const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
                                     uint4* __restrict__ win_k, uint4* __restrict__ win_v,
                                     const int32_t* __restrict__ seq_len, int B, int max_len) {
    constexpr int D = 128, CH = D / 8;              // 16-byte chunks per row
    const long e = long(blockIdx.x) * blockDim.x + threadIdx.x;
    if (e >= long(B) * g.H * CH) return;
    const int ch = int(e % CH), h = int((e / CH) % g.H), b = int(e / (long(CH) * g.H));
    const int p = min(seq_len[b], max_len) - 1;
    if (p < 0) return;
    const int slot = p < g.sink ? p : g.sink + (p - g.sink) % (g.W + g.page);
    const long dst = (((long(b) * g.T + step) * g.H + h) * g.Wcap + slot) * CH + ch;
    const long src = (long(b) * g.H + h) * CH + ch;
    if (k_new) win_k[dst] = k_new[src];
    if (v_new) win_v[dst] = v_new[src];
}
}  // namespace
}  // namespace lvq

extern "C" lvq_status lvq_window_append(const lvq_geom* gp, int32_t step, const void* k_new, const void* v_new,
                                        void* win_k, void* win_v, const int32_t* seq_len, int32_t max_len,
                                        int32_t B, hipStream_t stream) {
    Geo g;
    lvq_status st = validate_geom(gp, &g);
    if (st != LVQ_OK) return st;
    LVQ_REQUIRE(step >= 0 && step < g.T, LVQ_ERR_INVALID_ARG, "lvq_window_append: step %d out of [0,%d)", step, g.T);
    LVQ_REQUIRE(B >= 0 && max_len >= 1, LVQ_ERR_INVALID_ARG, "lvq_window_append: B=%d max_len=%d", B, max_len);
    if (B == 0) return LVQ_OK;
    LVQ_REQUIRE(k_new || v_new, LVQ_ERR_INVALID_ARG, "lvq_window_append: k_new and v_new both NULL");
    LVQ_REQUIRE((!k_new || win_k) && (!v_new || win_v) && seq_len, LVQ_ERR_INVALID_ARG,
                "lvq_window_append: NULL window or seq_len");
    const bool aligned = (reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) |
                          reinterpret_cast<uintptr_t>(win_k) | reinterpret_cast<uintptr_t>(win_v)) % 16 == 0;
    LVQ_REQUIRE(aligned, LVQ_ERR_INVALID_ARG, "lvq_window_append: buffers must be 16-byte aligned");
    const long n = long(B) * g.H * (g.D / 8);
    hipLaunchKernelGGL(window_append_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, g, step,
                       static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new), static_cast<uint4*>(win_k),
                       static_cast<uint4*>(win_v), seq_len, int(B), int(max_len));
    return check_launch("lvq_window_append");
}
