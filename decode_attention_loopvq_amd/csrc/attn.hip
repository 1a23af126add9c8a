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
    const uint4* rope16;        // packed fp16 cos/sin (lvq_rope_table_f16; parts A and B, common.h)
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
// group_request for the R consecutive slots from i0, with the order entries read together (one uniform branch).
template <int R>
__device__ __forceinline__ void group_requests(const AttnArgs& a, int i0, int (&rq)[R]) {
    int r[R];
    if (a.order) {
#pragma unroll
        for (int j = 0; j < R; ++j) r[j] = a.order[min(i0 + j, a.B - 1)];
    } else {
#pragma unroll
        for (int j = 0; j < R; ++j) r[j] = i0 + j;
    }
#pragma unroll
    for (int j = 0; j < R; ++j) rq[j] = i0 + j < a.B && r[j] >= 0 && r[j] < a.B ? r[j] : a.B;
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
            float kA[32], kB[32];
#pragma unroll
            for (int q = 0; q < GPC; ++q) {
                const int ia = krow[index_byte(0, NG, gA + q, tok)], ib = krow[index_byte(0, NG, gB + q, tok)];
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
                const int ia = vrow[index_byte(1, NG, gA + q, tok)], ib = vrow[index_byte(1, NG, gB + q, tok)];
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
// Helpers of the bf16 index-page kernels (index_attn_kernel, index_mfma_kernel; their own comments
// describe them).
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
constexpr int kMaxSplits = 1024;                  // splits per request at most
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
        const int L = clamp_len(a, min(rb, a.B - 1));   // read for every slot, so that the loads issue together
        const int np8 = rb < a.B ? n_index_pages(L, g) * g.page : 0;
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
    const uint4* rope_b = a.rope16 + long(a.rope_len) * 32;   // the table's chunk-major part
    auto load_tr = [&](int c, auto qc) {
        constexpr int qq = decltype(qc)::value;
        const int p = min(g.sink + c * kChunk + lane, a.rope_len - 1);
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) tr[4 * qq + mm] = rope_b[long(4 * qq + mm) * a.rope_len + p];
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
    // The rows are loop-invariant, so the compiler would hoist all 128 dwords out of the chunk loop and
    // park most of them in VGPR lanes (a v_readlane per use); the empty asm keeps each step's 16 loads
    // in the step that issues them.
    auto load_q = [&](auto qc, auto jc, uint32_t (&qs)[16]) {
        constexpr int qq = decltype(qc)::value, j = decltype(jc)::value;
        uint64_t pv = reinterpret_cast<uint64_t>(qrow[j]);
        asm volatile("" : "+s"(pv));
        const const_ptr<uint32_t> p = reinterpret_cast<const_ptr<uint32_t>>(pv);
#pragma unroll
        for (int u = 0; u < 16; ++u) qs[u] = p[16 * qq + u];
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
// Index-page partial for bf16 codebooks with c = 8 (16 index groups per token): the scores on the matrix
// cores.  One workgroup per (head, split, group of R = 4 requests), 256 threads (4 waves), two workgroups
// per CU.  Wave w takes the 16-token blocks w, w + 4, ... of the split for all four requests.
//
// Score of index token t of request r: with psi(p) the query turned back by the key's angle (rotate-half
// pairing, channel i with i + 64, angle p * th_i),
//   psi_i = cos(p th_i) q_i + sin(p th_i) q_{i+64},   psi_{i+64} = cos(p th_i) q_{i+64} - sin(p th_i) q_i,
// q . R(p) k = k . psi(p), and k is the concatenation of the 16 codewords its indices name.  Per block of 16
// tokens and request, four v_mfma_f32_16x16x32_f16 with the gathered codewords as the rows of A (8 channels
// = one group per lane and k-block) and psi as the columns of B give C[row][col] = codeword(row) .
// psi(col) summed over the 32 k-slots of each MFMA; the diagonal entries, where the row holds the column's
// token, are the scores.  MFMA lane l = (n, kb) = (l & 15, l >> 4) holds row / column n and k-block kb;
// k-slot (kb, m) of token t holds group P(4 kb + m) ^ t (the key-row byte layout, lvq.h), so that
//  - lanes n = 0..15 of one k-block gather 16 distinct groups: with the step's K slice in LDS as fp16,
//    codeword-major (row r of 256 bytes holds the 16 groups' codewords r), a 16-lane LDS phase reads 16
//    distinct 16-byte columns, conflict-free;
//  - lane (n, kb) holds for every m the 4 index bytes of dword kb of its token's key row;
//  - slots m and m + 2 hold RoPE partner groups (x and x ^ 8) of one block of 8 frequencies, so a lane
//    forms psi of both from one set of cos/sin: slot 0 is the lo group for n < 8 and the hi group for
//    n >= 8, and the latter lanes read the packed table's copy with negated sines (qa, qb swapped):
//    psi_m = qa cos + qb sin',  psi_{m+2} = qb cos - qa sin'.
// psi depends only on the position and the request's query, so the lane's query (two blocks of 8
// frequencies, lo and hi halves, as fp16 pairs pre-scaled by sm_scale * log2 e) stays in registers and the
// position's cos/sin (one 64-byte load per lane and block) serve the four requests.  Request j's A rows are
// its tokens permuted (row n holds token n ^ 4j), so that token n's diagonal entry lands in lane
// (n, (n >> 2) ^ j), register n & 3: each lane ends with exactly one score per block, of request
// kb ^ (n >> 2), taken by 15 selects.
//
// Weights: the workgroup's maximum per request; the K slice's LDS becomes bins [256 codewords][64 slots]
// (slot 4 g + r); each lane adds exp2(s - max), in fixed point with fix_bits fraction bits, to the 16 bins of
// its (request, token)'s value indices.  Value row byte i holds group i ^ (t & 15), so the 64 lanes of one
// atomic hit 64 distinct (request, group) slots, i.e. 64 distinct banks.  Each bin address is one v_perm of
// the index dword with a lane constant.
//
// Contraction: o = sum_r bin[g][r] * B_t^V[g][r] / sum of weights, as in the c = 4 kernel.
// ---------------------------------------------------------------------------
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMBlk = 16;                                      // tokens per MFMA block
constexpr int kMBlocksPerWave = kMaxSplitTok / kMBlk / 4 + 3;  // score registers per lane (whole rounds of 4)

__device__ __forceinline__ uint32_t pack_q2(uint32_t w, float sc) {
    const h2_t v = {(_Float16)(bf16_lo(w) * sc), (_Float16)(bf16_hi(w) * sc)};
    return __builtin_bit_cast(uint32_t, v);
}

template <bool KS>
__global__ void __launch_bounds__(kIThreads, 2) index_mfma_kernel(AttnArgs a) {
    constexpr int D = 128, K = 256, NG = 16, C = 8, R = 4, NT = kIThreads, NW = NT / 64;
    constexpr int NB = kMBlocksPerWave;
    constexpr int PL = R * C;                       // partial sums per contraction lane
    __shared__ __align__(16) unsigned char lds[K * 256];
    __shared__ float wmax[NW][R];
    __shared__ __align__(16) float cpart[NW][64][2 * R];   // contraction partials per wave (lane, channel pair)
    __shared__ uint32_t lpart[NW][R];                      // weight totals per wave
    __shared__ __align__(16) uint32_t qf16[R][D / 2];      // query rows as fp16 pairs times sm_scale * log2 e
    // Page ids of the split's pages, grouped by page pair (one 16-token block): entry (P, h, j) holds request
    // j's page 2 P + (h ^ (j >> 1)), so that lane (n, kb), whose row of request j holds token n ^ 4 j (page
    // half (n >> 3) ^ (j >> 1)), finds its four page ids of a block in one 16-byte read at (P, n >> 3).
    __shared__ __align__(16) uint32_t pid_lds[kMaxSplitTok / 16][2][R];
    uint32_t* bins = reinterpret_cast<uint32_t*>(lds);
    const Geo& g = a.geo;
    const int h = blockIdx.x, split = blockIdx.y, r0 = blockIdx.z * R;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, kb = lane >> 4;
    int rq[R];
    group_requests<R>(a, r0, rq);
    // index-token ranges of the requests in this split (8-token pages; every length read, without branches,
    // so that the loads issue together)
    int lo[R], hi[R];
    bool any = false;
    int len[R];
#pragma unroll
    for (int j = 0; j < R; ++j) len[j] = a.seq_len[min(rq[j], a.B - 1)];
    // Loads that need no length are issued before the lengths are waited for: the step's K slice of head h
    // (16-byte chunk e = tid + NT * i is codeword e >> 4 of group e & 15 of the global layout
    // [group][codeword][8]; it goes to LDS byte 16 e = 256 * codeword + 16 * group) and the query element this
    // thread packs (wave w converts request w's row, one dword = two channels per lane, into qf16).  A
    // workgroup without work leaves them unused.
    uint4 stage[16];
    {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.slice_k) +
                                                          h * a.slice_hstride);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int e = tid + NT * i;
            stage[i] = src[(e & 15) * K + (e >> 4)];
        }
    }
    // The split's page-table entries (page ids, per request), also issued before the lengths: a request with
    // work starts its range at the split's first page, so entry pp is page split * pps + pp of its row,
    // clamped to the row (in bounds whatever the lengths); pages past a request's range are replaced by
    // physical page 0 once the lengths are known, so that every pool load below reads valid memory (their
    // tokens are masked).
    constexpr int kPt = R * (kMaxSplitTok / 8) / NT;   // page-table entries per thread
    static_assert(R * (kMaxSplitTok / 8) % NT == 0, "page-table fill");
    uint32_t ptv[kPt];
#pragma unroll
    for (int i = 0; i < kPt; ++i) {
        const int e = tid + NT * i;
        const int j = e / (kMaxSplitTok / 8), pp = e % (kMaxSplitTok / 8);
        int row = min(rq[0], a.B - 1);
#pragma unroll
        for (int jj = 1; jj < R; ++jj)
            if (j == jj) row = min(rq[jj], a.B - 1);
        ptv[i] = uint32_t(a.pt[long(row) * a.pt_stride + min(split * a.pps + pp, a.pt_stride - 1)]);
    }
    static_assert(R * D / 2 == NT, "one query dword per thread");
    int qrow = rq[0];
#pragma unroll
    for (int j = 1; j < R; ++j)
        if (wave == j) qrow = rq[j];
    const uint32_t qraw = reinterpret_cast<const uint32_t*>(a.q + (long(min(qrow, a.B - 1)) * g.H + h) * D)[lane];
    {
        const int split_tok = a.pps * 8;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int L = min(max(len[j], 0), a.max_len);
            const int np8 = rq[j] < a.B ? max(L - g.sink - g.W, 0) & ~7 : 0;
            lo[j] = min(np8, split * split_tok);
            hi[j] = min(np8, (split + 1) * split_tok);
            any |= hi[j] > lo[j];
        }
    }
    if (!any) {
        // (the early loads are consumed on this path too, so that the compiler issues them above the
        // lengths' wait instead of sinking them below this branch)
#pragma unroll
        for (int i = 0; i < 16; ++i) asm volatile("" ::"v"(stage[i].x));
#pragma unroll
        for (int i = 0; i < kPt; ++i) asm volatile("" ::"v"(ptv[i]));
        asm volatile("" ::"v"(qraw));
        for (int e = tid; e < R * D; e += NT) {
            const int j = e / D, d = e % D, rb = rq[j];
            if (rb >= a.B) continue;
            const long row = (long(rb) * g.H + h) * a.S_tot + split;
            a.part_o[row * D + d] = 0.f;
            if (d == 0) a.part_lse[row] = -INFINITY;
        }
        return;
    }
    int t_lo = 0x7fffffff, t_hi = 0;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (hi[j] > lo[j]) {
            t_lo = min(t_lo, lo[j]);
            t_hi = max(t_hi, hi[j]);
        }
    }
    // page ids past each request's range (its index tokens end at hi[j]) -> physical page 0
#pragma unroll
    for (int i = 0; i < kPt; ++i) {
        const int e = tid + NT * i;
        const int j = e / (kMaxSplitTok / 8), pp = e % (kMaxSplitTok / 8);
        int hij = hi[0];
#pragma unroll
        for (int jj = 1; jj < R; ++jj)
            if (j == jj) hij = hi[jj];
        if (8 * (split * a.pps + pp) >= hij) ptv[i] = 0u;
    }
    // The lane's query: blocks f1 = ((2 kb) ^ n) & 7 and f2 = f1 ^ 1 of 8 frequencies, qa = the half of
    // slot 0's group, qb the partner half (read from qf16 once the first score loads are issued).
    const int hl = (n >> 3) & 1;
    const int f1 = ((2 * kb) ^ n) & 7;
    uint32_t qa[R][2][4], qb[R][2][4];
#pragma unroll
    for (int i = 0; i < kPt; ++i) {
        const int e = tid + NT * i;
        const int j = e / (kMaxSplitTok / 8), pp = e % (kMaxSplitTok / 8);
        pid_lds[pp >> 1][(pp & 1) ^ (j >> 1)][j] = ptv[i];
    }
    qf16[wave][lane] = pack_q2(qraw, a.scale_log2);
    // Gather address constants: byte j of ck[m] is 16 * (group of key-row byte 4 kb + m of token n ^ 4 j),
    // i.e. 16 * (P(4 kb + m) ^ n ^ 4 j) with P(4 kb + m) = (m & 1) | 2 kb | 8 (m >> 1) (the key-row byte
    // permutation, see index_byte).
    uint32_t ck[4];
    {
        const uint32_t c0 = (uint32_t(16 * ((2 * kb) ^ n)) * 0x01010101u) ^ 0xC0804000u;
#pragma unroll
        for (int m = 0; m < 4; ++m) ck[m] = c0 ^ (uint32_t(16 * ((m & 1) | ((m >> 1) << 3))) * 0x01010101u);
    }
    // The lane's own (request, token) of every block: request ro = kb ^ (n >> 2), token tau0 + n.
    const int ro = kb ^ (n >> 2);
    // bits 0, 1 of ro and of n for the score selects, hidden from the optimiser so that the selects stay a
    // tree of 15 rather than becoming a dynamic register index
    auto opaque_bit = [](int x, int bit) { asm volatile("" : "+v"(x)); return (x & bit) != 0; };
    const bool br0 = opaque_bit(ro, 1), br1 = opaque_bit(ro, 2), bn0 = opaque_bit(n, 1), bn1 = opaque_bit(n, 2);
    int lo_o = lo[0], hi_o = hi[0];
#pragma unroll
    for (int j = 1; j < R; ++j)
        if (ro == j) { lo_o = lo[j]; hi_o = hi[j]; }

    const uint32_t page_bytes = uint32_t(g.page_bytes);
    const unsigned char* slab = a.pool + (long(a.beta) * g.H + h) * 2 * 8 * NG;   // (block, head) K rows of page 0
    const uint4* rope = a.rope16;
    const int nblk = (t_hi - t_lo + kMBlk - 1) / kMBlk;   // blocks of the workgroup
    const int nk = wave < nblk ? (nblk - wave + NW - 1) / NW : 0;   // blocks of this wave: wave + NW k, k < nk
    // Loads never branch: a block past the end is clamped to the last one.
    auto tau0_of = [&](int k) { return t_lo + kMBlk * min(wave + NW * k, nblk - 1); };
    // Per-lane parts of the load addresses (blocks start at multiples of 16 tokens, so token n ^ 4 j of a
    // block sits in page (tau0 - t_lo) / 8 + ((n ^ 4 j) >> 3) at row (n ^ 4 j) & 7).
    // page id of request j's page `page` (relative to the split's first)
    auto pid_of = [&](int j, int page) { return pid_lds[page >> 1][(page & 1) ^ (j >> 1)][j]; };
    const unsigned char* kbase[R];                  // dword kb of that row in page 0's (block, head) K rows
#pragma unroll
    for (int j = 0; j < R; ++j) kbase[j] = slab + ((n ^ (4 * j)) & 7) * NG + 4 * kb;
    const uint4* rope_l1 = rope + 16 * hl + 2 * f1;          // the lane's cos/sin chunks at position 0
    const uint4* rope_l2 = rope + 16 * hl + 2 * (f1 ^ 1);
    // the lane's four page ids of the wave's k-th block (request j's in component j)
    auto read_pids = [&](int k) {
        return *reinterpret_cast<const uint4*>(&pid_lds[(tau0_of(k) - t_lo) >> 4][n >> 3][0]);
    };
    // key-row dwords of a block from its page ids: dword kb of token n ^ 4 j of request j; with a key scale
    // stream (KS) also the scale of the lane's own (request ro, token n), whose page is request ro's entry of
    // the page half n >> 3: the lane's own for ro < 2, else the one lane n ^ 8 holds for its request ro ^ 2
    // (brought by a row rotation), so that no LDS read waits in the score loop.  The scale stays fp16 bits
    // until its block is scored: converting it here would wait for the load at once.
    auto issue_ik = [&](const uint4& pd, uint32_t (&ik)[R], uint32_t& ksv) {
        const uint32_t pid[R] = {pd.x, pd.y, pd.z, pd.w};
#pragma unroll
        for (int j = 0; j < R; ++j)
            ik[j] = *reinterpret_cast<const uint32_t*>(kbase[j] + uint64_t(pid[j]) * page_bytes);
        if constexpr (KS) {
            const uint32_t x01 = br0 ? pd.y : pd.x, x23 = br0 ? pd.w : pd.z;
            const uint32_t own = br1 ? x23 : x01, other = br1 ? x01 : x23;   // requests ro and ro ^ 2
            const uint32_t rot = uint32_t(__builtin_amdgcn_update_dpp(int(other), int(other), 0x128, 0xf, 0xf, false));
            const uint32_t pid_own = br1 ? rot : own;                          // row_ror:8, from lane n ^ 8
            ksv = a.kscale[(uint64_t(pid_own) * g.T + a.step) * 8 + (n & 7)];
        }
    };
    auto load_ik = [&](int k, uint32_t (&ik)[R], uint32_t& ksv) { issue_ik(read_pids(k), ik, ksv); };
    // cos/sin chunks of the lane's token (block f1: 2, block f2: 2)
    struct CsBuf { uint4 cs[4]; };
    auto load_cs = [&](int k, CsBuf& b) {
        const int tau0 = tau0_of(k);
        const uint32_t p = uint32_t(min(g.sink + tau0 + n, a.rope_len - 1));
        const uint4* r1 = rope_l1 + uint64_t(p) * 32;
        const uint4* r2 = rope_l2 + uint64_t(p) * 32;
        b.cs[0] = r1[0];
        b.cs[1] = r1[1];
        b.cs[2] = r2[0];
        b.cs[3] = r2[1];
    };
    float sreg[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) sreg[i] = -INFINITY;
    float rmax = -INFINITY;
    // The wave's k-th block: the scores of the four requests, the lane's own kept.
    // Codeword gathers of request j of a block from its key-row dwords (one v_perm and one 16-byte LDS read
    // per MFMA slot).
    auto gather = [&](auto jc, uint32_t ikj, uint4 (&G)[4]) {
        constexpr int j = decltype(jc)::value;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t sel = 0x0c0c0000u | (uint32_t(4 + m) << 8) | uint32_t(j);
            G[m] = *reinterpret_cast<const uint4*>(lds + __builtin_amdgcn_perm(ikj, ck[m], sel));
        }
    };
    // psi of request j times its gathered codewords: the four MFMAs of one accumulator
    auto request_mfma = [&](auto jc, const uint4 (&G)[4], const uint32_t (&c)[2][4], const uint32_t (&s)[2][4]) {
        constexpr int j = decltype(jc)::value;
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int u = m & 1;
            uint32_t psi[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const h2_t cc = as_h2(c[u][q]), ss = as_h2(s[u][q]);
                const h2_t x = as_h2(qa[j][u][q]), y = as_h2(qb[j][u][q]);
                const h2_t v = m < 2 ? __builtin_elementwise_fma(x, cc, y * ss)
                                     : __builtin_elementwise_fma(y, cc, -(x * ss));
                psi[q] = __builtin_bit_cast(uint32_t, v);
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(f16x8_t, G[m]),
                __builtin_bit_cast(f16x8_t, make_uint4(psi[0], psi[1], psi[2], psi[3])), acc, 0, 0, 0);
        }
        return acc;
    };
    using J0 = std::integral_constant<int, 0>;
    using J1 = std::integral_constant<int, 1>;
    using J2 = std::integral_constant<int, 2>;
    using J3 = std::integral_constant<int, 3>;
    // The wave's k-th block: the scores of the four requests, the lane's own kept.  The gathers of request 0
    // arrive in G0 (issued during the block before); each request's gathers are issued one request ahead,
    // and the next block's request 0 into G0 (ikn: its key-row dwords).
    // The loads for later blocks are issued inside: the page ids of block k + 4 before the gathers of request
    // 2 (so that waiting for them never waits for gathers issued after them), block k + 4's key-row dwords into
    // ik once its last gathers are issued, block k + 2's cos/sin into b once psi is formed.
    auto score_blk = [&](int k, uint32_t (&ik)[R], uint32_t& ksv, CsBuf& b, uint4 (&G0)[4],
                         const uint32_t (&ikn)[R]) {
        uint32_t c[2][4], s[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            c[u][0] = b.cs[2 * u].x; c[u][1] = b.cs[2 * u].y; c[u][2] = b.cs[2 * u + 1].x; c[u][3] = b.cs[2 * u + 1].y;
            s[u][0] = b.cs[2 * u].z; s[u][1] = b.cs[2 * u].w; s[u][2] = b.cs[2 * u + 1].z; s[u][3] = b.cs[2 * u + 1].w;
        }
        const uint32_t ks_bits = ksv;                   // (read before the set is reloaded)
        f32x4_t acc[R];
        uint4 G1[4], G2[4], G3[4];
        gather(J1{}, ik[1], G1);
        const uint4 pd = read_pids(k + 4);
        acc[0] = request_mfma(J0{}, G0, c, s);
        gather(J2{}, ik[2], G2);
        acc[1] = request_mfma(J1{}, G1, c, s);
        gather(J3{}, ik[3], G3);
        issue_ik(pd, ik, ksv);
        acc[2] = request_mfma(J2{}, G2, c, s);
        gather(J0{}, ikn[0], G0);
        acc[3] = request_mfma(J3{}, G3, c, s);
        load_cs(k + 2, b);
        // the lane's own score: request ro, register n & 3 of its accumulator (15 selects on the lane bits)
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x01 = br0 ? acc[1][i] : acc[0][i];
            const float x23 = br0 ? acc[3][i] : acc[2][i];
            e[i] = br1 ? x23 : x01;
        }
        const float e01 = bn0 ? e[1] : e[0];
        const float e23 = bn0 ? e[3] : e[2];
        float sc = bn1 ? e23 : e01;
        if constexpr (KS) sc *= f16_to_f32(uint16_t(ks_bits));
        const int tau = t_lo + kMBlk * (wave + NW * k) + n;
        sc = (k < nk && tau >= lo_o && tau < hi_o) ? sc : -INFINITY;
        rmax = fmaxf(rmax, sc);
        sreg[k] = sc;
    };
    __syncthreads();                                      // page ids in LDS
    // key-row dwords four blocks ahead (set k % 4), cos/sin two blocks ahead (set k % 2); each set is reloaded
    // while its block is scored.  The first loads are issued before the K slice is stored to LDS.
    uint32_t IK0[R], IK1[R], IK2[R], IK3[R];
    uint32_t KS0 = 0u, KS1 = 0u, KS2 = 0u, KS3 = 0u;
    CsBuf C0, C1;
    if (nk > 0) {
        load_ik(0, IK0, KS0);
        load_ik(1, IK1, KS1);
        load_ik(2, IK2, KS2);
        load_ik(3, IK3, KS3);
        load_cs(0, C0);
        load_cs(1, C1);
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const uint4 wa = *reinterpret_cast<const uint4*>(&qf16[j][32 * hl + 4 * (f1 ^ s)]);
            const uint4 wb = *reinterpret_cast<const uint4*>(&qf16[j][32 * (hl ^ 1) + 4 * (f1 ^ s)]);
            qa[j][s][0] = wa.x; qa[j][s][1] = wa.y; qa[j][s][2] = wa.z; qa[j][s][3] = wa.w;
            qb[j][s][0] = wb.x; qb[j][s][1] = wb.y; qb[j][s][2] = wb.z; qb[j][s][3] = wb.w;
        }
    }
    {   // K slice, bf16 -> fp16
        uint4* dst = reinterpret_cast<uint4*>(lds);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            dst[tid + NT * i] = make_uint4(bf16x2_to_f16x2(stage[i].x), bf16x2_to_f16x2(stage[i].y),
                                           bf16x2_to_f16x2(stage[i].z), bf16x2_to_f16x2(stage[i].w));
    }
    __syncthreads();                                      // K slice staged
    if (nk > 0) {
        uint4 G0[4];
        gather(J0{}, IK0[0], G0);
        // whole rounds of four blocks: a round's blocks past the wave's last one rescore that block with their
        // scores discarded (the loop has one exit, so the loads in flight are counted across iterations)
        for (int k = 0; k < nk; k += 4) {
            score_blk(k, IK0, KS0, C0, G0, IK1);
            score_blk(k + 1, IK1, KS1, C1, G0, IK2);
            score_blk(k + 2, IK2, KS2, C0, G0, IK3);
            score_blk(k + 3, IK3, KS3, C1, G0, IK0);
        }
    }
    // value rows of the lane's own (request, token) of the wave's k-th block, the first four loaded now
    const unsigned char* vbase = slab + (8 + (n & 7)) * NG;   // the lane's value row in page 0
    auto load_vr = [&](int k) -> uint4 {
        const uint32_t pid = pid_of(ro, ((tau0_of(k) - t_lo) >> 3) + (n >> 3));
        return *reinterpret_cast<const uint4*>(vbase + uint64_t(pid) * page_bytes);
    };
    uint4 VR0 = make_uint4(0u, 0u, 0u, 0u), VR1 = VR0, VR2 = VR0, VR3 = VR0;
    if (nk > 0) {
        VR0 = load_vr(0);
        VR1 = load_vr(1);
        VR2 = load_vr(2);
        VR3 = load_vr(3);
    }

    // ---- weights ----
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const float mw = wave_max_dpp(ro == j ? rmax : -INFINITY);
        if (lane == 0) wmax[wave][j] = mw;
    }
    __syncthreads();                                // every wave is done with the K slice
#pragma unroll
    for (int i = 0; i < K * 64 / 4 / NT; ++i) reinterpret_cast<uint4*>(bins)[tid + i * NT] = make_uint4(0u, 0u, 0u, 0u);
    // V slice dwords of this lane's contraction part, needed once the bins are complete: wave w takes
    // codewords 64 w .. 64 w + 63; lane l = 4 g + q takes dword q (channels 2 q, 2 q + 1) of group g's rows.
    constexpr int kCw = K / NW;
    uint32_t vd[kCw];
    {
        const uint32_t* vsl = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.slice_v) +
                                                                h * a.slice_hstride);
        const uint32_t* src = vsl + ((lane >> 2) * K + kCw * wave) * (C / 2) + (lane & 3);
#pragma unroll
        for (int t = 0; t < kCw; ++t) vd[t] = src[t * (C / 2)];
    }
    __syncthreads();                                // bins cleared, wave maxima visible
    float M[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        M[j] = wmax[0][j];
#pragma unroll
        for (int w = 1; w < NW; ++w) M[j] = fmaxf(M[j], wmax[w][j]);
    }
    float Mo = M[0];
#pragma unroll
    for (int j = 1; j < R; ++j) if (ro == j) Mo = M[j];
    // bin byte offsets of the lane's value-row bytes: byte i of cv[w] = 4 * (4 * ((4 w + i) ^ n) + ro)
    uint32_t cv[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t v = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) v |= uint32_t(4 * (4 * ((4 * w + i) ^ n) + ro)) << (8 * i);
        cv[w] = v;
    }
    const float fix_scale = float(1u << a.fix_bits);
    auto bin_blk = [&](float sc, const uint4& v4) {
        // out-of-range tokens hold -inf: weight 0 (their rows are valid memory, their bins any)
        const uint32_t wgt = sc == -INFINITY ? 0u : uint32_t(fmaf(__builtin_amdgcn_exp2f(sc - Mo), fix_scale, 0.5f));
        const uint32_t vw[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const uint32_t sel = 0x0c0c0000u | (uint32_t(4 + (m & 3)) << 8) | uint32_t(m & 3);
            const uint32_t addr = __builtin_amdgcn_perm(vw[m >> 2], cv[m >> 2], sel);
            uint32_t* bin = static_cast<uint32_t*>(__builtin_assume_aligned(lds + addr, 4));
            __hip_atomic_fetch_add(bin, wgt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    };
    // value rows four blocks ahead (set k % 4); whole rounds of four blocks as above (discarded scores are
    // -inf: weight 0).  A round's scores are read from the (dynamically indexed) score registers at the start
    // of the round before, when the only loads in flight are the value rows that round needs at once.
    float S0 = sreg[0], S1 = sreg[1], S2 = sreg[2], S3 = sreg[3];
    for (int k = 0; k < nk; k += 4) {
        const float N0 = sreg[min(k + 4, NB - 1)], N1 = sreg[min(k + 5, NB - 1)];
        const float N2 = sreg[min(k + 6, NB - 1)], N3 = sreg[min(k + 7, NB - 1)];
        bin_blk(S0, VR0);
        VR0 = load_vr(k + 4);
        bin_blk(S1, VR1);
        VR1 = load_vr(k + 5);
        bin_blk(S2, VR2);
        VR2 = load_vr(k + 6);
        bin_blk(S3, VR3);
        VR3 = load_vr(k + 7);
        S0 = N0; S1 = N1; S2 = N2; S3 = N3;
    }
    __syncthreads();

    // ---- contraction on the matrix cores ----
    // o[r][8 g + c] = sum over codewords w of bin[w][4 g + r] * V_g[w][c]: per group a 4 x 4 block product per
    // channel set, the 16 groups as the 16 blocks of v_mfma_f32_4x4x1_16b_f32 (lane 4 g + i supplies row i of
    // block g's A = the bin of request i, lane 4 g + j column j of its B = channel 2 j (set 0) or 2 j + 1
    // (set 1) of the codeword; register i of lane 4 g + j receives (request i, channel 2 j + set)).  fp32
    // throughout (a bin converts with relative rounding 2^-24).  Lanes 0..3 (group 0) also total the bins of
    // their request in integers: the sum of its weights.
    {
        f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, acc2 = acc0, acc3 = acc0;
        uint32_t lsum = 0u;
        const uint32_t* brow = bins + kCw * wave * 64 + lane;
#pragma unroll
        for (int t = 0; t < kCw; t += 2) {
            const uint32_t u0 = brow[t * 64], u1 = brow[(t + 1) * 64];
            lsum += u0 + u1;
            const float a0 = float(u0), a1 = float(u1);
            acc0 = __builtin_amdgcn_mfma_f32_4x4x1f32(a0, bf16_lo(vd[t]), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_4x4x1f32(a0, bf16_hi(vd[t]), acc1, 0, 0, 0);
            acc2 = __builtin_amdgcn_mfma_f32_4x4x1f32(a1, bf16_lo(vd[t + 1]), acc2, 0, 0, 0);
            acc3 = __builtin_amdgcn_mfma_f32_4x4x1f32(a1, bf16_hi(vd[t + 1]), acc3, 0, 0, 0);
        }
        float4* dst = reinterpret_cast<float4*>(&cpart[wave][lane][0]);
        dst[0] = make_float4(acc0[0] + acc2[0], acc0[1] + acc2[1], acc0[2] + acc2[2], acc0[3] + acc2[3]);
        dst[1] = make_float4(acc1[0] + acc3[0], acc1[1] + acc3[1], acc1[2] + acc3[2], acc1[3] + acc3[3]);
        if (lane < R) lpart[wave][lane] = lsum;
    }
    __syncthreads();
    {
        // thread (l, i): request i, channels 8 (l >> 2) + 2 (l & 3) + {0, 1}
        const int l = tid >> 2, i = tid & 3, rb = rq[i];
        int lo_i = lo[0], hi_i = hi[0];
        float Mi = M[0];
#pragma unroll
        for (int j = 1; j < R; ++j)
            if (i == j) { lo_i = lo[j]; hi_i = hi[j]; Mi = M[j]; }
        if (rb < a.B) {
            const long orow = (long(rb) * g.H + h) * a.S_tot + split;
            const int d = 8 * (l >> 2) + 2 * (l & 3);
            float2* po = reinterpret_cast<float2*>(a.part_o + orow * D + d);
            if (hi_i <= lo_i) {
                *po = make_float2(0.f, 0.f);
                if (d == 0) a.part_lse[orow] = -INFINITY;
            } else {
                float o0 = 0.f, o1 = 0.f;
                uint32_t L = 0u;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    o0 += cpart[w][l][i];
                    o1 += cpart[w][l][R + i];
                    L += lpart[w][i];
                }
                const float Lf = float(L);
                *po = make_float2(o0 / Lf, o1 / Lf);
                if (d == 0) a.part_lse[orow] = (Mi + (log2f(Lf) - float(a.fix_bits))) * kLn2;
            }
        }
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
constexpr int kWinPrefetch = 4;                   // index-page partials loaded at the start of the merge

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
    uint2 qlo, qhi;                                // the lane's query channels (i, then i + 64), bf16 bits: converted
                                                   // once the window loads are issued, not at once after their load
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
    w.qlo = *reinterpret_cast<const uint2*>(qp);
    w.qhi = *reinterpret_cast<const uint2*>(qp + 64);
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
    // the query times sm_scale * log2 e, formed here (an opaque copy keeps the conversion, and so the wait for
    // the query's load, below this batch's loads rather than hoisted above the first batch)
    uint32_t qw[4] = {w.qlo.x, w.qlo.y, w.qhi.x, w.qhi.y};
#pragma unroll
    for (int u = 0; u < 4; ++u) asm volatile("" : "+v"(qw[u]));
    float ql[4], qh[4];
    ql[0] = bf16_lo(qw[0]) * a.scale_log2; ql[1] = bf16_hi(qw[0]) * a.scale_log2;
    ql[2] = bf16_lo(qw[1]) * a.scale_log2; ql[3] = bf16_hi(qw[1]) * a.scale_log2;
    qh[0] = bf16_lo(qw[2]) * a.scale_log2; qh[1] = bf16_hi(qw[2]) * a.scale_log2;
    qh[2] = bf16_lo(qw[3]) * a.scale_log2; qh[3] = bf16_hi(qw[3]) * a.scale_log2;
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
            const float psl = fmaf(ql[u], c4[u], qh[u] * s4[u]);
            const float psh = fmaf(qh[u], c4[u], -(ql[u] * s4[u]));
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
    return std::max(1, std::min(s, kMaxSplits));
}

// Pages per split: a multiple of 8 (64 tokens), so that score chunks never straddle splits.
int pages_per_split(int max_pages, int S) { return max_pages > 0 ? ceil_div(ceil_div(max_pages, S), 8) * 8 : 8; }

// Scratch of the index-page partial (bf16 codebooks): the packed query rows, 256 B per (request, head).
size_t quant_scratch_bytes(const Geo& g, int B) { return size_t(B) * g.H * 64 * sizeof(uint32_t); }

// Bytes of the packed fp16 RoPE table built in the workspace for a call given none (bf16 codebooks),
// positions 0 .. max_len - 1, rounded up to 256.
size_t rope_scratch_bytes(const Geo& g, int max_len) {
    return g.cb == LVQ_BF16 ? (size_t(max_len) * kRopeF16HalvesPerPos * 2 + 255) / 256 * 256 : 0;
}

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
    if (validate_geom(gp, &g) != LVQ_OK || B < 0 || max_len < 0 || num_splits < 0) return 0;
    const int S = num_splits > 0 ? num_splits : choose_splits(g, B, max_len);
    return partials_bytes(g, B, S + 1) + quant_scratch_bytes(g, B) + rope_scratch_bytes(g, max_len);
}

extern "C" size_t lvq_quant_partial_workspace(const lvq_geom* gp, int32_t B, int32_t max_len) {
    Geo g;
    if (validate_geom(gp, &g) != LVQ_OK || B < 0 || max_len < 0) return 0;
    return quant_scratch_bytes(g, B) + rope_scratch_bytes(g, max_len);
}

namespace lvq {
namespace {

// Checks shared by the attention entry points; fills the kernel arguments
// except the partial buffers.
lvq_status prepare(const char* fn, const lvq_geom* gp, int32_t step, const void* q, const int32_t* seq_len,
                   int32_t max_len, const float* rope_cos, const float* rope_sin, const void* rope_f16,
                   int32_t rope_len, float sm_scale, int32_t B, AttnArgs* a) {
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
    a->step = step;
    a->beta = step / g.Tc;
    a->q = static_cast<const uint16_t*>(q);
    a->seq_len = seq_len;
    a->rc = rope_cos;
    a->rs = rope_sin;
    a->rope16 = g.cb == LVQ_BF16 ? static_cast<const uint4*>(rope_f16) : nullptr;
    a->scale_log2 = sm_scale * kLog2e;
    a->B = B;
    a->max_len = max_len;
    a->rope_len = rope_len;
    return LVQ_OK;
}

// The packed fp16 RoPE table (common.h) from the caller's fp32 cos/sin, for a call given none: each value
// rounded once from fp32 to binary16 (which can differ from the fp64 value rounded once, as
// lvq_rope_table_f16 builds it, only where the fp32 value lies on a binary16 rounding midpoint).
__global__ void rope_pack_kernel(const float* __restrict__ rc, const float* __restrict__ rs, int len,
                                 _Float16* __restrict__ out) {
    const long total = long(len) * 64;
    for (long e = blockIdx.x * long(blockDim.x) + threadIdx.x; e < total; e += long(gridDim.x) * blockDim.x)
        store_rope_f16(out, len, e >> 6, int(e & 63), (_Float16)rc[e], (_Float16)rs[e]);
}

// For bf16 codebooks without a packed table: builds one for positions 0 .. max_len - 1 at `table`
// (rope_scratch_bytes) and points the kernels at it.
lvq_status pack_rope_if_needed(AttnArgs& a, void* table, hipStream_t stream) {
    if (a.geo.cb != LVQ_BF16 || a.rope16) return LVQ_OK;
    const long total = long(a.max_len) * 64;
    hipLaunchKernelGGL(rope_pack_kernel, dim3(unsigned(std::min<long>((total + 255) / 256, 2048))), dim3(256), 0,
                       stream, a.rc, a.rs, a.max_len, static_cast<_Float16*>(table));
    a.rope16 = static_cast<const uint4*>(table);
    a.rope_len = a.max_len;
    return check_launch("packed RoPE table");
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
            if (a.kscale) hipLaunchKernelGGL((index_mfma_kernel<true>), grid, dim3(kIThreads), 0, stream, a);
            else hipLaunchKernelGGL((index_mfma_kernel<false>), grid, dim3(kIThreads), 0, stream, a);
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
    LVQ_REQUIRE(num_splits >= 1 && num_splits <= kMaxSplits && S_tot >= num_splits, LVQ_ERR_INVALID_ARG,
                "lvq_quant_partial: num_splits %d, S_tot %d", num_splits, S_tot);
    if (B == 0) return LVQ_OK;
    const int max_pages = max_index_pages(g, max_len);
    LVQ_REQUIRE(slices && part_o && part_lse && ws, LVQ_ERR_INVALID_ARG, "lvq_quant_partial: NULL pointer");
    const size_t need = quant_scratch_bytes(g, B) + (a.rope16 ? 0 : rope_scratch_bytes(g, max_len));
    LVQ_REQUIRE(ws_bytes >= need, LVQ_ERR_WORKSPACE, "lvq_quant_partial: workspace %zu < %zu bytes", ws_bytes,
                need);
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
    if ((st = pack_rope_if_needed(a, static_cast<unsigned char*>(ws) + quant_scratch_bytes(g, B), stream)) != LVQ_OK)
        return st;
    return launch_quant(a, ws, stream);
}

extern "C" lvq_status lvq_window_partial(const lvq_geom* gp, int32_t step, const void* q, const int32_t* seq_len,
                                         int32_t max_len, const void* win_k, const void* win_v,
                                         const float* rope_cos, const float* rope_sin, int32_t rope_len,
                                         float sm_scale, float* part_o, float* part_lse, int32_t slot,
                                         int32_t S_tot, int32_t B, hipStream_t stream) {
    AttnArgs a{};
    lvq_status st = prepare("lvq_window_partial", gp, step, q, seq_len, max_len, rope_cos, rope_sin, nullptr,
                            rope_len, sm_scale, B, &a);
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
    LVQ_REQUIRE(num_splits >= 0 && num_splits <= kMaxSplits, LVQ_ERR_INVALID_ARG, "%s: num_splits %d", fn,
                num_splits);
    LVQ_REQUIRE(pt_stride >= 0, LVQ_ERR_INVALID_ARG, "%s: negative pt_stride", fn);
    if (B == 0) return LVQ_OK;
    LVQ_REQUIRE(win_k && win_v && slices && out, LVQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    const int max_pages = max_index_pages(g, max_len);
    LVQ_REQUIRE(max_pages == 0 || (pool && page_table), LVQ_ERR_INVALID_ARG, "%s: NULL pool or page table", fn);
    LVQ_REQUIRE(pt_stride >= max_pages, LVQ_ERR_INVALID_ARG, "%s: pt_stride %d < %d pages", fn, pt_stride, max_pages);
    LVQ_REQUIRE(g.cb != LVQ_BF16 || max_pages <= kMaxSplits * (kMaxSplitTok / g.page), LVQ_ERR_UNSUPPORTED,
                "%s: a context of %d index pages exceeds the %d (%d splits of %d pages) the bf16 kernels take", fn,
                max_pages, kMaxSplits * (kMaxSplitTok / g.page), kMaxSplits, kMaxSplitTok / g.page);
    const int S = num_splits > 0 ? num_splits : choose_splits(g, B, max_len);
    LVQ_REQUIRE(splits_fit(g, max_pages, S), LVQ_ERR_INVALID_ARG,
                "%s: %d splits of %d index pages exceed %d tokens per split", fn, S, max_pages, kMaxSplitTok);
    // (the room for a packed RoPE table only when the call brings none)
    const size_t need = partials_bytes(g, B, S + 1) + quant_scratch_bytes(g, B) +
                        (a.rope16 ? 0 : rope_scratch_bytes(g, max_len));
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
    const size_t rows = size_t(B) * g.H * (S + 1);
    a.part_o = static_cast<float*>(ws);
    a.part_lse = a.part_o + rows * g.D;
    a.S_tot = S + 1;
    a.num_splits = S;
    a.pps = pages_per_split(max_pages, S);
    unsigned char* scratch = static_cast<unsigned char*>(ws) + partials_bytes(g, B, S + 1);
    if ((st = pack_rope_if_needed(a, scratch + quant_scratch_bytes(g, B), stream)) != LVQ_OK) return st;
    if ((st = launch_quant(a, scratch, stream)) != LVQ_OK) return st;
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
// Debug check of the page table and lengths the attention and encode kernels take on trust: one workgroup;
// wave w takes requests w, w + 16, ..., its lanes the request's index pages; counts in LDS.
// ---------------------------------------------------------------------------
namespace lvq {
namespace {
constexpr int kCheckThreads = 1024;

__global__ void __launch_bounds__(kCheckThreads) check_pages_kernel(Geo g, const int32_t* __restrict__ pt,
                                                                     int pt_stride,
                                                                     const int32_t* __restrict__ seq_len, int B,
                                                                     int max_len, int n_pool,
                                                                     int32_t* __restrict__ bad) {
    __shared__ int n_bad, first_bad, n_len;
    if (threadIdx.x == 0) {
        n_bad = 0;
        first_bad = 0x7fffffff;
        n_len = 0;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = kCheckThreads / 64;
    for (int b = wave; b < B; b += nw) {
        const int L0 = seq_len[b];
        if (lane == 0 && (L0 < 0 || L0 > max_len)) atomicAdd(&n_len, 1);
        const int np = n_index_pages(min(max(L0, 0), max_len), g);
        for (int lp = lane; lp < np; lp += 64) {
            const int v = pt[long(b) * pt_stride + lp];
            if (v < 0 || v >= n_pool) {
                atomicAdd(&n_bad, 1);
                atomicMin(&first_bad, b);
            }
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        bad[0] = n_bad;
        bad[1] = first_bad == 0x7fffffff ? -1 : first_bad;
        bad[2] = n_len;
    }
}
}  // namespace
}  // namespace lvq

extern "C" lvq_status lvq_check_pages(const lvq_geom* gp, const int32_t* page_table, int32_t pt_stride,
                                      const int32_t* seq_len, int32_t max_len, int32_t n_pool_pages, int32_t B,
                                      int32_t* bad, hipStream_t stream) {
    Geo g;
    const lvq_status st = validate_geom(gp, &g);
    if (st != LVQ_OK) return st;
    LVQ_REQUIRE(B >= 0 && max_len >= 1 && n_pool_pages >= 1, LVQ_ERR_INVALID_ARG,
                "lvq_check_pages: B=%d max_len=%d n_pool_pages=%d", B, max_len, n_pool_pages);
    const int max_pages = max_index_pages(g, max_len);
    LVQ_REQUIRE(pt_stride >= max_pages, LVQ_ERR_INVALID_ARG, "lvq_check_pages: pt_stride %d < %d pages", pt_stride,
                max_pages);
    LVQ_REQUIRE(bad && (B == 0 || (seq_len && (max_pages == 0 || page_table))), LVQ_ERR_INVALID_ARG,
                "lvq_check_pages: NULL pointer");
    hipLaunchKernelGGL(check_pages_kernel, dim3(1), dim3(kCheckThreads), 0, stream, g, page_table, pt_stride, seq_len,
                       B, max_len, n_pool_pages, bad);
    return check_launch("lvq_check_pages");
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
