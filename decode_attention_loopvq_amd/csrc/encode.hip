// LoopVQ codebook slicing, RoPE table and index-page encoding.
//
// LoopVQ page ("LoopVQ: Sub 1-bit KV Cache Quantization for Looped
// Transformers"): "method steps" step 1 (loop-axis coupling), step 4 (paged
// index cache, encode after the block's last loop step, one page every 8
// generated tokens), step 5 (per-step codebook slice B_t cut once at load);
// background "RoPE" (precomputed cos/sin table).
#include <vector>

#include "common.h"

#include <cmath>
#include <type_traits>

namespace lvq {
namespace {

// ---------------------------------------------------------------------------
// B_t slices: slices[t][h][kv][g][r][i] = codebooks[t/Tc][h][kv][g][r][i*Tc + t%Tc]
// ---------------------------------------------------------------------------
template <typename E>
__global__ void slice_kernel(const E* __restrict__ cb, E* __restrict__ out, int Tc, int H,
                             int NG, int K, int G, long total) {
    const int c = G / Tc;
    for (long e = blockIdx.x * long(blockDim.x) + threadIdx.x; e < total; e += long(gridDim.x) * blockDim.x) {
        long r = e;
        const int i = int(r % c); r /= c;
        const int cw = int(r % K); r /= K;
        const int g = int(r % NG); r /= NG;
        const int kv = int(r % 2); r /= 2;
        const int h = int(r % H); r /= H;
        const int t = int(r);
        const int beta = t / Tc, m = t % Tc;
        const long src = ((((long(beta) * H + h) * 2 + kv) * NG + g) * K + cw) * G + i * Tc + m;
        out[e] = cb[src];
    }
}

// ---------------------------------------------------------------------------
// RoPE table in fp64, rounded once to fp32.
// ---------------------------------------------------------------------------
// Frequency of each column of a RoPE table: column i holds frequency f[i] (i itself without a channel
// permutation).
constexpr int kMaxHalf = 256;
struct FreqMap {
    int16_t f[kMaxHalf];
};

FreqMap identity_freqs() {
    FreqMap fm;
    for (int i = 0; i < kMaxHalf; ++i) fm.f[i] = int16_t(i);
    return fm;
}

__global__ void rope_table_kernel(int len, int D, double base, float* __restrict__ cs,
                                  float* __restrict__ sn, const FreqMap fm) {
    const int half = D / 2;
    const long total = long(len) * half;
    for (long e = blockIdx.x * long(blockDim.x) + threadIdx.x; e < total; e += long(gridDim.x) * blockDim.x) {
        const int p = int(e / half), i = int(e % half);
        const double theta = pow(base, -2.0 * double(fm.f[i]) / double(D));
        const double a = double(p) * theta;
        cs[e] = float(cos(a));
        sn[e] = float(sin(a));
    }
}

// ---------------------------------------------------------------------------
// Packed fp16 table for the index-page pass (layout rope_f16 in lvq.h): 32
// chunks of 8 halves per position p; chunk m < 16 (frequencies 4m..4m+3) at
// out[(p * 32 + m) * 8 ..] holds cos x4 then sin x4, chunk 16 + m the same
// with the sines negated.
// ---------------------------------------------------------------------------
// fp64 -> binary16 with one rounding (nearest even): round to fp32 with
// round-to-odd first (fp32 keeps more than two extra bits), then RNE.
__device__ __forceinline__ _Float16 f64_to_f16_rn(double x) {
    float f = float(x);
    if (double(f) != x) {
        uint32_t u = __float_as_uint(f);
        if (fabs(double(f)) > fabs(x)) --u;      // truncate toward zero
        f = __uint_as_float(u | 1u);             // inexact: odd last bit
    }
    return (_Float16)f;
}

__global__ void rope_f16_kernel(int len, double base, _Float16* __restrict__ out, const FreqMap fm) {
    const long total = long(len) * 64;
    for (long e = blockIdx.x * long(blockDim.x) + threadIdx.x; e < total; e += long(gridDim.x) * blockDim.x) {
        const int p = int(e / 64), i = int(e % 64);
        const double theta = pow(base, -2.0 * double(fm.f[i]) / 128.0);
        const double ang = double(p) * theta;
        store_rope_f16(out, len, p, i, f64_to_f16_rn(cos(ang)), f64_to_f16_rn(sin(ang)));
    }
}

// ---------------------------------------------------------------------------
// Encode: one workgroup per (page, head, K|V, request); one thread per
// (token of the page, index group).  The nearest codeword is found by a
// direct-difference scan in fp64 with each product and sum rounded
// separately, keeping the first minimum (lowest index on ties).
// ---------------------------------------------------------------------------
template <typename CB>
__device__ __forceinline__ double cb_elem(const CB* p);
template <>
__device__ __forceinline__ double cb_elem<uint16_t>(const uint16_t* p) { return double(bf16_to_f32(*p)); }
template <>
__device__ __forceinline__ double cb_elem<float>(const float* p) { return double(*p); }

// Index-token number (from the first paged position) of token i of logical page lp.
__device__ __forceinline__ int slot_token(int lp, int i, int page) { return lp * page + i; }

template <typename CB>
__global__ void encode_scan_kernel(Geo geo, int block, const uint16_t* __restrict__ xk,
                                   const uint16_t* __restrict__ xv, long s0, long s1, long s2, long s3,
                                   const int64_t* __restrict__ tok0, const CB* __restrict__ cb,
                                   uint8_t* __restrict__ pool, const int32_t* __restrict__ pt, int pt_stride,
                                   const int32_t* __restrict__ first_page, const int32_t* __restrict__ n_pages) {
    const int slot = blockIdx.x;
    const int h = blockIdx.y >> 1, kv = blockIdx.y & 1;
    const int b = blockIdx.z;
    if (slot >= n_pages[b]) return;
    const uint16_t* x = kv == 0 ? xk : xv;
    if (x == nullptr) return;
    const int NG = geo.NG, c = geo.c, Tc = geo.Tc, G = geo.G, K = geo.K;
    const int tid = threadIdx.x;
    const int i_tok = tid / NG, g = tid % NG;
    const int lp = first_page[b] + slot;
    const long phys = pt[long(b) * pt_stride + lp];
    const long row = (tok0 ? tok0[b] : 0) + long(slot) * geo.page + i_tok;

    double z[32];
    const uint16_t* xb = x + long(b) * s0 + long(h) * s1 + row * s2;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
        if (k < G) {
            const int i = k / Tc, m = k % Tc;   // coordinate i*Tc + m <- step m, channel g*c + i
            z[k] = double(bf16_to_f32(xb[long(m) * s3 + g * c + i]));
        }
    }
    const CB* e = cb + (((long(block) * geo.H + h) * 2 + kv) * NG + g) * long(K) * G;
    double best = 0.0;
    int best_r = 0;
    for (int r = 0; r < K; ++r) {
        double d = 0.0;
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            if (k < G) {
                const double diff = __dsub_rn(z[k], cb_elem(e + long(r) * G + k));
                d = __dadd_rn(d, __dmul_rn(diff, diff));
            }
        }
        if (r == 0 || d < best) {
            best = d;
            best_r = r;
        }
    }
    // Index rows are permuted by the index-token number (layout in lvq.h).
    const int tau = slot_token(lp, i_tok, geo.page);
    const int byte = index_byte(kv, NG, g, tau);
    pool[phys * geo.page_bytes + ((long(block) * geo.H + h) * 2 + kv) * geo.page * NG + i_tok * NG + byte] =
        uint8_t(best_r);
}


// ---------------------------------------------------------------------------
// Encoder for bf16 codebooks on the matrix cores (G <= 32).
//
// argmin_r ||z - e_r||^2 = argmax_r (z . e_r - ||e_r||^2 / 2): a contraction
// of the coupled vectors with the codebook, [tokens x G] x [G x 256], done
// by v_mfma_f32_16x16x32_bf16 with the accumulator started at -||e_r||^2/2
// (products of bf16 values are exact in fp32; sums round in fp32).
//
// Workgroup: 8 waves, one index group each (groups 8*octet .. 8*octet+7), a
// block of kEncTile * kEncTilesPerWg tokens of one (request, head, K|V).
// A wave keeps its group's codebook as 16 operand fragments (codewords
// 16t .. 16t+15) in registers and -||e||^2/2 of its 256 codewords in LDS.
// MFMA lane l holds row / column l & 15 and coordinates k = 8*(l >> 4) .. +7
// of its operands (the codebook's own coordinate order i*T_c + m;
// coordinates past G are zero), and result rows 4*(l >> 4) .. +3 of column
// l & 15.  Per 16-token tile: 16 MFMAs with the codewords as rows and the
// tokens as columns, so lane (q, n) holds 64 scores of token n (codewords
// 16t + 4q + i); its best two, then the best two of the 4 lanes of the
// column through two lane swaps; the lowest index wins exact ties.  Where the
// best two scores lie within twice the fp32 error bound of a score, the
// token's nearest codeword is taken again from fp64 direct differences over
// all 256 codewords, so that every pick is the exact nearest codeword (the
// first one among equal distances).
//
// XREQ (few pages per request, as in the decode-time encode of one page):
// a workgroup takes token slots u = b * tpr + j of all requests (tpr =
// 8 * max_pages, j < 8 * n_pages[b] valid), so that each head's codebooks are
// loaded once for the whole batch instead of once per request.
// ---------------------------------------------------------------------------
constexpr int kEncTile = 16;
constexpr int kEncTilesPerWg = 32;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct EncArgs {
    Geo geo;
    int block;
    const uint16_t* xk;
    const uint16_t* xv;
    long s0, s1, s2, s3;
    const int64_t* tok0;
    const uint16_t* cb;
    uint8_t* pool;
    const int32_t* pt;
    int pt_stride;
    const int32_t* first_page;
    const int32_t* n_pages;
    int noct;                   // group octets, NG / 8
    int B;
    int tpr;                    // XREQ: token slots per request (8 * max_pages)
};

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
    return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xf, 0xf, false);
}

template <int TC, bool XREQ>
__global__ void __launch_bounds__(512) encode_mfma_kernel(EncArgs a) {
    constexpr int IPL = 8 / TC;                  // channels per lane and step
    const Geo& g = a.geo;
    const int G = g.G, c = g.c;
    const int oct = blockIdx.y % a.noct;
    const int kv = (blockIdx.y / a.noct) & 1;
    const int h = blockIdx.y / (2 * a.noct);
    const int b = XREQ ? 0 : blockIdx.z;        // (XREQ: per token slot, below)
    const int ntok = XREQ ? a.B * a.tpr : a.n_pages[b] * g.page;   // XREQ: token slots
    const int tok_base = blockIdx.x * (kEncTile * kEncTilesPerWg);
    if (tok_base >= ntok) return;
    const uint16_t* x = kv == 0 ? a.xk : a.xv;
    if (x == nullptr) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int grp = oct * 8 + (tid >> 6);
    const int n = lane & 15, q = lane >> 4;
    const bool kin = 8 * q < G;                  // this lane's coordinates exist

    // codebook fragments and -||e||^2 / 2 per column
    const uint16_t* e = a.cb + ((((long(a.block) * g.H + h) * 2 + kv) * g.NG + grp) * g.K) * long(G);
    bf16x8_t bfr[16];
    float cinit[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        uint4 w = *reinterpret_cast<const uint4*>(e + long(16 * t + n) * G + (kin ? 8 * q : 0));
        w = make_uint4(w.x & (kin ? ~0u : 0u), w.y & (kin ? ~0u : 0u), w.z & (kin ? ~0u : 0u), w.w & (kin ? ~0u : 0u));
        bfr[t] = __builtin_bit_cast(bf16x8_t, w);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
        float s = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            s = fmaf(bf16_lo(ww[u]), bf16_lo(ww[u]), s);
            s = fmaf(bf16_hi(ww[u]), bf16_hi(ww[u]), s);
        }
        s += __shfl_xor(s, 16, 64);
        s += __shfl_xor(s, 32, 64);
        cinit[t] = -0.5f * s;
    }

    // lanes past G read the group's first channels (a valid address) and zero them
    const long xbase = long(b) * a.s0 + long(h) * a.s1 + long(grp) * c + (kin ? (8 * q) / TC : 0);
    const uint32_t kmask = kin ? 0xffffffffu : 0u;
    const long row0 = (a.tok0 ? a.tok0[b] : 0);
    const int fp = a.first_page[b];
    const long blk_off = ((long(a.block) * g.H + h) * 2 + kv) * g.page * g.NG;
    // XREQ: token slot u -> (request, token of the request, whether the slot holds a token)
    auto slot = [&](int u, int& bu, int& ju) {
        bu = min(u / a.tpr, a.B - 1);
        ju = u - bu * a.tpr;
        return ju < a.n_pages[bu] * g.page;
    };
    // coupled-vector coordinates k = 8q .. 8q+7 of token j (row of this lane): the raw words are loaded one
    // tile ahead and interleaved into coordinate order (element u = (i - i0) * TC + m) when used
    struct RawA { uint32_t w[TC][(IPL + 1) / 2]; };
    auto load_a = [&](int j) {
        RawA r;
        const uint16_t* xr;
        if constexpr (XREQ) {                    // a slot without a token loads nothing (zeros)
            int bu, ju;
            if (!slot(min(j, ntok - 1), bu, ju)) {
#pragma unroll
                for (int m = 0; m < TC; ++m)
#pragma unroll
                    for (int w = 0; w < (IPL + 1) / 2; ++w) r.w[m][w] = 0u;
                return r;
            }
            xr = x + xbase + long(bu) * a.s0 + ((a.tok0 ? a.tok0[bu] : 0) + ju) * a.s2;
        } else {
            xr = x + xbase + (row0 + min(j, ntok - 1)) * a.s2;
        }
#pragma unroll
        for (int m = 0; m < TC; ++m) {
            if constexpr (IPL == 8) {
                const uint4 w = *reinterpret_cast<const uint4*>(xr + m * a.s3);
                r.w[m][0] = w.x; r.w[m][1] = w.y; r.w[m][2] = w.z; r.w[m][3] = w.w;
            } else if constexpr (IPL == 4) {
                const uint2 w = *reinterpret_cast<const uint2*>(xr + m * a.s3);
                r.w[m][0] = w.x; r.w[m][1] = w.y;
            } else if constexpr (IPL == 2) {
                r.w[m][0] = *reinterpret_cast<const uint32_t*>(xr + m * a.s3);
            } else {
                r.w[m][0] = xr[m * a.s3];
            }
        }
        return r;
    };
    auto build_a = [&](const RawA& r) {
        auto elem = [&](int u) -> uint32_t {         // bf16 bits of coordinate 8q + u
            const int m = u % TC, il = u / TC;
            return (r.w[m][il >> 1] >> (16 * (il & 1))) & 0xffffu;
        };
        uint32_t d[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) d[w] = (elem(2 * w) | (elem(2 * w + 1) << 16)) & kmask;
        return __builtin_bit_cast(bf16x8_t, make_uint4(d[0], d[1], d[2], d[3]));
    };

    // indices of the block's tokens for the 8 groups of this octet, written out at the end
    __shared__ __align__(16) uint8_t idx[kEncTile * kEncTilesPerWg][8];
    // per wave and tile, the tokens whose best two scores lie within the error bound (bit n: token t0 + n)
    __shared__ uint16_t near_tok[8][kEncTilesPerWg];
    // the operand chunks (lane q's 8 coordinates) of the first such token of a wave's first kStash tiles
    // that have one, in tile order
    constexpr int kStash = 8;
    __shared__ __align__(16) uint4 zstash[8][kStash][4];
    // -||e_r||^2 / 2 of the wave's group in codeword order (each wave writes and reads only its own row)
    __shared__ __align__(16) float cnorm[8][256];
    {
        const int w8 = tid >> 6;
#pragma unroll
        for (int t = 0; t < 16; ++t) cnorm[w8][16 * t + n] = cinit[t];   // (the 4 lanes of a column agree)
    }
    // Error bound of a score (sums in fp32; products of bf16 values exact): |s^ - s| <= eps =
    // kScoreErr * (||z|| E + E^2), E the largest codeword norm of the group.  kScoreErr is twice the fp32
    // bound gamma_32 = 32 * 2^-24 / (1 - 32 * 2^-24) of a 33-term sum, which also covers an accumulation that
    // does not round to nearest, plus 5% for the rounding of eps itself (zsq, the square root); E^2 in place
    // of E^2 / 2 covers the rounding of the norms.  Where the best and second-best scores of a token differ
    // by more than 2 eps, the best is the exact nearest codeword.
    constexpr float kScoreErr = 4.0e-6f;
    float e2max = 0.f;
#pragma unroll
    for (int t = 0; t < 16; ++t) e2max = fmaxf(e2max, -2.f * cinit[t]);
    e2max = __builtin_amdgcn_readfirstlane(wave_max(e2max));
    const float emax = __builtin_amdgcn_readfirstlane(sqrtf(e2max));
    // Tile of 16 tokens with the codewords as rows: lane (q, n) gets the scores of token t0 + n for
    // codewords 16t + 4q + i (t < 16, i < 4) and keeps its best two: per MFMA output the maximum of its 4
    // scores against the running best, the 4 scores of the best output so far kept, and the second best
    // among the other outputs' maxima (a median of three); at the end the best and second of the kept 4
    // resolve the lane's pair.  Then the best two of the 4 lanes n, n + 16, n + 32, n + 48 through two lane
    // swaps.  Equal scores need no order here: a token whose best two lie within 2 eps (equal ones
    // included) is decided again by exact distances (recheck).
    auto merge = [](float& best, float& second, int& r, float ob, float os, int orr) {
        const bool take = ob > best;                     // (equal scores: flagged, so either index serves)
        second = __builtin_amdgcn_fmed3f(best, ob, fmaxf(second, os));   // max(min(best, ob), second, os)
        best = take ? ob : best;
        r = take ? orr : r;
    };
    // The nearest codeword of one token by direct differences in fp64, from registers: lane (q, n) takes its
    // 16 codewords 16 t + n over coordinates 8 q .. 8 q + 7 (its operand fragments), summed in coordinate
    // order, against the token's same coordinates (zw, as the tile's operand); the four chunks of each
    // codeword are added across the lanes n, n + 16, n + 32, n + 48 in a fixed order; then the minimum over
    // the 256 codewords, the lowest index among equal distances.
    auto recheck = [&](const uint4& zw) {
        const uint32_t zc[4] = {zw.x, zw.y, zw.z, zw.w};
        double zd[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) zd[u] = double((u & 1) ? bf16_hi(zc[u >> 1]) : bf16_lo(zc[u >> 1]));
        double bd = 0.0;
        int br = -1;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            // opaque copy: the conversions below stay here instead of being hoisted out of the callers' loops
            // as 256 doubles held in registers
            const uint4 ew = __builtin_bit_cast(uint4, bfr[t]);
            uint32_t e4[4] = {ew.x, ew.y, ew.z, ew.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) asm volatile("" : "+v"(e4[u]));
            double d = 0.0;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const double diff = zd[u] - double((u & 1) ? bf16_hi(e4[u >> 1]) : bf16_lo(e4[u >> 1]));
                d = fma(diff, diff, d);
            }
            // chunks q and q ^ 2 (lane swap of 32), then the pairs (lane swap of 16): ((d0 + d2) + (d1 + d3))
            const uint64_t db = __builtin_bit_cast(uint64_t, d);
            const auto l32 = __builtin_amdgcn_permlane32_swap(uint32_t(db), uint32_t(db), false, false);
            const auto h32 = __builtin_amdgcn_permlane32_swap(uint32_t(db >> 32), uint32_t(db >> 32), false, false);
            const double a0 = __builtin_bit_cast(double, (uint64_t(uint32_t(h32[0])) << 32) | uint32_t(l32[0]));
            const double a1 = __builtin_bit_cast(double, (uint64_t(uint32_t(h32[1])) << 32) | uint32_t(l32[1]));
            const double s2 = q < 2 ? a0 + a1 : a1 + a0;           // chunk q first: the same sum in both lanes
            const uint64_t sb = __builtin_bit_cast(uint64_t, s2);
            const auto l16 = __builtin_amdgcn_permlane16_swap(uint32_t(sb), uint32_t(sb), false, false);
            const auto h16 = __builtin_amdgcn_permlane16_swap(uint32_t(sb >> 32), uint32_t(sb >> 32), false, false);
            const double b0 = __builtin_bit_cast(double, (uint64_t(uint32_t(h16[0])) << 32) | uint32_t(l16[0]));
            const double b1 = __builtin_bit_cast(double, (uint64_t(uint32_t(h16[1])) << 32) | uint32_t(l16[1]));
            const double tot = (q & 1) == 0 ? b0 + b1 : b1 + b0;
            if (br < 0 || tot < bd) { bd = tot; br = 16 * t + n; }
            __builtin_amdgcn_sched_barrier(0);           // one codeword row at a time: few live registers
        }
        // across the 16 codeword rows n of a row of lanes (the q copies agree): partners l ^ 1, l ^ 2 (quad
        // permutes), then 7 - l and 15 - l within the row (half-row and row mirrors); the lexicographic
        // minimum of (distance, index) is symmetric, so both lanes of a pair keep the same result
        auto step = [&](auto partner) {
            const uint64_t db = __builtin_bit_cast(uint64_t, bd);
            const double od = __builtin_bit_cast(double, (uint64_t(uint32_t(partner(int(db >> 32)))) << 32) |
                                                         uint32_t(partner(int(uint32_t(db)))));
            const int orr = partner(br);
            const bool take = od < bd || (od == bd && orr < br);
            bd = take ? od : bd;
            br = take ? orr : br;
        };
        step([](int x) { return dpp_i<0xB1>(x); });      // quad_perm [1, 0, 3, 2]
        step([](int x) { return dpp_i<0x4E>(x); });      // quad_perm [2, 3, 0, 1]
        step([](int x) { return dpp_i<0x141>(x); });     // row_half_mirror
        step([](int x) { return dpp_i<0x140>(x); });     // row_mirror
        return __builtin_amdgcn_readfirstlane(br);
    };
    uint64_t any_near = 0;                               // some token of the wave's tiles near a tie
    int n_tiles_near = 0;                                // tiles with such tokens so far (wave-uniform)
    auto tile_fn = [&](int t0, const RawA& raw) {
        const bf16x8_t Bcur = build_a(raw);
        const float* cn = &cnorm[tid >> 6][4 * q];
        // each tile of scores is scanned four MFMAs after it is issued, so that few accumulators are live
        constexpr int kLag = 4;
        f32x4_t acc[16];
        float best = -INFINITY, sec = -INFINITY;
        float w0 = -INFINITY, w1 = -INFINITY, w2 = -INFINITY, w3 = -INFINITY;
        int rt = 0;
        // maxima as medians with +inf: three-way ones become single max3 instructions (a two-way maximum of
        // raw MFMA results would be preceded by canonicalising moves)
        auto fmax2 = [](float x, float y) { return __builtin_amdgcn_fmed3f(x, y, INFINITY); };
        auto scan = [&](int t) {
            const float v0 = acc[t][0], v1 = acc[t][1], v2 = acc[t][2], v3 = acc[t][3];
            const float m3 = fmax2(fmax2(v0, v1), v2);
            const float nb = fmax2(fmax2(best, m3), v3);         // max(best, the output's maximum)
            const bool gt = nb > best;
            sec = gt ? best : fmax2(fmax2(sec, m3), v3);
            best = nb;
            rt = gt ? t : rt;
            w0 = gt ? v0 : w0;
            w1 = gt ? v1 : w1;
            w2 = gt ? v2 : w2;
            w3 = gt ? v3 : w3;
        };
#pragma unroll
        for (int t = 0; t < 16 + kLag; ++t) {
            if (t < 16) {
                const f32x4_t ci = *reinterpret_cast<const f32x4_t*>(cn + 16 * t);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[t], Bcur, ci, 0, 0, 0);
            }
            if (t >= kLag) scan(t - kLag);
        }
        // the lane's best two: the kept output's largest (its index) and the larger of its second largest
        // and the other outputs' best
        float second;
        int r;
        {
            const float a01 = fmax2(w0, w1), a23 = fmax2(w2, w3);
            const float b01 = fminf(w0, w1), b23 = fminf(w2, w3);
            second = fmax2(sec, __builtin_amdgcn_fmed3f(a01, a23, fmax2(b01, b23)));
            const int i = a01 >= a23 ? (w0 >= w1 ? 0 : 1) : (w2 >= w3 ? 2 : 3);
            r = 16 * rt + 4 * q + i;
        }
        {   // lanes l and l ^ 32, then l and l ^ 16 (the combine is symmetric, so both lanes of a pair agree)
            const auto bv = __builtin_amdgcn_permlane32_swap(__float_as_uint(best), __float_as_uint(best), false, false);
            const auto sv = __builtin_amdgcn_permlane32_swap(__float_as_uint(second), __float_as_uint(second), false, false);
            const auto rv = __builtin_amdgcn_permlane32_swap(uint32_t(r), uint32_t(r), false, false);
            const uint32_t b0 = bv[0], b1 = bv[1], s0v = sv[0], s1v = sv[1], r0v = rv[0], r1v = rv[1];
            best = __uint_as_float(b0);
            second = __uint_as_float(s0v);
            r = int(r0v);
            merge(best, second, r, __uint_as_float(b1), __uint_as_float(s1v), int(r1v));
        }
        {
            const auto bv = __builtin_amdgcn_permlane16_swap(__float_as_uint(best), __float_as_uint(best), false, false);
            const auto sv = __builtin_amdgcn_permlane16_swap(__float_as_uint(second), __float_as_uint(second), false, false);
            const auto rv = __builtin_amdgcn_permlane16_swap(uint32_t(r), uint32_t(r), false, false);
            const uint32_t b0 = bv[0], b1 = bv[1], s0v = sv[0], s1v = sv[1], r0v = rv[0], r1v = rv[1];
            best = __uint_as_float(b0);
            second = __uint_as_float(s0v);
            r = int(r0v);
            merge(best, second, r, __uint_as_float(b1), __uint_as_float(s1v), int(r1v));
        }
        // ||z||^2 of the column's token (the 4 lanes of the column hold 8 coordinates each)
        const uint4 bw = __builtin_bit_cast(uint4, Bcur);
        float zsq = 0.f;
        {
            const uint32_t w4[4] = {bw.x, bw.y, bw.z, bw.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                zsq = fmaf(bf16_lo(w4[u]), bf16_lo(w4[u]), zsq);
                zsq = fmaf(bf16_hi(w4[u]), bf16_hi(w4[u]), zsq);
            }
            // the column's other lanes (l ^ 32, l ^ 16) through lane swaps, no LDS traffic
            const auto a32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(zsq), __float_as_uint(zsq), false, false);
            zsq = __uint_as_float(a32[0]) + __uint_as_float(a32[1]);
            const auto a16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(zsq), __float_as_uint(zsq), false, false);
            zsq = __uint_as_float(a16[0]) + __uint_as_float(a16[1]);
        }
        const float eps = kScoreErr * (__builtin_amdgcn_sqrtf(zsq) * emax + e2max);
        const uint64_t near = __builtin_amdgcn_ballot_w64(q == 0 && best - second <= 2.f * eps);
        if (q == 0) idx[(t0 - tok_base) + n][grp & 7] = uint8_t(r);
        if (lane == 0) near_tok[tid >> 6][(t0 - tok_base) / kEncTile] = uint16_t(near);
        any_near |= near;
        // (straight-line code: a loop here would make the compiler wait for the next tile's loads)
        if (near != 0 && n_tiles_near < kStash) {       // rare: the tile's first such token stashed
            if (n == int(__builtin_ctzll(near))) zstash[tid >> 6][n_tiles_near][q] = bw;
            ++n_tiles_near;
        }
    };
    // two alternating buffers: the loads of tile k+1 are in flight while tile k computes
    RawA rawA = load_a(tok_base + n), rawB;
    const int t_end = min(ntok, tok_base + kEncTile * kEncTilesPerWg);
    for (int t0 = tok_base; t0 < t_end; t0 += 2 * kEncTile) {
        rawB = load_a(t0 + kEncTile + n);              // (clamped to the last token at the end)
        tile_fn(t0, rawA);
        if (t0 + kEncTile >= t_end) break;
        rawA = load_a(t0 + 2 * kEncTile + n);
        tile_fn(t0 + kEncTile, rawB);
    }
    // The tokens marked near a tie, decided again (rare), in tile order: stashed chunks where there are,
    // the coordinates loaded again for the others.
    for (int tt = 0, k = 0; any_near != 0 && tt * kEncTile < t_end - tok_base; ++tt) {
        uint32_t near = near_tok[tid >> 6][tt];
        for (bool first = true; near != 0; near &= near - 1, first = false) {
            const int j = tok_base + tt * kEncTile + __builtin_ctz(near);
            const bool stashed = first && k < kStash;
            k += first ? 1 : 0;
            const uint4 zw = stashed ? zstash[tid >> 6][max(k - 1, 0)][q] : __builtin_bit_cast(uint4, build_a(load_a(j)));
            const int rx = recheck(zw);
            if (lane == 0) idx[j - tok_base][grp & 7] = uint8_t(rx);
        }
    }
    __syncthreads();
    // one thread per token: the octet's 8 index bytes, one 8-byte store (value rows: the octet's bytes sit
    // in the half row (octet ^ (tau >> 3 & 1)) XOR-permuted by tau & 7)
    int j = tok_base + tid, bj = b, fpj = fp;
    bool has = tid < kEncTile * kEncTilesPerWg && j < t_end;
    if constexpr (XREQ) {
        if (has) {
            int ju;
            has = slot(j, bj, ju);
            j = ju;
            fpj = a.first_page[bj];
        }
    }
    if (has) {
        const int lp = fpj + j / g.page, ri = j % g.page;
        const long phys = a.pt[long(bj) * a.pt_stride + lp];
        const int tau = lp * g.page + ri;
        uint8_t* row = a.pool + phys * g.page_bytes + blk_off + ri * g.NG;
        if (kv == 0 && g.NG == 16) {
            // key rows of 16 groups (layout in lvq.h): the octet's groups 8*oct + u sit in the bytes j with
            // bit 1 of j equal to oct ^ bit 3 of tau, two adjacent bytes at a time
            const int hb = (oct ^ (tau >> 3)) & 1;
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
                const int j = 4 * pr + 2 * hb;
                const int u0 = key_group_of_byte(j, tau) - 8 * oct, u1 = key_group_of_byte(j + 1, tau) - 8 * oct;
                *reinterpret_cast<uint16_t*>(row + j) = uint16_t(idx[tid][u0] | (uint32_t(idx[tid][u1]) << 8));
            }
        } else if (kv == 0) {
            *reinterpret_cast<uint2*>(row + 8 * oct) = *reinterpret_cast<const uint2*>(idx[tid]);
        } else {
            // group 8*oct + u goes to byte (8*oct + u) ^ (tau & 15)
            const int rot = tau & 15;
            uint8_t v8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v8[u ^ (rot & 7)] = idx[tid][u];
            *reinterpret_cast<uint2*>(row + 8 * (oct ^ (rot >> 3))) = *reinterpret_cast<const uint2*>(v8);
        }
    }
}

int grid_for(long total, int threads) {
    long b = (total + threads - 1) / threads;
    if (b > 65536) b = 65536;
    if (b < 1) b = 1;
    return int(b);
}

}  // namespace
}  // namespace lvq

using namespace lvq;

extern "C" lvq_status lvq_slice_codebooks(const lvq_geom* g, const void* codebooks, void* slices,
                                          hipStream_t stream) {
    Geo geo;
    lvq_status st = validate_geom(g, &geo);
    if (st != LVQ_OK) return st;
    LVQ_REQUIRE(codebooks && slices, LVQ_ERR_INVALID_ARG, "lvq_slice_codebooks: NULL pointer");
    const long total = long(geo.T) * geo.H * 2 * geo.NG * geo.K * geo.c;
    const int threads = 256;
    if (geo.cb == LVQ_BF16)
        hipLaunchKernelGGL(slice_kernel<uint16_t>, dim3(grid_for(total, threads)), dim3(threads), 0, stream,
                           static_cast<const uint16_t*>(codebooks), static_cast<uint16_t*>(slices), geo.Tc,
                           geo.H, geo.NG, geo.K, geo.G, total);
    else
        hipLaunchKernelGGL(slice_kernel<float>, dim3(grid_for(total, threads)), dim3(threads), 0, stream,
                           static_cast<const float*>(codebooks), static_cast<float*>(slices), geo.Tc,
                           geo.H, geo.NG, geo.K, geo.G, total);
    return check_launch("lvq_slice_codebooks");
}

extern "C" lvq_status lvq_rope_table(int32_t len, int32_t D, double base, float* cos_out, float* sin_out,
                                     hipStream_t stream) {
    LVQ_REQUIRE(len > 0 && D > 0 && D % 2 == 0, LVQ_ERR_INVALID_ARG, "lvq_rope_table: bad len=%d D=%d", len, D);
    LVQ_REQUIRE(base > 1.0, LVQ_ERR_INVALID_ARG, "lvq_rope_table: base must exceed 1");
    LVQ_REQUIRE(cos_out && sin_out, LVQ_ERR_INVALID_ARG, "lvq_rope_table: NULL pointer");
    LVQ_REQUIRE(D / 2 <= kMaxHalf, LVQ_ERR_UNSUPPORTED, "lvq_rope_table: D=%d (at most %d)", D, 2 * kMaxHalf);
    const long total = long(len) * (D / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3(grid_for(total, 256)), dim3(256), 0, stream, len, D, base,
                       cos_out, sin_out, identity_freqs());
    return check_launch("lvq_rope_table");
}

extern "C" lvq_status lvq_rope_table_f16(int32_t len, int32_t D, double base, void* out, hipStream_t stream) {
    LVQ_REQUIRE(len > 0, LVQ_ERR_INVALID_ARG, "lvq_rope_table_f16: bad len=%d", len);
    LVQ_REQUIRE(D == 128, LVQ_ERR_UNSUPPORTED, "lvq_rope_table_f16: D=%d (128 supported)", D);
    LVQ_REQUIRE(base > 1.0, LVQ_ERR_INVALID_ARG, "lvq_rope_table_f16: base must exceed 1");
    LVQ_REQUIRE(out, LVQ_ERR_INVALID_ARG, "lvq_rope_table_f16: NULL pointer");
    hipLaunchKernelGGL(rope_f16_kernel, dim3(grid_for(long(len) * 64, 256)), dim3(256), 0, stream, len, base,
                       static_cast<_Float16*>(out), identity_freqs());
    return check_launch("lvq_rope_table_f16");
}

namespace lvq {
namespace {
// The checks of lvq_channel_perm_check with error messages naming `fn`.
lvq_status check_channel_perm(const char* fn, const Geo& g, const int32_t* perm) {
    LVQ_REQUIRE(perm, LVQ_ERR_INVALID_ARG, "%s: NULL permutation", fn);
    const int D = g.D, half = D / 2;
    std::vector<int> seen(D, 0);
    for (int j = 0; j < D; ++j) {
        LVQ_REQUIRE(perm[j] >= 0 && perm[j] < D && !seen[perm[j]], LVQ_ERR_INVALID_ARG,
                    "%s: not a permutation of 0..%d (entry %d = %d)", fn, D - 1, j, perm[j]);
        seen[perm[j]] = 1;
    }
    for (int j = 0; j < half; ++j) {
        if (perm[j] < half && perm[j + half] == perm[j] + half) continue;
        // where do the two channels of the RoPE pair of stored channel j sit?
        const int i = perm[j] < half ? perm[j] : perm[j] - half;
        int a = -1, b = -1;
        for (int k = 0; k < D; ++k) {
            if (perm[k] == i) a = k;
            if (perm[k] == i + half) b = k;
        }
        LVQ_REQUIRE(a / g.c != b / g.c, LVQ_ERR_UNSUPPORTED,
                    "%s: stored channels %d and %d (RoPE pair %d, %d) fall in one index group of %d channels; "
                    "the kernels rotate channel j with channel j + %d, a different group", fn, a, b, i, i + half,
                    g.c, half);
        LVQ_REQUIRE(false, LVQ_ERR_UNSUPPORTED,
                    "%s: stored channels %d and %d (RoPE pair %d, %d) are not j and j + %d with the lower one "
                    "first", fn, a, b, i, i + half, half);
    }
    return LVQ_OK;
}
}  // namespace
}  // namespace lvq

extern "C" lvq_status lvq_channel_perm_check(const lvq_geom* gp, const int32_t* perm) {
    lvq::Geo g;
    lvq_status st = lvq::validate_geom(gp, &g);
    if (st != LVQ_OK) return st;
    return lvq::check_channel_perm("lvq_channel_perm_check", g, perm);
}

extern "C" lvq_status lvq_rope_table_perm(const lvq_geom* gp, const int32_t* perm, int32_t len, double base,
                                          float* cos_out, float* sin_out, void* f16_out, hipStream_t stream) {
    lvq::Geo g;
    lvq_status st = lvq::validate_geom(gp, &g);
    if (st != LVQ_OK) return st;
    st = lvq::check_channel_perm("lvq_rope_table_perm", g, perm);
    if (st != LVQ_OK) return st;
    LVQ_REQUIRE(len > 0, LVQ_ERR_INVALID_ARG, "lvq_rope_table_perm: bad len=%d", len);
    LVQ_REQUIRE(base > 1.0, LVQ_ERR_INVALID_ARG, "lvq_rope_table_perm: base must exceed 1");
    LVQ_REQUIRE((cos_out != nullptr) == (sin_out != nullptr) && (cos_out || f16_out), LVQ_ERR_INVALID_ARG,
                "lvq_rope_table_perm: give cos and sin tables, a packed table, or both");
    LVQ_REQUIRE(g.D / 2 <= kMaxHalf, LVQ_ERR_UNSUPPORTED, "lvq_rope_table_perm: D=%d (at most %d)", g.D,
                2 * kMaxHalf);
    LVQ_REQUIRE(!f16_out || g.D == 128, LVQ_ERR_UNSUPPORTED, "lvq_rope_table_perm: packed table for D=%d "
                "(128 supported)", g.D);
    FreqMap fm = identity_freqs();
    for (int j = 0; j < g.D / 2; ++j) fm.f[j] = int16_t(perm[j]);
    if (cos_out) {
        const long total = long(len) * (g.D / 2);
        hipLaunchKernelGGL(rope_table_kernel, dim3(grid_for(total, 256)), dim3(256), 0, stream, len, g.D, base,
                           cos_out, sin_out, fm);
        st = check_launch("lvq_rope_table_perm");
        if (st != LVQ_OK) return st;
    }
    if (f16_out) {
        hipLaunchKernelGGL(rope_f16_kernel, dim3(grid_for(long(len) * 64, 256)), dim3(256), 0, stream, len,
                           base, static_cast<_Float16*>(f16_out), fm);
        st = check_launch("lvq_rope_table_perm");
    }
    return st;
}

extern "C" lvq_status lvq_encode(const lvq_geom* g, int32_t block, const void* x_k, const void* x_v,
                                 const int64_t x_strides[4], const int64_t* x_tok0, const void* codebooks,
                                 uint8_t* pool, const int32_t* page_table, int32_t pt_stride,
                                 const int32_t* first_page, const int32_t* n_pages, int32_t B,
                                 int32_t max_pages, hipStream_t stream) {
    Geo geo;
    lvq_status st = validate_geom(g, &geo);
    if (st != LVQ_OK) return st;
    LVQ_REQUIRE(block >= 0 && block < geo.NB, LVQ_ERR_INVALID_ARG, "lvq_encode: block %d out of [0,%d)", block,
                geo.NB);
    LVQ_REQUIRE(x_k || x_v, LVQ_ERR_INVALID_ARG, "lvq_encode: both x_k and x_v are NULL");
    LVQ_REQUIRE(x_strides && codebooks && pool && page_table && first_page && n_pages, LVQ_ERR_INVALID_ARG,
                "lvq_encode: NULL pointer");
    LVQ_REQUIRE(B >= 0 && max_pages >= 0 && pt_stride >= 0, LVQ_ERR_INVALID_ARG, "lvq_encode: negative size");
    LVQ_REQUIRE(B <= 65535, LVQ_ERR_UNSUPPORTED, "lvq_encode: batch %d above 65535", B);
    if (B == 0 || max_pages == 0) return LVQ_OK;
    LVQ_REQUIRE(max_pages <= 0x7fffffff, LVQ_ERR_UNSUPPORTED, "lvq_encode: too many pages");
    // The matrix-core encoder takes whole 8-coordinate operand fragments and interleaves T_c in {1, 2, 4, 8}
    // loop steps per fragment; other shapes take the exact scan.
    const bool mfma_shape = geo.G % 8 == 0 && (geo.Tc == 1 || geo.Tc == 2 || geo.Tc == 4 || geo.Tc == 8);
    if (geo.cb == LVQ_BF16 && mfma_shape && geo.NG % 8 == 0) {
        EncArgs ea{geo, block, static_cast<const uint16_t*>(x_k), static_cast<const uint16_t*>(x_v),
                   long(x_strides[0]), long(x_strides[1]), long(x_strides[2]), long(x_strides[3]), x_tok0,
                   static_cast<const uint16_t*>(codebooks), pool, page_table, pt_stride, first_page, n_pages,
                   geo.NG / 8, B, 0};
        const long tokens = long(max_pages) * geo.page;
        constexpr long kBlk = kEncTile * kEncTilesPerWg;
        if (tokens <= 64 && long(B) * tokens <= 0x7fff0000L) {
            // few pages per request: token slots of all requests per workgroup, codebooks loaded once per
            // head for the whole batch
            ea.B = B;
            ea.tpr = int(tokens);
            const dim3 grid(unsigned((long(B) * tokens + kBlk - 1) / kBlk), geo.H * 2 * (geo.NG / 8), 1);
            switch (geo.Tc) {
                case 1: hipLaunchKernelGGL((encode_mfma_kernel<1, true>), grid, dim3(512), 0, stream, ea); break;
                case 2: hipLaunchKernelGGL((encode_mfma_kernel<2, true>), grid, dim3(512), 0, stream, ea); break;
                case 4: hipLaunchKernelGGL((encode_mfma_kernel<4, true>), grid, dim3(512), 0, stream, ea); break;
                case 8: hipLaunchKernelGGL((encode_mfma_kernel<8, true>), grid, dim3(512), 0, stream, ea); break;
                default: break;
            }
            return check_launch("lvq_encode");
        }
        // token blocks fastest and a multiple of 8: the octets of one block share an XCD's L2
        const long nblk = (tokens + kBlk - 1) / kBlk;
        LVQ_REQUIRE(nblk <= 0x7ffffff8L, LVQ_ERR_UNSUPPORTED, "lvq_encode: too many pages");
        const dim3 grid(unsigned((nblk + 7) / 8 * 8), geo.H * 2 * (geo.NG / 8), B);
        switch (geo.Tc) {
            case 1: hipLaunchKernelGGL((encode_mfma_kernel<1, false>), grid, dim3(512), 0, stream, ea); break;
            case 2: hipLaunchKernelGGL((encode_mfma_kernel<2, false>), grid, dim3(512), 0, stream, ea); break;
            case 4: hipLaunchKernelGGL((encode_mfma_kernel<4, false>), grid, dim3(512), 0, stream, ea); break;
            case 8: hipLaunchKernelGGL((encode_mfma_kernel<8, false>), grid, dim3(512), 0, stream, ea); break;
            default: break;
        }
        return check_launch("lvq_encode");
    }
    const dim3 grid(max_pages, geo.H * 2, B);
    const dim3 threads(geo.page * geo.NG);
    if (geo.cb == LVQ_BF16)
        hipLaunchKernelGGL(encode_scan_kernel<uint16_t>, grid, threads, 0, stream, geo, block,
                           static_cast<const uint16_t*>(x_k), static_cast<const uint16_t*>(x_v),
                           long(x_strides[0]), long(x_strides[1]), long(x_strides[2]), long(x_strides[3]),
                           x_tok0, static_cast<const uint16_t*>(codebooks), pool, page_table, pt_stride,
                           first_page, n_pages);
    else
        hipLaunchKernelGGL(encode_scan_kernel<float>, grid, threads, 0, stream, geo, block,
                           static_cast<const uint16_t*>(x_k), static_cast<const uint16_t*>(x_v),
                           long(x_strides[0]), long(x_strides[1]), long(x_strides[2]), long(x_strides[3]),
                           x_tok0, static_cast<const float*>(codebooks), pool, page_table, pt_stride,
                           first_page, n_pages);
    return check_launch("lvq_encode");
}

// ---------------------------------------------------------------------------
// Weighted codebook update: one Lloyd step of Fisher-weighted k-means (LoopVQ page: background
// "Fisher-weighted k-means" and "method steps" step 2).  The assignment is the encoder's (a scalar
// weight scales all of a sample's distances alike, so the nearest codeword does not depend on it): run
// lvq_encode on the calibration pages first.  Then every coupled vector z of those pages, with weight w,
// adds w*z and w to the sums of the codeword its page holds, and each codeword of loop block `block`
// becomes sum(w z) / sum(w), rounded once to the codebook dtype, or keeps its value when its cluster's
// weight sum is not positive.
//
// The sums are exact fixed-point integers, not float atomics (on this chip an fp32 add to LDS runs at
// about 1/40 of the rate of an integer one).  A workgroup first scans its samples for a = max |w z_k|
// and m = max |w| and counts them (N); then w*z (exact in fp64: a 24-bit times an 8-bit significand) is
// scaled by 2^e with N * a * 2^e < 2^51, rounded to the nearest integer and added into a 64-bit LDS
// sum, likewise w with its own 2^ew.  No sum can reach 2^52, each addend is off by at most 2^-e / 2
// (relative 2^-52 of the largest term times N), and integer adds commute, so the result does not
// depend on the order of the adds.  A NaN or infinite weight or coordinate makes the whole group's
// codebook NaN.
// ---------------------------------------------------------------------------
namespace lvq {
namespace {

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;          // NaN stays NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

// Round a double once to bf16 (nearest, ties to even).  The fp32 step rounds to nearest too; where it
// lands exactly halfway between two bf16 values without d being there, nudge it one fp32 step towards
// d so that the second rounding goes the way d does.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double d) {
    const float f = float(d);
    uint32_t u = __float_as_uint(f);
    if ((u & 0xffffu) == 0x8000u && double(f) != d) u = fabs(d) > fabs(double(f)) ? u + 1 : u - 1;
    return f32_to_bf16_rne(__uint_as_float(u));
}

// x * 2^e rounded to the nearest integer (ties to even), for |x| < 2^51: adding 1.5 * 2^52 leaves the
// integer in the low significand bits.
__device__ __forceinline__ long long round_to_int(double x) {
    constexpr double kMagic = 6755399441055744.0;                     // 1.5 * 2^52
    return __double_as_longlong(x + kMagic) - __double_as_longlong(kMagic);
}

// Scale exponent for N terms of magnitude at most `amax`: the largest e with N * amax * 2^e < 2^51.
__device__ __forceinline__ int sum_exponent(double amax, long n) {
    if (!(amax > 0.0)) return 0;
    int ex;
    frexp(amax * double(n) * (1.0 + 0x1p-20), &ex);                   // amax * n < 2^ex
    return 51 - ex;
}

// One workgroup per (head, K|V, group): its threads take the sampled tokens of all requests in turn
// (request b, page slot, token of the page) and, after a barrier, turn the 256 sums into codewords.  No
// other workgroup touches them.
//
// A group's channels are 2c bytes of each 256-byte step row, so the NG workgroups of one (head, K|V)
// read the same cache lines.  Workgroups go to the 8 XCDs round-robin by linear id; with XCD_MAP the id
// is split as (slot s = id / 8, XCD x = id % 8) and the (head, K|V) pair x + 8 * (s / NG) takes group
// s % NG, so that all groups of one pair run on one XCD and share its L2 (needs 2H % 8 == 0).
// VEC: a group's c channels of one step are read as one 2c-byte load (x 2c-byte aligned, strides
// multiples of c).
constexpr int kKmThreads = 1024;

template <int C>
struct VecOf;
template <>
struct VecOf<4> { using type = uint2; };
template <>
struct VecOf<8> { using type = uint4; };

// The G coordinates of one token's coupled vector as floats in slots z[0 .. G-1] (fixed slots, so that
// z stays in registers).  VEC_C > 0: slot m*c + i holds step m, channel g*c + i (one vector load per
// step); otherwise slot k holds coordinate k.  km_coord gives the coordinate of a slot: coordinate
// i*Tc + m <- step m, channel g*c + i.
template <int VEC_C>
__device__ __forceinline__ void load_coupled(const uint16_t* xb, long s3, int Tc, int G, float (&z)[32]) {
    if constexpr (VEC_C > 0) {
        using V = typename VecOf<VEC_C>::type;
        constexpr int kMaxTc = 32 / VEC_C;
#pragma unroll
        for (int m = 0; m < kMaxTc; ++m) {
            if (m < Tc) {
                const V v = *reinterpret_cast<const V*>(xb + long(m) * s3);
                const uint32_t* u = reinterpret_cast<const uint32_t*>(&v);
#pragma unroll
                for (int i = 0; i < VEC_C; ++i)
                    z[m * VEC_C + i] = bf16_to_f32(uint16_t(i & 1 ? u[i >> 1] >> 16 : u[i >> 1] & 0xffffu));
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < 32; ++k)
            if (k < G) z[k] = bf16_to_f32(xb[long(k % Tc) * s3 + k / Tc]);
    }
}

template <int VEC_C>
__device__ __forceinline__ int km_coord(int k, int Tc) {
    if constexpr (VEC_C > 0) return (k % VEC_C) * Tc + k / VEC_C;
    else return k;
}

template <typename CB, bool XCD_MAP, int VEC_C>
__global__ void __launch_bounds__(kKmThreads) kmeans_update_kernel(
        Geo geo, int block, const uint16_t* __restrict__ xk, const uint16_t* __restrict__ xv, long s0, long s1,
        long s2, long s3, const int64_t* __restrict__ tok0, const float* __restrict__ wk,
        const float* __restrict__ wv, long w0, long w1, long w2, const uint8_t* __restrict__ pool,
        const int32_t* __restrict__ pt, int pt_stride, const int32_t* __restrict__ first_page,
        const int32_t* __restrict__ n_pages, int B, int max_pages, CB* __restrict__ cb) {
    __shared__ unsigned long long sums[256 * 33];   // [K][G + 1]: sum of w z (G) and of w, fixed point
    __shared__ unsigned long long bound[2];         // max |w z_k|, max |w| (non-negative doubles as bits)
    __shared__ uint32_t nonfinite;
    const int NG = geo.NG, c = geo.c, Tc = geo.Tc, G = geo.G, K = geo.K;
    int g, pair;
    if constexpr (XCD_MAP) {
        const int id = blockIdx.x, slot = id >> 3;
        g = slot % NG;
        pair = (id & 7) + 8 * (slot / NG);
    } else {
        g = blockIdx.x % NG;
        pair = blockIdx.x / NG;
    }
    const int h = pair >> 1, kv = pair & 1;
    const uint16_t* x = kv == 0 ? xk : xv;
    const float* wt = kv == 0 ? wk : wv;
    if (x == nullptr) return;
    for (int e = threadIdx.x; e < K * (G + 1); e += kKmThreads) sums[e] = 0ull;
    if (threadIdx.x == 0) {
        bound[0] = bound[1] = 0ull;
        nonfinite = 0u;
    }
    __syncthreads();

    // pass 1: bounds and sample count
    long n_tok = 0;
    double amax = 0.0, wmax = 0.0;
    bool bad = false;
    for (int b = 0; b < B; ++b) {
        const int np = min(n_pages[b], max_pages);
        const long row0 = tok0 ? tok0[b] : 0;
        n_tok += long(np) * geo.page;
        for (int j = threadIdx.x; j < np * geo.page; j += kKmThreads) {
            const long row = row0 + j;
            const float w = wt[long(b) * w0 + long(h) * w1 + row * w2 + g];
            float z[32];
            load_coupled<VEC_C>(x + long(b) * s0 + long(h) * s1 + row * s2 + g * c, s3, Tc, G, z);
            float zmax = 0.f;
            bool zbad = false;
#pragma unroll
            for (int k = 0; k < 32; ++k)
                if (k < G) {
                    zmax = fmaxf(zmax, fabsf(z[k]));
                    zbad |= !(fabsf(z[k]) <= 3.4028235e38f);
                }
            bad |= zbad || !(fabsf(w) <= 3.4028235e38f);
            amax = fmax(amax, double(fabsf(w)) * double(zmax));
            wmax = fmax(wmax, double(fabsf(w)));
        }
    }
    if (bad) atomicOr(&nonfinite, 1u);
    for (int off = 32; off > 0; off >>= 1) {
        amax = fmax(amax, __shfl_xor(amax, off));
        wmax = fmax(wmax, __shfl_xor(wmax, off));
    }
    if ((threadIdx.x & 63) == 0) {
        atomicMax(&bound[0], static_cast<unsigned long long>(__double_as_longlong(amax)));
        atomicMax(&bound[1], static_cast<unsigned long long>(__double_as_longlong(wmax)));
    }
    __syncthreads();
    const int ez = sum_exponent(__longlong_as_double(static_cast<long long>(bound[0])), n_tok);
    const int ew = sum_exponent(__longlong_as_double(static_cast<long long>(bound[1])), n_tok);
    const double scale_z = ldexp(1.0, ez), scale_w = ldexp(1.0, ew);

    // pass 2: fixed-point sums per codeword
    if (nonfinite == 0u) {
        const long blk_off = ((long(block) * geo.H + h) * 2 + kv) * geo.page * NG;
        for (int b = 0; b < B; ++b) {
            const int np = min(n_pages[b], max_pages), fp = first_page[b];
            const long row0 = tok0 ? tok0[b] : 0;
            for (int j = threadIdx.x; j < np * geo.page; j += kKmThreads) {
                const int slot = j / geo.page, i_tok = j % geo.page;
                const int lp = fp + slot;
                const long row = row0 + j;
                // the page id, the token's data and its weight are loaded together; only the index byte waits
                const long phys = pt[long(b) * pt_stride + lp];
                const float w = wt[long(b) * w0 + long(h) * w1 + row * w2 + g];
                float z[32];
                load_coupled<VEC_C>(x + long(b) * s0 + long(h) * s1 + row * s2 + g * c, s3, Tc, G, z);
                const int tau = slot_token(lp, i_tok, geo.page);
                const int byte = index_byte(kv, NG, g, tau);         // index rows permuted (lvq.h)
                const int r = pool[phys * geo.page_bytes + blk_off + i_tok * NG + byte];
                unsigned long long* acc = sums + r * (G + 1);
                const double wz = double(w) * scale_z;                // exact: a power-of-two scale
#pragma unroll
                for (int k = 0; k < 32; ++k)
                    if (k < G)
                        atomicAdd(acc + km_coord<VEC_C>(k, Tc),
                                  static_cast<unsigned long long>(round_to_int(wz * double(z[k]))));
                atomicAdd(acc + G, static_cast<unsigned long long>(round_to_int(double(w) * scale_w)));
            }
        }
    }
    __syncthreads();
    CB* out = cb + ((((long(block) * geo.H + h) * 2 + kv) * NG + g) * K) * G;
    const bool all_nan = nonfinite != 0u;
    for (int e = threadIdx.x; e < K * G; e += kKmThreads) {
        const int r = e / G, k = e % G;
        double v;
        if (all_nan) {
            v = __longlong_as_double(0x7ff8000000000000LL);
        } else {
            const long long den = static_cast<long long>(sums[r * (G + 1) + G]);
            if (den <= 0) continue;                                   // empty cluster: the codeword stays
            v = ldexp(double(static_cast<long long>(sums[r * (G + 1) + k])) / double(den), ew - ez);
        }
        if constexpr (std::is_same<CB, uint16_t>::value) out[e] = f64_to_bf16_rne(v);
        else out[e] = float(v);
    }
}

struct KmArgs {
    Geo geo;
    int block;
    const uint16_t *xk, *xv;
    long s0, s1, s2, s3;
    const int64_t* tok0;
    const float *wk, *wv;
    long w0, w1, w2;
    const uint8_t* pool;
    const int32_t* pt;
    int pt_stride;
    const int32_t *first_page, *n_pages;
    int B, max_pages;
};

template <typename CB, bool XCD_MAP, int VEC_C>
void launch_kmeans(const KmArgs& a, void* cb, hipStream_t stream) {
    const dim3 grid(unsigned(a.geo.NG * 2 * a.geo.H));
    hipLaunchKernelGGL((kmeans_update_kernel<CB, XCD_MAP, VEC_C>), grid, dim3(kKmThreads), 0, stream, a.geo,
                       a.block, a.xk, a.xv, a.s0, a.s1, a.s2, a.s3, a.tok0, a.wk, a.wv, a.w0, a.w1, a.w2, a.pool,
                       a.pt, a.pt_stride, a.first_page, a.n_pages, a.B, a.max_pages, static_cast<CB*>(cb));
}

template <typename CB, bool XCD_MAP>
void launch_kmeans_vec(const KmArgs& a, int vec_c, void* cb, hipStream_t stream) {
    if (vec_c == 8) launch_kmeans<CB, XCD_MAP, 8>(a, cb, stream);
    else if (vec_c == 4) launch_kmeans<CB, XCD_MAP, 4>(a, cb, stream);
    else launch_kmeans<CB, XCD_MAP, 0>(a, cb, stream);
}

template <typename CB>
void launch_kmeans_map(const KmArgs& a, int vec_c, void* cb, hipStream_t stream) {
    if ((2 * a.geo.H) % 8 == 0) launch_kmeans_vec<CB, true>(a, vec_c, cb, stream);
    else launch_kmeans_vec<CB, false>(a, vec_c, cb, stream);
}

}  // namespace
}  // namespace lvq

extern "C" lvq_status lvq_codebook_update(const lvq_geom* g, int32_t block, const void* x_k, const void* x_v,
                                          const int64_t x_strides[4], const int64_t* x_tok0, const float* w_k,
                                          const float* w_v, const int64_t w_strides[3], void* codebooks,
                                          const uint8_t* pool, const int32_t* page_table, int32_t pt_stride,
                                          const int32_t* first_page, const int32_t* n_pages, int32_t B,
                                          int32_t max_pages, hipStream_t stream) {
    Geo geo;
    lvq_status st = validate_geom(g, &geo);
    if (st != LVQ_OK) return st;
    LVQ_REQUIRE(block >= 0 && block < geo.NB, LVQ_ERR_INVALID_ARG, "lvq_codebook_update: block %d out of [0,%d)",
                block, geo.NB);
    LVQ_REQUIRE(x_k || x_v, LVQ_ERR_INVALID_ARG, "lvq_codebook_update: both x_k and x_v are NULL");
    LVQ_REQUIRE((!x_k || w_k) && (!x_v || w_v), LVQ_ERR_INVALID_ARG, "lvq_codebook_update: missing weights");
    LVQ_REQUIRE(x_strides && w_strides && codebooks && pool && page_table && first_page && n_pages,
                LVQ_ERR_INVALID_ARG, "lvq_codebook_update: NULL pointer");
    LVQ_REQUIRE(B >= 0 && max_pages >= 0 && pt_stride >= 0, LVQ_ERR_INVALID_ARG,
                "lvq_codebook_update: negative size");
    LVQ_REQUIRE(geo.G <= 32, LVQ_ERR_UNSUPPORTED, "lvq_codebook_update: G=%d (at most 32)", geo.G);
    LVQ_REQUIRE(long(max_pages) * geo.page <= 0x7fffffffL, LVQ_ERR_UNSUPPORTED, "lvq_codebook_update: too many pages");
    if (B == 0 || max_pages == 0) return LVQ_OK;
    KmArgs a{geo, int(block), static_cast<const uint16_t*>(x_k), static_cast<const uint16_t*>(x_v),
             long(x_strides[0]), long(x_strides[1]), long(x_strides[2]), long(x_strides[3]), x_tok0, w_k, w_v,
             long(w_strides[0]), long(w_strides[1]), long(w_strides[2]), pool, page_table, int(pt_stride),
             first_page, n_pages, int(B), int(max_pages)};
    // one vector load per (token, step) when every row start of every given tensor is 2c-byte aligned
    int vec_c = (geo.c == 4 || geo.c == 8) ? geo.c : 0;
    for (const void* p : {x_k, x_v})
        if (p && reinterpret_cast<uintptr_t>(p) % (2 * geo.c) != 0) vec_c = 0;
    for (int i = 0; i < 4; ++i)
        if (vec_c && x_strides[i] % geo.c != 0) vec_c = 0;
    if (geo.cb == LVQ_BF16) launch_kmeans_map<uint16_t>(a, vec_c, codebooks, stream);
    else launch_kmeans_map<float>(a, vec_c, codebooks, stream);
    return check_launch("lvq_codebook_update");
}
