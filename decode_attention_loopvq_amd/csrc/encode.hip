// LoopVQ codebook slicing, RoPE table and index-page encoding.
//
// LoopVQ page ("LoopVQ: Sub 1-bit KV Cache Quantization for Looped
// Transformers"): "method steps" step 1 (loop-axis coupling), step 4 (paged
// index cache, encode after the block's last loop step, one page every 8
// generated tokens), step 5 (per-step codebook slice B_t cut once at load);
// background "RoPE" (precomputed cos/sin table).
#include "common.h"

#include <cmath>

namespace lvq {
namespace {

// ---------------------------------------------------------------------------
// B_t slices: slices[t][h][kv][g][r][i] = codebooks[t/Tc][h][kv][g][r][i*Tc + t%Tc]
// ---------------------------------------------------------------------------
template <typename E>
__global__ void slice_kernel(const E* __restrict__ cb, E* __restrict__ out, int T, int Tc, int H,
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
__global__ void rope_table_kernel(int len, int D, double base, float* __restrict__ cs,
                                  float* __restrict__ sn) {
    const int half = D / 2;
    const long total = long(len) * half;
    for (long e = blockIdx.x * long(blockDim.x) + threadIdx.x; e < total; e += long(gridDim.x) * blockDim.x) {
        const int p = int(e / half), i = int(e % half);
        const double theta = pow(base, -2.0 * double(i) / double(D));
        const double a = double(p) * theta;
        cs[e] = float(cos(a));
        sn[e] = float(sin(a));
    }
}

// ---------------------------------------------------------------------------
// Packed fp16 table for the index-page pass: chunk m (frequencies 4m..4m+3)
// of position p at out[(m * len + p) * 8 ..]: cos x4 then sin x4.
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

__global__ void rope_f16_kernel(int len, double base, _Float16* __restrict__ out) {
    const long total = long(len) * 64;
    for (long e = blockIdx.x * long(blockDim.x) + threadIdx.x; e < total; e += long(gridDim.x) * blockDim.x) {
        const int p = int(e / 64), i = int(e % 64);
        const double theta = pow(base, -2.0 * double(i) / 128.0);
        const double ang = double(p) * theta;
        const int m = i >> 2, k = i & 3;
        _Float16* o = out + (long(m) * len + p) * 8;
        o[k] = f64_to_f16_rn(cos(ang));
        o[4 + k] = f64_to_f16_rn(sin(ang));
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
    // Value rows are XOR-rotated by the index-token number (layout in lvq.h).
    const int tau = slot_token(lp, i_tok, geo.page);
    const int byte = kv == 0 ? g : (g ^ (tau & 15));
    pool[phys * geo.page_bytes + ((long(block) * geo.H + h) * 2 + kv) * geo.page * NG + i_tok * NG + byte] =
        uint8_t(best_r);
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
                           static_cast<const uint16_t*>(codebooks), static_cast<uint16_t*>(slices), geo.T,
                           geo.Tc, geo.H, geo.NG, geo.K, geo.G, total);
    else
        hipLaunchKernelGGL(slice_kernel<float>, dim3(grid_for(total, threads)), dim3(threads), 0, stream,
                           static_cast<const float*>(codebooks), static_cast<float*>(slices), geo.T, geo.Tc,
                           geo.H, geo.NG, geo.K, geo.G, total);
    return check_launch("lvq_slice_codebooks");
}

extern "C" lvq_status lvq_rope_table(int32_t len, int32_t D, double base, float* cos_out, float* sin_out,
                                     hipStream_t stream) {
    LVQ_REQUIRE(len > 0 && D > 0 && D % 2 == 0, LVQ_ERR_INVALID_ARG, "lvq_rope_table: bad len=%d D=%d", len, D);
    LVQ_REQUIRE(base > 1.0, LVQ_ERR_INVALID_ARG, "lvq_rope_table: base must exceed 1");
    LVQ_REQUIRE(cos_out && sin_out, LVQ_ERR_INVALID_ARG, "lvq_rope_table: NULL pointer");
    const long total = long(len) * (D / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3(grid_for(total, 256)), dim3(256), 0, stream, len, D, base,
                       cos_out, sin_out);
    return check_launch("lvq_rope_table");
}

extern "C" lvq_status lvq_rope_table_f16(int32_t len, int32_t D, double base, void* out, hipStream_t stream) {
    LVQ_REQUIRE(len > 0, LVQ_ERR_INVALID_ARG, "lvq_rope_table_f16: bad len=%d", len);
    LVQ_REQUIRE(D == 128, LVQ_ERR_UNSUPPORTED, "lvq_rope_table_f16: D=%d (128 supported)", D);
    LVQ_REQUIRE(base > 1.0, LVQ_ERR_INVALID_ARG, "lvq_rope_table_f16: base must exceed 1");
    LVQ_REQUIRE(out, LVQ_ERR_INVALID_ARG, "lvq_rope_table_f16: NULL pointer");
    hipLaunchKernelGGL(rope_f16_kernel, dim3(grid_for(long(len) * 64, 256)), dim3(256), 0, stream, len, base,
                       static_cast<_Float16*>(out));
    return check_launch("lvq_rope_table_f16");
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
