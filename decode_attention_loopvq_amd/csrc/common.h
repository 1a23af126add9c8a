// Internal helpers shared by the liblvq sources (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "lvq.h"

namespace lvq {

// ---------------------------------------------------------------------------
// Error reporting: every entry point validates, sets a thread-local message
// and returns a status before launching anything.
// ---------------------------------------------------------------------------
void set_error(const char* fmt, ...);
void clear_error();

#define LVQ_REQUIRE(cond, status, ...)          \
    do {                                        \
        if (!(cond)) {                          \
            ::lvq::set_error(__VA_ARGS__);      \
            return (status);                    \
        }                                       \
    } while (0)

// Check the launch that was just enqueued.
lvq_status check_launch(const char* what);

// ---------------------------------------------------------------------------
// Device-side scalar conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return float(v);
}
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
    _Float16 v = (_Float16)f;   // v_cvt_f16_f32: round to nearest even
    uint16_t h;
    __builtin_memcpy(&h, &v, 2);
    return h;
}

// ---------------------------------------------------------------------------
// The packed fp16 RoPE table of the index-page kernels (D = 128), 384 halves (768 B) per position, in two
// parts: part A [rope_len][32 chunks][8] (chunk m < 16 of position p: cos of frequencies
// 4m .. 4m+3, then sin of the same; chunk 16 + m: the same with the sines negated), read by the c = 8
// kernel, whose lanes take a position's chunks together; part B [16 chunks][rope_len][8] (chunks m < 16
// again, chunk-major), read by the c = 4 kernel, whose lanes of one load hold consecutive positions.
// ---------------------------------------------------------------------------
constexpr long kRopeF16HalvesPerPos = 384;
__device__ __forceinline__ void store_rope_f16(_Float16* __restrict__ out, long len, long p, int i, _Float16 c,
                                               _Float16 s) {
    const int m = i >> 2, k = i & 3;
    _Float16* a = out + (p * 32 + m) * 8;
    a[k] = c;
    a[4 + k] = s;
    a[16 * 8 + k] = c;
    a[16 * 8 + 4 + k] = -s;
    _Float16* b = out + len * 256 + (m * len + p) * 8;
    b[k] = c;
    b[4 + k] = s;
}

// Wave64 reductions through cross-lane moves.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}
// Wave64 maximum through DPP row rotations and four lane reads; the result is
// wave-uniform.  No LDS traffic (unlike cross-lane shuffles).
__device__ __forceinline__ float wave_max_dpp(float x) {
    // row_ror:8, 4, 2, 1 within each 16-lane row
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0x128, 0xf, 0xf, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0x124, 0xf, 0xf, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0x122, 0xf, 0xf, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0x121, 0xf, 0xf, false)));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

constexpr int kWave = 64;

inline int ceil_div(long a, long b) { return int((a + b - 1) / b); }

}  // namespace lvq

namespace lvq {

// LoopVQ geometry with the derived sizes every kernel uses.
struct Geo {
    int D, T, Tc, G, K, page, sink, W, H, cb;
    int c;        // channels per codeword per step, G / Tc
    int NG;       // index groups per token and step, D / c
    int NB;       // loop blocks, T / Tc
    int Wcap;     // window slots per (request, step, head): sink + W + page
    long page_bytes;   // bytes of one physical pool page: NB*H*2*page*NG
    int cb_bytes;      // bytes per codebook element
};

// Validate a caller's geometry; fills `out` on success.
lvq_status validate_geom(const lvq_geom* g, Geo* out);

// Byte position of group g in the index row of index-token tau (counted from the first paged position);
// layout in lvq.h.  Value rows: g ^ (tau & 15).  Key rows with 16 groups: the byte j with
// P(j) ^ (tau & 15) = g, P the fixed bit permutation (j3 j2 j1 j0) -> (j1 j3 j2 j0), so that the dword k of a
// key row holds groups {2k, 2k+1, 2k+8, 2k+9} ^ (tau & 15): two RoPE-paired group pairs.  Key rows with 32
// groups: g.
__host__ __device__ inline int index_byte(int kv, int NG, int g, int tau) {
    if (kv != 0) return g ^ (tau & 15);
    if (NG != 16) return g;
    const int b = g ^ (tau & 15);
    return (b & 1) | (((b >> 3) & 1) << 1) | (((b >> 1) & 1) << 2) | (((b >> 2) & 1) << 3);
}
// The group held by byte j of a key row with 16 groups (the inverse of index_byte for kv = 0).
__host__ __device__ inline int key_group_of_byte(int j, int tau) {
    const int p = (j & 1) | (((j >> 2) & 1) << 1) | (((j >> 3) & 1) << 2) | (((j >> 1) & 1) << 3);
    return p ^ (tau & 15);
}

// Supplies the workspace of a decode-attention call once its arguments are valid: given the bytes the call
// needs, sets *ws and *ws_bytes or returns an error.
using WorkspaceProvider = lvq_status (*)(size_t need, void** ws, size_t* ws_bytes);

// lvq_decode_attn with error messages naming `fn`; with a provider, the workspace comes from it (after every
// other argument has been checked) instead of from ws / ws_bytes.
lvq_status decode_attn_impl(const char* fn, const lvq_geom* gp, int32_t step, const void* q, const uint8_t* pool,
                            const int32_t* page_table, int32_t pt_stride, const int32_t* seq_len, int32_t max_len,
                            const int32_t* order, const void* k_scales, const void* win_k, const void* win_v,
                            const void* slices, const float* rope_cos, const float* rope_sin, const void* rope_f16,
                            int32_t rope_len, float sm_scale, float* out, float* lse_out, void* ws, size_t ws_bytes,
                            WorkspaceProvider provider, int32_t num_splits, int32_t B, hipStream_t stream);

}  // namespace lvq
