// Thread-local error messages and launch checks for the C ABI.
#include "common.h"

namespace lvq {

namespace {
thread_local char g_msg[512] = "";
}

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
    va_end(ap);
}

void clear_error() { g_msg[0] = '\0'; }

lvq_status check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_error("%s: %s", what, hipGetErrorString(e));
        return LVQ_ERR_HIP;
    }
    return LVQ_OK;
}

}  // namespace lvq

extern "C" const char* lvq_last_error(void) { return lvq::g_msg; }

namespace lvq {

lvq_status validate_geom(const lvq_geom* g, Geo* o) {
    LVQ_REQUIRE(g != nullptr, LVQ_ERR_INVALID_ARG, "geometry is NULL");
    LVQ_REQUIRE(g->D > 0 && g->T > 0 && g->Tc > 0 && g->G > 0 && g->K > 0 && g->page > 0 &&
                    g->sink >= 0 && g->window >= 0 && g->H > 0,
                LVQ_ERR_INVALID_ARG, "geometry has a non-positive size");
    LVQ_REQUIRE(g->T % g->Tc == 0 && g->G % g->Tc == 0, LVQ_ERR_INVALID_ARG,
                "T_c=%d must divide T=%d and G=%d", g->Tc, g->T, g->G);
    LVQ_REQUIRE(g->D == 128, LVQ_ERR_UNSUPPORTED, "head dimension %d unsupported (128)", g->D);
    LVQ_REQUIRE(g->K == 256, LVQ_ERR_UNSUPPORTED, "K=%d codewords unsupported (256, 8-bit indices)", g->K);
    LVQ_REQUIRE(g->page == 8, LVQ_ERR_UNSUPPORTED, "page of %d tokens unsupported (8)", g->page);
    const int c = g->G / g->Tc;
    LVQ_REQUIRE(c == 4 || c == 8, LVQ_ERR_UNSUPPORTED, "c = G/T_c = %d unsupported (4 or 8)", c);
    LVQ_REQUIRE(g->G <= 32, LVQ_ERR_UNSUPPORTED, "codeword dimension G=%d unsupported (at most 32)", g->G);
    LVQ_REQUIRE(g->window % g->page == 0, LVQ_ERR_UNSUPPORTED,
                "window %d must be a multiple of the page size", g->window);
    LVQ_REQUIRE(g->cb_dtype == LVQ_BF16 || g->cb_dtype == LVQ_FP32, LVQ_ERR_UNSUPPORTED,
                "codebook dtype %d unsupported", g->cb_dtype);
    o->D = g->D; o->T = g->T; o->Tc = g->Tc; o->G = g->G; o->K = g->K; o->page = g->page;
    o->sink = g->sink; o->W = g->window; o->H = g->H; o->cb = g->cb_dtype;
    o->c = c;
    o->NG = g->D / c;
    o->NB = g->T / g->Tc;
    o->Wcap = g->sink + g->window + g->page;
    o->page_bytes = long(o->NB) * o->H * 2 * o->page * o->NG;
    o->cb_bytes = g->cb_dtype == LVQ_BF16 ? 2 : 4;
    return LVQ_OK;
}

}  // namespace lvq
