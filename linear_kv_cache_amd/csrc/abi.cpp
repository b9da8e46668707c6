// Host-only parts of the C ABI: error reporting, version, KV-cache layout arithmetic.
#include <math.h>
#include <stdio.h>

#include <algorithm>
#include <string>
#include <vector>

#include "rf_internal.h"

namespace rf {

static thread_local std::string g_last_error;

rf_status fail(rf_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}

void clear_error() { g_last_error.clear(); }

rf_status check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(RF_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
    return RF_OK;
}

}  // namespace rf

extern "C" {

const char* rf_version(void) { return "ridgefill 0.1.0 gfx950"; }

const char* rf_last_error(void) { return rf::g_last_error.c_str(); }

rf_status rf_cache_layout(const rf_cache_desc* desc, rf_cache_layout_t* out) {
    rf::clear_error();
    RF_REQUIRE(desc && out, RF_ERR_INVALID_ARG, "rf_cache_layout: null argument");
    RF_REQUIRE(desc->n_kv_heads > 0 && desc->head_dim > 0 && desc->max_tokens >= 0, RF_ERR_INVALID_ARG,
               "rf_cache_layout: n_kv_heads, head_dim must be > 0 and max_tokens >= 0");
    RF_REQUIRE(rf::valid_dtype(desc->dtype), RF_ERR_INVALID_ARG, "rf_cache_layout: bad dtype");
    const int64_t H = desc->n_kv_heads, dh = desc->head_dim;
    rf_cache_layout_t L{};
    L.elem_bytes = (int64_t)rf::elem_bytes(desc->dtype);
    if (desc->layout == RF_LAYOUT_CONTIGUOUS) {
        L.n_blocks = desc->max_tokens;
        L.stride_block = 0;
        L.stride_token = H * dh;
        L.stride_head = dh;
        L.bytes_per_pool = desc->max_tokens * H * dh * L.elem_bytes;
    } else if (desc->layout == RF_LAYOUT_PAGED) {
        RF_REQUIRE(desc->block_size > 0, RF_ERR_INVALID_ARG, "rf_cache_layout: block_size must be > 0");
        const int64_t bs = desc->block_size;
        L.n_blocks = rf::ceil_div(desc->max_tokens, bs);
        L.stride_block = H * bs * dh;
        L.stride_head = bs * dh;
        L.stride_token = dh;
        L.bytes_per_pool = L.n_blocks * L.stride_block * L.elem_bytes;
    } else {
        return rf::fail(RF_ERR_INVALID_ARG, "rf_cache_layout: bad layout");
    }
    *out = L;
    return RF_OK;
}

rf_status rf_r2_assignment(const double* r2, int32_t n_tgt, int32_t n_src, int32_t nu, int32_t* out) {
    rf::clear_error();
    RF_REQUIRE(r2 && out, RF_ERR_INVALID_ARG, "rf_r2_assignment: null argument");
    RF_REQUIRE(n_tgt >= 0 && nu >= 1 && nu <= n_src, RF_ERR_INVALID_ARG,
               "rf_r2_assignment: need n_tgt >= 0 and 1 <= nu <= n_src");
    std::vector<int32_t> idx(n_src);
    for (int64_t l = 0; l < n_tgt; ++l) {
        const double* row = r2 + l * n_src;
        for (int32_t s = 0; s < n_src; ++s) idx[s] = s;
        // highest score first (NaN ranks last); equal scores keep the shallower layer first
        auto key = [&](int32_t s) { return std::isnan(row[s]) ? -INFINITY : row[s]; };
        std::stable_sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) { return key(a) > key(b); });
        std::sort(idx.begin(), idx.begin() + nu);
        for (int32_t j = 0; j < nu; ++j) out[l * nu + j] = idx[j];
    }
    return RF_OK;
}

rf_status rf_relative_depth_sources(int32_t n_src, int32_t n_tgt, int32_t nu, int32_t* out) {
    rf::clear_error();
    RF_REQUIRE(out, RF_ERR_INVALID_ARG, "rf_relative_depth_sources: null output");
    RF_REQUIRE(n_tgt >= 1 && nu >= 1 && nu <= n_src, RF_ERR_INVALID_ARG,
               "rf_relative_depth_sources: need n_tgt >= 1 and 1 <= nu <= n_src");
    // c(l) - 1 = a / q with a = (l - 1)(n_src - 1), q = n_tgt - 1 (c = 1 when n_tgt = 1).  The
    // band start s = round-half-up(c - (nu - 1)/2) = floor((2a + q(4 - nu)) / (2q)), clamped to
    // [1, n_src - nu + 1] (1-based).
    const int64_t q = n_tgt > 1 ? n_tgt - 1 : 1;
    for (int64_t l = 0; l < n_tgt; ++l) {
        const int64_t a = n_tgt > 1 ? l * (int64_t)(n_src - 1) : 0;
        const int64_t num = 2 * a + q * (4 - (int64_t)nu), den = 2 * q;
        int64_t s = num >= 0 ? num / den : -((-num + den - 1) / den);
        s = std::min<int64_t>(std::max<int64_t>(s, 1), (int64_t)n_src - nu + 1);
        for (int32_t j = 0; j < nu; ++j) out[l * nu + j] = (int32_t)(s - 1 + j);
    }
    return RF_OK;
}

}  // extern "C"
