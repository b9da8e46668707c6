// Host-side helpers shared by the library's translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "ridgefill.h"

namespace rf {

// Records the message for rf_last_error() on this thread and returns ``st``.
rf_status fail(rf_status st, const std::string& msg);
void clear_error();

// Checks the last launch (hipGetLastError) and converts a failure into RF_ERR_HIP.
rf_status check_launch(const char* what);

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }
__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t round_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

inline size_t elem_bytes(rf_dtype t) { return t == RF_F32 ? 4 : 2; }
// Width of each target's rows (and of its map's output): d_out, or d when d_out is 0.
inline int64_t gram_dy(const rf_gram_desc* g) { return g->d_out > 0 ? g->d_out : g->d; }
inline bool valid_dtype(rf_dtype t) { return t == RF_F32 || t == RF_BF16; }

// Head-wise translators on their own kernel (headwise.hip): BF16 maps with headwise = 1 and
// d_in = nu * n_kv_heads * head_dim, nu in 1..2.  Arguments validated by rf_translate.
bool translate_headwise_supported(const rf_translate_weights* w);
rf_status launch_translate_headwise(const rf_translate_weights* w, int32_t n_layers, const void* const* src_k,
                                    const void* const* src_v, int64_t ld_src, int64_t t0, int64_t t1, int64_t pos0,
                                    const rf_cache_desc* cache, const rf_cache_layout_t& L, void* const* kc,
                                    void* const* vc, const int32_t* table, int64_t n_table, const float* rope,
                                    hipStream_t stream);

}  // namespace rf

#define RF_REQUIRE(cond, status, msg)                  \
    do {                                               \
        if (!(cond)) return ::rf::fail((status), (msg)); \
    } while (0)
