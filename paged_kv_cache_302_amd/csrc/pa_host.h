// Host-side helpers shared by the libpa entry points: argument checks and
// launch error mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

inline int check_head_block(int head_size, int block_size) {
    if (block_size != 16) return PA_ERR_UNSUPPORTED;
    if (head_size != 64 && head_size != 128) return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

// kv_cache_dtype: PA_KV_FP16 (scales ignored) or PA_KV_FP8_E4M3 (scales
// positive and finite)
inline int check_kv_dtype(int kv_cache_dtype, float k_scale, float v_scale) {
    if (kv_cache_dtype == PA_KV_FP16) return PA_OK;
    if (kv_cache_dtype != PA_KV_FP8_E4M3) return PA_ERR_UNSUPPORTED;
    if (!(k_scale > 0.f) || !(v_scale > 0.f) || !__builtin_isfinite(k_scale) ||
        !__builtin_isfinite(v_scale))
        return PA_ERR_INVALID_ARG;
    return PA_OK;
}

inline int kv_elem_bytes(int kv_cache_dtype) { return kv_cache_dtype == PA_KV_FP8_E4M3 ? 1 : 2; }

inline int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace pa
