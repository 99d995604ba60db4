// Device helpers for the gfx950 paged-attention kernels: vector types,
// wavefront (64-lane) cross-lane moves and reductions, and exp2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kBlock = 16;       // tokens per KV block
constexpr int kX = 8;            // fp16 elements per 16-byte K chunk
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float as_float(int v) { return __builtin_bit_cast(float, v); }
__device__ __forceinline__ int as_int(float v) { return __builtin_bit_cast(int, v); }

// v_exp_f32: 2^x, exact at 0 (gives 1), 0 at -inf.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane (lane ^ 16), via ds_swizzle in bit-mask mode
// (and_mask 0x1f, xor_mask 0x10): stays inside each 32-lane half.
__device__ __forceinline__ float xor16(float v) {
    return as_float(__builtin_amdgcn_ds_swizzle(as_int(v), 0x401F));
}

// Value held by lane (lane ^ 32), through the LDS crossbar (ds_bpermute).
__device__ __forceinline__ float xor32(float v) {
    return as_float(__builtin_amdgcn_ds_bpermute((lane_id() ^ 32) << 2, as_int(v)));
}

// Value held by lane `src` (any lane), through ds_bpermute.
__device__ __forceinline__ int fetch_lane(int v, int src) {
    return __builtin_amdgcn_ds_bpermute(src << 2, v);
}

// DPP moves inside a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return as_float(__builtin_amdgcn_update_dpp(0, as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;     // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4E;     // quad_perm(2,3,0,1)
constexpr int kDppRor4 = 0x124;    // row_ror:4
constexpr int kDppRor8 = 0x128;    // row_ror:8

// Max / sum over the 16 lanes of each row (every lane of the row gets it).
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp<kDppXor1>(v));
    v = fmaxf(v, dpp<kDppXor2>(v));
    v = fmaxf(v, dpp<kDppRor4>(v));
    v = fmaxf(v, dpp<kDppRor8>(v));
    return v;
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppRor4>(v);
    v += dpp<kDppRor8>(v);
    return v;
}

// Max / sum over the four lanes {l, l^16, l^32, l^48} (same column of the
// four 16-lane rows).
__device__ __forceinline__ float col4_max(float v) {
    v = fmaxf(v, xor16(v));
    return fmaxf(v, xor32(v));
}
__device__ __forceinline__ float col4_sum(float v) {
    v += xor16(v);
    return v + xor32(v);
}

// Full-wave reductions (all lanes receive the result).
__device__ __forceinline__ float wave_max(float v) { return col4_max(row16_max(v)); }
__device__ __forceinline__ float wave_sum(float v) { return col4_sum(row16_sum(v)); }

// fp32 accumulate of two fp16 products: a.x*b.x + a.y*b.y + c (v_dot2_f32_f16).
__device__ __forceinline__ float dot2(f16x2 a, f16x2 b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
}

__device__ __forceinline__ f16x2 pack2(float a, float b) {
    return f16x2{(f16)a, (f16)b};
}

}  // namespace pa
