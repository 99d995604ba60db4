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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

// ---------------------------------------------------------------------------
// fp8 KV cache (OCP E4M3: sign, 4 exponent bits with bias 7, 3 mantissa bits,
// no infinity, S.1111.111 = NaN, largest finite 448)
// ---------------------------------------------------------------------------
constexpr int kX8 = 16;          // fp8 elements per 16-byte K chunk
constexpr float kE4M3Max = 448.f;

// Two E4M3 codes (bytes 0,1 of w, or 2,3 with HI) -> two fp16, exactly
// (every E4M3 value is an fp16 value; NaN stays NaN).
template <bool HI>
__device__ __forceinline__ f16x2 e4m3x2_to_f16x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// Four codes of a 32-bit word -> four fp16 (byte b -> element b).
__device__ __forceinline__ f16x4 e4m3x4_to_f16x4(uint32_t w) {
    const f16x2 lo = e4m3x2_to_f16x2<false>(w), hi = e4m3x2_to_f16x2<true>(w);
    return f16x4{lo.x, lo.y, hi.x, hi.y};
}

// The E4M3 code of x: nearest value, ties to even, finite values beyond 448
// saturated to +-448, NaN -> 0x7F.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
    if (x != x) return 0x7Fu;
    const float c = fminf(fmaxf(x, -kE4M3Max), kE4M3Max);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
}

// Bytes of w at token positions >= n (within the 4 tokens t0..t0+3 the word
// holds) cleared: masked slots of a partly filled block may hold any bits.
__device__ __forceinline__ uint32_t keep_tokens(uint32_t w, int t0, int n) {
    const int k = n - t0;                   // tokens of this word to keep
    if (k >= 4) return w;
    if (k <= 0) return 0u;
    return w & ((1u << (8 * k)) - 1u);
}

}  // namespace pa
