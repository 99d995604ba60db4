// The two directions of the paged indirection (page "读 vLLM 的
// PagedAttention kernel", §3.2: the write path scatters tokens to physical
// slots through slot_mapping, the read path gathers them back through the
// block table).
//
// reshape_and_cache: one thread per (token, KV head, 8-element chunk of the
// head dims).  The chunk is one 16-byte load of key; in the x-packed K pool it
// is one 16-byte store (k_cache[b, h, c, o, 0..7]).  V is stored transposed
// (v_cache[b, h, d, o]): the same 16-byte load of value becomes eight 2-byte
// stores 32 bytes apart.  A pure copy, so bit-exact.  Into an fp8 pool each
// element becomes its E4M3 code of x / scale (nearest, ties to even,
// saturated at +-448, NaN -> 0x7F), the division in fp32: the K chunk is an
// 8-byte store (half of a 16-element x chunk), V eight 1-byte stores.
//
// pa_gather_kv: the inverse, for testing the read-side indirection alone.
// One thread per (sequence, logical block, token slot, KV head, chunk).
//
// copy_blocks: the device half of copy-on-write (page "vLLM 的
// PagedAttention：KV cache 为什么要分页", §4.2): a whole physical block --
// every KV head, every slot, K and V -- duplicated into a fresh block.  A
// block of either pool is one contiguous run of num_kv_heads*head_size*16
// fp16, so the copy is 16-byte vectors, workgroup (pair, 4 KiB piece).
#include "pa_device.h"
#include "pa_host.h"
#include "pa_blocks.h"

namespace pa {

template <int D>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const f16* __restrict__ key, const f16* __restrict__ value, f16* __restrict__ k_cache,
    f16* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping, int num_tokens,
    int num_kv_heads, long long num_slots, long long key_stride, long long value_stride) {
    constexpr int C = D / kX;
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long total = (long long)num_tokens * num_kv_heads * C;
    if (gid >= total) return;
    const int c = (int)(gid % C);
    const int h = (int)((gid / C) % num_kv_heads);
    const int i = (int)(gid / ((long long)C * num_kv_heads));
    const long long slot = slot_mapping[i];
    if (slot < 0 || slot >= num_slots) return;
    const long long b = slot / kBlock;
    const int o = (int)(slot % kBlock);
    const f16x8 kv = *reinterpret_cast<const f16x8*>(key + i * key_stride + h * D + c * kX);
    const f16x8 vv = *reinterpret_cast<const f16x8*>(value + i * value_stride + h * D + c * kX);
    const size_t tile = ((size_t)b * num_kv_heads + h) * (size_t)(D * kBlock);
    *reinterpret_cast<f16x8*>(k_cache + tile + ((size_t)c * kBlock + o) * kX) = kv;
    f16* vdst = v_cache + tile + (size_t)(c * kX) * kBlock + o;
#pragma unroll
    for (int j = 0; j < kX; ++j) vdst[j * kBlock] = vv[j];
}

template <int D>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const f16* __restrict__ key, const f16* __restrict__ value, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping, int num_tokens,
    int num_kv_heads, long long num_slots, long long key_stride, long long value_stride,
    float k_scale, float v_scale) {
    constexpr int C = D / kX;          // 8-element chunks of a head
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long total = (long long)num_tokens * num_kv_heads * C;
    if (gid >= total) return;
    const int c = (int)(gid % C);
    const int h = (int)((gid / C) % num_kv_heads);
    const int i = (int)(gid / ((long long)C * num_kv_heads));
    const long long slot = slot_mapping[i];
    if (slot < 0 || slot >= num_slots) return;
    const long long b = slot / kBlock;
    const int o = (int)(slot % kBlock);
    const f16x8 kv = *reinterpret_cast<const f16x8*>(key + i * key_stride + h * D + c * kX);
    const f16x8 vv = *reinterpret_cast<const f16x8*>(value + i * value_stride + h * D + c * kX);
    u32x2 kc = {0u, 0u};
#pragma unroll
    for (int j = 0; j < kX; ++j) kc[j >> 2] |= f32_to_e4m3((float)kv[j] / k_scale) << (8 * (j & 3));
    const size_t tile = ((size_t)b * num_kv_heads + h) * (size_t)(D * kBlock);   // bytes
    // d = 8c + j lives in x-chunk d / 16 at element d % 16 = 8(c % 2) + j
    *reinterpret_cast<u32x2*>(k_cache + tile + ((size_t)(c >> 1) * kBlock + o) * kX8 + 8 * (c & 1)) = kc;
    uint8_t* vdst = v_cache + tile + (size_t)(c * kX) * kBlock + o;
#pragma unroll
    for (int j = 0; j < kX; ++j) vdst[j * kBlock] = (uint8_t)f32_to_e4m3((float)vv[j] / v_scale);
}

template <int D, class T>
__global__ __launch_bounds__(256) void gather_kv_kernel(
    T* __restrict__ k_out, T* __restrict__ v_out, const T* __restrict__ k_cache,
    const T* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ seq_lens, const int64_t* __restrict__ cu_seq_lens,
    int num_kv_heads, int max_blocks_per_seq, int num_blocks, int wgs_per_block, T nan) {
    constexpr int X = 16 / sizeof(T);  // elements per 16-byte K chunk
    constexpr int C = D / X;
    typedef T chunk_t __attribute__((ext_vector_type(X)));
    // workgroup -> (sequence, logical block, part of the block's items)
    const int sb = blockIdx.x / wgs_per_block;
    const int part = blockIdx.x - sb * wgs_per_block;
    const int s = sb / max_blocks_per_seq;
    const int lb = sb - s * max_blocks_per_seq;
    const int item = part * blockDim.x + threadIdx.x;  // (slot o, head h, chunk c)
    if (item >= kBlock * num_kv_heads * C) return;
    const int c = item % C;
    const int h = (item / C) % num_kv_heads;
    const int o = item / (C * num_kv_heads);
    const int L = seq_lens[s];
    const int t = lb * kBlock + o;
    if (t >= L || lb >= max_blocks_per_seq) return;
    const int phys = block_tables[(size_t)s * max_blocks_per_seq + lb];
    const size_t row = ((size_t)cu_seq_lens[s] + t) * num_kv_heads + h;
    chunk_t kv, vv;
    if (phys < 0 || phys >= num_blocks) {
        for (int j = 0; j < X; ++j) kv[j] = vv[j] = nan;
    } else {
        const size_t tile = ((size_t)phys * num_kv_heads + h) * (size_t)(D * kBlock);
        kv = *reinterpret_cast<const chunk_t*>(k_cache + tile + ((size_t)c * kBlock + o) * X);
        const T* vsrc = v_cache + tile + (size_t)(c * X) * kBlock + o;
#pragma unroll
        for (int j = 0; j < X; ++j) vv[j] = vsrc[j * kBlock];
    }
    *reinterpret_cast<chunk_t*>(k_out + row * D + c * X) = kv;
    *reinterpret_cast<chunk_t*>(v_out + row * D + c * X) = vv;
}

__global__ __launch_bounds__(256) void copy_blocks_kernel(
    f16* __restrict__ k_cache, f16* __restrict__ v_cache, const int32_t* __restrict__ pairs,
    int num_blocks, long long chunks_per_block) {
    const int src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
    const long long c = (long long)blockIdx.y * blockDim.x + threadIdx.x;   // 16-byte chunk
    if (c >= chunks_per_block) return;
    const size_t so = (size_t)src * chunks_per_block + c, d = (size_t)dst * chunks_per_block + c;
    f16x8* kc = reinterpret_cast<f16x8*>(k_cache);
    f16x8* vc = reinterpret_cast<f16x8*>(v_cache);
    const f16x8 kv = kc[so], vv = vc[so];
    kc[d] = kv;
    vc[d] = vv;
}

}  // namespace pa

using namespace pa;

extern "C" int copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int num_pairs,
                           int num_kv_heads, int head_size, int block_size, int num_blocks,
                           int kv_cache_dtype, void* stream) {
    int rc = check_head_block(head_size, block_size);
    if (rc != PA_OK) return rc;
    rc = check_kv_dtype(kv_cache_dtype, 1.f, 1.f);
    if (rc != PA_OK) return rc;
    if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_INVALID_ARG;
    if (!k_cache || !v_cache) return PA_ERR_INVALID_ARG;
    if (num_pairs == 0) return PA_OK;   // block_pairs may be NULL then
    if (!block_pairs) return PA_ERR_INVALID_ARG;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned4(block_pairs)) return PA_ERR_MISALIGNED;
    const long long chunks = (long long)num_kv_heads * head_size * kBlock * kv_elem_bytes(kv_cache_dtype) / 16;
    const long long parts = (chunks + 255) / 256;
    if (parts > 65535) return PA_ERR_INVALID_ARG;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)num_pairs, (unsigned)parts), dim3(256), 0,
                       as_stream(stream), static_cast<f16*>(k_cache), static_cast<f16*>(v_cache),
                       block_pairs, num_blocks, chunks);
    return launch_status();
}

extern "C" int reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                 const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                 int head_size, int block_size, int num_blocks,
                                 int64_t key_stride, int64_t value_stride, int kv_cache_dtype,
                                 float k_scale, float v_scale, void* stream) {
    int rc = check_head_block(head_size, block_size);
    if (rc != PA_OK) return rc;
    rc = check_kv_dtype(kv_cache_dtype, k_scale, v_scale);
    if (rc != PA_OK) return rc;
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_INVALID_ARG;
    const int64_t row = (int64_t)num_kv_heads * head_size;
    if (key_stride < row || value_stride < row) return PA_ERR_INVALID_ARG;
    if (!k_cache || !v_cache) return PA_ERR_INVALID_ARG;
    if (num_tokens == 0) return PA_OK;   // key, value, slot_mapping may be NULL then
    if (!key || !value || !slot_mapping) return PA_ERR_INVALID_ARG;
    if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned8(slot_mapping) || key_stride % 8 != 0 || value_stride % 8 != 0)
        return PA_ERR_MISALIGNED;
    const long long items = (long long)num_tokens * num_kv_heads * (head_size / kX);
    const long long grid = (items + 255) / 256;
    if (grid > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
    const long long slots = (long long)num_blocks * kBlock;
    hipStream_t st = as_stream(stream);
    auto k = static_cast<const f16*>(key);
    auto v = static_cast<const f16*>(value);
    if (kv_cache_dtype == PA_KV_FP8_E4M3) {
        auto kc8 = static_cast<uint8_t*>(k_cache);
        auto vc8 = static_cast<uint8_t*>(v_cache);
        if (head_size == 128)
            hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<128>, dim3((unsigned)grid), dim3(256), 0,
                               st, k, v, kc8, vc8, slot_mapping, num_tokens, num_kv_heads, slots,
                               (long long)key_stride, (long long)value_stride, k_scale, v_scale);
        else
            hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<64>, dim3((unsigned)grid), dim3(256), 0,
                               st, k, v, kc8, vc8, slot_mapping, num_tokens, num_kv_heads, slots,
                               (long long)key_stride, (long long)value_stride, k_scale, v_scale);
        return launch_status();
    }
    auto kc = static_cast<f16*>(k_cache);
    auto vc = static_cast<f16*>(v_cache);
    if (head_size == 128)
        hipLaunchKernelGGL(reshape_and_cache_kernel<128>, dim3((unsigned)grid), dim3(256), 0, st, k,
                           v, kc, vc, slot_mapping, num_tokens, num_kv_heads, slots,
                           (long long)key_stride, (long long)value_stride);
    else
        hipLaunchKernelGGL(reshape_and_cache_kernel<64>, dim3((unsigned)grid), dim3(256), 0, st, k,
                           v, kc, vc, slot_mapping, num_tokens, num_kv_heads, slots,
                           (long long)key_stride, (long long)value_stride);
    return launch_status();
}

extern "C" int pa_gather_kv(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            const int64_t* cu_seq_lens, int num_seqs, int num_kv_heads,
                            int head_size, int block_size, int max_blocks_per_seq, int num_blocks,
                            int kv_cache_dtype, void* stream) {
    int rc = check_head_block(head_size, block_size);
    if (rc != PA_OK) return rc;
    rc = check_kv_dtype(kv_cache_dtype, 1.f, 1.f);
    if (rc != PA_OK) return rc;
    if (num_seqs < 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
        return PA_ERR_INVALID_ARG;
    if (!k_out || !v_out || !k_cache || !v_cache || !block_tables || !seq_lens || !cu_seq_lens)
        return PA_ERR_INVALID_ARG;
    if (!aligned16(k_out) || !aligned16(v_out) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned4(block_tables) || !aligned4(seq_lens) || !aligned8(cu_seq_lens))
        return PA_ERR_MISALIGNED;
    if (num_seqs == 0) return PA_OK;
    const bool fp8 = kv_cache_dtype == PA_KV_FP8_E4M3;
    const int items = kBlock * num_kv_heads * (head_size / (fp8 ? kX8 : kX));
    const int wgs = (items + 255) / 256;
    const long long grid = (long long)num_seqs * max_blocks_per_seq * wgs;
    if (grid > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
    hipStream_t st = as_stream(stream);
#define PA_GATHER(DD, T, NANV)                                                                     \
    hipLaunchKernelGGL((gather_kv_kernel<DD, T>), dim3((unsigned)grid), dim3(256), 0, st,          \
                       static_cast<T*>(k_out), static_cast<T*>(v_out),                            \
                       static_cast<const T*>(k_cache), static_cast<const T*>(v_cache),            \
                       block_tables, seq_lens, cu_seq_lens, num_kv_heads, max_blocks_per_seq,     \
                       num_blocks, wgs, NANV)
    const f16 nan16 = __builtin_bit_cast(f16, (unsigned short)0x7E00);
    if (fp8) {
        if (head_size == 128) PA_GATHER(128, uint8_t, (uint8_t)0x7F);
        else PA_GATHER(64, uint8_t, (uint8_t)0x7F);
    } else {
        if (head_size == 128) PA_GATHER(128, f16, nan16);
        else PA_GATHER(64, f16, nan16);
    }
#undef PA_GATHER
    return launch_status();
}
