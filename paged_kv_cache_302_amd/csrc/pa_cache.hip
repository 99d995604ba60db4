// The two directions of the paged indirection (page "读 vLLM 的
// PagedAttention kernel", §3.2: the write path scatters tokens to physical
// slots through slot_mapping, the read path gathers them back through the
// block table).
//
// reshape_and_cache: token i's K and V rows for every KV head go to flat
// slot slot_mapping[i] (block s / 16, offset s % 16), K into the x-packed
// k_cache[b, h, d / x, o, d % x], V transposed into v_cache[b, h, d, o].  A
// pure copy, so bit-exact.  Into an fp8 pool each element becomes its E4M3
// code of x / scale (nearest, ties to even, saturated at +-448, NaN -> 0x7F),
// the division in fp32.
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

// reshape_and_cache: one workgroup per (16 consecutive tokens, KV head).  The
// 16 key and value rows are read whole (coalesced 16-byte loads) into LDS.  K
// chunks then go out with 16 consecutive lanes on the 16 tokens of one chunk
// (in a block filled in order: 256 contiguous bytes), and V with 16
// consecutive lanes on the 16 tokens of one dimension row (32 contiguous
// bytes, 16 for fp8), so the transposed V row of a block is written by one
// store instruction instead of 16 scattered ones.  Every token still goes to
// its own slot, so any slot mapping is handled.
template <int D, bool FP8>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const f16* __restrict__ key, const f16* __restrict__ value, void* __restrict__ k_cache,
    void* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping, int num_tokens,
    int num_kv_heads, long long num_slots, long long key_stride, long long value_stride,
    float k_scale, float v_scale) {
    constexpr int R = D + 8;                       // padded LDS row (elements)
    __shared__ __align__(16) f16 sk[kBlock * R];
    __shared__ __align__(16) f16 sv[kBlock * R];
    __shared__ long long sslot[kBlock];
    const int t = threadIdx.x;
    const long long i0 = (long long)blockIdx.x * kBlock;
    const int h = blockIdx.y;
    const int nt = (int)min((long long)kBlock, (long long)num_tokens - i0);
    if (t < kBlock) {
        long long sl = -1;
        if (t < nt) {
            sl = slot_mapping[i0 + t];
            if (sl >= num_slots) sl = -1;
        }
        sslot[t] = sl;
    }
    constexpr int CH = D / kX;                     // 16-byte chunks per row
    for (int e = t; e < kBlock * CH; e += 256) {
        const int o = e / CH, c = e - o * CH;
        if (o < nt) {
            const long long i = i0 + o;
            *reinterpret_cast<f16x8*>(sk + o * R + c * kX) =
                *reinterpret_cast<const f16x8*>(key + i * key_stride + h * D + c * kX);
            *reinterpret_cast<f16x8*>(sv + o * R + c * kX) =
                *reinterpret_cast<const f16x8*>(value + i * value_stride + h * D + c * kX);
        }
    }
    __syncthreads();
    const size_t tile_elems = (size_t)D * kBlock;
    if constexpr (!FP8) {
        f16* kc = static_cast<f16*>(k_cache);
        f16* vc = static_cast<f16*>(v_cache);
        for (int e = t; e < kBlock * CH; e += 256) {
            const int c = e / kBlock, o = e - c * kBlock;
            const long long sl = sslot[o];
            if (sl < 0) continue;
            const size_t tile = ((size_t)(sl / kBlock) * num_kv_heads + h) * tile_elems;
            *reinterpret_cast<f16x8*>(kc + tile + ((size_t)c * kBlock + (int)(sl % kBlock)) * kX) =
                *reinterpret_cast<const f16x8*>(sk + o * R + c * kX);
        }
        for (int e = t; e < kBlock * D; e += 256) {
            const int d = e / kBlock, o = e - d * kBlock;
            const long long sl = sslot[o];
            if (sl < 0) continue;
            const size_t tile = ((size_t)(sl / kBlock) * num_kv_heads + h) * tile_elems;
            vc[tile + (size_t)d * kBlock + (int)(sl % kBlock)] = sv[o * R + d];
        }
    } else {
        uint8_t* kc = static_cast<uint8_t*>(k_cache);
        uint8_t* vc = static_cast<uint8_t*>(v_cache);
        constexpr int CH8 = D / kX8;               // 16-element x chunks of the fp8 pool
        for (int e = t; e < kBlock * CH8; e += 256) {
            const int c = e / kBlock, o = e - c * kBlock;
            const long long sl = sslot[o];
            if (sl < 0) continue;
            u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 0; j < kX8; ++j)
                w[j >> 2] |= f32_to_e4m3((float)sk[o * R + c * kX8 + j] / k_scale) << (8 * (j & 3));
            const size_t tile = ((size_t)(sl / kBlock) * num_kv_heads + h) * tile_elems;
            *reinterpret_cast<u32x4*>(kc + tile + ((size_t)c * kBlock + (int)(sl % kBlock)) * kX8) = w;
        }
        for (int e = t; e < kBlock * D; e += 256) {
            const int d = e / kBlock, o = e - d * kBlock;
            const long long sl = sslot[o];
            if (sl < 0) continue;
            const size_t tile = ((size_t)(sl / kBlock) * num_kv_heads + h) * tile_elems;
            vc[tile + (size_t)d * kBlock + (int)(sl % kBlock)] =
                (uint8_t)f32_to_e4m3((float)sv[o * R + d] / v_scale);
        }
    }
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

extern "C" int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int num_pairs,
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

extern "C" int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
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
    if (num_kv_heads > 65535) return PA_ERR_INVALID_ARG;   // grid.y
    const long long slots = (long long)num_blocks * kBlock;
    hipStream_t st = as_stream(stream);
    auto k = static_cast<const f16*>(key);
    auto v = static_cast<const f16*>(value);
    const dim3 grid((unsigned)((num_tokens + kBlock - 1) / kBlock), (unsigned)num_kv_heads);
    const bool f8 = kv_cache_dtype == PA_KV_FP8_E4M3;
#define PA_CW(DD, F8)                                                                              \
    hipLaunchKernelGGL((reshape_and_cache_kernel<DD, F8>), grid, dim3(256), 0, st, k, v, k_cache,  \
                       v_cache, slot_mapping, num_tokens, num_kv_heads, slots,                     \
                       (long long)key_stride, (long long)value_stride, k_scale, v_scale)
    if (head_size == 128) {
        if (f8) PA_CW(128, true);
        else PA_CW(128, false);
    } else {
        if (f8) PA_CW(64, true);
        else PA_CW(64, false);
    }
#undef PA_CW
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
