// pa_reduce: second pass of the partitioned decode (page "读 vLLM 的
// PagedAttention kernel", §3.3: partitions are computed in parallel and merged
// afterwards).  The merge is the exact log-sum-exp one:
//     M = max_p m_p,  w_p = l_p exp(m_p - M),  out = sum_p (w_p / sum_q w_q) o_p
// over p < ceil(L / PS).  Each weight is divided by the total before the
// sum, so a single partition comes back bit-exactly (w / w = 1).
//
// The kernel is latency-bound (tens of MB spread over a few hundred rows of
// partials), so it is built to cost about one memory round trip: one
// workgroup of NWR wavefronts per (sequence, query head), NWR sized to the
// partition count (one wave when a sequence has at most 16 partitions, then
// with as many row slots as there can be partitions; up to 16 waves for 256
// and more); as soon as the length is known every thread
// requests its m_p / l_p (with the length, before it is known) and every
// wave its (up to 16) o_p rows -- the rows do not depend on the weights --
// then the max and the weight sum are reduced through LDS, the weights stay
// in LDS, each wave folds its rows with them, and the wave sums are added in
// LDS.  Longer sequences loop over further chunks of rows.
#include <math.h>

#include "pa_device.h"
#include "pa_host.h"

namespace pa {

__device__ __forceinline__ float* orow_of(float* out, int sh, int D) { return out + (size_t)sh * D; }

// ROWS: o_p rows per wave per chunk (16, fewer when a one-wave workgroup
// covers all max_num_partitions with fewer)
template <int D, int NWR, int ROWS>
__global__ __launch_bounds__(64 * NWR) void pa_reduce_kernel(
    float* __restrict__ out, const float* __restrict__ tmp_out, const float* __restrict__ exp_sums,
    const float* __restrict__ max_logits, const int32_t* __restrict__ seq_lens, int num_heads,
    int max_num_partitions, int partition_size) {
    constexpr int VEC = D / 64;
    constexpr int kReduceWaves = NWR;
    constexpr int kReduceThreads = 64 * NWR;
    constexpr int kReduceChunk = NWR * ROWS;   // partitions per chunk
    typedef float vec_t __attribute__((ext_vector_type(VEC)));
    __shared__ float s_red[kReduceWaves];
    __shared__ vec_t s_acc[kReduceWaves][64];

    __shared__ float s_w[kReduceThreads];   // weight l_p e^{m_p - M} of partition p = tid

    const int sh = blockIdx.x;  // s * num_heads + h
    const int s = sh / num_heads;
    const int h = sh - s * num_heads;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // partials are [S][P][H](x D): consecutive partitions of one (s, h) are
    // num_heads entries apart
    const size_t base = (size_t)s * max_num_partitions * num_heads + h;
    const size_t pstride = num_heads;
    const float* mp = max_logits + base;
    const float* lp = exp_sums + base;
    const float* o = tmp_out + base * D + lane * VEC;
    auto m = [&](int q) { return mp[(size_t)q * pstride]; };
    auto l = [&](int q) { return lp[(size_t)q * pstride]; };

    // This thread's m_p / l_p are requested together with the length: every
    // p < max_num_partitions lies inside the scratch, and the values of
    // partitions past the sequence are dropped once the length is known.  No
    // branch on the length comes before these loads are used.
    const int L = seq_lens[s];
    const int pq = tid < max_num_partitions ? tid : max_num_partitions - 1;
    const float m_raw = m(pq);
    const float l_raw = l(pq);
    const int n_all = L > 0 ? (L - 1) / partition_size + 1 : 0;
    const bool bad = n_all > max_num_partitions;   // NaN rows; L <= 0: zeros
    const int n = bad ? 0 : n_all;

    // this wave's first chunk of o_p rows: they do not depend on the weights.
    // Every row is requested (past the last partition: the last one again,
    // left out of the fold), so no load sits under a branch, where the
    // compiler would wait for it before the next one.
    const int p_last = n > 0 ? n - 1 : 0;
    auto row = [&](int p) {
        return __builtin_nontemporal_load(
            reinterpret_cast<const vec_t*>(o + (size_t)min(p, p_last) * pstride * D));
    };
    vec_t rows[ROWS];
#pragma unroll
    for (int j = 0; j < ROWS; ++j) rows[j] = row(w + kReduceWaves * j);
    const float m0 = tid < n ? m_raw : -INFINITY;
    const float l0 = tid < n ? l_raw : 0.f;

    // M = max_p m_p
    float mx = m0;
    for (int p = tid + kReduceThreads; p < n; p += kReduceThreads) mx = fmaxf(mx, m(p));
    mx = wave_max(mx);
    if (lane == 0) s_red[w] = mx;
    __syncthreads();
    float M = s_red[0];
#pragma unroll
    for (int v = 1; v < kReduceWaves; ++v) M = fmaxf(M, s_red[v]);
    __syncthreads();

    // W = sum_p l_p exp(m_p - M); the weights of the first kReduceThreads
    // partitions stay in LDS for the fold
    const float w0 = tid < n ? l0 * exp2_fast((m0 - M) * kLog2e) : 0.f;
    s_w[tid] = w0;
    float ws = w0;
    for (int p = tid + kReduceThreads; p < n; p += kReduceThreads)
        ws += l(p) * exp2_fast((m(p) - M) * kLog2e);
    ws = wave_sum(ws);
    if (lane == 0) s_red[w] = ws;
    __syncthreads();
    float W = 0.f;
#pragma unroll
    for (int v = 0; v < kReduceWaves; ++v) W += s_red[v];
    auto weight = [&](int p) {
        return p < kReduceThreads ? s_w[p] : l(p) * exp2_fast((m(p) - M) * kLog2e);
    };

    // out = sum_p (w_p / W) o_p
    vec_t acc = {};
#pragma unroll
    for (int j = 0; j < ROWS; ++j) {
        const int p = w + kReduceWaves * j;
        if (p < n) acc += (weight(p) / W) * rows[j];
    }
    for (int chunk = kReduceChunk; chunk < n; chunk += kReduceChunk) {
#pragma unroll
        for (int j = 0; j < ROWS; ++j) rows[j] = row(chunk + w + kReduceWaves * j);
#pragma unroll
        for (int j = 0; j < ROWS; ++j) {
            const int p = chunk + w + kReduceWaves * j;
            if (p < n) acc += (weight(p) / W) * rows[j];
        }
    }
    s_acc[w][lane] = acc;
    __syncthreads();
    if (w == 0) {
        vec_t t = s_acc[0][lane];
#pragma unroll
        for (int v = 1; v < kReduceWaves; ++v) t += s_acc[v][lane];
        if (n == 0) {   // empty sequence: zeros; too many partitions: NaN
            const float f = bad ? NAN : 0.f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) t[e] = f;
        }
        *reinterpret_cast<vec_t*>(orow_of(out, sh, D) + lane * VEC) = t;
    }
}

}  // namespace pa

using namespace pa;

extern "C" int pa_reduce(float* out, const float* tmp_out, const float* exp_sums,
                         const float* max_logits, const int32_t* seq_lens, int num_seqs,
                         int num_heads, int head_size, int max_num_partitions, int partition_size,
                         void* stream) {
    if (head_size != 64 && head_size != 128) return PA_ERR_UNSUPPORTED;
    if (num_seqs < 0 || num_heads <= 0 || max_num_partitions <= 0 || partition_size <= 0)
        return PA_ERR_INVALID_ARG;
    if (!out || !tmp_out || !exp_sums || !max_logits || !seq_lens) return PA_ERR_INVALID_ARG;
    if (!aligned16(out) || !aligned16(tmp_out) || !aligned4(exp_sums) || !aligned4(max_logits) ||
        !aligned4(seq_lens))
        return PA_ERR_MISALIGNED;
    if (num_seqs == 0) return PA_OK;
    const long long grid = (long long)num_seqs * num_heads;
    if (grid > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
    hipStream_t st = as_stream(stream);
    // waves per workgroup: one per 16 partitions, between 1 and 16; a single
    // wave takes only as many rows per chunk as there can be partitions
    int nwr = 1;
    while (nwr < 16 && nwr * 16 < max_num_partitions) nwr *= 2;
    int rows = 16;
    if (nwr == 1)
        while (rows > 1 && rows / 2 >= max_num_partitions) rows /= 2;
#define PA_REDUCE_LAUNCH(DD, NN, RR)                                                                  \
    hipLaunchKernelGGL((pa_reduce_kernel<DD, NN, RR>), dim3((unsigned)grid), dim3(64 * NN), 0, st, out, \
                       tmp_out, exp_sums, max_logits, seq_lens, num_heads, max_num_partitions,        \
                       partition_size)
#define PA_REDUCE_BY_WAVES(DD)                                 \
    switch (nwr * 32 + rows) {                                 \
        case 32 + 1: PA_REDUCE_LAUNCH(DD, 1, 1); break;        \
        case 32 + 2: PA_REDUCE_LAUNCH(DD, 1, 2); break;        \
        case 32 + 4: PA_REDUCE_LAUNCH(DD, 1, 4); break;        \
        case 32 + 8: PA_REDUCE_LAUNCH(DD, 1, 8); break;        \
        case 32 + 16: PA_REDUCE_LAUNCH(DD, 1, 16); break;      \
        case 64 + 16: PA_REDUCE_LAUNCH(DD, 2, 16); break;      \
        case 128 + 16: PA_REDUCE_LAUNCH(DD, 4, 16); break;     \
        case 256 + 16: PA_REDUCE_LAUNCH(DD, 8, 16); break;     \
        default: PA_REDUCE_LAUNCH(DD, 16, 16); break;          \
    }
    if (head_size == 128) {
        PA_REDUCE_BY_WAVES(128)
    } else {
        PA_REDUCE_BY_WAVES(64)
    }
#undef PA_REDUCE_BY_WAVES
#undef PA_REDUCE_LAUNCH
    return launch_status();
}
