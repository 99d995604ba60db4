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
// partition count (one wave when a sequence has at most 16 partitions, up to
// 16 waves for 256 and more); as soon as the length is known every thread
// requests its m_p / l_p and every wave requests its (up to 16) o_p rows --
// the rows do not depend on the weights -- then the max and the weight sum
// are reduced through LDS, each wave folds its rows with their weights, and
// the wave sums are added in LDS.  Longer sequences loop over further
// chunks of rows.
#include <math.h>

#include "pa_device.h"
#include "pa_host.h"

namespace pa {

constexpr int kReduceRows = 16;   // o_p rows per wave per chunk

template <int D, int NWR>
__global__ __launch_bounds__(64 * NWR) void pa_reduce_kernel(
    float* __restrict__ out, const float* __restrict__ tmp_out, const float* __restrict__ exp_sums,
    const float* __restrict__ max_logits, const int32_t* __restrict__ seq_lens, int num_heads,
    int max_num_partitions, int partition_size) {
    constexpr int VEC = D / 64;
    constexpr int kReduceWaves = NWR;
    constexpr int kReduceThreads = 64 * NWR;
    constexpr int kReduceChunk = NWR * kReduceRows;   // partitions per chunk
    typedef float vec_t __attribute__((ext_vector_type(VEC)));
    __shared__ float s_red[kReduceWaves];
    __shared__ vec_t s_acc[kReduceWaves][64];

    const int sh = blockIdx.x;  // s * num_heads + h
    const int s = sh / num_heads;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int L = seq_lens[s];
    float* orow = out + (size_t)sh * D;
    const int n = L > 0 ? (L - 1) / partition_size + 1 : 0;
    if (n == 0 || n > max_num_partitions) {
        for (int d = tid; d < D; d += kReduceThreads) orow[d] = (n == 0) ? 0.f : NAN;
        return;
    }
    // partials are [S][P][H](x D): consecutive partitions of one (s, h) are
    // num_heads entries apart
    const int h = sh - s * num_heads;
    const size_t base = (size_t)s * max_num_partitions * num_heads + h;
    const size_t pstride = num_heads;
    const float* mp = max_logits + base;
    const float* lp = exp_sums + base;
    const float* o = tmp_out + base * D + lane * VEC;
    auto m = [&](int q) { return mp[(size_t)q * pstride]; };
    auto l = [&](int q) { return lp[(size_t)q * pstride]; };

    // requests: this thread's m_p / l_p (first 1024 partitions) and this
    // wave's first chunk of rows, all before any reduction
    const float m0 = tid < n ? m(tid) : -INFINITY;
    const float l0 = tid < n ? l(tid) : 0.f;
    vec_t rows[kReduceRows];
#pragma unroll
    for (int j = 0; j < kReduceRows; ++j) {
        const int p = w + kReduceWaves * j;
        rows[j] = p < n ? __builtin_nontemporal_load(reinterpret_cast<const vec_t*>(o + (size_t)p * pstride * D))
                        : vec_t{};
    }

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

    // W = sum_p l_p exp(m_p - M)
    float ws = tid < n ? l0 * exp2_fast((m0 - M) * kLog2e) : 0.f;
    for (int p = tid + kReduceThreads; p < n; p += kReduceThreads)
        ws += l(p) * exp2_fast((m(p) - M) * kLog2e);
    ws = wave_sum(ws);
    if (lane == 0) s_red[w] = ws;
    __syncthreads();
    float W = 0.f;
#pragma unroll
    for (int v = 0; v < kReduceWaves; ++v) W += s_red[v];

    // out = sum_p (w_p / W) o_p
    vec_t acc = {};
#pragma unroll
    for (int j = 0; j < kReduceRows; ++j) {
        const int p = w + kReduceWaves * j;
        if (p < n) acc += ((l(p) * exp2_fast((m(p) - M) * kLog2e)) / W) * rows[j];
    }
    for (int chunk = kReduceChunk; chunk < n; chunk += kReduceChunk) {
#pragma unroll
        for (int j = 0; j < kReduceRows; ++j) {
            const int p = chunk + w + kReduceWaves * j;
            rows[j] = p < n ? __builtin_nontemporal_load(reinterpret_cast<const vec_t*>(o + (size_t)p * pstride * D))
                            : vec_t{};
        }
#pragma unroll
        for (int j = 0; j < kReduceRows; ++j) {
            const int p = chunk + w + kReduceWaves * j;
            if (p < n) acc += ((l(p) * exp2_fast((m(p) - M) * kLog2e)) / W) * rows[j];
        }
    }
    s_acc[w][lane] = acc;
    __syncthreads();
    if (w == 0) {
        vec_t t = s_acc[0][lane];
#pragma unroll
        for (int v = 1; v < kReduceWaves; ++v) t += s_acc[v][lane];
        *reinterpret_cast<vec_t*>(orow + lane * VEC) = t;
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
    // waves per workgroup: one per 16 partitions, between 1 and 16
    int nwr = 1;
    while (nwr < 16 && nwr * kReduceRows < max_num_partitions) nwr *= 2;
#define PA_REDUCE_LAUNCH(DD, NN)                                                                 \
    hipLaunchKernelGGL((pa_reduce_kernel<DD, NN>), dim3((unsigned)grid), dim3(64 * NN), 0, st, out, \
                       tmp_out, exp_sums, max_logits, seq_lens, num_heads, max_num_partitions,    \
                       partition_size)
#define PA_REDUCE_BY_WAVES(DD)                  \
    switch (nwr) {                              \
        case 1: PA_REDUCE_LAUNCH(DD, 1); break;   \
        case 2: PA_REDUCE_LAUNCH(DD, 2); break;   \
        case 4: PA_REDUCE_LAUNCH(DD, 4); break;   \
        case 8: PA_REDUCE_LAUNCH(DD, 8); break;   \
        default: PA_REDUCE_LAUNCH(DD, 16); break; \
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
