// pa_reduce: second pass of the partitioned decode (page "读 vLLM 的
// PagedAttention kernel", §3.3: partitions are computed in parallel and merged
// afterwards).  The merge is the exact log-sum-exp one:
//     M = max_p m_p,  w_p = l_p exp(m_p - M),  out = sum_p (w_p / sum_q w_q) o_p
// over p < ceil(L / PS).  Each weight is divided by the total before the
// sum, so a single partition comes back bit-exactly (w / w = 1).
//
// One workgroup of 4 wavefronts per (sequence, query head).  The partials'
// m_p and l_p are read by all threads (two short passes: the max, then the
// weight sum); the o_p rows are split across the waves (wave w takes
// p = w, w+4, ...), each lane owning D/64 consecutive head dims, with four
// rows in flight per wave; the four wave sums are added in LDS.
#include <math.h>

#include "pa_device.h"
#include "pa_host.h"

namespace pa {

constexpr int kReduceWaves = 4;

template <int D>
__global__ __launch_bounds__(64 * kReduceWaves) void pa_reduce_kernel(
    float* __restrict__ out, const float* __restrict__ tmp_out, const float* __restrict__ exp_sums,
    const float* __restrict__ max_logits, const int32_t* __restrict__ seq_lens, int num_heads,
    int max_num_partitions, int partition_size) {
    constexpr int VEC = D / 64;
    typedef float vec_t __attribute__((ext_vector_type(VEC)));
    __shared__ float s_red[kReduceWaves];
    __shared__ vec_t s_acc[kReduceWaves][64];

    const int sh = blockIdx.x;  // s * num_heads + h
    const int s = sh / num_heads;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int L = seq_lens[s];
    float* orow = out + (size_t)sh * D;
    const int n = L > 0 ? (L - 1) / partition_size + 1 : 0;
    if (n == 0 || n > max_num_partitions) {
        for (int d = tid; d < D; d += 64 * kReduceWaves) orow[d] = (n == 0) ? 0.f : NAN;
        return;
    }
    const float* m = max_logits + (size_t)sh * max_num_partitions;
    const float* l = exp_sums + (size_t)sh * max_num_partitions;
    const float* o = tmp_out + (size_t)sh * max_num_partitions * D;

    // M = max_p m_p
    float mx = -INFINITY;
    for (int p = tid; p < n; p += 64 * kReduceWaves) mx = fmaxf(mx, m[p]);
    mx = wave_max(mx);
    if (lane == 0) s_red[w] = mx;
    __syncthreads();
    float M = s_red[0];
#pragma unroll
    for (int v = 1; v < kReduceWaves; ++v) M = fmaxf(M, s_red[v]);
    __syncthreads();

    // W = sum_p l_p exp(m_p - M)
    float ws = 0.f;
    for (int p = tid; p < n; p += 64 * kReduceWaves) ws += l[p] * exp2_fast((m[p] - M) * kLog2e);
    ws = wave_sum(ws);
    if (lane == 0) s_red[w] = ws;
    __syncthreads();
    float W = 0.f;
#pragma unroll
    for (int v = 0; v < kReduceWaves; ++v) W += s_red[v];

    // out = sum_p (w_p / W) o_p
    vec_t acc = {};
    int p = w;
    for (; p + 3 * kReduceWaves < n; p += 4 * kReduceWaves) {
        vec_t r[4];
        float c[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int pp = p + u * kReduceWaves;
            r[u] = *reinterpret_cast<const vec_t*>(o + (size_t)pp * D + lane * VEC);
            c[u] = (l[pp] * exp2_fast((m[pp] - M) * kLog2e)) / W;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc += c[u] * r[u];
    }
    for (; p < n; p += kReduceWaves) {
        const vec_t r = *reinterpret_cast<const vec_t*>(o + (size_t)p * D + lane * VEC);
        const float c = (l[p] * exp2_fast((m[p] - M) * kLog2e)) / W;
        acc += c * r;
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
    if (head_size == 128)
        hipLaunchKernelGGL(pa_reduce_kernel<128>, dim3((unsigned)grid), dim3(64 * kReduceWaves), 0,
                           st, out, tmp_out, exp_sums, max_logits, seq_lens, num_heads,
                           max_num_partitions, partition_size);
    else
        hipLaunchKernelGGL(pa_reduce_kernel<64>, dim3((unsigned)grid), dim3(64 * kReduceWaves), 0,
                           st, out, tmp_out, exp_sums, max_logits, seq_lens, num_heads,
                           max_num_partitions, partition_size);
    return launch_status();
}
