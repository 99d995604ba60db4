// pa_decode_v2_noalloc: partitioned decode (pa_decode_v2) and its merge
// (pa_reduce) in one call whose partials live in a fixed device array of this
// library instead of caller-provided scratch, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops).
//
// The array `scratch` is a file-scope __device__ array: every GPU that runs
// this code holds one copy of PA_NOALLOC_SCRATCH_BYTES until the process
// ends.  Its host-side name is only a stand-in, so the device address of each
// GPU's copy is looked up once per device (hipGetSymbolAddress, with that
// device current) on the first call there and kept; kernels are only ever
// given that address.  Calls on one GPU share its copy: calls that overlap
// on one GPU (two streams, two threads) race.  Nothing in it needs clearing:
// the decode writes every partial the merge reads.
#include <mutex>

#include "pa.h"
#include "pa_host.h"

static_assert(PA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size must keep 256-byte alignment");

static __device__ __align__(256) char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of each GPU's copy (null until looked up)

// The device address of `dev`'s copy of the array, looked up on first use
// with `dev` current; null if the lookup fails.
void* scratch_of(int dev) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev]) return g_scratch[dev];
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || ptr == nullptr) {
        (void)hipGetLastError();
        return nullptr;
    }
    g_scratch[dev] = ptr;
    return ptr;
}

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace

extern "C" int pa_decode_v2_noalloc(float* out, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* block_tables,
                                    const int32_t* seq_lens, int num_seqs, int num_heads,
                                    int num_kv_heads, int head_size, int block_size,
                                    int max_blocks_per_seq, int num_blocks, int max_num_partitions,
                                    int partition_size, float scale, int kv_cache_dtype,
                                    float k_scale, float v_scale, void* stream) {
    if (!out || num_seqs < 0 || num_heads <= 0 || max_num_partitions <= 0)
        return PA_ERR_INVALID_ARG;
    if (head_size != 64 && head_size != 128) return PA_ERR_UNSUPPORTED;
    // partials [S][P][H][D] then exp_sums and max_logits [S][P][H], each
    // starting on a 256-byte boundary
    const size_t rows = (size_t)num_seqs * max_num_partitions * num_heads;
    const size_t o_bytes = round256(rows * head_size * sizeof(float));
    const size_t s_bytes = round256(rows * sizeof(float));
    if (o_bytes + 2 * s_bytes > kScratchBytes) return PA_ERR_SCRATCH_TOO_SMALL;
    if (num_seqs == 0) return PA_OK;
    hipDevice_t dev = 0;
    if (hipStreamGetDevice(pa::as_stream(stream), &dev) != hipSuccess) {
        (void)hipGetLastError();
        return PA_ERR_INVALID_ARG;
    }
    if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
    char* base = static_cast<char*>(scratch_of(dev));
    if (!base) return PA_ERR_LAUNCH;
    float* tmp_out = reinterpret_cast<float*>(base);
    float* exp_sums = reinterpret_cast<float*>(base + o_bytes);
    float* max_logits = reinterpret_cast<float*>(base + o_bytes + s_bytes);
    int rc = pa_decode_v2(tmp_out, exp_sums, max_logits, q, k_cache, v_cache, block_tables,
                          seq_lens, num_seqs, num_heads, num_kv_heads, head_size, block_size,
                          max_blocks_per_seq, num_blocks, max_num_partitions, partition_size,
                          scale, kv_cache_dtype, k_scale, v_scale, stream);
    if (rc != PA_OK) return rc;
    return pa_reduce(out, tmp_out, exp_sums, max_logits, seq_lens, num_seqs, num_heads, head_size,
                     max_num_partitions, partition_size, stream);
}
