// Multi-token queries over the paged cache (prefill, chunked prefill,
// speculative verify): the phase on either side of decode (page "vLLM 的
// PagedAttention：KV cache 为什么要分页", §2: prefill writes the prompt's K/V,
// decode then reads them; page "KV Cache与PagedAttention内存管理", 自回归推理:
// softmax(QK^T/sqrt(d_k))V with a causal mask in prefill).
//
// Sequence s holds L_s cached tokens, the last n_s of which have queries
// (rows query_start_loc[s] .. +n_s of q and out).  Query j sits at position
// p = L_s - n_s + j and attends keys 0..p; its K/V, like every earlier
// token's, are already in the pools (written by reshape_and_cache).  n_s = 1
// is a decode step; n_s = L_s is a plain prefill.
//
// Work unit: one wavefront per (sequence, 16-row query tile, KV head, head
// chunk).  The 16 columns of the MFMA score tile S^T = K Q^T are (token,
// head) pairs of one KV group -- 16/G consecutive query tokens times the G
// heads, or 16 heads of one token when G >= 16 -- so every K/V tile read
// serves 16 query rows and the MFMA runs full (MHA included: 16 tokens of
// one head).  The unit walks blocks 0 .. p_last/16 in order with the decode
// kernels' table windows and paired tiles; each column's causal limit is a
// lane-local mask (the softmax state of a column lives in its own lanes),
// and block 0 -- visible to every column -- comes first, so no column's
// running max is still -inf when a later, fully masked block arrives.  Tiles
// are read with cached loads: the query tiles of one sequence re-read the
// same blocks.
#include "pa_paths.h"

namespace pa {

template <class Path, int D>
__global__ __launch_bounds__(64) void pa_prefill_kernel(DecodeParams p,
                                                        const int32_t* __restrict__ qsl,
                                                        int tpu, int q_tiles) {
    extern __shared__ float lds[];
    const int kvhc_count = p.num_kv_heads * p.head_chunks;
    const int kvhc = blockIdx.x % kvhc_count;
    const int sq = blockIdx.x / kvhc_count;
    const int s = sq / q_tiles, qt = sq - s * q_tiles;
    const int kvh = kvhc / p.head_chunks;
    const int hc = kvhc - kvh * p.head_chunks;
    const int gleft = p.group - hc * 16;
    const int gc = gleft < 16 ? gleft : 16;            // heads of this chunk
    const int q0 = qsl[s];
    const int nq = qsl[s + 1] - q0;
    const int j0 = qt * tpu;
    if (j0 >= nq) return;
    const int ntok = min(tpu, nq - j0);
    const int L = p.seq_lens[s];
    const int nb_seq = (L + kBlock - 1) / kBlock;
    bool bad = nq > L || nb_seq > p.max_blocks_per_seq;

    // this lane's column: token jj of the tile, head hh
    const int i = lane_id() & 15;
    const int jj = i / gc;
    const int hh = kvh * p.group + hc * 16 + (i - jj * gc);
    const bool col_ok = jj < ntok && i < tpu * gc;
    const int pos = L - nq + j0 + jj;                  // the column's query position
    const int pos_last = L - nq + j0 + ntok - 1;

    typename Path::State st;
    Path::init(st);
    typename Path::QRegs qr;
    Path::load_q_row(qr, p.q + ((size_t)(q0 + j0 + jj) * p.num_heads + hh) * D, col_ok && !bad);

    const int n = bad ? 0 : pos_last / kBlock + 1;      // blocks 0 .. pos_last / 16
    constexpr int TB = D * kBlock * Path::kElem;
    const char* kbase = p.k_cache + (size_t)kvh * TB;
    const char* vbase = p.v_cache + (size_t)kvh * TB;
    const size_t blk_stride = (size_t)p.num_kv_heads * TB;
    const int32_t* row = p.block_tables + (size_t)s * p.max_blocks_per_seq;
    const float sl2 = p.scale_log2;

    if (n > 0) {
        // the same walk as the decode kernels (table windows of 64 entries,
        // paired tiles, a zero-size request past the last block)
        int cur = table_window<1>(row, 0, n, 0);
        int nxt = table_window<1>(row, 0, n, 64);
        auto phys = [&](int kw, int j) {
            const int d = min(j, n - 1) - kw;
            const int v = d < 64 ? __builtin_amdgcn_readlane(cur, d) : __builtin_amdgcn_readlane(nxt, d - 64);
            const bool ok = (unsigned)v < (unsigned)p.num_blocks;
            bad = bad || !ok;
            return ok ? v : 0;
        };
        auto tile_k = [&](int id) { return kbase + (size_t)id * blk_stride; };
        auto tile_v = [&](int id) { return vbase + (size_t)id * blk_stride; };
        auto valid = [&](int k) { return min(kBlock, L - k * kBlock); };
        // the last key offset of block k this column sees (padding columns: all)
        auto lim = [&](int k) { return col_ok ? min(kBlock - 1, pos - k * kBlock) : kBlock - 1; };
        auto live = [&](int j) { return j < n ? TB : 0; };
        typename Path::Tile ta, tb;
        int id = phys(0, 0);
        Path::template load<false>(ta, tile_k(id), tile_v(id), TB);
        int k = 0;
        for (int kw = 0;; kw += 64) {
            const int pend = table_window<1>(row, 0, n, kw + 128);
            const int kend = min(n, kw + 64) & ~1;
            for (; k < kend; k += 2) {
                id = phys(kw, k + 1);
                Path::template load<false>(tb, tile_k(id), tile_v(id), TB);
                Path::process(st, ta, qr, valid(k), sl2, lim(k));
                id = phys(kw, k + 2);
                Path::template load<false>(ta, tile_k(id), tile_v(id), live(k + 2));
                Path::process(st, tb, qr, valid(k + 1), sl2, lim(k + 1));
            }
            if (kw + 64 >= n) break;
            cur = nxt;
            nxt = pend;
        }
        if (k < n) Path::process(st, ta, qr, valid(k), sl2, lim(k));
    }

    // rows of the tile through LDS, then whole 16-byte stores per lane (the
    // G heads of one token are one contiguous run of G*D floats)
    const float ltot = Path::wave_l(st);
    float* s_o = lds;                 // [16][D]
    float* s_m = lds + 16 * D;        // [16]
    float* s_l = s_m + 16;            // [16]
    Path::stage(st, ltot, s_o, s_m, s_l, 16);
    const f32x4* src = reinterpret_cast<const f32x4*>(s_o);
    const int cols = ntok * gc;       // valid columns: 0 .. cols-1
    for (int e = lane_id(); e < cols * (D / 4); e += 64) {
        const int c = (4 * e) / D;
        const int cj = c / gc;
        const int ch = kvh * p.group + hc * 16 + (c - cj * gc);
        f32x4 v = src[e] * (p.v_scale / s_l[c]);
        if (bad) v = f32x4{NAN, NAN, NAN, NAN};
        float* orow = p.out + ((size_t)(q0 + j0 + cj) * p.num_heads + ch) * D;
        st_stream(reinterpret_cast<f32x4*>(orow) + (e - c * (D / 4)), v);
    }
}

}  // namespace pa

using namespace pa;

extern "C" int pa_prefill(float* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* seq_lens,
                          const int32_t* query_start_loc, int num_seqs, int num_heads,
                          int num_kv_heads, int head_size, int block_size, int max_blocks_per_seq,
                          int num_blocks, int max_query_len, float scale, int kv_cache_dtype,
                          float k_scale, float v_scale, void* stream) {
    int rc = check_decode_args(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads,
                               num_kv_heads, head_size, block_size, max_blocks_per_seq, num_blocks,
                               scale, kv_cache_dtype, k_scale, v_scale);
    if (rc != PA_OK) return rc;
    if (!out || !query_start_loc || max_query_len < 0) return PA_ERR_INVALID_ARG;
    if (!aligned16(out) || !aligned4(query_start_loc)) return PA_ERR_MISALIGNED;
    if (num_seqs == 0 || max_query_len == 0) return PA_OK;
    DecodeParams p = make_params(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads,
                                 num_kv_heads, max_blocks_per_seq, num_blocks, scale,
                                 kv_cache_dtype, k_scale, v_scale);
    p.out = out;
    const int G = num_heads / num_kv_heads;
    p.head_chunks = G > 16 ? (G + 15) / 16 : 1;
    const int tpu = G >= 16 ? 1 : 16 / G;               // query tokens per tile
    const int q_tiles = (max_query_len + tpu - 1) / tpu;
    const long long grid = (long long)num_seqs * q_tiles * num_kv_heads * p.head_chunks;
    if (grid > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
    const size_t lds = (16 * (size_t)head_size + 32) * sizeof(float);
    hipStream_t st = as_stream(stream);
    const bool fp8 = kv_cache_dtype == PA_KV_FP8_E4M3;
#define PA_PREFILL(PATH, DD)                                                                   \
    hipLaunchKernelGGL((pa_prefill_kernel<PATH<DD>, DD>), dim3((unsigned)grid), dim3(64), lds, st, \
                       p, query_start_loc, tpu, q_tiles)
    if (head_size == 128) {
        if (fp8) PA_PREFILL(MfmaPath8, 128);
        else PA_PREFILL(MfmaPath, 128);
    } else {
        if (fp8) PA_PREFILL(MfmaPath8, 64);
        else PA_PREFILL(MfmaPath, 64);
    }
#undef PA_PREFILL
    return launch_status();
}
