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
// One workgroup of four wavefronts per (sequence, four consecutive query
// tiles, KV head, head chunk); the waves share the K/V block pairs through an
// LDS ring (pa_prefill_ring_kernel below), fp16 and fp8 pools alike.
//
// Work unit of a wavefront:
// The columns of the MFMA score tiles S^T = K Q^T are (token, head) pairs of
// one KV group -- 16 NG / G consecutive query tokens times the G heads, or
// NG tokens of 16 heads when G >= 16 -- in NG groups of 16, so every K/V
// tile read serves 16 NG query rows and the MFMA runs full (MHA included:
// 16 NG tokens of one head).  The unit walks block pairs 0 .. p_last/32 in
// order; each column's causal limit is a lane-local mask (the softmax state
// of a column lives in its own lanes), and block 0 -- visible to every
// column -- comes first, so no column's running max is still -inf when a
// later, fully masked block arrives.
#include "pa_paths.h"

#ifndef PA_PREFILL_TILE_MAJOR
#define PA_PREFILL_TILE_MAJOR 0   // grid order: 0 = sequence-major, 1 = query-tile-major
#endif
#ifndef PA_PREFILL_GROUPS
#define PA_PREFILL_GROUPS 2   // 16-column groups per wave (query rows per K/V tile read / 16)
#endif

namespace pa {

constexpr int kPrefillGroups = PA_PREFILL_GROUPS;

// --------------------------------------------------------------------------
// NG groups of 16 columns per wave: every K/V tile read (and, for fp8 pools,
// converted) once feeds NG score tiles and NG PV updates, so a tile serves
// 16*NG query rows.  Each group keeps its own lane-local softmax state.
//
// Blocks are taken in pairs.  The weights of both blocks of a pair share one
// running max, so PV runs over 32 tokens with one 16x16x32 MFMA per 16 head
// dims: lane (i, g) supplies V^T rows 16nt+i at tokens 4g..4g+3 of the first
// block followed by the same tokens of the second, and, as the B operand, its
// own weights of those eight tokens -- the k-order is permuted identically on
// both sides, so the contraction is unchanged.
//
// The running max is raised lazily: a column's max m (log2 units) changes
// only when a score exceeds it by more than kLazy, so weights exp2(t - m) stay
// below 2^kLazy and the accumulator rescale (NT * 4 multiplies per group) is
// skipped on most blocks.  l and acc are always taken relative to the same m,
// so acc / l is unchanged up to rounding.
// --------------------------------------------------------------------------
template <class Base, int NG>
struct MfmaGroups {
    using Path = Base;
    static constexpr int kNG = NG;
    static constexpr int D = Base::kD;
    static constexpr int KC = D / 32;
    static constexpr int NT = D / 16;
    static constexpr int kElem = Base::kElem;
    static constexpr float kLazy = 8.f;
    using Tile = typename Base::Tile;

    struct State {
        f32x4 acc[NG][NT];   // lane (g,i): O^T[d = 16nt + 4g + r][column 16gr + i]
        float m[NG];         // running max of the column, log2 units (score * scale * log2 e)
        float l[NG];         // this lane's share of the column's weight sum
    };
    struct QRegs {
        typename Base::QRegs q[NG];
    };
    struct Half {            // the first block of a pair: scores and V operands
        f32x4 s[NG];
        f16x4 v[NT];
    };

    __device__ static void init(State& st) {
#pragma unroll
        for (int gr = 0; gr < NG; ++gr) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) st.acc[gr][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            st.m[gr] = -INFINITY;
            st.l[gr] = 0.f;
        }
    }

    // Raw scores of one block (q . k).  Tokens at or past nvalid are masked,
    // and, when `causal` (a block that reaches past the earliest column's
    // position), tokens past lim[gr], the last offset this lane's column of
    // group gr may see.  For fp16 tiles, masked V entries are cleared too.
    __device__ __forceinline__ static void scores(f32x4 (&s)[NG], Tile& t, const QRegs& qr, float sl2,
                                                  int nvalid, bool causal, const int (&lim)[NG]) {
        const int g = lane_id() >> 4;
#pragma unroll
        for (int gr = 0; gr < NG; ++gr) s[gr] = f32x4{0.f, 0.f, 0.f, 0.f};
        // group by group, so one group's scores are complete (and its softmax
        // can start) while the next group's MFMAs run; K operands (converted
        // once for fp8 tiles) are shared by the groups
        f16x8 a[KC];
#pragma unroll
        for (int c = 0; c < KC; ++c) a[c] = Base::a_k(t, c);
#pragma unroll
        for (int gr = 0; gr < NG; ++gr)
#pragma unroll
            for (int c = 0; c < KC; ++c)
                s[gr] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[c], qr.q[gr].q[c], s[gr], 0, 0, 0);
        if (nvalid < kBlock || causal) {
#pragma unroll
            for (int gr = 0; gr < NG; ++gr)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (4 * g + r >= nvalid || 4 * g + r > lim[gr]) s[gr][r] = -INFINITY;
        }
        if (nvalid < kBlock) Base::mask_v(t, nvalid);
    }

    // Online-softmax step of group gr over NB raw score tiles: raises the
    // column's running max where a wave-wide ballot finds a score more than
    // kLazy above it (rescaling l and acc), then returns the fp16 weights
    // exp2(s * sl2 - m).  sl2 > 0, so the max of the scaled scores is the
    // scaled max.
    template <int NB>
    __device__ __forceinline__ static void raise_max(State& st, int gr, const f32x4 (&s)[NB][NG],
                                                     float sl2) {
        // IEEE maximum (v_maximum3_f32, no quieting of its inputs first): the
        // scores are finite or -inf (masked), so it is plain max here
        auto mx = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
        float v = mx(mx(s[0][gr][0], s[0][gr][1]), mx(s[0][gr][2], s[0][gr][3]));
#pragma unroll
        for (int b = 1; b < NB; ++b)
            v = mx(v, mx(mx(s[b][gr][0], s[b][gr][1]), mx(s[b][gr][2], s[b][gr][3])));
        const float bm = v * sl2;
        if (__builtin_amdgcn_ballot_w64(bm > st.m[gr] + kLazy) != 0) {
            const float mn = fmaxf(st.m[gr], col4_max(bm));
            const float corr = exp2_fast(st.m[gr] - mn);
            st.l[gr] *= corr;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) st.acc[gr][nt] *= corr;
            st.m[gr] = mn;
        }
    }
    template <int NB>
    __device__ __forceinline__ static void weights(State& st, int gr, const f32x4 (&s)[NB][NG],
                                                   float sl2, f16x4 (&p)[NB]) {
        float sum = 0.f;
        const float nm = -st.m[gr];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float pr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) pr[r] = exp2_fast(fmaf(s[b][gr][r], sl2, nm));
            sum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
            p[b] = f16x4{(f16)pr[0], (f16)pr[1], (f16)pr[2], (f16)pr[3]};
        }
        st.l[gr] += sum;
    }
    template <int NB>
    __device__ __forceinline__ static void weights_group(State& st, int gr, const f32x4 (&s)[NB][NG],
                                                         float sl2, f16x4 (&p)[NB]) {
        raise_max<NB>(st, gr, s, sl2);
        weights<NB>(st, gr, s, sl2, p);
    }

    // One block alone (the last block of a unit with an odd block count).
    __device__ __forceinline__ static void single(State& st, Tile& t, const QRegs& qr, float sl2,
                                                  int nvalid, bool causal, const int (&lim)[NG]) {
        f32x4 s[1][NG];
        scores(s[0], t, qr, sl2, nvalid, causal, lim);
#pragma unroll
        for (int gr = 0; gr < NG; ++gr) {
            f16x4 p[1];
            weights_group<1>(st, gr, s, sl2, p);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                st.acc[gr][nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(Base::a_v(t, nt), p[0], st.acc[gr][nt], 0, 0, 0);
        }
    }

    // First block of a pair: its scores and V operands are kept, so its
    // registers can take the next tile while the second block is processed.
    __device__ __forceinline__ static void first(Half& h, Tile& t, const QRegs& qr, float sl2,
                                                 int nvalid, bool causal, const int (&lim)[NG]) {
        scores(h.s, t, qr, sl2, nvalid, causal, lim);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) h.v[nt] = Base::a_v(t, nt);
    }

    // Second block of a pair: weights of both blocks, then PV over 32 tokens.
    __device__ __forceinline__ static void second(State& st, const Half& h, Tile& t, const QRegs& qr,
                                                  float sl2, int nvalid, bool causal,
                                                  const int (&lim)[NG]) {
        f32x4 s[2][NG];
#pragma unroll
        for (int gr = 0; gr < NG; ++gr) s[0][gr] = h.s[gr];
        scores(s[1], t, qr, sl2, nvalid, causal, lim);
        // group by group: the PV MFMAs of one group run while the VALU
        // computes the next group's weights (7-9% over all weights first)
        f16x8 a[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const f16x4 b = Base::a_v(t, nt);
            a[nt] = f16x8{h.v[nt][0], h.v[nt][1], h.v[nt][2], h.v[nt][3], b[0], b[1], b[2], b[3]};
        }
#pragma unroll
        for (int gr = 0; gr < NG; ++gr) {
            f16x4 p[2];
            weights_group<2>(st, gr, s, sl2, p);
            const f16x8 w = {p[0][0], p[0][1], p[0][2], p[0][3], p[1][0], p[1][1], p[1][2], p[1][3]};
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                st.acc[gr][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[nt], w, st.acc[gr][nt], 0, 0, 0);
        }
    }

    // Rows of group gr to LDS: s_acc[i * D + d] unnormalised, s_inv[i] the
    // column's factor v_scale / (weight sum), one division per column.
    __device__ static void stage_group(const State& st, int gr, float* s_acc, float* s_inv,
                                       float v_scale) {
        const int l = lane_id(), i = l & 15, g = l >> 4;
#pragma unroll
        for (int x = 0; x < NG; ++x) {
            if (x != gr) continue;
            const float ltot = col4_sum(st.l[x]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                *reinterpret_cast<f32x4*>(s_acc + i * D + 16 * nt + 4 * g) = st.acc[x][nt];
            if (g == 0) s_inv[i] = v_scale / ltot;
        }
    }

};


// The (token, head) columns of one wave: lane column c = 16 gr + i is query
// token j0 + c / gc and head c % gc of the chunk.  Loads the Q operands (zeros
// for padding columns or a bad sequence) and each column's position.
template <class G2>
__device__ __forceinline__ void load_columns(typename G2::QRegs& qr, int (&pos)[G2::kNG],
                                             bool (&col_ok)[G2::kNG], const f16* q, int num_heads,
                                             int head0, int gc, int q0, int j0, int ntok, int L,
                                             int nq, bool bad) {
    constexpr int D = G2::D;
    const int i = lane_id() & 15;
#pragma unroll
    for (int gr = 0; gr < G2::kNG; ++gr) {
        const int c = 16 * gr + i;
        const int jj = c / gc;
        col_ok[gr] = jj < ntok;
        pos[gr] = L - nq + j0 + jj;
        G2::Path::load_q_row(qr.q[gr], q + ((size_t)(q0 + j0 + jj) * num_heads + head0 + (c - jj * gc)) * D,
                             col_ok[gr] && !bad);
    }
}

// Floats of a wave's output staging area: 16 rows of D, the 16 columns'
// factors, and the output row index of each of the wave's 16 NG columns.
template <class G2>
constexpr int stage_floats() {
    return 16 * G2::D + 16 + 16 * G2::kNG;
}

// The wave's result rows, group by group through its LDS area s_o
// (stage_floats), then whole 16-byte stores (the heads of one token are one
// contiguous run of gc D floats); NaN rows for a bad sequence.  Each
// column's output row (one integer division) and factor (one float
// division) are computed once, not per stored element.
template <class G2>
__device__ __forceinline__ void store_rows(const typename G2::State& st, float* s_o, float* out,
                                           int num_heads, int head0, int gc, int q0, int j0,
                                           int ntok, float v_scale, bool bad) {
    constexpr int D = G2::D;
    constexpr int NCOL = 16 * G2::kNG;
    float* s_inv = s_o + 16 * D;
    int* s_row = reinterpret_cast<int*>(s_o + 16 * D + 16);
    const int cols = ntok * gc;
    const int lane = lane_id();
    if (lane < NCOL) {   // a row index fits 32 bits: out would not fit in memory otherwise
        const int cj = lane / gc;
        s_row[lane] = (q0 + j0 + cj) * num_heads + head0 + (lane - cj * gc);
    }
    const f32x4* src = reinterpret_cast<const f32x4*>(s_o);
#pragma unroll
    for (int gr = 0; gr < G2::kNG; ++gr) {
        if (16 * gr >= cols) break;
        G2::stage_group(st, gr, s_o, s_inv, v_scale);
        const int cg = min(16, cols - 16 * gr);
        for (int e = lane; e < cg * (D / 4); e += 64) {
            const int ci = e / (D / 4);
            f32x4 v = src[e] * s_inv[ci];
            if (bad) v = f32x4{NAN, NAN, NAN, NAN};
            float* orow = out + (size_t)s_row[16 * gr + ci] * D;
            st_stream(reinterpret_cast<f32x4*>(orow) + (e - ci * (D / 4)), v);
        }
    }
}

// Query rows covered + 0 .. nq - 1 of a sequence with more queries than the
// grid's tiles cover: NaN for this unit's heads.
template <int D>
__device__ __forceinline__ void nan_rows(float* out, int num_heads, int head0, int gc, int q0,
                                         int covered, int nq) {
    const int per_row = gc * D;
    for (int e = lane_id(); e < (nq - covered) * per_row; e += 64) {
        const int r = e / per_row, hd = e - r * per_row;
        out[((size_t)(q0 + covered + r) * num_heads + head0 + hd / D) * D + (hd % D)] = NAN;
    }
}

// Query rows [q0, q0 + nq) of sequence s, from query_start_loc.  A range
// that leaves [0, total_q) or runs backwards marks the sequence bad and is
// clipped to [0, total_q), so its NaN rows never leave q and out.
struct QueryRange {
    int q0, nq;
    bool bad;
};
__device__ __forceinline__ QueryRange query_range(const int32_t* qsl, int s, int total_q) {
    const int a = qsl[s], b = qsl[s + 1];
    QueryRange r;
    r.bad = a < 0 || b < a || b > total_q;
    r.q0 = min(max(a, 0), total_q);
    r.nq = min(max(b, r.q0), total_q) - r.q0;
    return r;
}

// --------------------------------------------------------------------------
// The ring form.  Four waves on consecutive query tiles of one
// (sequence, KV head, head chunk) walk the block pairs of their union range
// through an NS-slot LDS ring.  A slot holds one pair's K0, K1 and V tiles
// and is filled by gfx950's global-to-LDS loads (wave w loads the slot's
// w-th tile's worth, 1 KiB per instruction), so no register holds data in
// flight, and the loads of pair k + NS - 1 go out while pair k is computed.
// The compiler does not track when such loads land, so the waits are
// explicit: loads complete in issue order, so at the top of iteration k a
// wave waits until only the pairs after k + 1 are outstanding, then a
// barrier makes every wave's share of pair k + 1 visible and frees the slot
// of pair k - 1 for refilling.
//
// Within a wave, pairs that need no mask are software-pipelined: iteration k
// raises the running max from pair k's scores (kept from iteration k - 1),
// then issues the score MFMAs of pair k + 1 and computes pair k's weights
// and PV MFMAs in the same stretch of code, so the matrix cores have the next
// pair's scores to work on while the VALU runs this pair's exp2.  Pairs that
// reach the causal diagonal or the sequence end take MfmaGroups' masked
// first / second / single steps on tiles read from LDS.  Either way a pair's
// arithmetic is the same, in the same order.
// --------------------------------------------------------------------------
#ifndef PA_PREFILL_RING_SLOTS
#define PA_PREFILL_RING_SLOTS 3   // pairs in the ring (3 x 16 KiB at D = 128)
#endif

// Where a pair's tiles sit in a ring slot ([K0 | K1 | V of both blocks],
// TB bytes per tile) and how the MFMA operands are read back.  K tiles keep
// their pool layout (16 bytes at 16 (l + 64 r) per lane, conflict-free).
// The two V tiles are interleaved:
//  - fp16: KiB nt holds head dims 16 nt .. 16 nt + 15 of block 0, then of
//    block 1, each half with the 16-byte piece of head dim d, tokens
//    8h .. 8h + 7 at position (d % 16) + 16 h; lane (i, g)'s operand (head
//    dim 16 nt + i, tokens 4g .. 4g + 3 of both blocks) is two 8-byte reads
//    512 bytes apart, each wave-wide read covering 512 consecutive bytes;
//  - fp8: the 16-byte rows (head dim d, 16 tokens) of the two blocks
//    alternate, block b's row d at 32 d + 16 b; lane (i, g)'s operand is two
//    4-byte reads 16 bytes apart, the wave's reads covering 512 consecutive
//    bytes.
// Each 1 KiB load instruction still reads whole 16-byte pieces of the pool.
template <class Path>
struct RingLayout {
    static constexpr int D = Path::kD;
    static constexpr int TB = D * kBlock * Path::kElem;   // bytes of one K (or V) tile
    static constexpr int CPW = TB / 1024;                 // load instructions per tile
    using Tile = typename Path::Tile;

    // V-loading lane l of load instruction c (0 .. 2 CPW - 1 over the
    // pair's V): the block (0 or 1) and the byte of that block's V tile
    __device__ __forceinline__ static int v_block(int l) {
        return Path::kElem == 2 ? l >> 5 : l & 1;
    }
    __device__ __forceinline__ static int v_src(int c, int l) {
        if constexpr (Path::kElem == 2) {
            const int q = l & 31;
            return 32 * (16 * c + (q & 15)) + 16 * (q >> 4);
        } else {
            return 16 * (32 * c + (l >> 1));
        }
    }
    // block b's K tile (raw) and V pieces into a tile as Path::load gives them
    __device__ __forceinline__ static void read_k(Tile& t, const char* sl, int b) {
        const int l = lane_id();
#pragma unroll
        for (int r = 0; r < CPW; ++r)
            t.k[r] = *reinterpret_cast<const std::remove_reference_t<decltype(t.k[0])>*>(sl + b * TB + 16 * (l + 64 * r));
    }
    __device__ __forceinline__ static int v_at(int nt, int b) {
        const int l = lane_id(), i = l & 15, g = l >> 4;
        if constexpr (Path::kElem == 2)
            return 2 * TB + 1024 * nt + 512 * b + 16 * (i + 16 * (g >> 1)) + 8 * (g & 1);
        else
            return 2 * TB + 32 * (16 * nt + i) + 16 * b + 4 * g;
    }
    __device__ __forceinline__ static void read_v(Tile& t, const char* sl, int b) {
#pragma unroll
        for (int nt = 0; nt < D / 16; ++nt)
            t.v[nt] = *reinterpret_cast<const std::remove_reference_t<decltype(t.v[0])>*>(sl + v_at(nt, b));
    }
    // the PV operand of the pair for head dims 16 nt .. 16 nt + 15
    __device__ __forceinline__ static f16x8 v_pair(const char* sl, int nt) {
        f16x4 v0, v1;
        if constexpr (Path::kElem == 2) {
            v0 = *reinterpret_cast<const f16x4*>(sl + v_at(nt, 0));
            v1 = *reinterpret_cast<const f16x4*>(sl + v_at(nt, 1));
        } else {
            v0 = e4m3x4_to_f16x4(*reinterpret_cast<const uint32_t*>(sl + v_at(nt, 0)));
            v1 = e4m3x4_to_f16x4(*reinterpret_cast<const uint32_t*>(sl + v_at(nt, 1)));
        }
        return f16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    }
};

template <class Path, int NG, int NS>
// (two resident waves per SIMD asked of the register allocator: at most 256 VGPRs)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void pa_prefill_ring_kernel(
    DecodeParams p, const int32_t* __restrict__ qsl, int total_q, int tpu, int q_tiles) {
    using G2 = MfmaGroups<Path, NG>;
    using Tile = typename Path::Tile;
    using RL = RingLayout<Path>;
    constexpr int D = Path::kD;
    constexpr int W = 4;                           // waves; wave w loads tile w of each pair
    constexpr int KC = D / 32, NT = D / 16;
    constexpr int TB = RL::TB;                     // bytes of one K (or V) tile
    constexpr int STAGE = 4 * TB;                  // K0 K1 V0 V1
    constexpr int CPW = RL::CPW;                   // load instructions per wave per pair
    static_assert(NS >= 3, "the ring needs a slot being read, one landing and one refilled");
    extern __shared__ __align__(16) char smem[];   // ring[NS][STAGE]; after the walk, per-wave staging
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = lane_id();
    const int kvhc_count = p.num_kv_heads * p.head_chunks;
    const int kvhc = blockIdx.x % kvhc_count;
    const int sq = blockIdx.x / kvhc_count;
#if PA_PREFILL_TILE_MAJOR
    const int rt = sq / p.num_seqs, s = sq - rt * p.num_seqs, qt = q_tiles - 1 - rt;
#else
    // a sequence's query tiles together (they read the same K/V), its last
    // tiles (the longest walks under the causal mask) first
    const int s = sq / q_tiles, qt = q_tiles - 1 - (sq - s * q_tiles);
#endif
    const int kvh = kvhc / p.head_chunks;
    const int hc = kvhc - kvh * p.head_chunks;
    const int gleft = p.group - hc * 16;
    const int gc = gleft < 16 ? gleft : 16;        // heads of this chunk
    const QueryRange qr_ = query_range(qsl, s, total_q);
    const int q0 = qr_.q0, nq = qr_.nq;
    const int jw = qt * W * tpu;                   // first query token of the workgroup
    if (jw >= nq) return;                          // the whole workgroup
    const int j0 = jw + wave * tpu;                // first query token of this wave
    const int ntok = max(0, min(tpu, nq - j0));
    const int L = p.seq_lens[s];
    const int nb_seq = (L + kBlock - 1) / kBlock;
    bool bad = qr_.bad || nq > L || nb_seq > p.max_blocks_per_seq;

    const int head0 = kvh * p.group + hc * 16;
    int pos[NG];
    bool col_ok[NG];
    typename G2::QRegs qr;
    load_columns<G2>(qr, pos, col_ok, p.q, p.num_heads, head0, gc, q0, j0, ntok, L, nq, bad);
    typename G2::State st;
    G2::init(st);

    const int ntok_wg = min(W * tpu, nq - jw);
    const int n = bad ? 0 : (L - nq + jw + ntok_wg - 1) / kBlock + 1;        // blocks of the workgroup
    const int np = (n + 1) / 2;                                              // pairs of the workgroup
    const int n_w = ntok == 0 ? 0 : (L - nq + j0 + ntok - 1) / kBlock + 1;   // blocks of this wave
    const int np_w = (n_w + 1) / 2;
    const int pos_first = L - nq + j0;             // the wave's earliest column
    // pairs of this wave that lie wholly before its earliest column: no mask
    const int nf = ntok == 0 ? 0 : min(np_w, (pos_first + 1) / (2 * kBlock));
    const float sl2 = p.scale_log2;

    if (np > 0) {
        const unsigned num_blocks = (unsigned)p.num_blocks;
        // block ids come through scalar loads (the table is read-only here),
        // so the vector load count holds only the ring's loads
        typedef const int32_t __attribute__((address_space(4)))* ctable_t;
        const ctable_t row = (ctable_t)(p.block_tables + (size_t)s * p.max_blocks_per_seq);
        // The two block ids of pair j are loaded one pair ahead of their use
        // and checked when used, so the scalar loads' latency is hidden.  A
        // wave's rows turn NaN when a block it attends over has an invalid id
        // (the load then reads block 0); other waves' rows are unaffected.
        struct Ids {
            int b0, b1;
        };
        auto load_ids = [&](int j) { return Ids{row[min(2 * j, n - 1)], row[min(2 * j + 1, n - 1)]}; };
        // waves 0 and 1 load K0 and K1 (pool layout); waves 2 and 3 load the
        // pair's two V tiles, interleaved (RingLayout)
        const bool is_v = wave >= 2;
        const char* tbase = (is_v ? p.v_cache : p.k_cache) + (size_t)kvh * TB;
        const size_t blk_stride = (size_t)p.num_kv_heads * TB;
        const bool v_second = RL::v_block(l) == 1;
        int goff[CPW];                             // this lane's source byte in its tile, per KiB piece
#pragma unroll
        for (int c = 0; c < CPW; ++c)
            goff[c] = is_v ? RL::v_src(CPW * (wave - 2) + c, l) : 16 * (64 * c + l);
        auto slot = [&](int j) { return smem + (j % NS) * STAGE; };
        auto issue = [&](int j, const Ids& ids) {
            const bool ok0 = (unsigned)ids.b0 < num_blocks, ok1 = (unsigned)ids.b1 < num_blocks;
            bad = bad || (2 * j < n_w && !ok0) || (2 * j + 1 < n_w && !ok1);
            const int id0 = ok0 ? ids.b0 : 0, id1 = ok1 ? ids.b1 : 0;
            const int id = is_v ? (v_second ? id1 : id0) : ((wave & 1) ? id1 : id0);
            const char* src = tbase + (size_t)id * blk_stride;
            char* dst = slot(j) + wave * TB;
#pragma unroll
            for (int c = 0; c < CPW; ++c)
                __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + goff[c]),
                                                 (__attribute__((address_space(3))) void*)(dst + 1024 * c),
                                                 16, 0, 0);
        };
        // prologue: pairs 0 .. NS - 2 requested, pair 0 waited for
        Ids nid = load_ids(0);
#pragma unroll
        for (int j = 0; j < NS - 1; ++j) {
            if (j < np) {
                issue(j, nid);
                nid = load_ids(j + 1);
            }
        }
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");

        // block b's K operands (fp8 tiles converted to fp16)
        auto k_operands = [&](f16x8 (&a)[KC], const char* sl, int b) {
            Tile t;
            RL::read_k(t, sl, b);
#pragma unroll
            for (int c = 0; c < KC; ++c) a[c] = Path::a_k(t, c);
        };
        auto scores_from = [&](f32x4 (&sc)[2][NG], const f16x8 (&a)[2][KC]) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
#pragma unroll
                for (int gr = 0; gr < NG; ++gr) {
                    sc[b][gr] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int c = 0; c < KC; ++c)
                        sc[b][gr] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[b][c], qr.q[gr].q[c], sc[b][gr], 0, 0, 0);
                }
            }
        };
        auto scores_pair = [&](f32x4 (&sc)[2][NG], const char* sl) {
            f16x8 a[2][KC];
            k_operands(a[0], sl, 0);
            k_operands(a[1], sl, 1);
            scores_from(sc, a);
        };
        auto lds_tile = [&](Tile& t, const char* sl, int b) {
            RL::read_k(t, sl, b);
            RL::read_v(t, sl, b);
        };

        // top of iteration k: pair k + 1 landed (every wave's share), the slot
        // of pair k - 1 refilled with pair k + NS - 1
        auto advance = [&](int k) {
            if (k + 1 >= np) return;
            if (k + NS - 2 < np)
                asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(CPW * (NS - 3)) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (k + NS - 1 < np) {
                issue(k + NS - 1, nid);
                nid = load_ids(k + NS);
            }
        };

        // 1. unmasked pairs, pipelined: the scores of pair k + 1 are computed
        // while pair k's weights and PV run.  Pair k's scores come in sc, pair
        // k + 1's go to sn; the loop is unrolled by two so the two score sets
        // swap roles instead of being copied.  The next pair's scores are
        // always computed (after the last unmasked pair its slot may hold
        // anything and they are dropped), so the score MFMAs and this pair's
        // VALU work share one stretch of code.
        auto fast_pair = [&](int kk, f32x4 (&sc)[2][NG], f32x4 (&sn)[2][NG]) {
            advance(kk);
            const char* sl = slot(kk);
            // the next pair's K operands are requested before the max check,
            // whose branch would otherwise keep them behind it
            Tile kt[2];
            RL::read_k(kt[0], slot(kk + 1), 0);
            RL::read_k(kt[1], slot(kk + 1), 1);
#pragma unroll
            for (int gr = 0; gr < NG; ++gr) G2::template raise_max<2>(st, gr, sc, sl2);
            f16x8 ka[2][KC];
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int c = 0; c < KC; ++c) ka[b][c] = Path::a_k(kt[b], c);
            scores_from(sn, ka);
            f16x8 av[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) av[nt] = RL::v_pair(sl, nt);
#pragma unroll
            for (int gr = 0; gr < NG; ++gr) {
                f16x4 pw[2];
                G2::template weights<2>(st, gr, sc, sl2, pw);
                const f16x8 w = {pw[0][0], pw[0][1], pw[0][2], pw[0][3], pw[1][0], pw[1][1], pw[1][2], pw[1][3]};
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    st.acc[gr][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[nt], w, st.acc[gr][nt], 0, 0, 0);
            }
        };
        int k = 0;
        if (nf > 0) {
            f32x4 sa[2][NG], sb[2][NG];
            scores_pair(sa, slot(0));
            for (; k + 1 < nf; k += 2) {
                fast_pair(k, sa, sb);
                fast_pair(k + 1, sb, sa);
            }
            if (k < nf) {
                fast_pair(k, sa, sb);
                ++k;
            }
        }
        // 2. pairs that reach the diagonal or the sequence end (MfmaGroups'
        // masked steps), then the rest of the workgroup's walk
        for (; k < np; ++k) {
            advance(k);
            if (k >= np_w) continue;
            const char* sl = slot(k);
            int lim[NG];
            const int kb = 2 * k;
#pragma unroll
            for (int gr = 0; gr < NG; ++gr)
                lim[gr] = col_ok[gr] ? min(kBlock - 1, pos[gr] - kb * kBlock) : kBlock - 1;
            Tile ta;
            lds_tile(ta, sl, 0);
            const int va = min(kBlock, L - kb * kBlock);
            const bool ca = kb * kBlock + kBlock - 1 > pos_first;
            if (kb + 1 < n_w) {
                typename G2::Half h;
                G2::first(h, ta, qr, sl2, va, ca, lim);
                Tile tb;
                lds_tile(tb, sl, 1);
#pragma unroll
                for (int gr = 0; gr < NG; ++gr)
                    lim[gr] = col_ok[gr] ? min(kBlock - 1, pos[gr] - (kb + 1) * kBlock) : kBlock - 1;
                G2::second(st, h, tb, qr, sl2, min(kBlock, L - (kb + 1) * kBlock),
                           (kb + 1) * kBlock + kBlock - 1 > pos_first, lim);
            } else {
                G2::single(st, ta, qr, sl2, va, ca, lim);
            }
        }
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }

    // per wave: its rows through its own LDS area (the ring is free after the
    // last barrier)
    store_rows<G2>(st, reinterpret_cast<float*>(smem) + wave * stage_floats<G2>(), p.out, p.num_heads,
                   head0, gc, q0, j0, ntok, p.v_scale, bad);
    if (qt == q_tiles - 1 && wave == 0 && nq > q_tiles * W * tpu)
        nan_rows<D>(p.out, p.num_heads, head0, gc, q0, q_tiles * W * tpu, nq);
}

}  // namespace pa

using namespace pa;

extern "C" int pa_prefill(float* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* seq_lens,
                          const int32_t* query_start_loc, int num_seqs, int total_q,
                          int num_heads, int num_kv_heads, int head_size, int block_size,
                          int max_blocks_per_seq, int num_blocks, int max_query_len, float scale,
                          int kv_cache_dtype, float k_scale, float v_scale, void* stream) {
    int rc = check_decode_args(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads,
                               num_kv_heads, head_size, block_size, max_blocks_per_seq, num_blocks,
                               scale, kv_cache_dtype, k_scale, v_scale);
    if (rc != PA_OK) return rc;
    if (!out || !query_start_loc || max_query_len < 0 || total_q < 0) return PA_ERR_INVALID_ARG;
    if (!aligned16(out) || !aligned4(query_start_loc)) return PA_ERR_MISALIGNED;
    if (num_seqs == 0 || max_query_len == 0 || total_q == 0) return PA_OK;
    DecodeParams p = make_params(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads,
                                 num_kv_heads, max_blocks_per_seq, num_blocks, scale,
                                 kv_cache_dtype, k_scale, v_scale);
    p.out = out;
    const int G = num_heads / num_kv_heads;
    p.head_chunks = G > 16 ? (G + 15) / 16 : 1;
    constexpr int NG = kPrefillGroups;
    const bool fp8 = kv_cache_dtype == PA_KV_FP8_E4M3;
    // four waves per workgroup, each on 16 NG / G query tokens (NG for G >= 16)
    constexpr int W = 4;
    constexpr int NS = PA_PREFILL_RING_SLOTS;
    const int tpu = G >= 16 ? NG : (16 * NG) / G;       // query tokens per wave
    const int q_tiles = (max_query_len + W * tpu - 1) / (W * tpu);
    const long long grid = (long long)num_seqs * q_tiles * num_kv_heads * p.head_chunks;
    if (grid > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
    const size_t ring = NS * 4 * (size_t)head_size * kBlock * kv_elem_bytes(kv_cache_dtype);
    const size_t stage = W * (16 * (size_t)head_size + 16 + 16 * NG) * sizeof(float);   // output staging
    const size_t lds = ring > stage ? ring : stage;
    hipStream_t st = as_stream(stream);
    const dim3 g((unsigned)grid);
#define PA_PREFILL_LAUNCH(KERNEL) \
    hipLaunchKernelGGL((KERNEL), g, dim3(64 * W), lds, st, p, query_start_loc, total_q, tpu, q_tiles)
    if (head_size == 128) {
        if (fp8) PA_PREFILL_LAUNCH((pa_prefill_ring_kernel<MfmaPath8<128>, NG, NS>));
        else PA_PREFILL_LAUNCH((pa_prefill_ring_kernel<MfmaPath<128>, NG, NS>));
    } else {
        if (fp8) PA_PREFILL_LAUNCH((pa_prefill_ring_kernel<MfmaPath8<64>, NG, NS>));
        else PA_PREFILL_LAUNCH((pa_prefill_ring_kernel<MfmaPath<64>, NG, NS>));
    }
#undef PA_PREFILL_LAUNCH
    return launch_status();
}
