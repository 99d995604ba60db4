// Paged decode attention for gfx950 (MI355X): pa_decode_v1 and pa_decode_v2.
//
// What is computed (page "读 vLLM 的 PagedAttention kernel", §2 flowchart,
// §3.3 and §3.4): for one query token per sequence, walk the sequence's block
// table in logical order; for each 16-token block load its K and V tiles from
// the pools (§3.1 layouts), score the block, fold it into a running
// (max, normaliser, accumulator) with an online softmax, and at the end
// write acc / l.  The partitioned variant (§3.3, PARTITION_SIZE > 0) does the
// same over fixed token ranges and writes per-partition (o_p, m_p, l_p) for
// pa_reduce to merge.
//
// Work decomposition.  A work unit is one (sequence, KV head, head chunk)
// in v1 and one (sequence, KV head, head chunk, partition) in v2; a unit
// serves every query head of its KV group (up to 16 per chunk), so each K/V
// byte is read once per KV head.  One workgroup of NW wavefronts runs one
// unit; wave w takes the unit's blocks w, w+NW, w+2NW, ... and the waves'
// states are merged through LDS with the same max/rescale algebra.
// Consecutive workgroups take the KV heads of the same (sequence, partition),
// so concurrently running waves read neighbouring 4 KiB tiles of the same
// physical blocks.  v2 enumerates only the partitions that exist (a prefix
// sum over seq_lens inside each workgroup), so the grid is dense in real
// work and the round-robin placement of workgroups on the eight XCDs stays
// balanced.
//
// Two inner paths:
//  * MFMA (G = H/KVH >= 2).  Scores S^T[t][h] = K[t][:] . Q[h][:] are one
//    16x16 tile per block: D/32 v_mfma_f32_16x16x32_f16 with A = the K tile
//    and B = Q^T.  In the x-packed K layout the 16-byte chunk of lane l at
//    element 512*c + 8*l is exactly A's row (token) l%16, k-group l/16 for
//    k-chunk c, so four coalesced 1 KiB global_load_dwordx4 per block feed
//    the MFMA with no shuffles.  The output tile puts head l%16 and tokens
//    4*(l/16)+r in lane l, which is already the B operand P^T of
//    O^T[d][h] += V^T[d][t] P^T[t][h] (v_mfma_f32_16x16x16_f16, A = V^T read
//    straight from the [d][t] V tile as 8-byte runs).  So the softmax state
//    of head h lives in the lanes with l%16 == h: the per-block max needs a
//    reduction over 4 lanes only, and the rescale of the accumulator is
//    lane-local.
//  * VALU (G == 1).  A single query row is a matrix-vector product, not a
//    dense contraction: lane l owns token l%16 for the scores (v_dot2_f32_f16
//    over its 32 head dims, then a 4-lane sum), the block max is a DPP row
//    reduction, and the PV product uses the 16-byte V chunk of lane l (head
//    dims 32c + l/2, 8 tokens) with fp16 weight pairs fetched by ds_bpermute.
//
// Masking.  Only the last block of a sequence can be partly filled.  Slots
// at or past the sequence length are selected out: their scores become -inf
// and their V elements are replaced by 0 before the product, so NaN or
// garbage in unused slots never reaches the output (0 * NaN would).
//
// Softmax arithmetic.  The running max is kept on the raw dot products; each
// weight is exp2((dot - m) * scale * log2 e), so the largest score of a block
// gets exactly 1 and a one-token sequence returns its V bit-exactly.
#include <math.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_host.h"

// Compile-time tuning knobs (defaults are the measured best on MI355X).
#ifndef PA_LOAD_POLICY
#define PA_LOAD_POLICY 1      // tile loads: 0 = cached, 1 = per unit (see load policy), 2 = nontemporal
#endif
#ifndef PA_V2_WAVES
#define PA_V2_WAVES 0         // waves per v2 workgroup (0 = heuristic)
#endif
#ifndef PA_V1_WAVES
#define PA_V1_WAVES 0         // waves per v1 workgroup (0 = heuristic)
#endif
#ifndef PA_UNIT_ORDER
#define PA_UNIT_ORDER 0       // v2 grid order: 0 = KV heads fastest, 1 = partitions fastest
#endif

namespace pa {

// Tile loads.  K/V that only this unit reads is streamed: nontemporal loads
// do not allocate in the caches, so they neither evict other data nor force
// write-backs of dirty lines (+8% on long contexts against cached loads).
// Blocks that other sequences also reference are read with cached loads,
// so the other readers hit in L2 (-35% time on a shared-prefix batch).
//
// A tile is read through a buffer resource whose base is the (wave-uniform)
// tile address and whose size is the tile's bytes, or 0 for a request that
// only keeps the load count of a loop iteration fixed: an out-of-range
// buffer load returns zeros without touching memory.
constexpr int kBufferDword3 = 0x00020000;   // raw 32-bit data format, no swizzle

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* tile, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(tile), 0, bytes, kBufferDword3);
}

template <bool NT, class T>
__device__ __forceinline__ T ld_tile(__amdgpu_buffer_rsrc_t r, int off) {
    constexpr int cpol = NT ? 2 : 0;   // 2 = nontemporal
    if constexpr (sizeof(T) == 16)
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, cpol));
    else if constexpr (sizeof(T) == 8)
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, cpol));
    else
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, cpol));
}

// Results are written once and not re-read by this kernel.  Plain stores
// allocate in L2 and reach HBM mid-stream, where each write burst costs a
// read/write turnaround: the partials of a 3.5 GB long-context call (27 MB)
// cost ~9% of its time as plain stores and ~3% as nontemporal ones.
#ifndef PA_NT_STORES
#define PA_NT_STORES 1
#endif
template <class T>
__device__ __forceinline__ void st_stream(T* p, T v) {
#if PA_NT_STORES
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

struct DecodeParams {
    float* out;           // v1: out[S,H,D]; v2: tmp_out[S,H,P,D]
    float* exp_sums;      // v2: [S,H,P]
    float* max_logits;    // v2: [S,H,P]
    const f16* q;
    const char* k_cache;  // pools as bytes: fp16 or fp8 (E4M3) elements
    const char* v_cache;
    const int32_t* block_tables;
    const int32_t* seq_lens;
    int num_seqs;
    int num_heads;
    int num_kv_heads;
    int group;            // H / KVH
    int head_chunks;      // ceil(group / 16) on the MFMA path, 1 on the VALU path
    int max_blocks_per_seq;
    int num_blocks;
    int max_num_partitions;
    int partition_size;   // tokens, multiple of 16 (v2)
    float scale;          // natural units (fp8: scale * k_scale)
    float scale_log2;     // scale * log2(e)
    float v_scale;        // fp8: V's per-tensor scale; fp16: 1
};

// --------------------------------------------------------------------------
// Block-table access: the wave's blocks k = 0..n-1 (logical block
// first + k*NW) have their physical ids cached 64 at a time in one VGPR
// (lane j of window i holds entry 64i + j, clamped to the last entry) and are
// read back with v_readlane.  Every lane always loads, so a window is a plain
// unconditional load with nothing to merge afterwards.
// --------------------------------------------------------------------------
template <int NW>
__device__ __forceinline__ int table_window(const int32_t* row, int first, int n, int kbase) {
    const int k = min(kbase + lane_id(), n - 1);
    return row[first + k * NW];
}

// --------------------------------------------------------------------------
// MFMA path (2 <= G): up to 16 query heads of one KV group per wave
// --------------------------------------------------------------------------
template <int D>
struct MfmaPath {
    static constexpr int KC = D / 32;   // 16x16x32 steps for the scores
    static constexpr int NT = D / 16;   // 16-wide head-dim tiles of the output
    static constexpr int kHeads = 16;
    static constexpr int kElem = 2;     // bytes per cache element (fp16)

    struct Tile {
        f16x8 k[KC];   // lane (g,i): K[t=i][d = 32c + 8g .. +7]
        f16x4 v[NT];   // lane (g,i): V[d = 16nt + i][t = 4g .. 4g+3]
    };
    struct State {
        f32x4 acc[NT]; // lane (g,i): O^T[d = 16nt + 4g + r][h = i]
        float m;       // running max of raw dot products of head i
        float l;       // sum of weights over this lane's tokens 4g..4g+3
    };
    struct QRegs {
        f16x8 q[KC];   // lane (g,i): Q[h = i][d = 32c + 8g .. +7]
    };

    __device__ static void load_q(QRegs& qr, const DecodeParams& p, int s, int h0, int nh) {
        const int l = lane_id(), i = l & 15, g = l >> 4;
        const f16* qrow = p.q + ((size_t)s * p.num_heads + h0 + i) * D + 8 * g;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            f16x8 z = {};
            qr.q[c] = (i < nh) ? *reinterpret_cast<const f16x8*>(qrow + 32 * c) : z;
        }
    }

    __device__ static void init(State& st) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) st.acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        st.m = -INFINITY;
        st.l = 0.f;
    }

    template <bool NTL>
    __device__ __forceinline__ static void load(Tile& t, const char* kt, const char* vt, int bytes) {
        const int l = lane_id(), i = l & 15, g = l >> 4;
        const auto rk = tile_rsrc(kt, bytes), rv = tile_rsrc(vt, bytes);
#pragma unroll
        for (int c = 0; c < KC; ++c) t.k[c] = ld_tile<NTL, f16x8>(rk, 16 * (l + 64 * c));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) t.v[nt] = ld_tile<NTL, f16x4>(rv, 8 * (4 * i + g + 64 * nt));
    }

    __device__ __forceinline__ static void process(State& st, Tile& t, const QRegs& qr,
                                                   int nvalid, float sl2) {
        const int l = lane_id(), g = l >> 4;
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KC; ++c)
            s = __builtin_amdgcn_mfma_f32_16x16x32_f16(t.k[c], qr.q[c], s, 0, 0, 0);
        if (nvalid < kBlock) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (4 * g + r >= nvalid) s[r] = -INFINITY;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (4 * g + r >= nvalid) t.v[nt][r] = (f16)0.f;
        }
        float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        bm = col4_max(bm);
        const float mn = fmaxf(st.m, bm);
        const float corr = exp2_fast((st.m - mn) * sl2);
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = exp2_fast((s[r] - mn) * sl2);
        st.l = st.l * corr + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
        st.m = mn;
        const f16x4 pv = {(f16)pr[0], (f16)pr[1], (f16)pr[2], (f16)pr[3]};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            st.acc[nt] *= corr;
            st.acc[nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(t.v[nt], pv, st.acc[nt], 0, 0, 0);
        }
    }

    // Per-head totals of the wave: l summed over the four token groups.
    __device__ static float wave_l(const State& st) { return col4_sum(st.l); }

    // Stage the wave's state for the cross-wave merge: acc[h][d] unnormalised.
    __device__ static void stage(const State& st, float ltot, float* s_acc, float* s_m,
                                 float* s_l, int nh) {
        const int l = lane_id(), i = l & 15, g = l >> 4;
        if (i >= nh) return;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            *reinterpret_cast<f32x4*>(s_acc + i * D + 16 * nt + 4 * g) = st.acc[nt];
        if (g == 0) {
            s_m[i] = st.m;
            s_l[i] = ltot;
        }
    }
};

// --------------------------------------------------------------------------
// VALU path (G == 1): one query head per wave
// --------------------------------------------------------------------------
template <int D>
struct ValuPath {
    static constexpr int KC = D / 32;
    static constexpr int kHeads = 1;
    static constexpr int kElem = 2;

    struct Tile {
        f16x8 k[KC];   // lane l: K[t = l%16][d = 32c + 8(l/16) .. +7]
        f16x8 v[KC];   // lane l: V[d = 32c + l/2][t = 8(l&1) .. +7]
    };
    struct State {
        float acc[KC]; // lane l: partial O[d = 32c + l/2] over tokens 8(l&1)..+7
        float m;       // running max of raw dot products
        float l;       // sum of weights of token l%16 over blocks
    };
    struct QRegs {
        f16x8 q[KC];   // lane l: q[d = 32c + 8(l/16) .. +7]
    };

    __device__ static void load_q(QRegs& qr, const DecodeParams& p, int s, int h0, int) {
        const int g = lane_id() >> 4;
        const f16* qrow = p.q + ((size_t)s * p.num_heads + h0) * D + 8 * g;
#pragma unroll
        for (int c = 0; c < KC; ++c) qr.q[c] = *reinterpret_cast<const f16x8*>(qrow + 32 * c);
    }

    __device__ static void init(State& st) {
#pragma unroll
        for (int c = 0; c < KC; ++c) st.acc[c] = 0.f;
        st.m = -INFINITY;
        st.l = 0.f;
    }

    template <bool NTL>
    __device__ __forceinline__ static void load(Tile& t, const char* kt, const char* vt, int bytes) {
        const int l = lane_id();
        const auto rk = tile_rsrc(kt, bytes), rv = tile_rsrc(vt, bytes);
#pragma unroll
        for (int c = 0; c < KC; ++c) t.k[c] = ld_tile<NTL, f16x8>(rk, 16 * (l + 64 * c));
#pragma unroll
        for (int c = 0; c < KC; ++c) t.v[c] = ld_tile<NTL, f16x8>(rv, 16 * (l + 64 * c));
    }

    __device__ __forceinline__ static void process(State& st, Tile& t, const QRegs& qr,
                                                   int nvalid, float sl2) {
        const int l = lane_id(), i = l & 15, h = l & 1;
        float part = 0.f;
#pragma unroll
        for (int c = 0; c < KC; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                part = dot2(f16x2{t.k[c][2 * j], t.k[c][2 * j + 1]},
                            f16x2{qr.q[c][2 * j], qr.q[c][2 * j + 1]}, part);
        float z = col4_sum(part);               // dot of token i, in every row
        if (nvalid < kBlock) {
            if (i >= nvalid) z = -INFINITY;
#pragma unroll
            for (int c = 0; c < KC; ++c)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (8 * h + j >= nvalid) t.v[c][j] = (f16)0.f;
        }
        const float bm = row16_max(z);
        const float mn = fmaxf(st.m, bm);
        const float corr = exp2_fast((st.m - mn) * sl2);
        const float pw = exp2_fast((z - mn) * sl2);
        st.l = st.l * corr + pw;
        st.m = mn;
        // even lane t holds the fp16 pair (p_t, p_{t+1}); lane l needs the
        // pairs of tokens 8h + 2kk, kk = 0..3
        const f16x2 pair = pack2(pw, dpp<kDppXor1>(pw));
        const int pair_bits = __builtin_bit_cast(int, pair);
        f16x2 pp[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            pp[kk] = __builtin_bit_cast(f16x2, fetch_lane(pair_bits, 8 * h + 2 * kk));
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            float a = st.acc[c] * corr;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                a = dot2(f16x2{t.v[c][2 * kk], t.v[c][2 * kk + 1]}, pp[kk], a);
            st.acc[c] = a;
        }
    }

    __device__ static float wave_l(const State& st) { return row16_sum(st.l); }

    __device__ static void stage(const State& st, float ltot, float* s_acc, float* s_m,
                                 float* s_l, int) {
        const int l = lane_id();
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            const float full = st.acc[c] + dpp<kDppXor1>(st.acc[c]);
            if ((l & 1) == 0) s_acc[32 * c + (l >> 1)] = full;
        }
        if (l == 0) {
            s_m[0] = st.m;
            s_l[0] = ltot;
        }
    }
};

// --------------------------------------------------------------------------
// fp8 (E4M3) cache, MFMA path.  The K pool packs 16 head dims per token
// chunk, so lane (g,i) loads token i's dims 16(g + 4r) .. +15 of k-chunk r
// with one 16-byte request per 64 dims; each 16 dims feed two 16x16x32
// score steps after an exact E4M3 -> fp16 conversion.  The sum over d does
// not care which dims a step takes, as long as Q^T is loaded the same way:
// step c uses d = 16(g + 4(c/2)) + 8(c%2) + e.  V rows are 16 bytes (one per
// head dim, 16 tokens), and lane (g,i) takes the 4 tokens 4g..4g+3 of row
// 16nt + i, the A operand of the PV step.  k_scale is folded into the
// softmax scale and v_scale into the final normalisation.
// --------------------------------------------------------------------------
template <int D>
struct MfmaPath8 : MfmaPath<D> {
    using Base = MfmaPath<D>;
    static constexpr int KC = D / 32;
    static constexpr int KR = D / 64;   // 16-byte K chunks per lane
    static constexpr int NT = D / 16;
    static constexpr int kElem = 1;

    struct Tile {
        u32x4 k[KR];    // lane (g,i): K codes of token i, dims 16(g + 4r) .. +15
        uint32_t v[NT]; // lane (g,i): V codes of dim 16nt + i, tokens 4g .. 4g+3
    };
    struct QRegs {
        f16x8 q[KC];    // lane (g,i): Q[h = i][d = 16(g + 4(c/2)) + 8(c%2) .. +7]
    };

    __device__ static void load_q(QRegs& qr, const DecodeParams& p, int s, int h0, int nh) {
        const int l = lane_id(), i = l & 15, g = l >> 4;
        const f16* qrow = p.q + ((size_t)s * p.num_heads + h0 + i) * D;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            f16x8 z = {};
            const int d0 = 16 * (g + 4 * (c >> 1)) + 8 * (c & 1);
            qr.q[c] = (i < nh) ? *reinterpret_cast<const f16x8*>(qrow + d0) : z;
        }
    }

    template <bool NTL>
    __device__ __forceinline__ static void load(Tile& t, const char* kt, const char* vt, int bytes) {
        const int l = lane_id(), i = l & 15, g = l >> 4;
        const auto rk = tile_rsrc(kt, bytes), rv = tile_rsrc(vt, bytes);
#pragma unroll
        for (int r = 0; r < KR; ++r) t.k[r] = ld_tile<NTL, u32x4>(rk, 16 * (l + 64 * r));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) t.v[nt] = ld_tile<NTL, uint32_t>(rv, 16 * (16 * nt + i) + 4 * g);
    }

    __device__ __forceinline__ static void process(typename Base::State& st, Tile& t,
                                                   const QRegs& qr, int nvalid, float sl2) {
        const int l = lane_id(), g = l >> 4;
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            const uint32_t w0 = t.k[c >> 1][2 * (c & 1)], w1 = t.k[c >> 1][2 * (c & 1) + 1];
            const f16x4 a0 = e4m3x4_to_f16x4(w0), a1 = e4m3x4_to_f16x4(w1);
            const f16x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            s = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qr.q[c], s, 0, 0, 0);
        }
        if (nvalid < kBlock) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (4 * g + r >= nvalid) s[r] = -INFINITY;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) t.v[nt] = keep_tokens(t.v[nt], 4 * g, nvalid);
        }
        float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        bm = col4_max(bm);
        const float mn = fmaxf(st.m, bm);
        const float corr = exp2_fast((st.m - mn) * sl2);
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = exp2_fast((s[r] - mn) * sl2);
        st.l = st.l * corr + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
        st.m = mn;
        const f16x4 pv = {(f16)pr[0], (f16)pr[1], (f16)pr[2], (f16)pr[3]};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            st.acc[nt] *= corr;
            st.acc[nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(e4m3x4_to_f16x4(t.v[nt]), pv,
                                                               st.acc[nt], 0, 0, 0);
        }
    }
};

// --------------------------------------------------------------------------
// fp8 (E4M3) cache, VALU path (G == 1).  Scores as in the fp16 path, with
// lane l holding token l%16's dims 16(l/16 + 4r) .. +15.  A V row is the 16
// tokens of one head dim in 16 bytes, so lane l takes whole rows d = 64r + l
// and needs all 16 weights: the eight fp16 weight pairs are the same for
// every lane and are read into scalar registers (v_readlane), and each
// lane's output dims are complete without a cross-lane sum.
// --------------------------------------------------------------------------
template <int D>
struct ValuPath8 {
    static constexpr int KR = D / 64;
    static constexpr int kHeads = 1;
    static constexpr int kElem = 1;

    struct Tile {
        u32x4 k[KR];   // lane l: K codes of token l%16, dims 16(l/16 + 4r) .. +15
        u32x4 v[KR];   // lane l: V codes of dim 64r + l, tokens 0..15
    };
    struct State {
        float acc[KR]; // lane l: O[d = 64r + l], unnormalised
        float m;       // running max of raw dot products
        float l;       // sum of weights of token l%16 over blocks
    };
    struct QRegs {
        f16x8 q[2 * KR];   // lane l: q[d = 16(l/16 + 4r) + 8j .. +7] at index 2r + j
    };

    __device__ static void load_q(QRegs& qr, const DecodeParams& p, int s, int h0, int) {
        const int g = lane_id() >> 4;
        const f16* qrow = p.q + ((size_t)s * p.num_heads + h0) * D;
#pragma unroll
        for (int r = 0; r < KR; ++r)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                qr.q[2 * r + j] = *reinterpret_cast<const f16x8*>(qrow + 16 * (g + 4 * r) + 8 * j);
    }

    __device__ static void init(State& st) {
#pragma unroll
        for (int r = 0; r < KR; ++r) st.acc[r] = 0.f;
        st.m = -INFINITY;
        st.l = 0.f;
    }

    template <bool NTL>
    __device__ __forceinline__ static void load(Tile& t, const char* kt, const char* vt, int bytes) {
        const int l = lane_id();
        const auto rk = tile_rsrc(kt, bytes), rv = tile_rsrc(vt, bytes);
#pragma unroll
        for (int r = 0; r < KR; ++r) t.k[r] = ld_tile<NTL, u32x4>(rk, 16 * (l + 64 * r));
#pragma unroll
        for (int r = 0; r < KR; ++r) t.v[r] = ld_tile<NTL, u32x4>(rv, 16 * (64 * r + l));
    }

    __device__ __forceinline__ static void process(State& st, Tile& t, const QRegs& qr,
                                                   int nvalid, float sl2) {
        const int l = lane_id(), i = l & 15;
        float part = 0.f;
#pragma unroll
        for (int r = 0; r < KR; ++r)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const f16x8& qh = qr.q[2 * r + (w >> 1)];
                const int e = 4 * (w & 1);
                const f16x4 kk = e4m3x4_to_f16x4(t.k[r][w]);
                part = dot2(f16x2{kk[0], kk[1]}, f16x2{qh[e], qh[e + 1]}, part);
                part = dot2(f16x2{kk[2], kk[3]}, f16x2{qh[e + 2], qh[e + 3]}, part);
            }
        float z = col4_sum(part);               // dot of token i, in every row
        if (nvalid < kBlock) {
            if (i >= nvalid) z = -INFINITY;
#pragma unroll
            for (int r = 0; r < KR; ++r)
#pragma unroll
                for (int w = 0; w < 4; ++w) t.v[r][w] = keep_tokens(t.v[r][w], 4 * w, nvalid);
        }
        const float bm = row16_max(z);
        const float mn = fmaxf(st.m, bm);
        const float corr = exp2_fast((st.m - mn) * sl2);
        const float pw = exp2_fast((z - mn) * sl2);
        st.l = st.l * corr + pw;
        st.m = mn;
        // even lane t holds the fp16 pair (p_t, p_{t+1}); every lane needs all
        // eight pairs, which are wave-uniform
        const int pair_bits = __builtin_bit_cast(int, pack2(pw, dpp<kDppXor1>(pw)));
        f16x2 wp[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            wp[k] = __builtin_bit_cast(f16x2, __builtin_amdgcn_readlane(pair_bits, 2 * k));
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            float a = st.acc[r] * corr;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const f16x4 vv = e4m3x4_to_f16x4(t.v[r][w]);
                a = dot2(f16x2{vv[0], vv[1]}, wp[2 * w], a);
                a = dot2(f16x2{vv[2], vv[3]}, wp[2 * w + 1], a);
            }
            st.acc[r] = a;
        }
    }

    __device__ static float wave_l(const State& st) { return row16_sum(st.l); }

    __device__ static void stage(const State& st, float ltot, float* s_acc, float* s_m,
                                 float* s_l, int) {
        const int l = lane_id();
#pragma unroll
        for (int r = 0; r < KR; ++r) s_acc[64 * r + l] = st.acc[r];
        if (l == 0) {
            s_m[0] = st.m;
            s_l[0] = ltot;
        }
    }
};

// --------------------------------------------------------------------------
// Load policy: a unit is taken to read shared blocks when the physical block
// at its first logical position also sits at that position in the table of
// the sequence before or after it (forked sequences, parallel samples and
// beams of one request share their prefix blocks and are batched next to
// each other).  Only the first block is compared: a shared prefix is a
// leading run of blocks.
// --------------------------------------------------------------------------
__device__ __forceinline__ bool shared_unit(const DecodeParams& p, int s, int blk) {
    const int32_t* bt = p.block_tables;
    const size_t w = (size_t)p.max_blocks_per_seq;
    const int b0 = bt[(size_t)s * w + blk];
    bool shared = false;
    if (s > 0 && blk * kBlock < p.seq_lens[s - 1]) shared = bt[(size_t)(s - 1) * w + blk] == b0;
    if (s + 1 < p.num_seqs && blk * kBlock < p.seq_lens[s + 1])
        shared = shared || bt[(size_t)(s + 1) * w + blk] == b0;
    return __builtin_amdgcn_readfirstlane((int)shared) != 0;
}

// --------------------------------------------------------------------------
// v2 unit lookup: the r-th existing partition, counting sequences in order
// and partitions p < ceil(L_s / PS) (capped at max_num_partitions).
// --------------------------------------------------------------------------
__device__ __forceinline__ int n_parts(int L, int PS, int Pmax) {
    if (L <= 0) return 0;
    const int n = (L - 1) / PS + 1;
    return n < Pmax ? n : Pmax;
}

__device__ int total_partitions(const DecodeParams& p) {
    int total = 0;
    for (int s0 = 0; s0 < p.num_seqs; s0 += 64) {
        const int s = s0 + lane_id();
        float np = (s < p.num_seqs) ? (float)n_parts(p.seq_lens[s], p.partition_size, p.max_num_partitions) : 0.f;
        total += (int)wave_sum(np);
    }
    return __builtin_amdgcn_readfirstlane(total);
}

__device__ bool find_partition(const DecodeParams& p, int r, int& s_out, int& p_out) {
    const int lane = lane_id();
    int base = 0;  // partitions of the sequences before this chunk (uniform)
    for (int s0 = 0; s0 < p.num_seqs; s0 += 64) {
        const int s = s0 + lane;
        const int np = (s < p.num_seqs) ? n_parts(p.seq_lens[s], p.partition_size, p.max_num_partitions) : 0;
        int incl = np;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(incl, off);
            if (lane >= off) incl += t;
        }
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (r < base + total) {
            const unsigned long long mask = __ballot(base + incl > r);
            const int first = __ffsll((long long)mask) - 1;
            const int excl = __builtin_amdgcn_readlane(incl - np, first);
            s_out = s0 + first;
            p_out = r - base - excl;
            return true;
        }
        base += total;
    }
    return false;
}

// --------------------------------------------------------------------------
// The kernel
// --------------------------------------------------------------------------
#ifndef PA_WAVES_PER_EU
#define PA_WAVES_PER_EU 0
#endif
template <class Path, int D, int NW, bool V2>
__global__ __launch_bounds__(64 * NW)
#if PA_WAVES_PER_EU
__attribute__((amdgpu_waves_per_eu(PA_WAVES_PER_EU)))
#endif
void pa_decode_kernel(DecodeParams p) {
    extern __shared__ float lds[];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, uniform
    const int kvhc_count = p.num_kv_heads * p.head_chunks;
#if PA_UNIT_ORDER == 1
    int kvhc, r_unit;
    if constexpr (V2) {
        const int R = total_partitions(p);
        if ((int)blockIdx.x >= R * kvhc_count) return;
        kvhc = blockIdx.x / R;
        r_unit = blockIdx.x % R;
    } else {
        kvhc = blockIdx.x % kvhc_count;
        r_unit = blockIdx.x / kvhc_count;
    }
#else
    const int kvhc = blockIdx.x % kvhc_count;
    const int r_unit = blockIdx.x / kvhc_count;
#endif
    const int kvh = kvhc / p.head_chunks;
    const int hc = kvhc - kvh * p.head_chunks;
    const int h0 = kvh * p.group + hc * Path::kHeads;
    const int nh_left = p.group - hc * Path::kHeads;
    const int nh = nh_left < Path::kHeads ? nh_left : Path::kHeads;

    int s, part = 0;
    if constexpr (V2) {
        if (!find_partition(p, r_unit, s, part)) return;
    } else {
        s = r_unit;
    }
    const int L = p.seq_lens[s];
    // v1 out[S][H][D]; v2 tmp_out[S][P][H][D]: either way the unit's heads
    // are consecutive rows, so its result is one contiguous run of memory
    const size_t out_head_stride = D;
    const size_t row0 = V2 ? ((size_t)s * p.max_num_partitions + part) * p.num_heads + h0
                           : (size_t)s * p.num_heads + h0;
    float* out_h0 = p.out + row0 * D;   // exp_sums / max_logits [S][P][H]: index row0 + j

    if (!V2 && L <= 0) {  // empty sequence: zeros (v2 has no partition for it)
        for (int e = threadIdx.x; e < nh * D; e += 64 * NW)
            st_stream(out_h0 + (size_t)(e / D) * out_head_stride + (e % D), 0.f);
        return;
    }
    const int nb_seq = (L + kBlock - 1) / kBlock;
    bool bad = nb_seq > p.max_blocks_per_seq;
    if constexpr (V2) bad = bad || (L - 1) / p.partition_size + 1 > p.max_num_partitions;

    // token / block range of this unit
    int tok_end = L, blk_begin = 0, blk_end = nb_seq;
    if constexpr (V2) {
        const int pb = p.partition_size / kBlock;
        blk_begin = part * pb;
        blk_end = min(nb_seq, blk_begin + pb);
        tok_end = min(L, (part + 1) * p.partition_size);
    }
    if (bad) blk_end = blk_begin;  // read nothing

    typename Path::State st;
    Path::init(st);
    typename Path::QRegs qr;
    Path::load_q(qr, p, s, h0, nh);

    // this wave's blocks: blk_begin + w + k*NW, k < n
    const int first = blk_begin + w;
    const int n = first < blk_end ? (blk_end - first + NW - 1) / NW : 0;
    constexpr int TB = D * kBlock * Path::kElem;           // bytes of one K or V tile
    const char* kbase = p.k_cache + (size_t)kvh * TB;
    const char* vbase = p.v_cache + (size_t)kvh * TB;
    const size_t blk_stride = (size_t)p.num_kv_heads * TB;
    const int32_t* row = p.block_tables + (size_t)s * p.max_blocks_per_seq;
    const float sl2 = p.scale_log2;

    if (n > 0) {
        // The wave walks its blocks in windows of 64 table entries: `cur` holds
        // window kw, `nxt` window kw + 64 (requested one window ahead), and
        // `pend` window kw + 128 (requested as window kw starts, so it has had
        // 64 blocks of time when it moves up).  Inside a window the tiles are
        // double-buffered in registers: block k + 1 is requested before block
        // k is processed.
        //
        // Every loop iteration requests the same number of tiles, so the wait
        // counts before each use are exact (a request under a branch makes the
        // compiler wait on the newer loads too): past the wave's last block
        // the request is an empty one (a zero-size buffer, no memory access).
        // The table index is clamped rather than the previous id kept, so the
        // compiler cannot prove two requests equal and replace one by a
        // register copy (which would drain the load queue).  An id outside
        // the pool marks the unit bad and reads block 0.
        int cur = table_window<NW>(row, first, n, 0);
        int nxt = table_window<NW>(row, first, n, 64);
        auto phys = [&](int kw, int j) {
            const int d = min(j, n - 1) - kw;
            const int v = d < 64 ? __builtin_amdgcn_readlane(cur, d) : __builtin_amdgcn_readlane(nxt, d - 64);
            const bool ok = (unsigned)v < (unsigned)p.num_blocks;
            bad = bad || !ok;
            return ok ? v : 0;
        };
        auto tile_k = [&](int id) { return kbase + (size_t)id * blk_stride; };
        auto tile_v = [&](int id) { return vbase + (size_t)id * blk_stride; };
        auto valid = [&](int k) { return min(kBlock, tok_end - (first + k * NW) * kBlock); };
        auto live = [&](int j) { return j < n ? TB : 0; };
        auto walk = [&](auto nt_tag) {
            constexpr bool NTL = decltype(nt_tag)::value;
            typename Path::Tile ta, tb;
            int id = phys(0, 0);
            Path::template load<NTL>(ta, tile_k(id), tile_v(id), TB);
            int k = 0;
            for (int kw = 0;; kw += 64) {
                const int pend = table_window<NW>(row, first, n, kw + 128);
                const int kend = min(n, kw + 64) & ~1;   // pairs; an odd last block is the tail
                for (; k < kend; k += 2) {
                    id = phys(kw, k + 1);
                    Path::template load<NTL>(tb, tile_k(id), tile_v(id), TB);
                    Path::process(st, ta, qr, valid(k), sl2);
                    id = phys(kw, k + 2);
                    Path::template load<NTL>(ta, tile_k(id), tile_v(id), live(k + 2));
                    Path::process(st, tb, qr, valid(k + 1), sl2);
                }
                if (kw + 64 >= n) break;
                cur = nxt;
                nxt = pend;
            }
            if (k < n) Path::process(st, ta, qr, valid(k), sl2);   // odd block count
        };
#if PA_LOAD_POLICY == 1
        if (shared_unit(p, s, blk_begin)) walk(std::false_type{});   // cached loads
        else walk(std::true_type{});
#else
        walk(std::integral_constant<bool, PA_LOAD_POLICY == 2>{});
#endif
    }

    const float ltot = Path::wave_l(st);
    if constexpr (NW == 1) {
        // The unit's result (nh rows of D, one contiguous run) goes out as
        // whole 1 KiB-per-instruction stores: stage the rows in LDS (this
        // wave only, so program order orders the accesses), then each lane
        // writes 16 contiguous bytes.  Storing straight from the MFMA layout
        // would write every cache line in two halves from two instructions.
        const int HP = Path::kHeads;
        float* s_o = lds;                 // [nh][D]
        float* s_m = lds + nh * D;        // [HP]
        float* s_l = s_m + HP;            // [HP]
        Path::stage(st, ltot, s_o, s_m, s_l, nh);
        const f32x4* src = reinterpret_cast<const f32x4*>(s_o);
        const int nv = nh * D / 4;
        for (int e = lane_id(); e < nv; e += 64) {
            const float inv = p.v_scale / s_l[(4 * e) / D];
            f32x4 v = src[e] * inv;
            if (bad) v = f32x4{NAN, NAN, NAN, NAN};
            st_stream(reinterpret_cast<f32x4*>(out_h0) + e, v);
        }
        if constexpr (V2) {
            // lane l < nh holds head l's max and total weight on both paths
            const int l = lane_id();
            if (l < nh) {
                st_stream(p.max_logits + row0 + l, bad ? NAN : st.m * p.scale);
                st_stream(p.exp_sums + row0 + l, bad ? NAN : ltot);
            }
        }
        return;
    } else {
        // merge the NW wave states through LDS
        const int HP = Path::kHeads;
        float* s_acc = lds;                              // [NW][nh][D]
        float* s_m = lds + NW * nh * D;                  // [NW][HP]
        float* s_l = s_m + NW * HP;                      // [NW][HP]
        int* s_bad = reinterpret_cast<int*>(s_l + NW * HP);  // [NW]
        float* s_fin = reinterpret_cast<float*>(s_bad + NW);  // [2][16]: merged m, l
        Path::stage(st, ltot, s_acc + w * nh * D, s_m + w * HP, s_l + w * HP, nh);
        if (lane_id() == 0) s_bad[w] = bad ? 1 : 0;
        __syncthreads();
        int any_bad = 0;
#pragma unroll
        for (int v = 0; v < NW; ++v) any_bad |= s_bad[v];
        for (int e = threadIdx.x; e < nh * D; e += 64 * NW) {
            const int j = e / D, d = e - j * D;
            float M = -INFINITY;
#pragma unroll
            for (int v = 0; v < NW; ++v) M = fmaxf(M, s_m[v * HP + j]);
            float num = 0.f, den = 0.f;
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                const float f = exp2_fast((s_m[v * HP + j] - M) * sl2);
                num += s_acc[(v * nh + j) * D + d] * f;
                den += s_l[v * HP + j] * f;
            }
            st_stream(out_h0 + (size_t)j * out_head_stride + d, any_bad ? NAN : num / den * p.v_scale);
            if (V2 && d == 0) {
                s_fin[j] = M;
                s_fin[16 + j] = den;
            }
        }
        if constexpr (V2) {
            __syncthreads();
            const int t = threadIdx.x;
            if (t < nh) {
                st_stream(p.max_logits + row0 + t, any_bad ? NAN : s_fin[t] * p.scale);
                st_stream(p.exp_sums + row0 + t, any_bad ? NAN : s_fin[16 + t]);
            }
        }
    }
}

// --------------------------------------------------------------------------
// Host side
// --------------------------------------------------------------------------
static size_t merge_lds_bytes(int NW, int nh_max, int D, int hp) {
    // NW == 1: the staging buffer of the final store; NW > 1: the merge
    return (size_t)NW * ((size_t)nh_max * D + 2 * hp) * sizeof(float) + NW * sizeof(int) +
           32 * sizeof(float);
}

template <class Path, int D, bool V2>
static int launch_nw(int NW, const DecodeParams& p, int grid, int nh_max, hipStream_t st) {
    // keep the merge buffer within the default 64 KiB of dynamic LDS
    while (NW > 1 && merge_lds_bytes(NW, nh_max, D, Path::kHeads) > 65536) NW /= 2;
    const size_t lds = merge_lds_bytes(NW, nh_max, D, Path::kHeads);
    switch (NW) {
        case 1: hipLaunchKernelGGL((pa_decode_kernel<Path, D, 1, V2>), dim3(grid), dim3(64), lds, st, p); break;
        case 2: hipLaunchKernelGGL((pa_decode_kernel<Path, D, 2, V2>), dim3(grid), dim3(128), lds, st, p); break;
        case 4: hipLaunchKernelGGL((pa_decode_kernel<Path, D, 4, V2>), dim3(grid), dim3(256), lds, st, p); break;
        case 8: hipLaunchKernelGGL((pa_decode_kernel<Path, D, 8, V2>), dim3(grid), dim3(512), lds, st, p); break;
        default: return PA_ERR_INVALID_ARG;
    }
    return launch_status();
}

template <bool V2>
static int launch_decode(const DecodeParams& p, int head_size, bool fp8, int NW, int grid,
                         hipStream_t st) {
    const bool mfma = p.group >= 2;
    const int nh_max = mfma ? (p.group < 16 ? p.group : 16) : 1;
    if (fp8) {
        if (head_size == 128)
            return mfma ? launch_nw<MfmaPath8<128>, 128, V2>(NW, p, grid, nh_max, st)
                        : launch_nw<ValuPath8<128>, 128, V2>(NW, p, grid, nh_max, st);
        return mfma ? launch_nw<MfmaPath8<64>, 64, V2>(NW, p, grid, nh_max, st)
                    : launch_nw<ValuPath8<64>, 64, V2>(NW, p, grid, nh_max, st);
    }
    if (head_size == 128)
        return mfma ? launch_nw<MfmaPath<128>, 128, V2>(NW, p, grid, nh_max, st)
                    : launch_nw<ValuPath<128>, 128, V2>(NW, p, grid, nh_max, st);
    return mfma ? launch_nw<MfmaPath<64>, 64, V2>(NW, p, grid, nh_max, st)
                : launch_nw<ValuPath<64>, 64, V2>(NW, p, grid, nh_max, st);
}

static int check_decode_args(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* seq_lens, int num_seqs,
                             int num_heads, int num_kv_heads, int head_size, int block_size,
                             int max_blocks_per_seq, int num_blocks, float scale,
                             int kv_cache_dtype, float k_scale, float v_scale) {
    int rc = check_head_block(head_size, block_size);
    if (rc != PA_OK) return rc;
    rc = check_kv_dtype(kv_cache_dtype, k_scale, v_scale);
    if (rc != PA_OK) return rc;
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
        num_blocks <= 0)
        return PA_ERR_INVALID_ARG;
    if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !isfinite(scale)) return PA_ERR_INVALID_ARG;
    if (!q || !k_cache || !v_cache || !block_tables || !seq_lens) return PA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned4(block_tables) ||
        !aligned4(seq_lens))
        return PA_ERR_MISALIGNED;
    return PA_OK;
}

static DecodeParams make_params(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* seq_lens,
                                int num_seqs, int num_heads, int num_kv_heads,
                                int max_blocks_per_seq, int num_blocks, float scale,
                                int kv_cache_dtype, float k_scale, float v_scale) {
    DecodeParams p{};
    const bool fp8 = kv_cache_dtype == PA_KV_FP8_E4M3;
    if (fp8) scale *= k_scale;   // logits of the scaled keys: scale * k_scale * (q . code)
    p.v_scale = fp8 ? v_scale : 1.0f;
    p.q = static_cast<const f16*>(q);
    p.k_cache = static_cast<const char*>(k_cache);
    p.v_cache = static_cast<const char*>(v_cache);
    p.block_tables = block_tables;
    p.seq_lens = seq_lens;
    p.num_seqs = num_seqs;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = num_heads / num_kv_heads;
    p.head_chunks = p.group >= 2 ? (p.group + 15) / 16 : 1;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.num_blocks = num_blocks;
    p.scale = scale;
    p.scale_log2 = scale * kLog2e;
    p.max_num_partitions = 1;
    p.partition_size = 0;
    return p;
}

// Waves per workgroup.  Each wave keeps two K/V tiles in flight, so
// covering the loaded HBM latency (~1.2 us at ~6.5 TB/s, i.e. ~8 MB in
// flight) takes about 8 MiB / (2 tiles) waves; twice that many are asked for
// because unit sizes vary with the sequence lengths, and the waves of the
// longest unit set the critical path.  No more waves than a quarter of a
// unit's blocks.
static int pick_waves(long long units, long long blocks_per_unit, int head_size, int elem) {
    const long long tile_bytes = 2LL * kBlock * head_size * elem;   // K + V
    const long long target = (8LL << 20) / tile_bytes;
    int nw = 1;
    while (nw < 8 && units * nw < target && (long long)(nw * 2) * 4 <= blocks_per_unit) nw *= 2;
    return nw;
}

}  // namespace pa

using namespace pa;

extern "C" int pa_decode_v1(float* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens, int num_seqs,
                            int num_heads, int num_kv_heads, int head_size, int block_size,
                            int max_blocks_per_seq, int num_blocks, float scale,
                            int kv_cache_dtype, float k_scale, float v_scale, void* stream) {
    int rc = check_decode_args(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads,
                               num_kv_heads, head_size, block_size, max_blocks_per_seq, num_blocks,
                               scale, kv_cache_dtype, k_scale, v_scale);
    if (rc != PA_OK) return rc;
    if (!out) return PA_ERR_INVALID_ARG;
    if (!aligned16(out)) return PA_ERR_MISALIGNED;
    if (num_seqs == 0) return PA_OK;
    DecodeParams p = make_params(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads,
                                 num_kv_heads, max_blocks_per_seq, num_blocks, scale,
                                 kv_cache_dtype, k_scale, v_scale);
    p.out = out;
    const long long units = (long long)num_seqs * num_kv_heads * p.head_chunks;
    if (units > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
    const bool fp8 = kv_cache_dtype == PA_KV_FP8_E4M3;
    const int nw = PA_V1_WAVES ? PA_V1_WAVES
                               : pick_waves(units, max_blocks_per_seq, head_size, fp8 ? 1 : 2);
    return launch_decode<false>(p, head_size, fp8, nw, (int)units, as_stream(stream));
}

extern "C" int pa_v2_max_partitions(int max_seq_len, int partition_size) {
    if (max_seq_len <= 0 || partition_size <= 0) return -1;
    return (max_seq_len - 1) / partition_size + 1;
}

extern "C" int pa_decode_v2(float* tmp_out, float* exp_sums, float* max_logits, const void* q,
                            const void* k_cache, const void* v_cache, const int32_t* block_tables,
                            const int32_t* seq_lens, int num_seqs, int num_heads, int num_kv_heads,
                            int head_size, int block_size, int max_blocks_per_seq, int num_blocks,
                            int max_num_partitions, int partition_size, float scale,
                            int kv_cache_dtype, float k_scale, float v_scale, void* stream) {
    int rc = check_decode_args(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads,
                               num_kv_heads, head_size, block_size, max_blocks_per_seq, num_blocks,
                               scale, kv_cache_dtype, k_scale, v_scale);
    if (rc != PA_OK) return rc;
    if (!tmp_out || !exp_sums || !max_logits) return PA_ERR_INVALID_ARG;
    if (max_num_partitions <= 0 || partition_size <= 0 || partition_size % 16 != 0)
        return PA_ERR_INVALID_ARG;
    if (!aligned16(tmp_out) || !aligned4(exp_sums) || !aligned4(max_logits))
        return PA_ERR_MISALIGNED;
    if (num_seqs == 0) return PA_OK;
    DecodeParams p = make_params(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads,
                                 num_kv_heads, max_blocks_per_seq, num_blocks, scale,
                                 kv_cache_dtype, k_scale, v_scale);
    p.out = tmp_out;
    p.exp_sums = exp_sums;
    p.max_logits = max_logits;
    p.max_num_partitions = max_num_partitions;
    p.partition_size = partition_size;
    const long long units = (long long)num_seqs * num_kv_heads * p.head_chunks * max_num_partitions;
    if (units > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
    // a sequence has on average about half of max_num_partitions partitions
    const bool fp8 = kv_cache_dtype == PA_KV_FP8_E4M3;
    const int nw = PA_V2_WAVES ? PA_V2_WAVES
                               : pick_waves(units / 2, partition_size / 16, head_size, fp8 ? 1 : 2);
    return launch_decode<true>(p, head_size, fp8, nw, (int)units, as_stream(stream));
}
