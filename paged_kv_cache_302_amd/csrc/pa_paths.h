// Building blocks shared by the paged decode and prefill kernels (gfx950):
// the parameter block, tile loads, the block-table window, the per-unit load
// policy, and the per-block "paths" that score a 16-token K/V tile against up
// to 16 query rows and fold it into an online softmax (MFMA path for
// 16-column tiles, VALU path for a single query row; fp16 and fp8 E4M3
// pools).  The design notes of each piece sit with it below; the decode
// kernels' notes are in pa_decode.hip.
#pragma once

#include <math.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_host.h"

// Compile-time tuning knobs (defaults are the measured best on MI355X).
#ifndef PA_LOAD_POLICY
#define PA_LOAD_POLICY 1      // tile loads: 0 = cached, 1 = per unit (see load policy), 2 = nontemporal
#endif

// Tiles in flight per wave in the decode walk (2 or 4), for fp16 and fp8 pools.
#ifndef PA_DEPTH_F16
#define PA_DEPTH_F16 2
#endif
#ifndef PA_DEPTH_F8
#define PA_DEPTH_F8 2
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

// An LDS slot holding the K and V tiles of one block (TB bytes each, K at 0,
// V at TB, each in its pool layout), written by loads that go from global
// memory to LDS without passing through registers: lane l's 16 bytes of each
// 1 KiB piece land at 16 l.  The compiler does not track when such loads have
// landed; the caller waits on the load count.
template <bool NTL, int TB>
__device__ __forceinline__ void load_slot(char* slot, const char* kt, const char* vt) {
    const int l = lane_id();
#pragma unroll
    for (int c = 0; c < TB / 1024; ++c) {
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(kt + 16 * l + 1024 * c),
                                         (__attribute__((address_space(3))) void*)(slot + 1024 * c), 16, 0,
                                         NTL ? 2 : 0);
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(vt + 16 * l + 1024 * c),
                                         (__attribute__((address_space(3))) void*)(slot + TB + 1024 * c), 16,
                                         0, NTL ? 2 : 0);
    }
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
    int unit_period;      // v2: compute units the unit order snakes over (1 = plain order)
    int num_cus;          // compute units of the device (0 = unknown)
    int resident;         // >0 when the device holds the whole grid at once
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
// unconditional load with nothing to merge afterwards.  `n` only bounds what
// is loaded (lanes past it repeat an earlier entry) and may exceed the
// wave's real block count; the index never leaves the row [0, row_len).
// --------------------------------------------------------------------------
template <int NW>
__device__ __forceinline__ int table_window(const int32_t* row, int first, int n, int kbase,
                                            int row_len) {
    const int k = max(min(kbase + lane_id(), n - 1), 0);
    return row[min(first + k * NW, row_len - 1)];
}

// 4 x 4 transpose of dwords across the four 16-lane rows of a wave: lane
// (i, g) ends with a[j] = what lane (i, j) held in a[g] (v_permlane32_swap
// exchanges rows 0-1 with 2-3, then v_permlane16_swap row 0 with 1 and 2
// with 3).
__device__ __forceinline__ void lane_transpose4(uint32_t (&a)[4]) {
    const auto x0 = __builtin_amdgcn_permlane32_swap(a[0], a[2], false, false);
    const auto x1 = __builtin_amdgcn_permlane32_swap(a[1], a[3], false, false);
    const auto y0 = __builtin_amdgcn_permlane16_swap(x0[0], x1[0], false, false);
    const auto y1 = __builtin_amdgcn_permlane16_swap(x0[1], x1[1], false, false);
    a[0] = y0[0];
    a[1] = y0[1];
    a[2] = y1[0];
    a[3] = y1[1];
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
    static constexpr int kD = D;
    static constexpr int kDepth = PA_DEPTH_F16;

    struct Tile {
        f16x8 k[KC];   // lane (g,i): K[t=i][d = 32c + 8g .. +7]
        f16x4 v[NT];   // lane (g,i): V[d = 16nt + i][t = 4g .. 4g+3]
    };
    // MFMA A operands of score step c and PV step nt (fp16 tiles are used as loaded)
    __device__ __forceinline__ static f16x8 a_k(const Tile& t, int c) { return t.k[c]; }
    __device__ __forceinline__ static f16x4 a_v(const Tile& t, int nt) { return t.v[nt]; }
    // V elements of tokens >= nvalid set to 0 (unused slots may hold NaN)
    __device__ __forceinline__ static void mask_v(Tile& t, int nvalid) {
        const int g = lane_id() >> 4;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (4 * g + r >= nvalid) t.v[nt][r] = (f16)0.f;
    }
    struct State {
        f32x4 acc[NT]; // lane (g,i): O^T[d = 16nt + 4g + r][h = i]
        float m;       // running max of raw dot products of head i
        float l;       // sum of weights over this lane's tokens 4g..4g+3
    };
    struct QRegs {
        f16x8 q[KC];   // lane (g,i): Q[h = i][d = 32c + 8g .. +7]
    };

    // column i of the tile = the query row `row` of lane (g, i), zeros if !ok
    __device__ static void load_q_row(QRegs& qr, const f16* row, bool ok) {
        const int g = lane_id() >> 4;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            f16x8 z = {};
            qr.q[c] = ok ? *reinterpret_cast<const f16x8*>(row + 32 * c + 8 * g) : z;
        }
    }
    // Rows past the unit's heads load the last real row and are zeroed
    // afterwards, so the loads are not under a branch and go out at once.
    __device__ static void load_q(QRegs& qr, const DecodeParams& p, int s, int h0, int nh) {
        const int i = lane_id() & 15;
        load_q_row(qr, p.q + ((size_t)s * p.num_heads + h0 + min(i, nh - 1)) * D, true);
        const f16x8 z = {};
#pragma unroll
        for (int c = 0; c < KC; ++c) qr.q[c] = i < nh ? qr.q[c] : z;
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

    // tiles are used as loaded (16-byte V rows with a quad-word transpose
    // across lanes, as the fp8 path does, measured slower for fp16 tiles)
    using Stage = Tile;
    template <bool NTL>
    __device__ __forceinline__ static void load_stage(Stage& t, const char* kt, const char* vt, int bytes) {
        load<NTL>(t, kt, vt, bytes);
    }
    __device__ __forceinline__ static Tile unstage(const Stage& s) { return s; }

    // LDS-staged tiles (load_slot): a slot's tiles read into the MFMA
    // operand registers, in the same layout as load(); with fp16 tiles the
    // ring takes only grids the device holds at once (measured faster there,
    // slower on larger grids of short units)
    static constexpr bool kRing = true;
    static constexpr int kTileBytes = D * kBlock * 2;
    static constexpr int kSlot = 2 * kTileBytes;
    static constexpr int kSlotLoads = kSlot / 1024;   // load instructions per slot
    template <bool NTL>
    __device__ __forceinline__ static void load_lds(char* slot, const char* kt, const char* vt) {
        load_slot<NTL, kTileBytes>(slot, kt, vt);
    }
    __device__ __forceinline__ static void read_lds(Tile& t, const char* slot) {
        const int l = lane_id(), i = l & 15, g = l >> 4;
#pragma unroll
        for (int c = 0; c < KC; ++c) t.k[c] = *reinterpret_cast<const f16x8*>(slot + 16 * (l + 64 * c));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            t.v[nt] = *reinterpret_cast<const f16x4*>(slot + kTileBytes + 8 * (4 * i + g + 64 * nt));
    }

    // nvalid: tokens of the block inside the sequence (the rest is never
    // read), masked to -inf before the softmax.  With ROWS, only the heads
    // whose lanes pass `keep` take the block in (the others' state is left
    // exactly as it was; the kept heads get the same arithmetic as without).
    template <bool ROWS = false>
    __device__ __forceinline__ static void process(State& st, Tile& t, const QRegs& qr,
                                                   int nvalid, float sl2, bool keep = true) {
        const int l = lane_id(), g = l >> 4;
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KC; ++c)
            s = __builtin_amdgcn_mfma_f32_16x16x32_f16(t.k[c], qr.q[c], s, 0, 0, 0);
        if (nvalid < kBlock) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (4 * g + r >= nvalid) s[r] = -INFINITY;
        }
        if (nvalid < kBlock) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (4 * g + r >= nvalid) t.v[nt][r] = (f16)0.f;
        }
        float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        bm = col4_max(bm);
        float mn = fmaxf(st.m, bm);
        float corr = exp2_fast((st.m - mn) * sl2);
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = exp2_fast((s[r] - mn) * sl2);
        if constexpr (ROWS) {
            mn = keep ? mn : st.m;
            corr = keep ? corr : 1.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) pr[r] = keep ? pr[r] : 0.f;
        }
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

    // Stage the wave's state for the cross-wave merge: acc[h][d] unnormalised
    // (rows i < nh whose lanes pass `live`).
    __device__ static void stage(const State& st, float ltot, float* s_acc, float* s_m,
                                 float* s_l, int nh, bool live = true) {
        const int l = lane_id(), i = l & 15, g = l >> 4;
        if (i >= nh || !live) return;
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
    static constexpr int kDepth = PA_DEPTH_F16;
    static constexpr bool kRing = false;

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

    // tiles are used as loaded
    using Stage = Tile;
    template <bool NTL>
    __device__ __forceinline__ static void load_stage(Stage& t, const char* kt, const char* vt, int bytes) {
        load<NTL>(t, kt, vt, bytes);
    }
    __device__ __forceinline__ static Tile unstage(const Stage& s) { return s; }

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
    static constexpr int kDepth = PA_DEPTH_F8;

    struct Tile {
        u32x4 k[KR];    // lane (g,i): K codes of token i, dims 16(g + 4r) .. +15
        uint32_t v[NT]; // lane (g,i): V codes of dim 16nt + i, tokens 4g .. 4g+3
    };
    __device__ __forceinline__ static f16x8 a_k(const Tile& t, int c) {
        const uint32_t w0 = t.k[c >> 1][2 * (c & 1)], w1 = t.k[c >> 1][2 * (c & 1) + 1];
        const f16x4 a0 = e4m3x4_to_f16x4(w0), a1 = e4m3x4_to_f16x4(w1);
        return f16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    }
    __device__ __forceinline__ static f16x4 a_v(const Tile& t, int nt) {
        return e4m3x4_to_f16x4(t.v[nt]);
    }
    __device__ __forceinline__ static void mask_v(Tile& t, int nvalid) {
        const int g = lane_id() >> 4;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) t.v[nt] = keep_tokens(t.v[nt], 4 * g, nvalid);
    }
    struct QRegs {
        f16x8 q[KC];    // lane (g,i): Q[h = i][d = 16(g + 4(c/2)) + 8(c%2) .. +7]
    };

    __device__ static void load_q_row(QRegs& qr, const f16* row, bool ok) {
        const int g = lane_id() >> 4;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            f16x8 z = {};
            const int d0 = 16 * (g + 4 * (c >> 1)) + 8 * (c & 1);
            qr.q[c] = ok ? *reinterpret_cast<const f16x8*>(row + d0) : z;
        }
    }
    // Rows past the unit's heads load the last real row and are zeroed
    // afterwards, so the loads are not under a branch and go out at once.
    __device__ static void load_q(QRegs& qr, const DecodeParams& p, int s, int h0, int nh) {
        const int i = lane_id() & 15;
        load_q_row(qr, p.q + ((size_t)s * p.num_heads + h0 + min(i, nh - 1)) * D, true);
        const f16x8 z = {};
#pragma unroll
        for (int c = 0; c < KC; ++c) qr.q[c] = i < nh ? qr.q[c] : z;
    }

    // Staged tiles: the V tile comes as whole 16-byte rows, lane (i, g)
    // taking rows 16 (kVR g + e) + i for e < kVR (two loads at D = 128
    // instead of eight 4-byte pieces), and is put into the Tile layout once
    // the loads have landed: after the dword transpose across the 16-lane
    // rows lane (i, g) holds dword g -- tokens 4g .. 4g+3 -- of the rows of
    // lanes (i, 0 .. 3).
    static constexpr int kVR = NT / 4;
    __device__ __forceinline__ static void v_from_rows(Tile& t, const u32x4 (&vr)[kVR]) {
#pragma unroll
        for (int e = 0; e < kVR; ++e) {
            uint32_t a[4] = {vr[e][0], vr[e][1], vr[e][2], vr[e][3]};
            lane_transpose4(a);
#pragma unroll
            for (int j = 0; j < 4; ++j) t.v[kVR * j + e] = a[j];
        }
    }
    struct Stage {
        u32x4 k[KR];
        u32x4 vr[kVR];
    };
    template <bool NTL>
    __device__ __forceinline__ static void load_stage(Stage& t, const char* kt, const char* vt, int bytes) {
        const int l = lane_id(), i = l & 15, g = l >> 4;
        const auto rk = tile_rsrc(kt, bytes), rv = tile_rsrc(vt, bytes);
#pragma unroll
        for (int r = 0; r < KR; ++r) t.k[r] = ld_tile<NTL, u32x4>(rk, 16 * (l + 64 * r));
#pragma unroll
        for (int e = 0; e < kVR; ++e) t.vr[e] = ld_tile<NTL, u32x4>(rv, 16 * (16 * (kVR * g + e) + i));
    }
    __device__ __forceinline__ static Tile unstage(const Stage& s) {
        Tile t;
#pragma unroll
        for (int r = 0; r < KR; ++r) t.k[r] = s.k[r];
        v_from_rows(t, s.vr);
        return t;
    }

    // No LDS ring for fp8 tiles: with the V rows fetched 16 bytes at a time
    // (load_stage) the register ring measured as fast or faster (long-context
    // decode 308.1 -> 305.0 us cold against the ring on every grid).
    static constexpr bool kRing = false;

    template <bool ROWS = false>
    __device__ __forceinline__ static void process(typename Base::State& st, Tile& t,
                                                   const QRegs& qr, int nvalid, float sl2,
                                                   bool keep = true) {
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
        }
        if (nvalid < kBlock) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) t.v[nt] = keep_tokens(t.v[nt], 4 * g, nvalid);
        }
        float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        bm = col4_max(bm);
        float mn = fmaxf(st.m, bm);
        float corr = exp2_fast((st.m - mn) * sl2);
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = exp2_fast((s[r] - mn) * sl2);
        if constexpr (ROWS) {   // as in the fp16 path
            mn = keep ? mn : st.m;
            corr = keep ? corr : 1.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) pr[r] = keep ? pr[r] : 0.f;
        }
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
    static constexpr int kDepth = PA_DEPTH_F8;
    static constexpr bool kRing = false;

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

    // tiles are used as loaded
    using Stage = Tile;
    template <bool NTL>
    __device__ __forceinline__ static void load_stage(Stage& t, const char* kt, const char* vt, int bytes) {
        load<NTL>(t, kt, vt, bytes);
    }
    __device__ __forceinline__ static Tile unstage(const Stage& s) { return s; }

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
// The check is split in two so that its loads can be issued together with
// the unit's other first loads and its answer taken only when needed.
struct NeighbourIds {
    int b0, bp, bn;   // the unit's first block id and the neighbours' entries there
    int lp, ln;       // the neighbours' lengths
    int blk;
    bool has_p, has_n;
};

__device__ __forceinline__ NeighbourIds neighbour_ids(const DecodeParams& p, int s, int blk) {
    const int32_t* bt = p.block_tables;
    const size_t w = (size_t)p.max_blocks_per_seq;
    NeighbourIds r;
    r.blk = min(blk, p.max_blocks_per_seq - 1);
    r.has_p = s > 0;
    r.has_n = s + 1 < p.num_seqs;
    const int sp = r.has_p ? s - 1 : s;
    const int sn = r.has_n ? s + 1 : s;
    // five independent loads (one round trip); neighbours' entries past their
    // lengths are read but not used
    r.b0 = bt[(size_t)s * w + r.blk];
    r.bp = bt[(size_t)sp * w + r.blk];
    r.bn = bt[(size_t)sn * w + r.blk];
    r.lp = p.seq_lens[sp];
    r.ln = p.seq_lens[sn];
    return r;
}

__device__ __forceinline__ bool shared_unit(const NeighbourIds& r) {
    // bitwise, not short-circuit: no branch between the loads and their use
    const bool shared = (r.has_p & (r.blk * kBlock < r.lp) & (r.bp == r.b0)) |
                        (r.has_n & (r.blk * kBlock < r.ln) & (r.bn == r.b0));
    return __builtin_amdgcn_readfirstlane((int)shared) != 0;
}

// --------------------------------------------------------------------------
// Host side: argument checks and the parameter block shared by the decode
// and prefill entry points
// --------------------------------------------------------------------------
inline int check_decode_args(const void* q, const void* k_cache, const void* v_cache,
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

inline DecodeParams make_params(const void* q, const void* k_cache, const void* v_cache,
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
    p.unit_period = 1;
    p.num_cus = 0;
    p.resident = 0;
    p.num_blocks = num_blocks;
    p.scale = scale;
    p.scale_log2 = scale * kLog2e;
    p.max_num_partitions = 1;
    p.partition_size = 0;
    return p;
}

}  // namespace pa
