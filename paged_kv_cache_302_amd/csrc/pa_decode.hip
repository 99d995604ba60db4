// Paged decode attention for gfx950 (MI355X): pa_decode_v1, pa_decode_v2 and
// pa_decode_v2_shared.
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
// pa_decode_v2_shared serves batches whose block tables share physical
// blocks (parallel samples, forks; page "vLLM 的 PagedAttention：KV cache
// 为什么要分页", §4.2): with G = 2, 4 or 8 one workgroup takes an aligned set of 16/G
// sequences for one (partition, KV head), and the members that read the same
// blocks over the partition are walked once (the set kernel below).
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

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "pa_device.h"
#include "pa_host.h"

#include "pa_paths.h"

#ifndef PA_V2_WAVES
#define PA_V2_WAVES 0         // waves per v2 workgroup (0 = heuristic)
#endif
#ifndef PA_V1_WAVES
#define PA_V1_WAVES 0         // waves per v1 workgroup (0 = heuristic)
#endif
#ifndef PA_SET_WAVES
#define PA_SET_WAVES 2        // waves per set-kernel workgroup: 1, 2 or 4 teams of PA_SET_SPLIT (0 = no set kernel)
#endif
#ifndef PA_SET_SPLIT
#define PA_SET_SPLIT 2        // set kernel: waves per class (the split of a class's blocks)
#endif

namespace pa {

// Stores of the results.  The v2 statistics (max_logits, exp_sums) are
// plain cached stores: a 128-byte line of [S][P][H] is written in 16-byte
// pieces by the KV heads' units of one partition (as nontemporal stores
// they cost the decodes 0.5-3%).  Result rows are nontemporal stores when
// the grid is larger than the device holds at once (cached, the long-context
// decode's 28 MB of rows cost it 4%) and cached stores when the whole grid
// is resident (1-3% faster on the short decodes).
__device__ __forceinline__ void st_stat(float* p, float v) { *p = v; }
template <class T>
__device__ __forceinline__ void st_row(T* p, T v, bool cached) {
    if (cached) {
        *p = v;
    } else {
        // (the empty statements keep the compiler from hoisting or sinking
        // the two stores into one plain store, which drops the hint)
        asm volatile("" ::: "memory");
        st_stream(p, v);
        asm volatile("" ::: "memory");
    }
}

// --------------------------------------------------------------------------
// v2 unit order.  The existing partitions (p < ceil(L_s / PS), capped at
// max_num_partitions) are numbered largest first: every full partition in
// (sequence, partition) order, then each sequence's partly filled last
// partition by decreasing block count, ties in sequence order (when the
// whole grid fits on the device at once; otherwise (sequence, partition)
// order).
// Workgroups that run at the same time are spread round robin over the CUs
// (workgroup b lands on CU b mod #CUs), and a CU's units share its memory
// path; the kernel takes consecutive ranks in a snake over the CUs (forward,
// then backward inside each XCD), so the CUs that got one more full unit get
// the smallest tails and every CU ends up with about the same number of
// blocks.  With more than 64 blocks per partition the tails are not sorted.
// --------------------------------------------------------------------------
// MI355X places consecutive workgroups on its 8 XCDs in turn.
constexpr int kXcds = 8;

__device__ __forceinline__ int n_parts(int L, int PS, int Pmax) {
    if (L <= 0) return 0;
    const int n = (L - 1) / PS + 1;
    return n < Pmax ? n : Pmax;
}

struct SeqParts {
    int len;    // L_s (0 past the last sequence)
    int np;     // partitions enumerated
    int tail;   // blocks of the last partition when it is partly filled, else 0
};

__device__ __forceinline__ SeqParts seq_parts(const DecodeParams& p, int len, int PB, bool sorted) {
    SeqParts r;
    r.len = len;
    r.np = n_parts(r.len, p.partition_size, p.max_num_partitions);
    const int nb = r.len > 0 ? (r.len - 1) / kBlock + 1 : 0;
    const int last = nb - (r.np - 1) * PB;   // blocks of partition np - 1 (if not capped)
    const bool capped = r.len > 0 && (r.len - 1) / p.partition_size + 1 > r.np;
    r.tail = (sorted && r.np > 0 && !capped && last < PB) ? last : 0;
    return r;
}

// The lengths of kLenChunks x 64 consecutive sequences, requested together:
// lane l of chunk c holds sequence g0 + 64c + l (0 past the last sequence).
// Every lane loads (the index is clamped), so the requests go out in one
// round trip and no load waits under a branch.
#ifndef PA_LEN_CHUNKS
#define PA_LEN_CHUNKS 4
#endif
constexpr int kLenChunks = PA_LEN_CHUNKS;
constexpr int kLenGroup = 64 * kLenChunks;
struct Lens {
    int v[kLenChunks];
};

__device__ __forceinline__ Lens load_lens(const DecodeParams& p, int g0) {
    Lens r;
#pragma unroll
    for (int c = 0; c < kLenChunks; ++c) {
        const int sq = g0 + 64 * c + lane_id();
        const int v = p.seq_lens[min(sq, p.num_seqs - 1)];
        r.v[c] = sq < p.num_seqs ? v : 0;
    }
    return r;
}

// first: the lengths of the first kLenGroup sequences (load_lens(p, 0));
// hist: 64 ints of LDS that only this wave uses
__device__ bool find_partition(const DecodeParams& p, int r, bool sort_tails, int& s_out,
                               int& p_out, int& L_out, const Lens& first, int* hist) {
    const int lane = lane_id();
    const int PB = p.partition_size / kBlock;
    const bool sorted = sort_tails && PB <= 64;
    // 1. full partitions (every partition when the tails are not sorted)
    int base = 0;
    for (int g0 = 0; g0 < p.num_seqs; g0 += kLenGroup) {
        const Lens ls = g0 == 0 ? first : load_lens(p, g0);
#pragma unroll
        for (int c = 0; c < kLenChunks; ++c) {
            const int s0 = g0 + 64 * c;
            if (s0 >= p.num_seqs) break;
            const SeqParts q = seq_parts(p, ls.v[c], PB, sorted);
            const int nfull = q.np - (q.tail > 0 ? 1 : 0);
            int incl = nfull;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int t = __shfl_up(incl, off);
                if (lane >= off) incl += t;
            }
            const int total = __builtin_amdgcn_readlane(incl, 63);
            if (r < base + total) {
                const unsigned long long mask = __ballot(base + incl > r);
                const int first_lane = __ffsll((long long)mask) - 1;
                s_out = s0 + first_lane;
                p_out = r - base - __builtin_amdgcn_readlane(incl - nfull, first_lane);
                // the length came with the prefix sum: no second, dependent load
                L_out = __builtin_amdgcn_readlane(q.len, first_lane);
                return true;
            }
            base += total;
        }
    }
    if (!sorted) return false;
    // 2. tails: a histogram of the tail sizes in LDS (one atomic add per
    // sequence), read back as lane c = the number of tails of c blocks
    int j = r - base;
    hist[lane] = 0;
    for (int g0 = 0; g0 < p.num_seqs; g0 += kLenGroup) {
        const Lens ls = g0 == 0 ? first : load_lens(p, g0);
#pragma unroll
        for (int c = 0; c < kLenChunks; ++c) {
            if (g0 + 64 * c >= p.num_seqs) break;
            const SeqParts q = seq_parts(p, ls.v[c], PB, true);
            if (q.tail > 0)
                __hip_atomic_fetch_add(hist + q.tail, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        }
    }
    const int cnt = hist[lane];
    // tails of more than c blocks come before class c: a suffix sum over lanes
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_down(incl, off);
        if (lane + off < 64) incl += t;
    }
    const int above = incl - cnt;
    const unsigned long long hit = __ballot(lane >= 1 && lane < PB && j >= above && j < above + cnt);
    if (hit == 0) return false;
    const int cls = __ffsll((long long)hit) - 1;
    j -= __builtin_amdgcn_readlane(above, cls);
    // 3. the j-th sequence (in order) whose tail has cls blocks
    for (int g0 = 0; g0 < p.num_seqs; g0 += kLenGroup) {
        const Lens ls = g0 == 0 ? first : load_lens(p, g0);
#pragma unroll
        for (int c = 0; c < kLenChunks; ++c) {
            const int s0 = g0 + 64 * c;
            if (s0 >= p.num_seqs) break;
            const SeqParts q = seq_parts(p, ls.v[c], PB, true);
            const unsigned long long m = __ballot(q.tail == cls);
            const int pc = __popcll(m);
            if (j < pc) {
                const int below = __popcll(m & ((1ull << lane) - 1ull));
                const unsigned long long pick = __ballot(q.tail == cls && below == j);
                const int first_lane = __ffsll((long long)pick) - 1;
                s_out = s0 + first_lane;
                p_out = __builtin_amdgcn_readlane(q.np, first_lane) - 1;
                L_out = __builtin_amdgcn_readlane(q.len, first_lane);
                return true;
            }
            j -= pc;
        }
    }
    return false;
}

// --------------------------------------------------------------------------
// Shared partitions (v2, MFMA path, G = 2, 4 or 8, one wave per unit).  A
// score tile has 16 query rows and one KV group fills only G of them, so
// sequences are taken in aligned sets of M = 16 / G.  The set's first
// sequence (the leader) computes its partition for every member whose
// block-table entries over the partition, and whose token range in it, equal
// its own (forks and samples of one prompt read the same blocks): member m's
// heads sit in tile rows mG .. mG + G - 1, and those members' own units
// return at once.  A member that differs computes its partition alone, in
// its own rows of the tile.  Every row's arithmetic is independent of the
// other rows, so the results are bit for bit those of separate units.
// --------------------------------------------------------------------------
constexpr int kMaxMembers = 8;

// Tile row i of a unit whose rows start at sequence `lead`: head h0 + i % gsz
// of sequence lead + i / gsz, for i < M * gsz.  Every row loads a valid query
// row (indices clamped) so that no load sits under a branch; rows outside
// `live` are zeroed once the members are known.
template <class Path>
__device__ __forceinline__ void load_q_rows(typename Path::QRegs& qr, const DecodeParams& p,
                                            int lead, int h0, int gsz, int M) {
    const int i = lane_id() & 15;
    const int m = min(i / gsz, M - 1), j = i - (i / gsz) * gsz;
    const int sm = min(lead + m, p.num_seqs - 1);
    Path::load_q_row(qr, p.q + ((size_t)sm * p.num_heads + h0 + min(j, gsz - 1)) * Path::kD, true);
}

// --------------------------------------------------------------------------
// The kernel
// --------------------------------------------------------------------------
#ifndef PA_WAVES_PER_EU
#define PA_WAVES_PER_EU 0
#endif
// RING: the tiles of a one-wave unit go through a two-slot LDS ring instead
// of registers (MFMA paths; see the walk below)
template <class Path, int D, int NW, bool V2, bool RING = false>
__global__ __launch_bounds__(64 * NW)
#if PA_WAVES_PER_EU
__attribute__((amdgpu_waves_per_eu(PA_WAVES_PER_EU)))
#endif
void pa_decode_kernel(DecodeParams p) {
    extern __shared__ float lds[];
    __shared__ int s_hist[NW][64];   // v2 partition lookup, one row per wave
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, uniform
    const int kvhc_count = p.num_kv_heads * p.head_chunks;
    int u = blockIdx.x;
    bool sorted = false;   // v2: largest-first order with the snake over the CUs
    Lens lens0;            // v2: the first sequences' lengths, for the partition lookup
    if constexpr (V2) {
        lens0 = load_lens(p, 0);
        sorted = p.resident > 0;

        if (sorted) {
            // a backward round reverses the CUs inside each XCD (workgroups
            // alternate over the 8 XCDs), so a unit keeps its XCD and L2
            const int per = p.unit_period, k = u / per, c = u - k * per;
            const bool back = (k & 1) && per >= kXcds;   // period 1: plain order
            u = k * per + (back ? per - kXcds - (c & ~(kXcds - 1)) + (c & (kXcds - 1)) : c);
        } else if (p.num_seqs <= 64 && p.unit_period % (kXcds * kvhc_count) == 0) {
            // A larger grid runs in (sequence, partition) order.  If no two
            // neighbouring sequences share their first block, each run of
            // 8 x (KV heads) workgroups gives XCD x every KV head of partition
            // rank 8g + x: a partition's 16 KiB of rows and its statistics
            // line then come from one XCD (its L2 merges the eight units'
            // pieces of the line), while the eight XCDs still read
            // neighbouring blocks at once.  Units that share blocks keep the
            // plain order, where a KV head's units (and its shared blocks) stay
            // on one XCD.  The lengths loaded for the check serve the
            // partition lookup below.
            const int ls = min(lane_id(), p.num_seqs - 1);
            const int l0 = lens0.v[0];
            const int f0 = p.block_tables[(size_t)ls * p.max_blocks_per_seq];
            const int f1 = __shfl_down(f0, 1), l1 = __shfl_down(l0, 1);
            const bool shared =
                __ballot(lane_id() + 1 < p.num_seqs && f0 == f1 && l0 > 0 && l1 > 0) != 0;
            if (!shared) {
                const int gx = kXcds * kvhc_count;
                const int g = u / gx, rem = u - g * gx;
                u = (g * kXcds + rem % kXcds) * kvhc_count + rem / kXcds;
            }
        }
    }
    const int kvhc = u % kvhc_count;
    const int r_unit = u / kvhc_count;
    const int kvh = kvhc / p.head_chunks;
    const int hc = kvhc - kvh * p.head_chunks;
    const int h0 = kvh * p.group + hc * Path::kHeads;
    const int nh_left = p.group - hc * Path::kHeads;
    const int nh = nh_left < Path::kHeads ? nh_left : Path::kHeads;

    int s, part = 0, L;
    if constexpr (V2) {
#ifdef PA_SORT_ALWAYS
        sorted = true;
#endif
        if (!find_partition(p, r_unit, sorted, s, part, L, lens0, s_hist[w])) return;
    } else {
        s = r_unit;
        L = p.seq_lens[s];
    }
    // v1 out[S][H][D]; v2 tmp_out[S][P][H][D]: either way a sequence's heads
    // of the unit are consecutive rows, one contiguous run of memory (out_row
    // below maps the tile rows)

    // Shared partitions: M members per unit (1: the unit's own heads only).
    // Only KV groups that fill the 16 rows evenly (G = 2, 4, 8): with others
    // (G = 7: two members) the member check cost GQA-7B batches, which share
    // nothing, 2% and could at best halve the shared reads.
    int M = 1;
    if constexpr (V2 && Path::kHeads == 16) {
        if (p.group <= kMaxMembers && 16 % p.group == 0 && p.head_chunks == 1 &&
            p.partition_size <= 64 * kBlock)
            M = 16 / p.group;
    }
    const int lead = s - s % M;          // first sequence of the aligned set
    const int self = s - lead;
    const int gsz = M > 1 ? p.group : nh;   // tile rows per member
    const int nrows = M * gsz;

    // Everything that depends only on (s, first block) is requested before
    // the length is used: the query, the first two table windows (bounded by
    // the row, not by the length) and the load-policy check.  In v1 these go
    // out together with the length load, so the first tile waits on one
    // round trip instead of two or three.
    const int pb = V2 ? p.partition_size / kBlock : 0;
    const int blk_begin = V2 ? part * pb : 0;
    const int first = blk_begin + w;       // this wave's blocks: first + k*NW, k < n
    const int32_t* row = p.block_tables + (size_t)s * p.max_blocks_per_seq;
    const int mbps = p.max_blocks_per_seq;
    const int n_req = first < mbps ? (mbps - first + NW - 1) / NW : 1;
    int cur = table_window<NW>(row, first, n_req, 0, mbps);
    int nxt = table_window<NW>(row, first, n_req, 64, mbps);
#if PA_LOAD_POLICY == 1
    const NeighbourIds nbr = neighbour_ids(p, s, blk_begin);
#endif
    typename Path::QRegs qr;
    // every member's query rows (rows of members not computed here are
    // zeroed once the members are known)
    if constexpr (Path::kHeads == 16) load_q_rows<Path>(qr, p, lead, h0, gsz, M);
    else Path::load_q(qr, p, s, h0, nh);
    // the set's lengths (scalar loads) and every member's table entries over
    // the partition (lane j: entry blk_begin + j), requested together with
    // the rest, so the comparison below waits on no further round trip
    int mlen[kMaxMembers], mrow[kMaxMembers];
    if (M > 1) {
        const int bi = min(blk_begin + lane_id(), mbps - 1);
#pragma unroll
        for (int i = 0; i < kMaxMembers; ++i) {
            const int f = min(lead + min(i, M - 1), p.num_seqs - 1);
            mlen[i] = p.seq_lens[f];
            mrow[i] = p.block_tables[(size_t)f * mbps + bi];
        }
    }
    // keep the scheduler from placing a use (and so a wait) between the loads
    __builtin_amdgcn_sched_barrier(0);
#if PA_LOAD_POLICY == 1
    const bool cached = shared_unit(nbr);
#endif
    unsigned members = 1u;   // bit m: the rows of sequence lead + m are computed here
    if (M > 1) {
        const int PS = p.partition_size;
        auto fits = [&](int len) {   // the partition exists and the sequence is well formed
            return len > part * PS && (len - 1) / PS + 1 <= p.max_num_partitions &&
                   (len + kBlock - 1) / kBlock <= mbps;
        };
        // a member shares the leader's unit when its token range in the
        // partition and every table entry over it equal the leader's
        const int tend = min(mlen[0], (part + 1) * PS);
        const int nblk = (tend - part * PS + kBlock - 1) / kBlock;   // <= 64 blocks
        unsigned match = 0;
#pragma unroll
        for (int i = 0; i < kMaxMembers; ++i) {
            const bool ok = i < M && lead + i < p.num_seqs && fits(mlen[0]) && fits(mlen[i]) &&
                            min(mlen[i], (part + 1) * PS) == tend;
            const bool same = __ballot(lane_id() < nblk && mrow[i] != mrow[0]) == 0;
            match |= (ok && same) ? 1u << i : 0u;
        }
        if (self != 0 && ((match >> self) & 1u)) return;   // the leader computes it
        members = self == 0 ? (match | 1u) : 1u << self;
    }
    // rows of the tile this unit writes
    auto live = [&](int i) { return i < nrows && ((members >> (i / gsz)) & 1u); };
    if constexpr (Path::kHeads == 16) {
        const int i = lane_id() & 15;
        const bool keep = live(i);
#pragma unroll
        for (int c = 0; c < Path::KC; ++c) qr.q[c] = keep ? qr.q[c] : f16x8{};
    }

    // No branch on L until the first tile request, so the compiler keeps the
    // loads above where they are: an empty v1 sequence (L <= 0; v2 has no
    // partition for it) walks no block and writes zeros.
    const bool empty = !V2 && L <= 0;
    const int nb_seq = empty ? 0 : (L + kBlock - 1) / kBlock;
    bool bad = nb_seq > mbps;
    if constexpr (V2) bad = bad || (L - 1) / p.partition_size + 1 > p.max_num_partitions;

    // token / block range of this unit
    int tok_end = L, blk_end = nb_seq;
    if constexpr (V2) {
        blk_end = min(nb_seq, blk_begin + pb);
        tok_end = min(L, (part + 1) * p.partition_size);
    }
    if (bad) blk_end = blk_begin;  // read nothing

    typename Path::State st;
    Path::init(st);

    const int n = first < blk_end ? (blk_end - first + NW - 1) / NW : 0;
    constexpr int TB = D * kBlock * Path::kElem;           // bytes of one K or V tile
    const char* kbase = p.k_cache + (size_t)kvh * TB;
    const char* vbase = p.v_cache + (size_t)kvh * TB;
    const size_t blk_stride = (size_t)p.num_kv_heads * TB;
    const float sl2 = p.scale_log2;

    {
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
        // the pool marks the unit bad and reads block 0.  A wave with no
        // block (n == 0) makes one empty request and processes nothing.
        auto phys = [&](int kw, int j) {
            const int d = max(min(j, n - 1), 0) - kw;
            const int v = d < 64 ? __builtin_amdgcn_readlane(cur, d) : __builtin_amdgcn_readlane(nxt, d - 64);
            const bool ok = (unsigned)v < (unsigned)p.num_blocks;
            bad = bad || (!ok && n > 0);   // with no block the entry is not the unit's
            return ok ? v : 0;
        };
        auto tile_k = [&](int id) { return kbase + (size_t)id * blk_stride; };
        auto tile_v = [&](int id) { return vbase + (size_t)id * blk_stride; };
        auto valid = [&](int k) { return min(kBlock, tok_end - (first + k * NW) * kBlock); };
        auto live = [&](int j) { return j < n ? TB : 0; };
        auto walk = [&](auto nt_tag) {
            constexpr bool NTL = decltype(nt_tag)::value;
            // a ring of DP tiles: block k lives in t[k % DP], and block
            // k + DP - 1 is requested just before block k is processed
            constexpr int DP = Path::kDepth;
            static_assert(DP == 2 || DP == 4, "the ring must divide a 64-entry window");
            typename Path::Stage t[DP];
            auto step = [&](const typename Path::Stage& ts, int kk) {
                typename Path::Tile tt = Path::unstage(ts);
                Path::process(st, tt, qr, valid(kk), sl2);
            };
#pragma unroll
            for (int j = 0; j < DP - 1; ++j) {
                const int id = phys(0, j);
                Path::template load_stage<NTL>(t[j], tile_k(id), tile_v(id), live(j));
            }
            int k = 0;
            for (int kw = 0;; kw += 64) {
                const int pend = table_window<NW>(row, first, n, kw + 128, mbps);
                const int kend = min(n, kw + 64) & ~(DP - 1);   // whole rings; the rest is the tail
                for (; k < kend; k += DP) {
#pragma unroll
                    for (int j = 0; j < DP; ++j) {
                        const int id = phys(kw, k + j + DP - 1);
                        Path::template load_stage<NTL>(t[(j + DP - 1) % DP], tile_k(id), tile_v(id),
                                                       live(k + j + DP - 1));
                        step(t[j], k + j);
                    }
                }
                if (kw + 64 >= n) break;
                cur = nxt;
                nxt = pend;
            }
            // the last n - k < DP blocks, already requested into t[0 ..]
#pragma unroll
            for (int j = 0; j < DP - 1; ++j)
                if (k + j < n) step(t[j], k + j);
        };
        // The LDS ring (units of grids the device holds at once, where it
        // measured faster: fewer registers per wave; elsewhere the register
        // ring is faster).  Block k + 1 is requested into the other slot just
        // before block k is read out of its slot and processed.  The compiler
        // does not track when a load into LDS has landed, so the waits are
        // explicit: loads complete in issue order, so with block k + 1's
        // kSlotLoads loads issued, block k's have landed once at most that
        // many are outstanding; with no request after block k, all of them.
        // Block k's slot is refilled (with block k + 2) only after block k
        // has been read out and processed.
        auto walk_ring = [&](auto nt_tag) {
            if constexpr (RING) {
                constexpr bool NTL = decltype(nt_tag)::value;
                char* ring = reinterpret_cast<char*>(lds);
                auto slot = [&](int k) { return ring + (k & 1) * Path::kSlot; };
                if (n > 0) {
                    const int id = phys(0, 0);
                    Path::template load_lds<NTL>(slot(0), tile_k(id), tile_v(id));
                }
                for (int kw = 0;; kw += 64) {
                    const int pend = table_window<NW>(row, first, n, kw + 128, mbps);
                    const int kend = min(n, kw + 64);
                    for (int k = kw; k < kend; ++k) {
                        if (k + 1 < n) {
                            const int id = phys(kw, k + 1);
                            Path::template load_lds<NTL>(slot(k + 1), tile_k(id), tile_v(id));
                            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(Path::kSlotLoads) : "memory");
                        } else {
                            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                        }
                        typename Path::Tile t;
                        Path::read_lds(t, slot(k));
                        Path::process(st, t, qr, valid(k), sl2);
                    }
                    if (kw + 64 >= n) break;
                    cur = nxt;
                    nxt = pend;
                }
            }
        };
#if PA_LOAD_POLICY == 1
        if constexpr (RING) {
            if (cached) walk_ring(std::false_type{});
            else walk_ring(std::true_type{});
        } else {
            if (cached) walk(std::false_type{});   // cached loads
            else walk(std::true_type{});
        }
#else
        if constexpr (RING) walk_ring(std::integral_constant<bool, PA_LOAD_POLICY == 2>{});
        else walk(std::integral_constant<bool, PA_LOAD_POLICY == 2>{});
#endif
    }

    const float ltot = Path::wave_l(st);
    // tile row i -> output row of head h0 + i % gsz of sequence lead + i / gsz
    // (M == 1: row0 + i)
    auto out_row = [&](int i) {
        const size_t sq = (size_t)(lead + i / gsz);
        const size_t r = V2 ? (sq * p.max_num_partitions + part) * p.num_heads
                            : sq * p.num_heads;
        return r + h0 + i % gsz;
    };
    if constexpr (NW == 1) {
        // The unit's result (nh rows of D, one contiguous run) goes out as
        // whole 1 KiB-per-instruction stores: stage the rows in LDS (this
        // wave only, so program order orders the accesses), then each lane
        // writes 16 contiguous bytes.  Storing straight from the MFMA layout
        // would write every cache line in two halves from two instructions.
        const int HP = Path::kHeads;
        float* s_o = lds;                 // [nrows][D]
        float* s_m = lds + nrows * D;     // [HP]
        float* s_l = s_m + HP;            // [HP]
        if constexpr (Path::kHeads == 16) Path::stage(st, ltot, s_o, s_m, s_l, nrows, live(lane_id() & 15));
        else Path::stage(st, ltot, s_o, s_m, s_l, nrows);
        const f32x4* src = reinterpret_cast<const f32x4*>(s_o);
        for (unsigned mm = members; mm != 0u; mm &= mm - 1u) {   // the rows of each member
            const int m = __ffs(mm) - 1;
            const int e1 = (m + 1) * gsz * (D / 4);
            for (int e = m * gsz * (D / 4) + lane_id(); e < e1; e += 64) {
                const int i = (4 * e) / D;
                const float inv = empty ? 0.f : p.v_scale / s_l[i];
                f32x4 v = src[e] * inv;
                if (bad) v = f32x4{NAN, NAN, NAN, NAN};
                st_row(reinterpret_cast<f32x4*>(p.out + out_row(i) * D) + (e - i * (D / 4)), v, p.resident > 0);
            }
        }
        if constexpr (V2) {
            // lane l < nrows holds tile row l's max and total weight on both paths
            const int l = lane_id();
            if (l < nrows && live(l)) {
                st_stat(p.max_logits + out_row(l), bad ? NAN : st.m * p.scale);
                st_stat(p.exp_sums + out_row(l), bad ? NAN : ltot);
            }
        }
        return;
    } else {
        // merge the NW wave states through LDS (the tile rows of every member
        // computed here)
        const int HP = Path::kHeads;
        float* s_acc = lds;                              // [NW][nrows][D]
        float* s_m = lds + NW * nrows * D;               // [NW][HP]
        float* s_l = s_m + NW * HP;                      // [NW][HP]
        int* s_bad = reinterpret_cast<int*>(s_l + NW * HP);  // [NW]
        float* s_fin = reinterpret_cast<float*>(s_bad + NW);  // [2][16]: merged m, l
        if constexpr (Path::kHeads == 16)
            Path::stage(st, ltot, s_acc + w * nrows * D, s_m + w * HP, s_l + w * HP, nrows,
                        live(lane_id() & 15));
        else
            Path::stage(st, ltot, s_acc + w * nrows * D, s_m + w * HP, s_l + w * HP, nrows);
        if (lane_id() == 0) s_bad[w] = bad ? 1 : 0;
        __syncthreads();
        int any_bad = 0;
#pragma unroll
        for (int v = 0; v < NW; ++v) any_bad |= s_bad[v];
        for (int e = threadIdx.x; e < nrows * D; e += 64 * NW) {
            const int j = e / D, d = e - j * D;
            if (!live(j)) continue;   // a member that computes its rows in its own unit
            float M = -INFINITY;
#pragma unroll
            for (int v = 0; v < NW; ++v) M = fmaxf(M, s_m[v * HP + j]);
            float num = 0.f, den = 0.f;
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                const float f = exp2_fast((s_m[v * HP + j] - M) * sl2);
                num += s_acc[(v * nrows + j) * D + d] * f;
                den += s_l[v * HP + j] * f;
            }
            const float o = empty ? 0.f : num / den * p.v_scale;
            st_row(p.out + out_row(j) * D + d, any_bad ? NAN : o, p.resident > 0);
            if (V2 && d == 0) {
                s_fin[j] = M;
                s_fin[16 + j] = den;
            }
        }
        if constexpr (V2) {
            __syncthreads();
            const int t = threadIdx.x;
            if (t < nrows && live(t)) {
                st_stat(p.max_logits + out_row(t), any_bad ? NAN : s_fin[t] * p.scale);
                st_stat(p.exp_sums + out_row(t), any_bad ? NAN : s_fin[16 + t]);
            }
        }
    }
}

// --------------------------------------------------------------------------
// Set kernel (pa_decode_v2_shared; MFMA path, G = 2, 4 or 8, PS <= 1024).
// One workgroup per (aligned set of M = 16/G sequences, partition, KV head):
// a score tile has 16 query rows and one KV group fills G of them, so the
// set's M groups fill the tile.  The set's members fall into classes: the
// leader together with every member whose token range in the partition and
// table entries over it equal the leader's (samples and forks of one prompt
// read the same blocks), and every other member alone.  Each class is
// computed once, by a team of SF waves: wave s of the team takes the class's
// blocks s, s + SF, ..., every member of the class in its own G tile rows, and
// the last wave of the team to finish merges the SF states (in wave order)
// through LDS and writes the class's rows.  The NW / SF teams of a workgroup
// take the classes in turn; a team with no class returns at once.  Every
// member's rows are thus the same SF-way split walk over the same K/V values
// whether or not the member shares its blocks: the results are bit for bit
// equal to those of private copies.  A class's blocks come straight from the
// table entries loaded for the class check (lane j: entry j of the
// partition), so the walk needs no table window.
//
// Against one unit per sequence, a shared partition is walked by SF waves at
// once instead of by one, the members it serves cost no workgroup, and
// (sequence, partition) follows from the workgroup index with no search over
// the lengths; a workgroup whose partition exists for no member (a partition
// past every member's length) returns after the length loads.
// --------------------------------------------------------------------------
template <class Path, int D, int NW, int SF>
__global__ __launch_bounds__(64 * NW) void pa_decode_set_kernel(DecodeParams p) {
    static_assert(NW % SF == 0, "teams of SF waves");
    constexpr int kTeams = NW / SF;
    extern __shared__ float lds[];
    float* s_acc = lds;                                  // [SF][16][D]
    float* s_m = lds + SF * 16 * D;                      // [SF][16]
    float* s_l = s_m + SF * 16;                          // [SF][16]
    int* s_bad = reinterpret_cast<int*>(s_l + SF * 16);  // [SF][kMaxMembers]
    int* s_done = s_bad + SF * kMaxMembers;              // [kMaxMembers]: waves done, per class
    if (threadIdx.x < kMaxMembers) s_done[threadIdx.x] = 0;
    __syncthreads();   // before any wave can return

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int team = w / SF, sub = w - team * SF;
    const int lane = lane_id();
    const int KVH = p.num_kv_heads, P = p.max_num_partitions, PS = p.partition_size;
    const int G = p.group, M = 16 / G;
    const int u = blockIdx.x;
    const int kvh = u % KVH;
    const int r = u / KVH;
    const int set = r / P, part = r - set * P;
    const int lead = set * M;
    const int h0 = kvh * G;
    const int mbps = p.max_blocks_per_seq;
    const int pb = PS / kBlock, blk_begin = part * pb;

    // One round trip: the members' lengths (scalar loads), their table entries
    // over the partition (lane j: entry blk_begin + j, clamped to the row) and
    // the 16 query rows (tile row i: head h0 + i % G of sequence lead + i / G).
    int mlen[kMaxMembers], mrow[kMaxMembers];
    {
        const int bi = min(blk_begin + lane, mbps - 1);
#pragma unroll
        for (int i = 0; i < kMaxMembers; ++i) {
            const int f = min(lead + min(i, M - 1), p.num_seqs - 1);
            mlen[i] = p.seq_lens[f];
            mrow[i] = p.block_tables[(size_t)f * mbps + bi];
        }
    }
    typename Path::QRegs qr;
    load_q_rows<Path>(qr, p, lead, h0, G, M);
    __builtin_amdgcn_sched_barrier(0);

    auto fits = [&](int len) {   // the partition exists and the sequence is well formed
        return len > part * PS && (len - 1) / PS + 1 <= P && (len + kBlock - 1) / kBlock <= mbps;
    };
    // The leader's class: members with the leader's token range in the
    // partition and its table entries over it, the last one excepted (after a
    // fork, copy-on-write gives every sample its own copy of the partly filled
    // last block).  When a member's last block differs, each member's last
    // block is walked on its own, in the class's tile but folded into its own
    // rows only, after the shared blocks: the same steps as its private walk.
    unsigned exists = 0, match = 0;
    bool own_last = false;
    {
        const int tend = min(mlen[0], (part + 1) * PS);
        const int nblk = (tend - part * PS + kBlock - 1) / kBlock;   // <= 64 blocks
#pragma unroll
        for (int i = 0; i < kMaxMembers; ++i) {
            const bool in = i < M && lead + i < p.num_seqs;
            exists |= (in && mlen[i] > part * PS) ? 1u << i : 0u;
            const bool ok = in && fits(mlen[0]) && fits(mlen[i]) &&
                            min(mlen[i], (part + 1) * PS) == tend;
            const unsigned long long diff = __ballot(lane < nblk && mrow[i] != mrow[0]);
            const bool body = (diff & ~(1ull << (max(nblk, 1) - 1))) == 0;
            match |= (ok && body) ? 1u << i : 0u;
            own_last = own_last || (ok && body && diff != 0);
        }
    }

    constexpr int TB = D * kBlock * Path::kElem;   // bytes of one K or V tile
    const char* kbase = p.k_cache + (size_t)kvh * TB;
    const char* vbase = p.v_cache + (size_t)kvh * TB;
    const size_t blk_stride = (size_t)KVH * TB;
    const float sl2 = p.scale_log2;

    int k_cls = 0;   // classes so far; class k goes to team k % kTeams
    for (unsigned todo = exists; todo != 0u; ++k_cls) {
        const int c = __ffs(todo) - 1;
        const unsigned cls = (c == 0 && (match & 1u)) ? (match & todo) : 1u << c;
        todo &= ~cls;
        if (k_cls % kTeams != team) continue;
        int L = mlen[0], rowc = mrow[0];
#pragma unroll
        for (int i = 1; i < kMaxMembers; ++i) {
            L = c == i ? mlen[i] : L;
            rowc = c == i ? mrow[i] : rowc;
        }
        // blocks of the class's partition; a malformed sequence reads none
        const int nb_seq = (L + kBlock - 1) / kBlock;
        bool bad = nb_seq > mbps || (L - 1) / PS + 1 > P;
        const int blk_end = bad ? blk_begin : min(nb_seq, blk_begin + pb);
        const int tok_end = min(L, (part + 1) * PS);
        const int first = blk_begin + sub;
        // Members' own last blocks (leader's class only): the shared walk
        // stops before the last block, and the wave whose share holds it
        // walks every member's copy after its shared blocks.
        const bool split = own_last && c == 0 && cls != 1u && blk_end > blk_begin;
        const int shared_end = split ? blk_end - 1 : blk_end;
        const int n_sh = first < shared_end ? (shared_end - first + SF - 1) / SF : 0;
        const int j_last = blk_end - 1 - blk_begin;   // the last block's index in the partition
        const int n = n_sh + ((split && j_last % SF == sub) ? __popc(cls) : 0);
        const int last_valid = tok_end - (blk_end - 1) * kBlock;
        auto member_of = [&](int j) {   // member whose own last block is walk step j >= n_sh
            unsigned b = cls;
            for (int x = n_sh; x < j; ++x) b &= b - 1u;
            return __ffs(b) - 1;
        };
        // lane m: member m's own last block (static register indices only)
        int own_ids = 0;
        if (split) {
#pragma unroll
            for (int i = 0; i < kMaxMembers; ++i) {
                const int v = __builtin_amdgcn_readlane(mrow[i], j_last);
                own_ids = lane == i ? v : own_ids;
            }
        }
        // Cached loads when other sequences read these blocks too (the class
        // has several members, or another member's partition starts on the
        // same block); the rest is streamed.
        bool cached = __popc(cls) > 1;
        {
            const int b0 = __builtin_amdgcn_readfirstlane(rowc);
#pragma unroll
            for (int i = 0; i < kMaxMembers; ++i)
                cached = cached || (((exists >> i) & 1u) != 0u && i != c &&
                                    __builtin_amdgcn_readfirstlane(mrow[i]) == b0);
        }

        typename Path::State st;
        Path::init(st);
        // The walk: steps j < n_sh are the wave's shared blocks, the rest
        // (SPLIT only) the members' own last blocks, each folded into its
        // member's rows only.  An id outside the pool marks the class bad
        // (a member's own last block: that member) and reads block 0.
        unsigned bad_own = 0;
        auto walk = [&](auto nt_tag, auto split_tag) {
            constexpr bool NTL = decltype(nt_tag)::value;
            constexpr bool SPLIT = decltype(split_tag)::value;
            constexpr int DP = Path::kDepth;
            auto phys = [&](int j) {   // physical id of walk step j (clamped to the last)
                j = max(min(j, n - 1), 0);
                if (!SPLIT || j < n_sh) {
                    const int v = __builtin_amdgcn_readlane(rowc, sub + j * SF);
                    const bool ok = (unsigned)v < (unsigned)p.num_blocks;
                    bad = bad || (!ok && n > 0);
                    return ok ? v : 0;
                }
                const int m = member_of(j);
                const int v = __builtin_amdgcn_readlane(own_ids, m);
                const bool ok = (unsigned)v < (unsigned)p.num_blocks;
                bad_own |= ok ? 0u : 1u << m;
                return ok ? v : 0;
            };
            auto valid = [&](int k) {
                return (!SPLIT || k < n_sh) ? min(kBlock, tok_end - (first + k * SF) * kBlock) : last_valid;
            };
            auto live = [&](int j) { return j < n ? TB : 0; };
            auto step = [&](const typename Path::Stage& ts, int k) {
                typename Path::Tile t = Path::unstage(ts);
                if constexpr (SPLIT)   // a shared block: every head; an own last block: its member's
                    Path::template process<true>(st, t, qr, valid(k), sl2,
                                                 k < n_sh || (lane & 15) / G == member_of(k));
                else
                    Path::process(st, t, qr, valid(k), sl2);
            };
            typename Path::Stage t[DP];
#pragma unroll
            for (int j = 0; j < DP - 1; ++j) {
                const int id = phys(j);
                Path::template load_stage<NTL>(t[j], kbase + (size_t)id * blk_stride,
                                               vbase + (size_t)id * blk_stride, live(j));
            }
            int k = 0;
            for (; k < (n & ~(DP - 1)); k += DP) {
#pragma unroll
                for (int j = 0; j < DP; ++j) {
                    const int id = phys(k + j + DP - 1);
                    Path::template load_stage<NTL>(t[(j + DP - 1) % DP], kbase + (size_t)id * blk_stride,
                                                   vbase + (size_t)id * blk_stride, live(k + j + DP - 1));
                    step(t[j], k + j);
                }
            }
#pragma unroll
            for (int j = 0; j < DP - 1; ++j)
                if (k + j < n) step(t[j], k + j);
        };
        if (split) walk(std::false_type{}, std::true_type{});   // a shared class: cached loads
        else if (cached) walk(std::false_type{}, std::false_type{});
        else walk(std::true_type{}, std::false_type{});

        // The class's rows of this wave's state (tile row i belongs to member
        // i / G, so classes never share rows), then a count of the team's
        // waves done with the class: the LDS writes above are complete before
        // the add (release), and the last wave sees all of them (acquire).
        const float ltot = Path::wave_l(st);
        Path::stage(st, ltot, s_acc + sub * 16 * D, s_m + sub * 16, s_l + sub * 16, 16,
                    ((cls >> ((lane & 15) / G)) & 1u) != 0u);
        if (lane < kMaxMembers && ((cls >> lane) & 1u))
            s_bad[sub * kMaxMembers + lane] = (bad || ((bad_own >> lane) & 1u)) ? 1 : 0;
        int prev = 0;
        if (lane == 0)
            prev = __hip_atomic_fetch_add(s_done + c, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (__builtin_amdgcn_readfirstlane(prev) != SF - 1) continue;

        // merge the SF states of the class's rows, in wave order
        for (unsigned mm = cls; mm != 0u; mm &= mm - 1u) {
            const int m = __ffs(mm) - 1;
            int any_bad = 0;
#pragma unroll
            for (int v = 0; v < SF; ++v) any_bad |= s_bad[v * kMaxMembers + m];
            const size_t orow = ((size_t)(lead + m) * P + part) * p.num_heads + h0;
            for (int e = lane; e < G * (D / 4); e += 64) {
                const int j = e / (D / 4), d4 = e - j * (D / 4), i = m * G + j;
                float mx = -INFINITY;
#pragma unroll
                for (int v = 0; v < SF; ++v) mx = fmaxf(mx, s_m[v * 16 + i]);
                f32x4 num = {0.f, 0.f, 0.f, 0.f};
                float den = 0.f;
#pragma unroll
                for (int v = 0; v < SF; ++v) {
                    const float f = exp2_fast((s_m[v * 16 + i] - mx) * sl2);
                    num += *reinterpret_cast<const f32x4*>(s_acc + (v * 16 + i) * D + 4 * d4) * f;
                    den += s_l[v * 16 + i] * f;
                }
                f32x4 o = num / den * p.v_scale;
                if (any_bad) o = f32x4{NAN, NAN, NAN, NAN};
                st_row(reinterpret_cast<f32x4*>(p.out + (orow + j) * D) + d4, o, p.resident > 0);
                if (d4 == 0) {
                    st_stat(p.max_logits + orow + j, any_bad ? NAN : mx * p.scale);
                    st_stat(p.exp_sums + orow + j, any_bad ? NAN : den);
                }
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
static int launch_nw(int NW, const DecodeParams& p0, int grid, int nh_max, hipStream_t st) {
    const int nh_unit = nh_max;
    // v2 MFMA units whose sequences may share a unit (the kernel's condition)
    const bool members = p0.group <= kMaxMembers && 16 % p0.group == 0 && p0.head_chunks == 1 &&
                         p0.partition_size <= 64 * kBlock;
    size_t lds = 0;
    const void* fn = nullptr;
    auto setup = [&](int nw) {
        NW = nw;
        // keep the merge buffer within the default 64 KiB of dynamic LDS
        while (NW > 1 && merge_lds_bytes(NW, nh_unit, D, Path::kHeads) > 65536) NW /= 2;
        // a v2 MFMA unit may hold several sequences' heads: 16 tile rows
        nh_max = V2 && Path::kHeads == 16 && members ? 16 : nh_unit;
        lds = merge_lds_bytes(NW, nh_max, D, Path::kHeads);
        switch (NW) {
            case 1: fn = reinterpret_cast<const void*>(&pa_decode_kernel<Path, D, 1, V2>); break;
            case 2: fn = reinterpret_cast<const void*>(&pa_decode_kernel<Path, D, 2, V2>); break;
            case 4: fn = reinterpret_cast<const void*>(&pa_decode_kernel<Path, D, 4, V2>); break;
            case 8: fn = reinterpret_cast<const void*>(&pa_decode_kernel<Path, D, 8, V2>); break;
            default: fn = nullptr;
        }
    };
    setup(NW);
    if (!fn) return PA_ERR_INVALID_ARG;
    DecodeParams p = p0;
    {
        // Only when the whole grid is resident at once does the placement fix
        // each CU's share: then a v2 kernel takes the balanced unit order.
        // With more units the dispatcher balances the CUs itself as slots
        // free up, and the plain order keeps the units that share blocks
        // (forks, samples of one prompt) running together.  Residency also
        // picks the result rows' store policy (v1 and v2).  The occupancy of
        // each (wave count, LDS size) is asked for once.
        static std::atomic<long long> occ_cache[5];   // (lds << 8) | (workgroups per CU + 1)
        auto resident_slots = [&](const void* f, int threads, size_t lds_bytes, int slot) {
            long long c = occ_cache[slot].load(std::memory_order_relaxed);
            int per_cu = 0;
            if (c != 0 && (size_t)(c >> 8) == lds_bytes) {
                per_cu = (int)(c & 0xff) - 1;
            } else {
                if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, threads, lds_bytes) != hipSuccess) {
                    (void)hipGetLastError();
                    per_cu = 0;
                }
                if (per_cu >= 0 && per_cu < 255)
                    occ_cache[slot].store(((long long)lds_bytes << 8) | (per_cu + 1), std::memory_order_relaxed);
            }
            return (long long)per_cu * p.num_cus;
        };
        // one-wave fp16 MFMA units walk their tiles through the LDS ring when
        // the device holds the whole grid at once
        if constexpr (V2 && Path::kRing) {
            if (NW == 1) {
                const size_t lds_ring = std::max(lds, (size_t)2 * Path::kSlot);
                const void* fr = reinterpret_cast<const void*>(&pa_decode_kernel<Path, D, 1, true, true>);
                const long long res = resident_slots(fr, 64, lds_ring, 4);
                if (grid <= res) {
                    p.resident = (int)res;
                    hipLaunchKernelGGL((pa_decode_kernel<Path, D, 1, true, true>), dim3(grid), dim3(64),
                                       lds_ring, st, p);
                    return launch_status();
                }
            }
        }
        // Long contexts (64 or more partitions of at least 16 blocks) on a
        // grid larger than the device holds at once: four waves per MFMA unit
        // (interleaved A/B: long-context decode 569.3 -> 563.1 us cold, fp8
        // pools 304.4 -> 299.7).  Not for shorter batches, where it measured
        // -2% to +7%, nor on the VALU path; it also gives up the one-wave
        // units' member sharing, which batches that share blocks get from
        // pa_decode_v2_shared.
        if constexpr (V2 && Path::kHeads == 16 && PA_V2_WAVES == 0) {
            if (NW == 1 && p.partition_size >= 16 * kBlock && p.max_num_partitions >= 64 &&
                grid > resident_slots(fn, 64, lds, 0))
                setup(4);
        }
        const int slot = NW == 1 ? 0 : NW == 2 ? 1 : NW == 4 ? 2 : 3;
        const long long resident = resident_slots(fn, 64 * NW, lds, slot);
        p.resident = grid <= resident ? (int)resident : 0;
    }
    switch (NW) {
        case 1: hipLaunchKernelGGL((pa_decode_kernel<Path, D, 1, V2>), dim3(grid), dim3(64), lds, st, p); break;
        case 2: hipLaunchKernelGGL((pa_decode_kernel<Path, D, 2, V2>), dim3(grid), dim3(128), lds, st, p); break;
        case 4: hipLaunchKernelGGL((pa_decode_kernel<Path, D, 4, V2>), dim3(grid), dim3(256), lds, st, p); break;
        case 8: hipLaunchKernelGGL((pa_decode_kernel<Path, D, 8, V2>), dim3(grid), dim3(512), lds, st, p); break;
        default: return PA_ERR_INVALID_ARG;
    }
    return launch_status();
}

// The set kernel: NW waves per (set, partition, KV head) workgroup, in teams
// of SF waves per class.
template <class Path, int D>
static int launch_set(const DecodeParams& p, int NW, int grid, hipStream_t st) {
    constexpr int SF = PA_SET_SPLIT;
    const size_t lds = (size_t)SF * (16 * D + 2 * 16 + kMaxMembers) * sizeof(float) +
                       kMaxMembers * sizeof(int);
    switch (NW) {
        case SF: hipLaunchKernelGGL((pa_decode_set_kernel<Path, D, SF, SF>), dim3(grid), dim3(64 * SF), lds, st, p); break;
        case 2 * SF: hipLaunchKernelGGL((pa_decode_set_kernel<Path, D, 2 * SF, SF>), dim3(grid), dim3(128 * SF), lds, st, p); break;
        case 4 * SF: hipLaunchKernelGGL((pa_decode_set_kernel<Path, D, 4 * SF, SF>), dim3(grid), dim3(256 * SF), lds, st, p); break;
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

// Compute units of the device that runs `stream` (cached per device; 0 if
// it cannot be read).
static int compute_units(void* stream) {
    static std::atomic<int> cache[64];
    hipDevice_t dev = 0;
    if (hipStreamGetDevice(as_stream(stream), &dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    if (dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 0) {
        (void)hipGetLastError();
        n = 0;
    }
    if (n > 0) cache[dev].store(n, std::memory_order_relaxed);
    return n;
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
    p.num_cus = compute_units(stream);   // residency (the row stores' policy)
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

// pa_decode_v2 and pa_decode_v2_shared: the set kernel only for the latter.
static int decode_v2(bool sets, float* tmp_out, float* exp_sums, float* max_logits, const void* q,
                     const void* k_cache, const void* v_cache, const int32_t* block_tables,
                     const int32_t* seq_lens, int num_seqs, int num_heads, int num_kv_heads,
                     int head_size, int block_size, int max_blocks_per_seq, int num_blocks,
                     int max_num_partitions, int partition_size, float scale, int kv_cache_dtype,
                     float k_scale, float v_scale, void* stream) {
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
    const bool fp8 = kv_cache_dtype == PA_KV_FP8_E4M3;
    // Batches declared to share blocks, with GQA groups that fill a score
    // tile evenly, go to the set kernel: one workgroup per (set of 16/G
    // sequences, partition, KV head).
    if (sets && PA_SET_WAVES > 0 && p.group >= 2 && p.group <= kMaxMembers && 16 % p.group == 0 &&
        partition_size <= 64 * kBlock) {
        const int M = 16 / p.group;
        const long long sets_n = (num_seqs + M - 1) / M;
        const long long grid = sets_n * max_num_partitions * num_kv_heads;
        if (grid > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
        hipStream_t st = as_stream(stream);
        if (fp8)
            return head_size == 128 ? launch_set<MfmaPath8<128>, 128>(p, PA_SET_WAVES, (int)grid, st)
                                    : launch_set<MfmaPath8<64>, 64>(p, PA_SET_WAVES, (int)grid, st);
        return head_size == 128 ? launch_set<MfmaPath<128>, 128>(p, PA_SET_WAVES, (int)grid, st)
                                : launch_set<MfmaPath<64>, 64>(p, PA_SET_WAVES, (int)grid, st);
    }
    // the grid covers whole snake rounds; workgroups past the real units exit
    p.num_cus = compute_units(stream);
    p.unit_period = p.num_cus > 0 && p.num_cus % kXcds == 0 ? p.num_cus : 1;
    const long long units = (long long)num_seqs * num_kv_heads * p.head_chunks * max_num_partitions;
    const long long grid = (units + p.unit_period - 1) / p.unit_period * p.unit_period;
    if (grid > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
    // a sequence has on average about half of max_num_partitions partitions
    const int nw = PA_V2_WAVES ? PA_V2_WAVES
                               : pick_waves(units / 2, partition_size / 16, head_size, fp8 ? 1 : 2);
    return launch_decode<true>(p, head_size, fp8, nw, (int)grid, as_stream(stream));
}

extern "C" int pa_decode_v2(float* tmp_out, float* exp_sums, float* max_logits, const void* q,
                            const void* k_cache, const void* v_cache, const int32_t* block_tables,
                            const int32_t* seq_lens, int num_seqs, int num_heads, int num_kv_heads,
                            int head_size, int block_size, int max_blocks_per_seq, int num_blocks,
                            int max_num_partitions, int partition_size, float scale,
                            int kv_cache_dtype, float k_scale, float v_scale, void* stream) {
    return decode_v2(false, tmp_out, exp_sums, max_logits, q, k_cache, v_cache, block_tables, seq_lens,
                     num_seqs, num_heads, num_kv_heads, head_size, block_size, max_blocks_per_seq,
                     num_blocks, max_num_partitions, partition_size, scale, kv_cache_dtype, k_scale,
                     v_scale, stream);
}

extern "C" int pa_decode_v2_shared(float* tmp_out, float* exp_sums, float* max_logits, const void* q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, const int32_t* seq_lens, int num_seqs,
                                   int num_heads, int num_kv_heads, int head_size, int block_size,
                                   int max_blocks_per_seq, int num_blocks, int max_num_partitions,
                                   int partition_size, float scale, int kv_cache_dtype,
                                   float k_scale, float v_scale, void* stream) {
    return decode_v2(true, tmp_out, exp_sums, max_logits, q, k_cache, v_cache, block_tables, seq_lens,
                     num_seqs, num_heads, num_kv_heads, head_size, block_size, max_blocks_per_seq,
                     num_blocks, max_num_partitions, partition_size, scale, kv_cache_dtype, k_scale,
                     v_scale, stream);
}
