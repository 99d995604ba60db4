// Host-side block manager of the paged KV cache (page "vLLM 的
// PagedAttention：KV cache 为什么要分页", §4.1 logical -> physical blocks
// allocated as a sequence grows, §4.2 shared prefix blocks with reference
// counts and copy-on-write; page "KV Cache与PagedAttention内存管理", 分页机制:
// a pool of fixed-size blocks handed out on demand and returned on release).
//
// State: a free stack of block ids, one reference count per block, and per
// sequence its block table and token count.  Every operation first checks
// that it can complete (ids, free blocks, output room) and only then
// mutates, so a failed call changes nothing.  A decode step costs O(batch)
// plus one hash lookup per sequence; nothing here touches the GPU.
#include <stdint.h>

#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa_blocks.h"

namespace {

struct Sequence {
    std::vector<int32_t> table;   // logical block -> physical block
    int64_t num_tokens = 0;
};

}  // namespace

struct pa_block_manager {
    int num_blocks = 0;
    int block_size = 0;
    std::vector<int32_t> free_stack;   // top = back()
    std::vector<int32_t> refcount;
    std::unordered_map<int64_t, Sequence> seqs;

    int32_t take() {
        const int32_t b = free_stack.back();
        free_stack.pop_back();
        refcount[b] = 1;
        return b;
    }
    int64_t slot(const Sequence& s, int64_t t) const {
        return (int64_t)s.table[t / block_size] * block_size + t % block_size;
    }
};

extern "C" pa_block_manager* pa_bm_create(int num_blocks, int block_size) {
    if (num_blocks <= 0 || block_size <= 0) return nullptr;
    pa_block_manager* bm = new (std::nothrow) pa_block_manager;
    if (!bm) return nullptr;
    try {
        bm->num_blocks = num_blocks;
        bm->block_size = block_size;
        bm->refcount.assign(num_blocks, 0);
        bm->free_stack.resize(num_blocks);
        for (int i = 0; i < num_blocks; ++i) bm->free_stack[i] = num_blocks - 1 - i;
    } catch (...) {
        delete bm;
        return nullptr;
    }
    return bm;
}

extern "C" void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

extern "C" int pa_bm_add_sequence(pa_block_manager* bm, int64_t seq_id, int num_tokens,
                                  int64_t* slots_out) {
    if (!bm || num_tokens < 0 || bm->seqs.count(seq_id)) return PA_ERR_INVALID_ARG;
    const int64_t need = ((int64_t)num_tokens + bm->block_size - 1) / bm->block_size;
    if (need > (int64_t)bm->free_stack.size()) return PA_ERR_NO_SPACE;
    // host allocations first, so a failure leaves the manager as it was
    std::unordered_map<int64_t, Sequence>::iterator it;
    try {
        it = bm->seqs.emplace(seq_id, Sequence{}).first;
    } catch (...) {
        return PA_ERR_NO_SPACE;
    }
    try {
        it->second.table.reserve(need);
    } catch (...) {
        bm->seqs.erase(it);
        return PA_ERR_NO_SPACE;
    }
    Sequence& s = it->second;
    for (int64_t i = 0; i < need; ++i) s.table.push_back(bm->take());
    s.num_tokens = num_tokens;
    if (slots_out)
        for (int64_t t = 0; t < num_tokens; ++t) slots_out[t] = bm->slot(s, t);
    return PA_OK;
}

extern "C" int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
    if (!bm) return PA_ERR_INVALID_ARG;
    auto it = bm->seqs.find(parent);
    if (it == bm->seqs.end() || bm->seqs.count(child)) return PA_ERR_INVALID_ARG;
    const std::vector<int32_t>* table;
    try {
        Sequence c = it->second;
        table = &bm->seqs.emplace(child, std::move(c)).first->second.table;
    } catch (...) {
        return PA_ERR_NO_SPACE;
    }
    for (int32_t b : *table) ++bm->refcount[b];
    return PA_OK;
}

extern "C" int pa_bm_free_sequence(pa_block_manager* bm, int64_t seq_id) {
    if (!bm) return PA_ERR_INVALID_ARG;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
    for (int32_t b : it->second.table)
        if (--bm->refcount[b] == 0) bm->free_stack.push_back(b);
    bm->seqs.erase(it);
    return PA_OK;
}

extern "C" int pa_bm_append_slots(pa_block_manager* bm, const int64_t* seq_ids, int num_seqs,
                                  int64_t* slots_out, int32_t* copies_out, int max_copies,
                                  int* num_copies) {
    if (!bm || num_seqs < 0 || max_copies < 0 || !num_copies) return PA_ERR_INVALID_ARG;
    if (num_seqs > 0 && (!seq_ids || !slots_out)) return PA_ERR_INVALID_ARG;
    if (max_copies > 0 && !copies_out) return PA_ERR_INVALID_ARG;
    const int B = bm->block_size;
    std::vector<Sequence*> batch;
    int64_t need = 0, ncopy = 0;
    try {
        // dry run: resolve ids, reject repeats, count new blocks and copies
        batch.reserve(num_seqs);
        std::unordered_set<int64_t> seen;
        std::unordered_map<int32_t, int32_t> pending;   // block -> count after earlier writes
        for (int i = 0; i < num_seqs; ++i) {
            auto it = bm->seqs.find(seq_ids[i]);
            if (it == bm->seqs.end() || !seen.insert(seq_ids[i]).second) return PA_ERR_INVALID_ARG;
            Sequence& s = it->second;
            batch.push_back(&s);
            if (s.num_tokens % B == 0) {
                ++need;
                continue;
            }
            const int32_t last = s.table[s.num_tokens / B];
            auto p = pending.find(last);
            const int32_t rc = p == pending.end() ? bm->refcount[last] : p->second;
            if (rc > 1) {
                ++need;
                ++ncopy;
                pending[last] = rc - 1;
            }
        }
        if (ncopy > max_copies) return PA_ERR_INVALID_ARG;
        if (need > (int64_t)bm->free_stack.size()) return PA_ERR_NO_SPACE;
        for (Sequence* s : batch)            // room for the new table entries
            if (s->num_tokens % B == 0) s->table.reserve(s->table.size() + 1);
    } catch (...) {
        return PA_ERR_NO_SPACE;
    }
    // commit: cannot fail from here on
    int nc = 0;
    for (int i = 0; i < num_seqs; ++i) {
        Sequence& s = *batch[i];
        const int64_t L = s.num_tokens;
        if (L % B == 0) {
            s.table.push_back(bm->take());
        } else {
            int32_t& entry = s.table[L / B];
            if (bm->refcount[entry] > 1) {   // shared: copy, then write the copy
                const int32_t fresh = bm->take();
                --bm->refcount[entry];
                copies_out[2 * nc] = entry;
                copies_out[2 * nc + 1] = fresh;
                ++nc;
                entry = fresh;
            }
        }
        slots_out[i] = bm->slot(s, L);
        s.num_tokens = L + 1;
    }
    *num_copies = nc;
    return PA_OK;
}

extern "C" int pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seq_ids, int num_seqs,
                                  int32_t* tables_out, int width, int32_t pad,
                                  int32_t* seq_lens_out) {
    if (!bm || num_seqs < 0 || width <= 0) return PA_ERR_INVALID_ARG;
    if (num_seqs > 0 && (!seq_ids || !tables_out)) return PA_ERR_INVALID_ARG;
    for (int i = 0; i < num_seqs; ++i) {
        auto it = bm->seqs.find(seq_ids[i]);
        if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
        if ((int64_t)it->second.table.size() > width) return PA_ERR_NO_SPACE;
        if (it->second.num_tokens > INT32_MAX) return PA_ERR_NO_SPACE;
    }
    for (int i = 0; i < num_seqs; ++i) {
        const Sequence& s = bm->seqs.find(seq_ids[i])->second;
        int32_t* row = tables_out + (int64_t)i * width;
        const int n = (int)s.table.size();
        for (int j = 0; j < n; ++j) row[j] = s.table[j];
        for (int j = n; j < width; ++j) row[j] = pad;
        if (seq_lens_out) seq_lens_out[i] = (int32_t)s.num_tokens;
    }
    return PA_OK;
}

extern "C" int pa_bm_num_free_blocks(const pa_block_manager* bm) {
    return bm ? (int)bm->free_stack.size() : PA_ERR_INVALID_ARG;
}

extern "C" int pa_bm_num_sequences(const pa_block_manager* bm) {
    return bm ? (int)bm->seqs.size() : PA_ERR_INVALID_ARG;
}

extern "C" int pa_bm_seq_len(const pa_block_manager* bm, int64_t seq_id) {
    if (!bm) return PA_ERR_INVALID_ARG;
    auto it = bm->seqs.find(seq_id);
    return it == bm->seqs.end() ? -1 : (int)it->second.num_tokens;
}

extern "C" int pa_bm_refcount(const pa_block_manager* bm, int block) {
    if (!bm || block < 0 || block >= bm->num_blocks) return -1;
    return bm->refcount[block];
}
