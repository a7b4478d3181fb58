// Host-side block pool with reference counts and copy-on-write of shared
// partial blocks ([vLLM-paging] "Copy-on-write 是共享的正确性边界" and its
// "最小分页与 COW 模拟"; [MiniPaged-Qwen] §9 "差异 3", §10.1).  It owns no
// device memory: it hands out block tables, token slots and the copy pairs
// that pa_copy_blocks executes.
#include <cstdio>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

// Token p of a sequence sits in block table[p / block_size] at offset
// p % block_size, so a sequence of length L names ceil(L / block_size) blocks
// and its last block holds L - (blocks - 1) * block_size tokens: the fill of
// a block follows from the lengths and is not stored.
struct pa_block_pool {
    struct Sequence {
        std::vector<int32_t> table;
        int64_t length = 0;
        bool live = false;
    };
    int num_blocks = 0;
    int block_size = 0;
    std::vector<int32_t> free_list;   // taken from the back
    std::vector<int32_t> refs;        // tables naming each block, 0 = free
    std::vector<Sequence> seqs;

    int32_t take() {
        const int32_t b = free_list.back();
        free_list.pop_back();
        refs[b] = 1;
        return b;
    }
    void drop(int32_t b) {
        if (--refs[b] == 0) free_list.push_back(b);
    }
    bool valid(int seq) const {
        return seq >= 0 && seq < (int)seqs.size() && seqs[seq].live;
    }
    // Offset the sequence's next token takes in its block; 0 opens a block.
    int next_offset(int seq) const { return (int)(seqs[seq].length % block_size); }
};

namespace {

int invalid(const char* fmt, long long v) {
    char buf[160];
    snprintf(buf, sizeof buf, fmt, v);
    return pa::report_error(PA_ERR_INVALID_ARG, buf);
}

int new_sequence(pa_block_pool* p) {
    try {
        p->seqs.emplace_back();
    } catch (const std::bad_alloc&) {
        return pa::report_error(PA_ERR_INVALID_ARG, "out of host memory");
    }
    p->seqs.back().live = true;
    return (int)p->seqs.size() - 1;
}

}  // namespace

extern "C" {

pa_block_pool* pa_pool_create(int num_blocks, int block_size) {
    if (num_blocks <= 0 || block_size <= 0) {
        pa::report_error(PA_ERR_INVALID_ARG, "pool sizes must be positive");
        return nullptr;
    }
    pa_block_pool* p = new (std::nothrow) pa_block_pool;
    if (!p) {
        pa::report_error(PA_ERR_INVALID_ARG, "out of host memory");
        return nullptr;
    }
    try {
        p->num_blocks = num_blocks;
        p->block_size = block_size;
        p->free_list.resize(num_blocks);
        for (int b = 0; b < num_blocks; ++b) p->free_list[b] = b;
        p->refs.assign(num_blocks, 0);
    } catch (const std::bad_alloc&) {
        delete p;
        pa::report_error(PA_ERR_INVALID_ARG, "out of host memory");
        return nullptr;
    }
    return p;
}

void pa_pool_destroy(pa_block_pool* pool) { delete pool; }

int pa_pool_add_sequence(pa_block_pool* pool) {
    if (!pool) return pa::report_error(PA_ERR_INVALID_ARG, "null pool");
    return new_sequence(pool);
}

int pa_pool_fork(pa_block_pool* pool, int seq) {
    if (!pool) return pa::report_error(PA_ERR_INVALID_ARG, "null pool");
    if (!pool->valid(seq)) return invalid("unknown sequence %lld", seq);
    std::vector<int32_t> table;
    try {
        table = pool->seqs[seq].table;
    } catch (const std::bad_alloc&) {
        return pa::report_error(PA_ERR_INVALID_ARG, "out of host memory");
    }
    const int id = new_sequence(pool);
    if (id < 0) return id;
    pa_block_pool::Sequence& child = pool->seqs[id];
    child.table.swap(table);
    child.length = pool->seqs[seq].length;   // seqs may have moved: index again
    for (int32_t b : child.table) ++pool->refs[b];
    return id;
}

int pa_pool_append(pa_block_pool* pool, const int* seqs, int n, int64_t* slots,
                   int32_t* copy_pairs, int* num_copies) {
    if (!pool) return pa::report_error(PA_ERR_INVALID_ARG, "null pool");
    if (n < 0) return invalid("negative count %lld", n);
    if (n > 0 && (!seqs || !slots || !copy_pairs || !num_copies))
        return pa::report_error(PA_ERR_INVALID_ARG, "null array");
    if (num_copies) *num_copies = 0;
    if (n == 0) return PA_OK;
    const int BS = pool->block_size;

    // Plan.  A token at offset 0 opens a fresh block.  A token at a later
    // offset goes into the sequence's last block, which it may write only
    // if no other table names it.  Taken in list order, the k-th listed
    // writer of a partial block that h tables name copies it while the
    // earlier writers' copies still leave other holders, i.e. unless
    // k == h: the block is written in place only by the last of its writers,
    // and only when every holder is listed.  So writers[b] (how many listed
    // sequences end in partial block b) settles every copy up front, and the
    // fresh blocks the batch takes are counted before anything changes: the
    // batch is applied whole or not at all.  Tables that open a block get
    // their room here, so that nothing below can fail.
    std::unordered_map<int32_t, int32_t> writers;
    int64_t fresh = 0;
    try {
        std::unordered_map<int, int> seen;
        for (int i = 0; i < n; ++i) {
            const int s = seqs[i];
            if (!pool->valid(s)) return invalid("unknown sequence %lld", s);
            if (!seen.emplace(s, i).second) return invalid("sequence %lld listed twice", s);
            std::vector<int32_t>& t = pool->seqs[s].table;
            if (pool->next_offset(s) == 0) {
                t.reserve(t.size() + 1);
                ++fresh;
            } else {
                ++writers[t.back()];
            }
        }
    } catch (const std::bad_alloc&) {
        return pa::report_error(PA_ERR_INVALID_ARG, "out of host memory");
    }
    for (const auto& w : writers)
        fresh += w.second == pool->refs[w.first] ? w.second - 1 : w.second;
    if (fresh > (int64_t)pool->free_list.size())
        return pa::report_error(PA_ERR_POOL_EXHAUSTED, "KV pool exhausted");

    // Apply, in list order (the order fresh blocks leave the free list).
    for (int i = 0; i < n; ++i) {
        const int s = seqs[i];
        pa_block_pool::Sequence& q = pool->seqs[s];
        const int off = pool->next_offset(s);
        if (off == 0) {
            q.table.push_back(pool->take());      // capacity reserved above
        } else {
            const int32_t held = q.table.back();
            int32_t& left = writers.find(held)->second;   // counted above
            const bool in_place = left == 1 && pool->refs[held] == 1;
            --left;
            if (!in_place) {
                const int32_t dst = pool->take();
                --pool->refs[held];               // other tables still name it
                q.table.back() = dst;
                copy_pairs[2 * *num_copies] = held;
                copy_pairs[2 * *num_copies + 1] = dst;
                ++*num_copies;
            }
        }
        slots[i] = (int64_t)q.table.back() * BS + off;
        ++q.length;
    }
    return PA_OK;
}

int pa_pool_release(pa_block_pool* pool, int seq) {
    if (!pool) return pa::report_error(PA_ERR_INVALID_ARG, "null pool");
    if (!pool->valid(seq)) return invalid("unknown sequence %lld", seq);
    pa_block_pool::Sequence& q = pool->seqs[seq];
    for (int32_t b : q.table) pool->drop(b);
    q.table.clear();
    q.table.shrink_to_fit();
    q.length = 0;
    q.live = false;
    return PA_OK;
}

int pa_pool_length(const pa_block_pool* pool, int seq) {
    if (!pool) return pa::report_error(PA_ERR_INVALID_ARG, "null pool");
    if (!pool->valid(seq)) return invalid("unknown sequence %lld", seq);
    return (int)pool->seqs[seq].length;
}

int pa_pool_table(const pa_block_pool* pool, int seq, int32_t* table, int capacity) {
    if (!pool) return pa::report_error(PA_ERR_INVALID_ARG, "null pool");
    if (!pool->valid(seq)) return invalid("unknown sequence %lld", seq);
    const std::vector<int32_t>& t = pool->seqs[seq].table;
    if (capacity > 0 && !table) return pa::report_error(PA_ERR_INVALID_ARG, "null table");
    const int n = (int)t.size();
    for (int j = 0; j < n && j < capacity; ++j) table[j] = t[j];
    return n;
}

int pa_pool_refcount(const pa_block_pool* pool, int block) {
    if (!pool) return pa::report_error(PA_ERR_INVALID_ARG, "null pool");
    if (block < 0 || block >= pool->num_blocks) return invalid("block %lld outside the pool", block);
    return pool->refs[block];
}

int pa_pool_free_blocks(const pa_block_pool* pool) {
    if (!pool) return pa::report_error(PA_ERR_INVALID_ARG, "null pool");
    return (int)pool->free_list.size();
}

}  // extern "C"
