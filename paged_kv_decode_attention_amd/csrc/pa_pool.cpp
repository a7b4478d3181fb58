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

struct pa_block_pool {
    struct Sequence {
        std::vector<int32_t> table;
        int64_t length = 0;
        bool live = false;
    };
    int num_blocks = 0;
    int block_size = 0;
    std::vector<int32_t> free_list;   // taken from the back
    std::vector<int32_t> refs;        // references per block, 0 = free
    std::vector<int32_t> fill;        // tokens each held block contains
    std::vector<Sequence> seqs;

    int32_t take() {
        const int32_t b = free_list.back();
        free_list.pop_back();
        refs[b] = 1;
        fill[b] = 0;
        return b;
    }
    void drop(int32_t b) {
        if (--refs[b] == 0) {
            fill[b] = 0;
            free_list.push_back(b);
        }
    }
    bool valid(int seq) const {
        return seq >= 0 && seq < (int)seqs.size() && seqs[seq].live;
    }
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
        p->fill.assign(num_blocks, 0);
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

    // Validate ids and count the blocks the appends take, applying the same
    // rules to a scratch copy of the reference counts they change (a shared
    // tail loses the reference of each sequence that copies it).  Tables that
    // grow get their room here, so that nothing below can fail half-way:
    // the batch is applied whole or not at all.
    int64_t need = 0;
    try {
        std::unordered_map<int, int> seen;
        std::unordered_map<int32_t, int32_t> tail_refs;
        for (int i = 0; i < n; ++i) {
            const int s = seqs[i];
            if (!pool->valid(s)) return invalid("unknown sequence %lld", s);
            if (!seen.emplace(s, i).second) return invalid("sequence %lld listed twice", s);
            std::vector<int32_t>& t = pool->seqs[s].table;
            if (t.empty() || pool->fill[t.back()] == BS) {
                t.reserve(t.size() + 1);
                ++need;
                continue;
            }
            auto it = tail_refs.find(t.back());
            int32_t& r = it != tail_refs.end()
                             ? it->second
                             : tail_refs.emplace(t.back(), pool->refs[t.back()]).first->second;
            if (r > 1) {
                --r;
                ++need;
            }
        }
    } catch (const std::bad_alloc&) {
        return pa::report_error(PA_ERR_INVALID_ARG, "out of host memory");
    }
    if (need > (int64_t)pool->free_list.size())
        return pa::report_error(PA_ERR_POOL_EXHAUSTED, "KV pool exhausted");
    for (int i = 0; i < n; ++i) {
        pa_block_pool::Sequence& q = pool->seqs[seqs[i]];
        if (q.table.empty() || pool->fill[q.table.back()] == BS) {
            q.table.push_back(pool->take());      // capacity reserved above
        } else if (pool->refs[q.table.back()] > 1) {
            const int32_t src = q.table.back();
            const int32_t dst = pool->take();
            pool->fill[dst] = pool->fill[src];
            --pool->refs[src];        // other sequences still hold it
            q.table.back() = dst;
            copy_pairs[2 * *num_copies] = src;
            copy_pairs[2 * *num_copies + 1] = dst;
            ++*num_copies;
        }
        const int32_t last = q.table.back();
        slots[i] = (int64_t)last * BS + pool->fill[last];
        ++pool->fill[last];
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
