// Host block pool: fixed 16-token KV blocks handed out on demand from a FIFO free
// queue, per-sequence block tables, reference-counted sharing.
//
// What it follows: "vLLM ve Triton ile maliyet optimizasyonu", §03 Yöntem, steps 1-3
// (blocks, block table, a new block only when the last one is full) and the paragraph
// on sharing; "vLLM Nedir? PagedAttention ile Production LLM Serving", section
// "PagedAttention" (reference-counted shared blocks) and section "Bir istek motorun
// içinde" (allocate_slots in the scheduling step; blocks of finished requests go back
// to the free queue; a request is dropped and its blocks returned when the pool is
// short, so a refused allocation must change nothing).
//
// The free queue is a ring buffer over num_blocks entries (a block is either queued
// or referenced, never both, so the ring never overflows). Sequences live in a hash
// map keyed by the caller's 64-bit id.
#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "status.hpp"

namespace pkv {
std::string& last_error() {
    static thread_local std::string msg;
    return msg;
}
}  // namespace pkv

using pkv::fail;
using pkv::ok;

struct kv_pool {
    int64_t num_blocks = 0;
    int32_t num_layers = 0, num_kv_heads = 0, head_dim = 0, dtype = 0;
    // FIFO free queue as a ring: entries [head, head + count) mod num_blocks
    std::vector<int32_t> ring;
    int64_t head = 0, count = 0;
    std::vector<int32_t> ref;
    struct Seq {
        std::vector<int32_t> blocks;
        int64_t len = 0;
    };
    std::unordered_map<int64_t, Seq> seqs;
    int64_t alloc_failures = 0;

    int32_t pop_front() {
        int32_t b = ring[head];
        head = head + 1 == num_blocks ? 0 : head + 1;
        --count;
        return b;
    }
    void push_back(int32_t b) {
        int64_t tail = head + count;
        if (tail >= num_blocks) tail -= num_blocks;
        ring[tail] = b;
        ++count;
    }
    Seq* find(int64_t id) {
        auto it = seqs.find(id);
        return it == seqs.end() ? nullptr : &it->second;
    }
    const Seq* find(int64_t id) const {
        auto it = seqs.find(id);
        return it == seqs.end() ? nullptr : &it->second;
    }
    // blocks a sequence of length len needs
    static int64_t blocks_for(int64_t len) { return (len + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE; }
};

extern "C" {

const char* pkv_last_error(void) { return pkv::last_error().c_str(); }

int64_t kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim,
                           int32_t dtype) {
    int e = pkv::cache_elem_bytes(dtype);
    if (num_layers <= 0 || num_kv_heads <= 0 || head_dim <= 0 || e == 0) {
        fail(PKV_EINVAL, "kv_bytes_per_token: bad shape or dtype");
        return -1;
    }
    return int64_t(2) * num_layers * num_kv_heads * head_dim * e;
}

int kv_pool_create(int64_t num_blocks, int32_t block_size, int32_t num_layers,
                   int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                   const int32_t* free_order, kv_pool** out) {
    if (!out) return fail(PKV_EINVAL, "kv_pool_create: out is NULL");
    *out = nullptr;
    if (num_blocks <= 0 || num_blocks > INT32_MAX)
        return fail(PKV_EINVAL, "kv_pool_create: num_blocks %lld out of range",
                    (long long)num_blocks);
    if (block_size != PKV_BLOCK_SIZE)
        return fail(PKV_EINVAL, "kv_pool_create: block_size must be 16, got %d", block_size);
    if (num_layers <= 0 || num_kv_heads <= 0 || head_dim <= 0 || pkv::cache_elem_bytes(dtype) == 0)
        return fail(PKV_EINVAL, "kv_pool_create: bad model shape or dtype");
    if (head_dim % (16 / pkv::cache_elem_bytes(dtype)) != 0)
        return fail(PKV_EINVAL, "kv_pool_create: head_dim must be a multiple of %d",
                    16 / pkv::cache_elem_bytes(dtype));
    kv_pool* p = new (std::nothrow) kv_pool();
    if (!p) return fail(PKV_ENOMEM, "kv_pool_create: out of host memory");
    p->num_blocks = num_blocks;
    p->num_layers = num_layers;
    p->num_kv_heads = num_kv_heads;
    p->head_dim = head_dim;
    p->dtype = dtype;
    p->ring.resize(num_blocks);
    p->ref.assign(num_blocks, 0);
    if (free_order) {
        std::vector<char> seen(num_blocks, 0);
        for (int64_t i = 0; i < num_blocks; ++i) {
            int32_t b = free_order[i];
            if (b < 0 || b >= num_blocks || seen[b]) {
                delete p;
                return fail(PKV_EINVAL, "kv_pool_create: free_order is not a permutation");
            }
            seen[b] = 1;
            p->ring[i] = b;
        }
    } else {
        for (int64_t i = 0; i < num_blocks; ++i) p->ring[i] = int32_t(i);
    }
    p->head = 0;
    p->count = num_blocks;
    *out = p;
    return ok();
}

void kv_pool_destroy(kv_pool* pool) { delete pool; }

int64_t kv_pool_bytes_per_token(const kv_pool* pool) {
    if (!pool) {
        fail(PKV_EINVAL, "kv_pool_bytes_per_token: pool is NULL");
        return -1;
    }
    return kv_bytes_per_token(pool->num_layers, pool->num_kv_heads, pool->head_dim, pool->dtype);
}

int kv_pool_cache_shape(const kv_pool* pool, int64_t k_shape[5], int64_t v_shape[4]) {
    if (!pool || !k_shape || !v_shape) return fail(PKV_EINVAL, "kv_pool_cache_shape: NULL");
    int x = 16 / pkv::cache_elem_bytes(pool->dtype);
    k_shape[0] = pool->num_blocks;
    k_shape[1] = pool->num_kv_heads;
    k_shape[2] = pool->head_dim / x;
    k_shape[3] = PKV_BLOCK_SIZE;
    k_shape[4] = x;
    v_shape[0] = pool->num_blocks;
    v_shape[1] = pool->num_kv_heads;
    v_shape[2] = pool->head_dim;
    v_shape[3] = PKV_BLOCK_SIZE;
    return ok();
}

int kv_pool_add_seq(kv_pool* pool, int64_t seq_id) {
    if (!pool) return fail(PKV_EINVAL, "kv_pool_add_seq: pool is NULL");
    if (pool->find(seq_id)) return fail(PKV_EINVAL, "kv_pool_add_seq: sequence %lld exists",
                                        (long long)seq_id);
    pool->seqs.emplace(seq_id, kv_pool::Seq{});
    return ok();
}

int kv_pool_share_prefix(kv_pool* pool, int64_t seq_id, int64_t src_seq_id, int32_t n_tokens) {
    if (!pool) return fail(PKV_EINVAL, "kv_pool_share_prefix: pool is NULL");
    kv_pool::Seq* dst = pool->find(seq_id);
    const kv_pool::Seq* src = pool->find(src_seq_id);
    if (!dst || !src) return fail(PKV_ENOENT, "kv_pool_share_prefix: unknown sequence");
    if (dst->len != 0 || !dst->blocks.empty())
        return fail(PKV_EINVAL, "kv_pool_share_prefix: target sequence is not empty");
    if (n_tokens < 0 || n_tokens % PKV_BLOCK_SIZE != 0 || n_tokens > src->len)
        return fail(PKV_EINVAL,
                    "kv_pool_share_prefix: n_tokens must be a multiple of 16 within the source");
    if (seq_id == src_seq_id) return fail(PKV_EINVAL, "kv_pool_share_prefix: same sequence");
    int64_t nb = n_tokens / PKV_BLOCK_SIZE;
    dst->blocks.assign(src->blocks.begin(), src->blocks.begin() + nb);
    for (int32_t b : dst->blocks) ++pool->ref[b];
    dst->len = n_tokens;
    return ok();
}

static int append_one_seq(kv_pool* pool, kv_pool::Seq* s, int32_t n_tokens, int32_t* slots) {
    int64_t need = kv_pool::blocks_for(s->len + n_tokens) - int64_t(s->blocks.size());
    if (need > pool->count) {
        ++pool->alloc_failures;
        return fail(PKV_ENOMEM, "kv_pool_append: need %lld blocks, %lld free", (long long)need,
                    (long long)pool->count);
    }
    for (int64_t k = 0; k < need; ++k) {
        int32_t b = pool->pop_front();
        pool->ref[b] = 1;
        s->blocks.push_back(b);
    }
    for (int32_t k = 0; k < n_tokens; ++k) {
        int64_t pos = s->len + k;
        slots[k] = s->blocks[pos / PKV_BLOCK_SIZE] * PKV_BLOCK_SIZE + int32_t(pos % PKV_BLOCK_SIZE);
    }
    s->len += n_tokens;
    return PKV_OK;
}

int kv_pool_append(kv_pool* pool, int64_t seq_id, int32_t n_tokens, int32_t* slot_mapping_out) {
    if (!pool) return fail(PKV_EINVAL, "kv_pool_append: pool is NULL");
    if (n_tokens < 0) return fail(PKV_EINVAL, "kv_pool_append: negative n_tokens");
    if (n_tokens > 0 && !slot_mapping_out) return fail(PKV_EINVAL, "kv_pool_append: NULL output");
    kv_pool::Seq* s = pool->find(seq_id);
    if (!s) return fail(PKV_ENOENT, "kv_pool_append: unknown sequence %lld", (long long)seq_id);
    int64_t max_len = int64_t(pool->num_blocks) * PKV_BLOCK_SIZE;
    if (s->len + n_tokens > max_len) {
        ++pool->alloc_failures;
        return fail(PKV_ENOMEM, "kv_pool_append: sequence longer than the whole pool");
    }
    int rc = append_one_seq(pool, s, n_tokens, slot_mapping_out);
    return rc == PKV_OK ? ok() : rc;
}

int kv_pool_append_batch(kv_pool* pool, const int64_t* seq_ids, int32_t n,
                         int32_t* slot_mapping_out) {
    if (!pool) return fail(PKV_EINVAL, "kv_pool_append_batch: pool is NULL");
    if (n < 0) return fail(PKV_EINVAL, "kv_pool_append_batch: negative n");
    if (n == 0) return ok();
    if (!seq_ids || !slot_mapping_out) return fail(PKV_EINVAL, "kv_pool_append_batch: NULL");
    std::vector<kv_pool::Seq*> seqs(n);
    std::unordered_set<int64_t> seen;
    seen.reserve(size_t(n) * 2);
    int64_t need = 0;
    for (int32_t i = 0; i < n; ++i) {
        seqs[i] = pool->find(seq_ids[i]);
        if (!seqs[i]) return fail(PKV_ENOENT, "kv_pool_append_batch: unknown sequence %lld",
                                  (long long)seq_ids[i]);
        if (!seen.insert(seq_ids[i]).second)
            return fail(PKV_EINVAL, "kv_pool_append_batch: duplicate sequence %lld",
                        (long long)seq_ids[i]);
        need += kv_pool::blocks_for(seqs[i]->len + 1) - int64_t(seqs[i]->blocks.size());
    }
    if (need > pool->count) {
        ++pool->alloc_failures;
        return fail(PKV_ENOMEM, "kv_pool_append_batch: need %lld blocks, %lld free",
                    (long long)need, (long long)pool->count);
    }
    for (int32_t i = 0; i < n; ++i) append_one_seq(pool, seqs[i], 1, slot_mapping_out + i);
    return ok();
}

int kv_pool_free_seq(kv_pool* pool, int64_t seq_id) {
    if (!pool) return fail(PKV_EINVAL, "kv_pool_free_seq: pool is NULL");
    auto it = pool->seqs.find(seq_id);
    if (it == pool->seqs.end())
        return fail(PKV_ENOENT, "kv_pool_free_seq: unknown sequence %lld", (long long)seq_id);
    for (int32_t b : it->second.blocks)
        if (--pool->ref[b] == 0) pool->push_back(b);
    pool->seqs.erase(it);
    return ok();
}

int kv_pool_seq_len(const kv_pool* pool, int64_t seq_id, int64_t* len_out) {
    if (!pool || !len_out) return fail(PKV_EINVAL, "kv_pool_seq_len: NULL");
    const kv_pool::Seq* s = pool->find(seq_id);
    if (!s) return fail(PKV_ENOENT, "kv_pool_seq_len: unknown sequence %lld", (long long)seq_id);
    *len_out = s->len;
    return ok();
}

int kv_pool_seq_blocks(const kv_pool* pool, int64_t seq_id, int32_t* blocks_out,
                       int32_t capacity, int32_t* n_out) {
    if (!pool || !n_out) return fail(PKV_EINVAL, "kv_pool_seq_blocks: NULL");
    const kv_pool::Seq* s = pool->find(seq_id);
    if (!s) return fail(PKV_ENOENT, "kv_pool_seq_blocks: unknown sequence %lld",
                        (long long)seq_id);
    int64_t nb = int64_t(s->blocks.size());
    *n_out = int32_t(nb);
    if (nb > capacity || (nb > 0 && !blocks_out))
        return fail(PKV_EINVAL, "kv_pool_seq_blocks: capacity %d < %lld", capacity,
                    (long long)nb);
    if (nb) std::memcpy(blocks_out, s->blocks.data(), sizeof(int32_t) * size_t(nb));
    return ok();
}

int kv_pool_free_queue(const kv_pool* pool, int32_t* blocks_out, int64_t capacity,
                       int64_t* n_out) {
    if (!pool || !n_out) return fail(PKV_EINVAL, "kv_pool_free_queue: NULL");
    *n_out = pool->count;
    if (pool->count > capacity || (pool->count > 0 && !blocks_out))
        return fail(PKV_EINVAL, "kv_pool_free_queue: capacity too small");
    for (int64_t k = 0; k < pool->count; ++k) {
        int64_t idx = pool->head + k;
        if (idx >= pool->num_blocks) idx -= pool->num_blocks;
        blocks_out[k] = pool->ring[idx];
    }
    return ok();
}

int kv_pool_refcount(const kv_pool* pool, int64_t blk, int32_t* ref_out) {
    if (!pool || !ref_out) return fail(PKV_EINVAL, "kv_pool_refcount: NULL");
    if (blk < 0 || blk >= pool->num_blocks) return fail(PKV_EINVAL, "kv_pool_refcount: bad block");
    *ref_out = pool->ref[blk];
    return ok();
}

int kv_pool_build_tables(const kv_pool* pool, const int64_t* seq_ids, int32_t n,
                         int32_t max_blocks, int32_t* tables_out, int32_t* seq_lens_out) {
    if (!pool) return fail(PKV_EINVAL, "kv_pool_build_tables: pool is NULL");
    if (n < 0 || max_blocks <= 0) return fail(PKV_EINVAL, "kv_pool_build_tables: bad sizes");
    if (n == 0) return ok();
    if (!seq_ids || !tables_out || !seq_lens_out)
        return fail(PKV_EINVAL, "kv_pool_build_tables: NULL");
    for (int32_t i = 0; i < n; ++i) {
        const kv_pool::Seq* s = pool->find(seq_ids[i]);
        if (!s) return fail(PKV_ENOENT, "kv_pool_build_tables: unknown sequence %lld",
                            (long long)seq_ids[i]);
        int64_t nb = int64_t(s->blocks.size());
        if (nb > max_blocks)
            return fail(PKV_EINVAL, "kv_pool_build_tables: sequence %lld has %lld blocks > %d",
                        (long long)seq_ids[i], (long long)nb, max_blocks);
        if (s->len > INT32_MAX) return fail(PKV_EINVAL, "kv_pool_build_tables: length overflow");
        int32_t* row = tables_out + int64_t(i) * max_blocks;
        if (nb) std::memcpy(row, s->blocks.data(), sizeof(int32_t) * size_t(nb));
        std::fill(row + nb, row + max_blocks, -1);
        seq_lens_out[i] = int32_t(s->len);
    }
    return ok();
}

int kv_pool_stats(const kv_pool* pool, kv_pool_stats_t* out) {
    if (!pool || !out) return fail(PKV_EINVAL, "kv_pool_stats: NULL");
    int64_t used = 0, shared = 0;
    for (int32_t r : pool->ref) {
        used += r > 0;
        shared += r > 1;
    }
    out->total_blocks = pool->num_blocks;
    out->free_blocks = pool->count;
    out->used_blocks = used;
    out->shared_blocks = shared;
    out->alloc_failures = pool->alloc_failures;
    out->num_seqs = int64_t(pool->seqs.size());
    return ok();
}

}  // extern "C"

extern "C" const char* pkv_version(void) { return "pkv 0.1.0 gfx950"; }
