// Host block pool: fixed-size KV blocks (8, 16 or 32 tokens, chosen when the pool is
// created) handed out on demand from a FIFO free queue, per-sequence block tables,
// reference-counted sharing.
//
// What it follows: "vLLM ve Triton ile maliyet optimizasyonu", §03 Yöntem, steps 1-3
// (blocks, block table, a new block only when the last one is full) and the paragraph
// on sharing; "vLLM Nedir? PagedAttention ile Production LLM Serving", section
// "PagedAttention" (reference-counted shared blocks) and section "Bir istek motorun
// içinde" (allocate_slots in the scheduling step; blocks of finished requests go back
// to the free queue; a request is dropped and its blocks returned when the pool is
// short, so a refused allocation must change nothing).
//
// Prefix caching and copy-on-write ("vLLM Nedir? ...", section "Prefix caching": full
// blocks are keyed by a chain of the previous block's key, the block's tokens
// and, for the first block, a salt; a request bringing the same chain references the
// cached block; "vLLM ve Triton ...", §03 on sharing: a shared block is copied when one
// of its users writes to it). Keys here: a 64-bit hash chain h_j = mix(h_{j-1}, tokens of
// block j) from h_{-1} = root(salt). A hit is checked against the block's own token
// ids and its parent's chain hash, so a false hit needs two different prefixes with one
// 64-bit chain hash. A block is keyed when it fills in a sequence whose token ids are all
// known; freed blocks keep their key in the free queue, which is the eviction order, and
// lose it when popped for a new use.
//
// The free queue is a doubly linked list over the block ids (a prefix hit takes a block
// out of its middle). Sequences live in a hash map keyed by the caller's 64-bit id.
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

namespace {
// splitmix64's output function (Steele, Lea, Flood, "Fast splittable pseudorandom number
// generators", 2014): a bijection of 64-bit words with full avalanche.
inline uint64_t mix64(uint64_t x) {
    x ^= x >> 30;
    x *= 0xbf58476d1ce4e5b9ull;
    x ^= x >> 27;
    x *= 0x94d049bb133111ebull;
    return x ^ (x >> 31);
}
inline uint64_t chain_root(uint64_t salt) { return mix64(salt ^ 0x9e3779b97f4a7c15ull); }
inline uint64_t chain_next(uint64_t parent, const int32_t* tok, int bs) {
    uint64_t h = parent;
    for (int k = 0; k < bs; ++k) h = mix64(h ^ uint64_t(uint32_t(tok[k])));
    return h;
}
}  // namespace

struct kv_pool {
    int64_t num_blocks = 0;
    int32_t bs = 16;                    // tokens per block: 8, 16 or 32
    int32_t num_layers = 0, num_kv_heads = 0, head_dim = 0, dtype = 0;
    // FIFO free queue as a doubly linked list over block ids (-1 ends)
    std::vector<int32_t> nxt, prv;
    std::vector<char> queued;
    int32_t fhead = -1, ftail = -1;
    int64_t count = 0;
    std::vector<int32_t> ref;
    // prefix cache: chain hash -> block; per block its key, parent hash and bs token ids
    std::unordered_map<uint64_t, int32_t> cache;
    std::vector<char> keyed;
    std::vector<uint64_t> key, key_parent;
    std::vector<int32_t> key_tokens;   // [num_blocks][bs]
    int64_t prefix_hits = 0;
    struct Seq {
        std::vector<int32_t> blocks;
        int64_t len = 0;
        uint64_t salt = 0;
        bool hashable = true;           // every token id known: full blocks get keys
        std::vector<uint64_t> chain;    // chain hash of each full block (hashable only)
        std::vector<int32_t> tail;      // token ids of the partly filled last block
    };
    std::unordered_map<int64_t, Seq> seqs;
    int64_t alloc_failures = 0;

    void unlink(int32_t b) {
        const int32_t p = prv[b], n = nxt[b];
        (p >= 0 ? nxt[p] : fhead) = n;
        (n >= 0 ? prv[n] : ftail) = p;
        prv[b] = nxt[b] = -1;
        queued[b] = 0;
        --count;
    }
    // a block for a new use: the front of the free queue, which loses its cache key
    int32_t pop_front() {
        const int32_t b = fhead;
        unlink(b);
        if (keyed[b]) {
            cache.erase(key[b]);
            keyed[b] = 0;
        }
        return b;
    }
    void push_back(int32_t b) {
        prv[b] = ftail;
        nxt[b] = -1;
        (ftail >= 0 ? nxt[ftail] : fhead) = b;
        ftail = b;
        queued[b] = 1;
        ++count;
    }
    // key block b (now full in s, as its block j) unless the key is taken already
    void register_full(Seq& s, int64_t j, const int32_t* tok) {
        const uint64_t parent = j == 0 ? chain_root(s.salt) : s.chain[size_t(j - 1)];
        const uint64_t h = chain_next(parent, tok, bs);
        s.chain.push_back(h);
        const int32_t b = s.blocks[size_t(j)];
        if (keyed[b] || cache.count(h)) return;
        cache.emplace(h, b);
        keyed[b] = 1;
        key[b] = h;
        key_parent[b] = parent;
        std::memcpy(&key_tokens[size_t(b) * bs], tok, sizeof(int32_t) * bs);
    }
    // the cached block for (parent hash, bs tokens), or -1
    int32_t lookup(uint64_t parent, const int32_t* tok, uint64_t* h_out) const {
        const uint64_t h = chain_next(parent, tok, bs);
        auto it = cache.find(h);
        if (it == cache.end()) return -1;
        const int32_t b = it->second;
        if (key_parent[b] != parent ||
            std::memcmp(&key_tokens[size_t(b) * bs], tok, sizeof(int32_t) * bs))
            return -1;
        *h_out = h;
        return b;
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
    int64_t blocks_for(int64_t len) const { return (len + bs - 1) / bs; }
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
    if (block_size != 8 && block_size != 16 && block_size != 32)
        return fail(PKV_EINVAL, "kv_pool_create: block_size must be 8, 16 or 32, got %d",
                    block_size);
    if (num_blocks * block_size > INT32_MAX)
        return fail(PKV_EINVAL, "kv_pool_create: %lld blocks of %d tokens overflow int32 slot ids",
                    (long long)num_blocks, block_size);
    if (num_layers <= 0 || num_kv_heads <= 0 || head_dim <= 0 || pkv::cache_elem_bytes(dtype) == 0)
        return fail(PKV_EINVAL, "kv_pool_create: bad model shape or dtype");
    if (head_dim % (16 / pkv::cache_elem_bytes(dtype)) != 0)
        return fail(PKV_EINVAL, "kv_pool_create: head_dim must be a multiple of %d",
                    16 / pkv::cache_elem_bytes(dtype));
    kv_pool* p = new (std::nothrow) kv_pool();
    if (!p) return fail(PKV_ENOMEM, "kv_pool_create: out of host memory");
    p->num_blocks = num_blocks;
    p->bs = block_size;
    p->num_layers = num_layers;
    p->num_kv_heads = num_kv_heads;
    p->head_dim = head_dim;
    p->dtype = dtype;
    p->nxt.assign(num_blocks, -1);
    p->prv.assign(num_blocks, -1);
    p->queued.assign(num_blocks, 0);
    p->ref.assign(num_blocks, 0);
    p->keyed.assign(num_blocks, 0);
    p->key.assign(num_blocks, 0);
    p->key_parent.assign(num_blocks, 0);
    p->key_tokens.assign(size_t(num_blocks) * block_size, 0);
    if (free_order) {
        std::vector<char> seen(num_blocks, 0);
        for (int64_t i = 0; i < num_blocks; ++i) {
            int32_t b = free_order[i];
            if (b < 0 || b >= num_blocks || seen[b]) {
                delete p;
                return fail(PKV_EINVAL, "kv_pool_create: free_order is not a permutation");
            }
            seen[b] = 1;
        }
        for (int64_t i = 0; i < num_blocks; ++i) p->push_back(free_order[i]);
    } else {
        for (int64_t i = 0; i < num_blocks; ++i) p->push_back(int32_t(i));
    }
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
    k_shape[3] = pool->bs;
    k_shape[4] = x;
    v_shape[0] = pool->num_blocks;
    v_shape[1] = pool->num_kv_heads;
    v_shape[2] = pool->head_dim;
    v_shape[3] = pool->bs;
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
    if (n_tokens < 0 || n_tokens % pool->bs != 0 || n_tokens > src->len)
        return fail(PKV_EINVAL, "kv_pool_share_prefix: n_tokens must be a multiple of the "
                                "block size (%d) within the source", pool->bs);
    if (seq_id == src_seq_id) return fail(PKV_EINVAL, "kv_pool_share_prefix: same sequence");
    int64_t nb = n_tokens / pool->bs;
    dst->blocks.assign(src->blocks.begin(), src->blocks.begin() + nb);
    for (int32_t b : dst->blocks) ++pool->ref[b];
    dst->len = n_tokens;
    dst->hashable = false;   // shared without token ids: its blocks get no keys
    return ok();
}

int kv_pool_add_seq_prefix(kv_pool* pool, int64_t seq_id, const int32_t* prompt,
                           int32_t n_prompt, uint64_t salt, int32_t* n_cached_out) {
    if (!pool || !n_cached_out) return fail(PKV_EINVAL, "kv_pool_add_seq_prefix: NULL");
    if (n_prompt < 0 || (n_prompt > 0 && !prompt))
        return fail(PKV_EINVAL, "kv_pool_add_seq_prefix: bad prompt");
    if (pool->find(seq_id))
        return fail(PKV_EINVAL, "kv_pool_add_seq_prefix: sequence %lld exists", (long long)seq_id);
    kv_pool::Seq s;
    s.salt = salt;
    uint64_t h = chain_root(salt);
    int64_t n = 0;
    while (n + pool->bs <= int64_t(n_prompt) - 1) {
        uint64_t hn = 0;
        const int32_t b = pool->lookup(h, prompt + n, &hn);
        if (b < 0) break;
        if (pool->queued[b]) pool->unlink(b);
        ++pool->ref[b];
        s.blocks.push_back(b);
        s.chain.push_back(hn);
        h = hn;
        n += pool->bs;
    }
    pool->prefix_hits += int64_t(s.blocks.size());
    s.len = n;
    pool->seqs.emplace(seq_id, std::move(s));
    *n_cached_out = int32_t(n);
    return ok();
}

int kv_pool_fork(kv_pool* pool, int64_t parent_id, int64_t child_id) {
    if (!pool) return fail(PKV_EINVAL, "kv_pool_fork: pool is NULL");
    const kv_pool::Seq* p = pool->find(parent_id);
    if (!p) return fail(PKV_ENOENT, "kv_pool_fork: unknown sequence %lld", (long long)parent_id);
    if (pool->find(child_id))
        return fail(PKV_EINVAL, "kv_pool_fork: sequence %lld exists", (long long)child_id);
    kv_pool::Seq c = *p;
    for (int32_t b : c.blocks) ++pool->ref[b];
    pool->seqs.emplace(child_id, std::move(c));
    return ok();
}

// Does appending to s first need a copy of its last block (partly filled and shared)?
static bool needs_copy(const kv_pool* pool, const kv_pool::Seq* s) {
    return s->len % pool->bs != 0 && pool->ref[s->blocks.back()] > 1;
}

static int64_t blocks_needed(const kv_pool* pool, const kv_pool::Seq* s, int64_t n_tokens) {
    return pool->blocks_for(s->len + n_tokens) - int64_t(s->blocks.size()) +
           (n_tokens > 0 && needs_copy(pool, s) ? 1 : 0);
}

// Append n_tokens (token ids in `tokens`, or NULL when unknown) after the caller checked
// that the free queue holds blocks_needed(). copy[0..1] gets (old, new) when the shared
// last block was copied, else (-1, -1).
static void append_one_seq(kv_pool* pool, kv_pool::Seq* s, int32_t n_tokens,
                           const int32_t* tokens, int32_t* slots, int32_t* copy) {
    copy[0] = copy[1] = -1;
    if (n_tokens > 0 && needs_copy(pool, s)) {
        const int32_t nb = pool->pop_front();
        pool->ref[nb] = 1;
        copy[0] = s->blocks.back();
        copy[1] = nb;
        --pool->ref[copy[0]];   // still referenced by the others
        s->blocks.back() = nb;
    }
    const int32_t bs = pool->bs;
    while (int64_t(s->blocks.size()) * bs < s->len + n_tokens) {
        const int32_t b = pool->pop_front();
        pool->ref[b] = 1;
        s->blocks.push_back(b);
    }
    for (int32_t k = 0; k < n_tokens; ++k) {
        int64_t pos = s->len + k;
        slots[k] = s->blocks[pos / bs] * bs + int32_t(pos % bs);
    }
    if (!tokens) {
        s->hashable = false;
        s->tail.clear();
    } else if (s->hashable) {
        for (int32_t k = 0; k < n_tokens; ++k) {
            s->tail.push_back(tokens[k]);
            if (int32_t(s->tail.size()) == bs) {   // block (len + k) / bs is now full
                pool->register_full(*s, (s->len + k) / bs, s->tail.data());
                s->tail.clear();
            }
        }
    }
    s->len += n_tokens;
}

static int append_checked(kv_pool* pool, const char* who, kv_pool::Seq* s, int32_t n_tokens,
                          const int32_t* tokens, int32_t* slots, int32_t* copy) {
    if (!tokens && n_tokens > 0 && needs_copy(pool, s))
        return fail(PKV_EINVAL, "%s: the last block is shared and partly filled; "
                                "kv_pool_append_tokens copies it", who);
    int64_t need = blocks_needed(pool, s, n_tokens);
    if (need > pool->count) {
        ++pool->alloc_failures;
        return fail(PKV_ENOMEM, "%s: need %lld blocks, %lld free", who, (long long)need,
                    (long long)pool->count);
    }
    int32_t unused[2];
    append_one_seq(pool, s, n_tokens, tokens, slots, copy ? copy : unused);
    return PKV_OK;
}

int kv_pool_append(kv_pool* pool, int64_t seq_id, int32_t n_tokens, int32_t* slot_mapping_out) {
    if (!pool) return fail(PKV_EINVAL, "kv_pool_append: pool is NULL");
    if (n_tokens < 0) return fail(PKV_EINVAL, "kv_pool_append: negative n_tokens");
    if (n_tokens > 0 && !slot_mapping_out) return fail(PKV_EINVAL, "kv_pool_append: NULL output");
    kv_pool::Seq* s = pool->find(seq_id);
    if (!s) return fail(PKV_ENOENT, "kv_pool_append: unknown sequence %lld", (long long)seq_id);
    int64_t max_len = int64_t(pool->num_blocks) * pool->bs;
    if (s->len + n_tokens > max_len) {
        ++pool->alloc_failures;
        return fail(PKV_ENOMEM, "kv_pool_append: sequence longer than the whole pool");
    }
    int rc = append_checked(pool, "kv_pool_append", s, n_tokens, nullptr, slot_mapping_out, nullptr);
    return rc == PKV_OK ? ok() : rc;
}

int kv_pool_append_tokens(kv_pool* pool, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                          int32_t* slot_mapping_out, int32_t* copy_out) {
    if (!pool) return fail(PKV_EINVAL, "kv_pool_append_tokens: pool is NULL");
    if (n_tokens < 0) return fail(PKV_EINVAL, "kv_pool_append_tokens: negative n_tokens");
    if (!copy_out || (n_tokens > 0 && (!slot_mapping_out || !tokens)))
        return fail(PKV_EINVAL, "kv_pool_append_tokens: NULL argument");
    kv_pool::Seq* s = pool->find(seq_id);
    if (!s) return fail(PKV_ENOENT, "kv_pool_append_tokens: unknown sequence %lld",
                        (long long)seq_id);
    if (s->len + n_tokens > int64_t(pool->num_blocks) * pool->bs) {
        ++pool->alloc_failures;
        return fail(PKV_ENOMEM, "kv_pool_append_tokens: sequence longer than the whole pool");
    }
    int rc = append_checked(pool, "kv_pool_append_tokens", s, n_tokens, tokens, slot_mapping_out,
                            copy_out);
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
        if (needs_copy(pool, seqs[i]))
            return fail(PKV_EINVAL, "kv_pool_append_batch: sequence %lld shares its partly "
                                    "filled last block; kv_pool_append_batch_tokens copies it",
                        (long long)seq_ids[i]);
        need += blocks_needed(pool, seqs[i], 1);
    }
    if (need > pool->count) {
        ++pool->alloc_failures;
        return fail(PKV_ENOMEM, "kv_pool_append_batch: need %lld blocks, %lld free",
                    (long long)need, (long long)pool->count);
    }
    int32_t unused[2];
    for (int32_t i = 0; i < n; ++i)
        append_one_seq(pool, seqs[i], 1, nullptr, slot_mapping_out + i, unused);
    return ok();
}

int kv_pool_append_batch_tokens(kv_pool* pool, const int64_t* seq_ids, const int32_t* tokens,
                                int32_t n, int32_t* slot_mapping_out, int32_t* copies_out,
                                int32_t* n_copies_out) {
    if (!pool) return fail(PKV_EINVAL, "kv_pool_append_batch_tokens: pool is NULL");
    if (n < 0 || !n_copies_out) return fail(PKV_EINVAL, "kv_pool_append_batch_tokens: bad n");
    *n_copies_out = 0;
    if (n == 0) return ok();
    if (!seq_ids || !tokens || !slot_mapping_out || !copies_out)
        return fail(PKV_EINVAL, "kv_pool_append_batch_tokens: NULL");
    std::vector<kv_pool::Seq*> seqs(n);
    std::unordered_set<int64_t> seen;
    seen.reserve(size_t(n) * 2);
    // Blocks the step needs, counted in batch order: when every table sharing a partly
    // filled block writes to it in this step, the last of them finds it unshared and
    // writes in place, so only the others copy it.
    std::unordered_map<int32_t, int32_t> copied;   // shared tail block -> copies so far
    int64_t need = 0;
    for (int32_t i = 0; i < n; ++i) {
        seqs[i] = pool->find(seq_ids[i]);
        if (!seqs[i]) return fail(PKV_ENOENT, "kv_pool_append_batch_tokens: unknown sequence %lld",
                                  (long long)seq_ids[i]);
        if (!seen.insert(seq_ids[i]).second)
            return fail(PKV_EINVAL, "kv_pool_append_batch_tokens: duplicate sequence %lld",
                        (long long)seq_ids[i]);
        const kv_pool::Seq* sq = seqs[i];
        if (sq->len % pool->bs == 0) {
            ++need;                                  // a fresh block for the token
        } else {
            const int32_t tb = sq->blocks.back();
            int32_t& c = copied[tb];
            if (pool->ref[tb] - c > 1) {             // still shared when its turn comes
                ++c;
                ++need;
            }
        }
    }
    if (need > pool->count) {
        ++pool->alloc_failures;
        return fail(PKV_ENOMEM, "kv_pool_append_batch_tokens: need %lld blocks, %lld free",
                    (long long)need, (long long)pool->count);
    }
    int32_t nc = 0;
    for (int32_t i = 0; i < n; ++i) {
        int32_t copy[2];
        append_one_seq(pool, seqs[i], 1, tokens + i, slot_mapping_out + i, copy);
        if (copy[0] >= 0) {
            copies_out[2 * nc] = copy[0];
            copies_out[2 * nc + 1] = copy[1];
            ++nc;
        }
    }
    *n_copies_out = nc;
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
    int64_t k = 0;
    for (int32_t b = pool->fhead; b >= 0; b = pool->nxt[b]) blocks_out[k++] = b;
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
    out->cached_blocks = int64_t(pool->cache.size());
    out->prefix_hit_blocks = pool->prefix_hits;
    return ok();
}

}  // extern "C"

extern "C" const char* pkv_version(void) { return "pkv 0.1.0 gfx950"; }
