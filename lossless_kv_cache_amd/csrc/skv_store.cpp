// skv_store.cpp -- prefix-cache store: coded caches kept in a caller-owned
// arena, found by the longest run of leading block hashes, evicted least
// recently used first.  Only skv_store_put and skv_store_decode touch the
// device; everything else is bookkeeping over arena offsets.
#include <algorithm>
#include <cstring>
#include <list>
#include <map>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "skv_internal.h"

namespace {

constexpr uint64_t kGranule = 256;
constexpr uint32_t kMaxBlocks = 1u << 20;
constexpr uint32_t kBlockTokens = 128;

uint64_t granules(uint64_t bytes) { return (bytes + kGranule - 1) & ~(kGranule - 1); }

struct Entry {
    uint64_t off = 0, span = 0;       // arena offset and granule-rounded size held
    uint64_t bytes = 0;               // container bytes (committed entries)
    std::vector<uint64_t> hashes;
    uint32_t pins = 0;
    bool committed = false;
    uint64_t used_tick = 0;           // last commit or lookup hit
    std::list<uint64_t>::iterator lru;
};

}  // namespace

struct __attribute__((visibility("hidden"))) skv_store {
    std::mutex mu;
    uint8_t* base = nullptr;
    uint64_t size = 0;
    std::map<uint64_t, uint64_t> free_runs;                   // offset -> length, coalesced
    std::unordered_map<uint64_t, Entry> entries;
    std::unordered_multimap<uint64_t, std::pair<uint64_t, uint32_t>> by_hash;   // hash -> (entry, block)
    std::list<uint64_t> lru;                                  // committed entries, least recent first
    uint64_t next_id = 1, tick = 0;
    uint64_t used = 0, container_bytes = 0;
    uint64_t inserts = 0, evictions = 0, hits = 0, misses = 0, hit_blocks = 0;

    // ---- free space
    bool take(uint64_t span, uint64_t* off) {
        for (auto it = free_runs.begin(); it != free_runs.end(); ++it) {
            if (it->second < span) continue;
            *off = it->first;
            const uint64_t rest = it->second - span;
            free_runs.erase(it);
            if (rest) free_runs.emplace(*off + span, rest);
            used += span;
            return true;
        }
        return false;
    }
    void give(uint64_t off, uint64_t len) {
        if (!len) return;
        used -= len;
        auto next = free_runs.lower_bound(off);
        if (next != free_runs.end() && next->first == off + len) {
            len += next->second;
            next = free_runs.erase(next);
        }
        if (next != free_runs.begin()) {
            auto prev = std::prev(next);
            if (prev->first + prev->second == off) {
                prev->second += len;
                return;
            }
        }
        free_runs.emplace(off, len);
    }
    uint64_t largest_free() const {
        uint64_t m = 0;
        for (const auto& kv : free_runs) m = std::max(m, kv.second);
        return m;
    }
    // Longest run the arena would have with every evictable entry gone.
    uint64_t largest_possible() const {
        std::vector<std::pair<uint64_t, uint64_t>> fixed;
        for (const auto& kv : entries)
            if (!kv.second.committed || kv.second.pins) fixed.emplace_back(kv.second.off, kv.second.span);
        std::sort(fixed.begin(), fixed.end());
        uint64_t at = 0, m = 0;
        for (const auto& f : fixed) {
            m = std::max(m, f.first - at);
            at = f.first + f.second;
        }
        return std::max(m, size - at);
    }

    // ---- entries
    void unindex(uint64_t id, const Entry& e) {
        for (uint32_t b = 0; b < e.hashes.size(); ++b) {
            auto r = by_hash.equal_range(e.hashes[b]);
            for (auto it = r.first; it != r.second; ++it) {
                if (it->second.first == id && it->second.second == b) {
                    by_hash.erase(it);
                    break;
                }
            }
        }
    }
    void drop(uint64_t id) {
        auto it = entries.find(id);
        Entry& e = it->second;
        if (e.committed) {
            unindex(id, e);
            lru.erase(e.lru);
            container_bytes -= e.bytes;
        }
        give(e.off, e.span);
        entries.erase(it);
    }
    void touch(uint64_t id, Entry& e) {
        e.used_tick = ++tick;
        lru.splice(lru.end(), lru, e.lru);
    }
    // Room for `span` bytes, evicting least recently used entries if needed.
    int place(uint64_t span, uint64_t* off) {
        if (span > size) return SKV_ERR_CAPACITY;
        if (take(span, off)) return SKV_OK;
        if (largest_possible() < span) return SKV_ERR_CAPACITY;
        for (auto it = lru.begin(); it != lru.end();) {
            const uint64_t id = *it++;
            if (entries[id].pins) continue;
            drop(id);
            ++evictions;
            if (take(span, off)) return SKV_OK;
        }
        return SKV_ERR_CAPACITY;   // not reached: the check above guarantees room
    }
    int reserve(const uint64_t* hashes, uint32_t nblocks, uint64_t bytes, uint64_t* id, void** addr) {
        if (!hashes || !id || nblocks == 0 || nblocks > kMaxBlocks || bytes == 0) return SKV_ERR_ARG;
        const uint64_t span = granules(bytes);
        uint64_t off = 0;
        const int rc = place(span, &off);
        if (rc != SKV_OK) return rc;
        Entry e;
        e.off = off;
        e.span = span;
        e.hashes.assign(hashes, hashes + nblocks);
        *id = next_id++;
        entries.emplace(*id, std::move(e));
        if (addr) *addr = base + off;
        return SKV_OK;
    }
    int commit(uint64_t id, uint64_t bytes) {
        auto it = entries.find(id);
        if (it == entries.end() || it->second.committed) return SKV_ERR_ARG;
        Entry& e = it->second;
        if (bytes == 0 || bytes > e.span) return SKV_ERR_ARG;
        const uint64_t span = granules(bytes);
        give(e.off + span, e.span - span);
        e.span = span;
        e.bytes = bytes;
        e.committed = true;
        for (uint32_t b = 0; b < e.hashes.size(); ++b) by_hash.emplace(e.hashes[b], std::make_pair(id, b));
        e.lru = lru.insert(lru.end(), id);
        e.used_tick = ++tick;
        container_bytes += bytes;
        ++inserts;
        return SKV_OK;
    }
    void lookup(const uint64_t* q, uint32_t nq, skv_store_hit* hit) {
        *hit = skv_store_hit{};
        for (uint32_t b = nq; b-- > 0;) {
            uint64_t best = 0;
            Entry* be = nullptr;
            auto r = by_hash.equal_range(q[b]);
            for (auto it = r.first; it != r.second; ++it) {
                if (it->second.second != b) continue;
                Entry& e = entries[it->second.first];
                if (std::memcmp(e.hashes.data(), q, sizeof(uint64_t) * (b + 1)) != 0) continue;
                if (!be || e.used_tick > be->used_tick) {
                    best = it->second.first;
                    be = &e;
                }
            }
            if (be) {
                ++be->pins;
                touch(best, *be);
                ++hits;
                hit_blocks += b + 1;
                hit->entry = best;
                hit->matched_blocks = b + 1;
                hit->entry_blocks = uint32_t(be->hashes.size());
                hit->container = base + be->off;
                hit->container_bytes = be->bytes;
                return;
            }
        }
        ++misses;
    }
    Entry* committed_entry(uint64_t id) {
        auto it = entries.find(id);
        return it == entries.end() || !it->second.committed ? nullptr : &it->second;
    }
};

extern "C" {

int skv_store_create(void* arena, uint64_t arena_bytes, skv_store** store) {
    if (!arena || !store || reinterpret_cast<uintptr_t>(arena) % kGranule != 0 || arena_bytes < kGranule ||
        arena_bytes % kGranule != 0)
        return SKV_ERR_ARG;
    skv_store* st = new (std::nothrow) skv_store;
    if (!st) return SKV_ERR_NOMEM;
    st->base = static_cast<uint8_t*>(arena);
    st->size = arena_bytes;
    st->free_runs.emplace(0, arena_bytes);
    *store = st;
    return SKV_OK;
}

void skv_store_destroy(skv_store* store) { delete store; }

int skv_store_reserve(skv_store* store, const uint64_t* hashes, uint32_t nblocks, uint64_t bytes, uint64_t* entry,
                      void** addr) {
    if (!store || !addr) return SKV_ERR_ARG;
    std::lock_guard<std::mutex> lk(store->mu);
    return store->reserve(hashes, nblocks, bytes, entry, addr);
}

int skv_store_commit(skv_store* store, uint64_t entry, uint64_t bytes) {
    if (!store) return SKV_ERR_ARG;
    std::lock_guard<std::mutex> lk(store->mu);
    return store->commit(entry, bytes);
}

int skv_store_abort(skv_store* store, uint64_t entry) {
    if (!store) return SKV_ERR_ARG;
    std::lock_guard<std::mutex> lk(store->mu);
    auto it = store->entries.find(entry);
    if (it == store->entries.end() || it->second.committed) return SKV_ERR_ARG;
    store->drop(entry);
    return SKV_OK;
}

int skv_store_put(skv_store* store, const uint64_t* hashes, uint32_t nblocks, const void* tables_blob,
                  const skv_shape* s, const void* d_target, const void* d_aux, void* d_work, size_t* work_bytes,
                  hipStream_t stream, uint64_t* entry, uint64_t* container_bytes) {
    if (!store || !s || !work_bytes) return SKV_ERR_ARG;
    if (!d_work) {
        size_t bound = 0;
        return skv_encode(tables_blob, s, d_target, d_aux, nullptr, 0, &bound, nullptr, work_bytes, stream);
    }
    if (!hashes || !entry || !container_bytes || s->tokens % kBlockTokens != 0 || nblocks != s->tokens / kBlockTokens)
        return SKV_ERR_ARG;
    skv::PendingEncode pe{};
    int rc = skv::encode_begin(tables_blob, s, d_target, d_aux, d_work, *work_bytes, stream, &pe);
    if (rc != SKV_OK) return rc;
    uint64_t id = 0;
    void* addr = nullptr;
    {
        std::lock_guard<std::mutex> lk(store->mu);
        rc = store->reserve(hashes, nblocks, pe.container_bytes, &id, &addr);
    }
    if (rc != SKV_OK) return rc;
    rc = skv::encode_finish(&pe, addr, pe.container_bytes, stream);
    std::lock_guard<std::mutex> lk(store->mu);
    if (rc != SKV_OK) {
        store->drop(id);
        return rc;
    }
    rc = store->commit(id, pe.container_bytes);
    if (rc == SKV_OK) {
        *entry = id;
        *container_bytes = pe.container_bytes;
    }
    return rc;
}

int skv_store_lookup(skv_store* store, const uint64_t* hashes, uint32_t nblocks, skv_store_hit* hit) {
    if (!store || !hit || (!hashes && nblocks)) return SKV_ERR_ARG;
    std::lock_guard<std::mutex> lk(store->mu);
    store->lookup(hashes, nblocks, hit);
    return SKV_OK;
}

int skv_store_release(skv_store* store, uint64_t entry) {
    if (!store) return SKV_ERR_ARG;
    std::lock_guard<std::mutex> lk(store->mu);
    Entry* e = store->committed_entry(entry);
    if (!e || e->pins == 0) return SKV_ERR_ARG;
    --e->pins;
    return SKV_OK;
}

int skv_store_decode(skv_store* store, const void* tables_blob, uint64_t entry, uint32_t token_begin,
                     uint32_t token_end, const void* d_aux, void* d_out, size_t out_capacity, void* d_work,
                     size_t* work_bytes, hipStream_t stream) {
    if (!store || !work_bytes) return SKV_ERR_ARG;
    if (!d_work)
        return token_end == 0 && token_begin == 0
                   ? skv_decode(tables_blob, nullptr, 0, nullptr, nullptr, 0, nullptr, work_bytes, stream)
                   : skv_decode_range(tables_blob, nullptr, 0, token_begin, token_end, nullptr, nullptr, 0, nullptr,
                                      work_bytes, stream);
    const void* cont = nullptr;
    uint64_t bytes = 0;
    {
        std::lock_guard<std::mutex> lk(store->mu);
        Entry* e = store->committed_entry(entry);
        if (!e) return SKV_ERR_ARG;
        ++e->pins;
        cont = store->base + e->off;
        bytes = e->bytes;
    }
    const int rc = token_end == 0 && token_begin == 0
                       ? skv_decode(tables_blob, cont, bytes, d_aux, d_out, out_capacity, d_work, work_bytes, stream)
                       : skv_decode_range(tables_blob, cont, bytes, token_begin, token_end, d_aux, d_out, out_capacity,
                                          d_work, work_bytes, stream);
    std::lock_guard<std::mutex> lk(store->mu);
    --store->entries[entry].pins;
    return rc;
}

int skv_store_erase(skv_store* store, uint64_t entry) {
    if (!store) return SKV_ERR_ARG;
    std::lock_guard<std::mutex> lk(store->mu);
    Entry* e = store->committed_entry(entry);
    if (!e) return SKV_ERR_ARG;
    if (e->pins) return SKV_ERR_BUSY;
    store->drop(entry);
    return SKV_OK;
}

int skv_store_stats(skv_store* store, skv_store_info* stats) {
    if (!store || !stats) return SKV_ERR_ARG;
    std::lock_guard<std::mutex> lk(store->mu);
    skv_store_info o{};
    o.arena_bytes = store->size;
    o.used_bytes = store->used;
    o.largest_free = store->largest_free();
    o.container_bytes = store->container_bytes;
    for (const auto& kv : store->entries) {
        if (!kv.second.committed) continue;
        ++o.entries;
        if (kv.second.pins) ++o.pinned;
    }
    o.inserts = store->inserts;
    o.evictions = store->evictions;
    o.hits = store->hits;
    o.misses = store->misses;
    o.hit_blocks = store->hit_blocks;
    *stats = o;
    return SKV_OK;
}

}  // extern "C"
