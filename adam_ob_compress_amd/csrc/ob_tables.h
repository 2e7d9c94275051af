// ob_tables.h -- the work-block tables of a plan, in plain C++17: built by the host runtime
// (ob_api.cpp), checked there and by tests/table_check.cpp (a CPU program), and, for uniform chunks,
// computed block by block by the no-allocation path's kernel (ob_noalloc.hip; constexpr functions
// are callable from device code).
#pragma once

#include <stdint.h>

#include <vector>

namespace ob {

// One work block: a contiguous run of elements inside one chunk.  Blocks of a chunk are consecutive,
// start at multiples of 64 elements and (except a chunk's last) hold a whole number of tiles.
struct Item {
    int64_t start;
    int32_t len;
    int32_t chunk;
};

// Append the blocks of `block_elems` elements of every chunk [off[c], off[c+1]) to `items` (each
// chunk's last block ragged) and set first[c] to the index of chunk c's first block, first[K] to the
// count.  False (tables untouched past what was appended) if the count would pass INT32_MAX.
inline bool build_block_table(const std::vector<int64_t>& off, int64_t block_elems, std::vector<Item>& items,
                              std::vector<int32_t>& first)
{
    const size_t K = off.size() - 1;
    first.assign(K + 1, 0);
    for (size_t c = 0; c < K; ++c) {
        first[c] = static_cast<int32_t>(items.size());
        for (int64_t s = off[c]; s < off[c + 1]; s += block_elems) {
            const int64_t len = off[c + 1] - s < block_elems ? off[c + 1] - s : block_elems;
            items.push_back(Item{s, static_cast<int32_t>(len), static_cast<int32_t>(c)});
            if (items.size() > static_cast<size_t>(INT32_MAX)) return false;
        }
    }
    first[K] = static_cast<int32_t>(items.size());
    return true;
}

// Block j of the table build_block_table makes for uniform chunks (chunk c = [c*chunk, min((c+1)*chunk,
// n)), K of them), computed on its own: nbf = blocks of every chunk but the last (ceil(chunk / be)).
constexpr Item uniform_item(int64_t j, int64_t n, int64_t chunk, int64_t K, int64_t be, int64_t nbf)
{
    int64_t c = K > 1 ? j / nbf : 0;
    if (c > K - 1) c = K - 1;
    const int64_t start = c * chunk + (j - c * nbf) * be;
    const int64_t end = c == K - 1 ? n : (c + 1) * chunk;
    return Item{start, static_cast<int32_t>(end - start < be ? end - start : be), static_cast<int32_t>(c)};
}

// What the kernels assume of a table, checked: nullptr when it holds, else the first failure.  Every
// chunk's blocks are consecutive entries tagged with the chunk, tile its elements exactly in order,
// each block but the chunk's last holds block_elems elements, every block starts at a multiple of 64
// and holds at least one element, and first[] indexes them.
inline const char* check_block_table(const std::vector<int64_t>& off, int64_t block_elems,
                                     const std::vector<Item>& items, const std::vector<int32_t>& first)
{
    const size_t K = off.size() - 1;
    if (block_elems <= 0 || block_elems % 1024 != 0) return "block size is not a whole number of tiles";
    if (first.size() != K + 1 || first[0] != 0 || static_cast<size_t>(first[K]) != items.size())
        return "first[] does not span the table";
    for (size_t c = 0; c < K; ++c) {
        if (first[c + 1] < first[c]) return "first[] decreases";
        if (first[c + 1] == first[c]) return "a chunk has no block";
        int64_t next = off[c];
        for (int32_t b = first[c]; b < first[c + 1]; ++b) {
            const Item& it = items[static_cast<size_t>(b)];
            if (it.chunk != static_cast<int32_t>(c)) return "a block is tagged with another chunk";
            if (it.start != next) return "blocks do not tile their chunk in order";
            if (it.start % 64 != 0) return "a block does not start at a multiple of 64";
            if (it.len < 1) return "an empty block";
            if (b + 1 < first[c + 1] && it.len != block_elems) return "an inner block is not full";
            if (it.len > block_elems) return "a block is longer than the block size";
            next = it.start + it.len;
        }
        if (next != off[c + 1]) return "blocks do not end at their chunk's end";
    }
    return nullptr;
}

// Chunk groups.  The compressed step runs its two passes group by group: pass 1 over the group's
// chunks, then pass 2 over the same chunks while what pass 1 read is still in the last-level cache.
// A group is consecutive chunks [c0, c1), its blocks [i1, i1 + n1) of the pass-1 table and
// [i2, i2 + n2) of the pass-2 table (f1 / f2: those tables' first-block indexes).
struct ChunkGroup {
    int32_t c0, c1;
    int32_t i1, n1;
    int32_t i2, n2;
};

inline ChunkGroup chunk_group(int64_t c0, int64_t c1, const std::vector<int32_t>& f1, const std::vector<int32_t>& f2)
{
    return {static_cast<int32_t>(c0), static_cast<int32_t>(c1), f1[c0], f1[c1] - f1[c0], f2[c0], f2[c1] - f2[c0]};
}

// Greedy groups: each as many chunks as keep it within max_elems elements (a larger chunk is a group of
// its own); max_elems <= 0 gives one group of all chunks.
inline void build_chunk_groups(const std::vector<int64_t>& off, const std::vector<int32_t>& f1,
                               const std::vector<int32_t>& f2, int64_t max_elems, std::vector<ChunkGroup>& out)
{
    const int64_t K = static_cast<int64_t>(off.size()) - 1;
    out.clear();
    for (int64_t c0 = 0; c0 < K;) {
        int64_t c1 = max_elems > 0 ? c0 + 1 : K;
        while (c1 < K && off[c1 + 1] - off[c0] <= max_elems) ++c1;
        out.push_back(chunk_group(c0, c1, f1, f2));
        c0 = c1;
    }
}

// For K uniform chunks (nbf blocks in each but the last; n_1 / n_2 blocks in all): the group of q chunks
// starting at chunk c0 (the last group takes what is left).
constexpr ChunkGroup uniform_chunk_group(int64_t c0, int64_t q, int64_t K, int64_t nbf1, int64_t n_1, int64_t nbf2,
                                         int64_t n_2)
{
    const int64_t c1 = c0 + q < K ? c0 + q : K;
    const int64_t e1 = c1 < K ? c1 * nbf1 : n_1, e2 = c1 < K ? c1 * nbf2 : n_2;
    return {static_cast<int32_t>(c0),           static_cast<int32_t>(c1),
            static_cast<int32_t>(c0 * nbf1),    static_cast<int32_t>(e1 - c0 * nbf1),
            static_cast<int32_t>(c0 * nbf2),    static_cast<int32_t>(e2 - c0 * nbf2)};
}

// nullptr if `groups` cover every chunk once, in order, each within max_elems elements unless it is a
// single chunk (max_elems <= 0: no limit), with block ranges that are exactly their chunks' blocks in
// both tables; otherwise what is wrong.
inline const char* check_chunk_groups(const std::vector<int64_t>& off, const std::vector<int32_t>& f1,
                                      const std::vector<int32_t>& f2, int64_t max_elems,
                                      const std::vector<ChunkGroup>& groups)
{
    const int64_t K = static_cast<int64_t>(off.size()) - 1;
    int64_t next = 0;
    for (const ChunkGroup& g : groups) {
        if (g.c0 != next) return "groups do not cover the chunks in order";
        if (g.c1 <= g.c0 || g.c1 > K) return "an empty or overlong group";
        if (max_elems > 0 && g.c1 - g.c0 > 1 && off[g.c1] - off[g.c0] > max_elems)
            return "a group of several chunks passes the element limit";
        if (g.i1 != f1[g.c0] || g.n1 != f1[g.c1] - f1[g.c0]) return "a group's pass-1 blocks are not its chunks'";
        if (g.i2 != f2[g.c0] || g.n2 != f2[g.c1] - f2[g.c0]) return "a group's pass-2 blocks are not its chunks'";
        next = g.c1;
    }
    return next == K ? nullptr : "groups do not reach the last chunk";
}

}  // namespace ob
