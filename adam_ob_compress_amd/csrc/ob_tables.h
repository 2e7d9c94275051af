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

}  // namespace ob
