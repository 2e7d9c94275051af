// table_check.cpp -- CPU checks of the plan's work-block tables (adam_ob_compress_amd/csrc/ob_tables.h),
// built with g++ by tests/test_tables.py; no HIP.
//
// Input on stdin, one shape per line: "n K o_0 o_1 ... o_K" (chunk offsets) or "u n chunk" (uniform
// chunks of `chunk` elements).  For every shape and every block size of the list below it builds the
// table as ob_plan_create does and requires ob::check_block_table to accept it; for uniform shapes it
// also requires ob::uniform_item (the no-allocation kernel's formula) to give every block of it.  Then
// it plants mistakes in tables (a block moved, dropped, duplicated, retagged, shortened; first[]
// shifted) and requires the checker to reject each.  Then the chunk groups of the compressed step's
// passes, for pairs of pass-1 / pass-2 block sizes and several element limits: ob::build_chunk_groups
// must pass ob::check_chunk_groups and be greedy (each group but the last would pass the limit with
// its next chunk); for uniform shapes ob::uniform_chunk_group (the no-allocation path's groups) must
// pass too; planted group mistakes must be rejected.  Prints "table_check ok" and the counts.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "ob_tables.h"

static const int64_t kBlockSizes[] = {1024, 2048, 4096, 8192, 24576, 1 << 20};

static const int64_t kGroupLimits[] = {0, 1, 64, 5000, 1 << 16, 1 << 20, 1 << 24, int64_t(1) << 26};

static int fail(const char* what, const std::string& shape, int64_t be)
{
    std::fprintf(stderr, "FAIL: %s (shape %s, block %lld)\n", what, shape.c_str(), static_cast<long long>(be));
    return 1;
}

int main()
{
    std::string line;
    long shapes = 0, tables = 0, blocks = 0, planted = 0, group_sets = 0;
    while (std::getline(std::cin, line)) {
        if (line.empty()) continue;
        std::istringstream in(line);
        std::vector<int64_t> off;
        bool uniform = false;
        int64_t n = 0, chunk = 0;
        if (line[0] == 'u') {
            char u;
            in >> u >> n >> chunk;
            uniform = true;
            const int64_t K = n > 0 ? (n + chunk - 1) / chunk : 0;
            for (int64_t c = 0; c < K; ++c) off.push_back(c * chunk);
            off.push_back(n);
        } else {
            int64_t K;
            in >> n >> K;
            off.resize(static_cast<size_t>(K) + 1);
            for (auto& o : off) in >> o;
        }
        const std::string shape = line.substr(0, 60);
        ++shapes;
        for (int64_t be : kBlockSizes) {
            std::vector<ob::Item> items;
            std::vector<int32_t> first;
            if (!ob::build_block_table(off, be, items, first)) return fail("build refused", shape, be);
            if (const char* why = ob::check_block_table(off, be, items, first)) return fail(why, shape, be);
            ++tables;
            blocks += static_cast<long>(items.size());
            const int64_t K = static_cast<int64_t>(off.size()) - 1;
            if (uniform && K > 0) {
                const int64_t nbf = K > 1 ? (chunk + be - 1) / be : 0;
                for (size_t j = 0; j < items.size(); ++j) {
                    const ob::Item a = items[j], b = ob::uniform_item(static_cast<int64_t>(j), n, chunk, K, be, nbf);
                    if (a.start != b.start || a.len != b.len || a.chunk != b.chunk)
                        return fail("uniform_item differs from the built table", shape, be);
                }
                for (int64_t c = 0; c <= K; ++c)
                    if (first[static_cast<size_t>(c)] != (c < K ? c * nbf : static_cast<int64_t>(items.size())))
                        return fail("first[] differs from c * blocks per chunk", shape, be);
            }
            // planted mistakes: each must be rejected
            if (items.size() >= 2) {
                std::vector<std::vector<ob::Item>> bad_items;
                auto t = items;
                t[1].start += 64;
                bad_items.push_back(t);                                  // moved
                t = items;
                t.erase(t.begin() + 1);
                bad_items.push_back(t);                                  // dropped
                t = items;
                t.insert(t.begin() + 1, items[1]);
                bad_items.push_back(t);                                  // duplicated
                t = items;
                t[0].chunk += 1;
                bad_items.push_back(t);                                  // retagged
                t = items;
                t[0].len -= 1;
                bad_items.push_back(t);                                  // shortened
                for (auto& bi : bad_items) {
                    if (!ob::check_block_table(off, be, bi, first)) return fail("a planted mistake passed", shape, be);
                    ++planted;
                }
                auto f = first;
                f[f.size() - 1] -= 1;
                if (!ob::check_block_table(off, be, items, f)) return fail("first[] shifted passed", shape, be);
                ++planted;
            }
        }
        // chunk groups over a pass-1 and a pass-2 table
        const int64_t K = static_cast<int64_t>(off.size()) - 1;
        const int64_t pairs[][2] = {{24576, 4096}, {4096, 4096}, {1 << 20, 2048}};
        for (const auto& pr : pairs) {
            std::vector<ob::Item> it1, it2;
            std::vector<int32_t> f1, f2;
            if (!ob::build_block_table(off, pr[0], it1, f1) || !ob::build_block_table(off, pr[1], it2, f2))
                return fail("build refused", shape, pr[0]);
            for (int64_t lim : kGroupLimits) {
                std::vector<ob::ChunkGroup> gs;
                ob::build_chunk_groups(off, f1, f2, lim, gs);
                if (const char* why = ob::check_chunk_groups(off, f1, f2, lim, gs)) return fail(why, shape, lim);
                ++group_sets;
                for (size_t j = 0; j + 1 < gs.size(); ++j)
                    if (off[gs[j].c1 + 1] - off[gs[j].c0] <= lim) return fail("a group is not greedy", shape, lim);
                if (lim <= 0 && gs.size() != (K > 0 ? 1u : 0u)) return fail("no limit but several groups", shape, lim);
                if (uniform && K > 0) {
                    const int64_t nbf1 = K > 1 ? (chunk + pr[0] - 1) / pr[0] : 0;
                    const int64_t nbf2 = K > 1 ? (chunk + pr[1] - 1) / pr[1] : 0;
                    const int64_t q = lim > 0 ? std::max<int64_t>(1, lim / chunk) : K;
                    std::vector<ob::ChunkGroup> us;
                    for (int64_t c0 = 0; c0 < K; c0 += q)
                        us.push_back(ob::uniform_chunk_group(c0, q, K, nbf1, static_cast<int64_t>(it1.size()), nbf2,
                                                             static_cast<int64_t>(it2.size())));
                    if (const char* why = ob::check_chunk_groups(off, f1, f2, lim, us))
                        return fail(why, shape, lim);
                    ++group_sets;
                }
                // planted mistakes
                std::vector<std::vector<ob::ChunkGroup>> bad;
                auto t = gs;
                t.pop_back();
                bad.push_back(t);                                        // last group dropped
                t = gs;
                t[0].n1 += 1;
                bad.push_back(t);                                        // one pass-1 block too many
                t = gs;
                t[0].i2 += 1;
                bad.push_back(t);                                        // pass-2 range shifted
                if (gs.size() >= 2) {
                    t = gs;
                    t[0].c1 -= 1;
                    bad.push_back(t);                                    // a chunk left out
                    t = gs;
                    t[0] = ob::chunk_group(gs[0].c0, gs[1].c1, f1, f2);
                    t.erase(t.begin() + 1);
                    if (lim > 0) bad.push_back(t);                       // two groups merged past the limit
                }
                for (auto& b : bad) {
                    if (!ob::check_chunk_groups(off, f1, f2, lim, b)) return fail("a planted group mistake passed", shape, lim);
                    ++planted;
                }
            }
        }
    }
    std::printf("table_check ok: %ld shapes, %ld tables, %ld blocks, %ld group sets, %ld planted mistakes rejected\n",
                shapes, tables, blocks, group_sets, planted);
    return 0;
}
