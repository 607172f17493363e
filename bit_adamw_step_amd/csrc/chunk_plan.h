// chunk_plan.h -- how a launch's work is cut into chunks and dealt to its workgroups (host
// code, no HIP dependency, so the CPU tests can build it on their own).  Not part of the
// public ABI.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <functional>
#include <queue>
#include <utility>
#include <vector>

namespace adamw4 {

constexpr int kPlanRows = 16;   // 128-value blocks a workgroup processes per iteration

// A run of `units` consecutive 128-value units of one tensor, from `first_unit` on.  An entry
// with units = 0 is padding and does nothing.
struct alignas(16) Chunk {
    uint32_t tensor;
    uint32_t first_unit;
    uint32_t units;
    uint32_t reserved;
};

// Chunk size: 64 units (8192 values, four workgroup iterations) for large lists; smaller when
// the list is too small to give each of the launch's workgroups about 8 chunks (so the last
// round of chunks leaves little idle time), but never below one workgroup iteration (16
// units).  Short chunks keep the launch's concurrent streams close together: in interleaved,
// warmed-up runs on MI355X, 64-unit chunks beat 256-unit ones by 0.8% (ZIP-SR) to 2.6%
// (ZE-EDEN) on the 2.7B list, 5% on the 834M list and 7% on one rank's eighth of the 2.7B
// list; 32 and 128 units came within 1% of 64.
inline uint32_t pick_chunk_units(uint64_t total_units, uint64_t workgroups) {
    const uint64_t target = total_units / (workgroups * 8);
    uint32_t cu = 64;
    while (cu > uint32_t(kPlanRows) && cu > target) cu >>= 1;
    return cu;
}

// The launch walks the chunk table with a grid stride: workgroup w takes entries w, w + G,
// w + 2G, ... (G workgroups), so the workgroups stream neighbouring chunks together (giving
// each workgroup one contiguous range of the list instead was 6% slower in the streaming
// probe).  The table is laid out so that this order is balanced:
//   1. the last partial round of chunks and the full round before it are re-cut, in list
//      order, into about 4 G pieces of (nearly) equal length in whole workgroup iterations, so
//      the launch ends on small pieces;
//   2. chunks are dealt in list order, each to the workgroup with the least work so far
//      (ceil(units / 16) iterations; ties to the lowest index, which is round-robin when the
//      chunks are equal);
//   3. workgroup w's k-th chunk is stored at entry k G + w; workgroups with fewer chunks get
//      empty entries (units = 0).
// Left alone when the list has at most G chunks.
inline void balance_chunks(std::vector<Chunk>& chunks, uint64_t workgroups) {
    const uint64_t n = chunks.size();
    const uint64_t G = workgroups;
    if (G < 2 || n <= G) return;
    // 1. re-cut the tail
    if (n % G != 0) {
        const uint64_t t0 = n - G - n % G;   // first re-cut chunk
        uint64_t total = 0;
        for (uint64_t i = t0; i < n; ++i) total += chunks[i].units;
        const uint64_t pieces = 4 * G;
        // end of piece j in the re-cut stretch: j * total / pieces rounded to a multiple of kPlanRows
        auto cut = [&](uint64_t j) -> uint64_t {
            if (j >= pieces) return total;
            return std::min<uint64_t>(total, (j * total / pieces + kPlanRows / 2) / kPlanRows * kPlanRows);
        };
        std::vector<Chunk> out(chunks.begin(), chunks.begin() + t0);
        uint64_t pos = 0, j = 1;
        for (uint64_t i = t0; i < n;) {
            // a run of contiguous chunks of one tensor
            Chunk run = chunks[i++];
            while (i < n && chunks[i].tensor == run.tensor &&
                   chunks[i].first_unit == run.first_unit + run.units)
                run.units += chunks[i++].units;
            const uint64_t end = pos + run.units;
            for (uint64_t cur = pos; cur < end;) {
                while (cut(j) <= cur) ++j;
                const uint64_t stop = std::min(cut(j), end);
                out.push_back(Chunk{run.tensor, uint32_t(run.first_unit + (cur - pos)),
                                    uint32_t(stop - cur), 0});
                cur = stop;
            }
            pos = end;
        }
        chunks.swap(out);
    }
    // 2. deal to the least-loaded workgroup
    using Load = std::pair<uint64_t, uint64_t>;   // (iterations so far, workgroup)
    std::priority_queue<Load, std::vector<Load>, std::greater<Load>> heap;
    for (uint64_t w = 0; w < G; ++w) heap.push(Load{0, w});
    std::vector<std::vector<uint32_t>> mine(G);
    for (uint64_t c = 0; c < chunks.size(); ++c) {
        Load l = heap.top();
        heap.pop();
        mine[l.second].push_back(uint32_t(c));
        l.first += (chunks[c].units + kPlanRows - 1) / kPlanRows;
        heap.push(l);
    }
    // 3. lay out the rounds
    size_t rounds = 0;
    for (const auto& m : mine) rounds = std::max(rounds, m.size());
    std::vector<Chunk> table(rounds * G, Chunk{0, 0, 0, 0});
    for (uint64_t w = 0; w < G; ++w)
        for (size_t k = 0; k < mine[w].size(); ++k) table[k * G + w] = chunks[mine[w][k]];
    chunks.swap(table);
}

}  // namespace adamw4
