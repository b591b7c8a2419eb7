// Split-KV helpers shared by the C ABI and the tests' expectations: split counts and the
// workspace layout (key ranges processed by separate workgroups, then merged by their LSE).
#pragma once

#include "fa_internal.h"

namespace fa {

// Split-KV (key ranges processed by separate workgroups, then merged by their LSE).
constexpr int kMaxKvSplits = 64;
// Workspace of fa_fwd_splitkv: partial O (fp32) and partial LSE per split, 256-byte aligned.
inline size_t splitkv_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int splits) {
    if (splits <= 1) return 0;
    const size_t rows = (size_t)(B * H * N);
    const size_t o_bytes = (size_t)splits * rows * (size_t)d * sizeof(float);
    const size_t l_bytes = (size_t)splits * rows * sizeof(float);
    return (o_bytes + 255) / 256 * 256 + (l_bytes + 255) / 256 * 256;
}
// The chooser's split count: enough workgroups for two per CU, each split at least two
// key tiles.  A grid that already fills the chip is split only when its last round of
// workgroups would run nearly empty (a quarter of the slots or less, within three rounds):
// then the split count with the fewest rounds per unit of work, 2 or 3 (B=2 H=8 N=4097
// d=128: 528 workgroups on 512 slots, 209 us unsplit, 190 us in 3 parts).  Otherwise the
// partials' extra HBM traffic outweighs the balance and the answer is 1.
inline int choose_kv_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d) {
    const int64_t grid = B * H * ceil_div(Nq, 128);
    const int64_t tiles = ceil_div(Nk, splitkv_block_k(d));
    const int64_t slots = 2 * kCus;
    if (grid >= slots) {
        const int64_t rounds = ceil_div(grid, slots), last = grid - (rounds - 1) * slots;
        if (rounds > 3 || 4 * last > slots) return 1;
        int best = 1;
        double best_cost = (double)rounds;
        for (int s = 2; s <= 3 && s <= tiles / 2; ++s) {
            const double cost = (double)ceil_div(grid * s, slots) / s;
            if (cost < best_cost) best = s, best_cost = cost;
        }
        return best;
    }
    int64_t s = ceil_div(2 * kCus, grid);
    if (s > tiles / 2) s = tiles / 2;
    if (s > kMaxKvSplits) s = kMaxKvSplits;
    return s < 2 ? 1 : (int)s;
}

}  // namespace fa
