// Internal declarations shared by the C ABI (fa_api.hip) and the kernels.
//
// The tile / occupancy chooser lives here as a pure host function so that the
// library can report its plan without a GPU (fa_fwd_plan) and the CPU tests can
// check it.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "fa.h"

namespace fa {

// Kernel arguments of the forward pass (passed by value).
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int n;          // query rows per head (N, or Nq when queries and keys differ in length)
    int nk;         // keys per head (= n for self-attention)
    int n_qblk;     // ceil(n / Br)
    int n_blocks;   // workgroups in the grid = B*H*n_qblk (*splits)
    float c;        // scale * log2(e): scores are taken to base 2 inside the kernel
    // bf16/fp16 forward: a redone tile sets the running maximum this far (base 2) above its own
    // maximum, so P stays at most 2^-8 there and later tiles need a larger jump to be redone.
    // (An argument, so it sits in a scalar register: as a literal the compiler holds it in a
    // vector register, and the 168-register kernels then spill.)  fp16 uses none: its P
    // would lose range to underflow.
    float m_headroom = 8.f;
    // split-KV only: key tiles [s*tiles_per_split, (s+1)*tiles_per_split) per split s;
    // normalised fp32 partials, that of head bh, split s and query row part_row0 + i at
    // o_part + bh*po_head + s*po_split + i*d (d floats) and lse_part + bh*pl_head + s*pl_split + i
    // (a split-KV call: [splits][B*H*N][d] and [splits][B*H*N]; the tail rows ahead of an
    // 8-wave launch: per head, in the first rows of that head's O).  The grid covers query
    // blocks qblk0 .. qblk0 + n_qblk - 1 of each head.
    int splits;
    int tiles_per_split;
    float* o_part;
    float* lse_part;
    int64_t po_head = 0, po_split = 0, pl_head = 0, pl_split = 0;
    int part_row0 = 0;
    int qblk0 = 0;
};

// Arguments of the split-KV merge: `rows` merged rows, rows_per_head of them per head (head
// bh's row i is output row out_row0 + i of that head, whose O and LSE hold out_head rows);
// partials laid out as in FwdArgs.
struct MergeArgs {
    const float* o_part;
    const float* lse_part;
    void* o;
    float* lse;
    int64_t rows;
    int rows_per_head;
    int splits;
    int64_t po_head, po_split, pl_head, pl_split;
    int64_t out_head;
    int out_row0;
};

// Kernel arguments of the backward pass.
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    float* dsum;    // workspace: D = rowsum(dO * O), [B, H, N]
    float* l2;      // workspace: LSE * log2(e), [B, H, N]
    int n;
    int n_blk;      // 128-row blocks per head (query blocks for dQ, key blocks for dK/dV)
    int n_blocks;
    float c;        // scale * log2(e)
    float scale;
};

// Workspace of the backward: two fp32 values per row, each array 256-byte aligned.
inline size_t bwd_workspace_bytes(int64_t B, int64_t H, int64_t N) {
    const size_t one = (size_t)(B * H * N) * sizeof(float);
    return 2 * ((one + 255) / 256 * 256);
}

// Kernel variants compiled into the library.  kind: 0 = fp32, 1 = fp16, 2 = bf16.
struct FwdVariant {
    int dtype;      // fa_dtype
    int d;          // head dim
    int rows_per_wave;
    int block_k;
    int waves;
};

constexpr int kWaveSize = 64;
constexpr int kXcds = 8;          // MI355X: 8 accelerator complex dies, 32 CUs each
constexpr int kCus = 256;
constexpr int kLdsPerCu = 160 * 1024;

// ceil(a / b) for a >= 0, b > 0, without forming a + b - 1 (no overflow near INT64_MAX)
inline int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0); }

// LDS bytes of one forward workgroup: a K tile and a V tile per stage.
inline int fwd_lds_bytes(int dtype, int d, int block_k, int stages) {
    const int elt = dtype == FA_F32 ? 4 : 2;
    if (dtype == FA_F32) {
        // one K and one V tile per wave (4 waves), rows padded by one element
        return 4 * 2 * block_k * (d + 1) * elt;
    }
    return stages * (2 * block_k * d * elt);
}

// LDS stages of a bf16/fp16 plan: three for the ping-pong schedule (8 waves, non-causal
// d = 64), whose late wave group still reads V of the previous tile while the next one is
// copied; two otherwise.
inline int fwd_stages(int d, int waves, int causal) { return (waves == 8 && d == 64 && !causal) ? 3 : 2; }

// Relative throughput of one CU running m resident forward workgroups (index m), measured
// across grids of one to three rounds at N = 2049..4097 and the long workloads: a lone 4-wave
// workgroup (one wave per SIMD) cannot overlap its own softmax with its MFMAs; two or three
// overlap each other's; one 8-wave workgroup (two waves per SIMD, half the L2 -> LDS traffic
// per FLOP) runs as well as three 4-wave ones.
constexpr double kEff4[4] = {0.0, 0.6, 1.0, 1.05};
constexpr double kEff8[2] = {0.0, 1.05};

// Time of a grid of w workgroups of `unit` work each (1 = 256 query rows against all keys),
// at most per_cu resident per CU: whole rounds of per_cu per CU, then a last partial round
// whose busiest CU holds ceil(rem / kCus) of them.
inline double grid_time(int64_t w, double unit, int per_cu, const double* eff) {
    const int64_t slots = (int64_t)per_cu * kCus;
    const int64_t full = w / slots, rem = w % slots;
    double t = (double)full * per_cu * unit / eff[per_cu];
    if (rem) {
        const int m = (int)ceil_div(rem, kCus);
        t += m * unit / eff[m];
    }
    return t;
}

// Key tile of the split-KV path (the 4-wave tile-loop kernel's Bc).
inline int splitkv_block_k(int64_t d) { return d == 128 ? 64 : 128; }

// Last rows ahead of an 8-wave launch ("tail first").  When N = 256 k + r with 1 <= r <= 128,
// the 8-wave grid's last block of each head holds r rows on its first ceil(r / 32) waves, which
// sweep every key while the others idle: on a grid of whole rounds those blocks make a round of
// their own.  Instead the r
// rows of every head are computed first by the split-KV kernel, S workgroups per head over
// S key ranges, their normalised partials parked in the first rows of that head's O (which
// the 8-wave launch overwrites later, in stream order); the 8-wave launch then covers the k
// full blocks, and the first block of each head merges those partials into the last rows'
// O and LSE before its own outputs overwrite them.  S aims at 256
// workgroups in all and at most 16 key tiles per range, within what the parked partials may
// occupy: 4 S r (d + 1) bytes of the head's 256 k d 2 bytes of O.  Measured against the
// plans before it (interleaved, N(0,1) inputs unless noted): B2 H8 N4097 d128 151.4 -> 139.2
// us (edge workload heads 161.4 -> 150.8), B4 H8 N4097 292.5 -> 265.5, B2 H4 N8193 275.3 ->
// 256.1, B2 H16 N4097 d64 182.5 -> 162.8, B2 H8 N16385 2.05 -> 1.88 ms, B8 H8 N4097 527 ->
// 505 us.  The tail rows read every head's K and V once more, so with many heads the
// launches cost more than the round they save (B16 H64 N2049: 2.13 ms on the 4-wave plan,
// 2.33 ms this way); tail_first_cost prices that.
constexpr int kTailFirstMaxRows = 128;   // one 128-row block of the split-KV kernel per head
inline int tail_first_splits(int64_t B, int64_t H, int64_t N, int64_t d) {
    const int64_t full = N / 256, r = N % 256;
    if (full <= 0 || r < 1 || r > kTailFirstMaxRows || B * H <= 0) return 1;
    const int64_t tiles = ceil_div(N, splitkv_block_k(d));
    int64_t s = ceil_div(256, B * H);
    if (s < ceil_div(tiles, 16)) s = ceil_div(tiles, 16);
    if (s > 64) s = 64;   // kMaxKvSplits
    if (s > tiles) s = tiles;
    const int64_t room = full * 256 * d * 2 / (4 * r * (d + 1));   // partials that fit in O
    if (s > room) s = room;
    return s < 2 ? 1 : (int)s;
}
// The tail-first launches in units of grid_time (one 256-row block against all N keys): a
// fixed 8 us, the second pass over every head's K and V at 6 TB/s, and the split workgroups'
// rounds (two per CU, one busy wave each) at 1 us per key tile; one unit at 4.5 TFLOP/s per
// CU for d = 128 and 3.6 for d = 64 (the 8-wave kernels' measured rates).  Fitted to the
// tail launches' share of measured times: about 15 us at B2 H8 N4097, 33 us at B8 H16
// N2049, 300 us at B16 H64 N2049.
inline double tail_first_cost(int64_t B, int64_t H, int64_t N, int64_t d, int s) {
    const double kv_us = (double)(B * H) * (double)N * (double)d * 4.0 / 6e6;
    const int64_t tiles = ceil_div(N, splitkv_block_k(d));
    const double rounds = (double)ceil_div(B * H * s, 2 * kCus);
    const double tail_us = 8.0 + kv_us + rounds * (double)ceil_div(tiles, s) * 1.0;
    const double unit_us = 256.0 * (double)N * (double)d * 4.0 / (d == 128 ? 4.5e6 : 3.6e6);
    return tail_us / unit_us;
}

// The chooser.  Inputs are already validated (d in {64,128}, dtype known, N > 0).
//
// bf16/fp16: 32 query rows per wave (one 32-row MFMA column block), two waves per SIMD.
//  * Non-causal, N >= 2048: the plan grid_time costs lowest, over 8 waves (Br = 256), 4 waves
//    at two workgroups per CU and 4 waves at three.  It picks the measured best plan on every
//    grid tried: 8 waves for full rounds (B4 H32 N16384), for B3 H8 N4097 (408 blocks of 256;
//    218 against 233-238 us) and B2 H8 N2049 (58 against 62-63 us); three 4-wave workgroups
//    per CU for B2 H8 N4097 (176 against 190-201 us), B4 H8 N4097 (288 against 304-307 us)
//    and d = 64 B2 H16 N4097 (180 against 196 us); 4 waves at two per CU for B1 H8 N4096.
//    The rules below serve causal grids and shorter heads.
//  * Long sequences: 8 waves per workgroup (Br = 256, one workgroup per CU) and Bc = 128
//    keys per LDS stage (128 KiB of K/V stages at d = 128).  A K/V tile then serves twice
//    as many queries -- half the L2 -> LDS traffic per FLOP -- with half as many
//    barriers per key, which measured 4-10% faster at N >= 8192.
//  * Otherwise (N < 2048, or a grid that would leave most of its last round of
//    workgroups idle, as B*H = 16, N = 4097 does): 4 waves per workgroup (Br = 128, two
//    workgroups per CU), Bc = 64 at d = 128 and 128 at d = 64 (64 KiB of stages).
//  * Causal at d = 128 where the 8-wave plan would apply: 4 waves and Bc = 32 instead
//    (32 KiB of stages, <= 168 VGPRs), three workgroups and three waves per SIMD.  The
//    causal grid mixes long and short query blocks and its diagonal tiles carry masking
//    work; the third wave hides those stalls (4% faster at B=4 H=32 N=16384, while the
//    non-causal kernel is 2.6% slower this way).
//  * Non-causal d = 128 on the 4-wave plan, when three workgroups per CU take fewer
//    rounds x workgroups-per-CU than two (e.g. 528 or 640 workgroups, just over one round
//    of 512): Bc = 32 and three workgroups per CU, so the grid runs as one round instead of
//    a full round and a nearly empty one (8% faster at B=2 H=8 N=4097 and B=5 H=8 N=2048).
//    Causal grids are left alone: their workgroups differ in length, and there the same
//    switch measured 8-21% slower.
//  * Non-causal d = 128 with N < 2048 and at least two workgroups of 128 rows per CU: the
//    same 32-key plan.  Short heads are bound by latency and HBM, and a third resident
//    workgroup per CU overlaps one's copies with another's compute (B=16 H=64: N=128 35 ->
//    31 us, N=640 -3%, N=1024 -3%, N=2047 -0.7%).  Smaller grids keep Bc = 64 (at 64
//    workgroups the 32-key plan measured up to 3% slower).
//  * The same for d = 64: 64-key tiles (32 KiB of stages, 132 VGPRs), three workgroups per
//    CU (B=16 H=64: N=128 22 -> 19.5 us, N=512 118 -> 101 us, N=1024 -6%, N=2047 -1.3%).
// fp32: 32 query rows per workgroup, its 4 waves splitting the 32-key tiles among
// themselves (latency-bound sizes only).
inline fa_plan choose_fwd_plan(int64_t B, int64_t H, int64_t N, int64_t d, int dtype, int causal) {
    fa_plan p{};
    p.waves = 4;
    p.kv_splits = 1;
    p.wave_kv_splits = 1;
    p.tail_kv_splits = 1;   // set by the caller once the plan is final
    p.rows_per_wave = 32;
    if (dtype == FA_F32) {
        p.block_k = 32;
        p.wave_kv_splits = 4;
    } else if (!causal && N >= 2048) {
        // Three plans, costed by grid_time: 8 waves (one 256-row workgroup per CU), 4 waves at
        // two workgroups per CU (Bc 64 at d = 128, 128 at d = 64) or at three (Bc 32 / 64).
        const int64_t g8 = B * H * ceil_div(N, 8 * 32), g4 = B * H * ceil_div(N, 4 * 32);
        double t8 = grid_time(g8, 1.0, 1, kEff8);
        if (const int s = tail_first_splits(B, H, N, d); s > 1) {   // the last rows ahead of the launch
            const double first = grid_time(B * H * (N / 256), 1.0, 1, kEff8) + tail_first_cost(B, H, N, d, s);
            if (first < t8) t8 = first;
        }
        const double t2 = grid_time(g4, 0.5, 2, kEff4);
        const double t3 = grid_time(g4, 0.5, 3, kEff4);
        if (t8 <= t2 && t8 <= t3) {
            p.waves = 8;
            p.block_k = 128;
        } else {
            p.waves = 4;
            p.block_k = t2 <= t3 ? (d == 128 ? 64 : 128) : (d == 128 ? 32 : 64);
        }
    } else {
        const int64_t g8 = B * H * ceil_div(N, 8 * 32);   // workgroups at Br = 256
        const bool eight = N >= 2048 && (g8 >= 2 * kCus || g8 % kCus == 0);
        p.waves = eight ? 8 : 4;
        p.block_k = eight ? 128 : (d == 128 ? 64 : 128);
        if (eight && causal && d == 128) {   // see above: three waves per SIMD
            p.waves = 4;
            p.block_k = 32;
        }
        if (!eight && !causal && d == 128) {
            // rounds x workgroups per CU, in units of one 128-row workgroup's work
            const int64_t g4 = B * H * ceil_div(N, 4 * 32);
            if (ceil_div(g4, 3 * kCus) * 3 < ceil_div(g4, 2 * kCus) * 2) p.block_k = 32;
            if (N < 2048 && g4 >= 2 * kCus) p.block_k = 32;
        }
        if (!eight && !causal && d == 64 && N < 2048 && B * H * ceil_div(N, 4 * 32) >= 2 * kCus)
            p.block_k = 64;   // d = 64 short heads: 64-key tiles, three workgroups per CU
    }
    p.block_q = p.waves * p.rows_per_wave / p.wave_kv_splits;
    p.lds_bytes = fwd_lds_bytes(dtype, (int)d, p.block_k, fwd_stages((int)d, p.waves, causal));
    p.grid = B * H * ceil_div(N, p.block_q);
    return p;
}

// Workgroups of a bf16/fp16 forward plan resident per CU (the kernels' launch bounds).
inline int fwd_per_cu(int64_t d, int block_k, int waves) {
    return waves == 8 ? 1 : (block_k * d == 32 * 128 ? 3 : 2);
}

// Key split of the last query block of each head (fa_plan.tail_kv_splits).  A last block of at
// most 32 rows leaves all but its first wave idle while that one sweeps every key tile; the
// non-causal 4-wave kernels can instead give those rows to all four waves, each taking a
// quarter of the tiles.  Measured interleaved against the plain kernel: 10-15% faster when
// the whole grid is resident at once (B2 H8 N4097 d128 165 -> 148 us, B2 H4 N8193 321 -> 272
// us, B2 H8 N4097 d64 105 -> 89 us), where the one busy wave of the last block holds up its
// CU; 0.6-6.5% slower when the grid takes more than one round (B8 H16 N1025 79 -> 85 us),
// and slower with few key tiles (each wave then waits out a copy latency per tile).  On the
// 8-wave plans (four of the eight waves splitting, the LDS holding four V tiles) it measured
// within -6% and +2% of the plain kernel: with 128-key tiles each wave's K loads, six in
// flight from a wave that runs alone, took about 5.6 us per tile.
// On the 8-wave plans the answer is the tail-first split count S (above), when the rows
// qualify, the problem is self-attention (Nk = N) and the grid it leaves costs less.
inline int fwd_tail_kv_splits(const fa_plan& p, int dtype, int64_t B, int64_t H, int64_t N, int64_t Nk,
                              int64_t d, int causal) {
    if (dtype == FA_F32 || causal || p.kv_splits > 1 || N <= 0) return 1;
    if (p.waves == 8) {
        if (Nk != N) return 1;
        const int s = tail_first_splits(B, H, N, d);
        if (s <= 1) return 1;
        const double plain = grid_time(B * H * ceil_div(N, 256), 1.0, 1, kEff8);
        const double first = grid_time(B * H * (N / 256), 1.0, 1, kEff8) + tail_first_cost(B, H, N, d, s);
        return first < plain ? s : 1;
    }
    if (p.waves != 4) return 1;
    const int64_t last_rows = N - (ceil_div(N, p.block_q) - 1) * p.block_q;
    if (last_rows > 32 || ceil_div(Nk, p.block_k) < 32) return 1;
    if (p.grid > (int64_t)fwd_per_cu(d, p.block_k, p.waves) * kCus) return 1;
    return 4;
}

// Whether a (d, Bc, waves) forward kernel is compiled for this dtype (the shapes the
// dispatch in fa_fwd_kernel.hip launches).  fp32 has one: 32-key tiles, 4 waves.
inline bool fwd_variant_compiled(int dtype, int64_t d, int block_k, int waves) {
    if (dtype == FA_F32) return block_k == 32 && waves == 4;
    if (d == 128) return (block_k == 128 && waves == 8) || (block_k == 64 && waves == 4) || (block_k == 32 && waves == 4);
    if (d == 64) return (block_k == 128 && waves == 8) || (block_k == 128 && waves == 4) || (block_k == 64 && waves == 4);
    return false;
}

// Query rows per workgroup of a variant: 32 per wave for bf16/fp16; 32 in all for fp32,
// whose four waves share their rows and split the key tiles.
inline int fwd_block_q(int dtype, int waves) { return dtype == FA_F32 ? 32 : 32 * waves; }

// Parses "Br,Bc,W" (three positive decimal integers, nothing else).  Returns false if
// malformed.
inline bool parse_tile_override(const char* s, int* br, int* bc, int* w) {
    int v[3];
    for (int i = 0; i < 3; ++i) {
        if (*s < '0' || *s > '9') return false;
        long x = 0;
        while (*s >= '0' && *s <= '9') {
            x = x * 10 + (*s++ - '0');
            if (x > 1 << 20) return false;
        }
        v[i] = (int)x;
        if (i < 2 && *s++ != ',') return false;
    }
    if (*s != 0) return false;
    *br = v[0], *bc = v[1], *w = v[2];
    return true;
}

// The chooser's plan with a measured-tuning override applied: tile = "Br,Bc,W" (or NULL /
// empty for none) replaces Br, Bc and the wave count when it names a compiled variant for
// this dtype and head dim.  Returns false (plan untouched) when it does not.
inline bool apply_tile_override(fa_plan* p, const char* tile, int64_t B, int64_t H, int64_t N, int64_t d,
                                int dtype, int causal) {
    if (!tile || !*tile) return true;
    int br, bc, w;
    if (!parse_tile_override(tile, &br, &bc, &w)) return false;
    if (!fwd_variant_compiled(dtype, d, bc, w) || br != fwd_block_q(dtype, w)) return false;
    p->block_q = br;
    p->block_k = bc;
    p->waves = w;
    p->rows_per_wave = 32;
    p->wave_kv_splits = dtype == FA_F32 ? 4 : 1;
    p->lds_bytes = fwd_lds_bytes(dtype, (int)d, bc, fwd_stages((int)d, w, causal));
    p->grid = B * H * ceil_div(N, br);
    return true;
}

// Sets the plan's last-block key split for Nk keys per head, and the grid it launches (the
// 8-wave launch of a tail-first plan covers the full 256-row blocks only).
inline void finalize_tail(fa_plan* p, int dtype, int64_t B, int64_t H, int64_t N, int64_t Nk, int64_t d,
                          int causal) {
    p->tail_kv_splits = fwd_tail_kv_splits(*p, dtype, B, H, N, Nk, d, causal);
    p->grid = B * H * (p->waves == 8 && p->tail_kv_splits > 1 ? N / p->block_q : ceil_div(N, p->block_q));
}

}  // namespace fa

// Launchers implemented in fa_fwd_kernel.hip.  Return 0 on success or the
// hipError_t of the launch.
int fa_launch_fwd(const fa::FwdArgs& a, const fa_plan& plan, int dtype, int d, int causal,
                  hipStream_t stream);
// Split-KV forward (bf16/fp16, non-causal): a.splits > 1, a.o_part / a.lse_part set;
// launches the partial kernel over a's grid and then the merge of m's rows.
int fa_launch_fwd_splitkv(const fa::FwdArgs& a, const fa::MergeArgs& m, int dtype, int d, hipStream_t stream);
// rows = B*H*N.  Launches the preprocess, dQ and dK/dV kernels in stream order.
int fa_launch_bwd(const fa::BwdArgs& a, int64_t rows, int dtype, int d, int causal, hipStream_t stream);
