// Fused attention forward for gfx950 (MI355X, CDNA4).
//
// One workgroup computes Br query rows of one (batch, head).  It keeps its Q rows in
// registers as MFMA operands and streams K/V tiles of Bc keys through LDS (two
// stages), keeping per query row a running maximum m, a running exp-sum l and an
// unnormalised fp32 accumulator O, all rescaled by 2^(m_old - m_new) when the
// maximum moves.  S and P live only in registers; O is divided by l once at the end
// and written with LSE = m + ln l.  This is the online softmax of
// "从零理解Flash Attention中的online softmax" (section 3.1), in the loop order of
// FlashAttention-2 ("FlashAttention 硬件感知计算剖析", section 四.2: query blocks
// outer, each output written once, normalisation deferred to the end as in the
// FA2 section 2.1.2 of the FA1/FA2 comparison page), parallel over
// (batch, head, query block).
//
// CDNA4 mapping (not the pages' CUDA design):
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_{bf16,f16}:
//    K is the A operand (32 keys x 16 dims, from LDS), Q^T the B operand (kept in
//    VGPRs for the whole loop).  In the 32x32 accumulator layout lane L holds column
//    L%32 -- one query -- and 16 key rows, so a row max/sum is an in-lane reduction
//    plus one exchange with lane L^32 (v_permlane32_swap).
//  * The probabilities P^T are used straight from those accumulator registers as the
//    B operand of O^T += V^T P^T (after packing to bf16/fp16): the MFMA's contraction
//    index is permuted to the keys each lane holds, and the A operand (V^T) is gathered
//    from row-major V in LDS in the same key order by two transposing LDS reads
//    (ds_read_b64_tr_b16).  No LDS round trip for P.
//  * O^T's accumulator also has one query per lane, so the per-row rescale is a
//    multiply by a per-lane scalar.
//  * P is formed with the running maximum m as it stands; no per-tile row maximum is
//    taken.  Exact softmax does not depend on m (the same m is used for l, O and LSE),
//    which only has to keep P finite and in range: a tile is redone with its own maximum,
//    and O and l rescaled, only when a row's sum of P over the tile leaves [0, 2^15] --
//    the first tile (m = -inf) or a maximum that jumped.  In bf16 the redone tile sets m 8
//    above its maximum (P <= 2^-8 there; bf16 keeps fp32's exponent range), so the next
//    redo needs a jump of more than 23.
//  * LDS tiles use an XOR swizzle of 16-byte chunks so the 16 lanes that read one
//    chunk column of consecutive rows hit distinct banks.
//  * Workgroup ids are remapped so consecutive query blocks of one head land on the
//    same XCD (hardware dispatch is round-robin over the 8 XCDs) and share its L2.
//
// fp32 inputs use v_mfma_f32_32x32x2_f32 with the same transposed formulation.

#include "fa_device.h"

namespace fa {

// ------------------------------------------------------- bf16 / fp16 kernel ---
//
// WAVES waves x 32 query rows (Br = 32 WAVES): 4 waves and two workgroups per CU (three
// with 32-key tiles at d = 128 or 64-key tiles at d = 64), or 8 waves and one workgroup
// per CU -- two or three waves per SIMD, so one wave's softmax VALU work overlaps
// another's MFMAs.  K/V tiles of BC keys are copied
// HBM -> LDS with buffer_load_dwordx4 ... lds (no staging registers), two stages, one
// barrier per tile.  Rows past N read as zeros (buffer range check) and
// their scores are masked to -inf, so they contribute exactly 0.  PP (8 waves,
// non-causal d = 64) selects the ping-pong schedule described at its loop: three stages,
// the two waves of each SIMD half a tile apart.
//
// V operand of O^T += V^T P^T: lane L needs V[key][d] for d = 32db + L%32 and the 8
// keys the P^T accumulator registers of lane L hold.  V stays row-major in LDS and
// ds_read_b64_tr_b16 gathers it: within each group of 16 lanes, lane c of the group
// receives element c%4 of the 8-byte pieces addressed by lanes 4e + c/4 (e = 0..3),
// so if lane r of the group addresses V[k0 + r/4][d0 + 4(r%4) .. +3], lane c gets
// V[k0 + e][d0 + c] for e = 0..3: four keys of its own column.

// Merges S normalised partials (O_s, LSE_s) of one row by their log-sum-exp, the two-block
// merge of "FlashAttention 硬件感知计算剖析" (section 二) generalised to S parts:
//     LSE = ln sum_s e^{LSE_s},   O = sum_s e^{LSE_s - LSE} O_s.
// The calling lane owns dims 8 part .. 8 part + 7 (two 16-byte loads per partial); partial s
// of the row sits at o_part + s * po_split (D floats) and lse_part[s * pl_split].  The parts
// are taken eight at a time, their loads issued together, and folded in with a running
// maximum (the same merge applied chunk by chunk), so a row costs one pass over them.  The
// lane writes its 8 dims of O; lse (if not null) gets the row's LSE.
template <typename T, int D>
__device__ __forceinline__ void merge_partials(const float* __restrict__ o_part, const float* __restrict__ lse_part,
                                               int64_t po_split, int64_t pl_split, int splits, int part,
                                               T* __restrict__ o_row, float* __restrict__ lse) {
    constexpr int CH = 8;
    float mx = -INFINITY, den = 0.f;
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < splits; s0 += CH) {
        float l[CH];
        f32x4 x0[CH], x1[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            l[i] = -INFINITY;
            x0[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            x1[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (s0 + i < splits) {
                const int64_t s = s0 + i;
                l[i] = lse_part[s * pl_split];
                x0[i] = *reinterpret_cast<const f32x4*>(o_part + s * po_split + part * 8);
                x1[i] = *reinterpret_cast<const f32x4*>(o_part + s * po_split + part * 8 + 4);
            }
        }
        float cm = mx;
#pragma unroll
        for (int i = 0; i < CH; ++i) cm = fmaxf(cm, l[i]);
        if (cm == -INFINITY) continue;   // only empty key ranges so far (LSE_s = -inf, O_s = 0)
        const float r = __expf(mx - cm);   // 0 while mx = -inf
        den *= r;
        a0 *= r;
        a1 *= r;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const float w = __expf(l[i] - cm);
            den += w;
            a0 += w * x0[i];
            a1 += w * x1[i];
        }
        mx = cm;
    }
    const float inv = 1.f / den;
    a0 *= inv;
    a1 *= inv;
    u32x4 out;
    out[0] = Elt<T>::pack2(a0[0], a0[1]);
    out[1] = Elt<T>::pack2(a0[2], a0[3]);
    out[2] = Elt<T>::pack2(a1[0], a1[1]);
    out[3] = Elt<T>::pack2(a1[2], a1[3]);
    *reinterpret_cast<u32x4*>(o_row + part * 8) = out;
    if (lse) *lse = mx + __logf(den);
}

template <typename T, int D, int BC, int WAVES, bool CAUSAL, bool SPLIT = false, bool PP = false, bool TAIL = false>
__global__ __launch_bounds__(64 * WAVES, WAVES == 4 ? (BC * D == 32 * 128 ? 3 : 2) : 1) void fwd_kernel(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)   // buffer-resource types exist only in the device pass
    constexpr int NT = 64 * WAVES, QPW = 32, BR = WAVES * QPW;
    constexpr int KB = BC / 32;       // 32-key row blocks of S^T per tile
    constexpr int DB = D / 32;        // 32-dim row blocks of O^T
    constexpr int DS = D / 16;        // k-steps of S^T = K Q^T
    constexpr int KS = BC / 16;       // k-steps of O^T += V^T P^T
    constexpr int RB = D * 2;         // bytes per K/V row
    constexpr int CPR = D / 8;        // 16-byte chunks per row
    constexpr int TILE = BC * RB;     // bytes of one K (or V) tile
    constexpr int LOADS = TILE / (NT * 16);   // direct loads per thread per tile, K or V
    // fp16: the fp16-rounded row sum serves O and the LSE alike (its relative error, at most
    // 2^-11 per term, moves the LSE by less than 1e-3); bf16 keeps an fp32 sum for the LSE
    constexpr bool ONE_SUM = __is_same(T, _Float16);
    static_assert(LOADS >= 1 && TILE % (NT * 16) == 0, "tile must be whole 4 KiB blocks");
    static_assert(!(SPLIT && CAUSAL), "split-KV is non-causal");
    static_assert(!PP || (WAVES == 8 && !CAUSAL && !SPLIT), "ping-pong: 8 waves, non-causal");
    // TAIL: on 4 waves the last-block key split; on 8 waves the merge of the last rows
    // computed ahead of the launch (tail first)
    static_assert(!TAIL || (!CAUSAL && !SPLIT), "last-block variants: non-causal");

    // A stage is a K tile and a V tile.  Each stage is an array of its own, so the compiler
    // can prove that the copies into one stage do not alias the reads of the other and adds no
    // wait for them.  The 8-wave plans' stages (32 KiB tiles at d = 128, three stages in the
    // ping-pong schedule) reach past 64 KiB, where a read's position no longer fits the 16-bit
    // offset field of ds_read and every read would add it to its address register; there the
    // K and V tiles are arrays of their own, K first, so the K reads of every stage lie in the
    // first 64 KiB, and the V reads take their tiles' position in their base registers.
    struct Stage {
        lds_u8* k;
        lds_u8* v;
    };
    constexpr bool kSplitKV = WAVES == 8;
    Stage stage0, stage1, stage2{nullptr, nullptr};   // (stage2: the ping-pong schedule's third)
    if constexpr (kSplitKV) {
        __shared__ __attribute__((aligned(1024))) unsigned char k0_raw[TILE];
        __shared__ __attribute__((aligned(1024))) unsigned char k1_raw[TILE];
        if constexpr (PP) {
            __shared__ __attribute__((aligned(1024))) unsigned char k2_raw[TILE];
            __shared__ __attribute__((aligned(1024))) unsigned char v2_raw[TILE];
            stage2 = Stage{(lds_u8*)k2_raw, (lds_u8*)v2_raw};
        }
        __shared__ __attribute__((aligned(1024))) unsigned char v0_raw[TILE];
        __shared__ __attribute__((aligned(1024))) unsigned char v1_raw[TILE];
        stage0 = Stage{(lds_u8*)k0_raw, (lds_u8*)v0_raw};
        stage1 = Stage{(lds_u8*)k1_raw, (lds_u8*)v1_raw};
    } else {
        __shared__ __attribute__((aligned(1024))) unsigned char stage0_raw[2 * TILE];
        __shared__ __attribute__((aligned(1024))) unsigned char stage1_raw[2 * TILE];
        stage0 = Stage{(lds_u8*)stage0_raw, (lds_u8*)stage0_raw + TILE};
        stage1 = Stage{(lds_u8*)stage1_raw, (lds_u8*)stage1_raw + TILE};
    }
    // the four tile arrays of stages 0 and 1, in turn (staging areas of the epilogue and the
    // last-block key split)
    auto area = [&](int i) -> lds_u8* { return i == 0 ? stage0.k : i == 1 ? stage0.v : i == 2 ? stage1.k : stage1.v; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keep it scalar
    const int h = lane >> 5, l32 = lane & 31;
    const int N = a.n, NK = a.nk;   // query rows, keys (equal unless a split-KV call differs)
    // ping-pong: waves w and w + 4 share a SIMD (the dispatcher deals a workgroup's waves
    // round-robin over its four SIMDs); the late group runs half a tile behind the early one
    const bool late = PP && wave >= 4;

    const int bid = remap_xcd(blockIdx.x, a.n_blocks);
    // split-KV: the splits of one query block are neighbours in the grid (same XCD, L2)
    const int nsplit = SPLIT ? a.splits : 1;
    const int bh = bid / (a.n_qblk * nsplit);
    const int rem = bid - bh * (a.n_qblk * nsplit);
    int qblk = rem / nsplit;
    const int split = rem - qblk * nsplit;
    if (CAUSAL) qblk = a.n_qblk - 1 - qblk;   // longest rows first
    if (SPLIT) qblk += a.qblk0;
    const int64_t head = (int64_t)bh * N * D, khead = (int64_t)bh * NK * D;
    const T* __restrict__ Qh = reinterpret_cast<const T*>(a.q) + head;
    const T* __restrict__ Kh = reinterpret_cast<const T*>(a.k) + khead;
    const T* __restrict__ Vh = reinterpret_cast<const T*>(a.v) + khead;
    T* __restrict__ Oh = reinterpret_cast<T*>(a.o) + head;
    float* __restrict__ Lh = a.lse + (int64_t)bh * N;

    // Tail first (the 8-wave TAIL variants): the last rows of each head (from row part_row0
    // on) were computed ahead of this launch into partials parked in the head's first O
    // rows; the head's first block merges them into those rows' O and LSE before its own
    // outputs overwrite the partials (its epilogue comes after many tile barriers, by which
    // time every merge load of the workgroup has returned).
    if constexpr (TAIL && WAVES == 8) {
        if (qblk == 0) {
            const int part = tid % (D / 8);
            for (int i = tid / (D / 8); i < N - a.part_row0; i += NT / (D / 8))
                merge_partials<T, D>(a.o_part + bh * a.po_head + (int64_t)i * D, a.lse_part + bh * a.pl_head + i,
                                     a.po_split, a.pl_split, a.splits, part, Oh + (int64_t)(a.part_row0 + i) * D,
                                     part == 0 ? Lh + a.part_row0 + i : nullptr);
        }
    }

    // TAIL: a block whose rows all fit in its first wave (the one-row last block when N is one
    // more than a multiple of Br; one-query decoding) would leave its other waves idle while
    // the first sweeps every key.  There every wave (four: the two stages hold four V tiles)
    // takes the first wave's rows and a quarter of the key tiles, and the four partial results
    // are merged through LDS at the end.  A variant of its own, launched where it measured
    // faster, so the others keep their code.
    constexpr bool kTailSplit = TAIL && WAVES == 4;
    const bool tail_split = kTailSplit && N - qblk * BR <= QPW;
    const int q_wave = qblk * BR + (tail_split ? 0 : wave * QPW);   // first query row of this wave
    const int query = q_wave + l32;              // the query this lane's columns belong to
    // A wave whose 32 rows all lie past N (the last query block; one-query decoding) skips
    // the tile work, not the copies or barriers: its rows are never stored.
    const bool has_rows = q_wave < N;
    const float c = a.c;

    // ---- Q^T fragments (B operand): query row `query`, dims 16s + 8h .. +7
    u32x4 qf[DS];
    {
        const int row = query < N ? query : 0;
#pragma unroll
        for (int s = 0; s < DS; ++s)
            qf[s] = *reinterpret_cast<const u32x4*>(Qh + (int64_t)row * D + s * 16 + h * 8);
    }

    // ---- per-lane LDS offsets (tile and stage offsets are added as immediates)
    int koff[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) koff[s] = l32 * RB + 16 * ((2 * s + h) ^ swz<CPR>(l32));
    int voff[2][DB];
    {
        const int g = lane >> 4, r = lane & 15;
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int key = 8 * aa + 4 * h + (r >> 2);
                const int dim = 32 * db + 16 * (g & 1) + 4 * (r & 3);
                // (from the V tile; from the stage's K tile where V follows it in one array)
                voff[aa][db] = (kSplitKV ? 0 : TILE) + key * RB + 16 * ((dim >> 3) ^ swz<CPR>(key)) + 2 * (dim & 7);
            }
    }

    // ---- direct HBM -> LDS copy of tile j into a stage, through buffer resources that
    // cover exactly this head's K (V): reads past row NK - 1 return zeros, so the ragged
    // last tile needs no special case (its padded keys are also masked to -inf).
    // Wave w, copy i fills the 1 KiB block i*4 + w of the tile; lane L's 16 bytes land
    // at block + 16 L, i.e. row `row`, swizzled chunk `ch`.  The tile offset is added to
    // the per-lane (VGPR) offset, not passed as the scalar offset, so the buffer's range
    // check sees the full byte offset whichever of the two it covers.
    const int head_bytes = NK * D * 2;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, head_bytes, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, head_bytes, kBufferRsrcWord3);
    int src_off[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int off = i * (NT * 16) + wave * 1024 + lane * 16;   // byte offset in the tile
        const int row = off / RB;
        const int ch = ((off % RB) >> 4) ^ swz<CPR>(row);
        src_off[i] = row * RB + ch * 16;
    }
    // s_waitcnt immediate for vmcnt(2 LOADS) -- one tile's K and V copies still in flight --
    // in the gfx9 encoding (vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt left unwaited)
    constexpr int kTileLoads = 2 * LOADS;
    static_assert(kTileLoads < 64, "vmcnt is six bits");
    constexpr unsigned kWaitOneTileInFlight = 0x0F70u | (kTileLoads & 15) | ((kTileLoads >> 4) << 14);
    auto issue_tile = [&](int j, const Stage& st) {
        const int soff = j * BC * RB;
#if defined(FA_LDS_POISON)
        // Debug build: the 16 bytes each copy below will deliver first hold NaN (all-ones
        // bits, NaN in bf16, fp16 and fp32), so a read that races its copy -- a missing wait
        // or barrier -- turns into NaN outputs instead of stale, plausible data.
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int at = i * (NT * 16) + wave * 1024 + lane * 16;
            *reinterpret_cast<lds_u32x4*>(st.k + at) = u32x4{~0u, ~0u, ~0u, ~0u};
            *reinterpret_cast<lds_u32x4*>(st.v + at) = u32x4{~0u, ~0u, ~0u, ~0u};
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the poison lands before the copies
#endif
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int at = i * (NT * 16) + wave * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)(st.k + at), 16,
                                                     src_off[i] + soff, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)(st.v + at), 16,
                                                     src_off[i] + soff, 0, 0, 0);
        }
    };

    // ---- running state
    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int t = 0; t < 16; ++t) o[db][t] = 0.f;
    float m = -INFINITY, lsum = 0.f, lrnd = 0.f;
    bool max_first = false;   // the next tile takes its maximum before forming P
    // bf16 causal d = 64, 8 waves: the O divisor (the sum of P as rounded for the MFMA) comes
    // from the matrix cores, as row 0 of one more 32-row block of O^T whose V^T operand is a
    // row of ones (lanes 0 and 32 hold its keys) -- KS more MFMAs per tile on a pipe this
    // VALU-bound kernel leaves two thirds idle, instead of 8 v_dot2 per 16 scores (3% faster
    // at B4 H16 N4096; the ping-pong kernel measured no gain and keeps the v_dot2 sum).
    constexpr bool kSumOnMfma = D == 64 && WAVES == 8 && !ONE_SUM && CAUSAL;
    f32x16 osum;
    u32x4 ones{0u, 0u, 0u, 0u};
    if constexpr (kSumOnMfma) {
#pragma unroll
        for (int t = 0; t < 16; ++t) osum[t] = 0.f;
        if (l32 == 0) ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    }

    int n_tiles = (NK + BC - 1) / BC;
    if (CAUSAL) n_tiles = min(n_tiles, (min(N, (qblk + 1) * BR) + BC - 1) / BC);
    int t0 = 0;   // first key tile of this workgroup
    if (SPLIT) {
        t0 = split * a.tiles_per_split;
        n_tiles = min(n_tiles, t0 + a.tiles_per_split);
    }

    u32x4 pf[KS];   // P of the current tile, packed: the B operand of O^T += V^T P^T
    // S, the masks, P and the row sums of tile j; kread(i) gives the K fragment of k-step i
    auto qk_soft_with = [&](int j, auto kread, int jfirst) __attribute__((always_inline)) {
        const int kbase = j * BC;
        // MFMA-heavy stretches run at raised wave priority, so the SIMD issues them ahead of
        // the other wave's VALU work (measured 0.4-3% faster in every variant).
        __builtin_amdgcn_s_setprio(1);
        // ---- S^T = K_j Q^T
        f32x16 s[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int t = 0; t < 16; ++t) s[kb][t] = 0.f;
        // One 32-key block at a time: its DS k-steps run back to back on one accumulator, so
        // each MFMA takes the previous one's result as its C operand directly.  Round-robin
        // over the KB accumulators measured slower (a bare MFMA loop on gfx950 runs at 71%
        // busy with 2 or 4 interleaved accumulators, 87% with 1 or 8).  K fragments are read
        // KPF steps ahead; the schedule barriers keep the compiler from interleaving again.
        constexpr int NQK = KB * DS, KPF = 6;
        u32x4 kf[KPF + 1];
#pragma unroll
        for (int i = 0; i < KPF; ++i) kf[i] = kread(i);
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
            if (i + KPF < NQK) kf[(i + KPF) % (KPF + 1)] = kread(i + KPF);
            s[i / DS] = Elt<T>::mma(kf[i % (KPF + 1)], qf[i % DS], s[i / DS]);
            __builtin_amdgcn_sched_barrier(0);
        }

        __builtin_amdgcn_s_setprio(0);
        // ---- masks: keys past NK (tail tile), keys after the query (causal)
        const bool ragged = kbase + BC > NK;
        const bool diag = CAUSAL && (kbase + BC - 1 > q_wave);
        if (ragged || diag) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const int key = kbase + kb * 32 + 8 * (t >> 2) + 4 * h + (t & 3);
                    bool drop = key >= NK;
                    if (CAUSAL) drop = drop || key > query;
                    if (drop) s[kb][t] = -INFINITY;
                }
        }

        // ---- P = 2^(s*c - m), packed; the O divisor sums the rounded values, LSE the fp32
        // ones (fp16: the rounded sum serves both).  P is first formed with the running
        // maximum m as it stands: the exact softmax does not depend on m, which only has to
        // keep P finite and in range.  A tile is redone with its own maximum (plus the bf16
        // headroom) when some row's tile sum leaves [0, 2^15] -- the first tile (m = -inf),
        // or a row maximum that jumped by more than 15 (bf16: 23) in base-2 units.
        float acc0, acc1, racc0, racc1;
        auto make_p = [&](float neg_m) {
            acc0 = 0.f, acc1 = 0.f, racc0 = 0.f, racc1 = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                float p[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) p[t] = fast_exp2(__builtin_fmaf(s[kb][t], c, neg_m));
                if constexpr (!ONE_SUM) {
                    // (from the first terms: 0 + p is an add the compiler may not drop)
#pragma unroll
                    for (int t = 0; t < 16; t += 2) {
                        acc0 = kb == 0 && t == 0 ? p[t] : acc0 + p[t];
                        acc1 = kb == 0 && t == 0 ? p[t + 1] : acc1 + p[t + 1];
                    }
                }
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    u32x4 f;
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        f[w] = Elt<T>::pack2(p[8 * half + 2 * w], p[8 * half + 2 * w + 1]);
                        if constexpr (!kSumOnMfma) {
                            if (w & 1) racc1 = Elt<T>::sum2(f[w], racc1);
                            else racc0 = Elt<T>::sum2(f[w], racc0);
                        }
                    }
                    pf[2 * kb + half] = f;
                }
            }
        };
        // The workgroup's first tile meets m = -inf, which would fail the test anyway: it takes
        // its own maximum at once.  (NaN, from -inf scores against m = -inf, fails the test.)
        // Non-causal bf16: after a tile whose maximum jumped, the next one does the same; on
        // heads whose maxima keep jumping (one-hot or large scores) most first attempts would
        // fail.  (The causal and fp16 kernels measured slower with it.)
        constexpr bool kMaxFirst = !CAUSAL && !ONE_SUM;
        bool redo = true;
        if (j != jfirst && !(kMaxFirst && max_first)) {
            make_p(-m);
            redo = __builtin_amdgcn_ballot_w64(!((ONE_SUM ? racc0 + racc1 : acc0 + acc1) <= kMaxTileSum)) != 0;
        }
        if (redo) {
            float x0 = -INFINITY, x1 = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int t = 0; t < 16; t += 4) {
                    x0 = vmax3(x0, s[kb][t], s[kb][t + 1]);
                    x1 = vmax3(x1, s[kb][t + 2], s[kb][t + 3]);
                }
            const float xm = pair_max(__builtin_elementwise_maximum(x0, x1));
            if constexpr (kMaxFirst) max_first = j != jfirst && __builtin_amdgcn_ballot_w64(xm * c > m + 12.f) != 0;
            const float mx = ONE_SUM ? xm * c : __builtin_fmaf(xm, c, a.m_headroom);
            const float mnew = fmaxf(m, mx);
            const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mnew);
            m = mnew;
            lsum *= alpha;
            lrnd *= alpha;
            if constexpr (kSumOnMfma) osum[0] *= alpha;   // (its other elements stay 0)
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int t = 0; t < 16; ++t) o[db][t] *= alpha;
            make_p(-m);
        }
        if constexpr (!ONE_SUM) lsum += acc0 + acc1;
        if constexpr (!kSumOnMfma) lrnd += racc0 + racc1;
    };
    auto qk_soft = [&](int j, const lds_u8* sbase) __attribute__((always_inline)) {
        qk_soft_with(j, [&](int i) { return lds_read16(sbase, koff[i % DS] + (i / DS) * 32 * RB); }, t0);
    };
    // O^T += V_j^T P^T; vo(aa, db) gives the lane's LDS offsets of V_j from sbase
    auto pv_from = [&](const lds_u8* sbase, auto vo) __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(1);
        // (same order: the KS k-steps of one 32-dim block of O^T back to back, V^T fragments
        // gathered VPF steps ahead)
        {
            constexpr int NPV = KS * DB, VPF = 4;
            auto vread = [&](int i) {
                const int db = i / KS, ks = i % KS;
                const u32x2 lo = lds_read_tr(sbase, vo(0, db) + ks * 16 * RB);
                const u32x2 hi = lds_read_tr(sbase, vo(1, db) + ks * 16 * RB);
                return u32x4{lo[0], lo[1], hi[0], hi[1]};
            };
            u32x4 vf[VPF + 1];
#pragma unroll
            for (int i = 0; i < VPF; ++i) vf[i] = vread(i);
#pragma unroll
            for (int i = 0; i < NPV; ++i) {
                if (i + VPF < NPV) vf[(i + VPF) % (VPF + 1)] = vread(i + VPF);
                o[i / KS] = Elt<T>::mma(vf[i % (VPF + 1)], pf[i % KS], o[i / KS]);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (kSumOnMfma) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) osum = Elt<T>::mma(ones, pf[ks], osum);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };
    auto pv = [&](const lds_u8* sbase) __attribute__((always_inline)) {
        pv_from(sbase, [&](int aa, int db) { return voff[aa][db]; });
    };
    // Split layout: the V reads address from stage 0's K tile, with V's position (past the
    // first 64 KiB) inside the base registers vrel, which an empty asm makes opaque so the
    // compiler cannot split the constant back out of them; what remains, the stage's and the
    // k-step's offsets, fits the instruction's offset field.
    int vrel[2][DB];
    if constexpr (kSplitKV) {
        const int vk = (int)(uintptr_t)stage0.v - (int)(uintptr_t)stage0.k;
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                vrel[aa][db] = voff[aa][db] + vk;
                asm volatile("" : "+v"(vrel[aa][db]));
            }
    }
    auto pv_stage = [&](const Stage& st) __attribute__((always_inline)) {
        if constexpr (kSplitKV) {
            const int dv = (int)(uintptr_t)st.v - (int)(uintptr_t)stage0.v;
            pv_from(stage0.k, [&](int aa, int db) { return vrel[aa][db] + dv; });
        } else {
            pv(st.k);
        }
    };
    auto compute_tile = [&](int j, const Stage& st) __attribute__((always_inline)) {
        qk_soft(j, st.k);
        pv_stage(st);
    };

    // Ping-pong schedule (d = 64, where the softmax takes longer than the MFMAs): every wave
    // runs qk_soft(j) then pv(j) per tile, but the two groups take the tile barrier at
    // different points -- the early group after pv(j), the late group between qk_soft(j) and
    // pv(j).  Each wave passes one barrier per tile, and a barrier event pairs the early
    // group's end of tile j with the late group's middle of tile j, so the late group runs
    // half a tile behind and each group's MFMAs fall in the other's softmax.
    // Stages: tile j + 1 is copied, at the start of step j, into the stage of tile j - 2; both
    // groups are done with it by then (the late group's last read, V of tile j - 2, comes
    // before the barrier that ends its step j - 1).  So three stages, the loop unrolled by
    // three to keep every stage a distinct array at compile time.
    auto pp_step = [&](int j, const Stage& cur) __attribute__((always_inline)) {
        if (has_rows) qk_soft(j, cur.k);
        if (late) {
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's copies have landed
            __syncthreads();
        }
        if (has_rows) pv_stage(cur);
        if (!late) {
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
        }
    };
    if (tail_split) {
        if constexpr (kTailSplit) {
            // Wave w takes key tiles [tb, te).  Its V tiles go HBM -> LDS into a region of its
            // own (one tile; the two stages hold four) and its K fragments straight into
            // registers, read as the score MFMAs consume them (through the same prefetch window
            // as the LDS reads of the other blocks), so the waves meet only at the merge.
            const int per = (n_tiles + WAVES - 1) / WAVES;
            const int tb = min(n_tiles, wave * per), te = min(n_tiles, tb + per);
            lds_u8* const region = area(wave);
            constexpr int VLOADS = TILE / 1024;   // 1 KiB copies per V tile
            auto issue_v = [&](int j) {   // row-major V tile, swizzled as in issue_tile
#if defined(FA_LDS_POISON)
#pragma unroll
                for (int i = 0; i < VLOADS; ++i)
                    *reinterpret_cast<lds_u32x4*>(region + i * 1024 + lane * 16) = u32x4{~0u, ~0u, ~0u, ~0u};
                __builtin_amdgcn_s_waitcnt(0xC07F);
#endif
#pragma unroll
                for (int i = 0; i < VLOADS; ++i) {
                    const int off = i * 1024 + lane * 16;
                    const int row = off / RB;
                    const int ch = ((off % RB) >> 4) ^ swz<CPR>(row);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)(region + i * 1024), 16,
                                                             j * BC * RB + row * RB + ch * 16, 0, 0, 0);
                }
            };
            // V offsets in the region, recomputed here from the hardware lane id (as a value the
            // compiler cannot equate with the one before the branch, so no input of this path
            // stays live across the other path's loop)
            const int tl = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
            int tvoff[2][DB];
            {
                const int g = tl >> 4, r = tl & 15, th = tl >> 5;
#pragma unroll
                for (int aa = 0; aa < 2; ++aa)
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const int key = 8 * aa + 4 * th + (r >> 2);
                        const int dim = 32 * db + 16 * (g & 1) + 4 * (r & 3);
                        tvoff[aa][db] = key * RB + 16 * ((dim >> 3) ^ swz<CPR>(key)) + 2 * (dim & 7);
                    }
            }
            if (tb < te) issue_v(tb);
            for (int j = tb; j < te; ++j) {
                // k-step i: keys j Bc + 32 (i / DS) + l32, dims 16 (i % DS) + 8 h .. + 7 -- the
                // fragment the LDS reads deliver
                qk_soft_with(j, [&](int i) {
                    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                        krs, (j * BC + (i / DS) * 32 + l32) * RB + ((i % DS) * 16 + h * 8) * 2, 0, 0));
                }, tb);
                __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this tile's V has landed
                pv_from(region, [&](int aa, int db) { return tvoff[aa][db]; });
                if (j + 1 < te) {
                    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the V reads are done
                    issue_v(j + 1);
                }
            }
            // Merge into wave 0, one partial at a time: O^T through stage 0's two tiles and the
            // row statistics through tail_stats, both in the accumulator layout, so each lane of
            // wave 0 combines the entries of the same lane of wave w.
            __shared__ float tail_stats[3 * 64];
            typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
            static_assert(DB * 4 * 64 * 16 <= 2 * TILE, "a wave's O^T fits in stage 0");
            auto opart = [&](int db, int g) {   // 16-byte slot (db, g) of this lane
                const int at = ((db * 4 + g) * 64 + lane) * 16;
                return (lds_f32x4*)(at < TILE ? stage0.k + at : stage0.v + (at - TILE));
            };
#pragma unroll 1
            for (int w = 1; w < WAVES; ++w) {
                __syncthreads();
                if (wave == w) {
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int g = 0; g < 4; ++g)
                            *opart(db, g) = f32x4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
                    tail_stats[lane] = m;
                    tail_stats[64 + lane] = lsum;
                    tail_stats[128 + lane] = lrnd;
                }
                __syncthreads();
                const float mw = tail_stats[lane];
                if (wave == 0 && mw != -INFINITY) {   // a wave without key tiles adds nothing
                    const float mn = fmaxf(m, mw);
                    const float a0 = fast_exp2(m - mn), aw = fast_exp2(mw - mn);
                    m = mn;
                    lsum = lsum * a0 + tail_stats[64 + lane] * aw;
                    lrnd = lrnd * a0 + tail_stats[128 + lane] * aw;
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const f32x4 x = *opart(db, g);
#pragma unroll
                            for (int e = 0; e < 4; ++e) o[db][4 * g + e] = o[db][4 * g + e] * a0 + x[e] * aw;
                        }
                }
            }
        }
    } else if constexpr (PP) {
        if (t0 < n_tiles) issue_tile(t0, stage0);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        for (int j = t0; j < n_tiles; j += 3) {
            if (j + 1 < n_tiles) issue_tile(j + 1, stage1);
            pp_step(j, stage0);
            if (j + 1 >= n_tiles) break;
            if (j + 2 < n_tiles) issue_tile(j + 2, stage2);
            pp_step(j + 1, stage1);
            if (j + 2 >= n_tiles) break;
            if (j + 3 < n_tiles) issue_tile(j + 3, stage0);
            pp_step(j + 2, stage2);
        }
    } else {
        // The first tile is computed ahead of the loop with the second tile's copy already in
        // flight: both are issued together and the wait covers only the first (vector-memory
        // loads complete in order), so the second copy overlaps the first one's wait as well
        // as its compute.  Heads of a few tiles are bound by these copy latencies.
        auto computes = [&](int j) { return has_rows && (!CAUSAL || j * BC <= q_wave + QPW - 1); };
        if (t0 < n_tiles) {
            issue_tile(t0, stage0);
            if (t0 + 1 < n_tiles) {
                issue_tile(t0 + 1, stage1);
                // No release fence before this barrier: it would wait for the second tile's
                // copies too, which no wave reads before the next full barrier.
                __builtin_amdgcn_s_waitcnt(kWaitOneTileInFlight);
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            } else {
                __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's LDS copies have landed
                __syncthreads();
            }
            if (computes(t0)) compute_tile(t0, stage0);
            __builtin_amdgcn_s_waitcnt(0x0F70);       // the second tile has landed
            __syncthreads();
        }
        for (int j = t0 + 1; j < n_tiles; j += 2) {
            // stage 1 holds tile j; tile j + 1 streams into stage 0 meanwhile
            if (j + 1 < n_tiles) issue_tile(j + 1, stage0);
            if (computes(j)) compute_tile(j, stage1);
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
            if (j + 1 >= n_tiles) break;
            // stage 0 holds tile j + 1
            if (j + 2 < n_tiles) issue_tile(j + 2, stage1);
            if (computes(j + 1)) compute_tile(j + 1, stage0);
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
        }
    }

    // ---- epilogue: O / l, LSE = (m + log2 l) ln 2
    if constexpr (kSumOnMfma) lrnd = osum[0];   // lanes 0-31; 0 on lanes 32-63 (row 4)
    const float lr = pair_sum(lrnd);
    const float lt = ONE_SUM ? lr : pair_sum(lsum);
    const float inv = 1.0f / lr;
    if (SPLIT) {   // normalised fp32 partials of this key range (an empty range: O 0, LSE -inf)
        if (query < N) {
            const bool empty = t0 >= n_tiles;
            const int64_t i = query - a.part_row0;
            float* orow = a.o_part + bh * a.po_head + split * a.po_split + i * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = empty ? 0.f : o[db][4 * g + e] * inv;
                    *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * g + 4 * h) = w;
                }
            if (h == 0)
                a.lse_part[bh * a.pl_head + split * a.pl_split + i] =
                    empty ? -INFINITY : (m + __builtin_amdgcn_logf(lt)) * kLn2;
        }
        return;
    }
    // O leaves through LDS: each wave writes its 32 rows there in the accumulator layout (one
    // row per lane, 8-byte pieces) and reads them back 16 bytes per lane along the rows, so
    // every global store instruction writes whole contiguous rows instead of 8-byte pieces
    // of 32 rows.  The stages are free once every wave has passed this barrier (in the
    // ping-pong schedule the late group's last P V reads a stage after its last tile barrier).
    __syncthreads();
    if (has_rows && (!tail_split || wave == 0)) {
        constexpr int WPT = BC / 32;               // waves whose 32 rows fit in one tile
        static_assert(WAVES <= 4 * WPT, "the four tiles of stages 0 and 1 stage every wave's rows");
        lds_u8* obuf;
        if constexpr (kSplitKV) obuf = area(wave / WPT) + (wave % WPT) * (QPW * RB);
        else obuf = (wave / (2 * WPT) == 0 ? stage0.k : stage1.k) + (wave % (2 * WPT)) * (QPW * RB);
        // Staging layout: 16-byte chunk c of row r sits in slot c ^ ochunk(r) and its two
        // 8-byte halves are swapped when ohalf(r) is set.  A write instruction puts one
        // 8-byte piece of each of the wave's 32 rows; with this layout the pieces of any 16
        // consecutive lanes fill 128 distinct bytes modulo 128, those of 32 lanes 256
        // distinct bytes modulo 256, and lanes r and r + 32 share a slot, so the writes are
        // free of bank conflicts however the LDS groups lanes.  A read of 16 bytes along a row
        // still covers one row's slots exactly once per group of lanes.
        auto ochunk = [](int r) { return CPR == 16 ? (r & 15) : ((r >> 1) & 7); };
        auto ohalf = [](int r) { return CPR == 16 ? ((r >> 3) ^ (r >> 4)) & 1 : (r ^ (r >> 4)) & 1; };
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = Elt<T>::pack2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv);
                w[1] = Elt<T>::pack2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
                *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
                    obuf + l32 * RB + 16 * ((4 * db + g) ^ ochunk(l32)) + 8 * (h ^ ohalf(l32))) = w;
            }
        // the wave reads back what its other lanes wrote
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        constexpr int LPR = RB / 16, RPI = 64 / LPR, NR = QPW / RPI;   // lanes per row, rows per read, reads
        const int ch = lane % LPR;
        u32x4 v[NR];
#pragma unroll
        for (int k = 0; k < NR; ++k) {   // every read in flight before the first store
            const int row = k * RPI + lane / LPR;
            v[k] = lds_read16(obuf, row * RB + 16 * (ch ^ ochunk(row)));
        }
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const int row = k * RPI + lane / LPR;
            const u32x4 x = ohalf(row) ? u32x4{v[k][2], v[k][3], v[k][0], v[k][1]} : v[k];
            if (q_wave + QPW <= N || q_wave + row < N)
                *reinterpret_cast<u32x4*>(Oh + (int64_t)(q_wave + row) * D + ch * 8) = x;
        }
        if (h == 0 && query < N) Lh[query] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
    }
#endif
}

// ---------------------------------------------------------- split-KV merge ---
//
// One row per D / 8 lanes, each lane 8 dims: merge_partials above.
template <typename T, int D>
__global__ __launch_bounds__(256) void splitkv_merge_kernel(MergeArgs a) {
    constexpr int LPR = D / 8, RPB = 256 / LPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    const int part = threadIdx.x % LPR;
    if (row >= a.rows) return;
    const int64_t bh = row / a.rows_per_head, i = row - bh * a.rows_per_head;
    const int64_t orow = bh * a.out_head + a.out_row0 + i;
    merge_partials<T, D>(a.o_part + bh * a.po_head + i * D, a.lse_part + bh * a.pl_head + i, a.po_split, a.pl_split,
                         a.splits, part, reinterpret_cast<T*>(a.o) + orow * D, part == 0 ? a.lse + orow : nullptr);
}

template <typename T, int D, int BC>
static hipError_t launch_splitkv_t(const FwdArgs& a, const MergeArgs& m, hipStream_t st) {
    hipLaunchKernelGGL((fwd_kernel<T, D, BC, 4, false, true>), dim3((unsigned)a.n_blocks), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || m.rows == 0) return e;   // (no rows: the next launch merges them)
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((splitkv_merge_kernel<T, D>), dim3((unsigned)((m.rows + RPB - 1) / RPB)), dim3(256), 0, st, m);
    return hipGetLastError();
}

// ------------------------------------------------------------- fp32 kernel ---
//
// Same transposed formulation with v_mfma_f32_32x32x2_f32: each MFMA contracts two dims
// (lane half h supplies dim 2s+h) or two keys.  fp32 inputs are small problems here, so
// the kernel is built for latency: a workgroup owns 32 query rows, and its four waves
// split the key tiles among themselves (tile j goes to wave j % 4), each keeping its own
// running m, l and O for the 32 rows and its own K/V tile in LDS.  The four partial
// states are then merged through LDS with the two-block rule of "FlashAttention
// 硬件感知计算剖析" (section 二): M = max_w m_w, l = sum_w 2^(m_w - M) l_w,
// O = sum_w (2^(m_w - M) / l) O_w, one reciprocal per row.  Four times fewer tiles run
// back to back per wave.

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_kernel_f32(FwdArgs a) {
    constexpr int NT = 256, WAVES = 4, QPW = 32, BC = 32;
    constexpr int DB = D / 32;
    constexpr int DS = D / 2;
    constexpr int LD = D + 1;        // padded row stride (floats)
    constexpr int WTILE = 2 * BC * LD;   // one wave's K and V tile (floats)
    static_assert(WAVES * WTILE >= WAVES * QPW * D + 3 * WAVES * QPW, "merge area fits the tiles");
    __shared__ float lds[WAVES * WTILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, l32 = lane & 31;
    const int N = a.n;

    const int bid = remap_xcd(blockIdx.x, a.n_blocks);
    const int bh = bid / a.n_qblk;
    int qblk = bid - bh * a.n_qblk;
    if (CAUSAL) qblk = a.n_qblk - 1 - qblk;
    const int64_t head = (int64_t)bh * N * D;
    const float* __restrict__ Qh = reinterpret_cast<const float*>(a.q) + head;
    const float* __restrict__ Kh = reinterpret_cast<const float*>(a.k) + head;
    const float* __restrict__ Vh = reinterpret_cast<const float*>(a.v) + head;
    float* __restrict__ Oh = reinterpret_cast<float*>(a.o) + head;
    float* __restrict__ Lh = a.lse + (int64_t)bh * N;

    const int q0 = qblk * QPW;       // the workgroup's (and every wave's) first query row
    const int query = q0 + l32;
    const float c = a.c;
    float* ks_ = lds + wave * WTILE;
    float* vs_ = ks_ + BC * LD;

    float qf[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = (query < N) ? Qh[(int64_t)query * D + 2 * s + h] : 0.f;

    int n_tiles = (N + BC - 1) / BC;
    if (CAUSAL) n_tiles = min(n_tiles, (min(N, q0 + QPW) + BC - 1) / BC);

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int t = 0; t < 16; ++t) o[db][t] = 0.f;
    float m = -INFINITY, lsum = 0.f;

    // A wave's next tile is fetched into registers (16 bytes per load) while it computes
    // the current one.  Lane L holds float4 number L + 64 i of the tile (row-major).
    constexpr int V4 = BC * D / 4 / 64;   // float4s per lane, K or V
    f32x4 kreg[V4], vreg[V4];
    auto fetch = [&](int j) {
#pragma unroll
        for (int i = 0; i < V4; ++i) {
            const int idx = lane + 64 * i, r = idx / (D / 4), c4 = idx % (D / 4);
            const bool ok = j * BC + r < N;
            const int64_t off = (int64_t)(ok ? j * BC + r : 0) * D + 4 * c4;
            kreg[i] = *reinterpret_cast<const f32x4*>(Kh + off);
            vreg[i] = *reinterpret_cast<const f32x4*>(Vh + off);
            if (!ok) kreg[i] = vreg[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    if (wave < n_tiles) fetch(wave);

    for (int j = wave; j < n_tiles; j += WAVES) {
        const int kbase = j * BC;
        // this wave's tile into its LDS slot; LDS operations of one wave complete in
        // order, so the reads of the previous tile are done before these writes land
#pragma unroll
        for (int i = 0; i < V4; ++i) {
            const int idx = lane + 64 * i, r = idx / (D / 4), c4 = idx % (D / 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ks_[r * LD + 4 * c4 + e] = kreg[i][e];
                vs_[r * LD + 4 * c4 + e] = vreg[i][e];
            }
        }
        if (j + WAVES < n_tiles) fetch(j + WAVES);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        f32x16 s;
#pragma unroll
        for (int t = 0; t < 16; ++t) s[t] = 0.f;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(ks_[l32 * LD + 2 * ds + h], qf[ds], s, 0, 0, 0);

#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int key = kbase + 8 * (t >> 2) + 4 * h + (t & 3);
            bool drop = key >= N;
            if (CAUSAL) drop = drop || key > query;
            if (drop) s[t] = -INFINITY;
        }
        float x = -INFINITY;
#pragma unroll
        for (int t = 0; t < 16; ++t) x = fmaxf(x, s[t]);
        const float mx = pair_max(x) * c;
        // lazy rescale: the maximum moves only when a tile exceeds it by 2^8 (P <= 256)
        if (__builtin_amdgcn_ballot_w64(mx > m + 8.0f) != 0) {
            const float mnew = fmaxf(m, mx);
            const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mnew);
            m = mnew;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int t = 0; t < 16; ++t) o[db][t] *= alpha;
        }
        const float neg_m = (m == -INFINITY) ? 0.f : -m;
        float p[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            p[t] = fast_exp2(__builtin_fmaf(s[t], c, neg_m));
            lsum += p[t];
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int key = 8 * (t >> 2) + 4 * h + (t & 3);
#pragma unroll
            for (int db = 0; db < DB; ++db)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs_[key * LD + db * 32 + l32], p[t], o[db], 0, 0, 0);
        }
    }

    // ---- merge the waves' partial states (a wave without tiles has m = -inf, l = 0, O = 0)
    const float lt = pair_sum(lsum);
    __syncthreads();                                  // every wave is done with its tiles
    float* mo = lds;                                  // [WAVES][QPW][D] partial O
    float* mm = lds + WAVES * QPW * D;                // [WAVES][QPW] m
    float* ml = mm + WAVES * QPW;                     // [WAVES][QPW] l
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int t = 0; t < 16; ++t)
            mo[(wave * QPW + l32) * D + db * 32 + 8 * (t >> 2) + 4 * h + (t & 3)] = o[db][t];
    if (h == 0) {
        mm[wave * QPW + l32] = m;
        ml[wave * QPW + l32] = lt;
    }
    __syncthreads();
    // per row: M, l, one reciprocal, and the weight 2^(m_w - M) / l of each wave's O
    float* mwt = ml + WAVES * QPW;                    // [WAVES][QPW] weights
    if (tid < QPW) {
        const int r = tid;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) M = fmaxf(M, mm[w * QPW + r]);
        float sc[WAVES], l = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float mw = mm[w * QPW + r];
            sc[w] = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
            l += sc[w] * ml[w * QPW + r];
        }
        const float inv = 1.0f / l;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) mwt[w * QPW + r] = sc[w] * inv;
        if (q0 + r < N) Lh[q0 + r] = (M + __builtin_amdgcn_logf(l)) * kLn2;
    }
    __syncthreads();
    for (int idx = tid; idx < QPW * D; idx += NT) {
        const int r = idx / D, col = idx % D;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) acc += mwt[w * QPW + r] * mo[(w * QPW + r) * D + col];
        if (q0 + r < N) Oh[(int64_t)(q0 + r) * D + col] = acc;
    }
}

// ------------------------------------------------------------------ dispatch ---

// tail: the plan's last-block variant -- on 4 waves the key split (its waves share the
// block's rows), on 8 waves the merge of the last rows computed ahead (tail first)
template <typename T, int D, int BC, int WAVES>
static hipError_t launch_t(const FwdArgs& a, int causal, bool tail, hipStream_t st) {
    const dim3 grid((unsigned)a.n_blocks), block(64 * WAVES);
    if (causal) {
        hipLaunchKernelGGL((fwd_kernel<T, D, BC, WAVES, true>), grid, block, 0, st, a);
    } else if (tail) {
        hipLaunchKernelGGL((fwd_kernel<T, D, BC, WAVES, false, false, false, true>), grid, block, 0, st, a);
    } else {
        hipLaunchKernelGGL((fwd_kernel<T, D, BC, WAVES, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

// The compiled (d, Bc, waves) shapes; the chooser only emits these.
template <typename T>
static hipError_t launch_half(const FwdArgs& a, const fa_plan& p, int d, int causal, hipStream_t st) {
    const bool tail = p.tail_kv_splits > 1;
    if (d == 128 && p.block_k == 128 && p.waves == 8) return launch_t<T, 128, 128, 8>(a, causal, tail, st);
    if (d == 64 && p.block_k == 128 && p.waves == 8) {
        if (causal) return launch_t<T, 64, 128, 8>(a, causal, false, st);
        // non-causal d = 64 on the ping-pong schedule
        if (tail)
            hipLaunchKernelGGL((fwd_kernel<T, 64, 128, 8, false, false, true, true>), dim3((unsigned)a.n_blocks), dim3(512),
                               0, st, a);
        else
            hipLaunchKernelGGL((fwd_kernel<T, 64, 128, 8, false, false, true>), dim3((unsigned)a.n_blocks), dim3(512), 0, st, a);
        return hipGetLastError();
    }
    if (d == 128 && p.block_k == 64 && p.waves == 4) return launch_t<T, 128, 64, 4>(a, causal, tail, st);
    if (d == 64 && p.block_k == 128 && p.waves == 4) return launch_t<T, 64, 128, 4>(a, causal, tail, st);
    if (d == 64 && p.block_k == 64 && p.waves == 4) return launch_t<T, 64, 64, 4>(a, causal, tail, st);
    if (d == 128 && p.block_k == 32 && p.waves == 4) return launch_t<T, 128, 32, 4>(a, causal, tail, st);
    return hipErrorInvalidConfiguration;
}

}  // namespace fa

int fa_launch_fwd_splitkv(const fa::FwdArgs& a, const fa::MergeArgs& m, int dtype, int d, hipStream_t st) {
    using namespace fa;
    hipError_t e;
    if (dtype == FA_BF16)
        e = d == 128 ? launch_splitkv_t<__bf16, 128, 64>(a, m, st) : launch_splitkv_t<__bf16, 64, 128>(a, m, st);
    else
        e = d == 128 ? launch_splitkv_t<_Float16, 128, 64>(a, m, st) : launch_splitkv_t<_Float16, 64, 128>(a, m, st);
    return (int)e;
}

int fa_launch_fwd(const fa::FwdArgs& a, const fa_plan& plan, int dtype, int d, int causal, hipStream_t st) {
    using namespace fa;
    hipError_t e;
    if (dtype == FA_BF16) {
        e = launch_half<__bf16>(a, plan, d, causal, st);
    } else if (dtype == FA_F16) {
        e = launch_half<_Float16>(a, plan, d, causal, st);
    } else {
        const dim3 grid((unsigned)a.n_blocks), block(256);
        if (d == 128) {
            if (causal) hipLaunchKernelGGL((fwd_kernel_f32<128, true>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((fwd_kernel_f32<128, false>), grid, block, 0, st, a);
        } else {
            if (causal) hipLaunchKernelGGL((fwd_kernel_f32<64, true>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((fwd_kernel_f32<64, false>), grid, block, 0, st, a);
        }
        e = hipGetLastError();
    }
    return (int)e;
}
