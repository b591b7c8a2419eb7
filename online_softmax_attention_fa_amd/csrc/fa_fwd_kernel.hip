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
//    index is permuted, and V^T is stored in LDS in the same permuted key order so the
//    A operand is one 16-byte LDS read per lane.  No LDS round trip for P.
//  * O^T's accumulator also has one query per lane, so the per-row rescale is a
//    multiply by a per-lane scalar.
//  * The maximum used for the exponent is only moved when a tile's maximum exceeds it
//    by more than 2^8 (base-2 units); exact softmax does not depend on that choice
//    (the same m is used for l, O and LSE), P stays <= 256, and the O rescale runs
//    only on the few tiles where the maximum jumps.
//  * LDS tiles use an XOR swizzle of 16-byte chunks so the 16 lanes that read one
//    chunk column of consecutive rows hit distinct banks.
//  * Workgroup ids are remapped so consecutive query blocks of one head land on the
//    same XCD (hardware dispatch is round-robin over the 8 XCDs) and share its L2.
//
// fp32 inputs use v_mfma_f32_32x32x2_f32 with the same transposed formulation.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309417f;
// Lazy-rescale threshold in base-2 exponent units (P <= 2^8).
constexpr float kRescaleThreshold = 8.0f;

// ------------------------------------------------------------------ helpers ---

template <typename T> struct Elt;
template <> struct Elt<__bf16> {
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ unsigned pack2(float x, float y) {
        f32x2 v = {x, y};
        return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
    }
    // acc + x0 + x1 for a packed pair (v_dot2 against (1, 1))
    static __device__ __forceinline__ float sum2(unsigned packed, float acc) {
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, acc, false);
    }
};
template <> struct Elt<_Float16> {
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ unsigned pack2(float x, float y) {
        f32x2 v = {x, y};
        return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2));
    }
    static __device__ __forceinline__ float sum2(unsigned packed, float acc) {
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), one, acc, false);
    }
};

// Maps the hardware workgroup id to a logical one so that the workgroups the
// dispatcher sends to one XCD (ids congruent mod 8) cover a contiguous logical range.
__device__ __forceinline__ int remap_xcd(int bid, int n) {
    const int xcd = bid % kXcds, local = bid / kXcds;
    const int per = n / kXcds, rem = n % kXcds;
    return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// Value of x in lane L^32 combined with x: returns {x[L%32], x[L%32 + 32]} in some order.
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte chunk swizzle: chunk c of row r is stored at chunk c ^ swz(r).  For any 16
// consecutive rows read at one logical chunk the physical 16-byte slots differ modulo
// 256 bytes (and the first 8 modulo 128 bytes).
template <int CPR>
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & (CPR - 1); }

__device__ __forceinline__ u32x4 lds_read16(const unsigned char* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// ------------------------------------------------------- bf16 / fp16 kernel ---

template <typename T, int D, int QPW, int BC, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_kernel(FwdArgs a) {
    constexpr int NT = 256, WAVES = 4;
    constexpr int BR = WAVES * QPW;
    constexpr int QB = QPW / 32;      // 32-query column blocks per wave
    constexpr int KB = BC / 32;       // 32-key row blocks per tile
    constexpr int DB = D / 32;        // 32-dim row blocks of O^T
    constexpr int DS = D / 16;        // k-steps of S^T = K Q^T
    constexpr int KS = BC / 16;       // k-steps of O^T += V^T P^T
    constexpr int CPR_K = D / 8;      // 16-byte chunks per K row
    constexpr int CPR_V = BC / 8;     // 16-byte chunks per V^T row
    constexpr int K_BYTES = BC * D * 2;
    constexpr int V_BYTES = D * BC * 2;
    constexpr int STAGE = K_BYTES + V_BYTES;
    constexpr int K_CHUNKS = BC * CPR_K / NT;          // K chunks staged per thread
    constexpr int V_UNITS = (BC / 4) * (D / 8);        // 4 keys x 8 dims per unit
    static_assert(K_CHUNKS >= 1 && (BC * CPR_K) % NT == 0, "K staging shape");
    static_assert(V_UNITS == NT, "V staging: one unit per thread");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, l32 = lane & 31;
    const int N = a.n;

    const int bid = remap_xcd(blockIdx.x, a.n_blocks);
    const int bh = bid / a.n_qblk;
    int qblk = bid - bh * a.n_qblk;
    if (CAUSAL) qblk = a.n_qblk - 1 - qblk;   // longest rows first
    const int64_t head = (int64_t)bh * N * D;
    const T* __restrict__ Qh = reinterpret_cast<const T*>(a.q) + head;
    const T* __restrict__ Kh = reinterpret_cast<const T*>(a.k) + head;
    const T* __restrict__ Vh = reinterpret_cast<const T*>(a.v) + head;
    T* __restrict__ Oh = reinterpret_cast<T*>(a.o) + head;
    float* __restrict__ Lh = a.lse + (int64_t)bh * N;

    const int q_wave = qblk * BR + wave * QPW;     // first query row of this wave
    const float c = a.c;

    // ---- Q^T fragments (B operand): lane holds query q_wave + qb*32 + l32, dims 16s+8h..+7
    u32x4 qf[QB][DS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = q_wave + qb * 32 + l32;
#pragma unroll
        for (int s = 0; s < DS; ++s) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row < N) v = *reinterpret_cast<const u32x4*>(Qh + (int64_t)row * D + s * 16 + h * 8);
            qf[qb][s] = v;
        }
    }

    // ---- tile range
    int n_tiles = (int)((N + BC - 1) / BC);
    if (CAUSAL) {
        const int q_end = min(N, (qblk + 1) * BR);            // exclusive
        n_tiles = min(n_tiles, (q_end + BC - 1) / BC);
    }

    // ---- staging registers for the next K/V tile
    u32x4 kst[K_CHUNKS];
    u32x4 vst[4];
    auto load_tile = [&](int j) {
        const int kbase = j * BC;
#pragma unroll
        for (int i = 0; i < K_CHUNKS; ++i) {
            const int cidx = i * NT + tid;
            const int row = cidx / CPR_K, ch = cidx % CPR_K;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (kbase + row < N) v = *reinterpret_cast<const u32x4*>(Kh + (int64_t)(kbase + row) * D + ch * 8);
            kst[i] = v;
        }
        const int kg = tid / (D / 8), dc = tid % (D / 8);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = kbase + kg * 4 + r;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (key < N) v = *reinterpret_cast<const u32x4*>(Vh + (int64_t)key * D + dc * 8);
            vst[r] = v;
        }
    };
    auto store_tile = [&](int stage) {
        unsigned char* kb_ = smem + stage * STAGE;
        unsigned char* vb_ = kb_ + K_BYTES;
#pragma unroll
        for (int i = 0; i < K_CHUNKS; ++i) {
            const int cidx = i * NT + tid;
            const int row = cidx / CPR_K, ch = cidx % CPR_K;
            *reinterpret_cast<u32x4*>(kb_ + row * (D * 2) + 16 * (ch ^ swz<CPR_K>(row))) = kst[i];
        }
        // V^T: this thread holds keys 4kg..4kg+3 x dims 8dc..8dc+7; write, for each dim,
        // the 4 keys as one 8-byte piece at their permuted position (see header).
        const int kg = tid / (D / 8), dc = tid % (D / 8);
        const int k0 = kg * 4;
        const int g16 = k0 >> 4, kk = k0 & 15;
        const int pa = kk >> 3, ph = (kk >> 2) & 1;
        const int chunk = 2 * g16 + ph;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int w = e >> 1;
            unsigned lo, hi;
            if ((e & 1) == 0) {
                lo = (vst[0][w] & 0xffffu) | (vst[1][w] << 16);
                hi = (vst[2][w] & 0xffffu) | (vst[3][w] << 16);
            } else {
                lo = (vst[0][w] >> 16) | (vst[1][w] & 0xffff0000u);
                hi = (vst[2][w] >> 16) | (vst[3][w] & 0xffff0000u);
            }
            const int dd = dc * 8 + e;
            u32x2 piece = {lo, hi};
            *reinterpret_cast<u32x2*>(vb_ + dd * (BC * 2) + 16 * (chunk ^ swz<CPR_V>(dd)) + 8 * pa) = piece;
        }
    };

    // ---- running state
    f32x16 o[DB][QB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int t = 0; t < 16; ++t) o[db][qb][t] = 0.f;
    float m[QB], lsum[QB], lrnd[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) { m[qb] = -INFINITY; lsum[qb] = 0.f; lrnd[qb] = 0.f; }

    if (n_tiles > 0) {
        load_tile(0);
        store_tile(0);
        if (n_tiles > 1) load_tile(1);
    }
    __syncthreads();

    for (int j = 0; j < n_tiles; ++j) {
        const int kbase = j * BC;
        const unsigned char* kbuf = smem + (j & 1) * STAGE;
        const unsigned char* vbuf = kbuf + K_BYTES;

        // A wave whose rows all lie before this tile (causal) has nothing to do here.
        const bool active = !CAUSAL || (kbase <= q_wave + QPW - 1);
        if (active) {
            // ---- S^T = K_j Q^T
            f32x16 s[KB][QB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int t = 0; t < 16; ++t) s[kb][qb][t] = 0.f;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const int row = kb * 32 + l32;
                    const u32x4 kf = lds_read16(kbuf + row * (D * 2) + 16 * ((2 * ds + h) ^ swz<CPR_K>(row)));
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) s[kb][qb] = Elt<T>::mma(kf, qf[qb][ds], s[kb][qb]);
                }
            }

            // ---- masks: keys past N (tail tile), keys after the query (causal)
            const bool tail = kbase + BC > N;
            const bool diag = CAUSAL && (kbase + BC - 1 > q_wave);
            if (tail || diag) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) {
                        const int query = q_wave + qb * 32 + l32;
#pragma unroll
                        for (int t = 0; t < 16; ++t) {
                            const int key = kbase + kb * 32 + 8 * (t >> 2) + 4 * h + (t & 3);
                            bool drop = key >= N;
                            if (CAUSAL) drop = drop || key > query;
                            if (drop) s[kb][qb][t] = -INFINITY;
                        }
                    }
            }

            // ---- row maxima of this tile and the (lazy) rescale
            float mx[QB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float x0 = -INFINITY, x1 = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int t = 0; t < 16; t += 2) {
                        x0 = fmaxf(x0, s[kb][qb][t]);
                        x1 = fmaxf(x1, s[kb][qb][t + 1]);
                    }
                mx[qb] = pair_max(fmaxf(x0, x1)) * c;
            }
            bool need = false;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) need = need || (mx[qb] > m[qb] + kRescaleThreshold);
            if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const float mnew = fmaxf(m[qb], mx[qb]);
                    const float alpha = (m[qb] == -INFINITY) ? 0.f : fast_exp2(m[qb] - mnew);
                    m[qb] = mnew;
                    lsum[qb] *= alpha;
                    lrnd[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int t = 0; t < 16; ++t) o[db][qb][t] *= alpha;
                }
            }

            // ---- P = 2^(s*c - m), packed to the MFMA element type.  Two row sums: of
            // the rounded values (divides O, so the weights applied to V sum exactly to
            // the divisor) and of the fp32 values (gives LSE).
            u32x4 pf[KS][QB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float neg_m = (m[qb] == -INFINITY) ? 0.f : -m[qb];
                float acc0 = 0.f, acc1 = 0.f, racc0 = 0.f, racc1 = 0.f;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    float p[16];
#pragma unroll
                    for (int t = 0; t < 16; ++t) p[t] = fast_exp2(__builtin_fmaf(s[kb][qb][t], c, neg_m));
#pragma unroll
                    for (int t = 0; t < 16; t += 2) { acc0 += p[t]; acc1 += p[t + 1]; }
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        u32x4 f;
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            f[w] = Elt<T>::pack2(p[8 * half + 2 * w], p[8 * half + 2 * w + 1]);
                            if (w & 1) racc1 = Elt<T>::sum2(f[w], racc1);
                            else racc0 = Elt<T>::sum2(f[w], racc0);
                        }
                        pf[2 * kb + half][qb] = f;
                    }
                }
                lsum[qb] += acc0 + acc1;
                lrnd[qb] += racc0 + racc1;
            }

            // ---- O^T += V_j^T P^T
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int dd = db * 32 + l32;
                    const u32x4 vf = lds_read16(vbuf + dd * (BC * 2) + 16 * ((2 * ks + h) ^ swz<CPR_V>(dd)));
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) o[db][qb] = Elt<T>::mma(vf, pf[ks][qb], o[db][qb]);
                }
            }
        }

        // ---- next tile into the other stage; its loads were issued one iteration ago
        if (j + 1 < n_tiles) {
            store_tile((j + 1) & 1);
            if (j + 2 < n_tiles) load_tile(j + 2);
        }
        __syncthreads();
    }

    // ---- epilogue: O / l, LSE = (m + log2 l) ln 2
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = q_wave + qb * 32 + l32;
        const float lt = pair_sum(lsum[qb]);
        const float inv = 1.0f / pair_sum(lrnd[qb]);
        if (row < N) {
            T* orow = Oh + (int64_t)row * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 w;
                    w[0] = Elt<T>::pack2(o[db][qb][4 * g + 0] * inv, o[db][qb][4 * g + 1] * inv);
                    w[1] = Elt<T>::pack2(o[db][qb][4 * g + 2] * inv, o[db][qb][4 * g + 3] * inv);
                    *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * g + 4 * h) = w;
                }
            if (h == 0) Lh[row] = (m[qb] + __builtin_amdgcn_logf(lt)) * kLn2;
        }
    }
}

// ------------------------------------------------------------- fp32 kernel ---
//
// Same transposed formulation with v_mfma_f32_32x32x2_f32: each MFMA contracts two
// dims (lane half h supplies dim 2s+h) or two keys.  Used for fp32 inputs, which are
// small here; single LDS stage, 32 keys per tile, 32 queries per wave.

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_kernel_f32(FwdArgs a) {
    constexpr int NT = 256, WAVES = 4, QPW = 32, BC = 32;
    constexpr int BR = WAVES * QPW;
    constexpr int DB = D / 32;
    constexpr int DS = D / 2;
    constexpr int LD = D + 1;        // padded row stride (floats)
    __shared__ float ks_[BC * LD];
    __shared__ float vs_[BC * LD];

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

    const int q_wave = qblk * BR + wave * QPW;
    const int query = q_wave + l32;
    const float c = a.c;

    float qf[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = (query < N) ? Qh[(int64_t)query * D + 2 * s + h] : 0.f;

    int n_tiles = (N + BC - 1) / BC;
    if (CAUSAL) n_tiles = min(n_tiles, (min(N, (qblk + 1) * BR) + BC - 1) / BC);

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int t = 0; t < 16; ++t) o[db][t] = 0.f;
    float m = -INFINITY, lsum = 0.f;

    for (int j = 0; j < n_tiles; ++j) {
        const int kbase = j * BC;
        __syncthreads();
        for (int idx = tid; idx < BC * D; idx += NT) {
            const int r = idx / D, col = idx % D;
            const bool ok = kbase + r < N;
            ks_[r * LD + col] = ok ? Kh[(int64_t)(kbase + r) * D + col] : 0.f;
            vs_[r * LD + col] = ok ? Vh[(int64_t)(kbase + r) * D + col] : 0.f;
        }
        __syncthreads();
        if (CAUSAL && kbase > q_wave + QPW - 1) continue;

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
        if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleThreshold) != 0) {
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

    const float lt = pair_sum(lsum);
    const float inv = 1.0f / lt;
    if (query < N) {
        float* orow = Oh + (int64_t)query * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int t = 0; t < 16; ++t) orow[db * 32 + 8 * (t >> 2) + 4 * h + (t & 3)] = o[db][t] * inv;
        if (h == 0) Lh[query] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
    }
}

// ------------------------------------------------------------------ dispatch ---

template <typename T, int D, int QPW, int BC>
static hipError_t launch_t(const FwdArgs& a, int causal, hipStream_t st) {
    const dim3 grid((unsigned)a.n_blocks), block(256);
    if (causal)
        hipLaunchKernelGGL((fwd_kernel<T, D, QPW, BC, true>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((fwd_kernel<T, D, QPW, BC, false>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_half(const FwdArgs& a, const fa_plan& p, int d, int causal, hipStream_t st) {
    (void)p;
    if (d == 128) return launch_t<T, 128, 32, 64>(a, causal, st);
    return launch_t<T, 64, 32, 128>(a, causal, st);
}

}  // namespace fa

int fa_launch_fwd(const fa::FwdArgs& a, const fa_plan& plan, int dtype, int d, int causal, void* stream) {
    using namespace fa;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
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
