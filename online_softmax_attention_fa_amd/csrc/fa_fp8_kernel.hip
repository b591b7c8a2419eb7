// Block-scaled fp8 mode for gfx950: the quantiser and the attention forward on E4M3 codes.
//
// The pages keep K and V in 8 bits with a scale and dequantise per tile
// ("从零理解Flash Attention中的online softmax", section 9.1), and name native FP8 with
// block-wise scale factors ("FlashAttention 硬件感知计算剖析", the FlashAttention-3
// summary).  Here Q, K and V are OCP E4M3 codes with one power-of-two scale per 64 rows
// of a (batch, head); the forward multiplies codes on v_mfma_f32_32x32x64_f8f6f4 (twice
// the bf16 rate) and also rounds P to E4M3 for the P V product.  The method is
// otherwise the bf16 kernel's online softmax: running maximum, running sum, unnormalised
// fp32 O, one division at the end, LSE saved.
//
// Scales never enter the MFMAs:
//  * Q's and K's block scales multiply c = scale * log2(e) per 32-key row block of S^T
//    (a wave's 32 queries lie in one Q block, a 32-key block in one K block);
//  * V's block scale 2^(e_v) enters as 2^(e_v - e_vmax) in P's exponent (one add per
//    64-key block), the sums take the inverse factor, and 2^(e_vmax) multiplies O at the
//    end.  P stays at most the E4M3 maximum because the unscaled P is.
//
// Operand layouts (one 32x32x64 MFMA: 64 lanes x 32 bytes per operand; lane L's bytes
// pair with the same bytes of lane L of the other operand, L%32 giving the row / column):
//  * S^T = K Q^T: lane L reads 32 dims of key 32kb + L%32 (A) and holds 32 dims of its
//    query (B) -- dims 64s + 32(L/32) .. +31 for k-step s.
//  * O^T += V^T P^T: the S^T accumulator leaves lane L with keys 8j + 4(L/32) + r
//    (j, r < 4) of each 32-key block.  For a 64-key step, v_permlane32_swap trades the
//    second block's codes of lanes 0-31 for the first block's of lanes 32-63; taking the
//    swapped pair of registers as dwords 2j and 2j + 1 gives lane L the 32 keys
//    64s + 32(L/32) + 0 .. 31 in order.  V is stored transposed (V^T, keys contiguous), so
//    the A operand is two plain 16-byte LDS reads of the same 32 keys.

#include "fa_device.h"
#include "fa_fp8.h"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kFp8Max = 448.0f;
// P = 2^(s c - m + kFp8POffset), i.e. 2 at the running maximum.  A tile is redone with
// its own row maximum when a lane's sum of P over the tile exceeds kFp8MaxTileSum: every
// P is then at most 448, the largest E4M3 value (and at most 2 after the redo).
constexpr float kFp8POffset = 1.0f;
constexpr float kFp8MaxTileSum = kFp8Max;
// V block factors below 2^-60 of the head's largest are treated as 2^-60: P times such a
// factor is far below the smallest E4M3 value either way.
constexpr int kFp8MinVShift = -60;

__device__ __forceinline__ f32x16 mma_fp8(i32x8 a, i32x8 b, f32x16 c) {
    // cbsz = blgp = 0: both operands E4M3; zero scale operands give the unscaled MFMA
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Four fp32 values to E4M3 codes, round to nearest even; value i lands in byte i.
__device__ __forceinline__ unsigned pack4_fp8(float x0, float x1, float x2, float x3, int old = 0) {
    // the first conversion fills bytes 0-1 and the second bytes 2-3, so the word's
    // starting contents (`old`) never matter; passing a dead register saves initialising one
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, old, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
    return (unsigned)w;
}

// Exponent e of a block scale 2^e: the smallest e with amax <= 448 * 2^e, clamped to
// [-126, 127]; -126 for an all-zero block, 0 when amax is not finite (the non-finite
// elements then encode as NaN codes).
__device__ __forceinline__ int fp8_block_exponent(float amax) {
    if (amax == 0.f) return -126;
    if (!(amax <= 3.40282347e38f)) return 0;
    int e = __builtin_amdgcn_frexp_expf(amax) - 9;   // amax / 2^e in [256, 512)
    if (amax > __builtin_amdgcn_ldexpf(kFp8Max, e)) ++e;
    return min(max(e, -126), 127);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = __builtin_elementwise_maximum(x, __shfl_xor(x, off));
    return x;
}

// ---------------------------------------------------------------- quantiser ---
//
// One workgroup of 256 threads per (batch*head, 64-row block): load the block (rows past
// N as zeros), reduce |x| to the block maximum, pick the scale, encode x / 2^e.  The
// transposed layout writes V^T [d][Np] through an LDS copy of the block's codes; its
// grid also covers the padding blocks up to Np, which receive zeros.
template <typename T, int D, bool TRANSPOSE>
__global__ __launch_bounds__(256) void quant_fp8_kernel(QuantArgs a) {
    constexpr int VPR = D / 8;                      // 16-byte input vectors per row
    constexpr int VEC = kFp8Block * VPR / 256;      // vectors per thread
    const int tid = threadIdx.x;
    const int bh = blockIdx.x / a.blocks_per_head;
    const int blk = blockIdx.x - bh * a.blocks_per_head;
    const int N = a.n;
    const int r0 = blk * kFp8Block;
    const T* __restrict__ xh = reinterpret_cast<const T*>(a.x) + (int64_t)bh * N * D;

    float v[VEC][8];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        const int vi = tid + 256 * i;
        const int row = r0 + vi / VPR, col = (vi % VPR) * 8;
        if (row < N) {
            typedef T t8 __attribute__((ext_vector_type(8)));
            const t8 x = *reinterpret_cast<const t8*>(xh + (int64_t)row * D + col);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[i][e] = (float)x[e];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[i][e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = __builtin_elementwise_maximum(amax, fabsf(v[i][e]));
    }
    __shared__ float wmax[4];
    amax = wave_max(amax);
    if ((tid & 63) == 0) wmax[tid >> 6] = amax;
    __syncthreads();
    amax = __builtin_elementwise_maximum(__builtin_elementwise_maximum(wmax[0], wmax[1]),
                                         __builtin_elementwise_maximum(wmax[2], wmax[3]));
    const int e = fp8_block_exponent(amax);
    if (tid == 0 && r0 < N) a.scales[(int64_t)bh * a.nb + blk] = __builtin_amdgcn_ldexpf(1.0f, e);

    u32x2 code[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i)
#pragma unroll
        for (int w = 0; w < 2; ++w)
            code[i][w] = pack4_fp8(__builtin_amdgcn_ldexpf(v[i][4 * w + 0], -e), __builtin_amdgcn_ldexpf(v[i][4 * w + 1], -e),
                                   __builtin_amdgcn_ldexpf(v[i][4 * w + 2], -e), __builtin_amdgcn_ldexpf(v[i][4 * w + 3], -e));

    if constexpr (!TRANSPOSE) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            const int vi = tid + 256 * i;
            const int row = r0 + vi / VPR, col = (vi % VPR) * 8;
            if (row < N) *reinterpret_cast<u32x2*>(a.x8 + ((int64_t)bh * N + row) * D + col) = code[i];
        }
    } else {
        __shared__ __attribute__((aligned(16))) unsigned char tile[kFp8Block * D];
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            const int vi = tid + 256 * i;
            *reinterpret_cast<u32x2*>(tile + (vi / VPR) * D + (vi % VPR) * 8) = code[i];
        }
        __syncthreads();
        // 16 keys of one V^T row per item: D rows x 4 items per block
#pragma unroll
        for (int i = 0; i < D * 4 / 256; ++i) {
            const int it = tid + 256 * i;
            const int dr = it >> 2, kc = it & 3;
            u32x4 w;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                unsigned x = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) x |= (unsigned)tile[(16 * kc + 4 * q + b) * D + dr] << (8 * b);
                w[q] = x;
            }
            *reinterpret_cast<u32x4*>(a.x8 + ((int64_t)bh * D + dr) * a.np + r0 + 16 * kc) = w;
        }
    }
}

// ---------------------------------------------------------------- forward ---

// 16-byte chunk swizzle for 128-byte (8 chunks) and 64-byte (4 chunks) LDS rows: the
// 16 consecutive rows one ds_read_b128 lane group reads at one logical chunk land in
// 16 distinct 16-byte slots of a 256-byte bank window.
template <int CPR>
__device__ __forceinline__ int swz_fp8(int row) {
    if constexpr (CPR == 8) return swz<8>(row);
    else return (row >> 2) & 3;
}

// Three waves per SIMD (three 4-wave workgroups per CU, <= 168 VGPRs): with 64-key tiles a
// workgroup needs 32 KiB of LDS and the registers fit; the third wave hides more of each
// wave's MFMA -> softmax -> MFMA dependency chain than the 128-key tile's longer steps did
// (8% faster at B=4 H=32 N=16384 d=128).
template <typename TO, int D, int WAVES, bool CAUSAL>
__global__ __launch_bounds__(64 * WAVES, 3) void fwd_fp8_kernel(Fp8Args a) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int NT = 64 * WAVES, QPW = 32, BR = WAVES * QPW, BC = kFp8TileK;
    constexpr int CPV = BC / 16;       // 16-byte chunks per V^T row
    constexpr int KB = BC / 32;        // 32-key row blocks of S^T per tile
    constexpr int DB = D / 32;         // 32-dim row blocks of O^T
    constexpr int DS = D / 64;         // k-steps of S^T
    constexpr int KS = BC / 64;        // k-steps of O^T (one V scale block each)
    constexpr int RK = D, RV = BC;     // bytes per K row, per V^T row
    constexpr int CPK = D / 16;
    constexpr int KTILE = BC * RK, VTILE = D * RV, STAGE = KTILE + VTILE;
    constexpr int KLOADS = KTILE / (NT * 16), VLOADS = VTILE / (NT * 16);
    static_assert(KLOADS >= 1 && VLOADS >= 1 && KTILE % (NT * 16) == 0 && VTILE % (NT * 16) == 0,
                  "tiles must be whole blocks of the workgroup's 16-byte copies");

    __shared__ __attribute__((aligned(1024))) unsigned char stage0_raw[STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char stage1_raw[STAGE];
    lds_u8* const stage0 = (lds_u8*)stage0_raw;
    lds_u8* const stage1 = (lds_u8*)stage1_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int N = a.n, NP = a.np, NB = a.nb;

    const int bid = remap_xcd(blockIdx.x, a.n_blocks);
    const int bh = bid / a.n_qblk;
    int qblk = bid - bh * a.n_qblk;
    if (CAUSAL) qblk = a.n_qblk - 1 - qblk;   // longest rows first
    const unsigned char* __restrict__ Qh = a.q8 + (int64_t)bh * N * D;
    const unsigned char* __restrict__ Kh = a.k8 + (int64_t)bh * N * D;
    const unsigned char* __restrict__ Vh = a.vt8 + (int64_t)bh * D * NP;
    // Scale tables are read-only for the kernel's lifetime: read them through the constant
    // address space, i.e. with scalar loads.  (Vector loads would be counted with the
    // tile copies in flight, and waiting for a scale would then wait for the next tile.)
    typedef __attribute__((address_space(4))) const float cfloat;
    const cfloat* qsh = (const cfloat*)(a.qs + (int64_t)bh * NB);
    const cfloat* ksh = (const cfloat*)(a.ks + (int64_t)bh * NB);
    const cfloat* vsh = (const cfloat*)(a.vs + (int64_t)bh * NB);
    TO* __restrict__ Oh = reinterpret_cast<TO*>(a.o) + (int64_t)bh * N * D;
    float* __restrict__ Lh = a.lse + (int64_t)bh * N;

    const int q_wave = qblk * BR + wave * QPW;
    const int query = q_wave + l32;

    // ---- scales: Q's block for this wave's rows; the head's largest V block scale
    const float cw = a.c * qsh[min(q_wave / kFp8Block, NB - 1)];
    float vmax = 0.f;
    for (int i = lane; i < NB; i += 64) vmax = fmaxf(vmax, vsh[i]);
    vmax = wave_max(vmax);
    const int ev_max = __builtin_amdgcn_frexp_expf(vmax) - 1;   // vmax = 2^ev_max

    // ---- Q^T fragments (B operand of S^T): dims 64s + 32h .. +31 of this lane's query
    i32x8 qf[DS];
    {
        const int row = query < N ? query : 0;
#pragma unroll
        for (int s = 0; s < DS; ++s) {
            const u32x4* p = reinterpret_cast<const u32x4*>(Qh + (int64_t)row * D + 64 * s + 32 * h);
            const u32x4 lo = p[0], hi = p[1];
            qf[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
    }

    // ---- per-lane LDS read offsets (row-block and stage offsets are added as immediates)
    int koff[DS][2], voff[KS][2];
#pragma unroll
    for (int s = 0; s < DS; ++s)
#pragma unroll
        for (int e = 0; e < 2; ++e) koff[s][e] = l32 * RK + 16 * ((4 * s + 2 * h + e) ^ swz_fp8<CPK>(l32));
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int e = 0; e < 2; ++e) voff[s][e] = KTILE + l32 * RV + 16 * ((4 * s + 2 * h + e) ^ swz_fp8<CPV>(l32));

    // ---- HBM -> LDS copies: lane L of wave w, copy i fills 16 bytes at i*NT*16 + w*1024 + 16L
    // of the K (V^T) tile; the source is the chunk the swizzle stores there.  K rows past
    // N read as zeros (buffer range); V^T rows are padded to Np with zero codes.
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, N * D, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, D * NP, kBufferRsrcWord3);
    int ksrc[KLOADS], vsrc[VLOADS];
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
        const int off = i * (NT * 16) + wave * 1024 + lane * 16;
        const int row = off / RK;
        ksrc[i] = row * RK + 16 * (((off % RK) >> 4) ^ swz_fp8<CPK>(row));
    }
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
        const int off = i * (NT * 16) + wave * 1024 + lane * 16;
        const int dr = off / RV;
        vsrc[i] = dr * NP + 16 * (((off % RV) >> 4) ^ swz_fp8<CPV>(dr));
    }
    auto issue_tile = [&](int j, lds_u8* stage) {
#pragma unroll
        for (int i = 0; i < KLOADS; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)(stage + i * (NT * 16) + wave * 1024),
                                                     16, ksrc[i] + j * BC * RK, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < VLOADS; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)(stage + KTILE + i * (NT * 16) + wave * 1024),
                                                     16, vsrc[i] + j * BC, 0, 0, 0);
    };

    f32x16 o[DB];
    // P codes of the current 64-key step, the B operand of O^T += V^T P^T: dword 2q + kk
    // holds word q of 32-key block kk (kept across steps so the codes overwrite the last
    // step's in place)
    i32x8 pb = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int t = 0; t < 16; ++t) o[db][t] = 0.f;
    float m = -INFINITY, lsum = 0.f;
    int n_tiles = (N + BC - 1) / BC;
    if (CAUSAL) n_tiles = min(n_tiles, (min(N, (qblk + 1) * BR) + BC - 1) / BC);

    // Per 64-key block: the K scale folded into c, the V scale as an exponent shift of P and
    // the inverse factor for the sums.  They are the same for every lane, but there is no
    // scalar float arithmetic, so derived per tile they cost about ten VALU instructions in a
    // kernel bound by its VALU work.  Instead lane L derives block 64 c + L's, for 64 blocks
    // at a time (chunk c), and each tile reads its block's back with v_readlane.
    float ck_l = 0.f, vshe_l = 0.f, vw_l = 0.f;
    int chunk = -1;
    auto lane_value = [](float x, int l) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
    };
    auto compute_tile = [&](int j, const lds_u8* sbase) {
        const int kbase = j * BC;
        float ck[KS], vsh_e[KS], vw[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int blk = min(j * KS + s, NB - 1);
            if (blk >> 6 != chunk) {   // uniform: once per 64 blocks
                chunk = blk >> 6;
                const int lb = min(64 * chunk + lane, NB - 1);
                ck_l = fmaxf(cw * ksh[lb], 1.17549435e-38f);
                const int sh = max(__builtin_amdgcn_frexp_expf(vsh[lb]) - 1 - ev_max, kFp8MinVShift);
                vshe_l = (float)sh + kFp8POffset;
                vw_l = __builtin_amdgcn_ldexpf(1.0f, -sh);
            }
            ck[s] = lane_value(ck_l, blk & 63);
            vsh_e[s] = lane_value(vshe_l, blk & 63);
            vw[s] = lane_value(vw_l, blk & 63);
        }

        __builtin_amdgcn_s_setprio(1);
        f32x16 s[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int t = 0; t < 16; ++t) s[kb][t] = 0.f;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                const u32x4 lo = lds_read16(sbase, koff[ds][0] + kb * 32 * RK);
                const u32x4 hi = lds_read16(sbase, koff[ds][1] + kb * 32 * RK);
                const i32x8 kf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                s[kb] = mma_fp8(kf, qf[ds], s[kb]);
            }
        }
        __builtin_amdgcn_s_setprio(0);

        if (CAUSAL) {
            if (kbase + BC > N || kbase + BC - 1 > q_wave) {   // keys after the query or past N
                const int last = min(query, N - 1) - kbase - 4 * h;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int t = 0; t < 16; ++t)
                        if (kb * 32 + 8 * (t >> 2) + (t & 3) > last) s[kb][t] = -INFINITY;
            }
        } else if (kbase + BC > N) {   // keys past N
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const int key = kbase + kb * 32 + 8 * (t >> 2) + 4 * h + (t & 3);
                    if (key >= N) s[kb][t] = -INFINITY;
                }
        }

        // P, its sums and O^T += V^T P^T one 64-key step at a time: the softmax of a step
        // overlaps the score MFMAs still running for the next step and the P V MFMAs of the
        // previous one.  Each step is its own online-softmax block: it is redone with its
        // own maximum when a lane's sum of P over it leaves range.
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float tsum;
            auto make_p = [&](float neg_m) {
                const float nm = neg_m + vsh_e[ks];
                float acc0, acc1;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    float p[16];
#pragma unroll
                    for (int t = 0; t < 16; ++t) p[t] = fast_exp2(__builtin_fmaf(s[2 * ks + kk][t], ck[ks], nm));
                    // (the sums start from their first terms: 0 + p is an instruction the
                    // compiler may not drop, as it would turn -0 into +0)
#pragma unroll
                    for (int t = 0; t < 16; t += 2) {
                        acc0 = kk == 0 && t == 0 ? p[t] : acc0 + p[t];
                        acc1 = kk == 0 && t == 0 ? p[t + 1] : acc1 + p[t + 1];
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        pb[2 * q + kk] = (int)pack4_fp8(p[4 * q], p[4 * q + 1], p[4 * q + 2], p[4 * q + 3], pb[2 * q + kk]);
                }
                tsum = (acc0 + acc1) * vw[ks];
            };
            make_p(-m);
            if (__builtin_amdgcn_ballot_w64(!(tsum <= kFp8MaxTileSum)) != 0) {
                float x0 = -INFINITY, x1 = -INFINITY;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int t = 0; t < 16; t += 4) {
                        x0 = vmax3(x0, s[2 * ks + kk][t], s[2 * ks + kk][t + 1]);
                        x1 = vmax3(x1, s[2 * ks + kk][t + 2], s[2 * ks + kk][t + 3]);
                    }
                const float mx = pair_max(__builtin_elementwise_maximum(x0, x1) * ck[ks]);
                const float mnew = fmaxf(m, mx);
                const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mnew);
                m = mnew;
                lsum *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int t = 0; t < 16; ++t) o[db][t] *= alpha;
                make_p(-m);
            }
            lsum += tsum;

            __builtin_amdgcn_s_setprio(1);
            // lanes 0-31 keep block 2ks's codes and take block 2ks+1's from lanes 32-63
            // (and the reverse), interleaved so that dword i holds keys 4i .. 4i+3 of the
            // lane's 32, the order of V^T in LDS
            // (swapped in place: the pair stays in the operand's registers)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const auto r = __builtin_amdgcn_permlane32_swap((unsigned)pb[2 * q], (unsigned)pb[2 * q + 1], false, false);
                pb[2 * q] = (int)r[0];
                pb[2 * q + 1] = (int)r[1];
            }
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const u32x4 n0 = lds_read16(sbase, voff[ks][0] + db * 32 * RV);
                const u32x4 n1 = lds_read16(sbase, voff[ks][1] + db * 32 * RV);
                const i32x8 va = {(int)n0[0], (int)n0[1], (int)n0[2], (int)n0[3], (int)n1[0], (int)n1[1], (int)n1[2], (int)n1[3]};
                o[db] = mma_fp8(va, pb, o[db]);
            }
            __builtin_amdgcn_s_setprio(0);
        }
    };

    issue_tile(0, stage0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    for (int j = 0; j < n_tiles; j += 2) {
        // (causal: every wave computes every tile up to the block's diagonal; skipping the
        // few tiles past a wave's own rows costs more in registers than it saves)
        if (j + 1 < n_tiles) issue_tile(j + 1, stage1);
        compute_tile(j, stage0);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (j + 1 >= n_tiles) break;
        if (j + 2 < n_tiles) issue_tile(j + 2, stage0);
        compute_tile(j + 1, stage1);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    }

    // ---- epilogue: O = 2^(e_vmax) O_acc / l, LSE = (m - offset + log2 l) ln 2
    const float lt = pair_sum(lsum);
    const float inv = vmax / lt;
    if (query < N) {
        TO* orow = Oh + (int64_t)query * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = Elt<TO>::pack2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv);
                w[1] = Elt<TO>::pack2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
                *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * g + 4 * h) = w;
            }
        if (h == 0) Lh[query] = (m - kFp8POffset + __builtin_amdgcn_logf(lt)) * kLn2;
    }
#endif
}

template <typename T, int D>
int launch_quant_t(const QuantArgs& a, int64_t bh, int transpose, hipStream_t stream) {
    const dim3 grid((unsigned)(bh * a.blocks_per_head));
    if (transpose)
        hipLaunchKernelGGL((quant_fp8_kernel<T, D, true>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((quant_fp8_kernel<T, D, false>), grid, dim3(256), 0, stream, a);
    return (int)hipGetLastError();
}

template <typename TO, int D>
int launch_fp8_t(const Fp8Args& a, int causal, hipStream_t stream) {
    constexpr int WAVES = kFp8BlockQ / 32;
    if (causal)
        hipLaunchKernelGGL((fwd_fp8_kernel<TO, D, WAVES, true>), dim3(a.n_blocks), dim3(64 * WAVES), 0, stream, a);
    else
        hipLaunchKernelGGL((fwd_fp8_kernel<TO, D, WAVES, false>), dim3(a.n_blocks), dim3(64 * WAVES), 0, stream, a);
    return (int)hipGetLastError();
}

}  // namespace fa

int fa_launch_quantize_fp8(const fa::QuantArgs& a, int64_t bh, int in_dtype, int d, int transpose, hipStream_t stream) {
    if (in_dtype == FA_BF16)
        return d == 128 ? fa::launch_quant_t<__bf16, 128>(a, bh, transpose, stream)
                        : fa::launch_quant_t<__bf16, 64>(a, bh, transpose, stream);
    return d == 128 ? fa::launch_quant_t<_Float16, 128>(a, bh, transpose, stream)
                    : fa::launch_quant_t<_Float16, 64>(a, bh, transpose, stream);
}

int fa_launch_fwd_fp8(const fa::Fp8Args& a, int out_dtype, int d, int causal, hipStream_t stream) {
    if (out_dtype == FA_BF16)
        return d == 128 ? fa::launch_fp8_t<__bf16, 128>(a, causal, stream) : fa::launch_fp8_t<__bf16, 64>(a, causal, stream);
    return d == 128 ? fa::launch_fp8_t<_Float16, 128>(a, causal, stream) : fa::launch_fp8_t<_Float16, 64>(a, causal, stream);
}
