// Recompute-based attention backward for gfx950.
//
// The forward saved LSE = m + ln l per row, so P is rebuilt exactly from it without
// the running-maximum recurrence ("从原理出发理解 Flash Attention Part2", section 2.4;
// "从零理解Flash Attention中的online softmax", section 5.1).  With D_i = sum_k dO_ik O_ik
// (which equals rowsum(P * dP)):
//
//     P = exp(scale Q K^T - LSE),  dP = dO V^T,  dS = P * (dP - D),
//     dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
//
// Three kernels, no atomics (results are deterministic):
//  * bwd_pre:  D and LSE * log2(e) per row, into the caller's workspace;
//  * bwd_dq:   one workgroup per (b, h, 128 query rows), streaming K and V tiles;
//              S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T -- the forward kernel's
//              structure with dS in place of P and K^T (transposing LDS read) in place
//              of V^T;
//  * bwd_dkdv: one workgroup per (b, h, 128 key rows), streaming Q and dO tiles;
//              S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS.
// In all MFMA products the contraction index of an accumulator-layout operand is the
// permuted one described in the forward kernel, and the transposing LDS read of the other
// operand gathers it in the same order.

#include "fa_device.h"

namespace fa {

typedef __attribute__((address_space(3))) float lds_f32;

// -------------------------------------------------------------- preprocess ---
// D[r] = sum_d dO[r][d] O[r][d] (fp32); L2[r] = LSE[r] * log2(e).  16 (d=128) or 8
// (d=64) lanes per row, 16 bytes each.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                      const float* __restrict__ LSE, float* __restrict__ Dout,
                                                      float* __restrict__ L2, int64_t rows) {
    constexpr int LPR = D / 8;                 // lanes per row
    constexpr int RPB = 256 / LPR;             // rows per block
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    const int part = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(O + row * D + part * 8);
        const u32x4 b = *reinterpret_cast<const u32x4*>(dO + row * D + part * 8);
#pragma unroll
        for (int w = 0; w < 4; ++w) acc = Elt<T>::dot2(a[w], b[w], acc);
    }
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (row < rows && part == 0) {
        Dout[row] = acc;
        L2[row] = LSE[row] * 1.4426950408889634074f;
    }
}

// ---------------------------------------------------------------- dQ kernel ---
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int NT = 256, QPW = 32, BR = 4 * QPW, BC = 64;
    constexpr int KB = BC / 32, DB = D / 32, DS = D / 16, KS = BC / 16;
    constexpr int RB = D * 2, CPR = D / 8, TILE = BC * RB, STAGE = 2 * TILE;
    constexpr int LOADS = TILE / (NT * 16);
    static_assert(LOADS >= 1 && TILE % (NT * 16) == 0, "tile shape");

    __shared__ __attribute__((aligned(1024))) unsigned char stage0_raw[STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char stage1_raw[STAGE];
    lds_u8* const stage0 = (lds_u8*)stage0_raw;
    lds_u8* const stage1 = (lds_u8*)stage1_raw;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int N = a.n;
    const int bid = remap_xcd(blockIdx.x, a.n_blocks);
    const int bh = bid / a.n_blk;
    int qblk = bid - bh * a.n_blk;
    if (CAUSAL) qblk = a.n_blk - 1 - qblk;
    const int64_t head = (int64_t)bh * N * D;
    const T* Qh = reinterpret_cast<const T*>(a.q) + head;
    const T* Kh = reinterpret_cast<const T*>(a.k) + head;
    const T* Vh = reinterpret_cast<const T*>(a.v) + head;
    const T* dOh = reinterpret_cast<const T*>(a.dout) + head;
    T* dQh = reinterpret_cast<T*>(a.dq) + head;

    const int q_wave = qblk * BR + wave * QPW;
    const int query = q_wave + l32;
    const int row = query < N ? query : 0;
    const float c = a.c;

    u32x4 qf[DS], dof[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) {
        qf[s] = *reinterpret_cast<const u32x4*>(Qh + (int64_t)row * D + s * 16 + h * 8);
        dof[s] = *reinterpret_cast<const u32x4*>(dOh + (int64_t)row * D + s * 16 + h * 8);
    }
    const float l2 = a.l2[(int64_t)bh * N + row];
    const float dd = a.dsum[(int64_t)bh * N + row];

    int koff[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) koff[s] = l32 * RB + 16 * ((2 * s + h) ^ swz<CPR>(l32));
    int ktr[2][DB];   // transposing reads of K (as K^T)
    {
        const int g = lane >> 4, r = lane & 15;
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int key = 8 * aa + 4 * h + (r >> 2);
                const int dim = 32 * db + 16 * (g & 1) + 4 * (r & 3);
                ktr[aa][db] = key * RB + 16 * ((dim >> 3) ^ swz<CPR>(key)) + 2 * (dim & 7);
            }
    }
    const int head_bytes = N * D * 2;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, head_bytes, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, head_bytes, kBufferRsrcWord3);
    int src_off[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int off = i * (NT * 16) + wave * 1024 + lane * 16;
        const int r = off / RB;
        const int ch = ((off % RB) >> 4) ^ swz<CPR>(r);
        src_off[i] = r * RB + ch * 16;
    }
    auto issue = [&](int j, lds_u8* stage) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            lds_u8* dst = stage + i * (NT * 16) + wave * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)dst, 16,
                                                     src_off[i] + j * BC * RB, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)(dst + TILE), 16,
                                                     src_off[i] + j * BC * RB, 0, 0, 0);
        }
    };

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int t = 0; t < 16; ++t) acc[db][t] = 0.f;

    int n_tiles = (N + BC - 1) / BC;
    if (CAUSAL) n_tiles = min(n_tiles, (min(N, (qblk + 1) * BR) + BC - 1) / BC);

    auto tile = [&](int j, const lds_u8* sbase) {
        if (CAUSAL && j * BC > q_wave + QPW - 1) return;
        const int kbase = j * BC;
        f32x16 s[KB], dp[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int t = 0; t < 16; ++t) { s[kb][t] = 0.f; dp[kb][t] = 0.f; }
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                s[kb] = Elt<T>::mma(lds_read16(sbase, koff[ds] + kb * 32 * RB), qf[ds], s[kb]);
                dp[kb] = Elt<T>::mma(lds_read16(sbase, TILE + koff[ds] + kb * 32 * RB), dof[ds], dp[kb]);
            }
        // masks in a branch of their own (uniform per wave), so full tiles run none of it
        const bool tail = kbase + BC > N;
        const bool diag = CAUSAL && (kbase + BC - 1 > q_wave);
        if (tail || diag) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const int key = kbase + kb * 32 + 8 * (t >> 2) + 4 * h + (t & 3);
                    bool drop = key >= N;
                    if (CAUSAL) drop = drop || key > query;
                    if (drop) s[kb][t] = -INFINITY;
                }
        }
        u32x4 dsf[KS];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            float v[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const float p = fast_exp2(__builtin_fmaf(s[kb][t], c, -l2));
                v[t] = p * (dp[kb][t] - dd);
            }
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                u32x4 f;
#pragma unroll
                for (int w = 0; w < 4; ++w) f[w] = Elt<T>::pack2(v[8 * half + 2 * w], v[8 * half + 2 * w + 1]);
                dsf[2 * kb + half] = f;
            }
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const u32x2 lo = lds_read_tr(sbase, ktr[0][db] + ks * 16 * RB);
                const u32x2 hi = lds_read_tr(sbase, ktr[1][db] + ks * 16 * RB);
                const u32x4 kt = {lo[0], lo[1], hi[0], hi[1]};
                acc[db] = Elt<T>::mma(kt, dsf[ks], acc[db]);
            }
    };

    issue(0, stage0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
#pragma unroll 1
    for (int j = 0; j < n_tiles; j += 2) {
        if (j + 1 < n_tiles) issue(j + 1, stage1);
        tile(j, stage0);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (j + 1 < n_tiles) {   // (no mid-loop exit: one set of accumulators at the loop's end)
            if (j + 2 < n_tiles) issue(j + 2, stage0);
            tile(j + 1, stage1);
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
        }
    }

    if (query < N) {
        T* orow = dQh + (int64_t)query * D;
        const float sc = a.scale;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = Elt<T>::pack2(acc[db][4 * g + 0] * sc, acc[db][4 * g + 1] * sc);
                w[1] = Elt<T>::pack2(acc[db][4 * g + 2] * sc, acc[db][4 * g + 3] * sc);
                *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * g + 4 * h) = w;
            }
    }
#endif
}

// ------------------------------------------------------------ dK / dV kernel ---
// At d = 128 the two fp32 accumulators (128 registers), the K and V rows (64) and the S
// and dP tiles fill the 256 registers of two waves per SIMD.  Non-causal, two waves per
// SIMD with a few spilled loop invariants measured 11% faster than one wave per SIMD;
// the causal variant's extra mask code spills more, and it keeps one wave per SIMD.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    // d = 128 takes 32-query tiles to stay within the register file.
    constexpr int NT = 256, KPW = 32, BK = 4 * KPW, BQ = D == 128 ? 32 : 64;
    constexpr int QB = BQ / 32, DB = D / 32, DS = D / 16, QS = BQ / 16;
    constexpr int RB = D * 2, CPR = D / 8, TILE = BQ * RB;
    // Q tile, dO tile, L2[64], D[64]: the row-value slots are sized for one 64-lane copy
    // each; with 32-query tiles the upper 32 slots receive the next rows and go unread.
    constexpr int STAGE = 2 * TILE + 2 * 64 * 4;
    constexpr int LOADS = TILE / (NT * 16);
    static_assert(LOADS >= 1 && TILE % (NT * 16) == 0 && BQ <= 64, "tile shape");

    __shared__ __attribute__((aligned(1024))) unsigned char stage0_raw[STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char stage1_raw[STAGE];
    // d = 128: the workgroup's V rows (B operand of dP^T = V dO^T) are kept in LDS rather
    // than in registers.  The 32 VGPRs this frees keep the dK/dV accumulators out of
    // scratch at two waves per SIMD (causal included): 10% faster non-causal, 17% causal.
    // At d = 64 nothing spills and the registers are faster.
    constexpr bool VLDS = D == 128;
    lds_u8* vkeep = nullptr;
    if constexpr (VLDS) {
        __shared__ __attribute__((aligned(1024))) unsigned char vkeep_raw[4 * KPW * RB];
        vkeep = (lds_u8*)vkeep_raw;
    }
    lds_u8* const stage0 = (lds_u8*)stage0_raw;
    lds_u8* const stage1 = (lds_u8*)stage1_raw;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int N = a.n;
    const int bid = remap_xcd(blockIdx.x, a.n_blocks);
    const int bh = bid / a.n_blk;
    const int kblk = bid - bh * a.n_blk;
    const int64_t head = (int64_t)bh * N * D;
    const T* Qh = reinterpret_cast<const T*>(a.q) + head;
    const T* Kh = reinterpret_cast<const T*>(a.k) + head;
    const T* Vh = reinterpret_cast<const T*>(a.v) + head;
    const T* dOh = reinterpret_cast<const T*>(a.dout) + head;
    T* dKh = reinterpret_cast<T*>(a.dk) + head;
    T* dVh = reinterpret_cast<T*>(a.dv) + head;

    const int k_wave = kblk * BK + wave * KPW;
    const int key = k_wave + l32;
    const float c = a.c;

    // K^T and V^T as B operands: this lane's key, dims 16s + 8h .. +7 (V from LDS at d = 128,
    // row-major with the 16-byte chunk swizzle, so the 16 rows of a lane group hit distinct
    // banks)
    u32x4 kf[DS], vf[VLDS ? 1 : DS];
    const int vrow = (wave * KPW + l32) * RB;
    {
        const int r = key < N ? key : 0;
#pragma unroll
        for (int s = 0; s < DS; ++s) {
            kf[s] = *reinterpret_cast<const u32x4*>(Kh + (int64_t)r * D + s * 16 + h * 8);
            const u32x4 vv = *reinterpret_cast<const u32x4*>(Vh + (int64_t)r * D + s * 16 + h * 8);
            if constexpr (VLDS)
                *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(vkeep + vrow + 16 * ((2 * s + h) ^ swz<CPR>(l32))) = vv;
            else
                vf[s] = vv;
        }
    }
    auto vfrag = [&](int s) -> u32x4 {
        if constexpr (VLDS) return lds_read16(vkeep, vrow + 16 * ((2 * s + h) ^ swz<CPR>(l32)));
        else return vf[s];
    };
    int qoff[DS];   // A-operand reads of the Q / dO tiles (rows = queries)
#pragma unroll
    for (int s = 0; s < DS; ++s) qoff[s] = l32 * RB + 16 * ((2 * s + h) ^ swz<CPR>(l32));
    int qtr[2][DB];   // transposing reads of the Q / dO tiles (as Q^T / dO^T)
    {
        const int g = lane >> 4, r = lane & 15;
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int q = 8 * aa + 4 * h + (r >> 2);
                const int dim = 32 * db + 16 * (g & 1) + 4 * (r & 3);
                qtr[aa][db] = q * RB + 16 * ((dim >> 3) ^ swz<CPR>(q)) + 2 * (dim & 7);
            }
    }
    const int head_bytes = N * D * 2;
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void*)Qh, (short)0, head_bytes, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc((void*)dOh, (short)0, head_bytes, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.l2 + (int64_t)bh * N), (short)0, N * 4, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t drs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.dsum + (int64_t)bh * N), (short)0, N * 4, kBufferRsrcWord3);
    int src_off[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int off = i * (NT * 16) + wave * 1024 + lane * 16;
        const int r = off / RB;
        const int ch = ((off % RB) >> 4) ^ swz<CPR>(r);
        src_off[i] = r * RB + ch * 16;
    }
    // query tile i into a stage; rows past N read as zeros
    auto issue = [&](int i, lds_u8* stage) {
#pragma unroll
        for (int k = 0; k < LOADS; ++k) {
            lds_u8* dst = stage + k * (NT * 16) + wave * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (__attribute__((address_space(3))) void*)dst, 16,
                                                     src_off[k] + i * BQ * RB, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ors, (__attribute__((address_space(3))) void*)(dst + TILE), 16,
                                                     src_off[k] + i * BQ * RB, 0, 0, 0);
        }
        if (wave == 0) {   // 64 lanes x 4 bytes: L2 and D of rows i*BQ .. i*BQ + 63
            __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, (__attribute__((address_space(3))) void*)(stage + 2 * TILE), 4,
                                                     lane * 4 + i * BQ * 4, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, (__attribute__((address_space(3))) void*)(stage + 2 * TILE + 64 * 4), 4,
                                                     lane * 4 + i * BQ * 4, 0, 0, 0);
        }
    };

    f32x16 dv[DB], dk[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int t = 0; t < 16; ++t) { dv[db][t] = 0.f; dk[db][t] = 0.f; }

    const int n_qt = (N + BQ - 1) / BQ;
    const int i0 = CAUSAL ? (kblk * BK) / BQ : 0;   // earlier query tiles see none of these keys

    auto tile = [&](int i, const lds_u8* sbase) {
        const int qbase = i * BQ;
        if (CAUSAL && qbase + BQ - 1 < k_wave) return;   // every query before every key of the wave
        f32x16 s[QB], dp[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int t = 0; t < 16; ++t) { s[qb][t] = 0.f; dp[qb][t] = 0.f; }
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                s[qb] = Elt<T>::mma(lds_read16(sbase, qoff[ds] + qb * 32 * RB), kf[ds], s[qb]);
                dp[qb] = Elt<T>::mma(lds_read16(sbase, TILE + qoff[ds] + qb * 32 * RB), vfrag(ds), dp[qb]);
            }
        // Phase fences: keep the scheduler from hoisting one phase's LDS reads into the
        // previous one, which overruns the register budget.
        __builtin_amdgcn_sched_barrier(0);
        // masks in a branch of their own (uniform per wave), so full tiles run none of it
        const bool tail = qbase + BQ > N;
        const bool diag = CAUSAL && (k_wave + KPW - 1 > qbase);
        if (tail || diag) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const int q = qbase + qb * 32 + 8 * (t >> 2) + 4 * h + (t & 3);
                    bool drop = q >= N;
                    if (CAUSAL) drop = drop || key > q;
                    if (drop) s[qb][t] = -INFINITY;
                }
        }
        const lds_f32* l2t = (const lds_f32*)(sbase + 2 * TILE);
        const lds_f32* ddt = (const lds_f32*)(sbase + 2 * TILE + 64 * 4);
        u32x4 pfb[QS], dsb[QS];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float pv[16], dsv[16];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int r0 = qb * 32 + 8 * g + 4 * h;   // rows r0 .. r0 + 3 of this lane
                const f32x4 l4 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(l2t + r0);
                const f32x4 d4 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(ddt + r0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 4 * g + e;
                    const float p = fast_exp2(__builtin_fmaf(s[qb][t], c, -l4[e]));
                    pv[t] = p;
                    dsv[t] = p * (dp[qb][t] - d4[e]);
                }
            }
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                u32x4 f, g2;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    f[w] = Elt<T>::pack2(pv[8 * half + 2 * w], pv[8 * half + 2 * w + 1]);
                    g2[w] = Elt<T>::pack2(dsv[8 * half + 2 * w], dsv[8 * half + 2 * w + 1]);
                }
                pfb[2 * qb + half] = f;
                dsb[2 * qb + half] = g2;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int qs = 0; qs < QS; ++qs)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const u32x2 olo = lds_read_tr(sbase, TILE + qtr[0][db] + qs * 16 * RB);
                const u32x2 ohi = lds_read_tr(sbase, TILE + qtr[1][db] + qs * 16 * RB);
                const u32x4 ot = {olo[0], olo[1], ohi[0], ohi[1]};
                dv[db] = Elt<T>::mma(ot, pfb[qs], dv[db]);
                const u32x2 qlo = lds_read_tr(sbase, qtr[0][db] + qs * 16 * RB);
                const u32x2 qhi = lds_read_tr(sbase, qtr[1][db] + qs * 16 * RB);
                const u32x4 qt = {qlo[0], qlo[1], qhi[0], qhi[1]};
                dk[db] = Elt<T>::mma(qt, dsb[qs], dk[db]);
            }
    };

    if (i0 < n_qt) issue(i0, stage0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
#pragma unroll 1
    for (int i = i0; i < n_qt; i += 2) {
        if (i + 1 < n_qt) issue(i + 1, stage1);
        tile(i, stage0);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (i + 1 < n_qt) {   // (no mid-loop exit: one set of accumulators at the loop's end)
            if (i + 2 < n_qt) issue(i + 2, stage0);
            tile(i + 1, stage1);
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
        }
    }

    if (key < N) {
        T* vrow = dVh + (int64_t)key * D;
        T* krow = dKh + (int64_t)key * D;
        const float sc = a.scale;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w, z;
                w[0] = Elt<T>::pack2(dv[db][4 * g + 0], dv[db][4 * g + 1]);
                w[1] = Elt<T>::pack2(dv[db][4 * g + 2], dv[db][4 * g + 3]);
                z[0] = Elt<T>::pack2(dk[db][4 * g + 0] * sc, dk[db][4 * g + 1] * sc);
                z[1] = Elt<T>::pack2(dk[db][4 * g + 2] * sc, dk[db][4 * g + 3] * sc);
                *reinterpret_cast<u32x2*>(vrow + db * 32 + 8 * g + 4 * h) = w;
                *reinterpret_cast<u32x2*>(krow + db * 32 + 8 * g + 4 * h) = z;
            }
    }
#endif
}

// ------------------------------------------------------------------ dispatch ---

template <typename T, int D>
static hipError_t launch_bwd_t(const BwdArgs& a, int64_t rows, int causal, hipStream_t st) {
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st,
                       reinterpret_cast<const T*>(a.o), reinterpret_cast<const T*>(a.dout), a.lse, a.dsum, a.l2, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    BwdArgs b = a;
    b.n_blk = (int)ceil_div(a.n, 128);
    b.n_blocks = (int)(rows / a.n) * b.n_blk;
    if (causal) {
        hipLaunchKernelGGL((bwd_dq_kernel<T, D, true>), dim3(b.n_blocks), dim3(256), 0, st, b);
        hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, true>), dim3(b.n_blocks), dim3(256), 0, st, b);
    } else {
        hipLaunchKernelGGL((bwd_dq_kernel<T, D, false>), dim3(b.n_blocks), dim3(256), 0, st, b);
        hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, false>), dim3(b.n_blocks), dim3(256), 0, st, b);
    }
    return hipGetLastError();
}

}  // namespace fa

int fa_launch_bwd(const fa::BwdArgs& a, int64_t rows, int dtype, int d, int causal, hipStream_t st) {
    using namespace fa;
    hipError_t e;
    if (dtype == FA_BF16) e = d == 128 ? launch_bwd_t<__bf16, 128>(a, rows, causal, st) : launch_bwd_t<__bf16, 64>(a, rows, causal, st);
    else e = d == 128 ? launch_bwd_t<_Float16, 128>(a, rows, causal, st) : launch_bwd_t<_Float16, 64>(a, rows, causal, st);
    return (int)e;
}
