// Internal declarations of the block-scaled fp8 mode, shared by the C ABI (fa_api.hip)
// and its kernels (fa_fp8_kernel.hip).
#pragma once

#include "fa_internal.h"

namespace fa {

// ------------------------------------------------------------ block-scaled fp8 ---
// Q, K and V in OCP E4M3 with one power-of-two scale per 64 rows of a (batch, head).
constexpr int kFp8Block = 64;      // rows per scale block
constexpr int kFp8TileK = 64;      // keys per LDS tile of the fp8 forward (one scale block)
constexpr int kFp8Pad = 128;       // V^T rows are padded to a multiple of this (code 0)
inline int64_t fp8_padded_len(int64_t N) { return ceil_div(N, kFp8Pad) * kFp8Pad; }
inline int64_t fp8_scale_blocks(int64_t N) { return ceil_div(N, kFp8Block); }

// Quantiser arguments.  One workgroup per (batch*head, 64-row block).
struct QuantArgs {
    const void* x;      // [B, H, N, d] bf16 / fp16
    unsigned char* x8;  // [B, H, N, d] codes, or [B, H, d, Np] when transposed
    float* scales;      // [B, H, nb]
    int n;
    int np;             // padded length (transposed layout only)
    int nb;             // scale blocks per head = ceil(N / 64)
    int blocks_per_head;   // grid blocks per head: nb, or Np / 64 when transposed
};

// fp8 forward arguments.
struct Fp8Args {
    const unsigned char* q8;   // [B, H, N, d]
    const unsigned char* k8;   // [B, H, N, d]
    const unsigned char* vt8;  // [B, H, d, Np]
    const float* qs;           // [B, H, nb] block scales (powers of two)
    const float* ks;
    const float* vs;
    void* o;                   // [B, H, N, d] bf16 / fp16
    float* lse;                // [B, H, N]
    int n;
    int np;
    int nb;
    int n_qblk;
    int n_blocks;
    float c;                   // scale * log2(e)
};
// Query rows per workgroup of the fp8 forward: 4 waves x 32 rows, three workgroups per CU
// (64-key tiles: 32 KiB of LDS, at most 168 VGPRs).  Measured at B=4 H=32 N=16384 d=128: two
// 4-wave workgroups per CU were 8% faster than one 8-wave workgroup (independent workgroups
// drift out of phase, so one's softmax overlaps another's MFMAs, where the waves of one
// workgroup meet at every tile's barrier), and a third per CU another 8%.
constexpr int kFp8BlockQ = 128;

}  // namespace fa

// Launchers implemented in fa_fp8_kernel.hip (0 or the hipError_t of the launch).
// in_dtype: input type of the quantiser; out_dtype: O's type in the forward.
int fa_launch_quantize_fp8(const fa::QuantArgs& a, int64_t bh, int in_dtype, int d, int transpose, hipStream_t stream);
int fa_launch_fwd_fp8(const fa::Fp8Args& a, int out_dtype, int d, int causal, hipStream_t stream);

