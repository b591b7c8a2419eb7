// C ABI of libfa.so: argument validation, the launch plan, device checks, dispatch.
// Every validation step runs before any HIP call, so the error paths work (and are
// tested) on a machine without a GPU.

#include <hip/hip_runtime.h>

#include <math.h>
#include <mutex>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fa_fp8.h"
#include "fa_internal.h"
#include "fa_splitkv.h"

// Static split-KV scratch of fa_fwd_splitkv_qk_noalloc: every GPU the library runs on holds
// its own copy for the life of the process.  In host code `scratch` names a host-side
// stand-in, not device memory: kernels get the device address that hipGetSymbolAddress
// returns for the current device (device_scratch below), never `scratch` itself.
static constexpr size_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kVersion = 400;  // 0.4.0
constexpr int kMaxDevices = 64;
constexpr int64_t kMaxGrid = int64_t(1) << 31;   // workgroups per launch (32-bit ids)

struct DeviceInfo {
    std::once_flag once;
    bool gfx950 = false;
    // address of this device's copy of `scratch` (fa_fwd_splitkv_qk_noalloc), looked up once
    std::once_flag scratch_once;
    void* scratch = nullptr;
};
DeviceInfo g_devices[kMaxDevices];

// FA_OK if the calling thread's current HIP device is a gfx950.
fa_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return FA_ERR_DEVICE;
    }
    DeviceInfo& info = g_devices[dev];
    std::call_once(info.once, [&] {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess)
            info.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        (void)hipGetLastError();
    });
    return info.gfx950 ? FA_OK : FA_ERR_DEVICE;
}

// Device address of the current device's `scratch` (the device must have passed
// check_device), or nullptr if the runtime could not resolve it.
void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    DeviceInfo& info = g_devices[dev];
    std::call_once(info.scratch_once, [&] {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess) info.scratch = ptr;
        else (void)hipGetLastError();
    });
    return info.scratch;
}

// FA_LOG set (and not "0"): each launch prints its plan to stderr.  Read on every call.
bool log_enabled() {
    const char* e = getenv("FA_LOG");
    return e && *e && strcmp(e, "0") != 0;
}

const char* dtype_name(int dtype) { return dtype == FA_F32 ? "fp32" : dtype == FA_F16 ? "fp16" : "bf16"; }

// The chooser's plan, or the FA_TILE override when set (FA_ERR_TILE if it names no compiled
// kernel for this dtype and head dim).  *overridden tells which.
fa_status make_plan(int64_t B, int64_t H, int64_t N, int64_t d, int dtype, int causal, fa_plan* plan,
                    bool* overridden) {
    *plan = fa::choose_fwd_plan(B, H, N, d, dtype, causal);
    const char* tile = getenv("FA_TILE");
    *overridden = tile && *tile;
    if (!fa::apply_tile_override(plan, tile, B, H, N, d, dtype, causal)) return FA_ERR_TILE;
    fa::finalize_tail(plan, dtype, B, H, N, N, d, causal);
    return FA_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Whether the byte ranges [p, p + np) and [q, q + nq) share a byte.
bool overlaps(const void* p, size_t np, const void* q, size_t nq) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + nq && b < a + np;
}

// Shape / dtype checks shared by the plan query and the launches.
fa_status check_problem(int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
    if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
    if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    // per-head byte offsets (16-bit elements) are 32-bit signed inside the kernels
    if (N >= (int64_t(1) << 30) / d) return FA_ERR_SHAPE;   // N * d >= 2^30, without forming N * d
    if (B > 0 && H > (int64_t(1) << 31) / B) return FA_ERR_SHAPE;
    const int64_t bh = B * H;
    if (bh > 0 && N > 0 && bh * fa::ceil_div(N, 128) >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
    return FA_OK;
}

// Nk keys per head for N query rows (Nk = N except in a split-KV call with unequal lengths;
// already validated there).
fa_status fwd_common(const void* Q, const void* K, const void* V, void* O, float* LSE,
                     int64_t B, int64_t H, int64_t N, int64_t d, float scale, fa_dtype dtype,
                     hipStream_t stream, int causal, int64_t Nk = -1) {
    if (Nk < 0) Nk = N;
    fa_status st = check_problem(B, H, N, d, dtype);
    if (st != FA_OK) return st;
    if (B * H * N == 0) return FA_OK;   // empty tensors may carry NULL data pointers
    if (!Q || !K || !V || !O || !LSE) return FA_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(LSE, 4))
        return FA_ERR_ALIGN;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
    fa_plan plan;
    bool overridden;
    st = make_plan(B, H, N, d, dtype, causal, &plan, &overridden);
    if (st != FA_OK) return st;
    if (plan.grid >= kMaxGrid) return FA_ERR_SHAPE;
    fa::finalize_tail(&plan, dtype, B, H, N, Nk, d, causal);
    // Tail first parks its partials in O ahead of the main launch: not when O shares memory
    // with an input (or the LSE), which would then be overwritten before it is read.
    const size_t elt = dtype == FA_F32 ? 4 : 2, qo_bytes = (size_t)(B * H * N * d) * elt;
    const size_t kv_bytes = (size_t)(B * H * Nk * d) * elt, lse_bytes = (size_t)(B * H * N) * sizeof(float);
    bool tail_first = plan.waves == 8 && plan.tail_kv_splits > 1;
    if (tail_first && (overlaps(O, qo_bytes, Q, qo_bytes) || overlaps(O, qo_bytes, K, kv_bytes) ||
                       overlaps(O, qo_bytes, V, kv_bytes) || overlaps(O, qo_bytes, LSE, lse_bytes))) {
        tail_first = false;
        plan.tail_kv_splits = 1;
        plan.grid = B * H * fa::ceil_div(N, plan.block_q);
    }
    const int64_t n_main = tail_first ? N / 256 * 256 : N;
    if (log_enabled()) {
        char tail_note[96] = "";
        if (tail_first)
            snprintf(tail_note, sizeof tail_note, " (the last %lld rows first: %d key ranges per head, merged)",
                     (long long)(N - n_main), plan.tail_kv_splits);
        else if (plan.tail_kv_splits > 1)
            snprintf(tail_note, sizeof tail_note, " (the last block's waves split the key tiles)");
        fprintf(stderr, "fa_fwd%s: B=%lld H=%lld N=%lld Nk=%lld d=%lld %s -> Br=%d Bc=%d waves=%d grid=%lld lds=%d%s%s%s\n",
                causal ? "_causal" : "", (long long)B, (long long)H, (long long)N, (long long)Nk, (long long)d,
                dtype_name(dtype), plan.block_q, plan.block_k, plan.waves, (long long)plan.grid, plan.lds_bytes,
                plan.wave_kv_splits > 1 ? " (waves split the key tiles)" : "", tail_note,
                overridden ? " (FA_TILE)" : "");
    }
    st = check_device();
    if (st != FA_OK) return st;

    fa::FwdArgs a;
    a.q = Q;
    a.k = K;
    a.v = V;
    a.o = O;
    a.lse = LSE;
    a.n = (int)N;
    a.nk = (int)Nk;
    a.n_qblk = (int)(tail_first ? n_main / plan.block_q : fa::ceil_div(N, plan.block_q));
    a.n_blocks = (int)plan.grid;
    a.c = (float)((double)scale * 1.4426950408889634074);  // scale * log2(e)
    a.splits = 1;
    a.tiles_per_split = 0;
    a.o_part = nullptr;
    a.lse_part = nullptr;
    if (tail_first) {
        // the last r rows of every head: split-KV partials parked in the head's first O rows;
        // the main launch's first block of each head merges them into its rows n_main .. N - 1
        // before its own outputs overwrite them
        const int S = plan.tail_kv_splits;
        const int64_t r = N - n_main, tiles = fa::ceil_div(N, fa::splitkv_block_k(d));
        fa::FwdArgs t = a;
        t.qblk0 = (int)(n_main / 128);
        t.n_qblk = 1;
        t.splits = S;
        t.tiles_per_split = (int)fa::ceil_div(tiles, S);
        t.n_blocks = (int)(B * H * S);
        t.o_part = reinterpret_cast<float*>(O);
        t.lse_part = t.o_part + (int64_t)S * r * d;
        t.po_head = t.pl_head = N * d * (int64_t)elt / (int64_t)sizeof(float);
        t.po_split = r * d;
        t.pl_split = r;
        t.part_row0 = (int)n_main;
        fa::MergeArgs m{};   // no rows: no merge launch
        if (fa_launch_fwd_splitkv(t, m, dtype, (int)d, stream) != 0) return FA_ERR_LAUNCH;
        a.splits = S;
        a.o_part = t.o_part;
        a.lse_part = t.lse_part;
        a.po_head = t.po_head;
        a.po_split = t.po_split;
        a.pl_head = t.pl_head;
        a.pl_split = t.pl_split;
        a.part_row0 = t.part_row0;
    }
    const int e = fa_launch_fwd(a, plan, dtype, (int)d, causal, stream);
    return e == 0 ? FA_OK : FA_ERR_LAUNCH;
}

// Shapes of a split-KV call: N query rows and Nk keys per head, both within the 32-bit
// index math; queries with no keys to attend to are a shape error.
fa_status check_splitkv(int64_t B, int64_t H, int64_t N, int64_t Nk, int64_t d, int dtype, int32_t splits) {
    fa_status st = check_problem(B, H, N, d, dtype);
    if (st != FA_OK) return st;
    st = check_problem(B, H, Nk, d, dtype);
    if (st != FA_OK) return st;
    if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
    if (splits < 0 || splits > fa::kMaxKvSplits) return FA_ERR_SHAPE;
    if (B * H * N > 0 && Nk == 0) return FA_ERR_SHAPE;
    return FA_OK;
}

// The split count a call will use: splits = 0 picks, more than the key tiles is clamped.
int32_t effective_splits(int64_t B, int64_t H, int64_t N, int64_t Nk, int64_t d, int32_t splits) {
    if (splits == 0) splits = fa::choose_kv_splits(B, H, N, Nk, d);
    const int64_t tiles = fa::ceil_div(Nk, fa::splitkv_block_k(d));
    return splits > tiles ? (int32_t)tiles : splits;
}

// use_scratch: the partials go to the static `scratch` (fa_fwd_splitkv_qk_noalloc); ws and
// ws_bytes are then ignored.
fa_status splitkv_common(const void* Q, const void* K, const void* V, void* O, float* LSE, void* ws,
                         size_t ws_bytes, int64_t B, int64_t H, int64_t N, int64_t Nk, int64_t d, float scale,
                         fa_dtype dtype, int32_t splits, hipStream_t stream, bool use_scratch = false) {
    fa_status st = check_splitkv(B, H, N, Nk, d, dtype, splits);
    if (st != FA_OK) return st;
    if (B * H * N == 0) return FA_OK;
    if (!Q || !K || !V || !O || !LSE) return FA_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(LSE, 4))
        return FA_ERR_ALIGN;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
    splits = effective_splits(B, H, N, Nk, d, splits);
    const int64_t tiles = fa::ceil_div(Nk, fa::splitkv_block_k(d));
    if (splits <= 1) return fwd_common(Q, K, V, O, LSE, B, H, N, d, scale, dtype, stream, 0, Nk);
    if (B * H * fa::ceil_div(N, 128) * splits >= kMaxGrid) return FA_ERR_SHAPE;
    const size_t need = fa::splitkv_workspace_bytes(B, H, N, d, splits);
    if (use_scratch) {
        if (need > kScratchBytes) return FA_ERR_SCRATCH;
    } else if (!ws || !aligned(ws, 256) || ws_bytes < need) {
        return FA_ERR_WORKSPACE;
    }
    if (log_enabled())
        fprintf(stderr,
                "fa_fwd_splitkv: B=%lld H=%lld Nq=%lld Nk=%lld d=%lld %s -> splits=%d of %lld key tiles (Bc=%d), "
                "grid=%lld, partials %zu bytes in %s\n",
                (long long)B, (long long)H, (long long)N, (long long)Nk, (long long)d, dtype_name(dtype), splits,
                (long long)tiles, fa::splitkv_block_k(d), (long long)(B * H * fa::ceil_div(N, 128) * splits), need,
                use_scratch ? "the static scratch" : "the caller's workspace");
    st = check_device();
    if (st != FA_OK) return st;
    if (use_scratch) {
        ws = device_scratch();
        if (!ws) return FA_ERR_DEVICE;
    }

    fa::FwdArgs a;
    a.q = Q;
    a.k = K;
    a.v = V;
    a.o = O;
    a.lse = LSE;
    a.n = (int)N;
    a.nk = (int)Nk;
    a.n_qblk = (int)fa::ceil_div(N, 128);
    a.splits = splits;
    a.tiles_per_split = (int)fa::ceil_div(tiles, splits);
    a.n_blocks = (int)(B * H * a.n_qblk * splits);
    a.c = (float)((double)scale * 1.4426950408889634074);
    const size_t o_bytes = (size_t)splits * (size_t)(B * H * N) * (size_t)d * sizeof(float);
    a.o_part = reinterpret_cast<float*>(ws);
    a.lse_part = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(ws) + (o_bytes + 255) / 256 * 256);
    a.po_head = N * d;   // [splits][B*H*N][d] and [splits][B*H*N]
    a.po_split = B * H * N * d;
    a.pl_head = N;
    a.pl_split = B * H * N;
    fa::MergeArgs m;
    m.o_part = a.o_part;
    m.lse_part = a.lse_part;
    m.o = O;
    m.lse = LSE;
    m.rows = B * H * N;
    m.rows_per_head = (int)N;
    m.splits = splits;
    m.po_head = a.po_head;
    m.po_split = a.po_split;
    m.pl_head = a.pl_head;
    m.pl_split = a.pl_split;
    m.out_head = N;
    m.out_row0 = 0;
    const int e = fa_launch_fwd_splitkv(a, m, dtype, (int)d, stream);
    return e == 0 ? FA_OK : FA_ERR_LAUNCH;
}

// Shape checks of the fp8 mode: check_problem plus the padded V^T head in 32-bit offsets.
fa_status check_fp8_problem(int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
    fa_status st = check_problem(B, H, N, d, dtype);
    if (st != FA_OK) return st;
    if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
    if (N > 0 && fa::fp8_padded_len(N) * d >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
    return FA_OK;
}

fa_status bwd_common(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                     const float* LSE, void* dQ, void* dK, void* dV, void* ws, size_t ws_bytes,
                     int64_t B, int64_t H, int64_t N, int64_t d, float scale, fa_dtype dtype,
                     hipStream_t stream, int causal) {
    fa_status st = check_problem(B, H, N, d, dtype);
    if (st != FA_OK) return st;
    if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
    if (B * H * N == 0) return FA_OK;
    if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV) return FA_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(dO, 16) ||
        !aligned(dQ, 16) || !aligned(dK, 16) || !aligned(dV, 16) || !aligned(LSE, 4))
        return FA_ERR_ALIGN;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
    if (!ws || !aligned(ws, 256) || ws_bytes < fa::bwd_workspace_bytes(B, H, N)) return FA_ERR_WORKSPACE;
    if (log_enabled())
        fprintf(stderr, "fa_bwd%s: B=%lld H=%lld N=%lld d=%lld %s -> preprocess, dQ over 128-row query blocks, "
                "dK/dV over 128-key blocks\n", causal ? "_causal" : "", (long long)B, (long long)H, (long long)N,
                (long long)d, dtype_name(dtype));
    st = check_device();
    if (st != FA_OK) return st;

    const size_t one = fa::bwd_workspace_bytes(B, H, N) / 2;
    fa::BwdArgs a;
    a.q = Q;
    a.k = K;
    a.v = V;
    a.o = O;
    a.dout = dO;
    a.lse = LSE;
    a.dq = dQ;
    a.dk = dK;
    a.dv = dV;
    a.dsum = reinterpret_cast<float*>(ws);
    a.l2 = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(ws) + one);
    a.n = (int)N;
    a.n_blk = 0;
    a.n_blocks = 0;
    a.c = (float)((double)scale * 1.4426950408889634074);
    a.scale = scale;
    const int e = fa_launch_bwd(a, B * H * N, dtype, (int)d, causal, stream);
    return e == 0 ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t fa_fwd_splitkv_qk_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, fa_dtype dtype,
                                         int32_t splits) {
    if (check_splitkv(B, H, Nq, Nk, d, dtype, splits) != FA_OK || B * H * Nq == 0) return 0;
    return fa::splitkv_workspace_bytes(B, H, Nq, d, effective_splits(B, H, Nq, Nk, d, splits));
}

int32_t fa_fwd_splitkv_qk_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, fa_dtype dtype) {
    if (check_splitkv(B, H, Nq, Nk, d, dtype, 0) != FA_OK || B * H * Nq == 0) return 1;
    return fa::choose_kv_splits(B, H, Nq, Nk, d);
}

fa_status fa_fwd_splitkv_qk(const void* Q, const void* K, const void* V, void* O, float* LSE, void* workspace,
                            size_t ws_bytes, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                            fa_dtype dtype, int32_t splits, hipStream_t stream) {
    return splitkv_common(Q, K, V, O, LSE, workspace, ws_bytes, B, H, Nq, Nk, d, scale, dtype, splits, stream);
}

fa_status fa_fwd_splitkv_qk_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B,
                                    int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale, fa_dtype dtype,
                                    int32_t splits, hipStream_t stream) {
    return splitkv_common(Q, K, V, O, LSE, nullptr, 0, B, H, Nq, Nk, d, scale, dtype, splits, stream,
                          /*use_scratch=*/true);
}

size_t fa_fwd_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, fa_dtype dtype, int32_t splits) {
    return fa_fwd_splitkv_qk_workspace_bytes(B, H, N, N, d, dtype, splits);
}

int32_t fa_fwd_splitkv_splits(int64_t B, int64_t H, int64_t N, int64_t d, fa_dtype dtype) {
    return fa_fwd_splitkv_qk_splits(B, H, N, N, d, dtype);
}

fa_status fa_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* LSE, void* workspace,
                         size_t ws_bytes, int64_t B, int64_t H, int64_t N, int64_t d, float scale, fa_dtype dtype,
                         int32_t splits, hipStream_t stream) {
    return splitkv_common(Q, K, V, O, LSE, workspace, ws_bytes, B, H, N, N, d, scale, dtype, splits, stream);
}

int64_t fa_fp8_padded_len(int64_t N) {
    return (N < 0 || N > INT64_MAX - fa::kFp8Pad) ? 0 : fa::fp8_padded_len(N);
}

int64_t fa_fp8_scale_blocks(int64_t N) { return N < 0 ? 0 : fa::fp8_scale_blocks(N); }

fa_status fa_quantize_fp8(const void* X, void* X8, float* scales, int64_t B, int64_t H, int64_t N, int64_t d,
                          fa_dtype dtype, int32_t transpose, hipStream_t stream) {
    fa_status st = check_fp8_problem(B, H, N, d, dtype);
    if (st != FA_OK) return st;
    if (transpose != 0 && transpose != 1) return FA_ERR_UNSUPPORTED;
    if (B * H * N == 0) return FA_OK;
    const int64_t per_head = transpose ? fa::fp8_padded_len(N) / fa::kFp8Block : fa::fp8_scale_blocks(N);
    if (B * H * per_head >= kMaxGrid) return FA_ERR_SHAPE;
    if (!X || !X8 || !scales) return FA_ERR_NULL;
    if (!aligned(X, 16) || !aligned(X8, 16) || !aligned(scales, 4)) return FA_ERR_ALIGN;
    st = check_device();
    if (st != FA_OK) return st;
    fa::QuantArgs a;
    a.x = X;
    a.x8 = reinterpret_cast<unsigned char*>(X8);
    a.scales = scales;
    a.n = (int)N;
    a.np = (int)fa::fp8_padded_len(N);
    a.nb = (int)fa::fp8_scale_blocks(N);
    a.blocks_per_head = transpose ? a.np / fa::kFp8Block : a.nb;
    const int e = fa_launch_quantize_fp8(a, B * H, dtype, (int)d, transpose, stream);
    return e == 0 ? FA_OK : FA_ERR_LAUNCH;
}

namespace {
fa_status fwd_fp8_common(const void* Q8, const void* K8, const void* Vt8, const float* q_scale, const float* k_scale,
                         const float* v_scale, void* O, float* LSE, int64_t B, int64_t H, int64_t N, int64_t d,
                         float scale, fa_dtype out_dtype, hipStream_t stream, int causal) {
    fa_status st = check_fp8_problem(B, H, N, d, out_dtype);
    if (st != FA_OK) return st;
    if (B * H * N == 0) return FA_OK;
    if (!Q8 || !K8 || !Vt8 || !q_scale || !k_scale || !v_scale || !O || !LSE) return FA_ERR_NULL;
    if (!aligned(Q8, 16) || !aligned(K8, 16) || !aligned(Vt8, 16) || !aligned(O, 16) || !aligned(q_scale, 4) ||
        !aligned(k_scale, 4) || !aligned(v_scale, 4) || !aligned(LSE, 4))
        return FA_ERR_ALIGN;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
    if (log_enabled())
        fprintf(stderr, "fa_fwd_fp8%s: B=%lld H=%lld N=%lld d=%lld -> O %s, Br=%d Bc=64 waves=4 grid=%lld\n",
                causal ? "_causal" : "", (long long)B, (long long)H, (long long)N, (long long)d, dtype_name(out_dtype),
                fa::kFp8BlockQ, (long long)(B * H * fa::ceil_div(N, fa::kFp8BlockQ)));
    st = check_device();
    if (st != FA_OK) return st;
    fa::Fp8Args a;
    a.q8 = reinterpret_cast<const unsigned char*>(Q8);
    a.k8 = reinterpret_cast<const unsigned char*>(K8);
    a.vt8 = reinterpret_cast<const unsigned char*>(Vt8);
    a.qs = q_scale;
    a.ks = k_scale;
    a.vs = v_scale;
    a.o = O;
    a.lse = LSE;
    a.n = (int)N;
    a.np = (int)fa::fp8_padded_len(N);
    a.nb = (int)fa::fp8_scale_blocks(N);
    a.n_qblk = (int)fa::ceil_div(N, fa::kFp8BlockQ);
    a.n_blocks = (int)(B * H * a.n_qblk);
    a.c = (float)((double)scale * 1.4426950408889634074);
    const int e = fa_launch_fwd_fp8(a, out_dtype, (int)d, causal, stream);
    return e == 0 ? FA_OK : FA_ERR_LAUNCH;
}
}  // namespace

fa_status fa_fwd_fp8(const void* Q8, const void* K8, const void* Vt8, const float* q_scale, const float* k_scale,
                     const float* v_scale, void* O, float* LSE, int64_t B, int64_t H, int64_t N, int64_t d,
                     float scale, fa_dtype out_dtype, hipStream_t stream) {
    return fwd_fp8_common(Q8, K8, Vt8, q_scale, k_scale, v_scale, O, LSE, B, H, N, d, scale, out_dtype, stream, 0);
}

fa_status fa_fwd_fp8_causal(const void* Q8, const void* K8, const void* Vt8, const float* q_scale,
                            const float* k_scale, const float* v_scale, void* O, float* LSE, int64_t B, int64_t H,
                            int64_t N, int64_t d, float scale, fa_dtype out_dtype, hipStream_t stream) {
    return fwd_fp8_common(Q8, K8, Vt8, q_scale, k_scale, v_scale, O, LSE, B, H, N, d, scale, out_dtype, stream, 1);
}

size_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, fa_dtype dtype) {
    if (check_problem(B, H, N, d, dtype) != FA_OK) return 0;
    return fa::bwd_workspace_bytes(B, H, N);
}

fa_status fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                 const float* LSE, void* dQ, void* dK, void* dV, void* workspace, size_t ws_bytes,
                 int64_t B, int64_t H, int64_t N, int64_t d, float scale, fa_dtype dtype, hipStream_t stream) {
    return bwd_common(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, ws_bytes, B, H, N, d, scale, dtype, stream, 0);
}

fa_status fa_bwd_causal(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                        const float* LSE, void* dQ, void* dK, void* dV, void* workspace, size_t ws_bytes,
                        int64_t B, int64_t H, int64_t N, int64_t d, float scale, fa_dtype dtype,
                        hipStream_t stream) {
    return bwd_common(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, ws_bytes, B, H, N, d, scale, dtype, stream, 1);
}


fa_status fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                 int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                 fa_dtype dtype, hipStream_t stream) {
    return fwd_common(Q, K, V, O, LSE, B, H, N, d, scale, dtype, stream, 0);
}

fa_status fa_fwd_causal(const void* Q, const void* K, const void* V, void* O, float* LSE,
                        int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                        fa_dtype dtype, hipStream_t stream) {
    return fwd_common(Q, K, V, O, LSE, B, H, N, d, scale, dtype, stream, 1);
}

fa_status fa_fwd_plan(int64_t B, int64_t H, int64_t N, int64_t d, fa_dtype dtype, int causal,
                      fa_plan* plan) {
    if (!plan) return FA_ERR_NULL;
    fa_status st = check_problem(B, H, N, d, dtype);
    if (st != FA_OK) return st;
    memset(plan, 0, sizeof(*plan));
    if (B * H * N == 0) return FA_OK;
    bool overridden;
    fa_plan p;
    st = make_plan(B, H, N, d, dtype, causal, &p, &overridden);
    if (st != FA_OK) return st;
    *plan = p;
    return plan->grid >= kMaxGrid ? FA_ERR_SHAPE : FA_OK;
}

const char* fa_status_str(fa_status s) {
    switch (s) {
        case FA_OK: return "FA_OK";
        case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
        case FA_ERR_SHAPE: return "FA_ERR_SHAPE: negative or too large B/H/N";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dim must be 64 or 128, dtype f32/f16/bf16";
        case FA_ERR_ALIGN: return "FA_ERR_ALIGN: tensors need 16-byte alignment (LSE 4-byte)";
        case FA_ERR_SCALE: return "FA_ERR_SCALE: scale must be finite and > 0";
        case FA_ERR_DEVICE: return "FA_ERR_DEVICE: no HIP device or the current device is not gfx950";
        case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: kernel launch failed";
        case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
        case FA_ERR_TILE: return "FA_ERR_TILE: FA_TILE names no compiled kernel for this dtype and head dim";
        case FA_ERR_SCRATCH:
            return "FA_ERR_SCRATCH: the split partials need more than the static scratch (FA_NOALLOC_SCRATCH_BYTES)";
    }
    return "FA_ERR_UNKNOWN";
}

int fa_version(void) { return kVersion; }

}  // extern "C"
