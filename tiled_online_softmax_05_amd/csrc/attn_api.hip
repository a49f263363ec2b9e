// C ABI of libattn.so: argument validation, the tile / occupancy selector
// and dispatch to the gfx950 kernels.  See include/attn.h for the contract.
#include "attn.h"
#include "attn_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

namespace attn {
namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return ATTN_OK;
}

__global__ void empty_rows_kernel(void* __restrict__ o, int o_bytes, float* __restrict__ lse,
                                  size_t o_elems, size_t rows) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < o_elems; i += stride) {
        if (o_bytes == 4)
            static_cast<float*>(o)[i] = 0.f;
        else
            static_cast<uint16_t*>(o)[i] = 0;  // +0.0 in bf16
    }
    if (lse != nullptr)
        for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows; i += stride)
            lse[i] = -INFINITY;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

int in_bytes(int dtype) { return dtype == ATTN_F32 ? 4 : 2; }
int out_bytes(int dtype) { return dtype == ATTN_BF16 ? 2 : 4; }

// The selector.  Query rows per workgroup shrink until the grid has at
// least one workgroup per compute unit (256 on MI355X) or the smallest
// shape is reached; key rows per tile follow the key length.
int select(int d, int Sq, int Skv, int BH, int dtype, bool causal, Tiles* t) {
    constexpr long kCUs = 256;
    auto wgs = [&](int bm) { return (long)BH * ((Sq + bm - 1) / bm); };
    if (dtype == ATTN_F32) {
        if (!(d == 32 || d == 64 || d == 128))
            return fail(ATTN_ERR_UNSUPPORTED, "fp32 head dim %d not built (32, 64, 128)", d);
        int bn = Skv > 32 ? 64 : (Skv > 16 ? 32 : 16);
        int bm = 64;
        while (bm > 16 && (wgs(bm) < kCUs || Sq <= bm / 2)) bm /= 2;
        t->block_m = bm;
        t->block_n = bn;
        t->waves = bm / 16;
        t->lds_bytes = f32_lds_bytes(d, bm, bn);
        return ATTN_OK;
    }
    if (!(d == 64 || d == 128))
        return fail(ATTN_ERR_UNSUPPORTED, "bf16 head dim %d not built (64, 128)", d);
    // Workgroups of 128 query rows (four waves, two workgroups per CU) when
    // that gives every CU a workgroup, else 64; causal workgroups take a heavy
    // and a light query tile each.  32-key tiles: the pipelined kernel holds
    // two score tiles in registers, and 64-key tiles would not fit at two
    // waves per SIMD.  (256-row workgroups of eight waves are built for d=128
    // but measured no faster.)
    auto items = [&](int bm) {
        const long n_qt = (Sq + bm - 1) / bm;
        return (long)BH * (causal ? (n_qt + 1) / 2 : n_qt);
    };
    int bm = items(128) >= kCUs ? 128 : 64;
    int bn = 32;
    t->block_m = bm;
    t->block_n = bn;
    t->waves = bm / 32;
    t->lds_bytes = bf16_lds_bytes(d, bm, bn);
    return ATTN_OK;
}

int validate(const Problem& p) {
    if (p.dtype != ATTN_F32 && p.dtype != ATTN_BF16 && p.dtype != ATTN_BF16_OUT_F32)
        return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", p.dtype);
    if (p.B < 0 || p.H < 0 || p.Sq < 0 || p.Skv < 0)
        return fail(ATTN_ERR_INVALID_ARG, "negative size (B=%d H=%d Sq=%d Skv=%d)", p.B, p.H,
                    p.Sq, p.Skv);
    if (p.d <= 0) return fail(ATTN_ERR_INVALID_ARG, "head dim %d must be positive", p.d);
    if (p.dtype == ATTN_F32 ? !(p.d == 32 || p.d == 64 || p.d == 128)
                            : !(p.d == 64 || p.d == 128))
        return fail(ATTN_ERR_UNSUPPORTED, "head dim %d not built for dtype %d", p.d, p.dtype);
    if (!std::isfinite(p.scale) || !(p.scale > 0.f))
        return fail(ATTN_ERR_INVALID_ARG, "scale must be finite and > 0 (got %g)",
                    (double)p.scale);
    const int64_t bh = (int64_t)p.B * p.H;
    if (bh > INT32_MAX) return fail(ATTN_ERR_INVALID_ARG, "B*H too large");
    if (bh * (int64_t)p.Sq > INT32_MAX || bh * (int64_t)p.Skv > INT32_MAX)
        return fail(ATTN_ERR_INVALID_ARG, "B*H*S exceeds 2^31 rows");
    // one head's Q, K or V (at 4 bytes per element) must stay below 2 GiB:
    // the kernels address a head with 32-bit byte offsets
    if ((int64_t)p.Sq * p.d * 4 > INT32_MAX || (int64_t)p.Skv * p.d * 4 > INT32_MAX)
        return fail(ATTN_ERR_INVALID_ARG, "sequence too long for one head (S*d*4 >= 2^31)");
    if (bh == 0 || p.Sq == 0) return ATTN_OK;
    if (p.q == nullptr || p.o == nullptr)
        return fail(ATTN_ERR_INVALID_ARG, "q and o must be non-null");
    if (p.Skv > 0 && (p.k == nullptr || p.v == nullptr))
        return fail(ATTN_ERR_INVALID_ARG, "k and v must be non-null when Skv > 0");
    const void* ptrs[4] = {p.q, p.k, p.v, p.o};
    for (const void* ptr : ptrs)
        if (ptr != nullptr && (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0)
            return fail(ATTN_ERR_MISALIGNED, "q, k, v, o must be 16-byte aligned");
    if (p.lse != nullptr && (reinterpret_cast<uintptr_t>(p.lse) & 3u) != 0)
        return fail(ATTN_ERR_MISALIGNED, "lse must be 4-byte aligned");
    const size_t nq = (size_t)bh * p.Sq * p.d, nkv = (size_t)bh * p.Skv * p.d;
    const size_t ob = nq * out_bytes(p.dtype);
    const int ib = in_bytes(p.dtype);
    if (overlaps(p.o, ob, p.q, nq * ib) || overlaps(p.o, ob, p.k, nkv * ib) ||
        overlaps(p.o, ob, p.v, nkv * ib) || overlaps(p.o, ob, p.lse, (size_t)bh * p.Sq * 4))
        return fail(ATTN_ERR_INVALID_ARG, "o overlaps an input or lse");
    return ATTN_OK;
}

int run(const Problem& p, int block_m, int block_n) {
    int st = validate(p);
    if (st != ATTN_OK) return st;
    const int bh = p.B * p.H;
    if (bh == 0 || p.Sq == 0) return ok();
    Tiles t{};
    if (block_m == 0 && block_n == 0) {
        st = select(p.d, p.Sq, p.Skv, bh, p.dtype, p.causal, &t);
        if (st != ATTN_OK) return st;
    } else {
        const bool sup = p.dtype == ATTN_F32 ? f32_tiles_supported(p.d, block_m, block_n)
                                             : bf16_tiles_supported(p.d, block_m, block_n);
        if (!sup)
            return fail(ATTN_ERR_UNSUPPORTED, "tile %dx%d not built for d=%d dtype=%d", block_m,
                        block_n, p.d, p.dtype);
        t.block_m = block_m;
        t.block_n = block_n;
    }
    hipError_t e;
    if (p.Skv == 0) {
        const size_t elems = (size_t)bh * p.Sq * p.d;
        const int blocks = (int)std::min<size_t>((elems + 255) / 256, 4096);
        hipLaunchKernelGGL(empty_rows_kernel, dim3(blocks), dim3(256), 0, p.stream, p.o,
                           out_bytes(p.dtype), p.lse, elems, (size_t)bh * p.Sq);
        e = hipGetLastError();
    } else if (p.dtype == ATTN_F32) {
        e = launch_f32(p, t);
    } else {
        e = launch_bf16(p, t);
    }
    if (e != hipSuccess)
        return fail(ATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace
}  // namespace attn

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int Sq, int Skv, int d, float scale, int causal, int dtype, void* stream) {
    return attn_fwd_tiles(q, k, v, o, lse, B, H, Sq, Skv, d, scale, causal, dtype, stream, 0, 0);
}

int attn_fwd_tiles(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int H, int Sq, int Skv, int d, float scale, int causal, int dtype,
                   void* stream, int block_m, int block_n) {
    if (causal != 0 && causal != 1)
        return attn::fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
    if (block_m < 0 || block_n < 0 || ((block_m == 0) != (block_n == 0)))
        return attn::fail(ATTN_ERR_INVALID_ARG, "block_m, block_n must both be 0 or positive");
    attn::Problem p{q, k, v, o, lse, B, H, Sq, Skv, d, scale, causal == 1, dtype,
                    static_cast<hipStream_t>(stream)};
    return attn::run(p, block_m, block_n);
}

int attn_select_tiles(int d, int Sq, int Skv, int BH, int dtype, int causal, int* block_m,
                      int* block_n, int* waves, int* lds_bytes) {
    if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_BF16_OUT_F32)
        return attn::fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (causal != 0 && causal != 1)
        return attn::fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
    if (d <= 0 || Sq < 0 || Skv < 0 || BH < 0)
        return attn::fail(ATTN_ERR_INVALID_ARG, "negative or zero size");
    attn::Tiles t{};
    const int st = attn::select(d, Sq, Skv, BH, dtype, causal == 1, &t);
    if (st != ATTN_OK) return st;
    if (block_m) *block_m = t.block_m;
    if (block_n) *block_n = t.block_n;
    if (waves) *waves = t.waves;
    if (lds_bytes) *lds_bytes = t.lds_bytes;
    return attn::ok();
}

const char* attn_last_error(void) { return attn::g_last_error.c_str(); }

int attn_version(void) { return 100; }

}  // extern "C"
