// C ABI of libattn.so: argument validation, the tile / occupancy selector
// and dispatch to the gfx950 kernels.  See include/attn.h for the contract.
#include "attn.h"
#include "attn_internal.h"
#include "attn_device.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

// Partial states of attn_fwd_split_noalloc's key chunks.  Each device keeps
// its own copy at its own address; host code uses that address, never this
// name, which on the host is only a stand-in for the symbol.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

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

// Merge of the key chunks' partial states.  Chunk c of a query row holds
// O_c = a_c / l_c and LSE_c = m_c + ln l_c (-inf when the chunk saw no key
// of the row).  The online normalisation's rescale rule applied to whole
// states gives, with M = max_c LSE_c and w_c = exp(LSE_c - M),
//     O = sum_c w_c O_c / sum_c w_c,   LSE = M + ln sum_c w_c,
// and O = 0, LSE = -inf when no chunk saw a key.  One thread per (row, four
// channels) runs over the chunks in batches of kMergeBatch, all of a batch's
// loads in flight together, keeping a running maximum M and rescaling its
// running sums by exp(M_old - M_new) when a batch raises it (the same rule
// once more).  Differences LSE_c - M are taken in fp64 (LSE reaches
// hundreds), their exponentials (<= 1) in fp32, the sums in fp64.
constexpr int kMergeBatch = 8;

__global__ void merge_kernel(const float* __restrict__ part_o,
                             const double* __restrict__ part_lse, void* __restrict__ o,
                             int o_kind, float* __restrict__ lse, size_t rows, int d,
                             int n_splits) {
    const int d4 = d / 4;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * d4) return;
    const size_t row = idx / d4;
    const int ch = 4 * (int)(idx - row * d4);
    double M = -INFINITY, W = 0.0;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int c0 = 0; c0 < n_splits; c0 += kMergeBatch) {
        double lc[kMergeBatch];
        f32x4 oc[kMergeBatch];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            const int c = c0 + u;
            lc[u] = -INFINITY;
            oc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (c < n_splits) {
                lc[u] = part_lse[c * rows + row];
                oc[u] = *reinterpret_cast<const f32x4*>(part_o + (c * rows + row) * d + ch);
            }
        }
        double mb = -INFINITY;
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) mb = fmax(mb, lc[u]);
        if (mb == -INFINITY) continue;          // no chunk of the batch saw a key of the row
        const double mn = fmax(M, mb);
        const double r = M == -INFINITY ? 0.0 : (double)expf((float)(M - mn));
        W *= r;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] *= r;
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            if (lc[u] == -INFINITY) continue;
            const double w = (double)expf((float)(lc[u] - mn));
            W += w;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += w * (double)oc[u][i];
        }
        M = mn;
    }
    const double inv = W > 0.0 ? 1.0 / W : 0.0;
    if (o_kind == 0) {
        const f32x4 v = {(float)(acc[0] * inv), (float)(acc[1] * inv), (float)(acc[2] * inv),
                         (float)(acc[3] * inv)};
        *reinterpret_cast<f32x4*>(static_cast<float*>(o) + row * d + ch) = v;
    } else if (o_kind == 1) {
        __bf16* out = static_cast<__bf16*>(o) + row * d + ch;
        for (int i = 0; i < 4; ++i) out[i] = (__bf16)(float)(acc[i] * inv);
    } else {
        _Float16* out = static_cast<_Float16*>(o) + row * d + ch;
        for (int i = 0; i < 4; ++i) out[i] = (_Float16)(float)(acc[i] * inv);
    }
    if (lse != nullptr && ch == 0) lse[row] = W > 0.0 ? (float)(M + log(W)) : -INFINITY;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

bool known_dtype(int dtype) { return dtype >= ATTN_F32 && dtype <= ATTN_F16_OUT_F32; }
int in_bytes(int dtype) { return dtype == ATTN_F32 ? 4 : 2; }
int out_bytes(int dtype) { return dtype == ATTN_BF16 || dtype == ATTN_F16 ? 2 : 4; }
// output element of the merge kernel: 0 fp32, 1 bf16, 2 fp16
int out_kind(int dtype) { return dtype == ATTN_BF16 ? 1 : (dtype == ATTN_F16 ? 2 : 0); }

// Compute units of an MI355X: the selectors aim to give each one work.
constexpr long kCUs = 256;

// The selector.  Query rows per workgroup shrink until the grid has at
// least one workgroup per compute unit or the smallest shape is reached;
// key rows per tile follow the key length.
int select(int d, int Sq, int Skv, int BH, int dtype, bool causal, Tiles* t) {
    auto wgs = [&](int bm) { return (long)BH * ((Sq + bm - 1) / bm); };
    if (dtype == ATTN_F32) {
        if (!(d == 16 || d == 32 || d == 64 || d == 128))
            return fail(ATTN_ERR_UNSUPPORTED, "fp32 head dim %d not built (16, 32, 64, 128)", d);
        int bn = Skv > 32 ? 64 : (Skv > 16 ? 32 : 16);
        int bm = 64;
        while (bm > 16 && (wgs(bm) < kCUs || Sq <= bm / 2)) bm /= 2;
        // Few 16-row query tiles over a long key range: 128-key tiles that
        // eight waves share, 16 keys each, twice the waves of 64-key tiles
        // (measured: 16.4 against 20.9 us for 8 queries x 1000 keys, B*H = 6;
        // 17.1 against 18.4 us for 512 x 512, B*H = 8, d = 64)
        if (bm == 16 && d <= 64 && Skv > 128 && wgs(16) < 512) bn = 128;
        t->block_m = bm;
        t->block_n = bn;
        t->waves = bm / 16 * f32_key_waves(d, bm, bn, wgs(bm));
        t->lds_bytes = f32_lds_bytes(d, bm, bn);
        return ATTN_OK;
    }
    if (!(d == 32 || d == 64 || d == 128))
        return fail(ATTN_ERR_UNSUPPORTED, "16-bit head dim %d not built (32, 64, 128)", d);
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
    // d = 32: a 32-key tile would hold only two score MFMAs per step, too few
    // to hide the softmax under; 64-key tiles (two score tiles of 32 registers
    // each still fit at two waves per SIMD when d is this small).  d = 64:
    // 64-key tiles in 128-row workgroups, which still fit two waves per SIMD
    // and halve the per-step overhead per score (measured 81.6 against
    // 84.0 us at S = 4096, H = 32, causal; 575 against 601 us at S = 16384,
    // H = 16); the 64-row kernel with 64-key tiles does not fit two waves
    // per SIMD, so it keeps 32-key tiles.
    // d = 32 in 128-row workgroups: 128-key tiles, for the same reason
    // (57.3 against 58.2 us at S = 4096, H = 32; 402 against 407 us at
    // S = 16384, H = 16).
    int bn = d == 32 ? (bm == 128 ? 128 : 64) : (d == 64 && bm == 128 ? 64 : 32);
    t->block_m = bm;
    t->block_n = bn;
    t->waves = bm / 32;
    t->lds_bytes = bf16_lds_bytes(d, bm, bn);
    return ATTN_OK;
}

// Workspace of attn_fwd_split: partial O [n, B*H, Sq, d] fp32, then (at a
// 256-byte boundary) partial LSE [n, B*H, Sq] fp64.
int64_t part_o_bytes(int64_t rows, int d, int n) { return (n * rows * d * 4 + 255) / 256 * 256; }
int64_t split_workspace(int64_t rows, int d, int n) { return part_o_bytes(rows, d, n) + n * rows * 8; }

// Key chunks for attn_fwd_split.  Without a split the grid has `items`
// workgroups; when that falls short of the target, the key range is cut into
// chunks of whole key tiles so that the chunks multiply it up to the target
// (at most 64 chunks).  Target: one 16-bit workgroup per CU (two or more
// waves each, two workgroups resident per CU); four fp32 waves per CU, one
// per SIMD (an fp32 wave owns 16 query rows, and the smaller fp32 grids are
// one wave per workgroup).  Measured on fp32 shapes of 128-1000 query rows:
// 2-3x faster than one workgroup per CU; the 16-bit choice was within 10 %
// of the best forced count on every decode and prefill shape tried, and
// twice as many chunks was slower there.  `want` = 0 asks for that choice;
// otherwise the caller's count, rounded to whole tiles.  Returns the chunk
// count and length.
void split_plan(const Tiles& t, int Sq, int Skv, int BH, int dtype, bool causal, int want,
                int* n_splits, int* kv_chunk) {
    const long n_qt = (Sq + t.block_m - 1) / t.block_m;
    const long items = (long)BH * (dtype == ATTN_F32 ? n_qt : (causal ? (n_qt + 1) / 2 : n_qt));
    const long have = dtype == ATTN_F32 ? items * t.waves : items;   // waves / workgroups
    const long target = dtype == ATTN_F32 ? 4 * kCUs : kCUs;
    const long key_tiles = (Skv + t.block_n - 1) / t.block_n;
    long n = want;
    if (n <= 0)
        n = have >= target ? 1 : std::min<long>(64, (target + have - 1) / std::max(have, 1L));
    // fp32 over fewer than four key tiles: the merge kernel costs more than
    // the shorter key walk saves (8 queries x 257 keys: 3 chunks 10.1 us,
    // one 8.4 us)
    if (want <= 0 && dtype == ATTN_F32 && key_tiles < 4) n = 1;
    n = std::max<long>(1, std::min<long>(n, key_tiles));
    long chunk = (Skv + n - 1) / n;
    chunk = (chunk + t.block_n - 1) / t.block_n * t.block_n;
    *kv_chunk = (int)std::max<long>(chunk, t.block_n);
    *n_splits = (int)((Skv + *kv_chunk - 1) / *kv_chunk);
    if (*n_splits < 1) *n_splits = 1;
}

int validate(const Problem& p) {
    if (!known_dtype(p.dtype)) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", p.dtype);
    if (p.B < 0 || p.H < 0 || p.Sq < 0 || p.Skv < 0)
        return fail(ATTN_ERR_INVALID_ARG, "negative size (B=%d H=%d Sq=%d Skv=%d)", p.B, p.H,
                    p.Sq, p.Skv);
    if (p.d <= 0) return fail(ATTN_ERR_INVALID_ARG, "head dim %d must be positive", p.d);
    if (p.dtype == ATTN_F32 ? !(p.d == 16 || p.d == 32 || p.d == 64 || p.d == 128)
                            : !(p.d == 32 || p.d == 64 || p.d == 128))
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

// Device address of `scratch` per device, found once per device with that
// device current.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_on_current_device(hipStream_t stream, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(ATTN_ERR_UNSUPPORTED, "device %d is beyond the %d devices the scratch covers",
                    dev, kMaxDevices);
    if (stream != nullptr) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess)
            return fail(ATTN_ERR_HIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
        if (sdev != dev)
            return fail(ATTN_ERR_INVALID_ARG, "stream belongs to device %d, device %d is current",
                        (int)sdev, dev);
    }
    void* ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch[dev].load(std::memory_order_relaxed);
        if (ptr == nullptr) {
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess || ptr == nullptr)
                return fail(ATTN_ERR_HIP, "no address for the static scratch on device %d: %s",
                            dev, hipGetErrorString(e));
            if ((reinterpret_cast<uintptr_t>(ptr) & 255u) != 0)
                return fail(ATTN_ERR_HIP, "static scratch on device %d is not 256-byte aligned",
                            dev);
            g_scratch[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return ATTN_OK;
}

// want_splits < 0: no split (attn_fwd); >= 0: attn_fwd_split with the
// caller's workspace, or with the static scratch when `static_scratch`.
int run(const Problem& p_in, int block_m, int block_n, int want_splits = -1,
        void* workspace = nullptr, int64_t workspace_bytes = 0, bool static_scratch = false) {
    Problem p = p_in;
    int st = validate(p);
    if (st != ATTN_OK) return st;
    const int bh = p.B * p.H;
    if (want_splits >= 0) {
        // the size is checked once the chunk count is known (below)
        if (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
            return fail(ATTN_ERR_MISALIGNED, "workspace must be 256-byte aligned");
        const size_t ib = (size_t)in_bytes(p.dtype);
        const size_t nq = (size_t)bh * p.Sq * p.d, nkv = (size_t)bh * p.Skv * p.d;
        const size_t wb = (size_t)std::max<int64_t>(workspace_bytes, 0);
        if (overlaps(workspace, wb, p.q, nq * ib) || overlaps(workspace, wb, p.k, nkv * ib) ||
            overlaps(workspace, wb, p.v, nkv * ib) ||
            overlaps(workspace, wb, p.o, nq * out_bytes(p.dtype)) ||
            overlaps(workspace, wb, p.lse, (size_t)bh * p.Sq * 4))
            return fail(ATTN_ERR_INVALID_ARG, "workspace overlaps an input or an output");
    }
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
        t.waves = p.dtype == ATTN_F32
                      ? block_m / 16 *
                            f32_key_waves(p.d, block_m, block_n,
                                          bh * (long)((p.Sq + block_m - 1) / block_m))
                      : block_m / 32;
    }
    hipError_t e;
    if (p.Skv == 0) {
        const size_t elems = (size_t)bh * p.Sq * p.d;
        const int blocks = (int)std::min<size_t>((elems + 255) / 256, 4096);
        hipLaunchKernelGGL(empty_rows_kernel, dim3(blocks), dim3(256), 0, p.stream, p.o,
                           out_bytes(p.dtype), p.lse, elems, (size_t)bh * p.Sq);
        e = hipGetLastError();
    } else {
        int n = 1, chunk = p.Skv;
        if (want_splits >= 0)
            split_plan(t, p.Sq, p.Skv, bh, p.dtype, p.causal, want_splits, &n, &chunk);
        if (n > 1) {
            const int64_t rows = (int64_t)bh * p.Sq;
            const int64_t need = split_workspace(rows, p.d, n);
            if (static_scratch) {
                if (need > ATTN_NOALLOC_SCRATCH_BYTES)
                    return fail(ATTN_ERR_INVALID_ARG,
                                "%d key chunks over %lld query rows need %lld bytes of scratch, "
                                "more than the static %lld",
                                n, (long long)rows, (long long)need,
                                (long long)ATTN_NOALLOC_SCRATCH_BYTES);
                st = scratch_on_current_device(p.stream, &workspace);
                if (st != ATTN_OK) return st;
                workspace_bytes = ATTN_NOALLOC_SCRATCH_BYTES;
            }
            if (workspace == nullptr || workspace_bytes < need)
                return fail(ATTN_ERR_INVALID_ARG, "workspace of %lld bytes too small (need %lld)",
                            (long long)workspace_bytes, (long long)need);
            p.n_splits = n;
            p.kv_chunk = chunk;
            p.part_o = static_cast<float*>(workspace);
            p.part_lse = reinterpret_cast<double*>(static_cast<char*>(workspace) +
                                                   part_o_bytes(rows, p.d, n));
        }
        e = p.dtype == ATTN_F32 ? launch_f32(p, t) : launch_bf16(p, t);
        if (e == hipSuccess && n > 1) e = launch_merge(p);
    }
    if (e != hipSuccess)
        return fail(ATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

hipError_t launch_merge(const Problem& p) {
    const size_t rows = (size_t)p.B * p.H * p.Sq;
    const size_t threads = rows * (p.d / 4);
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    hipLaunchKernelGGL(merge_kernel, dim3(blocks), dim3(256), 0, p.stream, p.part_o,
                       p.part_lse, p.o, out_kind(p.dtype), p.lse, rows, p.d, p.n_splits);
    return hipGetLastError();
}

}  // namespace attn

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int Sq, int Skv, int d, float scale, int causal, int dtype, void* stream) {
    return attn_fwd_tiles(q, k, v, o, lse, B, H, Sq, Skv, d, scale, causal, dtype, stream, 0, 0);
}

int attn_fwd_tiles(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int H, int Sq, int Skv, int d, float scale, int causal, int dtype,
                   void* stream, int block_m, int block_n) {
    if (causal < 0 || causal > 2)
        return attn::fail(ATTN_ERR_INVALID_ARG, "causal must be 0, 1 or 2 (got %d)", causal);
    if (block_m < 0 || block_n < 0 || ((block_m == 0) != (block_n == 0)))
        return attn::fail(ATTN_ERR_INVALID_ARG, "block_m, block_n must both be 0 or positive");
    attn::Problem p{q, k, v, o, lse, B, H, Sq, Skv, d, scale, causal != 0, dtype,
                    static_cast<hipStream_t>(stream)};
    p.causal_off = causal == 2 ? 0 : Skv - Sq;
    return attn::run(p, block_m, block_n);
}

int attn_select_tiles(int d, int Sq, int Skv, int BH, int dtype, int causal, int* block_m,
                      int* block_n, int* waves, int* lds_bytes) {
    if (!attn::known_dtype(dtype))
        return attn::fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (causal < 0 || causal > 2)
        return attn::fail(ATTN_ERR_INVALID_ARG, "causal must be 0, 1 or 2 (got %d)", causal);
    if (d <= 0 || Sq < 0 || Skv < 0 || BH < 0)
        return attn::fail(ATTN_ERR_INVALID_ARG, "negative or zero size");
    attn::Tiles t{};
    const int st = attn::select(d, Sq, Skv, BH, dtype, causal != 0, &t);
    if (st != ATTN_OK) return st;
    if (block_m) *block_m = t.block_m;
    if (block_n) *block_n = t.block_n;
    if (waves) *waves = t.waves;
    if (lds_bytes) *lds_bytes = t.lds_bytes;
    return attn::ok();
}

int attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int H, int Sq, int Skv, int d, float scale, int causal, int dtype,
                   void* stream, int n_splits, void* workspace, long long workspace_bytes) {
    if (causal < 0 || causal > 2)
        return attn::fail(ATTN_ERR_INVALID_ARG, "causal must be 0, 1 or 2 (got %d)", causal);
    if (n_splits < 0 || n_splits > 4096)
        return attn::fail(ATTN_ERR_INVALID_ARG, "n_splits must be in [0, 4096] (got %d)",
                          n_splits);
    attn::Problem p{q, k, v, o, lse, B, H, Sq, Skv, d, scale, causal != 0, dtype,
                    static_cast<hipStream_t>(stream)};
    p.causal_off = causal == 2 ? 0 : Skv - Sq;
    return attn::run(p, 0, 0, n_splits, workspace, workspace_bytes);
}

int attn_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Sq, int Skv, int d, float scale, int causal,
                           int dtype, void* stream, int n_splits) {
    if (causal < 0 || causal > 2)
        return attn::fail(ATTN_ERR_INVALID_ARG, "causal must be 0, 1 or 2 (got %d)", causal);
    if (n_splits < 0 || n_splits > 4096)
        return attn::fail(ATTN_ERR_INVALID_ARG, "n_splits must be in [0, 4096] (got %d)",
                          n_splits);
    attn::Problem p{q, k, v, o, lse, B, H, Sq, Skv, d, scale, causal != 0, dtype,
                    static_cast<hipStream_t>(stream)};
    p.causal_off = causal == 2 ? 0 : Skv - Sq;
    return attn::run(p, 0, 0, n_splits, nullptr, 0, true);
}

int attn_select_splits(int d, int Sq, int Skv, int BH, int dtype, int causal, int* n_splits,
                       int* kv_chunk) {
    int bm = 0, bn = 0, waves = 0, lds = 0;
    const int st = attn_select_tiles(d, Sq, Skv, BH, dtype, causal, &bm, &bn, &waves, &lds);
    if (st != ATTN_OK) return st;
    attn::Tiles t{bm, bn, waves, lds};
    int n = 1, chunk = Skv;
    if (Skv > 0) attn::split_plan(t, Sq, Skv, BH, dtype, causal != 0, 0, &n, &chunk);
    if (n_splits) *n_splits = n;
    if (kv_chunk) *kv_chunk = chunk;
    return attn::ok();
}

long long attn_split_workspace_bytes(int B, int H, int Sq, int d, int n_splits) {
    if (B < 0 || H < 0 || Sq < 0 || d <= 0 || n_splits < 1 || n_splits > 4096) {
        attn::fail(ATTN_ERR_INVALID_ARG, "invalid size for the split workspace");
        return -1;
    }
    attn::ok();
    return (long long)attn::split_workspace((int64_t)B * H * Sq, d, n_splits);
}

const char* attn_last_error(void) { return attn::g_last_error.c_str(); }

int attn_version(void) { return 102; }

}  // extern "C"
