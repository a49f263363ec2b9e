// Internal declarations shared by the kernel translation units and the C ABI
// (host side).  Not installed; the public surface is include/attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace attn {

// One launch's problem description, already validated by the C ABI.
struct Problem {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;          // may be null
    int B, H, Sq, Skv, d;
    float scale;
    bool causal;
    int dtype;           // attn_dtype
    hipStream_t stream;
    // Split of the key range (attn_fwd_split): key chunk c = blockIdx.y
    // covers keys [c * kv_chunk, (c + 1) * kv_chunk).  With part_o set, the
    // kernels write each chunk's partial state -- O_c = a_c / l_c (fp32) and
    // LSE_c (fp64) -- to [n_splits, B*H, Sq, d] and [n_splits, B*H, Sq]
    // instead of o and lse, and launch_merge() combines them.
    // Causal diagonal: query row i sees keys j <= i + causal_off (Skv - Sq for
    // end-aligned masking, 0 for start-aligned).
    int causal_off = 0;
    int n_splits = 1;
    int kv_chunk = 0x7FFFFFFF;
    float* part_o = nullptr;
    double* part_lse = nullptr;
};

// Tile shape chosen by the selector or forced by the caller.
struct Tiles {
    int block_m;   // query rows per workgroup
    int block_n;   // key rows per K/V tile
    int waves;     // 64-wide waves per workgroup
    int lds_bytes; // LDS per workgroup
};

// Kernel families.  Each returns hipSuccess or the launch error, and
// hipErrorInvalidValue when no kernel was built for (d, tiles).
hipError_t launch_f32(const Problem& p, const Tiles& t);
hipError_t launch_bf16(const Problem& p, const Tiles& t);
// Fill O with zeros and LSE with -inf (Skv == 0: no row sees a key).
hipError_t launch_empty_rows(const Problem& p);
// Combine the n_splits partial states in part_o / part_lse into o and lse.
hipError_t launch_merge(const Problem& p);

// Tile shapes that have a kernel, and their LDS footprint.
bool f32_tiles_supported(int d, int block_m, int block_n);
bool bf16_tiles_supported(int d, int block_m, int block_n);
int f32_lds_bytes(int d, int block_m, int block_n);
// fp32 waves per 16-row query block (key groups of one workgroup), 1 unless
// block_m = 16: with 128-key tiles 8 (4 at d = 128); otherwise 4, 2 or 1 as
// the query-tile grid has fewer than 512, fewer than 1024 or more tiles, at
// most block_n / 16
int f32_key_waves(int d, int block_m, int block_n, long query_tiles);
int bf16_lds_bytes(int d, int block_m, int block_n);

}  // namespace attn
