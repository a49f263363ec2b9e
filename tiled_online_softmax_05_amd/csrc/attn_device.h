// Device-side helpers shared by the gfx950 attention kernels: vector types,
// MFMA wrappers and the workgroup -> (head, query tile) order.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Workgroup order.  Workgroups are numbered so that consecutive ids walk
// over the (batch, head) pairs of one query-tile rank.  With causal masking
// the rank runs from the last query tile (the most key tiles) to the first,
// so the hardware dispatcher, which hands out workgroups in id order, starts
// the longest ones first.  Because the dispatcher deals consecutive ids to
// the 8 XCDs in turn, every query tile of head bh lands on XCD (bh mod 8)
// whenever the number of heads is a multiple of 8, and that XCD's L2 keeps
// the head's K/V tiles for all of them.
__device__ __forceinline__ void tile_coords(int n_bh, int n_qt, bool causal, int& bh, int& qt) {
    const int idx = blockIdx.x;
    const int rank = idx / n_bh;
    bh = idx - rank * n_bh;
    qt = causal ? (n_qt - 1 - rank) : rank;
}

// Pairing of query tiles for causal attention: workgroup rank r runs the
// heavy tile n_qt-1-r and then the light tile r (second = -1 when the two
// coincide), so all workgroups carry equal work.  Non-causal workgroups run
// one tile each.  Consecutive ids walk the (batch, head) pairs as in
// tile_coords, with the same XCD placement.
__host__ __device__ __forceinline__ int tile_pair_count(int n_qt, bool causal) {
    return causal ? (n_qt + 1) / 2 : n_qt;
}
__device__ __forceinline__ void tile_pair_coords(int n_bh, int n_qt, bool causal, int& bh,
                                                 int& first, int& second) {
    const int idx = blockIdx.x;
    const int rank = idx / n_bh;
    bh = idx - rank * n_bh;
    if (causal) {
        first = n_qt - 1 - rank;
        second = rank < first ? rank : -1;
    } else {
        first = rank;
        second = -1;
    }
}

// Key range [0, kv_end) a workgroup of query rows [q_first, q_last] visits:
// causal rows see keys j <= i + off (off = Skv - Sq when the mask is aligned
// to the end of the key sequence, 0 when aligned to its start).
__device__ __forceinline__ int kv_limit(int q_last, int off, int Skv, bool causal) {
    if (!causal) return Skv;
    int e = q_last + off + 1;
    return e < 0 ? 0 : (e > Skv ? Skv : e);
}

}  // namespace attn
