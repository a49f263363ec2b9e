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

// Workgroup order.  The hardware dispatcher hands workgroups out in id order
// and deals consecutive ids to the 8 XCDs in turn (id mod 8), each XCD with
// its own L2.  Ids are therefore enumerated XCD-major: with n workgroups and
// n % 8 == 0, XCD x receives the linear slots x * n/8 ... (x + 1) * n/8 - 1 in
// order, and linear slot L means (head L / per_head, rank L % per_head).  Each
// XCD thus works through whole heads one after the other, all resident
// workgroups of a head sweeping the same K/V tiles, so the L2 holds the
// window those workgroups share; heavy ranks (the most key tiles) come first
// within a head.  Grids that are not a multiple of 8 keep the plain order.
__device__ __forceinline__ int xcd_major_slot(int n) {
    const int idx = blockIdx.x;
    if ((n & 7) != 0) return idx;
    return (idx & 7) * (n >> 3) + (idx >> 3);
}

// Workgroup -> (head, query tile), one tile per workgroup; causal ranks run
// from the last query tile (the most key tiles) to the first.
__device__ __forceinline__ void tile_coords(int n_bh, int n_qt, bool causal, int& bh, int& qt) {
    const int L = xcd_major_slot(n_bh * n_qt);
    bh = L / n_qt;
    const int rank = L - bh * n_qt;
    qt = causal ? (n_qt - 1 - rank) : rank;
}

// Pairing of query tiles for causal attention: workgroup rank r runs the
// heavy tile n_qt-1-r and then the light tile r (second = -1 when the two
// coincide), so all workgroups carry equal work.  Non-causal workgroups run
// one tile each.  Same XCD-major order as tile_coords.
__host__ __device__ __forceinline__ int tile_pair_count(int n_qt, bool causal) {
    return causal ? (n_qt + 1) / 2 : n_qt;
}
__device__ __forceinline__ void tile_pair_coords(int n_bh, int n_qt, bool causal, int& bh,
                                                 int& first, int& second) {
    const int per_head = tile_pair_count(n_qt, causal);
    const int L = xcd_major_slot(n_bh * per_head);
    bh = L / per_head;
    const int rank = L - bh * per_head;
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
