// 16-bit attention forward for gfx950: bf16 or fp16 inputs on the matching
// MFMA, fp32 accumulation (one template, instantiated for both types).
//
// The online softmax of "Tiled attention: preserving results without a full
// score matrix" (section "Online normalization") over query tiles and key
// tiles as in the tiled lab function of "Verify tiled attention".  Each
// 64-wide wave owns 32 query rows; the waves of a workgroup share one K/V
// tile staged in LDS.  K/V tiles travel HBM -> LDS by DMA well ahead of their
// use, so the loads overlap with the MFMA work.
//
// Contractions use v_mfma_f32_32x32x16_bf16 / _f16 (A 32x16, B 16x32, D 32x32):
//   lane = 32 h + c (h in 0..1, c in 0..31);
//   A: lane holds A[c][8h .. 8h+7];  B: lane holds B[8h .. 8h+7][c];
//   D: lane holds D[8 (r/4) + 4 h + (r%4)][c] for r = 0..15.
//
// Scores are computed transposed, S^T = K Q^T, so that a lane's 16 results
// all belong to one query row (c): the row maximum and sum are in-lane
// reductions plus one exchange with lane c + 32.  The K rows of each 32-key
// block are stored in LDS in the order sigma^-1, chosen so that D row
// 8a + 4h + b carries key 16 (a/2) + 8 h + 4 (a%2) + b: a lane then holds 8
// consecutive keys per 16-key step, which is exactly the B operand layout
// of the next contraction O^T = V^T P^T.
//
// Exponentials are base 2 with scale * log2(e) folded into one FMA; the
// running maximum m is kept in that scaled base-2 domain.  Every key tile
// takes its row maxima and updates m as the online normalisation
// prescribes, lazily: m moves, and l and the accumulator are rescaled by
// 2^(m_old - m_new), only when a tile's maximum exceeds m by more than
// kSlack.  The test runs on raw scores against thr = (m + kSlack) /
// (scale log2 e), on each lane's half of its row (a row passes exactly when
// one half does), so the common tile costs one compare per lane; the
// exchange with lane c + 32 and the rescale run in a wave-uniform branch
// only on tiles where some row passes.  Probabilities therefore stay at
// 2^kSlack or below (up to the rounding of thr), and most tiles skip the
// rescale.
#include "attn.h"
#include "attn_internal.h"
#include "attn_device.h"

#include <cmath>
#include <type_traits>

namespace attn {
namespace {

constexpr float kLog2ef = 1.44269504088896341f;
// Slack of the running maximum, in base-2 exponent units: m moves (and l
// and a are rescaled by 2^(m_old - m_new)) only when a tile's maximum
// exceeds it by more than this, so every probability stays at about
// 2^kSlack = 256 or below (well inside fp16's range as well as bf16's) and
// most tiles skip the accumulator rescale.
constexpr float kSlack = 8.f;
constexpr float kLn2f = 0.693147180559945309f;

// Key held by LDS row r (0..31) of a 32-key block: D row 8a + 4h + b of the
// score contraction must carry key 16 (a/2) + 8 h + 4 (a%2) + b.
__device__ __forceinline__ int sigma(int r) {
    const int a = r >> 3, h = (r >> 2) & 1, b = r & 3;
    return 16 * (a >> 1) + 8 * h + 4 * (a & 1) + b;
}

// s_waitcnt immediates: vmcnt = n (6 bits on gfx9: [3:0] and [15:14]),
// expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int wait_vmcnt(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Descriptor word 3 for raw (unswizzled) buffer access on gfx9-family parts.
constexpr int kBufferFlags = 0x00020000;

// A buffer resource over [base, base + bytes): loads past the end return 0,
// which is how the tails of Q, K and V read as zero rows without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kBufferFlags);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// The same descriptor as four words, for the DMA below.
__device__ __forceinline__ i32x4 buffer_words(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4{(int32_t)(uint32_t)a, (int32_t)((a >> 32) & 0xFFFF), (int32_t)bytes,
                 kBufferFlags};
}

// HBM -> LDS DMA of 16 bytes per lane (buffer_load ... lds): lane l's bytes
// land at LDS byte address lds + 16 l, offsets past the descriptor's range
// read 0.  Written as inline asm so that the compiler does not track it as
// an LDS write: the kernel orders every DMA against the LDS reads itself
// (explicit vmcnt waits and barriers around the ring of buffers), while the
// compiler's tracking cannot tell the ring's buffers apart across steps and
// would wait for prefetches that no read depends on.  Hidden from the
// compiler's counters, these loads can only make its own vmcnt waits for
// ordinary loads stricter.  M0 must be written one instruction before the
// DMA that reads it.
// M0 is a reserved register: clang warns that clobbering it is not
// preserved across the statement, which is what is meant here (the compiler
// sets M0 itself before each of its own uses).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds, uint32_t voffset) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voffset), "s"(rsrc)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}


// Empty register-level barrier: makes x an output of a volatile statement at
// this point, so IR passes cannot sink the code producing x past it (the
// sched_barrier fences only order machine instructions).
template <typename T>
__device__ __forceinline__ void pin(T& x) {
    asm volatile("" : "+v"(x));
}

// Workgroup barrier for the LDS ring.  __syncthreads() also fences memory
// at workgroup scope, and the compiler implements that release by waiting
// for every load in flight -- including the DMA just issued for tiles two
// steps ahead, which would cut the prefetch depth to one step.  Here the
// caller first waits (s_waitcnt) for exactly the DMA the next step reads;
// LDS operand reads have been consumed by then; the memory clobber keeps the
// compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void ring_barrier() {
    asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ float other_half_max(float x) {
    // v_permlane32_swap: lane l (< 32) receives lane l + 32 and vice versa.
    // The maximum as one plain v_max_f32: fmaxf would first quiet both
    // values (two more instructions), which scores that are finite or -inf
    // never need.
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    float m;
    asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
    return m;
}

__device__ __forceinline__ float other_half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The score and P.V contraction for either 16-bit input type (A 32x16, B
// 16x32, fp32 D 32x32; the same lane layout for both).
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c, int, int, int) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_32x32x16(f16x8 a, f16x8 b, f32x16 c, int, int, int) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Software-pipelined main loop (skewed).  Step j holds the raw scores S_j in
// registers and K_{j+1}, V_{j-1} in LDS.  The matrix cores compute
// S_{j+1} = K_{j+1} Q^T and add P_{j-1} V_{j-1} to the accumulator, the two
// kinds of MFMA alternating, while the VALU runs the online-softmax update
// of S_j between them (row max, reference and rescale factor, exponentials,
// row sums, packing into P_j).  K and V live in four LDS buffers each (K_t
// in sK[t % 4], V_t in sV[t % 4]); step j starts the DMA of K_{j+4} and
// V_{j+2} into the buffers its predecessor finished reading and ends with one
// workgroup barrier after waiting for the DMA issued one step earlier, so
// the tiles step j + 1 reads (K_{j+2}, V_j) are already visible during step
// j.  The instruction order is fixed by hand (sched_barrier fences): every
// MFMA operand is read from LDS two MFMAs ahead of its use, across step
// boundaries too (the last MFMAs of step j read the first operands of step
// j + 1 before the barrier), and the VALU work is cut into slices placed
// between consecutive MFMAs.
template <typename T, int D, int BN, int WAVES, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_bf16_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                          const T* __restrict__ V, void* __restrict__ Out,
                          float* __restrict__ LSE, int n_bh, int Sq, int Skv, float sl2,
                          int n_qt, int off, int kv_chunk, float* __restrict__ part_o,
                          double* __restrict__ part_lse) {
    typedef T V8 __attribute__((ext_vector_type(8)));   // MFMA operand: 8 elements
    typedef T V4 __attribute__((ext_vector_type(4)));
    constexpr int BM = 32 * WAVES;
    constexpr int NT = 64 * WAVES;
    constexpr int KS = D / 16;         // k-steps of the score contraction
    constexpr int NKB = BN / 32;       // 32-key blocks per tile
    constexpr int ND = D / 32;         // 32-channel output blocks
    constexpr int DCH = D / 8;         // 16-byte chunks per K/V row
    constexpr int ROWB = D * 2;        // bytes per K/V row
    constexpr int CHUNKS = BN * DCH;   // 16-byte chunks per K or V tile
    constexpr int PER = CHUNKS / NT;   // chunks each thread moves per tile
    constexpr int NA = NKB * KS;       // score MFMAs per step
    constexpr int NB = 2 * NKB * ND;   // P.V MFMAs per step
    constexpr int NV = 16 * NKB;       // scores per lane per tile
    static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
    static_assert(CHUNKS % NT == 0, "every lane moves the same number of chunks");
    static_assert(DCH == 4 || DCH == 8 || DCH == 16, "K swizzle covers 4, 8 or 16 chunks per row");
    static_assert(NA >= 4 && NB >= ND + 1, "schedule needs a few MFMAs per phase");

    // Four buffers each for K and V: K_t lives in sK[t % 4], V_t in
    // sV[t % 4].  Separate arrays (not one indexed at run time) let the
    // compiler see that the DMA into one buffer never aliases reads of
    // another.
    __shared__ __attribute__((aligned(16))) T sK0[BN * D];
    __shared__ __attribute__((aligned(16))) T sK1[BN * D];
    __shared__ __attribute__((aligned(16))) T sK2[BN * D];
    __shared__ __attribute__((aligned(16))) T sK3[BN * D];
    __shared__ __attribute__((aligned(16))) T sV0[BN * D];
    __shared__ __attribute__((aligned(16))) T sV1[BN * D];
    __shared__ __attribute__((aligned(16))) T sV2[BN * D];
    __shared__ __attribute__((aligned(16))) T sV3[BN * D];
    // vmcnt value that leaves exactly one step's DMA (K and V) in flight
    constexpr int kWaitOlderDma = wait_vmcnt(2 * PER);
    static_assert(5 * PER < 64, "DMA counts must fit the 6-bit vmcnt field");

    // K layout in LDS: unpadded rows of DCH 16-byte chunks; chunk q of row r
    // sits at position q ^ k_swz(r).  An operand read (16 lanes = 16
    // consecutive rows, one chunk) then touches 16 distinct 16-byte bank
    // groups of the 64-bank LDS (with 4 chunks per row, rows r and r + 4
    // share banks before the swizzle, and (r / 4) % 4 separates them).
    auto k_swz = [](int r) {
        return DCH == 16 ? (r & 15) : (DCH == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3));
    };
    // V layout in LDS: row = key, chunk q of row key at q ^ v_swz(key).  The
    // transposing operand read of 32 lanes covers 4 keys x 4 chunks; the
    // swizzle puts those 16 chunks in 16 distinct bank groups (64-byte rows,
    // d = 32, already do: 4 consecutive keys fill the 256 bytes of the banks).
    auto v_swz = [](int key) {
        return DCH == 16 ? 4 * (key & 3) : (DCH == 8 ? 4 * ((key >> 1) & 1) : 0);
    };

    // Workgroup -> (head, query tiles).  Causal: one workgroup runs query
    // tile n_qt-1-r and then tile r, so every workgroup visits the same
    // number of key tiles and the grid finishes in one round.
    int bh, qt_first, qt_second;
    tile_pair_coords(n_bh, n_qt, CAUSAL, bh, qt_first, qt_second);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;
    const int c = lane & 31;
    // raw-score units per scaled base-2 unit, for the running-maximum test
    const float inv_sl2 = 1.f / sl2;

    const T* Qh = Q + (size_t)bh * Sq * D;
    const T* Kh = K + (size_t)bh * Skv * D;
    const T* Vh = V + (size_t)bh * Skv * D;

    // ---- K/V staging: HBM -> LDS by DMA ----
    // Slot S = i * NT + tid (16 bytes) of LDS row S / DCH holds chunk
    // (S % DCH) ^ swizzle(row) of that row's key.  Each tile gets a
    // descriptor over rows [kv0, Skv) of the head (empty from Skv on), so
    // rows at or past Skv fall outside its range and read 0; the tile offset
    // moves the base on the scalar unit and each lane's offset within a tile
    // is fixed for the whole kernel.
    auto tile_words = [&](const T* head, int kv0) {
        const int k0 = min(kv0, Skv);
        return buffer_words(head + (size_t)k0 * D, (uint32_t)(Skv - k0) * ROWB);
    };
    auto load_k = [&](int kv0, T* dst) {
        const i32x4 r = tile_words(Kh, kv0);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int S = i * NT + tid;
            const int row = S / DCH;
            const int chunk = (S % DCH) ^ k_swz(row);
            const int key = (row & ~31) + sigma(row & 31);
            dma16(r, lds_addr(dst + (i * NT + wave * 64) * 8), (uint32_t)key * ROWB + 16 * chunk);
        }
    };
    auto load_v = [&](int kv0, T* dst) {
        const i32x4 r = tile_words(Vh, kv0);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int S = i * NT + tid;
            const int key = S / DCH;
            const int chunk = (S % DCH) ^ v_swz(key);
            dma16(r, lds_addr(dst + (i * NT + wave * 64) * 8), (uint32_t)key * ROWB + 16 * chunk);
        }
    };

    // Byte offset of this lane's K operand (row c, chunk 2 ks + h) within a K
    // buffer, per k-step of the score contraction.
    int koff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        koff[ks] = c * ROWB + 16 * ((2 * ks + h) ^ k_swz(c));
        pin(koff[ks]);
    }

    // ---- one query tile: Q operand, online softmax over its key tiles, O/LSE ----
    auto run_tile = [&](int qt) __attribute__((always_inline)) {
    const int q0w = qt * BM + wave * 32;
    const int qi = q0w + c;

    // Q^T operand: lane holds q[qi][16 ks + 8 h .. +7]; rows past Sq read 0
    V8 qop[KS];
    {
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(Qh, (uint32_t)Sq * ROWB);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 x = buffer_load16(rq, (uint32_t)qi * ROWB + 32 * ks + 16 * h);
            qop[ks] = __builtin_bit_cast(V8, x);
        }
        // Retire the Q loads here, on every path: vmcnt is in-order, and Q
        // loads still in flight at the loop entry would make every tile wait
        // for its own K/V loads before the first MFMA.  (The empty asm uses
        // the registers, so the loads cannot sink below this point.)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) pin(qop[ks]);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }

    float m = -INFINITY;     // running maximum, scale*log2(e) units
    float m_ref = 0.f;       // m, or 0 while the row has seen no key
    float thr = -INFINITY;   // (m + kSlack) / (scale log2 e): a raw tile maximum
                             // above it moves m
    float l = 0.f;           // this lane's part of the normaliser
    f32x16 acc[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) acc[i] = f32x16{};

    // key chunk blockIdx.y of the (possibly split) key range
    const int q_last = min(Sq, (qt + 1) * BM) - 1;
    const int kv_begin = (int)blockIdx.y * kv_chunk;
    const int kv_end = min(kv_limit(q_last, off, Skv, CAUSAL), kv_begin + min(kv_chunk, Skv));
    const int n_tiles = kv_end > kv_begin ? (kv_end - kv_begin + BN - 1) / BN : 0;
    // last key this lane's query may see (for the masked tiles)
    const int lim = CAUSAL ? min(Skv - 1, qi + off) : Skv - 1;

    // ---- operand reads ----
    // K operand of score MFMA t: key block kb = t % NKB, k-step ks = t / NKB
    // (the accumulators of the key blocks alternate)
    // (the swizzle of row kb * 32 + c equals that of row c, so key block kb
    // only adds a constant; kept opaque, the lane's byte offset per k-step
    // is one register and the buffer and key block fold into the read's
    // immediate offset)
    auto k_operand = [&](const T* sk, int t) -> V8 {
        const int kb = t % NKB, ks = t / NKB;
        return *reinterpret_cast<const V8*>(reinterpret_cast<const char*>(sk) +
                                            kb * 32 * ROWB + koff[ks]);
    };
    // V operand of P.V MFMA t: k-step s = t / ND (keys 16 s .. 16 s + 15),
    // channel block i = t % ND; two transposing reads, keys 8 h + 4 u .. + 3
    const int g16 = lane & 15;
    const int cblk = lane & 16;
    auto v_operand = [&](const T* sv, int t) -> V8 {
        const int s = t / ND, i = t % ND;
        V4 part[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int key = 16 * s + 8 * h + 4 * u + (g16 >> 2);
            const int d = 32 * i + cblk + 4 * (g16 & 3);
            const T* src = sv + key * D + 8 * ((d >> 3) ^ v_swz(key)) + (d & 7);
            part[u] = __builtin_bit_cast(
                V4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4*)(src)));
        }
        return __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
    };

    auto mask = [&](int kv0, f32x16* st) {
        // only tiles crossing the key end or the causal diagonal
        const bool need = (kv0 + BN > Skv) || (CAUSAL && kv0 + BN - 1 > q0w + off);
        if (need) {
            const int base = lim - kv0 - 8 * h;     // visible iff key offset <= base
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int jo = kb * 32 + 16 * (r >> 3) + (r & 7);
                    if (jo > base) st[kb][r] = -INFINITY;
                }
        }
    };

    // One step of the skewed pipeline.  While the VALU turns the scores st
    // of tile j into probabilities pn and moves m and l, the matrix cores
    // compute the scores sn of tile j + 1 from K in sk (when QK) and add
    // P_{j-1} V_{j-1} (probabilities po, V in sv) to the accumulator (when
    // PV).  Score and P.V MFMAs alternate, so each has softmax work to hide
    // under it.  The row-maximum test of tile j comes first (slots 0 and 1); the
    // accumulator moves to a new m only after the P.V MFMAs, and only when
    // some row of the wave raised it.  The first two K and V operands arrive
    // in kp / vp, read during the previous step; with PF the step reads
    // those of the next step from sk_pre / sv_pre in their place.
    auto fused = [&](auto QK, auto PV, auto PF, const T* __restrict__ sk,
                     const T* __restrict__ sv, const f32x16* st, f32x16* sn,
                     const V8 (*po)[2], V8 (*pn)[2], V8* kp, V8* vp,
                     const T* __restrict__ sk_pre,
                     const T* __restrict__ sv_pre) __attribute__((always_inline)) {
        constexpr bool qk = decltype(QK)::value;
        constexpr bool pv = decltype(PV)::value;
        constexpr bool pf = decltype(PF)::value;
        constexpr int NM = (qk ? NA : 0) + (pv ? NB : 0);   // MFMAs of the step
        constexpr int NS = NM > 4 ? NM : 4;                  // schedule slots
        constexpr int S0 = 2;                                // first slot with exponentials
        V8 ka[3], va[3];
        if constexpr (qk) {
            ka[0] = kp[0];
            ka[1] = kp[1];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) sn[kb] = f32x16{};
        }
        if constexpr (pv) {
            va[0] = vp[0];
            va[1] = vp[1];
        }
        // (psum starts at -0, which an added value replaces exactly, so no
        // add of the start value is issued; alpha is set and read only when
        // the step rescales)
        float mx = -INFINITY, alpha, psum = -0.f;
        bool rescale = false;
        // While it interleaves MFMAs and softmax, the wave outranks a wave of
        // the other workgroup on the same SIMD that is issuing DMA, waiting at
        // its barrier or finishing a step (measured: 2 % faster than equal
        // priorities; per-MFMA raises were slower).
        __builtin_amdgcn_s_setprio(2);
        float ex[NV];
        // row sum of values [p0, p1), packed to 16 bits in groups of 8
        auto sum_pack = [&](int p0, int p1) {
#pragma unroll
            for (int e = p0; e < p1; ++e) {
                psum += ex[e];
                if ((e & 7) == 7) {
                    const int b = e - 7;
                    V8& pk = pn[e / 16][(e / 8) & 1];
                    pk = __builtin_convertvector(
                        (f32x8){ex[b], ex[b + 1], ex[b + 2], ex[b + 3], ex[b + 4], ex[b + 5],
                                ex[b + 6], ex[b + 7]},
                        V8);
                    pin(pk);
                }
            }
            pin(psum);
        };
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            // MFMA of slot s: alternate score / P.V when both run
            const bool is_qk = qk && (!pv || (s & 1) == 0);
            const int t = (qk && pv) ? s / 2 : s;
            if (s >= NM) {
                // no MFMA in this slot
            } else if (is_qk) {
                if (t + 2 < NA) ka[(t + 2) % 3] = k_operand(sk, t + 2);
                else if (pf) kp[t + 2 - NA] = k_operand(sk_pre, t + 2 - NA);
                const int kb = t % NKB, ks = t / NKB;
                sn[kb] = mfma_32x32x16(ka[t % 3], qop[ks], sn[kb], 0, 0, 0);
            } else {
                if (t + 2 < NB) va[(t + 2) % 3] = v_operand(sv, t + 2);
                else if (pf) vp[t + 2 - NB] = v_operand(sv_pre, t + 2 - NB);
                const int u = t / ND, i = t % ND;
                acc[i] = mfma_32x32x16(va[t % 3], po[u / 2][u % 2],
                                                                 acc[i], 0, 0, 0);
            }
            if (s == 0) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kb][r]);
            }
            if (s == 1) {
                // mx covers this lane's half of the row's values: a row's
                // maximum passes its threshold exactly when one half does
                rescale = __any(mx > thr);
                // (rare: the maximum moves on few tiles; a wave-uniform branch)
                if (rescale) {
                    mx = other_half_max(mx);            // the row's maximum
                    const bool grow = mx > thr;         // true on the row's first visible tile
                    const float mt = mx * sl2;          // tile max, scaled base-2 domain
                    // 2^(m - mt): 0 when m = -inf; no rescale (1) while m stays put
                    alpha = grow ? __builtin_amdgcn_exp2f(m - mt) : 1.f;
                    m = grow ? mt : m;
                    m_ref = (m == -INFINITY) ? 0.f : m;     // 0 while the row has seen no key
                    thr = (m + kSlack) * inv_sl2;
                    pin(thr);
                    // (volatile: keeps the compiler from turning the branch
                    // into selects that compute all of this on every tile)
                    pin(alpha);
                    pin(m_ref);
                }
            }
            if (s >= S0) {
                // exponentials of values [e0, e1) of this slot; the row sum
                // and the 16-bit packing of the previous slot's values, so
                // that no add reads an exponential issued just before it
                const int e0 = (s - S0) * NV / (NS - S0), e1 = (s - S0 + 1) * NV / (NS - S0);
#pragma unroll
                for (int e = e0; e < e1; ++e) {
                    ex[e] = __builtin_amdgcn_exp2f(fmaf(st[e / 16][e % 16], sl2, -m_ref));
                    pin(ex[e]);
                }
                if (s > S0) sum_pack((s - S0 - 1) * NV / (NS - S0), e0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        if constexpr (pf && !pv) {
            // (the first step has no P.V to carry the V prefetch)
            vp[0] = v_operand(sv_pre, 0);
            vp[1] = v_operand(sv_pre, 1);
        }
        sum_pack((NS - S0 - 1) * NV / (NS - S0), NV);     // the last slot's values
        // acc holds sum_{t <= j-1} relative to the old maximum; move it to
        // the new one before P_j V_j is added in the next step
        if (rescale) {
            l *= alpha;
#pragma unroll
            for (int i = 0; i < ND; ++i) acc[i] *= alpha;
        }
        l += psum;
    };

    using std::integral_constant;
    using T_ = integral_constant<bool, true>;
    using F_ = integral_constant<bool, false>;
    // P.V of the last tile: acc += P V from sv.
    auto pv_tile = [&](const T* sv, const V8 (*p)[2]) {
        V8 va[3];
        va[0] = v_operand(sv, 0);
        va[1] = v_operand(sv, 1);
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            if (t + 2 < NB) va[(t + 2) % 3] = v_operand(sv, t + 2);
            const int u = t / ND, i = t % ND;
            acc[i] = mfma_32x32x16(va[t % 3], p[u / 2][u % 2], acc[i],
                                                             0, 0, 0);
        }
    };

    using std::integral_constant;
    using T_ = integral_constant<bool, true>;
    using F_ = integral_constant<bool, false>;
    // Steady-state step j: scores of tile j + 1, P.V of tile j - 1, softmax
    // of tile j; DMA of K_{j+4} and V_{j+2}; first operands of step j + 1
    // from K_{j+2} and V_j.  The buffers arrive as distinct restrict
    // pointers: once inlined, every LDS access and DMA in the step carries
    // scoped no-alias metadata, which lets the compiler see that the DMA into
    // the free buffers never overlaps the operand reads of the busy ones (the
    // transposing read otherwise waits for all DMA in flight).
    auto step = [&](auto PV, int j, f32x16* st, V8 (*po)[2], V8* kp, V8* vp,
                    const T* __restrict__ k_next, const T* __restrict__ k_pre,
                    T* __restrict__ k_free, const T* __restrict__ v_prev,
                    const T* __restrict__ v_pre, T* __restrict__ v_free) {
        const int kv0 = kv_begin + j * BN;
        load_k(kv0 + 4 * BN, k_free);           // K_{j+4}: zero rows or unused past the end
        load_v(kv0 + 2 * BN, v_free);           // V_{j+2}
        mask(kv0, st);
        f32x16 sn[NKB];
        V8 pn[NKB][2];
        fused(T_{}, PV, T_{}, k_next, v_prev, st, sn, po, pn, kp, vp, k_pre, v_pre);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            st[kb] = sn[kb];
            po[kb][0] = pn[kb][0];
            po[kb][1] = pn[kb][1];
        }
        __builtin_amdgcn_s_waitcnt(kWaitOlderDma);   // K_{j+3}, V_{j+1} have landed
        ring_barrier();
    };

    if (n_tiles > 0) {
        // ---- prologue: K_0 .. K_3, V_0, V_1 in flight; S_0 from K_0 ----
        load_k(kv_begin, sK0);
        load_k(kv_begin + BN, sK1);
        load_k(kv_begin + 2 * BN, sK2);
        load_v(kv_begin, sV0);
        load_k(kv_begin + 3 * BN, sK3);
        load_v(kv_begin + BN, sV1);
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(5 * PER));   // K_0 has landed
        ring_barrier();
        f32x16 st[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            st[kb] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                st[kb] = mfma_32x32x16(k_operand(sK0, ks * NKB + kb),
                                                                 qop[ks], st[kb], 0, 0, 0);
        }
        // K_1, K_2 and V_0 have landed: step 0 reads K_1 and, for step 1,
        // K_2 and V_0
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * PER));
        ring_barrier();

        // ---- steps 0 .. n_tiles - 2 (each has a next tile) ----
        // buffers of step j: K_{j+1}, K_{j+2}, free slot of K_j, V_{j-1},
        // V_j, free slot of V_{j-2}
        V8 po[NKB][2];      // probabilities of the previous tile
        V8 kp[2], vp[2];    // first two K and V operands of the next step
        kp[0] = k_operand(sK1, 0);
        kp[1] = k_operand(sK1, 1);
        int j = 0;
        if (n_tiles > 1) {
            // no P.V yet
            step(F_{}, 0, st, po, kp, vp, sK1, sK2, sK0, sV3, sV0, sV2);
            j = 1;
            for (; j + 4 < n_tiles; j += 4) {
                step(T_{}, j, st, po, kp, vp, sK2, sK3, sK1, sV0, sV1, sV3);
                step(T_{}, j + 1, st, po, kp, vp, sK3, sK0, sK2, sV1, sV2, sV0);
                step(T_{}, j + 2, st, po, kp, vp, sK0, sK1, sK3, sV2, sV3, sV1);
                step(T_{}, j + 3, st, po, kp, vp, sK1, sK2, sK0, sV3, sV0, sV2);
            }
            if (j + 1 < n_tiles) {               // j % 4 == 1 here
                step(T_{}, j, st, po, kp, vp, sK2, sK3, sK1, sV0, sV1, sV3);
                ++j;
            }
            if (j + 1 < n_tiles) {
                step(T_{}, j, st, po, kp, vp, sK3, sK0, sK2, sV1, sV2, sV0);
                ++j;
            }
            if (j + 1 < n_tiles) {
                step(T_{}, j, st, po, kp, vp, sK0, sK1, sK3, sV2, sV3, sV1);
                ++j;
            }
        }
        // ---- last tile j = n_tiles - 1: P.V of tile j - 1 (its first
        // operands in vp), softmax of tile j, then its P.V.  All DMA has
        // landed first (also what the next query tile needs).
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        const int r = j % 4;
        const T* v_last = r == 0 ? sV0 : (r == 1 ? sV1 : (r == 2 ? sV2 : sV3));
        const T* v_prev = r == 0 ? sV3 : (r == 1 ? sV0 : (r == 2 ? sV1 : sV2));
        mask(kv_begin + j * BN, st);
        V8 pn[NKB][2];
        if (j > 0)
            fused(F_{}, T_{}, F_{}, nullptr, v_prev, st, nullptr, po, pn, kp, vp, nullptr,
                  nullptr);
        else
            fused(F_{}, F_{}, F_{}, nullptr, nullptr, st, nullptr, po, pn, kp, vp, nullptr,
                  nullptr);
        pv_tile(v_last, pn);
    }

    // ---- epilogue: O = a / l, LSE = ln 2 * (m + log2 l) ----
    const float lt = other_half_sum(l);
    if (qi < Sq) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const size_t row = (size_t)bh * Sq + qi;
        if (part_o != nullptr) {
            // partial state of this key chunk: O_c = a_c / l_c, LSE_c in fp64
            const size_t prow = (size_t)blockIdx.y * n_bh * Sq + row;
#pragma unroll
            for (int i = 0; i < ND; ++i)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int ch = 32 * i + 8 * r4 + 4 * h;
                    const f32x4 o4 = {acc[i][4 * r4 + 0] * inv, acc[i][4 * r4 + 1] * inv,
                                      acc[i][4 * r4 + 2] * inv, acc[i][4 * r4 + 3] * inv};
                    *reinterpret_cast<f32x4*>(part_o + prow * D + ch) = o4;
                }
            // (fp32 logarithm as in the unsplit LSE below, summed in fp64)
            if (h == 0)
                part_lse[prow] =
                    lt > 0.f ? ((double)m + (double)log2f(lt)) * (double)kLn2f : -INFINITY;
        } else {
            const size_t obase = row * D;
#pragma unroll
            for (int i = 0; i < ND; ++i)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int ch = 32 * i + 8 * r4 + 4 * h;
                    f32x4 o4 = {acc[i][4 * r4 + 0] * inv, acc[i][4 * r4 + 1] * inv,
                                acc[i][4 * r4 + 2] * inv, acc[i][4 * r4 + 3] * inv};
                    if constexpr (OUT_F32) {
                        *reinterpret_cast<f32x4*>(static_cast<float*>(Out) + obase + ch) = o4;
                    } else {
                        *reinterpret_cast<V4*>(static_cast<T*>(Out) + obase + ch) =
                            __builtin_convertvector(o4, V4);
                    }
                }
            if (LSE != nullptr && h == 0)
                LSE[row] = lt > 0.f ? (m + log2f(lt)) * kLn2f : -INFINITY;
        }
    }
    };

    // The query tiles of the workgroup in turn, through one copy of the
    // pipeline (the second starts after a barrier: the LDS buffers are
    // reused).
#pragma nounroll
    for (int t = 0; t < 2; ++t) {
        const int qt = t == 0 ? qt_first : qt_second;
        if (qt < 0) break;
        if (t > 0) __syncthreads();
        run_tile(qt);
    }
}

template <typename T, int D, int BN, int WAVES, bool OUT_F32>
hipError_t launch_one(const Problem& p) {
    constexpr int BM = 32 * WAVES;
    const int n_bh = p.B * p.H;
    const int n_qt = (p.Sq + BM - 1) / BM;
    const dim3 grid((unsigned)(n_bh * tile_pair_count(n_qt, p.causal)), (unsigned)p.n_splits);
    const dim3 block(64 * WAVES);
    const float sl2 = p.scale * kLog2ef;
    const T* q = static_cast<const T*>(p.q);
    const T* k = static_cast<const T*>(p.k);
    const T* v = static_cast<const T*>(p.v);
    if (p.causal)
        hipLaunchKernelGGL((attn_fwd_bf16_kernel<T, D, BN, WAVES, true, OUT_F32>), grid, block, 0,
                           p.stream, q, k, v, p.o, p.lse, n_bh, p.Sq, p.Skv, sl2, n_qt,
                           p.causal_off, p.kv_chunk, p.part_o, p.part_lse);
    else
        hipLaunchKernelGGL((attn_fwd_bf16_kernel<T, D, BN, WAVES, false, OUT_F32>), grid, block, 0,
                           p.stream, q, k, v, p.o, p.lse, n_bh, p.Sq, p.Skv, sl2, n_qt,
                           p.causal_off, p.kv_chunk, p.part_o, p.part_lse);
    return hipGetLastError();
}

template <typename T, int D, bool OUT_F32>
hipError_t by_tiles(const Problem& p, int bm, int bn) {
    if constexpr (D == 32) {
        // a 32-key tile holds only two score MFMAs at d = 32: 64- or 128-key
        // tiles
        if (bm == 128 && bn == 128) return launch_one<T, D, 128, 4, OUT_F32>(p);
        if (bm == 128 && bn == 64) return launch_one<T, D, 64, 4, OUT_F32>(p);
        if (bm == 64 && bn == 64) return launch_one<T, D, 64, 2, OUT_F32>(p);
    } else {
        if constexpr (D == 128) {
            if (bm == 256 && bn == 32) return launch_one<T, D, 32, 8, OUT_F32>(p);
        }
        if (bm == 128 && bn == 64) return launch_one<T, D, 64, 4, OUT_F32>(p);
        if (bm == 128 && bn == 32) return launch_one<T, D, 32, 4, OUT_F32>(p);
        if (bm == 64 && bn == 64) return launch_one<T, D, 64, 2, OUT_F32>(p);
        if (bm == 64 && bn == 32) return launch_one<T, D, 32, 2, OUT_F32>(p);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool bf16_tiles_supported(int d, int block_m, int block_n) {
    if (!(d == 32 || d == 64 || d == 128)) return false;
    if (d == 32)
        return ((block_m == 64 || block_m == 128) && block_n == 64) ||
               (block_m == 128 && block_n == 128);
    if (block_m == 256) return d == 128 && block_n == 32;
    return (block_m == 64 || block_m == 128) && (block_n == 32 || block_n == 64);
}

int bf16_lds_bytes(int d, int /*block_m*/, int block_n) {
    return 4 * 2 * block_n * d * 2;   // K and V, four buffers each
}

namespace {
template <typename T>
hipError_t by_dim(const Problem& p, const Tiles& t, bool out_f32) {
    if (p.d == 128)
        return out_f32 ? by_tiles<T, 128, true>(p, t.block_m, t.block_n)
                       : by_tiles<T, 128, false>(p, t.block_m, t.block_n);
    if (p.d == 32)
        return out_f32 ? by_tiles<T, 32, true>(p, t.block_m, t.block_n)
                       : by_tiles<T, 32, false>(p, t.block_m, t.block_n);
    return out_f32 ? by_tiles<T, 64, true>(p, t.block_m, t.block_n)
                   : by_tiles<T, 64, false>(p, t.block_m, t.block_n);
}
}  // namespace

hipError_t launch_bf16(const Problem& p, const Tiles& t) {
    if (!bf16_tiles_supported(p.d, t.block_m, t.block_n)) return hipErrorInvalidValue;
    switch (p.dtype) {
        case ATTN_BF16: return by_dim<__bf16>(p, t, false);
        case ATTN_BF16_OUT_F32: return by_dim<__bf16>(p, t, true);
        case ATTN_F16: return by_dim<_Float16>(p, t, false);
        case ATTN_F16_OUT_F32: return by_dim<_Float16>(p, t, true);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
