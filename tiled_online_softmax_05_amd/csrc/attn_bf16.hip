// bf16 attention forward for gfx950 (bf16 MFMA, fp32 accumulation).
//
// The online softmax of "Tiled attention: preserving results without a full
// score matrix" (section "Online normalization") over query tiles and key
// tiles as in the tiled lab function of "Verify tiled attention".  Each
// 64-wide wave owns 32 query rows; the waves of a workgroup share one K/V
// tile staged in LDS.  The next tile's HBM loads are issued before the
// current tile is computed, so they overlap with the MFMA work.
//
// Contractions use v_mfma_f32_32x32x16_bf16 (A 32x16, B 16x32, D 32x32):
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
// of the next contraction O^T = V^T P^T.  V is stored transposed in LDS
// ([channel][key]) so the A operand of that contraction is one 16-byte read.
//
// Exponentials are base 2 with scale * log2(e) folded into one FMA; the
// running maximum m is kept in that scaled base-2 domain.
#include "attn_internal.h"
#include "attn_device.h"

#include <cmath>

namespace attn {
namespace {

constexpr float kLog2ef = 1.44269504088896341f;
constexpr float kLn2f = 0.693147180559945309f;

// LDS row of key k (0..31) inside its 32-key block (inverse of sigma).
__device__ __forceinline__ int key_slot(int k) {
    const int a = 2 * (k >> 4) + ((k >> 2) & 1);
    const int h = (k >> 3) & 1;
    return 8 * a + 4 * h + (k & 3);
}

// s_waitcnt immediate: vmcnt = 0, expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVmcnt0 = 0x0F70;

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

template <int D, int BN, int WAVES, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                          const __bf16* __restrict__ V, void* __restrict__ Out,
                          float* __restrict__ LSE, int n_bh, int Sq, int Skv, float sl2,
                          int n_qt) {
    constexpr int BM = 32 * WAVES;
    constexpr int NT = 64 * WAVES;
    constexpr int KP = D + 8;          // sK row pitch (bf16 elements)
    constexpr int VP = BN + 8;         // sVt row pitch (bf16 elements)
    constexpr int KS = D / 16;         // k-steps of the score contraction
    constexpr int NKB = BN / 32;       // 32-key blocks per tile
    constexpr int ND = D / 32;         // 32-channel output blocks
    constexpr int DCH = D / 8;         // 16-byte chunks per K/V row
    constexpr int ROWB = D * 2;        // bytes per K/V row
    constexpr int K_ITEMS = BN * DCH;              // one 16-byte chunk each
    constexpr int V_ITEMS = (BN / 4) * DCH;        // 4 keys x 8 channels each
    constexpr int K_PER = (K_ITEMS + NT - 1) / NT;
    constexpr int V_PER = (V_ITEMS + NT - 1) / NT;
    static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");

    __shared__ __attribute__((aligned(16))) __bf16 sK[BN * KP];
    __shared__ __attribute__((aligned(16))) __bf16 sVt[D * VP];

    int bh, qt;
    tile_coords(n_bh, n_qt, CAUSAL, bh, qt);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int c = lane & 31;
    const int off = Skv - Sq;
    const int q0w = qt * BM + wave * 32;
    const int qi = q0w + c;

    const __bf16* Qh = Q + (size_t)bh * Sq * D;
    const __bf16* Kh = K + (size_t)bh * Skv * D;
    const __bf16* Vh = V + (size_t)bh * Skv * D;

    // Q^T operand: lane holds q[qi][16 ks + 8 h .. +7]; rows past Sq read 0
    bf16x8 qop[KS];
    {
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(Qh, (uint32_t)Sq * ROWB);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 x = buffer_load16(rq, (uint32_t)qi * ROWB + 32 * ks + 16 * h);
            qop[ks] = __builtin_bit_cast(bf16x8, x);
        }
        // Retire the Q loads here, on every path: vmcnt is in-order, and Q
        // loads still in flight at the loop entry would make every tile wait
        // for its own K/V prefetch before the first MFMA.
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }

    float m = -INFINITY;     // running max of scale*log2(e)*s
    float l = 0.f;           // this lane's part of the normaliser
    f32x16 acc[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) acc[i] = f32x16{};

    const int q_last = min(Sq, (qt + 1) * BM) - 1;
    const int kv_end = kv_limit(q_last, Sq, Skv, CAUSAL);
    // last key this lane's query may see (for the masked tiles)
    const int lim = CAUSAL ? min(Skv - 1, qi + off) : Skv - 1;

    // ---- K/V tile staging: HBM -> registers -> LDS ----
    // One descriptor per head; the tile offset rides in the per-lane offset so
    // rows at or past Skv fall outside the descriptor's range and read 0.
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(Kh, (uint32_t)Skv * ROWB);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(Vh, (uint32_t)Skv * ROWB);
    constexpr bool K_FULL = K_ITEMS % NT == 0;   // every thread has K_PER items
    constexpr bool V_FULL = V_ITEMS % NT == 0;
    u32x4 kreg[K_PER];
    u32x4 vreg[V_PER][4];
    auto load_tile = [&](int kv0) {
        const uint32_t tile_off = (uint32_t)kv0 * ROWB;
#pragma unroll
        for (int i = 0; i < K_PER; ++i) {
            const int e = tid + i * NT;
            const int row = e / DCH, ch = e % DCH;
            if (K_FULL || e < K_ITEMS)
                kreg[i] = buffer_load16(rk, tile_off + row * ROWB + 16 * ch);
        }
#pragma unroll
        for (int i = 0; i < V_PER; ++i) {
            const int e = tid + i * NT;
            const int kg = e / DCH, ch = e % DCH;
            if (V_FULL || e < V_ITEMS) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    vreg[i][t] = buffer_load16(rv, tile_off + (4 * kg + t) * ROWB + 16 * ch);
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < K_PER; ++i) {
            const int e = tid + i * NT;
            if (K_FULL || e < K_ITEMS) {
                const int row = e / DCH, ch = e % DCH;
                const int slot = (row & ~31) + key_slot(row & 31);
                *reinterpret_cast<u32x4*>(&sK[slot * KP + 8 * ch]) = kreg[i];
            }
        }
#pragma unroll
        for (int i = 0; i < V_PER; ++i) {
            const int e = tid + i * NT;
            if (V_FULL || e < V_ITEMS) {
                const int kg = e / DCH, ch = e % DCH;
                // channels 8 ch + 2 w and 8 ch + 2 w + 1 of keys 4 kg .. 4 kg + 3
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    u32x2 lo, hi;
                    lo[0] = __builtin_amdgcn_perm(vreg[i][1][w], vreg[i][0][w], 0x05040100u);
                    lo[1] = __builtin_amdgcn_perm(vreg[i][3][w], vreg[i][2][w], 0x05040100u);
                    hi[0] = __builtin_amdgcn_perm(vreg[i][1][w], vreg[i][0][w], 0x07060302u);
                    hi[1] = __builtin_amdgcn_perm(vreg[i][3][w], vreg[i][2][w], 0x07060302u);
                    const int ch0 = 8 * ch + 2 * w;
                    *reinterpret_cast<u32x2*>(&sVt[ch0 * VP + 4 * kg]) = lo;
                    *reinterpret_cast<u32x2*>(&sVt[(ch0 + 1) * VP + 4 * kg]) = hi;
                }
            }
        }
    };

    if (kv_end > 0) {
        load_tile(0);
        store_tile();
    }
    __syncthreads();

    for (int kv0 = 0; kv0 < kv_end; kv0 += BN) {
        const bool has_next = kv0 + BN < kv_end;
        if (has_next) load_tile(kv0 + BN);

        // ---- S^T = K Q^T (raw scores, fp32) ----
        f32x16 st[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            st[kb] = f32x16{};
            const __bf16* krow = &sK[(kb * 32 + c) * KP + 8 * h];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 16 * ks);
                st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[ks], st[kb], 0, 0, 0);
            }
        }

        // ---- mask: only tiles crossing the key end or the causal diagonal ----
        const bool need_mask = (kv0 + BN > Skv) || (CAUSAL && kv0 + BN - 1 > q0w + off);
        if (need_mask) {
            const int base = lim - kv0 - 8 * h;     // visible iff key offset <= base
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int jo = kb * 32 + 16 * (r >> 3) + (r & 7);
                    if (jo > base) st[kb][r] = -INFINITY;
                }
        }

        // ---- online softmax update ----
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m, mx * sl2);
        const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m - m_ref);   // 0 while m = -inf

        bf16x8 pb[NKB][2];
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                f32x8 pf;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float pv = __builtin_amdgcn_exp2f(fmaf(st[kb][8 * half + j], sl2, -m_ref));
                    pf[j] = pv;
                    psum += pv;
                }
                pb[kb][half] = __builtin_convertvector(pf, bf16x8);
            }
        l = l * alpha + psum;
        // the accumulator changes only where the maximum rose (alpha != 1)
        if (__any(m_new > m)) {
#pragma unroll
            for (int i = 0; i < ND; ++i) acc[i] *= alpha;
        }
        m = m_new;

        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int kcol = 32 * kb + 16 * half + 8 * h;
#pragma unroll
                for (int i = 0; i < ND; ++i) {
                    const bf16x8 a =
                        *reinterpret_cast<const bf16x8*>(&sVt[(32 * i + c) * VP + kcol]);
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][half], acc[i],
                                                                     0, 0, 0);
                }
            }

        __syncthreads();
        if (has_next) {
            store_tile();
            __syncthreads();
        }
    }

    // ---- epilogue: O = a / l, LSE = ln 2 * (m + log2 l) ----
    const float lt = l + __shfl_xor(l, 32);
    if (qi < Sq) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const size_t obase = ((size_t)bh * Sq + qi) * D;
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
                    *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(Out) + obase + ch) =
                        __builtin_convertvector(o4, bf16x4);
                }
            }
        if (LSE != nullptr && h == 0)
            LSE[(size_t)bh * Sq + qi] = lt > 0.f ? (m + log2f(lt)) * kLn2f : -INFINITY;
    }
}

template <int D, int BN, int WAVES, bool OUT_F32>
hipError_t launch_one(const Problem& p) {
    constexpr int BM = 32 * WAVES;
    const int n_bh = p.B * p.H;
    const int n_qt = (p.Sq + BM - 1) / BM;
    const dim3 grid((unsigned)(n_bh * n_qt));
    const dim3 block(64 * WAVES);
    const float sl2 = p.scale * kLog2ef;
    const __bf16* q = static_cast<const __bf16*>(p.q);
    const __bf16* k = static_cast<const __bf16*>(p.k);
    const __bf16* v = static_cast<const __bf16*>(p.v);
    if (p.causal)
        hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, BN, WAVES, true, OUT_F32>), grid, block, 0,
                           p.stream, q, k, v, p.o, p.lse, n_bh, p.Sq, p.Skv, sl2, n_qt);
    else
        hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, BN, WAVES, false, OUT_F32>), grid, block, 0,
                           p.stream, q, k, v, p.o, p.lse, n_bh, p.Sq, p.Skv, sl2, n_qt);
    return hipGetLastError();
}

template <int D, bool OUT_F32>
hipError_t by_tiles(const Problem& p, int bm, int bn) {
    if (bm == 128 && bn == 64) return launch_one<D, 64, 4, OUT_F32>(p);
    if (bm == 128 && bn == 32) return launch_one<D, 32, 4, OUT_F32>(p);
    if (bm == 64 && bn == 64) return launch_one<D, 64, 2, OUT_F32>(p);
    if (bm == 64 && bn == 32) return launch_one<D, 32, 2, OUT_F32>(p);
    return hipErrorInvalidValue;
}

}  // namespace

bool bf16_tiles_supported(int d, int block_m, int block_n) {
    return (d == 64 || d == 128) && (block_m == 64 || block_m == 128) &&
           (block_n == 32 || block_n == 64);
}

int bf16_lds_bytes(int d, int /*block_m*/, int block_n) {
    return (block_n * (d + 8) + d * (block_n + 8)) * 2;
}

hipError_t launch_bf16(const Problem& p, const Tiles& t) {
    if (!bf16_tiles_supported(p.d, t.block_m, t.block_n)) return hipErrorInvalidValue;
    const bool out_f32 = p.dtype == 2;
    if (p.d == 128)
        return out_f32 ? by_tiles<128, true>(p, t.block_m, t.block_n)
                       : by_tiles<128, false>(p, t.block_m, t.block_n);
    return out_f32 ? by_tiles<64, true>(p, t.block_m, t.block_n)
                   : by_tiles<64, false>(p, t.block_m, t.block_n);
}

}  // namespace attn
