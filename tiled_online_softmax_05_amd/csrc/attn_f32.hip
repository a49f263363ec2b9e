// fp32 attention forward for gfx950.
//
// The online softmax of "Tiled attention: preserving results without a full
// score matrix" (section "Online normalization"), tiled over query rows and
// key rows as in the tiled lab function of "Verify tiled attention".  Each
// 64-wide wave owns 16 query rows; the workgroup's waves share one K/V tile
// staged in LDS.  A workgroup has WQ x KW waves: WQ blocks of 16 query rows,
// and KW waves per block that split every key tile among them (wave group
// kg takes keys kg * BN/KW .. of each tile), each running the online softmax
// over its own keys; at the end the KW states (m, l, a) of a row are merged
// through LDS with the rescale rule applied to whole states.  KW > 1 fills
// the SIMDs when the grid has few query tiles, with no workspace.
//
// Precision: scores are contracted on the fp64 matrix cores
// (v_mfma_f64_16x16x4_f64).  Products of two fp32 numbers are exact in fp64,
// so s_ij keeps full fp32-relative accuracy even when |s| reaches hundreds;
// the max shift s - m is taken in fp64, then exponentials, the normaliser l
// and the P.V contraction (v_mfma_f32_16x16x4_f32) run in fp32.
//
// Lane layout of a wave (lane = 16 g + c, g in 0..3, c in 0..15):
//   S^T = K Q^T, one 16x16 block per 16 keys.  v_mfma_f64_16x16x4_f64 leaves
//   D[g + 4r][c] in lane (g, c), register r, so a lane holds query c and keys
//   g + 4r (r = 0..3) of the block.  The head-dim contraction is split into
//   four contiguous quarters, quarter g fed by lane group g, so each lane
//   reads its K row and Q row as contiguous 16-byte vectors.
//   O^T = V^T P^T: the probabilities a lane already holds are exactly the B
//   operand of v_mfma_f32_16x16x4_f32 (k index g <-> key g + 4r in step r),
//   and lane (g, c) accumulates output channels 4g + r' of each 16-wide
//   channel block for query c (that instruction's result layout is
//   D[4g + r'][c]).  The rescale factor is therefore one scalar per lane.
#include "attn_internal.h"
#include "attn_device.h"

#include <cmath>

namespace attn {
namespace {

constexpr double kLog2e = 1.4426950408889634074;

template <int D, int BN, int WQ, int KW, bool CAUSAL>
__global__ __launch_bounds__(64 * WQ * KW)
void attn_fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                         const float* __restrict__ V, float* __restrict__ O,
                         float* __restrict__ LSE, int n_bh, int Sq, int Skv, double scale,
                         int n_qt, int off, int kv_chunk, float* __restrict__ part_o,
                         double* __restrict__ part_lse, int paired) {
    constexpr int WAVES = WQ * KW;
    constexpr int BM = 16 * WQ;
    constexpr int NT = 64 * WAVES;
    constexpr int KB = BN / KW;    // keys of a tile per wave
    static_assert(KB % 16 == 0, "a wave takes whole 16-key blocks");
    static_assert(KW == 1 || WQ == 1, "key-split workgroups hold one 16-row query block");
    constexpr int DQ = D / 4;      // head-dim quarter per lane group
    constexpr int KP = D + 4;      // K row pitch in floats: 16-byte reads of 8 rows spread over all banks
    constexpr int VP = D + 16;     // V row pitch: rows r and r+1 read by lanes 0-15 / 16-31 hit disjoint banks
    constexpr int NKB = KB / 16;   // 16-key blocks per tile and wave
    constexpr int ND = D / 16;     // 16-wide output channel blocks
    __shared__ __attribute__((aligned(16))) float sK[BN * KP];
    __shared__ __attribute__((aligned(16))) float sV[BN * VP];

    // Causal grids with more query tiles than compute units pair them: the
    // workgroup runs query tile n_qt-1-r and then tile r, so all workgroups
    // carry about the same number of key tiles.  Smaller grids keep one tile
    // per workgroup (heaviest first), where running two in a row would only
    // lengthen the longest path.
    int bh, qt_first, qt_second = -1;
    if (CAUSAL && paired)
        tile_pair_coords(n_bh, n_qt, true, bh, qt_first, qt_second);
    else
        tile_coords(n_bh, n_qt, CAUSAL, bh, qt_first);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wq = wave % WQ;      // query block of the wave
    const int kg = wave / WQ;      // key group of the wave
    const int g = lane >> 4;
    const int c = lane & 15;
    const int kw0 = kg * KB;       // first key of a tile this wave takes

    const float* Qh = Q + (size_t)bh * Sq * D;
    const float* Kh = K + (size_t)bh * Skv * D;
    const float* Vh = V + (size_t)bh * Skv * D;

    // ---- one query tile ----
    auto run_tile = [&](int qt) __attribute__((always_inline)) {
    const int qi = qt * BM + wq * 16 + c;

    // Q^T operand, widened to fp64: q[qi][g*DQ + t].
    double qreg[DQ];
    if (qi < Sq) {
        const f32x4* src = reinterpret_cast<const f32x4*>(Qh + (size_t)qi * D + g * DQ);
#pragma unroll
        for (int t = 0; t < DQ / 4; ++t) {
            f32x4 x = src[t];
            qreg[4 * t + 0] = x[0];
            qreg[4 * t + 1] = x[1];
            qreg[4 * t + 2] = x[2];
            qreg[4 * t + 3] = x[3];
        }
    } else {
#pragma unroll
        for (int t = 0; t < DQ; ++t) qreg[t] = 0.0;
    }

    double m = -INFINITY;       // running maximum of scaled scores
    float l = 0.f;              // this lane's part of the running normaliser
    f32x4 acc[ND];              // unnormalised output accumulator
#pragma unroll
    for (int i = 0; i < ND; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // key chunk blockIdx.y of the (possibly split) key range
    const int q_last = min(Sq, (qt + 1) * BM) - 1;
    const int kv_begin = (int)blockIdx.y * kv_chunk;
    const int kv_end = min(kv_limit(q_last, off, Skv, CAUSAL), kv_begin + min(kv_chunk, Skv));

    // K/V tile staging.  Element e (one 16-byte vector) of a tile is row
    // e / (D/4), vector e % (D/4); rows at or past Skv read as zeros.  When a
    // thread's share of a tile fits in a few registers (PF vectors per
    // operand), the next tile is fetched into registers right after the
    // current one reaches LDS, so its global-memory latency overlaps the
    // current tile's arithmetic; otherwise each tile is loaded and stored in
    // one pass.
    constexpr int NE = BN * (D / 4);
    constexpr int PF = NE % NT == 0 ? NE / NT : 0;
    constexpr bool kPrefetch = PF > 0 && PF <= (KW == 8 ? 4 : 8);
    f32x4 kpf[kPrefetch ? PF : 1], vpf[kPrefetch ? PF : 1];
    auto fetch_vec = [&](int kv0, int e, f32x4& kx, f32x4& vx) {
        const int row = e / (D / 4);
        const int c4 = e - row * (D / 4);
        const int key = kv0 + row;
        kx = f32x4{0.f, 0.f, 0.f, 0.f};
        vx = f32x4{0.f, 0.f, 0.f, 0.f};
        if (key < Skv) {
            kx = *reinterpret_cast<const f32x4*>(Kh + (size_t)key * D + 4 * c4);
            vx = *reinterpret_cast<const f32x4*>(Vh + (size_t)key * D + 4 * c4);
        }
    };
    auto store_vec = [&](int e, const f32x4& kx, const f32x4& vx) {
        const int row = e / (D / 4);
        const int c4 = e - row * (D / 4);
        *reinterpret_cast<f32x4*>(&sK[row * KP + 4 * c4]) = kx;
        *reinterpret_cast<f32x4*>(&sV[row * VP + 4 * c4]) = vx;
    };
    if constexpr (kPrefetch) {
        if (kv_begin < kv_end) {
#pragma unroll
            for (int i = 0; i < PF; ++i) fetch_vec(kv_begin, tid + i * NT, kpf[i], vpf[i]);
        }
    }

    for (int kv0 = kv_begin; kv0 < kv_end; kv0 += BN) {
        __syncthreads();
        if constexpr (kPrefetch) {
#pragma unroll
            for (int i = 0; i < PF; ++i) store_vec(tid + i * NT, kpf[i], vpf[i]);
        } else {
            for (int e = tid; e < NE; e += NT) {
                f32x4 kx, vx;
                fetch_vec(kv0, e, kx, vx);
                store_vec(e, kx, vx);
            }
        }
        __syncthreads();
        if constexpr (kPrefetch) {
            if (kv0 + BN < kv_end) {
#pragma unroll
                for (int i = 0; i < PF; ++i) fetch_vec(kv0 + BN, tid + i * NT, kpf[i], vpf[i]);
            }
        }

        // scores s = scale * q.k in fp64, masked to -inf where invisible
        double s[NKB][4];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f64x4 st = {0.0, 0.0, 0.0, 0.0};
            const float* krow = &sK[(kw0 + kb * 16 + c) * KP + g * DQ];
#pragma unroll
            for (int t = 0; t < DQ; t += 4) {
                f32x4 kx = *reinterpret_cast<const f32x4*>(krow + t);
                st = __builtin_amdgcn_mfma_f64_16x16x4f64((double)kx[0], qreg[t + 0], st, 0, 0, 0);
                st = __builtin_amdgcn_mfma_f64_16x16x4f64((double)kx[1], qreg[t + 1], st, 0, 0, 0);
                st = __builtin_amdgcn_mfma_f64_16x16x4f64((double)kx[2], qreg[t + 2], st, 0, 0, 0);
                st = __builtin_amdgcn_mfma_f64_16x16x4f64((double)kx[3], qreg[t + 3], st, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = kv0 + kw0 + kb * 16 + g + 4 * r;
                const bool vis = (j < Skv) && (!CAUSAL || j <= qi + off);
                s[kb][r] = vis ? st[r] * scale : -INFINITY;
            }
        }

        // m_new = max(m, max_j s_j) over the whole row (4 lane groups)
        double mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmax(mx, s[kb][r]);
        mx = fmax(mx, __shfl_xor(mx, 16));
        mx = fmax(mx, __shfl_xor(mx, 32));
        const double m_new = fmax(m, mx);
        // reference point for the exponentials; 0 while the row has seen no key
        const double m_ref = (m_new == -INFINITY) ? 0.0 : m_new;
        const float alpha = exp2f((float)((m - m_ref) * kLog2e));   // 0 when m = -inf

        float p[NKB][4];
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[kb][r] = exp2f((float)((s[kb][r] - m_ref) * kLog2e));
                psum += p[kb][r];
            }
        l = l * alpha + psum;
#pragma unroll
        for (int i = 0; i < ND; ++i) acc[i] *= alpha;
        m = m_new;

        // a += P V
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float* vrow = &sV[(kw0 + kb * 16 + g + 4 * r) * VP + c];
#pragma unroll
                for (int i = 0; i < ND; ++i)
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(vrow[16 * i], p[kb][r], acc[i],
                                                                  0, 0, 0);
            }
    }

    // O = a / l, LSE = m + ln l; rows that saw no key keep O = 0, LSE = -inf
    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    if constexpr (KW > 1) {
        // Merge the key groups' states of each row: M = max_k m_k,
        // w_k = e^(m_k - M) (0 for a group that saw no key), l = sum w_k l_k,
        // a = sum w_k a_k.  The tile buffers are free once every wave has
        // finished its last tile.
        static_assert(KW * 16 * D <= BN * KP, "merged accumulators fit the K buffer");
        static_assert(KW * 16 * 12 <= BN * VP * 4, "row states fit the V buffer");
        float* red_a = sK;                                         // [KW][16][D]
        double* red_m = reinterpret_cast<double*>(sV);             // [KW][16]
        float* red_l = sV + 2 * KW * 16;                           // [KW][16]
        __syncthreads();
#pragma unroll
        for (int i = 0; i < ND; ++i)
            *reinterpret_cast<f32x4*>(&red_a[(kg * 16 + c) * D + 16 * i + 4 * g]) = acc[i];
        if (g == 0) {
            red_m[kg * 16 + c] = m;
            red_l[kg * 16 + c] = lt;
        }
        __syncthreads();
        if (kg != 0) return;       // key group 0 finishes the rows (of this tile)
        double M = -INFINITY;
#pragma unroll
        for (int k = 0; k < KW; ++k) M = fmax(M, red_m[k * 16 + c]);
        lt = 0.f;
#pragma unroll
        for (int i = 0; i < ND; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KW; ++k) {
            const double mk = red_m[k * 16 + c];
            const float w = mk == -INFINITY ? 0.f : exp2f((float)((mk - M) * kLog2e));
            lt += w * red_l[k * 16 + c];
#pragma unroll
            for (int i = 0; i < ND; ++i)
                acc[i] += w * *reinterpret_cast<const f32x4*>(&red_a[(k * 16 + c) * D + 16 * i + 4 * g]);
        }
        m = M;
    }
    if (qi < Sq) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const double lse = lt > 0.f ? m + log((double)lt) : -INFINITY;
        const size_t row = (size_t)bh * Sq + qi;
        if (part_o == nullptr) {
            float* orow = O + row * D + 4 * g;
#pragma unroll
            for (int i = 0; i < ND; ++i)
                *reinterpret_cast<f32x4*>(orow + 16 * i) = acc[i] * inv;
            if (LSE != nullptr && g == 0) LSE[row] = (float)lse;
        } else {
            // partial state of this key chunk: O_c = a_c / l_c, LSE_c in fp64
            const size_t prow = (size_t)blockIdx.y * n_bh * Sq + row;
            float* orow = part_o + prow * D + 4 * g;
#pragma unroll
            for (int i = 0; i < ND; ++i)
                *reinterpret_cast<f32x4*>(orow + 16 * i) = acc[i] * inv;
            if (g == 0) part_lse[prow] = lse;
        }
    }
    };

    // The query tiles of the workgroup in turn, through one copy of the tile
    // code (the second starts after a barrier: the LDS buffers are reused).
#pragma nounroll
    for (int t = 0; t < 2; ++t) {
        const int qt = t == 0 ? qt_first : qt_second;
        if (qt < 0) break;
        if (t > 0) __syncthreads();
        run_tile(qt);
    }
}

template <int D, int BN, int WQ, int KW>
hipError_t launch_one(const Problem& p) {
    constexpr int BM = 16 * WQ;
    const int n_bh = p.B * p.H;
    const int n_qt = (p.Sq + BM - 1) / BM;
    // pair causal query tiles when there are more of them than compute units
    const int paired = p.causal && (long)n_bh * n_qt > 256 ? 1 : 0;
    const dim3 grid((unsigned)(n_bh * (paired ? tile_pair_count(n_qt, true) : n_qt)),
                    (unsigned)p.n_splits);
    const dim3 block(64 * WQ * KW);
    const double scale = (double)p.scale;
    const float* q = static_cast<const float*>(p.q);
    const float* k = static_cast<const float*>(p.k);
    const float* v = static_cast<const float*>(p.v);
    float* o = static_cast<float*>(p.o);
    if (p.causal)
        hipLaunchKernelGGL((attn_fwd_f32_kernel<D, BN, WQ, KW, true>), grid, block, 0, p.stream,
                           q, k, v, o, p.lse, n_bh, p.Sq, p.Skv, scale, n_qt, p.causal_off, p.kv_chunk,
                           p.part_o, p.part_lse, paired);
    else
        hipLaunchKernelGGL((attn_fwd_f32_kernel<D, BN, WQ, KW, false>), grid, block, 0, p.stream,
                           q, k, v, o, p.lse, n_bh, p.Sq, p.Skv, scale, n_qt, p.causal_off, p.kv_chunk,
                           p.part_o, p.part_lse, paired);
    return hipGetLastError();
}

template <int D, int BN>
hipError_t by_waves(const Problem& p, int wq, int kw) {
    if (kw == 1) {
        if constexpr (BN == 128) {
            // 128-key tiles are built for 16-row query blocks only
            if (wq == 1) return launch_one<D, BN, 1, 1>(p);
            return hipErrorInvalidValue;
        } else {
            switch (wq) {
                case 1: return launch_one<D, BN, 1, 1>(p);
                case 2: return launch_one<D, BN, 2, 1>(p);
                case 4: return launch_one<D, BN, 4, 1>(p);
                default: return hipErrorInvalidValue;
            }
        }
    }
    if (wq != 1) return hipErrorInvalidValue;
    if constexpr (BN >= 32) {
        if (kw == 2) return launch_one<D, BN, 1, 2>(p);
    }
    if constexpr (BN >= 64) {
        if (kw == 4) return launch_one<D, BN, 1, 4>(p);
    }
    if constexpr (BN >= 128 && D < 128) {
        if (kw == 8) return launch_one<D, BN, 1, 8>(p);
    }
    return hipErrorInvalidValue;
}

template <int D>
hipError_t by_bn(const Problem& p, int bn, int wq, int kw) {
    switch (bn) {
        case 16: return by_waves<D, 16>(p, wq, kw);
        case 32: return by_waves<D, 32>(p, wq, kw);
        case 64: return by_waves<D, 64>(p, wq, kw);
        case 128: return by_waves<D, 128>(p, wq, kw);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool f32_tiles_supported(int d, int block_m, int block_n) {
    const bool dm = d == 16 || d == 32 || d == 64 || d == 128;
    const bool bm = block_m == 16 || block_m == 32 || block_m == 64;
    const bool bn = block_n == 16 || block_n == 32 || block_n == 64 ||
                    (block_n == 128 && block_m == 16);
    return dm && bm && bn;
}

int f32_lds_bytes(int d, int /*block_m*/, int block_n) {
    return block_n * ((d + 4) + (d + 16)) * (int)sizeof(float);
}

int f32_key_waves(int d, int block_m, int block_n, long query_tiles) {
    if (block_m != 16) return 1;
    // 128-key tiles: eight waves of 16 keys each (four at d = 128, where
    // eight would not fit two waves per SIMD in registers)
    if (block_n == 128) return d == 128 ? 4 : 8;
    const int kw = query_tiles >= 1024 ? 1 : (query_tiles >= 512 ? 2 : 4);
    return kw < block_n / 16 ? kw : block_n / 16;
}

hipError_t launch_f32(const Problem& p, const Tiles& t) {
    if (!f32_tiles_supported(p.d, t.block_m, t.block_n)) return hipErrorInvalidValue;
    const int wq = t.block_m / 16;
    const long n_qt = (p.Sq + t.block_m - 1) / t.block_m;
    const int kw = f32_key_waves(p.d, t.block_m, t.block_n, (long)p.B * p.H * n_qt);
    switch (p.d) {
        case 16: return by_bn<16>(p, t.block_n, wq, kw);
        case 32: return by_bn<32>(p, t.block_n, wq, kw);
        case 64: return by_bn<64>(p, t.block_n, wq, kw);
        case 128: return by_bn<128>(p, t.block_n, wq, kw);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
