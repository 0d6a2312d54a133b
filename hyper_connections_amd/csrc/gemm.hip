// Multi-row INT4-affine dequantizing GEMM on the matrix cores: the batched chunked-prefill
// projection (m <= 128) and the multi-row arm of the GEMV (m <= 16, e.g. the LM head over
// several rows, with argmax).
//
// "src/real_forward.rs" (turbospark-runtime 0.3.0), fields batched_gemv_prefill and
// prefill_steel: resident GEMVs of a prefill micro-batch run as one M-row GEMM. The pages'
// Metal kernels (per-thread accumulator arrays; a simdgroup-matrix variant) are prior art;
// this is a gfx950 design around v_mfma_f32_32x32x16_f16:
//
//  * A block owns a 32*MT x 64 output tile (activation rows x weight rows). Its waves (four or
//    eight) split K into contiguous ranges of stages (S k-blocks of 64 each); each wave keeps the
//    whole tile in its accumulators and works out of a private LDS region, so waves never wait
//    for each other until the end.
//  * Operands reach LDS through fully coalesced 16-byte loads (consecutive lanes walk one row's
//    bytes), issued a stage ahead and parked in registers while the current stage computes.
//    Reading MFMA fragments straight from row-major memory would touch 32 separate cache lines
//    per instruction instead.
//  * The weight tile is the B operand: lane l takes weight row l % 32 and a 32-wide k slice,
//    turns its 16 bytes of codes into fp16 q*s+b in registers (the nibble trick of unpack8 and
//    one packed fma) and feeds four MFMA steps. The activation tile is the A operand, read with
//    the same permutation of k inside each group of eight, so both operands agree on which k
//    each register slot holds.
//  * The waves' partial tiles meet in LDS (one slice each, written at once) and every output
//    is summed over them in a fixed order, so results are deterministic. The epilogue writes fp16 or fp32 and, for the GEMV arm, a per-block
//    argmax partial per row, reduced by the same small final kernel the M=1 path uses.
#include "dhp_internal.hpp"

#include <math.h>
#include <limits.h>

typedef float f16x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int BN = 64;         // output columns (weight rows) per block
constexpr int LDW = BN + 4;    // LDS row pitch in floats

DHP_DEV h8 dequant8(uint32_t w, h2 s2, h2 b2, const NibConsts& k) {
    h2 q[4];
    unpack8(w, q, k);
    const h2 p0 = __builtin_elementwise_fma(q[0], s2, b2);
    const h2 p1 = __builtin_elementwise_fma(q[1], s2, b2);
    const h2 p2 = __builtin_elementwise_fma(q[2], s2, b2);
    const h2 p3 = __builtin_elementwise_fma(q[3], s2, b2);
    return h8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

DHP_DEV h8 permute_x8(u32x4 u) {
    h2 p[4];
    permute8(u.x, u.y, u.z, u.w, p);
    return h8{p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
}

// One wave's share of a block: output tile 32*MT (activation rows) x 64 (weight rows), and a
// contiguous range of 64-k blocks walked in stages of S k-blocks. Each stage is fetched from
// global memory with fully coalesced 16-byte loads (for S = 4, eight lanes cover one 128-byte
// line of a weight row), parked in registers while the previous stage computes, then written
// to this wave's private LDS region, from which the MFMA fragments are read. Row pitches carry
// 16 extra bytes so consecutive rows start four banks apart.
template <int MT, int S>
struct WaveLds {
    static constexpr int WP = 32 * S + 16;    // bytes per weight row (codes of S k-blocks)
    static constexpr int XP = 128 * S + 16;   // bytes per activation row (64 * S halves)
    static constexpr int SBP = S + 1;         // uint32 (scale | bias << 16) per weight row
    static constexpr int W_BYTES = 64 * WP;
    static constexpr int X_BYTES = 32 * MT * XP;
    static constexpr int SB_BYTES = 64 * SBP * 4;
    static constexpr int TRASH = W_BYTES + X_BYTES + SB_BYTES;   // 16 bytes per lane: rows past the tile
    static constexpr int BYTES = TRASH + 64 * 16;
    static constexpr int WL = 2 * S;          // 16-byte weight loads per lane per stage
    static constexpr int XL = 4 * MT * S;     // 16-byte activation loads per lane per stage (max)
};

template <int MT, int S>
struct StageRegs {
    u32x4 w[WaveLds<MT, S>::WL];
    u32x4 x[WaveLds<MT, S>::XL];
    uint32_t sc[S], bi[S];
    int kbs;                                   // first k-block of the stage
};

// Per-lane load and store addresses of a stage, computed once per wave (only the k offset
// changes from stage to stage).
template <int MT, int S>
struct StagePlan {
    const uint8_t* wsrc[WaveLds<MT, S>::WL];   // weight row start + byte offset of this lane's chunk
    int wkb[WaveLds<MT, S>::WL];               // k-block of that chunk within a stage
    int wdst[WaveLds<MT, S>::WL];              // LDS byte offset
    const _Float16* xbase;                     // first activation row of the tile (wave-uniform)
    int xoff[WaveLds<MT, S>::XL];              // halves from xbase (row clamped into the tile)
    int xkb[WaveLds<MT, S>::XL];
    int xdst[WaveLds<MT, S>::XL];              // LDS byte offset (the trash slot for rows past the tile)
    const uint16_t* ssrc;
    const uint16_t* bsrc;
};

template <int MT, int S>
DHP_DEV void stage_plan(StagePlan<MT, S>& p, int lane, const uint8_t* codes, const uint16_t* scales,
                        const uint16_t* biases, const _Float16* X, int n0, int N, int m0, int xrows,
                        int K, int KB, int hmix = 0) {
    // hmix > 0: tile column r is weight row (r / 16) * hmix + n0 + r % 16 (four streams of 16
    // positions, for the fused stream mix); otherwise n0 + r
    auto wrow = [&](int r) { return hmix > 0 ? (r >> 4) * hmix + n0 + (r & 15) : min(n0 + r, N - 1); };
    using L = WaveLds<MT, S>;
    const size_t row_bytes = (size_t)K >> 1;
#pragma unroll
    for (int i = 0; i < L::WL; ++i) {
        const int c = i * 64 + lane;
        const int row = c / (2 * S), cc = c % (2 * S);
        p.wsrc[i] = codes + (size_t)wrow(row) * row_bytes + (cc & 1) * 16;
        p.wkb[i] = cc >> 1;
        p.wdst[i] = row * L::WP + cc * 16;
    }
    p.xbase = X + (size_t)m0 * K;
#pragma unroll
    for (int i = 0; i < L::XL; ++i) {
        const int c = i * 64 + lane;
        const int row = c / (8 * S), cc = c % (8 * S);
        p.xoff[i] = min(row, xrows - 1) * K + (cc & 7) * 8;
        p.xkb[i] = cc >> 3;
        p.xdst[i] = (row < xrows) ? L::W_BYTES + row * L::XP + cc * 16 : L::TRASH + 16 * lane;
    }
    const size_t n = (size_t)wrow(lane);
    p.ssrc = scales + n * KB;
    p.bsrc = biases + n * KB;
}

// Global loads of the stage that starts at k-block kbs (k-blocks at or past kb1 are padding:
// their addresses are clamped to the last real k-block and their scale and bias read as zero,
// so they dequantize to exact zeros).
template <int MT, int S>
DHP_DEV void stage_load(StageRegs<MT, S>& r, const StagePlan<MT, S>& p, int kbs, int kb1) {
    using L = WaveLds<MT, S>;
#pragma unroll
    for (int i = 0; i < L::WL; ++i)
        r.w[i] = *reinterpret_cast<const u32x4*>(p.wsrc[i] + (size_t)min(kbs + p.wkb[i], kb1 - 1) * 32);
    // every activation load is issued (rows past the tile are clamped to its last row and parked
    // in a trash slot), so loads and stores stay unconditional and the compiler can count them
#pragma unroll
    for (int i = 0; i < L::XL; ++i)
        r.x[i] = *reinterpret_cast<const u32x4*>(p.xbase + (p.xoff[i] + min(kbs + p.xkb[i], kb1 - 1) * 64));
    // scales and biases: the raw 16-bit words (any arithmetic on them here would make the wave
    // wait for this stage's loads right after issuing them)
#pragma unroll
    for (int q = 0; q < S; ++q) {
        const int kb = min(kbs + q, kb1 - 1);
        r.sc[q] = p.ssrc[kb];
        r.bi[q] = p.bsrc[kb];
    }
    // k-blocks past kb1 are masked when the stage is parked in LDS, not here: a select on a
    // loaded value would make the wave wait for this stage's loads right after issuing them
    r.kbs = kbs;
}

template <int MT, int S>
DHP_DEV void stage_store(const StageRegs<MT, S>& r, const StagePlan<MT, S>& p, uint8_t* lds, int lane, int kb1) {
    using L = WaveLds<MT, S>;
#pragma unroll
    for (int i = 0; i < L::WL; ++i) *reinterpret_cast<u32x4*>(lds + p.wdst[i]) = r.w[i];
#pragma unroll
    for (int i = 0; i < L::XL; ++i) *reinterpret_cast<u32x4*>(lds + p.xdst[i]) = r.x[i];
    uint32_t* sb = reinterpret_cast<uint32_t*>(lds + L::W_BYTES + L::X_BYTES);
    // padding k-blocks (at or past kb1) get scale and bias 0: their codes dequantize to zeros
#pragma unroll
    for (int q = 0; q < S; ++q) sb[lane * L::SBP + q] = (r.kbs + q < kb1) ? (r.sc[q] | (r.bi[q] << 16)) : 0u;
}

// MFMAs of one stage from LDS. B fragment of lane (li, g) for k-block q4: weight row 32 nt + li,
// codes q4*32 + 16 g .. +16 (32 codes, four MFMA steps); A fragment: activation row 32 mt + li,
// halves q4*64 + 32 g + 8 q .. +8 (permuted like the codes).
template <int MT, int S>
DHP_DEV void stage_mfma(const uint8_t* lds, int li, int g, f16x16 (*acc)[2], const NibConsts& nk) {
    using L = WaveLds<MT, S>;
    const uint8_t* xl = lds + L::W_BYTES;
    const uint32_t* sb = reinterpret_cast<const uint32_t*>(lds + L::W_BYTES + L::X_BYTES);
#pragma unroll
    for (int q4 = 0; q4 < S; ++q4) {
        u32x4 cw[2];
        h2 s2[2], b2[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int row = 32 * nt + li;
            cw[nt] = *reinterpret_cast<const u32x4*>(lds + row * L::WP + q4 * 32 + 16 * g);
            const uint32_t sbv = sb[row * L::SBP + q4];
            const _Float16 s16 = (_Float16)bf16_to_f32(sbv & 0xFFFFu);
            const _Float16 b16 = (_Float16)bf16_to_f32(sbv >> 16);
            s2[nt] = h2{s16, s16};
            b2[nt] = h2{b16, b16};
        }
        // one MFMA step at a time: its two B fragments, then the MT activation fragments
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            h8 b[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) b[nt] = dequant8(cw[nt][q], s2[nt], b2[nt], nk);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const u32x4 xv = *reinterpret_cast<const u32x4*>(xl + (32 * mt + li) * L::XP + q4 * 128 + 64 * g + 16 * q);
                const h8 a = permute_x8(xv);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b[nt], acc[mt][nt], 0, 0, 0);
            }
        }
    }
}

// A second weight sharing the activations and K of a launch: column blocks from `nb` on take it
// (its rows, its output Y with its own N). nb >= the grid's column blocks means none.
struct GemmAlt {
    const uint8_t* codes;
    const uint16_t* scales;
    const uint16_t* biases;
    void* Y;
    int N;
    int nb;
    // the fused stream mix (MIX kernels): mixed[m][h] = (1/4) sum_c sigmoid(y[m][c*H + h]) *
    // normed[m][c*H + h] over 4 streams of H positions; y itself is not stored
    const _Float16* normed;
    _Float16* mixed;
    int H;
};

template <int MT, int S, int WAVES, bool F32OUT, bool ARGMAX, int DEPTH, bool ALT, bool MIX>
__global__ __launch_bounds__(64 * WAVES) void k_gemm_mfma(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, const _Float16* __restrict__ X, int M, int N, int K,
    void* __restrict__ Y, float* __restrict__ part_v, int* __restrict__ part_i, int kb_split, GemmAlt alt) {
    using L = WaveLds<MT, S>;
    constexpr int ROWS = 32 * MT;
    extern __shared__ __align__(16) uint8_t lds_all[];   // one region per wave; reused by the epilogue
    float* tile = reinterpret_cast<float*>(lds_all);

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int li = lane & 31;
    const int g = lane >> 5;
    const bool second = ALT && (int)blockIdx.x >= alt.nb;     // the same in the whole block
    if (second) {
        codes = alt.codes;
        scales = alt.scales;
        biases = alt.biases;
        Y = alt.Y;
        N = alt.N;
    }
    // MIX: a block owns 16 positions of each of the 4 streams
    const int n0 = MIX ? (int)blockIdx.x * 16 : (second ? (int)blockIdx.x - alt.nb : (int)blockIdx.x) * BN;
    const int m0 = blockIdx.y * ROWS;
    const int KB = K >> 6;
    const int xrows = min(ROWS, M - m0);       // activation rows that exist in this tile
    uint8_t* lds = lds_all + wave * L::BYTES;

    f16x16 acc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f16x16{};

    // the block's share of K (blockIdx.z of a split-K launch: k-blocks [zb0, zb1), a multiple of
    // S apart; the whole of K otherwise), then a stage-aligned split of it over the waves
    const int zb0 = blockIdx.z * kb_split, zb1 = min(KB, zb0 + kb_split);
    const int ST = (zb1 - zb0 + S - 1) / S;
    const int st0 = zb0 / S + (ST * wave) / WAVES, st1 = zb0 / S + (ST * (wave + 1)) / WAVES;
    const int kb1 = min(st1 * S, zb1);
    if constexpr (F32OUT) Y = reinterpret_cast<float*>(Y) + (size_t)blockIdx.z * M * N;   // the split's partial
    const bool has = st0 < st1;
    StagePlan<MT, S> plan;
    StageRegs<MT, S> r0, r1;
    // two register sets: while stage st computes out of LDS, stages st+1 and st+2 are in flight
    if (has) {
        stage_plan<MT, S>(plan, lane, codes, scales, biases, X, n0, N, m0, xrows, K, KB, MIX ? alt.H : 0);
        stage_load<MT, S>(r0, plan, st0 * S, kb1);
        if constexpr (DEPTH == 2) stage_load<MT, S>(r1, plan, (st0 + 1) * S, kb1);
    }
    if (DEPTH == 1 && has) {
        // one register set: the next stage is in flight while this one computes
        const NibConsts nk = nib_consts();
        int st = st0;
        for (; st + 1 < st1; ++st) {
            stage_store<MT, S>(r0, plan, lds, lane, kb1);
            __builtin_amdgcn_wave_barrier();
            stage_load<MT, S>(r0, plan, (st + 1) * S, kb1);
            stage_mfma<MT, S>(lds, li, g, acc, nk);
            __builtin_amdgcn_wave_barrier();
        }
        stage_store<MT, S>(r0, plan, lds, lane, kb1);
        __builtin_amdgcn_wave_barrier();
        stage_mfma<MT, S>(lds, li, g, acc, nk);
    }
    if (DEPTH == 2 && has) {
        const NibConsts nk = nib_consts();
        // The steady-state loop has no branch around a load (the compiler then waits for exactly
        // the set it is about to park): the stage count is padded to even (the padding stage's
        // k-blocks are past kb1, so it is loaded clamped and never multiplied) and the last pair
        // is peeled off.
        const int st1e = st0 + ((st1 - st0 + 1) & ~1);
        int st = st0;
        for (; st + 2 < st1e; st += 2) {
            stage_store<MT, S>(r0, plan, lds, lane, kb1);
            __builtin_amdgcn_wave_barrier();
            stage_load<MT, S>(r0, plan, (st + 2) * S, kb1);
            stage_mfma<MT, S>(lds, li, g, acc, nk);
            __builtin_amdgcn_wave_barrier();
            stage_store<MT, S>(r1, plan, lds, lane, kb1);
            __builtin_amdgcn_wave_barrier();
            stage_load<MT, S>(r1, plan, (st + 3) * S, kb1);
            stage_mfma<MT, S>(lds, li, g, acc, nk);
            __builtin_amdgcn_wave_barrier();
        }
        stage_store<MT, S>(r0, plan, lds, lane, kb1);
        __builtin_amdgcn_wave_barrier();
        stage_mfma<MT, S>(lds, li, g, acc, nk);
        __builtin_amdgcn_wave_barrier();
        if (st + 1 < st1) {
            stage_store<MT, S>(r1, plan, lds, lane, kb1);
            __builtin_amdgcn_wave_barrier();
            stage_mfma<MT, S>(lds, li, g, acc, nk);
        }
    }
    __syncthreads();                           // staging regions are now free for the epilogue

    // every wave parks its partial tile in a slice of its own; then each thread sums its outputs
    // over the slices in a fixed order (the last wave's first, down to wave 0), so a result does
    // not depend on timing
    constexpr int SLICE = ROWS * LDW;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);
                tile[wave * SLICE + i * LDW + 32 * nt + li] = acc[mt][nt][r];
            }
    __syncthreads();

    // epilogue: all threads over ROWS x 64 outputs; TPR threads per row, contiguous columns
    constexpr int TPR = 64 * WAVES / ROWS;
    constexpr int CPT = BN / TPR;
    const int row = threadIdx.x / TPR;
    const int c0 = (threadIdx.x % TPR) * CPT;
    const int m = m0 + row;
    float bv = -INFINITY;
    int bi = INT_MAX;
    if (m < M) {
        float v[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            v[c] = tile[(WAVES - 1) * SLICE + row * LDW + c0 + c];
#pragma unroll
            for (int w = WAVES - 2; w >= 0; --w) v[c] += tile[w * SLICE + row * LDW + c0 + c];
        }
        const int nb = n0 + c0;
        // the thread's CPT contiguous outputs in one or two 16-byte stores when the row allows
        const bool vec = (reinterpret_cast<uintptr_t>(Y) & 15) == 0 && (N & 7) == 0 && nb + CPT <= N;
        if constexpr (MIX) {
            // the row's four threads hold its four streams (16 positions each): sigmoid times the
            // normed value, summed over the streams across the quad, then the mean; each thread
            // writes 4 of the 16 positions
            static_assert(TPR == 4 && CPT == 16, "the fused mix needs 4 threads of 16 columns per row");
            const int c = threadIdx.x % TPR;
            const size_t wide = (size_t)4 * alt.H;
            const u32x4* np = reinterpret_cast<const u32x4*>(alt.normed + (size_t)m * wide + (size_t)c * alt.H + n0);
            const u32x4 na = np[0], nb8 = np[1];
            const uint32_t nw[8] = {na.x, na.y, na.z, na.w, nb8.x, nb8.y, nb8.z, nb8.w};
            float sm[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const h2 pr = as_h2(nw[k >> 1]);
                sm[k] = sigmoid_f(v[k]) * (float)((k & 1) ? pr.y : pr.x);
                sm[k] = group_sum<4>(sm[k]);
            }
            _Float16* mp = alt.mixed + (size_t)m * alt.H + n0 + 4 * c;
            const h2 lo = {(_Float16)(sm[4 * c] * 0.25f), (_Float16)(sm[4 * c + 1] * 0.25f)};
            const h2 hi = {(_Float16)(sm[4 * c + 2] * 0.25f), (_Float16)(sm[4 * c + 3] * 0.25f)};
            *reinterpret_cast<uint2*>(mp) = uint2{h2_bits(lo), h2_bits(hi)};
        } else if (vec) {
            if constexpr (F32OUT) {
                float* yp = reinterpret_cast<float*>(Y) + (size_t)m * N + nb;
#pragma unroll
                for (int j = 0; j < CPT; j += 4) *reinterpret_cast<f4v*>(yp + j) = f4v{v[j], v[j + 1], v[j + 2], v[j + 3]};
            } else {
                _Float16* yp = reinterpret_cast<_Float16*>(Y) + (size_t)m * N + nb;
#pragma unroll
                for (int j = 0; j < CPT; j += 4) {
                    const h2 lo = {(_Float16)v[j], (_Float16)v[j + 1]}, hi = {(_Float16)v[j + 2], (_Float16)v[j + 3]};
                    *reinterpret_cast<uint2*>(yp + j) = uint2{h2_bits(lo), h2_bits(hi)};
                }
            }
        } else {
#pragma unroll
            for (int c = 0; c < CPT; ++c)
                if (nb + c < N) {
                    if constexpr (F32OUT) reinterpret_cast<float*>(Y)[(size_t)m * N + nb + c] = v[c];
                    else reinterpret_cast<_Float16*>(Y)[(size_t)m * N + nb + c] = (_Float16)v[c];
                }
        }
        if constexpr (ARGMAX) {
#pragma unroll
            for (int c = 0; c < CPT; ++c)
                if (nb + c < N && better(v[c], nb + c, bv, bi)) { bv = v[c]; bi = nb + c; }
        }
    }
    if constexpr (ARGMAX) {
        static_assert(TPR == 16 || TPR == 8 || TPR == 4, "threads per row");
        best_step<DPP_XOR1>(bv, bi);
        best_step<DPP_XOR2>(bv, bi);
        if constexpr (TPR >= 8) best_step<DPP_HALF_MIRROR>(bv, bi);
        if constexpr (TPR == 16) best_step<DPP_MIRROR>(bv, bi);
        if (threadIdx.x % TPR == 0 && m < M) {
            part_v[(size_t)m * gridDim.x + blockIdx.x] = bv;
            part_i[(size_t)m * gridDim.x + blockIdx.x] = bi;
        }
    }
}

template <int MT, int S, int WAVES, bool F32OUT, bool ARGMAX, int DEPTH, bool ALT, bool MIX = false>
hipError_t launch_one(dim3 grid, hipStream_t s, const uint8_t* c, const uint16_t* sc, const uint16_t* bi,
                      const _Float16* xh, int M, int N, int K, void* y, float* pv, int* pi, int kb_split,
                      const GemmAlt& alt) {
    using L = WaveLds<MT, S>;
    constexpr size_t red = (size_t)WAVES * 32 * MT * LDW * 4;    // one partial tile per wave
    constexpr size_t lds = (WAVES * L::BYTES > red) ? WAVES * L::BYTES : red;
    // more than 64 KiB of dynamic LDS must be allowed per function (and device) once
    static unsigned long long configured = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipGetLastError();
    const unsigned long long bit = 1ull << (dev & 63);
    if (!(__atomic_load_n(&configured, __ATOMIC_ACQUIRE) & bit)) {
        const hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&k_gemm_mfma<MT, S, WAVES, F32OUT, ARGMAX, DEPTH, ALT, MIX>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        __atomic_fetch_or(&configured, bit, __ATOMIC_RELEASE);
    }
    hipLaunchKernelGGL((k_gemm_mfma<MT, S, WAVES, F32OUT, ARGMAX, DEPTH, ALT, MIX>), grid, dim3(64 * WAVES), lds, s, c, sc, bi, xh, M,
                       N, K, y, pv, pi, kb_split, alt);
    return hipGetLastError();
}

template <int MT, int S, int WAVES, int DEPTH = 2>
hipError_t launch_mt(bool f32, bool am, dim3 grid, hipStream_t s, const dhp_int4* w, const void* x,
                     int M, void* y, float* pv, int* pi, int kb_split, const GemmAlt& alt = GemmAlt{nullptr, nullptr, nullptr, nullptr, 0, 1 << 30, nullptr, nullptr, 0}) {
    const auto* c = static_cast<const uint8_t*>(w->codes);
    const auto* sc = static_cast<const uint16_t*>(w->scales);
    const auto* bi = static_cast<const uint16_t*>(w->biases);
    const auto* xh = static_cast<const _Float16*>(x);
    const int N = w->rows, K = w->cols;
    // the second weight only in split-K launches (fp32 partials, no argmax)
    if (alt.codes) return launch_one<MT, S, WAVES, true, false, DEPTH, true>(grid, s, c, sc, bi, xh, M, N, K, y, pv, pi, kb_split, alt);
    if (f32 && am) return launch_one<MT, S, WAVES, true, true, DEPTH, false>(grid, s, c, sc, bi, xh, M, N, K, y, pv, pi, kb_split, alt);
    if (am) return launch_one<MT, S, WAVES, false, true, DEPTH, false>(grid, s, c, sc, bi, xh, M, N, K, y, pv, pi, kb_split, alt);
    if (f32) return launch_one<MT, S, WAVES, true, false, DEPTH, false>(grid, s, c, sc, bi, xh, M, N, K, y, pv, pi, kb_split, alt);
    return launch_one<MT, S, WAVES, false, false, DEPTH, false>(grid, s, c, sc, bi, xh, M, N, K, y, pv, pi, kb_split, alt);
}

}  // namespace

// Argmax partial count of the MFMA path for N output columns.
int dhp_gemm_blocks_n(int N) { return (N + BN - 1) / BN; }

int launch_gemm_mfma(const dhp_int4* w, const void* x, int M, void* y, int y_f32, int32_t* argmax,
                     void* ws, size_t ws_part_stride, hipStream_t s) {
    const int N = w->rows;
    const int MT = (M <= 32) ? 1 : 2;
    const int rows = 32 * MT;
    const dim3 grid((unsigned)dhp_gemm_blocks_n(N), (unsigned)((M + rows - 1) / rows));
    float* pv = argmax ? static_cast<float*>(ws) : nullptr;
    int* pi = argmax ? reinterpret_cast<int*>(static_cast<char*>(ws) + ws_part_stride) : nullptr;
    if (argmax && grid.y != 1) return dhp_fail(DHP_ERR_UNSUPPORTED, "argmax with m=%d", M);
    // 64-k stages. Up to 32 rows: eight waves, two stages in flight each. 64-row tiles: one stage
    // in flight per wave, with eight waves when K has at least 16 k-blocks and four otherwise.
    // Measured for M=128, N=8192, K=2560: 14.2 us (eight waves, one stage in flight) against
    // 16.2 (four, two) and 16.7 (eight, two: ~160 KB in flight per CU); for the hyper-connection
    // chunk, whose up projection has K = 320 (five k-blocks), four waves are faster.
    const bool am = argmax != nullptr;
    const int KB = w->cols / 64;
    const hipError_t e = (MT == 1) ? launch_mt<1, 1, 8>(y_f32, am, grid, s, w, x, M, y, pv, pi, KB)
                 : (KB >= 16) ? launch_mt<2, 1, 8, 1>(y_f32, am, grid, s, w, x, M, y, pv, pi, KB)
                              : launch_mt<2, 1, 4, 1>(y_f32, am, grid, s, w, x, M, y, pv, pi, KB);
    if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "gemm launch: %s", hipGetErrorString(e));
    if (argmax) {
        const hipError_t e2 = launch_argmax_final(pv, pi, (int)grid.x, M, argmax, s);
        if (e2 != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "argmax launch: %s", hipGetErrorString(e2));
    }
    return DHP_OK;
}

// Split-K form for long, narrow contractions (few output columns, many k): `splits` blocks share
// the K of every output tile, each writing its fp32 partial to y + split * M * N; the caller sums
// the `splits` partials in split order. The K / 64 k-blocks must divide evenly into the splits.
// With w2 (same K and group), the same launch also computes x . w2^T into y2_partials (its own
// N2 columns, laid out the same way): its column blocks follow w's in the grid.
int launch_gemm_mfma_splitk(const dhp_int4* w, const void* x, int M, float* y_partials, int splits, hipStream_t s,
                            const dhp_int4* w2, float* y2_partials) {
    const int N = w->rows, KB = w->cols / 64;
    if (splits < 1 || KB % splits) return dhp_fail(DHP_ERR_UNSUPPORTED, "%d k-blocks in %d splits", KB, splits);
    if (w2 && (w2->cols != w->cols || !y2_partials))
        return dhp_fail(DHP_ERR_UNSUPPORTED, "second split-K weight: K %d against %d", w2->cols, w->cols);
    const int MT = (M <= 32) ? 1 : 2;
    const int rows = 32 * MT;
    const int kb_split = KB / splits;
    const int nb = dhp_gemm_blocks_n(N);
    GemmAlt alt{nullptr, nullptr, nullptr, nullptr, 0, 1 << 30, nullptr, nullptr, 0};
    if (w2) alt = GemmAlt{static_cast<const uint8_t*>(w2->codes), static_cast<const uint16_t*>(w2->scales),
                          static_cast<const uint16_t*>(w2->biases), y2_partials, w2->rows, nb, nullptr, nullptr, 0};
    const int nbx = nb + (w2 ? dhp_gemm_blocks_n(w2->rows) : 0);
    const dim3 grid((unsigned)nbx, (unsigned)((M + rows - 1) / rows), (unsigned)splits);
    const hipError_t e = (MT == 1) ? launch_mt<1, 1, 8>(true, false, grid, s, w, x, M, y_partials, nullptr, nullptr, kb_split, alt)
                   : (kb_split >= 16) ? launch_mt<2, 1, 8, 1>(true, false, grid, s, w, x, M, y_partials, nullptr, nullptr, kb_split, alt)
                                      : launch_mt<2, 1, 4, 1>(true, false, grid, s, w, x, M, y_partials, nullptr, nullptr, kb_split, alt);
    if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "split-K gemm launch: %s", hipGetErrorString(e));
    return DHP_OK;
}

// The up projection of a chunked hyper-connection read with its stream mix fused into the
// epilogue (4 streams of H positions; the fp32 up result is never stored):
// mixed[m][h] = (1/4) sum_c sigmoid((x . w^T)[m][c*H + h]) * normed[m][c*H + h]. Only for the
// configuration whose epilogue gives each row's four streams to four adjacent threads: 64-row
// tiles (m > 32) on four waves (K / 64 < 16); dhp_gemm_upmix_fits says when.
bool dhp_gemm_upmix_fits(const dhp_int4* w, int M, int C, int H) {
    return C == 4 && M > 32 && M <= 128 && w->cols / 64 < 16 && H % 16 == 0 && w->rows == 4 * H;
}

int launch_gemm_mfma_upmix(const dhp_int4* w, const void* x, int M, const void* normed, void* mixed, int H,
                           hipStream_t s) {
    const dim3 grid((unsigned)(H / 16), (unsigned)((M + 63) / 64));
    const GemmAlt alt{nullptr, nullptr, nullptr, nullptr, 0, 1 << 30, static_cast<const _Float16*>(normed),
                      static_cast<_Float16*>(mixed), H};
    const int KB = w->cols / 64;
    const hipError_t e = launch_one<2, 1, 4, true, false, 1, false, true>(
        grid, s, static_cast<const uint8_t*>(w->codes), static_cast<const uint16_t*>(w->scales),
        static_cast<const uint16_t*>(w->biases), static_cast<const _Float16*>(x), M, w->rows, w->cols, nullptr, nullptr,
        nullptr, KB, alt);
    if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "up+mix gemm launch: %s", hipGetErrorString(e));
    return DHP_OK;
}
