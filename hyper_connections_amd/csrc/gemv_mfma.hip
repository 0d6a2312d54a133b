// Multi-row arm of the dequantizing GEMV (2 <= m <= 16, e.g. the LM head over a few rows, with
// argmax), streamed like the M=1 GEMV but with the m-way reuse on the matrix cores.
//
// "src/real_forward.rs" (turbospark-runtime 0.3.0), field batched_gemv_prefill: the multi-row
// GEMM gives the same outputs as m separate GEMVs. Design for gfx950 (v_mfma_f32_16x16x32_f16):
//
//  * The activations (m <= 16 rows, K <= 2560) are staged once per block in LDS, with k permuted
//    inside every group of eight exactly as the nibble unpack orders the codes, so an A fragment
//    is one 16-byte LDS read with no shuffling. Lanes of fragment rows m..15 read the last real
//    row again: they only feed result rows that are never stored.
//  * Each wave streams 16-row weight tiles over the whole K with a grid stride. Lane (n, g) of a
//    wave (n = lane % 16, g = lane / 16) loads 16 bytes of weight row n0 + n covering
//    k = 128 c + 32 g .. +32; the four 32-bit words of that load are the B fragments of the four
//    MFMA steps of chunk c (virtual k of step t, slot e: 128 c + 32 g + 8 t + perm(e)). Four
//    lanes read 64 contiguous bytes of a row, the next chunk the following 64.
//  * The scales and biases of a 16-row tile are contiguous in memory (rows n0 .. n0+15), so a
//    wave fetches them with a few coalesced dword loads, converts each group's pair to fp16 once
//    and parks it in its own LDS slice as (s, s | b, b), from where every lane reads the pair of
//    its row and group with one 8-byte LDS read. Fetching them per chunk from 16 rows at a time
//    would cost one cache-line lookup per row per 2-byte load and starve the address unit.
//  * A tile is walked in parts of five chunks: the next part's codes are in flight while one
//    computes, and the next tile's first part (with its scales) while the last one computes.
//    Keeping more in flight per CU measured slower: HBM reads slow down past a few tens of KB
//    outstanding per CU.
//  * Each 16-lane row of the result is summed by the matrix core, so a tile needs no cross-lane
//    reduction; the argmax keeps, per lane, the best of its four rows over the tiles it saw, then
//    reduces over lanes (DPP), waves (LDS) and blocks (the shared final kernel).
#include "dhp_internal.hpp"

#include <math.h>
#include <limits.h>

typedef float f4x __attribute__((ext_vector_type(4)));

namespace {

constexpr int WAVES = 4;
constexpr int MAXCH = 20;            // 128-k chunks at the largest K (2560)
constexpr int PART = 5;              // chunks per part: a tile is walked in NPART parts
constexpr int NPART = MAXCH / PART;

DHP_DEV h8 deq8(uint32_t w, h2 s2, h2 b2, const NibConsts& k) {
    h2 q[4];
    unpack8(w, q, k);
    const h2 p0 = __builtin_elementwise_fma(q[0], s2, b2);
    const h2 p1 = __builtin_elementwise_fma(q[1], s2, b2);
    const h2 p2 = __builtin_elementwise_fma(q[2], s2, b2);
    const h2 p3 = __builtin_elementwise_fma(q[3], s2, b2);
    return h8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

constexpr int SB_DW = 5;            // dwords of scales (and of biases) a lane fetches per tile
constexpr int SB_PITCH = 2 * MAXCH + 1;     // LDS (s,s|b,b) entries per tile row (G <= 40, + 1 pad:
                                             // the 16 rows of one 8-byte read land on distinct banks)

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct PartRegs {
    u32x4 c[PART];
};

struct TileSB {
    uint32_t s[SB_DW], b[SB_DW];
};

// Loads of chunks [c0, c0 + PART) of weight row `row` for lane group g (chunks >= nch are
// clamped to the last chunk and never used).
DHP_DEV void load_part(PartRegs& r, const uint8_t* crow, int c0, int nch, int g) {
#pragma unroll
    for (int i = 0; i < PART; ++i) {
        const int c = min(c0 + i, nch - 1);
        r.c[i] = *reinterpret_cast<const u32x4*>(crow + (size_t)c * 64 + 16 * g);
    }
}

// The tile's scale and bias dwords (two bf16 groups each): tile dword i = lane + 64 j, clamped to
// the last dword of the arrays (a clamped dword only feeds columns >= N, which are not stored).
DHP_DEV void load_tile_sb(TileSB& t, const uint32_t* s32, const uint32_t* b32, size_t first, size_t last,
                          int lane) {
#pragma unroll
    for (int j = 0; j < SB_DW; ++j) {
        const size_t i = min(first + (size_t)(lane + 64 * j), last);
        t.s[j] = s32[i];
        t.b[j] = b32[i];
    }
}

// Park the tile's pairs in the wave's LDS slice: entry (row, group) = (s, s | b, b) as fp16.
DHP_DEV void store_tile_sb(const TileSB& t, uint32_t* sbl, int lane, int half_g, int dwords) {
#pragma unroll
    for (int j = 0; j < SB_DW; ++j) {
        const int i = lane + 64 * j;
        if (i < dwords) {
            const int row = i / half_g, grp = 2 * (i - row * half_g);
            const _Float16 s0 = (_Float16)bf16_to_f32(t.s[j] & 0xFFFFu);
            const _Float16 s1 = (_Float16)__builtin_bit_cast(float, t.s[j] & 0xFFFF0000u);
            const _Float16 b0 = (_Float16)bf16_to_f32(t.b[j] & 0xFFFFu);
            const _Float16 b1 = (_Float16)__builtin_bit_cast(float, t.b[j] & 0xFFFF0000u);
            u32x2* e = reinterpret_cast<u32x2*>(sbl + 2 * (row * SB_PITCH + grp));
            e[0] = u32x2{h2_bits(h2{s0, s0}), h2_bits(h2{b0, b0})};
            e[1] = u32x2{h2_bits(h2{s1, s1}), h2_bits(h2{b1, b1})};
        }
    }
}

DHP_DEV void mfma_part(const PartRegs& r, const uint8_t* xl, int xpitch, const uint32_t* sbrow, int c0, int nch,
                       int arow, int g, f4x& acc, const NibConsts& nk) {
#pragma unroll
    for (int i = 0; i < PART; ++i) {
        if (c0 + i < nch) {
            const u32x2 e = *reinterpret_cast<const u32x2*>(sbrow + 2 * (2 * (c0 + i) + (g >> 1)));
            const h2 s2 = as_h2(e.x), b2 = as_h2(e.y);
            const uint32_t ww[4] = {r.c[i].x, r.c[i].y, r.c[i].z, r.c[i].w};
            const uint8_t* ap = xl + arow * xpitch + ((c0 + i) * 128 + 32 * g) * 2;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const u32x4 av = *reinterpret_cast<const u32x4*>(ap + 16 * t);
                const h8 a = __builtin_bit_cast(h8, av);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, deq8(ww[t], s2, b2, nk), acc, 0, 0, 0);
            }
        }
    }
}

// NCHT: the number of 128-k chunks when fixed at compile time (K = 128 * NCHT; chunk offsets
// then become immediate load offsets and the per-chunk guards disappear), 0 for any K.
template <int NCHT, bool F32OUT, bool ARGMAX>
__global__ __launch_bounds__(WAVES * 64) void k_gemv_mfma16(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, const _Float16* __restrict__ X, int M, int N, int K,
    void* __restrict__ Y, float* __restrict__ part_v, int* __restrict__ part_i) {
    extern __shared__ __align__(16) uint8_t xl[];      // [M][K halves, permuted by eights] + pad
    if constexpr (NCHT != 0) K = NCHT * 128;
    const int xpitch = 2 * K + 16;
    // after the activations: one (s,s|b,b) slice of 16 x SB_PITCH entries per wave
    uint32_t* sbl = reinterpret_cast<uint32_t*>(xl + (size_t)M * xpitch) + (threadIdx.x >> 6) * (16 * SB_PITCH * 2);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int nch = K >> 7;                           // 128-k chunks
    const int G = K >> 6;
    const int half_g = G >> 1;                        // scale dwords per row
    const int tile_dw = 16 * half_g;                  // scale dwords per tile
    const size_t last_dw = (size_t)N * half_g - 1;
    const auto* s32 = reinterpret_cast<const uint32_t*>(scales);
    const auto* b32 = reinterpret_cast<const uint32_t*>(biases);
    const size_t row_bytes = (size_t)K >> 1;

    const NibConsts nk = nib_consts();
    float bv[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    int bi[4] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};
    const int ntiles = (N + 15) >> 4;
    const int stride = gridDim.x * WAVES;
    // A rows: lane n reads activation row n, clamped to the last real row (rows >= M only feed
    // result rows that are never stored)
    const int arow = min(n, M - 1);
    int tile = blockIdx.x * WAVES + wave;
    PartRegs buf[2];
    TileSB sb;
    if (tile < ntiles) {
        const int row = min(tile * 16 + n, N - 1);
        load_tile_sb(sb, s32, b32, (size_t)tile * tile_dw, last_dw, lane);
        load_part(buf[0], codes + (size_t)row * row_bytes, 0, nch, g);
    }

    // stage the activations, permuted (x0,x4,x1,x5,x2,x6,x3,x7) within each group of eight, while
    // the first tile's weights are in flight; every load of a pass is issued before the first
    // store (a load-then-store loop would pay one memory round trip per iteration)
    {
        constexpr int XB = 10;                         // 16-byte loads per thread per pass
        const int per_row = K >> 3;
        const int total = M * per_row;
        for (int base = 0; base < total; base += XB * WAVES * 64) {
            u32x4 u[XB];
#pragma unroll
            for (int k = 0; k < XB; ++k) {
                const int i = min(base + k * WAVES * 64 + (int)threadIdx.x, total - 1);
                const int m = i / per_row, j = i - m * per_row;
                u[k] = *reinterpret_cast<const u32x4*>(X + (size_t)m * K + 8 * j);
            }
#pragma unroll
            for (int k = 0; k < XB; ++k) {
                const int i = base + k * WAVES * 64 + (int)threadIdx.x;
                if (i < total) {
                    const int m = i / per_row, j = i - m * per_row;
                    h2 p[4];
                    permute8(u[k].x, u[k].y, u[k].z, u[k].w, p);
                    *reinterpret_cast<u32x4*>(xl + m * xpitch + 16 * j) =
                        u32x4{h2_bits(p[0]), h2_bits(p[1]), h2_bits(p[2]), h2_bits(p[3])};
                }
            }
        }
    }
    __syncthreads();
    const uint32_t* sbrow = sbl + 2 * n * SB_PITCH;
    // loads are unconditional (clamped rows and chunks) so the compiler can count them and wait
    // only for the data about to be used
    for (; tile < ntiles; tile += stride) {
        const int n0 = tile * 16;
        const int row = min(n0 + n, N - 1);
        f4x acc = {0.0f, 0.0f, 0.0f, 0.0f};
        // the previous tile's LDS reads were issued before these writes (one wave, in order)
        __builtin_amdgcn_wave_barrier();
        store_tile_sb(sb, sbl, lane, half_g, tile_dw);
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // the tile in NPART parts: one part is in flight while the previous one computes, and the
        // next tile's scales and first part while the last one computes. More in flight per CU
        // reads HBM slower (whole half tiles in flight measured 10-15 % slower).
        const int ntile = tile + stride;
        const int nrow = min(ntile * 16 + n, N - 1);
#pragma unroll
        for (int p = 0; p < NPART; ++p) {
            if (p + 1 < NPART) {
                load_part(buf[(p + 1) & 1], codes + (size_t)row * row_bytes, (p + 1) * PART, nch, g);
            } else {
                load_tile_sb(sb, s32, b32, min((size_t)ntile * tile_dw, last_dw), last_dw, lane);
                load_part(buf[(p + 1) & 1], codes + (size_t)nrow * row_bytes, 0, nch, g);
            }
            mfma_part(buf[p & 1], xl, xpitch, sbrow, p * PART, nch, arow, g, acc, nk);
        }
        // lane (n, g) holds rows 4 g .. 4 g + 3 of column n0 + n
        const int col = n0 + n;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * g + r;
            if (m < M && col < N) {
                const float v = acc[r];
                if constexpr (F32OUT) reinterpret_cast<float*>(Y)[(size_t)m * N + col] = v;
                else reinterpret_cast<_Float16*>(Y)[(size_t)m * N + col] = (_Float16)v;
                if constexpr (ARGMAX)
                    if (better(v, col, bv[r], bi[r])) { bv[r] = v; bi[r] = col; }
            }
        }
    }

    if constexpr (ARGMAX) {
        // over the 16 lanes of each row group (one DPP row), then over the waves of the block
        __shared__ float sv[WAVES][16];
        __shared__ int si[WAVES][16];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v = bv[r];
            int i = bi[r];
            best_step<DPP_XOR1>(v, i);
            best_step<DPP_XOR2>(v, i);
            best_step<DPP_HALF_MIRROR>(v, i);
            best_step<DPP_MIRROR>(v, i);
            if (n == 0) { sv[wave][4 * g + r] = v; si[wave][4 * g + r] = i; }
        }
        __syncthreads();
        if ((int)threadIdx.x < M) {
            const int m = threadIdx.x;
            float v = sv[0][m];
            int i = si[0][m];
            for (int w = 1; w < WAVES; ++w)
                if (better(sv[w][m], si[w][m], v, i)) { v = sv[w][m]; i = si[w][m]; }
            part_v[(size_t)m * gridDim.x + blockIdx.x] = v;
            part_i[(size_t)m * gridDim.x + blockIdx.x] = i;
        }
    }
}

}  // namespace

hipError_t launch_argmax_final(const float* pv, const int* pi, int nparts, int m, int32_t* out, hipStream_t s);

// Whether the streamed matrix-core arm takes this call (else the LDS-staged GEMM does): its scale
// and bias fetches are dword loads, so those arrays must be 4-byte aligned.
bool dhp_gemv_mfma16_fits(const dhp_int4* w, int M) {
    const int K = w->cols;
    return M >= 2 && M <= 16 && K % 128 == 0 && K <= MAXCH * 128 &&
           reinterpret_cast<uintptr_t>(w->scales) % 4 == 0 && reinterpret_cast<uintptr_t>(w->biases) % 4 == 0;
}

namespace {

template <int NCHT, bool F32OUT, bool ARGMAX>
hipError_t launch_variant(const dhp_int4* w, const void* x, int M, void* y, float* pv, int* pi, int dev, int cus,
                          hipStream_t s, int* blocks_out) {
    const int N = w->rows, K = w->cols;
    const size_t lds = (size_t)M * (2 * K + 16) + (size_t)WAVES * 16 * SB_PITCH * 8;
    const void* fn = reinterpret_cast<const void*>(&k_gemv_mfma16<NCHT, F32OUT, ARGMAX>);
    // more than 64 KiB of dynamic LDS must be allowed once per device; the occupancy (blocks per
    // CU, from registers and LDS) is cached per device and m
    static unsigned long long configured = 0;
    static int resident[64][17];
    if (!(__atomic_load_n(&configured, __ATOMIC_ACQUIRE) & (1ull << (dev & 63)))) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 16 * (2 * MAXCH * 128 + 16) + WAVES * 16 * SB_PITCH * 8);
        if (e != hipSuccess) return e;
        __atomic_fetch_or(&configured, 1ull << (dev & 63), __ATOMIC_RELEASE);
    }
    int per_cu = __atomic_load_n(&resident[dev & 63][M], __ATOMIC_RELAXED);
    if (per_cu == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, WAVES * 64, lds) != hipSuccess || per_cu < 1)
            per_cu = 1;
        __atomic_store_n(&resident[dev & 63][M], per_cu, __ATOMIC_RELAXED);
    }
    // one resident round of blocks: the waves stride over the tiles, so more blocks than fit
    // would only run as a tail
    const int ntiles = (N + 15) / 16;
    int blocks = (ntiles + WAVES - 1) / WAVES;
    if (blocks > per_cu * cus) blocks = per_cu * cus;
    *blocks_out = blocks;
    hipLaunchKernelGGL((k_gemv_mfma16<NCHT, F32OUT, ARGMAX>), dim3((unsigned)blocks), dim3(WAVES * 64), lds, s,
                       static_cast<const uint8_t*>(w->codes), static_cast<const uint16_t*>(w->scales),
                       static_cast<const uint16_t*>(w->biases), static_cast<const _Float16*>(x), M, N, K, y, pv, pi);
    return hipGetLastError();
}

template <int NCHT>
hipError_t launch_nch(const dhp_int4* w, const void* x, int M, void* y, int y_f32, bool am, float* pv, int* pi,
                      int dev, int cus, hipStream_t s, int* blocks) {
    if (y_f32 && am) return launch_variant<NCHT, true, true>(w, x, M, y, pv, pi, dev, cus, s, blocks);
    if (y_f32) return launch_variant<NCHT, true, false>(w, x, M, y, pv, pi, dev, cus, s, blocks);
    if (am) return launch_variant<NCHT, false, true>(w, x, M, y, pv, pi, dev, cus, s, blocks);
    return launch_variant<NCHT, false, false>(w, x, M, y, pv, pi, dev, cus, s, blocks);
}

}  // namespace

int launch_gemv_mfma16(const dhp_int4* w, const void* x, int M, void* y, int y_f32, int32_t* argmax, void* ws,
                       size_t ws_part_stride, hipStream_t s, int cus) {
    float* pv = argmax ? static_cast<float*>(ws) : nullptr;
    int* pi = argmax ? reinterpret_cast<int*>(static_cast<char*>(ws) + ws_part_stride) : nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "hipGetDevice");
    int blocks = 0;
    const bool am = argmax != nullptr;
    hipError_t e = (w->cols == MAXCH * 128)
                       ? launch_nch<MAXCH>(w, x, M, y, y_f32, am, pv, pi, dev, cus, s, &blocks)
                       : launch_nch<0>(w, x, M, y, y_f32, am, pv, pi, dev, cus, s, &blocks);
    if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "gemv_mfma16 launch: %s", hipGetErrorString(e));
    if (argmax) {
        e = launch_argmax_final(pv, pi, blocks, M, argmax, s);
        if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "argmax launch: %s", hipGetErrorString(e));
    }
    return DHP_OK;
}
