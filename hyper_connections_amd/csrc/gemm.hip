// Multi-row INT4-affine dequantizing GEMM on the matrix cores: the batched chunked-prefill
// projection (m <= 128) and the multi-row arm of the GEMV (m <= 16, e.g. the LM head over
// several rows, with argmax).
//
// "src/real_forward.rs" (turbospark-runtime 0.3.0), fields batched_gemv_prefill and
// prefill_steel: resident GEMVs of a prefill micro-batch run as one M-row GEMM. The pages'
// Metal kernels (per-thread accumulator arrays; a simdgroup-matrix variant) are prior art;
// this is a gfx950 design around v_mfma_f32_32x32x16_f16:
//
//  * The weight tile is the B operand. Lane l of a wave owns weight row n0 + (l % 32) and a
//    32-wide k slice (l / 32 picks the half of a 64-k block): one 16-byte load holds its codes
//    for four MFMA steps, and the group's scale and bias are one load each. Codes become fp16
//    q*s + b in registers (the nibble trick of unpack8, then one packed fma): there is no LDS
//    staging of weights at all.
//  * The activation tile is the A operand, read from global memory with the same permutation
//    of k inside each group of eight that the nibble unpack produces, so both operands agree
//    on which k each register slot holds.
//  * A block owns a 32*MT x 64 output tile. Its four waves split K (64-k blocks w, w+4, ...),
//    each keeping the whole tile in accumulators; the four partial tiles are summed through
//    LDS in a fixed order (3, 2, 1, 0), so results are deterministic.
//  * The epilogue writes fp16 or fp32 and, for the GEMV arm, a per-block argmax partial per
//    row, reduced by the same small final kernel the M=1 path uses.
#include "dhp_internal.hpp"

#include <math.h>
#include <limits.h>

typedef float f16x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int BN = 64;         // output columns (weight rows) per block
constexpr int LDW = BN + 4;    // LDS row pitch in floats

DHP_DEV h8 dequant8(uint32_t w, h2 s2, h2 b2) {
    h2 q[4];
    unpack8(w, q);
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

template <int MT, bool F32OUT, bool ARGMAX>
__global__ __launch_bounds__(256) void k_gemm_mfma(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, const _Float16* __restrict__ X, int M, int N, int K,
    void* __restrict__ Y, float* __restrict__ part_v, int* __restrict__ part_i) {
    constexpr int ROWS = 32 * MT;
    __shared__ float tile[ROWS * LDW];

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int li = lane & 31;
    const int g = lane >> 5;
    const int n0 = blockIdx.x * BN;
    const int m0 = blockIdx.y * ROWS;
    const int KB = K >> 6;
    const size_t row_bytes = (size_t)K >> 1;

    // this lane's weight rows and activation rows (clamped reads, zero operands when out of range)
    bool nv[2];
    const uint8_t* crow[2];
    const uint16_t* srow[2];
    const uint16_t* brow[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int n = n0 + 32 * nt + li;
        nv[nt] = n < N;
        const int nc = nv[nt] ? n : 0;
        crow[nt] = codes + (size_t)nc * row_bytes + 16 * g;
        srow[nt] = scales + (size_t)nc * KB;
        brow[nt] = biases + (size_t)nc * KB;
    }
    bool mv[MT];
    const _Float16* xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = m0 + 32 * mt + li;
        mv[mt] = m < M;
        xrow[mt] = X + (size_t)(mv[mt] ? m : 0) * K + 32 * g;
    }

    f16x16 acc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f16x16{};

    for (int kb = wave; kb < KB; kb += 4) {
        u32x4 cw[2];
        uint32_t sw[2], bw[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            cw[nt] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(crow[nt] + (size_t)kb * 32));
            sw[nt] = srow[nt][kb];
            bw[nt] = brow[nt][kb];
        }
        u32x4 xw[MT][4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const u32x4* xp = reinterpret_cast<const u32x4*>(xrow[mt] + (size_t)kb * 64);
#pragma unroll
            for (int s = 0; s < 4; ++s) xw[mt][s] = xp[s];
        }
        h8 b[2][4];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const _Float16 s16 = (_Float16)bf16_to_f32(sw[nt]);
            const _Float16 b16 = (_Float16)bf16_to_f32(bw[nt]);
            const h2 s2 = {s16, s16}, b2 = {b16, b16};
            const uint32_t ww[4] = {cw[nt].x, cw[nt].y, cw[nt].z, cw[nt].w};
#pragma unroll
            for (int s = 0; s < 4; ++s) b[nt][s] = nv[nt] ? dequant8(ww[s], s2, b2) : h8{};
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const h8 a = mv[mt] ? permute_x8(xw[mt][s]) : h8{};
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b[nt][s], acc[mt][nt], 0, 0, 0);
            }
        }
    }

    // fixed-order reduction of the four K slices: wave 3, then 2, 1, 0
#pragma unroll
    for (int w = 3; w >= 0; --w) {
        if (wave == w) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int i = 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);
                        const int j = 32 * nt + li;
                        float* p = &tile[i * LDW + j];
                        *p = (w == 3) ? acc[mt][nt][r] : *p + acc[mt][nt][r];
                    }
        }
        __syncthreads();
    }

    // epilogue: 256 threads over ROWS x 64 outputs; TPR threads per row, contiguous columns
    constexpr int TPR = 256 / ROWS;
    constexpr int CPT = BN / TPR;
    const int row = threadIdx.x / TPR;
    const int c0 = (threadIdx.x % TPR) * CPT;
    const int m = m0 + row;
    float bv = -INFINITY;
    int bi = INT_MAX;
    if (m < M) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int n = n0 + c0 + c;
            if (n < N) {
                const float v = tile[row * LDW + c0 + c];
                if constexpr (F32OUT) reinterpret_cast<float*>(Y)[(size_t)m * N + n] = v;
                else reinterpret_cast<_Float16*>(Y)[(size_t)m * N + n] = (_Float16)v;
                if constexpr (ARGMAX)
                    if (better(v, n, bv, bi)) { bv = v; bi = n; }
            }
        }
    }
    if constexpr (ARGMAX) {
        static_assert(TPR == 8 || TPR == 4, "threads per row");
        best_step<DPP_XOR1>(bv, bi);
        best_step<DPP_XOR2>(bv, bi);
        if constexpr (TPR == 8) best_step<DPP_HALF_MIRROR>(bv, bi);
        if (threadIdx.x % TPR == 0 && m < M) {
            part_v[(size_t)m * gridDim.x + blockIdx.x] = bv;
            part_i[(size_t)m * gridDim.x + blockIdx.x] = bi;
        }
    }
}

template <int MT>
hipError_t launch_mt(bool f32, bool am, dim3 grid, hipStream_t s, const dhp_int4* w, const void* x,
                     int M, void* y, float* pv, int* pi) {
    const auto* c = static_cast<const uint8_t*>(w->codes);
    const auto* sc = static_cast<const uint16_t*>(w->scales);
    const auto* bi = static_cast<const uint16_t*>(w->biases);
    const auto* xh = static_cast<const _Float16*>(x);
    const int N = w->rows, K = w->cols;
    if (f32 && am) hipLaunchKernelGGL((k_gemm_mfma<MT, true, true>), grid, dim3(256), 0, s, c, sc, bi, xh, M, N, K, y, pv, pi);
    else if (f32) hipLaunchKernelGGL((k_gemm_mfma<MT, true, false>), grid, dim3(256), 0, s, c, sc, bi, xh, M, N, K, y, pv, pi);
    else if (am) hipLaunchKernelGGL((k_gemm_mfma<MT, false, true>), grid, dim3(256), 0, s, c, sc, bi, xh, M, N, K, y, pv, pi);
    else hipLaunchKernelGGL((k_gemm_mfma<MT, false, false>), grid, dim3(256), 0, s, c, sc, bi, xh, M, N, K, y, pv, pi);
    return hipGetLastError();
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
    const hipError_t e = (MT == 1) ? launch_mt<1>(y_f32, argmax != nullptr, grid, s, w, x, M, y, pv, pi)
                                   : launch_mt<2>(y_f32, argmax != nullptr, grid, s, w, x, M, y, pv, pi);
    if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "gemm launch: %s", hipGetErrorString(e));
    if (argmax) {
        const hipError_t e2 = launch_argmax_final(pv, pi, (int)grid.x, M, argmax, s);
        if (e2 != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "argmax launch: %s", hipGetErrorString(e2));
    }
    return DHP_OK;
}
