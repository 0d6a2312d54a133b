// M=1 INT4-affine dequantizing GEMV (decode projections and the LM head) and the
// deterministic two-stage argmax over its fp32 outputs (per-block partials, then one small
// reduction kernel per output row).
//
// "src/real_forward.rs" (turbospark-runtime 0.3.0), module doc: dequant_int4_gemv_simd
// streams resident INT4-affine weights/scales/biases with nothing staged per dispatch.
// The Metal kernel's simdgroup layout is not followed here; this is a wave64 design:
//
//  * 16 lanes own one weight row. Lane j reads 16-byte code chunks j, j+16, j+32, ... of
//    the row, so one load instruction of a 16-lane group covers 256 contiguous bytes and a
//    wave streams four rows at once. Large matrices stream with the nontemporal hint (weights
//    that are read once, from HBM); small ones, whose launches are latency-bound, use ordinary
//    loads.
//  * Per 64-weight group the affine form is factored: s * sum(q*x) + b * sum(x). The group's
//    sum(q*x) is formed exactly on integers (the activations as three int8 pieces relative to
//    the group's largest magnitude, v_dot4_i32_i8 over the codes; see xg_stage_octet), so its
//    value does not depend on the order of the products. Lane j holds one of the group's two
//    chunks; the neighbouring lane holds the other, and one DPP exchange adds the halves.
//  * The activations' pieces are the same for every row: each block converts them once into
//    LDS (eight lanes per group) and, where K = 16 * CPL * 32 with CPL <= 5, every lane keeps
//    the pieces of its own chunks in registers. A block walks rows with a grid stride and
//    keeps the next row group's codes in flight while it computes the current one.
//  * Lanes 2j' and 2j'+1 run chain j' (j' = 0..7) over the groups j', j'+8, j'+16, ..., one fp32
//    step per group; the 8 chains of a row meet in a fixed butterfly, so a row's value does not
//    depend on which block, wave or lane group computed it: duplicated rows give equal bits,
//    which is what the argmax tie rule needs, and the multi-row kernel (gemv_rows.hip)
//    reproduces every row bit for bit.
#include "dhp_internal.hpp"

#include <math.h>
#include <limits.h>

namespace {

constexpr int LPR = 16;            // lanes per weight row
constexpr int MAX_BLOCK = 256;
constexpr int GEMV_MAX_BLOCKS = 4096;

struct RowRegs {
    u32x4 c;
    uint32_t s, b;
};

template <int CPL, bool NT>
DHP_DEV void load_row(const u32x4* __restrict__ codes, const uint16_t* __restrict__ scales,
                      const uint16_t* __restrict__ biases, int row, int j, RowRegs* r) {
    constexpr int CH = LPR * CPL;
    constexpr int G = CH / 2;
    const u32x4* cr = codes + (size_t)row * CH;
    const uint16_t* sr = scales + (size_t)row * G;
    const uint16_t* br = biases + (size_t)row * G;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int ch = j + LPR * i;
        r[i].c = NT ? __builtin_nontemporal_load(cr + ch) : cr[ch];
        r[i].s = sr[ch >> 1];
        r[i].b = br[ch >> 1];
    }
}

template <bool ARGMAX>
DHP_DEV void block_argmax_write(float bv, int bi, bool leader, float* part_v, int* part_i) {
    if constexpr (ARGMAX) {
        __shared__ float sv[MAX_BLOCK / LPR];
        __shared__ int si[MAX_BLOCK / LPR];
        const int g = threadIdx.x / LPR;
        if (leader) {
            sv[g] = bv;
            si[g] = bi;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            float v = sv[0];
            int i = si[0];
            const int ng = blockDim.x / LPR;
            for (int k = 1; k < ng; ++k)
                if (better(sv[k], si[k], v, i)) { v = sv[k]; i = si[k]; }
            part_v[blockIdx.x] = v;
            part_i[blockIdx.x] = i;
        }
    }
}

// Stage the activations' group pieces (XG_DW words per group) into LDS, eight lanes per group.
DHP_DEV void stage_x(const _Float16* __restrict__ x, int G, uint32_t* __restrict__ xs) {
    for (int it = threadIdx.x; it < 8 * G; it += blockDim.x) {
        const int i = it & 7;
        uint32_t* dst = xs + (size_t)(it >> 3) * XG_DW;
        const float2 sp = xg_stage_octet(x + (size_t)(it >> 3) * 64, i, dst + 4 * (i & 3) + 2 * (i >> 2), 16);
        if (i == 0) *reinterpret_cast<float2*>(dst + 48) = sp;
    }
    __syncthreads();
}

// The 24 piece words and the (sum, power of two) pair of chunk ch from the staged groups.
DHP_DEV void load_chunk_pieces(const uint32_t* __restrict__ xs, int ch, uint32_t (&xq)[24], float2& sp) {
    const uint32_t* src = xs + (size_t)(ch >> 1) * XG_DW + 2 * (ch & 1);
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint2 v = *reinterpret_cast<const uint2*>(src + 16 * p + 4 * w);
            xq[8 * p + 2 * w] = v.x;
            xq[8 * p + 2 * w + 1] = v.y;
        }
    sp = *reinterpret_cast<const float2*>(xs + (size_t)(ch >> 1) * XG_DW + 48);
}

// The group's exact sum from this lane's chunk and its neighbour's (lanes 2j', 2j'+1 hold the
// group's two chunks), then the group's chain step; both lanes of the pair end with equal bits.
DHP_DEV float group_step(float acc, int d_chunk, uint32_t s16, uint32_t b16, float2 sp) {
    const int d = d_chunk + dpp_i<DPP_XOR1>(d_chunk);
    return xg_group_acc(acc, d, bf16_to_f32(s16), bf16_to_f32(b16), sp.x, sp.y);
}

// Register-resident activation pieces: K = 16 * CPL * 32.
template <int CPL, bool F32OUT, bool ARGMAX, bool NT>
__global__ __launch_bounds__(MAX_BLOCK) void k_gemv_m1_reg(
    const u32x4* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, const _Float16* __restrict__ x, void* __restrict__ y,
    int N, float* __restrict__ part_v, int* __restrict__ part_i) {
    __shared__ __align__(16) uint32_t xs[LPR * CPL / 2 * XG_DW];
    const int t = threadIdx.x;
    const int j = t % LPR;
    const int rpb = blockDim.x / LPR;
    const int stride = gridDim.x * rpb;
    // A wave owns four consecutive rows per step. Control flow follows the wave's first row, so
    // every lane runs the same iterations and the loads stay unconditional (rows past N are
    // clamped to the last row and their results are not stored). A guard around a load would
    // make the compiler wait for every load in flight at the first use of any of them.
    const int rw = (t & 63) / LPR;
    int base = __builtin_amdgcn_readfirstlane(blockIdx.x * rpb + (t >> 6) * (64 / LPR));
    // The compiler issues the next row group's loads (into fresh registers) before computing the
    // current one; large matrices keep a second register set (below).
    RowRegs r[CPL];
    load_row<CPL, NT>(codes, scales, biases, min(base + rw, N - 1), j, r);

    // the first codes are in flight while the block converts the activations
    stage_x(x, LPR * CPL / 2, xs);
    uint32_t xq[CPL][24];
    float2 sp[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) load_chunk_pieces(xs, j + LPR * i, xq[i], sp[i]);

    float best_v = -INFINITY;
    int best_i = INT_MAX;
    auto one = [&](const RowRegs (&rr)[CPL], int b) {
        const int row = b + rw;
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) acc = group_step(acc, dot32_i8(rr[i].c, xq[i]), rr[i].s, rr[i].b, sp[i]);
        acc = group_sum<LPR, 2>(acc);
        if (j == 0 && row < N) {
            if constexpr (F32OUT) reinterpret_cast<float*>(y)[row] = acc;
            else reinterpret_cast<_Float16*>(y)[row] = (_Float16)acc;
            if constexpr (ARGMAX)
                if (better(acc, row, best_v, best_i)) { best_v = acc; best_i = row; }
        }
    };
    if constexpr (NT) {
        // large matrices: two row groups in flight per wave (a second register set), one computing
        // while the other loads (39.8 against 40.8 us for the LM head with a cold last-level cache)
        RowRegs r2[CPL];
        load_row<CPL, NT>(codes, scales, biases, min(base + stride + rw, N - 1), j, r2);
        for (; base < N; base += 2 * stride) {
            one(r, base);
            load_row<CPL, NT>(codes, scales, biases, min(base + 2 * stride + rw, N - 1), j, r);
            if (base + stride < N) one(r2, base + stride);      // uniform over the wave
            load_row<CPL, NT>(codes, scales, biases, min(base + 3 * stride + rw, N - 1), j, r2);
        }
    } else {
        for (; base < N; base += stride) {
            one(r, base);
            load_row<CPL, NT>(codes, scales, biases, min(base + stride + rw, N - 1), j, r);
        }
    }
    block_argmax_write<ARGMAX>(best_v, best_i, j == 0, part_v, part_i);
}

// Any K (multiple of 64, <= 16384): the activations' pieces stay in LDS; lane j walks chunks
// j, j+16, ... of each row with the same operations, in the same order, as k_gemv_m1_reg (the
// two lanes of a pair always hold the two chunks of one group: K is a multiple of 64).
template <bool F32OUT, bool ARGMAX>
__global__ __launch_bounds__(MAX_BLOCK) void k_gemv_m1_lds(
    const u32x4* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, const _Float16* __restrict__ x, void* __restrict__ y,
    int N, int K, float* __restrict__ part_v, int* __restrict__ part_i) {
    extern __shared__ __align__(16) uint32_t xs_dyn[];      // [G][XG_DW]
    const int CH = K / 32;
    const int G = K / 64;
    stage_x(x, G, xs_dyn);

    const int t = threadIdx.x;
    const int j = t % LPR;
    const int rpb = blockDim.x / LPR;
    float best_v = -INFINITY;
    int best_i = INT_MAX;
    // whole 16-lane groups share a row, so the DPP sums below see only live lanes
    for (int row = blockIdx.x * rpb + t / LPR; row < N; row += gridDim.x * rpb) {
        const u32x4* cr = codes + (size_t)row * CH;
        const uint16_t* sr = scales + (size_t)row * G;
        const uint16_t* br = biases + (size_t)row * G;
        float acc = 0.0f;
        for (int ch = j; ch < CH; ch += LPR) {
            const u32x4 c = cr[ch];
            uint32_t xq[24];
            float2 sp;
            load_chunk_pieces(xs_dyn, ch, xq, sp);
            acc = group_step(acc, dot32_i8(c, xq), sr[ch >> 1], br[ch >> 1], sp);
        }
        acc = group_sum<LPR, 2>(acc);
        if (j == 0) {
            if constexpr (F32OUT) reinterpret_cast<float*>(y)[row] = acc;
            else reinterpret_cast<_Float16*>(y)[row] = (_Float16)acc;
            if constexpr (ARGMAX)
                if (better(acc, row, best_v, best_i)) { best_v = acc; best_i = row; }
        }
    }
    block_argmax_write<ARGMAX>(best_v, best_i, j == 0, part_v, part_i);
}

// Second argmax stage: one block per output row reduces that row's block partials.
__global__ __launch_bounds__(256) void k_argmax_final(const float* __restrict__ part_v,
                                                      const int* __restrict__ part_i, int nparts,
                                                      int32_t* __restrict__ out) {
    const float* pv = part_v + (size_t)blockIdx.x * nparts;
    const int* pi = part_i + (size_t)blockIdx.x * nparts;
    float bv = -INFINITY;
    int bi = INT_MAX;
    // up to 4 partials per thread are loaded together (one round trip); more take further passes
    constexpr int U = 4;
    for (int base = 0; base < nparts; base += U * (int)blockDim.x) {
        float v[U];
        int ix[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = min(base + u * (int)blockDim.x + (int)threadIdx.x, nparts - 1);
            v[u] = pv[i];
            ix[u] = pi[i];
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (base + u * (int)blockDim.x + (int)threadIdx.x < nparts && better(v[u], ix[u], bv, bi)) {
                bv = v[u];
                bi = ix[u];
            }
    }
    wave_best(bv, bi);
    __shared__ float sv[4];
    __shared__ int si[4];
    if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = bv; si[threadIdx.x >> 6] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < (int)(blockDim.x >> 6); ++w)
            if (better(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
        out[blockIdx.x] = bi;
    }
}

template <int CPL, bool NT>
hipError_t launch_reg_nt(bool f32, bool am, dim3 g, dim3 b, hipStream_t s, const u32x4* c,
                         const uint16_t* sc, const uint16_t* bi, const _Float16* x, void* y, int N,
                         float* pv, int* pi) {
    if (f32 && am) hipLaunchKernelGGL((k_gemv_m1_reg<CPL, true, true, NT>), g, b, 0, s, c, sc, bi, x, y, N, pv, pi);
    else if (f32) hipLaunchKernelGGL((k_gemv_m1_reg<CPL, true, false, NT>), g, b, 0, s, c, sc, bi, x, y, N, pv, pi);
    else if (am) hipLaunchKernelGGL((k_gemv_m1_reg<CPL, false, true, NT>), g, b, 0, s, c, sc, bi, x, y, N, pv, pi);
    else hipLaunchKernelGGL((k_gemv_m1_reg<CPL, false, false, NT>), g, b, 0, s, c, sc, bi, x, y, N, pv, pi);
    return hipGetLastError();
}

// Rows from which the weights stream with the nontemporal hint: measured with a cold last-level
// cache, the LM head (151936 rows) took 40.6 us with it and 43.4 without, the 2560-row GEMV
// 5.7 us with it and 5.0 without.
constexpr int NT_MIN_ROWS = 16384;

template <int CPL>
hipError_t launch_reg(bool f32, bool am, dim3 g, dim3 b, hipStream_t s, const u32x4* c,
                      const uint16_t* sc, const uint16_t* bi, const _Float16* x, void* y, int N,
                      float* pv, int* pi) {
    if (N >= NT_MIN_ROWS) return launch_reg_nt<CPL, true>(f32, am, g, b, s, c, sc, bi, x, y, N, pv, pi);
    return launch_reg_nt<CPL, false>(f32, am, g, b, s, c, sc, bi, x, y, N, pv, pi);
}

}  // namespace

int dhp_gemm_blocks_n(int N);

// Bytes of the fp32 half of the argmax partials: [m][parts] values, then [m][parts] indices.
size_t dhp_argmax_part_stride(int32_t n_rows, int32_t m) {
    int parts = dhp_gemm_blocks_n(n_rows);
    if (parts < GEMV_MAX_BLOCKS) parts = GEMV_MAX_BLOCKS;
    return (size_t)parts * (size_t)m * sizeof(float);
}

size_t dhp_gemv_argmax_ws(int32_t n_rows, int32_t m) { return 2 * dhp_argmax_part_stride(n_rows, m); }

hipError_t launch_argmax_final(const float* pv, const int* pi, int nparts, int m, int32_t* out, hipStream_t s) {
    hipLaunchKernelGGL(k_argmax_final, dim3((unsigned)m), dim3(256), 0, s, pv, pi, nparts, out);
    return hipGetLastError();
}

int launch_gemv_m1(const dhp_int4* w, const void* x, void* y, int y_f32, int32_t* argmax,
                   void* ws, hipStream_t s, const DeviceFacts& dev) {
    const int N = w->rows, K = w->cols;
    const int CH = K / 32;
    const bool am = argmax != nullptr;
    const auto* c = static_cast<const u32x4*>(w->codes);
    const auto* sc = static_cast<const uint16_t*>(w->scales);
    const auto* bi = static_cast<const uint16_t*>(w->biases);
    const auto* xh = static_cast<const _Float16*>(x);

    // Small problems spread over more, narrower blocks; large ones run a grid stride over
    // a few resident blocks per compute unit.
    // Blocks of four waves (every block converts the activations once, so one-wave blocks
    // would repeat that work for every four rows); at most two resident per compute unit.
    const int block = MAX_BLOCK;
    const int rpb = block / LPR;
    long blocks = (N + rpb - 1) / rpb;
    const long cap = 2L * dev.cus;
    if (blocks > cap) blocks = cap;
    if (blocks > GEMV_MAX_BLOCKS) blocks = GEMV_MAX_BLOCKS;
    // the fewest blocks that still take the same number of grid-stride steps: every block then
    // works in every step, and the last step has no idle half of the grid
    {
        const long groups = (N + rpb - 1) / rpb;
        const long steps = (groups + blocks - 1) / blocks;
        blocks = (groups + steps - 1) / steps;
    }
    const int nparts = (int)blocks;

    float* pv = am ? static_cast<float*>(ws) : nullptr;
    int* pi = am ? reinterpret_cast<int*>(static_cast<char*>(ws) + dhp_argmax_part_stride(N, 1)) : nullptr;

    hipError_t e = hipSuccess;
    dim3 g((unsigned)blocks), b((unsigned)block);
    const int cpl = (CH % LPR == 0) ? CH / LPR : 0;
    switch (cpl) {
        case 1: e = launch_reg<1>(y_f32, am, g, b, s, c, sc, bi, xh, y, N, pv, pi); break;
        case 2: e = launch_reg<2>(y_f32, am, g, b, s, c, sc, bi, xh, y, N, pv, pi); break;
        case 3: e = launch_reg<3>(y_f32, am, g, b, s, c, sc, bi, xh, y, N, pv, pi); break;
        case 4: e = launch_reg<4>(y_f32, am, g, b, s, c, sc, bi, xh, y, N, pv, pi); break;
        case 5: e = launch_reg<5>(y_f32, am, g, b, s, c, sc, bi, xh, y, N, pv, pi); break;
        default: {
            const size_t lds = (size_t)(CH / 2) * XG_DW * 4;
            if (y_f32 && am) hipLaunchKernelGGL((k_gemv_m1_lds<true, true>), g, b, lds, s, c, sc, bi, xh, y, N, K, pv, pi);
            else if (y_f32) hipLaunchKernelGGL((k_gemv_m1_lds<true, false>), g, b, lds, s, c, sc, bi, xh, y, N, K, pv, pi);
            else if (am) hipLaunchKernelGGL((k_gemv_m1_lds<false, true>), g, b, lds, s, c, sc, bi, xh, y, N, K, pv, pi);
            else hipLaunchKernelGGL((k_gemv_m1_lds<false, false>), g, b, lds, s, c, sc, bi, xh, y, N, K, pv, pi);
            e = hipGetLastError();
        }
    }
    if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "gemv launch: %s", hipGetErrorString(e));
    if (am) {
        e = launch_argmax_final(pv, pi, nparts, 1, argmax, s);
        if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "argmax launch: %s", hipGetErrorString(e));
    }
    return DHP_OK;
}
