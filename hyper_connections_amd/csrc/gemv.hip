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
//    wave streams four rows at once.
//  * The activation slice a lane needs is the same for every row it visits, so it is
//    loaded once, rearranged into the pair order of the nibble unpack, and kept in
//    registers (K = 2560: 80 VGPRs). A block walks rows with a grid stride and keeps the
//    next row group's codes in flight while it computes the current one.
//  * Per 64-weight group the affine form is factored: s * sum(q*x) + b * sum(x); the
//    inner sum runs on v_dot2_f32_f16 over the codes in their offset fp16 form (see
//    unpack8_off), which carries a factor 16 through both halves; the finished row is
//    scaled by 1/16 (exact).
//  * The 16 partial sums of a row meet in a fixed butterfly, so a row's value does not
//    depend on which block, wave or lane group computed it: duplicated rows give equal
//    bits, which is what the argmax tie rule needs.
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

template <int CPL>
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
        r[i].c = __builtin_nontemporal_load(cr + ch);
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

// Register-resident activations: K = 16 * CPL * 32.
template <int CPL, bool F32OUT, bool ARGMAX>
__global__ __launch_bounds__(MAX_BLOCK) void k_gemv_m1_reg(
    const u32x4* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, const _Float16* __restrict__ x, void* __restrict__ y,
    int N, float* __restrict__ part_v, int* __restrict__ part_i) {
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
    // One register set: the compiler issues the next row group's loads (into fresh registers)
    // before computing the current one, so one group per wave is in flight. More in flight
    // (three sets) measured slower: past about 40 KB per CU the HBM read rate drops.
    RowRegs r[CPL];
    load_row<CPL>(codes, scales, biases, min(base + rw, N - 1), j, r);

    h2 xp[CPL][16];
    float xs[CPL], nc[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) xs[i] = load_x32_off(x + (size_t)(j + LPR * i) * 32, xp[i], nc[i]);

    const NibConsts nk = nib_consts();
    float best_v = -INFINITY;
    int best_i = INT_MAX;
    for (; base < N; base += stride) {
        const int row = base + rw;
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const float d = dot32_off(r[i].c, xp[i], nc[i], nk);
            acc = __builtin_fmaf(bf16_to_f32(r[i].s), d, acc);
            acc = __builtin_fmaf(bf16_to_f32(r[i].b), xs[i], acc);
        }
        acc = group_sum<LPR>(acc) * 0.0625f;
        if (j == 0 && row < N) {
            if constexpr (F32OUT) reinterpret_cast<float*>(y)[row] = acc;
            else reinterpret_cast<_Float16*>(y)[row] = (_Float16)acc;
            if constexpr (ARGMAX)
                if (better(acc, row, best_v, best_i)) { best_v = acc; best_i = row; }
        }
        load_row<CPL>(codes, scales, biases, min(base + stride + rw, N - 1), j, r);
    }
    block_argmax_write<ARGMAX>(best_v, best_i, j == 0, part_v, part_i);
}

// Any K (multiple of 64, <= 16384): activations staged once per block in LDS as permuted
// pairs plus per-chunk (16 sum, -1024 sum); lane j walks chunks j, j+16, ... of each row with
// the same operations, in the same order, as k_gemv_m1_reg.
template <bool F32OUT, bool ARGMAX>
__global__ __launch_bounds__(MAX_BLOCK) void k_gemv_m1_lds(
    const u32x4* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, const _Float16* __restrict__ x, void* __restrict__ y,
    int N, int K, float* __restrict__ part_v, int* __restrict__ part_i) {
    extern __shared__ u32x4 lds_x[];            // [CH][4] u32x4 = 16 permuted pairs per chunk
    const int CH = K / 32;
    const int G = K / 64;
    float2* lds_sum = reinterpret_cast<float2*>(lds_x + (size_t)CH * 4);
    for (int ch = threadIdx.x; ch < CH; ch += blockDim.x) {
        h2 p[16];
        float nc;
        const float xs = load_x32_off(x + (size_t)ch * 32, p, nc);
        lds_sum[ch] = float2{xs, nc};
        u32x4* dst = lds_x + (size_t)ch * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dst[i] = u32x4{h2_bits(p[4 * i]), h2_bits(p[4 * i + 1]), h2_bits(p[4 * i + 2]),
                           h2_bits(p[4 * i + 3])};
    }
    __syncthreads();

    const int t = threadIdx.x;
    const int j = t % LPR;
    const int rpb = blockDim.x / LPR;
    const NibConsts nk = nib_consts();
    float best_v = -INFINITY;
    int best_i = INT_MAX;
    // whole 16-lane groups share a row, so the DPP sum below sees only live lanes
    for (int row = blockIdx.x * rpb + t / LPR; row < N; row += gridDim.x * rpb) {
        const u32x4* cr = codes + (size_t)row * CH;
        const uint16_t* sr = scales + (size_t)row * G;
        const uint16_t* br = biases + (size_t)row * G;
        float acc = 0.0f;
        for (int ch = j; ch < CH; ch += LPR) {
            const u32x4 c = __builtin_nontemporal_load(cr + ch);
            h2 p[16];
            const u32x4* src = lds_x + (size_t)ch * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4 u = src[i];
                p[4 * i] = as_h2(u.x); p[4 * i + 1] = as_h2(u.y);
                p[4 * i + 2] = as_h2(u.z); p[4 * i + 3] = as_h2(u.w);
            }
            const float2 sn = lds_sum[ch];
            const float d = dot32_off(c, p, sn.y, nk);
            acc = __builtin_fmaf(bf16_to_f32(sr[ch >> 1]), d, acc);
            acc = __builtin_fmaf(bf16_to_f32(br[ch >> 1]), sn.x, acc);
        }
        acc = group_sum<LPR>(acc) * 0.0625f;
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

template <int CPL>
hipError_t launch_reg(bool f32, bool am, dim3 g, dim3 b, hipStream_t s, const u32x4* c,
                      const uint16_t* sc, const uint16_t* bi, const _Float16* x, void* y, int N,
                      float* pv, int* pi) {
    if (f32 && am) hipLaunchKernelGGL((k_gemv_m1_reg<CPL, true, true>), g, b, 0, s, c, sc, bi, x, y, N, pv, pi);
    else if (f32) hipLaunchKernelGGL((k_gemv_m1_reg<CPL, true, false>), g, b, 0, s, c, sc, bi, x, y, N, pv, pi);
    else if (am) hipLaunchKernelGGL((k_gemv_m1_reg<CPL, false, true>), g, b, 0, s, c, sc, bi, x, y, N, pv, pi);
    else hipLaunchKernelGGL((k_gemv_m1_reg<CPL, false, false>), g, b, 0, s, c, sc, bi, x, y, N, pv, pi);
    return hipGetLastError();
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
    const int rows_per_wave = 64 / LPR;
    const long waves = (N + rows_per_wave - 1) / rows_per_wave;
    int block = (waves < 4L * dev.cus) ? 64 : MAX_BLOCK;
    const int rpb = block / LPR;
    long blocks = (N + rpb - 1) / rpb;
    const long cap = (block == MAX_BLOCK) ? 2L * dev.cus : 16L * dev.cus;
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
        case 6: e = launch_reg<6>(y_f32, am, g, b, s, c, sc, bi, xh, y, N, pv, pi); break;
        case 8: e = launch_reg<8>(y_f32, am, g, b, s, c, sc, bi, xh, y, N, pv, pi); break;
        default: {
            const size_t lds = (size_t)CH * 64 + (size_t)CH * 8;
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
