// Multi-row INT4-affine GEMV (2 <= m <= 16 rows of activations) that gives every output exactly
// the bits the M=1 GEMV gives for that row alone.
//
// "src/real_forward.rs" (turbospark-runtime 0.3.0), field batched_gemv_prefill: the batched
// GEMV kernel and the per-row GEMV agree bit for bit (only the matrix-instruction variant, a
// separate option, differs). The M=1 kernels (gemv.hip) fix each output's arithmetic: 16 lanes
// ("virtual lanes" j = 0..15) each run a chain over the 32-code chunks j, j+16, j+32, ... of the
// row, d = -1024 sum(x) then sixteen v_dot2 over the offset-form codes, acc = fma(s, d, acc),
// acc = fma(b, 16 sum(x), acc); the 16 chains meet in the DPP butterfly (pairs, then quads,
// eights, sixteens); the row is scaled by 1/16. Here the same operations run in the same order,
// only spread differently:
//
//  * Four lanes own one weight row. Of each 16 chunks (one per virtual lane) the lane in quarter
//    p = 0..3 of its wave (lane bits 4 and 5) runs chunks 4p .. 4p+3, i.e. virtual lanes
//    4p .. 4p+3, for up to MR activation rows at once: each chunk's codes are unpacked once and
//    feed every activation row, whose chains stay in registers (4 * MR accumulators).
//  * The 16 rows of a wave read their 64-byte quarters of each 256-byte segment in one load
//    instruction, the next segment in flight while the current one computes.
//  * The activations are the same for every row. Each block stages them once in LDS, in the
//    form the M=1 kernels compute per chunk (x32_off_from: the permuted pairs, 16 * sum and
//    -1024 * sum), for as many chunks as fit (all of K = 2560 at 8 rows). The four lanes of a
//    quad run the same chunk for four rows; each reads a quarter of the chunk's activations
//    and the dots take the rest from the quad by DPP.
//  * At the end each lane sums its four chains (the butterfly's quad of virtual lanes), and two
//    exchanges across the quarters (the 16- and 32-lane swaps) add the quads in the butterfly's
//    order; floating-point addition is commutative, so every quarter ends with the same bits.
// The arithmetic is the M=1 kernels' for every K they take, so the two agree bit for bit
// wherever both run. The matrix-core kernels (gemv_mfma.hip, gemm.hip) round each dequantized
// weight to fp16 and sum in another order; they remain as an explicit option.
#include "dhp_internal.hpp"

#include <math.h>
#include <limits.h>

namespace {

constexpr int SEG = 16;          // chunks per segment: one per virtual lane
constexpr int QCH = 4;           // chunks of a segment per lane (virtual lanes 4p .. 4p+3)
constexpr int XW = 20;           // dwords per staged (chunk, activation row): 16 pair words, 16 sum, -1024 sum, pad
// dwords per staged chunk (its MR rows): 4 dwords of padding put the chunks that the four quarters of
// a wave read at once (4 chunks apart) 16 banks apart
constexpr int cstride(int MR) { return MR * XW + 4; }
constexpr int THREADS = 512;     // 8 waves
constexpr int ROWS_BLOCK = THREADS / 4;   // weight rows per block (16 per wave)
constexpr size_t STAGE_BYTES = 64 * 1024;   // LDS for the staged activations

// Chunks per staging window for MR activation rows: a multiple of 16, at most STAGE_BYTES.
constexpr int window_chunks(int MR) { return (int)(STAGE_BYTES / (cstride(MR) * 4)) / SEG * SEG; }

// Stage chunks w0 .. w0+W-1 (those below CH) of activation rows m0 .. m0+MR-1 (rows past mr
// repeat row mr - 1, so the compute loop needs no check per row; their results are never stored).
template <int MR>
DHP_DEV void stage_window(uint32_t* xs, const _Float16* __restrict__ x, int m0, int mr, int K, int CH, int w0, int W) {
    __syncthreads();                          // the previous window's reads are done
    for (int it = threadIdx.x; it < W * MR; it += THREADS) {
        const int j = it / MR, r = it - j * MR;
        const int c = w0 + j;
        if (c < CH) {
            const int rs = r < mr ? r : mr - 1;
            const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)(m0 + rs) * K + 32 * c);
            const u32x4 v[4] = {src[0], src[1], src[2], src[3]};
            h2 xp[16];
            float nc;
            const float s16 = x32_off_from(v, xp, nc);
            uint32_t* dst = xs + (size_t)j * cstride(MR) + r * XW;
#pragma unroll
            for (int l = 0; l < 4; ++l)                 // lane l of a quad reads words l, l+4, l+8, l+12
                *reinterpret_cast<u32x4*>(dst + 4 * l) =
                    u32x4{h2_bits(xp[l]), h2_bits(xp[4 + l]), h2_bits(xp[8 + l]), h2_bits(xp[12 + l])};
            dst[16] = __builtin_bit_cast(uint32_t, s16);
            dst[17] = __builtin_bit_cast(uint32_t, nc);
        }
    }
    __syncthreads();
}

// One lane's quarter of a segment of its row: 4 chunks of codes and the scales and biases of
// their 2 groups, packed as two bf16 per word. Chunks past the row are clamped to its last chunk
// (loaded, never used). With FULL (K % 512 == 0) the row's scales start 16-byte aligned and a
// quarter's pair of groups is one 4-byte load.
struct QuarterRegs {
    u32x4 c[QCH];
    uint32_t s, b;
};
template <bool FULL>
DHP_DEV void load_quarter(QuarterRegs& l, const u32x4* __restrict__ cr, const uint16_t* __restrict__ sr,
                          const uint16_t* __restrict__ br, int cb, int CH) {
#pragma unroll
    for (int i = 0; i < QCH; ++i) l.c[i] = __builtin_nontemporal_load(cr + min(cb + i, CH - 1));
    if constexpr (FULL) {
        const int g0 = min(cb, CH - QCH) >> 1;          // even: 4-byte aligned
        l.s = *reinterpret_cast<const uint32_t*>(sr + g0);
        l.b = *reinterpret_cast<const uint32_t*>(br + g0);
    } else {
        const int g0 = min(cb, CH - 1) >> 1, g1 = min(cb + 2, CH - 1) >> 1;
        l.s = (uint32_t)sr[g0] | ((uint32_t)sr[g1] << 16);
        l.b = (uint32_t)br[g0] | ((uint32_t)br[g1] << 16);
    }
}
// group h (0, 1) of a quarter: its scale or bias as fp32
DHP_DEV float half_bf16(uint32_t w, int h) { return __builtin_bit_cast(float, h ? (w & 0xFFFF0000u) : (w << 16)); }

// Eight pair dots (pairs 8h .. 8h+7 of a chunk, dot32_off's order) for NC activation rows at once,
// each row's activation word e taken from lane e & 3 of the quad by a DPP quad broadcast inside
// v_dot2c (every lane of a quad holds 16 bytes of the chunk's 64, so LDS delivers a quarter of
// what reading every word in every lane would). The compiler cannot see the instructions in the
// block, so the block keeps its own wait states: three on entry (a DPP instruction must not read a
// VGPR a VALU instruction wrote in the two cycles before), three on exit (a VALU instruction other
// than the same dot must not read a dot's result within three), and inside it a row's accumulator
// is written at least two instructions before it is read again (four rows: three other dots in
// between; two rows: one dot and a nop).
//   d[c]: row c's chain; t8: the 8 code pairs; xw2[c]: row c's words from component 2h, 2h+1.
DHP_DEV void dots_half4(float (&d)[4], const uint32_t (&t8)[8], const uint32_t (&xw2)[4][2]) {
    asm("s_nop 2\n\tv_dot2c_f32_f16_dpp %0, %12, %4 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %1, %14, %4 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %2, %16, %4 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %3, %18, %4 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %0, %12, %5 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %1, %14, %5 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %2, %16, %5 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %3, %18, %5 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %0, %12, %6 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %1, %14, %6 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %2, %16, %6 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %3, %18, %6 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %0, %12, %7 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %1, %14, %7 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %2, %16, %7 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %3, %18, %7 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %0, %13, %8 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %1, %15, %8 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %2, %17, %8 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %3, %19, %8 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %0, %13, %9 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %1, %15, %9 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %2, %17, %9 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %3, %19, %9 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %0, %13, %10 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %1, %15, %10 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %2, %17, %10 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %3, %19, %10 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %0, %13, %11 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %1, %15, %11 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %2, %17, %11 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %3, %19, %11 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\ts_nop 2"
        : "+v"(d[0]), "+v"(d[1]), "+v"(d[2]), "+v"(d[3])
        : "v"(t8[0]), "v"(t8[1]), "v"(t8[2]), "v"(t8[3]), "v"(t8[4]), "v"(t8[5]), "v"(t8[6]), "v"(t8[7]),
          "v"(xw2[0][0]), "v"(xw2[0][1]), "v"(xw2[1][0]), "v"(xw2[1][1]), "v"(xw2[2][0]), "v"(xw2[2][1]),
          "v"(xw2[3][0]), "v"(xw2[3][1]));
}
DHP_DEV void dots_half2(float (&d)[2], const uint32_t (&t8)[8], const uint32_t (&xw2)[2][2]) {
    asm("s_nop 2\n\tv_dot2c_f32_f16_dpp %0, %10, %2 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %1, %12, %2 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\ts_nop 0\n\tv_dot2c_f32_f16_dpp %0, %10, %3 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %1, %12, %3 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\ts_nop 0\n\tv_dot2c_f32_f16_dpp %0, %10, %4 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %1, %12, %4 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\ts_nop 0\n\tv_dot2c_f32_f16_dpp %0, %10, %5 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %1, %12, %5 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\ts_nop 0\n\tv_dot2c_f32_f16_dpp %0, %11, %6 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %1, %13, %6 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\ts_nop 0\n\tv_dot2c_f32_f16_dpp %0, %11, %7 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %1, %13, %7 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\ts_nop 0\n\tv_dot2c_f32_f16_dpp %0, %11, %8 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %1, %13, %8 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\ts_nop 0\n\tv_dot2c_f32_f16_dpp %0, %11, %9 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\tv_dot2c_f32_f16_dpp %1, %13, %9 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\ts_nop 0\n\ts_nop 2"
        : "+v"(d[0]), "+v"(d[1])
        : "v"(t8[0]), "v"(t8[1]), "v"(t8[2]), "v"(t8[3]), "v"(t8[4]), "v"(t8[5]), "v"(t8[6]), "v"(t8[7]),
          "v"(xw2[0][0]), "v"(xw2[0][1]), "v"(xw2[1][0]), "v"(xw2[1][1]));
}

// The 16 pair dots of one chunk for NC rows: d[c] starts at row c's -1024 sum and ends at
// 16 q.x; xw[c] is row c's 16 bytes (components 0..3 = words q, q+4, q+8, q+12 of quad lane q).
template <int NC>
DHP_DEV void dots_chunk(float (&d)[NC], const uint32_t (&t)[16], const u32x4 (&xw)[NC]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t t8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) t8[e] = t[8 * h + e];
        uint32_t x2[NC][2];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            x2[c][0] = h ? xw[c].z : xw[c].x;
            x2[c][1] = h ? xw[c].w : xw[c].y;
        }
        if constexpr (NC == 4) dots_half4(d, t8, x2);
        else dots_half2(d, t8, x2);
    }
}

// A compiler barrier for memory operations: LDS reads are not moved across it (without it the
// compiler hoists every LDS read of a line to the top and runs out of registers).
DHP_DEV void mem_fence_compiler() { asm volatile("" ::: "memory"); }

// The chains of chunks cb .. cb+3 (chunk cb + i extends this lane's chain i) for every activation
// row; xw: the staged blocks of chunk cb (its MR rows), then the next chunk's.
template <int MR, bool TAIL>
DHP_DEV void run_quarter(const QuarterRegs& l, const uint32_t* xw, float (&acc)[MR][QCH], int cb, int CH,
                         const NibConsts& nk, int q) {
#pragma unroll
    for (int i = 0; i < QCH; ++i) {
        mem_fence_compiler();                 // one chunk's activations read at a time
        // in a partial segment, chunks past the row run on clamped codes and stale LDS and are
        // discarded by a select (a branch here had the compiler hoist the whole segment's reads)
        const bool live = !TAIL || cb + i < CH;
        const float s = half_bf16(l.s, i >> 1);
        const float b = half_bf16(l.b, i >> 1);
        h2 tp[16];
        unpack8_off(l.c[i].x, tp, nk);
        unpack8_off(l.c[i].y, tp + 4, nk);
        unpack8_off(l.c[i].z, tp + 8, nk);
        unpack8_off(l.c[i].w, tp + 12, nk);
        uint32_t t[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) t[e] = h2_bits(tp[e]);
        constexpr int NC = MR >= 4 ? 4 : 2;       // rows per dot block
#pragma unroll
        for (int r0 = 0; r0 < MR; r0 += NC) {
            u32x4 xq[NC];
            float2 sn[NC];
            float d[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const uint32_t* blk = xw + (size_t)i * cstride(MR) + (r0 + c) * XW;
                xq[c] = *reinterpret_cast<const u32x4*>(blk + 4 * q);
                sn[c] = *reinterpret_cast<const float2*>(blk + 16);
                d[c] = sn[c].y;
            }
            dots_chunk<NC>(d, t, xq);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const float a0 = acc[r0 + c][i];
                const float a1 = __builtin_fmaf(b, sn[c].x, __builtin_fmaf(s, d[c], a0));
                acc[r0 + c][i] = live ? a1 : a0;
            }
            mem_fence_compiler();                 // one block of rows' activations in registers at a time
        }
    }
}

template <int MR, bool F32OUT, bool ARGMAX, bool FULL>
// Whole segments (K % 512 == 0): 128 VGPRs, four waves per SIMD, two blocks of eight waves per CU
// (their staged activations fit the LDS twice). With a partial last segment the selects need more
// registers: one block per CU, no spills.
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(FULL ? 4 : 2, FULL ? 4 : 2))) void k_gemv_rows(
    const u32x4* __restrict__ codes, const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    const _Float16* __restrict__ x, int m0, int mr, int N, int K, void* __restrict__ y,
    float* __restrict__ part_v, int* __restrict__ part_i) {
    extern __shared__ __align__(16) uint32_t xs[];     // [window chunks][cstride(MR)]: [MR][XW], pad
    constexpr int WMAX = window_chunks(MR);
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int q = lane & 3;                  // quad lane: which 16 bytes of a staged chunk it reads
    const int p = lane >> 4;                 // quarter: virtual lanes 4p .. 4p+3
    const int row = blockIdx.x * ROWS_BLOCK + wave * 16 + (lane & 15);
    const int rr = min(row, N - 1);          // rows past N compute the last row again, unstored
    const int CH = K >> 5, G = K >> 6;
    const u32x4* cr = codes + (size_t)rr * CH;
    const uint16_t* sr = scales + (size_t)rr * G;
    const uint16_t* br = biases + (size_t)rr * G;
    const int W = min(WMAX, (CH + SEG - 1) / SEG * SEG);
    const int pc = QCH * p;                  // this lane's first chunk in a segment

    float acc[MR][QCH];
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
        for (int j = 0; j < QCH; ++j) acc[r][j] = 0.0f;
    const NibConsts nk = nib_consts();

    // one segment computes while the next is in flight; segments alternate between two register sets
    QuarterRegs la, lb;
    load_quarter<FULL>(la, cr, sr, br, pc, CH);
    int w0 = -WMAX;
#pragma unroll 1
    for (int c0 = 0; c0 < CH; c0 += 2 * SEG) {
        if (c0 >= w0 + WMAX) {               // the next staging window (once, at K <= 3072 for 8 rows)
            w0 = c0;
            stage_window<MR>(xs, x, m0, mr, K, CH, w0, W);
        }
        load_quarter<FULL>(lb, cr, sr, br, c0 + SEG + pc, CH);
        run_quarter<MR, !FULL>(la, xs + (size_t)(c0 - w0 + pc) * cstride(MR), acc, c0 + pc, CH, nk, q);
        const int c1 = c0 + SEG;
        if (c1 < CH) {                       // uniform over the block
            if (c1 >= w0 + WMAX) {
                w0 = c1;
                stage_window<MR>(xs, x, m0, mr, K, CH, w0, W);
            }
            load_quarter<FULL>(la, cr, sr, br, c1 + SEG + pc, CH);
            run_quarter<MR, !FULL>(lb, xs + (size_t)(c1 - w0 + pc) * cstride(MR), acc, c1 + pc, CH, nk, q);
        }
    }

    __shared__ float bv_s[MR][THREADS / 64];
    __shared__ int bi_s[MR][THREADS / 64];
    float vals[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        // this lane's quad of virtual lanes, then the quads in the butterfly's order: the
        // 16-lane row swap adds quarters 0+1 and 2+3, the 32-lane swap the two halves (each
        // swap hands both operands to every lane; addition is commutative, so all quarters end
        // with the same bits)
        const float qv = (acc[r][0] + acc[r][1]) + (acc[r][2] + acc[r][3]);
        const auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, qv), __builtin_bit_cast(uint32_t, qv),
                                                        false, false);
        const float h = __builtin_bit_cast(float, (uint32_t)a[0]) + __builtin_bit_cast(float, (uint32_t)a[1]);
        const auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, h), __builtin_bit_cast(uint32_t, h),
                                                        false, false);
        const float v = (__builtin_bit_cast(float, (uint32_t)b[0]) + __builtin_bit_cast(float, (uint32_t)b[1])) * 0.0625f;
        vals[r] = v;
        const size_t o = (size_t)(m0 + r) * N + row;
        if (r < mr && row < N && (r & 3) == p) {   // one quarter stores each row
            if constexpr (F32OUT) reinterpret_cast<float*>(y)[o] = v;
            else reinterpret_cast<_Float16*>(y)[o] = (_Float16)v;
        }
    }
    if constexpr (ARGMAX) {
        // the wave's best weight row for activation rows r0 .. r0+3 at once: quarter p ranks
        // row r0 + p over its 16 lanes (the wave's 16 weight rows)
#pragma unroll
        for (int r0 = 0; r0 < MR; r0 += 4) {
            float mine = vals[r0];
#pragma unroll
            for (int q = 1; q < 4; ++q)
                if (r0 + q < MR && p == q) mine = vals[r0 + q];
            const int ar = r0 + p;
            const bool ok = row < N && ar < mr;
            float bv = ok ? mine : -INFINITY;
            int bi = ok ? row : INT_MAX;
            best_step<DPP_XOR1>(bv, bi);
            best_step<DPP_XOR2>(bv, bi);
            best_step<DPP_HALF_MIRROR>(bv, bi);
            best_step<DPP_MIRROR>(bv, bi);
            if ((lane & 15) == 0 && ar < mr) { bv_s[ar][wave] = bv; bi_s[ar][wave] = bi; }
        }
    }
    if constexpr (ARGMAX) {
        __syncthreads();
        if (t < mr) {
            float bv = bv_s[t][0];
            int bi = bi_s[t][0];
            for (int w = 1; w < THREADS / 64; ++w)
                if (better(bv_s[t][w], bi_s[t][w], bv, bi)) { bv = bv_s[t][w]; bi = bi_s[t][w]; }
            part_v[(size_t)(m0 + t) * gridDim.x + blockIdx.x] = bv;     // [act row][block], as the
            part_i[(size_t)(m0 + t) * gridDim.x + blockIdx.x] = bi;     // final reduction reads them
        }
    }
}

template <int MR, bool FULL>
hipError_t launch_rows_full(bool f32, bool am, dim3 g, size_t lds, hipStream_t s, const u32x4* c, const uint16_t* sc,
                            const uint16_t* bi, const _Float16* x, int m0, int mr, int N, int K, void* y, float* pv,
                            int* pi) {
    const dim3 b(THREADS);
    if (f32 && am) hipLaunchKernelGGL((k_gemv_rows<MR, true, true, FULL>), g, b, lds, s, c, sc, bi, x, m0, mr, N, K, y, pv, pi);
    else if (f32) hipLaunchKernelGGL((k_gemv_rows<MR, true, false, FULL>), g, b, lds, s, c, sc, bi, x, m0, mr, N, K, y, pv, pi);
    else if (am) hipLaunchKernelGGL((k_gemv_rows<MR, false, true, FULL>), g, b, lds, s, c, sc, bi, x, m0, mr, N, K, y, pv, pi);
    else hipLaunchKernelGGL((k_gemv_rows<MR, false, false, FULL>), g, b, lds, s, c, sc, bi, x, m0, mr, N, K, y, pv, pi);
    return hipGetLastError();
}

template <int MR>
hipError_t launch_rows_mr(bool f32, bool am, dim3 g, hipStream_t s, const u32x4* c, const uint16_t* sc,
                          const uint16_t* bi, const _Float16* x, int m0, int mr, int N, int K, void* y, float* pv,
                          int* pi) {
    const int CH = K >> 5;
    const int W = min(window_chunks(MR), (CH + SEG - 1) / SEG * SEG);
    const size_t lds = (size_t)W * cstride(MR) * 4;
    if (CH % SEG == 0) return launch_rows_full<MR, true>(f32, am, g, lds, s, c, sc, bi, x, m0, mr, N, K, y, pv, pi);
    return launch_rows_full<MR, false>(f32, am, g, lds, s, c, sc, bi, x, m0, mr, N, K, y, pv, pi);
}

}  // namespace

// Blocks of the multi-row GEMV for N weight rows (the argmax partials per activation row).
int dhp_gemv_rows_blocks(int N) { return (N + ROWS_BLOCK - 1) / ROWS_BLOCK; }

int launch_gemv_rows(const dhp_int4* w, const void* x, int M, void* y, int y_f32, int32_t* argmax, void* ws,
                     size_t ws_part_stride, hipStream_t s) {
    const int N = w->rows, K = w->cols;
    const int nb = dhp_gemv_rows_blocks(N);
    // the partials [M][nb] fit the workspace's half of ws_part_stride bytes
    if (argmax && (size_t)nb * M * sizeof(float) > ws_part_stride)
        return dhp_fail(DHP_ERR_UNSUPPORTED, "N=%d needs %d argmax partials per row", N, nb);
    float* pv = argmax ? static_cast<float*>(ws) : nullptr;
    int* pi = argmax ? reinterpret_cast<int*>(static_cast<char*>(ws) + ws_part_stride) : nullptr;
    const auto* c = static_cast<const u32x4*>(w->codes);
    const auto* sc = static_cast<const uint16_t*>(w->scales);
    const auto* bi = static_cast<const uint16_t*>(w->biases);
    const auto* xh = static_cast<const _Float16*>(x);
    const bool am = argmax != nullptr;
    const dim3 g((unsigned)nb);
    // activation rows in passes of up to 8 (each pass streams the weights once)
    for (int m0 = 0; m0 < M; m0 += 8) {
        const int mr = M - m0 < 8 ? M - m0 : 8;
        hipError_t e;
        if (mr <= 2) e = launch_rows_mr<2>(y_f32, am, g, s, c, sc, bi, xh, m0, mr, N, K, y, pv, pi);
        else if (mr <= 4) e = launch_rows_mr<4>(y_f32, am, g, s, c, sc, bi, xh, m0, mr, N, K, y, pv, pi);
        else e = launch_rows_mr<8>(y_f32, am, g, s, c, sc, bi, xh, m0, mr, N, K, y, pv, pi);
        if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "gemv rows launch: %s", hipGetErrorString(e));
    }
    if (argmax) {
        const hipError_t e2 = launch_argmax_final(pv, pi, nb, M, argmax, s);
        if (e2 != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "argmax launch: %s", hipGetErrorString(e2));
    }
    return DHP_OK;
}
