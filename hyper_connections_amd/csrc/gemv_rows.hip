// Multi-row INT4-affine GEMV (2 <= m <= 16 rows of activations) on the matrix cores that gives
// every output exactly the bits the M=1 GEMV gives for that row alone.
//
// "src/real_forward.rs" (turbospark-runtime 0.3.0), field batched_gemv_prefill: the batched
// GEMV kernel and the per-row GEMV agree bit for bit (only the matrix-instruction variant, a
// separate option, differs). The M=1 kernels (gemv.hip) fix each output's arithmetic: chain j
// (j = 0..7) takes the 64-code groups j, j+8, j+16, ... of the row, one fp32 step per group on
// the group's exact integer sum (xg_group_acc); the 8 chains meet in the butterfly (pairs,
// quads, eights). The integer sum is exact whatever the order of its products, so the matrix
// cores may form it:
//
//  * A wave owns a tile of 16 weight rows over all of K. v_mfma_i32_16x16x64_i8 takes one group
//    per instruction: B is the group's codes (lane (n, w) = weight row n, code word w of both
//    chunks, unpacked to int8 in unpack_i8's order), A holds four activation rows' three int8
//    pieces (fragment row 4a + p = activation row a, piece p; the fourth slot repeats piece 2 and
//    its result is unused), so lane (n, a) receives row a's three piece sums for weight row n and
//    joins them (D = P2 * 2^14 + P1 * 2^7 + P0, exact). Eight activation rows take two
//    instructions.
//  * Codes stream as in the M=1 kernels: 16 lanes read 256 contiguous bytes of one row (16-byte
//    nontemporal loads, four rows per instruction). A super-step is 16 chunks of the tile's 16
//    rows (8 groups, one per chain); the next one is in flight while one computes. A small LDS
//    region per wave turns it around: lane (n, w) reads back chunk c0 + 4u + w of row n, and two
//    swaps across the wave halves (v_permlane32_swap) and two across neighbouring 16-lane rows
//    (v_permlane16_swap) transpose each 4 x 4 block so that lane (n, w) holds code word w of the
//    four chunks.
//  * Scales and biases: where the tile's rows are whole and few enough groups (SBT), the tile's
//    16 rows of scales and biases arrive as one coalesced block into the wave's region; otherwise
//    each lane loads the scale and bias of its own chunk and they take the same turnaround.
//  * The activations' pieces (xg_stage_octet, the same conversion as the M=1 kernels) are staged
//    once per block in LDS; one block of twelve waves per compute unit, walking tiles.
//  * Each chain's steps run in group order, and the final butterfly adds the chains in the M=1
//    kernels' order (addition is commutative, so each pair gives the same bits either way round).
#include "dhp_internal.hpp"

#include <math.h>
#include <limits.h>

typedef int i32x4 __attribute__((ext_vector_type(4)));

namespace {

#ifndef DHP_ROWS_WPB
#define DHP_ROWS_WPB 12
#endif
constexpr int WPB = DHP_ROWS_WPB;        // waves per block
constexpr int THREADS = 64 * WPB;
constexpr int SUP = 16;                  // chunks per super-step: one per chain
constexpr size_t STAGE_MAX = 80 * 1024;  // LDS for the staged activations of one block
// One wave's region in LDS: the super-step's codes (16 rows of 16 chunks, rows padded by 16 bytes
// so that the 16-byte reads of eight rows hit distinct banks), then either
//  * the tile's scales and biases as one block (SBT: [scales 16 rows x G][biases 16 rows x G],
//    bf16, at most SBT_MAX bytes), written once per tile, or
//  * the super-step's scale and bias words (16 rows of 8 groups; a 40-byte row pitch keeps 16
//    rows' 8-byte reads on distinct banks), written every super-step.
constexpr int TR_PITCH = 272;
constexpr int SB_PITCH = 40;
constexpr int TR_CODES = 16 * TR_PITCH;
constexpr int SBT_MAX = 3072;
template <bool SBT> constexpr int region_bytes() { return TR_CODES + (SBT ? SBT_MAX : 16 * SB_PITCH); }

#define DHP_DEV_HOST_INLINE __host__ __device__ __forceinline__

// LDS of one block: the staged groups, then each row's (sum, power of two) pairs [MR][W/2] so that
// a lane reads two groups' pairs with one 16-byte read. Group g of activation rows 4mi .. 4mi+3 is
// one A operand block of AB_DW words laid out in lane order: the 16 bytes of piece word
// (p, 0..1, w, 0..1) of row 4mi + a at word 4 (12w + 3a + p), so the lanes of one fragment read
// consecutive 16-byte slots (slot p = 3 of a row repeats p = 2) without bank conflicts.
constexpr int AB_DW = 4 * 4 * 3 * 4;
constexpr size_t stage_bytes_per_chunk(int MR) { return (size_t)(MR / 4) * AB_DW * 4 / 2 + (size_t)MR * 4; }
// Bytes of a staging window of W chunks, rounded up to 16 (the turnaround regions follow).
DHP_DEV_HOST_INLINE size_t stage_bytes(int MR, int W) { return ((size_t)W * stage_bytes_per_chunk(MR) + 15) / 16 * 16; }

// Chunks per staging window for MR activation rows: all of K rounded up to 16 chunks when that fits
// (all of K = 2560 at 8 rows), else a multiple of 32, so that windows start where a pair of
// super-steps does.
template <int MR>
DHP_DEV_HOST_INLINE int window_chunks(int CH) {
    const int fit = (int)(STAGE_MAX / stage_bytes_per_chunk(MR));
    const int all = (CH + SUP - 1) / SUP * SUP;
    return all <= fit ? all : fit / (2 * SUP) * (2 * SUP);
}

// Stage chunks w0 .. w0+W-1 (those below CH; W and w0 even) of activation rows m0 .. m0+MR-1 (rows
// past mr repeat row mr - 1; their results are never stored).
template <int MR>
DHP_DEV void stage_window(uint32_t* xs, float2* sps, const _Float16* __restrict__ x, int m0, int mr, int K, int CH,
                          int w0, int W) {
    __syncthreads();                          // the previous window's reads are done
    const int WG = W / 2;
    const int n = 8 * min(WG, (CH - w0) / 2) * MR;   // eight lanes per (group, row)
    for (int it = threadIdx.x; it < n; it += THREADS) {
        const int item = it >> 3, i = it & 7;
        const int j = item / MR, r = item - j * MR;
        const int rs = r < mr ? r : mr - 1;
        uint32_t* d = xs + ((size_t)j * (MR / 4) + (r >> 2)) * AB_DW + 4 * (12 * (i & 3) + 3 * (r & 3)) + 2 * (i >> 2);
        const float2 sp = xg_stage_octet(x + (size_t)(m0 + rs) * K + 32 * w0 + 64 * j, i, d, 4);
        if (i == 0) sps[r * WG + j] = sp;
    }
    // groups past the row (the padding of a last, partial super-step): zero pieces and pairs, so
    // that their products are exact zeros
    const int jr = min(WG, (CH - w0) / 2);
    const int nz = (WG - jr) * (MR / 4) * AB_DW;
    for (int it = threadIdx.x; it < nz; it += THREADS) xs[(size_t)jr * (MR / 4) * AB_DW + it] = 0u;
    for (int it = threadIdx.x; it < (WG - jr) * MR; it += THREADS)
        sps[(it / (WG - jr)) * WG + jr + it % (WG - jr)] = float2{0.0f, 0.0f};
    __syncthreads();
}

// One super-step of one lane as loaded: lane (g, j) holds chunk c0 + j of tile row 4u + g in c[u],
// and (per-chunk path only) that chunk's group scale (low half) and bias (high half) in sb[u].
// Rows past N are clamped to the last row (computed again, never stored); chunks past the row to
// its last chunk.
typedef unsigned short u16x2v __attribute__((ext_vector_type(2)));
struct SupRegs {
    u32x4 c[4];
    u16x2v sb[4];
};
// cb, sb, bb: the tile's first row (uniform over the wave); rmax: the tile's last real row. With
// SBT the scales and biases come from the tile block instead.
template <bool SBT>
DHP_DEV void load_sup(SupRegs& l, const u32x4* __restrict__ cb, const uint16_t* __restrict__ sb,
                      const uint16_t* __restrict__ bb, int rmax, int c0, int g, int j, int CH, int G) {
    const int ch = min(c0 + j, CH - 1);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int r = min(4 * u + g, rmax);
        l.c[u] = __builtin_nontemporal_load(cb + (uint32_t)(r * CH + ch));
        if constexpr (!SBT) {
            const uint32_t o = (uint32_t)(r * G + (ch >> 1));
            l.sb[u] = u16x2v{sb[o], bb[o]};
        }
    }
}

// The tile block (SBT, every tile whole: N % 16 == 0): the 16 rows' scales, then their biases
// (32 G bytes each, contiguous in memory, 16-byte aligned), as 16-byte pieces p = lane + 64 i,
// i < 3 (64 G <= 3072). Pieces past 4 G read the last piece again and are not written.
DHP_DEV void load_tile_sb(u32x4 (&q)[3], const uint16_t* __restrict__ sb, const uint16_t* __restrict__ bb,
                          int G, int lane) {
    const int half = 32 * G;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int off = min(16 * (lane + 64 * i), 64 * G - 16);
        const bool isb = off >= half;
        q[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(isb ? bb : sb) + (isb ? off - half : off));
    }
}
DHP_DEV void store_tile_sb(const u32x4 (&q)[3], uint8_t* blk, int G, int lane) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int off = 16 * (lane + 64 * i);
        if (off < 64 * G) *reinterpret_cast<u32x4*>(blk + off) = q[i];
    }
}

// v_permlane32_swap: a's upper 32 lanes trade places with b's lower 32 lanes.
DHP_DEV void swap32(uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}
// v_permlane16_swap: a's odd 16-lane rows trade places with b's even rows.
DHP_DEV void swap16(uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}

// The chains' steps for the 8 groups of one super-step (group gi extends chain gi) for MI groups of
// four activation rows; xw: the staged pieces of the super-step's first group, spw: row 0's pair
// of that group (row r's at spw + r * WG); tw: the wave's turnaround region. Each quad of chunks
// (two groups) reads its LDS operands first, then runs its 2 * MI matrix instructions and their
// chain steps.
//
// PAD (K % 512 != 0): the row's last super-step runs past the row. Its padding groups have zero
// staged pieces and pairs (so D = 0, sum 0, power of two 0) and get -0 as scale and bias, so each
// of their steps is fma(fma(-0, 0, -0 * 0), 0, acc) = acc + (-0), which is acc for every acc,
// zeros of either sign included: the chains take the same values as in the M=1 kernels.
//
// sbq[u]: groups 2u, 2u + 1 of the super-step for row n. SBT: their two scales (x) and two biases
// (y) from the tile block, group 2u in the low halves (G even, so a padding group's pair is padding
// as a whole). Otherwise the per-super-step words: group 2u's (scale, bias) in x, group 2u + 1's
// in y.
template <int MI, bool PAD, bool SBT>
DHP_DEV void run_sup(const SupRegs& l, const uint32_t* xw, const float2* spw, int WG, float (&acc)[MI][SUP / 2],
                     int c0, int CH, int G, int lane, uint8_t* tw) {
    const int w = lane >> 4;                          // code word of a chunk; activation row of a result
    const int j = lane & 15;
    const int a_off = 4 * (12 * w + 3 * (j >> 2) + min(lane & 3, 2));   // A fragment words
    // turnaround: lane (w, j) wrote chunk c0 + j of tile rows 4u + w; lane (n = j, w) reads back
    // chunk c0 + 4u + w of row n (and, per super-step, the scale and bias words of row n)
    u32x4 cq[4];
    uint2 sbq[4];
    uint8_t* tsb = tw + TR_CODES;
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4*>(tw + (4 * u + w) * TR_PITCH + 16 * j) = l.c[u];
    if constexpr (!SBT) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint32_t pk = __builtin_bit_cast(uint32_t, l.sb[u]);
            if (PAD && c0 + j >= CH) pk = 0x80008000u;    // -0 scale and bias for a padding group
            // both lanes of a group write the same word
            *reinterpret_cast<uint32_t*>(tsb + (4 * u + w) * SB_PITCH + 4 * (j >> 1)) = pk;
        }
    }
    // the region is the wave's own: its LDS operations complete in order, so only the compiler
    // must not move the reads above the writes
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < 4; ++u) cq[u] = *reinterpret_cast<const u32x4*>(tw + j * TR_PITCH + 16 * (4 * u + w));
    if constexpr (SBT) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int ga = (c0 >> 1) + 2 * u;
            const int o = j * 2 * G + 2 * min(ga, G - 2);
            sbq[u] = uint2{*reinterpret_cast<const uint32_t*>(tsb + o), *reinterpret_cast<const uint32_t*>(tsb + 32 * G + o)};
            if (PAD && ga >= G) sbq[u] = uint2{0x80008000u, 0x80008000u};   // -0 for a padding pair
        }
    } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) sbq[u] = *reinterpret_cast<const uint2*>(tsb + j * SB_PITCH + 8 * u);
    }
    // and the next super-step's writes must not move above these reads
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        // one quad in registers at a time (the scheduler would interleave all of them)
        __builtin_amdgcn_sched_barrier(0);
        i32x4 aq[2][MI];
        float2 sp[2][MI];
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                aq[e][mi] = *reinterpret_cast<const i32x4*>(xw + (size_t)((2 * u + e) * MI + mi) * AB_DW + a_off);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const float4 v = *reinterpret_cast<const float4*>(spw + (4 * mi + w) * WG + 2 * u);
            sp[0][mi] = float2{v.x, v.y};
            sp[1][mi] = float2{v.z, v.w};
        }
        // lane (n, w) holds the four words of chunk c0 + 4u + w; afterwards word w of chunks
        // c0 + 4u .. c0 + 4u + 3 (groups 2u and 2u + 1 of the super-step)
        uint32_t r0 = cq[u].x, r1 = cq[u].y, r2 = cq[u].z, r3 = cq[u].w;
        swap32(r0, r2);
        swap32(r1, r3);
        swap16(r0, r1);
        swap16(r2, r3);
        const uint32_t wv[4] = {r0, r1, r2, r3};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int gi = 2 * u + e;
            uint32_t lo0, hi0, lo1, hi1;
            unpack_i8(wv[2 * e], lo0, hi0);
            unpack_i8(wv[2 * e + 1], lo1, hi1);
            const i32x4 bq = {(int)lo0, (int)hi0, (int)lo1, (int)hi1};
            float s, b;                                // group gi = 2u + e as fp32
            if constexpr (SBT) {
                s = __builtin_bit_cast(float, e ? (sbq[u].x & 0xFFFF0000u) : (sbq[u].x << 16));
                b = __builtin_bit_cast(float, e ? (sbq[u].y & 0xFFFF0000u) : (sbq[u].y << 16));
            } else {
                const uint32_t sbw = e ? sbq[u].y : sbq[u].x;
                s = __builtin_bit_cast(float, sbw << 16);
                b = __builtin_bit_cast(float, sbw & 0xFFFF0000u);
            }
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const i32x4 d = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[e][mi], bq, i32x4{0, 0, 0, 0}, 0, 0, 0);
                acc[mi][gi] = xg_group_acc(acc[mi][gi], d[2] * 16384 + d[1] * 128 + d[0], s, b, sp[e][mi].x, sp[e][mi].y);
            }
        }
    }
}

// One resident block per compute unit (the staged activations and the waves' regions need more
// than half its LDS). FULL: K % 512 == 0, no padding groups. ONE: all of K fits one staging
// window, staged once per block before the first tile. SBT (only with ONE): each tile's scales
// and biases arrive as one coalesced block (2.5 KB at K = 2560) instead of 2-byte loads per chunk;
// with a cold last-level cache the loads alone of the M=8 LM head took 44.7 against 47.4 us.
template <int MI, bool F32OUT, bool ARGMAX, bool FULL, bool ONE, bool SBT>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(WPB / 4, WPB / 4))) void k_gemv_rows(
    const u32x4* __restrict__ codes, const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    const _Float16* __restrict__ x, int m0, int mr, int N, int K, void* __restrict__ y,
    float* __restrict__ part_v, int* __restrict__ part_i) {
    constexpr int MR = 4 * MI;
    extern __shared__ __align__(16) uint32_t xs[];     // [W/2][MI][AB_DW], then the pairs [MR][W/2]
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int CH = K >> 5, G = K >> 6;
    const int W = window_chunks<MR>(CH);
    const int WG = W / 2;
    float2* sps = reinterpret_cast<float2*>(xs + (size_t)WG * MI * AB_DW);
    uint8_t* tw = reinterpret_cast<uint8_t*>(xs) + stage_bytes(MR, W) + (size_t)wave * region_bytes<SBT>();
    const int ngroups = ((N + 15) / 16 + WPB - 1) / WPB;
    if constexpr (ONE) stage_window<MR>(xs, sps, x, m0, mr, K, CH, 0, W);

    float best_v[MI];
    int best_i[MI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        best_v[mi] = -INFINITY;
        best_i[mi] = INT_MAX;
    }
    // With all of K staged once, every wave walks its own tiles (wave-major over the grid, so the
    // waves that take one tile more are spread over all blocks); otherwise the waves of a block
    // walk groups of WPB tiles together, restaging at each window.
    const int first = ONE ? wave * (int)gridDim.x + (int)blockIdx.x : (int)blockIdx.x;
    const int lim = ONE ? (N + 15) / 16 : ngroups;
    const int step = ONE ? WPB * (int)gridDim.x : (int)gridDim.x;
    for (int it = first; it < lim; it += step) {
        const int r0 = (ONE ? it : it * WPB + wave) * 16;   // the tile's first row, uniform over the wave
        const int row = r0 + n;
        // the tile's rows past N repeat row N - 1 (a block's last group of tiles may start past N)
        const int rb = min(r0, N - 1), rmax = max(N - 1 - r0, 0);
        const u32x4* cb = codes + (size_t)rb * CH;
        const uint16_t* sb = scales + (size_t)rb * G;
        const uint16_t* bb = biases + (size_t)rb * G;

        float acc[MI][SUP / 2];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int j = 0; j < SUP / 2; ++j) acc[mi][j] = 0.0f;

        // Super-steps in pairs, each loading the next while it computes; both loads of a pair are
        // unconditional (a load used only under a branch is sunk into it and then waited for at
        // once). A pair runs while its second super-step exists (the first is then whole; the
        // second may be partial), and an odd last super-step runs after the loop on the set
        // already loaded.
        SupRegs la, lb;
        u32x4 tq[3];
        if constexpr (SBT) load_tile_sb(tq, sb, bb, G, lane);
        load_sup<SBT>(la, cb, sb, bb, rmax, 0, g, n, CH, G);
        if constexpr (SBT) {
            // the previous tile's reads of the block come first in the wave's LDS order
            asm volatile("" ::: "memory");
            store_tile_sb(tq, tw + TR_CODES, G, lane);
            __builtin_amdgcn_wave_barrier();
            asm volatile("" ::: "memory");
        }
        int w0 = ONE ? 0 : -W;
        int c0 = 0;
#pragma unroll 1
        for (; c0 + SUP < CH; c0 += 2 * SUP) {
            if (!ONE && c0 >= w0 + W) {          // the next staging window (only when K does not fit)
                w0 = c0;
                stage_window<MR>(xs, sps, x, m0, mr, K, CH, w0, W);
            }
            load_sup<SBT>(lb, cb, sb, bb, rmax, c0 + SUP, g, n, CH, G);
            run_sup<MI, false, SBT>(la, xs + (size_t)(c0 - w0) / 2 * MI * AB_DW, sps + (c0 - w0) / 2, WG, acc, c0, CH, G,
                                    lane, tw);
            load_sup<SBT>(la, cb, sb, bb, rmax, c0 + 2 * SUP, g, n, CH, G);
            run_sup<MI, !FULL, SBT>(lb, xs + (size_t)(c0 + SUP - w0) / 2 * MI * AB_DW, sps + (c0 + SUP - w0) / 2, WG,
                                    acc, c0 + SUP, CH, G, lane, tw);
        }
        if (c0 < CH) {                           // uniform: one (possibly partial) super-step left
            if (!ONE && c0 >= w0 + W) {
                w0 = c0;
                stage_window<MR>(xs, sps, x, m0, mr, K, CH, w0, W);
            }
            run_sup<MI, !FULL, SBT>(la, xs + (size_t)(c0 - w0) / 2 * MI * AB_DW, sps + (c0 - w0) / 2, WG, acc, c0, CH, G,
                                    lane, tw);
        }

        // the chains meet in the M=1 kernels' butterfly order; lane (n, g) holds activation row
        // 4 mi + g of weight row n
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const float v = ((acc[mi][0] + acc[mi][1]) + (acc[mi][2] + acc[mi][3])) +
                            ((acc[mi][4] + acc[mi][5]) + (acc[mi][6] + acc[mi][7]));
            const int ar = 4 * mi + g;
            if (ar < mr && row < N) {
                const size_t o = (size_t)(m0 + ar) * N + row;
                if constexpr (F32OUT) reinterpret_cast<float*>(y)[o] = v;
                else reinterpret_cast<_Float16*>(y)[o] = (_Float16)v;
            }
            if constexpr (ARGMAX)
                if (row < N && better(v, row, best_v[mi], best_i[mi])) {
                    best_v[mi] = v;
                    best_i[mi] = row;
                }
        }
    }

    if constexpr (ARGMAX) {
        __shared__ float bv_s[MR][WPB];
        __shared__ int bi_s[MR][WPB];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            float bv = best_v[mi];
            int bi = best_i[mi];
            best_step<DPP_XOR1>(bv, bi);          // over the 16 weight rows of the 16-lane row
            best_step<DPP_XOR2>(bv, bi);
            best_step<DPP_HALF_MIRROR>(bv, bi);
            best_step<DPP_MIRROR>(bv, bi);
            if (n == 0) {
                bv_s[4 * mi + g][wave] = bv;
                bi_s[4 * mi + g][wave] = bi;
            }
        }
        __syncthreads();
        if (t < mr) {
            float bv = bv_s[t][0];
            int bi = bi_s[t][0];
            for (int w = 1; w < WPB; ++w)
                if (better(bv_s[t][w], bi_s[t][w], bv, bi)) { bv = bv_s[t][w]; bi = bi_s[t][w]; }
            part_v[(size_t)(m0 + t) * gridDim.x + blockIdx.x] = bv;     // [act row][block], as the
            part_i[(size_t)(m0 + t) * gridDim.x + blockIdx.x] = bi;     // final reduction reads them
        }
    }
}

// Dynamic LDS above 64 KiB must be allowed once per kernel and device.
template <int MI, bool F32OUT, bool ARGMAX, bool FULL, bool ONE, bool SBT>
hipError_t allow_lds(size_t lds) {
    static unsigned long long configured = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipGetLastError();
    const unsigned long long bit = 1ull << (dev & 63);
    if (__atomic_load_n(&configured, __ATOMIC_ACQUIRE) & bit) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&k_gemv_rows<MI, F32OUT, ARGMAX, FULL, ONE, SBT>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e == hipSuccess) __atomic_fetch_or(&configured, bit, __ATOMIC_RELEASE);
    return e;
}

template <int MI, bool FULL, bool ONE, bool SBT>
hipError_t launch_rows_full(bool f32, bool am, dim3 g, size_t lds, hipStream_t s, const u32x4* c, const uint16_t* sc,
                            const uint16_t* bi, const _Float16* x, int m0, int mr, int N, int K, void* y, float* pv,
                            int* pi) {
    const dim3 b(THREADS);
    const hipError_t e = f32 && am ? allow_lds<MI, true, true, FULL, ONE, SBT>(lds)
                         : f32     ? allow_lds<MI, true, false, FULL, ONE, SBT>(lds)
                         : am      ? allow_lds<MI, false, true, FULL, ONE, SBT>(lds)
                                   : allow_lds<MI, false, false, FULL, ONE, SBT>(lds);
    if (e != hipSuccess) return e;
    if (f32 && am)
        hipLaunchKernelGGL((k_gemv_rows<MI, true, true, FULL, ONE, SBT>), g, b, lds, s, c, sc, bi, x, m0, mr, N, K, y, pv, pi);
    else if (f32)
        hipLaunchKernelGGL((k_gemv_rows<MI, true, false, FULL, ONE, SBT>), g, b, lds, s, c, sc, bi, x, m0, mr, N, K, y, pv, pi);
    else if (am)
        hipLaunchKernelGGL((k_gemv_rows<MI, false, true, FULL, ONE, SBT>), g, b, lds, s, c, sc, bi, x, m0, mr, N, K, y, pv, pi);
    else
        hipLaunchKernelGGL((k_gemv_rows<MI, false, false, FULL, ONE, SBT>), g, b, lds, s, c, sc, bi, x, m0, mr, N, K, y, pv, pi);
    return hipGetLastError();
}

// Dynamic LDS a launch may take: the compute unit's 160 KiB less room for the static arrays.
constexpr size_t LDS_DYN_MAX = 160 * 1024 - 1024;

template <int MI>
hipError_t launch_rows_mi(bool f32, bool am, dim3 g, bool full, bool sb_aligned, hipStream_t s, const u32x4* c,
                          const uint16_t* sc, const uint16_t* bi, const _Float16* x, int m0, int mr, int N, int K,
                          void* y, float* pv, int* pi) {
    const int CH = K >> 5, G = K >> 6;
    const int W = window_chunks<4 * MI>(CH);
    const bool one = CH <= W;
    // the tile block: all of K in one window, whole tiles (N % 16 == 0), G even, 64 G bytes within
    // the region, 16-byte aligned scale and bias arrays, and the larger regions within the LDS
    const size_t lds_sbt = stage_bytes(4 * MI, W) + (size_t)WPB * region_bytes<true>();
    const bool sbt = one && N % 16 == 0 && G % 2 == 0 && 64 * G <= SBT_MAX && sb_aligned && lds_sbt <= LDS_DYN_MAX;
    if (sbt && full) return launch_rows_full<MI, true, true, true>(f32, am, g, lds_sbt, s, c, sc, bi, x, m0, mr, N, K, y, pv, pi);
    if (sbt) return launch_rows_full<MI, false, true, true>(f32, am, g, lds_sbt, s, c, sc, bi, x, m0, mr, N, K, y, pv, pi);
    const size_t lds = stage_bytes(4 * MI, W) + (size_t)WPB * region_bytes<false>();
    if (full && one) return launch_rows_full<MI, true, true, false>(f32, am, g, lds, s, c, sc, bi, x, m0, mr, N, K, y, pv, pi);
    if (full) return launch_rows_full<MI, true, false, false>(f32, am, g, lds, s, c, sc, bi, x, m0, mr, N, K, y, pv, pi);
    if (one) return launch_rows_full<MI, false, true, false>(f32, am, g, lds, s, c, sc, bi, x, m0, mr, N, K, y, pv, pi);
    return launch_rows_full<MI, false, false, false>(f32, am, g, lds, s, c, sc, bi, x, m0, mr, N, K, y, pv, pi);
}

}  // namespace

// Blocks of the multi-row GEMV for N weight rows (also the argmax partials per activation row):
// one resident block per compute unit.
int dhp_gemv_rows_blocks(int N, int cus) {
    const long groups = ((N + 15) / 16 + WPB - 1) / WPB;
    return (int)(groups < (long)cus ? groups : (long)cus);
}

int launch_gemv_rows(const dhp_int4* w, const void* x, int M, void* y, int y_f32, int32_t* argmax, void* ws,
                     size_t ws_part_stride, hipStream_t s, int cus) {
    const int N = w->rows, K = w->cols;
    const int nb = dhp_gemv_rows_blocks(N, cus);
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
    const bool full = K % 512 == 0;              // whole super-steps only
    const bool sb_aligned = ((uintptr_t)sc % 16) == 0 && ((uintptr_t)bi % 16) == 0;
    const dim3 g((unsigned)nb);
    // activation rows in passes of up to 8 (each pass streams the weights once)
    for (int m0 = 0; m0 < M; m0 += 8) {
        const int mr = M - m0 < 8 ? M - m0 : 8;
        hipError_t e;
        if (mr <= 4) e = launch_rows_mi<1>(y_f32, am, g, full, sb_aligned, s, c, sc, bi, xh, m0, mr, N, K, y, pv, pi);
        else e = launch_rows_mi<2>(y_f32, am, g, full, sb_aligned, s, c, sc, bi, xh, m0, mr, N, K, y, pv, pi);
        if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "gemv rows launch: %s", hipGetErrorString(e));
    }
    if (argmax) {
        const hipError_t e2 = launch_argmax_final(pv, pi, nb, M, argmax, s);
        if (e2 != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "argmax launch: %s", hipGetErrorString(e2));
    }
    return DHP_OK;
}
