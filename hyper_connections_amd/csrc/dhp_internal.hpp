// Internal declarations of libdecodehp: device helpers shared by the kernels, the
// per-device launch facts, and the launchers each kernel file exports to abi.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "decodehp.h"

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define DHP_DEV __device__ __forceinline__

// ------------------------------------------------------------------ bit helpers

DHP_DEV h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
DHP_DEV uint32_t h2_bits(h2 v) { return __builtin_bit_cast(uint32_t, v); }
DHP_DEV float bf16_to_f32(uint32_t b16) { return __builtin_bit_cast(float, b16 << 16); }
DHP_DEV float f16_to_f32(_Float16 h) { return (float)h; }

// Constants of the nibble unpack, held in VGPRs. An AND-OR with two 32-bit constants needs
// one of them in a register (one literal per VOP3 instruction); the empty asm hides their values
// so the compiler keeps them in registers and emits a single v_and_or_b32 per pair of codes
// instead of a separate AND and OR. Create once per kernel, outside loops.
struct NibConsts {
    uint32_t lo, hi, magic;
};
DHP_DEV NibConsts nib_consts() {
    NibConsts k{0x000F000Fu, 0x00F000F0u, 0x64006400u};
    asm("" : "+v"(k.lo), "+v"(k.hi), "+v"(k.magic));
    return k;
}

// Eight INT4 codes k0..k7 of one 32-bit word (byte j holds k=2j low, k=2j+1 high) become
// four exact fp16 pairs in the order (k0,k4) (k1,k5) (k2,k6) (k3,k7).
//
// A nibble OR-ed into the mantissa of fp16 1024.0 (0x6400, ulp 1) gives 1024 + q exactly;
// a nibble sitting four bits higher gives 1024 + 16 q, and (1024 + 16 q) / 16 - 64 = q.
// Both halves of a 32-bit word are handled at once, so one AND-OR makes two codes.
DHP_DEV void unpack8(uint32_t w, h2 q[4], const NibConsts& k) {
    const uint32_t w8 = w >> 8;
    const h2 c1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
    const h2 c64 = {(_Float16)64.0f, (_Float16)64.0f};
    const h2 c16th = {(_Float16)0.0625f, (_Float16)0.0625f};
    q[0] = as_h2((w & k.lo) | k.magic) - c1024;
    q[1] = __builtin_elementwise_fma(as_h2((w & k.hi) | k.magic), c16th, -c64);
    q[2] = as_h2((w8 & k.lo) | k.magic) - c1024;
    q[3] = __builtin_elementwise_fma(as_h2((w8 & k.hi) | k.magic), c16th, -c64);
}

// Eight consecutive fp16 activations (as four 32-bit words, x0x1 x2x3 x4x5 x6x7) rearranged
// into the pair order unpack8 produces: (x0,x4) (x1,x5) (x2,x6) (x3,x7).
DHP_DEV void permute8(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3, h2 out[4]) {
    out[0] = as_h2((d0 & 0xFFFFu) | (d2 << 16));
    out[1] = as_h2((d0 >> 16) | (d2 & 0xFFFF0000u));
    out[2] = as_h2((d1 & 0xFFFFu) | (d3 << 16));
    out[3] = as_h2((d1 >> 16) | (d3 & 0xFFFF0000u));
}

// Offset form of the 32-code dot product. Every code is moved four bits into the mantissa of
// an fp16 whose exponent field is that of 1024 (mantissa ulp 1), so each half reads
// t = 1024 + 16 q exactly: the pair (k1, k5) of a word is already there (bits 4-7 and 20-23),
// the pairs (k0, k4), (k2, k6), (k3, k7) need the word shifted by 4 left, 4 right or 8 right
// first. One AND-OR per pair, three shifts per word: 11 VALU per 8 codes with the four dot2
// (the exact unpack takes 13). Then
//     sum_k t_k x_k = 16 sum_k q_k x_k + 1024 sum_k x_k,
// so a dot whose fp32 accumulator starts at -1024 sum(x) ends at 16 q.x. The running sum
// carries magnitudes ~64 times those of q.x (the ratio of 1024 to 16), so its absolute rounding
// error grows with |x|; with the nibble in the low bits (t = 1024 + q) the ratio would be 1024
// and the error sixteen times larger. Callers keep the factor 16 on both halves of the affine
// form (s * dot + b * 16 sum(x)) and scale the finished row by 1/16, exact in binary.
DHP_DEV void unpack8_off(uint32_t w, h2 t[4], const NibConsts& k) {
    t[0] = as_h2(((w << 4) & k.hi) | k.magic);   // (k0, k4)
    t[1] = as_h2((w & k.hi) | k.magic);          // (k1, k5)
    t[2] = as_h2(((w >> 4) & k.hi) | k.magic);   // (k2, k6)
    t[3] = as_h2(((w >> 8) & k.hi) | k.magic);   // (k3, k7)
}

// 16 * (q . x) over one 32-code chunk: c holds the codes (16 bytes), xp the 16 permuted
// activation pairs, neg_corr = -1024 * (their sum).
DHP_DEV float dot32_off(const u32x4 c, const h2* xp, float neg_corr, const NibConsts& k) {
    float d = neg_corr;
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h2 t[4];
        unpack8_off(w[i], t, k);
        d = __builtin_amdgcn_fdot2(t[0], xp[4 * i], d, false);
        d = __builtin_amdgcn_fdot2(t[1], xp[4 * i + 1], d, false);
        d = __builtin_amdgcn_fdot2(t[2], xp[4 * i + 2], d, false);
        d = __builtin_amdgcn_fdot2(t[3], xp[4 * i + 3], d, false);
    }
    return d;
}

// 32 fp16 activations (four 16-byte words, k order) as 16 permuted pairs; returns 16 times their
// fp32 sum (the factor of the group bias in the offset form) and sets neg_corr = -1024 * sum.
DHP_DEV float x32_off_from(const u32x4 (&v)[4], h2* xp, float& neg_corr) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4 u = v[i];
        permute8(u.x, u.y, u.z, u.w, xp + 4 * i);
        const h2 a = as_h2(u.x), b = as_h2(u.y), c = as_h2(u.z), d = as_h2(u.w);
        s += (((float)a.x + (float)a.y) + ((float)b.x + (float)b.y)) +
             (((float)c.x + (float)c.y) + ((float)d.x + (float)d.y));
    }
    neg_corr = -1024.0f * s;
    return 16.0f * s;
}

// The same for the 32 activations at p (16-byte aligned).
DHP_DEV float load_x32_off(const _Float16* p, h2* xp, float& neg_corr) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
    const u32x4 v[4] = {q[0], q[1], q[2], q[3]};
    return x32_off_from(v, xp, neg_corr);
}

// sum over 32 codes of q * x for fp32 activations x[0..31] (contiguous k order).
DHP_DEV float dot32_f32(const u32x4 c, const float* x) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    float d = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = w[i] & 0x0F0F0F0Fu;          // k = 8i + 0, 2, 4, 6
        const uint32_t hi = (w[i] >> 4) & 0x0F0F0F0Fu;   // k = 8i + 1, 3, 5, 7
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            d = __builtin_fmaf((float)((lo >> (8 * b)) & 0xFFu), x[8 * i + 2 * b], d);
            d = __builtin_fmaf((float)((hi >> (8 * b)) & 0xFFu), x[8 * i + 2 * b + 1], d);
        }
    }
    return d;
}

// ------------------------------------------------------------------ exact group sums (the GEMV)
//
// The GEMV forms each 64-code group's dot on integers, so the group's value is exact and does
// not depend on the order of its products: the vector-ALU kernels (v_dot4_i32_i8) and the
// matrix-core multi-row kernel (v_mfma_i32_16x16x64_i8) produce the same bits. For one
// activation row and one group of 64 activations (the group of one scale and one bias):
//   e    = exponent of the group's largest |x| (0 for an all-zero group),
//   X_k  = rint(x_k * 2^(20 - e)); |X_k| < 2^21, exact for every x_k within 2^10 of the largest,
//   X_k  = P2 * 2^14 + P1 * 2^7 + P0 with P0, P1 in 0..127 and P2 in -128..127 (int8 pieces),
//   D    = sum_k q_k X_k over the group's 4-bit codes (|D| < 64 * 15 * 2^21 < 2^31: int32, exact),
//   the group's step of its chain: acc = fma(fma(s, float(D), b * float(sum_k X_k)), 2^(e-20), acc).
// The piece word (p, h, w, r) holds the bytes of X_p at k = 32h + 8w + r + {0, 2, 4, 6} (piece p,
// chunk h of the group, code word w of the chunk, parity r: the order in which unpack_i8 lays out
// the codes of word w). The M=1 kernels stage a group as XG_DW words: (p, h, w, r) at
// 16p + 4w + 2h + r, then float(sum_k X_k) and 2^(e-20) at words 48 and 49, two words of padding.
constexpr int XG_DW = 52;

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

DHP_DEV uint32_t pack_bytes(int a, int b, int c, int d) {
    return ((uint32_t)a & 0xFFu) | (((uint32_t)b & 0xFFu) << 8) | (((uint32_t)c & 0xFFu) << 16) | ((uint32_t)d << 24);
}

// Lanes 8t .. 8t+7 (all active, aligned to 8) convert one group: lane i = 0..7 reads k = 8i .. 8i+7
// of xg (the group's 64 fp16 activations, 16-byte aligned), i.e. chunk h = i / 4, code word
// w = i % 4, and writes its six piece words (p, h, w, r) at d[p * pstride + r] (d 8-byte aligned).
// Every lane of the eight returns (float(sum_k X_k), 2^(e-20)). The activations must be finite.
DHP_DEV float2 xg_stage_octet(const _Float16* __restrict__ xg, int i, uint32_t* __restrict__ d, int pstride) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(xg + 8 * i);
    // largest magnitude: fp16 magnitude bits order like the magnitudes
    const u16x2 m2 = __builtin_elementwise_max(
        __builtin_elementwise_max(__builtin_bit_cast(u16x2, v.x & 0x7FFF7FFFu), __builtin_bit_cast(u16x2, v.y & 0x7FFF7FFFu)),
        __builtin_elementwise_max(__builtin_bit_cast(u16x2, v.z & 0x7FFF7FFFu), __builtin_bit_cast(u16x2, v.w & 0x7FFF7FFFu)));
    int m = max((int)m2.x, (int)m2.y);
    m = max(m, __builtin_amdgcn_update_dpp(0, m, 0xB1, 0xF, 0xF, false));    // quad lanes 1,0,3,2
    m = max(m, __builtin_amdgcn_update_dpp(0, m, 0x4E, 0xF, 0xF, false));    // quad lanes 2,3,0,1
    m = max(m, __builtin_amdgcn_update_dpp(0, m, 0x141, 0xF, 0xF, false));   // reversed within 8 lanes
    const float mf = (float)__builtin_bit_cast(_Float16, (uint16_t)m);
    const int eb = (int)(__builtin_bit_cast(uint32_t, mf) >> 23);            // biased; 0 only for mf = 0
    const int e = eb ? eb - 127 : 0;
    const float sc = __builtin_bit_cast(float, (uint32_t)(147 - e) << 23);    // 2^(20 - e)
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
    int X[8];
    int sx = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const h2 p = as_h2(wv[u]);
        X[2 * u] = (int)__builtin_rintf((float)p.x * sc);
        X[2 * u + 1] = (int)__builtin_rintf((float)p.y * sc);
        sx += X[2 * u] + X[2 * u + 1];
    }
    sx += __builtin_amdgcn_update_dpp(0, sx, 0xB1, 0xF, 0xF, false);
    sx += __builtin_amdgcn_update_dpp(0, sx, 0x4E, 0xF, 0xF, false);
    sx += __builtin_amdgcn_update_dpp(0, sx, 0x141, 0xF, 0xF, false);
    uint32_t w[3][2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int a = X[r], b = X[2 + r], c = X[4 + r], e8 = X[6 + r];
        w[0][r] = pack_bytes(a & 127, b & 127, c & 127, e8 & 127);
        w[1][r] = pack_bytes((a >> 7) & 127, (b >> 7) & 127, (c >> 7) & 127, (e8 >> 7) & 127);
        w[2][r] = pack_bytes(a >> 14, b >> 14, c >> 14, e8 >> 14);
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) *reinterpret_cast<uint2*>(d + p * pstride) = uint2{w[p][0], w[p][1]};
    return float2{(float)sx, __builtin_bit_cast(float, (uint32_t)(107 + e) << 23)};   // 2^(e - 20)
}

// The codes of one code word (k = 8w .. 8w+7 of a chunk, byte j: k = 2j low nibble, 2j + 1 high)
// as int8: lo = k 0, 2, 4, 6 and hi = k 1, 3, 5, 7 of the word.
DHP_DEV void unpack_i8(uint32_t w, uint32_t& lo, uint32_t& hi) {
    lo = w & 0x0F0F0F0Fu;
    hi = (w >> 4) & 0x0F0F0F0Fu;
}

// One chunk's share of its group's exact sum: c the chunk's four code words, xq its 24 piece words
// (word 8p + 2w + r = piece word (p, h, w, r) of the chunk's group).
DHP_DEV int dot32_i8(const u32x4 c, const uint32_t* xq) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    int s0 = 0, s1 = 0, s2 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t lo, hi;
        unpack_i8(w[i], lo, hi);
        s0 = __builtin_amdgcn_sdot4((int)lo, (int)xq[2 * i], s0, false);
        s0 = __builtin_amdgcn_sdot4((int)hi, (int)xq[2 * i + 1], s0, false);
        s1 = __builtin_amdgcn_sdot4((int)lo, (int)xq[8 + 2 * i], s1, false);
        s1 = __builtin_amdgcn_sdot4((int)hi, (int)xq[9 + 2 * i], s1, false);
        s2 = __builtin_amdgcn_sdot4((int)lo, (int)xq[16 + 2 * i], s2, false);
        s2 = __builtin_amdgcn_sdot4((int)hi, (int)xq[17 + 2 * i], s2, false);
    }
    return s2 * 16384 + s1 * 128 + s0;
}

// One group's step of its chain (the same operations in every kernel; the empty asm keeps the
// bias product rounded on its own, so no kernel contracts it into a fused operation).
DHP_DEV float xg_group_acc(float acc, int d, float s, float b, float sx, float pe) {
    float bs = b * sx;
    asm volatile("" : "+v"(bs));
    return __builtin_fmaf(__builtin_fmaf(s, (float)d, bs), pe, acc);
}

// Cross-lane data movement with DPP (VALU-speed, no LDS round trip). Within each 16-lane
// row: XOR1 and XOR2 are quad permutes, then the half-row and row mirrors pair lanes across
// 4- and 8-lane boundaries. After the levels for width W every lane of an aligned W-lane
// group holds the same combination (addition is commutative, so partners agree bitwise).
constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // reverse within each 8 lanes
constexpr int DPP_MIRROR = 0x140;       // reverse within each 16 lanes

template <int CTRL>
DHP_DEV float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
DHP_DEV int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
DHP_DEV float readlane_f(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over aligned groups of W lanes (W in 2, 4, 8, 16, 64), starting at level FROM (a group
// of FROM lanes already holds equal values). W = 64 returns the wave total, uniform.
template <int W, int FROM = 1>
DHP_DEV float group_sum(float v) {
    static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16 || W == 64, "group width");
    if constexpr (FROM <= 1 && W >= 2) v += dpp_f<DPP_XOR1>(v);
    if constexpr (FROM <= 2 && W >= 4) v += dpp_f<DPP_XOR2>(v);
    if constexpr (FROM <= 4 && W >= 8) v += dpp_f<DPP_HALF_MIRROR>(v);
    if constexpr (FROM <= 8 && W >= 16) v += dpp_f<DPP_MIRROR>(v);
    if constexpr (W == 64)
        v = (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
    return v;
}

// The inject's add for a pair of residual values: fp16(fp32 fma(out, w, raw)). The empty asm
// keeps the fp32 result, so the compiler cannot merge the fma and the conversion into one
// mixed-precision fma that rounds once to fp16: that instruction gives another value when the
// fp32 result sits on an fp16 rounding midpoint, and every kernel that forms an inject must
// produce the same bits.
DHP_DEV h2 inject_pair(h2 raw, h2 out, float w) {
    float a = __builtin_fmaf((float)out.x, w, (float)raw.x);
    float b = __builtin_fmaf((float)out.y, w, (float)raw.y);
    asm volatile("" : "+v"(a), "+v"(b));
    return h2{(_Float16)a, (_Float16)b};
}

DHP_DEV float silu_f(float z) { return z / (1.0f + __expf(-z)); }
DHP_DEV float sigmoid_f(float z) { return 1.0f / (1.0f + __expf(-z)); }

// Argmax order: larger value first, lower index first among equal values.
DHP_DEV bool better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

template <int CTRL>
DHP_DEV void best_step(float& v, int& i) {
    const float ov = dpp_f<CTRL>(v);
    const int oi = dpp_i<CTRL>(i);
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
}

// Wave-wide best (value, index); every lane returns the same pair.
DHP_DEV void wave_best(float& v, int& i) {
    best_step<DPP_XOR1>(v, i);
    best_step<DPP_XOR2>(v, i);
    best_step<DPP_HALF_MIRROR>(v, i);
    best_step<DPP_MIRROR>(v, i);
    float bv = readlane_f(v, 0);
    int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 16; r < 64; r += 16) {
        const float ov = readlane_f(v, r);
        const int oi = __builtin_amdgcn_readlane(i, r);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    v = bv;
    i = bi;
}

// ------------------------------------------------------------------ host side

struct DeviceFacts {
    int device;
    int cus;
};

// Facts about the current device, cached per device. Returns false (and sets the error)
// when there is no usable gfx950 device.
bool dhp_current_device(DeviceFacts* out);
int dhp_fail(int code, const char* fmt, ...);

// Launchers (validation already done by abi.hip).
int launch_gemv_m1(const dhp_int4* w, const void* x, void* y, int y_f32, int32_t* argmax,
                   void* ws, hipStream_t s, const DeviceFacts& dev);
int launch_hc_read(const void* raw, const void* gamma, int C, int H, float eps, const dhp_int4* down,
                   const dhp_int4* up, const dhp_int4* inject, void* mixed, float* inject_w,
                   void* ws, hipStream_t s);
int launch_hc_inject(void* wide, const void* out, const float* w, int C, int H, hipStream_t s);
int launch_hc_inject_read(const void* prev, const void* out, const float* w, void* hidden, const void* gamma, int C,
                          int H, float eps, const dhp_int4* down, const dhp_int4* up, const dhp_int4* inject,
                          void* mixed, float* inject_w, void* ws, hipStream_t s);
int launch_moe(const void* x, const dhp_router* router, const void* sgate_row,
               const dhp_int4_experts* gate, const dhp_int4_experts* up, const dhp_int4_experts* down,
               const dhp_int4* sg, const dhp_int4* su, const dhp_int4* sd, int top_k, int boundary,
               void* out, int32_t* ids, float* weights, void* ws, hipStream_t s);
int launch_moe_prefill(const void* x, int m, const dhp_router* router, const void* sgate_row,
                       const dhp_int4_experts* gate, const dhp_int4_experts* up, const dhp_int4_experts* down,
                       const dhp_int4* sg, const dhp_int4* su, const dhp_int4* sd, int top_k, int boundary,
                       void* out, int32_t* ids, float* weights, void* ws, hipStream_t s);
size_t dhp_moe_prefill_ws(int32_t m, int32_t n_experts, int32_t top_k, int32_t inter, int32_t hidden);
size_t dhp_hc_read_batched_ws(int32_t m, int32_t C, int32_t H, int32_t R);
int launch_hc_read_batched(const void* raw, int m, const void* gamma, int C, int H, float eps, const dhp_int4* down,
                           const dhp_int4* up, const dhp_int4* inject, void* mixed, float* inject_w, void* ws,
                           hipStream_t s);
int launch_hc_inject_batched(void* wide, int m, const void* out, const float* w, int C, int H, hipStream_t s);
size_t dhp_argmax_part_stride(int32_t n_rows, int32_t m);
int launch_gemm_mfma_splitk(const dhp_int4* w, const void* x, int M, float* y_partials, int splits, hipStream_t s,
                            const dhp_int4* w2 = nullptr, float* y2_partials = nullptr);
bool dhp_gemm_upmix_fits(const dhp_int4* w, int M, int C, int H);
int launch_gemm_mfma_upmix(const dhp_int4* w, const void* x, int M, const void* normed, void* mixed, int H,
                           hipStream_t s);
int launch_gemm_mfma(const dhp_int4* w, const void* x, int M, void* y, int y_f32, int32_t* argmax,
                     void* ws, size_t ws_part_stride, hipStream_t s);
hipError_t launch_argmax_final(const float* pv, const int* pi, int nparts, int m, int32_t* out, hipStream_t s);
bool dhp_gemv_mfma16_fits(const dhp_int4* w, int M);
int launch_gemv_rows(const dhp_int4* w, const void* x, int M, void* y, int y_f32, int32_t* argmax, void* ws,
                     size_t ws_part_stride, hipStream_t s, int cus);
int launch_gemv_mfma16(const dhp_int4* w, const void* x, int M, void* y, int y_f32, int32_t* argmax, void* ws,
                       size_t ws_part_stride, hipStream_t s, int cus);
