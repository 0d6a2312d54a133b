// Routed mixture-of-experts decode for one token: router GEMV, on-device top-k with softmax
// over the selected experts, phase 1 (gate/up GEMV + silu(gate)*up), phase 2 (down GEMV +
// weighted k-way reduce) and the sigmoid-gated shared expert.
//
// "src/families/qwen4/mod.rs" (turbospark-runtime 0.3.0), section MoE; "src/families/qwen/
// state.rs", struct RealQwenState (fp32 router logits, unit router scales, gated shared
// expert); "src/real_forward.rs", module doc (phase-1 gate_up_act and phase-2 down_reduce
// kernels, with the router logits read back to the host for top-k between two command
// buffers). Here nothing returns to the host: three kernels on one stream.
//
//  k_moe_router : one wave per router row (fp32 logits into the workspace), one wave for the
//                 shared expert's scalar gate logit, and quarter-waves running the shared
//                 expert's gate/up pairs, which need no routing decision.
//  k_moe_phase1 : every block re-derives the top-k from the E logits (a handful of wave
//                 maxima, cheaper than another launch), then its quarter-waves run one
//                 (selected expert, row) pair each: gate and up rows against register-resident
//                 activations, act = silu(gate) * up in fp32. Block 0 writes ids and weights.
//  k_moe_phase2 : 16 lanes per output element walk the down rows of the selected experts and
//                 the shared expert (K = inter) against the fp32 activations staged in LDS,
//                 eight waves splitting the experts, each expert's partial weighted by its
//                 softmax weight; the shared part is scaled by sigmoid(g) and both halves meet
//                 in one fp16 rounding.
#include "dhp_internal.hpp"

#include <math.h>
#include <limits.h>

// The batched (chunk of M tokens) kernels below reproduce the decode kernels' results bit for
// bit, so every product and sum here is spelled out: no multiply and add may be fused unless
// written as an fma.
#pragma clang fp contract(off)

namespace {

constexpr int LPR = 16;
constexpr int MAX_E = 1024;

struct MoeArgs {
    const _Float16* x;
    const void* router;
    int router_kind;              // RK_BF16, RK_F32 or RK_I8
    const uint16_t* router_escale; // bf16 [hidden]: the router's per-element effective scale, or null
    const float* expert_scale;    // fp32 [E]: per-expert scale of the routing weights, or null
    const uint16_t* sgate_row;
    // routed experts: first tensor and byte strides
    const uint8_t* g_codes; const uint8_t* g_scales; const uint8_t* g_biases;
    const uint8_t* u_codes; const uint8_t* u_scales; const uint8_t* u_biases;
    const uint8_t* d_codes; const uint8_t* d_scales; const uint8_t* d_biases;
    long long gu_cstride, gu_sstride;     // gate and up share strides (same shapes)
    long long u_cstride, u_sstride;
    long long d_cstride, d_sstride;
    // shared expert
    const u32x4* sg_codes; const uint16_t* sg_scales; const uint16_t* sg_biases;
    const u32x4* su_codes; const uint16_t* su_scales; const uint16_t* su_biases;
    const u32x4* sd_codes; const uint16_t* sd_scales; const uint16_t* sd_biases;
    int E, hidden, inter, top_k, boundary;
    int M;             // tokens (1 for decode)
    int Epad;          // logits row pitch (batched: E rounded up to 4)
    float* logits;     // ws [M][Epad]
    float* gate_logit; // ws [M]
    float* act;        // ws [M][top_k + 1][inter]; slot top_k is the shared expert
    float* dsum;       // ws [M][top_k + 1][hidden] (batched only): each slot's down-row dots
    int32_t* route;    // ws [M][top_k + 1] (batched only): (token << 4 | slot), grouped by expert
    int32_t* items;    // ws [max items][4] (batched only): (expert, first route entry, count, 0)
    int32_t* nitems;   // ws [1] (batched only): work items in use
    u32x4* xraw;       // ws [M][4][hidden / 32] (decode: M = 1): each token's activations in the form of
                       // x32_off_from (16 permuted pairs per 32-value chunk, as 4 u32x4 planes)
    float2* xrsum;     // ws [M][hidden / 32] (decode: M = 1): per chunk, (16 * sum, -1024 * sum)
    _Float16* out;     // [M][hidden]
    int32_t* ids;      // [M][top_k]
    float* weights;    // [M][top_k]
};

// Registers of one (gate row, up row) pair for the 16-lane group whose lane index is j.
template <int CPL>
struct PairRegs {
    u32x4 cg[CPL], cu[CPL];
    uint32_t sg[CPL], bg[CPL], su[CPL], bu[CPL];
};

// Issue the code/scale/bias loads of gate row `row` and up row `row` (K = hidden = 512 * CPL).
template <int CPL>
DHP_DEV void load_pair(PairRegs<CPL>& p, const u32x4* gc, const uint16_t* gs, const uint16_t* gb,
                       const u32x4* uc, const uint16_t* us, const uint16_t* ub, int row, int j) {
    constexpr int CH = LPR * CPL;
    constexpr int G = CH / 2;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int ch = j + LPR * i;
        p.cg[i] = __builtin_nontemporal_load(gc + (size_t)row * CH + ch);
        p.cu[i] = __builtin_nontemporal_load(uc + (size_t)row * CH + ch);
        p.sg[i] = gs[(size_t)row * G + (ch >> 1)];
        p.bg[i] = gb[(size_t)row * G + (ch >> 1)];
        p.su[i] = us[(size_t)row * G + (ch >> 1)];
        p.bu[i] = ub[(size_t)row * G + (ch >> 1)];
    }
}

// silu(gate . x) * (up . x), the same value in every lane of the 16-lane group. The chunk dots
// use the offset code form (see dot32_off) with the activations' per-chunk corrections nc and
// sixteenfold sums xs; each finished dot is scaled back by 1/16 (exact).
// k_moep_phase1 repeats these operations in this order (reading its activations from LDS).
template <int CPL>
DHP_DEV float pair_act(const PairRegs<CPL>& p, const h2 (*xp)[16], const float* xs, const float* nc) {
    const NibConsts nk = nib_consts();
    float ag = 0.0f, au = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        ag = __builtin_fmaf(bf16_to_f32(p.sg[i]), dot32_off(p.cg[i], xp[i], nc[i], nk), ag);
        ag = __builtin_fmaf(bf16_to_f32(p.bg[i]), xs[i], ag);
        au = __builtin_fmaf(bf16_to_f32(p.su[i]), dot32_off(p.cu[i], xp[i], nc[i], nk), au);
        au = __builtin_fmaf(bf16_to_f32(p.bu[i]), xs[i], au);
    }
    ag = group_sum<LPR>(ag) * 0.0625f;
    au = group_sum<LPR>(au) * 0.0625f;
    return silu_f(ag) * au;
}

// fp32 dot of one router row of length hidden = 512 * CPL with the fp16 activations, one wave:
// lane l takes the row chunks l + 64 i (8 bf16 or 8 int8 values, or 4 fp32). With a per-element
// effective scale (the INT8 router kernel's, "src/families/qwen/state.rs", router_ones), each
// activation is multiplied by its scale first. The row's loads are issued on their own (a
// batched caller keeps the row and streams tokens past it); a row costs one memory round trip.
enum RouterKind { RK_BF16 = 0, RK_F32 = 1, RK_I8 = 2 };
template <int CPL, int KIND>
struct RouterRow {
    u32x4 w[KIND == RK_F32 ? 2 * CPL : CPL];   // bf16: 8 per chunk; fp32: 4 (as bits); int8: 8 in .x, .y
};
template <int CPL, bool SC>
struct RouterX {
    uint2 h[2 * CPL];      // 8-value chunks: chunk i = h[2i], h[2i+1]; fp32 rows: chunk i = h[i]
    uint2 e[SC ? 2 * CPL : 1];   // the effective scales, laid out like h (scaled routers only)
};
template <int CPL, int KIND>
DHP_DEV void router_row_load(RouterRow<CPL, KIND>& r, const void* row) {
    const int lane = threadIdx.x & 63;
    if constexpr (KIND != RK_I8) {
        const u32x4* p = static_cast<const u32x4*>(row);
#pragma unroll
        for (int i = 0; i < (KIND == RK_F32 ? 2 * CPL : CPL); ++i) r.w[i] = __builtin_nontemporal_load(p + lane + 64 * i);
    } else {
        typedef uint32_t u32x2n __attribute__((ext_vector_type(2)));
        const u32x2n* p = static_cast<const u32x2n*>(row);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const u32x2n q = __builtin_nontemporal_load(p + lane + 64 * i);
            r.w[i] = u32x4{q.x, q.y, 0u, 0u};
        }
    }
}
template <int CPL, int KIND, bool SC>
DHP_DEV void router_x_load(RouterX<CPL, SC>& v, const _Float16* x, const uint16_t* escale) {
    const int lane = threadIdx.x & 63;
    if constexpr (KIND != RK_F32) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const u32x4 q = *reinterpret_cast<const u32x4*>(x + 8 * (lane + 64 * i));
            v.h[2 * i] = uint2{q.x, q.y};
            v.h[2 * i + 1] = uint2{q.z, q.w};
            if constexpr (SC) {
                const u32x4 g = *reinterpret_cast<const u32x4*>(escale + 8 * (lane + 64 * i));
                v.e[2 * i] = uint2{g.x, g.y};
                v.e[2 * i + 1] = uint2{g.z, g.w};
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 2 * CPL; ++i) {
            v.h[i] = *reinterpret_cast<const uint2*>(x + 4 * (lane + 64 * i));
            if constexpr (SC) v.e[i] = *reinterpret_cast<const uint2*>(escale + 4 * (lane + 64 * i));
        }
    }
}
// The two activations of a packed fp16 pair, each times its bf16 scale when scaled.
template <bool SC>
DHP_DEV void x_pair(uint32_t xw, uint32_t ew, float& x0, float& x1) {
    const h2 xh = as_h2(xw);
    x0 = (float)xh.x;
    x1 = (float)xh.y;
    if constexpr (SC) {
        x0 = x0 * bf16_to_f32(ew & 0xFFFFu);
        x1 = x1 * bf16_to_f32(ew >> 16);
    }
}
template <int CPL, bool SC>
DHP_DEV uint32_t escale_word(const RouterX<CPL, SC>& v, int i, int half) {
    if constexpr (SC) return half ? v.e[i].y : v.e[i].x;
    else return 0u;
}
template <int CPL, int KIND, bool SC>
DHP_DEV float router_dot(const RouterRow<CPL, KIND>& r, const RouterX<CPL, SC>& v) {
    float acc = 0.0f;
    if constexpr (KIND == RK_BF16) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const uint32_t ww[4] = {r.w[i].x, r.w[i].y, r.w[i].z, r.w[i].w};
            const uint32_t xx[4] = {v.h[2 * i].x, v.h[2 * i].y, v.h[2 * i + 1].x, v.h[2 * i + 1].y};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float x0, x1;
                x_pair<SC>(xx[k], escale_word<CPL, SC>(v, 2 * i + (k >> 1), k & 1), x0, x1);
                acc = __builtin_fmaf(bf16_to_f32(ww[k] & 0xFFFFu), x0, acc);
                acc = __builtin_fmaf(bf16_to_f32(ww[k] >> 16), x1, acc);
            }
        }
    } else if constexpr (KIND == RK_F32) {
#pragma unroll
        for (int i = 0; i < 2 * CPL; ++i) {
            const f4v wv = __builtin_bit_cast(f4v, r.w[i]);   // whole-vector cast
            float x0, x1, x2, x3;
            x_pair<SC>(v.h[i].x, escale_word<CPL, SC>(v, i, 0), x0, x1);
            x_pair<SC>(v.h[i].y, escale_word<CPL, SC>(v, i, 1), x2, x3);
            acc = __builtin_fmaf(wv.x, x0, acc);
            acc = __builtin_fmaf(wv.y, x1, acc);
            acc = __builtin_fmaf(wv.z, x2, acc);
            acc = __builtin_fmaf(wv.w, x3, acc);
        }
    } else {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const uint32_t ww[2] = {r.w[i].x, r.w[i].y};
            const uint32_t xx[4] = {v.h[2 * i].x, v.h[2 * i].y, v.h[2 * i + 1].x, v.h[2 * i + 1].y};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float x0, x1;
                x_pair<SC>(xx[k], escale_word<CPL, SC>(v, 2 * i + (k >> 1), k & 1), x0, x1);
                const uint32_t w = ww[k >> 1] >> (16 * (k & 1));      // codes of elements 2k, 2k+1
                acc = __builtin_fmaf((float)(int8_t)(w & 0xFFu), x0, acc);
                acc = __builtin_fmaf((float)(int8_t)((w >> 8) & 0xFFu), x1, acc);
            }
        }
    }
    return group_sum<64>(acc);
}
template <int CPL, int KIND, bool SC>
DHP_DEV float wave_row_dot_t(const void* row, const _Float16* x, const uint16_t* escale) {
    RouterRow<CPL, KIND> r;
    RouterX<CPL, SC> v;
    router_row_load<CPL, KIND>(r, row);
    router_x_load<CPL, KIND, SC>(v, x, escale);
    return router_dot<CPL, KIND, SC>(r, v);
}
template <int CPL>
DHP_DEV float wave_row_dot(const void* row, int kind, const _Float16* x, const uint16_t* escale) {
    if (kind == RK_BF16)
        return escale ? wave_row_dot_t<CPL, RK_BF16, true>(row, x, escale) : wave_row_dot_t<CPL, RK_BF16, false>(row, x, escale);
    if (kind == RK_F32)
        return escale ? wave_row_dot_t<CPL, RK_F32, true>(row, x, escale) : wave_row_dot_t<CPL, RK_F32, false>(row, x, escale);
    return escale ? wave_row_dot_t<CPL, RK_I8, true>(row, x, escale) : wave_row_dot_t<CPL, RK_I8, false>(row, x, escale);
}

// Bytes of one router row of this kind.
DHP_DEV size_t router_row_bytes(int kind, int hidden) {
    return (size_t)hidden * (kind == RK_F32 ? 4 : kind == RK_BF16 ? 2 : 1);
}

// Lane j's activations for pair_act: chunks j + 16 i in the offset form of load_x32_off.
template <int CPL>
DHP_DEV void load_x_regs(const _Float16* x, int j, h2 (*xp)[16], float* xs, float* nc) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) xs[i] = load_x32_off(x + (size_t)(j + LPR * i) * 32, xp[i], nc[i]);
}

// Blocks [0, E): router rows. Block E: shared gate logit. Then 4 shared pairs per block; the last
// ceil(hidden / 2048) blocks write the token's activations in the offset form pair_act multiplies
// (x32_off_from: the permuted pairs, 16 * sum and -1024 * sum per 32-value chunk) to the workspace,
// once per token, for phase 1 to load instead of converting them again in every wave.
template <int CPL>
__global__ __launch_bounds__(64) void k_moe_router(MoeArgs a) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int xb0 = a.E + 1 + (a.inter + 3) / 4;
    if (b >= xb0) {
        const int CH32 = a.hidden >> 5;
        const int c = (b - xb0) * 64 + lane;
        if (c < CH32) {
            const u32x4* src = reinterpret_cast<const u32x4*>(a.x + 32 * c);
            const u32x4 v[4] = {src[0], src[1], src[2], src[3]};
            h2 xp[16];
            float nc;
            const float xs = x32_off_from(v, xp, nc);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                a.xraw[(size_t)q * CH32 + c] = u32x4{h2_bits(xp[4 * q]), h2_bits(xp[4 * q + 1]),
                                                     h2_bits(xp[4 * q + 2]), h2_bits(xp[4 * q + 3])};
            a.xrsum[c] = float2{xs, nc};
        }
        return;
    }
    if (b < a.E) {
        const size_t rb = router_row_bytes(a.router_kind, a.hidden);
        const float v = wave_row_dot<CPL>(static_cast<const uint8_t*>(a.router) + rb * b, a.router_kind, a.x,
                                          a.router_escale);
        if (lane == 0) a.logits[b] = v;
        return;
    }
    if (b == a.E) {
        const float v = wave_row_dot<CPL>(a.sgate_row, RK_BF16, a.x, nullptr);
        if (lane == 0) a.gate_logit[0] = v;
        return;
    }
    const int j = lane % LPR;
    const int row = (b - a.E - 1) * 4 + lane / LPR;
    const bool live = row < a.inter;      // 16-lane groups share a row; all lanes stay for the DPP sums
    PairRegs<CPL> p;
    load_pair<CPL>(p, a.sg_codes, a.sg_scales, a.sg_biases, a.su_codes, a.su_scales, a.su_biases,
                   live ? row : 0, j);
    h2 xp[CPL][16];
    float xs[CPL], nc[CPL];
    load_x_regs<CPL>(a.x, j, xp, xs, nc);
    const float v = pair_act<CPL>(p, xp, xs, nc);
    if (j == 0 && live) a.act[(size_t)a.top_k * a.inter + row] = v;
}

// Top-k by one wave. Every logit becomes an unsigned word that orders like the float (a NaN
// ranks as -inf; -0 is folded into +0, they compare equal) and lane l holds the words of the
// PER consecutive experts l*PER + i, so a lower lane always means lower expert indices. Each
// round takes the wave-wide maximum word; the lowest lane holding it gives up its entry (the
// lowest index among equal words), and the next round starts over.
// Padding entries (e >= E) hold 0, below every real logit (the -inf word is 0x007FFFFF).
DHP_DEV uint32_t order_word(float l) {
    l = (l == l) ? l + 0.0f : -INFINITY;
    const uint32_t u = __builtin_bit_cast(uint32_t, l);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
DHP_DEV float order_word_value(uint32_t u) {
    return __builtin_bit_cast(float, (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Wave-wide maximum, in every lane: DPP within each 16-lane row, then the gfx950 row swap
// (odd rows against even rows) and half swap (upper 32 lanes against lower 32).
DHP_DEV uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)dpp_i<DPP_XOR1>((int)v));
    v = max(v, (uint32_t)dpp_i<DPP_XOR2>((int)v));
    v = max(v, (uint32_t)dpp_i<DPP_HALF_MIRROR>((int)v));
    v = max(v, (uint32_t)dpp_i<DPP_MIRROR>((int)v));
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max((uint32_t)r[0], (uint32_t)r[1]);
    const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max((uint32_t)h[0], (uint32_t)h[1]);
}

// The logits a lane ranks: PER consecutive ones from lane * PER, in whole 16-byte loads clamped
// to the last full vector (the buffer must be readable up to index 4 * ((E - 1) / 4) + 3).
template <int PER>
struct TopkIn {
    u32x4 v[PER / 4];
};
template <int PER>
DHP_DEV void topk_load(TopkIn<PER>& t, const float* logits, int E) {
    static_assert(PER % 4 == 0, "whole 16-byte loads");
    const int lane = threadIdx.x & 63;
    const int last4 = ((E - 1) >> 2) << 2;
#pragma unroll
    for (int q = 0; q < PER / 4; ++q)
        t.v[q] = *reinterpret_cast<const u32x4*>(logits + min(lane * PER + 4 * q, last4));
}

// The first `rounds` entries of the top-k of the E logits (E <= 64 * PER); every lane returns
// the same ids and values.
template <int PER>
DHP_DEV void wave_topk(TopkIn<PER>& t, int E, int rounds, int* ids, float* vals) {
    const int lane = threadIdx.x & 63;
    uint32_t w[PER];
    int ix[PER];
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint32_t u = t.v[q][c];
            asm volatile("" : "+v"(u));  // every element is live: the loads stay whole vectors
            w[4 * q + c] = order_word(__builtin_bit_cast(float, u));
        }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        w[i] = (lane * PER + i < E) ? w[i] : 0u;
        ix[i] = i;
    }
    if constexpr (PER <= 4) {
        // sort each lane's entries: adjacent exchanges on a strict comparison keep equal words
        // in index order
#pragma unroll
        for (int p = 0; p < PER - 1; ++p) {
#pragma unroll
            for (int q = 0; q < PER - 1 - p; ++q) {
                const bool sw = w[q + 1] > w[q];
                const uint32_t w0 = w[q], w1 = w[q + 1];
                const int i0 = ix[q], i1 = ix[q + 1];
                w[q] = sw ? w1 : w0;
                w[q + 1] = sw ? w0 : w1;
                ix[q] = sw ? i1 : i0;
                ix[q + 1] = sw ? i0 : i1;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < DHP_MOE_MAX_TOP_K; ++r) {
        if (r >= rounds) break;
        if constexpr (PER <= 4) {
            const uint32_t m = wave_max_u32(w[0]);
            const int wl = __builtin_ctzll(__builtin_amdgcn_ballot_w64(w[0] == m));
            ids[r] = wl * PER + __builtin_amdgcn_readlane(ix[0], wl);
            vals[r] = order_word_value(m);
            const bool mine = lane == wl;
#pragma unroll
            for (int q = 0; q < PER - 1; ++q) {
                w[q] = mine ? w[q + 1] : w[q];
                ix[q] = mine ? ix[q + 1] : ix[q];
            }
            w[PER - 1] = mine ? 0u : w[PER - 1];
        } else {
            uint32_t best = w[0];
#pragma unroll
            for (int i = 1; i < PER; ++i) best = max(best, w[i]);
            const uint32_t m = wave_max_u32(best);
            const int wl = __builtin_ctzll(__builtin_amdgcn_ballot_w64(best == m));
            int first = PER - 1;
#pragma unroll
            for (int i = PER - 2; i >= 0; --i) first = (w[i] == m) ? i : first;
            ids[r] = wl * PER + __builtin_amdgcn_readlane(first, wl);
            vals[r] = order_word_value(m);
            const bool mine = lane == wl;
#pragma unroll
            for (int i = 0; i < PER; ++i) w[i] = (mine && i == first) ? 0u : w[i];
        }
    }
}

// The selected ids (largest logit first) and the softmax over their logits, each weight times its
// expert's scale when a per-expert scale is given ("src/families/qwen/state.rs", per_expert_ones),
// by one thread.
DHP_DEV void publish_topk(const int* ids, const float* vals, int top_k, const float* expert_scale,
                          int32_t* out_ids, float* out_w) {
    float wt[DHP_MOE_MAX_TOP_K];
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < DHP_MOE_MAX_TOP_K; ++r) {
        wt[r] = (r < top_k) ? __expf(vals[r] - vals[0]) : 0.0f;
        sum += wt[r];
    }
#pragma unroll
    for (int r = 0; r < DHP_MOE_MAX_TOP_K; ++r) {
        if (r < top_k) {
            out_ids[r] = ids[r];
            const float w = wt[r] / sum;
            out_w[r] = expert_scale ? w * expert_scale[ids[r]] : w;
        }
    }
}

template <int CPL, int PER>
__global__ __launch_bounds__(64) void k_moe_phase1(MoeArgs a) {
    const int lane = threadIdx.x;
    const int j = lane % LPR;
    TopkIn<PER> tin;
    topk_load<PER>(tin, a.logits, a.E);    // the routing decision waits on these: issue first
    h2 xp[CPL][16];
    float xs[CPL], nc[CPL];
    {   // the activations in offset form, written by the router kernel; independent of routing
        const int CH32 = a.hidden >> 5;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = j + LPR * i;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 u = a.xraw[(size_t)q * CH32 + c];
                xp[i][4 * q] = as_h2(u.x);
                xp[i][4 * q + 1] = as_h2(u.y);
                xp[i][4 * q + 2] = as_h2(u.z);
                xp[i][4 * q + 3] = as_h2(u.w);
            }
            const float2 sn = a.xrsum[c];
            xs[i] = sn.x;
            nc[i] = sn.y;
        }
    }

    // a block only needs the ranks up to its last (slot, row) pair; block 0 also needs all
    // top_k of them for the softmax weights
    const int last_pair = min((int)blockIdx.x * 4 + 3, a.top_k * a.inter - 1);
    const int rounds = (blockIdx.x == 0) ? a.top_k : last_pair / a.inter + 1;
    int ids[DHP_MOE_MAX_TOP_K];
    float vals[DHP_MOE_MAX_TOP_K];
    wave_topk<PER>(tin, a.E, rounds, ids, vals);

    const int pair = blockIdx.x * 4 + lane / LPR;      // (slot, row) flattened
    const bool live = pair < a.top_k * a.inter;
    const int slot = live ? pair / a.inter : 0;
    const int row = live ? pair % a.inter : 0;
    int e = ids[0];
#pragma unroll
    for (int r = 1; r < DHP_MOE_MAX_TOP_K; ++r)
        if (r == slot) e = ids[r];
    const auto* gc = reinterpret_cast<const u32x4*>(a.g_codes + (size_t)e * a.gu_cstride);
    const auto* gs = reinterpret_cast<const uint16_t*>(a.g_scales + (size_t)e * a.gu_sstride);
    const auto* gb = reinterpret_cast<const uint16_t*>(a.g_biases + (size_t)e * a.gu_sstride);
    const auto* uc = reinterpret_cast<const u32x4*>(a.u_codes + (size_t)e * a.u_cstride);
    const auto* us = reinterpret_cast<const uint16_t*>(a.u_scales + (size_t)e * a.u_sstride);
    const auto* ub = reinterpret_cast<const uint16_t*>(a.u_biases + (size_t)e * a.u_sstride);
    PairRegs<CPL> p;
    load_pair<CPL>(p, gc, gs, gb, uc, us, ub, row, j);

    // block 0 publishes the ids and the softmax over the selected logits
    if (blockIdx.x == 0 && lane == 0) publish_topk(ids, vals, a.top_k, a.expert_scale, a.ids, a.weights);

    const float v = pair_act<CPL>(p, xp, xs, nc);
    if (j == 0 && live) a.act[(size_t)slot * a.inter + row] = v;
}

// Phase 2 pieces shared by the decode and batched kernels, so both compute every value the
// same way. down_part: lane j's share of RHN down rows against one slot's fp32 activations,
// chunks j + 16 i of K = inter (the 32 floats of chunk ch at act + ch * pitch): per chunk
// s * (codes . act) + b * sum(act). group_sum<LPR> of it is the slot's down-row dot.
template <int RHN, int CPLD>
DHP_DEV void down_part(float (&p)[RHN], const u32x4 (&c)[RHN][CPLD], const uint32_t (&sv)[RHN][CPLD],
                       const uint32_t (&bv)[RHN][CPLD], const float* act, int pitch, int j, int CH) {
#pragma unroll
    for (int r = 0; r < RHN; ++r) p[r] = 0.0f;
#pragma unroll
    for (int i = 0; i < CPLD; ++i) {
        const int ch = j + LPR * i;
        if (ch < CH) {
            const f4v* ap = reinterpret_cast<const f4v*>(act + ch * pitch);
            float av[32];
            float xs = 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const f4v u = ap[q];
                av[4 * q] = u.x; av[4 * q + 1] = u.y; av[4 * q + 2] = u.z; av[4 * q + 3] = u.w;
                xs += (u.x + u.y) + (u.z + u.w);
            }
#pragma unroll
            for (int r = 0; r < RHN; ++r) {
                const float d = dot32_f32(c[r][i], av);
                p[r] = __builtin_fmaf(bf16_to_f32(sv[r][i]), d, p[r]);
                p[r] = __builtin_fmaf(bf16_to_f32(bv[r][i]), xs, p[r]);
            }
        }
    }
}

// One output of the layer from its slots' down-row dots d[s * dstride] (slot top_k is the shared
// expert): routed = sum_j w_j d_j, one fma per slot in slot order, plus sigmoid(g) * shared;
// with the fp16 boundary both halves are rounded to fp16 before the add.
DHP_DEV float moe_combine(const float (&w)[DHP_MOE_MAX_TOP_K], const float* d, int dstride, int top_k,
                          float gate_logit, int boundary) {
    float rr = 0.0f;
#pragma unroll
    for (int s = 0; s < DHP_MOE_MAX_TOP_K; ++s)
        if (s < top_k) rr = __builtin_fmaf(w[s], d[s * dstride], rr);
    const float ss = d[top_k * dstride] * sigmoid_f(gate_logit);
    if (boundary) return (float)(_Float16)rr + (float)(_Float16)ss;
    return rr + ss;
}

// Phase 2. A block of P2W waves owns 4 * RH consecutive outputs h (16 lanes and RH outputs per
// 16-lane group, the same rows in every wave). Wave w takes expert slots w, w + P2W (slot top_k
// is the shared expert): its lanes issue every code, scale and bias load of those slots first,
// the block stages the fp32 activations in LDS meanwhile, then each lane reduces its own chunk
// (K = inter; lane j takes chunks j + 16 i) of each down row. Each slot's dot is summed over its
// 16 lanes and parked in LDS; the outputs are combined from those in slot order. One output row
// per 16-lane group and eight waves measured fastest on the top-8 layer (16.7 us per call
// against 18.9 us with two rows and four waves; more rows per group or 12 waves were slower):
// more, smaller blocks put more independent loads in flight. A row's arithmetic does not depend
// on this grouping.
constexpr int RH = 1;
constexpr int P2W = 8;                 // waves per block
constexpr int NSLOT = DHP_MOE_MAX_TOP_K + 1;
constexpr int SLOTS_PER_WAVE = (NSLOT + P2W - 1) / P2W;
constexpr int ACT_PITCH = 36;          // floats per staged 32-float activation chunk

template <int CPLD>
__global__ __launch_bounds__(64 * P2W) void k_moe_phase2(MoeArgs a) {
    extern __shared__ float lds_act[];     // [(top_k + 1) * inter / 32][ACT_PITCH]
    __shared__ float dpart[NSLOT][4 * RH]; // [slot][16-lane group * RH + r]
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int j = lane % LPR;
    const int nslot = a.top_k + 1;
    const int CH = a.inter >> 5;
    const int G = a.inter >> 6;
    const int h0 = (blockIdx.x * 4 + lane / LPR) * RH;

    // the routing weights and the shared gate logit are read up front, with the expert ids
    float w[DHP_MOE_MAX_TOP_K];
#pragma unroll
    for (int s = 0; s < DHP_MOE_MAX_TOP_K; ++s) w[s] = a.weights[min(s, a.top_k - 1)];
    const float gate_logit = a.gate_logit[0];

    u32x4 c[SLOTS_PER_WAVE][RH][CPLD];
    uint32_t sv[SLOTS_PER_WAVE][RH][CPLD], bv[SLOTS_PER_WAVE][RH][CPLD];
#pragma unroll
    for (int t = 0; t < SLOTS_PER_WAVE; ++t) {
        const int slot = wave + P2W * t;
        if (slot < nslot) {
            const u32x4* dc;
            const uint16_t* ds;
            const uint16_t* db;
            if (slot == a.top_k) {
                dc = a.sd_codes; ds = a.sd_scales; db = a.sd_biases;
            } else {
                const int e = a.ids[slot];
                dc = reinterpret_cast<const u32x4*>(a.d_codes + (size_t)e * a.d_cstride);
                ds = reinterpret_cast<const uint16_t*>(a.d_scales + (size_t)e * a.d_sstride);
                db = reinterpret_cast<const uint16_t*>(a.d_biases + (size_t)e * a.d_sstride);
            }
#pragma unroll
            for (int r = 0; r < RH; ++r) {
                const int h = min(h0 + r, a.hidden - 1);
#pragma unroll
                for (int i = 0; i < CPLD; ++i) {
                    const int ch = min(j + LPR * i, CH - 1);
                    c[t][r][i] = __builtin_nontemporal_load(dc + (size_t)h * CH + ch);
                    sv[t][r][i] = ds[(size_t)h * G + (ch >> 1)];
                    bv[t][r][i] = db[(size_t)h * G + (ch >> 1)];
                }
            }
        }
    }

    // stage the activations of every slot in LDS, 32-float chunks at a 36-float pitch so the 16
    // lanes of a group (one chunk each) read distinct banks; all loads are issued (clamped) before
    // the first store, so the staging costs one round trip
    constexpr int AL = (NSLOT * 512 * CPLD + 256 * P2W - 1) / (256 * P2W);
    const int n = nslot * a.inter;
    f4v av4[AL];
#pragma unroll
    for (int k = 0; k < AL; ++k) {
        const int i = min(threadIdx.x * 4 + k * 256 * P2W, n - 4);
        av4[k] = *reinterpret_cast<const f4v*>(a.act + i);
    }
#pragma unroll
    for (int k = 0; k < AL; ++k) {
        const int i = threadIdx.x * 4 + k * 256 * P2W;
        if (i < n) *reinterpret_cast<f4v*>(lds_act + (i >> 5) * ACT_PITCH + (i & 31)) = av4[k];
    }
    __syncthreads();

#pragma unroll
    for (int t = 0; t < SLOTS_PER_WAVE; ++t) {
        const int slot = wave + P2W * t;
        if (slot < nslot) {
            float p[RH];
            down_part<RH, CPLD>(p, c[t], sv[t], bv[t], lds_act + slot * CH * ACT_PITCH, ACT_PITCH, j, CH);
#pragma unroll
            for (int r = 0; r < RH; ++r) {
                const float d = group_sum<LPR>(p[r]);
                if (j == 0) dpart[slot][(lane / LPR) * RH + r] = d;
            }
        }
    }
    __syncthreads();
    if (wave == 0 && j == 0) {
#pragma unroll
        for (int r = 0; r < RH; ++r) {
            const int h = h0 + r;
            if (h < a.hidden) {
                const float o = moe_combine(w, &dpart[0][(lane / LPR) * RH + r], 4 * RH, a.top_k, gate_logit, a.boundary);
                a.out[h] = (_Float16)o;
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// A chunk of M <= 128 tokens through the layer in one pass over a route list ("src/real_forward.rs",
// the forward state's routed-batch switch for chunked prefill): the results are identical, bit
// for bit, to M decode calls, because every per-token value is computed by the same helpers in
// the same order (router_dot, wave_topk and publish_topk, pair_act, down_part, moe_combine);
// what changes is that each expert's weights stream once per chunk for all the tokens routed
// to it.
//  k_moep_router : one wave per router row (and one for the shared gate row): the row is loaded
//                  once and dotted with a group of tokens, four tokens' activations in flight.
//  k_moep_topk   : one wave per token: the decode's top-k and softmax, and the token's activations
//                  in the offset form pair_act multiplies (once per token, into the workspace).
//  k_moep_phase1 : block = (16 rows, expert): the (token, slot) pairs routed to the expert, read
//                  off the ids, run through pair_act; the tokens' offset-form activations are copied
//                  into LDS a group at a time. Expert E is the shared one, taken by every token in
//                  slot top_k.
//  k_moep_phase2 : block = (64 down rows, expert): each routed (token, slot) gets its down-row
//                  dots (down_part, summed over 16 lanes), written to the workspace per slot.
//  k_moep_combine: every output of every token from its slots' dots (moe_combine).
constexpr int RT_TOK = 16;       // tokens per router block
constexpr int RT_GRP = 4;        // tokens whose activations are in flight together
// tokens staged per pass (the staging stays under 64 KiB of LDS at the largest shapes)
template <int CPL> constexpr int p1_tg() { return CPL <= 5 ? 8 : 4; }
template <int CPLD> constexpr int p2_tg() { return CPLD == 1 ? 16 : 8; }
constexpr int P2_RH = 4;         // down rows per 16-lane group in the batched phase 2
constexpr int P2_NT = 2;         // 64-row tiles per block in the batched phase 2
constexpr int ITEM_TOK = 16;     // (token, slot) pairs per work item

template <int CPL, int KIND, bool SC>
DHP_DEV void router_tokens(const MoeArgs& a, const void* row, const uint16_t* escale, int r, bool sgr) {
    constexpr int G = SC ? 2 : RT_GRP;                     // the scales take registers too
    const int lane = threadIdx.x & 63;
    RouterRow<CPL, KIND> rr;
    router_row_load<CPL, KIND>(rr, row);
    const int m0 = blockIdx.y * RT_TOK, m1 = min(m0 + RT_TOK, a.M);
    for (int mb = m0; mb < m1; mb += G) {
        RouterX<CPL, SC> v[G];
#pragma unroll
        for (int g = 0; g < G; ++g)
            router_x_load<CPL, KIND, SC>(v[g], a.x + (size_t)min(mb + g, m1 - 1) * a.hidden, escale);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int m = mb + g;
            const float d = router_dot<CPL, KIND, SC>(rr, v[g]);
            if (lane == 0 && m < m1) {
                if (sgr) a.gate_logit[m] = d;
                else a.logits[(size_t)m * a.Epad + r] = d;
            }
        }
    }
}

template <int CPL>
__global__ __launch_bounds__(256) void k_moep_router(MoeArgs a) {
    const int wave = threadIdx.x >> 6;
    const int r = blockIdx.x * 4 + wave;       // router row; E: the shared gate row
    if (r > a.E) return;                       // whole waves; no block synchronisation below
    const bool sgr = r == a.E;
    const int kind = sgr ? RK_BF16 : a.router_kind;
    const uint16_t* escale = sgr ? nullptr : a.router_escale;
    const void* row = sgr ? static_cast<const void*>(a.sgate_row)
                          : static_cast<const void*>(static_cast<const uint8_t*>(a.router) +
                                                     (size_t)r * router_row_bytes(a.router_kind, a.hidden));
    if (kind == RK_BF16) {
        if (escale) router_tokens<CPL, RK_BF16, true>(a, row, escale, r, sgr);
        else router_tokens<CPL, RK_BF16, false>(a, row, escale, r, sgr);
    } else if (kind == RK_F32) {
        if (escale) router_tokens<CPL, RK_F32, true>(a, row, escale, r, sgr);
        else router_tokens<CPL, RK_F32, false>(a, row, escale, r, sgr);
    } else {
        if (escale) router_tokens<CPL, RK_I8, true>(a, row, escale, r, sgr);
        else router_tokens<CPL, RK_I8, false>(a, row, escale, r, sgr);
    }
}

template <int PER>
__global__ __launch_bounds__(64) void k_moep_topk(MoeArgs a) {
    const int m = blockIdx.x;
    TopkIn<PER> tin;
    topk_load<PER>(tin, a.logits + (size_t)m * a.Epad, a.E);
    int ids[DHP_MOE_MAX_TOP_K];
    float vals[DHP_MOE_MAX_TOP_K];
    wave_topk<PER>(tin, a.E, a.top_k, ids, vals);
    if (threadIdx.x == 0)
        publish_topk(ids, vals, a.top_k, a.expert_scale, a.ids + (size_t)m * a.top_k,
                     a.weights + (size_t)m * a.top_k);
    // the token's activations in the form phase 1 multiplies, once per token (every phase-1
    // block that stages the token copies them instead of converting them again)
    const int CH32 = a.hidden >> 5;
    for (int c = threadIdx.x; c < CH32; c += 64) {
        const u32x4* src = reinterpret_cast<const u32x4*>(a.x + (size_t)m * a.hidden + 32 * c);
        const u32x4 v[4] = {src[0], src[1], src[2], src[3]};
        h2 xp[16];
        float nc;
        const float xs = x32_off_from(v, xp, nc);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            a.xraw[((size_t)m * 4 + q) * CH32 + c] = u32x4{h2_bits(xp[4 * q]), h2_bits(xp[4 * q + 1]),
                                                         h2_bits(xp[4 * q + 2]), h2_bits(xp[4 * q + 3])};
        a.xrsum[(size_t)m * CH32 + c] = float2{xs, nc};
    }
}

// Inclusive prefix sum over the 64 lanes of a wave.
DHP_DEV int wave_incl_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    return v;
}

// The route list and the work items, by one block of 1024 threads: the chunk's (token, slot)
// pairs counting-sorted by expert (the shared expert's M pairs first, then the routed experts in
// index order; within an expert any order, since every pair's results are computed and stored
// on their own), cut into items of at most ITEM_TOK pairs of one expert. The shared expert's
// items come first, so the blocks holding the longest list start first.
__global__ __launch_bounds__(1024) void k_moep_route(MoeArgs a) {
    __shared__ int cnt[MAX_E], base[MAX_E], ibase[MAX_E], fill[MAX_E];
    __shared__ int wsum[16][2];
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int E = a.E, M = a.M, k = a.top_k, n = M * k;
    if (t < E) { cnt[t] = 0; fill[t] = 0; }
    __syncthreads();
    for (int i = t; i < n; i += 1024) atomicAdd(&cnt[a.ids[i]], 1);     // n = M * k <= 1280
    __syncthreads();
    const int c = (t < E) ? cnt[t] : 0;
    const int ki = (c + ITEM_TOK - 1) / ITEM_TOK;
    const int sc = wave_incl_scan(c), sk = wave_incl_scan(ki);
    if (lane == 63) { wsum[wave][0] = sc; wsum[wave][1] = sk; }
    __syncthreads();
    int oc = 0, ok = 0;
    for (int w = 0; w < wave; ++w) { oc += wsum[w][0]; ok += wsum[w][1]; }
    const int nsh = (M + ITEM_TOK - 1) / ITEM_TOK;
    if (t < E) { base[t] = M + oc + sc - c; ibase[t] = nsh + ok + sk - ki; }
    __syncthreads();
    for (int i = t; i < n; i += 1024) {
        const int e = a.ids[i];
        a.route[base[e] + atomicAdd(&fill[e], 1)] = ((i / k) << 4) | (i % k);
    }
    if (t < M) a.route[t] = (t << 4) | k;
    if (t < nsh) *reinterpret_cast<int4*>(a.items + 4 * t) = int4{E, ITEM_TOK * t, min(ITEM_TOK, M - ITEM_TOK * t), 0};
    if (t < E)
        for (int j = 0; j < ki; ++j)
            *reinterpret_cast<int4*>(a.items + 4 * (ibase[t] + j)) =
                int4{t, base[t] + ITEM_TOK * j, min(ITEM_TOK, c - ITEM_TOK * j), 0};
    if (t == 1023) a.nitems[0] = nsh + ok + sk;           // the last thread holds the full totals
}

// An upper bound on the work items of a chunk: the shared expert's, plus at most one partial
// item per routed expert that appears on top of the full ones.
int max_items(int M, int E, int top_k) {
    return (M + ITEM_TOK - 1) / ITEM_TOK + (M * top_k) / ITEM_TOK + min(E, M * top_k);
}

template <int CPL>
__global__ __launch_bounds__(256, CPL <= 5 ? 3 : 2) void k_moep_phase1(MoeArgs a) {
    constexpr int CH32 = LPR * CPL;                   // 32-activation chunks per token
    constexpr int P1_TG = p1_tg<CPL>();
    constexpr int IT = (P1_TG * CH32 + 255) / 256;    // staged chunks per thread per pass
    extern __shared__ u32x4 xstage[];                 // [P1_TG][4][CH32] u32x4, then [P1_TG][CH32] float2
    float2* xsum = reinterpret_cast<float2*>(xstage + P1_TG * 4 * CH32);
    if ((int)blockIdx.y >= a.nitems[0]) return;        // the whole block
    const int4 item = *reinterpret_cast<const int4*>(a.items + 4 * blockIdx.y);
    const int e = item.x, n = item.z;
    const int32_t* list = a.route + item.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, j = lane % LPR;
    const int row = blockIdx.x * 16 + wave * 4 + lane / LPR;
    const bool live = row < a.inter;
    const u32x4 *gc, *uc;
    const uint16_t *gs, *gb, *us, *ub;
    if (e == a.E) {
        gc = a.sg_codes; gs = a.sg_scales; gb = a.sg_biases;
        uc = a.su_codes; us = a.su_scales; ub = a.su_biases;
    } else {
        gc = reinterpret_cast<const u32x4*>(a.g_codes + (size_t)e * a.gu_cstride);
        gs = reinterpret_cast<const uint16_t*>(a.g_scales + (size_t)e * a.gu_sstride);
        gb = reinterpret_cast<const uint16_t*>(a.g_biases + (size_t)e * a.gu_sstride);
        uc = reinterpret_cast<const u32x4*>(a.u_codes + (size_t)e * a.u_cstride);
        us = reinterpret_cast<const uint16_t*>(a.u_scales + (size_t)e * a.u_sstride);
        ub = reinterpret_cast<const uint16_t*>(a.u_biases + (size_t)e * a.u_sstride);
    }
    PairRegs<CPL> p;
    load_pair<CPL>(p, gc, gs, gb, uc, us, ub, live ? row : 0, j);
    const int nslot = a.top_k + 1;

    for (int base = 0; base < n; base += P1_TG) {
        const int tn = min(P1_TG, n - base);
        __syncthreads();                               // the previous group's reads are done
        // every load of the group first (items past the group clamped), then the stores
        // the tokens' activations were put in the offset form once per token (k_moep_topk): copy them
        u32x4 v[IT][4];
        float2 vs[IT];
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int it = min((int)threadIdx.x + 256 * k, tn * CH32 - 1);
            const int t = it / CH32, c = it - t * CH32;
            const size_t tok = (size_t)(list[base + t] >> 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) v[k][q] = a.xraw[(tok * 4 + q) * CH32 + c];
            vs[k] = a.xrsum[tok * CH32 + c];
        }
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int it = (int)threadIdx.x + 256 * k;
            if (it < tn * CH32) {
                const int t = it / CH32, c = it - t * CH32;
#pragma unroll
                for (int q = 0; q < 4; ++q) xstage[(t * 4 + q) * CH32 + c] = v[k][q];
                xsum[t * CH32 + c] = vs[k];
            }
        }
        __syncthreads();
        // pair_act's operations in its order for every token, the activations read a chunk at a
        // time. The codes' offset fp16 form depends only on the weights, so each chunk is unpacked
        // once for all the group's tokens; each token's sums run in pair_act's order, so its value
        // is the decode call's bit for bit.
        const NibConsts nk = nib_consts();
        float ag[P1_TG], au[P1_TG];
#pragma unroll
        for (int u = 0; u < P1_TG; ++u) ag[u] = au[u] = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = j + LPR * i;
            const uint32_t wg[4] = {p.cg[i].x, p.cg[i].y, p.cg[i].z, p.cg[i].w};
            const uint32_t wu[4] = {p.cu[i].x, p.cu[i].y, p.cu[i].z, p.cu[i].w};
            h2 tg[16], tu[16];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                unpack8_off(wg[w], tg + 4 * w, nk);
                unpack8_off(wu[w], tu + 4 * w, nk);
            }
#pragma unroll
            for (int t = 0; t < P1_TG; ++t) {
                if (t < tn) {
                    h2 xp[16];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const u32x4 v4 = xstage[(t * 4 + q) * CH32 + c];
                        xp[4 * q] = as_h2(v4.x); xp[4 * q + 1] = as_h2(v4.y);
                        xp[4 * q + 2] = as_h2(v4.z); xp[4 * q + 3] = as_h2(v4.w);
                    }
                    const float2 sn = xsum[t * CH32 + c];
                    float dg = sn.y, du = sn.y;
#pragma unroll
                    for (int e = 0; e < 16; ++e) dg = __builtin_amdgcn_fdot2(tg[e], xp[e], dg, false);
#pragma unroll
                    for (int e = 0; e < 16; ++e) du = __builtin_amdgcn_fdot2(tu[e], xp[e], du, false);
                    ag[t] = __builtin_fmaf(bf16_to_f32(p.sg[i]), dg, ag[t]);
                    ag[t] = __builtin_fmaf(bf16_to_f32(p.bg[i]), sn.x, ag[t]);
                    au[t] = __builtin_fmaf(bf16_to_f32(p.su[i]), du, au[t]);
                    au[t] = __builtin_fmaf(bf16_to_f32(p.bu[i]), sn.x, au[t]);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < P1_TG; ++t) {
            if (t < tn) {
                const float g1 = group_sum<LPR>(ag[t]) * 0.0625f;
                const float u1 = group_sum<LPR>(au[t]) * 0.0625f;
                const float v1 = silu_f(g1) * u1;
                const int ms = list[base + t];
                if (j == 0 && live) a.act[((size_t)(ms >> 4) * nslot + (ms & 15)) * a.inter + row] = v1;
            }
        }
    }
}

// A block owns P2_NT tiles of 64 down rows of one work item: the codes of all its tiles are in
// flight together, the item's activations are staged once for them, and the tiles are computed
// one after the other (each tile's codes become floats only when its turn comes).
template <int CPLD>
__global__ __launch_bounds__(256) void k_moep_phase2(MoeArgs a) {
    extern __shared__ float astage[];                  // [P2_TG][inter / 32][ACT_PITCH]
    if ((int)blockIdx.y >= a.nitems[0]) return;        // the whole block
    const int4 item = *reinterpret_cast<const int4*>(a.items + 4 * blockIdx.y);
    const int e = item.x, n = item.z;
    const int32_t* list = a.route + item.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, j = lane % LPR;
    const int CH = a.inter >> 5, G = a.inter >> 6;
    const int nslot = a.top_k + 1;
    const u32x4* dc;
    const uint16_t *ds, *db;
    if (e == a.E) {
        dc = a.sd_codes; ds = a.sd_scales; db = a.sd_biases;
    } else {
        dc = reinterpret_cast<const u32x4*>(a.d_codes + (size_t)e * a.d_cstride);
        ds = reinterpret_cast<const uint16_t*>(a.d_scales + (size_t)e * a.d_sstride);
        db = reinterpret_cast<const uint16_t*>(a.d_biases + (size_t)e * a.d_sstride);
    }
    int h0[P2_NT];
    u32x4 c[P2_NT][P2_RH][CPLD];
    uint32_t sv[P2_NT][P2_RH][CPLD], bv[P2_NT][P2_RH][CPLD];
#pragma unroll
    for (int q = 0; q < P2_NT; ++q) {
        h0[q] = ((blockIdx.x * P2_NT + q) * 16 + wave * 4 + lane / LPR) * P2_RH;
#pragma unroll
        for (int r = 0; r < P2_RH; ++r) {
            const int h = min(h0[q] + r, a.hidden - 1);
#pragma unroll
            for (int i = 0; i < CPLD; ++i) {
                const int ch = min(j + LPR * i, CH - 1);
                c[q][r][i] = __builtin_nontemporal_load(dc + (size_t)h * CH + ch);
                sv[q][r][i] = ds[(size_t)h * G + (ch >> 1)];
                bv[q][r][i] = db[(size_t)h * G + (ch >> 1)];
            }
        }
    }
    constexpr int P2_TG = p2_tg<CPLD>();
    constexpr int IT = P2_TG * 32 * CPLD * LPR / 4 / 256;   // f4v per thread per pass (inter <= 512 CPLD)
    for (int base = 0; base < n; base += P2_TG) {
        const int tn = min(P2_TG, n - base);
        __syncthreads();                               // the previous group's reads are done
        const int items = tn * (a.inter >> 2);
        f4v v[IT];
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int it = min((int)threadIdx.x + 256 * k, items - 1);
            const int t = it / (a.inter >> 2), qq = it - t * (a.inter >> 2);
            const int ms = list[base + t];
            v[k] = *reinterpret_cast<const f4v*>(a.act + ((size_t)(ms >> 4) * nslot + (ms & 15)) * a.inter + 4 * qq);
        }
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int it = (int)threadIdx.x + 256 * k;
            if (it < items) {
                const int t = it / (a.inter >> 2), i4 = 4 * (it - t * (a.inter >> 2));
                *reinterpret_cast<f4v*>(astage + (t * CH + (i4 >> 5)) * ACT_PITCH + (i4 & 31)) = v[k];
            }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < P2_NT; ++q) {
            // keeps this tile's code-to-float conversion here rather than hoisted above the loops
            // with every other tile's (which would hold all tiles' floats at once)
#pragma unroll
            for (int r = 0; r < P2_RH; ++r)
#pragma unroll
                for (int i = 0; i < CPLD; ++i) asm volatile("" : "+v"(c[q][r][i]));
            for (int t = 0; t < tn; ++t) {
                float p[P2_RH];
                down_part<P2_RH, CPLD>(p, c[q], sv[q], bv[q], astage + t * CH * ACT_PITCH, ACT_PITCH, j, CH);
                const int ms = list[base + t];
                float* dst = a.dsum + ((size_t)(ms >> 4) * nslot + (ms & 15)) * a.hidden;
#pragma unroll
                for (int r = 0; r < P2_RH; ++r) {
                    const float d = group_sum<LPR>(p[r]);
                    if (j == 0 && h0[q] + r < a.hidden) dst[h0[q] + r] = d;
                }
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_moep_combine(MoeArgs a) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= a.M * a.hidden) return;
    const int m = idx / a.hidden, h = idx - m * a.hidden;
    float w[DHP_MOE_MAX_TOP_K];
#pragma unroll
    for (int s = 0; s < DHP_MOE_MAX_TOP_K; ++s) w[s] = a.weights[(size_t)m * a.top_k + min(s, a.top_k - 1)];
    const float o = moe_combine(w, a.dsum + (size_t)m * (a.top_k + 1) * a.hidden + h, a.hidden, a.top_k,
                                a.gate_logit[m], a.boundary);
    a.out[idx] = (_Float16)o;
}

template <int CPL>
hipError_t launch_prefill_all(const MoeArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_moep_router<CPL>, dim3((a.E + 1 + 3) / 4, (a.M + RT_TOK - 1) / RT_TOK), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.E <= 256) hipLaunchKernelGGL((k_moep_topk<4>), dim3(a.M), dim3(64), 0, s, a);
    else hipLaunchKernelGGL((k_moep_topk<MAX_E / 64>), dim3(a.M), dim3(64), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int CH32 = LPR * CPL;
    const size_t lds1 = (size_t)p1_tg<CPL>() * CH32 * (4 * sizeof(u32x4) + sizeof(float2));
    hipLaunchKernelGGL(k_moep_route, dim3(1), dim3(1024), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int items = max_items(a.M, a.E, a.top_k);
    hipLaunchKernelGGL(k_moep_phase1<CPL>, dim3((a.inter + 15) / 16, items), dim3(256), lds1, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 g2((a.hidden + 16 * P2_RH * P2_NT - 1) / (16 * P2_RH * P2_NT), items);
    if (a.inter <= 512)
        hipLaunchKernelGGL(k_moep_phase2<1>, g2, dim3(256), (size_t)p2_tg<1>() * (a.inter / 32) * ACT_PITCH * 4, s, a);
    else
        hipLaunchKernelGGL(k_moep_phase2<2>, g2, dim3(256), (size_t)p2_tg<2>() * (a.inter / 32) * ACT_PITCH * 4, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_moep_combine, dim3((a.M * a.hidden + 255) / 256), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int CPL>
hipError_t launch_all(const MoeArgs& a, hipStream_t s) {
    const int shared_blocks = (a.inter + 3) / 4;
    const int x_blocks = (a.hidden / 32 + 63) / 64;
    hipLaunchKernelGGL(k_moe_router<CPL>, dim3(a.E + 1 + shared_blocks + x_blocks), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int pairs = a.top_k * a.inter;
    if (a.E <= 256) hipLaunchKernelGGL((k_moe_phase1<CPL, 4>), dim3((pairs + 3) / 4), dim3(64), 0, s, a);
    else hipLaunchKernelGGL((k_moe_phase1<CPL, MAX_E / 64>), dim3((pairs + 3) / 4), dim3(64), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = (size_t)(a.top_k + 1) * (a.inter / 32) * ACT_PITCH * sizeof(float);
    const dim3 g2((a.hidden + 4 * RH - 1) / (4 * RH));
    if (a.inter <= 512) hipLaunchKernelGGL(k_moe_phase2<1>, g2, dim3(64 * P2W), lds, s, a);
    else hipLaunchKernelGGL(k_moe_phase2<2>, g2, dim3(64 * P2W), lds, s, a);
    return hipGetLastError();
}

}  // namespace

// Decode workspace: logits fp32 [E], the gate logit, pad to 16 bytes, act fp32 [top_k + 1][inter];
// at the next 256-byte boundary the token's offset-form activations, sized for the largest hidden
// (4096: 128 chunks): 4 planes of u32x4 [128], then (16 sum, -1024 sum) float2 [128].
constexpr size_t MOE_XRAW_BYTES = 4 * 128 * sizeof(u32x4);
constexpr size_t MOE_XRSUM_BYTES = 128 * sizeof(float2);
static size_t moe_x_offset(int32_t n_experts, int32_t top_k, int32_t inter) {
    const size_t floats = (size_t)((n_experts + 4) & ~3) + (size_t)(top_k + 1) * inter;
    return (floats * sizeof(float) + 255) & ~(size_t)255;
}
size_t dhp_moe_ws(int32_t n_experts, int32_t top_k, int32_t inter) {
    return moe_x_offset(n_experts, top_k, inter) + MOE_XRAW_BYTES + MOE_XRSUM_BYTES;
}

namespace {
size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
// Batched workspace, in order: logits [m][Epad], gate logits [m], act [m][top_k + 1][inter],
// slot dots [m][top_k + 1][hidden] (fp32, each part 256-byte aligned).
struct PrefillWs {
    size_t logits, gate, act, dsum, route, items, nitems, xraw, xrsum, total;
};
PrefillWs prefill_ws(int m, int E, int top_k, int inter, int hidden) {
    PrefillWs w;
    const size_t epad = (size_t)((E + 3) & ~3);
    w.logits = 0;
    w.gate = w.logits + align256((size_t)m * epad * sizeof(float));
    w.act = w.gate + align256((size_t)m * sizeof(float));
    w.dsum = w.act + align256((size_t)m * (top_k + 1) * inter * sizeof(float));
    w.route = w.dsum + align256((size_t)m * (top_k + 1) * hidden * sizeof(float));
    w.items = w.route + align256((size_t)m * (top_k + 1) * sizeof(int32_t));
    w.nitems = w.items + align256((size_t)max_items(m, E, top_k) * 4 * sizeof(int32_t));
    w.xraw = w.nitems + 256;
    w.xrsum = w.xraw + align256((size_t)m * (hidden / 32) * 4 * sizeof(u32x4));
    w.total = w.xrsum + align256((size_t)m * (hidden / 32) * sizeof(float2));
    return w;
}

void fill_args(MoeArgs& a, const void* x, const dhp_router* router, const void* sgate_row,
               const dhp_int4_experts* gate, const dhp_int4_experts* up, const dhp_int4_experts* down,
               const dhp_int4* sg, const dhp_int4* su, const dhp_int4* sd, int top_k, int boundary, void* out,
               int32_t* ids, float* weights) {
    a.x = static_cast<const _Float16*>(x);
    a.router = router->weights;
    a.router_kind = router->dtype == DHP_F32 ? RK_F32 : router->dtype == DHP_I8 ? RK_I8 : RK_BF16;
    a.router_escale = static_cast<const uint16_t*>(router->elem_scale);
    a.expert_scale = router->expert_scale;
    a.sgate_row = static_cast<const uint16_t*>(sgate_row);
    a.g_codes = static_cast<const uint8_t*>(gate->first.codes);
    a.g_scales = static_cast<const uint8_t*>(gate->first.scales);
    a.g_biases = static_cast<const uint8_t*>(gate->first.biases);
    a.u_codes = static_cast<const uint8_t*>(up->first.codes);
    a.u_scales = static_cast<const uint8_t*>(up->first.scales);
    a.u_biases = static_cast<const uint8_t*>(up->first.biases);
    a.d_codes = static_cast<const uint8_t*>(down->first.codes);
    a.d_scales = static_cast<const uint8_t*>(down->first.scales);
    a.d_biases = static_cast<const uint8_t*>(down->first.biases);
    a.gu_cstride = gate->codes_stride;
    a.gu_sstride = gate->scales_stride;
    a.u_cstride = up->codes_stride;
    a.u_sstride = up->scales_stride;
    a.d_cstride = down->codes_stride;
    a.d_sstride = down->scales_stride;
    a.sg_codes = static_cast<const u32x4*>(sg->codes);
    a.sg_scales = static_cast<const uint16_t*>(sg->scales);
    a.sg_biases = static_cast<const uint16_t*>(sg->biases);
    a.su_codes = static_cast<const u32x4*>(su->codes);
    a.su_scales = static_cast<const uint16_t*>(su->scales);
    a.su_biases = static_cast<const uint16_t*>(su->biases);
    a.sd_codes = static_cast<const u32x4*>(sd->codes);
    a.sd_scales = static_cast<const uint16_t*>(sd->scales);
    a.sd_biases = static_cast<const uint16_t*>(sd->biases);
    a.E = gate->count;
    a.hidden = gate->first.cols;
    a.inter = gate->first.rows;
    a.top_k = top_k;
    a.boundary = boundary;
    a.out = static_cast<_Float16*>(out);
    a.ids = ids;
    a.weights = weights;
}
}  // namespace

size_t dhp_moe_prefill_ws(int32_t m, int32_t n_experts, int32_t top_k, int32_t inter, int32_t hidden) {
    return prefill_ws(m, n_experts, top_k, inter, hidden).total;
}

int launch_moe(const void* x, const dhp_router* router, const void* sgate_row,
               const dhp_int4_experts* gate, const dhp_int4_experts* up, const dhp_int4_experts* down,
               const dhp_int4* sg, const dhp_int4* su, const dhp_int4* sd, int top_k, int boundary,
               void* out, int32_t* ids, float* weights, void* ws, hipStream_t s) {
    MoeArgs a;
    fill_args(a, x, router, sgate_row, gate, up, down, sg, su, sd, top_k, boundary, out, ids, weights);
    a.M = 1;
    a.Epad = a.E;
    float* w = static_cast<float*>(ws);
    a.logits = w;
    a.gate_logit = w + a.E;
    a.act = w + ((a.E + 4) & ~3);        // 16-byte aligned
    a.dsum = nullptr;
    a.route = a.items = a.nitems = nullptr;
    char* xbase = static_cast<char*>(ws) + moe_x_offset(a.E, top_k, a.inter);
    a.xraw = reinterpret_cast<u32x4*>(xbase);
    a.xrsum = reinterpret_cast<float2*>(xbase + MOE_XRAW_BYTES);

    hipError_t e;
    switch (a.hidden / 512) {
        case 1: e = launch_all<1>(a, s); break;
        case 2: e = launch_all<2>(a, s); break;
        case 3: e = launch_all<3>(a, s); break;
        case 4: e = launch_all<4>(a, s); break;
        case 5: e = launch_all<5>(a, s); break;
        case 6: e = launch_all<6>(a, s); break;
        case 7: e = launch_all<7>(a, s); break;
        case 8: e = launch_all<8>(a, s); break;
        default: return dhp_fail(DHP_ERR_UNSUPPORTED, "hidden=%d", a.hidden);
    }
    if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "moe launch: %s", hipGetErrorString(e));
    return DHP_OK;
}

int launch_moe_prefill(const void* x, int m, const dhp_router* router, const void* sgate_row,
                       const dhp_int4_experts* gate, const dhp_int4_experts* up, const dhp_int4_experts* down,
                       const dhp_int4* sg, const dhp_int4* su, const dhp_int4* sd, int top_k, int boundary,
                       void* out, int32_t* ids, float* weights, void* ws, hipStream_t s) {
    MoeArgs a;
    fill_args(a, x, router, sgate_row, gate, up, down, sg, su, sd, top_k, boundary, out, ids, weights);
    a.M = m;
    a.Epad = (a.E + 3) & ~3;
    const PrefillWs lay = prefill_ws(m, a.E, top_k, a.inter, a.hidden);
    char* base = static_cast<char*>(ws);
    a.logits = reinterpret_cast<float*>(base + lay.logits);
    a.gate_logit = reinterpret_cast<float*>(base + lay.gate);
    a.act = reinterpret_cast<float*>(base + lay.act);
    a.dsum = reinterpret_cast<float*>(base + lay.dsum);
    a.route = reinterpret_cast<int32_t*>(base + lay.route);
    a.items = reinterpret_cast<int32_t*>(base + lay.items);
    a.nitems = reinterpret_cast<int32_t*>(base + lay.nitems);
    a.xraw = reinterpret_cast<u32x4*>(base + lay.xraw);
    a.xrsum = reinterpret_cast<float2*>(base + lay.xrsum);

    hipError_t e;
    switch (a.hidden / 512) {
        case 1: e = launch_prefill_all<1>(a, s); break;
        case 2: e = launch_prefill_all<2>(a, s); break;
        case 3: e = launch_prefill_all<3>(a, s); break;
        case 4: e = launch_prefill_all<4>(a, s); break;
        case 5: e = launch_prefill_all<5>(a, s); break;
        case 6: e = launch_prefill_all<6>(a, s); break;
        case 7: e = launch_prefill_all<7>(a, s); break;
        case 8: e = launch_prefill_all<8>(a, s); break;
        default: return dhp_fail(DHP_ERR_UNSUPPORTED, "hidden=%d", a.hidden);
    }
    if (e != hipSuccess) return dhp_fail(DHP_ERR_LAUNCH, "moe prefill launch: %s", hipGetErrorString(e));
    return DHP_OK;
}
