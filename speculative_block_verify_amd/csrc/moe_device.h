// Device helpers shared by the skinny (verify-width) and grouped (prefill)
// kernels: bf16/E4M3/E2M1 conversions, wave64 cross-lane operations, the
// per-row top-k, and the fp16 operand decode of the MFMA gate/up tiles.
#pragma once

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// scalar helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Order-preserving map of a float key onto uint32 (larger float -> larger
// integer; -0 and +0 map together).  Real keys never map to 0, which marks
// an empty or already-taken entry.
__device__ __forceinline__ uint32_t key_bits(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// E4M3FN byte -> fp32 (gfx950 converts OCP FP8 natively).
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t packed) {
    return __builtin_amdgcn_cvt_f32_fp8((int)packed, SEL);
}

// Eight E2M1 codes (one dword, column 2t in the low nibble of byte t) ->
// four bf16 pairs (exact: every E2M1 value is a bf16).
__device__ __forceinline__ void fp4x8_to_bf16(uint32_t v, bf16x2_t* out) {
    out[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 0);
    out[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 1);
    out[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 2);
    out[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 3);
}

__device__ __forceinline__ void fp4x8_to_f32(uint32_t v, float* out) {
    f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 0);
    f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 1);
    f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 2);
    f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 3);
    out[0] = p0.x; out[1] = p0.y; out[2] = p1.x; out[3] = p1.y;
    out[4] = p2.x; out[5] = p2.y; out[6] = p3.x; out[7] = p3.y;
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }

__device__ __forceinline__ float dot2(bf16x2_t a, bf16x2_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

// ---------------------------------------------------------------------------
// cross-lane helpers (wave64).  DPP row shifts accumulate inside 16-lane
// rows; readlane combines the four rows.  Summation order is fixed, so every
// result is deterministic.
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(dpp<CTRL>(__float_as_int(v)));
}
__device__ __forceinline__ float readlanef(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// inclusive prefix sum inside each 16-lane row
__device__ __forceinline__ float row_scan(float v) {
    v += dppf<0x111>(v);
    v += dppf<0x112>(v);
    v += dppf<0x114>(v);
    v += dppf<0x118>(v);
    return v;
}
__device__ __forceinline__ int row_scan_i(int v) {
    v += dpp<0x111>(v);
    v += dpp<0x112>(v);
    v += dpp<0x114>(v);
    v += dpp<0x118>(v);
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
    v = row_scan(v);
    return (readlanef(v, 15) + readlanef(v, 31)) + (readlanef(v, 47) + readlanef(v, 63));
}

__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = threadIdx.x & 63;
    v = row_scan_i(v);
    const int t0 = __builtin_amdgcn_readlane(v, 15);
    const int t1 = __builtin_amdgcn_readlane(v, 31);
    const int t2 = __builtin_amdgcn_readlane(v, 47);
    if (lane >= 16) v += t0;
    if (lane >= 32) v += t1;
    if (lane >= 48) v += t2;
    return v;
}

// Wave maximum: inclusive max-scan inside each 16-lane row, then the
// row_bcast:15 / row_bcast:31 steps carry rows 0-2 into lane 63 (lanes a
// step does not update keep their value: 0 is the identity of the maximum).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)dpp<0x111>((int)v));
    v = max(v, (uint32_t)dpp<0x112>((int)v));
    v = max(v, (uint32_t)dpp<0x114>((int)v));
    v = max(v, (uint32_t)dpp<0x118>((int)v));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Sum over aligned groups of G lanes; valid in the last lane of each group.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (G == 64) {
        return wave_sum(v);
    } else if constexpr (G == 32) {
        v = row_scan(v);
        const float lo = readlanef(v, 15) + readlanef(v, 31);
        const float hi = readlanef(v, 47) + readlanef(v, 63);
        return (threadIdx.x & 32) ? hi : lo;
    } else if constexpr (G == 16) {
        return row_scan(v);
    } else {
#pragma unroll
        for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
        return v;
    }
}

__device__ __forceinline__ float group_sum_rt(float v, int G) {
    switch (G) {
        case 64: return group_sum<64>(v);
        case 32: return group_sum<32>(v);
        case 16: return group_sum<16>(v);
        case 8: return group_sum<8>(v);
        case 4: return group_sum<4>(v);
        default: return group_sum<2>(v);
    }
}

// ---------------------------------------------------------------------------
// selection + dedup (one workgroup of kBlock threads)
// ---------------------------------------------------------------------------

struct SelectSmem {
    int32_t sel[kMaxSlots];
    float w[kMaxSlots];
    int32_t asg[kMaxSlots];
    int32_t inv[kMaxSlots];
    int32_t uniq[kMaxSlots];
    int32_t off[kMaxSlots + 1];
    int32_t n_unique;
    uint32_t rowmask[kMaxExperts];   // rows that selected each expert
    int32_t cstart[kMaxExperts];     // CSR offset of each expert
};

// Copy n floats global -> LDS with every load of a pass in flight at once.
__device__ __forceinline__ void stage_floats(float* dst, const float* src, int n, int tid, int nthr) {
    constexpr int U = 8;
    for (int base = 0; base < n; base += U * nthr) {
        float v[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int i = base + j * nthr + tid;
            v[j] = (i < n) ? src[i] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int i = base + j * nthr + tid;
            if (i < n) dst[i] = v[j];
        }
    }
}

// Count of set bits of a 64-lane mask in the lanes below this one.
__device__ __forceinline__ int lanes_below(unsigned long long m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Selection key of expert e with router logit l, as an order-preserving
// integer: the logit (softmax scoring) or sigmoid(l) + bias[e] (sigmoid
// scoring, the router tail of PR #844 section 4).
__device__ __forceinline__ uint32_t select_key(const SelectArgs& a, float l, int e) {
    float key = l;
    if (a.score_fn == 1) {
        const float sig = (float)(1.0 / (1.0 + exp(-(double)l)));
        key = sig + a.bias[e];
    }
    return key_bits(key);
}

// Top-k of row r by (key desc, index asc) with one wave.  Lane l owns the P
// experts l*P .. l*P+P-1 (contiguous) and keeps them sorted; each round takes
// the wave maximum of the lanes' heads.  Among equal keys the lowest lane
// wins, which (contiguous ownership, stable in-lane order) is the lowest
// expert index.  lr: the row's logits in LDS.
template <int P>
__device__ __forceinline__ void wave_topk(const SelectArgs& a, const float* lr, int r, SelectSmem& sm,
                                          bool weights = true) {
    const int lane = threadIdx.x & 63;
    const int E = a.E, k = a.k;
    uint32_t sk[P];
    int si[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int e = lane * P + p;
        uint32_t v = 0;
        if (e < E) {
            v = select_key(a, lr[e], e);
        }
        sk[p] = v;
        si[p] = p;
    }
    // stable insertion network, descending
#pragma unroll
    for (int i = 1; i < P; ++i) {
#pragma unroll
        for (int j = i; j > 0; --j) {
            const bool sw = sk[j] > sk[j - 1];
            const uint32_t ka = sk[j], kb = sk[j - 1];
            const int ia = si[j], ib = si[j - 1];
            sk[j - 1] = sw ? ka : kb; sk[j] = sw ? kb : ka;
            si[j - 1] = sw ? ia : ib; si[j] = sw ? ib : ia;
        }
    }
    int mine = 0;
    for (int j = 0; j < k; ++j) {
        const uint32_t head = sk[0];
        const uint32_t m = wave_max_u32(head);
        const unsigned long long mask = __ballot(head == m);
        const int L = __builtin_ctzll(mask);
        const int e = L * P + __builtin_amdgcn_readlane(si[0], L);
        if (lane == j) mine = e;
        if (lane == L) {
#pragma unroll
            for (int p = 0; p + 1 < P; ++p) { sk[p] = sk[p + 1]; si[p] = si[p + 1]; }
            sk[P - 1] = 0;
        }
    }
    if (!weights) {  // the caller needs the experts only
        if (lane < k) sm.sel[r * k + lane] = mine;
        return;
    }
    // mixture weights over the selection (routed scale not folded in)
    const float l = (lane < k) ? lr[mine] : 0.0f;
    float wv;
    if (a.score_fn == 0) {
        const float lmax = readlanef(l, 0);  // rank 0 holds the largest logit
        const float ex = (lane < k) ? expf(l - lmax) : 0.0f;
        const float s = wave_sum(ex);
        wv = ex / s;
    } else {
        const float sg = (lane < k) ? (float)(1.0 / (1.0 + exp(-(double)l))) : 0.0f;
        if (a.norm_topk) {
            const float s = wave_sum(sg);
            wv = sg / s;
        } else {
            wv = sg;
        }
    }
    if (lane < k) {
        sm.sel[r * k + lane] = mine;
        sm.w[r * k + lane] = wv;
    }
}

__device__ inline void wave_topk_rt(const SelectArgs& a, const float* lr, int r, SelectSmem& sm) {
    const int P = (a.E + 63) >> 6;
    if (P <= 1) wave_topk<1>(a, lr, r, sm);
    else if (P <= 2) wave_topk<2>(a, lr, r, sm);
    else if (P <= 4) wave_topk<4>(a, lr, r, sm);
    else if (P <= 8) wave_topk<8>(a, lr, r, sm);
    else wave_topk<16>(a, lr, r, sm);
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTileRows = 16;
constexpr int kSbCols = 256;

// Padded LDS layout of the fp16 x rows: 8 halfs of padding after every 64
// columns and 32 after each row, so the 64 lanes of an MFMA B-operand read
// (16 rows x 4 column blocks, 16 bytes each) spread over the banks.
__host__ __device__ constexpr int xh_row_stride(int H) { return H + (H / 64) * 8 + 32; }
__device__ __forceinline__ int xh_index(int m, int c, int H) { return m * xh_row_stride(H) + c + (c >> 6) * 8; }
constexpr int kMaxDynLds = 160 * 1024 - 1024;           // gfx950: 160 KiB per workgroup, minus static use

__device__ __forceinline__ uint32_t pick_word(const uint4& lo, const uint4& hi, int s) {
    const uint4& h = (s < 4) ? lo : hi;
    switch (s & 3) {
        case 0: return h.x;
        case 1: return h.y;
        case 2: return h.z;
        default: return h.w;
    }
}

// 8 FP4 codes (one dword) times one E4M3 scale -> 8 exact fp16 values
__device__ __forceinline__ f16x8_t decode8_f16(uint32_t codes, _Float16 scale) {
    const f16x2_t sc = {scale, scale};
    const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * sc;
    const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * sc;
    const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * sc;
    const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * sc;
    f16x8_t r;
    r[0] = p0.x; r[1] = p0.y; r[2] = p1.x; r[3] = p1.y;
    r[4] = p2.x; r[5] = p2.y; r[6] = p3.x; r[7] = p3.y;
    return r;
}

template <int SEL>
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t packed) {
    return (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)packed, SEL);
}

// ---------------------------------------------------------------------------
// x on the matrix cores.  bf16 activations enter the fp16 MFMA operands
// scaled by a power of two per row, 2^-sig with sig = ilogb(max_row |x|) - 14,
// so the row's largest magnitude lands in [2^14, 2^15): every bf16 value
// whose scaled magnitude is at least 2^-14 (those within 2^-28 of the row
// maximum) converts exactly, nothing overflows, and the accumulators are
// multiplied by 2^sig before the tensor scale.  Smaller values keep an
// absolute precision of 2^-24 * 2^sig, under 2^-38 of the row maximum.
// ---------------------------------------------------------------------------

// bf16 ones for every hidden column: the norm weight when none is given (one
// copy per translation unit).
static __device__ __align__(16) const uint16_t kBf16Ones[2048] = {
#define MOE_ONES8 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80
#define MOE_ONES64 MOE_ONES8, MOE_ONES8, MOE_ONES8, MOE_ONES8, MOE_ONES8, MOE_ONES8, MOE_ONES8, MOE_ONES8
#define MOE_ONES512 MOE_ONES64, MOE_ONES64, MOE_ONES64, MOE_ONES64, MOE_ONES64, MOE_ONES64, MOE_ONES64, MOE_ONES64
    MOE_ONES512, MOE_ONES512, MOE_ONES512, MOE_ONES512
#undef MOE_ONES512
#undef MOE_ONES64
#undef MOE_ONES8
};

// Larger of the two bf16 magnitudes in a packed pair, as magnitude bits
// (their integer order is the order of the magnitudes).
__device__ __forceinline__ uint32_t bf16pair_maxabs(uint32_t v) {
    return max(v & 0x7FFFu, (v >> 16) & 0x7FFFu);
}
__device__ __forceinline__ uint32_t bf16x8_maxabs(const uint4& v) {
    return max(max(bf16pair_maxabs(v.x), bf16pair_maxabs(v.y)), max(bf16pair_maxabs(v.z), bf16pair_maxabs(v.w)));
}

// sig of a row from the magnitude bits of its largest |x| (0 for an all-zero
// row; a row holding an infinity or NaN keeps sig 0 and propagates it).
__device__ __forceinline__ int row_sigma(uint32_t maxbits) {
    if (maxbits == 0u || maxbits >= 0x7F80u) return 0;
    return ilogbf(__uint_as_float(maxbits << 16)) - 14;
}

// A packed bf16 pair -> packed fp16 pair of the values times 2^-sig.
__device__ __forceinline__ uint32_t bf16pair_to_f16pair_scaled(uint32_t v, int neg_sig) {
    const f16x2_t h = {(_Float16)ldexpf(__uint_as_float(v << 16), neg_sig),
                       (_Float16)ldexpf(__uint_as_float(v & 0xFFFF0000u), neg_sig)};
    return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint4 bf16x8_to_f16x8_scaled(const uint4& v, int neg_sig) {
    uint4 o;
    o.x = bf16pair_to_f16pair_scaled(v.x, neg_sig);
    o.y = bf16pair_to_f16pair_scaled(v.y, neg_sig);
    o.z = bf16pair_to_f16pair_scaled(v.z, neg_sig);
    o.w = bf16pair_to_f16pair_scaled(v.w, neg_sig);
    return o;
}

// A 16-byte load marked non-temporal (global_load ... nt).  Used where a
// kernel streams a large matrix once and nothing re-reads it soon: measured
// on the lm_head stream it is 7% faster.  The MoE weight streams keep plain
// loads, since they measured slower with it (the verify layer's bursts are
// latency-bound, and the grouped kernels re-read experts across tiles).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
    const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// Code and scale registers of one superblock of one lane (gate and up).
struct GuSb {
    uint4 g0, g1, u0, u1;
    uint32_t gs, us;
};

// Lane (i = lane % 16, kb = lane / 16) of a 16-row tile: codes of gate and up
// row n0 + i at columns [sb*256 + kb*64, +64) (32 bytes each) and their four
// E4M3 scales; zeros when !live.
__device__ __forceinline__ GuSb gu_load_sb(const uint8_t* gq, const uint8_t* gs, const uint8_t* uq,
                                          const uint8_t* us, int H, int n0, int sb, bool live) {
    const int lane = threadIdx.x & 63;
    const int i = lane & 15, kb = lane >> 4;
    GuSb r;
    if (live) {
        const int k0 = sb * kSbCols + kb * 64;
        const size_t row = (size_t)(n0 + i);
        const uint8_t* qg = gq + row * (H / 2) + k0 / 2;
        const uint8_t* qu = uq + row * (H / 2) + k0 / 2;
        r.g0 = *reinterpret_cast<const uint4*>(qg);
        r.g1 = *reinterpret_cast<const uint4*>(qg + 16);
        r.u0 = *reinterpret_cast<const uint4*>(qu);
        r.u1 = *reinterpret_cast<const uint4*>(qu + 16);
        r.gs = *reinterpret_cast<const uint32_t*>(gs + row * (H / 16) + k0 / 16);
        r.us = *reinterpret_cast<const uint32_t*>(us + row * (H / 16) + k0 / 16);
    } else {
        r.g0 = r.g1 = r.u0 = r.u1 = make_uint4(0, 0, 0, 0);
        r.gs = r.us = 0;
    }
    return r;
}

}  // namespace moe
