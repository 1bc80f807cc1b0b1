// gfx950 kernels of the target's dense first layer (mlxfast README, "Why
// this challenge exists": layer 0 carries a dense SwiGLU MLP of intermediate
// 8192 instead of the MoE block), the first step of the prefill stack.
//
//   k_dense_gateup  g = x Wg^T and u = x Wu^T on v_mfma_f32_16x16x32_bf16
//                   (bf16 products are exact in fp32; fp32 sums), then
//                   h = silu(g) u in fp32, written as two bf16 values per
//                   element: hi = bf16(h), lo = bf16(h - hi) (16 significant
//                   bits between them, any magnitude);
//   k_dense_down    y = (hi + lo) Wd^T, two MFMAs per step into one fp32
//                   accumulator, over kDenseSplitK slices of the
//                   intermediate dimension (partial sums per slice);
//   k_dense_finish  one workgroup per row: the slices summed in slice order
//                   (+ residual), y32 and bf16 y, and the next layer's input
//                   bf16(gamma * y / sqrt(mean(y^2) + eps)).
//
// Three tile regimes (each deterministic; they group the k values of a
// 64-wide step into MFMA blocks differently, so their fp32 sums may differ
// in the last bits):
//   256 rows and more: k_dense_gateup_ring / k_dense_down_ring, 128 x 128
//     tiles on eight waves with both operands in a three-stage LDS ring
//     (described at those kernels);
//   65 .. 255 rows: 128-token x 64-column tiles (NTT = 8);
//   up to 64 rows: 64-token x 64-column tiles (NTT = 4).
// In the two register-staged regimes a workgroup covers 16 * NTT rows
// (tokens) x 64 output columns; wave w owns columns [16 w, 16 w + 16).  The weight rows are the MFMA A operand,
// read from global memory into registers one pipeline step ahead (lane
// (i, kb) holds 16 consecutive k values of weight row i); the token rows are
// the B operand, staged in LDS (double-buffered) and shared by the four
// waves.  The contraction order over k is the same permutation on both
// sides, so any lane assignment of k is valid.

#include "moe_device.h"

namespace moe {

typedef __bf16 dense_bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kDN = 64;                 // output columns per workgroup tile (4 waves x 16)
constexpr int kDK = 64;                 // k per pipeline step (2 MFMA k-blocks of 32)
constexpr int kDXStride = kDK + 8;      // LDS row stride in bf16 elements (144 B)
constexpr int kDenseSplitK = 4;         // slices of the intermediate dimension in the down GEMM

struct DenseArgs {
    const uint16_t* x;         // bf16 [T][H]
    const uint16_t* wg;        // bf16 [I][H]
    const uint16_t* wu;        // bf16 [I][H]
    const uint16_t* wd;        // bf16 [H][I]
    uint16_t* h_hi;            // bf16 [T][I]
    uint16_t* h_lo;            // bf16 [T][I]
    float* part;               // fp32 [kDenseSplitK][T][H]
    const uint16_t* residual;  // bf16 [T][H] or nullptr
    const uint16_t* gamma;     // bf16 [H] or nullptr (ones)
    float* y32;                // fp32 [T][H]
    uint16_t* y;               // bf16 [T][H] or nullptr
    uint16_t* x_next;          // bf16 [T][H] or nullptr
    float eps;
    int T, H, I;
};

__device__ __forceinline__ dense_bf16x8_t as_bf8(uint4 v) { return __builtin_bit_cast(dense_bf16x8_t, v); }

// Stage a (16 * NTT)-token x 64-k tile of a bf16 row-major [T][ld] matrix
// into LDS rows of kDXStride (tokens past T read row T - 1; never stored
// later): every thread moves NTT / 2 16-byte pieces.
template <int NTT>
__device__ __forceinline__ void dense_tile_load(const uint16_t* src, int ld, int t0, int T, int k0,
                                                uint4 (&v)[NTT / 2]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int p = 0; p < NTT / 2; ++p) {
        const int f = tid + p * kBlock;        // 16 * NTT rows x 8 pieces of 8 bf16
        const int r = f >> 3, c = (f & 7) * 8;
        const int t = min(t0 + r, T - 1);
        v[p] = *reinterpret_cast<const uint4*>(src + (size_t)t * ld + k0 + c);
    }
}
template <int NTT>
__device__ __forceinline__ void dense_tile_store(uint16_t* lds, const uint4 (&v)[NTT / 2]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int p = 0; p < NTT / 2; ++p) {
        const int f = tid + p * kBlock;
        const int r = f >> 3, c = (f & 7) * 8;
        *reinterpret_cast<uint4*>(lds + r * kDXStride + c) = v[p];
    }
}

// This lane's 16 k values (two 16-byte pieces) of weight row `row` at k0.
__device__ __forceinline__ void dense_w_load(const uint16_t* w, int ld, int row, int k0, uint4 (&v)[2]) {
    const int kb = (threadIdx.x & 63) >> 4;
    const uint4* p = reinterpret_cast<const uint4*>(w + (size_t)row * ld + k0 + kb * 16);
    v[0] = p[0];
    v[1] = p[1];
}

// B operand of MFMA step s for token tile tt: token row tt*16 + j, the same
// 8 k values as the A operand's lane (i, kb) at step s.
__device__ __forceinline__ dense_bf16x8_t dense_b(const uint16_t* lds, int tt, int s) {
    const int lane = threadIdx.x & 63, j = lane & 15, kb = lane >> 4;
    return *reinterpret_cast<const dense_bf16x8_t*>(lds + (tt * 16 + j) * kDXStride + kb * 16 + s * 8);
}

// ---------------------------------------------------------------------------
// gate/up + SwiGLU.  Grid: (I / 64, ceil(T / (16 * NTT))).
// ---------------------------------------------------------------------------
template <int NTT>
__global__ __launch_bounds__(kBlock) void k_dense_gateup(DenseArgs a) {
    constexpr int kDT = 16 * NTT;
    __shared__ __align__(16) uint16_t xs[2][kDT * kDXStride];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = lane & 15, q = lane >> 4;
    const int H = a.H, I = a.I, T = a.T;
    const int t0 = blockIdx.y * kDT;
    const int u0 = blockIdx.x * kDN + wave * 16;  // this wave's 16 units
    const int nsteps = H / kDK;
    f32x4_t accg[NTT], accu[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) accg[tt] = accu[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 gcur[2], ucur[2], gnext[2], unext[2], xv[NTT / 2];
    dense_w_load(a.wg, H, u0 + i, 0, gcur);
    dense_w_load(a.wu, H, u0 + i, 0, ucur);
    dense_tile_load<NTT>(a.x, H, t0, T, 0, xv);
    dense_tile_store<NTT>(xs[0], xv);
    __syncthreads();
    for (int step = 0; step < nsteps; ++step) {
        // the next step's operands in flight (the last step re-reads its own)
        const int kn = min(step + 1, nsteps - 1) * kDK;
        dense_w_load(a.wg, H, u0 + i, kn, gnext);
        dense_w_load(a.wu, H, u0 + i, kn, unext);
        dense_tile_load<NTT>(a.x, H, t0, T, kn, xv);
        const uint16_t* xb = xs[step & 1];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const dense_bf16x8_t ag = as_bf8(gcur[s]), au = as_bf8(ucur[s]);
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                const dense_bf16x8_t b = dense_b(xb, tt, s);
                accg[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag, b, accg[tt], 0, 0, 0);
                accu[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(au, b, accu[tt], 0, 0, 0);
            }
        }
        dense_tile_store<NTT>(xs[(step + 1) & 1], xv);
        __syncthreads();
        gcur[0] = gnext[0]; gcur[1] = gnext[1];
        ucur[0] = unext[0]; ucur[1] = unext[1];
    }
    // lane (j = i, q) holds units u0 + 4q .. +3 of token t0 + 16 tt + j
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
        const int t = t0 + tt * 16 + i;
        if (t >= T) continue;
        uint32_t hi2[2], lo2[2];
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
            uint16_t hb[2], lb[2];
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const float g = accg[tt][e + d], u = accu[tt][e + d];
                const float h = g / (1.0f + expf(-g)) * u;
                hb[d] = f32_to_bf16_rne(h);
                lb[d] = f32_to_bf16_rne(h - bf16_to_f32(hb[d]));
            }
            hi2[e / 2] = (uint32_t)hb[0] | ((uint32_t)hb[1] << 16);
            lo2[e / 2] = (uint32_t)lb[0] | ((uint32_t)lb[1] << 16);
        }
        const size_t o = (size_t)t * I + u0 + 4 * q;
        *reinterpret_cast<uint2*>(a.h_hi + o) = make_uint2(hi2[0], hi2[1]);
        *reinterpret_cast<uint2*>(a.h_lo + o) = make_uint2(lo2[0], lo2[1]);
    }
}

// ---------------------------------------------------------------------------
// down: partial y of one slice of the intermediate dimension.
// Grid: (H / 64, ceil(T / (16 * NTT)), kDenseSplitK).
// ---------------------------------------------------------------------------
template <int NTT>
__global__ __launch_bounds__(kBlock) void k_dense_down(DenseArgs a) {
    constexpr int kDT = 16 * NTT;
    __shared__ __align__(16) uint16_t hs[2][2][kDT * kDXStride];  // [buffer][hi, lo]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = lane & 15, q = lane >> 4;
    const int H = a.H, I = a.I, T = a.T;
    const int t0 = blockIdx.y * kDT;
    const int n0 = blockIdx.x * kDN + wave * 16;  // this wave's 16 output columns
    const int slice = I / kDenseSplitK, kbase = blockIdx.z * slice;
    const int nsteps = slice / kDK;
    f32x4_t acc[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 wcur[2], wnext[2], hv[NTT / 2], lv[NTT / 2];
    dense_w_load(a.wd, I, n0 + i, kbase, wcur);
    dense_tile_load<NTT>(a.h_hi, I, t0, T, kbase, hv);
    dense_tile_load<NTT>(a.h_lo, I, t0, T, kbase, lv);
    dense_tile_store<NTT>(hs[0][0], hv);
    dense_tile_store<NTT>(hs[0][1], lv);
    __syncthreads();
    for (int step = 0; step < nsteps; ++step) {
        const int kn = kbase + min(step + 1, nsteps - 1) * kDK;
        dense_w_load(a.wd, I, n0 + i, kn, wnext);
        dense_tile_load<NTT>(a.h_hi, I, t0, T, kn, hv);
        dense_tile_load<NTT>(a.h_lo, I, t0, T, kn, lv);
        const uint16_t* hb = hs[step & 1][0];
        const uint16_t* lb = hs[step & 1][1];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const dense_bf16x8_t aw = as_bf8(wcur[s]);
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, dense_b(hb, tt, s), acc[tt], 0, 0, 0);
                acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, dense_b(lb, tt, s), acc[tt], 0, 0, 0);
            }
        }
        dense_tile_store<NTT>(hs[(step + 1) & 1][0], hv);
        dense_tile_store<NTT>(hs[(step + 1) & 1][1], lv);
        __syncthreads();
        wcur[0] = wnext[0]; wcur[1] = wnext[1];
    }
    float* part = a.part + (size_t)blockIdx.z * T * H;
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
        const int t = t0 + tt * 16 + i;
        if (t < T)
            *reinterpret_cast<float4*>(part + (size_t)t * H + n0 + 4 * q) =
                make_float4(acc[tt][0], acc[tt][1], acc[tt][2], acc[tt][3]);
    }
}

// ---------------------------------------------------------------------------
// Prefill-sized calls (256 rows and more): 128-token x 128-column tiles on
// eight waves, both operands staged through a three-stage LDS ring by
// direct global-to-LDS loads (no registers hold a tile in flight).
//
// A stage is 48 KB: 48 blocks of 1 KB, each filled by one wave instruction
// (lane l's 16 bytes at byte 16 l of the block); wave w fills blocks
// 6w .. 6w + 5, so every wave has exactly Ring::Loads loads per stage in
// flight and a wait for "all but the newest stage" is vmcnt(Ring::Loads).
// Tiles are rows of 64 k values (8 pieces of 16 bytes); piece p of row r
// sits at position p ^ (r & 7) of its row, so the 16 rows an MFMA operand
// read touches spread over the banks.
// gate/up stage: x [128 tokens] then gate [128 units] then up [128 units].
// down stage:    h hi [128 tokens], h lo [128 tokens], then down [128 rows].
// ---------------------------------------------------------------------------

constexpr int kRingStages = 3;
constexpr int kRingRows = 384;                    // rows per stage
constexpr int kRingThreads = 512;                 // 8 waves
constexpr int kRingSplitK = 4;                    // down: slices of the intermediate dimension
// Ring geometry for a k step of KS (64: 48 KB stages, one workgroup per
// compute unit; 32 would give 24 KB stages and two, but more steps and
// barriers: slower): RB bytes per row, PP 16-byte pieces per row, and each
// wave's loads per stage.
template <int KS>
struct Ring {
    static constexpr int RB = KS * 2, PP = KS / 8;
    static constexpr int StageBytes = kRingRows * RB;
    static constexpr int LdsBytes = kRingStages * StageBytes;
    static constexpr int Loads = StageBytes / 1024 / (kRingThreads / 64);
};

// s_waitcnt with only the vector-memory count limited (to n <= 63)
#define DENSE_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// Issue this wave's loads of one stage: block c of the stage holds rows
// c * (1024 / RB) ..; row_src(r) gives the global row (KS k values from k0).
template <int KS, typename RowSrc>
__device__ __forceinline__ void ring_issue(unsigned char* stage, int k0, RowSrc&& row_src) {
    using G = Ring<KS>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int b = 0; b < G::Loads; ++b) {
        const int c = wave * G::Loads + b;
        const int r = c * (1024 / G::RB) + lane / G::PP, pos = lane % G::PP;
        const uint16_t* src = row_src(r) + k0 + ((pos ^ (r & (G::PP - 1))) << 3);
        __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                         (__attribute__((address_space(3))) void*)(stage + c * 1024), 16, 0, 0);
    }
}

// MFMA operand: 8 k values (piece p) of stage row r
template <int KS>
__device__ __forceinline__ dense_bf16x8_t ring_piece(const unsigned char* stage, int r, int p) {
    using G = Ring<KS>;
    return *reinterpret_cast<const dense_bf16x8_t*>(stage + r * G::RB + ((p ^ (r & (G::PP - 1))) << 4));
}

// gate/up + SwiGLU.  Grid: (I / 128, ceil(T / 128)).  Wave w: tokens
// 64 (w >> 2) .. +63, units 32 (w & 3) .. +31 of the tile.
template <int KS>
__global__ __launch_bounds__(kRingThreads) void k_dense_gateup_ring(DenseArgs a) {
    using G = Ring<KS>;
    extern __shared__ __align__(16) unsigned char ring[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = lane & 15, kb = lane >> 4;
    const int H = a.H, I = a.I, T = a.T;
    const int t0 = blockIdx.y * 128, u0 = blockIdx.x * 128;
    const int tw = (wave >> 2) * 64, uw = (wave & 3) * 32;
    const int nsteps = H / KS;
    auto row_src = [&](int r) -> const uint16_t* {
        const uint16_t* base = r < 128 ? a.x : (r < 256 ? a.wg : a.wu);
        const int row = r < 128 ? min(t0 + r, T - 1) : u0 + (r & 127);
        return base + (size_t)row * H;
    };
    f32x4_t accg[2][4], accu[2][4];
#pragma unroll
    for (int us = 0; us < 2; ++us)
#pragma unroll
        for (int ts = 0; ts < 4; ++ts) accg[us][ts] = accu[us][ts] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    ring_issue<KS>(ring, 0, row_src);
    ring_issue<KS>(ring + G::StageBytes, min(1, nsteps - 1) * KS, row_src);
    for (int step = 0; step < nsteps; ++step) {
        // this wave's part of this stage has landed (the next stage may still
        // be in flight); the barrier (no memory fence: that would wait for
        // every stage) makes every wave's part visible, and frees the slot
        // refilled below (each wave's reads of it finished in the last step)
        DENSE_WAIT_VM(G::Loads);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);  // no load or LDS read moves above the barrier
        ring_issue<KS>(ring + ((step + 2) % kRingStages) * G::StageBytes, min(step + 2, nsteps - 1) * KS, row_src);
        const unsigned char* st = ring + (step % kRingStages) * G::StageBytes;
#pragma unroll
        for (int kbk = 0; kbk < KS / 32; ++kbk) {
            const int p = kbk * 4 + kb;
            dense_bf16x8_t ag[2], au[2], bx[4];
#pragma unroll
            for (int us = 0; us < 2; ++us) {
                ag[us] = ring_piece<KS>(st, 128 + uw + us * 16 + i, p);
                au[us] = ring_piece<KS>(st, 256 + uw + us * 16 + i, p);
            }
#pragma unroll
            for (int ts = 0; ts < 4; ++ts) bx[ts] = ring_piece<KS>(st, tw + ts * 16 + i, p);
#pragma unroll
            for (int us = 0; us < 2; ++us)
#pragma unroll
                for (int ts = 0; ts < 4; ++ts) {
                    accg[us][ts] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag[us], bx[ts], accg[us][ts], 0, 0, 0);
                    accu[us][ts] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(au[us], bx[ts], accu[us][ts], 0, 0, 0);
                }
        }
    }
    DENSE_WAIT_VM(0);  // the trailing (repeated) stages' loads are done before the workgroup ends
    // lane (j = i, q = kb) holds units 4q .. 4q + 3 of its 16-unit block, token 16 ts + j
#pragma unroll
    for (int us = 0; us < 2; ++us)
#pragma unroll
        for (int ts = 0; ts < 4; ++ts) {
            const int t = t0 + tw + ts * 16 + i;
            if (t >= T) continue;
            uint32_t hi2[2], lo2[2];
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                uint16_t hb[2], lb[2];
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    const float g = accg[us][ts][e + d], u = accu[us][ts][e + d];
                    const float h = g / (1.0f + expf(-g)) * u;
                    hb[d] = f32_to_bf16_rne(h);
                    lb[d] = f32_to_bf16_rne(h - bf16_to_f32(hb[d]));
                }
                hi2[e / 2] = (uint32_t)hb[0] | ((uint32_t)hb[1] << 16);
                lo2[e / 2] = (uint32_t)lb[0] | ((uint32_t)lb[1] << 16);
            }
            const size_t o = (size_t)t * I + u0 + uw + us * 16 + 4 * kb;
            *reinterpret_cast<uint2*>(a.h_hi + o) = make_uint2(hi2[0], hi2[1]);
            *reinterpret_cast<uint2*>(a.h_lo + o) = make_uint2(lo2[0], lo2[1]);
        }
}

// down: partial y of one slice of the intermediate dimension.
// Grid: (H / 128, ceil(T / 128), kRingSplitK).  Wave w: tokens 64 (w >> 2)
// .. +63, output columns 32 (w & 3) .. +31 of the tile.
template <int KS>
__global__ __launch_bounds__(kRingThreads) void k_dense_down_ring(DenseArgs a) {
    using G = Ring<KS>;
    extern __shared__ __align__(16) unsigned char ring[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = lane & 15, kb = lane >> 4;
    const int H = a.H, I = a.I, T = a.T;
    const int t0 = blockIdx.y * 128, n0 = blockIdx.x * 128;
    const int tw = (wave >> 2) * 64, nw = (wave & 3) * 32;
    const int slice = I / kRingSplitK, kbase = blockIdx.z * slice;
    const int nsteps = slice / KS;
    auto row_src = [&](int r) -> const uint16_t* {
        const uint16_t* base = r < 128 ? a.h_hi : (r < 256 ? a.h_lo : a.wd);
        const int row = r < 256 ? min(t0 + (r & 127), T - 1) : n0 + (r & 127);
        return base + (size_t)row * I;
    };
    f32x4_t acc[2][4];
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
#pragma unroll
        for (int ts = 0; ts < 4; ++ts) acc[ns][ts] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    ring_issue<KS>(ring, kbase, row_src);
    ring_issue<KS>(ring + G::StageBytes, kbase + min(1, nsteps - 1) * KS, row_src);
    for (int step = 0; step < nsteps; ++step) {
        DENSE_WAIT_VM(G::Loads);  // as in k_dense_gateup_ring
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        ring_issue<KS>(ring + ((step + 2) % kRingStages) * G::StageBytes, kbase + min(step + 2, nsteps - 1) * KS,
                       row_src);
        const unsigned char* st = ring + (step % kRingStages) * G::StageBytes;
#pragma unroll
        for (int kbk = 0; kbk < KS / 32; ++kbk) {
            const int p = kbk * 4 + kb;
            dense_bf16x8_t aw[2], bh[4], bl[4];
#pragma unroll
            for (int ns = 0; ns < 2; ++ns) aw[ns] = ring_piece<KS>(st, 256 + nw + ns * 16 + i, p);
#pragma unroll
            for (int ts = 0; ts < 4; ++ts) {
                bh[ts] = ring_piece<KS>(st, tw + ts * 16 + i, p);
                bl[ts] = ring_piece<KS>(st, 128 + tw + ts * 16 + i, p);
            }
#pragma unroll
            for (int ns = 0; ns < 2; ++ns)
#pragma unroll
                for (int ts = 0; ts < 4; ++ts) {
                    acc[ns][ts] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[ns], bh[ts], acc[ns][ts], 0, 0, 0);
                    acc[ns][ts] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[ns], bl[ts], acc[ns][ts], 0, 0, 0);
                }
        }
    }
    DENSE_WAIT_VM(0);
    float* part = a.part + (size_t)blockIdx.z * T * H;
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
#pragma unroll
        for (int ts = 0; ts < 4; ++ts) {
            const int t = t0 + tw + ts * 16 + i;
            if (t < T)
                *reinterpret_cast<float4*>(part + (size_t)t * H + n0 + nw + ns * 16 + 4 * kb) =
                    make_float4(acc[ns][ts][0], acc[ns][ts][1], acc[ns][ts][2], acc[ns][ts][3]);
        }
}

// ---------------------------------------------------------------------------
// finish: one workgroup per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_dense_finish(DenseArgs a) {
    __shared__ float s_part[kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = blockIdx.x, H = a.H, T = a.T;
    constexpr int kMaxPer = 8;  // hidden <= 2048
    float yv[kMaxPer];
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < kMaxPer; ++c) {
        const int n = tid + c * kBlock;
        yv[c] = 0.0f;
        if (n < H) {
            float y = a.part[(size_t)t * H + n];
#pragma unroll
            for (int z = 1; z < kDenseSplitK; ++z) y += a.part[((size_t)z * T + t) * H + n];
            if (a.residual) y += bf16_to_f32(a.residual[(size_t)t * H + n]);
            a.y32[(size_t)t * H + n] = y;
            if (a.y) a.y[(size_t)t * H + n] = f32_to_bf16_rne(y);
            yv[c] = y;
            ss = fmaf(y, y, ss);
        }
    }
    if (!a.x_next) return;
    ss = wave_sum(ss);
    if (lane == 0) s_part[wave] = ss;
    __syncthreads();
    const float tot = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
    const float inv = 1.0f / sqrtf(tot / (float)H + a.eps);
#pragma unroll
    for (int c = 0; c < kMaxPer; ++c) {
        const int n = tid + c * kBlock;
        if (n < H) {
            const float gm = a.gamma ? bf16_to_f32(a.gamma[n]) : 1.0f;
            a.x_next[(size_t)t * H + n] = f32_to_bf16_rne(yv[c] * inv * gm);
        }
    }
}

// ---------------------------------------------------------------------------
// launcher and sizes
// ---------------------------------------------------------------------------

static_assert(kRingSplitK == kDenseSplitK, "the finish kernel sums kDenseSplitK partial slices");

bool dense_shape_ok(int H, int I) {
    return H >= kDN && H % kDN == 0 && H <= 2048 && I >= kDenseSplitK * kDK && I % (kDenseSplitK * kDK) == 0 &&
           I % kDN == 0;
}

size_t dense_workspace_bytes(int H, int I, int T) {
    const size_t hh = (size_t)T * I * 2 * 2;                 // hi + lo
    const size_t part = (size_t)kDenseSplitK * T * H * 4;
    return ((hh + 255) / 256 + (part + 255) / 256) * 256;
}

hipError_t launch_dense_mlp(const uint16_t* x, int T, int H, int I, const uint16_t* wg, const uint16_t* wu,
                            const uint16_t* wd, const uint16_t* residual, const uint16_t* gamma, float eps, float* y32,
                            uint16_t* y, uint16_t* x_next, void* workspace, hipStream_t st) {
    DenseArgs a{};
    a.x = x; a.wg = wg; a.wu = wu; a.wd = wd;
    char* ws = reinterpret_cast<char*>(workspace);
    a.h_hi = reinterpret_cast<uint16_t*>(ws);
    a.h_lo = a.h_hi + (size_t)T * I;
    a.part = reinterpret_cast<float*>(ws + ((size_t)T * I * 4 + 255) / 256 * 256);
    a.residual = residual; a.gamma = gamma;
    a.y32 = y32; a.y = y; a.x_next = x_next;
    a.eps = eps;
    a.T = T; a.H = H; a.I = I;
    // prefill-sized calls: the LDS-ring kernels (128 x 128 tiles, one
    // workgroup per compute unit); 128-token tiles above 64 rows (each
    // weight row loaded once per 128 tokens), 64-token tiles below
    constexpr int KS = 64;
    using G = Ring<KS>;
    static const hipError_t ring_attr = [] {
        hipError_t r = hipFuncSetAttribute(reinterpret_cast<const void*>(k_dense_gateup_ring<KS>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, G::LdsBytes);
        if (r == hipSuccess)
            r = hipFuncSetAttribute(reinterpret_cast<const void*>(k_dense_down_ring<KS>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, G::LdsBytes);
        return r;
    }();
    if (T >= 256 && H % 128 == 0 && I % 128 == 0) {
        if (ring_attr != hipSuccess) return ring_attr;
        const int tt = (T + 127) / 128;
        hipLaunchKernelGGL(k_dense_gateup_ring<KS>, dim3(I / 128, tt), dim3(kRingThreads), G::LdsBytes, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_dense_down_ring<KS>, dim3(H / 128, tt, kRingSplitK), dim3(kRingThreads), G::LdsBytes,
                           st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (T > 64) {
        const int tt = (T + 127) / 128;
        hipLaunchKernelGGL(k_dense_gateup<8>, dim3(I / kDN, tt), dim3(kBlock), 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_dense_down<8>, dim3(H / kDN, tt, kDenseSplitK), dim3(kBlock), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
        hipLaunchKernelGGL(k_dense_gateup<4>, dim3(I / kDN, 1), dim3(kBlock), 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_dense_down<4>, dim3(H / kDN, 1, kDenseSplitK), dim3(kBlock), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_dense_finish, dim3(T), dim3(kBlock), 0, st, a);
    return hipGetLastError();
}

}  // namespace moe
