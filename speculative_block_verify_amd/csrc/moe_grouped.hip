// gfx950 (CDNA4) kernels of the NVFP4 MoE layer in the grouped (prefill)
// regime: more than 16 rows, so each routed expert serves many tokens and the
// expert GEMMs are dense contractions for the matrix cores (the 512-row seed
// prefill of the mlxfast README, "Why this challenge exists"; PR #844
// section 8 notes the stock grouped GEMM needs several tokens per expert).
// Per layer, after the router GEMV on the matrix cores (k_router_mfma; up
// to 16 rows k_router_split, its column slices as workgroups of their own):
//   k_select_rows   top-k and mixture weights, one wave per row (the same
//                   selection code as the verify-width path; up to 16 rows
//                   k_select_rows_split, which first adds the router's
//                   partial logits and makes the fp16 copy of x);
//   k_gateup_grouped  every workgroup first groups the T*k slots itself in
//                   LDS: the canonical CSR by expert (unique experts
//                   ascending, slots ascending), a tile list of up to 32
//                   consecutive slots of one expert (plus the shared
//                   expert's 32-token tiles) and its own tiles' token rows,
//                   from counts, prefix sums and row bitmaps of the slot
//                   ids; workgroup 0 publishes the CSR and the tile list for
//                   the down and combine kernels.  Then (tile, 64
//                   intermediate rows) work items on the matrix
//                   cores: FP4 codes decoded in registers to fp16 times their
//                   E4M3 scale (exact), x columns staged in LDS as fp16 (the
//                   router's copy, x * 2^-sig per row, undone in the epilogue),
//                   v_mfma_f32_16x16x32_f16 with fp32 accumulation, SwiGLU
//                   epilogue writing fp32 h and each token's max |h| per slab;
//   k_down_grouped  (tile, 64 output rows) work items: h staged in LDS as a
//                   pair of fp16 values hi + lo of h * 2^-sigma, sigma a
//                   power of two per token chosen from its max |h| (so the
//                   pair keeps about 22 significant bits and cannot
//                   overflow), two MFMAs per k step into one fp32 accumulator,
//                   2^sigma and the tensor scale applied to the sum;
//   k_combine       one workgroup per row: y = rs * sum_j w_j o_j + shared
//                   (+ residual) in rank order (PR #844 section 5 expression
//                   order), y32 / bf16 y, and for stacked layers the next
//                   layer's bf16 RMS-normalised input.

#include "moe_device.h"

namespace moe {

// ---------------------------------------------------------------------------
// k_router_mfma: logits = x Wr^T for many rows on the matrix cores
//
// Workgroup tile: 32 rows x 16 experts (a grid that covers every compute
// unit at 512 rows), 8 waves; wave w sums the columns [w*H/8, (w+1)*H/8)
// for the whole tile (two 16x16 accumulators), with
// every operand load of the wave issued before its first MFMA, and the eight
// partial tiles are added in wave order through LDS.  MFMA step over 32
// columns c..c+31: lane (i, kb) feeds row i's columns c + 8kb .. +7 of x as
// its A k-block and of the router as its B k-block.  bf16 products are exact
// in fp32; rows past T and experts past E are read at clamped indices and
// not stored.
// ---------------------------------------------------------------------------

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));


template <int H>
__global__ __launch_bounds__(kRouterWaves * 64) void k_router_mfma(RouterArgs a) {
    __shared__ f32x4_t part[kRouterWaves - 1][2][64];
    __shared__ uint32_t s_xmax[kRouterWaves][32];  // per wave: largest |x| of each of the tile's rows
    constexpr int NS = H / kRouterWaves / 32;  // MFMA steps per wave
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i = lane & 15, kb = lane >> 4;
    const int T = a.K, E = a.E;
    const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 16;
    const int c0 = wave * (H / kRouterWaves) + 8 * kb;
    const uint16_t* xr0 = a.x_in + (size_t)min(t0 + i, T - 1) * H + c0;
    const uint16_t* xr1 = a.x_in + (size_t)min(t0 + 16 + i, T - 1) * H + c0;
    const uint16_t* wr0 = a.wr + (size_t)min(e0 + i, E - 1) * H + c0;
    uint4 x0[NS], x1[NS], w0[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        x0[s] = *reinterpret_cast<const uint4*>(xr0 + 32 * s);
        x1[s] = *reinterpret_cast<const uint4*>(xr1 + 32 * s);
        w0[s] = *reinterpret_cast<const uint4*>(wr0 + 32 * s);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the MFMAs
    f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, x0[s]), a1 = __builtin_bit_cast(bf16x8_t, x1[s]);
        const bf16x8_t b0 = __builtin_bit_cast(bf16x8_t, w0[s]);
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b0, acc[1], 0, 0, 0);
    }
    if (wave > 0) {
#pragma unroll
        for (int t = 0; t < 2; ++t) part[wave - 1][t][lane] = acc[t];
    }
    if (a.x_f16) {
        // largest |x| of rows i and 16 + i over this wave's columns (lanes
        // i, i + 16, i + 32, i + 48 hold them)
        uint32_t m0 = 0u, m1 = 0u;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            m0 = max(m0, bf16x8_maxabs(x0[s]));
            m1 = max(m1, bf16x8_maxabs(x1[s]));
        }
        m0 = max(m0, (uint32_t)__shfl_xor((int)m0, 16, 64));
        m0 = max(m0, (uint32_t)__shfl_xor((int)m0, 32, 64));
        m1 = max(m1, (uint32_t)__shfl_xor((int)m1, 16, 64));
        m1 = max(m1, (uint32_t)__shfl_xor((int)m1, 32, 64));
        if (kb == 0) {
            s_xmax[wave][i] = m0;
            s_xmax[wave][16 + i] = m1;
        }
    }
    __syncthreads();
    if (a.x_f16) {
        // The fp16 copy of x that the grouped gate/up kernel stages (bf16 ->
        // fp16 once per row, not per tile), scaled by the row's 2^-sig: each
        // wave's column range is written by one workgroup of the row tile's
        // column of workgroups (every one of them finds the same maxima).
        uint32_t m0 = 0u, m1 = 0u;
#pragma unroll
        for (int w = 0; w < kRouterWaves; ++w) {
            m0 = max(m0, s_xmax[w][i]);
            m1 = max(m1, s_xmax[w][16 + i]);
        }
        const int sg0 = row_sigma(m0), sg1 = row_sigma(m1);
        if (wave % gridDim.y == blockIdx.y) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const uint4 h0 = bf16x8_to_f16x8_scaled(x0[s], -sg0), h1 = bf16x8_to_f16x8_scaled(x1[s], -sg1);
                if (t0 + i < T) *reinterpret_cast<uint4*>(a.x_f16 + (size_t)(t0 + i) * H + c0 + 32 * s) = h0;
                if (t0 + 16 + i < T) *reinterpret_cast<uint4*>(a.x_f16 + (size_t)(t0 + 16 + i) * H + c0 + 32 * s) = h1;
            }
        }
        if (blockIdx.y == 0 && wave == 0 && kb == 0) {
            if (t0 + i < T) a.x_sig[t0 + i] = sg0;
            if (t0 + 16 + i < T) a.x_sig[t0 + 16 + i] = sg1;
        }
    }
    if (wave == 0) {
        // accumulator t = row half; lane (j = lane % 16, q = lane / 16) holds
        // rows 4q .. 4q+3 of expert column j
        const int j = lane & 15, q = lane >> 4;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4_t v = acc[t];
#pragma unroll
            for (int w = 0; w < kRouterWaves - 1; ++w) v += part[w][t][lane];
            const int e = e0 + j;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = t0 + 16 * t + 4 * q + r;
                if (row < T && e < E) a.logits[(size_t)row * E + e] = v[r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// k_router_split: the same logits for up to 16 rows, each column slice of
// k_router_mfma's waves as a one-wave workgroup of its own: (E/16) x 8
// workgroups instead of E/16, so the router rows stream from 8x the compute
// units.  Slice z's MFMA chain is wave z's chain of k_router_mfma (rows
// 0..15), and its 16x16 partial tile goes to a.logits[z][row][e];
// k_select_rows_split adds the slices in order, which is the order the
// many-row kernel adds its waves' tiles, so the logits are the same bits.
// ---------------------------------------------------------------------------

template <int H>
__global__ __launch_bounds__(64) void k_router_split(RouterArgs a) {
    constexpr int NS = H / kRouterWaves / 32;  // MFMA steps per slice
    const int lane = threadIdx.x, i = lane & 15, kb = lane >> 4;
    const int T = a.K, E = a.E;
    const int e0 = blockIdx.x * 16, z = blockIdx.y;
    const int c0 = z * (H / kRouterWaves) + 8 * kb;
    const uint16_t* xr0 = a.x_in + (size_t)min(i, T - 1) * H + c0;
    const uint16_t* wr0 = a.wr + (size_t)min(e0 + i, E - 1) * H + c0;
    uint4 x0[NS], w0[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        x0[s] = *reinterpret_cast<const uint4*>(xr0 + 32 * s);
        w0[s] = *reinterpret_cast<const uint4*>(wr0 + 32 * s);
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x0[s]),
                                                      __builtin_bit_cast(bf16x8_t, w0[s]), acc, 0, 0, 0);
    // lane (j, q) holds rows 4q .. 4q+3 of expert column j
    const int j = lane & 15, q = lane >> 4, e = e0 + j;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * q + r;
        if (row < T && e < E) a.logits[((size_t)z * T + row) * E + e] = acc[r];
    }
}

// ---------------------------------------------------------------------------
// k_select_rows: kWaves rows per workgroup
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kBlock) void k_select_rows(SelectArgs a) {
    __shared__ SelectSmem sm;
    extern __shared__ __align__(16) float lg[];  // [kWaves][E]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r0 = blockIdx.x * kWaves;
    const int nr = min(kWaves, a.K - r0);
    stage_floats(lg, a.logits + (size_t)r0 * a.E, nr * a.E, tid, kBlock);
    __syncthreads();
    if (wave < nr) {
        wave_topk_rt(a, lg + wave * a.E, wave, sm);
        // each lane reads back the entry it wrote itself
        if (lane < a.k) {
            a.ids[(size_t)(r0 + wave) * a.k + lane] = sm.sel[wave * a.k + lane];
            a.w[(size_t)(r0 + wave) * a.k + lane] = sm.w[wave * a.k + lane];
        }
    }
}

// k_select_rows with the router's slice partials added first (slice order)
// and the summed logits stored; each row's wave also writes the row's fp16
// copy of x and its exponent, as k_router_mfma does for many rows.
__global__ __launch_bounds__(kBlock) void k_select_rows_split(SelectSplitArgs a) {
    __shared__ SelectSmem sm;
    extern __shared__ __align__(16) float lg[];  // [kWaves][E]
    const SelectArgs& sa = a.s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = sa.K, E = sa.E, H = a.H;
    const int r0 = blockIdx.x * kWaves;
    const int nr = min(kWaves, K - r0);
    // this thread's logits (E <= kRouterSplitMaxExperts: at most four), every
    // slice's partial requested before the first is added
    static_assert(kWaves * kRouterSplitMaxExperts <= 4 * kBlock, "more than four logits per thread");
    float pv[4][kRouterWaves];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int t = tid + u * kBlock;
        const float* p = a.parts + (size_t)r0 * E + min(t, nr * E - 1);
#pragma unroll
        for (int z = 0; z < kRouterWaves; ++z) pv[u][z] = p[(size_t)z * K * E];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int t = tid + u * kBlock;
        float v = pv[u][0];
#pragma unroll
        for (int z = 1; z < kRouterWaves; ++z) v += pv[u][z];
        if (t < nr * E) {
            lg[t] = v;
            a.logits[(size_t)r0 * E + t] = v;
        }
    }
    if (wave < nr) {
        // the row's largest |x| -> its exponent, then the scaled fp16 copy
        // (H <= 2048: at most four 8-column pieces per lane)
        const int r = r0 + wave, n8 = H / 8;
        const uint4* xr = reinterpret_cast<const uint4*>(a.x_in + (size_t)r * H);
        uint4 v[4];
        uint32_t m = 0u;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int c = lane + 64 * t;
            v[t] = c < n8 ? xr[c] : make_uint4(0, 0, 0, 0);
            m = max(m, bf16x8_maxabs(v[t]));
        }
        const int sg = row_sigma(wave_max_u32(m));
        if (lane == 0) a.x_sig[r] = sg;
        uint4* xo = reinterpret_cast<uint4*>(a.x_f16 + (size_t)r * H);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int c = lane + 64 * t;
            if (c < n8) xo[c] = bf16x8_to_f16x8_scaled(v[t], -sg);
        }
    }
    __syncthreads();
    if (wave < nr) {
        wave_topk_rt(sa, lg + wave * E, wave, sm);
        if (lane < sa.k) {
            sa.ids[(size_t)(r0 + wave) * sa.k + lane] = sm.sel[wave * sa.k + lane];
            sa.w[(size_t)(r0 + wave) * sa.k + lane] = sm.w[wave * sa.k + lane];
        }
    }
}

// The grouping kernel's dynamic LDS: 4 bytes per (expert, 32-row word) of
// bitmap, plus 2 bytes of prefix count when that still fits.
constexpr int kGroupMaxLds = kMaxExperts * (kMaxGroupedRows / 32) * 4;
constexpr int kGroupLdsSlots = 4096;  // slot lists up to this length are ordered in LDS
constexpr int kGroupRegSlots = 8;     // slots per grouping thread whose expert ids stay in registers
__host__ __device__ inline bool group_pc_fits(int T, int E) {
    return (size_t)E * ((T + 31) / 32) * 6 <= (size_t)kGroupMaxLds;
}

// ---------------------------------------------------------------------------
// k_group: CSR + tile list (one workgroup of kGGroupThreads), for the
// routing-only entry point at grouped row counts (a layer groups inside its
// gate/up kernel)
//
// A row never selects an expert twice, so expert e's slots are one per row
// that picked it, in row order.  rm[w][e] is the bitmap of those rows
// (word w covers rows 32w .. 32w + 31; stored word-major, so the experts'
// threads read consecutive words):
//   count(e) = popcount(rm[*][e]),
//   rank of slot (r, j) inside its expert = popcount of rm[.][e] below bit r.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kGGroupThreads) void k_group(GroupArgs a) {
    // [W][E] row bitmaps, then (when group_pc_fits) [W][E] 16-bit prefix
    // popcounts: slots of expert e in rows below word w
    extern __shared__ uint32_t rm[];
    __shared__ int s_cstart[kMaxExperts];
    __shared__ int s_wsum[kGGroupThreads / 64][3];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = a.T, E = a.E, k = a.k, n = T * k, W = (T + 31) >> 5;
    const bool use_pc = group_pc_fits(T, E);
    if (a.status && tid == 0) *a.status = 0;
    uint16_t* pc = reinterpret_cast<uint16_t*>(rm + E * W);
    // the slot list is assembled in the static LDS buffer when it fits
    __shared__ int s_asg[kGroupLdsSlots];
    const bool use_lds_asg = n <= kGroupLdsSlots;
    // this thread's slots s = tid + i * kGGroupThreads; the expert ids of the
    // first kGroupRegSlots stay in registers, later ones are read again
    constexpr int kSlots = kMaxGroupedRows * kMaxTopK / kGGroupThreads;
    int ev[kGroupRegSlots];
#pragma unroll
    for (int i = 0; i < kGroupRegSlots; ++i) {
        const int s = tid + i * kGGroupThreads;
        ev[i] = s < n ? a.ids[s] : 0;
    }
    auto expert_of = [&](int i, int s) { return i < kGroupRegSlots ? ev[i < kGroupRegSlots ? i : 0] : a.ids[s]; };
    for (int i = tid; i < E * W; i += kGGroupThreads) rm[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        const int s = tid + i * kGGroupThreads;
        if (s < n) {
            const int r = s / k;
            atomicOr(&rm[(r >> 5) * E + expert_of(i, s)], 1u << (r & 31));
        }
    }
    __syncthreads();
    // thread e (E <= kGGroupThreads): slot count (and prefix per word), used
    // flag, tile count
    int c = 0;
    if (tid < E)
        for (int w = 0; w < W; ++w) {
            if (use_pc) pc[w * E + tid] = (uint16_t)c;
            c += __builtin_popcount(rm[w * E + tid]);
        }
    const int f = c > 0, nt = (c + kGChunk - 1) / kGChunk;
    const int ci = wave_incl_scan(c), fi = wave_incl_scan(f), ti = wave_incl_scan(nt);
    if (lane == 63) {
        s_wsum[wave][0] = ci;
        s_wsum[wave][1] = fi;
        s_wsum[wave][2] = ti;
    }
    __syncthreads();
    int cb = 0, fb = 0, tb = 0;
    for (int w = 0; w < wave; ++w) {
        cb += s_wsum[w][0];
        fb += s_wsum[w][1];
        tb += s_wsum[w][2];
    }
    const int cs = cb + ci - c, fs = fb + fi - f, tsn = tb + ti - nt;
    int4* tiles = reinterpret_cast<int4*>(a.tiles);
    if (tid < E) {
        s_cstart[tid] = cs;
        if (f) {
            a.uniq[fs] = tid;
            a.off[fs] = cs;
            for (int t = 0; t < nt; ++t) tiles[tsn + t] = make_int4(tid, cs + t * kGChunk, min(kGChunk, c - t * kGChunk), 0);
        }
    }
    if (tid == kGGroupThreads - 1) {
        int U = 0, NT = 0;
        for (int w = 0; w < kGGroupThreads / 64; ++w) {
            U += s_wsum[w][1];
            NT += s_wsum[w][2];
        }
        *a.n_unique = U;
        a.off[U] = n;
        int nsh = 0;
        if (a.has_shared) {
            nsh = (T + kGChunk - 1) / kGChunk;
            for (int t = 0; t < nsh; ++t) tiles[NT + t] = make_int4(-1, t * kGChunk, min(kGChunk, T - t * kGChunk), 0);
        }
        *a.n_tiles = NT + nsh;
    }
    __syncthreads();
    // rank of slot (r, j) inside its expert = slots of the expert in rows
    // below the word holding row r, plus the bits below r in that word
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        const int s = tid + i * kGGroupThreads;
        if (s < n) {
            const int e = expert_of(i, s), r = s / k;
            const uint32_t* m = rm + e;  // word w at m[w * E]
            int rank = __builtin_popcount(m[(r >> 5) * E] & ((1u << (r & 31)) - 1u));
            if (use_pc) {
                rank += pc[(r >> 5) * E + e];
            } else {
                for (int w = 0; w < (r >> 5); ++w) rank += __builtin_popcount(m[w * E]);
            }
            const int pos = s_cstart[e] + rank;
            if (use_lds_asg) s_asg[pos] = s;
            else a.asg[pos] = s;
            a.inv[s] = pos;
        }
    }
    if (use_lds_asg) {
        // the slot list leaves in position order: contiguous stores
        __syncthreads();
        for (int p = tid; p < n; p += kGGroupThreads) a.asg[p] = s_asg[p];
    }
}

// ---------------------------------------------------------------------------
// grouped gate/up
//
// Work item: (tile, 64-row slab of the intermediate dimension).  Wave w
// computes rows n0 = slab*64 + 16w .. +15 of gate and of up for the tile's
// tokens (up to 32: two 16-column MFMA tiles).  Lane (i = lane % 16,
// kb = lane / 16) owns columns [sb*256 + kb*64, +64) of weight row n0 + i in
// superblock sb (the layout of the verify-width tiles); its weights stream
// through the superblocks with four superblocks in flight.  The tokens' x
// columns of the current superblock sit in LDS as fp16 (double buffered),
// rows padded to 528 bytes (16 bytes times an odd number) so the 16 rows an
// MFMA B read touches fall in distinct bank groups.
// ---------------------------------------------------------------------------

constexpr int kGXStride = kSbCols + 8;  // halfs per staged token row
constexpr int kGuMaxItems = 16;          // work items of one persistent gate/up workgroup
constexpr int kGuGrid = 512;             // persistent gate/up workgroups (two per compute unit)

// One superblock's eight MFMA steps, software pipelined: step s + 1's x
// columns are read from LDS and its weights decoded before step s's MFMAs
// issue, so neither the LDS round trip nor the decode waits behind the
// matrix core.  Both 16-token column tiles are always multiplied: an item of
// at most 16 tokens has zeros in the second tile's x rows and its results
// are not stored.  The steps then hold no branch, which is what lets the
// compiler interleave the decode with the MFMAs (a per-step branch on the
// tile count kept every LDS read right before its MFMA); a scheduling
// barrier closes each step, so the decoded operands of at most two steps
// are in registers.
__device__ __forceinline__ void gg_mfma_sb(const GuSb& r, const _Float16* xb, f32x4_t* accg, f32x4_t* accu) {
    const int lane = threadIdx.x & 63, j = lane & 15, kb = lane >> 4;
    const _Float16 g0 = e4m3_to_f16<0>(r.gs), g1 = e4m3_to_f16<1>(r.gs);
    const _Float16 g2 = e4m3_to_f16<2>(r.gs), g3 = e4m3_to_f16<3>(r.gs);
    const _Float16 u0 = e4m3_to_f16<0>(r.us), u1 = e4m3_to_f16<1>(r.us);
    const _Float16 u2 = e4m3_to_f16<2>(r.us), u3 = e4m3_to_f16<3>(r.us);
    const _Float16* xr = xb + j * kGXStride + kb * 64;
    auto dec_g = [&](int s) { return decode8_f16(pick_word(r.g0, r.g1, s), (s < 2) ? g0 : (s < 4) ? g1 : (s < 6) ? g2 : g3); };
    auto dec_u = [&](int s) { return decode8_f16(pick_word(r.u0, r.u1, s), (s < 2) ? u0 : (s < 4) ? u1 : (s < 6) ? u2 : u3); };
    f16x8_t b[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) b[t] = *reinterpret_cast<const f16x8_t*>(xr + 16 * t * kGXStride);
    f16x8_t ag = dec_g(0), au = dec_u(0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        f16x8_t nb[2], nag = ag, nau = au;
        if (s < 7) {
#pragma unroll
            for (int t = 0; t < 2; ++t) nb[t] = *reinterpret_cast<const f16x8_t*>(xr + 16 * t * kGXStride + 8 * (s + 1));
            nag = dec_g(s + 1);
            nau = dec_u(s + 1);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            accg[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ag, b[t], accg[t], 0, 0, 0);
            accu[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(au, b[t], accu[t], 0, 0, 0);
        }
        if (s < 7) {
#pragma unroll
            for (int t = 0; t < 2; ++t) b[t] = nb[t];
            ag = nag;
            au = nau;
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The set-up's grouping tables, in the x double buffer before its first use:
// per expert its slot count, first CSR position and first routed tile, and
// the local index of the experts this workgroup's items need; then, for
// those experts, the bitmap of the rows that selected each (word w covers
// rows 32w .. 32w + 31) and the set bits in the words below each word.
constexpr int kGuWords = kMaxGroupedRows / 32;
constexpr int kGuIdRegs = 16;  // slot ids per thread kept in registers through the set-up
constexpr size_t kGuGroupLds = (size_t)4 * kMaxExperts * 4 + 4 + (size_t)kGuMaxItems * kGuWords * 6;

// Bit position of the r-th set bit of v (r < popcount(v)).
__device__ __forceinline__ int nth_set_bit(uint32_t v, int r) {
    int pos = 0;
#pragma unroll
    for (int b = 16; b > 0; b >>= 1) {
        const int c = __builtin_popcount(v & ((1u << b) - 1u));
        if (r >= c) {
            r -= c;
            v >>= b;
            pos += b;
        }
    }
    return pos;
}

template <int NSB>
__global__ __launch_bounds__(kBlock, 2) void k_gateup_grouped(GroupedGuArgs a, float* hmax, float* hmax_sh) {
    constexpr int H = NSB * kSbCols;
    // weight superblocks in registers (RING - 1 in flight ahead of the
    // MFMAs) and x superblocks loaded ahead of their LDS store; both divide
    // NSB, so a step's ring slot is fixed by its superblock index alone
    constexpr int RING = NSB < 4 ? NSB : 4;
    constexpr int XL = NSB < 2 ? 1 : 2;
    __shared__ __align__(16) _Float16 xb[2][kGChunk * kGXStride];
    static_assert(sizeof(xb) >= kGuGroupLds, "the grouping tables live in the x buffer during the set-up");
    __shared__ int s_tok[kGuMaxItems][kGChunk];
    __shared__ int s_tsig[kGuMaxItems][kGChunk];  // each token's x row exponent (the fp16 copy is x * 2^-sig)
    __shared__ int4 s_item[kGuMaxItems];   // {expert or -1 (shared), first asg position, tokens, slab}
    __shared__ float2 s_ts[kGuMaxItems];   // gate and up tensor scales
    __shared__ float s_max[kWaves][kGChunk];
    __shared__ int s_wsum[kWaves][3];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, q = lane >> 4;
    const uint8_t *const gq_r = a.gate.q, *const gs_r = a.gate.s, *const uq_r = a.up.q, *const us_r = a.up.s;
    const uint8_t *const gq_s = a.sgate.q, *const gs_s = a.sgate.s, *const uq_s = a.sup.q, *const us_s = a.sup.s;
    const int T = a.T, E = a.E, I = a.I, Is = a.Is, kk = a.k, n = T * kk, W = (T + 31) >> 5;
    const int nI = I / kGRows, nIs = max(Is / kGRows, 1);
    const int G = gridDim.x;

    // ---- set-up: the canonical CSR of the T*k slots by expert (experts
    // ascending, an expert's slots in row order) and the tile list of up to
    // kGChunk consecutive slots of one expert, as counts and prefix sums in
    // LDS.  A row never selects an expert twice, so an expert's slots are
    // one per row that picked it.
    int* g_cnt = reinterpret_cast<int*>(&xb[0][0]);  // [E] slots per expert
    int* g_cs = g_cnt + E;                            // [E] first CSR position
    int* g_ts = g_cs + E;                             // [E] first routed tile
    int* g_map = g_ts + E;                            // [E] local index (kGuMaxItems: none)
    uint32_t* g_bm = reinterpret_cast<uint32_t*>(g_map + E);                 // [kGuMaxItems][W]
    uint16_t* g_wp = reinterpret_cast<uint16_t*>(g_bm + kGuMaxItems * W);   // [kGuMaxItems][W]
    int ev[kGuIdRegs];
#pragma unroll
    for (int i = 0; i < kGuIdRegs; ++i) {
        const int s = tid + i * kBlock;
        ev[i] = s < n ? a.ids[s] : 0;
    }
    // f(slot, expert) over this thread's slots tid, tid + kBlock, ...
    auto for_slots = [&](auto&& f) {
#pragma unroll
        for (int i = 0; i < kGuIdRegs; ++i) {
            const int s = tid + i * kBlock;
            if (s < n) f(s, ev[i]);
        }
        for (int s = tid + kGuIdRegs * kBlock; s < n; s += kBlock) f(s, a.ids[s]);
    };
    for (int e = tid; e < E; e += kBlock) {
        g_cnt[e] = 0;
        g_map[e] = kGuMaxItems;
    }
    __syncthreads();
    for_slots([&](int, int e) { atomicAdd(&g_cnt[e], 1); });
    __syncthreads();
    // exclusive prefix sums over experts of the slot count, of the used flag
    // and of the tile count; each thread owns Q consecutive experts
    const int Q = (E + kBlock - 1) / kBlock;
    {
        int c = 0, f = 0, nt = 0;
        for (int u = 0; u < Q; ++u) {
            const int e = tid * Q + u;
            if (e < E) {
                const int ce = g_cnt[e];
                c += ce;
                f += ce > 0;
                nt += (ce + kGChunk - 1) / kGChunk;
            }
        }
        const int ci = wave_incl_scan(c), fi = wave_incl_scan(f), ti = wave_incl_scan(nt);
        if (lane == 63) {
            s_wsum[wave][0] = ci;
            s_wsum[wave][1] = fi;
            s_wsum[wave][2] = ti;
        }
        __syncthreads();
        int cs = ci - c, fs = fi - f, tsn = ti - nt;
        for (int w = 0; w < wave; ++w) {
            cs += s_wsum[w][0];
            fs += s_wsum[w][1];
            tsn += s_wsum[w][2];
        }
        int4* tiles = reinterpret_cast<int4*>(a.tiles);
        const bool pub = blockIdx.x == 0;  // workgroup 0 publishes the per-expert outputs
        for (int u = 0; u < Q; ++u) {
            const int e = tid * Q + u;
            if (e < E) {
                const int ce = g_cnt[e], nte = (ce + kGChunk - 1) / kGChunk;
                g_cs[e] = cs;
                g_ts[e] = tsn;
                if (pub && ce) {
                    a.uniq[fs] = e;
                    a.off[fs] = cs;
                    for (int t = 0; t < nte; ++t)
                        tiles[tsn + t] = make_int4(e, cs + t * kGChunk, min(kGChunk, ce - t * kGChunk), 0);
                }
                cs += ce;
                fs += ce > 0;
                tsn += nte;
            }
        }
    }
    int n_rt = 0, U = 0;
    for (int w = 0; w < kWaves; ++w) {
        U += s_wsum[w][1];
        n_rt += s_wsum[w][2];
    }
    const int n_sh = gq_s ? (T + kGChunk - 1) / kGChunk : 0;
    if (blockIdx.x == 0 && tid == 0) {
        int4* tiles = reinterpret_cast<int4*>(a.tiles);
        *a.n_unique = U;
        a.off[U] = n;
        for (int t = 0; t < n_sh; ++t) tiles[n_rt + t] = make_int4(-1, t * kGChunk, min(kGChunk, T - t * kGChunk), 0);
        *a.n_tiles = n_rt + n_sh;
        if (a.status) *a.status = 0;
    }
    const int items = n_rt * nI + n_sh * nIs;
    // this workgroup's items: blockIdx.x + k * G for k < n_my (<= kGuMaxItems by launch)
    const int n_my = items > (int)blockIdx.x ? min((items - 1 - (int)blockIdx.x) / G + 1, kGuMaxItems) : 0;
    if (n_my == 0) return;

    // every item's descriptor into LDS (tensor scales into registers, stored
    // once the first loads of the stream are out); a routed tile index ti
    // belongs to the last expert whose first tile is at or below ti
    float2 tsv = make_float2(0.f, 0.f);
    if (tid < n_my) {
        const int it = blockIdx.x + tid * G;
        if (it < n_rt * nI) {
            const int ti = it / nI;
            int lo = 0, hi = E - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (g_ts[mid] <= ti) lo = mid;
                else hi = mid - 1;
            }
            const int t = ti - g_ts[lo];
            s_item[tid] = make_int4(lo, g_cs[lo] + t * kGChunk, min(kGChunk, g_cnt[lo] - t * kGChunk), it % nI);
            atomicMin(&g_map[lo], tid);
            tsv = make_float2(a.gate.ts[lo], a.up.ts[lo]);
        } else {
            const int r = it - n_rt * nI, t = r / nIs;
            s_item[tid] = make_int4(-1, t * kGChunk, min(kGChunk, T - t * kGChunk), r % nIs);
            tsv = make_float2(a.sgate.ts[0], a.sup.ts[0]);
        }
    }
    for (int i = tid; i < kGuMaxItems * W; i += kBlock) g_bm[i] = 0u;
    __syncthreads();
    // The workgroup's items form one stream of n_my * NSB superblock steps;
    // weights and x are loaded ahead along that stream, across item
    // boundaries (past the last item: the last item again, L2 hits).
    auto load_w = [&](int k, int sb) {
        const int4 d = s_item[min(k, n_my - 1)];
        const bool routed = d.x >= 0;
        const int rows = routed ? I : Is;
        const size_t eq = (size_t)(routed ? d.x : 0) * rows * (H / 2), es = (size_t)(routed ? d.x : 0) * rows * (H / 16);
        const int n0 = d.w * kGRows + wave * 16;
        return gu_load_sb((routed ? gq_r : gq_s) + eq, (routed ? gs_r : gs_s) + es, (routed ? uq_r : uq_s) + eq,
                          (routed ? us_r : us_s) + es, H, n0, sb, true);
    };
    // the stream's first weights go out now, ahead of the rest of the set-up
    GuSb w[RING];
#pragma unroll
    for (int p = 0; p < RING - 1; ++p) w[p] = load_w(p / NSB, p % NSB);
    // row bitmaps of the experts this workgroup needs; row s / k as the
    // high word of s * ceil(2^32 / k), exact for s < 2^32 / k (k = 1: s)
    const uint32_t kmag = kk > 1 ? 0xFFFFFFFFu / (uint32_t)kk + 1u : 0u;
    for_slots([&](int s, int e) {
        const int li = g_map[e];
        if (li < kGuMaxItems) {
            const int r = kk > 1 ? (int)__umulhi((uint32_t)s, kmag) : s;
            atomicOr(&g_bm[li * W + (r >> 5)], 1u << (r & 31));
        }
    });
    __syncthreads();
    // set bits below each word: lanes 0-31 scan local expert li's words,
    // lanes 32-63 those of li + 1
    for (int li = 2 * wave; li < n_my; li += 2 * kWaves) {
        const int l2 = li + (lane >> 5), w = lane & 31;
        const bool live = l2 < n_my && w < W;
        const int pc = live ? __builtin_popcount(g_bm[l2 * W + w]) : 0;
        int v = wave_incl_scan(pc);
        const int low_total = __builtin_amdgcn_readlane(v, 31);
        if (lane >= 32) v -= low_total;
        if (live) g_wp[l2 * W + w] = (uint16_t)(v - pc);
    }
    __syncthreads();
    // token rows of every item (tokens past a tile repeat its last one);
    // a routed tile's m-th token is its expert's (first slot - CSR start +
    // m)-th row in ascending order: the word whose count below is the last
    // one not above that rank, then the bit inside it
    constexpr int kTokPer = kGuMaxItems * kGChunk / kBlock;
    int tsg[kTokPer];
#pragma unroll
    for (int u = 0; u < kTokPer; ++u) {
        const int t = tid + u * kBlock;
        tsg[u] = 0;
        if (t < n_my * kGChunk) {
            const int k = t >> 5, m = t & 31;
            const int4 d = s_item[k];
            int tok;
            if (d.x >= 0) {
                const int li = g_map[d.x];
                const int idx = d.y - g_cs[d.x] + min(m, d.z - 1);
                const uint32_t* bm = g_bm + li * W;
                const uint16_t* wp = g_wp + li * W;
                int lo = 0, hi = W - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if ((int)wp[mid] <= idx) lo = mid;
                    else hi = mid - 1;
                }
                tok = 32 * lo + nth_set_bit(bm[lo], idx - (int)wp[lo]);
            } else {
                tok = d.y + min(m, d.z - 1);
            }
            s_tok[k][m] = tok;
            tsg[u] = a.x_sig[tok];
        }
    }
    __syncthreads();

    // fp16 x columns of superblock sb of item k: 32 tokens x 32 pieces of 16
    // bytes, four pieces per thread, at the tokens' rows; zeros, not loaded,
    // for tokens past the item's tile
    auto load_x = [&](int k, int sb, uint4 (&v)[4]) {
        const int kc = min(k, n_my - 1);
        const int cnt = s_item[kc].z;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int f = t * kBlock + tid, m = f >> 5, c8 = f & 31;
            v[t] = m < cnt ? *reinterpret_cast<const uint4*>(a.x + (size_t)s_tok[kc][m] * H + sb * kSbCols + c8 * 8)
                           : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_x = [&](int buf, const uint4 (&v)[4]) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int f = t * kBlock + tid, m = f >> 5, c8 = f & 31;
            *reinterpret_cast<uint4*>(&xb[buf][m * kGXStride + c8 * 8]) = v[t];
        }
    };

    uint4 xv[XL][4];
#pragma unroll
    for (int p = 0; p < XL; ++p) load_x(p / NSB, p % NSB, xv[p]);
    // the set-up's row exponents and tensor scales
#pragma unroll
    for (int u = 0; u < kTokPer; ++u) {
        const int t = tid + u * kBlock;
        if (t < n_my * kGChunk) s_tsig[t >> 5][t & 31] = tsg[u];
    }
    if (tid < n_my) s_ts[tid] = tsv;
    store_x(0, xv[0]);
    __syncthreads();

    for (int k = 0; k < n_my; ++k) {
        const int4 d = s_item[k];
        const bool routed = d.x >= 0;
        const int p0 = d.y, cnt = d.z, slab = d.w;
        const int ntt = cnt > 16 ? 2 : 1;
        f32x4_t accg[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4_t accu[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            load_x(k + (sb + XL) / NSB, (sb + XL) % NSB, xv[(sb + XL) % XL]);
            if (RING > 1) w[(sb + RING - 1) % RING] = load_w(k + (sb + RING - 1) / NSB, (sb + RING - 1) % NSB);
            else w[0] = load_w(k, sb);
            gg_mfma_sb(w[sb % RING], xb[(k * NSB + sb) & 1], accg, accu);
            store_x((k * NSB + sb + 1) & 1, xv[(sb + 1) % XL]);
            __syncthreads();
        }

        // SwiGLU epilogue: lane (j, q) holds rows n0 + 4q .. +3 of token j
        const float gts = s_ts[k].x, uts = s_ts[k].y;
        const int n0 = slab * kGRows + wave * 16;
        float* hbase = routed ? a.h : a.h_sh;
        const int hstride = routed ? I : Is;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int m = tt * 16 + j;
            float4 hv = make_float4(0.f, 0.f, 0.f, 0.f);
            if (tt < ntt) {
                // undo the token's power-of-two x scale, then the tensor scales
                const int sg = s_tsig[k][m];
                float gv, uv;
                gv = ldexpf(accg[tt][0], sg) * gts; uv = ldexpf(accu[tt][0], sg) * uts; hv.x = gv / (1.0f + expf(-gv)) * uv;
                gv = ldexpf(accg[tt][1], sg) * gts; uv = ldexpf(accu[tt][1], sg) * uts; hv.y = gv / (1.0f + expf(-gv)) * uv;
                gv = ldexpf(accg[tt][2], sg) * gts; uv = ldexpf(accu[tt][2], sg) * uts; hv.z = gv / (1.0f + expf(-gv)) * uv;
                gv = ldexpf(accg[tt][3], sg) * gts; uv = ldexpf(accu[tt][3], sg) * uts; hv.w = gv / (1.0f + expf(-gv)) * uv;
                if (m < cnt) *reinterpret_cast<float4*>(hbase + (size_t)(p0 + m) * hstride + n0 + 4 * q) = hv;
            }
            // max |h| of token m over this wave's 16 rows (lanes j, j+16, j+32, j+48)
            float mx = fmaxf(fmaxf(fabsf(hv.x), fabsf(hv.y)), fmaxf(fabsf(hv.z), fabsf(hv.w)));
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            if (q == 0) s_max[wave][m] = mx;
        }
        __syncthreads();
        if (tid < cnt) {
            const float mx = fmaxf(fmaxf(s_max[0][tid], s_max[1][tid]), fmaxf(s_max[2][tid], s_max[3][tid]));
            if (routed) hmax[(size_t)(p0 + tid) * nI + slab] = mx;
            else hmax_sh[(size_t)(p0 + tid) * nIs + slab] = mx;
        }
    }
    // the CSR entries of the routed tiles whose first slab this workgroup
    // did: position p0 + m holds slot r*k + j, where row r = the m-th token
    // and j its selection rank of the tile's expert
    for (int t = tid; t < n_my * kGChunk; t += kBlock) {
        const int k = t >> 5, m = t & 31;
        const int4 d = s_item[k];
        if (d.x >= 0 && d.w == 0 && m < d.z) {
            const int r = s_tok[k][m];
            int jr = 0;
            for (int jj = 0; jj < kk; ++jj)
                if (a.ids[(size_t)r * kk + jj] == d.x) jr = jj;
            const int s = r * kk + jr;
            a.asg[d.y + m] = s;
            a.inv[s] = d.y + m;
        }
    }
}

// ---------------------------------------------------------------------------
// grouped down
//
// Work unit: (tile, 64-row slab of the output dimension), numbered tile by
// tile.  The workgroups are persistent, one launch-wide round of them, and
// each takes an equal contiguous run of units, so no workgroup waits on a
// partial last round; a run is one or two segments of consecutive slabs of
// one tile.  A segment stages the tile's h rows in LDS once, as
// hi = fp16(h * 2^-sigma) and lo = fp16(h * 2^-sigma - hi), sigma per token
// such that its max |h| maps into [2^14, 2^15); staged rows span NSB whole
// superblocks, zero past the row's length, stride NSB*256 + 8 halfs.  Then
// it walks its slabs: wave w computes output rows slab*64 + 16w .. +15 for
// the tile's tokens; lane (i, kb) holds the codes of row n0 + i at columns
// [sb*256 + kb*64, +64) of every superblock, and the next slab's codes are
// in flight while the current slab is on the matrix cores.
// ---------------------------------------------------------------------------

constexpr int kGMaxSb = kGMaxCols / kSbCols;  // superblocks of the longest staged h row


// a compile-time integer passed as a value (a tile's column-tile count)
template <int N>
struct IntC {
    static constexpr int value = N;
};

template <int NSB>
struct DownCodes {
    uint4 c0[NSB], c1[NSB];
    uint32_t sc[NSB];
};

template <int NSB>
__global__ __launch_bounds__(kBlock) void k_down_grouped(GroupedDownArgs a, const float* hmax, const float* hmax_sh) {
    extern __shared__ __align__(16) _Float16 hb[];  // hi [32][S], then lo [32][S]
    __shared__ int s_sig[kGChunk];
    constexpr int S = NSB * kSbCols + 8;  // staged row stride in halfs
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i = lane & 15, kb = lane >> 4, j = lane & 15, q = lane >> 4;
    const uint8_t *const dq_r = a.down.q, *const ds_r = a.down.s, *const dq_s = a.sdown.q, *const ds_s = a.sdown.s;
    const float *const dts_r = a.down.ts, *const dts_s = a.sdown.ts;
    const int H = a.H, I = a.I, Is = a.Is, T = a.T, kk = a.k;
    _Float16* hi = hb;
    _Float16* lo = hb + kGChunk * S;
    const int nS = H / kGRows;  // output slabs per tile
    const int n_tiles = *a.n_tiles;
    const int n_sh = dq_s ? (T + kGChunk - 1) / kGChunk : 0;
    const int n_rt = n_tiles - n_sh;
    const int units = n_tiles * nS;
    const int u_end = (int)((long long)units * (blockIdx.x + 1) / gridDim.x);
    for (int u = (int)((long long)units * blockIdx.x / gridDim.x); u < u_end;) {
        const int ti = u / nS, s_lo = u - ti * nS;
        const int n_seg = min(nS - s_lo, u_end - u);  // slabs s_lo .. s_lo + n_seg - 1 of tile ti
        u += n_seg;
        const bool routed = ti < n_rt;
        const int4 tl = reinterpret_cast<const int4*>(a.tiles)[ti];
        const int e = routed ? tl.x : 0, p0 = tl.y, cnt = tl.z;
        const int cols = routed ? I : Is;
        const int nslab = cols / kGRows;
        const uint8_t* mq = (routed ? dq_r : dq_s) + (size_t)e * H * (cols / 2);
        const uint8_t* ms = (routed ? ds_r : ds_s) + (size_t)e * H * (cols / 16);
        const float ts = (routed ? dts_r : dts_s)[e];

        // codes of slab s_lo + g (loads at clamped columns past the row's
        // length: their products meet the zero columns of the staged h)
        auto load_codes = [&](int g, DownCodes<NSB>& c) {
            const size_t row = (size_t)((s_lo + g) * kGRows + wave * 16 + i);
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const int col = min(sb * kSbCols + kb * 64, cols - 64);
                const uint8_t* p = mq + row * (cols / 2) + col / 2;
                c.c0[sb] = *reinterpret_cast<const uint4*>(p);
                c.c1[sb] = *reinterpret_cast<const uint4*>(p + 16);
                c.sc[sb] = *reinterpret_cast<const uint32_t*>(ms + row * (cols / 16) + col / 16);
            }
        };
        // The segment's loads in the order they are consumed (vector loads
        // complete in issue order): max |h| entries, the tile's h rows, then
        // the codes of the first slab.  Entry (token m, slab sl) of max |h|
        // goes to thread 16m + sl of each half of the workgroup (clamped).
        const float* hmb = routed ? hmax : hmax_sh;
        float hmv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int idx = u * kBlock + tid, m = idx >> 4, sl = idx & 15;
            hmv[u] = hmb[(size_t)(p0 + min(m, cnt - 1)) * nslab + min(sl, nslab - 1)];
        }
        // output rows of this lane's tokens j and 16 + j: a routed token's
        // slot (so the combine reads its rows without the CSR), a shared
        // token's row after the routed ones
        int orow[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int pm = p0 + min(tt * 16 + j, cnt - 1);
            orow[tt] = routed ? a.asg[pm] : T * kk + pm;
        }
        const float* hrow0 = routed ? a.h + (size_t)p0 * I : a.h_sh + (size_t)p0 * Is;
        float4 v[NSB][8];  // one superblock is 32 rows x 256 columns = 2048 float4
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int f = t * kBlock + tid, m = f >> 6, c4 = f & 63;
                const int col = min(sb * kSbCols + c4 * 4, cols - 4);
                // rows past the tile's tokens are zero when staged: not loaded
                v[sb][t] = m < cnt ? *reinterpret_cast<const float4*>(hrow0 + (size_t)m * cols + col)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        DownCodes<NSB> cA, cB;
        load_codes(0, cA);

        // per-token scale exponent: max over the token's slabs (16 lanes)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int idx = u * kBlock + tid, m = idx >> 4, sl = idx & 15;
            float mx = (m < cnt && sl < nslab) ? hmv[u] : 0.0f;
            mx = fmaxf(mx, __shfl_xor(mx, 8, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 4, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 2, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 1, 16));
            if (sl == 0) s_sig[m] = (mx > 0.0f) ? ilogbf(mx) - 14 : 0;
        }
        __syncthreads();
        // stage h as the fp16 pair, zero past the row's length and the tokens
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int f = t * kBlock + tid, m = f >> 6, c4 = f & 63;
                const int col = sb * kSbCols + c4 * 4;
                const int sg = -s_sig[m];
                const bool live = m < cnt && col < cols;
                const float x0 = live ? ldexpf(v[sb][t].x, sg) : 0.f, x1 = live ? ldexpf(v[sb][t].y, sg) : 0.f;
                const float x2 = live ? ldexpf(v[sb][t].z, sg) : 0.f, x3 = live ? ldexpf(v[sb][t].w, sg) : 0.f;
                const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1, h2 = (_Float16)x2, h3 = (_Float16)x3;
                f16x2_t a01 = {h0, h1}, a23 = {h2, h3};
                f16x2_t b01 = {(_Float16)(x0 - (float)h0), (_Float16)(x1 - (float)h1)};
                f16x2_t b23 = {(_Float16)(x2 - (float)h2), (_Float16)(x3 - (float)h3)};
                uint2 ph, pl;
                ph.x = __builtin_bit_cast(uint32_t, a01); ph.y = __builtin_bit_cast(uint32_t, a23);
                pl.x = __builtin_bit_cast(uint32_t, b01); pl.y = __builtin_bit_cast(uint32_t, b23);
                *reinterpret_cast<uint2*>(hi + m * S + col) = ph;
                *reinterpret_cast<uint2*>(lo + m * S + col) = pl;
            }
        }
        __syncthreads();

        const int ntt = cnt > 16 ? 2 : 1;
        // NT: the tile's 16-token column tiles (1 or 2), a compile-time
        // constant so that the MFMA steps hold no branch
        auto compute = [&](auto ntc, int g, const DownCodes<NSB>& c) {
            constexpr int NT = decltype(ntc)::value;
            f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            // Every superblock of the staged row, also past a shorter row's
            // length (zero h there): no data-dependent branch in the chain.
            // Software pipelined over the NSB * 8 MFMA steps: step q + 1's h
            // columns are read from LDS before step q's MFMAs issue; a
            // scheduling barrier closes each step, so at most two steps'
            // operands are in registers.
            const _Float16* hr = hi + j * S + kb * 64;
            const _Float16* lr = lo + j * S + kb * 64;
            auto ldb = [&](const _Float16* base, int q, int tt) {
                return *reinterpret_cast<const f16x8_t*>(base + tt * 16 * S + (q >> 3) * kSbCols + 8 * (q & 7));
            };
            f16x8_t bh[NT], bl[NT];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) { bh[tt] = ldb(hr, 0, tt); bl[tt] = ldb(lr, 0, tt); }
#pragma unroll
            for (int q = 0; q < NSB * 8; ++q) {
                const int sb = q >> 3, s = q & 7;
                f16x8_t nh[NT], nl[NT];
                if (q + 1 < NSB * 8) {
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) { nh[tt] = ldb(hr, q + 1, tt); nl[tt] = ldb(lr, q + 1, tt); }
                }
                const uint32_t scw = c.sc[sb];
                const _Float16 ssc = (s < 2)   ? e4m3_to_f16<0>(scw)
                                     : (s < 4) ? e4m3_to_f16<1>(scw)
                                     : (s < 6) ? e4m3_to_f16<2>(scw)
                                               : e4m3_to_f16<3>(scw);
                const f16x8_t aw = decode8_f16(pick_word(c.c0[sb], c.c1[sb], s), ssc);
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, bh[tt], acc[tt], 0, 0, 0);
                    acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, bl[tt], acc[tt], 0, 0, 0);
                }
                if (q + 1 < NSB * 8) {
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) { bh[tt] = nh[tt]; bl[tt] = nl[tt]; }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // lane (j, q) holds output rows n0 + 4q .. +3 of token j
            const int n0 = (s_lo + g) * kGRows + wave * 16;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int m = tt * 16 + j;
                if (m < cnt) {
                    const int sg = s_sig[m];
                    float4 ov;
                    ov.x = ldexpf(acc[tt][0], sg) * ts;
                    ov.y = ldexpf(acc[tt][1], sg) * ts;
                    ov.z = ldexpf(acc[tt][2], sg) * ts;
                    ov.w = ldexpf(acc[tt][3], sg) * ts;
                    *reinterpret_cast<float4*>(a.o + (size_t)orow[tt] * H + n0 + 4 * q) = ov;
                }
            }
        };
        // slabs in pairs: the other register set's loads are always issued
        // (the last slab's codes again at the end, an L2 hit) so the compiler
        // keeps an exact count of loads in flight
        auto run = [&](auto ntc) {
#pragma unroll 1
            for (int g = 0; g < n_seg; g += 2) {
                load_codes(g + 1 < n_seg ? g + 1 : n_seg - 1, cB);
                compute(ntc, g, cA);
                load_codes(g + 2 < n_seg ? g + 2 : n_seg - 1, cA);
                if (g + 1 < n_seg) compute(ntc, g + 1, cB);
            }
        };
        if (ntt > 1) run(IntC<2>{});
        else run(IntC<1>{});
        __syncthreads();  // staged rows and s_sig are replaced by the next segment
    }
}

// ---------------------------------------------------------------------------
// k_combine: one workgroup per row
// ---------------------------------------------------------------------------

constexpr int kCombineV4 = 2048 / 4 / kBlock;  // float4 per thread at the largest hidden size
constexpr int kCombineBatch = 8;                // slots whose rows are loaded together

__global__ __launch_bounds__(kBlock) void k_combine(CombineArgs a) {
    __shared__ float s_w[kMaxTopK];
    __shared__ float s_ss[kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = blockIdx.x, H = a.H, k = a.k;
    const int n4 = H / 4;  // float4 per row; thread tid owns float4 t * kBlock + tid
    if (tid < k) s_w[tid] = a.w[(size_t)r * k + tid];
    // the shared expert's row is requested with the first batch of slots
    float4 sh[kCombineV4];
#pragma unroll
    for (int t = 0; t < kCombineV4; ++t) {
        const int i4 = min(t * kBlock + tid, n4 - 1);
        sh[t] = a.has_shared ? reinterpret_cast<const float4*>(a.o + ((size_t)a.T * k + r) * H)[i4]
                             : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // y = rs * sum_j w_j o_j (j in rank order) + shared (+ residual), per element;
    // slot (r, j)'s row is o row r*k + j, so the first batch's loads leave
    // with the weights
    float4 acc[kCombineV4];
#pragma unroll
    for (int t = 0; t < kCombineV4; ++t) acc[t] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
        float4 ov[kCombineBatch][kCombineV4];
#pragma unroll
        for (int b = 0; b < kCombineBatch; ++b) {
            const float4* orow = reinterpret_cast<const float4*>(a.o + ((size_t)r * k + min(j0 + b, k - 1)) * H);
#pragma unroll
            for (int t = 0; t < kCombineV4; ++t) ov[b][t] = orow[min(t * kBlock + tid, n4 - 1)];
        }
        if (j0 == 0) __syncthreads();  // s_w visible (every thread takes the same batches)
#pragma unroll
        for (int b = 0; b < kCombineBatch; ++b) {
            if (j0 + b < k) {
                const float wv = s_w[j0 + b];
#pragma unroll
                for (int t = 0; t < kCombineV4; ++t) {
                    acc[t].x = fmaf(wv, ov[b][t].x, acc[t].x);
                    acc[t].y = fmaf(wv, ov[b][t].y, acc[t].y);
                    acc[t].z = fmaf(wv, ov[b][t].z, acc[t].z);
                    acc[t].w = fmaf(wv, ov[b][t].w, acc[t].w);
                }
            }
        }
    }
    float4 yv[kCombineV4];
    float ss = 0.0f;
#pragma unroll
    for (int t = 0; t < kCombineV4; ++t) {
        yv[t] = make_float4(0.f, 0.f, 0.f, 0.f);
        const int i4 = t * kBlock + tid;
        if (i4 < n4) {
            const size_t c = (size_t)r * H + 4 * i4;
            float4 y;
            y.x = a.rs * acc[t].x; y.y = a.rs * acc[t].y; y.z = a.rs * acc[t].z; y.w = a.rs * acc[t].w;
            if (a.has_shared) { y.x += sh[t].x; y.y += sh[t].y; y.z += sh[t].z; y.w += sh[t].w; }
            if (a.residual) {
                const uint2 rb = *reinterpret_cast<const uint2*>(a.residual + c);
                y.x += __uint_as_float(rb.x << 16); y.y += __uint_as_float(rb.x & 0xFFFF0000u);
                y.z += __uint_as_float(rb.y << 16); y.w += __uint_as_float(rb.y & 0xFFFF0000u);
            }
            *reinterpret_cast<float4*>(a.y32 + c) = y;
            if (a.y) {
                uint2 o;
                o.x = (uint32_t)f32_to_bf16_rne(y.x) | ((uint32_t)f32_to_bf16_rne(y.y) << 16);
                o.y = (uint32_t)f32_to_bf16_rne(y.z) | ((uint32_t)f32_to_bf16_rne(y.w) << 16);
                *reinterpret_cast<uint2*>(a.y + c) = o;
            }
            yv[t] = y;
            ss = fmaf(y.x, y.x, ss); ss = fmaf(y.y, y.y, ss); ss = fmaf(y.z, y.z, ss); ss = fmaf(y.w, y.w, ss);
        }
    }
    if (!a.x_next) return;
    // the next layer's input: bf16(y / sqrt(mean(y^2) + eps)), sums in a fixed order
    ss = wave_sum(ss);
    if (lane == 0) s_ss[wave] = ss;
    __syncthreads();
    const float tot = (s_ss[0] + s_ss[1]) + (s_ss[2] + s_ss[3]);
    const float sc = 1.0f / sqrtf(tot / (float)H + a.eps);
#pragma unroll
    for (int t = 0; t < kCombineV4; ++t) {
        const int i4 = t * kBlock + tid;
        if (i4 < n4) {
            // x_next = bf16((y * inv_rms) * gamma), fp32 products
            const uint2 g = *reinterpret_cast<const uint2*>((a.gamma ? a.gamma : kBf16Ones) + 4 * i4);
            uint2 o;
            o.x = (uint32_t)f32_to_bf16_rne(yv[t].x * sc * bf16_to_f32(g.x & 0xFFFFu)) |
                  ((uint32_t)f32_to_bf16_rne(yv[t].y * sc * bf16_to_f32(g.x >> 16)) << 16);
            o.y = (uint32_t)f32_to_bf16_rne(yv[t].z * sc * bf16_to_f32(g.y & 0xFFFFu)) |
                  ((uint32_t)f32_to_bf16_rne(yv[t].w * sc * bf16_to_f32(g.y >> 16)) << 16);
            *reinterpret_cast<uint2*>(a.x_next + (size_t)r * H + 4 * i4) = o;
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

namespace {

template <typename Kern, typename Args>
hipError_t launch_plain(Kern k, dim3 grid, dim3 block, size_t smem, hipStream_t st, const Args& a) {
    hipLaunchKernelGGL(k, grid, block, smem, st, a);
    return hipGetLastError();
}

size_t group_lds(int T, int E) { return (size_t)E * ((T + 31) / 32) * (group_pc_fits(T, E) ? 6 : 4); }
// superblocks of the longest staged h row, and the grouped down kernel's
// output slabs per work item
int down_nsb(int I, int Is) { return ((I > Is ? I : Is) + kSbCols - 1) / kSbCols; }
size_t down_lds(int I, int Is) {
    const int nsb = down_nsb(I, Is);
    return (size_t)2 * kGChunk * ((nsb == 3 ? 4 : nsb) * kSbCols + 8) * 2;
}

// largest dynamic LDS each kernel is launched with (static LDS comes on top)
constexpr int kGDownMaxLds = 2 * kGChunk * (kGMaxSb * kSbCols + 8) * 2;

}  // namespace

int grouped_max_tiles(int T, int E, int k, bool has_shared) {
    const int n = T * k;
    return (n < E ? n : E) + (n + kGChunk - 1) / kGChunk + (has_shared ? (T + kGChunk - 1) / kGChunk : 0);
}

bool grouped_lds_fits(int T, int E, int I, int Is) {
    return group_lds(T, E) <= (size_t)kGroupMaxLds && down_lds(I, Is) <= (size_t)kGDownMaxLds &&
           (size_t)kWaves * E * 4 <= (size_t)kMaxDynLds;
}

// persistent down workgroups per staged-row width (1, 2, 4 superblocks):
// one round of resident workgroups, from the occupancy query at set-up
static int g_down_grid[3] = {512, 512, 256};

hipError_t init_grouped_kernels() {
    hipError_t e;
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_group),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, kGroupMaxLds)) != hipSuccess)
        return e;
    const void* downs[] = {reinterpret_cast<const void*>(k_down_grouped<1>),
                           reinterpret_cast<const void*>(k_down_grouped<2>),
                           reinterpret_cast<const void*>(k_down_grouped<4>)};
    for (const void* f : downs)
        if ((e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kGDownMaxLds)) != hipSuccess)
            return e;
    int dev = 0, ncu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    for (int v = 0; v < 3; ++v) {
        int nb = 0;
        const size_t lds = (size_t)2 * kGChunk * ((1 << v) * kSbCols + 8) * 2;
        if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, downs[v], kBlock, lds)) != hipSuccess) return e;
        g_down_grid[v] = (nb > 0 ? nb : 1) * (ncu > 0 ? ncu : 1);
    }
    return hipSuccess;
}

hipError_t launch_router_mfma(const RouterArgs& a, hipStream_t st) {
    const dim3 g((a.K + 31) / 32, (a.E + 15) / 16), b(kRouterWaves * 64);
    switch (a.H) {
        case 256: return launch_plain(k_router_mfma<256>, g, b, 0, st, a);
        case 512: return launch_plain(k_router_mfma<512>, g, b, 0, st, a);
        case 1024: return launch_plain(k_router_mfma<1024>, g, b, 0, st, a);
        case 2048: return launch_plain(k_router_mfma<2048>, g, b, 0, st, a);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_router_split(const RouterArgs& a, hipStream_t st) {
    if (a.K > kRouterSplitMaxRows) return hipErrorInvalidValue;
    const dim3 g((a.E + 15) / 16, kRouterWaves), b(64);
    switch (a.H) {
        case 256: return launch_plain(k_router_split<256>, g, b, 0, st, a);
        case 512: return launch_plain(k_router_split<512>, g, b, 0, st, a);
        case 1024: return launch_plain(k_router_split<1024>, g, b, 0, st, a);
        case 2048: return launch_plain(k_router_split<2048>, g, b, 0, st, a);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_select_rows_split(const SelectSplitArgs& a, hipStream_t st) {
    if (a.H > 2048 || a.H % 8 || a.s.E > kRouterSplitMaxExperts) return hipErrorInvalidValue;
    const int grid = (a.s.K + kWaves - 1) / kWaves;
    return launch_plain(k_select_rows_split, dim3(grid), dim3(kBlock), (size_t)kWaves * a.s.E * 4, st, a);
}

hipError_t launch_select_rows(const SelectArgs& a, hipStream_t st) {
    const int grid = (a.K + kWaves - 1) / kWaves;
    return launch_plain(k_select_rows, dim3(grid), dim3(kBlock), (size_t)kWaves * a.E * 4, st, a);
}

hipError_t launch_group(const GroupArgs& a, hipStream_t st) {
    return launch_plain(k_group, dim3(1), dim3(kGGroupThreads), group_lds(a.T, a.E), st, a);
}

hipError_t launch_gateup_grouped(const GroupedGuArgs& a, float* hmax, float* hmax_sh, int max_tiles,
                                 hipStream_t st) {
    const int per = (a.I > a.Is ? a.I : a.Is) / kGRows;
    const long long items = (long long)max_tiles * per;
    // persistent workgroups, each walking at most kGuMaxItems items
    long long grid = items < kGuGrid ? items : kGuGrid;
    const long long need = (items + kGuMaxItems - 1) / kGuMaxItems;
    if (grid < need) grid = need;
    const dim3 g((unsigned)grid), b(kBlock);
    switch (a.H) {
        case 256: hipLaunchKernelGGL(k_gateup_grouped<1>, g, b, 0, st, a, hmax, hmax_sh); break;
        case 512: hipLaunchKernelGGL(k_gateup_grouped<2>, g, b, 0, st, a, hmax, hmax_sh); break;
        case 1024: hipLaunchKernelGGL(k_gateup_grouped<4>, g, b, 0, st, a, hmax, hmax_sh); break;
        case 2048: hipLaunchKernelGGL(k_gateup_grouped<8>, g, b, 0, st, a, hmax, hmax_sh); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_down_grouped(const GroupedDownArgs& a, const float* hmax, const float* hmax_sh, int max_tiles,
                               hipStream_t st) {
    const int nsb = down_nsb(a.I, a.Is);
    // one round of persistent workgroups (two per compute unit fit the
    // staged h and the registers), never more than there are units
    const long long units = (long long)max_tiles * (a.H / kGRows);
    const int resident = g_down_grid[nsb == 1 ? 0 : nsb == 2 ? 1 : 2];
    const int grid = (int)(units < resident ? units : resident);
    const dim3 g(grid), b(kBlock);
    const size_t lds = down_lds(a.I, a.Is);
    if (nsb == 1) hipLaunchKernelGGL((k_down_grouped<1>), g, b, lds, st, a, hmax, hmax_sh);
    else if (nsb == 2) hipLaunchKernelGGL((k_down_grouped<2>), g, b, lds, st, a, hmax, hmax_sh);
    else hipLaunchKernelGGL((k_down_grouped<4>), g, b, lds, st, a, hmax, hmax_sh);
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
    return launch_plain(k_combine, dim3(a.T), dim3(kBlock), 0, st, a);
}

}  // namespace moe
