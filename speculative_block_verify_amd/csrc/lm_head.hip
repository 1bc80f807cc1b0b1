// gfx950 kernels of the verify step's head: the lm_head GEMV over every
// verify row and greedy block acceptance (PR #844 section 5, trap 1: the
// verifier takes the argmax of every row, one greedy token per verify row;
// mlxfast README: a step keeps the longest accepted prefix, and a token is
// accepted on an exact match or on a tie of the top logit within 1e-6).
//
//   k_lm_head        logits = x W^T for up to 16 rows on the matrix cores
//                    (v_mfma_f32_16x16x32_bf16; bf16 products are exact in
//                    fp32, sums in fp32).  A wave owns 16-row tiles of W and
//                    streams them: lane (i, kb) reads 128 contiguous bytes
//                    of row v0 + i per 256-column superblock, up to four
//                    superblocks in flight across tile boundaries.  Each
//                    wave keeps a running argmax per verify row; the
//                    workgroup leaves one (logit, token) per row.
//   k_greedy_finalize  one workgroup: the argmax over the workgroups'
//                    partial results, then the acceptance walk.

#include "moe_device.h"

namespace moe {

typedef __bf16 lm_bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kLmMaxRows = 16;   // verify rows one MFMA B operand holds

// (logit, token) as one orderable 64-bit key: the larger logit wins, and
// among equal logits the lower token id.
__device__ __forceinline__ unsigned long long lm_key(float logit, int tok) {
    return ((unsigned long long)key_bits(logit) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)tok);
}
__device__ __forceinline__ float lm_key_logit(unsigned long long k) {
    const uint32_t u = (uint32_t)(k >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}
__device__ __forceinline__ int lm_key_token(unsigned long long k) {
    return (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFu));
}

struct LmArgs {
    const uint16_t* x;        // bf16 [K][H]
    const uint16_t* w;        // bf16 [V][H]
    const int32_t* draft;     // [K-1] draft tokens (row r's input token is draft[r-1]), or nullptr when K == 1
    float* logits;            // fp32 [K][V] or nullptr
    unsigned long long* part; // [gridDim.x][K] per-workgroup best key of each row
    float* draft_logit;       // [K] logit of draft[j] in row j (j < K-1)
    int K, V, H;
};

// The 8 weight pieces (16 bytes each) of lane (i, kb) in superblock sb of
// the tile at row v0: row min(v0 + i, V - 1), columns sb*256 + kb*64 .. +63.
// Always issued (a clamped row past the end): the compiler then keeps an
// exact count of the loads in flight.
template <int NSB>
__device__ __forceinline__ void lm_load(const LmArgs& a, int v0, int sb, uint4 (&r)[8]) {
    const int lane = threadIdx.x & 63, i = lane & 15, kb = lane >> 4;
    constexpr int H = NSB * kSbCols;
    const int row = min(v0 + i, a.V - 1);
    const uint4* p = reinterpret_cast<const uint4*>(a.w + (size_t)row * H + sb * kSbCols + kb * 64);
#pragma unroll
    for (int s = 0; s < 8; ++s) r[s] = ld16_nt(p + s);
}

template <int NSB>
__global__ __launch_bounds__(kBlock) void k_lm_head(LmArgs a) {
    constexpr int H = NSB * kSbCols;
    // superblocks in flight: a divisor of NSB, so each step's ring slot is
    // fixed by its superblock index
    constexpr int RING = NSB < 4 ? NSB : 4;
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);   // [K][padded H] bf16
    __shared__ int s_draft[kLmMaxRows];
    __shared__ unsigned long long s_best[kWaves][kLmMaxRows];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, q = lane >> 4, kb = q;
    const int K = a.K, V = a.V;
    const int n_tiles = (V + 15) / 16;
    const int gw = blockIdx.x * kWaves + wave, GW = gridDim.x * kWaves;
    const int n_my = gw < n_tiles ? (n_tiles - 1 - gw) / GW + 1 : 0;
    // row of this wave's tile k (k clamped to its last tile; a wave without
    // tiles reads tile 0's rows and computes nothing)
    auto tile_row = [&](int k) { return n_my > 0 ? (gw + min(k, n_my - 1) * GW) * 16 : 0; };

    // the first superblocks of this wave's stream, before x is staged
    uint4 ring[RING][8];
#pragma unroll
    for (int p = 0; p < RING; ++p) lm_load<NSB>(a, tile_row(p / NSB), p % NSB, ring[p]);

    // the K x rows in LDS (padded layout); the draft tokens
    for (int f = tid; f < K * (H / 8); f += kBlock) {
        const int m = f / (H / 8), c = (f % (H / 8)) * 8;
        *reinterpret_cast<uint4*>(xs + xh_index(m, c, H)) = *reinterpret_cast<const uint4*>(a.x + (size_t)m * H + c);
    }
    if (tid < kLmMaxRows) s_draft[tid] = (a.draft && tid < K - 1) ? a.draft[tid] : -1;
    __syncthreads();
    const int my_draft = s_draft[j];
    const bool live = j < K;
    const lm_bf16x8_t zero8 = {};
    const bool vec_out = (V & 3) == 0;

    unsigned long long best = 0ull;  // running best key of verify row j over this wave's tiles
    for (int k = 0; k < n_my; ++k) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            const uint16_t* xr = xs + xh_index(live ? j : 0, sb * kSbCols + kb * 64, H);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const lm_bf16x8_t av = __builtin_bit_cast(lm_bf16x8_t, ring[sb % RING][t]);
                const lm_bf16x8_t bv = live ? *reinterpret_cast<const lm_bf16x8_t*>(xr + 8 * t) : zero8;
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
            }
            // this slot takes the step RING ahead (clamped past the stream's end)
            lm_load<NSB>(a, tile_row(k + (sb + RING) / NSB), (sb + RING) % NSB, ring[sb % RING]);
        }
        // tile done: lane (j, q) holds rows v0 .. v0 + 3 of verify row j
        const int v0 = tile_row(k) + 4 * q;
        if (live) {
            if (a.logits) {
                float* o = a.logits + (size_t)j * V + v0;
                if (vec_out && v0 + 3 < V) {
                    *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (v0 + e < V) o[e] = acc[e];
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (v0 + e < V) {
                    const unsigned long long kk = lm_key(acc[e], v0 + e);
                    best = kk > best ? kk : best;
                }
            }
            if (my_draft >= v0 && my_draft < v0 + 4 && my_draft < V) {
                const int e = my_draft - v0;
                a.draft_logit[j] = e == 0 ? acc[0] : e == 1 ? acc[1] : e == 2 ? acc[2] : acc[3];
            }
        }
    }
    // best of verify row j over the wave (lanes j, j+16, j+32, j+48), then
    // over the workgroup's waves
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
        const unsigned long long other =
            ((unsigned long long)(uint32_t)__shfl_xor((int)(uint32_t)(best >> 32), o, 64) << 32) |
            (unsigned long long)(uint32_t)__shfl_xor((int)(uint32_t)best, o, 64);
        best = other > best ? other : best;
    }
    if (q == 0) s_best[wave][j] = best;
    __syncthreads();
    if (tid < K) {
        unsigned long long b = s_best[0][tid];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) b = s_best[w][tid] > b ? s_best[w][tid] : b;
        a.part[(size_t)blockIdx.x * K + tid] = b;
    }
}

// ---------------------------------------------------------------------------
// k_lm_head_rows: the same results for up to 4 verify rows on the vector
// ALUs, with every load of a wave 1 KB contiguous.  A wave streams groups of
// R consecutive vocabulary rows (R * 4 KB contiguous at hidden 2048): lane l
// reads columns [512 t + 8 l, +8) of each row (t < H / 512), the next group's
// loads in flight while the current one is reduced.  x stays in registers
// (the same columns of every verify row).  Per (vocabulary row, verify row)
// the lane's partial dot product (v_dot2_f32_bf16, fp32) is summed over the
// wave with DPP.
// ---------------------------------------------------------------------------

template <int NC, int MAXM, int R>
__global__ __launch_bounds__(kBlock) void k_lm_head_rows(LmArgs a) {
    constexpr int H = NC * 512;
    __shared__ unsigned long long s_best[kWaves][MAXM];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = a.K, V = a.V;
    const int n_groups = (V + R - 1) / R;
    const int gw = blockIdx.x * kWaves + wave, GW = gridDim.x * kWaves;
    const int n_my = gw < n_groups ? (n_groups - 1 - gw) / GW + 1 : 0;
    auto group_row = [&](int g) { return n_my > 0 ? (gw + min(g, n_my - 1) * GW) * R : 0; };
    auto load = [&](int v0, uint4 (&w)[R][NC]) {
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            const uint4* p = reinterpret_cast<const uint4*>(a.w + (size_t)min(v0 + rr, V - 1) * H) + lane;
#pragma unroll
            for (int t = 0; t < NC; ++t) w[rr][t] = ld16_nt(p + 64 * t);
        }
    };
    uint4 wa[R][NC], wb[R][NC];
    load(group_row(0), wa);
    uint4 xv[MAXM][NC];
#pragma unroll
    for (int m = 0; m < MAXM; ++m)
#pragma unroll
        for (int t = 0; t < NC; ++t)
            xv[m][t] = *reinterpret_cast<const uint4*>(a.x + (size_t)min(m, K - 1) * H + 512 * t + 8 * lane);
    int dr[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) dr[m] = (a.draft && m < K - 1) ? a.draft[m] : -1;

    unsigned long long best[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) best[m] = 0ull;
    auto reduce = [&](int v0, const uint4 (&w)[R][NC]) {
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            const int v = v0 + rr;
#pragma unroll
            for (int m = 0; m < MAXM; ++m) {
                float acc = 0.0f;
#pragma unroll
                for (int t = 0; t < NC; ++t) {
                    acc = dot2(as_bf16x2(w[rr][t].x), as_bf16x2(xv[m][t].x), acc);
                    acc = dot2(as_bf16x2(w[rr][t].y), as_bf16x2(xv[m][t].y), acc);
                    acc = dot2(as_bf16x2(w[rr][t].z), as_bf16x2(xv[m][t].z), acc);
                    acc = dot2(as_bf16x2(w[rr][t].w), as_bf16x2(xv[m][t].w), acc);
                }
                const float l = wave_sum(acc);
                if (m < K && v < V) {
                    const unsigned long long kk = lm_key(l, v);
                    best[m] = kk > best[m] ? kk : best[m];
                    if (lane == 0) {
                        if (a.logits) a.logits[(size_t)m * V + v] = l;
                        if (dr[m] == v) a.draft_logit[m] = l;
                    }
                }
            }
        }
    };
    // groups in pairs: the other register set's loads are always issued
    // (clamped past the end, L2 hits) so the count of loads in flight stays
    // exact
    for (int g = 0; g < n_my; g += 2) {
        load(group_row(g + 1), wb);
        reduce(group_row(g), wa);
        load(group_row(g + 2), wa);
        if (g + 1 < n_my) reduce(group_row(g + 1), wb);
    }
    if (lane == 0) {
#pragma unroll
        for (int m = 0; m < MAXM; ++m) s_best[wave][m] = best[m];
    }
    __syncthreads();
    if (tid < K) {
        unsigned long long b = 0ull;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
#pragma unroll
            for (int m = 0; m < MAXM; ++m)
                if (m == tid) b = s_best[w][m] > b ? s_best[w][m] : b;
        }
        a.part[(size_t)blockIdx.x * K + tid] = b;
    }
}

struct GreedyArgs {
    const unsigned long long* part;  // [n_parts][K]
    int n_parts, K;
    const int32_t* draft;            // [K-1] or nullptr
    const float* draft_logit;        // [K]
    float tie_tol;
    int V;
    int32_t* target;                 // [K]
    float* target_logit;             // [K]
    int32_t* n_accepted;             // [1]
    int32_t* emitted;                // [K]
    int32_t* n_emitted;              // [1]
};

__global__ __launch_bounds__(kBlock) void k_greedy_finalize(GreedyArgs a) {
    __shared__ unsigned long long s_row[kWaves][kLmMaxRows];
    __shared__ int s_tok[kLmMaxRows];
    __shared__ float s_log[kLmMaxRows];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = a.K;
    for (int r = 0; r < K; ++r) {
        unsigned long long b = 0ull;
        for (int p = tid; p < a.n_parts; p += kBlock) {
            const unsigned long long v = a.part[(size_t)p * K + r];
            b = v > b ? v : b;
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const unsigned long long other =
                ((unsigned long long)(uint32_t)__shfl_xor((int)(uint32_t)(b >> 32), o, 64) << 32) |
                (unsigned long long)(uint32_t)__shfl_xor((int)(uint32_t)b, o, 64);
            b = other > b ? other : b;
        }
        if (lane == 0) s_row[wave][r] = b;
    }
    __syncthreads();
    if (tid < K) {
        unsigned long long b = s_row[0][tid];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) b = s_row[w][tid] > b ? s_row[w][tid] : b;
        s_tok[tid] = lm_key_token(b);
        s_log[tid] = lm_key_logit(b);
        a.target[tid] = s_tok[tid];
        a.target_logit[tid] = s_log[tid];
    }
    __syncthreads();
    if (tid == 0) {
        // the longest accepted prefix: draft[r] is checked against row r
        int n = 0;
        while (n < K - 1) {
            const int d = a.draft[n];
            // a token id outside the vocabulary is never accepted
            if (d >= 0 && d < a.V && (d == s_tok[n] || a.draft_logit[n] >= s_log[n] - a.tie_tol)) {
                a.emitted[n] = d;
                ++n;
            } else {
                break;
            }
        }
        a.emitted[n] = s_tok[n];
        *a.n_accepted = n;
        *a.n_emitted = n + 1;
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

size_t lm_head_lds_bytes(int H, int K) { return (size_t)K * xh_row_stride(H) * 2; }

// workgroups of the lm_head launch (a persistent grid: every wave streams
// several tiles) and their partial results
int lm_head_grid(int V) {
    const int n_tiles = (V + 15) / 16;
    const int wgs = (n_tiles + kWaves - 1) / kWaves;
    return wgs < 2048 ? wgs : 2048;
}

// Which kernel serves K rows at hidden H: the row-streaming vector kernel up
// to 4 rows (H >= 512), the matrix-core tiles above.
constexpr int kLmRowsR = 2;  // vocabulary rows per group of the row kernel
bool lm_use_rows(int K, int H) { return K <= 4 && H >= 512; }
int lm_rows_grid(int V) {
    const int n_groups = (V + kLmRowsR - 1) / kLmRowsR;
    const int wgs = (n_groups + kWaves - 1) / kWaves;
    return wgs < 1024 ? wgs : 1024;
}
int lm_grid(int V, int K, int H) { return lm_use_rows(K, H) ? lm_rows_grid(V) : lm_head_grid(V); }

template <int NC>
hipError_t launch_rows(const LmArgs& a, int grid, hipStream_t st) {
    if (a.K <= 1) hipLaunchKernelGGL((k_lm_head_rows<NC, 1, kLmRowsR>), dim3(grid), dim3(kBlock), 0, st, a);
    else if (a.K <= 2) hipLaunchKernelGGL((k_lm_head_rows<NC, 2, kLmRowsR>), dim3(grid), dim3(kBlock), 0, st, a);
    else hipLaunchKernelGGL((k_lm_head_rows<NC, 4, kLmRowsR>), dim3(grid), dim3(kBlock), 0, st, a);
    return hipGetLastError();
}

hipError_t init_lm_head_kernels() {
    static hipError_t once = [] {
        const void* ks[] = {reinterpret_cast<const void*>(k_lm_head<1>), reinterpret_cast<const void*>(k_lm_head<2>),
                            reinterpret_cast<const void*>(k_lm_head<4>), reinterpret_cast<const void*>(k_lm_head<8>)};
        for (const void* k : ks) {
            hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)lm_head_lds_bytes(2048, kLmMaxRows));
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }();
    return once;
}

hipError_t launch_lm_head_greedy(const uint16_t* x, int K, const uint16_t* w, int V, int H, const int32_t* draft,
                                 float tie_tol, float* logits, int32_t* target, float* target_logit,
                                 int32_t* n_accepted, int32_t* emitted, int32_t* n_emitted, void* workspace,
                                 hipStream_t st) {
    hipError_t e = init_lm_head_kernels();
    if (e != hipSuccess) return e;
    const int grid = lm_grid(V, K, H);
    LmArgs a{};
    a.x = x; a.w = w; a.draft = draft; a.logits = logits;
    a.part = reinterpret_cast<unsigned long long*>(workspace);
    a.draft_logit = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + (size_t)grid * K * 8);
    a.K = K; a.V = V; a.H = H;
    const size_t lds = lm_head_lds_bytes(H, K);
    if (lm_use_rows(K, H)) {
        switch (H) {
            case 512: e = launch_rows<1>(a, grid, st); break;
            case 1024: e = launch_rows<2>(a, grid, st); break;
            default: e = launch_rows<4>(a, grid, st); break;
        }
    } else switch (H) {
        case 256: hipLaunchKernelGGL(k_lm_head<1>, dim3(grid), dim3(kBlock), lds, st, a); break;
        case 512: hipLaunchKernelGGL(k_lm_head<2>, dim3(grid), dim3(kBlock), lds, st, a); break;
        case 1024: hipLaunchKernelGGL(k_lm_head<4>, dim3(grid), dim3(kBlock), lds, st, a); break;
        case 2048: hipLaunchKernelGGL(k_lm_head<8>, dim3(grid), dim3(kBlock), lds, st, a); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || (e = hipGetLastError()) != hipSuccess) return e;
    GreedyArgs g{};
    g.part = a.part; g.n_parts = grid; g.K = K;
    g.draft = draft; g.draft_logit = a.draft_logit; g.tie_tol = tie_tol; g.V = V;
    g.target = target; g.target_logit = target_logit; g.n_accepted = n_accepted;
    g.emitted = emitted; g.n_emitted = n_emitted;
    hipLaunchKernelGGL(k_greedy_finalize, dim3(1), dim3(kBlock), 0, st, g);
    return hipGetLastError();
}

size_t lm_head_workspace_bytes(int V, int K) {
    const int g = lm_head_grid(V) > lm_rows_grid(V) ? lm_head_grid(V) : lm_rows_grid(V);
    return (size_t)g * K * 8 + (size_t)kLmMaxRows * 4;
}

}  // namespace moe
