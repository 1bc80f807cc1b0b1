// gfx950 (CDNA4) kernels of the NVFP4 MoE block-verify layer, verify-width
// regime (K <= 16 rows).  Per layer two launches:
//   k_route_gateup  router workgroups (router GEMV, one wave per expert row,
//             bf16 x staged in LDS, v_dot2_f32_bf16, fp32 accumulation;
//             when chaining layers x is the RMS-normalised previous output)
//             hand their logits over inside the launch to the shared
//             expert's gate/up tiles and the routed workgroups, which each
//             repeat the selection from the logits (top-k per row with a
//             DPP wave argmax, after the router tail of PR #844 section 4:
//             argPartition + takeAlong) and the dedup CSR (PR #844 section 8
//             notes the stock gather reads a repeated expert once per slot;
//             here each unique expert is streamed once), then loop over work
//             items (unique expert, 16 intermediate rows) on the matrix
//             cores: 128-bit loads of packed E2M1 codes, in-register decode,
//             fp16 MFMA, SwiGLU epilogue writing fp32 h;
//   k_down    one workgroup per 8 output rows: every unique expert's down
//             rows for that slab (fp32 decode, fp32 h), per-slot partials in
//             LDS, then the deterministic combine
//             y = rs * sum_j w_j o_j + shared (+ residual) in rank order
//             (PR #844 section 5 expression order).
// The routed work list is data dependent (the number of unique experts is
// known only on the device), so the gate/up grid is sized for the largest
// possible count (capped; workgroups loop) and surplus workgroups finish
// after the selection.  No kernel uses a device-wide fence: on this part an
// agent-scope release writes back the L2 and costs far more than a launch
// boundary inside a graph; the in-launch hand-off uses agent-scope relaxed
// stores completed with a wait on the memory counters instead.
// On request (at most 2 rows) k_route_gateup also carries the down
// projection as a third group of workgroups (down_role), making the layer
// one launch; it computes the same bits but measured slower than the two
// launches, so it is not the default.

#include <hip/hip_ext.h>

#include "moe_device.h"

namespace moe {


// Canonical dedup of the n = K*k selected slots with the whole workgroup.
// A row never selects an expert twice, so expert e's slots are one per row
// that picked it, in row order: with rowmask[e] the set of those rows,
//   count(e) = popcount(rowmask[e]),
//   rank of slot (r, j) inside its expert = popcount(rowmask[e] & (2^r - 1)).
// Exclusive prefix sums over experts of count(e) and of (count(e) > 0) give
// the CSR offset and the position in the ascending unique list.
// Results go to sm.asg / sm.inv / sm.uniq / sm.off / sm.n_unique.
__device__ __forceinline__ void dedup_block(SelectSmem& sm, uint32_t* rowmask, int32_t* cstart, int n, int k, int E) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ int s_wsum[kWaves][2];
    for (int e = tid; e < E; e += kBlock) rowmask[e] = 0u;
    __syncthreads();
    for (int s = tid; s < n; s += kBlock) atomicOr(&rowmask[sm.sel[s]], 1u << (s / k));
    __syncthreads();
    // each thread owns Q consecutive experts
    const int Q = (E + kBlock - 1) / kBlock;
    int c = 0, f = 0;
    for (int q = 0; q < Q; ++q) {
        const int e = tid * Q + q;
        if (e < E) {
            const int cn = __builtin_popcount(rowmask[e]);
            c += cn;
            f += (cn > 0);
        }
    }
    const int ci = wave_incl_scan(c), fi = wave_incl_scan(f);
    if (lane == 63) { s_wsum[wave][0] = ci; s_wsum[wave][1] = fi; }
    __syncthreads();
    int cb = 0, fb = 0;
    for (int w = 0; w < wave; ++w) { cb += s_wsum[w][0]; fb += s_wsum[w][1]; }
    int cs = cb + ci - c, fs = fb + fi - f;
    for (int q = 0; q < Q; ++q) {
        const int e = tid * Q + q;
        if (e < E) {
            const int cn = __builtin_popcount(rowmask[e]);
            cstart[e] = cs;
            if (cn) { sm.uniq[fs] = e; sm.off[fs] = cs; }
            cs += cn;
            fs += (cn > 0);
        }
    }
    if (tid == kBlock - 1) {
        int U = 0;
        for (int w = 0; w < kWaves; ++w) U += s_wsum[w][1];
        sm.n_unique = U;
        sm.off[U] = n;
    }
    __syncthreads();
    for (int s = tid; s < n; s += kBlock) {
        const int e = sm.sel[s], r = s / k;
        const int pos = cstart[e] + __builtin_popcount(rowmask[e] & ((1u << r) - 1u));
        sm.asg[pos] = s;
        sm.inv[s] = pos;
    }
}

// All rows' top-k, then the canonical dedup CSR, left in LDS and, if
// write_global, also in the SelectArgs outputs.  lg: K*E floats of LDS.
// Returns the number of unique experts.
// Top-k of every row (lg: the K*E logits already in LDS), one wave per row.
__device__ void select_rows(const SelectArgs& a, SelectSmem& sm, const float* lg) {
    const int wave = threadIdx.x >> 6;
    for (int r = wave; r < a.K; r += kWaves) wave_topk_rt(a, lg + r * a.E, r, sm);
}
template <int P>
__device__ __forceinline__ void select_rows_p(const SelectArgs& a, SelectSmem& sm, const float* lg, bool weights) {
    const int wave = threadIdx.x >> 6;
    for (int r = wave; r < a.K; r += kWaves) wave_topk<P>(a, lg + r * a.E, r, sm, weights);
}

// The canonical dedup CSR of the selection in sm (whole workgroup), written
// with ids and w to the SelectArgs outputs.  Returns the unique count.
__device__ __forceinline__ int dedup_publish(const SelectArgs& a, SelectSmem& sm) {
    const int tid = threadIdx.x;
    const int k = a.k, n = a.K * k;
    dedup_block(sm, sm.rowmask, sm.cstart, n, k, a.E);
    __syncthreads();
    const int U = sm.n_unique;
    for (int s = tid; s < n; s += kBlock) {
        a.asg[s] = sm.asg[s];
        a.inv[s] = sm.inv[s];
        a.ids[s] = sm.sel[s];
        a.w[s] = sm.w[s];
    }
    for (int u = tid; u <= U; u += kBlock) {
        if (u < U) a.uniq[u] = sm.uniq[u];
        a.off[u] = sm.off[u];
    }
    if (tid == 0) *a.n_unique = U;
    return U;
}

// All rows' top-k, then the canonical dedup CSR, published to the SelectArgs
// outputs.  lg: K*E floats of LDS.
__device__ int select_and_dedup(const SelectArgs& a, SelectSmem& sm, float* lg) {
    stage_floats(lg, a.logits, a.K * a.E, threadIdx.x, kBlock);
    __syncthreads();
    select_rows(a, sm, lg);
    __syncthreads();
    return dedup_publish(a, sm);
}

__host__ __device__ constexpr size_t select_smem_bytes(int K, int E) {
    return (sizeof(SelectSmem) + 15) / 16 * 16 + (size_t)K * E * sizeof(float);
}

// Selection from caller-provided logits (one workgroup).
__global__ __launch_bounds__(kBlock) void k_select(SelectArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    SelectSmem& sm = *reinterpret_cast<SelectSmem*>(smem);
    float* lg = reinterpret_cast<float*>(smem + (sizeof(SelectSmem) + 15) / 16 * 16);
    select_and_dedup(a, sm, lg);
}

// ---------------------------------------------------------------------------
// gate/up tile on the matrix cores: 16 rows of gate and of up for one expert
// against up to 16 rows of x (v_mfma_f32_16x16x32_f16).
//
// Operands.  Each weight is decoded FP4 -> fp16 (v_cvt_scalef32_pk_f16_fp4,
// scale operand 1) and multiplied by its E4M3 block scale with a packed fp16
// multiply: an E2M1 value times an E4M3 value has at most 6 significant bits
// and lies in [2^-10, 2688], so the fp16 product is exact.  x enters as fp16
// of x * 2^-sig with a per-row power of two (convert_rows: exact for every value
// within 2^-28 of the row's largest magnitude, no overflow at any bf16
// magnitude).  Products accumulate in fp32; 2^sig and the tensor scale
// multiply the sum.
//
// Layout.  Lane (i = lane % 16, kb = lane / 16).  A superblock is 256
// columns; lane (i, kb) owns columns [sb*256 + kb*64, +64) of weight row
// n0 + i: 32 contiguous code bytes and 4 scale bytes.  MFMA step s (0..7)
// feeds the lane's codes 8s..8s+7 as its A k-block, and lane (j, kb) feeds
// x row j at the same 8 columns as its B k-block; the contraction over k is
// order independent, so this permutation of k is consistent on both sides.
// The accumulator of lane (j, q) holds rows n0 + 4q .. +3 for x row j.  The
// 4 waves split the superblocks and add their partial sums through LDS in a
// fixed order.
// ---------------------------------------------------------------------------

constexpr int kRedFloats = kWaves * 2 * 64 * 4;  // cross-wave partials of the gate/up tile

struct GuRegs {
    GuSb sb0, sb1;  // this wave's superblocks wave and wave + kWaves
};


__device__ __forceinline__ GuRegs gu_load(const uint8_t* gq, const uint8_t* gs, const uint8_t* uq, const uint8_t* us,
                                         int H, int n0) {
    const int wave = threadIdx.x >> 6;
    const int nsb = H / kSbCols;
    GuRegs R;
    R.sb0 = gu_load_sb(gq, gs, uq, us, H, n0, wave, wave < nsb);
    R.sb1 = gu_load_sb(gq, gs, uq, us, H, n0, wave + kWaves, wave + kWaves < nsb);
    return R;
}


// The eight MFMA steps of one superblock.
// xr: this lane's x row in LDS at the superblock's first column of its
// 64-column block (8 consecutive halfs per MFMA step, no padding inside).
__device__ __forceinline__ void gu_mfma_sb(const GuSb& r, const _Float16* xr, bool has_x, f32x4_t& accg,
                                           f32x4_t& accu) {
    const f16x8_t zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    const _Float16 g0 = e4m3_to_f16<0>(r.gs), g1 = e4m3_to_f16<1>(r.gs);
    const _Float16 g2 = e4m3_to_f16<2>(r.gs), g3 = e4m3_to_f16<3>(r.gs);
    const _Float16 u0 = e4m3_to_f16<0>(r.us), u1 = e4m3_to_f16<1>(r.us);
    const _Float16 u2 = e4m3_to_f16<2>(r.us), u3 = e4m3_to_f16<3>(r.us);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const _Float16 gsc = (s < 2) ? g0 : (s < 4) ? g1 : (s < 6) ? g2 : g3;
        const _Float16 usc = (s < 2) ? u0 : (s < 4) ? u1 : (s < 6) ? u2 : u3;
        const f16x8_t ag = decode8_f16(pick_word(r.g0, r.g1, s), gsc);
        const f16x8_t au = decode8_f16(pick_word(r.u0, r.u1, s), usc);
        const f16x8_t b = has_x ? *reinterpret_cast<const f16x8_t*>(xr + 8 * s) : zero8;
        accg = __builtin_amdgcn_mfma_f32_16x16x32_f16(ag, b, accg, 0, 0, 0);
        accu = __builtin_amdgcn_mfma_f32_16x16x32_f16(au, b, accu, 0, 0, 0);
    }
}

// xh: fp16 x rows in LDS (padded layout, xh_index); rows >= m_cnt are not read.
// Writes h[j * hstride + n0 + r] for x rows j < m_cnt and the tile's 16 rows.
// xh: fp16 x rows in LDS (padded layout, xh_index).  MFMA column j < m_cnt
// takes x row xrows[j] and its h goes to row hrows[j] of hbase (identity
// maps when null).  Writes h[hrows[j]][n0 .. n0+15].
__device__ __forceinline__ void gu_compute(const GuRegs& R, float gts, float uts, int H, int n0,
                                           const _Float16* xh, const int* xsig, int m_cnt, const int* xrows,
                                           const int* hrows, float* hbase, int hstride, float* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, kb = lane >> 4;
    const int nsb = H / kSbCols;
    const int xr = (j < m_cnt) ? (xrows ? xrows[j] : j) : 0;
    f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
    // this wave's superblocks wave and wave + kWaves, in load order: the
    // first is multiplied while the second's loads are still in flight
    if (wave < nsb) gu_mfma_sb(R.sb0, xh + xh_index(xr, wave * kSbCols + kb * 64, H), j < m_cnt, accg, accu);
    if (wave + kWaves < nsb)
        gu_mfma_sb(R.sb1, xh + xh_index(xr, (wave + kWaves) * kSbCols + kb * 64, H), j < m_cnt, accg, accu);
    reinterpret_cast<f32x4_t*>(red)[(wave * 2 + 0) * 64 + lane] = accg;
    reinterpret_cast<f32x4_t*>(red)[(wave * 2 + 1) * 64 + lane] = accu;
    __syncthreads();
    if (wave == 0 && j < m_cnt) {
        f32x4_t g = reinterpret_cast<const f32x4_t*>(red)[lane];
        f32x4_t u = reinterpret_cast<const f32x4_t*>(red)[64 + lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
            g += reinterpret_cast<const f32x4_t*>(red)[(w * 2 + 0) * 64 + lane];
            u += reinterpret_cast<const f32x4_t*>(red)[(w * 2 + 1) * 64 + lane];
        }
        // undo the x row's power-of-two scale, then the tensor scales
        const int sg = xsig[xr];
        float4 h;
        float gv, uv;
        gv = ldexpf(g[0], sg) * gts; uv = ldexpf(u[0], sg) * uts; h.x = gv / (1.0f + expf(-gv)) * uv;
        gv = ldexpf(g[1], sg) * gts; uv = ldexpf(u[1], sg) * uts; h.y = gv / (1.0f + expf(-gv)) * uv;
        gv = ldexpf(g[2], sg) * gts; uv = ldexpf(u[2], sg) * uts; h.z = gv / (1.0f + expf(-gv)) * uv;
        gv = ldexpf(g[3], sg) * gts; uv = ldexpf(u[3], sg) * uts; h.w = gv / (1.0f + expf(-gv)) * uv;
        const int hr = hrows ? hrows[j] : j;
        // written through to the device-coherent level: a down workgroup of
        // the same launch may read it (after the completion hand-off)
        uint64_t* dst = reinterpret_cast<uint64_t*>(hbase + (size_t)hr * hstride + n0 + 4 * kb);
        __hip_atomic_store(dst, (uint64_t)__float_as_uint(h.x) | ((uint64_t)__float_as_uint(h.y) << 32),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(dst + 1, (uint64_t)__float_as_uint(h.z) | ((uint64_t)__float_as_uint(h.w) << 32),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// x staging for the matrix cores, in two phases around a workgroup barrier.
// Phase 1 (stage_x with padded = true): the K bf16 x rows go to LDS
// unconverted, in the padded fp16 layout.  Phase 2 (convert_rows, after the
// barrier): whole rows, one per wave at a time -- the wave finds the row's
// largest |x| (DPP maximum), scales the row by 2^-sig and converts it to
// fp16 in place; sig goes to xsig[row].  No wave waits for another here, so
// the waves that select no row convert while the others select.

// Phase 2 by waves w0 .. w0 + nw - 1 (the calling wave converts rows
// wave - w0, + nw, ...).  H <= 2048: at most four pieces per lane.
__device__ __forceinline__ void convert_rows(_Float16* xh, int K, int H, int* xsig, int w0, int nw) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (wave < w0 || wave >= w0 + nw) return;
    const int per_row = H / 8;
    for (int r = wave - w0; r < K; r += nw) {
        uint4 v[4];
        uint32_t m = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = lane + 64 * j;
            v[j] = (c < per_row) ? *reinterpret_cast<const uint4*>(xh + xh_index(r, c * 8, H)) : make_uint4(0, 0, 0, 0);
            m = max(m, bf16x8_maxabs(v[j]));
        }
        const int sg = row_sigma(wave_max_u32(m));
        if (lane == 0) xsig[r] = sg;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = lane + 64 * j;
            if (c < per_row) *reinterpret_cast<uint4*>(xh + xh_index(r, c * 8, H)) = bf16x8_to_f16x8_scaled(v[j], -sg);
        }
    }
}

// ---------------------------------------------------------------------------
// Router x.  When chaining layers, x is the RMS-normalised previous output
// times the norm weight (bf16), with the sums of squares taken from the down
// kernel's per-workgroup partials; every workgroup that needs x normalises
// all rows itself, and each router workgroup publishes its share of x.
// ---------------------------------------------------------------------------

constexpr int kRouterPieces = 4;  // 16-byte router pieces per lane (hidden <= 2048)

// Builds this layer's bf16 x in LDS from x_in (rows of this launch's chunk)
// or from y_prev: dense rows xs[K][H] (padded = false) or the padded layout
// of the matrix-core x operand (padded = true, xh_index).  With publish_n >
// 0 the workgroup also writes its share publish_idx of x to x_out.  Every
// caller runs the same arithmetic, so every workgroup holds the same bits.
__device__ __forceinline__ void stage_x(const RouterArgs& a, const uint16_t* x_in, int K, uint16_t* xs, float* s_inv,
                        int publish_idx, int publish_n, bool padded = false) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, KH = K * H, lgH = __builtin_ctz(H);  // H is a power of two
    auto dst = [&](int i) { return padded ? xs + xh_index(i >> lgH, i & (H - 1), H) : xs + i; };
    if (a.y_prev) {
        constexpr int CH = 2;  // float4 pairs (16 elements) per thread per pass
        float4 v[2 * CH];
        uint4 gv[CH];          // the norm weight of the same 8 columns (bf16)
        const uint16_t* const gam = a.gamma ? a.gamma : kBf16Ones;
        auto load_pass = [&](int base) {
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int i = base + (j * kBlock + tid) * 8;
                const bool ok = i < KH;
                v[2 * j] = ok ? *reinterpret_cast<const float4*>(a.y_prev + i) : make_float4(0, 0, 0, 0);
                v[2 * j + 1] = ok ? *reinterpret_cast<const float4*>(a.y_prev + i + 4) : make_float4(0, 0, 0, 0);
                gv[j] = *reinterpret_cast<const uint4*>(gam + (i & (H - 1)));
            }
        };
        load_pass(0);
        const int nparts = H / kDownRowsPerBlock;  // <= 256 for hidden <= 2048
        for (int r = wave; r < K; r += kWaves) {
            float pv[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int j = lane + 64 * t;
                pv[t] = (j < nparts) ? a.ssq[r * nparts + j] : 0.0f;
            }
            const float ss = wave_sum((pv[0] + pv[1]) + (pv[2] + pv[3]));
            if (lane == 0) s_inv[r] = 1.0f / sqrtf(ss / (float)H + a.eps);
        }
        __syncthreads();
        for (int base = 0; base < KH; base += kBlock * 8 * CH) {
            if (base > 0) load_pass(base);
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int i = base + (j * kBlock + tid) * 8;
                if (i < KH) {
                    // x = bf16((y * inv_rms) * gamma), fp32 products
                    const float sc = s_inv[i >> lgH];
                    const float4 p = v[2 * j], q = v[2 * j + 1];
                    const uint4 g = gv[j];
                    uint4 o;
                    o.x = (uint32_t)f32_to_bf16_rne(p.x * sc * bf16_to_f32(g.x & 0xFFFFu)) |
                          ((uint32_t)f32_to_bf16_rne(p.y * sc * bf16_to_f32(g.x >> 16)) << 16);
                    o.y = (uint32_t)f32_to_bf16_rne(p.z * sc * bf16_to_f32(g.y & 0xFFFFu)) |
                          ((uint32_t)f32_to_bf16_rne(p.w * sc * bf16_to_f32(g.y >> 16)) << 16);
                    o.z = (uint32_t)f32_to_bf16_rne(q.x * sc * bf16_to_f32(g.z & 0xFFFFu)) |
                          ((uint32_t)f32_to_bf16_rne(q.y * sc * bf16_to_f32(g.z >> 16)) << 16);
                    o.w = (uint32_t)f32_to_bf16_rne(q.z * sc * bf16_to_f32(g.w & 0xFFFFu)) |
                          ((uint32_t)f32_to_bf16_rne(q.w * sc * bf16_to_f32(g.w >> 16)) << 16);
                    *reinterpret_cast<uint4*>(dst(i)) = o;
                }
            }
        }
        __syncthreads();
        if (publish_n > 0) {  // this workgroup's share of the normalised x
            const int per = (KH / 8 + publish_n - 1) / publish_n * 8;
            const int i0 = publish_idx * per;
            for (int i = i0 + tid * 8; i < min(KH, i0 + per); i += kBlock * 8)
                *reinterpret_cast<uint4*>(a.x_out + i) = *reinterpret_cast<const uint4*>(dst(i));
        }
    } else {
        constexpr int CH = 4;
        for (int base = 0; base < KH; base += kBlock * 8 * CH) {
            uint4 v[CH];
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int i = base + (j * kBlock + tid) * 8;
                v[j] = (i < KH) ? *reinterpret_cast<const uint4*>(x_in + i) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int i = base + (j * kBlock + tid) * 8;
                if (i < KH) *reinterpret_cast<uint4*>(dst(i)) = v[j];
            }
        }
        __syncthreads();
    }
}

// Gate/up LDS: the selection's tables and staged logits, the padded fp16 x
// rows, the SwiGLU reduction scratch.
__host__ __device__ constexpr size_t gateup_smem_bytes(int K, int E, int H) {
    return select_smem_bytes(K, E) + (size_t)K * xh_row_stride(H) * 2 + (size_t)kRedFloats * 4;
}

// ---------------------------------------------------------------------------
// The down role of the fused layer launch (k_route_gateup with DOWN): one
// workgroup per kDownRowsPerBlock output rows, as k_down, but resident while
// gate/up runs.  It repeats the selection and dedup (from the hand-off
// logits, like a routed workgroup), requests the down weights of all its
// tasks into registers, waits for the gate/up completion flag, stages h
// (written through by the gate/up workgroups, read with device-coherent
// loads) in LDS and finishes as k_down: per-slot partial rows, the
// rank-order combine, y, y32 and the next layer's sum-of-squares partials.
// h is staged unpadded; float4 column c4 of a row sits at c4 ^ ((c4 >> 3) & 7)
// so the 16 chunk lanes of a weight row read distinct banks.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int h_swz(int c4) { return c4 ^ ((c4 >> 3) & 7); }

// Cache-policy bits of a load that reads the device-coherent level (what
// agent-scope atomic loads use on this part: sc1).
constexpr int kCachePolicyAgent = 16;

constexpr int kFusedMaxP = 4;  // experts per top-k lane (E <= 256) of the one-launch layer
constexpr int kFusedDownIlp = 1;  // down tasks of a wave computed interleaved (3: 133 registers)

// The down role's dynamic LDS: h rows (max(I, Is) floats each) and per-slot
// partial rows from offset 0 (over the selection's tables once they are
// done), then the routing lists copied out of those tables, and y.
__host__ __device__ constexpr size_t fused_down_lists_offset(int K, int k, int E, int I, int Is) {
    return ((size_t)(K * k + K) * (size_t)((I > Is ? I : Is) + kDownRowsPerBlock) * 4 > select_smem_bytes(K, E)
                ? (size_t)(K * k + K) * (size_t)((I > Is ? I : Is) + kDownRowsPerBlock) * 4
                : select_smem_bytes(K, E)) /
               16 * 16 + 16;
}
__host__ __device__ constexpr size_t fused_down_lds_bytes(int K, int k, int E, int I, int Is) {
    return fused_down_lists_offset(K, k, E, I, Is) + (size_t)(4 * K * k + 2) * 4 + (size_t)K * kDownRowsPerBlock * 4;
}

// Bounded wait of thread 0 for a hand-off flag; status := 1 if it gives up.
__device__ __forceinline__ void wait_flag(const uint32_t* flag, int32_t* status, int spin_limit) {
    if (threadIdx.x == 0) {
        int spins = 0;
        while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
            if (++spins > spin_limit) {
                __hip_atomic_store(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __syncthreads();
}

// The K*E router logits of this launch into LDS with device-coherent loads.
__device__ __forceinline__ void load_handoff_logits(float* lg, const float* logits, int n) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(logits);
    const int tid = threadIdx.x;
    constexpr int U = 4;
    for (int base = 0; base < n; base += U * kBlock) {
        uint32_t v[U];
#pragma unroll
        for (int q = 0; q < U; ++q) {
            const int i = base + q * kBlock + tid;
            v[q] = i < n ? __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
        }
#pragma unroll
        for (int q = 0; q < U; ++q) {
            const int i = base + q * kBlock + tid;
            if (i < n) lg[i] = __uint_as_float(v[q]);
        }
    }
}

template <int P>
__device__ __forceinline__ void down_role(const RouteGateUpArgs& a, unsigned char* smem, int db) {
    constexpr int NH = kDownRowsPerBlock;
    constexpr int NB = kFusedDownTasks;
    const DownArgs& d = a.d;
    const SelectArgs& sel = a.g.sel;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = d.H, K = d.K, k = d.k, n = K * k, E = sel.E, I = d.I, Is = d.Is;
    const bool has_sh = d.sdown.q != nullptr;
    const int n_base = db * NH;
    const int RL = max(I, has_sh ? Is : 0);
    const int total_rows = n + (has_sh ? K : 0);
    // dynamic LDS: h rows, then per-slot partial rows, routing lists, y
    float* hs = reinterpret_cast<float*>(smem);
    float* so = hs + (size_t)total_rows * RL;
    int* d_pe = reinterpret_cast<int*>(smem + fused_down_lists_offset(K, k, E, I, Is));  // expert of each h row
    int* d_inv = d_pe + n;
    float* d_w = reinterpret_cast<float*>(d_inv + n);
    float* s_y = d_w + n;
    SelectSmem& sm = *reinterpret_cast<SelectSmem*>(smem);
    float* lg = reinterpret_cast<float*>(smem + (sizeof(SelectSmem) + 15) / 16 * 16);

    // the next layer's router rows, requested into the memory-side cache
    uint4 pf = make_uint4(0, 0, 0, 0);
    if (d.prefetch) {
        const int n16 = d.prefetch_bytes >> 4;
        const int i = min(db * kBlock + tid, n16 - 1);
        pf = reinterpret_cast<const uint4*>(d.prefetch)[i];
    }

    // ---- selection and dedup from the router's logits
    wait_flag(a.counter + kHandoffFlagStride * (kSlotRouterFlag + blockIdx.x % kHandoffFlags), a.status,
              a.spin_limit);
    load_handoff_logits(lg, sel.logits, K * E);
    asm volatile("" ::"v"(pf.x), "v"(pf.y), "v"(pf.z), "v"(pf.w));  // the prefetch stays issued
    __syncthreads();
    select_rows_p<P>(sel, sm, lg, true);
    __syncthreads();
    dedup_block(sm, sm.rowmask, sm.cstart, n, k, E);
    __syncthreads();
    for (int i = tid; i < n; i += kBlock) {
        d_pe[i] = sm.sel[sm.asg[i]];
        d_inv[i] = sm.inv[i];
        d_w[i] = sm.w[i];
    }
    __syncthreads();

    // ---- the down weights of this wave's tasks, requested before the wait.
    // A task is one h row p (routed rows in dedup order, then the shared
    // rows) and 64 / CPR of this workgroup's output rows (gI tasks per h
    // row); task t belongs to wave t % kWaves.  A routed expert picked by
    // both rows has two tasks per row group that read the same weights (the
    // second read hits the cache).  Routed and shared rows have the same
    // length here (I == Is), so every task has the same lane map.
    const int CPR = I >> 5, lgI = __builtin_ctz(CPR);
    const int gI = max(1, NH / (64 / CPR)), lgG = __builtin_ctz(gI);
    const int nT = total_rows * gI;
    const int q = lane >> lgI, chunk = lane & (CPR - 1);
    uint4 code[NB];
    uint32_t scl[NB];
    float tsv[NB];
    int pt[NB];  // the task's h row (wave-uniform)
    {
        int ev[NB];  // the task's expert (wave-uniform: tensor scales become scalar loads)
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int t = min(i * kWaves + wave, nT - 1);
            pt[i] = t >> lgG;
            ev[i] = __builtin_amdgcn_readfirstlane(pt[i] < n ? d_pe[pt[i]] : 0);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            // unconditional loads (a task past the end repeats the last
            // task's addresses; its result is not stored)
            const int t = min(i * kWaves + wave, nT - 1);
            const bool shared_task = pt[i] >= n;
            const int e = ev[i];
            const uint8_t* mq = shared_task ? d.sdown.q : d.down.q;
            const uint8_t* ms = shared_task ? d.sdown.s : d.down.s;
            const float* mts = shared_task ? d.sdown.ts : d.down.ts;
            const int nl = ((t & (gI - 1)) << (6 - lgI)) + q;
            const size_t row = (size_t)e * H + n_base + (nl < NH ? nl : 0);
            tsv[i] = mts[e];
            code[i] = *reinterpret_cast<const uint4*>(mq + row * (I / 2) + chunk * 16);
            scl[i] = *reinterpret_cast<const uint16_t*>(ms + row * (I / 16) + chunk * 2);
        }
    }

    // ---- every gate/up workgroup has written h
    wait_flag(a.counter + kHandoffFlagStride * (kSlotDownFlag + blockIdx.x % kHandoffFlags), a.status,
              a.spin_limit);
    {
        // h rows (routed rows by dedup position, then the shared rows) into
        // LDS straight from the device-coherent level (global_load_lds with
        // the agent-scope cache bit): one wave instruction fills 64
        // consecutive float4 slots, slot j of row `row` taking column float4
        // h_swz(j) (the swizzle is its own inverse); no registers hold h.
        const int q4 = RL >> 2, lq4 = __builtin_ctz(q4);
        const int slots = total_rows * q4;
        for (int m = wave; m * 64 < slots; m += kWaves) {
            const int j = m * 64 + lane;
            if (j < slots) {
                const int row = j >> lq4, c4 = h_swz(j & (q4 - 1));
                const bool shared_row = row >= n;
                const int len4 = (shared_row ? Is : I) >> 2;
                const float* src = shared_row ? d.h_sh + (size_t)(row - n) * Is : d.h + (size_t)row * I;
                __builtin_amdgcn_global_load_lds(
                    (__attribute__((address_space(1))) void*)(src + 4 * min(c4, len4 - 1)),
                    (__attribute__((address_space(3))) void*)(hs + (size_t)m * 256), 16, 0, kCachePolicyAgent);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();

    // ---- tasks: the partial rows of this workgroup's output rows for every
    // h row, each (task) in k_down's arithmetic and order, kFusedDownIlp
    // tasks interleaved column block by column block (independent chains,
    // so a wave's LDS reads and FMAs overlap)
    {
        const int sw = chunk & 7;
        static_assert(NB % kFusedDownIlp == 0, "task groups");
#pragma unroll
        for (int i0 = 0; i0 < NB; i0 += kFusedDownIlp) {
            float acc[kFusedDownIlp][4];
#pragma unroll
            for (int i = 0; i < kFusedDownIlp; ++i) acc[i][0] = acc[i][1] = acc[i][2] = acc[i][3] = 0.0f;
#pragma unroll
            for (int t4 = 0; t4 < 8; ++t4) {
#pragma unroll
                for (int i = 0; i < kFusedDownIlp; ++i) {
                    const uint4& cd = code[i0 + i];
                    const uint32_t wd = t4 < 2 ? cd.x : t4 < 4 ? cd.y : t4 < 6 ? cd.z : cd.w;
                    f32x2_t wa, wb;  // the word's low or high four columns
                    if (t4 & 1) {
                        wa = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, 1.0f, 2);
                        wb = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, 1.0f, 3);
                    } else {
                        wa = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, 1.0f, 0);
                        wb = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, 1.0f, 1);
                    }
                    const float4 hv =
                        reinterpret_cast<const float4*>(hs + (size_t)pt[i0 + i] * RL + chunk * 32)[t4 ^ sw];
                    float& c = acc[i][t4 >> 1];
                    c = fmaf(wa.x, hv.x, c);
                    c = fmaf(wa.y, hv.y, c);
                    c = fmaf(wb.x, hv.z, c);
                    c = fmaf(wb.y, hv.w, c);
                }
            }
#pragma unroll
            for (int i = 0; i < kFusedDownIlp; ++i) {
                const int t = (i0 + i) * kWaves + wave;
                const float s0 = e4m3_to_f32<0>(scl[i0 + i]), s1 = e4m3_to_f32<1>(scl[i0 + i]);
                float pv = fmaf(acc[i][2] + acc[i][3], s1, (acc[i][0] + acc[i][1]) * s0);
                pv = (CPR == 16) ? group_sum<16>(pv) : group_sum_rt(pv, CPR);
                const int nl = ((t & (gI - 1)) << (6 - lgI)) + q;
                if (t < nT && nl < NH && chunk == CPR - 1) so[pt[i0 + i] * NH + nl] = pv * tsv[i0 + i];
            }
        }
    }
    __syncthreads();

    // ---- combine: y = rs * sum_j w_j o_j (rank order) + shared (+ residual)
    for (int i = tid; i < K * NH; i += kBlock) {
        const int r = i / NH, nl = i % NH, nn = n_base + nl;
        float acc = 0.0f;
        for (int j = 0; j < k; ++j) acc = fmaf(d_w[r * k + j], so[d_inv[r * k + j] * NH + nl], acc);
        float y = d.rs * acc;
        if (has_sh) y += so[(n + r) * NH + nl];
        if (d.residual) y += bf16_to_f32(d.residual[(size_t)r * H + nn]);
        d.y32[(size_t)r * H + nn] = y;
        if (d.y) d.y[(size_t)r * H + nn] = f32_to_bf16_rne(y);
        s_y[i] = y;
    }
    __syncthreads();
    if (d.ssq && tid < K) {
        float ss = 0.0f;
        for (int nl = 0; nl < NH; ++nl) ss = fmaf(s_y[tid * NH + nl], s_y[tid * NH + nl], ss);
        d.ssq[tid * a.n_down + db] = ss;
    }
}

// ---------------------------------------------------------------------------
// k_route_gateup: the router and the gate/up of one layer in one launch.
//   workgroups [0, n_router): the router GEMV (one wave per expert row);
//     each publishes its logits with agent-scope write-through
//     stores, waits until they have completed, then adds one to the hand-off
//     counter; the one that completes the count raises kHandoffFlags flags;
//   [n_router, n_router + Is/16): the shared expert's gate/up tiles (they
//     need x only);
//   the rest: routed gate/up workgroups.  They normalise x themselves while
//     the router runs, wait (bounded) for their flag (workgroup b polls flag
//     b % kHandoffFlags, so few poll any one address), read the logits with
//     agent-scope loads, repeat the top-k of every row (cheaper than a
//     separate launch or a grid-wide fence) and loop over work items (slot
//     r*k+j, 16 intermediate rows).  An item is done by the slot of the
//     first row that selected its expert, for every row that selected it,
//     so each unique expert is streamed once; items of later rows' slots of
//     the same expert are skipped.  h rows are indexed by position in the
//     canonical dedup order (expert ascending, then row), which each item
//     derives from the selection in LDS.  The first routed workgroup also
//     writes the canonical dedup CSR (for the down kernel) while its own
//     weight loads are in flight.
// Workgroups are dispatched in index order, so every router workgroup is
// resident before any workgroup that waits for it.  The counter is zero at
// launch (the previous layer's down kernel, or the call's first kernel,
// resets it).  A wait past its bound sets *status and goes on, so the
// launch always ends (the results are then invalid and the host reports
// the status).
// ---------------------------------------------------------------------------

// dynamic LDS limit of k_route_gateup: its static arrays (row lists, row
// scales, selection scratch) stay within 8 KB of the 160 KB
constexpr int kRgMaxDynLds = 160 * 1024 - 8 * 1024;

template <int P, int MAXM, bool DOWN>
__global__ __launch_bounds__(kBlock) void k_route_gateup(RouteGateUpArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_xrows[kWaves][kMaxRows];
    __shared__ int s_xsig[kMaxRows];
    __shared__ float s_inv[kMaxRows];
    const GateUpArgs& g = a.g;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = g.H, K = g.K, k = g.sel.k, I = g.I, n = K * k, E = g.sel.E;
    const int bid = blockIdx.x;

    if (bid < a.n_router) {
        // ---- router workgroup: this wave's router row, requested first
        if (DOWN && bid == 0 && a.clear && tid < kHandoffSlots)  // the next launch's hand-off set
            __hip_atomic_store(a.clear + kHandoffFlagStride * tid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
        const int e = bid * kWaves + wave;
        uint4 wv[kRouterPieces];
#pragma unroll
        for (int t = 0; t < kRouterPieces; ++t) {
            const int p = lane * 8 + t * 512;
            wv[t] = (e < E && p < H) ? *reinterpret_cast<const uint4*>(a.r.wr + (size_t)e * H + p)
                                     : make_uint4(0, 0, 0, 0);
        }
        stage_x(a.r, a.r.x_in, K, xs, s_inv, bid, a.n_router);
        if (e < E) {
            float acc[MAXM];
#pragma unroll
            for (int r = 0; r < MAXM; ++r) acc[r] = 0.0f;
#pragma unroll
            for (int t = 0; t < kRouterPieces; ++t) {
                const int p = lane * 8 + t * 512;
                if (p < H) {
#pragma unroll
                    for (int r = 0; r < MAXM; ++r) {
                        if (r < K) {
                            const uint4 xv = *reinterpret_cast<const uint4*>(xs + r * H + p);
                            float s = acc[r];
                            s = dot2(as_bf16x2(wv[t].x), as_bf16x2(xv.x), s);
                            s = dot2(as_bf16x2(wv[t].y), as_bf16x2(xv.y), s);
                            s = dot2(as_bf16x2(wv[t].z), as_bf16x2(xv.z), s);
                            s = dot2(as_bf16x2(wv[t].w), as_bf16x2(xv.w), s);
                            acc[r] = s;
                        }
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < MAXM; ++r) {
                if (r < K) {
                    const float t = wave_sum(acc[r]);
                    if (lane == 0)
                        __hip_atomic_store(reinterpret_cast<uint32_t*>(a.r.logits) + (size_t)r * E + e,
                                           __float_as_uint(t), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's logits have reached the coherent level
        __syncthreads();
        // the last router workgroup to finish raises every flag (one per
        // 2 KB, so the waiting workgroups poll many addresses, not one)
        if (wave == 0) {
            uint32_t old = 0u;
            if (lane == 0)
                old = __hip_atomic_fetch_add(a.counter + kHandoffFlagStride * kSlotRouterCount, 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
            old = (uint32_t)__builtin_amdgcn_readfirstlane((int)old);
            if (old == (uint32_t)(a.n_router - 1) && lane < kHandoffFlags)
                __hip_atomic_store(a.counter + kHandoffFlagStride * (kSlotRouterFlag + lane), 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }

    // ---- gate/up workgroups (gateup_smem_bytes layout)
    SelectSmem& sm = *reinterpret_cast<SelectSmem*>(smem);
    float* lg = reinterpret_cast<float*>(smem + (sizeof(SelectSmem) + 15) / 16 * 16);
    _Float16* xh = reinterpret_cast<_Float16*>(smem + select_smem_bytes(K, E));
    float* red = reinterpret_cast<float*>(smem + select_smem_bytes(K, E) + (size_t)K * xh_row_stride(H) * 2);
    const int n_sh = g.sgate.q ? g.Is / kTileRows : 0;
    const int n_rb = gridDim.x - a.n_router - n_sh - (DOWN ? a.n_down : 0), rb = bid - a.n_router - n_sh;
    if (DOWN && rb >= n_rb) {
        down_role<P>(a, smem, rb - n_rb);
        return;
    }
    const bool shared_blk = bid < a.n_router + n_sh;
    const int sh_tile = bid - a.n_router;
    const int nsr = I / kTileRows;
    GuRegs R;
    float gts = 0.0f, uts = 0.0f;
    if (shared_blk) {
        // shared expert tile: weights requested before x is formed
        R = gu_load(g.sgate.q, g.sgate.s, g.sup.q, g.sup.s, H, sh_tile * kTileRows);
        gts = g.sgate.ts[0];
        uts = g.sup.ts[0];
        stage_x(a.r, a.r.x_in, K, reinterpret_cast<uint16_t*>(xh), s_inv, 0, 0, true);
        convert_rows(xh, K, H, s_xsig, 0, kWaves);
        __syncthreads();
    } else {
        stage_x(a.r, a.r.x_in, K, reinterpret_cast<uint16_t*>(xh), s_inv, 0, 0, true);
        wait_flag(a.counter + kHandoffFlagStride * (kSlotRouterFlag + bid % kHandoffFlags), a.status, a.spin_limit);
        load_handoff_logits(lg, g.sel.logits, K * E);
        __syncthreads();
        select_rows_p<P>(g.sel, sm, lg, rb == 0);  // weights: only the workgroup that publishes them
        if (K < kWaves) convert_rows(xh, K, H, s_xsig, K, kWaves - K);
        else convert_rows(xh, K, H, s_xsig, 0, kWaves);
        __syncthreads();
    }
    const int items = shared_blk ? 1 : K * k * nsr;
    const int step = shared_blk ? 1 : n_rb;
    bool published = shared_blk || rb != 0;
    for (int it = shared_blk ? 0 : rb; it < items; it += step) {
        int n0, m_cnt, e = 0, off_e = 0;
        bool owner = true;
        const int* xrows = nullptr;
        if (shared_blk) {
            n0 = sh_tile * kTileRows;
            m_cnt = K;
        } else {
            const int s = it / nsr;
            e = sm.sel[s];
            n0 = (it % nsr) * kTileRows;
            // Every slot compared with e, one slot per lane (every wave
            // computes the same masks): the first slot of e, its slots in
            // ascending order (one per row that selected it), and the number
            // of slots whose expert is below e, which is where e's rows start
            // in the canonical dedup order.  h rows are written there, so the
            // down kernel reads them without the dedup lists.
            int first = -1, cnt = 0;
            for (int b = 0; b < n; b += 64) {
                const int v = (b + lane < n) ? sm.sel[b + lane] : 0x7fffffff;
                const unsigned long long meq = __ballot(v == e);
                off_e += __popcll(__ballot(v < e));
                if (v == e) s_xrows[wave][cnt + lanes_below(meq)] = (b + lane) / k;
                if (first < 0 && meq) first = b + __builtin_ctzll(meq);
                cnt += __popcll(meq);
            }
            owner = first == s;  // the item belongs to e's first slot
            if (owner) {
                const size_t eq = (size_t)e * I * (H / 2), es = (size_t)e * I * (H / 16);
                R = gu_load(g.gate.q + eq, g.gate.s + es, g.up.q + eq, g.up.s + es, H, n0);
                gts = g.gate.ts[e];
                uts = g.up.ts[e];
                m_cnt = cnt;
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                xrows = s_xrows[wave];
            }
        }
        if (!published) {
            dedup_publish(g.sel, sm);
            published = true;
        }
        if (!owner) continue;
        gu_compute(R, gts, uts, H, n0, xh, s_xsig, m_cnt, xrows, nullptr,
                   shared_blk ? g.h_sh : g.h + (size_t)off_e * I, shared_blk ? g.Is : I, red);
        __syncthreads();
    }
    if (!published) dedup_publish(g.sel, sm);
    if (DOWN) {
        // Completion: gate/up workgroup i adds one to counter i % m (m =
        // min(32, gate/up workgroups)); the one that completes a counter adds
        // one to the second level, and the one that completes that raises
        // the down workgroups' flags.  Every h store of this workgroup has
        // completed first.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (wave == 0) {
            const int n_gu = n_sh + n_rb;
            const int m = min(kHandoffFlags, n_gu);
            const int gi = bid - a.n_router;
            const int c = gi % m;
            const uint32_t expect = (uint32_t)(n_gu / m + (c < n_gu % m ? 1 : 0));
            uint32_t last = 0u;
            if (lane == 0) {
                const uint32_t o1 = __hip_atomic_fetch_add(a.counter + kHandoffFlagStride * (kSlotDoneCount + c), 1u,
                                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (o1 == expect - 1u) {
                    const uint32_t o2 = __hip_atomic_fetch_add(a.counter + kHandoffFlagStride * kSlotDoneLevel2, 1u,
                                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    last = (o2 == (uint32_t)(m - 1)) ? 1u : 0u;
                }
            }
            last = (uint32_t)__builtin_amdgcn_readfirstlane((int)last);
            if (last && lane < kHandoffFlags)
                __hip_atomic_store(a.counter + kHandoffFlagStride * (kSlotDownFlag + lane), 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// The router hand-off words (arrival counter and flags) of a set to zero
// (thread t <= kHandoffFlags clears one word).
__device__ __forceinline__ void handoff_clear(uint32_t* counter, int t) {
    if (t <= kHandoffFlags)
        __hip_atomic_store(counter + kHandoffFlagStride * t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The call's first kernel: both hand-off sets and the status word to zero.
__global__ void k_handoff_reset(uint32_t* sets, int32_t* status) {
    for (int t = threadIdx.x; t < 2 * kHandoffSlots; t += blockDim.x)
        __hip_atomic_store(sets + kHandoffFlagStride * t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) __hip_atomic_store(status, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// k_down (+ combine)
// ---------------------------------------------------------------------------

// Four down shapes by the size of the staged h chunk.  16 waves issue the
// weight loads from more waves at once: up to 32 KB of h (K = 1 at the
// 2048-hidden shape) with two tasks per wave in flight, up to 64 KB (K = 2)
// with three, up to 96 KB (K = 4) with four, so that all of a chunk's tasks
// go out in one batch with few unused slots.  Larger chunks: 8 waves with six
// tasks each, since at 16 waves the eight staging registers of h per thread
// would exceed the 128 VGPRs a wave may hold there.
constexpr int kDownThreadsBig = 512;
constexpr int kDownBatchTiny = 2;   // tasks per wave whose codes are in flight together
constexpr int kDownBatchSmall = 3;
constexpr int kDownBatchMid = 4;
constexpr int kDownBatchBig = 6;
// staging passes of one float4 per thread that cover a chunk of each shape
constexpr int kDownSuTiny = 32 * 1024 / (16 * kDownThreads);
constexpr int kDownSuSmall = 64 * 1024 / (16 * kDownThreads);
constexpr int kDownSuMid = 96 * 1024 / (16 * kDownThreads);
constexpr int kDownSuBig = kDownHLdsBytes / (16 * kDownThreadsBig);

// The h rows are processed in chunks that fit kDownHLdsBytes: positions
// 0..n-1 are the routed slots in dedup order (h row p, length I), n..n+K-1
// the shared expert's rows (length Is).
// SU: staging passes of one float4 per thread that cover one chunk of h
// (a.h_lds_bytes / 16 <= SU * NT, guaranteed by launch_down); NT threads per
// workgroup; NB tasks per wave whose loads are in flight together.
template <int SU, int NT, int NB>
__global__ __launch_bounds__(NT) void k_down(DownArgs a) {
    constexpr int NH = kDownRowsPerBlock;
    constexpr int kDownWaves = NT / 64;
    __shared__ float so[(kMaxSlots + kMaxRows) * NH];
    __shared__ int s_uniq[kMaxSlots];
    __shared__ int s_off[kMaxSlots + 1];
    __shared__ int s_inv[kMaxSlots];
    __shared__ float s_w[kMaxSlots];
    __shared__ float s_y[kMaxRows * NH];
    __shared__ int s_U;
    extern __shared__ __align__(16) float hs[];
    // wave index made visibly uniform: the task index, the expert and the
    // matrix choice below then live in scalar registers
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H, K = a.K, k = a.k, n = K * k;
    const int n_base = blockIdx.x * NH;
    // the router/gate-up launch of this layer has ended: its hand-off
    // counter starts the next layer at zero
    if (a.counter && blockIdx.x == 0) handoff_clear(a.counter, tid);
    const bool has_sh = a.sdown.q != nullptr;
    // matrix pointers read once; the per-task choice below selects values
    const uint8_t* const dq = a.down.q;
    const uint8_t* const ds = a.down.s;
    const float* const dts = a.down.ts;
    const uint8_t* const sq = a.sdown.q;
    const uint8_t* const ss = a.sdown.s;
    const float* const sts = a.sdown.ts;
    const int I = a.I, Is = a.Is;

    // Bytes the next launch reads first (the next layer's router rows),
    // requested now so that they are in the memory-side cache when it starts;
    // the value is consumed only by an empty asm statement once the routing
    // metadata below has arrived (vector loads complete in issue order, so
    // that adds no wait, and the registers are free for the rest).
    uint4 pf = make_uint4(0, 0, 0, 0);
    if (a.prefetch) {
        const int n16 = a.prefetch_bytes >> 4;
        const int i = min((int)(blockIdx.x * NT + tid), n16 - 1);
        pf = reinterpret_cast<const uint4*>(a.prefetch)[i];
    }

    // staged h rows: 4 floats of padding after every 32-column chunk, so the
    // 16 lanes of a weight row (one chunk each) do not share LDS banks
    const int RL = max(I, has_sh ? Is : 0);
    const int RLP = RL / 32 * 36;                   // padded LDS row stride
    const int CAP = (a.h_lds_bytes / 4) / RLP;      // rows per chunk
    const int total_rows = n + (has_sh ? K : 0);
    // Positions 0..n-1 are the routed rows of h in dedup order, n..n+K-1 the
    // shared expert's rows: neither needs the routing metadata, so the first
    // chunk of h is requested before it.  Up to SU passes of one float4 per
    // thread cover a whole chunk; inside a pass the loads are unconditional
    // at clamped addresses, and columns past a shorter row's length are
    // staged as zeros.
    static_assert(SU <= 16, "more than 16 staging passes of h");
    static_assert(NT >= 512, "a staged row (up to 2048 floats) must fit in one pass");
    const int q4 = RL / 4;                  // float4 per staged row (unpadded, a power of two)
    const int lq4 = __builtin_ctz(q4);
    // q4 <= NT, so a pass covers NT / q4 whole rows and this thread's row
    // offset and column are the same in every pass
    const int rpp = NT >> lq4, r0 = tid >> lq4, c4 = tid & (q4 - 1);
    float4 hv4[SU];
    auto load_h = [&](int c0, int c1) {
        const int nr = c1 - c0;
#pragma unroll
        for (int j = 0; j < SU; ++j) {
            if (j * rpp < nr) {  // uniform: passes past the chunk are skipped
                const int rr = c0 + min(j * rpp + r0, nr - 1);
                const bool shared_row = rr >= n;
                const uint32_t len4 = (uint32_t)(shared_row ? Is : I) >> 2;
                const uint32_t cc = min((uint32_t)c4, len4 - 1u);
                const float4* hb = reinterpret_cast<const float4*>(shared_row ? a.h_sh : a.h);
                hv4[j] = hb[(uint32_t)(shared_row ? rr - n : rr) * len4 + cc];
            }
        }
    };
    load_h(0, min(total_rows, CAP));

    // routing metadata: every load of a thread issued before any is used
    // (one round trip; n + 1 <= kMaxSlots + 1 <= 2 * NT)
    static_assert(kMaxSlots + 1 <= 2 * NT, "metadata exceeds two entries per thread");
    {
        const int i0 = tid, i1 = tid + NT;
        const int j0 = min(i0, n - 1), j1 = min(i1, n - 1);
        const int u0 = a.uniq[j0], u1 = a.uniq[j1];
        const int v0 = a.inv[j0], v1 = a.inv[j1];
        const float w0 = a.w[j0], w1 = a.w[j1];
        const int o0 = a.off[min(i0, n)], o1 = a.off[min(i1, n)];
        const int nu = *a.n_unique;
        if (i0 < n) { s_uniq[i0] = u0; s_inv[i0] = v0; s_w[i0] = w0; }
        if (i1 < n) { s_uniq[i1] = u1; s_inv[i1] = v1; s_w[i1] = w1; }
        if (i0 <= n) s_off[i0] = o0;
        if (i1 <= n) s_off[i1] = o1;
        if (tid == 0) s_U = nu;
    }
    asm volatile("" ::"v"(pf.x), "v"(pf.y), "v"(pf.z), "v"(pf.w));  // the prefetch stays issued
    __syncthreads();
    const int U = s_U;

    // lanes per weight row (one 32-column chunk each) and tasks per expert;
    // all powers of two, so lane and task indices split with shifts
    const int cprI = I >> 5, lgI = __builtin_ctz(cprI);
    const int gI = max(1, NH / (64 / cprI)), lgG = __builtin_ctz(gI);
    const int cprS = has_sh ? (Is >> 5) : 1, lgS = __builtin_ctz(cprS);
    const int gS = has_sh ? max(1, NH / (64 / cprS)) : 0;

    for (int c0 = 0; c0 < total_rows; c0 += CAP) {
        const int c1 = min(total_rows, c0 + CAP);
        // routed experts with slots in [c0, c1): a contiguous range of u
        int u_lo = 0, u_hi = 0;
        if (c0 == 0 && c1 >= n) {
            u_hi = U;
        } else if (c0 < n) {
            while (u_lo < U && s_off[u_lo + 1] <= c0) ++u_lo;
            u_hi = u_lo;
            while (u_hi < U && s_off[u_hi] < min(c1, n)) ++u_hi;
        }
        const bool sh_here = has_sh && c1 > n;
        const int nT = (u_hi - u_lo) * gI + (sh_here ? gS : 0);

        // codes, scales and tensor scales of this wave's first batch of tasks
        uint4 code[NB];
        uint32_t scl[NB];
        float tsv[NB];
        // every expert id of a batch is read from LDS before any of its
        // global loads is issued: one LDS wait per batch
        int ev[NB];
        auto batch_ids = [&](int tb) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int t = (tb * NB + i) * kDownWaves + wave;
                ev[i] = (t < (u_hi - u_lo) * gI) ? s_uniq[u_lo + (t >> lgG)] : 0;
            }
        };
        auto load_batch = [&](int tb) {
            // Loads are issued unconditionally (the counter of outstanding
            // loads then stays known to the compiler): a task past the end
            // reads row n_base of routed expert 0 and a lane past the
            // workgroup's rows reads row n_base; neither result is stored.
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int t = (tb * NB + i) * kDownWaves + wave;
                const bool routed = t < (u_hi - u_lo) * gI;
                const bool shared_task = !routed && t < nT;
                const int lgC = shared_task ? lgS : lgI;
                const int grp = routed ? (t & (gI - 1)) : (shared_task ? t - (u_hi - u_lo) * gI : 0);
                // the expert is the same in every lane: the task's first row
                // address is formed in scalar registers, and each lane adds
                // a 32-bit offset
                const int e = __builtin_amdgcn_readfirstlane(ev[i]);
                const uint8_t* mq = shared_task ? sq : dq;
                const uint8_t* ms = shared_task ? ss : ds;
                const float* mts = shared_task ? sts : dts;
                const uint32_t cols = (uint32_t)(shared_task ? Is : I);
                const int q = lane >> lgC, chunk = lane & ((1 << lgC) - 1);
                const int nl = (grp << (6 - lgC)) + q;
                const uint32_t lr = (uint32_t)(nl < NH ? nl : 0);
                const size_t row0 = (size_t)e * H + n_base;
                tsv[i] = mts[e];
                code[i] = *reinterpret_cast<const uint4*>(mq + row0 * (cols >> 1) + (lr * (cols >> 1) + (uint32_t)chunk * 16u));
                scl[i] = *reinterpret_cast<const uint16_t*>(ms + row0 * (cols >> 4) + (lr * (cols >> 4) + (uint32_t)chunk * 2u));
            }
        };
        // A later chunk of h (more than CAP rows) is requested here, after
        // the previous chunk's closing barrier; this chunk's weight loads go
        // out before its h is written to LDS.
        if (c0 > 0) load_h(c0, c1);
        batch_ids(0);
        load_batch(0);
        {
            // one LDS address per thread, advanced by a uniform stride per pass
            float* dst = hs + r0 * RLP + (c4 >> 3) * 36 + (c4 & 7) * 4;
#pragma unroll
            for (int j = 0; j < SU; ++j) {
                const int rr = j * rpp + r0;
                if (rr < c1 - c0) {
                    const int len4 = ((c0 + rr) >= n ? Is : I) / 4;
                    *reinterpret_cast<float4*>(dst + j * rpp * RLP) = c4 < len4 ? hv4[j] : make_float4(0, 0, 0, 0);
                }
            }
        }
        __syncthreads();  // staged h visible to every wave

        for (int tb = 0; tb * kDownWaves * NB < nT; ++tb) {
            if (tb > 0) {
                batch_ids(tb);
                load_batch(tb);
            }
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int t = (tb * NB + i) * kDownWaves + wave;
                if (t >= nT) break;
                const bool routed = t < (u_hi - u_lo) * gI;
                const int lgC = routed ? lgI : lgS, CPR = 1 << lgC;
                const int grp = routed ? (t & (gI - 1)) : t - (u_hi - u_lo) * gI;
                const int u = u_lo + (routed ? (t >> lgG) : 0);
                const float ts = tsv[i];
                int p_lo, p_hi;
                if (routed) { p_lo = max(s_off[u], c0); p_hi = min(s_off[u + 1], c1); }
                else { p_lo = max(n, c0); p_hi = c1; }
                const int q = lane >> lgC, chunk = lane & (CPR - 1);
                const int nl = (grp << (6 - lgC)) + q;
                float wf[32];
                fp4x8_to_f32(code[i].x, wf + 0); fp4x8_to_f32(code[i].y, wf + 8);
                fp4x8_to_f32(code[i].z, wf + 16); fp4x8_to_f32(code[i].w, wf + 24);
                const float s0 = e4m3_to_f32<0>(scl[i]), s1 = e4m3_to_f32<1>(scl[i]);
                for (int pp = p_lo; pp < p_hi; ++pp) {
                    const float4* hp = reinterpret_cast<const float4*>(hs + (size_t)(pp - c0) * RLP + chunk * 36);
                    // four independent chains of eight products
                    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int t4 = 0; t4 < 8; ++t4) {
                        const float4 hv = hp[t4];
                        float& c = acc[t4 >> 1];
                        c = fmaf(wf[4 * t4 + 0], hv.x, c);
                        c = fmaf(wf[4 * t4 + 1], hv.y, c);
                        c = fmaf(wf[4 * t4 + 2], hv.z, c);
                        c = fmaf(wf[4 * t4 + 3], hv.w, c);
                    }
                    float p = fmaf(acc[2] + acc[3], s1, (acc[0] + acc[1]) * s0);
                    p = (CPR == 16) ? group_sum<16>(p) : group_sum_rt(p, CPR);
                    if (nl < NH && chunk == CPR - 1) so[pp * NH + nl] = p * ts;
                }
            }
        }
        __syncthreads();  // chunk done before its LDS rows are replaced
    }

    // combine: y = rs * sum_j w_j o_j (rank order) + shared (+ residual)
    for (int i = tid; i < K * NH; i += NT) {
        const int r = i / NH, nl = i % NH, nn = n_base + nl;
        float acc = 0.0f;
        for (int j = 0; j < k; ++j) acc = fmaf(s_w[r * k + j], so[s_inv[r * k + j] * NH + nl], acc);
        float y = a.rs * acc;
        if (has_sh) y += so[(n + r) * NH + nl];
        if (a.residual) y += bf16_to_f32(a.residual[(size_t)r * H + nn]);
        a.y32[(size_t)r * H + nn] = y;
        if (a.y) a.y[(size_t)r * H + nn] = f32_to_bf16_rne(y);
        s_y[i] = y;
    }
    __syncthreads();
    // per-row partial sum of squares of this workgroup's columns (fixed order)
    if (a.ssq && tid < K) {
        float ss = 0.0f;
        for (int nl = 0; nl < NH; ++nl) ss = fmaf(s_y[tid * NH + nl], s_y[tid * NH + nl], ss);
        a.ssq[tid * gridDim.x + blockIdx.x] = ss;
    }
}

// ---------------------------------------------------------------------------
// k_dequant: the decodes of the GEMM kernels, written out.  Three routes
// reach e2m1(code) * e4m3(scale): the fp32 convert then an fp32 multiply
// (the down kernels' weights), the bf16 convert, and the fp16 operand
// decode of the gate/up matrix-core tiles (decode8_f16: fp16 convert, then
// a packed fp16 multiply by the fp16 scale).  A disagreement between them
// is reported as NaN; the product is then multiplied by the tensor scale in
// fp32.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kBlock) void k_dequant(Fp4Mat m, int n_experts, int rows, int cols, float* out) {
    const size_t chunks_per_row = (size_t)cols / 32;
    const size_t total = (size_t)n_experts * rows * chunks_per_row;
    for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < total; i += (size_t)gridDim.x * kBlock) {
        const size_t row = i / chunks_per_row;  // e * rows + n
        const int chunk = (int)(i % chunks_per_row);
        const int e = (int)(row / rows);
        const uint4 c = *reinterpret_cast<const uint4*>(m.q + row * (cols / 2) + chunk * 16);
        const uint32_t sc = *reinterpret_cast<const uint16_t*>(m.s + row * (cols / 16) + chunk * 2);
        float wf[32];
        bf16x2_t wb[16];
        fp4x8_to_f32(c.x, wf + 0); fp4x8_to_f32(c.y, wf + 8);
        fp4x8_to_f32(c.z, wf + 16); fp4x8_to_f32(c.w, wf + 24);
        fp4x8_to_bf16(c.x, wb + 0); fp4x8_to_bf16(c.y, wb + 4);
        fp4x8_to_bf16(c.z, wb + 8); fp4x8_to_bf16(c.w, wb + 12);
        const _Float16 h0 = e4m3_to_f16<0>(sc), h1 = e4m3_to_f16<1>(sc);
        const f16x8_t d0 = decode8_f16(c.x, h0), d1 = decode8_f16(c.y, h0);
        const f16x8_t d2 = decode8_f16(c.z, h1), d3 = decode8_f16(c.w, h1);
        const float s0 = e4m3_to_f32<0>(sc), s1 = e4m3_to_f32<1>(sc);
        const float ts = m.ts[e];
        float* o = out + row * cols + chunk * 32;
#pragma unroll
        for (int t = 0; t < 32; ++t) {
            const float fb = (float)((t & 1) ? wb[t >> 1].y : wb[t >> 1].x);
            const f16x8_t& d = (t < 8) ? d0 : (t < 16) ? d1 : (t < 24) ? d2 : d3;
            const float prod = wf[t] * (t < 16 ? s0 : s1);
            const bool agree = fb == wf[t] && (float)d[t & 7] == prod;
            o[t] = (agree ? prod : __builtin_nanf("")) * ts;
        }
    }
}

// ---------------------------------------------------------------------------
// k_stream_read: a plain streaming read of n16 16-byte pieces (the measured
// read ceiling next to the benchmark's figures).  Each workgroup reads its
// own contiguous range, the workgroup's threads side by side, 8 loads per
// thread in flight, marked non-temporal: of the patterns measured on the
// chip (grid-strided or contiguous ranges, plain or non-temporal loads),
// this one reads fastest.  A lane stores its XOR of what it read to *sink
// only when that equals a fixed constant, so the loads cannot be dropped
// (one same-address atomic per workgroup instead measured 10% slower: the
// atomics serialise).
// ---------------------------------------------------------------------------

constexpr uint32_t kStreamSinkMark = 0x9E3779B9u;

__global__ __launch_bounds__(kBlock) void k_stream_read(const uint4* __restrict__ p, size_t n16, uint32_t* sink) {
    constexpr int U = 8;
    const size_t lo = n16 * blockIdx.x / gridDim.x, hi = n16 * (blockIdx.x + 1) / gridDim.x;
    uint32_t acc = 0u;
    size_t i = lo + threadIdx.x;
    for (; i + (U - 1) * kBlock < hi; i += U * kBlock) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = ld16_nt(p + i + u * kBlock);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < hi; i += kBlock) {
        const uint4 v = ld16_nt(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == kStreamSinkMark) *sink = acc;
}

hipError_t launch_stream_read(const void* src, size_t n16, uint32_t* sink, hipStream_t st) {
    int dev = 0, n_cu = 0;
    hipError_t e;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    hipLaunchKernelGGL(k_stream_read, dim3(n_cu * 8), dim3(kBlock), 0, st, reinterpret_cast<const uint4*>(src), n16,
                       sink);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

int gateup_slab_rows(int) { return kTileRows; }

bool lds_fits(int K, int E, int H) {
    const size_t router = (size_t)K * H * 2;
    return gateup_smem_bytes(K, E, H) <= (size_t)kRgMaxDynLds && router <= (size_t)kRgMaxDynLds &&
           select_smem_bytes(K, E) <= (size_t)kMaxDynLds;
}

// Plain launch, or one whose start/stop events carry the kernel's own
// dispatch timestamps.
template <typename Kern, typename Args>
hipError_t launch(Kern k, dim3 grid, dim3 block, size_t smem, hipStream_t st, const Timing* t, const Args& a) {
    if (t)
        hipExtLaunchKernelGGL(k, grid, block, smem, st, t->start, t->stop, 0, a);
    else
        hipLaunchKernelGGL(k, grid, block, smem, st, a);
    return hipGetLastError();
}

// Dynamic LDS above the default per-launch limit: the selection stages
// K*E logits (up to 64 KiB) next to its fixed tables; the down kernel stages
// 64 KiB of h next to its static tables.

template <typename Kern>
hipError_t set_lds(Kern k, int bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

hipError_t init_kernels() {
    static hipError_t once = [] {
        hipError_t e;
        if ((e = set_lds(k_select, kMaxDynLds)) != hipSuccess) return e;
#define MOE_SET_RG(P)                                                                          \
        if ((e = set_lds(k_route_gateup<P, 2, false>, kRgMaxDynLds)) != hipSuccess) return e;     \
        if ((e = set_lds(k_route_gateup<P, 4, false>, kRgMaxDynLds)) != hipSuccess) return e;     \
        if ((e = set_lds(k_route_gateup<P, kMaxRows, false>, kRgMaxDynLds)) != hipSuccess) return e;
        MOE_SET_RG(1) MOE_SET_RG(2) MOE_SET_RG(4) MOE_SET_RG(8) MOE_SET_RG(16)
#undef MOE_SET_RG
        if ((e = set_lds(k_route_gateup<1, 2, true>, kRgMaxDynLds)) != hipSuccess) return e;
        if ((e = set_lds(k_route_gateup<2, 2, true>, kRgMaxDynLds)) != hipSuccess) return e;
        if ((e = set_lds(k_route_gateup<4, 2, true>, kRgMaxDynLds)) != hipSuccess) return e;
        if ((e = set_lds(k_down<kDownSuSmall, kDownThreads, kDownBatchSmall>, kDownHLdsBytes)) != hipSuccess)
            return e;
        if ((e = set_lds(k_down<kDownSuBig, kDownThreadsBig, kDownBatchBig>, kDownHLdsBytes)) != hipSuccess)
            return e;
        if ((e = set_lds(k_down<kDownSuMid, kDownThreads, kDownBatchMid>, kDownHLdsBytes)) != hipSuccess)
            return e;
        if ((e = set_lds(k_down<kDownSuTiny, kDownThreads, kDownBatchTiny>, kDownHLdsBytes)) != hipSuccess)
            return e;
        return init_grouped_kernels();
    }();
    return once;
}

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
    return launch(k_select, dim3(1), dim3(kBlock), select_smem_bytes(a.K, a.E), st, nullptr, a);
}

// The fused router + gate/up launch: n_router router workgroups, the
// shared expert's tiles, then routed workgroups, one per work item (slot,
// 16 intermediate rows) but no more than fit on the chip at once next to
// the others (the rest loop over items): a second dispatch round would
// repeat the selection after the first round's weights have streamed, and
// a waiting workgroup must never keep a router workgroup from starting.
template <typename Kern>
hipError_t launch_route_gateup_k(Kern k, const RouteGateUpArgs& a, hipStream_t st, const Timing* t) {
    size_t smem = gateup_smem_bytes(a.g.K, a.g.sel.E, a.g.H);
    if (a.n_down > 0) {
        const size_t dn = fused_down_lds_bytes(a.g.K, a.g.sel.k, a.g.sel.E, a.g.I, a.g.sgate.q ? a.g.Is : 0);
        if (dn > smem) smem = dn;
    }
    const int n_sh = a.g.sgate.q ? a.g.Is / kTileRows : 0;
    int grid = a.g.K * a.g.sel.k * (a.g.I / kTileRows);
    if (grid > kGateUpMaxGrid) grid = kGateUpMaxGrid;
    int dev = 0, n_cu = 0, per_cu = 0;
    hipError_t e;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kBlock, smem)) != hipSuccess) return e;
    const int fit = per_cu * n_cu - n_sh - a.n_router - a.n_down;
    if (fit >= 1 && grid > fit) grid = fit;
    return launch(k, dim3(a.n_router + n_sh + grid + a.n_down), dim3(kBlock), smem, st, t, a);
}

template <int P>
hipError_t launch_route_gateup_p(const RouteGateUpArgs& a, hipStream_t st, const Timing* t) {
    if (a.n_down > 0) {
        if constexpr (P <= kFusedMaxP) {
            if (a.g.K > 2) return hipErrorInvalidValue;
            return launch_route_gateup_k(k_route_gateup<P, 2, true>, a, st, t);
        } else {
            return hipErrorInvalidValue;
        }
    }
    if (a.g.K <= 2) return launch_route_gateup_k(k_route_gateup<P, 2, false>, a, st, t);
    if (a.g.K <= 4) return launch_route_gateup_k(k_route_gateup<P, 4, false>, a, st, t);
    return launch_route_gateup_k(k_route_gateup<P, kMaxRows, false>, a, st, t);
}

hipError_t launch_route_gateup(const RouteGateUpArgs& a, hipStream_t st, const Timing* t) {
    const int P = (a.g.sel.E + 63) >> 6;  // experts per lane of the top-k
    if (P <= 1) return launch_route_gateup_p<1>(a, st, t);
    if (P <= 2) return launch_route_gateup_p<2>(a, st, t);
    if (P <= 4) return launch_route_gateup_p<4>(a, st, t);
    if (P <= 8) return launch_route_gateup_p<8>(a, st, t);
    return launch_route_gateup_p<16>(a, st, t);
}

// Whether the down projection can run as the third workgroup group of the
// router + gate/up launch: at most two rows, every down task of a workgroup
// (one per h row and row group) held in registers (kFusedDownTasks per
// wave), the h rows and the routing
// lists within the launch's LDS, and H / kDownRowsPerBlock down workgroups
// resident next to the others; up to 256 experts (wider top-k lanes would
// push the launch past 128 registers per lane) and a shared expert, if any,
// as wide as a routed one.
bool fused_down_fits(int K, int k, int E, int H, int I, int Is) {
    if (K > 2 || (E + 63) / 64 > kFusedMaxP || (Is > 0 && Is != I)) return false;
    const int NH = kDownRowsPerBlock;
    const int cpr = I / 32, gI = (NH / (64 / cpr)) > 1 ? NH / (64 / cpr) : 1;
    if ((K * k + (Is > 0 ? K : 0)) * gI > kWaves * kFusedDownTasks) return false;
    const size_t lds = fused_down_lds_bytes(K, k, E, I, Is);
    if (lds > (size_t)kRgMaxDynLds) return false;
    return true;
}

hipError_t launch_handoff_reset(uint32_t* sets, int32_t* status, hipStream_t st) {
    hipLaunchKernelGGL(k_handoff_reset, dim3(1), dim3(kBlock), 0, st, sets, status);
    return hipGetLastError();
}

hipError_t launch_down(const DownArgs& a, hipStream_t st, const Timing* t) {
    // LDS for the h rows one launch stages (all of them when they fit in
    // kDownHLdsBytes, else chunks of that size): padded rows of max(I, Is)
    // floats, 36 per 32 columns
    const int n_rows = a.K * a.k + (a.sdown.q ? a.K : 0);
    const int RL = a.I > a.Is ? a.I : a.Is;
    const long long need = (long long)n_rows * (RL / 32 * 36) * 4;
    DownArgs b = a;
    b.h_lds_bytes = (int)(need < kDownHLdsBytes ? need : kDownHLdsBytes);
    const dim3 g(a.H / kDownRowsPerBlock);
    if (b.h_lds_bytes <= kDownSuTiny * kDownThreads * 16)
        return launch(k_down<kDownSuTiny, kDownThreads, kDownBatchTiny>, g, dim3(kDownThreads),
                      (size_t)b.h_lds_bytes, st, t, b);
    if (b.h_lds_bytes <= kDownSuSmall * kDownThreads * 16)
        return launch(k_down<kDownSuSmall, kDownThreads, kDownBatchSmall>, g, dim3(kDownThreads),
                      (size_t)b.h_lds_bytes, st, t, b);
    if (b.h_lds_bytes <= kDownSuMid * kDownThreads * 16)
        return launch(k_down<kDownSuMid, kDownThreads, kDownBatchMid>, g, dim3(kDownThreads),
                      (size_t)b.h_lds_bytes, st, t, b);
    return launch(k_down<kDownSuBig, kDownThreadsBig, kDownBatchBig>, g, dim3(kDownThreadsBig),
                  (size_t)b.h_lds_bytes, st, t, b);
}

hipError_t launch_dequant(Fp4Mat m, int n_experts, int rows, int cols, float* out, hipStream_t st) {
    const size_t total = (size_t)n_experts * rows * (cols / 32);
    size_t grid = (total + kBlock - 1) / kBlock;
    if (grid > 65536) grid = 65536;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(k_dequant, dim3((unsigned)grid), dim3(kBlock), 0, st, m, n_experts, rows, cols, out);
    return hipGetLastError();
}

}  // namespace moe
