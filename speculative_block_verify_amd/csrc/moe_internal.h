// Internal interface between the C ABI (moe_abi.hip) and the gfx950 kernels
// (moe_kernels.hip).  Not installed; the public surface is include/moe_verify.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Compile-time limits of the skinny (verify-width) path.
constexpr int kMaxRows = 16;       // K
constexpr int kMaxTopK = 32;       // k
constexpr int kMaxExperts = 1024;  // E
constexpr int kMaxSlots = kMaxRows * kMaxTopK;
constexpr int kBlock = 256;        // threads per workgroup (4 wave64)
constexpr int kWaves = kBlock / 64;
constexpr int kDownRowsPerBlock = 8;
constexpr int kDownThreads = 1024;  // 16 wave64 per down workgroup
constexpr int kDownHLdsBytes = 128 * 1024;  // most h rows staged in LDS per chunk (one down workgroup per compute unit)
constexpr int kGateUpMaxGrid = 1024;       // routed gate/up workgroups loop over work items
constexpr int kMetaUnique = 0;             // workspace word holding the unique-expert count
constexpr int kMetaTiles = 1;              // workspace word holding the grouped tile count

// Limits of the grouped (prefill) regime, used for K > kMaxRows rows.
constexpr int kMaxGroupedRows = 1024;      // T
constexpr int kGChunk = 32;                // tokens per grouped tile
constexpr int kGRows = 64;                 // weight rows per grouped workgroup (4 waves x 16)
constexpr int kGMaxCols = 1024;            // largest intermediate size the grouped down kernel stages
constexpr int kGGroupThreads = 1024;       // the grouping workgroup
constexpr int kGMaxGrid = 4096;            // grouped GEMM workgroups loop over work items beyond this

struct Fp4Mat {
    const uint8_t* q;
    const uint8_t* s;
    const float* ts;
};

// Inputs and outputs of the selection step (top-k + dedup).
struct SelectArgs {
    const float* logits;    // [K][E]
    const float* bias;      // [E] or nullptr
    int32_t* ids;           // [K][k]
    float* w;               // [K][k]
    int32_t* n_unique;      // [1]
    int32_t* uniq;          // [K*k]
    int32_t* off;           // [K*k+1]
    int32_t* asg;           // [K*k]
    int32_t* inv;           // [K*k]
    int K, E, k, score_fn, norm_topk;
};

// Router GEMV (and the RMS normalisation of the previous layer's output).
// The many-row router's column slices: one wave each, its partial logits
// added in slice order.  Up to kRouterSplitMaxRows rows each slice is a
// workgroup of its own (more workgroups for few rows), for up to
// kRouterSplitMaxExperts experts.
constexpr int kRouterWaves = 8;
constexpr int kRouterSplitMaxRows = 16;
constexpr int kRouterSplitMaxExperts = 256;

// Selection for the few-row grouped layer: the router's per-slice partial
// logits are added here (slice order), and the fp16 copy of x is made here.
struct SelectSplitArgs {
    SelectArgs s;           // s.logits unused
    const float* parts;     // [kRouterWaves][K][E] partial logits, one per column slice
    float* logits;          // [K][E] their sums (written)
    const uint16_t* x_in;   // bf16 [K][H]
    uint16_t* x_f16;        // fp16 bit patterns [K][H] of x_in * 2^-x_sig[row]
    int32_t* x_sig;         // [K]
    int H;
};
struct RouterArgs {
    const uint16_t* x_in;   // bf16 [K][H], read when y_prev == nullptr
    const float* y_prev;    // fp32 [K][H] to RMS-normalise into x, or nullptr
    const float* ssq;       // [K][H / kDownRowsPerBlock] partial sums of squares of y_prev
    const uint16_t* gamma;  // bf16 [H] norm weight applied to the normalised y_prev, or nullptr (ones)
    uint16_t* x_out;        // bf16 [K][H] normalised x (written when y_prev != nullptr)
    float eps;
    const uint16_t* wr;     // bf16 [E][H]
    float* logits;          // [K][E]
    uint16_t* x_f16;        // fp16 bit patterns [K][H] of x_in * 2^-x_sig[row], or nullptr (many-row router only)
    int32_t* x_sig;         // [K] per-row power-of-two exponent of that copy (with x_f16)
    int K, H, E;
};

// Gate/up + SwiGLU: the shared expert's tiles, then the routed work items;
// every routed workgroup recomputes the selection.
struct GateUpArgs {
    SelectArgs sel;         // its outputs are written by the first routed workgroup only
    const uint16_t* x;      // bf16 [K][H]
    Fp4Mat gate, up;        // [E][I][H/2]
    float* h;               // [K*k][I], rows by position in the canonical dedup order
    Fp4Mat sgate, sup;      // [1][Is][H/2] (q == nullptr: no shared expert)
    float* h_sh;            // [K][Is]
    int K, H, I, Is;
};

struct DownArgs {
    Fp4Mat down;            // [E][H][I/2]
    Fp4Mat sdown;           // [1][H][Is/2]
    const int32_t* n_unique;
    const int32_t* uniq;
    const int32_t* off;
    const int32_t* inv;
    const float* w;         // [K][k]
    const float* h;         // [K*k][I], rows by dedup position
    const float* h_sh;
    const uint16_t* residual;  // bf16 [K][H] or nullptr
    float* y32;             // [K][H]
    uint16_t* y;            // bf16 [K][H] or nullptr
    float* ssq;             // [K][H / kDownRowsPerBlock] per-workgroup sums of y^2
    const uint8_t* prefetch;   // bytes the next launch reads first (the next layer's router), or nullptr
    int prefetch_bytes;        // multiple of 16
    int h_lds_bytes;           // dynamic LDS of the launch: h rows staged per chunk (set by launch_down)
    uint32_t* counter;         // the router/gate-up hand-off counter to reset, or nullptr
    int K, H, I, Is, k;
    float rs;
};

// Hand-off words of one layer launch, each kHandoffFlagStride words apart
// (slot i at counter[kHandoffFlagStride * i]): the router arrival counter,
// the flags it raises, the gate/up completion counters, their second-level
// counter and the flags that releases.
constexpr int kHandoffFlags = 32;          // flags per fan-out
constexpr int kHandoffFlagStride = 512;    // words between two hand-off slots (2 KB)
constexpr int kSlotRouterCount = 0;
constexpr int kSlotRouterFlag = 1;                                   // + f, f < kHandoffFlags
constexpr int kSlotDoneCount = kSlotRouterFlag + kHandoffFlags;      // + c, c < kHandoffFlags
constexpr int kSlotDoneLevel2 = kSlotDoneCount + kHandoffFlags;
constexpr int kSlotDownFlag = kSlotDoneLevel2 + 1;                   // + f, f < kHandoffFlags
constexpr int kHandoffSlots = kSlotDownFlag + kHandoffFlags;
constexpr int kHandoffSetWords = kHandoffSlots * kHandoffFlagStride;  // one set; the workspace holds two
constexpr int kFusedDownTasks = 9;         // down tasks per wave whose weights one down workgroup holds

// Router + gate/up in one launch (k_route_gateup), optionally with the down
// projection and combine as a third group of workgroups (n_down > 0).
struct RouteGateUpArgs {
    RouterArgs r;           // router rows, x_in or y_prev/ssq/gamma, logits (written), x_out
    GateUpArgs g;           // selection + gate/up; g.x is not read (x is formed from r)
    DownArgs d;             // with n_down > 0: down + combine (its routing metadata and counter are not read)
    uint32_t* counter;      // this launch's hand-off set, zero at launch
    uint32_t* clear;        // a set to zero for the next launch (n_down > 0), or nullptr
    int32_t* status;        // set to 1 when a bounded wait gives up
    int n_router;           // router workgroups (E / 4, rounded up)
    int n_down;             // down workgroups (H / kDownRowsPerBlock), or 0
    int spin_limit;         // polls of a bounded wait
};

// --- grouped (prefill) regime ----------------------------------------------
// Tile list: int4 {e, p0, cnt, 0}.  Routed tiles first, experts ascending
// (e = the expert, p0 = the first asg position of up to kGChunk consecutive
// slots of e, cnt = their number), then the shared expert's tiles (e = -1,
// p0 = first token, cnt = tokens).  Word kMetaTiles of the workspace meta
// holds the total count.

struct GroupArgs {
    const int32_t* ids;     // [T][k]
    int32_t* n_unique;      // [1]
    int32_t* uniq;          // [T*k]
    int32_t* off;           // [T*k+1]
    int32_t* asg;           // [T*k]
    int32_t* inv;           // [T*k]
    int32_t* tiles;         // int4 [max tiles]
    int32_t* n_tiles;       // [1]
    int32_t* status;        // the call's hand-off status word, set to 0 (no hand-off here), or nullptr
    int T, E, k;
    int has_shared;
};

struct GroupedGuArgs {
    const uint16_t* x;      // fp16 bit patterns [T][H] of x * 2^-x_sig (the router's copy of the layer input)
    const int32_t* x_sig;   // [T] the row's power-of-two exponent
    Fp4Mat gate, up;        // [E][I][H/2]
    Fp4Mat sgate, sup;      // [1][Is][H/2] (q == nullptr: no shared expert)
    const int32_t* ids;     // [T][k] the rows' selected experts
    // The canonical CSR and tile list, which every workgroup rebuilds from
    // ids in LDS and publishes for the down and combine kernels: workgroup 0
    // the per-expert outputs, the workgroup of each routed tile's first slab
    // that tile's asg / inv entries.
    int32_t* n_unique;      // [1]
    int32_t* uniq;          // [T*k]
    int32_t* off;           // [T*k+1]
    int32_t* asg;           // [T*k]
    int32_t* inv;           // [T*k]
    int32_t* tiles;         // int4 [max tiles]
    int32_t* n_tiles;       // [1]
    int32_t* status;        // the call's hand-off status word, set to 0 (no hand-off here), or nullptr
    float* h;               // [T*k][I] by asg position
    float* h_sh;            // [T][Is]
    int T, H, I, Is, k, E;
};

struct GroupedDownArgs {
    Fp4Mat down;            // [E][H][I/2]
    Fp4Mat sdown;           // [1][H][Is/2]
    const int32_t* uniq;
    const int32_t* off;
    const int32_t* tiles;
    const int32_t* n_tiles;
    const int32_t* asg;     // [T*k] slot of each CSR position
    const float* h;
    const float* h_sh;
    float* o;               // [T*k + T][H]: the routed rows by slot (r*k + j), then the shared rows by token
    int T, H, I, Is, k;
};

struct CombineArgs {
    const float* o;         // as GroupedDownArgs::o
    const float* w;         // [T][k]
    const uint16_t* residual;  // bf16 [T][H] or nullptr
    float* y32;             // [T][H]
    uint16_t* y;            // bf16 [T][H] or nullptr
    uint16_t* x_next;       // bf16 RMS-normalised y for the next layer, or nullptr
    const uint16_t* gamma;  // bf16 [H] norm weight of x_next, or nullptr (ones)
    float eps, rs;
    int T, H, k, has_shared;
};

// Optional kernel timing: start/stop events stamped from the kernel's own
// dispatch (hipExtLaunchKernelGGL); nullptr = plain launch.
struct Timing {
    hipEvent_t start;
    hipEvent_t stop;
};

// Launchers (moe_kernels.hip).  Each returns the hipError_t of the launch.
hipError_t launch_select(const SelectArgs& a, hipStream_t st);  // logits given
hipError_t launch_down(const DownArgs& a, hipStream_t st, const Timing* t = nullptr);
hipError_t launch_route_gateup(const RouteGateUpArgs& a, hipStream_t st, const Timing* t = nullptr);
hipError_t launch_handoff_reset(uint32_t* sets, int32_t* status, hipStream_t st);  // both sets
bool fused_down_fits(int K, int k, int E, int H, int I, int Is);  // the down role in the router + gate/up launch
constexpr int kMetaStatus = 3;             // workspace word: nonzero after a bounded wait gave up
constexpr int kRouteSpinLimit = 1 << 22;   // polls (with a short sleep each) before a wait gives up
hipError_t launch_dequant(Fp4Mat m, int n_experts, int rows, int cols, float* out, hipStream_t st);
hipError_t launch_stream_read(const void* src, size_t n16, uint32_t* sink, hipStream_t st);

// Sliding-window KV ring (kv_ring.hip).
struct KvArgs {
    uint16_t* k;                // bf16 [L][n_kv][C][D]
    uint16_t* v;
    int32_t* len;               // device [1]: committed length
    const uint16_t* k_new;      // bf16 [L][K][n_kv][D] (write: layers layer .. layer + L - 1)
    const uint16_t* v_new;
    const int32_t* n_accepted;  // device [1] (commit)
    uint16_t* k_out;            // bf16 [K][n_kv][W][D] (window)
    uint16_t* v_out;
    int L, n_kv, D, W, C, K, layer, len0;  // L: layers written by a write (the ring's count otherwise)
};
hipError_t launch_kv_write(const KvArgs& a, hipStream_t st);
hipError_t launch_kv_commit(const KvArgs& a, hipStream_t st);
hipError_t launch_kv_reset(const KvArgs& a, hipStream_t st);
hipError_t launch_kv_window(const KvArgs& a, hipStream_t st);

// Dense first layer (dense.hip).
bool dense_shape_ok(int H, int I);
size_t dense_workspace_bytes(int H, int I, int T);
hipError_t launch_dense_mlp(const uint16_t* x, int T, int H, int I, const uint16_t* wg, const uint16_t* wu,
                            const uint16_t* wd, const uint16_t* residual, const uint16_t* gamma, float eps, float* y32,
                            uint16_t* y, uint16_t* x_next, void* workspace, hipStream_t st);

// Grouped regime (moe_grouped.hip).
hipError_t launch_router_mfma(const RouterArgs& a, hipStream_t st);  // many rows, plain bf16 x_in only
hipError_t launch_select_rows(const SelectArgs& a, hipStream_t st);  // ids and w only
// few rows (K <= kRouterSplitMaxRows): partial logits per column slice into
// a.logits ([kRouterWaves][K][E]), no fp16 copy of x
hipError_t launch_router_split(const RouterArgs& a, hipStream_t st);
hipError_t launch_select_rows_split(const SelectSplitArgs& a, hipStream_t st);
hipError_t launch_group(const GroupArgs& a, hipStream_t st);
// hmax [T*k][I/64] and hmax_sh [T][Is/64]: max |h| of each token per 64-row slab
hipError_t launch_gateup_grouped(const GroupedGuArgs& a, float* hmax, float* hmax_sh, int max_tiles,
                                 hipStream_t st);
hipError_t launch_down_grouped(const GroupedDownArgs& a, const float* hmax, const float* hmax_sh, int max_tiles,
                               hipStream_t st);
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);
hipError_t init_grouped_kernels();
int grouped_max_tiles(int T, int E, int k, bool has_shared);
bool grouped_lds_fits(int T, int E, int I, int Is);

// Verify-row lm_head + greedy acceptance (lm_head.hip).  workspace: at
// least lm_head_workspace_bytes(V, K) bytes, 16-byte aligned.
hipError_t launch_lm_head_greedy(const uint16_t* x, int K, const uint16_t* w, int V, int H, const int32_t* draft,
                                 float tie_tol, float* logits, int32_t* target, float* target_logit,
                                 int32_t* n_accepted, int32_t* emitted, int32_t* n_emitted, void* workspace,
                                 hipStream_t st);
size_t lm_head_workspace_bytes(int V, int K);
constexpr int kLmHeadMaxRows = 16;

// One-time kernel attributes (dynamic LDS sizes).
hipError_t init_kernels();

// Rows of gate (and of up) one gate/up work item covers at hidden H.
int gateup_slab_rows(int H);

// Whether the per-workgroup LDS the kernels need at (K, E, H) fits gfx950.
bool lds_fits(int K, int E, int H);

}  // namespace moe
