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
constexpr int kDownThreads = 512;  // 8 wave64 per down workgroup
constexpr int kDownHLdsBytes = 64 * 1024;  // h rows staged in LDS per chunk
constexpr int kGateUpMaxGrid = 1024;       // routed gate/up workgroups loop over work items
constexpr int kMetaUnique = 0;             // workspace word holding the unique-expert count

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
struct RouterArgs {
    const uint16_t* x_in;   // bf16 [K][H], read when y_prev == nullptr
    const float* y_prev;    // fp32 [K][H] to RMS-normalise into x, or nullptr
    const float* ssq;       // [K][H / kDownRowsPerBlock] partial sums of squares of y_prev
    uint16_t* x_out;        // bf16 [K][H] normalised x (written when y_prev != nullptr)
    float eps;
    const uint16_t* wr;     // bf16 [E][H]
    float* logits;          // [K][E]
    int K, H, E;
};

// Gate/up + SwiGLU: the shared expert's tiles, then the routed work items;
// every routed workgroup recomputes the selection.
struct GateUpArgs {
    SelectArgs sel;         // its outputs are written by the first routed workgroup only
    const uint16_t* x;      // bf16 [K][H]
    Fp4Mat gate, up;        // [E][I][H/2]
    float* h;               // [K*k][I], indexed by position in asg
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
    const float* h;
    const float* h_sh;
    const uint16_t* residual;  // bf16 [K][H] or nullptr
    float* y32;             // [K][H]
    uint16_t* y;            // bf16 [K][H] or nullptr
    float* ssq;             // [K][H / kDownRowsPerBlock] per-workgroup sums of y^2
    int K, H, I, Is, k;
    float rs;
};

// Optional kernel timing: start/stop events stamped from the kernel's own
// dispatch (hipExtLaunchKernelGGL); nullptr = plain launch.
struct Timing {
    hipEvent_t start;
    hipEvent_t stop;
};

// Launchers (moe_kernels.hip).  Each returns the hipError_t of the launch.
hipError_t launch_router(const RouterArgs& a, hipStream_t st, const Timing* t = nullptr);
hipError_t launch_select(const SelectArgs& a, hipStream_t st);  // logits given
hipError_t launch_gateup(const GateUpArgs& a, int max_unique, hipStream_t st, const Timing* t = nullptr);
hipError_t launch_down(const DownArgs& a, hipStream_t st, const Timing* t = nullptr);
hipError_t launch_dequant(Fp4Mat m, int n_experts, int rows, int cols, float* out, hipStream_t st);

// One-time kernel attributes (dynamic LDS sizes).
hipError_t init_kernels();

// Rows of gate (and of up) one gate/up work item covers at hidden H.
int gateup_slab_rows(int H);

// Whether the per-workgroup LDS the kernels need at (K, E, H) fits gfx950.
bool lds_fits(int K, int E, int H);

}  // namespace moe
