// gfx950 kernels of the verify step's sliding-window KV cache (PR #844
// section 8 items 1-2 and section 10: at K >= 2 rows the sliding layers
// rebuilt their keys and values by concatenation every step, and a wrapped
// rotating cache could not drop rejected rows, so a rejecting round replayed
// the forward).
//
// Layout: per layer, keys and values are rings of `capacity` slots per KV
// head, [n_layers][n_kv][capacity][head_dim] bf16; position q lives in slot
// q % capacity.  A device counter holds the committed length.  With
// capacity >= window + K - 1, writing a block of K rows never overwrites a
// position that any row of the block, or of the next block after any
// rollback, can still see; so
//   k_kv_write   copies the block's K rows of one layer or of consecutive
//                layers into their slots in place (the block's positions are
//                len .. len + K - 1, len read on the device) -- the seam needs
//                no special case;
//   k_kv_commit  advances the counter by 1 + n_accepted (read on the device:
//                the acceptance count the greedy step wrote), which drops
//                the rejected rows without moving any data;
//   k_kv_window  gathers what verify row r sees of one layer: positions
//                len + r - window + 1 .. len + r, oldest first (zeros before
//                position 0) -- for attention consumers and for parity.
// Every kernel reads the counter itself, so a step is graph-capturable with
// no host round trip.

#include "moe_device.h"

namespace moe {

// One 16-byte piece (8 bf16) per thread: piece i of the block's rows, keys
// then values, for layers a.layer .. a.layer + a.L - 1.
__global__ __launch_bounds__(kBlock) void k_kv_write(KvArgs a) {
    const int D8 = a.D >> 3;
    const size_t per = (size_t)a.L * a.K * a.n_kv * D8;  // pieces of keys (as many of values)
    const int len = *a.len;
    for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < 2 * per; i += (size_t)gridDim.x * kBlock) {
        const bool val = i >= per;
        const size_t j = val ? i - per : i;
        const int c8 = (int)(j % D8);
        size_t t = j / D8;
        const int h = (int)(t % a.n_kv);
        t /= a.n_kv;
        const int r = (int)(t % a.K);
        const int l = (int)(t / a.K) + a.layer;
        const int slot = (len + r) % a.C;
        const uint4 x = reinterpret_cast<const uint4*>(val ? a.v_new : a.k_new)[j];
        uint16_t* dst = (val ? a.v : a.k) + (((size_t)l * a.n_kv + h) * a.C + slot) * a.D + (size_t)c8 * 8;
        *reinterpret_cast<uint4*>(dst) = x;
    }
}

// The block's commit: keep row 0 and the accepted drafts (the count is
// clamped to [0, K - 1]).
__global__ void k_kv_commit(KvArgs a) {
    if (threadIdx.x == 0) {
        const int n = min(max(*a.n_accepted, 0), a.K - 1);
        *a.len += 1 + n;
    }
}

__global__ void k_kv_reset(KvArgs a) {
    if (threadIdx.x == 0) *a.len = a.len0;
}

// Window of each of the block's rows in one layer, one 16-byte piece per
// thread.
__global__ __launch_bounds__(kBlock) void k_kv_window(KvArgs a) {
    const int D8 = a.D >> 3;
    const size_t per = (size_t)a.K * a.n_kv * a.W * D8;
    const int len = *a.len;
    for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < 2 * per; i += (size_t)gridDim.x * kBlock) {
        const bool val = i >= per;
        const size_t j = val ? i - per : i;
        const int c8 = (int)(j % D8);
        size_t t = j / D8;
        const int w = (int)(t % a.W);
        t /= a.W;
        const int h = (int)(t % a.n_kv);
        const int r = (int)(t / a.n_kv);
        const int q = len + r - a.W + 1 + w;  // position, oldest first
        uint4 x = make_uint4(0, 0, 0, 0);
        if (q >= 0) {
            const uint16_t* src = (val ? a.v : a.k) + (((size_t)a.layer * a.n_kv + h) * a.C + q % a.C) * a.D;
            x = reinterpret_cast<const uint4*>(src)[c8];
        }
        reinterpret_cast<uint4*>(val ? a.v_out : a.k_out)[j] = x;
    }
}

static int kv_grid(size_t pieces) {
    const size_t g = (pieces + kBlock - 1) / kBlock;
    return (int)(g < 4096 ? (g > 0 ? g : 1) : 4096);
}

hipError_t launch_kv_write(const KvArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(k_kv_write, dim3(kv_grid(2 * (size_t)a.L * a.K * a.n_kv * (a.D / 8))), dim3(kBlock), 0, st,
                       a);
    return hipGetLastError();
}

hipError_t launch_kv_commit(const KvArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(k_kv_commit, dim3(1), dim3(64), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_kv_reset(const KvArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(k_kv_reset, dim3(1), dim3(64), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_kv_window(const KvArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(k_kv_window, dim3(kv_grid(2 * (size_t)a.K * a.n_kv * a.W * (a.D / 8))), dim3(kBlock), 0, st,
                       a);
    return hipGetLastError();
}

}  // namespace moe
