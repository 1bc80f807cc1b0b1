// C ABI of the NVFP4 MoE block-verify layer (include/moe_verify.h):
// argument validation, workspace layout, kernel sequencing, graph capture.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/moe_verify.h"
#include "moe_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// ---------------------------------------------------------------------------
// configuration checks
// ---------------------------------------------------------------------------

int check_inter(int I, int H, const char* name) {
    if (I % 32 || !pow2(I / 32) || I / 32 > 64)
        return fail(MOE_ERR_UNSUPPORTED, "%s=%d: need a power of two in [32, 2048]", name, I);
    const int slab = moe::gateup_slab_rows(H);
    if (I % slab) return fail(MOE_ERR_UNSUPPORTED, "%s=%d must be a multiple of %d at hidden=%d", name, I, slab, H);
    return MOE_OK;
}

// Extra limits of the grouped (prefill) kernels.
int check_grouped(const moe_cfg* c, int T) {
    if (c->inter % moe::kGRows || c->inter > moe::kGMaxCols)
        return fail(MOE_ERR_UNSUPPORTED, "inter=%d: the grouped path needs a multiple of %d up to %d", c->inter,
                    moe::kGRows, moe::kGMaxCols);
    if (c->shared_inter % moe::kGRows || c->shared_inter > moe::kGMaxCols)
        return fail(MOE_ERR_UNSUPPORTED, "shared_inter=%d: the grouped path needs a multiple of %d up to %d",
                    c->shared_inter, moe::kGRows, moe::kGMaxCols);
    if (!moe::grouped_lds_fits(T, c->n_experts, c->inter, c->shared_inter))
        return fail(MOE_ERR_UNSUPPORTED, "rows=%d x n_experts=%d exceeds the grouped LDS budget", T, c->n_experts);
    return MOE_OK;
}

// Whether the grouped kernels meet this shape at T rows (check_grouped's
// limits, without setting the error text).
bool grouped_shape_ok(const moe_cfg* c, int T) {
    return c->inter % moe::kGRows == 0 && c->inter <= moe::kGMaxCols && c->shared_inter % moe::kGRows == 0 &&
           c->shared_inter <= moe::kGMaxCols && moe::grouped_lds_fits(T, c->n_experts, c->inter, c->shared_inter);
}

// Rows from which MOE_REGIME_AUTO runs the grouped kernels (when the shape
// meets their limits): measured on the 40-layer stack at hidden 2048, 256
// experts, top-8, the grouped kernels take 2118 / 2736 us per stack at 8 / 16
// rows against 2592 / 6222 us for the verify-width launches, and lose at 4
// rows (1702 against 1260 us).
constexpr int kAutoGroupedRows = 8;

// Which kernels serve K rows under cfg: false = the verify-width launches
// (K <= 16), true = the grouped launches.
bool use_grouped(const moe_cfg* c, int K) {
    if (K > moe::kMaxRows || c->regime == MOE_REGIME_GROUPED) return true;
    if (c->regime == MOE_REGIME_VERIFY || c->regime == MOE_REGIME_VERIFY_ONE_LAUNCH) return false;
    return K >= kAutoGroupedRows && grouped_shape_ok(c, K);
}

// At verify width: whether a layer is one launch (router, gate/up and down
// workgroups with in-kernel hand-offs) rather than router + gate/up, then
// down.  Only on request: on MI355X the one-launch layer measured 931
// against 925 us per 40-layer stack at K = 2 and 801 against 759 at K = 1.
bool use_fused_down(const moe_cfg* c, int K) {
    return c->regime == MOE_REGIME_VERIFY_ONE_LAUNCH &&
           moe::fused_down_fits(K, c->top_k, c->n_experts, c->hidden, c->inter, c->shared_inter);
}

// The regime's own limits at K rows (after check_common).
int check_regime(const moe_cfg* c, int K) {
    if ((c->regime == MOE_REGIME_VERIFY || c->regime == MOE_REGIME_VERIFY_ONE_LAUNCH) && K > moe::kMaxRows)
        return fail(MOE_ERR_UNSUPPORTED, "the verify-width regimes serve at most %d rows (K=%d)", moe::kMaxRows, K);
    return use_grouped(c, K) ? check_grouped(c, K) : MOE_OK;
}

int check_cfg(const moe_cfg* c) {
    if (!c) return fail(MOE_ERR_INVALID, "cfg is NULL");
    if (c->hidden != 256 && c->hidden != 512 && c->hidden != 1024 && c->hidden != 2048)
        return fail(MOE_ERR_UNSUPPORTED, "hidden=%d: supported 256, 512, 1024, 2048", c->hidden);
    if (c->n_experts < 1 || c->n_experts > moe::kMaxExperts)
        return fail(MOE_ERR_UNSUPPORTED, "n_experts=%d: supported 1..%d", c->n_experts, moe::kMaxExperts);
    if (c->top_k < 1 || c->top_k > c->n_experts)
        return fail(MOE_ERR_INVALID, "top_k=%d must be in [1, n_experts=%d]", c->top_k, c->n_experts);
    if (c->top_k > moe::kMaxTopK) return fail(MOE_ERR_UNSUPPORTED, "top_k=%d > %d", c->top_k, moe::kMaxTopK);
    int rc = check_inter(c->inter, c->hidden, "inter");
    if (rc) return rc;
    if (c->shared_inter < 0) return fail(MOE_ERR_INVALID, "shared_inter=%d < 0", c->shared_inter);
    if (c->shared_inter > 0 && (rc = check_inter(c->shared_inter, c->hidden, "shared_inter"))) return rc;
    if (c->score_fn != MOE_SCORE_SOFTMAX && c->score_fn != MOE_SCORE_SIGMOID_BIAS)
        return fail(MOE_ERR_INVALID, "score_fn=%d unknown", c->score_fn);
    if (c->norm_topk != 0 && c->norm_topk != 1) return fail(MOE_ERR_INVALID, "norm_topk=%d not 0/1", c->norm_topk);
    if (c->score_fn == MOE_SCORE_SOFTMAX && !c->norm_topk)
        return fail(MOE_ERR_INVALID, "softmax scoring requires norm_topk=1");
    if (!std::isfinite(c->routed_scale)) return fail(MOE_ERR_INVALID, "routed_scale not finite");
    if (!(c->rms_eps >= 0.0f) || !std::isfinite(c->rms_eps)) return fail(MOE_ERR_INVALID, "rms_eps invalid");
    if (c->max_rows < 1) return fail(MOE_ERR_INVALID, "max_rows=%d < 1", c->max_rows);
    if (c->regime != MOE_REGIME_AUTO && c->regime != MOE_REGIME_VERIFY && c->regime != MOE_REGIME_GROUPED &&
        c->regime != MOE_REGIME_VERIFY_ONE_LAUNCH)
        return fail(MOE_ERR_INVALID, "regime=%d not a MOE_REGIME_*", c->regime);
    if (c->max_rows > moe::kMaxGroupedRows)
        return fail(MOE_ERR_UNSUPPORTED, "max_rows=%d > %d", c->max_rows, moe::kMaxGroupedRows);
    const int skinny_rows = c->max_rows < moe::kMaxRows ? c->max_rows : moe::kMaxRows;
    if (!moe::lds_fits(skinny_rows, c->n_experts, c->hidden))
        return fail(MOE_ERR_UNSUPPORTED, "max_rows=%d x n_experts=%d x hidden=%d exceeds the LDS budget",
                    skinny_rows, c->n_experts, c->hidden);
    if (c->max_rows > moe::kMaxRows) return check_grouped(c, c->max_rows);
    return MOE_OK;
}

int check_mat(const moe_nvfp4& m, const char* name, int layer = 0) {
    if (!m.q || !m.s || !m.ts) return fail(MOE_ERR_INVALID, "layer %d: %s has a NULL q/s/ts", layer, name);
    if (!aligned16(m.q) || !aligned16(m.s) || !aligned16(m.ts))
        return fail(MOE_ERR_INVALID, "layer %d: %s arrays must be 16-byte aligned", layer, name);
    return MOE_OK;
}

int check_weights(const moe_cfg* c, const moe_layer_weights* w, int layer) {
    if (!w) return fail(MOE_ERR_INVALID, "weights of layer %d are NULL", layer);
    if (!w->router_w || !aligned16(w->router_w))
        return fail(MOE_ERR_INVALID, "layer %d: router_w NULL or not 16-byte aligned", layer);
    if (w->norm_w && !aligned16(w->norm_w))
        return fail(MOE_ERR_INVALID, "layer %d: norm_w not 16-byte aligned", layer);
    if (c->score_fn == MOE_SCORE_SIGMOID_BIAS && !w->router_bias)
        return fail(MOE_ERR_INVALID, "layer %d: sigmoid scoring needs router_bias", layer);
    if (c->score_fn == MOE_SCORE_SOFTMAX && w->router_bias)
        return fail(MOE_ERR_INVALID, "layer %d: router_bias given with softmax scoring", layer);
    int rc;
    if ((rc = check_mat(w->gate, "gate", layer)) || (rc = check_mat(w->up, "up", layer)) ||
        (rc = check_mat(w->down, "down", layer)))
        return rc;
    const bool any_sh = w->sh_gate.q || w->sh_up.q || w->sh_down.q;
    if (c->shared_inter > 0) {
        if ((rc = check_mat(w->sh_gate, "sh_gate", layer)) || (rc = check_mat(w->sh_up, "sh_up", layer)) ||
            (rc = check_mat(w->sh_down, "sh_down", layer)))
            return rc;
    } else if (any_sh) {
        return fail(MOE_ERR_INVALID, "layer %d: shared expert weights given with shared_inter=0", layer);
    }
    return MOE_OK;
}

// ---------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------

struct Layout {
    int32_t* meta;
    uint32_t* handoff;      // two sets of hand-off words (moe::kHandoffSetWords each)
    float* logits;
    int32_t* ids;
    float* w;
    int32_t* uniq;
    int32_t* off;
    int32_t* asg;
    int32_t* inv;
    float* h;
    float* h_sh;
    float* ssq;
    uint16_t* xbuf;
    float* ybuf;
    uint16_t* ybf;          // bf16 [R][H]: the residual stream between stacked layers
    // grouped regime
    uint16_t* xbuf2;        // second bf16 input buffer (stacked layers alternate)
    int32_t* tiles;         // int4 [max tiles]
    float* hmax;            // [R*k][I/64]
    float* hmax_sh;         // [R][Is/64]
    float* o;               // [R*k + R][H]
    uint16_t* xh;           // fp16 copy of the layer input [R][H] (x * 2^-xsig per row)
    int32_t* xsig;          // [R] power-of-two exponent of each row of xh
    int max_tiles;
    size_t bytes;
};

Layout layout(const moe_cfg* c, void* base) {
    const size_t R = c->max_rows, E = c->n_experts, k = c->top_k, H = c->hidden;
    const size_t I = c->inter, Is = c->shared_inter;
    char* p = static_cast<char*>(base);
    size_t o = 0;
    Layout L{};
    auto take = [&](size_t bytes) { char* r = p ? p + o : nullptr; o += align256(bytes); return r; };
    L.meta = reinterpret_cast<int32_t*>(take(16 * 4));
    L.logits = reinterpret_cast<float*>(take(R * E * 4));
    L.handoff = reinterpret_cast<uint32_t*>(take((size_t)2 * moe::kHandoffSetWords * 4));
    L.ids = reinterpret_cast<int32_t*>(take(R * k * 4));
    L.w = reinterpret_cast<float*>(take(R * k * 4));
    L.uniq = reinterpret_cast<int32_t*>(take(R * k * 4));
    L.off = reinterpret_cast<int32_t*>(take((R * k + 1) * 4));
    L.asg = reinterpret_cast<int32_t*>(take(R * k * 4));
    L.inv = reinterpret_cast<int32_t*>(take(R * k * 4));
    L.h = reinterpret_cast<float*>(take(R * k * I * 4));
    L.h_sh = reinterpret_cast<float*>(take(R * (Is ? Is : 1) * 4));
    L.ssq = reinterpret_cast<float*>(take(R * (H / moe::kDownRowsPerBlock) * 4));
    L.xbuf = reinterpret_cast<uint16_t*>(take(R * H * 2));
    L.ybuf = reinterpret_cast<float*>(take(R * H * 4));
    L.ybf = reinterpret_cast<uint16_t*>(take(R * H * 2));
    L.xbuf2 = reinterpret_cast<uint16_t*>(take(R * H * 2));
    L.max_tiles = moe::grouped_max_tiles((int)R, (int)E, (int)k, Is > 0);
    L.tiles = reinterpret_cast<int32_t*>(take((size_t)L.max_tiles * 16));
    L.hmax = reinterpret_cast<float*>(take(R * k * ((I + 63) / 64) * 4));
    L.hmax_sh = reinterpret_cast<float*>(take(R * (Is ? (Is + 63) / 64 : 1) * 4));
    L.o = reinterpret_cast<float*>(take((R * k + R) * H * 4));
    L.xh = reinterpret_cast<uint16_t*>(take(R * H * 2));
    L.xsig = reinterpret_cast<int32_t*>(take(R * 4));
    L.bytes = o;
    return L;
}

moe::Fp4Mat mat(const moe_nvfp4& m) { return moe::Fp4Mat{m.q, m.s, m.ts}; }

// Every verify-width call starts both hand-off sets and the status word at
// zero (the workspace may hold anything).  Within a call, layer l uses set l % 2: a
// separate down kernel clears the router words of set 0 for the next layer,
// a one-launch layer clears the other set for the next layer.
int start_call(const Layout& L, hipStream_t st) {
    hipError_t e = moe::launch_handoff_reset(L.handoff, L.meta + moe::kMetaStatus, st);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "reset launch");
}

// ---------------------------------------------------------------------------
// one layer on the stream
// ---------------------------------------------------------------------------

struct LayerIO {
    const uint16_t* x_in;    // bf16 input (first layer / single layer), or nullptr
    const float* y_prev;     // fp32 output of the previous layer to normalise, or nullptr
    const uint16_t* gamma;   // the previous layer's norm weight (with y_prev), or nullptr
    const uint16_t* residual;
    float* y32;              // fp32 output (required)
    uint16_t* y;             // bf16 output or nullptr
};

// next_router: the router rows of the layer that follows in a stack (the down
// kernel requests them ahead of that layer's router launch), or nullptr.
// layer: the layer's index in the call (its parity picks the hand-off set).
int enqueue_layer(const moe_cfg* c, const moe_layer_weights* w, const LayerIO& io, int K, const Layout& L,
                  hipStream_t st, const moe::Timing* tm = nullptr, const uint16_t* next_router = nullptr,
                  int layer = 0) {
    hipError_t e;
    const bool has_sh = c->shared_inter > 0;
    const bool fused = use_fused_down(c, K);
    const moe::Fp4Mat none{nullptr, nullptr, nullptr};
    uint32_t* counter = fused ? L.handoff + (size_t)(layer & 1) * moe::kHandoffSetWords : L.handoff;
    int32_t* status = L.meta + moe::kMetaStatus;

    moe::RouteGateUpArgs ra{};
    ra.r.x_in = io.x_in;
    ra.r.y_prev = io.y_prev;
    ra.r.ssq = L.ssq;
    ra.r.gamma = io.gamma;
    ra.r.x_out = L.xbuf;
    ra.r.eps = c->rms_eps;
    ra.r.wr = w->router_w;
    ra.r.logits = L.logits;
    ra.r.K = K; ra.r.H = c->hidden; ra.r.E = c->n_experts;
    moe::GateUpArgs& ga = ra.g;
    ga.sel.logits = L.logits;
    ga.sel.bias = w->router_bias;
    ga.sel.ids = L.ids; ga.sel.w = L.w;
    ga.sel.n_unique = L.meta + moe::kMetaUnique;
    ga.sel.uniq = L.uniq; ga.sel.off = L.off; ga.sel.asg = L.asg; ga.sel.inv = L.inv;
    ga.sel.K = K; ga.sel.E = c->n_experts; ga.sel.k = c->top_k;
    ga.sel.score_fn = c->score_fn; ga.sel.norm_topk = c->norm_topk;
    ga.x = nullptr;
    ga.gate = mat(w->gate); ga.up = mat(w->up);
    ga.h = L.h;
    ga.sgate = has_sh ? mat(w->sh_gate) : none;
    ga.sup = has_sh ? mat(w->sh_up) : none;
    ga.h_sh = L.h_sh;
    ga.K = K; ga.H = c->hidden; ga.I = c->inter; ga.Is = c->shared_inter;
    ra.counter = counter;
    ra.status = status;
    ra.n_router = (c->n_experts + moe::kWaves - 1) / moe::kWaves;
    ra.spin_limit = moe::kRouteSpinLimit;

    moe::DownArgs& da = ra.d;
    da.down = mat(w->down);
    da.sdown = has_sh ? mat(w->sh_down) : none;
    da.n_unique = L.meta + moe::kMetaUnique;
    da.uniq = L.uniq; da.off = L.off; da.inv = L.inv;
    da.w = L.w; da.h = L.h; da.h_sh = L.h_sh;
    da.residual = io.residual;
    da.y32 = io.y32; da.y = io.y;
    da.ssq = L.ssq;
    da.K = K; da.H = c->hidden; da.I = c->inter; da.Is = c->shared_inter; da.k = c->top_k;
    da.rs = c->routed_scale;
    da.prefetch = reinterpret_cast<const uint8_t*>(next_router);
    da.prefetch_bytes = next_router ? 2 * c->n_experts * c->hidden : 0;
    if (fused) {
        // one launch: the down workgroups follow the gate/up ones
        ra.n_down = c->hidden / moe::kDownRowsPerBlock;
        ra.clear = L.handoff + (size_t)((layer + 1) & 1) * moe::kHandoffSetWords;
        if ((e = moe::launch_route_gateup(ra, st, tm ? &tm[0] : nullptr)) != hipSuccess)
            return hip_fail(e, "layer launch");
        return MOE_OK;
    }
    if ((e = moe::launch_route_gateup(ra, st, tm ? &tm[0] : nullptr)) != hipSuccess)
        return hip_fail(e, "router + gate/up launch");
    da.counter = counter;
    if ((e = moe::launch_down(da, st, tm ? &tm[1] : nullptr)) != hipSuccess) return hip_fail(e, "down launch");
    return MOE_OK;
}

// The grouped (prefill) kernels for one layer; x_next != nullptr also writes
// the next stacked layer's bf16 RMS-normalised input.
int enqueue_layer_grouped(const moe_cfg* c, const moe_layer_weights* w, const uint16_t* x, int K,
                          const uint16_t* residual, float* y32, uint16_t* y, uint16_t* x_next, const Layout& L,
                          hipStream_t st) {
    // x_next (stacked layers) is this layer's output normalised with its
    // norm weight
    hipError_t e;
    const bool has_sh = c->shared_inter > 0;
    const moe::Fp4Mat none{nullptr, nullptr, nullptr};
    int32_t* n_unique = L.meta + moe::kMetaUnique;
    int32_t* n_tiles = L.meta + moe::kMetaTiles;

    moe::RouterArgs ra{};
    ra.x_in = x;
    ra.wr = w->router_w;
    ra.logits = L.logits;
    ra.x_f16 = L.xh;
    ra.x_sig = L.xsig;
    ra.K = K; ra.H = c->hidden; ra.E = c->n_experts;

    moe::SelectArgs sa{};
    sa.logits = L.logits; sa.bias = w->router_bias;
    sa.ids = L.ids; sa.w = L.w;
    sa.K = K; sa.E = c->n_experts; sa.k = c->top_k;
    sa.score_fn = c->score_fn; sa.norm_topk = c->norm_topk;

    // Few rows: the router's column slices as workgroups of their own, their
    // partial logits in the down output buffer (written only later in the
    // layer), summed by the selection launch, which also makes the fp16 x.
    const size_t parts_floats = (size_t)moe::kRouterWaves * K * c->n_experts;
    const size_t o_floats = ((size_t)c->max_rows * c->top_k + c->max_rows) * c->hidden;
    if (K <= moe::kRouterSplitMaxRows && c->n_experts <= moe::kRouterSplitMaxExperts && c->hidden <= 2048 &&
        parts_floats <= o_floats) {
        ra.logits = L.o;
        ra.x_f16 = nullptr;
        ra.x_sig = nullptr;
        if ((e = moe::launch_router_split(ra, st)) != hipSuccess) return hip_fail(e, "router launch");
        moe::SelectSplitArgs ss{};
        ss.s = sa;
        ss.parts = L.o; ss.logits = L.logits;
        ss.x_in = x; ss.x_f16 = L.xh; ss.x_sig = L.xsig; ss.H = c->hidden;
        if ((e = moe::launch_select_rows_split(ss, st)) != hipSuccess) return hip_fail(e, "row selection launch");
    } else {
        if ((e = moe::launch_router_mfma(ra, st)) != hipSuccess) return hip_fail(e, "router launch");
        if ((e = moe::launch_select_rows(sa, st)) != hipSuccess) return hip_fail(e, "row selection launch");
    }

    // the gate/up workgroups group the slots themselves (and publish the CSR)
    const int max_tiles = moe::grouped_max_tiles(K, c->n_experts, c->top_k, has_sh);
    moe::GroupedGuArgs ga{};
    ga.x = L.xh;
    ga.x_sig = L.xsig;
    ga.gate = mat(w->gate); ga.up = mat(w->up);
    ga.sgate = has_sh ? mat(w->sh_gate) : none;
    ga.sup = has_sh ? mat(w->sh_up) : none;
    ga.ids = L.ids;
    ga.n_unique = n_unique; ga.uniq = L.uniq; ga.off = L.off; ga.asg = L.asg; ga.inv = L.inv;
    ga.tiles = L.tiles; ga.n_tiles = n_tiles;
    ga.status = L.meta + moe::kMetaStatus;
    ga.h = L.h; ga.h_sh = L.h_sh;
    ga.T = K; ga.H = c->hidden; ga.I = c->inter; ga.Is = c->shared_inter; ga.k = c->top_k; ga.E = c->n_experts;
    if ((e = moe::launch_gateup_grouped(ga, L.hmax, L.hmax_sh, max_tiles, st)) != hipSuccess)
        return hip_fail(e, "grouped gate/up launch");

    moe::GroupedDownArgs da{};
    da.down = mat(w->down);
    da.sdown = has_sh ? mat(w->sh_down) : none;
    da.uniq = L.uniq; da.off = L.off; da.tiles = L.tiles; da.n_tiles = n_tiles; da.asg = L.asg;
    da.h = L.h; da.h_sh = L.h_sh; da.o = L.o;
    da.T = K; da.H = c->hidden; da.I = c->inter; da.Is = c->shared_inter; da.k = c->top_k;
    if ((e = moe::launch_down_grouped(da, L.hmax, L.hmax_sh, max_tiles, st)) != hipSuccess)
        return hip_fail(e, "grouped down launch");

    moe::CombineArgs ca{};
    ca.o = L.o; ca.w = L.w;
    ca.residual = residual; ca.y32 = y32; ca.y = y; ca.x_next = x_next;
    ca.gamma = x_next ? w->norm_w : nullptr;
    ca.eps = c->rms_eps; ca.rs = c->routed_scale;
    ca.T = K; ca.H = c->hidden; ca.k = c->top_k; ca.has_shared = has_sh;
    if ((e = moe::launch_combine(ca, st)) != hipSuccess) return hip_fail(e, "combine launch");
    return MOE_OK;
}

int copy_debug(const moe_cfg* c, const moe_debug* d, int layer, int K, const Layout& L, const uint16_t* x_in,
               const float* y32, hipStream_t st) {
    if (!d) return MOE_OK;
    const size_t E = c->n_experts, k = c->top_k, H = c->hidden, n = (size_t)K * k;
    struct Item { void* dst; const void* src; size_t bytes; };
    const Item items[] = {
        {d->logits ? d->logits + layer * K * E : nullptr, L.logits, K * E * 4},
        {d->ids ? d->ids + layer * n : nullptr, L.ids, n * 4},
        {d->w ? d->w + layer * n : nullptr, L.w, n * 4},
        {d->n_unique ? d->n_unique + layer : nullptr, L.meta + moe::kMetaUnique, 4},
        {d->uniq ? d->uniq + layer * n : nullptr, L.uniq, n * 4},
        {d->off ? d->off + layer * (n + 1) : nullptr, L.off, (n + 1) * 4},
        {d->asg ? d->asg + layer * n : nullptr, L.asg, n * 4},
        {d->inv ? d->inv + layer * n : nullptr, L.inv, n * 4},
        {d->x_in ? d->x_in + layer * K * H : nullptr, x_in, K * H * 2},
        {d->y32 ? d->y32 + layer * K * H : nullptr, y32, K * H * 4},
        {d->status ? d->status + layer : nullptr, L.meta + moe::kMetaStatus, 4},
    };
    for (const Item& it : items) {
        if (!it.dst) continue;
        hipError_t e = hipMemcpyAsync(it.dst, it.src, it.bytes, hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess) return hip_fail(e, "debug copy");
    }
    return MOE_OK;
}

// The layer's residual input, copied before the layer runs (in a stack the
// residual stream is updated in place by the layer).
int copy_debug_residual(const moe_cfg* c, const moe_debug* d, int layer, int K, const uint16_t* residual,
                        hipStream_t st) {
    if (!d || !d->res_in || !residual) return MOE_OK;
    const size_t bytes = (size_t)K * c->hidden * 2;
    hipError_t e = hipMemcpyAsync(d->res_in + (size_t)layer * K * c->hidden, residual, bytes,
                                  hipMemcpyDeviceToDevice, st);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "debug copy");
}

int check_common(const moe_cfg* c, int K, void* ws, size_t ws_bytes) {
    int rc = check_cfg(c);
    if (rc) return rc;
    if (K < 1 || K > c->max_rows) return fail(MOE_ERR_INVALID, "K=%d outside [1, max_rows=%d]", K, c->max_rows);
    const size_t need = layout(c, nullptr).bytes;
    if (!ws) return fail(MOE_ERR_INVALID, "workspace is NULL");
    if (!aligned16(ws)) return fail(MOE_ERR_INVALID, "workspace not 16-byte aligned");
    if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    return MOE_OK;
}

int check_io(const void* x, const void* y, const void* y32, const void* residual) {
    if (!x || !aligned16(x)) return fail(MOE_ERR_INVALID, "x NULL or not 16-byte aligned");
    if (!y || !aligned16(y)) return fail(MOE_ERR_INVALID, "y NULL or not 16-byte aligned");
    if (y32 && !aligned16(y32)) return fail(MOE_ERR_INVALID, "y32 not 16-byte aligned");
    if (residual && !aligned16(residual)) return fail(MOE_ERR_INVALID, "residual not 16-byte aligned");
    return MOE_OK;
}

// residual == nullptr: no residual.  Otherwise the residual stream: layer 0
// adds `residual`, layer l >= 1 adds layer l-1's bf16 output, which the
// layers keep in L.ybf (each layer reads an element of it and then writes
// its own output there, in the same thread).
int enqueue_stack(const moe_cfg* c, const moe_layer_weights* layers, int n_layers, const uint16_t* x,
                  const uint16_t* residual, int K, uint16_t* y, float* y32, void* ws, hipStream_t st,
                  const moe_debug* dbg, const moe::Timing* tm = nullptr) {
    const Layout L = layout(c, ws);
    hipError_t e = moe::init_kernels();
    if (e != hipSuccess) return hip_fail(e, "kernel attributes");
    // the grouped kernels use no hand-off (their gate/up workgroup 0 clears
    // the status word)
    int rc0 = use_grouped(c, K) ? MOE_OK : start_call(L, st);
    if (rc0) return rc0;
    const bool stream_res = residual != nullptr;
    if (use_grouped(c, K)) {
        // grouped regime: each layer's combine writes the next layer's input,
        // alternating between two buffers so a layer's input stays readable
        for (int l = 0; l < n_layers; ++l) {
            const bool last = (l == n_layers - 1);
            const uint16_t* xin = (l == 0) ? x : ((l & 1) ? L.xbuf : L.xbuf2);
            uint16_t* xnext = last ? nullptr : ((l & 1) ? L.xbuf2 : L.xbuf);
            float* yo = last ? (y32 ? y32 : L.ybuf) : L.ybuf;
            const uint16_t* res = stream_res ? (l == 0 ? residual : L.ybf) : nullptr;
            uint16_t* yb = last ? y : (stream_res ? L.ybf : nullptr);
            int rc = copy_debug_residual(c, dbg, l, K, res, st);
            if (rc) return rc;
            rc = enqueue_layer_grouped(c, &layers[l], xin, K, res, yo, yb, xnext, L, st);
            if (rc) return rc;
            rc = copy_debug(c, dbg, l, K, L, xin, yo, st);
            if (rc) return rc;
        }
        return MOE_OK;
    }
    for (int l = 0; l < n_layers; ++l) {
        const bool last = (l == n_layers - 1);
        LayerIO io{};
        io.x_in = (l == 0) ? x : nullptr;
        io.y_prev = (l == 0) ? nullptr : L.ybuf;
        io.gamma = (l == 0) ? nullptr : layers[l - 1].norm_w;
        io.residual = stream_res ? (l == 0 ? residual : L.ybf) : nullptr;
        io.y32 = last ? (y32 ? y32 : L.ybuf) : L.ybuf;
        io.y = last ? y : (stream_res ? L.ybf : nullptr);
        int rc = copy_debug_residual(c, dbg, l, K, io.residual, st);
        if (rc) return rc;
        rc = enqueue_layer(c, &layers[l], io, K, L, st, tm ? tm + 2 * l : nullptr,
                           last ? nullptr : layers[l + 1].router_w, l);
        if (rc) return rc;
        rc = copy_debug(c, dbg, l, K, L, l == 0 ? x : L.xbuf, io.y32, st);
        if (rc) return rc;
    }
    return MOE_OK;
}

// ---------------------------------------------------------------------------
// the allocation-free entry point's scratch: a fixed device array (each GPU
// the library runs on holds its own copy until the process ends).  In host
// code `scratch` only names the symbol; its device address on each GPU comes
// from hipGetSymbolAddress with that GPU current, kept per device.
// ---------------------------------------------------------------------------

constexpr size_t kScratchBytes = size_t(5) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's scratch array (looked up on the first
// call on that device).
int scratch_of_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "get device");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "scratch symbol address");
        if (!p) return fail(MOE_ERR_HIP, "scratch symbol address is NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// exported entry points
// ---------------------------------------------------------------------------

extern "C" {

int moe_verify_version(void) { return 210; }

const char* moe_verify_last_error(void) { return g_err.c_str(); }

size_t moe_verify_workspace_bytes(const moe_cfg* cfg) {
    if (check_cfg(cfg)) return 0;
    return layout(cfg, nullptr).bytes;
}

size_t moe_verify_weight_bytes(const moe_cfg* c, int32_t n_unique, int32_t K, int32_t with_shared,
                               int32_t with_router) {
    if (check_cfg(c)) return 0;
    auto matb = [](size_t rows, size_t cols) { return rows * cols / 2 + rows * cols / 16 + 4; };
    const size_t H = c->hidden, I = c->inter, Is = c->shared_inter;
    size_t b = (size_t)n_unique * (2 * matb(I, H) + matb(H, I));
    if (with_shared && Is) b += 2 * matb(Is, H) + matb(H, Is);
    if (with_router) b += 2 * (size_t)c->n_experts * H;
    return b + 2 * 2 * (size_t)K * H;
}

int moe_verify_layer(const moe_cfg* cfg, const moe_layer_weights* w, const uint16_t* x, int32_t K,
                     const uint16_t* residual, uint16_t* y, float* y32, void* workspace, size_t workspace_bytes,
                     void* stream, const moe_debug* dbg) {
    int rc;
    if ((rc = check_common(cfg, K, workspace, workspace_bytes))) return rc;
    if ((rc = check_regime(cfg, K))) return rc;
    if ((rc = check_weights(cfg, w, 0))) return rc;
    if ((rc = check_io(x, y, y32, residual))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Layout L = layout(cfg, workspace);
    hipError_t e = moe::init_kernels();
    if (e != hipSuccess) return hip_fail(e, "kernel attributes");
    float* yo = y32 ? y32 : L.ybuf;
    if (!use_grouped(cfg, K) && (rc = start_call(L, st))) return rc;
    if ((rc = copy_debug_residual(cfg, dbg, 0, K, residual, st))) return rc;
    if (use_grouped(cfg, K)) {
        if ((rc = enqueue_layer_grouped(cfg, w, x, K, residual, yo, y, nullptr, L, st))) return rc;
        return copy_debug(cfg, dbg, 0, K, L, x, yo, st);
    }
    LayerIO io{};
    io.x_in = x;
    io.y_prev = nullptr;
    io.residual = residual;
    io.y32 = yo;
    io.y = y;
    if ((rc = enqueue_layer(cfg, w, io, K, L, st))) return rc;
    return copy_debug(cfg, dbg, 0, K, L, x, io.y32, st);
}

int moe_verify_layer_noalloc(const moe_cfg* cfg, const moe_layer_weights* w, const uint16_t* x, int32_t K,
                             const uint16_t* residual, uint16_t* y, float* y32, void* stream, const moe_debug* dbg) {
    int rc;
    if ((rc = check_cfg(cfg))) return rc;
    const size_t need = layout(cfg, nullptr).bytes;
    if (need > kScratchBytes)
        return fail(MOE_ERR_UNSUPPORTED, "this cfg needs %zu bytes of scratch; the allocation-free entry holds %zu "
                    "(lower max_rows)", need, kScratchBytes);
    void* ws = nullptr;
    if ((rc = scratch_of_current_device(&ws))) return rc;
    return moe_verify_layer(cfg, w, x, K, residual, y, y32, ws, kScratchBytes, stream, dbg);
}

size_t moe_verify_noalloc_scratch_bytes(void) { return kScratchBytes; }

int moe_verify_layer_grouped(const moe_cfg* cfg, const moe_layer_weights* w, const uint16_t* x, int32_t K,
                             const uint16_t* residual, uint16_t* y, float* y32, void* workspace,
                             size_t workspace_bytes, void* stream, const moe_debug* dbg) {
    int rc;
    if ((rc = check_common(cfg, K, workspace, workspace_bytes))) return rc;
    if ((rc = check_grouped(cfg, K))) return rc;
    if ((rc = check_weights(cfg, w, 0))) return rc;
    if ((rc = check_io(x, y, y32, residual))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Layout L = layout(cfg, workspace);
    hipError_t e = moe::init_kernels();
    if (e != hipSuccess) return hip_fail(e, "kernel attributes");
    float* yo = y32 ? y32 : L.ybuf;
    if ((rc = copy_debug_residual(cfg, dbg, 0, K, residual, st))) return rc;
    if ((rc = enqueue_layer_grouped(cfg, w, x, K, residual, yo, y, nullptr, L, st))) return rc;
    return copy_debug(cfg, dbg, 0, K, L, x, yo, st);
}

int moe_verify_stack(const moe_cfg* cfg, const moe_layer_weights* layers, int32_t n_layers, const uint16_t* x,
                     const uint16_t* residual, int32_t K, uint16_t* y, float* y32, void* workspace,
                     size_t workspace_bytes, void* stream, const moe_debug* dbg) {
    int rc;
    if ((rc = check_common(cfg, K, workspace, workspace_bytes))) return rc;
    if ((rc = check_regime(cfg, K))) return rc;
    if (!layers || n_layers < 1) return fail(MOE_ERR_INVALID, "need n_layers >= 1 and a layer array");
    for (int l = 0; l < n_layers; ++l)
        if ((rc = check_weights(cfg, &layers[l], l))) return rc;
    if ((rc = check_io(x, y, y32, residual))) return rc;
    return enqueue_stack(cfg, layers, n_layers, x, residual, K, y, y32, workspace, static_cast<hipStream_t>(stream),
                         dbg);
}

// ---------------------------------------------------------------------------
// the dense first layer and the prefill stack
// ---------------------------------------------------------------------------

namespace {

int check_dense_shape(int H, int I) {
    if (!moe::dense_shape_ok(H, I))
        return fail(MOE_ERR_UNSUPPORTED, "dense layer hidden=%d inter=%d: need hidden a multiple of 64 in [64, 2048] "
                    "and inter a multiple of 256", H, I);
    return MOE_OK;
}

int check_dense_weights(const moe_dense_weights* w) {
    if (!w) return fail(MOE_ERR_INVALID, "dense weights are NULL");
    if (!w->gate || !w->up || !w->down || !aligned16(w->gate) || !aligned16(w->up) || !aligned16(w->down))
        return fail(MOE_ERR_INVALID, "dense gate/up/down NULL or not 16-byte aligned");
    if (w->norm_w && !aligned16(w->norm_w)) return fail(MOE_ERR_INVALID, "dense norm_w not 16-byte aligned");
    return MOE_OK;
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// The prefill workspace: the MoE layout first, then the dense layer's
// scratch, its normalised output (the first MoE layer's input), its bf16
// output (the residual stream) and its fp32 output.
struct PrefillLayout {
    size_t moe, dense, xnext, ybf, y32, bytes;
};
PrefillLayout prefill_layout(const moe_cfg* c, int I) {
    PrefillLayout P{};
    const size_t R = (size_t)c->max_rows, H = (size_t)c->hidden;
    P.moe = 0;
    P.dense = round256(layout(c, nullptr).bytes);
    P.xnext = P.dense + round256(moe::dense_workspace_bytes(c->hidden, I, c->max_rows));
    P.ybf = P.xnext + round256(R * H * 2);
    P.y32 = P.ybf + round256(R * H * 2);
    P.bytes = P.y32 + round256(R * H * 4);
    return P;
}

}  // namespace

int32_t moe_kv_ring_capacity(int32_t window, int32_t max_rows) {
    if (window < 1 || max_rows < 1) {
        fail(MOE_ERR_INVALID, "window=%d and max_rows=%d must be >= 1", window, max_rows);
        return 0;
    }
    return window + max_rows - 1;
}

size_t moe_kv_ring_bytes(int32_t n_layers, int32_t n_kv, int32_t head_dim, int32_t capacity) {
    if (n_layers < 1 || n_kv < 1 || head_dim < 1 || capacity < 1) return 0;
    return (size_t)n_layers * n_kv * capacity * head_dim * 2;
}

static int check_ring(const moe_kv_ring* r, int K) {
    if (!r) return fail(MOE_ERR_INVALID, "ring is NULL");
    if (!r->k || !r->v || !r->len || !aligned16(r->k) || !aligned16(r->v))
        return fail(MOE_ERR_INVALID, "ring k/v/len NULL or k/v not 16-byte aligned");
    if (r->n_layers < 1 || r->n_kv < 1 || r->window < 1)
        return fail(MOE_ERR_INVALID, "ring n_layers=%d n_kv=%d window=%d must be >= 1", r->n_layers, r->n_kv,
                    r->window);
    if (r->head_dim < 8 || r->head_dim % 8) return fail(MOE_ERR_INVALID, "head_dim=%d: need a multiple of 8", r->head_dim);
    if (K < 1) return fail(MOE_ERR_INVALID, "K=%d < 1", K);
    if (r->capacity < r->window + K - 1)
        return fail(MOE_ERR_INVALID, "capacity=%d < window + K - 1 = %d: a rollback could lose visible rows",
                    r->capacity, r->window + K - 1);
    return MOE_OK;
}

static moe::KvArgs kv_args(const moe_kv_ring* r, int K) {
    moe::KvArgs a{};
    a.k = r->k; a.v = r->v; a.len = r->len;
    a.L = r->n_layers; a.n_kv = r->n_kv; a.D = r->head_dim; a.W = r->window; a.C = r->capacity; a.K = K;
    return a;
}

int moe_kv_ring_reset(const moe_kv_ring* ring, int32_t len, void* stream) {
    int rc;
    if ((rc = check_ring(ring, 1))) return rc;
    if (len < 0) return fail(MOE_ERR_INVALID, "len=%d < 0", len);
    moe::KvArgs a = kv_args(ring, 1);
    a.len0 = len;
    hipError_t e = moe::launch_kv_reset(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "ring reset launch");
}

static int kv_write(const moe_kv_ring* ring, int layer, int n_layers, const uint16_t* k_new, const uint16_t* v_new,
                    int K, void* stream) {
    if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new))
        return fail(MOE_ERR_INVALID, "k_new/v_new NULL or not 16-byte aligned");
    moe::KvArgs a = kv_args(ring, K);
    a.k_new = k_new; a.v_new = v_new; a.layer = layer; a.L = n_layers;
    hipError_t e = moe::launch_kv_write(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "ring write launch");
}

int moe_kv_ring_write(const moe_kv_ring* ring, const uint16_t* k_new, const uint16_t* v_new, int32_t K, void* stream) {
    int rc;
    if ((rc = check_ring(ring, K))) return rc;
    return kv_write(ring, 0, ring->n_layers, k_new, v_new, K, stream);
}

int moe_kv_ring_write_layer(const moe_kv_ring* ring, int32_t layer, const uint16_t* k_new, const uint16_t* v_new,
                            int32_t K, void* stream) {
    int rc;
    if ((rc = check_ring(ring, K))) return rc;
    if (layer < 0 || layer >= ring->n_layers)
        return fail(MOE_ERR_INVALID, "layer=%d outside [0, %d)", layer, ring->n_layers);
    return kv_write(ring, layer, 1, k_new, v_new, K, stream);
}

int moe_kv_ring_commit(const moe_kv_ring* ring, const int32_t* n_accepted, int32_t K, void* stream) {
    int rc;
    if ((rc = check_ring(ring, K))) return rc;
    if (!n_accepted) return fail(MOE_ERR_INVALID, "n_accepted is NULL");
    moe::KvArgs a = kv_args(ring, K);
    a.n_accepted = n_accepted;
    hipError_t e = moe::launch_kv_commit(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "ring commit launch");
}

int moe_kv_ring_window(const moe_kv_ring* ring, int32_t layer, int32_t K, uint16_t* k_out, uint16_t* v_out,
                       void* stream) {
    int rc;
    if ((rc = check_ring(ring, K))) return rc;
    if (layer < 0 || layer >= ring->n_layers)
        return fail(MOE_ERR_INVALID, "layer=%d outside [0, %d)", layer, ring->n_layers);
    if (!k_out || !v_out || !aligned16(k_out) || !aligned16(v_out))
        return fail(MOE_ERR_INVALID, "k_out/v_out NULL or not 16-byte aligned");
    moe::KvArgs a = kv_args(ring, K);
    a.layer = layer; a.k_out = k_out; a.v_out = v_out;
    hipError_t e = moe::launch_kv_window(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "ring window launch");
}

size_t moe_dense_workspace_bytes(int32_t hidden, int32_t inter, int32_t max_rows) {
    if (check_dense_shape(hidden, inter)) return 0;
    if (max_rows < 1) {
        fail(MOE_ERR_INVALID, "max_rows=%d < 1", max_rows);
        return 0;
    }
    return moe::dense_workspace_bytes(hidden, inter, max_rows);
}

int moe_dense_mlp(const uint16_t* x, int32_t T, int32_t hidden, int32_t inter, const moe_dense_weights* w,
                  const uint16_t* residual, float eps, uint16_t* y, float* y32, uint16_t* x_next, void* workspace,
                  size_t workspace_bytes, void* stream) {
    int rc;
    if ((rc = check_dense_shape(hidden, inter))) return rc;
    if (T < 1) return fail(MOE_ERR_INVALID, "T=%d < 1", T);
    if ((rc = check_dense_weights(w))) return rc;
    if ((rc = check_io(x, y, y32, residual))) return rc;
    if (!y32) return fail(MOE_ERR_INVALID, "y32 is NULL (the dense layer writes its fp32 output)");
    if (x_next && !aligned16(x_next)) return fail(MOE_ERR_INVALID, "x_next not 16-byte aligned");
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(MOE_ERR_INVALID, "eps invalid");
    const size_t need = moe::dense_workspace_bytes(hidden, inter, T);
    if (!workspace || !aligned16(workspace)) return fail(MOE_ERR_INVALID, "workspace NULL or not 16-byte aligned");
    if (workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    hipError_t e = moe::launch_dense_mlp(x, T, hidden, inter, w->gate, w->up, w->down, residual, w->norm_w, eps, y32, y,
                                         x_next, workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "dense layer launch");
}

size_t moe_prefill_workspace_bytes(const moe_cfg* cfg, int32_t dense_inter) {
    if (check_cfg(cfg)) return 0;
    if (check_dense_shape(cfg->hidden, dense_inter)) return 0;
    return prefill_layout(cfg, dense_inter).bytes;
}

int moe_prefill_stack(const moe_cfg* cfg, const moe_dense_weights* dense, int32_t dense_inter,
                      const moe_layer_weights* layers, int32_t n_layers, const uint16_t* x, const uint16_t* residual,
                      int32_t T, uint16_t* y, float* y32, float* dense_y32, void* workspace, size_t workspace_bytes,
                      void* stream, const moe_debug* dbg) {
    int rc;
    if ((rc = check_cfg(cfg))) return rc;
    if ((rc = check_dense_shape(cfg->hidden, dense_inter))) return rc;
    if ((rc = check_dense_weights(dense))) return rc;
    if (T < 1 || T > cfg->max_rows) return fail(MOE_ERR_INVALID, "T=%d outside [1, max_rows=%d]", T, cfg->max_rows);
    if ((rc = check_regime(cfg, T))) return rc;
    if (!layers || n_layers < 1) return fail(MOE_ERR_INVALID, "need n_layers >= 1 and a layer array");
    for (int l = 0; l < n_layers; ++l)
        if ((rc = check_weights(cfg, &layers[l], l))) return rc;
    if ((rc = check_io(x, y, y32, residual))) return rc;
    if (dense_y32 && !aligned16(dense_y32)) return fail(MOE_ERR_INVALID, "dense_y32 not 16-byte aligned");
    const PrefillLayout P = prefill_layout(cfg, dense_inter);
    if (!workspace || !aligned16(workspace)) return fail(MOE_ERR_INVALID, "workspace NULL or not 16-byte aligned");
    if (workspace_bytes < P.bytes)
        return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, P.bytes);
    char* ws = static_cast<char*>(workspace);
    uint16_t* xnext = reinterpret_cast<uint16_t*>(ws + P.xnext);
    uint16_t* ybf = reinterpret_cast<uint16_t*>(ws + P.ybf);
    float* yd = dense_y32 ? dense_y32 : reinterpret_cast<float*>(ws + P.y32);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = moe::init_kernels();
    if (e != hipSuccess) return hip_fail(e, "kernel attributes");
    e = moe::launch_dense_mlp(x, T, cfg->hidden, dense_inter, dense->gate, dense->up, dense->down, residual,
                              dense->norm_w, cfg->rms_eps, yd, ybf, xnext, ws + P.dense, st);
    if (e != hipSuccess) return hip_fail(e, "dense layer launch");
    return enqueue_stack(cfg, layers, n_layers, xnext, residual ? ybf : nullptr, T, y, y32, ws + P.moe, st, dbg);
}

int moe_verify_route(const moe_cfg* cfg, const float* logits, const float* bias, int32_t K,
                     const moe_route_out* out, void* workspace, size_t workspace_bytes, void* stream) {
    int rc;
    if ((rc = check_cfg(cfg))) return rc;
    if (K < 1 || K > cfg->max_rows) return fail(MOE_ERR_INVALID, "K=%d outside [1, max_rows=%d]", K, cfg->max_rows);
    if (!logits || !aligned16(logits)) return fail(MOE_ERR_INVALID, "logits NULL or not 16-byte aligned");
    if (cfg->score_fn == MOE_SCORE_SIGMOID_BIAS && !bias) return fail(MOE_ERR_INVALID, "sigmoid scoring needs bias");
    if (cfg->score_fn == MOE_SCORE_SOFTMAX && bias) return fail(MOE_ERR_INVALID, "bias given with softmax scoring");
    if (!out || !out->ids || !out->w || !out->n_unique || !out->uniq || !out->off || !out->asg || !out->inv)
        return fail(MOE_ERR_INVALID, "route outputs must all be non-NULL");
    if (K > moe::kMaxRows) {
        if ((rc = check_common(cfg, K, workspace, workspace_bytes))) return rc;
        if ((rc = check_grouped(cfg, K))) return rc;
    }
    hipError_t e = moe::init_kernels();
    if (e != hipSuccess) return hip_fail(e, "kernel attributes");
    moe::SelectArgs ra{};
    ra.logits = logits;
    ra.bias = bias;
    ra.ids = out->ids; ra.w = out->w; ra.n_unique = out->n_unique;
    ra.uniq = out->uniq; ra.off = out->off; ra.asg = out->asg; ra.inv = out->inv;
    ra.K = K; ra.E = cfg->n_experts; ra.k = cfg->top_k;
    ra.score_fn = cfg->score_fn; ra.norm_topk = cfg->norm_topk;
    if (K <= moe::kMaxRows) {
        e = moe::launch_select(ra, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "select launch");
        return MOE_OK;
    }
    // grouped regime: per-row selection, then the grouping workgroup (its
    // tile list goes to the workspace)
    const Layout L = layout(cfg, workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((e = moe::launch_select_rows(ra, st)) != hipSuccess) return hip_fail(e, "row selection launch");
    moe::GroupArgs ka{};
    ka.ids = out->ids; ka.n_unique = out->n_unique; ka.uniq = out->uniq; ka.off = out->off;
    ka.asg = out->asg; ka.inv = out->inv;
    ka.tiles = L.tiles; ka.n_tiles = L.meta + moe::kMetaTiles;
    ka.T = K; ka.E = cfg->n_experts; ka.k = cfg->top_k; ka.has_shared = cfg->shared_inter > 0;
    if ((e = moe::launch_group(ka, st)) != hipSuccess) return hip_fail(e, "grouping launch");
    return MOE_OK;
}

int moe_verify_dequant_nvfp4(const moe_nvfp4* m, int32_t n_experts, int32_t rows, int32_t cols, float* out,
                             void* stream) {
    if (!m) return fail(MOE_ERR_INVALID, "matrix is NULL");
    int rc = check_mat(*m, "matrix");
    if (rc) return rc;
    if (!out || !aligned16(out)) return fail(MOE_ERR_INVALID, "out NULL or not 16-byte aligned");
    if (n_experts < 1 || rows < 1 || cols < 32 || cols % 32)
        return fail(MOE_ERR_INVALID, "need n_experts, rows >= 1 and cols a positive multiple of 32");
    hipError_t e = moe::launch_dequant(mat(*m), n_experts, rows, cols, out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "dequant launch");
    return MOE_OK;
}

size_t moe_verify_lm_head_workspace_bytes(int32_t vocab, int32_t K) {
    if (vocab < 1 || K < 1 || K > moe::kLmHeadMaxRows) {
        fail(MOE_ERR_INVALID, "need vocab >= 1 and K in [1, %d]", moe::kLmHeadMaxRows);
        return 0;
    }
    return align256(moe::lm_head_workspace_bytes(vocab, K));
}

int moe_verify_lm_head_greedy(const uint16_t* x, int32_t K, const uint16_t* w, int32_t vocab, int32_t hidden,
                              const int32_t* draft, float tie_tol, float* logits, const moe_greedy_out* out,
                              void* workspace, size_t workspace_bytes, void* stream) {
    if (K < 1 || K > moe::kLmHeadMaxRows) return fail(MOE_ERR_INVALID, "K=%d outside [1, %d]", K, moe::kLmHeadMaxRows);
    if (hidden != 256 && hidden != 512 && hidden != 1024 && hidden != 2048)
        return fail(MOE_ERR_UNSUPPORTED, "hidden=%d: supported 256, 512, 1024, 2048", hidden);
    if (vocab < 1 || (long long)vocab * hidden > (1ll << 40)) return fail(MOE_ERR_INVALID, "vocab=%d invalid", vocab);
    if (!x || !aligned16(x)) return fail(MOE_ERR_INVALID, "x NULL or not 16-byte aligned");
    if (!w || !aligned16(w)) return fail(MOE_ERR_INVALID, "w NULL or not 16-byte aligned");
    if (K > 1 && !draft) return fail(MOE_ERR_INVALID, "K=%d rows need K-1 draft tokens", K);
    if (!(tie_tol >= 0.0f) || !std::isfinite(tie_tol)) return fail(MOE_ERR_INVALID, "tie_tol must be finite and >= 0");
    if (logits && !aligned16(logits)) return fail(MOE_ERR_INVALID, "logits not 16-byte aligned");
    if (!out || !out->target || !out->target_logit || !out->n_accepted || !out->emitted || !out->n_emitted)
        return fail(MOE_ERR_INVALID, "greedy outputs must all be non-NULL");
    const size_t need = align256(moe::lm_head_workspace_bytes(vocab, K));
    if (!workspace || !aligned16(workspace)) return fail(MOE_ERR_INVALID, "workspace NULL or not 16-byte aligned");
    if (workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    hipError_t e = moe::launch_lm_head_greedy(x, K, w, vocab, hidden, K > 1 ? draft : nullptr, tie_tol, logits,
                                              out->target, out->target_logit, out->n_accepted, out->emitted,
                                              out->n_emitted, workspace, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "lm_head launch");
    return MOE_OK;
}

int moe_verify_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    if (!src || !aligned16(src)) return fail(MOE_ERR_INVALID, "src NULL or not 16-byte aligned");
    if (!sink) return fail(MOE_ERR_INVALID, "sink is NULL");
    if (bytes == 0 || bytes % 16) return fail(MOE_ERR_INVALID, "bytes=%zu must be a positive multiple of 16", bytes);
    hipError_t e = moe::launch_stream_read(src, bytes / 16, sink, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "stream read launch");
    return MOE_OK;
}

int moe_verify_stack_timed(const moe_cfg* cfg, const moe_layer_weights* layers, int32_t n_layers,
                           const uint16_t* x, const uint16_t* residual, int32_t K, uint16_t* y, float* y32,
                           void* workspace, size_t workspace_bytes, void* stream, float* kernel_ms) {
    int rc;
    if ((rc = check_common(cfg, K, workspace, workspace_bytes))) return rc;
    if ((rc = check_regime(cfg, K))) return rc;
    if (!layers || n_layers < 1) return fail(MOE_ERR_INVALID, "need n_layers >= 1 and a layer array");
    if (!kernel_ms) return fail(MOE_ERR_INVALID, "kernel_ms is NULL");
    if (use_grouped(cfg, K))
        return fail(MOE_ERR_UNSUPPORTED, "per-kernel timing covers the verify-width kernels (K=%d runs the grouped "
                    "ones under this cfg)", K);
    for (int l = 0; l < n_layers; ++l)
        if ((rc = check_weights(cfg, &layers[l], l))) return rc;
    if ((rc = check_io(x, y, y32, residual))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int n_ev = 2 * n_layers;
    moe::Timing* tm = new moe::Timing[n_ev]();
    hipError_t e = hipSuccess;
    int made = 0;
    for (; made < n_ev; ++made) {
        if ((e = hipEventCreate(&tm[made].start)) != hipSuccess) break;
        if ((e = hipEventCreate(&tm[made].stop)) != hipSuccess) {
            (void)hipEventDestroy(tm[made].start);
            break;
        }
    }
    if (e == hipSuccess) {
        rc = enqueue_stack(cfg, layers, n_layers, x, residual, K, y, y32, workspace, st, nullptr, tm);
        if (!rc && (e = hipStreamSynchronize(st)) != hipSuccess) rc = hip_fail(e, "synchronize");
        const bool fused = use_fused_down(cfg, K);
        for (int i = 0; !rc && i < n_ev; ++i) {
            float ms = 0.0f;
            // a one-launch layer has no separate down kernel: its entry is 0
            if (!(fused && (i & 1)) && (e = hipEventElapsedTime(&ms, tm[i].start, tm[i].stop)) != hipSuccess)
                rc = hip_fail(e, "elapsed time");
            kernel_ms[i] = ms;
        }
        if (!rc) {
            int32_t status = 0;
            const Layout L = layout(cfg, workspace);
            if ((e = hipMemcpy(&status, L.meta + moe::kMetaStatus, 4, hipMemcpyDeviceToHost)) != hipSuccess)
                rc = hip_fail(e, "status read");
            else if (status)
                rc = fail(MOE_ERR_HIP, "a router/gate-up hand-off wait gave up (status %d)", status);
        }
    } else {
        rc = hip_fail(e, "event create");
    }
    for (int i = 0; i < made; ++i) {
        (void)hipEventDestroy(tm[i].start);
        (void)hipEventDestroy(tm[i].stop);
    }
    delete[] tm;
    return rc;
}

struct moe_stack_graph {
    hipGraph_t graph;
    hipGraphExec_t exec;
};

int moe_stack_graph_create(const moe_cfg* cfg, const moe_layer_weights* layers, int32_t n_layers,
                           const uint16_t* x, const uint16_t* residual, int32_t K, uint16_t* y, float* y32,
                           void* workspace, size_t workspace_bytes, void* stream, moe_stack_graph** out) {
    int rc;
    if (!out) return fail(MOE_ERR_INVALID, "out is NULL");
    *out = nullptr;
    if ((rc = check_common(cfg, K, workspace, workspace_bytes))) return rc;
    if ((rc = check_regime(cfg, K))) return rc;
    if (!layers || n_layers < 1) return fail(MOE_ERR_INVALID, "need n_layers >= 1 and a layer array");
    for (int l = 0; l < n_layers; ++l)
        if ((rc = check_weights(cfg, &layers[l], l))) return rc;
    if ((rc = check_io(x, y, y32, residual))) return rc;
    hipError_t e = moe::init_kernels();
    if (e != hipSuccess) return hip_fail(e, "kernel attributes");
    hipStream_t cap;
    if ((e = hipStreamCreateWithFlags(&cap, hipStreamNonBlocking)) != hipSuccess) return hip_fail(e, "stream create");
    (void)stream;
    if ((e = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal)) != hipSuccess) {
        (void)hipStreamDestroy(cap);
        return hip_fail(e, "begin capture");
    }
    rc = enqueue_stack(cfg, layers, n_layers, x, residual, K, y, y32, workspace, cap, nullptr);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(cap, &graph);
    (void)hipStreamDestroy(cap);
    if (rc) {
        if (graph) (void)hipGraphDestroy(graph);
        return rc;
    }
    if (e != hipSuccess) return hip_fail(e, "end capture");
    hipGraphExec_t exec;
    if ((e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0)) != hipSuccess) {
        (void)hipGraphDestroy(graph);
        return hip_fail(e, "graph instantiate");
    }
    moe_stack_graph* g = new moe_stack_graph{graph, exec};
    *out = g;
    return MOE_OK;
}

int moe_stack_graph_launch(moe_stack_graph* g, void* stream) {
    if (!g) return fail(MOE_ERR_INVALID, "graph is NULL");
    hipError_t e = hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "graph launch");
    return MOE_OK;
}

void moe_stack_graph_destroy(moe_stack_graph* g) {
    if (!g) return;
    (void)hipGraphExecDestroy(g->exec);
    (void)hipGraphDestroy(g->graph);
    delete g;
}

}  // extern "C"
