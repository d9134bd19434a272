// qmoe_api.cpp -- the C ABI of libqmoe.so: argument validation, workspace
// layout, path selection and launches.  Every check runs before the first
// launch, so an error return leaves the stream and all outputs untouched
// [qmoe.rs, QMoEKernel::execute validates every input before launching and
// returns early for zero rows; its checked_product / checked_bytes guard
// size arithmetic].
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "qmoe.h"
#include "qmoe_internal.h"

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = std::string("qmoe: ") + buf;
    return code;
}

int ok()
{
    g_error.clear();
    return QMOE_OK;
}

int hip_fail(hipError_t e, const char* what)
{
    return fail(QMOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---------------------------------------------------------------- kernel timer
}  // namespace

int qmoe::set_error(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = std::string("qmoe: ") + buf;
    return code;
}

qmoe::LaunchEvents& qmoe::launch_events()
{
    static thread_local LaunchEvents ev;
    return ev;
}

namespace {

struct Timer {
    std::mutex mu;
    int stage = -1;
    std::vector<hipEvent_t> start, stop;
    size_t used = 0;
};
Timer g_timer;
constexpr size_t kTimerPairs = 4096;

// The timed stage's next kernel records the event pair in its own dispatch
// packet (qmoe::launch), so the pair spans the kernel alone.
void timer_begin(int stage, hipStream_t)
{
    if (g_timer.stage == stage && g_timer.used < g_timer.start.size()) {
        qmoe::launch_events() = {g_timer.start[g_timer.used], g_timer.stop[g_timer.used]};
    }
}

void timer_end(int stage, hipStream_t)
{
    if (g_timer.stage == stage && g_timer.used < g_timer.start.size()) {
        if (qmoe::launch_events().start == nullptr) ++g_timer.used;  // consumed by a launch
        qmoe::launch_events() = {};
    }
}

static_assert(QMOE_DECODE_MAX_ROUTES == qmoe::kDecodeRoutes, "decode switch");
static_assert(QMOE_DECODE_MAX_ROUTES <= qmoe::kDecodeMaxRoutes, "decode plan capacity");

// ---------------------------------------------------------------- workspace
constexpr size_t kAlign = 256;

struct Layout {
    bool decode;
    int m_tile;
    int nbw;            // prefill: MFMA column blocks per wavefront (4, or 2: the narrow 64-row tile)
    int k_split_cap;    // prefill fc2: most K parts y2 and the fc2 work-list have room for
    int nt1, nt2;       // n-tiles of fc1 (activation columns) and fc2 (hidden columns)
    int64_t cap1, cap2;  // work-list capacities
    int64_t m_tiles;     // m-tile capacity
    int n_counters;      // decode: fc2 column blocks with a combine counter (0: separate combine)
    size_t ids, w, offsets, sorted, wl1, n1, wl2, n2, act, y2, counters, total;
};

// Decode fc2 launches fold the combine in when every fc2 column block (at
// most H/32 of them, the narrowest decode fc2 block) has a counter that one
// thread of the zeroing workgroup can clear.
constexpr int kFusedCounterCols = 32;
constexpr int kMaxFusedCounters = 512;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Prefill fc2 K split.  A work-list item of fc2 runs all of K = I, and the
// persistent grid holds one item per workgroup slot, so a layer whose items
// fill the last round poorly (or leave slots idle) finishes sooner with K cut
// into S parts: S times the items, each 1/S as long.  The estimate counts
// each expert's last m-tile as half full and assumes the 256 compute units of
// the target GPU; S = 2 or 4 is taken only when it cuts the estimated
// makespan (in full-K item times) by more than a tenth.  The choice depends on
// shapes only, so the workspace size does too.
// Resident workgroups per CU of each prefill tile.
int64_t tile_slots_per_cu(int mt, int nbw)
{
    return mt == qmoe::kPrefillMTLarge ? 1 : nbw == 2 ? 3 : 2;
}

int fc2_split(int64_t R, int E, int H, int I, int mt, int nbw = 4)
{
    constexpr int64_t kCUs = 256;
    const int64_t nt = ceil_div(H, qmoe::prefill_fc2_cols(mt, nbw));
    const int64_t items = (ceil_div(R, mt) + (E < R ? E : R) / 2) * nt;
    const int64_t slots = kCUs * tile_slots_per_cu(mt, nbw);
    int best = 1;
    double best_cost = (double)ceil_div(items, slots);
    for (int S = 2; S <= 4; S *= 2) {
        if (I % (S * qmoe::kSuperK)) continue;
        const double cost = (double)ceil_div(items * S, slots) / S;
        if (cost < 0.9 * best_cost) {
            best = S;
            best_cost = cost;
        }
    }
    return best;
}

// Routes above which no prefill layer splits fc2's K: a split pays only
// while the fc2 items need fewer than 10 rounds of the persistent grid (at 10
// or more, no S saves a tenth of the makespan), and the items grow with
// ceil(R / m_tile) per column block.
int64_t split_route_limit(int H)
{
    int64_t lim = 0;
    const int tiles[3][2] = {{qmoe::kPrefillMTSmall, 4}, {qmoe::kPrefillMTSmall, 2}, {qmoe::kPrefillMTLarge, 4}};
    for (const auto& tl : tiles) {
        const int64_t nt = ceil_div(H, qmoe::prefill_fc2_cols(tl[0], tl[1]));
        const int64_t slots = 256 * tile_slots_per_cu(tl[0], tl[1]);
        const int64_t r = tl[0] * (9 * slots / nt);
        if (r > lim) lim = r;
    }
    return lim;
}

// prefill_mt, nbw: the prefill tile to lay the work-lists out for; the narrow
// small tile (the default) yields the most items, so its layout bounds the
// others.
// The fc2 partial sums and work-list are sized for the largest K split any
// layer with at most R routes can take (S_max parts of up to
// min(R, split_route_limit) routes), so the workspace never shrinks as T grows
// and a workspace sized for the largest batch serves every smaller one.
bool make_layout(int64_t T, int H, int I, int E, int top_k, Layout* L,
                 int prefill_mt = qmoe::kPrefillMTSmall, int nbw = 2)
{
    int64_t R;
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || top_k <= 0 || !mul_ok(T, top_k, &R) ||
        R > INT32_MAX) {
        return false;
    }
    L->decode = R <= QMOE_DECODE_MAX_ROUTES;
    L->m_tile = L->decode ? qmoe::kDecodeMT : prefill_mt;
    L->nbw = nbw;
    {
        const int a = fc2_split(R, E, H, I, qmoe::kPrefillMTSmall, 4);
        const int a2 = fc2_split(R, E, H, I, qmoe::kPrefillMTSmall, 2);
        const int b = fc2_split(R, E, H, I, qmoe::kPrefillMTLarge);
        const int ab = a > a2 ? a : a2;
        L->k_split_cap = L->decode ? 1 : (ab > b ? ab : b);
    }
    const int fc1_cols = L->decode ? qmoe::kDecodeFc1Cols : qmoe::prefill_fc1_cols(L->m_tile, nbw);
    const int fc2_cols = L->decode ? qmoe::kDecodeFc2Cols : qmoe::prefill_fc2_cols(L->m_tile, nbw);
    L->nt1 = (int)ceil_div(I, fc1_cols);
    L->nt2 = (int)ceil_div(H, fc2_cols);
    auto tiles_of = [&](int64_t r) { return ceil_div(r, L->m_tile) + (E < r ? E : r); };
    const int64_t m_tiles = tiles_of(R);
    L->m_tiles = m_tiles;
    // y2 rows and fc2 work-list m-tiles, each the larger of the unsplit layer
    // and the largest split one with at most R routes
    int64_t y2_rows = R, wl2_tiles = m_tiles;
    if (!L->decode) {
        const int s_max = I % (4 * qmoe::kSuperK) == 0 ? 4 : I % (2 * qmoe::kSuperK) == 0 ? 2 : 1;
        const int64_t r_split = R < split_route_limit(H) ? R : split_route_limit(H);
        if (s_max * r_split > y2_rows) y2_rows = s_max * r_split;
        if (s_max * tiles_of(r_split) > wl2_tiles) wl2_tiles = s_max * tiles_of(r_split);
    }
    if (!mul_ok(m_tiles, L->nt1, &L->cap1) || !mul_ok(wl2_tiles, L->nt2, &L->cap2) || L->cap1 > INT32_MAX ||
        L->cap2 > INT32_MAX) {
        return false;
    }
    int64_t act_bytes, y2_bytes;
    if (!mul_ok(R, (int64_t)I * 2, &act_bytes) || !mul_ok(y2_rows, (int64_t)H * 4, &y2_bytes)) {
        return false;
    }
    // the projection kernels address hidden [T, H] and act [R, I] with 32-bit element offsets
    if (T * (int64_t)H >= (int64_t(1) << 32) || R * (int64_t)I >= (int64_t(1) << 32)) return false;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + (bytes ? bytes : 1));
        return at;
    };
    L->ids = take((size_t)R * 4);
    L->w = take((size_t)R * 4);
    L->offsets = take(((size_t)E + 1) * 4);
    L->sorted = take((size_t)R * 4);
    if (L->decode) {  // one m-tile list serves both projections
        L->wl1 = take((size_t)m_tiles * qmoe::kDecodeTileInts * 4);
        L->n1 = take(4);
        L->wl2 = L->wl1;
        L->n2 = L->n1;
    } else {
        L->wl1 = take((size_t)(L->cap1 > 0 ? L->cap1 : 1) * 12);
        L->n1 = take(4);
        L->wl2 = take((size_t)(L->cap2 > 0 ? L->cap2 : 1) * 12);
        L->n2 = take(4);
    }
    L->act = take((size_t)act_bytes);
    L->y2 = take((size_t)y2_bytes);
    const int64_t blocks = ceil_div(H, kFusedCounterCols);
    L->n_counters = L->decode && blocks <= kMaxFusedCounters ? (int)blocks : 0;
    L->counters = take((size_t)L->n_counters * 4);
    L->total = off;
    if (!L->decode) {
        // at least the largest decode layout of the same layer (its m-tile
        // list can outgrow the first prefill work-lists), so the size never
        // drops where the decode path ends
        Layout D;
        if (make_layout(QMOE_DECODE_MAX_ROUTES / top_k, H, I, E, top_k, &D) && D.total > L->total) {
            L->total = D.total;
        }
    }
    return true;
}

int check_bits(const char* name, int bits)
{
    if (bits == 1 || bits == 2 || bits == 3 || bits == 4 || bits == 8) return QMOE_OK;
    return fail(QMOE_ERR_INVALID_ARG, "%s bits=%d is not a weight width (1, 2, 3, 4 or 8)", name, bits);
}

int check_proj(const char* name, const qmoe_proj* p)
{
    if (!p) return fail(QMOE_ERR_INVALID_ARG, "%s is NULL", name);
    const int rc = check_bits(name, p->bits);
    if (rc) return rc;
    if (!p->codes || !p->scales) return fail(QMOE_ERR_INVALID_ARG, "%s codes/scales is NULL", name);
    if (!aligned(p->codes, 16)) return fail(QMOE_ERR_INVALID_ARG, "%s codes not 16-byte aligned", name);
    if (!aligned(p->scales, 2)) return fail(QMOE_ERR_INVALID_ARG, "%s scales not 2-byte aligned", name);
    return QMOE_OK;
}

qmoe::ProjArgs proj_args(const qmoe_proj* p, float zpo)
{
    qmoe::ProjArgs a;
    a.codes = p->codes;
    a.scales = p->scales;
    a.zp = p->zero_points;
    a.bits = p->bits;
    a.zp_fallback = p->zero_points ? 0.0f
                    : std::isnan(zpo) ? (float)(1 << (p->bits - 1))
                                      : zpo;
    // tensor zero points are integers; an offset must be a multiple of 1/2
    const float twice = a.zp_fallback * 2.0f;
    a.fast = p->zero_points != nullptr ||
             (twice == std::floor(twice) && a.zp_fallback > -256.0f && a.zp_fallback < 256.0f);
    return a;
}

int check_zpo(float zpo)
{
    if (std::isinf(zpo)) return fail(QMOE_ERR_INVALID_ARG, "zero_point_offset must be finite or NaN");
    return QMOE_OK;
}

int check_block_size(int bs)
{
    if (bs < 16 || !is_pow2(bs)) {
        return fail(QMOE_ERR_INVALID_ARG, "block_size=%d must be a power of two >= 16", bs);
    }
    return QMOE_OK;
}

}  // namespace

extern "C" {

const char* qmoe_last_error(void) { return g_error.c_str(); }

int qmoe_route(const float* logits, int64_t T, int32_t E, int32_t top_k, int32_t normalize,
               int32_t* topk_ids, float* topk_weights, void* stream)
{
    if (T < 0) return fail(QMOE_ERR_INVALID_ARG, "T=%lld < 0", (long long)T);
    if (E < 1 || E > 1024) return fail(QMOE_ERR_INVALID_ARG, "E=%d outside [1, 1024]", E);
    if (top_k < 1 || top_k > E) return fail(QMOE_ERR_INVALID_ARG, "top_k=%d outside [1, E=%d]", top_k, E);
    if (normalize != 0 && normalize != 1) return fail(QMOE_ERR_INVALID_ARG, "normalize must be 0 or 1");
    int64_t n;
    if (!mul_ok(T, E, &n) || !mul_ok(T, top_k, &n)) return fail(QMOE_ERR_INVALID_ARG, "T*E overflows");
    if (T == 0) return ok();
    if (!logits || !topk_ids || !topk_weights) return fail(QMOE_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4)) {
        return fail(QMOE_ERR_INVALID_ARG, "misaligned pointer");
    }
    hipStream_t s = (hipStream_t)stream;
    timer_begin(QMOE_STAGE_ROUTE, s);
    const hipError_t e = qmoe::launch_route(logits, T, E, top_k, normalize, topk_ids, topk_weights, s);
    timer_end(QMOE_STAGE_ROUTE, s);
    return e == hipSuccess ? ok() : hip_fail(e, "route launch");
}

int qmoe_router(const void* hidden, const void* gate_weight, int64_t T, int32_t H, int32_t E,
                int32_t dtype, int32_t top_k, int32_t normalize, float* logits_out,
                int32_t* topk_ids, float* topk_weights, void* stream)
{
    if (T < 0) return fail(QMOE_ERR_INVALID_ARG, "T=%lld < 0", (long long)T);
    if (E < 1 || E > 1024) return fail(QMOE_ERR_INVALID_ARG, "E=%d outside [1, 1024]", E);
    if (top_k < 1 || top_k > E) return fail(QMOE_ERR_INVALID_ARG, "top_k=%d outside [1, E=%d]", top_k, E);
    if (normalize != 0 && normalize != 1) return fail(QMOE_ERR_INVALID_ARG, "normalize must be 0 or 1");
    if (dtype != QMOE_DTYPE_F16 && dtype != QMOE_DTYPE_BF16) {
        return fail(QMOE_ERR_INVALID_ARG, "dtype=%d is neither F16 (1) nor BF16 (2)", dtype);
    }
    if (H < 1) return fail(QMOE_ERR_INVALID_ARG, "H=%d must be >= 1", H);
    if (H % 32) return fail(QMOE_ERR_UNSUPPORTED, "H=%d must be a multiple of 32", H);
    int64_t n;
    if (!mul_ok(T, E, &n) || !mul_ok(T, H, &n) || !mul_ok(T, top_k, &n)) {
        return fail(QMOE_ERR_INVALID_ARG, "sizes overflow");
    }
    if (T == 0) return ok();
    if (!hidden || !gate_weight || !topk_ids || !topk_weights) return fail(QMOE_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned(hidden, 16) || !aligned(gate_weight, 16) || !aligned(topk_ids, 4) ||
        !aligned(topk_weights, 4) || (logits_out && !aligned(logits_out, 4))) {
        return fail(QMOE_ERR_INVALID_ARG, "hidden/gate_weight must be 16-byte and outputs 4-byte aligned");
    }
    hipStream_t s = (hipStream_t)stream;
    timer_begin(QMOE_STAGE_ROUTE, s);
    const hipError_t e = qmoe::launch_router(hidden, gate_weight, T, H, E, top_k, normalize, dtype,
                                             logits_out, topk_ids, topk_weights, s);
    timer_end(QMOE_STAGE_ROUTE, s);
    return e == hipSuccess ? ok() : hip_fail(e, "router launch");
}

int64_t qmoe_worklist_capacity(int64_t T, int32_t top_k, int32_t E, int32_t m_tile,
                               int32_t n_tile, int32_t N)
{
    int64_t R, cap;
    if (T < 0 || top_k < 1 || E < 1 || m_tile < 1 || n_tile < 1 || N < 1 || !mul_ok(T, top_k, &R)) {
        return -1;
    }
    const int64_t m_tiles = ceil_div(R, m_tile) + (E < R ? E : R);
    if (!mul_ok(m_tiles, ceil_div(N, n_tile), &cap)) return -1;
    return cap;
}

int qmoe_group(const int32_t* topk_ids, int64_t T, int32_t top_k, int32_t E, int32_t m_tile,
               int32_t n_tile, int32_t N, int32_t* expert_offsets, int32_t* sorted_routes,
               int32_t* worklist, int64_t worklist_capacity, int32_t* n_items, void* stream)
{
    if (T < 0 || top_k < 1) return fail(QMOE_ERR_INVALID_ARG, "T=%lld, top_k=%d", (long long)T, top_k);
    if (E < 1 || E > 1024) return fail(QMOE_ERR_INVALID_ARG, "E=%d outside [1, 1024]", E);
    if (m_tile < 1 || n_tile < 1 || N < 1) return fail(QMOE_ERR_INVALID_ARG, "m_tile, n_tile, N must be >= 1");
    int64_t R;
    if (!mul_ok(T, top_k, &R) || R > INT32_MAX) return fail(QMOE_ERR_INVALID_ARG, "T*top_k must be < 2^31");
    const int64_t need = qmoe_worklist_capacity(T, top_k, E, m_tile, n_tile, N);
    if (need < 0 || need > INT32_MAX) return fail(QMOE_ERR_INVALID_ARG, "work-list size overflows");
    if (worklist_capacity < need) {
        return fail(QMOE_ERR_WORKSPACE, "worklist_capacity=%lld < %lld", (long long)worklist_capacity,
                    (long long)need);
    }
    if (!expert_offsets || !n_items || !worklist || (R > 0 && (!topk_ids || !sorted_routes))) {
        return fail(QMOE_ERR_INVALID_ARG, "NULL pointer");
    }
    hipStream_t s = (hipStream_t)stream;
    timer_begin(QMOE_STAGE_GROUP, s);
    const hipError_t e = qmoe::launch_group(topk_ids, (int)R, E, m_tile, (int)ceil_div(N, n_tile),
                                            expert_offsets, sorted_routes, worklist,
                                            worklist_capacity, n_items, 0, nullptr, 0, nullptr, s);
    timer_end(QMOE_STAGE_GROUP, s);
    return e == hipSuccess ? ok() : hip_fail(e, "group launch");
}

size_t qmoe_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t top_k, int32_t dtype)
{
    Layout L;
    if ((dtype != QMOE_DTYPE_F16 && dtype != QMOE_DTYPE_BF16) || !make_layout(T, H, I, E, top_k, &L)) {
        return 0;
    }
    return L.total;
}

int qmoe_forward(const void* hidden, const float* logits, int64_t T, int32_t H, int32_t I,
                 int32_t E, const qmoe_proj* fc1, const qmoe_proj* fc2, float zero_point_offset,
                 int32_t block_size, int32_t top_k, int32_t normalize, int32_t activation,
                 int32_t dtype, void* out, int32_t* topk_ids_out, float* topk_w_out,
                 void* workspace, size_t workspace_bytes, void* stream)
{
    return qmoe_forward_ex(hidden, logits, T, H, I, E, fc1, fc2, zero_point_offset, block_size,
                           top_k, normalize, activation, dtype, out, topk_ids_out, topk_w_out,
                           nullptr, workspace, workspace_bytes, stream);
}

int qmoe_forward_ex(const void* hidden, const float* logits, int64_t T, int32_t H, int32_t I,
                    int32_t E, const qmoe_proj* fc1, const qmoe_proj* fc2, float zero_point_offset,
                    int32_t block_size, int32_t top_k, int32_t normalize, int32_t activation,
                    int32_t dtype, void* out, int32_t* topk_ids_out, float* topk_w_out,
                    const qmoe_layer_opts* opts, void* workspace, size_t workspace_bytes,
                    void* stream)
{
    int rc;
    const qmoe_layer_opts defaults = {nullptr, nullptr, nullptr, nullptr, nullptr,
                                      QMOE_SWIGLU_INTERLEAVED, 1.0f, 0.0f, INFINITY};
    const qmoe_layer_opts& o = opts ? *opts : defaults;
    if (T < 0) return fail(QMOE_ERR_INVALID_ARG, "T=%lld < 0", (long long)T);
    if (H <= 0 || I <= 0) return fail(QMOE_ERR_INVALID_ARG, "H=%d and I=%d must be > 0", H, I);
    if (E < 1 || E > 1024) return fail(QMOE_ERR_INVALID_ARG, "E=%d outside [1, 1024]", E);
    if (top_k < 1 || top_k > E) return fail(QMOE_ERR_INVALID_ARG, "top_k=%d outside [1, E=%d]", top_k, E);
    if (normalize != 0 && normalize != 1) return fail(QMOE_ERR_INVALID_ARG, "normalize must be 0 or 1");
    if (activation != QMOE_ACT_SWIGLU && activation != QMOE_ACT_GEGLU) {
        return fail(QMOE_ERR_INVALID_ARG, "activation=%d is neither SWIGLU (0) nor GEGLU (1)", activation);
    }
    if (dtype != QMOE_DTYPE_F16 && dtype != QMOE_DTYPE_BF16) {
        return fail(QMOE_ERR_INVALID_ARG, "dtype=%d is neither F16 (1) nor BF16 (2)", dtype);
    }
    if ((rc = check_block_size(block_size))) return rc;
    if (H % block_size || I % block_size) {
        return fail(QMOE_ERR_INVALID_ARG, "H=%d and I=%d must be multiples of block_size=%d", H, I,
                    block_size);
    }
    if ((rc = check_proj("fc1", fc1)) || (rc = check_proj("fc2", fc2))) return rc;
    if ((rc = check_zpo(zero_point_offset))) return rc;
    if (H % qmoe::kSuperK || I % qmoe::kSuperK) {
        return fail(QMOE_ERR_UNSUPPORTED, "H=%d and I=%d must be multiples of %d", H, I, qmoe::kSuperK);
    }
    // operator options [qmoe.rs: swiglu_fusion in {0, 1, 2}, only with SwiGLU;
    // fc3 exactly when the gate is separate; biases, router_weights optional]
    if (o.swiglu_fusion < 0 || o.swiglu_fusion > 2) {
        return fail(QMOE_ERR_INVALID_ARG, "swiglu_fusion=%d must be 0, 1 or 2", o.swiglu_fusion);
    }
    if (o.swiglu_fusion != QMOE_SWIGLU_INTERLEAVED && activation != QMOE_ACT_SWIGLU) {
        return fail(QMOE_ERR_INVALID_ARG, "swiglu_fusion=%d is only valid with SWIGLU", o.swiglu_fusion);
    }
    if ((o.swiglu_fusion == QMOE_SWIGLU_SEPARATE) != (o.fc3 != nullptr)) {
        return fail(QMOE_ERR_INVALID_ARG, "fc3 is required exactly when swiglu_fusion = 0");
    }
    if (o.fc3) {
        if ((rc = check_proj("fc3", o.fc3))) return rc;
        if (o.fc3->bits != fc1->bits || (o.fc3->zero_points == nullptr) != (fc1->zero_points == nullptr)) {
            return fail(QMOE_ERR_UNSUPPORTED, "fc3 must have fc1's width and zero-point mode");
        }
    }
    if (o.fc3_bias && !o.fc3) return fail(QMOE_ERR_INVALID_ARG, "fc3_bias without fc3");
    if ((o.fc1_bias && !aligned(o.fc1_bias, 4)) || (o.fc2_bias && !aligned(o.fc2_bias, 4)) ||
        (o.fc3_bias && !aligned(o.fc3_bias, 4)) || (o.router_weights && !aligned(o.router_weights, 4))) {
        return fail(QMOE_ERR_INVALID_ARG, "biases and router_weights must be 4-byte aligned");
    }
    // layers with biases, another gate/up layout, router_weights or 1/8-bit codes
    // take the generic kernels (prefill tiles, decode plan + m-tile kernels)
    const bool wide_codes = fc1->bits == 1 || fc1->bits == 8 || fc2->bits == 1 || fc2->bits == 8;
    const bool generic = wide_codes || o.swiglu_fusion != QMOE_SWIGLU_INTERLEAVED || o.fc1_bias ||
                         o.fc2_bias || o.router_weights;
    Layout L;
    if (!make_layout(T, H, I, E, top_k, &L)) return fail(QMOE_ERR_INVALID_ARG, "sizes overflow");
    if (T == 0) return ok();
    // the large prefill tile when its registers fit (block_size >= 32, fast
    // zero points, scales staged through LDS: whole 8-block stages per row and
    // 16-byte aligned) and it still yields a few items per CU
    const qmoe::ProjArgs w1 = proj_args(fc1, zero_point_offset);
    const qmoe::ProjArgs w2 = proj_args(fc2, zero_point_offset);
    const bool stageable = H % (8 * block_size) == 0 && I % (8 * block_size) == 0 &&
                           aligned(w1.scales, 16) && aligned(w2.scales, 16);
    if (!L.decode && block_size >= 32 && w1.fast && w2.fast && stageable && !wide_codes &&
        (T * top_k / qmoe::kPrefillMTLarge) * ceil_div(I, qmoe::prefill_fc1_cols(qmoe::kPrefillMTLarge)) >= 1024) {
        make_layout(T, H, I, E, top_k, &L, qmoe::kPrefillMTLarge, 4);
    } else if (!L.decode) {
        // the 64-row tile: narrow (two column blocks per wavefront, twice the
        // items) when its wide form leaves fewer than two fc1 items per CU
        const int64_t R_ = T * top_k;
        const int64_t items = (ceil_div(R_, qmoe::kPrefillMTSmall) + (E < R_ ? E : R_) / 2) *
                              ceil_div(I, qmoe::prefill_fc1_cols(qmoe::kPrefillMTSmall, 4));
        if (items >= 2 * 256) make_layout(T, H, I, E, top_k, &L, qmoe::kPrefillMTSmall, 4);
    }
    if (!hidden || !logits || !out) return fail(QMOE_ERR_INVALID_ARG, "hidden, logits and out must be non-NULL");
    if (!aligned(hidden, 16) || !aligned(out, 16) || !aligned(logits, 4)) {
        return fail(QMOE_ERR_INVALID_ARG, "hidden/out must be 16-byte and logits 4-byte aligned");
    }
    if ((topk_ids_out && !aligned(topk_ids_out, 4)) || (topk_w_out && !aligned(topk_w_out, 4))) {
        return fail(QMOE_ERR_INVALID_ARG, "misaligned routing output");
    }
    if (!workspace || !aligned(workspace, kAlign)) {
        return fail(QMOE_ERR_INVALID_ARG, "workspace must be non-NULL and 256-byte aligned");
    }
    if (workspace_bytes < L.total) {
        return fail(QMOE_ERR_WORKSPACE, "workspace_bytes=%zu < %zu", workspace_bytes, L.total);
    }

    const int64_t R = T * top_k;
    // fc2 K parts: the shape policy's choice for this tile, halved until each
    // part holds whole super-steps and (for the large tile, which always
    // stages its scales) whole 8-block scale stages
    int k_split = L.decode ? 1 : fc2_split(R, E, H, I, L.m_tile, L.nbw);
    while (k_split > 1 && (I % (k_split * qmoe::kSuperK) ||
                           (L.m_tile == qmoe::kPrefillMTLarge && (I / k_split) % (8 * block_size)))) {
        k_split /= 2;
    }
    if (k_split > L.k_split_cap) k_split = L.k_split_cap;
    char* ws = static_cast<char*>(workspace);
    int32_t* ids = reinterpret_cast<int32_t*>(ws + L.ids);
    float* w = reinterpret_cast<float*>(ws + L.w);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
    int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
    int32_t* wl1 = reinterpret_cast<int32_t*>(ws + L.wl1);
    int32_t* n1 = reinterpret_cast<int32_t*>(ws + L.n1);
    int32_t* wl2 = reinterpret_cast<int32_t*>(ws + L.wl2);
    int32_t* n2 = reinterpret_cast<int32_t*>(ws + L.n2);
    void* act = ws + L.act;
    float* y2 = reinterpret_cast<float*>(ws + L.y2);
    int32_t* counters = L.n_counters ? reinterpret_cast<int32_t*>(ws + L.counters) : nullptr;
    int n_counters = L.n_counters;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;

    // Expert-stationary decode: every (expert, column block) gets a workgroup
    // that streams its weights before routing is known; fc1 routes by itself.
    // Chosen when every expert is likely selected, K fits one chunk and fc1's
    // block of weights fits the kernel's LDS staging (2-bit codes, no
    // zero-point tensor: the other variants run out of registers).
    // Streamed decode (at most 16 tokens and 64 routes): a workgroup per
    // (expert, block of weight rows), its wavefronts splitting K.  With
    // fewer routes than experts its workgroups route before they request
    // weights, so unselected experts read none; taken then up to 32 experts
    // (one to eight tokens, top-2, 2048 x 2048 int2: faster than the m-tile
    // list at 16 and 32 experts, slower at 64, where thousands of workgroups
    // start only to leave).
    const bool stream_mode = !generic && L.decode && T <= 16 && R <= 64 && (E <= R || E <= 32) &&
                             qmoe::stream_fits(w1, H, 2 * I, block_size, true) &&
                             qmoe::stream_fits(w2, I, H, block_size, false);
    const bool expert_mode = !generic && !stream_mode && L.decode && E <= 64 && E <= R && H <= 2048 &&
                             I <= 2048 && fc1->bits == 2 && fc1->zero_points == nullptr;
    // The combine folds into fc2 on the streamed path only: there a column
    // block's few expert workgroups finish together; the m-tile and
    // expert-stationary paths have many more arrivals per block and the
    // combining workgroup becomes a serial tail (measured slower than the
    // separate combine launch).
    if (!stream_mode) {
        counters = nullptr;
        n_counters = 0;
    }
    qmoe::DecodePlan plan{logits, (int)T, E, normalize, w, topk_ids_out, topk_w_out, offsets, sorted,
                          counters, n_counters};
    const qmoe::DecodePlan* dplan = expert_mode ? &plan : nullptr;
    // Row-block kernels for the m-tile list: an expert has at most one route
    // per token, so a tile holds at most min(T, 16) rows.
    const bool list_mode = L.decode && !expert_mode && !stream_mode;
    const int max_rows = (int)(T < qmoe::kDecodeMT ? T : qmoe::kDecodeMT);
    const bool rows1 = list_mode && !generic && qmoe::rows_fits(w1, H, 2 * I, block_size);
    const bool rows2 = list_mode && !generic && qmoe::rows_fits(w2, I, H, block_size);
    if (L.decode && !expert_mode && !stream_mode) {  // routing, grouping and the m-tile list in one launch
        timer_begin(QMOE_STAGE_ROUTE, s);
        e = qmoe::launch_decode_plan(logits, (int)T, E, top_k, normalize, w, topk_ids_out,
                                     topk_w_out, wl1, n1, counters, n_counters, s, o.router_weights);
        timer_end(QMOE_STAGE_ROUTE, s);
        if (e != hipSuccess) return hip_fail(e, "decode plan launch");
    } else if (!L.decode) {
        timer_begin(QMOE_STAGE_ROUTE, s);
        e = qmoe::launch_route(logits, T, E, top_k, normalize, ids, w, s, o.router_weights);
        timer_end(QMOE_STAGE_ROUTE, s);
        if (e != hipSuccess) return hip_fail(e, "route launch");

        timer_begin(QMOE_STAGE_GROUP, s);
        e = qmoe::launch_group(ids, (int)R, E, L.m_tile, L.nt1, offsets, sorted, wl1, L.cap1, n1,
                               L.nt2 * k_split, wl2, L.cap2, n2, s);
        timer_end(QMOE_STAGE_GROUP, s);
        if (e != hipSuccess) return hip_fail(e, "group launch");
    }

    qmoe::ProjLaunch p1{};
    p1.a = hidden;
    p1.w = w1;
    p1.K = H;
    p1.N = 2 * I;
    p1.block_size = block_size;
    p1.top_k = top_k;
    p1.m_tile = L.m_tile;
    p1.nbw = L.nbw;
    p1.offsets = offsets;
    p1.sorted = sorted;
    p1.worklist = wl1;
    p1.n_items = n1;
    p1.grid = L.cap1 > 0 ? L.cap1 : 1;
    p1.tiles_cap = L.m_tiles;
    p1.act = activation;
    p1.act_out = act;
    p1.ap = qmoe::ActParams{o.activation_alpha, o.activation_beta, o.swiglu_limit};
    p1.fusion = o.swiglu_fusion;
    if (o.fc3) p1.w3 = proj_args(o.fc3, zero_point_offset);
    p1.bias = o.fc1_bias;
    p1.bias3 = o.fc3_bias;
    timer_begin(QMOE_STAGE_FC1, s);
    e = stream_mode ? qmoe::launch_fc1_stream(p1, plan, dtype, s)
        : rows1     ? qmoe::launch_rows_decode(p1, true, max_rows, dtype, s)
        : L.decode  ? qmoe::launch_fc1_decode(p1, dplan, dtype, s)
                    : qmoe::launch_fc1_prefill(p1, dtype, s);
    timer_end(QMOE_STAGE_FC1, s);
    if (e != hipSuccess) return hip_fail(e, "fc1 launch");

    qmoe::ProjLaunch p2{};
    p2.a = act;
    p2.w = w2;
    p2.K = I;
    p2.N = H;
    p2.block_size = block_size;
    p2.top_k = top_k;
    p2.m_tile = L.m_tile;
    p2.nbw = L.nbw;
    p2.offsets = offsets;
    p2.sorted = sorted;
    p2.worklist = wl2;
    p2.n_items = n2;
    p2.grid = L.cap2 > 0 ? L.cap2 : 1;
    p2.tiles_cap = L.m_tiles;
    p2.y2 = y2;
    p2.k_split = k_split;
    p2.part_stride = R * (int64_t)H;
    p2.bias = o.fc2_bias;
    p2.fused = qmoe::FusedCombine{counters, w, out, (int)T};  // decode: fc2 combines (counters set)
    timer_begin(QMOE_STAGE_FC2, s);
    e = stream_mode ? qmoe::launch_fc2_stream(p2, plan, dtype, s)
        : rows2     ? qmoe::launch_rows_decode(p2, false, max_rows, dtype, s)
        : L.decode  ? qmoe::launch_fc2_decode(p2, dplan, dtype, s)
                    : qmoe::launch_fc2_prefill(p2, dtype, s);
    timer_end(QMOE_STAGE_FC2, s);
    if (e != hipSuccess) return hip_fail(e, "fc2 launch");

    if (counters == nullptr) {  // prefill (and very wide decode layers): the combine launch
        timer_begin(QMOE_STAGE_COMBINE, s);
        e = qmoe::launch_combine(y2, k_split, R * (int64_t)H, w, T, H, top_k, out, dtype, s);
        timer_end(QMOE_STAGE_COMBINE, s);
        if (e != hipSuccess) return hip_fail(e, "combine launch");
    }

    if (!L.decode && topk_ids_out) {
        e = hipMemcpyAsync(topk_ids_out, ids, (size_t)R * 4, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "copy topk_ids");
    }
    if (!L.decode && topk_w_out) {
        e = hipMemcpyAsync(topk_w_out, w, (size_t)R * 4, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "copy topk_weights");
    }
    return ok();
}

namespace {
// Workspace of the shared-expert layer: the routed layer's, then the one-expert
// shared layer's, its dtype output [T, H] and the token gates float32 [T].
struct SharedLayout {
    size_t routed, shared, shared_out, gates, total;
};

bool make_shared_layout(int64_t T, int H, int I, int E, int top_k, int I_shared, int dtype,
                        SharedLayout* S)
{
    const size_t a = qmoe_workspace_size(T, H, I, E, top_k, dtype);
    const size_t b = qmoe_workspace_size(T, H, I_shared, 1, 1, dtype);
    int64_t out_bytes;
    if (a == 0 || b == 0 || !mul_ok(T, (int64_t)H * 2, &out_bytes)) return false;
    S->routed = 0;
    S->shared = align_up(a);
    S->shared_out = S->shared + align_up(b);
    S->gates = S->shared_out + align_up((size_t)out_bytes);
    S->total = S->gates + align_up((size_t)T * 4 + 4);
    return true;
}
}  // namespace

size_t qmoe_shared_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t top_k,
                                  int32_t I_shared, int32_t dtype)
{
    SharedLayout S;
    if (I_shared < 1 || !make_shared_layout(T, H, I, E, top_k, I_shared, dtype, &S)) return 0;
    return S.total;
}

int qmoe_forward_shared(const void* hidden, const float* logits, int64_t T, int32_t H, int32_t I,
                        int32_t E, const qmoe_proj* fc1, const qmoe_proj* fc2, int32_t I_shared,
                        const qmoe_proj* shared_fc1, const qmoe_proj* shared_fc2,
                        const void* shared_gate, float zero_point_offset, int32_t block_size,
                        int32_t top_k, int32_t normalize, int32_t activation, int32_t dtype,
                        void* out, int32_t* topk_ids_out, float* topk_w_out, void* workspace,
                        size_t workspace_bytes, void* stream)
{
    int rc;
    if (I_shared < 1) return fail(QMOE_ERR_INVALID_ARG, "I_shared=%d must be >= 1", I_shared);
    if ((rc = check_block_size(block_size))) return rc;
    if (!shared_gate || !aligned(shared_gate, 16)) {
        return fail(QMOE_ERR_INVALID_ARG, "shared_gate must be non-NULL and 16-byte aligned");
    }
    if ((rc = check_proj("shared_fc1", shared_fc1)) || (rc = check_proj("shared_fc2", shared_fc2))) return rc;
    SharedLayout S;
    if (!make_shared_layout(T, H, I, E, top_k, I_shared, dtype, &S)) {
        return fail(QMOE_ERR_INVALID_ARG, "invalid sizes or dtype for the shared-expert layer");
    }
    if (I_shared % block_size || I_shared % qmoe::kSuperK) {
        return fail(QMOE_ERR_UNSUPPORTED, "I_shared=%d must be a multiple of block_size and of %d",
                    I_shared, qmoe::kSuperK);
    }
    if (workspace && workspace_bytes < S.total) {
        return fail(QMOE_ERR_WORKSPACE, "workspace_bytes=%zu < %zu", workspace_bytes, S.total);
    }
    if (!workspace || !aligned(workspace, kAlign)) {
        return fail(QMOE_ERR_INVALID_ARG, "workspace must be non-NULL and 256-byte aligned");
    }
    char* ws = static_cast<char*>(workspace);
    void* shared_out = ws + S.shared_out;
    float* gates = reinterpret_cast<float*>(ws + S.gates);
    hipStream_t s = (hipStream_t)stream;
    // 1) the routed layer into out (validates every routed argument; T = 0 ends here)
    if ((rc = qmoe_forward(hidden, logits, T, H, I, E, fc1, fc2, zero_point_offset, block_size, top_k,
                           normalize, activation, dtype, out, topk_ids_out, topk_w_out,
                           ws + S.routed, S.shared - S.routed, stream))) {
        return rc;
    }
    if (T == 0) return ok();
    // 2) token gates s[t] = sigmoid(x_t . g)
    hipError_t e = qmoe::launch_shared_gate(hidden, shared_gate, T, H, dtype, gates, s);
    if (e != hipSuccess) return hip_fail(e, "shared gate launch");
    // 3) the shared expert as a one-expert layer (every token on expert 0 with
    //    weight exactly 1: the finite gates serve as its one-column logits)
    if ((rc = qmoe_forward(hidden, gates, T, H, I_shared, 1, shared_fc1, shared_fc2, zero_point_offset,
                           block_size, 1, 1, activation, dtype, shared_out, nullptr, nullptr,
                           ws + S.shared, S.shared_out - S.shared, stream))) {
        return rc;
    }
    // 4) out += s[t] * shared_out, rounded once more to dtype
    e = qmoe::launch_gated_add(out, shared_out, gates, T, H, dtype, s);
    return e == hipSuccess ? ok() : hip_fail(e, "gated add launch");
}

int qmoe_dequantize(const qmoe_proj* p, int32_t E, int32_t N, int32_t K, int32_t block_size,
                    float zero_point_offset, int32_t dtype, int32_t* codes_out, void* w_out,
                    void* stream)
{
    int rc;
    if ((rc = check_proj("projection", p))) return rc;
    if (E < 1 || N < 1 || K < 1) return fail(QMOE_ERR_INVALID_ARG, "E, N, K must be >= 1");
    if ((rc = check_block_size(block_size))) return rc;
    if (K % block_size) return fail(QMOE_ERR_INVALID_ARG, "K=%d not a multiple of block_size", K);
    if (K % 32) return fail(QMOE_ERR_UNSUPPORTED, "K=%d must be a multiple of 32", K);
    if (dtype != QMOE_DTYPE_F16 && dtype != QMOE_DTYPE_BF16) return fail(QMOE_ERR_INVALID_ARG, "bad dtype");
    if ((rc = check_zpo(zero_point_offset))) return rc;
    if (!w_out || !aligned(w_out, 16) || (codes_out && !aligned(codes_out, 4))) {
        return fail(QMOE_ERR_INVALID_ARG, "w_out must be non-NULL and 16-byte aligned");
    }
    int64_t rows, elems;
    if (!mul_ok(E, N, &rows) || !mul_ok(rows, K, &elems)) return fail(QMOE_ERR_INVALID_ARG, "size overflow");
    hipStream_t s = (hipStream_t)stream;
    const hipError_t e = qmoe::launch_dequant(proj_args(p, zero_point_offset), rows, K, block_size,
                                              dtype, codes_out, w_out, s);
    return e == hipSuccess ? ok() : hip_fail(e, "dequant launch");
}

int qmoe_raw_codes(const qmoe_proj* p, int32_t E, int32_t N, int32_t K, int32_t dtype,
                   int32_t variant, int32_t* codes_out, void* stream)
{
    int rc;
    if ((rc = check_proj("projection", p))) return rc;
    if (E < 1 || N < 1 || K < 1) return fail(QMOE_ERR_INVALID_ARG, "E, N, K must be >= 1");
    if (K % 32) return fail(QMOE_ERR_UNSUPPORTED, "K=%d must be a multiple of 32", K);
    if (dtype != QMOE_DTYPE_F16 && dtype != QMOE_DTYPE_BF16) return fail(QMOE_ERR_INVALID_ARG, "bad dtype");
    if (variant != QMOE_RAW_SINGLE_BASE && variant != QMOE_RAW_MULTI_BASE) {
        return fail(QMOE_ERR_INVALID_ARG, "variant=%d is neither SINGLE_BASE (0) nor MULTI_BASE (1)", variant);
    }
    if (variant == QMOE_RAW_MULTI_BASE && p->bits == 3) {
        return fail(QMOE_ERR_UNSUPPORTED, "the multi-base raw codes take 2- and 4-bit codes only");
    }
    if (p->bits == 1 || p->bits == 8) {
        return fail(QMOE_ERR_UNSUPPORTED, "no kernel feeds raw %d-bit codes to the matrix cores", p->bits);
    }
    if (!codes_out || !aligned(codes_out, 4)) return fail(QMOE_ERR_INVALID_ARG, "codes_out must be non-NULL");
    int64_t rows, elems;
    if (!mul_ok(E, N, &rows) || !mul_ok(rows, K, &elems)) return fail(QMOE_ERR_INVALID_ARG, "size overflow");
    const hipError_t e = qmoe::launch_raw_codes(p->codes, p->bits, rows, K, dtype,
                                                variant == QMOE_RAW_MULTI_BASE, codes_out,
                                                (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "raw codes launch");
}

int qmoe_timer_start(int32_t stage)
{
    if (stage < QMOE_STAGE_ROUTE || stage > QMOE_STAGE_COMBINE) {
        return fail(QMOE_ERR_INVALID_ARG, "unknown stage %d", stage);
    }
    std::lock_guard<std::mutex> lock(g_timer.mu);
    if (g_timer.start.empty()) {
        g_timer.start.resize(kTimerPairs);
        g_timer.stop.resize(kTimerPairs);
        for (size_t i = 0; i < kTimerPairs; ++i) {
            hipError_t e = hipEventCreate(&g_timer.start[i]);
            if (e == hipSuccess) e = hipEventCreate(&g_timer.stop[i]);
            if (e != hipSuccess) {
                g_timer.start.clear();
                g_timer.stop.clear();
                return hip_fail(e, "timer event create");
            }
        }
    }
    g_timer.used = 0;
    g_timer.stage = stage;
    return ok();
}

int qmoe_timer_stop(double* total_ms, int64_t* launches)
{
    std::lock_guard<std::mutex> lock(g_timer.mu);
    double sum = 0.0;
    for (size_t i = 0; i < g_timer.used; ++i) {
        float ms = 0.0f;
        hipError_t e = hipEventSynchronize(g_timer.stop[i]);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, g_timer.start[i], g_timer.stop[i]);
        if (e != hipSuccess) {
            g_timer.stage = -1;
            return hip_fail(e, "timer read");
        }
        sum += ms;
    }
    if (total_ms) *total_ms = sum;
    if (launches) *launches = (int64_t)g_timer.used;
    g_timer.stage = -1;
    g_timer.used = 0;
    return ok();
}

}  // extern "C"
