// host_check.cpp -- drives every entry point of qmoe_api.cpp through its host
// code (validation, workspace layout, path choice, launch sequence) with the
// kernel launchers replaced by stubs.cpp; built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.  Any failed
// expectation aborts with a message; the sanitizers abort on their own
// findings.  Pointers stand for device memory and are never dereferenced.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "qmoe.h"
#include "stubs.h"

namespace {

int g_checks = 0;

#define EXPECT(cond, ...)                                        \
    do {                                                         \
        ++g_checks;                                              \
        if (!(cond)) {                                           \
            std::fprintf(stderr, "%s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);                   \
            std::fprintf(stderr, "\n");                          \
            std::abort();                                        \
        }                                                        \
    } while (0)

// 256-byte aligned host buffers standing in for device tensors
struct Buf {
    std::vector<char> mem;
    char* p = nullptr;
    explicit Buf(size_t bytes) : mem(bytes + 256)
    {
        p = mem.data() + (256 - reinterpret_cast<uintptr_t>(mem.data()) % 256);
    }
};

Buf g_tensors(1 << 16);
char* const kT = g_tensors.p;  // every input tensor argument (never read)

qmoe_proj proj(int bits, bool zp = false)
{
    return qmoe_proj{reinterpret_cast<const uint8_t*>(kT), kT, zp ? reinterpret_cast<const uint8_t*>(kT) : nullptr,
                     bits};
}

struct Shape {
    int64_t T;
    int H, I, E, k, bits1, bits2, bs, dtype;
};

std::string joined()
{
    std::string s;
    for (const auto& c : stub::calls) s += c + " ";
    return s;
}

int forward(const Shape& s, const qmoe_proj& fc1, const qmoe_proj& fc2, size_t ws_bytes, void* ws,
            const qmoe_layer_opts* opts = nullptr, float zpo = NAN)
{
    stub::calls.clear();
    return qmoe_forward_ex(kT, reinterpret_cast<const float*>(kT), s.T, s.H, s.I, s.E, &fc1, &fc2, zpo, s.bs,
                           s.k, 1, QMOE_ACT_SWIGLU, s.dtype, kT, nullptr, nullptr, opts, ws, ws_bytes,
                           nullptr);
}

// A valid layer call: QMOE_OK, every workspace buffer the launchers see
// inside [ws, ws + size), and the expected first and last launches.
void valid_layer(const Shape& s, bool rows_ok, bool stream_ok, const qmoe_layer_opts* opts = nullptr,
                 bool zp = false)
{
    const size_t need = qmoe_workspace_size(s.T, s.H, s.I, s.E, s.k, s.dtype);
    EXPECT(need > 0 && need % 256 == 0, "workspace size %zu for T=%lld", need, (long long)s.T);
    Buf ws(need);
    stub::ws_lo = ws.p;
    stub::ws_hi = ws.p + need;
    stub::rows_ok = rows_ok;
    stub::stream_ok = stream_ok;
    const qmoe_proj fc1 = proj(s.bits1, zp), fc2 = proj(s.bits2, zp);
    const int rc = forward(s, fc1, fc2, need, ws.p, opts);
    EXPECT(rc == QMOE_OK, "T=%lld H=%d I=%d E=%d k=%d: rc=%d (%s)", (long long)s.T, s.H, s.I, s.E, s.k, rc,
           qmoe_last_error());
    const std::string seq = joined();
    const int64_t R = s.T * s.k;
    if (R == 0) {
        EXPECT(stub::calls.empty(), "T=0 launched: %s", seq.c_str());
    } else if (R > QMOE_DECODE_MAX_ROUTES) {
        EXPECT(seq == "route group fc1_prefill fc2_prefill combine ", "prefill sequence: %s", seq.c_str());
    } else {
        EXPECT(stub::calls.size() >= 2 && stub::calls.size() <= 4, "decode sequence: %s", seq.c_str());
        const std::string& last = stub::calls.back();
        EXPECT(last == "combine" || last == "fc2_stream", "decode ends with %s", seq.c_str());
    }
    if (R > 0) {
        // a workspace one byte short is either rejected before any launch or,
        // where the chosen tile needs less, used within its bounds
        stub::ws_hi = ws.p + need - 1;
        const int short_rc = forward(s, fc1, fc2, need - 1, ws.p, opts);
        EXPECT((short_rc == QMOE_ERR_WORKSPACE && stub::calls.empty()) || short_rc == QMOE_OK,
               "short workspace: rc=%d calls=%s", short_rc, joined().c_str());
        // a clearly small one is always rejected before any launch
        const int tiny_rc = forward(s, fc1, fc2, 256, ws.p, opts);
        EXPECT(tiny_rc == QMOE_ERR_WORKSPACE && stub::calls.empty(), "small workspace: rc=%d calls=%s", tiny_rc,
               joined().c_str());
    }
    stub::ws_lo = stub::ws_hi = nullptr;
}

void expect_error(int rc, int code, const char* what)
{
    EXPECT(rc == code, "%s: rc=%d, expected %d (%s)", what, rc, code, qmoe_last_error());
    EXPECT(std::strlen(qmoe_last_error()) > 6, "%s: empty message", what);
    EXPECT(stub::calls.empty(), "%s: launched %s", what, joined().c_str());
}

void sizes()
{
    // capacity formula, overflow and invalid arguments
    EXPECT(qmoe_worklist_capacity(512, 2, 8, 128, 128, 2048) == (8 + 8) * 16, "capacity");
    EXPECT(qmoe_worklist_capacity(0, 2, 8, 16, 16, 16) == 0, "capacity T=0");
    EXPECT(qmoe_worklist_capacity(-1, 2, 8, 16, 16, 16) == -1, "capacity T<0");
    EXPECT(qmoe_worklist_capacity(INT64_MAX / 2, 1024, 1024, 16, 16, 1 << 30) == -1, "capacity overflow");
    EXPECT(qmoe_worklist_capacity(8, 2, 8, 0, 16, 16) == -1, "capacity m_tile 0");
    // workspace: zero for invalid or overflowing shapes, 256-aligned,
    // non-decreasing in T within each path
    EXPECT(qmoe_workspace_size(-1, 128, 128, 8, 2, 1) == 0, "workspace T<0");
    EXPECT(qmoe_workspace_size(INT64_MAX / 4, 4096, 14336, 8, 2, 2) == 0, "workspace overflow");
    EXPECT(qmoe_workspace_size(16, 0, 128, 8, 2, 1) == 0, "workspace H=0");
    const int shapes[][4] = {{2048, 2048, 8, 2}, {4096, 14336, 8, 2}, {2048, 768, 512, 10},
                             {256, 512, 8, 2}, {7168, 2048, 256, 8}, {128, 384, 1024, 1}};
    for (const auto& sh : shapes) {
        size_t prev = 0;
        for (int64_t T = 1; T <= 16384; T = T < 200 ? T + 1 : T * 17 / 16) {
            const size_t ws = qmoe_workspace_size(T, sh[0], sh[1], sh[2], sh[3], 2);
            EXPECT(ws % 256 == 0 && ws >= prev, "workspace H=%d I=%d E=%d k=%d T=%lld: %zu after %zu", sh[0],
                   sh[1], sh[2], sh[3], (long long)T, ws, prev);
            prev = ws;
        }
    }
    const size_t base = qmoe_workspace_size(512, 2048, 2048, 8, 2, 2);
    EXPECT(qmoe_shared_workspace_size(512, 2048, 2048, 8, 2, 1024, 2) > base, "shared workspace");
}

void layers()
{
    // decode (streamed, rows, m-tile) and prefill (both tile sizes) paths
    valid_layer({8, 2048, 2048, 8, 2, 2, 2, 128, 1}, false, true);
    valid_layer({8, 2048, 2048, 8, 2, 2, 2, 128, 1}, true, false);
    valid_layer({8, 2048, 2048, 8, 2, 2, 2, 128, 1}, false, false);
    valid_layer({6, 2048, 768, 512, 10, 3, 2, 128, 2}, true, false);
    valid_layer({16, 256, 512, 8, 2, 4, 4, 128, 1}, false, true);
    valid_layer({40, 256, 384, 16, 2, 4, 2, 64, 2}, false, false);
    valid_layer({41, 256, 384, 16, 2, 4, 2, 64, 2}, false, false);
    valid_layer({512, 2048, 2048, 8, 2, 4, 4, 128, 1}, false, false, nullptr, true);
    valid_layer({4096, 4096, 14336, 8, 2, 4, 4, 128, 2}, false, false);
    valid_layer({2048, 256, 8192, 4, 2, 4, 3, 32, 2}, false, false);
    valid_layer({3000, 640, 384, 1024, 7, 2, 3, 64, 1}, false, false);
    valid_layer({0, 128, 128, 4, 2, 4, 4, 32, 1}, false, false);
    valid_layer({1, 128, 128, 1, 1, 1, 8, 16, 2}, false, false);
    valid_layer({200, 256, 256, 4, 4, 8, 1, 32, 1}, false, false);

    // operator options: every layout, biases, router_weights
    qmoe_layer_opts o = QMOE_LAYER_OPTS_DEFAULT;
    const float* fbuf = reinterpret_cast<const float*>(kT);
    o.fc1_bias = fbuf;
    o.fc2_bias = fbuf;
    o.router_weights = fbuf;
    o.activation_alpha = 1.702f;
    o.activation_beta = 1.0f;
    o.swiglu_limit = 7.0f;
    valid_layer({8, 1024, 512, 8, 2, 4, 4, 128, 2}, true, true, &o);
    valid_layer({300, 1024, 512, 8, 2, 4, 4, 128, 2}, true, true, &o);
    o.swiglu_fusion = QMOE_SWIGLU_HALVES;
    valid_layer({70, 512, 256, 6, 2, 2, 4, 64, 1}, true, true, &o);
    const qmoe_proj fc3 = proj(2);
    o.swiglu_fusion = QMOE_SWIGLU_SEPARATE;
    o.fc3 = &fc3;
    o.fc3_bias = fbuf;
    valid_layer({70, 512, 256, 6, 2, 2, 4, 64, 1}, true, true, &o);
    valid_layer({5, 512, 256, 6, 2, 2, 4, 64, 1}, true, true, &o);
}

void errors()
{
    const size_t need = qmoe_workspace_size(64, 256, 256, 8, 2, 1);
    Buf ws(need);
    const Shape s{64, 256, 256, 8, 2, 4, 4, 32, 1};
    const qmoe_proj ok1 = proj(4), ok2 = proj(4);
    stub::calls.clear();
    auto fwd = [&](Shape x, qmoe_proj a, qmoe_proj b, const qmoe_layer_opts* o = nullptr, float zpo = NAN,
                   void* w = nullptr) {
        return forward(x, a, b, need, w ? w : ws.p, o, zpo);
    };
    Shape x = s;
    x.T = -1;
    expect_error(fwd(x, ok1, ok2), QMOE_ERR_INVALID_ARG, "T < 0");
    x = s;
    x.E = 1025;
    expect_error(fwd(x, ok1, ok2), QMOE_ERR_INVALID_ARG, "E > 1024");
    x = s;
    x.k = 9;
    expect_error(fwd(x, ok1, ok2), QMOE_ERR_INVALID_ARG, "top_k > E");
    x = s;
    x.bs = 48;
    expect_error(fwd(x, ok1, ok2), QMOE_ERR_INVALID_ARG, "block_size not a power of two");
    x = s;
    x.dtype = 3;
    expect_error(fwd(x, ok1, ok2), QMOE_ERR_INVALID_ARG, "dtype");
    x = s;
    x.H = 160;
    expect_error(fwd(x, ok1, ok2), QMOE_ERR_UNSUPPORTED, "H not a multiple of 128");
    expect_error(fwd(s, proj(5), ok2), QMOE_ERR_INVALID_ARG, "bits 5");
    expect_error(fwd(s, ok1, proj(6)), QMOE_ERR_INVALID_ARG, "bits 6");
    qmoe_proj bad = ok1;
    bad.codes = reinterpret_cast<const uint8_t*>(kT + 4);
    expect_error(fwd(s, bad, ok2), QMOE_ERR_INVALID_ARG, "misaligned codes");
    bad = ok1;
    bad.scales = nullptr;
    expect_error(fwd(s, bad, ok2), QMOE_ERR_INVALID_ARG, "NULL scales");
    expect_error(fwd(s, ok1, ok2, nullptr, INFINITY), QMOE_ERR_INVALID_ARG, "infinite zero_point_offset");
    expect_error(fwd(s, ok1, ok2, nullptr, NAN, kT + 128), QMOE_ERR_INVALID_ARG, "misaligned workspace");
    stub::calls.clear();
    EXPECT(qmoe_forward(nullptr, reinterpret_cast<const float*>(kT), 64, 256, 256, 8, &ok1, &ok2, NAN, 32, 2, 1,
                        QMOE_ACT_SWIGLU, 1, kT, nullptr, nullptr, ws.p, need, nullptr) == QMOE_ERR_INVALID_ARG,
           "NULL hidden");
    EXPECT(stub::calls.empty(), "NULL hidden launched");

    qmoe_layer_opts o = QMOE_LAYER_OPTS_DEFAULT;
    o.swiglu_fusion = 3;
    expect_error(fwd(s, ok1, ok2, &o), QMOE_ERR_INVALID_ARG, "swiglu_fusion 3");
    o = QMOE_LAYER_OPTS_DEFAULT;
    o.swiglu_fusion = QMOE_SWIGLU_SEPARATE;
    expect_error(fwd(s, ok1, ok2, &o), QMOE_ERR_INVALID_ARG, "separate layout without fc3");
    const qmoe_proj fc3_other = proj(2);
    o.fc3 = &fc3_other;
    expect_error(fwd(s, ok1, ok2, &o), QMOE_ERR_UNSUPPORTED, "fc3 of another width");
    o = QMOE_LAYER_OPTS_DEFAULT;
    o.fc3_bias = reinterpret_cast<const float*>(kT);
    expect_error(fwd(s, ok1, ok2, &o), QMOE_ERR_INVALID_ARG, "fc3_bias without fc3");
    o = QMOE_LAYER_OPTS_DEFAULT;
    o.fc1_bias = reinterpret_cast<const float*>(kT + 2);
    expect_error(fwd(s, ok1, ok2, &o), QMOE_ERR_INVALID_ARG, "misaligned bias");

    // the other entry points' checks
    stub::calls.clear();
    int32_t* ids = reinterpret_cast<int32_t*>(kT);
    float* w = reinterpret_cast<float*>(kT);
    expect_error(qmoe_route(w, 4, 0, 1, 1, ids, w, nullptr), QMOE_ERR_INVALID_ARG, "route E=0");
    expect_error(qmoe_route(w, 4, 8, 2, 2, ids, w, nullptr), QMOE_ERR_INVALID_ARG, "route normalize 2");
    expect_error(qmoe_route(w, 4, 8, 2, 1, nullptr, w, nullptr), QMOE_ERR_INVALID_ARG, "route NULL ids");
    expect_error(qmoe_router(kT, kT, 4, 100, 8, 1, 2, 1, w, ids, w, nullptr), QMOE_ERR_UNSUPPORTED,
                 "router H not a multiple of 32");
    expect_error(qmoe_router(kT, kT, 4, 128, 8, 3, 2, 1, w, ids, w, nullptr), QMOE_ERR_INVALID_ARG,
                 "router dtype");
    expect_error(qmoe_dequantize(&ok1, 2, 4, 100, 32, NAN, 1, ids, kT, nullptr), QMOE_ERR_INVALID_ARG,
                 "dequantize K not a multiple of block_size");
    const qmoe_proj wide = proj(8);
    expect_error(qmoe_raw_codes(&wide, 2, 4, 128, 1, QMOE_RAW_SINGLE_BASE, ids, nullptr), QMOE_ERR_UNSUPPORTED,
                 "raw codes 8-bit");
    const qmoe_proj three = proj(3);
    expect_error(qmoe_raw_codes(&three, 2, 4, 128, 1, QMOE_RAW_MULTI_BASE, ids, nullptr), QMOE_ERR_UNSUPPORTED,
                 "raw codes multi-base 3-bit");
    expect_error(qmoe_timer_start(99), QMOE_ERR_INVALID_ARG, "timer stage");

    // valid calls of the other entry points
    stub::calls.clear();
    EXPECT(qmoe_route(w, 4, 8, 2, 1, ids, w, nullptr) == QMOE_OK && joined() == "route ", "route");
    stub::calls.clear();
    EXPECT(qmoe_router(kT, kT, 4, 128, 8, 1, 2, 1, nullptr, ids, w, nullptr) == QMOE_OK && joined() == "router ",
           "router");
    stub::calls.clear();
    EXPECT(qmoe_dequantize(&ok1, 2, 4, 128, 32, 1.5f, 1, ids, kT, nullptr) == QMOE_OK, "dequantize");
    EXPECT(qmoe_raw_codes(&ok1, 2, 4, 128, 2, QMOE_RAW_MULTI_BASE, ids, nullptr) == QMOE_OK, "raw codes");
    EXPECT(joined() == "dequant raw_codes ", "hooks: %s", joined().c_str());
}

void shared_expert()
{
    const int64_t T = 300;
    const size_t need = qmoe_shared_workspace_size(T, 512, 256, 8, 2, 512, 2);
    Buf ws(need);
    stub::ws_lo = ws.p;
    stub::ws_hi = ws.p + need;
    const qmoe_proj p = proj(4);
    stub::calls.clear();
    const int rc = qmoe_forward_shared(kT, reinterpret_cast<const float*>(kT), T, 512, 256, 8, &p, &p, 512, &p, &p,
                                       kT, NAN, 128, 2, 1, QMOE_ACT_SWIGLU, 2, kT, nullptr, nullptr, ws.p, need,
                                       nullptr);
    EXPECT(rc == QMOE_OK, "shared: rc=%d (%s)", rc, qmoe_last_error());
    const std::string seq = joined();
    EXPECT(seq.find("shared_gate") != std::string::npos && stub::calls.back() == "gated_add", "shared: %s",
           seq.c_str());
    stub::calls.clear();
    EXPECT(qmoe_forward_shared(kT, reinterpret_cast<const float*>(kT), T, 512, 256, 8, &p, &p, 512, &p, &p, kT,
                               NAN, 128, 2, 1, QMOE_ACT_SWIGLU, 2, kT, nullptr, nullptr, ws.p, need - 256,
                               nullptr) == QMOE_ERR_WORKSPACE &&
               stub::calls.empty(),
           "shared short workspace");
    stub::ws_lo = stub::ws_hi = nullptr;
}

void timer()
{
    EXPECT(qmoe_timer_start(QMOE_STAGE_FC1) == QMOE_OK, "timer start");
    const int events = stub::events;
    EXPECT(events > 0, "timer created no events");
    EXPECT(qmoe_timer_start(QMOE_STAGE_FC2) == QMOE_OK && stub::events == events, "events created once");
    double ms = -1.0;
    int64_t launches = -1;
    EXPECT(qmoe_timer_stop(&ms, &launches) == QMOE_OK && launches == 0 && ms == 0.0, "timer stop");
}

}  // namespace

int main()
{
    sizes();
    layers();
    errors();
    shared_expert();
    timer();
    std::printf("host_check: %d checks passed\n", g_checks);
    return 0;
}
