// gemm_stream.hip -- decode projections that stream every selected expert's
// packed weights straight into the MFMA B registers.
//
// [PR 33569: the decode path serves small expanded-row counts, and its time
// is set by the packed-weight bytes; qmoe.rs QMoEKernel::execute: route,
// group, fc1 + activation, fc2, combine.]  With at most 16 tokens (and
// R = T*top_k <= 64 routes) every selected expert's weights are read once and
// multiplied with at most 16 rows (a token routes to an expert at most once),
// so a projection costs the time to stream its bytes plus the work left once
// the last of them arrives.
//
// One workgroup of eight wavefronts per (expert, block of weight rows).  The
// wavefronts split K: wavefront (rw, kw) owns S super-steps of 128 inputs
// starting at kw * S * 128 (a K slice of 32, 64 or 128 bytes of every weight
// row) for RBW blocks of 16 weight rows, so its A fragments (all 16 MFMA
// rows of the slice: the tokens for fc1, the expert's routed rows for fc2)
// fit in registers and are read from LDS once, not once per weight row block.
// Every global request covers whole 64-byte segments:
// - A: each wavefront copies its slice (rows past the last read as zeros
//   through a bounds-checked buffer resource, without memory traffic) with
//   contiguous 16-byte lanes into a wavefront-private LDS region and reads
//   its fragments back;
// - scales: the workgroup's rows are contiguous, so their scale rows form one
//   block copied to an LDS table with 16-byte lanes;
// - weights: lane 16g + c reads 16 contiguous bytes of weight row c (the
//   four lanes of a row cover its 64-byte slice) and the lane groups trade
//   8-byte pieces with v_permlane16_swap / v_permlane32_swap, so that lane
//   group g holds the 32-code span MFMA lane group g consumes in each
//   super-step (the same spans the prefill kernels read).
// The only other LDS traffic is one float32 partial tile per wavefront and
// row block (written over its own A region), summed over the K slices in
// slice order (deterministic) by the epilogue.  Workgroup barriers wait for
// LDS only (s_waitcnt lgkmcnt(0); s_barrier), never for the weight loads in
// flight.
//
// Order of requests: fc1 the router logits and the A slice (the tokens),
// fc2 the expert's offsets; the scales and the first half of the weight row
// blocks; then fc1 routes every token (the first workgroup writes the routing
// weights, expert offsets and sorted routes for fc2 and the combine) and a
// workgroup whose expert has no rows leaves; fc2's A slice and the second
// half of the weight blocks follow.  vmcnt retires loads in issue order, so
// each wait names exactly the loads it needs, and the A slice is requested
// before the weights it multiplies.  A slices cover AR = 8 or 16 rows (the
// tokens or the expert's rows fit in 8 for T <= 8); MFMA rows past AR hold
// whatever the LDS region held and are never stored.
//
// RAW (block_size a multiple of 128: one scale per lane and super-step): the
// B registers are the raw codes made exact dtype values by one v_and_or_b32
// each, with a base b_r per register r chosen so that the code's bits, where
// they already sit in the packed word (or nearly), weigh 1.  The zero point
// and the bases are taken out per super-step in float32:
// sum_k (q_k - zp) a_k = mfma(a, b_r + q) - sum_k (b_r(k) + zp) a_k; the last
// sum (the correction) starts the super-step's MFMA chain, and the scale
// multiplies the chain's result.  Otherwise each weight is dequantized in
// registers as (q - zp) * scale with a constant zero point.
#include "gemm_common.h"
#include "route_common.h"

namespace qmoe {
namespace {

constexpr int kWavesS = 8;
constexpr int kThreadsS = kWavesS * kWave;
constexpr int kRowsA = 16;               // MFMA rows: tokens (fc1) or the expert's rows (fc2)
constexpr int kMaxK = 2048;
constexpr int kTokW = kRowsA / kWavesS;  // tokens each wavefront routes (T <= 16)
constexpr int kGroupTok = 4;             // tokens per wavefront with 16 lanes per token (E <= 16)
constexpr int kMaxRoutesS = kWave;       // routes (T * top_k), one per lane of wavefront 0

// A kernel argument held in SGPRs from here on: the compiler may otherwise
// fetch it again where it is used, and a fetch issued after the weight
// loads waits behind them.
template <class T>
__device__ inline T held(T v)
{
    asm volatile("" : "+s"(v));
    return v;
}

// Buffer resource over `bytes` bytes from `base`: a load at an offset past the
// end returns zeros and touches no memory.
__device__ inline __amdgpu_buffer_rsrc_t bounded(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// The dtype's (1, 1) pair, the B operand of a plain sum in v_dot2.
template <int DT>
__device__ inline float dot2_sum(uint32_t a, float acc)
{
    if constexpr (DT == kF16) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, ones2<DT>()), acc, false);
    } else {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a), __builtin_bit_cast(b2, ones2<DT>()), acc,
                                               false);
    }
}

// Workgroup barrier for LDS data only: loads from global memory stay in flight.
__device__ inline void sync_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The 64-byte K slice of a weight row read by lane group g as bytes
// [16g, 16g+16) (8-byte pieces 2g and 2g+1) becomes pieces g and g + 4 of
// lane group g, super-steps 0 and 1 of its span: a transpose of 16-lane
// blocks by v_permlane16_swap (odd rows of the first operand with even rows
// of the second), then v_permlane32_swap (upper half of the first with lower
// half of the second).
__device__ inline void spans_of_slice(const u32x4& v, Span<2>& s0, Span<2>& s1)
{
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const auto a = __builtin_amdgcn_permlane16_swap(v[d], v[d + 2], false, false);
        const auto b = __builtin_amdgcn_permlane32_swap(a[0], a[1], false, false);
        s0.w[d] = b[0];
        s1.w[d] = b[1];
    }
}

// LDS of a workgroup (the wavefronts' A regions and the scale table), and
// the wavefronts per SIMD its registers are sized for: four (two workgroups
// per CU) unless the LDS or RBW = 8's registers leave room for one.
template <int S, int KSW, int RBW, bool RAW>
constexpr int stream_lds_bytes()
{
    return kWavesS * kRowsA * (S * kSuperK / 2 + 4) * 4 +
           16 * (kWavesS / KSW) * RBW * ((RAW ? kMaxK / kSuperK : kMaxK / 32) + 2) * 2;
}
template <int S, int KSW, int RBW, bool RAW>
constexpr int stream_waves()
{
    return RBW <= 4 && 2 * (stream_lds_bytes<S, KSW, RBW, RAW>() + 1024) <= 160 * 1024 ? 4 : 2;
}

// RF (route first, for layers with more experts than routes): a workgroup
// learns whether anyone selected its expert before it requests any weight
// byte, so unselected experts cost no HBM traffic; otherwise the weights are
// requested first and routing overlaps their latency.
template <int DT, int BITS, bool FC1, int S, int KSW, int RBW, int AR, bool GR, bool RAW, bool RF>
__global__ __launch_bounds__(kThreadsS, (stream_waves<S, KSW, RBW, RAW>())) void stream_kernel(ProjLaunch p, DecodePlan q)
{
    constexpr int RW = kWavesS / KSW;              // wavefronts along the rows
    constexpr int kBlocksWG = RW * RBW;            // 16-row weight blocks per workgroup
    constexpr int kRowsWG = 16 * kBlocksWG;
    constexpr int kEarly = (RBW + 1) / 2;          // row blocks requested before the rows are known
    constexpr int kSliceK = S * kSuperK;           // inputs of a K slice
    constexpr int kSliceB = kSliceK * BITS / 8;    // bytes of a weight row in a K slice: 32, 64 or 128
    constexpr int kAPitch = kSliceK / 2 + 4;       // A region row pitch in words (row r: bank 4r)
    constexpr int kAWords = kRowsA * kAPitch;      // A region of a wavefront
    constexpr int kARowsPerLoad = 512 / kSliceK;   // A rows one load instruction covers
    constexpr int kALoads = AR / kARowsPerLoad;    // 16-byte A loads per lane: AR rows (8 or 16)
    constexpr int kScBlocks = RAW ? kMaxK / kSuperK : kMaxK / 32;  // scale blocks per row at most
    constexpr int kScPitch = kScBlocks + 2;        // scale table row pitch in uint16 (odd word count)
    constexpr int kScUnits = (kRowsWG * kScBlocks / 8 + kThreadsS - 1) / kThreadsS;  // 16-byte units per thread
    constexpr Order O = RAW ? raw_order<BITS>() : code_order<DT, BITS>();
    static_assert(BITS == 2 || BITS == 4, "spans of whole 32-bit words");
    static_assert(kSliceB == 32 || kSliceB == 64 || kSliceB == 128, "K slice of a weight row");
    static_assert(RBW * 256 <= kAWords, "partial tiles fit the wavefront's A region");
    // per wavefront: its A slice [16][kAPitch] words, later its partial
    // tiles [RBW][16 MFMA rows][16 columns] float32
    __shared__ __attribute__((aligned(16))) uint32_t a_reg[kWavesS][kAWords];
    __shared__ __attribute__((aligned(16))) uint16_t sc_tab[kRowsWG * kScPitch];
    __shared__ int s_e[kMaxRoutesS];  // fc1: expert of route r
    __shared__ int s_route[kRowsA];   // fc2: route id of the expert's row m
    static_assert(sizeof(a_reg) + sizeof(sc_tab) == stream_lds_bytes<S, KSW, RBW, RAW>(), "LDS estimate");

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int c = lane & 15;
    const int kw = wave % KSW;  // the wavefront's K slice
    const int rw = wave / KSW;  // its row blocks
    const int K = p.K;
    const int k0 = kw * kSliceK;  // first input of the slice
    const int bs_shift = __builtin_ctz((unsigned)p.block_size);  // a power of two
    const int n_blocks = K >> bs_shift;
    const int nt = p.N / kRowsWG;
    const int e = blockIdx.x / nt;
    const int n = blockIdx.x - e * nt;
    const int row_bytes = K * BITS / 8;
    const int wr0 = n * kRowsWG + 16 * RBW * rw;  // first weight row of the wavefront within the expert
    uint32_t magic[4];  // RAW: per-register bases
#pragma unroll
    for (int r = 0; r < 4; ++r) magic[r] = opaque(raw_magic<DT, BITS>(r));
    const float zp = held(p.w.zp_fallback);
    const int act = held(p.act);
    uint16_t* const act_out = held(reinterpret_cast<uint16_t*>(p.act_out));
    float* const y2 = held(p.y2);
    uint32_t* const a_mine = a_reg[wave];

    // Every load below is issued unconditionally (indices clamped): a load
    // under a branch leaves its register undefined on the other path, and the
    // compiler then waits for it on the spot.
    // 0) fc1: router logits (GR: lane 16i + j holds expert j of token
    //    4 wave + i; otherwise tokens wave and wave + 8, expert lane);
    //    fc2: the expert's offsets
    constexpr int kLg = GR ? 1 : kTokW;
    float lg[kLg];
    int first = 0, count = 0;
    if constexpr (FC1) {
#pragma unroll
        for (int j = 0; j < kLg; ++j) {
            const int t = min(GR ? kGroupTok * wave + (lane >> 4) : wave + kWavesS * j, q.T - 1);
            lg[j] = q.logits[(int64_t)t * q.E + min(GR ? (lane & 15) : lane, q.E - 1)];
        }
    } else {
        first = q.offsets[e];
        count = q.offsets[e + 1] - first;
    }
    __builtin_amdgcn_sched_barrier(0);

    // The A slice: load i of a lane reads row kARowsPerLoad * i + lane / (64 /
    // kARowsPerLoad), 16 contiguous bytes; rows past the last read zeros
    u32x4 araw[kALoads];
    auto load_a = [&](const void* base, int rows) {
        const __amdgpu_buffer_rsrc_t rs = bounded(base, (uint32_t)rows * (uint32_t)K * 2u);
        constexpr int kLanesPerRow = 64 / kARowsPerLoad;
        const int r_in = lane / kLanesPerRow, ch = lane % kLanesPerRow;
#pragma unroll
        for (int i = 0; i < kALoads; ++i) {
            const int r = kARowsPerLoad * i + r_in;
            const uint32_t off = r < rows ? (uint32_t)(r * K + k0 + 8 * ch) * 2u : 0x80000000u;
            araw[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
        }
    };
    auto store_a = [&]() {
        constexpr int kLanesPerRow = 64 / kARowsPerLoad;
        const int r_in = lane / kLanesPerRow, ch = lane % kLanesPerRow;
#pragma unroll
        for (int i = 0; i < kALoads; ++i)
            *reinterpret_cast<u32x4*>(a_mine + (kARowsPerLoad * i + r_in) * kAPitch + 4 * ch) = araw[i];
    };
    // 1) fc1: the A slice (the tokens, known before routing)
    if constexpr (FC1) load_a(p.a, q.T);
    __builtin_amdgcn_sched_barrier(0);

    // 2) the scale rows of the workgroup's weight rows: one contiguous block
    //    of kRowsWG * n_blocks values, 16-byte units of 8 blocks
    const uint16_t* sc_src =
        reinterpret_cast<const uint16_t*>(p.w.scales) + ((int64_t)e * p.N + n * kRowsWG) * n_blocks;
    const int upr = n_blocks >> 3;  // units per row (n_blocks is a multiple of 8)
    const int n_units = kRowsWG * upr;
    u32x4 sc_unit[kScUnits];
    auto load_scales = [&]() {
#pragma unroll
        for (int k = 0; k < kScUnits; ++k) {
            const int u = min(tid + kThreadsS * k, n_units - 1);
            sc_unit[k] = *reinterpret_cast<const u32x4*>(sc_src + 8 * u);
        }
    };

    // weight row block rb: lane (g, c) reads bytes [16g, 16g+16) of row
    // wr0 + 16 rb + c's slice (and [64+16g, ...) for a 128-byte slice; a
    // 32-byte slice: bytes [8g, 8g+8), the span itself)
    constexpr int kWLoads = kSliceB == 128 ? 2 : 1;
    typedef typename std::conditional<kSliceB == 32, uint2, u32x4>::type WLoad;
    WLoad wraw[RBW][kWLoads];
    const uint8_t* w_row = p.w.codes + ((int64_t)e * p.N + wr0 + c) * row_bytes + (k0 * BITS / 8);
    auto load_w = [&](int rb) {
#pragma unroll
        for (int i = 0; i < kWLoads; ++i)
            wraw[rb][i] = *reinterpret_cast<const WLoad*>(w_row + rb * 16 * row_bytes + 64 * i +
                                                          (kSliceB == 32 ? 8 : 16) * g);
    };

    auto store_scales = [&]() {
#pragma unroll
        for (int k = 0; k < kScUnits; ++k) {
            const int u = tid + kThreadsS * k;
            if (u < n_units) {
                const int r = u / upr;
                uint32_t* dst = reinterpret_cast<uint32_t*>(sc_tab + r * kScPitch + 8 * (u - r * upr));
                dst[0] = sc_unit[k].x;
                dst[1] = sc_unit[k].y;
                dst[2] = sc_unit[k].z;
                dst[3] = sc_unit[k].w;
            }
        }
    };

    // 3) fc1: route every token (GR: four tokens per wavefront, so the first
    //    T / 4 wavefronts route; otherwise one wavefront per token); the
    //    other wavefronts go on to their A fragments
    auto route_all = [&]() {
        if constexpr (FC1) {
            const bool writer = blockIdx.x == 0;
            // the fc2 launch's column-block counters start at zero
            if (writer && tid < q.n_counters) {
                __hip_atomic_store(&q.counters[tid], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            auto emit_for = [&](int t) {
                return [&, t](int slot, int ex, float w) {
                    if (t >= q.T) return;
                    const int r = t * p.top_k + slot;
                    s_e[r] = ex;
                    if (writer) {
                        q.weights[r] = w;
                        if (q.ids_out) q.ids_out[r] = ex;
                        if (q.w_out) q.w_out[r] = w;
                    }
                };
            };
            if constexpr (GR) {
                if (kGroupTok * wave < q.T) {
                    route_group<16>(q.E, p.top_k, q.normalize, lg[0], emit_for(kGroupTok * wave + (lane >> 4)));
                }
            } else {
#pragma unroll
                for (int j = 0; j < kTokW; ++j) {
                    const int t = wave + kWavesS * j;
                    if (t >= q.T) break;
                    route_values<1>(q.E, p.top_k, q.normalize, [&](int) { return lg[j]; }, emit_for(t));
                }
            }
        }
    };
    // 5) fc1: this expert's routes (route r of token r / top_k) as masks over
    //    the R <= 64 routes, the first sorted position and the route count.
    //    The first workgroup writes every expert's offsets and sorted routes
    //    for fc2 and the combine (also when its own expert has none); then a
    //    workgroup whose expert nobody selected leaves.
    uint64_t mine = 0;
    auto rank_and_write = [&]() {
        if constexpr (FC1) {
            const int R = q.T * p.top_k;
            const int ex = lane < R ? s_e[lane] : -1;
            mine = __ballot(ex == e);
            first = __popcll(__ballot(lane < R && ex < e));
            count = __popcll(mine);
            // the writer writes before it may leave: its own expert can have no routes
            if (blockIdx.x == 0 && wave == 0) {
                if (lane < R) {
                    int less = 0, same_before = 0;
                    for (int r = 0; r < R; ++r) {
                        const int o = s_e[r];
                        less += o < ex;
                        same_before += (o == ex) & (r < lane);
                    }
                    q.sorted[less + same_before] = lane;
                }
                if (lane < q.E) {
                    int less = 0;
                    for (int r = 0; r < R; ++r) less += s_e[r] < lane;
                    q.offsets[lane] = less;
                }
                if (lane == 0) q.offsets[q.E] = R;
            }
        }
    };
    // fc2: an expert with no rows arrives on the column block only
    auto fc2_leave = [&]() {
        if constexpr (!FC1) {
            if (p.fused.counters) fc2_arrive_combine<DT>(p.fused, y2, p.N, p.top_k, n, n * kRowsWG, kRowsWG, q.E);
        }
    };

    if constexpr (RF) {  // routes and ranks before the first weight request
        if constexpr (FC1) {
            route_all();
            sync_lds();
            rank_and_write();
        }
        if (count == 0) {  // whole workgroup
            fc2_leave();
            return;
        }
    }
    load_scales();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rb = 0; rb < kEarly; ++rb) load_w(rb);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!RF) {
        if constexpr (FC1) {
            route_all();
        } else if (count == 0) {
            fc2_leave();
            return;
        }
    }

    // 4) fc2: the expert's route ids and rows (sorted activations); both: the
    //    rest of the weight row blocks, then the scale table (its barrier waits
    //    for LDS only)
    int my_route = 0;
    if constexpr (!FC1) {
        my_route = q.sorted[first + min(c, count - 1)];
        load_a(reinterpret_cast<const uint16_t*>(p.a) + (int64_t)first * K, count);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rb = kEarly; rb < RBW; ++rb) load_w(rb);
    __builtin_amdgcn_sched_barrier(0);
    store_scales();
    sync_lds();

    if constexpr (FC1 && !RF) {
        rank_and_write();
        if (count == 0) return;  // whole workgroup; its loads drain on their own
    }

    // 6) A fragments through the wavefront's own LDS region (no other
    //    wavefront reads it) into the MFMA register order; RAW: the
    //    corrections of MFMA rows 4g..4g+3 per super-step,
    //    -sum_k (b_r(k) + zp) a_k, from the lane's per-register sums (v_dot2
    //    with ones), added over the four lane groups
    store_a();
    u32x4 afr[S][4];
    f32x4 corr[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        uint32_t in[16], out[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(a_mine + c * kAPitch + 64 * s + 16 * g + 4 * i);
            in[4 * i + 0] = v.x;
            in[4 * i + 1] = v.y;
            in[4 * i + 2] = v.z;
            in[4 * i + 3] = v.w;
        }
        permute_span<O>(in, out);
#pragma unroll
        for (int t = 0; t < 4; ++t) afr[s][t] = u32x4{out[4 * t], out[4 * t + 1], out[4 * t + 2], out[4 * t + 3]};
        if constexpr (RAW) {
            float part = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float cls = 0.f;
#pragma unroll
                for (int t = 0; t < 4; ++t) cls = dot2_sum<DT>(out[4 * t + r], cls);
                part += -(raw_base<DT, BITS>(r) + zp) * cls;
            }
            part += __shfl_xor(part, 16);
            part += __shfl_xor(part, 32);
#pragma unroll
            for (int i = 0; i < 4; ++i) corr[s][i] = __shfl(part, 4 * g + i);
        }
    }

    // 7) the row blocks in order, each as soon as its bytes land
    const uint16_t* sc_mine = sc_tab + (16 * RBW * rw + c) * kScPitch;
    f32x4 acc[RBW];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
        Span<BITS> spn[S];
        if constexpr (kSliceB == 32) {
            spn[0].w[0] = wraw[rb][0].x;
            spn[0].w[1] = wraw[rb][0].y;
        } else if constexpr (BITS == 2) {
            spans_of_slice(wraw[rb][0], spn[0], spn[1]);
        } else {
#pragma unroll
            for (int s = 0; s < S; ++s)
#pragma unroll
                for (int d = 0; d < 4; ++d) spn[s].w[d] = wraw[rb][s][d];
        }
        acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int blk = (k0 + kSuperK * s + (RAW ? 0 : 32 * g)) >> bs_shift;
            const float scale = Dt<DT>::to_float(sc_mine[rb * 16 * kScPitch + blk]);
            if constexpr (RAW) {
                f32x4 part = corr[s];
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    part = Dt<DT>::mfma(afr[s][t], raw_step_based<DT, BITS>(spn[s], t, magic), part);
                acc[rb] += part * scale;
            } else {
                BlockParams bq;
                bq.zp = zp;
                bq.scale = scale;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    acc[rb] = Dt<DT>::mfma(afr[s][t], dequant_zp<DT, BITS, kZpConst>(spn[s], t, bq), acc[rb]);
            }
        }
        // row block rb + 1's unpacking may not be hoisted above this block's
        // MFMAs: it would wait for bytes that arrive later
        __builtin_amdgcn_sched_barrier(0);
    }

    // 8) partial tiles over the wavefront's own A region (its fragment reads
    //    are done: LDS accesses of a wavefront complete in order): lane (g, c)
    //    holds MFMA rows 4g..4g+3 of column c
    float* const part_mine = reinterpret_cast<float*>(a_mine);
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) part_mine[(rb * kRowsA + 4 * g + i) * 16 + c] = acc[rb][i];
    if constexpr (!FC1) {
        if (wave == 0 && lane < kRowsA) s_route[lane] = my_route;
    }
    sync_lds();

    // 9) epilogue: sums over the K slices in slice order; row block b of the
    //    workgroup belongs to wavefronts rw = b / RBW (block b % RBW)
    auto partial = [&](int k, int b, int m, int col) -> const float* {
        return reinterpret_cast<const float*>(a_reg[(b / RBW) * KSW + k]) + ((b % RBW) * kRowsA + m) * 16 + col;
    };
    if constexpr (FC1) {
        // weight rows 2j (gate) and 2j+1 (up) of activation column j
        constexpr int kCols = kRowsWG / 2;
        const int I = p.N / 2;
        for (int i = tid; i < kRowsA * kCols; i += kThreadsS) {
            const int m = i / kCols;
            const int j = i - m * kCols;
            // token m's route to this expert: the set bit of `mine` among its
            // top_k routes; its sorted position counts the expert's earlier routes
            if (m >= q.T) break;
            const uint64_t slots = (mine >> (m * p.top_k)) & ((p.top_k >= 64 ? 0ull : (1ull << p.top_k)) - 1ull);
            if (slots == 0) continue;
            const int r = m * p.top_k + __builtin_ctzll(slots);
            const int pos = first + __popcll(mine & ((1ull << r) - 1ull));
            float gate = 0.f, up = 0.f;
#pragma unroll
            for (int k = 0; k < KSW; ++k) {
                const float2 v = *reinterpret_cast<const float2*>(partial(k, (2 * j) >> 4, m, (2 * j) & 15));
                gate += v.x;
                up += v.y;
            }
            act_out[(int64_t)pos * I + n * kCols + j] = Dt<DT>::from_float(act_value<DT>(act, gate, up, p.ap));
        }
    } else {
        const bool through = p.fused.counters != nullptr;
        for (int i = tid; i < count * kRowsWG; i += kThreadsS) {
            const int m = i / kRowsWG;
            const int r = i - m * kRowsWG;
            float v = 0.f;
#pragma unroll
            for (int k = 0; k < KSW; ++k) v += *partial(k, r >> 4, m, r & 15);
            store_y2(&y2[(int64_t)s_route[m] * p.N + n * kRowsWG + r], v, through);
        }
        if (through) fc2_arrive_combine<DT>(p.fused, y2, p.N, p.top_k, n, n * kRowsWG, kRowsWG, q.E);
    }
}

template <int DT, int BITS, bool FC1, int S, int KSW, int RBW, int AR, bool GR, bool RAW>
void launch_rf(bool rf, dim3 grid, hipStream_t s, const ProjLaunch& p, const DecodePlan& plan)
{
    if (rf) launch(stream_kernel<DT, BITS, FC1, S, KSW, RBW, AR, GR, RAW, true>, grid, dim3(kThreadsS), s, p, plan);
    else launch(stream_kernel<DT, BITS, FC1, S, KSW, RBW, AR, GR, RAW, false>, grid, dim3(kThreadsS), s, p, plan);
}

// K slices of 64 bytes per weight row (32 at one 2-bit super-step, 128 at
// 4 bits over 2048 inputs): super-steps per wavefront S and wavefronts per
// row KSW (KSW * S = K / 128); row blocks per wavefront so that a workgroup
// holds 64 weight rows (128 with one wavefront per row).
template <bool FC1, int DT, int BITS, bool RAW, int S, int KSW>
hipError_t run(const ProjLaunch& p, const DecodePlan& plan, hipStream_t s)
{
    constexpr int RBW = KSW >= 2 ? KSW / 2 : 1;
    constexpr int kRowsWG = 16 * (kWavesS / KSW) * RBW;
    if (p.N % kRowsWG) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(plan.E * (p.N / kRowsWG)));
    // A rows: an expert has at most T rows; fc1 routes four tokens per
    // wavefront when every expert fits 16 lanes
    const bool group = FC1 && plan.E <= 16;
    // route first when some experts must go unselected
    const bool rf = plan.E > plan.T * p.top_k;
    if (plan.T <= 8) {
        if (group) launch_rf<DT, BITS, FC1, S, KSW, RBW, 8, FC1, RAW>(rf, grid, s, p, plan);
        else launch_rf<DT, BITS, FC1, S, KSW, RBW, 8, false, RAW>(rf, grid, s, p, plan);
    } else {
        if (group) launch_rf<DT, BITS, FC1, S, KSW, RBW, 16, FC1, RAW>(rf, grid, s, p, plan);
        else launch_rf<DT, BITS, FC1, S, KSW, RBW, 16, false, RAW>(rf, grid, s, p, plan);
    }
    return hipGetLastError();
}

template <bool FC1, int DT, int BITS, bool RAW>
hipError_t launch_slices(const ProjLaunch& p, const DecodePlan& plan, hipStream_t s)
{
    const int supers = p.K / kSuperK;
    if constexpr (BITS == 2) {
        switch (supers) {
        case 1: return run<FC1, DT, BITS, RAW, 1, 1>(p, plan, s);
        case 2: return run<FC1, DT, BITS, RAW, 2, 1>(p, plan, s);
        case 4: return run<FC1, DT, BITS, RAW, 2, 2>(p, plan, s);
        case 8: return run<FC1, DT, BITS, RAW, 2, 4>(p, plan, s);
        case 16: return run<FC1, DT, BITS, RAW, 2, 8>(p, plan, s);
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (supers) {
        case 1: return run<FC1, DT, BITS, RAW, 1, 1>(p, plan, s);
        case 2: return run<FC1, DT, BITS, RAW, 1, 2>(p, plan, s);
        case 4: return run<FC1, DT, BITS, RAW, 1, 4>(p, plan, s);
        case 8: return run<FC1, DT, BITS, RAW, 1, 8>(p, plan, s);
        case 16: return run<FC1, DT, BITS, RAW, 2, 8>(p, plan, s);
        default: return hipErrorInvalidValue;
        }
    }
}

template <bool FC1, int DT>
hipError_t launch_stream(const ProjLaunch& p, const DecodePlan& plan, hipStream_t s)
{
    if (!stream_fits(p.w, p.K, p.N, p.block_size, FC1)) return hipErrorInvalidValue;
    const bool raw = p.block_size % kSuperK == 0;
    if (p.w.bits == 2) {
        return raw ? launch_slices<FC1, DT, 2, true>(p, plan, s) : launch_slices<FC1, DT, 2, false>(p, plan, s);
    }
    return raw ? launch_slices<FC1, DT, 4, true>(p, plan, s) : launch_slices<FC1, DT, 4, false>(p, plan, s);
}

}  // namespace

bool stream_fits(const ProjArgs& w, int K, int N, int block_size, bool fc1)
{
    (void)fc1;
    const int bs = block_size;
    const int supers = K / kSuperK;
    // whole 8-block scale units per row (16-byte aligned) for the scale table
    return (w.bits == 2 || w.bits == 4) && w.zp == nullptr && K <= kMaxK && K % kSuperK == 0 &&
           (supers & (supers - 1)) == 0 && N % 128 == 0 && bs >= 32 && (bs & (bs - 1)) == 0 &&
           (K / bs) % 8 == 0 && reinterpret_cast<uintptr_t>(w.scales) % 16 == 0 &&
           (bs % kSuperK == 0 || w.fast);  // RAW takes any constant zero point
}

hipError_t launch_fc1_stream(const ProjLaunch& p, const DecodePlan& plan, int dtype, hipStream_t s)
{
    if (plan.T > kRowsA || plan.T * p.top_k > kMaxRoutesS || plan.E > kWave) return hipErrorInvalidValue;
    return dtype == kBF16 ? launch_stream<true, kBF16>(p, plan, s) : launch_stream<true, kF16>(p, plan, s);
}

hipError_t launch_fc2_stream(const ProjLaunch& p, const DecodePlan& plan, int dtype, hipStream_t s)
{
    // an expert holds at most one route per token, so at most T rows
    if (plan.T > kRowsA) return hipErrorInvalidValue;
    return dtype == kBF16 ? launch_stream<false, kBF16>(p, plan, s) : launch_stream<false, kF16>(p, plan, s);
}

}  // namespace qmoe
