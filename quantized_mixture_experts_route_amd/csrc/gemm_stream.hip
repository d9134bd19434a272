// gemm_stream.hip -- decode projections that stream every selected expert's
// packed weights and consume them piece by piece as they land.
//
// [PR 33569: the decode path serves small expanded-row counts, and its time
// is set by the packed-weight bytes; qmoe.rs QMoEKernel::execute: route,
// group, fc1 + activation, fc2, combine.]  With at most 16 tokens (and
// R = T*top_k <= 64 routes) every selected expert's weights are read once and
// multiplied with at most 16 rows (a token routes to an expert at most once),
// so a projection costs the time to stream its bytes plus the work left once
// the last of them arrives.  One workgroup of eight wavefronts per
// (expert, block of weight rows); wavefront w owns one block of 16 contiguous
// weight rows and a 1/KS share of K.  fc1 (KS = 1): 128 rows per workgroup,
// the 16 rows of a wavefront are 8 gate/up pairs, gate in MFMA columns 0-7
// and up in 8-15, paired in the epilogue by a DPP rotate, so nothing is
// reduced across wavefronts.  fc2 (KS = 2 when K allows): 64 rows per
// workgroup and two wavefronts per block, whose partial sums meet once in LDS.
//
// Order: fc1 loads the router logits of the wavefront's tokens, fc2 the
// expert's offsets and route ids; then the scale table of the workgroup's
// rows, one A row per wavefront (fc1 the tokens, all of them, since routing
// is not known yet; fc2 the expert's rows) and the first two weight pieces of
// the wavefront's block (one piece: one 128-byte line of each of its 16 rows,
// eight whole lines per load instruction).  The workgroup's shared work
// comes next: fc1 routes every token (the first workgroup writes the routing
// weights, expert offsets and sorted routes for fc2 and the combine), and A,
// its per-super-step corrections and the scales go to LDS.  Then each
// wavefront requests the rest of its pieces and waits for no other wavefront
// until fc2's two K shares meet at the end: requests are accepted only as
// fast as earlier data returns, so a workgroup barrier after them would hold
// every wavefront until the slowest had issued.  vmcnt retires loads in issue
// order, so each wait names exactly its own loads (and an L2 hit issued after
// the weight misses would wait for them: the small loads go first).  Piece j
// is consumed as soon as it lands: copied to a wavefront-private LDS slot,
// read back as MFMA spans, and multiplied with the A fragments of its
// super-steps, whose MFMA chains are interleaved.  Scheduling barriers keep
// the load groups in this order.
//
// MFMA mapping and dequantization are those of the other projection kernels:
// lane 16g + c feeds A row c (a routed row; zeros past the expert's rows,
// without reading LDS) and weight column c of the block, lane group g the inputs
// [32g, 32g+32) of each 128-input super-step in the code order of the dequant
// routines.  RAW (block_size a multiple of 128): the B registers are the raw
// codes made exact dtype values by one v_and_or_b32 each, with a base b_r per
// register r chosen so that the code's bits, where they already sit in the
// packed word (or nearly), weigh 1 (fp16 int2: 1024, 256, 64, 16; int4: 1024
// and 64), which saves most of the shifts that would bring every code down to
// bit 0.  The zero point and the bases are taken out per
// super-step in float32: sum_k (q_k - zp) a_k = mfma(a, b_r + q) -
// sum_k (b_r(k) + zp) a_k, the last sum formed once per A row and super-step
// while A is staged; the scale multiplies the difference.  Otherwise each
// weight is dequantized in registers with a constant zero point.
#include "gemm_common.h"
#include "route_common.h"

namespace qmoe {
namespace {

constexpr int kWavesS = 8;
constexpr int kThreadsS = kWavesS * kWave;
constexpr int kRowsA = 16;                   // A tile rows: tokens (fc1) or expert rows (fc2)
constexpr int kMaxK = 2048;
constexpr int kMaxSuper = kMaxK / kSuperK;
constexpr int kPitchA = kMaxK / 2 + 4;       // A tile row pitch in 32-bit words (row r: bank 4r)
constexpr int kLine = 128;                   // bytes of each weight row per piece
constexpr int kSlotPitch = kLine + 16;       // LDS slot row pitch: 36 words, 16 rows on distinct banks
constexpr int kMaxBlocks = 64;               // quantization blocks per row (K / block_size)
constexpr int kScPitch = kMaxBlocks + 4;     // scale table row pitch in uint16 (rows 8-byte aligned)
constexpr int kScUnits = 2;                  // 16-byte scale units per thread at most (128 rows x 8)
constexpr int kTokW = kRowsA / kWavesS;      // tokens each wavefront routes (T <= 16)
constexpr int kMaxRoutesS = kWave;           // routes (T * top_k), one per lane of wavefront 0
constexpr int kDppRor8 = 0x128;              // DPP row_ror:8: lane c reads lane c ^ 8 of its row

// A kernel argument held in SGPRs from here on: the compiler may otherwise
// fetch it again where it is used, and a fetch issued after the weight
// loads waits behind them.
template <class T>
__device__ inline T held(T v)
{
    asm volatile("" : "+s"(v));
    return v;
}

// The piece loop of the streamed projections.  Piece j of bv (load i: rows
// 8i + lane/8 of the 16-row block, 16 bytes at 16*(lane%8) of the piece)
// lands in the wavefront's LDS slot, row r at slot row slot_of(r); then its
// SPP super-steps run as independent MFMA chains.  a_row: this lane's A row
// (row_ok: a real one); sc_row: the scale table row of MFMA column c;
// corr(S): the RAW corrections of MFMA rows 4g..4g+3 at super-step S (s0 +
// local index).  Lanes past the real rows keep stale A fragments, which reach
// only MFMA rows that are never stored; a skipped super-step (past the K
// share) keeps them too and is cancelled by a zero scale.  Returns the sum of
// the chains.
template <int DT, int BITS, int P, bool RAW, class SlotOf, class Corr>
__device__ inline f32x4 consume_pieces(const u32x4 (&bv)[P][2], uint8_t* slot, SlotOf slot_of,
                                       const uint32_t* a_row, bool row_ok, const uint16_t* sc_row,
                                       Corr corr, int s0, int n_super, int bs_shift, float zp,
                                       const uint32_t (&magic)[4])
{
    constexpr int SPP = kLine * 8 / BITS / kSuperK;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int c = lane & 15;
    const int lrow = lane >> 3;
    const int lbyte = 16 * (lane & 7);
    f32x4 acc[SPP];
#pragma unroll
    for (int sp = 0; sp < SPP; ++sp) acc[sp] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 a4[SPP][4];
#pragma unroll
    for (int sp = 0; sp < SPP; ++sp)
#pragma unroll
        for (int t = 0; t < 4; ++t) a4[sp][t] = u32x4{0u, 0u, 0u, 0u};

#pragma unroll
    for (int j = 0; j < P; ++j) {
        if (j * SPP >= n_super) break;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            *reinterpret_cast<u32x4*>(slot + slot_of(8 * i + lrow) * kSlotPitch + lbyte) = bv[j][i];
        }
        // gather the piece: A fragments, spans, corrections and scales
        Span<BITS> spn[SPP];
        f32x4 rs[SPP];
        float scl[SPP];
#pragma unroll
        for (int sp = 0; sp < SPP; ++sp) {
            const int s = j * SPP + sp;
            const bool ok = s < n_super;  // uniform
            const int S = s0 + min(s, n_super - 1);  // the super-step in K
            if (ok && row_ok) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    a4[sp][t] = *reinterpret_cast<const u32x4*>(a_row + (S * kSuperK + 32 * g) / 2 + 4 * t);
                }
            }
            spn[sp] = load_span<BITS>(slot + c * kSlotPitch, sp * kSuperK + 32 * g);
            const float sv = Dt<DT>::to_float(sc_row[(S * kSuperK + (RAW ? 0 : 32 * g)) >> bs_shift]);
            scl[sp] = ok ? sv : 0.f;
            if constexpr (RAW) rs[sp] = corr(S);
        }
        if constexpr (RAW) {
            f32x4 part[SPP];
#pragma unroll
            for (int sp = 0; sp < SPP; ++sp) part[sp] = rs[sp];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int sp = 0; sp < SPP; ++sp)
                    part[sp] = Dt<DT>::mfma(a4[sp][t], raw_step_based<DT, BITS>(spn[sp], t, magic), part[sp]);
#pragma unroll
            for (int sp = 0; sp < SPP; ++sp) acc[sp] += part[sp] * scl[sp];
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int sp = 0; sp < SPP; ++sp) {
                    BlockParams bq;
                    bq.zp = zp;
                    bq.scale = scl[sp];
                    acc[sp] = Dt<DT>::mfma(a4[sp][t], dequant_zp<DT, BITS, kZpConst>(spn[sp], t, bq), acc[sp]);
                }
        }
    }
    f32x4 sum = acc[0];
#pragma unroll
    for (int sp = 1; sp < SPP; ++sp) sum += acc[sp];
    return sum;
}

// The A staging of the streamed projections: one A row of 16-byte chunks
// (chunk lane + 64*qq), permuted to the MFMA register order (int2 pairs the
// chunks of lanes l and l^1, both in the same row) into LDS row `dst`, and
// for RAW the row's per-super-step corrections -sum (b_r + zp) a (16 lanes
// hold one super-step) stored through put(super-step, value).
template <int DT, int BITS, bool RAW, class Put>
__device__ inline void stage_a_row(const u32x4 (&av)[4], bool valid, int cpr, uint32_t* dst, float zp, Put put)
{
    constexpr Order O = RAW ? raw_order<BITS>() : code_order<DT, BITS>();
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
        const int ch = lane + kWave * qq;
        u32x4 v;
        if constexpr (O == Order::kStride8) v = permute_chunk_pair(av[qq], lane & 1);
        else v = permute_chunk<O>(av[qq]);
        if constexpr (RAW) {
            float part = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float coef = -(raw_base<DT, BITS>(r) + zp);
                part += coef * Dt<DT>::to_float((uint16_t)(v[r] & 0xffffu));
                part += coef * Dt<DT>::to_float((uint16_t)(v[r] >> 16));
            }
            part += dpp_f32<kDppXor1>(part);
            part += dpp_f32<kDppXor2>(part);
            part += dpp_f32<kDppHalfMirror>(part);
            part += dpp_f32<kDppMirror>(part);
            if (valid && ch < cpr && (lane & 15) == 0) put(ch >> 4, part);
        }
        if (valid && ch < cpr) *reinterpret_cast<u32x4*>(dst + 4 * ch) = v;
    }
}

template <int DT, int BITS, bool FC1, int KS, int P, bool RAW>
__global__ __launch_bounds__(kThreadsS, 1) void stream_kernel(ProjLaunch p, DecodePlan q)
{
    constexpr int kBlocksWG = kWavesS / KS;             // 16-row weight blocks per workgroup
    constexpr int kRowsWG = 16 * kBlocksWG;             // weight rows per workgroup
    constexpr int kEarly = P < 2 ? P : 2;               // pieces requested before the shared work
    static_assert(BITS == 2 || BITS == 4, "a 128-byte line holds whole super-steps");
    static_assert(!FC1 || KS == 1, "fc1 pairs gate and up columns within one wavefront");
    __shared__ __attribute__((aligned(16))) uint32_t a_tile[kRowsA * kPitchA];
    __shared__ __attribute__((aligned(16))) uint8_t b_slot[kWavesS][16 * kSlotPitch];
    __shared__ __attribute__((aligned(16))) uint16_t sc_tab[kRowsWG * kScPitch];
    __shared__ float a_sum[kRowsA][kMaxSuper];  // RAW: -sum (b_r + zp) a of A row m over super-step s
    __shared__ __attribute__((aligned(16))) float m_sum[kMaxSuper][kRowsA];  // RAW: the same by MFMA row
    __shared__ __attribute__((aligned(16))) float red[KS == 2 ? kBlocksWG * kWave * 4 : 4];
    __shared__ int s_e[kMaxRoutesS];  // fc1: expert of route r
    __shared__ int s_arow[kRowsA];  // fc1: A tile row (token) of the expert's m-th route
    __shared__ int s_info[2];       // fc1: first sorted position, route count

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int c = lane & 15;
    const int rb = wave % kBlocksWG;  // the wavefront's weight row block
    const int kp = wave / kBlocksWG;  // its share of K
    const int K = p.K;
    const int KW = K / KS;            // inputs per wavefront
    const int s0 = kp * (KW / kSuperK);  // its first super-step
    const int n_super = KW / kSuperK;
    const int n_blocks = K / p.block_size;
    const int bs_shift = __builtin_ctz((unsigned)p.block_size);  // a power of two
    const int nt = p.N / kRowsWG;
    const int e = blockIdx.x / nt;
    const int n = blockIdx.x - e * nt;
    const int row_bytes = K * BITS / 8;
    const int wr0 = n * kRowsWG + 16 * rb;  // first weight row of the block within the expert
    const int col0 = FC1 ? wr0 / 2 : wr0;   // first output column (fc1: 8 activation columns)
    const uint16_t* a_src = reinterpret_cast<const uint16_t*>(p.a);
    uint32_t magic[4];  // RAW: per-register bases
#pragma unroll
    for (int r = 0; r < 4; ++r) magic[r] = opaque(raw_magic<DT, BITS>(r));
    const float zp = held(p.w.zp_fallback);
    const int act = held(p.act);
    uint16_t* const act_out = held(reinterpret_cast<uint16_t*>(p.act_out));
    float* const y2 = held(p.y2);

    // Every load below is issued unconditionally (indices clamped): a load
    // under a branch leaves its register undefined on the other path, and the
    // compiler then waits for it on the spot.
    // 0) fc1: router logits of tokens wave and wave + 8; fc2: the expert's
    //    rows in the sorted order (written by fc1) and their route ids
    float lg[kTokW];
    int first = 0, count = 0;
    int y2_row[4] = {0, 0, 0, 0};  // fc2: route ids of rows 4g..4g+3 (clamped)
    if constexpr (FC1) {
#pragma unroll
        for (int j = 0; j < kTokW; ++j) {
            const int t = min(wave + kWavesS * j, q.T - 1);
            lg[j] = q.logits[(int64_t)t * q.E + min(lane, q.E - 1)];
        }
    } else {
        first = q.offsets[e];
        count = q.offsets[e + 1] - first;
        if (count == 0) {  // no rows of this expert: arrive on the column block only
            if (p.fused.counters) fc2_arrive_combine<DT>(p.fused, y2, p.N, p.top_k, n, n * kRowsWG, kRowsWG, q.E);
            return;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) y2_row[i] = q.sorted[first + min(4 * g + i, count - 1)];
    }
    __builtin_amdgcn_sched_barrier(0);

    // 1) scale table: 16-byte units of 8 blocks, row-major over the workgroup's rows
    const uint16_t* sc_src =
        reinterpret_cast<const uint16_t*>(p.w.scales) + ((int64_t)e * p.N + n * kRowsWG) * n_blocks;
    const int upr = n_blocks >> 3;  // units per row
    const int n_units = kRowsWG * upr;
    u32x4 sc_unit[kScUnits];
#pragma unroll
    for (int k = 0; k < kScUnits; ++k) {
        const int u = min(tid + kThreadsS * k, n_units - 1);
        const int r = u / upr;
        sc_unit[k] = *reinterpret_cast<const u32x4*>(sc_src + r * n_blocks + 8 * (u - r * upr));
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2) A row `wave` (rows 8.. are loaded when staged): 16-byte chunk
    //    lane + 64*qq, so each load reads whole lines
    const int a_rows = FC1 ? q.T : count;
    const int cpr = K / 8;  // 16-byte chunks per A row (a multiple of 16)
    u32x4 av[4];
    auto load_a = [&](int m) {
        const uint16_t* row = a_src + (int64_t)(FC1 ? min(m, a_rows - 1) : first + min(m, a_rows - 1)) * K;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            av[qq] = *reinterpret_cast<const u32x4*>(row + 8 * min(lane + kWave * qq, cpr - 1));
        }
    };
    load_a(wave);
    __builtin_amdgcn_sched_barrier(0);

    // 3) the first kEarly weight pieces of the wavefront: piece j, load i
    //    reads rows 8i + lane/8 of the block, bytes [128j + 16*(lane%8), +16)
    //    of its K share (clamped into the share past its end; those
    //    super-steps are skipped).  The rest follow once the workgroup's
    //    shared work is done.
    const int kb0 = s0 * kSuperK * BITS / 8;  // first byte of the share in a row
    const int kbw = KW * BITS / 8;            // bytes of the share
    const uint8_t* wcodes = p.w.codes + ((int64_t)e * p.N + wr0) * row_bytes + kb0;
    const int lrow = lane >> 3;
    const int lbyte = 16 * (lane & 7);
    u32x4 bv[P][2];
    auto load_piece = [&](int j) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int ob = min(kLine * j + lbyte, kbw - 16);
            bv[j][i] = *reinterpret_cast<const u32x4*>(wcodes + (8 * i + lrow) * row_bytes + ob);
        }
    };
#pragma unroll
    for (int j = 0; j < kEarly; ++j) load_piece(j);
    __builtin_amdgcn_sched_barrier(0);

    // 4) fc1: route every token; this expert's routes in ascending order,
    //    and their first sorted position
    if constexpr (FC1) {
        const int R = q.T * p.top_k;
        const bool writer = blockIdx.x == 0;
        // the fc2 launch's column-block counters start at zero
        if (writer && tid < q.n_counters) {
            __hip_atomic_store(&q.counters[tid], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int j = 0; j < kTokW; ++j) {
            const int t = wave + kWavesS * j;
            if (t >= q.T) break;
            route_values<1>(q.E, p.top_k, q.normalize, [&](int) { return lg[j]; },
                            [&](int slot, int ex, float w) {
                                const int r = t * p.top_k + slot;
                                s_e[r] = ex;
                                if (writer) {
                                    q.weights[r] = w;
                                    if (q.ids_out) q.ids_out[r] = ex;
                                    if (q.w_out) q.w_out[r] = w;
                                }
                            });
        }
        __syncthreads();
        if (wave == 0) {
            const int ex = lane < R ? s_e[lane] : -1;
            const uint64_t mine = __ballot(ex == e);
            const uint64_t below = __ballot(lane < R && ex < e);
            if (ex == e) s_arow[__popcll(mine & ((1ull << lane) - 1ull))] = lane / p.top_k;
            if (lane == 0) {
                s_info[0] = __popcll(below);
                s_info[1] = __popcll(mine);
            }
            if (writer) {  // offsets and sorted routes of every expert, for fc2 and the combine
                if (lane < R) {
                    int less = 0, same_before = 0;
                    for (int r = 0; r < R; ++r) {
                        const int o = s_e[r];
                        less += o < ex;
                        same_before += (o == ex) & (r < lane);
                    }
                    q.sorted[less + same_before] = lane;
                }
                // no loop around the stores: the compiler would drain every
                // load in flight before entering it
                if (lane < q.E) {
                    int less = 0;
                    for (int r = 0; r < R; ++r) less += s_e[r] < lane;
                    q.offsets[lane] = less;
                }
                if (lane == 0) q.offsets[q.E] = R;
            }
        }
        __syncthreads();
        first = s_info[0];
        count = s_info[1];
        if (count == 0) return;  // whole workgroup; its first pieces drain on their own
    }

    // 5) A tile (permuted to the MFMA register order; int2 pairs the chunks of
    //    lanes l and l^1, both in the same row), the row sums of its
    //    super-steps (RAW) and the scale table to LDS
    auto store_a = [&](int m) {
        stage_a_row<DT, BITS, RAW>(av, m < a_rows, cpr, a_tile + m * kPitchA, zp,
                                   [&](int sstep, float v) { a_sum[m][sstep] = v; });
    };
    store_a(wave);
    if (a_rows > kWavesS) {  // rows 8..15
        load_a(wave + kWavesS);
        store_a(wave + kWavesS);
    }
#pragma unroll
    for (int k = 0; k < kScUnits; ++k) {
        const int u = tid + kThreadsS * k;
        if (u < n_units) {
            const int r = u / upr;
            uint32_t* dst = reinterpret_cast<uint32_t*>(sc_tab + r * kScPitch + 8 * (u - r * upr));
            *reinterpret_cast<u32x2*>(dst) = u32x2{sc_unit[k].x, sc_unit[k].y};
            *reinterpret_cast<u32x2*>(dst + 2) = u32x2{sc_unit[k].z, sc_unit[k].w};
        }
    }
    __syncthreads();
    const bool row_ok = c < count;
    const int arow = row_ok ? (FC1 ? s_arow[c] : c) : 0;
    if constexpr (RAW) {  // corrections by MFMA row: m_sum[s][m] = a_sum[A row of route m][s]
        if (tid < kMaxSuper * kRowsA) {
            const int s = tid >> 4, m = tid & 15;
            m_sum[s][m] = m < count ? a_sum[FC1 ? s_arow[m] : m][s] : 0.f;
        }
        __syncthreads();
    }

    // 6) the rest of the wavefront's weight pieces
#pragma unroll
    for (int j = kEarly; j < P; ++j) load_piece(j);
    __builtin_amdgcn_sched_barrier(0);

    // 7) the pieces, each as soon as it lands
    const uint32_t* a_row = a_tile + arow * kPitchA;
    // MFMA column c of the block: fc1 gate row 2c (c < 8) or up row 2(c-8)+1,
    // stored in slot c; fc2 row c
    const int wrow = FC1 ? 2 * (c & 7) + (c >> 3) : c;
    const uint16_t* sc_row = sc_tab + (16 * rb + wrow) * kScPitch;
    uint8_t* slot = b_slot[wave];

    f32x4 sum = consume_pieces<DT, BITS, P, RAW>(
        bv, slot, [&](int row) { return FC1 ? (row >> 1) + 8 * (row & 1) : row; }, a_row, row_ok, sc_row,
        [&](int S) { return *reinterpret_cast<const f32x4*>(&m_sum[S][4 * g]); }, s0, n_super, bs_shift, zp,
        magic);

    // 8) epilogue: lane (g, c) holds MFMA rows 4g..4g+3 of column c
    bool stores = true;
    if constexpr (KS == 2) {  // the second K share hands its sums to the first
        f32x4* r4 = reinterpret_cast<f32x4*>(red) + rb * kWave + lane;
        if (kp == 1) *r4 = sum;
        __syncthreads();
        stores = kp == 0;
        if (stores) sum += *r4;
    }
#pragma unroll
    for (int i = 0; i < 4 && stores; ++i) {
        const int m = 4 * g + i;
        if constexpr (FC1) {
            const float up = dpp_f32<kDppRor8>(sum[i]);  // column c + 8: the up row of column c
            if (m < count && c < 8) {
                const int I = p.N / 2;
                uint16_t* out = act_out + (int64_t)(first + m) * I;
                out[col0 + c] = Dt<DT>::from_float(act_value<DT>(act, sum[i], up, p.ap));
            }
        } else {
            if (m < count) store_y2(&y2[(int64_t)y2_row[i] * p.N + col0 + c], sum[i], p.fused.counters != nullptr);
        }
    }
    if constexpr (!FC1) {
        if (p.fused.counters) fc2_arrive_combine<DT>(p.fused, y2, p.N, p.top_k, n, n * kRowsWG, kRowsWG, q.E);
    }
}


template <bool FC1, int DT, int BITS, int KS, int P, bool RAW>
hipError_t run(const ProjLaunch& p, const DecodePlan& plan, hipStream_t s)
{
    const int rows_wg = 16 * kWavesS / KS;
    launch(stream_kernel<DT, BITS, FC1, KS, P, RAW>, dim3((unsigned)(plan.E * (p.N / rows_wg))),
           dim3(kThreadsS), s, p, plan);
    return hipGetLastError();
}

template <bool FC1, int DT, int BITS, int KS, bool RAW>
hipError_t launch_pieces(const ProjLaunch& p, const DecodePlan& plan, hipStream_t s)
{
    const int pieces = (p.K / KS * BITS / 8 + kLine - 1) / kLine;
    if (pieces <= 1) return run<FC1, DT, BITS, KS, 1, RAW>(p, plan, s);
    if (pieces <= 2) return run<FC1, DT, BITS, KS, 2, RAW>(p, plan, s);
    if (pieces <= 4) return run<FC1, DT, BITS, KS, 4, RAW>(p, plan, s);
    if constexpr (BITS == 4 && KS == 1) {
        if (pieces <= 8) return run<FC1, DT, BITS, KS, 8, RAW>(p, plan, s);
    }
    return hipErrorInvalidValue;
}

template <bool FC1, int DT, int BITS, bool RAW>
hipError_t launch_split(const ProjLaunch& p, const DecodePlan& plan, hipStream_t s)
{
    if constexpr (!FC1) {
        if (p.K % (2 * kSuperK) == 0) return launch_pieces<FC1, DT, BITS, 2, RAW>(p, plan, s);
    }
    return launch_pieces<FC1, DT, BITS, 1, RAW>(p, plan, s);
}

template <bool FC1, int DT>
hipError_t launch_stream(const ProjLaunch& p, const DecodePlan& plan, hipStream_t s)
{
    if (!stream_fits(p.w, p.K, p.N, p.block_size, FC1)) return hipErrorInvalidValue;
    const bool raw = p.block_size % kSuperK == 0;
    if (p.w.bits == 2) {
        return raw ? launch_split<FC1, DT, 2, true>(p, plan, s) : launch_split<FC1, DT, 2, false>(p, plan, s);
    }
    return raw ? launch_split<FC1, DT, 4, true>(p, plan, s) : launch_split<FC1, DT, 4, false>(p, plan, s);
}


}  // namespace

bool stream_fits(const ProjArgs& w, int K, int N, int block_size, bool fc1)
{
    (void)fc1;
    const int bs = block_size;
    return (w.bits == 2 || w.bits == 4) && w.zp == nullptr && K <= kMaxK && K % kSuperK == 0 &&
           N % (16 * kWavesS) == 0 && bs >= 32 && (bs & (bs - 1)) == 0 && (K / bs) % 8 == 0 &&
           K / bs <= kMaxBlocks && reinterpret_cast<uintptr_t>(w.scales) % 16 == 0 &&
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
