// gemm_decode.hip -- grouped projection for few routed rows per expert.
//
// When the expanded row count R = T*top_k is small [PR 33569: the decode
// GEMV handles up to 80 expanded rows], each selected expert's weights are
// streamed from HBM once per 16 of its rows, so time is set by packed-weight
// bytes and by how early those bytes are requested.  A workgroup of eight
// wavefronts computes up to 16 rows of one expert against NB column blocks of
// 16 weight rows.  The wavefronts split K (wavefront w takes 128-input
// super-steps w, w+8, ...); within a wavefront the 16 rows ride in the rows
// of a 16x16x32 MFMA, so the row count costs no VALU work and each weight
// element is dequantized once.
//
// Two kernels share that body:
//  - decode_kernel walks a list of m-tiles {expert, row0, rows, 0, token
//    ids[16], route ids[16]} written by the decode plan (item i = m-tile
//    i / nt, column block i % nt); it serves any number of experts.
//  - decode_expert_kernel gives every (expert, column block) a workgroup of
//    its own, so a workgroup knows which weights it streams before routing is
//    done: it requests them at once, and fc1 routes the tokens itself while
//    they are in flight (the workgroup of block 0 also writes the routing
//    weights, the expert offsets and the sorted routes for fc2 and the
//    combine).  Experts no route selected exit after routing.  Used when
//    every expert is likely selected (E <= R, E <= 64) and K fits one chunk,
//    so the workgroup keeps its weights in registers for all of its rows.
//
// Load order: A rows (one tile row per wavefront, coalesced), the item's
// scales for the K chunk (one 16-byte unit per thread, STAGED), then the
// packed-code spans of all the wavefront's super-steps, none of which is
// consumed yet.  Every load is issued unconditionally (indices are clamped)
// so that each wait covers exactly the loads it needs.  The A rows (permuted
// to the MFMA register order) and the scale table are written to LDS while
// the weight bytes are still in flight; each wavefront then reads its A
// fragments and scales from LDS.  The eight partial tiles are summed in LDS in
// a fixed order (no atomics), then the epilogue applies the gated activation
// (fc1) or writes float32 rows (fc2).
//
// RAW variant (block_size a multiple of 128, so every super-step lies in one
// quantization block): the B operand is the raw codes biased into exact dtype
// values (raw_step, one v_and_or_b32 per two weights) and the zero point and
// scale are applied per super-step in float32 from an extra MFMA against an
// all-ones B operand, which yields the row sums of A:
//   part = -(bias + zp) * rowsum + sum_t mfma(A_t, bias + codes_t)
//   acc += scale * part
#include "gemm_common.h"
#include "route_common.h"

namespace qmoe {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kBatch = 2;               // super-steps per wavefront per K chunk
constexpr int kChunkK = kWaves * kBatch * kSuperK;  // 2048 inputs of A staged at a time
constexpr int kPitch = kChunkK / 2 + 4;  // LDS row pitch in 32-bit words (+4 pad)
constexpr int kScPitch = kChunkK / 32 + 4;  // staged scale row pitch in uint16 (+4 pad)
static_assert(kDecodeMaxRoutes <= 2 * kWave, "route ranks use two wavefronts");

// Weight rows of column block n of expert e: fc1 rows 2*col0 .. 2*col0+63
// (gate/up interleaved), fc2 rows col0 .. col0+31.  trow[nb] is the row of
// (column block nb, lane c) within the block; returns the block's first row.
template <bool FC1, int NB>
__device__ inline int64_t block_rows(const ProjLaunch& p, int e, int n, int c, int& col0,
                                     int (&trow)[NB], WeightRow (&wr)[NB])
{
    constexpr int kCols = NB * 16;
    col0 = FC1 ? n * (kCols / 2) : n * kCols;
    const int64_t wrow0 = (int64_t)e * p.N + (FC1 ? 2 * col0 : col0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        trow[nb] = FC1 ? 32 * (nb / 2) + 2 * c + (nb & 1) : 16 * nb + c;
        if (FC1 && p.fusion != 1) {
            // gate/up halves or a separate fc3: block nb is the gate (even) or up
            // (odd) row of activation column col0 + 16 (nb / 2) + c
            const int I = p.N / 2;
            const bool up = nb & 1;
            const bool sep = p.fusion == 0;
            const int64_t rows_e = sep ? I : p.N;
            wr[nb] = weight_row(sep && up ? p.w3 : p.w,
                                (int64_t)e * rows_e + fc1_row(p.fusion, col0 + 16 * (nb / 2) + c, up, I),
                                p.K, p.block_size);
        } else {
            wr[nb] = weight_row(p.w, wrow0 + trow[nb], p.K, p.block_size);
        }
    }
    return wrow0;
}

// Loads of one K chunk that precede any use of them.
template <int BITS, int NB>
struct ChunkLoads {
    Span<BITS> sp[kBatch][NB];
    RawParams rp[kBatch][NB];
    u32x4 sc = {0u, 0u, 0u, 0u};  // STAGED: one 16-byte unit of the scale table
    int sc_row = 0, sc_part = 0, n_units = 0;
};

// Staged scales (STAGED): the scales of the item's weight rows for the K
// chunk are one 16-byte load per thread into an LDS table instead of one
// 2-byte load per lane, column block and super-step.  Needs a constant zero
// point, 32 <= block_size <= 256, a multiple of 8 blocks per row and
// 16-byte aligned scales (checked by the launcher).
template <int BITS, int NB, int ZP, bool STAGED, bool SPANS = true>
__device__ inline void issue_chunk_loads(ChunkLoads<BITS, NB>& L, const ProjLaunch& p,
                                         const WeightRow (&wr)[NB], int64_t wrow0, int kc, int kn,
                                         int wave, int g, int tid)
{
    constexpr int kCols = NB * 16;
    const int bs = p.block_size;
    const int n_super = kn / kSuperK;
    if constexpr (STAGED) {
        const int upr = kn / bs / 8;  // units per row
        L.n_units = kCols * upr;
        const int u = min(tid, L.n_units - 1);
        L.sc_row = u / upr;
        L.sc_part = u - L.sc_row * upr;
        L.sc = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.w.scales) +
                                               (wrow0 + L.sc_row) * (p.K / bs) + kc / bs +
                                               8 * L.sc_part);
    }
    // super-steps past the chunk reload the last one and are skipped
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
        const int s = min(wave + kWaves * b, n_super - 1);
        const int kk = kc + s * kSuperK + 32 * g;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            if constexpr (SPANS) L.sp[b][nb] = load_span<BITS>(wr[nb].codes, kk);
            if constexpr (!STAGED) L.rp[b][nb] = load_params<ZP>(wr[nb], kk, bs);
        }
    }
}

template <int BITS, int NB>
__device__ inline void store_scales(uint16_t* sc_tab, const ChunkLoads<BITS, NB>& L, int tid)
{
    if (tid < L.n_units) {
        uint32_t* dst = reinterpret_cast<uint32_t*>(sc_tab + L.sc_row * kScPitch + 8 * L.sc_part);
        *reinterpret_cast<u32x2*>(dst) = u32x2{L.sc.x, L.sc.y};
        *reinterpret_cast<u32x2*>(dst + 2) = u32x2{L.sc.z, L.sc.w};
    }
}

// One 32-value A span (this lane's) of LDS row `row`, in the MFMA register order.
template <Order O>
__device__ inline void store_a(uint32_t* lds, int row, int lane, const uint32_t (&a_stage)[16])
{
    uint32_t perm[16];
    permute_span<O>(a_stage, perm);
    uint32_t* dst = lds + row * kPitch + 16 * lane;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        *reinterpret_cast<u32x4*>(dst + 4 * v) =
            u32x4{perm[4 * v], perm[4 * v + 1], perm[4 * v + 2], perm[4 * v + 3]};
    }
}

// MFMAs of this wavefront's super-steps of chunk kc; lanes of rows >= rows
// feed zeros.
template <int DT, int BITS, int NB, int ZP, bool RAW, bool STAGED>
__device__ inline void mfma_chunk(f32x4 (&acc)[NB], const ChunkLoads<BITS, NB>& L,
                                  const uint32_t* lds, const uint16_t* sc_tab,
                                  const int (&trow)[NB], const WeightRow (&wr)[NB],
                                  const ProjLaunch& p, int kc, int n_super, int rows, int wave,
                                  int g, int c, uint32_t magic)
{
    const int bs = p.block_size;
    const u32x4 ones = {ones2<DT>(), ones2<DT>(), ones2<DT>(), ones2<DT>()};
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
        const int s = wave + kWaves * b;
        if (s >= n_super) continue;
        const int kk = kc + s * kSuperK + 32 * g;
        u32x4 a4[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(
                lds + c * kPitch + (s * kSuperK + 32 * g) / 2 + 4 * t);
            a4[t] = c < rows ? v : u32x4{0u, 0u, 0u, 0u};
        }
        auto params = [&](int nb, int kin) {
            if constexpr (STAGED) {
                BlockParams q;
                q.zp = p.w.zp_fallback;
                q.scale = Dt<DT>::to_float(sc_tab[trow[nb] * kScPitch + (kin - kc) / bs]);
                return q;
            } else {
                return decode_params<DT, BITS, ZP>(L.rp[b][nb], p.w.zp_fallback);
            }
        };
        if constexpr (RAW) {
            f32x4 rowsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; ++t) rowsum = Dt<DT>::mfma(a4[t], ones, rowsum);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const BlockParams q = params(nb, kc + s * kSuperK);
                f32x4 part = rowsum * (-(raw_bias<DT>() + q.zp));
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    part = Dt<DT>::mfma(a4[t], raw_step<DT, BITS>(L.sp[b][nb], t, magic), part);
                }
                acc[nb] += part * q.scale;
            }
        } else {
            const bool two_blocks = bs < 32;  // a 32-code span crosses a block boundary
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const BlockParams q0 = params(nb, kk);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    BlockParams q = q0;
                    if (!STAGED && two_blocks && t >= 2) {
                        q = decode_params<DT, BITS, ZP>(load_params<ZP>(wr[nb], kk + 16, bs),
                                                        p.w.zp_fallback);
                    }
                    const u32x4 bf = dequant_zp<DT, BITS, ZP>(L.sp[b][nb], t, q);
                    acc[nb] = Dt<DT>::mfma(a4[t], bf, acc[nb]);
                }
            }
        }
    }
}

// Sums the eight partial tiles in LDS (fixed order) and writes the item's
// outputs: fc1 the gated activation of row m at act row out_row(m), fc2
// float32 values at y2 row out_row(m).  Starts and ends with a barrier.
template <int DT, bool FC1, int NB, int MTR, class OutRow>
__device__ inline void reduce_store(uint32_t* lds, const f32x4 (&acc)[NB], const ProjLaunch& p,
                                    int e, int rows, int col0, int tid, int wave, int g, int c,
                                    OutRow out_row)
{
    constexpr int kCols = NB * 16;
    __syncthreads();  // every wavefront is done reading A from lds
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (MTR == kDecodeMT || 4 * g + i < MTR)
                red[(wave * MTR + 4 * g + i) * (kCols + 1) + nb * 16 + c] = acc[nb][i];
    __syncthreads();

    if constexpr (FC1) {
        const int I = p.N / 2;
        constexpr int kActCols = kCols / 2;
        for (int o = tid; o < MTR * kActCols; o += kThreads) {
            const int m = o / kActCols;
            const int j = o % kActCols;
            if (m >= rows) continue;
            const int gate_col = (j / 16) * 32 + (j % 16);  // blocks 2q gate, 2q+1 up
            float gate = 0.f, up = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                gate += red[(w * MTR + m) * (kCols + 1) + gate_col];
                up += red[(w * MTR + m) * (kCols + 1) + gate_col + 16];
            }
            if (p.bias || p.bias3) {  // expert biases of the gate and up rows
                const bool sep = p.fusion == 0;
                const int64_t base = (int64_t)e * (sep ? I : p.N);
                if (p.bias) gate += p.bias[base + fc1_row(p.fusion, col0 + j, false, I)];
                if (sep ? p.bias3 != nullptr : p.bias != nullptr) {
                    up += sep ? p.bias3[base + col0 + j] : p.bias[base + fc1_row(p.fusion, col0 + j, true, I)];
                }
            }
            uint16_t* out = reinterpret_cast<uint16_t*>(p.act_out) + (int64_t)out_row(m) * I;
            out[col0 + j] = Dt<DT>::from_float(act_value<DT>(p.act, gate, up, p.ap));
        }
    } else {
        for (int o = tid; o < MTR * kCols; o += kThreads) {
            const int m = o / kCols;
            const int h = o % kCols;
            if (m >= rows) continue;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) v += red[(w * MTR + m) * (kCols + 1) + h];
            if (p.bias) v += p.bias[(int64_t)e * p.N + col0 + h];
            store_y2(&p.y2[(int64_t)out_row(m) * p.N + col0 + h], v, p.fused.counters != nullptr);
        }
    }
    __syncthreads();  // lds is free again
}

// ---------------------------------------------------------------- m-tile list
template <int DT, int BITS, bool FC1, int NB, int ZP, bool RAW, bool STAGED>
__global__ __launch_bounds__(kThreads, 4) void decode_kernel(ProjLaunch p,
                                                             const int32_t* __restrict__ tiles,
                                                             const int32_t* __restrict__ n_tiles_ptr)
{
    static_assert(!FC1 || NB % 2 == 0, "fc1 column blocks come in gate/up pairs");
    static_assert(kWaves * kDecodeMT * (NB * 16 + 1) <= kDecodeMT * kPitch, "reduction fits");
    static_assert(!STAGED || ZP == kZpConst, "the staged table holds scales only");
    constexpr Order O = RAW ? raw_order<BITS>() : code_order<DT, BITS>();
    constexpr int kCols = NB * 16;  // weight rows per item
    static_assert(kCols * (kChunkK / 32) / 8 <= kThreads, "one staged unit per thread");
    __shared__ __attribute__((aligned(16))) uint32_t lds[kDecodeMT * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t sc_tab[STAGED ? kCols * kScPitch : 8];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int c = lane & 15;
    const int K = p.K;
    const int nt = p.N / kCols;  // column blocks of one m-tile
    const int n_items = *n_tiles_ptr * nt;
    const uint16_t* a_src = reinterpret_cast<const uint16_t*>(p.a);
    const uint32_t magic = opaque(DT == kF16 ? 0x64006400u : 0x43004300u);

    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int tile = item / nt;
        const int n = item - tile * nt;
        const int32_t* it = tiles + (int64_t)kDecodeTileInts * tile;
        const int e = it[0];
        const int row0 = it[1];
        const int rows = it[2];
        // A rows this wavefront stages: tile rows `wave` and `wave + 8`
        const int64_t a_row1 = FC1 ? it[kDecodeTileTokens + wave] : row0 + wave;
        const int64_t a_row2 = FC1 ? it[kDecodeTileTokens + wave + kWaves] : row0 + wave + kWaves;

        int col0;
        int trow[NB];
        WeightRow wr[NB];
        const int64_t wrow0 = block_rows<FC1, NB>(p, e, n, c, col0, trow, wr);

        f32x4 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int kc = 0; kc < K; kc += kChunkK) {
            const int kn = min(kChunkK, K - kc);
            const int n_super = kn / kSuperK;
            const int spans = kn / 32;            // 32-value A spans per row in this chunk
            const int sl = min(lane, spans - 1);  // this lane's span (clamped: loads stay in bounds)

            // 1) A row `wave` of the tile, requested before the weights
            uint32_t a_stage[16];
            if (wave < rows) load_a_span(a_src + a_row1 * K, kc + 32 * sl, a_stage);
            // 2) scales and packed weights, not consumed yet
            ChunkLoads<BITS, NB> L;
            issue_chunk_loads<BITS, NB, ZP, STAGED>(L, p, wr, wrow0, kc, kn, wave, g, tid);
            // 3) A rows and scales to LDS
            __syncthreads();  // previous chunk / item done with lds and sc_tab
            if (wave < rows && lane < spans) store_a<O>(lds, wave, lane, a_stage);
            if constexpr (STAGED) store_scales(sc_tab, L, tid);
            if (wave + kWaves < rows) {  // rows 8..15 (rare): after the weights
                load_a_span(a_src + a_row2 * K, kc + 32 * sl, a_stage);
                if (lane < spans) store_a<O>(lds, wave + kWaves, lane, a_stage);
            }
            __syncthreads();
            // 4) MFMAs
            mfma_chunk<DT, BITS, NB, ZP, RAW, STAGED>(acc, L, lds, sc_tab, trow, wr, p, kc, n_super,
                                                      rows, wave, g, c, magic);
            // Loads of skipped super-steps are still in flight here; draining them
            // now keeps the next chunk's loads from waiting on stale registers.
            __builtin_amdgcn_s_waitcnt(0);
        }

        // 5) partial tiles summed, then the epilogue (fc1: sorted position row0 + m;
        //    fc2: the row's route id)
        reduce_store<DT, FC1, NB, kDecodeMT>(lds, acc, p, e, rows, col0, tid, wave, g, c, [&](int m) {
            return FC1 ? row0 + m : it[kDecodeTileRoutes + m];
        });
        if constexpr (!FC1) {  // one arrival per m-tile on column block n
            if (p.fused.counters) fc2_arrive_combine<DT>(p.fused, p.y2, p.N, p.top_k, n, col0, kCols, n_items / nt);
        }
    }
}

// ---------------------------------------------------------------- row blocks
// The m-tile list again, for many experts with few rows each (tiles of at
// most MTR rows): every wavefront owns 16 weight rows of the tile's expert
// over the whole of K, so its partial sums never leave it and nothing is
// reduced across wavefronts.  The eight wavefronts of a workgroup (128
// weight rows) share the tile's A rows and their rows' scale table in LDS.
// A wavefront requests all of its code spans (one per 128-input super-step,
// in the MFMA lane layout of mfma_chunk) right after the scale units and the
// A rows, before it waits for anything, and consumes them in order, so the
// first MFMAs start while later spans are still in flight.  fc1: columns
// 0-7 of a wavefront are the gate rows and 8-15 the up rows of 8 activation
// columns, paired in the epilogue by a DPP rotate.
constexpr int kRowsWave = 16;
constexpr int kRowsItem = kWaves * kRowsWave;  // weight rows per workgroup
constexpr int kRowsScUnits = kRowsItem * (kChunkK / 32 / 8) / kThreads;  // 16-byte scale units per thread
constexpr int kDppRotate8 = 0x128;  // DPP row_ror:8: lane c reads lane c ^ 8 of its row

// (The 16-row A tile and the scale table take 83 KB of LDS, one workgroup
// per CU, so that form runs two wavefronts per SIMD whatever its registers.)
template <int DT, int BITS, bool FC1, int ZP, int MTR, int SS>
__global__ __launch_bounds__(kThreads, MTR == 16 ? 2 : 4) void decode_rows_kernel(ProjLaunch p,
                                                                  const int32_t* __restrict__ tiles,
                                                                  const int32_t* __restrict__ n_tiles_ptr)
{
    static_assert(ZP != kZpTensor, "scales only: a constant zero point");
    static_assert(MTR == 8 || MTR == 16, "A rows are staged by one or two rounds of wavefronts");
    constexpr Order O = code_order<DT, BITS>();
    __shared__ __attribute__((aligned(16))) uint32_t lds[MTR * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t sc_tab[kRowsItem * kScPitch];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int c = lane & 15;
    const int K = p.K;
    const int nt = p.N / kRowsItem;
    const int tile = blockIdx.x / nt;
    const int n = blockIdx.x - tile * nt;
    if (tile >= *n_tiles_ptr) {  // whole workgroup; fc2 still arrives on its column block
        if constexpr (!FC1) {
            if (p.fused.counters) {
                fc2_arrive_combine<DT>(p.fused, p.y2, p.N, p.top_k, n, n * kRowsItem, kRowsItem, gridDim.x / nt);
            }
        }
        return;
    }
    const int32_t* it = tiles + (int64_t)kDecodeTileInts * tile;
    const int e = it[0];
    const int row0 = it[1];
    const int rows = it[2];
    const int n_super = K / kSuperK;
    const int n_blocks = K / p.block_size;
    const int bs_shift = __builtin_ctz((unsigned)p.block_size);  // a power of two
    const int64_t wbase = (int64_t)e * p.N + (int64_t)n * kRowsItem;  // the workgroup's first weight row
    // MFMA column c: fc1 gate row 2c (c < 8) or up row 2(c-8)+1 of the
    // wavefront's 8 activation columns; fc2 row c
    const int trow = kRowsWave * wave + (FC1 ? 2 * (c & 7) + (c >> 3) : c);
    const int row_bytes = K * BITS / 8;
    const uint8_t* wcodes = p.w.codes + (wbase + trow) * row_bytes;
    const uint16_t* a_src = reinterpret_cast<const uint16_t*>(p.a);
    const int spans = K / 32;
    const int sl = min(lane, spans - 1);
    // fc2: route ids of MFMA rows 4g..4g+3 (entries past the tile's rows are 0)
    int y2_row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y2_row[i] = FC1 ? 0 : it[kDecodeTileRoutes + 4 * g + i];
    __builtin_amdgcn_sched_barrier(0);

    // 1) scale units: 8 blocks of one of the workgroup's rows each
    const uint16_t* sc_src = reinterpret_cast<const uint16_t*>(p.w.scales) + wbase * n_blocks;
    const int upr = n_blocks >> 3;
    const int n_units = kRowsItem * upr;
    u32x4 sc_unit[kRowsScUnits];
#pragma unroll
    for (int k = 0; k < kRowsScUnits; ++k) {
        const int u = min(tid + kThreads * k, n_units - 1);
        const int r = u / upr;
        sc_unit[k] = *reinterpret_cast<const u32x4*>(sc_src + r * n_blocks + 8 * (u - r * upr));
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2) A rows: tile row `wave` (and wave + 8), one 32-value span per lane
    auto a_row_of = [&](int m) -> int64_t {
        return FC1 ? it[kDecodeTileTokens + m] : row0 + min(m, rows - 1);
    };
    uint32_t a_stage[MTR / kWaves][16];
#pragma unroll
    for (int h = 0; h < MTR / kWaves; ++h) load_a_span(a_src + a_row_of(wave + kWaves * h) * K, 32 * sl, a_stage[h]);
    __builtin_amdgcn_sched_barrier(0);

    // 3) every code span of the wavefront (past K: the last one again, unused)
    Span<BITS> sp[SS];
#pragma unroll
    for (int s = 0; s < SS; ++s) sp[s] = load_span<BITS>(wcodes, min(s, n_super - 1) * kSuperK + 32 * g);
    __builtin_amdgcn_sched_barrier(0);

    // 4) A rows and scales to LDS
#pragma unroll
    for (int h = 0; h < MTR / kWaves; ++h) {
        const int m = wave + kWaves * h;
        if (m < rows && lane < spans) store_a<O>(lds, m, lane, a_stage[h]);
    }
#pragma unroll
    for (int k = 0; k < kRowsScUnits; ++k) {
        const int u = tid + kThreads * k;
        if (u < n_units) {
            const int r = u / upr;
            uint32_t* dst = reinterpret_cast<uint32_t*>(sc_tab + r * kScPitch + 8 * (u - r * upr));
            *reinterpret_cast<u32x2*>(dst) = u32x2{sc_unit[k].x, sc_unit[k].y};
            *reinterpret_cast<u32x2*>(dst + 2) = u32x2{sc_unit[k].z, sc_unit[k].w};
        }
    }
    __syncthreads();

    // 5) the spans in order; two accumulator chains.  MFMA rows past the
    //    tile's rows read a clamped LDS row and are never stored.
    const uint32_t* a_lds = lds + min(c, MTR - 1) * kPitch;
    const uint16_t* sc_row = sc_tab + trow * kScPitch;
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < SS; ++s) {
        if (s < n_super) {  // uniform
            const int kk = s * kSuperK + 32 * g;
            BlockParams q;
            q.zp = p.w.zp_fallback;
            q.scale = Dt<DT>::to_float(sc_row[kk >> bs_shift]);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(a_lds + kk / 2 + 4 * t);
                acc[s & 1] = Dt<DT>::mfma(a, dequant_zp<DT, BITS, ZP>(sp[s], t, q), acc[s & 1]);
            }
        }
    }
    const f32x4 sum = acc[0] + acc[1];

    // 6) epilogue: lane (g, c) holds MFMA rows 4g..4g+3 of column c
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if constexpr (FC1) {
            const float up = dpp_f32<kDppRotate8>(sum[i]);  // column c + 8: the up row of column c
            if (m < rows && c < 8) {
                const int I = p.N / 2;
                uint16_t* out = reinterpret_cast<uint16_t*>(p.act_out) + (int64_t)(row0 + m) * I;
                out[n * (kRowsItem / 2) + 8 * wave + c] = Dt<DT>::from_float(act_value<DT>(p.act, sum[i], up, p.ap));
            }
        } else {
            if (m < rows) {
                store_y2(&p.y2[(int64_t)y2_row[i] * p.N + n * kRowsItem + kRowsWave * wave + c], sum[i],
                         p.fused.counters != nullptr);
            }
        }
    }
    if constexpr (!FC1) {
        if (p.fused.counters) fc2_arrive_combine<DT>(p.fused, p.y2, p.N, p.top_k, n, n * kRowsItem, kRowsItem, gridDim.x / nt);
    }
}

// ---------------------------------------------------------------- expert-stationary
// m-tiles of kExpertRows rows (one A row per wavefront), so the A rows, the
// staged weights and the scale table share the LDS of two workgroups per CU.
constexpr int kExpertRows = kWaves;
constexpr int kTokensPerWave = (kDecodeRoutes + kWaves - 1) / kWaves;

// LDSB: the block's packed weights (<= 32 KB) are staged in LDS with fully
// coalesced 16-byte loads (each wave instruction reads whole cache lines)
// instead of the MFMA pattern of 16 rows x 8-16 bytes per instruction.
template <int BITS, int NB>
constexpr bool expert_lds_weights()
{
    return NB * 16 * kChunkK * BITS / 8 <= 32768 && BITS != 3;
}

template <int DT, int BITS, bool FC1, int NB, int ZP, bool RAW, bool STAGED>
__global__ __launch_bounds__(kThreads, 4) void decode_expert_kernel(ProjLaunch p, DecodePlan q)
{
    static_assert(!FC1 || NB % 2 == 0, "fc1 column blocks come in gate/up pairs");
    static_assert(!STAGED || ZP == kZpConst, "the staged table holds scales only");
    constexpr Order O = RAW ? raw_order<BITS>() : code_order<DT, BITS>();
    constexpr int kCols = NB * 16;
    constexpr bool LDSB = expert_lds_weights<BITS, NB>();
    // bytes per staged weight row, padded so that the 16 rows of an MFMA
    // fragment fall in distinct banks and 16-byte spans stay aligned
    constexpr int kBPitch = kChunkK * BITS / 8 + (BITS == 4 ? 16 : 8);
    constexpr int kBPieces = kCols * kChunkK * BITS / 8 / 16 / kThreads;  // 16-byte pieces per thread
    static_assert(kWaves * kExpertRows * (kCols + 1) <= kExpertRows * kPitch, "reduction fits");
    __shared__ __attribute__((aligned(16))) uint32_t lds[kExpertRows * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t sc_tab[STAGED ? kCols * kScPitch : 8];
    __shared__ __attribute__((aligned(16))) uint8_t b_lds[LDSB ? kCols * kBPitch : 16];
    __shared__ int s_e[kDecodeMaxRoutes];     // expert of route r (fc1)
    __shared__ int s_rows[kDecodeMaxRoutes];  // this expert's routes, ascending (fc1)
    __shared__ int s_count[4];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int c = lane & 15;
    const int K = p.K;  // one chunk: K <= kChunkK
    const int nt = p.N / kCols;
    const int e = blockIdx.x / nt;
    const int n = blockIdx.x - e * nt;
    const int n_super = K / kSuperK;
    const int spans = K / 32;
    const int sl = min(lane, spans - 1);
    const uint16_t* a_src = reinterpret_cast<const uint16_t*>(p.a);
    const uint32_t magic = opaque(DT == kF16 ? 0x64006400u : 0x43004300u);

    // 0) requested before the weights, so their waits do not queue behind
    //    them: fc1 the logits of this wavefront's tokens (addresses clamped),
    //    fc2 the expert's offsets (scalar loads, written by the fc1 launch)
    float lg[kTokensPerWave];
    int first = 0, count = 0;
    if constexpr (FC1) {
#pragma unroll
        for (int j = 0; j < kTokensPerWave; ++j) {  // uniform guard: only the tokens that exist
            const int t = wave + kWaves * j;
            lg[j] = t < q.T ? q.logits[(int64_t)t * q.E + min(lane, q.E - 1)] : 0.f;
        }
    } else {
        first = q.offsets[e];
        count = q.offsets[e + 1] - first;
    }

    // 1) this block's weights and scales
    int col0;
    int trow[NB];
    WeightRow wr[NB];
    const int64_t wrow0 = block_rows<FC1, NB>(p, e, n, c, col0, trow, wr);
    ChunkLoads<BITS, NB> L;
    u32x4 bpiece[LDSB ? kBPieces : 1];
    const int row_bytes = K * BITS / 8;
    const int b_total = kCols * row_bytes;  // the block's rows are contiguous
    if constexpr (LDSB) {
        const uint8_t* src = p.w.codes + wrow0 * row_bytes;
#pragma unroll
        for (int j = 0; j < kBPieces; ++j) {
            const int off = min(16 * (tid + kThreads * j), b_total - 16);
            bpiece[j] = *reinterpret_cast<const u32x4*>(src + off);
        }
        issue_chunk_loads<BITS, NB, ZP, STAGED, false>(L, p, wr, wrow0, 0, K, wave, g, tid);
    } else {
        issue_chunk_loads<BITS, NB, ZP, STAGED>(L, p, wr, wrow0, 0, K, wave, g, tid);
    }

    // 2) which routes chose expert e, and their first sorted position
    if constexpr (FC1) {
        const int R = q.T * p.top_k;
        const bool writer = blockIdx.x == 0;
        if (writer && tid < q.n_counters) {  // fc2's column-block counters start at zero
            __hip_atomic_store(&q.counters[tid], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int j = 0; j < kTokensPerWave; ++j) {
            const int t = wave + kWaves * j;
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
        // ranks among this expert's routes (ballots over two wavefronts)
        const bool mine = tid < R && s_e[tid] == e;
        const bool below = tid < R && s_e[tid] < e;
        const uint64_t mine_b = __ballot(mine);
        const uint64_t below_b = __ballot(below);
        if (wave < 2 && lane == 0) {
            s_count[wave] = __popcll(mine_b);
            s_count[2 + wave] = __popcll(below_b);
        }
        __syncthreads();
        if (mine) {
            s_rows[__popcll(mine_b & ((1ull << lane) - 1ull)) + (wave == 1 ? s_count[0] : 0)] = tid;
        }
        if (writer) {  // offsets and sorted routes of all experts, for fc2
            if (tid < R) {
                const int ex = s_e[tid];
                int less = 0, same_before = 0;
                for (int r = 0; r < R; ++r) {
                    less += s_e[r] < ex;
                    same_before += (s_e[r] == ex) & (r < tid);
                }
                q.sorted[less + same_before] = tid;
            }
            for (int ex = tid; ex <= q.E; ex += kThreads) {
                int less = 0;
                for (int r = 0; r < R; ++r) less += s_e[r] < ex;
                q.offsets[ex] = less;
            }
        }
        __syncthreads();
        count = s_count[0] + s_count[1];
        first = s_count[2] + s_count[3];
    }
    if (count == 0) {  // whole workgroup; the weight loads drain on their own
        if constexpr (!FC1) {
            if (p.fused.counters) fc2_arrive_combine<DT>(p.fused, p.y2, p.N, p.top_k, n, col0, kCols, q.E);
        }
        return;
    }

    // 3) the expert's rows, kExpertRows at a time, against the same weights
    for (int m0 = 0; m0 < count; m0 += kExpertRows) {
        const int rows = min(kExpertRows, count - m0);
        uint32_t a_stage[16];
        if (wave < rows) {
            const int64_t a_row = FC1 ? s_rows[m0 + wave] / p.top_k : first + m0 + wave;
            load_a_span(a_src + a_row * K, 32 * sl, a_stage);
        }
        __syncthreads();  // the previous tile's reduction is done with lds
        if (wave < rows && lane < spans) store_a<O>(lds, wave, lane, a_stage);
        if (m0 == 0) {
            if constexpr (STAGED) store_scales(sc_tab, L, tid);
            if constexpr (LDSB) {
#pragma unroll
                for (int j = 0; j < kBPieces; ++j) {
                    const int off = 16 * (tid + kThreads * j);
                    if (off < b_total) {
                        const int r = off / row_bytes;
                        uint8_t* dst = b_lds + r * kBPitch + (off - r * row_bytes);
                        *reinterpret_cast<u32x2*>(dst) = u32x2{bpiece[j].x, bpiece[j].y};
                        *reinterpret_cast<u32x2*>(dst + 8) = u32x2{bpiece[j].z, bpiece[j].w};
                    }
                }
            }
        }
        __syncthreads();
        if constexpr (LDSB) {
            if (m0 == 0) {  // this wavefront's spans, in the MFMA register layout
#pragma unroll
                for (int b = 0; b < kBatch; ++b) {
                    const int s = min(wave + kWaves * b, n_super - 1);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        L.sp[b][nb] = load_span<BITS>(b_lds + trow[nb] * kBPitch, s * kSuperK + 32 * g);
                    }
                }
            }
        }

        f32x4 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        mfma_chunk<DT, BITS, NB, ZP, RAW, STAGED>(acc, L, lds, sc_tab, trow, wr, p, 0, n_super,
                                                  rows, wave, g, c, magic);
        reduce_store<DT, FC1, NB, kExpertRows>(lds, acc, p, e, rows, col0, tid, wave, g, c, [&](int m) {
            return FC1 ? first + m0 + m : q.sorted[first + m0 + m];
        });
    }
    if constexpr (!FC1) {
        if (p.fused.counters) fc2_arrive_combine<DT>(p.fused, p.y2, p.N, p.top_k, n, col0, kCols, q.E);
    }
}

template <bool FC1, int DT, int NB, int BITS, int ZP, bool RAW, bool STAGED = false>
hipError_t launch_one(const ProjLaunch& p, const DecodePlan* plan, hipStream_t s)
{
    if (plan) {
        launch(decode_expert_kernel<DT, BITS, FC1, NB, ZP, RAW, STAGED>,
               dim3((unsigned)(plan->E * (p.N / (NB * 16)))), dim3(kThreads), s, p, *plan);
    } else {
        launch(decode_kernel<DT, BITS, FC1, NB, ZP, RAW, STAGED>, dim3((unsigned)p.grid),
               dim3(kThreads), s, p, p.worklist, p.n_items);
    }
    return hipGetLastError();
}

// Scales can be staged when every K chunk covers whole 16-byte units of every
// weight row's scales.
inline bool can_stage(const ProjLaunch& p)
{
    const int bs = p.block_size;
    return bs >= 32 && bs <= 256 && (p.K / bs) % 8 == 0 &&
           reinterpret_cast<uintptr_t>(p.w.scales) % 16 == 0;
}

template <bool FC1, int DT, int NB, int BITS>
hipError_t launch_zp(const ProjLaunch& p, const DecodePlan* plan, hipStream_t s)
{
    const int zp = zp_mode(p.w);
    // the staged scale table covers contiguous weight rows: interleaved fc1 only
    const bool staged = zp != kZpTensor && can_stage(p) && (!FC1 || p.fusion == 1);
    // raw codes: 2/3/4-bit (8-bit codes overflow the bf16 raw bias's exact range)
    constexpr bool kRawOk = BITS == 2 || BITS == 3 || BITS == 4;
    if constexpr (kRawOk) {
        if (p.block_size % kSuperK == 0) {  // zero point applied in float32: any value works
            if (zp == kZpTensor) return launch_one<FC1, DT, NB, BITS, kZpTensor, true>(p, plan, s);
            return staged ? launch_one<FC1, DT, NB, BITS, kZpConst, true, true>(p, plan, s)
                          : launch_one<FC1, DT, NB, BITS, kZpConst, true>(p, plan, s);
        }
    }
    if (zp == kZpTensor) return launch_one<FC1, DT, NB, BITS, kZpTensor, false>(p, plan, s);
    if (zp == kZpConst && staged) {
        return launch_one<FC1, DT, NB, BITS, kZpConst, false, true>(p, plan, s);
    }
    // any other constant zero point: float32 dequant (exact for the fast values too)
    return launch_one<FC1, DT, NB, BITS, kZpGeneric, false>(p, plan, s);
}

template <bool FC1, int DT, int BITS, int ZP, int MTR>
hipError_t launch_rows_ss(const ProjLaunch& p, hipStream_t s)
{
    const int n_super = p.K / kSuperK;
    const dim3 grid((unsigned)(p.tiles_cap * (p.N / kRowsItem)));
    if (n_super <= 4) {
        launch(decode_rows_kernel<DT, BITS, FC1, ZP, MTR, 4>, grid, dim3(kThreads), s, p, p.worklist, p.n_items);
    } else if (n_super <= 8) {
        launch(decode_rows_kernel<DT, BITS, FC1, ZP, MTR, 8>, grid, dim3(kThreads), s, p, p.worklist, p.n_items);
    } else {
        launch(decode_rows_kernel<DT, BITS, FC1, ZP, MTR, 16>, grid, dim3(kThreads), s, p, p.worklist, p.n_items);
    }
    return hipGetLastError();
}

template <bool FC1, int DT, int BITS>
hipError_t launch_rows_bits(const ProjLaunch& p, int max_rows, hipStream_t s)
{
    const bool generic = zp_mode(p.w) == kZpGeneric;
    if (max_rows <= 8) {
        return generic ? launch_rows_ss<FC1, DT, BITS, kZpGeneric, 8>(p, s)
                       : launch_rows_ss<FC1, DT, BITS, kZpConst, 8>(p, s);
    }
    return generic ? launch_rows_ss<FC1, DT, BITS, kZpGeneric, 16>(p, s)
                   : launch_rows_ss<FC1, DT, BITS, kZpConst, 16>(p, s);
}

template <bool FC1, int DT>
hipError_t launch_rows_dt(const ProjLaunch& p, int max_rows, hipStream_t s)
{
    switch (p.w.bits) {
    case 2: return launch_rows_bits<FC1, DT, 2>(p, max_rows, s);
    case 3: return launch_rows_bits<FC1, DT, 3>(p, max_rows, s);
    case 4: return launch_rows_bits<FC1, DT, 4>(p, max_rows, s);
    default: return hipErrorInvalidValue;
    }
}

template <bool FC1, int DT, int NB>
hipError_t launch_dt(const ProjLaunch& p, const DecodePlan* plan, hipStream_t s)
{
    switch (p.w.bits) {
    case 2: return launch_zp<FC1, DT, NB, 2>(p, plan, s);
    case 3: return launch_zp<FC1, DT, NB, 3>(p, plan, s);
    case 4: return launch_zp<FC1, DT, NB, 4>(p, plan, s);
    default: break;
    }
    if (plan == nullptr) {  // 1- and 8-bit codes: the m-tile kernels only
        if (p.w.bits == 1) return launch_zp<FC1, DT, NB, 1>(p, plan, s);
        if (p.w.bits == 8) return launch_zp<FC1, DT, NB, 8>(p, plan, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fc1_decode(const ProjLaunch& p, const DecodePlan* plan, int dtype, hipStream_t s)
{
    if (plan && (p.K > kChunkK || plan->E > kWave || plan->T > kTokensPerWave * kWaves ||
                 plan->T * p.top_k > kDecodeMaxRoutes)) {
        return hipErrorInvalidValue;
    }
    return dtype == kBF16 ? launch_dt<true, kBF16, kDecodeFc1Blocks>(p, plan, s)
                          : launch_dt<true, kF16, kDecodeFc1Blocks>(p, plan, s);
}

bool rows_fits(const ProjArgs& w, int K, int N, int block_size)
{
    const int bs = block_size;
    return w.zp == nullptr && K % kSuperK == 0 && K <= kChunkK && N % kRowsItem == 0 && bs >= 32 &&
           (bs & (bs - 1)) == 0 && (K / bs) % 8 == 0 && reinterpret_cast<uintptr_t>(w.scales) % 16 == 0;
}

hipError_t launch_rows_decode(const ProjLaunch& p, bool fc1, int max_rows, int dtype, hipStream_t s)
{
    if (!rows_fits(p.w, p.K, p.N, p.block_size) || max_rows < 1 || max_rows > kDecodeMT) {
        return hipErrorInvalidValue;
    }
    if (fc1) {
        return dtype == kBF16 ? launch_rows_dt<true, kBF16>(p, max_rows, s)
                              : launch_rows_dt<true, kF16>(p, max_rows, s);
    }
    return dtype == kBF16 ? launch_rows_dt<false, kBF16>(p, max_rows, s)
                          : launch_rows_dt<false, kF16>(p, max_rows, s);
}

hipError_t launch_fc2_decode(const ProjLaunch& p, const DecodePlan* plan, int dtype, hipStream_t s)
{
    if (plan && p.K > kChunkK) return hipErrorInvalidValue;
    return dtype == kBF16 ? launch_dt<false, kBF16, kDecodeFc2Blocks>(p, plan, s)
                          : launch_dt<false, kF16, kDecodeFc2Blocks>(p, plan, s);
}

}  // namespace qmoe
