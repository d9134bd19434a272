// gemm_decode.hip -- grouped projection for few routed rows per expert.
//
// When the expanded row count R = T*top_k is small [PR 33569: the decode
// GEMV handles up to 80 expanded rows], each selected expert's weights are
// streamed from HBM once per 16 of its rows, so time is set by packed-weight
// bytes and by how early those bytes are requested.  A workgroup of eight
// wavefronts takes one item (m-tile i / nt, column block i % nt): up to 16
// rows of one expert, described by the m-tile {expert, row0, rows, 0,
// token ids[16], route ids[16]} (one scalar fetch), against NB column blocks
// of 16 weight rows.  The wavefronts split K (wavefront w takes 128-input
// super-steps w, w+8, ...); within a wavefront the 16 rows ride in the rows
// of a 16x16x32 MFMA, so the row count costs no VALU work and each weight
// element is dequantized once.
//
// Load order: the wavefront requests its A row (tile row `wave`; the row ids
// come with the m-tile as scalar loads), then the item's scales for the K
// chunk (one 16-byte unit per thread, STAGED), then the packed-code spans of
// all its super-steps, none of which is consumed yet.  Every load is issued
// unconditionally (indices are clamped) so that each wait covers exactly the
// loads it needs.  The A rows (permuted to the MFMA register order) and the
// scale table are written to LDS while the weight bytes are still in flight;
// each wavefront then reads its A fragments and scales from LDS.  The eight
// partial tiles are summed in LDS in a fixed order (no atomics), then the
// epilogue applies the gated activation (fc1) or writes float32 rows (fc2).
//
// RAW variant (block_size a multiple of 128, so every super-step lies in one
// quantization block): the B operand is the raw codes biased into exact dtype
// values (raw_step, one v_and_or_b32 per two weights) and the zero point and
// scale are applied per super-step in float32 from an extra MFMA against an
// all-ones B operand, which yields the row sums of A:
//   part = -(bias + zp) * rowsum + sum_t mfma(A_t, bias + codes_t)
//   acc += scale * part
#include "gemm_common.h"

namespace qmoe {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kBatch = 2;               // super-steps per wavefront per K chunk
constexpr int kChunkK = kWaves * kBatch * kSuperK;  // 2048 inputs of A staged at a time
constexpr int kPitch = kChunkK / 2 + 4;  // LDS row pitch in 32-bit words (+4 pad)
constexpr int kScPitch = kChunkK / 32 + 4;  // staged scale row pitch in uint16 (+4 pad)

// Staged scales (STAGED): the scales of the item's weight rows for the K
// chunk are one 16-byte load per thread into an LDS table instead of one
// 2-byte load per lane, column block and super-step.  Needs a constant zero
// point, 32 <= block_size <= 256, a multiple of 8 blocks per row and
// 16-byte aligned scales (checked by the launcher).
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
    const int bs = p.block_size;
    const int n_blocks = K / bs;
    const int nt = p.N / kCols;  // column blocks of one m-tile
    const int n_items = *n_tiles_ptr * nt;
    const bool two_blocks = bs < 32;  // a 32-code span crosses a block boundary
    const uint16_t* a_src = reinterpret_cast<const uint16_t*>(p.a);
    const uint16_t* scales = reinterpret_cast<const uint16_t*>(p.w.scales);
    const uint32_t magic = opaque(DT == kF16 ? 0x64006400u : 0x43004300u);
    const u32x4 ones = {ones2<DT>(), ones2<DT>(), ones2<DT>(), ones2<DT>()};

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

        // weight rows of the item: fc1 rows 2*col0 .. 2*col0+63 (gate/up
        // interleaved), fc2 rows col0 .. col0+31; table row of (nb, c)
        const int col0 = FC1 ? n * (kCols / 2) : n * kCols;
        const int64_t wrow0 = (int64_t)e * p.N + (FC1 ? 2 * col0 : col0);
        int trow[NB];
        WeightRow wr[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            trow[nb] = FC1 ? 32 * (nb / 2) + 2 * c + (nb & 1) : 16 * nb + c;
            wr[nb] = weight_row(p.w, wrow0 + trow[nb], K, bs);
        }

        f32x4 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int kc = 0; kc < K; kc += kChunkK) {
            const int kn = min(kChunkK, K - kc);
            const int n_super = kn / kSuperK;
            const int spans = kn / 32;            // 32-value A spans per row in this chunk
            const int sl = min(lane, spans - 1);  // this lane's span (clamped: loads stay in bounds)

            // 1) A rows 0..7 of the tile, one row per wavefront, one 64-byte span
            //    per lane, requested before the weights (row ids are scalar loads)
            uint32_t a_stage[16];
            if (wave < rows) load_a_span(a_src + a_row1 * K, kc + 32 * sl, a_stage);
            // 2) staged scales: one 16-byte unit of the chunk's table per thread
            u32x4 sc_unit = {0u, 0u, 0u, 0u};
            int sc_row = 0, sc_part = 0, n_units = 0;
            if constexpr (STAGED) {
                const int upr = kn / bs / 8;  // units per row
                n_units = kCols * upr;
                const int u = min(tid, n_units - 1);
                sc_row = u / upr;
                sc_part = u - sc_row * upr;
                sc_unit = *reinterpret_cast<const u32x4*>(
                    scales + (wrow0 + sc_row) * n_blocks + kc / bs + 8 * sc_part);
            }
            // 3) packed weights of this wavefront's super-steps, not consumed yet
            //    (super-steps past the chunk reload the last one and are skipped)
            Span<BITS> sp[kBatch][NB];
            RawParams rp[kBatch][NB];
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int s = min(wave + kWaves * b, n_super - 1);
                const int kk = kc + s * kSuperK + 32 * g;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    sp[b][nb] = load_span<BITS>(wr[nb].codes, kk);
                    if constexpr (!STAGED) rp[b][nb] = load_params<ZP>(wr[nb], kk, bs);
                }
            }
            // 4) A rows and scales to LDS; A in the MFMA register order
            auto store_a = [&](int row) {
                uint32_t perm[16];
                permute_span<O>(a_stage, perm);
                uint32_t* dst = lds + row * kPitch + 16 * lane;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    *reinterpret_cast<u32x4*>(dst + 4 * v) =
                        u32x4{perm[4 * v], perm[4 * v + 1], perm[4 * v + 2], perm[4 * v + 3]};
                }
            };
            __syncthreads();  // previous chunk / item done with lds and sc_tab
            if (wave < rows && lane < spans) store_a(wave);
            if constexpr (STAGED) {
                if (tid < n_units) {
                    uint32_t* dst = reinterpret_cast<uint32_t*>(sc_tab + sc_row * kScPitch + 8 * sc_part);
                    *reinterpret_cast<u32x2*>(dst) = u32x2{sc_unit.x, sc_unit.y};
                    *reinterpret_cast<u32x2*>(dst + 2) = u32x2{sc_unit.z, sc_unit.w};
                }
            }
            if (wave + kWaves < rows) {  // rows 8..15 (rare): after the weights
                load_a_span(a_src + a_row2 * K, kc + 32 * sl, a_stage);
                if (lane < spans) store_a(wave + kWaves);
            }
            __syncthreads();

            // 5) MFMAs; lanes of rows >= rows feed zeros
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
                        return decode_params<DT, BITS, ZP>(rp[b][nb], p.w.zp_fallback);
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
                            part = Dt<DT>::mfma(a4[t], raw_step<DT, BITS>(sp[b][nb], t, magic), part);
                        }
                        acc[nb] += part * q.scale;
                    }
                } else {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const BlockParams q0 = params(nb, kk);
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            BlockParams q = q0;
                            if (!STAGED && two_blocks && t >= 2) {
                                q = decode_params<DT, BITS, ZP>(
                                    load_params<ZP>(wr[nb], kk + 16, bs), p.w.zp_fallback);
                            }
                            const u32x4 bf = dequant_zp<DT, BITS, ZP>(sp[b][nb], t, q);
                            acc[nb] = Dt<DT>::mfma(a4[t], bf, acc[nb]);
                        }
                    }
                }
            }
            // Loads of skipped super-steps are still in flight here; draining them
            // now keeps the next chunk's loads from waiting on stale registers.
            __builtin_amdgcn_s_waitcnt(0);
        }

        // 6) sum the eight partial tiles in LDS (fixed order), then the epilogue
        __syncthreads();  // every wavefront is done reading A from lds
        float* red = reinterpret_cast<float*>(lds);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                red[(wave * kDecodeMT + 4 * g + i) * (kCols + 1) + nb * 16 + c] = acc[nb][i];
        __syncthreads();

        if constexpr (FC1) {
            const int I = p.N / 2;
            constexpr int kActCols = kCols / 2;
            for (int o = tid; o < kDecodeMT * kActCols; o += kThreads) {
                const int m = o / kActCols;
                const int j = o % kActCols;
                if (m >= rows) continue;
                const int gate_col = (j / 16) * 32 + (j % 16);  // blocks 2q gate, 2q+1 up
                float gate = 0.f, up = 0.f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    gate += red[(w * kDecodeMT + m) * (kCols + 1) + gate_col];
                    up += red[(w * kDecodeMT + m) * (kCols + 1) + gate_col + 16];
                }
                uint16_t* out = reinterpret_cast<uint16_t*>(p.act_out) + (int64_t)(row0 + m) * I;
                out[col0 + j] = Dt<DT>::from_float(act_value<DT>(p.act, gate, up));
            }
        } else {
            for (int o = tid; o < kDecodeMT * kCols; o += kThreads) {
                const int m = o / kCols;
                const int h = o % kCols;
                if (m >= rows) continue;
                float v = 0.f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) v += red[(w * kDecodeMT + m) * (kCols + 1) + h];
                p.y2[(int64_t)it[kDecodeTileRoutes + m] * p.N + col0 + h] = v;
            }
        }
        __syncthreads();  // the next item reuses lds
    }
}

template <bool FC1, int DT, int NB, int BITS, int ZP, bool RAW, bool STAGED = false>
hipError_t launch_one(const ProjLaunch& p, hipStream_t s)
{
    launch(decode_kernel<DT, BITS, FC1, NB, ZP, RAW, STAGED>, dim3((unsigned)p.grid), dim3(kThreads),
           s, p, p.worklist, p.n_items);
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
hipError_t launch_zp(const ProjLaunch& p, hipStream_t s)
{
    const int zp = zp_mode(p.w);
    const bool staged = zp != kZpTensor && can_stage(p);
    if (p.block_size % kSuperK == 0) {  // zero point applied in float32: any value works
        if (zp == kZpTensor) return launch_one<FC1, DT, NB, BITS, kZpTensor, true>(p, s);
        return staged ? launch_one<FC1, DT, NB, BITS, kZpConst, true, true>(p, s)
                      : launch_one<FC1, DT, NB, BITS, kZpConst, true>(p, s);
    }
    if (zp == kZpTensor) return launch_one<FC1, DT, NB, BITS, kZpTensor, false>(p, s);
    if (zp == kZpConst && staged) return launch_one<FC1, DT, NB, BITS, kZpConst, false, true>(p, s);
    // any other constant zero point: float32 dequant (exact for the fast values too)
    return launch_one<FC1, DT, NB, BITS, kZpGeneric, false>(p, s);
}

template <bool FC1, int DT, int NB>
hipError_t launch_dt(const ProjLaunch& p, hipStream_t s)
{
    switch (p.w.bits) {
    case 2: return launch_zp<FC1, DT, NB, 2>(p, s);
    case 3: return launch_zp<FC1, DT, NB, 3>(p, s);
    case 4: return launch_zp<FC1, DT, NB, 4>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_fc1_decode(const ProjLaunch& p, int dtype, hipStream_t s)
{
    return dtype == kBF16 ? launch_dt<true, kBF16, kDecodeFc1Blocks>(p, s)
                          : launch_dt<true, kF16, kDecodeFc1Blocks>(p, s);
}

hipError_t launch_fc2_decode(const ProjLaunch& p, int dtype, hipStream_t s)
{
    return dtype == kBF16 ? launch_dt<false, kBF16, kDecodeFc2Blocks>(p, s)
                          : launch_dt<false, kF16, kDecodeFc2Blocks>(p, s);
}

}  // namespace qmoe
