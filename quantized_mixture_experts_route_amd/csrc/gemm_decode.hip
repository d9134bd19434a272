// gemm_decode.hip -- grouped projection for few routed rows per expert.
//
// When the expanded row count R = T*top_k is small [PR 33569: the decode
// GEMV handles up to 80 expanded rows], each selected expert's weights are
// streamed from HBM once per 16 of its rows, so time is set by packed-weight
// bytes and by how early those bytes are requested.  A workgroup of eight
// wavefronts takes one decode work-list item {expert, n, row0, rows, ids[16]}
// (one scalar fetch): up to 16 rows of the expert against NB column blocks of
// 16 weight rows.  The wavefronts split K (wavefront w takes 128-input
// super-steps w, w+8, ...); within a wavefront the 16 rows ride in the rows
// of a 16x16x32 MFMA, so the row count costs no VALU work and each weight
// element is dequantized once.
//
// Load order: the workgroup first requests its A rows (only the `rows` real
// ones, coalesced 16-byte loads), then every wavefront issues the packed-code
// spans and raw block scale / zero-point bits of all its super-steps, none of
// which is consumed yet.  The A rows are written to LDS (permuted to the MFMA
// register order) while the weight bytes are still in flight; each wavefront
// then reads its A fragments from LDS.  The eight partial tiles are summed in
// LDS in a fixed order (no atomics), then the epilogue applies the gated
// activation (fc1) or writes float32 rows (fc2).
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

template <int DT, int BITS, bool FC1, int NB, int ZP, bool RAW>
__global__ __launch_bounds__(kThreads, 4) void decode_kernel(ProjLaunch p,
                                                             const int32_t* __restrict__ items,
                                                             const int32_t* __restrict__ n_items_ptr)
{
    static_assert(!FC1 || NB % 2 == 0, "fc1 column blocks come in gate/up pairs");
    static_assert(kWaves * kDecodeMT * (NB * 16 + 1) <= kDecodeMT * kPitch, "reduction fits");
    constexpr Order O = RAW ? raw_order<BITS>() : code_order<DT, BITS>();
    constexpr int kCols = NB * 16;  // weight rows per item
    __shared__ __attribute__((aligned(16))) uint32_t lds[kDecodeMT * kPitch];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int c = lane & 15;
    const int K = p.K;
    const int n_items = *n_items_ptr;
    const bool two_blocks = p.block_size < 32;  // a 32-code span crosses a block boundary
    const uint16_t* a_src = reinterpret_cast<const uint16_t*>(p.a);
    const uint32_t magic = opaque(DT == kF16 ? 0x64006400u : 0x43004300u);
    const u32x4 ones = {ones2<DT>(), ones2<DT>(), ones2<DT>(), ones2<DT>()};

    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int32_t* it = items + (int64_t)kDecodeItemInts * item;
        const int e = it[0];
        const int nt = it[1];
        const int row0 = it[2];
        const int rows = it[3];

        int col0;
        WeightRow wr[NB];
        if constexpr (FC1) {
            col0 = nt * (kCols / 2);  // first activation column
#pragma unroll
            for (int q = 0; q < NB / 2; ++q) {
                const int64_t gate = (int64_t)e * p.N + 2 * (col0 + 16 * q + c);
                wr[2 * q] = weight_row(p.w, gate, K, p.block_size);
                wr[2 * q + 1] = weight_row(p.w, gate + 1, K, p.block_size);
            }
        } else {
            col0 = nt * kCols;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                wr[nb] = weight_row(p.w, (int64_t)e * p.N + col0 + 16 * nb + c, K, p.block_size);
            }
        }

        f32x4 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int kc = 0; kc < K; kc += kChunkK) {
            const int kn = min(kChunkK, K - kc);
            const int n_super = kn / kSuperK;
            const int spans = kn / 32;  // 32-value A spans per row in this chunk

            // 1) A rows of the chunk, first pass (up to 8 rows): one 64-byte span
            //    per thread, requested before the weights
            uint32_t a_stage[16];
            const int a_spans = rows * spans;
            auto load_a = [&](int q) {
                const int64_t src = FC1 ? it[4 + q / spans] : row0 + q / spans;
                load_a_span(a_src + src * K, kc + 32 * (q % spans), a_stage);
            };
            auto store_a = [&](int q) {
                uint32_t perm[16];
                permute_span<O>(a_stage, perm);
                uint32_t* dst = lds + (q / spans) * kPitch + 16 * (q % spans);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    *reinterpret_cast<u32x4*>(dst + 4 * v) =
                        u32x4{perm[4 * v], perm[4 * v + 1], perm[4 * v + 2], perm[4 * v + 3]};
                }
            };
            if (tid < a_spans) load_a(tid);
            // 2) packed weights of this wavefront's super-steps, not consumed yet
            Span<BITS> sp[kBatch][NB];
            RawParams rp[kBatch][NB];
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int s = wave + kWaves * b;
                if (s < n_super) {
                    const int kk = kc + s * kSuperK + 32 * g;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        sp[b][nb] = load_span<BITS>(wr[nb].codes, kk);
                        rp[b][nb] = load_params<ZP>(wr[nb], kk, p.block_size);
                    }
                }
            }
            // 3) A rows to LDS in the MFMA register order (rows 8..15 in a second pass)
            __syncthreads();  // previous chunk / item done with lds
            if (tid < a_spans) store_a(tid);
            if (tid + kThreads < a_spans) {
                load_a(tid + kThreads);
                store_a(tid + kThreads);
            }
            __syncthreads();

            // 4) MFMAs; lanes of rows >= rows feed zeros
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
                if constexpr (RAW) {
                    f32x4 rowsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int t = 0; t < 4; ++t) rowsum = Dt<DT>::mfma(a4[t], ones, rowsum);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const BlockParams q = decode_params<DT, BITS, ZP>(rp[b][nb], p.w.zp_fallback);
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
                        const BlockParams q0 = decode_params<DT, BITS, ZP>(rp[b][nb], p.w.zp_fallback);
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            BlockParams q = q0;
                            if (two_blocks && t >= 2) {
                                q = decode_params<DT, BITS, ZP>(
                                    load_params<ZP>(wr[nb], kk + 16, p.block_size), p.w.zp_fallback);
                            }
                            const u32x4 bf = dequant_zp<DT, BITS, ZP>(sp[b][nb], t, q);
                            acc[nb] = Dt<DT>::mfma(a4[t], bf, acc[nb]);
                        }
                    }
                }
            }
        }

        // 5) sum the eight partial tiles in LDS (fixed order), then the epilogue
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
                p.y2[(int64_t)it[4 + m] * p.N + col0 + h] = v;  // route id of row m
            }
        }
        __syncthreads();  // the next item reuses lds
    }
}

template <bool FC1, int DT, int NB, int BITS, int ZP, bool RAW>
hipError_t launch_one(const ProjLaunch& p, hipStream_t s)
{
    hipLaunchKernelGGL((decode_kernel<DT, BITS, FC1, NB, ZP, RAW>), dim3((unsigned)p.grid),
                       dim3(kThreads), 0, s, p, p.worklist, p.n_items);
    return hipGetLastError();
}

template <bool FC1, int DT, int NB, int BITS>
hipError_t launch_zp(const ProjLaunch& p, hipStream_t s)
{
    const int zp = zp_mode(p.w);
    if (p.block_size % kSuperK == 0) {  // zero point applied in float32: any value works
        return zp == kZpTensor ? launch_one<FC1, DT, NB, BITS, kZpTensor, true>(p, s)
                               : launch_one<FC1, DT, NB, BITS, kZpConst, true>(p, s);
    }
    switch (zp) {
    case kZpConst: return launch_one<FC1, DT, NB, BITS, kZpConst, false>(p, s);
    case kZpTensor: return launch_one<FC1, DT, NB, BITS, kZpTensor, false>(p, s);
    default: return launch_one<FC1, DT, NB, BITS, kZpGeneric, false>(p, s);
    }
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
