// gemm_prefill.hip -- grouped projection for many routed rows per expert.
//
// A workgroup of MT/16 wavefronts takes one work-list item: up to MT routed
// rows of one expert against 4*MT weight rows, each wavefront owning 64
// weight rows (4 MFMA column blocks of 16) for all MT rows, so each weight
// element is dequantized once per MT rows.  Every thread stages four 16-byte
// A chunks per K super-step, and a wavefront keeps within 256 registers, so
// two wavefronts share each SIMD and one hides the other's waits.  MT = 128 (8 wavefronts, 512 weight rows, one workgroup per CU) for
// large layers; MT = 64 (4 wavefronts, 256 weight rows, two per CU) when the
// large tile leaves too few items, and for 16-input blocks and generic zero
// points, whose extra registers only fit the small tile.
//
// Packed codes stream from HBM straight into registers, are dequantized there
// as (code - zp) * scale and fed to bf16/fp16 MFMA; the A rows (gathered
// hidden states for fc1, sorted activations for fc2) are staged per K
// super-step in a double-buffered LDS tile shared by the wavefronts, already
// permuted to the MFMA register order, while the next super-step's A rows and
// packed spans are in flight.
// [PR 32198: weights stay packed in HBM and are dequantized in registers
// inside the GEMM; gemm_quant_moe.rs, moe_fp8_grouped_gemm: workgroups stride
// over a compacted work-list, rows addressed through sorted route ids.]
//
// Item order: the work-list enumerates (expert, m-tile, n-tile) with n inner;
// the kernel walks each expert's items with m inner instead, so the m-tiles
// that share a block of weight rows run back to back, and maps workgroup ids
// so that consecutive items land on the same XCD (workgroups are dealt to the
// 8 XCDs round-robin): the weight block is then fetched from HBM once and
// re-read from that XCD's L2.
//
// fc1 (+ activation): a wavefront's 4 column blocks are the gate rows 2j and
// the up rows 2j+1 of 32 activation columns, arranged so that gate and up of
// one column land in the same lane and accumulator slot; the epilogue
// applies SwiGLU/GeGLU and writes the activation, rounded to the dtype, at
// the route's sorted position.  fc2: the epilogue writes float32 results at
// the route id's row of y2.
#include "gemm_common.h"

namespace qmoe {
namespace {

constexpr int kPitch = kSuperK / 2 + 4;  // LDS row pitch in 32-bit words (64 data + 4 pad)
constexpr int kXcds = 8;

// TWO: block_size 16, so the two halves of a 32-code span have their own
// scale and zero point.
// STAGED: each wavefront copies the scales of its 64 weight rows into LDS
// eight blocks at a time (one 16-byte load per lane, a row per lane, issued a
// stage ahead), and reads each super-step's scales from there; without it
// every super-step loads them from HBM, 16 rows per instruction.
// NBW: MFMA column blocks of 16 weight rows per wavefront: 4, or 2 (the
// narrow 64-row tile: twice the items for layers with few of them, so more
// wavefronts share each SIMD).
template <int DT, int BITS, bool FC1, int MT, int ZP, bool TWO, bool STAGED, int NBW>
__global__ __launch_bounds__(MT * 4, NBW == 4 ? 2 : 3) void prefill_kernel(ProjLaunch p)
{
    static_assert(NBW == 4 || (NBW == 2 && MT == kPrefillMTSmall), "the narrow tile is the 64-row one");
    constexpr Order O = code_order<DT, BITS>();
    constexpr int MB = MT / 16;
    constexpr int kThreads = MT * 4;        // 16 tile rows staged per wavefront
    constexpr int kWaveRows = 16 * NBW;     // weight rows per wavefront
    constexpr int kRows = MB * kWaveRows;   // weight rows per item
    __shared__ __attribute__((aligned(16))) uint32_t a_lds[2][MT * kPitch];
    __shared__ int row_src[MT];  // A row of tile row i
    __shared__ int row_dst[MT];  // fc2: y2 row (route id) of tile row i
    // STAGED: per wavefront, a row slot of 8 scales for each of its weight rows
    __shared__ __attribute__((aligned(16))) uint16_t sc_lds[STAGED ? MB : 1][STAGED ? kWaveRows * 8 : 1];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int c = lane & 15;
    const int K = p.K;
    const int n_items = *p.n_items;
    // fc2 may split K into p.k_split equal parts, each a work-list column of
    // its own (n-tile index ks * nt + n) writing float32 partial sums to part
    // ks of y2; the combine adds the parts in order
    const int k_split = FC1 ? 1 : p.k_split;
    const int n_super = K / kSuperK / k_split;  // super-steps per item
    const uint16_t* a_src = reinterpret_cast<const uint16_t*>(p.a);
    const uint32_t row_bytes = (uint32_t)K * BITS / 8;
    const uint32_t n_blocks = (uint32_t)(K / p.block_size);
    const uint32_t zp_bytes = BITS == 3 ? n_blocks : (n_blocks + 8 / BITS - 1) / (8 / BITS);
    const int bs_shift = __builtin_ctz((unsigned)p.block_size);  // block_size is a power of two
    const int nt = FC1 ? (p.N / 2 + kRows / 2 - 1) / (kRows / 2) : (p.N + kRows - 1) / kRows;
    const int ss_shift = bs_shift - 4;  // super-steps per scale stage: block_size / 16
    const int G = gridDim.x;  // a multiple of kXcds
    const int vb = (int)(blockIdx.x % kXcds) * (G / kXcds) + (int)(blockIdx.x / kXcds);

    for (int item = vb; item < n_items; item += G) {
        const int e = p.worklist[3 * item + 0];
        // the work-list's column index runs over nt * k_split (fc2: the K part, then the n-tile)
        const int local0 = p.worklist[3 * item + 1] * (nt * k_split) + p.worklist[3 * item + 2];
        const int first = p.offsets[e];
        const int count = p.offsets[e + 1] - first;
        const int mt_e = (count + MT - 1) / MT;
        const int mt = local0 % mt_e;  // m inner
        const int ntk = local0 / mt_e;
        const int ks = ntk / nt;        // K part
        const int ntile = ntk - ks * nt;
        const int s_begin = ks * n_super;  // first super-step of the part
        const int s_end = s_begin + n_super;
        const int row0 = first + mt * MT;
        const int rows = min(MT, count - mt * MT);

        // weight rows of this wavefront as 32-bit offsets from the expert's
        // (uniform) bases; a wavefront past the last column (partial n-tile)
        // reads the expert's first rows and stores nothing
        int col0;  // fc1: first activation column of this wave; fc2: first hidden column
        bool active;
        uint32_t wrow[NBW];  // weight row within the expert's tensor of column block nb
        // fc1 column blocks 0 and 2 are gate rows of activation columns col0 + c
        // and col0 + 16 + c, blocks 1 and 3 their up rows, placed by the gate/up
        // layout (interleaved, halves, or the separate fc3 tensor); the narrow
        // tile has blocks 0 and 1 only
        const int fusion = FC1 ? p.fusion : 1;
        const int I = p.N / 2;
        if constexpr (FC1) {
            col0 = ntile * (kRows / 2) + wave * (kWaveRows / 2);
            active = col0 < I;
#pragma unroll
            for (int h = 0; h < NBW / 2; ++h) {
                const int j = active ? col0 + 16 * h + c : 0;
                wrow[2 * h] = (uint32_t)fc1_row(fusion, j, false, I);
                wrow[2 * h + 1] = (uint32_t)fc1_row(fusion, j, true, I);
            }
        } else {
            col0 = ntile * kRows + wave * kWaveRows;
            active = col0 < p.N;
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) wrow[nb] = active ? col0 + nb * 16 + c : 0;
        }
        // rows per expert of the (first) tensor: fc1 holds only the gate rows when fc3 holds the up rows
        const int64_t rows_e = (FC1 && fusion == 0) ? I : p.N;
        const int64_t erow = (int64_t)e * rows_e;
        const uint8_t* codes_e = p.w.codes + erow * row_bytes;
        const uint16_t* scales_e = reinterpret_cast<const uint16_t*>(p.w.scales) + erow * n_blocks;
        const uint8_t* zp_e = ZP == kZpTensor ? p.w.zp + erow * zp_bytes : nullptr;
        const bool sep = FC1 && fusion == 0;  // up rows from fc3 (same width, block size and zp mode)
        const uint8_t* codes_u = sep ? p.w3.codes + erow * row_bytes : codes_e;
        const uint16_t* scales_u = sep ? reinterpret_cast<const uint16_t*>(p.w3.scales) + erow * n_blocks : scales_e;
        const uint8_t* zp_u = (ZP == kZpTensor && sep) ? p.w3.zp + erow * zp_bytes : zp_e;
        const uint8_t* codes_nb[NBW];
        const uint16_t* scales_nb[NBW];
        const uint8_t* zp_nb[NBW];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {  // odd blocks: the up rows
            codes_nb[nb] = (nb & 1) ? codes_u : codes_e;
            scales_nb[nb] = (nb & 1) ? scales_u : scales_e;
            zp_nb[nb] = (nb & 1) ? zp_u : zp_e;
        }

        // STAGED: lane l loads the scales of one of the wavefront's weight
        // rows (W = kWaveRows of them; the narrow tile's lanes W.. repeat lane
        // l - W and store nothing) into slot l: fc2 rows col0 + l; fc1 with
        // interleaved rows 2*col0 + l, slots interleaved so that the rows a
        // load of column block nb reads sit in 16 consecutive slots (no LDS
        // bank conflicts); fc1 with the other layouts the gate rows of columns
        // col0 + l (l < W/2) and the up rows of columns col0 + l - W/2.
        const int sl = lane & (kWaveRows - 1);
        const uint16_t* sc_row;
        int sc_slot_store;
        if (FC1 && fusion != 1) {
            const int jl = active ? col0 + (sl & (kWaveRows / 2 - 1)) : 0;
            const bool up = sl >= kWaveRows / 2;
            sc_row = (up ? scales_u : scales_e) + fc1_row(fusion, jl, up, I) * n_blocks;
            sc_slot_store = sl;
        } else {
            const uint32_t wr_base = active ? (FC1 ? 2 * col0 : col0) : 0;
            sc_row = scales_e + (wr_base + sl) * n_blocks;
            sc_slot_store = FC1 ? ((sl >> 1) | ((sl & 1) * (kWaveRows / 2))) : sl;
        }
        const int stage_end = s_end >> ss_shift;  // parts hold whole stages
        u32x4 sc_next;
        auto stage_load = [&](int stage) { sc_next = *reinterpret_cast<const u32x4*>(sc_row + 8 * stage); };

        __syncthreads();  // the previous item is done with row_src and a_lds
        for (int i = tid; i < MT; i += kThreads) {
            // rows past the tile repeat its first row: their outputs are never stored
            const int r = i < rows ? i : 0;
            const int route = p.sorted[row0 + r];
            row_src[i] = FC1 ? route / p.top_k : row0 + r;
            row_dst[i] = route;
        }
        __syncthreads();

        // A staging: wavefront w stages tile rows [16w, 16w+16) of each
        // super-step.  Load q of a thread reads the 16-byte chunk (lane & 15)
        // of row 16w + 4q + (lane >> 4), so each instruction covers four rows
        // with whole 128-byte lines; the chunk is permuted to its MFMA step on
        // the way to LDS (int2's order pairs neighbouring chunks, exchanged
        // between lanes l and l^1).
        const int a_j = lane & 15;
        const int a_r0 = 16 * wave + (lane >> 4);
        uint32_t a_off[4];  // element offsets (the host keeps A below 2^32 elements)
#pragma unroll
        for (int q = 0; q < 4; ++q) a_off[q] = (uint32_t)row_src[a_r0 + 4 * q] * (uint32_t)K + 8 * a_j;
        u32x4 a_stage[4];
        auto load_a = [&](int s) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                a_stage[q] = *reinterpret_cast<const u32x4*>(a_src + (a_off[q] + (uint32_t)(s * kSuperK)));
            }
        };
        auto store_a = [&](uint32_t* buf) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                u32x4 v;
                if constexpr (O == Order::kStride8) v = permute_chunk_pair(a_stage[q], lane & 1);
                else v = permute_chunk<O>(a_stage[q]);
                *reinterpret_cast<u32x4*>(buf + (a_r0 + 4 * q) * kPitch + 4 * a_j) = v;
            }
        };
        // scale and zero-point byte of the block holding input kk of row nb
        auto params = [&](int nb, int kk) {
            RawParams q;
            q.blk = kk >> bs_shift;
            if constexpr (STAGED) {
                // slot of column block nb's row c (see the staging above)
                constexpr int kSlot[4] = {0, FC1 ? kWaveRows / 2 : 16, FC1 ? 16 : 32, 48};
                q.scale = sc_lds[wave][(c + kSlot[nb]) * 8 + (q.blk & 7)];
            } else {
                q.scale = scales_nb[nb][wrow[nb] * n_blocks + q.blk];
            }
            q.zp = 0;
            if constexpr (ZP == kZpTensor) {
                q.zp = zp_nb[nb][wrow[nb] * zp_bytes + (BITS == 3 ? q.blk : q.blk / (8 / BITS))];
            }
            return q;
        };
        auto load_b = [&](int s, Span<BITS> (&sp)[NBW], RawParams (&bp)[NBW]) {
            const int kk = s * kSuperK + 32 * g;
            if constexpr (STAGED) {
                if ((s & ((1 << ss_shift) - 1)) == 0) {  // first super-step of a stage
                    if (lane < kWaveRows) *reinterpret_cast<u32x4*>(&sc_lds[wave][sc_slot_store * 8]) = sc_next;
                    const int next = (s >> ss_shift) + 1;
                    if (next < stage_end) stage_load(next);
                }
            }
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                sp[nb] = load_span<BITS>(codes_nb[nb] + wrow[nb] * row_bytes, kk);
                bp[nb] = params(nb, kk);
            }
        };

        f32x4 acc[MB][NBW];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

        auto compute = [&](const uint32_t* buf, const Span<BITS> (&cur)[NBW], const RawParams (&cbp)[NBW],
                           int s) {
            const int kk = s * kSuperK + 32 * g;
            auto frag = [&](int mb, int t) {
                return *reinterpret_cast<const u32x4*>(buf + (mb * 16 + c) * kPitch + 16 * g + 4 * t);
            };
            auto dq = [&](int t, int nb) {
                const RawParams rq = (TWO && t >= 2) ? params(nb, kk + 16) : cbp[nb];
                const BlockParams q = decode_params<DT, BITS, ZP>(rq, p.w.zp_fallback);
                return dequant_zp<DT, BITS, ZP>(cur[nb], t, q);
            };
            if constexpr (MT == kPrefillMTSmall) {
                // The 64-row tile often runs one wavefront per SIMD, with no
                // partner to fill its waits, so the step is software-pipelined
                // by hand: fragment f = 4t + mb is read two fragments ahead of
                // its MFMAs, and step t + 1's B registers are dequantized one
                // column block per row block, between the MFMAs of step t.
                // The scheduling barriers keep that order.
                static_assert(MB == 4 && NBW <= MB, "at most one column block dequantized per row block");
                constexpr int kF = 4 * MB;
                u32x4 ring[3];
                ring[0] = frag(0, 0);
                ring[1] = frag(1, 0);
                u32x4 bf[NBW], bn[NBW];
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) bf[nb] = dq(0, nb);
#pragma unroll
                for (int f = 0; f < kF; ++f) {
                    const int t = f / MB, mb = f % MB;
                    if (f + 2 < kF) ring[(f + 2) % 3] = frag((f + 2) % MB, (f + 2) / MB);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = Dt<DT>::mfma(ring[f % 3], bf[nb], acc[mb][nb]);
                    if (t + 1 < 4 && mb < NBW) bn[mb] = dq(t + 1, mb);
                    __builtin_amdgcn_sched_barrier(0);
                    if (mb == MB - 1) {
#pragma unroll
                        for (int nb = 0; nb < NBW; ++nb) bf[nb] = bn[nb];
                    }
                }
            } else {
                // two wavefronts per SIMD: the compiler's own order, which
                // measured faster here than the hand-pipelined one
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    u32x4 bf[NBW];
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb) bf[nb] = dq(t, nb);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        const u32x4 af = frag(mb, t);
#pragma unroll
                        for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = Dt<DT>::mfma(af, bf[nb], acc[mb][nb]);
                    }
                }
            }
        };

        Span<BITS> sp[NBW];
        RawParams bp[NBW];
        if constexpr (STAGED) stage_load(s_begin >> ss_shift);
        load_a(s_begin);
        load_b(s_begin, sp, bp);
        for (int s = s_begin; s < s_end; ++s) {
            uint32_t* buf = a_lds[s & 1];
            store_a(buf);
            Span<BITS> cur[NBW];
            RawParams cbp[NBW];
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                cur[nb] = sp[nb];
                cbp[nb] = bp[nb];
            }
            if (s + 1 < s_end) {  // in flight during the barrier and the MFMAs below
                load_a(s + 1);
                load_b(s + 1, sp, bp);
            }
            __syncthreads();
            // the MFMA phase at raised issue priority, so a wavefront that
            // reaches it is not held behind its SIMD partner's staging work
            __builtin_amdgcn_s_setprio(1);
            compute(buf, cur, cbp, s);
            __builtin_amdgcn_s_setprio(0);
        }

        if (!active) continue;
        // expert biases of this lane's four output columns [qmoe.rs,
        // qmoe_linear_impl: the bias entry of (expert, output row) is added to
        // the float32 projection output]; fc2 adds its bias in K part 0 only
        float bias_v[NBW];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) bias_v[nb] = 0.f;
        if constexpr (FC1) {
            const int js[2] = {col0 + c, col0 + 16 + c};
#pragma unroll
            for (int h = 0; h < NBW / 2; ++h) {
                if (p.bias) bias_v[2 * h] = p.bias[erow + fc1_row(fusion, js[h], false, I)];
                if (sep) {
                    if (p.bias3) bias_v[2 * h + 1] = p.bias3[erow + js[h]];
                } else if (p.bias) {
                    bias_v[2 * h + 1] = p.bias[erow + fc1_row(fusion, js[h], true, I)];
                }
            }
        } else if (p.bias && ks == 0) {
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) bias_v[nb] = p.bias[erow + col0 + nb * 16 + c];
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = mb * 16 + 4 * g + i;
                if (m >= rows) continue;
                if constexpr (FC1) {
                    uint16_t* out = reinterpret_cast<uint16_t*>(p.act_out) + (int64_t)(row0 + m) * I;
#pragma unroll
                    for (int h = 0; h < NBW / 2; ++h) {
                        out[col0 + 16 * h + c] = Dt<DT>::from_float(act_value<DT>(
                            p.act, acc[mb][2 * h][i] + bias_v[2 * h], acc[mb][2 * h + 1][i] + bias_v[2 * h + 1], p.ap));
                    }
                } else {
                    float* out = p.y2 + ks * p.part_stride + (int64_t)row_dst[m] * p.N;
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb) out[col0 + nb * 16 + c] = acc[mb][nb][i] + bias_v[nb];
                }
            }
        }
    }
}

// Compute units of the current device (cached per device).
int device_cus()
{
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        hipDeviceProp_t prop;
        cus[dev] = hipGetDeviceProperties(&prop, dev) == hipSuccess ? prop.multiProcessorCount : 256;
    }
    return cus[dev];
}

// Persistent grid: as many workgroups as are resident at once (never more
// than the item bound), rounded up to a multiple of the XCD count.
template <class Kernel>
int64_t persistent_grid(Kernel kernel, int threads, int64_t item_bound)
{
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
        per_cu < 1) {
        per_cu = 1;
    }
    int64_t g = (int64_t)device_cus() * per_cu;
    if (item_bound < g) g = item_bound;
    return (g + kXcds - 1) / kXcds * kXcds;
}

// Scales can be staged eight blocks at a time when every K part of a row
// holds whole stages and the 16-byte loads are aligned.
inline bool can_stage(const ProjLaunch& p, bool fc1)
{
    const int parts = fc1 ? 1 : p.k_split;
    // a K part holds a whole number (at least one) of 8-block stages; a part
    // shorter than a block has no stage of its own
    return p.block_size >= 32 && (p.K / parts) % (8 * p.block_size) == 0 &&
           reinterpret_cast<uintptr_t>(p.w.scales) % 16 == 0;
}

template <class Kernel>
hipError_t run(Kernel kernel, const ProjLaunch& p, int threads, hipStream_t s)
{
    const int64_t grid = persistent_grid(kernel, threads, p.grid > 0 ? p.grid : 1);
    launch(kernel, dim3((unsigned)grid), dim3(threads), s, p);
    return hipGetLastError();
}

template <bool FC1, int DT, int BITS, int MT, int ZP, int NBW>
hipError_t launch_nbw(const ProjLaunch& p, hipStream_t s)
{
    if (can_stage(p, FC1)) return run(prefill_kernel<DT, BITS, FC1, MT, ZP, false, true, NBW>, p, MT * 4, s);
    if constexpr (MT == kPrefillMTSmall) {
        if (p.block_size < 32) return run(prefill_kernel<DT, BITS, FC1, MT, ZP, true, false, NBW>, p, MT * 4, s);
        return run(prefill_kernel<DT, BITS, FC1, MT, ZP, false, false, NBW>, p, MT * 4, s);
    }
    return hipErrorInvalidValue;  // the large tile always stages its scales
}

template <bool FC1, int DT, int BITS, int MT, int ZP>
hipError_t launch_one(const ProjLaunch& p, hipStream_t s)
{
    if (!FC1 && (p.k_split < 1 || p.K % (p.k_split * kSuperK))) return hipErrorInvalidValue;
    if constexpr (MT == kPrefillMTSmall) {
        if (p.nbw == 2) return launch_nbw<FC1, DT, BITS, MT, ZP, 2>(p, s);
    }
    if (p.nbw != 4) return hipErrorInvalidValue;
    return launch_nbw<FC1, DT, BITS, MT, ZP, 4>(p, s);
}

// The large tile serves the fast zero-point modes with stageable scales only
// (the host picks the small tile otherwise).
template <bool FC1, int DT, int BITS, int MT>
hipError_t launch_zp(const ProjLaunch& p, hipStream_t s)
{
    switch (zp_mode(p.w)) {
    case kZpConst: return launch_one<FC1, DT, BITS, MT, kZpConst>(p, s);
    case kZpTensor: return launch_one<FC1, DT, BITS, MT, kZpTensor>(p, s);
    default:
        if constexpr (MT == kPrefillMTSmall) return launch_one<FC1, DT, BITS, MT, kZpGeneric>(p, s);
        return hipErrorInvalidValue;
    }
}

template <bool FC1, int DT, int MT>
hipError_t launch_bits(const ProjLaunch& p, hipStream_t s)
{
    switch (p.w.bits) {
    case 2: return launch_zp<FC1, DT, 2, MT>(p, s);
    case 3: return launch_zp<FC1, DT, 3, MT>(p, s);
    case 4: return launch_zp<FC1, DT, 4, MT>(p, s);
    default: break;
    }
    if constexpr (MT == kPrefillMTSmall) {  // 1- and 8-bit codes take the small tile
        if (p.w.bits == 1) return launch_zp<FC1, DT, 1, MT>(p, s);
        if (p.w.bits == 8) return launch_zp<FC1, DT, 8, MT>(p, s);
    }
    return hipErrorInvalidValue;
}

template <bool FC1>
hipError_t launch_prefill(const ProjLaunch& p, int dtype, hipStream_t s)
{
    if (p.m_tile == kPrefillMTLarge) {
        return dtype == kBF16 ? launch_bits<FC1, kBF16, kPrefillMTLarge>(p, s)
                              : launch_bits<FC1, kF16, kPrefillMTLarge>(p, s);
    }
    if (p.m_tile == kPrefillMTSmall) {
        return dtype == kBF16 ? launch_bits<FC1, kBF16, kPrefillMTSmall>(p, s)
                              : launch_bits<FC1, kF16, kPrefillMTSmall>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fc1_prefill(const ProjLaunch& p, int dtype, hipStream_t s)
{
    return launch_prefill<true>(p, dtype, s);
}

hipError_t launch_fc2_prefill(const ProjLaunch& p, int dtype, hipStream_t s)
{
    return launch_prefill<false>(p, dtype, s);
}

}  // namespace qmoe
