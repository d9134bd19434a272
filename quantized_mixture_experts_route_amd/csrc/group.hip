// group.hip -- expert grouping and tile work-lists in one workgroup.
//
// [qmoe.rs, launch_grouping]: per-expert route counts, their exclusive
// prefix sum (offsets), and the route ids grouped by expert.  Here the order
// inside a group is ascending route id, so the result is unique.
// [gemm_quant_moe.rs, moe_build_tile_worklist]: one item per (expert,
// m-tile, n-tile) of every expert with rows, experts ascending.  Items are
// three int32 {expert, m, n} so that n is not limited to 6 bits.
//
// Layout of the work: the R routes are cut into kWaves contiguous segments,
// one per wavefront.  Pass 1 counts each segment's routes per expert into an
// LDS table cnt[wave][expert].  A scan over (expert, wave) turns the table
// into each segment's first output slot per expert.  Pass 2 walks every
// segment again, 64 routes at a time and in order; lanes holding the same
// expert find each other with ballots over the expert's bits, take ranks
// from the popcount of lower peers, and the highest peer advances the slot.
// Nothing depends on atomic ordering, so the output is deterministic.
#include "qmoe_device.h"
#include "qmoe_internal.h"

namespace qmoe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxExperts = 1024;

// Exclusive scan of v[0..n) in LDS (n <= kMaxExperts); returns the total.
// Wavefront 0 scans 64 values at a time with shuffles and carries the sum
// from chunk to chunk; the others wait at the one barrier at the end (n is
// the expert count, so a workgroup-wide scan would cost more barriers than
// it saves).
__device__ int block_exclusive_scan(int* v, int n, int* part)
{
    const int tid = threadIdx.x;
    if (tid < kWave) {
        int carry = 0;
        for (int base = 0; base < n; base += kWave) {
            const int i = base + tid;
            const int x = i < n ? v[i] : 0;
            int incl = x;
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const int y = __shfl_up(incl, d, kWave);
                if (tid >= d) incl += y;
            }
            if (i < n) v[i] = carry + incl - x;
            carry += __shfl(incl, kWave - 1, kWave);
        }
        if (tid == 0) part[0] = carry;
    }
    __syncthreads();
    const int total = part[0];
    __syncthreads();  // part is reused by the next scan
    return total;
}

// Emits work-list triples {e, m, n} for items [0, min(total, cap)).
__device__ void emit_items(const int* item_base, int E, int n_tiles, int total, int32_t* wl,
                           int64_t cap)
{
    const int64_t limit = total < cap ? total : cap;
    for (int64_t idx = threadIdx.x; idx < limit; idx += kThreads) {
        // last expert whose first item is <= idx (empty experts share their
        // successor's base, so the last one of a run is the non-empty one)
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (item_base[mid] <= idx) lo = mid; else hi = mid - 1;
        }
        const int local = (int)idx - item_base[lo];
        wl[3 * idx + 0] = lo;
        wl[3 * idx + 1] = local / n_tiles;
        wl[3 * idx + 2] = local % n_tiles;
    }
}

__global__ __launch_bounds__(kThreads) void group_kernel(
    const int32_t* __restrict__ ids, int R, int E, int m_tile, int nt1,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted, int32_t* __restrict__ wl1,
    int64_t cap1, int32_t* __restrict__ n1, int nt2, int32_t* __restrict__ wl2, int64_t cap2,
    int32_t* __restrict__ n2)
{
    __shared__ int cnt[kWaves][kMaxExperts];
    __shared__ int total[kMaxExperts];
    __shared__ int items[kMaxExperts];
    __shared__ int part[kThreads];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int seg = (R + kWaves - 1) / kWaves;
    const int seg_lo = wave * seg < R ? wave * seg : R;
    const int seg_hi = seg_lo + seg < R ? seg_lo + seg : R;

    for (int i = tid; i < kWaves * E; i += kThreads) {
        cnt[i / E][i % E] = 0;
    }
    __syncthreads();

    // pass 1: per-segment counts (LDS atomics only count; the sum is order-free)
    for (int r = seg_lo + lane; r < seg_hi; r += kWave) {
        const int e = ids[r];
        if (e >= 0 && e < E) atomicAdd(&cnt[wave][e], 1);
    }
    __syncthreads();

    // per expert: running sum over segments, then scan over experts
    for (int e = tid; e < E; e += kThreads) {
        int run = 0;
        for (int w = 0; w < kWaves; ++w) {
            const int c = cnt[w][e];
            cnt[w][e] = run;
            run += c;
        }
        total[e] = run;
        items[e] = run > 0 ? ((run + m_tile - 1) / m_tile) : 0;  // m-tiles per expert
    }
    __syncthreads();
    const int grouped = block_exclusive_scan(total, E, part);  // total[e] -> offsets[e]
    for (int e = tid; e < E; e += kThreads) {
        offsets[e] = total[e];
        for (int w = 0; w < kWaves; ++w) cnt[w][e] += total[e];
    }
    if (tid == 0) offsets[E] = grouped;
    __syncthreads();

    // pass 2: stable placement, one wavefront per segment, 64 routes at a time
    const int ebits = E > 1 ? 32 - __builtin_clz((unsigned)(E - 1)) : 1;
    for (int base = seg_lo; base < seg_hi; base += kWave) {
        const int r = base + lane;
        const int e = r < seg_hi ? ids[r] : -1;
        const bool valid = e >= 0 && e < E;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < ebits; ++b) {
            const bool bit = valid && ((e >> b) & 1);
            const uint64_t set = __ballot(bit);
            peers &= bit ? set : ~set;
        }
        if (valid) {
            const uint64_t below = peers & ((1ull << lane) - 1ull);
            const int rank = __popcll(below);
            const int pos = cnt[wave][e] + rank;
            sorted[pos] = r;
        }
        __builtin_amdgcn_wave_barrier();
        if (valid && (peers >> lane) == 1ull) {  // highest lane of its peer set
            cnt[wave][e] += __popcll(peers);
        }
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();

    // work-lists: items per expert = m-tiles * n-tiles, scanned over experts
    for (int pass = 0; pass < 2; ++pass) {
        const int nt = pass == 0 ? nt1 : nt2;
        int32_t* wl = pass == 0 ? wl1 : wl2;
        int32_t* n_out = pass == 0 ? n1 : n2;
        const int64_t cap = pass == 0 ? cap1 : cap2;
        if (nt <= 0 || wl == nullptr) continue;
        for (int e = tid; e < E; e += kThreads) total[e] = items[e] * nt;
        __syncthreads();
        const int n_total = block_exclusive_scan(total, E, part);
        emit_items(total, E, nt, n_total, wl, cap);
        if (tid == 0) *n_out = n_total;
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_group(const int32_t* ids, int R, int E, int m_tile, int nt1, int32_t* offsets,
                        int32_t* sorted, int32_t* wl1, int64_t cap1, int32_t* n1, int nt2,
                        int32_t* wl2, int64_t cap2, int32_t* n2, hipStream_t s)
{
    launch(group_kernel, dim3(1), dim3(kThreads), s, ids, R, E, m_tile, nt1,
                       offsets, sorted, wl1, cap1, n1, nt2, wl2, cap2, n2);
    return hipGetLastError();
}

}  // namespace qmoe
