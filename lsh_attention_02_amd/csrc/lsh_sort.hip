// Stable sort of positions by bucket, one segment per (batch row, head, round)
// (ai-scholar Reformer article, section on LSH attention; modulabs-hub notes,
// "LSH attention": tokens sorted by bucket, then cut into equal chunks).
//
// Counting sort in three launches:
//   k_sort_hist     one workgroup per (segment, tile): LDS histogram of the
//                   tile's buckets -> counters[seg][tile][bucket]
//   k_sort_scan     one workgroup per segment: counters become the first slot
//                   of each (tile, bucket): sum of all earlier buckets plus the
//                   same bucket in earlier tiles
//   k_sort_scatter  one workgroup per (segment, tile): walks its tile in
//                   position order, 256 positions at a time; inside a wave,
//                   equal buckets are ranked by lane with ballots; the four
//                   waves take their offsets in order (barrier phases), so equal
//                   buckets keep position order across the whole segment.
// Outputs: perm[seg][slot] = position and cid[b,h][position][round] = slot / chunk
// (with the same-bucket variant: slot / chunk + 2 * rank of the bucket among the
// segment's non-empty buckets, computed by the scan).
#include "lsh_device.h"
#include "lsh_internal.h"

#include <mutex>

namespace lshk {
namespace {

constexpr int SORT_THREADS = 256;
constexpr int SCAN_THREADS = 1024;

__global__ __launch_bounds__(SORT_THREADS)
void k_sort_hist(const int32_t* __restrict__ buckets, int32_t* __restrict__ counters, int L,
                 int nb, int tile, int ntiles)
{
    extern __shared__ int hist[];
    const long seg = blockIdx.x / ntiles;
    const int t = blockIdx.x % ntiles;
    for (int b = threadIdx.x; b < nb; b += SORT_THREADS) hist[b] = 0;
    __syncthreads();
    const int32_t* bk = buckets + seg * L;
    const int p1 = min(L, (t + 1) * tile);
    for (int p = t * tile + threadIdx.x; p < p1; p += SORT_THREADS) {
        const int b = bk[p];
        if ((unsigned)b < (unsigned)nb) atomicAdd(&hist[b], 1);
    }
    __syncthreads();
    int32_t* out = counters + (seg * ntiles + t) * (long)nb;
    for (int b = threadIdx.x; b < nb; b += SORT_THREADS) out[b] = hist[b];
}

// Inclusive scan over the block; returns the block total in *total.
__device__ __forceinline__ int block_inclusive_scan(int x, int* wave_sums, int* total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int NW = SCAN_THREADS / 64;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) wave_sums[wave] = x;
    __syncthreads();
    if (wave == 0) {
        int s = lane < NW ? wave_sums[lane] : 0;
#pragma unroll
        for (int off = 1; off < NW; off <<= 1) {
            const int y = __shfl_up(s, off);
            if (lane >= off) s += y;
        }
        if (lane < NW) wave_sums[lane] = s;
    }
    __syncthreads();
    if (wave > 0) x += wave_sums[wave - 1];
    *total = wave_sums[NW - 1];
    __syncthreads();
    return x;
}

// ranks (may be null): ranks[seg][b] = number of non-empty buckets below b in
// the segment (used by the same-bucket variant's window ids).
__global__ __launch_bounds__(SCAN_THREADS)
void k_sort_scan(int32_t* __restrict__ counters, int32_t* __restrict__ ranks, int nb, int ntiles)
{
    __shared__ int wave_sums[SCAN_THREADS / 64];
    int32_t* c = counters + (long)blockIdx.x * ntiles * nb;
    int carry = 0, rank_carry = 0;
    for (int b0 = 0; b0 < nb; b0 += SCAN_THREADS) {
        const int b = b0 + threadIdx.x;
        int tot = 0;
        if (b < nb)
            for (int t = 0; t < ntiles; ++t) tot += c[(long)t * nb + b];
        int group_total;
        const int incl = block_inclusive_scan(tot, wave_sums, &group_total);
        if (b < nb) {
            int run = carry + incl - tot;              // first slot of bucket b
            for (int t = 0; t < ntiles; ++t) {
                const int x = c[(long)t * nb + b];
                c[(long)t * nb + b] = run;
                run += x;
            }
        }
        carry += group_total;
        if (ranks != nullptr) {                        // uniform over the block
            const int nz = tot > 0 ? 1 : 0;
            int group_nz;
            const int incl_nz = block_inclusive_scan(nz, wave_sums, &group_nz);
            if (b < nb) ranks[(long)blockIdx.x * nb + b] = rank_carry + incl_nz - nz;
            rank_carry += group_nz;
        }
    }
}

// Workgroups are dispatched to the 8 XCDs round-robin by launch index, and each
// XCD has its own L2.  The scatter's perm and cid stores are small and
// interleaved: a perm line takes slots from every tile of its segment and a cid
// line takes the rounds of 8 positions from every round's segment.  The launch
// index is therefore remapped so that all workgroups sharing a key (a (batch
// row, head) when there are at least 8 of them, else a segment) run on one XCD,
// where the partial lines combine in L2 before they are written back.
constexpr int NXCD = 8;

struct ScatterMap {
    long nkeys;        // keys: (batch row, head) pairs or segments
    int per_key;       // workgroups per key
    int rounds_per_key;   // n_r when a key is a (batch row, head), else 1
};

__global__ __launch_bounds__(SORT_THREADS)
void k_sort_scatter(const int32_t* __restrict__ buckets, const int32_t* __restrict__ counters,
                    const int32_t* __restrict__ ranks, int32_t* __restrict__ perm,
                    int16_t* __restrict__ cid, int L, int nb, int nbits, int tile, int ntiles,
                    int n_r, int chunk, ScatterMap map)
{
    extern __shared__ int next_slot[];
    const int xcd = blockIdx.x % NXCD;
    const long j = blockIdx.x / NXCD;
    const long key = (j / map.per_key) * NXCD + xcd;
    if (key >= map.nkeys) return;                  // padding of the last row of keys
    const int within = (int)(j % map.per_key);
    const long seg = key * map.rounds_per_key + within / ntiles;
    const int t = within % ntiles;
    const long bh = seg / n_r;
    const int r = (int)(seg % n_r);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

    const int32_t* cnt = counters + (seg * ntiles + t) * (long)nb;
    for (int b = threadIdx.x; b < nb; b += SORT_THREADS) next_slot[b] = cnt[b];
    __syncthreads();

    const int32_t* bk = buckets + seg * L;
    int32_t* pm = perm + seg * L;
    int16_t* cd = cid + bh * (long)L * n_r;
    const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int p0 = t * tile, p1 = min(L, p0 + tile);

    for (int sub = p0; sub < p1; sub += SORT_THREADS) {
        const int p = sub + threadIdx.x;
        const int b = p < p1 ? bk[p] : -1;
        const bool valid = (unsigned)b < (unsigned)nb;
        // peers = lanes of this wave holding the same bucket
        uint64_t peers = __ballot(valid);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool set = (b >> bit) & 1;
            const uint64_t m = __ballot(set);
            peers &= set ? m : ~m;
        }
        const int rank = __popcll(peers & lanes_below);
        const int leader = valid ? (__ffsll((unsigned long long)peers) - 1) : lane;
        int base = 0;
        for (int w = 0; w < SORT_THREADS / 64; ++w) {
            __syncthreads();
            if (wave == w && valid && lane == leader) {
                base = next_slot[b];
                next_slot[b] = base + __popcll(peers);
            }
        }
        base = __shfl(base, leader);
        const int slot = base + rank;
        // slots stay in range unless the buckets or the workspace change under
        // the sort (e.g. two overlapping calls sharing one workspace)
        if (valid && (unsigned)slot < (unsigned)L) {
            pm[slot] = p;
            // chunk id; with ranks, the window id chunk + 2 * rank(bucket)
            // (at most 65534, stored as the bit pattern of an unsigned 16-bit value)
            const int id = slot / chunk + (ranks != nullptr ? 2 * ranks[seg * nb + b] : 0);
            cd[(long)p * n_r + r] = (int16_t)(uint16_t)id;
        }
    }
}

}  // namespace

SortPlan sort_plan(long bh, int L, int n_rounds, int n_buckets)
{
    // Tiles hold at least 4 positions per bucket so that the counters stay a
    // fraction of the keys; at least 2048 and at most 65536 positions.
    long tile = 2048;
    while (tile < 4L * n_buckets && tile < 65536) tile <<= 1;
    if (tile > L) tile = L;
    SortPlan p;
    p.tile = (int)tile;
    p.ntiles = (int)((L + tile - 1) / tile);
    p.nseg = bh * n_rounds;
    p.counters = (size_t)p.nseg * p.ntiles * n_buckets;
    return p;
}

hipError_t launch_sort(const int32_t* buckets, int32_t* perm, int16_t* cid, int32_t* counters,
                       int32_t* ranks, const SortPlan& plan, long bh, int L, int n_rounds,
                       int n_buckets, int chunk, hipStream_t s)
{
    const size_t lds = (size_t)n_buckets * sizeof(int);
    // Up to 32768 buckets need 128 KiB of dynamic LDS per workgroup.
    static std::once_flag attr_once;
    std::call_once(attr_once, [] {
        (void)hipFuncSetAttribute((const void*)k_sort_hist,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 32768 * sizeof(int));
        (void)hipFuncSetAttribute((const void*)k_sort_scatter,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 32768 * sizeof(int));
    });
    int nbits = 0;
    while ((1 << nbits) < n_buckets) ++nbits;
    const unsigned blocks = (unsigned)(plan.nseg * plan.ntiles);
    hipLaunchKernelGGL(k_sort_hist, dim3(blocks), dim3(SORT_THREADS), lds, s, buckets, counters, L,
                       n_buckets, plan.tile, plan.ntiles);
    hipLaunchKernelGGL(k_sort_scan, dim3((unsigned)plan.nseg), dim3(SCAN_THREADS), 0, s, counters,
                       ranks, n_buckets, plan.ntiles);
    ScatterMap map;
    if (bh >= NXCD) { map.nkeys = bh; map.rounds_per_key = n_rounds; }
    else { map.nkeys = plan.nseg; map.rounds_per_key = 1; }
    map.per_key = map.rounds_per_key * plan.ntiles;
    const long rows = (map.nkeys + NXCD - 1) / NXCD;
    const unsigned sblocks = (unsigned)(rows * NXCD * map.per_key);
    hipLaunchKernelGGL(k_sort_scatter, dim3(sblocks), dim3(SORT_THREADS), lds, s, buckets, counters,
                       ranks, perm, cid, L, n_buckets, nbits, plan.tile, plan.ntiles, n_rounds,
                       chunk, map);
    return hipGetLastError();
}

}  // namespace lshk
