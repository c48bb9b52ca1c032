// Stable sort of positions by bucket, one segment per (batch row, head, round)
// (ai-scholar Reformer article, section on LSH attention; modulabs-hub notes,
// "LSH attention": tokens sorted by bucket, then cut into equal chunks).
//
// Counting sort in two or three launches.  Counting:
//   k_sort_count    one workgroup per segment, where every tile's histogram of
//                   the segment fits in LDS: counts per (tile, bucket), then
//                   the column prefixes (the bucket in earlier tiles) and the
//                   bucket totals
//   k_sort_hist     otherwise: one workgroup per (segment, tile of positions),
//                   LDS histogram of the tile -> counters[seg][tile][bucket];
//                   then k_sort_colscan (column prefixes and totals, for the
//                   placement kernels) or k_sort_scan (first slot of each
//                   (tile, bucket), for k_sort_scatter)
// Placement:
//   k_sort_place2 / k_sort_place
//                   one workgroup per (batch row, head, tile, group of rounds),
//                   one wave per round.  The wave orders its round's buckets
//                   of the tile (stable: positions are ranked in increasing
//                   order, equal buckets inside a wave found by ballots), then
//                   writes perm in that order, so that each bucket's slots of
//                   the tile are one contiguous run of stores.  The chunk ids
//                   of the tile's positions stay in LDS until every round of
//                   the group is placed and are written as whole rows of cid.
//   k_sort_scatter  (when a round's tile does not fit in LDS: many buckets with
//                   large tiles) one workgroup per (segment, tile): walks the
//                   tile 256 positions at a time, equal buckets ranked by lane
//                   with ballots, the four waves taking their offsets in order
//                   (barrier phases).
// Outputs: perm[seg][slot] = position and cid[b,h][position][round] = slot / chunk
// (with the same-bucket variant: slot / chunk + 2 * rank of the bucket among the
// segment's non-empty buckets, computed by the scan).
//
// Why the placement is staged: every store the L2 receives is one request, and
// a store instruction whose 64 lanes hit 64 different lines costs 64 of them.
// Stored per position, perm (4 bytes) and cid (2 bytes, at a 2 * n_rounds byte
// stride) cost about one request per element each, and the L2's request rate,
// not HBM, bounded the sort.  In tile order a wave's 64 perm stores fall in a
// few runs, and the cid rows of a tile form one contiguous block.
#include "lsh_attention.h"
#include "lsh_device.h"
#include "lsh_internal.h"

#include <algorithm>
#include <mutex>
#include <type_traits>

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
    // eight loads in flight per thread before the first LDS update
    for (int p = t * tile + threadIdx.x; p < p1; p += 8 * SORT_THREADS) {
        int v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = p + k * SORT_THREADS < p1 ? bk[min(p + k * SORT_THREADS, p1 - 1)] : -1;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (p + k * SORT_THREADS < p1) LSH_CHECK((unsigned)v[k] < (unsigned)nb);
            if ((unsigned)v[k] < (unsigned)nb) atomicAdd(&hist[v[k]], 1);
        }
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
// Thread b of a block of SCAN_THREADS buckets owns column b: up to SCAN_KEEP
// tiles' counts are loaded at once and kept in registers; more tiles take two
// passes (sum, then rewrite) in batches of SCAN_KEEP loads.
constexpr int SCAN_KEEP = 16;

__global__ __launch_bounds__(SCAN_THREADS)
void k_sort_scan(int32_t* __restrict__ counters, int32_t* __restrict__ ranks, int nb, int ntiles)
{
    __shared__ int wave_sums[SCAN_THREADS / 64];
    int32_t* c = counters + (long)blockIdx.x * ntiles * nb;
    int carry = 0, rank_carry = 0;
    for (int b0 = 0; b0 < nb; b0 += SCAN_THREADS) {
        const int b = b0 + threadIdx.x;
        const bool own = b < nb;
        int x[SCAN_KEEP];
        int tot = 0;
        if (own) {
            for (int t0 = 0; t0 < ntiles; t0 += SCAN_KEEP) {
#pragma unroll
                for (int k = 0; k < SCAN_KEEP; ++k)
                    x[k] = t0 + k < ntiles ? c[(long)(t0 + k) * nb + b] : 0;
#pragma unroll
                for (int k = 0; k < SCAN_KEEP; ++k) tot += x[k];
            }
        }
        int group_total;
        const int incl = block_inclusive_scan(tot, wave_sums, &group_total);
        if (own) {
            int run = carry + incl - tot;              // first slot of bucket b
            if (ntiles <= SCAN_KEEP) {
#pragma unroll
                for (int k = 0; k < SCAN_KEEP; ++k)
                    if (k < ntiles) {
                        c[(long)k * nb + b] = run;
                        run += x[k];
                    }
            } else {
                for (int t0 = 0; t0 < ntiles; t0 += SCAN_KEEP) {
#pragma unroll
                    for (int k = 0; k < SCAN_KEEP; ++k)
                        x[k] = t0 + k < ntiles ? c[(long)(t0 + k) * nb + b] : 0;
#pragma unroll
                    for (int k = 0; k < SCAN_KEEP; ++k)
                        if (t0 + k < ntiles) {
                            c[(long)(t0 + k) * nb + b] = run;
                            run += x[k];
                        }
                }
            }
        }
        carry += group_total;
        if (ranks != nullptr) {                        // uniform over the block
            const int nz = tot > 0 ? 1 : 0;
            int group_nz;
            const int incl_nz = block_inclusive_scan(nz, wave_sums, &group_nz);
            if (own) ranks[(long)blockIdx.x * nb + b] = rank_carry + incl_nz - nz;
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
        if (p < p1) LSH_CHECK(valid);
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
        if (valid) LSH_CHECK((unsigned)slot < (unsigned)L);
        if (valid && (unsigned)slot < (unsigned)L) {
            pm[slot] = p;
            // chunk id; with ranks, the window id chunk + 2 * rank(bucket)
            // (at most 65534, stored as the bit pattern of an unsigned 16-bit value)
            const int id = slot / chunk + (ranks != nullptr ? 2 * ranks[seg * nb + b] : 0);
            cd[(long)p * n_r + r] = (int16_t)(uint16_t)id;
        }
    }
}

// ---------------------------------------------------------------------------
// k_sort_colscan: the column half of the scan, for k_sort_place.  One thread per
// (segment, bucket): counters[seg][tile][b] becomes the number of positions of
// bucket b in the earlier tiles, and totals[seg][b] the bucket's count.  The
// offsets along the bucket axis are summed by k_sort_place itself.
constexpr int COLSCAN_THREADS = 256;

__global__ __launch_bounds__(COLSCAN_THREADS)
void k_sort_colscan(int32_t* __restrict__ counters, int32_t* __restrict__ totals, int nb, int ntiles,
                    int blocks_per_seg)
{
    const long seg = blockIdx.x / blocks_per_seg;
    const int b = (blockIdx.x % blocks_per_seg) * COLSCAN_THREADS + threadIdx.x;
    if (b >= nb) return;
    int32_t* c = counters + seg * ntiles * (long)nb + b;
    int run = 0;
    for (int t0 = 0; t0 < ntiles; t0 += SCAN_KEEP) {
        int x[SCAN_KEEP];
#pragma unroll
        for (int k = 0; k < SCAN_KEEP; ++k) x[k] = c[(long)min(t0 + k, ntiles - 1) * nb];
#pragma unroll
        for (int k = 0; k < SCAN_KEEP; ++k)
            if (t0 + k < ntiles) {
                c[(long)(t0 + k) * nb] = run;
                run += x[k];
            }
    }
    totals[seg * nb + b] = run;
}

// ---------------------------------------------------------------------------
// k_sort_count: k_sort_hist and k_sort_colscan in one launch, where every tile's
// histogram of a segment fits in LDS as 16-bit counts (tiles of at most 32768
// positions).  A segment's buckets are split into nsplit equal ranges, one
// workgroup each: it reads all of the segment's buckets, counts those in its
// range per (tile, bucket) in LDS, then thread b writes the column prefix of
// bucket b (its count in the earlier tiles) for every tile, and its total.  The
// counters go to HBM once, instead of being written, re-read and rewritten.  The
// workgroups of one segment run on one XCD, so that all but the first read of
// its buckets come from that XCD's L2 (see ScatterMap).
constexpr int COUNT_THREADS = 1024;
constexpr int COUNT_LOADS = 16;            // loads in flight per thread
constexpr size_t COUNT_LDS_LIMIT = 128 * 1024;

__global__ __launch_bounds__(COUNT_THREADS)
void k_sort_count(const int32_t* __restrict__ buckets, int32_t* __restrict__ colpre,
                  int32_t* __restrict__ totals, long nseg, int L, int nb, int tile_shift, int ntiles,
                  int nsplit)
{
    extern __shared__ uint32_t cnt2[];          // [tile][bucket / 2 in the range]: two 16-bit counts
    const int xcd = blockIdx.x % NXCD;
    const long j = blockIdx.x / NXCD;
    const long seg = (j / nsplit) * NXCD + xcd;
    if (seg >= nseg) return;                    // padding of the last row of segments
    const int bsz = nb / nsplit;                // even
    const int b0 = (int)(j % nsplit) * bsz;
    const int half = bsz >> 1;
    for (int i = threadIdx.x; i < ntiles * half; i += COUNT_THREADS) cnt2[i] = 0u;
    __syncthreads();
    const int32_t* bk = buckets + seg * (long)L;
    auto add = [&](int p, int b) __attribute__((always_inline)) {
        LSH_CHECK((unsigned)b < (unsigned)nb);
        const unsigned x = (unsigned)(b - b0);
        if (x < (unsigned)bsz)
            atomicAdd(&cnt2[(p >> tile_shift) * half + (x >> 1)], 1u << ((x & 1) << 4));
    };
    if ((L & 3) == 0) {                         // 16-byte aligned rows: 4 positions per load
        const int L4 = L >> 2;
        for (int i0 = threadIdx.x; i0 < L4; i0 += COUNT_LOADS * COUNT_THREADS) {
            int4 v[COUNT_LOADS];
#pragma unroll
            for (int k = 0; k < COUNT_LOADS; ++k)
                v[k] = reinterpret_cast<const int4*>(bk)[min(i0 + k * COUNT_THREADS, L4 - 1)];
#pragma unroll
            for (int k = 0; k < COUNT_LOADS; ++k) {
                if (i0 + k * COUNT_THREADS < L4) {
                    const int p = 4 * (i0 + k * COUNT_THREADS);
                    add(p, v[k].x); add(p + 1, v[k].y); add(p + 2, v[k].z); add(p + 3, v[k].w);
                }
            }
        }
    } else {
        for (int i0 = threadIdx.x; i0 < L; i0 += COUNT_LOADS * COUNT_THREADS) {
            int v[COUNT_LOADS];
#pragma unroll
            for (int k = 0; k < COUNT_LOADS; ++k) v[k] = bk[min(i0 + k * COUNT_THREADS, L - 1)];
#pragma unroll
            for (int k = 0; k < COUNT_LOADS; ++k)
                if (i0 + k * COUNT_THREADS < L) add(i0 + k * COUNT_THREADS, v[k]);
        }
    }
    __syncthreads();
    for (int x = threadIdx.x; x < bsz; x += COUNT_THREADS) {
        int32_t* cp = colpre + seg * (long)ntiles * nb + b0 + x;
        const int sh = (x & 1) << 4;
        uint32_t run = 0;
        for (int t = 0; t < ntiles; ++t) {
            const uint32_t c = (cnt2[t * half + (x >> 1)] >> sh) & 0xFFFFu;
            cp[(long)t * nb] = (int32_t)run;
            run += c;
        }
        totals[seg * (long)nb + b0 + x] = (int32_t)run;
    }
}

// Bucket ranges per segment for k_sort_count.  Long segments (at least 32768
// positions) are split until the workgroups cover the CUs, up to 4 ranges of an
// even number of buckets: at 64K positions, 64 segments and 1024 buckets, 4
// ranges measured 11.2 us against 12.0 for one (more ranges were slower: each
// workgroup still issues an LDS atomic instruction per 64 positions, with
// fewer lanes active).  Shorter segments, and skewed bucket counts (most
// positions in a few buckets, whose range then holds most of the atomics),
// gained nothing from splitting.
inline int count_splits(long nseg, int nb, int L)
{
    int s = 1;
    while (L >= 32768 && s < 4 && nseg * s < 256 && (nb / (2 * s)) % 2 == 0) s *= 2;
    return s;
}

// ---------------------------------------------------------------------------
// k_sort_place: one workgroup per (batch row, head, tile, group of RG rounds),
// wave w placing round g * RG + w of the tile.  Per wave, in LDS:
//   cnt[nb]     u32: next tile-local sorted index of each bucket
//   rep[nb]     u32: the representative lane of each bucket in a ranking step;
//               after the ranking, dlt[nb]: first slot of (tile, bucket) in
//               the segment minus its first tile-local index, so that
//               slot = tile-local index + dlt[bucket]
//   rk[nb]      u16 (padded to 8 bytes), same-bucket variant only: 2 * rank of
//               the bucket among the round's non-empty buckets
//   bt[P]       u16 (padded to 8 bytes): bucket of each tile position, then
//               its cid value
//   stg[P]      u16: the tile's positions in sorted order
//   peer[64]    u64: per representative lane, the lanes of its bucket
// Every step issues its loads before it uses any of them: with one workgroup
// per CU and a wave per SIMD nothing else hides their latency.
constexpr int PLACE_MAX_WAVES = 16;
constexpr int PLACE_BATCH = 8;              // ranking steps whose LDS atomics are issued together
constexpr int PLACE_LOADS = 16;             // loads in flight per lane

struct PlaceLayout {                         // offsets in 16-bit units within a wave's region
    int rep, rk, bt, stg, peer, words;
};

__host__ __device__ inline PlaceLayout place_layout(int nb, int P, bool same)
{
    auto up4 = [](int x) { return (x + 3) & ~3; };
    PlaceLayout l;
    l.rep = 2 * nb;                          // u32 per bucket; after the ranking, dlt
    l.rk = 4 * nb;
    l.bt = l.rk + (same ? up4(nb) : 0);
    l.stg = l.bt + up4(P);
    l.peer = l.stg + up4(P);                 // u64 per lane
    l.words = (l.peer + 4 * 64) / 2;
    return l;
}

// Stores the cid values of a tile's positions for RG rounds: one vector store of
// the RG u16 values per position (RG = 1, 2, 4, 8), or element by element.
template <int RGV>
__device__ __forceinline__ void store_cid_rows(int16_t* __restrict__ cd, const uint16_t* const* bts,
                                               int np, int n_r, int r0)
{
    for (int p = threadIdx.x; p < np; p += blockDim.x) {
        int16_t* dst = cd + (long)p * n_r + r0;
        if constexpr (RGV == 1) {
            dst[0] = (int16_t)bts[0][p];
        } else if constexpr (RGV == 2) {
            *reinterpret_cast<uint32_t*>(dst) = bts[0][p] | ((uint32_t)bts[1][p] << 16);
        } else if constexpr (RGV == 4) {
            u32x2 v;
            v.x = bts[0][p] | ((uint32_t)bts[1][p] << 16);
            v.y = bts[2][p] | ((uint32_t)bts[3][p] << 16);
            *reinterpret_cast<u32x2*>(dst) = v;
        } else if constexpr (RGV == 8) {
            u32x4 v;
            v.x = bts[0][p] | ((uint32_t)bts[1][p] << 16);
            v.y = bts[2][p] | ((uint32_t)bts[3][p] << 16);
            v.z = bts[4][p] | ((uint32_t)bts[5][p] << 16);
            v.w = bts[6][p] | ((uint32_t)bts[7][p] << 16);
            *reinterpret_cast<u32x4*>(dst) = v;
        }
    }
}

__device__ __forceinline__ uint32_t wave_exclusive_scan(uint32_t x, int lane, uint32_t* total)
{
    uint32_t incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    *total = __shfl(incl, 63);
    return incl - x;
}

// Inclusive sum over the 64 lanes with DPP moves: shifts by 1, 2, 4 and 8
// inside each row of 16 lanes, then the row totals carried across rows with the
// row broadcasts of lanes 15 and 31.
__device__ __forceinline__ uint32_t wave_inclusive_scan_dpp(uint32_t x)
{
    int v = (int)x;
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
    return (uint32_t)v;
}

template <bool SAME>
__global__ __launch_bounds__(PLACE_MAX_WAVES * 64)
void k_sort_place(const int32_t* __restrict__ buckets, const int32_t* __restrict__ colpre,
                  const int32_t* __restrict__ totals, int32_t* __restrict__ perm,
                  int16_t* __restrict__ cid, int L, int nb, int nbits, int P, int ntiles, int n_r,
                  int RG, int ngroups, long nkeys, int chunk, int chunk_shift)
{
    extern __shared__ uint32_t lds[];
    // all tiles of one (batch row, head, round group) on one XCD (see ScatterMap)
    const int xcd = blockIdx.x % NXCD;
    const long j = blockIdx.x / NXCD;
    const long key = (j / ntiles) * NXCD + xcd;
    if (key >= nkeys) return;                      // padding of the last row of keys
    const int t = (int)(j % ntiles);
    const long bh = key / ngroups;
    const int r0 = (int)(key % ngroups) * RG;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = r0 + w;
    const long seg = bh * n_r + r;
    const int p0 = t * P, np = min(P, L - p0);
    const PlaceLayout ly = place_layout(nb, P, SAME);

    uint16_t* base16 = reinterpret_cast<uint16_t*>(lds + (long)w * ly.words);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(base16);
    uint32_t* rep = reinterpret_cast<uint32_t*>(base16 + ly.rep);
    uint32_t* dlt = rep;                           // once the ranking is done
    uint16_t* rk = base16 + ly.rk;
    uint16_t* bt = base16 + ly.bt;
    uint16_t* stg = base16 + ly.stg;

    // 1. the round's buckets of the tile -> bt, and their histogram -> cnt
    for (int b = lane; b < nb; b += 64) {
        cnt[b] = 0;
        rep[b] = 0;
    }
    const int32_t* bk = buckets + seg * (long)L + p0;
    if ((L & 3) == 0) {                            // 16-byte aligned rows: 4 positions per load
        for (int s = 4 * lane; s < np; s += 4 * 64 * PLACE_LOADS) {
            int4 v[PLACE_LOADS];
#pragma unroll
            for (int k = 0; k < PLACE_LOADS; ++k)
                v[k] = *reinterpret_cast<const int4*>(bk + min(s + 256 * k, np - 4));   // np % 4 == 0
#pragma unroll
            for (int k = 0; k < PLACE_LOADS; ++k) {
                if (s + 256 * k < np) {
                    const int e[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
                    uint32_t h[2];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool ok = (unsigned)e[i] < (unsigned)nb;
                        LSH_CHECK(ok);
                        const uint32_t u = ok ? (uint32_t)e[i] : 0xFFFFu;
                        if (i % 2 == 0) h[i / 2] = u; else h[i / 2] |= u << 16;
                        if (ok) atomicAdd(&cnt[e[i]], 1u);
                    }
                    *reinterpret_cast<uint2*>(bt + s + 256 * k) = make_uint2(h[0], h[1]);
                }
            }
        }
    } else {
        for (int s = lane; s < np; s += 64 * PLACE_LOADS) {
            int v[PLACE_LOADS];
#pragma unroll
            for (int k = 0; k < PLACE_LOADS; ++k) v[k] = bk[min(s + 64 * k, np - 1)];
#pragma unroll
            for (int k = 0; k < PLACE_LOADS; ++k) {
                if (s + 64 * k < np) {
                    const bool ok = (unsigned)v[k] < (unsigned)nb;
                    LSH_CHECK(ok);
                    bt[s + 64 * k] = ok ? (uint16_t)v[k] : (uint16_t)0xFFFF;
                    if (ok) atomicAdd(&cnt[v[k]], 1u);
                }
            }
        }
    }
    // 2. first tile-local index of each bucket: an exclusive scan of cnt
    //    (lane l owns buckets [l * per, (l + 1) * per))
    const int per = (nb + 63) / 64;
    const int bl0 = min(nb, lane * per), bl1 = min(nb, bl0 + per);
    uint32_t s_cnt = 0;
    for (int b = bl0; b < bl1; ++b) s_cnt += cnt[b];
    uint32_t nvalid_u;
    uint32_t run_cnt = wave_exclusive_scan(s_cnt, lane, &nvalid_u);
    const int nvalid = (int)nvalid_u;
    for (int b = bl0; b < bl1; ++b) {
        const uint32_t c = cnt[b];
        cnt[b] = run_cnt;
        run_cnt += c;
    }
    // 3. rank the positions in increasing order.  Inside one step of 64
    //    positions the lanes of one bucket agree on a representative (the
    //    highest of their lane ids, an LDS max of (step + 1) * 64 + lane, above
    //    every earlier step's value), set their bits in its word of peer[] and
    //    read the word back: the lanes of equal bucket.  Across steps the
    //    per-bucket counters keep the order: one LDS add-and-return by the
    //    representative.  LDS operations of one wave execute in program order,
    //    so a batch of steps is issued before its results are waited for.
    unsigned long long* peer = reinterpret_cast<unsigned long long*>(base16 + ly.peer);
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    // Full batches run without per-position guards (a guarded LDS read becomes a
    // branch with a wait around it); the last, partial batch is guarded.
    auto rank_batch = [&](int s0, auto tail) __attribute__((always_inline)) {
        constexpr bool TAIL = decltype(tail)::value;
        int bb[PLACE_BATCH], rp[PLACE_BATCH], rnk[PLACE_BATCH], cntp[PLACE_BATCH];
        uint64_t pw[PLACE_BATCH];
        uint32_t base[PLACE_BATCH];
#pragma unroll
        for (int k = 0; k < PLACE_BATCH; ++k) {
            const int p = s0 + 64 * k + lane;
            const int b = (int)bt[TAIL ? min(p, P - 1) : p];
            bb[k] = (!TAIL || p < np) && b < nb ? b : -1;
        }
#pragma unroll
        for (int k = 0; k < PLACE_BATCH; ++k) {
            if (bb[k] >= 0) atomicMax(&rep[bb[k]], ((uint32_t)(s0 / 64 + k + 1) << 6) | (uint32_t)lane);
            rp[k] = (int)(rep[bb[k] >= 0 ? bb[k] : 0] & 63u);
        }
#pragma unroll
        for (int k = 0; k < PLACE_BATCH; ++k) {
            if (bb[k] >= 0 && rp[k] == lane) peer[lane] = 0ull;
            if (bb[k] >= 0) atomicOr(&peer[rp[k]], 1ull << lane);
            pw[k] = peer[rp[k]];
        }
#pragma unroll
        for (int k = 0; k < PLACE_BATCH; ++k) {
            rnk[k] = __popcll(pw[k] & below);
            cntp[k] = __popcll(pw[k]);
        }
#pragma unroll
        for (int k = 0; k < PLACE_BATCH; ++k) {
            base[k] = 0;
            if (bb[k] >= 0 && lane == rp[k]) base[k] = atomicAdd(&cnt[bb[k]], (uint32_t)cntp[k]);
        }
#pragma unroll
        for (int k = 0; k < PLACE_BATCH; ++k) {
            const uint32_t b0 = __shfl(base[k], rp[k]);
            if (bb[k] >= 0) stg[b0 + rnk[k]] = (uint16_t)(s0 + 64 * k + lane);
        }
    };
    int s0 = 0;
    for (; s0 + 64 * PLACE_BATCH <= np; s0 += 64 * PLACE_BATCH) rank_batch(s0, std::false_type{});
    if (s0 < np) rank_batch(s0, std::true_type{});

    // 2b. slot of each (tile, bucket) = (all positions of smaller buckets: a
    //     scan of the totals) + (the bucket in earlier tiles: colpre), stored
    //     as dlt = slot - first tile-local index.  After the ranking cnt[b] is
    //     the first index of bucket b + 1, so that of b is cnt[b - 1].
    {
        const int32_t* tot = totals + seg * (long)nb;
        const int32_t* cp = colpre + (seg * ntiles + t) * (long)nb;
        uint32_t s_tot = 0, s_nz = 0;
        for (int b0 = bl0; b0 < bl1; b0 += PLACE_LOADS) {
            int x[PLACE_LOADS];
#pragma unroll
            for (int k = 0; k < PLACE_LOADS; ++k) x[k] = tot[min(b0 + k, bl1 - 1)];
#pragma unroll
            for (int k = 0; k < PLACE_LOADS; ++k) {
                if (b0 + k < bl1) {
                    s_tot += (uint32_t)x[k];
                    s_nz += x[k] > 0 ? 1u : 0u;
                    dlt[b0 + k] = (uint32_t)x[k];          // the bucket's total, for now
                }
            }
        }
        uint32_t dummy;
        uint32_t run_tot = wave_exclusive_scan(s_tot, lane, &dummy);
        uint32_t run_nz = SAME ? wave_exclusive_scan(s_nz, lane, &dummy) : 0u;
        for (int b0 = bl0; b0 < bl1; b0 += PLACE_LOADS) {
            int x[PLACE_LOADS];
#pragma unroll
            for (int k = 0; k < PLACE_LOADS; ++k) x[k] = cp[min(b0 + k, bl1 - 1)];
#pragma unroll
            for (int k = 0; k < PLACE_LOADS; ++k) {
                if (b0 + k < bl1) {
                    const int b = b0 + k;
                    const uint32_t total = dlt[b];
                    const uint32_t first = b > 0 ? cnt[b - 1] : 0u;
                    dlt[b] = run_tot + (uint32_t)x[k] - first;
                    if constexpr (SAME) {
                        rk[b] = (uint16_t)(2 * run_nz);
                        run_nz += total > 0 ? 1u : 0u;
                    }
                    run_tot += total;
                }
            }
        }
    }

    // 4. perm in sorted order (each bucket's run of slots is contiguous); the
    //    position's cid value replaces its bucket in bt (each position once, so
    //    the reads of a batch never meet its writes)
    int32_t* pm = perm + seg * (long)L;
    auto write_batch = [&](int i0, auto tail) __attribute__((always_inline)) {
        constexpr bool TAIL = decltype(tail)::value;
        int p[PLACE_BATCH], b[PLACE_BATCH];
        uint32_t dl[PLACE_BATCH], id[PLACE_BATCH];
#pragma unroll
        for (int k = 0; k < PLACE_BATCH; ++k)
            p[k] = TAIL ? min((int)stg[min(i0 + 64 * k, P - 1)], P - 1) : (int)stg[i0 + 64 * k];
#pragma unroll
        for (int k = 0; k < PLACE_BATCH; ++k) b[k] = bt[p[k]];
#pragma unroll
        for (int k = 0; k < PLACE_BATCH; ++k) dl[k] = dlt[TAIL ? (b[k] < nb ? b[k] : 0) : b[k]];
#pragma unroll
        for (int k = 0; k < PLACE_BATCH; ++k) {
            const uint32_t slot = (uint32_t)(i0 + 64 * k) + dl[k];
            id[k] = chunk_shift >= 0 ? slot >> chunk_shift : slot / (uint32_t)chunk;
            if constexpr (SAME) id[k] += rk[TAIL ? (b[k] < nb ? b[k] : 0) : b[k]];
            // in range unless the input changed under the sort
            if (!TAIL || i0 + 64 * k < nvalid) LSH_CHECK(slot < (uint32_t)L);
            if ((!TAIL || i0 + 64 * k < nvalid) && slot < (uint32_t)L) pm[slot] = p0 + p[k];
        }
#pragma unroll
        for (int k = 0; k < PLACE_BATCH; ++k)
            if (!TAIL || i0 + 64 * k < nvalid) bt[p[k]] = (uint16_t)id[k];
    };
    int i0 = 0;
    for (; i0 + 64 * PLACE_BATCH <= nvalid; i0 += 64 * PLACE_BATCH) write_batch(i0 + lane, std::false_type{});
    if (i0 < nvalid) write_batch(i0 + lane, std::true_type{});
    __syncthreads();
    // 5. the tile's cid rows for the group's rounds
    const uint16_t* bts[PLACE_MAX_WAVES];
#pragma unroll
    for (int k = 0; k < PLACE_MAX_WAVES; ++k)
        bts[k] = reinterpret_cast<const uint16_t*>(lds + (long)k * ly.words) + ly.bt;
    int16_t* cd = cid + (bh * (long)L + p0) * n_r;
    switch (RG) {
        case 1: store_cid_rows<1>(cd, bts, np, n_r, r0); break;
        case 2: store_cid_rows<2>(cd, bts, np, n_r, r0); break;
        case 4: store_cid_rows<4>(cd, bts, np, n_r, r0); break;
        case 8: store_cid_rows<8>(cd, bts, np, n_r, r0); break;
        default:
            for (int e = threadIdx.x; e < np * RG; e += blockDim.x) {
                const int p = e / RG, k = e - p * RG;
                cd[(long)p * n_r + r0 + k] = (int16_t)bts[k][p];
            }
    }
}

// ---------------------------------------------------------------------------
// k_sort_place2: k_sort_place for tiles of at most 64 * BPL positions (BPL per
// lane), with far fewer LDS operations, most of them free of bank conflicts.
// Wave w places round r0 + w of the tile; per wave, in LDS:
//   tab[nb]   u64: low word the bucket's running count during the ranking,
//             then its first tile-local index (bits 0-15) and, same-bucket
//             variant, 2 * its rank among the round's non-empty buckets (bits
//             16-31); high word dlt = first slot of (tile, bucket) in the
//             segment minus its first tile-local index
//   stg[P]    u32: (bucket << 16) | position, in sorted order
//   bt[P]     u16: cid value of each tile position
// The tile's buckets stay in registers (position 64 k + lane in register k).
// Ranking step k: the lanes holding one bucket find each other with one ballot
// per bucket bit (the lanes whose bits all agree), the lowest of them adds the
// group's size to the bucket's count (an LDS add-and-return; the LDS
// operations of one wave execute in program order, so earlier steps come
// first), and each lane's rank is that old count plus the group members below
// it.  The histogram of the tile is the counts left at the end.
constexpr int PLACE2_MAX_BPL = 32;
// All rounds of a tile in one workgroup where they fit, so that each cid row is
// written whole by one workgroup (split rows were measured to add a write of
// the cid array's size in partial lines)
constexpr size_t PLACE2_LDS_TARGET = 160 * 1024;

struct Place2Layout {                             // offsets in bytes within a wave's region
    int stg, bt, bytes;
};

__host__ __device__ inline Place2Layout place2_layout(int nb, int P)
{
    Place2Layout l;
    l.stg = 8 * nb;
    l.bt = l.stg + 4 * P;
    l.bytes = (l.bt + 2 * P + 15) & ~15;
    return l;
}

constexpr int PLACE2_MAX_WAVES = 8;              // 256 VGPRs per lane: no spills at 32 steps

template <bool SAME, int BPL>
__global__ __launch_bounds__(PLACE2_MAX_WAVES * 64)
void k_sort_place2(const int32_t* __restrict__ buckets, const int32_t* __restrict__ colpre,
                   const int32_t* __restrict__ totals, int32_t* __restrict__ perm,
                   int16_t* __restrict__ cid, int L, int nb, int nbits, int P, int ntiles, int n_r,
                   int RG, int ngroups, long nkeys, int chunk, int chunk_shift)
{
    extern __shared__ uint32_t lds[];
    // all tiles of one (batch row, head, round group) on one XCD (see ScatterMap)
    const int xcd = blockIdx.x % NXCD;
    const long j = blockIdx.x / NXCD;
    const long key = (j / ntiles) * NXCD + xcd;
    if (key >= nkeys) return;                      // padding of the last row of keys
    const int t = (int)(j % ntiles);
    const long bh = key / ngroups;
    const int r0 = (int)(key % ngroups) * RG;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = r0 + w;
    const long seg = bh * n_r + r;
    const int p0 = t * P, np = min(P, L - p0);
    const Place2Layout ly = place2_layout(nb, P);

    char* base8 = reinterpret_cast<char*>(lds) + (long)w * ly.bytes;
    uint32_t* tab = reinterpret_cast<uint32_t*>(base8);             // tab[2 b] low, tab[2 b + 1] high
    uint32_t* stg = reinterpret_cast<uint32_t*>(base8 + ly.stg);
    uint16_t* bt = reinterpret_cast<uint16_t*>(base8 + ly.bt);

    // 1. the round's buckets of the tile into registers; counts to zero
    const int32_t* bk = buckets + seg * (long)L + p0;
    int bv[BPL];
#pragma unroll
    for (int k = 0; k < BPL; ++k) {
        const int p = 64 * k + lane;
        bv[k] = bk[min(p, np - 1)];
        if (p >= np) bv[k] = -1;
        else LSH_CHECK((unsigned)bv[k] < (unsigned)nb);
    }
    for (int b = lane; b < nb; b += 64) tab[2 * b] = 0u;

    // 2. ranks, 8 steps at a time (their group masks in registers); each
    //    step's register then holds (rank << 16) | bucket (0xFFFF: no bucket)
    constexpr int GRP = BPL < 8 ? BPL : 8;
#pragma unroll
    for (int k0 = 0; k0 < BPL; k0 += GRP) {
        uint32_t mlo[GRP], mhi[GRP];
#pragma unroll
        for (int k = 0; k < GRP; ++k) {
            const uint64_t v = __ballot((unsigned)bv[k0 + k] < (unsigned)nb);
            mlo[k] = (uint32_t)v;
            mhi[k] = (uint32_t)(v >> 32);
        }
        for (int bit = 0; bit < nbits; ++bit) {
#pragma unroll
            for (int k = 0; k < GRP; ++k) {
                const uint32_t x = (uint32_t)__builtin_amdgcn_sbfe(bv[k0 + k], bit, 1);   // 0 or ~0
                const uint64_t B = __ballot(x != 0u);
                // one three-input bitwise instruction per half
                mlo[k] &= ~((uint32_t)B ^ x);
                mhi[k] &= ~((uint32_t)(B >> 32) ^ x);
            }
        }
        uint64_t m[GRP];
#pragma unroll
        for (int k = 0; k < GRP; ++k) m[k] = ((uint64_t)mhi[k] << 32) | mlo[k];
        uint32_t old[GRP];
        int rep[GRP];
#pragma unroll
        for (int k = 0; k < GRP; ++k) {
            const int b = bv[k0 + k];
            const bool ok = (unsigned)b < (unsigned)nb;
            rep[k] = ok ? __builtin_ctzll(m[k]) : lane;
            old[k] = 0u;
            if (ok && rep[k] == lane) old[k] = atomicAdd(&tab[2 * b], (uint32_t)__popcll(m[k]));
        }
#pragma unroll
        for (int k = 0; k < GRP; ++k) {
            const int b = bv[k0 + k];
            const bool ok = (unsigned)b < (unsigned)nb;
            const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m[k] >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m[k], 0u));
            const uint32_t rank = (uint32_t)__shfl((int)old[k], rep[k]) + below;
            bv[k0 + k] = ok ? (int)((rank << 16) | (uint32_t)b) : 0xFFFF;
        }
    }

    // 3. tile-local first index of each bucket (exclusive scan of the counts);
    //    segment slot offsets (scan of the totals plus colpre) -> dlt.  Chunks
    //    of 64 consecutive buckets, lane l taking bucket 64 c + l, scanned
    //    across the lanes (DPP) with a running carry; nb <= 1024 here
    uint32_t nvalid_u;
    {
        const int32_t* tot = totals + seg * (long)nb;
        const int32_t* cp = colpre + (seg * ntiles + t) * (long)nb;
        constexpr int NCH = 1024 / 64;
        int tv[NCH], cv[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int b = min(64 * c + lane, nb - 1);
            tv[c] = 64 * c < nb ? tot[b] : 0;
            cv[c] = 64 * c < nb ? cp[b] : 0;
        }
        uint32_t carry_cnt = 0, carry_tot = 0, carry_nz = 0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if (64 * c < nb) {
                const int b = 64 * c + lane;
                const bool in = b < nb;
                const uint32_t cnt = in ? tab[2 * b] : 0u;
                const uint32_t tt = in ? (uint32_t)tv[c] : 0u;
                const uint32_t ic = wave_inclusive_scan_dpp(cnt);
                const uint32_t it = wave_inclusive_scan_dpp(tt);
                const uint32_t start = carry_cnt + ic - cnt;
                uint32_t lo = start;
                if constexpr (SAME) {
                    const uint32_t nz = tt > 0 ? 1u : 0u;
                    const uint32_t inz = wave_inclusive_scan_dpp(nz);
                    lo |= (2u * (carry_nz + inz - nz)) << 16;
                    carry_nz += (uint32_t)__builtin_amdgcn_readlane((int)inz, 63);
                }
                const uint32_t gfirst = carry_tot + it - tt + (uint32_t)cv[c];
                if (in) *reinterpret_cast<uint2*>(&tab[2 * b]) = make_uint2(lo, gfirst - start);
                carry_cnt += (uint32_t)__builtin_amdgcn_readlane((int)ic, 63);
                carry_tot += (uint32_t)__builtin_amdgcn_readlane((int)it, 63);
            }
        }
        nvalid_u = carry_cnt;
    }
    const int nvalid = (int)nvalid_u;

    // 4. each position to its sorted index (stg) and its cid value (bt).  The
    //    table entries of 8 steps are read before their stores: the compiler
    //    cannot tell that the stores (stg, bt) miss the table, so a read after
    //    a store would wait for it, one LDS round trip per step
    constexpr int PB = BPL < 8 ? BPL : 8;
#pragma unroll
    for (int k0 = 0; k0 < BPL; k0 += PB) {
        uint2 e[PB];
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            const int b = bv[k0 + j] & 0xFFFF;
            e[j] = *reinterpret_cast<const uint2*>(&tab[2 * (b < nb ? b : 0)]);
        }
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            const int k = k0 + j;
            const int p = 64 * k + lane;
            const int b = bv[k] & 0xFFFF;
            const bool ok = b < nb;
            const uint32_t li = (e[j].x & 0xFFFFu) + ((uint32_t)bv[k] >> 16);
            const uint32_t slot = li + e[j].y;
            uint32_t id = chunk_shift >= 0 ? slot >> chunk_shift : slot / (uint32_t)chunk;
            if constexpr (SAME) id += e[j].x >> 16;
            if (ok) stg[li] = ((uint32_t)b << 16) | (uint32_t)p;
            if (p < P) bt[p] = ok ? (uint16_t)id : (uint16_t)0xFFFF;
        }
    }

    // 5. perm in sorted order (each bucket's run of slots is contiguous)
    int32_t* pm = perm + seg * (long)L;
    for (int i0 = 0; i0 < nvalid; i0 += 64 * PLACE_BATCH) {
        uint32_t e[PLACE_BATCH], dl[PLACE_BATCH];
#pragma unroll
        for (int k = 0; k < PLACE_BATCH; ++k) e[k] = stg[min(i0 + 64 * k + lane, P - 1)];
#pragma unroll
        for (int k = 0; k < PLACE_BATCH; ++k) dl[k] = tab[2 * min((int)(e[k] >> 16), nb - 1) + 1];
#pragma unroll
        for (int k = 0; k < PLACE_BATCH; ++k) {
            const int i = i0 + 64 * k + lane;
            const uint32_t slot = (uint32_t)i + dl[k];
            // in range unless the input changed under the sort
            if (i < nvalid) LSH_CHECK(slot < (uint32_t)L);
            if (i < nvalid && slot < (uint32_t)L) pm[slot] = p0 + (int)(e[k] & 0xFFFFu);
        }
    }
    __syncthreads();
    // 6. the tile's cid rows for the group's rounds
    const uint16_t* bts[PLACE2_MAX_WAVES];
#pragma unroll
    for (int k = 0; k < PLACE2_MAX_WAVES; ++k)
        bts[k] = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(lds) + (long)k * ly.bytes + ly.bt);
    int16_t* cd = cid + (bh * (long)L + p0) * n_r;
    switch (RG) {
        case 1: store_cid_rows<1>(cd, bts, np, n_r, r0); break;
        case 2: store_cid_rows<2>(cd, bts, np, n_r, r0); break;
        case 4: store_cid_rows<4>(cd, bts, np, n_r, r0); break;
        case 8: store_cid_rows<8>(cd, bts, np, n_r, r0); break;
        default:
            for (int e = threadIdx.x; e < np * RG; e += blockDim.x) {
                const int p = e / RG, k = e - p * RG;
                cd[(long)p * n_r + r0 + k] = (int16_t)bts[k][p];
            }
    }
}

// Rounds per k_sort_place2 workgroup: the largest divisor of n_rounds (at most
// PLACE2_MAX_WAVES) whose waves' LDS fits in PLACE2_LDS_TARGET; 0 when the tile
// is longer than 64 * PLACE2_MAX_BPL positions or one round does not fit.
int place2_rounds_per_group(int nb, int P, int n_r)
{
    if (P > 64 * PLACE2_MAX_BPL) return 0;
    const size_t per = (size_t)place2_layout(nb, P).bytes;
    int best = 0;
    for (int rg = 1; rg <= n_r && rg <= PLACE2_MAX_WAVES; ++rg)
        if (n_r % rg == 0 && rg * per <= PLACE2_LDS_TARGET) best = rg;
    return best;
}

// Rounds per k_sort_place workgroup: the largest divisor of n_rounds (at most
// PLACE_MAX_WAVES) whose waves' LDS fits; 0 if not even one round fits, or if
// tile positions do not fit in 16 bits (then k_sort_scatter is used).
constexpr size_t PLACE_LDS_LIMIT = 160 * 1024;

int place_rounds_per_group(int nb, int P, int n_r, bool same)
{
    if (P > 65536) return 0;
    const size_t per = (size_t)place_layout(nb, P, same).words * 4;
    int best = 0;
    for (int rg = 1; rg <= n_r && rg <= PLACE_MAX_WAVES; ++rg)
        if (n_r % rg == 0 && rg * per <= PLACE_LDS_LIMIT) best = rg;
    return best;
}

}  // namespace

// The workspace of lsh_sort_noalloc: a static device array, one copy per GPU
// the library runs on, held until the process ends.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in for the
// symbol): sort_scratch() looks up its device address once per device.
static __device__ __align__(256) int32_t scratch[LSH_SORT_NOALLOC_MAX_BYTES / sizeof(int32_t)];

hipError_t sort_scratch(void** ptr)
{
    constexpr int MAX_DEVICES = 64;
    static std::mutex mu;
    static void* addr[MAX_DEVICES] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

SortPlan sort_plan(long bh, int L, int n_rounds, int n_buckets, bool same_bucket)
{
    // k_sort_place: tiles of at least 2 positions per bucket (and at least 2048),
    // so that every round of a workgroup fits in LDS; k_sort_scatter: at least 4
    // per bucket, so that the counters stay a fraction of the keys.  At most
    // 65536 positions and at most L.
    auto tile_for = [&](long per_bucket) {
        long tile = 2048;
        while (tile < per_bucket * n_buckets && tile < 65536) tile <<= 1;
        return tile > L ? (long)L : tile;
    };
    SortPlan p;
    long tile = tile_for(2);
    // Small problems: k_sort_place2 runs one workgroup per (b, h, group of
    // rounds, tile), and a wave walks its tile in steps of 64 positions; halve
    // the tile (down to 2 positions per bucket and 64 positions) while that
    // leaves fewer workgroups than CUs, so the placement spreads over the GPU
    // instead of walking long tiles on a few CUs.
    auto place2_wgs = [&](long t) -> long {
        const int rg2 = place2_rounds_per_group(n_buckets, (int)t, n_rounds);
        return rg2 > 0 ? bh * (n_rounds / rg2) * ((L + t - 1) / t) : 0;
    };
    while (place2_wgs(tile) > 0 && place2_wgs(tile) < 256 && tile / 2 >= std::max(64L, 2L * n_buckets))
        tile /= 2;
    p.rounds_per_group = place_rounds_per_group(n_buckets, (int)tile, n_rounds, same_bucket);
    if (p.rounds_per_group == 0) tile = tile_for(4);
    p.tile = (int)tile;
    p.ntiles = (int)((L + tile - 1) / tile);
    p.nseg = bh * n_rounds;
    p.counters = (size_t)p.nseg * p.ntiles * n_buckets;
    p.extra = (size_t)p.nseg * n_buckets;
    return p;
}

LSH_CHECK_ACCESSOR(check_count_sort)

hipError_t launch_sort(const int32_t* buckets, int32_t* perm, int16_t* cid, int32_t* counters,
                       int32_t* extra, bool same_bucket, const SortPlan& plan, long bh, int L,
                       int n_rounds, int n_buckets, int chunk, hipStream_t s)
{
    const size_t lds = (size_t)n_buckets * sizeof(int);
    // Up to 32768 buckets need 128 KiB of dynamic LDS per workgroup.
    static std::once_flag attr_once;
    std::call_once(attr_once, [] {
        (void)hipFuncSetAttribute((const void*)k_sort_hist,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 32768 * sizeof(int));
        (void)hipFuncSetAttribute((const void*)k_sort_scatter,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 32768 * sizeof(int));
        (void)hipFuncSetAttribute((const void*)k_sort_count,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)COUNT_LDS_LIMIT);
        (void)hipFuncSetAttribute((const void*)k_sort_place<false>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)PLACE_LDS_LIMIT);
        (void)hipFuncSetAttribute((const void*)k_sort_place<true>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)PLACE_LDS_LIMIT);
        auto p2 = [](const void* f) {
            (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)PLACE2_LDS_TARGET);
        };
        p2((const void*)k_sort_place2<false, 1>); p2((const void*)k_sort_place2<false, 2>);
        p2((const void*)k_sort_place2<false, 4>); p2((const void*)k_sort_place2<false, 8>);
        p2((const void*)k_sort_place2<false, 16>); p2((const void*)k_sort_place2<false, 32>);
        p2((const void*)k_sort_place2<true, 1>); p2((const void*)k_sort_place2<true, 2>);
        p2((const void*)k_sort_place2<true, 4>); p2((const void*)k_sort_place2<true, 8>);
        p2((const void*)k_sort_place2<true, 16>); p2((const void*)k_sort_place2<true, 32>);
    });
    int nbits = 0;
    while ((1 << nbits) < n_buckets) ++nbits;
    const unsigned blocks = (unsigned)(plan.nseg * plan.ntiles);
    const int rg = plan.rounds_per_group;
    // the placement kernels take column prefixes and totals: from k_sort_count
    // where the tile histograms fit in LDS (tile a power of two, or one tile)
    const int nsplit = count_splits(plan.nseg, n_buckets, L);
    const size_t count_lds = (size_t)plan.ntiles * (n_buckets / nsplit) * sizeof(uint16_t);
    const bool pow2_tile = (plan.tile & (plan.tile - 1)) == 0;
    if (rg > 0 && plan.tile <= 32768 && count_lds <= COUNT_LDS_LIMIT && (pow2_tile || plan.ntiles == 1)) {
        const int tile_shift = plan.ntiles == 1 ? 30 : __builtin_ctz((unsigned)plan.tile);
        const long rows = (plan.nseg + NXCD - 1) / NXCD;
        hipLaunchKernelGGL(k_sort_count, dim3((unsigned)(rows * NXCD * nsplit)), dim3(COUNT_THREADS), count_lds,
                           s, buckets, counters, extra, plan.nseg, L, n_buckets, tile_shift, plan.ntiles, nsplit);
    } else {
        hipLaunchKernelGGL(k_sort_hist, dim3(blocks), dim3(SORT_THREADS), lds, s, buckets, counters, L,
                           n_buckets, plan.tile, plan.ntiles);
        if (rg > 0) {
            const int bps = (n_buckets + COLSCAN_THREADS - 1) / COLSCAN_THREADS;
            hipLaunchKernelGGL(k_sort_colscan, dim3((unsigned)(plan.nseg * bps)), dim3(COLSCAN_THREADS), 0, s,
                               counters, extra, n_buckets, plan.ntiles, bps);
        }
    }
    if (rg > 0) {
        const int shift = (chunk & (chunk - 1)) == 0 ? __builtin_ctz((unsigned)chunk) : -1;
        const int rg2 = place2_rounds_per_group(n_buckets, plan.tile, n_rounds);
        if (rg2 > 0) {
            const int ngroups = n_rounds / rg2;
            const long nkeys = bh * ngroups;
            const long rows = (nkeys + NXCD - 1) / NXCD;
            const unsigned pblocks = (unsigned)(rows * NXCD * plan.ntiles);
            const size_t plds = (size_t)rg2 * place2_layout(n_buckets, plan.tile).bytes;
            int bpl = 1;
            while (64 * bpl < plan.tile) bpl <<= 1;
            auto go = [&](auto same, auto bplc) {
                constexpr bool SM = decltype(same)::value;
                constexpr int BP = decltype(bplc)::value;
                hipLaunchKernelGGL((k_sort_place2<SM, BP>), dim3(pblocks), dim3(64 * rg2), plds, s, buckets,
                                   counters, extra, perm, cid, L, n_buckets, nbits, plan.tile,
                                   plan.ntiles, n_rounds, rg2, ngroups, nkeys, chunk, shift);
            };
            auto by_bpl = [&](auto same) {
                switch (bpl) {
                    case 1: go(same, std::integral_constant<int, 1>{}); break;
                    case 2: go(same, std::integral_constant<int, 2>{}); break;
                    case 4: go(same, std::integral_constant<int, 4>{}); break;
                    case 8: go(same, std::integral_constant<int, 8>{}); break;
                    case 16: go(same, std::integral_constant<int, 16>{}); break;
                    default: go(same, std::integral_constant<int, 32>{}); break;
                }
            };
            if (same_bucket) by_bpl(std::true_type{});
            else by_bpl(std::false_type{});
            return hipGetLastError();
        }
        const int ngroups = n_rounds / rg;
        const long nkeys = bh * ngroups;
        const long rows = (nkeys + NXCD - 1) / NXCD;
        const unsigned pblocks = (unsigned)(rows * NXCD * plan.ntiles);
        const size_t plds = (size_t)rg * place_layout(n_buckets, plan.tile, same_bucket).words * 4;
        if (same_bucket)
            hipLaunchKernelGGL(k_sort_place<true>, dim3(pblocks), dim3(64 * rg), plds, s, buckets,
                               counters, extra, perm, cid, L, n_buckets, nbits, plan.tile,
                               plan.ntiles, n_rounds, rg, ngroups, nkeys, chunk, shift);
        else
            hipLaunchKernelGGL(k_sort_place<false>, dim3(pblocks), dim3(64 * rg), plds, s, buckets,
                               counters, extra, perm, cid, L, n_buckets, nbits, plan.tile,
                               plan.ntiles, n_rounds, rg, ngroups, nkeys, chunk, shift);
        return hipGetLastError();
    }
    int32_t* ranks = same_bucket ? extra : nullptr;
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
