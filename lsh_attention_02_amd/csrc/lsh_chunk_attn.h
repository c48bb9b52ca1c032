// Chunked LSH attention on gfx950, one output per hash round (kernel template;
// instantiated by the lsh_chunk_attn_*.hip files).
//
// For round r of (batch row, head) the positions are in sorted order perm; the
// sorted sequence is cut into chunks of C; the queries of chunk k attend to the
// keys of chunks k-1 and k (ai-scholar Reformer article and Ultralytics
// "Reformer" glossary, sections on LSH attention).  Scores follow the scaled
// dot-product form of the ai-scholar article; the query itself is penalised
// and later positions are dropped when causal (modulabs-hub notes, "LSH
// attention"); the duplicate-count term -log N_ij (N_ij = rounds whose window
// for i holds j) makes the round combine equal to attention over the union of
// the rounds' windows.
//
// Workgroup = C/16 waves; it walks a run of consecutive chunks of one
// (b, h, r).  Each chunk's qk rows (row-major) and v rows (transposed) are
// gathered once into LDS and kept for the next chunk, whose look-back window
// they form.  The rows of chunk k+1 (and k+2 where a second register set
// fits) are loaded into registers while chunk k is computed, so the gathers
// overlap the math.
// Wave w takes the 16 queries in rows 16w.. of the chunk (16x16 MFMA tiles,
// so that four waves share one chunk's LDS tiles and each SIMD holds two waves):
//   S^T[key, q] = K[key, :] · Q[q, :]     (A = key rows, B = query rows)
// so each lane holds one query's scores as registers (keys 4(l/16)+j of each
// 16-key tile), the softmax is in-register plus two cross-lane exchanges, and
// the probabilities feed the PV product directly as the B operand:
//   O^T[d, q] = V^T[d, key] · P^T[key, q]
// with V^T read from LDS in the same key order.  Rows of o_rounds and lse go
// back to original position order.  Scores are kept in base 2 (exp2/log2);
// -log2 N comes from a small LDS table addressed by 8 x (rounds outside).
//
// Duplicate counts: chunk ids of all rounds are packed two per 32-bit word
// (NDW words per token, padded with equal values on both sides, which always
// compare as inside).  For key chunk k and query chunk q of a round, the key is
// inside the query's window when u = k - (q - 1) (mod 2^16) is 0 or 1; per word
// that is one packed subtract and one saturating packed add (bit 15 = outside);
// one byte permute per two words gathers the flags and v_bcnt counts them.
#pragma once

#include <atomic>
#include <type_traits>

#include "lsh_device.h"
#include "lsh_internal.h"

namespace lshk {
namespace attn {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float SELF_PENALTY = 1.0e5f;               // score units
// Chunks per workgroup: a run of consecutive chunks shares each look-back
// load.  Runs are RUN chunks long unless the problem is small: then shorter
// runs spread it over about RUN_TARGET_WGS workgroups (a run of one chunk
// loads its look-back itself), so a few segments do not serialise on a few CUs.
constexpr int RUN = 16;
constexpr long RUN_TARGET_WGS = 1024;

inline int run_length(int nchunks, long segments)
{
    const long len = ((long)nchunks * segments + RUN_TARGET_WGS - 1) / RUN_TARGET_WGS;
    return (int)(len < 1 ? 1 : len > RUN ? RUN : len);
}

// The forward's run length: a workgroup's time grows with its run (one step
// per chunk, plus its look-back), and the launch takes as many rounds of
// workgroups as it has workgroups per `slots` (the workgroups the GPU holds at
// once); take the run of 1 .. RUN_MAX chunks with the fewest rounds x steps
// (the shorter on a tie).  A round only partly filled costs almost a whole
// one: clustered_16k's 1024 workgroups of 16 chunks on 768 slots took two,
// 768 of 22 one, 11% faster.
constexpr int RUN_MAX = 32;

inline int run_length_fit(int nchunks, long segments, long slots)
{
    int best = 1;
    long best_cost = -1;
    for (int len = 1; len <= RUN_MAX; ++len) {
        const long wgs = segments * ((nchunks + len - 1) / len);
        const long cost = ((wgs + slots - 1) / slots) * (len + 1);
        if (best_cost < 0 || cost < best_cost) { best = len; best_cost = cost; }
        if (len >= nchunks) break;
    }
    return best;
}

// Compute units of the current device (queried once per device).
inline int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

__device__ __forceinline__ uint32_t pk_sub_u16(uint32_t a, uint32_t b)
{
    uint32_t d;
    asm("v_pk_sub_u16 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
    return d;
}

// For each 16-bit half: u = k - q1 (mod 2^16), then sat(u + 0x7FFE).  Bit 15 of
// the result is set exactly when u >= 2, i.e. when the key lies outside the
// query's window in that round (u is 0 or 1 inside).
__device__ __forceinline__ uint32_t pk_outside_flags(uint32_t k, uint32_t q1)
{
    uint32_t u, t;
    asm("v_pk_sub_u16 %0, %2, %3\n\tv_pk_add_u16 %1, %0, %4 clamp"
        : "=&v"(u), "=v"(t)
        : "v"(k), "v"(q1), "v"(0x7FFE7FFEu));
    return t;
}

// Look-back around the end of the round: the key is also inside when
// u == nchunks (query in chunk 0, key in the last chunk; no other pair of
// chunk ids gives that difference).  With e = u ^ nchunks per half,
// sat(e + 0x7FFF) has bit 15 set unless e == 0, so AND-ing it into the flags
// clears "outside" for that case.  nch2 holds nchunks in both halves.
__device__ __forceinline__ uint32_t pk_outside_flags_wrap(uint32_t k, uint32_t q1, uint32_t nch2)
{
    uint32_t u, t, e, f;
    asm("v_pk_sub_u16 %0, %4, %5\n\t"
        "v_pk_add_u16 %1, %0, %6 clamp\n\t"
        "v_xor_b32 %2, %0, %7\n\t"
        "v_pk_add_u16 %3, %2, %8 clamp"
        : "=&v"(u), "=&v"(t), "=&v"(e), "=v"(f)
        : "v"(k), "v"(q1), "v"(0x7FFE7FFEu), "v"(nch2), "v"(0x7FFF7FFFu));
    return t & f;
}

template <bool WRAP>
__device__ __forceinline__ uint32_t outside_flags(uint32_t k, uint32_t q1, uint32_t nch2)
{
    if constexpr (WRAP) return pk_outside_flags_wrap(k, q1, nch2);
    else return pk_outside_flags(k, q1);
}

// 8 x (number of rounds in which the key is outside the query's window).
// v_perm_b32 selectors 8..11 replicate bit 15 / bit 31 of each source word into
// a byte, so one perm gathers the flags of two words (four rounds) as 0x00/0xFF
// bytes, which v_bcnt counts.
template <int NDW, bool WRAP>
__device__ __forceinline__ uint32_t rounds_outside8(const uint32_t (&q1)[NDW], const uint32_t* kc,
                                                    uint32_t nch2)
{
    uint32_t w[NDW];
    if constexpr (NDW == 1) {
        w[0] = kc[0];
    } else if constexpr (NDW == 2) {
        const uint2 x = *reinterpret_cast<const uint2*>(kc);
        w[0] = x.x; w[1] = x.y;
    } else {
#pragma unroll
        for (int h = 0; h < NDW / 4; ++h) {
            const uint4 x = *reinterpret_cast<const uint4*>(kc + 4 * h);
            w[4 * h] = x.x; w[4 * h + 1] = x.y; w[4 * h + 2] = x.z; w[4 * h + 3] = x.w;
        }
    }
    if constexpr (NDW == 1) {
        return __builtin_popcount(
            __builtin_amdgcn_perm(0u, outside_flags<WRAP>(w[0], q1[0], nch2), 0x0C0C0908u));
    } else {
        uint32_t acc = 0;
#pragma unroll
        for (int i = 0; i < NDW; i += 2)
            acc += __builtin_popcount(
                __builtin_amdgcn_perm(outside_flags<WRAP>(w[i + 1], q1[i + 1], nch2),
                                      outside_flags<WRAP>(w[i], q1[i], nch2), 0x0B0A0908u));
        return acc;
    }
}

// V^T rows hold a slot's keys in groups of 4 consecutive keys.
// 32-bit elements: group kg of row d is the 16 bytes at kg ^ vt_swz(d).
// 16-bit elements: groups kg and kg + 4 (kg with bit 2 clear) form one 16-byte
// pair: the two groups that one PV operand combines (keys 4g.. of tiles t0 and
// t0 + 1), so the operand is a single 16-byte read.  Pair p of row d sits at
// p ^ vt_pair_swz(d) = p ^ f(d % 16) ^ 5 (d / 16), f(r) = r (r / 2 at chunk 32;
// no d / 16 term at chunk 128 with d 128, where its per-dt addresses made the
// compiler spill).
// A 16-byte read is served in passes of 16 lanes (the lane quads of even, then
// odd, bit parity in each half-wave); each pass of the operand reads of rows
// 16 dt + r16 covers the 64 banks once (checked exhaustively, and measured:
// no conflict cycles).  The transposed 8-byte stores (lanes of odd pieces store
// their rows' elements in the order x ^ 1) measured 4 conflict cycles per store
// instruction, 8 instructions per chunk: negligible next to the reads.
template <int C>
__device__ __forceinline__ int vt_swz(int d)
{
    return (d ^ (d >> 3)) & (C / 4 - 1);
}

template <int C, int D>
__device__ __forceinline__ int vt_pair_swz(int d)
{
    const int r16 = d & 15;
    constexpr bool MIX = !(C == 128 && D == 128);
    return ((C == 32 ? r16 >> 1 : r16) ^ (MIX ? 5 * (d >> 4) : 0)) & (C / 8 - 1);
}

// byte offset of 4-key group kg within a 16-bit V^T row d
template <int C, int D>
__device__ __forceinline__ int vt_group_off(int kg, int d)
{
    const int pair = (kg & 3) | ((kg >> 3) << 2);
    return 16 * (pair ^ vt_pair_swz<C, D>(d)) + 8 * ((kg >> 2) & 1);
}

// qk rows in LDS.  A 16-byte LDS access is served in four passes of 16 lanes;
// in each half-wave, lane quads (lane / 4) of even and of odd bit parity form the
// two passes.  The layouts below keep both the row stores (lane = piece of 4-row
// groups) and the MFMA operand reads (lane = row r16 + 16 * piece group) free of
// bank conflicts under that grouping:
//   bf16, d 128: unpadded 256-byte rows, 16-byte piece p of row r stored at
//                p ^ (r ^ ((r & 4) << 1)) mod 16;
//   bf16, d 64:  rows padded to 160 bytes, no swizzle;
//   f32:         rows padded by 16 bytes (4-byte operand reads).
template <typename T, int D>
struct KLayout {
    static constexpr bool SWZ = sizeof(T) == 2 && D == 128;
    static constexpr int ROW = sizeof(T) == 4 ? D + 4 : (D == 128 ? D : D + 16);
    // element e (a multiple of the 16-byte piece or of the operand width) of row r
    static __device__ __forceinline__ int off(int r, int e) {
        if constexpr (SWZ) return r * ROW + 8 * ((e >> 3) ^ ((r ^ ((r & 4) << 1)) & 15)) + (e & 7);
        else return r * ROW + e;
    }
};

// Register sets for the gathered rows: with two, the rows of the next two
// chunks are in flight while one is computed (measured 1-2% faster at d 128,
// chunk 64).  Elsewhere the second set would cost a wave per SIMD.
template <typename T, int D, int C, int NDW, bool SAME>
constexpr int gather_sets()
{
    return sizeof(T) == 2 && D == 128 && C == 64 && NDW <= 4 && !SAME ? 2 : 1;
}

template <typename T, int D, int C, int NDW>
struct Lds {
    static constexpr int KROW = KLayout<T, D>::ROW;        // qk row (elements)
    static constexpr int VROWB = C * (int)sizeof(T);        // v^T row bytes (one slot's keys)
    // -log2(n_rounds - o) at byte offset 8*o, o = rounds outside (at most 16):
    // the popcount sum 8*o addresses it directly (first member: offset 0)
    float neg_log2[36];
    T k[2][C * KROW];
    char vt[2][D * VROWB];
    int pos[2][C];
    uint32_t cid[2][C * (NDW > 0 ? NDW : 1)];
    int rid[2][C];                 // same-bucket variant: this round's window id of each row
};

// NDW = 0: no duplicate-count term (LSH_FLAG_NO_DUP_CORRECTION).  WRAP: chunk 0
// looks back to the last chunk of its round (LSH_FLAG_WRAP_LOOKBACK).  SAME:
// keys outside the query's bucket of this round are dropped
// (LSH_FLAG_SAME_BUCKET; cid then holds window ids, and the test that puts a
// key in a query's window in a round also checks the bucket).
template <typename T, int D, int C, int NDW, bool WRAP, bool SAME>
__global__ __launch_bounds__(4 * C)
void k_chunk_attn(const T* __restrict__ qk, const T* __restrict__ v,
                  const int32_t* __restrict__ perm, const int16_t* __restrict__ cid,
                  T* __restrict__ o_rounds, float* __restrict__ lse, int L, int n_r, int causal,
                  float scale_log2, int nruns, int run_len)
{
    using M = Mfma16<T>;
    using S = Lds<T, D, C, NDW>;
    using KL = KLayout<T, D>;
    constexpr int NTH = 4 * C;                         // C/16 waves of 16 queries
    constexpr int KPL = M::KPL, KSTEP = M::KSTEP, NKS = D / KSTEP;
    constexpr int VROWB = S::VROWB;
    constexpr int CT = C / 16, NKT = 2 * CT, DT = D / 16;
    static_assert(sizeof(T) != 2 || DT % 2 == 0, "bf16 rows are stored as pairs of d tiles");
    constexpr int VE = 16 / (int)sizeof(T), VPR = D / VE;
    // score tiles per scheduling region: two accumulation chains at a time where
    // the registers allow it
    constexpr int SGRP = sizeof(T) == 2 && C <= 64 ? 2 : 1;
    // gather jobs: 4 consecutive rows x one 16-byte piece (of qk and of v)
    constexpr int JOBS = (C / 4) * VPR;
    constexpr int JPT = (JOBS + NTH - 1) / NTH;        // jobs per thread
    __shared__ __attribute__((aligned(16))) S sm;
    static_assert(offsetof(S, vt) % 16 == 0, "16-byte V^T reads");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;          // MFMA 16x16 lane coordinates

    int bid = blockIdx.x;
    const int r = bid % n_r;
    bid /= n_r;
    const int run = bid % nruns;
    // (batch row, head) pairs in descending order: the hash reads them in
    // ascending order and the combine that follows does too, so the first
    // heads walked here are the ones whose qk the hash read last, and the last
    // ones written here are the combine's first reads; both still sit in the
    // Infinity Cache at small enough sizes
    const long bh = (long)(gridDim.x / ((unsigned)nruns * (unsigned)n_r)) - 1 - bid / nruns;
    const int nchunks = L / C;
    const int k0 = run * run_len, k1 = min(k0 + run_len, nchunks);

    const T* qb = qk + bh * (long)L * D;
    const T* vb = v + bh * (long)L * D;
    const int32_t* pr = perm + (bh * n_r + r) * (long)L;
    const int16_t* cb = cid + bh * (long)L * n_r;
    T* ob = o_rounds + (bh * n_r + r) * (long)L * D;
    float* lb = lse + (bh * n_r + r) * (long)L;
    const uint32_t ones = 0x00010001u;
    const uint32_t nch2 = (uint32_t)nchunks * 0x00010001u;
    constexpr int NW = NDW > 0 ? NDW : 1;              // array extent when NDW = 0

    if (tid < 33) sm.neg_log2[tid] = (tid % 2 == 0 && tid / 2 < n_r) ? -__log2f((float)(n_r - tid / 2)) : 0.f;

    // Loaded values are kept raw until the iteration that stores them
    // (positions are clamped, chunk ids masked and packed there): processing a
    // value right after its load would make the wave wait for every earlier
    // load as well, the gathers meant to overlap the math included.  Every
    // iteration issues the same loads (past the run's end they repeat its last
    // chunk and are never stored), so the compiler's wait counts are the same
    // in every iteration.
    // Positions come from the caller's perm: every gather stays inside the row.
    auto clamp_pos = [&](int p) {
        LSH_CHECK((unsigned)p < (unsigned)L);
        return min(max(p, 0), L - 1);
    };

    // Per-row jobs: job m < C * NW loads word m % NW (rounds 2w and 2w+1) of
    // the packed chunk ids of row m / NW and, for m % NW == 0, the row's
    // position (and its window id in the same-bucket variant).
    constexpr int MJOBS = C * NW;
    constexpr int MJPT = (MJOBS + NTH - 1) / NTH;
    constexpr int NSET = gather_sets<T, D, C, NDW, SAME>();
    int gpos[NSET][JPT][4];    // raw perm entries of this thread's gather rows, per register set
    int mpos[NSET][MJPT];      // raw perm entries of this thread's per-row jobs
    u32x4 kreg[NSET][JPT][4], vreg[NSET][JPT][4];
    int rpos[NSET][MJPT];      // clamped positions of the per-row jobs' rows
    uint32_t clo[NSET][MJPT], chi[NSET][MJPT];   // raw chunk ids of rounds 2w and 2w+1
    uint32_t ridraw[NSET][MJPT];   // same-bucket variant: the row's window id in this round

    auto fetch_positions = [&](int kk, auto set) __attribute__((always_inline)) {
        constexpr int P = decltype(set)::value;
#pragma unroll
        for (int jb = 0; jb < JPT; ++jb) {
            const int job = tid + jb * NTH;
            const int rg = (job < JOBS ? job : 0) / VPR;
            const int4 p4 = *reinterpret_cast<const int4*>(pr + kk * C + 4 * rg);
            gpos[P][jb][0] = p4.x; gpos[P][jb][1] = p4.y; gpos[P][jb][2] = p4.z; gpos[P][jb][3] = p4.w;
        }
#pragma unroll
        for (int mj = 0; mj < MJPT; ++mj) {
            const int m = (tid + mj * NTH) % MJOBS;     // jobs past the end repeat (no branches)
            mpos[P][mj] = pr[kk * C + m / NW];
        }
    };
    auto fetch_rows = [&](auto set) __attribute__((always_inline)) {
        constexpr int P = decltype(set)::value;
#pragma unroll
        for (int jb = 0; jb < JPT; ++jb) {
            const int job = tid + jb * NTH;
            const int piece = (job < JOBS ? job : 0) % VPR;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const long row = (long)clamp_pos(gpos[P][jb][i]) * D + piece * VE;
                kreg[P][jb][i] = *reinterpret_cast<const u32x4*>(qb + row);
                vreg[P][jb][i] = *reinterpret_cast<const u32x4*>(vb + row);
            }
        }
#pragma unroll
        for (int mj = 0; mj < MJPT; ++mj) {
            const int m = (tid + mj * NTH) % MJOBS;
            rpos[P][mj] = clamp_pos(mpos[P][mj]);
            const int16_t* cr = cb + (long)rpos[P][mj] * n_r;
            if constexpr (NDW > 0) {
                const int w = m % NW;
                clo[P][mj] = (uint16_t)cr[min(2 * w, n_r - 1)];
                chi[P][mj] = (uint16_t)cr[min(2 * w + 1, n_r - 1)];
            }
            if constexpr (SAME) ridraw[P][mj] = (uint16_t)cr[r];
        }
    };
    auto store_rows = [&](int sl, auto set) __attribute__((always_inline)) {
        constexpr int P = decltype(set)::value;
#pragma unroll
        for (int jb = 0; jb < JPT; ++jb) {
            const int job = tid + jb * NTH;
            if (job < JOBS) {
                const int rg = job / VPR, piece = job % VPR;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<u32x4*>(&sm.k[sl][KL::off(4 * rg + i, piece * VE)]) = kreg[P][jb][i];
                // transpose the 4 rows x VE elements: element x of every row gives
                // the 4 keys 4rg..4rg+3 of v^T row d = piece*VE + x
#pragma unroll
                for (int x = 0; x < VE; ++x) {
                    if constexpr (sizeof(T) == 2) {
                        const int xe = x ^ (piece & 1);        // element order x ^ 1 on odd pieces
                        const int d = piece * VE + xe;
                        char* dst = sm.vt[sl] + d * VROWB + vt_group_off<C, D>(rg, d);
                        const uint32_t sel = 0x05040100u + 0x02020202u * (uint32_t)(xe & 1);
                        const uint32_t w0 = __builtin_amdgcn_perm(vreg[P][jb][1][x >> 1], vreg[P][jb][0][x >> 1], sel);
                        const uint32_t w1 = __builtin_amdgcn_perm(vreg[P][jb][3][x >> 1], vreg[P][jb][2][x >> 1], sel);
                        *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
                    } else {
                        const int d = piece * VE + x;
                        char* dst = sm.vt[sl] + d * VROWB + 16 * (rg ^ vt_swz<C>(d));
                        const u32x4 w4 = {vreg[P][jb][0][x], vreg[P][jb][1][x], vreg[P][jb][2][x], vreg[P][jb][3][x]};
                        *reinterpret_cast<u32x4*>(dst) = w4;
                    }
                }
            }
        }
#pragma unroll
        for (int mj = 0; mj < MJPT; ++mj) {
            const int m = tid + mj * NTH;
            if (m < MJOBS) {
                const int row = m / NW, w = m % NW;
                if (w == 0) {
                    sm.pos[sl][row] = rpos[P][mj];
                    if constexpr (SAME) sm.rid[sl][row] = (int)ridraw[P][mj];
                }
                // rounds past n_r hold 0 for keys and queries alike (always inside)
                if constexpr (NDW > 0) {
                    const uint32_t lo = 2 * w < n_r ? clo[P][mj] : 0u;
                    const uint32_t hi = 2 * w + 1 < n_r ? chi[P][mj] : 0u;
                    sm.cid[sl][row * NDW + w] = lo | (hi << 16);
                }
            }
        }
    };

    // Iteration it handles chunk chunk_of(it).  When chunk k0 has a look-back
    // chunk (k0 - 1, or the last chunk when wrapping around), iteration 0 only
    // loads it; the chunks k0 .. k1-1 follow.
    const bool lookback = k0 > 0 || (WRAP && nchunks > 1);
    const int it0 = lookback ? 1 : 0;
    const int nit = (k1 - k0) + it0;
    auto chunk_of = [&](int it) {
        const int c = k0 - it0 + min(it, nit - 1);     // past the end: the last chunk again
        return c < 0 ? c + nchunks : c;
    };

    // Chunk it in slot cur = it % 2 (its look-back in the other slot) against
    // the 16 queries of this wave.
    auto compute = [&](int it, int cur, int prv) __attribute__((always_inline)) {
            const bool has_prev = it > 0;
            const int qrow = wave * 16 + r16;
            const int qpos = sm.pos[cur][qrow];

            typename M::Frag bq[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                bq[ks] = M::load(&sm.k[cur][KL::off(qrow, ks * KSTEP + g * KPL)]);
            uint32_t q1[NW];           // query chunk ids minus one, per half
#pragma unroll
            for (int w = 0; w < NDW; ++w) q1[w] = pk_sub_u16(sm.cid[cur][qrow * NDW + w], ones);
            const int rq1 = SAME ? sm.rid[cur][qrow] - 1 : 0;   // query's window id minus one

            // ---- S^T tiles of 16 keys: [0, CT) previous chunk, [CT, 2CT) this one.
            //      Lane (r16, g) holds query r16 against keys 4g + j of each tile.
            f32x4 s[NKT];
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                if (t < CT && !has_prev) { s[t] = f32x4{}; continue; }
                const int slk = t < CT ? prv : cur;
                const int krow = (t % CT) * 16 + r16;
                s[t] = M::mma(M::load(&sm.k[slk][KL::off(krow, g * KPL)]), bq[0], f32x4{});
#pragma unroll
                for (int ks = 1; ks < NKS; ++ks)
                    s[t] = M::mma(M::load(&sm.k[slk][KL::off(krow, ks * KSTEP + g * KPL)]), bq[ks], s[t]);
                if (t % SGRP == SGRP - 1) __builtin_amdgcn_sched_barrier(0);
            }

            // ---- scale and duplicate counts; causal cut; at chunk 128 also the
            //      self penalty and the running max (the separate passes below
            //      make the compiler spill there)
            constexpr bool SELF_BRANCH = C <= 64;
            float mx = -INFINITY;
            // chunk 128, bf16 at d 64 with up to 8 rounds and no bucket test:
            // the penalty of key 4g + j in the diagonal tile (the query itself
            // when 4g + j == r16), added by one fma per current-chunk pair with
            // a factor that is uniform over the wave (1 on the diagonal tile).
            // The other chunk-128 kernels have no registers to spare for it
            // and keep the compare and select.
            constexpr bool SELF_FMA = C == 128 && D == 64 && sizeof(T) == 2 && !SAME && NDW <= 4;
            float pen[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) pen[j] = 4 * g + j == r16 ? -SELF_PENALTY * LOG2E : 0.f;
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                if (t < CT && !has_prev) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) s[t][j] = -INFINITY;
                    continue;
                }
                const int slk = t < CT ? prv : cur;
                const bool diag = t == CT + wave;   // the tile holding the queries themselves
                const int krow0 = (t % CT) * 16 + 4 * g;
                const int4 kp = *reinterpret_cast<const int4*>(&sm.pos[slk][krow0]);
                int4 kr = {0, 0, 0, 0};
                if constexpr (SAME) kr = *reinterpret_cast<const int4*>(&sm.rid[slk][krow0]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int kpos = j == 0 ? kp.x : j == 1 ? kp.y : j == 2 ? kp.z : kp.w;
                    float nlg = 0.f;
                    if constexpr (NDW > 0) {
                        const uint32_t outs8 = rounds_outside8<NDW, WRAP>(
                            q1, &sm.cid[slk][(krow0 + j) * NDW], nch2);
                        nlg = *reinterpret_cast<const float*>(
                            reinterpret_cast<const char*>(sm.neg_log2) + outs8);
                    }
                    float sc = fmaf(s[t][j], scale_log2, nlg);
                    if (SELF_FMA && t >= CT) sc = fmaf(diag ? 1.f : 0.f, pen[j], sc);
                    if (!SELF_BRANCH && !SELF_FMA && diag && kpos == qpos) sc -= SELF_PENALTY * LOG2E;
                    if (causal && kpos > qpos) sc = -INFINITY;
                    if constexpr (SAME) {
                        // another bucket: window ids differ by something other than 0 or 1
                        const int kid = j == 0 ? kr.x : j == 1 ? kr.y : j == 2 ? kr.z : kr.w;
                        if ((unsigned)(kid - rq1) > 1u) sc = -INFINITY;
                    }
                    s[t][j] = sc;
                    if (!SELF_BRANCH) mx = fmaxf(mx, sc);
                }
                if (t % SGRP == SGRP - 1) __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (SELF_BRANCH) {
                // ---- self penalty.  The query's own key is in the current
                //      chunk's tile CT + wave (the tile of this wave's query rows),
                //      as key 4g + j == r16: a round's chunks hold distinct
                //      positions, so that is the one key with kpos == qpos.  The
                //      branch is uniform (the empty asm keeps it a branch instead
                //      of selects on every tile).
#pragma unroll
                for (int w = 0; w < CT; ++w) {
                    if (w == wave) {
                        asm volatile("");
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (4 * g + j == r16) s[CT + w][j] -= SELF_PENALTY * LOG2E;
                    }
                }
                // ---- running max
#pragma unroll
                for (int t = 0; t < NKT; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j) mx = fmaxf(mx, s[t][j]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));

            float sum = 0.f;
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float p = __builtin_amdgcn_exp2f(s[t][j] - mx);
                    s[t][j] = p;
                    sum += p;
                }
            }
            sum += __shfl_xor(sum, 16);
            sum += __shfl_xor(sum, 32);

            // ---- O^T = V^T · P^T.  Lane (r16, g): row d = 16*dt + r16 of V^T;
            //      P^T column = query r16, keys 4g + j of the tile(s).
            f32x4 o[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{};
            if constexpr (KPL == 8) {
                // one instruction covers two 16-key tiles: slot i < 4 is key 4g+i of
                // tile t0, slot i >= 4 is key 4g+i-4 of tile t0+1
#pragma unroll
                for (int t0 = 0; t0 < NKT; t0 += 2) {
                    if (t0 < CT && !has_prev) continue;
                    const int slk = t0 < CT ? prv : cur;
                    const int key0 = (t0 % CT) * 16 + 4 * g;
                    bf16x8 b;
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        b[x] = (__bf16)s[t0][x];
                        b[4 + x] = (__bf16)s[t0 + 1][x];
                    }
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const int d = dt * 16 + r16;
                        // groups kg (tile t0) and kg + 4 (tile t0 + 1): one pair
                        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                            sm.vt[slk] + d * VROWB + vt_group_off<C, D>(key0 >> 2, d));
                        o[dt] = M::mma(a, b, o[dt]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                // one instruction per key column j: lane group g holds key 4g+j
#pragma unroll
                for (int t = 0; t < NKT; ++t) {
                    if (t < CT && !has_prev) continue;
                    const int slk = t < CT ? prv : cur;
                    const int key0 = (t % CT) * 16 + 4 * g;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
#pragma unroll
                        for (int dt = 0; dt < DT; ++dt) {
                            const int d = dt * 16 + r16;
                            const float a = *reinterpret_cast<const float*>(
                                sm.vt[slk] + d * VROWB + 16 * ((key0 >> 2) ^ vt_swz<C>(d)) + 4 * j);
                            o[dt] = M::mma(a, s[t][j], o[dt]);
                        }
                    }
                }
            }

            // ---- normalise, store the query's row and its lse.  Lane (r16, g)
            //      holds d = 16*dt + 4g + j of query r16.
            const float inv = 1.f / sum;
            T* orow = ob + (long)qpos * D;
            if constexpr (sizeof(T) == 2) {
                // pairs of d tiles as 16-byte pieces (store_tile_pair_bf16: half
                // the store instructions, 5.7% faster at d 128, chunk 64)
#pragma unroll
                for (int e = 0; e < DT / 2; ++e) {
                    const int dt0 = 2 * e, dt1 = 2 * e + 1;
                    store_tile_pair_bf16(reinterpret_cast<bf16_t*>(orow), g, dt0,
                                         pack_bf16x2(o[dt0][0] * inv, o[dt0][1] * inv),
                                         pack_bf16x2(o[dt0][2] * inv, o[dt0][3] * inv),
                                         pack_bf16x2(o[dt1][0] * inv, o[dt1][1] * inv),
                                         pack_bf16x2(o[dt1][2] * inv, o[dt1][3] * inv));
                }
            } else {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const f32x4 w = {o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv};
                    *reinterpret_cast<f32x4*>(orow + dt * 16 + 4 * g) = w;
                }
            }
            if (g == 0) lb[qpos] = (mx + __log2f(sum)) * LN2;
    };

    // One iteration: store chunk it into slot it % 2 (a compile-time slot: the
    // loop is unrolled by two), load the rows of chunk it+1 and the positions
    // of chunk it+2, compute chunk it.  The scheduling barriers in compute keep
    // the compiler from hoisting a whole phase's LDS reads at once, which would
    // raise the registers past two waves per SIMD.
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, NSET - 1>;
    auto step = [&](int it, auto slot) __attribute__((always_inline)) {
        constexpr int SL = decltype(slot)::value;
        using PS = std::integral_constant<int, NSET == 2 ? SL : 0>;
        using QS = std::integral_constant<int, NSET == 2 ? 1 - SL : 0>;
        store_rows(SL, PS{});          // slot of iteration it-2, released by the last barrier
        __syncthreads();
        if constexpr (NSET == 2) {
            // positions of chunk it+3 before the rows of chunk it+2, so that
            // waiting for them never waits for those rows
            fetch_positions(chunk_of(it + 3), QS{});
            fetch_rows(PS{});
        } else {
            fetch_rows(PS{});          // chunk it+1 (positions fetched an iteration ago)
            fetch_positions(chunk_of(it + 2), PS{});
        }
        if (it >= it0) compute(it, SL, 1 - SL);
        __syncthreads();
    };
    if constexpr (NSET == 2) {
        fetch_positions(chunk_of(0), S0{});
        fetch_positions(chunk_of(1), S1{});
        fetch_rows(S0{});
        fetch_positions(chunk_of(2), S0{});
        fetch_rows(S1{});
    } else {
        fetch_positions(chunk_of(0), S0{});
        fetch_rows(S0{});
        fetch_positions(chunk_of(1), S0{});
    }
    for (int it = 0; it < nit; it += 2) {
        step(it, std::integral_constant<int, 0>{});
        if (it + 1 < nit) step(it + 1, std::integral_constant<int, 1>{});
    }
}

template <typename T, int D, int C, int NDW, bool WRAP, bool SAME>
hipError_t launch_one(const void* qk, const void* v, const int32_t* perm, const int16_t* cid,
                      void* o_rounds, float* lse, long bh, int L, int n_r, int causal, float scale,
                      hipStream_t s)
{
    const int nchunks = L / C;
    // workgroups per CU of this kernel (registers and LDS), computed once
    static const int per_cu = [] {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, (const void*)k_chunk_attn<T, D, C, NDW, WRAP, SAME>,
                                                         4 * C, 0) != hipSuccess || b < 1)
            b = 1;
        return b;
    }();
    const int run_len = run_length_fit(nchunks, bh * n_r, (long)per_cu * device_cus());
    const int nruns = (nchunks + run_len - 1) / run_len;
    const long blocks = bh * nruns * n_r;
    hipLaunchKernelGGL((k_chunk_attn<T, D, C, NDW, WRAP, SAME>), dim3((unsigned)blocks), dim3(4 * C), 0, s,
                       static_cast<const T*>(qk), static_cast<const T*>(v), perm, cid,
                       static_cast<T*>(o_rounds), lse, L, n_r, causal, scale * LOG2E, nruns, run_len);
    return hipGetLastError();
}

// Dispatch on the number of packed chunk-id words (1, 2, 4 or 8 for up to 16
// rounds; 0 without the duplicate-count term).
template <typename T, int D, int C, bool WRAP, bool SAME>
hipError_t launch_ndw(const void* qk, const void* v, const int32_t* perm, const int16_t* cid,
                      void* o, float* lse, long bh, int L, int n_r, int causal, float scale,
                      bool dup, hipStream_t s)
{
#define LSH_ONE(NDW) \
    launch_one<T, D, C, NDW, WRAP, SAME>(qk, v, perm, cid, o, lse, bh, L, n_r, causal, scale, s)
    if (!dup) return LSH_ONE(0);
    if (n_r <= 2) return LSH_ONE(1);
    if (n_r <= 4) return LSH_ONE(2);
    if (n_r <= 8) return LSH_ONE(4);
    return LSH_ONE(8);
#undef LSH_ONE
}

// Dispatch on the variant flags (LSH_FLAG_NO_DUP_CORRECTION = 1,
// LSH_FLAG_WRAP_LOOKBACK = 2, LSH_FLAG_SAME_BUCKET = 4; the host rejects 2 | 4).
template <typename T, int D, int C>
hipError_t launch_flags(const void* qk, const void* v, const int32_t* perm, const int16_t* cid,
                        void* o, float* lse, long bh, int L, int n_r, int causal, float scale,
                        int flags, hipStream_t s)
{
    const bool dup = !(flags & 1);
    if (flags & 4)
        return launch_ndw<T, D, C, false, true>(qk, v, perm, cid, o, lse, bh, L, n_r, causal, scale, dup, s);
    if (flags & 2)
        return launch_ndw<T, D, C, true, false>(qk, v, perm, cid, o, lse, bh, L, n_r, causal, scale, dup, s);
    return launch_ndw<T, D, C, false, false>(qk, v, perm, cid, o, lse, bh, L, n_r, causal, scale, dup, s);
}

}  // namespace attn
}  // namespace lshk
