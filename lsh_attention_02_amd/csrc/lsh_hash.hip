// Angular LSH hash on gfx950: bucket = index of the largest entry of [p, -p],
// p = qk_i · R_r  (Ultralytics glossary "Reformer", section on LSH attention;
// modulabs-hub Reformer notes, "Locality sensitive hashing").
//
// One workgroup = 8 waves (4 for k_hash_tr at d 64); each wave owns HASH_NT
// tiles of 32 tokens of one (batch row, head).  The tokens are the MFMA column (lane) axis and the
// projection columns are the row (register) axis, so a token's projections
// land in two lanes (l, l+32) as registers and the argmax is an in-register
// scan followed by one cross-half exchange.  The token operands stay in
// registers for every round.
//
// R streams through LDS in groups of columns; the groups of all rounds form
// one sequence, and the next group is loaded while the current one feeds the
// MFMAs (two LDS buffers, one barrier per group).  At d 128 the column tiles
// are software-pipelined: each tile's argmax scan runs under the next tile's
// MFMAs.  Two kernels:
//   k_hash_tr (bf16, rows of R 16-byte aligned): the group is copied from
//     global memory straight into LDS in R's own [d][column] layout, and the
//     MFMA operands are read with the transposing LDS load;
//   k_hash (fp32, or unaligned rows): the group is loaded into registers,
//     transposed there to [column][d] and stored, so that each operand read
//     is contiguous.
// Both LDS layouts XOR-swizzle 16-byte pieces so that stores and operand reads
// are free of bank conflicts.
//
// argmax over [p, -p] is the argmax of |p| with the sign selecting the half:
// entry k of p and entry k of -p have the same magnitude.  The scan keeps the
// lowest column among exact |p| ties; an all-zero projection gives bucket 0.
#include "lsh_device.h"
#include "lsh_internal.h"

#include <climits>


namespace lshk {
namespace {

constexpr int HASH_WAVES = 8;
constexpr int HASH_NT = 2;
constexpr int HASH_THREADS = HASH_WAVES * 64;
constexpr int HASH_TOK_WG = HASH_WAVES * HASH_NT * 32;
constexpr int GROUP_COLS = 128;                  // R columns staged per step
constexpr int GROUP_TILES = GROUP_COLS / 32;

template <typename T, int D>
struct HashStage {
    static constexpr int VE = 16 / (int)sizeof(T);                // elements per 16-byte piece
    static constexpr int NP = D / VE;                              // pieces per R^T row
    static constexpr int ROWB = D * (int)sizeof(T);                // bytes per R^T row (no padding)
    static constexpr int CB = GROUP_COLS / VE;                     // column blocks per group
    static constexpr int BLOCKS = NP * CB;                         // VE x VE blocks per group
    static constexpr int PER_THREAD = (BLOCKS + HASH_THREADS - 1) / HASH_THREADS;
};

// LDS position of 16-byte piece p of R^T row c: p ^ swz(c).  With this XOR
// swizzle both the transposed block stores (16 lanes: one d-piece, 16 column
// blocks) and the MFMA operand reads (16 lanes: 16 consecutive rows, one piece)
// touch 16 distinct 16-byte bank groups.
template <int NP>
__device__ __forceinline__ int swz(int c) { return (c ^ (c >> 3)) & (NP - 1); }

// Global -> registers: block b of the group covers d-rows VE*(b / CB) .. +VE and
// columns c0 + VE*(b % CB) .. +VE (one 16-byte load per d-row; consecutive
// threads read consecutive column blocks of a row, coalesced).  Returns the
// mask of this thread's pieces that hold columns of R; stage_store zeroes the
// others.  With 16-byte aligned rows every lane loads a valid piece (clamped
// into the row) and nothing tests the loaded values here: a test would make
// the wave wait for every load in flight, the next group's included.
template <typename T, int D, int NREG>
__device__ __forceinline__ uint32_t stage_load(u32x4 (&reg)[NREG], const T* __restrict__ Rr, int c0,
                                               int ncol, bool vec_ok)
{
    using S = HashStage<T, D>;
    static_assert(NREG == S::PER_THREAD * S::VE && NREG <= 32, "one mask bit per piece");
    uint32_t valid = 0u;
    // (bf16 comes here only with unaligned rows: k_hash_tr takes the others)
    if (sizeof(T) == 4 && vec_ok) {                // ncol is a multiple of VE (and at least VE)
#pragma unroll
        for (int i = 0; i < S::PER_THREAD; ++i) {
            const int b = threadIdx.x + i * HASH_THREADS;
            const int bb = min(b, S::BLOCKS - 1);
            const int c = c0 + S::VE * (bb % S::CB);
            const int cc = min(c, ncol - S::VE);
#pragma unroll
            for (int y = 0; y < S::VE; ++y) {
                const int d = S::VE * (bb / S::CB) + y;
                reg[i * S::VE + y] = *reinterpret_cast<const u32x4*>(Rr + (long)d * ncol + cc);
                if (b < S::BLOCKS && c < ncol) valid |= 1u << (i * S::VE + y);
            }
        }
        return valid;
    }
#pragma unroll
    for (int i = 0; i < S::PER_THREAD; ++i) {
        const int b = threadIdx.x + i * HASH_THREADS;
#pragma unroll
        for (int y = 0; y < S::VE; ++y) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (b < S::BLOCKS) {
                const int d = S::VE * (b / S::CB) + y;
                const int c = c0 + S::VE * (b % S::CB);
                const T* src = Rr + (long)d * ncol + c;
#pragma unroll
                for (int x = 0; x < S::VE; ++x) {
                    if (c + x < ncol) {
                        uint32_t e;
                        if constexpr (sizeof(T) == 2) e = reinterpret_cast<const uint16_t*>(src)[x];
                        else e = __float_as_uint(reinterpret_cast<const float*>(src)[x]);
                        if constexpr (sizeof(T) == 2) v[x >> 1] |= e << (16 * (x & 1));
                        else v[x] = e;
                    }
                }
            }
            reg[i * S::VE + y] = v;
        }
    }
    return ~0u;                                    // zero-filled element by element
}

// Registers -> LDS: transpose each VE x VE block in registers; column x of the
// block becomes one 16-byte piece (VE consecutive d) of R^T row c.  Pieces
// outside stage_load's mask (columns past ncol) are stored as zeros.
template <typename T, int D, int NREG>
__device__ __forceinline__ void stage_store(u32x4 (&reg)[NREG], uint32_t valid, char* buf)
{
    using S = HashStage<T, D>;
#pragma unroll
    for (int k = 0; k < NREG; ++k)
        if (!((valid >> k) & 1u)) reg[k] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < S::PER_THREAD; ++i) {
        const int b = threadIdx.x + i * HASH_THREADS;
        if (b < S::BLOCKS) {
            const int p = b / S::CB;
            const int cbase = S::VE * (b % S::CB);
#pragma unroll
            for (int x = 0; x < S::VE; ++x) {
                u32x4 out;
                if constexpr (sizeof(T) == 2) {
                    // word w of column x = (row 2w, col x) | (row 2w+1, col x) << 16
                    const uint32_t sel = (x & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        out[w] = __builtin_amdgcn_perm(reg[i * 8 + 2 * w + 1][x >> 1],
                                                       reg[i * 8 + 2 * w][x >> 1], sel);
                } else {
#pragma unroll
                    for (int w = 0; w < 4; ++w) out[w] = reg[i * 4 + w][x];
                }
                const int c = cbase + x;
                *reinterpret_cast<u32x4*>(buf + c * S::ROWB + 16 * (p ^ swz<S::NP>(c))) = out;
            }
        }
    }
}

template <typename T, int D>
__global__ __launch_bounds__(HASH_THREADS)
void k_hash(const T* __restrict__ qk, const T* __restrict__ R, int32_t* __restrict__ buckets,
            int L, int n_r, int ncol, int tiles_per_bh)
{
    using M = Mfma<T>;
    using S = HashStage<T, D>;
    constexpr int KPL = M::KPL, KSTEP = M::KSTEP, NKS = D / KSTEP;
    __shared__ __attribute__((aligned(256))) char rt[2][GROUP_COLS * S::ROWB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const long bh = blockIdx.x / tiles_per_bh;
    const int tok0 = (blockIdx.x % tiles_per_bh) * HASH_TOK_WG + wave * HASH_NT * 32;
    const T* q = qk + bh * (long)L * D;

    // float: step ks takes d = 8 (ks / 4) + 4 hh + ks % 4 (the contraction order
    // is free as long as both operands use it), so a lane reads 4 consecutive
    // d per 4 steps, one 16-byte load, instead of one 4-byte load per step:
    // many narrow loads of scattered rows queue in the CU's address unit.
    // Tokens past L read row L - 1; their buckets are never stored.  Not at
    // d 128, whose 64 steps of operands do not fit in registers either way
    // (this order would raise the spill).
    constexpr bool F4 = sizeof(T) == 4 && D == 64;
    typename M::Frag bq[HASH_NT][NKS];
#pragma unroll
    for (int u = 0; u < HASH_NT; ++u) {
        const int tok = tok0 + 32 * u + n;
        if constexpr (F4) {
            const float* row = reinterpret_cast<const float*>(q) + (long)min(tok, L - 1) * D + 4 * hh;
#pragma unroll
            for (int m = 0; m < NKS / 4; ++m) {
                const float4 v = *reinterpret_cast<const float4*>(row + 8 * m);
                bq[u][4 * m] = v.x; bq[u][4 * m + 1] = v.y; bq[u][4 * m + 2] = v.z; bq[u][4 * m + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                bq[u][ks] = tok < L ? M::load(q + (long)tok * D + ks * KSTEP + hh * KPL) : M::zero();
        }
    }

    const int groups_per_round = (ncol + GROUP_COLS - 1) / GROUP_COLS;
    const int ngroups = n_r * groups_per_round;
    const bool vec_ok = (ncol % S::VE) == 0;           // 16-byte aligned R rows

    u32x4 reg[S::PER_THREAD * S::VE];
    uint32_t rvalid = stage_load<T, D>(reg, R, 0, ncol, vec_ok);
    stage_store<T, D>(reg, rvalid, rt[0]);
    __syncthreads();

    // Per token tile u, over the round so far: the largest |p| among this lane's
    // columns, the 32-column tile of the round that holds it (-1: none yet) and
    // that tile's 16 values of this lane.  A tile replaces the record only when
    // its maximum is strictly larger, and the first matching entry of the kept
    // tile is taken at the end of the round, so the lowest column wins exact ties.
    float bmag[HASH_NT];
    int btile[HASH_NT];
    f32x16 keep[HASH_NT];

    // Byte offsets of the tile-0 operand pieces of this lane (row n), per k-step.
    // Within a group, the swizzle of row 32*ct + n is swz(n) ^ (4*ct mod NP) (the
    // two parts occupy disjoint bits), which maps k-step ks of tile ct onto the
    // piece that k-step ks ^ kx(ct) has in tile 0; only a constant offset of
    // 32*ct rows remains, folded into the LDS instruction.
    constexpr bool kTable = NKS <= 8;
    int off0[kTable ? NKS : 1];
    if constexpr (kTable) {
        const int sw0 = swz<S::NP>(n);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int e = ks * KSTEP + hh * KPL;
            off0[ks] = n * S::ROWB + 16 * ((e / S::VE) ^ sw0) + (e % S::VE) * (int)sizeof(T);
        }
    }

    for (int g = 0; g < ngroups; ++g) {
        const int r = g / groups_per_round;
        const int c0 = (g % groups_per_round) * GROUP_COLS;
        if (c0 == 0) {
#pragma unroll
            for (int u = 0; u < HASH_NT; ++u) { bmag[u] = 0.f; btile[u] = -1; keep[u] = f32x16{}; }
        }
        if (g + 1 < ngroups) {
            const int r1 = (g + 1) / groups_per_round;
            const int c1 = ((g + 1) % groups_per_round) * GROUP_COLS;
            rvalid = stage_load<T, D>(reg, R + (long)r1 * D * ncol, c1, ncol, vec_ok);
        }
        const char* buf = rt[g & 1];
        // R^T rows past ncol hold zeros (stage_store), so their projections are
        // exactly 0 and can never beat a record: no column test is needed.
        const int tiles = min(GROUP_TILES, (ncol - c0 + 31) >> 5);
#pragma unroll
        for (int ct = 0; ct < GROUP_TILES; ++ct) {
            if (ct < tiles) {
                f32x16 acc[HASH_NT];
#pragma unroll
                for (int u = 0; u < HASH_NT; ++u) acc[u] = f32x16{};
                // all of the tile's operand reads first (kept there by the
                // scheduling barrier), so that their LDS latency is paid once
                typename M::Frag a[NKS];
                if constexpr (kTable) {
                    const int kx = ((4 * ct) & (S::NP - 1)) * S::VE / KSTEP;   // constant once unrolled
                    const char* tb = buf + ct * 32 * S::ROWB;
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        a[ks] = *reinterpret_cast<const typename M::Frag*>(tb + off0[ks ^ kx]);
                } else if constexpr (F4) {
                    // the d order of bq: piece 2m + hh of the row holds steps 4m .. 4m+3
                    const int c = ct * 32 + n;
                    const char* rowp = buf + c * S::ROWB;
                    const int sw = swz<S::NP>(c);
#pragma unroll
                    for (int m = 0; m < NKS / 4; ++m) {
                        const float4 v = *reinterpret_cast<const float4*>(rowp + 16 * ((2 * m + hh) ^ sw));
                        a[4 * m] = v.x; a[4 * m + 1] = v.y; a[4 * m + 2] = v.z; a[4 * m + 3] = v.w;
                    }
                } else {
                    const int c = ct * 32 + n;
                    const char* rowp = buf + c * S::ROWB;
                    const int sw = swz<S::NP>(c);
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const int e = ks * KSTEP + hh * KPL;
                        a[ks] = *reinterpret_cast<const typename M::Frag*>(
                            rowp + 16 * ((e / S::VE) ^ sw) + (e % S::VE) * (int)sizeof(T));
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
                    for (int u = 0; u < HASH_NT; ++u) acc[u] = M::mma(a[ks], bq[u][ks], acc[u]);
                }
                const int tile = (c0 >> 5) + ct;
#pragma unroll
                for (int u = 0; u < HASH_NT; ++u) {
                    float m = fabsf(acc[u][0]);
#pragma unroll
                    for (int j = 1; j < 16; ++j) m = __builtin_elementwise_maximum(m, fabsf(acc[u][j]));
                    const bool up = m > bmag[u];
                    bmag[u] = up ? m : bmag[u];
                    btile[u] = up ? tile : btile[u];
                    keep[u] = up ? acc[u] : keep[u];
                }
            }
        }
        if (c0 + GROUP_COLS >= ncol) {               // last group of round r
#pragma unroll
            for (int u = 0; u < HASH_NT; ++u) {
                // first kept entry with the record magnitude (one always matches:
                // the record is one of the kept values' magnitudes)
                int jj = 0;
                float bv = 0.f;
#pragma unroll
                for (int j = 15; j >= 0; --j) {
                    const bool hit = fabsf(keep[u][j]) == bmag[u];
                    jj = hit ? j : jj;
                    bv = hit ? keep[u][j] : bv;
                }
                int bi = btile[u] < 0 ? INT_MAX : 32 * btile[u] + 4 * hh + 8 * (jj >> 2) + (jj & 3);
                if (btile[u] < 0) bv = 0.f;
                const float ov = __shfl_xor(bv, 32);
                const int oi = __shfl_xor(bi, 32);
                if (fabsf(ov) > fabsf(bv) || (fabsf(ov) == fabsf(bv) && oi < bi)) { bv = ov; bi = oi; }
                if (bi == INT_MAX) bi = 0;           // every projection was exactly zero
                const int tok = tok0 + 32 * u + n;
                if (hh == 0 && tok < L)
                    buckets[((long)bh * n_r + r) * L + tok] = bi + (bv < 0.f ? ncol : 0);
            }
        }
        if (g + 1 < ngroups) stage_store<T, D>(reg, rvalid, rt[(g + 1) & 1]);
        __syncthreads();
    }
}


// ---- bf16 with 16-byte aligned R rows: R staged straight from global memory
// into LDS in its own [d][column] layout (one 16-byte global-to-LDS load per
// lane and piece, no registers, no transpose instructions), and the MFMA A
// operand read with the transposing LDS load: ds_read_b64_tr_b16 gives lane i
// of each 16-lane group element i % 4 of the 4 elements that lanes 4k + i / 4
// (k = 0..3) address.  When lane 4k + q addresses row d0 + k, columns
// cb + 4q .. +3, lane i receives column cb + i of rows d0 .. d0 + 3: four
// consecutive k of its A row.  Two such reads (rows d0 and d0 + 4) give the 8
// elements of one 32x32x16 operand.
// Workgroups of 8 waves at d 128 (one per CU: the registers allow two waves
// per SIMD), of 4 waves at d 64, where three waves per SIMD fit: three
// independent workgroups per CU, whose barriers do not hold each other up.
template <int D> constexpr int tr_waves() { return D == 64 ? 4 : 8; }
template <int D> constexpr bool hash_pipe() { return D == 128; }
constexpr int TR_COLS = 128;                     // R columns staged per step
constexpr int TR_PPR = TR_COLS / 8;              // 16-byte pieces per staged row
constexpr int TR_TILES = TR_COLS / 32;
constexpr int TR_ROWB = TR_COLS * 2;             // bytes per staged row

// Piece p (8 columns, 16 bytes) of staged row d sits at p ^ 4 (d % 4): the 32
// lanes of one read pass (4 consecutive rows x 8 half-pieces) then touch all 64
// banks once.
__device__ __forceinline__ int tr_piece(int p, int d) { return p ^ (4 * (d & 3)); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint64_t u64x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x4 tr_read(const char* p)
{
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)p);
    return __builtin_bit_cast(bf16x4, r);
}

// Group (r, c0) of R into buf: piece P = i * NTH + tid (NTH threads) is staged row
// P / 16, LDS slot P % 16 (global piece slot ^ 4 (row % 4)), so one wave
// instruction fills 1 KiB of consecutive LDS.  Pieces past ncol load a valid
// piece instead and are zeroed by tr_zero_tail once the loads have landed.
template <int D>
__device__ __forceinline__ void tr_stage(const bf16_t* __restrict__ Rr, int c0, int ncol, char* buf)
{
    constexpr int NTH = tr_waves<D>() * 64;
    constexpr int ITERS = D * TR_PPR / NTH;
    const int tid = threadIdx.x, wave = tid >> 6;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
        const int P = i * NTH + tid;
        const int d = P / TR_PPR;
        const int col = min(c0 + 8 * tr_piece(P % TR_PPR, d), ncol - 8);
        __builtin_amdgcn_global_load_lds(Rr + (long)d * ncol + col,
                                         (__attribute__((address_space(3))) void*)(buf + 16 * (i * NTH + wave * 64)),
                                         16, 0, 0);
    }
}

// tr_stage when ncol is a multiple of TR_COLS (no piece past ncol).  Step i
// advances every lane by NTH / 16 rows (a multiple of 4, so the swizzle is
// unchanged): a lane's byte offset within a step (loff) is the same for every
// step and group, and a group costs uniform base addresses only; wv is the
// wave index, uniform
template <int D>
__device__ __forceinline__ void tr_stage_full(const char* Rg, uint32_t loff, int ncol, int wv, char* buf)
{
    constexpr int NTH = tr_waves<D>() * 64;
    const long step = 2L * (NTH / TR_PPR) * ncol;
#pragma unroll
    for (int i = 0; i < D * TR_PPR / NTH; ++i)
        __builtin_amdgcn_global_load_lds(Rg + i * step + loff,
                                         (__attribute__((address_space(3))) void*)(buf + 16 * (i * NTH + wv * 64)),
                                         16, 0, 0);
}

template <int D>
__device__ __forceinline__ void tr_zero_tail(int c0, int ncol, char* buf)
{
    constexpr int NTH = tr_waves<D>() * 64;
#pragma unroll
    for (int i = 0; i < D * TR_PPR / NTH; ++i) {
        const int P = i * NTH + threadIdx.x;
        if (c0 + 8 * tr_piece(P % TR_PPR, P / TR_PPR) >= ncol)
            *reinterpret_cast<u32x4*>(buf + 16 * P) = u32x4{0u, 0u, 0u, 0u};
    }
}

template <int D>
__global__ __launch_bounds__(tr_waves<D>() * 64)
void k_hash_tr(const bf16_t* __restrict__ qk, const bf16_t* __restrict__ R, int32_t* __restrict__ buckets,
               int L, int n_r, int ncol, int tiles_per_bh)
{
    using M = Mfma<bf16_t>;
    constexpr int KPL = M::KPL, KSTEP = M::KSTEP, NKS = D / KSTEP;
    // two buffers as separate arrays, so that the compiler can tell the staged
    // loads into one from the operand reads of the other
    __shared__ __attribute__((aligned(1024))) char rt0[D * TR_ROWB];
    __shared__ __attribute__((aligned(1024))) char rt1[D * TR_ROWB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const long bh = blockIdx.x / tiles_per_bh;
    const int tok0 = (blockIdx.x % tiles_per_bh) * (tr_waves<D>() * HASH_NT * 32) + wave * HASH_NT * 32;
    const bf16_t* q = qk + bh * (long)L * D;

    typename M::Frag bq[HASH_NT][NKS];
#pragma unroll
    for (int u = 0; u < HASH_NT; ++u) {
        const int tok = tok0 + 32 * u + n;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            bq[u][ks] = tok < L ? M::load(q + (long)tok * D + ks * KSTEP + hh * KPL) : M::zero();
    }

    const int groups_per_round = (ncol + TR_COLS - 1) / TR_COLS;
    const int ngroups = n_r * groups_per_round;
    static_assert((tr_waves<D>() * 64 / TR_PPR) % 4 == 0, "staging step must keep the swizzle");
    const bool full = ncol % TR_COLS == 0;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    // this lane's staging offset (bytes) within a step of a group
    const uint32_t loff = (uint32_t)(2 * ((tid / TR_PPR) * ncol + 8 * tr_piece(tid % TR_PPR, tid / TR_PPR)));
    // group (r, c0) of R into buf
    auto stage = [&](int r, int c0, char* buf) __attribute__((always_inline)) {
        const bf16_t* Rr = R + (long)r * D * ncol;
        if (full) tr_stage_full<D>(reinterpret_cast<const char*>(Rr + c0), loff, ncol, wv, buf);
        else tr_stage<D>(Rr, c0, ncol, buf);
    };

    // this lane's transposing-read offsets, per column tile: group G = lane / 16
    // (column half G % 2, k half G / 2), lane 4k + q of it addresses row
    // 8 (G / 2) + k and columns 32 ct + 16 (G % 2) + 4q
    int toff[TR_TILES];
    {
        const int G = lane >> 4, j = lane & 15, k = j >> 2, qq = j & 3;
#pragma unroll
        for (int ct = 0; ct < TR_TILES; ++ct)
            toff[ct] = (8 * (G >> 1) + k) * TR_ROWB
                     + 16 * tr_piece(4 * ct + 2 * (G & 1) + (qq >> 1), k) + 8 * (qq & 1);
    }

    float bmag[HASH_NT];
    int btile[HASH_NT];
    f32x16 keep[HASH_NT];

    auto group_rc = [&](int g, int& r, int& c0) {
        r = g / groups_per_round;
        c0 = (g % groups_per_round) * TR_COLS;
    };
    {
        stage(0, 0, rt0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (TR_COLS > ncol) tr_zero_tail<D>(0, ncol, rt0);
        __syncthreads();
    }

    auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < HASH_NT; ++u) { bmag[u] = 0.f; btile[u] = -1; keep[u] = f32x16{}; }
    };
    // One column tile's projections (16 per lane and token tile) against the
    // round's record: the largest |p| so far, its tile, and that tile's
    // values, in two steps.  tile_max runs under the MFMAs; record is a
    // branch, so that lanes without a new record (and waves where no lane has
    // one, most late tiles of a long round) skip the copy, which moves 64-bit
    // register pairs.  The moves are written as asm: the compiler would
    // otherwise turn the branch back into one select per value.
    auto tile_max = [&](const f32x16& ac) __attribute__((always_inline)) {
        float m = fabsf(ac[0]);
#pragma unroll
        for (int j = 1; j < 16; ++j) m = __builtin_elementwise_maximum(m, fabsf(ac[j]));
        return m;
    };
    auto record = [&](int u, float m, const f32x16& ac, int tile) __attribute__((always_inline)) {
        if (m > bmag[u]) {
            bmag[u] = m;
            btile[u] = tile;
            const u64x8 src = __builtin_bit_cast(u64x8, ac);
            u64x8 dst;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                uint64_t t;
                asm volatile("v_mov_b64 %0, %1" : "=v"(t) : "v"(src[i]));
                dst[i] = t;
            }
            keep[u] = __builtin_bit_cast(f32x16, dst);
        }
    };
    // end of round r: first kept entry with the record magnitude (one always
    // matches), then the better of the two lanes that hold the token
    auto resolve = [&](int r) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < HASH_NT; ++u) {
            int jj = 0;
            float bv = 0.f;
#pragma unroll
            for (int j = 15; j >= 0; --j) {
                const bool hit = fabsf(keep[u][j]) == bmag[u];
                jj = hit ? j : jj;
                bv = hit ? keep[u][j] : bv;
            }
            int bi = btile[u] < 0 ? INT_MAX : 32 * btile[u] + 4 * hh + 8 * (jj >> 2) + (jj & 3);
            if (btile[u] < 0) bv = 0.f;
            const float ov = __shfl_xor(bv, 32);
            const int oi = __shfl_xor(bi, 32);
            if (fabsf(ov) > fabsf(bv) || (fabsf(ov) == fabsf(bv) && oi < bi)) { bv = ov; bi = oi; }
            if (bi == INT_MAX) bi = 0;
            const int tok = tok0 + 32 * u + n;
            if (hh == 0 && tok < L)
                buckets[((long)bh * n_r + r) * L + tok] = bi + (bv < 0.f ? ncol : 0);
        }
    };

    // d 128: software pipeline over column tiles.  The MFMAs of tile t go
    // into accumulator set t % 2 while the scan of tile t - 1 reads the other
    // set, about three VALU instructions per MFMA, and the operands of tile
    // t + 1 are read into the operand registers that each MFMA pair frees.  A
    // wave's own scan and LDS reads thus run under its matrix instructions
    // instead of waiting for the other wave of its SIMD (the group barriers
    // keep the two in phase).  The last tile of a group is scanned under the
    // first tile of the next group, and a round is resolved after the scan of
    // its last tile.  All four tiles of a group are computed: staged columns
    // past ncol hold zeros, whose projections are exactly 0 and never beat a
    // record.
    //
    // d 64: a second accumulator set would cost the third wave per SIMD, so
    // the pipeline runs over the two token tiles instead: the MFMAs of token
    // tile 0 run under the scan of token tile 1 of the previous column tile,
    // and those of token tile 1 under the scan of token tile 0 of this column
    // tile.  The operands of the next column tile of the group are read into a
    // second operand set at the start of each tile.
    constexpr bool PIPE = hash_pipe<D>();
    f32x16 acc[2][HASH_NT];                // d 64: acc[0] only
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int u = 0; u < HASH_NT; ++u) acc[s][u] = f32x16{};
    }
    reset();
    int ptile = 0, pr = 0;                 // previous group's last tile and round
    bool pend = false;                     // previous group ended its round

    auto group = [&](int g, const char* buf, char* nbuf) __attribute__((always_inline)) {
        int r, c0;
        group_rc(g, r, c0);
        int r1, c1;
        group_rc(min(g + 1, ngroups - 1), r1, c1);     // past the last group: the last again, never read
        stage(r1, c1, nbuf);
        const int tbase = c0 >> 5;
        typename M::Frag a[NKS];
        auto read_tile = [&](int ct, int ks) __attribute__((always_inline)) {
            const char* p = buf + toff[ct] + 16 * ks * TR_ROWB;
            a[ks] = __builtin_shufflevector(tr_read(p), tr_read(p + 4 * TR_ROWB),
                                            0, 1, 2, 3, 4, 5, 6, 7);
        };
#pragma unroll
        for (int ct = 0; ct < TR_TILES; ++ct) {
            // operands of tile 0; the others are read under the previous
            // tile's MFMAs
            if (ct == 0) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) read_tile(ct, ks);
            }
            __builtin_amdgcn_sched_barrier(0);
            f32x16 (&ac)[HASH_NT] = acc[ct & 1];
#pragma unroll
            for (int u = 0; u < HASH_NT; ++u) ac[u] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
                for (int u = 0; u < HASH_NT; ++u) ac[u] = M::mma(a[ks], bq[u][ks], ac[u]);
                if (ct + 1 < TR_TILES) read_tile(ct + 1, ks);   // into a[ks], now free
            }
            const f32x16 (&pv)[HASH_NT] = acc[(ct + 1) & 1];
            const int ptl = ct == 0 ? ptile : tbase + ct - 1;
            float pm[HASH_NT];
#pragma unroll
            for (int u = 0; u < HASH_NT; ++u) pm[u] = tile_max(pv[u]);
            // an IR-level scheduler would otherwise sink the maxima of a group
            // below all of its MFMAs
#pragma unroll
            for (int u = 0; u < HASH_NT; ++u) asm volatile("" :: "v"(pm[u]));
#pragma unroll
            for (int i = 0; i < NKS; ++i) {
#pragma unroll
                for (int u = 0; u < HASH_NT; ++u) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
                    if (i > 0) __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);   // one VALU
                }
                if (ct + 1 < TR_TILES)
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);     // two LDS reads
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < HASH_NT; ++u) record(u, pm[u], pv[u], ptl);
            if (ct == 0) {
                if (pend) resolve(pr);
                if (c0 == 0) reset();
            }
        }
        ptile = tbase + TR_TILES - 1;
        pr = r;
        pend = c0 + TR_COLS >= ncol;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the next group has landed
        if (g + 1 < ngroups && c1 + TR_COLS > ncol) tr_zero_tail<D>(c1, ncol, nbuf);
        __syncthreads();
    };

    auto group_split = [&](int g, const char* buf, char* nbuf) __attribute__((always_inline)) {
        int r, c0;
        group_rc(g, r, c0);
        int r1, c1;
        group_rc(min(g + 1, ngroups - 1), r1, c1);     // past the last group: the last again, never read
        stage(r1, c1, nbuf);
        const int tbase = c0 >> 5;
        // column tiles of this group that hold columns below ncol (the others
        // are skipped; a tile is never partly past ncol, as ncol % 8 == 0 and
        // staged columns past it are zero)
        const int tiles = min(TR_TILES, (ncol - c0 + 31) >> 5);
        typename M::Frag a[NKS];
        auto read_tile = [&](int ct, int ks) __attribute__((always_inline)) {
            const char* p = buf + toff[ct] + 16 * ks * TR_ROWB;
            a[ks] = __builtin_shufflevector(tr_read(p), tr_read(p + 4 * TR_ROWB),
                                            0, 1, 2, 3, 4, 5, 6, 7);
        };
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) read_tile(0, ks);
#pragma unroll
        for (int ct = 0; ct < TR_TILES; ++ct) {
            if (ct < tiles) {
                __builtin_amdgcn_sched_barrier(0);
                // token tile 0 under the scan of the pending token tile 1
                acc[0][0] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) acc[0][0] = M::mma(a[ks], bq[0][ks], acc[0][0]);
                const float m1 = tile_max(acc[0][1]);
                asm volatile("" :: "v"(m1));
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);         // two MFMAs
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);         // five VALU
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_barrier(0);
                record(1, m1, acc[0][1], ptile);
                if (ct == 0) {
                    if (pend) resolve(pr);
                    if (c0 == 0) reset();
                }
                // token tile 1 under the scan of token tile 0; the operands of
                // the next column tile are read as each MFMA frees its set
                acc[0][1] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    acc[0][1] = M::mma(a[ks], bq[1][ks], acc[0][1]);
                    if (ct + 1 < TR_TILES) read_tile(ct + 1, ks);      // past `tiles`: read, unused
                }
                const float m0 = tile_max(acc[0][0]);
                asm volatile("" :: "v"(m0));
                const bool rd = ct + 1 < TR_TILES;                    // two LDS reads per MFMA
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                if (rd) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (rd) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (rd) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_barrier(0);
                record(0, m0, acc[0][0], tbase + ct);
                ptile = tbase + ct;
            }
        }
        pr = r;
        pend = c0 + TR_COLS >= ncol;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the next group has landed
        if (g + 1 < ngroups && c1 + TR_COLS > ncol) tr_zero_tail<D>(c1, ncol, nbuf);
        __syncthreads();
    };

    for (int g = 0; g < ngroups; g += 2) {
        if constexpr (PIPE) {
            group(g, rt0, rt1);
            if (g + 1 < ngroups) group(g + 1, rt1, rt0);
        } else {
            group_split(g, rt0, rt1);
            if (g + 1 < ngroups) group_split(g + 1, rt1, rt0);
        }
    }
    if constexpr (PIPE) {
#pragma unroll
        for (int u = 0; u < HASH_NT; ++u) record(u, tile_max(acc[1][u]), acc[1][u], ptile);
    } else {
        record(1, tile_max(acc[0][1]), acc[0][1], ptile);
    }
    resolve(pr);
}

template <typename T, int D>
hipError_t launch(const void* qk, const void* R, int32_t* buckets, long bh, int L, int n_r,
                  int ncol, hipStream_t s)
{
    const int tiles = (L + HASH_TOK_WG - 1) / HASH_TOK_WG;
    if constexpr (sizeof(T) == 2) {
        if (ncol % 8 == 0) {                // 16-byte aligned rows of R
            constexpr int TOK = tr_waves<D>() * HASH_NT * 32;
            const int trt = (L + TOK - 1) / TOK;
            hipLaunchKernelGGL((k_hash_tr<D>), dim3((unsigned)(bh * trt)), dim3(tr_waves<D>() * 64), 0, s,
                               static_cast<const bf16_t*>(qk), static_cast<const bf16_t*>(R), buckets,
                               L, n_r, ncol, trt);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((k_hash<T, D>), dim3((unsigned)(bh * tiles)), dim3(HASH_THREADS), 0, s,
                       static_cast<const T*>(qk), static_cast<const T*>(R), buckets, L, n_r, ncol,
                       tiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_hash(int dtype, int d_head, const void* qk, const void* R, int32_t* buckets,
                       long bh, int L, int n_rounds, int ncol, hipStream_t stream)
{
    if (dtype == 1)
        return d_head == 64 ? launch<bf16_t, 64>(qk, R, buckets, bh, L, n_rounds, ncol, stream)
                            : launch<bf16_t, 128>(qk, R, buckets, bh, L, n_rounds, ncol, stream);
    return d_head == 64 ? launch<float, 64>(qk, R, buckets, bh, L, n_rounds, ncol, stream)
                        : launch<float, 128>(qk, R, buckets, bh, L, n_rounds, ncol, stream);
}

}  // namespace lshk
