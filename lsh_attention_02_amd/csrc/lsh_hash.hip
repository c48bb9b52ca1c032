// Angular LSH hash on gfx950: bucket = index of the largest entry of [p, -p],
// p = qk_i · R_r  (Ultralytics glossary "Reformer", section on LSH attention;
// modulabs-hub Reformer notes, "Locality sensitive hashing").
//
// One workgroup = HASH_WAVES waves; each wave owns HASH_NT tiles of 32 tokens
// of one (batch row, head).  The tokens are the MFMA column (lane) axis and the
// projection columns are the row (register) axis, so a token's projections
// land in two lanes (l, l+32) as registers and the argmax is an in-register
// scan followed by one cross-half exchange.  The token operands stay in
// registers for every round.
//
// R streams through LDS in groups of GROUP_COLS columns, transposed to
// [column][d] so that each MFMA A-operand read is 16 contiguous bytes.  The
// groups of all rounds form one sequence; the next group is loaded from global
// memory into registers while the current one feeds the MFMAs (two LDS
// buffers, one barrier per group).
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
    static constexpr int VE = 16 / (int)sizeof(T);                // elements per 16-byte load
    static constexpr int ROW = D + VE;                             // LDS row of R^T, +16 bytes
    static constexpr int CHUNKS = D * GROUP_COLS / VE;             // 16-byte pieces per group
    static constexpr int PER_THREAD = (CHUNKS + HASH_THREADS - 1) / HASH_THREADS;
    static constexpr int COL_CHUNKS = GROUP_COLS / VE;             // pieces per d-row of a group
};

// Global -> registers: piece e of the group covers d = e / COL_CHUNKS,
// columns c0 + VE * (e % COL_CHUNKS) .. +VE.  Consecutive threads read
// consecutive pieces of a d-row of R (coalesced).
template <typename T, int D, int NREG>
__device__ __forceinline__ void stage_load(uint4 (&reg)[NREG], const T* __restrict__ Rr, int c0,
                                           int ncol, bool vec_ok)
{
    using S = HashStage<T, D>;
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
        const int e = threadIdx.x + i * HASH_THREADS;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (e < S::CHUNKS) {
            const int d = e / S::COL_CHUNKS;
            const int c = c0 + S::VE * (e % S::COL_CHUNKS);
            const T* src = Rr + (long)d * ncol + c;
            if (vec_ok && c + S::VE <= ncol) {
                v = *reinterpret_cast<const uint4*>(src);
            } else {
                T* ve = reinterpret_cast<T*>(&v);
#pragma unroll
                for (int x = 0; x < S::VE; ++x)
                    if (c + x < ncol) ve[x] = src[x];
            }
        }
        reg[i] = v;
    }
}

// Registers -> LDS, transposed: buf[column][d].
template <typename T, int D, int NREG>
__device__ __forceinline__ void stage_store(const uint4 (&reg)[NREG], T* buf)
{
    using S = HashStage<T, D>;
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
        const int e = threadIdx.x + i * HASH_THREADS;
        if (e < S::CHUNKS) {
            const int d = e / S::COL_CHUNKS;
            const int cl = S::VE * (e % S::COL_CHUNKS);
            const T* ve = reinterpret_cast<const T*>(&reg[i]);
#pragma unroll
            for (int x = 0; x < S::VE; ++x) buf[(cl + x) * S::ROW + d] = ve[x];
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
    __shared__ __attribute__((aligned(16))) T rt[2][GROUP_COLS * S::ROW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const long bh = blockIdx.x / tiles_per_bh;
    const int tok0 = (blockIdx.x % tiles_per_bh) * HASH_TOK_WG + wave * HASH_NT * 32;
    const T* q = qk + bh * (long)L * D;

    typename M::Frag bq[HASH_NT][NKS];
#pragma unroll
    for (int u = 0; u < HASH_NT; ++u) {
        const int tok = tok0 + 32 * u + n;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            bq[u][ks] = tok < L ? M::load(q + (long)tok * D + ks * KSTEP + hh * KPL) : M::zero();
    }

    const int groups_per_round = (ncol + GROUP_COLS - 1) / GROUP_COLS;
    const int ngroups = n_r * groups_per_round;
    const bool vec_ok = (ncol % S::VE) == 0;           // 16-byte aligned R rows

    uint4 reg[S::PER_THREAD];
    stage_load<T, D>(reg, R, 0, ncol, vec_ok);
    stage_store<T, D>(reg, rt[0]);
    __syncthreads();

    float bestv[HASH_NT];
    int besti[HASH_NT];
    for (int g = 0; g < ngroups; ++g) {
        const int r = g / groups_per_round;
        const int c0 = (g % groups_per_round) * GROUP_COLS;
        if (c0 == 0) {
#pragma unroll
            for (int u = 0; u < HASH_NT; ++u) { bestv[u] = 0.f; besti[u] = INT_MAX; }
        }
        if (g + 1 < ngroups) {
            const int r1 = (g + 1) / groups_per_round;
            const int c1 = ((g + 1) % groups_per_round) * GROUP_COLS;
            stage_load<T, D>(reg, R + (long)r1 * D * ncol, c1, ncol, vec_ok);
        }
        const T* buf = rt[g & 1];
        const int tiles = min(GROUP_TILES, (ncol - c0 + 31) >> 5);
        for (int ct = 0; ct < tiles; ++ct) {
            f32x16 acc[HASH_NT];
#pragma unroll
            for (int u = 0; u < HASH_NT; ++u) acc[u] = f32x16{};
            const T* arow = buf + (ct * 32 + n) * S::ROW + hh * KPL;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const typename M::Frag a = M::load(arow + ks * KSTEP);
#pragma unroll
                for (int u = 0; u < HASH_NT; ++u) acc[u] = M::mma(a, bq[u][ks], acc[u]);
            }
            const int cb = c0 + ct * 32 + 4 * hh;
            if (c0 + ct * 32 + 32 <= ncol) {
#pragma unroll
                for (int u = 0; u < HASH_NT; ++u) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const float v = acc[u][j];
                        if (fabsf(v) > fabsf(bestv[u])) {
                            bestv[u] = v;
                            besti[u] = cb + 8 * (j >> 2) + (j & 3);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int u = 0; u < HASH_NT; ++u) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int col = cb + 8 * (j >> 2) + (j & 3);
                        const float v = acc[u][j];
                        if (col < ncol && fabsf(v) > fabsf(bestv[u])) {
                            bestv[u] = v;
                            besti[u] = col;
                        }
                    }
                }
            }
        }
        if (c0 + GROUP_COLS >= ncol) {               // last group of round r
#pragma unroll
            for (int u = 0; u < HASH_NT; ++u) {
                float bv = bestv[u];
                int bi = besti[u];
                const float ov = __shfl_xor(bv, 32);
                const int oi = __shfl_xor(bi, 32);
                if (fabsf(ov) > fabsf(bv) || (fabsf(ov) == fabsf(bv) && oi < bi)) { bv = ov; bi = oi; }
                if (bi == INT_MAX) bi = 0;           // every projection was exactly zero
                const int tok = tok0 + 32 * u + n;
                if (hh == 0 && tok < L)
                    buckets[((long)bh * n_r + r) * L + tok] = bi + (bv < 0.f ? ncol : 0);
            }
        }
        if (g + 1 < ngroups) stage_store<T, D>(reg, rt[(g + 1) & 1]);
        __syncthreads();
    }
}

template <typename T, int D>
hipError_t launch(const void* qk, const void* R, int32_t* buckets, long bh, int L, int n_r,
                  int ncol, hipStream_t s)
{
    const int tiles = (L + HASH_TOK_WG - 1) / HASH_TOK_WG;
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
