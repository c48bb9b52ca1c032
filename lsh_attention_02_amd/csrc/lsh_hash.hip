// Angular LSH hash on gfx950: bucket = index of the largest entry of [p, -p],
// p = qk_i · R_r  (Ultralytics glossary "Reformer", section on LSH attention;
// modulabs-hub Reformer notes, "Locality sensitive hashing").
//
// One workgroup = HASH_WAVES waves; each wave owns HASH_NT tiles of 32 tokens
// of one (batch row, head).  The tokens are the MFMA column (lane) axis and the
// projection columns are the row (register) axis, so a token's projections
// land in two lanes (l, l+32) as registers and the argmax is an in-register
// scan followed by one cross-half exchange.  The token operands stay in
// registers for every round; R streams through LDS, transposed, one tile of
// 32 columns at a time (double-buffered).
//
// argmax over [p, -p] is the argmax of |p| with the sign selecting the half:
// entry k of p and entry k of -p have the same magnitude.  The scan keeps the
// lowest column among exact |p| ties; an all-zero projection gives bucket 0.
#include "lsh_device.h"
#include "lsh_internal.h"

#include <climits>

namespace lshk {
namespace {

constexpr int HASH_WAVES = 4;
constexpr int HASH_NT = 2;
constexpr int HASH_TOK_WG = HASH_WAVES * HASH_NT * 32;

template <typename T, int D>
__global__ __launch_bounds__(HASH_WAVES * 64)
void k_hash(const T* __restrict__ qk, const T* __restrict__ R, int32_t* __restrict__ buckets,
            int L, int n_r, int ncol, int tiles_per_bh)
{
    using M = Mfma<T>;
    constexpr int KPL = M::KPL, KSTEP = M::KSTEP, NKS = D / KSTEP;
    constexpr int ROW = D + 16 / (int)sizeof(T);     // LDS row of R^T, padded by 16 bytes
    __shared__ __attribute__((aligned(16))) T rt[2][32 * ROW];

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

    const int nct = (ncol + 31) >> 5;
    int it = 0;
    for (int r = 0; r < n_r; ++r) {
        const T* Rr = R + (long)r * D * ncol;
        float bestv[HASH_NT];
        int besti[HASH_NT];
#pragma unroll
        for (int u = 0; u < HASH_NT; ++u) { bestv[u] = 0.f; besti[u] = INT_MAX; }

        for (int ct = 0; ct < nct; ++ct, ++it) {
            T* buf = rt[it & 1];
            const int c0 = ct * 32;
            // Stage R[r][:, c0:c0+32] transposed: buf[c][d].  Reads are coalesced
            // along the columns.  The buffer written here was last read two
            // iterations ago, before the barrier of the previous iteration.
            for (int e = tid; e < 32 * D; e += HASH_WAVES * 64) {
                const int d = e >> 5, c = e & 31;
                buf[c * ROW + d] = (c0 + c < ncol) ? Rr[(long)d * ncol + c0 + c] : T{};
            }
            __syncthreads();

            f32x16 acc[HASH_NT];
#pragma unroll
            for (int u = 0; u < HASH_NT; ++u) acc[u] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const typename M::Frag a = M::load(buf + n * ROW + ks * KSTEP + hh * KPL);
#pragma unroll
                for (int u = 0; u < HASH_NT; ++u) acc[u] = M::mma(a, bq[u][ks], acc[u]);
            }

            const bool full = c0 + 32 <= ncol;
#pragma unroll
            for (int u = 0; u < HASH_NT; ++u) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int col = c0 + 8 * (j >> 2) + 4 * hh + (j & 3);
                    const float v = acc[u][j];
                    if ((full || col < ncol) && fabsf(v) > fabsf(bestv[u])) {
                        bestv[u] = v;
                        besti[u] = col;
                    }
                }
            }
        }

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
}

template <typename T, int D>
hipError_t launch(const void* qk, const void* R, int32_t* buckets, long bh, int L, int n_r,
                  int ncol, hipStream_t s)
{
    const int tiles = (L + HASH_TOK_WG - 1) / HASH_TOK_WG;
    hipLaunchKernelGGL((k_hash<T, D>), dim3((unsigned)(bh * tiles)), dim3(HASH_WAVES * 64), 0, s,
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
