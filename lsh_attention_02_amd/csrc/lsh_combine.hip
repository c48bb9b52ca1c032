// Round combine on gfx950 (modulabs-hub Reformer notes, "Multi-round LSH
// attention": the hash rounds are run several times and merged):
//   LSE_i = logsumexp_r lse[r, i],   o_i = sum_r exp(lse[r, i] - LSE_i) o_rounds[r, i].
// Streaming and bandwidth-bound: each thread owns 16 bytes of one output row
// and reads the same 16 bytes of that row in every round (coalesced rows).
// Every byte is read or written once, so the loads and stores are
// non-temporal (they do not displace cached data).
#include "lsh_device.h"
#include "lsh_internal.h"

namespace lshk {
namespace {

constexpr int COMB_THREADS = 256;
constexpr int MAX_ROUNDS = 16;

// NR: n_r rounded up to a power of two; rounds n_r .. NR-1 repeat round n_r - 1
// (a valid address) and are not used, so that every load of the thread is
// issued before the first one is waited for.
template <typename T, int D, int NR>
__global__ __launch_bounds__(COMB_THREADS)
void k_combine(const T* __restrict__ o_rounds, const float* __restrict__ lse, T* __restrict__ o,
               long rows, int L, int n_r)
{
    constexpr int VE = 16 / (int)sizeof(T);        // elements per thread
    constexpr int TPR = D / VE;                    // threads per row
    constexpr int RPB = COMB_THREADS / TPR;        // rows per block
    const long row = (long)blockIdx.x * RPB + threadIdx.x / TPR;
    const int part = threadIdx.x % TPR;
    if (row >= rows) return;
    const long bh = row / L;
    const int i = (int)(row % L);
    float l[NR];
    u32x4 raw[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const long rr = bh * n_r + min(r, n_r - 1);
        l[r] = lse[rr * L + i];
        raw[r] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(o_rounds + (rr * L + i) * D + part * VE));
    }
    float m = -INFINITY;
#pragma unroll
    for (int r = 0; r < NR; ++r)
        if (r < n_r) m = fmaxf(m, l[r]);
    float acc[VE];
#pragma unroll
    for (int x = 0; x < VE; ++x) acc[x] = 0.f;
    float wsum = 0.f;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        if (r < n_r) {
            const float w = __expf(l[r] - m);
            wsum += w;
            const T* e = reinterpret_cast<const T*>(&raw[r]);
#pragma unroll
            for (int x = 0; x < VE; ++x) acc[x] += w * to_f32(e[x]);
        }
    }
    const float inv = 1.f / wsum;
    u32x4 out;
    T* oe = reinterpret_cast<T*>(&out);
#pragma unroll
    for (int x = 0; x < VE; ++x) oe[x] = from_f32<T>(acc[x] * inv);
    __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(o + row * D + part * VE));
}

template <typename T, int D, int NR>
hipError_t launch_nr(const void* o_rounds, const float* lse, void* o, long bh, int L, int n_r,
                     hipStream_t s)
{
    constexpr int RPB = COMB_THREADS / (D / (16 / (int)sizeof(T)));
    const long rows = bh * L;
    const long blocks = (rows + RPB - 1) / RPB;
    hipLaunchKernelGGL((k_combine<T, D, NR>), dim3((unsigned)blocks), dim3(COMB_THREADS), 0, s,
                       static_cast<const T*>(o_rounds), lse, static_cast<T*>(o), rows, L, n_r);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch(const void* o_rounds, const float* lse, void* o, long bh, int L, int n_r,
                  hipStream_t s)
{
    if (n_r <= 1) return launch_nr<T, D, 1>(o_rounds, lse, o, bh, L, n_r, s);
    if (n_r <= 2) return launch_nr<T, D, 2>(o_rounds, lse, o, bh, L, n_r, s);
    if (n_r <= 4) return launch_nr<T, D, 4>(o_rounds, lse, o, bh, L, n_r, s);
    if (n_r <= 8) return launch_nr<T, D, 8>(o_rounds, lse, o, bh, L, n_r, s);
    return launch_nr<T, D, MAX_ROUNDS>(o_rounds, lse, o, bh, L, n_r, s);
}

}  // namespace

hipError_t launch_combine(int dtype, int d_head, const void* o_rounds, const float* lse, void* o,
                          long bh, int L, int n_rounds, hipStream_t stream)
{
    if (dtype == 1)
        return d_head == 64 ? launch<bf16_t, 64>(o_rounds, lse, o, bh, L, n_rounds, stream)
                            : launch<bf16_t, 128>(o_rounds, lse, o, bh, L, n_rounds, stream);
    return d_head == 64 ? launch<float, 64>(o_rounds, lse, o, bh, L, n_rounds, stream)
                        : launch<float, 128>(o_rounds, lse, o, bh, L, n_rounds, stream);
}

}  // namespace lshk
