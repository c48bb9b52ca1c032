// Projection GEMM with 256 x 256 workgroup tiles on gfx950 (the launches of
// lsh_linear.hip that have at least one such tile per CU come here).
//
//   y[m, n] = sum_k x[m, k] * w[n, k]    (bf16, fp32 accumulation; addressing and
//                                         epilogue as in lsh_linear.h)
//
// Four waves, each a 128 x 128 quarter of the tile as 4 x 4 tiles of
// v_mfma_f32_32x32x16_bf16: per 16-wide K sub-step a wave reads 8 operand
// fragments (4 of w, 4 of x) for 16 MFMAs, half the LDS bytes per MFMA of the
// 128 x 128 tiles (whose four 64 x 64 waves read 4 fragments for 4 MFMAs).  The
// accumulators (256 per lane) live in the accumulation registers.  The MFMA
// computes the transposed tile (w as the row operand), so each lane owns 4
// consecutive output columns of a row: one 8-byte store each.
//
// K steps of 64: the operand tiles (2 x 32 KiB, swizzled as lin_swz) are double
// buffered in LDS (128 KiB, one workgroup per CU).  Step kt+1 is held in
// registers while step kt is multiplied, stored into the other buffer after it,
// and step kt+2 is loaded right after the barrier; loads past the last step
// repeat it and rows past M or N repeat the last row (never stored), so the
// loop has no branches.  (Deeper software pipelining across the barrier, and a
// second register set for two steps in flight, measured no faster.)
#include "lsh_device.h"
#include "lsh_internal.h"
#include "lsh_linear.h"

namespace lshk {
namespace lin {
namespace {

constexpr int BIG_BM = 256, BIG_BN = 256, BIG_BK = 64;
constexpr int BIG_THREADS = 256;
constexpr int BIG_PIECES = BIG_BK / 8;                       // 16-byte pieces per row
constexpr int BIG_LOADS = BIG_BM * BIG_PIECES / BIG_THREADS; // pieces per thread per operand (8)

template <int IN, int OUT, int D, int EPI>
__global__ __launch_bounds__(BIG_THREADS)
void k_linear_big(const bf16_t* __restrict__ x, const bf16_t* __restrict__ w0,
                  const bf16_t* __restrict__ w1, bf16_t* __restrict__ y0, bf16_t* __restrict__ y1,
                  const bf16_t* __restrict__ bias, const bf16_t* __restrict__ resid, float sign,
                  LinShape s)
{
    __shared__ __attribute__((aligned(16))) bf16_t sa[2][BIG_BM * BIG_BK];
    __shared__ __attribute__((aligned(16))) bf16_t sw[2][BIG_BN * BIG_BK];

    const int t = xcd_tile(blockIdx.x, s.per_xcd);
    if (t >= s.nmat * s.mt * s.nt) return;             // padding of the last XCD's run
    const int z = t / (s.mt * s.nt), tm = (t / s.nt) % s.mt, tn = t % s.nt;
    const bf16_t* __restrict__ w = z ? w1 : w0;
    bf16_t* __restrict__ y = z ? y1 : y0;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m0 = tm * BIG_BM, n0 = tn * BIG_BN;
    const RowPos base{m0 / s.L, m0 % s.L};

    // piece tid + 256 i: row 32 i + tid / 8, piece tid % 8
    const int piece = tid % BIG_PIECES;
    u32x4 ra[BIG_LOADS], rw[BIG_LOADS];
    const int nk = s.K / BIG_BK;
    RowPos lrow[BIG_LOADS];
    int lm[BIG_LOADS], ln[BIG_LOADS];
#pragma unroll
    for (int i = 0; i < BIG_LOADS; ++i) {
        const int row = 32 * i + tid / BIG_PIECES;
        lm[i] = min(m0 + row, s.M - 1);
        ln[i] = min(n0 + row, s.N - 1);
        lrow[i] = row_pos(base, lm[i] - m0, s.L);
    }
    auto load = [&](int kt) {
        const int k = min(kt, nk - 1) * BIG_BK + 8 * piece;
#pragma unroll
        for (int i = 0; i < BIG_LOADS; ++i) {
            ra[i] = *reinterpret_cast<const u32x4*>(in_ptr<IN, D>(x, s, lm[i], lrow[i], k));
            rw[i] = *reinterpret_cast<const u32x4*>(w + (long)ln[i] * s.K + k);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < BIG_LOADS; ++i) {
            const int row = 32 * i + tid / BIG_PIECES;
            const int off = row * BIG_BK + 8 * lin_swz(row, piece);
            *reinterpret_cast<u32x4*>(&sa[buf][off]) = ra[i];
            *reinterpret_cast<u32x4*>(&sw[buf][off]) = rw[i];
        }
    };

    const int wm = wave >> 1, wn = wave & 1;           // this wave's 128 x 128 quarter
    const int r32 = lane & 31, kh = lane >> 5;
    f32x16 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

    auto read_frags = [&](int buf, int ks, bf16x8 (&ra_)[4], bf16x8 (&rw_)[4]) {
        const int pc = 2 * ks + kh;                    // k = 16 ks + 8 kh .. +8
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int ar = 128 * wm + 32 * u + r32, wr = 128 * wn + 32 * u + r32;
            ra_[u] = *reinterpret_cast<const bf16x8*>(&sa[buf][ar * BIG_BK + 8 * lin_swz(ar, pc)]);
            rw_[u] = *reinterpret_cast<const bf16x8*>(&sw[buf][wr * BIG_BK + 8 * lin_swz(wr, pc)]);
        }
    };
    // One LDS read after each MFMA: the fragments of sub-step ks+1 arrive while
    // sub-step ks multiplies (left alone, the compiler waits for each sub-step's
    // reads before its first MFMA).
    auto multiply = [&](int buf) {
        bf16x8 fa[2][4], fw[2][4];
        read_frags(buf, 0, fa[0], fw[0]);
#pragma unroll
        for (int ks = 0; ks < BIG_BK / 16; ++ks) {
            if (ks + 1 < BIG_BK / 16) read_frags(buf, ks + 1, fa[(ks + 1) & 1], fw[(ks + 1) & 1]);
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[ks & 1][b], fa[ks & 1][a],
                                                                       acc[a][b], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int ks = 0; ks < BIG_BK / 16 - 1; ++ks) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    };

    load(0);
    store(0);
    __syncthreads();
    load(1);
    for (int kt = 0; kt < nk; ++kt) {
        multiply(kt & 1);
        store((kt + 1) & 1);           // step kt+1 (a repeat past the end, never read)
        __syncthreads();
        load(kt + 2);
        __builtin_amdgcn_sched_barrier(0);
    }

    // D element j of tile (a, b): column n = 32b + 8(j/4) + 4 kh + (j%4), row m = 32a + r32
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int r = 128 * wm + 32 * a + r32, m = m0 + r;
        const RowPos p = row_pos(base, r, s.L);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
            for (int jg = 0; jg < 4; ++jg) {
                const int n = n0 + 128 * wn + 32 * b + 8 * jg + 4 * kh;
                if (m < s.M && n < s.N) {
                    const f32x16& c = acc[a][b];
                    store4<OUT, D, EPI>(y, s, m, p, n, c[4 * jg], c[4 * jg + 1], c[4 * jg + 2],
                                        c[4 * jg + 3], bias, resid, sign);
                }
            }
        }
    }
}

}  // namespace

template <int IN, int OUT, int D, int EPI>
hipError_t launch_big(const void* x, const void* w0, const void* w1, void* y0, void* y1, int nmat,
                      LinShape s, const void* bias, const void* resid, float sign, hipStream_t st)
{
    s.mt = (s.M + BIG_BM - 1) / BIG_BM;
    s.nt = (s.N + BIG_BN - 1) / BIG_BN;
    s.nmat = nmat;
    const long tiles = (long)nmat * s.mt * s.nt;
    s.per_xcd = (int)((tiles + NXCD - 1) / NXCD);
    const dim3 grid((unsigned)((long)s.per_xcd * NXCD));
    hipLaunchKernelGGL((k_linear_big<IN, OUT, D, EPI>), grid, dim3(BIG_THREADS), 0, st,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w0),
                       static_cast<const bf16_t*>(w1), static_cast<bf16_t*>(y0),
                       static_cast<bf16_t*>(y1), static_cast<const bf16_t*>(bias),
                       static_cast<const bf16_t*>(resid), sign, s);
    return hipGetLastError();
}

#define LSH_BIG(IN, OUT, D, EPI)                                                                   \
    template hipError_t launch_big<IN, OUT, D, EPI>(const void*, const void*, const void*, void*,   \
                                                    void*, int, LinShape, const void*, const void*, \
                                                    float, hipStream_t);
LSH_BIG(IN_ROWS, OUT_HEADS, 64, 0)
LSH_BIG(IN_ROWS, OUT_HEADS, 128, 0)
LSH_BIG(IN_HEADS, OUT_ROWS, 64, 0)
LSH_BIG(IN_HEADS, OUT_ROWS, 128, 0)
LSH_BIG(IN_HEADS, OUT_ROWS, 64, EPI_RESID)
LSH_BIG(IN_HEADS, OUT_ROWS, 128, EPI_RESID)
LSH_BIG(IN_ROWS, OUT_ROWS, 64, EPI_BIAS | EPI_RELU)
LSH_BIG(IN_ROWS, OUT_ROWS, 64, EPI_BIAS | EPI_RESID)
#undef LSH_BIG

}  // namespace lin
}  // namespace lshk
