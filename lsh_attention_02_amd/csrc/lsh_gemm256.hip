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
// consecutive output columns of a row.  The output tile goes out through LDS
// (below): stored straight from the accumulators, each store instruction would
// write 16 bytes into each of 32 rows, and with one workgroup per CU nothing
// hides those partial-line writes.
//
// K steps of 64: the operand tiles (2 x 32 KiB, swizzled as lin_swz) are double
// buffered in LDS (128 KiB, one workgroup per CU) and copied straight from
// global memory with global_load_lds_dwordx4: each lane copies one 16-byte
// piece, chosen so that the 1 KiB a wave instruction writes is 8 swizzled rows;
// no registers, LDS store instructions or waits on them sit between the MFMAs.
// Step kt is multiplied from one buffer while step kt+1 is copied into the
// other; the barrier after step kt (every wave done with its buffer, step kt+1
// landed) starts the copy of step kt+2 into the buffer just freed.  Copies
// past the last step repeat it and rows past M or N repeat the last row (never
// stored), so the loop has no branches.  The source rows are 32-bit byte
// offsets from a per-step base (operands under 4 GiB, checked by the caller).
// (Unrolling the loop by two, so that each buffer is a compile-time symbol,
// made the compiler hoist enough addresses to spill; copying through registers
// instead, as an earlier version did, measured 12-17% slower.)
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
    // two buffers per operand as separate arrays, so that the compiler can tell
    // the copy into one from the operand reads of the other
    __shared__ __attribute__((aligned(1024))) bf16_t sa0[BIG_BM * BIG_BK];
    __shared__ __attribute__((aligned(1024))) bf16_t sa1[BIG_BM * BIG_BK];
    __shared__ __attribute__((aligned(1024))) bf16_t sw0[BIG_BN * BIG_BK];
    __shared__ __attribute__((aligned(1024))) bf16_t sw1[BIG_BN * BIG_BK];

    const int t = xcd_tile(blockIdx.x, s.per_xcd);
    if (t >= s.nmat * s.mt * s.nt) return;             // padding of the last XCD's run
    const int z = t / (s.mt * s.nt), tm = (t / s.nt) % s.mt, tn = t % s.nt;
    const bf16_t* __restrict__ w = z ? w1 : w0;
    bf16_t* __restrict__ y = z ? y1 : y0;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m0 = tm * BIG_BM, n0 = tn * BIG_BN;
    const RowPos base{m0 / s.L, m0 % s.L};

    // LDS piece P = 256 i + tid of a step: row 32 i + tid / 8, slot tid % 8, which
    // holds the row's k piece (tid % 8) ^ swz (lin_swz is an involution); one
    // wave instruction copies 1 KiB of consecutive LDS (8 rows)
    const int piece = (tid % BIG_PIECES) ^ (((tid / BIG_PIECES) >> 1) & 7);
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
    // this thread's source rows as byte offsets (32-bit: operands under 4 GiB)
    // from a per-step base that only the step moves
    uint32_t aoff[BIG_LOADS], woff[BIG_LOADS];
#pragma unroll
    for (int i = 0; i < BIG_LOADS; ++i) {
        if constexpr (IN == IN_ROWS) aoff[i] = (uint32_t)((long)lm[i] * s.K * 2) + 16 * piece;
        else aoff[i] = (uint32_t)(((long)lrow[i].b * s.H * s.L + lrow[i].i) * D * 2) + 16 * piece;
        woff[i] = (uint32_t)((long)ln[i] * s.K * 2) + 16 * piece;
    }
    // global -> LDS copy of step kt (past the last step: the last again, never read)
    auto copy = [&](int kt, bf16_t* da, bf16_t* dw) __attribute__((always_inline)) {
        const int k0 = min(kt, nk - 1) * BIG_BK;
        long ka;
        if constexpr (IN == IN_ROWS) ka = k0;
        else ka = (long)(k0 / D) * s.L * D + k0 % D;
        const char* xa = reinterpret_cast<const char*>(x + ka);
        const char* xw = reinterpret_cast<const char*>(w + k0);
#pragma unroll
        for (int i = 0; i < BIG_LOADS; ++i) {
            const int off = (i * BIG_THREADS + wave * 64) * 8;      // elements
            __builtin_amdgcn_global_load_lds(xa + aoff[i],
                                             (__attribute__((address_space(3))) void*)(da + off), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(xw + woff[i],
                                             (__attribute__((address_space(3))) void*)(dw + off), 16, 0, 0);
        }
    };

    const int wm = wave >> 1, wn = wave & 1;           // this wave's 128 x 128 quarter
    const int r32 = lane & 31, kh = lane >> 5;
    f32x16 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

    // operand reads: rows 128 wm + 32 u + r32 (128 wn + ..), piece 2 ks + kh at
    // slot (2 ks + kh) ^ ((r32 / 2) % 8), as 32 u rows do not change the swizzle:
    // a per-lane offset per ks plus a constant per u
    int roff[BIG_BK / 16];
#pragma unroll
    for (int ks = 0; ks < BIG_BK / 16; ++ks) roff[ks] = r32 * BIG_BK + 8 * lin_swz(r32, 2 * ks + kh);
    auto read_frags = [&](const bf16_t* ba, const bf16_t* bw, int ks, bf16x8 (&ra_)[4], bf16x8 (&rw_)[4]) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            ra_[u] = *reinterpret_cast<const bf16x8*>(&ba[(128 * wm + 32 * u) * BIG_BK + roff[ks]]);
            rw_[u] = *reinterpret_cast<const bf16x8*>(&bw[(128 * wn + 32 * u) * BIG_BK + roff[ks]]);
        }
    };
    // One LDS read after each MFMA: the fragments of sub-step ks+1 arrive while
    // sub-step ks multiplies.
    auto multiply = [&](const bf16_t* ba, const bf16_t* bw) __attribute__((always_inline)) {
        bf16x8 fa[2][4], fw[2][4];
        read_frags(ba, bw, 0, fa[0], fw[0]);
#pragma unroll
        for (int ks = 0; ks < BIG_BK / 16; ++ks) {
            if (ks + 1 < BIG_BK / 16) read_frags(ba, bw, ks + 1, fa[(ks + 1) & 1], fw[(ks + 1) & 1]);
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

    // Step kt is multiplied from buffer kt % 2 while step kt + 1 is being copied
    // into the other; after the barrier that ends step kt (every wave done with
    // its buffer, step kt + 1 landed) the copy of step kt + 2 starts there.
    copy(0, sa0, sw0);
    copy(1, sa1, sw1);
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * BIG_LOADS) : "memory");   // step 0 landed
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        bf16_t* ba = (kt & 1) ? sa1 : sa0;
        bf16_t* bw = (kt & 1) ? sw1 : sw0;
        multiply(ba, bw);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");                  // step kt + 1 landed
        __syncthreads();
        copy(kt + 2, ba, bw);
        __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy outlives the workgroup

    // Epilogue through LDS, free now: 128 rows of the tile per pass as fp32
    // (each of the four 32 KiB operand arrays holds 32 rows of 1 KiB, the
    // 16-byte groups of a row XOR-swizzled by the row), written by the two
    // waves of that half; then every thread stores 8 columns of a row, so each
    // wave instruction writes whole rows instead of 16 bytes of 32 rows.
    // D element j of tile (a, b): column n = 32b + 8(j/4) + 4 kh + (j%4), row m = 32a + r32.
    __syncthreads();                                   // every wave past its operand reads
    float* const st[4] = {reinterpret_cast<float*>(sa0), reinterpret_cast<float*>(sa1),
                          reinterpret_cast<float*>(sw0), reinterpret_cast<float*>(sw1)};
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        if (wm == pass) {
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int jg = 0; jg < 4; ++jg) {
                        const int g = 32 * wn + 8 * b + 2 * jg + kh;      // 16-byte group of the row
                        const f32x16& c = acc[a][b];
                        *reinterpret_cast<f32x4*>(st[a] + r32 * 256 + 4 * (g ^ r32)) =
                            f32x4{c[4 * jg], c[4 * jg + 1], c[4 * jg + 2], c[4 * jg + 3]};
                    }
        }
        __syncthreads();
#pragma unroll
        for (int arr = 0; arr < 4; ++arr)
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                // 8 columns c8 of row r in column half hh: a wave covers 4 rows of one half
                const int idx = it * BIG_THREADS + tid;
                const int c8 = idx & 15, r = (idx >> 4) & 31, hh = idx >> 9;
                const int g0 = 32 * hh + 2 * c8;
                const float* row = st[arr] + r * 256;
                const f32x4 lo = *reinterpret_cast<const f32x4*>(row + 4 * (g0 ^ r));
                const f32x4 hi = *reinterpret_cast<const f32x4*>(row + 4 * ((g0 + 1) ^ r));
                const int rt = 128 * pass + 32 * arr + r;
                const int m = m0 + rt, n = n0 + 128 * hh + 8 * c8;
                if (m < s.M && n < s.N)                    // N is a multiple of 64
                    store8<OUT, D, EPI>(y, s, m, row_pos(base, rt, s.L), n, lo, hi, bias, resid, sign);
            }
        __syncthreads();                               // the arrays are rewritten by the next pass
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
