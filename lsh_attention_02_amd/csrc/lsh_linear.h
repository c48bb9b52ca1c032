// Shared pieces of the projection GEMMs (lsh_linear.hip: 128 x 128 workgroup
// tiles; lsh_gemm256.hip: 256 x 256 tiles for launches with enough tiles).
//   y[m, n] = sum_k x[m, k] * w[n, k]   (bf16 in and out, fp32 accumulation)
// with head-major or row-major addressing of x and y and a fused epilogue.
#pragma once

#include "lsh_device.h"

namespace lshk {
namespace lin {

enum { IN_ROWS = 0, IN_HEADS = 1 };
enum { OUT_ROWS = 0, OUT_HEADS = 1 };
enum { EPI_BIAS = 1, EPI_RELU = 2, EPI_RESID = 4 };

struct LinShape {
    int M, N, K;        // y [M, N] = x [M, K] * w[N, K]^T
    int L, H, D;        // sequence length, heads, head size (head-major addressing)
    int mt, nt;         // tiles along M and N
    int nmat;           // matrices (2: the qk and v projections share one launch)
    int per_xcd;        // tiles per XCD (see the tile mapping in the kernels)
};

constexpr int NXCD = 8;

// Row m = b*L + i of a tile whose first row m0 = b0*L + i0: (b, i) by carrying
// from (b0, i0), so the division by L happens once per tile.
struct RowPos { int b, i; };

__device__ __forceinline__ RowPos row_pos(RowPos base, int r, int L)
{
    RowPos p{base.b, base.i + r};
    while (p.i >= L) { p.i -= L; ++p.b; }        // at most (tile rows) / L steps
    return p;
}

// Address of the 8 input elements x[m, k .. k+7] (k a multiple of 8, inside one
// head of D elements).
template <int IN, int D>
__device__ __forceinline__ const bf16_t* in_ptr(const bf16_t* x, const LinShape& s, int m,
                                                RowPos p, int k)
{
    if constexpr (IN == IN_ROWS) {
        return x + (long)m * s.K + k;
    } else {
        const int h = k / D, c = k % D;
        return x + (((long)p.b * s.H + h) * s.L + p.i) * D + c;
    }
}

template <int OUT, int D>
__device__ __forceinline__ long out_index(const LinShape& s, int m, RowPos p, int n)
{
    if constexpr (OUT == OUT_ROWS) {
        return (long)m * s.N + n;
    } else {
        const int h = n / D, c = n % D;
        return (((long)p.b * s.H + h) * s.L + p.i) * D + c;
    }
}

// Operand tiles are row-major in LDS, 64 k (eight 16-byte pieces) per row.  A
// 16-byte LDS access is served in four passes of 16 lanes (in each half-wave,
// lane quads of even and of odd bit parity); an MFMA operand read takes one
// piece of 32 consecutive rows (lane = row).  XOR-ing the piece with
// (row / 2) % 8 puts the rows of every pass on distinct banks (rows alternate
// between the two 32-bank halves of a 128-byte row pair); the row stores (8
// lanes per row) are conflict-free under any permutation.
__device__ __forceinline__ int lin_swz(int row, int piece) { return piece ^ ((row >> 1) & 7); }

// Epilogue for 4 consecutive columns n .. n+3 of row m (N is a multiple of 4):
// + bias, ReLU, residual + sign * value, as EPI selects; rounded to bf16.
template <int OUT, int D, int EPI>
__device__ __forceinline__ void store4(bf16_t* __restrict__ y, const LinShape& s, int m, RowPos p,
                                       int n, float e0, float e1, float e2, float e3,
                                       const bf16_t* __restrict__ bias,
                                       const bf16_t* __restrict__ resid, float sign)
{
    float e[4] = {e0, e1, e2, e3};
    const long oi = out_index<OUT, D>(s, m, p, n);
    if constexpr ((EPI & EPI_BIAS) != 0) {
        const u32x2 bb = *reinterpret_cast<const u32x2*>(bias + n);
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] += bf16_to_f32((uint16_t)(bb[i >> 1] >> (16 * (i & 1))));
    }
    if constexpr ((EPI & EPI_RELU) != 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = fmaxf(e[i], 0.f);
    }
    if constexpr ((EPI & EPI_RESID) != 0) {
        const u32x2 rr = *reinterpret_cast<const u32x2*>(resid + oi);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            e[i] = fmaf(sign, e[i], bf16_to_f32((uint16_t)(rr[i >> 1] >> (16 * (i & 1)))));
    }
    const u32x2 v = {pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3])};
    *reinterpret_cast<u32x2*>(y + oi) = v;
}

// The same epilogue for 8 consecutive columns n .. n+7 of row m (n a multiple
// of 8, so inside one head), element by element as store4, with one 16-byte
// store.
template <int OUT, int D, int EPI>
__device__ __forceinline__ void store8(bf16_t* __restrict__ y, const LinShape& s, int m, RowPos p,
                                       int n, f32x4 lo, f32x4 hi, const bf16_t* __restrict__ bias,
                                       const bf16_t* __restrict__ resid, float sign)
{
    float e[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    const long oi = out_index<OUT, D>(s, m, p, n);
    if constexpr ((EPI & EPI_BIAS) != 0) {
        const u32x4 bb = *reinterpret_cast<const u32x4*>(bias + n);
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] += bf16_to_f32((uint16_t)(bb[i >> 1] >> (16 * (i & 1))));
    }
    if constexpr ((EPI & EPI_RELU) != 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = fmaxf(e[i], 0.f);
    }
    if constexpr ((EPI & EPI_RESID) != 0) {
        const u32x4 rr = *reinterpret_cast<const u32x4*>(resid + oi);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            e[i] = fmaf(sign, e[i], bf16_to_f32((uint16_t)(rr[i >> 1] >> (16 * (i & 1)))));
    }
    const u32x4 v = {pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                     pack_bf16x2(e[6], e[7])};
    *reinterpret_cast<u32x4*>(y + oi) = v;
}

// Tiles of a launch in (matrix, row tile, column tile) order; workgroups go to
// the 8 XCDs round-robin by launch index and each XCD has its own L2, so each
// XCD takes a contiguous run of tiles: the column tiles that share an input
// row tile run on one XCD and read it from its L2.
__device__ __forceinline__ int xcd_tile(int bid, int per_xcd) { return (bid % NXCD) * per_xcd + bid / NXCD; }

// 256 x 256-tile launch (lsh_gemm256.hip), instantiated there for the
// combinations the projections use.
template <int IN, int OUT, int D, int EPI>
hipError_t launch_big(const void* x, const void* w0, const void* w1, void* y0, void* y1, int nmat,
                      LinShape s, const void* bias, const void* resid, float sign, hipStream_t st);

}  // namespace lin
}  // namespace lshk
