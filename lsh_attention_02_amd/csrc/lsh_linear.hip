// Projections of the LSH-attention layer on gfx950: the shared query/key and the
// value projections of the input, and the output projection of the heads
// (modulabs-hub Reformer notes, "LSH attention": one shared projection for
// queries and keys; ai-scholar Reformer article, experiment set-up: d_model 1024,
// 8 heads).
//
//   y[m, n] = sum_k x[m, k] * w[n, k]        (w row-major [N, K], as a linear
//                                             layer's weight; fp32 accumulation)
//
// One bf16 GEMM kernel serves both directions through its addressing:
//   project in   x [B*L, d_model] row-major; output column n = h*d + c of row
//                m = b*L + i goes to qk/v[b, h, i, c] (the head-major layout of
//                the attention steps); grid.z picks (w_qk -> qk) or (w_v -> v);
//   project out  input row m = b*L + i, column k = h*d + c is o[b, h, i, c]
//                (the heads read in place); output y [B*L, d_model] row-major.
//
// Workgroup tile 128 x 128, K step 64, 4 waves of 64 x 64 (2 x 2 tiles of
// v_mfma_f32_32x32x16_bf16).  Both operand tiles are row-major in LDS with the
// eight 16-byte pieces of each 128-byte row XOR-swizzled by (row & 7), so the
// MFMA operand reads (8 rows, one piece) and the row stores are free of bank
// conflicts.  The next K step is loaded into registers while the current one is
// multiplied (two LDS buffers, one barrier per step).
#include "lsh_device.h"
#include "lsh_internal.h"

namespace lshk {
namespace {

constexpr int LIN_BM = 128, LIN_BN = 128, LIN_BK = 64;
constexpr int LIN_THREADS = 256;
constexpr int LIN_PIECES = LIN_BK / 8;                           // 16-byte pieces per tile row
constexpr int LIN_LOADS = LIN_BM * LIN_PIECES / LIN_THREADS;     // pieces per thread per operand

enum { IN_ROWS = 0, IN_HEADS = 1 };
enum { OUT_ROWS = 0, OUT_HEADS = 1 };

struct LinShape {
    int M, N, K;        // y [M, N] = x [M, K] * w[N, K]^T
    int L, H, D;        // sequence length, heads, head size (head-major addressing)
};

// Address of the 8 input elements x[m, k .. k+7] (k a multiple of 8, inside one head).
template <int IN>
__device__ __forceinline__ const bf16_t* in_ptr(const bf16_t* x, const LinShape& s, int m, int k)
{
    if constexpr (IN == IN_ROWS) {
        return x + (long)m * s.K + k;
    } else {
        const int b = m / s.L, i = m % s.L, h = k / s.D, c = k % s.D;
        return x + (((long)b * s.H + h) * s.L + i) * s.D + c;
    }
}

template <int OUT>
__device__ __forceinline__ long out_index(const LinShape& s, int m, int n)
{
    if constexpr (OUT == OUT_ROWS) {
        return (long)m * s.N + n;
    } else {
        const int b = m / s.L, i = m % s.L, h = n / s.D, c = n % s.D;
        return (((long)b * s.H + h) * s.L + i) * s.D + c;
    }
}

__device__ __forceinline__ int lin_swz(int row, int piece) { return piece ^ (row & 7); }

template <int IN, int OUT>
__global__ __launch_bounds__(LIN_THREADS)
void k_linear(const bf16_t* __restrict__ x, const bf16_t* __restrict__ w0,
              const bf16_t* __restrict__ w1, bf16_t* __restrict__ y0, bf16_t* __restrict__ y1,
              LinShape s)
{
    __shared__ __attribute__((aligned(16))) bf16_t sa[2][LIN_BM * LIN_BK];
    __shared__ __attribute__((aligned(16))) bf16_t sw[2][LIN_BN * LIN_BK];

    const bf16_t* __restrict__ w = blockIdx.z ? w1 : w0;
    bf16_t* __restrict__ y = blockIdx.z ? y1 : y0;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m0 = blockIdx.y * LIN_BM, n0 = blockIdx.x * LIN_BN;

    // operand loads: piece p = tid + 256*i covers row p / 8, 16-byte piece p % 8
    u32x4 ra[LIN_LOADS], rw[LIN_LOADS];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < LIN_LOADS; ++i) {
            const int p = tid + LIN_THREADS * i, row = p / LIN_PIECES, piece = p % LIN_PIECES;
            const int m = m0 + row, n = n0 + row, k = k0 + 8 * piece;
            ra[i] = m < s.M ? *reinterpret_cast<const u32x4*>(in_ptr<IN>(x, s, m, k)) : u32x4{};
            rw[i] = n < s.N ? *reinterpret_cast<const u32x4*>(w + (long)n * s.K + k) : u32x4{};
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < LIN_LOADS; ++i) {
            const int p = tid + LIN_THREADS * i, row = p / LIN_PIECES, piece = p % LIN_PIECES;
            const int off = row * LIN_BK + 8 * lin_swz(row, piece);
            *reinterpret_cast<u32x4*>(&sa[buf][off]) = ra[i];
            *reinterpret_cast<u32x4*>(&sw[buf][off]) = rw[i];
        }
    };

    const int wm = wave >> 1, wn = wave & 1;          // this wave's 64 x 64 quarter
    const int r32 = lane & 31, kh = lane >> 5;        // MFMA lane coordinates
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

    const int nk = s.K / LIN_BK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load((kt + 1) * LIN_BK);
#pragma unroll
        for (int ks = 0; ks < LIN_BK / 16; ++ks) {
            const int piece = 2 * ks + kh;            // k = 16 ks + 8 kh .. +8
            bf16x8 fa[2], fw[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int ra_row = 64 * wm + 32 * t + r32, rw_row = 64 * wn + 32 * t + r32;
                fa[t] = *reinterpret_cast<const bf16x8*>(&sa[buf][ra_row * LIN_BK + 8 * lin_swz(ra_row, piece)]);
                fw[t] = *reinterpret_cast<const bf16x8*>(&sw[buf][rw_row * LIN_BK + 8 * lin_swz(rw_row, piece)]);
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fw[b], acc[a][b], 0, 0, 0);
        }
        if (kt + 1 < nk) store(buf ^ 1);
        __syncthreads();
    }

    // D element j of tile (a, b): row 32a + 8(j/4) + 4 kh + (j%4), column 32b + r32
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int n = n0 + 64 * wn + 32 * b + r32;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int m = m0 + 64 * wm + 32 * a + 8 * (j >> 2) + 4 * kh + (j & 3);
                if (m < s.M && n < s.N) y[out_index<OUT>(s, m, n)] = from_f32<bf16_t>(acc[a][b][j]);
            }
        }
    }
}

template <int IN, int OUT>
hipError_t launch(const void* x, const void* w0, const void* w1, void* y0, void* y1, int nmat,
                  const LinShape& s, hipStream_t st)
{
    const dim3 grid((unsigned)((s.N + LIN_BN - 1) / LIN_BN), (unsigned)((s.M + LIN_BM - 1) / LIN_BM),
                    (unsigned)nmat);
    hipLaunchKernelGGL((k_linear<IN, OUT>), grid, dim3(LIN_THREADS), 0, st,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w0),
                       static_cast<const bf16_t*>(w1), static_cast<bf16_t*>(y0),
                       static_cast<bf16_t*>(y1), s);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_project_in(const void* x, const void* w_qk, const void* w_v, void* qk, void* v,
                             long rows, int L, int H, int D, int d_model, hipStream_t stream)
{
    const LinShape s{(int)rows, H * D, d_model, L, H, D};
    return launch<IN_ROWS, OUT_HEADS>(x, w_qk, w_v, qk, v, 2, s, stream);
}

hipError_t launch_project_out(const void* o, const void* w_o, void* y, long rows, int L, int H,
                              int D, int d_model, hipStream_t stream)
{
    const LinShape s{(int)rows, d_model, H * D, L, H, D};
    return launch<IN_HEADS, OUT_ROWS>(o, w_o, w_o, y, y, 1, s, stream);
}

}  // namespace lshk
