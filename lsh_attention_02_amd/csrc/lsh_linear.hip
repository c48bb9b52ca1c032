// Projections of the LSH-attention layer on gfx950: the shared query/key and the
// value projections of the input, and the output projection of the heads
// (modulabs-hub Reformer notes, "LSH attention": one shared projection for
// queries and keys; ai-scholar Reformer article, experiment set-up: d_model 1024,
// 8 heads).
//
//   y[m, n] = sum_k x[m, k] * w[n, k]        (w row-major [N, K], as a linear
//                                             layer's weight; fp32 accumulation)
//
// One bf16 GEMM kernel serves every projection through its addressing and its
// epilogue:
//   project in   x [B*L, d_model] row-major; output column n = h*d + c of row
//                m = b*L + i goes to qk/v[b, h, i, c] (the head-major layout of
//                the attention steps); grid.z picks (w_qk -> qk) or (w_v -> v);
//   project out  input row m = b*L + i, column k = h*d + c is o[b, h, i, c]
//                (the heads read in place); output y [B*L, d_model] row-major;
//   row-major    x [M, K] -> y [M, N], for the Reformer block's feed-forward
//                layer (Ultralytics "Reformer" glossary, "Capas reversibles y
//                división en fragmentos"; modulabs-hub notes, "Chunking").
// Epilogue (EPI bits): + bias[n], then ReLU, then y = residual + sign * value
// (the reversible block's half update, or its inverse with sign -1).
//
// Workgroup tile 128 x 128, K step 64, 4 waves of 64 x 64 (2 x 2 tiles of
// v_mfma_f32_32x32x16_bf16).  Both operand tiles are row-major in LDS with the
// eight 16-byte pieces of each 128-byte row XOR-swizzled by row, so the MFMA
// operand reads (16 rows, one piece) and the row stores are free of bank
// conflicts.  The next two K steps are loaded into registers while the current
// one is multiplied (two register sets, two LDS buffers, one barrier per step).
#include "lsh_device.h"
#include "lsh_internal.h"
#include "lsh_linear.h"

namespace lshk {
namespace {

using namespace lin;

constexpr int LIN_BM = 128, LIN_BN = 128, LIN_BK = 64;
constexpr int LIN_THREADS = 256;
constexpr int LIN_PIECES = LIN_BK / 8;                           // 16-byte pieces per tile row
constexpr int LIN_LOADS = LIN_BM * LIN_PIECES / LIN_THREADS;     // pieces per thread per operand

template <int IN, int OUT, int D, int EPI>
__global__ __launch_bounds__(LIN_THREADS)
void k_linear(const bf16_t* __restrict__ x, const bf16_t* __restrict__ w0,
              const bf16_t* __restrict__ w1, bf16_t* __restrict__ y0, bf16_t* __restrict__ y1,
              const bf16_t* __restrict__ bias, const bf16_t* __restrict__ resid, float sign,
              LinShape s)
{
    __shared__ __attribute__((aligned(16))) bf16_t sa[2][LIN_BM * LIN_BK];
    __shared__ __attribute__((aligned(16))) bf16_t sw[2][LIN_BN * LIN_BK];

    // Workgroups are dispatched to the 8 XCDs round-robin by launch index, and
    // each XCD has its own L2.  Each XCD takes a contiguous run of tiles in
    // (matrix, row tile, column tile) order, so the column tiles that share an
    // input row tile run on one XCD and read it from its L2.
    const int t = xcd_tile(blockIdx.x, s.per_xcd);
    if (t >= s.nmat * s.mt * s.nt) return;            // padding of the last XCD's run
    const int z = t / (s.mt * s.nt), tm = (t / s.nt) % s.mt, tn = t % s.nt;
    const bf16_t* __restrict__ w = z ? w1 : w0;
    bf16_t* __restrict__ y = z ? y1 : y0;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m0 = tm * LIN_BM, n0 = tn * LIN_BN;
    const RowPos base{m0 / s.L, m0 % s.L};

    // Operand loads: piece p = tid + 256*i covers row p / 8, 16-byte piece p % 8.
    // Rows past M or N repeat the last row: they only reach outputs that are not
    // stored.
    // Two register sets hold K steps kt+1 and kt+2 while step kt is multiplied,
    // so a load has two steps of math to arrive.  Loads past the last step
    // repeat the last step (in bounds, never stored): the loop body has no
    // branches, which lets the compiler wait for exactly the older set.
    u32x4 ra[2][LIN_LOADS], rw[2][LIN_LOADS];
    const int nk = s.K / LIN_BK;
    RowPos lrow[LIN_LOADS];                           // (b, i) of each load's row (head-major input)
    int lm[LIN_LOADS], ln[LIN_LOADS];
#pragma unroll
    for (int i = 0; i < LIN_LOADS; ++i) {
        const int row = (tid + LIN_THREADS * i) / LIN_PIECES;
        lm[i] = min(m0 + row, s.M - 1);
        ln[i] = min(n0 + row, s.N - 1);
        lrow[i] = row_pos(base, lm[i] - m0, s.L);
    }
    auto load = [&](int set, int kt) {
        const int k0 = min(kt, nk - 1) * LIN_BK;
#pragma unroll
        for (int i = 0; i < LIN_LOADS; ++i) {
            const int k = k0 + 8 * ((tid + LIN_THREADS * i) % LIN_PIECES);
            ra[set][i] = *reinterpret_cast<const u32x4*>(in_ptr<IN, D>(x, s, lm[i], lrow[i], k));
            rw[set][i] = *reinterpret_cast<const u32x4*>(w + (long)ln[i] * s.K + k);
        }
    };
    auto store = [&](int set, int buf) {
#pragma unroll
        for (int i = 0; i < LIN_LOADS; ++i) {
            const int p = tid + LIN_THREADS * i, row = p / LIN_PIECES, piece = p % LIN_PIECES;
            const int off = row * LIN_BK + 8 * lin_swz(row, piece);
            *reinterpret_cast<u32x4*>(&sa[buf][off]) = ra[set][i];
            *reinterpret_cast<u32x4*>(&sw[buf][off]) = rw[set][i];
        }
    };

    const int wm = wave >> 1, wn = wave & 1;          // this wave's 64 x 64 quarter
    const int r32 = lane & 31, kh = lane >> 5;        // MFMA lane coordinates
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

    // The MFMA computes the transposed tile, D[n][m] (weights as the row
    // operand): lane (r32, kh) then holds, for each group of four registers,
    // four consecutive output columns of one row, stored with one 8-byte write.
    // The fragments of sub-step ks+1 are read while sub-step ks multiplies: the
    // group barriers ask the scheduler for one LDS read after each MFMA (left to
    // itself it waits for each sub-step's reads before its first MFMA).
    auto read_frags = [&](int buf, int ks, bf16x8 (&fa)[2], bf16x8 (&fw)[2]) {
        const int piece = 2 * ks + kh;                // k = 16 ks + 8 kh .. +8
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int ra_row = 64 * wm + 32 * t + r32, rw_row = 64 * wn + 32 * t + r32;
            fa[t] = *reinterpret_cast<const bf16x8*>(&sa[buf][ra_row * LIN_BK + 8 * lin_swz(ra_row, piece)]);
            fw[t] = *reinterpret_cast<const bf16x8*>(&sw[buf][rw_row * LIN_BK + 8 * lin_swz(rw_row, piece)]);
        }
    };
    auto multiply = [&](int buf) {
        bf16x8 fa[2][2], fw[2][2];
        read_frags(buf, 0, fa[0], fw[0]);
#pragma unroll
        for (int ks = 0; ks < LIN_BK / 16; ++ks) {
            if (ks + 1 < LIN_BK / 16) read_frags(buf, ks + 1, fa[(ks + 1) & 1], fw[(ks + 1) & 1]);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[ks & 1][b], fa[ks & 1][a],
                                                                       acc[a][b], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int ks = 0; ks < LIN_BK / 16 - 1; ++ks) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    };

    // Set kt % 2 holds step kt; LDS buffer kt % 2 holds step kt while it is
    // multiplied.  The scheduling barriers keep each load group at the top of
    // its step (the compiler would otherwise sink the loads towards their LDS
    // stores, which exposes the memory latency).
    load(0, 0);
    load(1, 1);
    store(0, 0);
    __syncthreads();
    int kt = 0;
    for (; kt + 2 <= nk; kt += 2) {
        load(0, kt + 2);              // set 0 held step kt, already in LDS buffer 0
        __builtin_amdgcn_sched_barrier(0);
        multiply(0);
        store(1, 1);                  // step kt+1
        __syncthreads();
        load(1, kt + 3);
        __builtin_amdgcn_sched_barrier(0);
        multiply(1);
        store(0, 0);                  // step kt+2 (a repeat past the end, unused)
        __syncthreads();
    }
    if (kt < nk) multiply(0);         // odd step count: the last step is in buffer 0

    // D element j of tile (a, b): column n = 32b + 8(j/4) + 4 kh + (j%4), row m = 32a + r32
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int r = 64 * wm + 32 * a + r32, m = m0 + r;
        const RowPos p = row_pos(base, r, s.L);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int jg = 0; jg < 4; ++jg) {
                const int n = n0 + 64 * wn + 32 * b + 8 * jg + 4 * kh;   // N is a multiple of 4
                if (m < s.M && n < s.N) {
                    const f32x16& c = acc[a][b];
                    store4<OUT, D, EPI>(y, s, m, p, n, c[4 * jg], c[4 * jg + 1], c[4 * jg + 2],
                                        c[4 * jg + 3], bias, resid, sign);
                }
            }
        }
    }
}

// Launches with at least one 256 x 256 tile per CU take the larger tiles
// (half the LDS and L2 traffic per MFMA); smaller ones keep 128 x 128 tiles
// to fill the chip.  The larger tiles address their operands with 32-bit byte
// offsets, so x and w must each stay under 4 GiB there.
constexpr long BIG_MIN_TILES = 256;
constexpr long BIG_MAX_BYTES = 1L << 32;

template <int IN, int OUT, int D, int EPI>
hipError_t launch(const void* x, const void* w0, const void* w1, void* y0, void* y1, int nmat,
                  LinShape s, const void* bias, const void* resid, float sign, hipStream_t st)
{
    const long big = (long)nmat * ((s.M + 255) / 256) * ((s.N + 255) / 256);
    if (big >= BIG_MIN_TILES && (long)s.M * s.K * 2 < BIG_MAX_BYTES && (long)s.N * s.K * 2 < BIG_MAX_BYTES)
        return launch_big<IN, OUT, D, EPI>(x, w0, w1, y0, y1, nmat, s, bias, resid, sign, st);
    s.mt = (s.M + LIN_BM - 1) / LIN_BM;
    s.nt = (s.N + LIN_BN - 1) / LIN_BN;
    s.nmat = nmat;
    const long tiles = (long)nmat * s.mt * s.nt;
    s.per_xcd = (int)((tiles + NXCD - 1) / NXCD);
    const dim3 grid((unsigned)((long)s.per_xcd * NXCD));
    hipLaunchKernelGGL((k_linear<IN, OUT, D, EPI>), grid, dim3(LIN_THREADS), 0, st,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w0),
                       static_cast<const bf16_t*>(w1), static_cast<bf16_t*>(y0),
                       static_cast<bf16_t*>(y1), static_cast<const bf16_t*>(bias),
                       static_cast<const bf16_t*>(resid), sign, s);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_project_in(const void* x, const void* w_qk, const void* w_v, void* qk, void* v,
                             long rows, int L, int H, int D, int d_model, hipStream_t stream)
{
    const LinShape s{(int)rows, H * D, d_model, L, H, D, 0, 0, 0, 0};
    return D == 64 ? launch<IN_ROWS, OUT_HEADS, 64, 0>(x, w_qk, w_v, qk, v, 2, s, nullptr, nullptr, 0.f, stream)
                   : launch<IN_ROWS, OUT_HEADS, 128, 0>(x, w_qk, w_v, qk, v, 2, s, nullptr, nullptr, 0.f, stream);
}

hipError_t launch_project_out(const void* o, const void* w_o, void* y, long rows, int L, int H,
                              int D, int d_model, const void* resid, float sign, hipStream_t stream)
{
    const LinShape s{(int)rows, d_model, H * D, L, H, D, 0, 0, 0, 0};
    if (resid)
        return D == 64 ? launch<IN_HEADS, OUT_ROWS, 64, EPI_RESID>(o, w_o, w_o, y, y, 1, s, nullptr, resid, sign, stream)
                       : launch<IN_HEADS, OUT_ROWS, 128, EPI_RESID>(o, w_o, w_o, y, y, 1, s, nullptr, resid, sign, stream);
    return D == 64 ? launch<IN_HEADS, OUT_ROWS, 64, 0>(o, w_o, w_o, y, y, 1, s, nullptr, nullptr, 0.f, stream)
                   : launch<IN_HEADS, OUT_ROWS, 128, 0>(o, w_o, w_o, y, y, 1, s, nullptr, nullptr, 0.f, stream);
}

hipError_t launch_ffn(const void* x, const void* w1, const void* b1, const void* w2, const void* b2,
                      const void* resid, float sign, void* y, void* hidden, long rows, int d_model,
                      int d_ff, int chunk_rows, hipStream_t stream)
{
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* rb = static_cast<const bf16_t*>(resid);
    bf16_t* yb = static_cast<bf16_t*>(y);
    for (long r0 = 0; r0 < rows; r0 += chunk_rows) {
        const int cr = (int)(rows - r0 < chunk_rows ? rows - r0 : chunk_rows);
        // the row-major kernels take L = M: (b, i) never carries
        const LinShape s1{cr, d_ff, d_model, cr, 1, 64, 0, 0, 0, 0};
        hipError_t e = launch<IN_ROWS, OUT_ROWS, 64, EPI_BIAS | EPI_RELU>(
            xb + r0 * d_model, w1, w1, hidden, hidden, 1, s1, b1, nullptr, 0.f, stream);
        if (e != hipSuccess) return e;
        const LinShape s2{cr, d_model, d_ff, cr, 1, 64, 0, 0, 0, 0};
        e = launch<IN_ROWS, OUT_ROWS, 64, EPI_BIAS | EPI_RESID>(
            hidden, w2, w2, yb + r0 * d_model, yb + r0 * d_model, 1, s2, b2, rb + r0 * d_model, sign,
            stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace lshk
