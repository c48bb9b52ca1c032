// Chunked LSH attention on gfx950, one output per hash round.
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
// Workgroup = C/32 waves; it walks a run of consecutive chunks of one
// (b, h, r).  Each chunk's qk rows (row-major) and v rows (transposed) are
// gathered once into LDS and kept for the next chunk, whose look-back window
// they form.  Wave w takes the 32 queries in rows 32w.. of the chunk:
//   S^T[key, q] = K[key, :] · Q[q, :]     (A = key rows, B = query rows)
// so each lane holds one query's scores as registers (keys 8(j/4)+4h+(j%4) of
// each 32-key tile), the softmax is in-register plus one exchange between the
// two half-waves, and the probabilities feed the PV product directly as the B
// operand:
//   O^T[d, q] = V^T[d, key] · P^T[key, q]
// with V^T read from LDS in the same key order.  Rows of o_rounds and lse go
// back to original position order.  Scores are kept in base 2 (exp2/log2).
#include "lsh_device.h"
#include "lsh_internal.h"

namespace lshk {
namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float SELF_PENALTY = 1.0e5f;               // score units
constexpr int CIDW = 8;                              // uint32 words per chunk-id row (16 rounds)
constexpr int RUN = 8;                               // chunks per workgroup

template <typename T, int D, int C>
struct AttnLds {
    static constexpr int KROW = D + 16 / (int)sizeof(T);   // qk row, padded by 16 bytes
    static constexpr int VROW = C + 4;                      // v^T row (one slot's keys)
    T k[2][C * KROW];
    T vt[2][D * VROW];
    int pos[2][C];
    uint32_t cid[2][C * CIDW];
};

__device__ __forceinline__ u16x2 as_u16x2(uint32_t x) { return __builtin_bit_cast(u16x2, x); }

// Number of the first `ndw` packed chunk-id words in which query and key chunk
// ids differ by 0 or 1 (query minus key), counted per 16-bit half.
__device__ __forceinline__ int rounds_outside(const uint32_t* qc, const uint32_t* kc, int ndw)
{
    const u16x2 one = {1, 1};
    u16x2 acc = {0, 0};
#pragma unroll
    for (int w = 0; w < CIDW; ++w) {
        if (w < ndw) {
            const u16x2 d = as_u16x2(qc[w]) - as_u16x2(kc[w]);   // modulo 2^16 per half
            acc += __builtin_elementwise_min(d >> 1, one);        // 0 iff d in {0, 1}
        }
    }
    return (int)acc.x + (int)acc.y;
}

template <typename T, int D, int C>
__global__ __launch_bounds__(2 * C)
void k_chunk_attn(const T* __restrict__ qk, const T* __restrict__ v,
                  const int32_t* __restrict__ perm, const int16_t* __restrict__ cid,
                  T* __restrict__ o_rounds, float* __restrict__ lse, int L, int n_r, int causal,
                  float scale_log2, int nruns)
{
    using M = Mfma<T>;
    using S = AttnLds<T, D, C>;
    constexpr int NTH = 2 * C;
    constexpr int KPL = M::KPL, KSTEP = M::KSTEP, NKS = D / KSTEP;
    constexpr int KROW = S::KROW, VROW = S::VROW;
    constexpr int CT = C / 32, NKT = 2 * CT, DT = D / 32;
    constexpr int VE = 16 / (int)sizeof(T), VPR = D / VE;
    __shared__ __attribute__((aligned(16))) S sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;

    int bid = blockIdx.x;
    const int r = bid % n_r;
    bid /= n_r;
    const int run = bid % nruns;
    const long bh = bid / nruns;
    const int nchunks = L / C;
    const int k0 = run * RUN, k1 = min(k0 + RUN, nchunks);

    const T* qb = qk + bh * (long)L * D;
    const T* vb = v + bh * (long)L * D;
    const int32_t* pr = perm + (bh * n_r + r) * (long)L;
    const int16_t* cb = cid + bh * (long)L * n_r;
    T* ob = o_rounds + (bh * n_r + r) * (long)L * D;
    float* lb = lse + (bh * n_r + r) * (long)L;
    const int ndw = (n_r + 1) >> 1;

    for (int k = max(k0 - 1, 0); k < k1; ++k) {
        const int sl = k & 1;
        // ---- gather chunk k into slot sl (the slot of chunk k-2, no longer read)
#pragma unroll
        for (int i = 0; i < (C * VPR) / NTH; ++i) {
            const int e = tid + i * NTH;
            const int row = e / VPR, piece = e % VPR;
            // positions come from the caller's perm: keep the gather inside the row
            const long p = min(max(pr[k * C + row], 0), L - 1);
            const uint4 kv = *reinterpret_cast<const uint4*>(qb + p * D + piece * VE);
            const uint4 vv = *reinterpret_cast<const uint4*>(vb + p * D + piece * VE);
            *reinterpret_cast<uint4*>(&sm.k[sl][row * KROW + piece * VE]) = kv;
            const T* ve = reinterpret_cast<const T*>(&vv);
#pragma unroll
            for (int x = 0; x < VE; ++x) sm.vt[sl][(piece * VE + x) * VROW + row] = ve[x];
        }
        if (tid < C) {
            const int p = min(max(pr[k * C + tid], 0), L - 1);
            sm.pos[sl][tid] = p;
            const int16_t* cr = cb + (long)p * n_r;
#pragma unroll
            for (int w = 0; w < CIDW; ++w) {
                const uint32_t lo = (2 * w < n_r) ? (uint16_t)cr[2 * w] : 0u;
                const uint32_t hi = (2 * w + 1 < n_r) ? (uint16_t)cr[2 * w + 1] : 0u;
                sm.cid[sl][tid * CIDW + w] = lo | (hi << 16);
            }
        }
        __syncthreads();

        if (k >= k0) {
            const int cur = sl, prv = sl ^ 1;
            const bool has_prev = k > 0;
            const int qrow = wave * 32 + n;
            const int qpos = sm.pos[cur][qrow];

            typename M::Frag bq[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                bq[ks] = M::load(&sm.k[cur][qrow * KROW + ks * KSTEP + hh * KPL]);
            uint32_t qc[CIDW];
#pragma unroll
            for (int w = 0; w < CIDW; ++w) qc[w] = sm.cid[cur][qrow * CIDW + w];

            // ---- S^T tiles: tiles [0, CT) are the previous chunk, [CT, 2CT) this one
            f32x16 s[NKT];
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                s[t] = f32x16{};
                if (t < CT && !has_prev) continue;
                const int slk = t < CT ? prv : cur;
                const T* kr = &sm.k[slk][((t % CT) * 32 + n) * KROW + hh * KPL];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) s[t] = M::mma(M::load(kr + ks * KSTEP), bq[ks], s[t]);
            }

            // ---- scale, duplicate counts, self penalty, causal cut; running max
            float mx = -INFINITY;
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                if (t < CT && !has_prev) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) s[t][j] = -INFINITY;
                    continue;
                }
                const int slk = t < CT ? prv : cur;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int krow0 = (t % CT) * 32 + 8 * g + 4 * hh;
                    const int4 kp = *reinterpret_cast<const int4*>(&sm.pos[slk][krow0]);
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const int j = 4 * g + x;
                        const int kpos = x == 0 ? kp.x : x == 1 ? kp.y : x == 2 ? kp.z : kp.w;
                        const int outs = rounds_outside(qc, &sm.cid[slk][(krow0 + x) * CIDW], ndw);
                        const int cnt = max(n_r - outs, 1);
                        float sc = s[t][j] * scale_log2 - __log2f((float)cnt);
                        if (kpos == qpos) sc -= SELF_PENALTY * LOG2E;
                        if (causal && kpos > qpos) sc = -INFINITY;
                        s[t][j] = sc;
                        mx = fmaxf(mx, sc);
                    }
                }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));

            float sum = 0.f;
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float p = __builtin_amdgcn_exp2f(s[t][j] - mx);
                    s[t][j] = p;
                    sum += p;
                }
            }
            sum += __shfl_xor(sum, 32);

            // ---- O^T = V^T · P^T
            f32x16 o[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                if (t < CT && !has_prev) continue;
                const int slk = t < CT ? prv : cur;
                const int key0 = (t % CT) * 32;
                if constexpr (KPL == 8) {
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        bf16x8 b;
#pragma unroll
                        for (int x = 0; x < 8; ++x) b[x] = (__bf16)s[t][8 * half + x];
#pragma unroll
                        for (int dt = 0; dt < DT; ++dt) {
                            const T* vr = &sm.vt[slk][(dt * 32 + n) * VROW + key0 + 16 * half + 4 * hh];
                            const bf16x4 a0 = *reinterpret_cast<const bf16x4*>(vr);
                            const bf16x4 a1 = *reinterpret_cast<const bf16x4*>(vr + 8);
                            const bf16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
                            o[dt] = M::mma(a, b, o[dt]);
                        }
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int key = key0 + 8 * (j >> 2) + 4 * hh + (j & 3);
#pragma unroll
                        for (int dt = 0; dt < DT; ++dt) {
                            const float a = to_f32(sm.vt[slk][(dt * 32 + n) * VROW + key]);
                            o[dt] = M::mma(a, s[t][j], o[dt]);
                        }
                    }
                }
            }

            // ---- normalise, store the query's row and its lse
            const float inv = 1.f / sum;
            T* orow = ob + (long)qpos * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d0 = dt * 32 + 8 * g + 4 * hh;
                    if constexpr (sizeof(T) == 2) {
                        const uint32_t w0 = (uint32_t)f32_to_bf16_rne(o[dt][4 * g + 0] * inv) |
                                            ((uint32_t)f32_to_bf16_rne(o[dt][4 * g + 1] * inv) << 16);
                        const uint32_t w1 = (uint32_t)f32_to_bf16_rne(o[dt][4 * g + 2] * inv) |
                                            ((uint32_t)f32_to_bf16_rne(o[dt][4 * g + 3] * inv) << 16);
                        *reinterpret_cast<uint2*>(orow + d0) = make_uint2(w0, w1);
                    } else {
                        *reinterpret_cast<float4*>(orow + d0) =
                            make_float4(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv,
                                        o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv);
                    }
                }
            }
            if (hh == 0) lb[qpos] = (mx + __log2f(sum)) * LN2;
        }
        __syncthreads();
    }
}

template <typename T, int D, int C>
hipError_t launch(const void* qk, const void* v, const int32_t* perm, const int16_t* cid,
                  void* o_rounds, float* lse, long bh, int L, int n_r, int causal, float scale,
                  hipStream_t s)
{
    const int nchunks = L / C;
    const int nruns = (nchunks + RUN - 1) / RUN;
    const long blocks = bh * nruns * n_r;
    hipLaunchKernelGGL((k_chunk_attn<T, D, C>), dim3((unsigned)blocks), dim3(2 * C), 0, s,
                       static_cast<const T*>(qk), static_cast<const T*>(v), perm, cid,
                       static_cast<T*>(o_rounds), lse, L, n_r, causal, scale * LOG2E, nruns);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_c(int chunk, const void* qk, const void* v, const int32_t* perm,
                    const int16_t* cid, void* o, float* lse, long bh, int L, int n_r, int causal,
                    float scale, hipStream_t s)
{
    switch (chunk) {
        case 32: return launch<T, D, 32>(qk, v, perm, cid, o, lse, bh, L, n_r, causal, scale, s);
        case 64: return launch<T, D, 64>(qk, v, perm, cid, o, lse, bh, L, n_r, causal, scale, s);
        default:
            // float rows at d_head 128 with chunk 128 need more LDS than a CU has;
            // the host rejects that combination before launching.
            if constexpr (sizeof(T) == 4 && D == 128) return hipErrorInvalidValue;
            else return launch<T, D, 128>(qk, v, perm, cid, o, lse, bh, L, n_r, causal, scale, s);
    }
}

}  // namespace

hipError_t launch_chunk_attn(int dtype, int d_head, int chunk, const void* qk, const void* v,
                             const int32_t* perm, const int16_t* cid, void* o_rounds, float* lse,
                             long bh, int L, int n_rounds, int causal, float scale,
                             hipStream_t stream)
{
    if (dtype == 1)
        return d_head == 64
                   ? launch_c<bf16_t, 64>(chunk, qk, v, perm, cid, o_rounds, lse, bh, L, n_rounds,
                                          causal, scale, stream)
                   : launch_c<bf16_t, 128>(chunk, qk, v, perm, cid, o_rounds, lse, bh, L, n_rounds,
                                           causal, scale, stream);
    return d_head == 64 ? launch_c<float, 64>(chunk, qk, v, perm, cid, o_rounds, lse, bh, L,
                                              n_rounds, causal, scale, stream)
                        : launch_c<float, 128>(chunk, qk, v, perm, cid, o_rounds, lse, bh, L,
                                               n_rounds, causal, scale, stream);
}

}  // namespace lshk
