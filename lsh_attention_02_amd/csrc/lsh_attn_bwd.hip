// Backward pass of chunked LSH attention + round combine on gfx950 (bfloat16).
//
// The forward (ai-scholar Reformer article and Ultralytics "Reformer" glossary,
// sections on LSH attention; modulabs-hub notes, "LSH attention" and
// "Multi-round LSH attention") gives, after the combine, one softmax per query
// over all (round, key) pairs of its windows:
//     o_i = sum_r sum_j P_ijr v_j,   P_ijr = exp(s_ijr - LSE_i),
// with LSE_i the logsumexp of the rounds' lse.  For a loss gradient d_o at the
// combined output, with Delta_i = <d_o_i, o_i> and dS_ijr = P_ijr (<d_o_i, v_j> -
// Delta_i), the chain rule gives
//     dv_j += P_ijr d_o_i,  dqk_i += scale dS_ijr qk_j,  dqk_j += scale dS_ijr qk_i.
// The buckets are piecewise constant and carry no gradient; the scores are
// recomputed from qk (no attention matrix is kept by the forward).
//
// Kernels:
//   k_bwd_prep    per token-head: LSE (from the per-round lse) and Delta.
//   k_attn_bwd    per (b, h, round, run of chunks), like the forward: the chunk's
//                 rows are gathered into LDS once and kept as the next chunk's
//                 look-back.  Per query chunk c (keys: chunks c-1 and c):
//     phase 1  wave w takes queries 16w..16w+15.  S^T = K Q^T and dP^T = V dO^T
//              on MFMA (as the forward's scores), P and dS in registers; dQ^T =
//              K^T dS^T (as the forward's PV product, K^T in LDS).  P and dS also
//              go to LDS as [key][query] for phase 2.
//     phase 2  the keys: waves 2g, 2g+1 own the chunk held in LDS slot g (32
//              keys each) and accumulate dK^T = Q^T dS and dV^T = dO^T P over
//              the two tiles that chunk is a key of (as the current chunk, then
//              as the look-back of the next); a run ends with one extra tile
//              (the next run's first queries against its last chunk; with the
//              wrap-around variant the last run's extra tile is chunk 0), so
//              every position's key gradient is summed in one workgroup.
//              Results are per-round partials (bf16, original position order).
//              Used with wrap-around look-back and same-bucket windows.
//   k_bwd_q, k_bwd_k  the method (with or without the duplicate-count term):
//                 the query role and the key role of k_attn_bwd in two kernels
//                 with two workgroups per CU each (described with them below);
//                 the same partials, bit for bit.
//   k_bwd_reduce  dqk = sum_r (dq_r + dk_r), dv = sum_r dv_r in fp32.
#include "lsh_chunk_attn.h"

namespace lshk {
namespace attn {
namespace {


// P / dS rows in LDS: one row per window key (2C rows), C queries each, in
// 8-byte groups of 4 queries; group qg of row k is stored at qg ^ pswz(k).
// The phase-2 operand reads (8 bytes, 32 lanes: 16 keys x 2 groups) and the
// phase-1 stores (2 bytes, keys 4g + j of a tile, 64 queries) are then free of
// bank conflicts (rows alternate between the 32-bank halves).
__device__ __forceinline__ int pswz(int k) { return ((k >> 1) & 7) << 1; }

constexpr int PREP_RPT = 4;                         // rows per thread in k_bwd_prep

template <int D, int C, int NDW>
struct BwdLds {
    static constexpr int KROW = KLayout<bf16_t, D>::ROW;
    static constexpr int TROWB = C * 2;              // bytes of a transposed row (C keys)
    static constexpr int PROWB = C * 2;              // bytes of a P / dS row (C queries)
    static constexpr int NW = NDW > 0 ? NDW : 1;
    float neg_log2[36];                              // as in the forward (first member)
    bf16_t k[2][C * KROW];                           // qk rows, slot = iteration % 2
    bf16_t v[2][C * KROW];                           // v rows
    char kt[2][D * TROWB];                           // qk^T rows (d), keys in groups of 4
    char dot[D * TROWB];                             // d_o^T of the query chunk
    char p[2 * C * PROWB];                           // P[key][query] of the current tile
    char ds[2 * C * PROWB];                          // dS[key][query]
    int pos[2][C];
    uint32_t cid[2][C * NW];
    int rid[2][C];                                   // same-bucket variant: window ids, this round
    float lse2[C];                                   // combined logsumexp, log2 units
    float delta[C];
};

// WRAP: chunk 0 looks back to the last chunk of its round; SAME: keys outside
// the query's bucket of this round are dropped (cid holds window ids), as in the
// forward kernel.
template <int D, int C, int NDW, bool WRAP, bool SAME>
__global__ __launch_bounds__(4 * C)
void k_attn_bwd(const bf16_t* __restrict__ qk, const bf16_t* __restrict__ v,
                const bf16_t* __restrict__ d_o, const int32_t* __restrict__ perm,
                const int16_t* __restrict__ cid, const float* __restrict__ lse_c,
                const float* __restrict__ delta, bf16_t* __restrict__ dq_r,
                bf16_t* __restrict__ dk_r, bf16_t* __restrict__ dv_r, int L, int n_r,
                int causal, float scale, float scale_log2, int nruns, int run_len)
{
    using T = bf16_t;
    using M = Mfma16<T>;
    using S = BwdLds<D, C, NDW>;
    using KL = KLayout<T, D>;
    constexpr int NTH = 4 * C, W = C / 16;
    constexpr int KPL = M::KPL, KSTEP = M::KSTEP, NKS = D / KSTEP;
    constexpr int CT = C / 16, NKT = 2 * CT, DT = D / 16;
    constexpr int VE = 8, VPR = D / VE;
    constexpr int TROWB = S::TROWB, PROWB = S::PROWB;
    constexpr int JOBS = (C / 4) * VPR;
    constexpr int JPT = (JOBS + NTH - 1) / NTH;
    constexpr int NW = S::NW;
    constexpr int KSL = 2 * C / W;                   // keys per wave in phase 2
    constexpr int KTW = KSL / 16;                    // 16-key tiles per wave in phase 2
    static_assert(C == 64, "the P/dS layout assumes 64-query chunks");
    __shared__ __attribute__((aligned(16))) S sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;

    int bid = blockIdx.x;
    const int r = bid % n_r;
    bid /= n_r;
    const int run = bid % nruns;
    const long bh = bid / nruns;
    const int nchunks = L / C;
    const int k0 = run * run_len, k1 = min(k0 + run_len, nchunks);

    const T* qb = qk + bh * (long)L * D;
    const T* vb = v + bh * (long)L * D;
    const T* db = d_o + bh * (long)L * D;
    const int32_t* pr = perm + (bh * n_r + r) * (long)L;
    const int16_t* cb = cid + bh * (long)L * n_r;
    const float* lb = lse_c + bh * (long)L;
    const float* deb = delta + bh * (long)L;
    const long rbase = (bh * n_r + r) * (long)L * D;
    const uint32_t ones = 0x00010001u;
    const uint32_t nch2 = (uint32_t)nchunks * 0x00010001u;

    if (tid < 33) sm.neg_log2[tid] = (tid % 2 == 0 && tid / 2 < n_r) ? -__log2f((float)(n_r - tid / 2)) : 0.f;

    auto clamp_pos = [&](int p) {
        LSH_CHECK((unsigned)p < (unsigned)L);
        return min(max(p, 0), L - 1);
    };

    // Gathers for the next chunk, kept raw in registers until stored (as in the
    // forward).  Job = 4 consecutive rows x one 16-byte piece of qk, v and d_o.
    int gpos[JPT][4];
    int mypos = 0, qposraw = 0;
    u32x4 kreg[JPT][4], vreg[JPT][4], dreg[JPT][4];
    u32x4 dofrag[NKS];          // d_o fragments of this lane's query row (next chunk)
    uint32_t craw[2 * NW];
    uint32_t ridraw = 0;
    float lraw = 0.f, draw = 0.f;
    int rpos = 0;

    auto fetch_positions = [&](int kk) {
#pragma unroll
        for (int jb = 0; jb < JPT; ++jb) {
            const int job = tid + jb * NTH;
            const int rg = (job < JOBS ? job : 0) / VPR;
#pragma unroll
            for (int i = 0; i < 4; ++i) gpos[jb][i] = pr[kk * C + 4 * rg + i];
        }
        mypos = pr[kk * C + tid % C];
        qposraw = pr[kk * C + wave * 16 + r16];
    };
    auto fetch_rows = [&]() {
#pragma unroll
        for (int jb = 0; jb < JPT; ++jb) {
            const int job = tid + jb * NTH;
            const int piece = (job < JOBS ? job : 0) % VPR;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const long row = (long)clamp_pos(gpos[jb][i]) * D + piece * VE;
                kreg[jb][i] = *reinterpret_cast<const u32x4*>(qb + row);
                vreg[jb][i] = *reinterpret_cast<const u32x4*>(vb + row);
                dreg[jb][i] = *reinterpret_cast<const u32x4*>(db + row);
            }
        }
        const long qrow = (long)clamp_pos(qposraw) * D;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            dofrag[ks] = *reinterpret_cast<const u32x4*>(db + qrow + ks * KSTEP + g * KPL);
        rpos = clamp_pos(mypos);
        const int16_t* cr = cb + (long)rpos * n_r;
        if constexpr (NDW > 0) {
#pragma unroll
            for (int h = 0; h < 2 * NDW; ++h) craw[h] = (uint16_t)cr[min(h, n_r - 1)];
        }
        if constexpr (SAME) ridraw = (uint16_t)cr[r];
        lraw = lb[rpos];
        draw = deb[rpos];
    };
    // transposed store of 4 rows x VE elements into a [d][row] table (the
    // forward's 16-bit v^T layout: groups of 4 rows, paired as (rg, rg + 4))
    auto store_t = [&](char* base, const u32x4 (&reg)[4], int rg, int piece) {
#pragma unroll
        for (int x = 0; x < VE; ++x) {
            const int xe = x ^ (piece & 1);            // element order x ^ 1 on odd pieces
            const int d = piece * VE + xe;
            char* dst = base + d * TROWB + vt_group_off<C, D>(rg, d);
            const uint32_t sel = 0x05040100u + 0x02020202u * (uint32_t)(xe & 1);
            const uint32_t w0 = __builtin_amdgcn_perm(reg[1][x >> 1], reg[0][x >> 1], sel);
            const uint32_t w1 = __builtin_amdgcn_perm(reg[3][x >> 1], reg[2][x >> 1], sel);
            *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
        }
    };
    auto store_rows = [&](int sl) {
#pragma unroll
        for (int jb = 0; jb < JPT; ++jb) {
            const int job = tid + jb * NTH;
            if (job < JOBS) {
                const int rg = job / VPR, piece = job % VPR;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    *reinterpret_cast<u32x4*>(&sm.k[sl][KL::off(4 * rg + i, piece * VE)]) = kreg[jb][i];
                    *reinterpret_cast<u32x4*>(&sm.v[sl][KL::off(4 * rg + i, piece * VE)]) = vreg[jb][i];
                }
                store_t(sm.kt[sl], kreg[jb], rg, piece);
                store_t(sm.dot, dreg[jb], rg, piece);
            }
        }
        if (tid < C) {
            sm.pos[sl][tid] = rpos;
#pragma unroll
            for (int w = 0; w < NDW; ++w) {
                const uint32_t lo = 2 * w < n_r ? craw[2 * w] : 0u;
                const uint32_t hi = 2 * w + 1 < n_r ? craw[2 * w + 1] : 0u;
                sm.cid[sl][tid * NDW + w] = lo | (hi << 16);
            }
            if constexpr (SAME) sm.rid[sl][tid] = (int)ridraw;
            sm.lse2[tid] = lraw * LOG2E;
            sm.delta[tid] = draw;
        }
    };

    // Iteration it handles chunk chunk_of(it) in LDS slot it % 2: a look-back
    // chunk first (load only) when the run's first chunk has one, the query
    // chunks k0 .. k1-1, then the chunk after k1-1 when it has k1-1 as its
    // look-back (key side only: its queries against chunk k1-1).  With WRAP the
    // look-back of chunk 0 is the last chunk, and the chunk after the last is 0.
    const bool wraps = WRAP && nchunks > 1;
    const bool lookback = k0 > 0 || wraps;
    const bool extra = k1 < nchunks || wraps;
    const int it0 = lookback ? 1 : 0;
    const int nit = (k1 - k0) + it0 + (extra ? 1 : 0);
    auto chunk_of = [&](int it) {
        const int c = k0 - it0 + it;
        return c < 0 ? c + nchunks : c >= nchunks ? c - nchunks : c;
    };

    // phase-2 ownership: waves 2G, 2G+1 (G = wave / (W/2)) own the chunk in LDS
    // slot G; wave sub-slice sw covers keys KSL*sw .. of that chunk
    const int G = wave / (W / 2), sw = wave % (W / 2);
    f32x4 acck[DT][KTW], accv[DT][KTW];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int kt = 0; kt < KTW; ++kt) { acck[dt][kt] = f32x4{}; accv[dt][kt] = f32x4{}; }

    // write this wave's accumulated key gradients for the chunk in slot G
    auto write_keys = [&]() {
#pragma unroll
        for (int kt = 0; kt < KTW; ++kt) {
            const int krow = KSL * sw + 16 * kt + r16;
            const long pos = sm.pos[G][krow];
#pragma unroll
            for (int e = 0; e < DT / 2; ++e) {
                const int a = 2 * e, b = 2 * e + 1;
                store_tile_pair_bf16(dk_r + rbase + pos * D, g, a,
                                     pack_bf16x2(acck[a][kt][0] * scale, acck[a][kt][1] * scale),
                                     pack_bf16x2(acck[a][kt][2] * scale, acck[a][kt][3] * scale),
                                     pack_bf16x2(acck[b][kt][0] * scale, acck[b][kt][1] * scale),
                                     pack_bf16x2(acck[b][kt][2] * scale, acck[b][kt][3] * scale));
                store_tile_pair_bf16(dv_r + rbase + pos * D, g, a,
                                     pack_bf16x2(accv[a][kt][0], accv[a][kt][1]),
                                     pack_bf16x2(accv[a][kt][2], accv[a][kt][3]),
                                     pack_bf16x2(accv[b][kt][0], accv[b][kt][1]),
                                     pack_bf16x2(accv[b][kt][2], accv[b][kt][3]));
            }
        }
    };

    fetch_positions(chunk_of(0));
    fetch_rows();
    if (1 < nit) fetch_positions(chunk_of(1));

    for (int it = 0; it < nit; ++it) {
        const int c = chunk_of(it);
        const int sl = it & 1, sp = sl ^ 1;
        u32x4 dof[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) dof[ks] = dofrag[ks];
        store_rows(sl);
        __syncthreads();
        if (it + 1 < nit) {
            fetch_rows();
            if (it + 2 < nit) fetch_positions(chunk_of(it + 2));
        }
        if (it < it0) continue;        // look-back chunk: loaded only (next barrier follows the store)

        const bool is_extra = extra && it == nit - 1;
        const bool has_prev = c > 0 || wraps;

        // ---------------- phase 1: queries 16*wave + r16 of chunk c
        {
            const int qrow = wave * 16 + r16;
            const int qpos = sm.pos[sl][qrow];
            typename M::Frag bq[NKS], bd[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                bq[ks] = M::load(&sm.k[sl][KL::off(qrow, ks * KSTEP + g * KPL)]);
                bd[ks] = *reinterpret_cast<const bf16x8*>(&dof[ks]);
            }
            uint32_t q1[NW];
#pragma unroll
            for (int w = 0; w < NDW; ++w) q1[w] = pk_sub_u16(sm.cid[sl][qrow * NDW + w], ones);
            const int rq1 = SAME ? sm.rid[sl][qrow] - 1 : 0;   // query's window id minus one
            const float lse2 = sm.lse2[qrow], dlt = sm.delta[qrow];
            // a query whose windows hold only itself has LSE ~ -penalty: then its
            // self weight is exactly 1/n_r (every round has the same self score);
            // recomputing it from fp32 numbers near 1e5 would lose 2^-7
            const bool self_only = lse2 < -0.5f * SELF_PENALTY * LOG2E;
            const float self_p = 1.f / (float)n_r;

            f32x4 s[NKT], dp[NKT];
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                s[t] = f32x4{};
                dp[t] = f32x4{};
                if (t < CT ? !has_prev : is_extra) continue;
                const int slk = t < CT ? sp : sl;
                const int krow = (t % CT) * 16 + r16;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const int e = ks * KSTEP + g * KPL;
                    s[t] = M::mma(M::load(&sm.k[slk][KL::off(krow, e)]), bq[ks], s[t]);
                    dp[t] = M::mma(M::load(&sm.v[slk][KL::off(krow, e)]), bd[ks], dp[t]);
                }
                if (t & 1) __builtin_amdgcn_sched_barrier(0);
            }
            // P and dS (in place of s and dp)
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                if (t < CT ? !has_prev : is_extra) continue;
                const int slk = t < CT ? sp : sl;
                const bool diag = t == CT + wave;
                const int krow0 = (t % CT) * 16 + 4 * g;
                const int4 kp = *reinterpret_cast<const int4*>(&sm.pos[slk][krow0]);
                int4 kr = {0, 0, 0, 0};
                if constexpr (SAME) kr = *reinterpret_cast<const int4*>(&sm.rid[slk][krow0]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int kpos = j == 0 ? kp.x : j == 1 ? kp.y : j == 2 ? kp.z : kp.w;
                    float nlg = 0.f;
                    if constexpr (NDW > 0) {
                        const uint32_t outs8 = rounds_outside8<NDW, WRAP>(
                            q1, &sm.cid[slk][(krow0 + j) * NDW], nch2);
                        nlg = *reinterpret_cast<const float*>(
                            reinterpret_cast<const char*>(sm.neg_log2) + outs8);
                    }
                    const bool self = diag && kpos == qpos;
                    float p = __builtin_amdgcn_exp2f(fmaf(s[t][j], scale_log2, nlg) - lse2);
                    if (self) p = self_only ? self_p : 0.f;
                    if (causal && kpos > qpos) p = 0.f;
                    if constexpr (SAME) {
                        // another bucket: window ids differ by something other than 0 or 1
                        const int kid = j == 0 ? kr.x : j == 1 ? kr.y : j == 2 ? kr.z : kr.w;
                        if ((unsigned)(kid - rq1) > 1u) p = 0.f;
                    }
                    s[t][j] = p;
                    dp[t][j] = p * (dp[t][j] - dlt);
                }
                if (t & 1) __builtin_amdgcn_sched_barrier(0);
            }
            // P and dS to LDS, [window key][query], two queries per 4-byte store:
            // lanes 2i and 2i+1 (queries qe, qe+1) swap halves with one DPP move;
            // the even lane stores keys 4g+0 and 4g+2 of the pair, the odd lane
            // keys 4g+1 and 4g+3 (rows of both parities in each store: no bank
            // conflicts).
            const bool odd = (r16 & 1) != 0;
            const int qe = qrow & ~1;
            const int qge = qe >> 2, qoe = 2 * (qe & 3);
            auto store_pair = [&](char* base, int t, const f32x4& x) {
                const uint32_t p02 = pack_bf16x2(x[0], x[2]), p13 = pack_bf16x2(x[1], x[3]);
                const uint32_t send = odd ? p02 : p13, own = odd ? p13 : p02;
                const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);
                const uint32_t lo = odd ? recv : own, hi = odd ? own : recv;   // (query qe, qe + 1)
                const uint32_t wa = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                const uint32_t wb = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
                const int ka = t * 16 + 4 * g + (odd ? 1 : 0), kb = ka + 2;
                *reinterpret_cast<uint32_t*>(base + ka * PROWB + 8 * (qge ^ pswz(ka)) + qoe) = wa;
                *reinterpret_cast<uint32_t*>(base + kb * PROWB + 8 * (qge ^ pswz(kb)) + qoe) = wb;
            };
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                if (t < CT ? !has_prev : is_extra) continue;
                store_pair(sm.p, t, s[t]);
                store_pair(sm.ds, t, dp[t]);
            }
            // dQ^T = K^T dS^T (the extra tile's queries belong to the next run)
            if (!is_extra) {
                f32x4 o[DT];
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{};
#pragma unroll
                for (int t0 = 0; t0 < NKT; t0 += 2) {
                    if (t0 < CT && !has_prev) continue;
                    const int slk = t0 < CT ? sp : sl;
                    const int kg = ((t0 % CT) * 16 + 4 * g) >> 2;
                    bf16x8 b;
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        b[x] = (__bf16)dp[t0][x];
                        b[4 + x] = (__bf16)dp[t0 + 1][x];
                    }
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const int d = dt * 16 + r16;
                        const char* kr = sm.kt[slk] + d * TROWB;
                        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kr + vt_group_off<C, D>(kg, d));
                        o[dt] = M::mma(a, b, o[dt]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                T* orow = dq_r + rbase + (long)qpos * D;
#pragma unroll
                for (int e = 0; e < DT / 2; ++e) {
                    const int a = 2 * e, b = 2 * e + 1;
                    store_tile_pair_bf16(orow, g, a,
                                         pack_bf16x2(o[a][0] * scale, o[a][1] * scale),
                                         pack_bf16x2(o[a][2] * scale, o[a][3] * scale),
                                         pack_bf16x2(o[b][0] * scale, o[b][1] * scale),
                                         pack_bf16x2(o[b][2] * scale, o[b][3] * scale));
                }
            }
        }
        __syncthreads();

        // ---------------- phase 2: keys of the chunk in slot G
        {
            const bool cur_role = G == sl;               // slot G holds chunk c, else c - 1
            // the run's first query tile has a look-back that another run owns
            const bool active = cur_role ? !is_extra : (has_prev && it > it0);
            if (cur_role && !is_extra) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int kt = 0; kt < KTW; ++kt) { acck[dt][kt] = f32x4{}; accv[dt][kt] = f32x4{}; }
            }
            if (active) {
                const int wbase = cur_role ? C : 0;      // window rows of this slot's keys
                // queries 16 u0 + 4g + j and 16 (u0 + 1) + 4g + j: the Q^T and dO^T
                // fragments serve both key tiles of this wave
#pragma unroll
                for (int u0 = 0; u0 < CT; u0 += 2) {
                    const int qg = ((u0 * 16) >> 2) + g;
                    bf16x8 bp[KTW], bs[KTW];
#pragma unroll
                    for (int kt = 0; kt < KTW; ++kt) {
                        const int wk = wbase + KSL * sw + 16 * kt + r16;
                        const char* prow = sm.p + wk * PROWB;
                        const char* srow = sm.ds + wk * PROWB;
                        const int psw = pswz(wk);
                        const bf16x4 p0 = *reinterpret_cast<const bf16x4*>(prow + 8 * (qg ^ psw));
                        const bf16x4 p1 = *reinterpret_cast<const bf16x4*>(prow + 8 * ((qg + 4) ^ psw));
                        const bf16x4 s0 = *reinterpret_cast<const bf16x4*>(srow + 8 * (qg ^ psw));
                        const bf16x4 s1 = *reinterpret_cast<const bf16x4*>(srow + 8 * ((qg + 4) ^ psw));
                        bp[kt] = __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7);
                        bs[kt] = __builtin_shufflevector(s0, s1, 0, 1, 2, 3, 4, 5, 6, 7);
                    }
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const int d = dt * 16 + r16;
                        const int go = vt_group_off<C, D>(qg, d);   // groups qg and qg + 4: one pair
                        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(sm.kt[sl] + d * TROWB + go);
                        const bf16x8 ad = *reinterpret_cast<const bf16x8*>(sm.dot + d * TROWB + go);
#pragma unroll
                        for (int kt = 0; kt < KTW; ++kt) {
                            acck[dt][kt] = M::mma(aq, bs[kt], acck[dt][kt]);
                            accv[dt][kt] = M::mma(ad, bp[kt], accv[dt][kt]);
                        }
                        if (dt & 1) __builtin_amdgcn_sched_barrier(0);
                    }
                }
                if (!cur_role) write_keys();             // chunk c - 1 is complete
            }
        }
        __syncthreads();
    }
    // the run's last chunk is nobody's look-back: its keys are complete
    if (!extra && G == ((nit - 1) & 1)) write_keys();
}

// ---------------------------------------------------------------------------
// The method's backward split over two kernels that each leave room for two
// workgroups per CU (the fused k_attn_bwd above needs 150 KB of LDS and about
// 512 registers per lane: one workgroup, one wave per SIMD).  Both write the
// same per-round partials as the fused kernel, in the same order of
// accumulation (bit-identical results), and read LSE and Delta from k_bwd_prep.

typedef short i16x4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x4 tr4(const bf16_t* p)
{
    const i16x4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4s*)p);
    return __builtin_bit_cast(bf16x4, r);
}

// A operand (16 d x 32 rows of a row-major LDS table, k-slot x < 4: row R0 + x,
// x >= 4: row R1 + x - 4) for MFMA 16x16x32: two transposing reads.  Lane
// 4k + q of each 16-lane group addresses row R + k, columns c0 + 4q .. +3.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const bf16_t* tab, int R0, int R1, int c0, int lane)
{
    using KL = KLayout<bf16_t, D>;
    const int k = (lane & 15) >> 2, q = lane & 3;
    const bf16x4 a0 = tr4(tab + KL::off(R0 + k, c0 + 4 * q));
    const bf16x4 a1 = tr4(tab + KL::off(R1 + k, c0 + 4 * q));
    return __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int D, int NDW>
struct BwdQLds {
    static constexpr int C = 64;
    static constexpr int KROW = KLayout<bf16_t, D>::ROW;
    static constexpr int NW = NDW > 0 ? NDW : 1;
    float neg_log2[36];
    bf16_t k[2][C * KROW];
    bf16_t v[2][C * KROW];
    int pos[2][C];
    uint32_t cid[2][C * NW];
    float lse2[2][C];
    float delta[2][C];
};

// Query role (k_bwd_q): the run structure of the forward (the chunk's qk and v
// rows gathered once into LDS and kept as the next chunk's look-back; the next
// chunk's rows and this wave's d_o fragments held in registers meanwhile).  Per
// query chunk: S^T = K Q^T and dP^T = V dO^T as the forward's scores, P and dS
// in registers (LSE and Delta are inputs, so no reduction over keys), and
// dQ^T = K^T dS^T with K^T read from the row-major qk rows by transposing LDS
// reads instead of a transposed copy, which keeps the LDS at 68 KiB (two
// workgroups per CU).
template <int D, int NDW>
__global__ __launch_bounds__(256, 2)
void k_bwd_q(const bf16_t* __restrict__ qk, const bf16_t* __restrict__ v, const bf16_t* __restrict__ d_o,
             const int32_t* __restrict__ perm, const int16_t* __restrict__ cid,
             const float* __restrict__ lse_c, const float* __restrict__ delta, bf16_t* __restrict__ dq_r,
             int L, int n_r, int causal, float scale, float scale_log2, int nruns, int run_len)
{
    using T = bf16_t;
    using M = Mfma16<T>;
    using S = BwdQLds<D, NDW>;
    using KL = KLayout<T, D>;
    constexpr int C = 64, NTH = 256, CT = 4, NKT = 8, DT = D / 16;
    constexpr int KPL = M::KPL, KSTEP = M::KSTEP, NKS = D / KSTEP;
    constexpr int VE = 8, VPR = D / VE;
    constexpr int JOBS = (C / 4) * VPR;
    constexpr int JPT = (JOBS + NTH - 1) / NTH;
    constexpr int NW = S::NW;
    __shared__ __attribute__((aligned(16))) S sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    int bid = blockIdx.x;
    const int r = bid % n_r;
    bid /= n_r;
    const int run = bid % nruns;
    const long bh = bid / nruns;
    const int nchunks = L / C;
    const int k0 = run * run_len, k1 = min(k0 + run_len, nchunks);

    const T* qb = qk + bh * (long)L * D;
    const T* vb = v + bh * (long)L * D;
    const T* db = d_o + bh * (long)L * D;
    const int32_t* pr = perm + (bh * n_r + r) * (long)L;
    const int16_t* cb = cid + bh * (long)L * n_r;
    const float* lb = lse_c + bh * (long)L;
    const float* deb = delta + bh * (long)L;
    T* ob = dq_r + (bh * n_r + r) * (long)L * D;
    const uint32_t ones = 0x00010001u;
    const uint32_t nch2 = (uint32_t)nchunks * 0x00010001u;
    if (tid < 33) sm.neg_log2[tid] = (tid % 2 == 0 && tid / 2 < n_r) ? -__log2f((float)(n_r - tid / 2)) : 0.f;
    auto clamp_pos = [&](int p) {
        LSH_CHECK((unsigned)p < (unsigned)L);
        return min(max(p, 0), L - 1);
    };

    int gpos[JPT][4];
    u32x4 kreg[JPT][4], vreg[JPT][4];
    int mypos = 0, qposraw = 0, rpos = 0;
    u32x4 dofrag[NKS];
    uint32_t craw[2 * NW];
    float lraw = 0.f, draw = 0.f;

    auto fetch_positions = [&](int kk) {
#pragma unroll
        for (int jb = 0; jb < JPT; ++jb) {
            const int job = tid + jb * NTH;
            const int rg = (job < JOBS ? job : 0) / VPR;
#pragma unroll
            for (int i = 0; i < 4; ++i) gpos[jb][i] = pr[kk * C + 4 * rg + i];
        }
        mypos = pr[kk * C + tid % C];
        qposraw = pr[kk * C + wave * 16 + r16];
    };
    auto fetch_rows = [&]() {
#pragma unroll
        for (int jb = 0; jb < JPT; ++jb) {
            const int job = tid + jb * NTH;
            const int piece = (job < JOBS ? job : 0) % VPR;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const long row = (long)clamp_pos(gpos[jb][i]) * D + piece * VE;
                kreg[jb][i] = *reinterpret_cast<const u32x4*>(qb + row);
                vreg[jb][i] = *reinterpret_cast<const u32x4*>(vb + row);
            }
        }
        const long qrow = (long)clamp_pos(qposraw) * D;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            dofrag[ks] = *reinterpret_cast<const u32x4*>(db + qrow + ks * KSTEP + g * KPL);
        rpos = clamp_pos(mypos);
        const int16_t* cr = cb + (long)rpos * n_r;
        if constexpr (NDW > 0) {
#pragma unroll
            for (int h = 0; h < 2 * NDW; ++h) craw[h] = (uint16_t)cr[min(h, n_r - 1)];
        }
        lraw = lb[rpos];
        draw = deb[rpos];
    };
    auto store_rows = [&](int sl) {
#pragma unroll
        for (int jb = 0; jb < JPT; ++jb) {
            const int job = tid + jb * NTH;
            if (job < JOBS) {
                const int rg = job / VPR, piece = job % VPR;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    *reinterpret_cast<u32x4*>(&sm.k[sl][KL::off(4 * rg + i, piece * VE)]) = kreg[jb][i];
                    *reinterpret_cast<u32x4*>(&sm.v[sl][KL::off(4 * rg + i, piece * VE)]) = vreg[jb][i];
                }
            }
        }
        if (tid < C) {
            sm.pos[sl][tid] = rpos;
#pragma unroll
            for (int w = 0; w < NDW; ++w) {
                const uint32_t lo = 2 * w < n_r ? craw[2 * w] : 0u;
                const uint32_t hi = 2 * w + 1 < n_r ? craw[2 * w + 1] : 0u;
                sm.cid[sl][tid * NDW + w] = lo | (hi << 16);
            }
            sm.lse2[sl][tid] = lraw * LOG2E;
            sm.delta[sl][tid] = draw;
        }
    };

    const bool lookback = k0 > 0;
    const int it0 = lookback ? 1 : 0;
    const int nit = (k1 - k0) + it0;
    auto chunk_of = [&](int it) { return k0 - it0 + it; };

    fetch_positions(chunk_of(0));
    fetch_rows();
    if (1 < nit) fetch_positions(chunk_of(1));

    for (int it = 0; it < nit; ++it) {
        const int c = chunk_of(it);
        const int sl = it & 1, sp = sl ^ 1;
        u32x4 dof[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) dof[ks] = dofrag[ks];
        store_rows(sl);
        __syncthreads();
        if (it + 1 < nit) {
            fetch_rows();
            if (it + 2 < nit) fetch_positions(chunk_of(it + 2));
        }
        if (it >= it0) {
            const bool has_prev = c > 0;
            const int qrow = wave * 16 + r16;
            const int qpos = sm.pos[sl][qrow];
            typename M::Frag bq[NKS], bd[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                bq[ks] = M::load(&sm.k[sl][KL::off(qrow, ks * KSTEP + g * KPL)]);
                bd[ks] = *reinterpret_cast<const bf16x8*>(&dof[ks]);
            }
            uint32_t q1[NW];
#pragma unroll
            for (int w = 0; w < NDW; ++w) q1[w] = pk_sub_u16(sm.cid[sl][qrow * NDW + w], ones);
            const float lse2 = sm.lse2[sl][qrow], dlt = sm.delta[sl][qrow];
            const bool self_only = lse2 < -0.5f * SELF_PENALTY * LOG2E;
            const float self_p = 1.f / (float)n_r;

            f32x4 s[NKT], dp[NKT];
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                s[t] = f32x4{};
                dp[t] = f32x4{};
                if (t < CT && !has_prev) continue;
                const int slk = t < CT ? sp : sl;
                const int krow = (t % CT) * 16 + r16;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const int e = ks * KSTEP + g * KPL;
                    s[t] = M::mma(M::load(&sm.k[slk][KL::off(krow, e)]), bq[ks], s[t]);
                    dp[t] = M::mma(M::load(&sm.v[slk][KL::off(krow, e)]), bd[ks], dp[t]);
                }
                if (t & 1) __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                if (t < CT && !has_prev) continue;
                const int slk = t < CT ? sp : sl;
                const bool diag = t == CT + wave;
                const int krow0 = (t % CT) * 16 + 4 * g;
                const int4 kp = *reinterpret_cast<const int4*>(&sm.pos[slk][krow0]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int kpos = j == 0 ? kp.x : j == 1 ? kp.y : j == 2 ? kp.z : kp.w;
                    float nlg = 0.f;
                    if constexpr (NDW > 0) {
                        const uint32_t outs8 = rounds_outside8<NDW, false>(q1, &sm.cid[slk][(krow0 + j) * NDW], nch2);
                        nlg = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(sm.neg_log2) + outs8);
                    }
                    float p = __builtin_amdgcn_exp2f(fmaf(s[t][j], scale_log2, nlg) - lse2);
                    if (diag && kpos == qpos) p = self_only ? self_p : 0.f;
                    if (causal && kpos > qpos) p = 0.f;
                    dp[t][j] = p * (dp[t][j] - dlt);
                }
                if (t & 1) __builtin_amdgcn_sched_barrier(0);
            }
            f32x4 o[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{};
#pragma unroll
            for (int t0 = 0; t0 < NKT; t0 += 2) {
                if (t0 < CT && !has_prev) continue;
                const int slk = t0 < CT ? sp : sl;
                bf16x8 b;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    b[x] = (__bf16)dp[t0][x];
                    b[4 + x] = (__bf16)dp[t0 + 1][x];
                }
                const int R0 = (t0 % CT) * 16 + 4 * g, R1 = ((t0 + 1) % CT) * 16 + 4 * g;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    o[dt] = M::mma(tr_operand<D>(sm.k[slk], R0, R1, 16 * dt, lane), b, o[dt]);
                __builtin_amdgcn_sched_barrier(0);
            }
            T* orow = ob + (long)qpos * D;
#pragma unroll
            for (int e = 0; e < DT / 2; ++e) {
                const int a = 2 * e, b = 2 * e + 1;
                store_tile_pair_bf16(orow, g, a,
                                     pack_bf16x2(o[a][0] * scale, o[a][1] * scale),
                                     pack_bf16x2(o[a][2] * scale, o[a][3] * scale),
                                     pack_bf16x2(o[b][0] * scale, o[b][1] * scale),
                                     pack_bf16x2(o[b][2] * scale, o[b][3] * scale));
            }
        }
        __syncthreads();
    }
}

template <int D, int NDW>
struct BwdKLds {
    static constexpr int C = 64;
    static constexpr int KROW = KLayout<bf16_t, D>::ROW;
    static constexpr int NW = NDW > 0 ? NDW : 1;
    float neg_log2[36];
    bf16_t q[C * KROW];              // qk rows of the chunk (queries; and the keys of phase B)
    bf16_t dO[C * KROW];             // d_o rows of the chunk
    bf16_t v[C * KROW];              // v rows of the chunk (keys of phase B)
    int pos[C];
    uint32_t cid[C * NW];            // chunk ids (packed, raw): the keys' words
    uint32_t q1[C * NW];             // chunk ids minus one: the queries' words
    float lse2[C];
    float delta[C];
};

// Key role (k_bwd_k): a workgroup owns a run of key chunks [k0, k1); iteration
// q holds query chunk q in LDS (qk, d_o and v rows, one slot).  Phase A: the
// keys of chunk q - 1 (operands in registers since iteration q - 1) against the
// queries of chunk q, which completes them; phase B: the keys of chunk q against
// the queries of chunk q.  Wave w owns keys 16 w .. 16 w + 15.  S = Q K^T and
// dP = dO V^T put the queries on the row axis, so P and dS are in the B-operand
// layout of dK^T += Q^T dS and dV^T += dO^T P, whose A operands are read from
// the row-major qk and d_o rows with transposing LDS reads.  A chunk's rows are
// gathered at the top of its iteration: with the next chunk's rows held in
// registers (as in the query role) the kernel spilled 39 registers and took
// 2.2 ms at paper_64k against 1.6 ms; the second workgroup on the CU covers the
// gather instead.
template <int D, int NDW>
__global__ __launch_bounds__(256, 2)
void k_bwd_k(const bf16_t* __restrict__ qk, const bf16_t* __restrict__ v, const bf16_t* __restrict__ d_o,
             const int32_t* __restrict__ perm, const int16_t* __restrict__ cid,
             const float* __restrict__ lse_c, const float* __restrict__ delta, bf16_t* __restrict__ dk_r,
             bf16_t* __restrict__ dv_r, int L, int n_r, int causal, float scale, float scale_log2, int nruns,
             int run_len)
{
    using T = bf16_t;
    using M = Mfma16<T>;
    using S = BwdKLds<D, NDW>;
    using KL = KLayout<T, D>;
    constexpr int C = 64, NTH = 256, CT = 4, DT = D / 16;
    constexpr int KPL = M::KPL, KSTEP = M::KSTEP, NKS = D / KSTEP;
    constexpr int VE = 8, VPR = D / VE;
    constexpr int JOBS = (C / 4) * VPR;
    constexpr int JPT = (JOBS + NTH - 1) / NTH;
    constexpr int NW = S::NW;
    __shared__ __attribute__((aligned(16))) S sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    int bid = blockIdx.x;
    const int r = bid % n_r;
    bid /= n_r;
    const int run = bid % nruns;
    const long bh = bid / nruns;
    const int nchunks = L / C;
    const int k0 = run * run_len, k1 = min(k0 + run_len, nchunks);

    const T* qb = qk + bh * (long)L * D;
    const T* vb = v + bh * (long)L * D;
    const T* db = d_o + bh * (long)L * D;
    const int32_t* pr = perm + (bh * n_r + r) * (long)L;
    const int16_t* cb = cid + bh * (long)L * n_r;
    const float* lb = lse_c + bh * (long)L;
    const float* deb = delta + bh * (long)L;
    const long rbase = (bh * n_r + r) * (long)L * D;
    const uint32_t ones = 0x00010001u;
    const uint32_t nch2 = (uint32_t)nchunks * 0x00010001u;
    if (tid < 33) sm.neg_log2[tid] = (tid % 2 == 0 && tid / 2 < n_r) ? -__log2f((float)(n_r - tid / 2)) : 0.f;
    auto clamp_pos = [&](int p) {
        LSH_CHECK((unsigned)p < (unsigned)L);
        return min(max(p, 0), L - 1);
    };

    int gpos[JPT][4];
    u32x4 qreg[JPT][4], dreg[JPT][4], vreg[JPT][4];
    int mypos = 0, rpos = 0;
    uint32_t craw[2 * NW];
    float lraw = 0.f, draw = 0.f;

    auto fetch_positions = [&](int kk) {
#pragma unroll
        for (int jb = 0; jb < JPT; ++jb) {
            const int job = tid + jb * NTH;
            const int rg = (job < JOBS ? job : 0) / VPR;
#pragma unroll
            for (int i = 0; i < 4; ++i) gpos[jb][i] = pr[kk * C + 4 * rg + i];
        }
        mypos = pr[kk * C + tid % C];
    };
    auto fetch_rows = [&]() {
#pragma unroll
        for (int jb = 0; jb < JPT; ++jb) {
            const int job = tid + jb * NTH;
            const int piece = (job < JOBS ? job : 0) % VPR;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const long row = (long)clamp_pos(gpos[jb][i]) * D + piece * VE;
                qreg[jb][i] = *reinterpret_cast<const u32x4*>(qb + row);
                dreg[jb][i] = *reinterpret_cast<const u32x4*>(db + row);
                vreg[jb][i] = *reinterpret_cast<const u32x4*>(vb + row);
            }
        }
        rpos = clamp_pos(mypos);
        const int16_t* cr = cb + (long)rpos * n_r;
        if constexpr (NDW > 0) {
#pragma unroll
            for (int h = 0; h < 2 * NDW; ++h) craw[h] = (uint16_t)cr[min(h, n_r - 1)];
        }
        lraw = lb[rpos];
        draw = deb[rpos];
    };
    auto store_rows = [&]() {
#pragma unroll
        for (int jb = 0; jb < JPT; ++jb) {
            const int job = tid + jb * NTH;
            if (job < JOBS) {
                const int rg = job / VPR, piece = job % VPR;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int o = KL::off(4 * rg + i, piece * VE);
                    *reinterpret_cast<u32x4*>(&sm.q[o]) = qreg[jb][i];
                    *reinterpret_cast<u32x4*>(&sm.dO[o]) = dreg[jb][i];
                    *reinterpret_cast<u32x4*>(&sm.v[o]) = vreg[jb][i];
                }
            }
        }
        if (tid < C) {
            sm.pos[tid] = rpos;
#pragma unroll
            for (int w = 0; w < NDW; ++w) {
                const uint32_t lo = 2 * w < n_r ? craw[2 * w] : 0u;
                const uint32_t hi = 2 * w + 1 < n_r ? craw[2 * w + 1] : 0u;
                const uint32_t word = lo | (hi << 16);
                sm.cid[tid * NDW + w] = word;
                sm.q1[tid * NDW + w] = pk_sub_u16(word, ones);
            }
            sm.lse2[tid] = lraw * LOG2E;
            sm.delta[tid] = draw;
        }
    };

    // this wave's keys (registers): B operands of K and V rows, position, chunk-id words
    typename M::Frag bk[NKS], bvf[NKS];
    int kpos = 0;
    uint32_t kw[NW];
    f32x4 acck[DT], accv[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) { acck[dt] = f32x4{}; accv[dt] = f32x4{}; }

    auto load_keys = [&]() {
        const int krow = wave * 16 + r16;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            bk[ks] = M::load(&sm.q[KL::off(krow, ks * KSTEP + g * KPL)]);
            bvf[ks] = M::load(&sm.v[KL::off(krow, ks * KSTEP + g * KPL)]);
        }
        kpos = sm.pos[krow];
#pragma unroll
        for (int w = 0; w < NDW; ++w) kw[w] = sm.cid[krow * NDW + w];
    };
    // the keys of this wave against the queries in LDS; diag: the keys are the
    // chunk's own rows (the self pair lies in query tile `wave`)
    auto accumulate = [&](bool same_chunk) {
        const float self_p = 1.f / (float)n_r;
        // query tiles in two halves (u0, u0 + 1): S, dP, then dK^T, dV^T
#pragma unroll
        for (int u0 = 0; u0 < CT; u0 += 2) {
            f32x4 s[2], dp[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                s[h] = f32x4{};
                dp[h] = f32x4{};
                const int qrow = (u0 + h) * 16 + r16;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const int e = ks * KSTEP + g * KPL;
                    s[h] = M::mma(M::load(&sm.q[KL::off(qrow, e)]), bk[ks], s[h]);
                    dp[h] = M::mma(M::load(&sm.dO[KL::off(qrow, e)]), bvf[ks], dp[h]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int u = u0 + h;
                const int q0 = u * 16 + 4 * g;
                const int4 qp = *reinterpret_cast<const int4*>(&sm.pos[q0]);
                const float4 l2 = *reinterpret_cast<const float4*>(&sm.lse2[q0]);
                const float4 de = *reinterpret_cast<const float4*>(&sm.delta[q0]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int qpos = j == 0 ? qp.x : j == 1 ? qp.y : j == 2 ? qp.z : qp.w;
                    const float lse2 = j == 0 ? l2.x : j == 1 ? l2.y : j == 2 ? l2.z : l2.w;
                    const float dlt = j == 0 ? de.x : j == 1 ? de.y : j == 2 ? de.z : de.w;
                    float nlg = 0.f;
                    if constexpr (NDW > 0) {
                        uint32_t qw[NW];
#pragma unroll
                        for (int w = 0; w < NDW; ++w) qw[w] = sm.q1[(q0 + j) * NDW + w];
                        const uint32_t outs8 = rounds_outside8<NDW, false>(qw, kw, nch2);
                        nlg = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(sm.neg_log2) + outs8);
                    }
                    float p = __builtin_amdgcn_exp2f(fmaf(s[h][j], scale_log2, nlg) - lse2);
                    if (same_chunk && u == wave && kpos == qpos)
                        p = lse2 < -0.5f * SELF_PENALTY * LOG2E ? self_p : 0.f;
                    if (causal && kpos > qpos) p = 0.f;
                    s[h][j] = p;
                    dp[h][j] = p * (dp[h][j] - dlt);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            bf16x8 bp, bs;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                bp[x] = (__bf16)s[0][x];
                bp[4 + x] = (__bf16)s[1][x];
                bs[x] = (__bf16)dp[0][x];
                bs[4 + x] = (__bf16)dp[1][x];
            }
            const int R0 = u0 * 16 + 4 * g, R1 = (u0 + 1) * 16 + 4 * g;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                acck[dt] = M::mma(tr_operand<D>(sm.q, R0, R1, 16 * dt, lane), bs, acck[dt]);
                accv[dt] = M::mma(tr_operand<D>(sm.dO, R0, R1, 16 * dt, lane), bp, accv[dt]);
                if (dt & 1) __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    auto write_keys = [&]() {
        // lane (r16, g): key 16 w + r16, d = 16 dt + 4 g + j
#pragma unroll
        for (int e = 0; e < DT / 2; ++e) {
            const int a = 2 * e, b = 2 * e + 1;
            store_tile_pair_bf16(dk_r + rbase + (long)kpos * D, g, a,
                                 pack_bf16x2(acck[a][0] * scale, acck[a][1] * scale),
                                 pack_bf16x2(acck[a][2] * scale, acck[a][3] * scale),
                                 pack_bf16x2(acck[b][0] * scale, acck[b][1] * scale),
                                 pack_bf16x2(acck[b][2] * scale, acck[b][3] * scale));
            store_tile_pair_bf16(dv_r + rbase + (long)kpos * D, g, a,
                                 pack_bf16x2(accv[a][0], accv[a][1]), pack_bf16x2(accv[a][2], accv[a][3]),
                                 pack_bf16x2(accv[b][0], accv[b][1]), pack_bf16x2(accv[b][2], accv[b][3]));
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            acck[dt] = f32x4{};
            accv[dt] = f32x4{};
        }
    };

    const bool extra = k1 < nchunks;
    const int nit = (k1 - k0) + (extra ? 1 : 0);
    fetch_positions(k0);
    for (int it = 0; it < nit; ++it) {
        fetch_rows();                       // this chunk's rows (positions fetched an iteration ahead)
        store_rows();
        __syncthreads();
        if (it + 1 < nit) fetch_positions(k0 + it + 1);
        if (it > 0) {                       // phase A: the keys of chunk k0 + it - 1, completed
            accumulate(false);
            write_keys();
        }
        if (it < k1 - k0) {                 // phase B: the keys of chunk k0 + it
            load_keys();
            accumulate(true);
        }
        __syncthreads();
    }
    if (!extra) write_keys();               // the run's last chunk has no next chunk
}

// LSE_i = logsumexp_r lse[r, i]; Delta_i = <d_o_i, o_i>.  One thread per 16 bytes
// of a row (TPR threads per row, reduced by shuffles within the row's lanes).
template <int D>
__global__ __launch_bounds__(256)
void k_bwd_prep(const bf16_t* __restrict__ o, const bf16_t* __restrict__ d_o,
                const float* __restrict__ lse, float* __restrict__ lse_c,
                float* __restrict__ delta, long rows, int L, int n_r)
{
    // TPR threads per row, 16 bytes of o and d_o each; PREP_RPT rows per thread
    // (strided by the block's RPB rows), their loads all issued first
    constexpr int TPR = D / 8, RPB = 256 / TPR;
    const int part = threadIdx.x % TPR;
    const long row0 = (long)blockIdx.x * RPB * PREP_RPT + threadIdx.x / TPR;
    u32x4 a[PREP_RPT], b[PREP_RPT];
#pragma unroll
    for (int k = 0; k < PREP_RPT; ++k) {
        const long rr = min(row0 + (long)k * RPB, rows - 1);
        a[k] = *reinterpret_cast<const u32x4*>(o + rr * D + part * 8);
        b[k] = *reinterpret_cast<const u32x4*>(d_o + rr * D + part * 8);
    }
#pragma unroll
    for (int k = 0; k < PREP_RPT; ++k) {
        const long row = row0 + (long)k * RPB;
        const long rr = min(row, rows - 1);
        float acc = 0.f;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            acc = fmaf(bf16_to_f32((uint16_t)(a[k][x] & 0xFFFFu)), bf16_to_f32((uint16_t)(b[k][x] & 0xFFFFu)), acc);
            acc = fmaf(bf16_to_f32((uint16_t)(a[k][x] >> 16)), bf16_to_f32((uint16_t)(b[k][x] >> 16)), acc);
        }
        // LSE over the rounds: the row's lanes take rounds part, part + TPR, ..
        const long bh = rr / L;
        const int i = (int)(rr % L);
        float m = -INFINITY;
        for (int q = part; q < n_r; q += TPR) m = fmaxf(m, lse[(bh * n_r + q) * (long)L + i]);
#pragma unroll
        for (int s = 1; s < TPR; s <<= 1) {
            acc += __shfl_xor(acc, s);
            m = fmaxf(m, __shfl_xor(m, s));
        }
        float z = 0.f;
        for (int q = part; q < n_r; q += TPR) z += __expf(lse[(bh * n_r + q) * (long)L + i] - m);
#pragma unroll
        for (int s = 1; s < TPR; s <<= 1) z += __shfl_xor(z, s);
        if (row < rows && part == 0) {
            lse_c[row] = m + __logf(z);
            delta[row] = acc;
        }
    }
}

// dqk = sum_r (dq_r + dk_r), dv = sum_r dv_r (fp32).  One thread per 8 elements:
// 4 in each half of the row (elements 4p .. 4p+3 and D/2 + 4p .. +3), so that
// each load instruction reads, and each store instruction writes, contiguous
// whole lines of a row (128 and 256 bytes at d 128) rather than 16 bytes at a
// 32-byte stride.  The sums per element are the same.
template <int D>
__global__ __launch_bounds__(256)
void k_bwd_reduce(const bf16_t* __restrict__ dq_r, const bf16_t* __restrict__ dk_r,
                  const bf16_t* __restrict__ dv_r, float* __restrict__ dqk, float* __restrict__ dv,
                  long rows, int L, int n_r)
{
    constexpr int TPR = D / 8, RPB = 256 / TPR, HALF = D / 2;
    const long row = (long)blockIdx.x * RPB + threadIdx.x / TPR;
    const int part = threadIdx.x % TPR;
    if (row >= rows) return;
    const long bh = row / L;
    const int i = (int)(row % L);
    float aq[8], av[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) { aq[x] = 0.f; av[x] = 0.f; }
    for (int q = 0; q < n_r; ++q) {
        const long off = ((bh * n_r + q) * (long)L + i) * D + part * 4;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x2 a = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(dq_r + off + h * HALF));
            const u32x2 b = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(dk_r + off + h * HALF));
            const u32x2 c = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(dv_r + off + h * HALF));
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                aq[4 * h + 2 * x] += bf16_to_f32((uint16_t)(a[x] & 0xFFFFu)) + bf16_to_f32((uint16_t)(b[x] & 0xFFFFu));
                aq[4 * h + 2 * x + 1] += bf16_to_f32((uint16_t)(a[x] >> 16)) + bf16_to_f32((uint16_t)(b[x] >> 16));
                av[4 * h + 2 * x] += bf16_to_f32((uint16_t)(c[x] & 0xFFFFu));
                av[4 * h + 2 * x + 1] += bf16_to_f32((uint16_t)(c[x] >> 16));
            }
        }
    }
    float* oq = dqk + row * D + part * 4;
    float* ov = dv + row * D + part * 4;
    __builtin_nontemporal_store(f32x4{aq[0], aq[1], aq[2], aq[3]}, reinterpret_cast<f32x4*>(oq));
    __builtin_nontemporal_store(f32x4{aq[4], aq[5], aq[6], aq[7]}, reinterpret_cast<f32x4*>(oq + HALF));
    __builtin_nontemporal_store(f32x4{av[0], av[1], av[2], av[3]}, reinterpret_cast<f32x4*>(ov));
    __builtin_nontemporal_store(f32x4{av[4], av[5], av[6], av[7]}, reinterpret_cast<f32x4*>(ov + HALF));
}

template <int D, int C, int NDW, bool WRAP, bool SAME>
hipError_t launch_bwd_one(const BwdArgs& a, hipStream_t s)
{
    const int nchunks = a.L / C;
    const int run_len = run_length(nchunks, a.bh * a.n_r);     // as the forward's runs
    const int nruns = (nchunks + run_len - 1) / run_len;
    const long blocks = a.bh * nruns * a.n_r;
    hipLaunchKernelGGL((k_attn_bwd<D, C, NDW, WRAP, SAME>), dim3((unsigned)blocks), dim3(4 * C), 0, s,
                       static_cast<const bf16_t*>(a.qk), static_cast<const bf16_t*>(a.v),
                       static_cast<const bf16_t*>(a.d_o), a.perm, a.cid, a.lse_c, a.delta,
                       static_cast<bf16_t*>(a.dq_r), static_cast<bf16_t*>(a.dk_r),
                       static_cast<bf16_t*>(a.dv_r), a.L, a.n_r, a.causal, a.scale,
                       a.scale * LOG2E, nruns, run_len);
    return hipGetLastError();
}

// The split kernels (query role, then key role), one workgroup per (b, h,
// round, run of chunks), runs fitted to the workgroups the GPU holds at once.
template <int D, int NDW>
hipError_t launch_bwd_split(const BwdArgs& a, hipStream_t s)
{
    static const int per_cu_q = [] {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, (const void*)k_bwd_q<D, NDW>, 256, 0) != hipSuccess || b < 1)
            b = 1;
        return b;
    }();
    static const int per_cu_k = [] {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, (const void*)k_bwd_k<D, NDW>, 256, 0) != hipSuccess || b < 1)
            b = 1;
        return b;
    }();
    const int nchunks = a.L / 64;
    const long segs = a.bh * a.n_r;
    const int rlq = run_length_fit(nchunks, segs, (long)per_cu_q * device_cus());
    const int nrq = (nchunks + rlq - 1) / rlq;
    hipLaunchKernelGGL((k_bwd_q<D, NDW>), dim3((unsigned)(segs * nrq)), dim3(256), 0, s,
                       static_cast<const bf16_t*>(a.qk), static_cast<const bf16_t*>(a.v),
                       static_cast<const bf16_t*>(a.d_o), a.perm, a.cid, a.lse_c, a.delta,
                       static_cast<bf16_t*>(a.dq_r), a.L, a.n_r, a.causal, a.scale, a.scale * LOG2E, nrq, rlq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int rlk = run_length_fit(nchunks, segs, (long)per_cu_k * device_cus());
    const int nrk = (nchunks + rlk - 1) / rlk;
    hipLaunchKernelGGL((k_bwd_k<D, NDW>), dim3((unsigned)(segs * nrk)), dim3(256), 0, s,
                       static_cast<const bf16_t*>(a.qk), static_cast<const bf16_t*>(a.v),
                       static_cast<const bf16_t*>(a.d_o), a.perm, a.cid, a.lse_c, a.delta,
                       static_cast<bf16_t*>(a.dk_r), static_cast<bf16_t*>(a.dv_r), a.L, a.n_r, a.causal,
                       a.scale, a.scale * LOG2E, nrk, rlk);
    return hipGetLastError();
}

// The method (with or without the duplicate-count term) takes the split
// kernels; wrap-around look-back and same-bucket windows the fused kernel.
template <int D, bool WRAP, bool SAME>
hipError_t launch_bwd_ndw(const BwdArgs& a, hipStream_t s)
{
    if constexpr (!WRAP && !SAME) {
        if (!a.dup) return launch_bwd_split<D, 0>(a, s);
        if (a.n_r <= 2) return launch_bwd_split<D, 1>(a, s);
        if (a.n_r <= 4) return launch_bwd_split<D, 2>(a, s);
        if (a.n_r <= 8) return launch_bwd_split<D, 4>(a, s);
        return launch_bwd_split<D, 8>(a, s);
    } else {
        if (!a.dup) return launch_bwd_one<D, 64, 0, WRAP, SAME>(a, s);
        if (a.n_r <= 2) return launch_bwd_one<D, 64, 1, WRAP, SAME>(a, s);
        if (a.n_r <= 4) return launch_bwd_one<D, 64, 2, WRAP, SAME>(a, s);
        if (a.n_r <= 8) return launch_bwd_one<D, 64, 4, WRAP, SAME>(a, s);
        return launch_bwd_one<D, 64, 8, WRAP, SAME>(a, s);
    }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t s)
{
    const long rows = a.bh * a.L;
    constexpr int RPB = 256 / (D / 8);               // rows per 256-thread block
    const unsigned blocks = (unsigned)((rows + RPB - 1) / RPB);
    const unsigned pblocks = (unsigned)((rows + RPB * PREP_RPT - 1) / (RPB * PREP_RPT));
    hipLaunchKernelGGL((k_bwd_prep<D>), dim3(pblocks), dim3(256), 0, s,
                       static_cast<const bf16_t*>(a.o), static_cast<const bf16_t*>(a.d_o), a.lse,
                       a.lse_c, a.delta, rows, a.L, a.n_r);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.same_bucket) e = launch_bwd_ndw<D, false, true>(a, s);
    else if (a.wrap) e = launch_bwd_ndw<D, true, false>(a, s);
    else e = launch_bwd_ndw<D, false, false>(a, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_bwd_reduce<D>), dim3(blocks), dim3(256), 0, s,
                       static_cast<const bf16_t*>(a.dq_r), static_cast<const bf16_t*>(a.dk_r),
                       static_cast<const bf16_t*>(a.dv_r), a.dqk, a.dv, rows, a.L, a.n_r);
    return hipGetLastError();
}

}  // namespace
}  // namespace attn

LSH_CHECK_ACCESSOR(check_count_attn_bwd)

hipError_t launch_attn_backward(int d_head, const BwdArgs& a, hipStream_t stream)
{
    return d_head == 64 ? attn::launch_bwd_d<64>(a, stream) : attn::launch_bwd_d<128>(a, stream);
}

}  // namespace lshk
