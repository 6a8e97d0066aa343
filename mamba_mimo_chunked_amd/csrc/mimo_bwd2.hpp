// Stage-2 backward of the Mamba-3 MIMO scan (mamba3_mimo_bwd_bwd; Triton-Ascend
// pull request page: "practice" document -- cache semantics, the dstates
// recurrence, the gradient groups -- and the migration note's input/output
// table). With dPhiO the upstream gradient mapped to ranks (dout * mimo_o, or
// the per-rank dout), L = sum dPhiO * y, and per chunk c (rows i = (r, t),
// rank-major i = r*C + t, Q^/K^ rotated, K~ = K^ * factor_t, Psi = v * mimo_v,
// S_c the cached entry state, E[t][s] = exp(segsum[c][t][s]) for s < t):
//   dS_c      = exp(da_cs[last]) dS_{c+1} + Q^^T (exp(da_cs) dPhiO)      (dS_nc = 0)
//   dP        = dPhiO Psi^T,  A = E (Q^ K~^T),  W = E dP                 (token-masked)
//   dQ^       = exp(da_cs) dPhiO S_c^T + W K~       (+ same-token part, below)
//   dK~       = W^T Q^ + exp(da_cs_rev) Psi dS_{c+1}^T
//   dPsi      = A^T dPhiO + kappa dS_{c+1} + gamma (qk^T dPhiO)_same-token + d dPhiO
//   dqk[t]    = gamma_t dPhiO[t] Psi[t]^T  -> dq0 += dqk k0, dk0 += dqk^T q0, applied in
//               the rotated frame (the rotation is the same for q and k of a token)
// and the per-token partials DDA_CS, DDA_CS_REV, DFACTOR, DGAMMA, DDA, DSSDA and
// DANGLES from the same products. Everything is fp32 on small LDS-resident
// tiles (R*C, N, P <= 64); every contraction runs on fp32 MFMA.
//
// Work split: k_agg2 forms each sub-segment's dS increment from a zero start,
// k_scan_rev chains them from the end of the sequence, k_main2 walks each
// segment's chunks backwards from the dS entering it on the right, k_finish2
// sums the per-segment DMIMO_V and DD partials in segment order.
#pragma once

#include "mimo_kernels.hpp"

namespace mimo {
namespace b2 {

constexpr int NTHR = 512;      // the aggregate (two workgroups of eight waves per CU)
constexpr int NTHR2 = 512;     // the chunk pass (one workgroup per CU: eight waves hide more latency)
constexpr int NTHR1 = 256;     // the reverse scan and the final sums
constexpr int LD = 68;              // row pitch (floats) of every tile (16-byte rows, 4 mod 64)
constexpr int TILE = 64 * LD;       // floats per tile

struct Params2 {
    int B, S, H, G, R, N, P, C, W, nc, L, nseg, F, nsub, reduce_o, has_d, out_f32;
    const unsigned short *dout, *q, *k, *v, *states, *qk_dot, *trap;
    const float *q_bias, *k_bias, *mimo_v, *mimo_o, *da_cs, *da_cs_rev, *dt, *segsum, *angles, *d;
    void *dq, *dk, *dv;   // bf16 or fp32 (out_f32)
    float *dmimo_v, *dangles, *dfactor, *dgamma, *dda, *dssda, *dda_cs_rev, *dda_cs, *dd;
    float* agg;       // [B*H][nsub][N*P] sub-segment dS increments, then dS at segment boundaries
    float* decay;     // [B*H][nsub] products of the chunk state decays
    float* part_mv;   // [B*H][nseg][R*P] per-segment DMIMO_V partials
    float* part_d;    // [B*H][nseg] per-segment DD partials
};

__device__ __forceinline__ float bf(unsigned short x) { return __uint_as_float(static_cast<unsigned>(x) << 16); }

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// C(i, j) = sum_k A(i, k) B(k, j) (* sk[k]) for i < Mi, j < Nj, k < K (all <= 64) on
// [64][LD] LDS tiles, on fp32 MFMA (16 x 16 x 4). AK1: A(i, k) = A[i*LD + k], else
// A[k*LD + i]; BK1: B(k, j) = B[j*LD + k], else B[k*LD + j]. The output is 4 x 4
// blocks of 16 x 16: of the NT/64 waves, wave w owns row block w / (4/CW) and the CW =
// 16 / (NT/64) column blocks from CW * (w % (4/CW)), and hands each result to epi(i,
// j, value). The contraction index is split k = 16 kt + 4 q + v (q = lane / 16, v the
// accumulation step), so a lane reads four consecutive floats of a
// contraction-contiguous row in one 16-byte load, or one float of each of four rows;
// with LD = 4 (mod 64) neither pattern has bank conflicts. Every operand is read
// before the first MFMA. Values past K are zeroed (the tiles hold stale data there);
// rows and columns past Mi / Nj are dropped.
// RS: epi returns a term of a row sum; the sums over the wave's columns go to
// rs[(w % (4/CW)) * 64 + i] (one partial per column group, added in a fixed order
// by the reader after a barrier).
template <int NT, bool AK1, bool BK1, bool SK, bool RS = false, typename F>
__device__ __forceinline__ void gemm64(int Mi, int Nj, int K, const float* A, const float* B, const float* sk,
                                       F&& epi, float* rs = nullptr) {
    constexpr int NW = NT / 64, CW = 16 / NW, WR = 4 / CW;   // waves, column blocks a wave, waves a row block
    const int tid = tid_x(), w = tid >> 6, x = tid & 15, q = (tid >> 4) & 3;
    const int i0 = 16 * (w / WR), j0 = 16 * CW * (w % WR);
    if (i0 >= Mi) return;   // wave-uniform
    const int nk = (K + 15) >> 4;
    float a[4][4], bv[4][CW][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
        if (kt >= nk) break;   // wave-uniform
        const int kb = 16 * kt + 4 * q;
        if constexpr (AK1) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(A + (i0 + x) * LD + kb);
#pragma unroll
            for (int v = 0; v < 4; ++v) a[kt][v] = t[v];
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) a[kt][v] = A[(kb + v) * LD + i0 + x];
        }
        if constexpr (SK) {
            const f32x4 sc = *reinterpret_cast<const f32x4*>(sk + kb);
#pragma unroll
            for (int v = 0; v < 4; ++v) a[kt][v] *= sc[v];
        }
#pragma unroll
        for (int cb = 0; cb < CW; ++cb) {
            const int jb = j0 + 16 * cb;
            if (jb >= Nj) break;   // wave-uniform
            if constexpr (BK1) {
                const f32x4 t = *reinterpret_cast<const f32x4*>(B + (jb + x) * LD + kb);
#pragma unroll
                for (int v = 0; v < 4; ++v) bv[kt][cb][v] = t[v];
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v) bv[kt][cb][v] = B[(kb + v) * LD + jb + x];
            }
        }
    }
    if (K & 15) {   // wave-uniform: zero the last step's values past K (the tiles hold stale data there)
        const int kt = nk - 1, kb = 16 * kt + 4 * q;
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            if (t4 != kt) continue;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const bool in = kb + v < K;
                a[t4][v] = in ? a[t4][v] : 0.f;
#pragma unroll
                for (int cb = 0; cb < CW; ++cb) bv[t4][cb][v] = in ? bv[t4][cb][v] : 0.f;
            }
        }
    }
    f32x4 acc[CW];
#pragma unroll
    for (int cb = 0; cb < CW; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
        if (kt >= nk) break;
#pragma unroll
        for (int cb = 0; cb < CW; ++cb) {
            if (j0 + 16 * cb >= Nj) break;
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[cb] = mfma_f32(a[kt][v], bv[kt][cb][v], acc[cb]);
        }
    }
    float rsum[4] = {0.f, 0.f, 0.f, 0.f};
    const bool full = i0 + 16 <= Mi && j0 + 16 * CW <= Nj;   // wave-uniform
#pragma unroll
    for (int cb = 0; cb < CW; ++cb) {
        const int j = j0 + 16 * cb + x;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = i0 + 4 * q + v;
            if (full || (i < Mi && j < Nj)) {
                if constexpr (RS)
                    rsum[v] += epi(i, j, acc[cb][v]);
                else
                    epi(i, j, acc[cb][v]);
            }
        }
    }
    if constexpr (RS) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) rsum[v] += __shfl_xor(rsum[v], o);
        }
        if (x == 0) {
#pragma unroll
            for (int v = 0; v < 4; ++v) rs[(w % WR) * 64 + i0 + 4 * q + v] = rsum[v];
        }
    }
}

// Block-wide sum over NT threads (every thread passes its value; the result is
// valid in every thread).
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) s += red[w];
    return s;
}

// Per-token totals of row sums left by a product (rs[h * 64 + i], h < 2 column
// groups): token t's total over its rows r*C + t (r < R), in a fixed order, handed to
// out(t, total) by thread t.
template <typename O>
__device__ __forceinline__ void token_out(int cl, int R, int C, const float* rs, O&& out) {
    const int t = tid_x();
    if (t < cl) {
        float s = 0.f;
        for (int r = 0; r < R; ++r) s += rs[r * C + t] + rs[64 + r * C + t];
        out(t, s);
    }
}

// LDS layout (floats) of the chunk pass: q^, k^, Psi, dPhiO, S_c, dS, the causal
// block, W and an output tile, each [64][LD]; then per-row token scalars (row i =
// r*C + t: gamma, factor, exp(da_cs), exp(da_cs_rev)), a reduction scratch, the
// same-token tables [C][R][R] (dots, cached qk_dot) and two sets of row-sum partials
// [2][64]. The aggregate uses q^, dPhiO,
// dS, an output tile and exp(da_cs).
struct L2 {
    static constexpr int QH = 0, KH = TILE, PS = 2 * TILE, DPO = 3 * TILE, SC = 4 * TILE, DS = 5 * TILE,
                         AM = 6 * TILE, WM = 7 * TILE, OUT = 8 * TILE;
    static constexpr int GAM = 9 * TILE, FAC = GAM + 64, ECS = FAC + 64, EREV = ECS + 64, RED = EREV + 64,
                         DQK = RED + 8, QKC = DQK + 512, RS0 = QKC + 512, RS1 = RS0 + 128, TOTAL = RS1 + 128;
    static constexpr int A_QH = 0, A_DPO = TILE, A_U = 2 * TILE, A_G = 3 * TILE, A_ECS = 4 * TILE,
                         AGG_TOTAL = 4 * TILE + 64;
};

// e / d and e % d for 0 <= e < 16384 and 1 <= d <= 64 from d's reciprocal: the exact
// quotient of e + 1/2 is at least 1/(2d) >= 1/128 away from an integer and the
// rounded product is off by less than 0.002.
struct DivS {
    int d;
    float rd;
    __device__ explicit DivS(int d_) : d(d_), rd(1.0f / static_cast<float>(d_)) {}
    __device__ int q(int e) const { return static_cast<int>((static_cast<float>(e) + 0.5f) * rd); }
    __device__ int r(int e) const { return e - q(e) * d; }
};

// Items of the chunk load, a thread's items being e = tid + NT x for x < IX (every
// kind has at most 64 * 64 / 8 = 512 of them):
//   rotation items (i, n4): four columns n4.. of each half (n4 < N/2) of row i of q^
//     (and k^); the thread keeps cos and sin of its columns (1 and 0 where the
//     column is past the rotated width or the row past the chunk) for the output pass;
//   value items (i, p8): eight columns of dPhiO (and Psi) of row i; the thread keeps
//     its raw v (the rank-0 items' v is the chunk's v);
//   state items: eight consecutive values of the cached state.
// A thread's items are the same in every chunk, so the biases and projections they
// use are read once (Res). The loads of a chunk (Fetch) are issued a chunk ahead and
// staged into LDS (rotated, scaled, converted to fp32) at the start of the chunk.
template <int NT>
struct Items {
    static constexpr int IX = 512 / NT;
    static constexpr int SX = 64 * 64 / NT;   // segsum values a thread (C * C <= 4096)
};
template <int NT>
struct Keep {
    float cs[Items<NT>::IX][4], sn[Items<NT>::IX][4];
    u32x4 v[Items<NT>::IX];
};
template <int NT>
struct Res {
    f32x4 qb[Items<NT>::IX][2], kb[Items<NT>::IX][2], mo[Items<NT>::IX][2], mv[Items<NT>::IX][2];
};
template <int NT>
struct Fetch {
    u32x2 qw[Items<NT>::IX][2], kw[Items<NT>::IX][2];
    float ang[Items<NT>::IX][4];
    u32x4 dw[Items<NT>::IX], vw[Items<NT>::IX], sw[Items<NT>::IX];
    float s_cs, s_rev, s_dt, s_tr, s_dt1, s_tr1, qk;
    float seg[Items<NT>::SX];
};

// The index decompositions of the chunk-load items.
struct ItemDiv {
    DivS dC, dM4, dP8;
    __device__ ItemDiv(int C, int N, int P) : dC(C), dM4(N / 8), dP8(P / 8) {}
};

template <bool MAIN, int NT>
__device__ __forceinline__ void load_resident(const Params2& p, int h, const ItemDiv& dv, Res<NT>& res) {
    const int R = p.R, N = p.N, P = p.P, C = p.C, M = N / 2;
    const int tid = tid_x(), rows = R * C;
#pragma unroll
    for (int x = 0; x < Items<NT>::IX; ++x) {
        const int e = tid + NT * x;
        if (e < rows * (M / 4)) {
            const int i = dv.dM4.q(e), n4 = 4 * (e - i * (M / 4)), r = dv.dC.q(i);
            const float* qbp = p.q_bias + ((long)h * R + r) * N + n4;
            res.qb[x][0] = *reinterpret_cast<const f32x4*>(qbp);
            res.qb[x][1] = *reinterpret_cast<const f32x4*>(qbp + M);
            if (MAIN) {
                const float* kbp = p.k_bias + ((long)h * R + r) * N + n4;
                res.kb[x][0] = *reinterpret_cast<const f32x4*>(kbp);
                res.kb[x][1] = *reinterpret_cast<const f32x4*>(kbp + M);
            }
        }
        if (e < rows * (P / 8)) {
            const int i = dv.dP8.q(e), p8 = 8 * (e - i * (P / 8)), r = dv.dC.q(i);
            if (p.reduce_o) {
                const float* m = p.mimo_o + ((long)h * R + r) * P + p8;
                res.mo[x][0] = *reinterpret_cast<const f32x4*>(m);
                res.mo[x][1] = *reinterpret_cast<const f32x4*>(m + 4);
            }
            if (MAIN) {
                const float* m = p.mimo_v + ((long)h * R + r) * P + p8;
                res.mv[x][0] = *reinterpret_cast<const f32x4*>(m);
                res.mv[x][1] = *reinterpret_cast<const f32x4*>(m + 4);
            }
        }
    }
}

// Issue chunk c's global loads (rows past the chunk are not read).
template <bool MAIN, int NT>
__device__ __forceinline__ void fetch_chunk(const Params2& p, int b, int h, int g, int bh, int c, const ItemDiv& dv,
                                            Fetch<NT>& f) {
    const int R = p.R, N = p.N, P = p.P, C = p.C, W = p.W, M = N / 2;
    const int tid = tid_x(), rows = R * C, RR = R * R;
    const int c0 = c * C, cl = min(C, p.S - c0);
    const long tok0 = (long)b * p.S + c0;   // (b, c0) as a token index
    const long tb0 = (long)bh * p.S + c0;   // (b, h, c0) for the per-token arrays
#pragma unroll
    for (int x = 0; x < Items<NT>::IX; ++x) {
        const int e = tid + NT * x;
        if (e < rows * (M / 4)) {
            const int i = dv.dM4.q(e), n4 = 4 * (e - i * (M / 4));
            const int r = dv.dC.q(i), t = i - r * C;
            if (t < cl) {
                const long src = (((tok0 + t) * R + r) * p.G + g) * N + n4;
                f.qw[x][0] = *reinterpret_cast<const u32x2*>(p.q + src);
                f.qw[x][1] = *reinterpret_cast<const u32x2*>(p.q + src + M);
                if (MAIN) {
                    f.kw[x][0] = *reinterpret_cast<const u32x2*>(p.k + src);
                    f.kw[x][1] = *reinterpret_cast<const u32x2*>(p.k + src + M);
                }
                const float* ap = p.angles + ((tok0 + t) * p.H + h) * W;
#pragma unroll
                for (int v = 0; v < 4; ++v) f.ang[x][v] = n4 + v < W ? ap[n4 + v] : 0.f;
            }
        }
        if (e < rows * (P / 8)) {
            const int i = dv.dP8.q(e), p8 = 8 * (e - i * (P / 8));
            const int r = dv.dC.q(i), t = i - r * C;
            if (t < cl) {
                const long tk = tok0 + t;
                f.dw[x] = *reinterpret_cast<const u32x4*>(
                    p.dout + (p.reduce_o ? (tk * p.H + h) * P : ((tk * R + r) * p.H + h) * P) + p8);
                if (MAIN) f.vw[x] = *reinterpret_cast<const u32x4*>(p.v + (tk * p.H + h) * P + p8);
            }
        }
        if (MAIN && e < N * (P / 8))
            f.sw[x] = *reinterpret_cast<const u32x4*>(p.states + ((long)bh * p.nc + c) * N * P + 8 * e);
    }
    if (tid < cl) {
        f.s_cs = p.da_cs[tb0 + tid];
        if (MAIN) {
            f.s_rev = p.da_cs_rev[tb0 + tid];
            f.s_dt = p.dt[tb0 + tid];
            f.s_tr = bf(p.trap[tb0 + tid]);
            if (c0 + tid + 1 < p.S) {
                f.s_dt1 = p.dt[tb0 + tid + 1];
                f.s_tr1 = bf(p.trap[tb0 + tid + 1]);
            }
        }
    }
    if (MAIN) {
        if (tid < cl * RR) f.qk = bf(p.qk_dot[tb0 * RR + tid]);
#pragma unroll
        for (int x = 0; x < Items<NT>::SX; ++x) {
            const int e = tid + NT * x;
            const int t = dv.dC.q(e), s2 = e - t * C;
            if (e < C * C && s2 < t && t < cl) f.seg[x] = p.segsum[((long)bh * p.nc + c) * C * C + e];
        }
    }
}

// Stage chunk c from its fetched loads into LDS: rotated q^ (and k^, Psi, the cached
// state, qk_dot, exp(segsum) and the per-row scalars when MAIN), dPhiO and exp(da_cs).
// Rows past the chunk (t >= cl) are zero.
template <bool MAIN, int NT>
__device__ __forceinline__ void stage_chunk(const Params2& p, float* sm, int c, const ItemDiv& dv, const Fetch<NT>& f,
                                            const Res<NT>& res, Keep<NT>& keep) {
    const int R = p.R, N = p.N, P = p.P, C = p.C, W = p.W, M = N / 2;
    const int tid = tid_x(), rows = R * C, RR = R * R;
    const int c0 = c * C, cl = min(C, p.S - c0);
    float* QH = sm + (MAIN ? L2::QH : L2::A_QH);
    float* KH = sm + L2::KH;
    float* PS = sm + L2::PS;
    float* DPO = sm + (MAIN ? L2::DPO : L2::A_DPO);
    float* ECS = sm + (MAIN ? L2::ECS : L2::A_ECS);
#pragma unroll
    for (int x = 0; x < Items<NT>::IX; ++x) {
        const int e = tid + NT * x;
        if (e < rows * (M / 4)) {
            const int i = dv.dM4.q(e), n4 = 4 * (e - i * (M / 4));
            const bool live = i - dv.dC.q(i) * C < cl;
            float qa[4], qe[4], ka[4], ke[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float sn = 0.f, cs = 1.f;
                qa[v] = qe[v] = ka[v] = ke[v] = 0.f;
                if (live) {
                    const unsigned wa = f.qw[x][0][v >> 1], we = f.qw[x][1][v >> 1];
                    qa[v] = ((v & 1) ? hi16(wa) : lo16(wa)) + res.qb[x][0][v];
                    qe[v] = ((v & 1) ? hi16(we) : lo16(we)) + res.qb[x][1][v];
                    if (MAIN) {
                        const unsigned ua = f.kw[x][0][v >> 1], ue = f.kw[x][1][v >> 1];
                        ka[v] = ((v & 1) ? hi16(ua) : lo16(ua)) + res.kb[x][0][v];
                        ke[v] = ((v & 1) ? hi16(ue) : lo16(ue)) + res.kb[x][1][v];
                    }
                    if (n4 + v < W) sin_cos_ool(f.ang[x][v], sn, cs);
                }
                keep.cs[x][v] = cs;
                keep.sn[x][v] = sn;
                const float qa2 = cs * qa[v] - sn * qe[v], qe2 = sn * qa[v] + cs * qe[v];
                qa[v] = qa2;
                qe[v] = qe2;
                if (MAIN) {
                    const float ka2 = cs * ka[v] - sn * ke[v], ke2 = sn * ka[v] + cs * ke[v];
                    ka[v] = ka2;
                    ke[v] = ke2;
                }
            }
            *reinterpret_cast<f32x4*>(QH + i * LD + n4) = f32x4{qa[0], qa[1], qa[2], qa[3]};
            *reinterpret_cast<f32x4*>(QH + i * LD + M + n4) = f32x4{qe[0], qe[1], qe[2], qe[3]};
            if (MAIN) {
                *reinterpret_cast<f32x4*>(KH + i * LD + n4) = f32x4{ka[0], ka[1], ka[2], ka[3]};
                *reinterpret_cast<f32x4*>(KH + i * LD + M + n4) = f32x4{ke[0], ke[1], ke[2], ke[3]};
            }
        }
        if (e < rows * (P / 8)) {
            const int i = dv.dP8.q(e), p8 = 8 * (e - i * (P / 8));
            const bool live = i - dv.dC.q(i) * C < cl;
            float d8[8], s8[8];
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                const unsigned wd = f.dw[x][v >> 1];
                const float dv8 = (v & 1) ? hi16(wd) : lo16(wd);
                d8[v] = live ? (p.reduce_o ? dv8 * res.mo[x][v >> 2][v & 3] : dv8) : 0.f;
                if (MAIN) {
                    const unsigned wv = f.vw[x][v >> 1];
                    s8[v] = live ? ((v & 1) ? hi16(wv) : lo16(wv)) * res.mv[x][v >> 2][v & 3] : 0.f;
                }
            }
            *reinterpret_cast<f32x4*>(DPO + i * LD + p8) = f32x4{d8[0], d8[1], d8[2], d8[3]};
            *reinterpret_cast<f32x4*>(DPO + i * LD + p8 + 4) = f32x4{d8[4], d8[5], d8[6], d8[7]};
            if (MAIN) {
                *reinterpret_cast<f32x4*>(PS + i * LD + p8) = f32x4{s8[0], s8[1], s8[2], s8[3]};
                *reinterpret_cast<f32x4*>(PS + i * LD + p8 + 4) = f32x4{s8[4], s8[5], s8[6], s8[7]};
                keep.v[x] = live ? f.vw[x] : u32x4{0u, 0u, 0u, 0u};
            }
        }
        if (MAIN && e < N * (P / 8)) {
            const int n = dv.dP8.q(e), pc = 8 * (e - n * (P / 8));
            float* dst = sm + L2::SC + n * LD + pc;
            const u32x4 w = f.sw[x];
            *reinterpret_cast<f32x4*>(dst) = f32x4{lo16(w[0]), hi16(w[0]), lo16(w[1]), hi16(w[1])};
            *reinterpret_cast<f32x4*>(dst + 4) = f32x4{lo16(w[2]), hi16(w[2]), lo16(w[3]), hi16(w[3])};
        }
    }
    if (tid < C) {
        const bool tok_live = tid < cl;
        const float ecs = tok_live ? expf(f.s_cs) : 0.f;
        float gam = 0.f, fac = 0.f, er = 0.f;
        if (MAIN && tok_live) {
            gam = f.s_dt * (1.0f / (1.0f + expf(-f.s_tr)));
            const float beta = c0 + tid + 1 < p.S ? f.s_dt1 * (1.0f - 1.0f / (1.0f + expf(-f.s_tr1))) : 0.f;
            fac = gam + beta;
            er = expf(f.s_rev);
        }
        for (int r = 0; r < R; ++r) {
            const int i = r * C + tid;
            ECS[i] = ecs;
            if (MAIN) {
                sm[L2::GAM + i] = gam;
                sm[L2::FAC + i] = fac;
                sm[L2::EREV + i] = er;
            }
        }
    }
    if (MAIN) {
        if (tid < cl * RR) sm[L2::QKC + tid] = f.qk;
        // exp(segsum) of the chunk's strictly causal token pairs, in the output tile
        // (free until the dQ^ products)
#pragma unroll
        for (int x = 0; x < Items<NT>::SX; ++x) {
            const int e = tid + NT * x;
            const int t = dv.dC.q(e), s2 = e - t * C;
            if (e < C * C) sm[L2::OUT + t * LD + s2] = (s2 < t && t < cl) ? expf(f.seg[x]) : 0.f;
        }
    }
}

// Sub-segment aggregate: U <- Q^^T (exp(da_cs) dPhiO) + exp(da_cs[last]) U over the
// chunks of the sub-segment from the last one down, and the product of the decays.
// Sub-segment j covers part j % F of segment 1 + j / F (segment 0's aggregate is
// never needed).
__global__ __launch_bounds__(NTHR, 2) void k_agg2(Params2 p) {
    extern __shared__ __align__(16) float sm[];
    int seg, bh;
    Params pp = {};
    pp.B = p.B;
    pp.H = p.H;
    pp.G = p.G;
    if (!map_block(pp, p.nsub, seg, bh)) return;
    seg = uni(seg);
    bh = uni(bh);
    const int b = uni(bh / p.H), h = uni(bh - b * p.H), g = uni(h / (p.H / p.G));
    const int N = p.N, P = p.P, C = p.C, rows = p.R * p.C;
    const int La = p.L / p.F;
    const int c_begin = (1 + seg / p.F) * p.L + (seg % p.F) * La;
    const int c_end = min(c_begin + La, p.nc);
    float* QH = sm + L2::A_QH;
    float* DPO = sm + L2::A_DPO;
    float* U = sm + L2::A_U;
    float* ECS = sm + L2::A_ECS;
    for (int e = threadIdx.x; e < N * P; e += NTHR) U[(e / P) * LD + e % P] = 0.f;
    float dprod = 1.f;
    const ItemDiv dv(C, N, P);
    Keep<NTHR> keep;
    Res<NTHR> res;
    Fetch<NTHR> f;
    load_resident<false, NTHR>(p, h, dv, res);
    if (c_end > c_begin) fetch_chunk<false, NTHR>(p, b, h, g, bh, c_end - 1, dv, f);
    for (int c = c_end - 1; c >= c_begin; --c) {
        const int cl = min(C, p.S - c * C);
        bar();
        stage_chunk<false, NTHR>(p, sm, c, dv, f, res, keep);
        if (c > c_begin) fetch_chunk<false, NTHR>(p, b, h, g, bh, c - 1, dv, f);   // in flight during this chunk
        bar();
        const float dA = ECS[cl - 1];   // exp(da_cs) at the chunk's last token
        // U[n][p] = sum_i Q^[i][n] exp(da_cs[t_i]) dPhiO[i][p] + dA U[n][p]; the thread that
        // owns (n, p) in the product is the only one reading and writing U[n][p]
        // A(n, i) = Q^[i][n], B(i, p) = dPhiO[i][p] scaled per i by exp(da_cs[t_i])
        gemm64<NTHR, false, false, true>(N, P, rows, QH, DPO, ECS,
                                         [&](int n, int pc, float v) { U[n * LD + pc] = v + dA * U[n * LD + pc]; });
        dprod *= dA;
    }
    bar();
    float* out = p.agg + ((long)bh * p.nsub + seg) * N * P;
    for (int e = threadIdx.x; e < N * P; e += NTHR) out[e] = U[(e / P) * LD + e % P];
    if (threadIdx.x == 0) p.decay[(long)bh * p.nsub + seg] = dprod;
}

// dS at the start of every sub-segment, from the end of the sequence: E_j = U_j +
// D_j E_{j+1}; written in place where a segment begins (j % F == 0), which is the
// dS entering segment j / F from the right.
__global__ __launch_bounds__(NTHR1) void k_scan_rev(Params2 p) {
    const int bh = blockIdx.y;
    const int NP = p.N * p.P;
    const int e = blockIdx.x * NTHR1 + threadIdx.x;
    if (e >= NP) return;
    float* base = p.agg + (long)bh * p.nsub * NP + e;
    const float* dec = p.decay + (long)bh * p.nsub;
    float E = 0.f;
    constexpr int AHEAD = 32;
    for (int j0 = p.nsub - 1; j0 >= 0; j0 -= AHEAD) {
        float U[AHEAD], D[AHEAD];
#pragma unroll
        for (int x = 0; x < AHEAD; ++x) {
            const int j = j0 - x;
            if (j >= 0) {
                U[x] = base[(long)j * NP];
                D[x] = dec[j];
            }
        }
#pragma unroll
        for (int x = 0; x < AHEAD; ++x) {
            const int j = j0 - x;
            if (j >= 0) {
                E = __fmaf_rn(D[x], E, U[x]);
                if (j % p.F == 0) base[(long)j * NP] = E;
            }
        }
    }
}

// The rotated-frame gradient of q^ (KSIDE false: dQ^ in OUT plus the same-token part
// sum_r2 dqk'[t][r][r2] k^[t,r2]) or of k^ (KSIDE: factor_t dK~ with dK~ in OUT, plus
// sum_r2 dqk'[t][r2][r] q^[t,r2]), X being k^ or q^ and dqk' the gamma-scaled
// same-token dots, taken back to the input frame by the inverse rotation of the
// thread's rotation items (cos and sin kept from the load) and written to DQ or DK
// [B, S*R, H, N], four columns of each half a store. OUT is only read.
template <bool F32OUT, int NT, bool KSIDE>
__device__ __forceinline__ void finish_rot(const Params2& p, void* dst, const float* OUT, const float* X,
                                           const float* DQK, const float* FAC, const Keep<NT>& keep, int b, int h,
                                           int c0, int cl, const DivS& dC, const DivS& dM4) {
    const int R = p.R, N = p.N, C = p.C, M = N / 2, RR = R * R;
#pragma unroll
    for (int x = 0; x < Items<NT>::IX; ++x) {
        const int e = tid_x() + NT * x;
        if (e >= R * C * (M / 4)) continue;
        const int i = dM4.q(e), n4 = 4 * (e - i * (M / 4));
        const int r = dC.q(i), t = i - r * C;
        if (t >= cl) continue;
        const f32x4 a = *reinterpret_cast<const f32x4*>(OUT + i * LD + n4);
        const f32x4 ee = *reinterpret_cast<const f32x4*>(OUT + i * LD + M + n4);
        const float f = KSIDE ? FAC[i] : 1.f;
        float sa[4], se[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            sa[v] = a[v] * f;
            se[v] = ee[v] * f;
        }
        for (int r2 = 0; r2 < R; ++r2) {
            const float d = KSIDE ? DQK[t * RR + r2 * R + r] : DQK[t * RR + r * R + r2];
            const float* xr = X + (r2 * C + t) * LD;
            const f32x4 xa = *reinterpret_cast<const f32x4*>(xr + n4);
            const f32x4 xe = *reinterpret_cast<const f32x4*>(xr + M + n4);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                sa[v] = __fmaf_rn(d, xa[v], sa[v]);
                se[v] = __fmaf_rn(d, xe[v], se[v]);
            }
        }
        float a2[4], e2[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float cs = keep.cs[x][v], sn = keep.sn[x][v];
            a2[v] = cs * sa[v] + sn * se[v];
            e2[v] = -sn * sa[v] + cs * se[v];
        }
        const long o = (((long)b * p.S * R + (long)(c0 + t) * R + r) * p.H + h) * N + n4;
        if constexpr (F32OUT) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(dst) + o) = f32x4{a2[0], a2[1], a2[2], a2[3]};
            *reinterpret_cast<f32x4*>(static_cast<float*>(dst) + o + M) = f32x4{e2[0], e2[1], e2[2], e2[3]};
        } else {
            *reinterpret_cast<u32x2*>(static_cast<unsigned short*>(dst) + o) = u32x2{pk2(a2[0], a2[1]), pk2(a2[2], a2[3])};
            *reinterpret_cast<u32x2*>(static_cast<unsigned short*>(dst) + o + M) =
                u32x2{pk2(e2[0], e2[1]), pk2(e2[2], e2[3])};
        }
    }
}

// The chunk pass of one segment, chunks from the last down.
template <bool F32OUT>
__global__ __launch_bounds__(NTHR2, 1) void k_main2(Params2 p) {
    extern __shared__ __align__(16) float sm[];
    int seg, bh;
    Params pp = {};
    pp.B = p.B;
    pp.H = p.H;
    pp.G = p.G;
    if (!map_block(pp, p.nseg, seg, bh)) return;
    seg = uni(seg);
    bh = uni(bh);
    const int b = uni(bh / p.H), h = uni(bh - b * p.H), g = uni(h / (p.H / p.G));
    const int R = p.R, N = p.N, P = p.P, C = p.C, W = p.W, M = N / 2, RR = R * R;
    const int rows = R * C;
    const int tid = threadIdx.x;
    const int c_begin = seg * p.L;
    const int c_end = min(c_begin + p.L, p.nc);
    float* QH = sm + L2::QH;
    float* KH = sm + L2::KH;
    float* PS = sm + L2::PS;
    float* DPO = sm + L2::DPO;
    float* SC = sm + L2::SC;
    float* DS = sm + L2::DS;
    float* AM = sm + L2::AM;
    float* WM = sm + L2::WM;
    float* OUT = sm + L2::OUT;
    float* GAM = sm + L2::GAM;
    float* FAC = sm + L2::FAC;
    float* ECS = sm + L2::ECS;
    float* EREV = sm + L2::EREV;
    float* RED = sm + L2::RED;
    float* DQK = sm + L2::DQK;
    float* QKC = sm + L2::QKC;
    float* RS0 = sm + L2::RS0;
    float* RS1 = sm + L2::RS1;
    const float dval = p.has_d ? p.d[h] : 0.f;

    // dS entering the segment from the right
    {
        const float* E = (seg + 1 < p.nseg) ? p.agg + ((long)bh * p.nsub + seg * p.F) * N * P : nullptr;
        for (int e = tid; e < N * P; e += NTHR2) DS[(e / P) * LD + e % P] = E ? E[e] : 0.f;
    }
    const long tokS = (long)bh * p.S;
    const ItemDiv dv(C, N, P);
    const DivS &dC = dv.dC, &dM4 = dv.dM4, &dP8 = dv.dP8;
    const DivS dRR(RR), dP(P), dP4(P / 4);
    Keep<NTHR2> keep;
    Res<NTHR2> res;
    Fetch<NTHR2> f;
    load_resident<true, NTHR2>(p, h, dv, res);
    if (c_end > c_begin) fetch_chunk<true, NTHR2>(p, b, h, g, bh, c_end - 1, dv, f);
    // DDA of the previous chunk: its last token takes exp(da_cs[last]) times the sum of
    // the per-wave partials in RED (written after the chunk's dS product)
    int pend_c0 = 0, pend_cl = 0;
    float pend_dA = 0.f;
    auto flush_dda = [&]() {
        const int t = tid_x();
        if (t < pend_cl) {
            float tot = 0.f;
#pragma unroll
            for (int w = 0; w < NTHR2 / 64; ++w) tot += RED[w];
            p.dda[tokS + pend_c0 + t] = (t == pend_cl - 1) ? pend_dA * tot : 0.f;
        }
        pend_cl = 0;
    };
    float mvacc = 0.f;   // DMIMO_V item (r, p) = tid (R * P <= 512)
    float ddacc = 0.f;

    for (int c = c_end - 1; c >= c_begin; --c) {
        const int c0 = c * C;
        const int cl = min(C, p.S - c0);
        const int tid = tid_x();
        bar();
        flush_dda();
        stage_chunk<true, NTHR2>(p, sm, c, dv, f, res, keep);
        if (c > c_begin) fetch_chunk<true, NTHR2>(p, b, h, g, bh, c - 1, dv, f);   // in flight during this chunk
        bar();

        // ---- causal block A = E (Q^ K~^T) and dP = dPhiO Psi^T; dP's same-token entries
        // are the dots dPhiO[t,r] . Psi[t,r2] (DGAMMA, the D-skip sum, the same-token parts).
        // The same-token entries of A take the coefficients with which Psi[t,r2] enters
        // y[t,r] directly, gamma_t qk_dot[t][r][r2] (+ d where r = r2), so A^T dPhiO carries
        // those terms of dPsi.
        gemm64<NTHR2, true, true, false>(rows, rows, N, QH, KH, nullptr, [&](int i, int j, float v) {
            const int ri = dC.q(i), ti = i - ri * C, rj = dC.q(j), tj = j - rj * C;
            float a = 0.f;
            if (tj < ti && ti < cl) a = v * FAC[j] * OUT[ti * LD + tj];
            if (tj == ti && ti < cl) a = GAM[j] * QKC[ti * RR + ri * R + rj] + (i == j ? dval : 0.f);
            AM[i * LD + j] = a;
        });
        gemm64<NTHR2, true, true, false>(rows, rows, P, DPO, PS, nullptr, [&](int i, int j, float v) {
            WM[i * LD + j] = v;
            const int ri = dC.q(i), ti = i - ri * C, rj = dC.q(j), tj = j - rj * C;
            if (ti == tj && ti < cl) DQK[ti * RR + ri * R + rj] = v;
        });
        bar();
        if (tid < cl) {
            const int t = tid;
            float dg = 0.f;
            for (int rr = 0; rr < RR; ++rr) dg = __fmaf_rn(QKC[t * RR + rr], DQK[t * RR + rr], dg);
            p.dgamma[tokS + c0 + t] = dg;
            for (int r = 0; r < R; ++r) ddacc += DQK[t * RR + r * R + r];
        }
        // ---- DSSDA (per token pair: sum over rank pairs of A * dP), then W = E dP in place
        for (int e = tid; e < C * C; e += NTHR2) {
            const int t = dC.q(e), s = e - t * C;
            float acc = 0.f;
            const bool live = s < t && t < cl;
            const float ex = OUT[t * LD + s];   // zero unless live
            for (int r = 0; r < R; ++r)
                for (int r2 = 0; r2 < R; ++r2) {
                    const int i = r * C + t, j = r2 * C + s;
                    const float dp = WM[i * LD + j];
                    acc = __fmaf_rn(AM[i * LD + j], dp, acc);
                    WM[i * LD + j] = dp * ex;
                }
            p.dssda[(((long)bh * p.nc + c) * C + t) * C + s] = live ? acc : 0.f;
        }
        bar();
        // same-token factors of the diagonal: gamma_t times the dots
        for (int e = tid; e < cl * RR; e += NTHR2) DQK[e] *= GAM[dRR.q(e)];

        // ---- dQ^ = exp(da_cs) dPhiO S_c^T + W K~; DDA_CS[t] = sum over the token's rows of
        // q^ . (exp(da_cs) dPhiO S_c^T), as row sums of the first product
        gemm64<NTHR2, true, true, false, true>(
            rows, N, P, DPO, SC, nullptr,
            [&](int i, int n, float v) {
                const float o = v * ECS[i];
                OUT[i * LD + n] = o;
                return QH[i * LD + n] * o;
            },
            RS0);
        bar();
        token_out(cl, R, C, RS0, [&](int t, float v) { p.dda_cs[tokS + c0 + t] = v; });
        // W K~: B(j, n) = k^[j][n] scaled per j by the factor (folded into A)
        gemm64<NTHR2, true, false, true>(rows, N, rows, WM, KH, FAC,
                                         [&](int i, int n, float v) { OUT[i * LD + n] += v; });
        bar();
        // angle gradient, q part: d(a')/dθ = -e', d(e')/dθ = a' for the rotated pair (a', e')
        float dth[4];   // items (t, n): t < 64, n < 32 (W <= 32)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int e = tid + NTHR2 * x;
            const int t = e / 32, n = e % 32;
            float s = 0.f;
            if (t < cl && n < W)
                for (int r = 0; r < R; ++r) {
                    const int i = r * C + t;
                    s += OUT[i * LD + n] * (-QH[i * LD + M + n]) + OUT[i * LD + M + n] * QH[i * LD + n];
                }
            dth[x] = s;
        }
        // the same-token part, then back to the input frame: DQ (OUT is only read)
        finish_rot<F32OUT, NTHR2, false>(p, p.dq, OUT, KH, DQK, FAC, keep, b, h, c0, cl, dC, dM4);
        bar();

        // ---- dK~ = exp(da_cs_rev) Psi dS^T + W^T Q^; DDA_CS_REV from the first product's row
        // sums (k^ . its rows), DFACTOR from those of the whole dK~
        gemm64<NTHR2, true, true, false, true>(
            rows, N, P, PS, DS, nullptr,
            [&](int j, int n, float v) {
                const float o = v * EREV[j];
                OUT[j * LD + n] = o;
                return KH[j * LD + n] * o;
            },
            RS1);
        bar();
        token_out(cl, R, C, RS1, [&](int t, float v) { p.dda_cs_rev[tokS + c0 + t] = v * FAC[t]; });
        gemm64<NTHR2, false, false, false, true>(
            rows, N, rows, WM, QH, nullptr,
            [&](int j, int n, float v) {
                const float o = OUT[j * LD + n] + v;
                OUT[j * LD + n] = o;
                return KH[j * LD + n] * o;
            },
            RS0);
        bar();
        token_out(cl, R, C, RS0, [&](int t, float v) { p.dfactor[tokS + c0 + t] = v; });
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int e = tid + NTHR2 * x;
            const int t = e / 32, n = e % 32;
            if (t < cl && n < W) {
                float s = 0.f;
                for (int r = 0; r < R; ++r) {
                    const int i = r * C + t;
                    s += OUT[i * LD + n] * (-KH[i * LD + M + n]) + OUT[i * LD + M + n] * KH[i * LD + n];
                }
                dth[x] += s * FAC[t];
                p.dangles[((long)(b * p.S + c0 + t) * p.H + h) * W + n] = dth[x];
            }
        }
        // dk^ = factor dK~ plus the same-token part, then back to the input frame: DK
        finish_rot<F32OUT, NTHR2, true>(p, p.dk, OUT, QH, DQK, FAC, keep, b, h, c0, cl, dC, dM4);
        // v of the chunk into the W tile (free after the dK~ products), for DMIMO_V
        // (the rank-0 value items hold the chunk's v, zero past the chunk)
        if (tid < C * (P / 8)) {
            const int t = dP8.q(tid), p8 = 8 * (tid - t * (P / 8));
            const u32x4 w = keep.v[0];
            *reinterpret_cast<f32x4*>(WM + t * LD + p8) = f32x4{lo16(w[0]), hi16(w[0]), lo16(w[1]), hi16(w[1])};
            *reinterpret_cast<f32x4*>(WM + t * LD + p8 + 4) = f32x4{lo16(w[2]), hi16(w[2]), lo16(w[3]), hi16(w[3])};
        }
        bar();

        // ---- dPsi = kappa dS + A^T dPhiO (the latter with the same-token and d terms)
        gemm64<NTHR2, true, false, false>(rows, P, N, KH, DS, nullptr,
                                          [&](int j, int pc, float v) { OUT[j * LD + pc] = v * FAC[j] * EREV[j]; });
        gemm64<NTHR2, false, false, false>(rows, P, rows, AM, DPO, nullptr,
                                           [&](int j, int pc, float v) { OUT[j * LD + pc] += v; });
        bar();
        for (int e = tid; e < cl * (P / 4); e += NTHR2) {
            const int t = dP4.q(e), p4 = 4 * (e - t * (P / 4));
            float s[4] = {0.f, 0.f, 0.f, 0.f};
            for (int r = 0; r < R; ++r) {
                const f32x4 o = *reinterpret_cast<const f32x4*>(OUT + (r * C + t) * LD + p4);
                const f32x4 m = *reinterpret_cast<const f32x4*>(p.mimo_v + ((long)h * R + r) * P + p4);
#pragma unroll
                for (int v = 0; v < 4; ++v) s[v] = __fmaf_rn(o[v], m[v], s[v]);
            }
            const long o = ((long)(b * p.S + c0 + t) * p.H + h) * P + p4;
            if constexpr (F32OUT)
                *reinterpret_cast<f32x4*>(static_cast<float*>(p.dv) + o) = f32x4{s[0], s[1], s[2], s[3]};
            else
                *reinterpret_cast<u32x2*>(static_cast<unsigned short*>(p.dv) + o) = u32x2{pk2(s[0], s[1]), pk2(s[2], s[3])};
        }
        if (tid < R * P) {
            const int r = dP.q(tid), pc = tid - r * P;
            float s = 0.f;
            for (int t = 0; t < cl; ++t) s = __fmaf_rn(OUT[(r * C + t) * LD + pc], WM[t * LD + pc], s);
            mvacc += s;
        }

        // ---- dS_c = Q^^T (exp(da_cs) dPhiO) + exp(da_cs[last]) dS_{c+1}, and DDA: the state
        // decay exp(da_cs[last]) multiplies S_c in S_{c+1}, so DDA[last] = exp(da_cs[last])
        // sum(dS_{c+1} * S_c), summed from the elements each lane updates (a wave's partial
        // into RED, the total after the next barrier)
        const float dA = ECS[cl - 1];
        float part = 0.f;
        gemm64<NTHR2, false, false, true>(N, P, rows, QH, DPO, ECS, [&](int n, int pc, float v) {
            const float old = DS[n * LD + pc];
            part = __fmaf_rn(old, SC[n * LD + pc], part);
            DS[n * LD + pc] = v + dA * old;
        });
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o);
        if ((tid & 63) == 0) RED[tid >> 6] = part;
        pend_c0 = c0;
        pend_cl = cl;
        pend_dA = dA;
    }
    bar();
    flush_dda();

    // ---- per-segment partial sums of DMIMO_V and DD
    __syncthreads();
    if (tid < R * P) p.part_mv[((long)bh * p.nseg + seg) * R * P + tid] = mvacc;
    const float dd = block_sum<NTHR2>(ddacc, RED);
    if (tid == 0) p.part_d[(long)bh * p.nseg + seg] = dd;
}

// DMIMO_V [B,H,R,P] and DD [B,H]: the per-segment partials summed in segment order.
__global__ __launch_bounds__(NTHR1) void k_finish2(Params2 p) {
    const long RP = (long)p.R * p.P;
    const long e = (long)blockIdx.x * NTHR1 + threadIdx.x;
    const long tot = (long)p.B * p.H * RP;
    if (e < tot) {
        const long bh = e / RP, rp = e - bh * RP;
        float s = 0.f;
        for (int sg = 0; sg < p.nseg; ++sg) s += p.part_mv[(bh * p.nseg + sg) * RP + rp];
        p.dmimo_v[e] = s;
    }
    if (p.has_d && e < (long)p.B * p.H) {
        float s = 0.f;
        for (int sg = 0; sg < p.nseg; ++sg) s += p.part_d[e * p.nseg + sg];
        p.dd[e] = s;
    }
}

}  // namespace b2
}  // namespace mimo
