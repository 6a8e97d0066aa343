// Device code of the mamba_mimo_bwd_fwd HIP library: parameters, LDS layout,
// preparation stages and the two chunk kernels (templates over tile sizes).
// Instantiated per tile height in inst_mt*.hip; the host side lives in
// mimo_bwd_fwd.hip.
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "mimo_bwd_fwd.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

namespace mimo {

constexpr int kMaxRows = 128;  // C*R rows of a chunk tile (padded)

// ---------------------------------------------------------------- scalar helpers
// bf16 round-to-nearest-even of an fp32 value, returned as fp32.
__device__ __forceinline__ float bfr(float x) { return static_cast<float>(static_cast<__bf16>(x)); }
__device__ __forceinline__ float bf2f(unsigned short u) { return __uint_as_float(static_cast<unsigned>(u) << 16); }
__device__ __forceinline__ unsigned short f2bf(float x) {
    return __builtin_bit_cast(unsigned short, static_cast<__bf16>(x));
}
__device__ __forceinline__ float bfv(const __bf16 x) { return static_cast<float>(x); }
// precise logistic function for per-token scalars
__device__ __forceinline__ float sigmoid_precise(float x) { return 1.0f / (1.0f + expf(-x)); }

__device__ __forceinline__ f32x4 mfma(const bf16x8 a, const bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- parameters
struct Params {
    int B, S, H, G, R, N, P, C, Cp, W, nc, L, nseg, rd;
    int reduce_o, has_z, has_d, need_y;
    const unsigned short *dout, *q, *k, *v, *z, *trap;
    const float *q_bias, *k_bias, *mimo_v, *mimo_o, *mimo_z, *angles, *da_cs, *da_cs_rev, *dt, *d,
        *segsum;
    float *dmimo_o, *dmimo_z;
    unsigned short *states, *dz, *qk_dot;
    float *agg;     // [B*H][nseg-1][N*P]: segment state increments, then segment entry states
    float *decay;   // [B*H][nseg]: product of the chunk decays of each segment
    float *part_o;  // [B*H][nseg][R*P] partial dmimo_o (== dmimo_o when nseg == 1)
    float *part_z;  // [B*H][nseg][R*P] partial dmimo_z
};

// LDS carve-up shared by host and device. Element pitches keep rows 16-byte
// aligned and add 8 bf16 of padding per row.
struct Lds {
    int ldq;  // pitch of [*][NT] rows (sQ, sK, sSbT)
    int lda;  // pitch of [*][MT] rows (sA, sKapT, sPsiT)
    int r1, r2, r3, r4, sm1, sqk, sc, total;  // byte offsets / size
};

__host__ __device__ inline int align16(int x) { return (x + 15) & ~15; }

__host__ __device__ inline Lds lds_layout(int MT, int NT, int PT, int C, int R, int W, bool main) {
    Lds s;
    s.ldq = NT + 8;
    s.lda = MT + 8;
    int r1 = MT * s.ldq;
    if (MT * s.lda > r1) r1 = MT * s.lda;
    if (NT * s.lda > r1) r1 = NT * s.lda;
    int off = 0;
    s.r1 = off;
    off += align16(r1 * 2);
    s.r2 = off;
    if (main) off += align16(MT * s.ldq * 2);
    s.r3 = off;
    off += align16(PT * s.lda * 2);
    s.r4 = off;
    if (main) off += align16(PT * s.ldq * 2);
    int sm1 = 2 * C * W;
    if (main && C * C > sm1) sm1 = C * C;
    s.sm1 = off;
    off += align16(sm1 * 4);
    s.sqk = off;
    if (main) off += align16(C * R * R * 4);
    s.sc = off;
    off += align16((5 * kMaxRows + 8) * 4);
    s.total = off;
    return s;
}

// Per-token scalars of one chunk (tokens t < Cp; zero beyond the chunk's
// real tokens) and the cos/sin table of the rotation, [C][W] each.
// gamma_t = bf16(dt_t) * sigmoid(trap_t)                        (fp32)
// beta_t  = bf16(bf16(dt_{t+1}) * sigmoid(-trap_{t+1})), 0 at the last token
// factor_t = bf16(gamma_t + beta_t)
template <int NTHR>
__device__ __forceinline__ void prep_scalars(const Params& p, int bh, int b, int h, int c0, int cl,
                                             float* sc, float* scs, bool main) {
    const int tid = threadIdx.x;
    float* s_ecs = sc;
    float* s_gam = sc + kMaxRows;
    float* s_erev = sc + 2 * kMaxRows;
    float* s_fac = sc + 3 * kMaxRows;
    for (int t = tid; t < p.Cp; t += NTHR) {
        float gam = 0.f, fac = 0.f, ecs = 0.f, erev = 0.f;
        if (t < cl) {
            const long idx = (long)bh * p.S + c0 + t;
            const float dtb = bfr(p.dt[idx]);
            gam = dtb * sigmoid_precise(bf2f(p.trap[idx]));
            float beta = 0.f;
            if (c0 + t + 1 < p.S) beta = bfr(bfr(p.dt[idx + 1]) * sigmoid_precise(-bf2f(p.trap[idx + 1])));
            fac = bfr(gam + beta);
            erev = expf(p.da_cs_rev[idx]);
            if (main) ecs = expf(p.da_cs[idx]);
        }
        s_ecs[t] = ecs;
        s_gam[t] = gam;
        s_erev[t] = erev;
        s_fac[t] = fac;
    }
    if (tid == 0) sc[4 * kMaxRows] = expf(p.da_cs[(long)bh * p.S + c0 + cl - 1]);
    const int CW = p.C * p.W;
    for (int e = tid; e < CW; e += NTHR) {
        const int t = e / p.W, n = e - t * p.W;
        float cs = 0.f, sn = 0.f;
        if (t < cl) {
            const float th = p.angles[((long)(b * p.S + c0 + t) * p.H + h) * p.W + n];
            sincosf(th, &sn, &cs);
        }
        scs[e] = cs;
        scs[CW + e] = sn;
    }
}

// Load 8 consecutive bf16 (16 bytes) from global memory.
__device__ __forceinline__ u16x8 ld8(const unsigned short* ptr) { return *reinterpret_cast<const u16x8*>(ptr); }

// Biased, bf16-rounded values of one 8-column group: bf16(x + bf16(bias)).
__device__ __forceinline__ void bias8(const u16x8 x, const float* bias, float out[8]) {
    const float4 b0 = *reinterpret_cast<const float4*>(bias);
    const float4 b1 = *reinterpret_cast<const float4*>(bias + 4);
    const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = bfr(bf2f(x[e]) + bfr(bb[e]));
}

__device__ __forceinline__ void st8(__bf16* dst, const float v[8]) {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = static_cast<__bf16>(v[e]);
    *reinterpret_cast<bf16x8*>(dst) = o;
}

__device__ __forceinline__ void st8_zero(__bf16* dst) {
    *reinterpret_cast<u16x8*>(dst) = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
}

// Rotation of one column pair group: columns n (first half) and N/2 + n.
__device__ __forceinline__ void rotate8(float a[8], float e[8], int col0, int W, const float* cs,
                                        const float* sn) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int n = col0 + j;
        if (n < W) {
            const float c = cs[n], s = sn[n];
            const float x = a[j], y = e[j];
            a[j] = bfr(__fmul_rn(c, x) - __fmul_rn(s, y));
            e[j] = bfr(__fmul_rn(s, x) + __fmul_rn(c, y));
        }
    }
}

// ---------------------------------------------------------------- Psi^T fill
// sPsiT[p][r*Cp + t] = bf16(v[t,p] * bf16(mimo_v[r,p])), zero for padded
// tokens, ranks, rows and value columns.
template <int MT, int PT, int NTHR>
__device__ __forceinline__ void fill_psi(const Params& p, int b, int h, int c0, int cl, __bf16* sPsiT,
                                         int lda) {
    const int tid = threadIdx.x;
    constexpr int P8 = PT / 8;
    const int nit = p.Cp * P8;
    for (int it = tid; it < nit; it += NTHR) {
        const int t = it / P8, pc = (it - t * P8) * 8;
        const bool real = t < cl && pc < p.P;
        float vv[8];
        if (real) {
            const u16x8 x = ld8(p.v + ((long)(b * p.S + c0 + t) * p.H + h) * p.P + pc);
#pragma unroll
            for (int e = 0; e < 8; ++e) vv[e] = bf2f(x[e]);
        }
        for (int r = 0; r < p.R; ++r) {
            float mv[8];
            if (real) {
                const float* src = p.mimo_v + ((long)h * p.R + r) * p.P + pc;
                const float4 m0 = *reinterpret_cast<const float4*>(src);
                const float4 m1 = *reinterpret_cast<const float4*>(src + 4);
                mv[0] = m0.x; mv[1] = m0.y; mv[2] = m0.z; mv[3] = m0.w;
                mv[4] = m1.x; mv[5] = m1.y; mv[6] = m1.z; mv[7] = m1.w;
            }
            const int col = r * p.Cp + t;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                sPsiT[(pc + e) * lda + col] = static_cast<__bf16>(real ? bfr(vv[e] * bfr(mv[e])) : 0.f);
        }
    }
    // rows of the tile beyond R*Cp
    const int used = p.R * p.Cp;
    const int pad = MT - used;
    if (pad > 0) {
        for (int it = tid; it < PT * pad; it += NTHR) {
            const int pp = it / pad, i = used + (it - pp * pad);
            sPsiT[pp * lda + i] = static_cast<__bf16>(0.f);
        }
    }
}

// ---------------------------------------------------------------- segment aggregate
// U_s = state added by segment s from a zero start: U <- U*exp(da_cs[last]) + kappa^T Psi
// per chunk. Also the product of the chunk decays.
template <int MT, int NT, int PT, int NW>
__global__ __launch_bounds__(NW * 64) void k_agg(Params p) {
    constexpr int NTHR = NW * 64;
    constexpr int NG_MAX = NT / 16;
    constexpr int QK_IT = (MT * NG_MAX + NTHR - 1) / NTHR;
    constexpr int ST = (NT / 16) * (PT / 16);
    constexpr int STW = (ST + NW - 1) / NW;
    extern __shared__ __align__(16) unsigned char smem[];
    const Lds L = lds_layout(MT, NT, PT, p.C, p.R, p.W, false);
    __bf16* sKapT = reinterpret_cast<__bf16*>(smem + L.r1);
    __bf16* sPsiT = reinterpret_cast<__bf16*>(smem + L.r3);
    float* scs = reinterpret_cast<float*>(smem + L.sm1);
    float* sc = reinterpret_cast<float*>(smem + L.sc);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int seg = blockIdx.x, bh = blockIdx.y;
    const int b = bh / p.H, h = bh - b * p.H;
    const int g = h / (p.H / p.G);
    const int c_begin = seg * p.L;
    const int c_end = min(c_begin + p.L, p.nc);
    const int lda = L.lda;
    const int l16 = lane & 15, q4 = lane >> 4;

    f32x4 U[STW];
#pragma unroll
    for (int w = 0; w < STW; ++w) U[w] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dprod = 1.f;

    for (int c = c_begin; c < c_end; ++c) {
        const int c0 = c * p.C;
        const int cl = min(p.C, p.S - c0);
        prep_scalars<NTHR>(p, bh, b, h, c0, cl, sc, scs, false);
        __syncthreads();
        const float* s_erev = sc + 2 * kMaxRows;
        const float* s_fac = sc + 3 * kMaxRows;
        const float dl = sc[4 * kMaxRows];
        // kappa^T: rotated k, times factor (bf16), times exp(da_cs_rev) (bf16), transposed.
        const int ng = p.N / 16;
        const int nit = MT * ng;
#pragma unroll
        for (int j = 0; j < QK_IT; ++j) {
            const int it = tid + j * NTHR;
            if (it < nit) {
                const int i = it / ng, gg = it - i * ng;
                const int r = i / p.Cp, t = i - r * p.Cp;
                const int col0 = gg * 8, col1 = p.N / 2 + gg * 8;
                float ka[8], kb[8];
                if (r < p.R && t < cl) {
                    const long row = (((long)(b * p.S + c0 + t) * p.R + r) * p.G + g) * p.N;
                    const float* kbias = p.k_bias + ((long)h * p.R + r) * p.N;
                    bias8(ld8(p.k + row + col0), kbias + col0, ka);
                    bias8(ld8(p.k + row + col1), kbias + col1, kb);
                    rotate8(ka, kb, col0, p.W, scs + t * p.W, scs + p.C * p.W + t * p.W);
                    const float f = s_fac[t], er = s_erev[t];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        ka[e] = bfr(bfr(ka[e] * f) * er);
                        kb[e] = bfr(bfr(kb[e] * f) * er);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) ka[e] = kb[e] = 0.f;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sKapT[(col0 + e) * lda + i] = static_cast<__bf16>(ka[e]);
                    sKapT[(col1 + e) * lda + i] = static_cast<__bf16>(kb[e]);
                }
            }
        }
        // state columns beyond N
        for (int it = tid; it < (NT - p.N) * MT; it += NTHR) {
            const int n = p.N + it / MT, i = it % MT;
            sKapT[n * lda + i] = static_cast<__bf16>(0.f);
        }
        fill_psi<MT, PT, NTHR>(p, b, h, c0, cl, sPsiT, lda);
        __syncthreads();
#pragma unroll
        for (int w = 0; w < STW; ++w) {
            const int u = wave + w * NW;
            if (u < ST) {
                const int nt = u / (PT / 16), pt = u - nt * (PT / 16);
                f32x4 acc = U[w] * dl;
#pragma unroll
                for (int ks = 0; ks < MT / 32; ++ks) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(sKapT + (16 * nt + l16) * lda + 32 * ks + 8 * q4);
                    const bf16x8 bb = *reinterpret_cast<const bf16x8*>(sPsiT + (16 * pt + l16) * lda + 32 * ks + 8 * q4);
                    acc = mfma(a, bb, acc);
                }
                U[w] = acc;
            }
        }
        dprod *= dl;
        __syncthreads();
    }
    float* out = p.agg + ((long)bh * (p.nseg - 1) + seg) * p.N * p.P;
#pragma unroll
    for (int w = 0; w < STW; ++w) {
        const int u = wave + w * NW;
        if (u < ST) {
            const int nt = u / (PT / 16), pt = u - nt * (PT / 16);
            const int pc = 16 * pt + l16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int n = 16 * nt + 4 * q4 + v;
                if (n < p.N && pc < p.P) out[(long)n * p.P + pc] = U[w][v];
            }
        }
    }
    if (tid == 0) p.decay[(long)bh * p.nseg + seg] = dprod;
}

// ---------------------------------------------------------------- main chunk pass
// Template: RP = rank count rounded up to a power of two (ranks >= R are zero
// rows), CT = 16-token tiles per rank (Cp = 16*CT >= C), NT / PT = state and
// value dimensions rounded up to 32 / 64 / 128.
template <int RP, int CT, int NT, int PT>
struct MainCfg {
    static constexpr int MT = (RP * CT * 16 < 32) ? 32 : RP * CT * 16;
    static constexpr int NW = (MT == 128 && PT >= 64) ? 8 : 4;
};

template <int RP, int CT, int NT, int PT>
__global__ __launch_bounds__((MainCfg<RP, CT, NT, PT>::NW * 64), 2) void k_main(Params p) {
    constexpr int MT = MainCfg<RP, CT, NT, PT>::MT;
    constexpr int NW = MainCfg<RP, CT, NT, PT>::NW;
    constexpr int NTHR = NW * 64;
    constexpr int Cp = CT * 16;
    constexpr int QK_IT = (MT * (NT / 16) + NTHR - 1) / NTHR;  // q/k prep items per thread (bound)
    constexpr int PTT = PT / 16;
    constexpr int ST = (NT / 16) * PTT;                         // state tiles
    constexpr int STW = (ST + NW - 1) / NW;
    constexpr int MTT = MT / 16;
    constexpr int AT = MTT * MTT;                               // causal-block tiles
    constexpr int ATW = (AT + NW - 1) / NW;
    constexpr int NPAIRS = CT * PTT;                            // (token tile, value tile) pairs
    constexpr int PW = (NPAIRS + NW - 1) / NW;                  // pairs per wave

    extern __shared__ __align__(16) unsigned char smem[];
    const Lds L = lds_layout(MT, NT, PT, p.C, p.R, p.W, true);
    __bf16* sQ = reinterpret_cast<__bf16*>(smem + L.r1);     // also sA, sKapT
    __bf16* sA = sQ;
    __bf16* sKapT = sQ;
    __bf16* sK = reinterpret_cast<__bf16*>(smem + L.r2);
    __bf16* sPsiT = reinterpret_cast<__bf16*>(smem + L.r3);
    __bf16* sSbT = reinterpret_cast<__bf16*>(smem + L.r4);
    float* scs = reinterpret_cast<float*>(smem + L.sm1);     // cos/sin, then exp(segsum)
    float* sE = scs;
    float* sQK = reinterpret_cast<float*>(smem + L.sqk);
    float* sc = reinterpret_cast<float*>(smem + L.sc);
    const float* s_ecs = sc;
    const float* s_gam = sc + kMaxRows;
    const float* s_erev = sc + 2 * kMaxRows;
    const float* s_fac = sc + 3 * kMaxRows;
    constexpr int ldq = NT + 8, lda = MT + 8;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int seg = blockIdx.x, bh = blockIdx.y;
    const int b = bh / p.H, h = bh - b * p.H;
    const int g = h / (p.H / p.G);
    const int c_begin = seg * p.L;
    const int c_end = min(c_begin + p.L, p.nc);
    const int R = p.R;

    // ---- state entering the segment (fp32, MFMA accumulator layout: rows n, columns p)
    f32x4 Sacc[STW];
    {
        const float* E = (seg > 0) ? p.agg + ((long)bh * (p.nseg - 1) + seg - 1) * p.N * p.P : nullptr;
#pragma unroll
        for (int w = 0; w < STW; ++w) {
            const int u = wave + w * NW;
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
            if (E != nullptr && u < ST) {
                const int nt = u / PTT, pt = u % PTT;
                const int pc = 16 * pt + l16;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int n = 16 * nt + 4 * q4 + v;
                    if (n < p.N && pc < p.P) s[v] = E[(long)n * p.P + pc];
                }
            }
            Sacc[w] = s;
        }
    }
    // bf16(S) into sSbT (operand of the next inter term) and into states[c]
    auto emit_state = [&](int c) {
        unsigned short* dst = p.states + ((long)bh * p.nc + c) * p.N * p.P;
#pragma unroll
        for (int w = 0; w < STW; ++w) {
            const int u = wave + w * NW;
            if (u < ST) {
                const int nt = u / PTT, pt = u % PTT;
                const int pc = 16 * pt + l16;
                bf16x4 o;
#pragma unroll
                for (int v = 0; v < 4; ++v) o[v] = static_cast<__bf16>(Sacc[w][v]);
                *reinterpret_cast<bf16x4*>(sSbT + pc * ldq + 16 * nt + 4 * q4) = o;
                if (pc < p.P) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int n = 16 * nt + 4 * q4 + v;
                        if (n < p.N) dst[(long)n * p.P + pc] = f2bf(Sacc[w][v]);
                    }
                }
            }
        }
    };
    emit_state(c_begin);

    // ---- per-lane constants of this wave's output tiles: slot (ps, r) is
    // value tile pt of pair wave + ps*NW, rank r; lane column pc = 16*pt + l16.
    float cz[PW][RP], co[PW][RP], dmo[PW][RP], dmz[PW][RP];
#pragma unroll
    for (int ps = 0; ps < PW; ++ps) {
        const int pair = wave + ps * NW;
        const int pc = 16 * (pair % PTT) + l16;
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            cz[ps][r] = co[ps][r] = dmo[ps][r] = dmz[ps][r] = 0.f;
            if (pair < NPAIRS && r < R && pc < p.P) {
                if (p.has_z) cz[ps][r] = p.mimo_z[((long)h * R + r) * p.P + pc];
                if (p.reduce_o) co[ps][r] = bfr(p.mimo_o[((long)h * R + r) * p.P + pc]);
            }
        }
    }
    const float dval = p.has_d ? p.d[h] : 0.f;

    for (int c = c_begin; c < c_end; ++c) {
        const int c0 = c * p.C;
        const int cl = min(p.C, p.S - c0);

        // ---- phase 0: per-token scalars, cos/sin
        prep_scalars<NTHR>(p, bh, b, h, c0, cl, sc, scs, true);
        __syncthreads();

        // ---- phase A: biased q/k (unrotated into LDS, rotated kept in registers), Psi^T
        const int ng = p.N / 16;
        const int nit = MT * ng;
        bf16x8 rq0[QK_IT], rq1[QK_IT], rk0[QK_IT], rk1[QK_IT];
#pragma unroll
        for (int j = 0; j < QK_IT; ++j) {
            const int it = tid + j * NTHR;
            if (it < nit) {
                const int i = it / ng, gg = it - i * ng;
                const int r = i / Cp, t = i % Cp;
                const int col0 = gg * 8, col1 = p.N / 2 + gg * 8;
                float qa[8], qb[8], ka[8], kb[8];
                if (r < R && t < cl) {
                    const long row = (((long)(b * p.S + c0 + t) * R + r) * p.G + g) * p.N;
                    const float* qbias = p.q_bias + ((long)h * R + r) * p.N;
                    const float* kbias = p.k_bias + ((long)h * R + r) * p.N;
                    bias8(ld8(p.q + row + col0), qbias + col0, qa);
                    bias8(ld8(p.q + row + col1), qbias + col1, qb);
                    bias8(ld8(p.k + row + col0), kbias + col0, ka);
                    bias8(ld8(p.k + row + col1), kbias + col1, kb);
                    st8(sQ + i * ldq + col0, qa);
                    st8(sQ + i * ldq + col1, qb);
                    st8(sK + i * ldq + col0, ka);
                    st8(sK + i * ldq + col1, kb);
                    const float* cs = scs + t * p.W;
                    const float* sn = scs + p.C * p.W + t * p.W;
                    rotate8(qa, qb, col0, p.W, cs, sn);
                    rotate8(ka, kb, col0, p.W, cs, sn);
                    const float f = s_fac[t];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        ka[e] = bfr(ka[e] * f);
                        kb[e] = bfr(kb[e] * f);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) qa[e] = qb[e] = ka[e] = kb[e] = 0.f;
                    st8_zero(sQ + i * ldq + col0);
                    st8_zero(sQ + i * ldq + col1);
                    st8_zero(sK + i * ldq + col0);
                    st8_zero(sK + i * ldq + col1);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    rq0[j][e] = static_cast<__bf16>(qa[e]);
                    rq1[j][e] = static_cast<__bf16>(qb[e]);
                    rk0[j][e] = static_cast<__bf16>(ka[e]);
                    rk1[j][e] = static_cast<__bf16>(kb[e]);
                }
            }
        }
        // state columns beyond N are zero in both operands of the n-contractions
        if (p.N < NT) {
            const int zc = (NT - p.N) / 8;
            for (int it = tid; it < MT * zc; it += NTHR) {
                const int i = it / zc, col = p.N + 8 * (it - i * zc);
                st8_zero(sQ + i * ldq + col);
                st8_zero(sK + i * ldq + col);
            }
        }
        fill_psi<MT, PT, NTHR>(p, b, h, c0, cl, sPsiT, lda);
        __syncthreads();

        // ---- phase B: qk_dot (same token, unrotated) and exp(segsum)
        {
            const int RR = R * R;
            const int nq = cl * RR;
            for (int it = tid; it < nq; it += NTHR) {
                const int t = it / RR, rr = it - t * RR;
                const int r = rr / R, r2 = rr - r * R;
                const __bf16* xq = sQ + (r * Cp + t) * ldq;
                const __bf16* xk = sK + (r2 * Cp + t) * ldq;
                float sum = 0.f;
                for (int n = 0; n < p.N; n += 8) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(xq + n);
                    const bf16x8 bb = *reinterpret_cast<const bf16x8*>(xk + n);
#pragma unroll
                    for (int e = 0; e < 8; ++e) sum += bfv(a[e]) * bfv(bb[e]);
                }
                const float vq = bfr(sum);
                sQK[it] = vq;
                p.qk_dot[(((long)bh * p.S + c0 + t) * R + r) * R + r2] = f2bf(vq);
            }
            if (p.need_y) {
                const float* sg = p.segsum + ((long)bh * p.nc + c) * p.C * p.C;
                for (int e = tid; e < p.C * p.C; e += NTHR) sE[e] = expf(sg[e]);
            }
        }
        __syncthreads();

        // ---- phase C: rotated q and factor-scaled k into LDS
#pragma unroll
        for (int j = 0; j < QK_IT; ++j) {
            const int it = tid + j * NTHR;
            if (it < nit) {
                const int i = it / ng, gg = it - i * ng;
                const int col0 = gg * 8, col1 = p.N / 2 + gg * 8;
                if (p.need_y) {
                    *reinterpret_cast<bf16x8*>(sQ + i * ldq + col0) = rq0[j];
                    *reinterpret_cast<bf16x8*>(sQ + i * ldq + col1) = rq1[j];
                }
                *reinterpret_cast<bf16x8*>(sK + i * ldq + col0) = rk0[j];
                *reinterpret_cast<bf16x8*>(sK + i * ldq + col1) = rk1[j];
            }
        }
        __syncthreads();

        f32x4 acc[PW][RP];
        if (p.need_y) {
            // ---- inter = Q bf16(S), scaled by exp(da_cs[t]) per row
#pragma unroll
            for (int ps = 0; ps < PW; ++ps) {
                const int pair = wave + ps * NW;
                const int tt = pair / PTT, pt = pair % PTT;
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
                    if (pair < NPAIRS && r < R) {
                        const int it16 = r * CT + tt;
#pragma unroll
                        for (int ks = 0; ks < NT / 32; ++ks) {
                            const bf16x8 a = *reinterpret_cast<const bf16x8*>(sQ + (16 * it16 + l16) * ldq + 32 * ks + 8 * q4);
                            const bf16x8 bb = *reinterpret_cast<const bf16x8*>(sSbT + (16 * pt + l16) * ldq + 32 * ks + 8 * q4);
                            a4 = mfma(a, bb, a4);
                        }
#pragma unroll
                        for (int v = 0; v < 4; ++v) a4[v] *= s_ecs[16 * tt + 4 * q4 + v];
                    }
                    acc[ps][r] = a4;
                }
            }
            // ---- causal block A^T = K~ Q^T, masked on token index, times exp(segsum), bf16
            bf16x4 at[ATW];
#pragma unroll
            for (int w = 0; w < ATW; ++w) {
                const int u = wave + w * NW;
                at[w] = bf16x4{};
                const int jt = u / MTT, it16 = u % MTT;
                const int ri = it16 / CT, rj = jt / CT;
                const int tti = it16 % CT, ttj = jt % CT;
                if (u < AT && ri < R && rj < R && ttj <= tti) {
                    f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < NT / 32; ++ks) {
                        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + (16 * jt + l16) * ldq + 32 * ks + 8 * q4);
                        const bf16x8 bb = *reinterpret_cast<const bf16x8*>(sQ + (16 * it16 + l16) * ldq + 32 * ks + 8 * q4);
                        a4 = mfma(a, bb, a4);
                    }
                    const int ti = 16 * tti + l16;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int tj = 16 * ttj + 4 * q4 + v;
                        const bool keep = ti < cl && ti > tj;
                        const float e = keep ? sE[ti * p.C + tj] : 0.f;
                        at[w][v] = static_cast<__bf16>(keep ? a4[v] * e : 0.f);
                    }
                }
            }
            __syncthreads();   // every wave is done reading sQ
#pragma unroll
            for (int w = 0; w < ATW; ++w) {
                const int u = wave + w * NW;
                if (u < AT) {
                    const int jt = u / MTT, it16 = u % MTT;
                    *reinterpret_cast<bf16x4*>(sA + (16 * it16 + l16) * lda + 16 * jt + 4 * q4) = at[w];
                }
            }
            __syncthreads();
            // ---- intra = A Psi, accumulated onto the scaled inter term
#pragma unroll
            for (int ps = 0; ps < PW; ++ps) {
                const int pair = wave + ps * NW;
                const int tt = pair / PTT, pt = pair % PTT;
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    if (pair < NPAIRS && r < R) {
                        const int it16 = r * CT + tt;
                        f32x4 a4 = acc[ps][r];
#pragma unroll
                        for (int ks = 0; ks < MT / 32; ++ks) {
                            const bf16x8 a = *reinterpret_cast<const bf16x8*>(sA + (16 * it16 + l16) * lda + 32 * ks + 8 * q4);
                            const bf16x8 bb = *reinterpret_cast<const bf16x8*>(sPsiT + (16 * pt + l16) * lda + 32 * ks + 8 * q4);
                            a4 = mfma(a, bb, a4);
                        }
                        acc[ps][r] = a4;
                    }
                }
            }
            __syncthreads();   // every wave is done reading sA
        }

        // ---- kappa^T = bf16(K~ * exp(da_cs_rev)), transposed, into R1
        {
            constexpr int n8 = NT / 8;
            for (int it = tid; it < MT * n8; it += NTHR) {
                const int i = it / n8, nn = (it % n8) * 8;
                const int r = i / Cp, t = i % Cp;
                const bf16x8 x = *reinterpret_cast<const bf16x8*>(sK + i * ldq + nn);
                const float er = (r < R && t < cl) ? s_erev[t] : 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) sKapT[(nn + e) * lda + i] = static_cast<__bf16>(bfv(x[e]) * er);
            }
        }
        __syncthreads();

        // ---- state update S <- S * exp(da_cs[last]) + kappa^T Psi; bf16 copy for the next chunk
        {
            const float dl = sc[4 * kMaxRows];
#pragma unroll
            for (int w = 0; w < STW; ++w) {
                const int u = wave + w * NW;
                if (u < ST) {
                    const int nt = u / PTT, pt = u % PTT;
                    f32x4 a4 = Sacc[w] * dl;
#pragma unroll
                    for (int ks = 0; ks < MT / 32; ++ks) {
                        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sKapT + (16 * nt + l16) * lda + 32 * ks + 8 * q4);
                        const bf16x8 bb = *reinterpret_cast<const bf16x8*>(sPsiT + (16 * pt + l16) * lda + 32 * ks + 8 * q4);
                        a4 = mfma(a, bb, a4);
                    }
                    Sacc[w] = a4;
                }
            }
            if (c + 1 < c_end) emit_state(c + 1);
        }

        // ---- y = bf16(inter + intra + diag + d*Psi) and the gating gradients
        if (p.need_y) {
#pragma unroll
            for (int ps = 0; ps < PW; ++ps) {
                const int pair = wave + ps * NW;
                if (pair >= NPAIRS) continue;
                const int tt = pair / PTT, pt = pair % PTT;
                const int pc = 16 * pt + l16;
                const int tb = 16 * tt + 4 * q4;   // first of this lane's 4 tokens
                float psi[RP][4];
#pragma unroll
                for (int r2 = 0; r2 < RP; ++r2) {
                    if (r2 < R) {
                        const bf16x4 x = *reinterpret_cast<const bf16x4*>(sPsiT + pc * lda + r2 * Cp + tb);
#pragma unroll
                        for (int v = 0; v < 4; ++v) psi[r2][v] = bfv(x[v]);
                    } else {
#pragma unroll
                        for (int v = 0; v < 4; ++v) psi[r2][v] = 0.f;
                    }
                }
                float zv[4], dov[4], dzc[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    dzc[v] = zv[v] = dov[v] = 0.f;
                    const int t = tb + v;
                    if (t < cl && pc < p.P) {
                        const long ivp = ((long)(b * p.S + c0 + t) * p.H + h) * p.P + pc;
                        if (p.has_z) zv[v] = bf2f(p.z[ivp]);
                        if (p.reduce_o) dov[v] = bf2f(p.dout[ivp]);
                    }
                }
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    if (r >= R) continue;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int t = tb + v;
                        const bool real = t < cl && pc < p.P;
                        // diagonal: rank-ordered bf16 products and sums, times gamma
                        const float* qkrow = sQK + (t * R + r) * R;
                        float dg = 0.f;
#pragma unroll
                        for (int r2 = 0; r2 < RP; ++r2) {
                            if (r2 < R) {
                                const float qk = real ? qkrow[r2] : 0.f;
                                dg = bfr(dg + bfr(qk * psi[r2][v]));
                            }
                        }
                        dg = bfr(dg * s_gam[t]);
                        float o = acc[ps][r][v] + dg;
                        if (p.has_d) o += dval * psi[r][v];
                        const float y = bfr(o);
                        if (!real) continue;
                        if (p.has_z) {
                            const float pz = zv[v] * cz[ps][r];
                            const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-pz));
                            float G;
                            if (p.reduce_o) {
                                dmo[ps][r] += (y * (pz * sg)) * dov[v];
                                G = bfr(bfr(dov[v] * co[ps][r]) * y);
                            } else {
                                const long inr = (((long)(b * p.S + c0 + t) * R + r) * p.H + h) * p.P + pc;
                                G = bfr(bf2f(p.dout[inr]) * y);
                            }
                            const float gz = (G * sg) * (1.0f + pz * (1.0f - sg));
                            dzc[v] = bfr(dzc[v] + __fmul_rn(gz, cz[ps][r]));
                            dmz[ps][r] += gz * zv[v];
                        } else if (p.reduce_o) {
                            dmo[ps][r] += y * dov[v];
                        }
                    }
                }
                if (p.has_z) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int t = tb + v;
                        if (t < cl && pc < p.P)
                            p.dz[((long)(b * p.S + c0 + t) * p.H + h) * p.P + pc] = f2bf(dzc[v]);
                    }
                }
            }
        }
        __syncthreads();
    }

    // ---- per-segment partial sums of dmimo_o / dmimo_z: reduce over the 4 lane groups
    if (p.need_y) {
#pragma unroll
        for (int ps = 0; ps < PW; ++ps) {
#pragma unroll
            for (int r = 0; r < RP; ++r) {
                float so = dmo[ps][r], sz = dmz[ps][r];
                so += __shfl_xor(so, 16);
                so += __shfl_xor(so, 32);
                sz += __shfl_xor(sz, 16);
                sz += __shfl_xor(sz, 32);
                dmo[ps][r] = so;
                dmz[ps][r] = sz;
            }
        }
        if constexpr (CT == 1) {
#pragma unroll
            for (int ps = 0; ps < PW; ++ps) {
                const int pair = wave + ps * NW;
                const int pc = 16 * (pair % PTT) + l16;
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    if (pair < NPAIRS && r < R && q4 == 0 && pc < p.P) {
                        const long o = ((long)bh * p.nseg + seg) * R * p.P + (long)r * p.P + pc;
                        if (p.reduce_o) p.part_o[o] = dmo[ps][r];
                        if (p.has_z) p.part_z[o] = dmz[ps][r];
                    }
                }
            }
        } else {
            // the token tiles of one (rank, value tile) belong to different waves;
            // add them in token-tile order through LDS
            float* red = reinterpret_cast<float*>(smem);   // [2][CT][RP][PT]
            constexpr int per = RP * PT;
#pragma unroll
            for (int ps = 0; ps < PW; ++ps) {
                const int pair = wave + ps * NW;
                const int tt = pair / PTT, pc = 16 * (pair % PTT) + l16;
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    if (pair < NPAIRS && q4 == 0) {
                        red[tt * per + r * PT + pc] = dmo[ps][r];
                        red[CT * per + tt * per + r * PT + pc] = dmz[ps][r];
                    }
                }
            }
            __syncthreads();
            for (int e = tid; e < R * PT; e += NTHR) {
                const int r = e / PT, pc = e % PT;
                if (pc < p.P) {
                    float so = 0.f, sz = 0.f;
#pragma unroll
                    for (int tt = 0; tt < CT; ++tt) {
                        so += red[tt * per + r * PT + pc];
                        sz += red[CT * per + tt * per + r * PT + pc];
                    }
                    const long o = ((long)bh * p.nseg + seg) * R * p.P + (long)r * p.P + pc;
                    if (p.reduce_o) p.part_o[o] = so;
                    if (p.has_z) p.part_z[o] = sz;
                }
            }
        }
    }
}

typedef void (*kfn)(Params);

// k_agg: indexed by (MT, NT, PT); k_main: indexed by (RP, CT, NT, PT).
template <int MT, int NT, int PT>
kfn agg_for() {
    constexpr int NW = (MT == 128 && PT >= 64) ? 8 : 4;
    return k_agg<MT, NT, PT, NW>;
}

template <int RP, int CT, int NT, int PT>
kfn main_for() {
    return k_main<RP, CT, NT, PT>;
}

// Each returns the 9 kernels of one tile family, indexed 3 * idx(NT) + idx(PT)
// with idx(32, 64, 128) = 0, 1, 2.
#define MIMO_NP_TABLE(F) \
    F(32, 32), F(32, 64), F(32, 128), F(64, 32), F(64, 64), F(64, 128), F(128, 32), F(128, 64), F(128, 128)
const kfn* agg_table_mt32();
const kfn* agg_table_mt64();
const kfn* agg_table_mt128();
#define MIMO_DECL_MAIN(RP, CT) const kfn* main_table_rp##RP##_ct##CT();
MIMO_DECL_MAIN(1, 1) MIMO_DECL_MAIN(1, 2) MIMO_DECL_MAIN(1, 4)
MIMO_DECL_MAIN(2, 1) MIMO_DECL_MAIN(2, 2) MIMO_DECL_MAIN(2, 4)
MIMO_DECL_MAIN(4, 1) MIMO_DECL_MAIN(4, 2) MIMO_DECL_MAIN(8, 1)

}  // namespace mimo
