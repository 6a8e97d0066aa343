// fp32-intermediate chunk kernels: the same chunked MIMO scan as mimo_kernels.hpp
// with every intermediate kept in fp32 and the contractions on fp32 MFMA
// (v_mfma_f32_16x16x4_f32). They serve
//   * the FP32 variant of the backward first stage (Triton-Ascend
//     mamba_mimo_bwd_fwd pull request page, FP32 PyTorch reference: no bf16
//     rounding of any intermediate; outputs cast to their dtypes);
//   * the SISO forward (mamba3_siso_fwd_kernel migration page, "implementation
//     principle"): rank 1, unit value and gate projections, controls derived
//     from the per-token log decay adt, fp16 or bf16 inputs.
// Inputs q, k, v, z, dout are 16-bit (bf16, or fp16 when in_f16); outputs take
// the same 16-bit type (round to nearest even).
//
// Work split as in the bf16 path: k_chunk32<..., false> computes the state each
// sub-segment adds from a zero start (k_scan then chains them), k_chunk32<...,
// true> walks a segment's chunks from its entry state. Rows of a chunk tile are
// rank-major (i = r*Cp + t). MFMA operands come from LDS with the contraction
// index split as k = 16*kt + 4*q4 + v over the four accumulator steps v, so a
// lane reads four consecutive floats of a contraction-contiguous row:
//   inter = Q^ S       A: sQ[i][n]            B: the state tile in registers
//   A     = Q^ K~^T    A: sQ[i][n]            B: sK[j][n]
//   intra = A Psi      A: sA[i][j]            B: sPsi[j][p] (one float per step)
//   S'    = kappa^T Psi A: sK[i][n]*erev[t]   B: sPsi[i][p] (one float per step)
// Wave w owns the value tiles pt = w, w+4 (all state rows and all chunk rows of
// them), so the state a wave reads for the inter term is in its own registers
// and every rank of a (token, column) meets in one lane for the gating sums.
// With 128 chunk rows and N or P of 128 the q^, K~ and Psi tiles need 188 to 225 KB,
// more than a compute unit's LDS: those instances (KG) keep the K~ tile in a
// per-workgroup slot of global scratch (its other uses are unchanged; the chunk
// loop's barriers already order global memory) and the rest in LDS.
#pragma once

#include "mimo_kernels.hpp"

namespace mimo {
namespace f32 {

template <int MT, int NT, int PT>
struct Tile32 {
    static constexpr int NTHR = 256, NW = 4;
    static constexpr int MTT = MT / 16, NTT = NT / 16, PTT = PT / 16;
    static constexpr int PW = PTT >= NW ? PTT / NW : 1;   // value tiles per wave
    static constexpr int CX = MT < 64 ? MT : 64;          // chunk length bound (C <= MT, C <= 64)
    static constexpr int LQ = NT + 4;                     // row pitch (floats) of sQ, sK
    static constexpr int LA = MT + 4;                     // row pitch of the causal block
    static constexpr int LP = PT + 4;                     // row pitch of sPsi (fp32) and of y's partial sums
    static constexpr int LP16 = PT + 8;                   // row pitch of a 16-bit sPsi (unit projections)
    static constexpr int AT = (MTT * MTT + NW - 1) / NW;  // causal-block tiles per wave
};

// LDS layout in bytes (main: with the q tile, the causal block and the tables).
struct Lds32 {
    int q, k, psi, se, qk, sc, total;
};
// uv: unit value projections and controls derived from adt (the SISO forward): Psi is
// v itself, kept in its 16-bit input type, and exp(segsum) comes from the cumulative
// log decays instead of a table.
__host__ __device__ constexpr Lds32 lds32(int MT, int NT, int PT, bool main, bool uv = false, bool kg = false) {
    const int CX = MT < 64 ? MT : 64;
    // q^, then the causal block, then y's partial sums: the widest of the three rows
    const int wq = NT > MT ? (NT > PT ? NT : PT) : (MT > PT ? MT : PT);
    const int qa = main ? 4 * MT * (wq + 4) : 0;
    Lds32 l{0, 0, 0, 0, 0, 0, 0};
    int off = 0;
    l.q = off;
    off += qa;
    l.k = off;
    if (!kg) off += 4 * MT * (NT + 4);
    l.psi = off;
    off += uv ? 2 * MT * (PT + 8) : 4 * MT * (PT + 4);
    l.se = off;
    if (main && !uv) off += 4 * CX * (CX + 1);
    l.qk = off;
    if (main) off += 4 * MT * 8;
    l.sc = off;
    off += 4 * (6 * CX + 4);
    l.total = off;
    return l;
}

template <bool F16>
__device__ __forceinline__ float ld16(const unsigned short* p, long i) {
    const unsigned short x = p[i];
    if constexpr (F16) return static_cast<float>(__builtin_bit_cast(_Float16, x));
    return __uint_as_float(static_cast<unsigned>(x) << 16);
}
template <bool F16>
__device__ __forceinline__ void cvt16x4(u32x2 w, float* out) {
    const unsigned short h[4] = {static_cast<unsigned short>(w[0]), static_cast<unsigned short>(w[0] >> 16),
                                 static_cast<unsigned short>(w[1]), static_cast<unsigned short>(w[1] >> 16)};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        if constexpr (F16)
            out[d] = static_cast<float>(__builtin_bit_cast(_Float16, h[d]));
        else
            out[d] = __uint_as_float(static_cast<unsigned>(h[d]) << 16);
    }
}
template <bool F16>
__device__ __forceinline__ void ld16x4(const unsigned short* p, long i, float* out) {
    cvt16x4<F16>(*reinterpret_cast<const u32x2*>(p + i), out);
}
// fp32 -> 16-bit output, round to nearest even
template <bool F16>
__device__ __forceinline__ unsigned short st16(float x) {
    if constexpr (F16) return __builtin_bit_cast(unsigned short, static_cast<_Float16>(x));
    return static_cast<unsigned short>(pk2(0.f, x) >> 16);
}

__device__ __forceinline__ float sig32(float x) { return 1.0f / (1.0f + expf(-x)); }

// x[v] for a run-time v in [0, 4) by selects (no indexed register access)
__device__ __forceinline__ float pick4(const float* x, int v) {
    return v == 0 ? x[0] : (v == 1 ? x[1] : (v == 2 ? x[2] : x[3]));
}

__device__ __forceinline__ f32x4 mfma32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// MAIN = false: segment aggregate (state increment of a sub-segment from zero and
// its decay product). MAIN = true: the chunk pass (states, qk_dot, y and the
// backward's gating outputs, or the layer output when p.fwd).
// Two workgroups per compute unit where the LDS layout allows it.
template <int MT, int NT, int PT, bool MAIN, bool UV, bool KG = false>
constexpr int wg_per_cu32() {
    return lds32(MT, NT, PT, MAIN, UV, KG).total <= 80 * 1024 ? 2 : 1;
}

// A 16-bit value (bf16, or fp16 when F16) as fp32.
template <bool F16>
__device__ __forceinline__ float cvt16(unsigned short x) {
    if constexpr (F16) return static_cast<float>(__builtin_bit_cast(_Float16, x));
    return __uint_as_float(static_cast<unsigned>(x) << 16);
}

// EX: a shape-exact instance, whose sizes are constants, so that index arithmetic
// folds. EX = 1: the MIMO shape R = 4, C = 16, N = P = 64, rotated width 16 (MT = NT =
// PT = 64); its aggregate is held to four waves per SIMD, 128 VGPRs, since the
// aggregate's grid is sized for four workgroups per CU, which its LDS allows.
// EX = 2: the SISO shape R = 1, C = 64, N = 128 (all of it rotated: width 64),
// P = 64, unit projections (MT = 64, NT = 128, PT = 64).
template <int MT, int NT, int PT, bool MAIN, bool F16, bool UV = false, bool KG = false, int EX = 0>
__global__ __launch_bounds__(256, ((EX == 1 && !MAIN) ? 4 : wg_per_cu32<MT, NT, PT, MAIN, UV, KG>())) void k_chunk32(
    Params pin) {
    static_assert(EX == 0 || (EX == 1 && MT == 64 && NT == 64 && PT == 64 && !UV && !KG) ||
                      (EX == 2 && MT == 64 && NT == 128 && PT == 64 && UV && !KG),
                  "the exact shape's tile");
    Params p = pin;
    if constexpr (EX == 1) {
        p.R = 4;
        p.C = 16;
        p.N = 64;
        p.P = 64;
        p.W = 16;
    } else if constexpr (EX == 2) {
        p.R = 1;
        p.C = 64;
        p.N = 128;
        p.P = 64;
        p.W = 64;
    }
    using T = Tile32<MT, NT, PT>;
    constexpr int NW = T::NW, NTHR = T::NTHR, LQ = T::LQ, LA = T::LA, LP = T::LP, CX = T::CX;
    constexpr int MTT = T::MTT, NTT = T::NTT, PTT = T::PTT, PW = T::PW;
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr Lds32 L = lds32(MT, NT, PT, MAIN, UV, KG);
    float* sQ = reinterpret_cast<float*>(smem + L.q);   // q^ [MT][LQ], then the causal block [MT][LA],
    float* sA = sQ;                                       // then y's partial sums [MT][LP]
    float* sY = sQ;
    // k0, then K~ [MT][LQ] (with KG in this workgroup's scratch slot)
    float* sK = KG ? p.kslots + (long)blockIdx.x * MT * LQ : reinterpret_cast<float*>(smem + L.k);
    float* sPsi = reinterpret_cast<float*>(smem + L.psi); // Psi [MT][LP], or 16-bit [MT][LP16] when UV
    unsigned short* sPsi16 = reinterpret_cast<unsigned short*>(smem + L.psi);
    auto psi_at = [&](int row, int col) -> float {
        if constexpr (UV)
            return cvt16<F16>(sPsi16[row * T::LP16 + col]);
        else
            return sPsi[row * LP + col];
    };
    float* sE = reinterpret_cast<float*>(smem + L.se);    // exp(segsum) [CX][CX+1]
    float* sQK = reinterpret_cast<float*>(smem + L.qk);   // same-token dots [C][R][R]
    float* sc = reinterpret_cast<float*>(smem + L.sc);    // gamma, factor, ecs, erev, cs [CX] each; dl
    float* sGam = sc;
    float* sFac = sc + CX;
    float* sEcs = sc + 2 * CX;
    float* sRev = sc + 3 * CX;
    float* sCs = sc + 4 * CX;
    float* sDl = sc + 6 * CX;

    const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
    const int l16 = lane & 15, q4 = lane >> 4;
    int seg, bh;
    if (!map_block(p, MAIN ? p.nseg : p.nsub, seg, bh)) return;
    seg = uni(seg);
    bh = uni(bh);
    const int b = uni(bh / p.H), h = uni(bh - b * p.H);
    const int g = uni(h / (p.H / p.G));
    const int R = p.R, N = p.N, P = p.P, C = p.C, W = p.W, M = p.N / 2;
    const int Cp = (C + 15) / 16 * 16, CT = Cp / 16;
    int c_begin, c_end;
    if constexpr (MAIN) {
        c_begin = seg * p.L;
        c_end = min(c_begin + p.L, p.nc);
    } else {
        const int La = p.L / p.F;
        c_begin = seg * La;
        c_end = c_begin + La;
    }
    const long tokb = (long)bh * p.S;   // [B,H,S] row of this (batch, head)

    // ---- state entering the segment: wave w holds S[16nt + 4q4 + v][16pt + l16]
    // for its value tiles pt = w + NW*j (all nt)
    f32x4 S[PW][NTT];
#pragma unroll
    for (int j = 0; j < PW; ++j) {
        const int pt = wave + NW * j;
#pragma unroll
        for (int nt = 0; nt < NTT; ++nt) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
            if (MAIN && seg > 0 && pt < PTT) {
                const float* E = p.agg + ((long)bh * p.nsub + seg * p.F - 1) * N * P;
                const int pc = 16 * pt + l16;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int n = 16 * nt + 4 * q4 + v;
                    if (n < N && pc < P) s[v] = E[n * P + pc];
                }
            }
            S[j][nt] = s;
        }
    }
    // per-lane projections of this wave's columns, per rank
    float cz[PW][8], co[PW][8], dmo[PW][8], dmz[PW][8];
#pragma unroll
    for (int j = 0; j < PW; ++j) {
        const int pc = 16 * (wave + NW * j) + l16;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            cz[j][r] = co[j][r] = dmo[j][r] = dmz[j][r] = 0.f;
            if (MAIN && r < R && pc < P && wave + NW * j < PTT) {
                if (p.has_z) cz[j][r] = p.mimo_z ? p.mimo_z[((long)h * R + r) * P + pc] : 1.0f;
                if (p.reduce_o) co[j][r] = p.mimo_o[((long)h * R + r) * P + pc];
            }
        }
    }
    const float dval = (MAIN && p.has_d) ? p.d[h] : 0.f;
    float dprod = 1.f;

    // ---- the unit-projection (SISO) instances take a chunk's inputs into registers
    // first: raw 16-bit q, k, v of the thread's load items, the angles of its rotation
    // items, and (wave 0, lane t = token) the token's controls. With AHEAD (their
    // aggregate, whose chunks are short and load-bound) these are fetched one chunk
    // ahead, issued after the current chunk's rotation and consumed at the start of
    // the next, and the chunk loop's barriers wait for LDS only so that the loads stay
    // in flight through the state update. The other instances load at the point of
    // use (measured: the register fetch costs them occupancy).
    constexpr bool AHEAD = UV && !MAIN;
    auto sync = [] {
        if constexpr (AHEAD)
            bar();
        else
            __syncthreads();
    };
    constexpr int N4 = NT / 4, P4 = PT / 4;
    constexpr int QK_IT = MT * N4 / NTHR, PS_IT = MT * P4 / NTHR;   // exact: MT * NT >= 32 * 32
    constexpr int ROT_IT = MT * (NT / 2) / NTHR;                     // rotation items (t < MT, n < NT/2)
    u32x2 fq[QK_IT], fk[QK_IT], fv[PS_IT];
    float fang[ROT_IT];
    float fx0 = 0.f, fx1 = 0.f, fdt0 = 0.f, ftr0 = 0.f, fdt1 = 0.f, ftr1 = 0.f;
    auto fetch = [&](int cc) {
        if constexpr (!UV) return;
        const int tf = MAIN ? tid_x() : static_cast<int>(threadIdx.x);
        const int c0f = cc * C, clf = min(C, p.S - c0f);
#pragma unroll
        for (int k2 = 0; k2 < ROT_IT; ++k2) {
            const int e = tf + k2 * NTHR;
            const int t = e / (NT / 2), n = e % (NT / 2);
            fang[k2] = (t < clf && n < W) ? p.angles[((long)(b * p.S + c0f + t) * p.H + h) * W + n] : 0.f;
        }
#pragma unroll
        for (int k2 = 0; k2 < QK_IT; ++k2) {
            const int e = tf + k2 * NTHR;
            const int i = e / N4, n = 4 * (e % N4);
            const int r = i / Cp, t = i % Cp;
            fk[k2] = fq[k2] = u32x2{0u, 0u};
            if (r < R && t < clf && n < N) {
                const long src = (((long)(b * p.S + c0f + t) * R + r) * p.G + g) * N + n;
                fk[k2] = *reinterpret_cast<const u32x2*>(p.k + src);
                if (MAIN) fq[k2] = *reinterpret_cast<const u32x2*>(p.q + src);
            }
        }
#pragma unroll
        for (int k2 = 0; k2 < PS_IT; ++k2) {
            const int e = tf + k2 * NTHR;
            const int i = e / P4, pc = 4 * (e % P4);
            const int r = i / Cp, t = i % Cp;
            fv[k2] = u32x2{0u, 0u};
            if (r < R && t < clf && pc < P)
                fv[k2] = *reinterpret_cast<const u32x2*>(p.v + ((long)(b * p.S + c0f + t) * p.H + h) * P + pc);
        }
        if ((tf >> 6) == 0) {
            const int t = tf & 63;
            fx0 = fx1 = fdt0 = ftr0 = fdt1 = ftr1 = 0.f;
            if (t < clf) {
                const long T0 = tokb + c0f + t;
                fx0 = p.adt != nullptr ? p.adt[T0] : p.da_cs[T0];
                if (p.adt == nullptr) fx1 = p.da_cs_rev[T0];
                fdt0 = p.dt[T0];
                ftr0 = p.trapf ? p.trapf[T0] : bf2f(p.trap[T0]);
                if (c0f + t + 1 < p.S) {
                    fdt1 = p.dt[T0 + 1];
                    ftr1 = p.trapf ? p.trapf[T0 + 1] : bf2f(p.trap[T0 + 1]);
                }
            }
        }
    };
    if (AHEAD && c_begin < c_end) fetch(c_begin);

    // Wave priority (chunk passes with two workgroups per CU): a chunk's chain of
    // barrier-separated phases issues at a raised priority, the y epilogue (no barrier
    // until the chunk's end) at the normal one, so that the other workgroup's epilogue
    // fills the chain's gaps instead of delaying it
    constexpr bool PRIO = MAIN && wg_per_cu32<MT, NT, PT, MAIN, UV, KG>() == 2;
    for (int c = c_begin; c < c_end; ++c) {
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
        const int c0 = c * C;
        const int cl = min(C, p.S - c0);
        // The chunk pass runs two workgroups per CU (at most 256 VGPRs): its thread index
        // is made opaque per chunk so that index arithmetic is redone per chunk instead
        // of being held in registers across the loop (which spills).
        const int tid = MAIN ? tid_x() : static_cast<int>(threadIdx.x), lane = tid & 63, l16 = lane & 15,
                  q4 = lane >> 4;
        if constexpr (UV && !AHEAD) fetch(c);

        // ---- states[c] = S entering chunk c, in the output type
        if constexpr (MAIN) {
            if (!p.fwd) {
                unsigned short* dst = p.states + ((long)bh * p.nc + c) * N * P;
#pragma unroll
                for (int j = 0; j < PW; ++j) {
                    const int pc = 16 * (wave + NW * j) + l16;
                    if (wave + NW * j < PTT && pc < P) {
#pragma unroll
                        for (int nt = 0; nt < NTT; ++nt)
#pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                const int n = 16 * nt + 4 * q4 + v;
                                if (n < N) dst[n * P + pc] = st16<F16>(S[j][nt][v]);
                            }
                    }
                }
            }
        }

        // ---- token scalars of the chunk (wave 0, lane t = token)
        if (wave == 0) {
            const int t = lane;
            float cs = 0.f, rev = 0.f;
            if (p.adt != nullptr) {
                // chunk-local inclusive cumulative sum of the log decay
                float a = UV ? fx0 : ((t < cl) ? p.adt[tokb + c0 + t] : 0.f);   // zero past the chunk
#pragma unroll
                for (int o = 1; o < 64; o *= 2) {
                    const float u = __shfl_up(a, o);
                    if (lane >= o) a += u;
                }
                const float last = __shfl(a, cl - 1);
                cs = a;
                rev = last - a;
            } else if (t < cl) {
                cs = UV ? fx0 : p.da_cs[tokb + c0 + t];
                rev = UV ? fx1 : p.da_cs_rev[tokb + c0 + t];
            }
            if (t < CX) {
                float gam = 0.f, fac = 0.f;
                if (t < cl) {
                    const long T0 = tokb + c0 + t;
                    const float dt0 = UV ? fdt0 : p.dt[T0];
                    const float tr0 = UV ? ftr0 : (p.trapf ? p.trapf[T0] : bf2f(p.trap[T0]));
                    gam = dt0 * sig32(tr0);
                    float beta = 0.f;
                    if (c0 + t + 1 < p.S) {
                        const float dt1 = UV ? fdt1 : p.dt[T0 + 1];
                        const float tr1 = UV ? ftr1 : (p.trapf ? p.trapf[T0 + 1] : bf2f(p.trap[T0 + 1]));
                        beta = dt1 * (1.0f - sig32(tr1));
                    }
                    fac = gam + beta;
                }
                sGam[t] = gam;
                sFac[t] = fac;
                sEcs[t] = (t < cl) ? expf(cs) : 0.f;
                sRev[t] = (t < cl) ? expf(rev) : 0.f;
                sCs[t] = cs;
                if (t == cl - 1) sDl[0] = expf(cs);
            }
        }

        // ---- q0, k0 (biased, unrotated) and Psi into LDS (from the fetched values, or
        // loaded here: every load of a thread in flight together); zero outside the
        // problem. The angles of the rotation below are loaded here too.
        float ang[ROT_IT];
        if constexpr (!UV) {
#pragma unroll
            for (int k2 = 0; k2 < ROT_IT; ++k2) {
                const int e = tid + k2 * NTHR;
                const int t = e / (NT / 2), n = e % (NT / 2);
                ang[k2] = (t < cl && n < W) ? p.angles[((long)(b * p.S + c0 + t) * p.H + h) * W + n] : 0.f;
            }
        }
#pragma unroll
        for (int k2 = 0; k2 < QK_IT; ++k2) {
            const int e = tid + k2 * NTHR;
            const int i = e / N4, n = 4 * (e % N4);
            const int r = i / Cp, t = i % Cp;
            float qv[4] = {0.f, 0.f, 0.f, 0.f}, kv[4] = {0.f, 0.f, 0.f, 0.f};
            if (r < R && t < cl && n < N) {
                const long src = (((long)(b * p.S + c0 + t) * R + r) * p.G + g) * N + n;
                if constexpr (UV)
                    cvt16x4<F16>(fk[k2], kv);
                else
                    ld16x4<F16>(p.k, src, kv);
                const float* kb = p.k_bias + ((long)h * R + r) * N + n;
#pragma unroll
                for (int d = 0; d < 4; ++d) kv[d] += kb[d];
                if (MAIN) {
                    if constexpr (UV)
                        cvt16x4<F16>(fq[k2], qv);
                    else
                        ld16x4<F16>(p.q, src, qv);
                    const float* qb = p.q_bias + ((long)h * R + r) * N + n;
#pragma unroll
                    for (int d = 0; d < 4; ++d) qv[d] += qb[d];
                }
            }
            *reinterpret_cast<f32x4*>(sK + i * LQ + n) = f32x4{kv[0], kv[1], kv[2], kv[3]};
            if (MAIN) *reinterpret_cast<f32x4*>(sQ + i * LQ + n) = f32x4{qv[0], qv[1], qv[2], qv[3]};
        }
#pragma unroll
        for (int k2 = 0; k2 < PS_IT; ++k2) {
            const int e = tid + k2 * NTHR;
            const int i = e / P4, pc = 4 * (e % P4);
            const int r = i / Cp;
            if constexpr (UV) {
                *reinterpret_cast<u32x2*>(sPsi16 + i * T::LP16 + pc) = fv[k2];   // zero outside the problem
                continue;
            }
            float x[4] = {0.f, 0.f, 0.f, 0.f};
            const int t = i % Cp;
            if (r < R && t < cl && pc < P) ld16x4<F16>(p.v, ((long)(b * p.S + c0 + t) * p.H + h) * P + pc, x);
            if (p.mimo_v && r < R && pc < P) {
                const float* mv = p.mimo_v + ((long)h * R + r) * P + pc;
#pragma unroll
                for (int d = 0; d < 4; ++d) x[d] *= mv[d];
            }
            *reinterpret_cast<f32x4*>(sPsi + i * LP + pc) = f32x4{x[0], x[1], x[2], x[3]};
        }
        sync();

        // ---- same-token dots of the unrotated q, k (qk_dot) and exp(segsum)
        if constexpr (MAIN) {
            const int RR = R * R;
            for (int e = tid; e < cl * RR; e += NTHR) {
                const int t = e / RR, r = (e % RR) / R, r2 = e % R;
                const float* x = sQ + (r * Cp + t) * LQ;
                const float* y = sK + (r2 * Cp + t) * LQ;
                float s = 0.f;
                for (int n = 0; n < N; n += 4) {
                    const f32x4 a = *reinterpret_cast<const f32x4*>(x + n);
                    const f32x4 bb = *reinterpret_cast<const f32x4*>(y + n);
                    s = __fmaf_rn(a[0], bb[0], s);
                    s = __fmaf_rn(a[1], bb[1], s);
                    s = __fmaf_rn(a[2], bb[2], s);
                    s = __fmaf_rn(a[3], bb[3], s);
                }
                sQK[e] = s;
                if (!p.fwd) p.qk_dot[((long)bh * p.S + c0 + t) * RR + r * R + r2] = st16<F16>(s);
            }
            for (int e = tid; e < (UV || !p.need_y ? 0 : cl * cl); e += NTHR) {
                const int t = e / cl, s2 = e % cl;
                if (s2 < t) {
                    float sg;
                    if (p.adt != nullptr)
                        sg = sCs[t] - sCs[s2];
                    else
                        sg = p.segsum[(((long)bh * p.nc + c) * C + t) * C + s2];
                    sE[t * (CX + 1) + s2] = expf(sg);
                }
            }
        }
        sync();

        // ---- rotation of q and k (pairs n, N/2 + n for n < W) and K~ = k * factor
#pragma unroll
        for (int k2 = 0; k2 < ROT_IT; ++k2) {
            const int e = tid + k2 * NTHR;
            const int t = e / (NT / 2), n = e % (NT / 2);
            if (t >= cl || n >= M) continue;
            const float f = sFac[t];
            float cn = 1.f, sn = 0.f;
            if (n < W) {
                // the chunk pass's code would outgrow the instruction cache with the library
                // path inlined at every unrolled item; the aggregate's does not
                if constexpr (MAIN)
                    sin_cos_ool(UV ? fang[k2] : ang[k2], sn, cn);
                else
                    sin_cos(UV ? fang[k2] : ang[k2], sn, cn);
            }
            for (int r = 0; r < R; ++r) {
                float* kr = sK + (r * Cp + t) * LQ;
                const float ka = kr[n], ke = kr[M + n];
                kr[n] = (cn * ka - sn * ke) * f;
                kr[M + n] = (sn * ka + cn * ke) * f;
                if (MAIN && p.need_y) {   // rotated q serves y only (qk_dot took q0 above)
                    float* qr = sQ + (r * Cp + t) * LQ;
                    const float qa = qr[n], qe = qr[M + n];
                    qr[n] = cn * qa - sn * qe;
                    qr[M + n] = sn * qa + cn * qe;
                }
            }
        }
        // (with AHEAD: the next chunk's inputs, in flight through the state update)
        if (AHEAD && c + 1 < c_end) fetch(c + 1);
        sync();

        f32x4 acc[PW][MTT];
        if constexpr (MAIN) if (p.need_y) {   // y: inter, causal block, intra
            // ---- inter = Q^ S, rows scaled by exp(da_cs[t])
#pragma unroll
            for (int j = 0; j < PW; ++j) {
                const bool own = wave + NW * j < PTT;
#pragma unroll
                for (int it = 0; it < MTT; ++it) {
                    f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
                    if (own && (it / CT) < R) {
#pragma unroll
                        for (int nt = 0; nt < NTT; ++nt) {
                            const f32x4 qa = *reinterpret_cast<const f32x4*>(sQ + (16 * it + l16) * LQ + 16 * nt + 4 * q4);
#pragma unroll
                            for (int v = 0; v < 4; ++v) a4 = mfma32(qa[v], S[j][nt][v], a4);
                        }
                        const int tb = 16 * (it % CT) + 4 * q4;
#pragma unroll
                        for (int v = 0; v < 4; ++v) a4[v] *= (tb + v < CX) ? sEcs[tb + v] : 0.f;
                    }
                    acc[j][it] = a4;
                }
            }
            // ---- causal block A[i][j] = exp(segsum) * (Q^ K~^T)[i][j] for token(j) < token(i)
            f32x4 at[T::AT];
#pragma unroll
            for (int w = 0; w < T::AT; ++w) {
                const int u = wave + NW * w;
                const int it = u / MTT, jt = u % MTT;
                f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
                if (u < MTT * MTT && it / CT < R && jt / CT < R && (jt % CT) <= (it % CT)) {
#pragma unroll
                    for (int nt = 0; nt < NTT; ++nt) {
                        const f32x4 qa = *reinterpret_cast<const f32x4*>(sQ + (16 * it + l16) * LQ + 16 * nt + 4 * q4);
                        const f32x4 kb = *reinterpret_cast<const f32x4*>(sK + (16 * jt + l16) * LQ + 16 * nt + 4 * q4);
#pragma unroll
                        for (int v = 0; v < 4; ++v) a4 = mfma32(qa[v], kb[v], a4);
                    }
                    // lane holds rows 4q4+v of tile it, column l16 of tile jt
                    const int tj = 16 * (jt % CT) + l16;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int ti = 16 * (it % CT) + 4 * q4 + v;
                        if constexpr (UV)
                            a4[v] = (ti < cl && tj < ti) ? a4[v] * expf(sCs[ti] - sCs[tj]) : 0.f;
                        else
                            a4[v] = (ti < cl && tj < ti) ? a4[v] * sE[ti * (CX + 1) + tj] : 0.f;
                    }
                }
                at[w] = a4;
            }
            sync();   // every wave is done reading sQ
#pragma unroll
            for (int w = 0; w < T::AT; ++w) {
                const int u = wave + NW * w;
                if (u < MTT * MTT) {
                    const int it = u / MTT, jt = u % MTT;
#pragma unroll
                    for (int v = 0; v < 4; ++v) sA[(16 * it + 4 * q4 + v) * LA + 16 * jt + l16] = at[w][v];
                }
            }
            sync();
            // ---- intra = A Psi onto the scaled inter term
#pragma unroll
            for (int j = 0; j < PW; ++j) {
                const int pt = wave + NW * j;
                if (pt >= PTT) continue;
#pragma unroll
                for (int it = 0; it < MTT; ++it) {
                    if (it / CT >= R) continue;
                    f32x4 a4 = acc[j][it];
                    for (int jt = 0; jt < MTT; ++jt) {
                        if (jt / CT >= R || (jt % CT) > (it % CT)) continue;
                        const f32x4 aa = *reinterpret_cast<const f32x4*>(sA + (16 * it + l16) * LA + 16 * jt + 4 * q4);
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            a4 = mfma32(aa[v], psi_at(16 * jt + 4 * q4 + v, 16 * pt + l16), a4);
                    }
                    acc[j][it] = a4;
                }
            }
        }

        // ---- state update S <- S * exp(da_cs[last]) + kappa^T Psi, kappa = K~ * exp(da_cs_rev)
        {
            const float dl = sDl[0];
#pragma unroll
            for (int j = 0; j < PW; ++j) {
                const int pt = wave + NW * j;
                if (pt >= PTT) continue;
#pragma unroll
                for (int nt = 0; nt < NTT; ++nt) {
                    f32x4 a4 = S[j][nt] * dl;
                    for (int it = 0; it < MTT; ++it) {
                        if (it / CT >= R) continue;
                        const int tb = 16 * (it % CT) + 4 * q4;
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int row = 16 * it + 4 * q4 + v;
                            const float er = (tb + v < CX) ? sRev[tb + v] : 0.f;
                            a4 = mfma32(sK[row * LQ + 16 * nt + l16] * er, psi_at(row, 16 * pt + l16), a4);
                        }
                    }
                    S[j][nt] = a4;
                }
            }
            dprod *= dl;
        }

        if constexpr (MAIN) if (p.need_y) {
            // ---- y's partial sums (inter + intra) through LDS, so that the epilogue
            // can address them by run-time rank and token
            sync();   // every wave is done reading the causal block
            if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);   // the epilogue at normal priority
#pragma unroll
            for (int j = 0; j < PW; ++j) {
                const int pt = wave + NW * j;
                if (pt >= PTT) continue;
#pragma unroll
                for (int it = 0; it < MTT; ++it) {
                    if (it / CT >= R) continue;
#pragma unroll
                    for (int v = 0; v < 4; ++v) sY[(16 * it + 4 * q4 + v) * LP + 16 * pt + l16] = acc[j][it][v];
                }
            }
            // ---- y = inter + intra + gamma * sum_r2 qk[r][r2] Psi[r2] + d * Psi, then the
            // gating outputs (backward) or the layer output (forward). A lane reads back
            // only what it wrote itself. The gate inputs (z, reduced dout) of a token tile's
            // four tokens are loaded together, in one round trip.
            const int RR = R * R;
#pragma unroll
            for (int j = 0; j < PW; ++j) {
                const int pt = wave + NW * j;
                const int pc = 16 * pt + l16;
                if (pt >= PTT || pc >= P) continue;
                for (int tt = 0; tt < CT; ++tt) {
                    float zpre[4], dpre[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int t = 16 * tt + 4 * q4 + v;
                        const long ivp = ((long)(b * p.S + c0 + t) * p.H + h) * P + pc;
                        zpre[v] = (t < cl && p.has_z) ? ld16<F16>(p.z, ivp) : 0.f;
                        dpre[v] = (t < cl && !p.fwd && p.reduce_o) ? ld16<F16>(p.dout, ivp) : 0.f;
                    }
                    for (int v = 0; v < 4; ++v) {
                        const int t = 16 * tt + 4 * q4 + v;
                        if (t >= cl) continue;
                        const long ivp = ((long)(b * p.S + c0 + t) * p.H + h) * P + pc;
                        const float gam = sGam[t];
                        const float zr = pick4(zpre, v), dv = pick4(dpre, v);
                        float dzs = 0.f, osum = 0.f;
#pragma unroll
                        for (int r = 0; r < 8; ++r) {
                            if (r >= R) break;
                            float dg = 0.f;
                            for (int r2 = 0; r2 < R; ++r2)
                                dg = __fmaf_rn(sQK[t * RR + r * R + r2], psi_at(r2 * Cp + t, pc), dg);
                            const int row = r * Cp + t;
                            const float y = sY[row * LP + pc] + gam * dg + dval * psi_at(row, pc);
                            float pz = 0.f, sg = 0.f, silu = 1.f;
                            if (p.has_z) {
                                pz = zr * cz[j][r];
                                sg = sigmoid_fast(pz);   // hardware exp2 and reciprocal (about 1 ulp each)
                                silu = pz * sg;
                            }
                            if (p.fwd) {
                                if (p.reduce_o) {
                                    osum += co[j][r] * y * silu;
                                } else {
                                    const long oi = ((long)(b * p.S + c0 + t) * R + r) * p.H * P + (long)h * P + pc;
                                    p.o[oi] = st16<F16>(y * silu);
                                }
                                continue;
                            }
                            float G = 0.f;
                            if (p.reduce_o) {
                                dmo[j][r] += y * silu * dv;
                                G = dv * co[j][r] * y;
                            } else if (p.has_z) {
                                const long di = ((long)(b * p.S + c0 + t) * R + r) * p.H * P + (long)h * P + pc;
                                G = ld16<F16>(p.dout, di) * y;
                            }
                            if (p.has_z) {
                                const float gz = G * sg * (1.0f + pz * (1.0f - sg));
                                dzs += gz * cz[j][r];
                                dmz[j][r] += gz * zr;
                            }
                        }
                        if (p.fwd && p.reduce_o) p.o[ivp] = st16<F16>(osum);
                        if (!p.fwd && p.has_z) p.dz[ivp] = st16<F16>(dzs);
                    }
                }
            }
        }
        sync();   // the next chunk overwrites the tiles and tables
    }

    if constexpr (!MAIN) {
        float* out = p.agg + ((long)bh * p.nsub + seg) * N * P;
#pragma unroll
        for (int j = 0; j < PW; ++j) {
            const int pc = 16 * (wave + NW * j) + l16;
            if (wave + NW * j >= PTT || pc >= P) continue;
#pragma unroll
            for (int nt = 0; nt < NTT; ++nt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int n = 16 * nt + 4 * q4 + v;
                    if (n < N) out[n * P + pc] = S[j][nt][v];
                }
        }
        if (tid == 0) p.decay[(long)bh * p.nsub + seg] = dprod;
    } else if (!p.fwd && (p.reduce_o || p.has_z)) {
        // per-segment partial sums of dmimo_o / dmimo_z over this lane group's tokens
#pragma unroll
        for (int j = 0; j < PW; ++j) {
            const int pc = 16 * (wave + NW * j) + l16;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                float so = dmo[j][r], sz = dmz[j][r];
                so += __shfl_xor(so, 16);
                so += __shfl_xor(so, 32);
                sz += __shfl_xor(sz, 16);
                sz += __shfl_xor(sz, 32);
                if (q4 == 0 && r < R && wave + NW * j < PTT && pc < P) {
                    const long o = ((long)bh * p.nseg + seg) * R * P + (long)r * P + pc;
                    if (p.reduce_o) p.part_o[o] = so;
                    if (p.has_z) p.part_z[o] = sz;
                }
            }
        }
    }
}

// Kernel table: [bf16 = 0 / fp16 = 1][9 * idx(MT) + 3 * idx(NT) + idx(PT)] with
// idx(32, 64, 128) = 0, 1, 2; nullptr where the tile's LDS does not fit even with K~
// in scratch. Each MT's
// instances are compiled in a translation unit of their own (tiles_f32_mt*.hip). The
// *_uv tables hold the unit-projection instances (the SISO forward: MT of 32 and 64).
struct F32Set {
    kfn agg[2][27], main[2][27], agg_uv[2][27], main_uv[2][27];
    kfn agg_ex[2], main_ex[2];   // the shape-exact MIMO instances (by input dtype)
    kfn agg_sx[2], main_sx[2];   // the shape-exact SISO instances (by input dtype)
};
struct F32Part {
    kfn agg[2][9], main[2][9], agg_uv[2][9], main_uv[2][9];
    kfn agg_ex[2], main_ex[2];   // MT = 64 only
    kfn agg_sx[2], main_sx[2];   // MT = 64 only
};
const F32Part* f32_part_mt32();
const F32Part* f32_part_mt64();
const F32Part* f32_part_mt128();

// The instance of a tile: all tiles in LDS where they fit, else (not for the unit
// projections) K~ in scratch.
template <int MT, int NT, int PT, bool MAIN, bool UV>
constexpr bool kg32() {
    return lds32(MT, NT, PT, MAIN, UV).total > 160 * 1024;
}
template <int MT, int NT, int PT, bool MAIN, bool F16, bool UV>
constexpr kfn pick32() {
    if constexpr (!kg32<MT, NT, PT, MAIN, UV>())
        return k_chunk32<MT, NT, PT, MAIN, F16, UV>;
    else if constexpr (!UV && lds32(MT, NT, PT, MAIN, UV, true).total <= 160 * 1024)
        return k_chunk32<MT, NT, PT, MAIN, F16, UV, true>;
    else
        return nullptr;
}

#define MIMO_F32_NP(MT, MAIN, F16, UV)                                                                           \
    {pick32<MT, 32, 32, MAIN, F16, UV>(),  pick32<MT, 32, 64, MAIN, F16, UV>(),  pick32<MT, 32, 128, MAIN, F16, UV>(),  \
     pick32<MT, 64, 32, MAIN, F16, UV>(),  pick32<MT, 64, 64, MAIN, F16, UV>(),  pick32<MT, 64, 128, MAIN, F16, UV>(),  \
     pick32<MT, 128, 32, MAIN, F16, UV>(), pick32<MT, 128, 64, MAIN, F16, UV>(), pick32<MT, 128, 128, MAIN, F16, UV>()}
#define MIMO_F32_TABLES(MT, UV)                                                                         \
    {MIMO_F32_NP(MT, false, false, UV), MIMO_F32_NP(MT, false, true, UV)},                             \
        {MIMO_F32_NP(MT, true, false, UV), MIMO_F32_NP(MT, true, true, UV)}
#define MIMO_F32_PART(MT)                                                                               \
    const F32Part* f32_part_mt##MT() {                                                                  \
        static const F32Part part = {MIMO_F32_TABLES(MT, false), {}, {}, {}, {}};                        \
        return &part;                                                                                   \
    }
#define MIMO_F32_PART_UV(MT)                                                                            \
    const F32Part* f32_part_mt##MT() {                                                                  \
        static const F32Part part = {MIMO_F32_TABLES(MT, false), MIMO_F32_TABLES(MT, true), {}, {}, {}, {}}; \
        return &part;                                                                                   \
    }
// MT = 64 with the shape-exact instances
#define MIMO_F32_PART_UV_EX(MT)                                                                         \
    const F32Part* f32_part_mt##MT() {                                                                  \
        static const F32Part part = {MIMO_F32_TABLES(MT, false), MIMO_F32_TABLES(MT, true),              \
                                     {k_chunk32<64, 64, 64, false, false, false, false, 1>,             \
                                      k_chunk32<64, 64, 64, false, true, false, false, 1>},             \
                                     {k_chunk32<64, 64, 64, true, false, false, false, 1>,              \
                                      k_chunk32<64, 64, 64, true, true, false, false, 1>},              \
                                     {k_chunk32<64, 128, 64, false, false, true, false, 2>,             \
                                      k_chunk32<64, 128, 64, false, true, true, false, 2>},             \
                                     {k_chunk32<64, 128, 64, true, false, true, false, 2>,              \
                                      k_chunk32<64, 128, 64, true, true, true, false, 2>}};             \
        return &part;                                                                                   \
    }

}  // namespace f32
}  // namespace mimo
