// Stage-2 backward of the Mamba-3 MIMO scan (mamba3_mimo_bwd_bwd; Triton-Ascend
// pull request page: "practice" document -- cache semantics, the dstates
// recurrence, the gradient groups -- and the migration note's input/output
// table and supported range). With dPhiO the upstream gradient mapped to ranks
// (dout * mimo_o, or the per-rank dout), L = sum dPhiO * y, and per chunk c
// (rows i = (r, t), rank-major i = r*C + t, Q^/K^ rotated, K~ = K^ * factor_t,
// Psi = v * mimo_v, S_c the cached entry state, E[t][s] = exp(segsum[c][t][s])
// for s < t):
//   dS_c      = exp(da_cs[last]) dS_{c+1} + Q^^T (exp(da_cs) dPhiO)      (dS_nc = 0)
//   dP        = dPhiO Psi^T,  A = E (Q^ K~^T),  W = E dP                 (token-masked)
//   dQ^       = exp(da_cs) dPhiO S_c^T + W K~       (+ same-token part, below)
//   dK~       = W^T Q^ + exp(da_cs_rev) Psi dS_{c+1}^T
//   dPsi      = A^T dPhiO + kappa dS_{c+1} + gamma (qk^T dPhiO)_same-token + d dPhiO
//   dqk[t]    = gamma_t dPhiO[t] Psi[t]^T  -> dq0 += dqk k0, dk0 += dqk^T q0, applied in
//               the rotated frame (the rotation is the same for q and k of a token)
// and the per-token partials DDA_CS, DDA_CS_REV, DFACTOR, DGAMMA, DDA, DSSDA and
// DANGLES from the same products. Everything is fp32; every contraction runs on
// fp32 MFMA.
//
// Data tensors (dout, q, k, v, states, qk_dot, trap) are bf16, fp16 or fp32 (the
// page's supported dtypes), converted to fp32 on load; DQ, DK and DV are stored as
// bf16, fp16 or fp32 (round to nearest even).
//
// Two tile geometries. MD = 64 (R*C, N and P up to 64): nine 64 x 64 fp32 tiles
// stay in LDS, one workgroup a compute unit. MD = 128 (any of them up to 128): the
// nine tiles, 128 x 128 each (608 KB together), cannot be held in LDS, so each
// workgroup keeps them in a slot of its own in global scratch (served from the L2
// and the last-level cache), the small per-row tables stay in LDS, and every
// product runs one 16-row block a wave over the whole width. The page's own answer
// to a dstates tile beyond its on-chip budget is the same in kind: dstates in HBM
// scratch, streamed in row blocks (practice document, dstates UB management).
//
// Work split: k_agg2 forms each sub-segment's dS increment from a zero start,
// k_scan_rev chains them from the end of the sequence, k_main2 walks each
// segment's chunks backwards from the dS entering it on the right, k_finish2
// sums the per-segment DMIMO_V and DD partials in segment order.
#pragma once

#include <type_traits>

#include "mimo_kernels.hpp"

namespace mimo {
namespace b2 {

constexpr int NTHR = 512;      // the aggregate
constexpr int NTHR2 = 512;     // the chunk pass (one workgroup per CU: eight waves hide more latency)
constexpr int NTHR1 = 256;     // the reverse scan and the final sums

// element types of the data tensors and of DQ, DK, DV (the ABI's MIMO_DTYPE_* values)
enum { DT_BF16 = 0, DT_F16 = 1, DT_F32 = 2 };

template <int MD>
struct Geo {
    static constexpr int LD = MD + 4;   // row pitch (floats) of every tile: 16-byte rows, 4 (mod 64)
    static constexpr int TILE = MD * LD;
    static constexpr bool WIDE = MD > 64;
    static constexpr int RSW = WIDE ? 1 : 2;   // row-sum partials a product leaves per row
    // big tiles (LDS when MD = 64, the workgroup's scratch slot otherwise)
    static constexpr int QH = 0, KH = TILE, PS = 2 * TILE, DPO = 3 * TILE, SC = 4 * TILE, DS = 5 * TILE,
                         AM = 6 * TILE, WM = 7 * TILE, OUT = 8 * TILE, MAIN_TILES = 9 * TILE;
    static constexpr int A_QH = 0, A_DPO = TILE, A_U = 2 * TILE, AGG_TILES = 3 * TILE;
    // small per-row tables (LDS, after the tiles when those are in LDS): gamma, factor,
    // exp(da_cs), exp(da_cs_rev) per row; a reduction scratch; the same-token tables
    // [C][R][R] (dots, cached qk_dot); two sets of row-sum partials [RSW][MD]
    static constexpr int GAM = 0, FAC = GAM + MD, ECS = FAC + MD, EREV = ECS + MD, RED = EREV + MD,
                         DQK = RED + 8, QKC = DQK + 8 * MD, RS0 = QKC + 8 * MD, RS1 = RS0 + 2 * MD,
                         SMALL = RS1 + 2 * MD;
    // MD = 128: after the small tables, LDS-resident tiles: W, then the output tile
    // (the two most used of the chunk pass's nine); U in the aggregate
    static constexpr int W_LDS = SMALL, OUT_LDS = SMALL + TILE, U_LDS = SMALL;
    static constexpr int LDS_MAIN = (WIDE ? 2 * TILE : MAIN_TILES) + SMALL;   // floats
    static constexpr int LDS_AGG = (WIDE ? TILE : AGG_TILES) + SMALL;
};

struct Params2 {
    int B, S, H, G, R, N, P, C, W, nc, L, nseg, F, nsub, reduce_o, has_d, out_dt;
    const void *dout, *q, *k, *v, *states, *qk_dot, *trap;   // data dtype (template IT)
    const float *q_bias, *k_bias, *mimo_v, *mimo_o, *da_cs, *da_cs_rev, *dt, *segsum, *angles, *d;
    void *dq, *dk, *dv;   // bf16, fp16 or fp32 (out_dt)
    float *dmimo_v, *dangles, *dfactor, *dgamma, *dda, *dssda, *dda_cs_rev, *dda_cs, *dd;
    float* agg;       // [B*H][nsub][N*P] sub-segment dS increments, then dS at segment boundaries
    float* decay;     // [B*H][nsub] products of the chunk state decays
    float* part_mv;   // [B*H][nseg][R*P] per-segment DMIMO_V partials
    float* part_d;    // [B*H][nseg] per-segment DD partials
    float* slots;     // MD = 128: per-workgroup tile slots (one per block of the launch)
};

// ---------------------------------------------------------------- data loads and stores
__device__ __forceinline__ float h16f(unsigned w, int hi) {
    const unsigned short s = static_cast<unsigned short>(hi ? (w >> 16) : (w & 0xffffu));
    return static_cast<float>(__builtin_bit_cast(_Float16, s));
}
template <int IT>
__device__ __forceinline__ float half_of(unsigned w, int hi) {
    if constexpr (IT == DT_F16)
        return h16f(w, hi);
    else
        return hi ? hi16(w) : lo16(w);
}

// four / eight consecutive data elements as loaded
template <int IT>
struct V4 {
    u32x2 w;
    __device__ float operator[](int v) const { return half_of<IT>(w[v >> 1], v & 1); }
};
template <>
struct V4<DT_F32> {
    f32x4 w;
    __device__ float operator[](int v) const { return w[v]; }
};
template <int IT>
struct V8 {
    u32x4 w;
    __device__ float operator[](int v) const { return half_of<IT>(w[v >> 1], v & 1); }
};
template <>
struct V8<DT_F32> {
    f32x4 lo, hi;
    __device__ float operator[](int v) const { return v < 4 ? lo[v] : hi[v - 4]; }
};

// element offset i is a multiple of 4 (ld4) or 8 (ld8); rows start 16-byte aligned
template <int IT>
__device__ __forceinline__ V4<IT> ld4(const void* base, long i) {
    V4<IT> r;
    if constexpr (IT == DT_F32)
        r.w = *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + i);
    else
        r.w = *reinterpret_cast<const u32x2*>(static_cast<const unsigned short*>(base) + i);
    return r;
}
template <int IT>
__device__ __forceinline__ V8<IT> ld8(const void* base, long i) {
    V8<IT> r;
    if constexpr (IT == DT_F32) {
        r.lo = *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + i);
        r.hi = *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + i + 4);
    } else {
        r.w = *reinterpret_cast<const u32x4*>(static_cast<const unsigned short*>(base) + i);
    }
    return r;
}
template <int IT>
__device__ __forceinline__ V8<IT> zero8() {
    V8<IT> r;
    if constexpr (IT == DT_F32) {
        r.lo = f32x4{0.f, 0.f, 0.f, 0.f};
        r.hi = r.lo;
    } else {
        r.w = u32x4{0u, 0u, 0u, 0u};
    }
    return r;
}
template <int IT>
__device__ __forceinline__ float ld1(const void* base, long i) {
    if constexpr (IT == DT_F32)
        return static_cast<const float*>(base)[i];
    else
        return half_of<IT>(static_cast<const unsigned short*>(base)[i], 0);
}

__device__ __forceinline__ unsigned pkh(float a, float b) {   // two fp16, round to nearest even
    const unsigned short x = __builtin_bit_cast(unsigned short, static_cast<_Float16>(a));
    const unsigned short y = __builtin_bit_cast(unsigned short, static_cast<_Float16>(b));
    return static_cast<unsigned>(x) | (static_cast<unsigned>(y) << 16);
}
// four consecutive outputs at element offset o (a multiple of 4) in the output dtype
__device__ __forceinline__ void store4(void* dst, long o, int odt, float a, float b, float c, float d) {
    if (odt == DT_F32)
        *reinterpret_cast<f32x4*>(static_cast<float*>(dst) + o) = f32x4{a, b, c, d};
    else if (odt == DT_F16)
        *reinterpret_cast<u32x2*>(static_cast<unsigned short*>(dst) + o) = u32x2{pkh(a, b), pkh(c, d)};
    else
        *reinterpret_cast<u32x2*>(static_cast<unsigned short*>(dst) + o) = u32x2{pk2(a, b), pk2(c, d)};
}

template <int MD>
__device__ __forceinline__ void sync() {
    if constexpr (Geo<MD>::WIDE)
        __syncthreads();   // the tiles are in global memory: stores must be visible to the other waves
    else
        bar();
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- products
// C(i, j) = sum_k A(i, k) B(k, j) (* sk[k]) for i < Mi, j < Nj, k < K on fp32 MFMA (16
// x 16 x 4), handing each result to epi(i, j, value). AK1: A(i, k) = A[i*LD + k], else
// A[k*LD + i]; BK1: B(k, j) = B[j*LD + k], else B[k*LD + j]. The contraction index is
// split k = 16 kt + 4 q + v (q = lane / 16, v the accumulation step), so a lane reads
// four consecutive floats of a contraction-contiguous row in one 16-byte load, or one
// float of each of four rows; with LD = 4 (mod 64) neither pattern has LDS bank
// conflicts. Values past K are replaced by zero (the tiles may hold stale data
// there); rows and columns past Mi / Nj are dropped.
// RS: epi returns a term of a row sum; the sums over a wave's columns go to
// rs[g * MD + i], g < RSW one partial per column group (added in a fixed order by
// the reader after a barrier).
//
// MD = 64 (all <= 64, tiles in LDS): the output is 4 x 4 blocks of 16 x 16; of the NT/64
// waves, wave w owns row block w / (4/CW) and the CW = 16 / (NT/64) column blocks from
// CW * (w % (4/CW)). Every operand is read before the first MFMA.
template <int NT, bool AK1, bool BK1, bool SK, bool RS, typename F>
__device__ __forceinline__ void gemm64(int Mi, int Nj, int K, const float* A, const float* B, const float* sk,
                                       F&& epi, float* rs) {
    constexpr int LD = Geo<64>::LD;
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
    if (K & 15) {   // wave-uniform: zero the last step's values past K
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

// MD = 128 (all <= 128; the operands in global scratch or in LDS): eight waves, wave w
// owns row block w and every column block; the contraction runs in 16-wide steps, each
// step's operands loaded just before its MFMAs.
template <int NT, bool AK1, bool BK1, bool SK, bool RS, typename F>
__device__ __forceinline__ void gemm128(int Mi, int Nj, int K, const float* A, const float* B, const float* sk,
                                        F&& epi, float* rs) {
    static_assert(NT == 512, "one 16-row block a wave");
    constexpr int LD = Geo<128>::LD;
    const int tid = tid_x(), w = tid >> 6, x = tid & 15, q = (tid >> 4) & 3;
    const int ncb = (Nj + 15) >> 4, nk = (K + 15) >> 4;
    const int i0 = 16 * w;
    if (i0 >= Mi) return;   // wave-uniform
    f32x4 acc[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
        if (kt >= nk) break;   // wave-uniform
        const int kb = 16 * kt + 4 * q;
        float a[4], bv[8][4];
        if constexpr (AK1) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(A + (i0 + x) * LD + kb);
#pragma unroll
            for (int v = 0; v < 4; ++v) a[v] = t[v];
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) a[v] = A[(kb + v) * LD + i0 + x];
        }
        if constexpr (SK) {
            const f32x4 sc = *reinterpret_cast<const f32x4*>(sk + kb);
#pragma unroll
            for (int v = 0; v < 4; ++v) a[v] *= sc[v];
        }
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
            if (cb >= ncb) break;   // wave-uniform
            const int jb = 16 * cb;
            if constexpr (BK1) {
                const f32x4 t = *reinterpret_cast<const f32x4*>(B + (jb + x) * LD + kb);
#pragma unroll
                for (int v = 0; v < 4; ++v) bv[cb][v] = t[v];
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v) bv[cb][v] = B[(kb + v) * LD + jb + x];
            }
        }
        if (16 * kt + 16 > K) {   // wave-uniform: the last step, partly past K
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const bool in = kb + v < K;
                a[v] = in ? a[v] : 0.f;
#pragma unroll
                for (int cb = 0; cb < 8; ++cb) bv[cb][v] = in ? bv[cb][v] : 0.f;
            }
        }
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
            if (cb >= ncb) break;
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[cb] = mfma_f32(a[v], bv[cb][v], acc[cb]);
        }
    }
    float rsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
        if (cb >= ncb) break;
        const int j = 16 * cb + x;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = i0 + 4 * q + v;
            if (i < Mi && j < Nj) {
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
            for (int v = 0; v < 4; ++v) rs[i0 + 4 * q + v] = rsum[v];
        }
    }
}

template <int MD, int NT, bool AK1, bool BK1, bool SK, bool RS = false, typename F>
__device__ __forceinline__ void gemm(int Mi, int Nj, int K, const float* A, const float* B, const float* sk,
                                     F&& epi, float* rs = nullptr) {
    if constexpr (Geo<MD>::WIDE)
        gemm128<NT, AK1, BK1, SK, RS>(Mi, Nj, K, A, B, sk, epi, rs);
    else
        gemm64<NT, AK1, BK1, SK, RS>(Mi, Nj, K, A, B, sk, epi, rs);
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

// Per-token totals of row sums left by a product (rs[g * MD + i], g < RSW): token t's
// total over its rows r*C + t (r < R), in a fixed order, handed to out(t, total) by
// thread t.
template <int MD, typename O>
__device__ __forceinline__ void token_out(int cl, int R, int C, const float* rs, O&& out) {
    const int t = tid_x();
    if (t < cl) {
        float s = 0.f;
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int g = 0; g < Geo<MD>::RSW; ++g) s += rs[g * MD + r * C + t];
        }
        out(t, s);
    }
}

// e / d and e % d for 0 <= e < 16384 and 1 <= d <= 128 from d's reciprocal: the exact
// quotient of e + 1/2 is at least 1/(2d) >= 1/256 away from an integer and the
// rounded product is off by less than 0.002.
struct DivS {
    int d;
    float rd;
    __device__ explicit DivS(int d_) : d(d_), rd(1.0f / static_cast<float>(d_)) {}
    __device__ int q(int e) const {
        // a divisor the compiler sees as a constant (the shape-exact instances): a shift
        if (__builtin_constant_p(d) && d > 0) return static_cast<int>(static_cast<unsigned>(e) / static_cast<unsigned>(d));
        return static_cast<int>((static_cast<float>(e) + 0.5f) * rd);
    }
    __device__ int r(int e) const { return e - q(e) * d; }
};

// ---------------------------------------------------------------- chunk loads
// Items of the chunk load, a thread's items being e = tid + NT x for x < IX (every
// kind has at most MD * MD / 8 of them):
//   rotation items (i, n4): four columns n4.. of each half (n4 < N/2) of row i of q^
//     (and k^); the thread keeps cos and sin of its columns (1 and 0 where the
//     column is past the rotated width or the row past the chunk) for the output pass;
//   value items (i, p8): eight columns of dPhiO (and Psi) of row i; with MD = 64 the
//     thread keeps its raw v (the rank-0 items' v is the chunk's v);
//   state items: eight consecutive values of the cached state.
// With MD = 64 a thread's items are the same in every chunk, so the biases and
// projections they use are read once (Res), and the loads of a chunk (Fetch) are
// issued a chunk ahead and staged into LDS (rotated, scaled, converted to fp32) at
// the start of the chunk. With MD = 128 (four items of each kind a thread) holding
// all of that would overflow the registers: each item is loaded and staged in one go.
template <int NT, int MD>
struct Items {
    static constexpr int IX = MD * MD / 8 / NT;
    static constexpr int SX = MD * MD / NT;       // segsum values (C * C <= MD * MD)
    static constexpr int DX = MD * MD / 2 / NT;   // angle items (t, n): t < C <= MD, n < W <= MD / 2
    static constexpr int MX = 8 * MD / NT;        // DMIMO_V items (r, p): R * P <= 8 * MD
};
template <int NT, int MD, int IT>
struct Keep {
    float cs[Items<NT, MD>::IX][4], sn[Items<NT, MD>::IX][4];
    V8<IT> v[Items<NT, MD>::IX];
};
struct RRot {
    f32x4 qb[2], kb[2];
};
struct RVal {
    f32x4 mo[2], mv[2];
};
template <int NT, int MD>
struct Res {
    RRot rot[Items<NT, MD>::IX];
    RVal val[Items<NT, MD>::IX];
};
template <int IT>
struct FRot {
    V4<IT> q[2], k[2];
    float ang[4];
};
template <int IT>
struct FVal {
    V8<IT> d, v;
};
template <int NT, int MD, int IT>
struct Fetch {
    FRot<IT> rot[Items<NT, MD>::IX];
    FVal<IT> val[Items<NT, MD>::IX];
    V8<IT> st[Items<NT, MD>::IX];
    float s_cs, s_rev, s_dt, s_tr, s_dt1, s_tr1, qk;
    float seg[Items<NT, MD>::SX];
};

// The index decompositions of the chunk-load items.
struct ItemDiv {
    DivS dC, dM4, dP8;
    __device__ ItemDiv(int C, int N, int P) : dC(C), dM4(N / 8), dP8(P / 8) {}
};

// Where the tiles of one workgroup are.
struct Tiles {
    float *QH, *KH, *PS, *DPO, *SC, *DS, *AM, *WM, *OUT;
};

// The chunk being loaded.
struct ChunkAt {
    int b, h, g, bh, c, c0, cl;
    long tok0, tb0;   // (b, c0) as a token index; (b, h, c0) for the per-token arrays
};
__device__ __forceinline__ ChunkAt chunk_at(const Params2& p, int b, int h, int g, int bh, int c) {
    ChunkAt a;
    a.b = b; a.h = h; a.g = g; a.bh = bh; a.c = c;
    a.c0 = c * p.C;
    a.cl = min(p.C, p.S - a.c0);
    a.tok0 = (long)b * p.S + a.c0;
    a.tb0 = (long)bh * p.S + a.c0;
    return a;
}

template <bool MAIN>
__device__ __forceinline__ void res_rot(const Params2& p, int e, const ItemDiv& dv, int h, RRot& r) {
    const int R = p.R, N = p.N, M = N / 2;
    const int i = dv.dM4.q(e), n4 = 4 * (e - i * (M / 4)), rk = dv.dC.q(i);
    const float* qbp = p.q_bias + ((long)h * R + rk) * N + n4;
    r.qb[0] = *reinterpret_cast<const f32x4*>(qbp);
    r.qb[1] = *reinterpret_cast<const f32x4*>(qbp + M);
    if (MAIN) {
        const float* kbp = p.k_bias + ((long)h * R + rk) * N + n4;
        r.kb[0] = *reinterpret_cast<const f32x4*>(kbp);
        r.kb[1] = *reinterpret_cast<const f32x4*>(kbp + M);
    }
}
template <bool MAIN>
__device__ __forceinline__ void res_val(const Params2& p, int e, const ItemDiv& dv, int h, RVal& r) {
    const int R = p.R, P = p.P;
    const int i = dv.dP8.q(e), p8 = 8 * (e - i * (P / 8)), rk = dv.dC.q(i);
    if (p.reduce_o) {
        const float* m = p.mimo_o + ((long)h * R + rk) * P + p8;
        r.mo[0] = *reinterpret_cast<const f32x4*>(m);
        r.mo[1] = *reinterpret_cast<const f32x4*>(m + 4);
    }
    if (MAIN) {
        const float* m = p.mimo_v + ((long)h * R + rk) * P + p8;
        r.mv[0] = *reinterpret_cast<const f32x4*>(m);
        r.mv[1] = *reinterpret_cast<const f32x4*>(m + 4);
    }
}

// Rows past the chunk are not read.
template <bool MAIN, int IT>
__device__ __forceinline__ void fetch_rot(const Params2& p, int e, const ItemDiv& dv, const ChunkAt& a, FRot<IT>& f) {
    const int R = p.R, N = p.N, C = p.C, W = p.W, M = N / 2;
    const int i = dv.dM4.q(e), n4 = 4 * (e - i * (M / 4));
    const int r = dv.dC.q(i), t = i - r * C;
    if (t < a.cl) {
        const long src = (((a.tok0 + t) * R + r) * p.G + a.g) * N + n4;
        f.q[0] = ld4<IT>(p.q, src);
        f.q[1] = ld4<IT>(p.q, src + M);
        if (MAIN) {
            f.k[0] = ld4<IT>(p.k, src);
            f.k[1] = ld4<IT>(p.k, src + M);
        }
        const float* ap = p.angles + ((a.tok0 + t) * p.H + a.h) * W;
#pragma unroll
        for (int v = 0; v < 4; ++v) f.ang[v] = n4 + v < W ? ap[n4 + v] : 0.f;
    }
}
template <bool MAIN, int IT>
__device__ __forceinline__ void fetch_val(const Params2& p, int e, const ItemDiv& dv, const ChunkAt& a, FVal<IT>& f) {
    const int R = p.R, P = p.P, C = p.C;
    const int i = dv.dP8.q(e), p8 = 8 * (e - i * (P / 8));
    const int r = dv.dC.q(i), t = i - r * C;
    if (t < a.cl) {
        const long tk = a.tok0 + t;
        f.d = ld8<IT>(p.dout, (p.reduce_o ? (tk * p.H + a.h) * P : ((tk * R + r) * p.H + a.h) * P) + p8);
        if (MAIN) f.v = ld8<IT>(p.v, (tk * p.H + a.h) * P + p8);
    }
}
template <int IT>
__device__ __forceinline__ V8<IT> fetch_state(const Params2& p, int e, const ChunkAt& a) {
    return ld8<IT>(p.states, ((long)a.bh * p.nc + a.c) * p.N * p.P + 8 * e);
}

// Stage one rotation item: rotated q^ (and k^) rows into the tiles, cos and sin kept.
template <bool MAIN, int MD, int IT>
__device__ __forceinline__ void stage_rot(const Params2& p, const Tiles& T, int e, const ItemDiv& dv, int cl,
                                          const FRot<IT>& f, const RRot& res, float (&kcs)[4], float (&ksn)[4]) {
    constexpr int LD = Geo<MD>::LD;
    const int N = p.N, C = p.C, W = p.W, M = N / 2;
    const int i = dv.dM4.q(e), n4 = 4 * (e - i * (M / 4));
    const bool live = i - dv.dC.q(i) * C < cl;
    float qa[4], qe[4], ka[4], ke[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        float sn = 0.f, cs = 1.f;
        qa[v] = qe[v] = ka[v] = ke[v] = 0.f;
        if (live) {
            qa[v] = f.q[0][v] + res.qb[0][v];
            qe[v] = f.q[1][v] + res.qb[1][v];
            if (MAIN) {
                ka[v] = f.k[0][v] + res.kb[0][v];
                ke[v] = f.k[1][v] + res.kb[1][v];
            }
            if (n4 + v < W) sin_cos_ool(f.ang[v], sn, cs);
        }
        kcs[v] = cs;
        ksn[v] = sn;
        const float qa2 = cs * qa[v] - sn * qe[v], qe2 = sn * qa[v] + cs * qe[v];
        qa[v] = qa2;
        qe[v] = qe2;
        if (MAIN) {
            const float ka2 = cs * ka[v] - sn * ke[v], ke2 = sn * ka[v] + cs * ke[v];
            ka[v] = ka2;
            ke[v] = ke2;
        }
    }
    *reinterpret_cast<f32x4*>(T.QH + i * LD + n4) = f32x4{qa[0], qa[1], qa[2], qa[3]};
    *reinterpret_cast<f32x4*>(T.QH + i * LD + M + n4) = f32x4{qe[0], qe[1], qe[2], qe[3]};
    if (MAIN) {
        *reinterpret_cast<f32x4*>(T.KH + i * LD + n4) = f32x4{ka[0], ka[1], ka[2], ka[3]};
        *reinterpret_cast<f32x4*>(T.KH + i * LD + M + n4) = f32x4{ke[0], ke[1], ke[2], ke[3]};
    }
}
// Stage one value item: dPhiO (and Psi) rows; returns the raw v (zero past the chunk).
template <bool MAIN, int MD, int IT>
__device__ __forceinline__ V8<IT> stage_val(const Params2& p, const Tiles& T, int e, const ItemDiv& dv, int cl,
                                            const FVal<IT>& f, const RVal& res) {
    constexpr int LD = Geo<MD>::LD;
    const int P = p.P, C = p.C;
    const int i = dv.dP8.q(e), p8 = 8 * (e - i * (P / 8));
    const bool live = i - dv.dC.q(i) * C < cl;
    float d8[8], s8[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const float dv8 = f.d[v];
        d8[v] = live ? (p.reduce_o ? dv8 * res.mo[v >> 2][v & 3] : dv8) : 0.f;
        if (MAIN) s8[v] = live ? f.v[v] * res.mv[v >> 2][v & 3] : 0.f;
    }
    *reinterpret_cast<f32x4*>(T.DPO + i * LD + p8) = f32x4{d8[0], d8[1], d8[2], d8[3]};
    *reinterpret_cast<f32x4*>(T.DPO + i * LD + p8 + 4) = f32x4{d8[4], d8[5], d8[6], d8[7]};
    if (MAIN) {
        *reinterpret_cast<f32x4*>(T.PS + i * LD + p8) = f32x4{s8[0], s8[1], s8[2], s8[3]};
        *reinterpret_cast<f32x4*>(T.PS + i * LD + p8 + 4) = f32x4{s8[4], s8[5], s8[6], s8[7]};
    }
    return live ? f.v : zero8<IT>();
}
template <int MD, int IT>
__device__ __forceinline__ void stage_state(const Params2& p, const Tiles& T, int e, const ItemDiv& dv,
                                            const V8<IT>& w) {
    constexpr int LD = Geo<MD>::LD;
    const int n = dv.dP8.q(e), pc = 8 * (e - n * (p.P / 8));
    float* dst = T.SC + n * LD + pc;
    *reinterpret_cast<f32x4*>(dst) = f32x4{w[0], w[1], w[2], w[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{w[4], w[5], w[6], w[7]};
}

// Per-row token scalars of the chunk: exp(da_cs) (and, when MAIN, gamma, factor,
// exp(da_cs_rev)), written by thread t < C for every rank's row of token t; zero past
// the chunk.
template <bool MAIN, int MD>
__device__ __forceinline__ void stage_tok(const Params2& p, float* sm, const ChunkAt& a, float s_cs, float s_rev,
                                          float s_dt, float s_tr, float s_dt1, float s_tr1) {
    using GE = Geo<MD>;
    const int tid = tid_x();
    if (tid < p.C) {
        const bool tok_live = tid < a.cl;
        const float ecs = tok_live ? expf(s_cs) : 0.f;
        float gam = 0.f, fac = 0.f, er = 0.f;
        if (MAIN && tok_live) {
            gam = s_dt * (1.0f / (1.0f + expf(-s_tr)));
            const float beta = a.c0 + tid + 1 < p.S ? s_dt1 * (1.0f - 1.0f / (1.0f + expf(-s_tr1))) : 0.f;
            fac = gam + beta;
            er = expf(s_rev);
        }
        for (int r = 0; r < p.R; ++r) {
            const int i = r * p.C + tid;
            sm[GE::ECS + i] = ecs;
            if (MAIN) {
                sm[GE::GAM + i] = gam;
                sm[GE::FAC + i] = fac;
                sm[GE::EREV + i] = er;
            }
        }
    }
}

// MD = 64: issue chunk c's global loads (rows past the chunk are not read).
template <bool MAIN, int NT, int MD, int IT>
__device__ __forceinline__ void fetch_chunk(const Params2& p, const ChunkAt& a, const ItemDiv& dv,
                                            Fetch<NT, MD, IT>& f) {
    const int C = p.C, N = p.N, P = p.P, M = N / 2, RR = p.R * p.R;
    const int tid = tid_x(), rows = p.R * C;
#pragma unroll
    for (int x = 0; x < Items<NT, MD>::IX; ++x) {
        const int e = tid + NT * x;
        if (e < rows * (M / 4)) fetch_rot<MAIN, IT>(p, e, dv, a, f.rot[x]);
        if (e < rows * (P / 8)) fetch_val<MAIN, IT>(p, e, dv, a, f.val[x]);
        if (MAIN && e < N * (P / 8)) f.st[x] = fetch_state<IT>(p, e, a);
    }
    if (tid < a.cl) {
        f.s_cs = p.da_cs[a.tb0 + tid];
        if (MAIN) {
            f.s_rev = p.da_cs_rev[a.tb0 + tid];
            f.s_dt = p.dt[a.tb0 + tid];
            f.s_tr = ld1<IT>(p.trap, a.tb0 + tid);
            if (a.c0 + tid + 1 < p.S) {
                f.s_dt1 = p.dt[a.tb0 + tid + 1];
                f.s_tr1 = ld1<IT>(p.trap, a.tb0 + tid + 1);
            }
        }
    }
    if (MAIN) {
        if (tid < a.cl * RR) f.qk = ld1<IT>(p.qk_dot, a.tb0 * RR + tid);
#pragma unroll
        for (int x = 0; x < Items<NT, MD>::SX; ++x) {
            const int e = tid + NT * x;
            const int t = dv.dC.q(e), s2 = e - t * C;
            if (e < C * C && s2 < t && t < a.cl) f.seg[x] = p.segsum[((long)a.bh * p.nc + a.c) * C * C + e];
        }
    }
}

// MD = 64: stage chunk c from its fetched loads into LDS: rotated q^ (and k^, Psi, the
// cached state, qk_dot, exp(segsum) and the per-row scalars when MAIN), dPhiO and
// exp(da_cs). Rows past the chunk (t >= cl) are zero.
template <bool MAIN, int NT, int MD, int IT>
__device__ __forceinline__ void stage_chunk(const Params2& p, const Tiles& T, float* sm, const ChunkAt& a,
                                            const ItemDiv& dv, const Fetch<NT, MD, IT>& f, const Res<NT, MD>& res,
                                            Keep<NT, MD, IT>& keep) {
    using GE = Geo<MD>;
    const int C = p.C, N = p.N, P = p.P, M = N / 2, RR = p.R * p.R;
    const int tid = tid_x(), rows = p.R * C;
#pragma unroll
    for (int x = 0; x < Items<NT, MD>::IX; ++x) {
        const int e = tid + NT * x;
        if (e < rows * (M / 4)) stage_rot<MAIN, MD, IT>(p, T, e, dv, a.cl, f.rot[x], res.rot[x], keep.cs[x], keep.sn[x]);
        if (e < rows * (P / 8)) {
            const V8<IT> v = stage_val<MAIN, MD, IT>(p, T, e, dv, a.cl, f.val[x], res.val[x]);
            if (MAIN) keep.v[x] = v;
        }
        if (MAIN && e < N * (P / 8)) stage_state<MD, IT>(p, T, e, dv, f.st[x]);
    }
    stage_tok<MAIN, MD>(p, sm, a, f.s_cs, f.s_rev, f.s_dt, f.s_tr, f.s_dt1, f.s_tr1);
    if (MAIN) {
        if (tid < a.cl * RR) sm[GE::QKC + tid] = f.qk;
        // exp(segsum) of the chunk's strictly causal token pairs, in the output tile
        // (free until the dQ^ products)
#pragma unroll
        for (int x = 0; x < Items<NT, MD>::SX; ++x) {
            const int e = tid + NT * x;
            const int t = dv.dC.q(e), s2 = e - t * C;
            if (e < C * C) T.OUT[t * GE::LD + s2] = (s2 < t && t < a.cl) ? expf(f.seg[x]) : 0.f;
        }
    }
}

// MD = 128: load and stage chunk c item by item (the same values as fetch_chunk +
// stage_chunk; the rotation's cos and sin are kept, v is not).
template <bool MAIN, int NT, int MD, int IT>
__device__ __forceinline__ void stage_direct(const Params2& p, const Tiles& T, float* sm, const ChunkAt& a,
                                             const ItemDiv& dv, Keep<NT, MD, IT>& keep) {
    using GE = Geo<MD>;
    const int C = p.C, N = p.N, P = p.P, M = N / 2, RR = p.R * p.R;
    const int tid = tid_x(), rows = p.R * C;
#pragma unroll
    for (int x = 0; x < Items<NT, MD>::IX; ++x) {
        const int e = tid + NT * x;
        if (e < rows * (M / 4)) {
            FRot<IT> f;
            RRot r;
            fetch_rot<MAIN, IT>(p, e, dv, a, f);
            res_rot<MAIN>(p, e, dv, a.h, r);
            stage_rot<MAIN, MD, IT>(p, T, e, dv, a.cl, f, r, keep.cs[x], keep.sn[x]);
        }
    }
#pragma unroll
    for (int x = 0; x < Items<NT, MD>::IX; ++x) {
        const int e = tid + NT * x;
        if (e < rows * (P / 8)) {
            FVal<IT> f;
            RVal r;
            fetch_val<MAIN, IT>(p, e, dv, a, f);
            res_val<MAIN>(p, e, dv, a.h, r);
            (void)stage_val<MAIN, MD, IT>(p, T, e, dv, a.cl, f, r);
        }
        if (MAIN && e < N * (P / 8)) stage_state<MD, IT>(p, T, e, dv, fetch_state<IT>(p, e, a));
    }
    float s_cs = 0.f, s_rev = 0.f, s_dt = 0.f, s_tr = 0.f, s_dt1 = 0.f, s_tr1 = 0.f;
    if (tid < a.cl) {
        s_cs = p.da_cs[a.tb0 + tid];
        if (MAIN) {
            s_rev = p.da_cs_rev[a.tb0 + tid];
            s_dt = p.dt[a.tb0 + tid];
            s_tr = ld1<IT>(p.trap, a.tb0 + tid);
            if (a.c0 + tid + 1 < p.S) {
                s_dt1 = p.dt[a.tb0 + tid + 1];
                s_tr1 = ld1<IT>(p.trap, a.tb0 + tid + 1);
            }
        }
    }
    stage_tok<MAIN, MD>(p, sm, a, s_cs, s_rev, s_dt, s_tr, s_dt1, s_tr1);
    if (MAIN) {
        for (int e = tid; e < a.cl * RR; e += NT) sm[GE::QKC + e] = ld1<IT>(p.qk_dot, a.tb0 * RR + e);
        const float* seg = p.segsum + ((long)a.bh * p.nc + a.c) * C * C;
        for (int e = tid; e < C * C; e += NT) {
            const int t = dv.dC.q(e), s2 = e - t * C;
            T.OUT[t * GE::LD + s2] = (s2 < t && t < a.cl) ? expf(seg[e]) : 0.f;
        }
    }
}

template <int MD>
__device__ __forceinline__ Tiles tiles_at(float* base) {
    using GE = Geo<MD>;
    return Tiles{base + GE::QH, base + GE::KH, base + GE::PS, base + GE::DPO, base + GE::SC,
                 base + GE::DS, base + GE::AM, base + GE::WM, base + GE::OUT};
}

// ---------------------------------------------------------------- kernels
// Sub-segment aggregate: U <- Q^^T (exp(da_cs) dPhiO) + exp(da_cs[last]) U over the
// chunks of the sub-segment from the last one down, and the product of the decays.
// Sub-segment j covers part j % F of segment 1 + j / F (segment 0's aggregate is
// never needed).
// EX: the shape-exact instance (R = 4, C = 16, N = P = 64, rotated width 16): the sizes
// become constants, so index arithmetic folds (divisions by C, N/8, P/8 become shifts).
template <bool EX>
__device__ __forceinline__ void exact_shape(Params2& p) {
    if constexpr (EX) {
        p.R = 4;
        p.C = 16;
        p.N = 64;
        p.P = 64;
        p.W = 16;
    }
}

template <int IT, int MD, bool EX = false>
__global__ __launch_bounds__(NTHR, 2) void k_agg2(Params2 p) {
    exact_shape<EX>(p);
    using GE = Geo<MD>;
    constexpr int LD = GE::LD;
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
    float* tiles = GE::WIDE ? p.slots + (long)blockIdx.x * GE::AGG_TILES : sm + GE::SMALL;
    Tiles T = {};
    T.QH = tiles + GE::A_QH;
    T.DPO = tiles + GE::A_DPO;
    float* U = GE::WIDE ? sm + GE::U_LDS : tiles + GE::A_U;
    const float* ECS = sm + GE::ECS;
    for (int e = threadIdx.x; e < N * P; e += NTHR) U[(e / P) * LD + e % P] = 0.f;
    float dprod = 1.f;
    const ItemDiv dv(C, N, P);
    Keep<NTHR, MD, IT> keep;
    [[maybe_unused]] Res<NTHR, MD> res;
    [[maybe_unused]] Fetch<NTHR, MD, IT> f;
    if constexpr (!GE::WIDE) {
#pragma unroll
        for (int x = 0; x < Items<NTHR, MD>::IX; ++x) {
            const int e = tid_x() + NTHR * x;
            if (e < rows * (N / 8)) res_rot<false>(p, e, dv, h, res.rot[x]);
            if (e < rows * (P / 8)) res_val<false>(p, e, dv, h, res.val[x]);
        }
        if (c_end > c_begin) fetch_chunk<false>(p, chunk_at(p, b, h, g, bh, c_end - 1), dv, f);
    }
    for (int c = c_end - 1; c >= c_begin; --c) {
        const ChunkAt a = chunk_at(p, b, h, g, bh, c);
        sync<MD>();
        if constexpr (GE::WIDE) {
            stage_direct<false>(p, T, sm, a, dv, keep);
        } else {
            stage_chunk<false>(p, T, sm, a, dv, f, res, keep);
            if (c > c_begin) fetch_chunk<false>(p, chunk_at(p, b, h, g, bh, c - 1), dv, f);   // in flight
        }
        sync<MD>();
        const float dA = ECS[a.cl - 1];   // exp(da_cs) at the chunk's last token
        // U[n][p] = sum_i Q^[i][n] exp(da_cs[t_i]) dPhiO[i][p] + dA U[n][p]; the thread that
        // owns (n, p) in the product is the only one reading and writing U[n][p]
        // A(n, i) = Q^[i][n], B(i, p) = dPhiO[i][p] scaled per i by exp(da_cs[t_i])
        gemm<MD, NTHR, false, false, true>(
            N, P, rows, T.QH, T.DPO, ECS, [&](int n, int pc, float v) { U[n * LD + pc] = v + dA * U[n * LD + pc]; });
        dprod *= dA;
    }
    sync<MD>();
    float* out = p.agg + ((long)bh * p.nsub + seg) * N * P;
    for (int e = threadIdx.x; e < N * P; e += NTHR) out[e] = U[(e / P) * LD + e % P];
    if (threadIdx.x == 0) p.decay[(long)bh * p.nsub + seg] = dprod;
}

// The rotated-frame gradient of q^ (KSIDE false: dQ^ in OUT plus the same-token part
// sum_r2 dqk'[t][r][r2] k^[t,r2]) or of k^ (KSIDE: factor_t dK~ with dK~ in OUT, plus
// sum_r2 dqk'[t][r2][r] q^[t,r2]), X being k^ or q^ and dqk' the gamma-scaled
// same-token dots, taken back to the input frame by the inverse rotation of the
// thread's rotation items (cos and sin kept from the load) and written to DQ or DK
// [B, S*R, H, N], four columns of each half a store. OUT is only read.
template <int NT, int MD, int IT, bool KSIDE>
__device__ __forceinline__ void finish_rot(const Params2& p, void* dst, const float* OUT, const float* X,
                                           const float* DQK, const float* FAC, const Keep<NT, MD, IT>& keep, int b,
                                           int h, int c0, int cl, const DivS& dC, const DivS& dM4) {
    constexpr int LD = Geo<MD>::LD;
    const int R = p.R, N = p.N, C = p.C, M = N / 2, RR = R * R;
#pragma unroll
    for (int x = 0; x < Items<NT, MD>::IX; ++x) {
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
        store4(dst, o, p.out_dt, a2[0], a2[1], a2[2], a2[3]);
        store4(dst, o + M, p.out_dt, e2[0], e2[1], e2[2], e2[3]);
    }
}

// The chunk pass of one segment, chunks from the last down.
template <int IT, int MD, bool EX = false>
__global__ __launch_bounds__(NTHR2, 1) void k_main2(Params2 p) {
    exact_shape<EX>(p);
    using GE = Geo<MD>;
    using IS = Items<NTHR2, MD>;
    constexpr int LD = GE::LD, HM = MD / 2;
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
    Tiles T = tiles_at<MD>(GE::WIDE ? p.slots + (long)blockIdx.x * GE::MAIN_TILES : sm + GE::SMALL);
    if constexpr (GE::WIDE) {
        // the two most used tiles in LDS (their slot regions stay unused); the products
        // read their other operands from the slot
        T.OUT = sm + GE::OUT_LDS;
        T.WM = sm + GE::W_LDS;
    }
    float* QH = T.QH;
    float* KH = T.KH;
    float* PS = T.PS;
    float* DPO = T.DPO;
    float* SC = T.SC;
    float* DS = T.DS;
    float* AM = T.AM;
    float* WM = T.WM;
    float* OUT = T.OUT;
    float* GAM = sm + GE::GAM;
    float* FAC = sm + GE::FAC;
    float* ECS = sm + GE::ECS;
    float* EREV = sm + GE::EREV;
    float* RED = sm + GE::RED;
    float* DQK = sm + GE::DQK;
    float* QKC = sm + GE::QKC;
    float* RS0 = sm + GE::RS0;
    float* RS1 = sm + GE::RS1;
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
    Keep<NTHR2, MD, IT> keep;
    [[maybe_unused]] Res<NTHR2, MD> res;
    [[maybe_unused]] Fetch<NTHR2, MD, IT> f;
    if constexpr (!GE::WIDE) {
#pragma unroll
        for (int x = 0; x < IS::IX; ++x) {
            const int e = tid_x() + NTHR2 * x;
            if (e < rows * (N / 8)) res_rot<true>(p, e, dv, h, res.rot[x]);
            if (e < rows * (P / 8)) res_val<true>(p, e, dv, h, res.val[x]);
        }
        if (c_end > c_begin) fetch_chunk<true>(p, chunk_at(p, b, h, g, bh, c_end - 1), dv, f);
    }
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
    float mvacc[IS::MX];   // DMIMO_V items (r, p) = tid + NTHR2 x
#pragma unroll
    for (int x = 0; x < IS::MX; ++x) mvacc[x] = 0.f;
    float ddacc = 0.f;

    for (int c = c_end - 1; c >= c_begin; --c) {
        const ChunkAt a = chunk_at(p, b, h, g, bh, c);
        const int c0 = a.c0, cl = a.cl;
        const int tid = tid_x();
        sync<MD>();
        flush_dda();
        if constexpr (GE::WIDE) {
            stage_direct<true>(p, T, sm, a, dv, keep);
        } else {
            stage_chunk<true>(p, T, sm, a, dv, f, res, keep);
            if (c > c_begin) fetch_chunk<true>(p, chunk_at(p, b, h, g, bh, c - 1), dv, f);   // in flight
        }
        sync<MD>();

        // ---- causal block A = E (Q^ K~^T) and dP = dPhiO Psi^T; dP's same-token entries
        // are the dots dPhiO[t,r] . Psi[t,r2] (DGAMMA, the D-skip sum, the same-token parts).
        // The same-token entries of A take the coefficients with which Psi[t,r2] enters
        // y[t,r] directly, gamma_t qk_dot[t][r][r2] (+ d where r = r2), so A^T dPhiO carries
        // those terms of dPsi.
        gemm<MD, NTHR2, true, true, false>(rows, rows, N, QH, KH, nullptr, [&](int i, int j, float v) {
            const int ri = dC.q(i), ti = i - ri * C, rj = dC.q(j), tj = j - rj * C;
            float av = 0.f;
            if (tj < ti && ti < cl) av = v * FAC[j] * OUT[ti * LD + tj];
            if (tj == ti && ti < cl) av = GAM[j] * QKC[ti * RR + ri * R + rj] + (i == j ? dval : 0.f);
            AM[i * LD + j] = av;
        });
        gemm<MD, NTHR2, true, true, false>(rows, rows, P, DPO, PS, nullptr, [&](int i, int j, float v) {
            WM[i * LD + j] = v;
            const int ri = dC.q(i), ti = i - ri * C, rj = dC.q(j), tj = j - rj * C;
            if (ti == tj && ti < cl) DQK[ti * RR + ri * R + rj] = v;
        });
        sync<MD>();
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
        sync<MD>();
        // same-token factors of the diagonal: gamma_t times the dots
        for (int e = tid; e < cl * RR; e += NTHR2) DQK[e] *= GAM[dRR.q(e)];

        // ---- dQ^ = exp(da_cs) dPhiO S_c^T + W K~; DDA_CS[t] = sum over the token's rows of
        // q^ . (exp(da_cs) dPhiO S_c^T), as row sums of the first product
        gemm<MD, NTHR2, true, true, false, true>(
            rows, N, P, DPO, SC, nullptr,
            [&](int i, int n, float v) {
                const float o = v * ECS[i];
                OUT[i * LD + n] = o;
                return QH[i * LD + n] * o;
            },
            RS0);
        sync<MD>();
        token_out<MD>(cl, R, C, RS0, [&](int t, float v) { p.dda_cs[tokS + c0 + t] = v; });
        // W K~: B(j, n) = k^[j][n] scaled per j by the factor (folded into A)
        gemm<MD, NTHR2, true, false, true>(
            rows, N, rows, WM, KH, FAC, [&](int i, int n, float v) { OUT[i * LD + n] += v; });
        sync<MD>();
        // angle gradient, q part: d(a')/dθ = -e', d(e')/dθ = a' for the rotated pair (a', e')
        float dth[IS::DX];   // items (t, n): t < C, n < W <= MD / 2
#pragma unroll
        for (int x = 0; x < IS::DX; ++x) {
            const int e = tid + NTHR2 * x;
            const int t = e / HM, n = e % HM;
            float s = 0.f;
            if (t < cl && n < W)
                for (int r = 0; r < R; ++r) {
                    const int i = r * C + t;
                    s += OUT[i * LD + n] * (-QH[i * LD + M + n]) + OUT[i * LD + M + n] * QH[i * LD + n];
                }
            dth[x] = s;
        }
        // the same-token part, then back to the input frame: DQ (OUT is only read)
        finish_rot<NTHR2, MD, IT, false>(p, p.dq, OUT, KH, DQK, FAC, keep, b, h, c0, cl, dC, dM4);
        sync<MD>();

        // ---- dK~ = exp(da_cs_rev) Psi dS^T + W^T Q^; DDA_CS_REV from the first product's row
        // sums (k^ . its rows), DFACTOR from those of the whole dK~
        gemm<MD, NTHR2, true, true, false, true>(
            rows, N, P, PS, DS, nullptr,
            [&](int j, int n, float v) {
                const float o = v * EREV[j];
                OUT[j * LD + n] = o;
                return KH[j * LD + n] * o;
            },
            RS1);
        sync<MD>();
        token_out<MD>(cl, R, C, RS1, [&](int t, float v) { p.dda_cs_rev[tokS + c0 + t] = v * FAC[t]; });
        gemm<MD, NTHR2, false, false, false, true>(
            rows, N, rows, WM, QH, nullptr,
            [&](int j, int n, float v) {
                const float o = OUT[j * LD + n] + v;
                OUT[j * LD + n] = o;
                return KH[j * LD + n] * o;
            },
            RS0);
        sync<MD>();
        token_out<MD>(cl, R, C, RS0, [&](int t, float v) { p.dfactor[tokS + c0 + t] = v; });
#pragma unroll
        for (int x = 0; x < IS::DX; ++x) {
            const int e = tid + NTHR2 * x;
            const int t = e / HM, n = e % HM;
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
        finish_rot<NTHR2, MD, IT, true>(p, p.dk, OUT, QH, DQK, FAC, keep, b, h, c0, cl, dC, dM4);
        // v of the chunk into the W tile (free after the dK~ products), for DMIMO_V: with
        // MD = 64 the rank-0 value items hold it (zero past the chunk), else it is read again
        if constexpr (GE::WIDE) {
            for (int e = tid; e < C * (P / 8); e += NTHR2) {
                const int t = dP8.q(e), p8 = 8 * (e - t * (P / 8));
                const V8<IT> w = t < cl ? ld8<IT>(p.v, ((a.tok0 + t) * p.H + h) * P + p8) : zero8<IT>();
                *reinterpret_cast<f32x4*>(WM + t * LD + p8) = f32x4{w[0], w[1], w[2], w[3]};
                *reinterpret_cast<f32x4*>(WM + t * LD + p8 + 4) = f32x4{w[4], w[5], w[6], w[7]};
            }
        } else if (tid < C * (P / 8)) {
            const int t = dP8.q(tid), p8 = 8 * (tid - t * (P / 8));
            const V8<IT>& w = keep.v[0];
            *reinterpret_cast<f32x4*>(WM + t * LD + p8) = f32x4{w[0], w[1], w[2], w[3]};
            *reinterpret_cast<f32x4*>(WM + t * LD + p8 + 4) = f32x4{w[4], w[5], w[6], w[7]};
        }
        sync<MD>();

        // ---- dPsi = kappa dS + A^T dPhiO (the latter with the same-token and d terms)
        gemm<MD, NTHR2, true, false, false>(
            rows, P, N, KH, DS, nullptr, [&](int j, int pc, float v) { OUT[j * LD + pc] = v * FAC[j] * EREV[j]; });
        gemm<MD, NTHR2, false, false, false>(
            rows, P, rows, AM, DPO, nullptr, [&](int j, int pc, float v) { OUT[j * LD + pc] += v; });
        sync<MD>();
        for (int e = tid; e < cl * (P / 4); e += NTHR2) {
            const int t = dP4.q(e), p4 = 4 * (e - t * (P / 4));
            float s[4] = {0.f, 0.f, 0.f, 0.f};
            for (int r = 0; r < R; ++r) {
                const f32x4 o = *reinterpret_cast<const f32x4*>(OUT + (r * C + t) * LD + p4);
                const f32x4 m = *reinterpret_cast<const f32x4*>(p.mimo_v + ((long)h * R + r) * P + p4);
#pragma unroll
                for (int v = 0; v < 4; ++v) s[v] = __fmaf_rn(o[v], m[v], s[v]);
            }
            store4(p.dv, ((long)(b * p.S + c0 + t) * p.H + h) * P + p4, p.out_dt, s[0], s[1], s[2], s[3]);
        }
#pragma unroll
        for (int x = 0; x < IS::MX; ++x) {
            const int e = tid + NTHR2 * x;
            if (e < R * P) {
                const int r = dP.q(e), pc = e - r * P;
                float s = 0.f;
                for (int t = 0; t < cl; ++t) s = __fmaf_rn(OUT[(r * C + t) * LD + pc], WM[t * LD + pc], s);
                mvacc[x] += s;
            }
        }

        // ---- dS_c = Q^^T (exp(da_cs) dPhiO) + exp(da_cs[last]) dS_{c+1}, and DDA: the state
        // decay exp(da_cs[last]) multiplies S_c in S_{c+1}, so DDA[last] = exp(da_cs[last])
        // sum(dS_{c+1} * S_c), summed from the elements each lane updates (a wave's partial
        // into RED, the total after the next barrier)
        const float dA = ECS[cl - 1];
        float part = 0.f;
        gemm<MD, NTHR2, false, false, true>(N, P, rows, QH, DPO, ECS, [&](int n, int pc, float v) {
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
    sync<MD>();
    flush_dda();

    // ---- per-segment partial sums of DMIMO_V and DD
    __syncthreads();
#pragma unroll
    for (int x = 0; x < IS::MX; ++x) {
        const int e = tid + NTHR2 * x;
        if (e < R * P) p.part_mv[((long)bh * p.nseg + seg) * R * P + e] = mvacc[x];
    }
    const float dd = block_sum<NTHR2>(ddacc, RED);
    if (tid == 0) p.part_d[(long)bh * p.nseg + seg] = dd;
}

// The kernels of one data dtype, for the launch code (instantiated in one translation
// unit per dtype).
struct Kern {
    const void *agg, *main;
};
template <int IT>
Kern kernel_pair(int md, bool ex) {
    if (md == 64 && ex)
        return Kern{reinterpret_cast<const void*>(&k_agg2<IT, 64, true>), reinterpret_cast<const void*>(&k_main2<IT, 64, true>)};
    if (md == 64) return Kern{reinterpret_cast<const void*>(&k_agg2<IT, 64>), reinterpret_cast<const void*>(&k_main2<IT, 64>)};
    return Kern{reinterpret_cast<const void*>(&k_agg2<IT, 128>), reinterpret_cast<const void*>(&k_main2<IT, 128>)};
}
// ex: the shape-exact instances (R = 4, C = 16, N = P = 64, rotated width 16; md 64 only)
Kern kernels_bf16(int md, bool ex);
Kern kernels_f16(int md, bool ex);
Kern kernels_f32(int md, bool ex);

#ifdef MIMO_B2_COMMON_KERNELS
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
#endif

}  // namespace b2
}  // namespace mimo
