// Device code of the mamba_mimo_bwd_fwd HIP library: parameters, LDS layout,
// the per-chunk preparation stages and the two chunk kernels (templates over
// the tile shape). Instantiated per tile family in tiles_rp*_ct*.hip; the
// host side lives in mimo_bwd_fwd.hip.
//
// The arithmetic follows the Triton-Ascend mamba_mimo_bwd_fwd page's
// BF16-boundary PyTorch reference: bf16 (round to nearest even) at the same
// points, fp32 everywhere else. A bf16 rounding of an fp32 value is one
// v_cvt_pk_bf16_f32 with a zero low half: the result, read as fp32, is the
// rounded value. Two values that go to memory together are rounded and
// packed by one v_cvt_pk_bf16_f32.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mimo_bwd_fwd.h"

// No implicit fusion of a multiply and an add into an FMA anywhere below: the
// contract rounds some products on their own (rotation, diagonal, dz chain),
// and every instance of a kernel must compute the same fp32 operations. FMAs
// are written out (__builtin_fmaf / __fmaf_rn) where the rounding allows them.
#pragma clang fp contract(off)

namespace mimo {

// fp32 multiply and add, each rounded on its own. The HIP headers' __fmul_rn and
// __fadd_rn are plain operators compiled above this pragma, so a product of one
// feeding a sum of the other may still be fused; these may not.
__device__ __forceinline__ float fmul(float x, float y) { return x * y; }
__device__ __forceinline__ float fadd(float x, float y) { return x + y; }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));


// ---------------------------------------------------------------- bf16 helpers
// bf16(a) in the low and bf16(b) in the high half, round to nearest even.
__device__ __forceinline__ unsigned pk2(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ float lo16(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi16(unsigned u) { return __uint_as_float(u & 0xffff0000u); }
// bf16(x) as an fp32 value (one instruction: the rounded value lands in the high half)
__device__ __forceinline__ float rnd(float x) { return __uint_as_float(pk2(0.f, x)); }
__device__ __forceinline__ float bf2f(unsigned short u) { return __uint_as_float(static_cast<unsigned>(u) << 16); }
__device__ __forceinline__ unsigned short f2bf(float x) { return static_cast<unsigned short>(pk2(x, 0.f)); }
// the bf16 bits of a value that is already bf16-exact
__device__ __forceinline__ unsigned short bits16(float x) { return static_cast<unsigned short>(__float_as_uint(x) >> 16); }

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// One MFMA operand fragment of a row-major bf16 tile T[k][n] (pitch ld): lane
// (l16, q4) gets T[k0 + 8*q4 + 0..7][n0 + l16], the 8 consecutive contraction
// indices of column n0 + l16, from two transpose reads (ds_read_b64_tr_b16). In
// each 16-lane group, lane j of a read receives element j % 4 of the 4-element
// pieces supplied by lanes j/4, j/4 + 4, j/4 + 8 and j/4 + 12; so lane s points
// at row R0 + s/4, columns n0 + 4*(s%4) .. +3, and lane j gets rows R0 .. R0+3
// of column n0 + j.
__device__ __forceinline__ u32x4 frag_tr(const unsigned short* tile, int ld, int k0, int n0, int l16, int q4) {
    const unsigned short* a = tile + (k0 + 8 * q4 + (l16 >> 2)) * ld + n0 + 4 * (l16 & 3);
    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a));
    const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 4 * ld));
    const u32x2 ux = __builtin_bit_cast(u32x2, x), uy = __builtin_bit_cast(u32x2, y);
    return u32x4{ux[0], ux[1], uy[0], uy[1]};
}

// ---------------------------------------------------------------- fp32 math
// logistic function 1 / (1 + e^-x): hardware exp2 and reciprocal (about 2 ulp)
__device__ __forceinline__ float sigmoid_fast(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}

// sin and cos of x in radians. For |x| <= 8192: reduction to [-pi, pi] by a
// two-part 2*pi (fused multiply-adds), then the hardware sine and cosine of the
// angle in revolutions (measured on MI355X against double precision: at most
// 2.7e-7 absolute on [-pi, pi]). Larger arguments take the library's sincosf.
__device__ __forceinline__ void sin_cos(float x, float& s, float& c) {
    if (__builtin_fabsf(x) <= 8192.f) {
        const float k = __builtin_rintf(x * 0.159154936671257019f);
        float r = __builtin_fmaf(-k, 6.28318548202514648f, x);
        r = __builtin_fmaf(-k, -1.74845553146951720e-07f, r);
        const float u = r * 0.159154936671257019f;
        s = __builtin_amdgcn_sinf(u);
        c = __builtin_amdgcn_cosf(u);
    } else {
        sincosf(x, &s, &c);
    }
}

// sin_cos with its large-argument path out of line, for kernels that take many
// angles a thread: inlined copies of the library path would outgrow the
// instruction cache (64 KB, shared by two compute units).
__device__ inline __attribute__((noinline)) void sin_cos_far(float x, float& s, float& c) { sincosf(x, &s, &c); }
__device__ __forceinline__ void sin_cos_ool(float x, float& s, float& c) {
    if (__builtin_fabsf(x) <= 8192.f)
        sin_cos(x, s, c);
    else
        sin_cos_far(x, s, c);
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS accesses, not
// for its global memory traffic. __syncthreads() also waits for outstanding global
// loads into LDS (the staging prefetch below), which would serialise the prefetch
// with the chunk it is meant to overlap. The memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void bar() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The thread index as a value the compiler cannot move out of a loop: index and
// address arithmetic is then redone per chunk instead of being held in registers
// across the whole chunk loop (which spills). No instruction is emitted.
__device__ __forceinline__ int tid_x() {
    int x = threadIdx.x;
    asm volatile("" : "+v"(x));
    return x;
}

template <typename T>
__device__ __forceinline__ T lds_ld(const void* p) { return *reinterpret_cast<const T*>(p); }
template <typename T>
__device__ __forceinline__ void lds_st(void* p, T v) { *reinterpret_cast<T*>(p) = v; }

// ---------------------------------------------------------------- parameters
struct Params {
    int B, S, H, G, R, N, P, C, W, nc, L, nseg, rd;
    int F, nsub;    // the aggregate splits each segment but the last into F sub-segments of L/F chunks
    int reduce_o, has_z, has_d, need_y;
    int fwd;        // layer output o instead of the backward's outputs (no dout, states, qk_dot)
    const unsigned short *dout, *q, *k, *v, *z, *trap;
    const float *q_bias, *k_bias, *mimo_v, *mimo_o, *mimo_z, *angles, *da_cs, *da_cs_rev, *dt, *d, *segsum;
    float *dmimo_o, *dmimo_z;
    unsigned short *states, *dz, *qk_dot;
    unsigned short* o;   // layer output: [B,S,H,P] when reduce_o, else [B,S,R,H,P]
    // fp32-intermediate kernels only: per-token log decay [B,H,S] from which the
    // chunk controls are derived (nullptr: da_cs, da_cs_rev, segsum are given), and
    // an fp32 trap [B,H,S] used instead of the bf16 one when not nullptr
    const float *adt, *trapf;
    float* agg;     // [B*H][nsub][N*P]: sub-segment state increments, then the states after each
    float* decay;   // [B*H][nsub]: product of the chunk decays of each sub-segment
    float* part_o;  // [B*H][nseg][R*P] partial dmimo_o (== dmimo_o when nseg == 1)
    float* part_z;  // [B*H][nseg][R*P] partial dmimo_z
    float* kslots;  // fp32 path, 128-row tiles: per-workgroup K~ tiles [MT][NT+4] (one per block)
};

// LDS carve-up (byte offsets), shared by host and device. Every region but the
// last two depends only on the tile family (RP, CT, NT, PT), so inside a kernel
// their offsets and pitches are compile-time constants and one per-lane address
// register serves many accesses (the rest goes into the instructions' offset
// field). cos/sin and exp(segsum) are sized by the runtime C and W and come last.
struct Lds {
    int r1;   // bf16 main: [MT][LDQ] q | [MT][LDA] causal block | [NT][LDA] kappa^T; aggregate: [MT][KPN] kappa
    int r2;   // bf16 [MT][LDQ] k (main only)
    int r3;   // bf16 main: [PT][LDA] Psi^T; aggregate: [MT][PT+16] Psi
    int r4;   // bf16 [PT][LDQ] bf16(state)^T (main only)
    int qk;   // fp32 [Cp][RP*RP+RP] qk_dot, zero for padded ranks, RP pad words per token (main only)
    int dz;   // bf16 [Cp][PT+8] dz of the chunk, written out at the top of the next one (main only;
              // inside r2 when it fits there: k is dead from the kappa^T pass to the next chunk's phase A)
    int sc;   // fp32 [5][Cp] token scalars (exp(da_cs), gamma, exp(da_cs_rev), factor) + chunk decay
    int tb;   // bf16 tables: q_bias [RP][NT] (main only), k_bias [RP][NT], mimo_v [RP][PT]
    int cs;   // fp32 [2][C][W + 4] cos, sin (rows padded: 8 consecutive tokens hit distinct banks)
    int se;   // fp32 [C][C + 4] exp(segsum) (main only; rows padded likewise)
    int total;
};

__host__ __device__ constexpr int align16(int x) { return (x + 15) & ~15; }

// kpad: row pad (bf16) of the aggregate's kappa tile
__host__ __device__ constexpr Lds lds_layout_k(int RP, int CT, int NT, int PT, int C, int W, bool main, int kpad) {
    const int Cp = 16 * CT, MT = RP * Cp < 32 ? 32 : RP * Cp;
    const int ldq = NT + 8, lda = MT + 8;
    int r1 = main ? NT * lda : MT * (NT + kpad);
    if (main && MT * ldq > r1) r1 = MT * ldq;
    if (main && MT * lda > r1) r1 = MT * lda;
    Lds s{};
    int off = 0;
    s.r1 = off; off += align16(r1 * 2);
    s.r2 = off; if (main) off += align16(MT * ldq * 2);
    s.r3 = off; off += align16((main ? PT * lda : MT * (PT + 16)) * 2);
    s.r4 = off; if (main) off += align16(PT * ldq * 2);
    s.qk = off; if (main) off += align16(Cp * (RP * RP + RP) * 4);
    s.dz = off;
    if (main && Cp * (PT + 8) <= MT * ldq) s.dz = s.r2;
    else if (main) off += align16(Cp * (PT + 8) * 2);
    s.sc = off; off += align16((4 * Cp + 4) * 4);
    s.tb = off; off += align16(((main ? 2 : 1) * RP * NT + RP * PT) * 2);
    s.cs = off; off += align16(2 * C * (W + 4) * 4);
    s.se = off; if (main) off += align16(C * (C + 4) * 4);
    s.total = off;
    return s;
}

// Row pad (bf16) of the aggregate's kappa tile: 16 puts the four rows of a transpose
// read in four different 8-bank groups. Eight-wave families whose aggregate would
// then just miss two workgroups per CU (for the rotary divisor 4 layout, with its
// staging) take 8 when that brings them in: two rows of a read then share a bank
// group, but a second workgroup per CU is worth more.
__host__ __device__ constexpr int agg_kpad(int RP, int CT, int NT, int PT) {
    const int Cp = 16 * CT, MT = RP * Cp < 32 ? 32 : RP * Cp;
    const int NTHR = (MT == 128 && PT >= 64) ? 512 : 256;
    if (NTHR != 512) return 16;
    const int QK_IT = (MT * (NT / 16) + NTHR - 1) / NTHR;
    const int SMB = align16(Cp * PT * 2 + Cp * (NT / 4) * 4 + (6 * Cp + 1) * 4);
    const int QKB = QK_IT * 2 * NTHR * 16;
    int tot[2] = {0, 0};
    for (int k = 0; k < 2; ++k) {
        const int dyn = lds_layout_k(RP, CT, NT, PT, Cp, NT / 4, false, k == 0 ? 16 : 8).total;
        const bool lite = dyn + 256 + 2 * SMB <= 80 * 1024;
        const bool qkon = lite && dyn + 256 + 2 * SMB + QKB <= 80 * 1024;
        tot[k] = dyn + (lite ? 2 * SMB + (qkon ? QKB : 0) : 16);
    }
    return (tot[0] > 80 * 1024 && tot[1] <= 80 * 1024) ? 8 : 16;
}
__host__ __device__ constexpr Lds lds_layout(int RP, int CT, int NT, int PT, int C, int W, bool main) {
    return lds_layout_k(RP, CT, NT, PT, C, W, main, main ? 16 : agg_kpad(RP, CT, NT, PT));
}

// ---------------------------------------------------------------- tile family
// RP: rank count rounded up to a power of two (ranks >= R are zero rows);
// CT: 16-token tiles per rank (Cp = 16*CT >= C); NT / PT: state and value
// dimensions rounded up to 32, 64 or 128. Rows of a chunk tile are
// rank-major, row = r*Cp + t.
template <int RP, int CT, int NT, int PT>
struct Tile {
    static constexpr int Cp = 16 * CT;
    static constexpr int MT = (RP * Cp < 32) ? 32 : RP * Cp;   // rows (MFMA K-steps of 32)
    static constexpr int NW = (MT == 128 && PT >= 64) ? 8 : 4;  // waves per workgroup
    static constexpr int NTHR = NW * 64;
    static constexpr int LDQ = NT + 8;                          // pitch of [*][NT] bf16 rows
    static constexpr int LDA = MT + 8;                          // pitch of [*][MT] bf16 rows
    // pitches of row-major tiles read through transpose reads (frag_tr): 16 extra
    // bf16 put the 4 rows of one read in 4 different 8-bank groups (see agg_kpad)
    static constexpr int KPN = NT + agg_kpad(RP, CT, NT, PT);   // [MT][KPN] kappa (aggregate kernel)
    static constexpr int PPN = PT + 16;                         // [MT][PPN] Psi (aggregate kernel)
    static constexpr int PTT = PT / 16;
    static constexpr int QK_IT = (MT * (NT / 16) + NTHR - 1) / NTHR;      // q/k items per thread
    static constexpr int PSI_IT = (Cp * (PT / 8) + NTHR - 1) / NTHR;      // v items per thread
    static constexpr int ANG_IT = (Cp * (NT / 2) + NTHR - 1) / NTHR;      // angle items per thread
    static constexpr int SEG_IT = (Cp * Cp + NTHR - 1) / NTHR;            // segsum items per thread
    static constexpr int ST = (NT / 16) * PTT;                             // state tiles
    static constexpr int STW = (ST + NW - 1) / NW;
    static constexpr int MTT = MT / 16;
    static constexpr int AT = MTT * MTT;                                   // causal-block tiles
    static constexpr int ATW = (AT + NW - 1) / NW;
    static constexpr int NPAIRS = CT * PTT;                                // (token tile, value tile)
    static constexpr int PW = (NPAIRS + NW - 1) / NW;                      // pairs per wave
    static constexpr int PSI_ITEMS = (Cp / 2) * RP * (PT / 8);             // (token pair, rank, 8 values)
    static constexpr int KAP_ITEMS = (MT / 2) * (NT / 8);                  // (row pair, 8 state columns)
    static constexpr int QKT = RP * RP * CT;                               // same-token (qk_dot) tiles
    // work items that divide evenly over the waves need no bound check (the
    // compiler cannot see that wave < NW)
    static constexpr bool ST_FULL = ST % NW == 0;
    static constexpr bool AT_FULL = AT % NW == 0;
    static constexpr bool PAIRS_FULL = NPAIRS % NW == 0;
    static constexpr bool QKT_FULL = QKT % NW == 0;
    // Rotation split (rotary divisor 4, N = NT): the rotated 8-column groups
    // (first N/32 of each half) go to the first half of the threads, the others
    // to the second half, so that no wave runs the rotation with half its lanes
    // idle; the second half fills Psi^T meanwhile.
    static constexpr bool RSPLIT_OK = NT >= 32 && (MT * NT / 32) % (NTHR / 2) == 0;
};

// ---------------------------------------------------------------- staging of chunk inputs
// LITE tile families (their LDS leaves room for two workgroups per compute unit
// with the staging below) fetch the inputs of chunk c+1 straight into LDS
// (global_load_lds: lane l of a wave writes its 4 or 16 bytes at base + 4l or
// base + 16l; a 2-byte load fills the low half of the lane's 4-byte slot) while
// chunk c computes.
//   Small inputs (v, angles, segsum, token scalars): two buffers, chunk c in
//   buffer c & 1. Slot e holds input item e, so after the workgroup barrier
//   that follows each thread's wait for its own loads, any thread may read any
//   slot of the current buffer.
//   q and k (QKON, when that fits as well): one buffer. Each thread reads back
//   exactly the slots it fetched, into registers, before it issues the next
//   prefetch.
// The other families load their inputs into registers at the top of the chunk.
template <int RP, int CT, int NT, int PT, bool MAIN, bool EX>
struct Stage {
    using T = Tile<RP, CT, NT, PT>;
    static constexpr int NQ = MAIN ? 4 : 2;                        // q0, q1, k0, k1 (or k0, k1)
    // slot regions sized to the items a chunk can have (W <= NT/4 in the shape-exact
    // instances, NT/2 otherwise); lanes past the last item write nothing
    static constexpr int V = 0;                                    // slot t + Cp*pg: v[t][8pg .. 8pg+7]
    static constexpr int ANG = V + T::Cp * PT * 2;                 // slot e = t*W + n: angle
    static constexpr int SEG = ANG + T::Cp * (EX ? NT / 4 : NT / 2) * 4;   // slot e = ti*C + tj: segsum
    static constexpr int SCAL = SEG + (MAIN ? T::Cp * T::Cp * 4 : 0);      // 7 rows of Cp dwords
    static constexpr int SMB = align16(SCAL + (6 * T::Cp + 1) * 4);       // one small-input buffer
    static constexpr int QKB = T::QK_IT * NQ * T::NTHR * 16;       // q/k of one chunk
    // dynamic LDS of the family at its largest chunk (C = Cp, W = NT/2)
    static constexpr int DYN = lds_layout(RP, CT, NT, PT, T::Cp, EX ? NT / 4 : NT / 2, MAIN).total + 256;
    static constexpr bool LITE = DYN + 2 * SMB <= 80 * 1024;
    static constexpr bool QKON = LITE && DYN + 2 * SMB + QKB <= 80 * 1024;
    static constexpr int QK = 2 * SMB;
    static constexpr int BYTES = LITE ? 2 * SMB + (QKON ? QKB : 0) : 16;
    // The chunk pass's causal block in a tile of its own, after the layout's regions,
    // where that still leaves room for two workgroups per compute unit: its stores then
    // wait for no read of q, and the kappa^T pass for no read of the block. Extra
    // dynamic LDS of the chunk pass (0: the block reuses the q tile).
    static constexpr int SA = align16(T::MT * T::LDA * 2);
    static constexpr int SA_BYTES = (MAIN && LITE && DYN + BYTES + SA <= 80 * 1024) ? SA : 0;
    // scalar rows inside SCAL
    static constexpr int DT0 = 0, DT1 = 4 * T::Cp, TR0 = 8 * T::Cp, TR1 = 12 * T::Cp, CS = 16 * T::Cp,
                         REV = 20 * T::Cp, DLAST = 24 * T::Cp;
};

// q/k of one chunk in registers
template <int RP, int CT, int NT, int PT, bool MAIN>
struct ChunkQK {
    using T = Tile<RP, CT, NT, PT>;
    u32x4 q0[T::QK_IT], q1[T::QK_IT], k0[T::QK_IT], k1[T::QK_IT];   // columns col0.., N/2+col0..
};

// Small inputs of one chunk in registers (families that are not LITE): the
// thread's v, angle and segsum items, and in wave 0 the scalars of token `lane`.
template <int RP, int CT, int NT, int PT, bool MAIN>
struct SmallRegs {
    using T = Tile<RP, CT, NT, PT>;
    u32x4 v[T::PSI_IT];
    float ang[T::ANG_IT];
    float seg[MAIN ? T::SEG_IT : 1];
    float dt0, dt1, tr0, tr1, cs, rev, dlast;
};

// Per-thread item coordinates, fixed for the whole kernel. Global reads of a chunk
// are addressed as (chunk base, the same for every lane) + (byte offset of the
// lane's item inside the chunk, the same for every chunk), so that the offsets
// stay in registers for the whole kernel and the bases are scalar.
template <int RP, int CT, int NT, int PT>
struct Items {
    using T = Tile<RP, CT, NT, PT>;
    int qk_row[T::QK_IT];         // tile row (-1: no item)
    int qk_col[T::QK_IT];         // first column of the 8-column group in the first half
    unsigned qk_off[T::QK_IT];    // byte offset of (t, r, g, col) inside a chunk's q/k block
    int ang_t[T::ANG_IT];         // token of the angle item (-1: none)
    unsigned ang_off[T::ANG_IT];  // byte offset inside a chunk's angle block
    unsigned v_off[T::PSI_IT];    // byte offset of the 8-column v group inside a chunk's v block
};

// q/k items. ROWS_FAST: consecutive threads take consecutive tile rows (the
// chunk-aggregate kernel writes kappa^T transposed straight from registers).
// RSPLIT: the rotation split described at Tile::RSPLIT_OK (rows fastest within
// each half). Otherwise the 8-column groups of one row are adjacent.
template <int RP, int CT, int NT, int PT, bool ROWS_FAST, bool RSPLIT>
__device__ __forceinline__ void make_items(const Params& p, int g, Items<RP, CT, NT, PT>& it) {
    using T = Tile<RP, CT, NT, PT>;
    const int tid = threadIdx.x;
    const int ng = p.N / 16;
#pragma unroll
    for (int j = 0; j < T::QK_IT; ++j) {
        int i = -1, gg = 0;
        if constexpr (RSPLIT) {
            // rows fastest: 8 consecutive lanes write 8 rows of one column group,
            // which the padded row pitch spreads over all banks
            constexpr int GR = NT / 32, HALF = T::NTHR / 2;
            const int half = tid / HALF, e = tid % HALF + j * HALF;
            i = e % T::MT;
            gg = e / T::MT + half * GR;
        } else {
            const int e = tid + j * T::NTHR;
            if (e < T::MT * ng) {
                i = ROWS_FAST ? e % T::MT : e / ng;
                gg = ROWS_FAST ? e / T::MT : e - i * ng;
            }
        }
        it.qk_row[j] = i;
        it.qk_col[j] = 8 * gg;
        it.qk_off[j] = 0;
        if (i >= 0) {
            const int r = i / T::Cp, t = i % T::Cp;
            it.qk_off[j] = 2u * (unsigned)(((t * p.R + r) * p.G + g) * p.N + 8 * gg);
        }
    }
#pragma unroll
    for (int j = 0; j < T::ANG_IT; ++j) {
        const int e = tid + j * T::NTHR;
        it.ang_t[j] = -1;
        it.ang_off[j] = 0;
        if (e < p.C * p.W) {
            const int t = e / p.W, n = e - t * p.W;
            it.ang_t[j] = t;
            it.ang_off[j] = 4u * (unsigned)(t * p.H * p.W + n);
        }
    }
#pragma unroll
    for (int j = 0; j < T::PSI_IT; ++j) {
        const int e = tid + j * T::NTHR;
        const int t = e % T::Cp, pc = (e / T::Cp) * 8;
        it.v_off[j] = 2u * (unsigned)(t * p.H * p.P + pc);
    }
}

template <typename T>
__device__ __forceinline__ const T* at(const void* base, unsigned byte_off) {
    return reinterpret_cast<const T*>(static_cast<const unsigned char*>(base) + byte_off);
}

// Register loads of chunk c's q/k (c0 = first token, cl = real tokens).
template <int RP, int CT, int NT, int PT, bool MAIN>
__device__ __forceinline__ void load_qk(const Params& p, const Items<RP, CT, NT, PT>& it, int b, int c0, int cl,
                                        ChunkQK<RP, CT, NT, PT, MAIN>& in) {
    using T = Tile<RP, CT, NT, PT>;
    const int R = p.R;
    const unsigned short* qb = p.q + (long)(b * p.S + c0) * R * p.G * p.N;
    const unsigned short* kb = p.k + (long)(b * p.S + c0) * R * p.G * p.N;
    const unsigned short* qb2 = qb + p.N / 2;
    const unsigned short* kb2 = kb + p.N / 2;
#pragma unroll
    for (int j = 0; j < T::QK_IT; ++j) {
        const int i = it.qk_row[j];
        const int r = i / T::Cp, t = i % T::Cp;
        if (i >= 0 && r < R && t < cl) {
            const unsigned o = it.qk_off[j];
            if (MAIN) {
                in.q0[j] = *at<u32x4>(qb, o);
                in.q1[j] = *at<u32x4>(qb2, o);
            }
            in.k0[j] = *at<u32x4>(kb, o);
            in.k1[j] = *at<u32x4>(kb2, o);
        }
    }
}

// Register loads of chunk c's small inputs (the items a LITE family stages).
template <int RP, int CT, int NT, int PT, bool MAIN>
__device__ __forceinline__ void load_small(const Params& p, const Items<RP, CT, NT, PT>& it, int b, int h, int bh,
                                           int c, int c0, int cl, SmallRegs<RP, CT, NT, PT, MAIN>& in) {
    using T = Tile<RP, CT, NT, PT>;
    const int tid = threadIdx.x;
    const unsigned short* vb = p.v + ((long)(b * p.S + c0) * p.H + h) * p.P;
#pragma unroll
    for (int j = 0; j < T::PSI_IT; ++j) {
        const int e = tid + j * T::NTHR;
        const int t = e % T::Cp, pc = (e / T::Cp) * 8;
        if (e < T::Cp * (PT / 8) && t < cl && pc < p.P) in.v[j] = *at<u32x4>(vb, it.v_off[j]);
    }
    const long tok = (long)bh * p.S + c0;
    if (tid < cl) {
        in.dt0 = p.dt[tok + tid];
        in.tr0 = bf2f(p.trap[tok + tid]);
        in.rev = p.da_cs_rev[tok + tid];
        if (MAIN) in.cs = p.da_cs[tok + tid];
        if (c0 + tid + 1 < p.S) {
            in.dt1 = p.dt[tok + tid + 1];
            in.tr1 = bf2f(p.trap[tok + tid + 1]);
        }
    }
    if (tid == 0) in.dlast = p.da_cs[tok + cl - 1];
    const float* ab = p.angles + ((long)(b * p.S + c0) * p.H + h) * p.W;
#pragma unroll
    for (int j = 0; j < T::ANG_IT; ++j)
        if (it.ang_t[j] >= 0 && it.ang_t[j] < cl) in.ang[j] = *at<float>(ab, it.ang_off[j]);
    if (MAIN && p.need_y) {
        const float* sb = p.segsum + ((long)bh * p.nc + c) * p.C * p.C;
#pragma unroll
        for (int j = 0; j < T::SEG_IT; ++j) {
            const int e = tid + j * T::NTHR;
            if (e < p.C * p.C) in.seg[j] = sb[e];
        }
    }
}

// One global_load_lds per lane: 16, 4 or 2 bytes from base + off (base the same
// for every lane, off a 32-bit byte offset) into the wave's LDS block at dst_wave
// (M0 holds its LDS address: the low 32 bits of a generic pointer into LDS are
// the LDS byte address, the high half being the shared aperture). Written as inline assembly so that the compiler's
// wait-count tracking does not treat the address registers as pending until the
// load completes (it would then wait for the whole prefetch as soon as such a
// register is reused). The waits are explicit instead: s_waitcnt vmcnt(0) before
// the staged data is read, and lgkmcnt(0) after the reads, before the next
// prefetch overwrites them. M0 is saved and restored around the load; an SALU
// write of M0 needs one wait state before an LDS DMA.
// A wave-uniform pointer, pinned to scalar registers (a no-op when it already is).
// readfirstlane returns int: each half goes through unsigned so that it is
// zero-extended, never sign-extended, into the 64-bit address.
__device__ __forceinline__ unsigned rfl(unsigned x) { return static_cast<unsigned>(__builtin_amdgcn_readfirstlane(x)); }
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ const void* sgpr_ptr(const void* p) {
    const uint64_t x = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = rfl(static_cast<unsigned>(x));
    const uint64_t hi = rfl(static_cast<unsigned>(x >> 32));
    return reinterpret_cast<const void*>((hi << 32) | lo);
}
// Raw buffer resource over [base, base + bytes) of a wave-uniform base: loads at
// or beyond `bytes` return zero (word 3 is the gfx9 untyped-buffer format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(sgpr_ptr(base)), (short)0, (int)rfl(bytes), 0x00020000);
}
constexpr unsigned kOut = 0x80000000u;   // buffer offset that is always out of range
#define MIMO_DMA(NAME, INSN)                                                                          \
    __device__ __forceinline__ void NAME(const void* base, unsigned off, unsigned char* dst_wave) { \
        const void* sb = sgpr_ptr(base);                                                            \
        const unsigned m = rfl(static_cast<unsigned>(reinterpret_cast<uintptr_t>(dst_wave)));      \
        unsigned saved;                                                                             \
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t" INSN                       \
                     " %1, %2\n\ts_mov_b32 m0, %0"                                                  \
                     : "=&s"(saved)                                                                 \
                     : "v"(off), "s"(sb), "s"(m)                                                    \
                     : "memory");                                                                   \
    }
MIMO_DMA(dma16, "global_load_lds_dwordx4")
MIMO_DMA(dma4, "global_load_lds_dword")
MIMO_DMA(dma2, "global_load_lds_ushort")
#undef MIMO_DMA

// Issue the staging loads of chunk c (first token c0, cl real tokens): q/k into
// qkst (when QKON), the small inputs into the buffer smb. Every address is a
// scalar chunk base plus a per-lane offset that does not change from chunk to chunk.
template <int RP, int CT, int NT, int PT, bool MAIN, bool QKON, bool EX>
__device__ __forceinline__ void prefetch_chunk(const Params& p, const Items<RP, CT, NT, PT>& it, int b, int h, int bh,
                                               int c, int c0, int cl, unsigned char* qkst, unsigned char* smb) {
    using T = Tile<RP, CT, NT, PT>;
    using SG = Stage<RP, CT, NT, PT, MAIN, EX>;
    const int tid = threadIdx.x, wave = uni(tid >> 6);
    const int R = p.R;
    if constexpr (QKON) {
        const unsigned short* qb = p.q + (long)(b * p.S + c0) * R * p.G * p.N;
        const unsigned short* kb = p.k + (long)(b * p.S + c0) * R * p.G * p.N;
#pragma unroll
        for (int j = 0; j < T::QK_IT; ++j) {
            const int i = it.qk_row[j];
            const int r = i / T::Cp, t = i % T::Cp;
            unsigned char* d = qkst + (j * SG::NQ) * T::NTHR * 16 + wave * 1024;
            if (i >= 0 && r < R && t < cl) {
                const unsigned o = it.qk_off[j], o2 = o + p.N;   // second half: N/2 bf16 further
                if (MAIN) {
                    dma16(qb, o, d);
                    dma16(qb, o2, d + T::NTHR * 16);
                    dma16(kb, o, d + 2 * T::NTHR * 16);
                    dma16(kb, o2, d + 3 * T::NTHR * 16);
                } else {
                    dma16(kb, o, d);
                    dma16(kb, o2, d + T::NTHR * 16);
                }
            }
        }
    }
    const unsigned short* vb = p.v + ((long)(b * p.S + c0) * p.H + h) * p.P;
#pragma unroll
    for (int j = 0; j < T::PSI_IT; ++j) {
        const int e = tid + j * T::NTHR;
        const int t = e % T::Cp, pc = (e / T::Cp) * 8;
        if (e < T::Cp * (PT / 8) && t < cl && pc < p.P)
            dma16(vb, it.v_off[j], smb + SG::V + (j * T::NTHR + wave * 64) * 16);
    }
    const float* ab = p.angles + ((long)(b * p.S + c0) * p.H + h) * p.W;
#pragma unroll
    for (int j = 0; j < T::ANG_IT; ++j)
        if (it.ang_t[j] >= 0 && it.ang_t[j] < cl) dma4(ab, it.ang_off[j], smb + SG::ANG + (j * T::NTHR + wave * 64) * 4);
    if (MAIN && p.need_y) {
        const float* sb = p.segsum + ((long)bh * p.nc + c) * p.C * p.C;
#pragma unroll
        for (int j = 0; j < T::SEG_IT; ++j) {
            const int e = tid + j * T::NTHR;
            if (e < p.C * p.C) dma4(sb, 4u * e, smb + SG::SEG + (j * T::NTHR + wave * 64) * 4);
        }
    }
    // token scalars: dt and trap from wave 0, the cumulative log decays from wave 1
    const int lane = tid & 63;
    const long tok = (long)bh * p.S + c0;
    unsigned char* sc = smb + SG::SCAL;
    const unsigned o4 = 4u * lane, o2 = 2u * lane;
    if (wave == 0 && lane < cl) {
        dma4(p.dt + tok, o4, sc + SG::DT0);
        dma2(p.trap + tok, o2, sc + SG::TR0);
        if (c0 + lane + 1 < p.S) {
            dma4(p.dt + tok + 1, o4, sc + SG::DT1);
            dma2(p.trap + tok + 1, o2, sc + SG::TR1);
        }
    }
    if (wave == 1) {
        if (lane < cl) {
            dma4(p.da_cs_rev + tok, o4, sc + SG::REV);
            if (MAIN) dma4(p.da_cs + tok, o4, sc + SG::CS);
        }
        if (lane == 0) dma4(p.da_cs + tok + cl - 1, 0u, sc + SG::DLAST);
    }
}

// Copy this thread's staged q/k slots into registers.
template <int RP, int CT, int NT, int PT, bool MAIN, bool EX>
__device__ __forceinline__ void read_stage(const unsigned char* qkst, ChunkQK<RP, CT, NT, PT, MAIN>& in) {
    using T = Tile<RP, CT, NT, PT>;
    using SG = Stage<RP, CT, NT, PT, MAIN, EX>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < T::QK_IT; ++j) {
        const unsigned char* d = qkst + (j * SG::NQ) * T::NTHR * 16 + tid * 16;
        if (MAIN) {
            in.q0[j] = lds_ld<u32x4>(d);
            in.q1[j] = lds_ld<u32x4>(d + T::NTHR * 16);
            in.k0[j] = lds_ld<u32x4>(d + 2 * T::NTHR * 16);
            in.k1[j] = lds_ld<u32x4>(d + 3 * T::NTHR * 16);
        } else {
            in.k0[j] = lds_ld<u32x4>(d);
            in.k1[j] = lds_ld<u32x4>(d + T::NTHR * 16);
        }
    }
}

// Phase 0: token scalars, cos/sin, exp(segsum) into LDS. LITE families read the
// small-input buffer of the chunk and spread the token scalars over three waves;
// the others read their registers, token scalars in wave 0:
//   gamma_t = bf16(dt_t) * sigmoid(trap_t)                                    (fp32)
//   beta_t  = bf16(bf16(dt_{t+1}) * sigmoid(-trap_{t+1})), 0 at the last token
//   factor_t = bf16(gamma_t + beta_t)
//   exp(da_cs_t) (main only), exp(da_cs_rev_t)             (LITE: wave 1)
//   exp(da_cs) of the chunk's last token, the chunk decay  (LITE: wave 2)
// Tokens past the chunk's end get zero.
template <int RP, int CT, int NT, int PT, bool MAIN, bool EX>
__device__ __forceinline__ void phase0(const Params& p, const Items<RP, CT, NT, PT>& it, int c0, int cl,
                                       const unsigned char* smb, const SmallRegs<RP, CT, NT, PT, MAIN>& sr,
                                       unsigned char* smem, const Lds& L) {
    using T = Tile<RP, CT, NT, PT>;
    using SG = Stage<RP, CT, NT, PT, MAIN, EX>;
    constexpr bool LITE = SG::LITE;
    const int tid = threadIdx.x, wave = uni(tid >> 6), lane = tid & 63;
    float* sc = reinterpret_cast<float*>(smem + L.sc);
    const unsigned char* ss = smb + SG::SCAL + 4 * lane;
    if (wave == 0 && lane < T::Cp) {
        float gam = 0.f, fac = 0.f;
        if (lane < cl) {
            const float dt0 = LITE ? lds_ld<float>(ss + SG::DT0) : sr.dt0;
            const float tr0 = LITE ? bf2f(lds_ld<unsigned short>(ss + SG::TR0)) : sr.tr0;
            gam = fmul(rnd(dt0), sigmoid_fast(tr0));
            float beta = 0.f;
            if (c0 + lane + 1 < p.S) {
                const float dt1 = LITE ? lds_ld<float>(ss + SG::DT1) : sr.dt1;
                const float tr1 = LITE ? bf2f(lds_ld<unsigned short>(ss + SG::TR1)) : sr.tr1;
                beta = rnd(fmul(rnd(dt1), sigmoid_fast(-tr1)));
            }
            fac = rnd(fadd(gam, beta));
        }
        sc[T::Cp + lane] = gam;
        sc[3 * T::Cp + lane] = fac;
    }
    if (wave == (LITE ? 1 : 0) && lane < T::Cp) {
        float ecs = 0.f, erev = 0.f;
        if (lane < cl) {
            erev = expf(LITE ? lds_ld<float>(ss + SG::REV) : sr.rev);
            if (MAIN) ecs = expf(LITE ? lds_ld<float>(ss + SG::CS) : sr.cs);
        }
        sc[lane] = ecs;
        sc[2 * T::Cp + lane] = erev;
    }
    if (tid == (LITE ? 128 : 0)) sc[4 * T::Cp] = expf(LITE ? lds_ld<float>(smb + SG::SCAL + SG::DLAST) : sr.dlast);
    float* scs = reinterpret_cast<float*>(smem + L.cs);
    const int CW = p.C * p.W, WP = p.W + 4;
#pragma unroll
    for (int j = 0; j < T::ANG_IT; ++j) {
        const int e = tid + j * T::NTHR;
        if (e < CW) {
            const int t = it.ang_t[j], n = e - t * p.W;
            float s = 0.f, co = 0.f;
            if (t < cl) sin_cos(LITE ? lds_ld<float>(smb + SG::ANG + 4 * e) : sr.ang[j], s, co);
            scs[t * WP + n] = co;
            scs[(p.C + t) * WP + n] = s;
        }
    }
    if (MAIN && p.need_y) {
        float* se = reinterpret_cast<float*>(smem + L.se);
#pragma unroll
        for (int j = 0; j < T::SEG_IT; ++j) {
            const int e = tid + j * T::NTHR;
            if (e < p.C * p.C) {
                const int ti = e / p.C, tj = e - ti * p.C;
                se[ti * (p.C + 4) + tj] = expf(LITE ? lds_ld<float>(smb + SG::SEG + 4 * e) : sr.seg[(MAIN ? j : 0)]);
            }
        }
    }
}

// Psi^T: sPsiT[p][r*Cp + t] = bf16(v[t,p] * bf16(mimo_v[r,p])), zero for padded
// tokens, ranks and columns.
// LITE families: items (token pair, rank, 8 value columns) from the small-input
// buffer, handled by threads [t0, t0 + nth); the two tokens of a column go out as
// one 4-byte write. Consecutive lanes take consecutive ranks, then token pairs:
// the 32 lanes of a write hit 32 different banks, and each group of 8 lanes
// reads two v slots in different banks.
template <int RP, int CT, int NT, int PT, bool MAIN, bool EX>
__device__ __forceinline__ void fill_psi(const Params& p, int cl, const unsigned char* smb, unsigned char* smem,
                                         const Lds& L, int t0, int nth) {
    using T = Tile<RP, CT, NT, PT>;
    using SG = Stage<RP, CT, NT, PT, MAIN, EX>;
    constexpr int TPN = T::Cp / 2;
    unsigned short* sPsiT = reinterpret_cast<unsigned short*>(smem + L.r3);
    const unsigned short* smv = reinterpret_cast<const unsigned short*>(smem + L.tb) + 2 * RP * NT;
    for (int e = threadIdx.x - t0; e < T::PSI_ITEMS; e += nth) {
        const int r = e % RP, tp = (e / RP) % TPN, pg = e / (TPN * RP);
        const int t = 2 * tp;
        u32x4 va = lds_ld<u32x4>(smb + SG::V + (t + T::Cp * pg) * 16);
        u32x4 vb = lds_ld<u32x4>(smb + SG::V + (t + 1 + T::Cp * pg) * 16);
        const bool col_ok = 8 * pg < p.P;
        if (!(col_ok && t < cl)) va = u32x4{0u, 0u, 0u, 0u};       // slots of absent tokens are stale
        if (!(col_ok && t + 1 < cl)) vb = u32x4{0u, 0u, 0u, 0u};
        const u32x4 m = lds_ld<u32x4>(smv + r * PT + 8 * pg);
        unsigned short* dst = sPsiT + (8 * pg) * T::LDA + r * T::Cp + t;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const float m0 = lo16(m[d]), m1 = hi16(m[d]);
            lds_st<unsigned>(dst + (2 * d) * T::LDA, pk2(lo16(va[d]) * m0, lo16(vb[d]) * m0));
            lds_st<unsigned>(dst + (2 * d + 1) * T::LDA, pk2(hi16(va[d]) * m1, hi16(vb[d]) * m1));
        }
    }
}
// Other families: each thread's register v items (token t, 8 columns), every rank.
template <int RP, int CT, int NT, int PT, bool MAIN>
__device__ __forceinline__ void fill_psi_regs(const Params& p, int cl, const SmallRegs<RP, CT, NT, PT, MAIN>& in,
                                              unsigned char* smem, const Lds& L) {
    using T = Tile<RP, CT, NT, PT>;
    const int tid = threadIdx.x;
    unsigned short* sPsiT = reinterpret_cast<unsigned short*>(smem + L.r3);
    const unsigned short* smv = reinterpret_cast<const unsigned short*>(smem + L.tb) + 2 * RP * NT;
#pragma unroll
    for (int j = 0; j < T::PSI_IT; ++j) {
        const int e = tid + j * T::NTHR;
        if (e >= T::Cp * (PT / 8)) continue;
        const int t = e % T::Cp, pc = (e / T::Cp) * 8;   // consecutive threads: consecutive tokens
        const bool real = t < cl && pc < p.P;
        for (int r = 0; r < RP; ++r) {
            unsigned short* dst = sPsiT + pc * T::LDA + r * T::Cp + t;
            const u32x4 mv = lds_ld<u32x4>(smv + r * PT + pc);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                unsigned u = pk2(lo16(in.v[j][d]) * lo16(mv[d]), hi16(in.v[j][d]) * hi16(mv[d]));
                if (!real) u = 0u;
                dst[(2 * d) * T::LDA] = static_cast<unsigned short>(u);
                dst[(2 * d + 1) * T::LDA] = static_cast<unsigned short>(u >> 16);
            }
        }
    }
}

// Psi in row-major form, dst[r*Cp + t][p] (pitch PPN) = bf16(v[t,p] * bf16(mimo_v[r,p])),
// zero for padded tokens and columns (and ranks, whose table rows are zero). Items
// (token, 8 value columns) write that piece of the token's row in every rank.
// LITE families take v from the small-input buffer (threads [t0, t0 + nth),
// columns fastest: the 8 lanes of a write cover all banks); the others from
// their register items.
template <int RP, int CT, int NT, int PT, bool MAIN, bool EX>
__device__ __forceinline__ void fill_psi_nat(const Params& p, int cl, const unsigned char* smb,
                                             const SmallRegs<RP, CT, NT, PT, MAIN>& sr, unsigned short* dst,
                                             const unsigned short* smv, int t0, int nth) {
    using T = Tile<RP, CT, NT, PT>;
    using SG = Stage<RP, CT, NT, PT, MAIN, EX>;
    constexpr int PG = PT / 8;
    auto item = [&](int t, int pg, u32x4 v) {
        if (!(t < cl && 8 * pg < p.P)) v = u32x4{0u, 0u, 0u, 0u};   // absent tokens' data is stale
        float x[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            x[2 * d] = lo16(v[d]);
            x[2 * d + 1] = hi16(v[d]);
        }
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            const u32x4 m = lds_ld<u32x4>(smv + r * PT + 8 * pg);
            u32x4 o;
#pragma unroll
            for (int d = 0; d < 4; ++d) o[d] = pk2(x[2 * d] * lo16(m[d]), x[2 * d + 1] * hi16(m[d]));
            lds_st<u32x4>(dst + (r * T::Cp + t) * T::PPN + 8 * pg, o);
        }
    };
    if constexpr (SG::LITE) {
        for (int e = threadIdx.x - t0; e < T::Cp * PG; e += nth) {
            const int pg = e % PG, t = e / PG;
            item(t, pg, lds_ld<u32x4>(smb + SG::V + (t + T::Cp * pg) * 16));
        }
    } else {
#pragma unroll
        for (int j = 0; j < T::PSI_IT; ++j) {
            const int e = threadIdx.x + j * T::NTHR;
            if (e < T::Cp * PG) item(e % T::Cp, e / T::Cp, sr.v[j]);
        }
    }
}

// Tables filled once per workgroup: bf16(q_bias), bf16(k_bias), bf16(mimo_v) of
// head h, zero for padded ranks and columns; and the rows of Psi (Psi^T in the
// chunk kernel) beyond every rank, which no chunk writes.
template <int RP, int CT, int NT, int PT, bool NAT = false>
__device__ __forceinline__ void fill_tables(const Params& p, int h, unsigned char* smem, const Lds& L) {
    using T = Tile<RP, CT, NT, PT>;
    const int tid = threadIdx.x;
    // [RP][NT] q_bias (chunk pass only), [RP][NT] k_bias, [RP][PT] mimo_v
    unsigned short* tb = reinterpret_cast<unsigned short*>(smem + L.tb);
    constexpr int KB = NAT ? 0 : RP * NT;   // offset of k_bias
    for (int e = tid; e < RP * NT; e += T::NTHR) {
        const int r = e / NT, n = e % NT;
        const bool ok = r < p.R && n < p.N;
        const long src = ((long)h * p.R + r) * p.N + n;
        if constexpr (!NAT) tb[e] = ok ? f2bf(p.q_bias[src]) : 0;
        tb[KB + e] = ok ? f2bf(p.k_bias[src]) : 0;
    }
    for (int e = tid; e < RP * PT; e += T::NTHR) {
        const int r = e / PT, pc = e % PT;
        const bool ok = r < p.R && pc < p.P;
        tb[KB + RP * NT + e] = ok ? f2bf(p.mimo_v[((long)h * p.R + r) * p.P + pc]) : 0;
    }
    unsigned short* sPsiT = reinterpret_cast<unsigned short*>(smem + L.r3);
    constexpr int used = RP * T::Cp, pad = T::MT - used;
    if constexpr (pad > 0) {
        for (int e = tid; e < PT * pad; e += T::NTHR) {
            const int pp = e / pad, i = used + e % pad;
            if constexpr (NAT) sPsiT[i * T::PPN + pp] = 0;
            else sPsiT[pp * T::LDA + i] = 0;
        }
    }
}

// Biased, bf16-rounded values of one 8-column group of one row: x[d] = bf16(x + bias)
__device__ __forceinline__ void bias_group(u32x4 x, const unsigned short* bias, float out[8]) {
    const u32x4 b = lds_ld<u32x4>(bias);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        out[2 * d] = rnd(lo16(x[d]) + lo16(b[d]));
        out[2 * d + 1] = rnd(hi16(x[d]) + hi16(b[d]));
    }
}
__device__ __forceinline__ u32x4 pack8(const float x[8]) {
    return u32x4{pk2(x[0], x[1]), pk2(x[2], x[3]), pk2(x[4], x[5]), pk2(x[6], x[7])};
}
// Rotation of the column pairs (col0 + d, N/2 + col0 + d) with d < lim (every d
// when LIM >= 8): a holds the first-half values, e the second-half ones; the
// products are rounded separately, the sums are left unrounded (the caller rounds).
template <int LIM>
__device__ __forceinline__ void rotate8(float a[8], float e[8], int lim, const float* cs, const float* sn) {
    const f32x4 c0 = lds_ld<f32x4>(cs), c1 = lds_ld<f32x4>(cs + 4);
    const f32x4 s0 = lds_ld<f32x4>(sn), s1 = lds_ld<f32x4>(sn + 4);
    const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    const float s[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
    for (int d = 0; d < 8; ++d) {
        if (LIM >= 8 || d < lim) {
            const float x = a[d], y = e[d];
            a[d] = fmul(c[d], x) - fmul(s[d], y);
            e[d] = fmul(s[d], x) + fmul(c[d], y);
        }
    }
}

// ---------------------------------------------------------------- XCD-aware work mapping
// Workgroups are dealt to the 8 XCDs round-robin by block index, and each XCD
// has its own L2. The H/G heads that share a q/k group read the same q/k
// chunk, so they are mapped to the same XCD and to consecutive blocks of it.
// A work unit is (batch, group, segment); block k of XCD x takes head k % HPG
// of unit x + 8*(k / HPG). Returns false for the padding blocks of the grid.
__device__ __forceinline__ bool map_block(const Params& p, int nseg_k, int& seg, int& bh) {
    const int hpg = p.H / p.G;
    const int id = blockIdx.x;
    const int xcd = id & 7, k = id >> 3;
    const int unit = xcd + 8 * (k / hpg);
    if (unit >= p.B * p.G * nseg_k) return false;
    const int hh = k % hpg;
    seg = unit % nseg_k;
    const int bg = unit / nseg_k;          // b * G + g
    const int b = bg / p.G, g = bg % p.G;
    bh = b * p.H + g * hpg + hh;
    return true;
}

// ---------------------------------------------------------------- kernel specialisation
// EX: the call's shape equals the tile (R = RP, N = NT, P = PT, C = Cp) with rotary
// divisor 4, so sizes, pitches and bounds fold to constants. MODE: -1 reads the
// branch flags at run time; 0 = no y (neither reduced dout nor z); 1 = reduced
// dout with z; 2 = the layer output, reduced with z. Returns the parameters with
// those fields replaced by constants.
template <int RP, int CT, int NT, int PT, bool EX, int MODE>
__device__ __forceinline__ Params specialise(const Params& pin) {
    Params p = pin;
    if constexpr (EX) {
        p.R = RP;
        p.N = NT;
        p.P = PT;
        p.C = 16 * CT;
        p.rd = 4;
        p.W = NT / 4;
    }
    if constexpr (MODE == 0) {
        p.need_y = 0;
        p.reduce_o = 0;
        p.has_z = 0;
        p.fwd = 0;
    }
    if constexpr (MODE == 1 || MODE == 2) {
        p.need_y = 1;
        p.reduce_o = 1;
        p.has_z = 1;
        p.fwd = MODE == 2;
    }
    return p;
}

// ---------------------------------------------------------------- segment aggregate
// U_s = state added by segment s from a zero start: U <- U*exp(da_cs[last]) + kappa^T Psi
// per chunk; also the product of the chunk decays.
// ST: the chunk pass of a call that needs no y (neither reduced dout nor z: the outputs
// are the states and qk_dot only). The same walk over whole segments, from the state
// entering the segment; at the top of chunk c each lane writes its accumulator values of
// the state out as states[c] = bf16(S) (2-byte stores: 16 lanes cover 32 contiguous
// bytes of a row). Writing them straight from registers keeps the walk's LDS at the
// aggregate's, four workgroups per CU. qk_dot comes from k_qk.
template <int RP, int CT, int NT, int PT, bool EX, bool ST = false>
__global__ __launch_bounds__((Tile<RP, CT, NT, PT>::NTHR), 2) void k_agg(Params pin) {
    const Params p = specialise<RP, CT, NT, PT, EX, -1>(pin);
    using T = Tile<RP, CT, NT, PT>;
    using SG = Stage<RP, CT, NT, PT, false, EX>;
    extern __shared__ __align__(16) unsigned char smem[];
    const Lds L = lds_layout(RP, CT, NT, PT, p.C, p.W, false);
    unsigned short* sKap = reinterpret_cast<unsigned short*>(smem + L.r1);   // [MT][KPN] kappa
    unsigned short* sPsi = reinterpret_cast<unsigned short*>(smem + L.r3);   // [MT][PPN] Psi
    const float* sc = reinterpret_cast<const float*>(smem + L.sc);
    const float* scs = reinterpret_cast<const float*>(smem + L.cs);
    const unsigned short* tbk = reinterpret_cast<const unsigned short*>(smem + L.tb);   // the aggregate has no q_bias
    const unsigned short* smv = reinterpret_cast<const unsigned short*>(smem + L.tb) + RP * NT;

    const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
    const int l16 = lane & 15, q4 = lane >> 4;
    int seg, bh;
    if (!map_block(p, ST ? p.nseg : p.nsub, seg, bh)) return;
    // block-uniform indices, pinned to scalar registers (the divisions by run-time
    // sizes leave them in vector registers, and every address derived from them
    // would follow)
    seg = uni(seg);
    bh = uni(bh);
    const int b = uni(bh / p.H), h = uni(bh - b * p.H);
    const int g = uni(h / (p.H / p.G));
    int c_begin, c_end;
    if constexpr (ST) {
        c_begin = seg * p.L;
        c_end = min(c_begin + p.L, p.nc);
    } else {
        // sub-segment seg is piece k of segment s; pieces hold ceil(L / F) chunks, the
        // last one of a segment fewer (the host keeps every piece non-empty); all chunks
        // are full
        const int La = (p.L + p.F - 1) / p.F;
        const int s_ = uni(seg / p.F), k_ = seg - s_ * p.F;
        c_begin = s_ * p.L + k_ * La;
        c_end = min(c_begin + La, s_ * p.L + p.L);
    }
    const int R = p.R;
    // With one 8-column group per thread and rotary divisor 4, the threads of the
    // first half hold exactly the rotated groups; the second half fills Psi.
    constexpr bool SPLIT = SG::LITE && EX && T::QK_IT == 1 && T::MT * (NT / 32) == T::NTHR / 2;
    const int psi_t0 = SPLIT ? T::NTHR / 2 : 0, psi_n = SPLIT ? T::NTHR / 2 : T::NTHR;

    Items<RP, CT, NT, PT> it;
    make_items<RP, CT, NT, PT, true, false>(p, g, it);
    fill_tables<RP, CT, NT, PT, true>(p, h, smem, L);
    // kappa columns n >= N stay zero (every chunk writes each row's first N)
    for (int e = tid; e < T::MT * NT; e += T::NTHR) sKap[(e / NT) * T::KPN + e % NT] = 0;

    __shared__ __align__(16) unsigned char stg[SG::BYTES];
    unsigned char* qkst = stg + SG::QK;
    if constexpr (SG::LITE)
        prefetch_chunk<RP, CT, NT, PT, false, SG::QKON, EX>(p, it, b, h, bh, c_begin, c_begin * p.C,
                                                        min(p.C, p.S - c_begin * p.C), qkst, stg + (c_begin & 1) * SG::SMB);

    f32x4 U[T::STW];
#pragma unroll
    for (int w = 0; w < T::STW; ++w) U[w] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (ST && seg > 0) {
        // the state entering the segment (after the last piece of the segment before it)
        const float* E = p.agg + ((long)bh * p.nsub + seg * p.F - 1) * p.N * p.P;
#pragma unroll
        for (int w = 0; w < T::STW; ++w) {
            const int u = wave + w * T::NW;
            if (T::ST_FULL || u < T::ST) {
                const int nt = u / T::PTT, pt = u % T::PTT;
                const int pc = 16 * pt + l16;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int n = 16 * nt + 4 * q4 + v;
                    if (n < p.N && pc < p.P) U[w][v] = E[n * p.P + pc];
                }
            }
        }
    }
    float dprod = 1.f;

    for (int c = c_begin; c < c_end; ++c) {
        const int c0 = c * p.C;
        const int cl = min(p.C, p.S - c0);
        const unsigned char* smb = stg + (c & 1) * SG::SMB;
        ChunkQK<RP, CT, NT, PT, false> in = {};
        SmallRegs<RP, CT, NT, PT, false> sr = {};
        if constexpr (SG::LITE) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's staging loads of chunk c
            if constexpr (SG::QKON) {
                read_stage<RP, CT, NT, PT, false, EX>(qkst, in);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
            if (c + 1 < c_end)
                prefetch_chunk<RP, CT, NT, PT, false, SG::QKON, EX>(p, it, b, h, bh, c + 1, c0 + p.C,
                                                                min(p.C, p.S - c0 - p.C), qkst, stg + ((c + 1) & 1) * SG::SMB);
        } else {
            load_small(p, it, b, h, bh, c, c0, cl, sr);
        }
        if constexpr (!SG::QKON) load_qk(p, it, b, c0, cl, in);
        if constexpr (ST) {
            // states[c] = bf16(S entering chunk c): lane (l16, q4) of tile (nt, pt) holds rows
            // 16 nt + 4 q4 + v of column 16 pt + l16
            unsigned short* dst = p.states + ((long)bh * p.nc + c) * p.N * p.P;
#pragma unroll
            for (int w = 0; w < T::STW; ++w) {
                const int u = wave + w * T::NW;
                if (T::ST_FULL || u < T::ST) {
                    const int nt = u / T::PTT, pt = u % T::PTT;
                    const int pc = 16 * pt + l16, n0 = 16 * nt + 4 * q4;
                    const unsigned lo = pk2(U[w][0], U[w][1]), hi = pk2(U[w][2], U[w][3]);
                    const unsigned short x[4] = {static_cast<unsigned short>(lo), static_cast<unsigned short>(lo >> 16),
                                                 static_cast<unsigned short>(hi), static_cast<unsigned short>(hi >> 16)};
                    if (pc < p.P) {
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            if (n0 + v < p.N) dst[(n0 + v) * p.P + pc] = x[v];
                    }
                }
            }
        }
        bar();   // chunk c's staging loads of every thread have landed; previous chunk done with LDS
        phase0<RP, CT, NT, PT, false, EX>(p, it, c0, cl, smb, sr, smem, L);
        bar();
        // kappa = bf16(bf16(rot(bf16(k + bf16(k_bias))) * factor) * exp(da_cs_rev)), row-major;
        // rows of absent tokens and padded ranks are written as zero
#pragma unroll
        for (int j = 0; j < T::QK_IT; ++j) {
            const int i = it.qk_row[j];
            if (i < 0) continue;
            const int r = i / T::Cp, t = i % T::Cp;
            const int col0 = it.qk_col[j], col1 = p.N / 2 + col0;
            u32x4 oa = {0u, 0u, 0u, 0u}, oe = oa;
            if (r < R && t < cl) {
                float a[8], e[8];
                bias_group(in.k0[j], tbk + r * NT + col0, a);
                bias_group(in.k1[j], tbk + r * NT + col1, e);
                if (col0 < p.W) {
                    rotate8<(EX ? 8 : 0)>(a, e, p.W - col0, scs + t * (p.W + 4) + col0, scs + (p.C + t) * (p.W + 4) + col0);
#pragma unroll
                    for (int d = 0; d < 8; ++d) {
                        a[d] = rnd(a[d]);
                        e[d] = rnd(e[d]);
                    }
                }
                const float f = sc[3 * T::Cp + t], er = sc[2 * T::Cp + t];
#pragma unroll
                for (int d = 0; d < 8; ++d) {
                    a[d] = rnd(a[d] * f) * er;
                    e[d] = rnd(e[d] * f) * er;
                }
                oa = pack8(a);
                oe = pack8(e);
            }
            lds_st<u32x4>(sKap + i * T::KPN + col0, oa);
            lds_st<u32x4>(sKap + i * T::KPN + col1, oe);
        }
        if constexpr (SG::LITE) {
            if (tid >= psi_t0) fill_psi_nat<RP, CT, NT, PT, false, EX>(p, cl, smb, sr, sPsi, smv, psi_t0, psi_n);
        } else {
            fill_psi_nat<RP, CT, NT, PT, false, EX>(p, cl, smb, sr, sPsi, smv, 0, T::NTHR);
        }
        bar();
        const float dl = sc[4 * T::Cp];
#pragma unroll
        for (int w = 0; w < T::STW; ++w) {
            const int u = wave + w * T::NW;
            if (T::ST_FULL || u < T::ST) {
                const int nt = u / T::PTT, pt = u % T::PTT;
                f32x4 acc = U[w] * dl;
#pragma unroll
                for (int ks = 0; ks < T::MT / 32; ++ks)
                    acc = mfma(frag_tr(sKap, T::KPN, 32 * ks, 16 * nt, l16, q4),
                               frag_tr(sPsi, T::PPN, 32 * ks, 16 * pt, l16, q4), acc);
                U[w] = acc;
            }
        }
        dprod *= dl;
    }
    if constexpr (ST) return;
    float* out = p.agg + ((long)bh * p.nsub + seg) * p.N * p.P;
#pragma unroll
    for (int w = 0; w < T::STW; ++w) {
        const int u = wave + w * T::NW;
        if (T::ST_FULL || u < T::ST) {
            const int nt = u / T::PTT, pt = u % T::PTT;
            const int pc = 16 * pt + l16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int n = 16 * nt + 4 * q4 + v;
                if (n < p.N && pc < p.P) out[n * p.P + pc] = U[w][v];
            }
        }
    }
    if (tid == 0) p.decay[(long)bh * p.nsub + seg] = dprod;
}

// ---------------------------------------------------------------- main chunk pass
// dz rows of one chunk (first token c0, cl tokens) from LDS ([t][PT + 8] bf16) to
// global, 16 bytes a thread.
// Rows of a [B,S,H,P] bf16 output (dz, or the reduced layer output) staged in LDS
// by the epilogue, written out 16 bytes a thread.
template <int NTHR, int PT>
__device__ __forceinline__ void flush_dz(const Params& p, unsigned short* out, const unsigned short* sDz, int b, int h,
                                         int c0, int cl) {
    const int P8 = p.P / 8;
    unsigned short* dst = out + ((long)(b * p.S + c0) * p.H + h) * p.P;
    for (int e = threadIdx.x; e < cl * P8; e += NTHR) {
        const int t = e / P8, pc = (e - t * P8) * 8;
        *reinterpret_cast<u32x4*>(dst + (long)t * p.H * p.P + pc) = lds_ld<u32x4>(sDz + t * (PT + 8) + pc);
    }
}

// Rows of the per-rank layer output [B,S,R,H,P] of one chunk, staged in LDS by the
// epilogue as [r*Cp + t][PT + 8] bf16, written out 16 bytes a thread.
template <int NTHR, int PT>
__device__ __forceinline__ void flush_ranks(const Params& p, const unsigned short* sO, int Cp, int b, int h, int c0,
                                            int cl) {
    const int P8 = p.P / 8, per = cl * P8;
    for (int e = threadIdx.x; e < p.R * per; e += NTHR) {
        const int r = e / per, rem = e - r * per, t = rem / P8, pc = (rem - t * P8) * 8;
        unsigned short* dst = p.o + ((long)(b * p.S + c0 + t) * p.R + r) * p.H * p.P + (long)h * p.P + pc;
        *reinterpret_cast<u32x4*>(dst) = lds_ld<u32x4>(sO + (r * Cp + t) * (PT + 8) + pc);
    }
}

template <int RP, int CT, int NT, int PT, bool EX, int MODE>
__global__ __launch_bounds__((Tile<RP, CT, NT, PT>::NTHR), 2) void k_main(Params pin) {
    const Params p = specialise<RP, CT, NT, PT, EX, MODE>(pin);
    using T = Tile<RP, CT, NT, PT>;
    using SG = Stage<RP, CT, NT, PT, true, EX>;
    constexpr int MT = T::MT, NW = T::NW, NTHR = T::NTHR, Cp = T::Cp;
    constexpr int LDQ = T::LDQ, LDA = T::LDA, PTT = T::PTT, MTT = T::MTT;
    constexpr bool RSPLIT = EX && T::RSPLIT_OK;
    constexpr bool PSPLIT = RSPLIT && SG::LITE;   // the second half fills Psi^T
    extern __shared__ __align__(16) unsigned char smem[];
    const Lds L = lds_layout(RP, CT, NT, PT, p.C, p.W, true);
    constexpr bool SEPA = SG::SA_BYTES > 0;   // causal block in its own tile
    unsigned short* sQ = reinterpret_cast<unsigned short*>(smem + L.r1);   // also sKapT (and sA unless SEPA)
    unsigned short* sA = SEPA ? reinterpret_cast<unsigned short*>(smem + L.total) : sQ;
    unsigned short* sKapT = sQ;
    unsigned short* sK = reinterpret_cast<unsigned short*>(smem + L.r2);
    unsigned short* sPsiT = reinterpret_cast<unsigned short*>(smem + L.r3);
    unsigned short* sSbT = reinterpret_cast<unsigned short*>(smem + L.r4);
    const float* scs = reinterpret_cast<const float*>(smem + L.cs);
    const float* sE = reinterpret_cast<const float*>(smem + L.se);
    float* sQK = reinterpret_cast<float*>(smem + L.qk);
    unsigned short* sDz = reinterpret_cast<unsigned short*>(smem + L.dz);
    constexpr int QKS = RP * RP + RP;   // sQK pitch per token: a rank's RP values are 4*RP-byte aligned
    const float* sc = reinterpret_cast<const float*>(smem + L.sc);
    const unsigned short* tbq = reinterpret_cast<const unsigned short*>(smem + L.tb);
    const unsigned short* tbk = tbq + RP * NT;

    const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
    const int l16 = lane & 15, q4 = lane >> 4;
    int seg, bh;
    if (!map_block(p, p.nseg, seg, bh)) return;
    // block-uniform indices, pinned to scalar registers (see k_agg)
    seg = uni(seg);
    bh = uni(bh);
    const int b = uni(bh / p.H), h = uni(bh - b * p.H);
    const int g = uni(h / (p.H / p.G));
    const int c_begin = seg * p.L;
    const int c_end = min(c_begin + p.L, p.nc);
    const int R = p.R;
    const bool need_y = p.need_y;
    // the epilogue stages one [C,P] bf16 output per chunk in LDS: dz, or the reduced layer output
    const bool stage_out = p.fwd ? p.reduce_o : p.has_z;
    // the per-rank layer output is staged too when its RP*Cp rows fit the k tile
    // (dead from the kappa^T pass to the next chunk's phase A)
    constexpr bool RANKS_FIT = RP * Cp * (PT + 8) <= MT * LDQ;
    const bool stage_ranks = RANKS_FIT && p.fwd && !p.reduce_o;
    unsigned short* const out16 = p.fwd ? p.o : p.dz;
    // which threads fill Psi^T (LITE families): the second half under the rotation split, else all
    const int psi_t0 = PSPLIT ? NTHR / 2 : 0, psi_n = PSPLIT ? NTHR / 2 : NTHR;
    const bool rot_half = !RSPLIT || tid < NTHR / 2;   // threads whose q/k groups may be rotated

    Items<RP, CT, NT, PT> it;
    make_items<RP, CT, NT, PT, false, RSPLIT>(p, g, it);
    fill_tables<RP, CT, NT, PT>(p, h, smem, L);

    // ---- state entering the segment (fp32, MFMA accumulator layout: rows n, columns p)
    f32x4 Sacc[T::STW];
    {
        const float* E = (seg > 0) ? p.agg + ((long)bh * p.nsub + seg * p.F - 1) * p.N * p.P : nullptr;
#pragma unroll
        for (int w = 0; w < T::STW; ++w) {
            const int u = wave + w * NW;
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
            if (E != nullptr && (T::ST_FULL || u < T::ST)) {
                const int nt = u / PTT, pt = u % PTT;
                const int pc = 16 * pt + l16;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int n = 16 * nt + 4 * q4 + v;
                    if (n < p.N && pc < p.P) s[v] = E[n * p.P + pc];
                }
            }
            Sacc[w] = s;
        }
    }
    // bf16(S) into sSbT, the operand of the inter term; states[c] is copied out of
    // sSbT at the top of chunk c
    auto emit_state = [&]() {
#pragma unroll
        for (int w = 0; w < T::STW; ++w) {
            const int u = wave + w * NW;
            if (T::ST_FULL || u < T::ST) {
                const int nt = u / PTT, pt = u % PTT;
                const int pc = 16 * pt + l16;
                const u32x2 o = {pk2(Sacc[w][0], Sacc[w][1]), pk2(Sacc[w][2], Sacc[w][3])};
                lds_st<u32x2>(sSbT + pc * LDQ + 16 * nt + 4 * q4, o);
            }
        }
    };
    emit_state();

    // ---- per-lane constants of this wave's output tiles: slot (ps, r) is the
    // value tile of pair wave + ps*NW and rank r; lane column pc = 16*pt + l16.
    float cz[T::PW][RP], co[T::PW][RP], dmo[T::PW][RP], dmz[T::PW][RP];
#pragma unroll
    for (int ps = 0; ps < T::PW; ++ps) {
        const int pair = wave + ps * NW;
        const int pc = 16 * (pair % PTT) + l16;
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            cz[ps][r] = co[ps][r] = dmo[ps][r] = dmz[ps][r] = 0.f;
            if (pair < T::NPAIRS && r < R && pc < p.P) {
                if (p.has_z) cz[ps][r] = p.mimo_z[((long)h * R + r) * p.P + pc];
                if (p.reduce_o) co[ps][r] = rnd(p.mimo_o[((long)h * R + r) * p.P + pc]);
            }
        }
    }
    const float dval = p.has_d ? p.d[h] : 0.f;
    // byte offsets of this lane's gate inputs inside a chunk's [C, H, P] rows
    unsigned gate_off[T::PW][4];
#pragma unroll
    for (int ps = 0; ps < T::PW; ++ps) {
        const int pair = wave + ps * NW;
        const int tt = pair / PTT, pc = 16 * (pair % PTT) + l16;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int t = 16 * tt + 4 * q4 + v;
            gate_off[ps][v] = (pair < T::NPAIRS && pc < p.P) ? 2u * (unsigned)(t * p.H * p.P + pc) : kOut;
        }
    }
    __shared__ __align__(16) unsigned char stg[SG::BYTES];
    unsigned char* qkst = stg + SG::QK;
    if constexpr (SG::LITE)
        prefetch_chunk<RP, CT, NT, PT, true, SG::QKON, EX>(p, it, b, h, bh, c_begin, c_begin * p.C,
                                                       min(p.C, p.S - c_begin * p.C), qkst, stg + (c_begin & 1) * SG::SMB);

    for (int c = c_begin; c < c_end; ++c) {
        // Wave priority (four-wave tiles, two workgroups per CU): the chunk's chain of
        // barrier-separated phases issues at a raised priority, the epilogue
        // (independent VALU work, no barrier until the next chunk) at the normal one,
        // so that on a SIMD shared by the two workgroups the other workgroup's
        // epilogue fills the chain's gaps instead of delaying it
        if constexpr (NW == 4) __builtin_amdgcn_s_setprio(1);
        const int c0 = c * p.C;
        const int cl = min(p.C, p.S - c0);
        const unsigned char* smb = stg + (c & 1) * SG::SMB;

        ChunkQK<RP, CT, NT, PT, true> in = {};
        SmallRegs<RP, CT, NT, PT, true> sr = {};
        if constexpr (SG::LITE) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's staging loads of chunk c
            if constexpr (SG::QKON) {
                read_stage<RP, CT, NT, PT, true, EX>(qkst, in);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
            if (c + 1 < c_end)
                prefetch_chunk<RP, CT, NT, PT, true, SG::QKON, EX>(p, it, b, h, bh, c + 1, c0 + p.C,
                                                               min(p.C, p.S - c0 - p.C), qkst, stg + ((c + 1) & 1) * SG::SMB);
        } else {
            load_small(p, it, b, h, bh, c, c0, cl, sr);
        }
        if constexpr (!SG::QKON) load_qk(p, it, b, c0, cl, in);
        // gate inputs of this lane's tokens, raw bf16, consumed in the epilogue. The
        // loads are issued unconditionally (lanes without a token read the chunk's
        // first element) so that nothing waits for them before the epilogue.
        // Buffer loads over the chunk's rows of z and dout: lanes past the chunk's
        // end fall outside the buffer and read zero. Without gating the loads still
        // run (from v) so that every iteration loads and consumes the same
        // registers (see the end of the loop).
        unsigned short zraw[T::PW][4], draw[T::PW][4];
        {
            const long base = ((long)(b * p.S + c0)) * p.H * p.P + (long)h * p.P;
            const unsigned bytes = 2u * (unsigned)((cl - 1) * p.H * p.P + p.P);
            const auto zb = buffer((p.has_z ? p.z : (need_y && !p.fwd ? p.dout : p.v)) + base, bytes);
            const auto db = (p.reduce_o && !p.fwd) ? buffer(p.dout + base, bytes) : zb;
#pragma unroll
            for (int ps = 0; ps < T::PW; ++ps) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    zraw[ps][v] = __builtin_amdgcn_raw_buffer_load_b16(zb, gate_off[ps][v], 0, 0);
                    draw[ps][v] = __builtin_amdgcn_raw_buffer_load_b16(db, gate_off[ps][v], 0, 0);
                }
            }
        }
        bar();   // chunk c's staging loads of every thread have landed; previous chunk (and the tables) done

        // ---- states[c] = bf16(S entering chunk c), from sSbT ([p][n]) to [n][p], 16 bytes a thread
        if (!p.fwd) {
            unsigned short* dst = p.states + ((long)bh * p.nc + c) * p.N * p.P;
            const int P8 = p.P / 8;
            for (int e = tid; e < p.N * P8; e += NTHR) {
                const int pc = (e / p.N) * 8, n = e % p.N;   // consecutive threads: consecutive n
                const unsigned short* src = sSbT + pc * LDQ + n;
                u32x4 o;
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    o[d] = static_cast<unsigned>(src[(2 * d) * LDQ]) | (static_cast<unsigned>(src[(2 * d + 1) * LDQ]) << 16);
                *reinterpret_cast<u32x4*>(dst + n * p.P + pc) = o;
            }
        }
        // ---- dz of the previous chunk (always a full one), staged in LDS by its epilogue
        if (stage_out && c > c_begin) flush_dz<NTHR, PT>(p, out16, sDz, b, h, c0 - p.C, p.C);
        if (stage_ranks && c > c_begin) flush_ranks<NTHR, PT>(p, sDz, Cp, b, h, c0 - p.C, p.C);

        // ---- phase 0: token scalars, cos/sin, exp(segsum)
        phase0<RP, CT, NT, PT, true, EX>(p, it, c0, cl, smb, sr, smem, L);
        bar();

        // ---- phase A: biased q/k (unrotated into LDS, rotated and factor-scaled kept
        // in registers), Psi^T
        u32x4 rq0[T::QK_IT], rq1[T::QK_IT], rk0[T::QK_IT], rk1[T::QK_IT];
#pragma unroll
        for (int j = 0; j < T::QK_IT; ++j) {
            const int i = it.qk_row[j];
            if (i < 0) continue;
            const int r = i / Cp, t = i % Cp;
            const int col0 = it.qk_col[j], col1 = p.N / 2 + col0;
            float qa[8], qe[8], ka[8], ke[8];
            if (r < R && t < cl) {
                bias_group(in.q0[j], tbq + r * NT + col0, qa);
                bias_group(in.q1[j], tbq + r * NT + col1, qe);
                bias_group(in.k0[j], tbk + r * NT + col0, ka);
                bias_group(in.k1[j], tbk + r * NT + col1, ke);
            } else {
#pragma unroll
                for (int d = 0; d < 8; ++d) qa[d] = qe[d] = ka[d] = ke[d] = 0.f;
            }
            const u32x4 uqa = pack8(qa), uqe = pack8(qe);
            lds_st<u32x4>(sQ + i * LDQ + col0, uqa);
            lds_st<u32x4>(sQ + i * LDQ + col1, uqe);
            lds_st<u32x4>(sK + i * LDQ + col0, pack8(ka));
            lds_st<u32x4>(sK + i * LDQ + col1, pack8(ke));
            rq0[j] = uqa;
            rq1[j] = uqe;
            if (rot_half && col0 < p.W && r < R && t < cl) {
                const float* cs = scs + t * (p.W + 4) + col0;
                const float* sn = scs + (p.C + t) * (p.W + 4) + col0;
                rotate8<(RSPLIT ? 8 : 0)>(qa, qe, p.W - col0, cs, sn);
                rotate8<(RSPLIT ? 8 : 0)>(ka, ke, p.W - col0, cs, sn);
                rq0[j] = pack8(qa);
                rq1[j] = pack8(qe);
#pragma unroll
                for (int d = 0; d < 8; ++d) {
                    ka[d] = rnd(ka[d]);
                    ke[d] = rnd(ke[d]);
                }
            }
            const float f = sc[3 * Cp + t];
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                ka[d] *= f;
                ke[d] *= f;
            }
            rk0[j] = pack8(ka);
            rk1[j] = pack8(ke);
        }
        if (p.N < NT) {
            // state columns beyond N are zero in both operands of the n-contractions
            const int zc = (NT - p.N) / 8;
            for (int e = tid; e < MT * zc; e += NTHR) {
                const int i = e / zc, col = p.N + 8 * (e % zc);
                lds_st<u32x4>(sQ + i * LDQ + col, u32x4{0u, 0u, 0u, 0u});
                lds_st<u32x4>(sK + i * LDQ + col, u32x4{0u, 0u, 0u, 0u});
            }
        }
        if constexpr (SG::LITE) {
            if (tid >= psi_t0) fill_psi<RP, CT, NT, PT, true, EX>(p, cl, smb, smem, L, psi_t0, psi_n);
        } else {
            fill_psi_regs(p, cl, sr, smem, L);
        }
        bar();

        // ---- phase B: qk_dot of the same token (biased, unrotated) by MFMA, into sQK.
        // One rank: tile tt is Q0 rows times K0 rows over one token tile; its diagonal
        // holds the same-token dots. Lane (l16, q4) holds rows 4*q4 .. 4*q4+3 of
        // column l16, so the lanes with q4 == l16/4 hold one diagonal element each
        // (token 16*tt + l16).
        if constexpr (RP >= 2) {
            // Two or more ranks: tiles whose rows and columns are the 16 (token, rank) pairs of
            // TPT = 16 / RP consecutive tokens (row l16 = token u TPT + l16 / RP, rank
            // l16 % RP), K0 rows as the A operand and Q0 rows as B. Lane (l16, q4) then
            // holds dot(k0[row 4 q4 + i], q0[row l16]) for i = 0..3; those whose two
            // rows share a token are row r = l16 % RP of that token's dots, columns
            // (4 q4 + i) % RP: four of them (RP >= 4) or two (RP = 2), stored as one LDS
            // write. Each bf16 product is exact in fp32 and the K steps are the same, so
            // the sums are those of the rank-pair tiles. Padded rank pairs get zero.
            constexpr int TPT = 16 / RP, TL = Cp * RP / 16;
            const int rl = l16 % RP;
#pragma unroll
            for (int w = 0; w < (TL + NW - 1) / NW; ++w) {
                const int u = wave + w * NW;
                if (TL % NW == 0 || u < TL) {
                    const int tl = u * TPT + l16 / RP;
                    f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < NT / 32; ++ks) {
                        const u32x4 a = lds_ld<u32x4>(sK + (rl * Cp + tl) * LDQ + 32 * ks + 8 * q4);
                        const u32x4 bb = lds_ld<u32x4>(sQ + (rl * Cp + tl) * LDQ + 32 * ks + 8 * q4);
                        a4 = mfma(a, bb, a4);
                    }
                    if constexpr (RP >= 4) {
                        if ((4 * q4) / RP == l16 / RP) {
                            const int r20 = (4 * q4) % RP;
                            f32x4 o;
#pragma unroll
                            for (int i = 0; i < 4; ++i) o[i] = (rl < R && r20 + i < R) ? rnd(a4[i]) : 0.f;
                            lds_st<f32x4>(sQK + tl * QKS + rl * RP + r20, o);
                        }
                    } else {
                        if (q4 == (l16 >> 2)) {
                            const bool hi = (l16 >> 1) & 1;
                            const float x0 = hi ? a4[2] : a4[0], x1 = hi ? a4[3] : a4[1];
                            const f32x2 o = {rl < R ? rnd(x0) : 0.f, (rl < R && R > 1) ? rnd(x1) : 0.f};
                            lds_st<f32x2>(sQK + tl * QKS + rl * RP, o);
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int w = 0; w < (T::QKT + NW - 1) / NW; ++w) {
                const int u = wave + w * NW;
                if (T::QKT_FULL || u < T::QKT) {
                    const int rj = u % RP, ri = (u / RP) % RP, tt = u / (RP * RP);
                    float val = 0.f;
                    if (ri < R && rj < R) {
                        f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < NT / 32; ++ks) {
                            const u32x4 a = lds_ld<u32x4>(sQ + (16 * (ri * CT + tt) + l16) * LDQ + 32 * ks + 8 * q4);
                            const u32x4 bb = lds_ld<u32x4>(sK + (16 * (rj * CT + tt) + l16) * LDQ + 32 * ks + 8 * q4);
                            a4 = mfma(a, bb, a4);
                        }
                        const int v = l16 & 3;
                        const float x01 = (v & 1) ? a4[1] : a4[0], x23 = (v & 1) ? a4[3] : a4[2];
                        val = rnd((v & 2) ? x23 : x01);
                    }
                    if (q4 == (l16 >> 2)) sQK[(16 * tt + l16) * QKS + ri * RP + rj] = val;
                }
            }
        }
        bar();

        // ---- phase C: rotated q and factor-scaled k into LDS; qk_dot of the chunk out
#pragma unroll
        for (int j = 0; j < T::QK_IT; ++j) {
            const int i = it.qk_row[j];
            if (i < 0) continue;
            const int col0 = it.qk_col[j], col1 = p.N / 2 + col0;
            if (need_y && rot_half) {
                lds_st<u32x4>(sQ + i * LDQ + col0, rq0[j]);
                lds_st<u32x4>(sQ + i * LDQ + col1, rq1[j]);
            }
            lds_st<u32x4>(sK + i * LDQ + col0, rk0[j]);
            lds_st<u32x4>(sK + i * LDQ + col1, rk1[j]);
        }
        if (!p.fwd) {
            const int RR = R * R;
            unsigned short* qko = p.qk_dot + ((long)bh * p.S + c0) * RR;
            if constexpr (EX && (RP * RP) % 8 == 0) {
                // R = RP: a token's R*R values are contiguous in sQK; 8 per thread
                constexpr int G8 = RP * RP / 8;
                for (int e = tid; e < cl * G8; e += NTHR) {
                    const int t = e / G8, k8 = (e % G8) * 8;
                    const float* s = sQK + t * QKS + k8;
                    const u32x4 o = {pk2(s[0], s[1]), pk2(s[2], s[3]), pk2(s[4], s[5]), pk2(s[6], s[7])};
                    *reinterpret_cast<u32x4*>(qko + t * RR + k8) = o;
                }
            } else {
                for (int e = tid; e < cl * RR; e += NTHR) {
                    const int t = e / RR, rr = e % RR;
                    const int r = rr / R, r2 = rr % R;
                    qko[e] = bits16(sQK[t * QKS + r * RP + r2]);
                }
            }
        }
        bar();

        f32x4 acc[T::PW][RP];
        if (need_y) {
            // ---- inter = Q bf16(S), scaled by exp(da_cs[t]) per row; the bf16(S)
            // fragments of the wave's value tile serve every rank
#pragma unroll
            for (int ps = 0; ps < T::PW; ++ps) {
                const int pair = wave + ps * NW;
                const int tt = pair / PTT, pt = pair % PTT;
                const bool pok = T::PAIRS_FULL || pair < T::NPAIRS;
                u32x4 bS[NT / 32];
#pragma unroll
                for (int ks = 0; ks < NT / 32; ++ks)
                    bS[ks] = lds_ld<u32x4>(sSbT + (16 * pt + l16) * LDQ + 32 * ks + 8 * q4);
                const f32x4 e4 = lds_ld<f32x4>(sc + 16 * tt + 4 * q4);
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
                    if (pok && r < R) {
                        const int i16 = r * CT + tt;
#pragma unroll
                        for (int ks = 0; ks < NT / 32; ++ks)
                            a4 = mfma(lds_ld<u32x4>(sQ + (16 * i16 + l16) * LDQ + 32 * ks + 8 * q4), bS[ks], a4);
                        a4 *= e4;
                    }
                    acc[ps][r] = a4;
                }
            }
            // ---- causal block A^T = K~ Q^T, masked on token index, times exp(segsum), bf16.
            // The mask is applied with selects on values read unconditionally.
            u32x2 at[T::ATW];
#pragma unroll
            for (int w = 0; w < T::ATW; ++w) {
                const int u = wave + w * NW;
                at[w] = u32x2{0u, 0u};
                const int jt = u / MTT, i16 = u % MTT;
                const int ri = i16 / CT, rj = jt / CT;
                const int tti = i16 % CT, ttj = jt % CT;
                if ((T::AT_FULL || u < T::AT) && ri < R && rj < R && ttj <= tti) {
                    f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < NT / 32; ++ks) {
                        const u32x4 a = lds_ld<u32x4>(sK + (16 * jt + l16) * LDQ + 32 * ks + 8 * q4);
                        const u32x4 bb = lds_ld<u32x4>(sQ + (16 * i16 + l16) * LDQ + 32 * ks + 8 * q4);
                        a4 = mfma(a, bb, a4);
                    }
                    const int ti = 16 * tti + l16, tj0 = 16 * ttj + 4 * q4;
                    f32x4 e;
                    if constexpr (EX) {
                        e = lds_ld<f32x4>(sE + ti * (Cp + 4) + tj0);   // C == Cp: always inside the block
                    } else {
                        const int tic = min(ti, p.C - 1);
#pragma unroll
                        for (int v = 0; v < 4; ++v) e[v] = sE[tic * (p.C + 4) + min(tj0 + v, p.C - 1)];
                    }
                    float m[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const bool keep = ti < cl && ti > tj0 + v;
                        m[v] = keep ? a4[v] * e[v] : 0.f;
                    }
                    at[w] = u32x2{pk2(m[0], m[1]), pk2(m[2], m[3])};
                }
            }
            if constexpr (!SEPA) bar();   // every wave is done reading sQ (sA overlays it)
#pragma unroll
            for (int w = 0; w < T::ATW; ++w) {
                const int u = wave + w * NW;
                if (T::AT_FULL || u < T::AT) {
                    const int jt = u / MTT, i16 = u % MTT;
                    lds_st<u32x2>(sA + (16 * i16 + l16) * LDA + 16 * jt + 4 * q4, at[w]);
                }
            }
            bar();
            // ---- intra = A Psi, accumulated onto the scaled inter term; the Psi
            // fragments of the wave's value tile serve every rank
#pragma unroll
            for (int ps = 0; ps < T::PW; ++ps) {
                const int pair = wave + ps * NW;
                const int tt = pair / PTT, pt = pair % PTT;
                const bool pok = T::PAIRS_FULL || pair < T::NPAIRS;
                u32x4 bP[MT / 32];
#pragma unroll
                for (int ks = 0; ks < MT / 32; ++ks)
                    bP[ks] = lds_ld<u32x4>(sPsiT + (16 * pt + l16) * LDA + 32 * ks + 8 * q4);
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    if (pok && r < R) {
                        const int i16 = r * CT + tt;
                        f32x4 a4 = acc[ps][r];
#pragma unroll
                        for (int ks = 0; ks < MT / 32; ++ks)
                            a4 = mfma(lds_ld<u32x4>(sA + (16 * i16 + l16) * LDA + 32 * ks + 8 * q4), bP[ks], a4);
                        acc[ps][r] = a4;
                    }
                }
            }
            // the kappa^T pass writes the q tile, which no wave reads after the barrier above
            if constexpr (!SEPA) bar();   // every wave is done reading sA (it overlays that tile)
        }

        // ---- kappa^T = bf16(K~ * exp(da_cs_rev)), transposed, into R1: items (row
        // pair, 8 columns); the two rows of a column go out as one 4-byte write, and
        // consecutive lanes take consecutive row pairs (32 banks per 32 lanes)
        for (int e = tid; e < T::KAP_ITEMS; e += NTHR) {
            const int ip = e % (MT / 2), nn = (e / (MT / 2)) * 8;
            const int i = 2 * ip, r = i / Cp, t = i % Cp;
            const u32x4 xa = lds_ld<u32x4>(sK + i * LDQ + nn), xb = lds_ld<u32x4>(sK + (i + 1) * LDQ + nn);
            const bool rok = r < R;
            const float ea = (rok && t < cl) ? sc[2 * Cp + t] : 0.f;
            const float eb = (rok && t + 1 < cl) ? sc[2 * Cp + t + 1] : 0.f;
            unsigned short* dst = sKapT + nn * LDA + i;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                lds_st<unsigned>(dst + (2 * d) * LDA, pk2(lo16(xa[d]) * ea, lo16(xb[d]) * eb));
                lds_st<unsigned>(dst + (2 * d + 1) * LDA, pk2(hi16(xa[d]) * ea, hi16(xb[d]) * eb));
            }
        }
        bar();

        // ---- state update S <- S * exp(da_cs[last]) + kappa^T Psi; bf16 copy for the next chunk
        {
            const float dl = sc[4 * Cp];
#pragma unroll
            for (int w = 0; w < T::STW; ++w) {
                const int u = wave + w * NW;
                if (T::ST_FULL || u < T::ST) {
                    const int nt = u / PTT, pt = u % PTT;
                    f32x4 a4 = Sacc[w] * dl;
#pragma unroll
                    for (int ks = 0; ks < MT / 32; ++ks) {
                        const u32x4 a = lds_ld<u32x4>(sKapT + (16 * nt + l16) * LDA + 32 * ks + 8 * q4);
                        const u32x4 bb = lds_ld<u32x4>(sPsiT + (16 * pt + l16) * LDA + 32 * ks + 8 * q4);
                        a4 = mfma(a, bb, a4);
                    }
                    Sacc[w] = a4;
                }
            }
            emit_state();
        }

        if constexpr (NW == 4) __builtin_amdgcn_s_setprio(0);
        // ---- y = bf16(inter + intra + diag + d*Psi) and the gating gradients. Ranks
        // r >= R, tokens past the chunk's end and columns p >= P run on zero data
        // (zero Psi, qk pairs, projections, gate inputs and scales) and come out
        // as zero, so nothing here needs a bound.
        if (need_y) {
#pragma unroll
            for (int ps = 0; ps < T::PW; ++ps) {
                const int pair = wave + ps * NW;
                if (!T::PAIRS_FULL && pair >= T::NPAIRS) continue;
                const int tt = pair / PTT, pt = pair % PTT;
                const int pc = 16 * pt + l16;
                const int tb = 16 * tt + 4 * q4;   // first of this lane's 4 tokens
                float zr[4], dr[4];   // zero outside the chunk (buffer range)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    zr[v] = bf2f(zraw[ps][v]);
                    dr[v] = bf2f(draw[ps][v]);
                }
                float psi[RP][4];
#pragma unroll
                for (int r2 = 0; r2 < RP; ++r2) {
                    const u32x2 x = lds_ld<u32x2>(sPsiT + pc * LDA + r2 * Cp + tb);
                    psi[r2][0] = lo16(x[0]);
                    psi[r2][1] = hi16(x[0]);
                    psi[r2][2] = lo16(x[1]);
                    psi[r2][3] = hi16(x[1]);
                }
                const f32x4 gam4 = lds_ld<f32x4>(sc + Cp + tb);
                float dzc[4] = {0.f, 0.f, 0.f, 0.f};   // dz chain, or the layer output's rank sum
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    // diagonal: rank-ordered chain of bf16 products and bf16 sums, times gamma.
                    // The four tokens' chains advance together, one rank at a time, so that
                    // consecutive instructions are independent (a lone wave then issues at
                    // full rate); the operations of each chain are unchanged.
                    float qkv[4][RP], dg[4], y[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v)
#pragma unroll
                        for (int r2 = 0; r2 < RP; ++r2) qkv[v][r2] = sQK[(tb + v) * QKS + r * RP + r2];
#pragma unroll
                    for (int v = 0; v < 4; ++v) dg[v] = rnd(qkv[v][0] * psi[0][v]);
#pragma unroll
                    for (int r2 = 1; r2 < RP; ++r2) {
                        float pr[4];
#pragma unroll
                        for (int v = 0; v < 4; ++v) pr[v] = rnd(qkv[v][r2] * psi[r2][v]);
#pragma unroll
                        for (int v = 0; v < 4; ++v) dg[v] = rnd(dg[v] + pr[v]);
                    }
#pragma unroll
                    for (int v = 0; v < 4; ++v) dg[v] = rnd(dg[v] * gam4[v]);
#pragma unroll
                    for (int v = 0; v < 4; ++v) y[v] = rnd(__fmaf_rn(dval, psi[r][v], fadd(acc[ps][r][v], dg[v])));
                    if (p.fwd) {
                        // layer output: (y * bf16(mimo_o)) * silu(pz), summed over ranks in
                        // rank order (reduced) or stored per rank
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            float val = y[v];
                            if (p.reduce_o) val = fmul(val, co[ps][r]);
                            if (p.has_z) {
                                const float pz = zr[v] * cz[ps][r];
                                val = fmul(val, fmul(pz, sigmoid_fast(pz)));
                            }
                            if (p.reduce_o) {
                                dzc[v] = fadd(dzc[v], val);
                            } else if (stage_ranks) {
                                sDz[(r * Cp + tb + v) * (PT + 8) + pc] = bits16(rnd(val));
                            } else if (tb + v < cl && pc < p.P && r < R) {
                                const long oi = ((long)(b * p.S + c0 + tb + v) * R + r) * p.H * p.P + (long)h * p.P + pc;
                                p.o[oi] = bits16(rnd(val));
                            }
                        }
                    } else if (p.has_z) {
                        // gating, again the four tokens side by side; the dmimo sums keep
                        // their token order
                        float pz[4], sg[4], G[4], gz[4];
#pragma unroll
                        for (int v = 0; v < 4; ++v) pz[v] = zr[v] * cz[ps][r];
#pragma unroll
                        for (int v = 0; v < 4; ++v) sg[v] = sigmoid_fast(pz[v]);
                        if (p.reduce_o) {
#pragma unroll
                            for (int v = 0; v < 4; ++v) G[v] = rnd(rnd(dr[v] * co[ps][r]) * y[v]);
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                dmo[ps][r] = __fmaf_rn(fmul(y[v], fmul(pz[v], sg[v])), dr[v], dmo[ps][r]);
                        } else {
#pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                // per-rank dout [B,S,R,H,P]; lanes without a token read element 0
                                const bool okr = tb + v < cl && pc < p.P && r < R;
                                const long nb = ((long)(b * p.S + c0) * R + r) * p.H * p.P + (long)h * p.P;
                                const unsigned short raw = p.dout[okr ? nb + (long)(tb + v) * R * p.H * p.P + pc : 0];
                                G[v] = rnd((okr ? bf2f(raw) : 0.f) * y[v]);
                            }
                        }
#pragma unroll
                        for (int v = 0; v < 4; ++v) gz[v] = fmul(fmul(G[v], sg[v]), __fmaf_rn(pz[v], 1.0f - sg[v], 1.0f));
#pragma unroll
                        for (int v = 0; v < 4; ++v) dzc[v] = rnd(dzc[v] + fmul(gz[v], cz[ps][r]));
#pragma unroll
                        for (int v = 0; v < 4; ++v) dmz[ps][r] = __fmaf_rn(gz[v], zr[v], dmz[ps][r]);
                    } else if (p.reduce_o) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) dmo[ps][r] = __fmaf_rn(y[v], dr[v], dmo[ps][r]);
                    }
                }
                if (stage_out) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) sDz[(tb + v) * (PT + 8) + pc] = bits16(p.fwd ? rnd(dzc[v]) : dzc[v]);
                }
            }
        }
        // The gate inputs are consumed on every path, so that no load of them is
        // still pending when the next iteration reuses their registers (a pending
        // one would make that reuse wait for every load issued since, including
        // the prefetch).
#pragma unroll
        for (int ps = 0; ps < T::PW; ++ps)
#pragma unroll
            for (int v = 0; v < 4; ++v) asm volatile("" ::"v"(zraw[ps][v]), "v"(draw[ps][v]));
    }
    if (stage_out || stage_ranks) {
        // dz (or the layer output) of the segment's last chunk
        bar();
        const int cl_last = min(p.C, p.S - (c_end - 1) * p.C);
        if (stage_out) flush_dz<NTHR, PT>(p, out16, sDz, b, h, (c_end - 1) * p.C, cl_last);
        else flush_ranks<NTHR, PT>(p, sDz, Cp, b, h, (c_end - 1) * p.C, cl_last);
    }

    // ---- per-segment partial sums of dmimo_o / dmimo_z: reduce over the 4 lane groups
    if (need_y && !p.fwd) {
#pragma unroll
        for (int ps = 0; ps < T::PW; ++ps) {
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
            for (int ps = 0; ps < T::PW; ++ps) {
                const int pair = wave + ps * NW;
                const int pc = 16 * (pair % PTT) + l16;
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    if (pair < T::NPAIRS && r < R && q4 == 0 && pc < p.P) {
                        const long o = ((long)bh * p.nseg + seg) * R * p.P + (long)r * p.P + pc;
                        if (p.reduce_o) p.part_o[o] = dmo[ps][r];
                        if (p.has_z) p.part_z[o] = dmz[ps][r];
                    }
                }
            }
        } else {
            // the token tiles of one (rank, value tile) belong to different waves;
            // add them in token-tile order through LDS
            bar();
            float* red = reinterpret_cast<float*>(smem);   // [2][CT][RP][PT]
            constexpr int per = RP * PT;
#pragma unroll
            for (int ps = 0; ps < T::PW; ++ps) {
                const int pair = wave + ps * NW;
                const int tt = pair / PTT, pc = 16 * (pair % PTT) + l16;
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    if (pair < T::NPAIRS && q4 == 0) {
                        red[tt * per + r * PT + pc] = dmo[ps][r];
                        red[CT * per + tt * per + r * PT + pc] = dmz[ps][r];
                    }
                }
            }
            bar();
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

// The 9 (NT, PT) combinations of one (RP, CT) family, indexed 3 * idx(NT) + idx(PT)
// with idx(32, 64, 128) = 0, 1, 2: the generic instances and the shape-exact ones.
struct Family {
    kfn agg[9], agg_ex[9];
    kfn main[9], main_ex_rz[9], main_ex_fwd[9];
    kfn states[9], states_ex[9];   // the chunk pass of calls without y (k_agg in ST mode)
    int main_sa[9], main_ex_sa[9];  // extra dynamic LDS of the chunk pass (generic, shape-exact)
};

#define MIMO_NP_LIST(F, RP, CT)                                                                             \
    F(RP, CT, 32, 32), F(RP, CT, 32, 64), F(RP, CT, 32, 128), F(RP, CT, 64, 32), F(RP, CT, 64, 64),         \
        F(RP, CT, 64, 128), F(RP, CT, 128, 32), F(RP, CT, 128, 64), F(RP, CT, 128, 128)
#define MIMO_AGG_FN(RP, CT, NT, PT) k_agg<RP, CT, NT, PT, false>
#define MIMO_AGG_EX_FN(RP, CT, NT, PT) k_agg<RP, CT, NT, PT, true>
#define MIMO_MAIN_FN(RP, CT, NT, PT) k_main<RP, CT, NT, PT, false, -1>
#define MIMO_MAIN_EX1_FN(RP, CT, NT, PT) k_main<RP, CT, NT, PT, true, 1>
#define MIMO_MAIN_EX2_FN(RP, CT, NT, PT) k_main<RP, CT, NT, PT, true, 2>
#define MIMO_ST_FN(RP, CT, NT, PT) k_agg<RP, CT, NT, PT, false, true>
#define MIMO_ST_EX_FN(RP, CT, NT, PT) k_agg<RP, CT, NT, PT, true, true>
#define MIMO_SA_FN(RP, CT, NT, PT) Stage<RP, CT, NT, PT, true, false>::SA_BYTES
#define MIMO_SA_EX_FN(RP, CT, NT, PT) Stage<RP, CT, NT, PT, true, true>::SA_BYTES
#define MIMO_FAMILY(RP, CT)                                                                               \
    const Family* family_rp##RP##_ct##CT() {                                                              \
        static const Family f = {{MIMO_NP_LIST(MIMO_AGG_FN, RP, CT)},     {MIMO_NP_LIST(MIMO_AGG_EX_FN, RP, CT)}, \
                                 {MIMO_NP_LIST(MIMO_MAIN_FN, RP, CT)},    {MIMO_NP_LIST(MIMO_MAIN_EX1_FN, RP, CT)}, \
                                 {MIMO_NP_LIST(MIMO_MAIN_EX2_FN, RP, CT)}, \
                                 {MIMO_NP_LIST(MIMO_ST_FN, RP, CT)},      {MIMO_NP_LIST(MIMO_ST_EX_FN, RP, CT)}, \
                                 {MIMO_NP_LIST(MIMO_SA_FN, RP, CT)},      {MIMO_NP_LIST(MIMO_SA_EX_FN, RP, CT)}}; \
        return &f;                                                                                        \
    }
#define MIMO_DECL_FAMILY(RP, CT) const Family* family_rp##RP##_ct##CT();
MIMO_DECL_FAMILY(1, 1) MIMO_DECL_FAMILY(1, 2) MIMO_DECL_FAMILY(1, 4)
MIMO_DECL_FAMILY(2, 1) MIMO_DECL_FAMILY(2, 2) MIMO_DECL_FAMILY(2, 4)
MIMO_DECL_FAMILY(4, 1) MIMO_DECL_FAMILY(4, 2) MIMO_DECL_FAMILY(8, 1)

}  // namespace mimo
