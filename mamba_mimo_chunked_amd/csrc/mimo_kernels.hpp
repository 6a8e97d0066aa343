// Device code of the mamba_mimo_bwd_fwd HIP library: parameters, LDS layout,
// the per-chunk preparation stages and the two chunk kernels (templates over
// the tile shape). Instantiated per tile family in tiles_rp*_ct*.hip; the
// host side lives in mimo_bwd_fwd.hip.
//
// The arithmetic follows the Triton-Ascend mamba_mimo_bwd_fwd page's
// BF16-boundary PyTorch reference: bf16 (round to nearest even) at the same
// points, fp32 everywhere else. Two roundings are done by one
// v_cvt_pk_bf16_f32 whenever two independent values are ready together.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mimo_bwd_fwd.h"

namespace mimo {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTok = 64;  // tokens per chunk tile (Cp) at most

// ---------------------------------------------------------------- bf16 helpers
// bf16(a) in the low and bf16(b) in the high half, round to nearest even.
__device__ __forceinline__ unsigned pk2(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ float lo16(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi16(unsigned u) { return __uint_as_float(u & 0xffff0000u); }
// round two fp32 values to bf16 in place
__device__ __forceinline__ void rnd2(float& a, float& b) {
    const unsigned u = pk2(a, b);
    a = lo16(u);
    b = hi16(u);
}
__device__ __forceinline__ float rnd1(float a) { return lo16(pk2(a, 0.f)); }
__device__ __forceinline__ float bf2f(unsigned short u) { return __uint_as_float(static_cast<unsigned>(u) << 16); }
__device__ __forceinline__ unsigned short f2bf(float x) { return static_cast<unsigned short>(pk2(x, 0.f)); }

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
// a.lo*b.lo + a.hi*b.hi + c (bf16 pairs, fp32 accumulate)
__device__ __forceinline__ float dot2(unsigned a, unsigned b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
// logistic function: precise for the per-token controls, fast for the gate
__device__ __forceinline__ float sigmoid_precise(float x) { return 1.0f / (1.0f + expf(-x)); }
__device__ __forceinline__ float sigmoid_fast(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS accesses, not
// for its global memory traffic. __syncthreads() also waits for outstanding global
// loads into LDS (the staging prefetch below), which would serialise the prefetch
// with the chunk it is meant to overlap. The memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void bar() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <typename T>
__device__ __forceinline__ T lds_ld(const void* p) { return *reinterpret_cast<const T*>(p); }
template <typename T>
__device__ __forceinline__ void lds_st(void* p, T v) { *reinterpret_cast<T*>(p) = v; }

// ---------------------------------------------------------------- parameters
struct Params {
    int B, S, H, G, R, N, P, C, W, nc, L, nseg, rd;
    int F, nsub;    // the aggregate splits each segment but the last into F sub-segments of L/F chunks
    int reduce_o, has_z, has_d, need_y;
    const unsigned short *dout, *q, *k, *v, *z, *trap;
    const float *q_bias, *k_bias, *mimo_v, *mimo_o, *mimo_z, *angles, *da_cs, *da_cs_rev, *dt, *d, *segsum;
    float *dmimo_o, *dmimo_z;
    unsigned short *states, *dz, *qk_dot;
    float* agg;     // [B*H][nsub][N*P]: sub-segment state increments, then the states after each
    float* decay;   // [B*H][nsub]: product of the chunk decays of each sub-segment
    float* part_o;  // [B*H][nseg][R*P] partial dmimo_o (== dmimo_o when nseg == 1)
    float* part_z;  // [B*H][nseg][R*P] partial dmimo_z
};

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
    // work items that divide evenly over the waves need no bound check (the
    // compiler cannot see that wave < NW)
    static constexpr bool ST_FULL = ST % NW == 0;
    static constexpr bool AT_FULL = AT % NW == 0;
    static constexpr bool PAIRS_FULL = NPAIRS % NW == 0;
};

// LDS carve-up (byte offsets), shared by host and device. Every region but the
// last two depends only on the tile family (RP, CT, NT, PT), so inside a kernel
// their offsets and pitches are compile-time constants and one per-lane address
// register serves many accesses (the rest goes into the instructions' offset
// field). cos/sin and exp(segsum) are sized by the runtime C and W and come last.
struct Lds {
    int r1;   // bf16 [MT][LDQ] q (main) | [MT][LDA] causal block | [NT][LDA] kappa^T
    int r2;   // bf16 [MT][LDQ] k (main only)
    int r3;   // bf16 [PT][LDA] Psi^T
    int r4;   // bf16 [PT][LDQ] bf16(state)^T (main only)
    int qk;   // fp32 [Cp][RP*RP+1] qk_dot, zero for padded ranks, one pad word per token (main only)
    int dz;   // bf16 [Cp][PT+8] dz of the chunk, written out at the top of the next one (main only)
    int sc;   // fp32 [5][kTok] token scalars + chunk decay
    int tb;   // bf16 tables: q_bias [RP][NT], k_bias [RP][NT], mimo_v [RP][PT]
    int cs;   // fp32 [2][C][W] cos, sin
    int se;   // fp32 [C][C] exp(segsum) (main only)
    int total;
};

__host__ __device__ inline int align16(int x) { return (x + 15) & ~15; }

__host__ __device__ inline Lds lds_layout(int RP, int CT, int NT, int PT, int C, int W, bool main) {
    const int Cp = 16 * CT, MT = RP * Cp < 32 ? 32 : RP * Cp;
    const int ldq = NT + 8, lda = MT + 8;
    int r1 = NT * lda;
    if (main && MT * ldq > r1) r1 = MT * ldq;
    if (main && MT * lda > r1) r1 = MT * lda;
    Lds s;
    int off = 0;
    s.r1 = off; off += align16(r1 * 2);
    s.r2 = off; if (main) off += align16(MT * ldq * 2);
    s.r3 = off; off += align16(PT * lda * 2);
    s.r4 = off; if (main) off += align16(PT * ldq * 2);
    s.qk = off; if (main) off += align16(Cp * (RP * RP + 1) * 4);
    s.dz = off; if (main) off += align16(Cp * (PT + 8) * 2);
    s.sc = off; off += align16((5 * kTok + 4) * 4);
    s.tb = off; off += align16((2 * RP * NT + RP * PT) * 2);
    s.cs = off; off += align16(2 * C * W * 4);
    s.se = off; if (main) off += align16(C * C * 4);
    s.total = off;
    return s;
}

// ---------------------------------------------------------------- per-chunk inputs
// Everything one chunk reads from global memory, loaded in one go at the top
// of the chunk so that a single memory latency is paid per chunk.
template <int RP, int CT, int NT, int PT, bool MAIN>
struct ChunkIn {
    using T = Tile<RP, CT, NT, PT>;
    u32x4 q0[T::QK_IT], q1[T::QK_IT], k0[T::QK_IT], k1[T::QK_IT];   // columns col0.., N/2+col0..
    u32x4 v[T::PSI_IT];
    float dt0, dt1, tr0, tr1, cs, rev, dlast;
    float ang[T::ANG_IT];
    float seg[MAIN ? T::SEG_IT : 1];
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

// ROWS_FAST: consecutive threads take consecutive tile rows (the chunk-aggregate
// kernel writes kappa^T transposed straight from registers); otherwise the
// 8-column groups of one row are adjacent.
template <int RP, int CT, int NT, int PT, bool ROWS_FAST = false>
__device__ __forceinline__ void make_items(const Params& p, int g, Items<RP, CT, NT, PT>& it) {
    using T = Tile<RP, CT, NT, PT>;
    const int tid = threadIdx.x;
    const int ng = p.N / 16;
#pragma unroll
    for (int j = 0; j < T::QK_IT; ++j) {
        const int e = tid + j * T::NTHR;
        it.qk_row[j] = -1;
        it.qk_col[j] = 0;
        it.qk_off[j] = 0;
        if (e < T::MT * ng) {
            const int i = ROWS_FAST ? e % T::MT : e / ng;
            const int gg = ROWS_FAST ? e / T::MT : e - i * ng;
            const int r = i / T::Cp, t = i % T::Cp;
            it.qk_row[j] = i;
            it.qk_col[j] = 8 * gg;
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

// Global loads of chunk c (c0 = first token, cl = real tokens).
template <int RP, int CT, int NT, int PT, bool MAIN>
__device__ __forceinline__ void load_chunk(const Params& p, const Items<RP, CT, NT, PT>& it, int b, int h, int bh,
                                           int c, int c0, int cl, ChunkIn<RP, CT, NT, PT, MAIN>& in) {
    using T = Tile<RP, CT, NT, PT>;
    const int tid = threadIdx.x;
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

// ---------------------------------------------------------------- LDS staging of chunk inputs
// For tile families whose LDS leaves room for two workgroups per compute unit,
// the inputs of chunk c+1 are fetched straight into a staging area of LDS
// (global_load_lds: lane l of a wave writes its 4 or 16 bytes at base + 4l or
// base + 16l; a 2-byte load fills the low half of the lane's 4-byte slot)
// while chunk c computes. Each thread later reads back exactly the slots it
// fetched, so only its own outstanding loads have to be waited for.
template <int RP, int CT, int NT, int PT, bool MAIN>
struct Stage {
    using T = Tile<RP, CT, NT, PT>;
    static constexpr int NQ = MAIN ? 4 : 2;   // q0, q1, k0, k1 (or k0, k1)
    static constexpr int QK = 0;
    static constexpr int V = QK + T::QK_IT * NQ * T::NTHR * 16;
    static constexpr int ANG = V + T::PSI_IT * T::NTHR * 16;
    static constexpr int SEG = ANG + T::ANG_IT * T::NTHR * 4;
    static constexpr int SCAL = SEG + (MAIN ? T::SEG_IT * T::NTHR * 4 : 0);   // [7][64] dwords, wave 0
    static constexpr int BYTES = SCAL + 7 * 64 * 4;
    // dynamic LDS of the family at its largest chunk (C = Cp, R = RP, N = NT, P = PT)
    static constexpr int ldq = NT + 8, lda = T::MT + 8;
    static constexpr int r1 = (MAIN ? ((T::MT * ldq > NT * lda ? T::MT * ldq : NT * lda) > T::MT * lda
                                           ? (T::MT * ldq > NT * lda ? T::MT * ldq : NT * lda)
                                           : T::MT * lda)
                                     : NT * lda);
    static constexpr int DYN = 2 * r1 + (MAIN ? 2 * T::MT * ldq : 0) + 2 * PT * lda + (MAIN ? 2 * PT * ldq : 0) +
                               8 * T::Cp * (NT / 2) +
                               (MAIN ? 4 * T::Cp * T::Cp + 4 * T::Cp * (RP * RP + 1) + 2 * T::Cp * (PT + 8) : 0) +
                               4 * (5 * kTok + 4) + 2 * (2 * RP * NT + RP * PT) + 256;
    static constexpr bool ON = DYN + BYTES <= 80 * 1024;
};


// One global_load_lds per lane: 16, 4 or 2 bytes from base + off (base the same
// for every lane, off a 32-bit byte offset) into the wave's LDS block at dst_wave
// (M0 holds its LDS address: the low 32 bits of a generic pointer into LDS are
// the LDS byte address, the high half being the shared aperture). Written as inline assembly so that the compiler's
// wait-count tracking does not treat the address registers as pending until the
// load completes (it would then wait for the whole prefetch as soon as such a
// register is reused). The waits are explicit instead: s_waitcnt vmcnt(0) before
// a thread reads its staged slots, and lgkmcnt(0) after the reads, before the
// next prefetch overwrites them. M0 is saved and restored around the load; an
// SALU write of M0 needs one wait state before an LDS DMA.
// A wave-uniform pointer, pinned to scalar registers (a no-op when it already is).
// readfirstlane returns int: each half goes through unsigned so that it is
// zero-extended, never sign-extended, into the 64-bit address.
__device__ __forceinline__ unsigned rfl(unsigned x) { return static_cast<unsigned>(__builtin_amdgcn_readfirstlane(x)); }
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

// Issue the staging loads of chunk c (first token c0, cl real tokens). Every
// address is a scalar chunk base plus a per-lane offset that does not change
// from chunk to chunk.
template <int RP, int CT, int NT, int PT, bool MAIN>
__device__ __forceinline__ void prefetch_chunk(const Params& p, const Items<RP, CT, NT, PT>& it, int b, int h, int bh,
                                               int c, int c0, int cl, unsigned char* stg) {
    using T = Tile<RP, CT, NT, PT>;
    using SG = Stage<RP, CT, NT, PT, MAIN>;
    const int tid = threadIdx.x, wave = tid >> 6;
    const int R = p.R;
    const unsigned short* qb = p.q + (long)(b * p.S + c0) * R * p.G * p.N;
    const unsigned short* kb = p.k + (long)(b * p.S + c0) * R * p.G * p.N;
#pragma unroll
    for (int j = 0; j < T::QK_IT; ++j) {
        const int i = it.qk_row[j];
        const int r = i / T::Cp, t = i % T::Cp;
        unsigned char* d = stg + SG::QK + (j * SG::NQ) * T::NTHR * 16 + wave * 1024;
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
    const unsigned short* vb = p.v + ((long)(b * p.S + c0) * p.H + h) * p.P;
#pragma unroll
    for (int j = 0; j < T::PSI_IT; ++j) {
        const int e = tid + j * T::NTHR;
        const int t = e % T::Cp, pc = (e / T::Cp) * 8;
        if (e < T::Cp * (PT / 8) && t < cl && pc < p.P)
            dma16(vb, it.v_off[j], stg + SG::V + j * T::NTHR * 16 + wave * 1024);
    }
    const float* ab = p.angles + ((long)(b * p.S + c0) * p.H + h) * p.W;
#pragma unroll
    for (int j = 0; j < T::ANG_IT; ++j)
        if (it.ang_t[j] >= 0 && it.ang_t[j] < cl) dma4(ab, it.ang_off[j], stg + SG::ANG + j * T::NTHR * 4 + wave * 256);
    if (MAIN && p.need_y) {
        const float* sb = p.segsum + ((long)bh * p.nc + c) * p.C * p.C;
#pragma unroll
        for (int j = 0; j < T::SEG_IT; ++j) {
            const int e = tid + j * T::NTHR;
            if (e < p.C * p.C) dma4(sb, 4u * e, stg + SG::SEG + j * T::NTHR * 4 + wave * 256);
        }
    }
    if (wave == 0) {
        const long tok = (long)bh * p.S + c0;
        unsigned char* sc = stg + SG::SCAL;
        const unsigned o4 = 4u * tid, o2 = 2u * tid;
        if (tid < cl) {
            dma4(p.dt + tok, o4, sc);
            dma2(p.trap + tok, o2, sc + 2 * 256);
            dma4(p.da_cs_rev + tok, o4, sc + 5 * 256);
            if (MAIN) dma4(p.da_cs + tok, o4, sc + 4 * 256);
            if (c0 + tid + 1 < p.S) {
                dma4(p.dt + tok + 1, o4, sc + 1 * 256);
                dma2(p.trap + tok + 1, o2, sc + 3 * 256);
            }
        }
        if (tid == 0) dma4(p.da_cs + tok + cl - 1, 0u, sc + 6 * 256);
    }
}

// Copy this thread's staged slots of the current chunk into registers.
template <int RP, int CT, int NT, int PT, bool MAIN>
__device__ __forceinline__ void read_stage(const unsigned char* stg, ChunkIn<RP, CT, NT, PT, MAIN>& in) {
    using T = Tile<RP, CT, NT, PT>;
    using SG = Stage<RP, CT, NT, PT, MAIN>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < T::QK_IT; ++j) {
        const unsigned char* d = stg + SG::QK + (j * SG::NQ) * T::NTHR * 16 + tid * 16;
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
#pragma unroll
    for (int j = 0; j < T::PSI_IT; ++j) in.v[j] = lds_ld<u32x4>(stg + SG::V + j * T::NTHR * 16 + tid * 16);
#pragma unroll
    for (int j = 0; j < T::ANG_IT; ++j) in.ang[j] = lds_ld<float>(stg + SG::ANG + j * T::NTHR * 4 + tid * 4);
    if (MAIN) {
#pragma unroll
        for (int j = 0; j < (MAIN ? T::SEG_IT : 0); ++j)
            in.seg[j] = lds_ld<float>(stg + SG::SEG + j * T::NTHR * 4 + tid * 4);
    }
    if (tid < 64) {
        const unsigned char* sc = stg + SG::SCAL + tid * 4;
        in.dt0 = lds_ld<float>(sc);
        in.dt1 = lds_ld<float>(sc + 256);
        in.tr0 = bf2f(static_cast<unsigned short>(lds_ld<unsigned>(sc + 2 * 256)));
        in.tr1 = bf2f(static_cast<unsigned short>(lds_ld<unsigned>(sc + 3 * 256)));
        if (MAIN) in.cs = lds_ld<float>(sc + 4 * 256);
        in.rev = lds_ld<float>(sc + 5 * 256);
        in.dlast = lds_ld<float>(stg + SG::SCAL + 6 * 256);
    }
}

// Phase 0: token scalars, cos/sin, exp(segsum) into LDS.
// gamma_t = bf16(dt_t) * sigmoid(trap_t)                      (fp32)
// beta_t  = bf16(bf16(dt_{t+1}) * sigmoid(-trap_{t+1})), 0 at the last token
// factor_t = bf16(gamma_t + beta_t)
template <int RP, int CT, int NT, int PT, bool MAIN>
__device__ __forceinline__ void phase0(const Params& p, const Items<RP, CT, NT, PT>& it, int c0, int cl,
                                       const ChunkIn<RP, CT, NT, PT, MAIN>& in, unsigned char* smem, const Lds& L) {
    using T = Tile<RP, CT, NT, PT>;
    const int tid = threadIdx.x;
    float* sc = reinterpret_cast<float*>(smem + L.sc);
    if (tid < T::Cp) {
        float gam = 0.f, fac = 0.f, ecs = 0.f, erev = 0.f;
        if (tid < cl) {
            gam = rnd1(in.dt0) * sigmoid_precise(in.tr0);
            float beta = 0.f;
            if (c0 + tid + 1 < p.S) beta = rnd1(rnd1(in.dt1) * sigmoid_precise(-in.tr1));
            fac = rnd1(gam + beta);
            erev = expf(in.rev);
            if (MAIN) ecs = expf(in.cs);
        }
        sc[tid] = ecs;
        sc[kTok + tid] = gam;
        sc[2 * kTok + tid] = erev;
        sc[3 * kTok + tid] = fac;
    }
    if (tid == 0) sc[4 * kTok] = expf(in.dlast);
    float* scs = reinterpret_cast<float*>(smem + L.cs);
    const int CW = p.C * p.W;
#pragma unroll
    for (int j = 0; j < T::ANG_IT; ++j) {
        const int e = tid + j * T::NTHR;
        if (e < CW) {
            float s = 0.f, co = 0.f;
            if (it.ang_t[j] < cl) sincosf(in.ang[j], &s, &co);
            scs[e] = co;
            scs[CW + e] = s;
        }
    }
    if (MAIN && p.need_y) {
        float* se = reinterpret_cast<float*>(smem + L.se);
#pragma unroll
        for (int j = 0; j < T::SEG_IT; ++j) {
            const int e = tid + j * T::NTHR;
            if (e < p.C * p.C) se[e] = expf(in.seg[j]);
        }
    }
}

// bias + round of one 8-column group: bf16(x + bf16(bias)), packed
__device__ __forceinline__ u32x4 add_bias(u32x4 x, u32x4 bias) {
    u32x4 o;
#pragma unroll
    for (int d = 0; d < 4; ++d) o[d] = pk2(lo16(x[d]) + lo16(bias[d]), hi16(x[d]) + hi16(bias[d]));
    return o;
}

// Rotate the column pairs (col0 + e, N/2 + col0 + e) of one group: a is the
// first-half group, e the second; both packed bf16, rounded after rotation.
__device__ __forceinline__ void rotate_group(u32x4& a, u32x4& e, int col0, int W, const float* cs, const float* sn) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int n = col0 + 2 * d;
        if (n < W) {
            const float x0 = lo16(a[d]), x1 = hi16(a[d]);
            const float y0 = lo16(e[d]), y1 = hi16(e[d]);
            const float c0 = cs[n], c1 = cs[n + 1], s0 = sn[n], s1 = sn[n + 1];
            a[d] = pk2(__fmul_rn(c0, x0) - __fmul_rn(s0, y0), __fmul_rn(c1, x1) - __fmul_rn(s1, y1));
            e[d] = pk2(__fmul_rn(s0, x0) + __fmul_rn(c0, y0), __fmul_rn(s1, x1) + __fmul_rn(c1, y1));
        }
    }
}

__device__ __forceinline__ u32x4 scale_group(u32x4 a, float f) {
    u32x4 o;
#pragma unroll
    for (int d = 0; d < 4; ++d) o[d] = pk2(lo16(a[d]) * f, hi16(a[d]) * f);
    return o;
}

// Psi^T: sPsiT[p][r*Cp + t] = bf16(v[t,p] * bf16(mimo_v[r,p])), zero for padded tokens and columns.
template <int RP, int CT, int NT, int PT, bool MAIN>
__device__ __forceinline__ void fill_psi(const Params& p, int cl, const ChunkIn<RP, CT, NT, PT, MAIN>& in,
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
        for (int r = 0; r < p.R; ++r) {
            unsigned short* dst = sPsiT + pc * T::LDA + r * T::Cp + t;
            if (real) {
                const u32x4 mv = lds_ld<u32x4>(smv + r * PT + pc);
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const unsigned u = pk2(lo16(in.v[j][d]) * lo16(mv[d]), hi16(in.v[j][d]) * hi16(mv[d]));
                    dst[(2 * d) * T::LDA] = static_cast<unsigned short>(u);
                    dst[(2 * d + 1) * T::LDA] = static_cast<unsigned short>(u >> 16);
                }
            } else {
#pragma unroll
                for (int d = 0; d < 8; ++d) dst[d * T::LDA] = 0;
            }
        }
    }
}

// Tables filled once per workgroup: bf16(q_bias), bf16(k_bias), bf16(mimo_v) for head h,
// and the zero padding of Psi^T that no chunk overwrites.
template <int RP, int CT, int NT, int PT>
__device__ __forceinline__ void fill_tables(const Params& p, int h, unsigned char* smem, const Lds& L) {
    using T = Tile<RP, CT, NT, PT>;
    const int tid = threadIdx.x;
    unsigned short* tb = reinterpret_cast<unsigned short*>(smem + L.tb);   // [RP][NT] x2, [RP][PT]
    const int RN = p.R * p.N, RPn = p.R * p.P;
    for (int e = tid; e < RN; e += T::NTHR) {
        const int r = e / p.N, n = e - r * p.N;
        tb[r * NT + n] = f2bf(p.q_bias[(long)h * RN + e]);
        tb[RP * NT + r * NT + n] = f2bf(p.k_bias[(long)h * RN + e]);
    }
    for (int e = tid; e < RPn; e += T::NTHR) {
        const int r = e / p.P, pc = e - r * p.P;
        tb[2 * RP * NT + r * PT + pc] = f2bf(p.mimo_v[(long)h * RPn + e]);
    }
    unsigned short* sPsiT = reinterpret_cast<unsigned short*>(smem + L.r3);
    const int used = p.R * T::Cp, pad = T::MT - used;
    for (int e = tid; e < PT * pad; e += T::NTHR) {
        const int pp = e / pad, i = used + e % pad;
        sPsiT[pp * T::LDA + i] = 0;
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
// dout with z. Returns the parameters with those fields replaced by constants.
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
    }
    if constexpr (MODE == 1) {
        p.need_y = 1;
        p.reduce_o = 1;
        p.has_z = 1;
    }
    return p;
}

// ---------------------------------------------------------------- segment aggregate
// U_s = state added by segment s from a zero start: U <- U*exp(da_cs[last]) + kappa^T Psi
// per chunk; also the product of the chunk decays.
template <int RP, int CT, int NT, int PT, bool EX>
__global__ __launch_bounds__((Tile<RP, CT, NT, PT>::NTHR), 2) void k_agg(Params pin) {
    const Params p = specialise<RP, CT, NT, PT, EX, -1>(pin);
    using T = Tile<RP, CT, NT, PT>;
    extern __shared__ __align__(16) unsigned char smem[];
    const Lds L = lds_layout(RP, CT, NT, PT, p.C, p.W, false);
    unsigned short* sKapT = reinterpret_cast<unsigned short*>(smem + L.r1);
    const unsigned short* sPsiT = reinterpret_cast<const unsigned short*>(smem + L.r3);
    const float* sc = reinterpret_cast<const float*>(smem + L.sc);
    const float* scs = reinterpret_cast<const float*>(smem + L.cs);
    const unsigned short* tbk = reinterpret_cast<const unsigned short*>(smem + L.tb) + RP * NT;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    int seg, bh;
    if (!map_block(p, p.nsub, seg, bh)) return;
    const int b = bh / p.H, h = bh - b * p.H;
    const int g = h / (p.H / p.G);
    const int La = p.L / p.F;   // chunks per sub-segment (all full)
    const int c_begin = seg * La;
    const int c_end = c_begin + La;
    const int R = p.R;

    Items<RP, CT, NT, PT> it;
    make_items<RP, CT, NT, PT, true>(p, g, it);
    fill_tables<RP, CT, NT, PT>(p, h, smem, L);
    // kappa^T columns beyond the real rows, and rows n >= N, stay zero
    for (int e = tid; e < NT * T::MT; e += T::NTHR) sKapT[e / T::MT * T::LDA + e % T::MT] = 0;

    using SG = Stage<RP, CT, NT, PT, false>;
    __shared__ __align__(16) unsigned char stg[SG::ON ? SG::BYTES : 16];
    if constexpr (SG::ON) prefetch_chunk<RP, CT, NT, PT, false>(p, it, b, h, bh, c_begin, c_begin * p.C, min(p.C, p.S - c_begin * p.C), stg);

    f32x4 U[T::STW];
#pragma unroll
    for (int w = 0; w < T::STW; ++w) U[w] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dprod = 1.f;

    for (int c = c_begin; c < c_end; ++c) {
        const int c0 = c * p.C;
        const int cl = min(p.C, p.S - c0);
        ChunkIn<RP, CT, NT, PT, false> in = {};
        if constexpr (SG::ON) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's staging loads
            read_stage(stg, in);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (c + 1 < c_end) prefetch_chunk<RP, CT, NT, PT, false>(p, it, b, h, bh, c + 1, c0 + p.C, min(p.C, p.S - c0 - p.C), stg);
        } else {
            load_chunk(p, it, b, h, bh, c, c0, cl, in);
        }
        bar();   // previous chunk done with LDS (and tables written)
        phase0(p, it, c0, cl, in, smem, L);
        bar();
        // kappa^T = bf16(bf16(rot(bf16(k + bf16(k_bias))) * factor) * exp(da_cs_rev)), transposed
#pragma unroll
        for (int j = 0; j < T::QK_IT; ++j) {
            const int i = it.qk_row[j];
            if (i < 0) continue;
            const int r = i / T::Cp, t = i % T::Cp;
            if (r >= R || t >= cl) continue;   // stays zero from the initial fill / last chunk
            const int col0 = it.qk_col[j], col1 = p.N / 2 + col0;
            u32x4 a = add_bias(in.k0[j], lds_ld<u32x4>(tbk + r * NT + col0));
            u32x4 e = add_bias(in.k1[j], lds_ld<u32x4>(tbk + r * NT + col1));
            rotate_group(a, e, col0, p.W, scs + t * p.W, scs + p.C * p.W + t * p.W);
            const float f = sc[3 * kTok + t], er = sc[2 * kTok + t];
            a = scale_group(scale_group(a, f), er);
            e = scale_group(scale_group(e, f), er);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                sKapT[(col0 + 2 * d) * T::LDA + i] = static_cast<unsigned short>(a[d]);
                sKapT[(col0 + 2 * d + 1) * T::LDA + i] = static_cast<unsigned short>(a[d] >> 16);
                sKapT[(col1 + 2 * d) * T::LDA + i] = static_cast<unsigned short>(e[d]);
                sKapT[(col1 + 2 * d + 1) * T::LDA + i] = static_cast<unsigned short>(e[d] >> 16);
            }
        }
        if (cl < p.C) {
            // tail chunk: rows of tokens beyond the sequence are zero
            for (int e = tid; e < NT * T::MT; e += T::NTHR) {
                const int i = e % T::MT;
                if (i % T::Cp >= cl) sKapT[e / T::MT * T::LDA + i] = 0;
            }
        }
        fill_psi(p, cl, in, smem, L);
        bar();
        const float dl = sc[4 * kTok];
#pragma unroll
        for (int w = 0; w < T::STW; ++w) {
            const int u = wave + w * T::NW;
            if (T::ST_FULL || u < T::ST) {
                const int nt = u / T::PTT, pt = u % T::PTT;
                f32x4 acc = U[w] * dl;
#pragma unroll
                for (int ks = 0; ks < T::MT / 32; ++ks) {
                    const u32x4 a = lds_ld<u32x4>(sKapT + (16 * nt + l16) * T::LDA + 32 * ks + 8 * q4);
                    const u32x4 bb = lds_ld<u32x4>(sPsiT + (16 * pt + l16) * T::LDA + 32 * ks + 8 * q4);
                    acc = mfma(a, bb, acc);
                }
                U[w] = acc;
            }
        }
        dprod *= dl;
    }
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
template <int NTHR, int PT>
__device__ __forceinline__ void flush_dz(const Params& p, const unsigned short* sDz, int b, int h, int c0, int cl) {
    const int P8 = p.P / 8;
    unsigned short* dst = p.dz + ((long)(b * p.S + c0) * p.H + h) * p.P;
    for (int e = threadIdx.x; e < cl * P8; e += NTHR) {
        const int t = e / P8, pc = (e - t * P8) * 8;
        *reinterpret_cast<u32x4*>(dst + (long)t * p.H * p.P + pc) = lds_ld<u32x4>(sDz + t * (PT + 8) + pc);
    }
}

template <int RP, int CT, int NT, int PT, bool EX, int MODE>
__global__ __launch_bounds__((Tile<RP, CT, NT, PT>::NTHR), 2) void k_main(Params pin) {
    const Params p = specialise<RP, CT, NT, PT, EX, MODE>(pin);
    using T = Tile<RP, CT, NT, PT>;
    constexpr int MT = T::MT, NW = T::NW, NTHR = T::NTHR, Cp = T::Cp;
    constexpr int LDQ = T::LDQ, LDA = T::LDA, PTT = T::PTT, MTT = T::MTT;
    extern __shared__ __align__(16) unsigned char smem[];
    const Lds L = lds_layout(RP, CT, NT, PT, p.C, p.W, true);
    unsigned short* sQ = reinterpret_cast<unsigned short*>(smem + L.r1);   // also sA, sKapT
    unsigned short* sA = sQ;
    unsigned short* sKapT = sQ;
    unsigned short* sK = reinterpret_cast<unsigned short*>(smem + L.r2);
    unsigned short* sPsiT = reinterpret_cast<unsigned short*>(smem + L.r3);
    unsigned short* sSbT = reinterpret_cast<unsigned short*>(smem + L.r4);
    const float* scs = reinterpret_cast<const float*>(smem + L.cs);
    const float* sE = reinterpret_cast<const float*>(smem + L.se);
    float* sQK = reinterpret_cast<float*>(smem + L.qk);
    unsigned short* sDz = reinterpret_cast<unsigned short*>(smem + L.dz);
    constexpr int QKS = RP * RP + 1;   // sQK pitch per token
    const float* sc = reinterpret_cast<const float*>(smem + L.sc);
    const unsigned short* tbq = reinterpret_cast<const unsigned short*>(smem + L.tb);
    const unsigned short* tbk = tbq + RP * NT;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    int seg, bh;
    if (!map_block(p, p.nseg, seg, bh)) return;
    const int b = bh / p.H, h = bh - b * p.H;
    const int g = h / (p.H / p.G);
    const int c_begin = seg * p.L;
    const int c_end = min(c_begin + p.L, p.nc);
    const int R = p.R;
    const bool need_y = p.need_y;

    Items<RP, CT, NT, PT> it;
    make_items(p, g, it);
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
                if (p.reduce_o) co[ps][r] = rnd1(p.mimo_o[((long)h * R + r) * p.P + pc]);
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
    using SG = Stage<RP, CT, NT, PT, true>;
    __shared__ __align__(16) unsigned char stg[SG::ON ? SG::BYTES : 16];
    if constexpr (SG::ON) prefetch_chunk<RP, CT, NT, PT, true>(p, it, b, h, bh, c_begin, c_begin * p.C, min(p.C, p.S - c_begin * p.C), stg);

    for (int c = c_begin; c < c_end; ++c) {
        const int c0 = c * p.C;
        const int cl = min(p.C, p.S - c0);

        ChunkIn<RP, CT, NT, PT, true> in = {};
        if constexpr (SG::ON) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's staging loads
            read_stage(stg, in);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (c + 1 < c_end) prefetch_chunk<RP, CT, NT, PT, true>(p, it, b, h, bh, c + 1, c0 + p.C, min(p.C, p.S - c0 - p.C), stg);
        } else {
            load_chunk(p, it, b, h, bh, c, c0, cl, in);
        }
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
            const auto zb = buffer((p.has_z ? p.z : (need_y ? p.dout : p.v)) + base, bytes);
            const auto db = p.reduce_o ? buffer(p.dout + base, bytes) : zb;
#pragma unroll
            for (int ps = 0; ps < T::PW; ++ps) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    zraw[ps][v] = __builtin_amdgcn_raw_buffer_load_b16(zb, gate_off[ps][v], 0, 0);
                    draw[ps][v] = __builtin_amdgcn_raw_buffer_load_b16(db, gate_off[ps][v], 0, 0);
                }
            }
        }
        bar();   // previous chunk (and the tables) done

        // ---- states[c] = bf16(S entering chunk c), from sSbT ([p][n]) to [n][p], 16 bytes a thread
        {
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
        if (p.has_z && c > c_begin) flush_dz<NTHR, PT>(p, sDz, b, h, c0 - p.C, p.C);

        // ---- phase 0: token scalars, cos/sin, exp(segsum)
        phase0(p, it, c0, cl, in, smem, L);
        bar();

        // ---- phase A: biased q/k (unrotated into LDS, rotated kept in registers), Psi^T
        u32x4 rq0[T::QK_IT], rq1[T::QK_IT], rk0[T::QK_IT], rk1[T::QK_IT];
#pragma unroll
        for (int j = 0; j < T::QK_IT; ++j) {
            const int i = it.qk_row[j];
            if (i < 0) continue;
            const int r = i / Cp, t = i % Cp;
            const int col0 = it.qk_col[j], col1 = p.N / 2 + col0;
            u32x4 qa = {0u, 0u, 0u, 0u}, qb = qa, ka = qa, kb = qa;
            if (r < R && t < cl) {
                qa = add_bias(in.q0[j], lds_ld<u32x4>(tbq + r * NT + col0));
                qb = add_bias(in.q1[j], lds_ld<u32x4>(tbq + r * NT + col1));
                ka = add_bias(in.k0[j], lds_ld<u32x4>(tbk + r * NT + col0));
                kb = add_bias(in.k1[j], lds_ld<u32x4>(tbk + r * NT + col1));
            }
            lds_st<u32x4>(sQ + i * LDQ + col0, qa);
            lds_st<u32x4>(sQ + i * LDQ + col1, qb);
            lds_st<u32x4>(sK + i * LDQ + col0, ka);
            lds_st<u32x4>(sK + i * LDQ + col1, kb);
            if (r < R && t < cl) {
                const float* cs = scs + t * p.W;
                const float* sn = scs + p.C * p.W + t * p.W;
                rotate_group(qa, qb, col0, p.W, cs, sn);
                rotate_group(ka, kb, col0, p.W, cs, sn);
                const float f = sc[3 * kTok + t];
                ka = scale_group(ka, f);
                kb = scale_group(kb, f);
            }
            rq0[j] = qa;
            rq1[j] = qb;
            rk0[j] = ka;
            rk1[j] = kb;
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
        fill_psi(p, cl, in, smem, L);
        bar();

        // ---- phase B: qk_dot of the same token (biased, unrotated), fp32 accumulate;
        // padded rank pairs get zero
        {
            const int RR = R * R;
            unsigned short* qko = p.qk_dot + ((long)bh * p.S + c0) * RR;
            for (int e = tid; e < cl * RP * RP; e += NTHR) {
                const int rr = e / cl, t = e - rr * cl;   // consecutive threads: consecutive tokens
                const int r = rr / RP, r2 = rr % RP;
                float sum = 0.f;
                if (r < R && r2 < R) {
                    const unsigned short* xq = sQ + (r * Cp + t) * LDQ;
                    const unsigned short* xk = sK + (r2 * Cp + t) * LDQ;
                    for (int n = 0; n < p.N; n += 8) {
                        const u32x4 a = lds_ld<u32x4>(xq + n), bb = lds_ld<u32x4>(xk + n);
                        sum = dot2(a[0], bb[0], sum);
                        sum = dot2(a[1], bb[1], sum);
                        sum = dot2(a[2], bb[2], sum);
                        sum = dot2(a[3], bb[3], sum);
                    }
                    const unsigned u = pk2(sum, 0.f);
                    sum = lo16(u);
                    qko[t * RR + r * R + r2] = static_cast<unsigned short>(u);
                }
                sQK[t * QKS + rr] = sum;
            }
        }
        bar();

        // ---- phase C: rotated q and factor-scaled k into LDS
#pragma unroll
        for (int j = 0; j < T::QK_IT; ++j) {
            const int i = it.qk_row[j];
            if (i < 0) continue;
            const int col0 = it.qk_col[j], col1 = p.N / 2 + col0;
            if (need_y) {
                lds_st<u32x4>(sQ + i * LDQ + col0, rq0[j]);
                lds_st<u32x4>(sQ + i * LDQ + col1, rq1[j]);
            }
            lds_st<u32x4>(sK + i * LDQ + col0, rk0[j]);
            lds_st<u32x4>(sK + i * LDQ + col1, rk1[j]);
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
                        e = lds_ld<f32x4>(sE + ti * Cp + tj0);   // C == Cp: always inside the block
                    } else {
                        const int tic = min(ti, p.C - 1);
#pragma unroll
                        for (int v = 0; v < 4; ++v) e[v] = sE[tic * p.C + min(tj0 + v, p.C - 1)];
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
            bar();   // every wave is done reading sQ
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
            bar();   // every wave is done reading sA
        }

        // ---- kappa^T = bf16(K~ * exp(da_cs_rev)), transposed, into R1
        {
            constexpr int n8 = NT / 8;
            for (int e = tid; e < MT * n8; e += NTHR) {
                const int i = e % MT, nn = (e / MT) * 8;   // consecutive threads: consecutive rows
                const int r = i / Cp, t = i % Cp;
                const u32x4 x = lds_ld<u32x4>(sK + i * LDQ + nn);
                const float er = (r < R && t < cl) ? sc[2 * kTok + t] : 0.f;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const unsigned u = pk2(lo16(x[d]) * er, hi16(x[d]) * er);
                    sKapT[(nn + 2 * d) * LDA + i] = static_cast<unsigned short>(u);
                    sKapT[(nn + 2 * d + 1) * LDA + i] = static_cast<unsigned short>(u >> 16);
                }
            }
        }
        bar();

        // ---- state update S <- S * exp(da_cs[last]) + kappa^T Psi; bf16 copy for the next chunk
        {
            const float dl = sc[4 * kTok];
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

        // ---- y = bf16(inter + intra + diag + d*Psi) and the gating gradients. Ranks
        // r >= R run on zero data (zero Psi rows, qk pairs and projections) and add
        // nothing, so the rank loops need no bounds.
        if (need_y) {
#pragma unroll
            for (int ps = 0; ps < T::PW; ++ps) {
                const int pair = wave + ps * NW;
                if (!T::PAIRS_FULL && pair >= T::NPAIRS) continue;
                const int tt = pair / PTT, pt = pair % PTT;
                const int pc = 16 * pt + l16;
                const int tb = 16 * tt + 4 * q4;   // first of this lane's 4 tokens
                bool ok[4];
                float zr[4], dr[4];   // zero outside the chunk (buffer range)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    ok[v] = tb + v < cl && pc < p.P;
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
                const f32x4 gam4 = lds_ld<f32x4>(sc + kTok + tb);
                float dzc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    // diagonal of two tokens at a time: rank-ordered bf16 products and sums
                    float y[4];
#pragma unroll
                    for (int vp = 0; vp < 2; ++vp) {
                        const int va = 2 * vp, vb = va + 1;
                        const float* qa = sQK + (tb + va) * QKS + r * RP;
                        const float* qb = sQK + (tb + vb) * QKS + r * RP;
                        float da = qa[0] * psi[0][va], db = qb[0] * psi[0][vb];
                        rnd2(da, db);
#pragma unroll
                        for (int r2 = 1; r2 < RP; ++r2) {
                            float pa = qa[r2] * psi[r2][va], pb = qb[r2] * psi[r2][vb];
                            rnd2(pa, pb);
                            da += pa;
                            db += pb;
                            rnd2(da, db);
                        }
                        da *= gam4[va];
                        db *= gam4[vb];
                        rnd2(da, db);
                        float oa = acc[ps][r][va] + da, ob = acc[ps][r][vb] + db;
                        oa += dval * psi[r][va];
                        ob += dval * psi[r][vb];
                        rnd2(oa, ob);
                        // tokens past the chunk's end contribute nothing
                        y[va] = (tb + va < cl) ? oa : 0.f;
                        y[vb] = (tb + vb < cl) ? ob : 0.f;
                    }
                    if (p.has_z) {
                        float sg[4], pz[4], G[4], gz[4];
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            pz[v] = zr[v] * cz[ps][r];
                            sg[v] = sigmoid_fast(pz[v]);
                        }
                        if (p.reduce_o) {
#pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                dmo[ps][r] += (y[v] * (pz[v] * sg[v])) * dr[v];
                                G[v] = dr[v] * co[ps][r];
                            }
                            rnd2(G[0], G[1]);
                            rnd2(G[2], G[3]);
#pragma unroll
                            for (int v = 0; v < 4; ++v) G[v] *= y[v];
                        } else {
                            // per-rank dout [B,S,R,H,P]; lanes without a token read element 0
                            const long nb = ((long)(b * p.S + c0) * R + r) * p.H * p.P + (long)h * p.P;
#pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                const bool okr = ok[v] && r < R;
                                const unsigned short raw = p.dout[okr ? nb + (long)(tb + v) * R * p.H * p.P + pc : 0];
                                G[v] = (okr ? bf2f(raw) : 0.f) * y[v];
                            }
                        }
                        rnd2(G[0], G[1]);
                        rnd2(G[2], G[3]);
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            gz[v] = (G[v] * sg[v]) * (1.0f + pz[v] * (1.0f - sg[v]));
                            dzc[v] += __fmul_rn(gz[v], cz[ps][r]);
                            dmz[ps][r] += gz[v] * zr[v];
                        }
                        rnd2(dzc[0], dzc[1]);
                        rnd2(dzc[2], dzc[3]);
                    } else if (p.reduce_o) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) dmo[ps][r] += y[v] * dr[v];
                    }
                }
                if (p.has_z) {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (ok[v]) sDz[(tb + v) * (PT + 8) + pc] = f2bf(dzc[v]);
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
    if (p.has_z) {
        // dz of the segment's last chunk
        bar();
        const int cl_last = min(p.C, p.S - (c_end - 1) * p.C);
        flush_dz<NTHR, PT>(p, sDz, b, h, (c_end - 1) * p.C, cl_last);
    }

    // ---- per-segment partial sums of dmimo_o / dmimo_z: reduce over the 4 lane groups
    if (need_y) {
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
    kfn main[9], main_ex_noy[9], main_ex_rz[9];
};

#define MIMO_NP_LIST(F, RP, CT)                                                                             \
    F(RP, CT, 32, 32), F(RP, CT, 32, 64), F(RP, CT, 32, 128), F(RP, CT, 64, 32), F(RP, CT, 64, 64),         \
        F(RP, CT, 64, 128), F(RP, CT, 128, 32), F(RP, CT, 128, 64), F(RP, CT, 128, 128)
#define MIMO_AGG_FN(RP, CT, NT, PT) k_agg<RP, CT, NT, PT, false>
#define MIMO_AGG_EX_FN(RP, CT, NT, PT) k_agg<RP, CT, NT, PT, true>
#define MIMO_MAIN_FN(RP, CT, NT, PT) k_main<RP, CT, NT, PT, false, -1>
#define MIMO_MAIN_EX0_FN(RP, CT, NT, PT) k_main<RP, CT, NT, PT, true, 0>
#define MIMO_MAIN_EX1_FN(RP, CT, NT, PT) k_main<RP, CT, NT, PT, true, 1>
#define MIMO_FAMILY(RP, CT)                                                                               \
    const Family* family_rp##RP##_ct##CT() {                                                              \
        static const Family f = {{MIMO_NP_LIST(MIMO_AGG_FN, RP, CT)},     {MIMO_NP_LIST(MIMO_AGG_EX_FN, RP, CT)}, \
                                 {MIMO_NP_LIST(MIMO_MAIN_FN, RP, CT)},    {MIMO_NP_LIST(MIMO_MAIN_EX0_FN, RP, CT)}, \
                                 {MIMO_NP_LIST(MIMO_MAIN_EX1_FN, RP, CT)}};                               \
        return &f;                                                                                        \
    }
#define MIMO_DECL_FAMILY(RP, CT) const Family* family_rp##RP##_ct##CT();
MIMO_DECL_FAMILY(1, 1) MIMO_DECL_FAMILY(1, 2) MIMO_DECL_FAMILY(1, 4)
MIMO_DECL_FAMILY(2, 1) MIMO_DECL_FAMILY(2, 2) MIMO_DECL_FAMILY(2, 4)
MIMO_DECL_FAMILY(4, 1) MIMO_DECL_FAMILY(4, 2) MIMO_DECL_FAMILY(8, 1)

}  // namespace mimo
