// MI355X (gfx950) implementation of the first stage of the Mamba-3 MIMO
// combined backward ("mamba_mimo_bwd_fwd"), behind the C ABI declared in
// include/mimo_bwd_fwd.h.
//
// What is computed follows the Triton-Ascend mamba_mimo_bwd_fwd pull request
// page: its operator document (inputs/outputs, constraints, bf16 rounding
// boundaries) and its BF16-boundary PyTorch reference (bias and qk_dot,
// rotation, PsiV, trapezoidal discretisation, the chunk loop, the gating
// branches). The kernel split below is this library's own.
//
// Work decomposition. Chunks of one (batch, head) form a serial fp32 state
// recurrence S_{c+1} = S_c * exp(da_cs[last(c)]) + kappa_c^T Psi_c, which is
// elementwise-linear in the [N,P] state. The chunks are grouped into
// segments of L consecutive chunks, and each segment but the last into F
// sub-segments of L/F chunks:
//   k_agg   (sub-segment-parallel) the state each sub-segment adds from a zero
//                               start, and its decay product;
//   k_scan  ((n,p)-parallel)    the state entering every segment;
//   k_main  (segment-parallel)  walks its L chunks from the entry state: bf16
//                               entry states, qk_dot, the chunk-local causal
//                               block, y, and the gating gradients, with
//                               per-segment partial sums of dmimo_o/dmimo_z;
//   k_finish                    sums the partials over segments in order.
// With one segment only k_main runs. The bf16 rounding of the carried state
// (states[c] = bf16(S_c)) is applied to the fp32 state, so splitting the
// recurrence this way changes nothing but fp32 summation order.
//
// Chunk tile. Rows of a chunk are rank-major: row i = r*Cp + t for rank r and
// token t of the chunk, Cp = C rounded up to 16, so a 16-row MFMA tile holds
// 16 tokens of one rank, and the lane that holds token t of rank r in one
// tile holds token t of every rank in the rank's other tiles. That keeps the
// rank-ordered diagonal and dz chains, and the per-rank projection-gradient
// sums, inside one lane. The strictly causal mask works on token index.
// Padded rows and columns are zero in every operand.
//
// MFMA: v_mfma_f32_16x16x32_bf16, fp32 accumulate. Operand fragments are
// read from LDS as 8 consecutive bf16 along the contraction index, so each
// operand is stored contraction-contiguous:
//   A^T = K~ Q^T       sK [i][n], sQ [i][n]      (contract over n)
//   inter = Q bf16(S)  sQ [i][n], sSbT [p][n]
//   intra = A Psi      sA [i][j], sPsiT [p][j]  (contract over j)
//   S' = kappa^T Psi   sKapT [n][i], sPsiT [p][i]
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <string>

#define MIMO_B2_COMMON_KERNELS
#include "mimo_bwd2.hpp"
#include "mimo_f32.hpp"

namespace mimo {

// ---------------------------------------------------------------- segment scan
// Over the sub-segments j of one (batch, head): E_{j+1} = E_j * decay_j + U_j with
// E_0 = 0, written in place to agg[j] where the chunk kernel reads it, i.e. at the
// end of each segment ((j + 1) % F == 0). One thread per state element (the
// chain is latency-bound, so more waves keep more loads in flight); loads run
// up to 64 sub-segments ahead of the serial chain, so that the usual segment
// counts need a single round trip to memory.
// Short scans (up to SCAN_SPANS * SCAN_SPAN sub-segments): wave w of a block walks
// sub-segments [16w, 16w + 16) of 64 consecutive state elements. Each wave first
// folds its span from zero (its increment L and decay product D), the spans'
// carries are chained through LDS, and each wave then walks its span again from
// its carry, writing E at segment ends. All loads of a span are in flight at once.
constexpr int SCAN_SPAN = 16, SCAN_SPANS = 16;
__global__ __launch_bounds__(64 * SCAN_SPANS) void k_scan(Params p) {
    __shared__ float sL[SCAN_SPANS][64], sD[SCAN_SPANS][64];
    const int bh = blockIdx.y;
    const int NP = p.N * p.P;
    const int lane = threadIdx.x & 63, sp = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + lane;
    const bool ok = e < NP;
    const int ns = p.nsub, j0 = sp * SCAN_SPAN, n = min(SCAN_SPAN, ns - j0);
    float* base = p.agg + (long)bh * ns * NP + (ok ? e : 0);
    const float* dec = p.decay + (long)bh * ns + j0;
    float U[SCAN_SPAN], D[SCAN_SPAN];
#pragma unroll
    for (int j = 0; j < SCAN_SPAN; ++j) {
        U[j] = (j < n && ok) ? base[(long)(j0 + j) * NP] : 0.f;
        D[j] = (j < n) ? dec[j] : 1.f;
    }
    float L = 0.f, Dp = 1.f;
#pragma unroll
    for (int j = 0; j < SCAN_SPAN; ++j) {
        L = __fmaf_rn(L, D[j], U[j]);
        Dp *= D[j];
    }
    sL[sp][lane] = L;
    sD[sp][lane] = Dp;
    __syncthreads();
    float E = 0.f;
    for (int s = 0; s < sp; ++s) E = __fmaf_rn(E, sD[s][lane], sL[s][lane]);
#pragma unroll
    for (int j = 0; j < SCAN_SPAN; ++j) {
        E = __fmaf_rn(E, D[j], U[j]);
        if (ok && j < n && (j0 + j + 1) % p.F == 0) base[(long)(j0 + j) * NP] = E;
    }
}

// Longer scans: one thread per state element, E_{j+1} = E_j * D_j + U_j in
// order, loads running 64 sub-segments ahead.
__global__ __launch_bounds__(256) void k_scan_long(Params p) {
    const int bh = blockIdx.y;
    const int NP = p.N * p.P;
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= NP) return;
    const int ns = p.nsub;
    float* base = p.agg + (long)bh * ns * NP + e;
    const float* dec = p.decay + (long)bh * ns;
    float E = 0.f;
    constexpr int AHEAD = 64;
    for (int s0 = 0; s0 < ns; s0 += AHEAD) {
        float U[AHEAD], D[AHEAD];
#pragma unroll
        for (int j = 0; j < AHEAD; ++j) {
            if (s0 + j < ns) {
                U[j] = base[(long)(s0 + j) * NP];
                D[j] = dec[s0 + j];
            }
        }
#pragma unroll
        for (int j = 0; j < AHEAD; ++j) {
            if (s0 + j < ns) {
                E = __fmaf_rn(E, D[j], U[j]);
                if ((s0 + j + 1) % p.F == 0) base[(long)(s0 + j) * NP] = E;
            }
        }
    }
}

// dmimo = sum over segments of the partials, in segment order. Threads
// [0, tot) sum dmimo_o and threads [tot, 2 tot) dmimo_z when both are present,
// so that neither sum waits for the other's loads.
__global__ __launch_bounds__(256) void k_finish(Params p) {
    const long RP = (long)p.R * p.P, tot = (long)p.B * p.H * RP;
    long e = (long)blockIdx.x * 256 + threadIdx.x;
    bool z = !p.reduce_o;
    if (p.reduce_o && p.has_z && e >= tot) {
        e -= tot;
        z = true;
    }
    if (e >= tot) return;
    const long bh = e / RP, rp = e - bh * RP;
    const float* part = (z ? p.part_z : p.part_o) + bh * p.nseg * RP + rp;
    constexpr int AHEAD = 32;
    float s = 0.f;
    for (int s0 = 0; s0 < p.nseg; s0 += AHEAD) {
        float v[AHEAD];
#pragma unroll
        for (int j = 0; j < AHEAD; ++j) v[j] = (s0 + j < p.nseg) ? part[(long)(s0 + j) * RP] : 0.f;
#pragma unroll
        for (int j = 0; j < AHEAD; ++j)
            if (s0 + j < p.nseg) s += v[j];
    }
    (z ? p.dmimo_z : p.dmimo_o)[e] = s;
}

}  // namespace mimo

namespace {

using namespace mimo;

// ---------------------------------------------------------------- host side
thread_local std::string g_err;

mimo_status fail(mimo_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

// The kernels move q, k, v, z and dout rows and the bf16 outputs in 16-byte
// pieces: every such pointer must be 16-byte aligned (rows of N or P bf16 are a
// multiple of 16 bytes, so the base alignment carries over to every row).
mimo_status check_align16(std::initializer_list<const void*> ptrs, const char* names) {
    for (const void* x : ptrs)
        if (reinterpret_cast<uintptr_t>(x) % 16) return fail(MIMO_ERR_VALUE, "%s must be 16-byte aligned", names);
    return MIMO_OK;
}

struct Plan {
    int RP, CT, MT, NW, NT, PT, Cp, W, nc, L, nseg, F, nsub;
    bool ex;   // the shape-exact kernel instances apply
    size_t off_agg, off_decay, off_po, off_pz, ws_bytes;
    int lds_agg, lds_main, lds_states;   // lds_states: the no-y chunk pass (k_agg in ST mode)
};

int round_up(int x, int m) { return (x + m - 1) / m * m; }
int tile_size(int x) { return x <= 32 ? 32 : (x <= 64 ? 64 : 128); }
int next_pow2(int x) {
    int y = 1;
    while (y < x) y *= 2;
    return y;
}
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int tidx(int x) { return x == 32 ? 0 : (x == 64 ? 1 : 2); }

// MIMO_FORCE_GENERIC=1 in the environment disables the shape-exact kernel
// instances (used by the tests to compare both paths on the same inputs).
bool force_generic() {
    const char* e = getenv("MIMO_FORCE_GENERIC");
    return e != nullptr && e[0] == '1';
}

const Family* family(int RP, int CT) {
    switch (RP * 10 + CT) {
        case 11: return family_rp1_ct1();
        case 12: return family_rp1_ct2();
        case 14: return family_rp1_ct4();
        case 21: return family_rp2_ct1();
        case 22: return family_rp2_ct2();
        case 24: return family_rp2_ct4();
        case 41: return family_rp4_ct1();
        case 42: return family_rp4_ct2();
        case 81: return family_rp8_ct1();
        default: return nullptr;
    }
}

// fwd: the layer output (mimo_fwd), which needs no partial dmimo sums.
mimo_status make_plan(const mimo_bwd_fwd_args* a, Plan* pl, bool fwd = false) {
    if (a == nullptr) return fail(MIMO_ERR_VALUE, "args must not be NULL");
    const int64_t B = a->B, S = a->S, H = a->H, G = a->G, R = a->R, N = a->N, P = a->P;
    const int64_t C = a->chunk_size, rd = a->rotary_dim_divisor;
    if (B < 1 || S < 1 || R < 1 || G < 1) return fail(MIMO_ERR_VALUE, "B, S, R and G must be positive");
    if (H < 1 || N < 1 || P < 1) return fail(MIMO_ERR_VALUE, "H, N and P must be positive");
    if (C < 1 || C * R > 128) return fail(MIMO_ERR_VALUE, "chunk_size * R must be in [1, 128]");
    if (rd != 2 && rd != 4) return fail(MIMO_ERR_VALUE, "rotary_dim_divisor must be 2 or 4");
    if (N % rd || N % 2) return fail(MIMO_ERR_VALUE, "N must be even and divisible by rotary_dim_divisor");
    if (N > 128) return fail(MIMO_ERR_VALUE, "N greater than 128 is not supported");
    if (H % G) return fail(MIMO_ERR_VALUE, "H must be divisible by G");
    if (P > 128) return fail(MIMO_ERR_VALUE, "P greater than 128 is not supported");
    if ((a->z == nullptr) != (a->mimo_z == nullptr))
        return fail(MIMO_ERR_VALUE, "z and mimo_z must either both be present or both be NULL");
    if (N % 16) return fail(MIMO_ERR_UNSUPPORTED, "N must be a multiple of 16 (got %lld)", (long long)N);
    if (P % 16) return fail(MIMO_ERR_UNSUPPORTED, "P must be a multiple of 16 (got %lld)", (long long)P);
    if (C > 64) return fail(MIMO_ERR_UNSUPPORTED, "chunk_size above 64 is not supported");
    if (R > 8) return fail(MIMO_ERR_UNSUPPORTED, "R above 8 is not supported (got %lld)", (long long)R);
    // rows of a chunk tile: ranks padded to a power of two, tokens to 16, 32 or 64
    const int CT = next_pow2((int)((C + 15) / 16));
    const int RP = next_pow2((int)R);
    if (RP * CT > 8)
        return fail(MIMO_ERR_UNSUPPORTED,
                    "R=%lld with chunk_size=%lld needs %d tile rows (limit 128)", (long long)R, (long long)C,
                    16 * RP * CT);
    if (B * H * ((S + C - 1) / C + 8) > (int64_t)1 << 31)
        return fail(MIMO_ERR_UNSUPPORTED, "B * H * nchunks is too large");
    if (S > (int64_t)1 << 30) return fail(MIMO_ERR_UNSUPPORTED, "S above 2^30 is not supported");
    pl->RP = RP;
    pl->CT = CT;
    pl->Cp = 16 * CT;
    pl->W = (int)(N / rd);
    pl->NT = tile_size((int)N);
    pl->PT = tile_size((int)P);
    // must match Tile<RP, CT, NT, PT> in mimo_kernels.hpp
    pl->MT = 16 * RP * CT < 32 ? 32 : 16 * RP * CT;
    pl->NW = (pl->MT == 128 && pl->PT >= 64) ? 8 : 4;
    pl->nc = (int)((S + C - 1) / C);
    // segments: about two workgroups per compute unit, so that every
    // workgroup of the chunk kernel is resident at once. A call that needs no y
    // (states and qk_dot only) runs the aggregate's state walk as its chunk pass,
    // whose time is the chain of chunk steps of one workgroup: it takes twice as many
    // shorter segments (about four workgroups per compute unit for four-wave tiles).
    pl->ex = !force_generic() && R == RP && N == pl->NT && P == pl->PT && C == pl->Cp && rd == 4;
    const bool states_only = !fwd && a->mimo_o == nullptr && a->z == nullptr;
    const int64_t target = states_only && pl->NW == 4 ? 1024 : 512;
    int64_t L = (pl->nc * B * H + target - 1) / target;
    if (L < 1) L = 1;
    if (L > pl->nc) L = pl->nc;
    pl->L = (int)L;
    pl->nseg = (int)((pl->nc + L - 1) / L);
    if (pl->nseg > 65535) return fail(MIMO_ERR_UNSUPPORTED, "too many segments");
    // The aggregate kernel splits each segment but the last into F sub-segments of
    // ceil(L / F) chunks (the last piece shorter): its chain per workgroup shortens
    // with F while the workgroups still fit the GPU at once (about four per compute
    // unit for four-wave tiles, two for eight-wave ones); beyond that more pieces
    // only add scan traffic (the scan reads every sub-segment's [N,P] increment).
    {
        const int64_t slots = pl->NW == 8 ? 512 : 1024;
        const int64_t units = (int64_t)(pl->nseg - 1) * B * H;
        int64_t F = units > 0 ? slots / units : 1;
        if (F > (L + 3) / 4) F = (L + 3) / 4;   // pieces of at least four chunks
        if (F < 1) F = 1;
        while (F > 1 && (F - 1) * ((L + F - 1) / F) >= L) --F;   // every piece non-empty
        pl->F = (int)F;
    }
    pl->nsub = (pl->nseg - 1) * pl->F;
    const bool reduce_o = a->mimo_o != nullptr, has_z = a->z != nullptr;
    size_t off = 0;
    pl->off_agg = off;
    if (pl->nseg > 1) off = align256(off + (size_t)B * H * pl->nsub * N * P * 4);
    pl->off_decay = off;
    if (pl->nseg > 1) off = align256(off + (size_t)B * H * pl->nsub * 4);
    pl->off_po = off;
    if (pl->nseg > 1 && reduce_o && !fwd) off = align256(off + (size_t)B * H * pl->nseg * R * P * 4);
    pl->off_pz = off;
    if (pl->nseg > 1 && has_z && !fwd) off = align256(off + (size_t)B * H * pl->nseg * R * P * 4);
    pl->ws_bytes = off;
    Lds lm = lds_layout(RP, CT, pl->NT, pl->PT, (int)C, pl->W, true);
    Lds la = lds_layout(RP, CT, pl->NT, pl->PT, (int)C, pl->W, false);
    pl->lds_main = lm.total;
    pl->lds_agg = la.total;
    pl->lds_states = la.total;
    // the token-tile reduction of the dmimo partials reuses LDS from offset 0
    if (CT > 1) {
        const int red = 2 * CT * RP * pl->PT * 4;
        if (red > pl->lds_main) pl->lds_main = red;
    }
    if (pl->lds_main > 160 * 1024)
        return fail(MIMO_ERR_UNSUPPORTED, "shape needs %d bytes of LDS per workgroup (limit 163840)", pl->lds_main);
    return MIMO_OK;
}

std::mutex g_mu;
int g_arch_ok[64];  // 0 unknown, 1 gfx950, 2 other

mimo_status check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(MIMO_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= 64) return fail(MIMO_ERR_UNSUPPORTED, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_arch_ok[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(MIMO_ERR_HIP, "hipGetDeviceProperties failed");
        g_arch_ok[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    }
    if (g_arch_ok[dev] != 1) return fail(MIMO_ERR_UNSUPPORTED, "mamba_mimo_bwd_fwd requires a gfx950 (MI355X) device");
    return MIMO_OK;
}

mimo_status set_lds(kfn f, int bytes) {
    if (bytes <= 64 * 1024) return MIMO_OK;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(f), hipFuncAttributeMaxDynamicSharedMemorySize, bytes) !=
        hipSuccess)
        return fail(MIMO_ERR_HIP, "hipFuncSetAttribute(MaxDynamicSharedMemorySize=%d) failed", bytes);
    return MIMO_OK;
}

// qk_dot of the calls that need no y (their chunk pass is k_agg's state walk):
// qk_dot[b,h,t,r,r2] = bf16(q0[t,r] . k0[t,r2]), q0 = bf16(q + bf16(q_bias)) and k0
// likewise (biased, unrotated). One workgroup per (batch, q/k group, 16 tokens): in one
// round of loads it stages the group's raw q and k rows of the 16 tokens ([2][16] token
// rows of RP*NT bf16 plus 16 of padding, RP being R rounded up to a power of two; read
// once for all the group's heads; the padding puts the 16 tokens of a fragment read on
// distinct LDS banks) and the rounded biases of up to eight of the group's heads
// ([8][2][RP][NT], bf16 values held as fp32 so that the bias add needs no unpacking;
// zero past R, N and the sequence); wave w then serves heads w, w + 4, ... of the
// batch, and further batches of heads restage the biases. A head's dots come from
// 16 x 16 MFMA tiles whose rows and columns are (token, rank) pairs, with the chunk
// pass's fragments and K steps (each product is exact), so both give the same bits;
// each lane on a tile's block diagonal stores its part of one row of its token's dots.
template <int NT, int RP>   // RP: the rank count rounded up to a power of two (tile shape, LDS layout)
__global__ __launch_bounds__(256) void k_qk(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    // every row and bias table is laid out for RP ranks (padded ranks stay zero), so
    // that the staging index arithmetic is shifts and masks only
    constexpr int NT8 = NT / 8, TS = RP * NT + 16;   // token row pitch (bf16)
    constexpr unsigned LN8 = NT8 == 4 ? 2 : (NT8 == 8 ? 3 : 4), LR = RP == 1 ? 0 : (RP == 2 ? 1 : (RP == 4 ? 2 : 3));
    static_assert((1 << LN8) == NT8 && (1 << LR) == RP, "power-of-two tile sizes");
    unsigned short* sx = reinterpret_cast<unsigned short*>(smem);   // [2][16][TS]: q, then k
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, q4 = lane >> 4;
    const int ntt = (p.S + 15) / 16;
    const int unit = blockIdx.x;   // (b * G + g) * ntt + tile
    const int bg = unit / ntt, tile = unit - bg * ntt;
    const int b = bg / p.G, g = bg - b * p.G, hpg = p.H / p.G;
    const int R = p.R, N = p.N, t0 = 16 * tile;
    constexpr int KS = NT / 32;
    float* sb = reinterpret_cast<float*>(sx + 2 * 16 * TS);   // [8][2][RP][NT] rounded biases of a batch of heads
    for (int h0 = 0; h0 < hpg; h0 += 8) {
        const int nh = min(8, hpg - h0);
        const unsigned rows = h0 == 0 ? 2u * 16u * RP * NT8 : 0u, bias = (unsigned)nh * 2u * RP * NT8;
        if (h0 > 0) __syncthreads();   // every wave is done with the previous batch's biases
        for (unsigned e = tid; e < rows + bias; e += 256) {
            if (e < rows) {
                // e = ((which * 16 + tk) * RP + r) * NT8 + c8
                u32x4 w = {0u, 0u, 0u, 0u};
                const unsigned c8 = e & (NT8 - 1), rest = e >> LN8;
                const unsigned r = rest & (RP - 1), row = rest >> LR;
                const int t = t0 + (int)(row & 15u), col = 8 * (int)c8;
                if ((int)r < R && t < p.S && col < N) {
                    const unsigned short* x = (row >> 4) ? p.k : p.q;
                    w = *reinterpret_cast<const u32x4*>(x + ((((long)b * p.S + t) * R + r) * p.G + g) * N + col);
                }
                *reinterpret_cast<u32x4*>(sx + row * TS + r * NT + col) = w;
            } else {
                // e - rows = ((hh * 2 + which) * RP + r) * NT8 + c8
                f32x4 w0 = {0.f, 0.f, 0.f, 0.f}, w1 = w0;
                const unsigned e2 = e - rows, c8 = e2 & (NT8 - 1), rest = e2 >> LN8;
                const unsigned r = rest & (RP - 1), hw = rest >> LR;   // hw = hh * 2 + which
                const int col = 8 * (int)c8;
                if ((int)r < R && col < N) {
                    const float* bp = ((hw & 1u) ? p.k_bias : p.q_bias) + ((long)(g * hpg + h0 + (int)(hw >> 1)) * R + r) * N + col;
                    const f32x4 b0 = *reinterpret_cast<const f32x4*>(bp), b1 = *reinterpret_cast<const f32x4*>(bp + 4);
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        w0[d] = rnd(b0[d]);
                        w1[d] = rnd(b1[d]);
                    }
                }
                float* dst = sb + rest * NT + col;
                *reinterpret_cast<f32x4*>(dst) = w0;
                *reinterpret_cast<f32x4*>(dst + 4) = w1;
            }
        }
        __syncthreads();
        for (int hh = wave; hh < nh; hh += 4) {
            const int h = g * hpg + h0 + hh;
            // Tiles of TPT = 16 / RP tokens: rows and columns are the 16 (token, rank)
            // pairs of tokens u TPT .. u TPT + TPT - 1, row l16 = (token u TPT + l16 / RP,
            // rank l16 % RP). Lane (l16, q4) supplies that row of K0 (A operand) and of Q0
            // (B operand), columns 32 ks + 8 q4 .. + 7; it then holds
            // dot(k0[row 4 q4 + i], q0[row l16]) for i = 0..3, and those whose two rows
            // share a token are row r = l16 % RP of that token's dots, columns
            // (4 q4 + i) % RP (each product is exact, so the operand order does not
            // change the sums). A row past R or past the sequence only reaches dots that
            // are not stored (staged rows and biases past R are zero). The lane's offsets
            // pass through an empty asm statement, so that the raw-row reads, which do
            // not depend on the head, are redone per head instead of being held in
            // registers across the head loop.
            constexpr int TPT = 16 / RP;
            int rl = l16 % RP, tq = l16 / RP;
            asm volatile("" : "+v"(rl), "+v"(tq));
#pragma unroll
            for (int u = 0; u < RP; ++u) {
                const int tl = u * TPT + tq;
                f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int col = 32 * ks + 8 * q4;
                    u32x4 fr[2];
#pragma unroll
                    for (int which = 0; which < 2; ++which) {
                        const u32x4 raw = *reinterpret_cast<const u32x4*>(sx + (which * 16 + tl) * TS + rl * NT + col);
                        const float* bp = sb + ((hh * 2 + which) * RP + rl) * NT + col;
                        const f32x4 b0 = *reinterpret_cast<const f32x4*>(bp), b1 = *reinterpret_cast<const f32x4*>(bp + 4);
                        fr[which] = u32x4{pk2(lo16(raw[0]) + b0[0], hi16(raw[0]) + b0[1]),
                                          pk2(lo16(raw[1]) + b0[2], hi16(raw[1]) + b0[3]),
                                          pk2(lo16(raw[2]) + b1[0], hi16(raw[2]) + b1[1]),
                                          pk2(lo16(raw[3]) + b1[2], hi16(raw[3]) + b1[3])};
                    }
                    a4 = mfma(fr[1], fr[0], a4);
                }
                const int tt = t0 + tl;
                if (rl >= R || tt >= p.S) continue;
                unsigned short* out = p.qk_dot + (((long)(b * p.H + h) * p.S + tt) * R + rl) * R;
                if constexpr (RP >= 4) {
                    // four values, columns r20 .. r20 + 3
                    if ((4 * q4) / RP != tq) continue;
                    const int r20 = (4 * q4) % RP;
                    if (R == RP) {
                        *reinterpret_cast<u32x2*>(out + r20) = u32x2{pk2(a4[0], a4[1]), pk2(a4[2], a4[3])};
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (r20 + i < R) out[r20 + i] = bits16(rnd(a4[i]));
                    }
                } else if constexpr (RP == 2) {
                    // two values, columns 0 and 1
                    if (q4 != (l16 >> 2)) continue;
                    const bool hi = (l16 >> 1) & 1;
                    *reinterpret_cast<unsigned*>(out) = pk2(hi ? a4[2] : a4[0], hi ? a4[3] : a4[1]);
                } else {
                    // one value
                    if (q4 != (l16 >> 2)) continue;
                    const int v = l16 & 3;
                    const float x01 = (v & 1) ? a4[1] : a4[0], x23 = (v & 1) ? a4[3] : a4[2];
                    out[0] = bits16(rnd((v & 2) ? x23 : x01));
                }
            }
        }
    }
}

// LDS of k_qk: the staged rows (bf16, padded) and one batch of biases (fp32), both
// for the rank count rounded up to a power of two: at most 129 KB.
int qk_lds_bytes(const Params& p, int NT) {
    const int RP = p.R <= 1 ? 1 : (p.R <= 2 ? 2 : (p.R <= 4 ? 4 : 8));
    return 2 * 16 * (RP * NT + 16) * 2 + 2 * std::min(8, p.H / p.G) * RP * NT * 4;
}

mimo_status launch_qk(const Params& p, int NT, hipStream_t st) {
    const unsigned grid = (unsigned)((long)p.B * p.G * ((p.S + 15) / 16));
    const int lds = qk_lds_bytes(p, NT);
    Params pc = p;
    void* args[] = {&pc};
    // instances [NT 32, 64, 128][RP 1, 2, 4, 8]
    static const void* const table[3][4] = {
        {reinterpret_cast<const void*>(&k_qk<32, 1>), reinterpret_cast<const void*>(&k_qk<32, 2>),
         reinterpret_cast<const void*>(&k_qk<32, 4>), reinterpret_cast<const void*>(&k_qk<32, 8>)},
        {reinterpret_cast<const void*>(&k_qk<64, 1>), reinterpret_cast<const void*>(&k_qk<64, 2>),
         reinterpret_cast<const void*>(&k_qk<64, 4>), reinterpret_cast<const void*>(&k_qk<64, 8>)},
        {reinterpret_cast<const void*>(&k_qk<128, 1>), reinterpret_cast<const void*>(&k_qk<128, 2>),
         reinterpret_cast<const void*>(&k_qk<128, 4>), reinterpret_cast<const void*>(&k_qk<128, 8>)}};
    const int ri = p.R <= 1 ? 0 : (p.R <= 2 ? 1 : (p.R <= 4 ? 2 : 3));
    const void* f = table[NT == 32 ? 0 : (NT == 64 ? 1 : 2)][ri];
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
        return fail(MIMO_ERR_HIP, "hipFuncSetAttribute(MaxDynamicSharedMemorySize=%d) failed", lds);
    const hipError_t e = hipLaunchKernel(f, dim3(grid), dim3(256), args, (size_t)lds, st);
    if (e != hipSuccess) return fail(MIMO_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return MIMO_OK;
}

// 1-D grid of the chunk kernels (see map_block): 8 XCDs x H/G heads x units per XCD.
unsigned grid_blocks(const Params& p, int nseg_k) {
    const long units = (long)p.B * p.G * nseg_k;
    return (unsigned)(8L * (p.H / p.G) * ((units + 7) / 8));
}

mimo_status launch(kfn f, dim3 grid, dim3 block, int lds, hipStream_t st, Params& p) {
    void* args[] = {&p};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(f), grid, block, args, (size_t)lds, st);
    if (e != hipSuccess) return fail(MIMO_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return MIMO_OK;
}

// The state scan over sub-segments: the span kernel up to 256 of them, else the
// sequential one.
mimo_status launch_scan(Params& p, int bh, hipStream_t st) {
    const int NP = p.N * p.P;
    if (p.nsub <= SCAN_SPAN * SCAN_SPANS) {
        const int spans = (p.nsub + SCAN_SPAN - 1) / SCAN_SPAN;
        return launch(k_scan, dim3((NP + 63) / 64, bh), dim3(64 * spans), 0, st, p);
    }
    return launch(k_scan_long, dim3((NP + 255) / 256, bh), dim3(256), 0, st, p);
}

// The dmimo_o / dmimo_z sums: one thread per output element of each present gradient.
mimo_status launch_finish(Params& p, hipStream_t st) {
    const long tot = (long)p.B * p.H * p.R * p.P * ((p.reduce_o ? 1 : 0) + (p.has_z ? 1 : 0));
    if (tot == 0) return MIMO_OK;
    return launch(k_finish, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, p);
}

// The forward's arguments as those of the backward first stage (no dout, no
// backward outputs): both run the same plan and kernels.
mimo_bwd_fwd_args as_bwd_args(const mimo_fwd_args* f) {
    mimo_bwd_fwd_args a;
    memset(&a, 0, sizeof(a));
    a.B = f->B; a.S = f->S; a.H = f->H; a.G = f->G; a.R = f->R; a.N = f->N; a.P = f->P;
    a.chunk_size = f->chunk_size;
    a.rotary_dim_divisor = f->rotary_dim_divisor;
    a.q = f->q; a.k = f->k; a.v = f->v;
    a.q_bias = f->q_bias; a.k_bias = f->k_bias; a.mimo_v = f->mimo_v; a.mimo_o = f->mimo_o;
    a.z = f->z; a.mimo_z = f->mimo_z; a.angles = f->angles; a.da_cs = f->da_cs;
    a.da_cs_rev = f->da_cs_rev; a.dt = f->dt; a.trap = f->trap; a.d = f->d; a.segsum = f->segsum;
    a.workspace = f->workspace;
    a.workspace_bytes = f->workspace_bytes;
    return a;
}

// ---------------------------------------------------------------- fp32-intermediate path
// Problem of the fp32 kernels, in the MIMO operator's terms (the SISO forward maps
// onto it with R = 1, G = Hq, N = K, P = V and unit projections).
struct Prob32 {
    int64_t B, S, H, G, R, N, P;
    int C, W;
    bool reduce_o, has_z, has_d, fwd, f16;
    bool uv;   // unit projections and controls from adt (the SISO forward): the *_uv kernels
};

struct Plan32 {
    int MT, NT, PT, nc, L, nseg, F, nsub, ti, lds_main, lds_agg;
    bool kg_main, kg_agg;   // K~ tile in scratch (the kernel table picks those instances by the same rule)
    size_t off_agg, off_decay, off_po, off_pz, off_kslots, ws_bytes;
};

int tidx3(int x) { return x == 32 ? 0 : (x == 64 ? 1 : 2); }

const f32::F32Set* f32_set() {
    static const f32::F32Set set = [] {
        f32::F32Set s{};
        const f32::F32Part* parts[3] = {f32::f32_part_mt32(), f32::f32_part_mt64(), f32::f32_part_mt128()};
        for (int m = 0; m < 3; ++m)
            for (int d = 0; d < 2; ++d)
                for (int i = 0; i < 9; ++i) {
                    s.agg[d][9 * m + i] = parts[m]->agg[d][i];
                    s.main[d][9 * m + i] = parts[m]->main[d][i];
                    s.agg_uv[d][9 * m + i] = parts[m]->agg_uv[d][i];
                    s.main_uv[d][9 * m + i] = parts[m]->main_uv[d][i];
                }
        for (int d = 0; d < 2; ++d) {
            s.agg_ex[d] = parts[1]->agg_ex[d];
            s.main_ex[d] = parts[1]->main_ex[d];
            s.agg_sx[d] = parts[1]->agg_sx[d];
            s.main_sx[d] = parts[1]->main_sx[d];
        }
        return s;
    }();
    return &set;
}

mimo_status make_plan32(const Prob32& q, Plan32* pl) {
    if (q.B < 1 || q.S < 1 || q.R < 1 || q.G < 1 || q.H < 1 || q.N < 1 || q.P < 1)
        return fail(MIMO_ERR_VALUE, "B, S, H, G, R, N and P must be positive");
    if (q.C < 1) return fail(MIMO_ERR_VALUE, "chunk_size must be positive");
    if (q.H % q.G) return fail(MIMO_ERR_VALUE, "H must be divisible by the number of q/k heads");
    if (q.N % 2 || q.W < 0 || 2 * q.W > q.N) return fail(MIMO_ERR_VALUE, "the rotated width must be in [0, N/2]");
    if (q.N % 16 || q.N > 128) return fail(MIMO_ERR_UNSUPPORTED, "N must be a multiple of 16 up to 128 (got %lld)", (long long)q.N);
    if (q.P % 16 || q.P > 128) return fail(MIMO_ERR_UNSUPPORTED, "P must be a multiple of 16 up to 128 (got %lld)", (long long)q.P);
    if (q.C > 64) return fail(MIMO_ERR_UNSUPPORTED, "chunk_size above 64 is not supported");
    if (q.R > 8) return fail(MIMO_ERR_UNSUPPORTED, "R above 8 is not supported");
    const int Cp = (q.C + 15) / 16 * 16;
    const int rows = (int)q.R * Cp;
    if (rows > 128) return fail(MIMO_ERR_UNSUPPORTED, "R * chunk_size (rounded up to 16) above 128 is not supported");
    if (q.S > (int64_t)1 << 30 || q.B * q.H * ((q.S + q.C - 1) / q.C + 8) > (int64_t)1 << 31)
        return fail(MIMO_ERR_UNSUPPORTED, "problem too large");
    pl->MT = rows <= 32 ? 32 : (rows <= 64 ? 64 : 128);
    pl->NT = tile_size((int)q.N);
    pl->PT = tile_size((int)q.P);
    pl->ti = 9 * tidx3(pl->MT) + 3 * tidx3(pl->NT) + tidx3(pl->PT);
    pl->kg_main = f32::lds32(pl->MT, pl->NT, pl->PT, true, q.uv).total > 160 * 1024 && !q.uv;
    pl->kg_agg = f32::lds32(pl->MT, pl->NT, pl->PT, false, q.uv).total > 160 * 1024 && !q.uv;
    pl->lds_main = f32::lds32(pl->MT, pl->NT, pl->PT, true, q.uv, pl->kg_main).total;
    pl->lds_agg = f32::lds32(pl->MT, pl->NT, pl->PT, false, q.uv, pl->kg_agg).total;
    if (pl->lds_main > 160 * 1024 || pl->lds_agg > 160 * 1024)
        return fail(MIMO_ERR_UNSUPPORTED,
                    "the fp32-intermediate kernels need %d bytes of LDS for R*C=%d, N=%lld, P=%lld (limit 163840)",
                    pl->lds_main, rows, (long long)q.N, (long long)q.P);
    pl->nc = (int)((q.S + q.C - 1) / q.C);
    int64_t L = (pl->nc * q.B * q.H + 511) / 512;
    if (L < 1) L = 1;
    if (L > pl->nc) L = pl->nc;
    pl->L = (int)L;
    pl->nseg = (int)((pl->nc + L - 1) / L);
    if (pl->nseg > 65535) return fail(MIMO_ERR_UNSUPPORTED, "too many segments");
    // two sub-segments a segment only when segments are long (8 chunks or more): for
    // short ones the halved chain does not pay for twice the aggregate traffic
    pl->F = (L % 2 == 0 && L >= 8) ? 2 : 1;
    pl->nsub = (pl->nseg - 1) * pl->F;
    const bool part = !q.fwd && pl->nseg > 1;
    size_t off = 0;
    pl->off_agg = off;
    if (pl->nseg > 1) off = align256(off + (size_t)q.B * q.H * pl->nsub * q.N * q.P * 4);
    pl->off_decay = off;
    if (pl->nseg > 1) off = align256(off + (size_t)q.B * q.H * pl->nsub * 4);
    pl->off_po = off;
    if (part && q.reduce_o) off = align256(off + (size_t)q.B * q.H * pl->nseg * q.R * q.P * 4);
    pl->off_pz = off;
    if (part && q.has_z) off = align256(off + (size_t)q.B * q.H * pl->nseg * q.R * q.P * 4);
    pl->off_kslots = off;
    if (pl->kg_main || pl->kg_agg) {
        // one K~ tile per block of whichever launch keeps it in scratch (they run one after
        // the other and share the slots)
        Params pp = {};
        pp.B = (int)q.B; pp.H = (int)q.H; pp.G = (int)q.G;
        size_t blocks = pl->kg_main ? grid_blocks(pp, pl->nseg) : 0;
        if (pl->kg_agg && pl->nseg > 1 && grid_blocks(pp, pl->nsub) > blocks) blocks = grid_blocks(pp, pl->nsub);
        off = align256(off + blocks * pl->MT * (pl->NT + 4) * 4);
    }
    pl->ws_bytes = off;
    return MIMO_OK;
}

// Queue the fp32 kernels for a filled-in Params (pointers and flags set by the caller).
mimo_status run32(const Prob32& q, Params& p, void* workspace, size_t workspace_bytes, void* stream,
                  void* const* events) {
    Plan32 pl;
    mimo_status s = make_plan32(q, &pl);
    if (s != MIMO_OK) return s;
    if ((s = check_align16({p.dout, p.q, p.k, p.v, p.z, p.states, p.qk_dot, p.dz, p.o},
                           "dout, q, k, v, z, states, qk_dot, dz and o")) != MIMO_OK)
        return s;
    if (workspace_bytes < pl.ws_bytes || (pl.ws_bytes > 0 && workspace == nullptr))
        return fail(MIMO_ERR_VALUE, "workspace too small: need %zu bytes, got %zu", pl.ws_bytes, workspace_bytes);
    if (pl.ws_bytes > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255))
        return fail(MIMO_ERR_VALUE, "workspace must be 256-byte aligned");
    if (events != nullptr)
        for (int i = 0; i < MIMO_TIMED_EVENTS; ++i)
            if (events[i] == nullptr) return fail(MIMO_ERR_VALUE, "timing event %d is NULL", i);
    if ((s = check_device()) != MIMO_OK) return s;
    const f32::F32Set* set = f32_set();
    // shape-exact instances where the call's shape is theirs (a switch for tests can
    // force the generic ones)
    const bool ex = !force_generic() && !q.uv && pl.MT == 64 && pl.NT == 64 && pl.PT == 64 && q.R == 4 &&
                    q.C == 16 && q.N == 64 && q.P == 64 && q.W == 16 && !pl.kg_main && !pl.kg_agg;
    const bool sx = !force_generic() && q.uv && pl.MT == 64 && pl.NT == 128 && pl.PT == 64 && q.R == 1 &&
                    q.C == 64 && q.N == 128 && q.P == 64 && q.W == 64 && !pl.kg_main && !pl.kg_agg;
    const kfn kmain = ex   ? set->main_ex[q.f16]
                      : sx ? set->main_sx[q.f16]
                           : (q.uv ? set->main_uv : set->main)[q.f16][pl.ti];
    const kfn kagg = ex   ? set->agg_ex[q.f16]
                     : sx ? set->agg_sx[q.f16]
                          : (q.uv ? set->agg_uv : set->agg)[q.f16][pl.ti];
    if (kmain == nullptr || kagg == nullptr) return fail(MIMO_ERR_UNSUPPORTED, "no fp32 kernel for this tile shape");
    p.B = (int)q.B; p.S = (int)q.S; p.H = (int)q.H; p.G = (int)q.G; p.R = (int)q.R; p.N = (int)q.N; p.P = (int)q.P;
    p.C = q.C; p.W = q.W; p.nc = pl.nc; p.L = pl.L; p.nseg = pl.nseg; p.F = pl.F; p.nsub = pl.nsub;
    p.reduce_o = q.reduce_o; p.has_z = q.has_z; p.has_d = q.has_d; p.fwd = q.fwd;
    p.need_y = q.fwd || q.reduce_o || q.has_z;   // else the chunk pass emits states and qk_dot only
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    p.agg = pl.nseg > 1 ? reinterpret_cast<float*>(ws + pl.off_agg) : nullptr;
    p.decay = pl.nseg > 1 ? reinterpret_cast<float*>(ws + pl.off_decay) : nullptr;
    if (q.fwd) {
        p.part_o = p.part_z = nullptr;
    } else if (pl.nseg > 1) {
        p.part_o = q.reduce_o ? reinterpret_cast<float*>(ws + pl.off_po) : nullptr;
        p.part_z = q.has_z ? reinterpret_cast<float*>(ws + pl.off_pz) : nullptr;
    } else {
        p.part_o = p.dmimo_o;
        p.part_z = p.dmimo_z;
    }
    p.kslots = (pl.kg_main || pl.kg_agg) ? reinterpret_cast<float*>(ws + pl.off_kslots) : nullptr;
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto mark = [&](int i) -> mimo_status {
        if (events == nullptr) return MIMO_OK;
        if (hipEventRecord(static_cast<hipEvent_t>(events[i]), st) != hipSuccess)
            return fail(MIMO_ERR_HIP, "hipEventRecord failed");
        return MIMO_OK;
    };
    if ((s = set_lds(kmain, pl.lds_main)) != MIMO_OK) return s;
    if ((s = mark(0)) != MIMO_OK) return s;
    if (pl.nseg > 1) {
        if ((s = set_lds(kagg, pl.lds_agg)) != MIMO_OK) return s;
        if ((s = launch(kagg, dim3(grid_blocks(p, pl.nsub)), dim3(256), pl.lds_agg, st, p)) != MIMO_OK) return s;
        if ((s = mark(1)) != MIMO_OK) return s;
        if ((s = launch_scan(p, p.B * p.H, st)) != MIMO_OK) return s;
    } else if ((s = mark(1)) != MIMO_OK) {
        return s;
    }
    if ((s = mark(2)) != MIMO_OK) return s;
    if ((s = launch(kmain, dim3(grid_blocks(p, pl.nseg)), dim3(256), pl.lds_main, st, p)) != MIMO_OK) return s;
    if ((s = mark(3)) != MIMO_OK) return s;
    if (pl.nseg > 1 && !q.fwd && (q.reduce_o || q.has_z))
        if ((s = launch_finish(p, st)) != MIMO_OK) return s;
    if ((s = mark(4)) != MIMO_OK) return s;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MIMO_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return MIMO_OK;
}

// The MIMO operator's arguments as an fp32-path problem (bf16 inputs, fp32 controls).
mimo_status prob_from_mimo(const mimo_bwd_fwd_args* a, bool fwd, Prob32* q) {
    if (a == nullptr) return fail(MIMO_ERR_VALUE, "args must not be NULL");
    const int64_t rd = a->rotary_dim_divisor;
    if (rd != 2 && rd != 4) return fail(MIMO_ERR_VALUE, "rotary_dim_divisor must be 2 or 4");
    if (a->N < 1 || a->N % rd || a->N % 2) return fail(MIMO_ERR_VALUE, "N must be even and divisible by rotary_dim_divisor");
    if (a->chunk_size < 1 || (int64_t)a->chunk_size * a->R > 128) return fail(MIMO_ERR_VALUE, "chunk_size * R must be in [1, 128]");
    if ((a->z == nullptr) != (a->mimo_z == nullptr))
        return fail(MIMO_ERR_VALUE, "z and mimo_z must either both be present or both be NULL");
    *q = Prob32{a->B, a->S, a->H, a->G, a->R, a->N, a->P, a->chunk_size, (int)(a->N / rd),
                a->mimo_o != nullptr, a->z != nullptr, a->d != nullptr, fwd, false, false};
    return MIMO_OK;
}

Params params_from_mimo(const mimo_bwd_fwd_args* a) {
    Params p = {};
    p.dout = a->dout; p.q = a->q; p.k = a->k; p.v = a->v; p.z = a->z; p.trap = a->trap;
    p.q_bias = a->q_bias; p.k_bias = a->k_bias; p.mimo_v = a->mimo_v; p.mimo_o = a->mimo_o;
    p.mimo_z = a->mimo_z; p.angles = a->angles; p.da_cs = a->da_cs; p.da_cs_rev = a->da_cs_rev;
    p.dt = a->dt; p.d = a->d; p.segsum = a->segsum;
    p.dmimo_o = a->dmimo_o; p.dmimo_z = a->dmimo_z; p.states = a->states; p.dz = a->dz; p.qk_dot = a->qk_dot;
    return p;
}

mimo_status check_mimo_inputs(const mimo_bwd_fwd_args* a) {
    if (!a->q || !a->k || !a->v || !a->q_bias || !a->k_bias || !a->mimo_v || !a->angles || !a->da_cs ||
        !a->da_cs_rev || !a->dt || !a->trap || !a->segsum)
        return fail(MIMO_ERR_VALUE, "a required input pointer is NULL");
    return MIMO_OK;
}

mimo_status run_bwd32(const mimo_bwd_fwd_args* a, void* stream, void* const* events) {
    g_err.clear();
    Prob32 q;
    mimo_status s = prob_from_mimo(a, false, &q);
    if (s != MIMO_OK) return s;
    if ((s = check_mimo_inputs(a)) != MIMO_OK) return s;
    if (!a->dout && (q.reduce_o || q.has_z)) return fail(MIMO_ERR_VALUE, "dout must not be NULL");
    if (!a->states || !a->qk_dot) return fail(MIMO_ERR_VALUE, "states and qk_dot must not be NULL");
    if ((a->dmimo_o != nullptr) != q.reduce_o)
        return fail(MIMO_ERR_VALUE, "dmimo_o must be given exactly when mimo_o is given");
    if ((a->dz != nullptr) != q.has_z || (a->dmimo_z != nullptr) != q.has_z)
        return fail(MIMO_ERR_VALUE, "dz and dmimo_z must be given exactly when z is given");
    Params p = params_from_mimo(a);
    return run32(q, p, a->workspace, a->workspace_bytes, stream, events);
}

mimo_status run_fwd32(const mimo_fwd_args* f, void* stream, void* const* events) {
    g_err.clear();
    if (f == nullptr) return fail(MIMO_ERR_VALUE, "args must not be NULL");
    if (f->o == nullptr) return fail(MIMO_ERR_VALUE, "o must not be NULL");
    const mimo_bwd_fwd_args a = as_bwd_args(f);
    Prob32 q;
    mimo_status s = prob_from_mimo(&a, true, &q);
    if (s != MIMO_OK) return s;
    if ((s = check_mimo_inputs(&a)) != MIMO_OK) return s;
    Params p = params_from_mimo(&a);
    p.o = f->o;
    return run32(q, p, f->workspace, f->workspace_bytes, stream, events);
}

mimo_status prob_from_siso(const mimo_siso_fwd_args* a, Prob32* q) {
    if (a == nullptr) return fail(MIMO_ERR_VALUE, "args must not be NULL");
    if (a->chunk_size != 32 && a->chunk_size != 64) return fail(MIMO_ERR_VALUE, "chunk_size must be 32 or 64");
    if (a->Hq < 1 || a->H < 1 || a->H % a->Hq) return fail(MIMO_ERR_VALUE, "H must be divisible by Hq");
    if (a->A < 0 || a->A % 2 || 2 * a->A > a->K) return fail(MIMO_ERR_VALUE, "the angle width must be even and at most K/2");
    if (a->dtype != MIMO_DTYPE_BF16 && a->dtype != MIMO_DTYPE_FP16)
        return fail(MIMO_ERR_TYPE, "q, k, v and z must be bf16 or fp16");
    *q = Prob32{a->B, a->S, a->H, a->Hq, 1, a->K, a->V, a->chunk_size, (int)a->A,
                false, a->z != nullptr, a->d != nullptr, true, a->dtype == MIMO_DTYPE_FP16, true};
    return MIMO_OK;
}

mimo_status run_siso(const mimo_siso_fwd_args* a, void* stream, void* const* events) {
    g_err.clear();
    Prob32 q;
    mimo_status s = prob_from_siso(a, &q);
    if (s != MIMO_OK) return s;
    if (!a->q || !a->k || !a->v || !a->adt || !a->dt || !a->trap || !a->q_bias || !a->k_bias ||
        (!a->angles && a->A > 0))
        return fail(MIMO_ERR_VALUE, "a required input pointer is NULL");
    if (a->out == nullptr) return fail(MIMO_ERR_VALUE, "out must not be NULL");
    Params p = {};
    p.q = a->q; p.k = a->k; p.v = a->v; p.z = a->z;
    p.q_bias = a->q_bias; p.k_bias = a->k_bias; p.angles = a->angles; p.dt = a->dt; p.d = a->d;
    p.adt = a->adt; p.trapf = a->trap;
    p.o = a->out;
    return run32(q, p, a->workspace, a->workspace_bytes, stream, events);
}

// ---------------------------------------------------------------- stage-2 backward
struct PlanB2 {
    int nc, L, nseg, F, nsub, W, md;
    size_t off_agg, off_decay, off_mv, off_d, off_slots, ws_bytes;
};

mimo_status make_plan_b2(const mimo_bwd_bwd_args* a, PlanB2* pl) {
    if (a == nullptr) return fail(MIMO_ERR_VALUE, "args must not be NULL");
    const int64_t B = a->B, S = a->S, H = a->H, G = a->G, R = a->R, N = a->N, P = a->P, C = a->chunk_size;
    const int64_t rd = a->rotary_dim_divisor;
    if (B < 1 || S < 1 || H < 1 || G < 1 || R < 1 || N < 1 || P < 1)
        return fail(MIMO_ERR_VALUE, "B, S, H, G, R, N and P must be positive");
    if (C < 1) return fail(MIMO_ERR_VALUE, "chunk_size must be positive");
    if (H % G) return fail(MIMO_ERR_VALUE, "H must be divisible by G");
    if (rd != 2 && rd != 4) return fail(MIMO_ERR_VALUE, "rotary_dim_divisor must be 2 or 4");
    if (N % 2 || N % rd) return fail(MIMO_ERR_VALUE, "N must be even and divisible by rotary_dim_divisor");
    for (int32_t dt : {a->in_dtype, a->out_dtype})
        if (dt != MIMO_DTYPE_BF16 && dt != MIMO_DTYPE_FP16 && dt != MIMO_DTYPE_FP32)
            return fail(MIMO_ERR_VALUE, "in_dtype and out_dtype must be MIMO_DTYPE_BF16, _FP16 or _FP32");
    if (C * R > 128 || N > 128 || P > 128 || R > 8 || P % 8 || N % 8)
        return fail(MIMO_ERR_UNSUPPORTED,
                    "the stage-2 backward supports R * chunk_size, N and P up to 128, R up to 8 and N and P "
                    "multiples of 8");
    if (S > (int64_t)1 << 30 || B * H * ((S + C - 1) / C + 8) > (int64_t)1 << 31)
        return fail(MIMO_ERR_UNSUPPORTED, "problem too large");
    pl->md = (C * R <= 64 && N <= 64 && P <= 64) ? 64 : 128;
    pl->W = (int)(N / rd);
    pl->nc = (int)((S + C - 1) / C);
    // one workgroup per compute unit (the chunk pass keeps nine fp32 tiles in LDS, or
    // is bound by its registers with the tiles in scratch)
    int64_t L = (pl->nc * B * H + 255) / 256;
    if (L < 1) L = 1;
    if (L > pl->nc) L = pl->nc;
    pl->L = (int)L;
    pl->nseg = (int)((pl->nc + L - 1) / L);
    if (pl->nseg > 65535) return fail(MIMO_ERR_UNSUPPORTED, "too many segments");
    pl->F = (L % 2 == 0 && L >= 4) ? 2 : 1;
    pl->nsub = (pl->nseg - 1) * pl->F;
    size_t off = 0;
    pl->off_agg = off;
    if (pl->nseg > 1) off = align256(off + (size_t)B * H * pl->nsub * N * P * 4);
    pl->off_decay = off;
    if (pl->nseg > 1) off = align256(off + (size_t)B * H * pl->nsub * 4);
    pl->off_mv = off;
    off = align256(off + (size_t)B * H * pl->nseg * R * P * 4);
    pl->off_d = off;
    off = align256(off + (size_t)B * H * pl->nseg * 4);
    pl->off_slots = off;
    if (pl->md == 128) {
        // one tile slot per block of the chunk pass and of the aggregate (they run one
        // after the other and share the slots)
        Params pp = {};
        pp.B = (int)B; pp.H = (int)H; pp.G = (int)G;
        using G128 = b2::Geo<128>;
        const size_t main_f = (size_t)grid_blocks(pp, pl->nseg) * G128::MAIN_TILES;
        const size_t agg_f = pl->nseg > 1 ? (size_t)grid_blocks(pp, pl->nsub) * G128::AGG_TILES : 0;
        off = align256(off + 4 * (main_f > agg_f ? main_f : agg_f));
    }
    pl->ws_bytes = off;
    return MIMO_OK;
}

mimo_status run_b2(const mimo_bwd_bwd_args* a, void* stream, void* const* events) {
    g_err.clear();
    PlanB2 pl;
    mimo_status s = make_plan_b2(a, &pl);
    if (s != MIMO_OK) return s;
    if (!a->dout || !a->q || !a->k || !a->v || !a->q_bias || !a->k_bias || !a->mimo_v || !a->states ||
        !a->qk_dot || !a->da_cs || !a->da_cs_rev || !a->dt || !a->trap || !a->segsum || !a->angles)
        return fail(MIMO_ERR_VALUE, "a required input pointer is NULL");
    if (!a->dq || !a->dk || !a->dv || !a->dmimo_v || !a->dangles || !a->dfactor || !a->dgamma || !a->dda ||
        !a->dssda || !a->dda_cs_rev || !a->dda_cs)
        return fail(MIMO_ERR_VALUE, "an output pointer is NULL");
    if ((a->dd != nullptr) != (a->d != nullptr)) return fail(MIMO_ERR_VALUE, "dd must be given exactly when d is given");
    // rows of eight 16-bit or four fp32 values are moved as one 16-byte access
    for (const void* x : {(const void*)a->dout, (const void*)a->q, (const void*)a->k, (const void*)a->v,
                          (const void*)a->states, (const void*)a->q_bias, (const void*)a->k_bias,
                          (const void*)a->mimo_v, (const void*)a->mimo_o, (const void*)a->dq, (const void*)a->dk,
                          (const void*)a->dv})
        if (reinterpret_cast<uintptr_t>(x) % 16)
            return fail(MIMO_ERR_VALUE, "dout, q, k, v, states, q_bias, k_bias, mimo_v, mimo_o, dq, dk and dv "
                                        "must be 16-byte aligned");
    if (a->workspace_bytes < pl.ws_bytes || (pl.ws_bytes > 0 && a->workspace == nullptr))
        return fail(MIMO_ERR_VALUE, "workspace too small: need %zu bytes, got %zu", pl.ws_bytes, a->workspace_bytes);
    if (pl.ws_bytes > 0 && (reinterpret_cast<uintptr_t>(a->workspace) & 255))
        return fail(MIMO_ERR_VALUE, "workspace must be 256-byte aligned");
    if (events != nullptr)
        for (int i = 0; i < MIMO_TIMED_EVENTS; ++i)
            if (events[i] == nullptr) return fail(MIMO_ERR_VALUE, "timing event %d is NULL", i);
    if ((s = check_device()) != MIMO_OK) return s;
    b2::Params2 p = {};
    p.B = (int)a->B; p.S = (int)a->S; p.H = (int)a->H; p.G = (int)a->G; p.R = (int)a->R; p.N = (int)a->N;
    p.P = (int)a->P; p.C = a->chunk_size; p.W = pl.W; p.nc = pl.nc; p.L = pl.L; p.nseg = pl.nseg; p.F = pl.F;
    p.nsub = pl.nsub; p.reduce_o = a->mimo_o != nullptr; p.has_d = a->d != nullptr; p.out_dt = a->out_dtype;
    p.dout = a->dout; p.q = a->q; p.k = a->k; p.v = a->v; p.states = a->states; p.qk_dot = a->qk_dot;
    p.trap = a->trap; p.q_bias = a->q_bias; p.k_bias = a->k_bias; p.mimo_v = a->mimo_v; p.mimo_o = a->mimo_o;
    p.da_cs = a->da_cs; p.da_cs_rev = a->da_cs_rev; p.dt = a->dt; p.segsum = a->segsum; p.angles = a->angles;
    p.d = a->d;
    p.dq = a->dq; p.dk = a->dk; p.dv = a->dv; p.dmimo_v = a->dmimo_v; p.dangles = a->dangles;
    p.dfactor = a->dfactor; p.dgamma = a->dgamma; p.dda = a->dda; p.dssda = a->dssda;
    p.dda_cs_rev = a->dda_cs_rev; p.dda_cs = a->dda_cs; p.dd = a->dd;
    unsigned char* ws = static_cast<unsigned char*>(a->workspace);
    p.agg = pl.nseg > 1 ? reinterpret_cast<float*>(ws + pl.off_agg) : nullptr;
    p.decay = pl.nseg > 1 ? reinterpret_cast<float*>(ws + pl.off_decay) : nullptr;
    p.part_mv = reinterpret_cast<float*>(ws + pl.off_mv);
    p.part_d = reinterpret_cast<float*>(ws + pl.off_d);
    p.slots = pl.md == 128 ? reinterpret_cast<float*>(ws + pl.off_slots) : nullptr;

    hipStream_t st = static_cast<hipStream_t>(stream);
    auto mark = [&](int i) -> mimo_status {
        if (events == nullptr) return MIMO_OK;
        if (hipEventRecord(static_cast<hipEvent_t>(events[i]), st) != hipSuccess)
            return fail(MIMO_ERR_HIP, "hipEventRecord failed");
        return MIMO_OK;
    };
    auto launch2 = [&](const void* f, dim3 grid, int lds, int threads) -> mimo_status {
        void* args[] = {&p};
        const hipError_t e = hipLaunchKernel(f, grid, dim3(threads), args, (size_t)lds, st);
        if (e != hipSuccess) return fail(MIMO_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
        return MIMO_OK;
    };
    auto set_lds2 = [&](const void* f, int bytes) -> mimo_status {
        if (bytes <= 64 * 1024) return MIMO_OK;
        if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
            return fail(MIMO_ERR_HIP, "hipFuncSetAttribute(MaxDynamicSharedMemorySize=%d) failed", bytes);
        return MIMO_OK;
    };
    Params pp = {};
    pp.B = p.B; pp.H = p.H; pp.G = p.G;
    // shape-exact instances where the call's shape is theirs (see exact_shape); a switch
    // for tests can force the generic ones
    const bool ex2 = !force_generic() && pl.md == 64 && p.R == 4 && p.C == 16 && p.N == 64 && p.P == 64 && p.W == 16;
    const b2::Kern kern = a->in_dtype == MIMO_DTYPE_FP32   ? b2::kernels_f32(pl.md, ex2)
                          : a->in_dtype == MIMO_DTYPE_FP16 ? b2::kernels_f16(pl.md, ex2)
                                                           : b2::kernels_bf16(pl.md, ex2);
    const void* kmain = kern.main;
    const int lds_main = (pl.md == 64 ? b2::Geo<64>::LDS_MAIN : b2::Geo<128>::LDS_MAIN) * 4;
    const int lds_agg = (pl.md == 64 ? b2::Geo<64>::LDS_AGG : b2::Geo<128>::LDS_AGG) * 4;
    if ((s = set_lds2(kmain, lds_main)) != MIMO_OK) return s;
    if ((s = mark(0)) != MIMO_OK) return s;
    if (pl.nseg > 1) {
        const void* kagg = kern.agg;
        if ((s = set_lds2(kagg, lds_agg)) != MIMO_OK) return s;
        if ((s = launch2(kagg, dim3(grid_blocks(pp, pl.nsub)), lds_agg, b2::NTHR)) != MIMO_OK) return s;
        if ((s = mark(1)) != MIMO_OK) return s;
        const int NP = p.N * p.P;
        if ((s = launch2(reinterpret_cast<const void*>(&b2::k_scan_rev),
                         dim3((NP + b2::NTHR1 - 1) / b2::NTHR1, p.B * p.H), 0, b2::NTHR1)) != MIMO_OK)
            return s;
    } else if ((s = mark(1)) != MIMO_OK) {
        return s;
    }
    if ((s = mark(2)) != MIMO_OK) return s;
    if ((s = launch2(kmain, dim3(grid_blocks(pp, pl.nseg)), lds_main, b2::NTHR2)) != MIMO_OK) return s;
    if ((s = mark(3)) != MIMO_OK) return s;
    const long tot = (long)p.B * p.H * p.R * p.P;
    if ((s = launch2(reinterpret_cast<const void*>(&b2::k_finish2), dim3((unsigned)((tot + b2::NTHR1 - 1) / b2::NTHR1)),
                     0, b2::NTHR1)) != MIMO_OK)
        return s;
    if ((s = mark(4)) != MIMO_OK) return s;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MIMO_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return MIMO_OK;
}

// ---------------------------------------------------------------- fixed scratch
// The entry point that allocates nothing keeps the workspace (segment increments,
// decays, dmimo partials) in this array. Every device the library runs on holds its
// own copy until the process ends. In host code the array's name is only a
// stand-in: the device address comes from hipGetSymbolAddress, per device, with
// that device current, and only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[MIMO_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];   // device address of `scratch` on device i (nullptr: not looked up yet)

mimo_status scratch_on_current_device(void** ptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(MIMO_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= 64) return fail(MIMO_ERR_UNSUPPORTED, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(MIMO_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MIMO_OK;
}

}  // namespace

extern "C" {

int mimo_abi_version(void) { return MIMO_ABI_VERSION; }

const char* mimo_last_error(void) { return g_err.c_str(); }

mimo_status mimo_bwd_fwd_workspace_size(const mimo_bwd_fwd_args* args, size_t* bytes) {
    Plan pl;
    const mimo_status s = make_plan(args, &pl);
    if (s != MIMO_OK) return s;
    if (bytes == nullptr) return fail(MIMO_ERR_VALUE, "bytes must not be NULL");
    *bytes = pl.ws_bytes;
    return MIMO_OK;
}

// The backward first stage (out == nullptr) or the layer output o (out != nullptr,
// `a` built by as_bwd_args).
// A side stream and two events per (host thread, device), created on first use and kept
// for the life of the thread. A call whose chunk pass has an independent kernel (qk_dot
// of the calls without y) forks it onto the side stream after the caller's earlier work
// and joins it back before the chunk pass ends, so it can fill the CUs the chain leaves
// idle (the aggregate's tail, the scan, launch gaps). Default priority, like every stream
// here.
struct Side {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
thread_local Side g_side[64];

mimo_status side_stream(Side** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(MIMO_ERR_HIP, "hipGetDevice failed");
    Side& sd = g_side[dev];
    if (sd.s == nullptr) {
        hipStream_t st = nullptr;
        hipEvent_t f = nullptr, j = nullptr;
        if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess)
            return fail(MIMO_ERR_HIP, "hipStreamCreateWithFlags failed");
        if (hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess)
            return fail(MIMO_ERR_HIP, "hipEventCreateWithFlags failed");
        sd.s = st;
        sd.fork = f;
        sd.join = j;
    }
    *out = &sd;
    return MIMO_OK;
}

// fork: qk_dot of a no-y call on the side stream (false: in order on the call's stream,
// for the entry point that may create nothing)
static mimo_status run(const mimo_bwd_fwd_args* a, uint16_t* out, void* stream, void* const* events,
                       bool fork = true) {
    g_err.clear();
    const bool fwd = out != nullptr;
    Plan pl;
    mimo_status s = make_plan(a, &pl, fwd);
    if (s != MIMO_OK) return s;
    const bool reduce_o = a->mimo_o != nullptr, has_z = a->z != nullptr;
    if (!fwd && !a->dout && (reduce_o || has_z)) return fail(MIMO_ERR_VALUE, "dout must not be NULL");
    if (!a->q || !a->k || !a->v || !a->q_bias || !a->k_bias || !a->mimo_v || !a->angles || !a->da_cs ||
        !a->da_cs_rev || !a->dt || !a->trap || !a->segsum)
        return fail(MIMO_ERR_VALUE, "a required input pointer is NULL");
    if (!fwd) {
        if (!a->states || !a->qk_dot) return fail(MIMO_ERR_VALUE, "states and qk_dot must not be NULL");
        if ((a->dmimo_o != nullptr) != reduce_o)
            return fail(MIMO_ERR_VALUE, "dmimo_o must be given exactly when mimo_o is given");
        if ((a->dz != nullptr) != has_z || (a->dmimo_z != nullptr) != has_z)
            return fail(MIMO_ERR_VALUE, "dz and dmimo_z must be given exactly when z is given");
    }
    if ((s = check_align16({a->dout, a->q, a->k, a->v, a->z, a->states, a->qk_dot, a->dz, out},
                           "dout, q, k, v, z, states, qk_dot, dz and o")) != MIMO_OK)
        return s;
    if (a->workspace_bytes < pl.ws_bytes || (pl.ws_bytes > 0 && a->workspace == nullptr))
        return fail(MIMO_ERR_VALUE, "workspace too small: need %zu bytes, got %zu", pl.ws_bytes, a->workspace_bytes);
    if (pl.ws_bytes > 0 && (reinterpret_cast<uintptr_t>(a->workspace) & 255))
        return fail(MIMO_ERR_VALUE, "workspace must be 256-byte aligned");
    s = check_device();
    if (s != MIMO_OK) return s;

    Params p = {};
    p.B = (int)a->B; p.S = (int)a->S; p.H = (int)a->H; p.G = (int)a->G;
    p.R = (int)a->R; p.N = (int)a->N; p.P = (int)a->P; p.C = a->chunk_size;
    p.W = pl.W; p.nc = pl.nc; p.L = pl.L; p.nseg = pl.nseg; p.rd = a->rotary_dim_divisor;
    p.F = pl.F; p.nsub = pl.nsub;
    p.reduce_o = reduce_o; p.has_z = has_z; p.has_d = a->d != nullptr; p.need_y = fwd || reduce_o || has_z;
    p.fwd = fwd; p.o = out;
    p.dout = a->dout; p.q = a->q; p.k = a->k; p.v = a->v; p.z = a->z; p.trap = a->trap;
    p.q_bias = a->q_bias; p.k_bias = a->k_bias; p.mimo_v = a->mimo_v; p.mimo_o = a->mimo_o;
    p.mimo_z = a->mimo_z; p.angles = a->angles; p.da_cs = a->da_cs; p.da_cs_rev = a->da_cs_rev;
    p.dt = a->dt; p.d = a->d; p.segsum = a->segsum;
    p.dmimo_o = a->dmimo_o; p.dmimo_z = a->dmimo_z; p.states = a->states; p.dz = a->dz; p.qk_dot = a->qk_dot;
    unsigned char* ws = static_cast<unsigned char*>(a->workspace);
    p.agg = pl.nseg > 1 ? reinterpret_cast<float*>(ws + pl.off_agg) : nullptr;
    p.decay = pl.nseg > 1 ? reinterpret_cast<float*>(ws + pl.off_decay) : nullptr;
    if (fwd) {
        p.part_o = p.part_z = nullptr;
    } else if (pl.nseg > 1) {
        p.part_o = reduce_o ? reinterpret_cast<float*>(ws + pl.off_po) : nullptr;
        p.part_z = has_z ? reinterpret_cast<float*>(ws + pl.off_pz) : nullptr;
    } else {
        p.part_o = a->dmimo_o;
        p.part_z = a->dmimo_z;
    }

    const Family* fam = family(pl.RP, pl.CT);
    if (fam == nullptr) return fail(MIMO_ERR_UNSUPPORTED, "no kernel for this tile shape");
    // shape-exact instances when the call's shape equals the tile (see specialise())
    const int ti = tidx(pl.NT) * 3 + tidx(pl.PT);
    const bool ex = pl.ex;
    kfn kmain = fam->main[ti];
    int lds_main = pl.lds_main;
    // without y (no reduced dout, no z) the outputs are the states and qk_dot: the chunk
    // pass is the aggregate's state walk over whole segments (k_agg in ST mode) and
    // qk_dot a token-parallel kernel
    const bool states_only = !fwd && !p.need_y;
    if (fwd) {
        if (ex && p.reduce_o && p.has_z) kmain = fam->main_ex_fwd[ti];
    } else if (states_only) {
        kmain = ex ? fam->states_ex[ti] : fam->states[ti];
        lds_main = pl.lds_states;
    } else if (ex && p.reduce_o && p.has_z) {
        kmain = fam->main_ex_rz[ti];
    }
    if (!states_only) lds_main += kmain == fam->main[ti] ? fam->main_sa[ti] : fam->main_ex_sa[ti];
    const kfn kagg = ex ? fam->agg_ex[ti] : fam->agg[ti];
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int BH = p.B * p.H;
    auto mark = [&](int i) -> mimo_status {
        if (events == nullptr) return MIMO_OK;
        if (hipEventRecord(static_cast<hipEvent_t>(events[i]), st) != hipSuccess)
            return fail(MIMO_ERR_HIP, "hipEventRecord failed");
        return MIMO_OK;
    };
    if (events != nullptr)
        for (int i = 0; i < MIMO_TIMED_EVENTS; ++i)
            if (events[i] == nullptr) return fail(MIMO_ERR_VALUE, "timing event %d is NULL", i);
    if ((s = set_lds(kmain, lds_main)) != MIMO_OK) return s;
    if ((s = mark(0)) != MIMO_OK) return s;
    // the fork point is recorded before the chain; the side kernel is queued after the
    // chain's first kernel, which is on the critical path and so is dispatched first
    Side* sd = nullptr;
    if (states_only && fork) {
        if ((s = side_stream(&sd)) != MIMO_OK) return s;
        if (hipEventRecord(sd->fork, st) != hipSuccess) return fail(MIMO_ERR_HIP, "hipEventRecord failed");
    }
    auto side_qk = [&]() -> mimo_status {
        if (sd == nullptr) return MIMO_OK;
        if (hipStreamWaitEvent(sd->s, sd->fork, 0) != hipSuccess)
            return fail(MIMO_ERR_HIP, "fork onto the side stream failed");
        mimo_status r = launch_qk(p, pl.NT, sd->s);
        if (r != MIMO_OK) return r;
        if (hipEventRecord(sd->join, sd->s) != hipSuccess) return fail(MIMO_ERR_HIP, "hipEventRecord failed");
        return MIMO_OK;
    };
    if (pl.nseg > 1) {
        if ((s = set_lds(kagg, pl.lds_agg)) != MIMO_OK) return s;
        if ((s = launch(kagg, dim3(grid_blocks(p, pl.nsub)), dim3(pl.NW * 64), pl.lds_agg, st, p)) != MIMO_OK) return s;
        if ((s = side_qk()) != MIMO_OK) return s;
        if ((s = mark(1)) != MIMO_OK) return s;
        if ((s = launch_scan(p, BH, st)) != MIMO_OK) return s;
    } else {
        if ((s = mark(1)) != MIMO_OK) return s;
    }
    if ((s = mark(2)) != MIMO_OK) return s;
    if ((s = launch(kmain, dim3(grid_blocks(p, pl.nseg)), dim3(pl.NW * 64), lds_main, st, p)) != MIMO_OK) return s;
    if (pl.nseg <= 1 && (s = side_qk()) != MIMO_OK) return s;
    if (sd != nullptr && hipStreamWaitEvent(st, sd->join, 0) != hipSuccess)
        return fail(MIMO_ERR_HIP, "join of the side stream failed");
    if (states_only && sd == nullptr && (s = launch_qk(p, pl.NT, st)) != MIMO_OK) return s;
    if ((s = mark(3)) != MIMO_OK) return s;
    if (pl.nseg > 1 && p.need_y && !fwd)
        if ((s = launch_finish(p, st)) != MIMO_OK) return s;
    if ((s = mark(4)) != MIMO_OK) return s;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MIMO_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return MIMO_OK;
}

mimo_status mimo_bwd_fwd(const mimo_bwd_fwd_args* a, void* stream) { return run(a, nullptr, stream, nullptr); }

mimo_status mimo_bwd_fwd_timed(const mimo_bwd_fwd_args* a, void* stream, void* const* events) {
    if (events == nullptr) return fail(MIMO_ERR_VALUE, "events must not be NULL");
    return run(a, nullptr, stream, events);
}

mimo_status mimo_bwd_fwd_noalloc(const mimo_bwd_fwd_args* a, void* stream) {
    g_err.clear();
    Plan pl;
    mimo_status s = make_plan(a, &pl);
    if (s != MIMO_OK) return s;
    if (pl.ws_bytes > MIMO_NOALLOC_SCRATCH_BYTES)
        return fail(MIMO_ERR_UNSUPPORTED,
                    "this call needs %zu bytes of scratch; the fixed scratch of mimo_bwd_fwd_noalloc holds %zu "
                    "(use mimo_bwd_fwd with a workspace)",
                    pl.ws_bytes, (size_t)MIMO_NOALLOC_SCRATCH_BYTES);
    mimo_bwd_fwd_args b = *a;
    b.workspace = nullptr;
    b.workspace_bytes = 0;
    if (pl.ws_bytes > 0) {
        if ((s = scratch_on_current_device(&b.workspace)) != MIMO_OK) return s;
        b.workspace_bytes = MIMO_NOALLOC_SCRATCH_BYTES;
    }
    return run(&b, nullptr, stream, nullptr, false);
}

mimo_status mimo_fwd_workspace_size(const mimo_fwd_args* args, size_t* bytes) {
    if (args == nullptr) return fail(MIMO_ERR_VALUE, "args must not be NULL");
    const mimo_bwd_fwd_args a = as_bwd_args(args);
    Plan pl;
    const mimo_status s = make_plan(&a, &pl, true);
    if (s != MIMO_OK) return s;
    if (bytes == nullptr) return fail(MIMO_ERR_VALUE, "bytes must not be NULL");
    *bytes = pl.ws_bytes;
    return MIMO_OK;
}

static mimo_status run_fwd(const mimo_fwd_args* f, void* stream, void* const* events) {
    g_err.clear();
    if (f == nullptr) return fail(MIMO_ERR_VALUE, "args must not be NULL");
    if (f->o == nullptr) return fail(MIMO_ERR_VALUE, "o must not be NULL");
    const mimo_bwd_fwd_args a = as_bwd_args(f);
    return run(&a, f->o, stream, events);
}

mimo_status mimo_fwd(const mimo_fwd_args* a, void* stream) { return run_fwd(a, stream, nullptr); }

mimo_status mimo_fwd_timed(const mimo_fwd_args* a, void* stream, void* const* events) {
    if (events == nullptr) return fail(MIMO_ERR_VALUE, "events must not be NULL");
    return run_fwd(a, stream, events);
}

mimo_status mimo_bwd_fwd_f32_workspace_size(const mimo_bwd_fwd_args* args, size_t* bytes) {
    Prob32 q;
    mimo_status s = prob_from_mimo(args, false, &q);
    if (s != MIMO_OK) return s;
    Plan32 pl;
    if ((s = make_plan32(q, &pl)) != MIMO_OK) return s;
    if (bytes == nullptr) return fail(MIMO_ERR_VALUE, "bytes must not be NULL");
    *bytes = pl.ws_bytes;
    return MIMO_OK;
}

mimo_status mimo_bwd_fwd_f32(const mimo_bwd_fwd_args* a, void* stream) { return run_bwd32(a, stream, nullptr); }

mimo_status mimo_bwd_fwd_f32_timed(const mimo_bwd_fwd_args* a, void* stream, void* const* events) {
    if (events == nullptr) return fail(MIMO_ERR_VALUE, "events must not be NULL");
    return run_bwd32(a, stream, events);
}

mimo_status mimo_fwd_f32_workspace_size(const mimo_fwd_args* args, size_t* bytes) {
    if (args == nullptr) return fail(MIMO_ERR_VALUE, "args must not be NULL");
    const mimo_bwd_fwd_args a = as_bwd_args(args);
    Prob32 q;
    mimo_status s = prob_from_mimo(&a, true, &q);
    if (s != MIMO_OK) return s;
    Plan32 pl;
    if ((s = make_plan32(q, &pl)) != MIMO_OK) return s;
    if (bytes == nullptr) return fail(MIMO_ERR_VALUE, "bytes must not be NULL");
    *bytes = pl.ws_bytes;
    return MIMO_OK;
}

mimo_status mimo_fwd_f32(const mimo_fwd_args* a, void* stream) { return run_fwd32(a, stream, nullptr); }

mimo_status mimo_siso_fwd_workspace_size(const mimo_siso_fwd_args* args, size_t* bytes) {
    Prob32 q;
    mimo_status s = prob_from_siso(args, &q);
    if (s != MIMO_OK) return s;
    Plan32 pl;
    if ((s = make_plan32(q, &pl)) != MIMO_OK) return s;
    if (bytes == nullptr) return fail(MIMO_ERR_VALUE, "bytes must not be NULL");
    *bytes = pl.ws_bytes;
    return MIMO_OK;
}

mimo_status mimo_siso_fwd(const mimo_siso_fwd_args* a, void* stream) { return run_siso(a, stream, nullptr); }

mimo_status mimo_siso_fwd_timed(const mimo_siso_fwd_args* a, void* stream, void* const* events) {
    if (events == nullptr) return fail(MIMO_ERR_VALUE, "events must not be NULL");
    return run_siso(a, stream, events);
}

mimo_status mimo_bwd_bwd_workspace_size(const mimo_bwd_bwd_args* args, size_t* bytes) {
    PlanB2 pl;
    const mimo_status s = make_plan_b2(args, &pl);
    if (s != MIMO_OK) return s;
    if (bytes == nullptr) return fail(MIMO_ERR_VALUE, "bytes must not be NULL");
    *bytes = pl.ws_bytes;
    return MIMO_OK;
}

mimo_status mimo_bwd_bwd(const mimo_bwd_bwd_args* a, void* stream) { return run_b2(a, stream, nullptr); }

mimo_status mimo_bwd_bwd_timed(const mimo_bwd_bwd_args* a, void* stream, void* const* events) {
    if (events == nullptr) return fail(MIMO_ERR_VALUE, "events must not be NULL");
    return run_b2(a, stream, events);
}

}  // extern "C"
