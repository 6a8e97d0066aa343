/*
 * mimo_bwd_fwd.h -- C ABI of the MI355X (gfx950) implementation of the first
 * stage of the Mamba-3 MIMO combined backward, "mamba_mimo_bwd_fwd".
 *
 * Operation (Triton-Ascend mamba_mimo_bwd_fwd pull request page: operator
 * document, "inputs and outputs" tables and constraints; BF16-boundary
 * PyTorch reference, whole listing). For every batch b and value head h
 * (q/k group g = h / (H/G)) the call re-runs the chunked MIMO scan over the
 * sequence in chunks of C tokens and writes
 *   states [B,H,nc,N,P] bf16  -- the fp32 recurrent state *entering* chunk c,
 *                                rounded to bf16 (nc = ceil(S/C));
 *   qk_dot [B,H,S,R,R]  bf16  -- the same-token dot of the biased, unrotated
 *                                q (rank r_out) and k (rank r_in);
 *   dmimo_o [B,H,R,P]   fp32  -- (reduced dout only) output-projection gradient;
 *   dz      [B,S,H,P]   bf16  -- (z given) gradient of the gate input;
 *   dmimo_z [B,H,R,P]   fp32  -- (z given) gate-projection gradient.
 * dmimo_o and dmimo_z are per batch (not summed over B). Intermediate values
 * are rounded to bf16 at the same points as the pages' BF16-boundary
 * reference; dots, the state and the gradient sums accumulate in fp32.
 *
 * Layouts: every tensor is dense, row-major (C order), in the pages' shapes:
 *   dout   [B,S,H,P] when mimo_o != NULL ("reduced"), else [B,S,R,H,P]   bf16
 *   q, k   [B,S,R,G,N] bf16        v, z [B,S,H,P] bf16
 *   q_bias, k_bias [H,R,N] fp32    mimo_v, mimo_o, mimo_z [H,R,P] fp32
 *   angles [B,S,H,N/rotary_dim_divisor] fp32
 *   da_cs, da_cs_rev, dt [B,H,S] fp32     trap [B,H,S] bf16
 *   d [H] fp32                     segsum [B,H,nc,C,C] fp32
 * bf16 values are passed as their 16-bit patterns (uint16_t).
 * Alignment: dout, q, k, v, z and the bf16 outputs (states, qk_dot, dz, and o
 * of the layer output) are read and written in 16-byte pieces and must be
 * 16-byte aligned (MIMO_ERR_VALUE otherwise); the other pointers need their
 * element's natural alignment, and the workspace 256 bytes.
 *
 * Branches follow the pages: mimo_o != NULL selects the reduced dout layout
 * and enables dmimo_o; z != NULL enables dz and dmimo_z (mimo_z is then
 * required, and must be NULL otherwise); d != NULL adds the skip term.
 *
 * Ownership: the caller owns every buffer (inputs, outputs and the
 * workspace) and keeps them alive until the work queued on the stream has
 * finished. All pointers are device pointers of the current HIP device.
 * The library never allocates, frees or synchronises; it keeps no state
 * between calls except a per-device cache of the device architecture.
 *
 * Errors: every entry point returns a mimo_status. On error nothing has been
 * queued, and mimo_last_error() returns a message (thread-local storage).
 */
#ifndef MIMO_BWD_FWD_H
#define MIMO_BWD_FWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MIMO_ABI_VERSION 2

typedef enum {
    MIMO_OK = 0,
    MIMO_ERR_VALUE = 1,        /* bad shape, size, pointer or branch combination (ValueError) */
    MIMO_ERR_TYPE = 2,         /* reserved for dtype errors raised by bindings (TypeError)     */
    MIMO_ERR_UNSUPPORTED = 3,  /* valid on the pages but not supported here (NotImplementedError) */
    MIMO_ERR_HIP = 4           /* a HIP runtime call failed (RuntimeError)                     */
} mimo_status;

typedef struct mimo_bwd_fwd_args {
    /* sizes: batch, sequence, value heads, q/k groups, MIMO rank, state dim, value dim */
    int64_t B, S, H, G, R, N, P;
    int32_t chunk_size;          /* C >= 1, C*R <= 128                               */
    int32_t rotary_dim_divisor;  /* 2 or 4; N must be even and divisible by it       */
    /* inputs (device pointers; the optional ones may be NULL) */
    const uint16_t *dout, *q, *k, *v;
    const float *q_bias, *k_bias, *mimo_v;
    const float *mimo_o;         /* optional: selects reduced dout                    */
    const uint16_t *z;           /* optional                                          */
    const float *mimo_z;         /* required iff z != NULL                            */
    const float *angles, *da_cs, *da_cs_rev, *dt;
    const uint16_t *trap;
    const float *d;              /* optional                                          */
    const float *segsum;
    /* outputs (device pointers): dmimo_o must be non-NULL iff mimo_o is given,
     * dz and dmimo_z iff z is given; states and qk_dot always. */
    float *dmimo_o;
    uint16_t *states;
    uint16_t *dz;
    float *dmimo_z;
    uint16_t *qk_dot;
    /* scratch: device memory of at least mimo_bwd_fwd_workspace_size() bytes,
     * 256-byte aligned; its contents on entry do not matter. May be NULL when
     * the required size is 0. */
    void *workspace;
    size_t workspace_bytes;
} mimo_bwd_fwd_args;

/* Size in bytes of the workspace a call with these sizes and branches needs
 * (reads only the size fields, chunk_size and which optional pointers are
 * NULL). Returns MIMO_ERR_VALUE / MIMO_ERR_UNSUPPORTED for shapes the call
 * would reject. */
mimo_status mimo_bwd_fwd_workspace_size(const mimo_bwd_fwd_args *args, size_t *bytes);

/* Validate the arguments and queue the whole computation on `stream`
 * (a hipStream_t; NULL = the default stream of the current device).
 * Asynchronous: returns once the kernels are queued. A call without y (no
 * mimo_o and no z: the outputs are states and qk_dot) runs its qk_dot kernel
 * on a stream of the library's own (one per calling thread and device, made
 * on first use and kept, default priority), ordered after the work already
 * queued on `stream`; work queued on `stream` afterwards waits for it. Within the pages'
 * constraints (C*R <= 128, N, P <= 128, N even and divisible by the rotary
 * divisor, H % G == 0) this library further requires N and P to be
 * multiples of 16, C <= 64, R <= 8 and RP * CP <= 128, where RP is R rounded
 * up to a power of two and CP is C rounded up to 16, 32 or 64; other shapes
 * return MIMO_ERR_UNSUPPORTED. Requires a gfx950 device, else
 * MIMO_ERR_UNSUPPORTED. */
mimo_status mimo_bwd_fwd(const mimo_bwd_fwd_args *args, void *stream);

/* mimo_bwd_fwd with per-kernel timing, for measurement. `events` points to
 * MIMO_TIMED_EVENTS hipEvent_t handles the caller created (hipEventCreate) on
 * the current device. They are recorded on `stream` before the
 * segment-aggregate kernel, before the segment scan, before the chunk
 * kernel, after the chunk kernel and after the final reduction; a kernel
 * that does not run for this shape leaves its two events back to back.
 * Same operation, arguments, ownership and errors as mimo_bwd_fwd. */
#define MIMO_TIMED_EVENTS 5
mimo_status mimo_bwd_fwd_timed(const mimo_bwd_fwd_args *args, void *stream, void *const *events);

/* mimo_bwd_fwd without any allocation, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same operation, arguments, layouts, ownership and errors as
 * mimo_bwd_fwd, except that args->workspace and args->workspace_bytes are
 * ignored: the scratch lives in a fixed device array of
 * MIMO_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs on
 * until the process ends. A call whose workspace (mimo_bwd_fwd_workspace_size)
 * would exceed it returns MIMO_ERR_UNSUPPORTED and queues nothing. The array
 * is shared by every call on a device and keeps the last call's contents (no
 * call relies on them): calls that overlap on one device, from other streams
 * or threads, race on it and must be serialised by the caller. The call itself
 * allocates nothing and never calls hipMalloc or hipFree. */
#define MIMO_NOALLOC_SCRATCH_BYTES (64u << 20)
mimo_status mimo_bwd_fwd_noalloc(const mimo_bwd_fwd_args *args, void *stream);

/*
 * Layer output of the same chunked MIMO scan: the forward whose gradients the
 * backward's gating branches compute (Triton-Ascend mamba_mimo_bwd_fwd pull
 * request page, BF16-boundary PyTorch reference: dmimo_o, dz and dmimo_z are
 * the derivatives of sum(o * dout) with respect to mimo_o, z and mimo_z; the
 * pages give the backward only, so this is an inferred definition). With y the
 * backward's bf16 per-rank output and silu(pz) = pz * sigmoid(pz),
 * pz = z * mimo_z (the factor is 1 without z):
 *   mimo_o given:  o [B,S,H,P]   bf16 = bf16( sum_r (y * bf16(mimo_o)) * silu(pz) ),
 *                                        rank sum in rank order in fp32;
 *   mimo_o NULL:   o [B,S,R,H,P] bf16 = bf16( y * silu(pz) ).
 * Inputs, layouts, branch rules (except dout, which is absent), ownership,
 * shape limits and errors as for mimo_bwd_fwd_args / mimo_bwd_fwd; the call
 * writes o only.
 */
typedef struct mimo_fwd_args {
    int64_t B, S, H, G, R, N, P;
    int32_t chunk_size;
    int32_t rotary_dim_divisor;
    const uint16_t *q, *k, *v;
    const float *q_bias, *k_bias, *mimo_v;
    const float *mimo_o;         /* optional: selects the rank-reduced output          */
    const uint16_t *z;           /* optional                                           */
    const float *mimo_z;         /* required iff z != NULL                             */
    const float *angles, *da_cs, *da_cs_rev, *dt;
    const uint16_t *trap;
    const float *d;              /* optional                                           */
    const float *segsum;
    uint16_t *o;                 /* output (device pointer), never NULL                */
    void *workspace;             /* at least mimo_fwd_workspace_size() bytes, 256-byte aligned */
    size_t workspace_bytes;
} mimo_fwd_args;

/* Workspace bytes a mimo_fwd call with these sizes and branches needs. */
mimo_status mimo_fwd_workspace_size(const mimo_fwd_args *args, size_t *bytes);

/* Validate and queue the layer output on `stream` (asynchronous). */
mimo_status mimo_fwd(const mimo_fwd_args *args, void *stream);

/* mimo_fwd with the same MIMO_TIMED_EVENTS events as mimo_bwd_fwd_timed (the
 * final-reduction kernel does not run: its two events are back to back). */
mimo_status mimo_fwd_timed(const mimo_fwd_args *args, void *stream, void *const *events);

/*
 * FP32-intermediate variant (Triton-Ascend mamba_mimo_bwd_fwd pull request
 * page, FP32 PyTorch reference): the same operation with no bf16 rounding of
 * any intermediate value -- biased q/k, rotation, PsiV with unrounded mimo_v,
 * dt and the trapezoid weights (look-ahead weight dt[t+1]*(1 - sigmoid(trap
 * [t+1]))), kappa, the causal block, the fp32 state in the inter term, y, the
 * diagonal, dPhiO with unrounded mimo_o, and the dz sum all stay fp32, with
 * fp32 contractions. Outputs keep their dtypes (states, qk_dot, dz bf16 by
 * round-to-nearest-even; dmimo fp32). Arguments, layouts, ownership and errors
 * as for mimo_bwd_fwd, with these limits instead of its tile limits: N and P
 * multiples of 16 up to 128, chunk_size <= 64, R <= 8, R * (chunk_size rounded
 * up to 16) <= 128 (MIMO_ERR_UNSUPPORTED otherwise). Where R * chunk_size > 64
 * with N or P = 128 the fp32 tiles exceed one compute unit's LDS and the K~ tile
 * of each workgroup is kept in the workspace (MT x (N + 4) floats a block).
 */
mimo_status mimo_bwd_fwd_f32_workspace_size(const mimo_bwd_fwd_args *args, size_t *bytes);
mimo_status mimo_bwd_fwd_f32(const mimo_bwd_fwd_args *args, void *stream);
mimo_status mimo_bwd_fwd_f32_timed(const mimo_bwd_fwd_args *args, void *stream, void *const *events);

/* The layer output (mimo_fwd) with fp32 intermediates: o = sum_r mimo_o * y * silu(pz)
 * (or per rank) with y, the projections and the gate in fp32 and only o rounded
 * to bf16. Limits as for mimo_bwd_fwd_f32. */
mimo_status mimo_fwd_f32_workspace_size(const mimo_fwd_args *args, size_t *bytes);
mimo_status mimo_fwd_f32(const mimo_fwd_args *args, void *stream);

/*
 * SISO forward (mamba3_siso_fwd_kernel migration page: interface, inputs and
 * "implementation principle"). For batch b, head h (q/k head h / (H/Hq)):
 * q, k get their bias and a partial rotate-half by `angles` (pairs [0,A) with
 * [K/2, K/2+A)); gamma_t = dt_t * sigmoid(trap_t) and the look-ahead weight
 * dt_{t+1} * (1 - sigmoid(trap_{t+1})) scale k; inside each chunk the strictly
 * causal score q^_t . k~_s is weighted by exp(sum of adt over (s, t]), the
 * previous chunks enter through the carried state, the same-token term is
 * gamma_t (q^_t . k^_t) v_t, d[h] v_t is added, and with z the result is gated
 * by silu(z). Intermediates are fp32; the output takes the input dtype.
 * Layouts (dense, row-major): q, k [B,S,Hq,K]; v, z, out [B,S,H,V];
 * adt, dt, trap [B,H,S] fp32; q_bias, k_bias [H,K] fp32; angles [B,S,H,A]
 * fp32 (may be NULL when A = 0); d [H] fp32. chunk_size 32 or 64; H % Hq == 0; A even and <= K/2
 * (MIMO_ERR_VALUE otherwise). K and V must be multiples of 16 up to 128 and
 * the fp32 tiles must fit the LDS (MIMO_ERR_UNSUPPORTED otherwise). q, k, v, z
 * and out must be 16-byte aligned (MIMO_ERR_VALUE otherwise).
 * Ownership, asynchrony and errors as for mimo_bwd_fwd.
 */
#define MIMO_DTYPE_BF16 0
#define MIMO_DTYPE_FP16 1
#define MIMO_DTYPE_FP32 2   /* stage-2 backward only */
typedef struct mimo_siso_fwd_args {
    int64_t B, S, Hq, H, K, V;
    int32_t chunk_size;          /* 32 or 64                                           */
    int32_t A;                   /* rotated pairs: the last axis of angles             */
    int32_t dtype;               /* MIMO_DTYPE_BF16 or MIMO_DTYPE_FP16 for q, k, v, z, out */
    const uint16_t *q, *k, *v;
    const float *adt, *dt, *trap;
    const float *q_bias, *k_bias, *angles;
    const float *d;              /* optional                                           */
    const uint16_t *z;           /* optional                                           */
    uint16_t *out;
    void *workspace;             /* at least mimo_siso_fwd_workspace_size() bytes, 256-byte aligned */
    size_t workspace_bytes;
} mimo_siso_fwd_args;

mimo_status mimo_siso_fwd_workspace_size(const mimo_siso_fwd_args *args, size_t *bytes);
mimo_status mimo_siso_fwd(const mimo_siso_fwd_args *args, void *stream);
/* mimo_siso_fwd with the MIMO_TIMED_EVENTS events of mimo_bwd_fwd_timed. */
mimo_status mimo_siso_fwd_timed(const mimo_siso_fwd_args *args, void *stream, void *const *events);

/*
 * Stage-2 backward (mamba3_mimo_bwd_bwd; Triton-Ascend pull request page:
 * "practice" document and migration note). Consumes the first stage's states
 * and qk_dot and returns twelve gradients of L = sum dPhiO * y, with y the
 * pre-gate per-rank output (Z gating belongs to the first stage) and dPhiO =
 * dout * mimo_o (reduced) or the per-rank dout. Intermediates are fp32. Each
 * output is the derivative with respect to one use of one quantity, the caches
 * giving the values of the chunk entry states and same-token dots:
 *   dq, dk      [B, S*R, H, N]  the biased q, k of each head (row t*R + r)
 *   dv          [B,S,H,P]       dmimo_v [B,H,R,P] (per batch)   dd [B,H] (iff d)
 *   dangles     [B,S,H,N/rotary_dim_divisor]
 *   dfactor     [B,H,S]  the K scale factor_t = gamma_t + beta_t
 *   dgamma      [B,H,S]  gamma_t in the same-token term
 *   dda_cs      [B,H,S]  da_cs[t] in the inter-term scale exp(da_cs[t])
 *   dda         [B,H,S]  da_cs at each chunk's last token in the state decay (0 elsewhere)
 *   dda_cs_rev  [B,H,S]  da_cs_rev[t] in kappa = K~ * exp(da_cs_rev[t])
 *   dssda       [B,H,nc,C,C]  segsum[c][t][s], s < t (0 elsewhere)
 * Inputs as for mimo_bwd_fwd (dout reduced or not) plus states [B,H,nc,N,P] and
 * qk_dot [B,H,S,R,R]. The data tensors dout, q, k, v, states, qk_dot and trap
 * share one dtype, in_dtype: MIMO_DTYPE_BF16, MIMO_DTYPE_FP16 or MIMO_DTYPE_FP32
 * (the migration note's supported dtypes); the other inputs are fp32. dq, dk and
 * dv are stored in out_dtype (same choices; the page's default is the input
 * dtype, which the binding applies); the other outputs are fp32. Limits (the
 * migration note's range): R * chunk_size, N and P at most 128, R at most 8, N
 * and P multiples of 8 (MIMO_ERR_UNSUPPORTED otherwise). Beyond 64 in any of
 * them the chunk tiles are kept in the workspace (one slot per workgroup, about
 * 608 KB each). dout, q, k, v, states, q_bias, k_bias, mimo_v, mimo_o, dq, dk
 * and dv must be 16-byte aligned (MIMO_ERR_VALUE otherwise). Ownership,
 * asynchrony and errors as for mimo_bwd_fwd.
 */
typedef struct mimo_bwd_bwd_args {
    int64_t B, S, H, G, R, N, P;
    int32_t chunk_size;
    int32_t rotary_dim_divisor;
    int32_t in_dtype;            /* MIMO_DTYPE_* of dout, q, k, v, states, qk_dot, trap */
    int32_t out_dtype;           /* MIMO_DTYPE_* of dq, dk, dv                          */
    const void *dout, *q, *k, *v;
    const float *q_bias, *k_bias, *mimo_v;
    const void *states, *qk_dot;
    const float *da_cs, *da_cs_rev, *dt;
    const void *trap;
    const float *segsum, *angles;
    const float *mimo_o;         /* optional: selects reduced dout                    */
    const float *d;              /* optional                                          */
    void *dq, *dk, *dv;
    float *dmimo_v, *dangles, *dfactor, *dgamma, *dda, *dssda, *dda_cs_rev, *dda_cs;
    float *dd;                   /* required iff d != NULL                            */
    void *workspace;             /* at least mimo_bwd_bwd_workspace_size() bytes, 256-byte aligned */
    size_t workspace_bytes;
} mimo_bwd_bwd_args;

mimo_status mimo_bwd_bwd_workspace_size(const mimo_bwd_bwd_args *args, size_t *bytes);
mimo_status mimo_bwd_bwd(const mimo_bwd_bwd_args *args, void *stream);
/* mimo_bwd_bwd with the MIMO_TIMED_EVENTS events of mimo_bwd_fwd_timed (segment
 * aggregate, reverse scan, chunk pass, final sums). */
mimo_status mimo_bwd_bwd_timed(const mimo_bwd_bwd_args *args, void *stream, void *const *events);

/* Message describing the last error of the calling thread ("" if none). */
const char *mimo_last_error(void);

/* MIMO_ABI_VERSION of the library. */
int mimo_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MIMO_BWD_FWD_H */
