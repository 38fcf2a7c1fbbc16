/*
 * tos.h -- C ABI of libtos.so: fused attention forward pass with the tensorized
 * online softmax, for AMD Instinct MI355X (gfx950).
 *
 * The operation (FlashAttention-T page, section A3 "fused attention algorithm
 * flow" and Fig 2(a); section A2 "tensorized online softmax", Algorithm 1):
 *
 *   O[b,h,i,:] = sum_j softmax_j(scale * <q_i, k_j>) v_j
 *   lse[b,h,i] = ln sum_j exp(scale * <q_i, k_j>)
 *
 * over the valid keys j (all j < N, or j <= i when causal).  The softmax runs
 * online over blocks of keys with the surrogate maximum of section A2: the
 * subtracted maximum is the largest running row maximum over an X-row tile, so
 * the rescale of O is one uniform factor exp2(c*(m^_old - m^)) per tile and
 * Z = c*S - c*m^ feeds exp2 (c = scale*log2(e)).  An optional per-row fallback
 * guards against the all-underflow case of section A2 ("numerical stability
 * guarantees").
 *
 * Conventions for every entry point:
 *   - Tensors are contiguous row-major [B][H][N][d] (q, k, v, o) and [B][H][N]
 *     (lse), in device memory (hipMalloc / torch CUDA tensors).  Base pointers
 *     are 16-byte aligned.  Self-attention only: queries and keys share N.
 *   - The caller owns every buffer.  The library allocates no device memory
 *     and keeps no pointer after returning.  Its only global state is a
 *     per-device record of the compute-unit count, read on the first call
 *     that launches on the device (the kernels run one workgroup per compute
 *     unit, each over a list of query blocks).
 *   - Problems with fewer 256-row query blocks than the device has compute
 *     units (few heads, short sequences) can also cut each query block's keys
 *     into pieces that run on separate compute units and are merged by a
 *     second kernel on the same stream.  That needs a device workspace from
 *     the caller (tos_fwd_opts.workspace, sized by tos_attn_fwd_workspace_size);
 *     without one the call runs whole query blocks, with the same results up
 *     to rounding.
 *   - fp32 inputs at X = 1 or 16 without the fallback run, when 128-row
 *     workgroups would number fewer than the compute units, in workgroups of
 *     16 query rows whose waves split the keys and merge their partial
 *     results exactly (the same rescale by exp(m_old - m_new)) in LDS, with
 *     up to 4 workgroups sharing the head dim of O; no workspace is needed.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without synchronising.  A device fault surfaces at the
 *     caller's next synchronisation.
 *   - Arguments are validated before anything is launched: on any error status
 *     nothing has been written.
 *   - Thread safety: calls may be made concurrently from several host threads.
 */
#ifndef TOS_H
#define TOS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TOS_VERSION 2

typedef enum {
    TOS_OK = 0,
    TOS_ERR_INVALID_ARG = 1,   /* null required pointer, negative size, bad scale,
                                  aliasing output, misaligned pointer, bad option  */
    TOS_ERR_UNSUPPORTED = 2,   /* valid request outside what the kernels cover
                                  (head dim not 64/128, size limits, option not
                                  available for the dtype)                        */
    TOS_ERR_HIP = 3,           /* the HIP runtime rejected the launch             */
    TOS_ERR_SCRATCH = 4        /* tos_attn_fwd_noalloc: the problem needs more
                                  workspace than the library's static area holds */
} tos_status;

typedef enum {
    TOS_F32 = 0,       /* q, k, v, o: float32                                       */
    TOS_BF16 = 1,      /* q, k, v, o: bfloat16                                      */
    TOS_FP8_E4M3 = 2,  /* q, k, v: OCP float8 e4m3fn codes (x = descale * code);
                          o: bfloat16; descales are required in the options       */
    TOS_F16 = 3        /* q, k, v, o: IEEE float16 (the same kernel family as
                          bf16, with the fp16 matrix instructions)                */
} tos_dtype;

/* Where the element-wise softmax steps run: the vector unit or the matrix unit
 * (FlashAttention-T section A2: repurposed matrix instructions for the row sum,
 * Fig 5(b), and for scaling / fused multiply-add, Fig 5(a); the tensor-vector
 * split of Fig 6).  The matrix-unit forms are fp32 products for the scaling and
 * the FMA (gfx950 has no TF32 matrix instruction; bf16 products would round O
 * or Z past the tolerance) and 16-bit products against an all-ones operand for
 * the row sum.  split_num / split_den in tos_fwd_opts give the matrix unit's
 * share where a value takes one.  bf16 and f16 only; values other than
 * TOS_SPLIT_VALU and TOS_SPLIT_ROWSUM_MFMA need X = 32, no fallback and the
 * co-scheduled schedule (else TOS_ERR_UNSUPPORTED). */
typedef enum {
    TOS_SPLIT_VALU = 0,         /* everything on the vector unit (the row sum as
                                   dot products of packed P~ pairs with (1, 1))    */
    TOS_SPLIT_ROWSUM_MFMA = 1,  /* the row sum on the matrix unit: ones x P~^T.
                                   With split_den > 0, only a share of each key
                                   block's four 16-key steps (num/den, a multiple
                                   of 1/4; < 1 needs X = 32 and no fallback), the
                                   rest on the vector unit                         */
    TOS_SPLIT_SCALE_MFMA = 2,   /* the O rescale by the tile's factor alpha on the
                                   matrix unit (products against alpha I)          */
    TOS_SPLIT_HSPLIT = 3,       /* horizontal split (Fig 6(a)): in every 32x32 tile
                                   of S and of O, the register slices below the
                                   share num/den (1/4, 1/2 or 3/4) run
                                   Z = c*S - c*m^ and the O rescale on the matrix
                                   unit, the rest on the vector unit; the same
                                   share of the row-sum steps on the matrix unit  */
    TOS_SPLIT_VSPLIT = 4,       /* vertical split (Fig 6(b)) with share 1/2: the
                                   first of a block's two S tiles and the first
                                   half of O's tiles on the matrix unit, and half
                                   the row-sum steps                               */
    TOS_SPLIT_ALL_MFMA = 5      /* every step that has a matrix form on the matrix
                                   unit: Z (the offset -c*m^ carried into the
                                   accumulator by one more product), the O rescale
                                   and the row sum (the pages' AllTensor variant)  */
} tos_softmax_split;
/* Either way l sums the rounded P~ that the P~V product consumes, and a separate
 * unrounded fp32 sum gives lse.  Z and the O rescale take their matrix form in
 * the steady steps of the pipeline; a wave's first and last key blocks (where
 * logits may be masked) keep the vector form.  TOS_FP8_E4M3 has no vector form
 * for e4m3 pairs: its rounded sum is always the matrix-unit one, and it accepts
 * only TOS_SPLIT_VALU and TOS_SPLIT_ROWSUM_MFMA (both meaning that). */

/* Instruction schedule of the 16-bit kernels (an ablation of FlashAttention-T
 * section A2, "tensor-vector parallelism", Fig 7, and of its evaluation, Fig 9
 * and Fig 10). */
typedef enum {
    TOS_SCHEDULE_COSCHED = 0,    /* matrix and vector work of consecutive key
                                    blocks interleaved in one instruction stream
                                    (the default)                                    */
    TOS_SCHEDULE_SEQUENTIAL = 1  /* each key block's softmax, then the next block's
                                    QK^T, then the previous block's P~V, one after
                                    another; overlap only across the waves of a
                                    SIMD.  bf16 and f16 only, with the vector row
                                    sum, no AUTO fallback and X = 1 or 32; other
                                    combinations return TOS_ERR_UNSUPPORTED         */
} tos_schedule;

/* All-underflow handling (FlashAttention-T section A2, "numerical stability
 * guarantees": an implementation may fall back to per-row computation). */
typedef enum {
    TOS_FALLBACK_OFF = 0,    /* surrogate maximum throughout; a row whose
                                exponentials all underflow gets O = 0, lse = -inf  */
    TOS_FALLBACK_AUTO = 1,   /* per tile and key block, before exponentiating: if
                                c*(m^_new - min_i m_i) > tau the tile switches, for
                                the rest of the pass, to per-row maxima            */
    TOS_FALLBACK_FORCE = 2   /* per-row maxima from the first block                 */
} tos_fallback;

typedef struct {
    int size;              /* sizeof(tos_fwd_opts): the struct version             */
    int x_tile;            /* surrogate tile rows X: 0 = default (32), 1, 16, 32 or
                              64; X = 1 is the per-row online softmax; X = 64 (two
                              waves exchange their halves through LDS) needs
                              bf16/f16 and the VALU row sum, else
                              TOS_ERR_UNSUPPORTED                                  */
    int softmax_split;     /* a tos_softmax_split value                             */
    int fallback;          /* a tos_fallback value                                  */
    float fallback_tau;    /* AUTO threshold in log2 units, at most 126; 0 =
                              default (100 for f32/bf16 P~, 24 for f16 P~, 12 for
                              e4m3 P~).  The switch rescales by up to 2^tau, which
                              must stay finite in fp32                             */
    float q_descale;       /* fp8 only: real value = descale * stored code; > 0    */
    float k_descale;
    float v_descale;
    int* fallback_tiles;   /* NULL, or a device int the kernels add to, once per
                              X-row tile that ran with per-row maxima (AUTO switch
                              or FORCE).  The caller zeroes it.                    */
    int schedule;          /* a tos_schedule value                                  */
    int split_num;         /* the matrix unit's share split_num / split_den of the */
    int split_den;         /* softmax_split value (0 / 0: the value's default)     */
    void* workspace;       /* NULL, or device memory of workspace_bytes that the
                              bf16 / f16 kernels may use for pieces of query
                              blocks (see the conventions above); used only when
                              workspace_bytes >= tos_attn_fwd_workspace_size(...)
                              and the fallback is off; must not overlap the
                              tensors; its contents on entry do not matter      */
    size_t workspace_bytes;
    uint64_t* trace;       /* NULL, or a device buffer of trace_bytes: runs a
                              phase-stamped copy of the kernel (bf16, d = 128,
                              fallback off; X = 1 / 16 / 32 co-scheduled, X = 1 /
                              32 sequential, or X = 32 with the matrix-unit row
                              sum or everything on the matrix unit; else
                              TOS_ERR_UNSUPPORTED) that writes, per wave, s_memtime
                              cycles of its steps and their phases to 16 slots at
                              trace[(workgroup * 8 + wave) * 16]: 0 wave total,
                              1 steady steps, 2 their cycles, 3 phase A, 4 phase
                              B, 5 barrier wait, 6 edge steps, 7 their cycles,
                              8 their softmax section, 9 barrier wait, 10 the
                              wave total in s_memrealtime ticks (100 MHz), 11 /
                              12 s_memrealtime at the wave's first and last
                              stamp (13-15 unused).  The
                              buffer holds one workgroup per compute unit:
                              trace_bytes >= compute units * 1024 (else
                              TOS_ERR_INVALID_ARG); the caller zeroes it     */
    size_t trace_bytes;
} tos_fwd_opts;

/*
 * tos_attn_fwd -- O = softmax(scale * Q K^T) V and lse, as described above.
 *
 *   q, k, v   device pointers, [B][H][N][d] of `dtype` (see tos_dtype); the
 *             values must be finite (NaN or infinite inputs give unspecified
 *             outputs)
 *   o         device pointer, [B][H][N][d]: float32 for TOS_F32, float16 for
 *             TOS_F16, bfloat16 otherwise; must not overlap q, k, v or lse
 *   lse       device pointer to [B][H][N] float32 natural-log log-sum-exp of the
 *             scaled logits, or NULL to skip it
 *   B, H, N   batch, heads, sequence length; >= 0 (any zero: nothing to do,
 *             TOS_OK); B*H*ceil(N/128) must stay below 2^31
 *   d         head dimension: 64 or 128
 *   causal    0: every key; 1: key j <= query i (top-left aligned)
 *   scale     softmax scale applied to <q, k>; finite and > 0
 *   dtype     a tos_dtype value
 *   opts      NULL for defaults (X = 32, VALU row sum, no fallback), or options
 *   stream    hipStream_t to enqueue on
 *
 * Returns TOS_OK or an error status; see tos_status.
 */
tos_status tos_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                        tos_dtype dtype, const tos_fwd_opts* opts, void* stream);

/*
 * tos_attn_fwd_noalloc -- tos_attn_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments and results; opts->workspace must be NULL
 * (TOS_ERR_INVALID_ARG otherwise): the pieces' workspace is a static device
 * array of 17.3 MB (256 units x 256 rows x (2 x 128 + 8) bytes, what any call
 * with d <= 128 can need), which each GPU the library runs on holds until the
 * process ends.  A
 * call that would need more returns TOS_ERR_SCRATCH.  The call allocates
 * nothing; its first call on a device looks the array's address up.  Every
 * call on one GPU shares that array: calls that overlap in time on one GPU
 * (other streams, other host threads) race on it and must be serialised by
 * the caller; its contents on entry do not matter.
 */
tos_status tos_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                                tos_dtype dtype, const tos_fwd_opts* opts, void* stream);

/* Device workspace, in bytes, that tos_attn_fwd with these arguments and
 * options (NULL = defaults) would use to cut query blocks into pieces on the
 * current device: 0 when the problem has enough query blocks to fill the
 * device, or the options rule it out (fp32 or fp8 inputs, a fallback other
 * than off).  At most 256 x 256 x (2d + 8) bytes (17.3 MB at d = 128): per
 * unit, its partial O as fp16 rows, each scaled by a power of 2, then per row
 * its lse and that power's exponent as floats.
 * Returns TOS_ERR_INVALID_ARG for a NULL bytes pointer or sizes/options that
 * tos_attn_fwd would reject as invalid. */
tos_status tos_attn_fwd_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                                       tos_dtype dtype, const tos_fwd_opts* opts, size_t* bytes);

/* Fills *opts with the defaults (size set, X = 32, VALU, fallback off,
 * descales 1, co-scheduled, no workspace).  Returns TOS_ERR_INVALID_ARG for
 * NULL. */
tos_status tos_fwd_opts_default(tos_fwd_opts* opts);

/* Algorithmic matrix-unit work of one call: 4*B*H*N^2*d flops, halved when
 * causal (the throughput metric's convention). */
double tos_attn_fwd_flops(int64_t B, int64_t H, int64_t N, int64_t d, int causal);

/* A static, human-readable name for a status code. */
const char* tos_status_string(tos_status status);

/* TOS_VERSION of the built library. */
int tos_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TOS_H */
