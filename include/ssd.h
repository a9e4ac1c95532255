/*
 * ssd.h -- libssd: the Mamba-2 SSD chunked scan on AMD Instinct MI355X (gfx950).
 *
 * The library computes, for every sequence and head h (group g = h / (H/G)):
 *
 *     delta_t = softplus(dt_t + dt_bias_h)            (optionally clamped)
 *     h_t     = exp(delta_t * A_h) * h_{t-1} + x_t (outer) B_t      (P x N state)
 *     y_t     = h_t . C_t + D_h * x_t
 *     out_t   = y_t * silu(z_t)                        (when z is given)
 *
 * Mamba-3-Lite "SSD Reference", section "Math: the recurrence both functions
 * implement" (recurrence and closed form) and section "_discretise" (the step
 * exp(softplus(dt) A)); the dt bias, groups, D skip, SiLU gate and initial /
 * final states are those of the Mamba-2 SSD stages timed in mamba PR 1012 and
 * cudnn-frontend PR 1133 ("optional skip/SiLU", "initial/final-state").
 *
 * It is evaluated chunkwise in the five stages vLLM PR 27299 ("Purpose")
 * names -- chunk cumsum, BMM, chunk state, state passing, chunk scan -- each
 * exported below, plus a forward call that runs them all.  The chunkwise
 * algebra is the SSD Reference's: sections "Chunking and the discretized
 * log-decay", "Intra-chunk outputs and per-chunk states", "Inter-chunk
 * propagation" and "Readout".
 *
 * Conventions shared by every call
 * --------------------------------
 * - Symbols: b batch, T tokens per sequence (total tokens when packed),
 *   H heads, P head dim, G groups, N state dim, C chunk size.
 * - Batch mode: b sequences of T tokens, chunk c of sequence i covers tokens
 *   [cC, min(cC + C, T)); logical chunk id j = i * ceil(T/C) + c.
 * - Packed (varlen) mode (problem.nseq > 0, batch == 1): sequence i owns tokens
 *   [cu[i], cu[i+1]) and is cut into chunks counted from its own first token,
 *   so no chunk straddles a sequence boundary and the state restarts at every
 *   sequence.  Logical chunk ids run sequence by sequence.  The chunk table is
 *   built on the device by ssd_varlen_chunk_meta.
 * - K = ssd_num_chunks(problem) logical chunks (an upper bound in packed mode;
 *   entries past the real count are never read or written).
 * - Tensors are strided views (ssd_tensor): strides are in ELEMENTS, the
 *   innermost dimension (P or N) must be contiguous, every row start must be
 *   16-byte aligned.  x, B, C may be views into one packed xBC buffer.
 * - Intermediates are caller-owned, contiguous, in these layouts:
 *     dA_cumsum  float32 (K, H, C): within-chunk inclusive cumsum of
 *                delta * A; positions past a short chunk's end repeat the
 *                value at its last token (their log-decay counts as 0).
 *     CB         float32 (K, G, C, C): CB[j,g,l,s] = C_l . B_s; only s <= l
 *                inside the chunk is defined, other entries are unspecified.
 *     states     state_dtype (K, H, P, N).
 * - Initial and final states are float32 (nseq or b, H, P, N), contiguous.
 * - Ownership: the caller owns every buffer.  The library allocates nothing,
 *   keeps no pointer after a call returns, never synchronises the host, and
 *   holds no global state; calls on different streams may run concurrently.
 *   Every device call is asynchronous on the stream it is given.
 * - Errors: arguments are validated on the host before anything is launched,
 *   so a call that returns an error has launched nothing (except SSD_ERR_HIP,
 *   returned when a launch itself fails).  ssd_last_error_message() names the
 *   offending argument (thread-local).
 * - Determinism: results are bitwise identical run to run.  The staged
 *   forward, the backward, the complex-A and the norm calls use no atomics.
 *   The fused forward uses none either: it hands states between its two
 *   launches through memory, and every sum has a fixed order.
 */
#ifndef LIBSSD_SSD_H
#define LIBSSD_SSD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssd_status {
  SSD_OK = 0,
  SSD_ERR_NULL = 1,        /* a required pointer is NULL */
  SSD_ERR_SHAPE = 2,       /* a dimension is out of range or inconsistent */
  SSD_ERR_DTYPE = 3,       /* a tensor has a dtype this call does not take */
  SSD_ERR_STRIDE = 4,      /* inner stride != 1 or a row is not 16-byte aligned */
  SSD_ERR_UNSUPPORTED = 5, /* valid request this build does not implement */
  SSD_ERR_WORKSPACE = 6,   /* workspace missing or too small */
  SSD_ERR_HIP = 7          /* a HIP launch failed; the message has HIP's text */
} ssd_status;

typedef enum ssd_dtype { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

typedef enum ssd_algo {
  SSD_ALGO_STAGED = 0, /* the five stage kernels in sequence */
  SSD_ALGO_FUSED = 1,  /* one pass over the inputs (range aggregates, then outputs) */
  SSD_ALGO_AUTO = 2    /* FUSED where it applies (bf16 x, B, C; dstate <= 128; with
                          input_dt, delta >= 0 by construction), STAGED otherwise;
                          its workspace size is the larger of the two */
} ssd_algo;

/* A strided tensor view.  Shape is implied by the argument's role. */
typedef struct ssd_tensor {
  void* data;          /* device pointer; NULL = optional argument absent */
  ssd_dtype dtype;
  int64_t stride[3];   /* outer strides in elements, outermost first */
} ssd_tensor;

typedef struct ssd_problem {
  int32_t batch;       /* b (must be 1 in packed mode) */
  int32_t seqlen;      /* T: tokens per sequence, or total packed tokens */
  int32_t nheads;      /* H */
  int32_t headdim;     /* P: multiple of 16, <= 256 */
  int32_t ngroups;     /* G: divides H */
  int32_t dstate;      /* N: multiple of 16, <= 256 */
  int32_t chunk_size;  /* C: 32, 64, 128 or 256 */
  int32_t nseq;        /* packed mode: number of sequences; 0 = batch mode */
  const int32_t* cu_seqlens; /* packed mode: device, nseq + 1 offsets, cu[0] = 0,
                                non-decreasing, cu[nseq] = seqlen */
  const int32_t* chunk_meta; /* packed mode, stage calls: device chunk table
                                written by ssd_varlen_chunk_meta */
  int32_t dt_softplus; /* 1: delta = softplus(dt + dt_bias); 0: delta = dt + dt_bias */
  int32_t dt_clamp;    /* 1: clamp delta to [dt_min, dt_max] */
  float dt_min, dt_max;
  ssd_dtype state_dtype; /* storage of the per-chunk states (F32 or BF16) */
  int32_t input_dt;    /* 1: the input term is delta_t x_t (outer) B_t, the way
                          Mamba-2 implementations discretise the input (not
                          written on the pages); 0: x_t (outer) B_t, the
                          recurrence as the SSD Reference writes it ("Math").
                          The skip D x_t uses the raw x either way. */
} ssd_problem;

/* ---------------------------------------------------------------- queries */

/* Validate a problem (host only, no HIP call).  Checks: positive dims,
 * H % G == 0, P and N multiples of 16 in [16, 256], C in {32, 64, 128, 256},
 * packed mode => batch == 1 and cu_seqlens != NULL.  On failure returns the
 * status and sets the message naming the dimension. */
ssd_status ssd_problem_check(const ssd_problem* p);

/* K: logical chunks (batch mode: b * ceil(T/C); packed: ceil(T/C) + nseq, an
 * upper bound on the real count).  Returns -1 for an invalid problem. */
int64_t ssd_num_chunks(const ssd_problem* p);

/* Number of int32 entries of the packed-mode chunk table:
 * 4 + 3*K + (nseq + 1).  Layout:
 *   [0] number of real chunks Kr, [1] nseq, [2] C, [3] K
 *   [4 + 3j + 0] sequence of chunk j (-1 for j >= Kr)
 *   [4 + 3j + 1] first token of chunk j (0 for j >= Kr)
 *   [4 + 3j + 2] tokens in chunk j, 1..C (0 for j >= Kr)
 *   [4 + 3K + i] first chunk of sequence i, i = 0..nseq ([nseq] = Kr)
 * Returns 0 for an invalid problem. */
size_t ssd_varlen_meta_len(const ssd_problem* p);

/* Bytes of workspace ssd_forward needs for `algo` (0 is a valid answer). */
ssd_status ssd_workspace_size(const ssd_problem* p, ssd_algo algo, size_t* bytes);

/* ---------------------------------------------------------------- a6 */

/* Build the packed-mode chunk table on the device from p->cu_seqlens (read
 * on the device only, so the call can be captured in a HIP graph).
 * meta: device int32, ssd_varlen_meta_len(p) entries, written entirely.
 * Sequence-aligned chunking per the SSD Reference "Padding rule" applied to
 * each packed sequence (vLLM PR 27299, continuous batching).  cu_seqlens
 * must be valid (checked by the host twin, not on the device). */
ssd_status ssd_varlen_chunk_meta(const ssd_problem* p, int32_t* meta, hipStream_t stream);

/* Host twin of ssd_varlen_chunk_meta: cu_host is host memory with nseq + 1
 * entries; validates it (cu[0] == 0, non-decreasing, cu[nseq] == seqlen) and
 * writes the same table to meta_host (meta_len entries). */
ssd_status ssd_varlen_chunk_meta_host(const ssd_problem* p, const int32_t* cu_host,
                                      int32_t* meta_host, size_t meta_len);

/* ---------------------------------------------------------------- a1 */

/* Chunk cumsum.  delta = softplus(dt + dt_bias) (or without softplus, and
 * clamped when asked), a = delta * A_h, dA_cumsum[j,h,l] = sum_{l' <= l} a
 * within chunk j.  SSD Reference "Chunking and the discretized log-decay"
 * (A_log = softplus(dt) A, A_cumsum = cumsum over the chunk).
 *   dt        (b, T, H) F32 or BF16, strides {batch, token, head} (any)
 *   A         float32 (H), device
 *   dt_bias   float32 (H), device, or NULL for no bias
 *   dA_cumsum float32 (K, H, C), written
 *   dt_out    float32 (K, H, C) or NULL: delta per position (0 past a chunk's end)
 */
ssd_status ssd_chunk_cumsum(const ssd_problem* p, ssd_tensor dt, const float* A,
                            const float* dt_bias, float* dA_cumsum, float* dt_out,
                            hipStream_t stream);

/* ---------------------------------------------------------------- a2 */

/* BMM: CB[j,g,l,s] = sum_n C[t0+l, g, n] B[t0+s, g, n] for s <= l < len_j.
 * SSD Reference "Algorithm and tensor-shape contract", step 4 (Cb = Cc Bc^T).
 *   C, B  (b, T, G, N), same dtype (F32 or BF16), strides {batch, token, group}
 *   CB    float32 (K, G, C, C), written (entries with s > l left unspecified)
 */
ssd_status ssd_bmm_chunk(const ssd_problem* p, ssd_tensor C, ssd_tensor B, float* CB,
                         hipStream_t stream);

/* ---------------------------------------------------------------- a3 */

/* Chunk state: each chunk's end state from a zero start,
 *   states[j,h,p,n] = sum_{s < len} exp(cs[last] - cs[s]) f_s x[t0+s,h,p] B[t0+s,g,n]
 * with f_s = delta_s when p->input_dt, else 1.  SSD Reference "Intra-chunk
 * outputs and per-chunk states" (states einsum with decay_states =
 * exp(A_cumsum[-1] - A_cumsum)).
 *   x         (b, T, H, P), F32 or BF16 (same dtype as B)
 *   B         (b, T, G, N)
 *   dA_cumsum float32 (K, H, C) from ssd_chunk_cumsum
 *   dt_chunk  float32 (K, H, C): delta per position, ssd_chunk_cumsum's dt_out;
 *             required when p->input_dt, otherwise ignored (may be NULL)
 *   states    (K, H, P, N) in p->state_dtype, written
 */
ssd_status ssd_chunk_state(const ssd_problem* p, ssd_tensor x, ssd_tensor B,
                           const float* dA_cumsum, const float* dt_chunk, void* states,
                           hipStream_t stream);

/* ---------------------------------------------------------------- a4 */

/* State passing, the sequential scan over chunks of every sequence:
 *   Hin[first] = initial_states[i] (or 0),  Hin[j+1] = exp(Lambda_j) Hin[j] + S_j,
 *   final_states[i] = exp(Lambda_last) Hin[last] + S_last   (= initial state if empty)
 * with Lambda_j = dA_cumsum[j, h, len_j - 1].  Equivalent to the SSD
 * Reference's decay_chunk[z,c] = exp(CD[z-1] - CD[c]) 1[z>c] plus the initial
 * state term exp(CD[z-1]) H_{-1} ("Inter-chunk propagation").
 *   states         (K, H, P, N) state_dtype: chunk states S_j from ssd_chunk_state
 *   dA_cumsum      float32 (K, H, C)
 *   initial_states float32 (nseq or b, H, P, N) or NULL (zero)
 *   states_out     (K, H, P, N) state_dtype: carry-in Hin[j]; may alias `states`
 *   final_states   float32 (nseq or b, H, P, N) or NULL
 * The recurrence runs in float32 registers; only stored copies are rounded.
 */
ssd_status ssd_state_passing(const ssd_problem* p, const void* states,
                             const float* dA_cumsum, const float* initial_states,
                             void* states_out, float* final_states, hipStream_t stream);

/* ---------------------------------------------------------------- a5 */

/* Chunk scan: the output of every position l < len_j of chunk j,
 *   y[l] = exp(cs[l]) C_l . Hin[j]                                    (Y_off)
 *        + sum_{s <= l} exp(cs[l] - cs[s]) CB[l,s] f_s x_s             (Y_diag)
 *        + D_h x_l ;      out = y * silu(z)  if z is given
 * (f_s = delta_s when p->input_dt, else 1)
 * SSD Reference "Intra-chunk outputs" (L = exp(segsum) masked to s <= l,
 * Y_diag) and "Readout" (Y_off = C . state . exp(A_cumsum), Y = Y_diag + Y_off);
 * gate as cudnn-frontend PR 1133 "optional skip/SiLU" (D added before gating).
 *   CB        float32 (K, G, C, C) from ssd_bmm_chunk
 *   x         (b, T, H, P); C (b, T, G, N); same dtype
 *   dA_cumsum float32 (K, H, C)
 *   dt_chunk  float32 (K, H, C) as for ssd_chunk_state (input_dt only)
 *   states_in (K, H, P, N) state_dtype: carry-in states from ssd_state_passing
 *   D         float32 (H) or NULL
 *   z         (b, T, H, P) same dtype as x, or data == NULL
 *   out       (b, T, H, P) F32 or BF16, written
 */
ssd_status ssd_chunk_scan(const ssd_problem* p, const float* CB, ssd_tensor x, ssd_tensor C,
                          const float* dA_cumsum, const float* dt_chunk,
                          const void* states_in, const float* D, ssd_tensor z,
                          ssd_tensor out, hipStream_t stream);

/* ---------------------------------------------------------------- forward */

typedef struct ssd_fwd_args {
  ssd_tensor x;               /* (b, T, H, P) */
  ssd_tensor B;               /* (b, T, G, N) */
  ssd_tensor C;               /* (b, T, G, N) */
  ssd_tensor dt;              /* (b, T, H) */
  const float* A;             /* (H) */
  const float* dt_bias;       /* (H) or NULL */
  const float* D;             /* (H) or NULL */
  ssd_tensor z;               /* (b, T, H, P) or data == NULL */
  const float* initial_states;/* (nseq or b, H, P, N) float32 or NULL */
  ssd_tensor out;             /* (b, T, H, P) F32 or BF16 */
  float* final_states;        /* (nseq or b, H, P, N) float32 or NULL */
} ssd_fwd_args;

/* The whole forward pass.  SSD_ALGO_STAGED runs chunk cumsum, BMM, chunk
 * state, state passing and chunk scan (vLLM PR 27299 "Purpose", the five
 * stages).  SSD_ALGO_FUSED computes the same result in one pass over the
 * inputs (the same page: the cumsum and C.B^T are recomputed per tile and the
 * state is handed between workgroups instead of storing the per-chunk
 * intermediates): a launch that sums each range of chunks into one state,
 * a small launch that turns those into each range's carry-in, then the
 * output launch, which walks each range's chunks from its carry-in (plus a
 * small chunk-table kernel in packed mode); it always works on
 * 128-token chunks (the result does not depend on the chunk length), takes
 * bf16 x, B, C (and z) and dstate <= 128, and returns SSD_ERR_UNSUPPORTED
 * otherwise; it stores no per-chunk states (the carried state stays in
 * float32 registers and hand-off buffers), so p->state_dtype does not apply
 * to it; with input_dt it also needs delta > 0 by construction (softplus,
 * or a clamp with dt_min >= 0), since it folds log2(delta) into the decay
 * exponent.  initial_states and final_states must be 16-byte aligned for
 * it, and 127 token strides plus one row of each token tensor must stay
 * below 2 GiB (it addresses a chunk's rows as 32-bit offsets; AUTO takes
 * STAGED otherwise).  Its results are bit-identical run to run for a given problem shape;
 * two different shapes of one computation (e.g. a sequence split in two and
 * resumed from the final state) agree to fp32 rounding of the states.
 * In packed mode the chunk table is built inside the workspace.  workspace:
 * device memory of at least ssd_workspace_size(p, algo) bytes, 256-byte
 * aligned, owned by the caller, contents need not be initialised; it must not
 * be shared by calls that overlap in time.  The fused path hands the state
 * from one range of chunks to the next through the workspace between two
 * launches, so no workgroup ever waits for another. */
ssd_status ssd_forward(const ssd_problem* p, ssd_algo algo, const ssd_fwd_args* a,
                       void* workspace, size_t ws_bytes, hipStream_t stream);

/* The gated RMSNorm that follows the scan in the Mamba-2 mixer (mamba PR 1012,
 * "Summary": the gated-LayerNorm after the SSD; its formula is not on the
 * pages: Mamba-2's gated RMSNorm, gate first), fused into the forward:
 *     g = y silu(z)  (g = y when z is absent),   y = the scan output,
 *     out = g / sqrt(mean_group(g^2) + eps) * weight
 * over contiguous groups of group_size channels of each token's flattened
 * (H, P) axis, as ssd_gated_rmsnorm_fwd computes it from y and z. */
typedef struct ssd_norm_args {
  const float* weight;   /* (H * P) float32, 16-byte aligned */
  int32_t group_size;    /* a multiple of 64 dividing H * P, at most 256 groups per token */
  float eps;             /* >= 0 */
  float* rstd;           /* (b * T, H * P / group_size) float32, or NULL:
                            1 / sqrt(mean_group(g^2) + eps) per token and group */
} ssd_norm_args;

/* Bytes of workspace ssd_forward_gated_norm needs. */
ssd_status ssd_forward_gated_norm_workspace_size(const ssd_problem* p, const ssd_norm_args* n,
                                                 size_t* bytes);

/* The fused forward (SSD_ALGO_FUSED, same inputs and restrictions) with the
 * gated RMSNorm in its epilogue: the output launch gates its outputs, writes
 * g to `out` and, per token and 64-channel block, the sum of g^2 (from the
 * fp32 values); a last pass scales `out` in place by the group factor and the
 * weight.  Against ssd_forward followed by ssd_gated_rmsnorm_fwd this reads
 * neither y nor z a second time.  Needs headdim a multiple of 64 (the
 * channel blocks are the fused pass's 64-row units); returns
 * SSD_ERR_UNSUPPORTED otherwise.  With a bf16 `out`, g is rounded to bf16
 * once before the scaling (one more rounding than the two-call path's y). */
ssd_status ssd_forward_gated_norm(const ssd_problem* p, const ssd_fwd_args* a,
                                  const ssd_norm_args* n, void* workspace, size_t ws_bytes,
                                  hipStream_t stream);

/* Bytes of the device array behind ssd_forward_fused_static (one per GPU). */
#define SSD_FUSED_STATIC_SCRATCH_BYTES (32u << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * computation as ssd_forward(p, SSD_ALGO_FUSED, a, ...) with the fused pass's
 * scratch (hand-off aggregates, packed-mode chunk table)
 * in a file-scope device array of SSD_FUSED_STATIC_SCRATCH_BYTES bytes, one per
 * GPU, held until the process ends.  It calls no allocator.  The caller still
 * passes inputs and outputs.  A problem whose fused workspace
 * (ssd_workspace_size(p, SSD_ALGO_FUSED)) exceeds the array returns
 * SSD_ERR_WORKSPACE.  Every call on one GPU uses that GPU's one array (the
 * look-up of its address is the only set-up, once per device): calls that
 * overlap in time on one GPU, on any streams, race and must not be made. */
ssd_status ssd_forward_fused_static(const ssd_problem* p, const ssd_fwd_args* a,
                                    hipStream_t stream);

/* ---------------------------------------------------------------- backward */

typedef struct ssd_bwd_args {
  /* the forward's inputs, as in ssd_fwd_args */
  ssd_tensor x, B, C, dt;
  const float* A;
  const float* dt_bias;       /* (H) or NULL */
  const float* D;             /* (H) or NULL */
  ssd_tensor z;               /* (b, T, H, P) or data == NULL */
  const float* initial_states;/* (nseq or b, H, P, N) float32 or NULL (zero) */
  /* incoming gradients */
  ssd_tensor dout;            /* (b, T, H, P) F32 or BF16: gradient of out */
  const float* dfinal_states; /* (nseq or b, H, P, N) float32 or NULL (zero) */
  /* gradients, written; all float32 */
  ssd_tensor dx;              /* (b, T, H, P) */
  ssd_tensor dB, dC;          /* (b, T, G, N), summed over the heads of each group */
  ssd_tensor ddt;             /* (b, T, H): gradient w.r.t. the raw dt (0 where clamped) */
  ssd_tensor dz;              /* (b, T, H, P); required when z is given */
  float* dA;                  /* (H) */
  float* ddt_bias;            /* (H): ddt summed over all tokens */
  float* dD;                  /* (H) or NULL (written only when D is given) */
  float* dinitial_states;     /* (nseq or b, H, P, N) or NULL */
} ssd_bwd_args;

/* Bytes of workspace ssd_backward needs. */
ssd_status ssd_backward_workspace_size(const ssd_problem* p, size_t* bytes);

/* The gradient of L = sum(dout * out) + sum(dfinal_states * final_states)
 * with respect to every input of ssd_forward (the backward stages timed in
 * mamba PR 1012 "Measurements"; SSD Reference section 6 "The autograd
 * backward contract": gradients of every input, exact for the forward).
 * The adjoint of the recurrence, dL/dh_t = exp(delta_{t+1} A) dL/dh_{t+1} +
 * dy_t (outer) C_t, is itself an SSD scan run backwards in time; the call
 * runs the staged kernels on operands it prepares: the forward recompute and
 * the adjoint scan (read with B for dx) in full, then two chunk scans that
 * reuse their chunk states transposed (the adjoint read with x for dB, the
 * forward state read with dy for dC).  The step-size gradient of a token is
 * the sum, over the later tokens of its chunk, of dL/dcs_l (cs the chunk's
 * cumulative log-decay): row minus column sums of the strictly lower triangle
 * of exp(cs_l - cs_s) (C_l . B_s) (dy_l . x_s), plus the terms of the states
 * entering and leaving the chunk; no two terms of it cancel, so it stays
 * accurate under strong decay.  States and accumulations are fp32, sums of
 * many terms fp64; products are fp32 for fp32 inputs and, for bf16 inputs,
 * keep ~16 significant bits of each operand (bf16 hi + lo), well inside the
 * bf16 tolerance.  Packed mode is
 * supported (each sequence runs backwards on its own).  initial_states,
 * dfinal_states and dinitial_states must be 16-byte aligned.
 * Results are bit-identical run to run (no atomics, fixed sum orders).
 * workspace: at least ssd_backward_workspace_size(p) bytes, 256-byte
 * aligned, contents need not be initialised; calls that overlap in time must
 * not share it. */
ssd_status ssd_backward(const ssd_problem* p, const ssd_bwd_args* a, void* workspace,
                        size_t ws_bytes, hipStream_t stream);

/* Bytes of workspace ssd_backward_ex needs for `algo` with inputs x, B, C of
 * `in_dtype` (AUTO resolves exactly as the call does).  The per-chunk path
 * (FUSED) keeps two fp32 states per chunk and head (the state entering the
 * chunk and its gradient); it takes the heads in passes whose two state
 * buffers hold at most 256 MiB by default: 275 MB at Nemotron-Nano size (8192
 * tokens, 64 heads x 64, d_state 128: one pass), 342 MB at 65536 tokens x 80
 * heads (ten passes of 8 heads), against ~2.2 GB for STAGED at Nemotron-Nano
 * size. */
ssd_status ssd_backward_ex_workspace_size(const ssd_problem* p, ssd_algo algo,
                                          ssd_dtype in_dtype, size_t* bytes);

/* ssd_backward with a choice of algorithm: the same gradients, arguments and
 * conventions.
 *   SSD_ALGO_STAGED  the staged backward above (every supported problem);
 *   SSD_ALGO_FUSED   the per-chunk backward: two state passes at 128-token
 *                    chunks give the state entering every chunk (forward
 *                    recompute) and the gradient of the state leaving it (each
 *                    chunk's own gradient of its entering state, then the
 *                    state passing run backwards); then one kernel per (chunk,
 *                    head) forms y
 *                    (for dz), dx and the step-size gradient, and one per
 *                    (chunk, group, 64 state columns) forms dB and dC summed
 *                    over the group's heads (the chunkwise forward of the SSD
 *                    Reference, "Intra-chunk outputs and per-chunk states" and
 *                    "Inter-chunk propagation", differentiated factor by
 *                    factor).  Takes bf16 x, B, C, headdim 64 and dstate <= 128
 *                    (a multiple of 8), with at least one token, and 127
 *                    token strides plus one row of each token tensor below
 *                    2 GiB; returns SSD_ERR_UNSUPPORTED otherwise.  Same precision design
 *                    (bf16 hi + lo operands, fp32 states and accumulation, fp64
 *                    cumsum and step-size sums) and bit-identical results run to
 *                    run.  In packed mode, tokens past cu_seqlens[nseq] belong
 *                    to no sequence and get no gradient written.
 *   SSD_ALGO_AUTO    FUSED where it applies, STAGED otherwise.
 * Workspace: 256-byte aligned, contents need not be initialised, not shared by
 * calls that overlap in time.  STAGED needs its full size.  FUSED takes any
 * size down to that of its smallest head pass and then uses the largest
 * passes that fit (equal sizes; whole groups of heads, or multiples of eight
 * heads of one group when the group's heads are a multiple of eight: their dB
 * and dC are then summed over the passes in the same order as in one pass,
 * so every size gives the same bits); below that, SSD_ERR_WORKSPACE. */
ssd_status ssd_backward_ex(const ssd_problem* p, const ssd_bwd_args* a, ssd_algo algo,
                           void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- complex A */

/* The complex-A SSD scan of Mamba-3-Lite (SSD Reference, "Math: the recurrence
 * both functions implement", with "_discretise": abar_t = exp(softplus(dt_t) A_h)
 * for a complex per-head A_h and a real step dt_t):
 *
 *     h_t = abar_t h_{t-1} + B_t (outer) x_t,     y_t = sum_n C_t[n] h_t[n, :]
 *
 * x (P), B and C (N) are complex and per head (SSD Reference, "Shape contract":
 * B_t, C_t are (B, T, H, N)); nothing is conjugated.  There is no dt bias, no
 * D skip and no gate.  Evaluated chunkwise as the page's production scan does
 * ("Chunking and the discretized log-decay", "Intra-chunk outputs and
 * per-chunk states", "Inter-chunk propagation" with decay_chunk[z, c] =
 * exp(CD[z-1] - CD[c]) 1[z > c] and the init term exp(CD[z-1]) H_{-1},
 * "Readout"), batch mode only.
 *
 * Complex tensors hold interleaved (re, im) float32 pairs (complex64); their
 * ssd_tensor dtype is SSD_F32 and their strides count COMPLEX elements.
 */
typedef struct ssd_complex_problem {
  int32_t batch;       /* b >= 1 (1 in packed mode) */
  int32_t seqlen;      /* T >= 0: tokens per sequence, or total packed tokens */
  int32_t nheads;      /* H >= 1, (batch or nseq) * nheads <= 65535 */
  int32_t headdim;     /* P (the page's D): multiple of 16, <= 128 */
  int32_t dstate;      /* N: multiple of 16, <= 128 */
  int32_t chunk_size;  /* C: 32, 64, 128 or 256 (the result does not depend on it) */
  int32_t nseq;        /* packed mode: number of sequences; 0 = batch mode */
  const int32_t* cu_seqlens; /* packed mode: device, nseq + 1 offsets, cu[0] = 0,
                                non-decreasing, cu[nseq] = seqlen; each sequence is
                                chunked from its own first token and starts from its
                                initial state (or zero), as in the real scan's packed
                                mode.  Only ssd_complex_forward takes packed problems. */
} ssd_complex_problem;

/* Packed mode drops the batch axis of every token tensor ((T, H, P) etc., the
 * batch stride ignored) and indexes initial and final states by sequence. */
typedef struct ssd_complex_fwd_args {
  ssd_tensor x;        /* (b, T, H, P) complex; rows 16-byte aligned */
  ssd_tensor B;        /* (b, T, H, N) complex; rows 16-byte aligned */
  ssd_tensor C;        /* (b, T, H, N) complex; rows 16-byte aligned */
  ssd_tensor dt;       /* (b, T, H) float32 real, raw (softplus is applied) */
  const float* A;      /* (H) complex: 2H floats (re, im), device */
  const float* initial_states; /* (b, H, P, N) complex, contiguous, 16-byte
                                  aligned, or NULL (zero); the page's (D, N)
                                  layout ("Shape contract") */
  ssd_tensor out;      /* (b, T, H, P): out_complex = 0: float32, the real part
                          of y (the page's chunkwise return contract); strides
                          in floats.  out_complex = 1: complex y, strides in
                          complex elements */
  int32_t out_complex;
  float* final_states; /* (b, H, P, N) complex, contiguous, 16-byte aligned, or NULL */
} ssd_complex_fwd_args;

/* Validate a complex problem (host only).  On failure sets the message. */
ssd_status ssd_complex_problem_check(const ssd_complex_problem* p);

/* Bytes of workspace ssd_complex_forward needs: the per-chunk complex states
 * (K * H * P * N * 8 bytes, K = b * ceil(T/C), or ceil(T/C) + nseq when packed),
 * each chunk's step sum and, when packed, the chunk table. */
ssd_status ssd_complex_workspace_size(const ssd_complex_problem* p, size_t* bytes);

/* The forward pass: three kernels on `stream` -- every chunk's end state from a
 * zero start (SSD Reference "Algorithm and tensor-shape contract", step 6:
 * state = Xc^T (decay_states * Bc)), the sequential pass over chunks
 * ("Inter-chunk propagation"), and the output of every chunk (steps 3-5, Y_diag
 * = (L * Cb) Xc, plus "Readout": Y_off = C . state . exp(A_cumsum)).  Products
 * are fp32 matrix instructions, accumulation fp32.  workspace: at least
 * ssd_complex_workspace_size bytes, 256-byte aligned, caller-owned, contents
 * need not be initialised, not shared by calls that overlap in time.  Results
 * are bit-identical run to run. */
ssd_status ssd_complex_forward(const ssd_complex_problem* p, const ssd_complex_fwd_args* a,
                               void* workspace, size_t ws_bytes, hipStream_t stream);

/* The three stages ssd_complex_forward runs, for callers that keep the
 * intermediates (batch mode only: a packed problem returns SSD_ERR_UNSUPPORTED).
 * nc = ceil(T / C); chunk j = (batch row) * nc + c.
 *   states        float32 complex (b * nc, H, P, N), 16-byte aligned: the page's
 *                 internal states (B, n_chunks, H, D, N) ("Shape contract")
 *   chunk_dt_sum  float32 (H, b * nc), 16-byte aligned: sum of softplus(dt) over
 *                 each chunk's tokens (the chunk's total log-decay is this times A)
 *
 * ssd_complex_chunk_state: states[j] = sum_s exp(cs_last - cs_s) x_s (outer) B_s,
 * each chunk from a zero start (SSD Reference "Algorithm and tensor-shape
 * contract", step 6, decay_states = exp(A_cumsum[-1] - A_cumsum)); writes
 * chunk_dt_sum too. */
ssd_status ssd_complex_chunk_state(const ssd_complex_problem* p, ssd_tensor x, ssd_tensor B,
                                   ssd_tensor dt, const float* A, float* states,
                                   float* chunk_dt_sum, hipStream_t stream);

/* ssd_complex_state_passing: in place over `states`, the carry-in state of every
 * chunk, Hin[0] = initial_states (or 0), Hin[c+1] = exp(Lambda_c) Hin[c] + S_c
 * with Lambda_c = chunk_dt_sum * A; final_states = the state after the last
 * chunk (= initial_states when T = 0).  The SSD Reference's "Inter-chunk
 * propagation": decay_chunk[z, c] = exp(CD[z-1] - CD[c]) 1[z > c] plus the init
 * term exp(CD[z-1]) H_{-1}, evaluated as a sequential scan. */
ssd_status ssd_complex_state_passing(const ssd_complex_problem* p, const float* A,
                                     const float* chunk_dt_sum, const float* initial_states,
                                     float* states, float* final_states, hipStream_t stream);

/* ssd_complex_chunk_scan: the output of every token from the carry-in states,
 * y_l = sum_{s <= l} exp(cs_l - cs_s) (C_l . B_s) x_s + exp(cs_l) C_l . Hin
 * (SSD Reference "Algorithm and tensor-shape contract", steps 3-5, and
 * "Readout"); out as in ssd_complex_fwd_args. */
ssd_status ssd_complex_chunk_scan(const ssd_complex_problem* p, ssd_tensor x, ssd_tensor B,
                                  ssd_tensor C, ssd_tensor dt, const float* A,
                                  const float* states_in, ssd_tensor out, int32_t out_complex,
                                  hipStream_t stream);

/* ---------------------------------------------------------------- gated RMSNorm */

/* The normalisation that follows the scan in the Mamba-2 mixer: the
 * "gated-LayerNorm" of mamba PR 1012 ("Summary"; its backward is the
 * layer_norm_bwd stage of "Measurements").  The pages do not write its formula;
 * this is Mamba-2's gated RMSNorm with the gate applied before the norm, over
 * contiguous groups of group_size channels of each token's flattened (H, P) axis:
 *
 *     g = y silu(z)   (g = y when z is absent)
 *     out = g / sqrt(mean_group(g^2) + eps) * weight
 *
 * y is typically the ungated scan output (ssd_forward with z absent).  It is a
 * separate pass because a group spans several heads while the scan's
 * workgroups each own one head.  Tokens: (b, T, H, P) strided views as for the
 * scan (innermost contiguous, rows 16-byte aligned). */
typedef struct ssd_norm_problem {
  int32_t batch;       /* b >= 1 */
  int32_t seqlen;      /* T >= 0 */
  int32_t nheads;      /* H >= 1 */
  int32_t headdim;     /* P: a multiple of 8 */
  int32_t group_size;  /* divides H * P; a power of two in [8, 512] or a multiple of 512 */
  float eps;           /* >= 0 */
} ssd_norm_problem;

/* Forward.  y, z: F32 or BF16, same dtype (z may be absent); weight: float32
 * (H * P), 16-byte aligned; out: F32 or BF16; rstd: float32 (b * T, H * P /
 * group_size) or NULL: 1 / sqrt(mean_group(g^2) + eps) per token and group. */
ssd_status ssd_gated_rmsnorm_fwd(const ssd_norm_problem* p, ssd_tensor y, ssd_tensor z,
                                 const float* weight, ssd_tensor out, float* rstd,
                                 hipStream_t stream);

/* Bytes of workspace ssd_gated_rmsnorm_bwd needs. */
ssd_status ssd_gated_rmsnorm_bwd_workspace_size(const ssd_norm_problem* p, size_t* bytes);

/* Gradient of sum(dout * out) with respect to y, z and weight.  dout has y's
 * dtype; dy and dz are float32 (dz required when z is given); dweight: float32
 * (H * P), written (summed over all tokens in a fixed order: bit-identical run to
 * run).  workspace: at least ssd_gated_rmsnorm_bwd_workspace_size bytes, 256-byte
 * aligned, caller-owned, contents need not be initialised. */
ssd_status ssd_gated_rmsnorm_bwd(const ssd_norm_problem* p, ssd_tensor y, ssd_tensor z,
                                 const float* weight, ssd_tensor dout, ssd_tensor dy,
                                 ssd_tensor dz, float* dweight, void* workspace,
                                 size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- errors */

const char* ssd_status_string(ssd_status s);
/* Message of the last failing call on this thread ("" if none). */
const char* ssd_last_error_message(void);
/* Library version string. */
const char* ssd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBSSD_SSD_H */
