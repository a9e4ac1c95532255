// kernels.hpp -- host-side launchers of the libssd kernels (internal interface
// between the C ABI in api.cpp and the .hip translation units).  Every launcher
// assumes its arguments were validated by api.cpp and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace ssd {

enum DType { DT_F32 = 0, DT_BF16 = 1 };

hipError_t launch_varlen_meta(const Geo& g, const int32_t* cu_seqlens, int32_t* meta,
                              hipStream_t s);

hipError_t launch_chunk_cumsum(const Geo& g, TArg dt, int dt_dtype, const float* A,
                               const float* dt_bias, int softplus, int clamp, float dt_min,
                               float dt_max, float* cs, float* dt_out, hipStream_t s);

hipError_t launch_bmm_chunk(const Geo& g, TArg C, TArg B, int in_dtype, float* CB,
                            hipStream_t s);

// dtc: step size per position (K, H, C) when it scales the input term, or NULL
hipError_t launch_chunk_state(const Geo& g, TArg x, TArg B, int in_dtype, const float* cs,
                              const float* dtc, void* states, int st_dtype, hipStream_t s);

hipError_t launch_state_passing(const Geo& g, const void* states, int st_dtype,
                                const float* cs, const float* h0, void* states_out,
                                float* hfinal, hipStream_t s);

// Two independent scans over the chunks, side by side in one launch: the state
// passing over fp32 states (in place, from h0, no final state), and its adjoint,
// chunks last to first, in place on adj (fp32 (K, H, P, N)): U_j (the gradient
// chunk j's tokens send to its entering state) becomes dHout_j (the gradient of
// the state leaving chunk j through later tokens) from dfinal; dh0 (nseq, H, P,
// N) or NULL receives the initial state's gradient.
hipError_t launch_state_passing_pair(const Geo& g, float* states, const float* cs,
                                     const float* h0, float* adj, const float* dfinal, float* dh0,
                                     hipStream_t s);

// yoff (NULL to skip): also writes the inter-chunk part of
// the output, exp(cs_l) C_l . h_in, before the skip and the gate, as (tokens,
// H, P) fp32 on the packed axis.  st_trans (fp32 inputs only): the carry-in
// states are stored (K, H, N, P).  x_div (fp32 inputs only): head h reads row
// h / x_div of x.  split (fp32 inputs only): operands split into bf16 hi + lo,
// three bf16 matrix instructions per product (~16 significant bits per
// operand) instead of fp32 matrix instructions.
hipError_t launch_chunk_scan(const Geo& g, const float* CB, TArg x, TArg C, int in_dtype,
                             const float* cs, const float* dtc, const void* states, int st_dtype,
                             const float* D, TArg z, TArg out, int out_dtype, hipStream_t s,
                             float* yoff = nullptr, int st_trans = 0, int x_div = 1,
                             int split = 0);

// ---- fused forward (fused_fwd.hip)
constexpr int kFusedChunk = 128;             // internal chunk length of the fused pass
constexpr int kFusedTargetWorkgroups = 512;  // (unit, range) workgroups aimed for
// Work decomposition of the fused pass: P slabs of 64 rows per head, units =
// heads x slabs, n-tiles of the d_state capacity, chunks per range, ranges.
struct FusedPlan {
  int PS, U, NT, R, nr;
};
FusedPlan fused_plan(int64_t K, int H, int P, int N);

struct FusedLaunch {
  Geo g;                   // 128-token chunk geometry (meta = the fused chunk table)
  const int32_t* cu;       // cu_seqlens of a packed batch, NULL in batch mode
  int32_t* meta;           // chunk table to build (packed batch only)
  TArg x, B, C, dt, z, out;
  int dt_dtype, out_dtype;
  const float* A;
  const float* dt_bias;
  const float* D;
  const float* h0;
  float* hfinal;
  int softplus, clamp, input_dt;
  float dt_min, dt_max;
  FusedPlan plan;
  float* edec;             // nr * U
  float* agg;              // nr * U * 64 * 16 * NT
  float* psum = nullptr;   // gated RMSNorm fused in: ntok * U partial sums of g^2
  unsigned long long* trace = nullptr;  // SSD_FUSED_TRACE builds: kFusedTraceSlots per item
};
// Phase timestamps per (unit, range) item in SSD_FUSED_TRACE builds: [0] and
// [1] the aggregate launch's start and end for the item; the output launch's
// [2] start, [3] carry-in loaded; for chunks k < 4 five stamps [4 + 5k ..
// 8 + 5k] after its phases A (carry-in to LDS), B (Y_off), C (x and B to
// LDS), D (state, C.B^T, Y_diag) and E (gate, store); for chunks 4 <= k < 10
// the end of the chunk at [20 + k]; for the aggregate launch's first four
// chunk steps k, six stamps [32 + 6k .. 37 + 6k]: after its first barrier, the
// staging of x and B, the issue of the next loads, the second barrier, the
// decay weights and the products' issue; [slots - 2] end and [slots - 1] the
// XCD the item ran on.
constexpr int kFusedTraceSlots = 64;

// Up to four launches: the chunk table / empty sequences (packed mode or no
// tokens), the range aggregates (more than one range), their carry scan (more
// than two ranges), the outputs.
hipError_t launch_fused_fwd(const FusedLaunch& f, hipStream_t s);

// ---- backward (bwd.hip): tokens on the packed axis, ntok = b * T (batch) or
// T (packed, cu != NULL); scratch tensors are contiguous fp32 (ntok, rows, width)
struct BwdGeo {
  int ntok, T, nseq, H, P, G, N, hpg;
  const int32_t* cu;
};
hipError_t launch_bwd_gather(const BwdGeo& q, TArg src, int dtype, int R, int W, int rep,
                             int reverse, float* dst, hipStream_t s);
hipError_t launch_bwd_gate(const BwdGeo& q, TArg dout, int dout_dtype, TArg z, int z_dtype,
                           const float* y, float* dy, float* dy_rev, TArg dz, hipStream_t s);
hipError_t launch_bwd_steps(const BwdGeo& q, TArg dt, int dt_dtype, const float* A,
                            const float* dt_bias, int softplus, int clamp, float dt_min,
                            float dt_max, float* delta, float* gd, float* dt_rev, hipStream_t s);
hipError_t launch_bwd_tokens(const BwdGeo& q, TArg x, int x_dtype, const float* D,
                             const float* dy, const float* gx_rev, const float* delta, TArg dx,
                             float* dyx, float* xg, hipStream_t s);
hipError_t launch_bwd_group_sums(const BwdGeo& q, const float* gb_rev, const float* gc,
                                 const float* delta, TArg dB, TArg dC, hipStream_t s);
// the mirrored scans' chunk table (and, in batch mode, cu = {0, T, 2T, ..})
hipError_t launch_bwd_mirror_meta(const BwdGeo& q, int C, int K, int32_t* meta, int32_t* cu_out,
                                 hipStream_t s);
// step-size gradients per forward chunk (gf: the forward chunk geometry);
// part: 3 doubles per (chunk, head)
hipError_t launch_bwd_step_grads(const BwdGeo& q, const Geo& gf, const float* CB,
                                 const float* DX, const float* yo_f, const float* yo_r,
                                 const float* xf, const float* dy,
                                 const float* dyx, const float* delta, const float* gd,
                                 const float* A, const float* fwd_st, const float* mir_st,
                                 const float* gfirst, const float* dfinal, const float* xg,
                                 TArg ddt, double* part, float* dA, float* ddt_bias, float* dD,
                                 float* dh0, hipStream_t s);

// per head: dA, ddt_bias, dD from the chunks' shares in chunk order, and dh0 =
// G_first for sequences without tokens
hipError_t launch_bwd_step_heads(const BwdGeo& q, int K, const double* part,
                                 const float* gfirst, float* dA, float* ddt_bias, float* dD,
                                 float* dh0, hipStream_t s);

// ---- per-chunk backward (bwd_chunk.hip): 128-token chunks, bf16 x, B, C,
// headdim 64, d_state <= 128 (a multiple of 8)
constexpr int kBwdChunk = 128;
constexpr int kBwdHeadsPerSplit = 8;  // heads of a group per dB/dC workgroup
int bwd_chunk_splits(int hpg);        // head splits of a group (partials when > 1)
struct BwdChunkLaunch {
  Geo g;                    // chunk geometry at 128 tokens (meta: its chunk table)
  int ntok;
  TArg x, B, C, z, dout, dx, dz, dB, dC, ddt;
  int dout_dtype;
  const float* A;
  const float* D;
  const float* delta;       // (ntok, H)
  const float* gd;          // (ntok, H)
  const float* cs;          // (K, H, 128) the forward's chunk cumsum
  const float* hin;         // (K, H, P, N) forward carry-in states
  float* adj;               // (K, H, P, N): U_j, then (after the reverse state
                            // passing) dS_j, the gradient of the state leaving chunk j
  double* part;             // (K, H, 3)
  int input_dt;
  float* pdb;               // (splits, ntok, G, N) when bwd_chunk_splits(hpg) > 1
  float* pdc;               // or `partials`
  int partials;             // dB, dC through the split partials even with one split
                            // (a pass over part of a group's heads)
  int accumulate;           // add the pass's sum to what dB and dC hold (a later
                            // pass over the same group), in split order
};
// U_j = sum_l exp(cs_l) dy_l (outer) C_l per (chunk, head) into adj
hipError_t launch_bwd_adj_state(const BwdChunkLaunch& l, hipStream_t s);
// dz, dx, ddt, the per-chunk shares of dA, ddt_bias, dD; then dB, dC
hipError_t launch_bwd_chunk(const BwdChunkLaunch& l, hipStream_t s);

// ---- complex-A forward (complex_fwd.hip): per-head complex B, C (g.G = g.H),
// batch or packed mode (g.meta); x, B, C, out (complex) strides in complex elements,
// dt and out (real) in floats.  states: K * H * P * N complex; lam: H * K floats (each
// chunk's step sum).
hipError_t launch_cx_chunk_state(const Geo& g, TArg x, TArg B, TArg dt, const float* A,
                                 float* states, float* lam, hipStream_t s);
// in place: the chunk states become the carry-in states
hipError_t launch_cx_state_pass(const Geo& g, const float* A, const float* lam,
                                const float* h0, float* states, float* hfinal, hipStream_t s);
hipError_t launch_cx_chunk_scan(const Geo& g, TArg x, TArg B, TArg Cm, TArg dt,
                                const float* A, const float* states, TArg out, int out_complex,
                                hipStream_t s);

// ---- gated RMSNorm after the scan (gated_norm.hip); tokens on the packed axis
// ntok = b * T, T tokens per batch row; groups of gs channels of the (H, P) axis
struct NormGeo {
  int ntok, T, H, P, gs;
  float eps;
};
int norm_tiles(const NormGeo& g);  // rows of weight-gradient partials
hipError_t launch_norm_fwd(const NormGeo& g, TArg y, TArg z, int in_dtype, const float* w,
                           TArg out, int out_dtype, float* rstd, hipStream_t s);
// In place: out = g r weight, g the gated scan output already in `out`, r from
// psum (ntok x (H P / 64) sums of g^2 per 64-channel block).  gs a multiple of
// 64, H P / gs <= kNormFinishGroups.
constexpr int kNormFinishGroups = 256;
hipError_t launch_norm_finish(const NormGeo& g, const float* psum, const float* w, TArg out,
                              int out_dtype, float* rstd, hipStream_t s);
// part: norm_tiles * H * P floats; stats: ntok * (H P / gs) float2 (gs > 512 only)
hipError_t launch_norm_bwd(const NormGeo& g, TArg y, TArg z, int in_dtype, const float* w,
                           TArg dout, TArg dy, TArg dz, float* dw, float* part, float2* stats,
                           hipStream_t s);

}  // namespace ssd
