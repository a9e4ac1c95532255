// api.cpp -- the libssd C ABI: argument validation, workspace layout and the
// launch sequence of each call.  Every check runs on the host before anything
// is enqueued, so a call that fails validation has launched nothing.  No call
// allocates, synchronises or keeps pointers; all state lives in the arguments.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cmath>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "ssd.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_msg;

ssd_status fail(ssd_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_msg = buf;
  return s;
}

ssd_status ok() {
  g_msg.clear();
  return SSD_OK;
}

ssd_status hip_fail(hipError_t e, const char* where) {
  return fail(SSD_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

size_t dsize(ssd_dtype d) { return d == SSD_BF16 ? 2 : 4; }
int dcode(ssd_dtype d) { return d == SSD_BF16 ? ssd::DT_BF16 : ssd::DT_F32; }
bool valid_dtype(ssd_dtype d) { return d == SSD_F32 || d == SSD_BF16; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t num_chunks(const ssd_problem* p) {
  const int64_t nc = cdiv(p->seqlen, p->chunk_size);
  if (p->nseq > 0) return nc + p->nseq;
  return (int64_t)p->batch * nc;
}

ssd_status check_problem(const ssd_problem* p) {
  if (!p) return fail(SSD_ERR_NULL, "problem is NULL");
  if (p->batch < 1) return fail(SSD_ERR_SHAPE, "batch = %d must be >= 1", p->batch);
  if (p->seqlen < 0) return fail(SSD_ERR_SHAPE, "seqlen = %d must be >= 0", p->seqlen);
  if (p->nheads < 1) return fail(SSD_ERR_SHAPE, "nheads = %d must be >= 1", p->nheads);
  if (p->ngroups < 1) return fail(SSD_ERR_SHAPE, "ngroups = %d must be >= 1", p->ngroups);
  if (p->nheads % p->ngroups != 0)
    return fail(SSD_ERR_SHAPE, "nheads = %d is not a multiple of ngroups = %d", p->nheads,
                p->ngroups);
  if (p->headdim < 16 || p->headdim > 256 || p->headdim % 16 != 0)
    return fail(SSD_ERR_UNSUPPORTED, "headdim = %d: must be a multiple of 16 in [16, 256]",
                p->headdim);
  if (p->dstate < 16 || p->dstate > 256 || p->dstate % 16 != 0)
    return fail(SSD_ERR_UNSUPPORTED, "dstate = %d: must be a multiple of 16 in [16, 256]",
                p->dstate);
  const int C = p->chunk_size;
  if (C != 32 && C != 64 && C != 128 && C != 256)
    return fail(SSD_ERR_UNSUPPORTED, "chunk_size = %d: must be 32, 64, 128 or 256", C);
  if (p->nseq < 0) return fail(SSD_ERR_SHAPE, "nseq = %d must be >= 0", p->nseq);
  if (p->nseq > 0) {
    if (p->batch != 1)
      return fail(SSD_ERR_SHAPE, "packed mode (nseq = %d) requires batch == 1, got %d", p->nseq,
                  p->batch);
    if (!p->cu_seqlens) return fail(SSD_ERR_NULL, "packed mode requires cu_seqlens");
  }
  if (!valid_dtype(p->state_dtype)) return fail(SSD_ERR_DTYPE, "state_dtype is not F32 or BF16");
  if (p->dt_clamp && !(p->dt_min <= p->dt_max))
    return fail(SSD_ERR_SHAPE, "dt_min = %g > dt_max = %g", p->dt_min, p->dt_max);
  if (p->input_dt != 0 && p->input_dt != 1)
    return fail(SSD_ERR_SHAPE, "input_dt = %d: must be 0 or 1", p->input_dt);
  if ((int64_t)p->batch * p->seqlen > INT32_MAX)
    return fail(SSD_ERR_UNSUPPORTED, "batch * seqlen exceeds 2^31 - 1 tokens");
  return SSD_OK;
}

ssd::Geo make_geo(const ssd_problem* p, const int32_t* meta) {
  ssd::Geo g;
  g.b = p->batch;
  g.T = p->seqlen;
  g.H = p->nheads;
  g.P = p->headdim;
  g.G = p->ngroups;
  g.N = p->dstate;
  g.C = p->chunk_size;
  g.nc = (int)cdiv(p->seqlen, p->chunk_size);
  g.K = (int)num_chunks(p);
  g.nseq = p->nseq > 0 ? p->nseq : p->batch;
  g.hpg = p->nheads / p->ngroups;
  g.Hs = p->nheads;
  g.meta = p->nseq > 0 ? meta : nullptr;
  return g;
}

ssd::TArg targ(const ssd_tensor& t) {
  ssd::TArg a;
  a.p = t.data;
  a.s0 = t.stride[0];
  a.s1 = t.stride[1];
  a.s2 = t.stride[2];
  return a;
}

// A 16-byte-vector operand: every row (innermost dim contiguous) starts on a
// 16-byte boundary.
ssd_status check_vec_tensor(const ssd_tensor& t, const char* name, bool required,
                            bool allow_f32 = true, bool allow_bf16 = true) {
  if (!t.data) {
    if (required) return fail(SSD_ERR_NULL, "%s is NULL", name);
    return SSD_OK;
  }
  if (!valid_dtype(t.dtype) || (t.dtype == SSD_F32 && !allow_f32) ||
      (t.dtype == SSD_BF16 && !allow_bf16))
    return fail(SSD_ERR_DTYPE, "%s has an unsupported dtype", name);
  const size_t es = dsize(t.dtype);
  if (reinterpret_cast<uintptr_t>(t.data) % 16 != 0)
    return fail(SSD_ERR_STRIDE, "%s: data pointer is not 16-byte aligned", name);
  for (int i = 0; i < 3; ++i) {
    if (t.stride[i] < 0) return fail(SSD_ERR_STRIDE, "%s: stride[%d] is negative", name, i);
    if ((t.stride[i] * (int64_t)es) % 16 != 0)
      return fail(SSD_ERR_STRIDE,
                  "%s: stride[%d] = %lld elements does not keep rows 16-byte aligned", name, i,
                  (long long)t.stride[i]);
  }
  return SSD_OK;
}

ssd_status check_dt(const ssd_tensor& t, bool required = true) {
  if (!t.data) {
    if (required) return fail(SSD_ERR_NULL, "dt is NULL");
    return SSD_OK;
  }
  if (!valid_dtype(t.dtype)) return fail(SSD_ERR_DTYPE, "dt has an unsupported dtype");
  if (reinterpret_cast<uintptr_t>(t.data) % dsize(t.dtype) != 0)
    return fail(SSD_ERR_STRIDE, "dt: data pointer is not element aligned");
  for (int i = 0; i < 3; ++i)
    if (t.stride[i] < 0) return fail(SSD_ERR_STRIDE, "dt: stride[%d] is negative", i);
  return SSD_OK;
}

#define SSD_TRY(expr)            \
  do {                           \
    ssd_status _s = (expr);      \
    if (_s != SSD_OK) return _s; \
  } while (0)

#define SSD_HIP(expr, where)                       \
  do {                                             \
    hipError_t _e = (expr);                        \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

// With no tokens at all the token tensors may be empty (NULL data).
bool has_tokens(const ssd_problem* p) { return (int64_t)p->batch * p->seqlen > 0; }

ssd_status need_meta(const ssd_problem* p) {
  if (p->nseq > 0 && !p->chunk_meta)
    return fail(SSD_ERR_NULL, "packed mode: chunk_meta is NULL (build it with ssd_varlen_chunk_meta)");
  return SSD_OK;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct StagedWs {
  size_t meta, cs, dtc, cb, st, total;
};

StagedWs staged_layout(const ssd_problem* p) {
  StagedWs w;
  const int64_t K = num_chunks(p);
  size_t off = 0;
  w.meta = off;
  // (the chunk table's length, for a problem already validated)
  if (p->nseq > 0)
    off += align256(((size_t)ssd::kMetaHeader + 3 * (size_t)num_chunks(p) + p->nseq + 1) *
                    sizeof(int32_t));
  w.cs = off;
  off += align256((size_t)K * p->nheads * p->chunk_size * sizeof(float));
  w.dtc = off;  // step size per position, when it scales the input term
  if (p->input_dt) off += align256((size_t)K * p->nheads * p->chunk_size * sizeof(float));
  w.cb = off;
  off += align256((size_t)K * p->ngroups * p->chunk_size * p->chunk_size * sizeof(float));
  w.st = off;
  off += align256((size_t)K * p->nheads * p->headdim * p->dstate * dsize(p->state_dtype));
  w.total = off;
  return w;
}

struct FusedWs {
  ssd::FusedPlan plan;
  int64_t K;  // 128-token chunk slots
  size_t meta, edec, agg, psum = 0, trace = 0, total;
};

// Chunk slots at the fused pass's own chunk length.
int64_t fused_chunks(const ssd_problem* p) {
  const int64_t nc = cdiv(p->seqlen, ssd::kFusedChunk);
  if (p->nseq > 0) return nc + p->nseq;
  return (int64_t)p->batch * nc;
}

FusedWs fused_layout(const ssd_problem* p, bool norm = false) {
  FusedWs w;
  w.K = fused_chunks(p);
  w.plan = ssd::fused_plan(w.K, p->nheads, p->headdim, p->dstate);
  const int64_t slots = (int64_t)w.plan.nr * w.plan.U;
  size_t off = 0;
  w.meta = off;
  if (p->nseq > 0)
    off += align256((size_t)(ssd::kMetaHeader + 3 * w.K + p->nseq + 1) * sizeof(int32_t));
  w.edec = off;
  off += align256((size_t)slots * sizeof(float));
  w.agg = off;
  off += align256((size_t)slots * 64 * 16 * w.plan.NT * sizeof(float));
  w.psum = off;  // gated RMSNorm fused in: per token and 64-channel block, sum(g^2)
  if (norm) off += align256((size_t)p->batch * p->seqlen * (p->nheads * p->headdim / 64) * sizeof(float));
#ifdef SSD_FUSED_TRACE
  // profiling build only: per-item phase timestamps at the end of the workspace
  w.trace = off;
  off += align256((size_t)slots * ssd::kFusedTraceSlots * sizeof(unsigned long long));
#endif
  w.total = off;
  return w;
}

ssd_status check_state_ptr(const float* ptr, const char* name) {
  if (ptr && reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
    return fail(SSD_ERR_STRIDE, "%s: data pointer is not 16-byte aligned", name);
  return SSD_OK;
}

// The fused forward and the per-chunk backward address a 128-token chunk's rows
// of a token tensor as 32-bit byte offsets from its first row (so that the base
// stays in scalar registers): 127 token strides plus one row must stay below
// 2^31 bytes.
bool chunk_rows_fit(const ssd_tensor& t, int64_t row_elems) {
  if (!t.data) return true;
  const int64_t s1 = t.stride[1] < 0 ? -t.stride[1] : t.stride[1];
  return (s1 * 127 + row_elems) * (int64_t)dsize(t.dtype) < (int64_t(1) << 31);
}
bool fwd_rows_fit(const ssd_problem* p, const ssd_fwd_args* a) {
  const int64_t P = p->headdim, N = p->dstate;
  return chunk_rows_fit(a->x, P) && chunk_rows_fit(a->B, N) && chunk_rows_fit(a->C, N) &&
         chunk_rows_fit(a->dt, 1) && chunk_rows_fit(a->z, P) && chunk_rows_fit(a->out, P);
}
bool bwd_rows_fit(const ssd_problem* p, const ssd_bwd_args* a) {
  const int64_t P = p->headdim, N = p->dstate;
  return chunk_rows_fit(a->x, P) && chunk_rows_fit(a->B, N) && chunk_rows_fit(a->C, N) &&
         chunk_rows_fit(a->dt, 1) && chunk_rows_fit(a->z, P) && chunk_rows_fit(a->dout, P) &&
         chunk_rows_fit(a->dx, P) && chunk_rows_fit(a->dB, N) && chunk_rows_fit(a->dC, N) &&
         chunk_rows_fit(a->ddt, 1) && chunk_rows_fit(a->dz, P);
}

// What the fused path takes (the rest of its checks are in fused_forward).
bool fused_applies(const ssd_problem* p, const ssd_fwd_args* a) {
  if (has_tokens(p) && a->x.dtype != SSD_BF16) return false;
  if (!fwd_rows_fit(p, a)) return false;
  if (p->dstate > 128) return false;
  if (p->input_dt && !p->dt_softplus && !(p->dt_clamp && p->dt_min >= 0.0f)) return false;
  return true;
}

// The single-pass forward (SSD_ALGO_FUSED); arguments common to both paths
// were validated by ssd_forward.
ssd_status fused_forward(const ssd_problem* p, const ssd_fwd_args* a, void* workspace,
                         size_t ws_bytes, hipStream_t stream, const ssd_norm_args* norm = nullptr) {
  if (has_tokens(p) && a->x.dtype != SSD_BF16)
    return fail(SSD_ERR_UNSUPPORTED, "SSD_ALGO_FUSED takes bf16 x, B, C (use SSD_ALGO_STAGED)");
  if (p->dstate > 128)
    return fail(SSD_ERR_UNSUPPORTED, "SSD_ALGO_FUSED supports dstate <= 128, got %d (use SSD_ALGO_STAGED)",
                p->dstate);
  if (p->input_dt && !p->dt_softplus && !(p->dt_clamp && p->dt_min >= 0.0f))
    return fail(SSD_ERR_UNSUPPORTED,
                "SSD_ALGO_FUSED with input_dt needs delta >= 0 (softplus, or a clamp with "
                "dt_min >= 0); use SSD_ALGO_STAGED");
  if (!fwd_rows_fit(p, a))
    return fail(SSD_ERR_UNSUPPORTED,
                "SSD_ALGO_FUSED needs 127 token strides of every token tensor below 2 GiB; "
                "use SSD_ALGO_STAGED");
  SSD_TRY(check_state_ptr(a->initial_states, "initial_states"));
  SSD_TRY(check_state_ptr(a->final_states, "final_states"));
  const FusedWs w = fused_layout(p, norm != nullptr);
  if (!workspace) return fail(SSD_ERR_WORKSPACE, "workspace is NULL");
  if (ws_bytes < w.total)
    return fail(SSD_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, w.total);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(SSD_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  ssd::FusedLaunch f;
  f.meta = p->nseq > 0 ? reinterpret_cast<int32_t*>(ws + w.meta) : nullptr;
  f.g = make_geo(p, f.meta);
  f.g.C = ssd::kFusedChunk;
  f.g.nc = (int)cdiv(p->seqlen, ssd::kFusedChunk);
  f.g.K = (int)w.K;
  f.cu = p->nseq > 0 ? p->cu_seqlens : nullptr;
  f.x = targ(a->x); f.B = targ(a->B); f.C = targ(a->C); f.dt = targ(a->dt);
  f.z = targ(a->z); f.out = targ(a->out);
  f.dt_dtype = dcode(a->dt.dtype);
  f.out_dtype = dcode(a->out.dtype);
  f.A = a->A; f.dt_bias = a->dt_bias; f.D = a->D;
  f.h0 = a->initial_states; f.hfinal = a->final_states;
  f.softplus = p->dt_softplus; f.clamp = p->dt_clamp; f.input_dt = p->input_dt;
  f.dt_min = p->dt_min; f.dt_max = p->dt_max;
  f.plan = w.plan;
  f.edec = reinterpret_cast<float*>(ws + w.edec);
  f.agg = reinterpret_cast<float*>(ws + w.agg);
#ifdef SSD_FUSED_TRACE
  f.trace = reinterpret_cast<unsigned long long*>(ws + w.trace);
#endif
  if (norm) f.psum = reinterpret_cast<float*>(ws + w.psum);
  SSD_HIP(ssd::launch_fused_fwd(f, stream), "fused forward launch");
  if (norm) {
    ssd::NormGeo ng;
    ng.ntok = (int)((int64_t)p->batch * p->seqlen);
    ng.T = p->seqlen;
    ng.H = p->nheads;
    ng.P = p->headdim;
    ng.gs = norm->group_size;
    ng.eps = norm->eps;
    SSD_HIP(ssd::launch_norm_finish(ng, f.psum, norm->weight, targ(a->out), dcode(a->out.dtype),
                                    norm->rstd, stream),
            "gated rmsnorm finish launch");
  }
  return ok();
}


// The staged forward: a6 (packed mode, unless `meta_in` gives a prebuilt
// chunk table), a1-a5 in sequence.  Arguments were validated by the caller.
ssd_status staged_run(const ssd_problem* p, const ssd_fwd_args* a, const int32_t* meta_in,
                      void* workspace, size_t ws_bytes, hipStream_t stream,
                      float* yoff = nullptr, int split = 0) {
  const StagedWs w = staged_layout(p);
  if (w.total > 0 && !workspace) return fail(SSD_ERR_WORKSPACE, "workspace is NULL");
  if (ws_bytes < w.total)
    return fail(SSD_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, w.total);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(SSD_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  int32_t* meta = p->nseq > 0 ? reinterpret_cast<int32_t*>(ws + w.meta) : nullptr;
  if (meta_in) meta = const_cast<int32_t*>(meta_in);
  float* cs = reinterpret_cast<float*>(ws + w.cs);
  float* dtc = p->input_dt ? reinterpret_cast<float*>(ws + w.dtc) : nullptr;
  float* cb = reinterpret_cast<float*>(ws + w.cb);
  void* st = ws + w.st;
  ssd::Geo g = make_geo(p, meta);
  const int in = dcode(a->x.dtype), sd = dcode(p->state_dtype);
  if (p->nseq > 0 && !meta_in)
    SSD_HIP(ssd::launch_varlen_meta(g, p->cu_seqlens, meta, stream), "varlen_chunk_meta launch");
  SSD_HIP(ssd::launch_chunk_cumsum(g, targ(a->dt), dcode(a->dt.dtype), a->A, a->dt_bias,
                                   p->dt_softplus, p->dt_clamp, p->dt_min, p->dt_max, cs, dtc,
                                   stream),
          "chunk_cumsum launch");
  SSD_HIP(ssd::launch_bmm_chunk(g, targ(a->C), targ(a->B), in, cb, stream), "bmm_chunk launch");
  SSD_HIP(ssd::launch_chunk_state(g, targ(a->x), targ(a->B), in, cs, dtc, st, sd, stream),
          "chunk_state launch");
  SSD_HIP(ssd::launch_state_passing(g, st, sd, cs, a->initial_states, st, a->final_states,
                                    stream),
          "state_passing launch");
  SSD_HIP(ssd::launch_chunk_scan(g, cb, targ(a->x), targ(a->C), in, cs, dtc, st, sd, a->D,
                                 targ(a->z), targ(a->out), dcode(a->out.dtype), stream, yoff, 0,
                                 1, split),
          "chunk_scan launch");
  return ok();
}

// ---------------------------------------------------------------- backward

// The chunk scan of a backward run whose chunk states are another run's
// carry-in states, stored transposed, and whose cumsum is that run's too:
// C.B^T, then the chunk scan reading the states transposed.  fp32 operands;
// the run's x is per group of x_div heads.
ssd_status transposed_scan(const ssd_problem* p, const ssd_fwd_args* a, const int32_t* meta,
                           const float* cs, const float* dtc, const float* states, float* cb,
                           int x_div, int split, hipStream_t stream) {
  const ssd::Geo g = make_geo(p, meta);
  const int in = dcode(a->x.dtype);
  SSD_HIP(ssd::launch_bmm_chunk(g, targ(a->C), targ(a->B), in, cb, stream), "bmm_chunk launch");
  SSD_HIP(ssd::launch_chunk_scan(g, cb, targ(a->x), targ(a->C), in, cs, dtc, states,
                                 dcode(SSD_F32), nullptr, targ(a->z), targ(a->out),
                                 dcode(a->out.dtype), stream, nullptr, 1, x_div, split),
          "chunk_scan launch");
  return ok();
}

// The problems of the forward recompute and the three backward scans (see
// bwd.hip): fwd and dC keep the step definition (softplus, clamp) of the
// caller's problem, dx and dB take precomputed steps; dB and dC run on the
// transposed state (head dim N, state dim P, one group per head).  All keep
// fp32 chunk states.
struct BwdProblems {
  ssd_problem fwd, dx, dB, dC;
};

// The mirrored scans run in packed form (batch rows become sequences) with
// their own chunk table, whose boundaries mirror the forward ones.
ssd_problem mirrored(const ssd_problem& q, const ssd_problem* p) {
  ssd_problem m = q;
  m.batch = 1;
  m.seqlen = (int32_t)((int64_t)p->batch * p->seqlen);
  m.nseq = p->nseq > 0 ? p->nseq : p->batch;
  m.chunk_meta = nullptr;
  return m;
}

BwdProblems bwd_problems(const ssd_problem* p) {
  BwdProblems q;
  q.fwd = *p;
  q.fwd.state_dtype = SSD_F32;
  q.fwd.chunk_meta = nullptr;
  q.dx = q.fwd;
  q.dx.dt_softplus = 0;
  q.dx.dt_clamp = 0;
  q.dx.input_dt = 0;  // the adjoint's input dy (outer) C carries no step size
  q.dB = q.dx;
  q.dB.headdim = p->dstate;
  q.dB.dstate = p->headdim;
  q.dB.ngroups = p->nheads;
  q.dC = q.fwd;
  q.dC.headdim = p->dstate;
  q.dC.dstate = p->headdim;
  q.dC.ngroups = p->nheads;
  return q;
}

struct BwdWs {
  size_t yf, yo, dy, dyr, Cr, Br, Bf, xr, xf, delta, gd, dtr, dyx, xg, gx, gb, gc,
      gfirst, mmeta, mcu, part, run_fwd, run_dx, run_rest, fwd_bytes, dx_bytes, rest_bytes, total;
};

int64_t bwd_tokens(const ssd_problem* p) { return (int64_t)p->batch * p->seqlen; }
int bwd_nseq(const ssd_problem* p) { return p->nseq > 0 ? p->nseq : p->batch; }

BwdWs bwd_layout(const ssd_problem* p) {
  BwdWs w;
  const size_t nt = (size_t)bwd_tokens(p), H = p->nheads, P = p->headdim, N = p->dstate,
               G = p->ngroups, ns = (size_t)bwd_nseq(p);
  size_t off = 0;
  auto take = [&](size_t floats) {
    const size_t o = off;
    off += align256(floats * sizeof(float));
    return o;
  };
  w.yf = take(nt * H * P);
  w.yo = take(nt * H * P);
  w.dy = take(nt * H * P);
  w.dyr = take(nt * H * P);
  w.Cr = take(nt * G * N);
  w.Br = take(nt * G * N);
  w.Bf = take(nt * G * N);
  w.xr = take(nt * H * P);
  w.xf = take(nt * H * P);
  w.delta = take(nt * H);
  w.gd = take(nt * H);
  w.dtr = take(nt * H);
  w.dyx = take(nt * H);
  w.xg = take(p->input_dt ? nt * H : 0);
  w.gx = take(nt * H * P);
  w.gb = take(nt * H * N);
  w.gc = take(nt * H * N);
  w.gfirst = take(ns * H * P * N);
  const BwdProblems q = bwd_problems(p);
  const ssd_problem mdx = mirrored(q.dx, p), mdB = mirrored(q.dB, p);
  w.mmeta = off;
  off += align256(((size_t)ssd::kMetaHeader + 3 * (size_t)num_chunks(&mdx) + mdx.nseq + 1) *
                  sizeof(int32_t));
  w.mcu = off;
  off += align256((ns + 1) * sizeof(int32_t));
  w.part = off;
  off += align256((size_t)num_chunks(p) * H * 3 * sizeof(double));
  // the forward recompute and the mirrored dx scan keep their workspaces (the
  // dB and dC scans read their cumsums and chunk states, the step-size
  // gradients their chunk states and the forward's C.B^T); the dB and dC
  // scans need only a C.B^T buffer, shared, dC last (its C.B^T, dy.x^T, is
  // read by the step-size gradients too)
  w.fwd_bytes = staged_layout(&q.fwd).total;
  w.dx_bytes = staged_layout(&mdx).total;
  auto cb_bytes = [](const ssd_problem* r) {
    return (size_t)num_chunks(r) * r->ngroups * r->chunk_size * r->chunk_size * sizeof(float);
  };
  w.rest_bytes = std::max(cb_bytes(&mdB), cb_bytes(&q.dC));
  w.run_fwd = off;
  off += align256(w.fwd_bytes);
  w.run_dx = off;
  off += align256(w.dx_bytes);
  w.run_rest = off;
  off += align256(w.rest_bytes);
  w.total = off;
  return w;
}

// (b, T, rows, width) contiguous fp32 view of a scratch buffer
ssd_tensor scratch_view(void* ptr, const ssd_problem* p, int rows, int width) {
  ssd_tensor t;
  t.data = ptr;
  t.dtype = SSD_F32;
  t.stride[0] = (int64_t)p->seqlen * rows * width;
  t.stride[1] = (int64_t)rows * width;
  t.stride[2] = width;
  return t;
}

ssd_status check_grad_tensor(const ssd_tensor& t, const char* name, bool required) {
  SSD_TRY(check_vec_tensor(t, name, required, true, false));
  return SSD_OK;
}

// Arguments common to both forward paths.
ssd_status check_fwd_args(const ssd_problem* p, const ssd_fwd_args* a) {
  SSD_TRY(check_problem(p));
  if (!a) return fail(SSD_ERR_NULL, "args is NULL");
  SSD_TRY(check_vec_tensor(a->x, "x", has_tokens(p)));
  SSD_TRY(check_vec_tensor(a->B, "B", has_tokens(p)));
  SSD_TRY(check_vec_tensor(a->C, "C", has_tokens(p)));
  SSD_TRY(check_dt(a->dt, has_tokens(p)));
  SSD_TRY(check_vec_tensor(a->z, "z", false));
  SSD_TRY(check_vec_tensor(a->out, "out", has_tokens(p)));
  if (has_tokens(p) && (a->x.dtype != a->B.dtype || a->x.dtype != a->C.dtype))
    return fail(SSD_ERR_DTYPE, "x, B and C must share a dtype");
  if (a->z.data && a->z.dtype != a->x.dtype) return fail(SSD_ERR_DTYPE, "z must have x's dtype");
  if (!a->A) return fail(SSD_ERR_NULL, "A is NULL");
  return SSD_OK;
}

// The forward with the gated RMSNorm fused in: checks of the norm arguments.
ssd_status check_norm_args(const ssd_problem* p, const ssd_norm_args* n) {
  if (!n) return fail(SSD_ERR_NULL, "norm args is NULL");
  if (!n->weight) return fail(SSD_ERR_NULL, "norm weight is NULL");
  if (reinterpret_cast<uintptr_t>(n->weight) % 16 != 0)
    return fail(SSD_ERR_STRIDE, "norm weight is not 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(n->rstd) % 4 != 0)
    return fail(SSD_ERR_STRIDE, "rstd is not 4-byte aligned");
  if (!(n->eps >= 0.0f)) return fail(SSD_ERR_SHAPE, "eps = %g must be >= 0", n->eps);
  if (p->headdim % 64 != 0)
    return fail(SSD_ERR_UNSUPPORTED,
                "the fused gated norm needs headdim a multiple of 64, got %d (use ssd_forward "
                "and ssd_gated_rmsnorm_fwd)", p->headdim);
  const int W = p->nheads * p->headdim;
  const int gs = n->group_size;
  if (gs < 64 || gs % 64 != 0 || W % gs != 0)
    return fail(SSD_ERR_SHAPE, "group_size = %d must be a multiple of 64 dividing H * P = %d",
                gs, W);
  if (W / gs > ssd::kNormFinishGroups)
    return fail(SSD_ERR_UNSUPPORTED, "H * P / group_size = %d groups per token exceeds %d",
                W / gs, ssd::kNormFinishGroups);
  return SSD_OK;
}

}  // namespace

namespace ssd {
ssd_status api_fail(ssd_status s, const char* msg) { return fail(s, "%s", msg); }
}  // namespace ssd

extern "C" {

const char* ssd_version(void) { return "libssd 0.1 (gfx950)"; }

const char* ssd_status_string(ssd_status s) {
  switch (s) {
    case SSD_OK: return "SSD_OK";
    case SSD_ERR_NULL: return "SSD_ERR_NULL";
    case SSD_ERR_SHAPE: return "SSD_ERR_SHAPE";
    case SSD_ERR_DTYPE: return "SSD_ERR_DTYPE";
    case SSD_ERR_STRIDE: return "SSD_ERR_STRIDE";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE";
    case SSD_ERR_HIP: return "SSD_ERR_HIP";
  }
  return "SSD_ERR_UNKNOWN";
}

const char* ssd_last_error_message(void) { return g_msg.c_str(); }

ssd_status ssd_problem_check(const ssd_problem* p) {
  SSD_TRY(check_problem(p));
  return ok();
}

int64_t ssd_num_chunks(const ssd_problem* p) {
  if (check_problem(p) != SSD_OK) return -1;
  return num_chunks(p);
}

size_t ssd_varlen_meta_len(const ssd_problem* p) {
  if (check_problem(p) != SSD_OK || p->nseq <= 0) return 0;
  return (size_t)ssd::kMetaHeader + 3 * (size_t)num_chunks(p) + (size_t)p->nseq + 1;
}

ssd_status ssd_workspace_size(const ssd_problem* p, ssd_algo algo, size_t* bytes) {
  SSD_TRY(check_problem(p));
  if (!bytes) return fail(SSD_ERR_NULL, "bytes is NULL");
  if (algo != SSD_ALGO_STAGED && algo != SSD_ALGO_FUSED && algo != SSD_ALGO_AUTO)
    return fail(SSD_ERR_UNSUPPORTED, "unknown algo %d", (int)algo);
  const size_t fu = fused_layout(p).total, st = staged_layout(p).total;
  *bytes = algo == SSD_ALGO_FUSED ? fu : (algo == SSD_ALGO_STAGED ? st : (fu > st ? fu : st));
  return ok();
}

ssd_status ssd_varlen_chunk_meta(const ssd_problem* p, int32_t* meta, hipStream_t stream) {
  SSD_TRY(check_problem(p));
  if (p->nseq <= 0) return fail(SSD_ERR_SHAPE, "ssd_varlen_chunk_meta needs packed mode (nseq > 0)");
  if (!meta) return fail(SSD_ERR_NULL, "meta is NULL");
  ssd::Geo g = make_geo(p, meta);
  SSD_HIP(ssd::launch_varlen_meta(g, p->cu_seqlens, meta, stream), "varlen_chunk_meta launch");
  return ok();
}

ssd_status ssd_varlen_chunk_meta_host(const ssd_problem* p, const int32_t* cu, int32_t* meta,
                                      size_t meta_len) {
  SSD_TRY(check_problem(p));
  if (p->nseq <= 0) return fail(SSD_ERR_SHAPE, "ssd_varlen_chunk_meta_host needs packed mode");
  if (!cu || !meta) return fail(SSD_ERR_NULL, "cu_seqlens or meta is NULL");
  const size_t need = ssd_varlen_meta_len(p);
  if (meta_len < need)
    return fail(SSD_ERR_SHAPE, "meta_len = %zu, need %zu", meta_len, need);
  if (cu[0] != 0) return fail(SSD_ERR_SHAPE, "cu_seqlens[0] = %d, must be 0", cu[0]);
  for (int i = 0; i < p->nseq; ++i)
    if (cu[i + 1] < cu[i])
      return fail(SSD_ERR_SHAPE, "cu_seqlens decreases at %d (%d -> %d)", i, cu[i], cu[i + 1]);
  if (cu[p->nseq] != p->seqlen)
    return fail(SSD_ERR_SHAPE, "cu_seqlens[nseq] = %d, must equal seqlen = %d", cu[p->nseq],
                p->seqlen);
  const int C = p->chunk_size;
  const int64_t K = num_chunks(p);
  int32_t* first = meta + ssd::kMetaHeader + 3 * K;
  int32_t j = 0;
  for (int i = 0; i < p->nseq; ++i) {
    first[i] = j;
    const int L = cu[i + 1] - cu[i];
    for (int k = 0; k * C < L; ++k, ++j) {
      int32_t* e = meta + ssd::kMetaHeader + 3 * j;
      e[0] = i;
      e[1] = cu[i] + k * C;
      e[2] = L - k * C < C ? L - k * C : C;
    }
  }
  first[p->nseq] = j;
  for (int64_t r = j; r < K; ++r) {
    int32_t* e = meta + ssd::kMetaHeader + 3 * r;
    e[0] = -1; e[1] = 0; e[2] = 0;
  }
  meta[0] = j; meta[1] = p->nseq; meta[2] = C; meta[3] = (int32_t)K;
  return ok();
}

ssd_status ssd_chunk_cumsum(const ssd_problem* p, ssd_tensor dt, const float* A,
                            const float* dt_bias, float* dA_cumsum, float* dt_out,
                            hipStream_t stream) {
  SSD_TRY(check_problem(p));
  SSD_TRY(need_meta(p));
  SSD_TRY(check_dt(dt, has_tokens(p)));
  if (!A) return fail(SSD_ERR_NULL, "A is NULL");
  if (!dA_cumsum) return fail(SSD_ERR_NULL, "dA_cumsum is NULL");
  ssd::Geo g = make_geo(p, p->chunk_meta);
  SSD_HIP(ssd::launch_chunk_cumsum(g, targ(dt), dcode(dt.dtype), A, dt_bias, p->dt_softplus,
                                   p->dt_clamp, p->dt_min, p->dt_max, dA_cumsum, dt_out, stream),
          "chunk_cumsum launch");
  return ok();
}

ssd_status ssd_bmm_chunk(const ssd_problem* p, ssd_tensor C, ssd_tensor B, float* CB,
                         hipStream_t stream) {
  SSD_TRY(check_problem(p));
  SSD_TRY(need_meta(p));
  SSD_TRY(check_vec_tensor(C, "C", has_tokens(p)));
  SSD_TRY(check_vec_tensor(B, "B", has_tokens(p)));
  if (C.dtype != B.dtype) return fail(SSD_ERR_DTYPE, "B and C must share a dtype");
  if (!CB) return fail(SSD_ERR_NULL, "CB is NULL");
  ssd::Geo g = make_geo(p, p->chunk_meta);
  SSD_HIP(ssd::launch_bmm_chunk(g, targ(C), targ(B), dcode(C.dtype), CB, stream),
          "bmm_chunk launch");
  return ok();
}

ssd_status ssd_chunk_state(const ssd_problem* p, ssd_tensor x, ssd_tensor B,
                           const float* dA_cumsum, const float* dt_chunk, void* states,
                           hipStream_t stream) {
  SSD_TRY(check_problem(p));
  SSD_TRY(need_meta(p));
  SSD_TRY(check_vec_tensor(x, "x", has_tokens(p)));
  SSD_TRY(check_vec_tensor(B, "B", has_tokens(p)));
  if (x.dtype != B.dtype) return fail(SSD_ERR_DTYPE, "x and B must share a dtype");
  if (!dA_cumsum || !states) return fail(SSD_ERR_NULL, "dA_cumsum or states is NULL");
  if (p->input_dt && !dt_chunk) return fail(SSD_ERR_NULL, "input_dt: dt_chunk is NULL");
  ssd::Geo g = make_geo(p, p->chunk_meta);
  SSD_HIP(ssd::launch_chunk_state(g, targ(x), targ(B), dcode(x.dtype), dA_cumsum,
                                  p->input_dt ? dt_chunk : nullptr, states,
                                  dcode(p->state_dtype), stream),
          "chunk_state launch");
  return ok();
}

ssd_status ssd_state_passing(const ssd_problem* p, const void* states, const float* dA_cumsum,
                             const float* initial_states, void* states_out,
                             float* final_states, hipStream_t stream) {
  SSD_TRY(check_problem(p));
  SSD_TRY(need_meta(p));
  if (!states || !dA_cumsum || !states_out)
    return fail(SSD_ERR_NULL, "states, dA_cumsum or states_out is NULL");
  ssd::Geo g = make_geo(p, p->chunk_meta);
  SSD_HIP(ssd::launch_state_passing(g, states, dcode(p->state_dtype), dA_cumsum, initial_states,
                                    states_out, final_states, stream),
          "state_passing launch");
  return ok();
}

ssd_status ssd_chunk_scan(const ssd_problem* p, const float* CB, ssd_tensor x, ssd_tensor C,
                          const float* dA_cumsum, const float* dt_chunk,
                          const void* states_in, const float* D, ssd_tensor z,
                          ssd_tensor out, hipStream_t stream) {
  SSD_TRY(check_problem(p));
  SSD_TRY(need_meta(p));
  SSD_TRY(check_vec_tensor(x, "x", has_tokens(p)));
  SSD_TRY(check_vec_tensor(C, "C", has_tokens(p)));
  SSD_TRY(check_vec_tensor(z, "z", false));
  SSD_TRY(check_vec_tensor(out, "out", has_tokens(p)));
  if (x.dtype != C.dtype) return fail(SSD_ERR_DTYPE, "x and C must share a dtype");
  if (z.data && z.dtype != x.dtype) return fail(SSD_ERR_DTYPE, "z must have x's dtype");
  if (!CB || !dA_cumsum || !states_in)
    return fail(SSD_ERR_NULL, "CB, dA_cumsum or states_in is NULL");
  if (p->input_dt && !dt_chunk) return fail(SSD_ERR_NULL, "input_dt: dt_chunk is NULL");
  ssd::Geo g = make_geo(p, p->chunk_meta);
  SSD_HIP(ssd::launch_chunk_scan(g, CB, targ(x), targ(C), dcode(x.dtype), dA_cumsum,
                                 p->input_dt ? dt_chunk : nullptr, states_in,
                                 dcode(p->state_dtype), D, targ(z), targ(out), dcode(out.dtype),
                                 stream),
          "chunk_scan launch");
  return ok();
}

ssd_status ssd_forward(const ssd_problem* p, ssd_algo algo, const ssd_fwd_args* a,
                       void* workspace, size_t ws_bytes, hipStream_t stream) {
  SSD_TRY(check_fwd_args(p, a));
  if (algo != SSD_ALGO_STAGED && algo != SSD_ALGO_FUSED && algo != SSD_ALGO_AUTO)
    return fail(SSD_ERR_UNSUPPORTED, "unknown algo %d", (int)algo);
  if (algo == SSD_ALGO_AUTO) algo = fused_applies(p, a) ? SSD_ALGO_FUSED : SSD_ALGO_STAGED;
  if (algo == SSD_ALGO_FUSED) return fused_forward(p, a, workspace, ws_bytes, stream);
  return staged_run(p, a, nullptr, workspace, ws_bytes, stream);
}

ssd_status ssd_forward_gated_norm_workspace_size(const ssd_problem* p, const ssd_norm_args* n,
                                                 size_t* bytes) {
  SSD_TRY(check_problem(p));
  SSD_TRY(check_norm_args(p, n));
  if (!bytes) return fail(SSD_ERR_NULL, "bytes is NULL");
  *bytes = fused_layout(p, true).total;
  return ok();
}

ssd_status ssd_forward_gated_norm(const ssd_problem* p, const ssd_fwd_args* a,
                                  const ssd_norm_args* n, void* workspace, size_t ws_bytes,
                                  hipStream_t stream) {
  SSD_TRY(check_fwd_args(p, a));
  SSD_TRY(check_norm_args(p, n));
  return fused_forward(p, a, workspace, ws_bytes, stream, n);
}

ssd_status ssd_backward_workspace_size(const ssd_problem* p, size_t* bytes) {
  SSD_TRY(check_problem(p));
  if (!bytes) return fail(SSD_ERR_NULL, "bytes is NULL");
  *bytes = bwd_layout(p).total;
  return ok();
}

}  // extern "C"

namespace {

// Arguments of both backward paths.
ssd_status check_bwd_args(const ssd_problem* p, const ssd_bwd_args* a) {
  SSD_TRY(check_problem(p));
  if (!a) return fail(SSD_ERR_NULL, "args is NULL");
  const bool tok = has_tokens(p);
  SSD_TRY(check_vec_tensor(a->x, "x", tok));
  SSD_TRY(check_vec_tensor(a->B, "B", tok));
  SSD_TRY(check_vec_tensor(a->C, "C", tok));
  SSD_TRY(check_dt(a->dt, tok));
  SSD_TRY(check_vec_tensor(a->z, "z", false));
  SSD_TRY(check_vec_tensor(a->dout, "dout", tok));
  if (tok && (a->x.dtype != a->B.dtype || a->x.dtype != a->C.dtype))
    return fail(SSD_ERR_DTYPE, "x, B and C must share a dtype");
  if (a->z.data && a->z.dtype != a->x.dtype) return fail(SSD_ERR_DTYPE, "z must have x's dtype");
  if (!a->A) return fail(SSD_ERR_NULL, "A is NULL");
  SSD_TRY(check_grad_tensor(a->dx, "dx", tok));
  SSD_TRY(check_grad_tensor(a->dB, "dB", tok));
  SSD_TRY(check_grad_tensor(a->dC, "dC", tok));
  SSD_TRY(check_grad_tensor(a->dz, "dz", tok && a->z.data));
  SSD_TRY(check_dt(a->ddt, tok));
  if (a->ddt.data && a->ddt.dtype != SSD_F32) return fail(SSD_ERR_DTYPE, "ddt must be F32");
  if (!a->dA || !a->ddt_bias) return fail(SSD_ERR_NULL, "dA or ddt_bias is NULL");
  SSD_TRY(check_state_ptr(a->initial_states, "initial_states"));
  SSD_TRY(check_state_ptr(a->dfinal_states, "dfinal_states"));
  SSD_TRY(check_state_ptr(a->dinitial_states, "dinitial_states"));
  if (bwd_tokens(p) * (p->nheads > p->ngroups ? p->nheads : p->ngroups) > INT32_MAX)
    return fail(SSD_ERR_UNSUPPORTED, "backward: tokens x heads exceeds 2^31 - 1");
  return SSD_OK;
}

ssd_status workspace_ok(const void* workspace, size_t ws_bytes, size_t need) {
  if (!workspace) return fail(SSD_ERR_WORKSPACE, "workspace is NULL");
  if (ws_bytes < need)
    return fail(SSD_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(SSD_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  return SSD_OK;
}

// The staged backward (SSD_ALGO_STAGED); arguments validated by the caller.
ssd_status staged_backward(const ssd_problem* p, const ssd_bwd_args* a, void* workspace,
                           size_t ws_bytes, hipStream_t stream) {
  const BwdWs w = bwd_layout(p);
  if (!workspace) return fail(SSD_ERR_WORKSPACE, "workspace is NULL");
  if (ws_bytes < w.total)
    return fail(SSD_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, w.total);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(SSD_ERR_WORKSPACE, "workspace is not 256-byte aligned");

  char* ws = static_cast<char*>(workspace);
  auto f = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  const BwdProblems q = bwd_problems(p);
  const int H = p->nheads, P = p->headdim, N = p->dstate, G = p->ngroups;
  const int ns = bwd_nseq(p);
  ssd::BwdGeo bg;
  bg.ntok = (int)bwd_tokens(p);
  bg.T = p->seqlen;
  bg.nseq = ns;
  bg.H = H;
  bg.P = P;
  bg.G = G;
  bg.N = N;
  bg.hpg = H / G;
  bg.cu = p->nseq > 0 ? p->cu_seqlens : nullptr;
  const ssd_tensor none = {nullptr, SSD_F32, {0, 0, 0}};
  char* ws_fwd = ws + w.run_fwd;
  char* ws_dx = ws + w.run_dx;
  char* ws_rest = ws + w.run_rest;

  // 1. fp32 copies of the operands the fp32 scans read (mirrored in time for
  // the backward ones)
  const int in = dcode(a->x.dtype);
  struct Copy { ssd_tensor src; int R, W, rep, rev; size_t dst; };
  const Copy copies[] = {{a->C, G, N, 1, 1, w.Cr},     {a->B, G, N, 1, 1, w.Br},
                         {a->B, G, N, 1, 0, w.Bf},
                         {a->x, H, P, 1, 1, w.xr},     {a->x, H, P, 1, 0, w.xf}};
  for (const Copy& c : copies)
    SSD_HIP(ssd::launch_bwd_gather(bg, targ(c.src), in, c.R, c.W, c.rep, c.rev, f(c.dst), stream),
            "backward gather launch");

  // 2. forward recompute on the caller's operands (bf16 inputs take the bf16
  // kernels, whose derived operands are split hi + lo: fp32-accurate), with
  // fp32 states and output: y before the gate (for dz), its inter-chunk part
  // exp(cs_l) C_l . h_in (for the step sizes), and the carry-in state of every
  // chunk, kept in its workspace
  ssd_fwd_args fa;
  fa.x = a->x;
  fa.B = a->B;
  fa.C = a->C;
  fa.dt = a->dt;
  fa.A = a->A; fa.dt_bias = a->dt_bias; fa.D = a->D; fa.z = none;
  fa.initial_states = a->initial_states;
  fa.out = scratch_view(f(w.yf), p, H, P);
  fa.final_states = nullptr;
  SSD_TRY(staged_run(&q.fwd, &fa, nullptr, ws_fwd, w.fwd_bytes, stream, f(w.yo)));

  // 3. gate, steps, transposed states, the mirrored chunk table
  SSD_HIP(ssd::launch_bwd_gate(bg, targ(a->dout), dcode(a->dout.dtype), targ(a->z), in, f(w.yf),
                               f(w.dy), f(w.dyr), targ(a->dz), stream),
          "backward gate launch");
  SSD_HIP(ssd::launch_bwd_steps(bg, targ(a->dt), dcode(a->dt.dtype), a->A, a->dt_bias,
                                p->dt_softplus, p->dt_clamp, p->dt_min, p->dt_max, f(w.delta),
                                f(w.gd), f(w.dtr), stream),
          "backward steps launch");
  ssd_problem mdx = mirrored(q.dx, p), mdB = mirrored(q.dB, p);
  int32_t* mmeta = reinterpret_cast<int32_t*>(ws + w.mmeta);
  int32_t* mcu = p->nseq > 0 ? const_cast<int32_t*>(p->cu_seqlens)
                             : reinterpret_cast<int32_t*>(ws + w.mcu);
  SSD_HIP(ssd::launch_bwd_mirror_meta(bg, p->chunk_size, (int)num_chunks(&mdx), mmeta,
                                      p->nseq > 0 ? nullptr : mcu, stream),
          "backward chunk table launch");
  mdx.cu_seqlens = mcu;
  mdB.cu_seqlens = mcu;

  // 4. the three scans: dx and dB backwards in time (mirrored operands,
  // shifted steps, mirrored chunk table), dC forwards.  Their chunk scans
  // multiply fp32 operands; for bf16 inputs (held to the bf16 tolerance) the
  // operands are split into bf16 hi + lo, three bf16 matrix instructions per
  // product, ~16 significant bits per operand
  const int split = in == ssd::DT_BF16 ? 1 : 0;
  ssd_tensor dtr;
  dtr.data = f(w.dtr);
  dtr.dtype = SSD_F32;
  dtr.stride[0] = (int64_t)mdx.seqlen * H;
  dtr.stride[1] = H;
  dtr.stride[2] = 1;
  ssd_fwd_args ra;
  ra.x = scratch_view(f(w.dyr), &mdx, H, P);
  ra.B = scratch_view(f(w.Cr), &mdx, G, N);
  ra.C = scratch_view(f(w.Br), &mdx, G, N);
  ra.dt = dtr; ra.A = a->A; ra.dt_bias = nullptr; ra.D = nullptr; ra.z = none;
  ra.initial_states = a->dfinal_states;
  ra.out = scratch_view(f(w.gx), &mdx, H, P);
  ra.final_states = f(w.gfirst);
  // (its inter-chunk part goes to yf, free since the gate)
  SSD_TRY(staged_run(&mdx, &ra, mmeta, ws_dx, w.dx_bytes, stream, f(w.yf), split));
  // dB and dC: the chunk states these scans would compute are the dx and
  // forward scans' carry-in states transposed (G^T and S^T, with the initial
  // states already folded in), and their cumsums are those scans' own; so
  // only C.B^T and the chunk scan run, reading the states transposed
  const StagedWs lf = staged_layout(&q.fwd), lx = staged_layout(&mdx);
  const int32_t* fwd_meta = p->nseq > 0 ? reinterpret_cast<int32_t*>(ws_fwd + lf.meta) : nullptr;
  float* cb_rest = reinterpret_cast<float*>(ws_rest);
  ra.x = scratch_view(f(w.Cr), &mdB, G, N);  // (each group's row serves its heads)
  ra.B = scratch_view(f(w.dyr), &mdB, H, P);
  ra.C = scratch_view(f(w.xr), &mdB, H, P);
  ra.out = scratch_view(f(w.gb), &mdB, H, N);
  SSD_TRY(transposed_scan(&mdB, &ra, mmeta, reinterpret_cast<float*>(ws_dx + lx.cs), nullptr,
                          reinterpret_cast<float*>(ws_dx + lx.st), cb_rest, H / G, split,
                          stream));
  ra.x = scratch_view(f(w.Bf), p, G, N);
  ra.B = scratch_view(f(w.xf), p, H, P);
  ra.C = scratch_view(f(w.dy), p, H, P);
  ra.out = scratch_view(f(w.gc), p, H, N);
  SSD_TRY(transposed_scan(&q.dC, &ra, fwd_meta, reinterpret_cast<float*>(ws_fwd + lf.cs),
                          p->input_dt ? reinterpret_cast<float*>(ws_fwd + lf.dtc) : nullptr,
                          reinterpret_cast<float*>(ws_fwd + lf.st), cb_rest, H / G, split,
                          stream));

  // 5. gradients
  // (with the step size on the input term, dx and dB carry it and its
  // gradient gains x . G B)
  float* dlt = p->input_dt ? f(w.delta) : nullptr;
  float* xg = p->input_dt ? f(w.xg) : nullptr;
  SSD_HIP(ssd::launch_bwd_tokens(bg, targ(a->x), in, a->D, f(w.dy), f(w.gx), dlt, targ(a->dx),
                                 f(w.dyx), xg, stream),
          "backward tokens launch");
  SSD_HIP(ssd::launch_bwd_group_sums(bg, f(w.gb), f(w.gc), dlt, targ(a->dB), targ(a->dC),
                                     stream),
          "backward group sums launch");
  const ssd::Geo gf = make_geo(&q.fwd, fwd_meta);
  // (the dC scan's C.B^T is dy . x^T per head, and it ran last in ws_rest)
  SSD_HIP(ssd::launch_bwd_step_grads(
              bg, gf, reinterpret_cast<float*>(ws_fwd + lf.cb), cb_rest, f(w.yo), f(w.yf),
              f(w.xf), f(w.dy),
              f(w.dyx), f(w.delta), f(w.gd), a->A,
              reinterpret_cast<float*>(ws_fwd + lf.st), reinterpret_cast<float*>(ws_dx + lx.st),
              f(w.gfirst), a->dfinal_states, xg, targ(a->ddt),
              reinterpret_cast<double*>(ws + w.part),
              a->dA, a->ddt_bias, a->D ? a->dD : nullptr, a->dinitial_states, stream),
          "backward step gradients launch");
  return ok();
}

// ---- the per-chunk backward (SSD_ALGO_FUSED): the forward's carry-in states
// and the gradients of the states leaving every chunk (two state passes, the
// second backwards, at 128-token chunks), then the per-chunk gradient kernels of
// bwd_chunk.hip

bool bwd_fused_applies(const ssd_problem* p, ssd_dtype in_dtype) {
  return has_tokens(p) && in_dtype == SSD_BF16 && p->headdim == 64 && p->dstate <= 128 &&
         p->dstate % 8 == 0;
}

struct BwdChunkWs {
  size_t fmeta, cs, dtc, st, adj, delta, gd, part, pdb, pdc, total;
};

// The forward recompute of the per-chunk backward: 128-token chunks, fp32 states.
ssd_problem chunk_fwd_problem(const ssd_problem* p) {
  ssd_problem f = *p;
  f.chunk_size = ssd::kBwdChunk;
  f.state_dtype = SSD_F32;
  f.chunk_meta = nullptr;
  return f;
}

// A pass of the per-chunk backward covers `hb` heads: a whole number of groups,
// or (when a group's heads split into dB/dC workgroups of eight) a multiple of
// eight heads of one group, whose dB and dC are then summed over the group's
// passes in split order.
int pass_groups(const ssd_problem* p, int hb) {
  const int hpg = p->nheads / p->ngroups;
  return hb >= hpg ? hb / hpg : 1;
}
bool pass_in_group(const ssd_problem* p, int hb) { return hb < p->nheads / p->ngroups; }

// Workspace of one pass over `hb` heads: everything per head is sized for the
// pass, the chunk table for the problem.
BwdChunkWs bwd_chunk_layout(const ssd_problem* p, int hb) {
  BwdChunkWs w;
  const ssd_problem fp = chunk_fwd_problem(p);
  const size_t nt = (size_t)bwd_tokens(p), H = (size_t)hb, P = p->headdim, N = p->dstate,
               G = (size_t)pass_groups(p, hb);
  const size_t K = (size_t)num_chunks(&fp);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  w.fmeta = take(p->nseq > 0 ? (ssd::kMetaHeader + 3 * K + p->nseq + 1) * sizeof(int32_t) : 0);
  w.cs = take(K * H * ssd::kBwdChunk * sizeof(float));
  w.dtc = take(p->input_dt ? K * H * ssd::kBwdChunk * sizeof(float) : 0);
  w.st = take(K * H * P * N * sizeof(float));
  w.adj = take(K * H * P * N * sizeof(float));
  w.delta = take(nt * H * sizeof(float));
  w.gd = take(nt * H * sizeof(float));
  w.part = take(K * H * 3 * sizeof(double));
  const int splits = ssd::bwd_chunk_splits((int)(H / G));
  const bool partials = splits > 1 || pass_in_group(p, hb);
  w.pdb = take(partials ? (size_t)splits * nt * G * N * sizeof(float) : 0);
  w.pdc = take(partials ? (size_t)splits * nt * G * N * sizeof(float) : 0);
  w.total = off;
  return w;
}

// Heads per pass.  The two fp32 state buffers (the state entering every chunk
// and its gradient) grow with the heads of a pass; by default a pass holds at
// most kBwdStateBudget bytes of them, in passes of equal size.  With a given
// workspace: the largest passes that fit.  Pass sizes: multiples of the heads
// per group, and below that multiples of eight (one dB/dC workgroup's heads)
// when they divide a group evenly.
constexpr size_t kBwdStateBudget = size_t(256) << 20;

std::vector<int> pass_sizes(const ssd_problem* p) {
  const int H = p->nheads, hpg = H / p->ngroups, u = ssd::kBwdHeadsPerSplit;
  std::vector<int> v;
  if (hpg > u && hpg % u == 0)
    for (int h = u; h < hpg; h += u) v.push_back(h);
  for (int h = hpg; h <= H; h += hpg) v.push_back(h);
  return v;
}

// passes of equal size no larger than hmax (one of pass_sizes)
int balanced_pass(const ssd_problem* p, int hmax) {
  const int H = p->nheads, hpg = H / p->ngroups;
  if (hmax >= H) return H;
  if (hmax >= hpg) return (int)cdiv(cdiv(H, cdiv(H, hmax)), hpg) * hpg;
  const int u = ssd::kBwdHeadsPerSplit;
  return (int)cdiv(cdiv(hpg, cdiv(hpg, hmax)), u) * u;
}

int bwd_heads_default(const ssd_problem* p) {
  const ssd_problem fp = chunk_fwd_problem(p);
  const size_t per_head = 2 * (size_t)num_chunks(&fp) * p->headdim * p->dstate * sizeof(float);
  const std::vector<int> v = pass_sizes(p);
  int hb = v.front();
  for (int h : v)
    if ((size_t)h * per_head <= kBwdStateBudget) hb = h;
  return balanced_pass(p, hb);
}

// 0 when not even the smallest pass fits in ws_bytes
int bwd_heads_fit(const ssd_problem* p, size_t ws_bytes) {
  int hb = 0;
  for (int h : pass_sizes(p))
    if (bwd_chunk_layout(p, h).total <= ws_bytes) hb = h;
  return hb ? balanced_pass(p, hb) : 0;
}

ssd_status chunk_backward(const ssd_problem* p, const ssd_bwd_args* a, void* workspace,
                          size_t ws_bytes, hipStream_t stream) {
  const int H = p->nheads, G = p->ngroups, hpg = H / G;
  const int hb = bwd_heads_fit(p, ws_bytes);
  SSD_TRY(workspace_ok(workspace, ws_bytes, bwd_chunk_layout(p, hb ? hb : pass_sizes(p).front()).total));
  const BwdChunkWs w = bwd_chunk_layout(p, hb);
  char* ws = static_cast<char*>(workspace);
  auto f = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  const ssd_problem fp = chunk_fwd_problem(p);
  const int in = dcode(a->x.dtype);
  const size_t PN = (size_t)p->headdim * p->dstate;

  // the chunk table at 128 tokens (packed mode), shared by every pass
  int32_t* fmeta = p->nseq > 0 ? reinterpret_cast<int32_t*>(ws + w.fmeta) : nullptr;
  if (fmeta)
    SSD_HIP(ssd::launch_varlen_meta(make_geo(&fp, fmeta), p->cu_seqlens, fmeta, stream),
            "chunk table launch");

  // a tensor or per-head array moved to head h0 (group h0 / hpg)
  auto heads = [](ssd_tensor t, int64_t n) {
    if (t.data) t.data = static_cast<char*>(t.data) + n * t.stride[2] * (int64_t)dsize(t.dtype);
    return t;
  };
  auto at_head = [](auto* ptr, int64_t n) { return ptr ? ptr + n : ptr; };

  // the passes: (first head, heads), in head order
  std::vector<std::pair<int, int>> passes;
  if (!pass_in_group(p, hb)) {
    for (int h0 = 0; h0 < H; h0 += hb) passes.emplace_back(h0, std::min(hb, H - h0));
  } else {
    for (int g = 0; g < G; ++g)
      for (int k = 0; k < hpg; k += hb) passes.emplace_back(g * hpg + k, std::min(hb, hpg - k));
  }
  for (const auto& ps : passes) {
    const int h0 = ps.first, hn = ps.second, g0 = h0 / hpg;
    const bool in_group = pass_in_group(p, hb);
    ssd_problem pp = fp;
    pp.nheads = hn;
    pp.ngroups = in_group ? 1 : hn / hpg;
    ssd::Geo gf = make_geo(&pp, fmeta);
    gf.Hs = H;  // initial and final states keep the problem's head axis
    ssd::BwdGeo bg;
    bg.ntok = (int)bwd_tokens(p);
    bg.T = p->seqlen;
    bg.nseq = bwd_nseq(p);
    bg.H = hn;
    bg.P = p->headdim;
    bg.G = pp.ngroups;
    bg.N = p->dstate;
    bg.hpg = hn / pp.ngroups;
    bg.cu = p->nseq > 0 ? p->cu_seqlens : nullptr;
    const ssd_tensor x = heads(a->x, h0), B = heads(a->B, g0), C = heads(a->C, g0),
                     dt = heads(a->dt, h0);
    const float* A = a->A + h0;
    const float* dt_bias = at_head(a->dt_bias, h0);
    const float* h0s = at_head(a->initial_states, (int64_t)h0 * PN);

    // 1. forward recompute at 128-token chunks: cumsum, chunk states (the
    // carry-in states come with the adjoint's scan, step 3)
    float* dtc = p->input_dt ? f(w.dtc) : nullptr;
    SSD_HIP(ssd::launch_chunk_cumsum(gf, targ(dt), dcode(dt.dtype), A, dt_bias, p->dt_softplus,
                                     p->dt_clamp, p->dt_min, p->dt_max, f(w.cs), dtc, stream),
            "backward cumsum launch");
    SSD_HIP(ssd::launch_chunk_state(gf, targ(x), targ(B), in, f(w.cs), dtc, f(w.st),
                                    ssd::DT_F32, stream),
            "backward chunk state launch");

    // 2. step sizes and their derivatives
    SSD_HIP(ssd::launch_bwd_steps(bg, targ(dt), dcode(dt.dtype), A, dt_bias, p->dt_softplus,
                                  p->dt_clamp, p->dt_min, p->dt_max, f(w.delta), f(w.gd), nullptr,
                                  stream),
            "backward steps launch");

    // 3. the adjoint: each chunk's own gradient of its entering state; then
    // in one launch the forward state passing (chunk states -> carry-in
    // states) and the reverse one (dfinal in, the initial states' gradient
    // out), two independent scans over the chunks
    ssd::BwdChunkLaunch l;
    l.g = gf;
    l.ntok = bg.ntok;
    l.x = targ(x); l.B = targ(B); l.C = targ(C); l.z = targ(heads(a->z, h0));
    l.dout = targ(heads(a->dout, h0));
    l.dx = targ(heads(a->dx, h0)); l.dz = targ(heads(a->dz, h0));
    l.dB = targ(heads(a->dB, g0)); l.dC = targ(heads(a->dC, g0));
    l.ddt = targ(heads(a->ddt, h0));
    l.dout_dtype = dcode(a->dout.dtype);
    l.A = A; l.D = at_head(a->D, h0);
    l.delta = f(w.delta); l.gd = f(w.gd);
    l.cs = f(w.cs); l.hin = f(w.st); l.adj = f(w.adj);
    l.part = reinterpret_cast<double*>(ws + w.part);
    l.input_dt = p->input_dt;
    l.pdb = f(w.pdb);
    l.pdc = f(w.pdc);
    l.partials = in_group;
    l.accumulate = in_group && h0 % hpg != 0;
    SSD_HIP(ssd::launch_bwd_adj_state(l, stream), "backward adjoint chunk state launch");
    SSD_HIP(ssd::launch_state_passing_pair(gf, f(w.st), f(w.cs), h0s, f(w.adj),
                                           at_head(a->dfinal_states, (int64_t)h0 * PN),
                                           at_head(a->dinitial_states, (int64_t)h0 * PN), stream),
            "backward state passing launch");

    // 4. the per-chunk gradients, then the per-head sums
    SSD_HIP(ssd::launch_bwd_chunk(l, stream), "backward chunk kernels launch");
    SSD_HIP(ssd::launch_bwd_step_heads(bg, gf.K, reinterpret_cast<double*>(ws + w.part), nullptr,
                                       a->dA + h0, a->ddt_bias + h0,
                                       a->D ? a->dD + h0 : nullptr, nullptr, stream),
            "backward per-head sums launch");
  }
  return ok();
}

size_t bwd_workspace(const ssd_problem* p, ssd_algo algo, ssd_dtype in_dtype) {
  if (algo == SSD_ALGO_FUSED || (algo == SSD_ALGO_AUTO && bwd_fused_applies(p, in_dtype)))
    return bwd_chunk_layout(p, bwd_heads_default(p)).total;
  return bwd_layout(p).total;
}

}  // namespace

extern "C" {

ssd_status ssd_backward(const ssd_problem* p, const ssd_bwd_args* a, void* workspace,
                        size_t ws_bytes, hipStream_t stream) {
  SSD_TRY(check_bwd_args(p, a));
  return staged_backward(p, a, workspace, ws_bytes, stream);
}

ssd_status ssd_backward_ex_workspace_size(const ssd_problem* p, ssd_algo algo,
                                          ssd_dtype in_dtype, size_t* bytes) {
  SSD_TRY(check_problem(p));
  if (!bytes) return fail(SSD_ERR_NULL, "bytes is NULL");
  if (algo != SSD_ALGO_STAGED && algo != SSD_ALGO_FUSED && algo != SSD_ALGO_AUTO)
    return fail(SSD_ERR_SHAPE, "algo = %d is not STAGED, FUSED or AUTO", (int)algo);
  if (!valid_dtype(in_dtype)) return fail(SSD_ERR_DTYPE, "in_dtype is not F32 or BF16");
  *bytes = bwd_workspace(p, algo, in_dtype);
  return ok();
}

ssd_status ssd_backward_ex(const ssd_problem* p, const ssd_bwd_args* a, ssd_algo algo,
                           void* workspace, size_t ws_bytes, hipStream_t stream) {
  SSD_TRY(check_bwd_args(p, a));
  if (algo != SSD_ALGO_STAGED && algo != SSD_ALGO_FUSED && algo != SSD_ALGO_AUTO)
    return fail(SSD_ERR_SHAPE, "algo = %d is not STAGED, FUSED or AUTO", (int)algo);
  const ssd_dtype in = has_tokens(p) ? a->x.dtype : SSD_F32;
  if (algo == SSD_ALGO_FUSED && !bwd_fused_applies(p, in))
    return fail(SSD_ERR_UNSUPPORTED,
                "the per-chunk backward takes bf16 x, B, C with tokens, headdim 64 and dstate "
                "<= 128 (a multiple of 8); got headdim %d, dstate %d (use SSD_ALGO_STAGED)",
                p->headdim, p->dstate);
  if (algo == SSD_ALGO_FUSED && !bwd_rows_fit(p, a))
    return fail(SSD_ERR_UNSUPPORTED,
                "the per-chunk backward needs 127 token strides of every token tensor below "
                "2 GiB (use SSD_ALGO_STAGED)");
  if (algo == SSD_ALGO_FUSED ||
      (algo == SSD_ALGO_AUTO && bwd_fused_applies(p, in) && bwd_rows_fit(p, a)))
    return chunk_backward(p, a, workspace, ws_bytes, stream);
  return staged_backward(p, a, workspace, ws_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- complex A

static ssd_status check_cx_problem(const ssd_complex_problem* p) {
  if (!p) return fail(SSD_ERR_NULL, "problem is NULL");
  if (p->batch < 1) return fail(SSD_ERR_SHAPE, "batch = %d must be >= 1", p->batch);
  if (p->seqlen < 0) return fail(SSD_ERR_SHAPE, "seqlen = %d must be >= 0", p->seqlen);
  if (p->nheads < 1) return fail(SSD_ERR_SHAPE, "nheads = %d must be >= 1", p->nheads);
  if (p->nseq < 0) return fail(SSD_ERR_SHAPE, "nseq = %d must be >= 0", p->nseq);
  if (p->nseq > 0) {
    if (p->batch != 1)
      return fail(SSD_ERR_SHAPE, "packed mode (nseq = %d) requires batch == 1, got %d", p->nseq,
                  p->batch);
    if (!p->cu_seqlens) return fail(SSD_ERR_NULL, "packed mode requires cu_seqlens");
  }
  const int64_t nsq = p->nseq > 0 ? p->nseq : p->batch;
  if (nsq * p->nheads > 65535)
    return fail(SSD_ERR_UNSUPPORTED, "(batch or nseq) * nheads = %lld exceeds 65535",
                (long long)(nsq * p->nheads));
  if (p->headdim < 16 || p->headdim > 128 || p->headdim % 16 != 0)
    return fail(SSD_ERR_UNSUPPORTED, "headdim = %d: must be a multiple of 16 in [16, 128]",
                p->headdim);
  if (p->dstate < 16 || p->dstate > 128 || p->dstate % 16 != 0)
    return fail(SSD_ERR_UNSUPPORTED, "dstate = %d: must be a multiple of 16 in [16, 128]",
                p->dstate);
  const int C = p->chunk_size;
  if (C != 32 && C != 64 && C != 128 && C != 256)
    return fail(SSD_ERR_UNSUPPORTED, "chunk_size = %d: must be 32, 64, 128 or 256", C);
  if ((int64_t)p->batch * p->seqlen > INT32_MAX)
    return fail(SSD_ERR_UNSUPPORTED, "batch * seqlen exceeds 2^31 - 1 tokens");
  return SSD_OK;
}

// A complex operand: float32 pairs, rows 16-byte aligned (strides even in
// complex elements).
static ssd_status check_cx_tensor(const ssd_tensor& t, const char* name, bool required) {
  if (!t.data) {
    if (required) return fail(SSD_ERR_NULL, "%s is NULL", name);
    return SSD_OK;
  }
  if (t.dtype != SSD_F32) return fail(SSD_ERR_DTYPE, "%s must be complex64 (SSD_F32 pairs)", name);
  if (reinterpret_cast<uintptr_t>(t.data) % 16 != 0)
    return fail(SSD_ERR_STRIDE, "%s: data pointer is not 16-byte aligned", name);
  for (int i = 0; i < 3; ++i) {
    if (t.stride[i] < 0) return fail(SSD_ERR_STRIDE, "%s: stride[%d] is negative", name, i);
    if (t.stride[i] % 2 != 0)
      return fail(SSD_ERR_STRIDE,
                  "%s: stride[%d] = %lld complex elements does not keep rows 16-byte aligned",
                  name, i, (long long)t.stride[i]);
  }
  return SSD_OK;
}

static ssd_status check_cx_dt(const ssd_tensor& t, bool required) {
  if (!t.data) {
    if (required) return fail(SSD_ERR_NULL, "dt is NULL");
    return SSD_OK;
  }
  if (t.dtype != SSD_F32) return fail(SSD_ERR_DTYPE, "dt must be float32");
  if (reinterpret_cast<uintptr_t>(t.data) % 4 != 0)
    return fail(SSD_ERR_STRIDE, "dt: data pointer is not element aligned");
  for (int i = 0; i < 3; ++i)
    if (t.stride[i] < 0) return fail(SSD_ERR_STRIDE, "dt: stride[%d] is negative", i);
  return SSD_OK;
}

static ssd_status check_cx_out(const ssd_tensor& t, int out_complex, bool required) {
  if (out_complex != 0 && out_complex != 1)
    return fail(SSD_ERR_SHAPE, "out_complex = %d: must be 0 or 1", out_complex);
  if (!t.data) {
    if (required) return fail(SSD_ERR_NULL, "out is NULL");
    return SSD_OK;
  }
  if (t.dtype != SSD_F32) return fail(SSD_ERR_DTYPE, "out must be float32 or complex64");
  if (reinterpret_cast<uintptr_t>(t.data) % (out_complex ? 8 : 4) != 0)
    return fail(SSD_ERR_STRIDE, "out: data pointer is not element aligned");
  for (int i = 0; i < 3; ++i)
    if (t.stride[i] < 0) return fail(SSD_ERR_STRIDE, "out: stride[%d] is negative", i);
  return SSD_OK;
}

static ssd_status check_cx_A(const float* A) {
  if (!A) return fail(SSD_ERR_NULL, "A is NULL");
  if (reinterpret_cast<uintptr_t>(A) % 8 != 0)
    return fail(SSD_ERR_STRIDE, "A: data pointer is not 8-byte aligned");
  return SSD_OK;
}

static ssd_status check_aligned16(const void* ptr, const char* name, bool required) {
  if (!ptr) {
    if (required) return fail(SSD_ERR_NULL, "%s is NULL", name);
    return SSD_OK;
  }
  if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
    return fail(SSD_ERR_STRIDE, "%s is not 16-byte aligned", name);
  return SSD_OK;
}

static int64_t cx_num_chunks(const ssd_complex_problem* p) {
  const int64_t nc = cdiv(p->seqlen, p->chunk_size);
  return p->nseq > 0 ? nc + p->nseq : (int64_t)p->batch * nc;
}

// The complex scan on the shared chunk geometry: one "group" per head.
static ssd::Geo cx_geo(const ssd_complex_problem* p, const int32_t* meta) {
  ssd::Geo g;
  g.b = p->batch; g.T = p->seqlen; g.H = p->nheads; g.P = p->headdim; g.N = p->dstate;
  g.G = p->nheads; g.hpg = 1; g.Hs = p->nheads;
  g.C = p->chunk_size;
  g.nc = (int)cdiv(p->seqlen, p->chunk_size);
  g.K = (int)cx_num_chunks(p);
  g.nseq = p->nseq > 0 ? p->nseq : p->batch;
  g.meta = p->nseq > 0 ? meta : nullptr;
  return g;
}

struct CxWorkspace {
  size_t states, lam, meta, total;
};

static CxWorkspace cx_workspace(const ssd_complex_problem* p) {
  const int64_t K = cx_num_chunks(p);
  CxWorkspace w;
  w.states = 0;
  w.lam = align256((size_t)K * p->nheads * p->headdim * p->dstate * 8);
  w.meta = w.lam + align256((size_t)p->nheads * K * sizeof(float));
  const size_t meta_len = p->nseq > 0 ? (size_t)(ssd::kMetaHeader + 3 * K + p->nseq + 1) : 0;
  w.total = w.meta + align256(meta_len * sizeof(int32_t));
  return w;
}

extern "C" {

ssd_status ssd_complex_problem_check(const ssd_complex_problem* p) {
  SSD_TRY(check_cx_problem(p));
  return ok();
}

ssd_status ssd_complex_workspace_size(const ssd_complex_problem* p, size_t* bytes) {
  SSD_TRY(check_cx_problem(p));
  if (!bytes) return fail(SSD_ERR_NULL, "bytes is NULL");
  *bytes = cx_workspace(p).total;
  return ok();
}

ssd_status ssd_complex_forward(const ssd_complex_problem* p, const ssd_complex_fwd_args* a,
                               void* workspace, size_t ws_bytes, hipStream_t stream) {
  SSD_TRY(check_cx_problem(p));
  if (!a) return fail(SSD_ERR_NULL, "args is NULL");
  const bool tok = (int64_t)p->batch * p->seqlen > 0;
  SSD_TRY(check_cx_tensor(a->x, "x", tok));
  SSD_TRY(check_cx_tensor(a->B, "B", tok));
  SSD_TRY(check_cx_tensor(a->C, "C", tok));
  SSD_TRY(check_cx_dt(a->dt, tok));
  SSD_TRY(check_cx_out(a->out, a->out_complex, tok));
  SSD_TRY(check_cx_A(a->A));
  SSD_TRY(check_aligned16(a->initial_states, "initial_states", false));
  SSD_TRY(check_aligned16(a->final_states, "final_states", false));
  const CxWorkspace w = cx_workspace(p);
  if (w.total > 0 && !workspace) return fail(SSD_ERR_WORKSPACE, "workspace is NULL");
  if (ws_bytes < w.total)
    return fail(SSD_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, w.total);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(SSD_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  int32_t* meta = reinterpret_cast<int32_t*>(ws + w.meta);
  const ssd::Geo g = cx_geo(p, meta);
  if (p->nseq > 0)
    SSD_HIP(ssd::launch_varlen_meta(g, p->cu_seqlens, meta, stream), "chunk table launch");
  float* states = reinterpret_cast<float*>(ws + w.states);
  float* lam = reinterpret_cast<float*>(ws + w.lam);
  SSD_HIP(ssd::launch_cx_chunk_state(g, targ(a->x), targ(a->B), targ(a->dt), a->A, states, lam,
                                     stream),
          "complex chunk state launch");
  SSD_HIP(ssd::launch_cx_state_pass(g, a->A, lam, a->initial_states, states, a->final_states,
                                    stream),
          "complex state passing launch");
  SSD_HIP(ssd::launch_cx_chunk_scan(g, targ(a->x), targ(a->B), targ(a->C), targ(a->dt), a->A,
                                    states, targ(a->out), a->out_complex, stream),
          "complex chunk scan launch");
  return ok();
}

ssd_status ssd_complex_chunk_state(const ssd_complex_problem* p, ssd_tensor x, ssd_tensor B,
                                   ssd_tensor dt, const float* A, float* states,
                                   float* chunk_dt_sum, hipStream_t stream) {
  SSD_TRY(check_cx_problem(p));
  if (p->nseq > 0)
    return fail(SSD_ERR_UNSUPPORTED, "packed problems run through ssd_complex_forward only");
  const bool tok = (int64_t)p->batch * p->seqlen > 0;
  SSD_TRY(check_cx_tensor(x, "x", tok));
  SSD_TRY(check_cx_tensor(B, "B", tok));
  SSD_TRY(check_cx_dt(dt, tok));
  SSD_TRY(check_cx_A(A));
  SSD_TRY(check_aligned16(states, "states", tok));
  SSD_TRY(check_aligned16(chunk_dt_sum, "chunk_dt_sum", tok));
  SSD_HIP(ssd::launch_cx_chunk_state(cx_geo(p, nullptr), targ(x), targ(B), targ(dt), A, states,
                                     chunk_dt_sum, stream),
          "complex chunk state launch");
  return ok();
}

ssd_status ssd_complex_state_passing(const ssd_complex_problem* p, const float* A,
                                     const float* chunk_dt_sum, const float* initial_states,
                                     float* states, float* final_states, hipStream_t stream) {
  SSD_TRY(check_cx_problem(p));
  if (p->nseq > 0)
    return fail(SSD_ERR_UNSUPPORTED, "packed problems run through ssd_complex_forward only");
  const bool tok = (int64_t)p->batch * p->seqlen > 0;
  SSD_TRY(check_cx_A(A));
  SSD_TRY(check_aligned16(chunk_dt_sum, "chunk_dt_sum", tok));
  SSD_TRY(check_aligned16(states, "states", tok));
  SSD_TRY(check_aligned16(initial_states, "initial_states", false));
  SSD_TRY(check_aligned16(final_states, "final_states", false));
  SSD_HIP(ssd::launch_cx_state_pass(cx_geo(p, nullptr), A, chunk_dt_sum, initial_states, states,
                                    final_states, stream),
          "complex state passing launch");
  return ok();
}

ssd_status ssd_complex_chunk_scan(const ssd_complex_problem* p, ssd_tensor x, ssd_tensor B,
                                  ssd_tensor C, ssd_tensor dt, const float* A,
                                  const float* states_in, ssd_tensor out, int32_t out_complex,
                                  hipStream_t stream) {
  SSD_TRY(check_cx_problem(p));
  if (p->nseq > 0)
    return fail(SSD_ERR_UNSUPPORTED, "packed problems run through ssd_complex_forward only");
  const bool tok = (int64_t)p->batch * p->seqlen > 0;
  SSD_TRY(check_cx_tensor(x, "x", tok));
  SSD_TRY(check_cx_tensor(B, "B", tok));
  SSD_TRY(check_cx_tensor(C, "C", tok));
  SSD_TRY(check_cx_dt(dt, tok));
  SSD_TRY(check_cx_A(A));
  SSD_TRY(check_aligned16(states_in, "states_in", tok));
  SSD_TRY(check_cx_out(out, out_complex, tok));
  SSD_HIP(ssd::launch_cx_chunk_scan(cx_geo(p, nullptr), targ(x), targ(B), targ(C), targ(dt), A,
                                    states_in, targ(out), out_complex, stream),
          "complex chunk scan launch");
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------- gated RMSNorm

static ssd_status check_norm_problem(const ssd_norm_problem* p) {
  if (!p) return fail(SSD_ERR_NULL, "problem is NULL");
  if (p->batch < 1) return fail(SSD_ERR_SHAPE, "batch = %d must be >= 1", p->batch);
  if (p->seqlen < 0) return fail(SSD_ERR_SHAPE, "seqlen = %d must be >= 0", p->seqlen);
  if (p->nheads < 1) return fail(SSD_ERR_SHAPE, "nheads = %d must be >= 1", p->nheads);
  if (p->headdim < 8 || p->headdim % 8 != 0)
    return fail(SSD_ERR_UNSUPPORTED, "headdim = %d: must be a positive multiple of 8", p->headdim);
  const int64_t W = (int64_t)p->nheads * p->headdim;
  if (W > (1 << 24)) return fail(SSD_ERR_UNSUPPORTED, "nheads * headdim exceeds 2^24");
  const int gs = p->group_size;
  if (gs < 1 || W % gs != 0)
    return fail(SSD_ERR_SHAPE, "group_size = %d must divide nheads * headdim = %lld", gs,
                (long long)W);
  const bool pow2 = (gs & (gs - 1)) == 0;
  if (!((pow2 && gs >= 8 && gs <= 512) || gs % 512 == 0))
    return fail(SSD_ERR_UNSUPPORTED,
                "group_size = %d: must be a power of two in [8, 512] or a multiple of 512", gs);
  if (!(p->eps >= 0.0f) || p->eps == INFINITY)
    return fail(SSD_ERR_SHAPE, "eps = %g must be finite and >= 0", (double)p->eps);
  if ((int64_t)p->batch * p->seqlen > INT32_MAX)
    return fail(SSD_ERR_UNSUPPORTED, "batch * seqlen exceeds 2^31 - 1 tokens");
  // the kernels number (token, 8-channel vector) items in 32 bits
  if ((int64_t)p->batch * p->seqlen * (W / 8) > INT32_MAX)
    return fail(SSD_ERR_UNSUPPORTED,
                "batch * seqlen * nheads * headdim / 8 exceeds 2^31 - 1 (split the tokens)");
  return SSD_OK;
}

static ssd::NormGeo norm_geo(const ssd_norm_problem* p) {
  ssd::NormGeo g;
  g.ntok = p->batch * p->seqlen;
  g.T = p->seqlen > 0 ? p->seqlen : 1;
  g.H = p->nheads; g.P = p->headdim; g.gs = p->group_size; g.eps = p->eps;
  return g;
}

struct NormWorkspace {
  size_t part, stats, total;
};

static NormWorkspace norm_workspace(const ssd_norm_problem* p) {
  const ssd::NormGeo g = norm_geo(p);
  const size_t W = (size_t)p->nheads * p->headdim;
  NormWorkspace w;
  w.part = 0;
  w.stats = align256((size_t)ssd::norm_tiles(g) * W * sizeof(float));
  const size_t st = p->group_size > 512 ? (size_t)g.ntok * (W / p->group_size) * 8 : 0;
  w.total = w.stats + align256(st);
  return w;
}

static ssd_status check_norm_io(const ssd_norm_problem* p, const ssd_tensor& y,
                                const ssd_tensor& z, const float* weight) {
  const bool tok = (int64_t)p->batch * p->seqlen > 0;
  SSD_TRY(check_vec_tensor(y, "y", tok));
  SSD_TRY(check_vec_tensor(z, "z", false));
  if (z.data && y.data && z.dtype != y.dtype)
    return fail(SSD_ERR_DTYPE, "z must have the dtype of y");
  if (!weight) return fail(SSD_ERR_NULL, "weight is NULL");
  if (reinterpret_cast<uintptr_t>(weight) % 16 != 0)
    return fail(SSD_ERR_STRIDE, "weight is not 16-byte aligned");
  return SSD_OK;
}

extern "C" {

ssd_status ssd_gated_rmsnorm_fwd(const ssd_norm_problem* p, ssd_tensor y, ssd_tensor z,
                                 const float* weight, ssd_tensor out, float* rstd,
                                 hipStream_t stream) {
  SSD_TRY(check_norm_problem(p));
  SSD_TRY(check_norm_io(p, y, z, weight));
  const bool tok = (int64_t)p->batch * p->seqlen > 0;
  SSD_TRY(check_vec_tensor(out, "out", tok));
  if (reinterpret_cast<uintptr_t>(rstd) % 4 != 0)
    return fail(SSD_ERR_STRIDE, "rstd is not 4-byte aligned");
  if (!tok) return ok();
  SSD_HIP(ssd::launch_norm_fwd(norm_geo(p), targ(y), targ(z), dcode(y.dtype), weight, targ(out),
                               dcode(out.dtype), rstd, stream),
          "gated rmsnorm forward launch");
  return ok();
}

ssd_status ssd_gated_rmsnorm_bwd_workspace_size(const ssd_norm_problem* p, size_t* bytes) {
  SSD_TRY(check_norm_problem(p));
  if (!bytes) return fail(SSD_ERR_NULL, "bytes is NULL");
  *bytes = norm_workspace(p).total;
  return ok();
}

ssd_status ssd_gated_rmsnorm_bwd(const ssd_norm_problem* p, ssd_tensor y, ssd_tensor z,
                                 const float* weight, ssd_tensor dout, ssd_tensor dy,
                                 ssd_tensor dz, float* dweight, void* workspace,
                                 size_t ws_bytes, hipStream_t stream) {
  SSD_TRY(check_norm_problem(p));
  SSD_TRY(check_norm_io(p, y, z, weight));
  const bool tok = (int64_t)p->batch * p->seqlen > 0;
  SSD_TRY(check_vec_tensor(dout, "dout", tok));
  if (dout.data && y.data && dout.dtype != y.dtype)
    return fail(SSD_ERR_DTYPE, "dout must have the dtype of y");
  SSD_TRY(check_vec_tensor(dy, "dy", tok, true, false));
  SSD_TRY(check_vec_tensor(dz, "dz", tok && z.data != nullptr, true, false));
  if (!dweight) return fail(SSD_ERR_NULL, "dweight is NULL");
  const NormWorkspace w = norm_workspace(p);
  if (w.total > 0 && !workspace) return fail(SSD_ERR_WORKSPACE, "workspace is NULL");
  if (ws_bytes < w.total)
    return fail(SSD_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, w.total);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(SSD_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  SSD_HIP(ssd::launch_norm_bwd(norm_geo(p), targ(y), targ(z), dcode(y.data ? y.dtype : SSD_F32),
                               weight, targ(dout), targ(dy), targ(dz), dweight,
                               reinterpret_cast<float*>(ws + w.part),
                               reinterpret_cast<float2*>(ws + w.stats), stream),
          "gated rmsnorm backward launch");
  return ok();
}

}  // extern "C"
