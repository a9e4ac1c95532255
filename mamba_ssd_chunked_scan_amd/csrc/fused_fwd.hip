// fused_fwd.hip -- the whole SSD forward pass (stages 1-5) as one pass over the
// inputs: x, B, C, dt and z are read, out and the final states are written,
// and nothing chunk-sized goes through HBM in between.
//
// The math is the chunked algorithm of the SSD Reference ("Chunking and the
// discretized log-decay", "Intra-chunk outputs and per-chunk states",
// "Inter-chunk propagation", "Readout") with the D skip and SiLU gate of
// cudnn-frontend PR 1133, organised the way vLLM PR 27299 ("Purpose")
// describes its fused kernel: the log-decay cumsum and C.B^T are recomputed
// where they are consumed instead of being stored, and the chunk-to-chunk state
// is handed between workgroups through memory (here: per range of chunks,
// across launch boundaries, so that no workgroup waits for another).
//
// Work split.  The internal chunk is 128 tokens (the chunked result does not
// depend on the chunk length, so the problem's chunk_size only matters to the
// staged path).  A unit is (head h, 64-row slab of P); its chunks are cut into
// `nr` ranges of R consecutive chunks, and one workgroup owns one (unit,
// range).  Three launches (after a small table / empty-sequence kernel in
// packed mode):
//   1. the aggregate launch: every range whose last sequence continues into
//      the next range runs the chunk-state recurrence over its chunks from a
//      zero state -- or from the sequence's initial state when the sequence
//      starts inside the range -- and stores that aggregate with the range's
//      total decay E;
//   2. the carry launch: per unit, the ranges in order turn each aggregate into
//      the state at the end of its range (carry = E carry + agg, restarted
//      where a sequence starts), in place;
//   3. the output launch: a range whose first chunk continues a sequence
//      loads the state its predecessor ends with: its carry-in.
//      Then it walks its chunks: cumsum from dt, chunk state S_j, the carry-in
//      H_j of the chunk staged in LDS as bf16 hi + lo, C.B^T tile by tile,
//      Y_off + Y_diag (with the D skip on its diagonal), SiLU gate, store;
//      H_{j+1} = exp(Lambda_j) H_j + S_j in registers, and the final state at
//      a sequence's last chunk.
// The hand-offs between them are launch boundaries: no workgroup ever
// waits for another, so no wait can stall or time out, and the order of every
// sum is fixed (results are bit-identical run to run).  The aggregate launch
// has the output launch's work split, without its register and LDS demands
// beyond the chunk-state product.
// Placement.  Workgroup ids go to the 8 XCDs in turn; ids are mapped so that
// XCD x holds the units [x U / 8, (x + 1) U / 8) -- consecutive heads, so the
// heads of a group, which read the same B and C chunks, meet in one XCD's L2
// -- range first.
//
// Per chunk, per workgroup (4 waves, wave w).  x and B are staged in LDS in
// their natural layout (tokens x columns); operands that need the token axis
// as the reduction axis are read with the gfx950 LDS transpose read, so no
// thread ever transposes data itself.
//   * S_j^T (n x p) = B^T (n x s) . (w_s x_s) (s x p): wave w owns p-tile w
//     and all n-tiles; the carried state uses this accumulator layout (lane:
//     one p, four consecutive n per n-tile), which is also the layout of the
//     carry-in rows the Y_off operand reads from LDS;
//   * C.B^T: wave w computes the tiles (s-tile, l-tile) of its l-tiles w and
//     7 - w (balanced causal work), B rows from the LDS tile and C fragments
//     from global memory (n contiguous in both), while the B tile is still in
//     LDS; the tiles stay in registers.  The accumulator layout of a C.B^T
//     tile (lane: one l, four consecutive s) is used directly as the A operand
//     of Y_diag = M . x with the k (token) order permuted to match; the x
//     operand is read from the x tile in that same order, so M never goes
//     through LDS.  D x is folded into the same product: M gets D added on
//     its diagonal (y_l = sum_s M_ls x_s + D x_l).
// Precision: exact bf16 inputs, fp32-derived operands (decay-weighted x,
// M = L o CB + D I, the carried state) split into bf16 hi + lo, fp32
// accumulation, and an fp32 within-chunk cumsum (bf16 inputs only).
#include "kernels.hpp"
#include "stage_varlen.hpp"

namespace ssd {

namespace {

constexpr int FC = 128;                 // internal chunk length
constexpr int kCarryBatch = 8;          // aggregates loaded per round trip of the carry launch

// softplus(u) = max(u, 0) + log1p(exp(-|u|)).  log1p(e) for e in (0, 1] as
// log(1 + e) * e / ((1 + e) - 1): the quotient corrects the rounding of 1 + e
// (an exact identity in real arithmetic; a few ulp in fp32, also for e far
// below the fp32 spacing at 1, where 1 + e rounds to 1 and the result is e).
__device__ __forceinline__ float softplus_fast(float u) {
  const float e = __expf(-fabsf(u));
  const float t = 1.0f + e;
  const float d = t - 1.0f;
  const float l1p = d == 0.0f ? e : __logf(t) * (e * __builtin_amdgcn_rcpf(d));
  return fmaxf(u, 0.0f) + l1p;
}

#ifndef SSD_FUSED_XPAD
#define SSD_FUSED_XPAD 8
#endif
#ifndef SSD_FUSED_BPAD
#define SSD_FUSED_BPAD 8
#endif
#ifndef SSD_FUSED_HPAD
#define SSD_FUSED_HPAD 8
#endif
#ifndef SSD_FUSED_SG
#define SSD_FUSED_SG 4
#endif
#ifndef SSD_FUSED_YPAD
#define SSD_FUSED_YPAD 4
#endif
constexpr int FXLD = 64 + SSD_FUSED_XPAD;   // bf16 per row of the x tile in LDS
constexpr int FXV = (FC * 8) / 256;     // 16-byte x (and z, out) vectors per thread
constexpr int FYLD = 64 + SSD_FUSED_YPAD;  // floats per staged output row

template <int NT> struct FCfg {
  static constexpr int NMAX = 16 * NT;         // d_state capacity
  static constexpr int NKB = NT / 2;           // 32-wide k-blocks over n
  static constexpr int BV = FC * NMAX / 8 / 256;   // 16-byte B vectors per thread
  static constexpr int BLD = NMAX + SSD_FUSED_BPAD;  // bf16 per row of the B tile in LDS
  static constexpr int HLD = NMAX + SSD_FUSED_HPAD;  // bf16 per carry-in row in LDS
  static constexpr int OFF_CS = 0;             // cs[128]
  static constexpr int OFF_W = 512;            // w[128] = exp(Lambda - cs) (times delta)
  static constexpr int OFF_CSC = 1024;         // csc[128]: cs as a column (source) index
  static constexpr int OFF_MISC = 1536;        // broadcast words
  static constexpr int OFF_X = 1600;           // x [128 s][FXLD]
  static constexpr int X_BYTES = FC * FXLD * 2;
  static constexpr int OFF_R = OFF_X + X_BYTES;     // B, then carry-in, then y
  static constexpr int B_BYTES = FC * BLD * 2;
  static constexpr int H_BYTES = 2 * 64 * HLD * 2;
  static constexpr int Y_BYTES = FC * FYLD * 4;
  static constexpr int R_BYTES = B_BYTES > H_BYTES ? (B_BYTES > Y_BYTES ? B_BYTES : Y_BYTES)
                                                  : (H_BYTES > Y_BYTES ? H_BYTES : Y_BYTES);
  static constexpr int LDS = OFF_R + R_BYTES;
};

}  // namespace

struct FusedArgs {
  Geo g;                  // 128-token chunk geometry; meta = the fused chunk table
  TArg x, B, C, dt, z, out;
  const float* A;
  const float* dt_bias;
  const float* D;
  const float* h0;
  float* hfinal;
  int softplus, clamp, input_dt;
  float dt_min, dt_max;
  int U, PS, R, nr;       // units, P slabs per head, chunks per range, ranges
  int nmax;               // d_state capacity (16 NT): row pitch of an aggregate
  // gated RMSNorm fused in (NULL: off): per (token, unit) sum of the squares
  // of the unit's gated outputs, [token][U] (P a multiple of 64)
  float* psum;
  unsigned long long* trace;  // per-item phase timestamps (SSD_FUSED_TRACE builds only)
  float* edec;            // [r * U + u] total decay of the range's aggregate
  float* agg;             // [r * U + u][64][NMAX] aggregates
};

// Phase timestamps, compiled in only with -DSSD_FUSED_TRACE (the profiling
// build of mamba_ssd_chunked_scan_amd/fused_trace.py): lane 0 of wave 0 of the
// item's workgroup stores the 100 MHz device clock (s_memrealtime) into slot
// `k` of the item's kFusedTraceSlots words.
#ifdef SSD_FUSED_TRACE
#define SSD_TRACE(k)                                                                   \
  do {                                                                                 \
    if (tid == 0 && a.trace)                                                           \
      a.trace[(size_t)(r * a.U + u) * kFusedTraceSlots + (k)] =                        \
          __builtin_amdgcn_s_memrealtime();                                            \
  } while (0)
// the aggregate launch's chunk steps: stamp m of step ks (first four steps)
#define SSD_TRACE_AGG(m)                                                               \
  do {                                                                                 \
    if (tid == 0 && a.trace && ks < 4)                                                 \
      a.trace[(size_t)(r * a.U + u) * kFusedTraceSlots + 32 + 6 * ks + (m)] =          \
          __builtin_amdgcn_s_memrealtime();                                            \
  } while (0)
#else
#define SSD_TRACE(k) \
  do {               \
  } while (0)
#define SSD_TRACE_AGG(m) \
  do {                   \
  } while (0)
#endif

template <typename TO, typename TDt, int NT>
__global__ __launch_bounds__(256, 2) void k_fused_fwd(FusedArgs a) {
  using Cfg = FCfg<NT>;
  constexpr int NMAX = Cfg::NMAX, NKB = Cfg::NKB, BV = Cfg::BV, BLD = Cfg::BLD, HLD = Cfg::HLD;
  __shared__ __align__(16) char smem[Cfg::LDS];
  float* s_cs = reinterpret_cast<float*>(smem + Cfg::OFF_CS);
  float* s_w = reinterpret_cast<float*>(smem + Cfg::OFF_W);
  float* s_csc = reinterpret_cast<float*>(smem + Cfg::OFF_CSC);
  uint32_t* s_misc = reinterpret_cast<uint32_t*>(smem + Cfg::OFF_MISC);
  bf16* s_x = reinterpret_cast<bf16*>(smem + Cfg::OFF_X);
  bf16* s_b = reinterpret_cast<bf16*>(smem + Cfg::OFF_R);
  bf16* s_hh = reinterpret_cast<bf16*>(smem + Cfg::OFF_R);
  bf16* s_hl = s_hh + 64 * HLD;
  float* s_y = reinterpret_cast<float*>(smem + Cfg::OFF_R);

  const Geo& g = a.g;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int r16 = lane % 16, q = lane / 16;

  // (unit, range) of this workgroup: with U a multiple of 8, XCD x (which
  // runs ids x, x + 8, ...) holds units [x U / 8, (x + 1) U / 8), range first
  int r, u;
  if (a.U % kNumXcd == 0) {
    const int qn = a.U / kNumXcd, per = a.nr * qn;
    const int it = xcd_remap((int)blockIdx.x, a.nr * a.U);
    const int xq = it / per, rem = it - xq * per;
    r = rem / qn;
    u = xq * qn + rem % qn;
  } else {
    r = (int)blockIdx.x / a.U;
    u = (int)blockIdx.x % a.U;
  }
#ifdef SSD_FUSED_TRACE
  if (tid == 0 && a.trace) {
    a.trace[(size_t)(r * a.U + u) * kFusedTraceSlots + kFusedTraceSlots - 1] =
        (unsigned long long)(__builtin_amdgcn_s_getreg((15 << 11) | 20) & 15u);
  }
#endif
  const int h = u / a.PS, p0 = (u % a.PS) * 64;
  const int grp = h / g.hpg;
  const int pw = min(64, g.P - p0);
  const int Kr = g.meta ? meta_word(g.meta, 0) : g.K;
  const int j0 = r * a.R, j1 = min(j0 + a.R, Kr);
  if (j0 >= j1) return;

  // this lane's column of the carried state: p = p0 + pl, n = 16 nt + 4 q + i
  const int pl = wave * 16 + r16;
  const bool p_ok = pl < pw;
  const int64_t PN = (int64_t)g.P * g.N;
  // uniform part of a state offset, and the per-lane part (this lane's row and
  // first column; recomputed at each use so that it is never held across the
  // loops)
  auto state_base = [&](int seq) { return ((int64_t)seq * g.H + h) * PN + (int64_t)p0 * g.N; };
  auto lane_off = [&]() {
    const int t = opaque_tid();
    return (uint32_t)((((t / kWave) * 16 + t % 16) * g.N) + (t % kWave) / 16 * 4);
  };
  // aggregate of range rr: uniform base, and this lane's offset in it
  auto slot_base = [&](int rr) { return a.agg + ((int64_t)rr * a.U + u) * 64 * NMAX; };
  auto slot_lane = [&]() {
    const int t = opaque_tid();
    return (uint32_t)(((t / kWave) * 16 + t % 16) * NMAX + (t % kWave) / 16 * 4);
  };
  auto load_h0 = [&](f32x4 (&v)[NT], int seq) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      v[nt] = zero4();
      if (a.h0 && p_ok && nt * 16 < g.N)
        v[nt] = *reinterpret_cast<const f32x4*>(at(a.h0 + state_base(seq), lane_off() + nt * 16));
    }
  };

  const float Ah2 = a.A[h] * 1.4426950408889634f;  // A_h in base-2 units
  const float Dh = a.D ? a.D[h] : 0.0f;
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
  // registers a chunk's x, B and dt are loaded into before they go to LDS:
  // 16-byte row pieces, 8 (x) or NMAX / 8 (B) consecutive threads per row
  struct Stage {
    u32x4 x[FXV], b[BV];
    // raw bits of dt (bf16 zero-extended, or fp32), converted only where the
    // cumsum uses them: converting at the load would make the wave wait for
    // the load, and with it for every load issued before it
    uint32_t dt[2];
  };
  u32x4 zr[FXV];

  // Tile loads: a uniform base pointer (the chunk's first row) plus a 32-bit
  // per-lane element offset (at most 127 rows of the tensor), so addresses
  // stay in scalar registers.
  // Tile geometry of the 16-byte row pieces: x, z and out rows hold 8 pieces
  // (64 columns), B rows NMAX / 8.  A full chunk with a full P slab and N ==
  // NMAX (the common case) needs no clamping: each lane computes one base
  // offset and every further piece adds a uniform stride.  Other chunks take
  // the clamped path.
  constexpr int BPR = NMAX / 8;           // B pieces per row
  constexpr int BROWS = 256 / BPR;        // B rows per pass of the workgroup
  const bool dims_full = pw == 64 && g.N == NMAX;
  auto x_offsets = [&](const Chunk& c, int64_t s1, uint32_t (&off)[FXV]) {
    const int tid = opaque_tid();
    const int row0 = tid / 8, col = (tid % 8) * 8;
    if (dims_full && c.len == FC) {
      const uint32_t o = (uint32_t)(row0 * s1 + col), step = (uint32_t)(32 * s1);
#pragma unroll
      for (int k = 0; k < FXV; ++k) off[k] = o + k * step;
    } else {
#pragma unroll
      for (int k = 0; k < FXV; ++k)
        off[k] = (uint32_t)(min(row0 + 32 * k, c.len - 1) * s1 + min(col, pw - 8));
    }
  };
  auto load_z = [&](const Chunk& c) {
    const bf16* base = row_ptr<bf16>(a.z, c.b, c.t0, h) + p0;
    uint32_t off[FXV];
    x_offsets(c, a.z.s1, off);
#pragma unroll
    for (int k = 0; k < FXV; ++k) zr[k] = *reinterpret_cast<const u32x4*>(at(base, off[k]));
  };
  // ---- issue every global load of chunk c (dt, x, B into st; z when gating).
  // dt goes first: its wait (for the cumsum) then covers no x or B load
  auto load_chunk = [&](Stage& st, const Chunk& c, bool with_z) {
    {
      // (every wave loads dt, though only wave 0 uses it: loads under a
      // branch would leave the compiler's wait counts conservative)
      const TDt* dbase = row_ptr<TDt>(a.dt, c.b, c.t0, h);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t off = (uint32_t)(min(2 * lane + e, c.len - 1) * a.dt.s1);
        st.dt[e] = raw_bits(*at(dbase, off));
      }
    }
    const bf16* xbase = row_ptr<bf16>(a.x, c.b, c.t0, h) + p0;
    {
      uint32_t off[FXV];
      x_offsets(c, a.x.s1, off);
#pragma unroll
      for (int k = 0; k < FXV; ++k) st.x[k] = *reinterpret_cast<const u32x4*>(at(xbase, off[k]));
    }
    const bf16* bbase = row_ptr<bf16>(a.B, c.b, c.t0, grp);
    {
      const int tid = opaque_tid();
      const int row0 = tid / BPR, col = (tid % BPR) * 8;
      uint32_t off[BV];
      if (dims_full && c.len == FC) {
        const uint32_t o = (uint32_t)(row0 * a.B.s1 + col), step = (uint32_t)(BROWS * a.B.s1);
#pragma unroll
        for (int k = 0; k < BV; ++k) off[k] = o + k * step;
      } else {
#pragma unroll
        for (int k = 0; k < BV; ++k)
          off[k] = (uint32_t)(min(row0 + BROWS * k, c.len - 1) * a.B.s1 + min(col, g.N - 8));
      }
#pragma unroll
      for (int k = 0; k < BV; ++k) st.b[k] = *reinterpret_cast<const u32x4*>(at(bbase, off[k]));
    }
    if (with_z && a.z.p) load_z(c);
  };

  // ---- LDS: cumsum, decay weights, and x and B in their natural row-major
  // layout (tokens x columns).  Tokens past the chunk's end (loaded as copies
  // of its last token), columns past P and past N are zeroed here.
  // Within-chunk cumsum by wave 0, branch-free: lane l holds positions 2l and
  // 2l + 1.  fp32 with a DPP wave scan (the bf16 inputs of this path leave
  // ample room for fp32 rounding of cs; no LDS round trips).  softplus as
  // softplus_fast (hardware exp/log, log1p corrected).  The cumsum is
  // kept in base-2 units (cs * log2 e), so every decay factor below is one
  // hardware 2^x of a difference.
  auto stage_cs = [&](const Stage& st, const Chunk& c) {
    if (wave == 0) {
      float av[2], dv[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float uu = from_bits<TDt>(st.dt[e]) + bias;
        float d = uu;
        if (a.softplus) d = softplus_fast(uu);
        if (a.clamp) d = fminf(fmaxf(d, a.dt_min), a.dt_max);
        const bool in = 2 * lane + e < c.len;
        av[e] = in ? d * Ah2 : 0.0f;
        dv[e] = in && a.input_dt ? d : 1.0f;
      }
      const float pair = av[0] + av[1];
      const float incl = wave_inclusive_sum_dpp(pair);
      const float c0 = incl - pair + av[0], c1 = incl;
      s_cs[2 * lane] = c0;
      s_cs[2 * lane + 1] = c1;
      const int ll = c.len - 1;
      const float lam = __int_as_float(
          __builtin_amdgcn_readlane(__float_as_int((ll & 1) ? c1 : c0), ll >> 1));
      s_w[2 * lane] = 2 * lane < c.len ? fast_exp2(lam - c0) * dv[0] : 0.0f;
      s_w[2 * lane + 1] = 2 * lane + 1 < c.len ? fast_exp2(lam - c1) * dv[1] : 0.0f;
      // the source side of the decay exponent: with the step size on the input
      // term, exp2(cs_l - cs_s) delta_s = exp2(cs_l - (cs_s - log2 delta_s))
      // (delta >= 0 here; log2(0) = -inf gives the weight 0)
      s_csc[2 * lane] = a.input_dt ? c0 - __log2f(dv[0]) : c0;
      s_csc[2 * lane + 1] = a.input_dt ? c1 - __log2f(dv[1]) : c1;
      if (lane == 0) s_misc[1] = __float_as_uint(lam);
    }
  };
  auto stage_xb = [&](const Stage& st, const Chunk& c) {
    const int tid = opaque_tid();
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const int xrow = tid / 8, xcol = (tid % 8) * 8;
    const int brow = tid / BPR, bcol = (tid % BPR) * 8;
    bf16* xd = &s_x[xrow * FXLD + xcol];
    bf16* bd = &s_b[brow * BLD + bcol];
    if (dims_full && c.len == FC) {
#pragma unroll
      for (int k = 0; k < FXV; ++k) *reinterpret_cast<u32x4*>(xd + 32 * k * FXLD) = st.x[k];
#pragma unroll
      for (int k = 0; k < BV; ++k) *reinterpret_cast<u32x4*>(bd + BROWS * k * BLD) = st.b[k];
    } else {
#pragma unroll
      for (int k = 0; k < FXV; ++k)
        *reinterpret_cast<u32x4*>(xd + 32 * k * FXLD) =
            (xrow + 32 * k < c.len && xcol < pw) ? st.x[k] : zero;
#pragma unroll
      for (int k = 0; k < BV; ++k)
        *reinterpret_cast<u32x4*>(bd + BROWS * k * BLD) =
            (brow + BROWS * k < c.len && bcol < g.N) ? st.b[k] : zero;
    }
  };

  // ---- acc += S_j^T = B^T (w x): wave w owns p-tile w, all n-tiles.  Both
  // operands come from the natural-layout tiles through transpose reads.
  auto state_mma = [&](f32x4 (&acc)[NT]) {
#pragma unroll
    for (int kb = 0; kb < FC / 32; ++kb) {
      const int k0 = kb * 32 + q * 8;  // this lane group's 8 tokens
      const u32x4 xv = __builtin_bit_cast(u32x4, lds_frag_tr(s_x, FXLD, k0, k0 + 4, wave * 16));
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(&s_w[k0]);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(&s_w[k0 + 4]);
      f32x8 xw;
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        xw[2 * d] = bf16_lo_f32(xv[d]) * w0[2 * d];
        xw[2 * d + 1] = bf16_hi_f32(xv[d]) * w0[2 * d + 1];
        xw[4 + 2 * d] = bf16_lo_f32(xv[2 + d]) * w1[2 * d];
        xw[4 + 2 * d + 1] = bf16_hi_f32(xv[2 + d]) * w1[2 * d + 1];
      }
      const FragSplit b = split_f32x8(xw);
      // the B fragments in groups of SG, each group read before its products
      // (one LDS round trip per group instead of one per n-tile)
      constexpr int SG = SSD_FUSED_SG < NT ? SSD_FUSED_SG : NT;
#pragma unroll
      for (int n0 = 0; n0 < NT; n0 += SG) {
        FragBF bt[SG];
#pragma unroll
        for (int i = 0; i < SG; ++i) bt[i].v = lds_frag_tr(s_b, BLD, k0, k0 + 4, (n0 + i) * 16);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < SG; ++i) mma(acc[n0 + i], bt[i], b);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- sequence structure of the range
  Chunk cfirst;
  get_chunk(g, j0, cfirst);
  int f0, l0;
  seq_chunks(g, cfirst.seq, f0, l0);
  const bool need_fold = f0 < j0;        // the first chunk continues a sequence

  f32x4 carry[NT];

  SSD_TRACE(2);

  // ---- carry-in: the state the preceding range ends with, left in its
  // aggregate slot by the carry launch (which has ended, so nothing is waited
  // for)
  if (need_fold) {
    const float* src = slot_base(r - 1);
    const uint32_t lo = slot_lane();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) carry[nt] = *reinterpret_cast<const f32x4*>(at(src, lo + nt * 16));
  }
  // the first chunk's loads (after the carry-in's: a wait for that then
  // covers none of these)
  Chunk c;
  get_chunk(g, j0, c);
  Stage st;
  load_chunk(st, c, false);

  SSD_TRACE(3);
  // ---- the outputs, chunk by chunk.  Per chunk:
  //   A  the carry-in H_j (the initial state at a sequence's first chunk,
  //      loaded during the previous chunk) to LDS as bf16 hi + lo (the cumsum
  //      was staged at the end of the previous chunk)
  //   B  Y_off = exp(cs_l) C_l . H_j
  //   C  x and B tiles to LDS; this chunk's z and the next chunk's x, B, dt
  //      loads go out
  //   D  carry = exp(Lambda) carry + S_j (accumulated in place); per s-tile
  //      pair, C.B^T tiles -> M (+ D on the diagonal) -> Y_diag; the next
  //      chunk's C fragments go out
  //   E  y through LDS; gate, store; the next chunk's cumsum
  const int ltA = wave, ltB = 7 - wave;   // this wave's l-tiles
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 cfr[2][NKB];
  auto load_cfr = [&](const Chunk& cc) {
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int lrow = (ui ? ltB : ltA) * 16 + r16;
      const bf16* cbase = row_ptr<bf16>(a.C, cc.b, cc.t0, grp);
      const uint32_t roff = (uint32_t)(min(lrow, cc.len - 1) * a.C.s1);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        cfr[ui][kb] = *reinterpret_cast<const u32x4*>(
            at(cbase, roff + (uint32_t)min(kb * 32 + q * 8, g.N - 8)));
    }
  };
  int fj, lj;  // the current chunk's sequence: chunks [fj, lj)
  seq_chunks(g, c.seq, fj, lj);
  if (fj == j0) load_h0(carry, c.seq);  // (before the C fragments, as below)
  load_cfr(c);
  stage_cs(st, c);
  for (int j = j0; j < j1; ++j) {
    // ---- A
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      uint2 hi, lo;
      split_pair(carry[nt][0], carry[nt][1], hi.x, lo.x);
      split_pair(carry[nt][2], carry[nt][3], hi.y, lo.y);
      *reinterpret_cast<uint2*>(&s_hh[pl * HLD + nt * 16 + q * 4]) = hi;
      *reinterpret_cast<uint2*>(&s_hl[pl * HLD + nt * 16 + q * 4]) = lo;
    }
    // C rows past the chunk and columns past N contribute nothing
    if (!(dims_full && c.len == FC)) {
#pragma unroll
      for (int ui = 0; ui < 2; ++ui) {
        const bool lok = (ui ? ltB : ltA) * 16 + r16 < c.len;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          cfr[ui][kb] = (lok && kb * 32 + q * 8 < g.N) ? cfr[ui][kb] : zero;
      }
    }
    __syncthreads();

    const int kk = j - j0;  // (phase stamps of the profiling build)
    if (kk < 4) SSD_TRACE(4 + 5 * kk);
    // ---- B  (each carry-in fragment is read from LDS once and serves both
    // l-tiles)
    f32x4 acc[2][4];
#pragma unroll
    for (int ui = 0; ui < 2; ++ui)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) acc[ui][pt] = zero4();
    // The matrix phases (B and D) run at raised wave priority: the SIMD's
    // other wave, from another workgroup, is then more often in its VALU,
    // LDS or load phases while this one keeps the matrix unit fed (measured
    // 2.5% faster at the Nemotron-Nano size).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      FragBF cf0, cf1;
      cf0.v = __builtin_bit_cast(bf16x8, cfr[0][kb]);
      cf1.v = __builtin_bit_cast(bf16x8, cfr[1][kb]);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        FragSplit hs;
        hs.hi = *reinterpret_cast<const bf16x8*>(&s_hh[(pt * 16 + r16) * HLD + kb * 32 + q * 8]);
        hs.lo = *reinterpret_cast<const bf16x8*>(&s_hl[(pt * 16 + r16) * HLD + kb * 32 + q * 8]);
        mma(acc[0][pt], cf0, hs);
        mma(acc[1][pt], cf1, hs);
      }
      // keep the scheduler from hoisting every k-block's reads at once
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int lt = ui ? ltB : ltA;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ex = fast_exp2(s_cs[lt * 16 + q * 4 + i]);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[ui][pt][i] *= ex;
      }
    }
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();  // the carry-in rows are dead: the B tile takes their space
    if (kk < 4) SSD_TRACE(5 + 5 * kk);

    // ---- C
    stage_xb(st, c);
    // Loads complete in issue order as far as the wait counter is concerned, so
    // z (needed in this chunk's epilogue) goes out before the next chunk's x,
    // B and dt (needed one chunk later): waiting for z then never waits for
    // the prefetch.
    if (a.z.p) load_z(c);
    Chunk cn = c;
    int fn = fj, ln = lj;
    const bool more = j + 1 < j1;
    if (more) {
      get_chunk(g, j + 1, cn);
      if (cn.seq != c.seq) seq_chunks(g, cn.seq, fn, ln);
    }
    load_chunk(st, cn, false);  // unconditional (past the range it reloads the last chunk)
    __syncthreads();

    if (kk < 4) SSD_TRACE(6 + 5 * kk);
    // ---- D
    const float e = fast_exp2(__uint_as_float(s_misc[1]));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) carry[nt] *= e;
    __builtin_amdgcn_s_setprio(1);
    state_mma(carry);
    if (j == lj - 1 && a.hfinal && p_ok) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        if (nt * 16 < g.N)
          *reinterpret_cast<f32x4*>(at(a.hfinal + state_base(c.seq), lane_off() + nt * 16)) = carry[nt];
    }
    // Y_diag = (L o C.B^T + D I) x, one s-tile pair (kp) at a time; the
    // diagonal pair (the last) masks s > l and adds the skip D on s == l.
    // Rows past the chunk compute finite or discarded values: the epilogue
    // never stores them.  (A separate unmasked loop for the pairs below the
    // diagonal measured slower: its extra code costs more registers than the
    // selects it saves.)
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int lt = ui ? ltB : ltA;
      const int lrow = lt * 16 + r16;
      const float csl = s_cs[lrow];
      for (int kp = 0; kp <= lt / 2; ++kp) {
        const bool diag = kp == lt / 2;
        // C.B^T tiles (s-tile sa / sb, l-tile lt): B rows (n contiguous) from
        // the B tile as the A operand, the C fragments as the B operand
        const int sa = 2 * kp, sb = 2 * kp + 1;
        f32x4 va = zero4(), vb = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          FragBF ba, bb, cf;
          ba.v = *reinterpret_cast<const bf16x8*>(&s_b[(sa * 16 + r16) * BLD + kb * 32 + q * 8]);
          bb.v = *reinterpret_cast<const bf16x8*>(&s_b[(sb * 16 + r16) * BLD + kb * 32 + q * 8]);
          cf.v = __builtin_bit_cast(bf16x8, cfr[ui][kb]);
          mma(va, ba, cf);
          mma(vb, bb, cf);
        }
        // M in the accumulator layout (lane: one l, tokens 4 q + 0..3 of each
        // s-tile), used as the A operand with the tokens in that order; x is
        // read from the x tile in the same order
        const f32x4 csa = *reinterpret_cast<const f32x4*>(&s_csc[sa * 16 + q * 4]);
        const f32x4 csb = *reinterpret_cast<const f32x4*>(&s_csc[sb * 16 + q * 4]);
        f32x8 m;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const float ma = fast_exp2(csl - csa[e4]) * va[e4];
          const float mb = fast_exp2(csl - csb[e4]) * vb[e4];
          if (diag) {
            const int s_a = sa * 16 + q * 4 + e4, s_b2 = sb * 16 + q * 4 + e4;
            m[e4] = s_a < lrow ? ma : (s_a == lrow ? ma + Dh : 0.0f);
            m[4 + e4] = s_b2 < lrow ? mb : (s_b2 == lrow ? mb + Dh : 0.0f);
          } else {
            m[e4] = ma;
            m[4 + e4] = mb;
          }
        }
        const FragSplit mf = split_f32x8(m);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          FragBF xf;
          xf.v = lds_frag_tr(s_x, FXLD, sa * 16 + q * 4, sb * 16 + q * 4, pt * 16);
          mma(acc[ui][pt], mf, xf);
        }
      }
    }
    // A sequence that starts at the next chunk starts from its initial
    // state (carry is dead here: its final state was stored above).  Issued
    // before the C fragments, so that waiting for it does not wait for them.
    __builtin_amdgcn_s_setprio(0);
    if (more && fn == j + 1) load_h0(carry, cn.seq);
    load_cfr(cn);  // unconditional (past the range it reloads the last chunk)
    __syncthreads();  // the B tile is dead: its space takes y
    if (kk < 4) SSD_TRACE(7 + 5 * kk);

    // ---- E
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int lt = ui ? ltB : ltA;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s_y[(lt * 16 + q * 4 + i) * FYLD + pt * 16 + r16] = acc[ui][pt][i];
    }
    __syncthreads();
    // The next chunk's cumsum (cs is free: nothing reads it after the matrix
    // phase) goes before the stores below, whose completion a later wait for
    // its dt would also wait for.  Past the range's end it stages this chunk
    // again, unused.
    stage_cs(st, cn);
    TO* obase = row_ptr_mut<TO>(a.out, c.b, c.t0, h) + p0;
    const int etid = opaque_tid();
    const int erow = etid / 8, ecol = (etid % 8) * 8;
    const uint32_t eoff = (uint32_t)(erow * a.out.s1 + ecol), estep = (uint32_t)(32 * a.out.s1);
    const bool efull = dims_full && c.len == FC;
#pragma unroll
    for (int k = 0; k < FXV; ++k) {
      // computed for every row (rows past the chunk hold finite values), only
      // the store is conditional: straight-line code keeps the waits precise
      const int l = erow + 32 * k, pp = ecol;
      f32x8 y = Vec8<float>::load(s_y + l * FYLD + pp);
      if (a.z.p) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          y[2 * d] *= silu(bf16_lo_f32(zr[k][d]));
          y[2 * d + 1] *= silu(bf16_hi_f32(zr[k][d]));
        }
      }
      if (efull || (l < c.len && pp < pw)) Vec8<TO>::store(at(obase, eoff + k * estep), y);
      if (a.psum) {
        // the gated RMSNorm after the scan: sum(g^2) of this row's 64
        // channels (8 lanes of 8), one partial per (token, 64-channel block)
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += y[i] * y[i];
        ss = (l < c.len && pp < pw) ? ss : 0.0f;
        ss += __shfl_xor(ss, 1, kWave);
        ss += __shfl_xor(ss, 2, kWave);
        ss += __shfl_xor(ss, 4, kWave);
        if (ecol == 0 && l < c.len)
          a.psum[((int64_t)c.b * g.T + c.t0 + l) * a.U + u] = ss;
      }
    }
    c = cn;
    fj = fn;
    lj = ln;
    __syncthreads();  // y and x are dead before the next chunk's staging
    if (kk < 4) SSD_TRACE(8 + 5 * kk);
    else if (kk < 10) SSD_TRACE(24 + (kk - 4));
  }
  SSD_TRACE(kFusedTraceSlots - 2);
}

// Builds the 128-token chunk table of a packed batch and writes the final
// state of every sequence without tokens (launched only when there is one of
// the two to do).
__global__ __launch_bounds__(256) void k_fused_prep(Geo g, const int32_t* cu, int32_t* meta,
                                                    const float* h0, float* hfinal) {
  __shared__ int lds_waves[4];
  const int bid = blockIdx.x;
  if (bid == 0) {
    if (cu) varlen_meta_block(cu, g.nseq, g.T, g.C, g.K, meta, lds_waves);
    return;
  }
  const int seq = bid - 1;
  bool empty;
  if (cu) {
    int st, L;
    seq_span(cu, seq, g.T, st, L);
    empty = L == 0;
  } else {
    empty = g.T == 0;
  }
  if (!empty) return;
  const int64_t n = (int64_t)g.H * g.P * g.N;
  float* dst = hfinal + (int64_t)seq * n;
  const float* src = h0 ? h0 + (int64_t)seq * n : nullptr;
  for (int64_t i = threadIdx.x; i < n; i += 256) dst[i] = src ? src[i] : 0.0f;
}

// ---- The aggregate launch: one workgroup of 4 waves per (unit, range).  It
// sums its range's chunks into one state, exactly what the output launch's own
// recurrence would carry across the range: carry = exp(Lambda_j) carry + S_j
// from a zero state (or from the sequence's initial state when it starts
// inside the range), S_j = sum_s exp(Lambda_j - cs_s) x_s (outer) B_s (SSD
// Reference, "Intra-chunk outputs and per-chunk states").  Wave w owns rows
// p-tile w and every d_state column.  Each wave computes the chunk's cumsum
// and decay weights itself (no wave waits for another's), x and B go through
// LDS, and the chunk state is the product B^T (w x) on the matrix cores with
// the decay-weighted x split into bf16 hi + lo (each element split once).  Two
// register sets alternate, so chunk j + 2 is in flight while chunk j is
// multiplied.  Measured at the Nemotron-Nano size: this shape, at two
// workgroups per CU, is faster than eight waves per workgroup (each wave half
// the columns: every x element split twice) and than d_state split across
// workgroups at three or four per CU.
constexpr int kAggThreads = 256;
template <typename TDt, int NT>
__global__ __launch_bounds__(kAggThreads, 2) void k_fused_agg(FusedArgs a) {
  constexpr int NMAX = 16 * NT;
  constexpr int NTS = NT;                 // n-tiles per wave
  constexpr int XLD = 64 + SSD_FUSED_XPAD;  // bf16 per x row in LDS
  constexpr int BLD = NMAX + SSD_FUSED_BPAD;  // bf16 per B row in LDS
  constexpr int XV = FC * 8 / kAggThreads;  // 16-byte x pieces per thread
  constexpr int BPR = NMAX / 8;           // 16-byte pieces per B row
  constexpr int BROWS = kAggThreads / BPR;  // B rows per pass of the workgroup
  constexpr int BV = FC / BROWS;          // B pieces per thread
  constexpr int NW = kAggThreads / kWave;
  __shared__ __align__(16) bf16 s_x[FC * XLD];
  __shared__ __align__(16) bf16 s_b[FC * BLD];
  __shared__ __align__(16) float s_w[NW][FC];
  __shared__ __align__(16) uint32_t s_dt[FC];

  const Geo& g = a.g;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int r16 = lane % 16, q = lane / 16;
  const int pt = wave, nh = 0;

  // (unit, range): XCD x holds units [x U / 8, (x + 1) U / 8), range first
  int r, u;
  if (a.U % kNumXcd == 0) {
    const int qn = a.U / kNumXcd, per = a.nr * qn;
    const int it = xcd_remap((int)blockIdx.x, a.nr * a.U);
    const int xq = it / per, rem = it - xq * per;
    r = rem / qn;
    u = xq * qn + rem % qn;
  } else {
    r = (int)blockIdx.x / a.U;
    u = (int)blockIdx.x % a.U;
  }
  const int h = u / a.PS, p0 = (u % a.PS) * 64;
  const int grp = h / g.hpg;
  const int pw = min(64, g.P - p0);
  const int Kr = g.meta ? meta_word(g.meta, 0) : g.K;
  const int j0 = r * a.R, j1 = min(j0 + a.R, Kr);
  if (j0 >= j1) return;
  Chunk clast;
  get_chunk(g, j1 - 1, clast);
  int fs, ls;
  seq_chunks(g, clast.seq, fs, ls);
  if (!(j1 < ls)) return;                  // the next range does not continue it
  const bool reset = fs >= j0;             // the last sequence starts inside the range
#ifdef SSD_FUSED_TRACE
  if (tid == 0 && a.trace)
    a.trace[(size_t)(r * a.U + u) * kFusedTraceSlots + 0] = __builtin_amdgcn_s_memrealtime();
#endif

  const int pl = pt * 16 + r16;           // this lane's state row (p0 + pl)
  const int64_t PN = (int64_t)g.P * g.N;
  f32x4 carry[NTS];
#pragma unroll
  for (int nt = 0; nt < NTS; ++nt) {
    const int n = (nh * NTS + nt) * 16;
    carry[nt] = zero4();
    if (reset && a.h0 && pl < pw && n < g.N)
      carry[nt] = *reinterpret_cast<const f32x4*>(
          a.h0 + ((int64_t)clast.seq * g.H + h) * PN + (int64_t)(p0 + pl) * g.N + n + q * 4);
  }
  const float Ah2 = a.A[h] * 1.4426950408889634f;
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;

  struct Stage {
    u32x4 x[XV], b[BV];
    uint32_t dt;            // raw bits of token (thread % 128)'s dt
  };
  const bool dims_full = pw == 64 && g.N == NMAX;
  // Offsets are 32-bit element counts on a uniform base (scalar-base loads);
  // dt goes last, so that no address register of the x and B loads is ever
  // paired with a pending dt load (which would make the wave wait for it, and
  // with it for every older load: the prefetch would be lost).
  const uint32_t xs1 = (uint32_t)a.x.s1, bs1 = (uint32_t)a.B.s1, ds1 = (uint32_t)a.dt.s1;
  auto load = [&](Stage& st, const Chunk& c) {
    const int t = opaque_tid();
    const bf16* xbase = row_ptr<bf16>(a.x, c.b, c.t0, h) + p0;
    const uint32_t xrow = (uint32_t)t / 8, xcol = ((uint32_t)t % 8) * 8;
    const bf16* bbase = row_ptr<bf16>(a.B, c.b, c.t0, grp);
    const uint32_t brow = (uint32_t)t / BPR, bcol = ((uint32_t)t % BPR) * 8;
    constexpr uint32_t XROWS = kAggThreads / 8;
    if (dims_full && c.len == FC) {
      const uint32_t xo = xrow * xs1 + xcol, bo = brow * bs1 + bcol;
#pragma unroll
      for (int k = 0; k < XV; ++k)
        st.x[k] = *reinterpret_cast<const u32x4*>(at(xbase, xo + (uint32_t)k * XROWS * xs1));
#pragma unroll
      for (int k = 0; k < BV; ++k)
        st.b[k] = *reinterpret_cast<const u32x4*>(at(bbase, bo + (uint32_t)k * BROWS * bs1));
    } else {
      const uint32_t lm = (uint32_t)c.len - 1;
      const uint32_t xc = min(xcol, (uint32_t)pw - 8), bc = min(bcol, (uint32_t)g.N - 8);
#pragma unroll
      for (int k = 0; k < XV; ++k)
        st.x[k] = *reinterpret_cast<const u32x4*>(
            at(xbase, min(xrow + (uint32_t)k * XROWS, lm) * xs1 + xc));
#pragma unroll
      for (int k = 0; k < BV; ++k)
        st.b[k] = *reinterpret_cast<const u32x4*>(
            at(bbase, min(brow + (uint32_t)k * BROWS, lm) * bs1 + bc));
    }
    // dt travels with x and B (through LDS): it is consumed where they are,
    // so no load of it is ever waited for on its own
    const TDt* dbase = row_ptr<TDt>(a.dt, c.b, c.t0, h);
    st.dt = raw_bits(*at(dbase, min((uint32_t)t % FC, (uint32_t)c.len - 1) * ds1));
  };
  auto stage = [&](const Stage& st, const Chunk& c) {
    const int t = opaque_tid();
    const u32x4 zero = {0u, 0u, 0u, 0u};
    constexpr int XROWS = kAggThreads / 8;
    const int xrow = t / 8, xcol = (t % 8) * 8;
    const int brow = t / BPR, bcol = (t % BPR) * 8;
#pragma unroll
    for (int k = 0; k < XV; ++k)
      *reinterpret_cast<u32x4*>(&s_x[(xrow + XROWS * k) * XLD + xcol]) =
          (xrow + XROWS * k < c.len && xcol < pw) ? st.x[k] : zero;
#pragma unroll
    for (int k = 0; k < BV; ++k)
      *reinterpret_cast<u32x4*>(&s_b[(brow + BROWS * k) * BLD + bcol]) =
          (brow + BROWS * k < c.len && bcol < g.N) ? st.b[k] : zero;
    if (t < FC) s_dt[t] = st.dt;
  };
  // every wave: the chunk's decay weights into its own row of s_w; returns
  // the chunk's total log-decay (base 2)
  auto weights = [&](const Chunk& c) {
    float av[2], dv[2];
    const uint2 draw = *reinterpret_cast<const uint2*>(&s_dt[2 * lane]);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float uu = from_bits<TDt>(e ? draw.y : draw.x) + bias;
      float d = a.softplus ? softplus_fast(uu) : uu;
      if (a.clamp) d = fminf(fmaxf(d, a.dt_min), a.dt_max);
      const bool in = 2 * lane + e < c.len;
      av[e] = in ? d * Ah2 : 0.0f;
      dv[e] = in && a.input_dt ? d : 1.0f;
    }
    const float pair = av[0] + av[1];
    const float incl = wave_inclusive_sum_dpp(pair);
    const float c0 = incl - pair + av[0], c1 = incl;
    const int ll = c.len - 1;
    const float lam = __int_as_float(
        __builtin_amdgcn_readlane(__float_as_int((ll & 1) ? c1 : c0), ll >> 1));
    s_w[wave][2 * lane] = 2 * lane < c.len ? fast_exp2(lam - c0) * dv[0] : 0.0f;
    s_w[wave][2 * lane + 1] = 2 * lane + 1 < c.len ? fast_exp2(lam - c1) * dv[1] : 0.0f;
    return lam;
  };
  auto state_mma = [&]() {
#pragma unroll
    for (int kb = 0; kb < FC / 32; ++kb) {
      const int k0 = kb * 32 + q * 8;
      const u32x4 xv = __builtin_bit_cast(u32x4, lds_frag_tr(s_x, XLD, k0, k0 + 4, pt * 16));
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(&s_w[wave][k0]);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(&s_w[wave][k0 + 4]);
      f32x8 xw;
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        xw[2 * d] = bf16_lo_f32(xv[d]) * w0[2 * d];
        xw[2 * d + 1] = bf16_hi_f32(xv[d]) * w0[2 * d + 1];
        xw[4 + 2 * d] = bf16_lo_f32(xv[2 + d]) * w1[2 * d];
        xw[4 + 2 * d + 1] = bf16_hi_f32(xv[2 + d]) * w1[2 * d + 1];
      }
      // every B fragment of the k-block is read before the first product:
      // one LDS round trip per k-block instead of one per n-tile
      FragBF bt[NTS];
#pragma unroll
      for (int nt = 0; nt < NTS; ++nt) bt[nt].v = lds_frag_tr(s_b, BLD, k0, k0 + 4, (nh * NTS + nt) * 16);
      const FragSplit b = split_f32x8(xw);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < NTS; ++nt) mma(carry[nt], bt[nt], b);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int js = reset ? fs : j0;
  float E = 1.0f;
  Stage sa, sb;
  Chunk ca, cb;
  get_chunk(g, js, ca);
  load(sa, ca);
  get_chunk(g, min(js + 1, j1 - 1), cb);
  load(sb, cb);
#ifdef SSD_FUSED_TRACE
  int ks = 0;  // (the profiling build's step count)
#endif
  auto step = [&](Stage& st, Chunk& c, int j) {
    __syncthreads();  // every wave is done with the previous chunk's tiles
    SSD_TRACE_AGG(0);
    stage(st, c);
    SSD_TRACE_AGG(1);
    const Chunk cur = c;
    get_chunk(g, min(j + 2, j1 - 1), c);  // refill with chunk j + 2 (or the last, unused)
    load(st, c);
    SSD_TRACE_AGG(2);
    __syncthreads();
    SSD_TRACE_AGG(3);
    const float lam = weights(cur);
    SSD_TRACE_AGG(4);
    const float e = fast_exp2(lam);
#pragma unroll
    for (int nt = 0; nt < NTS; ++nt) carry[nt] *= e;
    E *= e;
    state_mma();
    SSD_TRACE_AGG(5);
#ifdef SSD_FUSED_TRACE
    ++ks;
#endif
  };
  // whole pairs, then an odd last chunk: the loop is only ever re-entered
  // after the second register set's step, so the wait counts at its head are
  // exact (with the second step conditional inside the loop, the compiler
  // drains every load there and the prefetch is lost)
  int j = js;
  for (; j + 1 < j1; j += 2) {
    step(sa, ca, j);
    step(sb, cb, j + 1);
  }
  if (j < j1) step(sa, ca, j);
  if (pl < pw) {
    float* dst = a.agg + ((int64_t)r * a.U + u) * 64 * NMAX + (int64_t)pl * NMAX + q * 4;
#pragma unroll
    for (int nt = 0; nt < NTS; ++nt) {
      const int n = (nh * NTS + nt) * 16;
      if (n < g.N) *reinterpret_cast<f32x4*>(dst + n) = carry[nt];
    }
  }
  if (tid == 0) a.edec[r * a.U + u] = E;
#ifdef SSD_FUSED_TRACE
  if (tid == 0 && a.trace)
    a.trace[(size_t)(r * a.U + u) * kFusedTraceSlots + 1] = __builtin_amdgcn_s_memrealtime();
#endif
}

// ---- The carry launch: per unit, the ranges in order replace each stored
// aggregate by the state at the end of its range (of the range's last
// sequence, the one that continues into the next range): the aggregate itself
// where that sequence starts inside the range (its aggregate already starts
// from the sequence's initial state), else E times the state the previous
// range ends with plus the aggregate -- the inter-chunk propagation of the SSD
// Reference ("Inter-chunk propagation") taken a whole range at a time.  Each
// thread owns four consecutive words of one unit's 64 x NMAX state; kCarryBatch
// slots are loaded before the first of them is combined.  Unit u runs on the
// XCD whose L2 holds its aggregates (the aggregate launch's placement).
template <int NT>
__global__ __launch_bounds__(256) void k_fused_carry(FusedArgs a) {
  constexpr int NMAX = 16 * NT;
  constexpr int PIECES = 64 * NMAX / 4;  // f32x4 pieces of one state
  constexpr int WPU = PIECES / 256;      // workgroups per unit
  static_assert(PIECES % 256 == 0, "a unit's state fills whole workgroups");
  const Geo& g = a.g;
  const int total = a.U * WPU;
  const int it = a.U % kNumXcd == 0 ? xcd_remap((int)blockIdx.x, total) : (int)blockIdx.x;
  const int u = it / WPU;
  const uint32_t off = (uint32_t)((it % WPU) * 256 + (int)threadIdx.x) * 4;
  const int Kr = g.meta ? meta_word(g.meta, 0) : g.K;
  const int nlast = a.nr - 1;  // the last range hands nothing on
  f32x4 prev = zero4();
  for (int b = 0; b < nlast; b += kCarryBatch) {
    // which slots take over the previous range's state: those of ranges
    // whose last sequence continues into the next range (they have an
    // aggregate) and came in from the previous range
    bool take[kCarryBatch];
#pragma unroll
    for (int m = 0; m < kCarryBatch; ++m) {
      const int rr = b + m;
      const int j0 = rr * a.R, j1 = min(j0 + a.R, Kr);
      take[m] = false;
      if (rr < nlast && j0 < j1) {
        Chunk clast;
        get_chunk(g, j1 - 1, clast);
        int fs, ls;
        seq_chunks(g, clast.seq, fs, ls);
        take[m] = j1 < ls && fs < j0;
      }
    }
    // (slots past the last one repeat it, unused: loads under a branch would
    // leave the compiler's wait counts conservative)
    f32x4 v[kCarryBatch];
    float e[kCarryBatch];
#pragma unroll
    for (int m = 0; m < kCarryBatch; ++m) {
      const int rm = min(b + m, nlast - 1);
      v[m] = *reinterpret_cast<const f32x4*>(
          at(a.agg + ((int64_t)rm * a.U + u) * 64 * NMAX, off));
      e[m] = a.edec[rm * a.U + u];
    }
    // where a sequence starts inside a range, its slot already holds the end
    // state (or is never read)
#pragma unroll
    for (int m = 0; m < kCarryBatch; ++m) {
      if (take[m]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[m][i] = fmaf(e[m], prev[i], v[m][i]);
        *reinterpret_cast<f32x4*>(at(a.agg + ((int64_t)(b + m) * a.U + u) * 64 * NMAX, off)) =
            v[m];
      }
      prev = v[m];
    }
  }
}

FusedPlan fused_plan(int64_t K, int H, int P, int N) {
  FusedPlan pl;
  pl.PS = (P + 63) / 64;
  pl.U = H * pl.PS;
  pl.NT = N <= 32 ? 2 : (N <= 64 ? 4 : 8);
  if (K <= 0) {
    pl.R = 1;
    pl.nr = 0;
    return pl;
  }
  int64_t nr = kFusedTargetWorkgroups / pl.U;
  nr = nr < 1 ? 1 : (nr > K ? K : nr);
  pl.R = (int)((K + nr - 1) / nr);
  pl.nr = (int)((K + pl.R - 1) / pl.R);
  return pl;
}

hipError_t launch_fused_fwd(const FusedLaunch& f, hipStream_t s) {
  const Geo& g = f.g;
  const FusedPlan& pl = f.plan;
  // the chunk table (packed mode), and final states of sequences without
  // tokens (only packed mode, or a batch without tokens, has any)
  if (f.cu || g.T == 0) {
    const int nfinal = f.hfinal ? g.nseq : 0;
    hipLaunchKernelGGL(k_fused_prep, dim3(1 + nfinal), dim3(256), 0, s, g, f.cu, f.meta, f.h0,
                       f.hfinal);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (pl.nr == 0) return hipSuccess;

  FusedArgs a;
  a.g = g;
  a.x = f.x; a.B = f.B; a.C = f.C; a.dt = f.dt; a.z = f.z; a.out = f.out;
  a.A = f.A; a.dt_bias = f.dt_bias; a.D = f.D; a.h0 = f.h0; a.hfinal = f.hfinal;
  a.softplus = f.softplus; a.clamp = f.clamp; a.dt_min = f.dt_min; a.dt_max = f.dt_max;
  a.input_dt = f.input_dt;
  a.U = pl.U; a.PS = pl.PS; a.R = pl.R; a.nr = pl.nr;
  a.edec = f.edec; a.agg = f.agg;
  a.psum = f.psum;
  a.trace = f.trace;
  const dim3 grid((unsigned)(pl.nr * pl.U));
  const bool ob = f.out_dtype == DT_BF16, db = f.dt_dtype == DT_BF16;
  a.nmax = 16 * pl.NT;
  // the aggregate launch (only when some range hands a state to the next)
  if (pl.nr > 1) {
#define SSD_FUSED_AGG(NT)                                                                    \
  do {                                                                                       \
    if (db) hipLaunchKernelGGL((k_fused_agg<bf16, NT>), grid, dim3(kAggThreads), 0, s, a);   \
    else hipLaunchKernelGGL((k_fused_agg<float, NT>), grid, dim3(kAggThreads), 0, s, a);     \
  } while (0)
    switch (pl.NT) {
      case 2: SSD_FUSED_AGG(2); break;
      case 4: SSD_FUSED_AGG(4); break;
      default: SSD_FUSED_AGG(8); break;
    }
#undef SSD_FUSED_AGG
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the carry launch (only when some range takes over a state that is not
    // the first range's own aggregate)
    if (pl.nr > 2) {
      const dim3 cgrid((unsigned)(pl.U * (64 * 16 * pl.NT / 4 / 256)));
      switch (pl.NT) {
        case 2: hipLaunchKernelGGL(k_fused_carry<2>, cgrid, dim3(256), 0, s, a); break;
        case 4: hipLaunchKernelGGL(k_fused_carry<4>, cgrid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL(k_fused_carry<8>, cgrid, dim3(256), 0, s, a); break;
      }
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
#define SSD_FUSED(TO, NT)                                                                   \
  do {                                                                                      \
    if (db) hipLaunchKernelGGL((k_fused_fwd<TO, bf16, NT>), grid, dim3(256), 0, s, a);       \
    else hipLaunchKernelGGL((k_fused_fwd<TO, float, NT>), grid, dim3(256), 0, s, a);         \
  } while (0)
  switch (pl.NT) {
    case 2: if (ob) SSD_FUSED(bf16, 2); else SSD_FUSED(float, 2); break;
    case 4: if (ob) SSD_FUSED(bf16, 4); else SSD_FUSED(float, 4); break;
    default: if (ob) SSD_FUSED(bf16, 8); else SSD_FUSED(float, 8); break;
  }
#undef SSD_FUSED
  return hipGetLastError();
}

}  // namespace ssd
