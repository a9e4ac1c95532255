// bwd_chunk.hip -- the per-chunk gradient kernels of the SSD backward pass
// (SSD_ALGO_FUSED of ssd_backward_ex).
//
// Once the state entering every 128-token chunk (Hin: the forward recompute's
// carry-in) and the gradient of the state leaving it through later tokens (dS)
// are known, what a chunk adds to each gradient depends on that chunk alone.
// dS comes from the adjoint of the state passing: k_bwd_adj_state forms, per
// chunk, the gradient its own tokens send to the state entering it,
// U_j = sum_l exp(cs_l) dy_l (outer) C_l, and the reverse scan (state_passing.hip)
// turns those into dS_j = exp(Lambda_{j+1}) dS_{j+1} + U_{j+1} (dfinal at a
// sequence's last chunk) and the initial state's gradient.  The chunked forward of the SSD
// Reference ("Intra-chunk outputs and per-chunk states", "Inter-chunk
// propagation", "Readout"), differentiated factor by factor (section 6 asks for
// exact gradients of every input), gives, with cs the chunk's inclusive cumsum
// of a = delta A, Lambda its value at the last token, L_ls = exp(cs_l - cs_s)
// for s <= l, f_s = delta_s when the step size scales the input term (else 1)
// and dy = dout silu(z):
//   y_l   = sum_s L_ls (C_l . B_s) f_s x_s + exp(cs_l) Hin C_l + D x_l
//           (recomputed: dz = dout y silu'(z))
//   dx_s  = f_s g_s + D dy_s,  g_s = sum_l L_ls (C_l . B_s) dy_l + exp(Lambda - cs_s) dS B_s
//   dC_l  = sum_h [sum_s L_ls f_s (dy_l . x_s) B_s + exp(cs_l) dy_l Hin]
//   dB_s  = sum_h f_s [sum_l L_ls (dy_l . x_s) C_l + exp(Lambda - cs_s) x_s dS]
//   dcs_l = sum_{s<l} M_ls - sum_{l'>l} M_l'l + Q_l - R_l
//           (+ at the chunk's last token: exp(Lambda) <dS, Hin> + sum_s R_s)
//     M_ls = L_ls (C_l . B_s) (dy_l . x_s) f_s,  Q_l = dy_l . (exp(cs_l) Hin C_l),
//     R_l = f_l x_l . (exp(Lambda - cs_l) dS B_l)
//   ddt_t = (A sum_{l >= t} dcs_l + [f = delta: x_t . g_t]) dstep/du
// (the diagonal terms of the two sums in dcs are equal and cancel, so neither
// holds them; no two remaining terms cancel, so the step-size gradient stays
// accurate under strong decay).
//
//   k_bwd_adj_state  one workgroup per (chunk, head): U_j;
//   k_bwd_dx   one workgroup per (chunk, head): y and dz, dx, dcs -> ddt, and
//              the chunk's shares of dA, ddt_bias and dD;
//   k_bwd_dbc  one workgroup per (chunk, group, 64-column slab of N): dB and
//              dC of the slab, summed over the group's heads in registers in
//              head order (groups of more than 8 heads are split into runs of
//              at most 8, whose partial sums k_bwd_dbc_sum adds in run order).
//
// Precision (bf16 x, B, C): inputs exact; operands derived in fp32 (dy, the
// decay-weighted C.B^T and dy.x^T, the states, decay-scaled x) split into bf16
// hi + lo, fp32 accumulation; the cumsum and the sums of the step-size
// gradient in fp64.  Every sum has a fixed order: results are bit-identical
// run to run.
//
// Matrix products on 16x16x32 bf16 tiles (fragment convention in common.hpp).
// A lane's fragment of "rows r0..r0+15 of a row-major matrix, k-block kb" is
// the same data whether it serves as the A operand (rows = output rows) or the
// B operand (rows = output columns), so the C and B rows (n contiguous) read
// from global memory serve both C.B^T layouts:
//   layout A, tiles [s][l] (lane: one l, tokens s = 4q + 0..3): the A operand
//     of products that reduce over s (y, dC), tokens permuted to match;
//   layout B, tiles [l][s] (lane: one s, tokens l = 4q + 0..3): the operand of
//     products that reduce over l (dx, dB).
// Operands that need the token axis as the reduction axis are read from LDS
// tiles in their natural layout with the LDS transpose read.
#include "kernels.hpp"
#include "stage_varlen.hpp"

namespace ssd {

namespace {

constexpr int BC = 128;     // chunk length of these kernels
constexpr int TLD = 72;     // bf16 per row of the x, dy, B, C and state tiles (64 + 8)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp_d(double v) { return fast_exp2((float)v * kLog2e); }

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}
// A lane move within each row of 16 lanes (DPP: no LDS traffic), for the
// sums below: quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2),
// row_half_mirror (lane i <-> 7 - i of its half row) and row_mirror (i <-> 15 -
// i).  After the two quad steps every lane of a quad holds the quad's sum, so
// the mirrors pair quad with quad and half with half exactly as lane ^ 4 and
// lane ^ 8 would: the same additions in the same order.
template <int CTRL>
__device__ __forceinline__ double row_move_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)b, CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}
template <int CTRL>
__device__ __forceinline__ float row_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
// sum over the 16 lanes of a lane group
__device__ __forceinline__ double group16_sum_f64(double v) {
  v += row_move_f64<kDppXor1>(v);
  v += row_move_f64<kDppXor2>(v);
  v += row_move_f64<kDppHalfMirror>(v);
  v += row_move_f64<kDppMirror>(v);
  return v;
}
__device__ __forceinline__ float group16_sum(float v) {
  v += row_move<kDppXor1>(v);
  v += row_move<kDppXor2>(v);
  v += row_move<kDppHalfMirror>(v);
  v += row_move<kDppMirror>(v);
  return v;
}
// Sum over the 4 lane groups (lanes l, l + 16, l + 32, l + 48) with the gfx950
// lane swaps: v_permlane16_swap exchanges rows 0 <-> 1 and 2 <-> 3 between its
// two operands and v_permlane32_swap the wave halves, so with both operands
// holding v, the two results add to v[l] + v[l ^ 16] (then ^ 32) in every lane
// (no LDS traffic; the same pair sums as shuffles).
__device__ __forceinline__ float across_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ double across_groups_f64(double v) {
  auto halves = [](double x, unsigned& lo, unsigned& hi) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(x);
    lo = (unsigned)u;
    hi = (unsigned)(u >> 32);
  };
  auto join = [](unsigned lo, unsigned hi) {
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
  };
  unsigned lo, hi;
  halves(v, lo, hi);
  auto l16 = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  auto h16 = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  v = join(l16[0], h16[0]) + join(l16[1], h16[1]);
  halves(v, lo, hi);
  auto l32 = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  auto h32 = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  return join(l32[0], h32[0]) + join(l32[1], h32[1]);
}

__device__ __forceinline__ float sigmoidf(float v) {
  return __builtin_amdgcn_rcpf(1.0f + fast_exp(-v));
}

// Eight consecutive fp32 from a 16-byte aligned address.
__device__ __forceinline__ f32x8 load8f(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f32x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) { r[i] = a[i]; r[i + 4] = b[i]; }
  return r;
}
__device__ __forceinline__ f32x8 bf8_to_f32(u32x4 v) {
  f32x8 r;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    r[2 * d] = bf16_lo_f32(v[d]);
    r[2 * d + 1] = bf16_hi_f32(v[d]);
  }
  return r;
}
__device__ __forceinline__ FragBF as_frag(u32x4 v) {
  FragBF f;
  f.v = __builtin_bit_cast(bf16x8, v);
  return f;
}
__device__ __forceinline__ FragSplit lds_split(const bf16* hi, const bf16* lo) {
  FragSplit f;
  f.hi = *reinterpret_cast<const bf16x8*>(hi);
  f.lo = *reinterpret_cast<const bf16x8*>(lo);
  return f;
}

struct BwdChunkArgs {
  Geo g;                  // 128-token chunk geometry; meta: the chunk table at 128 tokens
  TArg x, B, C, z, dout, dx, dz, dB, dC, ddt;
  int dout_bf16;
  const float* A;
  const float* D;
  const float* delta;     // (ntok, H) step size
  const float* gd;        // (ntok, H) d(step)/du, 0 where the clamp is active
  const float* cs;        // (K, H, 128) the forward's chunk cumsum (fp32)
  const float* hin;       // (K, H, P, N) forward carry-in states
  float* adj;             // (K, H, P, N) U_j (k_bwd_adj_state), then dS_j
  double* part;           // (K, H, 3): the chunk's shares of dA, ddt_bias, dD
  int input_dt;
  int nsl;                // 64-column slabs of N
  int ntok;               // tokens on the packed axis
  int nsplit, hps;        // k_bwd_dbc: head splits of a group, heads per split
  float* pdb;             // (nsplit, ntok, G, N) partial dB of each head split (partials)
  float* pdc;             // (nsplit, ntok, G, N) partial dC
  int partials;           // dB, dC go through pdb, pdc and k_bwd_dbc_sum
  int accumulate;         // k_bwd_dbc_sum adds to dB, dC instead of starting at zero
};

// The chunk, its sequence's chunks [fi, li), and the gradient of the state
// leaving it through later tokens (dS_j, from the reverse state passing).
struct ChunkCtx {
  Chunk c;
  int fi, li, jl, tp0;
  const float* ds;        // (P, N)
};
__device__ __forceinline__ bool chunk_ctx(const BwdChunkArgs& a, int j, int h, ChunkCtx& x) {
  const Geo& g = a.g;
  if (!get_chunk(g, j, x.c)) return false;
  seq_chunks(g, x.c.seq, x.fi, x.li);
  x.jl = j - x.fi;
  x.tp0 = x.c.b * g.T + x.c.t0;
  x.ds = a.adj + ((int64_t)j * g.H + h) * g.P * g.N;
  return true;
}

// The cumsum of stage_cumsum in two halves, for a workgroup that stages other
// tiles in between: waves 0 and 1 scan their 64 tokens each (partial), then,
// after every thread has called finish (it holds barriers), wave 1's tokens
// get wave 0's total.
__device__ __forceinline__ void stage_cumsum_partial(const BwdChunkArgs& a, const ChunkCtx& x,
                                                     int h, double* s_cs, float* s_f) {
  const int tid = threadIdx.x;
  if (tid < BC) {
    const bool in = tid < x.c.len;
    const float d = in ? a.delta[(int64_t)(x.tp0 + tid) * a.g.H + h] : 0.0f;
    s_cs[tid] = wave_inclusive_sum_f64(in ? (double)d * (double)a.A[h] : 0.0);
    s_f[tid] = in ? (a.input_dt ? d : 1.0f) : 0.0f;
  }
}
__device__ __forceinline__ void stage_cumsum_finish(double* s_cs, double* s_tmp) {
  const int tid = threadIdx.x;
  __syncthreads();
  if (tid == 0) s_tmp[0] = s_cs[kWave - 1];
  __syncthreads();
  if (tid >= kWave && tid < BC) s_cs[tid] += s_tmp[0];
  __syncthreads();
}

// ---------------------------------------------------------------- k_bwd_adj_state

// U_j (P x N) = sum_l exp(cs_l) dy_l (outer) C_l: wave w owns p-tile w, all
// n-tiles; exp(cs) dy (split hi + lo) and C staged in LDS in their natural
// layout (tokens x columns) and read with the transpose read, as the token is
// the reduction axis.
template <int NT>
__global__ __launch_bounds__(256, 2) void k_bwd_adj_state(BwdChunkArgs a) {
  constexpr int NMAX = 16 * NT, CLD = NMAX + 8, BPR = NMAX / 8, ROWS = 256 / BPR;
  __shared__ __align__(16) float s_e[BC];
  __shared__ __align__(16) bf16 s_dyh[BC * TLD];
  __shared__ __align__(16) bf16 s_dyl[BC * TLD];
  __shared__ __align__(16) bf16 s_c[BC * CLD];
  const Geo& g = a.g;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int r16 = lane % 16, q = lane / 16;
  const int item = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int j = item / g.H, h = item % g.H, grp = h / g.hpg;
  Chunk c;
  if (!get_chunk(g, j, c)) return;
  const int len = c.len;
  if (tid < BC) s_e[tid] = tid < len ? fast_exp(a.cs[((int64_t)j * g.H + h) * BC + tid]) : 0.0f;
  __syncthreads();
  {
    const int row0 = tid / 8, col = (tid % 8) * 8;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int l = row0 + 32 * k, lc = min(l, len - 1);
      f32x8 v;
      if (a.dout_bf16) {
        const bf16* db = row_ptr<bf16>(a.dout, c.b, c.t0, h);
        v = bf8_to_f32(*reinterpret_cast<const u32x4*>(at(db, (uint32_t)(lc * a.dout.s1 + col))));
      } else {
        v = load8f(at(row_ptr<float>(a.dout, c.b, c.t0, h), (uint32_t)(lc * a.dout.s1 + col)));
      }
      if (a.z.p) {
        const f32x8 zz = bf8_to_f32(*reinterpret_cast<const u32x4*>(
            at(row_ptr<bf16>(a.z, c.b, c.t0, h), (uint32_t)(lc * a.z.s1 + col))));
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] *= zz[i] * sigmoidf(zz[i]);
      }
      const float e = s_e[l];  // (0 past the chunk's end)
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] *= e;
      const FragSplit sp = split_f32x8(v);
      *reinterpret_cast<bf16x8*>(&s_dyh[l * TLD + col]) = sp.hi;
      *reinterpret_cast<bf16x8*>(&s_dyl[l * TLD + col]) = sp.lo;
    }
    const bf16* cb = row_ptr<bf16>(a.C, c.b, c.t0, grp);
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < BC / ROWS; ++k) {
      const int l = tid / BPR + ROWS * k, cc = (tid % BPR) * 8;
      const u32x4 v = *reinterpret_cast<const u32x4*>(
          at(cb, (uint32_t)(min(l, len - 1) * a.C.s1 + min(cc, g.N - 8))));
      *reinterpret_cast<u32x4*>(&s_c[l * CLD + cc]) = (l < len && cc < g.N) ? v : zero;
    }
  }
  __syncthreads();
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = zero4();
#pragma unroll
  for (int kb = 0; kb < BC / 32; ++kb) {
    const int k0 = kb * 32 + q * 8;
    FragSplit af;
    af.hi = lds_frag_tr(s_dyh, TLD, k0, k0 + 4, wave * 16);
    af.lo = lds_frag_tr(s_dyl, TLD, k0, k0 + 4, wave * 16);
    // every C fragment of the k-block before the products (one LDS round trip
    // per k-block instead of one per n-tile)
    FragBF bf[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bf[nt].v = lds_frag_tr(s_c, CLD, k0, k0 + 4, nt * 16);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) mma(acc[nt], af, bf[nt]);
    __builtin_amdgcn_sched_barrier(0);
  }
  float* dst = a.adj + ((int64_t)j * g.H + h) * g.P * g.N;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = nt * 16 + r16;
    if (n < g.N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(wave * 16 + q * 4 + i) * g.N + n] = acc[nt][i];
    }
  }
}

// ---------------------------------------------------------------- k_bwd_dx

// One workgroup of 8 waves per (chunk, head); x, dy (bf16 hi + lo), B and C
// staged in LDS.  Waves 0-3 form y^T (rows p, columns l; wave w: l-tiles w and
// 7 - w): Y_off^T = Hin C^T scaled by exp(cs_l), then Q_l, then Y_diag^T =
// x^T (L o C.B^T + D I)^T (the C.B^T tiles computed as [s][l], whose
// accumulator layout is directly the B operand), then dz.  Waves 4-7 form g^T
// (rows p, columns s; s-tiles w - 4 and 11 - w): the inter part exp(Lambda -
// cs_s) dS B_s and R_s, then the intra part dy^T (L o C.B^T) with the row and
// column sums of M = (L o C.B^T) o (dy.x^T) f, then dx.  Every output row
// (l or s) is complete in one wave: no staging tile.
template <int NT>
struct DxLds {
  static constexpr int NMAX = 16 * NT, CLD = NMAX + 8;
  static constexpr int OFF_CS = 0;                  // double[128]
  static constexpr int OFF_RED = 1024;              // double[16]
  static constexpr int OFF_ROWP = 1152;             // double[4][128] row sums of M per g-wave
  static constexpr int OFF_COL = OFF_ROWP + 4096;   // double[128] column sums of M
  static constexpr int OFF_F = OFF_COL + 1024;      // float[128]
  static constexpr int OFF_Q = OFF_F + 512;         // float[128]
  static constexpr int OFF_R = OFF_Q + 512;         // float[128]
  static constexpr int OFF_XG = OFF_R + 512;        // float[128]
  static constexpr int OFF_X = OFF_XG + 512;        // bf16[128][TLD]
  static constexpr int OFF_YH = OFF_X + BC * TLD * 2;
  static constexpr int OFF_YL = OFF_YH + BC * TLD * 2;
  static constexpr int OFF_B = OFF_YL + BC * TLD * 2;   // bf16[128][CLD]
  static constexpr int OFF_C = OFF_B + BC * CLD * 2;
  static constexpr int TOTAL = OFF_C + BC * CLD * 2;
};
static_assert(DxLds<8>::TOTAL <= 163840, "one workgroup per CU");

__device__ __forceinline__ double block_sum8(double v, double* red) {
  v = wave_sum_f64(v);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < 8; ++w) t += red[w];
  return t;
}

template <int NT>
__global__ __launch_bounds__(512, 1) void k_bwd_dx(BwdChunkArgs a) {
  using L = DxLds<NT>;
  constexpr int NKB = NT / 2, CLD = L::CLD, NMAX = L::NMAX;
  __shared__ __align__(16) char smem[L::TOTAL];
  double* s_cs = reinterpret_cast<double*>(smem + L::OFF_CS);
  double* s_red = reinterpret_cast<double*>(smem + L::OFF_RED);
  double* s_rowp = reinterpret_cast<double*>(smem + L::OFF_ROWP);
  double* s_col = reinterpret_cast<double*>(smem + L::OFF_COL);
  float* s_f = reinterpret_cast<float*>(smem + L::OFF_F);
  float* s_q = reinterpret_cast<float*>(smem + L::OFF_Q);
  float* s_r = reinterpret_cast<float*>(smem + L::OFF_R);
  float* s_xg = reinterpret_cast<float*>(smem + L::OFF_XG);
  bf16* s_x = reinterpret_cast<bf16*>(smem + L::OFF_X);
  bf16* s_yh = reinterpret_cast<bf16*>(smem + L::OFF_YH);
  bf16* s_yl = reinterpret_cast<bf16*>(smem + L::OFF_YL);
  bf16* s_b = reinterpret_cast<bf16*>(smem + L::OFF_B);
  bf16* s_c = reinterpret_cast<bf16*>(smem + L::OFF_C);
  double* s_dcs = s_rowp;  // (dcs_l replaces the row sums of token l, read by the same thread)

  const Geo& g = a.g;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int r16 = lane % 16, q = lane / 16;
  // (chunk, head): consecutive items are the heads of one chunk, which read the
  // same B and C rows; xcd_remap keeps runs of them on one XCD
  const int item = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int j = item / g.H, h = item % g.H, grp = h / g.hpg;
  double* pj = a.part + ((int64_t)j * g.H + h) * 3;
  ChunkCtx cx;
  if (!chunk_ctx(a, j, h, cx)) {
    if (tid == 0) pj[0] = pj[1] = pj[2] = 0.0;
    return;
  }
  const Chunk& c = cx.c;
  const int len = c.len;
  const int64_t PN = (int64_t)g.P * g.N;
  const float Ah = a.A[h];
  const float Dh = a.D ? a.D[h] : 0.0f;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // ---- stage: cumsum (waves 0-1), x and dy = dout silu(z) (hi + lo) rows, the
  // B and C tiles; D's gradient share sum(dy . x) on the way
  stage_cumsum_partial(a, cx, h, s_cs, s_f);
  const bf16* xb = row_ptr<bf16>(a.x, c.b, c.t0, h);
  const bf16* zb = a.z.p ? row_ptr<bf16>(a.z, c.b, c.t0, h) : nullptr;
  double dyx = 0.0;
  {
    const int row0 = tid / 8, col = (tid % 8) * 8;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int l = row0 + 64 * k, lc = min(l, len - 1);
      const bool in = l < len;
      const u32x4 xv = *reinterpret_cast<const u32x4*>(at(xb, (uint32_t)(lc * a.x.s1 + col)));
      f32x8 go;
      if (a.dout_bf16) {
        const bf16* db = row_ptr<bf16>(a.dout, c.b, c.t0, h);
        go = bf8_to_f32(*reinterpret_cast<const u32x4*>(at(db, (uint32_t)(lc * a.dout.s1 + col))));
      } else {
        go = load8f(at(row_ptr<float>(a.dout, c.b, c.t0, h), (uint32_t)(lc * a.dout.s1 + col)));
      }
      if (zb) {
        const f32x8 zz = bf8_to_f32(*reinterpret_cast<const u32x4*>(at(zb, (uint32_t)(lc * a.z.s1 + col))));
#pragma unroll
        for (int i = 0; i < 8; ++i) go[i] *= zz[i] * sigmoidf(zz[i]);
      }
      const f32x8 xf = bf8_to_f32(xv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        go[i] = in ? go[i] : 0.0f;
        dyx += (double)(go[i] * xf[i]);
      }
      const FragSplit sp = split_f32x8(go);
      *reinterpret_cast<u32x4*>(&s_x[l * TLD + col]) = in ? xv : zero;
      *reinterpret_cast<bf16x8*>(&s_yh[l * TLD + col]) = sp.hi;
      *reinterpret_cast<bf16x8*>(&s_yl[l * TLD + col]) = sp.lo;
    }
    constexpr int BPR = NMAX / 8, ROWS = 512 / BPR;
    const bf16* bbase = row_ptr<bf16>(a.B, c.b, c.t0, grp);
    const bf16* cbase = row_ptr<bf16>(a.C, c.b, c.t0, grp);
#pragma unroll
    for (int k = 0; k < BC / ROWS; ++k) {
      const int l = tid / BPR + ROWS * k, cc = (tid % BPR) * 8;
      const uint32_t off = (uint32_t)(min(l, len - 1) * a.B.s1 + min(cc, g.N - 8));
      const uint32_t offc = (uint32_t)(min(l, len - 1) * a.C.s1 + min(cc, g.N - 8));
      const bool ok = l < len && cc < g.N;
      const u32x4 vb = *reinterpret_cast<const u32x4*>(at(bbase, off));
      const u32x4 vc = *reinterpret_cast<const u32x4*>(at(cbase, offc));
      *reinterpret_cast<u32x4*>(&s_b[l * CLD + cc]) = ok ? vb : zero;
      *reinterpret_cast<u32x4*>(&s_c[l * CLD + cc]) = ok ? vc : zero;
    }
    for (int i = tid; i < 4 * BC; i += 512) s_rowp[i] = 0.0;
  }
  stage_cumsum_finish(s_cs, s_red + 15);
  const double lam = s_cs[len - 1];
  const float* hin = a.hin + ((int64_t)j * g.H + h) * PN;
  // a state row (P x N fp32, row p) as 8 fp32 n of k-block kb (0 past N)
  auto state8 = [&](const float* st, int p, int kb) -> f32x8 {
    const int n = kb * 32 + q * 8;
    f32x8 v = load8f(st + (int64_t)p * g.N + min(n, g.N - 8));
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = n < g.N ? v[i] : 0.0f;
    return v;
  };
  const int w4 = wave & 3;
  const int tA = w4, tB = 7 - w4;

  if (wave < 4) {
    // ==== y side: l-tiles tA, tB
    f32x4 yt[2][4];
#pragma unroll
    for (int ui = 0; ui < 2; ++ui)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) yt[ui][pt] = zero4();
    FragBF cf[2][NKB];
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int l = (ui ? tB : tA) * 16 + r16;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        cf[ui][kb].v = *reinterpret_cast<const bf16x8*>(&s_c[l * CLD + kb * 32 + q * 8]);
    }
    // <dS, Hin> over p-tile w (this wave's share of the decay gradient), every
    // row load issued before the first product
    double ip = 0.0;
    {
      f32x8 hw[NKB], dw[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        hw[kb] = state8(hin, w4 * 16 + r16, kb);
        dw[kb] = state8(cx.ds, w4 * 16 + r16, kb);
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i) ip += (double)hw[kb][i] * (double)dw[kb][i];
    }
    // Y_off^T = Hin C^T (rows p, columns l): a k-block's four state rows are
    // loaded together, then multiplied (one round trip to memory per k-block)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x8 hv[4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) hv[pt] = state8(hin, pt * 16 + r16, kb);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const FragSplit hf = split_f32x8(hv[pt]);
        mma(yt[0][pt], hf, cf[0][kb]);
        mma(yt[1][pt], hf, cf[1][kb]);
      }
    }
    ip = wave_sum_f64(ip);
    if (lane == 0) s_red[8 + w4] = ip;
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int l = (ui ? tB : tA) * 16 + r16;
      const float el = exp_d(s_cs[l]);
      float qs = 0.0f;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const uint2 hv = *reinterpret_cast<const uint2*>(&s_yh[l * TLD + pt * 16 + q * 4]);
        const uint2 lv = *reinterpret_cast<const uint2*>(&s_yl[l * TLD + pt * 16 + q * 4]);
        const float dy4[4] = {bf16_lo_f32(hv.x) + bf16_lo_f32(lv.x), bf16_hi_f32(hv.x) + bf16_hi_f32(lv.x),
                              bf16_lo_f32(hv.y) + bf16_lo_f32(lv.y), bf16_hi_f32(hv.y) + bf16_hi_f32(lv.y)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          yt[ui][pt][i] *= el;
          qs += dy4[i] * yt[ui][pt][i];
        }
      }
      qs = across_groups(qs);
      if (q == 0) s_q[l] = qs;
    }
    // Y_diag^T = x^T M^T, M = L o C.B^T (+ D on the diagonal)
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int lt = ui ? tB : tA;
      const int lrow = lt * 16 + r16;
      const double csl = s_cs[lrow];
      for (int kp = 0; kp <= lt / 2; ++kp) {
        const int sa = 2 * kp, sb = 2 * kp + 1;
        f32x4 va = zero4(), vb = zero4();
        // every B row fragment of the pair first (one LDS round trip), then
        // the products
        FragBF ba[NKB], bb[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          ba[kb].v = *reinterpret_cast<const bf16x8*>(&s_b[(sa * 16 + r16) * CLD + kb * 32 + q * 8]);
          bb[kb].v = *reinterpret_cast<const bf16x8*>(&s_b[(sb * 16 + r16) * CLD + kb * 32 + q * 8]);
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          mma(va, ba[kb], cf[ui][kb]);
          mma(vb, bb[kb], cf[ui][kb]);
        }
        // the x^T fragments go out before M is formed: their latency runs
        // under its exponentials
        FragBF xt[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
          xt[pt].v = lds_frag_tr(s_x, TLD, sa * 16 + q * 4, sb * 16 + q * 4, pt * 16);
        f32x8 m;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int s_a = sa * 16 + q * 4 + e4, s_b2 = sb * 16 + q * 4 + e4;
          const float ma = exp_d(csl - s_cs[s_a]) * s_f[s_a] * va[e4];
          const float mb = exp_d(csl - s_cs[s_b2]) * s_f[s_b2] * vb[e4];
          m[e4] = s_a < lrow ? ma : (s_a == lrow ? ma + Dh : 0.0f);
          m[4 + e4] = s_b2 < lrow ? mb : (s_b2 == lrow ? mb + Dh : 0.0f);
        }
        const FragSplit mf = split_f32x8(m);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) mma(yt[ui][pt], xt[pt], mf);
      }
    }
    // dz = dout y silu'(z), silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z)))
    if (zb) {
#pragma unroll
      for (int ui = 0; ui < 2; ++ui) {
        const int l = (ui ? tB : tA) * 16 + r16;
        const int lc = min(l, len - 1);
        float* dzr = row_ptr_mut<float>(a.dz, c.b, c.t0, h);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const int p = pt * 16 + q * 4;
          f32x4 go;
          if (a.dout_bf16) {
            const uint2 v = *reinterpret_cast<const uint2*>(
                at(row_ptr<bf16>(a.dout, c.b, c.t0, h), (uint32_t)(lc * a.dout.s1 + p)));
            go[0] = bf16_lo_f32(v.x); go[1] = bf16_hi_f32(v.x);
            go[2] = bf16_lo_f32(v.y); go[3] = bf16_hi_f32(v.y);
          } else {
            go = *reinterpret_cast<const f32x4*>(
                at(row_ptr<float>(a.dout, c.b, c.t0, h), (uint32_t)(lc * a.dout.s1 + p)));
          }
          const uint2 zv = *reinterpret_cast<const uint2*>(at(zb, (uint32_t)(lc * a.z.s1 + p)));
          const float z4[4] = {bf16_lo_f32(zv.x), bf16_hi_f32(zv.x), bf16_lo_f32(zv.y),
                               bf16_hi_f32(zv.y)};
          f32x4 o;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float sg = sigmoidf(z4[i]);
            o[i] = go[i] * yt[ui][pt][i] * (sg * (1.0f + z4[i] * (1.0f - sg)));
          }
          if (l < len) *reinterpret_cast<f32x4*>(at(dzr, (uint32_t)(l * a.dz.s1 + p))) = o;
        }
      }
    }
  } else {
    // ==== g side: s-tiles tA, tB
    f32x4 gt[2][4];
#pragma unroll
    for (int ui = 0; ui < 2; ++ui)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) gt[ui][pt] = zero4();
    FragBF bf[2][NKB];
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int s = (ui ? tB : tA) * 16 + r16;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        bf[ui][kb].v = *reinterpret_cast<const bf16x8*>(&s_b[s * CLD + kb * 32 + q * 8]);
    }
    // inter part g^T += dS B^T, scaled by exp(Lambda - cs_s); R_s.  A k-block's
    // four state rows are loaded together, then multiplied.
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x8 dv[4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) dv[pt] = state8(cx.ds, pt * 16 + r16, kb);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const FragSplit df = split_f32x8(dv[pt]);
        mma(gt[0][pt], df, bf[0][kb]);
        mma(gt[1][pt], df, bf[1][kb]);
      }
    }
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int s = (ui ? tB : tA) * 16 + r16;
      const float e = s < len ? exp_d(lam - s_cs[s]) : 0.0f;
      float rp = 0.0f;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const uint2 xv = *reinterpret_cast<const uint2*>(&s_x[s * TLD + pt * 16 + q * 4]);
        const float x4[4] = {bf16_lo_f32(xv.x), bf16_hi_f32(xv.x), bf16_lo_f32(xv.y),
                             bf16_hi_f32(xv.y)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          gt[ui][pt][i] *= e;
          rp += x4[i] * gt[ui][pt][i];
        }
      }
      rp = across_groups(rp);
      if (q == 0) s_r[s] = s_f[s] * rp;
    }
    // intra part g^T += dy^T (L o C.B^T) ([l][s] tiles: the B operand), with the
    // row and column sums of M in fp64
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int sbt = ui ? tB : tA;
      const int s = sbt * 16 + r16;
      FragBF xr[2];
#pragma unroll
      for (int kp = 0; kp < 2; ++kp)
        xr[kp].v = *reinterpret_cast<const bf16x8*>(&s_x[s * TLD + kp * 32 + q * 8]);
      const double css = s_cs[s];
      const float fs = s_f[s];
      double colp = 0.0;
      for (int lp = sbt / 2; lp < 4; ++lp) {
        const int la = 2 * lp, lb = 2 * lp + 1;
        f32x4 ca = zero4(), cb = zero4(), xa = zero4(), xb2 = zero4();
        FragBF c0[NKB], c1[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          c0[kb].v = *reinterpret_cast<const bf16x8*>(&s_c[(la * 16 + r16) * CLD + kb * 32 + q * 8]);
          c1[kb].v = *reinterpret_cast<const bf16x8*>(&s_c[(lb * 16 + r16) * CLD + kb * 32 + q * 8]);
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          mma(ca, c0[kb], bf[ui][kb]);
          mma(cb, c1[kb], bf[ui][kb]);
        }
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          const int pc = kp * 32 + q * 8;
          mma(xa, lds_split(&s_yh[(la * 16 + r16) * TLD + pc], &s_yl[(la * 16 + r16) * TLD + pc]),
              xr[kp]);
          mma(xb2, lds_split(&s_yh[(lb * 16 + r16) * TLD + pc], &s_yl[(lb * 16 + r16) * TLD + pc]),
              xr[kp]);
        }
        // the dy^T fragments go out before M is formed
        FragSplit dyt[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          dyt[pt].hi = lds_frag_tr(s_yh, TLD, la * 16 + q * 4, lb * 16 + q * 4, pt * 16);
          dyt[pt].lo = lds_frag_tr(s_yl, TLD, la * 16 + q * 4, lb * 16 + q * 4, pt * 16);
        }
        f32x8 m;
        double rowa[4], rowb[4];
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int l_a = la * 16 + q * 4 + e4, l_b = lb * 16 + q * 4 + e4;
          const float ea = exp_d(s_cs[l_a] - css), eb = exp_d(s_cs[l_b] - css);
          const bool oka = s <= l_a && l_a < len && s < len;
          const bool okb = s <= l_b && l_b < len && s < len;
          m[e4] = oka ? ea * ca[e4] : 0.0f;
          m[4 + e4] = okb ? eb * cb[e4] : 0.0f;
          const double pa = (oka && s < l_a) ? (double)(m[e4] * xa[e4] * fs) : 0.0;
          const double pb = (okb && s < l_b) ? (double)(m[4 + e4] * xb2[e4] * fs) : 0.0;
          rowa[e4] = pa;
          rowb[e4] = pb;
          colp += pa + pb;
        }
        const FragSplit mf = split_f32x8(m);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) mma(gt[ui][pt], dyt[pt], mf);
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const double ra = group16_sum_f64(rowa[e4]);
          const double rb = group16_sum_f64(rowb[e4]);
          if (r16 == 0) {
            s_rowp[w4 * BC + la * 16 + q * 4 + e4] += ra;
            s_rowp[w4 * BC + lb * 16 + q * 4 + e4] += rb;
          }
        }
      }
      colp = across_groups_f64(colp);
      if (q == 0) s_col[s] = colp;
    }
    // dx = f g + D dy; x . g for the step size on the input term
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int s = (ui ? tB : tA) * 16 + r16;
      const float fs = s_f[s];
      float* dxr = row_ptr_mut<float>(a.dx, c.b, c.t0, h);
      float e = 0.0f;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const int p = pt * 16 + q * 4;
        const uint2 hv = *reinterpret_cast<const uint2*>(&s_yh[s * TLD + p]);
        const uint2 lv = *reinterpret_cast<const uint2*>(&s_yl[s * TLD + p]);
        const uint2 xv = *reinterpret_cast<const uint2*>(&s_x[s * TLD + p]);
        const float dy4[4] = {bf16_lo_f32(hv.x) + bf16_lo_f32(lv.x), bf16_hi_f32(hv.x) + bf16_hi_f32(lv.x),
                              bf16_lo_f32(hv.y) + bf16_lo_f32(lv.y), bf16_hi_f32(hv.y) + bf16_hi_f32(lv.y)};
        const float x4[4] = {bf16_lo_f32(xv.x), bf16_hi_f32(xv.x), bf16_lo_f32(xv.y),
                             bf16_hi_f32(xv.y)};
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[i] = fs * gt[ui][pt][i] + Dh * dy4[i];
          e += x4[i] * gt[ui][pt][i];
        }
        if (s < len) *reinterpret_cast<f32x4*>(at(dxr, (uint32_t)(s * a.dx.s1 + p))) = o;
      }
      e = across_groups(e);
      if (q == 0) s_xg[s] = s < len ? e : 0.0f;
    }
  }

  // ---- dcs, and its suffix sums: dL/da_t
  __syncthreads();
  if (tid < BC) {
    const int l = tid;
    double v = 0.0, rl = 0.0;
    if (l < len) {
      rl = (double)s_r[l];
      v = s_rowp[l] + s_rowp[BC + l] + s_rowp[2 * BC + l] + s_rowp[3 * BC + l] - s_col[l] +
          (double)s_q[l] - rl;
    }
    s_dcs[l] = v;
    const double rs = wave_sum_f64(rl);
    if (lane == 0) s_red[12 + wave] = rs;
  }
  __syncthreads();
  if (tid == 0) {
    const double sip = s_red[8] + s_red[9] + s_red[10] + s_red[11];
    s_dcs[len - 1] += (double)exp_d(lam) * sip + s_red[12] + s_red[13];
  }
  __syncthreads();
  double sa = 0.0, sb = 0.0, suf = 0.0;
  if (tid < BC) {
    // suffix sums by a reversed inclusive scan: thread t holds token 127 - t
    suf = wave_inclusive_sum_f64(s_dcs[BC - 1 - tid]);
    if (tid == kWave - 1) s_red[14] = suf;
  }
  __syncthreads();
  if (tid < BC) {
    const int l = BC - 1 - tid;
    const double da = suf + (tid >= kWave ? s_red[14] : 0.0);
    if (l < len) {
      const int64_t it = (int64_t)(cx.tp0 + l) * g.H + h;
      const double gg = (da * (double)Ah + (a.input_dt ? (double)s_xg[l] : 0.0)) * (double)a.gd[it];
      row_ptr_mut<float>(a.ddt, c.b, c.t0 + l, h)[0] = (float)gg;
      sa = da * (double)a.delta[it];
      sb = gg;
    }
  }
  sa = block_sum8(sa, s_red);
  sb = block_sum8(sb, s_red);
  dyx = block_sum8(dyx, s_red);
  if (tid == 0) {
    pj[0] = sa;
    pj[1] = sb;
    pj[2] = dyx;
  }
}

// ---------------------------------------------------------------- k_bwd_dbc

// One workgroup of 8 waves per (chunk, group, head split, 64-column slab of N).
// Per head, every operand is staged in LDS: dy (bf16 hi + lo), x, and the
// slabs of Hin and dS (hi + lo); the chunk's B and C slabs once.  Waves 0-3
// form dC (wave w: l-tiles w and 7 - w), waves 4-7 dB (s-tiles w - 4 and
// 11 - w), each accumulating over the heads in registers.
struct DbcLds {
  static constexpr int OFF_CS = 0;                   // double[128]
  static constexpr int OFF_F = 1024;                 // float[128]
  static constexpr int OFF_EL = 1536;                // float[128] exp(cs_l)
  static constexpr int OFF_ES = 2048;                // float[128] f_s exp(Lambda - cs_s)
  static constexpr int OFF_TMP = 2560;               // double[8]
  static constexpr int T128 = BC * TLD * 2;          // a [128][TLD] bf16 tile
  static constexpr int T64 = 64 * TLD * 2;           // a [64][TLD] bf16 tile
  static constexpr int OFF_BT = 2624;                // B slab
  static constexpr int OFF_CT = OFF_BT + T128;       // C slab
  static constexpr int OFF_YH = OFF_CT + T128;       // dy hi
  static constexpr int OFF_YL = OFF_YH + T128;       // dy lo
  static constexpr int OFF_X = OFF_YL + T128;        // x
  static constexpr int OFF_HH = OFF_X + T128;        // Hin slab hi, lo
  static constexpr int OFF_HL = OFF_HH + T64;
  static constexpr int OFF_DH = OFF_HL + T64;        // dS slab hi, lo
  static constexpr int OFF_DL = OFF_DH + T64;
  static constexpr int TOTAL = OFF_DL + T64;
};
static_assert(DbcLds::TOTAL <= 163840, "one workgroup per CU");

__global__ __launch_bounds__(512, 1) void k_bwd_dbc(BwdChunkArgs a) {
  __shared__ __align__(16) char smem[DbcLds::TOTAL];
  double* s_cs = reinterpret_cast<double*>(smem + DbcLds::OFF_CS);
  float* s_f = reinterpret_cast<float*>(smem + DbcLds::OFF_F);
  float* s_el = reinterpret_cast<float*>(smem + DbcLds::OFF_EL);
  float* s_es = reinterpret_cast<float*>(smem + DbcLds::OFF_ES);
  double* s_tmp = reinterpret_cast<double*>(smem + DbcLds::OFF_TMP);
  bf16* s_bt = reinterpret_cast<bf16*>(smem + DbcLds::OFF_BT);
  bf16* s_ct = reinterpret_cast<bf16*>(smem + DbcLds::OFF_CT);
  bf16* s_yh = reinterpret_cast<bf16*>(smem + DbcLds::OFF_YH);
  bf16* s_yl = reinterpret_cast<bf16*>(smem + DbcLds::OFF_YL);
  bf16* s_x = reinterpret_cast<bf16*>(smem + DbcLds::OFF_X);
  bf16* s_hh = reinterpret_cast<bf16*>(smem + DbcLds::OFF_HH);
  bf16* s_hl = reinterpret_cast<bf16*>(smem + DbcLds::OFF_HL);
  bf16* s_dh = reinterpret_cast<bf16*>(smem + DbcLds::OFF_DH);
  bf16* s_dl = reinterpret_cast<bf16*>(smem + DbcLds::OFF_DL);

  const Geo& g = a.g;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int r16 = lane % 16, q = lane / 16;
  // (chunk, group, head split, slab): the items of one (chunk, group) are
  // consecutive
  const int item = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int per_j = g.G * a.nsplit * a.nsl;
  const int j = item / per_j;
  int rem = item % per_j;
  const int grp = rem / (a.nsplit * a.nsl);
  rem %= a.nsplit * a.nsl;
  const int sp = rem / a.nsl, n0 = (rem % a.nsl) * 64;
  const int h_lo = grp * g.hpg + sp * a.hps, h_hi = min(h_lo + a.hps, (grp + 1) * g.hpg);
  Chunk c;
  if (!get_chunk(g, j, c)) return;
  const int len = c.len;
  const int nw = min(64, g.N - n0);  // columns of this slab
  const int64_t PN = (int64_t)g.P * g.N;
  const int tp0 = c.b * g.T + c.t0;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // ---- B and C slabs of the chunk (rows past the chunk, columns past N: 0)
  {
    const bf16* bb = row_ptr<bf16>(a.B, c.b, c.t0, grp) + n0;
    const bf16* cb = row_ptr<bf16>(a.C, c.b, c.t0, grp) + n0;
    const int row0 = tid / 8, col = (tid % 8) * 8;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int l = row0 + 64 * k;
      const int lc = min(l, len - 1), cc = min(col, nw - 8);
      const bool ok = l < len && col < nw;
      const u32x4 vb = *reinterpret_cast<const u32x4*>(at(bb, (uint32_t)(lc * a.B.s1 + cc)));
      const u32x4 vc = *reinterpret_cast<const u32x4*>(at(cb, (uint32_t)(lc * a.C.s1 + cc)));
      *reinterpret_cast<u32x4*>(&s_bt[l * TLD + col]) = ok ? vb : zero;
      *reinterpret_cast<u32x4*>(&s_ct[l * TLD + col]) = ok ? vc : zero;
    }
  }

  const bool dc_side = wave < 4;
  const int w4 = wave & 3;
  const int tA = w4, tB = 7 - w4;  // l-tiles (dC side) or s-tiles (dB side)
  f32x4 acc[2][4];
#pragma unroll
  for (int ui = 0; ui < 2; ++ui)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[ui][nt] = zero4();

  // The next head's rows are loaded into registers while the current head is
  // multiplied (the products read LDS only, so the loads overlap them): dout
  // (or its bf16), z and x rows (2 x 8 columns each), and 8 columns of one row
  // of the Hin and dS slabs.
  const int row0 = tid / 8, col = (tid % 8) * 8;
  struct Pre {
    f32x8 go[2];
    u32x4 zv[2], xv[2];
    f32x8 hv, dv;
  } pre;
  auto issue = [&](int h) {
    const bf16* xb = row_ptr<bf16>(a.x, c.b, c.t0, h);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int lc = min(row0 + 64 * k, len - 1);
      if (a.dout_bf16) {
        const bf16* db = row_ptr<bf16>(a.dout, c.b, c.t0, h);
        pre.go[k] = bf8_to_f32(*reinterpret_cast<const u32x4*>(at(db, (uint32_t)(lc * a.dout.s1 + col))));
      } else {
        pre.go[k] = load8f(at(row_ptr<float>(a.dout, c.b, c.t0, h), (uint32_t)(lc * a.dout.s1 + col)));
      }
      pre.zv[k] = a.z.p ? *reinterpret_cast<const u32x4*>(
                              at(row_ptr<bf16>(a.z, c.b, c.t0, h), (uint32_t)(lc * a.z.s1 + col)))
                        : zero;
      pre.xv[k] = *reinterpret_cast<const u32x4*>(at(xb, (uint32_t)(lc * a.x.s1 + col)));
    }
    const int p = tid / 8;
    pre.hv = load8f(a.hin + ((int64_t)j * g.H + h) * PN + (int64_t)p * g.N + n0 + min(col, nw - 8));
    pre.dv = load8f(a.adj + ((int64_t)j * g.H + h) * PN + (int64_t)p * g.N + n0 + min(col, nw - 8));
  };
  issue(h_lo);
  for (int h = h_lo; h < h_hi; ++h) {
    ChunkCtx cx;
    chunk_ctx(a, j, h, cx);
    __syncthreads();  // the previous head is done with every staged tile
    // ---- stage: cumsum (waves 0-1), dy = dout silu(z) (hi + lo) and x rows,
    // the Hin and dS slabs (hi + lo), from the registers loaded above
    stage_cumsum_partial(a, cx, h, s_cs, s_f);
    {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int l = row0 + 64 * k;
        const bool in = l < len;
        f32x8 v = pre.go[k];
        if (a.z.p) {
          const f32x8 zz = bf8_to_f32(pre.zv[k]);
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] *= zz[i] * sigmoidf(zz[i]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = in ? v[i] : 0.0f;
        const FragSplit spl = split_f32x8(v);
        *reinterpret_cast<bf16x8*>(&s_yh[l * TLD + col]) = spl.hi;
        *reinterpret_cast<bf16x8*>(&s_yl[l * TLD + col]) = spl.lo;
        *reinterpret_cast<u32x4*>(&s_x[l * TLD + col]) = in ? pre.xv[k] : zero;
      }
      const int p = tid / 8;
      f32x8 hv = pre.hv, dv = pre.dv;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        hv[i] = col < nw ? hv[i] : 0.0f;
        dv[i] = col < nw ? dv[i] : 0.0f;
      }
      const FragSplit hs = split_f32x8(hv), ds = split_f32x8(dv);
      *reinterpret_cast<bf16x8*>(&s_hh[p * TLD + col]) = hs.hi;
      *reinterpret_cast<bf16x8*>(&s_hl[p * TLD + col]) = hs.lo;
      *reinterpret_cast<bf16x8*>(&s_dh[p * TLD + col]) = ds.hi;
      *reinterpret_cast<bf16x8*>(&s_dl[p * TLD + col]) = ds.lo;
    }
    stage_cumsum_finish(s_cs, s_tmp);
    if (tid < BC) {
      const bool in = tid < len;
      const double lam = s_cs[len - 1];
      s_el[tid] = in ? exp_d(s_cs[tid]) : 0.0f;
      s_es[tid] = in ? s_f[tid] * exp_d(lam - s_cs[tid]) : 0.0f;
    }
    __syncthreads();
    // (past the last head this reloads it, unused)
    issue(min(h + 1, h_hi - 1));

    if (dc_side) {
      // ---- dC_l += sum_s (L o dy.x^T f)_ls B_s + exp(cs_l) dy_l Hin, for l-tiles
      // tA, tB (dy.x^T as [s][l] tiles: the A operand of the product over s)
#pragma unroll
      for (int ui = 0; ui < 2; ++ui) {
        const int lt = ui ? tB : tA;
        const int l = lt * 16 + r16;
        FragSplit dyf[2];
#pragma unroll
        for (int kp = 0; kp < 2; ++kp)
          dyf[kp] = lds_split(&s_yh[l * TLD + kp * 32 + q * 8], &s_yl[l * TLD + kp * 32 + q * 8]);
        const double csl = s_cs[l];
        for (int kp2 = 0; kp2 <= lt / 2; ++kp2) {
          const int sa = 2 * kp2, sb = 2 * kp2 + 1;
          f32x4 va = zero4(), vb = zero4();
          // operand reads ahead of their products: the x rows, then (under
          // the decay weights) the B^T fragments
          FragBF xa[2], xb2[2];
#pragma unroll
          for (int kp = 0; kp < 2; ++kp) {
            xa[kp].v = *reinterpret_cast<const bf16x8*>(&s_x[(sa * 16 + r16) * TLD + kp * 32 + q * 8]);
            xb2[kp].v = *reinterpret_cast<const bf16x8*>(&s_x[(sb * 16 + r16) * TLD + kp * 32 + q * 8]);
          }
#pragma unroll
          for (int kp = 0; kp < 2; ++kp) {
            mma(va, xa[kp], dyf[kp]);
            mma(vb, xb2[kp], dyf[kp]);
          }
          FragBF bt[4];
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            bt[nt].v = lds_frag_tr(s_bt, TLD, sa * 16 + q * 4, sb * 16 + q * 4, nt * 16);
          f32x8 w;
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const int s_a = sa * 16 + q * 4 + e4, s_b = sb * 16 + q * 4 + e4;
            w[e4] = s_a <= l ? exp_d(csl - s_cs[s_a]) * s_f[s_a] * va[e4] : 0.0f;
            w[4 + e4] = s_b <= l ? exp_d(csl - s_cs[s_b]) * s_f[s_b] * vb[e4] : 0.0f;
          }
          const FragSplit wf = split_f32x8(w);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) mma(acc[ui][nt], wf, bt[nt]);
        }
        const float el = s_el[l];
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          FragSplit hs[4];
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            hs[nt].hi = lds_frag_tr(s_hh, TLD, kp * 32 + q * 8, kp * 32 + q * 8 + 4, nt * 16);
            hs[nt].lo = lds_frag_tr(s_hl, TLD, kp * 32 + q * 8, kp * 32 + q * 8 + 4, nt * 16);
          }
          f32x8 v = bf8_to_f32(__builtin_bit_cast(u32x4, dyf[kp].hi));
          const f32x8 lo = bf8_to_f32(__builtin_bit_cast(u32x4, dyf[kp].lo));
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = (v[i] + lo[i]) * el;
          const FragSplit af = split_f32x8(v);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) mma(acc[ui][nt], af, hs[nt]);
        }
      }
    } else {
      // ---- dB_s += f_s sum_l (L o dy.x^T)_ls C_l + f_s exp(Lambda - cs_s) x_s dS,
      // for s-tiles tA, tB (dy.x^T as [l][s] tiles: the A operand of the
      // product over l)
#pragma unroll
      for (int ui = 0; ui < 2; ++ui) {
        const int sbt = ui ? tB : tA;
        const int s = sbt * 16 + r16;
        FragBF xr[2];
#pragma unroll
        for (int kp = 0; kp < 2; ++kp)
          xr[kp].v = *reinterpret_cast<const bf16x8*>(&s_x[s * TLD + kp * 32 + q * 8]);
        const double css = s_cs[s];
        const float fs = s_f[s];
        for (int lp = sbt / 2; lp < 4; ++lp) {
          const int la = 2 * lp, lb = 2 * lp + 1;
          f32x4 va = zero4(), vb = zero4();
          // operand reads ahead of their products: the dy rows, then (under
          // the decay weights) the C^T fragments
          FragSplit ya[2], yb[2];
#pragma unroll
          for (int kp = 0; kp < 2; ++kp) {
            const int pc = kp * 32 + q * 8;
            ya[kp] = lds_split(&s_yh[(la * 16 + r16) * TLD + pc], &s_yl[(la * 16 + r16) * TLD + pc]);
            yb[kp] = lds_split(&s_yh[(lb * 16 + r16) * TLD + pc], &s_yl[(lb * 16 + r16) * TLD + pc]);
          }
#pragma unroll
          for (int kp = 0; kp < 2; ++kp) {
            mma(va, ya[kp], xr[kp]);
            mma(vb, yb[kp], xr[kp]);
          }
          FragBF ct[4];
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            ct[nt].v = lds_frag_tr(s_ct, TLD, la * 16 + q * 4, lb * 16 + q * 4, nt * 16);
          f32x8 w;
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const int l_a = la * 16 + q * 4 + e4, l_b = lb * 16 + q * 4 + e4;
            w[e4] = s <= l_a ? exp_d(s_cs[l_a] - css) * fs * va[e4] : 0.0f;
            w[4 + e4] = s <= l_b ? exp_d(s_cs[l_b] - css) * fs * vb[e4] : 0.0f;
          }
          const FragSplit wf = split_f32x8(w);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) mma(acc[ui][nt], wf, ct[nt]);
        }
        const float es = s_es[s];
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          FragSplit ds[4];
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            ds[nt].hi = lds_frag_tr(s_dh, TLD, kp * 32 + q * 8, kp * 32 + q * 8 + 4, nt * 16);
            ds[nt].lo = lds_frag_tr(s_dl, TLD, kp * 32 + q * 8, kp * 32 + q * 8 + 4, nt * 16);
          }
          f32x8 v = bf8_to_f32(__builtin_bit_cast(u32x4, xr[kp].v));
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] *= es;
          const FragSplit af = split_f32x8(v);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) mma(acc[ui][nt], af, ds[nt]);
        }
      }
    }
  }

  // ---- store: accumulator tile [row][n], lane: column n = 16 nt + r16, rows
  // 4 q + 0..3; dC from waves 0-3, dB from waves 4-7
  const TArg& out = dc_side ? a.dC : a.dB;
  float* part = dc_side ? a.pdc : a.pdb;
#pragma unroll
  for (int ui = 0; ui < 2; ++ui) {
    const int rt = ui ? tB : tA;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int n = nt * 16 + r16;
      if (n >= nw) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rt * 16 + q * 4 + i;
        if (r >= len) continue;
        if (!a.partials) {
          row_ptr_mut<float>(out, c.b, c.t0 + r, grp)[n0 + n] = acc[ui][nt][i];
        } else {
          part[(((int64_t)sp * a.ntok + tp0 + r) * g.G + grp) * g.N + n0 + n] = acc[ui][nt][i];
        }
      }
    }
  }
}

// ---- dB and dC of a chunk and group: the head splits' partial sums, added in
// split order (after what dB and dC hold when accumulating: an earlier pass's
// splits of the same group, so the order is the same as in one pass)
__global__ __launch_bounds__(256) void k_bwd_dbc_sum(BwdChunkArgs a) {
  const Geo& g = a.g;
  const int j = (int)blockIdx.x / g.G, grp = (int)blockIdx.x % g.G;
  Chunk c;
  if (!get_chunk(g, j, c)) return;
  const int tp0 = c.b * g.T + c.t0;
  const int nv = g.N / 4;
  for (int e = threadIdx.x; e < c.len * nv; e += 256) {
    const int r = e / nv, n = (e % nv) * 4;
    f32x4 sb = zero4(), sc = zero4();
    if (a.accumulate) {
      sb = *reinterpret_cast<const f32x4*>(row_ptr<float>(a.dB, c.b, c.t0 + r, grp) + n);
      sc = *reinterpret_cast<const f32x4*>(row_ptr<float>(a.dC, c.b, c.t0 + r, grp) + n);
    }
    for (int sp = 0; sp < a.nsplit; ++sp) {
      const int64_t o = (((int64_t)sp * a.ntok + tp0 + r) * g.G + grp) * g.N + n;
      sb += *reinterpret_cast<const f32x4*>(a.pdb + o);
      sc += *reinterpret_cast<const f32x4*>(a.pdc + o);
    }
    *reinterpret_cast<f32x4*>(row_ptr_mut<float>(a.dB, c.b, c.t0 + r, grp) + n) = sb;
    *reinterpret_cast<f32x4*>(row_ptr_mut<float>(a.dC, c.b, c.t0 + r, grp) + n) = sc;
  }
}

}  // namespace

int bwd_chunk_splits(int hpg) { return (hpg + kBwdHeadsPerSplit - 1) / kBwdHeadsPerSplit; }

namespace {
BwdChunkArgs chunk_args(const BwdChunkLaunch& l) {
  const Geo& g = l.g;
  BwdChunkArgs a;
  a.g = g;
  a.x = l.x; a.B = l.B; a.C = l.C; a.z = l.z; a.dout = l.dout;
  a.dx = l.dx; a.dz = l.dz; a.dB = l.dB; a.dC = l.dC; a.ddt = l.ddt;
  a.dout_bf16 = l.dout_dtype == DT_BF16;
  a.A = l.A; a.D = l.D; a.delta = l.delta; a.gd = l.gd;
  a.cs = l.cs; a.hin = l.hin; a.adj = l.adj;
  a.part = l.part;
  a.input_dt = l.input_dt;
  a.nsl = (g.N + 63) / 64;
  a.ntok = l.ntok;
  a.nsplit = bwd_chunk_splits(g.hpg);
  a.hps = (g.hpg + a.nsplit - 1) / a.nsplit;
  a.pdb = l.pdb;
  a.pdc = l.pdc;
  a.partials = a.nsplit > 1 || l.partials;
  a.accumulate = l.accumulate;
  return a;
}
}  // namespace

hipError_t launch_bwd_adj_state(const BwdChunkLaunch& l, hipStream_t s) {
  const Geo& g = l.g;
  if (g.K <= 0) return hipSuccess;
  const BwdChunkArgs a = chunk_args(l);
  const unsigned nx = (unsigned)((int64_t)g.K * g.H);
  if (g.N <= 64) hipLaunchKernelGGL(k_bwd_adj_state<4>, dim3(nx), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_bwd_adj_state<8>, dim3(nx), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_chunk(const BwdChunkLaunch& l, hipStream_t s) {
  const Geo& g = l.g;
  if (g.K <= 0) return hipSuccess;  // (dead chunk slots in packed mode exit at once)
  const BwdChunkArgs a = chunk_args(l);
  const unsigned nx = (unsigned)((int64_t)g.K * g.H);
  if (g.N <= 64) hipLaunchKernelGGL(k_bwd_dx<4>, dim3(nx), dim3(512), 0, s, a);
  else hipLaunchKernelGGL(k_bwd_dx<8>, dim3(nx), dim3(512), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned nb = (unsigned)((int64_t)g.K * g.G * a.nsplit * a.nsl);
  hipLaunchKernelGGL(k_bwd_dbc, dim3(nb), dim3(512), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess || !a.partials) return e;
  hipLaunchKernelGGL(k_bwd_dbc_sum, dim3((unsigned)((int64_t)g.K * g.G)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ssd
