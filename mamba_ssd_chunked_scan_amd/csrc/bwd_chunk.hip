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
constexpr int SLD = 68;     // floats per row of the staging tile
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp_d(double v) { return fast_exp2((float)v * kLog2e); }

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}
// sum over the 16 lanes of a lane group (xor 1, 2, 4, 8 stay inside it)
__device__ __forceinline__ double group16_sum_f64(double v) {
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) v += __shfl_xor(v, d, kWave);
  return v;
}
__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) v += __shfl_xor(v, d, kWave);
  return v;
}
// sum over the 4 lane groups (lanes l, l + 16, l + 32, l + 48)
__device__ __forceinline__ double across_groups_f64(double v) {
  v += __shfl_xor(v, 16, kWave);
  v += __shfl_xor(v, 32, kWave);
  return v;
}
__device__ __forceinline__ float across_groups(float v) {
  v += __shfl_xor(v, 16, kWave);
  v += __shfl_xor(v, 32, kWave);
  return v;
}

__device__ __forceinline__ double block_sum4(double v, double* lds) {
  v = wave_sum_f64(v);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  return lds[0] + lds[1] + lds[2] + lds[3];
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
  float* pdb;             // (nsplit, ntok, G, N) partial dB of each head split (nsplit > 1)
  float* pdc;             // (nsplit, ntok, G, N) partial dC
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

// fp64 inclusive cumsum of a = delta A over the chunk (waves 0 and 1, one
// token per thread; constant past the chunk's end), and f.
__device__ __forceinline__ void stage_cumsum(const BwdChunkArgs& a, const ChunkCtx& x, int h,
                                             double* s_cs, float* s_f, double* s_tmp) {
  const int tid = threadIdx.x;
  const float Ah = a.A[h];
  if (tid < BC) {
    const bool in = tid < x.c.len;
    const float d = in ? a.delta[(int64_t)(x.tp0 + tid) * a.g.H + h] : 0.0f;
    const double v = wave_inclusive_sum_f64(in ? (double)d * (double)Ah : 0.0);
    s_cs[tid] = v;
    s_f[tid] = in ? (a.input_dt ? d : 1.0f) : 0.0f;
    if (tid == kWave - 1) s_tmp[0] = v;
  }
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
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      FragBF bf;
      bf.v = lds_frag_tr(s_c, CLD, k0, k0 + 4, nt * 16);
      mma(acc[nt], af, bf);
    }
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

struct DxLds {
  static constexpr int OFF_CS = 0;                  // double[128]
  static constexpr int OFF_F = 1024;                // float[128]
  static constexpr int OFF_TMP = 1536;              // double[8]
  static constexpr int OFF_ROWP = 1600;             // double[4][128] row sums of M per wave
  static constexpr int OFF_COL = OFF_ROWP + 4096;   // double[128] column sums of M
  static constexpr int OFF_Q = OFF_COL + 1024;      // float[128]
  static constexpr int OFF_R = OFF_Q + 512;         // float[4][128] R partials per wave (p-tile)
  static constexpr int OFF_XG = OFF_R + 2048;       // float[128]
  static constexpr int OFF_DYH = OFF_XG + 512;      // bf16[128][TLD]
  static constexpr int OFF_DYL = OFF_DYH + BC * TLD * 2;
  static constexpr int OFF_X = OFF_DYL + BC * TLD * 2;   // bf16[128][TLD]; then staging
  static constexpr int STAGE_BYTES = BC * SLD * 4;
  static constexpr int X_BYTES = BC * TLD * 2;
  static constexpr int TOTAL = OFF_X + (STAGE_BYTES > X_BYTES ? STAGE_BYTES : X_BYTES);
};
static_assert(DxLds::TOTAL <= 81920, "two workgroups per CU");

template <int NT>
__global__ __launch_bounds__(256, 2) void k_bwd_dx(BwdChunkArgs a) {
  constexpr int NKB = NT / 2;
  __shared__ __align__(16) char smem[DxLds::TOTAL];
  double* s_cs = reinterpret_cast<double*>(smem + DxLds::OFF_CS);
  float* s_f = reinterpret_cast<float*>(smem + DxLds::OFF_F);
  double* s_tmp = reinterpret_cast<double*>(smem + DxLds::OFF_TMP);
  double* s_rowp = reinterpret_cast<double*>(smem + DxLds::OFF_ROWP);
  double* s_col = reinterpret_cast<double*>(smem + DxLds::OFF_COL);
  float* s_q = reinterpret_cast<float*>(smem + DxLds::OFF_Q);
  float* s_r = reinterpret_cast<float*>(smem + DxLds::OFF_R);
  float* s_xg = reinterpret_cast<float*>(smem + DxLds::OFF_XG);
  double* s_dcs = s_rowp;  // (dcs_l replaces the row sums of token l, read by the same thread)
  bf16* s_dyh = reinterpret_cast<bf16*>(smem + DxLds::OFF_DYH);
  bf16* s_dyl = reinterpret_cast<bf16*>(smem + DxLds::OFF_DYL);
  bf16* s_x = reinterpret_cast<bf16*>(smem + DxLds::OFF_X);
  float* s_st = reinterpret_cast<float*>(smem + DxLds::OFF_X);

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

  stage_cumsum(a, cx, h, s_cs, s_f, s_tmp);
  const double lam = s_cs[len - 1];

  // ---- x and dy = dout silu(z) to LDS (dy as bf16 hi + lo); D's gradient
  // share sum(dy . x) on the way
  const bf16* xb = row_ptr<bf16>(a.x, c.b, c.t0, h);
  const bf16* zb = a.z.p ? row_ptr<bf16>(a.z, c.b, c.t0, h) : nullptr;
  double dyx = 0.0;
  {
    const int row0 = tid / 8, col = (tid % 8) * 8;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int l = row0 + 32 * k;
      const int lc = min(l, len - 1);
      const bool in = l < len;
      const u32x4 xv = *reinterpret_cast<const u32x4*>(at(xb, (uint32_t)(lc * a.x.s1 + col)));
      f32x8 go;
      if (a.dout_bf16) {
        const bf16* db = row_ptr<bf16>(a.dout, c.b, c.t0, h);
        go = bf8_to_f32(*reinterpret_cast<const u32x4*>(at(db, (uint32_t)(lc * a.dout.s1 + col))));
      } else {
        const float* db = row_ptr<float>(a.dout, c.b, c.t0, h);
        go = load8f(at(db, (uint32_t)(lc * a.dout.s1 + col)));
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
      const u32x4 zero = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&s_x[l * TLD + col]) = in ? xv : zero;
      *reinterpret_cast<bf16x8*>(&s_dyh[l * TLD + col]) = sp.hi;
      *reinterpret_cast<bf16x8*>(&s_dyl[l * TLD + col]) = sp.lo;
    }
  }
  // <dS, Hin> (for the last token's Lambda term), fp64
  const float* hin = a.hin + ((int64_t)j * g.H + h) * PN;
  double ip = 0.0;
  {
    for (int k = tid * 4; k < PN; k += 256 * 4) {
      const f32x4 u = *reinterpret_cast<const f32x4*>(cx.ds + k);
      const f32x4 v = *reinterpret_cast<const f32x4*>(hin + k);
#pragma unroll
      for (int i = 0; i < 4; ++i) ip += (double)u[i] * (double)v[i];
    }
  }
  __syncthreads();

  // C and B row fragments (n contiguous): rows past the chunk and columns past
  // N read as zero
  const bf16* cbase = row_ptr<bf16>(a.C, c.b, c.t0, grp);
  const bf16* bbase = row_ptr<bf16>(a.B, c.b, c.t0, grp);
  auto nrow_frag = [&](const bf16* base, int64_t s1, int row, int kb) -> u32x4 {
    const int n = kb * 32 + q * 8;
    const u32x4 v = *reinterpret_cast<const u32x4*>(
        at(base, (uint32_t)(min(row, len - 1) * s1 + min(n, g.N - 8))));
    const u32x4 zero = {0u, 0u, 0u, 0u};
    return (row < len && n < g.N) ? v : zero;
  };
  // a state row (P x N fp32, row p) as an operand fragment of 8 n, split
  auto state_frag = [&](const float* st, int p, int kb, float scale) -> FragSplit {
    const int n = kb * 32 + q * 8;
    f32x8 v = load8f(st + (int64_t)p * g.N + min(n, g.N - 8));
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = n < g.N ? v[i] * scale : 0.0f;
    return split_f32x8(v);
  };

  const int ltA = wave, ltB = 7 - wave;

  // ---- Y_diag = (L o C.B^T + D I) x for l-tiles ltA, ltB (layout A tiles, as
  // in the fused forward): rows l, all four p-tiles
  f32x4 yd[2][4];
#pragma unroll
  for (int ui = 0; ui < 2; ++ui)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) yd[ui][pt] = zero4();
#pragma unroll
  for (int ui = 0; ui < 2; ++ui) {
    const int lt = ui ? ltB : ltA;
    const int lrow = lt * 16 + r16;
    u32x4 cf[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) cf[kb] = nrow_frag(cbase, a.C.s1, lrow, kb);
    const double csl = s_cs[lrow];
    for (int kp = 0; kp <= lt / 2; ++kp) {
      const int sa = 2 * kp, sb = 2 * kp + 1;
      f32x4 va = zero4(), vb = zero4();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        mma(va, as_frag(nrow_frag(bbase, a.B.s1, sa * 16 + r16, kb)), as_frag(cf[kb]));
        mma(vb, as_frag(nrow_frag(bbase, a.B.s1, sb * 16 + r16, kb)), as_frag(cf[kb]));
      }
      f32x8 m;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int s_a = sa * 16 + q * 4 + e4, s_b = sb * 16 + q * 4 + e4;
        const float ma = exp_d(csl - s_cs[s_a]) * s_f[s_a] * va[e4];
        const float mb = exp_d(csl - s_cs[s_b]) * s_f[s_b] * vb[e4];
        m[e4] = s_a < lrow ? ma : (s_a == lrow ? ma + Dh : 0.0f);
        m[4 + e4] = s_b < lrow ? mb : (s_b == lrow ? mb + Dh : 0.0f);
      }
      const FragSplit mf = split_f32x8(m);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        FragBF xf;
        xf.v = lds_frag_tr(s_x, TLD, sa * 16 + q * 4, sb * 16 + q * 4, pt * 16);
        mma(yd[ui][pt], mf, xf);
      }
    }
  }

  // ---- Y_off = exp(cs_l) C_l . Hin for p-tile `wave`, all l-tiles (each wave
  // splits only its own 16 rows of Hin)
  f32x4 yo[8];
#pragma unroll
  for (int lt = 0; lt < 8; ++lt) yo[lt] = zero4();
  {
    const int pr = wave * 16 + r16;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const FragSplit hf = state_frag(hin, pr, kb, 1.0f);
#pragma unroll
      for (int lt = 0; lt < 8; ++lt)
        mma(yo[lt], as_frag(nrow_frag(cbase, a.C.s1, lt * 16 + r16, kb)), hf);
    }
#pragma unroll
    for (int lt = 0; lt < 8; ++lt)
#pragma unroll
      for (int i = 0; i < 4; ++i) yo[lt][i] *= exp_d(s_cs[lt * 16 + q * 4 + i]);
  }
  __syncthreads();  // the x tile is dead: its space takes the staging tile
  // stage Y_off; Q_l = dy_l . Y_off_l; then add Y_diag: y
#pragma unroll
  for (int lt = 0; lt < 8; ++lt)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_st[(lt * 16 + q * 4 + i) * SLD + wave * 16 + r16] = yo[lt][i];
  __syncthreads();
  {
    const int l = tid / 2, p0 = (tid % 2) * 32;
    float qs = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4 hv = *reinterpret_cast<const u32x4*>(&s_dyh[l * TLD + p0 + 8 * k]);
      const u32x4 lv = *reinterpret_cast<const u32x4*>(&s_dyl[l * TLD + p0 + 8 * k]);
      const f32x8 hf = bf8_to_f32(hv), lf = bf8_to_f32(lv);
#pragma unroll
      for (int i = 0; i < 8; ++i) qs += (hf[i] + lf[i]) * s_st[l * SLD + p0 + 8 * k + i];
    }
    qs += __shfl_xor(qs, 1, kWave);
    if ((tid % 2) == 0) s_q[l] = qs;
  }
  __syncthreads();
#pragma unroll
  for (int ui = 0; ui < 2; ++ui) {
    const int lt = ui ? ltB : ltA;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_st[(lt * 16 + q * 4 + i) * SLD + pt * 16 + r16] += yd[ui][pt][i];
  }
  __syncthreads();
  // ---- dz = dout y silu'(z), silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z)))
  if (zb) {
    const int row0 = tid / 8, col = (tid % 8) * 8;
    float* dzb = row_ptr_mut<float>(a.dz, c.b, c.t0, h);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int l = row0 + 32 * k;
      const int lc = min(l, len - 1);
      f32x8 go;
      if (a.dout_bf16) {
        const bf16* db = row_ptr<bf16>(a.dout, c.b, c.t0, h);
        go = bf8_to_f32(*reinterpret_cast<const u32x4*>(at(db, (uint32_t)(lc * a.dout.s1 + col))));
      } else {
        const float* db = row_ptr<float>(a.dout, c.b, c.t0, h);
        go = load8f(at(db, (uint32_t)(lc * a.dout.s1 + col)));
      }
      const f32x8 zz = bf8_to_f32(*reinterpret_cast<const u32x4*>(at(zb, (uint32_t)(lc * a.z.s1 + col))));
      f32x8 o;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float sg = sigmoidf(zz[i]);
        o[i] = go[i] * s_st[l * SLD + col + i] * (sg * (1.0f + zz[i] * (1.0f - sg)));
      }
      if (l < len) Vec8<float>::store(at(dzb, (uint32_t)(l * a.dz.s1 + col)), o);
    }
  }
  __syncthreads();  // y is dead: the staging tile takes g

  // ---- inter-chunk part of g: exp(Lambda - cs_s) dS B_s, as g^T tiles (rows
  // p of p-tile `wave`, columns s of every s-tile); R partials on the way
  {
    f32x4 go_[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) go_[st] = zero4();
    {
      const int pr = wave * 16 + r16;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const FragSplit df = state_frag(cx.ds, pr, kb, 1.0f);
#pragma unroll
        for (int st = 0; st < 8; ++st)
          mma(go_[st], df, as_frag(nrow_frag(bbase, a.B.s1, st * 16 + r16, kb)));
      }
    }
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int s = st * 16 + r16;
      const float e = s < len ? exp_d(lam - s_cs[s]) : 0.0f;
      // x[s][p] for p = 16 wave + 4 q + 0..3
      const uint2 xv = *reinterpret_cast<const uint2*>(
          at(xb, (uint32_t)(min(s, len - 1) * a.x.s1 + wave * 16 + q * 4)));
      const float x4[4] = {bf16_lo_f32(xv.x), bf16_hi_f32(xv.x), bf16_lo_f32(xv.y),
                           bf16_hi_f32(xv.y)};
      float rp = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        go_[st][i] *= e;
        rp += x4[i] * go_[st][i];
      }
      rp = across_groups(rp);
      if (q == 0) s_r[wave * BC + s] = s < len ? rp : 0.0f;
      *reinterpret_cast<f32x4*>(&s_st[s * SLD + wave * 16 + q * 4]) = go_[st];
    }
  }

  // ---- intra-chunk part of g^T = dy^T (L o C.B^T) for s-tiles ltA, ltB
  // (layout B tiles), with the row and column sums of M = (L o C.B^T) o
  // (dy.x^T) f (strictly lower triangle) in fp64
  f32x4 gd_[2][4];
#pragma unroll
  for (int ui = 0; ui < 2; ++ui)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) gd_[ui][pt] = zero4();
  for (int i = tid; i < 4 * BC; i += 256) s_rowp[i] = 0.0;
  __syncthreads();  // (the g^T staging above, and the row sums' zeroing, are done)
#pragma unroll
  for (int ui = 0; ui < 2; ++ui) {
    const int sbt = ui ? ltB : ltA;
    const int s = sbt * 16 + r16;
    u32x4 bf[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) bf[kb] = nrow_frag(bbase, a.B.s1, s, kb);
    u32x4 xr[2];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(
          at(xb, (uint32_t)(min(s, len - 1) * a.x.s1 + kp * 32 + q * 8)));
      const u32x4 zero = {0u, 0u, 0u, 0u};
      xr[kp] = s < len ? v : zero;
    }
    const double css = s_cs[s];
    const float fs = s_f[s];
    double colp = 0.0;
    for (int lp = sbt / 2; lp < 4; ++lp) {
      const int la = 2 * lp, lb = 2 * lp + 1;
      f32x4 ca = zero4(), cb = zero4(), xa = zero4(), xb2 = zero4();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        mma(ca, as_frag(nrow_frag(cbase, a.C.s1, la * 16 + r16, kb)), as_frag(bf[kb]));
        mma(cb, as_frag(nrow_frag(cbase, a.C.s1, lb * 16 + r16, kb)), as_frag(bf[kb]));
      }
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        const int pc = kp * 32 + q * 8;
        mma(xa, lds_split(&s_dyh[(la * 16 + r16) * TLD + pc], &s_dyl[(la * 16 + r16) * TLD + pc]),
            as_frag(xr[kp]));
        mma(xb2, lds_split(&s_dyh[(lb * 16 + r16) * TLD + pc], &s_dyl[(lb * 16 + r16) * TLD + pc]),
            as_frag(xr[kp]));
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
      for (int pt = 0; pt < 4; ++pt) {
        FragSplit dyt;
        dyt.hi = lds_frag_tr(s_dyh, TLD, la * 16 + q * 4, lb * 16 + q * 4, pt * 16);
        dyt.lo = lds_frag_tr(s_dyl, TLD, la * 16 + q * 4, lb * 16 + q * 4, pt * 16);
        mma(gd_[ui][pt], dyt, mf);
      }
      // row sums of this pair of tiles: over the 16 columns s of the lane group
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const double ra = group16_sum_f64(rowa[e4]);
        const double rb = group16_sum_f64(rowb[e4]);
        if (r16 == 0) {
          s_rowp[wave * BC + la * 16 + q * 4 + e4] += ra;
          s_rowp[wave * BC + lb * 16 + q * 4 + e4] += rb;
        }
      }
    }
    colp = across_groups_f64(colp);
    if (q == 0) s_col[s] = colp;
  }
  // g = intra + inter in the staging tile (rows s, columns p)
#pragma unroll
  for (int ui = 0; ui < 2; ++ui) {
    const int sbt = ui ? ltB : ltA;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      f32x4* dst = reinterpret_cast<f32x4*>(&s_st[(sbt * 16 + r16) * SLD + pt * 16 + q * 4]);
      *dst = *dst + gd_[ui][pt];
    }
  }
  __syncthreads();
  // ---- dx = f g + D dy; x . g for the step size on the input term
  {
    const int row0 = tid / 8, col = (tid % 8) * 8;
    float* dxb = row_ptr_mut<float>(a.dx, c.b, c.t0, h);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int s = row0 + 32 * k;
      const f32x8 gv = Vec8<float>::load(s_st + s * SLD + col);
      const f32x8 hf = bf8_to_f32(*reinterpret_cast<const u32x4*>(&s_dyh[s * TLD + col]));
      const f32x8 lf = bf8_to_f32(*reinterpret_cast<const u32x4*>(&s_dyl[s * TLD + col]));
      const float fs = s_f[s];
      f32x8 o;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = fs * gv[i] + Dh * (hf[i] + lf[i]);
      if (s < len) Vec8<float>::store(at(dxb, (uint32_t)(s * a.dx.s1 + col)), o);
      if (a.input_dt) {
        const f32x8 xf = bf8_to_f32(*reinterpret_cast<const u32x4*>(
            at(xb, (uint32_t)(min(s, len - 1) * a.x.s1 + col))));
        float e = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) e += xf[i] * gv[i];
        e += __shfl_xor(e, 1, kWave);
        e += __shfl_xor(e, 2, kWave);
        e += __shfl_xor(e, 4, kWave);
        if ((tid % 8) == 0) s_xg[s] = s < len ? e : 0.0f;
      }
    }
  }
  // ---- dcs, and its suffix sums: dL/da_t
  const double sip = block_sum4(ip, s_tmp);  // (its barriers publish the sums above)
  if (tid < BC) {
    const int l = tid;
    double v = 0.0, rl = 0.0;
    if (l < len) {
      rl = (double)s_f[l] * ((double)s_r[l] + s_r[BC + l] + s_r[2 * BC + l] + s_r[3 * BC + l]);
      v = s_rowp[l] + s_rowp[BC + l] + s_rowp[2 * BC + l] + s_rowp[3 * BC + l] - s_col[l] +
          (double)s_q[l] - rl;
    }
    s_dcs[l] = v;
    // sum of R over the chunk (wave 0 and 1 each hold 64 tokens)
    const double rs = wave_sum_f64(rl);
    if (lane == 0) s_tmp[4 + wave] = rs;
  }
  __syncthreads();
  if (tid == 0)
    s_dcs[len - 1] += (double)exp_d(lam) * sip + s_tmp[4] + s_tmp[5];
  __syncthreads();
  double sa = 0.0, sb = 0.0, suf = 0.0;
  if (tid < BC) {
    // suffix sums by a reversed inclusive scan: thread t holds token 127 - t
    suf = wave_inclusive_sum_f64(s_dcs[BC - 1 - tid]);
    if (tid == kWave - 1) s_tmp[6] = suf;
  }
  __syncthreads();
  if (tid < BC) {
    const int l = BC - 1 - tid;
    const double da = suf + (tid >= kWave ? s_tmp[6] : 0.0);
    if (l < len) {
      const int64_t it = (int64_t)(cx.tp0 + l) * g.H + h;
      const double gg = (da * (double)Ah + (a.input_dt ? (double)s_xg[l] : 0.0)) * (double)a.gd[it];
      row_ptr_mut<float>(a.ddt, c.b, c.t0 + l, h)[0] = (float)gg;
      sa = da * (double)a.delta[it];
      sb = gg;
    }
  }
  sa = block_sum4(sa, s_tmp);
  sb = block_sum4(sb, s_tmp);
  dyx = block_sum4(dyx, s_tmp);
  if (tid == 0) {
    pj[0] = sa;
    pj[1] = sb;
    pj[2] = dyx;
  }
}

// ---------------------------------------------------------------- k_bwd_dbc

struct DbcLds {
  static constexpr int OFF_CS = 0;                   // double[128]
  static constexpr int OFF_F = 1024;                 // float[128]
  static constexpr int OFF_EL = 1536;                // float[128] exp(cs_l)
  static constexpr int OFF_ES = 2048;                // float[128] f_s exp(Lambda - cs_s)
  static constexpr int OFF_TMP = 2560;               // double[8]
  static constexpr int OFF_BT = 2624;                // bf16[128][TLD] B slab
  static constexpr int OFF_CT = OFF_BT + BC * TLD * 2;     // bf16[128][TLD] C slab
  static constexpr int OFF_SH = OFF_CT + BC * TLD * 2;     // bf16[64][TLD] state slab hi
  static constexpr int OFF_SL = OFF_SH + 64 * TLD * 2;     // bf16[64][TLD] state slab lo
  static constexpr int TOTAL = OFF_SL + 64 * TLD * 2;
};
static_assert(DbcLds::TOTAL <= 81920, "two workgroups per CU");

__global__ __launch_bounds__(256, 2) void k_bwd_dbc(BwdChunkArgs a) {
  __shared__ __align__(16) char smem[DbcLds::TOTAL];
  double* s_cs = reinterpret_cast<double*>(smem + DbcLds::OFF_CS);
  float* s_f = reinterpret_cast<float*>(smem + DbcLds::OFF_F);
  float* s_el = reinterpret_cast<float*>(smem + DbcLds::OFF_EL);
  float* s_es = reinterpret_cast<float*>(smem + DbcLds::OFF_ES);
  double* s_tmp = reinterpret_cast<double*>(smem + DbcLds::OFF_TMP);
  bf16* s_bt = reinterpret_cast<bf16*>(smem + DbcLds::OFF_BT);
  bf16* s_ct = reinterpret_cast<bf16*>(smem + DbcLds::OFF_CT);
  bf16* s_sh = reinterpret_cast<bf16*>(smem + DbcLds::OFF_SH);
  bf16* s_sl = reinterpret_cast<bf16*>(smem + DbcLds::OFF_SL);

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
  // ---- B and C slabs of the chunk (rows past the chunk, columns past N: 0)
  {
    const bf16* bb = row_ptr<bf16>(a.B, c.b, c.t0, grp) + n0;
    const bf16* cb = row_ptr<bf16>(a.C, c.b, c.t0, grp) + n0;
    const int row0 = tid / 8, col = (tid % 8) * 8;
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int l = row0 + 32 * k;
      const int lc = min(l, len - 1), cc = min(col, nw - 8);
      const bool ok = l < len && col < nw;
      const u32x4 vb = *reinterpret_cast<const u32x4*>(at(bb, (uint32_t)(lc * a.B.s1 + cc)));
      const u32x4 vc = *reinterpret_cast<const u32x4*>(at(cb, (uint32_t)(lc * a.C.s1 + cc)));
      *reinterpret_cast<u32x4*>(&s_bt[l * TLD + col]) = ok ? vb : zero;
      *reinterpret_cast<u32x4*>(&s_ct[l * TLD + col]) = ok ? vc : zero;
    }
  }

  const int ltA = wave, ltB = 7 - wave;
  f32x4 dc[2][4], db[2][4];
#pragma unroll
  for (int ui = 0; ui < 2; ++ui)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      dc[ui][nt] = zero4();
      db[ui][nt] = zero4();
    }

  // dy = dout silu(z): row fragment (8 consecutive p) of token l of the chunk;
  // rows past the chunk read as zero
  auto dy_row = [&](int h, int l, int kp) -> f32x8 {
    const int lc = min(l, len - 1), col = kp * 32 + q * 8;
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
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = l < len ? v[i] : 0.0f;
    return v;
  };
  auto x_row = [&](const bf16* xb, int s, int kp) -> u32x4 {
    const u32x4 v = *reinterpret_cast<const u32x4*>(
        at(xb, (uint32_t)(min(s, len - 1) * a.x.s1 + kp * 32 + q * 8)));
    const u32x4 zero = {0u, 0u, 0u, 0u};
    return s < len ? v : zero;
  };
  // stage rows p of a (P x N) fp32 state slab, times `scale`, as bf16 hi + lo
  auto stage_state = [&](const float* st, float scale) {
    const int p = tid / 4, cbase = (tid % 4) * 16;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int col = cbase + 8 * k;
      f32x8 v;
      if (st) {
        v = load8f(st + (int64_t)p * g.N + n0 + min(col, nw - 8));
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = col < nw ? v[i] * scale : 0.0f;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
      }
      const FragSplit sp = split_f32x8(v);
      *reinterpret_cast<bf16x8*>(&s_sh[p * TLD + col]) = sp.hi;
      *reinterpret_cast<bf16x8*>(&s_sl[p * TLD + col]) = sp.lo;
    }
  };

  for (int h = h_lo; h < h_hi; ++h) {
    ChunkCtx cx;
    chunk_ctx(a, j, h, cx);
    __syncthreads();  // the previous head is done with the cumsum and the state slab
    stage_cumsum(a, cx, h, s_cs, s_f, s_tmp);
    const double lam = s_cs[len - 1];
    if (tid < BC) {
      const bool in = tid < len;
      s_el[tid] = in ? exp_d(s_cs[tid]) : 0.0f;
      s_es[tid] = in ? s_f[tid] * exp_d(lam - s_cs[tid]) : 0.0f;
    }
    stage_state(a.hin + ((int64_t)j * g.H + h) * PN, 1.0f);
    __syncthreads();
    const bf16* xb = row_ptr<bf16>(a.x, c.b, c.t0, h);

    // ---- dC for l-tiles ltA, ltB: intra sum_s (L o dy.x^T f)_ls B_s (layout
    // A tiles: dy.x^T computed as [s][l]) and inter exp(cs_l) dy_l Hin
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int lt = ui ? ltB : ltA;
      const int l = lt * 16 + r16;
      FragSplit dyf[2];
      f32x8 dyv[2];
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        dyv[kp] = dy_row(h, l, kp);
        dyf[kp] = split_f32x8(dyv[kp]);
      }
      const double csl = s_cs[l];
      for (int kp2 = 0; kp2 <= lt / 2; ++kp2) {
        const int sa = 2 * kp2, sb = 2 * kp2 + 1;
        f32x4 va = zero4(), vb = zero4();
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          mma(va, as_frag(x_row(xb, sa * 16 + r16, kp)), dyf[kp]);
          mma(vb, as_frag(x_row(xb, sb * 16 + r16, kp)), dyf[kp]);
        }
        f32x8 w;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int s_a = sa * 16 + q * 4 + e4, s_b = sb * 16 + q * 4 + e4;
          w[e4] = s_a <= l ? exp_d(csl - s_cs[s_a]) * s_f[s_a] * va[e4] : 0.0f;
          w[4 + e4] = s_b <= l ? exp_d(csl - s_cs[s_b]) * s_f[s_b] * vb[e4] : 0.0f;
        }
        const FragSplit wf = split_f32x8(w);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          FragBF bt;
          bt.v = lds_frag_tr(s_bt, TLD, sa * 16 + q * 4, sb * 16 + q * 4, nt * 16);
          mma(dc[ui][nt], wf, bt);
        }
      }
      const float el = s_el[min(l, BC - 1)];
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        f32x8 v = dyv[kp];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] *= el;
        const FragSplit af = split_f32x8(v);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          FragSplit hs;
          hs.hi = lds_frag_tr(s_sh, TLD, kp * 32 + q * 8, kp * 32 + q * 8 + 4, nt * 16);
          hs.lo = lds_frag_tr(s_sl, TLD, kp * 32 + q * 8, kp * 32 + q * 8 + 4, nt * 16);
          mma(dc[ui][nt], af, hs);
        }
      }
    }
    __syncthreads();  // the Hin slab is dead: dS takes its place
    stage_state(cx.ds, 1.0f);
    __syncthreads();

    // ---- dB for s-tiles ltA, ltB: intra f_s sum_l (L o dy.x^T)_ls C_l (layout
    // B tiles: dy.x^T as [l][s]) and inter f_s exp(Lambda - cs_s) x_s dS
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int sbt = ui ? ltB : ltA;
      const int s = sbt * 16 + r16;
      u32x4 xr[2];
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) xr[kp] = x_row(xb, s, kp);
      const double css = s_cs[s];
      const float fs = s_f[min(s, BC - 1)];
      for (int lp = sbt / 2; lp < 4; ++lp) {
        const int la = 2 * lp, lb = 2 * lp + 1;
        f32x4 va = zero4(), vb = zero4();
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          mma(va, split_f32x8(dy_row(h, la * 16 + r16, kp)), as_frag(xr[kp]));
          mma(vb, split_f32x8(dy_row(h, lb * 16 + r16, kp)), as_frag(xr[kp]));
        }
        f32x8 w;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int l_a = la * 16 + q * 4 + e4, l_b = lb * 16 + q * 4 + e4;
          w[e4] = s <= l_a ? exp_d(s_cs[l_a] - css) * fs * va[e4] : 0.0f;
          w[4 + e4] = s <= l_b ? exp_d(s_cs[l_b] - css) * fs * vb[e4] : 0.0f;
        }
        const FragSplit wf = split_f32x8(w);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          FragBF ct;
          ct.v = lds_frag_tr(s_ct, TLD, la * 16 + q * 4, lb * 16 + q * 4, nt * 16);
          mma(db[ui][nt], wf, ct);
        }
      }
      const float es = s_es[min(s, BC - 1)];
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        f32x8 v = bf8_to_f32(xr[kp]);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] *= es;
        const FragSplit af = split_f32x8(v);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          FragSplit ds;
          ds.hi = lds_frag_tr(s_sh, TLD, kp * 32 + q * 8, kp * 32 + q * 8 + 4, nt * 16);
          ds.lo = lds_frag_tr(s_sl, TLD, kp * 32 + q * 8, kp * 32 + q * 8 + 4, nt * 16);
          mma(db[ui][nt], af, ds);
        }
      }
    }
  }

  // ---- store: accumulator tile [row][n], lane: column n = 16 nt + r16, rows
  // 4 q + 0..3
#pragma unroll
  for (int ui = 0; ui < 2; ++ui) {
    const int rt = ui ? ltB : ltA;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int n = nt * 16 + r16;
      if (n >= nw) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rt * 16 + q * 4 + i;
        if (r >= len) continue;
        if (a.nsplit == 1) {
          row_ptr_mut<float>(a.dC, c.b, c.t0 + r, grp)[n0 + n] = dc[ui][nt][i];
          row_ptr_mut<float>(a.dB, c.b, c.t0 + r, grp)[n0 + n] = db[ui][nt][i];
        } else {
          const int64_t o = (((int64_t)sp * a.ntok + tp0 + r) * g.G + grp) * g.N + n0 + n;
          a.pdc[o] = dc[ui][nt][i];
          a.pdb[o] = db[ui][nt][i];
        }
      }
    }
  }
}

// ---- dB and dC of a chunk and group: the head splits' partial sums, added in
// split order
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
  if (g.N <= 64) hipLaunchKernelGGL(k_bwd_dx<4>, dim3(nx), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_bwd_dx<8>, dim3(nx), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned nb = (unsigned)((int64_t)g.K * g.G * a.nsplit * a.nsl);
  hipLaunchKernelGGL(k_bwd_dbc, dim3(nb), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL(k_bwd_dbc_sum, dim3((unsigned)((int64_t)g.K * g.G)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ssd
