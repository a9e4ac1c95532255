// chunk_state.hip -- the standalone chunk-state kernels.  The bf16 body lives in
// stage_state.hpp; fp32 inputs use a simpler slab loop with fp32 matrix
// instructions.  With the step size on the input term (dtc != NULL) each
// token's decay weight is multiplied by its step size.
#include <algorithm>
#include <climits>

#include "kernels.hpp"
#include "stage_state.hpp"

namespace ssd {

template <typename ST, int C>
__global__ __launch_bounds__(256, 4) void k_chunk_state_bf16(Geo g, TArg x, TArg B,
                                                          const float* __restrict__ cs,
                                                          const float* __restrict__ dtc,
                                                          ST* __restrict__ states) {
  __shared__ __align__(16) char smem[chunk_state_lds_bytes<C>()];
  chunk_state_block<ST, C>(g, x, B, cs, dtc, states, blockIdx.x, blockIdx.y, blockIdx.z, smem);
}

// ------------------------------------------------------------------ bf16, C = 128: persistent
//
// Batch mode with whole 64 x NB blocks (P a multiple of 64, N of NB).  One
// item is the 64 (p) x NB (n) block z of the state of (chunk j, head h).  A
// persistent grid of WG_PER_CU workgroups per CU walks the items; while one
// item is multiplied and stored, the next item's x, B, cumsum and step sizes
// are already on their way into registers, so every workgroup keeps loads in
// flight through its whole life instead of waiting on memory once per item.
// An item's output block is read out of LDS at the end of its iteration and
// stored at the start of the next one, after the wait for that next item's
// loads: no store sits between a load and its wait, so the compiler's wait
// counts stay exact (every item is valid, no load is conditional).  x and B
// go to LDS in their natural row-major layout (16-byte rows as loaded) and
// the token-major operands come from the gfx950 LDS transpose read; the decay
// weight multiplies x after that read and x w is split into bf16 hi + lo
// there.  Items are ordered (chunk, head, block) -- the heads of a
// group are consecutive -- and each XCD walks a contiguous share of the
// workgroups, so the heads that share a B tile read it through one L2.  Same
// products in the same order as chunk_state_block (k-slot (q, e) of k-block kb
// is token 32 kb + 8 q + e in both), so both give the same bits.
// NB: the width of an item's block of n.  64 (the default) gives items of
// half the work at four workgroups per CU instead of three: at the
// Nemotron-Nano size 8192 items fill 1024 workgroups exactly (eight each),
// where 4096 items of width 128 left the last of six rounds a third full
// (measured 62.4 against 63.8 us; x is then read by two items, the second
// time from L2).
template <int NB> struct StatePers {
  static constexpr int WG_PER_CU = NB == 128 ? 3 : 4;
  static constexpr int XLD = 64 + 8;    // bf16 per x row
  static constexpr int BLD = NB + 8;    // bf16 per B row
  static constexpr int OLD = NB + 4;    // floats per staged output row
  static constexpr int NTI = NB / 16;   // n-tiles per item
  static constexpr int BV = NB / 16;    // 16-byte B pieces per thread
  static constexpr int BPR = NB / 8;    // 16-byte pieces per B row
  static constexpr int BROWS = 256 / BPR;  // B rows per pass of the workgroup
  static constexpr int OV = NB / 32;    // output 8-vectors per thread
  static constexpr int OFF_X = 0;
  static constexpr int OFF_B = OFF_X + 128 * XLD * 2;
  static constexpr int OFF_W = OFF_B + 128 * BLD * 2;
  static constexpr int LDS = OFF_W + 128 * 4;
  static_assert(64 * OLD * 4 <= 128 * BLD * 2, "the staged output tile fits in the B tile's space");
  static_assert(WG_PER_CU * LDS <= 160 * 1024, "the workgroups of a CU fit its LDS");
};

template <typename ST, int NB>
__global__ __launch_bounds__(256, StatePers<NB>::WG_PER_CU) void k_chunk_state_pers(
    Geo g, TArg x, TArg B, const float* __restrict__ cs, const float* __restrict__ dtc,
    ST* __restrict__ states, int nz, int nitems) {
  using L = StatePers<NB>;
  constexpr int XLD = L::XLD, BLD = L::BLD, OLD = L::OLD, NTI = L::NTI, BV = L::BV;
  constexpr int BPR = L::BPR, BROWS = L::BROWS, OV = L::OV;
  __shared__ __align__(16) char smem[L::LDS];
  bf16* s_x = reinterpret_cast<bf16*>(smem + L::OFF_X);
  bf16* s_b = reinterpret_cast<bf16*>(smem + L::OFF_B);
  float* s_o = reinterpret_cast<float*>(smem + L::OFF_B);
  float* s_w = reinterpret_cast<float*>(smem + L::OFF_W);
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int r16 = lane % 16, q = lane / 16;
  const int nwg = (int)gridDim.x;
  const int nzn = g.N / NB;
  // the step size is read unconditionally (from cs when there is none): a load
  // under a branch would make every later wait a wait for all memory operations
  const float* dsrc = dtc ? dtc : cs;

  struct Item {
    int j, h, p0, n0;
    Chunk c;
  };
  auto decode = [&](int it, Item& m) {
    const int z = it % nz, jh = it / nz;
    m.j = jh / g.H;
    m.h = jh - m.j * g.H;
    m.p0 = (z / nzn) * 64;
    m.n0 = (z % nzn) * NB;
    get_chunk(g, m.j, m.c);  // batch mode: every chunk slot holds tokens
  };
  // registers an item's inputs are loaded into: x rows as 8 threads x 16 B
  // (4 passes of 32 rows), B rows as NB / 8 threads x 16 B, the cumsum and
  // step size of token tid % 128 and the chunk's last cumsum
  struct Regs {
    u32x4 x[4], b[BV];
    float cs_s, cs_last, dt_s;
  };
  auto load = [&](const Item& m, Regs& r) {
    const Chunk& c = m.c;
    const int t = opaque_tid();
    const bf16* xb = row_ptr<bf16>(x, c.b, c.t0, m.h) + m.p0;
    const int xr = t / 8, xc = (t % 8) * 8;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      r.x[k] = *reinterpret_cast<const u32x4*>(xb + (int64_t)min(xr + 32 * k, c.len - 1) * x.s1 + xc);
    const bf16* bb = row_ptr<bf16>(B, c.b, c.t0, m.h / g.hpg) + m.n0;
    const int br = t / BPR, bc = (t % BPR) * 8;
#pragma unroll
    for (int k = 0; k < BV; ++k)
      r.b[k] = *reinterpret_cast<const u32x4*>(bb + (int64_t)min(br + BROWS * k, c.len - 1) * B.s1 + bc);
    const int64_t row = ((int64_t)m.j * g.H + m.h) * 128;
    const int s = min(t % 128, c.len - 1);
    r.cs_s = cs[row + s];
    r.cs_last = cs[row + c.len - 1];
    r.dt_s = dsrc[row + s];
  };

  int it = xcd_remap((int)blockIdx.x, nwg);
  if (it >= nitems) return;
  Item cur;
  Regs r;
  decode(it, cur);
  load(cur, r);
  // an item's output block, read out of LDS at the end of its iteration and
  // stored at the start of the next one, after that item's loads have been
  // waited for: the stores then never sit between a load and its wait
  f32x8 ov[OV];
  ST* pout = nullptr;
  auto store_prev = [&]() {
    const int t = opaque_tid();
#pragma unroll
    for (int k = 0; k < OV; ++k) {
      const int v = t + 256 * k;
      Vec8<ST>::store(pout + (int64_t)(v / BPR) * g.N + (v % BPR) * 8, ov[k]);
    }
  };
  while (true) {
    __syncthreads();  // the previous item's output block has been read out of LDS
    {
      // tokens past the chunk's end (loaded as copies of its last token) are
      // zeroed, and so is their weight
      const int len = cur.c.len;
      const int t = opaque_tid();
      const u32x4 zero = {0u, 0u, 0u, 0u};
      const int xr = t / 8, xc = (t % 8) * 8;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *reinterpret_cast<u32x4*>(&s_x[(xr + 32 * k) * XLD + xc]) = xr + 32 * k < len ? r.x[k] : zero;
      const int br = t / BPR, bc = (t % BPR) * 8;
#pragma unroll
      for (int k = 0; k < BV; ++k)
        *reinterpret_cast<u32x4*>(&s_b[(br + BROWS * k) * BLD + bc]) =
            br + BROWS * k < len ? r.b[k] : zero;
      if (t < 128) s_w[t] = t < len ? fast_exp(r.cs_last - r.cs_s) * (dtc ? r.dt_s : 1.0f) : 0.0f;
    }
    if (pout) store_prev();
    __syncthreads();
    // the next item's loads go out before this item's products (after the
    // last item this item's are loaded again, unused)
    const int nit = it + nwg;
    Item nxt;
    decode(nit < nitems ? nit : it, nxt);
    load(nxt, r);
    f32x4 acc[NTI];
#pragma unroll
    for (int nt = 0; nt < NTI; ++nt) acc[nt] = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int k0 = kb * 32 + q * 8;  // this lane group's 8 tokens
      const u32x4 xv = __builtin_bit_cast(u32x4, lds_frag_tr(s_x, XLD, k0, k0 + 4, wave * 16));
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
      const FragSplit a = split_f32x8(xw);
#pragma unroll
      for (int nt = 0; nt < NTI; ++nt) {
        FragBF b;
        b.v = lds_frag_tr(s_b, BLD, k0, k0 + 4, nt * 16);
        mma(acc[nt], a, b);
      }
    }
    __syncthreads();  // the B tile is dead: its space takes the output block
#pragma unroll
    for (int nt = 0; nt < NTI; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[(wave * 16 + q * 4 + i) * OLD + nt * 16 + r16] = acc[nt][i];
    __syncthreads();
    {
      const int t = opaque_tid();
#pragma unroll
      for (int k = 0; k < OV; ++k) {
        const int v = t + 256 * k;
        ov[k] = Vec8<float>::load(s_o + (v / BPR) * OLD + (v % BPR) * 8);
      }
      pout = states + ((int64_t)cur.j * g.H + cur.h) * g.P * g.N + (int64_t)cur.p0 * g.N + cur.n0;
    }
    if (nit >= nitems) break;
    cur = nxt;
    it = nit;
  }
  store_prev();
}

static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

#ifndef SSD_STATE_NB
#define SSD_STATE_NB 64
#endif
template <typename ST>
static hipError_t launch_state_pers(const Geo& g, TArg x, TArg B, const float* cs,
                                    const float* dtc, ST* st, hipStream_t s) {
  constexpr int NB = SSD_STATE_NB;
  const int nz = (g.P / 64) * (g.N / NB);
  const int64_t items = (int64_t)g.K * g.H * nz;
  const int nwg =
      (int)std::min<int64_t>(items, (int64_t)device_cus() * StatePers<NB>::WG_PER_CU);
  hipLaunchKernelGGL((k_chunk_state_pers<ST, NB>), dim3(nwg), dim3(256), 0, s, g, x, B, cs, dtc,
                     st, nz, (int)items);
  return hipGetLastError();
}

// ------------------------------------------------------------------ fp32 path

constexpr int kSlabF = 32;
struct StateLdsF32 {
  static constexpr int LD = kSlabF + 4;  // 144-byte rows
  float x[64 * LD];
  float bt[128 * LD];
  float w[256];
};

__global__ __launch_bounds__(256) void k_chunk_state_f32(Geo g, TArg x, TArg B,
                                                         const float* __restrict__ cs,
                                                         const float* __restrict__ dtc,
                                                         float* __restrict__ states_f,
                                                         bf16* __restrict__ states_b) {
  __shared__ StateLdsF32 L;
  constexpr int LD = StateLdsF32::LD;
  const int j = blockIdx.x, h = blockIdx.y;
  Chunk c;
  if (!get_chunk(g, j, c)) return;
  const int nzn = (g.N + 127) / 128;
  const int p0 = (blockIdx.z / nzn) * 64, n0 = (blockIdx.z % nzn) * 128;
  const int grp = h / g.hpg;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int r16 = lane % 16, q = lane / 16;
  const float* csr = cs + ((int64_t)j * g.H + h) * g.C;
  const float* dtr = dtc ? dtc + ((int64_t)j * g.H + h) * g.C : nullptr;
  const float last = csr[c.len - 1];
  for (int s = tid; s < g.C; s += blockDim.x)
    L.w[s] = s < c.len ? fast_exp(last - csr[s]) * (dtr ? dtr[s] : 1.0f) : 0.0f;
  __syncthreads();
  const int pt0 = p0 + wave * 16;
  const bool active = pt0 < g.P;
  const int ntn = min(8, (g.N - n0) / 16);
  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = zero4();
  for (int s0 = 0; s0 < c.len; s0 += kSlabF) {
    {
      const int s = tid / 8, pp = (tid % 8) * 8, p = p0 + pp;
      f32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (s0 + s < c.len && p < g.P) {
        v = Vec8<float>::load(row_ptr<float>(x, c.b, c.t0 + s0 + s, h) + p);
        const float ws = L.w[s0 + s];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] *= ws;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) L.x[(pp + i) * LD + s] = v[i];
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int v8 = tid + r * 256;
      const int s = v8 / 16, nn = (v8 % 16) * 8, n = n0 + nn;
      f32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (s0 + s < c.len && n < g.N) v = Vec8<float>::load(row_ptr<float>(B, c.b, c.t0 + s0 + s, grp) + n);
#pragma unroll
      for (int i = 0; i < 8; ++i) L.bt[(nn + i) * LD + s] = v[i];
    }
    __syncthreads();
    if (active) {
      FragF32 a;
      a.v = Vec8<float>::load(&L.x[(wave * 16 + r16) * LD + q * 8]);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (t < ntn) {
          FragF32 b;
          b.v = Vec8<float>::load(&L.bt[(t * 16 + r16) * LD + q * 8]);
          mma(acc[t], a, b);
        }
      }
    }
    __syncthreads();
  }
  if (!active) return;
  const int64_t base = ((int64_t)j * g.H + h) * g.P * g.N;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (t >= ntn) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t o = base + (int64_t)(pt0 + q * 4 + i) * g.N + n0 + t * 16 + r16;
      if (states_f) states_f[o] = acc[t][i];
      else states_b[o] = (bf16)acc[t][i];
    }
  }
}

template <typename ST>
static hipError_t launch_state_bf16(const Geo& g, TArg x, TArg B, const float* cs,
                                    const float* dtc, ST* st, hipStream_t s) {
  dim3 grid(g.K, g.H, ((g.P + 63) / 64) * ((g.N + 127) / 128));
  switch (g.C) {
    case 32: hipLaunchKernelGGL((k_chunk_state_bf16<ST, 32>), grid, dim3(256), 0, s, g, x, B, cs, dtc, st); break;
    case 64: hipLaunchKernelGGL((k_chunk_state_bf16<ST, 64>), grid, dim3(256), 0, s, g, x, B, cs, dtc, st); break;
    case 128: hipLaunchKernelGGL((k_chunk_state_bf16<ST, 128>), grid, dim3(256), 0, s, g, x, B, cs, dtc, st); break;
    default: hipLaunchKernelGGL((k_chunk_state_bf16<ST, 256>), grid, dim3(256), 0, s, g, x, B, cs, dtc, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_chunk_state(const Geo& g, TArg x, TArg B, int in_dtype, const float* cs,
                              const float* dtc, void* states, int st_dtype, hipStream_t s) {
  if (g.K == 0) return hipSuccess;
  const bool pers = g.C == 128 && !g.meta && g.P % 64 == 0 && g.N % SSD_STATE_NB == 0 &&
                    (int64_t)g.K * g.H * (g.P / 64) * (g.N / SSD_STATE_NB) < INT32_MAX;
  if (in_dtype == DT_BF16 && pers) {
    if (st_dtype == DT_BF16) return launch_state_pers<bf16>(g, x, B, cs, dtc, (bf16*)states, s);
    return launch_state_pers<float>(g, x, B, cs, dtc, (float*)states, s);
  }
  if (in_dtype == DT_BF16) {
    if (st_dtype == DT_BF16) return launch_state_bf16<bf16>(g, x, B, cs, dtc, (bf16*)states, s);
    return launch_state_bf16<float>(g, x, B, cs, dtc, (float*)states, s);
  }
  dim3 grid(g.K, g.H, ((g.P + 63) / 64) * ((g.N + 127) / 128));
  hipLaunchKernelGGL(k_chunk_state_f32, grid, dim3(256), 0, s, g, x, B, cs, dtc,
                     st_dtype == DT_BF16 ? nullptr : (float*)states,
                     st_dtype == DT_BF16 ? (bf16*)states : nullptr);
  return hipGetLastError();
}

}  // namespace ssd
