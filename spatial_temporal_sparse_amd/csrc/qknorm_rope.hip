// Fused QK-RMSNorm + 3D rotary embedding of Q and K.  The Sparse VideoGen pages name both
// operations as a cost worth a custom kernel (authors' article, closing "other
// optimisations" section; 机器之心 article, end of the layout section) without defining
// them; this kernel computes, per row of D channels,
//   y = x / sqrt(mean(x^2) + eps) * w,   then rotates channel pairs (2j, 2j+1) of the
//   frame / grid-row / grid-column slice (widths dt, dh, dw) by pos * base^(-2j/n).
//
// HBM-bound: each row is read once and written once (2 x D x 2 bytes), everything else is
// register or LDS work.  Loads and stores are non-temporal (nt): the outputs then go to HBM
// during this kernel instead of staying dirty in the Infinity Cache until the profiling pass
// that follows evicts them.  Measured at 720p, that moves about 0.03-0.04 ms from profiling to
// this kernel, and the two together take 0.78-0.81 ms against 0.83 ms with cached accesses.  D/8 lanes own a row (8 channels = one 16-byte vector each); the
// sum of squares is reduced across those lanes with DPP lane permutations.  The cos/sin of
// every (axis, position, pair) -- F*dt/2 + HH*dh/2 + WW*dw/2 entries -- are computed once
// per block and kept in LDS as fp32 pairs, so no transcendental runs per element: the
// inverse frequency of each (axis, pair) in fp64, each angle in fp64 reduced to [-pi, pi],
// its cosine and sine in fp32 (within about one fp32 ulp of the exact values).
#include "svg_internal.h"

namespace svg {

namespace {

constexpr int ROPE_THREADS = 256;
constexpr int ROPE_UNROLL = 2;     // rows per lane and batch (two batches in flight)

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
  return __uint_as_float(h << 16);
}

// v + the value of lane (l ^ m) within groups of four lanes, or mirrored within a row of 8 or
// 16 lanes, through DPP (no LDS round trip)
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
// sum over the N (8 or 16) consecutive lanes of a row group; every lane gets the total
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  v = dpp_add<0xB1>(v);      // quad_perm [1,0,3,2]: pairs
  v = dpp_add<0x4E>(v);      // quad_perm [2,3,0,1]: quads
  v = dpp_add<0x141>(v);     // row_half_mirror: groups of 8
  if constexpr (N == 16) v = dpp_add<0x140>(v);   // row_mirror: groups of 16
  return v;
}

template <int D>
__global__ __launch_bounds__(ROPE_THREADS) void qknorm_rope_kernel(RopeArgs a) {
  extern __shared__ float2 tab[];
  constexpr int LPR = D / 8;                 // lanes per row
  constexpr int RPP = ROPE_THREADS / LPR;    // rows per pass of the block
  const int which = blockIdx.y;              // 0: Q, 1: K
  const int tid = threadIdx.x;
  const int lane_c = tid % LPR;

  const u32x4* __restrict__ in = reinterpret_cast<const u32x4*>(a.in[which]);
  u32x4* __restrict__ out = reinterpret_cast<u32x4*>(a.out[which]);
  const int64_t total = (int64_t)a.BH * a.S;
  const int64_t stride = (int64_t)gridDim.x * RPP;
  const float inv_d = 1.0f / (float)D;

  // Batches of ROPE_UNROLL rows per lane, software-pipelined: the next batch is loaded before
  // the current one is processed.  The loads are unconditional (rows past the end repeat the
  // last row and are not stored), so the compiler can wait for the older batch only.
  auto load = [&](u32x4 (&raw)[ROPE_UNROLL], int64_t base) {
#pragma unroll
    for (int u = 0; u < ROPE_UNROLL; ++u) {
      const int64_t row = min(base + u * stride, total - 1);
      raw[u] = __builtin_nontemporal_load(&in[row * LPR + lane_c]);
    }
  };
  const int64_t step = stride * ROPE_UNROLL;
  u32x4 ra[ROPE_UNROLL], rb[ROPE_UNROLL];
  int64_t base = (int64_t)blockIdx.x * RPP + tid / LPR;
  // the first rows are fetched before the tables are built, so that their latency overlaps
  load(ra, base);

  // ---- per-block cos/sin tables: inverse frequencies base^(-2j/n) in fp64 (one pow per axis
  // and pair), angles pos * freq in fp64 reduced to [-pi, pi], cos/sin in fp32 ----
  __shared__ double invf[3 * 64];
  const int nt = a.dt / 2, nh = a.dh / 2, nw = a.dw / 2;
  if (tid < nt + nh + nw) {
    int j, n;
    if (tid < nt) { j = tid; n = a.dt; }
    else if (tid < nt + nh) { j = tid - nt; n = a.dh; }
    else { j = tid - nt - nh; n = a.dw; }
    invf[tid] = pow(a.base, -2.0 * (double)j / (double)n);
  }
  __syncthreads();
  const int Et = a.F * nt, Eh = a.HH * nh, Ew = a.WW * nw;
  for (int e = tid; e < Et + Eh + Ew; e += ROPE_THREADS) {
    int pos, f;
    if (e < Et) { pos = e / nt; f = e - pos * nt; }
    else if (e < Et + Eh) { const int r = e - Et; pos = r / nh; f = nt + r - pos * nh; }
    else { const int r = e - Et - Eh; pos = r / nw; f = nt + nh + r - pos * nw; }
    const double theta = (double)pos * invf[f];
    const double r2 = theta - 6.283185307179586 * rint(theta * 0.15915494309189535);
    float s, c;
    sincosf((float)r2, &s, &c);
    tab[e] = make_float2(c, s);
  }

  // ---- this lane's four channel pairs: table base and per-position stride ----
  int tab_base[4], tab_stride[4], axis[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pp = lane_c * 4 + i;
    if (pp < nt) { axis[i] = 0; tab_base[i] = pp; tab_stride[i] = nt; }
    else if (pp < nt + nh) { axis[i] = 1; tab_base[i] = Et + (pp - nt); tab_stride[i] = nh; }
    else { axis[i] = 2; tab_base[i] = Et + Eh + (pp - nt - nh); tab_stride[i] = nw; }
  }
  float w[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) w[c] = a.w[which][lane_c * 8 + c];
  __syncthreads();

  auto process = [&](const u32x4 (&raw)[ROPE_UNROLL], int64_t base) {
#pragma unroll
    for (int u = 0; u < ROPE_UNROLL; ++u) {
      const int64_t row = base + u * stride;
      // every lane of a row takes the same branch, so the shuffles below see whole rows
      if (row >= total) break;
      float x[8];
      const u32x4 wd = raw[u];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        x[2 * c] = bf16_bits_to_float(wd[c] & 0xffffu);
        x[2 * c + 1] = bf16_bits_to_float(wd[c] >> 16);
      }
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) ss = fmaf(x[c], x[c], ss);
      ss = group_sum<LPR>(ss);
      const float rs = rsqrtf(ss * inv_d + a.eps);

      const uint32_t tok = (uint32_t)(row - (int64_t)fdiv((uint32_t)row, a.divS) * a.S);
      const uint32_t f = fdiv(tok, a.divP);
      const uint32_t p = tok - f * (uint32_t)a.P;
      const uint32_t y = fdiv(p, a.divWW);
      const uint32_t xx = p - y * (uint32_t)a.WW;

      bf16x8 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float aa = x[2 * i] * rs * w[2 * i];
        const float bb = x[2 * i + 1] * rs * w[2 * i + 1];
        const int pos = axis[i] == 0 ? (int)f : (axis[i] == 1 ? (int)y : (int)xx);
        const float2 cs = tab[tab_base[i] + pos * tab_stride[i]];
        o[2 * i] = (bf16)(aa * cs.x - bb * cs.y);
        o[2 * i + 1] = (bf16)(aa * cs.y + bb * cs.x);
      }
      __builtin_nontemporal_store(__builtin_bit_cast(u32x4, o), &out[row * LPR + lane_c]);
    }
  };

  for (; base < total; base += 2 * step) {
    load(rb, base + step);
    process(ra, base);
    if (base + step >= total) break;
    load(ra, base + 2 * step);
    process(rb, base + step);
  }
}

}  // namespace

hipError_t launch_qknorm_rope(const RopeArgs& a, hipStream_t st) {
  const size_t lds = sizeof(float2) * (size_t)(a.F * (a.dt / 2) + a.HH * (a.dh / 2) + a.WW * (a.dw / 2));
  const int64_t total = (int64_t)a.BH * a.S;
  const int rpp = ROPE_THREADS / (a.D / 8);
  // a persistent grid of one block per CU and tensor, so that each block builds its cos/sin
  // tables once and then streams many rows (more blocks measured slower)
  int64_t blocks = (total + rpp * ROPE_UNROLL - 1) / (rpp * ROPE_UNROLL);
  if (blocks > 256) blocks = 256;
  const dim3 grid((unsigned)blocks, 2);
  if (a.D == 128) {
    qknorm_rope_kernel<128><<<grid, ROPE_THREADS, lds, st>>>(a);
  } else if (a.D == 64) {
    qknorm_rope_kernel<64><<<grid, ROPE_THREADS, lds, st>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace svg
