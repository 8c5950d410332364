// Head-adaptive block-sparse attention with an LSE-cached block search, after the AdaSpa
// abstract ("Training-free and Adaptive Sparse Attention for Efficient Long Video Generation",
// arXiv 2502.21079): the attention map is sparse in blocks; the log-sum-exp (LSE) of each query
// row changes little across denoising steps, so an LSE cached from an earlier full-attention
// step turns one pass of Q K^T into the exact attention mass of every block; each head then
// keeps, per query block, the fewest key blocks that carry a given share of that mass.
//
//   block_mass_kernel    M[i][j] = sum over rows q of query block i (256 rows) and keys k of key
//                        block j (64 keys) of exp(scale q.k - LSE_q): bf16 products on the
//                        matrix cores, fp32 exponentials and sums; a wavefront skips the
//                        exponentials of a tile in which all its weights are below 2^-40.
//   block_select_kernel  per (head, query block): key blocks in decreasing mass, the shortest
//                        prefix reaching `coverage` of the row's total mass (fp64 prefix sums).
//   block_lists_kernel   the chosen blocks of each query block in increasing order, and how
//                        many keys they hold, for the attention kernel's gathered key tiles.
#include "svg_internal.h"

namespace svg {

namespace {

constexpr int BM_NT = 512;                 // 8 wavefronts x 32 query rows = one query block

// v + the value of lane (l ^ m) within groups of four lanes, or mirrored within a row of 8 or
// 16 lanes, through DPP (no LDS round trip)
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
// sum over the 64 lanes, every lane gets it: DPP inside each row of 16 lanes, then the lane
// swaps between rows (16) and halves (32)
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xB1>(v);      // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);      // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);     // row_half_mirror
  v = dpp_add<0x140>(v);     // row_mirror
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);   // own row's sum in one entry, the partner row's in the other
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
constexpr int BM_KT = BLOCK_K_ROWS;        // keys per tile = one key block
constexpr int BM_TPI = 2;                  // key tiles per workgroup barrier

// 8 wavefronts of 32 rows each hold the query block as MFMA B operands; key tiles of 64 rows are
// the A operand from LDS, chunks XOR-swizzled by row.  The tiles are copied HBM -> LDS by
// buffer loads that write LDS directly (no register staging), two tiles per workgroup barrier,
// the next two in flight while the current ones are used (3% faster at 720p than staging
// through registers).  The accumulator S^T[key][query] gives lane l query l%32 and 16 keys
// per 32-key half; each lane sums its 32 weights, the wavefront reduces over its lanes (DPP
// inside rows of 16 lanes, then lane swaps across rows and halves: no LDS round trips, 2.3%
// faster than a shuffle tree at 720p), and one thread adds the eight wavefronts' sums in a
// fixed order, one iteration behind.  At most 128 VGPRs, so that two workgroups (four
// wavefronts per SIMD) share a CU: one's exponentials run under the other's matrix products
// (16% faster at D = 128 than one workgroup per CU at 130 VGPRs).
template <int D>
__global__ __launch_bounds__(BM_NT, 4) void block_mass_kernel(BlockMassArgs a) {
  constexpr int NKS = D / 16;
  constexpr int CPR = D / 8;
  constexpr int RPB = 16 / CPR;
  __shared__ __attribute__((aligned(1024))) bf16 kt[2][BM_TPI][BM_KT * D];
  __shared__ float part[2][BM_TPI][BM_NT / 64];

  const int32_t bh = blockIdx.x / a.nqb;
  const int32_t qb = blockIdx.x - bh * a.nqb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int32_t S = a.S;
  const int32_t row = qb * BLOCK_Q_ROWS + wave * 32 + l32;
  const bf16* qh = a.q + (size_t)bh * S * D;
  const bf16* kh = a.k + (size_t)bh * S * D;
  bf16x8 qf[NKS];
  const bf16* qr = qh + (size_t)min(row, S - 1) * D;
#pragma unroll
  for (int s = 0; s < NKS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qr + 16 * s + 8 * hh);
  const float c = a.scale * 1.44269504088896340736f;
  // rows past the sequence end weigh nothing
  const float l2 = row < S ? a.lse[(size_t)bh * S + row] * 1.44269504088896340736f : INFINITY;
  float* out = a.mass + (size_t)blockIdx.x * a.nkb;

  // one key tile's masses for this wavefront's 32 rows (the tile in LDS at ktile)
  auto tile_mass = [&](const bf16* ktile, int32_t t) -> float {
    f32x16 acc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[blk][r] = 0.f;
    // the products at the higher issue priority, so that the other workgroup's exponentials
    // fill the gaps between them (1% faster at 720p)
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int r = blk * 32 + l32;
        const bf16x8 ka =
            *reinterpret_cast<const bf16x8*>(&ktile[r * D + 8 * ((2 * s + hh) ^ ((r / RPB) & (CPR - 1)))]);
        acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], acc[blk], 0, 0, 0);
      }
    __builtin_amdgcn_s_setprio(0);
    float sum0 = 0.f, sum1 = 0.f;
    const int32_t kend = S - t * BM_KT;      // keys of this tile that exist
    // a tile whose largest weight for every query of the wavefront is below 2^-40 is skipped:
    // that moves a block's mass by less than 2^-26 (16384 weights), far below its fp32 rounding
    // at the row totals the choice compares against
    float mx = acc[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, acc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[1][r]);
    const bool live = __any(fmaf(mx, c, -l2) > -40.f);   // the same for every lane of the wavefront
    float s = 0.f;
    if (live) {
      if (kend >= BM_KT) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sum0 += __builtin_amdgcn_exp2f(fmaf(acc[0][r], c, -l2));
          sum1 += __builtin_amdgcn_exp2f(fmaf(acc[1][r], c, -l2));
        }
      } else {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = blk * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
            const float p = __builtin_amdgcn_exp2f(fmaf(acc[blk][r], c, -l2));
            if (key < kend) {
              if (blk == 0) sum0 += p; else sum1 += p;
            }
          }
      }
      // a skipped tile's wavefront sum is exactly 0 and needs no reduction
      s = wave_sum(sum0 + sum1);
    }
    return s;
  };
  // Rows past the sequence end lie outside the buffer, read as zero and are masked by kend.
  constexpr int ROW_BYTES = D * 2;
  constexpr int RPI = 1024 / ROW_BYTES;                       // tile rows per 1 KB instruction
  constexpr int IPW = BM_KT * ROW_BYTES / 1024 / (BM_NT / 64);  // instructions per wavefront and tile
  static_assert(IPW >= 1, "tile too small for the workgroup");
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)kh, (short)0, (int)(uint32_t)((uint32_t)S * ROW_BYTES), 0x00020000);
  auto dma = [&](int32_t t, bf16* dst) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int blkno = wave * IPW + i;
      const int r = blkno * RPI + lane / CPR;
      const int ch = (lane % CPR) ^ ((r / RPB) & (CPR - 1));
      const uint32_t voff = (uint32_t)(t * BM_KT + r) * ROW_BYTES + 16u * (uint32_t)ch;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)((char*)dst + blkno * 1024),
                                               16, voff, 0, 0, 0);
    }
  };
  const int32_t nt = a.nkb;
  const int32_t ni = (nt + BM_TPI - 1) / BM_TPI;
  auto issue = [&](int32_t it, int stage) {
#pragma unroll
    for (int u = 0; u < BM_TPI; ++u)
      if (it * BM_TPI + u < nt) dma(it * BM_TPI + u, kt[stage][u]);
  };
  auto flush = [&](int32_t it, int stage) {     // thread 0: the block masses of iteration it
#pragma unroll
    for (int u = 0; u < BM_TPI; ++u) {
      const int32_t t = it * BM_TPI + u;
      if (t < nt) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < BM_NT / 64; ++w) s += part[stage][u][w];
        out[t] = s;
      }
    }
  };
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(VMCNT0);
  __syncthreads();
  for (int32_t it = 0; it < ni; ++it) {
    const int stage = it & 1;
    if (it + 1 < ni) issue(it + 1, stage ^ 1);
    if (tid == 0 && it > 0) flush(it - 1, stage ^ 1);
#pragma unroll
    for (int u = 0; u < BM_TPI; ++u) {
      const int32_t t = it * BM_TPI + u;
      if (t < nt) {
        const float s = tile_mass(kt[stage][u], t);
        if (lane == 0) part[stage][u][wave] = s;
      }
    }
    __builtin_amdgcn_s_waitcnt(VMCNT0);
    __syncthreads();
  }
  if (tid == 0) flush(ni - 1, (ni - 1) & 1);
}

// Per (head, query block): bitonic sort of (mass, block) in LDS, decreasing mass and increasing
// block among equal masses; fp64 prefix sums of the sorted masses; the shortest prefix that
// reaches coverage * total (blocks of zero mass are never chosen).
constexpr int SEL_NT = 512;
__global__ __launch_bounds__(SEL_NT) void block_select_kernel(BlockSelectArgs a) {
  __shared__ float w[BLOCK_MAX_NKB];
  __shared__ int32_t ix[BLOCK_MAX_NKB];
  __shared__ double part[SEL_NT];
  __shared__ int32_t cut;
  const int tid = threadIdx.x;
  const int32_t nkb = a.nkb;
  const float* m = a.mass + (size_t)blockIdx.x * nkb;
  int n2 = 1;
  while (n2 < nkb) n2 <<= 1;
  for (int j = tid; j < n2; j += SEL_NT) {
    w[j] = j < nkb ? m[j] : -1.f;
    ix[j] = j;
  }
  if (tid == 0) cut = BLOCK_MAX_NKB;          // none yet
  __syncthreads();
  for (int k = 2; k <= n2; k <<= 1)
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int x = tid; x < n2; x += SEL_NT) {
        const int y = x ^ jj;
        if (y > x) {
          const bool up = (x & k) == 0;
          const float wx = w[x], wy = w[y];
          const int32_t ixx = ix[x], ixy = ix[y];
          const bool x_first = wx > wy || (wx == wy && ixx < ixy);
          if (x_first != up) {
            w[x] = wy; w[y] = wx;
            ix[x] = ixy; ix[y] = ixx;
          }
        }
      }
      __syncthreads();
    }
  // thread tid owns sorted positions [tid * per, (tid + 1) * per)
  const int per = (nkb + SEL_NT - 1) / SEL_NT;
  const int lo = min(tid * per, nkb), hi = min(lo + per, nkb);
  double own = 0.0;
  for (int r = lo; r < hi; ++r) own += w[r] > 0.f ? (double)w[r] : 0.0;
  part[tid] = own;
  __syncthreads();
  for (int o = 1; o < SEL_NT; o <<= 1) {
    const double v = tid >= o ? part[tid - o] : 0.0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  const double total = part[SEL_NT - 1];
  const double target = a.coverage * total;
  double run = part[tid] - own;
  for (int r = lo; r < hi; ++r) {
    if (!(w[r] > 0.f)) break;
    run += (double)w[r];
    if (run >= target) {
      atomicMin(&cut, r);
      break;
    }
  }
  __syncthreads();
  // no prefix reaches the target (rounding with coverage 1): every block of positive mass
  int32_t last = cut;
  if (last >= nkb) {
    last = -1;
    for (int r = 0; r < nkb; ++r)
      if (w[r] > 0.f) last = r;
  }
  uint8_t* srow = a.sel + (size_t)blockIdx.x * nkb;
  for (int j = tid; j < nkb; j += SEL_NT) srow[j] = 0;
  __syncthreads();
  for (int r = tid; r <= last; r += SEL_NT) srow[ix[r]] = 1;
}

// Per (head, query block): the chosen key blocks in increasing order, and the keys they hold
// (the sequence's last block may be partial; being the highest, it is last in the list).
constexpr int BL_NT = 256;
__global__ __launch_bounds__(BL_NT) void block_lists_kernel(BlockAttnArgs a) {
  __shared__ int32_t part[BL_NT];
  const int tid = threadIdx.x;
  const int32_t nkb = a.nkb;
  const uint8_t* srow = a.sel + (size_t)blockIdx.x * nkb;
  int32_t* out = a.blist + (size_t)blockIdx.x * nkb;
  const int per = (nkb + BL_NT - 1) / BL_NT;
  const int lo = min(tid * per, nkb), hi = min(lo + per, nkb);
  int32_t own = 0;
  for (int j = lo; j < hi; ++j) own += srow[j] ? 1 : 0;
  part[tid] = own;
  __syncthreads();
  for (int o = 1; o < BL_NT; o <<= 1) {
    const int32_t v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t pos = part[tid] - own;
  for (int j = lo; j < hi; ++j)
    if (srow[j]) out[pos++] = j;
  if (tid == 0) {
    const int32_t n = part[BL_NT - 1];
    int32_t keys = n * BLOCK_K_ROWS;
    if (n > 0 && srow[nkb - 1]) keys -= nkb * BLOCK_K_ROWS - a.S;
    a.blen[blockIdx.x] = keys;
  }
}

// Explicit instantiations, so that the host pass emits every launch stub the launchers use.
template __global__ void block_mass_kernel<128>(BlockMassArgs);
template __global__ void block_mass_kernel<64>(BlockMassArgs);

}  // namespace

hipError_t launch_block_mass(const BlockMassArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)a.BH * a.nqb));
  if (a.D == 128)
    block_mass_kernel<128><<<grid, BM_NT, 0, st>>>(a);
  else if (a.D == 64)
    block_mass_kernel<64><<<grid, BM_NT, 0, st>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_block_select(const BlockSelectArgs& a, hipStream_t st) {
  block_select_kernel<<<(unsigned)((int64_t)a.BH * a.nqb), SEL_NT, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_block_lists(const BlockAttnArgs& a, hipStream_t st) {
  block_lists_kernel<<<(unsigned)((int64_t)a.BH * a.nqb), BL_NT, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace svg
