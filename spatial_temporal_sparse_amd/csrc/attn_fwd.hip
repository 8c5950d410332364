// Block-sparse flash-style attention forward for gfx950 (MI355X).
//
// Each head attends under the token mask of its kind: spatial heads (frame-major) see their
// own frame and +-w_f frames, temporal heads (token-major, after the layout transformation)
// see their own location +-w_p in every frame, dense heads see everything (Sparse VideoGen
// authors' article, sections "Spatial Head", "Temporal Head" and "Layout Transformation";
// 机器之心 article, kernel section).  In the head's working layout every query row's allowed
// keys are one interval, so a 128-row query block needs exactly the key tiles between the
// first row's lower end and the last row's upper end; only boundary tiles need the
// per-element mask.
//
// Work decomposition: one workgroup (4 wavefronts of 64) per (head, 128-row query block);
// wavefront w owns query rows 32w..32w+31 of the block.  Key/value tiles of 64 rows are
// staged in LDS (double-buffered: the next tile's global loads are in flight while the
// current one is consumed) and shared by the four wavefronts.
//
// Per tile and wavefront, with v_mfma_f32_32x32x16_bf16 (lane l: row/col l%32, k-half l/32):
//   S^T[key][query] = K Q^T      A = K rows from LDS (one 16-byte read per MFMA),
//                                B = Q kept in registers for the whole loop.
//   The accumulator puts one query per lane (column l%32) and 16 keys per lane, so the row
//   max needs one cross-half exchange and the row sum none until the end.
//   O^T[d][query] += V^T P^T     A = V^T read from the row-major V tile with the LDS
//                                transpose read (ds_read_b64_tr_b16), B = P^T converted to
//                                bf16 straight from the S^T accumulator registers: the key
//                                order inside each 16-key step is permuted identically on
//                                both operands, which leaves the contraction unchanged.
//   The O^T accumulator again holds one query per lane, so the online-softmax rescale is a
//   per-lane scalar.  It is applied lazily: the running max only moves when a tile's max
//   exceeds it by more than 8 (log2 units), which bounds p by 2^8 and skips most rescales.
// exp2 with log2(e) folded into the softmax scale; fp32 accumulation; P rounded to bf16 for
// the PV product; output divided by the row sum and rounded to bf16 (round-to-nearest-even).
#include "svg_internal.h"

namespace svg {

namespace {

constexpr int BM = ATTN_BM;       // query rows per workgroup
constexpr int BN = ATTN_BN;       // keys per tile
constexpr int NT = 256;           // threads per workgroup
constexpr float RESCALE_SLACK = 8.0f;

template <int D>
struct Lds {
  static constexpr int KS = D + 8;    // K row stride (elements): 16-byte skew per row
  static constexpr int VS = D + 32;   // V row stride (elements): 64-byte skew per row
};

__global__ void head_order_kernel(const uint8_t* __restrict__ kind, int32_t* __restrict__ order, int32_t BH) {
  // Heavier heads first (spatial, dense), temporal heads last; stable within a class.
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int32_t n = 0;
  for (int32_t h = 0; h < BH; ++h)
    if (kind[h] != KIND_TEMPORAL) order[n++] = h;
  for (int32_t h = 0; h < BH; ++h)
    if (kind[h] == KIND_TEMPORAL) order[n++] = h;
}

template <int D>
__global__ __launch_bounds__(NT, 2) void attn_fwd_kernel(AttnArgs a, int32_t nqb) {
  constexpr int KS = Lds<D>::KS;
  constexpr int VS = Lds<D>::VS;
  constexpr int NDB = D / 32;                // 32-wide d blocks of the output
  constexpr int NKS = D / 16;                // k-steps of the QK^T product
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][BN * KS];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][BN * VS];

  const int32_t rank = blockIdx.x / nqb;
  const int32_t qb = blockIdx.x - rank * nqb;
  const int32_t bh = a.order ? a.order[rank] : rank;
  int kind = (a.force_dense || a.kind == nullptr) ? KIND_DENSE : (int)a.kind[bh];
  if (kind != KIND_SPATIAL && kind != KIND_TEMPORAL) kind = KIND_DENSE;
  const bool tmaj = kind == KIND_TEMPORAL;
  const size_t off = (size_t)bh * (size_t)a.S * D;
  const bf16* __restrict__ Q = (tmaj ? a.qt : a.q) + off;
  const bf16* __restrict__ K = (tmaj ? a.kt : a.k) + off;
  const bf16* __restrict__ V = (tmaj ? a.vt : a.v) + off;
  bf16* __restrict__ O = (tmaj ? a.ot : a.o) + off;

  Band band;
  band.S = a.S;
  band.dense = kind == KIND_DENSE;
  if (tmaj) { band.divG = a.divF; band.G = a.F; band.NG = a.P; band.w = a.w_p; }
  else { band.divG = a.divP; band.G = a.P; band.NG = a.F; band.w = a.w_f; }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int32_t q0 = qb * BM;
  const int32_t q_last = min(q0 + BM, a.S) - 1;
  int32_t lo_first, hi_first, lo_last, hi_last;
  band_interval(band, q0, lo_first, hi_first);
  band_interval(band, q_last, lo_last, hi_last);
  const int32_t t_begin = lo_first / BN;
  const int32_t t_end = (hi_last + BN - 1) / BN;

  const int32_t my_q = q0 + wave * 32 + l32;
  const int32_t my_qc = min(my_q, a.S - 1);
  int32_t my_lo, my_hi;
  band_interval(band, my_qc, my_lo, my_hi);

  bf16x8 qf[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s)
    qf[s] = *reinterpret_cast<const bf16x8*>(Q + (size_t)my_qc * D + 16 * s + 8 * hh);

  TileStager<D, BN, NT> stage;

  f32x16 oacc[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[j][r] = 0.f;
  float m_ref = -INFINITY;   // reference max (log2 units) the accumulators are scaled to
  float l_run = 0.f;         // this lane's share of the row sum, relative to m_ref
  const float c = a.scale * 1.44269504088896340736f;

  // transpose-read coordinates of this lane inside the V tile
  const int tg = lane >> 4;
  const int ti = lane & 15;
  const int v_row = 4 * (tg >> 1) + (ti >> 2);
  const int v_col = 16 * (tg & 1) + 4 * (ti & 3);

  stage.load(K, V, t_begin * BN, a.S, tid);
  stage.template store<KS, VS>(Ks[0], Vs[0], tid);
  __syncthreads();

  for (int32_t t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    const bool has_next = t + 1 < t_end;
    if (has_next) stage.load(K, V, (t + 1) * BN, a.S, tid);

    // ---- S^T = K Q^T for keys [k0, k0+64) (two 32-key blocks) ----
    f32x16 sacc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[blk][r] = 0.f;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(&Ks[buf][(blk * 32 + l32) * KS + 16 * s + 8 * hh]);
        sacc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[s], sacc[blk], 0, 0, 0);
      }
    }

    // ---- exact token mask on boundary tiles ----
    const int32_t k0 = t * BN;
    if (!(k0 >= lo_last && k0 + BN <= hi_first)) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int32_t key = k0 + blk * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key < my_lo || key >= my_hi) sacc[blk][r] = -INFINITY;
        }
    }

    // ---- online softmax (one query per lane; the other half-wave holds the other keys) ----
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[blk][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;
    const bool bump = mx > m_ref + RESCALE_SLACK;
    if (__any(bump)) {
      const float m_new = bump ? mx : m_ref;
      const float alpha = (m_ref == -INFINITY) ? 0.f : exp2f(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int j = 0; j < NDB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[j][r] *= alpha;
      m_ref = m_new;
    }
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    float rsum = 0.f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[blk][r], c, -m_use));
        sacc[blk][r] = p;
        rsum += p;
      }
    l_run += rsum;

    // ---- O^T += V^T P^T, four 16-key steps ----
#pragma unroll
    for (int s = 0; s < BN / 16; ++s) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (bf16)sacc[s >> 1][8 * (s & 1) + e];
      const bf16* vb = &Vs[buf][(16 * s + v_row) * VS + v_col];
#pragma unroll
      for (int j = 0; j < NDB; ++j) {
        const bf16x8 av = load_vt(vb + j * 32, VS);
        oacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, oacc[j], 0, 0, 0);
      }
    }

    if (has_next) stage.template store<KS, VS>(Ks[buf ^ 1], Vs[buf ^ 1], tid);
    __syncthreads();
  }

  // ---- epilogue: divide by the row sum, round to bf16, store this lane's query row ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l_tot;
  if (my_q < a.S) {
    bf16* orow = O + (size_t)my_q * D;
#pragma unroll
    for (int j = 0; j < NDB; ++j)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (bf16)(oacc[j][4 * rq + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * j + 8 * rq + 4 * hh) = ov;
      }
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  const int32_t nqb = (a.S + BM - 1) / BM;
  if (a.order != nullptr && a.kind != nullptr && !a.force_dense) {
    head_order_kernel<<<1, 64, 0, st>>>(a.kind, a.order, a.BH);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  AttnArgs b = a;
  if (a.kind == nullptr || a.force_dense) b.order = nullptr;
  const dim3 grid((unsigned)((int64_t)nqb * a.BH));
  if (a.D == 128) {
    attn_fwd_kernel<128><<<grid, NT, 0, st>>>(b, nqb);
  } else if (a.D == 64) {
    attn_fwd_kernel<64><<<grid, NT, 0, st>>>(b, nqb);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace svg
