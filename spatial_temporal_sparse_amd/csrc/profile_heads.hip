// Online profiling of each head's sparsity pattern, after 机器之心's article on Sparse
// VideoGen (dynamic adaptive sparsity strategy, steps 1-3) and the authors' article
// (section "Online Profiling Strategy"): for a small random sample of query rows, the
// attention output is computed under the spatial mask, under the temporal mask and with no
// mask; each head keeps the mask whose output has the smaller mean squared error against
// the unmasked output.
//
// Pass 1 (split-K): a workgroup takes one (head, key range, group of 64 sampled queries).
// Its eight wavefronts cover the two 32-query halves x the two 32-key halves of each 64-key
// tile x the two halves of the head dim (for the outputs; the scores are shared work).  Per
// tile, S^T = K Q^T on MFMA (as in the attention kernel), then three online softmax states
// -- dense, spatial, temporal -- each with its own row sum and O^T accumulator; the three PV
// products share the V^T operands read once from LDS.  The three states share one running
// reference max, the unmasked one: softmax does not depend on the reference, so each masked
// state only selects the unmasked exponentials of its keys.  This is exact up to rounding
// while a row's masked scores stay within 126 (log2 units) of its unmasked maximum; beyond
// that the masked exponentials underflow.
// Keys are frame-major here: the spatial mask is a per-query interval of frames, the
// temporal mask compares in-frame positions (key mod P).  Each wavefront writes its
// unnormalised partial state (reference max, row sum, O) to the workspace.
// Pass 2: one workgroup per (head, sampled row) merges that row's partial states with
// log-sum-exp weights, forms its three outputs (one channel per thread) and sums the two
// squared errors over the channels in fp64.
// Pass 3: one workgroup per head sums the per-row errors in a fixed order, stores mse (fp32)
// and the kind, deciding on the stored fp32 values (ties -> spatial).
// HBM-bound: K and V of every head are read once.
#include "svg_internal.h"

namespace svg {

namespace {

constexpr int NT = 512;            // partial pass
constexpr int NT_RED = 256;        // reduce pass
constexpr int TILE = 64;
constexpr int QG = 64;           // sampled queries per workgroup
constexpr int MAX_SPLIT = 128;
constexpr int TARGET_WGS = 512;
constexpr float RESCALE_SLACK = 8.0f;

template <int D>
struct PLds {
  static constexpr int KS = D + 8;
  static constexpr int VS = D + 32;
};

// Row sum and unnormalised O^T of one softmax state (its reference max is shared).
template <int NDB>
struct SoftmaxState {
  float l;
  f32x16 o[NDB];
};

// PBIG: a frame holds at least 32 tokens, so a lane's keys (a span of 28) cross at most one
// frame boundary and their in-frame positions follow from one division per tile.
template <int D, bool PBIG>
__global__ __launch_bounds__(NT, 1) void profile_partial_kernel(ProfileArgs a) {
  constexpr int KS = PLds<D>::KS;
  constexpr int VS = PLds<D>::VS;
  constexpr int NDBW = D / 64;     // 32-wide d blocks of the output per wavefront
  constexpr int NKS = D / 16;
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][TILE * KS];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][TILE * VS];
  __shared__ __attribute__((aligned(16))) bf16 Qs[QG * KS];   // the 64 sampled rows

  int32_t bid = blockIdx.x;
  const int32_t zq = bid % a.n_zq;
  bid /= a.n_zq;
  const int32_t split = bid % a.nsplit;
  const int32_t bh = bid / a.nsplit;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int qsub = wave & 1, kp = (wave >> 1) & 1, dhalf = wave >> 2;

  const size_t off = (size_t)bh * (size_t)a.S * D;
  const bf16* __restrict__ Q = a.q + off;
  const bf16* __restrict__ K = a.k + off;
  const bf16* __restrict__ V = a.v + off;

  const int32_t qi = zq * QG + qsub * 32 + l32;
  int32_t tq = a.idx[min(qi, a.n_q - 1)];
  tq = min(max(tq, 0), a.S - 1);
  const int32_t fq = (int32_t)fdiv((uint32_t)tq, a.divP);
  const int32_t pq = tq - fq * a.P;
  const int32_t sp_lo = max(0, fq - a.w_f) * a.P;
  const int32_t sp_hi = min(a.F, fq + a.w_f + 1) * a.P;

  // stage the sampled query rows once: wavefronts with kp == 0 and dhalf == 0 copy their rows
  if (kp == 0 && dhalf == 0) {
#pragma unroll
    for (int s = 0; s < NKS; ++s)
      *reinterpret_cast<bf16x8*>(&Qs[(qsub * 32 + l32) * KS + 16 * s + 8 * hh]) =
          *reinterpret_cast<const bf16x8*>(Q + (size_t)tq * D + 16 * s + 8 * hh);
  }

  const int32_t ks = split * a.keys_per_split;
  const int32_t ke = min(a.S, ks + a.keys_per_split);
  const int32_t ntiles = (ke - ks + TILE - 1) / TILE;

  TileStager<D, TILE, NT> stage;
  SoftmaxState<NDBW> st[3];
  float m_ref = -INFINITY;     // reference max (log2 units) shared by the three states
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    st[x].l = 0.f;
#pragma unroll
    for (int j = 0; j < NDBW; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) st[x].o[j][r] = 0.f;
  }
  const float c = a.scale * 1.44269504088896340736f;
  const int tg = lane >> 4, ti = lane & 15;
  const int v_row = 4 * (tg >> 1) + (ti >> 2);
  const int v_col = 16 * (tg & 1) + 4 * (ti & 3) + dhalf * (D / 2);

  if (ntiles > 0) {
    stage.load(K, V, ks, a.S, tid);
    stage.template store<KS, VS>(Ks[0], Vs[0], tid);
  }
  __syncthreads();
  for (int32_t t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const bool has_next = t + 1 < ntiles;
    if (has_next) stage.load(K, V, ks + (t + 1) * TILE, a.S, tid);

    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const bf16x8 ak = *reinterpret_cast<const bf16x8*>(&Ks[buf][(kp * 32 + l32) * KS + 16 * s + 8 * hh]);
      const bf16x8 bq = *reinterpret_cast<const bf16x8*>(&Qs[(qsub * 32 + l32) * KS + 16 * s + 8 * hh]);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, bq, sacc, 0, 0, 0);
    }

    const int32_t kbase = ks + t * TILE + kp * 32 + 4 * hh;
    // keys past the split's end (last tile only) do not exist
    if (ks + (t + 1) * TILE > ke) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kbase + 8 * (r >> 2) + (r & 3) >= ke) sacc[r] = -INFINITY;
    }
    // shared reference max with lazy rescaling of all three states
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;
    const bool bump = mx > m_ref + RESCALE_SLACK;
    if (__any(bump)) {
      const float m_new = bump ? mx : m_ref;
      const float alpha = (m_ref == -INFINITY) ? 0.f : exp2f(m_ref - m_new);
#pragma unroll
      for (int x = 0; x < 3; ++x) {
        st[x].l *= alpha;
#pragma unroll
        for (int j = 0; j < NDBW; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) st[x].o[j][r] *= alpha;
      }
      m_ref = m_new;
    }
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    // masks as unsigned range tests: spatial key - sp_lo < sp_hi - sp_lo (frame-major keys),
    // temporal |p_key - p_query| <= w_p on in-frame positions
    const uint32_t sp_base = (uint32_t)(kbase - sp_lo), sp_span = (uint32_t)(sp_hi - sp_lo);
    const int32_t pbase = PBIG ? (int32_t)fmod_((uint32_t)kbase, a.divP) : 0;
    const uint32_t tp_span = (uint32_t)(2 * a.w_p);
    float pd[16], psp[16], ptp[16];
    float ld = 0.f, lsp = 0.f, ltp = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int32_t dk = 8 * (r >> 2) + (r & 3);
      int32_t pk;
      if constexpr (PBIG) {
        pk = pbase + dk;
        pk -= (pk >= a.P) ? a.P : 0;
      } else {
        pk = (int32_t)fmod_((uint32_t)(kbase + dk), a.divP);
      }
      const bool in_sp = sp_base + (uint32_t)dk < sp_span;
      const bool in_tp = (uint32_t)(pk - pq + a.w_p) <= tp_span;
      const float pr = __builtin_amdgcn_exp2f(fmaf(sacc[r], c, -m_use));
      pd[r] = pr;
      psp[r] = in_sp ? pr : 0.f;
      ptp[r] = in_tp ? pr : 0.f;
      ld += pd[r];
      lsp += psp[r];
      ltp += ptp[r];
    }
    st[0].l += ld;
    st[1].l += lsp;
    st[2].l += ltp;

#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 b0, b1, b2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        b0[e] = (bf16)pd[8 * s + e];
        b1[e] = (bf16)psp[8 * s + e];
        b2[e] = (bf16)ptp[8 * s + e];
      }
      const bf16* vb = &Vs[buf][(kp * 32 + 16 * s + v_row) * VS + v_col];
#pragma unroll
      for (int j = 0; j < NDBW; ++j) {
        const bf16x8 av = load_vt(vb + j * 32, VS);
        st[0].o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b0, st[0].o[j], 0, 0, 0);
        st[1].o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b1, st[1].o[j], 0, 0, 0);
        st[2].o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b2, st[2].o[j], 0, 0, 0);
      }
    }
    if (has_next) stage.template store<KS, VS>(Ks[buf ^ 1], Vs[buf ^ 1], tid);
    __syncthreads();
  }

  // ---- write this wavefront's partial states (its half of the head dim) ----
  const int32_t nparts = 2 * a.nsplit;
  const int32_t part = split * 2 + kp;
  const int32_t qpad = a.n_zq * QG;
  const int32_t qloc = zq * QG + qsub * 32 + l32;
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    const float l_tot = st[x].l + __shfl_xor(st[x].l, 32, 64);
    const size_t slot = (((size_t)bh * nparts + part) * 3 + x) * qpad + qloc;
    if (hh == 0 && dhalf == 0) {
      a.part_ml[slot * 2 + 0] = m_ref;
      a.part_ml[slot * 2 + 1] = l_tot;
    }
    float* po = a.part_o + slot * D + dhalf * (D / 2);
#pragma unroll
    for (int j = 0; j < NDBW; ++j)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = st[x].o[j][4 * rq + e];
        *reinterpret_cast<f32x4*>(po + 32 * j + 8 * rq + 4 * hh) = v4;
      }
  }
}

template <int D>
__global__ __launch_bounds__(D) void profile_merge_kernel(ProfileArgs a) {
  __shared__ float sm[3][2 * MAX_SPLIT], sl[3][2 * MAX_SPLIT], wt[3][2 * MAX_SPLIT];
  __shared__ double red[2][D];
  const int32_t bh = blockIdx.x / a.n_q;
  const int32_t qg = blockIdx.x - bh * a.n_q;
  const int tid = threadIdx.x;
  const int32_t nparts = 2 * a.nsplit;
  const int32_t qpad = a.n_zq * QG;
  for (int t = tid; t < 3 * nparts; t += D) {
    const int x = t / nparts, p = t - (t / nparts) * nparts;
    const size_t slot = (((size_t)bh * nparts + p) * 3 + x) * qpad + qg;
    sm[x][p] = a.part_ml[slot * 2];
    sl[x][p] = a.part_ml[slot * 2 + 1];
  }
  __syncthreads();
  if (tid < 3) {
    float M = -INFINITY;
    for (int32_t p = 0; p < nparts; ++p) M = fmaxf(M, sm[tid][p]);
    float L = 0.f;
    for (int32_t p = 0; p < nparts; ++p) {
      const float w = (sm[tid][p] == -INFINITY) ? 0.f : exp2f(sm[tid][p] - M);
      wt[tid][p] = w;
      L += w * sl[tid][p];
    }
    const float inv = (L > 0.f) ? 1.f / L : 0.f;
    for (int32_t p = 0; p < nparts; ++p) wt[tid][p] *= inv;
  }
  __syncthreads();
  float o3[3];
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    float s = 0.f;
    for (int32_t p = 0; p < nparts; ++p) {
      const size_t slot = (((size_t)bh * nparts + p) * 3 + x) * qpad + qg;
      s = fmaf(wt[x][p], a.part_o[slot * D + tid], s);
    }
    o3[x] = s;
  }
  const double dsp = (double)o3[1] - (double)o3[0];
  const double dtp = (double)o3[2] - (double)o3[0];
  red[0][tid] = dsp * dsp;
  red[1][tid] = dtp * dtp;
  __syncthreads();
  for (int s = D / 2; s > 0; s >>= 1) {
    if (tid < s) {
      red[0][tid] += red[0][tid + s];
      red[1][tid] += red[1][tid + s];
    }
    __syncthreads();
  }
  if (tid == 0) {
    a.row_sq[2 * ((size_t)bh * a.n_q + qg) + 0] = red[0][0];
    a.row_sq[2 * ((size_t)bh * a.n_q + qg) + 1] = red[1][0];
  }
}

__global__ __launch_bounds__(NT_RED) void profile_finish_kernel(ProfileArgs a) {
  __shared__ double red[2][NT_RED];
  const int32_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  double acc_sp = 0.0, acc_tp = 0.0;
  for (int32_t q = tid; q < a.n_q; q += NT_RED) {
    acc_sp += a.row_sq[2 * ((size_t)bh * a.n_q + q) + 0];
    acc_tp += a.row_sq[2 * ((size_t)bh * a.n_q + q) + 1];
  }
  red[0][tid] = acc_sp;
  red[1][tid] = acc_tp;
  __syncthreads();
  for (int s = NT_RED / 2; s > 0; s >>= 1) {
    if (tid < s) {
      red[0][tid] += red[0][tid + s];
      red[1][tid] += red[1][tid + s];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double n = (double)a.n_q * a.D;
    const float msp = (float)(red[0][0] / n);
    const float mtp = (float)(red[1][0] / n);
    a.mse[2 * bh + 0] = msp;
    a.mse[2 * bh + 1] = mtp;
    a.kind[bh] = (uint8_t)(msp <= mtp ? KIND_SPATIAL : KIND_TEMPORAL);
  }
}

}  // namespace

ProfilePlan profile_plan(int32_t BH, int32_t S, int32_t D, int32_t n_q) {
  ProfilePlan p;
  p.n_zq = (n_q + QG - 1) / QG;
  // as many key splits as fit TARGET_WGS workgroups (two per CU) without a partial round
  int64_t want = TARGET_WGS / ((int64_t)BH * p.n_zq);
  const int64_t max_tiles = (S + TILE - 1) / TILE;
  if (want > MAX_SPLIT) want = MAX_SPLIT;
  if (want > max_tiles) want = max_tiles;
  if (want < 1) want = 1;
  const int64_t per = (S + want - 1) / want;
  p.keys_per_split = (int32_t)(((per + TILE - 1) / TILE) * TILE);
  p.nsplit = (int32_t)((S + p.keys_per_split - 1) / p.keys_per_split);
  const size_t slots = (size_t)BH * (2 * p.nsplit) * 3 * (size_t)(p.n_zq * QG);
  p.ml_floats = slots * 2;
  p.o_floats = slots * (size_t)D;
  p.sq_doubles = (size_t)BH * n_q * 2;
  return p;
}

hipError_t launch_profile(const ProfileArgs& a, hipStream_t st) {
  const dim3 g1((unsigned)((int64_t)a.BH * a.nsplit * a.n_zq));
  const dim3 g2((unsigned)((int64_t)a.BH * a.n_q));
  const dim3 g3((unsigned)a.BH);
  const bool pbig = a.P >= 32;
  if (a.D == 128) {
    if (pbig) profile_partial_kernel<128, true><<<g1, NT, 0, st>>>(a);
    else profile_partial_kernel<128, false><<<g1, NT, 0, st>>>(a);
    profile_merge_kernel<128><<<g2, 128, 0, st>>>(a);
  } else if (a.D == 64) {
    if (pbig) profile_partial_kernel<64, true><<<g1, NT, 0, st>>>(a);
    else profile_partial_kernel<64, false><<<g1, NT, 0, st>>>(a);
    profile_merge_kernel<64><<<g2, 64, 0, st>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  profile_finish_kernel<<<g3, NT_RED, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace svg
