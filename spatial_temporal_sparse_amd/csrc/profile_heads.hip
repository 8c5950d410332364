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

// Unnormalised O^T of one softmax state (reference max and row sums are kept beside it).
template <int NDB>
struct SoftmaxState {
  f32x16 o[NDB];
};

// Scores -> P of one tile for one wavefront: the half DH of its 32 keys (16 keys, score
// registers 8*DH .. 8*DH+7) in all three states, row sums of that half, bf16 P^T operands.
// The reference max m_use is shared (see the header).
template <int DH, bool PBIG>
__device__ __forceinline__ void half_softmax(const f32x16& sacc, float c, float m_use, int32_t kbase, uint32_t sp_base,
                                             uint32_t sp_span, int32_t pbase, int32_t pq, const ProfileArgs& a,
                                             float (&l)[3], bf16x8 (&pb)[3]) {
  const uint32_t tp_span = (uint32_t)(2 * a.w_p);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int r = 8 * DH + e;
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
    const float ps = in_sp ? pr : 0.f;
    const float pt = in_tp ? pr : 0.f;
    l[0] += pr;
    l[1] += ps;
    l[2] += pt;
    pb[0][e] = (bf16)pr;
    pb[1][e] = (bf16)ps;
    pb[2][e] = (bf16)pt;
  }
}

// PBIG: a frame holds at least 32 tokens, so a lane's keys (a span of 28) cross at most one
// frame boundary and their in-frame positions follow from one division per tile.
//
// The two wavefronts of a (query half, key half) pair -- dhalf 0 and 1, which own the two
// halves of the head dim of the outputs -- compute the same scores but split the softmax: each
// turns its 16 of the 32 keys into P (three states) and hands its bf16 P^T to the other
// through LDS.  The exchange crosses the workgroup barrier at the end of the tile, so the PV
// products of tile t run in step t+1; V is triple-buffered for that.  Both compute the
// (cheap) row max of all 32 keys, so they agree on every rescale.
template <int D, bool PBIG>
__global__ __launch_bounds__(NT, 1) void profile_partial_kernel(ProfileArgs a) {
  constexpr int KS = PLds<D>::KS;
  constexpr int VS = PLds<D>::VS;
  constexpr int NDBW = D / 64;     // 32-wide d blocks of the output per wavefront
  constexpr int NKS = D / 16;
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][TILE * KS];
  __shared__ __attribute__((aligned(16))) bf16 Vs[3][TILE * VS];
  __shared__ __attribute__((aligned(16))) bf16 Qs[QG * KS];   // the 64 sampled rows
  __shared__ __attribute__((aligned(16))) bf16x8 Px[2][NT / 64][3][64];   // P^T exchange

  int32_t bid = blockIdx.x;
  const int32_t zq = bid % a.n_zq;
  bid /= a.n_zq;
  const int32_t split = bid % a.nsplit;
  const int32_t bh = bid / a.nsplit;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int qsub = wave & 1, kp = (wave >> 1) & 1, dhalf = wave >> 2;
  const int partner = wave ^ 4;

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

  // two register stages: tile t+2 is fetched while tile t is computed and tile t+1 waits in
  // registers for its LDS buffer, so two tiles per workgroup are in flight from HBM
  TileStager<D, TILE, NT> stage_a, stage_b;
  SoftmaxState<NDBW> st[3];
  float m_ref = -INFINITY;     // reference max (log2 units) shared by the three states
  float l[3] = {0.f, 0.f, 0.f};   // this wavefront's half of the row sums
#pragma unroll
  for (int x = 0; x < 3; ++x)
#pragma unroll
    for (int j = 0; j < NDBW; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) st[x].o[j][r] = 0.f;
  bf16x8 pown[3];              // this wavefront's P^T of the previous tile
  const float c = a.scale * 1.44269504088896340736f;
  const int tg = lane >> 4, ti = lane & 15;
  const int v_row = 4 * (tg >> 1) + (ti >> 2);
  const int v_col = 16 * (tg & 1) + 4 * (ti & 3) + dhalf * (D / 2);

  if (ntiles > 0) {
    stage_a.load(K, V, ks, a.S, tid);
    stage_a.template store<KS, VS>(Ks[0], Vs[0], tid);
  }
  // Fetches are unconditional (past the last tile they repeat it, and nothing stores that copy):
  // a conditional fetch would make the compiler wait for every load in flight before storing
  // the older stage.
  const int32_t t_last = max(ntiles - 1, 0);
  stage_b.load(K, V, ks + min(1, t_last) * TILE, a.S, tid);
  __syncthreads();
  // step t: fetch tile t+2 into `fetch`, compute, then move tile t+1 from `ready` into LDS
  auto step = [&](int32_t t, TileStager<D, TILE, NT>& fetch, TileStager<D, TILE, NT>& ready) {
    fetch.load(K, V, ks + min(t + 2, t_last) * TILE, a.S, tid);

    // ---- PV of tile t-1: own P^T for key step dhalf, the partner's for the other ----
    if (t >= 1) {
      bf16x8 pq3[3];
#pragma unroll
      for (int x = 0; x < 3; ++x) pq3[x] = Px[(t - 1) & 1][partner][x][lane];
      const bf16* vt = Vs[(t - 1) % 3];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16* vb = &vt[(kp * 32 + 16 * s + v_row) * VS + v_col];
        const bool mine = s == dhalf;
#pragma unroll
        for (int j = 0; j < NDBW; ++j) {
          const bf16x8 av = load_vt(vb + j * 32, VS);
#pragma unroll
          for (int x = 0; x < 3; ++x)
            st[x].o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, mine ? pown[x] : pq3[x], st[x].o[j], 0, 0, 0);
        }
      }
    }

    if (t < ntiles) {
      const int buf = t & 1;
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
      // shared reference max (over all 32 keys, in both wavefronts of the pair) with lazy
      // rescaling of all three states; the accumulators hold the products up to tile t-1
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
          l[x] *= alpha;
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
      if (dhalf == 0)
        half_softmax<0, PBIG>(sacc, c, m_use, kbase, sp_base, sp_span, pbase, pq, a, l, pown);
      else
        half_softmax<1, PBIG>(sacc, c, m_use, kbase, sp_base, sp_span, pbase, pq, a, l, pown);
#pragma unroll
      for (int x = 0; x < 3; ++x) Px[t & 1][wave][x][lane] = pown[x];
    }
    if (t + 1 < ntiles) ready.template store<KS, VS>(Ks[(t + 1) & 1], Vs[(t + 1) % 3], tid);
    __syncthreads();
  };
  for (int32_t t = 0; t <= ntiles; t += 2) {
    step(t, stage_a, stage_b);
    if (t + 1 > ntiles) break;
    step(t + 1, stage_b, stage_a);
  }

  // ---- row sums of the pair, then this wavefront's partial states (its half of the head dim)
  float* lx = reinterpret_cast<float*>(&Px[0][0][0][0]);     // reused: [NT / 64][3][64]
#pragma unroll
  for (int x = 0; x < 3; ++x) lx[(wave * 3 + x) * 64 + lane] = l[x];
  __syncthreads();
#pragma unroll
  for (int x = 0; x < 3; ++x) l[x] += lx[(partner * 3 + x) * 64 + lane];
  const int32_t nparts = 2 * a.nsplit;
  const int32_t part = split * 2 + kp;
  const int32_t qpad = a.n_zq * QG;
  const int32_t qloc = zq * QG + qsub * 32 + l32;
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    const float l_tot = l[x] + __shfl_xor(l[x], 32, 64);
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
