// Online profiling of each head's sparsity pattern, after 机器之心's article on Sparse
// VideoGen (dynamic adaptive sparsity strategy, steps 1-3) and the authors' article
// (section "Online Profiling Strategy"): for a small random sample of query rows, the
// attention output is computed under the spatial mask, under the temporal mask and with no
// mask; each head keeps the mask whose output has the smaller mean squared error against
// the unmasked output.
//
// Pass 1 (split-K): a workgroup of four wavefronts takes one (head, key split, group of 64
// sampled queries), 16 queries per wavefront, and two workgroups share a CU, so that one's
// matrix products overlap the other's exponentials.  Split s of n holds the head's key tiles
// s, s + n, s + 2n, ...: the n workgroups of a head, which run at the same time, stream
// neighbouring tiles (3% faster at 720p than contiguous key ranges per split).  Per 64-key
// tile and wavefront, with v_mfma_f32_16x16x32_bf16 (lane l: row/column l%16, k-quarter l/16):
//   S^T[key][query] = K Q^T       A = K rows from LDS, B = the wavefront's Q rows, kept in
//                                 registers; lane l holds 16 scores of query l%16.
//   O_x^T[d][query] += V^T P_x^T  for the three softmax states x (dense, spatial, temporal):
//                                 A = V^T from the LDS transpose read, shared by the three
//                                 products; B = P_x^T converted to bf16 straight from the
//                                 score registers (the key order inside each 32-key step is
//                                 permuted identically on both operands).
// The three states share one running reference max, the unmasked one: softmax does not
// depend on the reference, so each masked state only selects the unmasked exponentials of
// its keys.  This is exact up to rounding while a row's masked scores stay within about 126
// (log2 units) of the split's unmasked maximum; beyond that the masked exponentials
// underflow.  A masked state whose row sum in a split falls below 2^-100 although the split
// holds keys of its mask is therefore marked (row sum -1) instead of stored, and pass 2
// recomputes that state of that row exactly, with its own maximum.
// Keys are frame-major here: the spatial mask is a per-query interval of frames, the
// temporal mask compares in-frame positions (key mod P).  Each wavefront writes the
// unnormalised partial state (reference max, row sum, O) of its queries to the workspace.
// Key and value tiles are copied HBM -> LDS (global_load_lds_dwordx4, no register staging)
// into two buffers, one tile ahead of their use.
// Pass 2: one workgroup per (head, sampled row) merges that row's partial states with
// log-sum-exp weights taken against each state's own largest log-mass (so that no split's
// weight underflows against another state's maximum), forms its three outputs (one channel
// per thread; a marked state by the exact fallback) and sums the two squared errors over the
// channels in fp64.
// Pass 3: one workgroup per head sums the per-row errors in a fixed order, stores mse (fp32)
// and the kind, deciding on the stored fp32 values (ties -> spatial).
// HBM-bound: K and V of every head are read once.
#include "svg_internal.h"

namespace svg {

namespace {

constexpr int NT = 256;            // partial pass: four wavefronts
constexpr int NT_RED = 256;        // reduce pass
constexpr int TILE = 64;           // keys per tile
constexpr int NBUF = 2;            // tile buffers (copies run NBUF-1 tiles ahead)
constexpr int NKB = TILE / 16;     // 16-key score blocks per tile
constexpr int NST = TILE / 32;     // 32-key PV steps per tile
constexpr int QG = 64;             // sampled queries per workgroup
constexpr int MAX_SPLIT = 128;
constexpr int MERGE_PF = 32;       // splits whose partial outputs the merge loads up front
constexpr int TARGET_WGS = 512;    // two workgroups per CU
constexpr float RESCALE_SLACK = 8.0f;
// A masked state's row sum in a split below this (relative to the split's unmasked reference)
// may have lost keys to underflow; such a state is recomputed exactly.
constexpr float UNDERFLOW_GUARD = 0x1p-100f;
// Cache policy of the tile copies: non-temporal (nt), since every K and V row is read once.
// Measured at 720p: the profiling call 0.327 -> 0.309 ms inside the layer and 0.350 -> 0.281 ms
// with the caches flushed; the Wan-like grid 0.192 -> 0.160 ms.
constexpr int CPOL_NT = 2;

// s_waitcnt immediate (gfx9 encoding): at most vm vector-memory loads and lgkm LDS operations
// outstanding, exports not waited for.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | ((vm >> 4) << 14); }

// Tile geometry in LDS: rows of D bf16 (no padding), 16-byte chunks XOR-swizzled per row.
template <int D>
struct PTile {
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int RPB = 16 / CPR;         // rows per 256-byte bank period
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = TILE * ROW_BYTES;
  static constexpr int CPW = 2 * TILE_BYTES / 1024 / (NT / 64);   // 1 KB copies per wavefront and tile (K + V)
  // K is read 16 rows x one chunk per 16 lanes: spread those rows over all 16 chunk slots.
  static __device__ __forceinline__ int swz_k(int r) { return (r / RPB) & (CPR - 1); }
  // V is read by the transpose read, 8 rows x two adjacent chunks per 32 lanes: give each of
  // the 8 rows its own pair of chunk slots.
  static __device__ __forceinline__ int swz_v(int r) { return 2 * ((r / RPB) & (CPR / 2 - 1)); }
};

// value of x held by lane l^16 / l^32 combined with x by max or by sum
__device__ __forceinline__ float max_x16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(fmaxf(x, __uint_as_float(r[0])), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(fmaxf(x, __uint_as_float(r[0])), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);   // own value in one entry, partner's in the other
}
__device__ __forceinline__ float sum_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Copy of one K or V tile (rows k0.., clamped to S-1) into LDS by the four wavefronts: each
// wavefront fills CPW/2 consecutive KB of the tile, every lane 16 bytes of one row.
template <int D>
__device__ __forceinline__ void tile_copy(const bf16* __restrict__ src, int32_t k0, int32_t S, bf16* dst, int wave,
                                          int lane, bool is_v) {
  using T = PTile<D>;
  constexpr int PER = T::CPW / 2;
  constexpr int RPI = 1024 / T::ROW_BYTES;     // tile rows per instruction
  const int pc = lane % T::CPR;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int blk = wave * PER + i;
    const int row = blk * RPI + lane / T::CPR;
    const int lc = pc ^ (is_v ? T::swz_v(row) : T::swz_k(row));
    const uint32_t boff = (uint32_t)min(k0 + row, S - 1) * (uint32_t)T::ROW_BYTES + 16u * (uint32_t)lc;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(src) + boff,
                                     (__attribute__((address_space(3))) void*)((char*)dst + blk * 1024), 16, 0, CPOL_NT);
  }
}

// Workgroup barrier without a memory fence (a fenced one would also wait for the copies
// still in flight for later tiles).  The empty asm statements keep LDS accesses on their side.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per-lane state: three O^T accumulators (D/16 blocks of 16 channels x 16 queries each),
// the shared reference max and the lane's shares of the three row sums.
template <int D>
struct PState {
  f32x4 o[3][D / 16];
  float m_ref;
  float l[3];
};

// sum of the eight bf16 values of p added to acc (v_dot2_f32_bf16 against (1, 1))
__device__ __forceinline__ float add_bf16x8(const bf16x8& p, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 6, 7), one, acc, false);
}

// Temporal-mask modes.  A lane's keys in a tile are kl + dk, dk = 16 kb + r (kb < 4, r < 4).
//   TP_INTERVAL: frames of >= 64 tokens (the lane's keys, a span of 52, cross at most one
//     frame boundary) and a band that leaves >= 52 positions of a frame out
//     (P - 2 w_p - 1 >= 52).  The keys of the band in the first frame, [lo0, hi0] in dk, and in
//     the next, [lo0 + P, hi0 + P], are then at least 52 apart, so at most one of them meets
//     the lane's keys: one interval [a, b) of dk per tile, clipped at the frame boundary.
//   TP_PER_KEY: in-frame position of every key by one division.
constexpr int TP_PER_KEY = 0;
constexpr int TP_INTERVAL = 1;

// One 64-key tile for one wavefront: scores, masks, softmax, PV products.
template <int D, int TPM>
__device__ __forceinline__ void profile_tile(PState<D>& st, const bf16x8 (&qf)[D / 32], const char* kt, const bf16* vt,
                                             int32_t k0, int32_t ke, float c, int32_t sp_lo, uint32_t sp_span,
                                             int32_t pq, const ProfileArgs& a, int lane) {
  using T = PTile<D>;
  constexpr int NKS = D / 32;
  constexpr int NDB = D / 16;
  const int g = lane >> 4, i16 = lane & 15;

  // ---- S^T = K Q^T: two 16-key blocks ----
  f32x4 sacc[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int r = 16 * kb + i16;
      const bf16x8 ak = *reinterpret_cast<const bf16x8*>(kt + r * T::ROW_BYTES + 16 * ((4 * ks + g) ^ T::swz_k(r)));
      sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, qf[ks], sacc[kb], 0, 0, 0);
    }

  // ---- keys past the sequence end (the head's last tile only) do not exist ----
  const int32_t kl = k0 + 4 * g;                // key of element (kb, r): kl + 16 kb + r
  if (k0 + TILE > ke) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (kl + 16 * kb + r >= ke) sacc[kb][r] = -INFINITY;
  }

  // ---- shared reference max with lazy rescaling of all three states ----
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[kb][r]);
  mx = max_x32(max_x16(mx)) * c;
  const bool bump = mx > st.m_ref + RESCALE_SLACK;
  if (__any(bump)) {
    const float m_new = bump ? mx : st.m_ref;
    const float alpha = (st.m_ref == -INFINITY) ? 0.f : exp2f(st.m_ref - m_new);
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      st.l[x] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) st.o[x][db] *= alpha;
    }
    st.m_ref = m_new;
  }
  const float m_use = (st.m_ref == -INFINITY) ? 0.f : st.m_ref;

  // ---- masks as unsigned range tests on dk: spatial keys [sp_lo, sp_lo + sp_span) (frame-major),
  // temporal keys within w_p of the query's in-frame position, in the same frame ----
  const int32_t sp_a = sp_lo - kl;
  int32_t tp_a = 0;
  uint32_t tp_span = 0;
  if constexpr (TPM == TP_INTERVAL) {
    const int32_t pbase = (int32_t)fmod_((uint32_t)kl, a.divP);
    const int32_t wth = a.P - pbase;             // dk >= wth: next frame
    const int32_t lo0 = pq - a.w_p - pbase, hi0 = lo0 + 2 * a.w_p;
    const bool first = hi0 >= 0;
    tp_a = first ? max(lo0, 0) : max(lo0 + a.P, wth);
    const int32_t tp_b = first ? min(hi0 + 1, wth) : hi0 + a.P + 1;
    tp_span = (uint32_t)max(tp_b - tp_a, 0);
  }
  bf16x8 pb[NST][3];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int32_t dk = 16 * kb + r;
      bool in_tp;
      if constexpr (TPM == TP_INTERVAL) {
        in_tp = (uint32_t)(dk - tp_a) < tp_span;
      } else {
        const int32_t pk = (int32_t)fmod_((uint32_t)(kl + dk), a.divP);
        in_tp = (uint32_t)(pk - pq + a.w_p) <= (uint32_t)(2 * a.w_p);
      }
      const bool in_sp = (uint32_t)(dk - sp_a) < sp_span;
      const float pr = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], c, -m_use));
      pb[kb >> 1][0][4 * (kb & 1) + r] = (bf16)pr;
      pb[kb >> 1][1][4 * (kb & 1) + r] = (bf16)(in_sp ? pr : 0.f);
      pb[kb >> 1][2][4 * (kb & 1) + r] = (bf16)(in_tp ? pr : 0.f);
    }
  // row sums of the bf16 weights the PV products use
#pragma unroll
  for (int x = 0; x < 3; ++x)
#pragma unroll
    for (int s = 0; s < NST; ++s) st.l[x] = add_bf16x8(pb[s][x], st.l[x]);

  // ---- O_x^T += V^T P_x^T, per 32-key step s.  The transpose read hands lane i of each
  // 16-lane group column i of the 4 rows x 16 columns its group addressed: group g reads keys
  // 32s+4g..32s+4g+3 (and, 16 rows further, 32s+16+4g..), the keys whose scores lane l holds
  // in sacc[2s] and sacc[2s+1]. ----
  const int vr = 4 * g + (i16 >> 2);
  const int vc = 4 * (i16 & 3);                 // column inside the 16-channel block
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    const char* v0 = reinterpret_cast<const char*>(vt) + (32 * s + vr) * T::ROW_BYTES;
    const char* v1 = v0 + 16 * T::ROW_BYTES;
    const int sw0 = T::swz_v(32 * s + vr), sw1 = T::swz_v(32 * s + vr + 16);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int col = 16 * db + vc;
      const int cb = 2 * (col & 7);
      const i16x4 lo = lds_read_tr(reinterpret_cast<const bf16*>(v0 + 16 * ((col >> 3) ^ sw0) + cb));
      const i16x4 hi = lds_read_tr(reinterpret_cast<const bf16*>(v1 + 16 * ((col >> 3) ^ sw1) + cb));
      const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int x = 0; x < 3; ++x)
        st.o[x][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[s][x], st.o[x][db], 0, 0, 0);
    }
  }
}

template <int D, int TPM>
__global__ __launch_bounds__(NT, 2) void profile_partial_kernel(ProfileArgs a) {
  using T = PTile<D>;
  constexpr int NKS = D / 32;
  constexpr int NDB = D / 16;
  __shared__ __attribute__((aligned(1024))) bf16 K0[TILE * D];
  __shared__ __attribute__((aligned(1024))) bf16 K1[TILE * D];
  __shared__ __attribute__((aligned(1024))) bf16 V0[TILE * D];
  __shared__ __attribute__((aligned(1024))) bf16 V1[TILE * D];

  int32_t bid = blockIdx.x;
  const int32_t zq = bid % a.n_zq;
  bid /= a.n_zq;
  const int32_t split = bid % a.nsplit;
  const int32_t bh = bid / a.nsplit;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i16 = lane & 15;

  const size_t off = (size_t)bh * (size_t)a.S * D;
  const bf16* __restrict__ Q = a.q + off;
  const bf16* __restrict__ K = a.k + off;
  const bf16* __restrict__ V = a.v + off;

  // this split's tiles: split, split + nsplit, split + 2 nsplit, ... of the head's key tiles
  const int32_t n_tiles_all = (a.S + TILE - 1) / TILE;
  const int32_t ntiles = split < n_tiles_all ? (n_tiles_all - 1 - split) / a.nsplit + 1 : 0;
  const int32_t ks = split * TILE;
  const int32_t kstride = a.nsplit * TILE;
  const int32_t ke = a.S;

  // this lane's query: q = l%16 of the wavefront's 16
  const int32_t qi = zq * QG + wave * 16 + i16;
  int32_t tq = a.idx[min(qi, a.n_q - 1)];
  tq = min(max(tq, 0), a.S - 1);
  const int32_t fq = (int32_t)fdiv((uint32_t)tq, a.divP);
  const int32_t pq = tq - fq * a.P;
  const int32_t sp_lo = max(0, fq - a.w_f) * a.P;
  const int32_t sp_hi = min(a.F, fq + a.w_f + 1) * a.P;
  bf16x8 qf[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(Q + (size_t)tq * D + 32 * s + 8 * g);

  // copies of the first NBUF-1 tiles (after the query loads, which therefore retire first)
  __builtin_amdgcn_sched_barrier(0);
  tile_copy<D>(K, ks, a.S, K0, wave, lane, false);
  tile_copy<D>(V, ks, a.S, V0, wave, lane, true);

  PState<D> st;
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    st.l[x] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) st.o[x][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  st.m_ref = -INFINITY;
  const float c = a.scale * 1.44269504088896340736f;

  // tile t: its copies (issued NBUF-1 tiles earlier) retire, the barrier publishes them and
  // frees the buffer of tile t-1, which receives tile t+NBUF-1.  Copies past the last tile
  // repeat rows of the sequence into buffers no later tile reads.
  auto step = [&](int32_t t, const bf16* kt, const bf16* vt, bf16* kn, bf16* vn) {
    __builtin_amdgcn_s_waitcnt(waitcnt_imm((NBUF - 2) * T::CPW, 0));
    tile_barrier();
    tile_copy<D>(K, ks + (t + NBUF - 1) * kstride, a.S, kn, wave, lane, false);
    tile_copy<D>(V, ks + (t + NBUF - 1) * kstride, a.S, vn, wave, lane, true);
    profile_tile<D, TPM>(st, qf, reinterpret_cast<const char*>(kt), vt, ks + t * kstride, ke, c, sp_lo,
                         (uint32_t)(sp_hi - sp_lo), pq, a, lane);
  };
  for (int32_t t = 0; t < ntiles; t += NBUF) {
    step(t, K0, V0, K1, V1);
    if (t + 1 >= ntiles) break;
    step(t + 1, K1, V1, K0, V0);
  }
  __builtin_amdgcn_s_waitcnt(VMCNT0);

  // ---- does this split hold keys of each mask for this lane's query? ----
  bool has_keys[3];
  has_keys[0] = true;
  {
    // does the split hold a tile of key range [lo, hi] (hi >= lo)?  Its first tile >= the
    // range's first is that tile plus the distance to the split's residue.
    const int32_t ns = a.nsplit;
    auto holds = [&](int32_t lo, int32_t hi) {
      const int32_t t0 = lo / TILE, t1 = hi / TILE;
      const int32_t t = t0 + ((split - t0) % ns + ns) % ns;
      return t <= t1;
    };
    has_keys[1] = holds(sp_lo, sp_hi - 1);
    const int32_t plo = max(0, pq - a.w_p), phi = min(a.P - 1, pq + a.w_p);
    bool any = false;
    for (int32_t f = 0; f < a.F && !any; ++f) any = holds(f * a.P + plo, f * a.P + phi);
    has_keys[2] = any;
  }

  // ---- this wavefront's partial states: row sums over the four lane groups ----
  const int32_t qpad = a.n_zq * QG;
  const int32_t qloc = zq * QG + wave * 16 + i16;
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    float l_tot = sum_x32(sum_x16(st.l[x]));
    if (x > 0 && has_keys[x] && !(l_tot >= UNDERFLOW_GUARD)) l_tot = -1.f;   // mark for the exact fallback
    const size_t slot = (((size_t)bh * a.nsplit + split) * 3 + x) * qpad + qloc;
    if (g == 0) {
      a.part_ml[slot * 2 + 0] = st.m_ref;
      a.part_ml[slot * 2 + 1] = l_tot;
    }
    // lane l holds channels 16 db + 4 g + r of its query
    float* po = a.part_o + slot * D + 4 * g;
#pragma unroll
    for (int db = 0; db < NDB; ++db) *reinterpret_cast<f32x4*>(po + 16 * db) = st.o[x][db];
  }
}

// Explicit instantiations: without them the host pass emitted the launch stub of only one of
// the two kernels that the launcher chooses between.
template __global__ void profile_partial_kernel<128, TP_PER_KEY>(ProfileArgs);
template __global__ void profile_partial_kernel<128, TP_INTERVAL>(ProfileArgs);
template __global__ void profile_partial_kernel<64, TP_PER_KEY>(ProfileArgs);
template __global__ void profile_partial_kernel<64, TP_INTERVAL>(ProfileArgs);

// Exact attention output (channel tid) of sampled row tq under mask x (1 spatial, 2 temporal),
// with the state's own maximum and fp32 weights: the fallback for a state whose exponentials
// underflowed against the shared reference.  All D threads of the workgroup take part.
template <int D>
__device__ float exact_masked_row(const ProfileArgs& a, int32_t bh, int32_t tq, int x, float* qs, float* wb,
                                  float* red) {
  const int tid = threadIdx.x;
  const size_t off = (size_t)bh * (size_t)a.S * D;
  const bf16* K = a.k + off;
  const bf16* V = a.v + off;
  const int32_t fq = (int32_t)fdiv((uint32_t)tq, a.divP);
  const int32_t pq = tq - fq * a.P;
  int32_t n_keys, base, wlen;
  if (x == 1) {
    base = max(0, fq - a.w_f) * a.P;
    n_keys = min(a.F, fq + a.w_f + 1) * a.P - base;
    wlen = n_keys;
  } else {
    base = max(0, pq - a.w_p);
    wlen = min(a.P - 1, pq + a.w_p) - base + 1;
    n_keys = a.F * wlen;
  }
  auto key = [&](int32_t n) { return x == 1 ? base + n : (n / wlen) * a.P + base + n % wlen; };
  auto score = [&](int32_t t) {
    const bf16* kr = K + (size_t)t * D;
    float s = 0.f;
#pragma unroll 4
    for (int c8 = 0; c8 < D; c8 += 8) {
      const bf16x8 kv = *reinterpret_cast<const bf16x8*>(kr + c8);
#pragma unroll
      for (int j = 0; j < 8; ++j) s = fmaf(qs[c8 + j], (float)kv[j], s);
    }
    return s;
  };
  qs[tid] = (float)a.q[off + (size_t)tq * D + tid];
  __syncthreads();
  // maximum of the state's scores
  float m = -INFINITY;
  for (int32_t n = tid; n < n_keys; n += D) m = fmaxf(m, score(key(n)));
  red[tid] = m;
  __syncthreads();
  for (int s2 = D / 2; s2 > 0; s2 >>= 1) {
    if (tid < s2) red[tid] = fmaxf(red[tid], red[tid + s2]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  const float c = a.scale * 1.44269504088896340736f;
  // weights D keys at a time; thread tid then accumulates channel tid over them
  float o = 0.f, l = 0.f;
  for (int32_t n0 = 0; n0 < n_keys; n0 += D) {
    const int32_t n = n0 + tid;
    const float w = n < n_keys ? exp2f((score(key(n)) - M) * c) : 0.f;
    wb[tid] = w;
    l += w;
    __syncthreads();
    const int32_t cnt = min(D, n_keys - n0);
    for (int32_t j = 0; j < cnt; ++j) o = fmaf(wb[j], (float)V[(size_t)key(n0 + j) * D + tid], o);
    __syncthreads();
  }
  red[tid] = l;
  __syncthreads();
  for (int s2 = D / 2; s2 > 0; s2 >>= 1) {
    if (tid < s2) red[tid] += red[tid + s2];
    __syncthreads();
  }
  const float L = red[0];
  __syncthreads();
  return o / L;
}

template <int D>
__global__ __launch_bounds__(D) void profile_merge_kernel(ProfileArgs a) {
  __shared__ float sm[3][MAX_SPLIT], sl[3][MAX_SPLIT], wt[3][MAX_SPLIT];
  __shared__ int marked[3];
  __shared__ double red[2][D];
  __shared__ float fb_q[D], fb_w[D], fb_red[D];
  const int32_t bh = blockIdx.x / a.n_q;
  const int32_t qg = blockIdx.x - bh * a.n_q;
  const int tid = threadIdx.x;
  const int32_t nparts = a.nsplit;
  const int32_t qpad = a.n_zq * QG;
  auto slot_of = [&](int x, int32_t p) { return (((size_t)bh * nparts + p) * 3 + x) * qpad + qg; };
  for (int t = tid; t < 3 * nparts; t += D) {
    const int x = t / nparts, p = t - (t / nparts) * nparts;
    const size_t slot = slot_of(x, p);
    sm[x][p] = a.part_ml[slot * 2];
    sl[x][p] = a.part_ml[slot * 2 + 1];
  }
  // the first MERGE_PF splits' partial outputs are fetched now, so that their latency overlaps
  // that of the (m, l) loads and the weights
  float pre[3][MERGE_PF];
#pragma unroll
  for (int x = 0; x < 3; ++x)
#pragma unroll
    for (int p = 0; p < MERGE_PF; ++p) pre[x][p] = p < nparts ? a.part_o[slot_of(x, p) * D + tid] : 0.f;
  __syncthreads();
  if (tid < 3) {
    // split p holds 2^(sm + log2 sl) of the state's mass; weights are taken against the largest
    int mk = 0;
    float M = -INFINITY;
    for (int32_t p = 0; p < nparts; ++p) {
      if (sl[tid][p] < 0.f) mk = 1;
      if (sl[tid][p] > 0.f) M = fmaxf(M, sm[tid][p] + __log2f(sl[tid][p]));
    }
    float L = 0.f;
    for (int32_t p = 0; p < nparts; ++p) {
      const float w = sl[tid][p] > 0.f ? exp2f(sm[tid][p] - M) : 0.f;
      wt[tid][p] = w;
      L += w * sl[tid][p];
    }
    const float inv = (L > 0.f) ? 1.f / L : 0.f;
    for (int32_t p = 0; p < nparts; ++p) wt[tid][p] *= inv;
    marked[tid] = mk;
  }
  __syncthreads();
  float o3[3];
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    if (marked[x]) {   // uniform across the workgroup
      const int32_t tq = min(max(a.idx[qg], 0), a.S - 1);
      o3[x] = exact_masked_row<D>(a, bh, tq, x, fb_q, fb_w, fb_red);
      continue;
    }
    float s = 0.f;
#pragma unroll
    for (int p = 0; p < MERGE_PF; ++p)
      if (p < nparts) s = fmaf(wt[x][p], pre[x][p], s);
    for (int32_t p = MERGE_PF; p < nparts; ++p) s = fmaf(wt[x][p], a.part_o[slot_of(x, p) * D + tid], s);
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
  // as many key splits as fit TARGET_WGS workgroups (two per CU) in one round
  int64_t want = TARGET_WGS / ((int64_t)BH * p.n_zq);
  const int64_t max_tiles = (S + TILE - 1) / TILE;
  if (want > MAX_SPLIT) want = MAX_SPLIT;
  if (want > max_tiles) want = max_tiles;
  if (want < 1) want = 1;
  p.nsplit = (int32_t)want;
  const size_t slots = (size_t)BH * p.nsplit * 3 * (size_t)(p.n_zq * QG);
  p.ml_floats = slots * 2;
  p.o_floats = slots * (size_t)D;
  p.sq_doubles = (size_t)BH * n_q * 2;
  return p;
}

hipError_t launch_profile(const ProfileArgs& a, hipStream_t st) {
  const dim3 g1((unsigned)((int64_t)a.BH * a.nsplit * a.n_zq));
  const dim3 g2((unsigned)((int64_t)a.BH * a.n_q));
  const dim3 g3((unsigned)a.BH);
  // the band test per tile needs frames of >= 64 tokens and >= 52 positions outside the band
  const bool interval = a.P >= 64 && (int64_t)a.P - 2 * (int64_t)a.w_p - 1 >= 52;
  if (a.D == 128) {
    if (interval) profile_partial_kernel<128, TP_INTERVAL><<<g1, NT, 0, st>>>(a);
    else profile_partial_kernel<128, TP_PER_KEY><<<g1, NT, 0, st>>>(a);
    profile_merge_kernel<128><<<g2, 128, 0, st>>>(a);
  } else if (a.D == 64) {
    if (interval) profile_partial_kernel<64, TP_INTERVAL><<<g1, NT, 0, st>>>(a);
    else profile_partial_kernel<64, TP_PER_KEY><<<g1, NT, 0, st>>>(a);
    profile_merge_kernel<64><<<g2, 64, 0, st>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  profile_finish_kernel<<<g3, NT_RED, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace svg
