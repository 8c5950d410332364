// Semantic clustering path (Sparse VideoGen2, technical summary of the explainer page, section 2):
// k-means of the Q and K rows of every head, the permutation that makes each cluster contiguous,
// centroid-based top-p selection of key clusters per query cluster, and the key lists the
// attention kernel gathers from.
//
// k-means (section 2A) is Lloyd's iteration: every row goes to the nearest centroid, then every
// centroid moves to the mean of its rows.  The assignment is a dense contraction (rows x
// centroids over D) and runs on the matrix cores: centroids are rounded to bf16, the bf16 rows
// are multiplied against them with fp32 accumulation, and each row keeps the centroid with the
// largest x.c - |c|^2 / 2 (the smallest distance; ties to the lowest index).  The update first
// sorts the tokens by cluster with a stable counting sort (the permutation of section 2A) and
// then averages each cluster's rows in fp64, so the centroids do not depend on the order in
// which the hardware happens to run.
//
// The top-p selection (section 2B) is tiny (C_q x C_k centroid products per head) and runs in
// fp64: the estimated share of attention of key cluster j for query cluster i is
// n_j exp(s_ij) / sum_j' n_j' exp(s_ij'), s_ij = scale * c_qi . c_kj (a centroid stands for all
// n_j keys of its cluster); key clusters are taken in decreasing share until the shares reach p.
#include "svg_internal.h"

namespace svg {

namespace {

constexpr int AS_BM = 128;     // rows per assignment workgroup (4 wavefronts x 32)
constexpr int AS_BN = 64;      // centroids per LDS tile
constexpr int AS_NT = 256;

// Rounds every centroid to bf16 and stores half its squared norm (of the rounded values), one
// wavefront per centroid; padding centroids past C get +inf, so that they never win.
__global__ __launch_bounds__(256) void kmeans_prep_kernel(const float* __restrict__ cent, bf16* __restrict__ cb,
                                                          float* __restrict__ hn, int32_t BH, int32_t C, int32_t Cpad,
                                                          int32_t D) {
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= (int64_t)BH * Cpad) return;
  const int32_t bh = (int32_t)(i / Cpad), c = (int32_t)(i - (int64_t)bh * Cpad);
  bf16* dst = cb + i * D;
  float s = 0.f;
  for (int d = lane; d < D; d += 64) {
    const bf16 v = c < C ? (bf16)cent[((int64_t)bh * C + c) * D + d] : (bf16)0.f;
    dst[d] = v;
    const float f = (float)v;
    s = fmaf(f, f, s);
  }
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) hn[i] = c < C ? 0.5f * s : INFINITY;
}

// Cold start: centroid c of every head is the row at token idx[c] (clamped into [0, S)).
__global__ void kmeans_init_kernel(const bf16* __restrict__ x, const int32_t* __restrict__ idx, float* __restrict__ cent,
                                   int32_t BH, int32_t S, int32_t C, int32_t D) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)BH * C * D) return;
  const int32_t d = (int32_t)(i % D);
  const int64_t r = i / D;
  const int32_t c = (int32_t)(r % C);
  const int32_t bh = (int32_t)(r / C);
  const int32_t t = min(max(idx[c], 0), S - 1);
  cent[i] = (float)x[((int64_t)bh * S + t) * D + d];
}

// Nearest centroid of 128 rows per workgroup.  Wavefront w holds rows 32w..32w+31 as the B
// operand of v_mfma_f32_32x32x16_bf16 (one row per lane column); tiles of 64 centroids are the
// A operand from LDS, double-buffered: the next tile's global loads are in flight while the
// current one is multiplied.  The accumulator starts at -|c|^2/2 of its centroid, so it ends at
// the score x.c - |c|^2/2 itself.  It gives each lane one row and 16 centroids per 32-block in
// increasing order: a lane takes the tile's maximum, and only when that beats its best so far
// looks up which centroid gave it (the first one, the lowest index among equals).  Four
// workgroups fit a CU (at most 128 VGPRs), so that one's loads overlap the others' products.
template <int D>
__global__ __launch_bounds__(AS_NT, 4) void kmeans_assign_kernel(const bf16* __restrict__ x, const bf16* __restrict__ cb,
                                                              const float* __restrict__ hn, int32_t* __restrict__ labels,
                                                              int32_t S, int32_t Cpad, int32_t nrb) {
  constexpr int NKS = D / 16;
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int RPB = 16 / CPR;               // rows per 256-byte bank period
  constexpr int PER_T = AS_BN * CPR / AS_NT;  // 16-byte chunks each thread moves per tile
  __shared__ __attribute__((aligned(16))) bf16 ct[2][AS_BN * D];
  __shared__ __attribute__((aligned(16))) float th[2][AS_BN];

  const int32_t bh = blockIdx.x / nrb;
  const int32_t rb = blockIdx.x - bh * nrb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int32_t row = rb * AS_BM + wave * 32 + l32;
  const bf16* xh = x + (size_t)bh * S * D;
  const bf16* cbh = cb + (size_t)bh * Cpad * D;
  const float* hnh = hn + (size_t)bh * Cpad;

  bf16x8 xf[NKS];
  const bf16* xr = xh + (size_t)min(row, S - 1) * D;
#pragma unroll
  for (int s = 0; s < NKS; ++s) xf[s] = *reinterpret_cast<const bf16x8*>(xr + 16 * s + 8 * hh);

  // chunk o = tid + AS_NT * i of a tile: row o / CPR, chunk o % CPR, stored at slot
  // chunk ^ ((row / RPB) & (CPR - 1)) of its row
  u32x4 pre[PER_T];
  float pre_h = 0.f;
  auto fetch = [&](int32_t c0) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int o = tid + AS_NT * i;
      pre[i] = *reinterpret_cast<const u32x4*>(cbh + (size_t)(c0 + o / CPR) * D + 8 * (o % CPR));
    }
    if (tid < AS_BN) pre_h = -hnh[c0 + tid];
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int o = tid + AS_NT * i;
      const int r = o / CPR, q = o % CPR;
      *reinterpret_cast<u32x4*>(&ct[buf][r * D + 8 * (q ^ ((r / RPB) & (CPR - 1)))]) = pre[i];
    }
    if (tid < AS_BN) th[buf][tid] = pre_h;
  };

  float best = -INFINITY;
  int32_t best_c = 0;
  const int nt = Cpad / AS_BN;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    if (t + 1 < nt) fetch((t + 1) * AS_BN);
    f32x16 acc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 h4 = *reinterpret_cast<const f32x4*>(&th[buf][blk * 32 + 8 * g4 + 4 * hh]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[blk][4 * g4 + e] = h4[e];
      }
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int r = blk * 32 + l32;
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(&ct[buf][r * D + 8 * ((2 * s + hh) ^ ((r / RPB) & (CPR - 1)))]);
        acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xf[s], acc[blk], 0, 0, 0);
      }
    float m = acc[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) m = fmaxf(m, acc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) m = fmaxf(m, acc[1][r]);
    if (m > best) {
      // the first centroid of the tile that reaches m: scan from the last one down
      int cl = 0;
#pragma unroll
      for (int blk = 1; blk >= 0; --blk)
#pragma unroll
        for (int r = 15; r >= 0; --r)
          if (acc[blk][r] == m) cl = blk * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
      best = m;
      best_c = t * AS_BN + cl;
    }
    if (t + 1 < nt) stash(buf ^ 1);
    __syncthreads();
  }
  // the two lane halves hold interleaved centroids: larger score wins, then lower index
  const auto rb2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(best), __float_as_uint(best), false, false);
  const auto rc2 = __builtin_amdgcn_permlane32_swap((uint32_t)best_c, (uint32_t)best_c, false, false);
  const float ob = __uint_as_float(hh ? rb2[0] : rb2[1]);
  const int32_t oc = (int32_t)(hh ? rc2[0] : rc2[1]);
  if (ob > best || (ob == best && oc < best_c)) best_c = oc;
  if (hh == 0 && row < S) labels[(size_t)bh * S + row] = best_c;
}

constexpr int CHUNK = 256;      // tokens per counting-sort chunk (one wavefront's share)

// counts[bh][chunk][c]: tokens of the chunk in cluster c.
__global__ __launch_bounds__(CHUNK) void cluster_hist_kernel(const int32_t* __restrict__ labels,
                                                             int32_t* __restrict__ counts, int32_t S, int32_t C,
                                                             int32_t nchunk) {
  extern __shared__ int32_t cnt[];
  const int32_t chunk = blockIdx.x, bh = blockIdx.y;
  for (int c = threadIdx.x; c < C; c += CHUNK) cnt[c] = 0;
  __syncthreads();
  const int32_t t = chunk * CHUNK + threadIdx.x;
  if (t < S) atomicAdd(&cnt[min(max(labels[(size_t)bh * S + t], 0), C - 1)], 1);
  __syncthreads();
  int32_t* out = counts + ((size_t)bh * nchunk + chunk) * C;
  for (int c = threadIdx.x; c < C; c += CHUNK) out[c] = cnt[c];
}

// In place: counts[bh][chunk][c] -> first sorted position of the chunk's tokens of cluster c
// (clusters in index order, chunks in order inside a cluster); offsets[bh][c] = start of
// cluster c, offsets[bh][C] = S.  Thread c walks cluster c's counts down the chunks (adjacent
// threads read adjacent words), several loads in flight at a time.
constexpr int SCAN_NT = 1024;
constexpr int SCAN_UNR = 8;
__global__ __launch_bounds__(SCAN_NT) void cluster_scan_kernel(int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ offsets, int32_t S, int32_t C,
                                                               int32_t nchunk) {
  __shared__ int32_t part[SCAN_NT];
  const int32_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t* cnt = counts + (size_t)bh * nchunk * C;
  // thread tid owns clusters tid, tid + SCAN_NT, ... (at most C / SCAN_NT + 1 of them); their
  // totals are scanned in cluster order below, one pass per owned cluster
  int32_t* off = offsets + (size_t)bh * (C + 1);
  int32_t carry = 0;
  for (int c0 = 0; c0 < C; c0 += SCAN_NT) {
    const int c = c0 + tid;
    int32_t own = 0;
    if (c < C) {
      int32_t k = 0;
      for (; k + SCAN_UNR <= nchunk; k += SCAN_UNR) {
        int32_t v[SCAN_UNR];
#pragma unroll
        for (int e = 0; e < SCAN_UNR; ++e) v[e] = cnt[(size_t)(k + e) * C + c];
#pragma unroll
        for (int e = 0; e < SCAN_UNR; ++e) own += v[e];
      }
      for (; k < nchunk; ++k) own += cnt[(size_t)k * C + c];
    }
    __syncthreads();
    part[tid] = own;
    __syncthreads();
    // inclusive scan of the totals of clusters c0 .. c0 + SCAN_NT - 1 (Hillis-Steele)
    for (int o = 1; o < SCAN_NT; o <<= 1) {
      const int32_t w = tid >= o ? part[tid - o] : 0;
      __syncthreads();
      part[tid] += w;
      __syncthreads();
    }
    int32_t run = carry + part[tid] - own;
    carry += part[SCAN_NT - 1];
    if (c < C) {
      off[c] = run;
      int32_t k = 0;
      for (; k + SCAN_UNR <= nchunk; k += SCAN_UNR) {
        int32_t v[SCAN_UNR];
#pragma unroll
        for (int e = 0; e < SCAN_UNR; ++e) v[e] = cnt[(size_t)(k + e) * C + c];
#pragma unroll
        for (int e = 0; e < SCAN_UNR; ++e) {
          cnt[(size_t)(k + e) * C + c] = run;
          run += v[e];
        }
      }
      for (; k < nchunk; ++k) {
        const int32_t n = cnt[(size_t)k * C + c];
        cnt[(size_t)k * C + c] = run;
        run += n;
      }
    }
  }
  if (tid == 0) off[C] = S;
}

// Stable scatter: one wavefront walks its chunk 64 tokens at a time; tokens of one round with
// equal labels are ranked by lane, and rounds go in token order.  (Labels and the indices read
// from them are clamped in range here and below, so that inconsistent inputs cannot address
// memory outside the buffers.)
__global__ __launch_bounds__(64) void cluster_scatter_kernel(const int32_t* __restrict__ labels,
                                                             const int32_t* __restrict__ base,
                                                             int32_t* __restrict__ perm, int32_t S, int32_t C,
                                                             int32_t nchunk) {
  extern __shared__ int32_t ctr[];
  const int32_t chunk = blockIdx.x, bh = blockIdx.y;
  const int lane = threadIdx.x;
  const int32_t* b = base + ((size_t)bh * nchunk + chunk) * C;
  for (int c = lane; c < C; c += 64) ctr[c] = b[c];
  __syncthreads();
  const int32_t t0 = chunk * CHUNK, t1 = min(t0 + CHUNK, S);
  const uint64_t below = (1ull << lane) - 1ull;
  for (int32_t r0 = t0; r0 < t1; r0 += 64) {
    const int32_t t = r0 + lane;
    const bool valid = t < t1;
    const int32_t lab = valid ? min(max(labels[(size_t)bh * S + t], 0), C - 1) : -1;
    uint64_t pending = __ballot(valid);
    int32_t pos = 0;
    while (pending) {
      const int leader = __builtin_ctzll(pending);
      const int32_t L = __shfl(lab, leader);
      const uint64_t same = __ballot(lab == L) & pending;
      if (lab == L) pos = ctr[L] + __popcll(same & below);
      __builtin_amdgcn_wave_barrier();
      if (lane == leader) ctr[L] += __popcll(same);
      __builtin_amdgcn_wave_barrier();
      pending &= ~same;
    }
    if (valid) perm[(size_t)bh * S + pos] = t;
  }
}

// Mean of each cluster's rows in fp64, one workgroup per (cluster, head).  A row is read as
// 16-byte pieces by D/8 lanes, so one wavefront load covers 64*8/D rows ("slots"); each
// wavefront keeps UNR such loads in flight.  Row j of the cluster goes to a fixed (wavefront,
// unroll step, slot), and the partial sums are combined in a fixed order, so the result does
// not depend on timing.  An empty cluster keeps its centroid.
constexpr int UP_NT = 256;
constexpr int UP_UNR = 4;
template <int D>
__global__ __launch_bounds__(UP_NT) void kmeans_update_kernel(const bf16* __restrict__ x, const int32_t* __restrict__ perm,
                                                              const int32_t* __restrict__ offsets,
                                                              float* __restrict__ cent, int32_t S, int32_t C) {
  constexpr int LPR = D / 8;                   // lanes per row
  constexpr int SLOTS = 64 / LPR;              // rows per wavefront load
  constexpr int NW = UP_NT / 64;
  constexpr int PER_IT = NW * UP_UNR * SLOTS;  // rows per workgroup iteration
  __shared__ double red[NW * SLOTS][D];
  const int32_t c = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = lane / LPR, piece = lane % LPR;
  const int32_t* off = offsets + (size_t)bh * (C + 1);
  const int32_t j0 = off[c], j1 = off[c + 1];
  if (j1 <= j0) return;
  const bf16* xh = x + (size_t)bh * S * D + 8 * piece;
  const int32_t* ph = perm + (size_t)bh * S;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  for (int32_t jb = j0; jb < j1; jb += PER_IT) {
    u32x4 v[UP_UNR];
    bool ok[UP_UNR];
#pragma unroll
    for (int u = 0; u < UP_UNR; ++u) {
      const int32_t j = jb + (u * NW + wave) * SLOTS + slot;
      ok[u] = j < j1;
      const int32_t t = min(max(ph[min(j, j1 - 1)], 0), S - 1);
      v[u] = *reinterpret_cast<const u32x4*>(xh + (size_t)t * D);
    }
#pragma unroll
    for (int u = 0; u < UP_UNR; ++u) {
      if (!ok[u]) continue;
      const bf16x8 b = __builtin_bit_cast(bf16x8, v[u]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += (double)(float)b[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[wave * SLOTS + slot][8 * piece + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    double s = 0.0;
    for (int i = 0; i < NW * SLOTS; ++i) s += red[i][tid];
    cent[((size_t)bh * C + c) * D + tid] = (float)(s / (double)(j1 - j0));
  }
}

// ---------------------------------------------------------------------------------------------
// Centroid top-p selection, one workgroup per (head, query cluster).
// ---------------------------------------------------------------------------------------------
constexpr int TP_NT = 256;
constexpr int TP_MAXC = 1024;

__global__ __launch_bounds__(TP_NT) void centroid_topp_kernel(const float* __restrict__ cq, const float* __restrict__ ck,
                                                              const int32_t* __restrict__ k_off,
                                                              uint8_t* __restrict__ sel, int32_t Cq, int32_t Ck,
                                                              int32_t D, double scale, double p) {
  __shared__ double qv[128];
  __shared__ double w[TP_MAXC];
  __shared__ int32_t ix[TP_MAXC];
  __shared__ double red[TP_NT];
  const int32_t i = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x;
  const float* qrow = cq + ((size_t)bh * Cq + i) * D;
  const float* kh = ck + (size_t)bh * Ck * D;
  const int32_t* off = k_off + (size_t)bh * (Ck + 1);
  for (int d = tid; d < D; d += TP_NT) qv[d] = (double)qrow[d];
  __syncthreads();
  // scores; empty key clusters get -inf
  double mx = -INFINITY;
  for (int j = tid; j < Ck; j += TP_NT) {
    const float* kr = kh + (size_t)j * D;
    double s = 0.0;
    for (int d = 0; d < D; ++d) s = fma(qv[d], (double)kr[d], s);
    s = (off[j + 1] > off[j]) ? scale * s : -INFINITY;
    w[j] = s;
    mx = fmax(mx, s);
  }
  red[tid] = mx;
  __syncthreads();
  for (int o = TP_NT / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] = fmax(red[tid], red[tid + o]);
    __syncthreads();
  }
  mx = red[0];
  __syncthreads();
  double z = 0.0;
  for (int j = tid; j < Ck; j += TP_NT) {
    const double e = (double)(off[j + 1] - off[j]) * exp(w[j] - mx);
    w[j] = e;
    z += e;
  }
  red[tid] = z;
  __syncthreads();
  for (int o = TP_NT / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  z = red[0];
  // shares, padded to a power of two with entries that sort last
  int n2 = 1;
  while (n2 < Ck) n2 <<= 1;
  for (int j = tid; j < n2; j += TP_NT) {
    if (j < Ck) {
      w[j] = w[j] / z;
      ix[j] = j;
    } else {
      w[j] = -1.0;
      ix[j] = j;
    }
  }
  __syncthreads();
  // bitonic sort: decreasing share, increasing index among equal shares
  for (int k = 2; k <= n2; k <<= 1)
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int a = tid; a < n2; a += TP_NT) {
        const int b = a ^ jj;
        if (b > a) {
          const bool up = (a & k) == 0;
          const double wa = w[a], wb = w[b];
          const int32_t ia = ix[a], ib = ix[b];
          const bool a_first = wa > wb || (wa == wb && ia < ib);
          if (a_first != up) {
            w[a] = wb; w[b] = wa;
            ix[a] = ib; ix[b] = ia;
          }
        }
      }
      __syncthreads();
    }
  uint8_t* srow = sel + ((size_t)bh * Cq + i) * Ck;
  for (int j = tid; j < Ck; j += TP_NT) srow[j] = 0;
  __syncthreads();
  // the shortest prefix reaching p, summed in order
  if (tid == 0) {
    double acc = 0.0;
    for (int r = 0; r < Ck; ++r) {
      if (w[r] <= 0.0) break;
      srow[ix[r]] = 1;
      acc += w[r];
      if (acc >= p) break;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Key list of each (head, query cluster): the sorted positions of its selected key clusters, in
// cluster order, mapped to token rows; and its length.
// ---------------------------------------------------------------------------------------------
constexpr int KL_NT = 256;
__global__ __launch_bounds__(KL_NT) void cluster_keylist_kernel(const uint8_t* __restrict__ sel,
                                                                const int32_t* __restrict__ k_perm,
                                                                const int32_t* __restrict__ k_off,
                                                                int32_t* __restrict__ klist, int32_t* __restrict__ klen,
                                                                int32_t S, int32_t Cq, int32_t Ck) {
  __shared__ int32_t start[TP_MAXC + 1];   // first list position of the m-th selected cluster
  __shared__ int32_t cid[TP_MAXC];         // its cluster index
  __shared__ int32_t part[KL_NT];
  const int32_t i = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x;
  const uint8_t* srow = sel + ((size_t)bh * Cq + i) * Ck;
  const int32_t* off = k_off + (size_t)bh * (Ck + 1);
  // thread tid owns clusters [tid * per, ...): selected count and key count
  const int per = (Ck + KL_NT - 1) / KL_NT;
  const int c_lo = min(tid * per, Ck), c_hi = min(c_lo + per, Ck);
  // A cluster's size comes from the caller's offsets; it is clamped to [0, S], and every key
  // count below saturates at S, so a list never outgrows its S-entry row whatever the offsets.
  auto csize = [&](int c) { return min(max(off[c + 1] - off[c], 0), S); };
  int32_t nsel = 0, nkey = 0;
  for (int c = c_lo; c < c_hi; ++c)
    if (srow[c]) { ++nsel; nkey = min(nkey + csize(c), S); }
  part[tid] = nsel;
  __syncthreads();
  for (int o = 1; o < KL_NT; o <<= 1) {
    const int32_t v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t m = part[tid] - nsel;
  const int32_t msel = part[KL_NT - 1];
  __syncthreads();
  part[tid] = nkey;
  __syncthreads();
  // inclusive scan with saturating addition (associative on non-negative counts)
  for (int o = 1; o < KL_NT; o <<= 1) {
    const int32_t v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] = min(part[tid] + v, S);
    __syncthreads();
  }
  int32_t pos = tid > 0 ? part[tid - 1] : 0;
  const int32_t L = part[KL_NT - 1];
  for (int c = c_lo; c < c_hi; ++c)
    if (srow[c]) {
      start[m] = pos;
      cid[m] = c;
      ++m;
      pos = min(pos + csize(c), S);
    }
  if (tid == 0) {
    start[msel] = L;
    klen[(size_t)bh * Cq + i] = L;
  }
  __syncthreads();
  int32_t* out = klist + ((size_t)bh * Cq + i) * S;
  const int32_t* kp = k_perm + (size_t)bh * S;
  for (int32_t q = tid; q < L; q += KL_NT) {
    // last selected cluster whose start is <= q
    int lo = 0, hi = msel - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (start[mid] <= q) lo = mid; else hi = mid - 1;
    }
    out[q] = min(max(kp[min(max(off[cid[lo]] + (q - start[lo]), 0), S - 1)], 0), S - 1);
  }
}

// Work items of the attention kernel: (query cluster << 16) | 256-row tile, per head, in cluster
// order; unused slots -1.  One workgroup per head: thread c counts cluster c's tiles, a block scan
// places them.
constexpr int IT_NT = 1024;
__global__ __launch_bounds__(IT_NT) void cluster_items_kernel(const int32_t* __restrict__ q_off,
                                                             int32_t* __restrict__ items, int32_t Cq,
                                                             int32_t per_head, int32_t tile_rows) {
  __shared__ int32_t part[IT_NT];
  const int32_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t* off = q_off + (size_t)bh * (Cq + 1);
  int32_t* it = items + (size_t)bh * per_head;
  int32_t carry = 0;
  for (int32_t c0 = 0; c0 < Cq; c0 += IT_NT) {
    const int32_t c = c0 + tid;
    const int32_t rows = c < Cq ? max(off[c + 1] - off[c], 0) : 0;
    const int32_t nt = (rows + tile_rows - 1) / tile_rows;
    __syncthreads();
    part[tid] = nt;
    __syncthreads();
    for (int o = 1; o < IT_NT; o <<= 1) {
      const int32_t v = tid >= o ? part[tid - o] : 0;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    const int32_t first = carry + part[tid] - nt;
    for (int32_t t = 0; t < nt && first + t < per_head; ++t) it[first + t] = (c << 16) | t;
    carry += part[IT_NT - 1];
  }
  for (int32_t n = carry + tid; n < per_head; n += IT_NT) it[n] = -1;
}

// Explicit instantiations, so that the host pass emits every launch stub the launchers use.
template __global__ void kmeans_assign_kernel<64>(const bf16*, const bf16*, const float*, int32_t*, int32_t, int32_t,
                                                  int32_t);
template __global__ void kmeans_assign_kernel<128>(const bf16*, const bf16*, const float*, int32_t*, int32_t, int32_t,
                                                   int32_t);
template __global__ void kmeans_update_kernel<64>(const bf16*, const int32_t*, const int32_t*, float*, int32_t, int32_t);
template __global__ void kmeans_update_kernel<128>(const bf16*, const int32_t*, const int32_t*, float*, int32_t,
                                                   int32_t);

inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

}  // namespace

int32_t kmeans_cpad(int32_t C) { return (C + AS_BN - 1) / AS_BN * AS_BN; }
int32_t cluster_nchunk(int32_t S) { return (S + CHUNK - 1) / CHUNK; }

hipError_t launch_kmeans(const KmeansArgs& a, hipStream_t st) {
  const int32_t Cpad = kmeans_cpad(a.C);
  const int32_t nchunk = cluster_nchunk(a.S);
  if (a.init_idx) {
    kmeans_init_kernel<<<cdiv((int64_t)a.BH * a.C * a.D, 256), 256, 0, st>>>(a.x, a.init_idx, a.cent, a.BH, a.S, a.C,
                                                                             a.D);
  }
  const int32_t nrb = (a.S + AS_BM - 1) / AS_BM;
  for (int32_t it = 0; it < a.iters; ++it) {
    kmeans_prep_kernel<<<cdiv((int64_t)a.BH * Cpad, 4), 256, 0, st>>>(a.cent, a.cb, a.hn, a.BH, a.C, Cpad, a.D);
    if (a.D == 128)
      kmeans_assign_kernel<128><<<(unsigned)(a.BH * nrb), AS_NT, 0, st>>>(a.x, a.cb, a.hn, a.labels, a.S, Cpad, nrb);
    else
      kmeans_assign_kernel<64><<<(unsigned)(a.BH * nrb), AS_NT, 0, st>>>(a.x, a.cb, a.hn, a.labels, a.S, Cpad, nrb);
    const dim3 g2((unsigned)nchunk, (unsigned)a.BH);
    cluster_hist_kernel<<<g2, CHUNK, a.C * sizeof(int32_t), st>>>(a.labels, a.counts, a.S, a.C, nchunk);
    cluster_scan_kernel<<<(unsigned)a.BH, SCAN_NT, 0, st>>>(a.counts, a.offsets, a.S, a.C, nchunk);
    cluster_scatter_kernel<<<g2, 64, a.C * sizeof(int32_t), st>>>(a.labels, a.counts, a.perm, a.S, a.C, nchunk);
    const dim3 g3((unsigned)a.C, (unsigned)a.BH);
    if (a.D == 128)
      kmeans_update_kernel<128><<<g3, UP_NT, 0, st>>>(a.x, a.perm, a.offsets, a.cent, a.S, a.C);
    else
      kmeans_update_kernel<64><<<g3, UP_NT, 0, st>>>(a.x, a.perm, a.offsets, a.cent, a.S, a.C);
  }
  return hipGetLastError();
}

hipError_t launch_centroid_topp(const ToppArgs& a, hipStream_t st) {
  const dim3 g((unsigned)a.Cq, (unsigned)a.BH);
  centroid_topp_kernel<<<g, TP_NT, 0, st>>>(a.cq, a.ck, a.k_off, a.sel, a.Cq, a.Ck, a.D, a.scale, a.p);
  return hipGetLastError();
}

hipError_t launch_cluster_lists(const ClusterListArgs& a, hipStream_t st) {
  const dim3 g((unsigned)a.Cq, (unsigned)a.BH);
  cluster_keylist_kernel<<<g, KL_NT, 0, st>>>(a.sel, a.k_perm, a.k_off, a.klist, a.klen, a.S, a.Cq, a.Ck);
  cluster_items_kernel<<<(unsigned)a.BH, IT_NT, 0, st>>>(a.q_off, a.items, a.Cq, a.items_per_head, a.tile_rows);
  return hipGetLastError();
}

}  // namespace svg
