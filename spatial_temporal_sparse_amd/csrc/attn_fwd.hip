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
// Work decomposition: one workgroup of 8 wavefronts per (head, 256-row query block), two
// groups of 4 wavefronts with 128 rows each (32 rows per wavefront), scheduled in ping-pong
// (see "Ping-pong schedule" below).  Key tiles of 64 rows are double-buffered and value tiles
// triple-buffered in LDS, shared by all 8 wavefronts.  They are copied from HBM straight into LDS
// (global_load_lds_dwordx4: no register staging); each wavefront instruction fills 1 KB of
// LDS, and the 16-byte chunks of a row are XOR-swizzled by row on the global side so that
// both LDS read patterns below are free of bank conflicts.
//
// Per tile and wavefront, with v_mfma_f32_32x32x16_bf16 (lane l: row/col l%32, k-half l/32):
//   S^T[key][query] = K Q^T      A = K rows from LDS (one 16-byte read per MFMA),
//                                B = Q kept in registers for the whole loop.
//   The accumulator puts one query per lane (column l%32) and 16 keys per lane, so the row
//   max needs one cross-half exchange (v_permlane32_swap) and the row sum none until the end.
//   O^T[d][query] += V^T P^T     A = V^T read from the row-major V tile with the LDS
//                                transpose read (ds_read_b64_tr_b16), B = P^T converted to
//                                bf16 straight from the S^T accumulator registers: the key
//                                order inside each 16-key step is permuted identically on
//                                both operands, which leaves the contraction unchanged.
//   The O^T accumulator again holds one query per lane, so the online-softmax rescale is a
//   per-lane scalar.  It is applied lazily: the reference moves only when a weight would
//   exceed 2^8, which the tile's row sum reveals (see phase_softmax), so most tiles need
//   neither a rescale nor a maximum.
// exp2 with log2(e) folded into the softmax scale; fp32 accumulation; P rounded to bf16 for
// the PV product; output divided by the row sum of those bf16 weights (so they sum to 1) and
// rounded to bf16 (round-to-nearest-even).
#include "svg_internal.h"

namespace svg {

namespace {

constexpr int BN = ATTN_BN;       // keys per tile

// Workgroups are handed to the 8 XCDs round-robin by index, and each XCD has its own L2.
// Consecutive query blocks of a head read (almost) the same key/value tiles in the same
// order, so each XCD is given runs of XCD_RUN consecutive work items -- about as many as it
// keeps resident -- instead of every 8th item.
#ifndef SVG_ATTN_XCD_RUN
#define SVG_ATTN_XCD_RUN 32
#endif
// LDS operand reads are issued for this many MFMAs ahead of the one that consumes them (the
// LDS read latency exceeds two back-to-back MFMAs).
#ifndef SVG_ATTN_M_AHEAD
#define SVG_ATTN_M_AHEAD 3
#endif
constexpr int NXCD = 8;
constexpr int XCD_RUN = SVG_ATTN_XCD_RUN;

// Bijection on [0, n): block b runs on XCD b % 8; XCD x takes runs x, x+8, x+16, ... of
// XCD_RUN consecutive items.  A tail of fewer than 8 runs keeps the identity order.
__device__ __forceinline__ int32_t xcd_item(int32_t b, int32_t n) {
  const int32_t full = (n / (NXCD * XCD_RUN)) * (NXCD * XCD_RUN);
  if (b >= full) return b;
  const int32_t x = b % NXCD, slot = b / NXCD;
  return (x + NXCD * (slot / XCD_RUN)) * XCD_RUN + slot % XCD_RUN;
}

// Tile geometry in LDS: rows of D bf16 (no padding), 16-byte chunks XOR-swizzled per row.
template <int D>
struct TileLds {
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int RPB = 16 / CPR;         // rows per 256-byte bank period
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;
  // K is read 16 rows x one chunk per 16 lanes: spread those rows over all 16 chunk slots.
  static __device__ __forceinline__ int swz_k(int r) { return (r / RPB) & (CPR - 1); }
  // V is read by the transpose read, 4 rows x 4 consecutive chunks per 32 lanes: give each
  // of the 4 rows its own group of 4 chunk slots.
  static __device__ __forceinline__ int swz_v(int r) { return 4 * ((r / RPB) & (CPR / 4 - 1)); }
};

__global__ void head_order_kernel(const uint8_t* __restrict__ kind, int32_t* __restrict__ order, int32_t BH,
                                  int32_t* __restrict__ queue) {
  // Heavier heads first (spatial, dense), temporal heads last; stable within a class.  Also
  // clears the per-XCD work counters of the persistent kernel.
  if (queue != nullptr && threadIdx.x < NXCD && blockIdx.x == 0) queue[threadIdx.x] = 0;
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int32_t n = 0;
  for (int32_t h = 0; h < BH; ++h)
    if (kind[h] != KIND_TEMPORAL) order[n++] = h;
  for (int32_t h = 0; h < BH; ++h)
    if (kind[h] == KIND_TEMPORAL) order[n++] = h;
}

// ------------------------------------------------------------------------------------------
// Ping-pong schedule.  A workgroup of 8 wavefronts owns 256 query rows: group A (wavefronts
// 0-3) rows 0-127 and group B (wavefronts 4-7) rows 128-255, 32 rows per wavefront; the two
// wavefronts that share a SIMD belong to different groups.  Both groups walk the same key
// tiles t_0..t_{T-1} (the union of their ranges) in phases separated by workgroup barriers:
//   M(i) : O^T += V^T P^T for tile i-1, then S^T = K Q^T for tile i     (matrix cores)
//   X(i) : mask, online softmax and bf16 packing of P for tile i        (vector ALUs)
// Group A runs M(0) X(0) M(1) X(1) ... M(T); group B runs the same sequence one phase later,
// so in every phase one group feeds the matrix cores while the other does exponentials.  The
// two parts of an M phase are one scheduling region, so the K reads of QK^T are already in
// flight while the last PV products run.  The group in its M phase issues first (s_setprio):
// its MFMAs are few and long, and the exponentials fill the issue slots between them.
// Every phase runs the same code for every tile index: a tile outside a group's range is a
// boundary tile whose element mask empties it (P^T = 0; running max and sum unchanged).
// The HBM -> LDS copies are split between the groups and issued at the start of each group's
// vector phase: in X(j), the phase after its M(j), group A copies K(t_{j+1}) (into the K
// buffer M(j-1) read) and group B copies V(t_{j+1}) (into the V buffer of V(t_{j-2})).  A copy
// holds its wavefront at issue, and the vector phases have the slack for it.  Each group
// waits for its copies at the end of that X phase and the barrier after it publishes them,
// one phase (K) or two phases (V) before their first reader.  So no copy is in flight during
// an M phase; each M phase still starts with an explicit wait on vector memory (free at run
// time) so that the compiler knows it and counts the LDS waits instead of draining them.  After that wait at the end of its X phase, a group reads the first V^T
// operand of its next M phase: that V tile was published a phase earlier.  The K buffers are
// two distinct LDS objects and the phase loop is unrolled by four, so every K access names one
// of them.
// ------------------------------------------------------------------------------------------
constexpr int PP_BM = 256;        // query rows per workgroup
constexpr int PP_NT = 512;        // 8 wavefronts

// Per-lane state of one query row (lane's query = column l%32 of its wavefront's 32 rows).
template <int D>
struct RowState {
  f32x16 oacc[D / 32];       // O^T accumulator, one 32-row d block per entry
  f32x16 sacc[2];            // S^T of the current tile (two 32-key blocks)
  bf16x8 pb[BN / 16];        // P^T of the previous tile as bf16 MFMA operands (16 keys each)
  float m_ref;               // reference max (log2 units) of oacc / l_run
  float l_run;               // this lane's share of the row sum
  bool m_set;                // m_ref has been set from an allowed key (same in both halves of a row)
};

// the value of x held by lane l^32
__device__ __forceinline__ float other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // lanes 0-31 find their partner in r[1], lanes 32-63 in r[0]; the other entry is x itself
  return __uint_as_float(r[0]) + __uint_as_float(r[1]) - x;
}
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(fmaxf(x, __uint_as_float(r[0])), __uint_as_float(r[1]));
}

// S^T = K Q^T for the 64 keys of a tile: two independent 32-key accumulation chains.
template <int D>
__device__ __forceinline__ void phase_qk(RowState<D>& st, const bf16x8 (&qf)[D / 16], const char* kb, int l32,
                                         int hh) {
  using T = TileLds<D>;
  constexpr int NKS = D / 16;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.sacc[blk][r] = 0.f;
#pragma unroll
  for (int s = 0; s < NKS; ++s)
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int r = blk * 32 + l32;
      const bf16x8 ak = *reinterpret_cast<const bf16x8*>(kb + r * T::ROW_BYTES + 16 * ((2 * s + hh) ^ T::swz_k(r)));
      st.sacc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[s], st.sacc[blk], 0, 0, 0);
    }
}

// V^T operands of a matrix phase's first PV products that its wavefront reads at the end of its
// previous (vector) phase, so that the phase opens with an MFMA instead of an LDS wait (deeper
// prefetch measured no better)
constexpr int NPRE = 1;
// V^T operand of PV step 0, d block j
template <int D>
__device__ __forceinline__ bf16x8 read_vt0(const char* vbase, int v_row, int v_col, int j) {
  using T = TileLds<D>;
  const char* v0 = vbase + v_row * T::ROW_BYTES;
  const char* v1 = v0 + 8 * T::ROW_BYTES;
  const int col = 32 * j + v_col;
  const int cb = 2 * (col & 7);
  const i16x4 lo = lds_read_tr(reinterpret_cast<const bf16*>(v0 + 16 * ((col >> 3) ^ T::swz_v(v_row)) + cb));
  const i16x4 hi = lds_read_tr(reinterpret_cast<const bf16*>(v1 + 16 * ((col >> 3) ^ T::swz_v(v_row + 8)) + cb));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// O^T += V^T P^T for the 64 keys of a tile (four 16-key steps).
template <int D>
__device__ __forceinline__ void phase_pv(RowState<D>& st, const char* vbase, int v_row, int v_col,
                                         const bf16x8 (&av0)[NPRE]) {
  using T = TileLds<D>;
  constexpr int NDB = D / 32;
#pragma unroll
  for (int s = 0; s < BN / 16; ++s) {
    const int r0 = 16 * s + v_row;          // rows of the two transpose reads: r0, r0 + 8
    const char* v0 = vbase + r0 * T::ROW_BYTES;
    const char* v1 = v0 + 8 * T::ROW_BYTES;
    const int sw0 = T::swz_v(r0), sw1 = T::swz_v(r0 + 8);
#pragma unroll
    for (int j = 0; j < NDB; ++j) {
      bf16x8 av;
      if (s == 0 && j < NPRE) {
        av = av0[j];                        // read at the end of the previous phase
      } else {
        const int col = 32 * j + v_col;     // logical element column
        const int cb = 2 * (col & 7);       // byte inside the 16-byte chunk
        const i16x4 lo = lds_read_tr(reinterpret_cast<const bf16*>(v0 + 16 * ((col >> 3) ^ sw0) + cb));
        const i16x4 hi = lds_read_tr(reinterpret_cast<const bf16*>(v1 + 16 * ((col >> 3) ^ sw1) + cb));
        av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      st.oacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, st.pb[s], st.oacc[j], 0, 0, 0);
    }
  }
}

// Scheduling groups of an M phase that runs PV (NPV MFMAs, two transpose reads each) and then
// QK (NQK MFMAs, one 16-byte read each) as one region: before MFMA m the reads of MFMAs up to
// m + AHM have been issued, across the PV -> QK boundary.
template <int NPV>
constexpr int m_reads_upto(int m) {
  const int r = (m < NPV ? 2 * (m + 1) : 2 * NPV + (m + 1 - NPV)) - 2 * NPRE;
  return r > 0 ? r : 0;
}
template <int M_, int NPV, int NQK, int AHM, int ISSUED>
__device__ __forceinline__ void order_m_phase() {
  if constexpr (M_ < NPV + NQK) {
    constexpr int last = M_ + AHM < NPV + NQK - 1 ? M_ + AHM : NPV + NQK - 1;
    constexpr int want = m_reads_upto<NPV>(last);
    if constexpr (M_ < NPRE) {
      // the first MFMAs' operands are already in registers: they go first
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (want > ISSUED) __builtin_amdgcn_sched_group_barrier(0x100, want - ISSUED, 0);
    } else {
      if constexpr (want > ISSUED) __builtin_amdgcn_sched_group_barrier(0x100, want - ISSUED, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    order_m_phase<M_ + 1, NPV, NQK, AHM, (want > ISSUED ? want : ISSUED)>();
  }
}
// One M phase: PV of the previous tile, then QK of the current one, as one region.
template <int D>
__device__ __forceinline__ void phase_m(RowState<D>& st, const bf16x8 (&qf)[D / 16], const char* vbase, const char* kb,
                                        int v_row, int v_col, int l32, int hh, const bf16x8 (&av0)[NPRE]) {
  phase_pv<D>(st, vbase, v_row, v_col, av0);
  phase_qk<D>(st, qf, kb, l32, hh);
  order_m_phase<0, (BN / 16) * (D / 32), 2 * (D / 16), SVG_ATTN_M_AHEAD, 0>();
}


// bf16 P^T operands from the lane's 32 weights, and the row sums of those bf16 weights (the
// ones the PV product uses), two at a time (v_dot2_f32_bf16 against (1, 1)), in two chains
template <int D>
__device__ __forceinline__ float pack_weights(RowState<D>& st, const float (&p)[2][16]) {
#pragma unroll
  for (int s = 0; s < BN / 16; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) st.pb[s][e] = (bf16)p[s >> 1][8 * (s & 1) + e];
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
  for (int s = 0; s < BN / 16; ++s) {
    const bf16x8 q = st.pb[s];
    rs0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q, q, 0, 1), one, rs0, false);
    rs1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q, q, 2, 3), one, rs1, false);
    rs0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q, q, 4, 5), one, rs0, false);
    rs1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q, q, 6, 7), one, rs1, false);
  }
  return rs0 + rs1;
}

// Exact token mask (boundary tiles), online softmax, bf16 P^T operands.
//
// The weights are taken against a reference m_ref (log2 units) that only moves when it must.
// The first tile holding an allowed key of the row sets it to that tile's maximum score; after
// that the fast path exponentiates against the current reference and checks the lane's sum of
// the bf16 weights.  A sum of at most 2^8 means no weight exceeds 2^8 (and none overflowed);
// otherwise the slow path takes the tile's true maximum, moves the reference up to it
// (rescaling O and the sum) and exponentiates again.  So the reference always lies between
// the row's largest score so far minus 8 and that score, the bound the lazy rescaling of the
// running maximum gave, and a tile costs one compare on the sum instead of a 32-score
// maximum and its cross-lane exchange.
template <int D>
__device__ __forceinline__ void phase_softmax(RowState<D>& st, int32_t k0, bool edge, int32_t my_lo, int32_t my_hi,
                                              float c, int hh) {
  constexpr int NDB = D / 32;
  bool has_keys = true;
  if (edge) {
    // element (blk, r) holds key k0 + 4 hh + off, off = 32 blk + 8 (r >> 2) + (r & 3); the
    // lane's allowed offsets are [lo, hi).  Each bound costs a compare and a select per score,
    // and only where some lane of the wavefront needs it.
    const int32_t lo = my_lo - k0 - 4 * hh, hi = my_hi - k0 - 4 * hh;
    has_keys = lo < BN && hi > 0 && lo < hi;
    if (__any(lo > 0)) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int32_t off = blk * 32 + 8 * (r >> 2) + (r & 3);
          st.sacc[blk][r] = off < lo ? -INFINITY : st.sacc[blk][r];
        }
    }
    if (__any(hi < BN)) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int32_t off = blk * 32 + 8 * (r >> 2) + (r & 3);
          st.sacc[blk][r] = off >= hi ? -INFINITY : st.sacc[blk][r];
        }
    }
  }
  // x = scale * log2(e) * s - m_ref in place, then the exponentials: each exponential's input
  // was formed 32 instructions earlier, and the slow path recovers the scores from x
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.sacc[blk][r] = fmaf(st.sacc[blk][r], c, -st.m_ref);
  __builtin_amdgcn_sched_barrier(0);
  float p[2][16];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int r = 0; r < 16; ++r) p[blk][r] = __builtin_amdgcn_exp2f(st.sacc[blk][r]);
  float rs = pack_weights<D>(st, p);
  if (__any(!(rs <= 256.f) | (!st.m_set & has_keys))) {
    // the tile's largest x over both halves of the row (-inf: no allowed key)
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st.sacc[blk][r]);
    mx = max_halves(mx);
    // the first allowed key sets the reference; later it only moves up
    const bool set_now = !st.m_set && mx > -INFINITY;
    const float up = (mx > 0.f || set_now) ? mx : 0.f;
    const float alpha = st.m_set ? __builtin_amdgcn_exp2f(-up) : 0.f;
    st.l_run *= alpha;
#pragma unroll
    for (int j = 0; j < NDB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.oacc[j][r] *= alpha;
    st.m_ref += up;
    st.m_set = st.m_set || set_now;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) p[blk][r] = __builtin_amdgcn_exp2f(st.sacc[blk][r] - up);
    rs = pack_weights<D>(st, p);
  }
  st.l_run += rs;
}

// Workgroup barrier without a memory fence.  The only data one wavefront hands another
// through LDS here are the copied tiles, whose completion the issuing wavefronts wait for
// explicitly (vmcnt) before the barrier that publishes them; every LDS read is consumed by
// its own wavefront before that wavefront reaches the next barrier.  A fenced barrier would
// also wait for the copies just issued for the phase after next.  The empty asm statements
// keep the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void phase_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Row of the tensor in memory that holds row u of the head's working layout: u itself, or
// for a temporal head read in place (fused layout transformation) the frame-major row of
// token-major row u = p*F + f, namely f*P + p.
struct RowMap {
  FastDiv divF;
  int32_t F, P;
  bool tm;                     // u is token-major, memory is frame-major
  __device__ __forceinline__ int32_t operator()(int32_t u) const {
    if (!tm) return u;
    const int32_t p = (int32_t)fdiv((uint32_t)u, divF);
    return (u - p * F) * P + p;
  }
};

// Where a workgroup's rows and keys come from.  Rows are numbered in a logical order (the
// head's working layout, or a query cluster's sorted rows); each source maps a logical query
// or key to the row of the tensor that holds it, clamping past the end (such rows are masked or
// not stored; q_row_in takes rows below the row count), and gives each query's allowed keys
// (u below the row count) as one interval of logical key positions.
//
// BandSource: a head of the spatial/temporal path; keys are the same rows as queries and each
// query's interval follows from its band.
struct BandSource {
  static constexpr bool kGather = false;
  static constexpr bool kSkipDead = false;
  RowMap rmap;
  Band band;
  int32_t S;
  __device__ __forceinline__ int32_t q_row(int32_t u) const { return rmap(min(u, S - 1)); }
  __device__ __forceinline__ int32_t q_row_in(int32_t u) const { return rmap(u); }
  __device__ __forceinline__ int32_t kv_row(int32_t j) const { return rmap(min(j, S - 1)); }
  __device__ __forceinline__ void interval(int32_t u, int32_t& lo, int32_t& hi) const {
    band_interval(band, u, lo, hi);
  }
};
// ClusterSource: the rows of one query cluster (sorted positions -> tokens) against the key
// list of that cluster (the concatenated tokens of its selected key clusters), all of which
// every query attends to.  Key rows are read from the list, one phase ahead.
struct ClusterSource {
  static constexpr bool kGather = true;
  static constexpr bool kSkipDead = true;
  const int32_t* qp;           // tokens of the query cluster
  const int32_t* kl;           // its key list
  int32_t n, L;
  int32_t S;
  __device__ __forceinline__ int32_t q_row(int32_t u) const { return min(max(qp[min(u, n - 1)], 0), S - 1); }
  __device__ __forceinline__ int32_t q_row_in(int32_t u) const { return min(max(qp[u], 0), S - 1); }
  __device__ __forceinline__ int32_t kv_row(int32_t j) const { return kl[min(j, L - 1)]; }
  __device__ __forceinline__ void interval(int32_t, int32_t& lo, int32_t& hi) const {
    lo = 0;
    hi = L;
  }
};

// BlockSource: one 256-row query block in token order against the keys of its chosen 64-key
// blocks, every one of which its queries attend.  Blocks are listed in increasing order, so
// only the last may be the sequence's partial block: list position j is key 64 bl[j / 64] +
// j % 64.
struct BlockSource {
  static constexpr bool kGather = true;
  static constexpr bool kSkipDead = false;
  const int32_t* bl;           // chosen key blocks, increasing
  int32_t q0, n, L, S;
  __device__ __forceinline__ int32_t q_row(int32_t u) const { return q0 + min(u, n - 1); }
  __device__ __forceinline__ int32_t q_row_in(int32_t u) const { return q0 + u; }
  __device__ __forceinline__ int32_t kv_row(int32_t j) const {
    const int32_t jj = min(j, L - 1);
    return min(bl[jj >> 6] * 64 + (jj & 63), S - 1);
  }
  __device__ __forceinline__ void interval(int32_t, int32_t& lo, int32_t& hi) const {
    lo = 0;
    hi = L;
  }
};

// Copy of one K or V tile into LDS by the four wavefronts of one group (wb = 0..3): per
// wavefront, PER_WAVE instructions of 1 KB each.  The address is the wavefront-uniform head
// base plus a 32-bit per-lane offset (the host checks that a head fits in 4 GB).  Every lane
// copies 16 bytes of one row, so the rows of a tile may come from anywhere: row_of(i, r) is the
// tensor row that instruction i of this lane reads for tile row r.
template <int D>
struct CopyPlan {
  static constexpr int PER_WAVE = TileLds<D>::TILE_BYTES / 1024 / 4;
  static constexpr int RPI = 1024 / TileLds<D>::ROW_BYTES;    // tile rows per instruction
};

template <int D, class RowOf>
__device__ __forceinline__ void pp_load(const bf16* __restrict__ src, bf16* dst, int wb, int lane, bool is_v,
                                        RowOf row_of) {
  using T = TileLds<D>;
  using CP = CopyPlan<D>;
  const int pc = lane % T::CPR;
#pragma unroll
  for (int i = 0; i < CP::PER_WAVE; ++i) {
    const int kb = (wb * CP::PER_WAVE + i) * 1024;
    const int row = (wb * CP::PER_WAVE + i) * CP::RPI + lane / T::CPR;
    const int lc = pc ^ (is_v ? T::swz_v(row) : T::swz_k(row));
    const uint32_t boff = (uint32_t)row_of(i, row) * (uint32_t)T::ROW_BYTES + 16u * (uint32_t)lc;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(src) + boff,
                                     (__attribute__((address_space(3))) void*)((char*)dst + kb), 16, 0, 0);
  }
}

// Tensor rows of the tile at logical key k0 that this lane copies, read ahead of the copy.
template <int D, class Src>
__device__ __forceinline__ void tile_rows(const Src& src, int32_t k0, int wb, int lane,
                                          int32_t (&prow)[CopyPlan<D>::PER_WAVE]) {
  using CP = CopyPlan<D>;
#pragma unroll
  for (int i = 0; i < CP::PER_WAVE; ++i)
    prow[i] = src.kv_row(k0 + (wb * CP::PER_WAVE + i) * CP::RPI + lane / TileLds<D>::CPR);
}

// The ping-pong loop of one workgroup: 256 logical query rows from q0 (rows at or past n_rows
// are computed on clamped inputs and not stored).
// With LSE, each stored row also gets its natural-log log-sum-exp, from the running max and
// the row sum of the bf16 weights: ln 2 * (m + log2 l), m the max in log2 units of the scaled
// logits.
template <int D, class Src, bool LSE = false>
__device__ __forceinline__ void pp_attention(const Src& src, const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                             const bf16* __restrict__ V, bf16* __restrict__ O, int32_t n_rows,
                                             int32_t q0, float scale, float* __restrict__ lse = nullptr) {
  constexpr int NDB = D / 32;
  constexpr int NKS = D / 16;
  constexpr int PW = CopyPlan<D>::PER_WAVE;
  __shared__ __attribute__((aligned(1024))) bf16 K0[BN * D];
  __shared__ __attribute__((aligned(1024))) bf16 K1[BN * D];
  __shared__ __attribute__((aligned(1024))) bf16 Vb[3][BN * D];     // V(t_j) in Vb[j % 3]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // wavefronts w and w+4 share a SIMD, so the groups are wavefronts 0-3 and 4-7
  const int grp = wave >> 2;                 // 0: group A, 1: group B
  const int wig = __builtin_amdgcn_readfirstlane(wave & 3);   // wavefront within its group
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // tiles of the whole workgroup (union of both groups' ranges)
  const int32_t q_last = min(q0 + PP_BM, n_rows) - 1;
  int32_t lo0, hi0, lo1, hi1;
  src.interval(q0, lo0, hi0);
  src.interval(q_last, lo1, hi1);
  const int32_t t_begin = lo0 / BN;
  const int32_t T = (hi1 + BN - 1) / BN - t_begin;

  // this group's rows and tiles
  const int32_t g0 = q0 + grp * (PP_BM / 2);
  const bool g_live = g0 < n_rows;
  const int32_t g1 = min(g0 + PP_BM / 2, n_rows) - 1;
  int32_t glo_first = 0, ghi_first = 0, glo_last = 0, ghi_last = 0;
  if (g_live) {
    src.interval(g0, glo_first, ghi_first);
    src.interval(g1, glo_last, ghi_last);
  }

  const int32_t my_q = g0 + wig * 32 + l32;
  int32_t my_lo, my_hi;
  src.interval(min(my_q, n_rows - 1), my_lo, my_hi);

  // first tiles: K(t_0) by group A, V(t_0) by group B
  {
    const int32_t k0 = t_begin * BN;
    auto rows = [&](int, int r) { return src.kv_row(k0 + r); };
    if (grp == 0) pp_load<D>(K, K0, wig, lane, false, rows);
    else pp_load<D>(V, Vb[0], wig, lane, true, rows);
  }
  // gathered key rows of the copy that follows this group's next matrix phase
  int32_t nrow[PW];
  if constexpr (Src::kGather) tile_rows<D>(src, (t_begin + 1) * BN, wig, lane, nrow);
  bf16x8 qf[NKS];
  {
    const bf16* qrow = Q + (size_t)src.q_row(my_q) * D;
#pragma unroll
    for (int s = 0; s < NKS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * hh);
  }

  RowState<D> st;
#pragma unroll
  for (int j = 0; j < NDB; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.oacc[j][r] = 0.f;
#pragma unroll
  for (int s = 0; s < BN / 16; ++s) st.pb[s] = bf16x8{};
  st.m_ref = 0.f;
  st.m_set = false;
  st.l_run = 0.f;
  // M(0) reads V(t_{-1}) from Vb[2] with P^T = 0: zero it so that the product is exactly zero
  for (int o = tid; o < BN * D / 8; o += PP_NT) reinterpret_cast<u32x4*>(Vb[2])[o] = u32x4{0u, 0u, 0u, 0u};
  const float c = scale * 1.44269504088896340736f;
  const int tg = lane >> 4;
  const int ti = lane & 15;
  const int v_row = 4 * (tg >> 1) + (ti >> 2);
  const int v_col = 16 * (tg & 1) + 4 * (ti & 3);

  // everything loaded so far retires before the phase loop (see the note on counters above)
  __builtin_amdgcn_s_waitcnt(ALLCNT0);
  __syncthreads();

  // edge(i): tile t_begin+i needs the element mask for some row of this group -- a boundary
  // tile, or one outside the group's range (also any tile of a group with no rows)
  auto edge = [&](int32_t i) {
    const int32_t k0 = (t_begin + i) * BN;
    return !(g_live && k0 >= glo_last && k0 + BN <= ghi_first);
  };
  // M(i): PV(i-1) reads vprev, QK(i) reads kcur.  M(0) adds P^T = 0 times the zeroed V buffer;
  // the scores of the tile past the end (stale K buffer) are masked away by X(T).
  bf16x8 av0[NPRE];
#pragma unroll
  for (int j = 0; j < NPRE; ++j) av0[j] = read_vt0<D>(reinterpret_cast<const char*>(Vb[2]), v_row, v_col, j);
  // A group with no rows (the last 256-row tile of a query cluster often holds 128 rows or
  // fewer) skips its products and exponentials, but still copies, waits and meets every
  // barrier: the other group's phases then run alone on the SIMDs.  Only the cluster kernel
  // does this (2.7% faster at 720p).  In the band and block-list kernels, where a dead group
  // is rare, the branch changed the register allocation and cost 1.3% and 1.2%.
  constexpr bool skip_dead = Src::kSkipDead;
  auto do_m = [&](const bf16* vprev, const bf16* kcur) {
    __builtin_amdgcn_s_waitcnt(VMCNT0);
    if (!skip_dead || g_live)
      phase_m<D>(st, qf, reinterpret_cast<const char*>(vprev), reinterpret_cast<const char*>(kcur), v_row, v_col,
                 l32, hh, av0);
  };
  // after a group's vector phase X(i) and its copies: the first V^T operand of its next matrix
  // phase, and (gathered keys) the rows of the copy that follows that phase, tile i + 2
  auto pre = [&](const bf16* vnext) {
#pragma unroll
    for (int j = 0; j < NPRE; ++j) av0[j] = read_vt0<D>(reinterpret_cast<const char*>(vnext), v_row, v_col, j);
  };
  auto do_x = [&](int32_t i) {
    __builtin_amdgcn_s_setprio(0);
    if (!skip_dead || g_live) phase_softmax<D>(st, (t_begin + i) * BN, edge(i), my_lo, my_hi, c, hh);
    if constexpr (Src::kGather) tile_rows<D>(src, (t_begin + i + 2) * BN, wig, lane, nrow);
    __builtin_amdgcn_s_setprio(2);
  };
  // copies after M(j): group A K(t_{j+1}) -> kdst, group B V(t_{j+1}) -> Vb[(j+1) % 3]
  auto rows_of = [&](int32_t j) {
    const int32_t k0 = (t_begin + j + 1) * BN;
    return [&, k0](int i, int r) {
      if constexpr (Src::kGather) {
        (void)k0;
        return nrow[i];
      } else {
        return src.kv_row(k0 + r);
      }
    };
  };
  // The copies of tile t_{j+1} are issued at the start of the issuing group's vector phase
  // X(j), the phase after its M(j): group A copies K into the K buffer M(j-1) read, group B
  // copies V into the V buffer of V(t_{j-2}), which PV(j-2) read in M(j-1).
  auto copy_k = [&](int32_t j, bf16* kdst) {
    if (j >= 0 && j + 1 < T) pp_load<D>(K, kdst, wig, lane, false, rows_of(j));
  };
  auto copy_v = [&](int32_t j) {
    if (j >= 0 && j + 1 < T) pp_load<D>(V, Vb[(j + 1) % 3], wig, lane, true, rows_of(j));
  };
  auto vbuf = [&](int32_t j) { return Vb[(j + 3) % 3]; };   // V(t_j), j >= -1

  // At D = 64 the vector phase is the longer of the two, so the copies go to the end of the
  // issuing group's matrix phase M(j) instead (the buffers they fill are free from then on;
  // they retire at the end of X(j) all the same): 3.5% faster on the CogVideoX-like grid,
  // while at D = 128 the start of X(j) measured 1% faster than the end of M(j).
  constexpr bool after_m = D == 64;
  const int32_t n_phase = 2 * T + 2;
  for (int32_t m = 0;; ++m) {
    // phase 4m: A: M(2m) [V(2m-1), K0]; B: copies V(t_{2m}), X(2m-1), its copies retire
    if (grp == 0) {
      do_m(vbuf(2 * m - 1), K0);
      if constexpr (after_m) copy_k(2 * m, K1);
    } else {
      if constexpr (!after_m) copy_v(2 * m - 1);
      do_x(2 * m - 1);
      __builtin_amdgcn_s_waitcnt(VMCNT0);
      pre(vbuf(2 * m - 1));
    }
    phase_barrier();
    if (4 * m + 1 >= n_phase) break;
    // phase 4m+1: A: copies K(t_{2m+1}) -> K1, X(2m), its copies retire; B: M(2m) [V(2m-1), K0]
    if (grp == 0) {
      if constexpr (!after_m) copy_k(2 * m, K1);
      do_x(2 * m);
      __builtin_amdgcn_s_waitcnt(VMCNT0);
      pre(vbuf(2 * m));
    } else {
      do_m(vbuf(2 * m - 1), K0);
      if constexpr (after_m) copy_v(2 * m);
    }
    phase_barrier();
    if (4 * m + 2 >= n_phase) break;
    // phase 4m+2: A: M(2m+1) [V(2m), K1]; B: copies V(t_{2m+1}), X(2m), its copies retire
    if (grp == 0) {
      do_m(vbuf(2 * m), K1);
      if constexpr (after_m) copy_k(2 * m + 1, K0);
    } else {
      if constexpr (!after_m) copy_v(2 * m);
      do_x(2 * m);
      __builtin_amdgcn_s_waitcnt(VMCNT0);
      pre(vbuf(2 * m));
    }
    phase_barrier();
    if (4 * m + 3 >= n_phase) break;
    // phase 4m+3: A: copies K(t_{2m+2}) -> K0, X(2m+1), its copies retire; B: M(2m+1) [V(2m), K1]
    if (grp == 0) {
      if constexpr (!after_m) copy_k(2 * m + 1, K0);
      do_x(2 * m + 1);
      __builtin_amdgcn_s_waitcnt(VMCNT0);
      pre(vbuf(2 * m + 1));
    } else {
      do_m(vbuf(2 * m), K1);
      if constexpr (after_m) copy_v(2 * m + 1);
    }
    phase_barrier();
    if (4 * m + 4 >= n_phase) break;
  }

  // ---- epilogue: divide by the row sum, round to bf16, store this lane's query row ----
  if (my_q < n_rows) {
    const float l_tot = st.l_run + other_half(st.l_run);
    const float inv = 1.f / l_tot;
    bf16* orow = O + (size_t)src.q_row_in(my_q) * D;
#pragma unroll
    for (int j = 0; j < NDB; ++j)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (bf16)(st.oacc[j][4 * rq + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * j + 8 * rq + 4 * hh) = ov;
      }
    if constexpr (LSE) {
      if (hh == 0) lse[src.q_row_in(my_q)] = 0.69314718055994531f * (st.m_ref + __log2f(l_tot));
    }
  }
}

template <int D>
__device__ __forceinline__ void band_item(const AttnArgs& a, int32_t nqb, int32_t item) {
  const int32_t rank = item / nqb;
  const int32_t qb = item - rank * nqb;
  const int32_t bh = a.order ? a.order[rank] : rank;
  int kind = (a.force_dense || a.kind == nullptr) ? KIND_DENSE : (int)a.kind[bh];
  if (kind != KIND_SPATIAL && kind != KIND_TEMPORAL) kind = KIND_DENSE;
  const bool tmaj = kind == KIND_TEMPORAL;
  // temporal heads work in token-major order; they read token-major copies (qt, kt, vt -> ot)
  // or, fused, the frame-major tensors through the row map
  const bool own_t = tmaj && !a.fused_t;
  const size_t off = (size_t)bh * (size_t)a.S * D;
  BandSource src;
  src.rmap.divF = a.divF;
  src.rmap.F = a.F;
  src.rmap.P = a.P;
  src.rmap.tm = tmaj && a.fused_t;
  src.S = a.S;
  src.band.S = a.S;
  src.band.dense = kind == KIND_DENSE;
  if (tmaj) { src.band.divG = a.divF; src.band.G = a.F; src.band.NG = a.P; src.band.w = a.w_p; }
  else { src.band.divG = a.divP; src.band.G = a.P; src.band.NG = a.F; src.band.w = a.w_f; }
  pp_attention<D>(src, (own_t ? a.qt : a.q) + off, (own_t ? a.kt : a.k) + off, (own_t ? a.vt : a.v) + off,
                  (own_t ? a.ot : a.o) + off, a.S, qb * PP_BM, a.scale);
}

template <int D>
__global__ __launch_bounds__(PP_NT, 1) void attn_fwd_kernel(AttnArgs a, int32_t nqb) {
  band_item<D>(a, nqb, xcd_item((int32_t)blockIdx.x, (int32_t)gridDim.x));
}

// Up to this many band items (256 query rows each) per CU the persistent grid below is used:
// with few items per CU the per-XCD queue evens out the tail (Wan 480p, 20 items per CU: 3-6%
// faster; CogVideoX, 13 per CU: 1-5%), while with more (HunyuanVideo 720p, 44 per CU) the
// one-item grid measured 1% faster.
constexpr int32_t PERSIST_MAX_ITEMS_PER_CU = 32;

// The same work with one workgroup per CU that takes items until none are left.  Workgroup w
// runs on XCD w % 8 (workgroups reach the XCDs round-robin) and takes the items the one-item
// kernel would have given that XCD, in the same order, from a per-XCD counter: the k-th item
// of XCD x is xcd_item(8 k + x).  The next item's index is fetched while the current one runs.
template <int D>
__global__ __launch_bounds__(PP_NT, 1) void attn_fwd_persistent_kernel(AttnArgs a, int32_t nqb, int32_t n_items) {
  __shared__ int32_t next_b;
  const int32_t x = (int32_t)blockIdx.x % NXCD;
  if (threadIdx.x == 0) next_b = atomicAdd(&a.queue[x], 1) * NXCD + x;
  __syncthreads();
  int32_t b = next_b;
  while (b < n_items) {
    __syncthreads();                     // every thread has read next_b
    if (threadIdx.x == 0) next_b = atomicAdd(&a.queue[x], 1) * NXCD + x;
    band_item<D>(a, nqb, xcd_item(b, n_items));
    __syncthreads();
    b = next_b;
  }
}

// One workgroup per (head, query cluster, 256-row tile of that cluster); unused item slots of a
// head (-1) exit at once.
template <int D>
__global__ __launch_bounds__(PP_NT, 1) void cluster_attn_kernel(ClusterAttnArgs a) {
  const int32_t item = xcd_item((int32_t)blockIdx.x, (int32_t)gridDim.x);
  const int32_t bh = item / a.items_per_head;
  const int32_t code = a.items[item];
  if (code < 0) return;
  const int32_t qc = code >> 16, qt = code & 0xFFFF;
  const int32_t* qoff = a.q_off + (size_t)bh * (a.Cq + 1);
  // (offsets and list lengths are clamped into range: inconsistent inputs cannot address
  // memory outside the buffers; the key lists hold in-range rows)
  const int32_t qbeg = min(max(qoff[qc], 0), a.S);
  ClusterSource src;
  src.S = a.S;
  src.n = min(max(qoff[qc + 1] - qbeg, 0), a.S - qbeg);
  src.L = min(max(a.klen[(size_t)bh * a.Cq + qc], 0), a.S);
  if (src.n == 0 || src.L == 0) return;
  src.qp = a.q_perm + (size_t)bh * a.S + qbeg;
  src.kl = a.klist + ((size_t)bh * a.Cq + qc) * a.S;
  const size_t off = (size_t)bh * (size_t)a.S * D;
  pp_attention<D>(src, a.q + off, a.k + off, a.v + off, a.o + off, src.n, qt * PP_BM, a.scale);
}

// Dense attention that also writes every row's log-sum-exp.
template <int D>
__global__ __launch_bounds__(PP_NT, 1) void attn_lse_kernel(AttnArgs a, int32_t nqb) {
  const int32_t item = xcd_item((int32_t)blockIdx.x, (int32_t)gridDim.x);
  const int32_t bh = item / nqb;
  const int32_t qb = item - bh * nqb;
  const size_t off = (size_t)bh * (size_t)a.S * D;
  BandSource src;
  src.rmap.divF = a.divF;
  src.rmap.F = a.F;
  src.rmap.P = a.P;
  src.rmap.tm = false;
  src.S = a.S;
  src.band.S = a.S;
  src.band.dense = 1;
  src.band.divG = a.divP;
  src.band.G = a.P;
  src.band.NG = a.F;
  src.band.w = 0;
  pp_attention<D, BandSource, true>(src, a.q + off, a.k + off, a.v + off, a.o + off, a.S, qb * PP_BM, a.scale,
                                    a.lse + (size_t)bh * a.S);
}

// One workgroup per (head, 256-row query block): attention over the block's chosen key blocks.
template <int D>
__global__ __launch_bounds__(PP_NT, 1) void block_attn_kernel(BlockAttnArgs a) {
  const int32_t item = xcd_item((int32_t)blockIdx.x, (int32_t)gridDim.x);
  const int32_t bh = item / a.nqb;
  const int32_t qb = item - bh * a.nqb;
  BlockSource src;
  src.S = a.S;
  src.q0 = qb * PP_BM;
  src.n = min(PP_BM, a.S - src.q0);
  src.L = min(max(a.blen[item], 0), a.S);
  if (src.L == 0) return;
  src.bl = a.blist + (size_t)item * a.nkb;
  const size_t off = (size_t)bh * (size_t)a.S * D;
  pp_attention<D>(src, a.q + off, a.k + off, a.v + off, a.o + off, src.n, 0, a.scale);
}

// Explicit instantiations, so that the host pass emits every launch stub the launchers use.
template __global__ void attn_fwd_kernel<128>(AttnArgs, int32_t);
template __global__ void attn_fwd_kernel<64>(AttnArgs, int32_t);
template __global__ void attn_fwd_persistent_kernel<128>(AttnArgs, int32_t, int32_t);
template __global__ void attn_fwd_persistent_kernel<64>(AttnArgs, int32_t, int32_t);
template __global__ void cluster_attn_kernel<128>(ClusterAttnArgs);
template __global__ void cluster_attn_kernel<64>(ClusterAttnArgs);
template __global__ void attn_lse_kernel<128>(AttnArgs, int32_t);
template __global__ void attn_lse_kernel<64>(AttnArgs, int32_t);
template __global__ void block_attn_kernel<128>(BlockAttnArgs);
template __global__ void block_attn_kernel<64>(BlockAttnArgs);

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  const int32_t nqb = (a.S + PP_BM - 1) / PP_BM;
  if (a.order != nullptr && a.kind != nullptr && !a.force_dense) {
    head_order_kernel<<<1, 64, 0, st>>>(a.kind, a.order, a.BH, a.queue);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  AttnArgs b = a;
  if (a.kind == nullptr || a.force_dense) b.order = nullptr;
  const int32_t n_items = (int32_t)((int64_t)nqb * a.BH);
  if (b.order != nullptr && b.queue != nullptr) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if ((int64_t)n_items <= (int64_t)PERSIST_MAX_ITEMS_PER_CU * cus) {
      // at least one workgroup per XCD residue, so that every per-XCD counter is drained
      int32_t g = cus < n_items ? cus : n_items;
      if (g < NXCD) g = n_items < NXCD ? n_items : NXCD;
      const dim3 pgrid((unsigned)g);
      if (a.D == 128) attn_fwd_persistent_kernel<128><<<pgrid, PP_NT, 0, st>>>(b, nqb, n_items);
      else if (a.D == 64) attn_fwd_persistent_kernel<64><<<pgrid, PP_NT, 0, st>>>(b, nqb, n_items);
      else return hipErrorInvalidValue;
      return hipGetLastError();
    }
  }
  const dim3 grid((unsigned)n_items);
  if (a.D == 128) {
    attn_fwd_kernel<128><<<grid, PP_NT, 0, st>>>(b, nqb);
  } else if (a.D == 64) {
    attn_fwd_kernel<64><<<grid, PP_NT, 0, st>>>(b, nqb);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_cluster_attention(const ClusterAttnArgs& a, hipStream_t st) {
  static_assert(CLUSTER_TILE_ROWS == PP_BM, "cluster work items are attention workgroups");
  const dim3 grid((unsigned)((int64_t)a.items_per_head * a.BH));
  if (a.D == 128) {
    cluster_attn_kernel<128><<<grid, PP_NT, 0, st>>>(a);
  } else if (a.D == 64) {
    cluster_attn_kernel<64><<<grid, PP_NT, 0, st>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention_lse(const AttnArgs& a, hipStream_t st) {
  const int32_t nqb = (a.S + PP_BM - 1) / PP_BM;
  const dim3 grid((unsigned)((int64_t)nqb * a.BH));
  if (a.D == 128) {
    attn_lse_kernel<128><<<grid, PP_NT, 0, st>>>(a, nqb);
  } else if (a.D == 64) {
    attn_lse_kernel<64><<<grid, PP_NT, 0, st>>>(a, nqb);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_block_attention(const BlockAttnArgs& a, hipStream_t st) {
  static_assert(BLOCK_Q_ROWS == PP_BM && BLOCK_K_ROWS == BN, "search blocks are the attention kernel's tiles");
  const dim3 grid((unsigned)((int64_t)a.nqb * a.BH));
  if (a.D == 128) {
    block_attn_kernel<128><<<grid, PP_NT, 0, st>>>(a);
  } else if (a.D == 64) {
    block_attn_kernel<64><<<grid, PP_NT, 0, st>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace svg
