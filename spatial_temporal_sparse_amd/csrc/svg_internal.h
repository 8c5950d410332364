// Internal declarations shared by the HIP kernels and the C-ABI layer of libsvg.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace svg {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 16-byte move unit

// s_waitcnt immediate (gfx9 encoding) that waits for every outstanding vector-memory load
// and for nothing else: vmcnt = 0, expcnt = 7, lgkmcnt = 15.
constexpr int VMCNT0 = 0x0F70;
// ... and that also waits for every outstanding LDS / scalar-memory operation (lgkmcnt = 0).
constexpr int ALLCNT0 = 0x0070;

constexpr int KIND_SPATIAL = 0;
constexpr int KIND_TEMPORAL = 1;
constexpr int KIND_DENSE = 2;

// Exact unsigned division n / d for 0 <= n < 2^31 and 1 <= d < 2^31 by multiply-high
// (Granlund & Montgomery, "Division by invariant integers using multiplication", 1994):
// with s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1, n / d = (mulhi(n, m) + n) >> s.
struct FastDiv {
  uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.s = s;
  f.m = (uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1);
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}
__device__ __forceinline__ uint32_t fmod_(uint32_t n, const FastDiv& f) {
  return n - fdiv(n, f) * f.d;
}

// The token mask of a head, in the head's working layout, is a band of groups: row r
// belongs to group r / G and may attend keys of groups within +-w of it, of NG groups of
// G tokens.  Spatial heads (frame-major): G = P, NG = F, w = w_f.  Temporal heads
// (token-major): G = F, NG = P, w = w_p.  Each row's allowed keys therefore form one
// contiguous interval [lo, hi) whose ends are non-decreasing in r.
struct Band {
  FastDiv divG;
  int32_t G, NG, w;
  int32_t dense;   // 1: every key of [0, S)
  int32_t S;
};

__device__ __forceinline__ void band_interval(const Band& b, int32_t r, int32_t& lo, int32_t& hi) {
  if (b.dense) {
    lo = 0;
    hi = b.S;
    return;
  }
  const int32_t grp = (int32_t)fdiv((uint32_t)r, b.divG);
  lo = max(0, grp - b.w) * b.G;
  hi = min(b.NG, grp + b.w + 1) * b.G;
}

// ------------------------------------------------------------------------------------------
// LDS transpose read (ds_read_b64_tr_b16) used by the attention and profiling kernels.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ i16x4 lds_read_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// ------------------------------------------------------------------------------------------
// Launchers (one per kernel family); each returns hipGetLastError() after enqueueing.
// ------------------------------------------------------------------------------------------
struct PermuteArgs {
  const void* src;
  void* dst;
  const uint8_t* kind;   // may be null: every head
  int32_t select;
  int32_t BH, S;
  int32_t row_bytes;     // D * elem_bytes, a multiple of 16
  // dst row r <- src row (r mod A) * Bm + r div A
  FastDiv divA;
  int32_t Bm;
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t st);

struct BlockMaskArgs {
  const uint8_t* kind;
  uint8_t* out;
  int32_t BH, S, F, P, w_f, w_p, bm, bn, nqb, nkb;
  FastDiv divP, divF;
};
hipError_t launch_block_mask(const BlockMaskArgs& a, hipStream_t st);

struct RopeArgs {
  const bf16* in[2];
  bf16* out[2];
  const float* w[2];
  float eps;
  double base;
  int32_t BH, S, F, HH, WW, P, D, dt, dh, dw;
  FastDiv divS, divP, divWW;
};
hipError_t launch_qknorm_rope(const RopeArgs& a, hipStream_t st);

struct AttnArgs {
  const bf16 *q, *k, *v;      // frame-major
  const bf16 *qt, *kt, *vt;   // token-major
  bf16 *o, *ot;
  const uint8_t* kind;        // null: all dense
  int32_t* order;             // [BH] head order scratch (null: identity, no kind)
  int32_t* queue;             // [8] per-XCD work counters of the persistent kernel (null: none)
  int32_t BH, S, F, P, D, w_f, w_p;
  FastDiv divP, divF;
  float scale;
  int32_t force_dense;
  int32_t fused_t;            // temporal heads read q/k/v and write o through the permutation
  float* lse;                 // [BH][S] log-sum-exp of each row (launch_attention_lse only)
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t st);
hipError_t launch_attention_lse(const AttnArgs& a, hipStream_t st);   // dense, with lse

struct ProfileArgs {
  const bf16 *q, *k, *v;
  const int32_t* idx;
  int32_t n_q, n_zq;          // sampled rows; groups of 64 rows
  int32_t BH, S, F, P, D, w_f, w_p;
  FastDiv divP;
  float scale;
  int32_t nsplit;             // key splits: split s holds key tiles s, s + nsplit, ...
  float* part_ml;             // [BH][nsplit][3][n_zq*64][2]
  float* part_o;              // [BH][nsplit][3][n_zq*64][D]
  double* row_sq;             // [BH][n_q][2] squared errors of each sampled row
  float* mse;                 // [BH][2]
  uint8_t* kind;              // [BH]
};
hipError_t launch_profile(const ProfileArgs& a, hipStream_t st);

// Split-K plan of the profiling kernel, shared by the launcher and the workspace query.
struct ProfilePlan {
  int32_t n_zq, nsplit;
  size_t ml_floats, o_floats, sq_doubles;
};
ProfilePlan profile_plan(int32_t BH, int32_t S, int32_t D, int32_t n_q);

// ------------------------------------------------------------------------------------------
// Semantic clustering path
// ------------------------------------------------------------------------------------------
struct KmeansArgs {
  const bf16* x;              // [BH][S][D] rows to cluster
  const int32_t* init_idx;    // [C] cold-start token indices, or null: start from cent
  float* cent;                // [BH][C][D] centroids, in and out
  int32_t* labels;            // [BH][S] cluster of each row (last assignment)
  int32_t* perm;              // [BH][S] tokens sorted by cluster (stable)
  int32_t* offsets;           // [BH][C+1] first sorted position of each cluster
  bf16* cb;                   // workspace [BH][Cpad][D] bf16 centroids
  float* hn;                  // workspace [BH][Cpad] half squared norms
  int32_t* counts;            // workspace [BH][nchunk][C]
  int32_t BH, S, D, C, iters;
};
int32_t kmeans_cpad(int32_t C);
int32_t cluster_nchunk(int32_t S);
hipError_t launch_kmeans(const KmeansArgs& a, hipStream_t st);

struct ToppArgs {
  const float *cq, *ck;       // [BH][Cq][D], [BH][Ck][D]
  const int32_t* k_off;       // [BH][Ck+1]
  uint8_t* sel;               // [BH][Cq][Ck]
  int32_t BH, Cq, Ck, D;
  double scale, p;
};
constexpr int TOPP_MAX_CK = 1024;
hipError_t launch_centroid_topp(const ToppArgs& a, hipStream_t st);

// Query rows of one attention workgroup in the clustering path (one query cluster's rows).
constexpr int CLUSTER_TILE_ROWS = 256;
inline int32_t cluster_items_per_head(int32_t S, int32_t Cq) {
  return (S + CLUSTER_TILE_ROWS - 1) / CLUSTER_TILE_ROWS + Cq;
}

struct ClusterListArgs {
  const uint8_t* sel;
  const int32_t *k_perm, *k_off, *q_off;
  int32_t* klist;             // [BH][Cq][S] token rows of each query cluster's keys
  int32_t* klen;              // [BH][Cq]
  int32_t* items;             // [BH][items_per_head]
  int32_t BH, S, Cq, Ck, items_per_head, tile_rows;
};
hipError_t launch_cluster_lists(const ClusterListArgs& a, hipStream_t st);

struct ClusterAttnArgs {
  const bf16 *q, *k, *v;
  bf16* o;
  const int32_t *q_perm, *q_off, *klist, *klen, *items;
  int32_t BH, S, D, Cq, items_per_head;
  float scale;
};
hipError_t launch_cluster_attention(const ClusterAttnArgs& a, hipStream_t st);

// ------------------------------------------------------------------------------------------
// Block-sparse path with an LSE-cached block search
// ------------------------------------------------------------------------------------------
constexpr int BLOCK_Q_ROWS = 256;   // query rows of a search block (an attention workgroup)
constexpr int BLOCK_K_ROWS = 64;    // keys of a search block (an attention key tile)
constexpr int BLOCK_MAX_NKB = 4096; // key blocks per row that the selection sorts in LDS

struct BlockMassArgs {
  const bf16 *q, *k;
  const float* lse;           // [BH][S]
  float* mass;                // [BH][nqb][nkb]
  int32_t BH, S, D, nqb, nkb;
  float scale;
};
hipError_t launch_block_mass(const BlockMassArgs& a, hipStream_t st);

struct BlockSelectArgs {
  const float* mass;          // [BH][nqb][nkb]
  uint8_t* sel;               // [BH][nqb][nkb]
  int32_t BH, nqb, nkb;
  double coverage;
};
hipError_t launch_block_select(const BlockSelectArgs& a, hipStream_t st);

struct BlockAttnArgs {
  const bf16 *q, *k, *v;
  bf16* o;
  const uint8_t* sel;         // [BH][nqb][nkb]
  int32_t* blist;             // workspace [BH][nqb][nkb]: chosen key blocks, increasing
  int32_t* blen;              // workspace [BH][nqb]: keys of those blocks
  int32_t BH, S, D, nqb, nkb;
  float scale;
};
hipError_t launch_block_lists(const BlockAttnArgs& a, hipStream_t st);
hipError_t launch_block_attention(const BlockAttnArgs& a, hipStream_t st);

constexpr int ATTN_BM = 128;
constexpr int ATTN_BN = 64;

}  // namespace svg
