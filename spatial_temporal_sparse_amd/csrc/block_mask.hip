// Tile mask of each head's score matrix in the head's working layout.  A spatial head's
// map is a block band around the diagonal and a temporal head's map is a set of slash
// lines with the frame size as stride (Sparse VideoGen authors' article, sections "Spatial
// Head" and "Temporal Head"); after the layout transformation the latter is a block band
// too.  Every row's allowed keys form one interval whose ends grow with the row, so the
// union over a query block is the interval [lo(first row), hi(last row)) and a tile is
// needed exactly when it meets that interval.
#include "svg_internal.h"

namespace svg {

namespace {

__global__ __launch_bounds__(256) void block_mask_kernel(BlockMaskArgs a) {
  const size_t total = (size_t)a.BH * a.nqb * a.nkb;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const int32_t j = (int32_t)(e % a.nkb);
    const size_t rest = e / a.nkb;
    const int32_t i = (int32_t)(rest % a.nqb);
    const int32_t bh = (int32_t)(rest / a.nqb);
    int kind = a.kind ? (int)a.kind[bh] : KIND_DENSE;
    Band b;
    b.S = a.S;
    b.dense = (kind != KIND_SPATIAL && kind != KIND_TEMPORAL);
    if (kind == KIND_SPATIAL) {
      b.divG = a.divP; b.G = a.P; b.NG = a.F; b.w = a.w_f;
    } else {
      b.divG = a.divF; b.G = a.F; b.NG = a.P; b.w = a.w_p;
    }
    const int32_t r0 = i * a.bm;
    const int32_t r1 = min(a.S, r0 + a.bm) - 1;
    int32_t lo0, hi0, lo1, hi1;
    band_interval(b, r0, lo0, hi0);
    band_interval(b, r1, lo1, hi1);
    const int32_t k0 = j * a.bn;
    const int32_t k1 = min(a.S, k0 + a.bn);   // tile keys [k0, k1)
    a.out[e] = (uint8_t)(k0 < hi1 && k1 > lo0);
  }
}

}  // namespace

hipError_t launch_block_mask(const BlockMaskArgs& a, hipStream_t st) {
  const size_t total = (size_t)a.BH * a.nqb * a.nkb;
  size_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) blocks = 1;
  block_mask_kernel<<<dim3((unsigned)blocks), 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace svg
