// C ABI of libsvg: argument checks, workspace sizing and kernel launches.  Every argument
// is validated on the host before anything is enqueued; HIP launch errors map to
// SVG_ERR_HIP.  Nothing here allocates device memory or synchronises the host.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/svg.h"
#include "svg_internal.h"

#define SVG_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

svg_status fail(svg_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

svg_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SVG_OK;
  return fail(SVG_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Geometry checks shared by every call.  `need_d` requires D in {64, 128}.
svg_status check_geom(const svg_geom& g, bool need_d) {
  if (g.B <= 0 || g.H <= 0 || g.F <= 0 || g.HH <= 0 || g.WW <= 0 || g.D <= 0)
    return fail(SVG_ERR_INVALID, "geometry fields must be > 0 (B=%d H=%d F=%d HH=%d WW=%d D=%d)", g.B, g.H, g.F, g.HH,
                g.WW, g.D);
  const int64_t P = (int64_t)g.HH * g.WW;
  const int64_t S = P * g.F;
  if (S >= (int64_t)1 << 30) return fail(SVG_ERR_INVALID, "S = F*HH*WW = %lld is too large", (long long)S);
  const int64_t BH = (int64_t)g.B * g.H;
  if (BH >= (int64_t)1 << 24) return fail(SVG_ERR_INVALID, "B*H = %lld is too large", (long long)BH);
  if (BH * S >= (int64_t)1 << 31)
    return fail(SVG_ERR_INVALID, "B*H*S = %lld rows exceeds 2^31", (long long)(BH * S));
  if (need_d && g.D != 64 && g.D != 128) return fail(SVG_ERR_UNSUPPORTED, "head dim D=%d: only 64 and 128 are built", g.D);
  return SVG_OK;
}

svg_status check_windows(const svg_windows& w) {
  if (w.frames < 0 || w.positions < 0)
    return fail(SVG_ERR_INVALID, "windows must be >= 0 (frames=%d positions=%d)", w.frames, w.positions);
  return SVG_OK;
}

svg_status check_ptrs(std::initializer_list<std::pair<const void*, const char*>> ps) {
  for (auto& p : ps) {
    if (p.first == nullptr) return fail(SVG_ERR_INVALID, "%s is NULL", p.second);
    if (!aligned16(p.first)) return fail(SVG_ERR_INVALID, "%s is not 16-byte aligned", p.second);
  }
  return SVG_OK;
}

int32_t clamp_window(int32_t w, int32_t n) { return w > n ? n : w; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t profile_ws_bytes(const svg_geom& g, int32_t n_q) {
  const int32_t S = g.F * g.HH * g.WW;
  svg::ProfilePlan p = svg::profile_plan(g.B * g.H, S, g.D, n_q);
  return align_up(p.ml_floats * sizeof(float), 256) + align_up(p.o_floats * sizeof(float), 256) +
         align_up(p.sq_doubles * sizeof(double), 256);
}

// the head order, then the persistent kernel's per-XCD work counters
size_t attn_ws_bytes(const svg_geom& g) { return align_up((size_t)g.B * g.H * sizeof(int32_t), 256) + 256; }

}  // namespace

static svg_status svg_qknorm_rope_impl(const void* q, const void* k, void* q_out, void* k_out, const float* wq,
                                       const float* wk, float eps, float rope_base, int32_t dt, int32_t dh, int32_t dw,
                                       svg_geom g, void* stream, bool launch) {
  svg_status s;
  if ((s = check_geom(g, true)) != SVG_OK) return s;
  if ((s = check_ptrs({{q, "q"}, {k, "k"}, {q_out, "q_out"}, {k_out, "k_out"}, {wq, "wq"}, {wk, "wk"}})) != SVG_OK)
    return s;
  if (!(eps > 0.f) || !std::isfinite(eps)) return fail(SVG_ERR_INVALID, "eps must be finite and > 0");
  if (!(rope_base > 0.f) || !std::isfinite(rope_base)) return fail(SVG_ERR_INVALID, "rope_base must be finite and > 0");
  if (dt < 0 || dh < 0 || dw < 0 || (dt & 1) || (dh & 1) || (dw & 1) || dt + dh + dw != g.D)
    return fail(SVG_ERR_INVALID, "rope slices dt=%d dh=%d dw=%d must be even, >= 0 and sum to D=%d", dt, dh, dw, g.D);
  const int64_t entries = (int64_t)g.F * (dt / 2) + (int64_t)g.HH * (dh / 2) + (int64_t)g.WW * (dw / 2);
  if (entries * 8 > 64 * 1024)
    return fail(SVG_ERR_UNSUPPORTED, "rope tables (%lld entries) exceed 64 KiB of LDS", (long long)entries);
  if (!launch) return SVG_OK;
  svg::RopeArgs a;
  a.in[0] = (const svg::bf16*)q;
  a.in[1] = (const svg::bf16*)k;
  a.out[0] = (svg::bf16*)q_out;
  a.out[1] = (svg::bf16*)k_out;
  a.w[0] = wq;
  a.w[1] = wk;
  a.eps = eps;
  a.base = (double)rope_base;
  a.BH = g.B * g.H;
  a.S = g.F * g.HH * g.WW;
  a.F = g.F;
  a.HH = g.HH;
  a.WW = g.WW;
  a.P = g.HH * g.WW;
  a.D = g.D;
  a.dt = dt;
  a.dh = dh;
  a.dw = dw;
  a.divS = svg::make_fastdiv((uint32_t)a.S);
  a.divP = svg::make_fastdiv((uint32_t)(g.HH * g.WW));
  a.divWW = svg::make_fastdiv((uint32_t)g.WW);
  return hip_status(svg::launch_qknorm_rope(a, (hipStream_t)stream), "svg_qknorm_rope");
}

SVG_API svg_status svg_qknorm_rope(const void* q, const void* k, void* q_out, void* k_out, const float* wq,
                                   const float* wk, float eps, float rope_base, int32_t dt, int32_t dh, int32_t dw,
                                   svg_geom g, void* stream) {
  return svg_qknorm_rope_impl(q, k, q_out, k_out, wq, wk, eps, rope_base, dt, dh, dw, g, stream, true);
}

// The attention and profiling kernels address a head's rows with 32-bit byte offsets.
static svg_status check_head_bytes(const svg_geom& g) {
  const int64_t S = (int64_t)g.F * g.HH * g.WW;
  if (S * g.D * 2 >= ((int64_t)1 << 32))
    return fail(SVG_ERR_UNSUPPORTED, "one head of S=%lld rows x D=%d exceeds 4 GB", (long long)S, g.D);
  return SVG_OK;
}

static svg_status svg_profile_heads_impl(const void* q, const void* k, const void* v, const int32_t* q_idx, int32_t n_q,
                                         svg_geom g, svg_windows w, float scale, float* mse_out, uint8_t* kind_out,
                                         void* ws, size_t ws_bytes, void* stream, bool launch) {
  svg_status s;
  if ((s = check_geom(g, true)) != SVG_OK) return s;
  if ((s = check_windows(w)) != SVG_OK) return s;
  if ((s = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}})) != SVG_OK) return s;
  if ((s = check_head_bytes(g)) != SVG_OK) return s;
  if (q_idx == nullptr || mse_out == nullptr || kind_out == nullptr)
    return fail(SVG_ERR_INVALID, "q_idx, mse_out and kind_out must not be NULL");
  if (((uintptr_t)q_idx & 3u) || ((uintptr_t)mse_out & 3u))
    return fail(SVG_ERR_INVALID, "q_idx and mse_out must be 4-byte aligned");
  const int32_t S = g.F * g.HH * g.WW;
  if (n_q < 1 || n_q > S) return fail(SVG_ERR_INVALID, "n_q=%d must be in [1, S=%d]", n_q, S);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(SVG_ERR_INVALID, "scale must be finite and > 0");
  const size_t need = profile_ws_bytes(g, n_q);
  if (ws == nullptr || ws_bytes < need)
    return fail(SVG_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws == nullptr ? (size_t)0 : ws_bytes);
  if (!aligned16(ws)) return fail(SVG_ERR_INVALID, "ws is not 16-byte aligned");
  if (!launch) return SVG_OK;
  svg::ProfilePlan plan = svg::profile_plan(g.B * g.H, S, g.D, n_q);
  svg::ProfileArgs a;
  a.q = (const svg::bf16*)q;
  a.k = (const svg::bf16*)k;
  a.v = (const svg::bf16*)v;
  a.idx = q_idx;
  a.n_q = n_q;
  a.n_zq = plan.n_zq;
  a.BH = g.B * g.H;
  a.S = S;
  a.F = g.F;
  a.P = g.HH * g.WW;
  a.D = g.D;
  a.w_f = clamp_window(w.frames, g.F);
  a.w_p = clamp_window(w.positions, a.P);
  a.divP = svg::make_fastdiv((uint32_t)a.P);
  a.scale = scale;
  a.nsplit = plan.nsplit;
  a.part_ml = (float*)ws;
  a.part_o = (float*)((char*)ws + align_up(plan.ml_floats * sizeof(float), 256));
  a.row_sq = (double*)((char*)a.part_o + align_up(plan.o_floats * sizeof(float), 256));
  a.mse = mse_out;
  a.kind = kind_out;
  return hip_status(svg::launch_profile(a, (hipStream_t)stream), "svg_profile_heads");
}

SVG_API svg_status svg_profile_heads(const void* q, const void* k, const void* v, const int32_t* q_idx, int32_t n_q,
                                     svg_geom g, svg_windows w, float scale, float* mse_out, uint8_t* kind_out,
                                     void* ws, size_t ws_bytes, void* stream) {
  return svg_profile_heads_impl(q, k, v, q_idx, n_q, g, w, scale, mse_out, kind_out, ws, ws_bytes, stream, true);
}

static svg_status permute_common(const void* src, void* dst, int32_t elem_bytes, const uint8_t* kind, int32_t select,
                                 svg_geom g, void* stream, bool inverse) {
  svg_status s;
  if ((s = check_geom(g, false)) != SVG_OK) return s;
  if ((s = check_ptrs({{src, "src"}, {dst, "dst"}})) != SVG_OK) return s;
  if (elem_bytes != 2 && elem_bytes != 4) return fail(SVG_ERR_INVALID, "elem_bytes=%d must be 2 or 4", elem_bytes);
  const int64_t row_bytes = (int64_t)g.D * elem_bytes;
  if (row_bytes != 128 && row_bytes != 256 && row_bytes != 512)
    return fail(SVG_ERR_UNSUPPORTED, "row of D*elem_bytes=%lld bytes: 128, 256 or 512 supported", (long long)row_bytes);
  const int32_t S = g.F * g.HH * g.WW;
  const size_t bytes = (size_t)g.B * g.H * S * row_bytes;
  const char* a0 = (const char*)src;
  const char* b0 = (const char*)dst;
  if (a0 < b0 + bytes && b0 < a0 + bytes) return fail(SVG_ERR_INVALID, "src and dst overlap");
  svg::PermuteArgs a;
  a.src = src;
  a.dst = dst;
  a.kind = kind;
  a.select = select;
  a.BH = g.B * g.H;
  a.S = S;
  a.row_bytes = (int32_t)row_bytes;
  const int32_t P = g.HH * g.WW;
  a.divA = svg::make_fastdiv((uint32_t)(inverse ? P : g.F));
  a.Bm = inverse ? g.F : P;
  return hip_status(svg::launch_permute(a, (hipStream_t)stream), inverse ? "svg_unpermute" : "svg_permute");
}

SVG_API svg_status svg_permute(const void* src, void* dst, int32_t elem_bytes, const uint8_t* kind, int32_t select,
                               svg_geom g, void* stream) {
  return permute_common(src, dst, elem_bytes, kind, select, g, stream, false);
}

SVG_API svg_status svg_unpermute(const void* src, void* dst, int32_t elem_bytes, const uint8_t* kind, int32_t select,
                                 svg_geom g, void* stream) {
  return permute_common(src, dst, elem_bytes, kind, select, g, stream, true);
}

SVG_API svg_status svg_build_block_mask(const uint8_t* kind, svg_geom g, svg_windows w, int32_t bm, int32_t bn,
                                        uint8_t* mask_out, void* stream) {
  svg_status s;
  if ((s = check_geom(g, false)) != SVG_OK) return s;
  if ((s = check_windows(w)) != SVG_OK) return s;
  if (kind == nullptr || mask_out == nullptr) return fail(SVG_ERR_INVALID, "kind and mask_out must not be NULL");
  const int32_t S = g.F * g.HH * g.WW;
  if (bm < 1 || bn < 1 || bm > (1 << 30) || bn > (1 << 30))
    return fail(SVG_ERR_INVALID, "bm=%d, bn=%d must be in [1, 2^30]", bm, bn);
  svg::BlockMaskArgs a;
  a.kind = kind;
  a.out = mask_out;
  a.BH = g.B * g.H;
  a.S = S;
  a.F = g.F;
  a.P = g.HH * g.WW;
  a.w_f = clamp_window(w.frames, g.F);
  a.w_p = clamp_window(w.positions, a.P);
  a.bm = bm;
  a.bn = bn;
  a.nqb = (S + bm - 1) / bm;
  a.nkb = (S + bn - 1) / bn;
  a.divP = svg::make_fastdiv((uint32_t)a.P);
  a.divF = svg::make_fastdiv((uint32_t)g.F);
  return hip_status(svg::launch_block_mask(a, (hipStream_t)stream), "svg_build_block_mask");
}

static void fill_attn(svg::AttnArgs& a, svg_geom g, svg_windows w, float scale) {
  a.BH = g.B * g.H;
  a.S = g.F * g.HH * g.WW;
  a.F = g.F;
  a.P = g.HH * g.WW;
  a.D = g.D;
  a.w_f = clamp_window(w.frames, g.F);
  a.w_p = clamp_window(w.positions, a.P);
  a.divP = svg::make_fastdiv((uint32_t)a.P);
  a.divF = svg::make_fastdiv((uint32_t)g.F);
  a.scale = scale;
  a.lse = nullptr;
}

static svg_status svg_sparse_attn_impl(const void* q, const void* k, const void* v, const void* qt, const void* kt,
                                       const void* vt, const uint8_t* kind, svg_geom g, svg_windows w, float scale, void* o,
                                       void* ot, void* ws, size_t ws_bytes, void* stream, bool launch) {
  svg_status s;
  if ((s = check_geom(g, true)) != SVG_OK) return s;
  if ((s = check_windows(w)) != SVG_OK) return s;
  if ((s = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}, {o, "o"}})) != SVG_OK) return s;
  // all four token-major tensors NULL: temporal heads are read and written in place (fused)
  const bool fused = qt == nullptr && kt == nullptr && vt == nullptr && ot == nullptr;
  if (kind != nullptr && !fused) {
    if ((s = check_ptrs({{qt, "qt"}, {kt, "kt"}, {vt, "vt"}, {ot, "ot"}})) != SVG_OK) return s;
  }
  if ((s = check_head_bytes(g)) != SVG_OK) return s;
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(SVG_ERR_INVALID, "scale must be finite and > 0");
  const size_t need = attn_ws_bytes(g);
  if (kind != nullptr && (ws == nullptr || ws_bytes < need))
    return fail(SVG_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws == nullptr ? (size_t)0 : ws_bytes);
  if (kind != nullptr && ((uintptr_t)ws & 3u)) return fail(SVG_ERR_INVALID, "ws is not 4-byte aligned");
  if (!launch) return SVG_OK;
  svg::AttnArgs a;
  a.q = (const svg::bf16*)q;
  a.k = (const svg::bf16*)k;
  a.v = (const svg::bf16*)v;
  a.qt = (const svg::bf16*)(qt ? qt : q);
  a.kt = (const svg::bf16*)(kt ? kt : k);
  a.vt = (const svg::bf16*)(vt ? vt : v);
  a.o = (svg::bf16*)o;
  a.ot = (svg::bf16*)(ot ? ot : o);
  a.kind = kind;
  a.order = kind ? (int32_t*)ws : nullptr;
  a.queue = kind ? (int32_t*)((char*)ws + align_up((size_t)g.B * g.H * sizeof(int32_t), 256)) : nullptr;
  a.force_dense = 0;
  a.fused_t = fused ? 1 : 0;
  fill_attn(a, g, w, scale);
  return hip_status(svg::launch_attention(a, (hipStream_t)stream), "svg_sparse_attn");
}

SVG_API svg_status svg_sparse_attn(const void* q, const void* k, const void* v, const void* qt, const void* kt,
                                   const void* vt, const uint8_t* kind, svg_geom g, svg_windows w, float scale, void* o,
                                   void* ot, void* ws, size_t ws_bytes, void* stream) {
  return svg_sparse_attn_impl(q, k, v, qt, kt, vt, kind, g, w, scale, o, ot, ws, ws_bytes, stream, true);
}

static svg_status svg_dense_attn_impl(const void* q, const void* k, const void* v, svg_geom g, float scale, void* o,
                                      void* stream, bool launch) {
  svg_status s;
  if ((s = check_geom(g, true)) != SVG_OK) return s;
  if ((s = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}, {o, "o"}})) != SVG_OK) return s;
  if ((s = check_head_bytes(g)) != SVG_OK) return s;
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(SVG_ERR_INVALID, "scale must be finite and > 0");
  if (!launch) return SVG_OK;
  svg::AttnArgs a;
  a.fused_t = 0;
  a.q = a.qt = (const svg::bf16*)q;
  a.k = a.kt = (const svg::bf16*)k;
  a.v = a.vt = (const svg::bf16*)v;
  a.o = a.ot = (svg::bf16*)o;
  a.kind = nullptr;
  a.order = nullptr;
  a.queue = nullptr;
  a.force_dense = 1;
  fill_attn(a, g, svg_windows{0, 0}, scale);
  return hip_status(svg::launch_attention(a, (hipStream_t)stream), "svg_dense_attn");
}

SVG_API svg_status svg_dense_attn(const void* q, const void* k, const void* v, svg_geom g, float scale, void* o,
                                  void* stream) {
  return svg_dense_attn_impl(q, k, v, g, scale, o, stream, true);
}

// svg_layer runs profiling and attention one after the other on its stream, so they share
// one workspace.
static size_t layer_ws_bytes(const svg_geom& g, int32_t n_q) {
  const size_t p = profile_ws_bytes(g, n_q), a = attn_ws_bytes(g);
  return p > a ? p : a;
}

SVG_API int32_t svg_dense_step(int32_t step, int32_t n_steps, float dense_fraction) {
  if (n_steps <= 0 || step < 0 || step >= n_steps || !(dense_fraction >= 0.f && dense_fraction <= 1.f))
    return fail(SVG_ERR_INVALID, "step=%d of n_steps=%d, dense_fraction=%g: need 0 <= step < n_steps, fraction in [0, 1]",
                step, n_steps, (double)dense_fraction);
  return (double)step < (double)dense_fraction * (double)n_steps ? 1 : 0;
}

SVG_API svg_status svg_layer(const void* q, const void* k, const void* v, const float* wq, const float* wk, float eps,
                             float rope_base, int32_t dt, int32_t dh, int32_t dw, void* qn, void* kn,
                             const int32_t* q_idx, int32_t n_q, svg_geom g, svg_windows w, float scale, int32_t dense,
                             void* o, float* mse_out, uint8_t* kind_out, void* ws, size_t ws_bytes, void* stream) {
  const bool norm = wq != nullptr || wk != nullptr;
  const void* qa = norm ? qn : q;       // what profiling and attention read
  const void* ka = norm ? kn : k;
  // pass 0 checks every stage, pass 1 enqueues them: a failed check enqueues nothing
  for (int pass = 0; pass < 2; ++pass) {
    const bool launch = pass == 1;
    svg_status s;
    if (norm && (s = svg_qknorm_rope_impl(q, k, qn, kn, wq, wk, eps, rope_base, dt, dh, dw, g, stream, launch)) != SVG_OK)
      return s;
    if (dense) {
      if ((s = svg_dense_attn_impl(qa, ka, v, g, scale, o, stream, launch)) != SVG_OK) return s;
    } else {
      if ((s = svg_profile_heads_impl(qa, ka, v, q_idx, n_q, g, w, scale, mse_out, kind_out, ws, ws_bytes, stream,
                                      launch)) != SVG_OK)
        return s;
      if ((s = svg_sparse_attn_impl(qa, ka, v, nullptr, nullptr, nullptr, kind_out, g, w, scale, o, nullptr, ws,
                                    ws_bytes, stream, launch)) != SVG_OK)
        return s;
    }
  }
  return SVG_OK;
}

// ---------------------------------------------------------------------------------------------
// svg_layer without a workspace argument: its scratch is a static device array, one copy per
// device.  Host code never passes the array's name to a kernel (on the host it only stands in
// for the symbol); it uses the device address looked up with hipGetSymbolAddress.
// ---------------------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[SVG_LAYER_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The current device's copy of the scratch array; `stream` must belong to that device.
svg_status noalloc_scratch(void* stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "svg_layer_noalloc (hipGetDevice)");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SVG_ERR_UNSUPPORTED, "svg_layer_noalloc: device %d is beyond the %d devices it serves", dev,
                kMaxDevices);
  int sdev = dev;
  e = hipStreamGetDevice((hipStream_t)stream, &sdev);
  if (e != hipSuccess) return hip_status(e, "svg_layer_noalloc (hipStreamGetDevice)");
  if (sdev != dev)
    return fail(SVG_ERR_INVALID, "svg_layer_noalloc: the stream belongs to device %d, device %d is current", sdev, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "svg_layer_noalloc (hipGetSymbolAddress)");
    if (p == nullptr || ((uintptr_t)p & 255u))
      return fail(SVG_ERR_HIP, "svg_layer_noalloc: scratch symbol at %p is not 256-byte aligned", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SVG_OK;
}

}  // namespace

SVG_API svg_status svg_layer_noalloc(const void* q, const void* k, const void* v, const float* wq, const float* wk,
                                     float eps, float rope_base, int32_t dt, int32_t dh, int32_t dw, void* qn,
                                     void* kn, const int32_t* q_idx, int32_t n_q, svg_geom g, svg_windows w,
                                     float scale, int32_t dense, void* o, float* mse_out, uint8_t* kind_out,
                                     void* stream) {
  svg_status s;
  if ((s = check_geom(g, true)) != SVG_OK) return s;
  const int32_t S = g.F * g.HH * g.WW;
  if (!dense) {
    if (n_q < 1 || n_q > S) return fail(SVG_ERR_INVALID, "n_q=%d must lie in [1, S=%d]", n_q, S);
    const size_t need = layer_ws_bytes(g, n_q);
    if (need > SVG_LAYER_NOALLOC_SCRATCH_BYTES)
      return fail(SVG_ERR_WORKSPACE, "svg_layer_noalloc: this layer needs %zu bytes of scratch, the static array holds %zu",
                  need, (size_t)SVG_LAYER_NOALLOC_SCRATCH_BYTES);
  }
  void* ws = nullptr;
  if ((s = noalloc_scratch(stream, &ws)) != SVG_OK) return s;
  return svg_layer(q, k, v, wq, wk, eps, rope_base, dt, dh, dw, qn, kn, q_idx, n_q, g, w, scale, dense, o, mse_out,
                   kind_out, ws, SVG_LAYER_NOALLOC_SCRATCH_BYTES, stream);
}

// ---------------------------------------------------------------------------------------------
// Semantic clustering path
// ---------------------------------------------------------------------------------------------
namespace {

constexpr int32_t KMEANS_MAX_C = 4096;
constexpr int32_t KMEANS_MAX_ITERS = 1000;
constexpr int32_t CLUSTER_MAX_CQ = 32767;      // work items hold the query cluster in 15 bits

int32_t geom_S(const svg_geom& g) { return g.F * g.HH * g.WW; }

struct KmeansWs {
  size_t cb, hn, counts, total;
};
KmeansWs kmeans_ws(const svg_geom& g, int32_t C) {
  const size_t BH = (size_t)g.B * g.H;
  const size_t Cpad = (size_t)svg::kmeans_cpad(C);
  KmeansWs w;
  w.cb = 0;
  w.hn = w.cb + align_up(BH * Cpad * g.D * 2, 256);
  w.counts = w.hn + align_up(BH * Cpad * sizeof(float), 256);
  w.total = w.counts + align_up(BH * (size_t)svg::cluster_nchunk(geom_S(g)) * C * sizeof(int32_t), 256);
  return w;
}

struct ClusterWs {
  size_t klist, klen, items, total;
};
ClusterWs cluster_ws(const svg_geom& g, int32_t Cq) {
  const size_t BH = (size_t)g.B * g.H;
  const size_t S = (size_t)geom_S(g);
  ClusterWs w;
  w.klist = 0;
  w.klen = align_up(BH * Cq * S * sizeof(int32_t), 256);
  w.items = w.klen + align_up(BH * Cq * sizeof(int32_t), 256);
  w.total = w.items + align_up(BH * (size_t)svg::cluster_items_per_head((int32_t)S, Cq) * sizeof(int32_t), 256);
  return w;
}

svg_status check_ws(const void* ws, size_t ws_bytes, size_t need, const char* what) {
  if (ws == nullptr || ws_bytes < need)
    return fail(SVG_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", what, ws == nullptr ? 0 : ws_bytes,
                need);
  if (!aligned16(ws)) return fail(SVG_ERR_INVALID, "%s: workspace is not 16-byte aligned", what);
  return SVG_OK;
}

}  // namespace

SVG_API svg_status svg_kmeans(const void* x, svg_geom g, int32_t C, int32_t iters, const int32_t* init_idx,
                              float* centroids, int32_t* labels, int32_t* perm, int32_t* offsets, void* ws,
                              size_t ws_bytes, void* stream) {
  svg_status s;
  if ((s = check_geom(g, true)) != SVG_OK) return s;
  if ((s = check_ptrs({{x, "x"}, {centroids, "centroids"}, {labels, "labels"}, {perm, "perm"}, {offsets, "offsets"}})) !=
      SVG_OK)
    return s;
  const int32_t S = geom_S(g);
  if (C < 1 || C > S || C > KMEANS_MAX_C)
    return fail(SVG_ERR_INVALID, "cluster count C=%d must lie in [1, min(S=%d, %d)]", C, S, KMEANS_MAX_C);
  if (iters < 1 || iters > KMEANS_MAX_ITERS)
    return fail(SVG_ERR_INVALID, "iters=%d must lie in [1, %d]", iters, KMEANS_MAX_ITERS);
  const KmeansWs w = kmeans_ws(g, C);
  if ((s = check_ws(ws, ws_bytes, w.total, "svg_kmeans")) != SVG_OK) return s;
  svg::KmeansArgs a;
  a.x = (const svg::bf16*)x;
  a.init_idx = init_idx;
  a.cent = centroids;
  a.labels = labels;
  a.perm = perm;
  a.offsets = offsets;
  a.cb = (svg::bf16*)((char*)ws + w.cb);
  a.hn = (float*)((char*)ws + w.hn);
  a.counts = (int32_t*)((char*)ws + w.counts);
  a.BH = g.B * g.H;
  a.S = S;
  a.D = g.D;
  a.C = C;
  a.iters = iters;
  return hip_status(svg::launch_kmeans(a, (hipStream_t)stream), "svg_kmeans");
}

SVG_API svg_status svg_centroid_topp(const float* cq, const float* ck, const int32_t* k_offsets, svg_geom g,
                                     int32_t Cq, int32_t Ck, float scale, float p, uint8_t* sel, void* stream) {
  svg_status s;
  if ((s = check_geom(g, true)) != SVG_OK) return s;
  if ((s = check_ptrs({{cq, "cq"}, {ck, "ck"}, {k_offsets, "k_offsets"}, {sel, "sel"}})) != SVG_OK) return s;
  const int32_t S = geom_S(g);
  if (Cq < 1 || Cq > S) return fail(SVG_ERR_INVALID, "query cluster count Cq=%d must lie in [1, S=%d]", Cq, S);
  if (Ck < 1 || Ck > S || Ck > svg::TOPP_MAX_CK)
    return fail(SVG_ERR_INVALID, "key cluster count Ck=%d must lie in [1, min(S=%d, %d)]", Ck, S, svg::TOPP_MAX_CK);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(SVG_ERR_INVALID, "scale must be finite and > 0");
  if (!(p > 0.f && p <= 1.f)) return fail(SVG_ERR_INVALID, "p=%g must lie in (0, 1]", (double)p);
  svg::ToppArgs a;
  a.cq = cq;
  a.ck = ck;
  a.k_off = k_offsets;
  a.sel = sel;
  a.BH = g.B * g.H;
  a.Cq = Cq;
  a.Ck = Ck;
  a.D = g.D;
  a.scale = (double)scale;
  a.p = (double)p;
  return hip_status(svg::launch_centroid_topp(a, (hipStream_t)stream), "svg_centroid_topp");
}

SVG_API svg_status svg_cluster_attn(const void* q, const void* k, const void* v, const int32_t* q_perm,
                                    const int32_t* q_offsets, const int32_t* k_perm, const int32_t* k_offsets,
                                    const uint8_t* sel, svg_geom g, int32_t Cq, int32_t Ck, float scale, void* o,
                                    void* ws, size_t ws_bytes, void* stream) {
  svg_status s;
  if ((s = check_geom(g, true)) != SVG_OK) return s;
  if ((s = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}, {q_perm, "q_perm"}, {q_offsets, "q_offsets"}, {k_perm, "k_perm"},
                       {k_offsets, "k_offsets"}, {sel, "sel"}, {o, "o"}})) != SVG_OK)
    return s;
  if ((s = check_head_bytes(g)) != SVG_OK) return s;
  const int32_t S = geom_S(g);
  if (Cq < 1 || Cq > S || Cq > CLUSTER_MAX_CQ)
    return fail(SVG_ERR_INVALID, "query cluster count Cq=%d must lie in [1, min(S=%d, %d)]", Cq, S, CLUSTER_MAX_CQ);
  if (Ck < 1 || Ck > S || Ck > svg::TOPP_MAX_CK)
    return fail(SVG_ERR_INVALID, "key cluster count Ck=%d must lie in [1, min(S=%d, %d)]", Ck, S, svg::TOPP_MAX_CK);
  if ((int64_t)S > (int64_t)65535 * svg::CLUSTER_TILE_ROWS)
    return fail(SVG_ERR_UNSUPPORTED, "S=%d: a query cluster may span more than 65535 tiles", S);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(SVG_ERR_INVALID, "scale must be finite and > 0");
  const ClusterWs w = cluster_ws(g, Cq);
  if ((s = check_ws(ws, ws_bytes, w.total, "svg_cluster_attn")) != SVG_OK) return s;
  const int32_t BH = g.B * g.H;
  const int32_t per_head = svg::cluster_items_per_head(S, Cq);
  svg::ClusterListArgs l;
  l.sel = sel;
  l.k_perm = k_perm;
  l.k_off = k_offsets;
  l.q_off = q_offsets;
  l.klist = (int32_t*)((char*)ws + w.klist);
  l.klen = (int32_t*)((char*)ws + w.klen);
  l.items = (int32_t*)((char*)ws + w.items);
  l.BH = BH;
  l.S = S;
  l.Cq = Cq;
  l.Ck = Ck;
  l.items_per_head = per_head;
  l.tile_rows = svg::CLUSTER_TILE_ROWS;
  if ((s = hip_status(svg::launch_cluster_lists(l, (hipStream_t)stream), "svg_cluster_attn (key lists)")) != SVG_OK)
    return s;
  svg::ClusterAttnArgs a;
  a.q = (const svg::bf16*)q;
  a.k = (const svg::bf16*)k;
  a.v = (const svg::bf16*)v;
  a.o = (svg::bf16*)o;
  a.q_perm = q_perm;
  a.q_off = q_offsets;
  a.klist = l.klist;
  a.klen = l.klen;
  a.items = l.items;
  a.BH = BH;
  a.S = S;
  a.D = g.D;
  a.Cq = Cq;
  a.items_per_head = per_head;
  a.scale = scale;
  return hip_status(svg::launch_cluster_attention(a, (hipStream_t)stream), "svg_cluster_attn");
}

// ---------------------------------------------------------------------------------------------
// Block-sparse path with an LSE-cached block search
// ---------------------------------------------------------------------------------------------
namespace {

int32_t n_qblocks(const svg_geom& g) { return (geom_S(g) + svg::BLOCK_Q_ROWS - 1) / svg::BLOCK_Q_ROWS; }
int32_t n_kblocks(const svg_geom& g) { return (geom_S(g) + svg::BLOCK_K_ROWS - 1) / svg::BLOCK_K_ROWS; }

svg_status check_blocks(const svg_geom& g) {
  if (n_kblocks(g) > svg::BLOCK_MAX_NKB)
    return fail(SVG_ERR_UNSUPPORTED, "S=%d: more than %d key blocks of %d", geom_S(g), svg::BLOCK_MAX_NKB,
                svg::BLOCK_K_ROWS);
  return SVG_OK;
}

size_t block_ws_bytes(const svg_geom& g) {
  const size_t rows = (size_t)g.B * g.H * n_qblocks(g);
  return align_up(rows * n_kblocks(g) * sizeof(int32_t), 256) + align_up(rows * sizeof(int32_t), 256);
}

}  // namespace

SVG_API svg_status svg_dense_attn_lse(const void* q, const void* k, const void* v, svg_geom g, float scale, void* o,
                                      float* lse, void* stream) {
  svg_status s;
  if ((s = check_geom(g, true)) != SVG_OK) return s;
  if ((s = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}, {o, "o"}, {lse, "lse"}})) != SVG_OK) return s;
  if ((s = check_head_bytes(g)) != SVG_OK) return s;
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(SVG_ERR_INVALID, "scale must be finite and > 0");
  svg::AttnArgs a;
  a.fused_t = 0;
  a.q = a.qt = (const svg::bf16*)q;
  a.k = a.kt = (const svg::bf16*)k;
  a.v = a.vt = (const svg::bf16*)v;
  a.o = a.ot = (svg::bf16*)o;
  a.kind = nullptr;
  a.order = nullptr;
  a.queue = nullptr;
  a.force_dense = 1;
  fill_attn(a, g, svg_windows{0, 0}, scale);
  a.lse = lse;
  return hip_status(svg::launch_attention_lse(a, (hipStream_t)stream), "svg_dense_attn_lse");
}

SVG_API svg_status svg_block_mass(const void* q, const void* k, const float* lse, svg_geom g, float scale, float* mass,
                                  void* stream) {
  svg_status s;
  if ((s = check_geom(g, true)) != SVG_OK) return s;
  if ((s = check_ptrs({{q, "q"}, {k, "k"}, {lse, "lse"}, {mass, "mass"}})) != SVG_OK) return s;
  if ((s = check_blocks(g)) != SVG_OK) return s;
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(SVG_ERR_INVALID, "scale must be finite and > 0");
  svg::BlockMassArgs a;
  a.q = (const svg::bf16*)q;
  a.k = (const svg::bf16*)k;
  a.lse = lse;
  a.mass = mass;
  a.BH = g.B * g.H;
  a.S = geom_S(g);
  a.D = g.D;
  a.nqb = n_qblocks(g);
  a.nkb = n_kblocks(g);
  a.scale = scale;
  return hip_status(svg::launch_block_mass(a, (hipStream_t)stream), "svg_block_mass");
}

SVG_API svg_status svg_block_select(const float* mass, svg_geom g, float coverage, uint8_t* sel, void* stream) {
  svg_status s;
  if ((s = check_geom(g, true)) != SVG_OK) return s;
  if ((s = check_ptrs({{mass, "mass"}, {sel, "sel"}})) != SVG_OK) return s;
  if ((s = check_blocks(g)) != SVG_OK) return s;
  if (!(coverage > 0.f && coverage <= 1.f)) return fail(SVG_ERR_INVALID, "coverage=%g must lie in (0, 1]", (double)coverage);
  svg::BlockSelectArgs a;
  a.mass = mass;
  a.sel = sel;
  a.BH = g.B * g.H;
  a.nqb = n_qblocks(g);
  a.nkb = n_kblocks(g);
  a.coverage = (double)coverage;
  return hip_status(svg::launch_block_select(a, (hipStream_t)stream), "svg_block_select");
}

SVG_API svg_status svg_block_sparse_attn(const void* q, const void* k, const void* v, const uint8_t* sel, svg_geom g,
                                         float scale, void* o, void* ws, size_t ws_bytes, void* stream) {
  svg_status s;
  if ((s = check_geom(g, true)) != SVG_OK) return s;
  if ((s = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}, {sel, "sel"}, {o, "o"}})) != SVG_OK) return s;
  if ((s = check_head_bytes(g)) != SVG_OK) return s;
  if ((s = check_blocks(g)) != SVG_OK) return s;
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(SVG_ERR_INVALID, "scale must be finite and > 0");
  const size_t need = block_ws_bytes(g);
  if ((s = check_ws(ws, ws_bytes, need, "svg_block_sparse_attn")) != SVG_OK) return s;
  svg::BlockAttnArgs a;
  a.q = (const svg::bf16*)q;
  a.k = (const svg::bf16*)k;
  a.v = (const svg::bf16*)v;
  a.o = (svg::bf16*)o;
  a.sel = sel;
  a.BH = g.B * g.H;
  a.S = geom_S(g);
  a.D = g.D;
  a.nqb = n_qblocks(g);
  a.nkb = n_kblocks(g);
  a.blist = (int32_t*)ws;
  a.blen = (int32_t*)((char*)ws + align_up((size_t)a.BH * a.nqb * a.nkb * sizeof(int32_t), 256));
  a.scale = scale;
  if ((s = hip_status(svg::launch_block_lists(a, (hipStream_t)stream), "svg_block_sparse_attn (lists)")) != SVG_OK)
    return s;
  return hip_status(svg::launch_block_attention(a, (hipStream_t)stream), "svg_block_sparse_attn");
}

SVG_API size_t svg_workspace_bytes(int32_t op, const svg_geom* g, int32_t n_q) {
  if (g == nullptr) return 0;
  const bool need_d = true;
  std::string saved = g_last_error;
  const bool good = check_geom(*g, need_d) == SVG_OK;
  g_last_error = saved;
  if (!good) return 0;
  if (op == SVG_OP_PROFILE) {
    const int32_t S = g->F * g->HH * g->WW;
    if (n_q < 1 || n_q > S) return 0;
    return profile_ws_bytes(*g, n_q);
  }
  if (op == SVG_OP_SPARSE_ATTN) return attn_ws_bytes(*g);
  if (op == SVG_OP_LAYER) {
    const int32_t S = g->F * g->HH * g->WW;
    if (n_q < 1 || n_q > S) return 0;
    return layer_ws_bytes(*g, n_q);
  }
  if (op == SVG_OP_KMEANS) {
    const int32_t S = g->F * g->HH * g->WW;
    if (n_q < 1 || n_q > S || n_q > KMEANS_MAX_C) return 0;
    return kmeans_ws(*g, n_q).total;
  }
  if (op == SVG_OP_CLUSTER_ATTN) {
    const int32_t S = g->F * g->HH * g->WW;
    if (n_q < 1 || n_q > S || n_q > CLUSTER_MAX_CQ) return 0;
    return cluster_ws(*g, n_q).total;
  }
  if (op == SVG_OP_BLOCK_ATTN) {
    if (n_kblocks(*g) > svg::BLOCK_MAX_NKB) return 0;
    return block_ws_bytes(*g);
  }
  return 0;
}

SVG_API svg_status svg_rope_split(int32_t D, int32_t* dt, int32_t* dh, int32_t* dw) {
  if (dt == nullptr || dh == nullptr || dw == nullptr) return fail(SVG_ERR_INVALID, "svg_rope_split: NULL output");
  if (D < 6 || (D & 1)) return fail(SVG_ERR_INVALID, "svg_rope_split: D=%d must be even and >= 6", D);
  const int32_t third = 2 * (D / 6);
  *dt = D - 2 * third;
  *dh = third;
  *dw = third;
  return SVG_OK;
}

SVG_API float svg_default_scale(int32_t D) { return D > 0 ? (float)(1.0 / std::sqrt((double)D)) : 0.f; }

SVG_API void svg_tile_shape(int32_t* bm, int32_t* bn) {
  if (bm) *bm = svg::ATTN_BM;
  if (bn) *bn = svg::ATTN_BN;
}

SVG_API const char* svg_status_string(svg_status s) {
  switch (s) {
    case SVG_OK: return "SVG_OK: success";
    case SVG_ERR_INVALID: return "SVG_ERR_INVALID: invalid argument";
    case SVG_ERR_UNSUPPORTED: return "SVG_ERR_UNSUPPORTED: request not supported by the library";
    case SVG_ERR_HIP: return "SVG_ERR_HIP: HIP runtime error";
    case SVG_ERR_WORKSPACE: return "SVG_ERR_WORKSPACE: workspace missing or too small";
    default: return "unknown svg_status";
  }
}

SVG_API const char* svg_last_error(void) { return g_last_error.c_str(); }
