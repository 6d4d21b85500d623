// fp32 window+sink attention (same semantics as the bf16 kernel, launch.h AttnArgs), and
// the dtype dispatcher.
//
// The fp32 path serves small fp32 streams, where exactness (max error 1e-5) matters more
// than speed: one lane per (query row, head), fp32 FMA dot products, an online softmax with
// the accurate expf, and 32-key K/V tiles staged through LDS so that a workgroup's 64 rows
// share each key load.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "launch.h"

namespace ll {

int launch_attention_bf16(const AttnArgs& a, void* stream, char* err);

namespace {

constexpr int kRows = 64;   // query rows per workgroup (one wave)
constexpr int kKeys = 32;   // keys per LDS tile

struct SegF {
  const float* k;
  const float* v;
  int64_t head_stride, row_stride;
  int32_t n;
};

struct ParamsF {
  const float* q;
  float* o;
  int64_t q_row;
  int32_t nq, n_qblk;
  SegF a, b;
  int32_t vis_mode, vT, vC, v_nsink;
  int64_t v_base, v_F, v_sink0;
  float scale;
};

__device__ int32_t row_limit_f(const ParamsF& p, int32_t row) {
  const int32_t total = p.a.n + p.b.n;
  if (p.vis_mode == 0) return total;
  const int32_t r = row / p.vT;
  const int64_t f = r < p.v_nsink ? p.v_sink0 + r : p.v_base + (r - p.v_nsink);
  const int64_t X = (f / p.vC + 1) * p.vC;
  const int64_t xs = X - p.v_sink0;
  const int64_t ns = xs < 0 ? 0 : (xs < p.v_nsink ? xs : int64_t(p.v_nsink));
  const int64_t top = X < p.v_F ? X : p.v_F;
  const int64_t nr = top > p.v_base ? top - p.v_base : 0;
  return int32_t((ns + nr) * p.vT);
}

template <int D>
__global__ __launch_bounds__(kRows) void attn_f32_kernel(ParamsF p) {
  __shared__ float ks[kKeys][D];
  __shared__ float vs[kKeys][D];
  const int h = blockIdx.x / p.n_qblk;
  const int qb = blockIdx.x % p.n_qblk;
  const int row = qb * kRows + threadIdx.x;
  const bool active = row < p.nq;
  const int lrow = active ? row : p.nq - 1;
  const int lim = row_limit_f(p, lrow);
  const int kend = row_limit_f(p, min(qb * kRows + kRows - 1, p.nq - 1));

  float q[D], acc[D];
  const float* qp = p.q + int64_t(lrow) * p.q_row + int64_t(h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = qp[d] * p.scale;
    acc[d] = 0.f;
  }
  float m = -__builtin_inff(), l = 0.f;

  for (int k0 = 0; k0 < kend; k0 += kKeys) {
    __syncthreads();
    for (int e = threadIdx.x; e < kKeys * D; e += kRows) {
      const int kk = e / D, d = e % D;
      const int j = k0 + kk;
      float kv = 0.f, vv = 0.f;
      if (j < p.a.n) {
        const int64_t off = h * p.a.head_stride + int64_t(j) * p.a.row_stride + d;
        kv = p.a.k[off];
        vv = p.a.v[off];
      } else if (j < p.a.n + p.b.n) {
        const int64_t off = h * p.b.head_stride + int64_t(j - p.a.n) * p.b.row_stride + d;
        kv = p.b.k[off];
        vv = p.b.v[off];
      }
      ks[kk][d] = kv;
      vs[kk][d] = vv;
    }
    __syncthreads();
    const int kn = min(kKeys, lim - k0);
    for (int kk = 0; kk < kn; ++kk) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = __builtin_fmaf(q[d], ks[kk][d], s);
      const float mn = fmaxf(m, s);
      const float alpha = expf(m - mn);
      const float pw = expf(s - mn);
      l = l * alpha + pw;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(pw, vs[kk][d], acc[d] * alpha);
      m = mn;
    }
  }
  if (active) {
    float* op = p.o + int64_t(row) * p.q_row + int64_t(h) * D;
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
  }
}

}  // namespace

int launch_attention(const AttnArgs& a, void* stream, char* err) {
  if (a.qx != nullptr && a.x.n > 0 && !(a.dtype == 1 && a.D == 128)) {
    // no fused kernel for this shape: the self part, then the cross part as its own launch
    AttnArgs self = a;
    self.qx = nullptr;
    self.ox = nullptr;
    self.x = KeySeg{};
    if (int r = launch_attention(self, stream, err)) return r;
    AttnArgs cx = self;
    cx.q = a.qx;
    cx.o = a.ox;
    cx.seg[0] = a.x;
    cx.seg[1] = a.x;
    cx.seg[1].n = 0;
    cx.vis = Visibility{};
    cx.ws = nullptr;
    return launch_attention(cx, stream, err);
  }
  if (a.dtype == 1) return launch_attention_bf16(a, stream, err);
  if (a.dtype != 0) {
    snprintf(err, 256, "dtype %d", a.dtype);
    return 1;
  }
  if (a.seg[0].fp4 || a.seg[1].fp4) {
    snprintf(err, 256, "FP4 keys need bf16");
    return 1;
  }
  if (a.nq <= 0) return 0;
  ParamsF p{};
  p.q = static_cast<const float*>(a.q);
  p.o = static_cast<float*>(a.o);
  p.q_row = int64_t(a.H) * a.D;
  p.nq = a.nq;
  p.n_qblk = (a.nq + kRows - 1) / kRows;
  auto seg = [](const KeySeg& s) {
    SegF d{};
    d.k = static_cast<const float*>(s.k);
    d.v = static_cast<const float*>(s.v);
    d.head_stride = s.head_stride;
    d.row_stride = s.row_stride;
    d.n = s.n;
    return d;
  };
  p.a = seg(a.seg[0]);
  p.b = seg(a.seg[1]);
  p.vis_mode = a.vis.mode;
  p.vT = a.vis.T;
  p.vC = a.vis.C;
  p.v_nsink = a.vis.n_sink;
  p.v_base = a.vis.base;
  p.v_F = a.vis.F;
  p.v_sink0 = a.vis.sink0;
  p.scale = a.scale;
  const dim3 grid(p.n_qblk * a.H);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.D == 64) {
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(kRows), 0, s, p);
  } else if (a.D == 128) {
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(kRows), 0, s, p);
  } else {
    snprintf(err, 256, "head_dim %d", a.D);
    return 1;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(err, 256, "%s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

}  // namespace ll
