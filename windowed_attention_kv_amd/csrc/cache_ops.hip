// Cache kernels: fused K+V append/evict (commit and recache rewrite), the FP4 KV codec and
// slot-order export.
//
// Commit ("LongLive" summary page, 方法 §3 高效长推理): a chunk's K/V frames are written into
// the layer's slots; a window slot is overwritten in place, which IS the eviction of the frame
// W earlier, so eviction moves no bytes. One launch covers K and V (blockIdx.y), with
// 16-byte coalesced loads and stores over consecutive token rows.
//
// FP4 store ("LongLive 2.0" distributed-inference page, NVFP4 / KV cache section; element
// and scale encodings of the OCP MX v1.0 E2M1 / E8M0 tables): per block of 16 bf16 values
// along head_dim, scale byte sb = max(exponent_field(max|x|) - 2, 0) and each element is
// rounded to the e2m1 grid of |x| * 2^(127-sb), ties to the even code, saturating at 6.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "launch.h"

namespace ll {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// 2^(sb-127) as an fp32 value (sb = 0 gives the denormal 2^-127)
__device__ __forceinline__ float e8m0_value(uint32_t sb) {
  return __uint_as_float(sb ? (sb << 23) : 0x00400000u);
}

// Quantise 16 bf16 values (two uint4) into 8 packed bytes (uint2) and return the scale byte.
// The block scale is computed with integer ops on the bit patterns (|x| orders like its low
// 15 bits); the element rounding uses gfx950's scaled bf16->fp4 conversion, which divides by
// the scale, rounds to nearest-even on the e2m1 grid and saturates at 6 -- bit-identical to
// the codec's definition for every finite bf16 input at every scale byte (checked
// exhaustively against the CPU oracle).
__device__ __forceinline__ uint32_t quant16(uint4 a, uint4 b, uint2& packed) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
    amax = max(amax, max(lo, hi));
  }
  const uint32_t b8 = amax >> 7;             // exponent field of the block max
  const uint32_t sb = b8 > 2u ? b8 - 2u : 0u;
  const float scale = e8m0_value(sb);
  uint32_t out[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, w[4 * h + 0]), scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, w[4 * h + 1]), scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, w[4 * h + 2]), scale, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, w[4 * h + 3]), scale, 3);
    out[h] = r;
  }
  packed = make_uint2(out[0], out[1]);
  return sb;
}

// Quantise 64 consecutive bf16 values (four 16-element blocks) at `src`: 32 packed bytes
// and the 4 scale bytes (block i in byte i).
__device__ __forceinline__ void quant64(const uint8_t* src, uint4& pk0, uint4& pk1, uint32_t& sc) {
  uint4 x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = reinterpret_cast<const uint4*>(src)[i];
  uint2 p[4];
  sc = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) sc |= quant16(x[2 * b], x[2 * b + 1], p[b]) << (8 * b);
  pk0 = make_uint4(p[0].x, p[0].y, p[1].x, p[1].y);
  pk1 = make_uint4(p[2].x, p[2].y, p[3].x, p[3].y);
}

struct ScatterP {
  int32_t row0;              // first token row of this launch (launches are split below 2^24 units)
  int32_t ring0;             // window slot (frame id mod W) of the first non-lead frame
  float inv_w;               // 1 / W
  const uint8_t* src[2];
  uint8_t* dst[2];
  uint8_t* dst_scales[2];
  int32_t H, D, T, es;       // es: element size in bytes
  int32_t n_lead, lead_slot0, ring_base, W, slots;
  int64_t first_ring;
  int32_t spill_lo, spill_hi, spill_slot0;
};

// i / d for 0 <= i < 2^24 and 0 < d < 2^16, via a float reciprocal and one correction step
// (the float estimate is off by at most one).
__device__ __forceinline__ int32_t fdiv(int32_t i, int32_t d, float inv) {
  int32_t q = int32_t(float(i) * inv);
  const int32_t r = i - q * d;
  q += (r < 0) ? -1 : (r >= d ? 1 : 0);
  return q;
}

// Slot of source frame rank r: the lead ranks (spilled sink frames of a recache rewrite) go to
// consecutive sink slots, the rest to the window ring.
__device__ __forceinline__ int32_t slot_of_rank(const ScatterP& p, int32_t r) {
  if (r < p.n_lead) return p.lead_slot0 + r;
  const int32_t k = p.ring0 + (r - p.n_lead);
  return p.ring_base + (k - p.W * fdiv(k, p.W, p.inv_w));
}

// Slot that receives the old contents of rank r's destination before it is overwritten
// (a sink frame leaving the window), or -1.
__device__ __forceinline__ int32_t spill_slot(const ScatterP& p, int32_t r) {
  return (r >= p.spill_lo && r < p.spill_hi) ? p.spill_slot0 + (r - p.spill_lo) : -1;
}

// dense: one workgroup per (token row, K|V), 16-byte units; the row's slot is computed once
__global__ __launch_bounds__(256) void scatter_dense_kernel(ScatterP p, int32_t n_units, int32_t units,
                                                            float inv_units, float inv_t, int32_t uph_log2) {
  const int32_t tr = p.row0 + blockIdx.x;
  const int which = blockIdx.y;
  const int32_t r = tr / p.T, t = tr - r * p.T;
  const int32_t slot = slot_of_rank(p, r);
  const int32_t spill = spill_slot(p, r);
  const int32_t row_bytes = p.D * p.es;
  const int32_t uph = row_bytes >> 4;
  const uint8_t* src = p.src[which] + int64_t(tr) * units * 16;
  const int64_t head_plane = int64_t(p.slots) * p.T * row_bytes;
  const int64_t dst_row = (int64_t(slot) * p.T + t) * row_bytes;
  const int64_t spill_row = (int64_t(spill) * p.T + t) * row_bytes;
  if (spill >= 0) {
    // a sink frame leaves the window: the same thread reads the old 16 bytes, moves them to
    // the sink slot, then overwrites them (rare rows; the common loop below stays plain)
    for (int32_t u = threadIdx.x; u < units; u += blockDim.x) {
      const int32_t h = u >> uph_log2, cc = u & (uph - 1);
      const uint4 x = *reinterpret_cast<const uint4*>(src + int64_t(u) * 16);
      uint8_t* dp = p.dst[which] + h * head_plane + dst_row + cc * 16;
      const uint4 old = *reinterpret_cast<const uint4*>(dp);
      *reinterpret_cast<uint4*>(p.dst[which] + h * head_plane + spill_row + cc * 16) = old;
      *reinterpret_cast<uint4*>(dp) = x;
    }
    return;
  }
  for (int32_t u = threadIdx.x; u < units; u += blockDim.x) {
    const int32_t h = u >> uph_log2, cc = u & (uph - 1);
    const uint4 x = *reinterpret_cast<const uint4*>(src + int64_t(u) * 16);
    *reinterpret_cast<uint4*>(p.dst[which] + h * head_plane + dst_row + cc * 16) = x;
  }
}

// fp4: one thread per 64 elements (4 scale blocks) of a (token, head) row, one workgroup per
// kFp4Rows token rows and K|V: 32 packed bytes and one 4-byte scale word per thread.
// D % 64 == 0.
constexpr int kFp4Rows = 8;
__global__ __launch_bounds__(256) void scatter_fp4_kernel(ScatterP p, int32_t n_units, int32_t units,
                                                          float inv_units, float inv_t, int32_t gph_log2) {
  const int which = blockIdx.y;
  const int64_t head_rows = int64_t(p.slots) * p.T;
  const int32_t tr0 = p.row0 + blockIdx.x * kFp4Rows;
  const int32_t nrows = n_units / units;
  const int32_t nr = min(kFp4Rows, p.row0 + nrows - tr0);
  // frame ranks of this workgroup's rows; when one of them moves a sink frame out of the
  // window, a first pass moves the old codes and scales (bytes, no re-quantisation) to the
  // sink slot before any of them is overwritten (rare; the common pass stays plain)
  const int32_t r_first = tr0 / p.T, r_last = (tr0 + nr - 1) / p.T;
  if (r_last >= p.spill_lo && r_first < p.spill_hi) {
    for (int32_t i = threadIdx.x; i < nr * units; i += blockDim.x) {
      const int32_t rl = i / units, g = i - rl * units;
      const int32_t tr = tr0 + rl;
      const int32_t r = tr / p.T, t = tr - r * p.T;
      const int32_t spill = spill_slot(p, r);
      if (spill < 0) continue;
      const int32_t h = g >> gph_log2, cc = g & ((1 << gph_log2) - 1);
      const int64_t row = h * head_rows + int64_t(slot_of_rank(p, r)) * p.T + t;
      const int64_t srow = h * head_rows + int64_t(spill) * p.T + t;
      const uint4* dp = reinterpret_cast<const uint4*>(p.dst[which] + row * (p.D / 2) + cc * 32);
      uint4* sdp = reinterpret_cast<uint4*>(p.dst[which] + srow * (p.D / 2) + cc * 32);
      const uint4 o0 = dp[0], o1 = dp[1];
      const uint32_t os = *reinterpret_cast<const uint32_t*>(p.dst_scales[which] + row * (p.D / 16) + cc * 4);
      sdp[0] = o0;
      sdp[1] = o1;
      *reinterpret_cast<uint32_t*>(p.dst_scales[which] + srow * (p.D / 16) + cc * 4) = os;
    }
    __syncthreads();
  }
  for (int32_t i = threadIdx.x; i < nr * units; i += blockDim.x) {
    const int32_t rl = i / units, g = i - rl * units;
    const int32_t tr = tr0 + rl;
    const int32_t r = tr / p.T, t = tr - r * p.T;
    const int32_t h = g >> gph_log2, cc = g & ((1 << gph_log2) - 1);
    uint4 pk0, pk1;
    uint32_t sc;
    quant64(p.src[which] + (int64_t(tr) * units + g) * 128, pk0, pk1, sc);
    const int64_t row = h * head_rows + int64_t(slot_of_rank(p, r)) * p.T + t;
    uint8_t* dp = p.dst[which] + row * (p.D / 2) + cc * 32;
    reinterpret_cast<uint4*>(dp)[0] = pk0;
    reinterpret_cast<uint4*>(dp)[1] = pk1;
    *reinterpret_cast<uint32_t*>(p.dst_scales[which] + row * (p.D / 16) + cc * 4) = sc;
  }
}

// standalone codec: one thread per 64 elements when the row length allows, else per 16
__global__ __launch_bounds__(256) void quant64_kernel(const uint8_t* x, int64_t ngrp, uint8_t* packed,
                                                      uint8_t* scales) {
  for (int64_t g = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; g < ngrp;
       g += int64_t(gridDim.x) * blockDim.x) {
    uint4 pk0, pk1;
    uint32_t sc;
    quant64(x + g * 128, pk0, pk1, sc);
    reinterpret_cast<uint4*>(packed + g * 32)[0] = pk0;
    reinterpret_cast<uint4*>(packed + g * 32)[1] = pk1;
    *reinterpret_cast<uint32_t*>(scales + g * 4) = sc;
  }
}

__global__ __launch_bounds__(256) void quant_kernel(const uint8_t* x, int64_t nblk, uint8_t* packed,
                                                    uint8_t* scales) {
  for (int64_t b = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; b < nblk;
       b += int64_t(gridDim.x) * blockDim.x) {
    const uint4 x0 = *reinterpret_cast<const uint4*>(x + b * 32);
    const uint4 x1 = *reinterpret_cast<const uint4*>(x + b * 32 + 16);
    uint2 pk;
    const uint32_t sb = quant16(x0, x1, pk);
    *reinterpret_cast<uint2*>(packed + b * 8) = pk;
    scales[b] = uint8_t(sb);
  }
}

struct ExportP {
  const uint8_t* src[2];
  const uint8_t* src_scales[2];
  uint8_t* out[2];
  uint8_t* out_scales[2];
  int32_t H, T, slots;
  int32_t row_bytes;    // bytes of one (token, head) row: D*es dense, D/2 fp4
  int32_t srow_bytes;   // scale bytes of one (token, head) row (fp4), else 0
};

// one workgroup per slot-order token row; head-major plane -> token-major output
__global__ __launch_bounds__(256) void export_kernel(ExportP p) {
  const int64_t tr = blockIdx.x;
  const int which = blockIdx.y;
  const int64_t rows_per_head = int64_t(p.slots) * p.T;
  const int32_t uph = p.row_bytes >> 2;            // 4-byte units (fp4 rows may be 32 bytes)
  for (int32_t u = threadIdx.x; u < p.H * uph; u += blockDim.x) {
    const int32_t h = u / uph, c = u - h * uph;
    const uint32_t x = *reinterpret_cast<const uint32_t*>(
        p.src[which] + (h * rows_per_head + tr) * p.row_bytes + c * 4);
    *reinterpret_cast<uint32_t*>(p.out[which] + (tr * p.H + h) * p.row_bytes + c * 4) = x;
  }
  if (p.srow_bytes) {
    for (int32_t u = threadIdx.x; u < p.H * p.srow_bytes; u += blockDim.x) {
      const int32_t h = u / p.srow_bytes, c = u - h * p.srow_bytes;
      p.out_scales[which][(tr * p.H + h) * p.srow_bytes + c] =
          p.src_scales[which][(h * rows_per_head + tr) * p.srow_bytes + c];
    }
  }
}

// workspace clearing: one 32-bit word per thread
__global__ __launch_bounds__(256) void zero_kernel(uint32_t* p, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

int finish(char* err) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(err, 256, "%s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

int block_for(int units) {
  int b = (units + 63) / 64 * 64;
  return b < 64 ? 64 : (b > 256 ? 256 : b);
}

}  // namespace

int launch_scatter(const ScatterArgs& a, void* stream, char* err) {
  if (a.n_frames <= 0) return 0;
  ScatterP p{};
  p.src[0] = static_cast<const uint8_t*>(a.k_src);
  p.src[1] = static_cast<const uint8_t*>(a.v_src);
  p.dst[0] = static_cast<uint8_t*>(a.k_dst);
  p.dst[1] = static_cast<uint8_t*>(a.v_dst);
  p.dst_scales[0] = a.k_dst_scales;
  p.dst_scales[1] = a.v_dst_scales;
  p.H = a.H;
  p.D = a.D;
  p.T = a.T;
  p.es = a.dtype == 1 ? 2 : 4;
  p.n_lead = a.n_lead;
  p.lead_slot0 = a.lead_slot0;
  p.ring_base = a.ring_base;
  p.W = a.W;
  p.slots = a.slots;
  p.first_ring = a.first_ring;
  p.ring0 = int32_t(a.first_ring % a.W);
  p.spill_lo = a.spill_lo;
  p.spill_hi = a.spill_hi;
  p.spill_slot0 = a.spill_slot0;
  p.inv_w = 1.0f / float(a.W);
  const int32_t n_rows = a.n_frames * a.T;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float inv_t = 1.0f / float(a.T);
  if (a.fp4 && a.D % 64) {
    snprintf(err, 256, "the FP4 store needs head_dim %% 64 == 0");
    return 1;
  }
  const int32_t gph = a.D / 64;
  const int32_t uph = a.D * p.es / 16;             // 8, 16 or 32
  const int32_t units = a.fp4 ? a.H * gph : a.H * uph;
  const int32_t rows_per_launch = ((1 << 24) - 1) / units;
  for (int32_t r0 = 0; r0 < n_rows; r0 += rows_per_launch) {
    p.row0 = r0;
    const int32_t n_units = min(rows_per_launch, n_rows - r0) * units;
    if (a.fp4) {
      const int blocks = (n_units / units + kFp4Rows - 1) / kFp4Rows;
      // as many threads as the workgroup's rows have 64-element units (whole waves, at most
      // 256): 12 heads x 128 -> 8 rows x 24 units = 192 threads, none idle
      const int fp4_threads = min(256, (kFp4Rows * units + 63) / 64 * 64);
      hipLaunchKernelGGL(scatter_fp4_kernel, dim3(blocks, 2), dim3(fp4_threads), 0, s, p, n_units, units,
                         1.0f / float(units), inv_t, gph == 2 ? 1 : 0);
    } else {
      const int blocks = n_units / units;
      hipLaunchKernelGGL(scatter_dense_kernel, dim3(blocks, 2), dim3(block_for(units)), 0, s, p, n_units, units,
                         1.0f / float(units), inv_t, uph == 8 ? 3 : (uph == 16 ? 4 : 5));
    }
  }
  return finish(err);
}

int launch_quant(const QuantArgs& a, void* stream, char* err) {
  const int64_t nblk = a.rows * a.row_len / 16;
  if (nblk == 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.row_len % 64 == 0) {
    const int64_t ngrp = nblk / 4;
    int64_t grid = (ngrp + 255) / 256;
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(quant64_kernel, dim3(unsigned(grid)), dim3(256), 0, s,
                       static_cast<const uint8_t*>(a.x), ngrp, a.packed, a.scales);
  } else {
    int64_t grid = (nblk + 255) / 256;
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(quant_kernel, dim3(unsigned(grid)), dim3(256), 0, s,
                       static_cast<const uint8_t*>(a.x), nblk, a.packed, a.scales);
  }
  return finish(err);
}

int launch_export(const ExportArgs& a, void* stream, char* err) {
  ExportP p{};
  p.src[0] = static_cast<const uint8_t*>(a.k_src);
  p.src[1] = static_cast<const uint8_t*>(a.v_src);
  p.src_scales[0] = a.k_src_scales;
  p.src_scales[1] = a.v_src_scales;
  p.out[0] = static_cast<uint8_t*>(a.k_out);
  p.out[1] = static_cast<uint8_t*>(a.v_out);
  p.out_scales[0] = a.k_out_scales;
  p.out_scales[1] = a.v_out_scales;
  p.H = a.H;
  p.T = a.T;
  p.slots = a.slots;
  if (a.fp4) {
    p.row_bytes = a.D / 2;
    p.srow_bytes = a.D / 16;
  } else {
    p.row_bytes = a.D * (a.dtype == 1 ? 2 : 4);
    p.srow_bytes = 0;
  }
  const dim3 grid(a.slots * a.T, 2);
  hipLaunchKernelGGL(export_kernel, grid, dim3(block_for(a.H * p.row_bytes / 4)), 0,
                     static_cast<hipStream_t>(stream), p);
  return finish(err);
}

int launch_zero(void* p, int64_t bytes, void* stream, char* err) {
  if (bytes <= 0) return 0;
  if (bytes % 4 != 0 || (bytes / 4 + 255) / 256 >= (int64_t(1) << 31)) {
    snprintf(err, 256, "zero fill of %lld bytes", (long long)bytes);
    return 1;
  }
  const int64_t n = bytes / 4;
  hipLaunchKernelGGL(zero_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint32_t*>(p), n);
  return finish(err);
}

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

}  // namespace ll
