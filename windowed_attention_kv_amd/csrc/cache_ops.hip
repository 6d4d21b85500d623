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
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Streaming (non-temporal) 16-byte accesses for data touched once in whole cache lines: the
// commits' source rows and the cache rows they write (every lane of a wave takes one 16-byte
// piece, so one instruction covers whole lines). The standalone codec keeps plain loads (its
// input is often in the caches).
__device__ __forceinline__ uint4 load_nt(const uint8_t* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}
__device__ __forceinline__ void store_nt(uint8_t* p, uint4 x) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, x), reinterpret_cast<u32x4_t*>(p));
}

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

// Work mapping of every commit kernel: destination-major. A workgroup of 256 threads covers
// consecutive token rows of ONE head and one plane (K or V), and the workgroups of a row span
// enumerate the heads fastest, so the heads of a span run side by side and together read the
// span's source rows whole while each writes one contiguous run of its head's slot. One
// 16-byte source load per thread and row (an FP4 lane takes two rows), non-temporal loads and
// stores (the data is touched once). Against a row-major mapping (each thread one unit of
// several token rows of all heads, plain accesses), at the layer shape with cold sources (one
// GPU, same box): the 30-layer dense batch 73% of 8 TB/s instead of 65%, the FP4 batch 69-70%
// instead of 61%, single-layer commits 57% instead of 54% (dense) and 47% instead of 43% (FP4);
// a commit that also moves three sink frames, 55% instead of 59%. (Dense threads taking two or
// four rows: 70% and 68%.)

// Every kernel below issues its source load first and computes the destination while it is in
// flight; the helpers take the loaded value.

// Dense: one 16-byte unit x. A destination that holds a sink frame leaving the window (mv set)
// first has its old 16 bytes moved to the sink slot by the same thread, then is overwritten.
__device__ __forceinline__ void commit_unit_dense(uint4 x, uint8_t* dp, uint8_t* mv) {
  if (mv) *reinterpret_cast<uint4*>(mv) = *reinterpret_cast<const uint4*>(dp);
  store_nt(dp, x);
}

// FP4: lane c of a head row's D / 8 lanes (lpr_log2 = log2(D / 8): 3 or 4) quantises its 8
// elements. The two lanes of a 16-element block take its scale from the larger of their two
// maxima (one lane exchange) and each packs its own 8 codes into 4 bytes; the row's scale bytes
// (4 or 8) are gathered into the row's first lane, which stores them at once (with the
// non-temporal stores, 7 points of 8 TB/s faster than plain stores and one 4-byte scale store
// per 8 lanes on the 30-layer batch in a timing harness). pk / sc: the destination row's packed codes and scales;
// mv_pk / mv_sc: where a leaving sink frame's old bytes go first (null: none), moved by the
// lane that then overwrites them. Every lane of the wave calls this (lane exchanges); lanes
// with !live store nothing.
__device__ __forceinline__ void commit_lane_fp4(uint4 x, uint8_t* pk, uint8_t* sc, uint8_t* mv_pk,
                                                uint8_t* mv_sc, int32_t c, int32_t lpr_log2, bool live) {
  // the destination addresses are computed while the load is in flight, not after it inside
  // the branch below (an empty asm use keeps the compiler from sinking them there)
  asm volatile("" ::"v"(pk), "v"(sc));
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) amax = max(amax, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  amax = max(amax, uint32_t(__shfl_xor(int(amax), 1)));
  const uint32_t b8 = amax >> 7;             // exponent field of the block max
  const uint32_t sb = b8 > 2u ? b8 - 2u : 0u;
  const float scale = e8m0_value(sb);
  uint32_t q = 0;
  q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, __builtin_bit_cast(bf16x2_t, w[0]), scale, 0);
  q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, __builtin_bit_cast(bf16x2_t, w[1]), scale, 1);
  q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, __builtin_bit_cast(bf16x2_t, w[2]), scale, 2);
  q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, __builtin_bit_cast(bf16x2_t, w[3]), scale, 3);
  // scale byte of block c / 2 at byte (c / 2) % 4 of its 8-lane group's word; lane 0 of a
  // 16-lane row also takes the second group's word
  uint32_t sw = sb << (8 * ((c >> 1) & 3));
  sw |= uint32_t(__shfl_xor(int(sw), 2));
  sw |= uint32_t(__shfl_xor(int(sw), 4));
  const uint32_t sw_hi = uint32_t(__shfl_xor(int(sw), 8));
  if (!live) return;
  uint32_t* const dp = reinterpret_cast<uint32_t*>(pk) + c;
  if (mv_pk) {
    reinterpret_cast<uint32_t*>(mv_pk)[c] = *dp;
    if (c == 0) {
      if (lpr_log2 == 4) *reinterpret_cast<uint2*>(mv_sc) = *reinterpret_cast<const uint2*>(sc);
      else *reinterpret_cast<uint32_t*>(mv_sc) = *reinterpret_cast<const uint32_t*>(sc);
    }
  }
  __builtin_nontemporal_store(q, dp);
  if (c == 0) {
    if (lpr_log2 == 4) __builtin_nontemporal_store(u32x2_t{sw, sw_hi}, reinterpret_cast<u32x2_t*>(sc));
    else __builtin_nontemporal_store(sw, reinterpret_cast<uint32_t*>(sc));
  }
}

// FP4 rows per lane: a lane's waves spend part of their life quantising and exchanging with no
// load in flight, so each lane loads two rows before working on either (70% of 8 TB/s on the
// 30-layer batch in a timing harness against 65% with one, 68% with four)
constexpr int kFp4Units = 2;

// Single-layer commit and recache rewrite: grid (H x row spans, K|V), rows p.row0.. of this
// launch; each source frame rank goes to slot_of_rank (lead ranks to sink slots, the rest to
// the window ring), and a rank in the spill range first moves the sink frame it overwrites.
// dense: uph = 16-byte units per head row (8, 16 or 32), 256 / uph rows per workgroup
__global__ __launch_bounds__(256) void scatter_dense_kernel(ScatterP p, int32_t nrows, int32_t uph_log2) {
  const int which = blockIdx.y;
  const int32_t h = int32_t(blockIdx.x) % p.H;
  const int32_t span = int32_t(blockIdx.x) / p.H;
  const int32_t lr = span * (256 >> uph_log2) + int32_t(threadIdx.x >> uph_log2);
  if (lr >= nrows) return;
  const int32_t tr = p.row0 + lr;
  const int32_t cc = threadIdx.x & ((1 << uph_log2) - 1);
  const int32_t row_bytes = 16 << uph_log2;
  const uint4 x = load_nt(p.src[which] + ((int64_t(tr) * p.H + h) * row_bytes + cc * 16));
  const int32_t r = tr / p.T, t = tr - r * p.T;
  const int32_t spill = spill_slot(p, r);
  uint8_t* const head = p.dst[which] + int64_t(h) * p.slots * p.T * row_bytes + cc * 16;
  commit_unit_dense(x, head + (int64_t(slot_of_rank(p, r)) * p.T + t) * row_bytes,
                    spill >= 0 ? head + (int64_t(spill) * p.T + t) * row_bytes : nullptr);
}

// fp4: D / 8 lanes per head row (lpr_log2 = 3 or 4); each lane takes kFp4Units rows, 256 / (D / 8)
// apart, loading all of them before quantising any, so a workgroup covers kFp4Units * 256 /
// (D / 8) rows
__global__ __launch_bounds__(256) void scatter_fp4_kernel(ScatterP p, int32_t nrows, int32_t lpr_log2) {
  const int which = blockIdx.y;
  const int32_t h = int32_t(blockIdx.x) % p.H;
  const int32_t span = int32_t(blockIdx.x) / p.H;
  const int32_t c = threadIdx.x & ((1 << lpr_log2) - 1);
  const int32_t rpw = 256 >> lpr_log2;
  const int32_t D = 8 << lpr_log2;
  uint4 x[kFp4Units];
  int32_t tr[kFp4Units];
  bool live[kFp4Units];
#pragma unroll
  for (int k = 0; k < kFp4Units; ++k) {
    const int32_t lr = (span * kFp4Units + k) * rpw + int32_t(threadIdx.x >> lpr_log2);
    live[k] = lr < nrows;
    tr[k] = p.row0 + (live[k] ? lr : nrows - 1);   // rows past the end still join the exchanges
    x[k] = load_nt(p.src[which] + (int64_t(tr[k]) * p.H + h) * (D * 2) + c * 16);
  }
  const int64_t head_rows = int64_t(p.slots) * p.T;
#pragma unroll
  for (int k = 0; k < kFp4Units; ++k) {
    const int32_t r = tr[k] / p.T, t = tr[k] - r * p.T;
    const int64_t row = h * head_rows + int64_t(slot_of_rank(p, r)) * p.T + t;
    const int32_t spill = spill_slot(p, r);
    const int64_t mrow = h * head_rows + int64_t(spill) * p.T + t;
    commit_lane_fp4(x[k], p.dst[which] + row * (D / 2), p.dst_scales[which] + row * (D / 16),
                    spill >= 0 ? p.dst[which] + mrow * (D / 2) : nullptr,
                    spill >= 0 ? p.dst_scales[which] + mrow * (D / 16) : nullptr, c, lpr_log2, live[k]);
  }
}

// ---- batched commit: one chunk into many layers per launch ----
// A single layer's commit moves ~57 MB (dense) or ~37 MB (FP4) at the layer shape, too little
// for one launch to ramp up to full HBM bandwidth; committing every layer of a denoise step
// in one launch moves 30x that. blockIdx.y = 2 * layer + (K | V); the per-layer pointers and
// ring position travel in the kernel arguments.
struct LayerP {
  const uint8_t* src[2];
  uint8_t* dst[2];
  uint8_t* dst_scales[2];
  int32_t ring0;                       // window slot of the chunk's first frame
  int32_t spill_lo, spill_hi, spill_slot0;
};

struct CommitLayersP {
  int32_t H, D, T, W, slots, es;
  int32_t n_rows;                      // token rows of the chunk (C * T)
  int32_t units;                       // dense: 16-byte units per token row; fp4: 64-element groups
  LayerP l[kMaxCommitLayers];
};

// window slot of frame rank r of the chunk (ring0 < W, r < C <= W)
__device__ __forceinline__ int32_t commit_slot(int32_t ring0, int32_t r, int32_t W) {
  const int32_t k = ring0 + r;
  return k >= W ? k - W : k;
}

// dense: uph = 16-byte units per head row (8, 16 or 32), 256 / uph rows per workgroup
__global__ __launch_bounds__(256) void commit_layers_dense_kernel(CommitLayersP p, int32_t uph_log2) {
  const int which = blockIdx.y & 1;
  const int layer = blockIdx.y >> 1;
  const int32_t h = int32_t(blockIdx.x) % p.H;
  const int32_t span = int32_t(blockIdx.x) / p.H;
  const int32_t tr = span * (256 >> uph_log2) + int32_t(threadIdx.x >> uph_log2);
  if (tr >= p.n_rows) return;
  const int32_t cc = threadIdx.x & ((1 << uph_log2) - 1);
  const int32_t lo = p.l[layer].spill_lo, hi = p.l[layer].spill_hi, s0 = p.l[layer].spill_slot0;
  const int32_t row_bytes = 16 << uph_log2;
  const uint4 x = load_nt(p.l[layer].src[which] + ((int64_t(tr) * p.H + h) * row_bytes + cc * 16));
  const int32_t r = tr / p.T, t = tr - r * p.T;
  uint8_t* const head = p.l[layer].dst[which] + int64_t(h) * p.slots * p.T * row_bytes + cc * 16;
  commit_unit_dense(x, head + (int64_t(commit_slot(p.l[layer].ring0, r, p.W)) * p.T + t) * row_bytes,
                    r >= lo && r < hi ? head + (int64_t(s0 + (r - lo)) * p.T + t) * row_bytes : nullptr);
}

// fp4: D / 8 lanes per head row (lpr_log2 = 3 or 4), kFp4Units rows per lane as above
__global__ __launch_bounds__(256) void commit_layers_fp4_kernel(CommitLayersP p, int32_t lpr_log2) {
  const int which = blockIdx.y & 1;
  const int layer = blockIdx.y >> 1;
  const int32_t h = int32_t(blockIdx.x) % p.H;
  const int32_t span = int32_t(blockIdx.x) / p.H;
  const int32_t c = threadIdx.x & ((1 << lpr_log2) - 1);
  const int32_t rpw = 256 >> lpr_log2;
  const int32_t D = 8 << lpr_log2;
  uint4 x[kFp4Units];
  int32_t tr[kFp4Units];
  bool live[kFp4Units];
#pragma unroll
  for (int k = 0; k < kFp4Units; ++k) {
    const int32_t t0 = (span * kFp4Units + k) * rpw + int32_t(threadIdx.x >> lpr_log2);
    live[k] = t0 < p.n_rows;
    tr[k] = live[k] ? t0 : p.n_rows - 1;   // rows past the end still join the exchanges
    x[k] = load_nt(p.l[layer].src[which] + (int64_t(tr[k]) * p.H + h) * (D * 2) + c * 16);
  }
  const int32_t lo = p.l[layer].spill_lo, hi = p.l[layer].spill_hi, s0 = p.l[layer].spill_slot0;
  const int64_t head_rows = int64_t(p.slots) * p.T;
  uint8_t* const dst = p.l[layer].dst[which];
  uint8_t* const dsc = p.l[layer].dst_scales[which];
#pragma unroll
  for (int k = 0; k < kFp4Units; ++k) {
    const int32_t r = tr[k] / p.T, t = tr[k] - r * p.T;
    const int64_t row = h * head_rows + int64_t(commit_slot(p.l[layer].ring0, r, p.W)) * p.T + t;
    const bool move = r >= lo && r < hi;
    const int64_t mrow = h * head_rows + int64_t(s0 + (r - lo)) * p.T + t;
    commit_lane_fp4(x[k], dst + row * (D / 2), dsc + row * (D / 16),
                    move ? dst + mrow * (D / 2) : nullptr, move ? dsc + mrow * (D / 16) : nullptr,
                    c, lpr_log2, live[k]);
  }
}

// Standalone codec. Rows whose length is a multiple of 64: the input is one flat run of
// 16-byte units (8 elements each) and every 8-lane group (64 elements, four scale blocks) lies
// inside one row, so unit u's codes go to packed bytes 4u.. and its block's scale to byte u / 2:
// a lane per unit with the commit's per-lane arithmetic (commit_lane_fp4: pair max, scaled
// conversions, the group's four scale bytes gathered into one word stored by its first lane),
// non-temporal stores, and kQuantUnits units per lane loaded before any is converted. Loads
// stay plain, so an input just written (or quantised again) is served from the caches. Against
// one thread per 64 elements (eight 16-byte loads of one line each): 93-94% instead of 63% of
// 8 TB/s over a commit's bytes (28.8 MB in, 30 launches), 74% instead of 75.5% on a 147 MB
// input. Other row lengths: one thread per 16-element block.
constexpr int kQuantUnits = 4;
__global__ __launch_bounds__(256) void quant64_kernel(const uint8_t* x, int64_t n_units, uint8_t* packed,
                                                      uint8_t* scales) {
  const int32_t c = threadIdx.x & 7;
  for (int64_t base = int64_t(blockIdx.x) * 256 * kQuantUnits; base < n_units;
       base += int64_t(gridDim.x) * 256 * kQuantUnits) {
    // the loop bound is uniform over the workgroup, and n_units is a multiple of 8, so every
    // 8-lane group is wholly inside or wholly past the end
    uint4 v[kQuantUnits];
    int64_t u[kQuantUnits];
#pragma unroll
    for (int k = 0; k < kQuantUnits; ++k) {
      u[k] = base + k * 256 + threadIdx.x;
      v[k] = *reinterpret_cast<const uint4*>(x + (u[k] < n_units ? u[k] : n_units - 1) * 16);
    }
#pragma unroll
    for (int k = 0; k < kQuantUnits; ++k) {
      const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
      uint32_t amax = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = max(amax, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
      amax = max(amax, uint32_t(__shfl_xor(int(amax), 1)));
      const uint32_t b8 = amax >> 7;             // exponent field of the block max
      const uint32_t sb = b8 > 2u ? b8 - 2u : 0u;
      const float scale = e8m0_value(sb);
      uint32_t q = 0;
      q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, __builtin_bit_cast(bf16x2_t, w[0]), scale, 0);
      q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, __builtin_bit_cast(bf16x2_t, w[1]), scale, 1);
      q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, __builtin_bit_cast(bf16x2_t, w[2]), scale, 2);
      q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, __builtin_bit_cast(bf16x2_t, w[3]), scale, 3);
      uint32_t sw = sb << (8 * ((c >> 1) & 3));
      sw |= uint32_t(__shfl_xor(int(sw), 2));
      sw |= uint32_t(__shfl_xor(int(sw), 4));
      if (u[k] < n_units) {
        __builtin_nontemporal_store(q, reinterpret_cast<uint32_t*>(packed + u[k] * 4));
        if (c == 0) __builtin_nontemporal_store(sw, reinterpret_cast<uint32_t*>(scales + (u[k] >> 1)));
      }
    }
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
  if (a.fp4 && a.D % 64) {
    snprintf(err, 256, "the FP4 store needs head_dim %% 64 == 0");
    return 1;
  }
  const int32_t uph = a.D * p.es / 16;             // 8, 16 or 32
  const int32_t lg = a.fp4 ? (a.D == 64 ? 3 : 4) : (uph == 8 ? 3 : (uph == 16 ? 4 : 5));
  const int32_t rows_per_wg = (256 >> lg) * (a.fp4 ? kFp4Units : 1);
  // one launch covers at most 2^24 token rows (frame ranks stay far below the float-reciprocal
  // division's 2^24 limit)
  constexpr int32_t kRowsPerLaunch = 1 << 24;
  for (int32_t r0 = 0; r0 < n_rows; r0 += kRowsPerLaunch) {
    p.row0 = r0;
    const int32_t nr = min(kRowsPerLaunch, n_rows - r0);
    const dim3 grid(((nr + rows_per_wg - 1) / rows_per_wg) * a.H, 2);
    if (a.fp4) hipLaunchKernelGGL(scatter_fp4_kernel, grid, dim3(256), 0, s, p, nr, lg);
    else hipLaunchKernelGGL(scatter_dense_kernel, grid, dim3(256), 0, s, p, nr, lg);
  }
  return finish(err);
}

int launch_commit_layers(const CommitLayersArgs& a, void* stream, char* err) {
  if (a.n_layers <= 0) return 0;
  if (a.fp4 && a.D % 64) {
    snprintf(err, 256, "the FP4 store needs head_dim %% 64 == 0");
    return 1;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t es = a.dtype == 1 ? 2 : 4;
  const int32_t n_rows = a.C * a.T;
  for (int32_t l0 = 0; l0 < a.n_layers; l0 += kMaxCommitLayers) {
    const int32_t nl = min(kMaxCommitLayers, a.n_layers - l0);
    CommitLayersP p{};
    p.H = a.H;
    p.D = a.D;
    p.T = a.T;
    p.W = a.W;
    p.slots = a.slots;
    p.es = es;
    p.n_rows = n_rows;
    for (int32_t i = 0; i < nl; ++i) {
      const CommitLayer& c = a.layers[l0 + i];
      LayerP& L = p.l[i];
      L.src[0] = static_cast<const uint8_t*>(c.k_src);
      L.src[1] = static_cast<const uint8_t*>(c.v_src);
      L.dst[0] = static_cast<uint8_t*>(c.k_dst);
      L.dst[1] = static_cast<uint8_t*>(c.v_dst);
      L.dst_scales[0] = c.k_dst_scales;
      L.dst_scales[1] = c.v_dst_scales;
      L.ring0 = int32_t(c.first_ring % a.W);
      L.spill_lo = c.spill_lo;
      L.spill_hi = c.spill_hi;
      L.spill_slot0 = c.spill_slot0;
    }
    if (a.fp4) {
      // lanes per head row: D / 8 (8 or 16)
      const int32_t lpr_log2 = a.D == 64 ? 3 : 4;
      const int32_t rows_per_wg = (256 >> lpr_log2) * kFp4Units;
      const int32_t spans = (n_rows + rows_per_wg - 1) / rows_per_wg;
      p.units = a.H * (a.D / 64);
      hipLaunchKernelGGL(commit_layers_fp4_kernel, dim3(spans * a.H, 2 * nl), dim3(256), 0, s, p, lpr_log2);
    } else {
      const int32_t uph = a.D * es / 16;             // 8, 16 or 32
      const int32_t uph_log2 = uph == 8 ? 3 : (uph == 16 ? 4 : 5);
      const int32_t spans = (n_rows + (256 >> uph_log2) - 1) / (256 >> uph_log2);
      p.units = a.H * uph;
      hipLaunchKernelGGL(commit_layers_dense_kernel, dim3(spans * a.H, 2 * nl), dim3(256), 0, s, p, uph_log2);
    }
  }
  return finish(err);
}

int launch_quant(const QuantArgs& a, void* stream, char* err) {
  const int64_t nblk = a.rows * a.row_len / 16;
  if (nblk == 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.row_len % 64 == 0) {
    const int64_t n_units = nblk * 2;
    int64_t grid = (n_units + 256 * kQuantUnits - 1) / (256 * kQuantUnits);
    if (grid > (int64_t(1) << 20)) grid = int64_t(1) << 20;
    hipLaunchKernelGGL(quant64_kernel, dim3(unsigned(grid)), dim3(256), 0, s,
                       static_cast<const uint8_t*>(a.x), n_units, a.packed, a.scales);
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
