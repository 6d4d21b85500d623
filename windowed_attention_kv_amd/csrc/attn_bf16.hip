// Window+sink chunk attention, bf16 in / fp32 accumulate / bf16 out, for gfx950 (MI355X).
//
// What it computes ("LongLive" summary page, 方法 §3 高效长推理, and 方法 §1 KV 重缓存 for the
// recache prefill and its prompt cross-attention): for every head h and query row i
//   o[i,h,:] = sum_j softmax_j(scale * q[i,h,:] . k[j,h,:]) v[j,h,:]
// over the keys j visible to row i. The keys come from two segments read back to back: the
// layer's filled cache slots (head-major, optionally FP4 e2m1/e8m0) and the call's own K/V
// (token-major bf16). Visibility is either "all keys" (chunk attention, cross-attention) or
// the block-causal limit of the recache prefill (launch.h, Visibility).
//
// Design (MI355X-first, not a port of any listed design):
//  * a wave keeps 32 query rows of Q in registers as the B operand of
//    v_mfma_f32_32x32x16_bf16 and computes S^T = K Q^T, so each lane owns ONE query row: row
//    max / row sum are in-lane reductions plus one v_permlane32_swap, never a cross-lane tree;
//  * P^T goes straight from the S accumulator into the B operand of O^T = V^T P^T (no LDS
//    round trip);
//  * online softmax in the exp2 domain with a lazy rescale: a tile's weights are taken against
//    the running max as it stands, and only when a lane's weights sum to more than 2^8 does
//    the wave compute the tile max, rescale O (64 multiplies per lane) and redo the weights;
//    softmax is shift-invariant, so this changes rounding only;
//  * FP4 cache tiles are dequantised exactly while being written to LDS, so the MFMA inner
//    loop is identical for both cache formats ("LongLive 2.0" distributed-inference page,
//    NVFP4 and KV cache section: fused dequantisation);
//  * workgroups are mapped so that each XCD (own L2) works on a contiguous range of
//    (head, query block) tiles: the query blocks of one head share their K/V in one L2;
//    block-causal (recache) launches instead dispatch the heaviest block rank of every head
//    first, longest job first over the whole grid;
//  * each MFMA operand is read from LDS four MFMAs ahead of its use (scheduling groups), and
//    the wave priority is raised for the MFMA blocks and lowered for the softmax, so of the
//    two waves sharing a SIMD the one with MFMAs to issue wins and the other's VALU work runs
//    in the matrix pipe's shadow.
// Two kernels: attn_bf16_direct_kernel (head_dim 128: 8 waves, 128-key tiles loaded straight
// into LDS, V read with transposing LDS reads, optional split schedule for calls with fewer
// query blocks than CUs) and attn_bf16_kernel (head_dim 64: 4 waves, 64-key tiles staged
// through registers and stored transposed).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "launch.h"

namespace ll {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef float v4f32_t __attribute__((ext_vector_type(4)));
typedef float v2f32_t __attribute__((ext_vector_type(2)));
typedef uint32_t v4u32_t __attribute__((ext_vector_type(4)));
typedef uint32_t v2u32_t __attribute__((ext_vector_type(2)));

constexpr int BN = 64;          // keys per tile
constexpr float kLazyBound = 256.0f;   // largest allowed sum of a lane's weights in a tile
// start of the running max: finite, so that a visible score gives exp2(+huge) = +inf (forcing
// the first rescale) and a masked one (-inf) gives 0, and no weight or sum is ever NaN
constexpr float kNoMax = -1e30f;

struct DevSeg {
  const uint8_t* k;   // dense: bf16 base; fp4: packed base
  const uint8_t* v;
  const uint8_t* ks;  // fp4 scales
  const uint8_t* vs;
  int64_t head_stride;  // elements
  int64_t row_stride;   // elements
  int32_t n;
  int32_t fp4;
};

struct Params {
  const uint16_t* q;
  uint16_t* o;
  int64_t q_row;     // elements between query rows (H * D)
  int32_t H, nq, n_qblk, n_wg;
  DevSeg a, b;
  int32_t vis_mode, vT, vC, v_nsink, v_base, v_F, v_sink0;
  float c;           // softmax scale * log2(e)
  // split mode (direct kernel): nt key tiles per block, the first `main` of them on the
  // block's own workgroup, the rest spread over the n_self_wg - H * n_qblk spare workgroups
  int32_t split, nt, main;
  // fused cross-attention (direct kernel, mode 0): workgroups n_self_wg.. run whole blocks of
  // ox = softmax(scale qx K_x^T) V_x over the x segment
  int32_t n_self_wg;
  const uint16_t* qx;
  uint16_t* ox;
  DevSeg x;
  float* part;       // per-thread piece state: n_blocks main slots, then the tail slots
  uint32_t* cnt;     // per-block arrival counters, zero between launches
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Key limit of query row `row` (keys j < limit are visible). Frame ids fit 31 bits (the host
// rejects streams beyond that).
__device__ __forceinline__ int32_t row_limit(const Params& p, int32_t row) {
  if (p.vis_mode == 0) return p.a.n + p.b.n;
  const int32_t r = row / p.vT;
  const int32_t f = r < p.v_nsink ? p.v_sink0 + r : p.v_base + (r - p.v_nsink);
  const int32_t X = (f / p.vC + 1) * p.vC;
  const int32_t xs = X - p.v_sink0;
  const int32_t ns = xs < 0 ? 0 : (xs < p.v_nsink ? xs : p.v_nsink);
  const int32_t top = X < p.v_F ? X : p.v_F;
  const int32_t nr = top > p.v_base ? top - p.v_base : 0;
  return (ns + nr) * p.vT;
}

// FP4 -> bf16 for the 8 codes of one 32-bit word (element e in bits 4e..4e+3) with scale
// byte sb: value = (-1)^s * grid[code & 7] * 2^(sb-127), grid = {0,.5,1,1.5,2,3,4,6}, using
// gfx950's scaled fp4->bf16 conversion (exact: every such value is a bf16, subnormals
// included; every code byte at every scale byte the encoder produces, 0..252, is read back
// through this path and checked against the oracle, in both attention kernels).
__device__ __forceinline__ uint4 dequant8(uint32_t w, uint32_t sb) {
  const float scale = __uint_as_float(sb ? (sb << 23) : 0x00400000u);
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3)));
}

template <int D, int NW>
struct Cfg {
  static constexpr int NT = NW * 64;           // threads
  static constexpr int NDC = D / 8;            // 16-byte columns per key row
  static constexpr int NKG = NT / NDC;         // key groups per tile pass
  static constexpr int KPT = BN / NKG;         // keys per thread per tile
  static_assert(KPT == 1 || KPT == 2 || KPT == 4, "unsupported staging split");
  static constexpr int KP = D * 2 + 16;        // K row pitch: 16 bytes of padding per row
  static constexpr int K_BYTES = BN * KP;      // one K tile  [BN][D] (padded rows)
  static constexpr int VT_BYTES = D * BN * 2;  // one V^T tile [D][BN]
  static constexpr int BUF = K_BYTES + VT_BYTES;
  static constexpr int LDS = 2 * BUF;
};

// K rows are padded to D*2+16 bytes: 16 consecutive rows at the same column land on 16
// distinct 16-byte bank groups, and every read address is lane base + immediate.
template <int D>
__device__ __forceinline__ int k_off(int key, int c) {
  return key * (D * 2 + 16) + (c << 4);
}
// V^T rows (64 keys = 128 bytes) use an XOR swizzle of the 16-byte column by
// (d ^ d>>3) & 7, which keeps both the transposing writes and the column reads spread
// over the banks
__device__ __forceinline__ int vt_off(int d, int c) {
  return d * (BN * 2) + ((c ^ ((d ^ (d >> 3)) & 7)) << 4);
}
// position of key k inside its 16-key group in the V^T tile: 4-key quads 0,1,2,3 -> 0,2,1,3
__device__ __forceinline__ int vt_pos(int k) {
  const int a = (k >> 2) & 3;
  const int ap = ((a & 1) << 1) | (a >> 1);
  return (k & ~15) | (ap << 2) | (k & 3);
}

// Buffer resource over `bytes` bytes at `base`: loads at offsets >= bytes return zero, which
// is how keys past a segment's end (and the ragged tail) are read as zeros without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}

template <int D, int NW, bool FP4>
struct Stage {
  using C = Cfg<D, NW>;
  // per-head resources: segment A (cache, head-major; dense or fp4 planes) and segment B
  // (the call's own K/V, token-major)
  __amdgpu_buffer_rsrc_t ak, av, aks, avs, bk, bv;
  int32_t na, a_row, b_row;   // keys in A; row strides in bytes (fp4: packed bytes)
  uint4 kr[C::KPT], vr[C::KPT];
  uint32_t kw[C::KPT], vw[C::KPT], ksb[C::KPT], vsb[C::KPT];

  __device__ __forceinline__ void init(const Params& p, int h) {
    na = p.a.n;
    if (FP4) {
      a_row = int32_t(p.a.row_stride / 2);
      const int64_t e0 = h * p.a.head_stride;
      ak = rsrc(p.a.k + e0 / 2, uint32_t(p.a.n) * a_row);
      av = rsrc(p.a.v + e0 / 2, uint32_t(p.a.n) * a_row);
      aks = rsrc(p.a.ks + e0 / 16, uint32_t(p.a.n) * (a_row / 8));
      avs = rsrc(p.a.vs + e0 / 16, uint32_t(p.a.n) * (a_row / 8));
    } else {
      a_row = int32_t(p.a.row_stride * 2);
      const int64_t e0 = h * p.a.head_stride;
      ak = rsrc(p.a.k + e0 * 2, uint32_t(p.a.n) * a_row);
      av = rsrc(p.a.v + e0 * 2, uint32_t(p.a.n) * a_row);
    }
    b_row = int32_t(p.b.row_stride * 2);
    const uint32_t bbytes = p.b.n > 0 ? uint32_t(p.b.n - 1) * b_row + D * 2 : 0u;
    bk = rsrc(p.b.k + h * p.b.head_stride * 2, bbytes);
    bv = rsrc(p.b.v + h * p.b.head_stride * 2, bbytes);
  }

  __device__ __forceinline__ void load_a(int j0, int dc) {
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int j = j0 + i;
      if (FP4) {
        const uint32_t off = uint32_t(j) * a_row + dc * 4;
        kw[i] = __builtin_amdgcn_raw_buffer_load_b32(ak, off, 0, 0);
        vw[i] = __builtin_amdgcn_raw_buffer_load_b32(av, off, 0, 0);
        const uint32_t so = uint32_t(j) * (a_row / 8) + (dc >> 1);
        ksb[i] = __builtin_amdgcn_raw_buffer_load_b8(aks, so, 0, 0);
        vsb[i] = __builtin_amdgcn_raw_buffer_load_b8(avs, so, 0, 0);
      } else {
        const uint32_t off = uint32_t(j) * a_row + dc * 16;
        kr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ak, off, 0, 0));
        vr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(av, off, 0, 0));
      }
    }
  }

  // keys j0.. of segment B (j0 may be negative: those rows read as zero)
  __device__ __forceinline__ void load_b(int j0, int dc, bool accumulate) {
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const uint32_t off = uint32_t(j0 + i) * uint32_t(b_row) + dc * 16;
      const uint4 x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(bk, off, 0, 0));
      const uint4 y = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(bv, off, 0, 0));
      if (accumulate) {
        kr[i] = make_uint4(kr[i].x | x.x, kr[i].y | x.y, kr[i].z | x.z, kr[i].w | x.w);
        vr[i] = make_uint4(vr[i].x | y.x, vr[i].y | y.y, vr[i].z | y.z, vr[i].w | y.w);
      } else {
        kr[i] = x;
        vr[i] = y;
      }
    }
  }

  // stage tile `tile` into registers; `mixed` marks the one tile that straddles A and B
  __device__ __forceinline__ void load(int tile, int dc, int kg) {
    const int t0 = tile * BN;
    const int j0 = t0 + kg * C::KPT;
    if (t0 + BN <= na) {
      load_a(j0, dc);
    } else if (t0 >= na) {
      if (FP4) {
#pragma unroll
        for (int i = 0; i < C::KPT; ++i) kw[i] = vw[i] = ksb[i] = vsb[i] = 0;
      }
      load_b(j0 - na, dc, false);
    } else {
      load_a(j0, dc);
      if (FP4) {
#pragma unroll
        for (int i = 0; i < C::KPT; ++i) kr[i] = vr[i] = make_uint4(0, 0, 0, 0);
      }
      load_b(j0 - na, dc, !FP4);
      if (FP4) {
        // keys of A keep their codes, keys of B their bf16 values; mark B keys with sb 0xFFFF
#pragma unroll
        for (int i = 0; i < C::KPT; ++i)
          if (j0 + i >= na) ksb[i] = vsb[i] = 0xFFFFu;
      }
    }
  }

  __device__ __forceinline__ void store(uint8_t* buf, int tile, int dc, int kg) {
    uint8_t* kt = buf;
    uint8_t* vt = buf + C::K_BYTES;
    if (FP4) {
      const int t0 = tile * BN;
      if (t0 < na) {
#pragma unroll
        for (int i = 0; i < C::KPT; ++i) {
          if (ksb[i] != 0xFFFFu) {
            kr[i] = dequant8(kw[i], ksb[i]);
            vr[i] = dequant8(vw[i], vsb[i]);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int key = kg * C::KPT + i;
      *reinterpret_cast<uint4*>(kt + k_off<D>(key, dc)) = kr[i];
    }
    // V: transpose KPT keys x 8 dims in registers, write 8 rows of V^T
    const int pos = vt_pos(kg * C::KPT);
    const int col = pos >> 3, sub = (pos & 7) * 2;
    const uint32_t* w[C::KPT];
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) w[i] = reinterpret_cast<const uint32_t*>(&vr[i]);
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const int d = dc * 8 + dd;
      const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
      uint8_t* dst = vt + vt_off(d, col) + sub;
      if constexpr (C::KPT == 4) {
        uint2 x;
        x.x = __builtin_amdgcn_perm(w[1][dd >> 1], w[0][dd >> 1], sel);
        x.y = __builtin_amdgcn_perm(w[3][dd >> 1], w[2][dd >> 1], sel);
        *reinterpret_cast<uint2*>(dst) = x;
      } else if constexpr (C::KPT == 2) {
        *reinterpret_cast<uint32_t*>(dst) = __builtin_amdgcn_perm(w[1][dd >> 1], w[0][dd >> 1], sel);
      } else {
        const uint32_t x = w[0][dd >> 1];
        *reinterpret_cast<uint16_t*>(dst) = uint16_t((dd & 1) ? (x >> 16) : (x & 0xFFFF));
      }
    }
  }
};

// Online softmax of one 64-key tile for the lane's query row: S^T values s (2 x 16 per lane,
// masked keys already -inf) -> bf16 weights pb (the B operand of the PV product), updating the
// running max m (exp2 domain, scaled by c), the running sum l and, when the max moves, O.
// Lazy rescale: the weights are first taken against the running max as it stands. Each is at
// most the lane's sum of them, so while no lane's sum exceeds 2^8 the tile needs no rescale
// (softmax is shift-invariant; only rounding changes) and the tile max is never computed.
// Otherwise (the first tile, or scores well above the running max) the wave takes the tile
// max, rescales O and l and recomputes the weights. The row sum adds the bf16-rounded weights
// (v_dot2 with ones), exactly the weights the PV product uses.
template <int D>
__device__ __forceinline__ float tile_weights(const f32x16_t (&s)[2], float c, float m,
                                              bf16x8_t (&pb)[2][2]) {
  float psum[4] = {0.f, 0.f, 0.f, 0.f};
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    float e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -m));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u[i] = pack_bf16x2(e[8 * j + 2 * i], e[8 * j + 2 * i + 1]);
        psum[i] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u[i]), ones, psum[i], false);
      }
      pb[kb][j] = __builtin_bit_cast(bf16x8_t, make_uint4(u[0], u[1], u[2], u[3]));
    }
  }
  return (psum[0] + psum[1]) + (psum[2] + psum[3]);
}

template <int D>
__device__ __forceinline__ void softmax_update(f32x16_t (&s)[2], float c, float& m_run,
                                               float& l_run, f32x16_t (&oacc)[D / 32],
                                               bf16x8_t (&pb)[2][2]) {
  float ls = tile_weights<D>(s, c, m_run, pb);
  if (__builtin_amdgcn_ballot_w64(ls > kLazyBound)) {
    float t8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      t8[i] = fmaxf(fmaxf(s[0][2 * i], s[0][2 * i + 1]), fmaxf(s[1][2 * i], s[1][2 * i + 1]));
#pragma unroll
    for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w; ++i) t8[i] = fmaxf(t8[i], t8[i + w]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(t8[0]), __float_as_uint(t8[0]),
                                                     false, false);
    const float mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
    if (mt > m_run) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - mt);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
      m_run = mt;
    }
    ls = tile_weights<D>(s, c, m_run, pb);
  }
  l_run += ls;
}

template <int D, int NW, bool FP4>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bf16_kernel(Params p) {
  using C = Cfg<D, NW>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  // XCD-aware tile order: workgroup ids are dealt round-robin over the 8 XCDs; give each XCD
  // a contiguous range of tiles so neighbouring query blocks of a head share an L2.
  const int G = p.n_wg;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, idx = bid >> 3;
  const int qd = G >> 3, rm = G & 7;
  const int tile_id = (xcd < rm ? xcd * (qd + 1) : rm * (qd + 1) + (xcd - rm) * qd) + idx;
  // block-causal: heaviest block rank of every head first, in dispatch (workgroup id) order
  const int h = p.vis_mode == 1 ? int(blockIdx.x) % p.H : tile_id / p.n_qblk;
  const int qblk = p.n_qblk - 1 - (p.vis_mode == 1 ? int(blockIdx.x) / p.H : tile_id % p.n_qblk);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int row0 = qblk * (NW * 32);
  const int row = row0 + wave * 32 + l32;            // this lane's query row
  const int lrow = row < p.nq ? row : p.nq - 1;
  const int lim = row_limit(p, lrow);
  const int wave_first = min(row0 + wave * 32, p.nq - 1);
  const int wave_min_lim = row_limit(p, wave_first);
  const int kend = row_limit(p, min(row0 + NW * 32 - 1, p.nq - 1));
  const int ntiles = (kend + BN - 1) / BN;

  // Q^T as the MFMA B operand: lane (n = l32, khalf = hi) holds q[row][16s + 8hi .. +7]
  bf16x8_t qreg[D / 16];
  {
    const uint16_t* qp = p.q + int64_t(row < p.nq ? row : 0) * p.q_row + h * D + 8 * hi;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      uint4 x = row < p.nq ? *reinterpret_cast<const uint4*>(qp + 16 * s) : make_uint4(0, 0, 0, 0);
      qreg[s] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16_t{};
  float m_run = kNoMax;
  float l_run = 0.f;

  // per-lane LDS offsets (tile-invariant): K row l32 column hi; V^T row l32 at the four
  // (kb ^ db&1, j) column patterns
  const int k_lane = k_off<D>(l32, hi);
  int v_lane[4];
#pragma unroll
  for (int sel = 0; sel < 4; ++sel) v_lane[sel] = vt_off(l32, 4 * (sel >> 1) + 2 * (sel & 1) + hi);

  const int dc = tid % C::NDC, kg = tid / C::NDC;
  Stage<D, NW, FP4> st;
  st.init(p, h);
  st.load(0, dc, kg);
  st.store(smem, 0, dc, kg);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) st.load(t + 1, dc, kg);
    const uint8_t* kt = smem + (t & 1) * C::BUF;
    const uint8_t* vt = kt + C::K_BYTES;

    // S^T[key][query] for two 32-key blocks: lane reads K row kb*32 + l32, column 2ss + hi
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16_t{};
#pragma unroll
      for (int ss = 0; ss < D / 16; ++ss) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kt + k_lane + kb * 32 * C::KP + ss * 32);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ss], s[kb], 0, 0, 0);
      }
    }

    // mask keys beyond this row's limit (only on tiles that reach past the wave's smallest)
    const int key0 = t * BN;
    if (key0 + BN > wave_min_lim) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key >= lim) s[kb][r] = -__builtin_inff();
        }
    }

    bf16x8_t pb[2][2];
    softmax_update<D>(s, p.c, m_run, l_run, oacc, pb);

    // O^T[d][query] += V^T[d][key] P^T[key][query]; lane reads V^T row db*32 + l32 at
    // column 4kb + 2j + hi, whose swizzle depends on (kb ^ db&1, j): four lane bases
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int sel = ((kb ^ (db & 1)) << 1) | j;
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(vt + v_lane[sel] + db * 32 * (BN * 2));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][j], oacc[db], 0, 0, 0);
        }
    }

    if (t + 1 < ntiles) st.store(smem + ((t + 1) & 1) * C::BUF, t + 1, dc, kg);
    __syncthreads();
  }

  // epilogue: combine the two half-row sums, normalise, store bf16
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run),
                                                     false, false);
    l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (row < p.nq) {
    const float inv = 1.0f / l_run;
    uint16_t* op = p.o + int64_t(row) * p.q_row + h * D + 4 * hi;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 u;
        u.x = pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
        u.y = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(op + db * 32 + 8 * g) = u;
      }
  }
}

// ---------------------------------------------------------------------------------------
// Dense bf16, head_dim 128: K and V tiles go global -> LDS with gfx950's direct-to-LDS buffer
// loads (no staging registers, no transposing writes). V stays key-major in LDS; the V^T
// operand of the PV product is read with ds_read_b64_tr_b16, which, within each 16-lane
// group, hands lane i element j of the 4x4 blocks supplied by lanes 4j + i/4 -- so lanes
// pointing at V[k0 + s/4][d0 + 4(s%4)] receive V[k0 + j][d0 + i], the keys-in-registers
// layout the MFMA needs. Tiles are 64 rows x 256 bytes with XOR-swizzled 16-byte chunks:
//   K: chunk c of row r at c ^ (r & 15)       (16 consecutive rows at one c: distinct banks)
//   V: chunk c of row r at c ^ ((r & 3) << 2) (the 4 rows x 2 lane groups of one
//      transposing read land on 16 distinct chunks)
// One direct load writes 1 KB (4 rows) of a tile; lane i fills physical chunk i%16 of row
// i/16 and so fetches the logical chunk that the swizzle puts there. Each key segment (cache
// slots, then the call's own K/V) is tiled on its own; rows past a segment's end are read
// as zeros through the buffer resource's range check and masked.
// ---------------------------------------------------------------------------------------
constexpr int DT_ROW = 256;                 // bytes per key row (128 bf16)
// MFMA operand reads in flight ahead of the MFMA that uses them; scheduling-group masks of
// the AMDGPU backend (MFMA, LDS read)
constexpr int kPipe = 4;
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;
// cache-policy bits of a buffer access for the agent-scope (sc1) policy: the encoding an
// agent-scope atomic load or store of one word gets
constexpr int kSc1 = 16;
// s_waitcnt immediate for vmcnt <= 4 with expcnt and lgkmcnt at 0 (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt in 6:4, lgkmcnt in 11:8)
constexpr int kWaitVm4 = 0x0004;

// LDS plan of the direct kernel: SUB 64-key sub-tiles per barrier, K then V, double-buffered
template <int SUB>
struct DtCfg {
  static constexpr int ROWS = BN * SUB;
  static constexpr int TILE = ROWS * DT_ROW;   // one K or V tile
  static constexpr int BUF = 2 * TILE;
  static constexpr int LDS = 2 * BUF;
};

// Transposing LDS read (ds_read_b64_tr_b16). Reached through a restrict pointer, the call
// carries alias-scope metadata like a plain load does; without it the backend makes every
// such read wait for all direct-to-LDS loads in flight, including the next tile's, which
// writes the other buffer. The kernel orders its LDS buffers itself (wait + barrier before
// a loaded tile is read).
__device__ __forceinline__ v4i16_t lds_read_tr(const uint8_t* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)p);
}

// V^T operand i of the PV product (i = 4 db + 2 kb + j: head dims 32 db.., keys 32 kb + 16 j..)
// from a key-major V sub-tile at vt: two transposing reads of 4 key rows each
__device__ __forceinline__ bf16x8_t read_v_operand(const uint8_t* vt, const int (&vbase)[4], int i) {
  const int db = i / 4, kb = (i / 2) & 1, j = i & 1;
  const uint8_t* a0 = vt + vbase[db] + (kb * 32 + 16 * j) * DT_ROW;
  const v4i16_t lo = lds_read_tr(a0);
  const v4i16_t hi4 = lds_read_tr(a0 + 8 * DT_ROW);
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, 0, 0, 0);
}

// Work split. Plain: one workgroup per (head, query block), all of its key tiles. Split
// (when there are fewer blocks than CUs): workgroup b < n_blocks runs block b's first
// `main` key tiles, so the query blocks of a head still sweep the keys in step and share
// them in L2; the remaining n_blocks x (nt - main) "tail" units (one key tile of one block
// each), block-major, are cut into equal contiguous ranges over the spare workgroups. A
// split block is finished by the last of its workgroups to arrive: each writes its
// unnormalised state (O, running max, running sum) to a workspace slot and bumps the
// block's counter; the one that sees the count complete merges the slots (main piece
// first, then the tail pieces in range order) and stores O. No workgroup ever waits on
// another.
// A piece's state in its workspace slot. Wide form (the dense chunk-attention instantiation):
// thread t's 64 O values as 16 groups of 4 (group g at byte (g * threads + t) * 16), then its
// running max and sum as one 8-byte pair (at byte 16 * 16 * threads + 8 t), so publishing and
// merging move 16-byte and 8-byte words (12-head chunk attention 2.5% faster than one word per
// access). Word form (FP4 and fused cross-attention instantiations, where the wide form was
// 1-2% slower, by code placement: their tile loops are unchanged): value r of thread t at word
// r * threads + t. A launch runs one instantiation, so its pieces share one form.
template <int NW>
struct SplitState {
  static constexpr int REGS = 66;               // 64 O values, running max, running sum
  static constexpr int SLOT_FLOATS = REGS * NW * 64;
  static constexpr int ML_OFFSET = 16 * 16 * NW * 64;   // bytes before the (max, sum) pairs
  static_assert(NW != 8 || SLOT_FLOATS * 4 == kSplitSlotBytes, "slot size");
};

// first unit of range g, and the range holding unit u, for U units over G ranges
__device__ __forceinline__ int64_t range_start(int64_t g, int64_t U, int64_t G) { return g * U / G; }
__device__ __forceinline__ int64_t range_of(int64_t u, int64_t U, int64_t G) { return ((u + 1) * G - 1) / U; }

template <int NW, int SUB, bool FP4, bool CROSS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_direct_kernel(Params p) {
  constexpr int D = 128;
  using T = DtCfg<SUB>;
  using SS = SplitState<NW>;
  constexpr bool kWideState = !FP4 && !CROSS;   // piece-state form (SplitState)
  constexpr int DT_TILE = T::TILE, DT_BUF = T::BUF, DT_LDS = T::LDS, TR = T::ROWS;
  constexpr int IPW = DT_TILE / 1024 / NW;  // direct loads per wave per tensor per tile
  static_assert(IPW * NW * 1024 == DT_TILE, "tile must split evenly over the waves");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_last;

  // XCD-aware order: workgroup ids are dealt round-robin over the 8 XCDs; each XCD gets a
  // contiguous range of logical ids, so the query blocks of one head share an L2. Under the
  // split schedule each XCD instead gets its proportional share of the main pieces (a
  // contiguous range of blocks) and of the spare workgroups, whose block-major tail ranges
  // then cover that XCD's own blocks: the tail tiles stay in the L2 that serves them, and no
  // XCD carries more main pieces than in a whole-block launch.
  // (ids from n_self_wg on are the fused cross-attention workgroups: they keep their ids, so
  // they are dispatched after every self-attention workgroup)
  const int G = p.n_wg;
  const int bid = blockIdx.x;
  int g = bid;
  if (bid < p.n_self_wg) {
    const int xcd = bid & 7, idx = bid >> 3;
    const int qd = p.n_self_wg >> 3, rm = p.n_self_wg & 7;
    const int pre0 = xcd * qd + min(xcd, rm);   // ids dealt to the XCDs before this one
    g = pre0 + idx;
    if (p.split) {
      const int nb = p.H * p.n_qblk;
      const int pre1 = pre0 + qd + (xcd < rm ? 1 : 0);
      const int m0 = int(int64_t(pre0) * nb / p.n_self_wg);
      const int m1 = int(int64_t(pre1) * nb / p.n_self_wg);
      g = idx < m1 - m0 ? m0 + idx : nb + (pre0 - m0) + (idx - (m1 - m0));
    }
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // LDS read lane bases. K (A operand of S^T = K Q^T): row kb*32 + l32, logical chunk
  // 2ss + hi -> one base per ss. V (A operand of O^T = V^T P^T, via the transposing read):
  // lane s of a 16-lane group points at row k0 + s/4, column db*32 + 16g + 4(s%4); the
  // swizzle XORs db's two bits, so four bases.
  int kbase[D / 16];
#pragma unroll
  for (int ss = 0; ss < D / 16; ++ss) kbase[ss] = l32 * DT_ROW + (((2 * ss + hi) ^ (l32 & 15)) << 4);
  int vbase[4];
  {
    const int sl = lane & 15, g1 = (lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int c = 4 * db + 2 * g1 + ((sl >> 1) & 1);
      vbase[db] = (4 * hi + (sl >> 2)) * DT_ROW + ((c ^ ((sl >> 2) << 2)) << 4) + 8 * (sl & 1);
    }
  }

  // direct-load lane offsets inside a tile: instruction n of this wave fills rows
  // (wave*IPW + n)*4 + lane/16, physical chunk lane%16
  int lrow[IPW], ck[IPW], cv[IPW];
#pragma unroll
  for (int n = 0; n < IPW; ++n) {
    lrow[n] = (wave * IPW + n) * 4 + (lane >> 4);
    ck[n] = (lane & 15) ^ (lrow[n] & 15);
    cv[n] = (lane & 15) ^ ((lrow[n] & 3) << 2);
  }

  // zero both buffers once, so rows that a range-checked load skips never hold non-finite bits
  for (int i = tid; i < DT_LDS / 16; i += NW * 64) reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  // split mode: tail units and spare workgroups
  const int nblk = p.H * p.n_qblk;
  const int tail = p.nt - p.main;
  const int64_t UT = int64_t(nblk) * tail;
  const int GSELF = p.n_self_wg;
  const int GS = GSELF - nblk;
  const bool xwg = CROSS && g >= GSELF;        // a fused cross-attention workgroup
  const bool spare = !xwg && p.split && g >= nblk;
  const int64_t u0 = spare ? range_start(g - nblk, UT, GS) : 0;
  const int64_t u1 = spare ? range_start(g - nblk + 1, UT, GS) : 0;
  int64_t u = u0;
  // cross workgroups: an equal contiguous range of whole cross blocks each
  const int GX = G - GSELF;
  int bx = xwg ? int(range_start(g - GSELF, nblk, GX)) : 0;
  const int bx1 = xwg ? int(range_start(g - GSELF + 1, nblk, GX)) : 0;
  bool single_done = false;

  for (;;) {
    // ---- next piece: block (h, qblk), key tiles [t0, t1) ----
    int h, qblk, t0, t1, blk = 0, slot = 0;
    bool whole, xjob = false;
    if (xwg) {
      if (bx >= bx1) break;
      blk = bx++;
      h = blk / p.n_qblk;
      qblk = blk - h * p.n_qblk;
      t0 = 0;
      t1 = -1;
      whole = true;
      xjob = true;
    } else if (spare) {
      if (u >= u1) break;
      blk = int(u / tail);
      t0 = int(u - int64_t(blk) * tail);
      t1 = p.main + int(min<int64_t>(tail, t0 + (u1 - u)));
      t0 += p.main;
      h = blk / p.n_qblk;
      qblk = blk - h * p.n_qblk;
      whole = false;
      // tail piece (spare s, block b) -> slot n_blocks + s + b: along the unit order s and b
      // never decrease and one of them grows at every new piece, so the slots are distinct
      slot = g + blk;
      u += t1 - t0;
    } else if (p.split) {
      if (single_done) break;
      single_done = true;
      blk = g;
      h = blk / p.n_qblk;
      qblk = blk - h * p.n_qblk;
      t0 = 0;
      t1 = p.main;
      whole = false;
      slot = blk;
    } else {
      if (single_done) break;
      single_done = true;
      if (p.vis_mode == 1) {
        // block-causal: later query blocks see more keys. Dispatch order is the workgroup id,
        // so the heaviest block rank of every head goes first (longest job first over the
        // whole grid), spread round-robin over the XCDs
        h = bid % p.H;
        qblk = p.n_qblk - 1 - bid / p.H;
      } else {
        h = g / p.n_qblk;
        qblk = p.n_qblk - 1 - (g % p.n_qblk);
      }
      t0 = 0;
      t1 = -1;  // all of the block's tiles, set below
      whole = true;
    }

    // the piece's key segments: self = (cache, own chunk), cross = (x, none)
    // (selected field by field: a runtime-selected reference to a kernel-argument struct
    // would make the compiler copy the arguments to scratch memory)
    const uint8_t* const sa_k = xjob ? p.x.k : p.a.k;
    const uint8_t* const sa_v = xjob ? p.x.v : p.a.v;
    const int64_t sa_hs = xjob ? p.x.head_stride : p.a.head_stride;
    const int64_t sa_rs = xjob ? p.x.row_stride : p.a.row_stride;
    const int na = xjob ? p.x.n : p.a.n;
    const int nb = xjob ? 0 : p.b.n;
    const int row0 = qblk * (NW * 32);
    const int row = row0 + wave * 32 + l32;
    const int lim = xjob ? na : row_limit(p, row < p.nq ? row : p.nq - 1);
    const bool wave_live = row0 + wave * 32 < p.nq;   // uniform over the wave
    const int wave_min_lim = xjob ? na : row_limit(p, min(row0 + wave * 32, p.nq - 1));
    const int kend = xjob ? na : row_limit(p, min(row0 + NW * 32 - 1, p.nq - 1));
    // tiles per segment; in block-causal mode only segment A holds keys and the last visible
    // key of the block bounds the loop
    const int ntA = ((p.vis_mode == 0 ? na : min(na, kend)) + TR - 1) / TR;
    const int ntB = p.vis_mode == 0 ? (nb + TR - 1) / TR : 0;
    if (t1 < 0) t1 = ntA + ntB;
    const bool fp4a = FP4 && !xjob;          // segment A of this piece is the FP4 cache

    bf16x8_t qreg[D / 16];
    {
      const uint16_t* qp = (xjob ? p.qx : p.q) + int64_t(row < p.nq ? row : 0) * p.q_row + h * D + 8 * hi;
#pragma unroll
      for (int ss = 0; ss < D / 16; ++ss) {
        const uint4 x = row < p.nq ? *reinterpret_cast<const uint4*>(qp + 16 * ss) : make_uint4(0, 0, 0, 0);
        qreg[ss] = __builtin_bit_cast(bf16x8_t, x);
      }
    }
    f32x16_t oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16_t{};
    float m_run = kNoMax;
    float l_run = 0.f;

    // FP4 cache tiles (segment A under FP4) are staged through registers instead: thread
    // tid holds row tid/4, elements 32*(tid%4).. of the tile -- 16 packed bytes and 2 scale
    // bytes per tensor -- and dequant_half() writes K or V as bf16 into the same swizzled
    // layout the direct loads produce. The loads of an FP4 tile go out a whole tile ahead of
    // its dequantisation (load_fp4), so the conversions find their data in registers.
    uint4 kq = make_uint4(0, 0, 0, 0), vq = make_uint4(0, 0, 0, 0);
    uint32_t kqs = 0, vqs = 0;
    const int fr = tid >> 2, fq = tid & 3;
    auto fp4_tile = [&](int t) { return fp4a && t < ntA; };
    auto dequant_half = [&](uint8_t* buf, int v_off, int row_mask, bool k_half) {
      const int rsw = k_half ? (fr & 15) : ((fr & 3) << 2);
      const uint4 q4 = k_half ? kq : vq;
      const uint32_t qs = k_half ? kqs : vqs;
      const uint32_t w[4] = {q4.x, q4.y, q4.z, q4.w};
      uint8_t* dst = buf + (k_half ? 0 : v_off) + (fr & row_mask) * DT_ROW;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int lc = 4 * fq + c;                            // logical 16-byte chunk (8 elements)
        *reinterpret_cast<uint4*>(dst + ((lc ^ rsw) << 4)) = dequant8(w[c], (qs >> (8 * (c >> 1))) & 0xFF);
      }
    };
    auto load_fp4 = [&](int t, bool k_half) {
      const int r0 = t * TR;
      const int64_t e0 = h * p.a.head_stride + int64_t(r0) * p.a.row_stride;
      const int left = p.a.n - r0;
      const uint32_t pbytes = left > 0 ? uint32_t(left) * (D / 2) : 0u;
      const __amdgpu_buffer_rsrc_t rc = rsrc((k_half ? p.a.k : p.a.v) + e0 / 2, pbytes);
      const __amdgpu_buffer_rsrc_t rs = rsrc((k_half ? p.a.ks : p.a.vs) + e0 / 16, pbytes / 8);
      const uint4 x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, uint32_t(fr) * (D / 2) + fq * 16, 0, 0));
      const uint32_t s = __builtin_amdgcn_raw_buffer_load_b16(rs, uint32_t(fr) * (D / 16) + fq * 2, 0, 0);
      if (k_half) {
        kq = x;
        kqs = s;
      } else {
        vq = x;
        vqs = s;
      }
    };
    // wait for this wave's direct loads of the next tile; when the FP4 loads of the tile after
    // it are already in flight (only possible with no direct load outstanding: FP4 tiles come
    // first) they are the last 4 and are left running
    auto wait_tile = [&](bool fp4_ahead) {
      if (fp4_ahead) __builtin_amdgcn_s_waitcnt(kWaitVm4);
      else __builtin_amdgcn_s_waitcnt(0);
    };

    auto issue = [&](int t, uint8_t* buf) {
      const bool inA = t < ntA;
      if constexpr (FP4) {
        if (inA && fp4a) return;   // FP4 tiles come through registers, loaded ahead
      }
      const int r0 = (inA ? t : t - ntA) * TR;                  // first row of the tile in the segment
      const int64_t rp = (inA ? sa_rs : p.b.row_stride) * 2;     // row pitch in bytes
      const int64_t hs = inA ? sa_hs : p.b.head_stride;
      const uint8_t* kb0 = (inA ? sa_k : p.b.k) + (h * hs) * 2 + int64_t(r0) * rp;
      const uint8_t* vb0 = (inA ? sa_v : p.b.v) + (h * hs) * 2 + int64_t(r0) * rp;
      const int left = (inA ? na : nb) - r0;                     // rows of this segment from r0 on
      const uint32_t bytes = left > 0 ? uint32_t(left - 1) * uint32_t(rp) + DT_ROW : 0u;
      const __amdgpu_buffer_rsrc_t rk = rsrc(kb0, bytes), rv = rsrc(vb0, bytes);
#pragma unroll
      for (int n = 0; n < IPW; ++n) {
        const uint32_t ro = uint32_t(lrow[n]) * uint32_t(rp);
        lds_load16(rk, buf + (wave * IPW + n) * 1024, ro + (ck[n] << 4));
        lds_load16(rv, buf + DT_TILE + (wave * IPW + n) * 1024, ro + (cv[n] << 4));
      }
    };

    if (FP4 && fp4_tile(t0)) {
      load_fp4(t0, true);
      load_fp4(t0, false);
      dequant_half(smem + (t0 & 1) * DT_BUF, DT_TILE, TR - 1, true);
      dequant_half(smem + (t0 & 1) * DT_BUF, DT_TILE, TR - 1, false);
    } else {
      issue(t0, smem + (t0 & 1) * DT_BUF);
    }
    const bool ahead0 = FP4 && t0 + 1 < t1 && fp4_tile(t0 + 1);
    if (ahead0) {
      load_fp4(t0 + 1, true);
      load_fp4(t0 + 1, false);
    }
    wait_tile(ahead0);
    __syncthreads();

    for (int t = t0; t < t1; ++t) {
      if (t + 1 < t1) issue(t + 1, smem + ((t + 1) & 1) * DT_BUF);
#pragma unroll
      for (int u2 = 0; u2 < SUB; ++u2) {
      const uint8_t* kt = smem + (t & 1) * DT_BUF + u2 * BN * DT_ROW;
      const uint8_t* vt = kt + DT_TILE;

      const bool inA = t < ntA;
      const int r0 = (inA ? t : t - ntA) * TR + u2 * BN;       // first row of the sub-tile
      const int seg_left = (inA ? na : nb) - r0;
      // a sub-tile wholly past the end is skipped, and so is all the work of a wave whose 32
      // rows lie past the last query row (the ragged last block of a head: 3 of its 8 waves
      // hold rows at the layer shape); such a wave still issues its share of every tile's
      // loads and meets every barrier. (FP4: computed fully masked instead, so every sub-tile
      // reaches its share of the next tile's dequantisation and the loads after it.)
      if (!FP4 && (seg_left <= 0 || !wave_live)) continue;
      const int key0 = (inA ? 0 : na) + r0;

      // S^T = K Q^T: 16 MFMAs, each fed by one 16-byte LDS read. The reads run kPipe MFMAs
      // ahead of their use (pinned by the scheduling groups below), so the LDS latency hides
      // behind the matrix pipe instead of stalling every MFMA.
      // Wave priority: raised for the MFMA blocks, lowered for the softmax (and the FP4
      // dequantisation), so that of the two waves sharing a SIMD the one with MFMAs to issue
      // wins and the other's VALU work fills the matrix pipe's shadow; that pulls the pair
      // out of phase.
      __builtin_amdgcn_s_setprio(1);
      f32x16_t s[2];
      s[0] = f32x16_t{};
      s[1] = f32x16_t{};
      {
        constexpr int NS = 2 * (D / 16);
        bf16x8_t ka[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i)
          ka[i] = *reinterpret_cast<const bf16x8_t*>(kt + kbase[i % (D / 16)] + (i / (D / 16)) * 32 * DT_ROW);
#pragma unroll
        for (int i = 0; i < NS; ++i)
          s[i / (D / 16)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i], qreg[i % (D / 16)],
                                                                   s[i / (D / 16)], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kPipe, 0);
#pragma unroll
        for (int i = 0; i < NS - kPipe; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, kPipe, 0);
      }
      // Dense tiles: the V operands of the first kPipe PV MFMAs are read right after the QK
      // MFMAs, so they land during the softmax and the PV block starts on an MFMA instead of
      // an LDS wait (16 more registers; the FP4 instantiation has none to spare).
      constexpr bool kVEarly = !FP4;
      bf16x8_t va_early[kPipe];
      if constexpr (kVEarly) {
#pragma unroll
        for (int i = 0; i < kPipe; ++i) va_early[i] = read_v_operand(vt, vbase, i);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kPipe, 0);
      }

      // mask: rows past the segment's end, and keys past this row's block-causal limit
      if (seg_left < BN || key0 + BN > wave_min_lim) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kr = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (kr >= seg_left || key0 + kr >= lim) s[kb][r] = -__builtin_inff();
          }
      }

      bf16x8_t pb[2][2];
      __builtin_amdgcn_s_setprio(0);
      softmax_update<D>(s, p.c, m_run, l_run, oacc, pb);
      if constexpr (FP4) {
        // next tile's FP4 data (loaded a tile ahead) -> bf16 at low priority, next to the
        // softmax: K in the first sub-tile, V in the last; the freed registers then take the
        // loads of the tile after. When the next tile is not FP4 (or past the piece) the
        // stores go to a 16 KB scratch area above the two buffers instead (K and V rows folded
        // onto 64 rows), so no branch is needed
        if (u2 == 0 || u2 == SUB - 1) {
          const bool k_half = u2 == 0;
          const bool real = t + 1 < t1 && fp4_tile(t + 1);
          dequant_half(real ? smem + ((t + 1) & 1) * DT_BUF : smem + 2 * DT_BUF,
                       real ? DT_TILE : 0, real ? TR - 1 : BN - 1, k_half);
          if (t + 2 < t1 && fp4_tile(t + 2)) load_fp4(t + 2, k_half);
        }
      }
      __builtin_amdgcn_s_setprio(1);

      // O^T += V^T P^T: 16 MFMAs, each fed by two transposing LDS reads, pipelined like S
      {
        constexpr int NP = (D / 32) * 4;
        bf16x8_t va[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) va[i] = kVEarly && i < kPipe ? va_early[i] : read_v_operand(vt, vbase, i);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const int db = i / 4, kb = (i / 2) & 1, j = i & 1;
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pb[kb][j], oacc[db], 0, 0, 0);
        }
        if (!kVEarly) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kPipe, 0);
#pragma unroll
        for (int i = 0; i < NP - kPipe; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, kPipe, 0);
      }
      __builtin_amdgcn_s_setprio(0);
      }

      wait_tile(FP4 && t + 2 < t1 && fp4_tile(t + 2));   // this wave's direct loads of tile t+1 have landed
      __syncthreads();
    }

    if (!whole) {
      // ---- split block: publish this piece, and merge if it is the block's last ----
      // The piece state is stored and read back with agent-scope (L2-coherent) accesses, and
      // the counter bump is preceded by one release fence (write-back of dirty L2 lines): no
      // acquire fence, whose L2 invalidation would evict the K/V every other workgroup on
      // the XCD is reusing. The merging workgroup reads only after an atomic on the counter
      // returned the completing count.
      const int64_t bu0 = int64_t(blk) * tail;                   // the block's first tail unit
      const int gs_first = int(range_of(bu0, UT, GS));
      const int gs_last = int(range_of(bu0 + tail - 1, UT, GS));
      const int n_tail_pieces = gs_last - gs_first + 1;
      // The main piece first looks at the counter: when every tail piece has already arrived
      // (the usual case when the spare workgroups have less work than a main piece), it
      // merges the tails into its own registers and never publishes its state, which saves
      // the write and read-back of one slot per block at the end of the launch.
      bool from_regs = false;
      if (!spare) {
        if (tid == 0) {
          const uint32_t c = __hip_atomic_load(p.cnt + blk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const int done = int(c) == n_tail_pieces;
          if (done) __hip_atomic_store(p.cnt + blk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          s_last = done;
        }
        __syncthreads();
        from_regs = s_last != 0;
        __syncthreads();   // s_last is written again below
      }
      if (!from_regs) {
        if constexpr (kWideState) {
          const __amdgpu_buffer_rsrc_t wpart = rsrc(p.part, 0xFFFFFFFFu);
          const uint32_t sbase = uint32_t(int64_t(slot) * SS::SLOT_FLOATS * 4);
          // 16-byte and 8-byte buffer stores with the agent-scope (sc1) policy, the encoding
          // an agent-scope atomic store of one word gets
#pragma unroll
          for (int g = 0; g < 16; ++g) {
            const f32x16_t& o = oacc[g >> 2];
            const int i = 4 * (g & 3);
            const v4f32_t w = {o[i], o[i + 1], o[i + 2], o[i + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32_t, w), wpart,
                                                   sbase + uint32_t((g * NW * 64 + tid) * 16), 0, kSc1);
          }
          const v2f32_t ml = {m_run, l_run};
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u32_t, ml), wpart,
                                                sbase + uint32_t(SS::ML_OFFSET + tid * 8), 0, kSc1);
        } else {
          float* sp = p.part + int64_t(slot) * SS::SLOT_FLOATS + wave * 64 + lane;
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              __hip_atomic_store(sp + (db * 16 + i) * NW * 64, oacc[db][i], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(sp + 64 * NW * 64, m_run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(sp + 65 * NW * 64, l_run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __builtin_amdgcn_s_waitcnt(0);   // this thread's stores are complete
        __syncthreads();
        if (tid == 0) {
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
          const uint32_t old = __hip_atomic_fetch_add(p.cnt + blk, 1u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
          const int last = int(old) == n_tail_pieces;   // main piece + tail pieces - 1
          if (last) __hip_atomic_store(p.cnt + blk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          s_last = last;
        }
        __syncthreads();
        if (!s_last) continue;
      }
      // merge: the main piece, then the tail pieces in range order (the result does not
      // depend on which workgroup merges: starting from the main piece's registers is the
      // same arithmetic as loading it first into a zero state), online: the sum is rescaled
      // whenever a piece brings a larger running max. Reads use 16-byte and 8-byte buffer
      // loads with the agent-scope (sc1) cache policy, the encoding of an agent-scope atomic
      // load; as plain loads they may be issued back to back. A piece's 66 values (17 loads)
      // are in registers before any is used (scheduling barrier): left to itself, the compiler
      // waited after every load in the FP4 instantiation, whose registers run at the limit,
      // and a merge of many pieces then took hundreds of microseconds.
      const __amdgpu_buffer_rsrc_t rpart = rsrc(p.part, 0xFFFFFFFFu);
      float m_all = m_run;
      if (!from_regs) {
        m_all = kNoMax;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16_t{};
        l_run = 0.f;
      }
      for (int gs = from_regs ? gs_first : gs_first - 1; gs <= gs_last; ++gs) {
        const int sl = gs < gs_first ? blk : nblk + gs + blk;
        float b[SS::REGS];
        if constexpr (kWideState) {
          const uint32_t base = uint32_t(int64_t(sl) * SS::SLOT_FLOATS * 4);
#pragma unroll
          for (int g = 0; g < 16; ++g) {
            const v4f32_t w = __builtin_bit_cast(v4f32_t, __builtin_amdgcn_raw_buffer_load_b128(
                rpart, base + uint32_t((g * NW * 64 + tid) * 16), 0, kSc1));
#pragma unroll
            for (int i = 0; i < 4; ++i) b[4 * g + i] = w[i];
          }
          const v2f32_t ml = __builtin_bit_cast(v2f32_t, __builtin_amdgcn_raw_buffer_load_b64(
              rpart, base + uint32_t(SS::ML_OFFSET + tid * 8), 0, kSc1));
          b[64] = ml[0];
          b[65] = ml[1];
        } else {
          const uint32_t base = uint32_t((int64_t(sl) * SS::SLOT_FLOATS + wave * 64 + lane) * 4);
#pragma unroll
          for (int r = 0; r < SS::REGS; ++r)
            b[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rpart, base + r * NW * 64 * 4, 0, kSc1));
        }
        __builtin_amdgcn_sched_barrier(0);
        const float m_p = b[64];
        if (m_p > m_all) {   // this piece raises the lane's running max: rescale the sum
          const float a = __builtin_amdgcn_exp2f(m_all - m_p);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) oacc[db] *= a;
          l_run *= a;
          m_all = m_p;
        }
        const float f = m_p == m_all ? 1.0f : __builtin_amdgcn_exp2f(m_p - m_all);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] += b[db * 16 + i] * f;
        l_run += b[65] * f;
      }
      m_run = m_all;
    }

    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run),
                                                       false, false);
      l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (row < p.nq) {
      const float inv = 1.0f / l_run;
      uint16_t* op = (xjob ? p.ox : p.o) + int64_t(row) * p.q_row + h * D + 4 * hi;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          uint2 v2;
          v2.x = pack_bf16x2(oacc[db][4 * gq + 0] * inv, oacc[db][4 * gq + 1] * inv);
          v2.y = pack_bf16x2(oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv);
          *reinterpret_cast<uint2*>(op + db * 32 + 8 * gq) = v2;
        }
    }
  }
}

// One flag per device and kernel: the dynamic-LDS limit is a per-device attribute of the
// kernel, so it is raised once on every device the kernel is launched on.
struct DeviceFlags {
  static constexpr int kMax = 64;
  std::atomic<bool> set[kMax] = {};
};

int allow_lds(const void* kern, int bytes, DeviceFlags& flags, char* err) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    snprintf(err, 256, "no current device");
    return 1;
  }
  if (dev < DeviceFlags::kMax && flags.set[dev].load(std::memory_order_acquire)) return 0;
  if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess) {
    snprintf(err, 256, "cannot set %d bytes of LDS", bytes);
    return 1;
  }
  if (dev < DeviceFlags::kMax) flags.set[dev].store(true, std::memory_order_release);
  return 0;
}

template <int NW, int SUB, bool FP4, bool CROSS>
int launch_direct(const Params& p, int grid, hipStream_t stream, char* err) {
  auto kern = attn_bf16_direct_kernel<NW, SUB, FP4, CROSS>;
  constexpr int DT_LDS = DtCfg<SUB>::LDS + (FP4 ? BN * DT_ROW : 0);
  static DeviceFlags attr_set;
  if (int r = allow_lds(reinterpret_cast<const void*>(kern), DT_LDS, attr_set, err)) return r;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), DT_LDS, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(err, 256, "%s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

template <int D, int NW, bool FP4>
int launch_t(const Params& p, int grid, hipStream_t stream, char* err) {
  using C = Cfg<D, NW>;
  auto kern = attn_bf16_kernel<D, NW, FP4>;
  static DeviceFlags attr_set;
  if (int r = allow_lds(reinterpret_cast<const void*>(kern), C::LDS, attr_set, err)) return r;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), C::LDS, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(err, 256, "%s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

}  // namespace

// ---- the static split-schedule workspace (no allocation on the caller's side) ----
// One copy per device, resident while the library is loaded: 256 KB of arrival counters and
// 512 piece-state slots of 135,168 bytes (69.5 MB in all), enough for the split schedule of
// any call on a device of up to 256 compute units.
static __device__ __align__(256) uint8_t scratch[kStaticWsBytes];
static_assert(kStaticWsCounters * 4 == 256 * 1024, "counter region size");

namespace {
struct StaticWs {
  static constexpr int kMaxDevices = 64;
  std::mutex mu;
  void* ptr[kMaxDevices] = {};
};
StaticWs g_static_ws;
}  // namespace

int static_workspace(void** ptr, void* stream, char* err) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= StaticWs::kMaxDevices) {
    snprintf(err, 256, "no usable current device for the static workspace");
    return 1;
  }
  std::lock_guard<std::mutex> lock(g_static_ws.mu);
  if (!g_static_ws.ptr[dev]) {
    // the symbol's device address on this device (the array's name is only a host-side
    // stand-in); then clear the counters once, with a kernel: every split launch leaves the
    // counters it used at zero again
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      snprintf(err, 256, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      return 1;
    }
    if (int r = launch_zero(p, kStaticWsCounters * 4, stream, err)) return r;
    g_static_ws.ptr[dev] = p;
  }
  *ptr = g_static_ws.ptr[dev];
  return 0;
}

int launch_attention_bf16(const AttnArgs& a, void* stream, char* err) {
  constexpr int NW = 4;
  Params p{};
  p.q = static_cast<const uint16_t*>(a.q);
  p.o = static_cast<uint16_t*>(a.o);
  p.q_row = int64_t(a.H) * a.D;
  p.H = a.H;
  p.nq = a.nq;
  auto seg = [](const KeySeg& s) {
    DevSeg d{};
    d.k = static_cast<const uint8_t*>(s.k);
    d.v = static_cast<const uint8_t*>(s.v);
    d.ks = s.k_scales;
    d.vs = s.v_scales;
    d.head_stride = s.head_stride;
    d.row_stride = s.row_stride;
    d.n = s.n;
    d.fp4 = s.fp4;
    return d;
  };
  p.a = seg(a.seg[0]);
  p.b = seg(a.seg[1]);
  if (p.b.fp4) {
    snprintf(err, 256, "only the first key segment may be FP4");
    return 1;
  }
  p.vis_mode = a.vis.mode;
  p.vT = a.vis.T;
  p.vC = a.vis.C;
  p.v_nsink = a.vis.n_sink;
  p.v_base = int32_t(a.vis.base);
  p.v_F = int32_t(a.vis.F);
  p.v_sink0 = int32_t(a.vis.sink0);
  p.c = a.scale * 1.4426950408889634f;
  if (a.nq <= 0) return 0;
  if (p.a.n + p.b.n <= 0) {
    snprintf(err, 256, "attention over zero keys");
    return 1;
  }
  p.n_qblk = (a.nq + NW * 32 - 1) / (NW * 32);
  p.n_wg = p.n_qblk * a.H;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fp4 = p.a.fp4 != 0;
  if (a.D == 128) {
    // 8 waves x 32 rows per workgroup, 128 keys per barrier, 2 workgroup waves per SIMD;
    // dense tiles come in by direct-to-LDS loads, FP4 cache tiles through registers with the
    // dequantisation fused into the LDS write
    constexpr int DNW = 8, DSUB = 2, TR = DtCfg<DSUB>::ROWS;
    static_assert(DNW * 32 == kSplitRows && TR == kSplitKeys, "split workspace geometry");
    p.n_qblk = (a.nq + DNW * 32 - 1) / (DNW * 32);
    const int blocks = p.n_qblk * a.H;
    p.n_wg = blocks;
    const bool cross = a.qx != nullptr && a.x.n > 0;
    if (cross && a.x.fp4) {
      snprintf(err, 256, "fused cross-attention needs bf16 text keys");
      return 1;
    }
    if (cross && fp4) {
      // the FP4 kernel is built without cross blocks (fewer live scalar registers): the self
      // part, then the cross part as a dense launch
      AttnArgs self = a;
      self.qx = nullptr;
      self.ox = nullptr;
      self.x = KeySeg{};
      if (int r = launch_attention_bf16(self, stream, err)) return r;
      AttnArgs cx = self;
      cx.q = a.qx;
      cx.o = a.ox;
      cx.seg[0] = a.x;
      cx.seg[1] = a.x;
      cx.seg[1].n = 0;
      cx.ws = nullptr;
      return launch_attention_bf16(cx, stream, err);
    }
    if (a.vis.mode == 0 && a.ws && a.n_cu > blocks && blocks <= a.ws_blocks) {
      // Split when the best main/tail cut is shorter than one whole block. Cost in key
      // tiles, with kPieceCost tiles per piece for its prologue (Q load, first tile not
      // overlapped) and its publish (a spare workgroup runs at most ceil(span/tail) + 1
      // pieces), and kMergeCost per piece the merging workgroup reads. The model's best cut
      // matches the measured best on MI355X at 1 to 12 heads x 4680 rows (at 12 heads, 228
      // blocks: main 168 of 184 tiles, 3% faster than whole blocks; it predicts 5%, since
      // the 28 extra busy CUs lower the sustained clock). The decision ignores fused
      // cross-attention blocks, so the self part of a fused launch runs the same schedule
      // (and gives the same bits) as a plain chunk call.
      constexpr int64_t kPieceCost = 4, kMergeCost = 1;
      const int nt = (p.a.n + TR - 1) / TR + (p.b.n + TR - 1) / TR;
      const int64_t spare = a.n_cu - blocks;
      // best cut (main tiles) and its predicted time, with piece_cost tiles per piece
      auto plan = [&](int64_t piece_cost, int& best_main, int64_t& best) {
        best_main = nt;
        best = nt;
        for (int m = 1; m < nt; ++m) {
          const int64_t tail = nt - m;
          const int64_t ut = int64_t(blocks) * tail;
          const int64_t gs = ut < spare ? ut : spare;
          const int64_t span = (ut + gs - 1) / gs;
          const int64_t c_main = m + piece_cost;
          const int64_t c_spare = span + piece_cost * ((span + tail - 1) / tail + 1);
          // the last workgroup of a block then reads every piece of it (main + tails)
          const int64_t merge = kMergeCost * ((tail + span - 1) / span + 2);
          const int64_t mk = (c_main > c_spare ? c_main : c_spare) + merge;
          if (mk < best) {
            best = mk;
            best_main = m;
          }
        }
      };
      int best_main;
      int64_t best;
      plan(kPieceCost, best_main, best);
      // An FP4 piece starts by loading and decoding its first tile before anything overlaps,
      // so when an FP4 call has at most a quarter as many blocks as CUs its cut is placed with
      // 6 tiles per piece (a longer main piece, fewer tail tiles): 2-6% faster than the dense
      // cut at 3 heads x 4680 rows (two A/B runs), the same at 1 and 2 heads; at 6 and 12
      // heads it was 1-2% slower, so there the dense cut stays. Whether to split is decided
      // with the dense cost.
      if (fp4 && 4 * int64_t(blocks) <= a.n_cu && best_main < nt && best * 100 < int64_t(nt) * 97) {
        int fp4_main;
        int64_t fp4_best;
        plan(6, fp4_main, fp4_best);
        if (fp4_main < nt) best_main = fp4_main;
      }
      const int64_t ut = int64_t(blocks) * (nt - best_main);
      const int64_t gs = ut < spare ? ut : spare;
      if (best_main < nt && best * 100 < int64_t(nt) * 97 && 2 * (blocks + gs) <= a.ws_slots) {
        uint8_t* ws = static_cast<uint8_t*>(a.ws);
        p.split = 1;
        p.nt = nt;
        p.main = best_main;
        p.n_wg = int(blocks + gs);
        p.cnt = reinterpret_cast<uint32_t*>(ws);
        p.part = reinterpret_cast<float*>(ws + split_slots_offset(a.ws_blocks));
      }
    }
    p.n_self_wg = p.n_wg;
    if (cross) {
      // cross blocks go to the CUs the self-attention leaves idle (several blocks each), or,
      // when there are none, to one extra workgroup per block
      const int idle = a.n_cu > p.n_self_wg ? a.n_cu - p.n_self_wg : 0;
      p.n_wg = p.n_self_wg + (idle > 0 ? (idle < blocks ? idle : blocks) : blocks);
      p.qx = static_cast<const uint16_t*>(a.qx);
      p.ox = static_cast<uint16_t*>(a.ox);
      p.x = seg(a.x);
    }
    // cross blocks only exist in their own instantiation, so the common kernels carry no
    // cross fields or per-piece segment selection
    if (cross) return launch_direct<DNW, DSUB, false, true>(p, p.n_wg, s, err);
    return fp4 ? launch_direct<DNW, DSUB, true, false>(p, p.n_wg, s, err)
               : launch_direct<DNW, DSUB, false, false>(p, p.n_wg, s, err);
  }
  if (a.D == 64) {
    return fp4 ? launch_t<64, NW, true>(p, p.n_wg, s, err) : launch_t<64, NW, false>(p, p.n_wg, s, err);
  }
  snprintf(err, 256, "head_dim %d", a.D);
  return 1;
}

}  // namespace ll
