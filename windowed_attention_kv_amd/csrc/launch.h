// Internal interface between the C-ABI host layer (ll_host.cpp) and the kernel launchers.
// Plain C++ structs with no HIP types, so the host layer also builds against a recording
// backend (fake_launch.cpp) for CPU-only tests of its validation and slot arithmetic.
#pragma once

#include <cstdint>

namespace ll {

// One key segment of an attention call. Key j of head h lives at
//   dense: base + h * head_stride + j * row_stride        (elements of the call dtype)
//   fp4  : packed + (h * head_stride + j * row_stride) / 2 bytes,
//          scales + (h * head_stride + j * row_stride) / 16 bytes
struct KeySeg {
  const void* k = nullptr;
  const void* v = nullptr;
  const uint8_t* k_scales = nullptr;  // fp4 only
  const uint8_t* v_scales = nullptr;  // fp4 only
  int64_t head_stride = 0;
  int64_t row_stride = 0;
  int32_t n = 0;                      // keys in the segment
  int32_t fp4 = 0;
};

// Visibility of keys to query row i (keys are indexed across seg[0] then seg[1]):
//   mode 0: every key is visible;
//   mode 1 (block-causal over held frames): row i is in the held frame of rank r = i / T,
//     frame fr(r) = r < n_sink ? sink0 + r : base + (r - n_sink) (the held sink frames
//     sink0.. come first, then the window frames base..F-1, all ascending); with
//     X = (fr / C + 1) * C the key limit is
//     T * (clamp(X - sink0, 0, n_sink) + max(0, min(F, X) - base)); keys j < limit are visible.
struct Visibility {
  int32_t mode = 0;
  int32_t T = 0, C = 0, n_sink = 0;
  int64_t base = 0, F = 0, sink0 = 0;
};

struct AttnArgs {
  int32_t dtype = 0;        // 0 f32, 1 bf16
  int32_t H = 0, D = 0;
  const void* q = nullptr;  // [nq, H, D] token-major
  void* o = nullptr;        // [nq, H, D]
  int32_t nq = 0;
  KeySeg seg[2];
  Visibility vis;
  float scale = 0.f;
  // optional workspace for the split (stream-K) schedule of mode-0 calls: ws_blocks 32-bit
  // arrival counters (zero between launches), then ws_slots piece-state slots of
  // kSplitSlotBytes each, from byte split_slots_offset(ws_blocks)
  void* ws = nullptr;
  int32_t ws_blocks = 0, ws_slots = 0;
  int32_t n_cu = 0;         // compute units of the device
  // optional cross-attention of the same launch: ox = softmax(scale qx K_x^T) V_x over all of
  // segment x (never masked), for the same nq rows and heads; fused into the head_dim-128
  // bf16 kernel, a second launch otherwise
  const void* qx = nullptr;
  void* ox = nullptr;
  KeySeg x;
};

// bytes of one piece-state slot of the split schedule: 66 floats per thread of an 8-wave
// workgroup (64 O values, running max, running sum)
constexpr int64_t kSplitSlotBytes = int64_t(66) * 8 * 64 * 4;
// query rows and key rows per unit of the split schedule (head_dim 128, bf16)
constexpr int32_t kSplitRows = 256, kSplitKeys = 128;
inline int64_t split_slots_offset(int64_t ws_blocks) { return (ws_blocks * 4 + 255) / 256 * 256; }

// Copy (or FP4-quantise) frames of a [n_frames*T, H, D] token-major K/V pair into cache
// slots. Source frame r goes to slot slot_of_rank(r):
//   r < n_lead ? lead_slot0 + r : ring_base + (first_ring + r - n_lead) mod W
// (the lead frames are sink frames in sink slots, the rest go to the window slots). For
// r in [spill_lo, spill_hi) the destination slot's old contents are first moved to slot
// spill_slot0 + (r - spill_lo) (a sink frame leaving the window).
struct ScatterArgs {
  int32_t dtype = 0;
  int32_t fp4 = 0;
  int32_t H = 0, D = 0, T = 0;
  int32_t n_frames = 0;
  int32_t n_lead = 0, lead_slot0 = 0;
  int32_t ring_base = 0, W = 0;
  int64_t first_ring = 0;   // frame id of the first non-lead frame (window slot = id mod W)
  int32_t spill_lo = 0, spill_hi = 0, spill_slot0 = 0;
  const void* k_src = nullptr;
  const void* v_src = nullptr;
  // destination: head-major planes [H][slots*T][D] (dense) or packed/scales (fp4)
  void* k_dst = nullptr;
  void* v_dst = nullptr;
  uint8_t* k_dst_scales = nullptr;
  uint8_t* v_dst_scales = nullptr;
  int32_t slots = 0;
};

// One layer of a batched commit: the chunk's K/V (token-major, C frames) go to window slots
// (first_ring + r) mod W, r = 0..C-1; for r in [spill_lo, spill_hi) the destination slot's
// old contents first move to slot spill_slot0 + (r - spill_lo) (a sink frame leaving the
// window), as in ScatterArgs.
struct CommitLayer {
  const void* k_src = nullptr;
  const void* v_src = nullptr;
  void* k_dst = nullptr;             // head-major planes [H][slots*T][D] (dense) or packed (fp4)
  void* v_dst = nullptr;
  uint8_t* k_dst_scales = nullptr;   // fp4 only
  uint8_t* v_dst_scales = nullptr;
  int64_t first_ring = 0;            // frame id of the chunk's first frame
  int32_t spill_lo = 0, spill_hi = 0, spill_slot0 = 0;
};

// Commit of one chunk into n_layers layers of the same geometry in one launch per
// kMaxCommitLayers layers (the per-layer table travels in the kernel arguments).
constexpr int kMaxCommitLayers = 32;
struct CommitLayersArgs {
  int32_t dtype = 0, fp4 = 0;
  int32_t H = 0, D = 0, T = 0, C = 0, W = 0, slots = 0;
  int32_t n_layers = 0;
  const CommitLayer* layers = nullptr;   // host array of n_layers entries
};

struct QuantArgs {
  const void* x = nullptr;
  int64_t rows = 0;
  int32_t row_len = 0;
  uint8_t* packed = nullptr;
  uint8_t* scales = nullptr;
};

// Export head-major cache planes into slot-order token-major arrays.
struct ExportArgs {
  int32_t dtype = 0, fp4 = 0;
  int32_t H = 0, D = 0, T = 0, slots = 0;
  const void* k_src = nullptr;
  const void* v_src = nullptr;
  const uint8_t* k_src_scales = nullptr;
  const uint8_t* v_src_scales = nullptr;
  void* k_out = nullptr;
  void* v_out = nullptr;
  uint8_t* k_out_scales = nullptr;
  uint8_t* v_out_scales = nullptr;
};

// The library's own split-schedule workspace, for callers that cannot allocate: a static
// device array of kStaticWsBytes holding kStaticWsCounters 32-bit arrival counters (a
// kStaticWsCounters * 4-byte region, as split_slots_offset lays it out) and then
// kStaticWsSlots piece-state slots. static_workspace() returns its address on the current
// device (looked up once per device) and, the first time on a device, clears its counters with
// a kernel on `stream`.
constexpr int64_t kStaticWsCounters = 65536;
constexpr int64_t kStaticWsSlots = 512;
constexpr int64_t kStaticWsBytes = kStaticWsCounters * 4 + kStaticWsSlots * kSplitSlotBytes;
int static_workspace(void** ptr, void* stream, char* err);

// Each launcher returns 0 on success or a nonzero code, with a message in `err`
// (at least 256 bytes).
int launch_attention(const AttnArgs& a, void* stream, char* err);
int launch_scatter(const ScatterArgs& a, void* stream, char* err);
int launch_commit_layers(const CommitLayersArgs& a, void* stream, char* err);
int launch_quant(const QuantArgs& a, void* stream, char* err);
int launch_export(const ExportArgs& a, void* stream, char* err);
// zero `bytes` (a multiple of 4) at p with a kernel on the stream
int launch_zero(void* p, int64_t bytes, void* stream, char* err);
// compute units of the current device (0 if it cannot be queried)
int device_cu_count();

}  // namespace ll
