// C-ABI host layer: descriptor validation, device-memory layout, per-layer ring metadata and
// kernel launch plumbing. Nothing here touches device memory; every device operation is an
// enqueue through launch.h.
//
// Cache model ("LongLive" summary page, 方法 §3 高效长推理): each layer holds W window slots
// that rotate and S sink slots after them, so its size depends only on S + W. Frame f enters
// window slot f mod W; a sink frame of the current shot moves to its sink slot when the
// window evicts it (slot rules at n_spilled below). The held frames always fill a slot prefix,
// which is what lets one attention kernel read the cache as a single contiguous key range per
// head.
//
// Device memory layout (per layer, K then V; each plane 256-byte aligned):
//   dense: [H][(S+W)*T][D] elements of the dtype (head-major, so one head's keys are contiguous)
//   fp4  : packed [H][(S+W)*T][D/2] bytes, then scales [H][(S+W)*T][D/16] bytes
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/ll.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

ll_status fail(ll_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ll_status fail(ll_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

ll_status ok() {
  g_err[0] = 0;
  return LL_OK;
}

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t k_off, v_off, ks_off, vs_off;  // byte offsets inside one layer
  size_t layer_bytes;
  // workspace of the split attention schedule, after the last layer (bf16 head_dim 128,
  // dense or FP4 store): arrival counters for every (head, query block) of a chunk call, then two
  // piece-state slots per workgroup of the largest split launch
  size_t ws_bytes;
  int32_t ws_blocks, ws_slots;
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

ll_status check_desc(const ll_cache_desc* d) {
  if (!d) return fail(LL_EINVAL, "desc is NULL");
  if (d->abi_version != LL_ABI_VERSION)
    return fail(LL_EINVAL, "abi_version %u, library is %u", d->abi_version, LL_ABI_VERSION);
  if (d->num_layers < 1 || d->num_layers > 4096) return fail(LL_EINVAL, "num_layers %d", d->num_layers);
  if (d->num_heads < 1 || d->num_heads > 1024) return fail(LL_EINVAL, "num_heads %d", d->num_heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(LL_EUNSUPPORTED, "head_dim %d (64 or 128)", d->head_dim);
  if (d->tokens_per_frame < 1) return fail(LL_EINVAL, "tokens_per_frame %d", d->tokens_per_frame);
  if (d->chunk_frames < 1) return fail(LL_EINVAL, "chunk_frames %d", d->chunk_frames);
  if (d->sink_frames < 0) return fail(LL_EINVAL, "sink_frames %d", d->sink_frames);
  if (d->window_frames < 1) return fail(LL_EINVAL, "window_frames %d", d->window_frames);
  if (d->window_frames < d->chunk_frames)
    return fail(LL_EUNSUPPORTED, "window_frames %d < chunk_frames %d", d->window_frames,
                d->chunk_frames);
  if (d->dtype != LL_F32 && d->dtype != LL_BF16) return fail(LL_EINVAL, "dtype %d", d->dtype);
  if (d->kv_format != LL_KV_DENSE && d->kv_format != LL_KV_FP4)
    return fail(LL_EINVAL, "kv_format %d", d->kv_format);
  if (d->kv_format == LL_KV_FP4 && d->dtype != LL_BF16)
    return fail(LL_EUNSUPPORTED, "the FP4 KV store needs bf16 tensors");
  // key indices and per-head element offsets must fit the kernels' 32-bit key counters
  const int64_t slots = int64_t(d->sink_frames) + d->window_frames;
  const int64_t cache_keys = slots * d->tokens_per_frame;
  const int64_t own_keys = int64_t(d->chunk_frames) * d->tokens_per_frame;
  if (slots > 4096 || cache_keys + own_keys > (int64_t(1) << 30))
    return fail(LL_EINVAL, "too many keys per head (%lld cache + %lld chunk)",
                (long long)cache_keys, (long long)own_keys);
  // the kernels address one head's cache plane, and any [rows, H, D] tensor of up to
  // (S+W)*T rows, with 32-bit byte offsets
  const int64_t es = d->dtype == LL_BF16 ? 2 : 4;
  const int64_t row_bytes = int64_t(d->num_heads) * d->head_dim * es;
  if (cache_keys * row_bytes >= (int64_t(1) << 31) || own_keys * row_bytes >= (int64_t(1) << 31))
    return fail(LL_EUNSUPPORTED, "tensors of %lld rows x %lld bytes exceed 2 GiB",
                (long long)std::max(cache_keys, own_keys), (long long)row_bytes);
  if (!(d->softmax_scale <= 0.f) && !std::isfinite(d->softmax_scale))
    return fail(LL_EINVAL, "softmax_scale is not finite");
  return LL_OK;
}

Layout layout_of(const ll_cache_desc* d, int n_cu) {
  const size_t slots = size_t(d->sink_frames) + d->window_frames;
  const size_t elems = slots * d->tokens_per_frame * d->num_heads * d->head_dim;
  Layout L{};
  if (d->kv_format == LL_KV_FP4) {
    const size_t pk = round_up(elems / 2), sc = round_up(elems / 16);
    L.k_off = 0;
    L.ks_off = pk;
    L.v_off = pk + sc;
    L.vs_off = 2 * pk + sc;
    L.layer_bytes = 2 * (pk + sc);
  } else {
    const size_t es = d->dtype == LL_BF16 ? 2 : 4;
    const size_t pl = round_up(elems * es);
    L.k_off = 0;
    L.v_off = pl;
    L.ks_off = L.vs_off = 0;
    L.layer_bytes = 2 * pl;
  }
  L.ws_bytes = 0;
  L.ws_blocks = L.ws_slots = 0;
  if (d->dtype == LL_BF16 && d->head_dim == 128 && n_cu > 0) {
    const int64_t n = int64_t(d->chunk_frames) * d->tokens_per_frame;
    const int64_t blocks = int64_t(d->num_heads) * ((n + ll::kSplitRows - 1) / ll::kSplitRows);
    const int64_t nt = (int64_t(slots) * d->tokens_per_frame + ll::kSplitKeys - 1) / ll::kSplitKeys +
                       (n + ll::kSplitKeys - 1) / ll::kSplitKeys;
    const int64_t G = std::min<int64_t>(n_cu, blocks * nt);
    L.ws_blocks = int32_t(blocks);
    L.ws_slots = int32_t(2 * G);
    L.ws_bytes = size_t(ll::split_slots_offset(blocks) + 2 * G * ll::kSplitSlotBytes);
  }
  return L;
}

size_t total_bytes(const ll_cache_desc* d, const Layout& L) {
  return L.layer_bytes * size_t(d->num_layers) + L.ws_bytes;
}

}  // namespace

struct ll_cache {
  ll_cache_desc d;
  Layout L;
  uint8_t* mem;
  size_t bytes;
  float scale;
  int n_cu;
  bool ws_ready;                // split-schedule counters zeroed (on the calls' stream)
  std::vector<int64_t> frames;  // frames committed per layer
  std::vector<int64_t> shot;    // first frame of the current shot per layer
};

namespace {

int32_t slots_of(const ll_cache* c) { return c->d.sink_frames + c->d.window_frames; }

// Slot layout: W window slots, then S sink slots. Frame f enters window slot f mod W; a sink
// frame of the current shot (first frame B) moves to sink slot W + (f - B) when the window
// evicts it. Held frames: the spilled sink frames B..B+k-1, then the window frames
// max(0, F-W)..F-1; their slots are the prefix [0, min(F, W) + k).
int64_t n_spilled(int64_t F, int64_t S, int64_t W, int64_t B) {
  return std::min<int64_t>(std::max<int64_t>(F - W - B, 0), S);
}
int64_t window_base(int64_t F, int64_t W) { return F > W ? F - W : 0; }
int64_t held_count(int64_t F, int64_t S, int64_t W, int64_t B) {
  return std::min<int64_t>(F, W) + n_spilled(F, S, W, B);
}

uint8_t* plane(const ll_cache* c, int layer, size_t off) {
  return c->mem + size_t(layer) * c->L.layer_bytes + off;
}

ll_status check_layer(const ll_cache* c, int32_t layer) {
  if (!c) return fail(LL_EINVAL, "cache handle is NULL");
  if (layer < 0 || layer >= c->d.num_layers)
    return fail(LL_EINVAL, "layer %d out of range [0, %d)", layer, c->d.num_layers);
  return LL_OK;
}

ll_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(LL_EINVAL, "%s is NULL", name);
  if (!aligned(p, 16)) return fail(LL_EINVAL, "%s is not 16-byte aligned", name);
  return LL_OK;
}

ll_status device_status(int rc, const char* what, const char* msg) {
  if (rc == 0) return LL_OK;
  return fail(LL_EDEVICE, "%s: %s", what, msg);
}

// Key segment over the cache's filled slot prefix of one layer.
ll::KeySeg cache_segment(const ll_cache* c, int32_t layer) {
  const ll_cache_desc& d = c->d;
  const int64_t nvalid = held_count(c->frames[layer], d.sink_frames, d.window_frames, c->shot[layer]);
  ll::KeySeg s;
  s.k = plane(c, layer, c->L.k_off);
  s.v = plane(c, layer, c->L.v_off);
  s.fp4 = d.kv_format == LL_KV_FP4;
  if (s.fp4) {
    s.k_scales = plane(c, layer, c->L.ks_off);
    s.v_scales = plane(c, layer, c->L.vs_off);
  }
  s.head_stride = int64_t(slots_of(c)) * d.tokens_per_frame * d.head_dim;
  s.row_stride = d.head_dim;
  s.n = int32_t(nvalid * d.tokens_per_frame);
  return s;
}

ll::KeySeg input_segment(const ll_cache_desc& d, const void* k, const void* v, int32_t n) {
  ll::KeySeg s;
  s.k = k;
  s.v = v;
  s.head_stride = d.head_dim;
  s.row_stride = int64_t(d.num_heads) * d.head_dim;
  s.n = n;
  return s;
}

ll::ScatterArgs scatter_base(const ll_cache* c, int32_t layer) {
  const ll_cache_desc& d = c->d;
  ll::ScatterArgs a;
  a.dtype = d.dtype;
  a.fp4 = d.kv_format == LL_KV_FP4;
  a.H = d.num_heads;
  a.D = d.head_dim;
  a.T = d.tokens_per_frame;
  a.ring_base = 0;
  a.W = d.window_frames;
  a.slots = slots_of(c);
  a.k_dst = plane(c, layer, c->L.k_off);
  a.v_dst = plane(c, layer, c->L.v_off);
  if (a.fp4) {
    a.k_dst_scales = plane(c, layer, c->L.ks_off);
    a.v_dst_scales = plane(c, layer, c->L.vs_off);
  }
  return a;
}

// Validation shared by the single-layer and batched commits.
ll_status check_commit(const ll_cache* cache, int32_t layer, const void* k, const void* v) {
  if (ll_status s = check_layer(cache, layer)) return s;
  if (ll_status s = check_ptr(k, "k")) return s;
  if (ll_status s = check_ptr(v, "v")) return s;
  const int64_t F = cache->frames[layer];
  if (F + cache->d.chunk_frames >= (int64_t(1) << 31) - 1)
    return fail(LL_ESTATE, "layer %d has committed %lld frames: frame ids must fit 31 bits", layer,
                (long long)F);
  return LL_OK;
}

// Where the next chunk of `layer` goes: frame F+r (r < C) enters window slot (F+r) mod W and
// evicts frame e = F+r-W (C <= W, so e < F); a sink frame of the current shot (B <= e < B+S)
// moves to sink slot W + (e - B) first.
ll::CommitLayer commit_plan(const ll_cache* c, int32_t layer, const void* k, const void* v) {
  const ll_cache_desc& d = c->d;
  const int64_t F = c->frames[layer];
  const int64_t S = d.sink_frames, C = d.chunk_frames, W = d.window_frames, B = c->shot[layer];
  ll::CommitLayer p;
  p.k_src = k;
  p.v_src = v;
  p.k_dst = plane(c, layer, c->L.k_off);
  p.v_dst = plane(c, layer, c->L.v_off);
  if (d.kv_format == LL_KV_FP4) {
    p.k_dst_scales = plane(c, layer, c->L.ks_off);
    p.v_dst_scales = plane(c, layer, c->L.vs_off);
  }
  p.first_ring = F;
  const int64_t lo = std::max<int64_t>(0, B + W - F);
  const int64_t hi = std::min<int64_t>(C, B + S + W - F);
  if (lo < hi) {
    p.spill_lo = int32_t(lo);
    p.spill_hi = int32_t(hi);
    p.spill_slot0 = int32_t(W + (F + lo - W - B));
  }
  return p;
}

}  // namespace

extern "C" {

ll_status ll_cache_size(const ll_cache_desc* desc, size_t* device_bytes) {
  if (ll_status s = check_desc(desc)) return s;
  if (!device_bytes) return fail(LL_EINVAL, "device_bytes is NULL");
  *device_bytes = total_bytes(desc, layout_of(desc, ll::device_cu_count()));
  return ok();
}

ll_status ll_cache_create(const ll_cache_desc* desc, void* device_mem, size_t device_bytes,
                          ll_cache** out) {
  if (ll_status s = check_desc(desc)) return s;
  if (!out) return fail(LL_EINVAL, "out is NULL");
  if (!device_mem) return fail(LL_EINVAL, "device_mem is NULL");
  if (!aligned(device_mem, kAlign)) return fail(LL_EINVAL, "device_mem is not 256-byte aligned");
  const int n_cu = ll::device_cu_count();
  const Layout L = layout_of(desc, n_cu);
  const size_t need = total_bytes(desc, L);
  if (device_bytes < need)
    return fail(LL_EINVAL, "device_bytes %zu < required %zu", device_bytes, need);
  ll_cache* c = new (std::nothrow) ll_cache;
  if (!c) return fail(LL_EINVAL, "out of host memory");
  c->d = *desc;
  c->L = L;
  c->mem = static_cast<uint8_t*>(device_mem);
  c->bytes = device_bytes;
  c->scale = desc->softmax_scale > 0.f ? desc->softmax_scale
                                       : float(1.0 / std::sqrt(double(desc->head_dim)));
  c->n_cu = n_cu;
  c->ws_ready = false;
  try {
    c->frames.assign(size_t(desc->num_layers), 0);
    c->shot.assign(size_t(desc->num_layers), 0);
  } catch (...) {  // no exception crosses the C ABI
    delete c;
    return fail(LL_EINVAL, "out of host memory");
  }
  *out = c;
  return ok();
}

ll_status ll_cache_destroy(ll_cache* cache) {
  delete cache;
  return ok();
}

ll_status ll_cache_reset(ll_cache* cache) {
  if (!cache) return fail(LL_EINVAL, "cache handle is NULL");
  std::fill(cache->frames.begin(), cache->frames.end(), 0);
  std::fill(cache->shot.begin(), cache->shot.end(), 0);
  return ok();
}

ll_status ll_cache_new_shot(ll_cache* cache, int32_t layer) {
  if (ll_status s = check_layer(cache, layer)) return s;
  cache->shot[layer] = cache->frames[layer];
  return ok();
}

}  // extern "C"

namespace {

// chunk attention, optionally with the fused text cross-attention (qx != nullptr); with
// static_ws the split schedule's workspace is the library's static device array instead of
// the cache's own
ll_status attn_chunk_impl(ll_cache* cache, int32_t layer, const void* q, const void* k,
                          const void* v, void* o, const void* qx, const void* k_text,
                          const void* v_text, int32_t n_text, void* ox, void* stream,
                          bool static_ws = false) {
  if (ll_status s = check_layer(cache, layer)) return s;
  if (ll_status s = check_ptr(q, "q")) return s;
  if (ll_status s = check_ptr(k, "k")) return s;
  if (ll_status s = check_ptr(v, "v")) return s;
  if (ll_status s = check_ptr(o, "o")) return s;
  const ll_cache_desc& d = cache->d;
  if (qx) {
    if (ll_status s = check_ptr(k_text, "k_text")) return s;
    if (ll_status s = check_ptr(v_text, "v_text")) return s;
    if (ll_status s = check_ptr(ox, "ox")) return s;
    if (n_text < 1 || int64_t(n_text) * d.num_heads * d.head_dim * (d.dtype == LL_BF16 ? 2 : 4) >=
                          (int64_t(1) << 31))
      return fail(LL_EINVAL, "n_text %d", n_text);
  }
  const int32_t n = d.chunk_frames * d.tokens_per_frame;
  ll::AttnArgs a;
  a.dtype = d.dtype;
  a.H = d.num_heads;
  a.D = d.head_dim;
  a.q = q;
  a.o = o;
  a.nq = n;
  a.seg[0] = cache_segment(cache, layer);
  a.seg[1] = input_segment(d, k, v, n);
  a.scale = cache->scale;
  char msg[256] = "";
  if (cache->L.ws_bytes && static_ws) {
    if (cache->L.ws_blocks > ll::kStaticWsCounters || cache->L.ws_slots > ll::kStaticWsSlots)
      return fail(LL_EINVAL,
                  "the split schedule of this cache needs %d counters and %d piece slots; the "
                  "static workspace holds %lld and %lld", cache->L.ws_blocks, cache->L.ws_slots,
                  (long long)ll::kStaticWsCounters, (long long)ll::kStaticWsSlots);
    void* ws = nullptr;
    if (ll_status s = device_status(ll::static_workspace(&ws, stream, msg), "static workspace", msg))
      return s;
    a.ws = ws;
    a.ws_blocks = int32_t(ll::kStaticWsCounters);
    a.ws_slots = int32_t(ll::kStaticWsSlots);
  } else if (cache->L.ws_bytes) {
    uint8_t* ws = cache->mem + cache->L.layer_bytes * size_t(d.num_layers);
    if (!cache->ws_ready) {
      if (ll_status s = device_status(
              ll::launch_zero(ws, ll::split_slots_offset(cache->L.ws_blocks), stream, msg),
              "workspace init", msg))
        return s;
      cache->ws_ready = true;
    }
    a.ws = ws;
    a.ws_blocks = cache->L.ws_blocks;
    a.ws_slots = cache->L.ws_slots;
  }
  a.n_cu = cache->n_cu;
  if (qx) {
    a.qx = qx;
    a.ox = ox;
    a.x = input_segment(d, k_text, v_text, n_text);
  }
  return device_status(ll::launch_attention(a, stream, msg), "attention launch", msg) ?: ok();
}

}  // namespace

extern "C" {

ll_status ll_attn_chunk(ll_cache* cache, int32_t layer, const void* q, const void* k,
                        const void* v, void* o, void* stream) {
  return attn_chunk_impl(cache, layer, q, k, v, o, nullptr, nullptr, nullptr, 0, nullptr, stream);
}

ll_status ll_attn_chunk_noalloc(ll_cache* cache, int32_t layer, const void* q, const void* k,
                                const void* v, void* o, void* stream) {
  return attn_chunk_impl(cache, layer, q, k, v, o, nullptr, nullptr, nullptr, 0, nullptr, stream,
                         true);
}

ll_status ll_attn_chunk_cross(ll_cache* cache, int32_t layer, const void* q, const void* k,
                              const void* v, const void* qx, const void* k_text,
                              const void* v_text, int32_t n_text, void* o, void* ox,
                              void* stream) {
  if (!qx) return fail(LL_EINVAL, "qx is NULL");
  return attn_chunk_impl(cache, layer, q, k, v, o, qx, k_text, v_text, n_text, ox, stream);
}

ll_status ll_cache_commit(ll_cache* cache, int32_t layer, const void* k, const void* v,
                          void* stream) {
  if (ll_status s = check_commit(cache, layer, k, v)) return s;
  const ll::CommitLayer c = commit_plan(cache, layer, k, v);
  ll::ScatterArgs a = scatter_base(cache, layer);
  a.n_frames = cache->d.chunk_frames;
  a.n_lead = 0;
  a.first_ring = c.first_ring;
  a.spill_lo = c.spill_lo;
  a.spill_hi = c.spill_hi;
  a.spill_slot0 = c.spill_slot0;
  a.k_src = k;
  a.v_src = v;
  char msg[256] = "";
  if (ll_status s = device_status(ll::launch_scatter(a, stream, msg), "commit launch", msg))
    return s;
  cache->frames[layer] += cache->d.chunk_frames;
  return ok();
}

ll_status ll_cache_commit_layers(ll_cache* cache, int32_t first_layer, int32_t n_layers,
                                 const void* const* k, const void* const* v, void* stream) {
  if (!cache) return fail(LL_EINVAL, "cache handle is NULL");
  if (!k || !v) return fail(LL_EINVAL, "k/v pointer array is NULL");
  if (n_layers < 1 || first_layer < 0 || first_layer >= cache->d.num_layers ||
      n_layers > cache->d.num_layers - first_layer)
    return fail(LL_EINVAL, "layers [%d, %d + %d) out of range [0, %d)", first_layer, first_layer,
                n_layers, cache->d.num_layers);
  for (int32_t i = 0; i < n_layers; ++i)
    if (ll_status s = check_commit(cache, first_layer + i, k[i], v[i])) return s;
  std::vector<ll::CommitLayer> plan;
  try {
    plan.reserve(size_t(n_layers));
  } catch (...) {  // no exception crosses the C ABI
    return fail(LL_EINVAL, "out of host memory");
  }
  for (int32_t i = 0; i < n_layers; ++i) plan.push_back(commit_plan(cache, first_layer + i, k[i], v[i]));
  const ll_cache_desc& d = cache->d;
  ll::CommitLayersArgs a;
  a.dtype = d.dtype;
  a.fp4 = d.kv_format == LL_KV_FP4;
  a.H = d.num_heads;
  a.D = d.head_dim;
  a.T = d.tokens_per_frame;
  a.C = d.chunk_frames;
  a.W = d.window_frames;
  a.slots = slots_of(cache);
  a.n_layers = n_layers;
  a.layers = plan.data();
  char msg[256] = "";
  if (ll_status s = device_status(ll::launch_commit_layers(a, stream, msg), "commit launch", msg))
    return s;
  for (int32_t i = 0; i < n_layers; ++i) cache->frames[first_layer + i] += d.chunk_frames;
  return ok();
}

ll_status ll_recache(ll_cache* cache, int32_t layer, const void* q, const void* k,
                     const void* v, const void* qx, const void* k_text, const void* v_text,
                     int32_t n_text, void* o, void* ox, void* stream) {
  if (ll_status s = check_layer(cache, layer)) return s;
  const char* names[] = {"q", "k", "v", "qx", "k_text", "v_text", "o", "ox"};
  const void* ptrs[] = {q, k, v, qx, k_text, v_text, o, ox};
  for (int i = 0; i < 8; ++i)
    if (ll_status s = check_ptr(ptrs[i], names[i])) return s;
  if (n_text < 1 || int64_t(n_text) * cache->d.num_heads * cache->d.head_dim *
                           (cache->d.dtype == LL_BF16 ? 2 : 4) >= (int64_t(1) << 31))
    return fail(LL_EINVAL, "n_text %d", n_text);
  const ll_cache_desc& d = cache->d;
  const int64_t F = cache->frames[layer];
  const int64_t S = d.sink_frames, W = d.window_frames;
  const int64_t B = cache->shot[layer];
  const int64_t held = held_count(F, S, W, B);
  if (held == 0) return fail(LL_ESTATE, "recache of layer %d, which holds no frame", layer);
  const int64_t nsink = n_spilled(F, S, W, B), base = window_base(F, W);
  const int32_t n = int32_t(held * d.tokens_per_frame);
  char msg[256] = "";

  // (i) self-attention, block-causal over the held frames' chunks
  ll::AttnArgs a;
  a.dtype = d.dtype;
  a.H = d.num_heads;
  a.D = d.head_dim;
  a.q = q;
  a.o = o;
  a.nq = n;
  a.seg[0] = input_segment(d, k, v, n);
  a.seg[1] = input_segment(d, k, v, 0);
  a.vis.mode = 1;
  a.vis.T = d.tokens_per_frame;
  a.vis.C = d.chunk_frames;
  a.vis.n_sink = int32_t(nsink);
  a.vis.base = base;
  a.vis.F = F;
  a.vis.sink0 = B;
  a.scale = cache->scale;
  // (ii) cross-attention to the new prompt's text tokens, in the same launch
  a.qx = qx;
  a.ox = ox;
  a.x = input_segment(d, k_text, v_text, n_text);
  a.n_cu = cache->n_cu;
  if (ll_status s = device_status(ll::launch_attention(a, stream, msg), "recache attention", msg))
    return s;
  // (iii) rewrite every held frame's slot with the new K/V
  ll::ScatterArgs w = scatter_base(cache, layer);
  w.n_frames = int32_t(held);
  w.n_lead = int32_t(nsink);
  w.lead_slot0 = int32_t(W);
  w.first_ring = base;
  w.k_src = k;
  w.v_src = v;
  if (ll_status s = device_status(ll::launch_scatter(w, stream, msg), "recache rewrite", msg))
    return s;
  return ok();
}

ll_status ll_kv_quant(const void* x_bf16, int64_t rows, int32_t row_len, uint8_t* packed,
                      uint8_t* scales, void* stream) {
  if (rows < 0) return fail(LL_EINVAL, "rows %lld", (long long)rows);
  if (row_len <= 0 || row_len % 16) return fail(LL_EINVAL, "row_len %d (multiple of 16)", row_len);
  if (rows == 0) return ok();
  if (ll_status s = check_ptr(x_bf16, "x")) return s;
  if (!packed || !scales) return fail(LL_EINVAL, "packed/scales is NULL");
  // the kernels store 8 elements' codes as one 4-byte word and 64 elements' scale bytes as one
  // word (row_len % 64 == 0), else 16 elements' codes as one 8-byte word and single scale bytes
  const bool g64 = row_len % 64 == 0;
  if (!aligned(packed, g64 ? 4 : 8))
    return fail(LL_EINVAL, "packed is not %d-byte aligned", g64 ? 4 : 8);
  if (g64 && !aligned(scales, 4)) return fail(LL_EINVAL, "scales is not 4-byte aligned");
  if (rows > (int64_t(1) << 40) / row_len) return fail(LL_EINVAL, "input too large");
  ll::QuantArgs a;
  a.x = x_bf16;
  a.rows = rows;
  a.row_len = row_len;
  a.packed = packed;
  a.scales = scales;
  char msg[256] = "";
  return device_status(ll::launch_quant(a, stream, msg), "quant launch", msg) ?: ok();
}

ll_status ll_cache_state(const ll_cache* cache, int32_t layer, int64_t* frames_committed,
                         int32_t* slot_frame) {
  if (ll_status s = check_layer(cache, layer)) return s;
  const int64_t F = cache->frames[layer];
  const int64_t S = cache->d.sink_frames, W = cache->d.window_frames;
  if (frames_committed) *frames_committed = F;
  if (slot_frame) {
    const int64_t B = cache->shot[layer];
    for (int32_t i = 0; i < slots_of(cache); ++i) slot_frame[i] = -1;
    for (int64_t j = 0; j < n_spilled(F, S, W, B); ++j) slot_frame[W + j] = int32_t(B + j);
    for (int64_t f = window_base(F, W); f < F; ++f) slot_frame[f % W] = int32_t(f);
  }
  return ok();
}

ll_status ll_cache_export(const ll_cache* cache, int32_t layer, void* k_out, void* v_out,
                          uint8_t* k_scales, uint8_t* v_scales, void* stream) {
  if (ll_status s = check_layer(cache, layer)) return s;
  if (ll_status s = check_ptr(k_out, "k_out")) return s;
  if (ll_status s = check_ptr(v_out, "v_out")) return s;
  const ll_cache_desc& d = cache->d;
  ll::ExportArgs a;
  a.dtype = d.dtype;
  a.fp4 = d.kv_format == LL_KV_FP4;
  if (a.fp4 && (!k_scales || !v_scales)) return fail(LL_EINVAL, "k_scales/v_scales is NULL");
  a.H = d.num_heads;
  a.D = d.head_dim;
  a.T = d.tokens_per_frame;
  a.slots = slots_of(cache);
  a.k_src = plane(cache, layer, cache->L.k_off);
  a.v_src = plane(cache, layer, cache->L.v_off);
  if (a.fp4) {
    a.k_src_scales = plane(cache, layer, cache->L.ks_off);
    a.v_src_scales = plane(cache, layer, cache->L.vs_off);
  }
  a.k_out = k_out;
  a.v_out = v_out;
  a.k_out_scales = k_scales;
  a.v_out_scales = v_scales;
  char msg[256] = "";
  return device_status(ll::launch_export(a, stream, msg), "export launch", msg) ?: ok();
}

const char* ll_last_error(void) { return g_err; }

}  // extern "C"
