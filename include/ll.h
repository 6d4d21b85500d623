/* ll.h -- C ABI of the window+sink chunk-attention KV library for MI355X (gfx950).
 *
 * The library implements the hot path of frame-level autoregressive video generation with
 * short-window attention and a frame sink over a rolling per-layer KV cache:
 *
 *   - "LongLive" summary page (yunpan.plus), 方法 §3 高效长推理: attention limited to a fixed
 *     local window so that compute and the per-layer KV cache size depend only on the
 *     window; the first frame-chunk pinned as global sink tokens, kept in the cache for good
 *     and joined to every layer's keys and values.
 *   - same page, 方法 §1 KV 重缓存: at a prompt switch the cache is recomputed from the
 *     frames already generated, paired with the new prompt (cross-attention in the DiT).
 *   - "LongLive 2.0" distributed-inference page (blog.hotdry.top), section on NVFP4 and KV
 *     cache compression: an FP4 KV-cache store with a fused dequantisation kernel.
 *
 * Tensor layout. Every Q/K/V/O tensor passed to the library is a row-major [tokens, H, D]
 * array (D contiguous, then heads, then tokens) of the cache's dtype. Token t of a chunk
 * belongs to frame (first frame of the chunk) + t / tokens_per_frame.
 *
 * Ownership. Tensor pointers are DEVICE pointers owned by the caller; they must stay valid
 * until the work enqueued on `stream` has finished. The cache's device memory is
 * allocated by the caller (ll_cache_size bytes) and must outlive the handle. The handle
 * itself is host memory owned by the library (ll_cache_destroy frees it, never the device
 * memory). `stream` is a hipStream_t; NULL means the null stream.
 *
 * Asynchrony. Compute calls only enqueue kernels and return. The handle's host metadata
 * (frames committed, slot map) advances at enqueue time, so all calls on one handle must be
 * issued in program order on one stream (or the caller synchronises). A handle is not
 * thread-safe. No call reads anything back from the device.
 *
 * Errors. Every call returns an ll_status. All validation happens before anything is
 * enqueued; on any error no metadata changes and nothing is enqueued, except LL_EDEVICE
 * (the HIP runtime refused a launch): metadata still stays unchanged, but cache contents that
 * an earlier launch of the same call already wrote (a batched commit of more than 32 layers
 * runs several launches) are then undefined, so reset the cache after LL_EDEVICE.
 * ll_last_error() gives a message for the last failing call on the calling thread.
 * No call aborts the process.
 */
#ifndef LL_H_
#define LL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LL_ABI_VERSION 1u

typedef enum {
  LL_OK = 0,
  LL_EINVAL = 1,       /* bad argument: null/misaligned pointer, out-of-range size or layer */
  LL_ESTATE = 2,       /* call not valid in the current cache state (e.g. recache of an empty layer) */
  LL_EUNSUPPORTED = 3, /* valid request the library does not implement (head_dim, dtype/format mix) */
  LL_EDEVICE = 4       /* the HIP runtime reported an error (launch failure, no device) */
} ll_status;

typedef enum { LL_F32 = 0, LL_BF16 = 1 } ll_dtype;

/* LL_KV_FP4: each (token, head) row of K and V is stored as D/2 bytes of e2m1 codes (element
 * 2j in the low nibble of byte j, sign in bit 3 of a code) plus D/16 e8m0 scale bytes (one per
 * 16 consecutive elements along D, value 2^(byte-127)). Quantised on commit; the own chunk of
 * an attention call stays in the cache dtype. Requires dtype == LL_BF16. */
typedef enum { LL_KV_DENSE = 0, LL_KV_FP4 = 1 } ll_kv_format;

typedef struct {
  uint32_t abi_version;    /* must be LL_ABI_VERSION */
  int32_t num_layers;      /* 1..4096 */
  int32_t num_heads;       /* H: 1..1024 */
  int32_t head_dim;        /* D: 64 or 128 */
  int32_t tokens_per_frame;/* T >= 1 */
  int32_t chunk_frames;    /* C >= 1: frames produced (and committed) per chunk; C <= W */
  int32_t sink_frames;     /* S >= 0: frames 0..S-1 are pinned for good ("sink_size") */
  int32_t window_frames;   /* W >= 1: committed frames kept before the chunk ("local_attn_size") */
  int32_t dtype;           /* ll_dtype of Q/K/V/O and of the dense cache */
  int32_t kv_format;       /* ll_kv_format ("kv_quant") */
  float softmax_scale;     /* <= 0 selects 1/sqrt(head_dim) */
} ll_cache_desc;

typedef struct ll_cache ll_cache; /* opaque host handle */

/* Bytes of device memory a cache with this descriptor needs: S+W frame slots per layer for K
 * and V (dense or FP4 planes), and, for a bf16 head_dim-128 cache, a workspace after
 * the last layer for the split schedule of ll_attn_chunk (used when a call has fewer
 * (head, 256-row query block) pairs than the device has compute units, e.g. a few heads per
 * GPU): one 32-bit counter per (head, query block), padded to 256 bytes, then
 * 2 * min(CUs, blocks * tiles) slots of 135,168 bytes, with tiles = ceil((S+W)*T/128) +
 * ceil(C*T/128). The CU count is that of the device current at the call, so create the
 * cache with the same device current. Fails with LL_EINVAL / LL_EUNSUPPORTED on a bad
 * descriptor. Size limits (the kernels use 32-bit byte offsets within a K or V plane):
 * (S+W)*T*H*D times the dtype's element size must stay below 2^31 bytes (FP4 caches are held
 * to the bf16 bound, since the own chunk stays bf16), else LL_EUNSUPPORTED; S+W <= 4096
 * slots, else LL_EINVAL. */
ll_status ll_cache_size(const ll_cache_desc* desc, size_t* device_bytes);

/* Create a handle over caller-owned device memory `device_mem` (256-byte aligned, at least
 * ll_cache_size bytes). All layers start empty. Enqueues nothing. */
ll_status ll_cache_create(const ll_cache_desc* desc, void* device_mem, size_t device_bytes,
                          ll_cache** out);

/* Free the handle (not the device memory). NULL is accepted. */
ll_status ll_cache_destroy(ll_cache* cache);

/* Mark every layer empty and back at the first shot (host metadata only). */
ll_status ll_cache_reset(ll_cache* cache);

/* Shot boundary of a multi-shot video for `layer` ("LongLive 2.0" distributed-inference
 * page, section on sequence parallelism and the attention sink: the multi-shot sink is reset
 * at every shot boundary). The next committed frame starts a new shot: from now on the sink
 * is that shot's first S frames, the previous shot's sink frames stop being visible (unless
 * they are still among the last W committed frames), and the window is unchanged. Host
 * metadata only; nothing moves. Call it for every layer at the boundary. LL_EINVAL for a bad
 * handle or layer. */
ll_status ll_cache_new_shot(ll_cache* cache, int32_t layer);

/* Window+sink chunk attention for the next chunk of `layer` (chunk index = frames
 * committed / C). q, k, v, o: [C*T, H, D]. For each head and query row:
 *   o = softmax(scale * q K^T) V over the keys of every frame the layer holds (the sink
 *   frames plus the last W committed frames; a frame counts once) followed by the chunk's
 *   own k, v (attended bidirectionally, never quantised).
 * May be called any number of times before the chunk is committed (one call per denoise
 * step); the cache's frames are not modified. Pointers 16-byte aligned. The first call on a
 * handle also clears the split-schedule counters (a kernel on `stream`); calls share the
 * workspace, so calls on one handle must not overlap on different streams. */
ll_status ll_attn_chunk(ll_cache* cache, int32_t layer, const void* q, const void* k,
                        const void* v, void* o, void* stream);

/* ll_attn_chunk for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same computation and
 * the same schedule (bit-identical o), but the split schedule's workspace (per-block arrival
 * counters and partial-result slots) is a static device array inside the library instead of
 * the workspace part of the cache's memory. The array holds 65,536 counters and 512 slots of
 * 135,168 bytes (69.5 MB per device, resident while the library is loaded); a cache whose
 * split schedule needs more (ll_cache_size's counters and slots) gets LL_EINVAL with a
 * message, before anything is enqueued. The first call on a device looks the array up and
 * clears its counters (a kernel on `stream`); every launch leaves them at zero again. The
 * call allocates nothing, host or device. All calls on one device share the array: calls that
 * overlap on one device (different streams, or different threads without ordering) race and
 * give undefined results. Errors otherwise as ll_attn_chunk. */
ll_status ll_attn_chunk_noalloc(ll_cache* cache, int32_t layer, const void* q, const void* k,
                                const void* v, void* o, void* stream);

/* ll_attn_chunk plus the chunk's text cross-attention in the same launch. In every DiT block
 * of the generator the self-attention over the frames is followed by a cross-attention of the
 * same tokens to the prompt's text tokens ("LongLive" summary page, 方法 §1 KV 重缓存, which
 * pairs the frames with the prompt through this cross-attention). Computes o exactly as
 * ll_attn_chunk does, and
 *   ox = softmax(scale * qx K_text^T) V_text over all n_text text keys (no mask),
 * with qx, ox: [C*T, H, D] and k_text, v_text: [n_text, H, D], n_text >= 1, in the cache's
 * dtype (the text K/V are never quantised). For a dense bf16 head_dim-128 cache both parts
 * run in one kernel launch (the cross blocks take the compute units the self-attention leaves
 * idle); otherwise (FP4 store, head_dim 64, fp32) as two launches on `stream`. Errors as
 * ll_attn_chunk, plus LL_EINVAL for a NULL text pointer or an n_text out of range. */
ll_status ll_attn_chunk_cross(ll_cache* cache, int32_t layer, const void* q, const void* k,
                              const void* v, const void* qx, const void* k_text,
                              const void* v_text, int32_t n_text, void* o, void* ox,
                              void* stream);

/* Append the chunk's K/V ([C*T, H, D], the final denoise step's values) as frames
 * F..F+C-1 (F = frames committed) and advance F by C. Slots 0..W-1 are the window, W..W+S-1
 * the sink: frame f goes to window slot f mod W, evicting frame f-W; an evicted frame that is
 * one of the current shot's first S frames (first frame B) is moved to sink slot W + (f-W-B)
 * in the same launch. One fused launch writes K and V (bit copies, or FP4 quantisation
 * under LL_KV_FP4; moved sink frames keep their bytes). */
ll_status ll_cache_commit(ll_cache* cache, int32_t layer, const void* k, const void* v,
                          void* stream);

/* ll_cache_commit for the layers first_layer .. first_layer + n_layers - 1 in one launch
 * (one launch per 32 layers): layer first_layer + i takes k[i], v[i] ([C*T, H, D] device
 * pointers; k and v are HOST arrays of n_layers pointers, read during the call only). Each
 * layer gets exactly what ll_cache_commit would give it (its own frame count and shot), so
 * layers may be at different frames. Committing every layer of a denoise step at once moves
 * 30x a single layer's bytes per launch, which a one-layer launch is too small to stream at
 * the device's copy rate ("为什么视频生成是一个基础设施问题", §3 and §4: KV-cache update and
 * movement become visible costs once the denoise steps are few). Every layer is validated before anything is enqueued; on any error no layer's
 * metadata changes. LL_EINVAL for a bad handle, layer range, or a NULL / misaligned pointer. */
ll_status ll_cache_commit_layers(ll_cache* cache, int32_t first_layer, int32_t n_layers,
                                 const void* const* k, const void* const* v, void* stream);

/* Prompt-switch recache of `layer` ("LongLive" page, 方法 §1 KV 重缓存). The rows are the
 * frames the layer holds, in ascending frame id (n = held_frames * T rows):
 *   q, k, v, qx, o, ox: [n, H, D]; k_text, v_text: [n_text, H, D], n_text >= 1.
 *   o  = block-causal self-attention: a query in frame fq sees key row of frame fk iff
 *        fk / C <= fq / C (integer division);
 *   ox = cross-attention of qx to all n_text text keys (no mask);
 * then every held frame keeps its id and slot and takes the new k, v as its value
 * (quantised under LL_KV_FP4). LL_ESTATE if the layer holds no frame. */
ll_status ll_recache(ll_cache* cache, int32_t layer, const void* q, const void* k,
                     const void* v, const void* qx, const void* k_text, const void* v_text,
                     int32_t n_text, void* o, void* ox, void* stream);

/* Standalone FP4 codec ("LongLive 2.0" distributed-inference page, section on NVFP4 and KV
 * cache compression: the KV cache stored in FP4; the e2m1 element and e8m0 scale encodings
 * and the shared-exponent rule are those of the OCP Microscaling Formats v1.0 spec, the pages
 * naming only "FP4"). x ([rows, row_len] bf16, row_len % 16 == 0) ->
 * packed [rows, row_len/2] bytes and scales [rows, row_len/16] e8m0 bytes. Per block of 16:
 * scale byte = max(exponent_field(max|x|) - 2, 0); codes = |x| * 2^-(scale-127) rounded to
 * {0,.5,1,1.5,2,3,4,6}, ties to the even code, saturating at 6; sign bit copied. Inputs
 * must be finite. Bit-exact and deterministic. x must be 16-byte aligned, packed 4-byte
 * aligned (8-byte when row_len % 64 != 0) and scales 4-byte aligned when row_len % 64 == 0;
 * LL_EINVAL for a NULL or misaligned pointer, rows < 0 or a row_len that is not a positive
 * multiple of 16 (rows == 0 is a no-op). */
ll_status ll_kv_quant(const void* x_bf16, int64_t rows, int32_t row_len, uint8_t* packed,
                      uint8_t* scales, void* stream);

/* Host metadata of `layer`: frames committed and, for each of the S+W slots, the frame id
 * stored there (-1 if empty). slot_frame may be NULL. */
ll_status ll_cache_state(const ll_cache* cache, int32_t layer, int64_t* frames_committed,
                         int32_t* slot_frame);

/* Copy `layer`'s cache out in slot order (device to device, enqueued on `stream`):
 * dense: k_out, v_out [(S+W)*T, H, D] of the cache dtype (scales ignored);
 * FP4: k_out, v_out packed [(S+W)*T*H, D/2] bytes, k_scales, v_scales [(S+W)*T*H, D/16].
 * Rows of empty slots hold whatever the memory held. */
ll_status ll_cache_export(const ll_cache* cache, int32_t layer, void* k_out, void* v_out,
                          uint8_t* k_scales, uint8_t* v_scales, void* stream);

/* Message of the last failing call on this thread ("" if none). Valid until the next call. */
const char* ll_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LL_H_ */
