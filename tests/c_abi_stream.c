/* A plain-C consumer of the library's C ABI (include/ll.h): streams chunks through one layer of
 * a cache and writes every chunk's attention output, for tests/test_c_abi.py to compare with the
 * oracle. No Python and no torch: device memory comes from the HIP runtime directly.
 *
 *   c_abi_stream --abi           print LL_ABI_VERSION and exit (touches no GPU)
 *   c_abi_stream <dir>           run the stream described by <dir>/desc.txt:
 *       "H D T C S W chunks dtype kv_format" (dtype 0 fp32 / 1 bf16, kv_format 0 dense / 1 fp4);
 *       for chunk c it reads <dir>/q_c.bin, k_c.bin, v_c.bin (raw [C*T, H, D] arrays of the
 *       dtype), runs ll_attn_chunk, writes <dir>/o_c.bin, then ll_cache_commit.
 * Exit status 0 on success; on failure it prints the call and ll_last_error(). */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ll.h"

static int fail_ll(const char* what, ll_status s) {
  fprintf(stderr, "%s: status %d: %s\n", what, (int)s, ll_last_error());
  return 1;
}

static int fail_hip(const char* what, hipError_t e) {
  fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return 1;
}

static int read_file(const char* path, void* buf, size_t bytes) {
  FILE* f = fopen(path, "rb");
  if (!f) return 0;
  const size_t n = fread(buf, 1, bytes, f);
  fclose(f);
  return n == bytes;
}

static int write_file(const char* path, const void* buf, size_t bytes) {
  FILE* f = fopen(path, "wb");
  if (!f) return 0;
  const size_t n = fwrite(buf, 1, bytes, f);
  fclose(f);
  return n == bytes;
}

int main(int argc, char** argv) {
  if (argc == 2 && strcmp(argv[1], "--abi") == 0) {
    printf("%u\n", LL_ABI_VERSION);
    return 0;
  }
  if (argc != 2) {
    fprintf(stderr, "usage: %s <dir> | --abi\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  char path[4096];
  int H, D, T, C, S, W, chunks, dtype, kv_format;
  snprintf(path, sizeof path, "%s/desc.txt", dir);
  FILE* f = fopen(path, "r");
  if (!f || fscanf(f, "%d %d %d %d %d %d %d %d %d", &H, &D, &T, &C, &S, &W, &chunks, &dtype,
                   &kv_format) != 9) {
    fprintf(stderr, "cannot read %s\n", path);
    if (f) fclose(f);
    return 2;
  }
  fclose(f);

  ll_cache_desc d;
  memset(&d, 0, sizeof d);
  d.abi_version = LL_ABI_VERSION;
  d.num_layers = 1;
  d.num_heads = H;
  d.head_dim = D;
  d.tokens_per_frame = T;
  d.chunk_frames = C;
  d.sink_frames = S;
  d.window_frames = W;
  d.dtype = dtype;
  d.kv_format = kv_format;
  d.softmax_scale = 0.0f;   /* 1/sqrt(head_dim) */

  size_t bytes = 0;
  ll_status s = ll_cache_size(&d, &bytes);
  if (s != LL_OK) return fail_ll("ll_cache_size", s);
  void* mem = NULL;
  hipError_t e = hipMalloc(&mem, bytes);
  if (e != hipSuccess) return fail_hip("hipMalloc(cache)", e);
  ll_cache* cache = NULL;
  s = ll_cache_create(&d, mem, bytes, &cache);
  if (s != LL_OK) return fail_ll("ll_cache_create", s);

  const size_t elems = (size_t)C * T * H * D;
  const size_t tbytes = elems * (dtype == LL_BF16 ? 2 : 4);
  void* host = malloc(tbytes);
  void* dq = NULL;
  void* dk = NULL;
  void* dv = NULL;
  void* dout = NULL;
  if (!host) return 1;
  if ((e = hipMalloc(&dq, tbytes)) != hipSuccess || (e = hipMalloc(&dk, tbytes)) != hipSuccess ||
      (e = hipMalloc(&dv, tbytes)) != hipSuccess || (e = hipMalloc(&dout, tbytes)) != hipSuccess)
    return fail_hip("hipMalloc(tensors)", e);

  const char* names[3] = {"q", "k", "v"};
  void* dev[3] = {dq, dk, dv};
  for (int c = 0; c < chunks; ++c) {
    for (int i = 0; i < 3; ++i) {
      snprintf(path, sizeof path, "%s/%s_%d.bin", dir, names[i], c);
      if (!read_file(path, host, tbytes)) {
        fprintf(stderr, "cannot read %s\n", path);
        return 2;
      }
      if ((e = hipMemcpy(dev[i], host, tbytes, hipMemcpyHostToDevice)) != hipSuccess)
        return fail_hip("hipMemcpy(in)", e);
    }
    s = ll_attn_chunk(cache, 0, dq, dk, dv, dout, NULL);
    if (s != LL_OK) return fail_ll("ll_attn_chunk", s);
    if ((e = hipMemcpy(host, dout, tbytes, hipMemcpyDeviceToHost)) != hipSuccess)
      return fail_hip("hipMemcpy(out)", e);
    snprintf(path, sizeof path, "%s/o_%d.bin", dir, c);
    if (!write_file(path, host, tbytes)) {
      fprintf(stderr, "cannot write %s\n", path);
      return 2;
    }
    s = ll_cache_commit(cache, 0, dk, dv, NULL);
    if (s != LL_OK) return fail_ll("ll_cache_commit", s);
  }
  if ((e = hipDeviceSynchronize()) != hipSuccess) return fail_hip("hipDeviceSynchronize", e);
  int64_t frames = 0;
  s = ll_cache_state(cache, 0, &frames, NULL);
  if (s != LL_OK) return fail_ll("ll_cache_state", s);
  printf("frames committed %lld\n", (long long)frames);
  ll_cache_destroy(cache);
  hipFree(dq);
  hipFree(dk);
  hipFree(dv);
  hipFree(dout);
  hipFree(mem);
  free(host);
  return 0;
}
