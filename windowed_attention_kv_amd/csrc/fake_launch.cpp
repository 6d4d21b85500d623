// Recording launch backend: built with ll_host.cpp into a separate CPU-only library so the
// host layer's validation, error paths and slot arithmetic can be tested without a GPU.
// Every launch is appended to a log that the tests read through the llfake_* functions;
// llfake_fail_next() makes the next launch report a device error.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "launch.h"

namespace {

struct Record {
  int kind;              // 0 attention, 1 scatter, 2 quant, 3 export, 4 zero, 5 commit layer
  int64_t f[24];
};

std::vector<Record> g_log;
int g_fail = 0;

int maybe_fail(char* err) {
  if (g_fail > 0) {
    --g_fail;
    snprintf(err, 256, "injected launch failure");
    return 1;
  }
  return 0;
}

}  // namespace

namespace ll {

int launch_attention(const AttnArgs& a, void*, char* err) {
  if (maybe_fail(err)) return 1;
  Record r{0, {a.dtype, a.H, a.D, a.nq, a.seg[0].n, a.seg[0].fp4, a.seg[0].head_stride,
               a.seg[0].row_stride, a.seg[1].n, a.seg[1].head_stride, a.seg[1].row_stride,
               a.vis.mode, a.vis.n_sink, a.vis.base, a.vis.F, a.vis.sink0,
               a.ws != nullptr, a.ws_blocks, a.ws_slots, a.n_cu,
               a.qx != nullptr, a.ox != nullptr, a.x.n, a.x.row_stride}};
  g_log.push_back(r);
  return 0;
}

int launch_scatter(const ScatterArgs& a, void*, char* err) {
  if (maybe_fail(err)) return 1;
  Record r{1, {a.dtype, a.fp4, a.H, a.D, a.T, a.n_frames, a.n_lead, a.lead_slot0, a.ring_base, a.W,
               a.first_ring, a.slots, a.spill_lo, a.spill_hi, a.spill_slot0, 0}};
  g_log.push_back(r);
  return 0;
}

// one record per layer of a batched commit
int launch_commit_layers(const CommitLayersArgs& a, void*, char* err) {
  if (maybe_fail(err)) return 1;
  for (int i = 0; i < a.n_layers; ++i) {
    const CommitLayer& c = a.layers[i];
    Record r{5, {a.dtype, a.fp4, a.H, a.D, a.T, a.C, a.W, a.slots, a.n_layers, i, c.first_ring,
                 c.spill_lo, c.spill_hi, c.spill_slot0,
                 int64_t(reinterpret_cast<uintptr_t>(c.k_src)), int64_t(reinterpret_cast<uintptr_t>(c.v_src)),
                 int64_t(reinterpret_cast<uintptr_t>(c.k_dst)), int64_t(reinterpret_cast<uintptr_t>(c.v_dst)),
                 int64_t(reinterpret_cast<uintptr_t>(c.k_dst_scales)),
                 int64_t(reinterpret_cast<uintptr_t>(c.v_dst_scales))}};
    g_log.push_back(r);
  }
  return 0;
}

int launch_quant(const QuantArgs& a, void*, char* err) {
  if (maybe_fail(err)) return 1;
  Record r{2, {a.rows, a.row_len}};
  g_log.push_back(r);
  return 0;
}

int launch_export(const ExportArgs& a, void*, char* err) {
  if (maybe_fail(err)) return 1;
  Record r{3, {a.dtype, a.fp4, a.H, a.D, a.T, a.slots}};
  g_log.push_back(r);
  return 0;
}

int launch_zero(void* p, int64_t bytes, void*, char* err) {
  if (maybe_fail(err)) return 1;
  Record r{4, {int64_t(reinterpret_cast<uintptr_t>(p)), bytes}};
  g_log.push_back(r);
  return 0;
}

int g_fake_cus = 256;
int device_cu_count() { return g_fake_cus; }

// a recorded stand-in address for the static workspace (never dereferenced)
int static_workspace(void** ptr, void*, char* err) {
  if (maybe_fail(err)) return 1;
  *ptr = reinterpret_cast<void*>(uintptr_t(1) << 40);
  return 0;
}

}  // namespace ll

extern "C" {

void llfake_reset(void) {
  g_log.clear();
  g_fail = 0;
}

void llfake_fail_next(int n) { g_fail = n; }

// compute units the recording backend reports for caches created afterwards
void llfake_set_cus(int n) { ll::g_fake_cus = n; }

int llfake_count(void) { return int(g_log.size()); }

// kind of record i (or -1) and its 24 integer fields
int llfake_record(int i, int64_t* fields) {
  if (i < 0 || i >= int(g_log.size())) return -1;
  for (int j = 0; j < 24; ++j) fields[j] = g_log[size_t(i)].f[j];
  return g_log[size_t(i)].kind;
}

}  // extern "C"
