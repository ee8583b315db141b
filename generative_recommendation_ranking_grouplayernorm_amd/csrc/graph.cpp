// Captured serving forwards: one mtgr_hstu_stack_fwd call (and, for a
// serving graph, the candidate head after it) recorded as a HIP graph on a
// private stream, then replayed with a single launch.
#include <new>

#include "kernels.h"

using namespace mtgr;

struct mtgr_graph_s {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  // the captured batch's metadata, checked before each replay in validation
  // mode
  const int32_t* offsets = nullptr;
  const uint8_t* group_ids = nullptr;
  int32_t B = 0;
  int64_t T = 0;
};

namespace {

void release(mtgr_graph_s* g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  delete g;
}

// Records fn(stream) on a private stream and instantiates the graph.  In
// validation mode the metadata is checked first (on the null stream: no
// kernel can be recorded while it runs).
template <typename F>
int capture(F fn, const int32_t* offsets, const uint8_t* group_ids, int32_t B, int64_t T, mtgr_graph* out) {
  if (validation_enabled()) {
    const int vr = validate_jagged(offsets, group_ids, B, T, 4, true, 0, nullptr);
    if (vr) return vr;
  }
  hipStream_t cs = nullptr;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return MTGR_ERR_HIP;
  mtgr_graph_s* g = new (std::nothrow) mtgr_graph_s;
  if (!g) {
    (void)hipStreamDestroy(cs);
    return MTGR_ERR_HIP;
  }
  int r;
  if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    r = MTGR_ERR_HIP;
  } else {
    r = fn((mtgr_stream_t)cs);
    // End the capture whatever happened, so the stream is usable again.
    hipGraph_t graph = nullptr;
    const hipError_t e = hipStreamEndCapture(cs, &graph);
    g->graph = graph;
    if (r == MTGR_OK && (e != hipSuccess || !graph)) r = MTGR_ERR_HIP;
  }
  if (r == MTGR_OK && hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0) != hipSuccess) {
    g->exec = nullptr;
    r = MTGR_ERR_HIP;
  }
  (void)hipStreamDestroy(cs);
  if (r != MTGR_OK) {
    release(g);
    // A failed capture can leave a sticky launch error behind.
    (void)hipGetLastError();
    return r;
  }
  g->offsets = offsets;
  g->group_ids = group_ids;
  g->B = B;
  g->T = T;
  *out = g;
  return MTGR_OK;
}

}  // namespace

extern "C" {

int mtgr_stack_graph_create(const mtgr_layer_params* layers, int32_t L, const void* x_in, void* x_out,
                            const int32_t* offsets, const uint8_t* group_ids, const int64_t* timestamps, int32_t B,
                            int64_t T, float attn_scale, int dt, void* workspace, size_t ws_bytes,
                            mtgr_graph* out) {
  if (!out) return MTGR_ERR_INVALID_ARG;
  *out = nullptr;
  // Timing events recorded during capture would become graph nodes.
  if (profiling_enabled()) return MTGR_ERR_INVALID_ARG;
  // Empty batches launch nothing; refuse them here so that every handle
  // holds a graph with work in it.
  if (T <= 0 || B <= 0) return MTGR_ERR_INVALID_ARG;
  int r = stack_fwd_validate(layers, L, x_in, x_out, offsets, group_ids, timestamps, B, T, dt, workspace, ws_bytes);
  if (r) return r;
  return capture(
      [&](mtgr_stream_t s) {
        return stack_fwd_run(layers, L, x_in, x_out, offsets, group_ids, timestamps, B, T, attn_scale, dt,
                             workspace, ws_bytes, (hipStream_t)s, false);
      },
      offsets, group_ids, B, T, out);
}

int mtgr_serving_graph_create(const mtgr_layer_params* layers, int32_t L, const mtgr_head_params* head,
                              const void* x_in, void* x_out, float* logits, int64_t n_cand,
                              const int32_t* offsets, const uint8_t* group_ids, const int64_t* timestamps,
                              int32_t B, int64_t T, float attn_scale, int dt, void* workspace, size_t ws_bytes,
                              void* head_ws, size_t head_ws_bytes, mtgr_graph* out) {
  if (!out) return MTGR_ERR_INVALID_ARG;
  *out = nullptr;
  if (profiling_enabled()) return MTGR_ERR_INVALID_ARG;
  if (T <= 0 || B <= 0 || n_cand < 1 || !logits) return MTGR_ERR_INVALID_ARG;
  int r = stack_fwd_validate(layers, L, x_in, x_out, offsets, group_ids, timestamps, B, T, dt, workspace, ws_bytes);
  if (r) return r;
  r = head_validate(head, x_out, layers[0].d, offsets, group_ids, B, T, n_cand, dt);
  if (r) return r;
  if (head->d != layers[0].d) return MTGR_ERR_INVALID_ARG;
  if (head_ws_bytes < head_workspace_bytes(B, n_cand, head->d, head->h, head->n_tasks, dt) || !head_ws)
    return MTGR_ERR_WORKSPACE_TOO_SMALL;
  return capture(
      [&](mtgr_stream_t s) {
        int rr = stack_fwd_run(layers, L, x_in, x_out, offsets, group_ids, timestamps, B, T, attn_scale, dt,
                               workspace, ws_bytes, (hipStream_t)s, false);
        if (rr) return rr;
        return head_fwd_run(head, x_out, layers[0].d, offsets, group_ids, B, T, n_cand, logits, dt, head_ws,
                            head_ws_bytes, (hipStream_t)s, false);
      },
      offsets, group_ids, B, T, out);
}

int mtgr_stack_graph_launch(mtgr_graph g, mtgr_stream_t stream) {
  if (!g || !g->exec) return MTGR_ERR_INVALID_ARG;
  if (validation_enabled()) {
    const int vr = validate_jagged(g->offsets, g->group_ids, g->B, g->T, 4, true, 0, (hipStream_t)stream);
    if (vr) return vr;
  }
  return hipGraphLaunch(g->exec, (hipStream_t)stream) == hipSuccess ? MTGR_OK : MTGR_ERR_HIP;
}

int mtgr_stack_graph_destroy(mtgr_graph g) {
  release(g);
  return MTGR_OK;
}

}  // extern "C"
