// Step graphs: capture the launches of one step on a stream once, replay
// them every step.  The rollout engine captures one decode graph per
// batch-size bucket during warm-up and replays the nearest bucket at or
// above the live batch, padding it with no-op rows; replay is what closes
// most of its gap to vLLM (scripts/benchmarks commit log 1847125,
// flex_attention paged-KV engine entry, "Why this works" item 3).
//
// Every pkv_* launch is replay-safe: kernels take lengths, tables and slot
// positions from device arrays and size their grids from host upper bounds
// only, and no call enqueues a memset or a host read.
#include <new>

#include "../../include/pkv.h"
#include "common.h"

struct pkv_graph_s {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

namespace {
pkv_status graph_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }
}  // namespace

extern "C" {

pkv_status pkv_graph_begin(hipStream_t stream) {
  if (stream == nullptr) return PKV_ERR_NULL_ARG;  // the legacy null stream cannot be captured
  return graph_status(hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal));
}

pkv_status pkv_graph_end(hipStream_t stream, pkv_graph* graph) {
  if (stream == nullptr || graph == nullptr) return PKV_ERR_NULL_ARG;
  *graph = nullptr;
  hipGraph_t g = nullptr;
  if (hipStreamEndCapture(stream, &g) != hipSuccess || g == nullptr) {
    if (g != nullptr) (void)hipGraphDestroy(g);
    return PKV_ERR_HIP;
  }
  hipGraphExec_t x = nullptr;
  if (hipGraphInstantiate(&x, g, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(g);
    return PKV_ERR_HIP;
  }
  pkv_graph h = new (std::nothrow) pkv_graph_s{g, x};
  if (h == nullptr) {
    (void)hipGraphExecDestroy(x);
    (void)hipGraphDestroy(g);
    return PKV_ERR_HIP;
  }
  *graph = h;
  return PKV_OK;
}

pkv_status pkv_graph_launch(pkv_graph graph, hipStream_t stream) {
  if (graph == nullptr) return PKV_ERR_NULL_ARG;
  return graph_status(hipGraphLaunch(graph->exec, stream));
}

pkv_status pkv_graph_nodes(pkv_graph graph, int32_t* kernel_nodes, int32_t* other_nodes) {
  if (graph == nullptr || kernel_nodes == nullptr || other_nodes == nullptr)
    return PKV_ERR_NULL_ARG;
  size_t n = 0;
  if (hipGraphGetNodes(graph->graph, nullptr, &n) != hipSuccess) return PKV_ERR_HIP;
  int32_t kern = 0, other = 0;
  if (n > 0) {
    hipGraphNode_t* nodes = new (std::nothrow) hipGraphNode_t[n];
    if (nodes == nullptr) return PKV_ERR_HIP;
    hipError_t e = hipGraphGetNodes(graph->graph, nodes, &n);
    for (size_t i = 0; e == hipSuccess && i < n; ++i) {
      hipGraphNodeType t;
      e = hipGraphNodeGetType(nodes[i], &t);
      if (e == hipSuccess) (t == hipGraphNodeTypeKernel ? kern : other) += 1;
    }
    delete[] nodes;
    if (e != hipSuccess) return PKV_ERR_HIP;
  }
  *kernel_nodes = kern;
  *other_nodes = other;
  return PKV_OK;
}

pkv_status pkv_graph_destroy(pkv_graph graph) {
  if (graph == nullptr) return PKV_OK;
  const hipError_t a = hipGraphExecDestroy(graph->exec);
  const hipError_t b = hipGraphDestroy(graph->graph);
  delete graph;
  return (a == hipSuccess && b == hipSuccess) ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"
