// Decode-step graphs: capture the fixed sequence of a decode step once,
// instantiate it, and before each launch point its kernels at the step's
// buffers by updating the instantiated graph's kernel-node parameters
// (INT4 quantization page, Part 2, steps 2-4: capture a profile run between
// begin/end capture, instantiate, set the node parameters of the dynamic
// inputs and outputs, launch the whole graph at once).
//
// The update is node by node: the caller captures the same sequence of
// library calls again with the new pointers (capture only records the
// launches; nothing runs), and every kernel node of the instantiated graph
// takes the parameters of its counterpart in the new capture. Counterparts
// are found by position in dependency order, and must launch the same kernel
// with the same grid, block and LDS size; otherwise nothing is changed and the
// update fails, since the step is then not the one the graph was built from.

#include <new>
#include <vector>

#include "common.hpp"

namespace {

struct Graph {
  hipGraph_t graph = nullptr;         // the captured graph the executable was built from
  hipGraphExec_t exec = nullptr;
  std::vector<hipGraphNode_t> kernels;  // its kernel nodes in dependency order
};

// Kernel nodes of g in dependency order (Kahn's algorithm over the node list,
// taking ready nodes in list order), or false if the runtime refused a query.
bool kernel_order(hipGraph_t g, std::vector<hipGraphNode_t>& out) {
  size_t n = 0;
  if (hipGraphGetNodes(g, nullptr, &n) != hipSuccess) return false;
  std::vector<hipGraphNode_t> nodes(n);
  if (n && hipGraphGetNodes(g, nodes.data(), &n) != hipSuccess) return false;
  std::vector<size_t> pending(n, 0);
  std::vector<std::vector<size_t>> users(n);
  for (size_t i = 0; i < n; ++i) {
    size_t nd = 0;
    if (hipGraphNodeGetDependencies(nodes[i], nullptr, &nd) != hipSuccess) return false;
    std::vector<hipGraphNode_t> deps(nd);
    if (nd && hipGraphNodeGetDependencies(nodes[i], deps.data(), &nd) != hipSuccess) return false;
    pending[i] = nd;
    for (size_t d = 0; d < nd; ++d)
      for (size_t j = 0; j < n; ++j)
        if (nodes[j] == deps[d]) users[j].push_back(i);
  }
  std::vector<bool> done(n, false);
  out.clear();
  for (size_t taken = 0; taken < n; ++taken) {
    size_t pick = n;
    for (size_t i = 0; i < n && pick == n; ++i)
      if (!done[i] && pending[i] == 0) pick = i;
    if (pick == n) return false;                   // a cycle: not a captured graph
    done[pick] = true;
    for (size_t u : users[pick]) --pending[u];
    hipGraphNodeType t;
    if (hipGraphNodeGetType(nodes[pick], &t) != hipSuccess) return false;
    if (t == hipGraphNodeTypeKernel) out.push_back(nodes[pick]);
  }
  return true;
}

bool same_launch(const hipKernelNodeParams& a, const hipKernelNodeParams& b) {
  return a.func == b.func && a.gridDim.x == b.gridDim.x && a.gridDim.y == b.gridDim.y &&
         a.gridDim.z == b.gridDim.z && a.blockDim.x == b.blockDim.x &&
         a.blockDim.y == b.blockDim.y && a.blockDim.z == b.blockDim.z &&
         a.sharedMemBytes == b.sharedMemBytes;
}

int end_capture(hipStream_t stream, hipGraph_t* g) {
  if (hipStreamEndCapture(stream, g) != hipSuccess || !*g) {
    (void)hipGetLastError();
    return W4_ERR_HIP;
  }
  return W4_OK;
}

}  // namespace

extern "C" int w4_graph_begin(hipStream_t stream) {
  if (!stream) return W4_ERR_NULL;                   // the legacy stream cannot be captured
  return hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal) == hipSuccess
             ? W4_OK
             : W4_ERR_HIP;
}

extern "C" int w4_graph_end(hipStream_t stream, w4_graph_t* out) {
  if (!stream || !out) return W4_ERR_NULL;
  *out = nullptr;
  hipGraph_t g = nullptr;
  const int st = end_capture(stream, &g);
  if (st != W4_OK) return st;
  Graph* h = new (std::nothrow) Graph;
  if (!h) {
    (void)hipGraphDestroy(g);
    return W4_ERR_HIP;
  }
  h->graph = g;
  if (!kernel_order(g, h->kernels) ||
      hipGraphInstantiate(&h->exec, g, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipGraphDestroy(g);
    delete h;
    return W4_ERR_HIP;
  }
  *out = reinterpret_cast<w4_graph_t>(h);
  return W4_OK;
}

extern "C" int w4_graph_update(w4_graph_t graph, hipStream_t stream) {
  if (!graph || !stream) return W4_ERR_NULL;
  Graph* h = reinterpret_cast<Graph*>(graph);
  hipGraph_t g = nullptr;
  const int st = end_capture(stream, &g);
  if (st != W4_OK) return st;
  std::vector<hipGraphNode_t> fresh;
  int status = W4_OK;
  if (!kernel_order(g, fresh)) {
    status = W4_ERR_HIP;
  } else if (fresh.size() != h->kernels.size()) {
    status = W4_ERR_ARG;
  } else {
    // check every pair before changing anything
    std::vector<hipKernelNodeParams> np(fresh.size());
    for (size_t i = 0; i < fresh.size() && status == W4_OK; ++i) {
      hipKernelNodeParams old{};
      if (hipGraphKernelNodeGetParams(fresh[i], &np[i]) != hipSuccess ||
          hipGraphKernelNodeGetParams(h->kernels[i], &old) != hipSuccess)
        status = W4_ERR_HIP;
      else if (!same_launch(np[i], old))
        status = W4_ERR_ARG;
    }
    for (size_t i = 0; i < fresh.size() && status == W4_OK; ++i)
      if (hipGraphExecKernelNodeSetParams(h->exec, h->kernels[i], &np[i]) != hipSuccess)
        status = W4_ERR_HIP;
  }
  (void)hipGetLastError();
  (void)hipGraphDestroy(g);                          // the executable holds copies of the parameters
  return status;
}

extern "C" int w4_graph_launch(w4_graph_t graph, hipStream_t stream) {
  if (!graph) return W4_ERR_NULL;
  Graph* h = reinterpret_cast<Graph*>(graph);
  return hipGraphLaunch(h->exec, stream) == hipSuccess ? W4_OK : W4_ERR_HIP;
}

extern "C" int w4_graph_kernel_nodes(w4_graph_t graph) {
  if (!graph) return W4_ERR_NULL;
  return (int)reinterpret_cast<Graph*>(graph)->kernels.size();
}

extern "C" int w4_graph_destroy(w4_graph_t graph) {
  if (!graph) return W4_OK;
  Graph* h = reinterpret_cast<Graph*>(graph);
  int status = W4_OK;
  if (h->exec && hipGraphExecDestroy(h->exec) != hipSuccess) status = W4_ERR_HIP;
  if (h->graph && hipGraphDestroy(h->graph) != hipSuccess) status = W4_ERR_HIP;
  delete h;
  return status;
}
