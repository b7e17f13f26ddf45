// k_mask.hip -- ancestor bitmask of every draft-tree node.
//
// Visibility rule (JetFlow blog page, "What JetFlow Does Differently"): a node
// sees the prefix and its ancestors in the tree, not its siblings or
// descendants.  Row i of the mask holds bit j iff j is an ancestor of i (i
// itself included).  One workgroup per sequence: the parent array is staged in
// LDS and every lane walks its nodes' chains there, four 64-bit words per walk.
// Trees are either N nodes per sequence (rows b*N + i) or packed: sequence b
// owns rows node_off[b] .. node_off[b+1]-1, its parents local to it.
#include "jf_internal.h"

namespace jf {
namespace {

constexpr int kMaskThreads = 256;
constexpr int kMaxN = 4096;

struct NodeOffsets {
    int off[kMaxBatch + 1];
};

__global__ __launch_bounds__(kMaskThreads) void k_tree_mask(const int32_t *__restrict__ parent,
                                                            int N_uniform, int W, bool packed,
                                                            NodeOffsets no,
                                                            uint64_t *__restrict__ mask,
                                                            int32_t *__restrict__ depth,
                                                            int32_t *__restrict__ seq_status) {
    __shared__ int32_t par[kMaxN];
    __shared__ int32_t first_bad;
    const int b = blockIdx.x;
    const int64_t base = packed ? (int64_t)no.off[b] : (int64_t)b * N_uniform;
    const int N = packed ? no.off[b + 1] - no.off[b] : N_uniform;
    const int32_t *prow = parent + base;
    for (int i = threadIdx.x; i < N; i += kMaskThreads) par[i] = prow[i];
    if (threadIdx.x == 0) first_bad = INT32_MAX;
    __syncthreads();

    for (int i = threadIdx.x; i < N; i += kMaskThreads) {
        // Validate the chain and measure its length (the depth).
        int j = i, steps = 0;
        bool ok = true;
        while (j != -1) {
            if (j < -1 || j >= N || steps >= N) { ok = false; break; }
            ++steps;
            j = par[j];
        }
        uint64_t *row = mask + (base + i) * W;
        if (!ok) {
            atomicMin(&first_bad, i);
            for (int w = 0; w < W; ++w) row[w] = 0;
            if (depth) depth[base + i] = 0;
            continue;
        }
        if (depth) depth[base + i] = steps;
        // Collect the chain's bits, four words per walk.
        for (int w0 = 0; w0 < W; w0 += 4) {
            uint64_t acc0 = 0, acc1 = 0, acc2 = 0, acc3 = 0;
            for (int a = i; a != -1; a = par[a]) {
                int wi = (a >> 6) - w0;
                uint64_t bit = 1ull << (a & 63);
                acc0 |= wi == 0 ? bit : 0ull;
                acc1 |= wi == 1 ? bit : 0ull;
                acc2 |= wi == 2 ? bit : 0ull;
                acc3 |= wi == 3 ? bit : 0ull;
            }
            row[w0] = acc0;
            if (w0 + 1 < W) row[w0 + 1] = acc1;
            if (w0 + 2 < W) row[w0 + 2] = acc2;
            if (w0 + 3 < W) row[w0 + 3] = acc3;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0 && seq_status) seq_status[b] = first_bad == INT32_MAX ? -1 : first_bad;
}

}  // namespace

hipError_t launch_tree_mask(const int32_t *parent, const int32_t *node_off, int B, int N,
                            uint64_t *mask, int32_t *depth, int32_t *seq_status, hipStream_t s) {
    const int W = (N + 63) / 64;
    NodeOffsets no;
    if (node_off)
        for (int b = 0; b <= B; ++b) no.off[b] = node_off[b];
    else
        no.off[0] = 0;
    hipLaunchKernelGGL(k_tree_mask, dim3(B), dim3(kMaskThreads), 0, s, parent, N, W,
                       node_off != nullptr, no, mask, depth, seq_status);
    return hipGetLastError();
}

}  // namespace jf
