// Device-resident candidate-tree topology.
#pragma once
#include <stdint.h>

#include <vector>

namespace medusa {

struct TreeDev {
    int N = 0;          // nodes (root included)
    int W = 0;          // 64-bit mask words per row, ceil(N / 64)
    int K = 0;          // heads the tree was declared for
    int topk = 0;       // top-k the tree was declared for
    int max_depth = 0;  // deepest node
    int max_rank = 0;   // largest rank used
    int* parent = nullptr;     // device [N]
    int* depth = nullptr;      // device [N]
    int* rank = nullptr;       // device [N]
    uint64_t* mask = nullptr;  // device [N][W]
    int* status = nullptr;     // device word: STATUS_* bits set by the kernels (atomic OR)
    std::vector<int> h_parent, h_depth, h_rank;
    std::vector<uint64_t> h_mask;
};

// What the per-head top-k merge needs to build the candidate tree in the same
// launch (medusa_heads_forward_tree): the tree, the sequences' root tokens and
// prefix lengths, and the outputs of the tree build.
struct TreeBuild {
    const TreeDev* t = nullptr;
    const int32_t* root_tok = nullptr;   // [B]
    const int32_t* cache_len = nullptr;  // [B]
    int32_t* node_tok = nullptr;         // [B][N]
    int32_t* node_pos = nullptr;         // [B][N]
    uint64_t* anc_mask = nullptr;        // [N][W], may be null
};

// per-depth alphas of the planted continuation (depth d uses a[min(d, 15)])
struct PlantAlphas {
    float a[16];
};

}  // namespace medusa
