// Internal host-side representation of Shape:Stride layouts, shared by the
// C-ABI layout functions and the GEMM planner. Not part of the public ABI.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "lt.h"

namespace lt {

// A nested layout: one preorder tree code for shape and stride together
// (0 = leaf, k > 0 = tuple of k children) and the leaves left to right.
struct Tree {
    std::vector<int8_t> code;
    std::vector<int64_t> s;   // extents
    std::vector<int64_t> d;   // strides

    static Tree leaf(int64_t s, int64_t d) { return Tree{{0}, {s}, {d}}; }
    static Tree tuple(const std::vector<Tree>& kids);
    // A single leaf if pairs has one entry, else a flat tuple of them.
    static Tree flat(const std::vector<std::pair<int64_t, int64_t>>& pairs);

    bool is_leaf() const { return code.size() == 1 && code[0] == 0; }
    int rank() const { return is_leaf() ? 1 : code[0]; }
    std::vector<Tree> modes() const;          // top-level modes
    Tree mode(int i) const { return modes()[i]; }
};

// status-returning helpers (LT_OK on success)
lt_status from_pod(const lt_layout* L, Tree* out);
lt_status to_pod(const Tree& t, lt_layout* out);
lt_status tree_size(const Tree& t, int64_t* out);     // product, overflow-checked
lt_status tree_cosize(const Tree& t, int64_t* out);
lt_status tree_eval(const Tree& t, int64_t idx, int64_t* out);
Tree coalesce(const Tree& t);
lt_status compose(const Tree& A, const Tree& B, Tree* out);
lt_status complement(const Tree& B, int64_t M, Tree* out);
lt_status divide_shape(const Tree& A, int n, const int64_t* tiler, bool zipped, Tree* out);
lt_status logical_product(const Tree& A, const Tree& B, Tree* out);
lt_status make_tv(int n, const int64_t* thr, const int64_t* val, const uint8_t* blocked, Tree* out);
std::string format(const Tree& t);

}  // namespace lt
