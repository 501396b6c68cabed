// Host layout algebra behind the C ABI (lt_* layout functions).
//
// A layout is a function from coordinates to offsets, written Shape:Stride,
// with shape and stride congruent nested tuples ("CUTLASS and CuTe layouts",
// "A layout is a shape and a stride"; "3.5 CUTLASS II — CuTe 레이아웃·텐서",
// 3.5.3-3.5.4; "Layouts as Algebra: CUTLASS & CuTe", "The formula gets a
// name" and "A shape is a tree"). All arithmetic is int64 with overflow
// checks; nothing here touches a device.

#include <algorithm>
#include <cctype>
#include <cstring>

#include "layout_host.hpp"

namespace lt {

namespace {

bool mul_ok(int64_t a, int64_t b, int64_t* r) { return !__builtin_mul_overflow(a, b, r); }
bool add_ok(int64_t a, int64_t b, int64_t* r) { return !__builtin_add_overflow(a, b, r); }

// End of the subtree that starts at code[pos]; counts its leaves.
size_t subtree_end(const std::vector<int8_t>& code, size_t pos, int* leaves) {
    int pending = 1;
    while (pending > 0) {
        if (pos >= code.size()) return SIZE_MAX;
        int8_t c = code[pos++];
        pending -= 1;
        if (c == 0) {
            ++*leaves;
        } else {
            pending += c;
        }
    }
    return pos;
}

}  // namespace

// The algebra is defined for layouts with at least one coordinate; an extent
// of 0 (an empty operand) is only meaningful to evaluate and to the GEMM.
static bool empty(const Tree& t) {
    for (int64_t s : t.s)
        if (s == 0) return true;
    return false;
}

Tree Tree::tuple(const std::vector<Tree>& kids) {
    Tree t;
    t.code.push_back(static_cast<int8_t>(kids.size()));
    for (const Tree& k : kids) {
        t.code.insert(t.code.end(), k.code.begin(), k.code.end());
        t.s.insert(t.s.end(), k.s.begin(), k.s.end());
        t.d.insert(t.d.end(), k.d.begin(), k.d.end());
    }
    return t;
}

Tree Tree::flat(const std::vector<std::pair<int64_t, int64_t>>& pairs) {
    if (pairs.size() == 1) return leaf(pairs[0].first, pairs[0].second);
    std::vector<Tree> kids;
    for (auto& p : pairs) kids.push_back(leaf(p.first, p.second));
    return tuple(kids);
}

std::vector<Tree> Tree::modes() const {
    if (is_leaf()) return {*this};
    std::vector<Tree> out;
    size_t pos = 1;
    size_t leaf0 = 0;
    for (int k = 0; k < code[0]; ++k) {
        int nl = 0;
        size_t end = subtree_end(code, pos, &nl);
        Tree m;
        m.code.assign(code.begin() + pos, code.begin() + end);
        m.s.assign(s.begin() + leaf0, s.begin() + leaf0 + nl);
        m.d.assign(d.begin() + leaf0, d.begin() + leaf0 + nl);
        out.push_back(std::move(m));
        pos = end;
        leaf0 += nl;
    }
    return out;
}

lt_status from_pod(const lt_layout* L, Tree* out) {
    if (!L) return LT_ERR_INVALID_ARGUMENT;
    if (L->nleaves < 1 || L->nleaves > LT_MAX_LEAVES || L->nnodes < 1 || L->nnodes > LT_MAX_NODES)
        return LT_ERR_INVALID_LAYOUT;
    Tree t;
    t.code.assign(L->tree, L->tree + L->nnodes);
    for (int8_t c : t.code)
        if (c < 0) return LT_ERR_INVALID_LAYOUT;
    int nl = 0;
    size_t end = subtree_end(t.code, 0, &nl);
    if (end != t.code.size() || nl != L->nleaves) return LT_ERR_INVALID_LAYOUT;
    t.s.assign(L->shape, L->shape + L->nleaves);
    t.d.assign(L->stride, L->stride + L->nleaves);
    for (int i = 0; i < L->nleaves; ++i)
        if (t.s[i] < 0 || t.d[i] < 0) return LT_ERR_INVALID_LAYOUT;
    int64_t n;
    lt_status st = tree_size(t, &n);
    if (st != LT_OK) return st;
    *out = std::move(t);
    return LT_OK;
}

lt_status to_pod(const Tree& t, lt_layout* out) {
    if (t.s.size() > LT_MAX_LEAVES || t.code.size() > LT_MAX_NODES) return LT_ERR_CAPACITY;
    lt_layout L;
    std::memset(&L, 0, sizeof(L));
    L.nleaves = static_cast<int32_t>(t.s.size());
    L.nnodes = static_cast<int32_t>(t.code.size());
    std::copy(t.s.begin(), t.s.end(), L.shape);
    std::copy(t.d.begin(), t.d.end(), L.stride);
    std::copy(t.code.begin(), t.code.end(), L.tree);
    *out = L;
    return LT_OK;
}

lt_status tree_size(const Tree& t, int64_t* out) {
    int64_t n = 1;
    for (int64_t s : t.s)
        if (!mul_ok(n, s, &n)) return LT_ERR_OUT_OF_RANGE;
    *out = n;
    return LT_OK;
}

// Strides are non-negative, so the largest offset is reached at the last
// coordinate: sum of (extent - 1) * stride. cosize is that plus one.
lt_status tree_cosize(const Tree& t, int64_t* out) {
    for (int64_t s : t.s)
        if (s == 0) {   // no coordinates, nothing reached
            *out = 0;
            return LT_OK;
        }
    int64_t top = 0;
    for (size_t i = 0; i < t.s.size(); ++i) {
        int64_t term;
        if (!mul_ok(t.s[i] - 1, t.d[i], &term) || !add_ok(top, term, &top)) return LT_ERR_OUT_OF_RANGE;
    }
    if (!add_ok(top, 1, out)) return LT_ERR_OUT_OF_RANGE;
    return LT_OK;
}

// Colexicographic unravel: leaf 0 varies fastest.
lt_status tree_eval(const Tree& t, int64_t idx, int64_t* out) {
    int64_t n;
    lt_status st = tree_size(t, &n);
    if (st != LT_OK) return st;
    if (idx < 0 || idx >= n) return LT_ERR_OUT_OF_RANGE;
    int64_t off = 0;
    for (size_t i = 0; i < t.s.size(); ++i) {
        int64_t c = idx % t.s[i];
        idx /= t.s[i];
        int64_t term;
        if (!mul_ok(c, t.d[i], &term) || !add_ok(off, term, &off)) return LT_ERR_OUT_OF_RANGE;
    }
    *out = off;
    return LT_OK;
}

Tree coalesce(const Tree& t) {
    std::vector<std::pair<int64_t, int64_t>> run;
    for (size_t i = 0; i < t.s.size(); ++i) {
        if (t.s[i] == 1) continue;
        if (!run.empty()) {
            auto& last = run.back();
            int64_t next;
            if (mul_ok(last.first, last.second, &next) && next == t.d[i]) {
                last.first *= t.s[i];
                continue;
            }
        }
        run.emplace_back(t.s[i], t.d[i]);
    }
    if (run.empty()) return Tree::leaf(1, 0);
    return Tree::flat(run);
}

// ---------------------------------------------------------------------------
// composition
// ---------------------------------------------------------------------------

namespace {

struct Leaf {
    int64_t s, d;
};

// Per-digit footprint of one leaf of B inside A's mixed radix: the largest
// digit value it can produce at each of A's coalesced leaves.
struct Walk {
    std::vector<Leaf> out;
    std::vector<int64_t> maxdigit;   // one per A leaf
};

// Walk one leaf s:d of B through A's coalesced leaves ("Layouts as Algebra",
// "Composition, worked by hand"): a step of d first passes over the leaves
// of A that it spans whole and cuts the one it lands in; then s such steps
// are laid over the remaining leaves, one result leaf per boundary crossed.
// Every cut must be exact.
lt_status walk_leaf(const std::vector<Leaf>& a, int64_t s, int64_t d, Walk* w) {
    w->out.clear();
    w->maxdigit.assign(a.size(), 0);
    if (s == 1) {
        w->out.push_back({1, 0});
        return LT_OK;
    }
    if (d == 0) {
        w->out.push_back({s, 0});
        return LT_OK;
    }
    size_t i = 0;
    int64_t cut = 1;           // multiplier inside leaf i (the leaf starts at digit value granularity `cut`)
    int64_t rest = d;
    while (rest > 1) {
        if (i >= a.size()) return LT_ERR_NOT_ADMISSIBLE;
        int64_t ext = a[i].s;
        if (rest % ext == 0) {
            rest /= ext;
            ++i;
        } else if (ext % rest == 0) {
            cut = rest;
            rest = 1;
        } else {
            return LT_ERR_NOT_ADMISSIBLE;
        }
    }
    rest = s;
    while (rest > 1) {
        if (i >= a.size()) return LT_ERR_NOT_ADMISSIBLE;
        int64_t ext = a[i].s / cut;    // what is left of leaf i above the cut
        int64_t stride = a[i].d * cut;
        if (ext == 1) {
            ++i;
            cut = 1;
            continue;
        }
        if (rest % ext == 0) {
            w->out.push_back({ext, stride});
            w->maxdigit[i] = (ext - 1) * cut;
            rest /= ext;
            ++i;
            cut = 1;
        } else if (ext % rest == 0) {
            w->out.push_back({rest, stride});
            w->maxdigit[i] = (rest - 1) * cut;
            rest = 1;
        } else {
            return LT_ERR_NOT_ADMISSIBLE;
        }
    }
    return LT_OK;
}

}  // namespace

lt_status compose(const Tree& A, const Tree& B, Tree* out) {
    if (empty(A) || empty(B)) return LT_ERR_INVALID_LAYOUT;
    Tree ac = coalesce(A);
    std::vector<Leaf> a;
    for (size_t i = 0; i < ac.s.size(); ++i) a.push_back({ac.s[i], ac.d[i]});
    int64_t sizeA;
    lt_status st = tree_size(A, &sizeA);
    if (st != LT_OK) return st;

    // Rebuild B's tree with each leaf replaced by its walk.
    Tree r;
    std::vector<int64_t> digit_sum(a.size(), 0);
    size_t li = 0;
    for (int8_t c : B.code) {
        if (c != 0) {
            r.code.push_back(c);
            continue;
        }
        Walk w;
        st = walk_leaf(a, B.s[li], B.d[li], &w);
        if (st != LT_OK) return st;
        if (B.s[li] > 1 && B.d[li] > 0)
            for (size_t k = 0; k < a.size(); ++k) digit_sum[k] += w.maxdigit[k];
        if (w.out.size() == 1) {
            r.code.push_back(0);
        } else {
            r.code.push_back(static_cast<int8_t>(w.out.size()));
            for (size_t k = 0; k < w.out.size(); ++k) r.code.push_back(0);
        }
        for (const Leaf& l : w.out) {
            r.s.push_back(l.s);
            r.d.push_back(l.d);
        }
        ++li;
    }

    // The result adds the leaves' contributions; A(B(x)) adds B's offsets
    // first. They agree when the digits of B's leaves, written in A's mixed
    // radix, never carry: the per-digit maxima sum below each extent. When
    // they might carry, decide by checking every coordinate.
    bool no_carry = true;
    for (size_t k = 0; k < a.size(); ++k)
        if (digit_sum[k] > a[k].s - 1) no_carry = false;
    if (!no_carry) {
        int64_t nB;
        st = tree_size(B, &nB);
        if (st != LT_OK) return st;
        if (nB > (int64_t(1) << 26)) return LT_ERR_UNSUPPORTED;
        for (int64_t x = 0; x < nB; ++x) {
            int64_t b, ab, rx;
            tree_eval(B, x, &b);
            if (b >= sizeA) return LT_ERR_NOT_ADMISSIBLE;
            tree_eval(A, b, &ab);
            tree_eval(r, x, &rx);
            if (ab != rx) return LT_ERR_NOT_ADMISSIBLE;
        }
    }
    if (r.s.size() > LT_MAX_LEAVES || r.code.size() > LT_MAX_NODES) return LT_ERR_CAPACITY;
    *out = std::move(r);
    return LT_OK;
}

// ---------------------------------------------------------------------------
// complement
// ---------------------------------------------------------------------------

// B's leaves with a positive stride, taken in increasing stride order, must
// each start where the footprint of the smaller ones ends (or at a multiple
// of it); every gap becomes a complement leaf, and a last leaf runs up to M
// ("Layouts as Algebra", "Divide is tiling": the layout of what B misses).
lt_status complement(const Tree& B, int64_t M, Tree* out) {
    if (empty(B)) return LT_ERR_INVALID_LAYOUT;
    if (M < 1) return LT_ERR_INVALID_ARGUMENT;
    std::vector<Leaf> live;
    for (size_t i = 0; i < B.s.size(); ++i)
        if (B.d[i] > 0 && B.s[i] > 1) live.push_back({B.s[i], B.d[i]});
    std::sort(live.begin(), live.end(), [](const Leaf& x, const Leaf& y) {
        return x.d != y.d ? x.d < y.d : x.s < y.s;
    });
    std::vector<std::pair<int64_t, int64_t>> gaps;
    int64_t covered = 1;
    for (const Leaf& l : live) {
        if (l.d % covered != 0) return LT_ERR_NOT_ADMISSIBLE;
        gaps.emplace_back(l.d / covered, covered);
        if (!mul_ok(l.s, l.d, &covered)) return LT_ERR_OUT_OF_RANGE;
    }
    if (M < covered || M % covered != 0) return LT_ERR_NOT_ADMISSIBLE;
    gaps.emplace_back(M / covered, covered);
    *out = coalesce(Tree::flat(gaps));
    return LT_OK;
}

// ---------------------------------------------------------------------------
// divides
// ---------------------------------------------------------------------------

namespace {

lt_status divide_mode(const Tree& m, int64_t b, Tree* tile, Tree* rest) {
    int64_t n;
    lt_status st = tree_size(m, &n);
    if (st != LT_OK) return st;
    if (b < 1) return LT_ERR_INVALID_ARGUMENT;
    if (n % b != 0) return LT_ERR_NOT_DIVISIBLE;
    Tree bl = Tree::leaf(b, 1);
    Tree bc;
    st = complement(bl, n, &bc);
    if (st != LT_OK) return st;
    Tree r;
    st = compose(m, Tree::tuple({bl, bc}), &r);
    if (st != LT_OK) return st;
    std::vector<Tree> two = r.modes();
    *tile = two[0];
    *rest = two[1];
    return LT_OK;
}

}  // namespace

lt_status divide_shape(const Tree& A, int n, const int64_t* tiler, bool zipped, Tree* out) {
    if (empty(A)) return LT_ERR_INVALID_LAYOUT;
    std::vector<Tree> modes = A.modes();
    if (n < 1 || n > static_cast<int>(modes.size()) || !tiler) return LT_ERR_INVALID_ARGUMENT;
    std::vector<Tree> tiles, rests, parts;
    for (int i = 0; i < n; ++i) {
        Tree t, r;
        lt_status st = divide_mode(modes[i], tiler[i], &t, &r);
        if (st != LT_OK) return st;
        tiles.push_back(t);
        rests.push_back(r);
        parts.push_back(Tree::tuple({t, r}));
    }
    for (size_t i = n; i < modes.size(); ++i) {
        rests.push_back(modes[i]);
        parts.push_back(modes[i]);
    }
    Tree res = zipped ? Tree::tuple({Tree::tuple(tiles), Tree::tuple(rests)}) : Tree::tuple(parts);
    if (res.s.size() > LT_MAX_LEAVES || res.code.size() > LT_MAX_NODES) return LT_ERR_CAPACITY;
    *out = std::move(res);
    return LT_OK;
}

// ---------------------------------------------------------------------------
// products and thread-value layouts
// ---------------------------------------------------------------------------

// logical_product(A, B) = (A, complement(A, size(A) * cosize(B)) o B): mode 0
// is the tile A, mode 1 lays copies of it out in the pattern B, each copy in
// the room A leaves free ("Layouts as Algebra", "Divide is tiling": the
// mirror of logical_divide = A o (B, B*)).
lt_status logical_product(const Tree& A, const Tree& B, Tree* out) {
    if (empty(A) || empty(B)) return LT_ERR_INVALID_LAYOUT;
    int64_t na, cb, M;
    lt_status st = tree_size(A, &na);
    if (st != LT_OK) return st;
    st = tree_cosize(B, &cb);
    if (st != LT_OK) return st;
    if (!mul_ok(na, cb, &M)) return LT_ERR_OUT_OF_RANGE;
    Tree ac, rep;
    st = complement(A, M, &ac);
    if (st != LT_OK) return st;
    st = compose(ac, B, &rep);
    if (st != LT_OK) return st;
    Tree res = Tree::tuple({A, rep});
    if (res.s.size() > LT_MAX_LEAVES || res.code.size() > LT_MAX_NODES) return LT_ERR_CAPACITY;
    *out = std::move(res);
    return LT_OK;
}

// Thread-value layout of a column-major tile with extent thr[i]*val[i] in
// mode i ("Layouts as Algebra", "The threads are a layout too"). Per mode:
// interleaved, logical_product(T:1, V:1) = (T,V):(1,T) (on one step the
// threads take consecutive offsets); blocked, logical_product(V:1, T:1) with
// its two modes swapped = (T,V):(V,1) (each thread owns a run of V). Each
// mode's pair is composed with the tile's mode layout E_i:S_i (S_i the
// product of the earlier extents), and the modes are zipped into
// ((T_0,...),(V_0,...)).
lt_status make_tv(int n, const int64_t* thr, const int64_t* val, const uint8_t* blocked, Tree* out) {
    if (n < 1 || n > 8 || !thr || !val) return LT_ERR_INVALID_ARGUMENT;
    std::vector<Tree> tm, vm;
    int64_t stride = 1;
    for (int i = 0; i < n; ++i) {
        if (thr[i] < 1 || val[i] < 1) return LT_ERR_INVALID_LAYOUT;
        const bool blk = blocked && blocked[i];
        Tree p;
        lt_status st = blk ? logical_product(Tree::leaf(val[i], 1), Tree::leaf(thr[i], 1), &p)
                           : logical_product(Tree::leaf(thr[i], 1), Tree::leaf(val[i], 1), &p);
        if (st != LT_OK) return st;
        if (blk) p = Tree::tuple({p.mode(1), p.mode(0)});
        int64_t ext;
        if (!mul_ok(thr[i], val[i], &ext)) return LT_ERR_OUT_OF_RANGE;
        Tree scaled;
        st = compose(Tree::leaf(ext, stride), p, &scaled);
        if (st != LT_OK) return st;
        tm.push_back(scaled.mode(0));
        vm.push_back(scaled.mode(1));
        if (!mul_ok(stride, ext, &stride)) return LT_ERR_OUT_OF_RANGE;
    }
    Tree res = n == 1 ? Tree::tuple({tm[0], vm[0]}) : Tree::tuple({Tree::tuple(tm), Tree::tuple(vm)});
    if (res.s.size() > LT_MAX_LEAVES || res.code.size() > LT_MAX_NODES) return LT_ERR_CAPACITY;
    *out = std::move(res);
    return LT_OK;
}

// ---------------------------------------------------------------------------
// text
// ---------------------------------------------------------------------------

namespace {

void fmt_part(const Tree& t, const std::vector<int64_t>& vals, size_t* pos, size_t* leaf, std::string* o) {
    int8_t c = t.code[(*pos)++];
    if (c == 0) {
        *o += std::to_string(vals[(*leaf)++]);
        return;
    }
    *o += '(';
    for (int k = 0; k < c; ++k) {
        if (k) *o += ',';
        fmt_part(t, vals, pos, leaf, o);
    }
    *o += ')';
}

struct Parser {
    const char* p;
    std::vector<int8_t> code;
    std::vector<int64_t> vals;
    bool ok = true;

    void skip() {
        while (*p == ' ' || *p == '_' || *p == '\t' || *p == '\n') ++p;
    }
    void node() {
        skip();
        if (*p == '(') {
            ++p;
            size_t at = code.size();
            code.push_back(0);
            int k = 0;
            for (;;) {
                node();
                if (!ok) return;
                ++k;
                skip();
                if (*p == ',') {
                    ++p;
                    continue;
                }
                if (*p == ')') {
                    ++p;
                    break;
                }
                ok = false;
                return;
            }
            if (k > 127) {
                ok = false;
                return;
            }
            code[at] = static_cast<int8_t>(k);
            return;
        }
        if (!std::isdigit(static_cast<unsigned char>(*p))) {
            ok = false;
            return;
        }
        int64_t v = 0;
        while (std::isdigit(static_cast<unsigned char>(*p))) {
            if (!mul_ok(v, 10, &v) || !add_ok(v, *p - '0', &v)) {
                ok = false;
                return;
            }
            ++p;
        }
        code.push_back(0);
        vals.push_back(v);
    }
};

}  // namespace

std::string format(const Tree& t) {
    std::string o;
    size_t pos = 0, leaf = 0;
    fmt_part(t, t.s, &pos, &leaf, &o);
    o += ':';
    pos = 0;
    leaf = 0;
    fmt_part(t, t.d, &pos, &leaf, &o);
    return o;
}

}  // namespace lt

// ===========================================================================
// C ABI
// ===========================================================================

using lt::Tree;

extern "C" {

const char* lt_status_string(lt_status s) {
    switch (s) {
        case LT_OK: return "ok";
        case LT_ERR_INVALID_ARGUMENT: return "invalid argument";
        case LT_ERR_INVALID_LAYOUT: return "invalid layout (incongruent tree, extent < 1 or stride < 0)";
        case LT_ERR_NOT_ADMISSIBLE: return "not admissible: no layout represents this composition/complement";
        case LT_ERR_NOT_DIVISIBLE: return "tiler does not divide the shape";
        case LT_ERR_OUT_OF_RANGE: return "index or coordinate out of range, or int64 overflow";
        case LT_ERR_MISALIGNED_OPERAND: return "misaligned operand: 16-bit operands need 16-byte aligned bases and strides";
        case LT_ERR_UNSUPPORTED: return "unsupported layout/dtype combination";
        case LT_ERR_ARCH_MISMATCH: return "architecture mismatch: this library runs on gfx950 only";
        case LT_ERR_LDS_OVERFLOW: return "tile and stages exceed the LDS budget";
        case LT_ERR_WORKSPACE: return "workspace missing or too small";
        case LT_ERR_HIP: return "HIP runtime error";
        case LT_ERR_CAPACITY: return "capacity exceeded (layout leaves/nodes or text buffer)";
    }
    return "unknown status";
}

lt_status lt_layout_validate(const lt_layout* L) {
    Tree t;
    return lt::from_pod(L, &t);
}

lt_status lt_layout_parse(const char* text, lt_layout* out) {
    if (!text || !out) return LT_ERR_INVALID_ARGUMENT;
    lt::Parser ps{text};
    ps.node();
    if (!ps.ok) return LT_ERR_INVALID_ARGUMENT;
    std::vector<int8_t> shape_code = ps.code;
    std::vector<int64_t> shape = ps.vals;
    ps.skip();
    if (*ps.p != ':') return LT_ERR_INVALID_ARGUMENT;
    ++ps.p;
    ps.code.clear();
    ps.vals.clear();
    ps.node();
    if (!ps.ok) return LT_ERR_INVALID_ARGUMENT;
    ps.skip();
    if (*ps.p != '\0') return LT_ERR_INVALID_ARGUMENT;
    if (ps.code != shape_code) return LT_ERR_INVALID_LAYOUT;   // not congruent
    Tree t{shape_code, shape, ps.vals};
    for (size_t i = 0; i < t.s.size(); ++i)
        if (t.s[i] < 0) return LT_ERR_INVALID_LAYOUT;
    int64_t n;
    lt_status st = lt::tree_size(t, &n);
    if (st != LT_OK) return st;
    return lt::to_pod(t, out);
}

lt_status lt_layout_format(const lt_layout* L, char* buf, size_t cap, size_t* needed) {
    Tree t;
    lt_status st = lt::from_pod(L, &t);
    if (st != LT_OK) return st;
    std::string s = lt::format(t);
    if (needed) *needed = s.size() + 1;
    if (!buf || cap < s.size() + 1) return LT_ERR_CAPACITY;
    std::memcpy(buf, s.c_str(), s.size() + 1);
    return LT_OK;
}

lt_status lt_make_layout(int32_t rank, const int64_t* shape, const int64_t* stride, lt_layout* out) {
    if (rank < 1 || rank > LT_MAX_LEAVES || !shape || !stride || !out) return LT_ERR_INVALID_ARGUMENT;
    std::vector<std::pair<int64_t, int64_t>> p;
    for (int i = 0; i < rank; ++i) {
        if (shape[i] < 0 || stride[i] < 0) return LT_ERR_INVALID_LAYOUT;
        p.emplace_back(shape[i], stride[i]);
    }
    Tree t = Tree::flat(p);
    int64_t n;
    lt_status st = lt::tree_size(t, &n);
    if (st != LT_OK) return st;
    return lt::to_pod(t, out);
}

static lt_status make_compact(int32_t rank, const int64_t* shape, bool colmajor, lt_layout* out) {
    if (rank < 1 || rank > LT_MAX_LEAVES || !shape || !out) return LT_ERR_INVALID_ARGUMENT;
    std::vector<int64_t> st(rank);
    int64_t run = 1;
    for (int k = 0; k < rank; ++k) {
        int i = colmajor ? k : rank - 1 - k;
        if (shape[i] < 0) return LT_ERR_INVALID_LAYOUT;
        st[i] = run;
        if (__builtin_mul_overflow(run, shape[i], &run)) return LT_ERR_OUT_OF_RANGE;
    }
    return lt_make_layout(rank, shape, st.data(), out);
}

lt_status lt_make_colmajor(int32_t rank, const int64_t* shape, lt_layout* out) {
    return make_compact(rank, shape, true, out);
}

lt_status lt_make_rowmajor(int32_t rank, const int64_t* shape, lt_layout* out) {
    return make_compact(rank, shape, false, out);
}

lt_status lt_make_tuple(int32_t n, const lt_layout* modes, lt_layout* out) {
    if (n < 1 || n > 127 || !modes || !out) return LT_ERR_INVALID_ARGUMENT;
    std::vector<Tree> kids(n);
    for (int i = 0; i < n; ++i) {
        lt_status st = lt::from_pod(&modes[i], &kids[i]);
        if (st != LT_OK) return st;
    }
    Tree t = Tree::tuple(kids);
    int64_t sz;
    lt_status st = lt::tree_size(t, &sz);
    if (st != LT_OK) return st;
    return lt::to_pod(t, out);
}

lt_status lt_mode(const lt_layout* L, int32_t i, lt_layout* out) {
    Tree t;
    lt_status st = lt::from_pod(L, &t);
    if (st != LT_OK) return st;
    if (!out || i < 0 || i >= t.rank()) return LT_ERR_INVALID_ARGUMENT;
    return lt::to_pod(t.mode(i), out);
}

lt_status lt_size(const lt_layout* L, int64_t* out) {
    Tree t;
    lt_status st = lt::from_pod(L, &t);
    if (st != LT_OK) return st;
    if (!out) return LT_ERR_INVALID_ARGUMENT;
    return lt::tree_size(t, out);
}

lt_status lt_cosize(const lt_layout* L, int64_t* out) {
    Tree t;
    lt_status st = lt::from_pod(L, &t);
    if (st != LT_OK) return st;
    if (!out) return LT_ERR_INVALID_ARGUMENT;
    return lt::tree_cosize(t, out);
}

lt_status lt_rank(const lt_layout* L, int32_t* out) {
    Tree t;
    lt_status st = lt::from_pod(L, &t);
    if (st != LT_OK) return st;
    if (!out) return LT_ERR_INVALID_ARGUMENT;
    *out = t.rank();
    return LT_OK;
}

lt_status lt_depth(const lt_layout* L, int32_t* out) {
    Tree t;
    lt_status st = lt::from_pod(L, &t);
    if (st != LT_OK) return st;
    if (!out) return LT_ERR_INVALID_ARGUMENT;
    // depth = deepest tuple nesting; walk the preorder code with a stack of
    // remaining children per open tuple.
    int depth = 0;
    std::vector<int> open;
    for (int8_t c : t.code) {
        if (!open.empty()) --open.back();
        if (c > 0) {
            open.push_back(c);
            depth = std::max<int>(depth, static_cast<int>(open.size()));
        }
        while (!open.empty() && open.back() == 0) open.pop_back();
    }
    *out = depth;
    return LT_OK;
}

lt_status lt_eval_index(const lt_layout* L, int64_t idx, int64_t* offset) {
    Tree t;
    lt_status st = lt::from_pod(L, &t);
    if (st != LT_OK) return st;
    if (!offset) return LT_ERR_INVALID_ARGUMENT;
    return lt::tree_eval(t, idx, offset);
}

lt_status lt_eval_coord(const lt_layout* L, const int64_t* coord, int32_t ncoord, int64_t* offset) {
    Tree t;
    lt_status st = lt::from_pod(L, &t);
    if (st != LT_OK) return st;
    if (!coord || !offset) return LT_ERR_INVALID_ARGUMENT;
    int64_t off = 0;
    if (ncoord == static_cast<int32_t>(t.s.size())) {
        // natural coordinate: one entry per leaf
        for (size_t i = 0; i < t.s.size(); ++i) {
            if (coord[i] < 0 || coord[i] >= t.s[i]) return LT_ERR_OUT_OF_RANGE;
            off += coord[i] * t.d[i];
        }
        *offset = off;
        return LT_OK;
    }
    if (ncoord != t.rank()) return LT_ERR_INVALID_ARGUMENT;
    std::vector<Tree> ms = t.modes();
    for (int i = 0; i < ncoord; ++i) {
        int64_t v;
        st = lt::tree_eval(ms[i], coord[i], &v);
        if (st != LT_OK) return st;
        off += v;
    }
    *offset = off;
    return LT_OK;
}

lt_status lt_coalesce(const lt_layout* L, lt_layout* out) {
    Tree t;
    lt_status st = lt::from_pod(L, &t);
    if (st != LT_OK) return st;
    if (!out) return LT_ERR_INVALID_ARGUMENT;
    if (lt::empty(t)) return LT_ERR_INVALID_LAYOUT;
    return lt::to_pod(lt::coalesce(t), out);
}

lt_status lt_compose(const lt_layout* A, const lt_layout* B, lt_layout* out) {
    Tree a, b, r;
    lt_status st = lt::from_pod(A, &a);
    if (st != LT_OK) return st;
    st = lt::from_pod(B, &b);
    if (st != LT_OK) return st;
    if (!out) return LT_ERR_INVALID_ARGUMENT;
    st = lt::compose(a, b, &r);
    if (st != LT_OK) return st;
    return lt::to_pod(r, out);
}

lt_status lt_complement(const lt_layout* B, int64_t M, lt_layout* out) {
    Tree b, r;
    lt_status st = lt::from_pod(B, &b);
    if (st != LT_OK) return st;
    if (!out) return LT_ERR_INVALID_ARGUMENT;
    st = lt::complement(b, M, &r);
    if (st != LT_OK) return st;
    return lt::to_pod(r, out);
}

lt_status lt_logical_divide(const lt_layout* A, const lt_layout* tiler, lt_layout* out) {
    Tree a, b, bc, r;
    lt_status st = lt::from_pod(A, &a);
    if (st != LT_OK) return st;
    st = lt::from_pod(tiler, &b);
    if (st != LT_OK) return st;
    if (!out) return LT_ERR_INVALID_ARGUMENT;
    if (lt::empty(a) || lt::empty(b)) return LT_ERR_INVALID_LAYOUT;
    int64_t na, nb;
    lt::tree_size(a, &na);
    lt::tree_size(b, &nb);
    if (na % nb != 0) return LT_ERR_NOT_DIVISIBLE;
    st = lt::complement(b, na, &bc);
    if (st != LT_OK) return st;
    st = lt::compose(a, Tree::tuple({b, bc}), &r);
    if (st != LT_OK) return st;
    return lt::to_pod(r, out);
}

lt_status lt_logical_product(const lt_layout* A, const lt_layout* B, lt_layout* out) {
    Tree a, b, r;
    lt_status st = lt::from_pod(A, &a);
    if (st != LT_OK) return st;
    st = lt::from_pod(B, &b);
    if (st != LT_OK) return st;
    if (!out) return LT_ERR_INVALID_ARGUMENT;
    st = lt::logical_product(a, b, &r);
    if (st != LT_OK) return st;
    return lt::to_pod(r, out);
}

lt_status lt_make_tv_layout(int32_t n, const int64_t* thr, const int64_t* val, const uint8_t* blocked,
                            lt_layout* out) {
    if (!out) return LT_ERR_INVALID_ARGUMENT;
    Tree r;
    lt_status st = lt::make_tv(n, thr, val, blocked, &r);
    if (st != LT_OK) return st;
    return lt::to_pod(r, out);
}

lt_status lt_logical_divide_shape(const lt_layout* A, int32_t n, const int64_t* tiler, lt_layout* out) {
    Tree a, r;
    lt_status st = lt::from_pod(A, &a);
    if (st != LT_OK) return st;
    if (!out) return LT_ERR_INVALID_ARGUMENT;
    st = lt::divide_shape(a, n, tiler, false, &r);
    if (st != LT_OK) return st;
    return lt::to_pod(r, out);
}

lt_status lt_zipped_divide(const lt_layout* A, int32_t n, const int64_t* tiler, lt_layout* out) {
    Tree a, r;
    lt_status st = lt::from_pod(A, &a);
    if (st != LT_OK) return st;
    if (!out) return LT_ERR_INVALID_ARGUMENT;
    st = lt::divide_shape(a, n, tiler, true, &r);
    if (st != LT_OK) return st;
    return lt::to_pod(r, out);
}

lt_status lt_local_tile(const lt_layout* A, int32_t n, const int64_t* tiler, const int64_t* coord,
                        const uint8_t* step, int64_t* offset, lt_layout* out) {
    Tree a;
    lt_status st = lt::from_pod(A, &a);
    if (st != LT_OK) return st;
    if (n < 1 || n > LT_MAX_LEAVES || !tiler || !coord || !offset || !out) return LT_ERR_INVALID_ARGUMENT;
    std::vector<int64_t> tl, cd;
    for (int i = 0; i < n; ++i) {
        if (step && !step[i]) continue;
        tl.push_back(tiler[i]);
        cd.push_back(coord[i]);
    }
    if (static_cast<int>(tl.size()) != a.rank()) return LT_ERR_INVALID_ARGUMENT;
    Tree zd;
    st = lt::divide_shape(a, static_cast<int>(tl.size()), tl.data(), true, &zd);
    if (st != LT_OK) return st;
    std::vector<Tree> two = zd.modes();
    std::vector<Tree> tile_modes = two[0].modes();
    std::vector<Tree> rest_modes = two[1].modes();
    int64_t off = 0;
    std::vector<Tree> keep = tile_modes;
    for (size_t i = 0; i < cd.size(); ++i) {
        if (cd[i] < 0) {
            keep.push_back(rest_modes[i]);
            continue;
        }
        int64_t v;
        st = lt::tree_eval(rest_modes[i], cd[i], &v);
        if (st != LT_OK) return st;
        off += v;
    }
    Tree res = keep.size() == tile_modes.size() ? two[0] : Tree::tuple(keep);
    lt_layout tmp;
    st = lt::to_pod(res, &tmp);
    if (st != LT_OK) return st;
    *offset = off;
    *out = tmp;
    return LT_OK;
}

lt_status lt_local_partition(const lt_layout* T, const lt_layout* thr, int64_t t, const uint8_t* step,
                             int64_t* offset, lt_layout* out) {
    Tree tt, th;
    lt_status st = lt::from_pod(T, &tt);
    if (st != LT_OK) return st;
    st = lt::from_pod(thr, &th);
    if (st != LT_OK) return st;
    if (!offset || !out) return LT_ERR_INVALID_ARGUMENT;
    int64_t nthr;
    lt::tree_size(th, &nthr);
    if (t < 0 || t >= nthr) return LT_ERR_OUT_OF_RANGE;
    // Invert thr at t: thr must be a bijection onto [0, size). Sorting the
    // leaves by stride, each stride must equal the product of the extents
    // below it; then leaf i's coordinate is (t / stride_i) mod extent_i.
    std::vector<int> order(th.s.size());
    for (size_t i = 0; i < order.size(); ++i) order[i] = static_cast<int>(i);
    std::sort(order.begin(), order.end(), [&](int x, int y) { return th.d[x] < th.d[y]; });
    int64_t expect = 1;
    std::vector<int64_t> leafc(th.s.size(), 0);
    for (int i : order) {
        if (th.s[i] == 1) continue;
        if (th.d[i] != expect) return LT_ERR_INVALID_ARGUMENT;
        leafc[i] = (t / th.d[i]) % th.s[i];
        expect *= th.s[i];
    }
    // per-mode coordinate: re-ravel the leaf coordinates colex inside each mode
    std::vector<Tree> tmodes = th.modes();
    std::vector<int64_t> thr_shape, thr_coord;
    size_t leaf = 0;
    for (const Tree& m : tmodes) {
        int64_t sz, c = 0, mul = 1;
        lt::tree_size(m, &sz);
        for (size_t k = 0; k < m.s.size(); ++k, ++leaf) {
            c += leafc[leaf] * mul;
            mul *= m.s[k];
        }
        thr_shape.push_back(sz);
        thr_coord.push_back(c);
    }
    std::vector<int64_t> tl, cd;
    for (size_t i = 0; i < thr_shape.size(); ++i) {
        if (step && !step[i]) continue;
        tl.push_back(thr_shape[i]);
        cd.push_back(thr_coord[i]);
    }
    if (tl.empty() || static_cast<int>(tl.size()) > tt.rank()) return LT_ERR_INVALID_ARGUMENT;
    Tree zd;
    st = lt::divide_shape(tt, static_cast<int>(tl.size()), tl.data(), true, &zd);
    if (st != LT_OK) return st;
    std::vector<Tree> two = zd.modes();
    std::vector<Tree> tile_modes = two[0].modes();
    int64_t off = 0;
    for (size_t i = 0; i < cd.size(); ++i) {
        int64_t v;
        st = lt::tree_eval(tile_modes[i], cd[i], &v);
        if (st != LT_OK) return st;
        off += v;
    }
    lt_layout tmp;
    st = lt::to_pod(two[1], &tmp);
    if (st != LT_OK) return st;
    *offset = off;
    *out = tmp;
    return LT_OK;
}

const char* lt_version(void) { return "layout-algebra-tiled-amd 0.1 (gfx950)"; }

}  // extern "C"
