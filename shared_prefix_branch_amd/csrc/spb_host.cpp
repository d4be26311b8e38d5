// spb_host.cpp -- the host half of libspb: request validation, the pass packer
// and metadata builder, metadata upload, kernel-argument checks and the
// floor join.  Pure C++17 plus the HIP runtime's copy call; no kernels here.
//
// Packing follows the pages: inputs are packed into token-budget passes, the
// content read once and every question a branch of the same pass [PyPI
// "spinf-serve 0.1.1", "What it does": Many questions, one read; Throughput].
// Option strings become token tries [PyPI, "Layout": compiler.py]; request
// limits default to the man page's [man page "spinf-serve", PARAMETERS].
#define SPB_HD
#include "spb_meta.h"
#include "spb_launch.h"
#include "../../include/spb.h"

#include <algorithm>
#include <unordered_map>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <new>
#include <set>
#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

using namespace spb;

namespace {

thread_local std::string g_err;

spb_status fail(spb_status code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

spb_status ok() {
  g_err.clear();
  return SPB_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ----------------------------------------------------------------- questions

// One question compiled: its template length and the trie of its options.
struct Question {
  int L = 0;
  int n_nodes = 0;
  int n_opt = 0;
  std::vector<int> node_depth;                  // [n_nodes]
  std::vector<std::vector<int>> node_anc;       // [n_nodes][depth]: node indices of the ancestors, self last
  // scored rows of one branch: 0 = template's last row, 1 + i = node i
  std::vector<std::vector<int>> targets;        // [1 + n_nodes]: distinct next tokens
  // per option: (local scored row, index into that row's targets) per token
  std::vector<std::vector<std::pair<int, int>>> steps;
  int n_targets = 0;
  int n_steps = 0;
  int E() const { return L + n_nodes; }
};

spb_status compile_question(const spb_problem &P, int q, const spb_pack_opts &o, Question &Q) {
  Q.L = P.q_len[q];
  if (Q.L < 1) return fail(SPB_ERR_ARG, "question %d: template length %d < 1", q, Q.L);
  if (Q.L > o.max_query_tokens)
    return fail(SPB_ERR_LIMIT, "question %d: template of %d tokens exceeds max_query_tokens %d", q, Q.L,
                o.max_query_tokens);
  int o0 = P.opt_off[q], o1 = P.opt_off[q + 1];
  if (o1 < o0) return fail(SPB_ERR_ARG, "opt_off not monotone at question %d", q);
  Q.n_opt = o1 - o0;
  if (Q.n_opt < 1) return fail(SPB_ERR_ARG, "question %d has no options", q);
  if (Q.n_opt > o.max_options)
    return fail(SPB_ERR_LIMIT, "question %d: %d options exceed max_options %d", q, Q.n_opt, o.max_options);
  std::vector<std::vector<int>> opts(Q.n_opt);
  std::set<std::vector<int>> seen;
  for (int k = 0; k < Q.n_opt; ++k) {
    int t0 = P.tok_off[o0 + k], t1 = P.tok_off[o0 + k + 1];
    if (t1 < t0) return fail(SPB_ERR_ARG, "tok_off not monotone at option %d", o0 + k);
    int n = t1 - t0;
    if (n < 1) return fail(SPB_ERR_ARG, "question %d option %d is empty", q, k);
    if (n > o.max_option_tokens)
      return fail(SPB_ERR_LIMIT, "question %d option %d: %d tokens exceed max_option_tokens %d", q, k, n,
                  o.max_option_tokens);
    if (n - 1 > kMaxDepth) return fail(SPB_ERR_LIMIT, "option of %d tokens exceeds the trie depth %d", n, kMaxDepth);
    for (int t = t0; t < t1; ++t) {
      if (P.tok[t] < 0 || P.tok[t] >= P.vocab)
        return fail(SPB_ERR_ARG, "question %d option %d: token id %d outside [0, %d)", q, k, P.tok[t], P.vocab);
      opts[k].push_back(P.tok[t]);
    }
    if (!seen.insert(opts[k]).second) return fail(SPB_ERR_ARG, "question %d: option %d is a duplicate", q, k);
  }
  // trie nodes: distinct proper prefixes in first-appearance order
  std::map<std::vector<int>, int> node_of;
  std::vector<std::vector<int>> prefixes;
  for (auto &op : opts)
    for (size_t k = 1; k < op.size(); ++k) {
      std::vector<int> pre(op.begin(), op.begin() + k);
      if (!node_of.count(pre)) {
        node_of[pre] = (int)prefixes.size();
        prefixes.push_back(pre);
      }
    }
  Q.n_nodes = (int)prefixes.size();
  if (Q.E() > 32767) return fail(SPB_ERR_LIMIT, "question %d: template + trie of %d rows exceeds 32767", q, Q.E());
  Q.node_depth.resize(Q.n_nodes);
  Q.node_anc.resize(Q.n_nodes);
  for (int i = 0; i < Q.n_nodes; ++i) {
    const auto &pre = prefixes[i];
    Q.node_depth[i] = (int)pre.size();
    for (size_t k = 1; k <= pre.size(); ++k) {
      std::vector<int> a(pre.begin(), pre.begin() + k);
      Q.node_anc[i].push_back(node_of[a]);
    }
  }
  Q.targets.assign(1 + Q.n_nodes, {});
  Q.steps.assign(Q.n_opt, {});
  for (int k = 0; k < Q.n_opt; ++k) {
    const auto &op = opts[k];
    for (size_t t = 0; t < op.size(); ++t) {
      int src = t == 0 ? 0 : 1 + node_of[std::vector<int>(op.begin(), op.begin() + t)];
      auto &tg = Q.targets[src];
      int idx = -1;
      for (size_t j = 0; j < tg.size(); ++j)
        if (tg[j] == op[t]) idx = (int)j;
      if (idx < 0) {
        idx = (int)tg.size();
        tg.push_back(op[t]);
      }
      Q.steps[k].push_back({src, idx});
    }
    Q.n_steps += (int)op.size();
  }
  for (auto &tg : Q.targets) Q.n_targets += (int)tg.size();
  return SPB_OK;
}

// ----------------------------------------------------------------- plan

// Large host buffers of a plan (rows, item tables, metadata) come from a
// process-wide cache of freed blocks, so a serving loop that packs one batch
// after another reuses memory that is already mapped instead of faulting in
// fresh pages on every pack.  Blocks of 64 KiB .. 64 MiB, in power-of-two
// classes; at most 256 MiB are kept; smaller requests go to operator new.
class BlockCache {
 public:
  static constexpr int kMinLog = 16, kMaxLog = 26;
  static constexpr size_t kKeepBytes = size_t(256) << 20;
  static int cls(size_t bytes) {
    int c = kMinLog;
    while (c <= kMaxLog && (size_t(1) << c) < bytes) ++c;
    return c;
  }
  static void *get(size_t bytes) {
    const int c = cls(bytes);
    if (bytes < (size_t(1) << kMinLog) || c > kMaxLog) return ::operator new(bytes);
    {
      std::lock_guard<std::mutex> g(m());
      auto &fl = lists()[c - kMinLog];
      if (!fl.empty()) {
        void *p = fl.back();
        fl.pop_back();
        kept() -= size_t(1) << c;
        return p;
      }
    }
    return ::operator new(size_t(1) << c);
  }
  static void put(void *p, size_t bytes) {
    const int c = cls(bytes);
    if (bytes < (size_t(1) << kMinLog) || c > kMaxLog) {
      ::operator delete(p);
      return;
    }
    {
      std::lock_guard<std::mutex> g(m());
      if (kept() + (size_t(1) << c) <= kKeepBytes) {
        lists()[c - kMinLog].push_back(p);
        kept() += size_t(1) << c;
        return;
      }
    }
    ::operator delete(p);
  }

 private:
  // never destroyed: plans may be freed while the process exits
  static std::mutex &m() {
    static std::mutex *mu = new std::mutex;
    return *mu;
  }
  static std::vector<void *> *lists() {
    static std::vector<void *> *l = new std::vector<void *>[kMaxLog - kMinLog + 1];
    return l;
  }
  static size_t &kept() {
    static size_t k = 0;
    return k;
  }
};

template <class T>
struct CachedAlloc {
  using value_type = T;
  CachedAlloc() = default;
  template <class U>
  CachedAlloc(const CachedAlloc<U> &) {}
  T *allocate(size_t n) { return static_cast<T *>(BlockCache::get(n * sizeof(T))); }
  void deallocate(T *p, size_t n) { BlockCache::put(p, n * sizeof(T)); }
  template <class U>
  bool operator==(const CachedAlloc<U> &) const { return true; }
  template <class U>
  bool operator!=(const CachedAlloc<U> &) const { return false; }
};
template <class T>
using cvec = std::vector<T, CachedAlloc<T>>;

struct PassPlan {
  int n_tokens = 0;
  int n_segments = 0;
  int64_t pairs = 0;
  cvec<int64_t> logical_row;
  cvec<int32_t> pos;  // position of each row on its own root path
  cvec<SpbRow> rows;
  cvec<SpbTile> tiles;
  std::vector<SpbBranch> branches;
  cvec<SpbItem> items[3];
  cvec<SpbChunk> bchunks;
  struct HostStem {
    int start, L, pre, post, parent;  // parent: index in stems, -1 none
  };
  std::vector<HostStem> stems;  // stems placed in this pass, in placement order
  int stem_base = 0;            // next free DFS number in this pass
  std::vector<int32_t> logical_branch;
  std::vector<int32_t> scored, tgt_off, tgt_tok, opt_step_off, step_slot, step_row;
  struct Blob {  // the pass metadata, allocated without a zero fill
    unsigned char *p = nullptr;
    size_t n = 0;
    Blob() = default;
    Blob(const Blob &) = delete;
    Blob &operator=(const Blob &) = delete;
    Blob(Blob &&o) noexcept : p(o.p), n(o.n) { o.p = nullptr; o.n = 0; }
    Blob &operator=(Blob &&o) noexcept {
      if (this != &o) {
        reset(0);
        p = o.p;
        n = o.n;
        o.p = nullptr;
        o.n = 0;
      }
      return *this;
    }
    ~Blob() { reset(0); }
    void reset(size_t bytes) {
      if (p) BlockCache::put(p, n);
      p = bytes ? static_cast<unsigned char *>(BlockCache::get(bytes)) : nullptr;
      n = bytes;
    }
    unsigned char *data() { return p; }
    const unsigned char *data() const { return p; }
    size_t size() const { return n; }
  } blob;
};

}  // namespace

struct spb_plan {
  std::vector<PassPlan> passes;
  bool floors = false;
  int n_content_branches = 0, n_content_options = 0;
  std::vector<int> lb_question, lb_pass, lb_slot;  // per logical branch (content, then floors)
  std::vector<int> content_opt_off;                // [n_content_branches + 1]
  std::vector<int> floor_lb_of_q;                  // question -> logical branch of its floor, -1
  std::vector<int> q_nopt;
  std::vector<int64_t> input_row_off;   // [n_logical_inputs + 1]
  std::vector<int32_t> input_floor_q;   // [n_logical_inputs]
};

namespace {

// A run of template tokens shared by several of one input's questions.
struct Stem {
  int len;            // tokens
  int parent;         // index of the enclosing stem, -1 = none (below the content)
  int pre, post;      // DFS interval among the input's stems (pre < post)
  int64_t first_row;  // logical row of its first token
  int chain_len;      // tokens of its ancestors (not counting itself)
};

struct Unit {  // one logical input to place
  int C;
  int64_t first_row;                 // logical row of its first token
  std::vector<int> qs;               // questions (branches) in order
  std::vector<int> lbs;              // logical branch id of each branch
  std::vector<int64_t> br_first_row; // logical row of each branch's own template token 0
  std::vector<int> own_L;            // per branch: own template tokens (after its shared ones)
  std::vector<int> br_stem;          // per branch: deepest stem on its path, -1 none
  std::vector<Stem> stems;
  int E(size_t bi, const std::vector<Question> &Q) const { return own_L[bi] + Q[qs[bi]].n_nodes; }
  int chain(size_t bi) const { return br_stem[bi] < 0 ? 0 : stems[br_stem[bi]].chain_len + stems[br_stem[bi]].len; }
};

// Shared template prefixes of an input: a proper prefix (never the last token)
// of a question's template is shared when at least two of the input's
// questions start with it.  Shared tokens form stems, each a run that ends
// where a question leaves the shared part or the shared trie branches; stems
// are numbered (and their tokens given logical rows) at first appearance in
// question order.  tmpl: the template of each question (empty: none given).
void build_stems(Unit &u, const std::vector<Question> &Q, const std::vector<std::vector<int>> &tmpl) {
  const size_t nb = u.qs.size();
  u.own_L.assign(nb, 0);
  u.br_stem.assign(nb, -1);
  for (size_t b = 0; b < nb; ++b) u.own_L[b] = Q[u.qs[b]].L;
  if (tmpl.empty() || nb < 2) return;
  // trie of the questions' proper template prefixes (node 0: the empty
  // prefix); cnt[n]: questions of which node n's prefix is a proper prefix.
  // cnt never grows along a path, so a question's shared tokens are the
  // leading nodes of its path with cnt >= 2.
  std::unordered_map<uint64_t, int> child;
  std::vector<int> cnt(1, 0), par(1, -1);
  std::vector<std::vector<int>> path(nb);
  for (size_t b = 0; b < nb; ++b) {
    const auto &T = tmpl[u.qs[b]];
    int n = 0;
    for (size_t k = 0; k + 1 < T.size(); ++k) {
      const uint64_t key = ((uint64_t)(uint32_t)n << 32) | (uint32_t)T[k];
      auto it = child.find(key);
      if (it == child.end()) {
        it = child.emplace(key, (int)cnt.size()).first;
        cnt.push_back(0);
        par.push_back(n);
      }
      n = it->second;
      cnt[n]++;
      path[b].push_back(n);
    }
  }
  const int nn = (int)cnt.size();
  std::vector<int> s(nb, 0);
  for (size_t b = 0; b < nb; ++b)
    while (s[b] < (int)path[b].size() && cnt[path[b][s[b]]] >= 2) ++s[b];
  // per shared node: its shared children, and whether some question's shared
  // part ends there
  std::vector<int> nkids(nn, 0), seg_of(nn, -1);
  std::vector<char> exits(nn, 0);
  for (int n = 1; n < nn; ++n)
    if (cnt[n] >= 2) nkids[par[n]]++;
  for (size_t b = 0; b < nb; ++b)
    if (s[b] > 0) exits[path[b][s[b] - 1]] = 1;
  for (size_t b = 0; b < nb; ++b) {
    for (int k = 1; k <= s[b]; ++k) {
      const int n = path[b][k - 1];
      if (seg_of[n] >= 0) continue;
      int parent = -1;
      if (k > 1) {
        const int up = path[b][k - 2];
        if (!exits[up] && nkids[up] == 1) {  // the run continues
          seg_of[n] = seg_of[up];
          u.stems[seg_of[up]].len++;
          continue;
        }
        parent = seg_of[up];
      }
      Stem st{};
      st.len = 1;
      st.parent = parent;
      seg_of[n] = (int)u.stems.size();
      u.stems.push_back(st);
    }
    if (s[b] > 0) u.br_stem[b] = seg_of[path[b][s[b] - 1]];
    u.own_L[b] = (int)tmpl[u.qs[b]].size() - s[b];
  }
  // DFS numbering (children in creation order) and ancestor token counts
  const int ns = (int)u.stems.size();
  std::vector<std::vector<int>> ch(ns);
  std::vector<int> roots;
  for (int i = 0; i < ns; ++i) (u.stems[i].parent < 0 ? roots : ch[u.stems[i].parent]).push_back(i);
  int clock = 0;
  std::vector<std::pair<int, int>> stack;  // (stem, next child)
  for (int r : roots) {
    u.stems[r].pre = clock++;
    u.stems[r].chain_len = 0;
    stack.push_back({r, 0});
    while (!stack.empty()) {
      auto &top = stack.back();
      if (top.second < (int)ch[top.first].size()) {
        const int c = ch[top.first][top.second++];
        u.stems[c].pre = clock++;
        u.stems[c].chain_len = u.stems[top.first].chain_len + u.stems[top.first].len;
        stack.push_back({c, 0});
      } else {
        u.stems[top.first].post = clock++;
        stack.pop_back();
      }
    }
  }
}

struct Packer {
  const std::vector<Question> &Q;
  int B;
  std::vector<PassPlan> passes;
  int group_start = 0;      // first row of the current tiling group in the current pass
  bool group_empty_content = false;
  std::vector<std::pair<int, int>> groups;  // per current pass: [g0, g1) tiling groups
  std::vector<std::vector<std::pair<int, int>>> pass_groups;
  std::vector<int> group_seg;               // content start of each group
  std::vector<std::vector<int>> pass_group_seg;

  explicit Packer(const std::vector<Question> &q, int budget) : Q(q), B(budget) { open(); }

  PassPlan &cur() { return passes.back(); }
  int fill() { return (int)cur().rows.size(); }

  void open() {
    passes.emplace_back();
    passes.back().rows.reserve((size_t)std::min(B, 1 << 16));
    passes.back().logical_row.reserve((size_t)std::min(B, 1 << 16));
    passes.back().pos.reserve((size_t)std::min(B, 1 << 16));
    pass_groups.emplace_back();
    pass_group_seg.emplace_back();
  }
  void close_if_nonempty() {
    if (!cur().rows.empty()) open();
  }

  // starts a tiling group for a content segment, or joins the running run of
  // empty-content units
  void begin_group(int C) {
    auto &G = pass_groups.back();
    auto &S = pass_group_seg.back();
    int f = fill();
    if (C == 0 && !G.empty() && S.back() < 0 && G.back().second == f) return;  // extend the C=0 run
    G.push_back({f, f});
    S.push_back(C > 0 ? f : -1);
  }
  void end_rows() { pass_groups.back().back().second = fill(); }

  void place_content(const Unit &u, int &seg) {
    begin_group(u.C);
    PassPlan &P = cur();
    seg = fill();
    for (int t = 0; t < u.C; ++t) {
      SpbRow r{};
      r.cvis = t + 1;
      r.seg = seg;
      r.br = -1;
      r.e = t;
      r.spre = -1;
      P.rows.push_back(r);
      P.logical_row.push_back(u.first_row + t);
      P.pos.push_back(t);
      P.pairs += t + 1;
    }
    if (u.C > 0) P.n_segments++;
    end_rows();
  }

  // Stem placement state of the unit being placed in the current pass: the
  // pass row of each stem placed (-1 not yet) and the pass's DFS base.
  std::vector<int> stem_start, stem_index;
  int stem_base = 0;
  void reset_stems(const Unit &u) {
    stem_start.assign(u.stems.size(), -1);
    stem_index.assign(u.stems.size(), -1);
    stem_base = cur().stem_base;
    cur().stem_base += 2 * (int)u.stems.size();
  }
  // places stem s (after its ancestors) unless the pass already holds it
  void place_stem(const Unit &u, int s, int seg) {
    if (stem_start[s] >= 0) return;
    const Stem &st = u.stems[s];
    if (st.parent >= 0) place_stem(u, st.parent, seg);
    PassPlan &P = cur();
    const int start = fill();
    stem_start[s] = start;
    stem_index[s] = (int)P.stems.size();
    P.stems.push_back({start, st.len, stem_base + st.pre, stem_base + st.post,
                       st.parent >= 0 ? stem_index[st.parent] : -1});
    for (int j = 0; j < st.len; ++j) {
      SpbRow r{};
      r.cvis = u.C;
      r.seg = u.C > 0 ? seg : start;
      r.br = start;
      r.e = j;
      r.L = st.len;
      r.spre = stem_base + st.pre;
      r.stem = 1;
      P.rows.push_back(r);
      P.logical_row.push_back(st.first_row + j);
      P.pos.push_back(u.C + st.chain_len + j);
      P.pairs += u.C + st.chain_len + j + 1;
    }
    end_rows();
  }
  // stems not yet in the pass that branch bi needs
  int stems_needed(const Unit &u, int bi) const {
    int n = 0;
    for (int s = u.br_stem[bi]; s >= 0; s = u.stems[s].parent)
      if (stem_start[s] < 0) n += u.stems[s].len;
    return n;
  }

  void place_branch(const Unit &u, int bi, int seg, std::vector<int> &lb_pass, std::vector<int> &lb_slot) {
    if (u.br_stem[bi] >= 0) place_stem(u, u.br_stem[bi], seg);
    PassPlan &P = cur();
    const Question &q = Q[u.qs[bi]];
    const int L = u.own_L[bi];
    const int chain = u.chain(bi);
    const int spre = u.br_stem[bi] >= 0 ? stem_base + u.stems[u.br_stem[bi]].pre : -1;
    int start = fill();
    SpbBranch b{};
    b.start = start;
    b.L = L;
    b.E = L + q.n_nodes;
    b.n_opt = q.n_opt;
    b.question = u.qs[bi];
    lb_pass[u.lbs[bi]] = (int)passes.size() - 1;
    lb_slot[u.lbs[bi]] = (int)P.branches.size();
    P.branches.push_back(b);
    P.logical_branch.push_back(u.lbs[bi]);
    for (int j = 0; j < L; ++j) {
      SpbRow r{};
      r.cvis = u.C;
      r.seg = u.C > 0 ? seg : start;
      r.br = start;
      r.e = j;
      r.L = L;
      r.spre = spre;
      P.rows.push_back(r);
      P.logical_row.push_back(u.br_first_row[bi] + j);
      P.pos.push_back(u.C + chain + j);
      P.pairs += u.C + chain + j + 1;
    }
    for (int i = 0; i < q.n_nodes; ++i) {
      SpbRow r{};
      r.cvis = u.C;
      r.seg = u.C > 0 ? seg : start;
      r.br = start;
      r.e = L + i;
      r.L = L;
      r.depth = q.node_depth[i];
      r.spre = spre;
      int a[4] = {0, 0, 0, 0};
      for (int k = 0; k < r.depth; ++k) a[k] = L + q.node_anc[i][k];
      r.anc01 = (int32_t)((uint32_t)a[0] | ((uint32_t)a[1] << 16));
      r.anc23 = (int32_t)((uint32_t)a[2] | ((uint32_t)a[3] << 16));
      P.rows.push_back(r);
      P.logical_row.push_back(u.br_first_row[bi] + L + i);
      P.pos.push_back(u.C + chain + L - 1 + r.depth);
      P.pairs += u.C + chain + L + r.depth;
    }
    end_rows();
  }

  void place(const Unit &u, std::vector<int> &lb_pass, std::vector<int> &lb_slot) {
    int64_t size = u.C;
    for (size_t bi = 0; bi < u.qs.size(); ++bi) size += u.E(bi, Q);
    for (const Stem &s : u.stems) size += s.len;
    int seg = 0;
    if (size <= B - fill() || size <= B) {
      if (size > B - fill()) close_if_nonempty();
      place_content(u, seg);
      reset_stems(u);
      for (size_t bi = 0; bi < u.qs.size(); ++bi) place_branch(u, (int)bi, seg, lb_pass, lb_slot);
      return;
    }
    // larger than a pass: spill at branch boundaries, content and the stems a
    // pass's branches need re-staged
    if (u.C + (u.qs.empty() ? 0 : u.chain(0) + u.E(0, Q)) > B - fill()) close_if_nonempty();
    place_content(u, seg);
    reset_stems(u);
    for (size_t bi = 0; bi < u.qs.size(); ++bi) {
      if (stems_needed(u, (int)bi) + u.E(bi, Q) > B - fill()) {
        open();
        place_content(u, seg);
        reset_stems(u);
      }
      place_branch(u, (int)bi, seg, lb_pass, lb_slot);
    }
  }
};

void build_tiles(PassPlan &P, const std::vector<std::pair<int, int>> &groups, const std::vector<int> &gseg) {
  std::vector<int> branch_at(P.rows.size(), -1);  // branch start row -> index in the branch table
  for (size_t b = 0; b < P.branches.size(); ++b) branch_at[P.branches[b].start] = (int)b;
  for (size_t g = 0; g < groups.size(); ++g) {
    int g0 = groups[g].first, g1 = groups[g].second;
    for (int r0 = g0; r0 < g1; r0 += kTileRows) {
      SpbTile t{};
      t.row0 = r0;
      t.nrows = std::min(kTileRows, g1 - r0);
      t.seg = gseg[g] >= 0 ? gseg[g] : r0;
      int maxc = 0;
      for (int r = r0; r < r0 + t.nrows; ++r) maxc = std::max(maxc, P.rows[r].cvis);
      t.ncc = (maxc + kChunk - 1) / kChunk;
      t.b_lo = t.b_hi = 0;
      // branches intersecting [r0, r0 + nrows): the branch table is in row order
      int lo = -1, hi = -1;
      for (int r = r0; r < r0 + t.nrows; ++r) {
        if (P.rows[r].br < 0 || P.rows[r].stem) continue;
        const int bi = branch_at[P.rows[r].br];
        if (lo < 0) lo = bi;
        hi = bi;
      }
      int bchunks = 0;
      if (lo >= 0) {
        t.b_lo = lo;
        t.b_hi = hi + 1;
        for (int b = lo; b <= hi; ++b) {
          const SpbBranch &B = P.branches[b];
          int last = std::min(B.start + B.E, r0 + t.nrows) - 1 - B.start;
          bchunks += last / kBranchChunk + 1;
        }
      }
      t.cost = t.ncc + bchunks;
      P.tiles.push_back(t);
    }
  }
  // longest work first, so the tail of the grid holds the short items
  std::stable_sort(P.tiles.begin(), P.tiles.end(), [](const SpbTile &a, const SpbTile &b) { return a.cost > b.cost; });
}

// Work items of the bf16 attention kernel at 32, 64 and 128 rows: each tile
// split into row ranges, each with the content chunks its own rows see and the
// chunks of the branches meeting its rows, longest first.
void build_items(PassPlan &P) {
  std::unordered_map<int, int> stem_at;  // pre number -> index in P.stems
  for (size_t s = 0; s < P.stems.size(); ++s) stem_at[P.stems[s].pre] = (int)s;
  cvec<SpbItem> items;
  cvec<SpbChunk> flat;                // chunk lists of the items, in item order
  std::vector<std::pair<int, int>> stems;  // (pre, index) of an item's stems
  std::vector<int> order;
  for (int g = 0; g < 3; ++g) {
    const int rows_per = 32 << g;
    items.clear();
    flat.clear();
    for (const SpbTile &t : P.tiles) {
      for (int r0 = t.row0; r0 < t.row0 + t.nrows; r0 += rows_per) {
        SpbItem it{};
        it.row0 = r0;
        it.nrows = std::min(rows_per, t.row0 + t.nrows - r0);
        it.seg = t.seg;
        it.boff = (int)flat.size();
        int maxc = 0;
        // stems on the paths of the item's rows (a stem row's own stem, a
        // branch row's deepest stem, and their ancestors), root first
        stems.clear();
        int last_spre = -1;
        for (int r = r0; r < r0 + it.nrows; ++r) {
          const SpbRow &R = P.rows[r];
          maxc = std::max(maxc, R.cvis);
          if (R.br < 0 || R.spre < 0 || R.spre == last_spre) continue;
          last_spre = R.spre;
          for (int s = stem_at.at(R.spre); s >= 0; s = P.stems[s].parent) stems.push_back({P.stems[s].pre, s});
        }
        it.ncc = (maxc + kChunk - 1) / kChunk;
        std::sort(stems.begin(), stems.end());
        stems.erase(std::unique(stems.begin(), stems.end()), stems.end());
        for (auto &ps : stems) {
          const auto &S = P.stems[ps.second];
          for (int c = 0; c * kBranchChunk < S.L; ++c) {
            const int nvis = std::min(S.L - c * kBranchChunk, kBranchChunk);
            flat.push_back(SpbChunk{S.start + c * kBranchChunk, kStemChunk | (ps.second << 10) | c, S.pre,
                                    S.post | (nvis << 24)});
          }
        }
        for (int b = t.b_lo; b < t.b_hi; ++b) {
          const SpbBranch &B = P.branches[b];
          if (B.start + B.E <= r0 || B.start >= r0 + it.nrows) continue;
          const int last = std::min(B.start + B.E, r0 + it.nrows) - 1 - B.start;
          for (int c = 0; c <= last / kBranchChunk; ++c)
            flat.push_back(SpbChunk{B.start + c * kBranchChunk, (b << 10) | c, 0, 0});
        }
        it.bn = (int)flat.size() - it.boff;
        it.cost = it.ncc + it.bn;
        items.push_back(it);
      }
    }
    // longest first (stable: ties keep row order)
    order.resize(items.size());
    for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return items[a].cost > items[b].cost; });
    P.items[g].clear();
    P.items[g].reserve(items.size());
    P.bchunks.reserve(P.bchunks.size() + flat.size());
    for (int i : order) {
      SpbItem it = items[i];
      const int src = it.boff;
      it.boff = (int)P.bchunks.size();
      P.bchunks.insert(P.bchunks.end(), flat.begin() + src, flat.begin() + src + it.bn);
      P.items[g].push_back(it);
    }
  }
}

void build_scoring(PassPlan &P, const std::vector<Question> &Q) {
  int opt = 0;
  P.tgt_off.push_back(0);
  P.opt_step_off.push_back(0);
  for (auto &b : P.branches) {
    const Question &q = Q[b.question];
    b.opt0 = opt;
    b.scored0 = (int)P.scored.size();
    b.n_scored = 1 + q.n_nodes;
    P.scored.push_back(b.start + b.L - 1);
    for (int i = 0; i < q.n_nodes; ++i) P.scored.push_back(b.start + b.L + i);
    for (int s = 0; s <= q.n_nodes; ++s) {
      for (int t : q.targets[s]) P.tgt_tok.push_back(t);
      P.tgt_off.push_back((int)P.tgt_tok.size());
    }
    for (int k = 0; k < q.n_opt; ++k) {
      for (auto st : q.steps[k]) {
        int row = b.scored0 + st.first;
        P.step_row.push_back(row);
        P.step_slot.push_back(P.tgt_off[row] + st.second);
      }
      P.opt_step_off.push_back((int)P.step_slot.size());
    }
    opt += q.n_opt;
  }
}

template <class V>
void put(unsigned char *blob, size_t off, const V &v) {
  if (!v.empty()) memcpy(blob + off, v.data(), v.size() * sizeof(v[0]));
}

void build_blob(PassPlan &P, int pass) {
  SpbMetaHeader h{};
  h.magic = kMetaMagic;
  h.version = kMetaVersion;
  h.pass = pass;
  h.n_tokens = (int)P.rows.size();
  h.n_tiles = (int)P.tiles.size();
  h.n_branches = (int)P.branches.size();
  h.n_options = (int)P.opt_step_off.size() - 1;
  h.n_scored = (int)P.scored.size();
  h.n_targets = (int)P.tgt_tok.size();
  h.n_steps = (int)P.step_slot.size();
  size_t off = align256(sizeof(SpbMetaHeader));
  std::vector<std::pair<size_t, size_t>> gaps{{sizeof(SpbMetaHeader), off}};  // padding, zeroed below
  auto place = [&](int64_t &field, size_t bytes) {
    field = (int64_t)off;
    gaps.push_back({off + bytes, align256(off + bytes)});
    off = align256(off + bytes);
  };
  place(h.off_rows, P.rows.size() * sizeof(SpbRow));
  place(h.off_tiles, P.tiles.size() * sizeof(SpbTile));
  place(h.off_branches, P.branches.size() * sizeof(SpbBranch));
  place(h.off_scored, P.scored.size() * 4);
  place(h.off_tgt_off, P.tgt_off.size() * 4);
  place(h.off_tgt_tok, P.tgt_tok.size() * 4);
  place(h.off_opt_step_off, P.opt_step_off.size() * 4);
  place(h.off_step_slot, P.step_slot.size() * 4);
  place(h.off_step_row, P.step_row.size() * 4);
  for (int g = 0; g < 3; ++g) {
    h.n_items[g] = (int)P.items[g].size();
    place(h.off_items[g], P.items[g].size() * sizeof(SpbItem));
  }
  h.n_bchunks = (int)P.bchunks.size();
  place(h.off_bchunks, P.bchunks.size() * sizeof(SpbChunk));
  h.total_bytes = (int64_t)off;
  P.blob.reset(off);
  unsigned char *B = P.blob.data();
  for (auto &g : gaps) memset(B + g.first, 0, g.second - g.first);
  memcpy(B, &h, sizeof h);
  put(B, h.off_rows, P.rows);
  put(B, h.off_tiles, P.tiles);
  put(B, h.off_branches, P.branches);
  put(B, h.off_scored, P.scored);
  put(B, h.off_tgt_off, P.tgt_off);
  put(B, h.off_tgt_tok, P.tgt_tok);
  put(B, h.off_opt_step_off, P.opt_step_off);
  put(B, h.off_step_slot, P.step_slot);
  put(B, h.off_step_row, P.step_row);
  for (int g = 0; g < 3; ++g) put(B, h.off_items[g], P.items[g]);
  put(B, h.off_bchunks, P.bchunks);
  P.n_tokens = h.n_tokens;
}

// Workspace of spb_score_options: slice partials, captured logits, LSE per
// row, gathered hidden states.  Returns the total; off[] gets the offsets.
size_t score_workspace_layout(int n_scored, int n_targets, int vocab, int hidden_dim, int kind, size_t *off) {
  int n_chunks = 0, mb = 0;
  head_m_layout(n_scored, &n_chunks, &mb);
  size_t sizes[4] = {(size_t)n_scored * n_vocab_slices(vocab) * 2 * sizeof(float), (size_t)n_targets * sizeof(float),
                     (size_t)n_scored * sizeof(float),
                     (size_t)n_chunks * 32 * mb * (size_t)hidden_dim * 2 * head_planes(kind)};
  size_t o = 0;
  for (int i = 0; i < 4; ++i) {
    if (off) off[i] = o;
    o += align256(sizes[i]);
  }
  return o;
}

// Workspace of spb_score_options_batch: the single-pass layout over the
// combined rows and targets, then the combined target CSR (offsets, tokens).
size_t score_batch_workspace_layout(int m_tot, int t_tot, int vocab, int hidden_dim, int kind, size_t *off) {
  size_t o4[4];
  size_t o = score_workspace_layout(m_tot, t_tot, vocab, hidden_dim, kind, o4);
  if (off) {
    for (int i = 0; i < 4; ++i) off[i] = o4[i];
    off[4] = o;
  }
  o += align256((size_t)(m_tot + 1) * sizeof(int32_t));
  if (off) off[5] = o;
  o += align256((size_t)(t_tot > 0 ? t_tot : 1) * sizeof(int32_t));
  return o;
}

const SpbMetaHeader &header(const PassPlan &P) { return *reinterpret_cast<const SpbMetaHeader *>(P.blob.data()); }

// Limits of the attention kernel's metadata fields: stem index below bit 20
// of a chunk's info word (below the stem flag), DFS numbers below 2^24, and
// at most kMaxTileChunks key chunks in one work item's list.
spb_status check_attention_limits(const PassPlan &P, int pass) {
  if (P.stems.size() >= (1u << 20) || P.stem_base >= (1 << 24))
    return fail(SPB_ERR_LIMIT, "pass %d holds %zu shared template stems, too many", pass, P.stems.size());
  for (int g = 0; g < 3; ++g)
    for (const SpbItem &it : P.items[g])
      if (it.cost > kMaxTileChunks)
        return fail(SPB_ERR_LIMIT, "pass %d: an attention tile needs %d key chunks, more than %d", pass, it.cost,
                    kMaxTileChunks);
  return ok();
}

spb_status check_pass(const spb_plan *plan, int32_t pass) {
  if (!plan) return fail(SPB_ERR_ARG, "plan is NULL");
  if (pass < 0 || pass >= (int32_t)plan->passes.size())
    return fail(SPB_ERR_ARG, "pass %d outside [0, %zu)", pass, plan->passes.size());
  return SPB_OK;
}

}  // namespace

// ===================================================================== C ABI

extern "C" {

const char *spb_last_error(void) { return g_err.c_str(); }

const char *spb_fingerprint(void) {
  static char fp[160];
  snprintf(fp, sizeof fp, "spb-0.1 gfx950 meta%d attn:rows%d,chunk%d,mfma32x32 head:vslice%d,k64 numerics:1",
           kMetaVersion, kTileRows, kChunk, kVocabTile);
  return fp;
}

void spb_pack_opts_default(spb_pack_opts *o) {
  if (!o) return;
  o->token_budget = 16384;
  o->floors = 1;
  o->max_content_tokens = 4096;
  o->max_query_tokens = 256;
  o->max_options = 1000;
  o->max_option_tokens = 5;
  o->max_prompts_per_input = 10000;
  o->max_processed_tokens = 2000000;
}

spb_status spb_pack_pass(const spb_problem *P, const spb_pack_opts *opts, spb_plan **out) {
  if (!P || !out) return fail(SPB_ERR_ARG, "problem and out must not be NULL");
  *out = nullptr;
  spb_pack_opts o;
  spb_pack_opts_default(&o);
  if (opts) o = *opts;
  if (o.token_budget < 1) return fail(SPB_ERR_ARG, "token_budget %d < 1", o.token_budget);
  if (P->n_inputs < 0 || P->n_questions < 0) return fail(SPB_ERR_ARG, "negative input or question count");
  if (P->vocab < 1) return fail(SPB_ERR_ARG, "vocab %d < 1", P->vocab);
  if ((P->n_inputs > 0 && (!P->content_len || !P->branch_off)) || (P->n_questions > 0 && (!P->q_len || !P->opt_off)))
    return fail(SPB_ERR_ARG, "NULL problem array");
  if (P->n_inputs > 0 && P->branch_off[0] != 0) return fail(SPB_ERR_ARG, "branch_off[0] must be 0");
  if (P->n_questions > 0 && P->opt_off[0] != 0) return fail(SPB_ERR_ARG, "opt_off[0] must be 0");
  int n_opt_total = P->n_questions > 0 ? P->opt_off[P->n_questions] : 0;
  if (n_opt_total < 0) return fail(SPB_ERR_ARG, "opt_off not monotone");
  if (n_opt_total > 0 && (!P->tok_off || !P->tok)) return fail(SPB_ERR_ARG, "NULL option arrays");
  if (n_opt_total > 0 && P->tok_off[0] != 0) return fail(SPB_ERR_ARG, "tok_off[0] must be 0");
  for (int q = 0; q < P->n_questions; ++q)
    if (P->opt_off[q + 1] < P->opt_off[q]) return fail(SPB_ERR_ARG, "opt_off not monotone at question %d", q);

  std::vector<Question> Q(P->n_questions);
  for (int q = 0; q < P->n_questions; ++q) {
    spb_status s = compile_question(*P, q, o, Q[q]);
    if (s != SPB_OK) return s;
  }
  std::vector<std::vector<int>> tmpl;  // template token ids per question (empty: not given)
  if (P->tmpl_tok) {
    tmpl.resize(P->n_questions);
    int64_t off = 0;
    for (int q = 0; q < P->n_questions; ++q) {
      tmpl[q].assign(P->tmpl_tok + off, P->tmpl_tok + off + Q[q].L);
      off += Q[q].L;
    }
  }
  std::unique_ptr<spb_plan> plan(new (std::nothrow) spb_plan());
  if (!plan) return fail(SPB_ERR_ARG, "out of host memory");
  plan->floors = o.floors != 0;
  plan->q_nopt.resize(P->n_questions);
  for (int q = 0; q < P->n_questions; ++q) plan->q_nopt[q] = Q[q].n_opt;

  // logical units: inputs, then floors
  std::vector<Unit> units;
  int64_t row = 0;
  int lb = 0;
  int64_t processed = 0;
  for (int i = 0; i < P->n_inputs; ++i) {
    Unit u;
    u.C = P->content_len[i];
    if (u.C < 0) return fail(SPB_ERR_ARG, "input %d: content_len %d < 0", i, u.C);
    if (u.C > o.max_content_tokens)
      return fail(SPB_ERR_LIMIT, "input %d: content of %d tokens exceeds max_content_tokens %d", i, u.C,
                  o.max_content_tokens);
    if (u.C > o.token_budget)
      return fail(SPB_ERR_LIMIT, "input %d: content of %d tokens exceeds the token budget %d", i, u.C, o.token_budget);
    int b0 = P->branch_off[i], b1 = P->branch_off[i + 1];
    if (b1 < b0) return fail(SPB_ERR_ARG, "branch_off not monotone at input %d", i);
    if (b1 - b0 > o.max_prompts_per_input)
      return fail(SPB_ERR_LIMIT, "input %d: %d questions exceed max_prompts_per_input %d", i, b1 - b0,
                  o.max_prompts_per_input);
    if (b1 > b0 && !P->branch_q) return fail(SPB_ERR_ARG, "branch_q is NULL");
    u.first_row = row;
    row += u.C;
    for (int b = b0; b < b1; ++b) {
      int q = P->branch_q[b];
      if (q < 0 || q >= P->n_questions) return fail(SPB_ERR_ARG, "input %d asks question %d outside [0, %d)", i, q,
                                                    P->n_questions);
      if ((int64_t)u.C + Q[q].E() > o.token_budget)
        return fail(SPB_ERR_LIMIT, "input %d: content %d + question %d (%d rows) exceeds the token budget %d", i, u.C,
                    q, Q[q].E(), o.token_budget);
      u.qs.push_back(q);
      u.lbs.push_back(lb++);
      plan->lb_question.push_back(q);
    }
    build_stems(u, Q, tmpl);
    // logical rows: per branch, the shared tokens of its template not yet
    // numbered (stems root first), then its own template and trie nodes
    std::vector<char> numbered(u.stems.size(), 0);
    for (size_t bi = 0; bi < u.qs.size(); ++bi) {
      std::vector<int> chain;
      for (int s = u.br_stem[bi]; s >= 0; s = u.stems[s].parent) chain.push_back(s);
      for (auto it = chain.rbegin(); it != chain.rend(); ++it)
        if (!numbered[*it]) {
          numbered[*it] = 1;
          u.stems[*it].first_row = row;
          row += u.stems[*it].len;
        }
      u.br_first_row.push_back(row);
      row += u.E(bi, Q);
    }
    units.push_back(std::move(u));
  }
  plan->n_content_branches = lb;
  plan->content_opt_off.push_back(0);
  for (int b = 0; b < lb; ++b) plan->content_opt_off.push_back(plan->content_opt_off.back() + Q[plan->lb_question[b]].n_opt);
  plan->n_content_options = plan->content_opt_off.back();
  plan->floor_lb_of_q.assign(P->n_questions, -1);
  if (plan->floors) {
    std::vector<char> asked(P->n_questions, 0);
    for (int b = 0; b < lb; ++b) asked[plan->lb_question[b]] = 1;
    for (int q = 0; q < P->n_questions; ++q) {
      if (!asked[q]) continue;
      Unit u;
      u.C = 0;
      u.first_row = row;
      u.qs.push_back(q);
      u.lbs.push_back(lb);
      u.br_first_row.push_back(row);
      build_stems(u, Q, tmpl);  // one question: nothing shared
      plan->floor_lb_of_q[q] = lb++;
      plan->lb_question.push_back(q);
      row += Q[q].E();
      units.push_back(std::move(u));
    }
  }
  for (auto &u : units) {
    plan->input_row_off.push_back(u.first_row);
    plan->input_floor_q.push_back(-1);
  }
  plan->input_row_off.push_back(row);
  for (size_t n = (size_t)P->n_inputs; n < units.size(); ++n) plan->input_floor_q[n] = units[n].qs[0];
  plan->lb_pass.assign(lb, -1);
  plan->lb_slot.assign(lb, -1);

  Packer pk(Q, o.token_budget);
  for (auto &u : units) {
    pk.place(u, plan->lb_pass, plan->lb_slot);
  }
  if (pk.cur().rows.empty() && pk.passes.size() > 1) {
    pk.passes.pop_back();
    pk.pass_groups.pop_back();
    pk.pass_group_seg.pop_back();
  }
  for (auto &p : pk.passes) processed += (int64_t)p.rows.size();
  if (processed > o.max_processed_tokens)
    return fail(SPB_ERR_LIMIT, "%lld processed tokens exceed max_processed_tokens %lld", (long long)processed,
                (long long)o.max_processed_tokens);
  for (size_t k = 0; k < pk.passes.size(); ++k) {
    PassPlan &pp = pk.passes[k];
    build_tiles(pp, pk.pass_groups[k], pk.pass_group_seg[k]);
    build_items(pp);
    // what the attention kernel can run is decided here, so that a plan it
    // would refuse is never handed out (raised limits, e.g. a long content)
    spb_status lim = check_attention_limits(pp, (int)k);
    if (lim != SPB_OK) return lim;
    build_scoring(pp, Q);
    build_blob(pp, (int)k);
  }
  plan->passes = std::move(pk.passes);
  *out = plan.release();
  return ok();
}

void spb_plan_free(spb_plan *plan) { delete plan; }

spb_status spb_plan_num_passes(const spb_plan *plan, int32_t *n) {
  if (!plan || !n) return fail(SPB_ERR_ARG, "NULL argument");
  *n = (int32_t)plan->passes.size();
  return ok();
}

spb_status spb_plan_info(const spb_plan *plan, int32_t pass, spb_pass_info *out) {
  if (!plan || !out) return fail(SPB_ERR_ARG, "NULL argument");
  spb_pass_info s{};
  auto add = [&](const PassPlan &P) {
    const SpbMetaHeader &h = header(P);
    s.n_tokens += h.n_tokens;
    s.n_segments += P.n_segments;
    s.n_branches += h.n_branches;
    s.n_options += h.n_options;
    s.n_scored_rows += h.n_scored;
    s.n_targets += h.n_targets;
    s.n_tiles += h.n_tiles;
    s.unmasked_pairs += P.pairs;
    s.meta_bytes = std::max(s.meta_bytes, P.blob.size());
  };
  if (pass == -1) {
    for (auto &P : plan->passes) add(P);
  } else {
    spb_status st = check_pass(plan, pass);
    if (st != SPB_OK) return st;
    add(plan->passes[pass]);
  }
  s.n_passes = (int32_t)plan->passes.size();
  s.n_content_branches = plan->n_content_branches;
  s.n_content_options = plan->n_content_options;
  s.n_logical_inputs = (int32_t)plan->input_floor_q.size();
  *out = s;
  return ok();
}

spb_status spb_plan_rows(const spb_plan *plan, int32_t pass, int64_t *logical_row, int32_t *scored_row) {
  spb_status st = check_pass(plan, pass);
  if (st != SPB_OK) return st;
  const PassPlan &P = plan->passes[pass];
  if (logical_row) memcpy(logical_row, P.logical_row.data(), P.logical_row.size() * sizeof(int64_t));
  if (scored_row) memcpy(scored_row, P.scored.data(), P.scored.size() * sizeof(int32_t));
  return ok();
}

spb_status spb_plan_positions(const spb_plan *plan, int32_t pass, int32_t *host_out) {
  spb_status st = check_pass(plan, pass);
  if (st != SPB_OK) return st;
  if (!host_out) return fail(SPB_ERR_ARG, "host_out is NULL");
  const PassPlan &P = plan->passes[pass];
  if (!P.pos.empty()) memcpy(host_out, P.pos.data(), P.pos.size() * sizeof(int32_t));
  return ok();
}

spb_status spb_plan_branches(const spb_plan *plan, int32_t pass, int32_t *logical_branch, int32_t *opt_first) {
  spb_status st = check_pass(plan, pass);
  if (st != SPB_OK) return st;
  const PassPlan &P = plan->passes[pass];
  for (size_t b = 0; b < P.branches.size(); ++b) {
    if (logical_branch) logical_branch[b] = P.logical_branch[b];
    if (opt_first) opt_first[b] = P.branches[b].opt0;
  }
  return ok();
}

spb_status spb_plan_inputs(const spb_plan *plan, int64_t *row_off, int32_t *floor_question) {
  if (!plan) return fail(SPB_ERR_ARG, "plan is NULL");
  if (row_off) memcpy(row_off, plan->input_row_off.data(), plan->input_row_off.size() * sizeof(int64_t));
  if (floor_question)
    memcpy(floor_question, plan->input_floor_q.data(), plan->input_floor_q.size() * sizeof(int32_t));
  return ok();
}

}  // extern "C"

namespace {
// The pass rows a row attends to, in attention order (content, stems root
// first, own branch), from the same metadata and rule the kernels use.
template <typename Emit>
void visible_keys(const PassPlan &P, int row, Emit emit) {
  const SpbRow &r = P.rows[row];
  for (int j = 0; j < r.cvis; ++j) emit(r.seg + j);
  // stems on the row's path, root first: all their tokens, the row's own stem
  // causally
  std::vector<std::pair<int, const PassPlan::HostStem *>> path;
  for (auto &s : P.stems)
    if (r.br >= 0 && s.pre <= r.spre && r.spre < s.post) path.push_back({s.pre, &s});
  std::sort(path.begin(), path.end(), [](auto &a, auto &b) { return a.first < b.first; });
  for (auto &ps : path) {
    const bool own = r.stem && ps.second->start == r.br;
    const int n = own ? r.e + 1 : ps.second->L;
    for (int j = 0; j < n; ++j) emit(ps.second->start + j);
  }
  if (r.br >= 0 && !r.stem) {
    int E = r.L;
    for (auto &b : P.branches)
      if (b.start == r.br) E = b.E;
    for (int ep = 0; ep < E; ++ep)
      if (branch_visible(r, ep)) emit(r.br + ep);
  }
}
}  // namespace

extern "C" {

spb_status spb_plan_visible(const spb_plan *plan, int32_t pass, int32_t row, int32_t *keys, int32_t cap,
                            int32_t *n_keys) {
  spb_status st = check_pass(plan, pass);
  if (st != SPB_OK) return st;
  const PassPlan &P = plan->passes[pass];
  if (row < 0 || row >= (int32_t)P.rows.size()) return fail(SPB_ERR_ARG, "row %d outside the pass", row);
  if (!n_keys || (cap > 0 && !keys)) return fail(SPB_ERR_ARG, "NULL argument");
  int n = 0;
  visible_keys(P, row, [&](int y) {
    if (n < cap) keys[n] = y;
    ++n;
  });
  *n_keys = n;
  if (n > cap) return fail(SPB_ERR_SIZE, "%d keys exceed cap %d", n, cap);
  return ok();
}

spb_status spb_plan_slot(const spb_plan *plan, int32_t logical_branch, spb_slot_info *out) {
  if (!plan || !out) return fail(SPB_ERR_ARG, "NULL argument");
  if (logical_branch < 0 || logical_branch >= (int32_t)plan->lb_pass.size())
    return fail(SPB_ERR_ARG, "logical branch %d outside [0, %zu)", logical_branch, plan->lb_pass.size());
  spb_slot_info s{};
  s.pass = plan->lb_pass[logical_branch];
  const PassPlan &P = plan->passes[s.pass];
  const SpbBranch &b = P.branches[plan->lb_slot[logical_branch]];
  s.row = b.start + b.L - 1;
  s.position = P.pos[s.row];
  bool over = false;
  int prev = -2;
  visible_keys(P, s.row, [&](int y) {
    if (y == prev + 1 && s.n_ranges > 0) {
      s.ranges[s.n_ranges - 1][1]++;
    } else if (s.n_ranges < SPB_MAX_SLOT_RANGES) {
      s.ranges[s.n_ranges][0] = y;
      s.ranges[s.n_ranges][1] = 1;
      s.n_ranges++;
    } else {
      over = true;
    }
    prev = y;
  });
  if (over) return fail(SPB_ERR_LIMIT, "slot prefix needs more than %d key ranges", SPB_MAX_SLOT_RANGES);
  *out = s;
  return ok();
}

spb_status spb_plan_upload(const spb_plan *plan, int32_t pass, void *d_meta, size_t bytes, void *stream) {
  spb_status st = check_pass(plan, pass);
  if (st != SPB_OK) return st;
  const PassPlan &P = plan->passes[pass];
  if (!d_meta) return fail(SPB_ERR_ARG, "d_meta is NULL");
  if ((uintptr_t)d_meta % 256) return fail(SPB_ERR_ARG, "d_meta must be 256-byte aligned");
  if (bytes < P.blob.size()) return fail(SPB_ERR_SIZE, "metadata needs %zu bytes, buffer has %zu", P.blob.size(), bytes);
  hipError_t e = hipMemcpyAsync(d_meta, P.blob.data(), P.blob.size(), hipMemcpyHostToDevice, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SPB_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
  return ok();
}

spb_status spb_plan_meta_copy(const spb_plan *plan, int32_t pass, void *host_dst, size_t bytes) {
  spb_status st = check_pass(plan, pass);
  if (st != SPB_OK) return st;
  const PassPlan &P = plan->passes[pass];
  if (!host_dst) return fail(SPB_ERR_ARG, "host_dst is NULL");
  if (bytes < P.blob.size()) return fail(SPB_ERR_SIZE, "metadata needs %zu bytes, buffer has %zu", P.blob.size(), bytes);
  std::memcpy(host_dst, P.blob.data(), P.blob.size());
  return ok();
}

spb_status spb_branch_attention(const spb_plan *plan, int32_t pass, const void *d_meta, const spb_attn_args *a,
                                void *stream) {
  spb_status st = check_pass(plan, pass);
  if (st != SPB_OK) return st;
  if (!a || !d_meta) return fail(SPB_ERR_ARG, "NULL argument");
  const PassPlan &P = plan->passes[pass];
  const SpbMetaHeader &h = header(P);
  if (a->head_dim != 64 && a->head_dim != 128) return fail(SPB_ERR_DTYPE, "head_dim %d not in {64, 128}", a->head_dim);
  if (a->hq < 1 || a->hkv < 1 || a->hq % a->hkv) return fail(SPB_ERR_DTYPE, "hq %d not a multiple of hkv %d", a->hq, a->hkv);
  int g = a->hq / a->hkv;
  if (g != 1 && g != 2 && g != 4) return fail(SPB_ERR_DTYPE, "hq / hkv = %d not in {1, 2, 4}", g);
  if (a->in_dtype != SPB_F32 && a->in_dtype != SPB_BF16 && a->in_dtype != SPB_FP8_E4M3)
    return fail(SPB_ERR_DTYPE, "in_dtype %d unsupported", a->in_dtype);
  if (a->out_dtype != SPB_F32 && a->out_dtype != SPB_BF16) return fail(SPB_ERR_DTYPE, "out_dtype %d unsupported", a->out_dtype);
  if (a->in_dtype == SPB_FP8_E4M3 && a->head_dim != 128) return fail(SPB_ERR_DTYPE, "fp8 inputs need head_dim 128");
  if (a->rows < h.n_tokens) return fail(SPB_ERR_SIZE, "buffers hold %lld rows, the pass has %d", (long long)a->rows, h.n_tokens);
  if (h.n_tokens > 0 && (!a->q || !a->k || !a->v || !a->o)) return fail(SPB_ERR_ARG, "NULL tensor");
  float sq = a->in_dtype == SPB_FP8_E4M3 ? a->s_q : 1.f;
  float sk = a->in_dtype == SPB_FP8_E4M3 ? a->s_k : 1.f;
  float sv = a->in_dtype == SPB_FP8_E4M3 ? a->s_v : 1.f;
  if (!(sq > 0.f) || !(sk > 0.f) || !(sv > 0.f) || !std::isfinite(sq * sk * sv))
    return fail(SPB_ERR_ARG, "fp8 scales must be finite and > 0");
  if ((uintptr_t)d_meta % 256) return fail(SPB_ERR_ARG, "d_meta must be 256-byte aligned");
  if (a->in_dtype == SPB_BF16 && (uint64_t)h.n_tokens * (uint64_t)a->hkv * (uint64_t)a->head_dim * 2u > 0xFFFFFFFFull)
    return fail(SPB_ERR_LIMIT, "a bf16 pass's K/V (%d tokens x %d heads x %d) must stay under 4 GiB", h.n_tokens, a->hkv,
                a->head_dim);
  const bool wide = a->in_dtype == SPB_FP8_E4M3 && a->workspace;
  if (wide) {
    const uint64_t need = (uint64_t)h.n_tokens * (uint64_t)a->hkv * (uint64_t)a->head_dim * 2u;
    if (a->workspace_bytes < need)
      return fail(SPB_ERR_SIZE, "attention workspace needs %llu bytes, got %zu", (unsigned long long)need,
                  a->workspace_bytes);
    if ((uintptr_t)a->workspace % 256) return fail(SPB_ERR_ARG, "workspace must be 256-byte aligned");
    if ((uintptr_t)a->v % 16) return fail(SPB_ERR_ARG, "v must be 16-byte aligned");
    if (need > 0xFFFFFFFFull)
      return fail(SPB_ERR_LIMIT, "a pass's widened V (%d tokens x %d heads x %d) must stay under 4 GiB", h.n_tokens,
                  a->hkv, a->head_dim);
  }
  if (h.n_tiles == 0) return ok();
  st = check_attention_limits(P, pass);  // also checked when the plan was packed
  if (st != SPB_OK) return st;
  AttnLaunch L{};
  L.q = a->q; L.k = a->k; L.v = a->v; L.o = a->o;
  L.in_dtype = a->in_dtype; L.out_dtype = a->out_dtype;
  L.hq = a->hq; L.hkv = a->hkv; L.head_dim = a->head_dim;
  L.scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.0f / std::sqrt((float)a->head_dim);
  L.s_q = sq; L.s_k = sk; L.s_v = sv;
  L.n_tokens = h.n_tokens;
  L.n_tiles = h.n_tiles;
  const char *base = (const char *)d_meta;
  L.rows = base + h.off_rows;
  L.tiles = base + h.off_tiles;
  L.branches = base + h.off_branches;
  for (int g = 0; g < 3; ++g) {
    L.items[g] = base + h.off_items[g];
    L.n_items[g] = h.n_items[g];
  }
  L.bchunks = base + h.off_bchunks;
  L.v_wide = wide ? a->workspace : nullptr;
  int e = launch_attention(L, stream);
  if (e) return fail(SPB_ERR_HIP, "branch attention launch: %s", hip_error_string(e));
  return ok();
}

spb_status spb_mfma_calibration(float *d_out, int32_t work_groups, int32_t iters, int32_t random_operands,
                                void *stream) {
  if (!d_out) return fail(SPB_ERR_ARG, "d_out is NULL");
  if (work_groups < 1 || iters < 1) return fail(SPB_ERR_ARG, "work_groups %d and iters %d must be >= 1", work_groups, iters);
  if (work_groups > (1 << 20)) return fail(SPB_ERR_LIMIT, "work_groups %d above 2^20", work_groups);
  int e = launch_mfma_calibration(d_out, work_groups, iters, random_operands ? 1 : 0, stream);
  if (e) return fail(SPB_ERR_HIP, "calibration launch: %s", hip_error_string(e));
  return ok();
}

spb_status spb_attention_workspace_bytes(const spb_plan *plan, int32_t pass, int32_t in_dtype, int32_t hkv,
                                         int32_t head_dim, size_t *out) {
  spb_status st = check_pass(plan, pass);
  if (st != SPB_OK) return st;
  if (!out) return fail(SPB_ERR_ARG, "NULL argument");
  if (hkv < 1 || head_dim < 1) return fail(SPB_ERR_ARG, "hkv %d and head_dim %d must be >= 1", hkv, head_dim);
  const SpbMetaHeader &h = header(plan->passes[pass]);
  *out = in_dtype == SPB_FP8_E4M3 ? (size_t)h.n_tokens * (size_t)hkv * (size_t)head_dim * 2u : 0;
  return ok();
}

spb_status spb_score_workspace_bytes(const spb_plan *plan, int32_t pass, int32_t vocab, int32_t hidden_dim,
                                     int32_t lm_head_kind, size_t *out) {
  spb_status st = check_pass(plan, pass);
  if (st != SPB_OK) return st;
  if (!out || vocab < 1 || hidden_dim < 1) return fail(SPB_ERR_ARG, "bad argument");
  if (lm_head_kind < SPB_HEAD_F32OUT || lm_head_kind > SPB_HEAD_FP32)
    return fail(SPB_ERR_ARG, "lm_head_kind %d outside 0..2", lm_head_kind);
  const SpbMetaHeader &h = header(plan->passes[pass]);
  *out = score_workspace_layout(h.n_scored, h.n_targets, vocab, hidden_dim, lm_head_kind, nullptr);
  return ok();
}

namespace {

// spb_score_options' checks and launches; own_scratch: the workspace is the
// library's allocation-free scratch of the current device instead of the
// caller's a->workspace.
spb_status score_options_at(const spb_plan *plan, int32_t pass, const void *d_meta, const spb_score_args *a,
                            void *stream, bool own_scratch) {
  spb_status st = check_pass(plan, pass);
  if (st != SPB_OK) return st;
  if (!a || !d_meta) return fail(SPB_ERR_ARG, "NULL argument");
  const PassPlan &P = plan->passes[pass];
  const SpbMetaHeader &h = header(P);
  if (a->h_dtype != SPB_BF16 && a->h_dtype != SPB_F32) return fail(SPB_ERR_DTYPE, "h_dtype %d unsupported", a->h_dtype);
  if (a->hidden_dim < 64 || a->hidden_dim % 64) return fail(SPB_ERR_DTYPE, "hidden_dim %d not a positive multiple of 64", a->hidden_dim);
  if (a->vocab < 1) return fail(SPB_ERR_ARG, "vocab %d < 1", a->vocab);
  if ((int64_t)a->vocab * a->hidden_dim * 2 > (int64_t)UINT32_MAX)
    return fail(SPB_ERR_DTYPE, "the lm head (%lld bytes) exceeds 4 GiB", (long long)a->vocab * a->hidden_dim * 2);
  for (int t : P.tgt_tok)
    if (t >= a->vocab) return fail(SPB_ERR_ARG, "option token %d >= vocab %d", t, a->vocab);
  if (a->rows < h.n_tokens) return fail(SPB_ERR_SIZE, "hidden holds %lld rows, the pass has %d", (long long)a->rows, h.n_tokens);
  if (a->lm_head_kind < SPB_HEAD_F32OUT || a->lm_head_kind > SPB_HEAD_FP32)
    return fail(SPB_ERR_ARG, "lm_head_kind %d outside 0..2", a->lm_head_kind);
  const size_t need = score_workspace_layout(h.n_scored, h.n_targets, a->vocab, a->hidden_dim, a->lm_head_kind, nullptr);
  if (own_scratch) {
    if (need > kScoreScratchBytes)
      return fail(SPB_ERR_SIZE, "the pass's head workspace needs %zu bytes, more than the %zu bytes of the "
                  "allocation-free scratch (%d scored rows)", need, kScoreScratchBytes, h.n_scored);
  } else if (a->workspace_bytes < need) {
    return fail(SPB_ERR_SIZE, "workspace needs %zu bytes, got %zu", need, a->workspace_bytes);
  }
  if (h.n_scored > 0 && (!a->hidden || !a->lm_head || (!own_scratch && !a->workspace) || !a->lp || !a->p ||
                         !a->residual))
    return fail(SPB_ERR_ARG, "NULL tensor");
  if ((uintptr_t)d_meta % 256 || (!own_scratch && (uintptr_t)a->workspace % 256))
    return fail(SPB_ERR_ARG, "d_meta and workspace must be 256-byte aligned");
  if (h.n_scored == 0) return ok();
  char *ws = (char *)a->workspace;
  if (own_scratch) {
    void *scr = nullptr;
    int e = score_scratch(&scr);
    if (e) return fail(SPB_ERR_HIP, "allocation-free scratch: %s", hip_error_string(e));
    ws = (char *)scr;
  }
  ScoreLaunch L{};
  L.hidden = a->hidden; L.h_dtype = a->h_dtype; L.hidden_dim = a->hidden_dim;
  L.lm_head = a->lm_head; L.vocab = a->vocab;
  L.n_scored = h.n_scored; L.n_targets = h.n_targets; L.n_branches = h.n_branches; L.n_options = h.n_options;
  const char *base = (const char *)d_meta;
  L.scored = base + h.off_scored;
  L.tgt_off = base + h.off_tgt_off;
  L.tgt_tok = base + h.off_tgt_tok;
  L.branches = base + h.off_branches;
  L.opt_step_off = base + h.off_opt_step_off;
  L.step_slot = base + h.off_step_slot;
  L.step_row = base + h.off_step_row;
  size_t off[4];
  score_workspace_layout(h.n_scored, h.n_targets, a->vocab, a->hidden_dim, a->lm_head_kind, off);
  L.part = (float *)(ws + off[0]);
  L.tz = (float *)(ws + off[1]);
  L.lse = (float *)(ws + off[2]);
  L.hg = ws + off[3];
  L.lp = a->lp; L.p = a->p; L.residual = a->residual;
  L.ev_begin = a->gemm_event_begin; L.ev_end = a->gemm_event_end;
  L.kind = a->lm_head_kind;
  int e = launch_score(L, stream);
  if (e) return fail(SPB_ERR_HIP, "score launch: %s", hip_error_string(e));
  return ok();
}

}  // namespace

spb_status spb_score_options(const spb_plan *plan, int32_t pass, const void *d_meta, const spb_score_args *a,
                             void *stream) {
  return score_options_at(plan, pass, d_meta, a, stream, false);
}

spb_status spb_score_options_noalloc(const spb_plan *plan, int32_t pass, const void *d_meta,
                                     const spb_score_args *a, void *stream) {
  return score_options_at(plan, pass, d_meta, a, stream, true);
}

namespace {

// Distinct, valid pass indices; sums of scored rows and targets.
spb_status check_batch(const spb_plan *plan, int32_t n, const int32_t *passes, int64_t *m_tot, int64_t *t_tot) {
  if (!plan) return fail(SPB_ERR_ARG, "plan is NULL");
  if (n < 1 || n > kMaxBatchPasses) return fail(SPB_ERR_LIMIT, "a batch holds 1..%d passes, got %d", kMaxBatchPasses, n);
  if (!passes) return fail(SPB_ERR_ARG, "passes is NULL");
  std::vector<char> seen(plan->passes.size(), 0);
  *m_tot = *t_tot = 0;
  for (int i = 0; i < n; ++i) {
    spb_status st = check_pass(plan, passes[i]);
    if (st != SPB_OK) return st;
    if (seen[passes[i]]++) return fail(SPB_ERR_ARG, "pass %d appears twice in the batch", passes[i]);
    const SpbMetaHeader &h = header(plan->passes[passes[i]]);
    *m_tot += h.n_scored;
    *t_tot += h.n_targets;
  }
  if (*m_tot > INT32_MAX / 2 || *t_tot > INT32_MAX / 2) return fail(SPB_ERR_LIMIT, "batch too large");
  return ok();
}

}  // namespace

spb_status spb_score_batch_workspace_bytes(const spb_plan *plan, int32_t n, const int32_t *passes, int32_t vocab,
                                           int32_t hidden_dim, int32_t lm_head_kind, size_t *out) {
  int64_t m_tot = 0, t_tot = 0;
  spb_status st = check_batch(plan, n, passes, &m_tot, &t_tot);
  if (st != SPB_OK) return st;
  if (!out || vocab < 1 || hidden_dim < 1) return fail(SPB_ERR_ARG, "bad argument");
  if (lm_head_kind < SPB_HEAD_F32OUT || lm_head_kind > SPB_HEAD_FP32)
    return fail(SPB_ERR_ARG, "lm_head_kind %d outside 0..2", lm_head_kind);
  *out = score_batch_workspace_layout((int)m_tot, (int)t_tot, vocab, hidden_dim, lm_head_kind, nullptr);
  return ok();
}

spb_status spb_score_options_batch(const spb_plan *plan, int32_t n, const int32_t *passes, const void *const *d_metas,
                                   const spb_score_args *args, void *workspace, size_t workspace_bytes,
                                   void *stream) {
  int64_t m_tot = 0, t_tot = 0;
  spb_status st = check_batch(plan, n, passes, &m_tot, &t_tot);
  if (st != SPB_OK) return st;
  if (!d_metas || !args) return fail(SPB_ERR_ARG, "NULL argument");
  const spb_score_args &a0 = args[0];
  if (a0.h_dtype != SPB_BF16 && a0.h_dtype != SPB_F32) return fail(SPB_ERR_DTYPE, "h_dtype %d unsupported", a0.h_dtype);
  if (a0.hidden_dim < 64 || a0.hidden_dim % 64)
    return fail(SPB_ERR_DTYPE, "hidden_dim %d not a positive multiple of 64", a0.hidden_dim);
  if (a0.vocab < 1) return fail(SPB_ERR_ARG, "vocab %d < 1", a0.vocab);
  if ((int64_t)a0.vocab * a0.hidden_dim * 2 > (int64_t)UINT32_MAX)
    return fail(SPB_ERR_DTYPE, "the lm head (%lld bytes) exceeds 4 GiB", (long long)a0.vocab * a0.hidden_dim * 2);
  if (a0.lm_head_kind < SPB_HEAD_F32OUT || a0.lm_head_kind > SPB_HEAD_FP32)
    return fail(SPB_ERR_ARG, "lm_head_kind %d outside 0..2", a0.lm_head_kind);
  const size_t need =
      score_batch_workspace_layout((int)m_tot, (int)t_tot, a0.vocab, a0.hidden_dim, a0.lm_head_kind, nullptr);
  if (workspace_bytes < need) return fail(SPB_ERR_SIZE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if (m_tot > 0 && (!workspace || !a0.lm_head)) return fail(SPB_ERR_ARG, "NULL workspace or lm head");
  if ((uintptr_t)workspace % 256) return fail(SPB_ERR_ARG, "workspace must be 256-byte aligned");
  std::unique_ptr<ScoreBatchLaunch> B(new ScoreBatchLaunch());
  ScoreBatchLaunch &L = *B;
  L.n = 0;
  int m_off = 0, t_off = 0;
  for (int i = 0; i < n; ++i) {
    const spb_score_args &a = args[i];
    const PassPlan &P = plan->passes[passes[i]];
    const SpbMetaHeader &h = header(P);
    if (a.h_dtype != a0.h_dtype || a.hidden_dim != a0.hidden_dim || a.vocab != a0.vocab || a.lm_head != a0.lm_head ||
        a.lm_head_kind != a0.lm_head_kind)
      return fail(SPB_ERR_ARG, "batch entry %d disagrees with entry 0 on the hidden dtype/size or the lm head", i);
    for (int t : P.tgt_tok)
      if (t >= a.vocab) return fail(SPB_ERR_ARG, "option token %d >= vocab %d", t, a.vocab);
    if (a.rows < h.n_tokens)
      return fail(SPB_ERR_SIZE, "hidden of pass %d holds %lld rows, the pass has %d", passes[i], (long long)a.rows, h.n_tokens);
    if (!d_metas[i] || (uintptr_t)d_metas[i] % 256) return fail(SPB_ERR_ARG, "d_metas[%d] NULL or not 256-byte aligned", i);
    if (h.n_scored == 0) continue;  // no branches either: nothing to score
    if (!a.hidden || !a.lp || !a.p || !a.residual) return fail(SPB_ERR_ARG, "NULL tensor in batch entry %d", i);
    ScoreLaunch &S = L.pass[L.n];
    S.hidden = a.hidden;
    S.n_scored = h.n_scored; S.n_targets = h.n_targets; S.n_branches = h.n_branches; S.n_options = h.n_options;
    const char *base = (const char *)d_metas[i];
    S.scored = base + h.off_scored;
    S.tgt_off = base + h.off_tgt_off;
    S.tgt_tok = base + h.off_tgt_tok;
    S.branches = base + h.off_branches;
    S.opt_step_off = base + h.off_opt_step_off;
    S.step_slot = base + h.off_step_slot;
    S.step_row = base + h.off_step_row;
    S.lp = a.lp; S.p = a.p; S.residual = a.residual;
    L.m_off[L.n] = m_off;
    L.t_off[L.n] = t_off;
    m_off += h.n_scored;
    t_off += h.n_targets;
    ++L.n;
  }
  if (L.n == 0) return ok();
  L.m_tot = m_off;
  L.t_tot = t_off;
  L.h_dtype = a0.h_dtype;
  L.hidden_dim = a0.hidden_dim;
  L.lm_head = a0.lm_head;
  L.vocab = a0.vocab;
  L.kind = a0.lm_head_kind;
  size_t off[6];
  score_batch_workspace_layout(L.m_tot, L.t_tot, a0.vocab, a0.hidden_dim, a0.lm_head_kind, off);
  char *ws = (char *)workspace;
  L.part = (float *)(ws + off[0]);
  L.tz = (float *)(ws + off[1]);
  L.lse = (float *)(ws + off[2]);
  L.hg = ws + off[3];
  L.ctgt_off = (int32_t *)(ws + off[4]);
  L.ctgt_tok = (int32_t *)(ws + off[5]);
  L.ev_begin = a0.gemm_event_begin;
  L.ev_end = a0.gemm_event_end;
  int e = launch_score_batch(L, stream);
  if (e) return fail(SPB_ERR_HIP, "batched score launch: %s", hip_error_string(e));
  return ok();
}

spb_status spb_score_finalize(const spb_plan *plan, const float *const *lp_pp, const float *const *p_pp,
                              const float *const *res_pp, float *lp, float *p, float *residual, float *floor_p,
                              float *lift) {
  if (!plan) return fail(SPB_ERR_ARG, "plan is NULL");
  if ((lp && !lp_pp) || ((p || floor_p || lift) && !p_pp) || (residual && !res_pp))
    return fail(SPB_ERR_ARG, "per-pass input arrays missing");
  for (size_t k = 0; k < plan->passes.size(); ++k)
    if ((lp && !lp_pp[k]) || ((p || floor_p || lift) && !p_pp[k]) || (residual && !res_pp[k]))
      return fail(SPB_ERR_ARG, "per-pass array %zu is NULL", k);
  const float nan = std::nanf("");
  for (int b = 0; b < plan->n_content_branches; ++b) {
    int q = plan->lb_question[b];
    int ps = plan->lb_pass[b], sl = plan->lb_slot[b];
    const SpbBranch &B = plan->passes[ps].branches[sl];
    int fb = plan->floor_lb_of_q[q];
    const SpbBranch *F = nullptr;
    int fps = -1;
    if (fb >= 0) {
      fps = plan->lb_pass[fb];
      F = &plan->passes[fps].branches[plan->lb_slot[fb]];
    }
    if (residual) residual[b] = res_pp[ps][sl];
    for (int o = 0; o < B.n_opt; ++o) {
      int dst = plan->content_opt_off[b] + o;
      if (lp) lp[dst] = lp_pp[ps][B.opt0 + o];
      float pv = (p || lift) ? p_pp[ps][B.opt0 + o] : 0.f;
      if (p) p[dst] = pv;
      float fv = F ? p_pp[fps][F->opt0 + o] : nan;
      if (floor_p) floor_p[dst] = fv;
      if (lift) lift[dst] = F ? pv - fv : nan;
    }
  }
  return ok();
}

spb_status spb_rope_table(float *host_out, int32_t n_pos, int32_t head_dim, double base) {
  if (!host_out) return fail(SPB_ERR_ARG, "host_out is NULL");
  if (n_pos < 1 || head_dim < 2 || head_dim % 2) return fail(SPB_ERR_ARG, "n_pos %d, head_dim %d", n_pos, head_dim);
  if (!(base > 1.0) || !std::isfinite(base)) return fail(SPB_ERR_ARG, "rope base must be finite and > 1");
  const int half = head_dim / 2;
  for (int i = 0; i < half; ++i) {
    const double theta = std::pow(base, -2.0 * i / head_dim);
    for (int p = 0; p < n_pos; ++p) {
      const double a = p * theta;
      host_out[((size_t)p * half + i) * 2] = (float)std::cos(a);
      host_out[((size_t)p * half + i) * 2 + 1] = (float)std::sin(a);
    }
  }
  return ok();
}

static bool misaligned16(const void *p) { return (uintptr_t)p % 16 != 0; }

spb_status spb_rmsnorm(const spb_rmsnorm_args *a, void *stream) {
  if (!a) return fail(SPB_ERR_ARG, "args is NULL");
  if (a->rows < 0 || a->dim < 4 || a->dim % 4) return fail(SPB_ERR_ARG, "rows %lld, dim %d (dim % 4 == 0)",
                                                             (long long)a->rows, a->dim);
  if (!(a->eps >= 0.f) || !std::isfinite(a->eps)) return fail(SPB_ERR_ARG, "eps must be finite and >= 0");
  if (a->rows == 0) return ok();
  if (!a->x || !a->gain || !a->out) return fail(SPB_ERR_ARG, "NULL tensor");
  if (misaligned16(a->x) || misaligned16(a->gain) || misaligned16(a->out))
    return fail(SPB_ERR_ARG, "tensors must be 16-byte aligned");
  NormLaunch L{a->x, (const uint16_t *)a->gain, (uint16_t *)a->out, (long long)a->rows, a->dim, a->eps};
  int e = launch_rmsnorm(L, stream);
  if (e) return fail(SPB_ERR_HIP, "rmsnorm launch: %s", hip_error_string(e));
  return ok();
}

spb_status spb_linear(const spb_linear_args *a, void *stream) {
  if (!a) return fail(SPB_ERR_ARG, "args is NULL");
  if (a->mode < SPB_LINEAR_BF16 || a->mode > SPB_LINEAR_F32) return fail(SPB_ERR_ARG, "mode %d", a->mode);
  if (a->m < 0 || a->m > 0x7FFFFFFF) return fail(SPB_ERR_ARG, "m %lld", (long long)a->m);
  if (a->k < 64 || a->k % 64) return fail(SPB_ERR_ARG, "k %d must be a positive multiple of 64", a->k);
  if (a->fp8 && a->k % 128) return fail(SPB_ERR_ARG, "fp8 k %d must be a multiple of 128", a->k);
  if (a->fp8 && (!(a->scale_x > 0.f) || !(a->scale_w > 0.f) || !std::isfinite(a->scale_x * a->scale_w)))
    return fail(SPB_ERR_ARG, "fp8 scales must be finite and > 0");
  if (a->n < 8 || a->n % 8) return fail(SPB_ERR_ARG, "n %d must be a positive multiple of 8", a->n);
  const uint64_t es = a->fp8 ? 1u : 2u;  // bytes per operand element
  if ((uint64_t)a->m * (uint64_t)a->k * es >= (1ull << 32) || (uint64_t)a->n * (uint64_t)a->k * es >= (1ull << 32))
    return fail(SPB_ERR_LIMIT, "x (%lld x %d) and W (%d x %d) must each stay under 4 GiB", (long long)a->m, a->k,
                a->n, a->k);
  if (a->m == 0) return ok();
  if (!a->x || !a->w || misaligned16(a->x) || misaligned16(a->w))
    return fail(SPB_ERR_ARG, "x and W must be non-NULL and 16-byte aligned");
  LinearLaunch L{};
  L.x = (const uint16_t *)a->x;
  L.w = (const uint16_t *)a->w;
  L.m = (int)a->m;
  L.n = a->n;
  L.k = a->k;
  L.mode = a->mode;
  switch (a->mode) {
    case SPB_LINEAR_BF16:
    case SPB_LINEAR_SILU_GATE:
      if (a->mode == SPB_LINEAR_SILU_GATE && a->n % 64)
        return fail(SPB_ERR_ARG, "silu-gate n %d must be a multiple of 64", a->n);
      if (!a->y || misaligned16(a->y)) return fail(SPB_ERR_ARG, "y must be non-NULL and 16-byte aligned");
      L.y = (uint16_t *)a->y;
      break;
    case SPB_LINEAR_RESIDUAL:
      if (!a->resid || misaligned16(a->resid)) return fail(SPB_ERR_ARG, "resid must be non-NULL and 16-byte aligned");
      L.resid = a->resid;
      break;
    case SPB_LINEAR_F32:
      if (!a->yf || misaligned16(a->yf)) return fail(SPB_ERR_ARG, "yf must be non-NULL and 16-byte aligned");
      L.yf = a->yf;
      break;
    case SPB_LINEAR_QKV_ROPE:
      if (a->head_dim != 64 && a->head_dim != 128) return fail(SPB_ERR_DTYPE, "head_dim %d not in {64, 128}", a->head_dim);
      if (a->hq < 1 || a->hkv < 1 || a->hq % a->hkv) return fail(SPB_ERR_ARG, "hq %d, hkv %d", a->hq, a->hkv);
      if ((int64_t)(a->hq + 2 * a->hkv) * a->head_dim != a->n)
        return fail(SPB_ERR_ARG, "n %d != (hq + 2 hkv) head_dim = %d", a->n, (a->hq + 2 * a->hkv) * a->head_dim);
      if (!a->q || !a->k_out || !a->v || !a->pos || !a->rope_table || a->n_pos < 1)
        return fail(SPB_ERR_ARG, "q, k, v, pos and rope_table must be non-NULL, n_pos >= 1");
      if (misaligned16(a->q) || misaligned16(a->k_out) || misaligned16(a->v) || misaligned16(a->rope_table))
        return fail(SPB_ERR_ARG, "q, k, v and rope_table must be 16-byte aligned");
      L.q = (uint16_t *)a->q;
      L.kk = (uint16_t *)a->k_out;
      L.v = (uint16_t *)a->v;
      L.hq = a->hq;
      L.hkv = a->hkv;
      L.head_dim = a->head_dim;
      L.pos = a->pos;
      L.rope = a->rope_table;
      L.n_pos = a->n_pos;
      break;
  }
  L.ev_begin = a->gemm_event_begin;
  L.ev_end = a->gemm_event_end;
  L.fp8 = a->fp8 ? 1 : 0;
  L.scale = a->fp8 ? a->scale_x * a->scale_w : 1.f;
  int e = launch_linear(L, stream);
  if (e) return fail(SPB_ERR_HIP, "linear launch: %s", hip_error_string(e));
  return ok();
}

spb_status spb_quantize_e4m3(const spb_quantize_args *a, void *stream) {
  if (!a) return fail(SPB_ERR_ARG, "args is NULL");
  if (a->n < 0) return fail(SPB_ERR_ARG, "n %lld", (long long)a->n);
  if (a->src_dtype != SPB_F32 && a->src_dtype != SPB_BF16) return fail(SPB_ERR_DTYPE, "src_dtype %d", a->src_dtype);
  if (!(a->scale > 0.f) || !std::isfinite(a->scale)) return fail(SPB_ERR_ARG, "scale must be finite and > 0");
  if (a->n == 0) return ok();
  if (!a->src || !a->dst || misaligned16(a->src) || (uintptr_t)a->dst % 8)
    return fail(SPB_ERR_ARG, "src (16-byte aligned) and dst (8-byte aligned) required");
  QuantLaunch L{};
  if (a->src_dtype == SPB_F32)
    L.src_f32 = (const float *)a->src;
  else
    L.src_bf16 = (const uint16_t *)a->src;
  L.dst = (uint8_t *)a->dst;
  L.n = a->n;
  L.inv_scale = 1.0f / a->scale;
  int e = launch_quantize_e4m3(L, stream);
  if (e) return fail(SPB_ERR_HIP, "quantize launch: %s", hip_error_string(e));
  return ok();
}

spb_status spb_gather_rows(const spb_gather_args *a, void *stream) {
  if (!a) return fail(SPB_ERR_ARG, "args is NULL");
  if (a->rows < 0 || a->dim < 1 || a->n_src < 1) return fail(SPB_ERR_ARG, "rows, dim or n_src");
  if (a->rows == 0) return ok();
  if (!a->src || !a->idx || (!a->dst_f32) == (!a->dst_bf16)) return fail(SPB_ERR_ARG, "src, idx and one dst");
  if (a->pos && (!a->pos_base || a->per < 1)) return fail(SPB_ERR_ARG, "pos needs pos_base and per >= 1");
  GatherLaunch L{};
  L.src = (const uint16_t *)a->src;
  L.idx = a->idx;
  L.rows = a->rows;
  L.n_src = a->n_src;
  L.dim = a->dim;
  L.dst_f32 = a->dst_f32;
  L.dst_bf16 = (uint16_t *)a->dst_bf16;
  L.pos = a->pos;
  L.pos_base = a->pos_base;
  L.per = a->per;
  L.pos_add = a->pos_add;
  int e = launch_gather_rows(L, stream);
  if (e) return fail(SPB_ERR_HIP, "gather launch: %s", hip_error_string(e));
  return ok();
}

spb_status spb_topk_workspace_bytes(int64_t rows, int32_t vocab, size_t *out) {
  if (!out || rows < 0 || vocab < 1) return fail(SPB_ERR_ARG, "rows %lld, vocab %d", (long long)rows, vocab);
  *out = topk_workspace_bytes(rows, vocab);
  return ok();
}

spb_status spb_topk_lse(const spb_topk_args *a, void *stream) {
  if (!a) return fail(SPB_ERR_ARG, "args is NULL");
  if (a->rows < 0 || a->rows > 0x7FFFFFFF || a->vocab < 1 || a->k < 1 || a->k > kMaxTopK)
    return fail(SPB_ERR_ARG, "rows %lld, vocab %d, k %d (1..%d)", (long long)a->rows, a->vocab, a->k, kMaxTopK);
  if (a->rows == 0) return ok();
  if (!a->logits || !a->ids || !a->lp || !a->lse) return fail(SPB_ERR_ARG, "NULL tensor");
  if (a->mask_of_row && (!a->masks || a->n_masks < 1))
    return fail(SPB_ERR_ARG, "mask_of_row needs masks");
  const size_t need = topk_workspace_bytes(a->rows, a->vocab);
  if (!a->workspace || a->workspace_bytes < need || misaligned16(a->workspace))
    return fail(SPB_ERR_SIZE, "top-k needs a 16-byte aligned workspace of %zu bytes", need);
  TopkLaunch L{a->logits, (long long)a->rows, a->vocab, a->k, a->masks, a->mask_of_row, a->stop_of_row,
               a->ids, a->lp, a->lse, a->workspace};
  int e = launch_topk_lse(L, stream);
  if (e) return fail(SPB_ERR_HIP, "top-k launch: %s", hip_error_string(e));
  return ok();
}

spb_status spb_decode_attention(const spb_decode_attn_args *a, void *stream) {
  if (!a) return fail(SPB_ERR_ARG, "args is NULL");
  if (a->head_dim != 64 && a->head_dim != 128) return fail(SPB_ERR_DTYPE, "head_dim %d not in {64, 128}", a->head_dim);
  if (a->hq < 1 || a->hkv < 1 || a->hq % a->hkv) return fail(SPB_ERR_DTYPE, "hq %d, hkv %d", a->hq, a->hkv);
  const int g = a->hq / a->hkv;
  if (g != 1 && g != 2 && g != 4) return fail(SPB_ERR_DTYPE, "hq / hkv = %d not in {1, 2, 4}", g);
  if (a->rows < 0 || a->beams < 1 || a->beams > kMaxBeams || a->rows % a->beams)
    return fail(SPB_ERR_ARG, "rows %d must be a multiple of beams %d (1..%d)", a->rows, a->beams, kMaxBeams);
  if (a->t_cap < 1 || a->n_path < 0 || a->n_path >= a->t_cap || a->n_pass_rows < 1)
    return fail(SPB_ERR_ARG, "t_cap %d, n_path %d, n_pass_rows %d", a->t_cap, a->n_path, a->n_pass_rows);
  if (a->rows == 0) return ok();
  if ((int64_t)a->t_cap * a->rows > 0x7FFFFFFF) return fail(SPB_ERR_LIMIT, "decode cache too large");
  if (!a->q || !a->k_pass || !a->v_pass || !a->k_dec || !a->v_dec || !a->o || !a->ranges || !a->n_ranges ||
      !a->path)
    return fail(SPB_ERR_ARG, "NULL tensor");
  if (misaligned16(a->k_pass) || misaligned16(a->k_dec)) return fail(SPB_ERR_ARG, "K caches must be 16-byte aligned");
  DecodeAttnLaunch L{};
  L.q = (const uint16_t *)a->q;
  L.kp = (const uint16_t *)a->k_pass;
  L.vp = (const uint16_t *)a->v_pass;
  L.kd = (const uint16_t *)a->k_dec;
  L.vd = (const uint16_t *)a->v_dec;
  L.o = (uint16_t *)a->o;
  L.R = a->rows;
  L.beams = a->beams;
  L.hq = a->hq;
  L.hkv = a->hkv;
  L.head_dim = a->head_dim;
  L.ranges = a->ranges;
  L.n_ranges = a->n_ranges;
  L.path = a->path;
  L.t_cap = a->t_cap;
  L.n_path = a->n_path;
  L.n_pass_rows = a->n_pass_rows;
  L.n_dec_rows = a->t_cap * a->rows;
  L.scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.0f / std::sqrt((float)a->head_dim);
  int e = launch_decode_attention(L, stream);
  if (e) return fail(SPB_ERR_HIP, "decode attention launch: %s", hip_error_string(e));
  return ok();
}

spb_status spb_beam_step(const spb_beam_args *a, void *stream) {
  if (!a) return fail(SPB_ERR_ARG, "args is NULL");
  if (a->n_slots < 0 || a->beams < 1 || a->beams > kMaxBeams || a->k < 1 || a->k > kMaxTopK || a->t_cap < 1 ||
      a->step < 0 || a->step >= a->t_cap)
    return fail(SPB_ERR_ARG, "n_slots %d, beams %d, k %d, t_cap %d, step %d", a->n_slots, a->beams, a->k, a->t_cap,
                a->step);
  if (a->n_slots == 0) return ok();
  if (!a->stop || !a->ids || !a->lp || !a->tok_out || !a->len_out || !a->fin_out || !a->path_out || !a->nb_out ||
      !a->score_out || !a->feed)
    return fail(SPB_ERR_ARG, "NULL tensor");
  if (a->step > 0 && (!a->tok_in || !a->len_in || !a->fin_in || !a->path_in || !a->nb_in || !a->score_in))
    return fail(SPB_ERR_ARG, "steps after the first need the previous state");
  BeamLaunch L{};
  L.n_slots = a->n_slots;
  L.beams = a->beams;
  L.k = a->k;
  L.t_cap = a->t_cap;
  L.step = a->step;
  L.stop = a->stop;
  L.ids = a->ids;
  L.lp = a->lp;
  L.tok_in = a->tok_in;
  L.len_in = a->len_in;
  L.fin_in = a->fin_in;
  L.path_in = a->path_in;
  L.nb_in = a->nb_in;
  L.score_in = a->score_in;
  L.tok_out = a->tok_out;
  L.len_out = a->len_out;
  L.fin_out = a->fin_out;
  L.path_out = a->path_out;
  L.nb_out = a->nb_out;
  L.score_out = a->score_out;
  L.feed = a->feed;
  int e = launch_beam_step(L, stream);
  if (e) return fail(SPB_ERR_HIP, "beam step launch: %s", hip_error_string(e));
  return ok();
}

}  // extern "C"
