// layout.cpp -- host implementation of the shape:stride layout functions declared in htlayout.h.
//
// The algorithms are this library's reading of the definitions and worked examples on the pages
// ("CUTLASS, CuTe, and CUDA Tile", introduction and "Partitioning: complement and divide"):
//
//  * eval: inner product of the natural coordinate with the stride; an integer standing for a
//    nested mode is split over it with the leftmost sub-mode fastest.
//  * coalesce: flatten, drop size-1 modes, merge neighbours (s0:d0)(s1:d1) when d1 == s0*d0.
//  * compose(A, B): distributes over the modes of B.  For a leaf mode s:d of B, A (flattened) is
//    first divided by d -- whole leading modes whose size divides what is left of d are dropped,
//    and the mode where d runs out keeps size/d with its stride times d -- and then s is taken
//    from the remaining modes in order, splitting the last mode used.  The last mode of A is
//    treated as unbounded, so a B reaching past size(A) extends it.  A mode of B that yields
//    several modes becomes a nested tuple, which keeps the result compatible with B.
//  * complement(A, M): walk A's modes by increasing stride; every gap between the extent reached
//    so far and the next stride becomes a new mode, and a final mode extends the extent to M.
//  * logical_divide(A, B) = compose(A, (B, complement(B, size(A)))).
//  * zipped_divide(A, <B0, B1>) = ((tile0, tile1), (rest0, rest1)) from the per-mode divides.
#include "../../include/htlayout.h"

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

namespace {

struct Tup {
  bool leaf = true;
  int64_t v = 0;
  std::vector<Tup> c;
  static Tup L(int64_t x) { Tup t; t.leaf = true; t.v = x; return t; }
  static Tup N(std::vector<Tup> xs) { Tup t; t.leaf = false; t.c = std::move(xs); return t; }
};

struct Layout {
  Tup shape, stride;
};

// ---- parsing ------------------------------------------------------------------------------
struct Parser {
  const char* p;
  bool ok = true;
  void ws() { while (*p == ' ' || *p == '_' || *p == '\t') ++p; }
  Tup item() {
    ws();
    if (*p == '(') {
      ++p;
      std::vector<Tup> xs;
      xs.push_back(item());
      ws();
      while (ok && *p == ',') { ++p; xs.push_back(item()); ws(); }
      if (*p != ')') { ok = false; return Tup(); }
      ++p;
      return Tup::N(std::move(xs));
    }
    bool neg = false;
    if (*p == '-') { neg = true; ++p; ws(); }
    if (*p < '0' || *p > '9') { ok = false; return Tup(); }
    int64_t v = 0;
    while (*p >= '0' && *p <= '9') {
      if (v > (INT64_MAX - 9) / 10) { ok = false; return Tup(); }
      v = v * 10 + (*p - '0');
      ++p;
      ws();
    }
    return Tup::L(neg ? -v : v);
  }
};

bool congruent(const Tup& a, const Tup& b) {
  if (a.leaf != b.leaf) return false;
  if (a.leaf) return true;
  if (a.c.size() != b.c.size()) return false;
  for (size_t i = 0; i < a.c.size(); ++i)
    if (!congruent(a.c[i], b.c[i])) return false;
  return true;
}

bool parse_tuple(const char* s, const char* end, Tup* out) {
  std::string tmp(s, end);
  Parser ps{tmp.c_str()};
  Tup t = ps.item();
  ps.ws();
  if (!ps.ok || *ps.p != '\0') return false;
  *out = t;
  return true;
}

bool parse_layout(const char* text, Layout* out) {
  if (!text) return false;
  const char* colon = std::strchr(text, ':');
  if (!colon) return false;
  Layout l;
  if (!parse_tuple(text, colon, &l.shape)) return false;
  if (!parse_tuple(colon + 1, colon + std::strlen(colon), &l.stride)) return false;
  if (!congruent(l.shape, l.stride)) return false;
  *out = l;
  return true;
}

bool positive_shape(const Tup& t) {
  if (t.leaf) return t.v >= 1;
  for (auto& x : t.c)
    if (!positive_shape(x)) return false;
  return true;
}

// ---- printing -----------------------------------------------------------------------------
void print(const Tup& t, std::string& s) {
  if (t.leaf) { s += std::to_string(t.v); return; }
  s += '(';
  for (size_t i = 0; i < t.c.size(); ++i) {
    if (i) s += ',';
    print(t.c[i], s);
  }
  s += ')';
}

std::string to_string(const Layout& l) {
  std::string s;
  print(l.shape, s);
  s += ':';
  print(l.stride, s);
  return s;
}

int emit(const std::string& s, char* out, size_t cap) {
  if (!out || s.size() + 1 > cap) return HT_ERR_CAPACITY;
  std::memcpy(out, s.c_str(), s.size() + 1);
  return HT_OK;
}

// ---- basic functions ----------------------------------------------------------------------
int64_t size_of(const Tup& t) {
  if (t.leaf) return t.v;
  int64_t n = 1;
  for (auto& x : t.c) n *= size_of(x);
  return n;
}

void flatten(const Tup& s, const Tup& d, std::vector<int64_t>& fs, std::vector<int64_t>& fd) {
  if (s.leaf) { fs.push_back(s.v); fd.push_back(d.v); return; }
  for (size_t i = 0; i < s.c.size(); ++i) flatten(s.c[i], d.c[i], fs, fd);
}

// Inner product of a coordinate with the stride; `coord` may be an integer for a nested mode.
bool inner(const Tup& coord, const Tup& shape, const Tup& stride, int64_t* acc) {
  if (shape.leaf) {
    if (!coord.leaf || coord.v < 0) return false;
    *acc += coord.v * stride.v;
    return true;
  }
  if (coord.leaf) {  // split an integer over the nested mode, leftmost fastest
    int64_t idx = coord.v;
    if (idx < 0) return false;
    for (size_t i = 0; i < shape.c.size(); ++i) {
      int64_t n = size_of(shape.c[i]);
      int64_t here = (i + 1 == shape.c.size()) ? idx : idx % n;
      if (!inner(Tup::L(here), shape.c[i], stride.c[i], acc)) return false;
      if (i + 1 < shape.c.size()) idx /= n;
    }
    return true;
  }
  if (coord.c.size() != shape.c.size()) return false;
  for (size_t i = 0; i < shape.c.size(); ++i)
    if (!inner(coord.c[i], shape.c[i], stride.c[i], acc)) return false;
  return true;
}

// Coordinate within the shape (each leaf coordinate below its extent)?
bool in_range(const Tup& coord, const Tup& shape) {
  if (coord.leaf) return coord.v >= 0 && coord.v < size_of(shape);
  if (shape.leaf || coord.c.size() != shape.c.size()) return false;
  for (size_t i = 0; i < shape.c.size(); ++i)
    if (!in_range(coord.c[i], shape.c[i])) return false;
  return true;
}

Layout make_flat(const std::vector<int64_t>& s, const std::vector<int64_t>& d) {
  Layout r;
  if (s.empty()) { r.shape = Tup::L(1); r.stride = Tup::L(0); return r; }
  if (s.size() == 1) { r.shape = Tup::L(s[0]); r.stride = Tup::L(d[0]); return r; }
  std::vector<Tup> ss, dd;
  for (size_t i = 0; i < s.size(); ++i) { ss.push_back(Tup::L(s[i])); dd.push_back(Tup::L(d[i])); }
  r.shape = Tup::N(ss);
  r.stride = Tup::N(dd);
  return r;
}

Layout coalesce(const Layout& l) {
  std::vector<int64_t> fs, fd, os, od;
  flatten(l.shape, l.stride, fs, fd);
  for (size_t i = 0; i < fs.size(); ++i) {
    if (fs[i] == 1) continue;
    if (!os.empty() && fd[i] == os.back() * od.back()) {
      os.back() *= fs[i];
      continue;
    }
    os.push_back(fs[i]);
    od.push_back(fd[i]);
  }
  return make_flat(os, od);
}

// compose A with one leaf mode s:d of B.
int compose_leaf(const std::vector<int64_t>& as_in, const std::vector<int64_t>& at_in, int64_t s,
                 int64_t d, Layout* out) {
  if (s == 1) { *out = make_flat({1}, {0}); return HT_OK; }
  if (d == 0) { *out = make_flat({s}, {0}); return HT_OK; }
  if (d < 0 || s < 1) return HT_ERR_NOT_COMPOSABLE;
  std::vector<int64_t> as = as_in, at = at_in;
  size_t n = as.size(), i = 0;
  int64_t rd = d;
  // divide out the stride d
  while (rd > 1) {
    if (i + 1 == n) {  // unbounded last mode
      at[i] *= rd;
      if (as[i] % rd == 0) as[i] /= rd; else as[i] = 0;  // 0 marks "past the end"
      rd = 1;
      break;
    }
    if (rd % as[i] == 0) { rd /= as[i]; ++i; }
    else if (as[i] % rd == 0) { as[i] /= rd; at[i] *= rd; rd = 1; }
    else return HT_ERR_NOT_COMPOSABLE;
  }
  // take s elements from the remaining modes
  std::vector<int64_t> os, od;
  int64_t rs = s;
  while (rs > 1) {
    if (i + 1 >= n) { os.push_back(rs); od.push_back(at[n - 1]); rs = 1; break; }
    if (as[i] == 1) { ++i; continue; }
    if (as[i] % rs == 0) { os.push_back(rs); od.push_back(at[i]); rs = 1; }
    else if (rs % as[i] == 0) { os.push_back(as[i]); od.push_back(at[i]); rs /= as[i]; ++i; }
    else return HT_ERR_NOT_COMPOSABLE;
  }
  *out = make_flat(os, od);
  return HT_OK;
}

int compose_rec(const std::vector<int64_t>& as, const std::vector<int64_t>& at, const Tup& bs,
                const Tup& bd, Tup* rs, Tup* rd) {
  if (bs.leaf) {
    Layout l;
    int rc = compose_leaf(as, at, bs.v, bd.v, &l);
    if (rc) return rc;
    *rs = l.shape;
    *rd = l.stride;
    return HT_OK;
  }
  std::vector<Tup> ss, dd;
  for (size_t i = 0; i < bs.c.size(); ++i) {
    Tup s, d;
    int rc = compose_rec(as, at, bs.c[i], bd.c[i], &s, &d);
    if (rc) return rc;
    ss.push_back(s);
    dd.push_back(d);
  }
  *rs = Tup::N(ss);
  *rd = Tup::N(dd);
  return HT_OK;
}

int compose(const Layout& a, const Layout& b, Layout* out) {
  std::vector<int64_t> as, at;
  flatten(a.shape, a.stride, as, at);
  return compose_rec(as, at, b.shape, b.stride, &out->shape, &out->stride);
}

int complement(const Layout& a, int64_t m, Layout* out) {
  std::vector<int64_t> fs, fd;
  flatten(a.shape, a.stride, fs, fd);
  std::vector<std::pair<int64_t, int64_t>> modes;  // (stride, size)
  for (size_t i = 0; i < fs.size(); ++i)
    if (fs[i] > 1 && fd[i] != 0) {
      if (fd[i] < 0) return HT_ERR_NO_COMPLEMENT;
      modes.push_back({fd[i], fs[i]});
    }
  std::sort(modes.begin(), modes.end());
  std::vector<int64_t> os, od;
  int64_t cur = 1;
  for (auto& md : modes) {
    int64_t d = md.first, s = md.second;
    if (d % cur != 0) return HT_ERR_NO_COMPLEMENT;
    int64_t gap = d / cur;
    if (gap > 1) { os.push_back(gap); od.push_back(cur); }
    cur = s * d;
  }
  int64_t rest = (m + cur - 1) / cur;
  if (rest > 1) { os.push_back(rest); od.push_back(cur); }
  *out = coalesce(make_flat(os, od));
  return HT_OK;
}

int logical_divide(const Layout& a, const Layout& b, Layout* out) {
  Layout c;
  int rc = complement(b, size_of(a.shape), &c);
  if (rc) return rc;
  Layout cat;
  cat.shape = Tup::N({b.shape, c.shape});
  cat.stride = Tup::N({b.stride, c.stride});
  return compose(a, cat, out);
}

// A flat tuple whose entries are integers or "_" (keep the whole mode), e.g. "(1,_)", "_" or
// "3"; "X" entries are accepted when `allow_x` (projection steps, "(1,X,1)").  Kept entries are
// returned as -1, X entries as -2.
bool parse_slots(const char* text, bool allow_x, std::vector<int64_t>* out) {
  if (!text) return false;
  std::string t;
  for (const char* q = text; *q; ++q)
    if (*q != ' ' && *q != '\t') t += *q;
  if (t.empty()) return false;
  if (t.front() == '(') {
    if (t.back() != ')') return false;
    t = t.substr(1, t.size() - 2);
  }
  std::vector<int64_t> v;
  size_t i = 0;
  while (true) {
    size_t j = t.find(',', i);
    std::string e = t.substr(i, j == std::string::npos ? std::string::npos : j - i);
    if (e == "_") {
      v.push_back(-1);
    } else if (e == "X" && allow_x) {
      v.push_back(-2);
    } else {
      if (e.empty() || e.size() > 18) return false;
      int64_t x = 0;
      for (char ch : e) {
        if (ch < '0' || ch > '9') return false;
        x = x * 10 + (ch - '0');
      }
      v.push_back(x);
    }
    if (j == std::string::npos) break;
    i = j + 1;
  }
  *out = std::move(v);
  return true;
}

// Top-level modes of a layout (a rank-1 layout with a leaf shape is its own single mode).
std::vector<Layout> modes_of(const Layout& l) {
  std::vector<Layout> m;
  if (l.shape.leaf) {
    m.push_back(l);
  } else {
    for (size_t i = 0; i < l.shape.c.size(); ++i) m.push_back({l.shape.c[i], l.stride.c[i]});
  }
  return m;
}

// zipped_divide by a by-mode tiler of tile sizes: mode i < tiles.size() is logically divided by
// tiles[i]:1 into (tile_i, rest_i); the modes past the tiler stay whole in the rest part.  The
// result is returned as the list of tile modes and the list of rest modes, in order.  Each tile
// size must divide its mode's size.
int zipped_divide_by(const Layout& a, const std::vector<int64_t>& tiles, std::vector<Layout>* tile,
                     std::vector<Layout>* rest) {
  std::vector<Layout> m = modes_of(a);
  if (tiles.size() > m.size()) return HT_ERR_RANGE;
  tile->clear();
  rest->clear();
  for (size_t i = 0; i < m.size(); ++i) {
    if (i >= tiles.size()) {
      rest->push_back(m[i]);
      continue;
    }
    if (tiles[i] < 1 || size_of(m[i].shape) % tiles[i] != 0) return HT_ERR_NOT_COMPOSABLE;
    Layout d;
    int rc = logical_divide(m[i], Layout{Tup::L(tiles[i]), Tup::L(1)}, &d);
    if (rc) return rc;
    tile->push_back({d.shape.c[0], d.stride.c[0]});
    rest->push_back({d.shape.c[1], d.stride.c[1]});
  }
  return HT_OK;
}

// Slices a list of modes: entries >= 0 fix a (1-D) coordinate of that mode, whose offset is
// added to *offset; entries -1 keep the mode, appended to `kept`.
int slice_modes(const std::vector<Layout>& modes, const std::vector<int64_t>& coord,
                int64_t* offset, std::vector<Layout>* kept) {
  if (coord.size() != modes.size()) return HT_ERR_RANGE;
  for (size_t i = 0; i < modes.size(); ++i) {
    if (coord[i] == -1) {
      kept->push_back(modes[i]);
      continue;
    }
    if (coord[i] < 0 || coord[i] >= size_of(modes[i].shape)) return HT_ERR_RANGE;
    int64_t acc = 0;
    inner(Tup::L(coord[i]), modes[i].shape, modes[i].stride, &acc);
    *offset += acc;
  }
  return HT_OK;
}

Layout join_modes(const std::vector<Layout>& m) {
  if (m.empty()) return Layout{Tup::L(1), Tup::L(0)};
  if (m.size() == 1) return m[0];
  Layout r;
  std::vector<Tup> s, d;
  for (auto& x : m) {
    s.push_back(x.shape);
    d.push_back(x.stride);
  }
  r.shape = Tup::N(std::move(s));
  r.stride = Tup::N(std::move(d));
  return r;
}

}  // namespace

extern "C" {

int ht_layout_eval(const char* layout, const int64_t* coord, int rank, int64_t* out) {
  Layout l;
  if (!parse_layout(layout, &l) || !out || (rank > 0 && !coord)) return HT_ERR_PARSE;
  // rank 1: one integer over the whole layout; rank r > 1: one integer per top-level mode
  Tup c;
  if (rank == 1) {
    c = Tup::L(coord[0]);
  } else if (rank > 1 && !l.shape.leaf && (size_t)rank == l.shape.c.size()) {
    std::vector<Tup> xs;
    for (int i = 0; i < rank; ++i) xs.push_back(Tup::L(coord[i]));
    c = Tup::N(std::move(xs));
  } else {
    return HT_ERR_RANGE;
  }
  if (!in_range(c, l.shape)) return HT_ERR_RANGE;
  int64_t acc = 0;
  if (!inner(c, l.shape, l.stride, &acc)) return HT_ERR_RANGE;
  *out = acc;
  return HT_OK;
}

int ht_layout_eval_str(const char* layout, const char* coord, int64_t* out) {
  Layout l;
  if (!parse_layout(layout, &l) || !coord || !out) return HT_ERR_PARSE;
  Tup c;
  if (!parse_tuple(coord, coord + std::strlen(coord), &c)) return HT_ERR_PARSE;
  if (!in_range(c, l.shape)) return HT_ERR_RANGE;
  int64_t acc = 0;
  if (!inner(c, l.shape, l.stride, &acc)) return HT_ERR_RANGE;
  *out = acc;
  return HT_OK;
}

int ht_layout_size(const char* layout, int64_t* out) {
  Layout l;
  if (!parse_layout(layout, &l) || !out) return HT_ERR_PARSE;
  *out = size_of(l.shape);
  return HT_OK;
}

int ht_layout_table(const char* layout, int64_t* out, int64_t cap) {
  Layout l;
  if (!parse_layout(layout, &l) || !positive_shape(l.shape)) return HT_ERR_PARSE;
  int64_t n = size_of(l.shape);
  if (!out || cap < n) return HT_ERR_CAPACITY;
  for (int64_t i = 0; i < n; ++i) {
    int64_t acc = 0;
    inner(Tup::L(i), l.shape, l.stride, &acc);
    out[i] = acc;
  }
  return HT_OK;
}

int ht_layout_coalesce(const char* layout, char* out, size_t cap) {
  Layout l;
  if (!parse_layout(layout, &l) || !positive_shape(l.shape)) return HT_ERR_PARSE;
  return emit(to_string(coalesce(l)), out, cap);
}

int ht_layout_compose(const char* a, const char* b, char* out, size_t cap) {
  Layout la, lb, r;
  if (!parse_layout(a, &la) || !parse_layout(b, &lb)) return HT_ERR_PARSE;
  if (!positive_shape(la.shape) || !positive_shape(lb.shape)) return HT_ERR_PARSE;
  int rc = compose(la, lb, &r);
  if (rc) return rc;
  return emit(to_string(r), out, cap);
}

int ht_layout_complement(const char* a, int64_t m, char* out, size_t cap) {
  Layout la, r;
  if (!parse_layout(a, &la) || !positive_shape(la.shape)) return HT_ERR_PARSE;
  if (m < 1) return HT_ERR_RANGE;
  int rc = complement(la, m, &r);
  if (rc) return rc;
  return emit(to_string(r), out, cap);
}

int ht_layout_logical_divide(const char* a, const char* b, char* out, size_t cap) {
  Layout la, lb, r;
  if (!parse_layout(a, &la) || !parse_layout(b, &lb)) return HT_ERR_PARSE;
  if (!positive_shape(la.shape) || !positive_shape(lb.shape)) return HT_ERR_PARSE;
  int rc = logical_divide(la, lb, &r);
  if (rc) return rc;
  return emit(to_string(r), out, cap);
}

int ht_layout_zipped_divide(const char* a, const char* tiler0, const char* tiler1, char* out,
                            size_t cap) {
  Layout la, t0, t1;
  if (!parse_layout(a, &la) || !parse_layout(tiler0, &t0) || !parse_layout(tiler1, &t1))
    return HT_ERR_PARSE;
  if (la.shape.leaf || la.shape.c.size() != 2) return HT_ERR_PARSE;
  Layout m0{la.shape.c[0], la.stride.c[0]}, m1{la.shape.c[1], la.stride.c[1]};
  Layout d0, d1;
  int rc = logical_divide(m0, t0, &d0);
  if (rc) return rc;
  rc = logical_divide(m1, t1, &d1);
  if (rc) return rc;
  // d = (tile, rest) per mode; zip into ((tile0, tile1), (rest0, rest1))
  Layout z;
  z.shape = Tup::N({Tup::N({d0.shape.c[0], d1.shape.c[0]}), Tup::N({d0.shape.c[1], d1.shape.c[1]})});
  z.stride = Tup::N({Tup::N({d0.stride.c[0], d1.stride.c[0]}), Tup::N({d0.stride.c[1], d1.stride.c[1]})});
  return emit(to_string(z), out, cap);
}

int ht_layout_local_tile(const char* a, const char* tiler, const char* coord, const char* proj,
                         int64_t* offset, char* out, size_t cap) {
  Layout la;
  if (!parse_layout(a, &la) || !positive_shape(la.shape) || !offset) return HT_ERR_PARSE;
  std::vector<int64_t> tiles, crd;
  if (!parse_slots(tiler, false, &tiles) || !parse_slots(coord, false, &crd)) return HT_ERR_PARSE;
  for (int64_t t : tiles)
    if (t < 1) return HT_ERR_PARSE;  // a tiler entry is a tile size, never "_"
  if (proj) {
    // keep the tiler and coordinate entries whose step is 1, drop those marked X
    std::vector<int64_t> step;
    if (!parse_slots(proj, true, &step)) return HT_ERR_PARSE;
    if (step.size() != tiles.size() || step.size() != crd.size()) return HT_ERR_RANGE;
    std::vector<int64_t> t2, c2;
    for (size_t i = 0; i < step.size(); ++i) {
      if (step[i] == -2) continue;
      if (step[i] != 1) return HT_ERR_PARSE;
      t2.push_back(tiles[i]);
      c2.push_back(crd[i]);
    }
    tiles.swap(t2);
    crd.swap(c2);
  }
  std::vector<Layout> tile, rest, kept;
  int rc = zipped_divide_by(la, tiles, &tile, &rest);
  if (rc) return rc;
  int64_t off = 0;
  rc = slice_modes(rest, crd, &off, &kept);
  if (rc) return rc;
  std::vector<Layout> res = tile;
  res.insert(res.end(), kept.begin(), kept.end());
  rc = emit(to_string(join_modes(res)), out, cap);
  if (rc) return rc;
  *offset = off;
  return HT_OK;
}

int ht_layout_local_partition(const char* a, const char* thr_shape, int64_t idx, int64_t* offset,
                              char* out, size_t cap) {
  Layout la;
  if (!parse_layout(a, &la) || !positive_shape(la.shape) || !offset) return HT_ERR_PARSE;
  std::vector<int64_t> thr;
  if (!parse_slots(thr_shape, false, &thr)) return HT_ERR_PARSE;
  int64_t nthr = 1;
  for (int64_t t : thr) {
    if (t < 1) return HT_ERR_PARSE;
    nthr *= t;
  }
  if (idx < 0 || idx >= nthr) return HT_ERR_RANGE;
  std::vector<Layout> tile, rest;
  int rc = zipped_divide_by(la, thr, &tile, &rest);
  if (rc) return rc;
  // the thread's coordinate in the thread shape, leftmost mode fastest
  std::vector<int64_t> tc;
  for (int64_t t : thr) {
    tc.push_back(idx % t);
    idx /= t;
  }
  int64_t off = 0;
  std::vector<Layout> none;
  rc = slice_modes(tile, tc, &off, &none);
  if (rc) return rc;
  rc = emit(to_string(join_modes(rest)), out, cap);
  if (rc) return rc;
  *offset = off;
  return HT_OK;
}

int64_t ht_swizzle(int64_t offset, int bbits, int mbase, int sshift) {
  if (bbits <= 0) return offset;
  int64_t mask = ((int64_t(1) << bbits) - 1) << (mbase + sshift);
  return offset ^ ((offset & mask) >> sshift);
}

int ht_tile_plan(int64_t m, int64_t n, int64_t k, int bytes_per_elem, int64_t budget_bytes,
                 ht_tile_stats* out) {
  if (!out || m < 0 || n < 0 || k < 0 || bytes_per_elem < 1) return HT_ERR_RANGE;
  out->flops = 2 * m * n * k;
  out->bytes = int64_t(bytes_per_elem) * (m * k + k * n + m * n);
  out->intensity = out->bytes ? double(out->flops) / double(out->bytes) : 0.0;
  out->double_buffer_bytes = 2 * int64_t(bytes_per_elem) * (m * k + k * n);
  out->fits = out->double_buffer_bytes <= budget_bytes;
  return HT_OK;
}

double ht_pipeline_time(int64_t n, double load, double compute) {
  if (n <= 0) return 0.0;
  return load + compute + double(n - 1) * std::max(load, compute);
}

}  // extern "C"
