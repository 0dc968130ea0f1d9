"""Pointwise definitions of the shape:stride layout algebra (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).  Nothing here is an algorithm from the GPU
library; each function is the definition the pages give, evaluated point by point.

Sources (page title and section):
* "CUTLASS, CuTe, and CUDA Tile" (learn-kernels.com), introduction: a layout is a function from
  integers to integers; (4,3):(3,1) evaluates (1,0) to 3 and (0,1) to 1; a column-major layout
  acts like a flat 1-D layout on 1-D coordinates; coalesce keeps the function; composition is
  R(c) = A(B(c)) and its result is compatible with B.
* Same page, "Partitioning: complement and divide": complement(A, M) is bounded by M, has a
  codomain disjoint from A's and is ordered (positive, increasing strides); logical_divide(A, B)
  is A composed with the concatenation of B and B's complement under size(A); zipped_divide
  gathers the tile modes first and the rest modes second.
* "A10 - CuTe, CUTLASS & CuTile", section 2: the index is the inner product of the natural
  coordinate with the stride; the hierarchical table of (2,(2,2)):(4,(2,1)) fixes how a single
  integer is split over a nested mode (leftmost sub-mode fastest).
* "CUTLASS, CuTe, and CUDA Tile", the local_tile listing after "Partitioning: complement and
  divide": local_tile is zipped_divide by the tiler followed by slicing the rest part with the
  block's coordinate ("_" keeps a mode); a Step with X entries first drops modes.  "CUTLASS"
  (stanleyjacob.dev), Part V, and "A10 - CuTe, CUTLASS & CuTile", "Partitioning Tensors":
  local_partition hands a thread its elements of a tile under a thread layout (the reading used:
  the tile part is sliced at the thread's coordinate and every rest mode is kept).
* "A10 - CuTe, CUTLASS & CuTile", section 3.4: Swizzle<BBits, MBase, SShift> XORs the BBits-wide field that starts
  SShift bits above MBase into the field that starts at MBase.
"""
from __future__ import annotations

import re
from functools import reduce

# A layout is a pair (shape, stride); each is an int or a tuple of (nested) shapes/strides.


def parse(text: str):
    """Parse the pages' notation, e.g. "((2,2),3):((24,2),8)" or "_12:_1"."""
    text = text.replace(" ", "").replace("_", "")
    if ":" not in text:
        raise ValueError(f"not a layout: {text!r}")
    s, d = text.split(":", 1)
    shape, stride = _parse_tuple(s), _parse_tuple(d)
    if not congruent(shape, stride):
        raise ValueError("shape and stride are not congruent")
    return shape, stride


def _parse_tuple(text: str):
    tokens = re.findall(r"\(|\)|,|-?\d+", text)
    pos = 0

    def item():
        nonlocal pos
        tok = tokens[pos]
        if tok == "(":
            pos += 1
            elems = [item()]
            while tokens[pos] == ",":
                pos += 1
                elems.append(item())
            if tokens[pos] != ")":
                raise ValueError("unbalanced")
            pos += 1
            return tuple(elems)
        pos += 1
        return int(tok)

    out = item()
    if pos != len(tokens):
        raise ValueError(f"trailing tokens in {text!r}")
    return out


def fmt(shape, stride=None) -> str:
    """Print in the pages' notation."""
    def f(x):
        if isinstance(x, tuple):
            return "(" + ",".join(f(e) for e in x) + ")"
        return str(x)
    if stride is None:
        shape, stride = shape
    return f(shape) + ":" + f(stride)


def congruent(a, b) -> bool:
    if isinstance(a, tuple) != isinstance(b, tuple):
        return False
    if isinstance(a, tuple):
        return len(a) == len(b) and all(congruent(x, y) for x, y in zip(a, b))
    return True


def size(shape) -> int:
    if isinstance(shape, tuple):
        return reduce(lambda x, y: x * size(y), shape, 1)
    return shape


def flatten(x):
    if isinstance(x, tuple):
        return tuple(leaf for e in x for leaf in flatten(e))
    return (x,)


def split(index: int, shape):
    """Natural coordinate of a single integer: leftmost mode fastest, recursively."""
    if not isinstance(shape, tuple):
        return index
    out = []
    for i, s in enumerate(shape):
        n = size(s)
        if i == len(shape) - 1:
            out.append(split(index, s))
        else:
            out.append(split(index % n, s))
            index //= n
    return tuple(out)


def evaluate(layout, coord) -> int:
    """Inner product of the natural coordinate with the stride.  `coord` may be one integer, or
    a tuple congruent with the shape at the top level whose entries are integers (split over that
    mode) or tuples (recursive)."""
    shape, stride = layout
    if isinstance(coord, int):
        coord = split(coord, shape)
    return _inner(coord, shape, stride)


def _inner(coord, shape, stride) -> int:
    if isinstance(shape, tuple):
        if isinstance(coord, int):
            coord = split(coord, shape)
        if len(coord) != len(shape):
            raise ValueError("coordinate rank does not match the shape")
        return sum(_inner(c, s, d) for c, s, d in zip(coord, shape, stride))
    if isinstance(coord, tuple):
        raise ValueError("coordinate deeper than the shape")
    return coord * stride


def table(layout):
    """The layout as a function on 1-D coordinates 0 .. size-1."""
    return [evaluate(layout, i) for i in range(size(layout[0]))]


def compose_table(a, b):
    """Definition of composition: R(c) = A(B(c)) for every 1-D coordinate c of B."""
    return [evaluate(a, evaluate(b, c)) for c in range(size(b[0]))]


def top_sizes(layout):
    shape = layout[0]
    if isinstance(shape, tuple):
        return tuple(size(s) for s in shape)
    return (shape,)


def compatible(r, b) -> bool:
    """Every coordinate of B is a valid coordinate of R: same top-level rank, same mode sizes."""
    return top_sizes(r) == top_sizes(b)


def bank_set(offsets, banks=32):
    """Distinct banks touched by a set of word offsets (bank = offset mod banks)."""
    return {o % banks for o in offsets}


def swizzle(offset: int, bbits: int, mbase: int, sshift: int) -> int:
    """offset XOR ((offset & yyy_mask) >> SShift), yyy_mask = BBits ones starting at MBase+SShift."""
    mask = ((1 << bbits) - 1) << (mbase + sshift)
    return offset ^ ((offset & mask) >> sshift)


def complement_brute(a, m: int):
    """Complement by construction from its definition: the offsets not reached by A are added
    as new generators, smallest first, so that image(A) + image(R) is a direct sum covering
    0 .. m-1.  Returns (shape, stride) with increasing strides, or None if no such R exists."""
    img = sorted(set(table(a)))
    if len(img) != size(a[0]):
        return None  # A is not injective
    covered = set(img)
    gens = [0]
    for x in range(m):
        if x not in covered:
            new = {y + x for y in img}
            if new & covered:
                return None
            covered |= new
            gens.append(x)
    # all sums  a + g  must be distinct and exactly 0..m-1
    sums = sorted(y + g for y in img for g in gens)
    if sums != list(range(m)):
        return None
    gens = sorted(gens)
    # express the generator set as a layout with increasing strides (colex enumeration sorted)
    shape, stride = [], []
    run = gens
    while len(run) > 1:
        d = run[1] - run[0]
        n = 1
        while n < len(run) and run[n] == n * d:
            n += 1
        if len(run) % n:
            return None
        block = run[:n]
        for k in range(len(run) // n):
            if run[k * n:(k + 1) * n] != [v + run[k * n] for v in block]:
                return None
        shape.append(n)
        stride.append(d)
        run = run[::n]
    if not shape:
        return (1, 0)
    if len(shape) == 1:
        return (shape[0], stride[0])
    return (tuple(shape), tuple(stride))


# ---- local_tile / local_partition -----------------------------------------------------------

def _modes(layout):
    shape, stride = layout
    if isinstance(shape, tuple):
        return list(zip(shape, stride))
    return [(shape, stride)]


def divide_mode(mode, t: int):
    """logical_divide(mode, t:1) by its definition, mode o (t:1, complement(t:1, size(mode))),
    as a table over the 1-D coordinates x + t*r of the concatenation, and the rest size."""
    comp = complement_brute((t, 1), size(mode[0]))
    if comp is None:
        raise ValueError("no complement")
    concat = ((t, comp[0]), (1, comp[1]))
    return compose_table(mode, concat), size(comp[0])


def zipped_divide_by(layout, tiles):
    """zipped_divide by a by-mode tiler of tile sizes: mode i < len(tiles) is divided by
    tiles[i]:1, later modes stay whole in the rest part.  Returns (tile sizes, rest sizes, f)
    with f(tile_coord, rest_coord) the offset, each coordinate a tuple of 1-D mode indices."""
    modes = _modes(layout)
    if len(tiles) > len(modes):
        raise ValueError("tiler longer than the layout")
    tabs, rest = [], []
    for i, m in enumerate(modes):
        if i < len(tiles):
            if size(m[0]) % tiles[i]:
                raise ValueError("tile size does not divide the mode")
            tab, nr = divide_mode(m, tiles[i])
            tabs.append(tab)
            rest.append(nr)
        else:
            rest.append(size(m[0]))

    def f(tc, rc):
        off = 0
        for i, m in enumerate(modes):
            if i < len(tiles):
                off += tabs[i][tc[i] + tiles[i] * rc[i]]
            else:
                off += evaluate(m, rc[i])
        return off

    return tuple(tiles), tuple(rest), f


def local_tile(layout, tiler, coord, proj=None):
    """Block view: zipped_divide by `tiler`, then the rest part sliced at `coord` (None keeps a
    mode).  `proj` entries of "X" drop the matching tiler and coord entries first.  Returns
    (mode sizes of the view, g) with g(c) the offset of view coordinate c (a tuple of 1-D mode
    indices: the tile modes, then the kept rest modes)."""
    if proj is not None:
        keep = [i for i, st in enumerate(proj) if st != "X"]
        tiler = [tiler[i] for i in keep]
        coord = [coord[i] for i in keep]
    tiles, rest, f = zipped_divide_by(layout, tiler)
    if len(coord) != len(rest):
        raise ValueError("coordinate rank does not match the rest part")
    kept = [i for i, c in enumerate(coord) if c is None]
    for i, c in enumerate(coord):
        if c is not None and not 0 <= c < rest[i]:
            raise ValueError("coordinate outside its mode")

    def g(c):
        rc = list(coord)
        for j, i in enumerate(kept):
            rc[i] = c[len(tiles) + j]
        return f(tuple(c[:len(tiles)]), tuple(rc))

    return tuple(tiles) + tuple(rest[i] for i in kept), g


def local_partition(layout, thr_shape, idx: int):
    """Thread view: zipped_divide by the thread shape, then the tile part sliced at thread idx's
    coordinate in that shape (leftmost fastest); every rest mode is kept.  Returns (mode sizes, g)
    as local_tile does."""
    n = size(tuple(thr_shape))
    if not 0 <= idx < n:
        raise ValueError("thread index outside the thread shape")
    tiles, rest, f = zipped_divide_by(layout, thr_shape)
    tc = []
    for t in thr_shape:
        tc.append(idx % t)
        idx //= t
    return tuple(rest), lambda c: f(tuple(tc), tuple(c))
