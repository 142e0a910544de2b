"""Write lncc_maps.hpp: thread -> task maps of stages BC and D of the LNCC
kernel for window radius 4 (the w = 9 window), chosen so that their LDS
accesses are free of bank conflicts on gfx950.

LDS on gfx950 has 64 banks of 4 bytes. How a wave's lanes are served was
measured on an MI355X with two active lanes on the same banks, read off the
SQ_LDS_BANK_CONFLICT counter (profiles/lds_lane_groups_gfx950.txt):
  16-byte reads  16 lanes per pass, in the groups GA = {0-3, 12-15, 20-27}
                 and GB = {4-11, 16-19, 28-31} of each half-wave;
  8-byte writes  16 consecutive lanes per pass.
Lanes served in one pass must touch distinct banks. A half-wave therefore
splits into four cells of 8 lanes, the intersections of {GA, GB} with the
write groups {0-15, 16-31}.

Stage BC: a task is a column bc of the coefficient region and a pair of rows
2bs, 2bs + 1 (CX = 40 columns, 12 row pairs). It reads its column of the
x-boxed moment sums with 16-byte loads at (f*CX + bc)*ROWP + 2bs + 2i
doubles (bank group u = (ROWP/2*bc + bs) mod 16) and writes three
coefficients with 8-byte stores at (k*CY + 2bs + r)*CXP + bc doubles (bank
pair v = (2*CXP*bs + bc) mod 32).

Stage D: a task is a coefficient field df, a row dr (CY = 24) and a segment
of 8 columns dsg (4 per row). It reads 16 doubles of its row with 16-byte
loads at (df*CY + dr)*CXP + 8*dsg + 2i (u = (CXP/2*(df*CY + dr) + 4*dsg)
mod 16) and writes its 8 x-boxed values transposed with 8-byte stores at
(df*TX + 8*dsg + k)*TYP + dr (v = (TYP*(TX*df + 8*dsg) + dr) mod 32). Its
288 tasks stay on the first five waves.

Each map is an integer feasibility problem (scipy's HiGHS): a binary x[t][c]
puts task t in cell c; a cell holds at most 8 tasks, a read group (two
cells) at most one task of each u and a write group (two cells) at most one
of each v. The lanes of a cell take its tasks in task order; unused lanes
get 0xFFFF (no task).

Usage: python gen_lncc_maps.py  (rewrites lncc_maps.hpp next to this file)
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
NTHREADS = 512
GA = (0, 1, 2, 3, 12, 13, 14, 15, 20, 21, 22, 23, 24, 25, 26, 27)
GB = (4, 5, 6, 7, 8, 9, 10, 11, 16, 17, 18, 19, 28, 29, 30, 31)
# cells of a half-wave: (GA, lanes 0-15), (GA, 16-31), (GB, 0-15), (GB, 16-31)
CELLS = tuple(tuple(l for l in g if lo <= l < lo + 16) for g in (GA, GB) for lo in (0, 16))

# layout of the radius-4 kernel (TX = 32, TY = 16): coefficient region CX x CY,
# LDS strides in doubles of the moment sums, coefficients and x-boxed coefficients
TX, CX, CY, ROWP, CXP, TYP = 32, 40, 24, 34, 42, 26


def bc_tasks():
    tasks = [(bc, bs) for bs in range(CY // 2) for bc in range(CX)]
    u = [((ROWP // 2) * bc + bs) % 16 for bc, bs in tasks]
    v = [(2 * CXP * bs + bc) % 32 for bc, bs in tasks]
    return tasks, u, v


def d_tasks():
    tasks = [(dr, dsg, df) for df in range(3) for dsg in range(TX // 8) for dr in range(CY)]
    u = [((CXP // 2) * (df * CY + dr) + 4 * dsg) % 16 for dr, dsg, df in tasks]
    v = [(TYP * (TX * df + 8 * dsg) + dr) % 32 for dr, dsg, df in tasks]
    return tasks, u, v


def solve(u, v, nhalves):
    """Lane -> task index (or None) over the first nhalves half-waves."""
    from scipy.optimize import Bounds, LinearConstraint, milp
    from scipy.sparse import lil_matrix
    T, C = len(u), 4 * nhalves
    rows, lo, hi = [], [], []

    def add(cols, a, b):
        rows.append(cols)
        lo.append(a)
        hi.append(b)

    for t in range(T):
        add([t * C + c for c in range(C)], 1, 1)
    for c in range(C):
        add([t * C + c for t in range(T)], 0, 8)
    for h in range(nhalves):
        for cells in ((0, 1), (2, 3)):      # read groups GA, GB
            for uu in set(u):
                add([t * C + 4 * h + c for t in range(T) if u[t] == uu for c in cells], 0, 1)
        for cells in ((0, 2), (1, 3)):      # write groups 0-15, 16-31
            for vv in set(v):
                add([t * C + 4 * h + c for t in range(T) if v[t] == vv for c in cells], 0, 1)
    A = lil_matrix((len(rows), T * C))
    for r, cols in enumerate(rows):
        for col in cols:
            A[r, col] = 1
    res = milp(c=np.zeros(T * C), constraints=LinearConstraint(A.tocsr(), lo, hi), integrality=np.ones(T * C),
               bounds=Bounds(0, 1), options={"time_limit": 900})
    if res.x is None:
        raise SystemExit(f"no conflict-free map: {res.message}")
    cell_of = np.argmax(res.x.reshape(T, C), axis=1)
    lanes = [None] * NTHREADS
    for c in range(C):
        h, cc = divmod(c, 4)
        for j, t in enumerate(t for t in range(T) if cell_of[t] == c):
            lanes[32 * h + CELLS[cc][j]] = t
    return lanes


def check(lanes, u, v, ntasks):
    """Every task on exactly one lane; no two lanes of a read group share u,
    no two lanes of a write group share v."""
    assert sorted(t for t in lanes if t is not None) == list(range(ntasks)), "not a task permutation"
    for h in range(NTHREADS // 32):
        for g in (GA, GB):
            us = [u[lanes[32 * h + l]] for l in g if lanes[32 * h + l] is not None]
            assert len(us) == len(set(us)), f"read conflict in half-wave {h}"
        for lo in (0, 16):
            vs = [v[lanes[32 * h + l]] for l in range(lo, lo + 16) if lanes[32 * h + l] is not None]
            assert len(vs) == len(set(vs)), f"write conflict in half-wave {h}"


def build():
    tb, ub, vb = bc_tasks()
    lb = solve(ub, vb, NTHREADS // 32)
    check(lb, ub, vb, len(tb))
    td, ud, vd = d_tasks()
    ld = solve(ud, vd, 10)
    check(ld, ud, vd, len(td))
    bc = [0xFFFF if t is None else (tb[t][1] << 8) | tb[t][0] for t in lb]
    d = [0xFFFF if t is None else (td[t][2] << 12) | (td[t][1] << 8) | td[t][0] for t in ld]
    return bc, d


def table(name, vals):
    body = ",\n".join("    " + ", ".join(f"0x{e:04x}" for e in vals[i:i + 8]) for i in range(0, len(vals), 8))
    return f"__constant__ unsigned short {name}[{len(vals)}] = {{\n{body}}};\n"


def write(bc, d, path):
    with open(path, "w") as fh:
        fh.write("// Generated by gen_lncc_maps.py (do not edit): thread -> task maps of stages BC\n"
                 "// and D of the LNCC kernel for window radius 4, free of LDS bank conflicts.\n"
                 "// BC entry: (row pair bs << 8) | column bc.  D entry: (field df << 12) |\n"
                 "// (8-column segment dsg << 8) | row dr.  0xffff = no task.\n"
                 "#pragma once\n\nnamespace ngv {\n\n" + table("kLnccBcMapR4", bc) + "\n" + table("kLnccDMapR4", d) +
                 "\n}  // namespace ngv\n")


def read(path):
    txt = open(path).read()
    out = []
    for name in ("kLnccBcMapR4", "kLnccDMapR4"):
        i = txt.index("{", txt.index(name))
        out.append([int(x, 16) for x in txt[i + 1:txt.index("};", i)].replace("\n", " ").split(",") if x.strip()])
    return out


if __name__ == "__main__":
    bc, d = build()
    out = os.path.join(HERE, "lncc_maps.hpp")
    write(bc, d, out)
    assert read(out) == [bc, d]
    print(f"wrote {out}")
    sys.exit(0)
