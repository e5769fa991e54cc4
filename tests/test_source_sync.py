"""The tiled P2G kernel keeps its own copy of the rows loop (the shared
item_rows function, inlined into that kernel, is scheduled differently and
measured 16% slower on the blob workload).  The two copies must compute the
same thing: outside the per-record pad and range handling, which differs on
purpose (the tiled path's records were range-checked at binning), their
source must agree token for token."""
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "material_point_particle_amd",
                    "csrc")
START = "for (uint32_t j = 0; j < rows; ++j) {"
END = "atomicAdd(&acc[ch * TS::nodes + lb + off], sum);"
CUT_FROM = "rec[4 * q + 3] = t.w; }"
CUT_TO = "group_hoist<DIM>(rec, a.nf, a.dx, a.last_base, a.S, h[k]);"


def _rows_loop(path: str, anchor: str) -> str:
    src = open(path).read()
    src = src[src.index(anchor):]
    text = src[src.index(START):src.index(END) + len(END)]
    text = re.sub(r"//[^\n]*", "", text)
    text = " ".join(text.split())
    i, j = text.index(CUT_FROM) + len(CUT_FROM), text.index(CUT_TO)
    return text[:i] + " " + text[j:]


def test_tiled_rows_loop_matches_the_shared_one():
    tiled = _rows_loop(os.path.join(CSRC, "p2g.hip"), "p2g_tiled_kernel(TiledArgs a)")
    shared = _rows_loop(os.path.join(CSRC, "p2g_device.hpp"), "__device__ __forceinline__ void item_rows")
    assert len(tiled) > 1500
    assert tiled == shared
