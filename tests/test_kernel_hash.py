"""The kernel hash that ties profiles/ to the code they measured: comment
and whitespace edits keep it, code and build-flag changes move it, and
every committed kernel profile carries the current one (a profile of other
code would be stale)."""
import glob
import os
import re

from layer_streamed_optimizer_amd import build, rocprof_summary as rs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _reader(edit=lambda name, text: text):
    def read(name):
        with open(os.path.join(rs.HERE, name), encoding="utf-8") as f:
            return edit(name, f.read())
    return read


def test_comments_and_whitespace_do_not_move_the_hash():
    base = rs.kernel_hash()
    assert rs.kernel_hash(_reader()) == base
    commented = _reader(lambda n, t: "// a new first line\n/* a block\n comment */\n" + t.replace("\n", "\n\n    "))
    assert rs.kernel_hash(commented) == base


def test_code_and_flags_move_the_hash():
    base = rs.kernel_hash()
    changed = _reader(lambda n, t: t.replace("fmaf(c.b1, m, c.c1 * g)", "fmaf(c.b1, m, g)")
                      if n.endswith("lso_adam.hip") else t)
    assert rs.kernel_hash(changed) != base
    retiled = _reader(lambda n, t: t.replace("#define LSO_TILE_ELEMS 8192u", "#define LSO_TILE_ELEMS 16384u")
                      if n.endswith("lso.h") else t)
    assert rs.kernel_hash(retiled) != base   # the header's tile size is kernel code too
    saved = list(build.FLAGS)
    try:
        build.FLAGS.append("-DSOMETHING")
        assert rs.kernel_hash() != base
    finally:
        build.FLAGS[:] = saved
    assert rs.kernel_hash() == base


def test_hash_does_not_depend_on_where_the_tree_is():
    """The build's include flags name the tree's absolute path; a copy of
    the tree at another path (as a run elsewhere sees it) has the same hash."""
    base = rs.kernel_hash()
    saved = list(build.FLAGS)
    saved_root = build.ROOT
    try:
        build.FLAGS[:] = [f.replace(saved_root, "/some/other/place/tree") for f in saved]
        build.ROOT = "/some/other/place/tree"
        assert rs.kernel_hash() == base
        build.FLAGS.append("-I/usr/include/elsewhere")   # outside the tree: counts as written
        assert rs.kernel_hash() != base
    finally:
        build.FLAGS[:] = saved
        build.ROOT = saved_root
    assert rs.kernel_hash() == base


def test_committed_kernel_profiles_are_of_the_current_code():
    current = rs.kernel_hash()
    seen = 0
    for path in glob.glob(os.path.join(ROOT, "profiles", "*.md")):
        for h in re.findall(r"kernel_source_sha256: ([0-9a-f]{16})", open(path, encoding="utf-8").read()):
            assert h == current, f"{os.path.basename(path)} was taken with kernel {h}, the code is {current}"
            seen += 1
    assert seen >= 8
