"""The per-unit compiler flags of the build: every unit named in
build.SOURCE_FLAGS is a source the build compiles, it compiles a kernel file
of the package under a macro (and nothing else), and the kernel file splits
its instantiations between the two units by that macro, so no kernel and no
entry point is defined twice or left out."""

import os
import re

from exact_attention_69_amd import build


def read(name):
    return open(os.path.join(build.CSRC, name), encoding="utf-8").read()


def test_flagged_units_are_built_sources():
    names = {os.path.basename(s) for s in build.sources()}
    assert build.SOURCE_FLAGS, "no per-unit flags"
    for unit, flags in build.SOURCE_FLAGS.items():
        assert unit in names, f"{unit} is not compiled by the build"
        assert flags and all(isinstance(f, str) for f in flags)


def test_flagged_units_include_their_kernel_file_under_a_macro():
    for unit in build.SOURCE_FLAGS:
        code = [l for l in read(unit).splitlines() if l.strip() and not l.strip().startswith("//")]
        assert len(code) == 2, f"{unit}: expected a #define and an #include, got {code}"
        m_def = re.fullmatch(r"#define (\w+) 1", code[0].strip())
        m_inc = re.fullmatch(r'#include "(\w+\.hip)"', code[1].strip())
        assert m_def and m_inc, code
        macro, home = m_def.group(1), m_inc.group(1)
        src = read(home)
        # the home file switches on the macro in both directions: the unit's
        # launch function under #ifdef, the dispatch and entry points under
        # #ifndef / #else
        assert f"#ifdef {macro}" in src and f"#ifndef {macro}" in src, f"{home} does not split on {macro}"
        # the launch function the unit defines is declared for the other unit
        fn = re.search(rf"#ifdef {macro}\s*\nhipError_t (\w+)\(", src)
        assert fn, f"{home}: no launch function under #ifdef {macro}"
        assert f"{fn.group(1)}(" in read("launch.hpp"), f"{fn.group(1)} is not declared in launch.hpp"
        assert src.count(f"{fn.group(1)}(") >= 2, f"{home} never calls {fn.group(1)}"
