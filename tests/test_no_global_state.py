"""The library keeps no mutable global state (CPU only: reads the sources).

The C ABI promises that every entry point is thread-safe and that the library
keeps no mutable state between calls.  This test parses the HIP sources and
fails on any object with static storage that is not constant:

* a ``static`` variable inside a function or a struct body;
* a namespace-scope variable that is neither ``constexpr`` nor ``const``.

The deliberate exceptions belong to the allocation-free backward entry point
(documented in the header next to it): its workspace, a device array named
``scratch`` (declared ``__device__``), and ``scratch_addr``, the atomic
per-device record of that array's device address, written once per device.
"""
import glob
import os
import re

import pytest

from vision_transformer_local_amd import build as B

ALLOWED_DEVICE_ARRAYS = {"scratch"}
ALLOWED_ATOMIC_TABLES = {"scratch_addr"}


def _strip(src):
    """Source without comments, string and character literals, or directives."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            i = src.find("\n", i)
            i = n if i < 0 else i
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(c + c)
            i = j + 1
        elif c == "#" and (i == 0 or src[i - 1] == "\n"):
            while True:  # directive, with line continuations
                j = src.find("\n", i)
                if j < 0:
                    i = n
                    break
                if src[j - 1] != "\\":
                    i = j
                    break
                i = j + 1
        else:
            out.append(c)
            i += 1
    return "".join(out)


def _statements(code):
    """(text, terminator, at_namespace_scope) for every ';'- or '{'-ended piece."""
    stack, buf = [], []
    for c in code:
        if c in ";{}":
            text = " ".join("".join(buf).split())
            buf = []
            ns_scope = all(k == "ns" for k in stack)
            if c == "{":
                kind = "ns" if re.match(r"^(inline\s+)?namespace\b|^extern\s+\S+$", text) else "other"
                yield text, c, ns_scope
                stack.append(kind)
            elif c == "}":
                if stack:
                    stack.pop()
            else:
                yield text, c, ns_scope
        else:
            buf.append(c)


SKIP_HEAD = re.compile(r"^(typedef|using|template|struct|class|enum|union|namespace|extern|"
                       r"static_assert|return|friend|public|private|protected)\b")


def _violations(path):
    code = _strip(open(path).read())
    bad = []
    for text, term, ns_scope in _statements(code):
        if term != ";" or not text:
            continue
        decl = text.split("=", 1)[0]
        if "(" in decl and not re.search(r"\]\s*$", decl):
            continue  # a function declaration (or a call statement)
        words = decl.replace("*", " * ").split()
        if ns_scope:
            if SKIP_HEAD.match(text) or not re.match(r"^[A-Za-z_]", text):
                continue
            if "constexpr" in words or "const" in words or "__constant__" in words:
                continue
            name = re.findall(r"(\w+)\s*(?:\[[^\]]*\])*\s*$", decl)
            if "__device__" in words and name and name[0] in ALLOWED_DEVICE_ARRAYS:
                continue
            if (name and name[0] in ALLOWED_ATOMIC_TABLES
                    and re.match(r"^std::atomic<", text)):
                continue
            bad.append(text)
        elif text.startswith("static ") or " static " in (" " + text):
            if re.match(r"^static\s+(constexpr|const)\b", text) or text.startswith("static_assert"):
                continue
            bad.append(text)
    return bad


SOURCES = sorted(glob.glob(os.path.join(B.CSRC, "*.hip")) + glob.glob(os.path.join(B.CSRC, "*.h")))


@pytest.mark.parametrize("path", SOURCES, ids=os.path.basename)
def test_no_mutable_static_objects(path):
    assert _violations(path) == []


def test_detector_flags_mutable_statics(tmp_path):
    """The parser finds what the test is for (a function-scope cache, a
    namespace-scope counter) and lets constants, functions and the scratch
    array through."""
    src = tmp_path / "x.hip"
    src.write_text(
        "namespace na2d {\n"
        "constexpr int kA = 3;\n"
        "const float kB[2] = {1.f, 2.f};\n"
        "int counter = 0;\n"
        "static __device__ __align__(256) char scratch[1024];\n"
        "__device__ int other[4];\n"
        "hipError_t launch(int a, int b);\n"
        "struct S { static constexpr int N = 2; static void run(int x); int y; };\n"
        "int device_cus() {\n"
        "  static int cache[64];  // lazily filled\n"
        "  static const int fixed = 3;\n"
        "  int local = 2;\n"
        "  return cache[0] + local + fixed;\n"
        "}\n"
        "}  // namespace na2d\n")
    bad = _violations(str(src))
    assert bad == ["int counter = 0", "__device__ int other[4]", "static int cache[64]"]
