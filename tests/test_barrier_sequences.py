"""The two wave roles of the backward in-chunk kernel run in separate branches of one
kernel and meet only at workgroup barriers, so they must execute the same sequence of
barriers: a barrier that one role adds and the other does not would pair unrelated points
of the two roles (and the hardware gives no error for that).  This CPU test reads the
kernel source and derives, for each role function, the sequence of barriers it executes:
`lds_barrier()` (L) and `dma_barrier()` (D) in program order, with loops kept as
(header: body) groups and `if constexpr` branches resolved for each configuration of the
kernel (dstate 256 or not; B and C whole or in column slices).  The strip role must match the state role for dstate <= 128 and the dstate-256
state role for dstate 256.  A barrier under a run-time `if`, or in a helper called from a
role, is rejected: the check would not see whether both roles take it.
"""
import os
import re

import pytest

SRC = os.path.join(os.path.dirname(__file__), "..", "mamba_ssd_chunked_03_amd", "csrc",
                   "chunk_bwd_mfma.hip")


def _strip_comments(s):
    s = re.sub(r"/\*.*?\*/", " ", s, flags=re.S)
    return re.sub(r"//[^\n]*", " ", s)


def function_body(src, name):
    """Text between the braces of the definition `void name(...) { ... }`."""
    m = re.search(r"\bvoid\s+" + re.escape(name) + r"\s*\(", src)
    assert m, name
    depth = 1
    j = m.end()
    while depth:  # the parameter list
        if src[j] == "(":
            depth += 1
        elif src[j] == ")":
            depth -= 1
        j += 1
    j = src.index("{", j)
    depth, k = 1, j + 1
    while depth:
        if src[k] == "{":
            depth += 1
        elif src[k] == "}":
            depth -= 1
        k += 1
    return src[j + 1:k - 1]


_TOKEN = re.compile(
    r"(?P<lds>\blds_barrier\s*\(\s*\)\s*;)"
    r"|(?P<dma>\bdma_barrier\s*\(\s*\)\s*;)"
    r"|(?P<cexpr>\bif\s+constexpr\s*\()"
    r"|(?P<for>\bfor\s*\()"
    r"|(?P<if>\bif\s*\()"
    r"|(?P<else>\belse\b)"
    r"|(?P<open>\{)"
    r"|(?P<close>\})")


def _paren(s, i):
    """Index after the parenthesis group that starts just before i (s[i-1] == '(')."""
    depth = 1
    while depth:
        if s[i] == "(":
            depth += 1
        elif s[i] == ")":
            depth -= 1
        i += 1
    return i


def parse(body):
    """Nested list of 'L', 'D', ('for', header, [...]), ('cif', cond, [...], [...]) and
    ('if', cond, [...]) for the run-time ifs (kept to be checked for barriers)."""
    pos = 0
    root = []
    # stack of (list being filled, kind of the open brace)
    stack = [(root, "root")]
    while True:
        m = _TOKEN.search(body, pos)
        if not m:
            break
        kind = m.lastgroup
        pos = m.end()
        cur = stack[-1][0]
        if kind in ("lds", "dma"):
            cur.append("L" if kind == "lds" else "D")
            continue
        if kind in ("for", "cexpr", "if"):
            end = _paren(body, pos)
            head = re.sub(r"\s+", "", body[pos:end - 1])
            pos = end
            node = {"for": ("for", head, []), "cexpr": ("cif", head, [], []),
                    "if": ("if", head, [])}[kind]
            cur.append(node)
            nxt = re.match(r"\s*\{", body[pos:])
            if nxt:
                pos += nxt.end()
                stack.append((node[2], kind))
            else:  # a single statement: look for a barrier up to the next ';'
                semi = body.index(";", pos)
                stmt = body[pos:semi + 1]
                for b in re.findall(r"\b(lds|dma)_barrier\s*\(", stmt):
                    node[2].append("L" if b == "lds" else "D")
                pos = semi + 1
            continue
        if kind == "else":
            prev = cur[-1] if cur else None
            nxt = re.match(r"\s*\{", body[pos:])
            assert nxt, "else without braces"
            pos += nxt.end()
            if isinstance(prev, tuple) and prev[0] == "cif":
                stack.append((prev[3], "else"))
            else:
                holder = ("if", "else", [])
                cur.append(holder)
                stack.append((holder[2], "else"))
            continue
        if kind == "open":
            stack.append(([], "block"))
            cur.append(("block", stack[-1][0]))
            continue
        if kind == "close":
            stack.pop()
            continue
    assert len(stack) == 1, "unbalanced braces"
    return root


def has_barrier(nodes):
    for n in nodes:
        if n in ("L", "D"):
            return True
        if isinstance(n, tuple):
            for part in n[2:]:
                if isinstance(part, list) and has_barrier(part):
                    return True
            if n[0] == "block" and has_barrier(n[1]):
                return True
    return False


def sequence(nodes, flags):
    """The barrier sequence with `if constexpr` on the configuration flags (C_::EXT,
    C_::SLICED, or their negation) resolved by `flags`."""
    out = []
    for n in nodes:
        if n in ("L", "D"):
            out.append(n)
        elif n[0] == "block":
            out.extend(sequence(n[1], flags))
        elif n[0] == "for":
            inner = sequence(n[2], flags)
            if inner:
                out.append((n[1], tuple(inner)))
        elif n[0] == "cif":
            cond = n[1]
            neg = cond.startswith("!")
            if cond.lstrip("!") in flags:
                take = flags[cond.lstrip("!")] != neg
            else:
                assert not has_barrier(n[2]) and not has_barrier(n[3]), \
                    f"barrier under if constexpr ({cond})"
                continue
            out.extend(sequence(n[2] if take else n[3], flags))
        elif n[0] == "if":
            assert not has_barrier(n[2]), f"barrier under a run-time if ({n[1]})"
    return out


@pytest.fixture(scope="module")
def src():
    with open(SRC) as f:
        return _strip_comments(f.read())


def test_parser_sees_every_barrier(src):
    """Every barrier call in each role's text is in its parsed sequence (no construct the
    parser skips hides one)."""
    for name in ("bwd_strip_role", "bwd_state_role", "bwd_state_role_ext"):
        body = function_body(src, name)
        n_text = len(re.findall(r"\b(?:lds|dma)_barrier\s*\(", body))

        def count(nodes):
            c = 0
            for n in nodes:
                if n in ("L", "D"):
                    c += 1
                elif n[0] == "block":
                    c += count(n[1])
                else:
                    c += sum(count(p) for p in n[2:] if isinstance(p, list))
            return c

        assert count(parse(body)) == n_text, name


# (dstate 256, B / C in column slices for C B^T): every configuration the kernel has
CONFIGS = [(False, False), (False, True), (True, True)]


@pytest.mark.parametrize("ext,sliced", CONFIGS,
                         ids=["whole_bc", "sliced_bc", "dstate_256"])
def test_roles_run_the_same_barriers(src, ext, sliced):
    flags = {"C_::EXT": ext, "C_::SLICED": sliced}
    strip = sequence(parse(function_body(src, "bwd_strip_role")), flags)
    state_name = "bwd_state_role_ext" if ext else "bwd_state_role"
    state = sequence(parse(function_body(src, state_name)), flags)
    assert strip, "no barriers found"
    assert strip == state, f"\nstrip: {strip}\nstate: {state}"


def test_roles_call_no_barrier_helpers(src):
    """Barriers only appear in the role functions themselves and the kernels (no helper
    that a role calls issues one): the per-role count above would miss them."""
    barrier = re.compile(r"\b(?:lds|dma)_barrier\s*\(|__syncthreads|s_barrier")
    helpers = ("issue_item", "issue_bc", "issue_rows", "row_factors")
    for h in helpers:
        assert not barrier.search(function_body(src, h)), h
    # nor a lambda inside a role (its body is parsed where it is defined, not called)
    for name in ("bwd_strip_role", "bwd_state_role", "bwd_state_role_ext"):
        body = function_body(src, name)
        for m in re.finditer(r"\[[&=]?\]\s*\([^)]*\)\s*\{", body):
            depth, k = 1, m.end()
            while depth:
                depth += {"{": 1, "}": -1}.get(body[k], 0)
                k += 1
            assert not barrier.search(body[m.end():k]), name


def test_check_catches_a_mismatch(src):
    """The check itself: one barrier removed from the strip role's head loop is found."""
    body = function_body(src, "bwd_strip_role")
    i = body.index("lds_barrier();", body.index("for (int hh"))
    broken = body[:i] + body[i + len("lds_barrier();"):]
    flags = {"C_::EXT": False, "C_::SLICED": False}
    state = sequence(parse(function_body(src, "bwd_state_role")), flags)
    assert sequence(parse(broken), flags) != state
