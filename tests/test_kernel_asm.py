"""Properties of the compiled kernels that their speed depends on, checked on the
compiler's gfx950 assembly (CPU only: hipcc cross-compiles, nothing runs).

- No tile loop of an instance that runs at scale reloads a spilled register: a reload
  is a vector-memory load, and it would wait behind every tile copy in flight.
- Inside a plain tile loop, the only vector-memory waits are the ones right before the
  end-of-step barrier (the copies' own wait): a wait elsewhere would make the step
  wait for the prefetch it just issued. (The exact-path bodies, which split P and dS
  into two bf16 parts for rows that see at most 128 keys, spill and are exempt.)
- M0 is written only by the tile copies (its value is not known to the compiler).
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "flashattention_tiled_attention_amd", "csrc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# kernels (mangled-name fragments) whose tile loops must be clean: every instance the
# benchmarked workloads launch
HOT = {
    "attn_fwd.hip": ["fwd_kernelILi128ELi128ELb1E", "fwd_kernelILi64ELi64ELb0E", "fwd_kernelILi64ELi64ELb1E",
                     "fwd_kernelILi128ELi64ELb1E", "fwd_win_kernelILi128ELi128E"],
    "attn_bwd.hip": ["dq_kernelILi128ELi128ELb1E", "dq_kernelILi128ELi128ELb0E", "dkv_kernelILi128ELi128ELb1E",
                     "dkv_kernelILi128ELi128ELb0E", "dq_kernelILi64ELi64ELb0E", "dkv1_kernelILi64ELi64ELb0E",
                     "dq_kernelILi128ELi64ELb1E", "dkv_kernelILi128ELi64ELb1E", "dq_win_kernelILi128ELi128E"],
    "attn_sparse.hip": ["sparse_fwd_kernelILi128E", "sparse_dq_kernelILi128E"],
}


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = {}
    d = tmp_path_factory.mktemp("asm")
    for src in HOT:
        s = str(d / (src + ".s"))
        subprocess.run([HIPCC] + FLAGS + ["-o", s, os.path.join(CSRC, src)], check=True, capture_output=True)
        out[src] = open(s).read().split("\n")
    return out


def functions(lines):
    """(name, body lines) of every kernel in an assembly listing."""
    res = []
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\w+):", l)
        if m and "kernel" in m.group(1):
            end = next(j for j in range(i, len(lines)) if lines[j].startswith(".Lfunc_end"))
            res.append((m.group(1), lines[i:end]))
    return res


def loops_of(body):
    """Line ranges of every loop: a backward branch to a label above it whose
    target block reaches the branch again. (The compiler also places one-way
    blocks below the code they jump back into; those close no cycle.)"""
    labels = {}
    starts = [0]
    for k, l in enumerate(body):
        m = re.match(r"^(\.LBB\d+_\d+):", l)
        if m:
            labels[m.group(1)] = k
        if m or re.match(r"^; %bb\.\d+:", l):
            starts.append(k)
    starts = sorted(set(starts))
    block_of = {}
    for n, s in enumerate(starts):
        end = starts[n + 1] if n + 1 < len(starts) else len(body)
        for k in range(s, end):
            block_of[k] = n
    succ = {n: set() for n in range(len(starts))}
    branches = []
    for n, s in enumerate(starts):
        end = starts[n + 1] if n + 1 < len(starts) else len(body)
        falls = True
        for k in range(s, end):
            m = re.search(r"(s_cbranch_\w+|s_branch)\s+(\.LBB\d+_\d+)", body[k])
            if m and m.group(2) in labels:
                succ[n].add(block_of[labels[m.group(2)]])
                branches.append((k, m.group(2)))
                if m.group(1) == "s_branch":
                    falls = False
            if re.search(r"\bs_endpgm\b|\bs_setpc_b64\b", body[k]):
                falls = False
        if falls and n + 1 < len(starts):
            succ[n].add(n + 1)

    def reaches(a, b):
        seen, todo = set(), [a]
        while todo:
            x = todo.pop()
            if x == b:
                return True
            if x not in seen:
                seen.add(x)
                todo.extend(succ[x])
        return False

    loops = set()
    for k, t in branches:
        if labels[t] < k and reaches(block_of[labels[t]], block_of[k]):
            loops.add((labels[t], k))
    return sorted(loops)


def tile_loops(body):
    """For every MFMA, the smallest loop that contains it: the tile loops."""
    loops = loops_of(body)
    found = set()
    for k, l in enumerate(body):
        if "v_mfma" in l:
            inside = [(a, b) for a, b in loops if a <= k <= b]
            if inside:
                found.add(min(inside, key=lambda ab: ab[1] - ab[0]))
    return sorted(found)


PLAIN_MFMAS = {"fwd": 32, "dq_": 48, "dkv": 10 ** 9}  # MFMAs of a plain tile-loop body


def plain_limit(name):
    return next(v for key, v in PLAIN_MFMAS.items() if key in name)


def dims(name):
    """(D, Dv) of an instance from its mangled template arguments."""
    m = re.search(r"ILi(\d+)ELi(\d+)E", name)
    return int(m.group(1)), int(m.group(2))


def is_plain_loop(name, mfmas, seg=()):
    """Whether a tile loop with this many MFMAs (and these lines) belongs to a plain
    (not exact-path) body. The dQ kernels' plain loop runs one or two key tiles per
    iteration, each with D/16 + Dv/16 score and dP MFMAs and 2 D/32 dQ MFMAs per
    32-key half; their exact bodies have a pass without the dQ MFMAs and one with
    twice as many, so the counts never coincide. The dK/dV kernels' exact loop is the
    one that reads the dQ stage's per-tile flag with a scalar load."""
    if "dkv" in name:
        return not any(x.strip().startswith("s_load") for x in seg)
    if "dq_" in name and "sparse" not in name:
        D, Dv = dims(name)
        per_tile = 2 * (D // 16 + Dv // 16 + 2 * (D // 32))
        return mfmas in (per_tile, 2 * per_tile)
    return mfmas <= plain_limit(name)


def hot_functions(asm):
    for src, frags in HOT.items():
        for name, body in functions(asm[src]):
            if any(f in name for f in frags):
                yield name, body


def test_hot_instances_found(asm):
    names = [n for n, _ in hot_functions(asm)]
    assert len(names) == sum(len(v) for v in HOT.values()), names


def test_no_spill_reload_in_tile_loops(asm):
    for name, body in hot_functions(asm):
        loops = tile_loops(body)
        assert loops, name
        for a, b in loops:
            # exact-path bodies (split P / dS operands) are allowed their spills: they
            # run on the few rows that see at most 128 keys
            mfmas = sum("v_mfma" in body[k] for k in range(a, b + 1))
            reloads = [body[k].strip() for k in range(a, b + 1) if "scratch_load" in body[k]]
            assert not reloads or not is_plain_loop(name, mfmas, body[a:b + 1]), \
                "%s: spill reload in a plain tile loop (%d MFMAs): %s" % (name, mfmas, reloads[:3])


def test_vmcnt_waits_only_before_barriers(asm):
    for name, body in hot_functions(asm):
        all_loops = loops_of(body)
        mfmas = lambda a, b: sum("v_mfma" in body[k] for k in range(a, b + 1))
        for a, b in tile_loops(body):
            parents = [(c, d) for c, d in all_loops if c <= a and d >= b and (c, d) != (a, b)]
            parent = min(parents, key=lambda cd: cd[1] - cd[0]) if parents else None
            if not is_plain_loop(name, mfmas(a, b), body[a:b + 1]) or \
                    (parent and not is_plain_loop(name, mfmas(*parent), body[parent[0]:parent[1] + 1])):
                continue  # an exact-path body (split operands; its spills are allowed)
            for k in range(a, b + 1):
                m = re.search(r"s_waitcnt.*vmcnt\((\d+)\)", body[k])
                if not m:
                    continue
                if int(m.group(1)) > 0:
                    # a wait by count (the dK/dV stage ring: later copies stay in
                    # flight); only a full wait could stall on the prefetch
                    continue
                nxt = [body[j].strip() for j in range(k + 1, min(k + 12, len(body)))
                       if body[j].strip() and not body[j].strip().startswith(";")]
                ok = any(x.startswith("s_barrier") for x in nxt[:3]) or \
                    any(x.startswith(("ds_write", "v_mul_f32", "v_xor_b32")) for x in nxt[:3])  # row statistics
                assert ok, "%s: vector-memory wait inside a tile loop not before a barrier: %s -> %s" % (
                    name, body[k].strip(), nxt[:3])


def test_m0_written_only_by_tile_copies(asm):
    for src, lines in asm.items():
        for k, l in enumerate(lines):
            if re.search(r"\bm0\b", l) and not l.strip().startswith(";"):
                # the copy's own M0 write; its source is whichever scalar register the
                # compiler gave the asm operand (vcc_lo included)
                assert re.match(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)$", l.strip()), \
                    "%s: unexpected M0 use: %s" % (src, l.strip())
                nxt = [x.strip() for x in lines[k + 1:k + 3]]
                assert nxt[0] == "s_nop 0" and nxt[1].startswith(("global_load_lds_dwordx4", "global_load_lds_dword ")), \
                    (src, nxt)


def test_scalar_copy_bases_are_not_sign_extended(asm):
    """The saddr tile copies take a 64-bit base rebuilt from two readfirstlane halves.
    readfirstlane returns a signed int, and a low half widened as signed would fill the
    high half with ones for any address with bit 31 set: the compiler then emits
    s_bfe_i64 to build the base. None of the attention kernels needs a signed 64-bit
    field extract, so its absence pins the unsigned widening."""
    found = 0
    for src, lines in asm.items():
        for l in lines:
            t = l.strip()
            if re.match(r"global_load_lds_dwordx4 v\d+, s\[\d+:\d+\]", t):
                found += 1
            assert not t.startswith("s_bfe_i64"), "%s: sign-extending field extract: %s" % (src, t)
    assert found > 0, "no saddr tile copies found"
