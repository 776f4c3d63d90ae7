"""Mutation sweep of the oracle's C source against the CPU oracle pins.

Not collected by pytest (about ten minutes with six workers). Every site of
oracle/hisparse_oracle.c outside comments gets each applicable mutation on its
own: a relational operator flipped (< <=, > >=, == !=), && and || swapped,
+ 1 and - 1 swapped, ++ turned into --, a binary + into - and * into +, a 0
into 1 and a -1 into 0, a statement or a one-line if deleted. Each mutant is
built with gcc and the oracle pin files run against it in a child process;
a mutant survives if every pin passes. The survivors that no input can tell
apart from the real oracle are listed in EQUIVALENT with the reason; any
other survivor makes the script exit with status 1.

    python3 tests/mutation_sweep.py [--workers 6]
"""

import argparse
import json
import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "hisparse_oracle.c")
PINS = ["tests/test_oracle_closed_forms.py", "tests/test_oracle_copies_and_errors.py",
        "tests/test_oracle_golden.py", "tests/test_oracle_kv.py", "tests/test_oracle_model.py",
        "tests/test_oracle_paged.py", "tests/test_oracle_plan.py", "tests/test_oracle_traces.py",
        "tests/test_oracle_contract.py"]

OPS = [(r"(?<![<>=!])<(?![<=])", "<="), (r"<=", "<"), (r"(?<![-<>=])>(?![>=])", ">="), (r">=", ">"),
       (r"==", "!="), (r"!=", "=="), (r"&&", "||"), (r"\|\|", "&&"), (r"\+ 1\b", "- 1"),
       (r"- 1\b", "+ 1"), (r"\+\+", "--"), (r"(?<=[\w\)\]]) \+ (?=[\w\(])", " - "),
       (r"(?<=[\w\)\]]) \* (?=[\w\(])", " + "), (r"\b0\b", "1"), (r"-1\b", "0")]

# (source line, stripped; mutation) -> why no input tells the mutant apart
EQUIVALENT = {
    ("return (a->index > b->index) - (a->index < b->index);", "<-><="):
        "top-k indices are distinct: the comparator never sees equal keys",
    ("return (a->index > b->index) - (a->index < b->index);", ">->>="):
        "top-k indices are distinct: the comparator never sees equal keys",
    ("if (!a || a->B < 0 || a->K < 0 || a->H < 0 || a->R < 0) return ORACLE_EARG;", "||->&&@2"):
        "a negative K alone still fails: the per-call buffers cannot be allocated",
    ("if (!p->hot_block_table || p->hot_block_size <= 0 || p->hot_table_stride * p->hot_block_size < a->H)", "<=-><"):
        "a hot block size of 0 gives a table of 0 slots, below H",
    ("if (p->resident_block_table && (p->resident_block_size <= 0 || p->resident_num_blocks < 0))", "<=-><"):
        "a resident block size of 0 differs from the hot block size, rejected next",
    ("if (!seen) return ORACLE_EARG;", "delete"): "allocation failure",
    ("if (!seen) return ORACLE_EARG;", "delete-if"): "allocation failure",
    ("free(seen);", "delete"): "a leak",
    ("const int32_t nreal = (a->num_real >= 0 && a->num_real < B) ? a->num_real : B;", "<-><="):
        "num_real == B gives B either way",
    ("int16_t *hits = (int16_t *)malloc(sizeof(int16_t) * (size_t)H);", "*->+"):
        "an undersized buffer: memory safety, seen only by a sanitizer",
    ("if (!pending || !hits || !evict || !new_lru) {", "||->&&@0"): "allocation failure",
    ("if (!pending || !hits || !evict || !new_lru) {", "||->&&@1"): "allocation failure",
    ("if (!pending || !hits || !evict || !new_lru) {", "||->&&@2"): "allocation failure",
    ("free(pending); free(hits); free(evict); free(new_lru);", "delete"): "a leak",
    ("const int64_t L = a->paged ? 0 : a->seq_lens[b];", "0->1"):
        "L is not read under paged addressing",
    ("continue;", "delete"): "the paged branch's fall-through writes -1, which the miss pass overwrites",
    ("pending_t key = {tok, 0, 0};", "0->1@0"): "the search compares tokens only",
    ("pending_t key = {tok, 0, 0};", "0->1@1"): "the search compares tokens only",
    ("if (n < 0) n = 0;", "<-><="): "a count of 0 or below copies nothing either way",
    ("if (n < 0) n = 0;", "0->1"): "a count of 0 or below copies nothing either way",
    ("if (n < 0) n = 0;", "delete"): "a count of 0 or below copies nothing either way",
    ("if (n > K) n = K;", ">->>="): "a count of K is clamped to K",
}


def _code(line):
    for mark in ("/*", "//"):
        i = line.find(mark)
        if i >= 0:
            line = line[:i]
    return line


def mutants(lines):
    """(line index, label, new line) for every mutation site."""
    out = []
    in_comment = False
    for n, ln in enumerate(lines):
        s = ln.strip()
        if in_comment:
            in_comment = "*/" not in s
            continue
        if s.startswith("/*") and "*/" not in s:
            in_comment = True
            continue
        if not s or s[0] in "#*" or s.startswith("/*") or s.startswith("//"):
            continue
        code = _code(ln)
        for pat, rep in OPS:
            sym = {"(?<![<>=!])<(?![<=])": "<", "(?<![-<>=])>(?![>=])": ">", r"\|\|": "||",
                   r"\+ 1\b": "+1", r"- 1\b": "-1", r"\+\+": "++", r"\b0\b": "0", r"-1\b": "-1",
                   r"(?<=[\w\)\]]) \+ (?=[\w\(])": "+", r"(?<=[\w\)\]]) \* (?=[\w\(])": "*"}.get(pat, pat)
            for k, m in enumerate(re.finditer(pat, code)):
                label = f"{sym}->{rep.strip()}@{k}"
                out.append((n, label, code[:m.start()] + rep + code[m.end():] + ln[len(code):]))
        if code.rstrip().endswith(";") and not re.match(
                r"\s*(return|int|const|char|int16_t|int32_t|int64_t|pending_t|uint|size_t|static|typedef|\}|break)", code):
            out.append((n, "delete", ""))
        if re.match(r"\s*if \(.*\) (continue|return [^;]+|\{ .* \});\s*$", code):
            out.append((n, "delete-if", ""))
    return out


def equivalent(line, label):
    key = line.strip()
    for (src, lab), why in EQUIVALENT.items():
        if src == key and (label == lab or (("@" not in lab) and label.split("@")[0] == lab)):
            return why
    return None


def run_one(lines, m):
    n, label, new = m
    mutated = list(lines)
    mutated[n] = new
    d = tempfile.mkdtemp()
    try:
        c = os.path.join(d, "m.c")
        with open(c, "w") as f:
            f.write("\n".join(mutated))
        lib = os.path.join(d, "libm.so")
        if subprocess.run(["gcc", "-std=c11", "-O1", "-w", "-fPIC", "-shared", "-I",
                           os.path.dirname(SRC), "-o", lib, c], capture_output=True).returncode:
            return "nocompile"
        code = (f"import sys; sys.path[:0] = [{ROOT!r}, {os.path.join(ROOT, 'tests')!r}]; "
                f"import oracle; oracle.use_library({lib!r}); import pytest; "
                f"sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider'] + {PINS!r}))")
        try:
            r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, timeout=300)
        except subprocess.TimeoutExpired:
            return "killed"      # a mutant that loops forever is caught too
        return "killed" if r.returncode else "survived"
    finally:
        subprocess.run(["rm", "-rf", d])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workers", type=int, default=6)
    args = ap.parse_args()
    lines = open(SRC).read().split("\n")
    ms = mutants(lines)
    with ThreadPoolExecutor(args.workers) as ex:
        res = list(ex.map(lambda m: run_one(lines, m), ms))
    counts = {}
    unexpected = []
    for m, r in zip(ms, res):
        counts[r] = counts.get(r, 0) + 1
        if r == "survived":
            why = equivalent(lines[m[0]], m[1])
            print(f"{'equivalent' if why else 'SURVIVED':10s} line {m[0] + 1} {m[1]}: {lines[m[0]].strip()}"
                  + (f"  ({why})" if why else ""))
            if not why:
                unexpected.append(m)
    print(json.dumps({"mutants": len(ms), **counts, "unexpected": len(unexpected)}))
    sys.exit(1 if unexpected else 0)


if __name__ == "__main__":
    main()
