"""Irreps strings, path enumeration and the output-slot rule (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages build the operation from irreps specifications ("The GPU memory
optimization with Larger angular momentum" discussion, the answer about
modifying the irreps of the README example) and draw the CG tensor as one
block per coupling path (sciencestack.ai page, Figures 1-2).  They fix no
grammar, layout or slot rule; the readings adopted here are:

* grammar   ``MULxLP`` terms joined by ``+`` (whitespace ignored), MUL >= 1,
            0 <= L <= 7, P in {e, o};
* layout    blocks concatenated in string order; inside a block the element
            (channel u, component m) sits at ``offset + u*(2L+1) + (m+L)``;
* paths     i1 over the input irreps, i2 over the SH irreps, then l3 from
            |l1-l2| to l1+l2 ascending with parity p1*p2; a path exists only if
            (l3, p3) occurs in the output irreps;
* slots     if (l3, p3) occurs once in the output, every path producing it
            sums into that block; if it occurs k > 1 times, exactly k paths
            must produce it and the j-th path writes the j-th occurrence;
            anything else is an error;
* weights   uvu: per row/edge the concatenation over paths of ``[mul]``;
            uvw: the concatenation over paths of ``[mul_in][mul_out]``.
"""
from dataclasses import dataclass, field
from typing import List, Tuple

LMAX = 7


class IrrepsError(ValueError):
    pass


@dataclass(frozen=True)
class Irrep:
    mul: int
    l: int
    p: int  # +1 for 'e', -1 for 'o'

    @property
    def dim(self) -> int:
        return self.mul * (2 * self.l + 1)


def parse_irreps(text: str) -> List[Irrep]:
    """Parse ``"32x0e+32x1o"`` into a list of Irrep, in string order."""
    s = "".join(str(text).split())
    if not s:
        raise IrrepsError("empty irreps string")
    out = []
    for term in s.split("+"):
        if "x" not in term:
            raise IrrepsError(f"term {term!r} lacks 'MULx'")
        mul_s, lp = term.split("x", 1)
        if not mul_s.isdigit() or len(lp) < 2 or not lp[:-1].isdigit() or lp[-1] not in "eo":
            raise IrrepsError(f"bad irreps term {term!r}")
        mul, l = int(mul_s), int(lp[:-1])
        if mul < 1:
            raise IrrepsError(f"multiplicity must be >= 1 in {term!r}")
        if l > LMAX:
            raise IrrepsError(f"l={l} exceeds {LMAX} in {term!r}")
        out.append(Irrep(mul, l, 1 if lp[-1] == "e" else -1))
    return out


def offsets(irreps: List[Irrep]) -> List[int]:
    offs, acc = [], 0
    for ir in irreps:
        offs.append(acc)
        acc += ir.dim
    return offs


def total_dim(irreps: List[Irrep]) -> int:
    return sum(ir.dim for ir in irreps)


@dataclass
class Path:
    i1: int
    i2: int
    l1: int
    l2: int
    l3: int
    p3: int
    slot: int = -1
    w_off: int = 0  # offset of this path's weights inside one weight row / the shared block


@dataclass
class Problem:
    ins: List[Irrep]
    sh: List[Irrep]
    out: List[Irrep]
    mode: str
    paths: List[Path] = field(default_factory=list)

    @property
    def d_in(self):
        return total_dim(self.ins)

    @property
    def d_sh(self):
        return total_dim(self.sh)

    @property
    def d_out(self):
        return total_dim(self.out)

    @property
    def weight_numel(self):
        """uvu: weights per row/edge.  uvw: total shared weights."""
        if self.mode == "uvu":
            return sum(self.ins[p.i1].mul for p in self.paths)
        return sum(self.ins[p.i1].mul * self.out[p.slot].mul for p in self.paths)


def build_problem(in_irreps: str, sh_irreps: str, out_irreps: str, mode: str) -> Problem:
    """Enumerate the coupling paths and assign each one its output block."""
    if mode not in ("uvu", "uvw"):
        raise IrrepsError(f"mode must be 'uvu' or 'uvw', got {mode!r}")
    ins, sh, out = parse_irreps(in_irreps), parse_irreps(sh_irreps), parse_irreps(out_irreps)
    for ir in sh:
        if ir.mul != 1:
            raise IrrepsError("every SH irrep must have multiplicity 1")
    out_keys = [(o.l, o.p) for o in out]
    paths = []
    for i1, a in enumerate(ins):
        for i2, b in enumerate(sh):
            for l3 in range(abs(a.l - b.l), a.l + b.l + 1):
                p3 = a.p * b.p
                if (l3, p3) in out_keys:
                    paths.append(Path(i1, i2, a.l, b.l, l3, p3))
    # slot rule
    for key in set(out_keys):
        occ = [q for q, k in enumerate(out_keys) if k == key]
        prod = [p for p in paths if (p.l3, p.p3) == key]
        if not prod:
            raise IrrepsError(f"output irrep l={key[0]} p={key[1]} is produced by no path")
        if len(occ) == 1:
            for p in prod:
                p.slot = occ[0]
        elif len(occ) == len(prod):
            for p, q in zip(prod, occ):
                p.slot = q
        else:
            raise IrrepsError(
                f"output irrep l={key[0]} p={key[1]} occurs {len(occ)} times but {len(prod)} paths produce it")
    w = 0
    for p in paths:
        p.w_off = w
        if mode == "uvu":
            if out[p.slot].mul != ins[p.i1].mul:
                raise IrrepsError("uvu needs mul_out == mul_in on every path")
            w += ins[p.i1].mul
        else:
            w += ins[p.i1].mul * out[p.slot].mul
    return Problem(ins, sh, out, mode, paths)


def sh_irreps(lmax: int) -> str:
    """``1x0e+1x1o+...`` up to lmax, natural parity (-1)^l."""
    return "+".join(f"1x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(lmax + 1))


def per_path_out_irreps(in_irreps: str, lmax_sh: int, lmax_out: int, both_parities: bool = True) -> str:
    """Output string with one block per path (canonical order), l3 <= lmax_out.

    This is how the conv workloads ask for "every allowed path" as its own
    output block.
    """
    ins = parse_irreps(in_irreps)
    terms = []
    for a in ins:
        for l2 in range(lmax_sh + 1):
            p2 = 1 if l2 % 2 == 0 else -1
            for l3 in range(abs(a.l - l2), min(a.l + l2, lmax_out) + 1):
                p3 = a.p * p2
                if not both_parities and p3 != (1 if l3 % 2 == 0 else -1):
                    continue
                terms.append(f"{a.mul}x{l3}{'e' if p3 == 1 else 'o'}")
    return "+".join(terms)
