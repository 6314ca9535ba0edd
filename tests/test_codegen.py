"""Generated-code checks of the GEMM kernels (CPU only: hipcc emits gfx950
assembly without a GPU), for every (input type, output type, epilogue)
instantiation the library builds.

The K loop of the pipelined kernel (direct-to-LDS, for every operand type
and B layout) must keep its accumulators in the
accumulator register file and touch no scratch memory: accumulator moves or
spill reloads there cost up to half the kernel's rate (a reload is followed
by a wait for every outstanding load, which drains the load pipeline). Every
kernel (the register-staged ones too) must be free of the spill sequence that
reuses an accumulator register as a spill slot ("Reload Reuse"): in one
instantiation that sequence stored a lane value from the wrong register. And
every kernel's 16-byte C stores must take their offset straight from the
select that drops masked lanes.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from dense_tiled_gemm_tgemm_amd import build as hip_build

HIPCC = hip_build.HIPCC
pytestmark = pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="no hipcc")

# (input type, output type, epilogue): every combination tgemm_inst.hip is built for
CASES = [(ab, ct, epi) for ab in (0, 1, 2) for ct in (0, 1, 2) for epi in (0, 1)]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm")
    flags = [f for f in hip_build.FLAGS if f not in ("-fPIC", "-Wall", "-Wno-unused-function")]

    def one(case):
        ab, ct, epi = case
        path = os.path.join(out, f"inst_{ab}{ct}{epi}.s")
        cmd = [HIPCC, *flags, f"-DTG_AB={ab}", f"-DTG_CT={ct}", f"-DTG_EPI={epi}", "--cuda-device-only", "-S",
               os.path.join(hip_build.CSRC, "tgemm_inst.hip"), "-o", path]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        with open(path) as f:
            return case, f.read()

    with ThreadPoolExecutor(min(len(CASES), hip_build._jobs())) as ex:
        return dict(ex.map(one, CASES))


# kernel symbols: tgemm_dma_kernel (every operand type), tgemm_rs_kernel
# (16-bit operands, general), tgemm_f32in_rs_kernel (binary32 operands, general)
_PIPELINED = ("tgemm_dma_kernel",)
_ALL = _PIPELINED + ("tgemm_rs_kernel", "tgemm_f32in_rs_kernel")


def _kernels(text, families=_ALL):
    """(name, body lines) of every kernel of the given families in an assembly file."""
    for m in re.finditer(r"^(_ZN2tg\d+(tgemm_\w+?_kernel)I\w+):", text, re.M):
        if m.group(2) not in families:
            continue
        end = text.index(".Lfunc_end", m.end())
        yield m.group(1), text[m.end():end].splitlines()


def _innermost_mfma_loop(body):
    """Instructions of the blocks at the deepest loop level that holds MFMAs."""
    blocks, cur = [], ("", [])
    for line in body:
        t = line.strip()
        lab = re.match(r"^\.LBB\w+:(.*)", t)
        if lab:
            blocks.append(cur)
            cur = (lab.group(1), [])
        elif t and not t.startswith((";", ".")):
            cur[1].append(t)
    blocks.append(cur)

    def depth(comment):
        d = re.search(r"Depth=(\d+)", comment)
        return int(d.group(1)) if d else 0

    # a block of the K loop holds at least one slice: 16 MFMAs for the 64-row tiles
    mfma_depths = [depth(c) for c, ins in blocks if sum(i.startswith("v_mfma") for i in ins) >= 16]
    deepest = max(mfma_depths, default=0)
    assert deepest > 0, "no K loop found"
    return [i for c, ins in blocks if depth(c) == deepest for i in ins]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "ab%d_ct%d_epi%d" % c)
def test_k_loop_keeps_accumulators_in_place(asm, case):
    names = []
    for name, body in _kernels(asm[case], _PIPELINED):
        names.append(name)
        loop = _innermost_mfma_loop(body)
        moves = [i for i in loop if i.startswith(("v_accvgpr_write", "v_accvgpr_read", "v_accvgpr_mov"))]
        scratch = [i for i in loop if "scratch_" in i]
        assert not scratch, (name, scratch[:4])
        # a few writes for fragment bookkeeping are tolerated; a split
        # accumulator shows up as one move per accumulator register
        assert len(moves) <= 24, (name, len(moves), moves[:6])
    assert len(names) >= (10 if case[0] == 2 else 4), names


@pytest.mark.parametrize("case", CASES, ids=lambda c: "ab%d_ct%d_epi%d" % c)
def test_every_kernel_family_is_checked(asm, case):
    """The symbol pattern finds both kernel families of the instantiation (a
    renamed kernel would otherwise drop out of the checks unnoticed)."""
    fams = {re.match(r"_ZN2tg\d+(tgemm_\w+?_kernel)", n).group(1) for n, _ in _kernels(asm[case])}
    want = {"tgemm_dma_kernel", "tgemm_f32in_rs_kernel"} if case[0] == 2 else {"tgemm_dma_kernel", "tgemm_rs_kernel"}
    assert fams == want, fams


@pytest.mark.parametrize("case", CASES, ids=lambda c: "ab%d_ct%d_epi%d" % c)
def test_no_accumulator_spill_slot_reuse(asm, case):
    for name, body in _kernels(asm[case]):
        bad = [l.strip() for l in body if "Reload Reuse" in l]
        assert not bad, (name, bad[:4])


def _unguarded_c_stores(ins):
    """(count of 16-byte buffer stores, those whose offset does not come
    straight from a select against 0x80000000) in a list of instructions.
    The C stores are the only buffer stores of these kernels; each store site
    exists twice, streamed (nt sc1) and with the default policy."""
    oob = {m.group(1) for l in ins for m in [re.match(r"v_bfrev_b32_e32 (v\d+), 1$", l)] if m}
    n, bad = 0, []
    for i, l in enumerate(ins):
        if not l.startswith("buffer_store_dwordx4"):
            continue
        n += 1
        m = re.match(r"buffer_store_dwordx4 v\[\d+:\d+\], (v\d+), s\[\d+:\d+\], 0 offen( nt sc1)?$", l)
        if not m:
            bad.append(l)
            continue
        j = i - 1
        while j >= 0 and not re.match(r"\S+ %s," % m.group(1), ins[j]):
            j -= 1
        d = ins[j] if j >= 0 else ""
        if not (d.startswith("v_cndmask_b32") and (any(r in d.split(", ")[1:] for r in oob) or "0x80000000" in d)):
            bad.append(l)
    return n, bad


def test_unguarded_store_check_catches_planted_mistakes():
    """The check below on hand-made instruction lists: a guarded store passes;
    an immediate offset, or an offset register that is not the select's
    result, is reported."""
    good = ["v_bfrev_b32_e32 v9, 1", "v_cndmask_b32_e64 v6, v9, v6, s[18:19]",
            "buffer_store_dwordx4 v[10:13], v6, s[60:63], 0 offen nt sc1"]
    assert _unguarded_c_stores(good) == (1, [])
    imm = good[:2] + ["buffer_store_dwordx4 v[10:13], v6, s[60:63], 0 offen offset:64 nt sc1"]
    assert len(_unguarded_c_stores(imm)[1]) == 1
    plain = ["v_bfrev_b32_e32 v9, 1", "v_add_u32_e32 v6, 64, v7",
             "buffer_store_dwordx4 v[10:13], v6, s[60:63], 0 offen nt sc1"]
    assert len(_unguarded_c_stores(plain)[1]) == 1


@pytest.mark.parametrize("case", CASES, ids=lambda c: "ab%d_ct%d_epi%d" % c)
def test_c_store_offsets_drop_masked_lanes(asm, case):
    """The 16-byte C stores are predicated by offset, not by branch: a lane
    that must not store presents 0x80000000, beyond the C resource's record
    count, and the hardware drops the store. Every such store's offset must
    therefore come straight from a select against that value, with no constant
    folded into the instruction's immediate offset (which would move a dropped
    lane's offset back into range)."""
    n = 0
    for name, body in _kernels(asm[case]):
        ins = [l.strip() for l in body if l.strip() and not l.strip().startswith((";", "."))]
        k, bad = _unguarded_c_stores(ins)
        assert not bad, (name, bad[:3])
        streamed = sum(1 for l in ins if l.startswith("buffer_store_dwordx4") and l.endswith("nt sc1"))
        pol = _store_policy(name)
        if pol is None:
            # the policy follows C's alignment at run time: both forms of every store
            assert 2 * streamed == k, (name, streamed, k)
        else:
            # built for one policy (the persistent 64-deep kernel): that form only
            assert k > 0 and streamed == (k if pol == 1 else 0), (name, streamed, k)
        n += k
    assert n >= 64, n


def _store_policy(name):
    """The C store policy a direct-to-LDS kernel was built for (its last
    template argument: 1 streamed, 0 default), or None where it is chosen at
    run time (-1, mangled n1) and for the other kernel families."""
    m = re.match(r"_ZN2tg16tgemm_dma_kernelI\w*?Lb[01]ELi(n1|0|1)EEEvNS_4ArgsE$", name)
    if not m or m.group(1) == "n1":
        return None
    return int(m.group(1))


def test_store_policy_parse():
    assert _store_policy("_ZN2tg16tgemm_dma_kernelILi0ELi1ELi64ELi2ELi8ELb0ELi1EEEvNS_4ArgsE") == 1
    assert _store_policy("_ZN2tg16tgemm_dma_kernelILi0ELi1ELi64ELi2ELi8ELb0ELi0EEEvNS_4ArgsE") == 0
    assert _store_policy("_ZN2tg16tgemm_dma_kernelILi0ELi1ELi32ELi3ELi4ELb1ELin1EEEvNS_4ArgsE") is None
    assert _store_policy("_ZN2tg15tgemm_rs_kernelILi0ELi0ELb1EEEvNS_4ArgsE") is None
