"""Register budget of every HIP kernel, checked on the CPU.

Each source is compiled for gfx950 with the library's own flags to AMD
assembly, and the code-object metadata of every kernel is read back: no vector
register may spill, no kernel may use scratch (private) memory, and scalar
registers may spill into vector-register lanes only where listed below.  A
spill that appears with a new template instance or a code change shows up
here instead of as a slowdown on the GPU.
"""
import concurrent.futures as cf
import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = ["taylor_decode.hip", "taylor_prefill.hip", "taylor_prefill_n3.hip", "taylor_prefill_n3_c128.hip",
           "taylor_prefill_fb.hip", "taylor_prefill_small.hip", "softmax_attn.hip", "taylor_decode_bf16.hip",
           "taylor_hybrid.hip"]

# Scalar spills allowed per kernel (mangled-name prefix -> count): none.  (The
# 128-token n = 3 prefill once kept up to 8 scalar registers in vector-register
# lanes; a form of its causal mask that needed 25 cost the long prefill 7%.)
SGPR_SPILL_ALLOWANCE = {}


def _build_module():
    spec = importlib.util.spec_from_file_location("rsp_build", os.path.join(ROOT, "recurrent_state_phi_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _kernel_metadata(asm: str):
    """(name, {key: int}) for every kernel in the amdhsa.kernels metadata list."""
    start = asm.index("amdhsa.kernels:")
    kernels, cur = [], None
    for line in asm[start:].splitlines()[1:]:
        if line.startswith("  - "):
            cur = {}
            kernels.append(cur)
            line = "    " + line[4:]
        elif not line.startswith("    ") and line.strip():
            if cur is not None and not line.startswith(" "):
                break
        m = re.match(r"^    \.(\w+):\s+(\S+)", line)
        if cur is not None and m:
            cur[m.group(1)] = m.group(2)
    return [(k["name"], k) for k in kernels if "name" in k]


@pytest.fixture(scope="module")
def metadata(tmp_path_factory):
    b = _build_module()
    if shutil.which(b.HIPCC) is None and not os.path.exists(b.HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm")

    def compile_one(src):
        dst = out / (src + ".s")
        cmd = [b.HIPCC, "-x", "hip", *b.FLAGS, *b.EXTRA.get(src, []), "--cuda-device-only", "-S",
               os.path.join(b.CSRC, src), "-o", str(dst)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        return src, _kernel_metadata(dst.read_text())

    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        return dict(ex.map(compile_one, SOURCES))


@pytest.mark.parametrize("src", SOURCES)
def test_no_spills_and_no_scratch(metadata, src):
    kernels = metadata[src]
    assert kernels, f"no kernels found in {src}"
    bad = []
    for name, k in kernels:
        allow = next((n for p, n in SGPR_SPILL_ALLOWANCE.items() if name.startswith(p)), 0)
        if int(k["vgpr_spill_count"]) != 0 or int(k["private_segment_fixed_size"]) != 0 \
                or int(k["sgpr_spill_count"]) > allow:
            bad.append((name, k["vgpr_spill_count"], k["sgpr_spill_count"], k["private_segment_fixed_size"]))
    assert not bad, f"kernels that spill (name, vgpr spills, sgpr spills, scratch bytes): {bad}"


# ---------------------------------------------------------------------------
# The hand-over between the workgroups of one sequence in the single-launch
# prefills (n = 3, and n = 1, 2).  Its correctness rests on the emitted code, not on the HIP
# memory model: state images move through the workspace with buffer accesses
# whose cache-policy bit sc1 selects device scope (stores write through the
# XCD's L2, loads do not hit a stale L2 line; CDNA3/CDNA4 instruction-set
# reference, the cache-control bits SC0/SC1/NT of vector memory instructions
# and the memory-scope table they encode), and a writer raises its flag only
# after every wave has waited for its stores to complete (s_waitcnt vmcnt(0))
# and met the others at a barrier.  A compiler change that dropped the bit or
# moved the wait would corrupt prefixes silently, so both are checked here in
# the assembly of every translation unit that holds such a kernel.
# ---------------------------------------------------------------------------
# unit -> (kernel name fragment, number of instances)
HANDOVER_UNITS = {"taylor_prefill_n3.hip": ("prefill_n3_kernel", 2),
                  "taylor_prefill_n3_c128.hip": ("prefill_n3_kernel", 2),
                  "taylor_prefill_small.hip": ("prefill_small_kernel", 8)}
N3_UNITS = [u for u, (k, _) in HANDOVER_UNITS.items() if k == "prefill_n3_kernel"]


def _functions(asm: str):
    """{mangled name: list of instruction lines} for every function in the listing."""
    out, cur, name = {}, None, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            name, cur = m.group(1), []
            out[name] = cur
            continue
        if cur is not None and line.startswith(".Lfunc_end"):
            cur, name = None, None
            continue
        if cur is not None:
            s = line.split(";", 1)[0].strip()
            if s and not s.startswith(".") and not s.endswith(":"):
                cur.append(s)
    return out


@pytest.fixture(scope="module")
def n3_asm(tmp_path_factory):
    b = _build_module()
    if shutil.which(b.HIPCC) is None and not os.path.exists(b.HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm_n3")
    res = {}
    for src, (kname, _) in HANDOVER_UNITS.items():
        dst = out / (src + ".s")
        cmd = [b.HIPCC, "-x", "hip", *b.FLAGS, *b.EXTRA.get(src, []), "--cuda-device-only", "-S",
               os.path.join(b.CSRC, src), "-o", str(dst)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        res[src] = {k: v for k, v in _functions(dst.read_text()).items() if kname in k}
    return res


@pytest.mark.parametrize("src", list(HANDOVER_UNITS))
def test_n3_image_accesses_are_device_scope(n3_asm, src):
    """Every state-image access carries the device-scope bit (sc1).  The n = 1, 2
    kernel makes no other buffer accesses, so there every one must carry it.  The
    n = 3 kernels also load their input rows (q, k, v) with buffer loads, which
    need no such bit: those units have no plain buffer stores (inputs are never
    written), their plain buffer loads are 16-byte row pieces, and the image loads
    of the prefix step (tens per instance) all carry sc1."""
    fns = n3_asm[src]
    assert len(fns) == HANDOVER_UNITS[src][1], f"expected {HANDOVER_UNITS[src][1]} kernel instances in {src}, got {list(fns)}"
    for name, ins in fns.items():
        buf = [i for i in ins if i.startswith("buffer_load") or i.startswith("buffer_store")]
        assert any(i.startswith("buffer_store") for i in buf) and any(i.startswith("buffer_load") for i in buf), name
        missing = [i for i in buf if not re.search(r"\bsc1\b", i)]
        if src in N3_UNITS:
            stores = [i for i in missing if i.startswith("buffer_store")]
            assert not stores, f"{name}: image stores without the device-scope bit: {stores[:4]}"
            odd = [i for i in missing if not i.startswith("buffer_load_dwordx4 ")]
            assert not odd, f"{name}: plain buffer loads other than 16-byte input pieces: {odd[:4]}"
            scoped = [i for i in buf if i.startswith("buffer_load") and re.search(r"\bsc1\b", i)]
            assert len(scoped) >= 24, f"{name}: only {len(scoped)} device-scope image loads"
        else:
            assert not missing, f"{name}: image accesses without the device-scope bit: {missing[:4]}"
        # flag polls are device-scope loads of the header
        polls = [i for i in ins if i.startswith("global_load_dword ") and re.search(r"\bsc1\b", i)]
        assert polls, f"{name}: no device-scope flag poll found"


@pytest.mark.parametrize("src", list(HANDOVER_UNITS))
def test_n3_flag_raised_only_after_stores_complete(n3_asm, src):
    """Every hand-over signal is preceded, with no vector store in between, by an
    s_barrier, and before that by an s_waitcnt that waits for vmcnt(0): the flag
    stores (device-scope dword stores into the header other than the error word at
    byte 4), which publish an image, and the non-returning atomic adds that count
    the segments done reading the caller's state (the last segment overwrites that
    state once the count is full; the returning add is the ticket counter)."""
    store = re.compile(r"^(buffer_store|global_store|flat_store|global_atomic|buffer_atomic|flat_atomic)")
    for name, ins in n3_asm[src].items():
        flags = [j for j, i in enumerate(ins)
                 if i.startswith("global_store_dword ") and re.search(r"\bsc1\b", i) and "offset:4 " not in i + " "]
        counts = [j for j, i in enumerate(ins) if i.startswith("global_atomic_add ") and not re.search(r"\bsc0\b", i)]
        # n = 3: a plain segment's publication and a group leader's, and their two
        # reports; n = 1, 2: the segment sum and the inclusive prefix (no reports:
        # only segment 0 reads the caller's state)
        assert len(flags) >= 2, f"{name}: expected at least two flag stores, found {len(flags)}"
        if src in N3_UNITS:
            assert len(counts) >= 2, f"{name}: expected at least two read reports, found {len(counts)}"
        for j in flags + counts:
            seen_barrier = seen_wait = False
            for i in reversed(ins[:j]):
                if i.startswith("s_barrier"):
                    seen_barrier = True
                elif seen_barrier and i.startswith("s_waitcnt") and "vmcnt(0)" in i:
                    seen_wait = True
                    break
                elif store.match(i):
                    break
            assert seen_barrier and seen_wait, \
                f"{name}: flag store {ins[j]!r} not preceded by s_waitcnt vmcnt(0) and s_barrier"
