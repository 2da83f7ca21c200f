"""CPU tests of the C-ABI boundary: the library loads and exports every entry
point the header declares, the ctypes struct matches the C layout, and every
argument check fires before any HIP call (so they run without a GPU)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import sparse_moe_transformer_route_amd as hm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hy_moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hy_(?:moe|indexer)_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(hm.EXPORTED)
    L = ctypes.CDLL(hm.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", hm.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (hy_(?:moe|indexer)_\w+)", out))
    assert set(names) <= exported


def test_struct_layout_matches_c(tmp_path):
    fields = [f[0] for f in hm.HyMoeArgs._fields_]
    src = tmp_path / "layout.c"
    body = "\n".join(f'  printf("{f} %zu\\n", offsetof(hy_moe_args, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "hy_moe.h"\nint main(void){\n'
                   f'  printf("sizeof %zu\\n", sizeof(hy_moe_args));\n{body}\n  return 0;\n}}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split("\n")
               if line)
    assert int(got["sizeof"]) == ctypes.sizeof(hm.HyMoeArgs)
    for f in fields:
        assert int(got[f]) == getattr(hm.HyMoeArgs, f).offset, f


FAKE = 0x100000  # 16-byte aligned non-null address; never dereferenced by the checks


def base_args(T=4, d=256, E=16, k=2, I=128):
    a = hm.HyMoeArgs()
    a.x = a.W_router = a.W_gate = a.W_up = a.W_down = FAKE
    a.Ws_gate = a.Ws_up = a.Ws_down = a.out = FAKE
    a.T, a.d, a.E, a.k, a.I = T, d, E, k, I
    return a


def call(a):
    return hm.lib().hy_moe_forward_ex(ctypes.byref(a), None)


@pytest.mark.parametrize("field,value,status", [
    ("k", 0, hm.ERR_INVALID_ARG), ("k", 17, hm.ERR_INVALID_ARG), ("T", -1, hm.ERR_INVALID_ARG),
    ("d", 0, hm.ERR_INVALID_ARG), ("I", -128, hm.ERR_INVALID_ARG), ("E", 0, hm.ERR_INVALID_ARG),
    ("d", 192, hm.ERR_UNSUPPORTED), ("I", 64, hm.ERR_UNSUPPORTED), ("x", None, hm.ERR_INVALID_ARG),
    ("out", None, hm.ERR_INVALID_ARG), ("W_down", None, hm.ERR_INVALID_ARG), ("Ws_up", None, hm.ERR_INVALID_ARG),
    ("x", FAKE + 2, hm.ERR_INVALID_ARG), ("expert_format", 7, hm.ERR_INVALID_ARG), ("path", 9, hm.ERR_INVALID_ARG),
    ("workspace", FAKE + 64, hm.ERR_INVALID_ARG), ("topk_idx", FAKE + 2, hm.ERR_INVALID_ARG),
])
def test_argument_checks(field, value, status):
    a = base_args()
    setattr(a, field, value)
    assert call(a) == status


def test_envelope_limits():
    a = base_args(E=2048, k=8)
    assert call(a) == hm.ERR_UNSUPPORTED
    a = base_args(E=32, k=17)
    assert call(a) == hm.ERR_UNSUPPORTED
    a = base_args(T=2 ** 28, k=8, E=64)
    assert call(a) == hm.ERR_UNSUPPORTED
    assert hm.lib().hy_moe_forward_ex(None, None) == hm.ERR_INVALID_ARG


def test_probe_argument_checks():
    m = re.search(r"#define HY_MOE_PROBE_OPERAND_BYTES (\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == hm.PROBE_OPERAND_BYTES
    L = hm.lib()
    out = ctypes.c_float()
    assert L.hy_moe_probe_mfma_bf16(None, hm.PROBE_OPERAND_BYTES, ctypes.byref(out), None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_probe_mfma_bf16(FAKE, hm.PROBE_OPERAND_BYTES - 16, ctypes.byref(out), None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_probe_mfma_bf16(FAKE + 8, hm.PROBE_OPERAND_BYTES, ctypes.byref(out), None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_probe_mfma_bf16(FAKE, hm.PROBE_OPERAND_BYTES, None, None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_probe_mfma_fp8(None, hm.PROBE_OPERAND_BYTES, ctypes.byref(out), None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_probe_mfma_fp8(FAKE, hm.PROBE_OPERAND_BYTES - 16, ctypes.byref(out), None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_probe_mfma_fp8(FAKE + 8, hm.PROBE_OPERAND_BYTES, ctypes.byref(out), None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_probe_mfma_fp8(FAKE, hm.PROBE_OPERAND_BYTES, None, None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_probe_hbm_read(None, 1 << 20, ctypes.byref(out), None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_probe_hbm_read(FAKE, 8, ctypes.byref(out), None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_probe_hbm_read(FAKE + 4, 1 << 20, ctypes.byref(out), None) == hm.ERR_INVALID_ARG


def test_grouped_path_byte_limit():
    # the grouped GEMM addresses x and the hidden activations with 32-bit byte offsets
    a = base_args(T=2 ** 18, d=8192, E=64, k=8, I=128)  # x: 2^32 bytes
    a.path = hm.PATH_GROUPED
    assert call(a) == hm.ERR_UNSUPPORTED
    a = base_args(T=2 ** 18, d=128, E=64, k=7, I=2048)  # h: 8 * 2^18 rows * 4 KiB = 2^33 bytes
    a.path = hm.PATH_GROUPED
    assert call(a) == hm.ERR_UNSUPPORTED


def test_ternary_requires_codes_and_scales():
    a = base_args()
    a.expert_format = hm.WEIGHTS_SHERRY_TERNARY
    assert call(a) == hm.ERR_INVALID_ARG
    a.Wq_gate = a.Wq_up = a.Wq_down = a.S_gate = a.S_up = a.S_down = FAKE
    a.Wq_down = FAKE + 2  # codes and scales must be 4-byte aligned
    assert call(a) == hm.ERR_INVALID_ARG
    a.Wq_down = FAKE
    a.S_up = FAKE + 2
    assert call(a) == hm.ERR_INVALID_ARG


def test_small_workspace_rejected():
    a = base_args()
    a.workspace = FAKE
    a.workspace_bytes = hm.workspace_size(4, 256, 16, 2, 128) - 1
    assert call(a) == hm.ERR_WORKSPACE


def test_empty_batch_is_a_no_op_without_touching_pointers():
    a = hm.HyMoeArgs()
    a.T, a.d, a.E, a.k, a.I = 0, 256, 16, 2, 128
    assert call(a) == hm.OK
    L = hm.lib()
    assert L.hy_moe_forward(None, None, None, None, None, None, None, None, 0, 256, 16, 2, 128, None, None) == hm.OK


def test_workspace_size_monotone_and_zero_for_invalid():
    sizes = [hm.workspace_size(T, 6144, 256, 8, 2048) for T in (1, 32, 1024, 8192)]
    assert all(s > 0 for s in sizes) and sizes == sorted(sizes)
    assert hm.workspace_size(8, 6144, 256, 0, 2048) == 0
    assert hm.workspace_size(8, 100, 256, 8, 2048) == 0
    assert hm.workspace_size(8, 6144, 256, 8, 2048, 6) == 0
    assert hm.workspace_size(8192, 6144, 256, 8, 2048) % 256 == 0


def test_status_strings():
    assert hm.status_string(hm.OK) == "ok"
    for s in (hm.ERR_INVALID_ARG, hm.ERR_UNSUPPORTED, hm.ERR_WORKSPACE, hm.ERR_HIP):
        assert hm.status_string(s) not in ("ok", "unknown status")
    assert hm.status_string(12345) == "unknown status"


def test_sherry_pack_host_round_trips_with_oracle_decoder():
    rng = np.random.default_rng(0)
    rows, cols = 5, 256
    zpos = rng.integers(0, 4, size=(rows, cols // 4))
    signs = rng.choice([-1, 1], size=(rows, cols))
    tern = signs.astype(np.int8)
    for r in range(rows):
        for g in range(cols // 4):
            tern[r, 4 * g + zpos[r, g]] = 0
    packed = hm.sherry_pack_host(tern)
    assert packed.shape == (rows, cols // 128 * 5)
    dec, _ = oracle.sherry_decode(packed)
    assert np.array_equal(dec, tern)
    # all 32 codes in one block, in code order: packing the oracle's decoding of
    # words 0..31-coded block reproduces the words
    B = sum(c << (5 * c) for c in range(32))
    words = np.array([[(B >> (32 * i)) & 0xFFFFFFFF for i in range(5)]], np.uint32)
    dec, _ = oracle.sherry_decode(words)
    assert np.array_equal(hm.sherry_pack_host(dec), words)


def test_sherry_pack_host_rejects_bad_groups():
    tern = np.ones((1, 128), np.int8)  # no zero in any group
    packed = np.full((1, 5), 0xDEADBEEF, np.uint32)
    rc = hm.lib().hy_moe_sherry_pack_host(tern.ctypes.data, 1, 128, packed.ctypes.data)
    assert rc == hm.ERR_INVALID_ARG and (packed == 0xDEADBEEF).all()
    tern = np.zeros((1, 128), np.int8)  # four zeros per group
    assert hm.lib().hy_moe_sherry_pack_host(tern.ctypes.data, 1, 128, packed.ctypes.data) == hm.ERR_INVALID_ARG
    assert hm.lib().hy_moe_sherry_pack_host(tern.ctypes.data, 1, 100, packed.ctypes.data) == hm.ERR_INVALID_ARG


def test_one_hip_runtime_in_process():
    # The library must bind to the HIP runtime torch loaded (device memory and
    # streams come from torch); a second runtime copy would not share them.
    import hy_inputs
    hy_inputs.dev_lib()
    maps = open("/proc/self/maps").read().splitlines()
    runtimes = {line.split()[-1] for line in maps if "libamdhip64" in line}
    assert len(runtimes) == 1, runtimes


def test_indexer_argument_checks():
    L = hm.lib()
    out = FAKE

    def ix(q=FAKE, w=FAKE, keys=FAKE, B=2, H=32, D=128, S=1000, K=64, idx=out, scores=FAKE, ws=None, wsb=0):
        return L.hy_indexer_topk(q, w, keys, B, H, D, S, K, idx, scores, ws, wsb, None, None)
    assert ix(H=16) == hm.ERR_UNSUPPORTED
    assert ix(D=64) == hm.ERR_UNSUPPORTED
    assert ix(B=70000) == hm.ERR_UNSUPPORTED
    assert ix(K=0) == hm.ERR_INVALID_ARG
    assert ix(S=-1) == hm.ERR_INVALID_ARG
    assert ix(q=None) == hm.ERR_INVALID_ARG
    assert ix(keys=FAKE + 8) == hm.ERR_INVALID_ARG          # keys must be 16-byte aligned
    assert ix(scores=None) == hm.ERR_INVALID_ARG            # no workspace
    assert ix(scores=None, ws=FAKE, wsb=16) == hm.ERR_WORKSPACE
    assert ix(B=0, q=None, keys=None) == hm.OK              # empty: no pointer is touched
    assert ix(S=0, q=None, keys=None) == hm.OK
    assert L.hy_indexer_workspace_size(4, 1000) >= 4 * 1000 * 4


def call_noalloc(a):
    return hm.lib().hy_moe_forward_noalloc(ctypes.byref(a), None)


def test_noalloc_argument_checks_run_before_any_hip_call():
    # every rejection below happens on the host, before the static scratch is resolved
    a = base_args()
    a.workspace, a.workspace_bytes = FAKE, hm.workspace_size(4, 256, 16, 2, 128)
    assert call_noalloc(a) == hm.ERR_INVALID_ARG           # no workspace may be passed
    a = base_args()
    a.workspace_bytes = 1
    assert call_noalloc(a) == hm.ERR_INVALID_ARG
    a = base_args()
    a.k = 0
    assert call_noalloc(a) == hm.ERR_INVALID_ARG
    a = base_args()
    a.x = None
    assert call_noalloc(a) == hm.ERR_INVALID_ARG
    assert hm.lib().hy_moe_forward_noalloc(None, None) == hm.ERR_INVALID_ARG
    a = base_args(T=0)
    assert call_noalloc(a) == hm.OK                        # empty batch: a no-op
    a = base_args(T=252, d=6144, E=256, k=8, I=2048)        # needs more than the static scratch
    assert hm.workspace_size(252, 6144, 256, 8, 2048) > hm.NOALLOC_SCRATCH_BYTES
    assert call_noalloc(a) == hm.ERR_WORKSPACE


def test_noalloc_limit_stated_in_header():
    # the header states the largest Hy4-shape batch the static scratch admits
    text = open(HEADER).read()
    assert "#define HY_MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text
    assert hm.NOALLOC_SCRATCH_BYTES == 64 << 20
    limit = int(re.search(r"that admits T <= (\d+)", text).group(1))
    limit8 = int(re.search(r"\(T <= (\d+) with\s+\*\s+HY_MOE_WEIGHTS_FP8_W8A8", text).group(1))
    for fmt, lim in ((hm.WEIGHTS_BF16, limit), (hm.WEIGHTS_SHERRY_TERNARY, limit), (hm.WEIGHTS_FP8_E4M3, limit),
                     (hm.WEIGHTS_FP8_W8A8, limit8)):
        assert hm.workspace_size(lim, 6144, 256, 8, 2048, fmt) <= hm.NOALLOC_SCRATCH_BYTES
        assert hm.workspace_size(lim + 1, 6144, 256, 8, 2048, fmt) > hm.NOALLOC_SCRATCH_BYTES


def test_fp8_w8a8_argument_checks():
    a = base_args(T=4, d=512, E=16, k=2, I=256)
    a.expert_format = hm.WEIGHTS_FP8_W8A8
    a.W_gate = a.W_up = a.W_down = None
    a.Wq_gate = a.Wq_up = a.Wq_down = a.S_gate = a.S_up = a.S_down = FAKE
    a.workspace = FAKE
    a.workspace_bytes = hm.workspace_size(4, 512, 16, 2, 256, hm.WEIGHTS_FP8_W8A8) - 1
    assert call(a) == hm.ERR_WORKSPACE
    a.workspace, a.workspace_bytes = None, 0
    a.path = hm.PATH_STREAM
    assert call(a) == hm.ERR_UNSUPPORTED              # grouped path only
    a.path = hm.PATH_AUTO
    a.d = 384
    assert call(a) == hm.ERR_UNSUPPORTED              # d % 256
    a.d, a.I = 512, 128
    assert call(a) == hm.ERR_UNSUPPORTED              # I % 256
    a.I = 256
    a.S_down = FAKE + 2
    assert call(a) == hm.ERR_INVALID_ARG
    # the W8A8 workspace holds the MXFP8 rows: larger than the weight-only FP8 one at prefill
    # sizes would be without its bf16 expert outputs
    assert hm.workspace_size(8192, 6144, 256, 8, 2048, hm.WEIGHTS_FP8_W8A8) > 0


def test_mxfp8_quantize_argument_checks():
    L = hm.lib()
    assert L.hy_moe_mxfp8_quantize(FAKE, 4, 48, FAKE, FAKE, None) == hm.ERR_INVALID_ARG   # cols % 32
    assert L.hy_moe_mxfp8_quantize(FAKE, -1, 64, FAKE, FAKE, None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_mxfp8_quantize(None, 4, 64, FAKE, FAKE, None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_mxfp8_quantize(FAKE + 8, 4, 64, FAKE, FAKE, None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_mxfp8_quantize(FAKE, 0, 64, None, None, None) == hm.OK              # empty: no-op



def test_block_bf16_argument_checks():
    L = hm.lib()
    BIG = 0x10000000  # far from FAKE: the buffers do not overlap
    assert L.hy_moe_block_bf16(FAKE, BIG, 2, 24, 128, None) == hm.ERR_INVALID_ARG     # rows % 16
    assert L.hy_moe_block_bf16(FAKE, BIG, 2, 32, 96, None) == hm.ERR_INVALID_ARG      # cols % 64
    assert L.hy_moe_block_bf16(FAKE, BIG, -1, 32, 128, None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_block_bf16(None, BIG, 2, 32, 128, None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_block_bf16(FAKE, BIG + 8, 2, 32, 128, None) == hm.ERR_INVALID_ARG  # misaligned
    # overlapping buffers: 2 x 32 x 128 bf16 = 16 KB from FAKE; dst 4 KB in
    assert L.hy_moe_block_bf16(FAKE, FAKE + 4096, 2, 32, 128, None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_block_bf16(FAKE + 4096, FAKE, 2, 32, 128, None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_block_bf16(None, None, 0, 32, 128, None) == hm.OK                  # empty: no-op


def test_blocked_format_checks_and_workspace():
    # the blocked format takes the bf16 pointers, checks and workspace
    a = base_args(T=4, d=512, E=16, k=2, I=256)
    a.expert_format = hm.WEIGHTS_BF16_BLOCKED
    a.W_down = FAKE + 2
    assert call(a) == hm.ERR_INVALID_ARG
    a.W_down = None
    assert call(a) == hm.ERR_INVALID_ARG
    for T in (1, 32, 8192):
        assert hm.workspace_size(T, 6144, 256, 8, 2048, hm.WEIGHTS_BF16_BLOCKED) == \
            hm.workspace_size(T, 6144, 256, 8, 2048, hm.WEIGHTS_BF16)
    assert hm.workspace_size(4, 512, 16, 2, 256, 6) == 0  # no such format


def test_block_sherry_argument_checks():
    L = hm.lib()
    BIG = 0x10000000
    assert L.hy_moe_block_sherry(FAKE, BIG, 2, 24, 512, None) == hm.ERR_INVALID_ARG     # rows % 16
    assert L.hy_moe_block_sherry(FAKE, BIG, 2, 32, 384, None) == hm.ERR_INVALID_ARG     # cols % 512
    assert L.hy_moe_block_sherry(FAKE, BIG, -1, 32, 512, None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_block_sherry(FAKE, None, 2, 32, 512, None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_block_sherry(FAKE + 4, BIG, 2, 32, 512, None) == hm.ERR_INVALID_ARG  # misaligned
    # 2 x 32 rows x 80 bytes = 5 KB of codes from FAKE; dst 4 KB in overlaps, 5 KB in does not
    assert L.hy_moe_block_sherry(FAKE, FAKE + 4096, 2, 32, 512, None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_block_sherry(FAKE + 4096, FAKE, 2, 32, 512, None) == hm.ERR_INVALID_ARG
    assert L.hy_moe_block_sherry(None, None, 0, 32, 512, None) == hm.OK                  # empty: no-op


def test_blocked_sherry_format_checks_and_workspace():
    # the blocked Sherry format takes the ternary pointers; codes 16-byte aligned, d and I % 512
    a = base_args(T=4, d=512, E=16, k=2, I=512)
    a.expert_format = hm.WEIGHTS_SHERRY_BLOCKED
    assert call(a) == hm.ERR_INVALID_ARG  # no codes or scales
    a.Wq_gate = a.Wq_up = a.Wq_down = a.S_gate = a.S_up = a.S_down = FAKE
    a.Wq_up = FAKE + 4  # 4-byte alignment suffices for row-major codes, not for blocked ones
    assert call(a) == hm.ERR_INVALID_ARG
    a.Wq_up = FAKE
    for d, I in ((512, 256), (384, 512), (2 ** 20, 2 ** 17)):  # the last: one code matrix of 2^31 bytes
        b = base_args(T=4, d=d, E=16, k=2, I=I)
        b.expert_format = hm.WEIGHTS_SHERRY_BLOCKED
        b.Wq_gate = b.Wq_up = b.Wq_down = b.S_gate = b.S_up = b.S_down = FAKE
        assert call(b) == hm.ERR_UNSUPPORTED
    for T in (1, 32, 8192):
        assert hm.workspace_size(T, 6144, 256, 8, 2048, hm.WEIGHTS_SHERRY_BLOCKED) == \
            hm.workspace_size(T, 6144, 256, 8, 2048, hm.WEIGHTS_SHERRY_TERNARY)


def test_shared_format_checks():
    # a Sherry shared expert needs the Sherry expert format itself, d and I % 512 and
    # 16-byte aligned codes; the bf16 shared pointers are then not required
    def sherry_args(d=512, I=512, fmt=None):
        a = base_args(T=4, d=d, E=16, k=2, I=I)
        a.expert_format = hm.WEIGHTS_SHERRY_TERNARY if fmt is None else fmt
        a.Wq_gate = a.Wq_up = a.Wq_down = a.S_gate = a.S_up = a.S_down = FAKE
        a.Ws_gate = a.Ws_up = a.Ws_down = None
        a.shared_format = a.expert_format
        return a
    a = base_args()
    a.shared_format = hm.WEIGHTS_SHERRY_TERNARY  # bf16 routed experts
    assert call(a) == hm.ERR_INVALID_ARG
    a = sherry_args(fmt=hm.WEIGHTS_FP8_E4M3)
    assert call(a) == hm.ERR_INVALID_ARG
    a = sherry_args()
    a.shared_format = 7
    assert call(a) == hm.ERR_INVALID_ARG
    a = sherry_args()
    a.shared_format = hm.WEIGHTS_SHERRY_BLOCKED  # must equal the expert format
    assert call(a) == hm.ERR_INVALID_ARG
    a = sherry_args()
    a.Wq_up = FAKE + 4
    assert call(a) == hm.ERR_INVALID_ARG
    assert call(sherry_args(I=256)) == hm.ERR_UNSUPPORTED
    assert call(sherry_args(d=384)) == hm.ERR_UNSUPPORTED
    a = sherry_args()
    a.shared_format = hm.WEIGHTS_BF16  # then the bf16 shared pointers are required
    assert call(a) == hm.ERR_INVALID_ARG
