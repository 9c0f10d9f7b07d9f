"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/*.h declares, and host-detectable argument errors come back as
the documented status codes before anything is launched (fake, never
dereferenced, device addresses are passed)."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tree_draft_verification_amd", "libeagle3.so")


def declared_symbols():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(eagle3_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libeagle3.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_every_declared_symbol_is_exported(lib):
    names = declared_symbols()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n


def test_binding_resolves_the_same_names():
    from tree_draft_verification_amd import binding
    for n in declared_symbols():
        assert hasattr(binding, n), n


def test_status_strings(lib):
    lib.eagle3_status_string.restype = ctypes.c_char_p
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = lib.eagle3_status_string(code).decode()
        assert s.startswith("EAGLE3_")
    assert lib.eagle3_abi_version() == 3


FAKE = 0x10000          # 16-byte aligned, never dereferenced on the host
MISALIGNED = 0x10008


def test_tree_mask_errors(lib):
    f = lib.eagle3_tree_mask
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 4
    assert f(FAKE, 1, 0, 1, FAKE, None, None, None) == -1          # T < 1
    assert f(FAKE, 1, 65, 1, FAKE, None, None, None) == -2         # T > 64 W
    assert f(FAKE, 1, 129, 2, FAKE, None, None, None) == -2
    assert f(FAKE, 1, 10, 3, FAKE, None, None, None) == -2         # W > 2
    assert f(None, 1, 10, 1, FAKE, None, None, None) == -1         # null parent
    assert f(None, 0, 10, 1, None, None, None, None) == 0          # empty batch is a no-op


ACCEPT_ARGTYPES = ([ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
                   + [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p])


def test_accept_errors(lib):
    f = lib.eagle3_accept_path
    f.argtypes = ACCEPT_ARGTYPES
    assert f(FAKE, FAKE, FAKE, 1, FAKE, 2, 8, FAKE, FAKE, FAKE, 0, None, None) == -1   # both parent and mask
    assert f(FAKE, None, None, 1, FAKE, 2, 8, FAKE, FAKE, FAKE, 0, None, None) == -1   # neither
    assert f(FAKE, FAKE, None, 1, FAKE, 2, 70, FAKE, FAKE, FAKE, 0, None, None) == -2  # T > 64 W
    # validate mode needs the vocabulary size
    assert f(FAKE, FAKE, None, 1, FAKE, 2, 8, FAKE, FAKE, FAKE, 0, FAKE, None) == -1
    assert f(FAKE, FAKE, None, 1, FAKE, 0, 8, FAKE, FAKE, FAKE, 0, FAKE, None) == -1


def test_rmsnorm_errors(lib):
    f = lib.eagle3_rmsnorm
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p]
    assert f(FAKE, None, 4, 100, 1e-5, 1, FAKE, None) == -2      # K % 8
    assert f(MISALIGNED, None, 4, 128, 1e-5, 1, FAKE, None) == -1
    assert f(FAKE, None, 4, 128, 1e-5, 7, FAKE, None) == -2      # dtype
    assert f(FAKE, None, -1, 128, 1e-5, 1, FAKE, None) == -1


def test_lmhead_errors(lib):
    ws = lib.eagle3_lmhead_workspace
    ws.restype = ctypes.c_size_t
    ws.argtypes = [ctypes.c_int] * 5
    need = ws(61, 128256, 4096, 1, 1)
    assert need >= 61 * 501 * 2 * 8
    f = lib.eagle3_lmhead_argmax
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 5 + [ctypes.c_void_p] * 5 + [ctypes.c_size_t, ctypes.c_void_p]
    assert f(FAKE, FAKE, 61, 128256, 4096, 1, 1, FAKE, None, None, None, FAKE, need - 1, None) == -6
    assert f(FAKE, FAKE, 61, 128256, 4000, 1, 1, FAKE, None, None, None, FAKE, need, None) == -2  # K % 64
    assert f(FAKE, FAKE, 61, 128256, 4096, 17, 1, FAKE, None, None, None, FAKE, 1 << 30, None) == -2
    assert f(MISALIGNED, FAKE, 61, 128256, 4096, 1, 1, FAKE, None, None, None, FAKE, need, None) == -1
    # a hidden state of 4 GiB or more is beyond the 32-bit load offsets of the GEMM core
    assert f(FAKE, FAKE, 1 << 19, 128256, 4096, 1, 1, FAKE, None, None, None, FAKE, 1 << 62, None) == -2


def test_lmhead_noalloc_rejects_calls_past_its_array(lib):
    f = lib.eagle3_lmhead_argmax_noalloc
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 5 + [ctypes.c_void_p] * 5
    # 100000 rows over a 128256-row head need ~2.4 GB of records: refused before any launch
    assert f(FAKE, FAKE, 100000, 128256, 4096, 1, 1, FAKE, None, None, None, None) == -6
    assert f(FAKE, FAKE, 61, 128256, 4096, 17, 1, FAKE, None, None, None, None) == -2
    assert f(None, None, 0, 128256, 4096, 1, 1, None, None, None, None, None) == 0


def test_tree_attn_errors(lib):
    from tree_draft_verification_amd.binding import TreeAttnArgs
    f = lib.eagle3_tree_attn
    f.argtypes = [ctypes.POINTER(TreeAttnArgs), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    wsq = lib.eagle3_tree_attn_workspace
    wsq.restype = ctypes.c_size_t
    wsq.argtypes = [ctypes.POINTER(TreeAttnArgs)]

    def args(**kw):
        a = TreeAttnArgs(dtype=1, B=1, Tq=61, Tk=61, Hq=32, Hkv=8, D=128, W=1, scale=128 ** -0.5,
                         q=FAKE, k_tree=FAKE, v_tree=FAKE, k_cache=FAKE, v_cache=FAKE, num_blocks=65,
                         block_size=16, block_table=FAKE, max_blocks=64, prefix_len=FAKE, mask=FAKE, parent=None,
                         out=FAKE, lse=None, split_keys=0)
        for k, v in kw.items():
            setattr(a, k, v)
        return a

    assert f(ctypes.byref(args(D=64)), None, 0, None) == -2           # bf16 needs D = 128
    assert f(ctypes.byref(args(Hq=30)), None, 0, None) == -2          # Hq % Hkv
    assert f(ctypes.byref(args(Tk=65)), None, 0, None) == -2          # Tk > 64 W
    assert f(ctypes.byref(args(block_size=32)), None, 0, None) == -2
    assert f(ctypes.byref(args(scale=0.0)), None, 0, None) == -1
    assert f(ctypes.byref(args(mask=None)), None, 0, None) == -1      # neither mask nor parent
    assert f(ctypes.byref(args(q=MISALIGNED)), None, 0, None) == -1
    assert f(ctypes.byref(args(split_keys=100)), None, 0, None) == -2  # not a multiple of 64 keys
    assert f(ctypes.byref(args(split_keys=-64)), None, 0, None) == -2
    # one sequence x 8 KV heads is 8 work-groups: split automatically into 4
    # splits of 256 keys (1024-key table), partials in fp32 + (max, sum)
    rows = 1 * 8 * 4 * 256
    assert wsq(ctypes.byref(args())) == rows * 128 * 4 + rows * 8
    assert wsq(ctypes.byref(args(split_keys=512))) == (rows // 2) * 128 * 4 + (rows // 2) * 8
    assert wsq(ctypes.byref(args(split_keys=1024))) == 0              # one split: no partials
    assert wsq(ctypes.byref(args(B=64))) == 0                         # 512 work-groups: no split


def test_empty_batches_are_no_ops(lib):
    """A call over zero rows / sequences returns OK before any pointer check or
    launch (null pointers everywhere, no GPU needed)."""
    from tree_draft_verification_amd.binding import GemmArgs, TreeAttnArgs
    f = lib.eagle3_lmhead_argmax
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 5 + [ctypes.c_void_p] * 5 + [ctypes.c_size_t, ctypes.c_void_p]
    assert f(None, None, 0, 128256, 4096, 1, 1, None, None, None, None, None, 0, None) == 0
    f = lib.eagle3_accept_path
    f.argtypes = ACCEPT_ARGTYPES
    assert f(None, None, None, 1, None, 0, 61, None, None, None, 0, None, None) == 0
    f = lib.eagle3_rmsnorm
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p]
    assert f(None, None, 0, 4096, 1e-5, 1, None, None) == 0
    f = lib.eagle3_tree_attn
    f.argtypes = [ctypes.POINTER(TreeAttnArgs), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    a = TreeAttnArgs(dtype=1, B=0, Tq=61, Tk=61, Hq=32, Hkv=8, D=128, W=1, scale=128 ** -0.5, num_blocks=0,
                     block_size=16, max_blocks=1, split_keys=0, parent=FAKE)
    assert f(ctypes.byref(a), None, 0, None) == 0
    f = lib.eagle3_gemm
    f.argtypes = [ctypes.POINTER(GemmArgs), ctypes.c_void_p]
    g = GemmArgs(dtype=1, M=0, N=4096, nseg=1)
    assert f(ctypes.byref(g), None) == 0
    f = lib.eagle3_draft_fuse
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_void_p] * 3 + [ctypes.c_int] * 4 + [ctypes.c_void_p] * 3 + [ctypes.c_size_t, ctypes.c_void_p]
    assert f(None, None, None, None, None, None, None, None, 0, 4096, 128256, 1, None, None, None, 0, None) == 0


def test_vocab_map_errors(lib):
    f = lib.eagle3_vocab_map
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p]
    assert f(FAKE, -1, FAKE, 10, FAKE, None, None) == -1      # n < 0
    assert f(FAKE, 4, FAKE, 0, FAKE, None, None) == -1        # empty trimmed vocabulary
    assert f(FAKE, 4, None, 10, FAKE, None, None) == -1       # no map
    assert f(None, 4, FAKE, 10, FAKE, None, None) == -1       # no ids
    assert f(FAKE, 4, FAKE, 10, None, None, None) == -1       # no output
    assert f(None, 0, FAKE, 10, None, None, None) == 0        # nothing to map, no status: a no-op


def test_node_positions_errors(lib):
    f = lib.eagle3_node_positions
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert f(FAKE, FAKE, -1, 4, FAKE, None) == -1
    assert f(FAKE, FAKE, 2, 0, FAKE, None) == -1
    assert f(None, FAKE, 2, 4, FAKE, None) == -1
    assert f(FAKE, FAKE, 2, 4, None, None) == -1
    assert f(None, None, 0, 4, None, None) == 0


def test_spec_advance_errors(lib):
    f = lib.eagle3_spec_advance
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 + [ctypes.c_void_p] * 8 + [ctypes.c_int, ctypes.c_void_p]
    ok = [FAKE] * 6
    assert f(FAKE, FAKE, FAKE, 2, 0, 9, *ok, None, None, 0, None) == -1           # T < 1
    assert f(FAKE, FAKE, FAKE, 2, 61, 0, *ok, None, None, 0, None) == -1          # R < 1
    assert f(FAKE, FAKE, FAKE, 2, 61, 9, *ok, FAKE, None, 8, None) == -1          # out_seq without out_len
    assert f(FAKE, FAKE, FAKE, 2, 61, 9, *ok, FAKE, FAKE, 0, None) == -1          # out_seq of no room
    assert f(None, FAKE, FAKE, 2, 61, 9, *ok, None, None, 0, None) == -1          # no accept_len
    assert f(FAKE, FAKE, FAKE, 2, 61, 9, *([FAKE] * 5 + [None]), None, None, 0, None) == -1   # no root
    assert f(None, None, None, 0, 61, 9, *([None] * 6), None, None, 0, None) == 0             # empty batch
