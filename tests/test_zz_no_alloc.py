"""The allocation-free verify entry point (sve_verify_accept_noalloc: static
per-GPU scratch array instead of a caller workspace) against the workspace
form sve_verify_accept, both called through the C ABI, bit for bit (token
ids and counts), on two calls in a row with the second smaller, and against
the oracle's greedy acceptance (thinkspread, 'The economics of speculative
decoding', opening section)."""
import ctypes as C

import numpy as np
import pytest
import torch

import synth
from oracle.verify import greedy_accept
from speculative_verify_extend_amd import _lib
from tests.gpu_helpers import announce, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def _both(lib, logits: np.ndarray, drafts: np.ndarray):
    m, vocab = logits.shape
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda()
    dr = torch.from_numpy(drafts.astype(np.int32)).cuda() if m > 1 else None
    ws_bytes = lib.sve_verify_workspace_bytes(m, vocab)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    r_ws = torch.full((2 + m,), -7, dtype=torch.int32, device="cuda")
    r_na = torch.full((2 + m,), -9, dtype=torch.int32, device="cuda")
    assert lib.sve_verify_accept(_ptr(lg), m, vocab, _ptr(dr), _ptr(r_ws), _ptr(ws), ws_bytes,
                                 st) == _lib.SVE_OK
    assert lib.sve_verify_accept_noalloc(_ptr(lg), m, vocab, _ptr(dr), _ptr(r_na),
                                         st) == _lib.SVE_OK
    torch.cuda.synchronize()
    return r_ws.cpu().numpy(), r_na.cpu().numpy()


def test_noalloc_matches_workspace_form_on_two_calls_second_smaller():
    lib = _lib.load()
    cases = [(8, synth.VERIFY_VOCAB, 5, 31), (3, 4097, 1, 32)]
    for m, vocab, n_match, seed in cases:
        announce(f"verify noalloc m={m} V={vocab}")
        logits, drafts, _ = synth.verify_case(seed, m, vocab, n_match)
        r_ws, r_na = _both(lib, logits, drafts)
        assert np.array_equal(r_ws, r_na)
        acc, nxt, top = greedy_accept(logits, drafts)
        assert r_na[0] == acc == n_match and r_na[1] == nxt
        assert r_na[2:].tolist() == top.tolist()


def test_noalloc_at_the_largest_vocabulary_then_one_row():
    lib = _lib.load()
    for m, vocab, n_match, seed in [(16, _lib.SVE_VERIFY_NOALLOC_MAX_V, 9, 33), (1, 10, 0, 34)]:
        announce(f"verify noalloc m={m} V={vocab}")
        logits, drafts, _ = synth.verify_case(seed, m, vocab, n_match)
        r_ws, r_na = _both(lib, logits, drafts)
        assert np.array_equal(r_ws, r_na)
        assert r_na[0] == n_match
