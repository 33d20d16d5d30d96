"""GPU parity of greedy verify acceptance against the oracle (bit-exact: the
results are token ids and counts), and the verify -> accept -> cut back flow
on a resident KV slot (thinkspread, 'The economics of speculative decoding',
opening section)."""
import numpy as np
import pytest
import torch

import speculative_verify_extend_amd as sve
import synth
from oracle.verify import greedy_accept, rollback_len
from tests.gpu_helpers import announce, dev_bf16, host_bits, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _check(logits: np.ndarray, drafts: np.ndarray):
    m = logits.shape[0]
    acc, nxt, t = greedy_accept(logits, drafts)
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda()
    dr = torch.from_numpy(drafts.astype(np.int32)).cuda() if m > 1 else None
    res = sve.verify_accept(lg, dr).cpu().numpy()
    assert res[0] == acc and res[1] == nxt
    assert res[2:].tolist() == t.tolist()
    return acc


@pytest.mark.parametrize("m", list(range(1, 9)) + [16])
def test_full_vocab_matches_oracle(m):
    """A Qwen-family vocabulary (151936 ids), m = k + 1 verify rows."""
    for n_match in sorted({0, (m - 1) // 2, m - 1}):
        announce(f"verify accept V={synth.VERIFY_VOCAB} m={m} match={n_match}")
        logits, drafts, _ = synth.verify_case(20 + m, m, synth.VERIFY_VOCAB, n_match)
        assert _check(logits, drafts) == n_match


@pytest.mark.parametrize("vocab", [1, 7, 4095, 4096, 4097, 10001])
def test_ragged_vocab_sizes(vocab):
    """One chunk, a partial chunk, the scalar path (V % 4 != 0), a chunk
    boundary and several chunks."""
    announce(f"verify accept V={vocab}")
    logits, drafts, _ = synth.verify_case(3, 4, max(vocab, 5), 2)
    logits = np.ascontiguousarray(logits[:, :vocab])
    drafts = np.minimum(drafts, vocab - 1).astype(np.int32)
    _check(logits, drafts)


def test_ties_nans_and_signed_zeros():
    announce("verify accept ties/nan")
    logits, drafts, planted = synth.verify_case(8, 6, 9000, 3, tie=True)
    _check(logits, drafts)  # planted ties: the lower id
    x = logits.copy()
    x[1, 7000] = np.nan
    x[1, 9] = np.nan  # first NaN wins
    x[2, :] = -0.0
    x[2, 4321] = 0.0  # equal to -0.0: id 0 wins
    x[3, :] = -np.inf
    x[4, :] = np.float32(-3.0e38)
    _check(x, drafts)


def test_random_logits_without_plant():
    announce("verify accept random")
    g = np.random.default_rng(4)
    logits = g.standard_normal((8, 50000), dtype=np.float32)
    drafts = g.integers(0, 50000, 7).astype(np.int32)
    drafts[:2] = np.argmax(logits[:2], axis=1)  # (draft construction only)
    assert _check(logits, drafts) >= 2


def test_verify_step_on_a_slot_cuts_back_to_the_accepted_rows():
    """Append the m = k+1 verify rows after P cached ones, accept on the GPU,
    cut the slot back to P + accepted + 1, and check the next step's select
    reuses exactly those rows and that they are the appended ones."""
    hq, hkv, d, P, k = 8, 2, 128, 200, 3
    m = k + 1
    for n_match in (0, 2, 3):
        announce(f"verify flow match={n_match}")
        st = sve.KVSlots(1, 2, hq, hkv, d, 512, 256)
        c = synth.attention_case(30 + n_match, hq, hkv, d, P, m)
        logits, drafts, planted = synth.verify_case(40 + n_match, m, 1000, n_match)
        prefix = np.arange(100, 100 + P, dtype=np.int32)
        inputs = np.concatenate([[7], drafts]).astype(np.int32)
        slot, reused = st.kv_slot_select(np.concatenate([prefix, inputs]))
        assert (slot, reused) == (0, 0)
        for layer in range(2):
            st.extend_attn(0, layer, dev_bf16(c["q_prefix"]), dev_bf16(c["k_prefix"]),
                           dev_bf16(c["v_prefix"]))
            st.extend_attn(0, layer, dev_bf16(c["q"]), dev_bf16(c["k"]), dev_bf16(c["v"]))
        res = sve.verify_accept(torch.from_numpy(logits).cuda(),
                                torch.from_numpy(drafts).cuda()).cpu().numpy()
        acc, nxt, _ = greedy_accept(logits, drafts)
        assert (res[0], res[1]) == (acc, nxt) and acc == n_match
        keep = rollback_len(P, int(res[0]))
        st.kv_truncate(0, keep)
        assert [st.kv_len(0, layer) for layer in range(2)] == [keep, keep]
        kk, vv = st.kv_read(0, 1, 0, keep)
        assert np.array_equal(host_bits(kk), np.concatenate([c["k_prefix"], c["k"][:acc + 1]]))
        assert np.array_equal(host_bits(vv), np.concatenate([c["v_prefix"], c["v"][:acc + 1]]))
        nxt_prompt = np.concatenate([prefix, inputs[:acc + 1], [res[1]], [5, 6]]).astype(np.int32)
        slot, reused = st.kv_slot_select(nxt_prompt)
        assert (slot, reused) == (0, keep)
