"""The byte-level BPE tokenizer ("Let's make GPT-2 in assembly", Step 3) on the
CPU: the oracle (oracle/bpe_tokenizer.py) pinned to GPT-2's published
pre-tokenizer pattern (run by the regex package) and to the tokenizers
package's byte-level BPE, on a synthetic merge table (the published vocab.json
and merges.txt are not available); then the library's native tokenizer against
the oracle, id for id, and its error handling."""
import json
import os

import numpy as np
import pytest

import synth
import transformer_decode_token_amd as g2
from oracle.bpe_tokenizer import BPE, chunks

# GPT-2's published pre-tokenizer pattern (needs \\p{L}, \\p{N}: the regex package)
GPT2_PATTERN = r"""'s|'t|'re|'ve|'m|'ll|'d| ?\p{L}+| ?\p{N}+| ?[^\s\p{L}\p{N}]+|\s+(?!\S)|\s+"""

# the kinds of text the gpt2.s verify script names: contractions, runs of spaces,
# newlines, tabs, digits, punctuation (written here, not taken from it)
CASES = ["Hello world", "don't stop   me now\n\tok", "it's 2024!!  Numbers: 12345 and 3.14",
         "  leading\n\n\nlines  ", "x''s !'s '  ve 'll 'd 'm 're 've", "tabs\t\tand\r\nCRLF\r\n",
         "\x0b\x0cvt\x1cfs", "   ", " ", "'", "''", "a'", "It'S", "one  two   three    four",
         "(parens) [brackets] {braces} <angles>", "a-b_c.d,e;f:g!h?i", "$3.50 + 20% = 4.20",
         "\n", "\t\t", "end with space ", "x" * 300]


@pytest.fixture(scope="module")
def files(tmp_path_factory):
    return synth.make_bpe_files(str(tmp_path_factory.mktemp("bpe")))


@pytest.fixture(scope="module")
def reference(files):
    from tokenizers import Tokenizer, decoders, models, pre_tokenizers
    tk = Tokenizer(models.BPE.from_file(*files))
    tk.pre_tokenizer = pre_tokenizers.ByteLevel(add_prefix_space=False)
    tk.decoder = decoders.ByteLevel()
    return tk


def random_ascii(rng, n):
    alphabet = list("abcdefghijklmnopqrstuvwxyzABCDEFGHIJKLMNOPQRSTUVWXYZ0123456789") + \
        list(" " * 12) + list("\n\t\r'.,!?;:-\"()$%&@#*") + ["'s", "'t", "'re", "'ll", "  ", "\n\n"]
    return "".join(alphabet[i] for i in rng.integers(0, len(alphabet), n))


def test_oracle_chunks_match_gpt2_pattern():
    import regex
    pat = regex.compile(GPT2_PATTERN)
    rng = np.random.default_rng(12)
    texts = CASES + [random_ascii(rng, int(rng.integers(1, 200))) for _ in range(300)] + \
        [synth.synthetic_text(s, 200) for s in range(5)]
    for t in texts:
        assert chunks(t.encode()) == [c.encode() for c in pat.findall(t)], repr(t)


def test_oracle_encode_matches_tokenizers_bytelevel_bpe(files, reference):
    orc = BPE(*files)
    rng = np.random.default_rng(13)
    texts = CASES + [random_ascii(rng, int(rng.integers(1, 200))) for _ in range(200)] + \
        [synth.synthetic_text(s, 300) for s in range(5)]
    for t in texts:
        ids = orc.encode(t.encode())
        assert ids == reference.encode(t).ids, repr(t)
        assert orc.decode(ids) == t.encode()


def test_non_ascii_letters_by_the_pages_rule(files):
    """Bytes above 127 are letters (gpt2.s docs, Limitations): UTF-8 letters
    split as GPT-2 splits them; other non-ASCII symbols join the letter runs."""
    import regex
    pat = regex.compile(GPT2_PATTERN)
    t = "café naïve Zürich"
    assert chunks(t.encode()) == [c.encode() for c in pat.findall(t)]
    assert chunks("a…b".encode()) == ["a…b".encode()]      # one chunk here, three for GPT-2
    assert [c.encode() for c in pat.findall("a…b")] == [b"a", "…".encode(), b"b"]


def test_native_tokenizer_matches_oracle(files):
    orc = BPE(*files)
    tok = g2.gpt2_tokenizer_load(*files)
    rng = np.random.default_rng(14)
    texts = CASES + [random_ascii(rng, int(rng.integers(1, 300))) for _ in range(400)] + \
        [synth.synthetic_text(s, 500) for s in range(8)] + ["café naïve Zürich a…b ÿĀ"]
    for t in texts:
        want = orc.encode(t.encode())
        got = g2.gpt2_tokenize(tok, t)
        assert got.tolist() == want, repr(t)
        assert g2.gpt2_detokenize(tok, got) == t.encode()
    # every byte, one at a time and all together
    raw = bytes(range(256))
    assert g2.gpt2_tokenize(tok, raw).tolist() == orc.encode(raw)
    assert g2.gpt2_detokenize(tok, g2.gpt2_tokenize(tok, raw)) == raw
    assert g2.gpt2_tokenize(tok, b"").size == 0
    tok.close()


def test_host_allocation_failure_is_an_error_code(files, monkeypatch):
    # an exception inside an exported call becomes its error code (here a failed host
    # allocation, injected after the files are read), never an abort across the C ABI
    monkeypatch.setenv("GPT2DEC_FAIL_HOST_ALLOC", "1")
    with pytest.raises(g2.Gpt2Error) as e:
        g2.gpt2_tokenizer_load(*files)
    assert e.value.code == g2.GPT2_E_NOMEM and "host allocation" in str(e.value)
    monkeypatch.delenv("GPT2DEC_FAIL_HOST_ALLOC")
    g2.gpt2_tokenizer_load(*files).close()


def test_native_tokenizer_errors(files, tmp_path):
    import ctypes as C
    tok = g2.gpt2_tokenizer_load(*files)
    L = g2.lib()
    n = C.c_int(0)
    ids = np.zeros(2, np.int32)
    assert L.gpt2_tokenize(tok.handle, b"hello there world", 17, ids.ctypes.data, 2, C.byref(n)) == g2.GPT2_E_INVAL
    assert n.value > 2
    m = C.c_size_t(0)
    bad = np.array([0, 999999], np.int32)
    assert L.gpt2_detokenize(tok.handle, bad.ctypes.data, 2, None, 0, C.byref(m)) == g2.GPT2_E_INVAL
    buf = C.create_string_buffer(1)
    good = g2.gpt2_tokenize(tok, "hello")
    assert L.gpt2_detokenize(tok.handle, good.ctypes.data, good.size, buf, 1, C.byref(m)) == g2.GPT2_E_INVAL
    assert m.value == 5
    tok.close()
    vocab = json.load(open(files[0], encoding="utf-8"))
    merges = open(files[1], encoding="utf-8").read().splitlines()

    def write(v, ms):
        vj, mt = tmp_path / "v.json", tmp_path / "m.txt"
        vj.write_text(json.dumps(v), encoding="utf-8")
        mt.write_text("\n".join(ms) + "\n", encoding="utf-8")
        return str(vj), str(mt)
    cases = {
        "no token for byte": (dict((k, v) for k, v in vocab.items() if k != "a"), merges),
        "lacks": (vocab, merges + ["zzzq zzzr"]),
        "not two tokens": (vocab, merges + ["a b c"]),
        "outside the byte-level alphabet": ({**vocab, "一": 99999}, merges),
    }
    for needle, (v, ms) in cases.items():
        with pytest.raises(g2.Gpt2Error) as e:
            g2.gpt2_tokenizer_load(*write(v, ms))
        assert e.value.code == g2.GPT2_E_INVAL and needle in g2.gpt2_last_error(), g2.gpt2_last_error()
    with pytest.raises(g2.Gpt2Error):
        g2.gpt2_tokenizer_load(str(tmp_path / "absent.json"), files[1])
