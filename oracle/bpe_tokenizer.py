"""CPU oracle of GPT-2's byte-level BPE tokenizer (TEST INFRASTRUCTURE ONLY).

Plain Python, written from "Let's make GPT-2 in assembly", Step 3 (Text to
tokens) and the gpt2.s docs (Limitations):

- Text is split into chunks: an ending 's, 't, 're, 've, 'm, 'll or 'd; a run of
  letters, of digits, or of other symbols, each with one optional space in
  front; or a run of whitespace.  A whitespace run that a non-space follows
  leaves its last character to the next chunk (GPT-2 keeps the space with the
  word after it).  Every byte above 127 counts as a letter, as the docs state
  for gpt2.s, so ASCII text splits exactly as GPT-2's pattern does.
- Each chunk starts as single bytes; repeatedly, the two neighbours whose pair
  has the lowest rank in the merge list join, until no pair has a rank.
- vocab.json names tokens in GPT-2's byte-level alphabet (printable bytes as
  themselves, the others as the code points 256, 257, ... in byte order);
  merges.txt lists the pairs in rank order after a "#version" line.

Only tests/ may import this module.
"""
import json

WHITESPACE = set(b" \t\n\x0b\x0c\r")


def byte_alphabet():
    """byte -> character of GPT-2's byte-level alphabet."""
    kept = list(range(ord("!"), ord("~") + 1)) + list(range(0xA1, 0xAD)) + list(range(0xAE, 0x100))
    out, extra = {}, 0
    for b in range(256):
        if b in kept:
            out[b] = chr(b)
        else:
            out[b] = chr(256 + extra)
            extra += 1
    return out


def _kind(b):
    if b in WHITESPACE:
        return "space"
    if (65 <= b <= 90) or (97 <= b <= 122) or b >= 128:
        return "letter"
    if 48 <= b <= 57:
        return "digit"
    return "other"


def chunks(data: bytes):
    """The pre-tokenizer's chunks of a byte string, in order."""
    out, i, n = [], 0, len(data)
    while i < n:
        b = data[i]
        if b == ord("'"):
            rest = data[i + 1:i + 3]
            if rest[:2] in (b"re", b"ve", b"ll"):
                out.append(data[i:i + 3])
                i += 3
                continue
            if rest[:1] in (b"s", b"t", b"m", b"d"):
                out.append(data[i:i + 2])
                i += 2
                continue
        start = i
        if b == ord(" ") and i + 1 < n and _kind(data[i + 1]) != "space":
            i += 1
        k = _kind(data[i])
        if k != "space":
            j = i
            while j < n and _kind(data[j]) == k:
                j += 1
            out.append(data[start:j])
            i = j
            continue
        # a whitespace run [i, j)
        j = i
        while j < n and _kind(data[j]) == "space":
            j += 1
        if j < n and j - i >= 2:
            j -= 1  # its last character goes with what follows
        out.append(data[i:j])
        i = j
    return out


class BPE:
    def __init__(self, vocab_json, merges_txt):
        with open(vocab_json, encoding="utf-8") as f:
            vocab = json.load(f)
        alpha = byte_alphabet()
        back = {c: b for b, c in alpha.items()}
        self.ids = {bytes(back[c] for c in tok): i for tok, i in vocab.items()}
        self.tok = {i: t for t, i in self.ids.items()}
        self.rank = {}
        with open(merges_txt, encoding="utf-8") as f:
            lines = [ln.rstrip("\n") for ln in f]
        for ln in lines:
            if ln.startswith("#version") or not ln:
                continue
            a, b = ln.split(" ")
            pair = (bytes(back[c] for c in a), bytes(back[c] for c in b))
            self.rank.setdefault(pair, len(self.rank))

    def merge(self, chunk: bytes):
        parts = [bytes([b]) for b in chunk]
        while len(parts) > 1:
            best, where = None, None
            for k in range(len(parts) - 1):
                r = self.rank.get((parts[k], parts[k + 1]))
                if r is not None and (best is None or r < best):
                    best, where = r, k
            if best is None:
                break
            parts = parts[:where] + [parts[where] + parts[where + 1]] + parts[where + 2:]
        return parts

    def encode(self, data: bytes):
        return [self.ids[p] for c in chunks(data) for p in self.merge(c)]

    def decode(self, ids):
        return b"".join(self.tok[i] for i in ids)
