"""Second, independently written model of the same coder, in Python integers.

TEST INFRASTRUCTURE ONLY: used by the CPU tests for exhaustive brute force on
tiny inputs, where speed does not matter.  It is deliberately written in a
different style from the C oracle (a symbol is first turned into a list of
"operations", the encoder is a fold of state transformers over that list,
and arbitrary-precision integers make every overflow visible as a failed
range assertion), so that a slip in one is unlikely to be repeated in the
other.

Sources on the pages: kompressor README ("Why", "Credits": CompressAI's
64-bit ryg_rans-style coder); torch_ans 0.3.0 "Usage" table (rans64: 64-bit
state, 32-bit stream words, 16-bit frequencies) and "Low-level API
Reference" (indexed CDFs, offsets, coded range [offset, offset+size-2),
zig-zag bypass of out-of-range values); kompressor BENCHMARKS.md section 4
(decode by a scan of the CDF row).  The same readings R1-R11 as the C oracle
apply; they are stated there.
"""
from __future__ import annotations

M_BITS = 16
M = 1 << M_BITS
LOW = 1 << 31          # smallest normalised state
HIGH = 1 << 63         # states stay below this
WORD = 1 << 32
NIB = 4                # bypass group width in bits


def partition(n: int, lanes: int):
    """Half-open position ranges of the lanes."""
    return [((j * n) // lanes, ((j + 1) * n) // lanes) for j in range(lanes)]


def operations(symbol: int, row: list, offset: int):
    """Operations for one symbol, in decoding order.

    ('f', lo, width) codes a slot of the CDF row; ('b', d) stores a 4-bit digit.
    """
    esc = len(row) - 2
    rel = symbol - offset
    if 0 <= rel < esc:
        return [("f", row[rel], row[rel + 1] - row[rel])]
    if rel < 0:
        raw = 2 * (-rel) - 1
    else:
        raw = 2 * (rel - esc)
    if raw >= 1 << 31:
        raise ValueError("escape distance out of range")
    digits = []
    while raw >> (NIB * len(digits)):
        digits.append((raw >> (NIB * len(digits))) & 15)
    ops = [("f", row[esc], row[esc + 1] - row[esc])]
    count = len(digits)
    while count >= 15:
        ops.append(("b", 15))
        count -= 15
    ops.append(("b", count))
    ops.extend(("b", d) for d in digits)
    return ops


def _push(state: int, op, out: list) -> int:
    """Apply one operation to the encoder state; spilled words go to `out`."""
    assert LOW <= state < HIGH
    if op[0] == "f":
        _, lo, width = op
        if state >= (LOW >> M_BITS) * WORD * width:   # f * 2^47
            out.append(state % WORD)
            state //= WORD
        q, r = divmod(state, width)
        state = q * M + r + lo
    else:
        if state >= (LOW >> NIB) * WORD:             # 2^59
            out.append(state % WORD)
            state //= WORD
        state = state * (1 << NIB) + op[1]
    assert LOW <= state < HIGH
    return state


def encode_single(ops: list) -> list:
    """A standard single rANS64 stream for a list of operations (decode order)."""
    state, spilled = LOW, []
    for op in reversed(ops):
        state = _push(state, op, spilled)
    return [state % WORD, state // WORD] + spilled[::-1]


def encode(symbols, indexes, rows, offsets, lanes: int) -> list:
    """Container words: [L, end_0..end_{L-1}] + lane streams."""
    streams = []
    for b, e in partition(len(symbols), lanes):
        ops = []
        for i in range(b, e):
            ops += operations(symbols[i], rows[indexes[i]], offsets[indexes[i]])
        streams.append(encode_single(ops))
    ends, total = [], 0
    for s in streams:
        total += len(s)
        ends.append(total)
    return [lanes] + ends + [w for s in streams for w in s]


class _Reader:
    def __init__(self, words):
        self.words = list(words)
        if len(self.words) < 2:
            raise ValueError("lane too short")
        self.state = self.words[0] + self.words[1] * WORD
        self.pos = 2

    def _normalise(self):
        if self.state < LOW:
            if self.pos >= len(self.words):
                raise ValueError("ran out of words")
            self.state = self.state * WORD + self.words[self.pos]
            self.pos += 1

    def slot(self, row):
        c = self.state % M
        k = max(i for i in range(len(row) - 1) if row[i] <= c)
        lo, width = row[k], row[k + 1] - row[k]
        self.state = width * (self.state // M) + c - lo
        self._normalise()
        return k

    def digit(self):
        d = self.state % 16
        self.state //= 16
        self._normalise()
        return d


def decode_single(words, indexes, rows, offsets):
    rd = _Reader(words)
    out = []
    for r in indexes:
        row, esc = rows[r], len(rows[r]) - 2
        k = rd.slot(row)
        if k == esc:
            count = t = rd.digit()
            while t == 15:
                t = rd.digit()
                count += t
            if count > 8:
                raise ValueError("bypass group count too large")
            raw = sum(rd.digit() << (NIB * j) for j in range(count))
            k = -(raw // 2) - 1 if raw % 2 else raw // 2 + esc
        out.append(k + offsets[r])
    if rd.state != LOW or rd.pos != len(rd.words):
        raise ValueError("lane did not end cleanly")
    return out


def decode(words, indexes, rows, offsets, lanes: int):
    if words[0] != lanes:
        raise ValueError("lane count mismatch")
    ends = words[1:1 + lanes]
    body = words[1 + lanes:]
    out, prev = [], 0
    for (b, e), end in zip(partition(len(indexes), lanes), ends):
        out += decode_single(body[prev:end], indexes[b:e], rows, offsets)
        prev = end
    return out
