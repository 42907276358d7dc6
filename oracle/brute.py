"""Brute-force reference for the block-based fixed-length BF16 stream.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Pure Python, bit by bit, for
tiny inputs only (a few thousand elements). It restates the stream definition
a second, independent way -- as one long list of bits and by exhaustive search
of the block width -- so that the C oracle can be checked against it byte for
byte.

Sources: "ENEC: A Lossless AI Model Compression Method Enabling Fast Inference
on Ascend NPUs", Abstract (block-based fixed-length encoding, bit-width
quantization, branch-free integer transformation, intra-segment prefix scan);
"ZipServ: Fast and Memory-Efficient LLM Inference with Hardware-Aware Lossless
Compression", Abstract (fixed-length format, parallel decoding).
"""

HEADER = 256
SEG = 64

# element type -> (bytes, bits, exponent shift, exponent bits); the rest of a
# value (sign, mantissa) is kept as an (exponent shift + 1)-bit field
DTYPES = {1: (2, 16, 7, 8), 2: (2, 16, 10, 5), 3: (4, 32, 23, 8)}


def split_dt(x, dtype):
    """Bit pattern -> (exponent field, sign+mantissa field), by bit lists."""
    _, nbits, sh, eb = DTYPES[dtype]
    bits = [(x >> k) & 1 for k in range(nbits)]
    exp = sum(bits[sh + k] << k for k in range(eb))
    sm = sum(bits[k] << k for k in range(sh)) + (bits[nbits - 1] << sh)
    return exp, sm


def join_dt(exp, sm, dtype):
    _, nbits, sh, eb = DTYPES[dtype]
    bits = [0] * nbits
    for k in range(sh):
        bits[k] = (sm >> k) & 1
    for k in range(eb):
        bits[sh + k] = (exp >> k) & 1
    bits[nbits - 1] = (sm >> sh) & 1
    return sum(b << k for k, b in enumerate(bits))


def _align(v, a):
    return -(-v // a) * a


def split(x):
    """BF16 bit pattern -> (exponent byte, sign+mantissa byte)."""
    bits = [(x >> k) & 1 for k in range(16)]          # bit k of x
    exp = sum(bits[7 + k] << k for k in range(8))      # bits 7..14
    sm = sum(bits[k] << k for k in range(7)) + (bits[15] << 7)
    return exp, sm


def join(exp, sm):
    bits = [0] * 16
    for k in range(7):
        bits[k] = (sm >> k) & 1
    for k in range(8):
        bits[7 + k] = (exp >> k) & 1
    bits[15] = (sm >> 7) & 1
    return sum(b << k for k, b in enumerate(bits))


def width_by_search(codes, allowed=range(9)):
    """Smallest w of `allowed` (ascending) with every code < 2**w."""
    for w in allowed:
        if all(c < (1 << w) for c in codes):
            return w
    raise ValueError("code above 255")


POW2_WIDTHS = (0, 1, 2, 4, 8)


def _le(v, nbytes):
    return [(v >> (8 * i)) & 0xFF for i in range(nbytes)]


def _header(flags, B, n, nb, nseg, sm_off, meta_off, segoff_off, payload_off,
            payload_bytes, raw_off, total, dtype=1):
    h = list(b"ENCB") + _le(1, 2) + _le(dtype, 2) + _le(flags, 4) + _le(B, 4)
    h += _le(SEG, 4) + _le(0, 4)
    for v in (n, nb, nseg, sm_off, meta_off, segoff_off, payload_off,
              payload_bytes, raw_off, total):
        h += _le(v, 8)
    return h + [0] * (HEADER - len(h))


def encode(xs, B, pow2=False, dtype=1):
    """Stream bytes for the bit patterns xs (list of ints) of element type
    dtype at block size B; pow2: widths restricted to POW2_WIDTHS (flag 2)."""
    n = len(xs)
    size = DTYPES[dtype][0]
    S = DTYPES[dtype][2] + 1
    raw = _header(1, B, n, 0, 0, 0, 0, 0, 0, 0, HEADER, HEADER + size * n, dtype)
    for x in xs:
        raw += _le(x, size)
    if n == 0:
        return bytes(raw)
    blocks = [xs[i:i + B] for i in range(0, n, B)]
    nb = len(blocks)
    nseg = -(-nb // SEG)
    metas, payloads = [], []
    for blk in blocks:
        exps = [split_dt(v, dtype)[0] for v in blk]
        base = min(exps)
        codes = [e - base for e in exps]
        w = width_by_search(codes, POW2_WIDTHS if pow2 else range(9))
        bitlist = []
        for c in codes:                      # LSB first, consecutive fields
            bitlist += [(c >> b) & 1 for b in range(w)]
        while len(bitlist) % 8:
            bitlist.append(0)
        body = [sum(bitlist[8 * k + b] << b for b in range(8))
                for k in range(len(bitlist) // 8)]
        while len(body) % 16:
            body.append(0)
        metas.append((base, w))
        payloads.append(body)
    sm_off = HEADER
    meta_off = sm_off + _align(-(-S * n // 8), 256)
    segoff_off = meta_off + _align(2 * nb, 256)
    payload_off = segoff_off + _align(8 * nseg, 256)
    segoffs = [sum(len(p) for p in payloads[:SEG * s]) for s in range(nseg)]
    payload_bytes = sum(len(p) for p in payloads)
    total = payload_off + payload_bytes
    if total >= HEADER + size * n:
        return bytes(raw)
    out = _header(2 if pow2 else 0, B, n, nb, nseg, sm_off, meta_off, segoff_off, payload_off,
                  payload_bytes, 0, total, dtype)
    smbits = []
    for v in xs:                             # S-bit fields, LSB first
        sm = split_dt(v, dtype)[1]
        smbits += [(sm >> b) & 1 for b in range(S)]
    while len(smbits) % 8:
        smbits.append(0)
    out += [sum(smbits[8 * k + b] << b for b in range(8)) for k in range(len(smbits) // 8)]
    out += [0] * (meta_off - len(out))
    for base, w in metas:
        out += [base, w]
    out += [0] * (segoff_off - len(out))
    for so in segoffs:
        out += _le(so, 8)
    out += [0] * (payload_off - len(out))
    for p in payloads:
        out += p
    assert len(out) == total
    return bytes(out)


def _get(s, off, nbytes):
    return sum(s[off + i] << (8 * i) for i in range(nbytes))


def decode(s):
    """Bit patterns decoded from stream bytes s (walks every block)."""
    assert bytes(s[:4]) == b"ENCB"
    dtype = _get(s, 6, 2)
    size, _, sh, eb = DTYPES[dtype]
    S = sh + 1
    flags, B = _get(s, 8, 4), _get(s, 12, 4)
    n = _get(s, 24, 8)
    if flags == 1:
        return [_get(s, HEADER + size * j, size) for j in range(n)]
    nb = _get(s, 32, 8)
    sm_off, meta_off = _get(s, 48, 8), _get(s, 56, 8)
    payload_off = _get(s, 72, 8)
    out = []
    pos = payload_off
    for i in range(nb):
        L = min(B, n - i * B)
        base, w = s[meta_off + 2 * i], s[meta_off + 2 * i + 1]
        bitstream = [(s[pos + k // 8] >> (k % 8)) & 1 for k in range(L * w)]
        for t in range(L):
            d = sum(bitstream[t * w + b] << b for b in range(w))
            j = i * B + t
            sm = sum(((s[sm_off + (j * S + b) // 8] >> ((j * S + b) % 8)) & 1) << b for b in range(S))
            out.append(join_dt((base + d) & ((1 << eb) - 1), sm, dtype))
        pos += _align(-(-L * w // 8), 16)
    return out


def validate(s):
    """(kind, index) of the first failing deep condition of a coded stream
    with a consistent header, restated by walking the blocks in order:
    1 = a width above 8, or not a power of two in a stream flagged 2 (index:
    block), 2 = a stored segment offset that is
    not the running total of padded payload sizes, or a payload_bytes field
    that is not the grand total (index: segment, or nseg for payload_bytes),
    3 = some base + code above 255 (index: block). (0, 0) = valid."""
    flags, B = _get(s, 8, 4), _get(s, 12, 4)
    if flags & 1:
        return 0, 0
    emax = (1 << DTYPES[_get(s, 6, 2)][3]) - 1
    n, nb, nseg = _get(s, 24, 8), _get(s, 32, 8), _get(s, 40, 8)
    meta_off, segoff_off = _get(s, 56, 8), _get(s, 64, 8)
    payload_off, payload_bytes = _get(s, 72, 8), _get(s, 80, 8)
    widths = [s[meta_off + 2 * i + 1] for i in range(nb)]
    allowed = POW2_WIDTHS if flags == 2 else range(9)
    for i, w in enumerate(widths):
        if w not in allowed:
            return 1, i
    sizes = [_align(-(-min(B, n - i * B) * w // 8), 16) for i, w in enumerate(widths)]
    expected = [sum(sizes[:SEG * k]) for k in range(nseg)] + [sum(sizes)]
    stored = [_get(s, segoff_off + 8 * k, 8) for k in range(nseg)] + [payload_bytes]
    for k in range(nseg + 1):
        if stored[k] != expected[k]:
            return 2, k
    pos = payload_off
    for i in range(nb):
        L, base, w = min(B, n - i * B), s[meta_off + 2 * i], widths[i]
        for t in range(L):
            d = sum(((s[pos + (t * w + b) // 8] >> ((t * w + b) % 8)) & 1) << b for b in range(w))
            if base + d > emax:
                return 3, i
        pos += sizes[i]
    return 0, 0
