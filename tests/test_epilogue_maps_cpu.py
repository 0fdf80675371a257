"""Index maps of the 256-tile kernel's symmetric epilogues and of the fp32
split-contraction tiles, emulated on the CPU (no GPU needed).

The diagonal-tile completion (`diag_fill`) and the mirrored store
(`store_transposed`) read the staged tile with ds_read_b64_tr_b16, whose lane
semantics on gfx950 are: within each group of 16 lanes, lane j supplies the
address of four consecutive 16-bit values, and lane i receives value i % 4 of
the chunks supplied by lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4.  The
emulation below runs the kernels' own address formulas (the staged layout
`soff`, the per-lane supplier addresses, the uniform skip conditions) through
that rule and checks:
  * diag_fill turns a tile whose upper elements (c >= r) are valid into the
    exactly symmetric tile; every value a lane uses was read from an upper
    position, and no upper position ever changes value, so the result does
    not depend on the order in which waves and lanes run;
  * store_transposed writes the transpose of the staged tile, each output
    element once;
  * the four waves of a split-contraction fp32 tile cover every k of a k-tile
    exactly once;
  * the Y block and the weights fetched during the last k-tiles land where
    the staged layout reads them.
Planted mistakes (a swapped supplier address, a wrong skip or merge
condition, a shifted Y placement boundary) each fail one of these.
"""
import numpy as np
import pytest

N = 256          # tile edge
KSTAGE = 32768   # bytes per ring slot


def soff(row, col, ky):
    """Byte offset of staged element (row, col): 512-byte rows, 16-byte chunk
    c at c ^ (row & 31); with ky, rows 192.. one slot further on."""
    off = row * 512 + ((((col >> 3) ^ (row & 31))) << 4) + (col & 7) * 2
    return off + (KSTAGE if (ky and row >= 192) else 0)


class Lds:
    """A staged 16-bit tile addressed through soff, with access logs."""

    def __init__(self, tile, ky):
        self.ky = ky
        self.mem = {}
        self.where = {}
        for r in range(N):
            for c in range(N):
                a = soff(r, c, ky)
                assert a not in self.mem
                self.mem[a] = tile[r, c]
                self.where[a] = (r, c)

    def read4(self, row, col):
        """The four consecutive values one lane of a transposed read points at."""
        a = soff(row, col, self.ky)
        assert a % 8 == 0, "ds_read_b64_tr_b16 needs 8-byte aligned addresses"
        out = []
        for k in range(4):
            assert soff(row, col + k, self.ky) == a + 2 * k, "the four values must be contiguous"
            out.append((self.mem[a + 2 * k], (row, col + k)))
        return out

    def tr_read(self, supplier):
        """One ds_read_b64_tr_b16 of a 16-lane group: supplier[j] = (row, col)."""
        chunks = [self.read4(*supplier[j]) for j in range(16)]
        return [[chunks[i // 4 + 4 * t][i % 4] for t in range(4)] for i in range(16)]

    def tile(self):
        t = np.empty((N, N), dtype=np.float64)
        for a, (r, c) in self.where.items():
            t[r, c] = self.mem[a]
        return t


def tr_chunk(lds, r0, c0):
    """tr_chunk<kY>(lds, r0, c0, j) for the 16 lanes of a group: lane i gets
    staged rows c0 .. c0+7 at column r0 + i (values and their positions)."""
    lo = lds.tr_read([(c0 + (j >> 2), r0 + 4 * (j & 3)) for j in range(16)])
    hi = lds.tr_read([(c0 + 4 + (j >> 2), r0 + 4 * (j & 3)) for j in range(16)])
    return [lo[i] + hi[i] for i in range(16)]


def staged_upper(seed):
    rng = np.random.default_rng(seed)
    up = rng.standard_normal((N, N))
    full = np.triu(up) + np.triu(up, 1).T
    garbage = rng.standard_normal((N, N)) * 1e6
    staged = np.where(np.arange(N)[None, :] >= np.arange(N)[:, None], full, garbage)
    return full, staged


@pytest.mark.parametrize("ky", [False, True])
def test_diag_fill_completes_the_symmetric_tile_from_upper_reads(ky):
    full, staged = staged_upper(3 + ky)
    lds = Lds(staged, ky)
    writes = []
    for w in range(8):                      # waves
        for it in range(16):
            r0 = 16 * it
            if 32 * w >= r0 + 15:           # no lower element in the wave's chunks
                continue
            merge = 32 * w + 31 >= r0       # some upper element: direct reads too
            for g in range(4):              # 16-lane groups of the wave
                c0 = 8 * (4 * w + g)
                t = tr_chunk(lds, r0, c0)
                for i in range(16):
                    r = r0 + i
                    vals = [v for v, _ in t[i]]
                    srcs = [p for _, p in t[i]]
                    if merge:
                        d = [lds.mem[soff(r, c0 + e, ky)] for e in range(8)]
                        for e in range(8):
                            if c0 + e >= r:
                                vals[e], srcs[e] = d[e], (r, c0 + e)
                    for e in range(8):      # every value used is an upper element
                        sr, sc = srcs[e]
                        assert sc >= sr, ("lower source", r, c0 + e, srcs[e])
                    if c0 < r:
                        writes.append((r, c0, vals))
    # apply the writes in any order: upper positions keep their value
    order = np.random.default_rng(0).permutation(len(writes))
    for k in order:
        r, c0, vals = writes[k]
        for e in range(8):
            a = soff(r, c0 + e, ky)
            if c0 + e >= r:
                assert vals[e] == lds.mem[a], "an upper element would change"
            lds.mem[a] = vals[e]
    assert np.array_equal(lds.tile(), full)


@pytest.mark.parametrize("ky", [False, True])
def test_store_transposed_writes_the_transpose_once(ky):
    rng = np.random.default_rng(11 + ky)
    staged = rng.standard_normal((N, N))
    lds = Lds(staged, ky)
    out = np.full((N, N), np.nan)
    for w in range(8):
        for it in range(16):
            for g in range(4):
                c0 = 8 * (4 * w + g)
                t = tr_chunk(lds, 16 * it, c0)
                for i in range(16):
                    r = 16 * it + i
                    for e in range(8):
                        assert np.isnan(out[r, c0 + e]), "written twice"
                        out[r, c0 + e] = t[i][e][0]
    assert np.array_equal(out, staged.T)


def test_split_contraction_waves_cover_each_k_once():
    """gemm32_kernel: wave w reads 16-byte chunk 4·(w/2) + 2·(lane/32) + w%2
    (four fp32 k) of a 128-byte k-row; MFMA e of the wave takes element e of
    it in lanes 0-31 and 32-63 (the instruction's two k)."""
    seen = {}
    for w in range(4):
        for lh in range(2):
            ch = 4 * (w >> 1) + 2 * lh + (w & 1)
            for e in range(4):
                k = 4 * ch + e
                assert k not in seen
                seen[k] = (w, lh, e)
    assert sorted(seen) == list(range(32))
    # the rows a wave finishes after the reduction: 8w + 4·(lane/32) + q
    rows = sorted(8 * w + 4 * lh + q for w in range(4) for lh in range(2) for q in range(4))
    assert rows == list(range(32))


def test_fetched_block_lands_where_the_staged_layout_reads_it():
    """The Gram products' Y block and the weight update's weights are fetched
    during the last k-tiles by global_load_lds (quarter q of 64 rows into
    ring slot q, the last quarter one slot beyond the ring; wave w, load p:
    rows 8w + 2p and 8w + 2p + 1 of the quarter, lane l at byte l·16 of the
    instruction's 1 KiB, fetching logical chunk (l % 32) ^ (row & 31)).  The
    epilogue reads that block through soff with the Y placement."""
    placed = {}
    for q in range(4):
        base = (4 if q == 3 else q) * KSTAGE
        for w in range(8):
            for p in range(4):
                for lane in range(64):
                    r_in = w * 8 + 2 * p + (lane >> 5)
                    chunk = (lane & 31) ^ (r_in & 31)
                    addr = base + (w * 8 + 2 * p) * 512 + lane * 16
                    placed[(64 * q + r_in, chunk)] = addr
    assert len(placed) == N * 32
    for (row, chunk), addr in placed.items():
        assert soff(row, 8 * chunk, True) == addr, (row, chunk)
