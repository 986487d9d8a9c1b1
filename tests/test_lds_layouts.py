"""CPU model of the LDS layout of the int8-K decode's weight tables
(quantized_kv_cache_q8_amd/csrc/decode.hip, k_decode_pair_mv): the K wave's 16-byte
stores of a token's rows and the V wave's transposing 16-bit reads of its matrix
operand.  The model restates the kernel's address formulas; the GPU parity tests check
the kernel itself.  The lane mapping of ds_read_b64_tr_b16 is the one measured on the
GPU (within each 16 lanes, lane i receives element i % 4 of the 8 bytes addressed by
lanes 4 e + i / 4, e = 0 .. 3)."""

TABLE_BYTES = 64 * 32


def token_base(t):
    g8, j = t >> 3, t & 7
    return 256 * g8 + 128 * ((j >> 2) ^ (g8 & 1)) + 32 * (j & 3)


def store_addr(t, half):
    # the 16-byte store of rows 8 half .. 8 half + 7 of token t
    return token_base(t) + 16 * (half ^ ((t >> 3) & 1))


def read_addr(qv, iv, hh, rd):
    # the 8 bytes lane (qv, iv) addresses in transposing read rd of token half hh
    sw = qv & 1
    return (256 * qv + 1024 * hh + 128 * (rd ^ sw) + 32 * (iv >> 2)
            + 16 * (((iv & 3) >> 1) ^ sw) + 8 * (iv & 1))


def _table():
    mem = {}
    for t in range(64):
        for half in range(2):
            for e in range(8):
                a = store_addr(t, half) + 2 * e
                assert a not in mem
                mem[a] = (t, 8 * half + e)
    return mem


def test_stores_fill_the_table_once():
    mem = _table()
    assert len(mem) == 64 * 16 and min(mem) == 0 and max(mem) == TABLE_BYTES - 2


def test_reads_give_each_lane_its_row_of_eight_tokens_in_order():
    mem = _table()
    for hh in range(2):
        for qv in range(4):
            g8 = 4 * hh + qv
            for i in range(16):
                got = []
                for rd in range(2):
                    addrs = [read_addr(qv, iv, hh, rd) for iv in range(16)]
                    got += [mem[addrs[4 * e + i // 4] + 2 * (i % 4)] for e in range(4)]
                # k-slot e of lane (qv, i): row i of token 8 g8 + e
                assert got == [(8 * g8 + e, i) for e in range(8)]


def test_no_bank_conflicts():
    # 64 banks of 4 bytes; a 16-byte store serves 16 lanes at once, an 8-byte read 32
    for half in range(2):
        for q in range(4):
            banks = [((store_addr(t, half) >> 2) + k) % 64 for t in range(16 * q, 16 * q + 16)
                     for k in range(4)]
            assert len(set(banks)) == 64
    for hh in range(2):
        for rd in range(2):
            for pair in range(2):
                banks = [((read_addr(qv, iv, hh, rd) >> 2) + k) % 64
                         for qv in (2 * pair, 2 * pair + 1) for iv in range(16) for k in range(2)]
                assert len(set(banks)) == 64
