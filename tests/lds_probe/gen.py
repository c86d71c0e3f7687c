"""Test table for the LDS read probe (probe.hip), one line per dispatch.

  - pass membership: every lane reads its own 16 (b128) or 8 (b64
    transposing) bytes, contiguous, except lane j, moved onto lane 0's bank
    (address 4096); a conflict means lane j shares a pass with the lane that
    owns that bank;
  - bank period: lane 1 at distance d from lane 0, every other lane on one
    shared address (a broadcast);
  - the four operand read patterns of the attention kernels (32x32x16 and
    16x16x32 row-major, and both transposing forms) under candidate 64-row
    D = 128 tile layouts.

usage: python3 gen.py TESTS_OUT LEGEND_OUT"""
import json, sys
tests, legend = [], []
def add(kind, offs8, name):
    assert len(offs8) == 8 and all(len(o) == 64 for o in offs8)
    for o in offs8:
        for a in o: assert 0 <= a <= 65536 - 16 and a % (16 if kind == 0 else 8) == 0, (name, a)
    tests.append((kind, offs8)); legend.append(name)
rep = lambda o: [list(o)] * 8
for kind, w in ((0, 16), (1, 8)):
    base = [w * l for l in range(64)]
    add(kind, rep(base), f"k{kind} base")
    for j in range(1, 64):
        o = list(base); o[j] = 4096
        add(kind, rep(o), f"k{kind} member {j}")
for kind, w in ((0, 16), (1, 8)):
    for d in [8, 16, 32, 48, 64, 96, 128, 192, 256, 384, 512, 768, 1024, 2048, 4096]:
        if d % w: continue
        o = [8192 + 48] * 64; o[0] = 0; o[1] = d
        add(kind, rep(o), f"k{kind} period {d}")
def swz(r): return ((r & 3) << 2 | (r & 4) >> 1) ^ (3 * ((r >> 3) & 1))
def L_xor(r, c): return (r * 16 + (c ^ swz(r))) * 16
def L_nat(r, c): return r * 256 + 16 * c
def mk_pt(bb, gs, fx=128, fh=16, krow=32):
    def L(r, c):
        return gs * (r >> 4) + bb[(r >> 2) & 3] + krow * (r & 3) + fh * (c & 1) + fx * (c >> 1)
    return L
# swizzled tile of the forward; natural rows; pair-major blocks (block starts, group stride)
layouts = {
    'xor': L_xor, 'natural': L_nat,
    'pt_1152': mk_pt([0, 1152, 2192, 3344], 4368),
    'pt_1040': mk_pt([0, 1040, 2176, 3216], 4240),
    'pt_plain': mk_pt([0, 1024, 2048, 3072], 4096),
    'pt_new': mk_pt([0, 1152, 2304, 3456], 4496),
    'quad': lambda r, c: 4208 * (r >> 4) + [0, 1056, 2112, 3168][(r >> 2) & 3] + 256 * (c >> 2) + 64 * (r & 3) + 16 * (c & 3),
}
def P1(L):
    return [[L(l % 32, 2 * x + l // 32) for l in range(64)] for x in range(8)]
def P2(L):
    return [[L(16 * b + l % 16, 4 * x + l // 16) for l in range(64)] for b in range(2) for x in range(4)]
def tr_addr(L, r, e): return L(r, e >> 3) + 2 * (e & 7)
def P3(L):
    return [[tr_addr(L, 4 * (l // 32) + 8 * v + (l % 16) // 4, 32 * t + 16 * ((l // 16) % 2) + 4 * (l % 4)) for l in range(64)]
            for t in range(4) for v in range(2)]
def P4(L):
    return [[tr_addr(L, 16 * (t % 2) + 4 * (l // 16) + (l % 16) // 4, 16 * (t // 2) + 4 * (l % 4)) for l in range(64)] for t in range(8)]
for name, L in layouts.items():
    add(0, P1(L), f"layout {name} P1"); add(0, P2(L), f"layout {name} P2")
    add(1, P3(L), f"layout {name} P3"); add(1, P4(L), f"layout {name} P4")
with open(sys.argv[1], 'w') as f:
    f.write(f"{len(tests)}\n")
    for kind, o8 in tests:
        f.write(f"{kind} " + " ".join(str(a) for o in o8 for a in o) + "\n")
json.dump(legend, open(sys.argv[2], 'w'))
print(len(tests), "tests")
