"""Writes decode_bf16_asm.inc: the instruction streams of the bf16 latent
decode kernel's software-pipelined tile step (decode_mfma.hip).

    python gen_decode_bf16_asm.py > decode_bf16_asm.inc

One step of a workgroup (four waves, 128 heads of one query) consumes two
32-token tiles held in LDS: it scores tile k+1 against the register-resident
latent query and turns the scores into softmax numerators, and it adds tile
k's numerator-weighted value rows into the output accumulators.

  scores   S^T[t, h] = sum_d K[t, d] Q[h, d]: 36 MFMAs (32x32x16 bf16) in one
           accumulator chain (dependent MFMAs issue back to back here)
  softmax  p = 2^(S*scale*log2(e) - m_ref) against a per-head reference fixed
           at the first visible tile; the numerators of this wave's 32 heads
           go to LDS as bf16 (the B operand of the weighted sum)
  sum      O^T[c, h] += sum_t V^T[c, t] P^T[t, h]: 32 MFMAs; this wave owns
           latent columns 128*wave..+127 of all 128 heads (4 column tiles x 4
           head groups), so each transposed value fragment is read once and
           used for four head groups

The MFMA stream is the 36 score MFMAs with 12 sum MFMAs spread evenly
among them, then the remaining 20 sum MFMAs with the
softmax's VALU work placed between them.  LDS reads are
issued ahead and waited for with lgkmcnt counts computed here from the issue
order; the nine tile copies of the wave are spread over the first part.

Operands (named in the kernel):
  %[o0]..%[o15]   O^T accumulators, o{4j+g}: column tile j, head group g
  %[q0]..%[q35]   latent query fragments, 16 dims each
  %[ka0..3]       per-lane LDS byte offsets of the key fragments
  %[va0..3]       per-lane LDS byte offsets of this wave's value fragments
  %[pa]           16 * lane
  %[bk], %[bv], %[bp]  LDS byte address of the key tile, the value tile and
                  the P^T buffer of the tile being summed
  %[bpw]          LDS byte address where this wave's P^T of the scored tile goes
  %[scale]        softmax scale times log2(e)
  %[mref], %[mseen], %[lrun], %[exc]  per-head softmax state: reference,
                  running maximum, running sum, largest excess over the
                  reference (in/out)
  %[vlim], %[tok] masked streams only: token t (0..31) of the scored tile is
                  visible iff t < vlim - tok
  %[cb], %[cd], %[cl], %[k1152], %[c0..4]   the tile copy (see copy())
The streams use v177-v255, vcc, m0 and scc as scratch.

The same streams serve two more row formats of the latent cache:
  NoPE  rows of 512 bf16 values (no RoPE part): 32 query fragments, eight
        copies per wave, 64 chunks per tile row
  FP4   rows of 576 E2M1 codes with an E8M0 scale per 32 values (320 bytes):
        the stored rows are staged in LDS by copies the kernel issues, and
        the step stream expands tile k+2 into the bf16 tile layout between
        the weighted-sum MFMAs of its second part (each wave its own eight
        rows: one 4-byte code word and one scale byte per lane and row, four
        conversions, one 16-byte store), with the inputs
  %[xs]           LDS byte address of this wave's staged rows of tile k+2
  %[xt]           LDS byte address of this wave's rows of bf16 tile k+2
  %[xw]           64 * (wave & 1): the swizzle term the wave's rows share
  %[xtl0], %[xtl1]  per-lane offsets of the rows' last eight chunks (the
                  RoPE part): code word | scale byte << 16 in the staged
                  rows, and the destination in the bf16 tile
"""
import sys

FIRST_SCRATCH = 177
KADDR = [177, 178, 179, 180]          # key read address per qk offset
VADDR = [181, 182, 183, 184]          # value read address per (h2, parity)
PADDR = 185                           # P^T read address
CT, CO = 186, 187                     # copy temporaries
KF = [188, 192, 196]                  # key fragment slots (4 VGPRs each)
PF = [200, 204, 208, 212]             # P^T fragments, one per head group
VF = [216, 220]                       # value fragment slots (lo pair, hi pair)
SA = 224                              # score accumulator, then scores / numerators
SB = 240                              # score chain B, then bf16 numerators + temps
PW = KADDR[0]                         # P^T write address (keys are done by then)
NEG_INF = "0xff800000"
WRITE_TAGS = ("pw", "xw")                     # LDS ops that write no register


# One accumulator chain for the scores (dependent MFMAs issue back to back on
# this GPU at no cost), so the softmax needs no chain sum; the softmax scale
# is applied inside the exponent's fma, after the row maximum of the raw
# scores (scale > 0, so the maximum commutes with it).
SINGLE_CHAIN = True


class Geo:
    """Tile geometry of a row width D (bf16 elements per cache row)."""

    def __init__(self, d):
        self.d = d
        self.nk = d // 16                 # 16-wide query fragments
        self.half = self.nk // 2          # fragments per score chain
        self.chunks = d // 8              # 16-byte chunks per tile row
        self.copies = d * 2 * 32 // 1024 // 4   # 1 KB copies per wave and tile
        if SINGLE_CHAIN:
            self.kseq = list(range(self.nk))
        else:
            self.kseq = [f for i in range(self.half) for f in (i, self.half + i)]


G576 = Geo(576)
G512 = Geo(512)


def vr(base, n=4):
    return f"v[{base}:{base + n - 1}]"


class Stream:
    def __init__(self, geo=G576):
        self.geo = geo
        self.lines = []
        self.issued = []      # LDS op tags in issue order
        self.done = 0         # ops known complete (prefix of issued)

    def emit(self, s):
        self.lines.append(s)

    def lds(self, tag, text):
        self.issued.append(tag)
        self.emit(text)

    def wait_for(self, tag):
        last = max(i for i, t in enumerate(self.issued) if t == tag)
        if last < self.done:
            return
        n = min(len(self.issued) - (last + 1), 15)
        self.emit(f"s_waitcnt lgkmcnt({n})")
        self.done = len(self.issued) - n

    def wait_all(self):
        # every LDS read has landed (the scratch registers are free after the
        # stream); LDS writes issued after the last read may stay in flight
        # (the kernel waits for them before its next barrier)
        reads = [i for i, t in enumerate(self.issued) if t[0] not in WRITE_TAGS]
        if not reads or reads[-1] < self.done:
            return
        n = min(len(self.issued) - (reads[-1] + 1), 15)
        self.emit(f"s_waitcnt lgkmcnt({n})")
        self.done = len(self.issued) - n

    # ---- LDS reads
    def kread(self, s, slot):
        self.lds(("k", s), f"ds_read_b128 {vr(KF[slot])}, v{KADDR[s & 3]} offset:{128 * (s >> 2)}")

    def vread(self, vi):
        # value fragment vi = (k-step ks, column tile j of this wave's four)
        ks, j = vi >> 2, vi & 3
        slot = VF[vi % len(VF)]
        off = ks * 16 * self.geo.chunks * 16 + (j >> 1) * 128
        self.lds(("v", vi), f"ds_read_b64_tr_b16 {vr(slot, 2)}, v{VADDR[j & 1]} offset:{off}")
        self.lds(("v", vi), f"ds_read_b64_tr_b16 {vr(slot + 2, 2)}, v{VADDR[2 + (j & 1)]} offset:{off}")

    def pread(self, ks, g):
        self.lds(("p", ks, g), f"ds_read_b128 {vr(PF[g])}, v{PADDR} offset:{(2 * g + ks) * 1024}")

    # ---- MFMAs
    def pv(self, i):
        # MFMA i = (k-step ks, column tile j, head group g): O^T[j][g] += V^T(ks, j) P^T(ks, g)
        ks, j, g = i >> 4, (i >> 2) & 3, i & 3
        vi = ks * 4 + j
        self.wait_for(("v", vi))
        self.wait_for(("p", ks, g))
        o = j * 4 + g
        self.emit(f"v_mfma_f32_32x32x16_bf16 %[o{o}], {vr(VF[vi % len(VF)])}, {vr(PF[g])}, %[o{o}]")
        if g == 0 and vi + len(VF) - 1 < 8:
            self.vread(vi + len(VF) - 1)    # into the slot of fragment vi-1, now free
        if ks == 0 and j == 3:
            self.pread(1, g)                # P^T(0, g) has had its last use

    def copy(self, ii):
        # Copy ii of the wave: %[c{ii/2}] holds, in its low (even ii) or high
        # (odd ii) 16 bits, the lane's byte column (11 bits) and tile row
        # (5 bits, clamped to the tile's last valid row); the wave's ii-th
        # copy lands 4096*ii bytes after its first one.
        reg, sh = f"%[c{ii // 2}]", 16 * (ii & 1)
        self.emit(f"v_bfe_u32 v{CT}, {reg}, {sh + 11}, 5")
        self.emit(f"v_min_u32 v{CT}, %[cl], v{CT}")
        self.emit(f"v_bfe_u32 v{CO}, {reg}, {sh}, 11")
        self.emit(f"v_mad_u32_u24 v{CO}, v{CT}, %[k1152], v{CO}")
        self.emit(f"s_add_u32 m0, %[cd], {4096 * ii}")
        self.emit(f"global_load_lds_dwordx4 v{CO}, %[cb]")

    def op(self, items):
        """Emit one op group: plain lines, ("lds", tag, text) for LDS
        instructions (counted for the waits) and ("wait", tag)."""
        for it in items:
            if isinstance(it, str):
                self.emit(it)
            elif it[0] == "lds":
                self.lds(it[1], it[2])
            else:
                self.wait_for(it[1])

    def text(self):
        return "\n".join(self.lines)


def softmax_ops(masked):
    """VALU work turning the scores into bf16 numerators in LDS.
    Each entry is a list of instructions kept together."""
    a = [SA + r for r in range(16)]
    b = [SB + r for r in range(16)]
    mx, t1, t2, mu, ps, lim, neg = b[8], b[9], b[10], b[11], b[12], b[13], b[14]
    ops = []
    if not SINGLE_CHAIN:
        for r in range(16):
            ops.append([f"v_add_f32 v{a[r]}, v{a[r]}, v{b[r]}"])
        for r in range(16):
            ops.append([f"v_mul_f32 v{a[r]}, %[scale], v{a[r]}"])
    if masked:
        # (-inf goes through a VGPR: v_cndmask reads vcc over the constant bus)
        ops.append([f"v_subrev_u32 v{lim}, %[tok], %[vlim]", f"v_mov_b32 v{neg}, {NEG_INF}"])
        for r in range(16):
            t = 8 * (r >> 2) + (r & 3)   # token of register r (lane half adds 4, folded into vlim)
            ops.append([f"v_cmp_lt_i32 vcc, {t}, v{lim}",
                        f"v_cndmask_b32 v{a[r]}, v{neg}, v{a[r]}, vcc"])
    # row maximum over this lane's 16 tokens, then over the lane pair (l, l^32)
    m = [b[0], b[1], b[2], b[3], b[4], b[5], b[6]]
    ops.append([f"v_max3_f32 v{m[0]}, v{a[0]}, v{a[1]}, v{a[2]}"])
    ops.append([f"v_max3_f32 v{m[1]}, v{a[3]}, v{a[4]}, v{a[5]}"])
    ops.append([f"v_max3_f32 v{m[2]}, v{a[6]}, v{a[7]}, v{a[8]}"])
    ops.append([f"v_max3_f32 v{m[3]}, v{a[9]}, v{a[10]}, v{a[11]}"])
    ops.append([f"v_max3_f32 v{m[4]}, v{a[12]}, v{a[13]}, v{a[14]}"])
    ops.append([f"v_max3_f32 v{m[5]}, v{m[0]}, v{m[1]}, v{a[15]}"])
    ops.append([f"v_max3_f32 v{m[6]}, v{m[2]}, v{m[3]}, v{m[4]}"])
    ops.append([f"v_max_f32 v{mx}, v{m[5]}, v{m[6]}"])
    ops.append([f"v_mov_b32 v{t1}, v{mx}", f"v_mov_b32 v{t2}, v{mx}", "s_nop 1",
                f"v_permlane32_swap_b32 v{t1}, v{t2}", f"v_max_f32 v{mx}, v{t1}, v{t2}"])
    if SINGLE_CHAIN:
        ops.append([f"v_mul_f32 v{mx}, %[scale], v{mx}"])
    # running maximum; reference fixed at the first tile with a visible key;
    # largest excess of a tile maximum over the reference
    ops.append([f"v_max_f32 %[mseen], %[mseen], v{mx}"])
    ops.append([f"v_cmp_eq_f32 vcc, {NEG_INF}, %[mref]", f"v_cndmask_b32 %[mref], %[mref], v{mx}, vcc"])
    ops.append([f"v_sub_f32 v{t1}, v{mx}, %[mref]", f"v_max_f32 %[exc], %[exc], v{t1}"])
    ops.append([f"v_cmp_eq_f32 vcc, {NEG_INF}, %[mref]", f"v_cndmask_b32_e64 v{mu}, %[mref], 0, vcc"])
    for r in range(16):
        if SINGLE_CHAIN:
            ops.append([f"v_fma_f32 v{a[r]}, v{a[r]}, %[scale], -v{mu}", f"v_exp_f32 v{a[r]}, v{a[r]}"])
        else:
            ops.append([f"v_sub_f32 v{a[r]}, v{a[r]}, v{mu}", f"v_exp_f32 v{a[r]}, v{a[r]}"])
    ops.append([f"v_add_f32 v{ps}, v{a[0]}, v{a[1]}"])
    for r in range(2, 16):
        ops.append([f"v_add_f32 v{ps}, v{ps}, v{a[r]}"])
    ops.append([f"v_add_f32 %[lrun], %[lrun], v{ps}"])
    for i in range(8):
        ops.append([f"v_cvt_pk_bf16_f32 v{b[i]}, v{a[2 * i]}, v{a[2 * i + 1]}"])
    ops.append([f"v_add_u32 v{PW}, %[bpw], %[pa]",
                ("lds", ("pw",), f"ds_write_b128 v{PW}, {vr(b[0])}"),
                ("lds", ("pw",), f"ds_write_b128 v{PW}, {vr(b[4])} offset:1024")])
    return ops


def addresses(st, keys, values):
    if keys:
        for q in range(4):
            st.emit(f"v_add_u32 v{KADDR[q]}, %[bk], %[ka{q}]")
    if values:
        for j in range(4):
            st.emit(f"v_add_u32 v{VADDR[j]}, %[bv], %[va{j}]")
        st.emit(f"v_add_u32 v{PADDR}, %[bp], %[pa]")


def mfma_results_ready(st):
    # VALU code reads the results of the MFMAs just issued
    st.emit("s_nop 7")
    st.emit("s_nop 7")
    st.emit("s_nop 3")


def scores(st, kseq, p):
    """Score MFMA at position p of kseq, with the key read KF slots ahead
    (two chains, A over fragments 0..half-1 and B over the rest, when
    SINGLE_CHAIN is off)."""
    f = kseq[p]
    h = st.geo.half
    st.wait_for(("k", f))
    if SINGLE_CHAIN:
        chain, acc = SA, ("0" if f == 0 else vr(SA, 16))
    else:
        chain = SA if f < h else SB
        acc = "0" if f in (0, h) else vr(chain, 16)
    st.emit(f"v_mfma_f32_32x32x16_bf16 {vr(chain, 16)}, {vr(KF[p % len(KF)])}, %[q{f}], {acc}")
    if p + len(KF) < len(kseq):
        st.kread(kseq[p + len(KF)], p % len(KF))


def first(geo=G576):
    """Scores and softmax numerators of the first tile of a pass."""
    st = Stream(geo)
    st.emit("s_nop 4")
    addresses(st, True, False)
    for p in range(len(KF)):
        st.kread(geo.kseq[p], p)
    for p in range(len(geo.kseq)):
        scores(st, geo.kseq, p)
    mfma_results_ready(st)
    for op in softmax_ops(True):
        st.op(op)
    return st.text()


# FP4 expansion registers (free in the step's second part: the key address
# and key fragment registers, after the last score MFMA)
XS, XSS, XW = KADDR[1], KADDR[2], KADDR[3]    # code, scale and store bases
XSLOT = [(188, 192), (194, 198)]              # (4 output VGPRs, scale/address)
XTAIL = 193                                   # second address of the tail chunk
FP8KR_STEP_VMEM = 13     # copies a step issues after the staged rows it expands: 8 RoPE, 4 code, 1 scale
FP4_ROW = 320                                 # bytes per stored row
FP4_CODES = 288                               # code bytes per stored row


def swz_even(j):
    # the tile layout's chunk swizzle of row j for a wave with even index
    u = j >> 1
    return u ^ ((u & 1) << 2)


def fp4_cvt(o, e):
    # four conversions of the code word in o+3 (read last), scale in e
    sels = ["", " op_sel:[1,0,0]", " op_sel:[0,1,0]", " op_sel:[1,1,0]"]
    return [f"v_cvt_scalef32_pk_bf16_fp4 v{o + i}, v{o + 3}, v{e}{sels[i]}" for i in range(4)]


def fp4_expand_ops():
    """Op groups expanding this wave's eight rows of one staged FP4 tile into
    the bf16 tile (chunk c of row t at t*72 + (c ^ swz(t))): a setup, then per
    row j reads (slot j%2), conversion, store; reads run one row ahead."""
    rows = 8
    ops = [[f"v_lshrrev_b32 v{XS}, 2, %[pa]", f"v_add_u32 v{XS}, %[xs], v{XS}",
            f"v_lshrrev_b32 v{XSS}, 6, %[pa]", f"v_add_u32 v{XSS}, %[xs], v{XSS}",
            f"v_xor_b32 v{XW}, %[xw], %[pa]", f"v_add_u32 v{XW}, %[xt], v{XW}"]]

    def reads(j):
        o, e = XSLOT[j % 2]
        if j < rows:
            return [("lds", ("xr", j), f"ds_read_b32 v{o + 3}, v{XS} offset:{FP4_ROW * j}"),
                    ("lds", ("xr", j), f"ds_read_u8 v{e}, v{XSS} offset:{FP4_ROW * j + FP4_CODES}")]
        return [f"v_and_b32 v{e}, 0xffff, %[xtl0]", f"v_add_u32 v{e}, %[xs], v{e}",
                f"v_lshrrev_b32 v{XTAIL}, 16, %[xtl0]", f"v_add_u32 v{XTAIL}, %[xs], v{XTAIL}",
                ("lds", ("xr", j), f"ds_read_b32 v{o + 3}, v{e} offset:256"),
                ("lds", ("xr", j), f"ds_read_u8 v{XTAIL}, v{XTAIL} offset:{FP4_CODES + 16}")]

    def convert(j):
        o, e = XSLOT[j % 2]
        sc = e if j < rows else XTAIL
        return [("wait", ("xr", j)), f"v_lshlrev_b32 v{sc}, 23, v{sc}"] + fp4_cvt(o, sc)

    def store(j):
        o, e = XSLOT[j % 2]
        if j < rows:
            return [f"v_xor_b32 v{e}, {16 * swz_even(j)}, v{XW}",
                    ("lds", ("xw", j), f"ds_write_b128 v{e}, {vr(o)} offset:{1152 * j}")]
        return [f"v_add_u32 v{e}, %[xt], %[xtl1]", ("lds", ("xw", j), f"ds_write_b128 v{e}, {vr(o)}")]

    ops.append(reads(0))
    for j in range(rows + 1):
        if j + 1 <= rows:
            ops.append(reads(j + 1))
        ops.append(convert(j))
        ops.append(store(j))
    return ops


# FP8-KR expansion registers (free in the step's second part: the key
# fragment slots, and the copy temporaries, since expanding steps issue no
# copies)
XC, XSC = KADDR[1], KADDR[2]                  # code and scale read addresses
XCODE = [(CT, CO, 190), (188, 189, 191)]      # (code pair, scale) per read slot
XOUT = [192, 196]                             # four bf16 pairs per row, by row parity
FP8_CODES = 512                               # staged code bytes per row
FP8_SCALES = 4096                             # offset of the staged row scales


def fp8kr_expand_ops(vm_wait):
    """Op groups expanding this wave's eight staged rows of an e4m3 latent
    tile (512 codes per row, one power-of-two scale per row) into the bf16
    tile: four conversions of two codes each, which apply the scale exactly
    (e4m3 times a power of two is exact in bf16).  Lane l converts codes
    8l..8l+7 of each row (chunk l of the row); reads run one row ahead.  The
    RoPE part of the tile arrives by direct copies, not here.
    vm_wait: vmcnt that leaves this wave's staged rows landed."""
    rows = 8
    ops = [[f"s_waitcnt vmcnt({vm_wait})",
            f"v_lshrrev_b32 v{XC}, 1, %[pa]", f"v_add_u32 v{XC}, %[xs], v{XC}",
            f"v_mov_b32 v{XSC}, %[xs]",
            f"v_xor_b32 v{XW}, %[xw], %[pa]", f"v_add_u32 v{XW}, %[xt], v{XW}"]]

    def reads(j):
        c0, c1, sc = XCODE[j % 2]
        return [("lds", ("xr", j), f"ds_read_b64 v[{c0}:{c1}], v{XC} offset:{FP8_CODES * j}"),
                ("lds", ("xr", j), f"ds_read_b32 v{sc}, v{XSC} offset:{FP8_SCALES + 4 * j}")]

    def convert(j):
        c0, c1, sc = XCODE[j % 2]
        o = XOUT[j % 2]
        return [("wait", ("xr", j)),
                f"v_cvt_scalef32_pk_bf16_fp8 v{o}, v{c0}, v{sc}",
                f"v_cvt_scalef32_pk_bf16_fp8 v{o + 1}, v{c0}, v{sc} op_sel:[1,0,0]",
                f"v_cvt_scalef32_pk_bf16_fp8 v{o + 2}, v{c1}, v{sc}",
                f"v_cvt_scalef32_pk_bf16_fp8 v{o + 3}, v{c1}, v{sc} op_sel:[1,0,0]"]

    def store(j):
        c0, c1, sc = XCODE[j % 2]
        return [f"v_xor_b32 v{sc}, {16 * swz_even(j)}, v{XW}",
                ("lds", ("xw", j), f"ds_write_b128 v{sc}, {vr(XOUT[j % 2])} offset:{1152 * j}")]

    ops.append(reads(0))
    for j in range(rows):
        if j + 1 < rows:
            ops.append(reads(j + 1))
        ops.append(convert(j))
        ops.append(store(j))
    return ops


def merge(a, b):
    """Alternate two op lists, spreading the shorter one evenly."""
    if len(a) < len(b):
        a, b = b, a
    out, bi = [], 0
    for n, op in enumerate(a):
        out.append(op)
        while bi < len(b) and (bi + 1) * len(a) <= (n + 1) * len(b):
            out.append(b[bi])
            bi += 1
    out.extend(b[bi:])
    return out


# Weighted-sum MFMAs placed among the score MFMAs of the step's first part
# (the rest go to the second part, between the softmax's and the expansion's
# VALU work).  One per two score MFMAs (18 of 32) was the first form; 12
# measured 1.5% faster for the FP4 and fp8-latent streams and the same for
# the bf16 one.
FIRST_SUMS = 12


def step(copies, masked, geo=G576, expand=False, fp8_wait=None, first_sums=None):
    st = Stream(geo)
    st.emit("s_nop 4")
    addresses(st, True, True)
    for p in range(len(KF)):
        st.kread(geo.kseq[p], p)
    for g in range(4):
        st.pread(0, g)
    for vi in range(len(VF) - 1):
        st.vread(vi)
    n = len(geo.kseq)
    f = first_sums if first_sums is not None else (FIRST_SUMS if FIRST_SUMS is not None else geo.half)
    i = 0
    for p in range(n):
        scores(st, geo.kseq, p)
        # sum MFMA i follows score MFMA p when (p+1) f / n crosses an integer
        if (p + 1) * f // n > p * f // n:
            st.pv(i)
            if copies:
                # copy c follows sum MFMA round(c f / copies): spread over the first part
                for c in range(geo.copies):
                    if (c * f + geo.copies // 2) // geo.copies == i:
                        st.copy(c)
            i += 1
    mfma_results_ready(st)
    ops = softmax_ops(masked)
    if expand:
        ops = merge(ops, fp4_expand_ops())
    if fp8_wait is not None:
        ops = merge(ops, fp8kr_expand_ops(fp8_wait))
    rest = list(range(f, 32))
    per = -(-len(ops) // (len(rest) + 1))
    for n, i in enumerate(rest):
        for op in ops[n * per:(n + 1) * per]:
            st.op(op)
        st.pv(i)
    for op in ops[len(rest) * per:]:
        st.op(op)
    st.wait_all()
    mfma_results_ready(st)
    return st.text()


def pv_only(geo=G576):
    """Weighted sum of the last tile of a pass."""
    st = Stream(geo)
    st.emit("s_nop 4")
    addresses(st, False, True)
    for g in range(4):
        st.pread(0, g)
    for vi in range(len(VF) - 1):
        st.vread(vi)
    for i in range(32):
        st.pv(i)
    mfma_results_ready(st)
    return st.text()


def as_c_string(name, text):
    body = "\n".join(f'  "{line}\\n\\t"' for line in text.splitlines())
    return f"#define {name} \\\n" + " \\\n".join(body.splitlines()) + "\n"


def main():
    out = ["// Generated by gen_decode_bf16_asm.py; do not edit.", ""]
    regs = ", ".join(f'"v{r}"' for r in range(FIRST_SCRATCH, 256))
    out.append(f"#define MLA_BF16_ASM_SCRATCH {regs}\n")
    out.append(as_c_string("MLA_BF16_STEP_COPY", step(True, False)))
    out.append(as_c_string("MLA_BF16_STEP_MASKED", step(False, True)))
    out.append(as_c_string("MLA_BF16_FIRST", first()))
    out.append(as_c_string("MLA_BF16_PV_ONLY", pv_only()))
    out.append(as_c_string("MLA_NOPE_STEP_COPY", step(True, False, G512)))
    out.append(as_c_string("MLA_NOPE_STEP_MASKED", step(False, True, G512)))
    out.append(as_c_string("MLA_NOPE_FIRST", first(G512)))
    out.append(as_c_string("MLA_NOPE_PV_ONLY", pv_only(G512)))
    out.append(as_c_string("MLA_FP4_STEP_EXPAND", step(False, False, G576, expand=True)))
    out.append(as_c_string("MLA_FP8KR_STEP_EXPAND", step(False, False, G576, fp8_wait=FP8KR_STEP_VMEM)))
    sys.stdout.write("\n".join(out))


if __name__ == "__main__":
    main()
