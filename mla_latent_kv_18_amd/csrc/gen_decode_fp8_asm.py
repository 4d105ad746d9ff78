"""Writes decode_fp8_asm.inc: the instruction streams of the fp8 latent
decode kernel's software-pipelined tile step (decode_fp8.hip).

    python gen_decode_fp8_asm.py > decode_fp8_asm.inc

A workgroup has four waves; wave w owns 32 heads of one query position.
Tiles are 64 tokens of e4m3 cache rows (one K-step of the fp8 MFMA for the
weighted sum) plus their 64 fp32 token scales.  Step k of a wave has two
phases:

  scores   S^T = K Q^T for tile k+1: 9 K-steps of 64 latent dims, two
           32-token blocks (beta), hi and lo query planes: 36 MFMAs
           (v_mfma_scale_f32_32x32x64_f8f6f4) into two accumulators.
           Between them: the encoding of tile k's value-side weights
           P' = p * kscale[t] into two e4m3 terms with a power-of-two scale
           per (head, 32-token block), straight into the B-operand registers
           of the weighted sum, and the wave's copies of tile k+2.
  sum      O^T += V^T P'^T for tile k: 16 column tiles x (hi, lo) = 32 MFMAs.
           Between them: the softmax of tile k+1, s = S * kscale[t] *
           qscale[h] * scale * log2(e), p = 2^(s - m_ref), P' = p * kscale[t],
           and its block maxima; P' and the maxima go to a private LDS area
           of the wave, read back by the next step's encoding.

So every VALU stretch sits beside MFMAs of another tile: the encoding of
tile k beside the scores of tile k+1, the softmax of tile k+1 beside the sum
of tile k.

Tile layout in LDS (16-row groups): 16-byte chunk c of row t at slot
576(t >> 4) + 16c + ((t & 15) ^ 4(c & 1)); the 64 token scales follow at
byte 36864.  Wave-wide copy i (0..35) fills slots 64i..64i+63.

Operands (named in the kernel):
  %[o0]..%[o15]   O^T accumulators, one per 32 latent columns
  %[qh0..8], %[ql0..8]  hi and lo latent query codes, 64 dims per K-step
  %[ka0], %[ka1]  per-lane key byte offsets (chunk parity 0 / 1)
  %[vo]           per-lane transposed value byte offset
  %[pa]           16 * lane
  %[bk], %[bv]    LDS byte address of the scored tile and of the summed tile
  %[sw]           LDS byte address of this wave's P' area (9216 B: value
                  group g at 1024*g + 16*lane, block maxima at 8192 + 16*lane)
  %[qmul]         per-head qscale * softmax scale * log2(e), at least the
                  smallest normal float (the streams rely on qmul > 0)
  %[mref], %[mseen], %[lrun], %[exc]  per-head softmax state (in/out)
  %[vlim], %[tok], %[domask]  token t (0..63) of the scored tile is visible
                  iff t < vlim - tok; the mask is applied when domask != 0
  %[docopy]       the step copies a tile when non-zero
  %[cb], %[cd], %[cl], %[csb], %[csd], %[k576], %[rl], %[q16], %[r0..8],
  %[k0..8]        the tile copy (see Stream.copy)
The streams use v176-v255, vcc, m0 and scc as scratch.
"""
import sys

FIRST_SCRATCH = 176
S127, S123 = 176, 177                 # E8M0 scale constants 2^0, 2^-4
KA = [178, 179]                       # key read addresses (chunk parity)
VA = 180                              # value read address
T0 = 181                              # temporary (copy offset while copying)
MYS, MYSL = 182, 183                  # E8M0 scales of the P' codes (hi, lo)
PH, PL = 184, 192                     # P' codes being summed (8 VGPRs each)
KF = [200, 208]                       # key operand slots (8 VGPRs each)
VF = 216                              # value operand slot of even column tiles (8 VGPRs)
VF2 = 208                             # ... of odd column tiles: the upper key slot, free once scores are done
SA, SB = 224, 240                     # score accumulators (beta 0, 1)
KS = list(range(200, 216))            # token scales, in the key slots once scores are done
KT0, KT1 = KS[0], KS[1]               # softmax temporaries while the key slots hold no scales
# the token scales pass through KS[0..7] four at a time (two buffers), so
# that KS[8..15] can hold the second value operand
SCA = KA[0]                           # token-scale read address (keys are done by then)
PAD = KA[1]                           # P' area address when P' is written (keys are done)
CT = T0                               # copy offset
# encoding working set (the value slot, free during the score phase)
XB = 216                              # the 4-value P' group being encoded
DEC = 220                             # 2 decoded hi terms, then the lo-term scale
DV = 222                              # div0, div1 (block scales as floats)
SPA = VA                              # P' area address during the encoding
NEG_INF = "0xff800000"


def vr(base, n=8):
    return f"v[{base}:{base + n - 1}]"


class Stream:
    def __init__(self):
        self.lines = []
        self.issued = []
        self.done = 0

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
        if self.done < len(self.issued):
            self.emit("s_waitcnt lgkmcnt(0)")
            self.done = len(self.issued)

    # ---- LDS reads
    def kread(self, s, beta, slot):
        # key operand of K-step s, block beta: chunks 4s + 2hf + {0, 1} of row tq + 32 beta
        off = 18432 * beta + 1024 * s
        base = KF[slot]
        self.lds(("k", s, beta), f"ds_read_b128 {vr(base, 4)}, v{KA[0]} offset:{off}")
        self.lds(("k", s, beta), f"ds_read_b128 {vr(base + 4, 4)}, v{KA[1]} offset:{off}")

    def vread(self, ct):
        base = VF if ct % 2 == 0 else VF2
        for j in range(4):
            self.lds(("v", ct), f"ds_read_b64_tr_b8 {vr(base + 2 * j, 2)}, v{VA} offset:{512 * ct + 9216 * j}")

    def kchunk(self, tag, c):
        # token scales of block c >> 2, lane tokens 8(c & 3) + 4hf .. +3, into buffer c & 1
        self.lds((tag, c), f"ds_read_b128 {vr(KS[4 * (c & 1)], 4)}, v{SCA} offset:{128 * (c >> 2) + 32 * (c & 3)}")

    def spill_maxima(self):
        # block maxima of the P' being encoded (pmax0, pmax1 per lane)
        self.emit(f"v_add_u32 v{SPA}, %[sw], %[pa]")
        self.lds(("sm",), f"ds_read_b64 v[{DV}:{DV + 1}], v{SPA} offset:8192")

    def spill_group(self, g):
        # P' values of group g (block g >> 2, registers 4(g & 3)..+3) into XB
        self.lds(("sp", g), f"ds_read_b128 {vr(XB, 4)}, v{SPA} offset:{1024 * g}")

    # ---- MFMAs
    def qk(self, s, beta, lo, slot):
        self.wait_for(("k", s, beta))
        acc = SA if beta == 0 else SB
        c = "0" if (s == 0 and not lo) else vr(acc, 16)
        q = f"%[ql{s}]" if lo else f"%[qh{s}]"
        sb = S123 if lo else S127
        self.emit(f"v_mfma_scale_f32_32x32x64_f8f6f4 {vr(acc, 16)}, {vr(KF[slot])}, {q}, {c}, "
                  f"v{S127}, v{sb} op_sel_hi:[0,0,0]")

    def pv(self, i):
        # MFMA i: column-tile pair i >> 2 in the order (ct, hi), (ct+1, hi),
        # (ct, lo), (ct+1, lo); even column tiles in VF, odd ones in VF2
        pair, r = i >> 2, i & 3
        ct = 2 * pair + (r & 1)
        lo = r >= 2
        self.wait_for(("v", ct))
        p, sc = (PL, MYSL) if lo else (PH, MYS)
        v = VF if ct % 2 == 0 else VF2
        self.emit(f"v_mfma_scale_f32_32x32x64_f8f6f4 %[o{ct}], {vr(v)}, {vr(p)}, %[o{ct}], "
                  f"v{S127}, v{sc} op_sel_hi:[0,0,0]")

    def copy(self, ii):
        # copy ii of the wave: tile row %[r{ii}] + the lane's row in its group
        # (clamped to the tile's last valid row), byte column %[k{ii}] + the
        # lane's 16-byte chunk; it lands 4096*ii bytes after the wave's first.
        # Skipped when %[docopy] is 0 (no tile left to copy).
        self.emit("s_cmp_lg_u32 %[docopy], 0")
        self.emit(f"s_cbranch_scc0 .Lnc%=_{ii}")
        self.emit(f"v_add_u32 v{CT}, %[r{ii}], %[rl]")
        self.emit(f"v_min_u32 v{CT}, %[cl], v{CT}")
        self.emit(f"v_mad_u32_u24 v{CT}, v{CT}, %[k576], %[q16]")
        self.emit(f"v_add_u32 v{CT}, %[k{ii}], v{CT}")
        self.emit(f"s_add_u32 m0, %[cd], {4096 * ii}")
        self.emit(f"global_load_lds_dwordx4 v{CT}, %[cb]")
        self.emit(f".Lnc%=_{ii}:")

    def copy_scales(self):
        self.emit("s_cmp_lg_u32 %[docopy], 0")
        self.emit("s_cbranch_scc0 .Lncs%=")
        self.emit(f"v_lshrrev_b32 v{CT}, 4, %[pa]")             # lane
        self.emit(f"v_min_u32 v{CT}, %[cl], v{CT}")
        self.emit(f"v_lshlrev_b32 v{CT}, 2, v{CT}")
        self.emit("s_mov_b32 m0, %[csd]")
        self.emit(f"global_load_lds_dword v{CT}, %[csb]")
        self.emit(".Lncs%=:")

    def text(self):
        return "\n".join(self.lines)


def setup(st, keys, values):
    st.emit("s_nop 4")
    st.emit(f"v_mov_b32 v{S127}, 0x7f")
    st.emit(f"v_mov_b32 v{S123}, 0x7b")
    if keys:
        st.emit(f"v_add_u32 v{KA[0]}, %[bk], %[ka0]")
        st.emit(f"v_add_u32 v{KA[1]}, %[bk], %[ka1]")
    if values:
        st.emit(f"v_add_u32 v{VA}, %[bv], %[vo]")


def results_ready(st):
    st.emit("s_nop 7")
    st.emit("s_nop 7")
    st.emit("s_nop 3")


def scale_ops(st, ops, tag, a, b):
    """Multiply a[r] (block 0) and b[r] (block 1) by their token scales, read
    four at a time into two alternating buffers, two chunks ahead."""
    ops.append(("lds", lambda: (st.kchunk(tag, 0), st.kchunk(tag, 1))))
    for c in range(8):
        ops.append(("wait", (tag, c)))
        regs = (a if c < 4 else b)[4 * (c & 3):4 * (c & 3) + 4]
        buf = KS[4 * (c & 1):4 * (c & 1) + 4]
        ops.append([f"v_mul_f32 v{regs[i]}, v{regs[i]}, v{buf[i]}" for i in range(4)])
        if c + 2 < 8:
            ops.append(("lds", lambda c=c: st.kchunk(tag, c + 2)))


def softmax_ops(st, masked):
    """VALU work on the two score accumulators up to the value-side weights
    P' = p * kscale (in SA, SB) and their per-block maxima; list of groups of
    instructions (LDS reads are issued through st so that waits are counted)."""
    a = [SA + r for r in range(16)]
    b = [SB + r for r in range(16)]
    ops = []
    # t = S * kscale, block by block (token scales of the scored tile); the
    # per-head factor qmul > 0 is applied to the maximum and inside the
    # exponent's fma (s = t * qmul)
    ops.append([f"v_lshrrev_b32 v{T0}, 9, %[pa]", f"v_lshl_add_u32 v{SCA}, v{T0}, 4, %[bks]"])
    scale_ops(st, ops, "ks", a, b)
    if masked:
        # tokens past the visible end of the scored tile; skipped when %[domask] is 0
        lim, neg = T0, KT0
        grp = ["s_cmp_lg_u32 %[domask], 0", "s_cbranch_scc0 .Lnm%=",
               f"v_subrev_u32 v{lim}, %[tok], %[vlim]", f"v_mov_b32 v{neg}, {NEG_INF}"]
        for beta, regs in ((0, a), (1, b)):
            for r in range(16):
                t = 32 * beta + 8 * (r >> 2) + (r & 3)
                grp += [f"v_cmp_lt_i32 vcc, {t}, v{lim}", f"v_cndmask_b32 v{regs[r]}, v{neg}, v{regs[r]}, vcc"]
        grp.append(".Lnm%=:")
        ops.append(grp)
    # row maximum over 32 tokens (two interleaved chains, T0 over block 0 and
    # KT0 over block 1), then over the lane pair (l, l^32)
    mx, t1, mu = T0, KT1, KT1             # (t1 dies before mu is set)

    def max_chains(acc_a, acc_b, last):
        chains = []
        for acc, v in ((acc_a, a), (acc_b, b)):
            c = [f"v_max3_f32 v{acc}, v{v[0]}, v{v[1]}, v{v[2]}"]
            c += [f"v_max3_f32 v{acc}, v{acc}, v{v[i]}, v{v[i + 1]}" for i in range(3, 15, 2)]
            c.append(f"v_max_f32 v{acc}, v{acc}, v{v[15]}")
            chains.append(c)
        for x, y in zip(*chains):
            ops.append([x, y])
        ops.append(last)

    max_chains(mx, KT0, [f"v_max_f32 v{mx}, v{mx}, v{KT0}", f"v_mul_f32 v{mx}, %[qmul], v{mx}"])
    ops.append([f"v_mov_b32 v{t1}, v{mx}", "s_nop 1",
                f"v_permlane32_swap_b32 v{t1}, v{mx}", f"v_max_f32 v{mx}, v{t1}, v{mx}"])
    ops.append([f"v_max_f32 %[mseen], %[mseen], v{mx}"])
    ops.append([f"v_cmp_eq_f32 vcc, {NEG_INF}, %[mref]", f"v_cndmask_b32 %[mref], %[mref], v{mx}, vcc"])
    ops.append([f"v_sub_f32 v{t1}, v{mx}, %[mref]", f"v_max_f32 %[exc], %[exc], v{t1}"])
    ops.append([f"v_cmp_eq_f32 vcc, {NEG_INF}, %[mref]", f"v_cndmask_b32_e64 v{mu}, %[mref], 0, vcc"])
    vals = a + b
    for r0 in range(0, 32, 4):   # four fmas, then their four exponentials
        ops.append([f"v_fma_f32 v{vals[r]}, v{vals[r]}, %[qmul], -v{mu}" for r in range(r0, r0 + 4)] +
                   [f"v_exp_f32 v{vals[r]}, v{vals[r]}" for r in range(r0, r0 + 4)])
    # row sum in four partial sums (KS[0..3]: no token scales are held now)
    ps = KS[0:4]
    ops.append([f"v_add_f32 v{ps[j]}, v{vals[j]}, v{vals[j + 4]}" for j in range(4)])
    for r0 in range(8, 32, 4):
        ops.append([f"v_add_f32 v{ps[j]}, v{ps[j]}, v{vals[r0 + j]}" for j in range(4)])
    ops.append([f"v_add_f32 v{ps[0]}, v{ps[0]}, v{ps[1]}", f"v_add_f32 v{ps[2]}, v{ps[2]}, v{ps[3]}",
                f"v_add_f32 v{ps[0]}, v{ps[0]}, v{ps[2]}", f"v_add_f32 %[lrun], %[lrun], v{ps[0]}"])
    # value-side weights P' = p * kscale and their block maxima (pmax0 in T0, pmax1 in KT1)
    scale_ops(st, ops, "kp", a, b)
    max_chains(T0, KT1, [])
    ops.pop()
    for t in (T0, KT1):  # the token scales are done: their registers are temporaries
        ops.append([f"v_mov_b32 v{KT0}, v{t}", "s_nop 1",
                    f"v_permlane32_swap_b32 v{KT0}, v{t}", f"v_max_f32 v{t}, v{KT0}, v{t}"])
    ops.append(("lds", lambda: spill_writes(st)))
    return ops


def spill_writes(st):
    """P' (SA, SB) and its block maxima (T0, KT1) to the wave's area."""
    st.emit(f"v_add_u32 v{PAD}, %[sw], %[pa]")
    for g in range(8):
        acc = SA if g < 4 else SB
        st.lds(("w",), f"ds_write_b128 v{PAD}, {vr(acc + 4 * (g & 3), 4)} offset:{1024 * g}")
    st.lds(("w",), f"ds_write_b32 v{PAD}, v{T0} offset:8192")
    st.lds(("w",), f"ds_write_b32 v{PAD}, v{KT1} offset:8196")


def encode_setup(st):
    """Block scales of the P' being encoded, from its block maxima (in DV,
    DV+1): MYS/MYSL (E8M0 scales of the hi and lo terms of this lane's
    K-block) and div0/div1 (the hi-term scales as floats, in place)."""
    e0, e1 = DV, DV + 1
    st.wait_for(("sm",))
    for e in (e0, e1):
        # exponent of the block maximum, clamped so that both scales stay normal
        st.emit(f"v_bfe_u32 v{e}, v{e}, 23, 8")
        st.emit(f"v_max_u32 v{e}, 11, v{e}")
        st.emit(f"v_min_u32 v{e}, 0xfe, v{e}")
    # E8M0 scale of this lane's K-block: block hf of the lane
    st.emit("s_mov_b32 vcc_lo, 0")
    st.emit("s_mov_b32 vcc_hi, -1")
    st.emit(f"v_cndmask_b32 v{MYS}, v{e0}, v{e1}, vcc")
    st.emit(f"v_subrev_u32 v{MYS}, 7, v{MYS}")
    st.emit(f"v_subrev_u32 v{MYSL}, 4, v{MYS}")
    for e in (e0, e1):
        st.emit(f"v_subrev_u32 v{e}, 7, v{e}")
        st.emit(f"v_lshlrev_b32 v{e}, 23, v{e}")              # div = 2^(e - 134)


def encode_group(st, g):
    """Two e4m3 terms of P' group g: hi codes into PH[g], lo codes into PL[g];
    the lo terms use div / 16 (the exponent field lowered by 4)."""
    div = DV + (g >> 2)
    x = [XB + i for i in range(4)]
    h, l = PH + g, PL + g
    st.wait_for(("sp", g))
    st.emit(f"v_cvt_scalef32_pk_fp8_f32 v{h}, v{x[0]}, v{x[1]}, v{div}")
    st.emit(f"v_cvt_scalef32_pk_fp8_f32 v{h}, v{x[2]}, v{x[3]}, v{div} op_sel:[0,0,0,1]")
    st.emit(f"v_cvt_pk_f32_fp8_e32 v[{DEC}:{DEC + 1}], v{h}")
    st.emit(f"v_fma_f32 v{x[0]}, -v{DEC}, v{div}, v{x[0]}")
    st.emit(f"v_fma_f32 v{x[1]}, -v{DEC + 1}, v{div}, v{x[1]}")
    st.emit(f"v_cvt_pk_f32_fp8_sdwa v[{DEC}:{DEC + 1}], v{h} src0_sel:WORD_1")
    st.emit(f"v_fma_f32 v{x[2]}, -v{DEC}, v{div}, v{x[2]}")
    st.emit(f"v_fma_f32 v{x[3]}, -v{DEC + 1}, v{div}, v{x[3]}")
    st.emit(f"v_subrev_u32 v{DEC}, 0x2000000, v{div}")
    st.emit(f"v_cvt_scalef32_pk_fp8_f32 v{l}, v{x[0]}, v{x[1]}, v{DEC}")
    st.emit(f"v_cvt_scalef32_pk_fp8_f32 v{l}, v{x[2]}, v{x[3]}, v{DEC} op_sel:[0,0,0,1]")


def encode_ops(st):
    """The encoding as groups of instructions to spread between MFMAs; each
    P' group is read once the previous one is encoded."""
    ops = [("lds", lambda: (st.spill_maxima(), st.spill_group(0))),
           ("fn", lambda: encode_setup(st))]
    for g in range(8):
        ops.append(("fn", lambda g=g: encode_group(st, g)))
        if g + 1 < 8:
            ops.append(("lds", lambda g=g: st.spill_group(g + 1)))
    return ops


def run_ops(st, ops):
    for op in ops:
        if isinstance(op, tuple):
            if op[0] in ("lds", "fn"):
                op[1]()
            else:
                st.wait_for(op[1])
        else:
            for line in op:
                st.emit(line)


def pv_and_next_values(st, i):
    """Sum MFMA i; once column tile ct has had its lo MFMA, column tile ct + 2
    is read into its slot."""
    st.pv(i)
    pair, r = i >> 2, i & 3
    if r >= 2 and pair + 1 < 8:
        st.vread(2 * pair + (r & 1) + 2)


def flatten(ops):
    """Instruction groups split into single instructions (groups holding a
    branch stay whole), so that interleave() spreads VALU work by count."""
    out = []
    for op in ops:
        if isinstance(op, list) and not any(l.startswith("s_cbranch") or l.endswith(":") or l.startswith("s_nop")
                                            for l in op):
            out.extend([l] for l in op)
        else:
            out.append(op)
    return out


def interleave(st, ops, n_slots, emit_slot, mfma_first):
    """emit_slot(i) for i < n_slots with the ops spread evenly between them.
    With mfma_first each MFMA issues before the waits and VALU work of its
    slot, so that it runs while they wait (the sum phase, whose softmax waits
    on token-scale reads); otherwise the slot's ops come first (the score
    phase, whose encoding reads were issued a slot earlier)."""
    ops = flatten(ops)
    n, j = len(ops), 0
    for i in range(n_slots):
        if mfma_first:
            emit_slot(i)
        target = -(-(i + 1) * n // n_slots)
        run_ops(st, ops[j:target])
        j = target
        if not mfma_first:
            emit_slot(i)
    run_ops(st, ops[j:])


def score_phase(st, copies, enc):
    """The 36 score MFMAs of the tile at %[bk]; between them the encoding of
    the P' in the wave's area (enc), the wave's tile copies (copies) and, once
    the encoding is done, the read of the first value column tile."""
    st.kread(0, 0, 0)
    st.kread(0, 1, 1)
    ops = encode_ops(st) if enc else []
    n_enc = 27 if enc else 0              # MFMA slots the encoding is spread over

    def slot(i):
        s, j = divmod(i, 4)
        beta, lo = ((0, 0), (1, 0), (0, 1), (1, 1))[j]
        st.qk(s, beta, lo, beta)
        if lo and s + 1 < 9:
            st.kread(s + 1, beta, beta)
        if j == 3 and copies:
            st.copy(s)
    if enc:
        interleave(st, ops, n_enc, slot, False)
        for i in range(n_enc, 36):
            slot(i)
            if i == n_enc:
                st.emit(f"v_add_u32 v{VA}, %[bv], %[vo]")
                st.vread(0)
    else:
        for i in range(36):
            slot(i)


def sum_phase(st, soft, masked, second_value=True, final_wait=True):
    """The 32 sum MFMAs of the tile at %[bv] (codes in PH/PL, scales in
    MYS/MYSL, value column tile 0 already requested, tile 1 requested here);
    between them the softmax of the scores just computed and its P' writes
    (soft).  Without final_wait the stream may end with this wave's P'
    writes in flight: only the wave itself reads them, in order."""
    if second_value:
        st.vread(1)                       # the upper key slot is free once scores are done
    st.emit("s_nop 7")                    # encoded operands written by VALU
    if soft:
        results_ready(st)
        ops = softmax_ops(st, masked)
        interleave(st, ops, 32, lambda i: pv_and_next_values(st, i), True)
    else:
        for i in range(32):
            pv_and_next_values(st, i)
    if final_wait:
        st.wait_all()
        results_ready(st)


def step():
    """Step k: encoding of tile k and scores of tile k+1 (with the copies of
    tile k+2), then the sum of tile k and the softmax of tile k+1."""
    st = Stream()
    setup(st, True, False)
    st.copy_scales()
    score_phase(st, True, True)
    sum_phase(st, True, True, final_wait=False)
    return st.text()


def first():
    """Scores and softmax of the first tile of a pass."""
    st = Stream()
    setup(st, True, False)
    score_phase(st, False, False)
    results_ready(st)
    run_ops(st, softmax_ops(st, True))
    st.wait_all()
    return st.text()


def last():
    """Encoding and sum of the last tile of a pass."""
    st = Stream()
    setup(st, False, False)
    run_ops(st, encode_ops(st))
    st.emit(f"v_add_u32 v{VA}, %[bv], %[vo]")
    st.vread(0)
    sum_phase(st, False, False)
    return st.text()


def as_c_string(name, text):
    body = "\n".join(f'  "{line}\\n\\t"' for line in text.splitlines())
    return f"#define {name} \\\n" + " \\\n".join(body.splitlines()) + "\n"


def main():
    out = ["// Generated by gen_decode_fp8_asm.py; do not edit.", ""]
    regs = ", ".join(f'"v{r}"' for r in range(FIRST_SCRATCH, 256))
    out.append(f"#define MLA_FP8_ASM_SCRATCH {regs}\n")
    out.append(as_c_string("MLA_FP8_STEP", step()))
    out.append(as_c_string("MLA_FP8_FIRST", first()))
    out.append(as_c_string("MLA_FP8_LAST", last()))
    sys.stdout.write("\n".join(out))


if __name__ == "__main__":
    main()
