"""Writes decode_bf16_asm.inc: the instruction streams of the bf16 latent
decode kernel's software-pipelined tile step (decode_mfma.hip).

    python gen_decode_bf16_asm.py > decode_bf16_asm.inc

One step of a workgroup (four waves, 128 heads of one query) consumes two
32-token tiles held in LDS: it scores tile k+1 against the register-resident
latent query and turns the scores into softmax numerators, and it adds tile
k's numerator-weighted value rows into the output accumulators.

  scores   S^T[t, h] = sum_d K[t, d] Q[h, d]: 36 MFMAs (32x32x16 bf16), in two
           independent chains (query fragments 0-17 and 18-35) that are added
           at the end, so that consecutive chain MFMAs never wait on each other
  softmax  p = 2^(S*scale*log2(e) - m_ref) against a per-head reference fixed
           at the first visible tile; the numerators of this wave's 32 heads
           go to LDS as bf16 (the B operand of the weighted sum)
  sum      O^T[c, h] += sum_t V^T[c, t] P^T[t, h]: 32 MFMAs; this wave owns
           latent columns 128*wave..+127 of all 128 heads (4 column tiles x 4
           head groups), so each transposed value fragment is read once and
           used for four head groups

The MFMA stream is [score A, score B, sum] x 18, then the remaining 14 sum
MFMAs with the softmax's VALU work placed between them.  LDS reads are
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
SA = 224                              # score chain A, then scores / numerators
SB = 240                              # score chain B, then bf16 numerators + temps
PW = KADDR[0]                         # P^T write address (keys are done by then)
NEG_INF = "0xff800000"


def vr(base, n=4):
    return f"v[{base}:{base + n - 1}]"


class Stream:
    def __init__(self):
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
        if self.done < len(self.issued):
            self.emit("s_waitcnt lgkmcnt(0)")
            self.done = len(self.issued)

    # ---- LDS reads
    def kread(self, s, slot):
        self.lds(("k", s), f"ds_read_b128 {vr(KF[slot])}, v{KADDR[s & 3]} offset:{128 * (s >> 2)}")

    def vread(self, vi):
        # value fragment vi = (k-step ks, column tile j of this wave's four)
        ks, j = vi >> 2, vi & 3
        slot = VF[vi % len(VF)]
        off = ks * 16 * 72 * 16 + (j >> 1) * 128
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

    def text(self):
        return "\n".join(self.lines)


def softmax_ops(masked):
    """VALU work turning the two score chains into bf16 numerators in LDS.
    Each entry is a list of instructions kept together."""
    a = [SA + r for r in range(16)]
    b = [SB + r for r in range(16)]
    mx, t1, t2, mu, ps, lim, neg = b[8], b[9], b[10], b[11], b[12], b[13], b[14]
    ops = []
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
    # running maximum; reference fixed at the first tile with a visible key;
    # largest excess of a tile maximum over the reference
    ops.append([f"v_max_f32 %[mseen], %[mseen], v{mx}"])
    ops.append([f"v_cmp_eq_f32 vcc, {NEG_INF}, %[mref]", f"v_cndmask_b32 %[mref], %[mref], v{mx}, vcc"])
    ops.append([f"v_sub_f32 v{t1}, v{mx}, %[mref]", f"v_max_f32 %[exc], %[exc], v{t1}"])
    ops.append([f"v_cmp_eq_f32 vcc, {NEG_INF}, %[mref]", f"v_cndmask_b32_e64 v{mu}, %[mref], 0, vcc"])
    for r in range(16):
        ops.append([f"v_sub_f32 v{a[r]}, v{a[r]}, v{mu}", f"v_exp_f32 v{a[r]}, v{a[r]}"])
    ops.append([f"v_add_f32 v{ps}, v{a[0]}, v{a[1]}"])
    for r in range(2, 16):
        ops.append([f"v_add_f32 v{ps}, v{ps}, v{a[r]}"])
    ops.append([f"v_add_f32 %[lrun], %[lrun], v{ps}"])
    for i in range(8):
        ops.append([f"v_cvt_pk_bf16_f32 v{b[i]}, v{a[2 * i]}, v{a[2 * i + 1]}"])
    ops.append([f"v_add_u32 v{PW}, %[bpw], %[pa]",
                f"ds_write_b128 v{PW}, {vr(b[0])}",
                f"ds_write_b128 v{PW}, {vr(b[4])} offset:1024"])
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
    """Score MFMA at position p of kseq (chain A takes fragment i, chain B
    fragment 18 + i), with the key read KF slots ahead."""
    f = kseq[p]
    st.wait_for(("k", f))
    chain = SA if f < 18 else SB
    acc = "0" if f in (0, 18) else vr(chain, 16)
    st.emit(f"v_mfma_f32_32x32x16_bf16 {vr(chain, 16)}, {vr(KF[p % len(KF)])}, %[q{f}], {acc}")
    if p + len(KF) < len(kseq):
        st.kread(kseq[p + len(KF)], p % len(KF))


KSEQ = [f for i in range(18) for f in (i, 18 + i)]


def first():
    """Scores and softmax numerators of the first tile of a pass."""
    st = Stream()
    st.emit("s_nop 4")
    addresses(st, True, False)
    for p in range(len(KF)):
        st.kread(KSEQ[p], p)
    for p in range(len(KSEQ)):
        scores(st, KSEQ, p)
    mfma_results_ready(st)
    for op in softmax_ops(True):
        for line in op:
            st.emit(line)
    return st.text()


def step(copies, masked):
    st = Stream()
    st.emit("s_nop 4")
    addresses(st, True, True)
    for p in range(len(KF)):
        st.kread(KSEQ[p], p)
    for g in range(4):
        st.pread(0, g)
    for vi in range(len(VF) - 1):
        st.vread(vi)
    for p in range(len(KSEQ)):
        scores(st, KSEQ, p)
        if p & 1:
            i = p >> 1
            st.pv(i)
            if copies and i % 2 == 0 and i // 2 < 9:
                st.copy(i // 2)
    mfma_results_ready(st)
    ops = softmax_ops(masked)
    rest = list(range(18, 32))
    per = -(-len(ops) // (len(rest) + 1))
    for n, i in enumerate(rest):
        for op in ops[n * per:(n + 1) * per]:
            for line in op:
                st.emit(line)
        st.pv(i)
    for op in ops[len(rest) * per:]:
        for line in op:
            st.emit(line)
    st.wait_all()
    mfma_results_ready(st)
    return st.text()


def pv_only():
    """Weighted sum of the last tile of a pass."""
    st = Stream()
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
    sys.stdout.write("\n".join(out))


if __name__ == "__main__":
    main()
