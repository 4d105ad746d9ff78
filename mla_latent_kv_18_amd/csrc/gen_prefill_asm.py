"""Writes prefill_asm.inc: the instruction streams of the prefill attention
kernel's tile step (prefill_mfma.hip).

    python gen_prefill_asm.py > prefill_asm.inc

A wave owns 32 queries of one head; keys and values arrive in 64-key tiles
held in LDS, each split into two 32-key halves A and B.  One step is one
stream over one tile:

  scores A   S_A^T = K_A Q^T: 12 MFMAs (32x32x16 bf16), key fragments read
             four MFMAs ahead;
  scores B   12 MFMAs, with the softmax of half A between them;
  sum A      O^T += V_A^T P_A^T: 8 MFMAs (4 column tiles x 2 k-steps), with
             the softmax of half B between them;
  sum B      8 MFMAs.

Softmax of a half (per lane: one query, 16 keys; the other 16 keys of that
query sit in lane l ^ 32): mask (tiles on the diagonal only), the largest
raw score seen (for the reference check), numerators p = 2^(s*scale - m_ref)
against a per-query reference m_ref fixed at the pass's first tile, their
sum, bf16 numerators (written over the half's first eight score registers,
which the sum reads as its B operand).  The first step of a pass computes
both halves' scores first and sets m_ref to the tile's largest scaled score
over the lane pair.  Every LDS wait count is computed here from the issue
order, and every MFMA that reads a register a VALU instruction wrote within
the last five instructions gets wait states first.

A second stream, the copies, issues the wave's five 1 KB global->LDS copies
of one tile (see copies()).

Operands (named in the kernel):
  %[o0]..%[o3]    O^T accumulators, column tile j (in/out)
  %[q0]..%[q11]   query fragments (Q^T, 16 dims each; 8..11 the RoPE part)
  %[kq0]..%[kq3]  per-lane LDS byte offsets of the key fragments
  %[va0]..%[va3]  per-lane LDS byte offsets of the value fragments
  %[kb], %[vb]    LDS byte addresses of the tile's key rows and value rows
  %[scale]        softmax scale times log2(e)
  %[mref]         the reference (log2 units; set by the first step)
  %[mseen]        largest raw score seen (in/out)
  %[lrun]         running sum of the numerators (in/out)
  %[msk]          nonzero for tiles that reach past some query's last
                  visible key: then key index i of the tile (0..63, register
                  order below, lane half 0) is visible iff i <= %[lim]
The streams use v186-v255, vcc and scc as scratch.
"""
import sys

FIRST_SCRATCH, LAST_SCRATCH = 186, 255
SA, SB = 186, 202                 # scores of the two 32-key halves; registers 0-7 of a
PA, PB = SA, SB                   # half take its bf16 numerators (2 k-steps x 4 VGPRs)
KF = [218, 222, 226, 230]         # key fragment ring
VF = [234, 238, 242]              # value fragment ring
KADDR = [246, 247, 248, 249]
VADDR = KADDR                     # value addresses replace the key addresses after the last key read
T = list(range(250, 256))         # softmax temporaries
NEG_INF = "0xff800000"
NK = 12                           # 16-wide k-steps of a 192-wide key
HALF_KEY_BYTES = 32 * 24 * 16     # key rows of one half (24 chunks of 16 B a row)


def regs_of(tok):
    """VGPR numbers named by an operand token (v12 or v[12:15])."""
    if tok.startswith("v["):
        a, b = tok[2:-1].split(":")
        return set(range(int(a), int(b) + 1))
    if tok.startswith("v") and tok[1:].isdigit():
        return {int(tok[1:])}
    return set()


def vr(base, n=4):
    return f"v[{base}:{base + n - 1}]"


class Stream:
    def __init__(self):
        self.lines = []
        self.issued = []
        self.done = 0

    def emit(self, s):
        # an MFMA reading a VGPR that a VALU instruction wrote less than five
        # instructions earlier gets wait states first
        if s.startswith("v_mfma"):
            srcs = set()
            for tok in s.replace(",", " ").split()[2:]:
                srcs |= regs_of(tok)
            recent = set()
            for prev in self.lines[-5:]:
                if prev.startswith("v_") and not prev.startswith("v_mfma"):
                    recent |= regs_of(prev.replace(",", " ").split()[1])
            if srcs & recent:
                self.lines.append("s_nop 4")
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
        if len(self.issued) > self.done:
            self.emit("s_waitcnt lgkmcnt(0)")
            self.done = len(self.issued)

    def op(self, items):
        for it in items:
            self.emit(it)

    def text(self):
        return "\n".join(self.lines)


# score MFMA p (0..23): half p // 12, k-step p % 12
def kread(st, p):
    u, s = divmod(p, NK)
    st.lds(("k", p), f"ds_read_b128 {vr(KF[p % len(KF)])}, v{KADDR[s & 3]} offset:{u * HALF_KEY_BYTES + 128 * (s >> 2)}")


def score(st, p):
    u, s = divmod(p, NK)
    st.wait_for(("k", p))
    dst = SA if u == 0 else SB
    acc = "0" if s == 0 else vr(dst, 16)
    st.emit(f"v_mfma_f32_32x32x16_bf16 {vr(dst, 16)}, {vr(KF[p % len(KF)])}, %[q{s}], {acc}")
    if p + len(KF) < 2 * NK:
        kread(st, p + len(KF))
        if p + len(KF) == 2 * NK - 1:
            value_addresses(st)


# sum MFMA i (0..15): k-step ks = i // 4 of the tile (half ks // 2), column tile j = i % 4
def vread(st, i):
    ks, j = i >> 2, i & 3
    slot = VF[i % len(VF)]
    off = ks * 4096 + (j >> 1) * 128
    st.lds(("v", i), f"ds_read_b64_tr_b16 {vr(slot, 2)}, v{VADDR[j & 1]} offset:{off}")
    st.lds(("v", i), f"ds_read_b64_tr_b16 {vr(slot + 2, 2)}, v{VADDR[2 + (j & 1)]} offset:{off}")


def pv(st, i):
    ks, j = i >> 2, i & 3
    st.wait_for(("v", i))
    p = (PA if ks < 2 else PB) + 4 * (ks & 1)
    st.emit(f"v_mfma_f32_32x32x16_bf16 %[o{j}], {vr(VF[i % len(VF)])}, {vr(p)}, %[o{j}]")
    if i + len(VF) < 16:
        vread(st, i + len(VF))


def key_of(u, r):
    # key index within the tile of register r of half u, lane half 0 (half 1 adds 4)
    return 32 * u + 8 * (r >> 2) + (r & 3)


def mask_ops(u):
    """Masking of half u, one group skipped unless %[msk] is set (tiles that
    reach past some query's last visible key)."""
    s = SA if u == 0 else SB
    g = ["s_cmp_eq_u32 %[msk], 0", f"s_cbranch_scc1 .Lpf_nomask{u}_%=", f"v_mov_b32 v{T[0]}, {NEG_INF}"]
    for r in range(16):
        g += [f"v_cmp_le_i32 vcc, {key_of(u, r)}, %[lim]", f"v_cndmask_b32 v{s + r}, v{T[0]}, v{s + r}, vcc"]
    g.append(f".Lpf_nomask{u}_%=:")
    return [g]


def max_ops(regs, dst):
    """dst = max over regs (16 or 32 registers), as op groups."""
    m = T[1:6]
    ops = []
    if len(regs) == 16:
        for i in range(5):
            ops.append([f"v_max3_f32 v{m[i]}, v{regs[3 * i]}, v{regs[3 * i + 1]}, v{regs[3 * i + 2]}"])
        ops.append([f"v_max3_f32 v{m[0]}, v{m[0]}, v{m[1]}, v{m[2]}"])
        ops.append([f"v_max3_f32 v{m[3]}, v{m[3]}, v{m[4]}, v{regs[15]}"])
        ops.append([f"v_max_f32 v{dst}, v{m[0]}, v{m[3]}"])
        return ops
    # 32: five groups of six then the two left
    for i in range(5):
        a = regs[6 * i: 6 * i + 6]
        ops.append([f"v_max3_f32 v{m[i]}, v{a[0]}, v{a[1]}, v{a[2]}", f"v_max3_f32 v{m[i]}, v{m[i]}, v{a[3]}, v{a[4]}",
                    f"v_max_f32 v{m[i]}, v{m[i]}, v{a[5]}"])
    ops.append([f"v_max3_f32 v{m[0]}, v{m[0]}, v{m[1]}, v{m[2]}"])
    ops.append([f"v_max3_f32 v{m[3]}, v{m[3]}, v{m[4]}, v{regs[30]}"])
    ops.append([f"v_max3_f32 v{dst}, v{m[0]}, v{m[3]}, v{regs[31]}"])
    return ops


def numerator_ops(u):
    """p = 2^(s*scale - m_ref), their sum into %[lrun], bf16 numerators."""
    s = SA if u == 0 else SB
    p = PA if u == 0 else PB
    ps = T[1]
    ops = []
    for r in range(16):
        ops.append([f"v_fma_f32 v{s + r}, v{s + r}, %[scale], -%[mref]", f"v_exp_f32 v{s + r}, v{s + r}"])
    ops.append([f"v_add_f32 v{ps}, v{s}, v{s + 1}"])
    for r in range(2, 16):
        ops.append([f"v_add_f32 v{ps}, v{ps}, v{s + r}"])
    ops.append([f"v_add_f32 %[lrun], %[lrun], v{ps}"])
    for i in range(8):
        ops.append([f"v_cvt_pk_bf16_f32 v{p + i}, v{s + 2 * i}, v{s + 2 * i + 1}"])
    return ops


def half_softmax_ops(u):
    s = SA if u == 0 else SB
    ops = mask_ops(u)
    mx = T[0]
    ops += max_ops([s + r for r in range(16)], mx)
    ops.append([f"v_max_f32 %[mseen], %[mseen], v{mx}"])
    return ops + numerator_ops(u)


def key_addresses(st):
    for q in range(4):
        st.emit(f"v_add_u32 v{KADDR[q]}, %[kb], %[kq{q}]")


def value_addresses(st):
    for j in range(4):
        st.emit(f"v_add_u32 v{VADDR[j]}, %[vb], %[va{j}]")


def results_ready(st):
    # VALU reads of MFMA results
    st.emit("s_nop 7")
    st.emit("s_nop 7")
    st.emit("s_nop 3")


def spread(st, mfmas, ops):
    """Issue the MFMA callables with the op groups spread evenly between them."""
    n = len(mfmas)
    per = -(-len(ops) // n)
    for i, f in enumerate(mfmas):
        f()
        for op in ops[i * per:(i + 1) * per]:
            st.op(op)


def step(first):
    st = Stream()
    st.emit("s_nop 4")
    key_addresses(st)
    for p in range(len(KF)):
        kread(st, p)
    for p in range(NK):
        score(st, p)
    if first:
        # both halves, then the reference from the tile's largest score
        for p in range(NK, 2 * NK):
            score(st, p)
            if p >= 2 * NK - len(VF):
                vread(st, p - (2 * NK - len(VF)))
        results_ready(st)
        ops = mask_ops(0) + mask_ops(1)
        mx, t1, t2 = T[0], T[1], T[2]
        ops += max_ops([SA + r for r in range(16)] + [SB + r for r in range(16)], mx)
        ops.append([f"v_mov_b32 v{t1}, v{mx}", f"v_mov_b32 v{t2}, v{mx}", "s_nop 1",
                    f"v_permlane32_swap_b32 v{t1}, v{t2}", f"v_max_f32 v{mx}, v{t1}, v{t2}"])
        ops.append([f"v_max_f32 %[mseen], %[mseen], v{mx}", f"v_mul_f32 %[mref], %[scale], v{mx}"])
        for op in ops + numerator_ops(0):
            st.op(op)
        spread(st, [lambda i=i: pv(st, i) for i in range(8)], numerator_ops(1))
    else:
        # scores B with the softmax of A between them; the first group waits
        # for the results of chain A
        results_ready_after = [False]

        def score_b(p):
            score(st, p)
            if p >= 2 * NK - len(VF):
                vread(st, p - (2 * NK - len(VF)))
        mf = [lambda p=p: score_b(p) for p in range(NK, 2 * NK)]
        ops_a = half_softmax_ops(0)
        # chain A's last MFMA needs its wait states before the first read
        ops_a[0] = ["s_nop 7", "s_nop 7", "s_nop 3"] + ops_a[0]
        spread(st, mf, ops_a)
        results_ready(st)
        spread(st, [lambda i=i: pv(st, i) for i in range(8)], half_softmax_ops(1))
    for i in range(8, 16):
        pv(st, i)
    st.wait_all()
    results_ready(st)
    return st.text()


def copies():
    """The wave's five 1 KB global->LDS copies of one tile (copy j lands at
    %[cd] + 8192 j).  Copies 0-2 fill key rows: lane address %[cp{j}] + row *
    %[cs{j}] (its chunk of key row 0 of the sequence, and the row stride of
    the array the chunk comes from); copies 3, 4 fill value rows: %[vbase] +
    row * %[vs] + column.  Row = tile row r (byte j of %[d0], or byte 0 of
    %[d1] for copy 4) clamped to %[rlast], the tile's last row in the
    sequence, plus %[row0] for the key copies; the value columns are bytes 1, 2
    of %[d1]."""
    st = Stream()
    R, C, A = T[0], T[1], T[2]
    for j in range(5):
        src, sh = ("%[d0]", 8 * j) if j < 4 else ("%[d1]", 0)
        st.emit(f"v_bfe_u32 v{R}, {src}, {sh}, 8")
        st.emit(f"v_min_u32 v{R}, %[rlast], v{R}")
        st.emit(f"s_add_u32 m0, %[cd], {8192 * j}")
        if j < 3:
            st.emit(f"v_add_u32 v{R}, %[row0], v{R}")
            st.emit(f"v_mad_u64_u32 v[{A}:{A + 1}], vcc, v{R}, %[cs{j}], %[cp{j}]")
            st.emit(f"global_load_lds_dwordx4 v[{A}:{A + 1}], off")
        else:
            st.emit(f"v_bfe_u32 v{C}, %[d1], {8 * (j - 2)}, 8")
            st.emit(f"v_mad_u32_u24 v{C}, v{R}, %[vs], v{C}")
            st.emit(f"global_load_lds_dwordx4 v{C}, %[vbase]")
    return st.text()


def as_c_string(name, text):
    body = "\n".join(f'  "{line}\\n\\t"' for line in text.splitlines())
    return f"#define {name} \\\n" + " \\\n".join(body.splitlines()) + "\n"


def main():
    out = ["// Generated by gen_prefill_asm.py; do not edit.", ""]
    regs = ", ".join(f'"v{r}"' for r in range(FIRST_SCRATCH, LAST_SCRATCH + 1))
    out.append(f"#define MLA_PF_ASM_SCRATCH {regs}\n")
    out.append(as_c_string("MLA_PF_STEP", step(False)))
    out.append(as_c_string("MLA_PF_FIRST", step(True)))
    out.append(as_c_string("MLA_PF_COPY", copies()))
    sys.stdout.write("\n".join(out))


if __name__ == "__main__":
    main()
