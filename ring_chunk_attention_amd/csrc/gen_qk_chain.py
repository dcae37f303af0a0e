#!/usr/bin/env python3
"""Writes mla_qk_chain.inc: the 576-wide Q.K MFMA chain of the attention
kernel as inline asm, optionally with the softmax of the previous key tile
interleaved into it.

    python3 gen_qk_chain.py            # rewrite mla_qk_chain.inc beside this file
    python3 gen_qk_chain.py --check    # exit 1 if the file is out of date

Why asm: the chain's accumulator must stay in VGPRs (the output accumulators
own the AGPRs), the K fragments must stream from LDS a fixed distance ahead
of the MFMA that uses them, and the softmax VALU work has to sit between the
MFMAs.  With one wave per SIMD, an MFMA leaves room for only a few
independent VALU instructions before the next one is due (about four adds,
or two or three exponentials); the compiler neither keeps the accumulator in
VGPRs nor spreads the softmax that way.

The chain: 36 k-steps of v_mfma_f32_32x32x16_bf16, S^T += K_c Q_c^T, k-steps
0..31 from the 512-column sub-tile (fragment address a[c%4] + (c/4) KB),
32..35 from the 64-column sub-tile (b[c-32]).  NBUF fragment registers; the
read for step c+NBUF goes out right after the MFMA of step c, and
lgkmcnt(n) waits until at most n LDS operations are outstanding (they
complete in order; the only others in the block are the two P writes, issued
after every read).

The softmax of the previous tile's scores x[0..15] (this lane's 16 keys of
its query row, already masked with -inf where a key is not visible):
  m     = max(x) over both lane halves (permlane32 swap), times sc;
  m_run = max(m_run, m); m_ref = m if m_ref is -inf (the row's first visible
  tile); mu = m_ref, or 0 while it is still -inf;
  y_i   = exp2(sc * x_i - mu);  l_part += sum y_i (exact);
  x_k   = bf16 pair (y_2k, y_2k+1) (round to nearest even), k = 0..7;
  l_rnd += sum of the rounded weights (each half of the pair widened to
           fp32 by a shift or a mask: v_dot2 runs at a quarter of the rate);
  the two 16-byte P fragments x[0..3] and x[4..7] are written to LDS at
  paddr and paddr + 1 KB.
sc > 0 is the score scale in log2 units (x raw) or 1 (x already scaled).
The scores live in v[XR:XR+15] (a register constraint of the caller), so that
the asm can name single registers; the last MFMA of the chain writes the new
scores there, after the softmax has read them and the P writes have gone
out.

Placement: each softmax instruction goes to the earliest MFMA step at or
after the steps of the instructions it depends on, within a budget of VALU
issue time per step.  Where the pair needs wait states (a VCC write before
v_cndmask reads it, a VGPR write before v_permlane32_swap reads it, a
transcendental result before its first use, a permlane result before its
first use, and, to be safe, a VALU result before a P write stores it) the
consumer goes to a later step, so that the step's waitcnt,
MFMA and read separate the two.  The block ends with
24 wait states so that no VALU outside reads the MFMA result too early.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "mla_qk_chain.inc")

KS, KSA, NBUF = 36, 32, 6
XR = 200                       # first register of the score tuple
NEG_INF = "0xff800000"
BUDGET = 3.5                   # VALU issue time per MFMA step, in v_add_f32 units
LAST_STEP = KS - 2             # the softmax is done before the last MFMA


def frag(c):
    """Address operand and byte offset of k-step c's K fragment."""
    if c < KSA:
        return f"%[a{c % 4}]", (c // 4) * 1024
    return f"%[b{c - KSA}]", 0


def x(i):
    return f"v{XR + i}"


def softmax_ops():
    """(name, text, cost, deps) in program order."""
    ops = []

    def op(name, text, cost=1.0, deps=(), hazard=()):
        """deps may share a step with the op; hazard deps may not."""
        ops.append((name, text, cost, tuple((d, 0) for d in deps) + tuple((d, 1) for d in hazard)))

    # tile max of this lane's 16 scores (before the first MFMA, while its K
    # fragment is on the way: these carry step -1)
    op("mx", f"v_max3_f32 %[m], {x(0)}, {x(1)}, {x(2)}\n"
             f"v_max3_f32 %[m], %[m], {x(3)}, {x(4)}\n"
             f"v_max3_f32 %[m], %[m], {x(5)}, {x(6)}\n"
             f"v_max3_f32 %[m], %[m], {x(7)}, {x(8)}\n"
             f"v_max3_f32 %[m], %[m], {x(9)}, {x(10)}\n"
             f"v_max3_f32 %[m], %[m], {x(11)}, {x(12)}\n"
             f"v_max3_f32 %[m], %[m], {x(13)}, {x(14)}\n"
             f"v_max_f32 %[m], %[m], {x(15)}\n"
             f"v_mov_b32 %[tmp], %[m]", 0.0)
    # the other lane half (lane l +- 32 holds the row's other 16 keys)
    op("swap", "v_permlane32_swap_b32 %[m], %[tmp]", 2.0, hazard=["mx"])
    op("mxx", "v_max_f32 %[m], %[m], %[tmp]\n"
              "v_mul_f32 %[m], %[sc], %[m]\n"
              "v_max_f32 %[mrun], %[mrun], %[m]\n"
              f"v_cmp_eq_f32 vcc, {NEG_INF}, %[mref]", 3.5, hazard=["swap"])
    op("mref", "v_cndmask_b32 %[mref], %[mref], %[m], vcc\n"
               f"v_cmp_eq_f32 vcc, {NEG_INF}, %[mref]", 2.0, hazard=["mxx"])
    op("mu", "v_cndmask_b32_e64 %[mu], %[mref], 0, vcc", 1.0, hazard=["mref"])
    for j in range(16):
        op(f"fma{j}", f"v_fma_f32 {x(j)}, {x(j)}, %[sc], -%[mu]", 1.0, ["mu"])
        op(f"exp{j}", f"v_exp_f32 {x(j)}, {x(j)}", 1.6, [f"fma{j}"])
        op(f"add{j}", f"v_add_f32 %[lp], %[lp], {x(j)}", 1.0, [f"add{j - 1}"] if j else [], hazard=[f"exp{j}"])
        if j % 2 == 1:
            k = j // 2
            # pair k -> x[k]: after both adds (they read the fp32 values), and
            # after pair k/2, which reads x[k]
            deps = [f"add{j - 1}", f"add{j}"] + ([f"cvt{k // 2}"] if k else [])
            op(f"cvt{k}", f"v_cvt_pk_bf16_f32 {x(k)}, {x(j - 1)}, {x(j)}", 1.0, deps,
               hazard=[f"exp{j - 1}", f"exp{j}"])
            op(f"rlo{k}", f"v_lshlrev_b32 %[r0], 16, {x(k)}\n"
                          f"v_add_f32 %[lr], %[lr], %[r0]", 2.0,
               [f"cvt{k}"] + ([f"rhi{k - 1}"] if k else []))
            op(f"rhi{k}", f"v_and_b32 %[r1], 0xffff0000, {x(k)}\n"
                          f"v_add_f32 %[lr], %[lr], %[r1]", 2.0, [f"rlo{k}"])
    op("wr", f"ds_write_b128 %[pa], v[{XR}:{XR + 3}]\n"
             f"ds_write_b128 %[pa], v[{XR + 4}:{XR + 7}] offset:1024", 1.0,
       hazard=[f"cvt{k}" for k in range(8)])
    return ops


def schedule():
    """Step of each softmax op (see the module doc)."""
    step, load = {}, {}
    for name, _, cost, deps in softmax_ops():
        if name == "mx":
            step[name] = -1
            continue
        s = max(step[d] + hz for d, hz in deps)
        while load.get(s, 0.0) > 0.0 and load.get(s, 0.0) + cost > BUDGET and s < LAST_STEP:
            s += 1
        if s > LAST_STEP:
            raise SystemExit(f"softmax does not fit before the last MFMA ({name})")
        step[name] = s
        load[s] = load.get(s, 0.0) + cost
    return step


def chain(with_softmax):
    slots = {}
    if with_softmax:
        st = schedule()
        for name, text, _, _ in softmax_ops():
            slots.setdefault(st[name], []).extend(text.split("\n"))
    acc = "%[s]"
    lines = ["s_waitcnt lgkmcnt(0)"]
    for c in range(NBUF):
        a, o = frag(c)
        lines.append(f"ds_read_b128 %[t{c % NBUF}], {a} offset:{o}")
    lines += slots.get(-1, [])
    writes_out = 0   # P writes issued (they count in lgkmcnt after the reads)
    for c in range(KS):
        pending = min(NBUF - 1, KS - 1 - c)
        lines.append(f"s_waitcnt lgkmcnt({pending + writes_out})")
        src_c = "0" if c == 0 else acc
        dst = f"v[{XR}:{XR + 15}]" if (with_softmax and c == KS - 1) else acc
        lines.append(f"v_mfma_f32_32x32x16_bf16 {dst}, %[t{c % NBUF}], %[q{c}], {src_c}")
        if c + NBUF < KS:
            a, o = frag(c + NBUF)
            lines.append(f"ds_read_b128 %[t{c % NBUF}], {a} offset:{o}")
        for l in slots.get(c, []):
            lines.append(l)
            if l.startswith("ds_write"):
                writes_out += 1
    lines += ["s_nop 7", "s_nop 7", "s_nop 7"]
    return lines


def emit_function(name, with_softmax):
    lines = chain(with_softmax)
    body = "\n".join(f'      "{l}\\n"' for l in lines)
    outs = [f'[t{k}] "=&v"(t{k})' for k in range(NBUF)]
    ins = [f'[q{c}] "v"(qf[{c}])' for c in range(KS)]
    ins += [f'[a{k}] "v"(a{k})' for k in range(4)] + [f'[b{k}] "v"(b{k})' for k in range(4)]
    params = "const bf16x8* qf, uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,\n" \
             "    uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3"
    pre = "  u32x4 t0, t1, t2, t3, t4, t5;\n"
    if with_softmax:
        params = "f32x16& x, " + params + \
            ",\n    float sc, float& m_ref, float& m_run, float& l_part, float& l_rnd, uint32_t paddr"
        outs = ['[s] "=&v"(s)', f'[x] "+{{v[{XR}:{XR + 15}]}}"(x)'] + outs
        outs += ['[mref] "+v"(m_ref)', '[mrun] "+v"(m_run)', '[lp] "+v"(l_part)', '[lr] "+v"(l_rnd)']
        outs += ['[m] "=&v"(m)', '[tmp] "=&v"(tmp)', '[mu] "=&v"(mu)', '[r0] "=&v"(r0)', '[r1] "=&v"(r1)']
        ins += ['[sc] "s"(sc)', '[pa] "v"(paddr)']
        clobbers = '"vcc", "memory"'
        pre += "  f32x16 s;\n  float m, tmp, mu, r0, r1;\n"
    else:
        params = "f32x16& s, " + params
        outs = ['[s] "=&v"(s)'] + outs
        clobbers = '"memory"'
    return (f"__device__ __forceinline__ void {name}({params}) {{\n{pre}"
            f"  asm volatile(\n{body}\n"
            f"      : {', '.join(outs)}\n"
            f"      : {', '.join(ins)}\n"
            f"      : {clobbers});\n}}\n")



# ---------------------------------------------------------------------------
# One whole key-loop step of the shared-latent form in one block: the Q.K
# chain of tile t+2 (with the softmax of S(t+1) in it) interleaved with the
# P.V MFMAs of tile t, their LDS reads, and the copies of tile t+3.
# ---------------------------------------------------------------------------
TS_NBUF = 4          # K fragment registers of the chain inside the step
TS_BUDGET = 2.5      # VALU issue time per MFMA slot (3.0 and 3.5 measured ~0.5% slower)
VFA, VFB = 216, 220  # the two V fragment tuples (v[216:219], v[220:223])
N_PV = 32            # P.V MFMAs: 2 key halves x 4 value blocks x 4 row blocks


TS_TAIL = 4          # P.V MFMAs after the last chain step


def ts_order():
    """MFMA slots: P.V and chain MFMAs alternate; the chain ends TS_TAIL P.V
    MFMAs before the block does, so that the issue of those MFMAs covers the
    wait states between the last chain MFMA (it writes the new scores over
    x) and the first VALU read of x after the block."""
    seq = []
    n_pair = N_PV - TS_TAIL
    for i in range(n_pair):
        seq += [("P", i), ("C", i)]
    seq += [("C", c) for c in range(n_pair, KS)]
    seq += [("P", i) for i in range(n_pair, N_PV)]
    return seq


def ts_schedule(nslots):
    step, load = {}, {}
    # the P write and the last pack at least two MFMAs before the chain ends
    last = nslots - TS_TAIL - 3
    for name, _, cost, deps in softmax_ops():
        if name == "mx":
            step[name] = -1
            continue
        s = max(step[d] + hz for d, hz in deps)
        while load.get(s, 0.0) > 0.0 and load.get(s, 0.0) + cost > TS_BUDGET and s < last:
            s += 1
        if s > last:
            raise SystemExit(f"softmax does not fit in the tile step ({name})")
        step[name] = s
        load[s] = load.get(s, 0.0) + cost
    return step


TS_COPY_EVERY = 3     # slots between the copies, from the start of the block


def ts_copy_slots(seq):
    """The nine copies of a tile go out one every TS_COPY_EVERY MFMA slots from
    the start of the block (measured: early copies beat copies spread over
    the whole block by 3-4%)."""
    return {TS_COPY_EVERY * i: i for i in range(9)}


def tile_step_lines():
    seq = ts_order()
    st = ts_schedule(len(seq))
    sm_slots = {}
    for name, text, _, _ in softmax_ops():
        sm_slots.setdefault(st[name], []).extend(text.split("\n"))
    copies = ts_copy_slots(seq)

    lines = ["s_waitcnt lgkmcnt(0)", "s_mov_b32 %[m0sv], m0"]
    lds = []            # LDS operations in issue order
    known = [-1]        # every LDS op up to this index has completed

    def lds_op(line):
        lines.append(line)
        lds.append(line)
        return len(lds) - 1

    def need(ids):
        d = max(ids)
        if d <= known[0]:
            return
        n = len(lds) - 1 - d
        n = min(n, 15)
        lines.append(f"s_waitcnt lgkmcnt({n})")
        known[0] = len(lds) - 1 - n

    def vregs(g):
        r = VFA if g % 2 == 0 else VFB
        return r

    def v_reads(g):
        c, j = g // 4, g % 4
        r = vregs(g)
        imm = (j >> 1) * 1024 + c * 16384
        return (lds_op(f"ds_read_b64_tr_b16 v[{r}:{r + 1}], %[vb{j & 1}0] offset:{imm}"),
                lds_op(f"ds_read_b64_tr_b16 v[{r + 2}:{r + 3}], %[vb{j & 1}1] offset:{imm}"))

    pf_id = [lds_op(f"ds_read_b128 %[pf{rb}], %[pr] offset:{rb * 2048}") for rb in range(4)]
    vf_id = {0: v_reads(0)}
    k_id = {}
    for c in range(TS_NBUF):
        a, o = frag(c)
        k_id[c] = lds_op(f"ds_read_b128 %[t{c % TS_NBUF}], {a} offset:{o}")
    lines += sm_slots.get(-1, [])

    for k, (kind, i) in enumerate(seq):
        if kind == "P":
            g, rb = i // 4, i % 4
            j = g % 4
            need(list(vf_id[g]) + [pf_id[rb]])
            r = vregs(g)
            lines.append(f"v_mfma_f32_32x32x16_bf16 %[o{rb}{j}], v[{r}:{r + 3}], %[pf{rb}], %[o{rb}{j}]")
            if rb == 0 and g + 1 < 8:
                vf_id[g + 1] = v_reads(g + 1)
            if g == 3:  # last use of pf[rb] in the first key half: load the second
                pf_id[rb] = lds_op(f"ds_read_b128 %[pf{rb}], %[pr] offset:{rb * 2048 + 1024}")
        else:
            c = i
            need([k_id[c]])
            src_c = "0" if c == 0 else "%[s]"
            dst = f"v[{XR}:{XR + 15}]" if c == KS - 1 else "%[s]"
            lines.append(f"v_mfma_f32_32x32x16_bf16 {dst}, %[t{c % TS_NBUF}], %[q{c}], {src_c}")
            if c + TS_NBUF < KS:
                a, o = frag(c + TS_NBUF)
                k_id[c + TS_NBUF] = lds_op(f"ds_read_b128 %[t{c % TS_NBUF}], {a} offset:{o}")
        for l in sm_slots.get(k, []):
            if l.startswith("ds_write"):
                lds_op(l)
            else:
                lines.append(l)
        if k in copies:
            cp = copies[k]
            if cp < 8:
                lines += [f"s_add_u32 m0, %[m0a], {cp * 896}", "s_nop 0",
                          f"buffer_load_dwordx4 %[oa], %[ra], 0 offen offset:{cp * 128} lds"]
            else:
                lines += ["s_mov_b32 m0, %[m0b]", "s_nop 0",
                          "buffer_load_dwordx4 %[ob], %[rb], 0 offen offset:0 lds"]
    # (no trailing nops: the last P.V MFMAs cover the chain result, and their
    # own AGPR results are read only after the key loop, behind a barrier and
    # the nops the caller places there)
    lines += ["s_mov_b32 m0, %[m0sv]"]
    return lines


# The LDS addresses of the step move to the next step's buffers inside the
# block: each register gets its buffer delta (a scalar operand) added right
# after its last use, where the MFMAs hide the add, instead of between the
# blocks.  (An LDS read takes its address when it issues.)
TS_ROTATE = ([(f"a{k}", "da") for k in range(4)] + [(f"b{k}", "db") for k in range(4)]
             + [(f"vb{par}{h}", "dv") for par in range(2) for h in range(2)])


def rotate_addresses(lines):
    adds = {}
    for reg, delta in TS_ROTATE + [("pa", "dp")]:
        last = max(i for i, l in enumerate(lines) if f"%[{reg}]" in l)
        adds.setdefault(last, []).append(f"v_add_u32 %[{reg}], %[{delta}], %[{reg}]")
    last = max(i for i, l in enumerate(lines) if "%[pr]" in l)
    adds.setdefault(last, []).append("v_subrev_u32 %[pr], %[dp], %[pr]")   # pr - dp
    out = []
    for i, l in enumerate(lines):
        out.append(l)
        out += adds.get(i, [])
    return out


def emit_tile_step(rotate):
    """The tile step as a function: tile_step takes the step's LDS addresses;
    tile_step_rot also moves them to the next step's buffers (rotate_addresses)."""
    lines = tile_step_lines()
    if rotate:
        lines = rotate_addresses(lines)
    body = "\n".join(f'      "{l}\\n"' for l in lines)
    outs = ['[s] "=&v"(s)', f'[x] "+{{v[{XR}:{XR + 15}]}}"(x)']
    outs += [f'[t{k}] "=&v"(t{k})' for k in range(TS_NBUF)]
    outs += [f'[pf{k}] "=&v"(pf{k})' for k in range(4)]
    outs += [f'[vfa] "=&{{v[{VFA}:{VFA + 3}]}}"(vfa)', f'[vfb] "=&{{v[{VFB}:{VFB + 3}]}}"(vfb)']
    outs += ['[mref] "+v"(m_ref)', '[mrun] "+v"(m_run)', '[lp] "+v"(l_part)', '[lr] "+v"(l_rnd)']
    outs += ['[m] "=&v"(m)', '[tmp] "=&v"(tmp)', '[mu] "=&v"(mu)', '[r0] "=&v"(r0)', '[r1] "=&v"(r1)']
    outs += [f'[o{rb}{j}] "+a"(O[{rb}][{j}])' for rb in range(4) for j in range(4)]
    outs += ['[m0sv] "=&s"(m0sv)']
    ins = [f'[q{c}] "v"(qf[{c}])' for c in range(KS)]
    ins += ['[sc] "s"(sc)']
    ins += ['[oa] "v"(oa)', '[ob] "v"(ob)', '[ra] "s"(ra)', '[rb] "s"(rb)', '[m0a] "s"(m0a)', '[m0b] "s"(m0b)']
    if rotate:
        outs += [f'[a{k}] "+v"(a[{k}])' for k in range(4)] + [f'[b{k}] "+v"(b[{k}])' for k in range(4)]
        outs += ['[pa] "+v"(pw)', '[pr] "+v"(pr)']
        outs += [f'[vb{par}{h}] "+v"(vb[{2 * par + h}])' for par in range(2) for h in range(2)]
        ins += ['[da] "s"(da)', '[db] "s"(db)', '[dv] "s"(dv)', '[dp] "s"(dp)']
        name = "tile_step_rot"
        params = ("f32x16& x, f32x16 (&O)[4][4], const bf16x8* qf,\n"
                  "    uint32_t (&a)[4], uint32_t (&b)[4], float sc, float& m_ref, float& m_run, float& l_part,\n"
                  "    float& l_rnd, uint32_t& pw, uint32_t& pr, uint32_t (&vb)[4], uint32_t oa, uint32_t ob,\n"
                  "    const u32x4& ra, const u32x4& rb, uint32_t m0a, uint32_t m0b, int da, int db, int dv, int dp")
    else:
        ins += [f'[a{k}] "v"(a{k})' for k in range(4)] + [f'[b{k}] "v"(b{k})' for k in range(4)]
        ins += ['[pa] "v"(pw)', '[pr] "v"(pr)']
        ins += [f'[vb{par}{h}] "v"(vb[{2 * par + h}])' for par in range(2) for h in range(2)]
        name = "tile_step"
        params = ("f32x16& x, f32x16 (&O)[4][4], const bf16x8* qf,\n"
                  "    uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, uint32_t b0, uint32_t b1, uint32_t b2,\n"
                  "    uint32_t b3, float sc, float& m_ref, float& m_run, float& l_part, float& l_rnd, uint32_t pw,\n"
                  "    uint32_t pr, const uint32_t* vb, uint32_t oa, uint32_t ob, const u32x4& ra, const u32x4& rb,\n"
                  "    uint32_t m0a, uint32_t m0b")
    pre = ("  f32x16 s;\n  u32x4 t0, t1, t2, t3, pf0, pf1, pf2, pf3, vfa, vfb;\n"
           "  float m, tmp, mu, r0, r1;\n  uint32_t m0sv;\n")
    return (f"__device__ __forceinline__ void {name}({params}) {{\n{pre}"
            f"  asm volatile(\n{body}\n"
            f"      : {', '.join(outs)}\n"
            f"      : {', '.join(ins)}\n"
            f'      : "vcc", "scc", "memory");\n}}\n')


def render():
    head = ("// Generated by gen_qk_chain.py from its description of the chain; do not\n"
            "// edit by hand (rerun the script).  Included by mla_attn_kernels.inc inside its\n"
            "// anonymous namespace, after the vector typedefs.\n\n")
    return (head
            + "// S^T = K Q^T over the 576 columns of one key tile.\n"
            + emit_function("qk_chain", False) + "\n"
            + "// The same chain with the softmax of the previous tile's scores x\n"
            + "// interleaved (P fragments to LDS at paddr, row stats updated in\n"
            + "// place); x returns the new scores.\n"
            + emit_function("qk_chain_softmax", True) + "\n"
            + "// One key-loop step of the shared-latent form: P V of tile t into O (P at\n"
            + "// pr, V of the tile by the four bases vb), the Q.K chain of tile t+2 (K\n"
            + "// fragments by a, b) with the softmax of S(t+1) = x in it (P to pw, new\n"
            + "// scores to x), and the nine copies of tile t+3 (buffer resources ra/rb,\n"
            + "// offsets oa/ob, LDS bases for M0 m0a/m0b), all interleaved.\n"
            + emit_tile_step(False) + "\n"
            + "// The same step that also returns a, b, vb and pw moved by da, db, dv and\n"
            + "// dp, and pr by -dp: the next step's addresses, added inside the block.\n"
            + emit_tile_step(True))


def main():
    text = render()
    if "--check" in sys.argv:
        cur = open(OUT).read() if os.path.exists(OUT) else ""
        if cur != text:
            print(f"{OUT} is out of date; rerun {os.path.basename(__file__)}")
            sys.exit(1)
        return
    with open(OUT, "w") as f:
        f.write(text)


if __name__ == "__main__":
    main()
